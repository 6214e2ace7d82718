"""Seeded synthetic workloads for the local MoE forward pass.

This module only *draws inputs*: router logits [T, E], tokens [T, H] and expert weights
(gate/up [E, I, H], down [E, H, I]) with the shapes and value distributions of the five
workloads this library is measured on, plus the deliberately tied and NaN/inf router rows
that exercise the routing contract of the ruDNN user guide (section 4, "Routing contract").
It contains no step of the method itself (no softmax, selection, grouping, SwiGLU or
combine), so both the CPU oracle and the GPU path can consume it without sharing any of
the method's arithmetic.

Recipe (all draws are fp32, then rounded to the storage dtype with round-to-nearest-even):

* Router logits use numpy ``Generator(PCG64(SeedSequence([seed, stream])))``: stream 0 is the
  N(0, 1) noise, stream 1 the expert-rank permutation of the Zipf bias, stream 2 the special
  rows.  A Zipf(s) load skew adds ``b_e = -s * ln(r_e)`` to column e, with ``r`` a seeded
  permutation of 1..E, i.e. a rank-r expert gets weight proportional to r**-s on the softmax
  scale.
* After rounding to the logits dtype every pair of logits in a row is at least 1e-3 apart
  (exact duplicates included); offending entries (the higher expert id of a close pair) are
  redrawn until the row is clean.  Deliberate ties are added afterwards.
* Tokens are N(0, 1); gate/up are N(0, 1) / sqrt(H) and down N(0, 1) / sqrt(I) (std = one
  over the square root of the fan-in).  They are drawn with torch's generator on the device
  the tensor lives on, seeded per (seed, stream, expert): stream 3 is tokens, 4 gate, 5 up,
  6 down.  The same seed on another device gives other (equally distributed) values, so a
  test always hands the *same bytes* to both sides.
* The gate (router) weights of the fused projection are N(0, 1) / sqrt(H) [E, H] (stream 7),
  so the logits of N(0, 1) tokens are about N(0, 1).  Its special inputs (numpy stream 8 picks
  the rows): token rows holding a NaN or a +inf, all-zero token rows (every logit 0, a full
  tie), and "twin" experts whose router row is a copy of a lower expert's (equal logits for
  every token).
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import numpy as np
import torch

__all__ = [
    "DTYPES", "DTYPE_CODE", "SPECIAL_KINDS", "SIGMOID_SPECIAL_KINDS", "SigmoidRouting", "Workload", "WORKLOADS",
    "make_logits", "make_sigmoid_logits", "make_tokens", "make_experts", "make_router", "make_projection_inputs",
    "PROJECTION_SPECIAL_KINDS",
]

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
# Numeric codes shared by the C boundary and the oracle (a plain enumeration, no arithmetic).
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}

# Special router rows.  T* rows hold deliberate exact ties, N* rows are "NaN rows" in the sense
# of the routing contract (a NaN, a +inf, or nothing but -inf).
SPECIAL_KINDS = ("uniform", "boundary_tie", "top_tie", "partial_neginf", "nan", "posinf", "all_neginf")

# Special rows of the group-limited sigmoid workloads: two experts with equal logit and equal
# bias, two groups with equal logits and equal biases, and rows with a NaN / +inf / -inf logit.
SIGMOID_SPECIAL_KINDS = ("expert_tie", "group_tie", "nan", "posinf", "neginf")

# Special token rows of the fused gate projection: one element NaN, one element +inf, all zero.
PROJECTION_SPECIAL_KINDS = ("nan", "posinf", "zero")

_SEP = 1e-3  # minimum gap between distinct logits of one row (after rounding to the dtype)


@dataclass(frozen=True)
class SigmoidRouting:
    """Options of group-limited sigmoid routing (ruDNN user guide, section 10) and the spread of
    the drawn FP32 correction bias."""
    groups: int
    selected_groups: int
    group_top_two: bool
    renormalize: bool
    scale: float
    bias_std: float


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int | None          # None: no expert weights (identity experts)
    E: int
    top_k: int
    dtype: str             # tokens and expert weights
    logits_dtype: str
    renormalize: tuple     # the renormalisation settings this workload is run with
    zipf_s: float | None   # per-expert load skew, None for none
    seed: int
    special: tuple = (0, 0, 0, 0, 0, 0, 0)  # row counts per SPECIAL_KINDS (or SIGMOID_SPECIAL_KINDS) entry
    sigmoid: SigmoidRouting | None = None   # group-limited sigmoid routing instead of softmax

    def with_T(self, T: int) -> "Workload":
        """Same recipe with T rows; special-row counts scale with T (at least one of each kind
        the full workload has, when T allows)."""
        if T == self.T:
            return self
        counts = []
        for c in self.special:
            counts.append(0 if c == 0 else max(1, round(c * T / self.T)))
        while sum(counts) > T:
            i = int(np.argmax(counts))
            counts[i] -= 1
        return dataclasses.replace(self, T=T, special=tuple(counts))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # Tiny fp32 layer: 4 tied rows and 3 NaN rows among its 64.
    "tiny": Workload("tiny", 64, 128, 256, 8, 2, "f32", "f32", (True,), None, 101,
                     special=(1, 1, 1, 1, 1, 1, 1)),
    # Routing + dispatch only (identity experts): 1% tied rows, 0.5% NaN rows.
    "route_dispatch": Workload("route_dispatch", 65536, 2048, None, 128, 8, "bf16", "bf16",
                               (True, False), 1.1, 102, special=(164, 164, 164, 163, 110, 109, 109)),
    # Decode-shaped, weight-bandwidth-bound layer.
    "decode": Workload("decode", 16, 7168, 2048, 256, 8, "bf16", "bf16", (True,), None, 103),
    # Mixtral-shaped layer, near-uniform load.
    "mixtral": Workload("mixtral", 4096, 4096, 14336, 8, 2, "bf16", "bf16", (True,), None, 104),
    # Fine-grained, skewed load (some experts >10x the mean, some empty), fp16.
    "skewed": Workload("skewed", 8192, 2048, 768, 128, 8, "f16", "f16", (False,), 1.2, 105),
    # Group-limited sigmoid routing (section 10) on the decode shape's 256 experts: 8 groups of
    # 32, 4 groups chosen by the sum of their two best corrected scores, top-8, renormalised,
    # scaled by 2.5.  Routing only, many rows: 0.5% tied rows, 0.3% rows with NaN/inf logits.
    "sigmoid_route": Workload("sigmoid_route", 65536, 7168, None, 256, 8, "bf16", "bf16", (True,), None, 106,
                              special=(164, 164, 66, 66, 66),
                              sigmoid=SigmoidRouting(8, 4, True, True, 2.5, 0.05)),
    # The decode layer routed that way.
    "sigmoid_decode": Workload("sigmoid_decode", 16, 7168, 2048, 256, 8, "bf16", "bf16", (True,), None, 107,
                               sigmoid=SigmoidRouting(8, 4, True, True, 2.5, 0.05)),
}


def _np_rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def _round_to(vals: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 -> dtype (RNE, by torch) -> back to fp32; the result is exactly representable."""
    t = torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32))
    return t.to(DTYPES[dtype]).to(torch.float32).numpy()


def _separate(vals: np.ndarray, noise: np.ndarray, bias: np.ndarray, dtype: str,
              rng: np.random.Generator) -> np.ndarray:
    """Redraw entries until every pair of a row is >= _SEP apart after rounding.

    Each pass re-checks only the rows changed by the previous pass."""
    rows = np.arange(vals.shape[0])
    E = vals.shape[1]
    for _ in range(10000):
        sub = vals[rows]
        order = np.argsort(sub, axis=1, kind="stable")
        sv = np.take_along_axis(sub, order, axis=1).astype(np.float64)
        bad = np.diff(sv, axis=1) < _SEP
        if not bad.any():
            return vals
        r, p = np.nonzero(bad)
        hi = np.maximum(order[r, p], order[r, p + 1])
        key = np.unique(rows[r].astype(np.int64) * E + hi)
        rr, cc = key // E, key % E
        noise[rr, cc] = rng.standard_normal(len(key), dtype=np.float32)
        vals[rr, cc] = _round_to(noise[rr, cc] + bias[cc], dtype)
        rows = np.unique(rr)
    raise RuntimeError("logit separation did not converge")


def make_logits(w: Workload):
    """Router logits for workload ``w``.

    Returns ``(logits, special)``: ``logits`` is a CPU tensor [T, E] in the logits dtype and
    ``special`` maps each special-row kind to the sorted row positions that hold it.
    """
    T, E, k = w.T, w.E, w.top_k
    rng0, rng1, rng2 = _np_rng(w.seed, 0), _np_rng(w.seed, 1), _np_rng(w.seed, 2)
    if w.zipf_s is not None:
        ranks = rng1.permutation(E).astype(np.float64) + 1.0
        bias = (-w.zipf_s * np.log(ranks)).astype(np.float32)
    else:
        bias = np.zeros(E, np.float32)
    noise = rng0.standard_normal((T, E), dtype=np.float32)
    vals = _round_to(noise + bias[None, :], w.logits_dtype)
    if E > 1:
        vals = _separate(vals, noise, bias, w.logits_dtype, rng0)

    n_special = sum(w.special)
    positions = np.sort(rng2.choice(T, size=n_special, replace=False)) if n_special else np.zeros(0, int)
    perm = rng2.permutation(n_special)
    special = {}
    cursor = 0
    for kind, count in zip(SPECIAL_KINDS, w.special):
        rows = np.sort(positions[perm[cursor:cursor + count]])
        cursor += count
        special[kind] = rows
        for r in rows:
            row = vals[r]
            if kind == "uniform":
                row[:] = _round_to(np.array([rng2.standard_normal()], np.float32), w.logits_dtype)[0]
            elif kind == "boundary_tie":
                # the k-th and (k+1)-th largest logits made equal
                if E <= k:
                    raise ValueError("a boundary tie needs E > top_k")
                desc = np.argsort(-row.astype(np.float64), kind="stable")
                row[desc[k]] = row[desc[k - 1]]
            elif kind == "top_tie":
                a = int(np.argmax(row))
                others = [e for e in range(E) if e != a]
                c = int(others[rng2.integers(len(others))])
                row[c] = row[a]
            elif kind == "partial_neginf":
                f = max(1, (k - 1) // 2)
                keep = rng2.choice(E, size=f, replace=False)
                mask = np.ones(E, bool)
                mask[keep] = False
                row[mask] = -np.inf
            elif kind == "nan":
                row[rng2.integers(E)] = np.nan
            elif kind == "posinf":
                row[rng2.integers(E)] = np.inf
            elif kind == "all_neginf":
                row[:] = -np.inf
    logits = torch.from_numpy(vals).to(DTYPES[w.logits_dtype])
    return logits, special


def make_tied_logits(T: int, E: int, dtype: str, seed: int, levels: int = 0) -> torch.Tensor:
    """Router logits with no separation between entries, so that equal values are frequent:
    N(0, 1) rounded to ``dtype`` (bf16 holds 128 values per binade, so a row of 1024 repeats
    many), or with ``levels`` > 0 drawn uniformly from the ``levels`` integers centred on 0
    (every row then is mostly ties).  CPU tensor [T, E] in ``dtype``."""
    rng = _np_rng(seed, 0)
    if levels > 0:
        vals = (rng.integers(0, levels, (T, E)) - levels // 2).astype(np.float32)
    else:
        vals = _round_to(rng.standard_normal((T, E), dtype=np.float32), dtype)
    return torch.from_numpy(vals).to(DTYPES[dtype])


def make_sigmoid_logits(w: Workload):
    """Router logits and FP32 correction bias for a group-limited sigmoid workload.

    Logits: N(0, 1) (stream 0), rounded to the logits dtype and separated like the softmax
    workloads.  Bias [E]: N(0, bias_std) in FP32 (stream 1), with twins so that exact ties can
    be built: in every group the experts 2i and 2i + 1 (i < per / 4) share a bias value, and the
    last group repeats the second-to-last group's biases.  Returns ``(logits, bias, special)``
    (CPU tensors; ``special`` maps each SIGMOID_SPECIAL_KINDS entry to its sorted rows)."""
    sg = w.sigmoid
    if sg is None:
        raise ValueError(f"workload {w.name!r} does not use sigmoid routing")
    T, E, G = w.T, w.E, sg.groups
    per = E // G
    rng0, rng1, rng2 = _np_rng(w.seed, 0), _np_rng(w.seed, 1), _np_rng(w.seed, 2)
    bias = (rng1.standard_normal(E) * sg.bias_std).astype(np.float32)
    for g in range(G):
        for i in range(per // 4):
            bias[g * per + 2 * i + 1] = bias[g * per + 2 * i]
    if G >= 2:
        bias[(G - 1) * per:] = bias[(G - 2) * per:(G - 1) * per]
    noise = rng0.standard_normal((T, E), dtype=np.float32)
    vals = _round_to(noise, w.logits_dtype)
    if E > 1:
        vals = _separate(vals, noise, np.zeros(E, np.float32), w.logits_dtype, rng0)

    n_special = sum(w.special)
    positions = np.sort(rng2.choice(T, size=n_special, replace=False)) if n_special else np.zeros(0, int)
    perm = rng2.permutation(n_special)
    special = {}
    cursor = 0
    for kind, count in zip(SIGMOID_SPECIAL_KINDS, w.special):
        rows = np.sort(positions[perm[cursor:cursor + count]])
        cursor += count
        special[kind] = rows
        for r in rows:
            row = vals[r]
            if kind == "expert_tie":
                # a bias-twin pair takes the row's largest logit
                if per < 4:
                    raise ValueError("expert ties need at least 4 experts per group")
                g, i = int(rng2.integers(G)), int(rng2.integers(per // 4))
                row[g * per + 2 * i] = row[g * per + 2 * i + 1] = row.max()
            elif kind == "group_tie":
                if G < 2:
                    raise ValueError("group ties need two groups")
                row[(G - 1) * per:] = row[(G - 2) * per:(G - 1) * per]
            elif kind == "nan":
                row[rng2.integers(E)] = np.nan
            elif kind == "posinf":
                row[rng2.integers(E)] = np.inf
            elif kind == "neginf":
                row[rng2.integers(E)] = -np.inf
    logits = torch.from_numpy(vals).to(DTYPES[w.logits_dtype])
    return logits, torch.from_numpy(bias), special


def _torch_gen(device, seed: int, stream: int, sub: int = 0) -> torch.Generator:
    s = int(np.random.SeedSequence([seed, stream, sub]).generate_state(1, np.uint64)[0]) & (2**63 - 1)
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def make_tokens(w: Workload, device="cpu") -> torch.Tensor:
    """Tokens [T, H] ~ N(0, 1) in the token dtype, on ``device``."""
    g = _torch_gen(device, w.seed, 3)
    x = torch.randn(w.T, w.H, generator=g, device=device, dtype=torch.float32)
    return x.to(DTYPES[w.dtype])


def make_experts(w: Workload, device="cpu"):
    """Expert weights ``(gate, up, down)``: gate/up [E, I, H] ~ N(0, 1)/sqrt(H), down
    [E, H, I] ~ N(0, 1)/sqrt(I), drawn expert by expert, on ``device``."""
    if w.I is None:
        raise ValueError(f"workload {w.name!r} has no expert weights")
    E, H, I = w.E, w.H, w.I
    dt = DTYPES[w.dtype]
    gate = torch.empty(E, I, H, dtype=dt, device=device)
    up = torch.empty(E, I, H, dtype=dt, device=device)
    down = torch.empty(E, H, I, dtype=dt, device=device)
    for e in range(E):
        for stream, dst, shape, fan_in in ((4, gate, (I, H), H), (5, up, (I, H), H), (6, down, (H, I), I)):
            g = _torch_gen(device, w.seed, stream, e)
            v = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
            dst[e].copy_((v * (1.0 / math.sqrt(fan_in))).to(dt))
    return gate, up, down


def make_router(w: Workload, device="cpu") -> torch.Tensor:
    """Gate (router) weights [E, H] ~ N(0, 1) / sqrt(H) in the token dtype, on ``device``."""
    g = _torch_gen(device, w.seed, 7)
    v = torch.randn(w.E, w.H, generator=g, device=device, dtype=torch.float32)
    return (v * (1.0 / math.sqrt(w.H))).to(DTYPES[w.dtype])


def make_projection_inputs(w: Workload, device="cpu", special=(0, 0, 0), twins: int = 0):
    """Tokens [T, H] and router [E, H] for the fused projection, with ``special`` = counts of
    token rows per PROJECTION_SPECIAL_KINDS and ``twins`` router rows overwritten by a copy of
    a lower expert's row.  Returns ``(x, router, info)``: info maps each special kind to its
    sorted token rows and ``"twins"`` to a list of (lower expert, copy) pairs."""
    x = make_tokens(w, device)
    router = make_router(w, device)
    rng = _np_rng(w.seed, 8)
    n = sum(special)
    if n > w.T:
        raise ValueError("more special rows than tokens")
    rows = rng.permutation(w.T)[:n]
    info = {}
    at = 0
    for kind, cnt in zip(PROJECTION_SPECIAL_KINDS, special):
        r = np.sort(rows[at:at + cnt])
        at += cnt
        info[kind] = r
        for t in r:
            t = int(t)
            if kind == "zero":
                x[t].zero_()
            else:
                x[t, int(rng.integers(w.H))] = float("nan") if kind == "nan" else float("inf")
    pairs = []
    if twins:
        if 2 * twins > w.E:
            raise ValueError("more twins than expert pairs")
        perm = rng.permutation(w.E)[:2 * twins].reshape(twins, 2)
        for a, b in perm:
            lo, hi = int(min(a, b)), int(max(a, b))
            router[hi].copy_(router[lo])
            pairs.append((lo, hi))
    info["twins"] = pairs
    return x, router, info
