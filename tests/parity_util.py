"""Helpers shared by the GPU parity tests: the comparison rule and case logging."""
import sys

import numpy as np
import torch

from oracle import oracle


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def assert_close(got: torch.Tensor, ref: torch.Tensor, dt: str, what: str = ""):
    """FP32: |a - r| <= 1e-4 |r| + 1e-5; BF16/F16: |a - r| <= 2e-2 |r| + 2e-2 rms(r) over the
    finite reference elements; NaN positions and infinities must match exactly."""
    g = got.detach().double().cpu()
    r = ref.detach().double().cpu()
    assert g.shape == r.shape, what
    gn, rn = torch.isnan(g), torch.isnan(r)
    assert torch.equal(gn, rn), f"{what}: NaN positions differ ({int((gn != rn).sum())} elements)"
    inf = torch.isinf(r)
    assert torch.equal(g[inf], r[inf]), f"{what}: infinities differ"
    fin = torch.isfinite(r)
    if not fin.any():
        return
    d = (g - r).abs()[fin]
    ra = r.abs()[fin]
    if dt == "f32":
        bound = 1e-4 * ra + 1e-5
    else:
        rms = r[fin].pow(2).mean().sqrt()
        bound = 2e-2 * ra + 2e-2 * rms
    bad = d > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())}/{d.numel()} elements out of tolerance; "
                           f"max abs err {d.max():.3g}, max rel {(d / ra.clamp_min(1e-30)).max():.3g}")


def sampled_oracle_forward(x, logits, rows, k, renorm, gate, up, down):
    """The oracle's forward on the given tokens only: route, each selected expert on the
    token's row (only the experts used are copied to the host), combine."""
    xs, ls = x[rows].cpu(), logits[rows].cpu()
    ridx, rw, _ = oracle.route(ls, k, renorm)
    used = np.unique(ridx)
    remap = {int(e): i for i, e in enumerate(used)}
    sel = torch.from_numpy(used.astype(np.int64)).to(gate.device)
    g, u, dn = gate[sel].cpu(), up[sel].cpu(), down[sel].cpu()
    n = len(rows)
    order = np.argsort(ridx.ravel(), kind="stable")  # group rows by expert
    xr = xs.repeat_interleave(k, 0)[torch.from_numpy(order)]
    eor = np.array([remap[int(e)] for e in ridx.ravel()[order]], np.int32)
    yr = oracle.expert_rows(xr, eor, g, u, dn)
    y = torch.empty_like(yr)
    y[torch.from_numpy(order)] = yr
    tmap = np.arange(n * k, dtype=np.int32).reshape(n, k)
    return oracle.combine(y, tmap, rw)
