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


def full_oracle_forward(x, logits, k, renorm, gate, up, down):
    """The oracle's staged forward over every token: route, dispatch, the SwiGLU experts, combine.
    Only the experts that receive rows are copied to the host (ids renumbered in increasing
    order, so the dispatched row order is the same as with all E experts)."""
    ridx, rw, _ = oracle.route(logits.cpu(), k, renorm)
    E = gate.shape[0]
    used = np.unique(ridx)
    remap = np.full(E, -1, np.int64)
    remap[used] = np.arange(len(used))
    sel = torch.from_numpy(used.astype(np.int64)).to(gate.device)
    g, u, dn = gate[sel].cpu(), up[sel].cpu(), down[sel].cpu()
    say("oracle dispatch", len(used), "active experts")
    rdisp, roffs_c, rmap, _ = oracle.dispatch(remap[ridx].astype(np.uint32), x.cpu(), len(used))
    say("oracle experts", rdisp.shape[0], "rows")
    ry = oracle.experts_forward(rdisp, roffs_c, g, u, dn)
    say("oracle combine")
    rout = oracle.combine(ry, rmap, rw)
    counts = np.bincount(ridx.ravel().astype(np.int64), minlength=E)
    roffs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return ridx, rdisp, roffs, ry, rout
