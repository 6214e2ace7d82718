"""Helpers shared by the GPU parity tests: the comparison rule and case logging."""
import sys

import torch


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
