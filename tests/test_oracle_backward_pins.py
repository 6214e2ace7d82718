"""Pins of the oracle's first-order training functions (ruDNN user guide, section 12): FP32
weights of a fixed selection and their logits gradient, combine_backward, dispatch_backward and
the SwiGLU experts' backward.  Each is checked against something other than the oracle's own
formula: torch autograd in float64 (a library routine), central finite differences of the
oracle's (separately pinned) weights, the adjoint identity of dispatch, and closed forms."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle


def _rows(T, E, k, seed, repeats=True):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    if repeats:  # a few rows repeat an index (gather semantics)
        for t in range(0, T, 5):
            idx[t, -1] = idx[t, 0]
    return idx


def _torch_weights(x, idx, scoring, renorm, scale):
    sc = torch.softmax(x, dim=1) if scoring == "softmax" else torch.sigmoid(x)
    w = sc.gather(1, torch.from_numpy(idx).long())
    if renorm:
        w = w / w.sum(dim=1, keepdim=True)
    return w * scale


CASES = [(s, r, c) for s in ("softmax", "sigmoid") for r in (False, True) for c in (1.0, 2.5)]


@pytest.mark.parametrize("scoring,renorm,scale", CASES)
def test_router_weights_equal_torch(scoring, renorm, scale):
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(30, 16, generator=g) * 2).float()
    idx = _rows(30, 16, 4, 1)
    w, wx = oracle.selected_router_weights(x, idx, scoring, renorm, scale)
    ref = _torch_weights(x.double(), idx, scoring, renorm, scale)
    assert np.allclose(wx, ref.numpy(), rtol=1e-13, atol=0)
    assert torch.equal(w, ref.float())                      # one rounding of the exact value


@pytest.mark.parametrize("scoring,renorm,scale", CASES)
def test_router_backward_equals_autograd(scoring, renorm, scale):
    g = torch.Generator().manual_seed(6)
    x = (torch.randn(30, 16, generator=g) * 2).float()
    gw = torch.randn(30, 4, generator=g).float()
    idx = _rows(30, 16, 4, 2)
    xd = x.double().requires_grad_(True)
    (_torch_weights(xd, idx, scoring, renorm, scale) * gw.double()).sum().backward()
    got = oracle.selected_router_backward(x, idx, gw, scoring, renorm, scale)
    ref = xd.grad
    # exact zeros (unselected experts under renormalisation) come out of a cancellation on both
    # sides: an absolute floor far below every real gradient
    assert torch.allclose(got.double(), ref, rtol=2**-22, atol=1e-12)
    # with 16-bit logits the gradient is the same value rounded once to that dtype (one ulp)
    for dt, p, q in ((torch.bfloat16, 8, 2.0 ** -133), (torch.float16, 11, 2.0 ** -24)):  # q: subnormal quantum
        xl = x.to(dt)
        xd = xl.double().requires_grad_(True)
        (_torch_weights(xd, idx, scoring, renorm, scale) * gw.double()).sum().backward()
        got = oracle.selected_router_backward(xl, idx, gw, scoring, renorm, scale).double()
        assert torch.all((got - xd.grad).abs() <= 2.0 ** (1 - p) * xd.grad.abs() + q + 1e-12)


@pytest.mark.parametrize("scoring,renorm", [(s, r) for s in ("softmax", "sigmoid") for r in (False, True)])
def test_router_backward_equals_finite_differences(scoring, renorm):
    rng = np.random.default_rng(9)
    T, E, k, scale = 6, 10, 3, 1.5
    x = torch.from_numpy(rng.normal(size=(T, E))).float()
    idx = _rows(T, E, k, 3)
    gw = torch.from_numpy(rng.normal(size=(T, k))).float()
    got = oracle.selected_router_backward(x, idx, gw, scoring, renorm, scale).double()
    h = 2.0 ** -12
    for e in range(E):
        xp, xm = x.clone(), x.clone()
        xp[:, e] += h
        xm[:, e] -= h
        step = (xp[:, e].double() - xm[:, e].double()).numpy()
        _, wp = oracle.selected_router_weights(xp, idx, scoring, renorm, scale)
        _, wm = oracle.selected_router_weights(xm, idx, scoring, renorm, scale)
        fd = ((wp - wm) * gw.double().numpy()).sum(axis=1) / step
        assert np.allclose(got[:, e].numpy(), fd, rtol=1e-5, atol=1e-7), e


def test_router_closed_forms():
    x = torch.tensor([[0.3, -1.0, 2.0, 0.0]], dtype=torch.float32)
    # one expert chosen twice and renormalised: each weight is exactly scale / 2, gradient 0
    w, _ = oracle.selected_router_weights(x, [[2, 2]], "softmax", True, 3.0)
    assert w.tolist() == [[1.5, 1.5]]
    d = oracle.selected_router_backward(x, [[2, 2]], torch.tensor([[0.7, -0.2]]), "softmax", True, 3.0)
    assert torch.all(d.abs() < 1e-7)
    # sigmoid without renormalisation: d w / d x = scale * s (1 - s) at the chosen logit only
    d = oracle.selected_router_backward(x, [[1]], torch.tensor([[1.0]]), "sigmoid", False, 2.0)
    s = 1 / (1 + math.exp(1.0))
    assert d[0, 1].item() == pytest.approx(2.0 * s * (1 - s), rel=1e-7)
    assert d[0, [0, 2, 3]].abs().max().item() == 0.0
    # softmax over all experts, all chosen, renormalised: the weights are the softmax itself
    w, wx = oracle.selected_router_weights(x, [[0, 1, 2, 3]], "softmax", True, 1.0)
    assert np.allclose(wx, torch.softmax(x.double(), 1).numpy(), rtol=1e-15)


def test_router_invalid_index_gives_a_nan_row():
    x = torch.randn(4, 8).float()
    for bad in (8, -1, 1 << 40):
        idx = np.array([[0, 1], [2, bad], [3, 4], [5, 6]])
        w, _ = oracle.selected_router_weights(x, idx, "softmax", True, 1.0)
        d = oracle.selected_router_backward(x, idx, torch.ones(4, 2), "sigmoid", False, 1.0)
        assert torch.isnan(w[1]).all() and torch.isnan(d[1]).all()
        assert torch.isfinite(w[[0, 2, 3]]).all() and torch.isfinite(d[[0, 2, 3]]).all()


def _perm_map(T, k, seed):
    return np.random.default_rng(seed).permutation(T * k).astype(np.int32).reshape(T, k)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_combine_backward_equals_autograd(dt):
    g = torch.Generator().manual_seed(4)
    T, k, H = 12, 3, 20
    y = torch.randn(T * k, H, generator=g).to(dt)
    w = torch.rand(T, k, generator=g).to(dt)
    dout = torch.randn(T, H, generator=g).to(dt)
    tm = _perm_map(T, k, 1)
    yd = y.double().requires_grad_(True)
    wd = w.double().requires_grad_(True)
    out = (wd.unsqueeze(-1) * yd[torch.from_numpy(tm).long()]).sum(dim=1)
    (out * dout.double()).sum().backward()
    dexp, dw = oracle.combine_backward(y, tm, w, dout)
    assert torch.equal(dexp.view(torch.int16) if dt != torch.float32 else dexp,
                       yd.grad.to(dt).view(torch.int16) if dt != torch.float32 else yd.grad.to(dt))
    assert torch.equal(dw, wd.grad.float())


def test_combine_backward_invalid_entry():
    T, k, H = 3, 2, 4
    y = torch.randn(T * k, H)
    w = torch.rand(T, k)
    tm = _perm_map(T, k, 2)
    tm[1, 1] = -1
    dexp, dw = oracle.combine_backward(y, tm, w, torch.ones(T, H))
    assert torch.isnan(dw[1]).all() and torch.isfinite(dw[[0, 2]]).all()
    assert torch.allclose(dexp[int(tm[1, 0])], w[1, 0].expand(H))   # the valid entry still gets w * dout


def test_dispatch_backward_is_the_adjoint_of_dispatch():
    rng = np.random.default_rng(3)
    T, k, E, H = 40, 3, 7, 9
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.uint32)
    x = torch.from_numpy(rng.normal(size=(T, H))).float()
    disp, offs, tm, _ = oracle.dispatch(idx, x, E)
    d = torch.from_numpy(rng.normal(size=(T * k, H))).float()
    dx = oracle.dispatch_backward(d, tm)
    lhs = float((disp.double() * d.double()).sum())
    rhs = float((x.double() * dx.double()).sum())
    assert lhs == pytest.approx(rhs, rel=1e-6)
    # top_k = 1 with a permutation map: the backward is the inverse permutation, bit for bit
    tm1 = _perm_map(T, 1, 5)
    d1 = torch.from_numpy(rng.normal(size=(T, H))).float()
    assert torch.equal(oracle.dispatch_backward(d1, tm1), d1[torch.from_numpy(tm1[:, 0]).long()])
    tm[0, 0] = T * k  # outside the rows: NaN row
    assert torch.isnan(oracle.dispatch_backward(d, tm)[0]).all()


def _torch_experts(x, offs, gate, up, down):
    outs = []
    for e in range(gate.shape[0]):
        xe = x[offs[e]:offs[e + 1]]
        gg = xe @ gate[e].T
        uu = xe @ up[e].T
        h = torch.nn.functional.silu(gg) * uu
        outs.append(h @ down[e].T)
    return torch.cat(outs, dim=0)


def test_experts_backward_equals_autograd():
    g = torch.Generator().manual_seed(12)
    E, H, I = 3, 24, 16
    offs = np.array([0, 7, 7, 19], np.int32)  # an empty expert in the middle
    rows = int(offs[-1])
    x = torch.randn(rows, H, generator=g)
    gate = torch.randn(E, I, H, generator=g) / math.sqrt(H)
    up = torch.randn(E, I, H, generator=g) / math.sqrt(H)
    down = torch.randn(E, H, I, generator=g) / math.sqrt(I)
    dy = torch.randn(rows, H, generator=g)
    leaves = [t.double().requires_grad_(True) for t in (x, gate, up, down)]
    (_torch_experts(leaves[0], offs, *leaves[1:]) * dy.double()).sum().backward()
    dx, dg, du, dd = oracle.experts_backward(x, offs, gate, up, down, dy)
    # FP32 storage of h, dg, du and the outputs: a few FP32 ulps of the float64 gradients
    for got, ref in ((dx, leaves[0].grad), (dg, leaves[1].grad), (du, leaves[2].grad), (dd, leaves[3].grad)):
        scale = ref.abs().max().item()
        assert torch.allclose(got.double(), ref, rtol=1e-5, atol=1e-6 * scale)
    assert torch.all(dg[1] == 0) and torch.all(du[1] == 0) and torch.all(dd[1] == 0)   # no rows, no gradient


def test_experts_backward_single_expert_is_a_dense_swiglu_gradient():
    # one expert, bf16 storage: the gradient of a dense SwiGLU MLP from torch.nn.functional in float64,
    # within the bf16 storage of h, dg and du
    g = torch.Generator().manual_seed(13)
    H, I, n = 32, 48, 10
    x = torch.randn(n, H, generator=g).bfloat16()
    gate = (torch.randn(1, I, H, generator=g) / math.sqrt(H)).bfloat16()
    up = (torch.randn(1, I, H, generator=g) / math.sqrt(H)).bfloat16()
    down = (torch.randn(1, H, I, generator=g) / math.sqrt(I)).bfloat16()
    dy = torch.randn(n, H, generator=g).bfloat16()
    leaves = [t.double().requires_grad_(True) for t in (x, gate, up, down)]
    y = torch.nn.functional.linear(torch.nn.functional.silu(torch.nn.functional.linear(leaves[0], leaves[1][0])) *
                                   torch.nn.functional.linear(leaves[0], leaves[2][0]), leaves[3][0])
    (y * dy.double()).sum().backward()
    dx, dg, du, dd = oracle.experts_backward(x, np.array([0, n], np.int32), gate, up, down, dy)
    for got, ref in ((dx, leaves[0].grad), (dg, leaves[1].grad), (du, leaves[2].grad), (dd, leaves[3].grad)):
        err = (got.double() - ref).norm() / ref.norm()
        assert err < 2e-2, err
