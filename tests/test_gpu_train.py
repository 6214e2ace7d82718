"""GPU parity of the first-order training calls (ruDNN user guide, section 12) against the
oracle: router weights of a fixed selection and their logits gradient, combine_backward and
dispatch_backward.  Weights (FP32) and gradients within the tolerances of the forward suites
(FP32: 1e-4 relative + 1e-5; BF16/F16: 2e-2 relative with a 2e-2 RMS floor); dweights, an FP32
dot product over H, within 1e-4 relative plus 1e-6 of the sum of the absolute products (its
FP32 accumulation bound); NaN positions exactly."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_23_amd import moe
from mixture_experts_layer_23_amd.inputs import DTYPES, WORKLOADS, Workload, make_logits, make_tokens
from oracle import oracle
from parity_util import assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def _selection(T, E, k, seed, itype, invalid=0):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int64)
    for t in range(0, T, 7):  # repeated indices (gather semantics)
        idx[t, k - 1] = idx[t, 0]
    bad_rows = []
    for i in range(invalid):
        t = int(rng.integers(T))
        idx[t, int(rng.integers(k))] = E if (i % 2 == 0 or itype == "u32") else -1
        bad_rows.append(t)
    if itype == "i64":
        ti = torch.from_numpy(idx)
    else:
        ti = torch.from_numpy(idx.astype(np.int32) if itype == "i32" else idx.astype(np.uint32).view(np.int32))
    return idx, ti, sorted(set(bad_rows))


ROUTER_CASES = [
    # (T, E, k, logits dtype, scoring, renorm, scale, index type)
    (1000, 128, 8, "bf16", "softmax", True, 1.0, "u32"),
    (1000, 128, 8, "bf16", "softmax", False, 1.0, "i32"),
    (333, 64, 64, "f16", "softmax", True, 2.5, "i64"),
    (65, 1000, 7, "f32", "sigmoid", True, 2.5, "u32"),
    (257, 256, 8, "bf16", "sigmoid", False, 1.0, "i64"),
    (4096, 8, 2, "bf16", "softmax", True, 1.0, "u32"),
    (3, 5, 5, "f32", "softmax", False, 0.5, "i32"),
]


@pytest.mark.parametrize("T,E,k,dt,scoring,renorm,scale,itype", ROUTER_CASES)
def test_selected_router_weights_and_backward(T, E, k, dt, scoring, renorm, scale, itype):
    say("selected-router", T, E, k, dt, scoring, renorm, scale, itype)
    w = Workload("sr", T, 16, None, E, k, dt, dt, (renorm,), None, 800 + T + E)
    logits, _ = make_logits(w)
    idx, ti, bad = _selection(T, E, k, T + E, itype, invalid=3 if T > 10 else 0)
    g = torch.from_numpy(np.random.default_rng(1).normal(size=(T, k))).float()
    unsigned = itype == "u32"
    wg = moe.selected_router_weights(logits.to(DEV), ti.to(DEV), scoring, renorm, scale, unsigned=unsigned)
    wr, _ = oracle.selected_router_weights(logits, idx, scoring, renorm, scale)
    assert_close(wg, wr, "f32", "weights")
    dg = moe.selected_router_backward(logits.to(DEV), ti.to(DEV), g.to(DEV), scoring, renorm, scale,
                                      unsigned=unsigned)
    dr = oracle.selected_router_backward(logits, idx, g, scoring, renorm, scale)
    assert_close(dg, dr, dt, "logits gradient")
    for t in bad:
        assert torch.isnan(wg[t]).all() and torch.isnan(dg[t].float()).all()


def test_selected_router_follows_route():
    # the weights of route's own selection equal route's weights (softmax, both renorm modes)
    w = WORKLOADS["route_dispatch"].with_T(8192)
    logits, special = make_logits(w)
    lg = logits.to(DEV)
    for renorm in (True, False):
        idx, wt = moe.route(lg, w.top_k, renorm)
        sw = moe.selected_router_weights(lg, idx, "softmax", renorm, 1.0)
        nan_rows = np.concatenate([special["nan"], special["posinf"], special["all_neginf"]])
        keep = np.setdiff1d(np.arange(w.T), nan_rows)
        assert_close(sw[keep].to(torch.bfloat16), wt[keep], "bf16", "weights vs route")


def _dw_check(got, ref, dout, y, tm):
    """FP32 dot products over H: relative 1e-4 plus 1e-6 of sum |dout * y|."""
    T, k = tm.shape
    yg = y.float()[torch.from_numpy(tm.astype(np.int64)).clamp(0, y.shape[0] - 1)]  # [T, k, H]
    mag = (dout.float().unsqueeze(1) * yg).abs().sum(-1)
    g, r = got.double().cpu(), ref.double()
    fin = torch.isfinite(r)
    assert torch.equal(torch.isnan(g), torch.isnan(r))
    assert torch.all((g - r).abs()[fin] <= 1e-4 * r.abs()[fin] + 1e-6 * mag.double()[fin])


@pytest.mark.parametrize("T,k,E,H,dt,wdt", [(2000, 8, 128, 2048, "bf16", "bf16"), (513, 2, 8, 4096, "f16", "f32"),
                                            (64, 3, 8, 136, "f32", "bf16"), (1, 1, 1, 8, "bf16", "bf16")])
def test_combine_and_dispatch_backward(T, k, E, H, dt, wdt):
    say("combine/dispatch backward", T, k, E, H, dt, wdt)
    w = Workload("cb", T, H, None, E, k, dt, wdt, (True,), None, 900 + T + H)
    logits, _ = make_logits(w)
    x = make_tokens(w, DEV)
    idx, wt = moe.route(logits.to(DEV), k, True)
    d = moe.dispatch(idx, x, E)
    g = torch.Generator(device=DEV).manual_seed(T + H)
    y = torch.randn(T * k, H, generator=g, device=DEV).to(DTYPES[dt])
    dout = torch.randn(T, H, generator=g, device=DEV).to(DTYPES[dt])
    tm = d.token_map.cpu().numpy()
    dexp, dw = moe.combine_backward(y, d.token_map, wt, dout)
    rexp, rdw = oracle.combine_backward(y.cpu(), tm, wt.cpu(), dout.cpu())
    assert_close(dexp, rexp, dt, "dexpert")
    _dw_check(dw, rdw, dout.cpu(), y.cpu(), tm)
    dd = torch.randn(T * k, H, generator=g, device=DEV).to(DTYPES[dt])
    dx = moe.dispatch_backward(dd, d.token_map)
    assert_close(dx, oracle.dispatch_backward(dd.cpu(), tm), dt, "dinput")


def test_combine_and_dispatch_backward_full_size():
    w = WORKLOADS["route_dispatch"]
    say("combine/dispatch backward full", w.T, w.top_k, w.H)
    logits, special = make_logits(w)
    x = make_tokens(w, DEV)
    idx, wt = moe.route(logits.to(DEV), w.top_k, True)
    d = moe.dispatch(idx, x, w.E)
    g = torch.Generator(device=DEV).manual_seed(77)
    dout = torch.randn(w.T, w.H, generator=g, device=DEV).bfloat16()
    # identity experts: expert_output = the dispatched rows
    dexp, dw = moe.combine_backward(d.dispatched, d.token_map, wt, dout)
    tm = d.token_map.cpu().numpy()
    rexp, rdw = oracle.combine_backward(d.dispatched.cpu(), tm, wt.cpu(), dout.cpu())
    assert_close(dexp, rexp, "bf16", "dexpert")
    _dw_check(dw, rdw, dout.cpu(), d.dispatched.cpu(), tm)
    dx = moe.dispatch_backward(dexp, d.token_map)
    assert_close(dx, oracle.dispatch_backward(rexp, tm), "bf16", "dinput")
    # NaN rows of the routing carry NaN weights, hence NaN dexpert rows and dinput rows
    nan_rows = np.concatenate([special["nan"], special["posinf"], special["all_neginf"]])
    assert torch.isnan(dx[torch.from_numpy(nan_rows).to(DEV)].float()).all()


def test_invalid_map_entries():
    say("backward invalid map entries")
    T, k, H = 40, 2, 64
    g = torch.Generator(device=DEV).manual_seed(5)
    y = torch.randn(T * k, H, generator=g, device=DEV).bfloat16()
    tm = torch.from_numpy(np.random.default_rng(2).permutation(T * k).astype(np.int32).reshape(T, k)).to(DEV)
    tm[3, 1] = -1
    tm[7, 0] = T * k
    w = torch.rand(T, k, generator=g, device=DEV).bfloat16()
    dout = torch.randn(T, H, generator=g, device=DEV).bfloat16()
    dexp, dw = moe.combine_backward(y, tm, w, dout)
    assert torch.isnan(dw[[3, 7]]).all() and torch.isfinite(dw[[0, 1, 2, 4]]).all()
    rexp, rdw = oracle.combine_backward(y.cpu(), tm.cpu().numpy(), w.cpu(), dout.cpu())
    assert_close(dexp, rexp, "bf16", "dexpert")
    dx = moe.dispatch_backward(y, tm)
    assert torch.isnan(dx[[3, 7]].float()).all() and torch.isfinite(dx[[0, 1, 2]].float()).all()


# ------------------------------------------------------------------------------------------
# experts backward
# ------------------------------------------------------------------------------------------

from mixture_experts_layer_23_amd.inputs import make_experts  # noqa: E402

BWD_LAYERS = {
    "f32_tiny": Workload("eb_f32", 64, 128, 256, 8, 2, "f32", "f32", (True,), None, 1001),
    "bf16_small": Workload("eb_bf16", 300, 256, 512, 8, 2, "bf16", "bf16", (True,), None, 1002),
    "f16_ragged": Workload("eb_f16", 77, 136, 72, 33, 5, "f16", "f16", (False,), None, 1003),
    "bf16_skewed": Workload("eb_skew", 600, 264, 136, 16, 4, "bf16", "bf16", (True,), 1.5, 1004),
}


@pytest.mark.parametrize("name", list(BWD_LAYERS))
def test_experts_backward_parity(name):
    w = BWD_LAYERS[name]
    say("experts backward", name, "T", w.T, "H", w.H, "I", w.I, "E", w.E, "k", w.top_k)
    logits, _ = make_logits(w)
    x = make_tokens(w, DEV)
    gate, up, down = make_experts(w, DEV)
    ex = moe.SwiGluExperts(gate, up, down)
    idx, wt = moe.route(logits.to(DEV), w.top_k, w.renormalize[0])
    d = moe.dispatch(idx, x, w.E)
    g = torch.Generator(device=DEV).manual_seed(w.seed)
    dy = (torch.randn(d.dispatched.shape, generator=g, device=DEV) * 0.1).to(DTYPES[w.dtype])
    dx, dgate, dup, ddown = ex.backward_dispatched(d, dy)
    rdx, rdg, rdu, rdd = oracle.experts_backward(d.dispatched.cpu(), d.expert_offsets.cpu().numpy(), gate.cpu(),
                                                 up.cpu(), down.cpu(), dy.cpu())
    assert_close(dx, rdx, w.dtype, "grad_dispatched")
    # weight gradients: FP32 sums over the expert's rows of products of dtype operands
    tol = "f32" if w.dtype == "f32" else w.dtype
    assert_close(dgate, rdg, tol, "dgate")
    assert_close(dup, rdu, tol, "dup")
    assert_close(ddown, rdd, tol, "ddown")
    # repeatable bit for bit
    dx2, dg2, du2, dd2 = ex.backward_dispatched(d, dy)
    assert torch.equal(dx2, dx) and torch.equal(dg2, dgate) and torch.equal(du2, dup) and torch.equal(dd2, ddown)


def test_experts_backward_no_rows():
    w = BWD_LAYERS["bf16_small"]
    gate, up, down = make_experts(w, DEV)
    ex = moe.SwiGluExperts(gate, up, down)
    x = torch.empty(0, w.H, dtype=torch.bfloat16, device=DEV)
    offs = torch.zeros(w.E + 1, dtype=torch.int32, device=DEV)
    dx, dg, du, dd = moe.experts_backward(ex, x, offs, x)
    assert dx.shape == (0, w.H) and not dg.any() and not du.any() and not dd.any()


def test_experts_backward_mixtral_sampled():
    """Full Mixtral-shaped layer (8192 dispatched rows, H 4096, I 14336).  Exact sub-problems the
    oracle can afford: grad_dispatched of sampled rows (each row depends only on itself), and the
    weight gradients of two experts restricted to 16 intermediate units (gate/up rows, down
    columns), which depend on those units only."""
    w = WORKLOADS["mixtral"]
    say("experts backward mixtral sampled")
    logits, _ = make_logits(w)
    x = make_tokens(w, DEV)
    gate, up, down = make_experts(w, DEV)
    ex = moe.SwiGluExperts(gate, up, down)
    idx, wt = moe.route(logits.to(DEV), w.top_k, True)
    d = moe.dispatch(idx, x, w.E)
    g = torch.Generator(device=DEV).manual_seed(4)
    dy = (torch.randn(d.dispatched.shape, generator=g, device=DEV) * 0.05).bfloat16()
    dx, dgate, dup, ddown = ex.backward_dispatched(d, dy)
    torch.cuda.synchronize()
    offs = d.expert_offsets.cpu().numpy()
    rng = np.random.default_rng(11)
    rows = np.sort(rng.choice(int(offs[-1]), size=6, replace=False))
    gate_c, up_c, down_c = gate.cpu(), up.cpu(), down.cpu()
    for r in rows:
        e = int(np.searchsorted(offs, r, side="right") - 1)
        # the row alone, through its own expert only
        rdx, _, _, _ = oracle.experts_backward(d.dispatched[r:r + 1].cpu(), np.array([0, 1], np.int32),
                                               gate_c[e:e + 1], up_c[e:e + 1], down_c[e:e + 1], dy[r:r + 1].cpu())
        assert_close(dx[r:r + 1], rdx, "bf16", f"grad_dispatched row {r}")
    units = torch.from_numpy(np.sort(rng.choice(w.I, size=16, replace=False))).to(DEV)
    for e in (0, w.E - 1):
        a, b = int(offs[e]), int(offs[e + 1])
        uc = units.cpu()
        g1, u1 = gate_c[e:e + 1, uc].contiguous(), up_c[e:e + 1, uc].contiguous()
        d1 = down_c[e:e + 1][:, :, uc].contiguous()
        _, rdg, rdu, rdd = oracle.experts_backward(d.dispatched[a:b].cpu(), np.array([0, b - a], np.int32), g1, u1, d1,
                                                   dy[a:b].cpu())
        assert_close(dgate[e, units].cpu(), rdg[0], "bf16", f"dgate expert {e}")
        assert_close(dup[e, units].cpu(), rdu[0], "bf16", f"dup expert {e}")
        assert_close(ddown[e][:, units].cpu(), rdd[0], "bf16", f"ddown expert {e}")
