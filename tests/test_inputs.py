"""The seeded input generator: determinism, separation of distinct logits, special rows, skew."""
import math

import numpy as np
import pytest
import torch

from mixture_experts_layer_23_amd.inputs import WORKLOADS, Workload, make_experts, make_logits, make_tokens


def _nan_like(special):
    return np.concatenate([special["nan"], special["posinf"], special["all_neginf"]])


@pytest.mark.parametrize("name", ["tiny", "skewed", "decode", "mixtral"])
def test_same_seed_same_bytes(name):
    w = WORKLOADS[name].with_T(min(WORKLOADS[name].T, 512))
    a, sa = make_logits(w)
    b, sb = make_logits(w)
    assert torch.equal(a.view(torch.int16) if a.element_size() == 2 else a.view(torch.int32),
                       b.view(torch.int16) if b.element_size() == 2 else b.view(torch.int32))
    assert all(np.array_equal(sa[k], sb[k]) for k in sa)
    small = w.replace(H=32, I=16 if w.I else None, E=min(w.E, 8))
    assert torch.equal(make_tokens(small), make_tokens(small))
    if small.I:
        for x, y in zip(make_experts(small), make_experts(small)):
            assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["tiny", "route_dispatch", "skewed", "decode"])
def test_distinct_logits_are_separated(name):
    w = WORKLOADS[name].with_T(min(WORKLOADS[name].T, 4096))
    logits, special = make_logits(w)
    v = logits.double().numpy()
    deliberate = set(np.concatenate(list(special.values())).tolist()) if special else set()
    ordinary = np.array([t for t in range(w.T) if t not in deliberate])
    gaps = np.diff(np.sort(v[ordinary], axis=1), axis=1)
    assert gaps.min() >= 1e-3
    # logits never sit more than 80 below the row max (no fp32 exp underflow)
    fin = v[ordinary]
    assert (fin.max(1, keepdims=True) - fin).max() < 80


def test_special_rows_match_their_kind():
    w = WORKLOADS["route_dispatch"].with_T(8192)
    logits, sp = make_logits(w)
    v = logits.double().numpy()
    k = w.top_k
    assert sum(len(r) for r in sp.values()) == sum(w.special)
    for r in sp["uniform"]:
        assert np.all(v[r] == v[r][0])
    for r in sp["boundary_tie"]:
        s = np.sort(v[r])[::-1]
        assert s[k - 1] == s[k]
    for r in sp["top_tie"]:
        assert np.sum(v[r] == v[r].max()) == 2
    for r in sp["partial_neginf"]:
        assert 1 <= np.isfinite(v[r]).sum() < k and np.all(v[r][~np.isfinite(v[r])] == -np.inf)
    for r in sp["nan"]:
        assert np.isnan(v[r]).sum() == 1
    for r in sp["posinf"]:
        assert np.sum(v[r] == np.inf) == 1
    for r in sp["all_neginf"]:
        assert np.all(v[r] == -np.inf)


def test_full_size_special_row_counts():
    w = WORKLOADS["route_dispatch"]
    assert sum(w.special[:4]) == 655 and sum(w.special[4:]) == 328  # 1% and 0.5% of 65536
    t = WORKLOADS["tiny"]
    assert sum(t.special[:4]) == 4 and sum(t.special[4:]) == 3


def test_weight_scale_is_one_over_sqrt_fan_in():
    w = WORKLOADS["skewed"].replace(E=2, H=512, I=384, dtype="f32")
    gate, up, down = make_experts(w)
    assert abs(gate.std().item() * np.sqrt(512) - 1) < 0.02
    assert abs(up.std().item() * np.sqrt(512) - 1) < 0.02
    assert abs(down.std().item() * np.sqrt(384) - 1) < 0.02
    assert not torch.equal(gate, up)


def test_sigmoid_inputs_deterministic_and_structured():
    from mixture_experts_layer_23_amd.inputs import SIGMOID_SPECIAL_KINDS, make_sigmoid_logits
    w = WORKLOADS["sigmoid_route"].with_T(4096)
    a, ba, sa = make_sigmoid_logits(w)
    b, bb, sb = make_sigmoid_logits(w)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(ba, bb)
    assert ba.dtype == torch.float32 and ba.shape == (w.E,)
    G = w.sigmoid.groups
    per = w.E // G
    bias = ba.numpy()
    for g in range(G):                                   # bias twins inside each group
        for i in range(per // 4):
            assert bias[g * per + 2 * i] == bias[g * per + 2 * i + 1]
    assert np.array_equal(bias[(G - 1) * per:], bias[(G - 2) * per:(G - 1) * per])   # group twins
    x = a.float().numpy()
    assert set(sa) == set(SIGMOID_SPECIAL_KINDS)
    for t in sa["expert_tie"]:
        row = x[t]
        top = np.nonzero(row == np.nanmax(row))[0]
        assert len(top) >= 2 and any(e % per % 2 == 0 and e + 1 in top and e % per < per // 2 for e in top)
    for t in sa["group_tie"]:
        assert np.array_equal(x[t][(G - 1) * per:], x[t][(G - 2) * per:(G - 1) * per])
    for t in sa["nan"]:
        assert np.isnan(x[t]).sum() == 1
    for t in sa["posinf"]:
        assert (x[t] == np.inf).sum() == 1
    for t in sa["neginf"]:
        assert (x[t] == -np.inf).sum() == 1
    ordinary = np.setdiff1d(np.arange(w.T), np.concatenate(list(sa.values())))
    d = np.diff(np.sort(x[ordinary], axis=1), axis=1)
    assert d.min() >= 1e-3                               # separated logits elsewhere


def test_projection_inputs_deterministic_and_structured():
    from mixture_experts_layer_23_amd.inputs import PROJECTION_SPECIAL_KINDS, make_projection_inputs, make_router
    w = Workload("proj", 200, 64, None, 16, 2, "bf16", "bf16", (True,), None, 77)
    r = make_router(w)
    assert r.shape == (16, 64) and r.dtype == torch.bfloat16
    assert abs(float(r.float().std()) * math.sqrt(64) - 1.0) < 0.1      # N(0, 1) / sqrt(H)
    x1, r1, i1 = make_projection_inputs(w, special=(2, 3, 4), twins=3)
    x2, r2, i2 = make_projection_inputs(w, special=(2, 3, 4), twins=3)
    assert torch.equal(x1.view(torch.int16), x2.view(torch.int16)) and torch.equal(r1.view(torch.int16),
                                                                                 r2.view(torch.int16))
    assert [len(i1[k]) for k in PROJECTION_SPECIAL_KINDS] == [2, 3, 4]
    rows = np.concatenate([i1[k] for k in PROJECTION_SPECIAL_KINDS])
    assert len(set(rows.tolist())) == 9                                  # distinct rows
    xf = x1.float()
    for t in i1["nan"]:
        assert int(torch.isnan(xf[t]).sum()) == 1
    for t in i1["posinf"]:
        assert int((xf[t] == float("inf")).sum()) == 1
    for t in i1["zero"]:
        assert (xf[t] == 0).all()
    assert len(i1["twins"]) == 3
    for a, b in i1["twins"]:
        assert a < b and torch.equal(r1[a].view(torch.int16), r1[b].view(torch.int16))
    ordinary = np.setdiff1d(np.arange(w.T), rows)
    assert torch.isfinite(xf[torch.from_numpy(ordinary)]).all()
