"""Pins of the oracle's group-limited sigmoid routing (ruDNN user guide, section 10) against
hand-derived cases, closed forms and invariants computed independently of the oracle.

CPU only; every expected value comes from the pages' definition, elementary mathematics, numpy
or scipy, never from the oracle itself or the GPU library."""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _num(v):
    if isinstance(v, list):
        return [_num(x) for x in v]
    if isinstance(v, str):
        return float(v)
    return v


def _cases():
    with open(os.path.join(HERE, "golden", "sigmoid_hand_cases.json")) as f:
        return json.load(f)["sigmoid_grouped"]


def _sig(x):
    if x == math.inf:
        return 1.0
    if x == -math.inf:
        return 0.0
    return 1.0 / (1.0 + math.exp(-x))


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_cases(case):
    lg = torch.tensor(_num(case["logits"]), dtype=torch.float64).to(DT[case["dtype"]])
    bias = None if case["bias"] is None else torch.tensor(_num(case["bias"]), dtype=torch.float32)
    idx, w, wx = oracle.route_sigmoid_grouped(lg, bias, case["top_k"], case["groups"], case["selected_groups"],
                                              case["group_top_two"], case["renormalize"], case["scale"])
    assert idx.tolist() == case["indices"]
    if case.get("nan_row"):
        assert np.isnan(wx).all() and torch.isnan(w.float()).all()
        return
    x = lg.double().tolist()
    for t, row in enumerate(case["indices"]):
        s = [_sig(x[t][e]) for e in row]
        den = sum(s) if case["renormalize"] else 1.0
        expect = [case["scale"] * v / den for v in s]
        np.testing.assert_allclose(wx[t], expect, rtol=1e-12, atol=1e-15)


def _random_case(rng, T, E, groups, dtype=torch.float32, bias_scale=0.1):
    x = torch.from_numpy(rng.standard_normal((T, E))).to(dtype)
    b = torch.from_numpy((rng.standard_normal(E) * bias_scale).astype(np.float32))
    return x, b


def _corrected(x, b):
    # FP32 decision values: sigmoid rounded to FP32, plus the FP32 bias in FP32
    s32 = expit(x.double().numpy()).astype(np.float32)
    return s32 if b is None else (s32 + b.numpy()).astype(np.float32)


def test_single_group_no_bias_is_plain_topk_by_logit():
    rng = np.random.default_rng(1)
    x, _ = _random_case(rng, 200, 32, 1)
    idx, w, wx = oracle.route_sigmoid_grouped(x, None, 5, 1, 1, False, False, 1.0)
    ref = np.argsort(-x.double().numpy(), axis=1, kind="stable")[:, :5]
    assert (idx == ref).all()
    np.testing.assert_allclose(wx, expit(np.take_along_axis(x.double().numpy(), ref, 1)), rtol=1e-12)


def test_all_groups_selected_is_topk_by_corrected_score():
    rng = np.random.default_rng(2)
    x, b = _random_case(rng, 300, 64, 8)
    idx, _, _ = oracle.route_sigmoid_grouped(x, b, 6, 8, 8, True, True, 1.0)
    c = _corrected(x, b)
    ref = np.argsort(-c, axis=1, kind="stable")[:, :6]
    assert (idx == ref).all()


@pytest.mark.parametrize("groups,sel,top_two,k", [(8, 4, True, 8), (8, 3, False, 5), (4, 1, True, 2), (16, 5, False, 9)])
def test_group_invariants(groups, sel, top_two, k):
    rng = np.random.default_rng(3 + groups + sel)
    T, E = 250, 64
    x, b = _random_case(rng, T, E, groups)
    idx, w, wx = oracle.route_sigmoid_grouped(x, b, k, groups, sel, top_two, True, 1.7)
    c = _corrected(x, b)
    per = E // groups
    cg = c.reshape(T, groups, per)
    top = -np.sort(-cg, axis=2)
    gscore = top[:, :, 0] if not top_two else (top[:, :, 0] + top[:, :, 1]).astype(np.float32)
    chosen_groups = np.argsort(-gscore, axis=1, kind="stable")[:, :sel]
    for t in range(T):
        eligible = np.concatenate([np.arange(g * per, (g + 1) * per) for g in sorted(chosen_groups[t])])
        assert set(idx[t] // per) <= set(chosen_groups[t])          # only chosen groups
        best = eligible[np.argsort(-c[t, eligible], kind="stable")[:k]]
        assert idx[t].tolist() == best.tolist()                      # the k best of them, in order
    np.testing.assert_allclose(wx.sum(1), 1.7, rtol=1e-12)           # renormalised, then scaled
    s = expit(np.take_along_axis(x.double().numpy(), idx.astype(np.int64), 1))
    np.testing.assert_allclose(wx, 1.7 * s / s.sum(1, keepdims=True), rtol=1e-12)   # original sigmoid


def test_bias_shift_changes_nothing():
    rng = np.random.default_rng(4)
    x, b = _random_case(rng, 200, 32, 4)
    a = oracle.route_sigmoid_grouped(x, b, 4, 4, 2, True, False, 1.0)
    shifted = b + 0.25  # exactly representable shift keeps FP32 ties and orders (values stay well apart)
    z = oracle.route_sigmoid_grouped(x, shifted, 4, 4, 2, True, False, 1.0)
    assert (a[0] == z[0]).all()
    np.testing.assert_allclose(a[2], z[2], rtol=0, atol=0)


def test_bias_never_enters_the_weights():
    rng = np.random.default_rng(5)
    x, _ = _random_case(rng, 100, 16, 1)
    big = torch.zeros(16, dtype=torch.float32)
    big[7] = 100.0  # expert 7 always chosen first
    idx, _, wx = oracle.route_sigmoid_grouped(x, big, 3, 1, 1, False, False, 3.0)
    assert (idx[:, 0] == 7).all()
    np.testing.assert_allclose(wx[:, 0], 3.0 * expit(x.double().numpy()[:, 7]), rtol=1e-12)


def test_argument_checks():
    x = torch.zeros(2, 8)
    for args in [(3, 3, 1, False), (2, 4, 5, False), (9, 2, 2, False), (5, 4, 2, False), (1, 8, 1, True)]:
        k, groups, sel, top_two = args
        with pytest.raises(ValueError):
            oracle.route_sigmoid_grouped(x, None, k, groups, sel, top_two, False, 1.0)
    with pytest.raises(ValueError):
        oracle.route_sigmoid_grouped(x, None, 1, 1, 1, False, False, 0.0)
