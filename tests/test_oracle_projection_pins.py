"""Pins of the oracle's router projection + routing (the gate projection that the ruDNN user
guide, section 5, leaves to the caller, followed by the section 4 routing) against numpy,
closed forms and invariants computed independently of the oracle."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle

DTS = [torch.bfloat16, torch.float16, torch.float32]


@pytest.mark.parametrize("dt", DTS)
def test_projection_is_one_rounding_of_the_float64_product(dt):
    g = torch.Generator().manual_seed(11)
    x = torch.randn(37, 200, generator=g).to(dt)
    W = (torch.randn(12, 200, generator=g) / 14).to(dt)
    ref = torch.from_numpy(x.double().numpy() @ W.double().numpy().T).to(dt)   # numpy matmul, one rounding
    got = oracle.project(x, W)
    assert torch.equal(got.view(torch.int16) if dt != torch.float32 else got, ref.view(torch.int16) if dt != torch.float32 else ref)


def test_route_projected_routes_the_rounded_logits():
    g = torch.Generator().manual_seed(12)
    x = torch.randn(64, 96, generator=g).bfloat16()
    W = (torch.randn(16, 96, generator=g) / 10).bfloat16()
    idx, w, lg = oracle.route_projected(x, W, 4, True)
    lg_np = torch.from_numpy(x.double().numpy() @ W.double().numpy().T).bfloat16()
    assert torch.equal(lg.view(torch.int16), lg_np.view(torch.int16))
    order = np.argsort(-lg_np.double().numpy(), axis=1, kind="stable")[:, :4]
    assert (idx == order).all()
    p = torch.softmax(lg_np.double(), dim=1).numpy()
    sel = np.take_along_axis(p, order, 1)
    np.testing.assert_allclose(w.double().numpy(), sel / sel.sum(1, keepdims=True), rtol=8e-3)


def test_zero_router_gives_uniform_rows():
    x = torch.randn(10, 32).bfloat16()
    W = torch.zeros(8, 32).bfloat16()
    idx, w, lg = oracle.route_projected(x, W, 3, False)
    assert (lg.float() == 0).all()
    assert (idx == np.arange(3)).all()                        # full tie: lower ids first
    assert torch.allclose(w.float(), torch.full((10, 3), 1 / 8), rtol=0, atol=1e-3)
    _, wr, _ = oracle.route_projected(x, W, 3, True)
    assert torch.allclose(wr.float(), torch.full((10, 3), 1 / 3), rtol=0, atol=2e-3)


def test_doubling_the_router_keeps_the_selection():
    g = torch.Generator().manual_seed(13)
    x = torch.randn(50, 64, generator=g).float()
    W = torch.randn(10, 64, generator=g).float() / 8
    a = oracle.route_projected(x, W, 3, True)
    b = oracle.route_projected(x, 2 * W, 3, True)
    assert (a[0] == b[0]).all()
    assert torch.equal(b[2], 2 * a[2])                        # exact: doubling commutes with rounding


def test_single_expert():
    x = torch.randn(6, 16)
    W = torch.randn(1, 16)
    for renorm in (True, False):
        idx, w, _ = oracle.route_projected(x, W, 1, renorm)
        assert (idx == 0).all() and torch.equal(w, torch.ones(6, 1))


def test_hand_case():
    # logits (1, 2, 3): top-2 are experts 2 and 1; softmax weights e^3/S, e^2/S with S = e + e^2 + e^3
    x = torch.tensor([[1.0, 2.0]])
    W = torch.tensor([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    idx, w, lg = oracle.route_projected(x, W, 2, False)
    assert lg.tolist() == [[1.0, 2.0, 3.0]] and idx.tolist() == [[2, 1]]
    S = math.e + math.e ** 2 + math.e ** 3
    np.testing.assert_allclose(w[0].double().numpy(), [math.e ** 3 / S, math.e ** 2 / S], rtol=1e-6)
    _, wr, _ = oracle.route_projected(x, W, 2, True)
    np.testing.assert_allclose(wr[0].double().numpy(), [math.e / (1 + math.e), 1 / (1 + math.e)], rtol=1e-6)
