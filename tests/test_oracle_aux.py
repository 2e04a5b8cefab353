"""Pins for the oracle's routing auxiliary loss (CPU only): library routines for the
textbook cases, finite differences for the gradient, closed forms and edge cases."""
import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle import msa_oracle as O

EPS = 1e-6


def _case(seed, B=4, N=9):
    rng = np.random.default_rng(seed)
    return rng.uniform(-1, 1, size=(B, N)), rng.random((B, N))


def test_bce_matches_torch_bce_with_logits():
    S, Y = _case(1)
    for tau in (1.0, 0.05):
        loss, _ = O.route_aux_loss(O.AUX_BCE, S, Y, tau)
        ref = F.binary_cross_entropy_with_logits(torch.tensor(S / tau), torch.tensor(Y), reduction="none")
        assert np.allclose(loss, ref.mean(dim=1).numpy(), rtol=1e-13, atol=1e-13)


def test_infonce_with_one_positive_is_cross_entropy():
    S, _ = _case(2)
    pos = np.array([0, 3, 8, 5])
    Y = np.zeros_like(S)
    Y[np.arange(4), pos] = 1.0
    for tau in (1.0, 0.07):
        loss, _ = O.route_aux_loss(O.AUX_INFONCE, S, Y, tau)
        ref = F.cross_entropy(torch.tensor(S / tau), torch.tensor(pos), reduction="none")
        assert np.allclose(loss, ref.numpy(), rtol=1e-13, atol=1e-13)


def test_gradient_matches_finite_differences():
    S, Y = _case(3)
    Ybin = (Y > 0.6).astype(float)
    Ybin[:, 0] = 1.0                                   # every query has a positive
    for kind, labels in ((O.AUX_BCE, Y), (O.AUX_INFONCE, Ybin), (O.AUX_INFONCE, Y)):
        for tau in (1.0, 0.1):
            _, dD = O.route_aux_loss(kind, S, labels, tau)
            for idx in np.ndindex(S.shape):
                sp, sm = S.copy(), S.copy()
                sp[idx] += EPS
                sm[idx] -= EPS
                fd = (O.route_aux_loss(kind, sp, labels, tau)[0].mean()
                      - O.route_aux_loss(kind, sm, labels, tau)[0].mean()) / (2 * EPS)
                assert abs(fd - dD[idx]) < 1e-7, (kind, tau, idx)


def test_closed_forms():
    S = np.zeros((2, 6))
    Y = np.random.default_rng(4).random((2, 6))
    loss, dD = O.route_aux_loss(O.AUX_BCE, S, Y, 1.0)
    assert np.allclose(loss, math.log(2.0))            # softplus(0) = log 2 whatever y is
    assert np.allclose(dD, (0.5 - Y) / 6 / 2)
    Yp = np.zeros((2, 6))
    Yp[0, :2] = 1.0                                     # 2 positives of 6: loss log 3
    Yp[1, 5] = 1.0                                      # 1 of 6: log 6
    loss, dD = O.route_aux_loss(O.AUX_INFONCE, S + 0.3, Yp, 0.5)
    assert np.allclose(loss, [math.log(3.0), math.log(6.0)])
    assert np.allclose(dD.sum(axis=1), 0.0, atol=1e-15)  # softmax and positive shares both sum to 1


def test_extreme_logits_stay_finite():
    S = np.array([[1000.0, -1000.0, 0.0]])
    loss, dD = O.route_aux_loss(O.AUX_BCE, S, np.array([[1.0, 1.0, 0.0]]), 1.0)
    assert np.isclose(loss[0], (0.0 + 1000.0 + math.log(2.0)) / 3)
    assert np.allclose(dD[0], [0.0, -1 / 3, 0.5 / 3])
    loss, dD = O.route_aux_loss(O.AUX_INFONCE, S, np.array([[0.0, 1.0, 0.0]]), 1.0)
    assert np.isclose(loss[0], 2000.0) and np.all(np.isfinite(dD))


def test_skipped_queries():
    S = np.array([[0.2, 0.1, -0.3], [-np.inf] * 3, [0.5, 0.4, 0.1]])
    Y = np.array([[1.0, 0.0, 0.0], [1.0, 0.0, 0.0], [0.0, 0.0, 0.0]])
    loss, dD = O.route_aux_loss(O.AUX_INFONCE, S, Y, 1.0)
    assert loss[1] == 0 and loss[2] == 0 and not dD[1:].any()   # empty query; no positive
    assert loss[0] > 0 and dD[0].any()
    loss, dD = O.route_aux_loss(O.AUX_BCE, S, Y, 1.0)
    assert loss[1] == 0 and not dD[1].any() and loss[2] > 0
