"""Pins of the oracle's forward (selected-token log-prob, LSE, tile merge).

Every check compares the oracle with something other than itself: pure-Python
brute force with math.fsum, torch's cross_entropy / logsumexp in fp64, closed
forms and invariants.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import f32_to_bf16_bits

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _tiny(seed, N, D, V, Vr, dtype, inv_tau=1.0):
    g = np.random.default_rng(seed)
    H = g.standard_normal((N, D)).astype(np.float32)
    W = (g.standard_normal((Vr, D)) * 0.3).astype(np.float32)
    if dtype == "bf16":
        H, W = f32_to_bf16_bits(H), f32_to_bf16_bits(W)
        if Vr > V:
            W[V:] = 0x7FC0
    elif Vr > V:
        W[V:] = np.nan
    y = g.integers(0, V, N)
    mask = (g.random(N) > 0.25).astype(np.uint8)
    return H, W, y, mask


def _brute(H64, W64, y, active, V, inv_tau):
    """Pure-Python loops: z = sum_d H W * inv_tau, lse = max + log fsum exp."""
    N, D = H64.shape
    logp, lse = [], []
    for t in range(N):
        z = [math.fsum(H64[t, d] * W64[v, d] for d in range(D)) * inv_tau for v in range(V)]
        m = max(z)
        l = m + math.log(math.fsum(math.exp(x - m) for x in z))
        lse.append(l)
        logp.append(z[y[t]] - l if active[t] else 0.0)
    return np.array(logp), np.array(lse)


@pytest.mark.parametrize("V,Vr,dtype,inv_tau", [(1, 1, "f32", 1.0), (7, 9, "bf16", 1.0),
                                                 (257, 257, "f32", 1.0 / 0.7),
                                                 (257, 260, "bf16", 2.0), (33, 64, "f32", 0.5)])
def test_forward_brute_force(V, Vr, dtype, inv_tau):
    H, W, y, mask = _tiny(V * 31 + Vr, 6, 5, V, Vr, dtype, inv_tau)
    act = oracle.active_tokens(y, mask, -100)
    logp, lse = oracle.forward(H, W, y, act, V, inv_tau, dtype)
    bl, bs = _brute(oracle.widen(H, dtype), oracle.widen(W, dtype), y, act, V, inv_tau)
    assert np.all(np.isfinite(lse)), "padded (NaN) rows leaked into the LSE"
    np.testing.assert_allclose(lse, bs, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(logp, bl, rtol=1e-12, atol=1e-12)
    assert np.all(logp[~act] == 0.0)


def test_forward_matches_torch_cross_entropy():
    H, W, y, mask = _tiny(5, 40, 16, 300, 300, "f32")
    act = oracle.active_tokens(y, mask, -100)
    logp, lse = oracle.forward(H, W, y, act, 300, 1.3, "f32")
    z = torch.from_numpy(H.astype(np.float64)) @ torch.from_numpy(W.astype(np.float64)).T * 1.3
    ce = torch.nn.functional.cross_entropy(z, torch.from_numpy(y), reduction="none").numpy()
    np.testing.assert_allclose(-logp[act], ce[act], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(z, 1).numpy(), rtol=1e-12)


def test_ignore_index_mode():
    H, W, y, _ = _tiny(9, 20, 8, 50, 50, "f32")
    y = y.copy()
    y[[2, 5, 11]] = -100
    act = oracle.active_tokens(y, None, -100)
    assert act.sum() == 17 and not act[[2, 5, 11]].any()
    logp, _ = oracle.forward(H, W, y, act, 50, 1.0, "f32")
    assert np.all(logp[[2, 5, 11]] == 0)
    # an explicit mask alone decides, whatever the target holds
    m = np.ones(20, np.uint8)
    assert oracle.active_tokens(y, m, -100).all()


def test_forward_invariants():
    H, W, y, mask = _tiny(11, 30, 12, 400, 400, "bf16")
    act = np.ones(30, bool)
    logp, lse = oracle.forward(H, W, y, act, 400, 1.0, "bf16")
    z = oracle.logits_rows(oracle.widen(H, "bf16"), oracle.widen(W, "bf16"), 400, 1.0)
    assert np.all(logp <= 0)
    assert np.all(lse >= z.max(1))
    assert np.all(lse <= z.max(1) + math.log(400) + 1e-12)
    p = np.exp(z - lse[:, None])
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=1e-13)


def test_uniform_logits_closed_form():
    """Zero weights give z = 0 everywhere: lse = ln V and logp = -ln V exactly."""
    V = 151
    H = np.ones((3, 8), np.float32)
    W = np.zeros((V, 8), np.float32)
    y = np.array([0, 75, 150])
    logp, lse = oracle.forward(H, W, y, np.ones(3, bool), V, 1.0, "f32")
    np.testing.assert_allclose(lse, math.log(V), rtol=1e-15)
    np.testing.assert_allclose(logp, -math.log(V), rtol=1e-15)


def test_dominant_logit_closed_form():
    """One logit b above V-1 zeros: lse = b + ln(1 + (V-1) e^-b)."""
    V, b = 10, 3.0
    H = np.array([[1.0, 0.0]], np.float32)
    W = np.zeros((V, 2), np.float32)
    W[4, 0] = b
    logp, lse = oracle.forward(H, W, np.array([4]), np.ones(1, bool), V, 1.0, "f32")
    assert lse[0] == pytest.approx(b + math.log1p((V - 1) * math.exp(-b)), rel=1e-15)
    assert logp[0] == pytest.approx(-math.log1p((V - 1) * math.exp(-b)), rel=1e-14)


@pytest.mark.parametrize("tile", [1, 7, 64, 128, 256, 1000])
def test_tiled_merge_reaches_plain_lse(tile):
    g = np.random.default_rng(tile)
    V, Vr = 1000, 1024
    z = g.standard_normal(V) * 4
    assert oracle.tiled_lse(z, Vr, tile) == pytest.approx(oracle.lse_rows(z[None])[0], rel=1e-12)


def test_tile_identity_partial():
    z = np.array([0.5, -1.0, 2.0])
    parts = oracle.tile_partials(z, 8, 2)
    assert parts[2] == (-np.inf, 0.0) and parts[3] == (-np.inf, 0.0)
    assert parts[1][0] == 2.0 and parts[1][1] == pytest.approx(1.0)
    # an extreme-range row: the merge must not overflow or lose the small tail
    z = np.array([800.0, -800.0, 799.0])
    assert oracle.tiled_lse(z, 3, 1) == pytest.approx(800 + math.log1p(math.exp(-1.0)), rel=1e-15)
