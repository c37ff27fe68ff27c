"""GPU parity of the group-relative advantage (grpo_group_advantage) with the
fp64 oracle, its bitwise repeatability, and its use as the objective's input."""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS
from tests import gpu_support as S

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def gb():
    from lm_head_selected_amd import binding
    return binding


def _rewards(kind, n, seed):
    g = np.random.default_rng(seed)
    if kind == "binary":
        return (g.random(n) < 0.4).astype(np.float32)
    return (g.standard_normal(n) * 2.0 + 0.5).astype(np.float32)


def _gpu(gb, r, G, eps, scale):
    rd = torch.from_numpy(r).cuda()
    adv = torch.empty_like(rd)
    gb.grpo_group_advantage(rd, G, eps, adv, scale_by_std=scale)
    torch.cuda.synchronize()
    return adv


@pytest.mark.parametrize("kind", ["binary", "gaussian"])
@pytest.mark.parametrize("G", [1, 4, 16, 64])
@pytest.mark.parametrize("scale", [True, False])
def test_advantage_parity(gb, kind, G, scale):
    r = _rewards(kind, G * 37, seed=G)
    eps = 1e-4
    got = _gpu(gb, r, G, eps, scale).cpu().numpy()
    exp = oracle.group_advantage(r, G, eps, scale_by_std=scale)
    np.testing.assert_allclose(got, exp, rtol=1e-5, atol=1e-5)
    if scale and G > 1:
        np.testing.assert_allclose(got.reshape(-1, G).sum(1), 0.0, atol=1e-4)


def test_advantage_constant_groups_eps_zero(gb):
    r = np.array([1, 1, 1, 1, 0, 1, 0, 1], np.float32)
    got = _gpu(gb, r, 4, 0.0, True).cpu().numpy()
    np.testing.assert_allclose(got, oracle.group_advantage(r, 4, 0.0), rtol=1e-6, atol=1e-7)
    assert np.all(got[:4] == 0.0)


def test_advantage_bitwise_and_in_place(gb):
    r = _rewards("gaussian", 16 * 500, seed=9)
    a = _gpu(gb, r, 16, 1e-6, True)
    b = _gpu(gb, r, 16, 1e-6, True)
    assert torch.equal(a, b)
    rd = torch.from_numpy(r).cuda()
    gb.grpo_group_advantage(rd, 16, 1e-6, rd)          # adv aliases rewards
    torch.cuda.synchronize()
    assert torch.equal(rd, a)


def test_advantage_feeds_the_objective(gb):
    """Rewards -> group advantages on the GPU -> forward; against the oracle run on
    the oracle's own advantages."""
    inp, lp, lse = S.build(CONFIGS[1])
    G = 4
    rew = _rewards("binary", inp["n_seqs"], seed=1)
    inp["adv"] = oracle.group_advantage(rew, G, 1e-4).astype(np.float32)
    d = S.to_device(inp)
    d["adv"] = _gpu(gb, rew, G, 1e-4, True)
    got = S.run(gb, inp, d, backward=False)
    exp = S.expect(inp, lp, lse, backward=False)
    act = oracle.active_tokens(inp["y"], inp["mask"], inp["ignore_index"])
    S.assert_forward(got, exp, "bf16", act)
