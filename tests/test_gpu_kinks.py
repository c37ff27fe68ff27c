"""GPU parity where the clip branch is a close call.

The default input recipe keeps every ratio a little away from the clip
boundaries.  Here the old-policy noise is left as drawn (and some tokens are put
exactly on a boundary), so ratios sit on and next to the kinks of the PPO min.
At a kink both branches of the min are correct, so the checks are:

  A. against the oracle on its own fp64 log-probs: a token (GRPO) or segment
     (GSPO) whose oracle log-ratio lies within the log-prob tolerance of a kink
     log(1 - eps_low) or log(1 + eps_high) may take either branch -- the GPU's
     log-probs may differ from the oracle's by that much -- so its coefficient
     must match one of the two branch coefficients; every other coefficient must
     match the oracle's;
  B. against the oracle evaluated on the GPU's own log-probs: the GPU's branch
     must then agree except within fp32 rounding of the log-ratio (a band derived
     below), which separates the objective stage from the forward's error;
  and the gradients against the oracle's backward with each near-kink token on
  the branch the GPU took.  The loss triple is continuous at a kink and is
  checked at the usual tolerance.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs
from tests import gpu_support as S

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

U32 = 2.0 ** -24        # fp32 unit roundoff


@pytest.fixture(scope="module")
def gb():
    from lm_head_selected_amd import binding
    return binding


def _kinks(inp):
    return np.array([math.log1p(-inp["eps_low"]), math.log1p(inp["eps_high"])])


def _near(x, kinks, band):
    return np.min(np.abs(np.asarray(x)[..., None] - kinks), axis=-1) <= band


def _coef_ok(c, exp, band, tol):
    """coef matches the oracle's, or, inside `band`, either branch coefficient."""
    c = c.astype(np.float64)
    scale = np.max(np.abs(exp["coef"]), initial=0)

    def close(e):
        return np.abs(c - e) <= tol["coef_rel"] * np.abs(e) + 1e-6 * scale

    either = close(exp["coef_unclipped"]) | close(exp["coef_clipped"])
    return np.where(band, either, close(exp["coef"]))


def _branch_as_gpu(c, exp, band):
    """The oracle's coefficient with each in-band token on the GPU's branch."""
    c = c.astype(np.float64)
    pick_u = np.abs(c - exp["coef_unclipped"]) <= np.abs(c - exp["coef_clipped"])
    branch = np.where(pick_u, exp["coef_unclipped"], exp["coef_clipped"])
    return np.where(band, branch, exp["coef"])


def _token_bands(inp, lp, got_lp, exp_a, exp_b, act):
    kinks = _kinks(inp)
    tol_lp = S.TOL[inp["dtype"]]["logp"]
    if inp["level"] == "token":
        # A: the GPU's logp is within tol_lp of the oracle's, so is its log-ratio
        band_a = act & _near(exp_a["log_ratio"], kinks, tol_lp)
        # B: logp - old and exp in fp32, and fp32 clip bounds: a few ulp of the ratio
        band_b = act & _near(exp_b["log_ratio"], kinks, 8 * U32 * (1 + np.abs(kinks).max()))
        return band_a, band_b, band_a.sum(), band_b.sum()
    sid = inp["sid"]
    # A: a segment mean of per-token errors each within tol_lp
    seg_a = _near(exp_a["rho"], kinks, tol_lp)
    # B: the GPU sums L fp32 log-ratios (each rounded once) and divides by L: error
    # at most (L + 1) u sum |l_t| / L, plus the fp32 exp and clip bounds
    ell = np.where(act, got_lp.astype(np.float64) - inp["old_logp"].astype(np.float64), 0.0)
    abs_sum = np.zeros(inp["n_seqs"])
    np.add.at(abs_sum, sid, np.abs(ell))
    L = np.maximum(exp_b["counts"], 1)
    bound = (L + 1) * U32 * abs_sum / L + 8 * U32
    seg_b = np.min(np.abs(exp_b["rho"][:, None] - kinks), axis=1) <= bound
    return act & seg_a[sid], act & seg_b[sid], seg_a.sum(), seg_b.sum()


def _check(gb, inp, lp, lse, chunk=0):
    act = oracle.active_tokens(inp["y"], inp["mask"], inp["ignore_index"])
    got = S.run(gb, inp, chunk_tokens=chunk)
    tol = S.TOL[inp["dtype"]]
    exp_a = oracle.objective(inp, lp)
    exp_b = oracle.objective(inp, got["logp"].astype(np.float64))
    band_a, band_b, n_a, n_b = _token_bands(inp, lp, got["logp"], exp_a, exp_b, act)
    print(f"near a kink: A {int(n_a)}, B {int(n_b)} "
          f"({'tokens' if inp['level'] == 'token' else 'segments'})", flush=True)
    # forward and loss triple as usual (continuous at a kink)
    assert np.max(np.abs(got["logp"] - lp)) <= tol["logp"]
    assert np.max(np.abs(got["lse"] - lse)) <= tol["lse"]
    for k, name in enumerate(("loss", "policy_loss", "kl")):
        e = exp_a[name]
        assert abs(float(got["out3"][k]) - e) <= tol["loss_rel"] * abs(e) + tol["loss_abs"], name
    np.testing.assert_array_equal(got["counts"], exp_a["counts"])
    assert np.all(got["coef"][~act] == 0.0)
    ok_a = _coef_ok(got["coef"], exp_a, band_a, tol)
    assert ok_a.all(), np.nonzero(~ok_a)[0][:10]
    ok_b = _coef_ok(got["coef"], exp_b, band_b, tol)
    assert ok_b.all(), np.nonzero(~ok_b)[0][:10]
    # gradients with each near-kink token on the GPU's branch
    coef = _branch_as_gpu(got["coef"], exp_a, band_a)
    dH, dW = oracle.backward(inp["H"], inp["W"], inp["y"], act, lse, coef, inp["v_real"],
                             inp["inv_tau"], 1.0, inp["dtype"], block=256)
    assert S.rel_l2(got["dH"], dH) <= tol["grad"]
    assert S.rel_l2(got["dW"], dW) <= tol["grad"]
    return n_a, n_b


def _on_kinks(inp, lp, rng, n_each):
    """Put n_each active tokens exactly on each clip boundary: old = logp - kink."""
    act = oracle.active_tokens(inp["y"], inp["mask"], inp["ignore_index"])
    idx = rng.choice(np.nonzero(act)[0], size=2 * n_each, replace=False)
    k = _kinks(inp)
    old = inp["old_logp"].astype(np.float64)
    old[idx[:n_each]] = lp[idx[:n_each]] - k[0]
    old[idx[n_each:]] = lp[idx[n_each:]] - k[1]
    inp["old_logp"] = old.astype(np.float32)
    return inp


@pytest.mark.parametrize("ci,chunk", [(1, 0), (2, 0), (2, 1024)])
def test_grpo_ratios_at_the_clip_boundaries(gb, ci, chunk):
    """Token level, old-policy noise N(0, 0.3) as drawn, plus 16 tokens exactly on
    each boundary: both reductions (sequence mean on the 1024-token case, token
    mean on the 4096-token one), with the KL term."""
    cfg = CONFIGS[ci]
    print(f"config {cfg.name}, chunk {chunk}", flush=True)
    inp = make_inputs(cfg, old_noise=0.3, off_kinks=False)
    inp, lp, lse = S.with_oracle_logprobs(inp)
    inp = _on_kinks(inp, lp, np.random.default_rng(ci), 16)
    n_a, _ = _check(gb, inp, lp, lse, chunk)
    assert n_a >= 32                              # the planted tokens at least


@pytest.mark.parametrize("beta", [0.0, 0.05])
def test_gspo_segments_at_the_clip_boundaries(gb, beta):
    """Segment level with the tight bounds eps = 3e-4 / 4e-4 and packed segments
    of 16-256 tokens, old-policy noise as drawn: many segment ratios lie within
    the tolerance of a boundary."""
    cfg = dataclasses.replace(CONFIGS[4], n_tokens=4096, d_model=256, v_real=5000, v_rows=5120,
                              w_std=0.05, seg_len_range=(16, 256), beta=beta,
                              ref_noise=0.1 if beta > 0 else None, mask_frac=0.1)
    print(f"GSPO beta {beta}", flush=True)
    inp = make_inputs(cfg, off_kinks=False)
    inp, lp, lse = S.with_oracle_logprobs(inp)
    # two segments with every log-ratio exactly on a boundary, so rho is too
    old = inp["old_logp"].astype(np.float64)
    for s, k in zip((3, 10), _kinks(inp)):
        on = inp["sid"] == s
        old[on] = lp[on] - k
    inp["old_logp"] = old.astype(np.float32)
    n_a, n_b = _check(gb, inp, lp, lse)
    assert n_a >= 5 and n_b >= 2
