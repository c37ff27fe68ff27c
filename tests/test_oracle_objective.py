"""Pins of the oracle's objective (GRPO clipped ratio + k3 KL, GSPO) and its
per-token coefficient, against hand-derived values, closed forms, special cases
and finite differences."""
import math

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_clip_truth_table():
    """Each (ratio, advantage) case worked by hand for eps_low=0.2, eps_high=0.28:
    the PPO min picks the clipped term only when the ratio is past the bound on
    the side the advantage favours, and that branch has zero gradient."""
    r = np.array([1.5, 1.5, 0.5, 0.5, 1.1, 1.0])
    a = np.array([1.0, -2.0, 1.0, -1.0, 0.5, -1.0], np.float32)
    old = np.full(6, -1.0)
    logp = np.log(r) + old
    sid = np.arange(6)
    act = np.ones(6, bool)
    out = oracle.grpo_objective(logp, old, None, a, sid, act, 6, 0.2, 0.28, 0.0, "token_mean")
    pol = np.array([-1.28, 3.0, -0.5, 0.8, -0.55, 1.0])
    dpol = np.array([0.0, 3.0, -0.5, 0.0, -0.55, 1.0])
    assert out["policy_loss"] == pytest.approx(pol.mean(), rel=1e-14)
    assert out["loss"] == pytest.approx(pol.mean(), rel=1e-14)
    np.testing.assert_allclose(out["coef"], dpol / 6, rtol=1e-13, atol=1e-15)
    assert out["kl"] == 0.0


@pytest.mark.parametrize("delta", [0.3, -0.7])
def test_k3_closed_form(delta):
    """ref - logp = delta on every token: kl = e^delta - delta - 1 and the KL part
    of the coefficient is beta * w * (1 - e^delta)."""
    n = 5
    logp = -np.linspace(1, 3, n)
    ref = logp + delta
    adv = np.zeros(1, np.float32)
    out = oracle.grpo_objective(logp, logp, ref, adv, np.zeros(n, int), np.ones(n, bool), 1,
                                0.2, 0.2, 0.25, "token_mean")
    k = math.exp(delta) - delta - 1
    assert out["kl"] == pytest.approx(k, rel=1e-13)
    assert out["policy_loss"] == 0.0
    assert out["loss"] == pytest.approx(0.25 * k, rel=1e-13)
    np.testing.assert_allclose(out["coef"], 0.25 / n * (1 - math.exp(delta)), rtol=1e-13)


def _batch(lens, masked, seed=0):
    g = np.random.default_rng(seed)
    sid = np.repeat(np.arange(len(lens)), lens)
    n = len(sid)
    act = np.ones(n, bool)
    act[masked] = False
    adv = g.standard_normal(len(lens)).astype(np.float32)
    logp = -g.random(n) * 5
    return sid, act, adv, logp


def test_ratio_one_closed_forms():
    """old = ref = logp: r = 1, kl = 0, and loss = -(mean advantage) — over active
    tokens for token-mean, over live sequences for sequence-mean.  Sequence 2 is
    fully masked and must drop out of the sequence count."""
    lens = [3, 5, 2, 6]
    masked = [0, 4, 8, 9, 10]         # seq 2 = tokens 8, 9 fully masked
    sid, act, adv, logp = _batch(lens, masked)
    a64 = adv.astype(np.float64)
    tm = oracle.grpo_objective(logp, logp, logp, adv, sid, act, 4, .2, .2, .1, "token_mean")
    assert tm["kl"] == 0.0
    assert tm["loss"] == pytest.approx(-a64[sid[act]].mean(), rel=1e-13)
    sm = oracle.grpo_objective(logp, logp, logp, adv, sid, act, 4, .2, .2, .1, "sequence_mean")
    assert sm["loss"] == pytest.approx(-a64[[0, 1, 3]].mean(), rel=1e-13)
    assert list(sm["counts"]) == [2, 4, 0, 5]
    # coefficient at r = 1: -a_t w_t; inactive tokens 0
    w = np.where(act, 1.0 / (sm["counts"][sid].clip(1) * 3), 0)
    np.testing.assert_allclose(sm["coef"], -a64[sid] * w, rtol=1e-13)
    assert np.all(tm["coef"][~act] == 0)


def test_zero_advantage_zero_beta():
    sid, act, adv, logp = _batch([4, 4], [1])
    out = oracle.grpo_objective(logp, logp + 0.1, None, adv * 0, sid, act, 2, .2, .2, 0.0,
                                "sequence_mean")
    assert out["loss"] == 0.0 and np.all(out["coef"] == 0)


def test_empty_batch_is_all_zero():
    sid, act, adv, logp = _batch([3, 2], [0, 1, 2, 3, 4])
    for red in ("token_mean", "sequence_mean"):
        out = oracle.grpo_objective(logp, logp, logp, adv, sid, act, 2, .2, .2, .1, red)
        assert (out["loss"], out["policy_loss"], out["kl"]) == (0.0, 0.0, 0.0)
        assert np.all(out["coef"] == 0) and np.all(out["counts"] == 0)
    out = oracle.gspo_objective(logp, logp, logp, adv, sid, act, 2, .2, .2, .1)
    assert (out["loss"], out["policy_loss"], out["kl"]) == (0.0, 0.0, 0.0)
    assert np.all(out["coef"] == 0)


def test_gspo_single_token_segments_equal_grpo_sequence_mean():
    """With one-token segments the segment ratio is the token ratio and every
    segment weighs 1/S_live: GSPO reduces to token GRPO with sequence-mean."""
    g = np.random.default_rng(3)
    n = 9
    sid = np.arange(n)
    act = np.ones(n, bool)
    act[4] = False
    adv = g.standard_normal(n).astype(np.float32)
    logp = -g.random(n) * 3
    old = logp + g.standard_normal(n) * 0.3
    ref = logp + g.standard_normal(n) * 0.2
    a = oracle.gspo_objective(logp, old, ref, adv, sid, act, n, .2, .28, .05)
    b = oracle.grpo_objective(logp, old, ref, adv, sid, act, n, .2, .28, .05, "sequence_mean")
    for k in ("loss", "policy_loss", "kl"):
        assert a[k] == pytest.approx(b[k], rel=1e-13)
    np.testing.assert_allclose(a["coef"], b["coef"], rtol=1e-12, atol=1e-15)


def test_gspo_constant_log_ratio_closed_form():
    """A segment whose tokens all have log-ratio rho has sigma = e^rho; worked by
    hand for three segments and eps = (3e-4, 4e-4)."""
    lens = [4, 3, 5]
    sid = np.repeat(np.arange(3), lens)
    act = np.ones(12, bool)
    act[5] = False                            # segment 1 keeps 2 active tokens
    rho = np.array([2e-4, 1e-3, -2e-3])
    adv = np.array([1.0, 0.5, -1.5], np.float32)
    logp = -np.arange(12) * 0.1
    old = logp - rho[sid]
    out = oracle.gspo_objective(logp, old, None, adv, sid, act, 3, 3e-4, 4e-4, 0.0)
    sig = np.exp(rho)
    # seg 0: inside the range -> -sigma*A ; seg 1: above 1+4e-4 with A>0 -> clipped
    # -(1+4e-4)*A ; seg 2: below 1-3e-4 with A<0 -> clipped -(1-3e-4)*A
    pol = np.array([-sig[0] * 1.0, -(1 + 4e-4) * 0.5, -(1 - 3e-4) * -1.5])
    assert out["policy_loss"] == pytest.approx(pol.mean(), rel=1e-13)
    np.testing.assert_allclose(out["sigma"], sig, rtol=1e-14)
    exp_coef = np.zeros(12)
    exp_coef[:4] = -1.0 * sig[0] / (3 * 4)    # only segment 0 is unclipped
    np.testing.assert_allclose(out["coef"], exp_coef, rtol=1e-13, atol=1e-18)
    assert list(out["counts"]) == [4, 2, 5]
    np.testing.assert_allclose(out["seg_mean_logp"][1], (logp[4] + logp[6]) / 2, rtol=1e-14)


def test_counts_are_exact_integers():
    g = np.random.default_rng(7)
    sid = np.sort(g.integers(0, 40, 3000))
    act = g.random(3000) > 0.3
    L = oracle.sequence_counts(sid, act, 45)
    assert L.dtype.kind == "i"
    np.testing.assert_array_equal(L, np.bincount(sid[act], minlength=45))


def _fd(f, x, h):
    x0 = x.copy()
    xp, xm = x0.copy(), x0.copy()
    xp += h
    xm -= h
    return (f(xp) - f(xm)) / (2 * h)


@pytest.mark.parametrize("level,reduction,beta", [("token", "token_mean", 0.04),
                                                   ("token", "fixed_constant", 0.06),
                                                   ("token", "sequence_mean", 0.1),
                                                   ("sequence_gspo", "sequence_mean", 0.07)])
def test_coef_is_the_logp_derivative(level, reduction, beta):
    """Central differences of the loss in each logp_t equal coef_t (no ratio lies
    within 0.01 of a clip boundary, so the loss is smooth at every point)."""
    g = np.random.default_rng(11)
    lens = [5, 1, 6, 4]
    sid = np.repeat(np.arange(4), lens)
    n = len(sid)
    act = np.ones(n, bool)
    act[[2, 7]] = False
    adv = g.standard_normal(4).astype(np.float32)
    logp0 = -g.random(n) * 4
    eps = (0.2, 0.28) if level == "token" else (0.05, 0.06)
    noise = g.choice([-0.5, -0.1, 0.03, 0.15, 0.6], n) + g.standard_normal(n) * 0.002
    if level != "token":
        # segment log-ratios -0.2, 0.01, 0.3, -0.02 plus zero-mean token jitter
        noise = np.array([0.2, -0.01, -0.3, 0.02])[sid] + np.tile([0.01, -0.01], n // 2)
    old = logp0 + noise
    ref = logp0 + g.standard_normal(n) * 0.2

    def run(lp):
        if level == "token":
            return oracle.grpo_objective(lp, old, ref, adv, sid, act, 4, *eps, beta, reduction,
                                         norm_const=37.5)
        return oracle.gspo_objective(lp, old, ref, adv, sid, act, 4, *eps, beta)

    out = run(logp0)
    if level == "token":
        assert 0 < np.sum(out["unclipped"] & act) < act.sum()
    else:
        assert 0 < out["unclipped"].sum() < 4
    for t in range(n):
        def f(v, t=t):
            lp = logp0.copy()
            lp[t] = v[0]
            return run(lp)["loss"]
        d = _fd(f, np.array([logp0[t]]), 1e-6)
        assert d == pytest.approx(out["coef"][t], rel=1e-6, abs=1e-10), t


def test_fixed_constant_at_the_active_count_is_the_token_mean():
    """fixed_constant divides the active-token sums by the caller's C; at
    C = T_act it is the masked token mean exactly, and the result scales as 1/C."""
    g = np.random.default_rng(5)
    lens = [4, 7, 3]
    sid, act, adv, logp = _batch(lens, [1, 5, 12])
    old = logp + g.standard_normal(len(sid)) * 0.3
    ref = logp + g.standard_normal(len(sid)) * 0.2
    T = int(act.sum())
    tm = oracle.grpo_objective(logp, old, ref, adv, sid, act, 3, .2, .28, .1, "token_mean")
    fc = oracle.grpo_objective(logp, old, ref, adv, sid, act, 3, .2, .28, .1, "fixed_constant",
                               norm_const=T)
    for k in ("loss", "policy_loss", "kl"):
        assert fc[k] == pytest.approx(tm[k], rel=1e-14)
    np.testing.assert_allclose(fc["coef"], tm["coef"], rtol=1e-14)
    big = oracle.grpo_objective(logp, old, ref, adv, sid, act, 3, .2, .28, .1, "fixed_constant",
                                norm_const=4.0 * T)
    for k in ("loss", "policy_loss", "kl"):
        assert big[k] == pytest.approx(tm[k] / 4.0, rel=1e-14)
    np.testing.assert_allclose(big["coef"], tm["coef"] / 4.0, rtol=1e-14)
    # sequences weigh by their token count, unlike sequence_mean
    sm = oracle.grpo_objective(logp, old, ref, adv, sid, act, 3, .2, .28, .1, "sequence_mean")
    assert abs(sm["policy_loss"] - tm["policy_loss"]) > 1e-6


def test_fixed_constant_empty_batch_and_bad_constant():
    sid, act, adv, logp = _batch([3, 2], [0, 1, 2, 3, 4])
    out = oracle.grpo_objective(logp, logp, logp, adv, sid, act, 2, .2, .2, .1,
                                "fixed_constant", norm_const=64.0)
    assert (out["loss"], out["policy_loss"], out["kl"]) == (0.0, 0.0, 0.0)
    assert np.all(out["coef"] == 0)
    with pytest.raises(ValueError):
        oracle.grpo_objective(logp, logp, logp, adv, sid, act, 2, .2, .2, .1, "fixed_constant")


def test_gspo_kl_weights_closed_form():
    """GSPO with beta > 0 on segments of unequal length, worked by hand.

    Segment 0: 1 active token; segment 1: 4 tokens, one masked, so L = 3; a third
    segment is fully masked and drops out of S_live (= 2).  old = logp, so every
    segment ratio is 1 (unclipped, pol_s = -A_s); ref - logp = delta_s is constant
    per segment: delta = (0.5, -0.2).
      k3(0.5)  = e^0.5 - 1.5          = 0.148721270700128
      k3(-0.2) = e^-0.2 + 0.2 - 1     = 0.018730753077982
    The KL term weighs each live segment equally (sequence mean):
      kl = (k3(0.5) + k3(-0.2)) / 2   = 0.083726011889055,
    whereas a token mean would give (k3(0.5) + 3 k3(-0.2)) / 4 = 0.051228.
    policy_loss = (-0.7 + 1.3) / 2 = 0.3; loss = 0.3 + 0.1 * kl.
    coef_t = (-A_s) / (S_live L_s) + beta (1 - e^delta_s) / (S_live L_s):
      segment 0: -0.7/2 + 0.1 (1 - e^0.5)/2      = -0.382436063535006
      segment 1:  1.3/6 + 0.1 (1 - e^-0.2)/6     =  0.219687820782017
    """
    sid = np.array([0, 1, 1, 1, 1, 2, 2])
    act = np.array([1, 1, 0, 1, 1, 0, 0], bool)
    logp = np.array([-0.3, -1.0, -2.0, -0.4, -2.5, -1.0, -1.0])
    delta = np.array([0.5, -0.2, 0.0])[sid]
    adv = np.array([0.7, -1.3, 2.0], np.float32)
    out = oracle.gspo_objective(logp, logp, logp + delta, adv, sid, act, 3, 0.2, 0.28, 0.1)
    assert out["kl"] == pytest.approx(0.083726011889055, rel=1e-13)
    assert out["policy_loss"] == pytest.approx(0.3, rel=1e-7)   # adv is fp32: 0.7, -1.3
    a = adv.astype(np.float64)
    assert out["policy_loss"] == pytest.approx(-(a[0] + a[1]) / 2.0, rel=1e-14)
    assert out["loss"] == pytest.approx(out["policy_loss"] + 0.1 * 0.083726011889055, rel=1e-13)
    c0 = -a[0] / 2 + 0.1 * (1 - np.exp(0.5)) / 2
    c1 = -a[1] / 6 + 0.1 * (1 - np.exp(-0.2)) / 6
    assert c0 == pytest.approx(-0.382436063535006, rel=1e-7)
    assert c1 == pytest.approx(0.219687820782017, rel=1e-7)
    np.testing.assert_allclose(out["coef"], [c0, c1, 0, c1, c1, 0, 0], rtol=1e-13, atol=0)
    assert list(out["counts"]) == [1, 3, 0]


def test_objective_dispatch_matches_direct_calls():
    """objective() passes the workload's level, clip bounds, beta, reduction and
    fixed_constant divisor through unchanged: equal to calling grpo_objective /
    gspo_objective directly, for distinct eps_low / eps_high, every reduction and
    both levels, with an explicit mask and in ignore_index mode."""
    g = np.random.default_rng(21)
    lens = [5, 3, 6, 2]
    sid = np.repeat(np.arange(4), lens)
    n = len(sid)
    y = g.integers(0, 50, n)
    mask = (g.random(n) > 0.2).astype(np.uint8)
    logp = -g.random(n) * 3
    base = dict(y=y, sid=sid, n_seqs=4, adv=g.standard_normal(4).astype(np.float32),
                # log-ratios near 0.25 (ratio 1.28): inside 1 + 0.31, outside 1 + 0.13,
                # so swapped clip bounds would change the result at both levels
                old_logp=(logp - 0.25 + g.standard_normal(n) * 0.05).astype(np.float32),
                ref_logp=(logp + g.standard_normal(n) * 0.2).astype(np.float32),
                eps_low=0.13, eps_high=0.31, beta=0.07, ignore_index=-100)
    y_ign = y.copy()
    y_ign[mask == 0] = -100
    for m, yy in ((mask, y), (None, y_ign)):
        act = oracle.active_tokens(yy, m, -100)
        for level, red, C in (("token", "token_mean", None), ("token", "sequence_mean", None),
                              ("token", "fixed_constant", 23.5),
                              ("sequence_gspo", "sequence_mean", None)):
            inp = dict(base, y=yy, mask=m, level=level, reduction=red)
            if C is not None:
                inp["norm_const"] = C
            got = oracle.objective(inp, logp)
            if level == "token":
                exp = oracle.grpo_objective(logp, base["old_logp"], base["ref_logp"], base["adv"],
                                            sid, act, 4, 0.13, 0.31, 0.07, red, C)
            else:
                exp = oracle.gspo_objective(logp, base["old_logp"], base["ref_logp"], base["adv"],
                                            sid, act, 4, 0.13, 0.31, 0.07)
            for k in ("loss", "policy_loss", "kl"):
                assert got[k] == exp[k], (level, red, k)
            np.testing.assert_array_equal(got["coef"], exp["coef"])
            np.testing.assert_array_equal(got["counts"], exp["counts"])
    # the two levels and the normalisers really differ on these inputs
    a = oracle.objective(dict(base, mask=mask, level="token", reduction="token_mean"), logp)
    b = oracle.objective(dict(base, mask=mask, level="token", reduction="sequence_mean"), logp)
    c = oracle.objective(dict(base, mask=mask, level="sequence_gspo",
                              reduction="sequence_mean"), logp)
    d = oracle.objective(dict(base, mask=mask, level="token", reduction="fixed_constant",
                              norm_const=23.5), logp)
    vals = [a["loss"], b["loss"], c["loss"], d["loss"]]
    assert len({round(v, 12) for v in vals}) == 4


@pytest.mark.parametrize("level", ["token", "sequence_gspo"])
def test_branch_coefficients_are_the_coef_on_either_side_of_a_kink(level):
    """coef_unclipped / coef_clipped are what coef becomes when a token's (or a
    segment's) ratio crosses the clip boundary: moving old_logp by 1e-9 across the
    kink makes the objective take the other branch, and its coef there equals the
    reported branch coefficient (within the 1e-9 shift)."""
    eps_l, eps_h, beta = 0.2, 0.28, 0.05
    lens = [3, 2]
    sid = np.repeat(np.arange(2), lens)
    n = len(sid)
    act = np.ones(n, bool)
    logp = np.array([-1.0, -2.0, -0.5, -1.5, -0.7])
    ref = logp + np.array([0.1, -0.2, 0.3, 0.05, -0.1])
    adv = np.array([1.5, -0.8], np.float32)
    k_hi, k_lo = np.log1p(eps_h), np.log1p(-eps_l)

    def run(old):
        if level == "token":
            return oracle.grpo_objective(logp, old, ref, adv, sid, act, 2, eps_l, eps_h, beta,
                                         "sequence_mean")
        return oracle.gspo_objective(logp, old, ref, adv, sid, act, 2, eps_l, eps_h, beta)

    # segment / token log-ratios placed 1e-9 past the boundary the advantage
    # favours: seq 0 (A > 0) just above 1 + eps_h (clipped), seq 1 (A < 0) just
    # below 1 - eps_l (clipped)
    for side in (+1.0, -1.0):
        lr = np.where(sid == 0, k_hi + side * 1e-9, k_lo - side * 1e-9)
        old = logp - lr
        here = run(old)
        there = run(logp - (lr - side * 2e-9 * np.where(sid == 0, 1.0, -1.0)))
        flip = here["unclipped"] != there["unclipped"]
        assert flip.all()
        for t in range(n):
            on = "coef_unclipped" if there["unclipped"][t if level == "token" else sid[t]] \
                else "coef_clipped"
            assert here[on][t] == pytest.approx(there["coef"][t], rel=1e-7, abs=1e-12)
            np.testing.assert_array_equal(
                here["coef"], np.where(
                    here["unclipped"] if level == "token" else here["unclipped"][sid],
                    here["coef_unclipped"], here["coef_clipped"]))
