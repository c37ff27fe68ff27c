"""Pins of the oracle's backward (dlogits, dH, dW): finite differences through
the whole forward + objective, torch autograd, and invariants."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

N, D, V, VR = 12, 6, 20, 23
INV_TAU = 1.0 / 0.7


def _setup(seed=0, level="token", reduction="sequence_mean", beta=0.05):
    g = np.random.default_rng(seed)
    H = g.standard_normal((N, D))
    W = g.standard_normal((VR, D)) * 0.5
    W[V:] = np.nan                                  # padded rows: never read
    y = g.integers(0, V, N)
    lens = [4, 3, 5]
    sid = np.repeat(np.arange(3), lens)
    act = np.ones(N, bool)
    act[[1, 9]] = False
    y[1] = 10 ** 9                                  # inactive target: never read
    adv = g.standard_normal(3).astype(np.float32)
    logp, lse = oracle.forward(H, W, y, act, V, INV_TAU, "f64")
    # ratios at least 0.05 away from every clip boundary
    noise = g.choice([-0.6, -0.05, 0.1, 0.5], N)
    old = logp + noise
    ref = logp + g.standard_normal(N) * 0.3
    eps = (0.2, 0.28) if level == "token" else (0.01, 0.02)
    if level == "sequence_gspo":
        noise_seg = np.array([0.3, -0.1, 0.0])
        old = logp + noise_seg[sid]

    def loss_of(Hx, Wx):
        lp, _ = oracle.forward(Hx, Wx, y, act, V, INV_TAU, "f64")
        if level == "token":
            return oracle.grpo_objective(lp, old, ref, adv, sid, act, 3, *eps, beta, reduction)
        return oracle.gspo_objective(lp, old, ref, adv, sid, act, 3, *eps, beta)

    out = loss_of(H, W)
    return dict(H=H, W=W, y=y, sid=sid, act=act, adv=adv, old=old, ref=ref, lse=lse,
                logp=logp, out=out, loss_of=loss_of, eps=eps, beta=beta)


@pytest.mark.parametrize("level,reduction", [("token", "token_mean"), ("token", "sequence_mean"),
                                             ("sequence_gspo", "sequence_mean")])
def test_gradients_match_finite_differences(level, reduction):
    s = _setup(1, level, reduction)
    gamma = 1.7
    dH, dW = oracle.backward(s["H"], s["W"], s["y"], s["act"], s["lse"], s["out"]["coef"], V,
                             INV_TAU, gamma, "f64")
    g = np.random.default_rng(5)
    h = 1e-6
    for _ in range(12):
        t, d = g.integers(0, N), g.integers(0, D)
        Hp, Hm = s["H"].copy(), s["H"].copy()
        Hp[t, d] += h
        Hm[t, d] -= h
        fd = gamma * (s["loss_of"](Hp, s["W"])["loss"] - s["loss_of"](Hm, s["W"])["loss"]) / (2 * h)
        assert dH[t, d] == pytest.approx(fd, rel=1e-6, abs=1e-9)
    for _ in range(12):
        v, d = g.integers(0, V), g.integers(0, D)
        Wp, Wm = s["W"].copy(), s["W"].copy()
        Wp[v, d] += h
        Wm[v, d] -= h
        fd = gamma * (s["loss_of"](s["H"], Wp)["loss"] - s["loss_of"](s["H"], Wm)["loss"]) / (2 * h)
        assert dW[v, d] == pytest.approx(fd, rel=1e-6, abs=1e-9)
    assert np.all(dW[V:] == 0)


def test_gradients_match_torch_autograd():
    """Sequence-mean GRPO with k3 KL differentiated by torch autograd in fp64."""
    s = _setup(2, "token", "sequence_mean", beta=0.3)
    H = torch.tensor(s["H"], requires_grad=True)
    W = torch.tensor(s["W"][:V], requires_grad=True)
    z = (H @ W.T) * INV_TAU
    act = torch.tensor(s["act"])
    yy = torch.tensor(np.where(s["act"], s["y"], 0))
    lp = torch.where(act, torch.log_softmax(z, 1).gather(1, yy[:, None])[:, 0], torch.zeros(()))
    old = torch.tensor(s["old"])
    ref = torch.tensor(s["ref"])
    a = torch.tensor(s["adv"].astype(np.float64))[torch.tensor(s["sid"])]
    r = torch.exp(lp - old)
    c = torch.clamp(r, 1 - s["eps"][0], 1 + s["eps"][1])
    pol = -torch.minimum(r * a, c * a)
    dl = ref - lp
    kl = torch.exp(dl) - dl - 1
    sid = torch.tensor(s["sid"])
    L = torch.zeros(3, dtype=torch.float64).index_add_(0, sid, act.double())
    w = act.double() / (L[sid] * (L > 0).sum())
    loss = (w * (pol + s["beta"] * kl)).sum()
    loss.backward()
    dH, dW = oracle.backward(s["H"], s["W"], s["y"], s["act"], s["lse"], s["out"]["coef"], V,
                             INV_TAU, 1.0, "f64")
    assert s["out"]["loss"] == pytest.approx(loss.item(), rel=1e-12)
    np.testing.assert_allclose(dH, H.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dW[:V], W.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_backward_invariants():
    s = _setup(3)
    coef = s["out"]["coef"]
    dH, dW = oracle.backward(s["H"], s["W"], s["y"], s["act"], s["lse"], coef, V, INV_TAU, 1.0,
                             "f64")
    # every dlogits row sums to zero, hence so do dW's columns over the vocabulary
    np.testing.assert_allclose(dW[:V].sum(0), 0.0, atol=1e-13)
    # dH_t = coef_t (W_{y_t} - sum_v p_tv W_v) / tau
    z = oracle.logits_rows(s["H"], s["W"], V, INV_TAU)
    p = np.exp(z - s["lse"][:, None])
    Wr = s["W"][:V]
    for t in np.nonzero(s["act"])[0]:
        exp_row = coef[t] * (Wr[s["y"][t]] - p[t] @ Wr) * INV_TAU
        np.testing.assert_allclose(dH[t], exp_row, rtol=1e-11, atol=1e-14)
    assert np.all(dH[~s["act"]] == 0.0)
    assert np.all(dW[V:] == 0.0)
    # linear in grad_output
    dH2, dW2 = oracle.backward(s["H"], s["W"], s["y"], s["act"], s["lse"], coef, V, INV_TAU,
                               -2.5, "f64")
    np.testing.assert_allclose(dH2, -2.5 * dH, rtol=1e-13, atol=1e-16)


def test_sampled_rows_equal_full_backward():
    s = _setup(4)
    coef = s["out"]["coef"]
    dH, dW = oracle.backward(s["H"], s["W"], s["y"], s["act"], s["lse"], coef, V, INV_TAU, 0.9,
                             "f64")
    rows = np.array([0, 1, 5, 11])
    np.testing.assert_allclose(
        oracle.dH_rows(s["H"], s["W"], s["y"], s["act"], s["lse"], coef, rows, V, INV_TAU, 0.9,
                       "f64", vblock=7), dH[rows], rtol=1e-12, atol=1e-15)
    vrows = np.array([0, 3, 19, 20, 22])
    np.testing.assert_allclose(
        oracle.dW_rows(s["H"], s["W"], s["y"], s["act"], s["lse"], coef, vrows, V, INV_TAU, 0.9,
                       "f64", tblock=5), dW[vrows], rtol=1e-12, atol=1e-15)


def test_sketch_equals_full_backward_times_probes():
    """backward_sketch returns (dH U, dW U) of the full backward for a [D, k] U:
    the same numbers (to rounding) as multiplying the full gradients, with zero
    rows for inactive tokens and for the padded vocabulary, on bf16 and fp64
    operands and in blocks that do not divide the token count."""
    s = _setup(5)
    coef = s["out"]["coef"]
    g = np.random.default_rng(9)
    U = g.standard_normal((D, 3))
    dH, dW = oracle.backward(s["H"], s["W"], s["y"], s["act"], s["lse"], coef, V, INV_TAU, 1.7,
                             "f64")
    sH, sW = oracle.backward_sketch(s["H"], s["W"], s["y"], s["act"], s["lse"], coef, U, V,
                                    INV_TAU, 1.7, "f64", block=5)
    np.testing.assert_allclose(sH, dH @ U, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(sW[:V], dW[:V] @ U, rtol=1e-11, atol=1e-14)
    assert np.all(sW[V:] == 0.0) and np.all(sH[~s["act"]] == 0.0)
    # a single wrong vocabulary row of dW changes that row of the sketch only
    dW_bad = dW.copy()
    dW_bad[7] *= 1.01
    diff = np.abs(dW_bad[:V] @ U - sW[:V]).max(axis=1)
    assert np.argmax(diff) == 7 and np.sort(diff)[-2] < 1e-10 * np.abs(sW).max()

    from synth import f32_to_bf16_bits
    Hb = f32_to_bf16_bits(s["H"].astype(np.float32))
    Wb = f32_to_bf16_bits(s["W"].astype(np.float32))
    lp, lse = oracle.forward(Hb, Wb, s["y"], s["act"], V, INV_TAU, "bf16")
    dH, dW = oracle.backward(Hb, Wb, s["y"], s["act"], lse, coef, V, INV_TAU, 1.0, "bf16")
    sH, sW = oracle.backward_sketch(Hb, Wb, s["y"], s["act"], lse, coef, U, V, INV_TAU, 1.0,
                                    "bf16", block=4)
    np.testing.assert_allclose(sH, dH @ U, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(sW, dW @ U, rtol=1e-11, atol=1e-14)
