"""Helpers for the GPU parity tests: move a synthetic workload to the device, run
the HIP path through the C ABI, and compute the oracle's expectations."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import oracle
from synth import attach_logprobs, make_inputs

TOL = {  # GPU versus the fp64 oracle
    "bf16": dict(logp=2e-3, lse=2e-3, loss_rel=1e-3, loss_abs=1e-5, coef_rel=3e-3, grad=1e-2),
    "f32": dict(logp=1e-5, lse=1e-5, loss_rel=1e-5, loss_abs=1e-6, coef_rel=1e-4, grad=1e-5),
}


def with_oracle_logprobs(inp: dict) -> tuple[dict, np.ndarray, np.ndarray]:
    act = oracle.active_tokens(inp["y"], inp["mask"], inp["ignore_index"])
    lp, lse = oracle.forward(inp["H"], inp["W"], inp["y"], act, inp["v_real"], inp["inv_tau"],
                             inp["dtype"], block=256)
    return attach_logprobs(inp, lp), lp, lse


def build(cfg, **overrides):
    """Inputs of a (possibly modified) workload with old/ref from the oracle."""
    if overrides:
        cfg = dataclasses.replace(cfg, **overrides)
    inp = make_inputs(cfg)
    inp, lp, lse = with_oracle_logprobs(inp)
    return inp, lp, lse


def to_device(inp: dict, dev="cuda"):
    def t(a, dt):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)

    if inp["dtype"] == "bf16":
        H = torch.from_numpy(inp["H"].view(np.int16)).to(dev).view(torch.bfloat16)
        W = torch.from_numpy(inp["W"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        H, W = t(inp["H"], torch.float32), t(inp["W"], torch.float32)
    return dict(H=H, W=W, y=t(inp["y"], torch.int64), mask=t(inp["mask"], torch.uint8),
                sid=t(inp["sid"], torch.int32), adv=t(inp["adv"], torch.float32),
                old=t(inp["old_logp"], torch.float32), ref=t(inp["ref_logp"], torch.float32))


def params(gb, inp, **kw):
    base = dict(n_tokens=inp["n_tokens"], d_model=inp["d_model"], v_real=inp["v_real"],
                v_rows=inp["v_rows"], n_seqs=inp["n_seqs"], dtype=inp["dtype"],
                reduction=inp["reduction"], level=inp["level"], inv_tau=inp["inv_tau"],
                eps_low=inp["eps_low"], eps_high=inp["eps_high"], beta=inp["beta"],
                ignore_index=inp["ignore_index"])
    base.update(kw)
    return gb.make_params(**base)


def run(gb, inp, d=None, *, backward=True, grad_output=None, keep_device=False, **pkw):
    """fwd (+ bwd) through the C ABI.  Returns numpy outputs (or device tensors)."""
    dev = torch.device("cuda")
    d = d or to_device(inp, dev)
    p = params(gb, inp, **pkw)
    head = gb.GrpoHead(p, dev, need_backward=backward)
    head.fwd(d["H"], d["W"], d["y"], d["mask"], d["sid"], d["adv"], d["old"], d["ref"])
    out = dict(logp=head.logp, lse=head.lse, coef=head.coef, out3=head.out3,
               counts=head.counts[: inp["n_seqs"]])
    if backward:
        g = None if grad_output is None else torch.tensor([grad_output], device=dev,
                                                          dtype=torch.float32)
        dH, dW = head.bwd(d["H"], d["W"], d["y"], d["mask"], grad_output=g)
        out.update(dH=dH, dW=dW)
    torch.cuda.synchronize()
    if keep_device:
        return out
    return {k: v.cpu().numpy() for k, v in out.items()}


def expect(inp, lp, lse, *, grad_output=1.0, backward=True):
    exp = oracle.objective(inp, lp)
    exp.update(logp=lp, lse=lse)
    if backward:
        act = oracle.active_tokens(inp["y"], inp["mask"], inp["ignore_index"])
        dH, dW = oracle.backward(inp["H"], inp["W"], inp["y"], act, lse, exp["coef"],
                                 inp["v_real"], inp["inv_tau"], grad_output, inp["dtype"],
                                 block=256)
        exp.update(dH=dH, dW=dW)
    return exp


def rel_l2(got, exp):
    n = np.linalg.norm(exp)
    return np.linalg.norm(np.asarray(got, np.float64) - exp) / (n if n > 0 else 1.0)


def assert_forward(got, exp, dtype, active):
    tol = TOL[dtype]
    assert np.all(got["logp"][~active] == 0.0)
    assert np.max(np.abs(got["logp"] - exp["logp"]), initial=0) <= tol["logp"]
    assert np.max(np.abs(got["lse"] - exp["lse"]), initial=0) <= tol["lse"]
    for k, name in enumerate(("loss", "policy_loss", "kl")):
        e = exp[name]
        assert abs(float(got["out3"][k]) - e) <= tol["loss_rel"] * abs(e) + tol["loss_abs"], \
            (name, float(got["out3"][k]), e)
    np.testing.assert_array_equal(got["counts"], exp["counts"])
    c, ce = got["coef"].astype(np.float64), exp["coef"]
    scale = np.max(np.abs(ce), initial=0)
    assert np.all(np.abs(c - ce) <= tol["coef_rel"] * np.abs(ce) + 1e-6 * scale)
    assert np.all(c[~active] == 0.0)


def assert_backward(got, exp, dtype, v_real):
    tol = TOL[dtype]["grad"]
    assert rel_l2(got["dH"], exp["dH"]) <= tol
    assert rel_l2(got["dW"], exp["dW"]) <= tol
    assert np.all(got["dW"][v_real:] == 0.0)
