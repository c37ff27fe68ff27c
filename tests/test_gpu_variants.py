"""GPU parity of the objective and gradient-output variants: the fixed_constant
(Dr. GRPO) normaliser, accumulation into dW, and bf16 gradient outputs."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs
from tests import gpu_support as S

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def gb():
    from lm_head_selected_amd import binding
    return binding


def _active(inp):
    return oracle.active_tokens(inp["y"], inp["mask"], inp["ignore_index"])


def _fixed(inp, c):
    inp = dict(inp)
    inp["reduction"] = "fixed_constant"
    inp["norm_const"] = c
    return inp


@pytest.mark.parametrize("ci", [0, 1, 2])
def test_fixed_constant_parity(gb, ci):
    inp, lp, lse = S.build(CONFIGS[ci])
    c = float(inp["n_tokens"])           # a generation budget: every token slot, active or not
    inp = _fixed(inp, c)
    print(f"config {CONFIGS[ci].name}, C = {c}", flush=True)
    got = S.run(gb, inp, norm_const=c)
    exp = S.expect(inp, lp, lse)
    S.assert_forward(got, exp, inp["dtype"], _active(inp))
    S.assert_backward(got, exp, inp["dtype"], inp["v_real"])


def test_fixed_constant_at_active_count_matches_token_mean(gb):
    inp, _, _ = S.build(CONFIGS[1], reduction="token_mean")
    d = S.to_device(inp)
    tm = S.run(gb, inp, d, backward=False, keep_device=True)
    T = float(_active(inp).sum())
    fc = S.run(gb, _fixed(inp, T), d, backward=False, keep_device=True, norm_const=T)
    assert torch.allclose(fc["out3"], tm["out3"], rtol=1e-6, atol=0)
    assert torch.allclose(fc["coef"], tm["coef"], rtol=1e-6, atol=0)


def test_fixed_constant_all_inactive_is_not_an_error(gb):
    cfg = dataclasses.replace(CONFIGS[1], n_tokens=512, seq_len=128)
    inp = make_inputs(cfg)
    inp["mask"][:] = 0
    inp, _, _ = S.with_oracle_logprobs(inp)
    got = S.run(gb, _fixed(inp, 256.0), backward=False, validate=True, norm_const=256.0)
    assert np.all(got["out3"] == 0.0) and np.all(got["coef"] == 0.0)


def test_accumulate_dw(gb):
    """dW (+)= the gradient: bitwise the fp32 sum of the caller's dW and the
    overwriting result (one chunk); padding rows untouched; dH overwritten."""
    inp, _, _ = S.build(CONFIGS[2])
    d = S.to_device(inp)
    base = S.run(gb, inp, d, keep_device=True)
    dev = torch.device("cuda")
    p = S.params(gb, inp, accumulate_dw=True)
    head = gb.GrpoHead(p, dev)
    head.fwd(d["H"], d["W"], d["y"], d["mask"], d["sid"], d["adv"], d["old"], d["ref"])
    g = torch.Generator(device="cpu").manual_seed(3)
    dW0 = torch.randn(inp["v_rows"], inp["d_model"], generator=g).to(dev)
    dW = dW0.clone()
    dH = torch.full((inp["n_tokens"], inp["d_model"]), 9.0, device=dev)
    head.bwd(d["H"], d["W"], d["y"], d["mask"], dH=dH, dW=dW)
    torch.cuda.synchronize()
    V = inp["v_real"]
    assert torch.equal(dW[:V], dW0[:V] + base["dW"][:V])
    assert torch.equal(dW[V:], dW0[V:])
    assert torch.equal(dH, base["dH"])


def test_accumulate_dw_over_chunks(gb):
    inp, lp, lse = S.build(CONFIGS[1])
    d = S.to_device(inp)
    dev = torch.device("cuda")
    p = S.params(gb, inp, accumulate_dw=True, chunk_tokens=256)
    head = gb.GrpoHead(p, dev)
    head.fwd(d["H"], d["W"], d["y"], d["mask"], d["sid"], d["adv"], d["old"], d["ref"])
    dW = torch.full((inp["v_rows"], inp["d_model"]), 0.5, device=dev)
    _, dW = head.bwd(d["H"], d["W"], d["y"], d["mask"], dW=dW)
    torch.cuda.synchronize()
    exp = S.expect(inp, lp, lse)
    assert S.rel_l2(dW.cpu().numpy() - 0.5, exp["dW"]) <= 1e-2


@pytest.mark.parametrize("ci", [1, 2])
def test_bf16_gradient_outputs(gb, ci):
    """bf16 dH and dW are the fp32 results rounded once to nearest even (one
    chunk), and within the gradient tolerance of the oracle."""
    inp, lp, lse = S.build(CONFIGS[ci])
    d = S.to_device(inp)
    f32 = S.run(gb, inp, d, keep_device=True)
    b16 = S.run(gb, inp, d, keep_device=True, grad_dtype="bf16")
    assert b16["dH"].dtype == torch.bfloat16 and b16["dW"].dtype == torch.bfloat16
    assert torch.equal(b16["dH"], f32["dH"].to(torch.bfloat16))
    assert torch.equal(b16["dW"], f32["dW"].to(torch.bfloat16))
    exp = S.expect(inp, lp, lse)
    assert S.rel_l2(b16["dH"].float().cpu().numpy(), exp["dH"]) <= 1e-2
    assert S.rel_l2(b16["dW"].float().cpu().numpy(), exp["dW"]) <= 1e-2
    assert torch.all(b16["dW"][inp["v_real"]:] == 0).item()


def test_bf16_gradient_outputs_chunked(gb):
    inp, lp, lse = S.build(CONFIGS[1])
    got = S.run(gb, inp, keep_device=True, grad_dtype="bf16", chunk_tokens=256)
    exp = S.expect(inp, lp, lse)
    assert S.rel_l2(got["dH"].float().cpu().numpy(), exp["dH"]) <= 1e-2
    assert S.rel_l2(got["dW"].float().cpu().numpy(), exp["dW"]) <= 1e-2
