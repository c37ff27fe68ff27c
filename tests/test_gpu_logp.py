"""GPU parity of the forward-only selected log-prob entry (grpo_head_logp):
against the fp64 oracle element by element, bitwise against the full forward's
logp and lse, and at the full Qwen3-8B head shape against the stored fp64
log-probs of every token."""
import dataclasses
import os

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, attach_logprobs, make_inputs
from tests import gpu_support as S
from tests.golden.make_fullsize import fingerprint, path_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def gb():
    from lm_head_selected_amd import binding
    return binding


def _logp(gb, inp, d=None, **pkw):
    d = d or S.to_device(inp)
    p = S.params(gb, inp, **pkw)
    ws = torch.empty(gb.logp_workspace_size(p), dtype=torch.uint8, device="cuda")
    n = inp["n_tokens"]
    logp = torch.empty(n, dtype=torch.float32, device="cuda")
    lse = torch.empty(n, dtype=torch.float32, device="cuda")
    gb.grpo_head_logp(p, d["H"], d["W"], d["y"], d["mask"], logp, lse, ws)
    torch.cuda.synchronize()
    return logp, lse


def _check(inp, got_lp, got_lse, exp_lp, exp_lse):
    act = oracle.active_tokens(inp["y"], inp["mask"], inp["ignore_index"])
    tol = S.TOL[inp["dtype"]]
    assert np.all(got_lp[~act] == 0.0)
    assert np.max(np.abs(got_lp - exp_lp), initial=0) <= tol["logp"]
    assert np.max(np.abs(got_lse - exp_lse), initial=0) <= tol["lse"]


@pytest.mark.parametrize("ci", [0, 1, 2])
def test_logp_parity_small_configs(gb, ci):
    print(f"config {CONFIGS[ci].name}", flush=True)
    inp, lp, lse = S.build(CONFIGS[ci])
    got_lp, got_lse = (x.cpu().numpy() for x in _logp(gb, inp))
    _check(inp, got_lp, got_lse, lp, lse)


@pytest.mark.parametrize("ci", [0, 1, 2])
def test_logp_bitwise_equal_to_full_forward(gb, ci):
    inp, _, _ = S.build(CONFIGS[ci])
    d = S.to_device(inp)
    lp, lse = _logp(gb, inp, d)
    full = S.run(gb, inp, d, backward=False, keep_device=True)
    assert torch.equal(lp, full["logp"]) and torch.equal(lse, full["lse"])
    lp2, lse2 = _logp(gb, inp, d)
    assert torch.equal(lp, lp2) and torch.equal(lse, lse2)


def test_logp_ignores_objective_fields(gb):
    inp, _, _ = S.build(CONFIGS[1])
    d = S.to_device(inp)
    a = _logp(gb, inp, d)
    b = _logp(gb, inp, d, n_seqs=0, eps_low=5.0, beta=-1.0, reduction=9, level=7)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_logp_ignore_index_and_tile_edges(gb):
    """No mask (targets equal to ignore_index are inactive), targets on tile edges."""
    cfg = dataclasses.replace(CONFIGS[2], n_tokens=768, seq_len=768)
    inp = make_inputs(cfg)
    V = cfg.v_real
    edge = np.array([0, 1, 255, 256, 257, 511, 512, V - 257, V - 256, V - 1])
    inp["y"][: len(edge)] = edge
    inp["y"][len(edge)::7] = -100
    assert inp["mask"] is None
    inp, lp, lse = S.with_oracle_logprobs(inp)
    got_lp, got_lse = (x.cpu().numpy() for x in _logp(gb, inp))
    _check(inp, got_lp, got_lse, lp, lse)


def test_logp_all_inactive_is_not_an_error(gb):
    cfg = dataclasses.replace(CONFIGS[1], n_tokens=512, seq_len=128)
    inp = make_inputs(cfg)
    inp["mask"][:] = 0
    inp, lp, lse = S.with_oracle_logprobs(inp)
    got_lp, got_lse = (x.cpu().numpy() for x in _logp(gb, inp, validate=True))
    assert np.all(got_lp == 0.0)
    assert np.max(np.abs(got_lse - lse)) <= 2e-3


def test_logp_validate_reports_bad_target(gb):
    cfg = dataclasses.replace(CONFIGS[1], n_tokens=512, seq_len=128)
    inp, _, _ = S.build(cfg)
    act = oracle.active_tokens(inp["y"], inp["mask"], inp["ignore_index"])
    t = int(np.nonzero(act)[0][3])
    inp["y"][t] = cfg.v_real + 5
    with pytest.raises(gb.GrpoHeadError) as e:
        _logp(gb, inp, validate=True)
    assert e.value.status == 4
    lp, _ = _logp(gb, inp)                       # without validation: NaN, no fault
    assert np.isnan(lp[t].item())


def test_logp_empty_batch(gb):
    p = gb.make_params(n_tokens=0, d_model=64, v_real=300, v_rows=320, n_seqs=0)
    ws = torch.empty(max(gb.logp_workspace_size(p), 1), dtype=torch.uint8, device="cuda")
    gb.grpo_head_logp(p, None, None, None, None, None, None, ws)   # nothing to do, no error
    torch.cuda.synchronize()


def test_logp_fullsize(gb):
    """Qwen3-8B head, 8192 tokens: every token against the stored fp64 log-probs."""
    ci = 3
    path = path_for(ci)
    assert os.path.exists(path), f"missing {path}: run tests/golden/make_fullsize.py"
    g = np.load(path, allow_pickle=False)
    print(f"config {CONFIGS[ci].name}: building inputs", flush=True)
    inp = make_inputs(CONFIGS[ci])
    assert str(g["fingerprint"]) == fingerprint(inp), "regenerated inputs differ"
    inp = attach_logprobs(inp, g["logp"])   # old/ref are not read here, only shaped
    print("running grpo_head_logp", flush=True)
    got_lp, got_lse = (x.cpu().numpy() for x in _logp(gb, inp))
    _check(inp, got_lp, got_lse, g["logp"], g["lse"])
