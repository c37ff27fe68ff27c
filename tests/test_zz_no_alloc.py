"""The allocation-free log-prob entry (grpo_head_logp_noalloc) against the
workspace entry (grpo_head_logp) through the C ABI: identical outputs on two calls
in a row, the second with a smaller input (the static scratch keeps the first
call's contents), plus a larger-than-scratch problem rejected before anything
runs, and parity with the fp64 oracle."""
import dataclasses

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


def _both(gb, inp):
    d = S.to_device(inp)
    p = S.params(gb, inp)
    n = inp["n_tokens"]
    ws = torch.empty(gb.logp_workspace_size(p), dtype=torch.uint8, device="cuda")
    ref = [torch.full((n,), 7.0, device="cuda") for _ in range(2)]
    got = [torch.full((n,), 7.0, device="cuda") for _ in range(2)]
    gb.grpo_head_logp(p, d["H"], d["W"], d["y"], d["mask"], ref[0], ref[1], ws)
    gb.grpo_head_logp_noalloc(p, d["H"], d["W"], d["y"], d["mask"], got[0], got[1])
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in ref], [x.cpu().numpy() for x in got]


def test_noalloc_equals_workspace_entry_twice_second_smaller(gb):
    big = CONFIGS[2]                                            # 4096 tokens, V 5000
    small = dataclasses.replace(CONFIGS[1], n_tokens=640, seq_len=128, v_real=4000,
                                v_rows=4100)                    # ragged, padded vocabulary
    for cfg in (big, small):
        print(f"case {cfg.name} n={cfg.n_tokens} v={cfg.v_real}", flush=True)
        inp, lp, lse = S.build(cfg)
        (r_lp, r_lse), (g_lp, g_lse) = _both(gb, inp)
        np.testing.assert_array_equal(g_lp, r_lp)
        np.testing.assert_array_equal(g_lse, r_lse)
        act = oracle.active_tokens(inp["y"], inp["mask"], inp["ignore_index"])
        assert np.all(g_lp[~act] == 0.0)
        tol = S.TOL[inp["dtype"]]
        assert np.max(np.abs(g_lp - lp)) <= tol["logp"]
        assert np.max(np.abs(g_lse - lse)) <= tol["lse"]


def test_noalloc_fp32_and_rejects_beyond_the_scratch(gb):
    inp, lp, lse = S.build(CONFIGS[0])
    (r_lp, r_lse), (g_lp, g_lse) = _both(gb, inp)
    np.testing.assert_array_equal(g_lp, r_lp)
    np.testing.assert_array_equal(g_lse, r_lse)
    # 20000 tokens of a 151936-row vocabulary need 95 MB of partials: rejected
    p = gb.make_params(n_tokens=20000, d_model=4096, v_real=151936, v_rows=152064, n_seqs=0,
                       dtype="bf16")
    assert gb.logp_workspace_size(p) > gb.NOALLOC_SCRATCH_BYTES
    out = torch.full((4,), 7.0, device="cuda")
    with pytest.raises(gb.GrpoHeadError) as e:
        gb.grpo_head_logp_noalloc(p, out, out, out, None, out, out)
    assert e.value.status == 1
    torch.cuda.synchronize()
    assert torch.all(out == 7.0).item()
