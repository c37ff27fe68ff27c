"""GPU parity of the backward's row compaction: only tokens with a non-zero
gradient scale g_t = grad_output * coef_t / tau run through the dlogits, dH and dW
products.  The cases put the live-row count on and around the 256-row tile
edges, across the 1024-token compaction blocks, in token chunks with no live row
at all, and at zero (a zero grad_output, clipped tokens without a KL term)."""
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


# 1536 tokens (two compaction blocks, six token tiles), D=256, V=5000 (ragged tail)
_CFG = dataclasses.replace(CONFIGS[2], n_tokens=1536, seq_len=512, mask_frac=0.0)


def _with_live(n_live: int, seed: int):
    inp = make_inputs(_CFG)
    rng = np.random.default_rng(seed)
    keep = rng.choice(_CFG.n_tokens, size=n_live, replace=False)
    inp["mask"] = np.zeros(_CFG.n_tokens, np.uint8)
    inp["mask"][keep] = 1
    return S.with_oracle_logprobs(inp)


@pytest.mark.parametrize("n_live", [1, 255, 256, 257, 1023, 1025, 1535])
@pytest.mark.parametrize("chunk", [0, 512])
def test_live_rows_around_tile_edges(gb, n_live, chunk):
    print(f"live rows {n_live}, chunk {chunk}", flush=True)
    inp, lp, lse = _with_live(n_live, seed=n_live)
    act = _active(inp)
    got = S.run(gb, inp, chunk_tokens=chunk)
    exp = S.expect(inp, lp, lse)
    S.assert_forward(got, exp, "bf16", act)
    S.assert_backward(got, exp, "bf16", inp["v_real"])
    assert np.all(got["dH"][~act] == 0.0)


def test_chunks_without_live_rows(gb):
    """Chunks of 256 tokens whose tokens are all masked, first and in the middle:
    the first writes a zero dW, the middle one adds nothing."""
    inp = make_inputs(_CFG)
    inp["mask"] = np.ones(_CFG.n_tokens, np.uint8)
    inp["mask"][0:256] = 0
    inp["mask"][768:1024] = 0
    inp, lp, lse = S.with_oracle_logprobs(inp)
    act = _active(inp)
    got = S.run(gb, inp, chunk_tokens=256)
    exp = S.expect(inp, lp, lse)
    S.assert_backward(got, exp, "bf16", inp["v_real"])
    assert np.all(got["dH"][~act] == 0.0)
    whole = S.run(gb, inp)
    assert S.rel_l2(whole["dW"], exp["dW"]) <= S.TOL["bf16"]["grad"]


def test_zero_grad_output_gives_zero_gradients(gb):
    inp, _, _ = S.build(CONFIGS[1])
    got = S.run(gb, inp, grad_output=0.0)
    assert np.all(got["dH"] == 0.0) and np.all(got["dW"] == 0.0)
    assert np.all(np.isfinite(got["dH"])) and np.all(np.isfinite(got["dW"]))


def test_clipped_tokens_without_kl_are_skipped(gb):
    """beta = 0 and old-policy noise N(0, 0.3): the clipped tokens have coef = 0 and
    drop out of the backward; the gradients still match the oracle's."""
    cfg = dataclasses.replace(CONFIGS[1], beta=0.0, ref_noise=None)
    inp = make_inputs(cfg, old_noise=0.3)
    inp, lp, lse = S.with_oracle_logprobs(inp)
    act = _active(inp)
    exp = S.expect(inp, lp, lse)
    dead = act & (exp["coef"] == 0.0)
    assert dead.sum() > 0.1 * act.sum()
    for chunk in (0, 256):
        got = S.run(gb, inp, chunk_tokens=chunk)
        S.assert_forward(got, exp, "bf16", act)
        S.assert_backward(got, exp, "bf16", inp["v_real"])
        assert np.all(got["dH"][dead] == 0.0)


def test_fp32_path_with_sparse_live_rows(gb):
    """The fp32 operand path (32 tokens per K stage) with 37 live rows of 300."""
    cfg = dataclasses.replace(CONFIGS[0], n_tokens=300, seq_len=100, mask_frac=0.0)
    inp = make_inputs(cfg)
    rng = np.random.default_rng(7)
    inp["mask"] = np.zeros(cfg.n_tokens, np.uint8)
    inp["mask"][rng.choice(cfg.n_tokens, size=37, replace=False)] = 1
    inp, lp, lse = S.with_oracle_logprobs(inp)
    act = _active(inp)
    got = S.run(gb, inp)
    exp = S.expect(inp, lp, lse)
    S.assert_forward(got, exp, "f32", act)
    S.assert_backward(got, exp, "f32", inp["v_real"])
    assert np.all(got["dH"][~act] == 0.0)


def test_compacted_backward_is_bitwise_repeatable(gb):
    inp, _, _ = _with_live(700, seed=3)
    d = S.to_device(inp)
    a = S.run(gb, inp, d, keep_device=True, chunk_tokens=512)
    b = S.run(gb, inp, d, keep_device=True, chunk_tokens=512)
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("chunk", [0, 66560])
def test_many_compaction_blocks(gb, chunk):
    """A chunk of 70000 tokens has 69 compaction blocks of 1024, beyond the 64 for
    which each block sums the counts before it itself: the block offsets then come
    from the scan kernel.  30% of the tokens are masked, scattered over every
    block; with chunks of 66560 tokens the first chunk takes the scan (65 blocks)
    and the second the in-block sum."""
    print(f"70000 tokens, chunk {chunk}", flush=True)
    cfg = dataclasses.replace(CONFIGS[2], n_tokens=70000, seq_len=1000, d_model=64, v_real=300,
                              v_rows=320, mask_frac=0.3)
    inp, lp, lse = S.build(cfg)
    act = _active(inp)
    got = S.run(gb, inp, chunk_tokens=chunk)
    exp = S.expect(inp, lp, lse)
    S.assert_forward(got, exp, "bf16", act)
    S.assert_backward(got, exp, "bf16", inp["v_real"])
    assert np.all(got["dH"][~act] == 0.0)
