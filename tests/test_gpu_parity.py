"""GPU parity of the HIP path against the fp64 oracle, element by element, on the
small workloads (several tiles plus ragged tails) and the edge cases."""
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


@pytest.mark.parametrize("ci", [0, 1, 2])
def test_parity_small_configs(gb, ci):
    inp, lp, lse = S.build(CONFIGS[ci])
    print(f"config {CONFIGS[ci].name}", flush=True)
    got = S.run(gb, inp)
    exp = S.expect(inp, lp, lse)
    S.assert_forward(got, exp, inp["dtype"], _active(inp))
    S.assert_backward(got, exp, inp["dtype"], inp["v_real"])


@pytest.mark.parametrize("ci", [0, 1, 2])
def test_bitwise_repeatable(gb, ci):
    inp, _, _ = S.build(CONFIGS[ci])
    d = S.to_device(inp)
    a = S.run(gb, inp, d, keep_device=True)
    b = S.run(gb, inp, d, keep_device=True)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_chunked_backward(gb):
    """Token chunks of 256: dW accumulated chunk by chunk in ascending order."""
    inp, lp, lse = S.build(CONFIGS[1])
    got = S.run(gb, inp, chunk_tokens=256)
    exp = S.expect(inp, lp, lse)
    S.assert_backward(got, exp, "bf16", inp["v_real"])
    again = S.run(gb, inp, chunk_tokens=256)
    assert np.array_equal(got["dW"], again["dW"])


def test_grad_output_scaling(gb):
    inp, lp, lse = S.build(CONFIGS[2])
    got = S.run(gb, inp, grad_output=-2.5)
    exp = S.expect(inp, lp, lse, grad_output=-2.5)
    S.assert_backward(got, exp, "bf16", inp["v_real"])


def test_padded_vocab_nan_rows_never_read(gb):
    """v_rows > v_real with NaN pad rows: results finite, dW pad rows exactly 0."""
    cfg = dataclasses.replace(CONFIGS[2], v_real=1000, v_rows=1300, n_tokens=512, seq_len=512)
    inp, lp, lse = S.build(cfg)
    assert np.isnan(S.oracle.widen(inp["W"][1000:], "bf16")).all()
    got = S.run(gb, inp)
    exp = S.expect(inp, lp, lse)
    S.assert_forward(got, exp, "bf16", _active(inp))
    S.assert_backward(got, exp, "bf16", 1000)
    assert np.all(got["dW"][1000:] == 0.0)


def test_clip_branches_forced(gb):
    """Old-policy noise N(0, 0.3): a large share of ratios is clipped, both ways."""
    cfg = CONFIGS[1]
    inp = make_inputs(cfg, old_noise=0.3)
    inp, lp, lse = S.with_oracle_logprobs(inp)
    exp = S.expect(inp, lp, lse)
    act = _active(inp)
    clipped = (~exp["unclipped"]) & act
    assert clipped.sum() > 0.1 * act.sum()
    got = S.run(gb, inp)
    S.assert_forward(got, exp, "bf16", act)
    S.assert_backward(got, exp, "bf16", inp["v_real"])
    # with beta = 0 the clipped tokens carry no gradient at all
    inp0 = dict(inp, beta=0.0)
    exp0 = S.expect(inp0, lp, lse, backward=False)
    got0 = S.run(gb, inp0, backward=False)
    assert np.all(got0["coef"][clipped] == 0.0)
    S.assert_forward(got0, exp0, "bf16", act)


def test_targets_at_tile_edges(gb):
    cfg = dataclasses.replace(CONFIGS[2], n_tokens=1024, seq_len=1024)
    inp = make_inputs(cfg)
    V = cfg.v_real
    edge = np.array([0, 1, 127, 128, 255, 256, 257, 511, 512, V - 257, V - 256, V - 1])
    inp["y"][: len(edge)] = edge
    inp["y"][len(edge): 2 * len(edge)] = V - 1
    inp, lp, lse = S.with_oracle_logprobs(inp)
    got = S.run(gb, inp)
    exp = S.expect(inp, lp, lse)
    S.assert_forward(got, exp, "bf16", _active(inp))
    S.assert_backward(got, exp, "bf16", V)


def test_ignore_index_mode(gb):
    """No mask: tokens whose target equals ignore_index are inactive."""
    cfg = dataclasses.replace(CONFIGS[2], n_tokens=768, seq_len=768)
    inp = make_inputs(cfg)
    inp["y"][::7] = -100
    inp, lp, lse = S.with_oracle_logprobs(inp)
    act = _active(inp)
    assert (~act).sum() == len(inp["y"][::7])
    got = S.run(gb, inp)
    exp = S.expect(inp, lp, lse)
    S.assert_forward(got, exp, "bf16", act)
    S.assert_backward(got, exp, "bf16", cfg.v_real)
    assert np.all(got["dH"][~act] == 0.0)


def test_fully_masked_sequence(gb):
    cfg = CONFIGS[1]
    inp = make_inputs(cfg)
    inp["mask"][128:256] = 0                        # sequence 1 has no active token
    inp, lp, lse = S.with_oracle_logprobs(inp)
    got = S.run(gb, inp)
    exp = S.expect(inp, lp, lse)
    assert exp["counts"][1] == 0
    S.assert_forward(got, exp, "bf16", _active(inp))
    S.assert_backward(got, exp, "bf16", cfg.v_real)


def test_all_tokens_inactive(gb):
    cfg = dataclasses.replace(CONFIGS[1], n_tokens=512, seq_len=128)
    inp = make_inputs(cfg)
    inp["mask"][:] = 0
    inp, lp, lse = S.with_oracle_logprobs(inp)
    got = S.run(gb, inp)
    assert np.all(got["out3"] == 0.0) and np.all(got["coef"] == 0.0)
    assert np.all(got["logp"] == 0.0) and np.all(got["counts"] == 0)
    assert np.all(got["dH"] == 0.0) and np.all(got["dW"] == 0.0)
    assert np.max(np.abs(got["lse"] - lse)) <= 2e-3
    with pytest.raises(gb.GrpoHeadError) as e:
        S.run(gb, inp, backward=False, validate=True)
    assert e.value.status == 3


def test_empty_batch(gb):
    dev = torch.device("cuda")
    p = gb.make_params(n_tokens=0, d_model=64, v_real=300, v_rows=320, n_seqs=3, dtype="bf16",
                       beta=0.1)
    head = gb.GrpoHead(p, dev)
    adv = torch.ones(3, device=dev)
    W = torch.randn(320, 64, device=dev).to(torch.bfloat16)
    head.out3.fill_(7.0)
    head.counts.fill_(9)
    head.fwd(None, W, None, None, None, adv, None, None)
    dW = torch.full((320, 64), 5.0, device=dev)
    head.bwd(None, W, None, None, dW=dW, dH=torch.empty(0, 64, device=dev))
    torch.cuda.synchronize()
    assert head.out3.abs().sum().item() == 0.0
    assert head.counts[:3].abs().sum().item() == 0
    assert dW.abs().sum().item() == 0.0


def test_validate_reports_bad_target(gb):
    cfg = dataclasses.replace(CONFIGS[1], n_tokens=512, seq_len=128)
    inp, _, _ = S.build(cfg)
    act = _active(inp)
    t = int(np.nonzero(act)[0][3])
    inp["y"][t] = cfg.v_real + 5
    with pytest.raises(gb.GrpoHeadError) as e:
        S.run(gb, inp, backward=False, validate=True)
    assert e.value.status == 4
    got = S.run(gb, inp, backward=False)            # no validation: NaN logp, no fault
    assert np.isnan(got["logp"][t])


def test_validate_reports_nonfinite(gb):
    cfg = dataclasses.replace(CONFIGS[1], n_tokens=512, seq_len=128)
    inp, _, _ = S.build(cfg)
    d = S.to_device(inp)
    d["H"][5, 3] = float("nan")
    with pytest.raises(gb.GrpoHeadError) as e:
        S.run(gb, inp, d, backward=False, validate=True)
    assert e.value.status == 5


def test_validate_reports_decreasing_sid(gb):
    cfg = dataclasses.replace(CONFIGS[1], n_tokens=512, seq_len=128)
    inp, _, _ = S.build(cfg)
    inp["sid"][200] = 0
    with pytest.raises(gb.GrpoHeadError) as e:
        S.run(gb, inp, backward=False, validate=True)
    assert e.value.status == 4


def test_validate_passes_clean_inputs(gb):
    inp, lp, lse = S.build(CONFIGS[1])
    got = S.run(gb, inp, validate=True)
    exp = S.expect(inp, lp, lse, backward=False)
    S.assert_forward(got, exp, "bf16", _active(inp))


def test_gspo_length_one_segments(gb):
    cfg = dataclasses.replace(CONFIGS[4], n_tokens=512, d_model=256, v_real=1000, v_rows=1024,
                              seq_len=1, mask_frac=0.1)
    inp, lp, lse = S.build(cfg)
    assert inp["n_seqs"] == 512
    got = S.run(gb, inp)
    exp = S.expect(inp, lp, lse)
    S.assert_forward(got, exp, "bf16", _active(inp))
    S.assert_backward(got, exp, "bf16", cfg.v_real)


def test_gspo_small_packed_segments_with_kl(gb):
    cfg = dataclasses.replace(CONFIGS[4], n_tokens=2048, d_model=256, v_real=3000, v_rows=3000,
                              seg_len_range=(16, 300), ref_noise=0.1, beta=0.05,
                              eps_low=0.02, eps_high=0.03, mask_frac=0.1)
    inp, lp, lse = S.build(cfg)
    got = S.run(gb, inp)
    exp = S.expect(inp, lp, lse)
    S.assert_forward(got, exp, "bf16", _active(inp))
    S.assert_backward(got, exp, "bf16", cfg.v_real)


def test_gspo_segment_reduce_standalone(gb):
    """The segment stage alone, on given fp32 log-probs, against the oracle on the
    same fp32 values; also the new_logprobs metric."""
    cfg = dataclasses.replace(CONFIGS[4], n_tokens=3000, d_model=64, v_real=10, v_rows=10,
                              seg_len_range=(1, 400), ref_noise=0.1, beta=0.02, mask_frac=0.2)
    inp = make_inputs(cfg)
    g = np.random.default_rng(0)
    lp32 = (-g.random(cfg.n_tokens) * 8).astype(np.float32)
    inp = S.attach_logprobs(inp, lp32.astype(np.float64))
    exp = oracle.objective(inp, lp32.astype(np.float64))
    dev = torch.device("cuda")
    d = S.to_device(inp)
    p = S.params(gb, inp)
    n, nseg = cfg.n_tokens, inp["n_seqs"]
    out3 = torch.empty(3, device=dev)
    coef = torch.empty(n, device=dev)
    segmean = torch.empty(nseg, device=dev)
    counts = torch.empty(nseg, dtype=torch.int32, device=dev)
    ws = torch.empty(gb.segment_workspace_size(p), dtype=torch.uint8, device=dev)
    gb.gspo_segment_reduce(p, torch.from_numpy(lp32).to(dev), d["old"], d["ref"], d["mask"],
                           d["y"], d["sid"], d["adv"], out3, coef, segmean, counts, ws)
    torch.cuda.synchronize()
    got = dict(out3=out3.cpu().numpy(), coef=coef.cpu().numpy(), counts=counts.cpu().numpy(),
               logp=np.where(_active(inp), lp32, 0), lse=np.zeros(n))
    exp.update(logp=np.where(_active(inp), lp32, 0), lse=np.zeros(n))
    S.assert_forward(got, exp, "f32", _active(inp))
    np.testing.assert_allclose(segmean.cpu().numpy(), exp["seg_mean_logp"], rtol=1e-5, atol=1e-5)
