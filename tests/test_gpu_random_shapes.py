"""GPU parity on a seeded sweep of small random shapes that the named workloads do not
reach: token counts from 1 upward, hidden sizes of 64 to 320 (odd and even numbers
of K stages, so both forward tile kernels run), real vocabularies from 1 row with
0 to 256 padded rows, token chunks, mask densities up to every token inactive,
both reductions and both element types; and packed GSPO segments of random
lengths with tight and loose clip bounds, with and without the KL term.  Each case
is checked against the oracle, dead tokens' dH rows must be exactly zero, and a
repeat must be bitwise equal."""
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


def _cases(n=16):
    rng = np.random.default_rng(20261202)
    out = []
    for k in range(n):
        dtype = "f32" if k % 4 == 0 else "bf16"
        seq_len = int(rng.integers(1, 200))
        n_seqs = int(rng.integers(1, 9))
        v_real = int(rng.integers(1, 1200))
        out.append(dict(
            k=k, dtype=dtype, seq_len=seq_len, n_tokens=seq_len * n_seqs,
            d_model=64 * int(rng.integers(1, 6)), v_real=v_real,
            v_rows=v_real + int(rng.choice([0, 1, 100, 256])),
            mask_frac=float(rng.choice([0.0, 0.1, 0.5, 0.95])),
            chunk=int(rng.choice([0, 256, 512])),
            reduction="sequence_mean" if k % 2 else "token_mean"))
    return out


# the extremes: a one-row vocabulary, one token, a one-row vocabulary padded to 256 rows
_EDGES = [
    dict(k=100, dtype="bf16", seq_len=50, n_tokens=300, d_model=64, v_real=1, v_rows=1,
         mask_frac=0.1, chunk=0, reduction="token_mean"),
    dict(k=101, dtype="bf16", seq_len=1, n_tokens=1, d_model=128, v_real=777, v_rows=800,
         mask_frac=0.0, chunk=0, reduction="sequence_mean"),
    dict(k=102, dtype="f32", seq_len=40, n_tokens=120, d_model=64, v_real=1, v_rows=256,
         mask_frac=0.0, chunk=256, reduction="sequence_mean"),
]

CASES = _cases(24) + _EDGES


@pytest.mark.parametrize("case", CASES, ids=lambda c: (
    f"{c['dtype']}_n{c['n_tokens']}_d{c['d_model']}_v{c['v_real']}r{c['v_rows']}"
    f"_m{c['mask_frac']}_c{c['chunk']}_{c['reduction'][:3]}"))
def test_random_shape_parity(gb, case):
    base = CONFIGS[0] if case["dtype"] == "f32" else CONFIGS[1]
    cfg = dataclasses.replace(
        base, name=f"random_{case['k']}", n_tokens=case["n_tokens"], seq_len=case["seq_len"],
        d_model=case["d_model"], v_real=case["v_real"], v_rows=case["v_rows"],
        mask_frac=case["mask_frac"], reduction=case["reduction"], seed=5000 + case["k"])
    print(f"case {case}", flush=True)
    _check(gb, cfg, case)


def _gspo_cases(n=8):
    rng = np.random.default_rng(20261203)
    out = []
    for k in range(n):
        tight = bool(k % 2)          # tight clip bounds: most segments take the clipped branch
        beta = 0.05 if k % 4 >= 2 else 0.0
        v_real = int(rng.integers(1, 1500))
        out.append(dict(
            k=200 + k, dtype="f32" if k == 3 else "bf16", n_tokens=int(rng.integers(1, 1800)),
            d_model=64 * int(rng.integers(1, 6)), v_real=v_real,
            v_rows=v_real + int(rng.choice([0, 100])),
            seg_len_range=(1, int(rng.integers(2, 400))),
            eps=(3e-4, 4e-4) if tight else (0.2, 0.2), beta=beta,
            mask_frac=float(rng.choice([0.0, 0.1, 0.5])), chunk=int(rng.choice([0, 256]))))
    return out


GSPO_CASES = _gspo_cases()


@pytest.mark.parametrize("case", GSPO_CASES, ids=lambda c: (
    f"{c['dtype']}_n{c['n_tokens']}_d{c['d_model']}_v{c['v_real']}r{c['v_rows']}"
    f"_seg{c['seg_len_range'][1]}_eps{c['eps'][0]}_b{c['beta']}_m{c['mask_frac']}"
    f"_c{c['chunk']}"))
def test_random_gspo_parity(gb, case):
    """Packed GSPO segments of random lengths, tight and loose clip bounds, with and
    without the KL term (no KL: clipped segments carry no gradient and drop out of
    the backward)."""
    cfg = dataclasses.replace(
        CONFIGS[4], name=f"random_gspo_{case['k']}", dtype=case["dtype"],
        n_tokens=case["n_tokens"], d_model=case["d_model"], v_real=case["v_real"],
        v_rows=case["v_rows"], seg_len_range=case["seg_len_range"], eps_low=case["eps"][0],
        eps_high=case["eps"][1], beta=case["beta"],
        ref_noise=0.1 if case["beta"] > 0 else None, mask_frac=case["mask_frac"],
        seed=6000 + case["k"])
    print(f"case {case}", flush=True)
    _check(gb, cfg, case)


def _check(gb, cfg, case):
    inp, lp, lse = S.with_oracle_logprobs(make_inputs(cfg))
    act = oracle.active_tokens(inp["y"], inp["mask"], inp["ignore_index"])
    d = S.to_device(inp)
    got = S.run(gb, inp, d, chunk_tokens=case["chunk"])
    exp = S.expect(inp, lp, lse)
    S.assert_forward(got, exp, case["dtype"], act)
    S.assert_backward(got, exp, case["dtype"], case["v_real"])
    assert np.all(got["dH"][~act] == 0.0)
    a = S.run(gb, inp, d, keep_device=True, chunk_tokens=case["chunk"])
    b = S.run(gb, inp, d, keep_device=True, chunk_tokens=case["chunk"])
    for key in a:
        assert torch.equal(a[key], b[key]), key
