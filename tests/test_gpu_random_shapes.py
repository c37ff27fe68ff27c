"""GPU parity on a seeded sweep of small random shapes that the named workloads do not
reach: token counts from 1 upward, hidden sizes of 64 to 320 (odd and even numbers
of K stages, so both forward tile kernels run), real vocabularies from 1 row with
0 to 256 padded rows, token chunks, mask densities up to every token inactive,
both reductions and both element types.  Each case is checked against the oracle,
dead tokens' dH rows must be exactly zero, and a repeat must be bitwise equal."""
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
