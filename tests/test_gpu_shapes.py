"""GPU parity on ragged shapes the named workloads do not cover: token counts that
are not a multiple of the 256-token tile, hidden sizes that leave a partial
256-wide tile in the gradient products, padded vocabularies, and token chunks with
a short last chunk, on both element types."""
import dataclasses

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


SHAPES = {
    "bf16_n700_d320_v1500": dict(base=1, n_tokens=700, seq_len=100, d_model=320, v_real=1500,
                                 v_rows=1536),
    "bf16_n260_d64_v257": dict(base=1, n_tokens=260, seq_len=65, d_model=64, v_real=257,
                               v_rows=300),
    "f32_n300_d192_v700": dict(base=0, n_tokens=300, seq_len=60, d_model=192, v_real=700,
                               v_rows=768),
}


@pytest.mark.parametrize("name", sorted(SHAPES))
@pytest.mark.parametrize("chunk", [0, 256])
def test_ragged_shape_parity(gb, name, chunk):
    kw = dict(SHAPES[name])
    base = CONFIGS[kw.pop("base")]
    cfg = dataclasses.replace(base, name=name, **kw)
    print(f"shape {name}, chunk {chunk}", flush=True)
    inp, lp, lse = S.build(cfg)
    d = S.to_device(inp)
    got = S.run(gb, inp, d, chunk_tokens=chunk)
    exp = S.expect(inp, lp, lse)
    act = oracle.active_tokens(inp["y"], inp["mask"], inp["ignore_index"])
    S.assert_forward(got, exp, inp["dtype"], act)
    S.assert_backward(got, exp, inp["dtype"], inp["v_real"])
    again = S.run(gb, inp, d, chunk_tokens=chunk, keep_device=True)
    for k in ("logp", "lse", "coef", "dH", "dW"):
        assert (again[k].cpu().numpy() == got[k]).all(), k
