"""One GPU's share of a vocabulary-parallel forward: each vocabulary shard's
partials and target logits on the global tile grid (grpo_head_shard_partials),
gathered in shard order and merged (grpo_head_merge_partials), must be bitwise
the single-GPU log-probs for every shard count; and the oracle agrees."""
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


def _single(gb, inp, d):
    p = S.params(gb, inp)
    ws = torch.empty(gb.logp_workspace_size(p), dtype=torch.uint8, device="cuda")
    n = inp["n_tokens"]
    lp = torch.empty(n, dtype=torch.float32, device="cuda")
    lse = torch.empty_like(lp)
    gb.grpo_head_logp(p, d["H"], d["W"], d["y"], d["mask"], lp, lse, ws)
    return lp, lse


def _sharded(gb, inp, d, bounds):
    """Run each shard into its slice of one gathered partials buffer (what an
    all-gather in shard order produces), add the shards' zy in shard order, merge."""
    p = S.params(gb, inp)
    n, D, V = inp["n_tokens"], inp["d_model"], inp["v_real"]
    n_vt = -(-V // 256)
    gathered = torch.full((n_vt * n * 2,), float("nan"), dtype=torch.float32, device="cuda")
    zy = torch.zeros(n, dtype=torch.float32, device="cuda")
    off = 0
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        nbytes = gb.shard_partials_bytes(p, lo, hi)
        part = gathered[off // 4: (off + nbytes) // 4]
        zs = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        w_shard = d["W"][lo:hi].contiguous()              # this rank's rows only
        gb.grpo_head_shard_partials(p, lo, hi, d["H"], w_shard, d["y"], d["mask"], part, zs)
        torch.cuda.synchronize()
        assert not torch.isnan(zs).any()                   # written for every token
        zy += zs
        off += nbytes
    assert off == n_vt * n * 8
    lp = torch.empty(n, dtype=torch.float32, device="cuda")
    lse = torch.empty_like(lp)
    gb.grpo_head_merge_partials(p, gathered, zy, d["y"], d["mask"], lp, lse)
    torch.cuda.synchronize()
    return lp, lse


def _bounds(v_rows, v_real, k):
    """k shards on the 256-row grid, the last one taking the ragged end and padding."""
    tiles = -(-v_real // 256)
    cuts = [round(i * tiles / k) * 256 for i in range(k)]
    return cuts + [v_rows]


@pytest.mark.parametrize("ci", [1, 2])
@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_sharded_logp_is_bitwise_the_single_gpu_result(gb, ci, k):
    inp, lp_o, lse_o = S.build(CONFIGS[ci])
    d = S.to_device(inp)
    bounds = _bounds(inp["v_rows"], inp["v_real"], k)
    print(f"config {CONFIGS[ci].name}, shards {bounds}", flush=True)
    lp1, lse1 = _single(gb, inp, d)
    lpk, lsek = _sharded(gb, inp, d, bounds)
    assert torch.equal(lp1, lpk) and torch.equal(lse1, lsek)
    act = oracle.active_tokens(inp["y"], inp["mask"], inp["ignore_index"])
    tol = S.TOL[inp["dtype"]]
    assert np.max(np.abs(lpk.cpu().numpy() - lp_o)) <= tol["logp"]
    assert np.max(np.abs(lsek.cpu().numpy() - lse_o)) <= tol["lse"]
    assert np.all(lpk.cpu().numpy()[~act] == 0.0)


def test_uneven_shards_and_a_one_tile_shard(gb):
    inp, _, _ = S.build(CONFIGS[2])
    d = S.to_device(inp)
    bounds = [0, 256, 512, 3072, inp["v_rows"]]
    lp1, lse1 = _single(gb, inp, d)
    lpk, lsek = _sharded(gb, inp, d, bounds)
    assert torch.equal(lp1, lpk) and torch.equal(lse1, lsek)
