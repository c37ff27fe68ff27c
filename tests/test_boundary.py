"""C-ABI boundary tests that need no GPU: the library loads, exports every
function include/grpo_head.h declares, and rejects bad arguments on the host
before touching the device."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

gb = pytest.importorskip("lm_head_selected_amd.binding",
                         reason="libgrpo_head.so not built (run __graft_entry__.build())")

HEADER = os.path.join(ROOT, "include", "grpo_head.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if"})


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(gb.EXPORTS), names
    lib = ctypes.CDLL(gb.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_params_struct_layout_matches_header():
    # 7 int64 + 4 int32 + 5 float + 3 int32, no padding
    assert ctypes.sizeof(gb.Params) == 7 * 8 + 4 * 4 + 5 * 4 + 3 * 4
    text = open(HEADER).read()
    body = re.search(r"typedef struct grpo_head_params \{(.*?)\}", text, re.S).group(1)
    fields = re.findall(r"\b(\w+);", body)
    assert fields == [f[0] for f in gb.Params._fields_]


def P(**kw):
    base = dict(n_tokens=1024, d_model=1024, v_real=4096, v_rows=4096, n_seqs=8, dtype="bf16",
                reduction="sequence_mean", inv_tau=1.0, eps_low=0.2, eps_high=0.2, beta=0.1)
    base.update(kw)
    return gb.make_params(**base)


def test_workspace_sizes():
    assert gb.fwd_workspace_size(P(reduction="fixed_constant", norm_const=4096.0)) > 0
    assert gb.workspace_size(P(grad_dtype="bf16", accumulate_dw=True)) > 0
    bad = P()
    bad.reserved = 1
    assert gb.workspace_size(bad) == 0
    p = P()
    fwd = gb.fwd_workspace_size(p)
    full = gb.workspace_size(p)
    # partials: 16 tiles x 1024 tokens x 8 B dominate the forward workspace
    assert fwd >= 16 * 1024 * 8
    # backward: the chunk's dlogits over the padded vocabulary, bf16
    assert full >= 1024 * 4096 * 2
    assert full >= fwd
    # fp32 path doubles the dlogits buffer
    assert gb.workspace_size(P(dtype="f32")) > full
    # chunking bounds the backward workspace
    assert gb.workspace_size(P(chunk_tokens=256)) < full
    assert gb.segment_workspace_size(P(d_model=0)) > 0


@pytest.mark.parametrize("bad", [dict(d_model=100), dict(d_model=0), dict(v_real=0),
                                 dict(v_rows=10), dict(n_seqs=0), dict(n_tokens=-1),
                                 dict(dtype=7), dict(reduction=5), dict(level=3),
                                 dict(inv_tau=0.0), dict(eps_low=1.0), dict(eps_low=-0.1),
                                 dict(beta=-1.0), dict(inv_tau=float("nan")),
                                 dict(chunk_tokens=-5), dict(reduction="fixed_constant"),
                                 dict(reduction="fixed_constant", norm_const=-2.0),
                                 dict(reduction="fixed_constant", norm_const=8.0,
                                      level="sequence_gspo"),
                                 dict(grad_dtype=5), dict(accumulate_dw=3)])
def test_invalid_params_rejected_without_gpu(bad):
    p = P(**bad)
    assert gb.workspace_size(p) == 0
    with pytest.raises(gb.GrpoHeadError) as e:
        gb.grpo_head_fwd(p, 1, 1, 1, None, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, ws_bytes=1 << 40,
                         stream=0)
    assert e.value.status == 1
    assert gb.lib.grpo_head_last_error().decode()


def test_null_buffers_rejected():
    p = P()
    with pytest.raises(gb.GrpoHeadError) as e:   # out3 NULL
        gb.grpo_head_fwd(p, 1, 1, 1, None, 1, 1, 1, 1, 1, 1, None, 1, 1, 1, ws_bytes=1 << 40,
                         stream=0)
    assert e.value.status == 1
    with pytest.raises(gb.GrpoHeadError) as e:   # beta > 0 without ref_logp
        gb.grpo_head_fwd(p, 1, 1, 1, None, 1, 1, 1, None, 1, 1, 1, 1, 1, 1, ws_bytes=1 << 40,
                         stream=0)
    assert e.value.status == 1 and "ref_logp" in str(e.value)
    with pytest.raises(gb.GrpoHeadError) as e:   # dW NULL
        gb.grpo_head_bwd(p, 1, 1, 1, None, 1, 1, None, 1, None, 1, ws_bytes=1 << 40, stream=0)
    assert e.value.status == 1


def test_workspace_too_small_rejected():
    p = P()
    need = gb.fwd_workspace_size(p)
    with pytest.raises(gb.GrpoHeadError) as e:
        gb.grpo_head_fwd(p, 1, 1, 1, None, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, ws_bytes=need - 1,
                         stream=0)
    assert e.value.status == 2
    with pytest.raises(gb.GrpoHeadError) as e:
        gb.grpo_head_bwd(p, 1, 1, 1, None, 1, 1, None, 1, 1, 1,
                         ws_bytes=gb.workspace_size(p) - 1, stream=0)
    assert e.value.status == 2
    q = P(level="sequence_gspo")
    with pytest.raises(gb.GrpoHeadError) as e:
        gb.gspo_segment_reduce(q, 1, 1, 1, None, 1, 1, 1, 1, 1, None, 1, 1,
                               ws_bytes=gb.segment_workspace_size(q) - 1, stream=0)
    assert e.value.status == 2


def test_segment_reduce_needs_targets_without_mask():
    q = P(level="sequence_gspo", beta=0.0)
    with pytest.raises(gb.GrpoHeadError) as e:
        gb.gspo_segment_reduce(q, 1, 1, None, None, None, 1, 1, 1, 1, None, 1, 1,
                               ws_bytes=1 << 30, stream=0)
    assert e.value.status == 1 and "mask" in str(e.value)


def test_logp_entry_checks_only_its_fields():
    # the objective and sequence fields play no part in the forward-only log-probs
    junk = P(n_seqs=0, eps_low=5.0, beta=-1.0, reduction=9, level=7)
    size = gb.logp_workspace_size(junk)
    assert size >= 16 * 1024 * 8                      # the per-tile partials
    assert size == gb.logp_workspace_size(P(n_seqs=3))
    assert size <= gb.fwd_workspace_size(P())
    for bad in (dict(d_model=100), dict(v_real=0), dict(v_rows=10), dict(dtype=7),
                dict(inv_tau=0.0), dict(n_tokens=-1)):
        p = P(**bad)
        assert gb.logp_workspace_size(p) == 0
        with pytest.raises(gb.GrpoHeadError) as e:
            gb.grpo_head_logp(p, 1, 1, 1, None, 1, 1, 1, ws_bytes=1 << 40, stream=0)
        assert e.value.status == 1


def test_logp_entry_rejects_null_buffers_and_small_workspace():
    p = P()
    with pytest.raises(gb.GrpoHeadError) as e:   # y NULL
        gb.grpo_head_logp(p, 1, 1, None, 1, 1, 1, 1, ws_bytes=1 << 40, stream=0)
    assert e.value.status == 1
    with pytest.raises(gb.GrpoHeadError) as e:   # lse NULL
        gb.grpo_head_logp(p, 1, 1, 1, None, 1, None, 1, ws_bytes=1 << 40, stream=0)
    assert e.value.status == 1
    with pytest.raises(gb.GrpoHeadError) as e:
        gb.grpo_head_logp(p, 1, 1, 1, None, 1, 1, 1, ws_bytes=gb.logp_workspace_size(p) - 1,
                          stream=0)
    assert e.value.status == 2


@pytest.mark.parametrize("n,G,eps,scale", [(8, 0, 0.0, 1), (8, 3, 0.0, 1), (8, 4, -1.0, 1),
                                           (8, 4, float("nan"), 1), (8, 4, 0.0, 2),
                                           (-4, 4, 0.0, 1)])
def test_advantage_rejects_bad_arguments(n, G, eps, scale):
    rc = gb.lib.grpo_group_advantage(1, n, G, eps, scale, 1, 0)
    assert rc == 1 and gb.lib.grpo_head_last_error().decode()


def test_advantage_null_buffers_and_empty():
    assert gb.lib.grpo_group_advantage(None, 8, 4, 0.0, 1, 1, 0) == 1
    assert gb.lib.grpo_group_advantage(None, 0, 4, 0.0, 1, None, 0) == 0   # nothing to do


def test_shard_bounds():
    p = P(v_real=5000, v_rows=5120)
    N = 1024
    assert gb.shard_partials_bytes(p, 0, 2560) == 10 * N * 8
    assert gb.shard_partials_bytes(p, 2560, 5120) == 10 * N * 8    # ragged end: 2440 rows
    assert gb.shard_partials_bytes(p, 4864, 5001) == 1 * N * 8     # end past v_real
    for lo, hi in [(100, 2560), (0, 2500), (2560, 2560), (-256, 256), (0, 5121)]:
        assert gb.shard_partials_bytes(p, lo, hi) == 0, (lo, hi)
        rc = gb.lib.grpo_head_shard_partials(ctypes.byref(p), lo, hi, 1, 1, 1, None, 1, 1, 0)
        assert rc == 1
    q = P(v_real=5000, v_rows=5376)
    assert gb.shard_partials_bytes(q, 5120, 5376) == 0             # padding only: no tiles
    assert gb.lib.grpo_head_merge_partials(ctypes.byref(p), None, 1, 1, None, 1, 1, 0) == 1


def test_segment_reduce_rejects_fixed_constant():
    # GSPO keeps its segment mean: a block asking for the fixed_constant normaliser
    # is rejected by the standalone seam as by grpo_head_fwd, whatever its level says
    for level in ("token", "sequence_gspo"):
        q = P(level=level, reduction="fixed_constant", norm_const=64.0, beta=0.0)
        assert gb.segment_workspace_size(q) == 0
        with pytest.raises(gb.GrpoHeadError) as e:
            gb.gspo_segment_reduce(q, 1, 1, None, 1, None, 1, 1, 1, 1, None, 1, 1,
                                   ws_bytes=1 << 30, stream=0)
        assert e.value.status == 1 and "fixed_constant" in str(e.value)
    assert gb.segment_workspace_size(P(level="token", beta=0.0)) > 0


def test_noalloc_logp_rejects_on_the_host():
    # argument checks run before any HIP call: a NULL buffer or a problem whose
    # scratch exceeds the static array is rejected with status 1, nothing enqueued
    p = gb.make_params(n_tokens=20000, d_model=4096, v_real=151936, v_rows=152064, n_seqs=0,
                       dtype="bf16")
    assert gb.logp_workspace_size(p) > gb.NOALLOC_SCRATCH_BYTES
    with pytest.raises(gb.GrpoHeadError) as e:
        gb.grpo_head_logp_noalloc(p, 1, 1, 1, None, 1, 1, stream=0)
    assert e.value.status == 1 and "scratch" in str(e.value)
    q = gb.make_params(n_tokens=8192, d_model=4096, v_real=151936, v_rows=152064, n_seqs=0,
                       dtype="bf16")
    assert gb.logp_workspace_size(q) <= gb.NOALLOC_SCRATCH_BYTES
    with pytest.raises(gb.GrpoHeadError) as e:
        gb.grpo_head_logp_noalloc(q, 1, 1, None, None, 1, 1, stream=0)
    assert e.value.status == 1
    assert gb.lib.grpo_head_logp_noalloc(None, 1, 1, 1, None, 1, 1, None) == 1
