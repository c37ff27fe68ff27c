"""ctypes binding over libgrpo_head.so (the C ABI in include/grpo_head.h).

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  If the
library has not been built the import fails loudly; nothing here computes a
result on the CPU.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libgrpo_head.so")

BF16, F32 = 0, 1
TOKEN_MEAN, SEQUENCE_MEAN, FIXED_CONSTANT = 0, 1, 2
GRAD_F32, GRAD_BF16 = 0, 1
LEVEL_TOKEN, LEVEL_SEQUENCE_GSPO = 0, 1

STATUS = {0: "OK", 1: "INVALID_ARGUMENT", 2: "WORKSPACE_TOO_SMALL", 3: "NO_ACTIVE_TOKENS",
          4: "TARGET_OUT_OF_RANGE", 5: "NONFINITE", 6: "HIP_ERROR"}

EXPORTS = ("grpo_head_fwd_workspace_size", "grpo_head_workspace_size",
           "gspo_segment_workspace_size", "grpo_head_fwd", "grpo_head_bwd",
           "gspo_segment_reduce", "grpo_head_logp", "grpo_head_logp_workspace_size",
           "grpo_group_advantage", "grpo_head_shard_partials", "grpo_head_shard_partials_bytes",
           "grpo_head_merge_partials", "grpo_head_set_stage_events", "grpo_head_last_error",
           "grpo_head_logp_noalloc")

NOALLOC_SCRATCH_BYTES = 64 << 20   # GRPO_HEAD_NOALLOC_SCRATCH_BYTES

# stage-event slots recorded by grpo_head_fwd / grpo_head_bwd
N_STAGE_EVENTS = 8
STAGES = {"fwd_tiles": (0, 1), "fwd_tail": (1, 2), "fwd_objective": (2, 3),
          "bwd_prep": (4, 5), "bwd_dlogits": (5, 6), "bwd_grads": (6, 7)}
# stages that are exactly one matrix-core launch, with that launch's kernel symbol stem
GEMM_STAGES = {"fwd_tiles": "fwd_tile_chain_kernel", "bwd_dlogits": "dlogits_kernel",
               "bwd_grads": "grad_products_kernel<__bf16, float>"}


class GrpoHeadError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("d_model", ctypes.c_int64),
                ("v_real", ctypes.c_int64), ("v_rows", ctypes.c_int64),
                ("n_seqs", ctypes.c_int64), ("ignore_index", ctypes.c_int64),
                ("chunk_tokens", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("reduction", ctypes.c_int32), ("level", ctypes.c_int32),
                ("validate", ctypes.c_int32), ("inv_tau", ctypes.c_float),
                ("eps_low", ctypes.c_float), ("eps_high", ctypes.c_float),
                ("beta", ctypes.c_float), ("norm_const", ctypes.c_float),
                ("accumulate_dw", ctypes.c_int32), ("grad_dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m "
                          "lm_head_selected_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    pp = ctypes.POINTER(Params)
    for name in ("grpo_head_fwd_workspace_size", "grpo_head_workspace_size",
                 "gspo_segment_workspace_size", "grpo_head_logp_workspace_size"):
        getattr(lib, name).argtypes = [pp]
        getattr(lib, name).restype = sz
    lib.grpo_head_fwd.argtypes = [pp] + [vp] * 13 + [vp, sz, vp]
    lib.grpo_head_fwd.restype = i32
    lib.grpo_head_bwd.argtypes = [pp] + [vp] * 9 + [vp, sz, vp]
    lib.grpo_head_bwd.restype = i32
    lib.gspo_segment_reduce.argtypes = [pp] + [vp] * 11 + [vp, sz, vp]
    lib.gspo_segment_reduce.restype = i32
    lib.grpo_head_logp.argtypes = [pp] + [vp] * 6 + [vp, sz, vp]
    lib.grpo_head_logp.restype = i32
    lib.grpo_head_logp_noalloc.argtypes = [pp] + [vp] * 6 + [vp]
    lib.grpo_head_logp_noalloc.restype = i32
    lib.grpo_group_advantage.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                         ctypes.c_int32, vp, vp]
    lib.grpo_group_advantage.restype = i32
    i64 = ctypes.c_int64
    lib.grpo_head_shard_partials.argtypes = [pp, i64, i64] + [vp] * 6 + [vp]
    lib.grpo_head_shard_partials.restype = i32
    lib.grpo_head_shard_partials_bytes.argtypes = [pp, i64, i64]
    lib.grpo_head_shard_partials_bytes.restype = sz
    lib.grpo_head_merge_partials.argtypes = [pp] + [vp] * 6 + [vp]
    lib.grpo_head_merge_partials.restype = i32
    lib.grpo_head_set_stage_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), i32]
    lib.grpo_head_set_stage_events.restype = i32
    lib.grpo_head_last_error.argtypes = []
    lib.grpo_head_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def make_params(*, n_tokens, d_model, v_real, v_rows=None, n_seqs, dtype="bf16",
                reduction="token_mean", level="token", inv_tau=1.0, eps_low=0.2,
                eps_high=0.2, beta=0.0, ignore_index=-100, chunk_tokens=0,
                validate=False, norm_const=0.0, accumulate_dw=False,
                grad_dtype="f32") -> Params:
    return Params(n_tokens=n_tokens, d_model=d_model, v_real=v_real,
                  v_rows=v_real if v_rows is None else v_rows, n_seqs=n_seqs,
                  ignore_index=ignore_index, chunk_tokens=chunk_tokens,
                  dtype={"bf16": BF16, "f32": F32}[dtype] if isinstance(dtype, str) else dtype,
                  reduction={"token_mean": TOKEN_MEAN, "sequence_mean": SEQUENCE_MEAN,
                             "fixed_constant": FIXED_CONSTANT}[reduction]
                  if isinstance(reduction, str) else reduction,
                  level={"token": LEVEL_TOKEN, "sequence_gspo": LEVEL_SEQUENCE_GSPO}[level]
                  if isinstance(level, str) else level,
                  validate=int(bool(validate)), inv_tau=inv_tau, eps_low=eps_low,
                  eps_high=eps_high, beta=beta, norm_const=norm_const,
                  accumulate_dw=int(accumulate_dw),
                  grad_dtype={"f32": GRAD_F32, "bf16": GRAD_BF16}[grad_dtype]
                  if isinstance(grad_dtype, str) else grad_dtype, reserved=0)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(rc: int):
    if rc != 0:
        raise GrpoHeadError(rc, lib.grpo_head_last_error().decode())


def set_stage_events(events) -> None:
    """Record the given torch.cuda.Event objects (or raw handles / None) at stage
    boundaries of later fwd/bwd calls; None switches timing off."""
    if events is None:
        _check(lib.grpo_head_set_stage_events(None, 0))
        return
    raw = [None if e is None else (e if isinstance(e, int) else e.cuda_event) for e in events]
    arr = (ctypes.c_void_p * len(raw))(*raw)
    _check(lib.grpo_head_set_stage_events(arr, len(raw)))


def fwd_workspace_size(p: Params) -> int:
    return lib.grpo_head_fwd_workspace_size(ctypes.byref(p))


def workspace_size(p: Params) -> int:
    return lib.grpo_head_workspace_size(ctypes.byref(p))


def segment_workspace_size(p: Params) -> int:
    return lib.gspo_segment_workspace_size(ctypes.byref(p))


def logp_workspace_size(p: Params) -> int:
    return lib.grpo_head_logp_workspace_size(ctypes.byref(p))


def grpo_head_fwd(p, H, W, y, mask, sid, adv, old_logp, ref_logp, logp, lse, out3, coef,
                  counts, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib.grpo_head_fwd(ctypes.byref(p), _ptr(H), _ptr(W), _ptr(y), _ptr(mask), _ptr(sid),
                             _ptr(adv), _ptr(old_logp), _ptr(ref_logp), _ptr(logp), _ptr(lse),
                             _ptr(out3), _ptr(coef), _ptr(counts), _ptr(ws), ws_bytes,
                             _stream(stream)))


def grpo_head_bwd(p, H, W, y, mask, lse, coef, grad_output, dH, dW, ws, ws_bytes=None,
                  stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib.grpo_head_bwd(ctypes.byref(p), _ptr(H), _ptr(W), _ptr(y), _ptr(mask), _ptr(lse),
                             _ptr(coef), _ptr(grad_output), _ptr(dH), _ptr(dW), _ptr(ws),
                             ws_bytes, _stream(stream)))


def gspo_segment_reduce(p, logp, old_logp, ref_logp, mask, y, sid, adv, out3, coef,
                        seg_mean_logp, counts, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib.gspo_segment_reduce(ctypes.byref(p), _ptr(logp), _ptr(old_logp), _ptr(ref_logp),
                                   _ptr(mask), _ptr(y), _ptr(sid), _ptr(adv), _ptr(out3),
                                   _ptr(coef), _ptr(seg_mean_logp), _ptr(counts), _ptr(ws),
                                   ws_bytes, _stream(stream)))


def grpo_head_logp(p, H, W, y, mask, logp, lse, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib.grpo_head_logp(ctypes.byref(p), _ptr(H), _ptr(W), _ptr(y), _ptr(mask), _ptr(logp),
                              _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def grpo_head_logp_noalloc(p, H, W, y, mask, logp, lse, stream=None):
    _check(lib.grpo_head_logp_noalloc(ctypes.byref(p), _ptr(H), _ptr(W), _ptr(y), _ptr(mask),
                                      _ptr(logp), _ptr(lse), _stream(stream)))


def grpo_group_advantage(rewards, group_size, eps, adv, scale_by_std=True, n_seqs=None,
                         stream=None):
    n = rewards.numel() if n_seqs is None else n_seqs
    _check(lib.grpo_group_advantage(_ptr(rewards), n, group_size, eps, int(scale_by_std),
                                    _ptr(adv), _stream(stream)))


def shard_partials_bytes(p, v_begin, v_end) -> int:
    return lib.grpo_head_shard_partials_bytes(ctypes.byref(p), v_begin, v_end)


def grpo_head_shard_partials(p, v_begin, v_end, H, W_shard, y, mask, partials, zy,
                             stream=None):
    _check(lib.grpo_head_shard_partials(ctypes.byref(p), v_begin, v_end, _ptr(H), _ptr(W_shard),
                                        _ptr(y), _ptr(mask), _ptr(partials), _ptr(zy),
                                        _stream(stream)))


def grpo_head_merge_partials(p, partials, zy, y, mask, logp, lse, stream=None):
    _check(lib.grpo_head_merge_partials(ctypes.byref(p), _ptr(partials), _ptr(zy), _ptr(y),
                                        _ptr(mask), _ptr(logp), _ptr(lse), _stream(stream)))


class GrpoHead:
    """Owns the outputs and the workspace for one problem shape; fwd() then bwd().

    Tensors passed in must already be on the GPU, contiguous, with the dtypes the
    C ABI documents (bf16 or fp32 H/W, int64 y, uint8 mask, int32 sid, fp32 rest).
    """

    def __init__(self, params: Params, device="cuda", need_backward=True):
        self.p = params
        dev = torch.device(device)
        N, S = params.n_tokens, params.n_seqs
        nbytes = workspace_size(params) if need_backward else fwd_workspace_size(params)
        if nbytes == 0:
            raise GrpoHeadError(1, lib.grpo_head_last_error().decode())
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.logp = torch.empty(N, **f32)
        self.lse = torch.empty(N, **f32)
        self.coef = torch.empty(N, **f32)
        self.out3 = torch.empty(3, **f32)
        self.counts = torch.empty(max(S, 1), dtype=torch.int32, device=dev)

    def fwd(self, H, W, y, mask, sid, adv, old_logp, ref_logp, stream=None):
        grpo_head_fwd(self.p, H, W, y, mask, sid, adv, old_logp, ref_logp, self.logp, self.lse,
                      self.out3, self.coef, self.counts, self.ws, stream=stream)
        return self.out3

    def bwd(self, H, W, y, mask, grad_output=None, dH=None, dW=None, stream=None):
        gdt = torch.bfloat16 if self.p.grad_dtype == GRAD_BF16 else torch.float32
        if dH is None:
            dH = torch.empty(self.p.n_tokens, self.p.d_model, dtype=gdt, device=W.device)
        if dW is None:
            dW = torch.empty(self.p.v_rows, self.p.d_model, dtype=gdt, device=W.device)
        grpo_head_bwd(self.p, H, W, y, mask, self.lse, self.coef, grad_output, dH, dW, self.ws,
                      stream=stream)
        return dH, dW
