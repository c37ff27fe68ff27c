"""Seeded synthetic workloads for the fused LM-head GRPO / GSPO head loss.

This module draws the inputs that both the GPU path and the CPU oracle consume:
hidden states H, LM-head weights W (with padded vocabulary rows), target ids,
the active-token mask, sequence / segment ids, per-sequence advantages and the
noise used to build the old-policy and reference log-probs.  It holds none of
the method's arithmetic: no logits, no log-softmax, no loss.

Every array is drawn from its own numpy PCG64 stream, keyed by
``(seed, array name, chunk index)`` through ``SeedSequence``; large arrays are
drawn in fixed 2**22-element chunks (threaded), so the values do not depend on
the thread count or on the order in which arrays are requested.  bf16 operands
are rounded once from the fp32 draw (round-to-nearest-even) and handed out as
raw ``uint16`` bit patterns, so every consumer sees bit-identical values.

Workload shapes follow the pages' test parametrisations:
  * Liger-Kernel PR #1160 "[GRPO] add chunked grpo streaming over vocab", review
    thread: the ``test_correctness`` case (8 sequences x 128 tokens, hidden 1024,
    vocab 4096, beta 0.1, clip 0.2/0.2, sequence-level reduction) and the
    ``test_selective_chunk_forward_matches_reference`` case (1 x 4096 tokens,
    hidden 256, vocab 5000: a ragged last vocab tile);
  * RL-Kernel PR #291 "Add deterministic DP-aware GRPO loss on the TP-aware
    logprob path", commit notes: the Qwen3-8B head target, with a real vocabulary
    smaller than the padded one and an active mask whose inactive targets need
    not hold ``ignore_index``;
  * Fast-LLM PR #554 "Fuse the GSPO segment seam into compiled blocks", What /
    Correctness: GSPO over packed, uneven segments.
The pages give no hidden sizes, value distributions or noise levels; the ones
used here (Qwen3-8B hidden 4096, vocab 151936 padded to 152064, N(0, 1) hidden
states, N(0, 0.02) weights, N(0, 0.05) / N(0, 0.1) log-prob noise) are the
plainest choices for those models and are listed with the recipe in the design
notes.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np

CHUNK = 1 << 22
BF16_NAN_BITS = np.uint16(0x7FC0)
DEFAULT_IGNORE_INDEX = -100

_KEYS = {
    "H": 1, "W": 2, "y": 3, "mask": 4, "adv": 5, "old": 6, "ref": 7, "seg": 8, "junk": 9,
}


@dataclass(frozen=True)
class Workload:
    """Shape, distributions and loss settings of one synthetic workload."""

    name: str
    n_tokens: int
    d_model: int
    v_real: int
    v_rows: int
    dtype: str                     # "bf16" or "f32": element type of H and W
    w_std: float
    h_std: float = 1.0
    seq_len: int = 0               # tokens per sequence (GRPO); 0 = packed segments
    seg_len_range: tuple = (64, 2048)
    old_noise: float = 0.05
    ref_noise: float | None = 0.1  # None: no reference log-prob (beta must be 0)
    eps_low: float = 0.2
    eps_high: float = 0.2
    beta: float = 0.04
    tau: float = 1.0
    reduction: str = "token_mean"  # or "sequence_mean"
    level: str = "token"           # or "sequence_gspo"
    mask_frac: float = 0.0         # exact fraction of inactive tokens; 0 = no mask
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def inv_tau(self) -> float:
        """1/tau rounded to fp32: the value every consumer scales logits by."""
        return float(np.float32(1.0 / self.tau))


CONFIGS = [
    Workload("tiny_grpo_fp32", n_tokens=32, d_model=64, v_real=257, v_rows=257, dtype="f32",
             w_std=0.02, seq_len=16, eps_low=0.2, eps_high=0.2, beta=0.04, tau=1.0,
             reduction="token_mean", mask_frac=0.10, seed=1000),
    Workload("grpo_b8_t128_d1024_v4096", n_tokens=1024, d_model=1024, v_real=4096, v_rows=4096,
             dtype="bf16", w_std=0.02, seq_len=128, eps_low=0.2, eps_high=0.2, beta=0.1, tau=1.0,
             reduction="sequence_mean", mask_frac=0.15, seed=1001),
    Workload("grpo_b1_t4096_d256_v5000", n_tokens=4096, d_model=256, v_real=5000, v_rows=5000,
             dtype="bf16", w_std=0.05, seq_len=4096, eps_low=0.2, eps_high=0.2, beta=0.05,
             tau=1.0, reduction="token_mean", mask_frac=0.0, seed=1002),
    Workload("qwen3_8b_head_grpo_n8192", n_tokens=8192, d_model=4096, v_real=151936,
             v_rows=152064, dtype="bf16", w_std=0.02, seq_len=1024, eps_low=0.2, eps_high=0.28,
             beta=0.04, tau=0.7, reduction="sequence_mean", mask_frac=0.10, seed=1003),
    Workload("qwen3_8b_head_gspo_n16384", n_tokens=16384, d_model=4096, v_real=151936,
             v_rows=152064, dtype="bf16", w_std=0.02, seq_len=0, seg_len_range=(64, 2048),
             old_noise=0.05, ref_noise=None, eps_low=3e-4, eps_high=4e-4, beta=0.0, tau=1.0,
             reduction="sequence_mean", level="sequence_gspo", mask_frac=0.0, seed=1004),
]


def config(index_or_name) -> Workload:
    if isinstance(index_or_name, int):
        return CONFIGS[index_or_name]
    for c in CONFIGS:
        if c.name == index_or_name:
            return c
    raise KeyError(index_or_name)


def _stream(seed: int, key: str, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _KEYS[key], chunk])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN_BITS
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(seed: int, key: str, n: int, std: float, as_bf16: bool, threads: int | None = None):
    """n iid N(0, std^2) draws (fp32), optionally rounded to bf16 bits, in fixed chunks."""
    out = np.empty(n, dtype=np.uint16 if as_bf16 else np.float32)
    nch = (n + CHUNK - 1) // CHUNK

    def work(i):
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        v = _stream(seed, key, i).standard_normal(hi - lo, dtype=np.float32)
        v *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(v) if as_bf16 else v

    if nch == 1:
        work(0)
    else:
        nt = threads or min(16, os.cpu_count() or 1)
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(work, range(nch)))
    return out


def segment_lengths(cfg: Workload) -> np.ndarray:
    """Per-sequence token counts: fixed length for GRPO batches; for packed GSPO
    segments, lengths uniform in seg_len_range drawn until they cover N, the last
    one truncated to fit."""
    n = cfg.n_tokens
    if cfg.seq_len:
        assert n % cfg.seq_len == 0
        return np.full(n // cfg.seq_len, cfg.seq_len, dtype=np.int64)
    g = _stream(cfg.seed, "seg")
    lo, hi = cfg.seg_len_range
    lens = []
    total = 0
    while total < n:
        L = int(g.integers(lo, hi + 1))
        L = min(L, n - total)
        lens.append(L)
        total += L
    return np.asarray(lens, dtype=np.int64)


def _keep_off_kinks(noise: np.ndarray, kinks, margin: float, groups=None, active=None):
    """Shift log-ratio noise so no ratio sits within `margin` of a clip boundary.

    The ratio's log is -noise (token level) or minus the active-token mean of the
    noise over a segment (segment level).  Near a boundary the clip branch can flip
    under fp32 rounding, so the recipe keeps a small gap there; the shift is at most
    2*margin.
    """
    noise = noise.astype(np.float64)
    if groups is None:
        for k in kinks:
            d = -noise - k
            near = np.abs(d) < margin
            s = np.where(d[near] >= 0, 1.0, -1.0)
            noise[near] = -(k + s * 2 * margin)
        return noise
    starts = np.concatenate([[0], np.cumsum(groups)[:-1]])
    for st, L in zip(starts, groups):
        sl = slice(st, st + L)
        act = active[sl] if active is not None else np.ones(L, bool)
        cnt = int(act.sum())
        if cnt == 0:
            continue
        for _ in range(4):
            rho = -float(noise[sl][act].sum()) / cnt
            moved = False
            for k in kinks:
                d = rho - k
                if abs(d) < margin:
                    target = k + (2 * margin if d >= 0 else -2 * margin)
                    noise[sl] -= (target - rho)
                    moved = True
            if not moved:
                break
    return noise


def make_inputs(cfg: Workload, seed: int | None = None, *, old_noise: float | None = None,
                nan_pad_rows: bool = True, threads: int | None = None,
                off_kinks: bool = True) -> dict:
    """Draw one workload.  Returns numpy arrays (bf16 operands as uint16 bits).

    off_kinks=False keeps the old-policy noise as drawn, so some ratios sit at or
    next to a clip boundary (the parity tests of the clip branch near a kink).

    Keys: H [N, D], W [V_r, D], y [N] int64, mask [N] uint8 or None, sid [N] int32,
    n_seqs, adv [S] float32, noise_old [N] float64, noise_ref [N] float64 or None,
    seg_lens [S] int64, plus the loss settings copied from the workload.
    """
    seed = cfg.seed if seed is None else seed
    n, d, v, vr = cfg.n_tokens, cfg.d_model, cfg.v_real, cfg.v_rows
    bf16 = cfg.dtype == "bf16"

    H = _normal(seed, "H", n * d, cfg.h_std, bf16, threads).reshape(n, d)
    W = _normal(seed, "W", vr * d, cfg.w_std, bf16, threads).reshape(vr, d)
    if nan_pad_rows and vr > v:
        # padded vocabulary rows must never reach a result: fill them with NaN
        W[v:] = BF16_NAN_BITS if bf16 else np.float32("nan")

    y = _stream(seed, "y").integers(0, v, size=n, dtype=np.int64)

    if cfg.mask_frac > 0:
        k = int(round(cfg.mask_frac * n))
        mask = np.ones(n, dtype=np.uint8)
        off = _stream(seed, "mask").choice(n, size=k, replace=False)
        mask[off] = 0
        # inactive targets may hold anything, including out-of-range ids
        junk = _stream(seed, "junk").choice(
            np.array([-1, v, v + 12345, 1 << 40, DEFAULT_IGNORE_INDEX], dtype=np.int64), size=k)
        y[off] = junk
    else:
        mask = None

    lens = segment_lengths(cfg)
    S = len(lens)
    sid = np.repeat(np.arange(S, dtype=np.int32), lens)
    adv = _stream(seed, "adv").standard_normal(S).astype(np.float32)

    active = mask.astype(bool) if mask is not None else np.ones(n, bool)
    sigma_old = cfg.old_noise if old_noise is None else old_noise
    noise_old = _stream(seed, "old").standard_normal(n) * sigma_old
    kinks = [math.log1p(-cfg.eps_low), math.log1p(cfg.eps_high)]
    if not off_kinks:
        pass
    elif cfg.level == "sequence_gspo":
        noise_old = _keep_off_kinks(noise_old, kinks, 2e-5, groups=lens, active=active)
    else:
        noise_old = _keep_off_kinks(noise_old, kinks, 1e-4)
    noise_ref = None
    if cfg.ref_noise is not None:
        noise_ref = _stream(seed, "ref").standard_normal(n) * cfg.ref_noise

    return dict(cfg=cfg, H=H, W=W, y=y, mask=mask, sid=sid, n_seqs=S, adv=adv,
                noise_old=noise_old, noise_ref=noise_ref, seg_lens=lens,
                n_tokens=n, d_model=d, v_real=v, v_rows=vr, dtype=cfg.dtype,
                inv_tau=cfg.inv_tau, eps_low=cfg.eps_low, eps_high=cfg.eps_high,
                beta=cfg.beta, reduction=cfg.reduction, level=cfg.level,
                ignore_index=DEFAULT_IGNORE_INDEX)


def attach_logprobs(inp: dict, policy_logp: np.ndarray) -> dict:
    """old = policy + old-noise, ref = policy + ref-noise, stored as fp32.

    `policy_logp` is the policy's selected-token log-prob for these inputs as the
    caller computed it (the tests and the bench use the CPU oracle's value).
    Inactive tokens get the noise alone; their values are never read.
    """
    out = dict(inp)
    base = np.asarray(policy_logp, dtype=np.float64)
    out["old_logp"] = (base + inp["noise_old"]).astype(np.float32)
    out["ref_logp"] = None if inp["noise_ref"] is None else (base + inp["noise_ref"]).astype(np.float32)
    return out
