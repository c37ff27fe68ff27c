"""Plain, slow fp64 CPU oracle for the fused LM-head GRPO / GSPO head loss.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code, constants or helpers with the GPU library, and the GPU library never
calls it.

Everything is computed from its plain definition in float64 with NumPy, from
exactly the operand values the GPU receives (bf16 bit patterns or fp32 values,
widened to fp64).  Row blocking over tokens is used only to bound memory: rows
are independent.  No tiling, online merging or fusion is used on the main path;
``tiled_lse`` spells out the tile-streamed merge separately so the tests can pin
that it reaches the plain definition.

Sources of each step (page title, section):
  * selected-token log-prob over vocab, computing only the target's log-prob:
    Liger-Kernel PR #1160 "[GRPO] add chunked grpo streaming over vocab", Summary.
  * real versus padded vocabulary, padded columns masked to -inf before the
    per-tile (max, sumexp) partials, the fp32 merge in fixed tile order and its
    (-inf, 0) identity: RL-Kernel PR #291 "Add deterministic DP-aware GRPO loss on
    the TP-aware logprob path", commit notes (ShardingSpec, ReductionSpec,
    DeterminismScope) and the review thread on ``_local_tile_stats``.
  * explicit active mask versus ``ignore_index``, inactive targets that need not
    hold ``ignore_index``: same page, commit notes (MaskMode).
  * the objective acts per token / per sequence; the loss triple
    (loss, policy_loss, kl); token normalisers ``global_active_tokens`` (masked
    mean), ``per_sequence_then_mean`` counting only sequences with active
    tokens, and ``fixed_constant`` (Dr. GRPO); no division by zero for an empty
    batch: same page, Overview / Key Changes and the zero-active-token review
    thread.
  * softmax recovered from the logits and the LSE for the backward: same page,
    review thread on the saved fp32 logits.
  * GSPO: per-token contributions aggregated per segment with ``index_add``, then
    the loss and an unscaled per-token backward coefficient, ``/ divisor`` and
    ``grad_output`` applied at run time: Fast-LLM PR #554 "Fuse the GSPO segment
    seam into compiled blocks", What.
The pages do not write out the clipped objective, the KL estimator or the GSPO
ratio.  This module uses the published forms: the PPO clipped surrogate
(Schulman et al. 2017, "Proximal Policy Optimization Algorithms", eq. 7) with
separate lower/upper clip bounds, the k3 KL estimator
exp(q - l) - (q - l) - 1 (J. Schulman, "Approximating KL Divergence", 2020), and
the GSPO sequence ratio exp(mean over the segment of log-ratio)
(Zheng et al. 2025, "Group Sequence Policy Optimization", eq. 7).

Parity pins for every function live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "widen", "active_tokens", "logits_rows", "lse_rows", "forward", "tile_partials",
    "tiled_lse", "sequence_counts", "grpo_objective", "gspo_objective", "objective",
    "dlogits_rows", "backward", "backward_sketch", "dH_rows", "dW_rows", "group_advantage",
]


# ---------------------------------------------------------------------------
# operands
# ---------------------------------------------------------------------------
def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """bf16 bit patterns (uint16), fp32 or fp64 values -> float64, value for value."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def active_tokens(y: np.ndarray, mask, ignore_index: int) -> np.ndarray:
    """MaskMode (RL-Kernel PR #291, commit notes): with an explicit mask the mask
    alone decides; without one, a token is active iff its target != ignore_index."""
    if mask is not None:
        return np.asarray(mask).astype(bool)
    return np.asarray(y) != ignore_index


# ---------------------------------------------------------------------------
# forward: selected-token log-prob
# ---------------------------------------------------------------------------
def logits_rows(H64: np.ndarray, W64: np.ndarray, v_real: int, inv_tau: float) -> np.ndarray:
    """z = (H . W[:V]^T) / tau for the given rows of H.  Padded rows W[V:] are not
    part of the vocabulary and are never touched (ShardingSpec: real vs padded)."""
    return (H64 @ W64[:v_real].T) * inv_tau


def lse_rows(z: np.ndarray) -> np.ndarray:
    """log sum_v exp(z_v) per row, with the row max subtracted for range."""
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def forward(H, W, y, active, v_real: int, inv_tau: float, dtype: str, rows=None,
            block: int = 64):
    """Selected-token log-prob and vocab LSE (LogprobOutputSpec: fp32 selected
    logprob and fp32 LSE; here in fp64).

    logp_t = z[t, y_t] - lse_t for active tokens and 0 otherwise; lse_t is
    computed for every row.  The target of an inactive token is never read.
    Returns (logp, lse) for `rows` (default: all tokens).
    """
    rows = np.arange(H.shape[0]) if rows is None else np.asarray(rows)
    W64 = widen(W[:v_real], dtype)
    logp = np.zeros(len(rows))
    lse = np.zeros(len(rows))
    for s in range(0, len(rows), block):
        r = rows[s:s + block]
        z = logits_rows(widen(H[r], dtype), W64, v_real, inv_tau)
        lse[s:s + len(r)] = lse_rows(z)
        for i, t in enumerate(r):
            if active[t]:
                logp[s + i] = z[i, int(y[t])] - lse[s + i]
    return logp, lse


def tile_partials(z_row: np.ndarray, v_rows: int, tile: int):
    """Per-tile (max, sumexp) over one logit row, tiles of `tile` columns covering
    the padded vocabulary [0, v_rows).  Columns >= len(z_row) (padding) count as
    -inf, and a tile with no real column yields the identity (-inf, 0) without
    evaluating exp(-inf - (-inf)) (RL-Kernel PR #291, commit notes and the
    ``_local_tile_stats`` review thread)."""
    v = len(z_row)
    parts = []
    for t0 in range(0, v_rows, tile):
        seg = z_row[t0:min(t0 + tile, v)]
        if len(seg) == 0:
            parts.append((-np.inf, 0.0))
            continue
        m = seg.max()
        parts.append((m, float(np.exp(seg - m).sum())))
    return parts


def tiled_lse(z_row: np.ndarray, v_rows: int, tile: int) -> float:
    """Fold per-tile partials in ascending tile order from the identity (-inf, 0):
    (M, S) + (m, s) = (max, S*e^(M-max) + s*e^(m-max)); lse = M + ln S
    (ReductionSpec: fp32 merge in a fixed global tile order; here fp64)."""
    M, S = -np.inf, 0.0
    for m, s in tile_partials(z_row, v_rows, tile):
        if m == -np.inf:
            continue
        if M == -np.inf:
            M, S = m, s
            continue
        top = max(M, m)
        S = S * np.exp(M - top) + s * np.exp(m - top)
        M = top
    return M + np.log(S)


# ---------------------------------------------------------------------------
# objective
# ---------------------------------------------------------------------------
def sequence_counts(sid, active, n_seqs: int) -> np.ndarray:
    """L_s = number of active tokens of sequence s."""
    L = np.zeros(n_seqs, dtype=np.int64)
    np.add.at(L, np.asarray(sid)[active], 1)
    return L


def _weights(sid, active, L, reduction: str, norm_const=None) -> np.ndarray:
    """Token weights of the loss normaliser (RL-Kernel PR #291, Key Changes,
    LossReductionSpec.token_normalizer):
      token_mean     (global_active_tokens, the masked mean): w_t = m_t / T_act
      sequence_mean  (per_sequence_then_mean):  w_t = m_t / (L_{s(t)} * S_live),
                      S_live counting only sequences with at least one active token.
      fixed_constant (Dr. GRPO): w_t = m_t / C for the caller's constant C > 0.
                      The page names this normaliser without fixing C; reading: C
                      is an input.
    An empty batch gives all-zero weights (no division by zero)."""
    w = np.zeros(len(sid))
    if reduction == "fixed_constant":
        if norm_const is None or not norm_const > 0:
            raise ValueError("fixed_constant needs norm_const > 0")
        w[active] = 1.0 / float(norm_const)
        return w
    T_act = int(active.sum())
    if T_act == 0:
        return w
    if reduction == "token_mean":
        w[active] = 1.0 / T_act
    elif reduction == "sequence_mean":
        S_live = int((L > 0).sum())
        w[active] = 1.0 / (L[np.asarray(sid)[active]] * S_live)
    else:
        raise ValueError(reduction)
    return w


def _k3(logp, ref):
    """k3 estimator of KL(policy || reference) per token: delta = ref - logp,
    kl = e^delta - delta - 1 (>= 0), and d kl / d logp = 1 - e^delta."""
    delta = ref - logp
    return np.exp(delta) - delta - 1.0, 1.0 - np.exp(delta)


def grpo_objective(logp, old, ref, adv, sid, active, n_seqs: int, eps_low: float,
                   eps_high: float, beta: float, reduction: str, norm_const=None) -> dict:
    """Token-level GRPO clipped objective with k3 KL.

    Per token (the objective is elementwise, RL-Kernel PR #291 Overview):
      r = exp(logp - old), c = clip(r, 1 - eps_low, 1 + eps_high), a = adv[sid],
      pol = -min(r*a, c*a), kl = k3(logp, ref).
    policy_loss = sum_t w_t pol_t, kl = sum_t w_t kl_t, loss = policy_loss + beta*kl
    (the (loss, policy_loss, kl) triple of GRPOLossResult).
    coef_t = d loss / d logp_t: the min takes the unclipped term (gradient -a*r)
    when r*a <= c*a, the constant clipped term (gradient 0) otherwise.
    coef_unclipped / coef_clipped are coef_t as it would be on each branch of the
    min; at a ratio on a clip boundary both branches are the derivative of one side.
    """
    sid = np.asarray(sid)
    logp = np.asarray(logp, np.float64)
    L = sequence_counts(sid, active, n_seqs)
    w = _weights(sid, active, L, reduction, norm_const)
    old = np.where(active, np.asarray(old, np.float64), logp)   # inactive: never read
    a = np.asarray(adv, np.float64)[sid]
    r = np.exp(logp - old)
    c = np.clip(r, 1.0 - eps_low, 1.0 + eps_high)
    unclipped = r * a <= c * a
    pol = -np.minimum(r * a, c * a)
    dpol = np.where(unclipped, -a * r, 0.0)
    if ref is not None:
        kl_t, dkl = _k3(logp, np.where(active, np.asarray(ref, np.float64), logp))
    else:
        kl_t, dkl = np.zeros_like(logp), np.zeros_like(logp)
    pol = np.where(active, pol, 0.0)
    kl_t = np.where(active, kl_t, 0.0)
    policy_loss = float((w * pol).sum())
    kl = float((w * kl_t).sum())
    coef = np.where(active, w * (dpol + beta * dkl), 0.0)
    coef_unclipped = np.where(active, w * (-a * r + beta * dkl), 0.0)
    coef_clipped = np.where(active, w * (beta * dkl), 0.0)
    return dict(loss=policy_loss + beta * kl, policy_loss=policy_loss, kl=kl, coef=coef,
                counts=L, unclipped=unclipped, log_ratio=logp - old,
                coef_unclipped=coef_unclipped, coef_clipped=coef_clipped)


def gspo_objective(logp, old, ref, adv, sid, active, n_seqs: int, eps_low: float,
                   eps_high: float, beta: float) -> dict:
    """Segment-level (GSPO) clipped objective.

    Per-token contributions m_t (logp_t - old_t) are aggregated per segment (the
    ``index_add`` of Fast-LLM PR #554, What), then per live segment
      rho_s = sum / L_s, sigma_s = exp(rho_s), c_s = clip(sigma_s),
      pol_s = -min(sigma_s A_s, c_s A_s),
    policy_loss = (1/S_live) sum_{live s} pol_s (the run-time divisor is S_live).
    The KL term is the token k3 with sequence-mean weights.  coef_t is the unscaled
    per-token backward coefficient d loss / d logp_t:
      m_t/(S_live L_s) * (-A_s sigma_s [sigma_s A_s <= c_s A_s]) + beta w_t (1 - e^delta_t).
    seg_mean_logp (the ``new_logprobs`` metric) is the active-token mean of logp per
    segment, 0 for a segment without active tokens.  rho is each segment's mean
    log-ratio; coef_unclipped / coef_clipped are coef_t as it would be with its
    segment on each branch of the min.
    """
    sid = np.asarray(sid)
    logp = np.asarray(logp, np.float64)
    L = sequence_counts(sid, active, n_seqs)
    S_live = int((L > 0).sum())
    old = np.where(active, np.asarray(old, np.float64), logp)   # inactive: never read
    contrib = np.where(active, logp - old, 0.0)
    seg_sum = np.zeros(n_seqs)
    np.add.at(seg_sum, sid, contrib)
    lsum = np.zeros(n_seqs)
    np.add.at(lsum, sid, np.where(active, logp, 0.0))
    live = L > 0
    Lsafe = np.where(live, L, 1)
    rho = np.where(live, seg_sum / Lsafe, 0.0)
    sigma = np.exp(rho)
    A = np.asarray(adv, np.float64)
    c = np.clip(sigma, 1.0 - eps_low, 1.0 + eps_high)
    pol_s = np.where(live, -np.minimum(sigma * A, c * A), 0.0)
    g_s = np.where(live & (sigma * A <= c * A), -A * sigma, 0.0)
    w = _weights(sid, active, L, "sequence_mean")
    if ref is not None:
        kl_t, dkl = _k3(logp, np.where(active, np.asarray(ref, np.float64), logp))
        kl_t = np.where(active, kl_t, 0.0)
    else:
        kl_t, dkl = np.zeros_like(logp), np.zeros_like(logp)
    if S_live == 0:
        zero = np.zeros(len(logp))
        return dict(loss=0.0, policy_loss=0.0, kl=0.0, coef=zero, counts=L,
                    seg_mean_logp=np.zeros(n_seqs), sigma=sigma, unclipped=g_s != 0,
                    rho=rho, coef_unclipped=zero, coef_clipped=zero)
    policy_loss = float(pol_s.sum() / S_live)
    kl = float((w * kl_t).sum())
    coef = np.where(active, g_s[sid] / (S_live * Lsafe[sid]) + beta * w * dkl, 0.0)
    coef_unclipped = np.where(active, -A[sid] * sigma[sid] / (S_live * Lsafe[sid])
                              + beta * w * dkl, 0.0)
    coef_clipped = np.where(active, beta * w * dkl, 0.0)
    return dict(loss=policy_loss + beta * kl, policy_loss=policy_loss, kl=kl, coef=coef,
                counts=L, seg_mean_logp=np.where(live, lsum / Lsafe, 0.0), sigma=sigma,
                unclipped=live & (sigma * A <= c * A), rho=rho,
                coef_unclipped=coef_unclipped, coef_clipped=coef_clipped)


def objective(inp: dict, logp) -> dict:
    """Dispatch on the workload's level (token GRPO or segment GSPO)."""
    active = active_tokens(inp["y"], inp["mask"], inp["ignore_index"])
    if inp["level"] == "sequence_gspo":
        return gspo_objective(logp, inp["old_logp"], inp["ref_logp"], inp["adv"], inp["sid"],
                              active, inp["n_seqs"], inp["eps_low"], inp["eps_high"], inp["beta"])
    return grpo_objective(logp, inp["old_logp"], inp["ref_logp"], inp["adv"], inp["sid"], active,
                          inp["n_seqs"], inp["eps_low"], inp["eps_high"], inp["beta"],
                          inp["reduction"], inp.get("norm_const"))


# ---------------------------------------------------------------------------
# advantage (the step before the path)
# ---------------------------------------------------------------------------
def group_advantage(rewards, group_size: int, eps: float, scale_by_std: bool = True):
    """Group-relative advantage of each sequence from its scalar reward.

    Sequences come in consecutive groups of ``group_size`` (the completions of one
    prompt).  Per group g with rewards r_i:
      mean_g = sum_i r_i / G,
      var_g  = sum_i (r_i - mean_g)^2 / G      (two passes: the mean is subtracted
                                                before squaring),
      A_i    = (r_i - mean_g) / (sqrt(var_g) + eps)   (0 when that divisor is 0,
               a constant group with eps = 0) or, without the std scaling (the
               Dr. GRPO choice), A_i = r_i - mean_g.
    Sources: the group-relative advantage acts per sequence (RL-Kernel PR #291,
    Overview); the two-pass variance subtracts the mean before squaring (same
    page, review thread on the TWO_PASS enum).  The pages fix neither the divisor
    of the variance nor eps; reading: the population variance of the group
    (divide by G) and a caller eps >= 0.
    """
    r = np.asarray(rewards, np.float64)
    if group_size < 1 or len(r) % group_size:
        raise ValueError("the number of sequences must be a multiple of group_size")
    out = np.zeros(len(r))
    for g0 in range(0, len(r), group_size):
        grp = r[g0:g0 + group_size]
        mean = sum(grp) / group_size
        dev = grp - mean
        if scale_by_std:
            var = sum(dev * dev) / group_size
            den = np.sqrt(var) + eps
            # a constant group with eps = 0 has nothing to scale: its advantages are 0
            out[g0:g0 + group_size] = dev / den if den > 0 else 0.0
        else:
            out[g0:g0 + group_size] = dev
    return out


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------
def dlogits_rows(z, lse, y, active, coef, inv_tau: float, grad_output: float) -> np.ndarray:
    """G_tv = d loss / d (H W^T)_tv = grad_output * coef_t * (1[v = y_t] - p_tv) / tau
    with p_tv = exp(z_tv - lse_t) (softmax from logits and LSE, RL-Kernel PR #291
    review thread on the saved logits).  Rows of inactive tokens are zero."""
    p = np.exp(z - lse[:, None])
    G = -p
    for i in range(len(y)):
        if active[i]:
            G[i, int(y[i])] += 1.0
    scale = np.where(active, grad_output * coef * inv_tau, 0.0)
    return G * scale[:, None]


def backward(H, W, y, active, lse, coef, v_real: int, inv_tau: float, grad_output: float,
             dtype: str, block: int = 64):
    """dH = G . W[:V] and dW[:V] = G^T . H, dW[V:] = 0 (padded rows get no gradient).
    Full matrices; memory O(N*D + V_r*D)."""
    N, D = H.shape
    W64 = widen(W[:v_real], dtype)
    dH = np.zeros((N, D))
    dW = np.zeros((W.shape[0], D))
    for s in range(0, N, block):
        r = np.arange(s, min(N, s + block))
        H64 = widen(H[r], dtype)
        z = logits_rows(H64, W64, v_real, inv_tau)
        G = dlogits_rows(z, lse[r], y[r], active[r], coef[r], inv_tau, grad_output)
        dH[r] = G @ W64
        dW[:v_real] += G.T @ H64
    return dH, dW


def backward_sketch(H, W, y, active, lse, coef, U, v_real: int, inv_tau: float,
                    grad_output: float, dtype: str, block: int = 256):
    """(dH . U, dW . U) for a [D, k] matrix U, without forming dH or dW.

    The same G as ``backward``; by associativity dH U = G (W[:V] U) and
    dW[:V] U = G^T (H U), and the padded rows of dW U are zero.  A few random
    columns U summarise every row of both gradients (a sketch), so a full-size
    gradient can be checked row by row, tile by tile, from [N, k] and [V_r, k]
    numbers.  Costs one logit pass."""
    N, D = H.shape
    U = np.asarray(U, np.float64)
    W64 = widen(W[:v_real], dtype)
    WU = W64 @ U
    sH = np.zeros((N, U.shape[1]))
    sW = np.zeros((W.shape[0], U.shape[1]))
    for s in range(0, N, block):
        r = np.arange(s, min(N, s + block))
        H64 = widen(H[r], dtype)
        z = logits_rows(H64, W64, v_real, inv_tau)
        G = dlogits_rows(z, lse[r], y[r], active[r], coef[r], inv_tau, grad_output)
        sH[r] = G @ WU
        sW[:v_real] += G.T @ (H64 @ U)
    return sH, sW


def dH_rows(H, W, y, active, lse, coef, rows, v_real: int, inv_tau: float,
            grad_output: float, dtype: str, vblock: int = 16384) -> np.ndarray:
    """dH for the given token rows only (same definition as ``backward``)."""
    rows = np.asarray(rows)
    H64 = widen(H[rows], dtype)
    out = np.zeros((len(rows), H.shape[1]))
    act = np.asarray(active)[rows]
    ys = np.asarray(y)[rows]
    # the row's softmax needs its full LSE, which the caller supplies
    for v0 in range(0, v_real, vblock):
        v1 = min(v_real, v0 + vblock)
        Wb = widen(W[v0:v1], dtype)
        z = (H64 @ Wb.T) * inv_tau
        p = np.exp(z - np.asarray(lse)[rows][:, None])
        G = -p
        for i in range(len(rows)):
            if act[i] and v0 <= ys[i] < v1:
                G[i, int(ys[i]) - v0] += 1.0
        scale = np.where(act, grad_output * np.asarray(coef)[rows] * inv_tau, 0.0)
        out += (G * scale[:, None]) @ Wb
    return out


def dW_rows(H, W, y, active, lse, coef, vrows, v_real: int, inv_tau: float,
            grad_output: float, dtype: str, tblock: int = 4096) -> np.ndarray:
    """dW for the given vocabulary rows only; rows >= v_real are zero."""
    vrows = np.asarray(vrows)
    out = np.zeros((len(vrows), H.shape[1]))
    real = vrows < v_real
    if not real.any():
        return out
    vr = vrows[real]
    Wv = widen(W[vr], dtype)
    acc = np.zeros((len(vr), H.shape[1]))
    N = H.shape[0]
    for t0 in range(0, N, tblock):
        t1 = min(N, t0 + tblock)
        H64 = widen(H[t0:t1], dtype)
        z = (H64 @ Wv.T) * inv_tau
        p = np.exp(z - np.asarray(lse)[t0:t1][:, None])
        G = -p
        act = np.asarray(active)[t0:t1]
        ys = np.asarray(y)[t0:t1]
        for j, v in enumerate(vr):
            hit = act & (ys == v)
            G[hit, j] += 1.0
        scale = np.where(act, grad_output * np.asarray(coef)[t0:t1] * inv_tau, 0.0)
        acc += (G * scale[:, None]).T @ H64
    out[real] = acc
    return out
