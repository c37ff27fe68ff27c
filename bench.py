"""Throughput of the fused LM-head GRPO loss (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--cpu-tokens T | --no-cpu-baseline]
    python bench.py --copy-calibration      # plain 1 GiB copies, for HBM counters

One step is one pass of the whole hot path over one batch: selected-token
log-prob over vocabulary tiles, fixed-order merge, GRPO (or GSPO) objective,
recomputed dlogits, dH and dW.  Inputs are synthetic and resident in HBM before
timing starts.  The old / reference log-probs are the fp64 CPU reference's
policy log-probs stored with the tests (tests/golden) plus the workload's seeded
noise, so no input is derived from the GPU's own results.  Prints one JSON line.
"""
import argparse
import hashlib
import glob
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
COPY_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_8b_head_grpo_n8192")
    ap.add_argument("--cpu-tokens", type=int, default=3072)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--clock-seconds", type=float, default=4.0,
                    help="seconds of extra steps during which the shader clock is sampled")
    ap.add_argument("--steps-only", action="store_true",
                    help="time the steps only (no log-prob entry, shard or variant timings): "
                         "for profiler runs whose per-kernel records should hold step "
                         "launches alone")
    return ap.parse_args()


def source_digest() -> str:
    """sha256 over the HIP sources and the C header: identifies the kernels that
    a stored counter measurement belongs to."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "lm_head_selected_amd", "csrc", "*")) +
                   glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_counters(workload: str):
    """The committed per-kernel counter record of this workload
    (profiles/counters_<workload>.json: copy-calibrated FETCH_SIZE / WRITE_SIZE,
    executed bf16 MFMA ops, MFMA busy cycles, clock), or None when there is none or
    the kernels changed since it was taken (its source digest differs)."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != source_digest():
        return None
    return rec


def stored_traffic(rec, kernel_stage: str):
    """HBM bytes (fetched + written) per launch of a stage's kernel, or None."""
    k = (rec or {}).get("kernels", {}).get(kernel_stage)
    if k is None:
        return None
    return int(k["fetch_bytes"] + k["write_bytes"])


def sample_clock(step, seconds: float, torch):
    """Measured shader clock while the step runs back to back: the SMU's current
    gfx clock of each XCD (amdsmi gpu metrics, refreshed about once a second),
    sampled every 50 ms over `seconds` of steps after one second of ramp-up.
    Returns a dict, or the reason it could not be read."""
    import threading
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
        amdsmi.amdsmi_get_gpu_metrics_info(h)
    except Exception as e:          # noqa: BLE001 - any failure means no telemetry
        return {"mhz": None, "source": f"amdsmi unavailable: {type(e).__name__}: {e}"}
    samples, stop = [], threading.Event()

    def sampler():
        t_start = time.perf_counter()
        while not stop.is_set():
            if time.perf_counter() - t_start >= 1.0:
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                xcd = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int)]
                if xcd:
                    samples.append(xcd)
            time.sleep(0.05)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds + 1.0:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:               # noqa: BLE001
        pass
    if not samples:
        return {"mhz": None, "source": "amdsmi gave no gfx clock readings"}
    arr = np.asarray(samples, dtype=np.float64)
    return {"mhz": round(float(arr.mean()), 1), "per_xcd_mhz": [round(float(v), 1) for v in
                                                                 arr.mean(axis=0)],
            "min_mhz": float(arr.min()), "max_mhz": float(arr.max()),
            "samples": int(len(arr)), "steps": n,
            "source": "amdsmi current_gfxclks (SMU telemetry) sampled every 50 ms while "
                      f"the same step ran back to back for {seconds:.0f} s after 1 s of ramp-up"}


def policy_logp(workload: str):
    """The fp64 CPU reference's selected-token log-probs for this workload, as
    stored by tests/golden/make_fullsize.py."""
    path = os.path.join(ROOT, "tests", "golden", f"fullsize_{workload}.npz")
    if not os.path.exists(path):
        raise SystemExit(f"no stored policy log-probs for workload {workload!r} ({path}); "
                         "the benchmark runs the full-size workloads only")
    with np.load(path) as z:
        return np.asarray(z["logp"], dtype=np.float64)


def device_inputs(inp, dev, torch):
    def t(a, dt):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    if inp["dtype"] == "bf16":
        H = torch.from_numpy(inp["H"].view(np.int16)).to(dev).view(torch.bfloat16)
        W = torch.from_numpy(inp["W"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        H, W = t(inp["H"], torch.float32), t(inp["W"], torch.float32)
    return dict(H=H, W=W, y=t(inp["y"], torch.int64), mask=t(inp["mask"], torch.uint8),
                sid=t(inp["sid"], torch.int32), adv=t(inp["adv"], torch.float32),
                old=t(inp["old_logp"], torch.float32), ref=t(inp["ref_logp"], torch.float32))


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch already loaded (same
    soname), for events the library records on its own launch stream."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.made = []

    def create(self):
        e = self.ct.c_void_p()
        rc = self.hip.hipEventCreate(self.ct.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        self.made.append(e.value)
        return e.value

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ct.c_void_p(a),
                                          self.ct.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def destroy(self):
        for e in self.made:
            self.hip.hipEventDestroy(self.ct.c_void_p(e))
        self.made = []


def cpu_baseline(inp, n_tok):
    """The fp64 oracle, as it stands, on the first n_tok tokens of the workload
    (treated as their own batch): forward, objective, backward."""
    import oracle
    from threadpoolctl import threadpool_info
    s = min(n_tok, inp["n_tokens"])
    y, mask, sid = inp["y"][:s], None if inp["mask"] is None else inp["mask"][:s], inp["sid"][:s]
    old = inp["old_logp"][:s]
    ref = None if inp["ref_logp"] is None else inp["ref_logp"][:s]
    t0 = time.perf_counter()
    act = oracle.active_tokens(y, mask, inp["ignore_index"])
    lp, lse = oracle.forward(inp["H"][:s], inp["W"], y, act, inp["v_real"], inp["inv_tau"],
                             inp["dtype"], block=256)
    n_s = int(sid.max()) + 1
    if inp["level"] == "sequence_gspo":
        obj = oracle.gspo_objective(lp, old, ref, inp["adv"][:n_s], sid, act, n_s,
                                    inp["eps_low"], inp["eps_high"], inp["beta"])
    else:
        obj = oracle.grpo_objective(lp, old, ref, inp["adv"][:n_s], sid, act, n_s,
                                    inp["eps_low"], inp["eps_high"], inp["beta"],
                                    inp["reduction"])
    oracle.backward(inp["H"][:s], inp["W"], y, act, lse, obj["coef"], inp["v_real"],
                    inp["inv_tau"], 1.0, inp["dtype"], block=256)
    dt = time.perf_counter() - t0
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(s / dt, 2), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": model, "host_cpus": os.cpu_count(),
            "blas": ", ".join(f"{p.get('internal_api')} {p.get('version')}" for p in blas) or None,
            "sample": f"first {s} of {inp['n_tokens']} tokens of the same workload as one batch "
                      f"(full D and V): fp64 forward + objective + backward, {dt:.1f} s"}


def copy_calibration():
    """Three launches of one elementwise kernel that reads COPY_BYTES and writes
    COPY_BYTES (b = -a over fp32), for scaling the HBM byte counters."""
    import torch
    dev = torch.device("cuda:0")
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": COPY_BYTES,
                      "copy_calibration_bytes_written": COPY_BYTES, "launches": 3}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the library "
              "runs on a single GPU (the multi-GPU sharding plan is design-only)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    from lm_head_selected_amd import binding as gb
    from synth import attach_logprobs, config, make_inputs

    cfg = config(args.workload)
    dev = torch.device("cuda:0")
    inp = attach_logprobs(make_inputs(cfg), policy_logp(cfg.name))
    d = device_inputs(inp, dev, torch)
    N, D, V = cfg.n_tokens, cfg.d_model, cfg.v_real
    p = gb.make_params(n_tokens=N, d_model=D, v_real=V, v_rows=cfg.v_rows, n_seqs=inp["n_seqs"],
                       dtype=cfg.dtype, reduction=cfg.reduction, level=cfg.level,
                       inv_tau=cfg.inv_tau, eps_low=cfg.eps_low, eps_high=cfg.eps_high,
                       beta=cfg.beta)
    head = gb.GrpoHead(p, dev)
    dH = torch.empty(N, D, dtype=torch.float32, device=dev)
    dW = torch.empty(cfg.v_rows, D, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        head.fwd(d["H"], d["W"], d["y"], d["mask"], d["sid"], d["adv"], d["old"], d["ref"],
                 stream=stream)
        head.bwd(d["H"], d["W"], d["y"], d["mask"], dH=dH, dW=dW, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the backward runs on the tokens whose gradient scale is non-zero (grad_output
    # = 1): active tokens with coef != 0; the others' dlogits rows are all zero
    coef_h = head.coef.cpu().numpy()
    active = (inp["mask"] != 0) if inp["mask"] is not None else (inp["y"] != inp["ignore_index"])
    n_live = int(np.count_nonzero(active & (coef_h != 0.0)))

    K = args.steps
    hev = HipEvents()
    evs = [[hev.create() for _ in range(gb.N_STAGE_EVENTS)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for k in range(K):
        gb.set_stage_events(evs[k])
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gb.set_stage_events(None)
    ms_step = start.elapsed_time(end) / K
    value = N / (ms_step / 1e3)

    extra = {} if args.steps_only else extra_timings(args, gb, p, d, head, inp, cfg, dH, dW,
                                                     stream, n_live, torch)
    if not args.steps_only:
        extra["clock"] = sample_clock(step, args.clock_seconds, torch)
    stages = {}
    for name, (a, b) in gb.STAGES.items():
        stages[name] = float(np.mean([hev.elapsed_ms(evs[k][a], evs[k][b]) for k in range(K)]))
    per_step = [hev.elapsed_ms(evs[k][0], evs[k][gb.N_STAGE_EVENTS - 1]) for k in range(K)]
    hev.destroy()
    report(args, cfg, inp, N, D, V, n_live, K, ms_step, value, wall, stages, per_step, extra)


def extra_timings(args, gb, p, d, head, inp, cfg, dH, dW, stream, n_live, torch):
    """The entry points and variants timed after the steps, on the same inputs."""
    N, D, V = cfg.n_tokens, cfg.d_model, cfg.v_real
    dev = d["H"].device
    K = args.steps
    # the forward-only selected log-prob entry (how a trainer gets the old and the
    # reference policy's log-probs) on the same inputs, timed after the steps
    lp_ws = torch.empty(gb.logp_workspace_size(p), dtype=torch.uint8, device=dev)
    lp_out = torch.empty(N, dtype=torch.float32, device=dev)
    lse_out = torch.empty(N, dtype=torch.float32, device=dev)

    def logp_call():
        gb.grpo_head_logp(p, d["H"], d["W"], d["y"], d["mask"], lp_out, lse_out, lp_ws,
                          stream=stream)

    logp_call()
    K2 = max(3, K // 2)
    l0, l1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    l0.record(stream)
    for _ in range(K2):
        logp_call()
    l1.record(stream)
    torch.cuda.synchronize()
    ms_logp = l0.elapsed_time(l1) / K2

    # one GPU's share of a 2-way vocabulary-parallel forward: the tile stage on
    # the first half of the vocabulary tiles (on the global tile grid), timed alone
    n_vt = -(-V // 256)
    v_half = (n_vt // 2) * 256
    sh_part = torch.empty(gb.shard_partials_bytes(p, 0, v_half), dtype=torch.uint8, device=dev)
    sh_zy = torch.empty(N, dtype=torch.float32, device=dev)
    w_half = d["W"][:v_half]

    def shard_call():
        gb.grpo_head_shard_partials(p, 0, v_half, d["H"], w_half, d["y"], d["mask"], sh_part,
                                    sh_zy, stream=stream)

    shard_call()
    torch.cuda.synchronize()
    l0.record(stream)
    for _ in range(K2):
        shard_call()
    l1.record(stream)
    torch.cuda.synchronize()
    ms_shard = l0.elapsed_time(l1) / K2

    # gradient-output variants, whole steps: bf16 dH/dW, and dW accumulated into
    pkw = dict(n_tokens=N, d_model=D, v_real=V, v_rows=cfg.v_rows, n_seqs=inp["n_seqs"],
               dtype=cfg.dtype, reduction=cfg.reduction, level=cfg.level, inv_tau=cfg.inv_tau,
               eps_low=cfg.eps_low, eps_high=cfg.eps_high, beta=cfg.beta)
    p_b16 = gb.make_params(**pkw, grad_dtype="bf16")
    p_acc = gb.make_params(**pkw, accumulate_dw=True)
    dH16 = torch.empty(N, D, dtype=torch.bfloat16, device=dev)
    dW16 = torch.empty(cfg.v_rows, D, dtype=torch.bfloat16, device=dev)

    def variant_ms(pv, dh, dw):
        def one():
            head.fwd(d["H"], d["W"], d["y"], d["mask"], d["sid"], d["adv"], d["old"], d["ref"],
                     stream=stream)
            gb.grpo_head_bwd(pv, d["H"], d["W"], d["y"], d["mask"], head.lse, head.coef, None,
                             dh, dw, head.ws, stream=stream)
        one()
        torch.cuda.synchronize()
        l0.record(stream)
        for _ in range(K2):
            one()
        l1.record(stream)
        torch.cuda.synchronize()
        return l0.elapsed_time(l1) / K2

    ms_b16 = variant_ms(p_b16, dH16, dW16)
    ms_acc = variant_ms(p_acc, dH, dW)

    # the same step with every token live, so the backward skips no row: the mask set
    # to all ones and the masked tokens' placeholder targets replaced by 0
    if d["mask"] is not None:
        y_all = torch.where(d["mask"] != 0, d["y"], torch.zeros_like(d["y"]))
        m_all = torch.ones_like(d["mask"])

        def all_live():
            head.fwd(d["H"], d["W"], y_all, m_all, d["sid"], d["adv"], d["old"], d["ref"],
                     stream=stream)
            head.bwd(d["H"], d["W"], y_all, m_all, dH=dH, dW=dW, stream=stream)
        all_live()
        torch.cuda.synchronize()
        l0.record(stream)
        for _ in range(K2):
            all_live()
        l1.record(stream)
        torch.cuda.synchronize()
        ms_all = l0.elapsed_time(l1) / K2
    else:
        ms_all = None
    lib = library_gemms(d, cfg, n_live, K2, torch) if cfg.dtype == "bf16" else None
    return {
        "library_gemm": lib,
        "logp_entry": {"ms": round(ms_logp, 3), "calls": K2,
                       "tokens_per_s": round(N / (ms_logp / 1e3), 1),
                       "tflops_2nvd": round(2.0 * N * V * D / (ms_logp / 1e3) / 1e12, 1)},
        "variant_steps_ms": {"bf16_grads": round(ms_b16, 3), "accumulate_dw": round(ms_acc, 3),
                             "all_rows_live": None if ms_all is None else round(ms_all, 3),
                             "steps": K2},
        "tp2_shard_tiles": {"v_rows": v_half, "ms": round(ms_shard, 3),
                            "tflops": round(2.0 * N * v_half * D / (ms_shard / 1e3) / 1e12, 1)},
    }


def library_gemms(d, cfg, n_live, reps, torch):
    """Context, not part of the step: the vendor BLAS (hipBLASLt through
    torch.matmul) on plain bf16 GEMMs of the step's three contraction shapes, with
    bf16 outputs and none of the softmax, loss or dlogits work: the logits H W^T
    (which it writes out, 2 N V_rows bytes), dH = G W and dW = G^T H over the live
    rows (G random, the dlogits shape).  Timed on torch's current stream."""
    N, D, Vr = cfg.n_tokens, cfg.d_model, cfg.v_rows
    H, W = d["H"], d["W"]
    G = torch.randn(n_live, Vr, device=H.device, dtype=torch.bfloat16) * 1e-3
    Hl = H[:n_live].contiguous()
    shapes = {"logits_H_Wt": (H, W.t(), 2.0 * N * Vr * D),
              "dH_G_W": (G, W, 2.0 * n_live * Vr * D),
              "dW_Gt_H": (G.t(), Hl, 2.0 * n_live * Vr * D)}
    out = {"note": "hipBLASLt via torch.matmul, bf16 in and out, plain GEMMs of the same "
                   "shapes (no softmax, loss or dlogits work); context only",
           "reps": reps}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total = 0.0
    for name, (a, b, flops) in shapes.items():
        c = a @ b
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        total += ms
        out[name] = {"ms": round(ms, 3), "tflops": round(flops / (ms / 1e3) / 1e12, 1)}
        del c
    out["sum_ms"] = round(total, 3)
    del G, Hl
    torch.cuda.empty_cache()
    return out


def epilogue_hbm(cfg, inp, N, D, V, n_live, stages):
    """HBM rate of the stages around the matrix-core launches: algorithmic bytes
    (each operand read once, each result written once) over the stage's event time.

      fwd_tail      target logits (an H row and a W row per active token, the target
                    id and mask) and the ordered merge (every tile partial, the target
                    logit, writing logp and lse)
      fwd_objective logp, old and reference log-probs, mask and sequence id read,
                    the coefficient written (per-sequence sums are a few KB)
      bwd_prep      row compaction (mask, coefficient, LSE read; row position
                    written per token; row index, (g, lse) pair and target id per
                    live row), the live H rows read and written twice (as rows and
                    transposed), the dead tokens' dH rows zeroed
    (The backward's target elements come out of the dlogits tile epilogue.)
    """
    esz = 2 if cfg.dtype == "bf16" else 4
    n_vt = -(-V // 256)
    active = int(np.count_nonzero(inp["mask"])) if inp["mask"] is not None else N
    has_ref = inp["ref_logp"] is not None
    ncp = -(-n_live // 256) * 256
    stage_bytes = {
        "fwd_tail": active * (2 * D * esz + 8 + 1 + 4) + N * (n_vt * 8 + 8 + 1 + 4 + 8),
        "fwd_objective": N * (4 + 4 + (4 if has_ref else 0) + 1 + 4 + 4),
        "bwd_prep": N * (1 + 4 + 4 + 4) + n_live * (4 + 8 + 8 + 4) + n_live * D * esz
                    + 2 * ncp * D * esz + (N - n_live) * D * 4,
    }
    out = {}
    for k, b in stage_bytes.items():
        if k in stages and stages[k] > 0:
            gbs = b / (stages[k] / 1e3) / 1e9
            out[k] = {"ms": round(stages[k], 4), "bytes": int(b), "GBps": round(gbs, 1),
                      "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    return out


def report(args, cfg, inp, N, D, V, n_live, K, ms_step, value, wall, stages, per_step, extra):
    """Print the JSON line."""
    from lm_head_selected_amd import binding as gb

    # algorithmic flops of each matrix-core launch: 2 D V (real vocabulary rows) per
    # row it processes: every token in the forward, the live rows in the backward
    # (the gradient launch runs both products, dH and dW: twice that)
    launch_flops = {"fwd_tiles": 2.0 * N * D * V, "bwd_dlogits": 2.0 * n_live * D * V,
                    "bwd_grads": 4.0 * n_live * D * V}
    counters = stored_counters(cfg.name)
    gemm = {}
    for s in gb.GEMM_STAGES:
        tf = launch_flops[s] / (stages[s] / 1e3) / 1e12
        gemm[s] = {"ms": round(stages[s], 3), "tflops": round(tf, 1),
                   "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        k = (counters or {}).get("kernels", {}).get(s)
        if k and k.get("mfma_flops"):
            # the matrix-core work the launch executed (the counter counts every MFMA,
            # padding rows and columns of partial tiles included), over the same time
            ex = k["mfma_flops"] / (stages[s] / 1e3) / 1e12
            gemm[s].update(executed_flops=k["mfma_flops"], tflops_executed=round(ex, 1),
                           frac_of_peak_executed=round(ex / PEAK_BF16_TFLOPS, 4),
                           mfma_busy=k.get("mfma_busy"), clock_ghz=k.get("clock_ghz"))
    dom = max(gb.GEMM_STAGES, key=lambda s: stages[s])
    achieved = launch_flops[dom] / (stages[dom] / 1e3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": stored_traffic(counters, dom),
                "kernel": gb.GEMM_STAGES[dom], "stage": dom,
                "flops_per_launch": launch_flops[dom], "launch_ms": round(stages[dom], 3)}
    if gemm[dom].get("executed_flops"):
        roofline["counters"] = {
            "executed_flops_per_launch": gemm[dom]["executed_flops"],
            "achieved_executed": gemm[dom]["tflops_executed"],
            "frac_executed": gemm[dom]["frac_of_peak_executed"],
            "mfma_busy": gemm[dom]["mfma_busy"], "clock_ghz": gemm[dom]["clock_ghz"],
            "source": f"profiles/counters_{cfg.name}.json (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, "
                      "SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE; same kernel sources)"}

    flops_8nvd = 8.0 * N * V * D
    flops_exec = (2.0 * N + 6.0 * n_live) * V * D
    epilogue = epilogue_hbm(cfg, inp, N, D, V, n_live, stages)
    out = {
        "metric": "tokens/s fwd+bwd fused GRPO head loss + % bf16 MFMA peak, D=4096 V=151936",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": N, "d_model": D, "v_real": V,
                   "v_rows": cfg.v_rows, "sequences": int(inp["n_seqs"]),
                   "reduction": cfg.reduction, "level": cfg.level, "parallelism": "none"},
        "step_ms_median": round(statistics.median(per_step), 3),
        "step_ms_min": round(min(per_step), 3),
        "backward_rows": n_live,
        "tflops_executed": round(flops_exec / (ms_step / 1e3) / 1e12, 1),
        "frac_of_peak_executed": round(flops_exec / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        # nominal accountings: they credit the backward's products for every token,
        # also the N - backward_rows tokens whose dlogits rows are zero and never run
        "nominal": {"tflops_8nvd": round(flops_8nvd / (ms_step / 1e3) / 1e12, 1),
                    "tflops_6nvd_model": round(0.75 * flops_8nvd / (ms_step / 1e3) / 1e12, 1),
                    "note": "credits skipped rows; not a measure of the executed work"},
        "gemm_launches": gemm,
        "epilogue_hbm": epilogue,
        "stages_ms": {k: round(v, 3) for k, v in stages.items()},
        "wall_s": round(wall, 3),
        "roofline": roofline,
    }
    out.update(extra)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
