"""Throughput of the fused LM-head GRPO loss (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--cpu-tokens T | --no-cpu-baseline]

One step is one pass of the whole hot path over one batch: selected-token
log-prob over vocabulary tiles, fixed-order merge, GRPO objective, recomputed
dlogits, dH and dW.  Inputs are synthetic and resident in HBM before timing
starts; old/reference log-probs are this policy's own log-probs plus seeded
noise.  Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_8b_head_grpo_n8192")
    ap.add_argument("--cpu-tokens", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def device_inputs(inp, dev, torch):
    def t(a, dt):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    if inp["dtype"] == "bf16":
        H = torch.from_numpy(inp["H"].view(np.int16)).to(dev).view(torch.bfloat16)
        W = torch.from_numpy(inp["W"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        H, W = t(inp["H"], torch.float32), t(inp["W"], torch.float32)
    return dict(H=H, W=W, y=t(inp["y"], torch.int64), mask=t(inp["mask"], torch.uint8),
                sid=t(inp["sid"], torch.int32), adv=t(inp["adv"], torch.float32))


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch already loaded (same
    soname), for events the library records on its stream."""

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


def cpu_baseline(inp, old, ref, n_tok):
    """The fp64 oracle, as it stands, on the first n_tok tokens of the workload
    (treated as their own batch): forward, objective, backward."""
    import oracle
    from threadpoolctl import threadpool_info
    s = min(n_tok, inp["n_tokens"])
    y, mask, sid = inp["y"][:s], None if inp["mask"] is None else inp["mask"][:s], inp["sid"][:s]
    t0 = time.perf_counter()
    act = oracle.active_tokens(y, mask, inp["ignore_index"])
    lp, lse = oracle.forward(inp["H"][:s], inp["W"], y, act, inp["v_real"], inp["inv_tau"],
                             inp["dtype"], block=256)
    n_s = int(sid.max()) + 1
    if inp["level"] == "sequence_gspo":
        obj = oracle.gspo_objective(lp, old[:s], None if ref is None else ref[:s], inp["adv"][:n_s],
                                    sid, act, n_s, inp["eps_low"], inp["eps_high"], inp["beta"])
    else:
        obj = oracle.grpo_objective(lp, old[:s], None if ref is None else ref[:s], inp["adv"][:n_s],
                                    sid, act, n_s, inp["eps_low"], inp["eps_high"], inp["beta"],
                                    inp["reduction"])
    oracle.backward(inp["H"][:s], inp["W"], y, act, lse, obj["coef"], inp["v_real"],
                    inp["inv_tau"], 1.0, inp["dtype"], block=256)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()
                   if p.get("user_api") == "blas"] or [1])
    return {"value": s / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {s} tokens of the same workload as one batch, fp64 forward + "
                      f"objective + backward in {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: this build "
              "has no multi-GPU path (the sharding plan is described in DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from lm_head_selected_amd import binding as gb
    from synth import config, make_inputs

    cfg = config(args.workload)
    dev = torch.device("cuda:0")
    inp = make_inputs(cfg)
    d = device_inputs(inp, dev, torch)
    N, D, V = cfg.n_tokens, cfg.d_model, cfg.v_real
    p = gb.make_params(n_tokens=N, d_model=D, v_real=V, v_rows=cfg.v_rows, n_seqs=inp["n_seqs"],
                       dtype=cfg.dtype, reduction=cfg.reduction, level=cfg.level,
                       inv_tau=cfg.inv_tau, eps_low=cfg.eps_low, eps_high=cfg.eps_high,
                       beta=cfg.beta)
    head = gb.GrpoHead(p, dev)

    # old/ref = this policy's log-prob + seeded noise (the forward is the product path)
    zeros = torch.zeros(N, device=dev)
    head.fwd(d["H"], d["W"], d["y"], d["mask"], d["sid"], d["adv"], zeros,
             zeros if cfg.beta > 0 else None)
    torch.cuda.synchronize()
    base = head.logp.double()
    nz = lambda a: None if a is None else torch.from_numpy(a).to(dev)  # noqa: E731
    old = (base + nz(inp["noise_old"])).float()
    ref = None if inp["noise_ref"] is None else (base + nz(inp["noise_ref"])).float()
    dH = torch.empty(N, D, dtype=torch.float32, device=dev)
    dW = torch.empty(cfg.v_rows, D, dtype=torch.float32, device=dev)

    def step():
        head.fwd(d["H"], d["W"], d["y"], d["mask"], d["sid"], d["adv"], old, ref)
        head.bwd(d["H"], d["W"], d["y"], d["mask"], dH=dH, dW=dW)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    hev = HipEvents()
    evs = [[hev.create() for _ in range(10)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for k in range(K):
        gb.set_stage_events(evs[k])
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gb.set_stage_events(None)
    ms_step = start.elapsed_time(end) / K
    value = N * K / (ms_step * K / 1e3)

    flops_gemm = 2.0 * N * V * D
    stages = {}
    for name, (a, b) in gb.STAGES.items():
        stages[name] = float(np.mean([hev.elapsed_ms(evs[k][a], evs[k][b]) for k in range(K)]))
    hev.destroy()
    gemm_stages = ("fwd_tiles", "bwd_dlogits", "bwd_dh", "bwd_dw")
    dom = max(gemm_stages, key=lambda s: stages[s])
    achieved = flops_gemm / (stages[dom] / 1e3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None}

    out = {
        "metric": "tokens/s fwd+bwd fused GRPO head loss + % bf16 MFMA peak, D=4096 V=151936",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": N, "d_model": D, "v_real": V,
                   "v_rows": cfg.v_rows, "sequences": int(inp["n_seqs"]),
                   "reduction": cfg.reduction, "level": cfg.level, "parallelism": "none"},
        "tflops_8nvd": round(4 * flops_gemm / (ms_step / 1e3) / 1e12, 1),
        "tflops_6nvd": round(3 * flops_gemm / (ms_step / 1e3) / 1e12, 1),
        "frac_of_peak_8nvd": round(4 * flops_gemm / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "stages_ms": {k: round(v, 3) for k, v in stages.items()},
        "wall_s": round(wall, 3),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, old.cpu().numpy(),
                                           None if ref is None else ref.cpu().numpy(),
                                           args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
