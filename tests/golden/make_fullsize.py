"""Write the fp64 oracle's results for the full-size workloads.

Calls only the oracle and the seeded generators.  Usage (from the repo root):
    python tests/golden/make_fullsize.py [config index ...]      # default: 3 4
For each workload it stores
  * logp, lse: the selected log-prob and LSE of every token (a full fp64 forward);
  * sketch_dH [N, k], sketch_dW [V_r, k]: dH U and dW U for k fixed random probe
    columns U [D, k] (PROBE_SEED), from the oracle's backward on the objective's
    coefficient with grad_output = 1 -- a summary of every row of both full-size
    gradients, too large to store whole (dW alone is 5 GB in fp64);
and a fingerprint of the regenerated inputs so readers can check they rebuilt the
same workload.
"""
import hashlib
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synth import CONFIGS, attach_logprobs, make_inputs  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_SEED = 20251203
PROBES = 4


def probes(d_model: int) -> np.ndarray:
    """The [D, PROBES] Gaussian probe columns of the gradient sketches."""
    return np.random.Generator(np.random.PCG64(PROBE_SEED)).standard_normal((d_model, PROBES))


def fingerprint(inp: dict) -> str:
    h = hashlib.sha256()
    for k in ("H", "y", "sid", "adv", "noise_old"):
        h.update(np.ascontiguousarray(inp[k]).tobytes())
    h.update(np.ascontiguousarray(inp["W"][:: 97]).tobytes())
    if inp["mask"] is not None:
        h.update(inp["mask"].tobytes())
    if inp["noise_ref"] is not None:
        h.update(inp["noise_ref"].tobytes())
    return h.hexdigest()


def path_for(index: int) -> str:
    return os.path.join(HERE, f"fullsize_{CONFIGS[index].name}.npz")


def main(indices):
    for i in indices:
        cfg = CONFIGS[i]
        t0 = time.time()
        inp = make_inputs(cfg)
        act = oracle.active_tokens(inp["y"], inp["mask"], inp["ignore_index"])
        logp, lse = oracle.forward(inp["H"], inp["W"], inp["y"], act, inp["v_real"],
                                   inp["inv_tau"], inp["dtype"], block=256)
        print(f"{cfg.name}: forward {time.time() - t0:.1f} s", flush=True)
        obj = oracle.objective(attach_logprobs(inp, logp), logp)
        sH, sW = oracle.backward_sketch(inp["H"], inp["W"], inp["y"], act, lse, obj["coef"],
                                        probes(cfg.d_model), inp["v_real"], inp["inv_tau"], 1.0,
                                        inp["dtype"], block=256)
        np.savez_compressed(path_for(i), logp=logp, lse=lse,
                            sketch_dH=sH.astype(np.float32), sketch_dW=sW.astype(np.float32),
                            fingerprint=np.array(fingerprint(inp)))
        print(f"{cfg.name}: {time.time() - t0:.1f} s", flush=True)


if __name__ == "__main__":
    main([int(a) for a in sys.argv[1:]] or [3, 4])
