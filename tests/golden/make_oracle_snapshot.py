"""Write tests/golden/oracle_step_snapshot.json: a small fused-step trajectory
computed by the CPU oracle alone, stored with its inputs.

The snapshot guards the oracle against unnoticed changes: a later change to
its arithmetic must regenerate this file, and its commit names the passage of
the sources (or the reading of it) that justifies the change.
Run: python tests/golden/make_oracle_snapshot.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from adamw_coat_fp8_amd import inputs  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_step_snapshot.json")
N, G, STEPS = 300, 16, 3


def hexf(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32).tolist()


def main():
    hp = dict(inputs.DEFAULT_HPARAMS)
    w = inputs.weights(N, 0, "cpu").numpy().copy()
    grads = [inputs.bf16_bits(inputs.gradient(N, 1e-3, t, 0, "cpu", kind="stress",
                                              group_size=G)).numpy().view(np.uint16).copy()
             for t in range(1, STEPS + 1)]
    rec = {"n": N, "group_size": G, "hparams": hp, "w0_bits": hexf(w),
           "grads_bf16": [g.tolist() for g in grads], "steps": []}
    m = oracle.QuantizedState.zeros(N, G)
    v = oracle.QuantizedState.zeros(N, G)
    for t in range(1, STEPS + 1):
        oracle.adamw_fp8_step(w, grads[t - 1], m, v, G, **hp, step=t)
        rec["steps"].append({"w_bits": hexf(w), "m_codes": m.codes.tolist(),
                             "m_scale_bits": hexf(m.scale), "m_k_bits": hexf(m.k),
                             "v_codes": v.codes.tolist(),
                             "v_scale_bits": hexf(v.scale), "v_k_bits": hexf(v.k)})
    with open(OUT, "w") as f:
        json.dump(rec, f, separators=(",", ":"))
    print(OUT)


if __name__ == "__main__":
    main()
