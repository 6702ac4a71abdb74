"""The oracle reproduces its committed snapshot bit for bit (see
tests/golden/make_oracle_snapshot.py for why the snapshot exists)."""
import json
import os

import numpy as np

import oracle

SNAP = os.path.join(os.path.dirname(__file__), "golden", "oracle_step_snapshot.json")


def _f(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


def test_oracle_matches_snapshot():
    rec = json.load(open(SNAP))
    n, G = rec["n"], rec["group_size"]
    w = _f(rec["w0_bits"]).copy()
    m = oracle.QuantizedState.zeros(n, G)
    v = oracle.QuantizedState.zeros(n, G)
    for t, (g, st) in enumerate(zip(rec["grads_bf16"], rec["steps"]), start=1):
        oracle.adamw_fp8_step(w, np.array(g, np.uint16), m, v, G, **rec["hparams"], step=t)
        assert np.array_equal(w.view(np.uint32), np.array(st["w_bits"], np.uint32))
        assert np.array_equal(m.codes, np.array(st["m_codes"], np.uint8))
        assert np.array_equal(v.codes, np.array(st["v_codes"], np.uint8))
        for arr, key in ((m.scale, "m_scale_bits"), (m.k, "m_k_bits"),
                         (v.scale, "v_scale_bits"), (v.k, "v_k_bits")):
            assert np.array_equal(arr.view(np.uint32), np.array(st[key], np.uint32))
