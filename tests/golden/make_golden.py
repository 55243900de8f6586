"""Write tests/golden/tiny_oracle.json: the oracle's outputs on the seeded
1-layer tiny workload (4 heads, 2 kv heads, head_dim 64, 4 slots x 128).

This script calls only the oracle and the seeded input generator.  The fixture
locks the oracle against accidental change; it is not an independent pin (the
pages print no worked numeric example for this step).

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from sequence_slot_kv_amd import workloads as wl  # noqa: E402


def compute():
    w = wl.tiny()
    L, li = w.layers[0], w.inputs[0]
    hk, hv = wl.history_host(w, 0)
    rc, out = oracle.decode_batch(L, hk, hv, li.q, li.k_new, li.v_new, w.positions, w.slots)
    assert rc == 0
    k_rows = np.stack([hk[s, p] for s, p in zip(w.slots, w.positions)])
    return w, out, k_rows


def main():
    w, out, k_rows = compute()
    doc = {
        "what": "oracle outputs on the seeded tiny workload (regression lock)",
        "source": "ZINC 'Forward Cuda Gemma', decodeBatch; inputs from workloads.tiny()",
        "positions": w.positions.tolist(),
        "slots": w.slots.tolist(),
        "out": [[float(x) for x in row] for row in out],
        "k_written": [[float(x) for x in row] for row in k_rows],
    }
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(doc, f, indent=0)


if __name__ == "__main__":
    main()
