"""Write tests/golden/tiny_e4m3_oracle.json from the oracle alone.

The pages print no worked numerical example for the operator, so this file is
a regression fixture: the oracle's output on a tiny seeded workload, stored as
fp32 bit patterns.  Regenerate only with a commit message that names the
reading of the pages that changed the oracle's arithmetic.

    python tests/golden/make_golden.py
"""
import json
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synthetic  # noqa: E402

SPEC = dict(context_lens=[7, 20], q_lens=[3, 20], num_q_heads=2, num_kv_heads=1, head_dim=8,
            block_size=16, seed=20241)


def compute():
    spec = synthetic.Spec(name="golden_tiny", **SPEC)
    w = synthetic.generate(spec)
    c = oracle.HostCache(w.num_blocks, 1, 16, 8, "e4m3", w.k_scale_head, w.v_scale_head)
    c.append(w.k, w.v, w.block_tables, w.cu_kv.astype(np.int32), np.zeros(2, np.int32))
    out, lse = oracle.attention(w.q, 2, c, w.block_tables, w.cu_q_lens, w.context_lens,
                                1.0 / math.sqrt(8.0))
    return w, c, out, lse


def main():
    w, c, out, lse = compute()
    doc = {
        "what": "oracle output on a tiny seeded E4M3 workload (regression fixture)",
        "source": "written by tests/golden/make_golden.py from oracle/ only",
        "spec": SPEC,
        "k_codes_crc": int(np.uint32(np.frombuffer(c.k.tobytes(), np.uint8).astype(np.uint64).sum())),
        "out_bits": out.view(np.uint32).reshape(-1).tolist(),
        "lse_bits": lse.view(np.uint32).reshape(-1).tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_e4m3_oracle.json")
    with open(path, "w") as f:
        json.dump(doc, f)
        f.write("\n")


if __name__ == "__main__":
    main()
