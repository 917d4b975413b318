"""Writes tests/golden/tiny_decode_oracle.json from the oracle alone.

The fixture freezes the oracle's result on the tiny decode workload (seeded,
4 requests, 8 q / 2 kv heads, head_dim 64, page size 16, lengths U[37,300]) so
that a later change to the oracle or to the input generator shows up as a
diff. Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import make_config  # noqa: E402


def compute():
    w = make_config(0, poison=True)
    o, lse = oracle.paged_decode(w.q.double().numpy(), w.k_cache.float().numpy(),
                                 w.v_cache.float().numpy(), w.kv_indptr.numpy(),
                                 w.kv_indices.numpy(), w.kv_len.numpy(), w.page_size,
                                 w.sm_scale)
    return w, o, lse


def main():
    w, o, lse = compute()
    out = {
        "what": "oracle paged_decode on the seeded tiny decode workload (seed 1234)",
        "kv_len": [int(x) for x in w.kv_len],
        "q_sum": float(w.q.double().sum()),
        "lse": [[float(x) for x in row] for row in lse],
        "o_first8": [[[float(x) for x in o[r, h, :8]] for h in range(o.shape[1])]
                     for r in range(o.shape[0])],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_decode_oracle.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
