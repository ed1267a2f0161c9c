"""Write pr1_final_pool.sha256: the SHA-256 of the final pool of the PR1
stream (seed 1, 1,000 descriptors over 16 fp32 vectors of 4096 values) as
the oracle computes it.  Calls only oracle/ (and workloads/ for the seeded
inputs).  Run from the repository root: python tests/golden/make_pr1_digest.py"""
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as W  # noqa: E402


def digest(arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(a.tobytes())
    return h.hexdigest()


def main():
    s = W.make_pr1()
    p = oracle.Pool([b.host_bytes() for b in s.buffers])
    p.run(s.recs)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "pr1_final_pool.sha256")
    with open(out, "w") as f:
        f.write(digest(p.arrays) + "  pr1 seed 1, 1000 descriptors, final pool (16 x 4096 fp32), oracle\n")
    print(open(out).read().strip())


if __name__ == "__main__":
    main()
