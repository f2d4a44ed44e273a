"""Writes tests/golden/c4_key_rows.npz: the oracle's dK and dV on 256 seeded key rows of
every head of the long-context workload (B=1, H=8, N=65536, d=64, bf16, non-causal).

dK_j and dV_j sum over every query row i, and each term needs row i's full softmax
(its normaliser and D_i), so the oracle needs O(N^2 d) fp64 work per head: minutes of
CPU time, too long for a test run. This script does it once, here, from the seeded
inputs of ``workloads`` and the oracle alone (``oracle.backward_key_rows``); nothing in
it comes from the HIP library. The file stores, besides the values, the SHA-256 of each
input tensor's bytes, so a test can tell when the inputs it regenerates differ from the
ones the values were computed from.

Run from the repository root:  python tests/golden/make_c4_key_rows.py [--jobs 4]
"""
import argparse
import hashlib
import os
import sys
import time

KEY_ROW_SEED_OFFSET = 100   # key rows: workloads.sample_rows(seed + 100, N, 256)
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c4_key_rows.npz")


def _one_head(args):
    h, threads, root = args
    os.environ["OPENBLAS_NUM_THREADS"] = str(threads)
    sys.path.insert(0, root)
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    import workloads as W
    w = W.get("c4")
    inp = W.make_inputs(w)
    keys = W.sample_rows(w.seed + KEY_ROW_SEED_OFFSET, w.seqlen, 256)
    q, k, v, do = (oracle.to_f64(x[0, :, h, :]) for x in (inp.q, inp.k, inp.v, inp.do))
    t0 = time.time()
    with threadpool_limits(limits=threads):
        dk, dv = oracle.backward_key_rows(q, k, v, do, w.scale, w.causal, keys)
    print(f"head {h}: {time.time() - t0:.0f} s", flush=True)
    return h, dk, dv


def digest(t) -> str:
    return hashlib.sha256(t.contiguous().view(-1).view(__import__("torch").uint8).numpy().tobytes()).hexdigest()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4, help="heads computed in parallel")
    ap.add_argument("--threads", type=int, default=2, help="BLAS threads per job")
    a = ap.parse_args()
    root = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    sys.path.insert(0, root)
    import numpy as np
    import workloads as W
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    w = W.get("c4")
    inp = W.make_inputs(w)
    keys = W.sample_rows(w.seed + KEY_ROW_SEED_OFFSET, w.seqlen, 256)
    dk = np.zeros((w.heads, keys.size, w.head_dim))
    dv = np.zeros_like(dk)
    # fresh interpreters (spawn): forking after torch and the BLAS have started their
    # threads can leave the children waiting on locks that no thread will release
    with ProcessPoolExecutor(max_workers=a.jobs, mp_context=mp.get_context("spawn")) as ex:
        for h, dkh, dvh in ex.map(_one_head, [(h, a.threads, root) for h in range(w.heads)]):
            dk[h], dv[h] = dkh, dvh
    np.savez_compressed(
        OUT, keys=keys, dk=dk.astype(np.float32), dv=dv.astype(np.float32), seed=np.int64(w.seed),
        key_row_seed=np.int64(w.seed + KEY_ROW_SEED_OFFSET),
        sha256=np.array([digest(x) for x in (inp.q, inp.k, inp.v, inp.do)]))
    print("wrote", OUT)


if __name__ == "__main__":
    main()
