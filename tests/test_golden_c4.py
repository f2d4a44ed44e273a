"""The stored expected values for the long-context workload's key rows
(tests/golden/c4_key_rows.npz, written by tests/golden/make_c4_key_rows.py from the
oracle alone) belong to the inputs the tests regenerate: same seeds, same row choice,
same input bytes. The GPU test compares the library's dK and dV with them."""
import hashlib
import os

import numpy as np
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "c4_key_rows.npz")


def test_c4_key_rows_fixture_matches_the_seeded_inputs():
    w = W.get("c4")
    z = np.load(GOLDEN)   # plain arrays only (allow_pickle stays False)
    assert int(z["seed"]) == w.seed and int(z["key_row_seed"]) == w.seed + 100
    assert np.array_equal(z["keys"], W.sample_rows(w.seed + 100, w.seqlen, 256))
    assert z["dk"].shape == z["dv"].shape == (w.heads, 256, w.head_dim)
    assert np.isfinite(z["dk"]).all() and np.isfinite(z["dv"]).all()
    inp = W.make_inputs(w)
    digests = [hashlib.sha256(t.contiguous().view(-1).view(torch.uint8).numpy().tobytes()).hexdigest()
               for t in (inp.q, inp.k, inp.v, inp.do)]
    assert list(z["sha256"]) == digests
