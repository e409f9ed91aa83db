"""The oracle's head pool (oracle/head_pool.py) gives the same results as one direct call
over all heads: heads are independent sequences, so splitting them into groups run in other
processes, and summing the batch-shared dU1 / dU2 over the groups, must reproduce the
direct call (to the rounding of that sum's order)."""
import numpy as np

import oracle
from chunk_gated_delta_amd.synth import random_inputs
from oracle.head_pool import HeadPool, cpu_model, host_workers


def test_head_pool_matches_direct_calls():
    B, H, T, D = 2, 3, 70, 16
    inp = random_inputs(B, H, T, D, D, dtype="f32", seed=5, erase="content", dists="softplus_decay",
                        with_dO=True, rank=4)
    tok = random_inputs(B, H, T, D, D, dtype="f32", seed=6, erase="sigmoid", dists="softplus_decay",
                        with_dO=True)
    c = {"b_x": inp["b_x"], "U1": inp["U1"] * 8.0, "U2": inp["U2"] * 8.0}
    kw = dict(q=inp["q"], k=inp["k"], v=inp["v"], log_g=inp["log_g"], w=inp["w"], L=32, content=c)
    kt = dict(q=tok["q"], k=tok["k"], v=tok["v"], log_g=tok["log_g"], w=tok["w"], b=tok["b"])
    with HeadPool(2) as pool:
        pf = pool.run("forward", B, H, groups=4, **kw)
        pb = pool.run("backward_content", B, H, groups=5, dO=inp["dO"], **kw)
        tb = pool.run("backward", B, H, groups=6, dO=tok["dO"], **kt)
    df = oracle.forward(**kw)
    db = oracle.backward_content(dO=inp["dO"], **kw)
    dt = oracle.backward(dO=tok["dO"], **kt)
    for a, b in zip(pf, df):
        np.testing.assert_array_equal(a, b)
    for key, val in db.items():
        if key in ("dU1", "dU2"):
            np.testing.assert_allclose(pb[key], val, rtol=1e-12, atol=1e-14)
        else:
            np.testing.assert_array_equal(pb[key], val)
    for key, val in dt.items():
        np.testing.assert_array_equal(tb[key], val)
    assert 1 <= host_workers() <= 16 and isinstance(cpu_model(), str) and cpu_model()
