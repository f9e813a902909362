"""Pins of the oracle's bias rule: hand-worked example, a per-expert loop,
and the closed form of the step (sign of T*K - N_r*c_i times gamma, one fp32 add)."""
import json
import os

import numpy as np

from oracle import moe


def test_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "bias_worked_example.json")) as f:
        fx = json.load(f)
    b = np.array(fx["bias"], dtype=np.float32)
    nb = moe.bias_update(b, np.array(fx["load"]), fx["T"], fx["K"])
    direction = np.sign(nb.astype(np.float64) - b.astype(np.float64)).astype(int)
    assert direction.tolist() == fx["direction"]
    np.testing.assert_allclose(nb, fx["bias_after"], rtol=0, atol=2.5e-7)


def test_matches_per_expert_loop_and_fp32_add():
    rng = np.random.default_rng(4)
    for Nr, T, K in ((16, 64, 4), (256, 8192, 8), (64, 4096, 6), (5, 7, 3)):
        load = rng.multinomial(T * K, np.ones(Nr) / Nr)
        load[rng.integers(0, Nr)] = T * K // Nr if (T * K) % Nr == 0 else load[0]
        b = rng.uniform(-0.01, 0.01, Nr).astype(np.float32)
        nb = moe.bias_update(b, load, T, K)
        g = np.float32(0.001)
        for i in range(Nr):
            if Nr * int(load[i]) > T * K:
                want = np.float32(b[i] - g)
            elif Nr * int(load[i]) < T * K:
                want = np.float32(b[i] + g)
            else:
                want = b[i]
            assert nb[i] == want
            assert nb[i].view(np.uint32) == np.float32(want).view(np.uint32)


def test_steps_stay_within_n_gamma():
    rng = np.random.default_rng(6)
    b = np.zeros(32, np.float32)
    b0 = b.copy()
    for n in range(1, 21):
        load = rng.multinomial(64 * 4, rng.dirichlet(np.ones(32)))
        b = moe.bias_update(b, load, 64, 4)
        assert np.all(np.abs(b.astype(np.float64) - b0) <= n * 0.001 * (1 + 1e-5))
