"""Pins for oracle.linear (Y = scale * x @ W^T + bias), independent of its code.

The linear layer is the batch-invariant operator the Tencent deterministic-
inference article lists in its closing section (the vLLM ``linear`` with a
weight of shape [N, K] and a bias of N values).  Pinned here by:
- the closed form x = 0: Y equals the bias exactly;
- the closed form x = I (M = K): Y = W^T + bias;
- brute force: a pure-Python triple loop on tiny integer inputs, which would
  catch a transposed weight, a dropped bias or a bias on the wrong axis;
- numpy int64 on integer inputs at a moderate size.
"""
import numpy as np
import torch

import oracle
import workloads as wl


def _bits(t):
    return wl.bits(t)


def test_zero_input_gives_the_bias():
    g = wl.gen(71)
    W = wl.uniform((24, 40), "f16", g)
    x = torch.zeros((5, 40), dtype=torch.float16)
    b = np.linspace(-3.0, 3.0, 24)
    Y, Ya = oracle.linear(_bits(x), _bits(W), "f16", bias=b)
    assert np.array_equal(Y, np.broadcast_to(b, Y.shape))
    assert np.array_equal(Ya, np.broadcast_to(np.abs(b), Y.shape))


def test_identity_input_gives_the_transposed_weight_plus_bias():
    g = wl.gen(72)
    W = wl.integers((16, 32), "bf16", g)  # N = 16, K = 32
    x = torch.eye(32, dtype=torch.bfloat16)
    b = np.arange(16, dtype=np.float64) - 7.5
    Y, _ = oracle.linear(_bits(x), _bits(W), "bf16", bias=b)
    assert np.array_equal(Y, W.to(torch.float64).numpy().T + b[None, :])


def test_brute_force_triple_loop():
    g = wl.gen(73)
    M, N, K = 3, 5, 7
    x = wl.integers((M, K), "f16", g)
    W = wl.integers((N, K), "f16", g)
    b = [float(v) for v in range(-2, 3)]
    Y, _ = oracle.linear(_bits(x), _bits(W), "f16", bias=b, scale=2.0)
    xv, wv = x.tolist(), W.tolist()
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                s += xv[i][k] * wv[j][k]
            assert Y[i, j] == 2.0 * s + b[j], (i, j)


def test_integer_inputs_match_numpy_int64():
    g = wl.gen(74)
    M, N, K = 33, 72, 200
    x = wl.integers((M, K), "e4m3", g)
    W = wl.integers((N, K), "e4m3", g)
    b = torch.randint(-50, 51, (N,), generator=g).numpy().astype(np.int64)
    Y, _ = oracle.linear(_bits(x), _bits(W), "e4m3", bias=b.astype(np.float64))
    ref = x.to(torch.int64).numpy() @ W.to(torch.int64).numpy().T + b[None, :]
    assert np.array_equal(Y, ref.astype(np.float64))
