"""Parity at the benchmark configurations' full sizes, in the launch modes
bench.py times.

The shapes are those of the decode GEMV (2B-class, one token, fused
quantization), the prefill GEMM (2B-class, 2048 tokens) and the 100B-class
layer (decode at 1, 8 and 32 tokens, prefill at 512).  The launch mode of
each case is the one bench.py picks for that batch: the fused decode
kernel up to 4 tokens, the standalone quantizer then bitlinear_gemv up to
64 tokens, and the quantizer then bitlinear_gemm beyond.

At these sizes the oracle computes sampled outputs one by one.  It
quantizes the sampled tokens' activation rows and ternarizes the sampled
weight rows with the whole matrix's beta, then forms their int32 dot
products exactly.  The GPU's int32 accumulators must match bit for bit, and
its fp32 outputs exactly: both sides evaluate (float)acc * (ds * beta) with
the same IEEE operations.  Properties that hold at any size are checked on
the whole output: every value is finite, and the fp32 output equals the
dequantized int32 output of the same launch.
"""
import functools

import numpy as np
import pytest
import torch

import bitlinear_matmul_02_amd as bl
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

# (workload, tokens, K, N, bench.py's launch mode)
CASES = [
    ("decode_gemv_2b_m1", 1, 2560, 6912, "fused"),
    ("decode_gemv_2b_m1", 1, 6912, 2560, "fused"),
    ("prefill_2b_m2048", 2048, 2560, 6912, "gemm"),
    ("prefill_2b_m2048", 2048, 6912, 2560, "gemm"),
    ("decode_100b_m1", 1, 8192, 28672, "fused"),
    ("decode_100b_m1", 1, 28672, 8192, "fused"),
    ("decode_100b_m8", 8, 8192, 28672, "gemv"),
    ("decode_100b_m8", 8, 28672, 8192, "gemv"),
    ("decode_100b_m32", 32, 8192, 28672, "gemv"),
    ("decode_100b_m32", 32, 28672, 8192, "gemv"),
    ("prefill_100b_m512", 512, 8192, 28672, "gemm"),
    ("prefill_100b_m512", 512, 28672, 8192, "gemm"),
]


@functools.lru_cache(maxsize=2)
def weights(N: int, K: int):
    """Latent weights, their beta (oracle) and the packed tiles on the device."""
    w = workloads.gen_weights(N, K, seed=11000 + N + K)
    beta = oracle.absmean(w)
    packed, b_dev = bl.pack_weights(torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    assert b_dev.cpu().numpy()[0] == beta
    return w, beta, packed, b_dev


def launch(mode, x, M, K, N, packed, beta, out_dtype):
    y = torch.empty((M, N), dtype=out_dtype, device=DEV)
    if mode == "fused":
        bl.bitlinear_forward_decode(x, packed, beta, N, y)
    else:
        x_q, x_ds = bl.quant_act(x)
        if mode == "gemm":
            ws = bl.workspace(bl.gemm_workspace_bytes(M, N, K), DEV)
            bl.bitlinear_gemm(x_q, x_ds, K, packed, beta, N, y, ws)
        else:
            ws = bl.workspace(bl.gemv_workspace_bytes(M, N, K), DEV)
            bl.bitlinear_gemv(x_q, x_ds, K, packed, beta, N, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("name,M,K,N,mode", CASES, ids=["%s-%dx%d->%d" % (c[0], c[1], c[2], c[3]) for c in CASES])
def test_config_sampled_parity(name, M, K, N, mode):
    assert mode != "fused" or bl.decode_fits(M, K)
    w, beta, packed, b_dev = weights(N, K)
    xb = workloads.gen_acts_bf16(M, K, seed=12000 + M + K, outliers=name.startswith("decode_gemv"))
    x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).to(DEV)
    acc = launch(mode, x, M, K, N, packed, b_dev, torch.int32)
    y = launch(mode, x, M, K, N, packed, b_dev, torch.float32)

    rng = np.random.default_rng(M * 131 + N)
    ms = np.sort(rng.choice(M, size=min(M, 16), replace=False))
    ns = np.sort(rng.choice(N, size=96, replace=False))
    ns = np.unique(np.concatenate([ns, [0, N - 1]]))  # the first and last output rows too
    q, ds, _ = oracle.quant_act(xb[ms], bf16_bits=True)
    t = oracle.ternarize(w[ns], beta)
    acc_ref = oracle.matmul_i32(q, t)
    y_ref = oracle.dequant(acc_ref, ds, beta)
    np.testing.assert_array_equal(acc[np.ix_(ms, ns)], acc_ref)
    np.testing.assert_array_equal(y[np.ix_(ms, ns)], y_ref)

    # any size: finite, and the fp32 output is the dequantized int32 output
    assert np.all(np.isfinite(y))
    _, ds_all, _ = oracle.quant_act(xb, bf16_bits=True)
    np.testing.assert_array_equal(y, oracle.dequant(acc, ds_all, beta))
