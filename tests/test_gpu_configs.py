"""Parity at the benchmark configurations' full sizes, on every output, in the
launch modes bench.py times.

The shapes are those of the single BitLinear (4 tokens, 512 -> 512), the
decode GEMV (2B-class, one token, fused quantization), the prefill GEMM
(2B-class, 2048 tokens) and the 100B-class layer (decode at 1, 8 and 32
tokens, prefill at 512).  The launch mode of each case is the one bench.py
picks for that batch: the fused decode kernel up to 4 tokens, the standalone
quantizer then bitlinear_gemv up to 64 tokens, and the quantizer then
bitlinear_gemm beyond.  The small config also runs through the other modes.

The oracle computes the whole product at these sizes (absmean ternarization
of the whole matrix, per-token absmax quantization, the naive int32 triple
loop over OpenMP threads, fp32 dequantization; about 120 G multiply-adds for
the largest case).  The GPU's int32 accumulators must equal the oracle's bit
for bit on every output; its fp32 outputs must equal the oracle's exactly
(both sides evaluate (float)acc * (ds * beta) with the same IEEE operations,
which is within the 1e-3 relative contract), and its bf16 outputs must equal
the oracle's round-to-nearest-even conversion of them.
"""
import functools
import os

import numpy as np
import pytest
import torch

import bitlinear_matmul_02_amd as bl
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
THREADS = max(1, min(16, os.cpu_count() or 1))

# (workload, tokens, K, N, launch mode)
CASES = [
    ("single_4x512x512", 4, 512, 512, "fused"),
    ("single_4x512x512", 4, 512, 512, "gemv"),
    ("single_4x512x512", 4, 512, 512, "gemm"),
    ("decode_gemv_2b_m1", 1, 2560, 6912, "fused"),
    ("decode_gemv_2b_m1", 1, 6912, 2560, "fused"),
    ("decode_gemv_2b_m1", 1, 2560, 6912, "gemv"),
    ("decode_gemv_2b_m1", 1, 6912, 2560, "gemv"),
    ("prefill_2b_m2048", 2048, 2560, 6912, "gemm"),
    ("prefill_2b_m2048", 2048, 6912, 2560, "gemm"),
    ("decode_100b_m1", 1, 8192, 28672, "fused"),
    ("decode_100b_m1", 1, 28672, 8192, "fused"),
    ("decode_100b_m1", 1, 8192, 28672, "gemv"),
    ("decode_100b_m1", 1, 28672, 8192, "gemv"),
    ("decode_100b_m8", 8, 8192, 28672, "gemv"),
    ("decode_100b_m8", 8, 28672, 8192, "gemv"),
    ("decode_100b_m32", 32, 8192, 28672, "gemv"),
    ("decode_100b_m32", 32, 28672, 8192, "gemv"),
    ("prefill_100b_m512", 512, 8192, 28672, "gemm"),
    ("prefill_100b_m512", 512, 28672, 8192, "gemm"),
]


@functools.lru_cache(maxsize=2)
def weights(N: int, K: int):
    """Ternary codes and beta (oracle) and the packed tiles on the device."""
    w = workloads.gen_weights(N, K, seed=11000 + N + K)
    beta = oracle.absmean(w)
    t = oracle.ternarize(w, beta)
    packed, b_dev = bl.pack_weights(torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    del w
    assert b_dev.cpu().numpy()[0] == beta
    return t, beta, packed, b_dev


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
        if ws is not None:
            assert int(torch.count_nonzero(ws)) == 0, "workspace not left zero"
    torch.cuda.synchronize()
    out = y.cpu()
    return (out.view(torch.int16).numpy().view(np.uint16) if out_dtype == torch.bfloat16 else out.numpy())


@pytest.mark.parametrize("name,M,K,N,mode", CASES, ids=["%s-%dx%d->%d-%s" % c for c in CASES])
def test_config_full_parity(name, M, K, N, mode):
    assert mode != "fused" or bl.decode_fits(M, K)
    t, beta, packed, b_dev = weights(N, K)
    xb = workloads.gen_acts_bf16(M, K, seed=12000 + M + K, outliers=name.startswith("decode_gemv"))
    x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).to(DEV)

    q, ds, _ = oracle.quant_act(xb, bf16_bits=True)
    acc_ref = oracle.matmul_i32(q, t, threads=THREADS)
    y_ref = oracle.dequant(acc_ref, ds, beta)

    acc = launch(mode, x, M, K, N, packed, b_dev, torch.int32)
    np.testing.assert_array_equal(acc, acc_ref)
    y = launch(mode, x, M, K, N, packed, b_dev, torch.float32)
    np.testing.assert_array_equal(y, y_ref)
    if M * N <= (1 << 22):
        yb = launch(mode, x, M, K, N, packed, b_dev, torch.bfloat16)
        np.testing.assert_array_equal(yb, oracle.to_bf16_bits(y_ref))
