"""Parity of the base-3 packed ternary path with the CPU oracle: packed bytes
and beta bit-exact, int32 accumulators bit-exact, fp32 / bf16 outputs within
1e-3 / 1e-2 relative (and in fact bit-equal) -- the same results as the 2-bit
path on the same weights."""
import numpy as np
import pytest
import torch

import bitlinear_matmul_02_amd as bl
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def to_dev_bf16(xb):
    return torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).to(DEV)


def rel_ok(got, ref, rtol):
    got, ref = got.astype(np.float64), ref.astype(np.float64)
    z = ref == 0
    return not np.any(got[z] != 0) and bool(np.all(np.abs(got[~z] - ref[~z]) <= rtol * np.abs(ref[~z])))


@pytest.mark.parametrize("N,K", [(1, 1), (16, 320), (17, 700), (640, 2560), (2560, 6912), (33, 1030)])
def test_pack_b3_parity(N, K):
    w = workloads.gen_weights(N, K, seed=N * 5 + K)
    packed, beta = bl.pack_weights_b3(torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    b = oracle.absmean(w)
    assert beta.cpu().numpy()[0] == b
    np.testing.assert_array_equal(packed.cpu().numpy(), oracle.pack_b3(oracle.ternarize(w, b)))


def gpu_b3(xb, w, out_dtype):
    M, K = xb.shape
    N = w.shape[0]
    packed, beta = bl.pack_weights_b3(torch.from_numpy(w).to(DEV))
    x_q, x_ds, rs = bl.quant_act(to_dev_bf16(xb), with_rowsum=True)
    y = torch.empty((M, N), dtype=out_dtype, device=DEV)
    bl.bitlinear_gemv_b3(x_q, x_ds, rs, K, packed, beta, N, y)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M,K,N", [(1, 2560, 6912), (1, 6912, 2560), (4, 512, 512), (8, 2560, 640), (3, 700, 333),
                                   (16, 1030, 48), (33, 2560, 100), (64, 320, 64), (8, 8192, 256), (2, 13, 20),
                                   (1, 28672, 64)])
def test_gemv_b3_parity(M, K, N):
    w = workloads.gen_weights(N, K, seed=M + K + N + 1)
    xb = workloads.gen_acts_bf16(M, K, seed=M * 5 + K, outliers=True)
    if M > 2:
        xb[M // 2] = 0
    ref = oracle.bitlinear_forward(xb, w, threads=8)
    acc = gpu_b3(xb, w, torch.int32).cpu().numpy()
    np.testing.assert_array_equal(acc, ref["acc"])
    y = gpu_b3(xb, w, torch.float32).cpu().numpy()
    assert rel_ok(y, ref["y"], 1e-3)
    np.testing.assert_array_equal(y, ref["y"])
    yb = gpu_b3(xb, w, torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(yb, ref["y_bf16"])


def test_gemv_b3_extremes():
    # all codes +1 / -1 with |q| = 127: |acc| = 127 * K at the largest K
    M, K, N = 2, 131072, 16
    w = np.ones((N, K), dtype=np.float32)
    w[1] = -1.0
    w[2] = 0.0
    x = np.full((M, K), 1.0, dtype=np.float32)
    x[1] = -2.0
    packed, beta = bl.pack_weights_b3(torch.from_numpy(w).to(DEV))
    x_q, x_ds, rs = bl.quant_act(torch.from_numpy(x).to(DEV), with_rowsum=True)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    bl.bitlinear_gemv_b3(x_q, x_ds, rs, K, packed, beta, N, acc)
    torch.cuda.synchronize()
    a = acc.cpu().numpy()
    # beta = mean |w| = 14/16, d = beta + 1e-8: w = +-1 -> round(1.14) = 1, w = 0 -> 0
    assert a[0, 0] == 127 * K and a[0, 1] == -127 * K and a[1, 0] == -127 * K and a[0, 2] == 0
