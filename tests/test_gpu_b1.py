"""Parity of the binary-weight (BitNet b1) path with the CPU oracle: packed
bytes and beta bit-exact, int32 accumulators bit-exact, fp32 / bf16 outputs
within 1e-3 / 1e-2 relative (and in fact bit-equal)."""
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


@pytest.mark.parametrize("N,K", [(1, 1), (16, 512), (17, 600), (640, 2560), (2560, 6912), (33, 1030)])
def test_pack_b1_parity(N, K):
    w = workloads.gen_weights(N, K, seed=N * 7 + K)
    w.flat[::97] = 0.0  # zeros map to +1
    packed, beta = bl.pack_weights_b1(torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    t = oracle.binarize(w)
    np.testing.assert_array_equal(packed.cpu().numpy(), oracle.pack_b1(t))
    assert beta.cpu().numpy()[0] == oracle.absmean(w)


def gpu_b1(xb, w, out_dtype, gemm=False):
    M, K = xb.shape
    N = w.shape[0]
    packed, beta = bl.pack_weights_b1(torch.from_numpy(w).to(DEV))
    x_q, x_ds, rs = bl.quant_act(to_dev_bf16(xb), with_rowsum=True)
    y = torch.empty((M, N), dtype=out_dtype, device=DEV)
    (bl.bitlinear_gemm_b1 if gemm else bl.bitlinear_gemv_b1)(x_q, x_ds, rs, K, packed, beta, N, y)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M,K,N", [(1, 2560, 6912), (1, 6912, 2560), (4, 512, 512), (8, 2560, 640), (3, 700, 333),
                                   (16, 1030, 48), (33, 2560, 100), (64, 512, 64), (8, 8192, 256), (2, 13, 20),
                                   (1, 28672, 64)])
def test_gemv_b1_parity(M, K, N):
    w = workloads.gen_weights(N, K, seed=M + K + N)
    xb = workloads.gen_acts_bf16(M, K, seed=M * 3 + K, outliers=True)
    if M > 2:
        xb[M // 2] = 0  # a zero token
    ref = oracle.bitlinear_forward_b1(xb, w, threads=8)
    acc = gpu_b1(xb, w, torch.int32).cpu().numpy()
    np.testing.assert_array_equal(acc, ref["acc"])
    y = gpu_b1(xb, w, torch.float32).cpu().numpy()
    assert rel_ok(y, ref["y"], 1e-3)
    np.testing.assert_array_equal(y, ref["y"])
    yb = gpu_b1(xb, w, torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    assert rel_ok(workloads.bf16_bits_to_f32(yb), workloads.bf16_bits_to_f32(ref["y_bf16"]), 1e-2)
    np.testing.assert_array_equal(yb, ref["y_bf16"])


def test_gemv_b1_extremes():
    # all weights +1 with all codes 127: |acc| = 127 * K at the largest shapes
    M, K, N = 2, 131072, 16
    w = np.ones((N, K), dtype=np.float32)
    w[1] = -1.0
    x = np.full((M, K), 1.0, dtype=np.float32)
    x[1] = -2.0
    packed, beta = bl.pack_weights_b1(torch.from_numpy(w).to(DEV))
    x_q, x_ds, rs = bl.quant_act(torch.from_numpy(x).to(DEV), with_rowsum=True)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    bl.bitlinear_gemv_b1(x_q, x_ds, rs, K, packed, beta, N, acc)
    torch.cuda.synchronize()
    a = acc.cpu().numpy()
    assert a[0, 0] == 127 * K and a[0, 1] == -127 * K and a[1, 0] == -127 * K and a[1, 1] == 127 * K


def test_gemv_b1_empty_batch():
    packed, beta = bl.pack_weights_b1(torch.zeros((16, 512), device=DEV))
    x_q = torch.zeros((0, bl.act_stride(512)), dtype=torch.int8, device=DEV)
    x_ds = torch.zeros((0,), dtype=torch.float32, device=DEV)
    rs = torch.zeros((0,), dtype=torch.int32, device=DEV)
    y = torch.zeros((0, 16), dtype=torch.float32, device=DEV)
    bl.bitlinear_gemv_b1(x_q, x_ds, rs, 512, packed, beta, 16, y)
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,K,N", [(1, 512, 16), (65, 1030, 48), (128, 2560, 256), (129, 768, 300), (300, 6912, 640),
                                   (2048, 2560, 512), (256, 13, 20)])
def test_gemm_b1_parity(M, K, N):
    w = workloads.gen_weights(N, K, seed=M * 11 + K + N)
    xb = workloads.gen_acts_bf16(M, K, seed=M + 2 * K)
    xb[M // 3] = 0
    ref = oracle.bitlinear_forward_b1(xb, w, threads=8)
    acc = gpu_b1(xb, w, torch.int32, gemm=True).cpu().numpy()
    np.testing.assert_array_equal(acc, ref["acc"])
    y = gpu_b1(xb, w, torch.float32, gemm=True).cpu().numpy()
    assert rel_ok(y, ref["y"], 1e-3)
    np.testing.assert_array_equal(y, ref["y"])
