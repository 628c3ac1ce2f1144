"""Parity of the training products (straight-through BitLinear) with the oracle.

The oracle sums exactly in fp64; the GPU sums bf16 x ternary (or bf16 x bf16)
products, each exact in fp32, with fp32 additions on the matrix cores and then
multiplies by beta.  The bar derived from that arithmetic: |gpu - ref| <=
2^-23 |ref| + L * 2^-24 * sum |terms| for a contraction of length L (the
worst-case bound of L fp32 additions).  Entries without heavy cancellation
(|ref| >= 1% of sum |terms|) must also meet the 1e-3 relative contract."""
import numpy as np
import pytest
import torch

import bitlinear_matmul_02_amd as bl
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check(got, ref, absterms, L):
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    bound = 2.0 ** -23 * np.abs(ref) + L * 2.0 ** -24 * absterms
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) - bound))
    plain = np.abs(ref) >= 0.01 * absterms
    assert np.all(np.abs(got - ref)[plain] <= 1e-3 * np.abs(ref)[plain])


@pytest.mark.parametrize("M,K,N", [(1, 256, 16), (4, 512, 512), (65, 700, 333), (128, 2560, 640), (200, 1030, 130),
                                   (257, 6912, 260), (3, 13, 5)])
def test_train_products_parity(M, K, N):
    rng = np.random.default_rng(M + K + N)
    w = workloads.gen_weights(N, K, seed=K + N)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    dy = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    packed, beta = bl.pack_weights(torch.from_numpy(w).to(DEV))
    y = torch.full((M, N), 7.0, device=DEV)
    dx = torch.full((M, K), 7.0, device=DEV)
    dw = torch.full((N, K), 7.0, device=DEV)
    bl.bitlinear_train_forward(x, packed, beta, N, y)
    bl.bitlinear_train_backward_input(dy, packed, beta, K, dx)
    bl.bitlinear_train_backward_weight(dy, x, dw)
    torch.cuda.synchronize()
    b = oracle.absmean(w)
    t = oracle.ternarize(w, b)
    xb, dyb = bf16_bits(x), bf16_bits(dy)
    xa = np.abs(workloads.bf16_bits_to_f32(xb).astype(np.float64))
    dya = np.abs(workloads.bf16_bits_to_f32(dyb).astype(np.float64))
    ta = np.abs(t).astype(np.float64)
    check(y.cpu().numpy(), oracle.train_forward(xb, t, b, threads=8), float(b) * (xa @ ta.T), K)
    check(dx.cpu().numpy(), oracle.train_dx(dyb, t, b, threads=8), float(b) * (dya @ ta), N)
    check(dw.cpu().numpy(), oracle.train_dw(dyb, xb, threads=8), dya.T @ xa, M)


def test_train_exact_small_integers():
    # integer inputs and a power-of-two beta: every sum is exact, results bit-equal
    M, K, N = 33, 512, 48
    rng = np.random.default_rng(5)
    x = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    dy = rng.integers(-3, 4, size=(M, N)).astype(np.float32)
    # half the weights +-1, half 0: beta = mean |w| = 0.5 exactly and t = w
    w = np.zeros((N, K), dtype=np.float32)
    idx = rng.permutation(N * K)[: N * K // 2]
    w.flat[idx] = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=idx.size)
    packed, beta = bl.pack_weights(torch.from_numpy(w).to(DEV))
    xd = torch.from_numpy(x).to(torch.bfloat16).to(DEV)
    dyd = torch.from_numpy(dy).to(torch.bfloat16).to(DEV)
    y = torch.empty((M, N), device=DEV)
    dx = torch.empty((M, K), device=DEV)
    dw = torch.empty((N, K), device=DEV)
    bl.bitlinear_train_forward(xd, packed, beta, N, y)
    bl.bitlinear_train_backward_input(dyd, packed, beta, K, dx)
    bl.bitlinear_train_backward_weight(dyd, xd, dw)
    torch.cuda.synchronize()
    b = oracle.absmean(w)
    t = oracle.ternarize(w, b)
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.train_forward(bf16_bits(xd), t, b))
    np.testing.assert_array_equal(dx.cpu().numpy(), oracle.train_dx(bf16_bits(dyd), t, b))
    np.testing.assert_array_equal(dw.cpu().numpy(), oracle.train_dw(bf16_bits(dyd), bf16_bits(xd)))


@pytest.mark.parametrize("product,M,K,N", [("forward", 2048, 512, 6144), ("input", 2048, 6144, 512),
                                           ("weight", 512, 6144, 2048)])
def test_train_products_large_blocks(product, M, K, N):
    """Grids of at least 192 blocks of 256 x 256 outputs take the 8-wave kernel
    with 32-wide stages; the oracle checks 64 sampled output rows (the first and
    last 8 and 48 drawn ones), every column."""
    rng = np.random.default_rng({"forward": 1, "input": 2, "weight": 3}[product])
    w = workloads.gen_weights(N, K, seed=K + N + 1)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    dy = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    packed, beta = bl.pack_weights(torch.from_numpy(w).to(DEV))
    b = oracle.absmean(w)
    t = oracle.ternarize(w, b)
    xb, dyb = bf16_bits(x), bf16_bits(dy)
    P = N if product == "weight" else M
    rows = np.unique(np.concatenate([np.arange(8), np.arange(P - 8, P), rng.choice(P, 48, replace=False)]))
    ta = np.abs(t).astype(np.float64)
    if product == "forward":
        out = torch.full((M, N), 7.0, device=DEV)
        bl.bitlinear_train_forward(x, packed, beta, N, out)
        ref = oracle.train_forward(xb[rows], t, b, threads=8)
        terms = float(b) * (np.abs(workloads.bf16_bits_to_f32(xb[rows]).astype(np.float64)) @ ta.T)
        L = K
    elif product == "input":
        out = torch.full((M, K), 7.0, device=DEV)
        bl.bitlinear_train_backward_input(dy, packed, beta, K, out)
        ref = oracle.train_dx(dyb[rows], t, b, threads=8)
        terms = float(b) * (np.abs(workloads.bf16_bits_to_f32(dyb[rows]).astype(np.float64)) @ ta)
        L = N
    else:
        out = torch.full((N, K), 7.0, device=DEV)
        bl.bitlinear_train_backward_weight(dy, x, out)
        dys = np.ascontiguousarray(dyb[:, rows])
        ref = oracle.train_dw(dys, xb, threads=8)
        terms = (np.abs(workloads.bf16_bits_to_f32(dys).astype(np.float64)).T
                 @ np.abs(workloads.bf16_bits_to_f32(xb).astype(np.float64)))
        L = M
    torch.cuda.synchronize()
    check(out.cpu().numpy()[rows], ref, terms, L)
