"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Every input is drawn on the host by ``workloads`` and fed byte-identically to
both sides.  Integer results (int8 codes, packed bytes, int32 accumulators)
must match bit for bit; dequantized outputs must be within 1e-3 relative
(fp32) / 1e-2 (bf16) of the oracle, and are in fact expected bit-equal since
both sides evaluate y = (float)acc * (ds * beta) with the same IEEE operations.
"""
import numpy as np
import pytest
import torch

import bitlinear_matmul_02_amd as bl
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
RTOL_F32, RTOL_BF16 = 1e-3, 1e-2


def to_dev_bf16(xb: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).to(DEV)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def rel_err_ok(got: np.ndarray, ref: np.ndarray, rtol: float) -> bool:
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    zero = ref == 0
    if np.any(got[zero] != 0):
        return False
    return bool(np.all(np.abs(got[~zero] - ref[~zero]) <= rtol * np.abs(ref[~zero])))


def gpu_pack(w: np.ndarray):
    return bl.pack_weights(torch.from_numpy(w).to(DEV))


def gpu_forward(xb, packed, beta, N, K, out_dtype, use_gemm):
    x = to_dev_bf16(xb)
    M = x.shape[0]
    y = torch.empty((M, N), dtype=out_dtype, device=DEV)
    if use_gemm == "fused":
        bl.bitlinear_forward_decode(x, packed, beta, N, y)
        torch.cuda.synchronize()
        return y
    x_q, x_ds = bl.quant_act(x)
    if use_gemm:
        ws = bl.workspace(bl.gemm_workspace_bytes(M, N, K), DEV)
        bl.bitlinear_gemm(x_q, x_ds, K, packed, beta, N, y, ws)
    else:
        ws = bl.workspace(bl.gemv_workspace_bytes(M, N, K), DEV)
        bl.bitlinear_gemv(x_q, x_ds, K, packed, beta, N, y, ws)
    torch.cuda.synchronize()
    return y


def check_product(xb, w, use_gemm, dtypes=("i32", "f32", "bf16"), ref=None):
    M, K = xb.shape
    N = w.shape[0]
    if ref is None:
        ref = oracle.bitlinear_forward(xb, w, threads=8)
    packed, beta = gpu_pack(w)
    assert beta.cpu().numpy()[0] == ref["beta"]
    if "i32" in dtypes:
        acc = gpu_forward(xb, packed, beta, N, K, torch.int32, use_gemm).cpu().numpy()
        np.testing.assert_array_equal(acc, ref["acc"])
    if "f32" in dtypes:
        y = gpu_forward(xb, packed, beta, N, K, torch.float32, use_gemm).cpu().numpy()
        assert rel_err_ok(y, ref["y"], RTOL_F32)
        np.testing.assert_array_equal(y, ref["y"])  # same IEEE ops on both sides
    if "bf16" in dtypes:
        yb = bf16_bits(gpu_forward(xb, packed, beta, N, K, torch.bfloat16, use_gemm))
        assert rel_err_ok(workloads.bf16_bits_to_f32(yb), workloads.bf16_bits_to_f32(ref["y_bf16"]), RTOL_BF16)
        np.testing.assert_array_equal(yb, ref["y_bf16"])


# --------------------------------------------------------------- quant_act
@pytest.mark.parametrize("M,K,outliers", [(1, 1, False), (1, 7, False), (3, 300, False), (4, 512, False),
                                          (1, 2560, True), (2, 6912, True), (8, 8192, False),
                                          (33, 28672, False), (5, 255, True), (2048, 64, False)])
@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_quant_act_parity(M, K, outliers, src):
    xb = workloads.gen_acts_bf16(M, K, seed=M * 7 + K, outliers=outliers)
    if src == "bf16":
        x = to_dev_bf16(xb)
        q_ref, ds_ref, rs_ref = oracle.quant_act(xb, bf16_bits=True)
    else:
        xf = workloads.bf16_bits_to_f32(xb) * np.float32(1.37)  # values beyond bf16 precision
        x = torch.from_numpy(xf).to(DEV)
        q_ref, ds_ref, rs_ref = oracle.quant_act(xf)
    x_q, x_ds, rs = bl.quant_act(x, with_rowsum=True)
    torch.cuda.synchronize()
    q = x_q.cpu().numpy()
    assert q.shape == (M, bl.act_stride(K))
    np.testing.assert_array_equal(q[:, :K], q_ref)
    assert not q[:, K:].any()
    np.testing.assert_array_equal(x_ds.cpu().numpy(), ds_ref)
    np.testing.assert_array_equal(rs.cpu().numpy(), rs_ref)


def test_quant_act_zero_row_and_unaligned_rows():
    K = 13  # odd row length: rows are not 16-byte aligned -> scalar path
    xb = workloads.gen_acts_bf16(3, K, seed=4)
    xb[1] = 0
    x = to_dev_bf16(xb)
    x_q, x_ds, rs = bl.quant_act(x, with_rowsum=True)
    q_ref, ds_ref, rs_ref = oracle.quant_act(xb, bf16_bits=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(x_q.cpu().numpy()[:, :K], q_ref)
    np.testing.assert_array_equal(x_ds.cpu().numpy(), ds_ref)
    assert rs_ref[1] == 0 and not q_ref[1].any()


# -------------------------------------------------------------------- pack
@pytest.mark.parametrize("N,K", [(1, 1), (16, 256), (17, 257), (35, 700), (512, 512), (640, 2560),
                                 (6912, 2560), (2560, 6912), (3, 5000)])
def test_pack_parity(N, K):
    w = workloads.gen_weights(N, K, seed=N + 31 * K)
    beta_ref = oracle.absmean(w)
    packed_ref = oracle.pack_t2(oracle.ternarize(w, beta_ref))
    packed, beta = gpu_pack(w)
    torch.cuda.synchronize()
    assert beta.cpu().numpy()[0] == beta_ref
    np.testing.assert_array_equal(packed.cpu().numpy(), packed_ref)


def test_pack_zero_and_tie_weights():
    # all-zero weights: beta = 0, every code 0
    w = np.zeros((20, 300), dtype=np.float32)
    packed, beta = gpu_pack(w)
    assert beta.cpu().item() == 0.0 and not packed.cpu().numpy().any()
    # exact ties: mean |w| = 0.5 exactly, so d = 0.5 and w/d hits 0.5, 1.5, 2.5
    pattern = np.array([0.25, -0.25, 0.25, -0.25, 0.75, -0.75, 1.25, -0.25], dtype=np.float32)
    w = np.tile(pattern, (16, 32))
    beta_ref = oracle.absmean(w)
    assert beta_ref == np.float32(0.5)
    packed, beta = gpu_pack(w)
    assert beta.cpu().numpy()[0] == beta_ref
    t_ref = oracle.ternarize(w, beta_ref)
    np.testing.assert_array_equal(t_ref[0, :8], [0, 0, 0, 0, 1, -1, 1, 0])
    np.testing.assert_array_equal(packed.cpu().numpy(), oracle.pack_t2(t_ref))


# --------------------------------------------------------------- products
def test_hand_example_on_gpu(golden_dir):  # noqa: C901
    import json
    import os
    with open(os.path.join(golden_dir, "hand_4x4.json")) as f:
        h = json.load(f)
    w = np.array(h["w"], dtype=np.float32)
    x = np.array(h["x"], dtype=np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    for use_gemm in (False, True, "fused"):
        packed, beta = gpu_pack(w)
        assert beta.cpu().item() == h["beta"]
        acc = gpu_forward(xb, packed, beta, 4, 4, torch.int32, use_gemm).cpu().numpy()
        np.testing.assert_array_equal(acc, np.array(h["acc"]))
        y = gpu_forward(xb, packed, beta, 4, 4, torch.float32, use_gemm).cpu().numpy()
        np.testing.assert_array_equal(y, np.array(h["y"], dtype=np.float32))


@pytest.mark.parametrize("M", [1, 2, 4, 8, 15, 16, 17, 31, 32, 33, 48, 64])
@pytest.mark.parametrize("N,K", [(16, 256), (40, 700), (512, 512), (100, 3000)])
def test_gemv_parity(M, N, K):
    w = workloads.gen_weights(N, K, seed=1000 + N)
    xb = workloads.gen_acts_bf16(M, K, seed=2000 + M, outliers=True)
    check_product(xb, w, use_gemm=False)


@pytest.mark.parametrize("M", [1, 2, 8, 16, 17, 33, 64])
@pytest.mark.parametrize("N,K", [(16, 256), (40, 700), (512, 512), (100, 3000), (2000, 300)])
def test_forward_decode_parity(M, N, K):
    if not bl.decode_fits(M, K):
        pytest.skip("activations exceed the fused kernel's LDS budget")
    w = workloads.gen_weights(N, K, seed=5000 + N)
    xb = workloads.gen_acts_bf16(M, K, seed=6000 + M, outliers=True)
    check_product(xb, w, use_gemm="fused")


def test_forward_decode_f32_input_and_zero_row():
    M, N, K = 3, 80, 1000
    w = workloads.gen_weights(N, K, seed=70)
    x = workloads.bf16_bits_to_f32(workloads.gen_acts_bf16(M, K, seed=71)) * np.float32(1.37)
    x[1] = 0
    q, ds, _ = oracle.quant_act(x)
    beta = oracle.absmean(w)
    acc = oracle.matmul_i32(q, oracle.ternarize(w, beta))
    y_ref = oracle.dequant(acc, ds, beta)
    packed, b = gpu_pack(w)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    bl.bitlinear_forward_decode(torch.from_numpy(x).to(DEV), packed, b, N, y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), y_ref)


@pytest.mark.parametrize("M", [1, 16, 65, 100, 128, 129, 300])
@pytest.mark.parametrize("N,K", [(16, 256), (40, 700), (200, 1000), (512, 512)])
def test_gemm_parity(M, N, K):
    w = workloads.gen_weights(N, K, seed=3000 + N)
    xb = workloads.gen_acts_bf16(M, K, seed=4000 + M)
    check_product(xb, w, use_gemm=True)


# 128 x 256 blocks: bitlinear_gemm takes them while ceil(M/128) * ceil(N/256)
# >= 384 (each case below is at or above that), with ragged token, output
# and k tails
@pytest.mark.parametrize("M,N,K", [(2048, 6144, 512), (1999, 6100, 1000), (3000, 4100, 700)])
def test_gemm_big_tile_parity(M, N, K):
    assert -(-M // 128) * -(-N // 256) >= 384
    w = workloads.gen_weights(N, K, seed=3100 + N)
    xb = workloads.gen_acts_bf16(M, K, seed=4100 + M)
    check_product(xb, w, use_gemm=True, ref=oracle.bitlinear_forward(xb, w, threads=16))


# Decode plans with many output groups and long k-runs per wave: one token
# block, 2-block workgroups, >= 512 groups and >= 32 k-tiles (8 tokens with
# operands from global memory; one token fused with rows staged in LDS)
@pytest.mark.parametrize("M,N,K,mode", [(8, 16400, 8192, "gemv"), (1, 16400, 8192, "fused"),
                                        (1, 16400, 8200, "gemv"), (2, 8200, 28700, "fused")])
def test_gemv_large_plans_parity(M, N, K, mode):
    w = workloads.gen_weights(N, K, seed=3200 + N)
    xb = workloads.gen_acts_bf16(M, K, seed=4200 + M, outliers=True)
    check_product(xb, w, use_gemm=mode if mode == "fused" else False, dtypes=("i32", "f32"),
                  ref=oracle.bitlinear_forward(xb, w, threads=16))


# Wide decode plans: one token block and 1024..2048 output blocks on 2-bit
# tiles, activation rows staged in LDS (fused, or int8 rows of up to 7 tokens
# of 8192): one workgroup per compute unit owns ceil(Nt / 256) output blocks
# and its waves take interleaved k-tiles.  Ragged N (last group clamps its
# blocks), ragged K (waves with one k-tile more), fewer k-tiles than waves,
# and 4..8 blocks per workgroup.
# From 9 tokens of 8192 the int8 rows take 16 pieces per thread (its own
# instantiation); up to 16 tokens and 144 KB of rows stay on this kernel.
@pytest.mark.parametrize("M,N,K,mode", [(3, 20000, 8200, "gemv"), (7, 16384, 4096, "gemv"), (1, 32768, 1000, "fused"),
                                        (2, 23000, 6000, "fused"), (5, 17000, 300, "gemv"), (1, 24576, 8192, "gemv"),
                                        (4, 28672, 8192, "gemv"), (6, 28000, 2000, "fused"), (16, 28672, 8192, "gemv"),
                                        (10, 20000, 8200, "gemv"), (13, 32768, 2048, "gemv"), (9, 16384, 16000, "gemv"),
                                        (16, 16384, 8192, "gemv"), (1, 32768, 8192, "fused"), (2, 16383, 4096, "gemv")])
def test_gemv_wide_plans_parity(M, N, K, mode):
    assert 1024 <= -(-N // 16) <= 2048
    w = workloads.gen_weights(N, K, seed=3300 + N)
    xb = workloads.gen_acts_bf16(M, K, seed=4300 + M, outliers=True)
    check_product(xb, w, use_gemm=mode if mode == "fused" else False,
                  ref=oracle.bitlinear_forward(xb, w, threads=16))


def test_gemv_just_past_the_wide_plans():
    """2049 output blocks (N = 32784) take the two-block plan again; results
    are the same."""
    M, N, K = 3, 32784, 1024
    w = workloads.gen_weights(N, K, seed=3400)
    xb = workloads.gen_acts_bf16(M, K, seed=4400, outliers=True)
    check_product(xb, w, use_gemm=False, dtypes=("i32", "f32"), ref=oracle.bitlinear_forward(xb, w, threads=16))


# ----------------------------------- up to 64 tokens on the int8 matrix cores
@pytest.mark.parametrize("M,N,K,split", [(1, 1000, 4096, True), (37, 333, 6925, True), (64, 6912, 2560, True),
                                         (24, 130, 2048, True), (17, 2560, 6912, True), (64, 64, 512, False),
                                         (64, 28672, 1024, False), (32, 8192, 28672, True), (33, 8192, 4096, True),
                                         (32, 65536, 512, False), (9, 300, 700, False)])
def test_gemm_small_batch_parity(M, N, K, split):
    """32-row blocks up to 32 tokens, 64-row blocks up to 64; with few blocks
    the k-steps are split across workgroups (int32 partial sums in the
    workspace, added and dequantized by a second kernel, which zeroes them
    again)."""
    need = bl.gemm_workspace_bytes(M, N, K)
    assert (need > 0) == split
    w = workloads.gen_weights(N, K, seed=7000 + N)
    xb = workloads.gen_acts_bf16(M, K, seed=8000 + M, outliers=True)
    ref = oracle.bitlinear_forward(xb, w, threads=8)
    for _ in range(2):  # the same cached workspace twice
        check_product(xb, w, use_gemm=True, ref=ref)
    if need > 0:
        ws = bl.workspace(need, DEV)
        torch.cuda.synchronize()
        assert not ws[:need].any().item()


# Up to 32 tokens on 16384 or more outputs, where the 32 x 256 blocks would
# split k across workgroups, the blocks are 32 x 128 and each workgroup's two
# halves take half of every k-step's matrix-core steps, adding their sums in
# LDS: no workspace.  Ragged N and K, one token, and every output mode.
@pytest.mark.parametrize("M,N,K", [(1, 17000, 3000), (5, 20000, 2000), (17, 16400, 2048), (32, 16384, 8192),
                                   (31, 30000, 2100)])
def test_gemm_small_batch_k_split_in_workgroup(M, N, K):
    assert bl.gemm_workspace_bytes(M, N, K) == 0
    w = workloads.gen_weights(N, K, seed=7500 + N)
    xb = workloads.gen_acts_bf16(M, K, seed=8500 + M, outliers=True)
    check_product(xb, w, use_gemm=True, ref=oracle.bitlinear_forward(xb, w, threads=16))


@pytest.mark.parametrize("M,N,K", [(12, 8192, 16384), (24, 16384, 8192), (33, 4096, 4096), (49, 300, 1000),
                                   (32, 2560, 2560), (11, 8192, 16384), (6, 28672, 8192), (12, 16384, 8192),
                                   (17, 28672, 8192)])
def test_gemv_large_batches(M, N, K):
    """bitlinear_gemv hands larger batches to the small-batch matrix-core path
    (from 12 tokens on 2^27 weights, 33 on 2^24, 49 on any) unless a wide plan
    covers them (up to 16 tokens, 1024..2048 output blocks, rows within 144 KB
    of LDS: 6 and 12 x 8192 -> 16384 / 28672 stay on this kernel, 17 tokens
    do not); results are the same either way."""
    w = workloads.gen_weights(N, K, seed=9000 + N)
    xb = workloads.gen_acts_bf16(M, K, seed=9500 + M)
    check_product(xb, w, use_gemm=False, dtypes=("i32", "f32"))


def test_gemv_split_k_workspace_left_zero():
    # a long K with few outputs makes the plan split K across workgroups
    M, N, K = 3, 48, 70000
    need = bl.gemv_workspace_bytes(M, N, K)
    assert need > 0
    w = workloads.gen_weights(N, K, seed=5)
    xb = workloads.gen_acts_bf16(M, K, seed=6)
    ref = oracle.bitlinear_forward(xb, w, threads=8)
    for _ in range(3):  # repeated calls reuse the same workspace
        check_product(xb, w, use_gemm=False, dtypes=("i32",), ref=ref)
    if need > 0:
        ws = bl.workspace(need, DEV)
        torch.cuda.synchronize()
        assert not ws[:need].any().item()


def test_workspace_shared_by_split_products():
    """One workspace serves the GEMV split across workgroups (needs zeros on
    entry) and the small-batch GEMM split (fills and re-zeroes its slices),
    alternately; every result stays exact and the buffer ends zero."""
    cases = [(3, 48, 70000), (32, 640, 6912)]  # (M, N, K): GEMV split-K, GEMM split
    need = max(max(bl.gemv_workspace_bytes(*c), bl.gemm_workspace_bytes(*c)) for c in cases)
    assert bl.gemv_workspace_bytes(*cases[0]) > 0 and bl.gemm_workspace_bytes(*cases[1]) > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    data = []
    for i, (M, N, K) in enumerate(cases):
        w = workloads.gen_weights(N, K, seed=60 + i)
        xb = workloads.gen_acts_bf16(M, K, seed=70 + i)
        packed, beta = gpu_pack(w)
        x_q, x_ds = bl.quant_act(to_dev_bf16(xb))
        data.append((x_q, x_ds, K, packed, beta, N, oracle.bitlinear_forward(xb, w, threads=8)["acc"]))
    for _ in range(3):
        for fn, (x_q, x_ds, K, packed, beta, N, acc) in zip((bl.bitlinear_gemv, bl.bitlinear_gemm), data):
            y = torch.empty((x_q.shape[0], N), dtype=torch.int32, device=DEV)
            fn(x_q, x_ds, K, packed, beta, N, y, ws)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(y.cpu().numpy(), acc)
    assert not ws.any().item()


def test_max_magnitude_accumulators():
    # q = +-127 everywhere and t = +-1 everywhere at the largest K: |acc| = 127*K
    K, N, M = bl.MAX_K, 32, 2
    w = np.full((N, K), 0.02, dtype=np.float32)
    w[1::2] = -0.02
    x = np.full((M, K), 3.0, dtype=np.float32)
    x[1] = -3.0
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    ref = oracle.bitlinear_forward(xb, w, threads=8)
    assert int(np.abs(ref["acc"]).max()) == 127 * K
    check_product(xb, w, use_gemm=False, dtypes=("i32", "f32"), ref=ref)
    check_product(xb, w, use_gemm=True, dtypes=("i32", "f32"), ref=ref)


def test_zero_token_and_zero_weights():
    K, N = 512, 64
    w = workloads.gen_weights(N, K, seed=8)
    w[5] = 0.0
    xb = workloads.gen_acts_bf16(4, K, seed=9)
    xb[2] = 0
    for use_gemm in (False, True):
        check_product(xb, w, use_gemm=use_gemm)


def test_empty_batch_is_noop():
    packed, beta = gpu_pack(workloads.gen_weights(16, 256, seed=1))
    x_q = torch.empty((0, 256), dtype=torch.int8, device=DEV)
    x_ds = torch.empty((0,), dtype=torch.float32, device=DEV)
    y = torch.empty((0, 16), dtype=torch.float32, device=DEV)
    bl.bitlinear_gemv(x_q, x_ds, 256, packed, beta, 16, y)
    bl.bitlinear_gemm(x_q, x_ds, 256, packed, beta, 16, y)
    torch.cuda.synchronize()


def test_runs_on_a_side_stream():
    M, N, K = 8, 256, 1024
    w = workloads.gen_weights(N, K, seed=12)
    xb = workloads.gen_acts_bf16(M, K, seed=13)
    ref = oracle.bitlinear_forward(xb, w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        packed, beta = gpu_pack(w)
        y = bl.linear(to_dev_bf16(xb), packed, beta, N, torch.int32)
    s.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), ref["acc"])


@pytest.mark.parametrize("M", [2, 8, 100])
def test_stream_argument_keeps_temporaries_alive(M):
    """Conveniences given a stream other than the current one enqueue there,
    while their outputs and temporaries come from the current stream's pool:
    these are recorded on the given stream, so memory freed on return (the
    pack workspace) or reused by the current stream right after is not handed
    out while that stream still works on it."""
    N, K = 512, 2048
    w = workloads.gen_weights(N, K, seed=14 + M)
    xb = workloads.gen_acts_bf16(M, K, seed=15 + M)
    ref = oracle.bitlinear_forward(xb, w)
    s = torch.cuda.Stream()
    wd, xd = torch.from_numpy(w).to(DEV), to_dev_bf16(xb)
    s.wait_stream(torch.cuda.current_stream())
    packed, beta = bl.pack_weights(wd, stream=s)
    # the current stream allocates and writes while s may still be packing
    junk = [torch.full((1 << 20,), 7, dtype=torch.int32, device=DEV) for _ in range(8)]
    y = bl.linear(xd, packed, beta, N, torch.int32, stream=s)
    junk += [torch.full((1 << 20,), 9, dtype=torch.int32, device=DEV) for _ in range(8)]
    s.synchronize()
    torch.cuda.synchronize()
    assert beta.cpu().numpy()[0] == ref["beta"]
    np.testing.assert_array_equal(y.cpu().numpy(), ref["acc"])
