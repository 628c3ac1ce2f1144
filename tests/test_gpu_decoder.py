"""Parity of the decoder glue and of the decode step over a BitLinear stack.

The glue (ReLU^2 gated product, residual sums fused into the product
epilogues) uses the same IEEE operations in the same order on both sides, so
every result is compared bit for bit; the fp32 tolerance of 1e-3 relative is
asserted first.
"""
import numpy as np
import pytest
import torch

import bitlinear_matmul_02_amd as bl
from bitlinear_matmul_02_amd import decoder
from bitlinear_matmul_02_amd.decoder import NAMES, DecoderStack, PackedLinear
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
RTOL_F32 = 1e-3


def assert_f32_parity(got, ref):
    got = np.asarray(got, dtype=np.float32)
    ref = np.asarray(ref, dtype=np.float32)
    zero = ref == 0
    assert not np.any(got[zero] != 0)
    assert np.all(np.abs(got[~zero].astype(np.float64) - ref[~zero]) <= RTOL_F32 * np.abs(ref[~zero].astype(np.float64)))
    np.testing.assert_array_equal(got, ref)


# ------------------------------------------------------------- relu2_mul
@pytest.mark.parametrize("count,offset", [(1, 0), (3, 0), (4, 0), (5, 1), (1000, 0), (6912, 0), (8 * 6912 + 3, 0),
                                          (4099, 3), (1 << 20, 0)])
def test_relu2_mul_parity(count, offset):
    rng = np.random.default_rng(count + offset)
    g = rng.standard_normal(count + offset).astype(np.float32) * 2
    u = rng.standard_normal(count + offset).astype(np.float32)
    g[offset::7] = 0.0
    gd, ud = torch.from_numpy(g).to(DEV), torch.from_numpy(u).to(DEV)
    h = torch.full((count + offset,), 7.0, dtype=torch.float32, device=DEV)
    bl.bitlinear_relu2_mul(gd[offset:], ud[offset:], h[offset:])
    torch.cuda.synchronize()
    out = h.cpu().numpy()
    assert np.all(out[:offset] == 7.0)  # nothing written before the range
    assert_f32_parity(out[offset:], oracle.relu2_mul(g[offset:], u[offset:]))


def test_relu2_mul_in_place():
    rng = np.random.default_rng(5)
    g = rng.standard_normal(6912).astype(np.float32)
    u = rng.standard_normal(6912).astype(np.float32)
    gd, ud = torch.from_numpy(g).to(DEV), torch.from_numpy(u).to(DEV)
    bl.bitlinear_relu2_mul(gd, ud, gd)  # h aliases g
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gd.cpu().numpy(), oracle.relu2_mul(g, u))


# ------------------------------------------------ RMS normalization fused into quantization
def norm_inputs(M, K, src, seed):
    xb = workloads.gen_acts_bf16(M, K, seed=seed)
    xf = workloads.bf16_bits_to_f32(xb)
    if src == "f32":
        xf = xf * np.float32(1.37) + np.float32(0.01)  # values beyond bf16 precision
        x = torch.from_numpy(xf).to(DEV)
    else:
        x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).to(DEV)
    if M > 1:
        xf[M // 2] = 0.0
        x[M // 2] = 0
    return x, xf


@pytest.mark.parametrize("M,K", [(1, 2560), (8, 6912), (3, 13), (2, 512), (33, 28672), (4, 100), (5, 4096)])
@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_quant_act_rmsnorm_parity(M, K, src):
    x, xf = norm_inputs(M, K, src, seed=M * 13 + K)
    q_ref, ds_ref, rs_ref = oracle.quant_act(oracle.rmsnorm(xf))
    x_q, x_ds, rs = bl.quant_act(x, with_rowsum=True, rmsnorm=True)
    torch.cuda.synchronize()
    q = x_q.cpu().numpy()
    np.testing.assert_array_equal(q[:, :K], q_ref)
    assert not q[:, K:].any()
    np.testing.assert_array_equal(x_ds.cpu().numpy(), ds_ref)
    np.testing.assert_array_equal(rs.cpu().numpy(), rs_ref)


# (1, 8192, 28672), (3, 1000, 20000) and (2, 1001, 17000) take wide plans (one
# workgroup per compute unit, interleaved k-tiles); the last with rows that
# are not whole 16-byte pieces.
@pytest.mark.parametrize("M,K,N", [(1, 2560, 2560), (1, 6912, 640), (3, 13, 40), (4, 100, 33), (8, 2560, 512),
                                   (2, 6912, 2560), (1, 8192, 28672), (3, 1000, 20000), (2, 1001, 17000)])
@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_forward_decode_rmsnorm_parity(M, K, N, src):
    if not bl.decode_fits(M, K):
        pytest.skip("rows do not fit the fused kernel's LDS")
    x, xf = norm_inputs(M, K, src, seed=M * 17 + K + N)
    w = workloads.gen_weights(N, K, seed=N + 7)
    beta = oracle.absmean(w)
    q, ds, _ = oracle.quant_act(oracle.rmsnorm(xf))
    acc_ref = oracle.matmul_i32(q, oracle.ternarize(w, beta), threads=8)
    packed, wb = bl.pack_weights(torch.from_numpy(w).to(DEV))
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    bl.bitlinear_forward_decode(x, packed, wb, N, acc, rmsnorm=True)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    bl.bitlinear_forward_decode(x, packed, wb, N, y, rmsnorm=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)
    assert_f32_parity(y.cpu().numpy(), oracle.dequant(acc_ref, ds, beta))


# ------------------------------------------------ several BitLinears / gated pair in one launch
def oracle_acc_y(xf, w, norm):
    beta = oracle.absmean(w)
    q, ds, _ = oracle.quant_act(oracle.rmsnorm(xf) if norm else xf)
    acc = oracle.matmul_i32(q, oracle.ternarize(w, beta), threads=8)
    return acc, oracle.dequant(acc, ds, beta)


MULTI_CASES = [(1, 2560, (2560, 640, 640)), (3, 700, (40, 333)), (8, 2560, (2560, 640, 640, 16)),
               (33, 512, (300, 17, 1000)), (64, 256, (64,)), (1, 6912, (2560,)), (5, 13, (7, 40))]


@pytest.mark.parametrize("M,K,Ns", MULTI_CASES)
@pytest.mark.parametrize("path", ["gemv", "fused"])
def test_multi_parity(M, K, Ns, path):
    norm = path == "fused" and K >= 256
    if path == "fused" and not bl.decode_fits(M, K):
        pytest.skip("rows do not fit the fused kernel's LDS")
    x, xf = norm_inputs(M, K, "f32", seed=M * 5 + K)
    ws = [workloads.gen_weights(N, K, seed=N * 3 + i) for i, N in enumerate(Ns)]
    packs = [bl.pack_weights(torch.from_numpy(w).to(DEV)) for w in ws]
    for dtype in (torch.int32, torch.float32):
        ys = [torch.full((M, N), 3.0, dtype=dtype, device=DEV) for N in Ns]
        if path == "fused":
            bl.bitlinear_forward_decode_multi(x, [p for p, _ in packs], [b for _, b in packs], Ns, ys, rmsnorm=norm)
        else:
            x_q, x_ds = bl.quant_act(x)
            bl.bitlinear_gemv_multi(x_q, x_ds, K, [p for p, _ in packs], [b for _, b in packs], Ns, ys)
        torch.cuda.synchronize()
        for w, y in zip(ws, ys):
            acc, yr = oracle_acc_y(xf, w, norm)
            if dtype == torch.int32:
                np.testing.assert_array_equal(y.cpu().numpy(), acc)
            else:
                assert_f32_parity(y.cpu().numpy(), yr)


def test_multi_accumulate():
    M, K, Ns = 2, 2560, (2560, 640)
    x, xf = norm_inputs(M, K, "f32", seed=9)
    ws = [workloads.gen_weights(N, K, seed=N + 1) for N in Ns]
    packs = [bl.pack_weights(torch.from_numpy(w).to(DEV)) for w in ws]
    rng = np.random.default_rng(3)
    y0 = [rng.standard_normal((M, N)).astype(np.float32) for N in Ns]
    ys = [torch.from_numpy(v).to(DEV) for v in y0]
    bl.bitlinear_forward_decode_multi(x, [p for p, _ in packs], [b for _, b in packs], Ns, ys, accumulate=True)
    torch.cuda.synchronize()
    for w, v, y in zip(ws, y0, ys):
        assert_f32_parity(y.cpu().numpy(), oracle.add_f32(v, oracle_acc_y(xf, w, False)[1]))


@pytest.mark.parametrize("M,K,N", [(1, 2560, 6912), (3, 700, 333), (8, 2560, 6912), (33, 512, 100), (64, 256, 48),
                                   (2, 13, 20)])
@pytest.mark.parametrize("path", ["gemv", "fused"])
def test_glu_parity(M, K, N, path):
    norm = path == "fused"
    if path == "fused" and not bl.decode_fits(M, K):
        pytest.skip("rows do not fit the fused kernel's LDS")
    x, xf = norm_inputs(M, K, "f32", seed=M + K + N)
    wg = workloads.gen_weights(N, K, seed=N + 11)
    wu = workloads.gen_weights(N, K, seed=N + 12)
    (pg, bg), (pu, bu) = (bl.pack_weights(torch.from_numpy(w).to(DEV)) for w in (wg, wu))
    h = torch.full((M, N), 5.0, dtype=torch.float32, device=DEV)
    if path == "fused":
        bl.bitlinear_forward_decode_glu(x, pg, bg, pu, bu, N, h, rmsnorm=norm)
    else:
        x_q, x_ds = bl.quant_act(x)
        bl.bitlinear_gemv_glu(x_q, x_ds, K, pg, bg, pu, bu, N, h)
    torch.cuda.synchronize()
    ref = oracle.relu2_mul(oracle_acc_y(xf, wg, norm)[1], oracle_acc_y(xf, wu, norm)[1])
    assert_f32_parity(h.cpu().numpy(), ref)


# ------------------------------------------------ requantization in the producer's epilogue
RQ_CASES = [(1, 2560, (2560, 640, 640)), (8, 2560, (2560, 640, 640)), (8, 6912, (2560,)), (8, 2560, (2560,)),
            (3, 700, (333, 40)), (33, 512, (300, 17)), (64, 256, (64,)), (12, 8192, (1000,)), (2, 13, (21,))]


@pytest.mark.parametrize("M,K,Ns", RQ_CASES)
@pytest.mark.parametrize("norm,accumulate", [(False, False), (True, True), (True, False)])
def test_decode_rq_parity(M, K, Ns, norm, accumulate):
    """Products of 1-3 BitLinears on int8 inputs, then the last workgroup
    quantizes output 0 (RMS-normalized when norm) for the next BitLinear: the
    outputs, the next int8 rows and scales equal the oracle's, and the arrival
    counter is zero again."""
    x, xf = norm_inputs(M, K, "f32", seed=M * 7 + K)
    ws = [workloads.gen_weights(N, K, seed=N * 5 + i) for i, N in enumerate(Ns)]
    packs = [bl.pack_weights(torch.from_numpy(w).to(DEV)) for w in ws]
    rng = np.random.default_rng(M + K)
    y0 = [rng.standard_normal((M, N)).astype(np.float32) for N in Ns]
    ys = [torch.from_numpy(v).to(DEV) for v in y0]
    x_q, x_ds = bl.quant_act(x)
    nq = torch.full((M, bl.act_stride(Ns[0])), 7, dtype=torch.int8, device=DEV)
    nds = torch.zeros((M,), dtype=torch.float32, device=DEV)
    cnt = torch.zeros((64,), dtype=torch.uint8, device=DEV)
    for rep in range(2):  # the counter is reused: it must come back zero
        if rep:
            for y, v in zip(ys, y0):
                y.copy_(torch.from_numpy(v))
        bl.bitlinear_decode_rq(x_q, x_ds, K, [p for p, _ in packs], [b for _, b in packs], list(Ns), ys, nq, nds, cnt,
                               accumulate=accumulate, next_rmsnorm=norm)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(cnt)) == 0
        outs = []
        for w, v, y in zip(ws, y0, ys):
            yr = oracle_acc_y(xf, w, False)[1]
            if accumulate:
                yr = oracle.add_f32(v, yr)
            assert_f32_parity(y.cpu().numpy(), yr)
            outs.append(yr)
        q_ref, ds_ref, _ = oracle.quant_act(oracle.rmsnorm(outs[0]) if norm else outs[0])
        got = nq.cpu().numpy()
        np.testing.assert_array_equal(got[:, :Ns[0]], q_ref)
        assert not got[:, Ns[0]:].any(), "padding columns must be zero"
        np.testing.assert_array_equal(nds.cpu().numpy(), ds_ref)


@pytest.mark.parametrize("M,K,N", [(1, 2560, 6912), (8, 2560, 6912), (3, 700, 333), (64, 256, 48)])
def test_decode_rq_glu_parity(M, K, N):
    x, xf = norm_inputs(M, K, "f32", seed=M + 2 * K + N)
    wg = workloads.gen_weights(N, K, seed=N + 21)
    wu = workloads.gen_weights(N, K, seed=N + 22)
    (pg, bg), (pu, bu) = (bl.pack_weights(torch.from_numpy(w).to(DEV)) for w in (wg, wu))
    h = torch.full((M, N), 5.0, dtype=torch.float32, device=DEV)
    x_q, x_ds = bl.quant_act(x)
    nq = torch.full((M, bl.act_stride(N)), 7, dtype=torch.int8, device=DEV)
    nds = torch.zeros((M,), dtype=torch.float32, device=DEV)
    cnt = torch.zeros((64,), dtype=torch.uint8, device=DEV)
    bl.bitlinear_decode_rq(x_q, x_ds, K, [pg, pu], [bg, bu], N, [h], nq, nds, cnt, glu=True)
    torch.cuda.synchronize()
    ref = oracle.relu2_mul(oracle_acc_y(xf, wg, False)[1], oracle_acc_y(xf, wu, False)[1])
    assert_f32_parity(h.cpu().numpy(), ref)
    q_ref, ds_ref, _ = oracle.quant_act(ref)
    np.testing.assert_array_equal(nq.cpu().numpy()[:, :N], q_ref)
    np.testing.assert_array_equal(nds.cpu().numpy(), ds_ref)
    assert int(torch.count_nonzero(cnt)) == 0


# ------------------------------------------------ residual sum in the epilogue
def oracle_linear_f32(x, w):
    beta = oracle.absmean(w)
    t = oracle.ternarize(w, beta)
    q, ds, _ = oracle.quant_act(x)
    return oracle.dequant(oracle.matmul_i32(q, t, threads=8), ds, beta)


@pytest.mark.parametrize("path", ["gemv", "gemm", "fused"])
# (2, 1000, 20000) takes a wide plan (1250 output blocks, one workgroup per
# compute unit), whose epilogue dispatches the output type once; (20, 2000,
# 20000) on the product takes 32 x 128 blocks with k split inside the workgroup
@pytest.mark.parametrize("M,K,N", [(1, 2560, 2560), (3, 700, 333), (8, 6912, 2560), (130, 512, 300),
                                   (2, 1000, 20000), (20, 2000, 20000)])
def test_accumulate_output(path, M, K, N):
    if path != "gemm" and M > bl.GEMV_MAX_M:
        pytest.skip("decode paths take at most 64 tokens")
    if path == "fused" and not bl.decode_fits(M, K):
        pytest.skip("rows do not fit the fused kernel's LDS")
    rng = np.random.default_rng(M * 31 + K)
    w = workloads.gen_weights(N, K, seed=K + N)
    x = workloads.bf16_bits_to_f32(workloads.gen_acts_bf16(M, K, seed=M + 3)) * np.float32(0.75)
    y0 = rng.standard_normal((M, N)).astype(np.float32) * 10
    ref = oracle.add_f32(y0, oracle_linear_f32(x, w))
    packed, beta = bl.pack_weights(torch.from_numpy(w).to(DEV))
    xd = torch.from_numpy(x).to(DEV)
    y = torch.from_numpy(y0).to(DEV)
    if path == "fused":
        bl.bitlinear_forward_decode(xd, packed, beta, N, y, accumulate=True)
    else:
        x_q, x_ds = bl.quant_act(xd)
        fn = bl.bitlinear_gemv if path == "gemv" else bl.bitlinear_gemm
        ws = bl.workspace((bl.gemv_workspace_bytes if path == "gemv" else bl.gemm_workspace_bytes)(M, N, K), DEV)
        fn(x_q, x_ds, K, packed, beta, N, y, ws, accumulate=True)
    torch.cuda.synchronize()
    assert_f32_parity(y.cpu().numpy(), ref)


def test_accumulate_needs_fp32_output():
    y = torch.zeros((1, 16), dtype=torch.bfloat16, device=DEV)
    x = torch.zeros((1, 256), dtype=torch.float32, device=DEV)
    packed, beta = bl.pack_weights(torch.zeros((16, 256), device=DEV))
    with pytest.raises(bl.BitLinearError):
        bl.bitlinear_forward_decode(x, packed, beta, 16, y, accumulate=True)


# ------------------------------------------------------------- decode step
def stack_inputs(n_layers):
    lat = []
    for l in range(n_layers):
        lat.append({name: workloads.gen_weights(N, K, seed=workloads.decoder_weight_seed(l, j))
                    for j, (name, K, N) in enumerate(workloads.LAYER_SHAPES)})
    return lat


def gpu_stack(lat, M, requant=False):
    layers = []
    for L in lat:
        d = {}
        for name, w in L.items():
            packed, beta = bl.pack_weights(torch.from_numpy(w).to(DEV))
            d[name] = PackedLinear(packed, beta, w.shape[0], w.shape[1])
        layers.append(d)
    return DecoderStack(layers, M, DEV, requant=requant)


def oracle_layer(x, L, cache):
    """One decoder layer on the oracle; cache holds (beta, t) per matrix."""
    def lin(inp, name):
        if name not in cache:
            beta = oracle.absmean(L[name])
            cache[name] = (beta, oracle.ternarize(L[name], beta))
        beta, t = cache[name]
        q, ds, _ = oracle.quant_act(inp)
        return oracle.dequant(oracle.matmul_i32(q, t, threads=8), ds, beta)
    xn = oracle.rmsnorm(x)
    q, k, v = lin(xn, "q"), lin(xn, "k"), lin(xn, "v")
    x = oracle.add_f32(x, lin(q, "o"))
    xn = oracle.rmsnorm(x)
    h = oracle.relu2_mul(lin(xn, "gate"), lin(xn, "up"))
    x = oracle.add_f32(x, lin(h, "down"))
    return x, {"q": q, "k": k, "v": v, "h": h}


@pytest.fixture(scope="module")
def two_layers():
    return stack_inputs(2)


@pytest.fixture(scope="module")
def four_layers():
    return stack_inputs(4)


@pytest.mark.parametrize("M", list(workloads.DECODE_STEP_BATCHES) + [2, 3, 64, 80])
def test_decode_step_layers_match_oracle(four_layers, M):
    x0 = workloads.bf16_bits_to_f32(workloads.gen_acts_bf16(M, workloads.D_MODEL, seed=workloads.DECODER_X0_SEED))
    stack = gpu_stack(four_layers, M)
    assert stack.fused == (M <= decoder.FUSED_MAX_M)
    x = torch.from_numpy(x0).to(DEV)
    xr = x0
    for l, L in enumerate(four_layers):
        stack.layer(l, x)
        torch.cuda.synchronize()
        xr, parts = oracle_layer(xr, L, {})
        assert_f32_parity(x.cpu().numpy(), xr)
        for name in ("q", "k", "v", "h"):
            assert_f32_parity(getattr(stack, name).cpu().numpy(), parts[name])


@pytest.mark.parametrize("M", [8, 33])
def test_decode_step_requant_matches_oracle(two_layers, M):
    """The decode step with the next input quantized in each product's
    epilogue (bitlinear_decode_rq) equals the oracle's chain over two layers."""
    x0 = workloads.bf16_bits_to_f32(workloads.gen_acts_bf16(M, workloads.D_MODEL, seed=workloads.DECODER_X0_SEED))
    stack = gpu_stack(two_layers, M, requant=True)
    assert stack.requant
    x = torch.from_numpy(x0).to(DEV)
    stack.step(x)
    torch.cuda.synchronize()
    xr = x0
    for L in two_layers:
        xr, _ = oracle_layer(xr, L, {})
    assert_f32_parity(x.cpu().numpy(), xr)
    assert int(torch.count_nonzero(stack.rq_ws)) == 0


@pytest.mark.parametrize("M", [1, 8])
def test_decode_step_graph_replays(two_layers, M):
    x0 = workloads.bf16_bits_to_f32(workloads.gen_acts_bf16(M, workloads.D_MODEL, seed=workloads.DECODER_X0_SEED))
    stack = gpu_stack(two_layers, M)
    x = torch.from_numpy(x0).to(DEV)
    stack.step(x)
    torch.cuda.synchronize()
    eager = x.cpu().numpy().copy()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        x.copy_(torch.from_numpy(x0).to(DEV))
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            stack.step(x)
    torch.cuda.synchronize()
    for _ in range(3):
        x.copy_(torch.from_numpy(x0).to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(x.cpu().numpy(), eager)
        stack.layer(0, torch.zeros_like(x))  # eager work between replays
        torch.cuda.synchronize()
