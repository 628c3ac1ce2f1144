"""bitlinear_gemv_noalloc: the decode product for callers that cannot allocate.

Called through the C ABI with no workspace (its split-k partial sums live in
the library's device-resident scratch array) and compared bit for bit with
bitlinear_gemv given a workspace, on consecutive calls: a shape whose k-range
is split across workgroups through the 8 MiB array (32 tokens, 28672 -> 8192,
the small-batch matrix-core path), then a smaller one split through the
decode kernel's own partial sums (1 token, K = 131072, 100 outputs), then one
that needs no scratch, then the first shape again.  Both entry points are
also checked against the oracle's int32 accumulators.
"""
import numpy as np
import pytest
import torch

import bitlinear_matmul_02_amd as bl
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

SHAPES = [(32, 28672, 8192), (1, 131072, 100), (1, 6912, 2560), (32, 28672, 8192)]  # (M, K, N)


def _case(M, K, N, seed):
    w = workloads.gen_weights(N, K, seed=seed)
    xb = workloads.gen_acts_bf16(M, K, seed=seed + 1)
    packed, beta = bl.pack_weights(torch.from_numpy(w).to(DEV))
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(DEV)
    x_q, x_ds = bl.quant_act(x)
    b = oracle.absmean(w)
    q, _, _ = oracle.quant_act(xb, bf16_bits=True)
    acc_ref = oracle.matmul_i32(q, oracle.ternarize(w, b), threads=16)
    return x_q, x_ds, packed, beta, acc_ref


def test_noalloc_matches_gemv_on_consecutive_calls():
    assert max(bl.gemv_workspace_bytes(M, N, K) for M, K, N in SHAPES) <= bl.NOALLOC_SCRATCH_BYTES
    assert bl.gemv_workspace_bytes(32, 8192, 28672) > 4 << 20  # the first shape uses most of the array
    assert bl.gemv_workspace_bytes(1, 100, 131072) > 0
    assert bl.gemv_workspace_bytes(1, 2560, 6912) == 0
    for i, (M, K, N) in enumerate(SHAPES):
        x_q, x_ds, packed, beta, acc_ref = _case(M, K, N, seed=21000 + 10 * (i % 3))
        ws = bl.workspace(bl.gemv_workspace_bytes(M, N, K), DEV)
        for dtype in (torch.int32, torch.float32):
            y_ref = torch.empty((M, N), dtype=dtype, device=DEV)
            y = torch.full((M, N), 7, dtype=dtype, device=DEV)
            bl.bitlinear_gemv(x_q, x_ds, K, packed, beta, N, y_ref, ws)
            bl.bitlinear_gemv_noalloc(x_q, x_ds, K, packed, beta, N, y)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(y.cpu().numpy(), y_ref.cpu().numpy())
            if dtype == torch.int32:
                np.testing.assert_array_equal(y.cpu().numpy(), acc_ref)
        # the residual-sum output mode through the scratch array as well
        base = torch.from_numpy(np.linspace(-1, 1, M * N, dtype=np.float32).reshape(M, N)).to(DEV)
        y_ref, y = base.clone(), base.clone()
        bl.bitlinear_gemv(x_q, x_ds, K, packed, beta, N, y_ref, ws, accumulate=True)
        bl.bitlinear_gemv_noalloc(x_q, x_ds, K, packed, beta, N, y, accumulate=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy(), y_ref.cpu().numpy())
        del x_q, x_ds, packed, beta


def test_noalloc_on_a_side_stream_and_empty_batch():
    M, K, N = 8, 28672, 8192
    x_q, x_ds, packed, beta, acc_ref = _case(M, K, N, seed=21100)
    s = torch.cuda.Stream()
    y = torch.empty((M, N), dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        bl.bitlinear_gemv_noalloc(x_q, x_ds, K, packed, beta, N, y, stream=s)
    s.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), acc_ref)
    empty = torch.empty((0, N), dtype=torch.float32, device=DEV)
    bl.bitlinear_gemv_noalloc(x_q[:0], x_ds[:0], K, packed, beta, N, empty)
