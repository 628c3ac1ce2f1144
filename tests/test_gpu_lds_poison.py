"""LDS race self-test: the library built with -DBL_LDS_POISON.

In that build every kernel that stages data in LDS fills it with a poison
pattern before first use, and the prefill GEMM poisons each staging buffer
again after the barrier that ends its k-step (csrc/bl_internal.h,
lds_poison).  A read of LDS that no thread of the workgroup wrote in this
launch and stage (a missing barrier, an offset past the staged bytes) then
sees the pattern instead of bytes left behind by an earlier launch of the same
call, which would often be the right ones.  Each case runs first on the
regular library (its int32 accumulators checked against the oracle), then on
the poisoned one, which must give the same bits.  Both libraries are built
in-tree by bitlinear_matmul_02_amd.build; the poisoned one is loaded only here.
"""
import os

import numpy as np
import pytest
import torch

import bitlinear_matmul_02_amd as bl
from bitlinear_matmul_02_amd import build as bl_build
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _bf16(xb: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).to(DEV)


def _host(*ts):
    torch.cuda.synchronize()
    return [t.cpu().numpy() if t.dtype != torch.bfloat16 else t.view(torch.int16).cpu().numpy() for t in ts]


def _weights(N, K, seed):
    w = workloads.gen_weights(N, K, seed=seed)
    packed, beta = bl.pack_weights(torch.from_numpy(w).to(DEV))
    return w, packed, beta


def _product(kind, M, K, N, seed):
    """int32 accumulators and fp32 outputs of one BitLinear; `kind` picks the
    entry point (and with it the kernel and plan)."""
    w, packed, beta = _weights(N, K, seed)
    xb = workloads.gen_acts_bf16(M, K, seed=seed + 1, outliers=True)
    x = _bf16(xb)
    outs = []
    for dt in (torch.int32, torch.float32):
        y = torch.empty((M, N), dtype=dt, device=DEV)
        if kind == "fused":
            bl.bitlinear_forward_decode(x, packed, beta, N, y)
        else:
            x_q, x_ds = bl.quant_act(x)
            fn = bl.bitlinear_gemm if kind == "gemm" else bl.bitlinear_gemv
            need = (bl.gemm_workspace_bytes if kind == "gemm" else bl.gemv_workspace_bytes)(M, N, K)
            fn(x_q, x_ds, K, packed, beta, N, y, bl.workspace(need, DEV))
        outs.append(y)
    return _host(*outs), (xb, w)


def _quant(M, K, src, rmsnorm):
    xb = workloads.gen_acts_bf16(M, K, seed=77 + M, outliers=True)
    x = _bf16(xb) if src == "bf16" else torch.from_numpy(workloads.bf16_bits_to_f32(xb)).to(DEV)
    x_q = torch.empty((M, bl.act_stride(K)), dtype=torch.int8, device=DEV)
    x_ds = torch.empty(M, dtype=torch.float32, device=DEV)
    x_rs = torch.empty(M, dtype=torch.int32, device=DEV)
    bl.bitlinear_quant_act(x, x_q, x_ds, x_rs, rmsnorm=rmsnorm)
    return _host(x_q, x_ds, x_rs)


def _fused_multi(M, K, Ns, rmsnorm):
    xb = workloads.gen_acts_bf16(M, K, seed=91, outliers=True)
    mats = [_weights(n, K, 500 + i) for i, n in enumerate(Ns)]
    ys = [torch.empty((M, n), dtype=torch.float32, device=DEV) for n in Ns]
    bl.bitlinear_forward_decode_multi(_bf16(xb), [m[1] for m in mats], [m[2] for m in mats], list(Ns), ys,
                                      rmsnorm=rmsnorm)
    return _host(*ys)


def _fused_glu(M, K, N):
    xb = workloads.gen_acts_bf16(M, K, seed=93, outliers=True)
    _, pg, bg = _weights(N, K, 601)
    _, pu, bu = _weights(N, K, 602)
    h = torch.empty((M, N), dtype=torch.float32, device=DEV)
    bl.bitlinear_forward_decode_glu(_bf16(xb), pg, bg, pu, bu, N, h)
    return _host(h)


def _formats(kind, M, K, N):
    w = workloads.gen_weights(N, K, seed=700 + N)
    xb = workloads.gen_acts_bf16(M, K, seed=701, outliers=True)
    x_q = torch.empty((M, bl.act_stride(K)), dtype=torch.int8, device=DEV)
    x_ds = torch.empty(M, dtype=torch.float32, device=DEV)
    x_rs = torch.empty(M, dtype=torch.int32, device=DEV)
    bl.bitlinear_quant_act(_bf16(xb), x_q, x_ds, x_rs)
    wt = torch.from_numpy(w).to(DEV)
    y = torch.empty((M, N), dtype=torch.int32, device=DEV)
    if kind in ("gemm_b1", "gemv_b1"):
        packed, beta = bl.pack_weights_b1(wt)
        fn = bl.bitlinear_gemm_b1 if kind == "gemm_b1" else bl.bitlinear_gemv_b1
    else:
        packed, beta = bl.pack_weights_b3(wt)
        fn = bl.bitlinear_gemv_b3
    fn(x_q, x_ds, x_rs, K, packed, beta, N, y)
    return _host(y)


def _train(mode, M, K, N):
    _, packed, beta = _weights(N, K, 800)
    x = _bf16(workloads.gen_acts_bf16(M, K, seed=801))
    dy = _bf16(workloads.gen_acts_bf16(M, N, seed=802))
    if mode == "forward":
        y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        bl.bitlinear_train_forward(x, packed, beta, N, y)
        return _host(y)
    if mode == "backward_input":
        dx = torch.empty((M, K), dtype=torch.float32, device=DEV)
        bl.bitlinear_train_backward_input(dy, packed, beta, K, dx)
        return _host(dx)
    dw = torch.empty((N, K), dtype=torch.float32, device=DEV)
    bl.bitlinear_train_backward_weight(dy, x, dw)
    return _host(dw)


# (name, products checked against the oracle, runner)
CASES = [
    # prefill GEMM: 128x256 blocks (384 of them), 128x128, 32x256 and 64x128
    # with k split over workgroups; ragged K
    ("gemm_128x256", True, lambda: _product("gemm", 2048, 520, 6144, 11)),
    ("gemm_128x128", True, lambda: _product("gemm", 300, 1000, 600, 12)),
    ("gemm_32x256_split", True, lambda: _product("gemm", 20, 8192, 1024, 13)),
    ("gemm_64x128_split", True, lambda: _product("gemm", 50, 4096, 2048, 14)),
    # decode GEMV: int8 rows staged in LDS, read from global memory, a wide
    # plan (one workgroup per CU), fused quantization (plain and wide)
    ("gemv_rows_in_lds", True, lambda: _product("gemv", 3, 2560, 6912, 21)),
    ("gemv_rows_global", True, lambda: _product("gemv", 8, 8192, 1040, 22)),
    ("gemv_wide", True, lambda: _product("gemv", 8, 4096, 16384, 23)),
    ("fused_decode", True, lambda: _product("fused", 2, 2560, 2560, 24)),
    ("fused_decode_wide", True, lambda: _product("fused", 1, 8192, 16400, 25)),
    ("fused_multi_rmsnorm", False, lambda: _fused_multi(1, 2560, (2560, 640, 640), True)),
    ("fused_glu", False, lambda: _fused_glu(3, 2560, 6912)),
    ("quant_act_bf16", False, lambda: _quant(5, 3000, "bf16", False)),
    ("quant_act_f32_rmsnorm", False, lambda: _quant(3, 8192, "f32", True)),
    ("gemm_b1", False, lambda: _formats("gemm_b1", 130, 1100, 700)),
    ("gemv_b1", False, lambda: _formats("gemv_b1", 4, 1100, 700)),
    ("gemv_b3", False, lambda: _formats("gemv_b3", 3, 2000, 500)),
    ("train_forward", False, lambda: _train("forward", 300, 640, 384)),
    ("train_backward_input", False, lambda: _train("backward_input", 300, 640, 384)),
    ("train_backward_weight", False, lambda: _train("backward_weight", 300, 640, 384)),
]


@pytest.fixture
def poisoned_library(monkeypatch):
    """Switch the binding to the poisoned build for the rest of the test."""
    assert os.path.exists(bl_build.POISON_LIB), "%s is not built" % bl_build.POISON_LIB

    def use():
        monkeypatch.setattr(bl, "LIB_PATH", bl_build.POISON_LIB)
        monkeypatch.setattr(bl, "_lib", None)
        return bl.lib()
    return use


@pytest.mark.parametrize("name,vs_oracle,run", CASES, ids=[c[0] for c in CASES])
def test_poisoned_lds_gives_the_same_bits(name, vs_oracle, run, poisoned_library):
    ref = run()
    if vs_oracle:  # the regular library's accumulators against the oracle
        (acc, _), (xb, w) = ref
        np.testing.assert_array_equal(acc, oracle.bitlinear_forward(xb, w, threads=16)["acc"])
        ref = ref[0]
    lib = poisoned_library()
    assert os.path.basename(lib._name) == os.path.basename(bl_build.POISON_LIB)
    got = run()
    if vs_oracle:
        got = got[0]
    assert len(got) == len(ref)
    for g, r in zip(got, ref):
        np.testing.assert_array_equal(g, r)
