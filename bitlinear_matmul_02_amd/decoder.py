"""Decode step over a stack of BitLinear decoder layers.

Each layer holds seven BitLinears (q, k, v, o, gate, up, down) and the glue
between them ("Key Technologies Enabling the BitNET Family", Architectural
Innovations and Optimizations: RMSNorm, squared ReLU in the feed-forward
layers, no biases): two RMS normalizations (gain 1), the squared-ReLU gated
feed-forward activation and two residual sums.  Attention itself is not part
of this path: the o projection takes the q projection's output in its place,
and k / v are computed and kept (as a KV cache would receive them).  Per
layer, with x the fp32 residual stream [M][d] and N(.) the RMS normalization:

    q, k, v = BL_q(N(x)), BL_k(N(x)), BL_v(N(x))
    x = x + BL_o(q)
    h = ReLU(BL_gate(N(x)))^2 * BL_up(N(x))
    x = x + BL_down(h)

The normalization is fused into the BitLinears' activation quantization
(``rmsnorm``), so N(x) is never written out.

Everything is enqueued on one stream by the library's kernels and allocates
nothing after construction, so a step can be captured in a HIP graph.  Up to
64 tokens a layer is four products: q/k/v in one multi launch, o with the
residual sum fused into its epilogue (``accumulate``), gate/up as one gated
launch that writes h directly, and down, again accumulating into x.  For at
most ``FUSED_MAX_M`` tokens the activation quantization (and normalization)
runs inside each product's prologue, so a layer is four launches; beyond that
each input is quantized once by its own launch.  Past 64 tokens the products
run on the matrix-core GEMM, one BitLinear per launch.

With ``requant=True`` (up to 64 tokens, past the fused limit) each product's
last workgroup instead quantizes the next product's input
(bitlinear_decode_rq: q for o, RMSNorm(x) for gate/up and for the next
layer's q/k/v, h for down), so a layer is four launches and a step adds one
quantizer launch for its input.  The results are the same; on MI355X it is
slower than the separate quantizer at every batch (the last workgroup's
reads of the finished rows run on one compute unit and wait on memory round
trips, while the quantizer spreads the rows over as many workgroups), so it
is not the default.
"""
from __future__ import annotations

import torch

from . import (GEMV_MAX_M, act_stride, bitlinear_decode_rq, bitlinear_forward_decode, bitlinear_forward_decode_glu,
               bitlinear_forward_decode_multi, bitlinear_gemm, bitlinear_gemv, bitlinear_gemv_glu,
               bitlinear_gemv_multi, bitlinear_quant_act, bitlinear_relu2_mul, decode_fits,
               gemm_workspace_bytes, gemv_workspace_bytes)

NAMES = ("q", "k", "v", "o", "gate", "up", "down")
# Measured on MI355X (30-layer 2B-class step, fused against standalone
# quantizer + product): 638 / 854 us at 1 token, 879 / 913 at 2, 974 / 936 at
# 3, 1169 / 976 at 4: beyond 2 tokens every workgroup re-quantizing the rows
# costs more than the launch it saves.
FUSED_MAX_M = 2


class PackedLinear:
    """One packed BitLinear: 2-bit tiles and the fp32 weight scale on the device."""

    def __init__(self, packed: torch.Tensor, beta: torch.Tensor, N: int, K: int):
        self.packed, self.beta, self.N, self.K = packed, beta, N, K


class DecoderStack:
    def __init__(self, layers: list[dict], M: int, device, requant: bool = False):
        """layers: one dict per layer mapping each of NAMES to a PackedLinear;
        requant: quantize each product's output in its epilogue (see above)."""
        self.layers = layers
        self.M = M
        dev = torch.device(device)
        first = layers[0]
        d, qn, kn, vn = first["q"].K, first["q"].N, first["k"].N, first["v"].N
        f = first["gate"].N
        for L in layers:
            assert set(L) == set(NAMES)
            assert (L["o"].K, L["o"].N, L["gate"].K, L["up"].K, L["up"].N, L["down"].K, L["down"].N) == \
                (qn, d, d, d, f, f, d)
        self.d, self.f = d, f
        z = lambda n: torch.zeros((M, n), dtype=torch.float32, device=dev)
        self.q, self.k, self.v, self.g, self.u, self.h = z(qn), z(kn), z(vn), z(f), z(f), z(f)
        self.fused = M <= FUSED_MAX_M and all(decode_fits(M, K) for K in (d, qn, f))
        self.gemv = M <= GEMV_MAX_M
        # requantizing epilogues: batches past the fused limit up to 64 tokens, on request
        self.requant = requant and self.gemv and not self.fused
        if not self.fused:
            self.xq = {K: torch.zeros((M, act_stride(K)), dtype=torch.int8, device=dev) for K in {d, qn, f}}
            self.xds = {K: torch.zeros((M,), dtype=torch.float32, device=dev) for K in {d, qn, f}}
            wsf = gemv_workspace_bytes if self.gemv else gemm_workspace_bytes
            ws = max(wsf(M, L[n].N, L[n].K) for L in layers for n in NAMES)
            self.ws = torch.zeros((max(ws, 1),), dtype=torch.uint8, device=dev)
        if self.requant:
            # the next products' int8 inputs: x (RMS-normalized), q and h
            self.rq_x = (torch.zeros((M, act_stride(d)), dtype=torch.int8, device=dev),
                         torch.zeros((M,), dtype=torch.float32, device=dev))
            self.rq_q = (torch.zeros((M, act_stride(qn)), dtype=torch.int8, device=dev),
                         torch.zeros((M,), dtype=torch.float32, device=dev))
            self.rq_h = (torch.zeros((M, act_stride(f)), dtype=torch.int8, device=dev),
                         torch.zeros((M,), dtype=torch.float32, device=dev))
            self.rq_ws = torch.zeros((256,), dtype=torch.uint8, device=dev)  # arrival counter

    # one BitLinear on an input already quantized into self.xq / self.xds
    def _product(self, lin: PackedLinear, y, accumulate, stream):
        fn = bitlinear_gemv if self.gemv else bitlinear_gemm
        fn(self.xq[lin.K], self.xds[lin.K], lin.K, lin.packed, lin.beta, lin.N, y, self.ws, stream,
           accumulate=accumulate)

    def _linears(self, x, lins, outs, accumulate, stream, rmsnorm=False):
        """outs[i] (+)= BL_i(x) (of N(x) with rmsnorm) for BitLinears sharing the input x."""
        if self.fused:
            for lin, y in zip(lins, outs):
                bitlinear_forward_decode(x, lin.packed, lin.beta, lin.N, y, stream, accumulate=accumulate,
                                         rmsnorm=rmsnorm)
            return
        K = lins[0].K
        bitlinear_quant_act(x, self.xq[K], self.xds[K], None, stream, rmsnorm=rmsnorm)
        for lin, y in zip(lins, outs):
            self._product(lin, y, accumulate, stream)

    def _layer_rq(self, i: int, x: torch.Tensor, stream, last: bool) -> None:
        """Layer i with requantizing epilogues; self.rq_x holds the quantized
        RMSNorm(x) on entry and (unless ``last``) on return."""
        L = self.layers[i]
        qkv = [L[n] for n in ("q", "k", "v")]
        d, ws = self.d, self.rq_ws
        xq, xds = self.rq_x
        bitlinear_decode_rq(xq, xds, d, [l.packed for l in qkv], [l.beta for l in qkv], [l.N for l in qkv],
                            [self.q, self.k, self.v], self.rq_q[0], self.rq_q[1], ws, stream)
        o = L["o"]
        bitlinear_decode_rq(self.rq_q[0], self.rq_q[1], o.K, [o.packed], [o.beta], [o.N], [x], xq, xds, ws, stream,
                            accumulate=True, next_rmsnorm=True)
        g, u = L["gate"], L["up"]
        bitlinear_decode_rq(xq, xds, d, [g.packed, u.packed], [g.beta, u.beta], g.N, [self.h], self.rq_h[0],
                            self.rq_h[1], ws, stream, glu=True)
        dn = L["down"]
        if last:
            bitlinear_gemv(self.rq_h[0], self.rq_h[1], dn.K, dn.packed, dn.beta, dn.N, x, self.ws, stream,
                           accumulate=True)
        else:
            bitlinear_decode_rq(self.rq_h[0], self.rq_h[1], dn.K, [dn.packed], [dn.beta], [dn.N], [x], xq, xds, ws,
                                stream, accumulate=True, next_rmsnorm=True)

    def layer(self, i: int, x: torch.Tensor, stream=None) -> None:
        L = self.layers[i]
        if self.requant:
            bitlinear_quant_act(x, self.rq_x[0], self.rq_x[1], None, stream, rmsnorm=True)
            self._layer_rq(i, x, stream, last=True)
            return
        if not self.gemv:  # prefill-sized batches: one GEMM per BitLinear
            self._linears(x, (L["q"], L["k"], L["v"]), (self.q, self.k, self.v), False, stream, rmsnorm=True)
            self._linears(self.q, (L["o"],), (x,), True, stream)
            self._linears(x, (L["gate"], L["up"]), (self.g, self.u), False, stream, rmsnorm=True)
            bitlinear_relu2_mul(self.g, self.u, self.h, stream)
            self._linears(self.h, (L["down"],), (x,), True, stream)
            return
        qkv = [L[n] for n in ("q", "k", "v")]
        g, u = L["gate"], L["up"]
        if self.fused:
            bitlinear_forward_decode_multi(x, [l.packed for l in qkv], [l.beta for l in qkv], [l.N for l in qkv],
                                           [self.q, self.k, self.v], stream, rmsnorm=True)
            self._linears(self.q, (L["o"],), (x,), True, stream)
            bitlinear_forward_decode_glu(x, g.packed, g.beta, u.packed, u.beta, g.N, self.h, stream, rmsnorm=True)
            self._linears(self.h, (L["down"],), (x,), True, stream)
            return
        d = self.d
        bitlinear_quant_act(x, self.xq[d], self.xds[d], None, stream, rmsnorm=True)
        bitlinear_gemv_multi(self.xq[d], self.xds[d], d, [l.packed for l in qkv], [l.beta for l in qkv],
                             [l.N for l in qkv], [self.q, self.k, self.v], stream)
        self._linears(self.q, (L["o"],), (x,), True, stream)
        bitlinear_quant_act(x, self.xq[d], self.xds[d], None, stream, rmsnorm=True)
        bitlinear_gemv_glu(self.xq[d], self.xds[d], d, g.packed, g.beta, u.packed, u.beta, g.N, self.h, stream)
        self._linears(self.h, (L["down"],), (x,), True, stream)

    def step(self, x: torch.Tensor, stream=None) -> None:
        """One decode step: x [M][d] fp32 (the residual stream) is updated in place."""
        assert x.dtype == torch.float32 and tuple(x.shape) == (self.M, self.d) and x.is_contiguous()
        if self.requant:
            bitlinear_quant_act(x, self.rq_x[0], self.rq_x[1], None, stream, rmsnorm=True)
            for i in range(len(self.layers)):
                self._layer_rq(i, x, stream, last=i == len(self.layers) - 1)
            return
        for i in range(len(self.layers)):
            self.layer(i, x, stream)
