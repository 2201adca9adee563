"""Streaming preparation of a stack of layers, one layer's weights resident.

"MACaQ: Fast, Model Agnostic Calibrated Quantization for Low-Precision
Weights and Activations" (paper card, Abstract) keeps the transforms layer
local, so quantization can stream through a model with only one layer in
memory at a time; the 122B example of the card's Key numbers and of "MACaQ -
Huawei open-sources a 4-bit quantizer ..." (How it works) rests on that.

Here the bf16 weights of every layer sit in pinned host memory. Two device
slots take turns: while layer i is calibrated, folded and prepared on the
compute stream (the library's kernels, `binding.calibrate`,
`make_multipliers`, `prepare_weights`), layer i+1's weights are copied into the
other slot and layer i-1's packed weights are copied back to pinned host
memory on a copy stream. Device memory holds two weight slots and two packed
buffers, whatever the depth of the stack. This module only orders copies and
library calls on streams; it does no arithmetic of its own.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding


@dataclass
class HostLayer:
    """One linear layer in host memory: bf16 weights [N, K] (pinned for
    asynchronous copies) and bf16 calibration rows [R, K]."""
    w: torch.Tensor
    xcal: torch.Tensor


@dataclass
class PreparedHostLayer:
    """The prepared layer back in pinned host memory: activation multiplier a
    [K], weight multiplier r [K], packed codes and scales (GEMM layout)."""
    a: torch.Tensor
    r: torch.Tensor
    codes: torch.Tensor
    scales: torch.Tensor
    N: int
    K: int
    b: int


class StreamingPreparer:
    """Prepares HostLayers in order with copies overlapped with preparation."""

    def __init__(self, device, max_n: int, max_k: int, max_calib_rows: int):
        self.dev = torch.device(device)
        self.copy = torch.cuda.Stream(self.dev)
        self.comp = torch.cuda.Stream(self.dev)
        self.w_slot = [torch.empty(max_n * max_k, dtype=torch.bfloat16, device=self.dev) for _ in range(2)]
        self.x_slot = [torch.empty(max_calib_rows * max_k, dtype=torch.bfloat16, device=self.dev) for _ in range(2)]
        cb = binding.packed_codes_bytes(max_n, max_k)
        sb = binding.packed_scales_bytes(max_n, max_k)
        self.p_slot = [(torch.empty(cb, dtype=torch.uint8, device=self.dev),
                        torch.empty(sb, dtype=torch.uint8, device=self.dev)) for _ in range(2)]
        self.m_slot = [(torch.empty(max_k, dtype=torch.float32, device=self.dev),
                        torch.empty(max_k, dtype=torch.float32, device=self.dev)) for _ in range(2)]
        self.max_n, self.max_k, self.max_r = max_n, max_k, max_calib_rows

    def run(self, layers: list[HostLayer], b: int) -> list[PreparedHostLayer]:
        out = []
        loaded = [torch.cuda.Event() for _ in range(2)]    # weights of slot j are on the device
        prepared = [torch.cuda.Event() for _ in range(2)]  # packed result of slot j is ready
        drained = [torch.cuda.Event() for _ in range(2)]   # slot j's packed result is back on the host
        for j in range(2):
            drained[j].record(self.copy)

        def load(i):
            j = i % 2
            L = layers[i]
            N, K = L.w.shape
            R = L.xcal.shape[0]
            assert N <= self.max_n and K <= self.max_k and R <= self.max_r
            with torch.cuda.stream(self.copy):
                # the slot is free once the packed result that used it went home
                self.copy.wait_event(drained[j])
                self.w_slot[j][:N * K].view(N, K).copy_(L.w, non_blocking=True)
                self.x_slot[j][:R * K].view(R, K).copy_(L.xcal, non_blocking=True)
                loaded[j].record(self.copy)

        if layers:
            load(0)
        for i, L in enumerate(layers):
            j = i % 2
            N, K = L.w.shape
            R = L.xcal.shape[0]
            if i + 1 < len(layers):
                load(i + 1)
            with torch.cuda.stream(self.comp):
                self.comp.wait_event(loaded[j])
                w = self.w_slot[j][:N * K].view(N, K)
                x = self.x_slot[j][:R * K].view(R, K)
                s = binding.calibrate(x)
                a_d, r_d = self.m_slot[j]
                a, r = binding.make_multipliers(s, b)
                a_d[:K].copy_(a)
                r_d[:K].copy_(r)
                cb = binding.packed_codes_bytes(N, K)
                sb = binding.packed_scales_bytes(N, K)
                packed = binding.Packed(self.p_slot[j][0][:cb], self.p_slot[j][1][:sb], N, K)
                binding.prepare_weights(w, r_d[:K], b, out=packed)
                prepared[j].record(self.comp)
            res = PreparedHostLayer(torch.empty(K, dtype=torch.float32, pin_memory=True),
                                    torch.empty(K, dtype=torch.float32, pin_memory=True),
                                    torch.empty(cb, dtype=torch.uint8, pin_memory=True),
                                    torch.empty(sb, dtype=torch.uint8, pin_memory=True), N, K, b)
            with torch.cuda.stream(self.copy):
                self.copy.wait_event(prepared[j])
                res.a.copy_(a_d[:K], non_blocking=True)
                res.r.copy_(r_d[:K], non_blocking=True)
                res.codes.copy_(packed.codes, non_blocking=True)
                res.scales.copy_(packed.scales, non_blocking=True)
                drained[j].record(self.copy)
            out.append(res)
        self.copy.synchronize()
        self.comp.synchronize()
        return out
