"""One MoE feed-forward layer on the GPU: device-resident weights and buffers,
and the forward pass as a chain of libmoe.so calls on one stream.

    route -> permute -> grouped gate/up -> grouped down -> [shared expert]
          -> combine -> stats

PyTorch only allocates device memory and supplies the stream; every step runs
in the library's HIP kernels.  Nothing is read back to the host inside
``forward``: grid sizes use the upper bound T*k rows.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import _lib
from .inputs import LayerInputs, LayerShape


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Copy a host array (bf16 bit patterns as uint16, or float32) to the GPU."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


class DeviceWeights:
    """Router, routed experts and shared expert of one layer in GPU memory.

    gate/up [E][F][d], down [E][d][F] (nn.Linear order, per expert)."""

    def __init__(self, inputs: LayerInputs, device="cuda"):
        s = inputs.shape
        self.shape, self.device = s, torch.device(device)
        td = torch_dtype(s.dtype)
        self.w_router = to_device(inputs.w_router, s.dtype, self.device)
        self.bias = None if inputs.bias is None else torch.from_numpy(inputs.bias).to(self.device)
        # selection-only bias (bias balancing): updated in place by MoeLayer.bias_update
        self.select_bias = (None if inputs.select_bias is None else
                            torch.from_numpy(inputs.select_bias.copy()).to(self.device))
        self.gate = torch.empty((s.E, s.F, s.d), dtype=td, device=self.device)
        self.up = torch.empty((s.E, s.F, s.d), dtype=td, device=self.device)
        self.down = torch.empty((s.E, s.d, s.F), dtype=td, device=self.device)

        def sink(e, g, u, dn):
            self.gate[e].copy_(to_device(g, s.dtype, self.device))
            self.up[e].copy_(to_device(u, s.dtype, self.device))
            self.down[e].copy_(to_device(dn, s.dtype, self.device))

        inputs.experts(sink=sink)
        sh = inputs.shared()
        self.shared = None if sh is None else tuple(to_device(m, s.dtype, self.device) for m in sh)
        torch.cuda.synchronize(self.device)

    def addresses(self) -> tuple:
        """Device addresses of every weight tensor (0 for an absent one)."""
        ts = (self.w_router, self.bias, self.select_bias, self.gate, self.up, self.down) + (self.shared or (None,) * 3)
        return tuple(0 if t is None else t.data_ptr() for t in ts)


class Buffers:
    """Every intermediate and output of the layer for T tokens (device memory).
    x_perm (the gathered copy of x) is only allocated with ``gathered=True``;
    by default the gate/up GEMM reads x through perm_token."""

    def __init__(self, shape: LayerShape, T: int, device="cuda", gathered: bool = False, scatter: bool = False):
        s = shape
        dev = torch.device(device)
        td = torch_dtype(s.dtype)
        R = T * s.k
        i32, f32 = torch.int32, torch.float32
        self.T = T
        self.logits = torch.empty((T, s.E), dtype=f32, device=dev)
        self.topk_idx = torch.empty((T, s.k), dtype=i32, device=dev)
        self.topk_w = torch.empty((T, s.k), dtype=f32, device=dev)
        self.near_tie = torch.empty((T,), dtype=i32, device=dev)
        self.counts = torch.empty((s.E,), dtype=i32, device=dev)
        self.offsets = torch.empty((s.E + 1,), dtype=i32, device=dev)
        self.row_of = torch.empty((T, s.k), dtype=i32, device=dev)
        self.perm_token = torch.empty((max(R, 1),), dtype=i32, device=dev)
        self.x_perm = torch.empty((max(R, 1), s.d), dtype=td, device=dev) if gathered else None
        self.a = torch.empty((max(R, 1), s.F), dtype=td, device=dev)
        self.y_perm = torch.empty((max(R, 1), s.d), dtype=td, device=dev)
        self.y = torch.empty((T, s.d), dtype=td, device=dev)
        self.f = torch.empty((s.E,), dtype=f32, device=dev)
        self.P = torch.empty((s.E,), dtype=f32, device=dev)
        self.l_aux = torch.empty((1,), dtype=f32, device=dev)
        self.max_over_mean = torch.empty((1,), dtype=f32, device=dev)
        self.ws_permute = torch.empty((max(_lib.moe_permute_workspace_bytes(T, s.k, s.E), 1),), dtype=torch.uint8,
                                      device=dev)
        self.ws_stats = torch.empty((max(_lib.moe_stats_workspace_bytes(T, s.E), 1),), dtype=torch.uint8,
                                    device=dev)
        # scatter combine: the float32 accumulator and row weights of moe_grouped_down_combine
        self.ws_scatter = (torch.empty((max(_lib.moe_down_combine_workspace_bytes(T, s.d, R), 1),),
                                       dtype=torch.uint8, device=dev) if scatter else None)
        # ordering between the main stream and a side stream running the statistics
        self.fork_event, self.stats_event = torch.cuda.Event(), torch.cuda.Event()
        # (key, moe_layer_args) of the last one-call forward on this buffer set
        self.layer_args = None
        if s.F_shared > 0:
            self.shared_offsets = torch.tensor([0, T], dtype=i32, device=dev)
            self.shared_a = torch.empty((max(T, 1), s.F_shared), dtype=td, device=dev)
            self.shared_y = torch.empty((max(T, 1), s.d), dtype=td, device=dev)
        else:
            self.shared_offsets = self.shared_a = self.shared_y = None


# Groups averaging at most this many rows (the weight-streaming GEMM regime) keep
# the statistics on the main stream.
SMALL_GROUP_ROWS = 16


class MoeLayer:
    """Forward pass of one MoE layer through libmoe.so.

    scatter_combine: the down GEMM adds its weighted rows straight into a float32
    accumulator (moe_grouped_down_combine) instead of writing y_perm for the
    gather combine; y then depends on the order of float32 atomic additions."""

    def __init__(self, weights: DeviceWeights, scatter_combine: bool = False):
        self.w = weights
        self.shape = weights.shape
        self.scatter_combine = scatter_combine

    def buffers(self, T: int, gathered: bool = False) -> Buffers:
        return Buffers(self.shape, T, self.w.device, gathered, scatter=self.scatter_combine)

    def route(self, x, b: Buffers, stream=None):
        s = self.shape
        _lib.moe_route(x, self.w.w_router, self.w.bias, b.T, s.d, s.E, s.k, s.mode, s.renorm, b.logits,
                       b.topk_idx, b.topk_w, b.near_tie, stream, select_bias=self.w.select_bias)

    def bias_update(self, b: Buffers, rate: float, stream=None):
        """One bias-balancing step from the demand counts of the last permute."""
        s = self.shape
        if self.w.select_bias is None:
            raise ValueError("this layer has no selection bias")
        _lib.moe_bias_update(b.counts, b.T, s.k, s.E, rate, self.w.select_bias, stream)

    def permute(self, x, b: Buffers, stream=None):
        """Dispatch; also gathers x_perm when the buffers hold one."""
        s = self.shape
        cap = _lib.moe_capacity(b.T, s.k, s.E, s.phi)
        _lib.moe_permute(b.topk_idx, b.T, s.k, s.E, cap, x, s.d, b.counts, b.offsets, b.row_of, b.perm_token,
                         b.x_perm, b.ws_permute, stream)

    def gate_up(self, x, b: Buffers, stream=None):
        s = self.shape
        R = b.T * s.k
        if b.x_perm is not None:
            _lib.moe_grouped_gate_up(b.x_perm, None, 0, b.offsets, s.E, R, s.d, s.F, self.w.gate, self.w.up, b.a,
                                     stream)
        else:
            _lib.moe_grouped_gate_up(x, b.perm_token, b.T, b.offsets, s.E, R, s.d, s.F, self.w.gate, self.w.up,
                                     b.a, stream)

    def down(self, b: Buffers, stream=None):
        s = self.shape
        _lib.moe_grouped_down(b.a, b.offsets, s.E, b.T * s.k, s.F, s.d, self.w.down, b.y_perm, stream)

    def experts(self, x, b: Buffers, stream=None):
        self.gate_up(x, b, stream)
        self.down(b, stream)

    def shared_expert(self, x, b: Buffers, stream=None):
        s = self.shape
        if self.w.shared is None:
            return
        g, u, dn = self.w.shared
        _lib.moe_grouped_swiglu(x, None, 0, b.shared_offsets, 1, b.T, s.d, s.F_shared, g, u, dn, b.shared_a,
                                b.shared_y, stream)

    def down_combine(self, b: Buffers, stream=None):
        """The down GEMM with the combine in its epilogue; adds shared_y, so the
        shared expert runs first."""
        s = self.shape
        if b.ws_scatter is None:
            raise ValueError("these buffers hold no scatter workspace (Buffers(..., scatter=True))")
        _lib.moe_grouped_down_combine(b.a, b.offsets, s.E, b.T * s.k, s.F, s.d, self.w.down, b.perm_token, b.row_of,
                                      b.topk_w, b.T, s.k, b.shared_y, b.y, b.ws_scatter, stream)

    def combine(self, b: Buffers, stream=None):
        s = self.shape
        _lib.moe_combine(b.y_perm, b.row_of, b.topk_w, b.shared_y, b.T, s.k, s.d, b.y, stream)

    def stats(self, b: Buffers, stream=None):
        s = self.shape
        _lib.moe_stats(b.counts, b.logits, b.T, s.k, s.E, s.alpha, b.f, b.P, b.l_aux, b.max_over_mean,
                       b.ws_stats, stream)

    def _fork_stats(self, b: Buffers, stream, side):
        """Balance statistics on `side`, after the work already queued on `stream`."""
        b.fork_event.record(stream)
        side.wait_event(b.fork_event)
        self.stats(b, side)
        b.stats_event.record(side)

    def forward(self, x: torch.Tensor, b: Optional[Buffers] = None, stream=None, side_stream=None,
                marks=None) -> Buffers:
        """Whole layer for x[T][d] (device).  Returns the buffers holding y and
        every intermediate; asynchronous on `stream`.

        side_stream: with large groups the balance statistics (which only read the
        scores and the counts) run there beside the combine, which leaves room on
        the CUs (measured at T = 16384: 1.558 -> 1.543 ms per layer).  `stream` waits
        for them before this returns, so later work on `stream` sees every output.
        Small groups (decode) keep them on `stream`: there the fork and join cost
        more than the overlap saves.  Results are identical either way.
        marks: three events recorded on `stream` before gate/up, between gate/up
        and down, and after down (for timing); a fourth, if given, after the
        shared expert.  With the scatter combine the order is gate/up, shared
        expert, down with the combine: the marks then fall before gate/up, after
        it, after the shared expert and after the down+combine call."""
        if b is None:
            b = self.buffers(x.shape[0])
        if b.T == 0:
            return b
        s = self.shape
        st = stream if stream is not None else torch.cuda.current_stream()
        if b.ws_scatter is None and b.x_perm is None:
            # the whole layer in one library call (the fused decode form inside it);
            # the materialized gather and the scatter combine take the separate calls
            # the struct holds device addresses only: reuse it while every address and
            # the shape are the same (a new tensor at a reused address is then as valid)
            key = (s, tuple(x.shape), x.dtype, x.data_ptr()) + self.w.addresses()
            if b.layer_args is None or b.layer_args[0] != key:
                cap = _lib.moe_capacity(b.T, s.k, s.E, s.phi)
                b.layer_args = (key, _lib.layer_args(s, x, self.w, b, cap))
            args = b.layer_args[1]
            side = side_stream if side_stream is not None and b.T * s.k > SMALL_GROUP_ROWS * s.E else None
            _lib.moe_layer_forward(args, st, side, b.fork_event if side else None, b.stats_event if side else None,
                                   marks)
            return b
        self.route(x, b, st)
        self.permute(x, b, st)
        if side_stream is not None and b.T * s.k <= SMALL_GROUP_ROWS * s.E:
            side_stream = None
        if marks is not None:
            marks[0].record(st)
        self.gate_up(x, b, st)
        if marks is not None:
            marks[1].record(st)
        if b.ws_scatter is not None:
            self.shared_expert(x, b, st)
            if marks is not None:
                marks[2].record(st)
            if side_stream is not None:
                self._fork_stats(b, st, side_stream)
            self.down_combine(b, st)
            if marks is not None and len(marks) > 3:
                marks[3].record(st)
            if side_stream is None:
                self.stats(b, st)
            else:
                st.wait_event(b.stats_event)
            return b
        self.down(b, st)
        if marks is not None:
            marks[2].record(st)
        self.shared_expert(x, b, st)
        if marks is not None and len(marks) > 3:
            marks[3].record(st)
        if side_stream is not None:
            self._fork_stats(b, st, side_stream)
        self.combine(b, st)
        if side_stream is None:
            self.stats(b, st)
        else:
            st.wait_event(b.stats_event)
        return b
