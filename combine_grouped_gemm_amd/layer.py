"""One GPU's share of a sparse MoE layer as a sequence of libmoe calls on one stream.

    router logits -> route -> dispatch layout -> permute -> grouped SwiGLU FFN (+ shared expert)
    -> combine

("MoE part 4" page, section 4 and 4.2; "EP / DeepEP explanation" page, sections 2-3.)
Given the router weight W_r the layer computes the logits z = x W_r^T itself; without
it, forward takes z.
All buffers are allocated once, at construction, so a forward pass enqueues
only kernels: no allocation, no host synchronisation, no device-to-host copy.

bf16 layers fold the permute into the gate/up GEMM by default (``gather=True``): its
operand rows are read straight from x through the layout's src_slot map, so the
permuted copy of x is never written.  f32 layers run the permute kernel.  fp8 layers with a
shared expert and more than 16 rows per expert on average quantize each token once (its
fp8 payload), turn the codes back into bf16 values once, and gather those rows the same way;
other fp8 layers run the quantize-on-permute kernel.  Layers with gathered rows also run
the shared expert inside the routed GEMM launches by default (``fuse_shared=True``): its
rows follow the routed rows in h and in the expert outputs.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (MOE_BF16, MOE_F32, MOE_FP8_E4M3, MOE_OP_DISPATCH_LAYOUT, MOE_OP_EXPERT_DGRAD, MOE_OP_EXPERT_GEMM,
               MOE_OP_GROUPED_FFN, MOE_OP_ROUTER, moe_combine, moe_combine_backward, moe_dispatch_layout,
               moe_dequantize_fp8, moe_expert_dgrad, moe_expert_down, moe_expert_down_shared,
               moe_expert_down_shared_e4m3, moe_expert_gate_up, moe_expert_gate_up_gathered,
               moe_expert_gate_up_gathered_shared, moe_expert_gate_up_gathered_shared_e4m3, moe_expert_gate_up_preact,
               moe_expert_wgrad, moe_grouped_ffn, moe_permute, moe_quantize_fp8, moe_route, moe_router_backward,
               moe_router_input_grad, moe_router_logits, moe_swiglu_backward, moe_workspace_bytes)


class MoELayer:
    """Pre-planned MoE layer for fixed sizes.

    ``dtype``: 'f32' (fp32 everywhere), 'bf16' (bf16 storage, fp32 accumulation) or
    'fp8' (bf16 hidden states; e4m3 payload and weights with per-128-column fp32
    scales; bf16 h, expert outputs and y).  Weights come in the storage dtype
    (bf16 for 'fp8'); the fp8 layer quantizes them once here, with the library's
    own row quantizer.  ``w_r`` [E, H] (storage dtype): the router weight; the
    logits then come from moe_router_logits on x.
    """

    def __init__(self, N: int, H: int, E: int, k: int, I: int, dtype: str, w13: torch.Tensor,
                 w2: torch.Tensor, shared_w13: Optional[torch.Tensor] = None,
                 shared_w2: Optional[torch.Tensor] = None, n_group: int = 0, topk_group: int = 0,
                 bias: Optional[torch.Tensor] = None, gather: bool = True, overlap_shared: bool = False,
                 fuse_shared: bool = True, gate_in_down: bool = False, w_r: Optional[torch.Tensor] = None):
        self.N, self.H, self.E, self.k, self.I = N, H, E, k, I
        self.dtype, self.n_group, self.topk_group, self.bias = dtype, n_group, topk_group, bias
        dev = w13.device
        self.device = dev
        self.fp8 = dtype == "fp8"
        # fp8 above decode sizes (more than 16 rows per expert on average) with a shared expert:
        # the gathered, fused path on e4m3 weights; at decode sizes the weight-streaming kernels
        self.fp8_gather = bool(self.fp8 and gather and fuse_shared and shared_w13 is not None and N * k > 16 * E)
        self.gather = gather and (dtype == "bf16" or self.fp8_gather)
        act = torch.float32 if dtype == "f32" else torch.bfloat16
        self.act_dtype = act
        rows = N * k
        if self.fp8:
            self.w13, self.w13_scale = moe_quantize_fp8(w13)
            self.w2, self.w2_scale = moe_quantize_fp8(w2)
            if shared_w13 is not None:
                self.sw13, self.sw13_scale = moe_quantize_fp8(shared_w13)
                self.sw2, self.sw2_scale = moe_quantize_fp8(shared_w2)
        else:
            self.w13, self.w2, self.w13_scale, self.w2_scale = w13, w2, None, None
            self.sw13, self.sw2 = shared_w13, shared_w2
            self.sw13_scale = self.sw2_scale = None
        self.shared = shared_w13 is not None
        self.fuse = bool(fuse_shared and self.shared and self.gather)
        # the routed rows' gates applied in the down GEMM's epilogue (combine then sums)
        self.gate_in_down = bool(gate_in_down and self.fuse and not self.fp8)
        i32 = dict(dtype=torch.int32, device=dev)
        self.w_r = w_r
        if w_r is not None:
            self.z = torch.empty((N, E), dtype=torch.float32, device=dev)
            x_dt = MOE_F32 if dtype == "f32" else MOE_BF16
            self.router_ws = torch.empty(max(moe_workspace_bytes(MOE_OP_ROUTER, N, H, 0, E, 0, x_dt), 256),
                                         dtype=torch.uint8, device=dev)
        self.topk_idx = torch.empty((N, k), **i32)
        self.topk_gate = torch.empty((N, k), dtype=torch.float32, device=dev)
        self.layout = (torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty(rows, **i32),
                       torch.empty(rows, **i32))
        self.layout_ws = torch.empty(max(moe_workspace_bytes(MOE_OP_DISPATCH_LAYOUT, N, 0, 0, E, k, 0), 256),
                                     dtype=torch.uint8, device=dev)
        a_dt = MOE_FP8_E4M3 if self.fp8 else (MOE_F32 if dtype == "f32" else MOE_BF16)
        self.a_dt = a_dt
        self.x_perm = None if self.gather else torch.empty((rows, H), dtype=torch.uint8 if self.fp8 else act,
                                                          device=dev)
        self.x_perm_scale = (torch.empty((rows, H // 128), dtype=torch.float32, device=dev)
                             if self.fp8 and not self.gather else None)
        if self.fp8_gather:
            # each token's fp8 payload (codes and block scales) and its values as bf16 rows
            self.x_q = torch.empty((N, H), dtype=torch.uint8, device=dev)
            self.x_q_scale = torch.empty((N, H // 128), dtype=torch.float32, device=dev)
            self.x_deq = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
        self.ffn_ws = None if self.fuse else torch.empty(
            max(moe_workspace_bytes(MOE_OP_GROUPED_FFN, rows, H, I, E, 1, a_dt), 256), dtype=torch.uint8, device=dev)
        if self.fuse:
            # routed rows then the shared expert's N rows, in h and in the expert outputs
            self.h_all = torch.empty((rows + N, I), dtype=torch.bfloat16, device=dev)
            self.out_all = torch.empty((rows + N, H), dtype=act, device=dev)
            self.fused_ws = torch.empty(max(moe_workspace_bytes(MOE_OP_EXPERT_GEMM, rows + N, H, I, E + 1, 1,
                                                                MOE_BF16 if self.fp8 else a_dt), 256),
                                        dtype=torch.uint8, device=dev)
        else:
            self._expert_out = torch.empty((rows, H), dtype=act, device=dev)
        if self.shared and not self.fuse:
            self.shared_offsets = torch.tensor([0, N], **i32)
            self.x_q = torch.empty((N, H), dtype=torch.uint8, device=dev) if self.fp8 else None
            self.x_q_scale = torch.empty((N, H // 128), dtype=torch.float32, device=dev) if self.fp8 else None
            self.shared_ws = torch.empty(max(moe_workspace_bytes(MOE_OP_GROUPED_FFN, N, H, I, 1, 1, a_dt), 256),
                                         dtype=torch.uint8, device=dev)
            self._shared_out = torch.empty((N, H), dtype=act, device=dev)
        # the shared expert needs only x: it runs on a second stream (default priority)
        # beside route / layout / the routed FFN, and combine waits for it
        self.side = torch.cuda.Stream(device=dev) if self.shared and overlap_shared and not self.fuse else None
        self.shared_done = torch.cuda.Event() if self.side is not None else None
        self.y = torch.empty((N, H), dtype=act, device=dev)
        self.save_au = False     # the next forward keeps the gate/up pre-activations (training)
        self.au_saved = False    # the last forward kept them
        self.au_all = None

    _WEIGHTS = ("w13", "w2", "w13_scale", "w2_scale", "sw13", "sw2", "sw13_scale", "sw2_scale", "w_r", "bias")
    _WEIGHT_GRADS = ("dw13", "dw2", "dsw13", "dsw2", "dw_r")

    def device_bytes(self) -> dict:
        """Bytes of device memory the layer holds, by kind (each allocation counted once).

        weights: the routed, shared and router weights, fp8 scales included; workspace: the
        library's scratch buffers; activations: the forward's other buffers (logits, routes,
        layout, permuted rows, h, expert outputs, y; the kept pre-activations once a training
        forward ran).  After a backward also weight_grads and backward (its intermediates and
        workspaces).  The caller's input x is not the layer's and is not counted.
        """
        seen, out = set(), {"weights": 0, "activations": 0, "workspace": 0}

        def add(kind, v):
            for t in (v if isinstance(v, tuple) else (v,)):
                if isinstance(t, torch.Tensor) and t.is_cuda and t.untyped_storage().data_ptr() not in seen:
                    seen.add(t.untyped_storage().data_ptr())
                    out[kind] = out.get(kind, 0) + t.untyped_storage().nbytes()

        for name, v in vars(self).items():
            if name != "grads":
                add("weights" if name in self._WEIGHTS else "workspace" if name.endswith("_ws") else "activations", v)
        for name, v in (getattr(self, "grads", None) or {}).items():
            add("weight_grads" if name in self._WEIGHT_GRADS else "backward", v)
        return out

    @property
    def expert_out(self) -> torch.Tensor:
        """The routed experts' outputs [N*k, H] of the last forward."""
        return self.out_all[:self.N * self.k] if self.fuse else self._expert_out

    @property
    def shared_out(self) -> torch.Tensor:
        """The shared expert's output [N, H] of the last forward."""
        return self.out_all[self.N * self.k:] if self.fuse else self._shared_out

    @property
    def h(self) -> torch.Tensor:
        """The intermediate h of the last routed FFN (a view into the workspace)."""
        if self.fuse:
            return self.h_all[:self.N * self.k]
        off = moe_workspace_bytes(MOE_OP_EXPERT_GEMM, self.N * self.k, self.H, self.I, self.E, 1, self.a_dt)
        esz = 4 if self.dtype == "f32" else 2
        n = self.N * self.k * self.I * esz
        return self.ffn_ws[off:off + n].view(torch.float32 if esz == 4 else torch.bfloat16).view(
            self.N * self.k, self.I)

    def router(self, x: torch.Tensor):
        """Router logits z = x W_r^T into self.z."""
        return moe_router_logits(x, self.w_r, self.z, self.router_ws)

    def route(self, z: torch.Tensor):
        return moe_route(z, self.k, self.bias, self.n_group, self.topk_group, self.topk_idx, self.topk_gate)

    def dispatch(self):
        return moe_dispatch_layout(self.topk_idx, self.E, self.layout, self.layout_ws)

    def permute(self, x: torch.Tensor):
        """The permuted payload (nothing to do when the gate/up GEMM gathers its rows)."""
        send_pos = self.layout[2]
        if self.fp8_gather:   # each token once: codes and scales, then their bf16 values
            moe_quantize_fp8(x, self.x_q, self.x_q_scale)
            return moe_dequantize_fp8(self.x_q, self.x_q_scale, self.x_deq)
        if self.gather:
            return None
        if self.fp8:
            return moe_permute(x, send_pos, self.k, MOE_FP8_E4M3, self.x_perm, self.x_perm_scale)
        return moe_permute(x, send_pos, self.k, None, self.x_perm)

    def gate_up(self, x: torch.Tensor):
        """Grouped gate/up GEMM + SwiGLU into h (gathered layers read x directly; fused
        layers also compute the shared expert's rows)."""
        if self.fuse and self.fp8:
            return moe_expert_gate_up_gathered_shared_e4m3(self.x_deq, self.layout[3], self.k, self.layout[1],
                                                           self.w13, self.w13_scale, self.sw13, self.sw13_scale,
                                                           h=self.h_all, ws=self.fused_ws)
        if self.fuse:
            return moe_expert_gate_up_gathered_shared(x, self.layout[3], self.k, self.layout[1], self.w13,
                                                      self.sw13, h=self.h_all, ws=self.fused_ws,
                                                      au=self.au_all if self.save_au else None)
        if self.gather:
            return moe_expert_gate_up_gathered(x, self.layout[3], self.k, self.layout[1], self.w13,
                                               h=self.h, ws=self.ffn_ws)
        return moe_expert_gate_up(self.x_perm, self.layout[1], self.w13, self.x_perm_scale, self.w13_scale,
                                  self.h, self.ffn_ws)

    def down(self):
        """Grouped down GEMM of h into the expert outputs."""
        if self.fuse and self.fp8:
            return moe_expert_down_shared_e4m3(self.h_all, self.layout[1], self.w2, self.w2_scale, self.sw2,
                                               self.sw2_scale, self.N * self.k, out=self.out_all, ws=self.fused_ws)
        if self.fuse:
            gates = (self.layout[3], self.topk_gate) if self.gate_in_down else (None, None)
            return moe_expert_down_shared(self.h_all, self.layout[1], self.w2, self.sw2, self.N * self.k,
                                          out=self.out_all, ws=self.fused_ws, src_slot=gates[0],
                                          topk_gate=gates[1])
        return moe_expert_down(self.h, self.layout[1], self.w2, self.w2_scale, self.expert_out, self.ffn_ws)

    def experts(self, x: Optional[torch.Tensor] = None):
        if self.gather:
            self.gate_up(x)
            return self.down()
        return moe_grouped_ffn(self.x_perm, self.layout[1], self.w13, self.w2, self.x_perm_scale,
                               self.w13_scale, self.w2_scale, self.expert_out, self.ffn_ws)

    def shared_expert(self, x: torch.Tensor):
        if self.fuse:
            return None   # computed by gate_up / down
        a, a_scale = x, None
        if self.fp8:
            a, a_scale = moe_quantize_fp8(x, self.x_q, self.x_q_scale)
        return moe_grouped_ffn(a, self.shared_offsets, self.sw13, self.sw2, a_scale, self.sw13_scale,
                               self.sw2_scale, self._shared_out, self.shared_ws)

    def combine(self):
        return moe_combine(self.expert_out, self.layout[2], None if self.gate_in_down else self.topk_gate,
                           self.shared_out if self.shared else None, self.y, k=self.k)

    def launch_shared_side(self, x: torch.Tensor):
        """Enqueue the shared expert on the side stream, after the work queued so far."""
        main = torch.cuda.current_stream(self.device)
        self.side.wait_stream(main)
        x.record_stream(self.side)
        with torch.cuda.stream(self.side):
            self.shared_expert(x)
            self.shared_done.record(self.side)

    def forward(self, x: torch.Tensor, z: Optional[torch.Tensor] = None, save_for_backward: bool = False) -> torch.Tensor:
        """y for tokens x; z: the router logits (computed from W_r when None).  With
        save_for_backward a bf16 layer that runs the shared expert inside the routed launches
        also keeps the gate/up pre-activations, which backward then reads instead of
        recomputing them."""
        self.save_au = bool(save_for_backward and self.fuse and not self.fp8)
        if self.save_au and self.au_all is None:
            self.au_all = torch.empty((self.N * self.k + self.N, 2 * self.I), dtype=torch.bfloat16,
                                      device=self.device)
        self.au_saved = self.save_au
        if self.side is not None:
            self.launch_shared_side(x)
        if z is None:
            if self.w_r is None:
                raise ValueError("forward needs the logits z, or a layer built with the router weight w_r")
            z = self.router(x)
        self.route(z)
        self.dispatch()
        self.permute(x)
        self.experts(x)
        if self.shared:
            if self.side is not None:
                torch.cuda.current_stream(self.device).wait_event(self.shared_done)
            else:
                self.shared_expert(x)
        self.combine()
        return self.y

    # ---- backward (bf16 layers that gather their rows from x)

    def _alloc_backward(self, dw_dtype: torch.dtype):
        N, H, E, k, I = self.N, self.H, self.E, self.k, self.I
        rows = N * k
        dev, bf = self.device, torch.bfloat16
        b = {}
        b["d_eo"] = torch.empty((rows, H), dtype=bf, device=dev)
        b["dg"] = torch.empty((N, k), dtype=torch.float32, device=dev)
        b["au"] = torch.empty((rows, 2 * I), dtype=bf, device=dev)
        b["dh"] = torch.empty((rows, I), dtype=bf, device=dev)
        b["d_au"] = torch.empty((rows, 2 * I), dtype=bf, device=dev)
        b["h"] = torch.empty((rows, I), dtype=bf, device=dev)
        b["d_perm"] = torch.empty((rows, H), dtype=bf, device=dev)
        b["x_perm"] = torch.empty((rows, H), dtype=bf, device=dev)
        b["dw13"] = torch.empty((E, 2 * I, H), dtype=dw_dtype, device=dev)
        b["dw2"] = torch.empty((E, H, I), dtype=dw_dtype, device=dev)
        b["gemm_ws"] = torch.empty(max(moe_workspace_bytes(MOE_OP_EXPERT_GEMM, max(rows, N), H, I, E, 1, MOE_BF16),
                                       256), dtype=torch.uint8, device=dev)
        b["dgrad_ws"] = torch.empty(max(moe_workspace_bytes(MOE_OP_EXPERT_DGRAD, max(rows, N), 0, 0, E, 0, 0), 256),
                                    dtype=torch.uint8, device=dev)
        if self.shared:
            # (the shared expert's steps have workspaces of their own: they may run on a
            # second stream beside the routed ones)
            b["gemm_ws_s"] = torch.empty(max(moe_workspace_bytes(MOE_OP_EXPERT_GEMM, N, H, I, 1, 1, MOE_BF16), 256),
                                         dtype=torch.uint8, device=dev)
            b["dgrad_ws_s"] = torch.empty(max(moe_workspace_bytes(MOE_OP_EXPERT_DGRAD, N, 0, 0, 1, 0, 0), 256),
                                          dtype=torch.uint8, device=dev)
            b["shared_offsets"] = torch.tensor([0, N], dtype=torch.int32, device=dev)
            b["au_s"] = torch.empty((N, 2 * I), dtype=bf, device=dev)
            b["dh_s"] = torch.empty((N, I), dtype=bf, device=dev)
            b["d_au_s"] = torch.empty((N, 2 * I), dtype=bf, device=dev)
            b["h_s"] = torch.empty((N, I), dtype=bf, device=dev)
            b["dx_s"] = torch.empty((N, H), dtype=bf, device=dev)
            b["dsw13"] = torch.empty((1, 2 * I, H), dtype=dw_dtype, device=dev)
            b["dsw2"] = torch.empty((1, H, I), dtype=dw_dtype, device=dev)
        if self.w_r is not None:
            b["dz"] = torch.empty((N, k), dtype=torch.float32, device=dev)
            b["dw_r"] = torch.empty((E, H), dtype=dw_dtype, device=dev)
            b["dx_r"] = torch.empty((N, H), dtype=bf, device=dev)
        b["dx"] = torch.empty((N, H), dtype=bf, device=dev)
        b["dw_dtype"] = dw_dtype
        self.grads = b

    def backward_steps(self, x: torch.Tensor, dy: torch.Tensor, dw_dtype: torch.dtype = torch.bfloat16) -> list:
        """The backward pass as (name, call) steps in stream order (see backward)."""
        if self.dtype != "bf16" or not self.gather:
            raise ValueError("the backward pass is built for bf16 layers that gather their rows from x")
        if self.gate_in_down:
            raise ValueError("backward needs the unscaled expert outputs (gate_in_down=False)")
        if getattr(self, "grads", None) is None or self.grads["dw_dtype"] != dw_dtype:
            self._alloc_backward(dw_dtype)
        b = self.grads
        k, N = self.k, self.N
        rows = N * k
        offsets, send_pos, src_slot = self.layout[1], self.layout[2], self.layout[3]
        # the pre-activations: kept by the forward, or recomputed here
        saved = self.au_saved
        au = self.au_all[:rows] if saved else b["au"]
        au_s = self.au_all[rows:] if saved else b.get("au_s")
        st = [
            ("combine_bwd", lambda: moe_combine_backward(dy, send_pos, self.topk_gate, self.expert_out, b["d_eo"],
                                                         b["dg"])),
        ]
        if not saved:
            st.append(("gate_up_preact", lambda: moe_expert_gate_up_preact(x, offsets, self.w13, rows, src_slot, k,
                                                                           b["au"], b["gemm_ws"])))
        st += [
            ("down_dgrad", lambda: moe_expert_dgrad(b["d_eo"], offsets, self.w2, b["dh"], b["dgrad_ws"])),
            ("swiglu_bwd", lambda: moe_swiglu_backward(au, b["dh"], b["d_au"], b["h"])),
            ("down_wgrad", lambda: moe_expert_wgrad(b["d_eo"], b["h"], offsets, dw=b["dw2"], rows=rows)),
            # the weight gradient of W13 reads the expert-ordered rows of x (a permuted copy:
            # the wgrad kernel streams its B operand in layout order)
            ("x_permute", lambda: moe_permute(x, send_pos, k, None, b["x_perm"])),
            ("gate_up_wgrad", lambda: moe_expert_wgrad(b["d_au"], b["x_perm"], offsets, dw=b["dw13"], rows=rows)),
            ("gate_up_dgrad", lambda: moe_expert_dgrad(b["d_au"], offsets, self.w13, b["d_perm"], b["dgrad_ws"])),
        ]
        rest = None
        if self.shared:
            so = b["shared_offsets"]
            if not saved:
                st.append(("shared_preact", lambda: moe_expert_gate_up_preact(x, so, self.sw13, N, None, 1,
                                                                              b["au_s"], b["gemm_ws_s"])))
            st += [
                ("shared_down_dgrad", lambda: moe_expert_dgrad(dy, so, self.sw2, b["dh_s"], b["dgrad_ws_s"])),
                ("shared_swiglu_bwd", lambda: moe_swiglu_backward(au_s, b["dh_s"], b["d_au_s"], b["h_s"])),
                ("shared_down_wgrad", lambda: moe_expert_wgrad(dy, b["h_s"], so, dw=b["dsw2"], rows=N)),
                ("shared_gate_up_wgrad", lambda: moe_expert_wgrad(b["d_au_s"], x, so, dw=b["dsw13"], rows=N)),
                ("shared_gate_up_dgrad", lambda: moe_expert_dgrad(b["d_au_s"], so, self.sw13, b["dx_s"],
                                                                  b["dgrad_ws_s"])),
            ]
            rest = b["dx_s"]
        if self.w_r is not None:
            # sum_j dz_tj W_r[e_tj] (+ the shared expert's input gradient)
            rest_r = rest
            st += [
                ("router_bwd", lambda: moe_router_backward(self.topk_gate, b["dg"], offsets, src_slot, x, b["dz"],
                                                           b["dw_r"])),
                ("router_dx", lambda: moe_router_input_grad(self.w_r, self.topk_idx, b["dz"], rest_r, b["dx_r"])),
            ]
            rest = b["dx_r"]
        rest_x = rest
        st.append(("dx", lambda: moe_combine(b["d_perm"], send_pos, None, rest_x, b["dx"], k=k)))
        return st

    def backward(self, x: torch.Tensor, dy: torch.Tensor, dw_dtype: torch.dtype = torch.bfloat16,
                 overlap_shared: bool = False) -> dict:
        """Gradients of the last forward for the upstream gradient dy [N, H] (bf16).

        The backward mirrors the forward ("DeepSeek MoE: EP and FSDP guide": dispatch's
        backward is combine): combine backward (d_expert_out, d_gate); the gate/up
        pre-activations recomputed; dh = d_expert_out W_down; SwiGLU backward; the weight
        gradients dW_down = d_expert_out^T h and dW13 = d_au^T x per expert; the input
        gradient of every slot d_au W13; the same for the shared expert on dy; the gates'
        and router's gradients; dx = the slots' gradients summed back to their tokens plus
        the shared expert's and the router's.  Buffers are allocated on the first call.
        Returns the dict of gradient tensors ('dx', 'dw13', 'dw2', 'dsw13', 'dsw2', 'dw_r', ...).
        With overlap_shared the shared expert's steps (which need only x, dy and its
        pre-activations) run on a second stream (default priority) beside the routed ones, and
        the input-gradient sum waits for them.
        """
        steps = self.backward_steps(x, dy, dw_dtype)
        if not (overlap_shared and self.shared):
            for _, f in steps:
                f()
            return self.grads
        main = torch.cuda.current_stream(self.device)
        if getattr(self, "bwd_side", None) is None:
            self.bwd_side = torch.cuda.Stream(device=self.device)
            self.bwd_side_done = torch.cuda.Event()
        side = self.bwd_side
        side.wait_stream(main)
        with torch.cuda.stream(side):
            for name, f in steps:
                if name.startswith("shared_"):
                    f()
            self.bwd_side_done.record(side)
        for name, f in steps:
            if name.startswith("shared_"):
                continue
            if name in ("router_dx", "dx") and not getattr(self, "_waited", False):
                main.wait_event(self.bwd_side_done)   # the shared expert's dx joins here
                self._waited = True
            f()
        self._waited = False
        for t in (x, dy):
            t.record_stream(side)
        return self.grads


class PipelinedMoE:
    """The layer over C chunks of tokens with one chunk's combine beside the next chunk's GEMMs.

    "EP / DeepEP explanation" page, section 7: cut the batch into chunks so that the dispatch
    and combine of one chunk overlap the expert computation of another (the pipelined time is
    about T_warm + sum over chunks of max(T_dispatch, T_experts, T_combine) + T_drain).  Here
    chunk c's router logits, route, layout and grouped GEMMs run on the caller's stream, and
    its combine on a second stream (default priority) once chunk c's down GEMM is done, while
    chunk c + 1's work starts on the first stream.  Each chunk is a MoELayer of N / C tokens
    over the same weights (bf16 layers); y is one [N, H] buffer, chunk c writing its rows.
    Routing is per token, so the result equals the unchunked layer's up to the tiles' row
    split (the same arithmetic per row).
    """

    def __init__(self, chunks: int, N: int, H: int, E: int, k: int, I: int, w13: torch.Tensor, w2: torch.Tensor,
                 shared_w13: Optional[torch.Tensor] = None, shared_w2: Optional[torch.Tensor] = None,
                 n_group: int = 0, topk_group: int = 0, bias: Optional[torch.Tensor] = None,
                 w_r: Optional[torch.Tensor] = None):
        if chunks < 1 or N % chunks:
            raise ValueError("N must split into equal chunks")
        self.N, self.H, self.chunks = N, H, chunks
        n = N // chunks
        dev = w13.device
        self.y = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
        self.parts = []
        for c in range(chunks):
            lay = MoELayer(n, H, E, k, I, "bf16", w13, w2, shared_w13, shared_w2, n_group, topk_group, bias,
                           w_r=w_r)
            lay.y = self.y[c * n:(c + 1) * n]   # (a contiguous block of rows)
            self.parts.append(lay)
        self.side = torch.cuda.Stream(device=dev)
        self.ready = [torch.cuda.Event() for _ in range(chunks)]
        self.done = torch.cuda.Event()

    def forward(self, x: torch.Tensor, z: Optional[torch.Tensor] = None) -> torch.Tensor:
        main = torch.cuda.current_stream(x.device)
        n = self.N // self.chunks
        self.side.wait_stream(main)
        for c, lay in enumerate(self.parts):
            xc = x[c * n:(c + 1) * n]
            zc = None if z is None else z[c * n:(c + 1) * n]
            if zc is None:
                zc = lay.router(xc)
            lay.route(zc)
            lay.dispatch()
            lay.permute(xc)
            lay.experts(xc)
            self.ready[c].record(main)
            self.side.wait_event(self.ready[c])
            with torch.cuda.stream(self.side):
                lay.combine()
        self.done.record(self.side)
        main.wait_event(self.done)
        x.record_stream(self.side)
        return self.y
