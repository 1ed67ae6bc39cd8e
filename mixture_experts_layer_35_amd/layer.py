"""Device-resident DeepSeekMoE layer: uploads weights once, owns the workspaces,
and calls ``moe_forward`` on each batch and ``moe_backward`` for its gradient.
Memory management only; the layer's arithmetic is entirely in libmoe's kernels.

For an e4m3 layer the bf16 master weights are uploaded and block-quantised on
the device by ``moe_quantize_weights_128x128`` (128 x 128 blocks, §3.3 of the
"DeepSeek-V3 Technical Report" page); the master copy is then released.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (MOE_BF16, MOE_E4M3, MOE_F32, MOE_WS_FORWARD, MoeShape, moe_backward,
               moe_backward_workspace_bytes, moe_forward, moe_quantize_weights_128x128,
               moe_transpose_expert_weights, moe_workspace_bytes)


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy float32 / bf16 bits (uint16) / int32 / uint8 -> device tensor of the same storage."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Inverse of to_device: bf16 comes back as uint16 bit patterns, e4m3 as uint8 codes."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def quantize_weights_128x128(w: torch.Tensor, stream=None):
    """[n, rows, cols] bf16/fp32 device tensor -> (e4m3 codes uint8, fp32 scales [n, rows/128, cols/128])."""
    n, rows, cols = w.shape
    q = torch.empty((n, rows, cols), dtype=torch.uint8, device=w.device)
    s = torch.empty((n, rows // 128, cols // 128), dtype=torch.float32, device=w.device)
    dt = MOE_BF16 if w.dtype == torch.bfloat16 else MOE_F32
    moe_quantize_weights_128x128(n, rows, cols, dt, w, q, s, stream)
    return q, s


class MoeLayer:
    def __init__(self, shape: MoeShape, gate_w, bias, routed_w, shared_w=None, routed_s=None, shared_s=None):
        self.shape = shape
        self.gate_w = gate_w
        self.bias = bias
        self.routed_w = tuple(routed_w)
        self.shared_w = tuple(shared_w) if shared_w is not None else None
        self.routed_s = tuple(routed_s) if routed_s is not None else None
        self.shared_s = tuple(shared_s) if shared_s is not None else None
        self._ws = None
        self._ws_T = -1
        self._bws = None
        self._bws_T = -1
        self._wt = None

    @classmethod
    def from_host(cls, shape: MoeShape, gate_w, bias, wg, wu, wd, swg=None, swu=None, swd=None, device="cuda"):
        """Upload host master weights (numpy); quantise them on the device when
        the shape's expert dtype is e4m3."""
        g = to_device(gate_w, device)
        b = to_device(np.asarray(bias, np.float32), device)
        fp8 = shape.w_dtype == MOE_E4M3

        def up(ws):
            if ws[0] is None:
                return None, None
            if not fp8:
                return tuple(to_device(w, device) for w in ws), None
            qs, ss = [], []
            for w in ws:
                dw = to_device(w, device)
                q, s = quantize_weights_128x128(dw)
                del dw
                qs.append(q)
                ss.append(s)
            return tuple(qs), tuple(ss)

        rw, rs = up((wg, wu, wd))
        sw, ss = up((swg, swu, swd))
        torch.cuda.synchronize()
        return cls(shape, g, b, rw, sw, rs, ss)

    def workspace(self, T: int) -> torch.Tensor:
        if self._ws is None or self._ws_T != T:
            self.shape.T = T
            n = moe_workspace_bytes(self.shape, MOE_WS_FORWARD)
            self._ws = torch.empty(max(n, 256), dtype=torch.uint8, device=self.gate_w.device)
            self._ws_T = T
        return self._ws

    def forward(self, u: torch.Tensor, out: torch.Tensor = None, topk_idx=None, topk_w=None, counts=None,
                scores=None, stream=None) -> torch.Tensor:
        T = u.shape[0]
        ws = self.workspace(T)
        self.shape.T = T
        if out is None:
            out = torch.empty((T, self.shape.d), dtype=u.dtype, device=u.device)
        moe_forward(self.shape, u, self.gate_w, self.bias, self.routed_w, self.routed_s, self.shared_w,
                    self.shared_s, out, topk_idx, topk_w, counts, scores, ws, stream)
        return out

    # ---- backward -----------------------------------------------------------

    def transposed_weights(self, stream=None):
        """(routed, shared) transposed copies ((W_down^T [n, I, d], [W_gate^T | W_up^T] [n, d, 2I]),
        e4m3 block scales or None) that the backward reads; built on first use.  Call
        drop_transposed() after changing the weights."""
        if self._wt is None:
            d, I = self.shape.d, self.shape.inter
            fp8 = self.shape.w_dtype == MOE_E4M3

            def tr(ws, ss):
                if ws is None:
                    return None, None
                wg, wu, wd = ws
                n = wg.shape[0]
                wdt = torch.empty((n, I, d), dtype=wd.dtype, device=wd.device)
                wgut = torch.empty((n, d, 2 * I), dtype=wg.dtype, device=wg.device)
                st = None
                if fp8:
                    st = (torch.empty((n, I // 128, d // 128), dtype=torch.float32, device=wd.device),
                          torch.empty((n, d // 128, 2 * I // 128), dtype=torch.float32, device=wd.device))
                moe_transpose_expert_weights(self.shape, n, ws, ss, (wdt, wgut), st, stream)
                return (wdt, wgut), st

            self._wt = (tr(self.routed_w, self.routed_s), tr(self.shared_w, self.shared_s))
        return self._wt

    def drop_transposed(self):
        self._wt = None

    def backward(self, u: torch.Tensor, dout: torch.Tensor, du: torch.Tensor = None, dgate_w=None, d_routed_w=None,
                 d_shared_w=None, dtopk_w=None, stream=None) -> torch.Tensor:
        """Gradients for the most recent forward(u) (its workspace holds the saved
        activations, so no other forward may run in between).  du is returned;
        dgate_w [N_r, d] fp32, d_routed_w / d_shared_w (dW_gate, dW_up, dW_down) and
        dtopk_w [T, K] fp32 are filled when given."""
        T = u.shape[0]
        if self._ws is None or self._ws_T != T:
            raise ValueError("backward needs the workspace of a forward call on the same batch")
        (rt, rts), (st, sts) = self.transposed_weights(stream)
        self.shape.T = T
        if self._bws is None or self._bws_T != T:
            n = moe_backward_workspace_bytes(self.shape)
            self._bws = torch.empty(max(n, 256), dtype=torch.uint8, device=u.device)
            self._bws_T = T
        if du is None:
            du = torch.empty((T, self.shape.d), dtype=u.dtype, device=u.device)
        moe_backward(self.shape, u, self.gate_w, self.routed_w, self.routed_s, rt, rts, self.shared_w, self.shared_s,
                     st, sts, self._ws, dout, du, dgate_w, d_routed_w, d_shared_w, dtopk_w, self._bws, stream)
        return du
