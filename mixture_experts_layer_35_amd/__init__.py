"""Python binding of libmoe, the MI355X (gfx950) DeepSeekMoE layer library.

Argument marshalling only: every function below has the name and argument
order of the C entry point declared in ``include/moe.h`` and forwards torch
device tensors as raw pointers.  All computation happens in the HIP kernels of
``libmoe.so``; there is no fallback path.  PyTorch provides device memory and
the current stream.

Build the library with ``python -m mixture_experts_layer_35_amd.build`` (or
``__graft_entry__.build()``); using any entry point without it raises
``MoeError``.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH names another build of the same sources (the sanitizer tier's
# host-instrumented library); the default is the in-tree libmoe.so
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_E4M3 = 0, 1, 2
MOE_ADD_RESIDUAL = 1
MOE_SAVE_SWIGLU_INPUTS = 2   # moe_forward keeps the SwiGLU inputs for moe_backward
MOE_WS_ROUTE, MOE_WS_PERMUTE, MOE_WS_FORWARD = 0, 1, 2
MOE_STATIC_WS_BYTES = 64 << 20   # the library's own forward workspace per GPU (moe_forward_static)

EXPORTED = ("moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_forward", "moe_forward_timed",
            "moe_forward_static",
            "moe_workspace_bytes",
            "moe_ffn_workspace_bytes", "moe_bias_update", "moe_seq_balance", "moe_seq_balance_workspace_bytes",
            "moe_transpose_expert_weights", "moe_backward", "moe_backward_timed", "moe_backward_workspace_bytes",
            "moe_quantize_1x128", "moe_quantize_weights_128x128", "moe_quantize_128x1", "moe_last_error",
            "moe_version")


class MoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (status %d)" % (msg, code))
        self.code = code


class MoeShape(ctypes.Structure):
    """Mirror of ``moe_shape`` (include/moe.h)."""
    _fields_ = [
        ("T", ctypes.c_int64), ("d", ctypes.c_int32), ("n_routed", ctypes.c_int32), ("n_shared", ctypes.c_int32),
        ("n_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("inter", ctypes.c_int32), ("act_dtype", ctypes.c_int32), ("router_dtype", ctypes.c_int32),
        ("w_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32), ("quant_block", ctypes.c_int32),
        ("routed_scale", ctypes.c_float), ("flags", ctypes.c_uint32),
    ]


def make_shape(T, d, n_routed, n_shared, n_groups, topk_groups, topk, inter, dtype="bf16", routed_scale=1.0,
               flags=0) -> MoeShape:
    """dtype: "fp32", "bf16" or "fp8" (bf16 u, e4m3 expert GEMMs, bf16 out)."""
    act = MOE_F32 if dtype == "fp32" else MOE_BF16
    w = MOE_E4M3 if dtype == "fp8" else act
    return MoeShape(T, d, n_routed, n_shared, n_groups, topk_groups, topk, inter, act, act, w, act, 128,
                    routed_scale, flags)


_lock = threading.Lock()
_lib = None


def lib():
    """The loaded libmoe.so (raises MoeError when it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise MoeError(MOE_ERR_HIP, "libmoe.so is not built (run __graft_entry__.build())")
            L = ctypes.CDLL(LIB_PATH)
            P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
            S = ctypes.POINTER(MoeShape)
            sig = {
                "moe_route": [S, P, P, P, P, P, P, P, P, sz, P],
                "moe_permute": [S, P, P, P, P, P, P, P, P, P, sz, P],
                "moe_grouped_ffn": [S, i32, P, i64, P, P, P, P, P, P, P, P, P, sz, P],
                "moe_combine": [S, P, P, P, P, P, P, P],
                "moe_forward": [S, P, P, P, P, P, P, P, P, P, P, P, P, P, sz, P],
                "moe_forward_timed": [S, P, P, P, P, P, P, P, P, P, P, P, P, P, sz, P, P],
                "moe_forward_static": [S, P, P, P, P, P, P, P, P, P, P, P, P, P],
                "moe_bias_update": [S, P, P, ctypes.c_float, P],
                "moe_seq_balance": [S, P, P, i64, ctypes.c_float, P, P, P, P, sz, P],
                "moe_transpose_expert_weights": [S, i32, P, P, P, P, P],
                "moe_backward": [S, P, P, P, P, P, P, P, P, P, P, P, sz, P, P, P, P, P, P, P, sz, P],
                "moe_backward_timed": [S, P, P, P, P, P, P, P, P, P, P, P, sz, P, P, P, P, P, P, P, sz, P, P],
                "moe_quantize_1x128": [i64, i32, i32, P, P, P, P],
                "moe_quantize_weights_128x128": [i64, i32, i32, i32, P, P, P, P],
                "moe_quantize_128x1": [i32, P, i64, i32, i32, P, P, P, P, P, P, P],
            }
            for name, args in sig.items():
                f = getattr(L, name)
                f.argtypes = args
                f.restype = ctypes.c_int
            L.moe_workspace_bytes.argtypes = [S, ctypes.c_int]
            L.moe_workspace_bytes.restype = sz
            L.moe_ffn_workspace_bytes.argtypes = [S, i64]
            L.moe_ffn_workspace_bytes.restype = sz
            L.moe_seq_balance_workspace_bytes.argtypes = [S, i64]
            L.moe_seq_balance_workspace_bytes.restype = sz
            L.moe_backward_workspace_bytes.argtypes = [S]
            L.moe_backward_workspace_bytes.restype = sz
            L.moe_last_error.argtypes = []
            L.moe_last_error.restype = ctypes.c_char_p
            L.moe_version.argtypes = []
            L.moe_version.restype = ctypes.c_char_p
            _lib = L
    return _lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(x):
    """Device pointer of a tensor (or an int address, or None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(ws):
    if ws is None:
        return 0
    return ws.numel() * ws.element_size()


def _ptr_array(items):
    if items is None:
        return None
    arr = (ctypes.c_void_p * 3)(*[_ptr(x) for x in items])
    return ctypes.cast(arr, ctypes.c_void_p), arr          # keep arr alive with the cast


def _check(rc):
    if rc != MOE_OK:
        raise MoeError(rc, lib().moe_last_error().decode())
    return rc


# ---------------------------------------------------------------------------
# entry points (include/moe.h)
# ---------------------------------------------------------------------------

def moe_version() -> str:
    return lib().moe_version().decode()


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_workspace_bytes(shape: MoeShape, which: int) -> int:
    n = lib().moe_workspace_bytes(ctypes.byref(shape), which)
    if n == 0 and shape.T > 0:
        err = moe_last_error()
        if err:
            raise MoeError(MOE_ERR_UNSUPPORTED, err)
    return n


def moe_ffn_workspace_bytes(shape: MoeShape, max_rows: int) -> int:
    return lib().moe_ffn_workspace_bytes(ctypes.byref(shape), max_rows)


def moe_route(shape, u, gate_w, bias, scores_in, scores_out, topk_idx, topk_w, ws=None, stream=None):
    return _check(lib().moe_route(ctypes.byref(shape), _ptr(u), _ptr(gate_w), _ptr(bias), _ptr(scores_in),
                                  _ptr(scores_out), _ptr(topk_idx), _ptr(topk_w), _ptr(ws), _nbytes(ws),
                                  _stream(stream)))


def moe_permute(shape, topk_idx, u, counts, offsets, perm_token, inv_perm, x_perm, x_scales, ws, stream=None):
    return _check(lib().moe_permute(ctypes.byref(shape), _ptr(topk_idx), _ptr(u), _ptr(counts), _ptr(offsets),
                                    _ptr(perm_token), _ptr(inv_perm), _ptr(x_perm), _ptr(x_scales), _ptr(ws),
                                    _nbytes(ws), _stream(stream)))


def moe_grouped_ffn(shape, n_exp, offsets, max_rows, gather, x, x_scales, w_gate, w_up, w_down, w_scales, y, ws,
                    stream=None):
    ws_arr = _ptr_array(w_scales)
    return _check(lib().moe_grouped_ffn(ctypes.byref(shape), n_exp, _ptr(offsets), max_rows, _ptr(gather), _ptr(x),
                                        _ptr(x_scales), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                        ws_arr[0] if ws_arr else None, _ptr(y), _ptr(ws), _nbytes(ws),
                                        _stream(stream)))


def moe_combine(shape, y_perm, inv_perm, topk_w, y_shared, residual, out, stream=None):
    return _check(lib().moe_combine(ctypes.byref(shape), _ptr(y_perm), _ptr(inv_perm), _ptr(topk_w), _ptr(y_shared),
                                    _ptr(residual), _ptr(out), _stream(stream)))


def moe_forward(shape, u, gate_w, bias, routed_w, routed_s, shared_w, shared_s, out, topk_idx_out=None,
                topk_w_out=None, counts_out=None, scores_out=None, ws=None, stream=None):
    rw, rs, sw, ss = (_ptr_array(x) for x in (routed_w, routed_s, shared_w, shared_s))
    return _check(lib().moe_forward(ctypes.byref(shape), _ptr(u), _ptr(gate_w), _ptr(bias), rw[0] if rw else None,
                                    rs[0] if rs else None, sw[0] if sw else None, ss[0] if ss else None, _ptr(out),
                                    _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(counts_out), _ptr(scores_out),
                                    _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_forward_static(shape, u, gate_w, bias, routed_w, routed_s, shared_w, shared_s, out, topk_idx_out=None,
                       topk_w_out=None, counts_out=None, scores_out=None, stream=None):
    """moe_forward with the library's own per-GPU workspace (no caller workspace)."""
    rw, rs, sw, ss = (_ptr_array(x) for x in (routed_w, routed_s, shared_w, shared_s))
    return _check(lib().moe_forward_static(ctypes.byref(shape), _ptr(u), _ptr(gate_w), _ptr(bias),
                                           rw[0] if rw else None, rs[0] if rs else None, sw[0] if sw else None,
                                           ss[0] if ss else None, _ptr(out), _ptr(topk_idx_out), _ptr(topk_w_out),
                                           _ptr(counts_out), _ptr(scores_out), _stream(stream)))


def moe_forward_timed(shape, u, gate_w, bias, routed_w, routed_s, shared_w, shared_s, out, topk_idx_out=None,
                      topk_w_out=None, counts_out=None, scores_out=None, ws=None, stream=None, stage_events=None):
    """stage_events: 6 raw hipEvent_t handles (ints) or None."""
    rw, rs, sw, ss = (_ptr_array(x) for x in (routed_w, routed_s, shared_w, shared_s))
    ev = None
    if stage_events is not None:
        arr = (ctypes.c_void_p * 6)(*stage_events)
        ev = ctypes.cast(arr, ctypes.c_void_p)
    return _check(lib().moe_forward_timed(ctypes.byref(shape), _ptr(u), _ptr(gate_w), _ptr(bias),
                                          rw[0] if rw else None, rs[0] if rs else None, sw[0] if sw else None,
                                          ss[0] if ss else None, _ptr(out), _ptr(topk_idx_out), _ptr(topk_w_out),
                                          _ptr(counts_out), _ptr(scores_out), _ptr(ws), _nbytes(ws),
                                          _stream(stream), ev))


def moe_bias_update(shape, counts, bias, gamma, stream=None):
    return _check(lib().moe_bias_update(ctypes.byref(shape), _ptr(counts), _ptr(bias), gamma, _stream(stream)))


def moe_seq_balance_workspace_bytes(shape: MoeShape, seq_len: int) -> int:
    return lib().moe_seq_balance_workspace_bytes(ctypes.byref(shape), seq_len)


def moe_seq_balance(shape, scores, topk_idx, seq_len, alpha, loss, counts=None, share=None, ws=None, stream=None):
    return _check(lib().moe_seq_balance(ctypes.byref(shape), _ptr(scores), _ptr(topk_idx), seq_len, alpha, _ptr(loss),
                                        _ptr(counts), _ptr(share), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_transpose_expert_weights(shape, n, w, w_s, wt, wt_s, stream=None):
    """w = (W_gate, W_up, W_down); wt = (W_down^T, [W_gate^T | W_up^T]); w_s / wt_s: the e4m3
    block scales (3 and 2 arrays) or None."""
    a, b, c, e = (_ptr_array(x) for x in (w, w_s, wt, wt_s))
    return _check(lib().moe_transpose_expert_weights(ctypes.byref(shape), n, a[0] if a else None,
                                                     b[0] if b else None, c[0] if c else None, e[0] if e else None,
                                                     _stream(stream)))


def moe_backward_workspace_bytes(shape: MoeShape) -> int:
    return lib().moe_backward_workspace_bytes(ctypes.byref(shape))


def _bwd_args(shape, u, gate_w, routed_w, routed_s, routed_wt, routed_wt_s, shared_w, shared_s, shared_wt,
              shared_wt_s, fwd_ws, dout, du, dgate_w, d_routed_w, d_shared_w, dtopk_w, ws, stream):
    arrs = [_ptr_array(x) for x in (routed_w, routed_s, routed_wt, routed_wt_s, shared_w, shared_s, shared_wt,
                                    shared_wt_s, d_routed_w, d_shared_w)]
    keep = [x for x in arrs if x]
    p = [x[0] if x else None for x in arrs]
    return keep, (ctypes.byref(shape), _ptr(u), _ptr(gate_w), p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7],
                  _ptr(fwd_ws), _nbytes(fwd_ws), _ptr(dout), _ptr(du), _ptr(dgate_w), p[8], p[9], _ptr(dtopk_w),
                  _ptr(ws), _nbytes(ws), _stream(stream))


def moe_backward(shape, u, gate_w, routed_w, routed_s, routed_wt, routed_wt_s, shared_w, shared_s, shared_wt,
                 shared_wt_s, fwd_ws, dout, du, dgate_w=None, d_routed_w=None, d_shared_w=None, dtopk_w=None, ws=None,
                 stream=None):
    """routed_w / shared_w: (W_gate, W_up, W_down); *_wt: (W_down^T, [W_gate^T | W_up^T]); *_s / *_wt_s: the
    e4m3 block scales or None; fwd_ws: the workspace tensor of the forward call whose output dout refers to."""
    keep, args = _bwd_args(shape, u, gate_w, routed_w, routed_s, routed_wt, routed_wt_s, shared_w, shared_s,
                           shared_wt, shared_wt_s, fwd_ws, dout, du, dgate_w, d_routed_w, d_shared_w, dtopk_w, ws,
                           stream)
    rc = lib().moe_backward(*args)
    del keep
    return _check(rc)


def moe_backward_timed(shape, u, gate_w, routed_w, routed_s, routed_wt, routed_wt_s, shared_w, shared_s, shared_wt,
                       shared_wt_s, fwd_ws, dout, du, dgate_w=None, d_routed_w=None, d_shared_w=None, dtopk_w=None,
                       ws=None, stream=None, stage_events=None):
    """stage_events: 10 raw hipEvent_t handles (ints) or None."""
    keep, args = _bwd_args(shape, u, gate_w, routed_w, routed_s, routed_wt, routed_wt_s, shared_w, shared_s,
                           shared_wt, shared_wt_s, fwd_ws, dout, du, dgate_w, d_routed_w, d_shared_w, dtopk_w, ws,
                           stream)
    ev = None
    if stage_events is not None:
        arr = (ctypes.c_void_p * 10)(*stage_events)
        ev = ctypes.cast(arr, ctypes.c_void_p)
    rc = lib().moe_backward_timed(*args, ev)
    del keep
    return _check(rc)


def moe_quantize_1x128(rows, cols, x_dtype, x, q, s, stream=None):
    return _check(lib().moe_quantize_1x128(rows, cols, x_dtype, _ptr(x), _ptr(q), _ptr(s), _stream(stream)))


def moe_quantize_128x1(n_seg, offsets, max_rows, cols, x_dtype, x, x_s, gather, q, s, block_base, stream=None):
    return _check(lib().moe_quantize_128x1(n_seg, _ptr(offsets), max_rows, cols, x_dtype, _ptr(x), _ptr(x_s),
                                           _ptr(gather), _ptr(q), _ptr(s), _ptr(block_base), _stream(stream)))


def moe_quantize_weights_128x128(nmat, rows, cols, w_dtype, w, q, s, stream=None):
    return _check(lib().moe_quantize_weights_128x128(nmat, rows, cols, w_dtype, _ptr(w), _ptr(q), _ptr(s),
                                                     _stream(stream)))
