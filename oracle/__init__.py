"""CPU oracle for the DeepSeekMoE layer forward pass (numpy front end).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU library never imports this
package, and this package never imports the GPU library.

The arithmetic lives in ``moe_oracle.c`` (plain loops, fp64 sums, one rounding
per stored value); this module only builds it with gcc, marshals numpy arrays
and documents each entry point.  Citations are to the "DeepSeek-V3 Technical
Report" page (papers-reader rewrite): §2.1.2 (DeepSeekMoE, auxiliary-loss-free
balancing, node-limited routing), §3.3 (fine-grained FP8 quantisation), §4.2
(hyper-parameters).

Parity pins for every function are in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

F32, BF16, E4M3, F64 = 0, 1, 2, 3
ADD_RESIDUAL = 1
NC = 128

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
# MOE_ORACLE_LIB names another build of moe_oracle.c to load (the sanitizer
# tier's AddressSanitizer / UndefinedBehaviorSanitizer build)
_LIB = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(out: str) -> str:
    """Compile moe_oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer
    (gcc; any report aborts) into ``out``; load it by running a process with
    MOE_ORACLE_LIB=out and gcc's libasan preloaded."""
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared", "-fPIC", _SRC,
           "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            i64, i32, f32, u32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_uint
            lib.oracle_round_format.restype = ctypes.c_double
            lib.oracle_round_format.argtypes = [ctypes.c_double, i32, i32, ctypes.c_double, i32]
            lib.oracle_round_bf16.restype = ctypes.c_double
            lib.oracle_round_bf16.argtypes = [ctypes.c_double]
            lib.oracle_encode_bf16.restype = ctypes.c_uint16
            lib.oracle_encode_bf16.argtypes = [ctypes.c_double]
            lib.oracle_round_e4m3.restype = ctypes.c_double
            lib.oracle_round_e4m3.argtypes = [ctypes.c_double]
            lib.oracle_encode_e4m3.restype = ctypes.c_uint8
            lib.oracle_encode_e4m3.argtypes = [ctypes.c_double]
            lib.oracle_decode_e4m3.restype = ctypes.c_double
            lib.oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
            lib.oracle_quant_1x128.restype = None
            lib.oracle_quant_1x128.argtypes = [i64, i32, i32, P, P, P]
            lib.oracle_quant_128x128.restype = None
            lib.oracle_quant_128x128.argtypes = [i64, i32, i32, i32, P, P, P]
            lib.oracle_route.restype = i32
            lib.oracle_route.argtypes = [i64, P, i32, i32, i32, i32, i32, i32, P, i32, P, P, P, P, P, P, f32]
            lib.oracle_permute.restype = None
            lib.oracle_permute.argtypes = [i64, i32, i32, P, P, P, P, P]
            lib.oracle_grouped_ffn.restype = i32
            lib.oracle_grouped_ffn.argtypes = [i32, P, i64, P, i32, i32, i32, P, P, i32, P, P, P, P, P, P,
                                               i32, i32, P]
            lib.oracle_combine.restype = None
            lib.oracle_combine.argtypes = [i64, P, i64, i32, i32, i32, i32, P, P, P, P, i32, P, P]
            lib.oracle_moe_forward.restype = i32
            lib.oracle_moe_forward.argtypes = ([i64, P, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, f32, u32]
                                               + [P] * 4 + [P] * 6 + [P] * 6 + [P] * 4)
            lib.oracle_bias_update.restype = None
            lib.oracle_bias_update.argtypes = [i32, i64, i32, P, P, f32]
            lib.oracle_layer_f64.restype = i32
            f64 = ctypes.c_double
            lib.oracle_layer_f64.argtypes = [i64, i32, i32, i32, i32, i32, i32, P, P, P, i32] + [P] * 6 + [f64, P, P]
            lib.oracle_moe_backward_f64.restype = i32
            lib.oracle_moe_backward_f64.argtypes = ([i64, i32, i32, i32, i32, i32, i32, P, P, P, i32] + [P] * 6
                                                    + [f64, P, i64, P, i32, P] + [P] * 9)
            lib.oracle_quant_128x1.restype = None
            lib.oracle_quant_128x1.argtypes = [i32, P, i32, i32, P, P, P, P, P]
            lib.oracle_moe_backward_fp8.restype = i32
            lib.oracle_moe_backward_fp8.argtypes = ([i64, i32, i32, i32, i32, i32, P, P, P] + [P] * 12
                                                    + [f64, P, i64, P, i32, P] + [P] * 9)
            lib.oracle_seq_balance.restype = None
            lib.oracle_seq_balance.argtypes = [i64, i32, i32, P, P, i64, f32, P, P, P]
            lib.oracle_num_threads.restype = i32
            lib.oracle_num_threads.argtypes = []
            _lib = lib
    return _lib


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------

def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def _storage(a):
    """Return (dtype code, contiguous array) for a float32 or bf16 array.
    bf16 arrays are carried as uint16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return F32, a
    if a.dtype == np.uint16:
        return BF16, a
    if a.dtype == np.float64:
        return F64, a
    raise TypeError("oracle inputs are float32, float64 or bf16 bit patterns (uint16), got %s" % a.dtype)


def _empty_like_code(code, shape):
    return np.empty(shape, dtype=np.float32 if code == F32 else np.uint16)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


# ----------------------------------------------------------------------------
# formats (§3.3 storage formats; bf16 as in the mixed-precision framework)
# ----------------------------------------------------------------------------

def round_format(x: float, p: int, emin: int, maxfin: float, sat: bool = False) -> float:
    return _load().oracle_round_format(float(x), p, emin, float(maxfin), int(sat))


def round_bf16(x: float) -> float:
    return _load().oracle_round_bf16(float(x))


def encode_bf16(x: float) -> int:
    return int(_load().oracle_encode_bf16(float(x)))


def round_e4m3(x: float) -> float:
    return _load().oracle_round_e4m3(float(x))


def encode_e4m3(x: float) -> int:
    return int(_load().oracle_encode_e4m3(float(x)))


def decode_e4m3(c: int) -> float:
    return _load().oracle_decode_e4m3(int(c))


def quant_1x128(x):
    """1 x 128 activation tiles (§3.3).  x: [rows, cols] float32 or bf16 bits.
    Returns (q uint8 [rows, cols], scales float32 [rows, cols/128])."""
    code, x = _storage(x)
    rows, cols = x.shape
    assert cols % NC == 0
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // NC), np.float32)
    _load().oracle_quant_1x128(rows, cols, code, _p(x), _p(q), _p(s))
    return q, s


def quant_128x128(w):
    """128 x 128 weight blocks (§3.3).  w: [n, rows, cols] float32 or bf16 bits.
    Returns (q uint8 [n, rows, cols], scales float32 [n, rows/128, cols/128])."""
    code, w = _storage(w)
    n, rows, cols = w.shape
    assert rows % NC == 0 and cols % NC == 0
    q = np.empty(w.shape, np.uint8)
    s = np.empty((n, rows // NC, cols // NC), np.float32)
    _load().oracle_quant_128x128(n, rows, cols, code, _p(w), _p(q), _p(s))
    return q, s


# ----------------------------------------------------------------------------
# routing, dispatch, FFN, combine, bias update (§2.1.2)
# ----------------------------------------------------------------------------

def route(u, gate_w, bias, *, G, Mg, K, scores_in=None, tokens=None, routed_scale=1.0):
    """Affinities, group-limited biased top-K selection and normalised gates.

    Returns (scores [n, Nr] fp32, topk_idx [n, K] int32, topk_w [n, K] fp32)
    for the listed tokens (all tokens when ``tokens`` is None).  ``scores_in``
    ([T, Nr] fp32) replaces the computed affinities (u and gate_w may then be
    None)."""
    lib = _load()
    bias = _c(bias, np.float32)
    Nr = bias.shape[0]
    if scores_in is not None:
        scores_in = _c(scores_in, np.float32)
        T = scores_in.shape[0]
        d = 0
        ucode = wcode = F32
    else:
        ucode, u = _storage(u)
        wcode, gate_w = _storage(gate_w)
        T, d = u.shape
    tok = None if tokens is None else _c(tokens, np.int64)
    n = T if tok is None else tok.shape[0]
    scores = np.empty((n, Nr), np.float32)
    idx = np.empty((n, K), np.int32)
    w = np.empty((n, K), np.float32)
    rc = lib.oracle_route(n, _p(tok), d, Nr, G, Mg, K, ucode, _p(u) if scores_in is None else None, wcode,
                          _p(gate_w) if scores_in is None else None, _p(bias), _p(scores_in), _p(scores),
                          _p(idx), _p(w), routed_scale)
    if rc:
        raise ValueError("oracle_route: unsupported shape (rc=%d)" % rc)
    return scores, idx, w


def permute(topk_idx, Nr):
    """counts [Nr], offsets [Nr+1], perm_token [T*K], inv_perm [T*K] (int32)."""
    idx = _c(topk_idx, np.int32)
    T, K = idx.shape
    counts = np.empty(Nr, np.int32)
    offsets = np.empty(Nr + 1, np.int32)
    perm = np.empty(T * K, np.int32)
    inv = np.empty(T * K, np.int32)
    _load().oracle_permute(T, K, Nr, _p(idx), _p(counts), _p(offsets), _p(perm), _p(inv))
    return counts, offsets, perm, inv


def grouped_ffn(offsets, x, wg, wu, wd, *, rows, x_scales=None, w_scales=None, w_code=None,
                h_code=None, y_code=None):
    """SwiGLU experts on the listed rows of x.

    x: [R, d] float32 / bf16 bits, or uint8 e4m3 with ``x_scales`` [R, d/128].
    wg, wu: [n, I, d]; wd: [n, d, I] (float32, bf16 bits, or uint8 with
    ``w_scales`` = (sg, su, sd)).  Returns y [len(rows), d] in ``y_code``."""
    offsets = _c(offsets, np.int32)
    rows = _c(rows, np.int64)
    n_exp = offsets.shape[0] - 1
    if x.dtype == np.uint8:
        xcode, x = E4M3, np.ascontiguousarray(x)
        x_scales = _c(x_scales, np.float32)
    else:
        xcode, x = _storage(x)
    if wg.dtype == np.uint8:
        wcode = E4M3
        wg, wu, wd = (np.ascontiguousarray(a) for a in (wg, wu, wd))
        sg, su, sd = (_c(s, np.float32) for s in w_scales)
    else:
        wcode, wg = _storage(wg)
        _, wu = _storage(wu)
        _, wd = _storage(wd)
        sg = su = sd = None
    _, I, d = wg.shape
    if h_code is None:
        h_code = E4M3 if wcode == E4M3 else xcode
    if y_code is None:
        y_code = F32 if xcode == F32 else BF16
    y = _empty_like_code(y_code, (rows.shape[0], d))
    rc = _load().oracle_grouped_ffn(n_exp, _p(offsets), rows.shape[0], _p(rows), d, I, xcode, _p(x), _p(x_scales),
                                    wcode, _p(wg), _p(wu), _p(wd), _p(sg), _p(su), _p(sd), h_code, y_code, _p(y))
    if rc:
        raise ValueError("oracle_grouped_ffn: row outside every expert")
    return y


def combine(y_perm, inv_perm, topk_w, *, T, y_shared=None, residual=None, tokens=None):
    """Gate-weighted sum of routed outputs plus shared outputs (+ residual).
    y_perm [T*K, d], y_shared [Ns, T, d] (or None), residual [T, d] (or None),
    all float32 or bf16 bits.  Returns out [n, d] in y_perm's storage."""
    ycode, y_perm = _storage(y_perm)
    inv = _c(inv_perm, np.int32)
    w = _c(topk_w, np.float32)
    K = w.shape[1]
    d = y_perm.shape[1]
    Ns = 0
    if y_shared is not None:
        _, y_shared = _storage(y_shared)
        y_shared = y_shared.reshape(-1, T, d)
        Ns = y_shared.shape[0]
    ucode = F32
    if residual is not None:
        ucode, residual = _storage(residual)
    tok = None if tokens is None else _c(tokens, np.int64)
    n = T if tok is None else tok.shape[0]
    out = _empty_like_code(ycode, (n, d))
    _load().oracle_combine(n, _p(tok), T, d, K, Ns, ycode, _p(y_perm), _p(inv), _p(w), _p(y_shared), ucode,
                           _p(residual), _p(out))
    return out


def moe_forward(u, gate_w, bias, routed, shared, *, G, Mg, K, w_code, out_code, tokens=None,
                scores_in=None, routed_scales=None, shared_scales=None, routed_scale=1.0, flags=0):
    """The whole layer for the listed tokens.

    routed = (wg [Nr,I,d], wu [Nr,I,d], wd [Nr,d,I]); shared = same with Ns
    (or None).  For E4M3 the weights are uint8 codes with 128 x 128 scales in
    routed_scales / shared_scales; u is then quantised per 1 x 128 tile here.
    Returns (out [n, d], topk_idx [n, K], topk_w [n, K], scores [n, Nr])."""
    acode, u = _storage(u)
    _, gate_w = _storage(gate_w)
    bias = _c(bias, np.float32)
    T, d = u.shape
    Nr = bias.shape[0]
    if w_code == E4M3:
        rg, ru, rd = (np.ascontiguousarray(a, dtype=np.uint8) for a in routed)
        rsg, rsu, rsd = (_c(s, np.float32) for s in routed_scales)
    else:
        rg, ru, rd = (np.ascontiguousarray(a) for a in routed)
        rsg = rsu = rsd = None
    I = rg.shape[1]
    Ns = 0
    sg = su = sd = ssg = ssu = ssd = None
    if shared is not None:
        sg, su, sd = (np.ascontiguousarray(a) for a in shared)
        Ns = sg.shape[0]
        if w_code == E4M3:
            ssg, ssu, ssd = (_c(s, np.float32) for s in shared_scales)
    tok = None if tokens is None else _c(tokens, np.int64)
    n = T if tok is None else tok.shape[0]
    if scores_in is not None:
        scores_in = _c(scores_in, np.float32)
    out = _empty_like_code(out_code, (n, d))
    idx = np.empty((n, K), np.int32)
    w = np.empty((n, K), np.float32)
    scores = np.empty((n, Nr), np.float32)
    rc = _load().oracle_moe_forward(n, _p(tok), d, Nr, Ns, G, Mg, K, I, acode, w_code, out_code, routed_scale,
                                    flags, _p(u), _p(gate_w), _p(bias), _p(scores_in),
                                    _p(rg), _p(ru), _p(rd), _p(rsg), _p(rsu), _p(rsd),
                                    _p(sg), _p(su), _p(sd), _p(ssg), _p(ssu), _p(ssd),
                                    _p(out), _p(idx), _p(w), _p(scores))
    if rc:
        raise ValueError("oracle_moe_forward failed (rc=%d)" % rc)
    return out, idx, w, scores


def bias_update(counts, bias, T, K, gamma=0.001):
    """One auxiliary-loss-free bias step (§2.1.2, gamma from §4.2).  Returns
    the new bias (float32 copy)."""
    counts = _c(counts, np.int32)
    b = np.array(bias, dtype=np.float32, copy=True)
    _load().oracle_bias_update(b.shape[0], T, K, _p(counts), _p(b), gamma)
    return b


def _layer_args(u, gate_w, topk_idx, routed, shared):
    au, u = _storage(u)
    ag, gate_w = _storage(gate_w)
    if au != ag:
        raise TypeError("u and gate_w must share a storage format")
    topk_idx = _c(topk_idx, np.int32)
    ws = [_storage(w) for w in routed] + ([_storage(w) for w in shared] if shared is not None else [])
    codes = {c for c, _ in ws}
    if len(codes) != 1:
        raise TypeError("expert weights must share a storage format")
    T, d = u.shape
    Nr = gate_w.shape[0]
    I = routed[0].shape[1]
    Ns = shared[0].shape[0] if shared is not None else 0
    K = topk_idx.shape[1]
    arrs = [w for _, w in ws] + [None] * (6 - len(ws))
    return T, d, Nr, Ns, K, I, au, u, gate_w, topk_idx, codes.pop(), arrs


def layer_f64(u, gate_w, topk_idx, routed, shared, routed_scale=1.0):
    """The layer with nothing rounded after decoding the inputs, for a fixed
    selection topk_idx (§2.1.2): returns (out [T, d] float64, gates [T, K]
    float64).  Inputs in float32, bf16 bits or float64."""
    T, d, Nr, Ns, K, I, au, u, gate_w, idx, wc, arrs = _layer_args(u, gate_w, topk_idx, routed, shared)
    out = np.empty((T, d), np.float64)
    g = np.empty((T, K), np.float64)
    rc = _load().oracle_layer_f64(T, d, Nr, Ns, K, I, au, _p(u), _p(gate_w), _p(idx), wc, *[_p(a) for a in arrs],
                                  routed_scale,
                                  _p(out), _p(g))
    if rc:
        raise ValueError("oracle_layer_f64 rc=%d" % rc)
    return out, g


def moe_backward(u, gate_w, topk_idx, routed, shared, dout, tokens=None, experts=None, dgate=True, dshared=True,
                 routed_scale=1.0):
    """Gradient of sum(dout * layer(...)) by the chain rule in fp64 for a fixed
    selection (see layer_f64).  Returns a dict with
      du [T, d] and dg [T, K] (rows of the listed tokens; others zero),
      dgate_w [Nr, d] (if dgate), dwg/dwu/dwd [len(experts) or Nr, ...] for the
      listed routed experts, dswg/dswu/dswd [Ns, ...] (if dshared)."""
    T, d, Nr, Ns, K, I, au, u, gate_w, idx, wc, arrs = _layer_args(u, gate_w, topk_idx, routed, shared)
    dout = _c(dout, np.float64)
    tok = None if tokens is None else _c(tokens, np.int64)
    exps = None if experts is None else _c(experts, np.int32)
    ne = Nr if exps is None else exps.shape[0]
    r = dict(du=np.zeros((T, d)), dg=np.zeros((T, K)),
             dgate_w=np.empty((Nr, d)) if dgate else None,
             dwg=np.empty((ne, I, d)), dwu=np.empty((ne, I, d)), dwd=np.empty((ne, d, I)),
             dswg=np.empty((Ns, I, d)) if dshared and Ns else None,
             dswu=np.empty((Ns, I, d)) if dshared and Ns else None,
             dswd=np.empty((Ns, d, I)) if dshared and Ns else None)
    rc = _load().oracle_moe_backward_f64(T, d, Nr, Ns, K, I, au, _p(u), _p(gate_w), _p(idx), wc,
                                         *[_p(a) for a in arrs], routed_scale, _p(dout), 0 if tok is None else tok.shape[0],
                                         _p(tok), 0 if exps is None else exps.shape[0], _p(exps),
                                         _p(r["du"]), _p(r["dg"]), _p(r["dgate_w"]), _p(r["dwg"]), _p(r["dwu"]),
                                         _p(r["dwd"]), _p(r["dswg"]), _p(r["dswu"]), _p(r["dswd"]))
    if rc:
        raise ValueError("oracle_moe_backward_f64 rc=%d" % rc)
    return r


def quant_128x1(x, offsets, x_scales=None, gather=None):
    """128 x 1 tiles along the rows of segments (the backward's weight-gradient
    operands; reading in moe_oracle.c).  x: [n, cols] float32, bf16 bits, or
    e4m3 codes (uint8) with 1 x 128 scales x_scales [n, cols/128]; offsets
    [n_seg + 1] int32 over the list rows; gather [rows] int32 or None.
    Returns (codes uint8 [rows, cols], scales float32 [n_blocks, cols]) with
    n_blocks = sum over segments of ceil(len / 128)."""
    offsets = _c(offsets, np.int32)
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint8:
        code, xs = E4M3, _c(x_scales, np.float32)
    else:
        code, x = _storage(x)
        xs = None
    cols = x.shape[1]
    assert cols % NC == 0
    g = None if gather is None else _c(gather, np.int32)
    rows = int(offsets[-1])
    lens = np.diff(offsets.astype(np.int64))
    nblk = int(((lens + NC - 1) // NC).sum())
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((max(nblk, 1), cols), np.float32)
    _load().oracle_quant_128x1(len(offsets) - 1, _p(offsets), cols, code, _p(x), _p(xs), _p(g), _p(q), _p(s))
    return q, s[:nblk]


def moe_backward_fp8(u, gate_w, topk_idx, routed_q, routed_s, shared_q, shared_s, dout, tokens=None, experts=None,
                     dgate=True, dshared=True, routed_scale=1.0):
    """Gradient of the FP8 layer (bf16 activations, e4m3 expert GEMMs with
    128 x 128 weight blocks) for a fixed selection, with the Dgrad and Wgrad
    GEMMs on FP8 operands (readings in moe_oracle.c).  u, gate_w: bf16 bits;
    routed_q / shared_q: e4m3 codes (gate, up, down) with block scales
    routed_s / shared_s; dout: float values of the bf16 upstream gradient.
    Returns the dict of moe_backward."""
    u = _c(u, np.uint16)
    gate_w = _c(gate_w, np.uint16)
    idx = _c(topk_idx, np.int32)
    T, d = u.shape
    Nr = gate_w.shape[0]
    K = idx.shape[1]
    I = routed_q[0].shape[1]
    Ns = shared_q[0].shape[0] if shared_q is not None else 0
    rq = [_c(a, np.uint8) for a in routed_q]
    rsc = [_c(a, np.float32) for a in routed_s]
    sq = [_c(a, np.uint8) for a in shared_q] if Ns else [None] * 3
    ssc = [_c(a, np.float32) for a in shared_s] if Ns else [None] * 3
    dout = _c(dout, np.float64)
    tok = None if tokens is None else _c(tokens, np.int64)
    exps = None if experts is None else _c(experts, np.int32)
    ne = Nr if exps is None else exps.shape[0]
    r = dict(du=np.zeros((T, d)), dg=np.zeros((T, K)),
             dgate_w=np.empty((Nr, d)) if dgate else None,
             dwg=np.empty((ne, I, d)), dwu=np.empty((ne, I, d)), dwd=np.empty((ne, d, I)),
             dswg=np.empty((Ns, I, d)) if dshared and Ns else None,
             dswu=np.empty((Ns, I, d)) if dshared and Ns else None,
             dswd=np.empty((Ns, d, I)) if dshared and Ns else None)
    rc = _load().oracle_moe_backward_fp8(T, d, Nr, Ns, K, I, _p(u), _p(gate_w), _p(idx), *[_p(a) for a in rq],
                                         *[_p(a) for a in rsc], *[_p(a) for a in sq], *[_p(a) for a in ssc],
                                         routed_scale, _p(dout), 0 if tok is None else tok.shape[0], _p(tok),
                                         0 if exps is None else exps.shape[0], _p(exps), _p(r["du"]), _p(r["dg"]),
                                         _p(r["dgate_w"]), _p(r["dwg"]), _p(r["dwu"]), _p(r["dwd"]), _p(r["dswg"]),
                                         _p(r["dswu"]), _p(r["dswd"]))
    if rc:
        raise ValueError("oracle_moe_backward_fp8 rc=%d" % rc)
    return r


def seq_balance(scores, topk_idx, seq_len, alpha=1e-4):
    """Complementary sequence-wise balance statistic per sequence of seq_len
    consecutive tokens (§2.1.2; alpha from §4.2): returns (loss [n_seq] fp32,
    counts [n_seq, Nr] int32 (selected slots per expert), P [n_seq, Nr] fp32
    (mean affinity share))."""
    scores = _c(scores, np.float32)
    topk_idx = _c(topk_idx, np.int32)
    T, Nr = scores.shape
    K = topk_idx.shape[1]
    n_seq = (T + seq_len - 1) // seq_len
    loss = np.empty(n_seq, np.float32)
    counts = np.empty((n_seq, Nr), np.int32)
    share = np.empty((n_seq, Nr), np.float32)
    _load().oracle_seq_balance(T, Nr, K, _p(scores), _p(topk_idx), seq_len, alpha, _p(loss), _p(counts), _p(share))
    return loss, counts, share


# ----------------------------------------------------------------------------
# numpy views of the storage formats (decoding only; used by tests)
# ----------------------------------------------------------------------------

def bf16_bits_to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
