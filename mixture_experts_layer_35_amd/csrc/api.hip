// api.hip -- the C ABI of libmoe (declared in include/moe.h): host-side
// argument checks, workspace layout and the launch sequence of each call.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "moe.h"
#include "internal.h"

namespace moe {

int device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

}  // namespace moe

using namespace moe;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_check(hipError_t e, const char *what) {
    if (e == hipSuccess) return MOE_OK;
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIPCHK(expr)                                      \
    do {                                                  \
        int rc_ = hip_check((expr), #expr);               \
        if (rc_ != MOE_OK) return rc_;                    \
    } while (0)

#define NEED(ptr)                                                                            \
    do {                                                                                     \
        if (!(ptr)) return fail(MOE_ERR_INVALID_ARG, "%s: %s must not be NULL", fn, #ptr); \
    } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int esize(int dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 2 : 1; }

// Checks everything about the shape that the kernels rely on.
int check_shape(const moe_shape *s, const char *fn) {
    if (!s) return fail(MOE_ERR_INVALID_ARG, "%s: shape must not be NULL", fn);
    if (s->T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T = %lld is negative", fn, (long long)s->T);
    if (s->d <= 0 || s->n_routed <= 0 || s->n_groups <= 0 || s->topk_groups <= 0 || s->topk <= 0 || s->inter <= 0 ||
        s->n_shared < 0)
        return fail(MOE_ERR_INVALID_ARG, "%s: sizes must be positive (n_shared >= 0)", fn);
    const bool f32 = s->act_dtype == MOE_F32 && s->router_dtype == MOE_F32 && s->w_dtype == MOE_F32 &&
                     s->out_dtype == MOE_F32;
    const bool bf16 = s->act_dtype == MOE_BF16 && s->router_dtype == MOE_BF16 && s->w_dtype == MOE_BF16 &&
                      s->out_dtype == MOE_BF16;
    const bool fp8 = s->act_dtype == MOE_BF16 && s->router_dtype == MOE_BF16 && s->w_dtype == MOE_E4M3 &&
                     s->out_dtype == MOE_BF16;
    if (!f32 && !bf16 && !fp8)
        return fail(MOE_ERR_UNSUPPORTED, "%s: dtype combination (act %d, router %d, w %d, out %d) is not supported",
                    fn, s->act_dtype, s->router_dtype, s->w_dtype, s->out_dtype);
    if (s->n_routed > kMaxExperts)
        return fail(MOE_ERR_UNSUPPORTED, "%s: n_routed = %d exceeds %d", fn, s->n_routed, kMaxExperts);
    if (s->n_routed % s->n_groups)
        return fail(MOE_ERR_UNSUPPORTED, "%s: n_routed = %d is not a multiple of n_groups = %d", fn, s->n_routed,
                    s->n_groups);
    if (s->n_groups > 64 || s->topk_groups > s->n_groups)
        return fail(MOE_ERR_UNSUPPORTED, "%s: need topk_groups <= n_groups <= 64 (got %d, %d)", fn, s->topk_groups,
                    s->n_groups);
    if (s->topk > 32 || (int64_t)s->topk > (int64_t)s->topk_groups * (s->n_routed / s->n_groups))
        return fail(MOE_ERR_UNSUPPORTED, "%s: topk = %d must be <= 32 and <= topk_groups * n_routed / n_groups", fn,
                    s->topk);
    if (s->topk > s->n_routed)
        return fail(MOE_ERR_UNSUPPORTED, "%s: topk = %d exceeds n_routed", fn, s->topk);
    if (s->n_shared > 8) return fail(MOE_ERR_UNSUPPORTED, "%s: n_shared = %d exceeds 8", fn, s->n_shared);
    if (s->d % 128 || s->inter % 128)
        return fail(MOE_ERR_UNSUPPORTED, "%s: d = %d and inter = %d must be multiples of 128", fn, s->d, s->inter);
    if (s->quant_block != 128)
        return fail(MOE_ERR_UNSUPPORTED, "%s: quant_block = %d (only 128 is supported)", fn, s->quant_block);
    if (s->T * (int64_t)s->topk >= (1ll << 31) || s->T * (int64_t)(s->n_shared ? s->n_shared : 1) >= (1ll << 31))
        return fail(MOE_ERR_UNSUPPORTED, "%s: T * topk and T * n_shared must be below 2^31", fn);
    if (s->flags & ~(MOE_ADD_RESIDUAL | MOE_SAVE_SWIGLU_INPUTS))
        return fail(MOE_ERR_INVALID_ARG, "%s: unknown flags 0x%x", fn, s->flags);
    return MOE_OK;
}

int ws_check(void *ws, size_t have, size_t need, const char *fn) {
    if (need == 0) return MOE_OK;
    if (!ws) return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got NULL", fn, need);
    if ((uintptr_t)ws & 255) return fail(MOE_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
    if (have < need) return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu", fn, need, have);
    return MOE_OK;
}

int dt_of(int d) { return d == MOE_F32 ? DT_F32 : d == MOE_BF16 ? DT_BF16 : DT_E4M3; }

// ---- workspace layouts --------------------------------------------------------

struct FwdLayout {
    size_t scores, idx, w, counts, offsets, bc, perm, inv, uq, us, h, hs, hsh, hshs, yperm, ysh, fq, ab, rpart, total;
};

FwdLayout fwd_layout(const moe_shape *s) {
    FwdLayout L{};
    const int64_t T = s->T, TK = T * s->topk, TS = T * s->n_shared;
    const bool fp8 = s->w_dtype == MOE_E4M3;
    const int hsz = fp8 ? 1 : esize(s->act_dtype);
    const int osz = esize(s->out_dtype);
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t r = o; o += align256(bytes); return r; };
    L.scores = take((size_t)T * s->n_routed * 4);
    L.idx = take((size_t)TK * 4);
    L.w = take((size_t)TK * 4);
    L.counts = take((size_t)s->n_routed * 4);
    L.offsets = take((size_t)(s->n_routed + 1) * 4);
    L.bc = take((size_t)perm_blocks(T) * s->n_routed * 4);
    L.perm = take((size_t)TK * 4);
    L.inv = take((size_t)TK * 4);
    L.uq = take(fp8 ? (size_t)T * s->d : 0);
    L.us = take(fp8 ? (size_t)T * (s->d / 128) * 4 : 0);
    L.h = take((size_t)TK * s->inter * hsz);
    L.hs = take(fp8 ? (size_t)TK * (s->inter / 128) * 4 : 0);
    L.hsh = take((size_t)TS * s->inter * hsz);
    L.hshs = take(fp8 ? (size_t)TS * (s->inter / 128) * 4 : 0);
    L.yperm = take((size_t)TK * s->d * osz);
    L.ysh = take((size_t)TS * s->d * osz);
    L.fq = take(FFN_QUEUE_INTS * 4);
    // SwiGLU inputs a | b of the routed rows, then of the shared rows (MOE_SAVE_SWIGLU_INPUTS)
    L.ab = take((s->flags & MOE_SAVE_SWIGLU_INPUTS) ? (size_t)(TK + TS) * 2 * s->inter * 4 : 0);
    // the split-K router's chunk partials of the gate products
    L.rpart = take(router_splitk_ok(dt_of(s->act_dtype), s->n_routed, s->n_groups, s->topk)
                       ? router_partial_bytes(T, s->d, s->n_routed) : 0);
    L.total = o;
    return L;
}

size_t ffn_ws(const moe_shape *s, int64_t max_rows) {
    const bool fp8 = s->w_dtype == MOE_E4M3;
    const int hsz = fp8 ? 1 : esize(s->act_dtype);
    return align256((size_t)max_rows * s->inter * hsz) + (fp8 ? align256((size_t)max_rows * (s->inter / 128) * 4) : 0) +
           align256(FFN_QUEUE_INTS * 4);
}

int run_ffn_pair(const moe_shape *s, const FfnProblem *gu, const FfnProblem *dn, int nprob, int *ctr, hipStream_t st) {
    FfnArgs a{};
    a.nprob = nprob;
    a.ctr = ctr;
    a.K = s->d;
    a.F = s->inter;
    for (int i = 0; i < nprob; ++i) a.p[i] = gu[i];
    HIPCHK(launch_ffn(dt_of(s->w_dtype), FFN_GATEUP, a, st));
    a.K = s->inter;
    a.F = s->d;
    for (int i = 0; i < nprob; ++i) a.p[i] = dn[i];
    HIPCHK(launch_ffn(dt_of(s->w_dtype), FFN_DOWN, a, st));
    return MOE_OK;
}

// ---- the library's own forward workspace (moe_forward_static) -------------------
//
// A file-scope device array: each GPU the library runs on holds its own copy for
// the life of the process.  In host code `scratch` only names the symbol; its
// device address comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is ever handed to kernels or copies.
constexpr size_t kStaticWsBytes = MOE_STATIC_WS_BYTES;
static __device__ __align__(256) char scratch[kStaticWsBytes];

constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void *g_static_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (nullptr and a message on failure).
void *static_workspace(int *rc, const char *fn) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *rc = fail(MOE_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *rc = fail(MOE_ERR_UNSUPPORTED, "%s: device %d is beyond the library's %d devices", fn, dev, kMaxDevices);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_static_mu);
    if (!g_static_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *rc = fail(MOE_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
            return nullptr;
        }
        g_static_ptr[dev] = p;
    }
    *rc = MOE_OK;
    return g_static_ptr[dev];
}

}  // namespace

extern "C" {

const char *moe_last_error(void) { return g_err.c_str(); }

const char *moe_version(void) { return "libmoe 0.1 (gfx950)"; }

size_t moe_workspace_bytes(const moe_shape *s, int which) {
    if (check_shape(s, "moe_workspace_bytes") != MOE_OK) return 0;
    switch (which) {
        case MOE_WS_ROUTE:
            return align256((size_t)s->T * s->n_routed * 4) +
                   (router_splitk_ok(dt_of(s->act_dtype), s->n_routed, s->n_groups, s->topk)
                        ? align256(router_partial_bytes(s->T, s->d, s->n_routed)) : 0);
        case MOE_WS_PERMUTE: return align256((size_t)perm_blocks(s->T) * s->n_routed * 4);
        case MOE_WS_FORWARD: return fwd_layout(s).total;
        default: fail(MOE_ERR_INVALID_ARG, "moe_workspace_bytes: unknown workspace kind %d", which); return 0;
    }
}

size_t moe_ffn_workspace_bytes(const moe_shape *s, int64_t max_rows) {
    if (check_shape(s, "moe_ffn_workspace_bytes") != MOE_OK) return 0;
    if (max_rows < 0) { fail(MOE_ERR_INVALID_ARG, "moe_ffn_workspace_bytes: max_rows < 0"); return 0; }
    return ffn_ws(s, max_rows);
}

int moe_route(const moe_shape *s, const void *u, const void *gate_w, const float *bias, const float *scores_in,
              float *scores_out, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes, void *stream) {
    const char *fn = "moe_route";
    int rc = check_shape(s, fn);
    if (rc) return rc;
    NEED(bias);
    NEED(topk_idx);
    NEED(topk_w);
    if (!scores_in) {
        NEED(u);
        NEED(gate_w);
    }
    float *scores = scores_out;
    const size_t sbytes = align256((size_t)s->T * s->n_routed * 4);
    if (!scores_in && !scores) {
        rc = ws_check(ws, ws_bytes, sbytes, fn);
        if (rc) return rc;
        scores = (float *)ws;
    }
    // the split-K gate GEMM when the workspace also holds its chunk partials
    float *part = nullptr;
    if (!scores_in && router_splitk_ok(dt_of(s->act_dtype), s->n_routed, s->n_groups, s->topk) && ws &&
        !((uintptr_t)ws & 255)) {
        const size_t off = scores_out ? 0 : sbytes;
        if (ws_bytes >= off + align256(router_partial_bytes(s->T, s->d, s->n_routed))) part = (float *)((char *)ws + off);
    }
    if (s->T == 0) return MOE_OK;
    hipStream_t st = (hipStream_t)stream;
    if (part) {
        HIPCHK(launch_router_splitk(u, gate_w, part, scores, bias, s->T, s->d, s->n_groups, s->topk_groups, s->topk,
                                    s->routed_scale, topk_idx, topk_w, st));
        return MOE_OK;
    }
    if (scores_in) {
        if (scores_out)
            HIPCHK(hipMemcpyAsync(scores_out, scores_in, (size_t)s->T * s->n_routed * 4, hipMemcpyDeviceToDevice, st));
        scores = (float *)scores_in;
    } else {
        HIPCHK(launch_router_gemm(dt_of(s->act_dtype), u, gate_w, scores, s->T, s->d, s->n_routed, st));
    }
    HIPCHK(launch_router_select(scores, bias, s->T, s->n_routed, s->n_groups, s->topk_groups, s->topk,
                                s->routed_scale, topk_idx, topk_w, st));
    return MOE_OK;
}

int moe_permute(const moe_shape *s, const int32_t *topk_idx, const void *u, int32_t *counts, int32_t *offsets,
                int32_t *perm_token, int32_t *inv_perm, void *x_perm, float *x_scales, void *ws, size_t ws_bytes,
                void *stream) {
    const char *fn = "moe_permute";
    int rc = check_shape(s, fn);
    if (rc) return rc;
    NEED(topk_idx);
    NEED(counts);
    NEED(offsets);
    NEED(perm_token);
    NEED(inv_perm);
    const bool fp8 = s->w_dtype == MOE_E4M3;
    if (x_perm) {
        NEED(u);
        if (fp8) NEED(x_scales);
    }
    rc = ws_check(ws, ws_bytes, align256((size_t)perm_blocks(s->T) * s->n_routed * 4), fn);
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    const int64_t TK = s->T * s->topk;
    int32_t *bc = (int32_t *)ws;
    HIPCHK(launch_perm_hist(topk_idx, s->T, s->topk, s->n_routed, bc, st));
    HIPCHK(launch_perm_scan(bc, s->T, s->n_routed, counts, offsets, st));
    HIPCHK(launch_perm_scatter(topk_idx, bc, s->T, s->topk, s->n_routed, perm_token, inv_perm, st));
    if (x_perm) {
        if (fp8)
            HIPCHK(launch_quant_rows(dt_of(s->act_dtype), u, perm_token, TK, s->d, (uint8_t *)x_perm, x_scales, st));
        else
            HIPCHK(launch_gather_rows(dt_of(s->act_dtype), u, perm_token, TK, s->d, x_perm, st));
    }
    return MOE_OK;
}

int moe_grouped_ffn(const moe_shape *s, int32_t n_exp, const int32_t *offsets, int64_t max_rows,
                    const int32_t *gather, const void *x, const float *x_scales, const void *w_gate,
                    const void *w_up, const void *w_down, const float *const *w_scales, void *y, void *ws,
                    size_t ws_bytes, void *stream) {
    const char *fn = "moe_grouped_ffn";
    int rc = check_shape(s, fn);
    if (rc) return rc;
    if (n_exp <= 0 || n_exp > kMaxExperts)
        return fail(MOE_ERR_UNSUPPORTED, "%s: n_exp = %d must be in [1, %d]", fn, n_exp, kMaxExperts);
    if (max_rows < 0 || max_rows >= (1ll << 31)) return fail(MOE_ERR_INVALID_ARG, "%s: max_rows out of range", fn);
    NEED(offsets);
    NEED(x);
    NEED(w_gate);
    NEED(w_up);
    NEED(w_down);
    NEED(y);
    const bool fp8 = s->w_dtype == MOE_E4M3;
    if (fp8) {
        NEED(x_scales);
        NEED(w_scales);
        if (!w_scales[0] || !w_scales[1] || !w_scales[2])
            return fail(MOE_ERR_INVALID_ARG, "%s: w_scales entries must not be NULL", fn);
    }
    rc = ws_check(ws, ws_bytes, ffn_ws(s, max_rows), fn);
    if (rc) return rc;
    if (max_rows == 0) return MOE_OK;
    char *h = (char *)ws;
    float *hs = fp8 ? (float *)(h + align256((size_t)max_rows * s->inter)) : nullptr;
    FfnProblem gu{}, dn{};
    gu.n_exp = dn.n_exp = n_exp;
    gu.offsets = dn.offsets = offsets;
    gu.gather = gather;
    gu.x = x;
    gu.xs = x_scales;
    gu.w0 = w_gate;
    gu.w1 = w_up;
    gu.s0 = fp8 ? w_scales[0] : nullptr;
    gu.s1 = fp8 ? w_scales[1] : nullptr;
    gu.out = h;
    gu.out_s = hs;
    dn.x = h;
    dn.xs = hs;
    dn.w0 = w_down;
    dn.s0 = fp8 ? w_scales[2] : nullptr;
    dn.out = y;
    int *ctr = (int *)(h + ffn_ws(s, max_rows) - align256(FFN_QUEUE_INTS * 4));
    return run_ffn_pair(s, &gu, &dn, 1, ctr, (hipStream_t)stream);
}

int moe_combine(const moe_shape *s, const void *y_perm, const int32_t *inv_perm, const float *topk_w,
                const void *y_shared, const void *residual, void *out, void *stream) {
    const char *fn = "moe_combine";
    int rc = check_shape(s, fn);
    if (rc) return rc;
    NEED(y_perm);
    NEED(inv_perm);
    NEED(topk_w);
    NEED(out);
    if (s->n_shared > 0) NEED(y_shared);
    if (s->flags & MOE_ADD_RESIDUAL) NEED(residual);
    HIPCHK(launch_combine(dt_of(s->out_dtype), dt_of(s->act_dtype), y_perm, inv_perm, topk_w,
                          s->n_shared ? y_shared : nullptr, s->n_shared,
                          (s->flags & MOE_ADD_RESIDUAL) ? residual : nullptr, out, s->T, s->d, s->topk,
                          (hipStream_t)stream));
    return MOE_OK;
}

int moe_forward(const moe_shape *s, const void *u, const void *gate_w, const float *bias,
                const void *const *routed_w, const float *const *routed_s, const void *const *shared_w,
                const float *const *shared_s, void *out, int32_t *topk_idx_out, float *topk_w_out,
                int32_t *counts_out, float *scores_out, void *ws, size_t ws_bytes, void *stream) {
    return moe_forward_timed(s, u, gate_w, bias, routed_w, routed_s, shared_w, shared_s, out, topk_idx_out,
                             topk_w_out, counts_out, scores_out, ws, ws_bytes, stream, nullptr);
}

}  // extern "C"

namespace {

// Every argument check of the forward that needs no workspace (shape, pointers).
int check_forward_args(const char *fn, const moe_shape *s, const void *u, const void *gate_w, const float *bias,
                       const void *const *routed_w, const float *const *routed_s, const void *const *shared_w,
                       const float *const *shared_s, void *out) {
    int rc = check_shape(s, fn);
    if (rc) return rc;
    NEED(u);
    NEED(gate_w);
    NEED(bias);
    NEED(routed_w);
    NEED(out);
    if (!routed_w[0] || !routed_w[1] || !routed_w[2])
        return fail(MOE_ERR_INVALID_ARG, "%s: routed_w entries must not be NULL", fn);
    const bool fp8 = s->w_dtype == MOE_E4M3;
    if (fp8) {
        NEED(routed_s);
        if (!routed_s[0] || !routed_s[1] || !routed_s[2])
            return fail(MOE_ERR_INVALID_ARG, "%s: routed_s entries must not be NULL", fn);
    }
    if (s->n_shared > 0) {
        NEED(shared_w);
        if (!shared_w[0] || !shared_w[1] || !shared_w[2])
            return fail(MOE_ERR_INVALID_ARG, "%s: shared_w entries must not be NULL", fn);
        if (fp8) {
            NEED(shared_s);
            if (!shared_s[0] || !shared_s[1] || !shared_s[2])
                return fail(MOE_ERR_INVALID_ARG, "%s: shared_s entries must not be NULL", fn);
        }
    }
    return MOE_OK;
}

int forward_impl(const char *fn, const moe_shape *s, const void *u, const void *gate_w, const float *bias,
                 const void *const *routed_w, const float *const *routed_s, const void *const *shared_w,
                 const float *const *shared_s, void *out, int32_t *topk_idx_out, float *topk_w_out,
                 int32_t *counts_out, float *scores_out, void *ws, size_t ws_bytes, void *stream, void *const *ev) {
    int rc = check_forward_args(fn, s, u, gate_w, bias, routed_w, routed_s, shared_w, shared_s, out);
    if (rc) return rc;
    const bool fp8 = s->w_dtype == MOE_E4M3;
    const FwdLayout L = fwd_layout(s);
    rc = ws_check(ws, ws_bytes, L.total, fn);
    if (rc) return rc;
    if (s->T == 0) return MOE_OK;

    hipStream_t st = (hipStream_t)stream;
    char *W = (char *)ws;
    const int64_t T = s->T, TK = T * s->topk;
    // the workspace keeps the affinities, selection and gates (moe_backward reads them);
    // the optional outputs get copies
    float *scores = (float *)(W + L.scores);
    int32_t *idx = (int32_t *)(W + L.idx);
    float *tw = (float *)(W + L.w);
    int32_t *counts = counts_out ? counts_out : (int32_t *)(W + L.counts);
    int32_t *offsets = (int32_t *)(W + L.offsets);
    int32_t *bc = (int32_t *)(W + L.bc);
    int32_t *perm = (int32_t *)(W + L.perm);
    int32_t *inv = (int32_t *)(W + L.inv);

    auto mark = [&](int i) -> hipError_t {
        return (ev && ev[i]) ? hipEventRecord((hipEvent_t)ev[i], st) : hipSuccess;
    };
    // 1. affinities and selection
    HIPCHK(mark(0));
    if (router_splitk_ok(dt_of(s->act_dtype), s->n_routed, s->n_groups, s->topk)) {
        HIPCHK(launch_router_splitk(u, gate_w, (float *)(W + L.rpart), scores, bias, T, s->d, s->n_groups,
                                    s->topk_groups, s->topk, s->routed_scale, idx, tw, st));
    } else {
        HIPCHK(launch_router_gemm(dt_of(s->act_dtype), u, gate_w, scores, T, s->d, s->n_routed, st));
        HIPCHK(launch_router_select(scores, bias, T, s->n_routed, s->n_groups, s->topk_groups, s->topk,
                                    s->routed_scale, idx, tw, st));
    }
    if (scores_out)
        HIPCHK(hipMemcpyAsync(scores_out, scores, (size_t)T * s->n_routed * 4, hipMemcpyDeviceToDevice, st));
    if (topk_idx_out) HIPCHK(hipMemcpyAsync(topk_idx_out, idx, (size_t)TK * 4, hipMemcpyDeviceToDevice, st));
    if (topk_w_out) HIPCHK(hipMemcpyAsync(topk_w_out, tw, (size_t)TK * 4, hipMemcpyDeviceToDevice, st));
    HIPCHK(mark(1));
    // 2. dispatch bookkeeping (rows are gathered inside the expert GEMM)
    HIPCHK(launch_perm_hist(idx, T, s->topk, s->n_routed, bc, st));
    HIPCHK(launch_perm_scan(bc, T, s->n_routed, counts, offsets, st));
    HIPCHK(launch_perm_scatter(idx, bc, T, s->topk, s->n_routed, perm, inv, st));
    // 3. fp8: one 1x128 quantisation per token
    const void *xin = u;
    const float *xs = nullptr;
    if (fp8) {
        HIPCHK(launch_quant_rows(dt_of(s->act_dtype), u, nullptr, T, s->d, (uint8_t *)(W + L.uq), (float *)(W + L.us),
                                 st));
        xin = W + L.uq;
        xs = (const float *)(W + L.us);
    }
    HIPCHK(mark(2));
    // 4. routed and shared experts
    FfnProblem gu[2] = {}, dn[2] = {};
    gu[0].n_exp = dn[0].n_exp = s->n_routed;
    gu[0].offsets = dn[0].offsets = offsets;
    gu[0].gather = perm;
    gu[0].x = xin;
    gu[0].xs = xs;
    gu[0].w0 = routed_w[0];
    gu[0].w1 = routed_w[1];
    gu[0].s0 = fp8 ? routed_s[0] : nullptr;
    gu[0].s1 = fp8 ? routed_s[1] : nullptr;
    gu[0].out = W + L.h;
    gu[0].out_s = fp8 ? (float *)(W + L.hs) : nullptr;
    dn[0].x = W + L.h;
    dn[0].xs = gu[0].out_s;
    dn[0].w0 = routed_w[2];
    dn[0].s0 = fp8 ? routed_s[2] : nullptr;
    dn[0].out = W + L.yperm;
    int nprob = 1;
    if (s->n_shared > 0) {
        nprob = 2;
        gu[1].n_exp = dn[1].n_exp = s->n_shared;
        gu[1].offsets = dn[1].offsets = nullptr;
        gu[1].rows_fixed = dn[1].rows_fixed = T;
        gu[1].x_local = 1;
        gu[1].x = xin;
        gu[1].xs = xs;
        gu[1].w0 = shared_w[0];
        gu[1].w1 = shared_w[1];
        gu[1].s0 = fp8 ? shared_s[0] : nullptr;
        gu[1].s1 = fp8 ? shared_s[1] : nullptr;
        gu[1].out = W + L.hsh;
        gu[1].out_s = fp8 ? (float *)(W + L.hshs) : nullptr;
        dn[1].x = W + L.hsh;
        dn[1].xs = gu[1].out_s;
        dn[1].w0 = shared_w[2];
        dn[1].s0 = fp8 ? shared_s[2] : nullptr;
        dn[1].out = W + L.ysh;
    }
    if (s->flags & MOE_SAVE_SWIGLU_INPUTS) {
        gu[0].ab = (float *)(W + L.ab);
        gu[1].ab = s->n_shared > 0 ? (float *)(W + L.ab) + (size_t)TK * 2 * s->inter : nullptr;
    }
    {
        FfnArgs a{};
        a.nprob = nprob;
        a.K = s->d;
        a.F = s->inter;
        a.ctr = (int *)(W + L.fq);
        // the shared experts' tiles go first: their row blocks of one weight block are list
        // neighbours, taken together by the workgroups of one XCD
        for (int i = 0; i < nprob; ++i) a.p[i] = gu[nprob - 1 - i];
        HIPCHK(launch_ffn(dt_of(s->w_dtype), (s->flags & MOE_SAVE_SWIGLU_INPUTS) ? FFN_GATEUP_SAVE : FFN_GATEUP, a,
                          st));
        HIPCHK(mark(3));
        a.K = s->inter;
        a.F = s->d;
        for (int i = 0; i < nprob; ++i) a.p[i] = dn[nprob - 1 - i];
        HIPCHK(launch_ffn(dt_of(s->w_dtype), FFN_DOWN, a, st));
        HIPCHK(mark(4));
    }
    // 5. gate-weighted combine plus shared experts
    HIPCHK(launch_combine(dt_of(s->out_dtype), dt_of(s->act_dtype), W + L.yperm, inv, tw,
                          s->n_shared ? W + L.ysh : nullptr, s->n_shared,
                          (s->flags & MOE_ADD_RESIDUAL) ? u : nullptr, out, T, s->d, s->topk, st));
    HIPCHK(mark(5));
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_timed(const moe_shape *s, const void *u, const void *gate_w, const float *bias,
                      const void *const *routed_w, const float *const *routed_s, const void *const *shared_w,
                      const float *const *shared_s, void *out, int32_t *topk_idx_out, float *topk_w_out,
                      int32_t *counts_out, float *scores_out, void *ws, size_t ws_bytes, void *stream,
                      void *const *ev) {
    return forward_impl("moe_forward", s, u, gate_w, bias, routed_w, routed_s, shared_w, shared_s, out, topk_idx_out,
                        topk_w_out, counts_out, scores_out, ws, ws_bytes, stream, ev);
}

int moe_forward_static(const moe_shape *s, const void *u, const void *gate_w, const float *bias,
                       const void *const *routed_w, const float *const *routed_s, const void *const *shared_w,
                       const float *const *shared_s, void *out, int32_t *topk_idx_out, float *topk_w_out,
                       int32_t *counts_out, float *scores_out, void *stream) {
    const char *fn = "moe_forward_static";
    int rc = check_forward_args(fn, s, u, gate_w, bias, routed_w, routed_s, shared_w, shared_s, out);
    if (rc) return rc;
    if (s->flags & MOE_SAVE_SWIGLU_INPUTS)
        return fail(MOE_ERR_UNSUPPORTED, "%s: MOE_SAVE_SWIGLU_INPUTS needs a caller workspace (moe_forward)", fn);
    const size_t need = fwd_layout(s).total;
    if (need > kStaticWsBytes)
        return fail(MOE_ERR_WORKSPACE, "%s: the forward needs %zu workspace bytes, above the library's %zu", fn, need,
                    kStaticWsBytes);
    void *ws = static_workspace(&rc, fn);
    if (!ws) return rc;
    return forward_impl(fn, s, u, gate_w, bias, routed_w, routed_s, shared_w, shared_s, out, topk_idx_out,
                        topk_w_out, counts_out, scores_out, ws, kStaticWsBytes, stream, nullptr);
}

// backward workspace: dy [TK][d], dg [TK], dz [TK], dh [R][I], dab [R][2I], dx [R][d] (R = TK + T*Ns);
// for e4m3 layers also the 1 x 128 tiles of dy, dO and [dA dB] (Dgrad inputs), the 128 x 1 tiles
// of the weight-gradient operands and the experts' run bases
struct BwdLayout {
    size_t dy, dg, dz, dh, dab, dx, fq;
    size_t dyq, dys, doq, dos, abq, abs_;                       // Dgrad inputs
    size_t bbase, p1q, p1s, q1q, q1s, p2q, p2s, q2q, q2s;      // routed Wgrad operands (down, gate/up)
    size_t sp1q, sp1s, sq1q, sq1s, sp2q, sp2s, sq2q, sq2s;      // shared Wgrad operands
    size_t total;
    int64_t rblk, sblk;                                         // run bounds: routed (all experts), one T-row segment
};

static BwdLayout bwd_layout(const moe_shape *s) {
    BwdLayout L{};
    const int64_t T = s->T, TK = T * s->topk, Ns = s->n_shared, R = TK + T * Ns;
    const int64_t d = s->d, I = s->inter;
    const int a = esize(s->act_dtype);
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t r = o; o += align256(bytes); return r; };
    L.dy = take((size_t)TK * d * a);
    L.dg = take((size_t)TK * 4);
    L.dz = take((size_t)TK * 4);
    L.dh = take((size_t)R * I * a);
    L.dab = take((size_t)R * 2 * I * a);
    L.dx = take((size_t)R * d * a);
    L.fq = take(FFN_QUEUE_INTS * 4);
    if (s->w_dtype == MOE_E4M3) {
        L.rblk = TK / 128 + s->n_routed + 1;
        L.sblk = (T + 127) / 128;
        L.dyq = take((size_t)TK * d);
        L.dys = take((size_t)TK * (d / 128) * 4);
        L.doq = take((size_t)T * d);
        L.dos = take((size_t)T * (d / 128) * 4);
        L.abq = take((size_t)R * 2 * I);
        L.abs_ = take((size_t)R * (2 * I / 128) * 4);
        L.bbase = take((size_t)(s->n_routed + 1) * 4);
        L.p1q = take((size_t)TK * d);
        L.p1s = take((size_t)L.rblk * d * 4);
        L.q1q = take((size_t)TK * I);
        L.q1s = take((size_t)L.rblk * I * 4);
        L.p2q = take((size_t)TK * 2 * I);
        L.p2s = take((size_t)L.rblk * 2 * I * 4);
        L.q2q = take((size_t)TK * d);
        L.q2s = take((size_t)L.rblk * d * 4);
        L.sp1q = take((size_t)T * d);
        L.sp1s = take((size_t)L.sblk * d * 4);
        L.sq1q = take((size_t)Ns * T * I);
        L.sq1s = take((size_t)Ns * L.sblk * I * 4);
        L.sp2q = take((size_t)Ns * T * 2 * I);
        L.sp2s = take((size_t)Ns * L.sblk * 2 * I * 4);
        L.sq2q = take((size_t)T * d);
        L.sq2s = take((size_t)L.sblk * d * 4);
    }
    L.total = o;
    return L;
}

size_t moe_backward_workspace_bytes(const moe_shape *s) {
    if (check_shape(s, "moe_backward_workspace_bytes") != MOE_OK) return 0;
    return bwd_layout(s).total;
}

int moe_transpose_expert_weights(const moe_shape *s, int32_t n, const void *const *w, const float *const *w_s,
                                 void *const *wt, float *const *wt_s, void *stream) {
    const char *fn = "moe_transpose_expert_weights";
    int rc = check_shape(s, fn);
    if (rc) return rc;
    if (n < 0) return fail(MOE_ERR_INVALID_ARG, "%s: n < 0", fn);
    if (n == 0) return MOE_OK;
    NEED(w);
    NEED(wt);
    if (!w[0] || !w[1] || !w[2] || !wt[0] || !wt[1])
        return fail(MOE_ERR_INVALID_ARG, "%s: weight entries must not be NULL", fn);
    const bool fp8 = s->w_dtype == MOE_E4M3;
    if (fp8) {
        NEED(w_s);
        NEED(wt_s);
        if (!w_s[0] || !w_s[1] || !w_s[2] || !wt_s[0] || !wt_s[1])
            return fail(MOE_ERR_INVALID_ARG, "%s: e4m3 scale entries must not be NULL", fn);
    }
    const int dt = dt_of(s->w_dtype), d = s->d, I = s->inter;
    hipStream_t st = (hipStream_t)stream;
    HIPCHK(launch_transpose(dt, w[2], n, d, I, wt[0], d, 0, st));        // [n][d][I] -> [n][I][d]
    HIPCHK(launch_transpose(dt, w[0], n, I, d, wt[1], 2 * I, 0, st));    // [n][I][d] -> [n][d][0:I]
    HIPCHK(launch_transpose(dt, w[1], n, I, d, wt[1], 2 * I, I, st));    // [n][I][d] -> [n][d][I:2I]
    if (fp8) {
        // 128 x 128 block scales follow their blocks
        const int db = d / 128, ib = I / 128;
        HIPCHK(launch_transpose_scales(w_s[2], n, db, ib, wt_s[0], db, 0, st));
        HIPCHK(launch_transpose_scales(w_s[0], n, ib, db, wt_s[1], 2 * ib, 0, st));
        HIPCHK(launch_transpose_scales(w_s[1], n, ib, db, wt_s[1], 2 * ib, ib, st));
    }
    return MOE_OK;
}

static bool all3(const void *const *p) { return p && p[0] && p[1] && p[2]; }
static bool all2(const void *const *p) { return p && p[0] && p[1]; }

static int backward_impl(const moe_shape *s, const void *u, const void *gate_w, const void *const *routed_w,
                         const float *const *routed_s, const void *const *routed_wt,
                         const float *const *routed_wt_s, const void *const *shared_w, const float *const *shared_s,
                         const void *const *shared_wt, const float *const *shared_wt_s, const void *fwd_ws,
                         size_t fwd_ws_bytes, const void *dout, void *du, float *dgate_w, void *const *d_routed_w,
                         void *const *d_shared_w, float *dtopk_w, void *ws, size_t ws_bytes, void *stream,
                         void *const *ev) {
    const char *fn = "moe_backward";
    int rc = check_shape(s, fn);
    if (rc) return rc;
    if (s->T == 0) return MOE_OK;
    NEED(u);
    NEED(gate_w);
    NEED(fwd_ws);
    NEED(dout);
    NEED(du);
    const bool fp8 = s->w_dtype == MOE_E4M3;
    const int Ns = s->n_shared;
    if (!all3(routed_w) || !all2(routed_wt))
        return fail(MOE_ERR_INVALID_ARG, "%s: routed weight entries must not be NULL", fn);
    if (fp8 && (!all3((const void *const *)routed_s) || !all2((const void *const *)routed_wt_s)))
        return fail(MOE_ERR_INVALID_ARG, "%s: e4m3 routed scale entries must not be NULL", fn);
    if (Ns > 0) {
        if (!all3(shared_w) || !all2(shared_wt))
            return fail(MOE_ERR_INVALID_ARG, "%s: shared weight entries must not be NULL", fn);
        if (fp8 && (!all3((const void *const *)shared_s) || !all2((const void *const *)shared_wt_s)))
            return fail(MOE_ERR_INVALID_ARG, "%s: e4m3 shared scale entries must not be NULL", fn);
    }
    if (d_routed_w && !all3((const void *const *)d_routed_w))
        return fail(MOE_ERR_INVALID_ARG, "%s: d_routed_w entries must not be NULL", fn);
    if (Ns > 0 && d_shared_w && !all3((const void *const *)d_shared_w))
        return fail(MOE_ERR_INVALID_ARG, "%s: d_shared_w entries must not be NULL", fn);
    const FwdLayout F = fwd_layout(s);
    if ((uintptr_t)fwd_ws & 255) return fail(MOE_ERR_INVALID_ARG, "%s: forward workspace must be 256-byte aligned", fn);
    if (fwd_ws_bytes < F.total)
        return fail(MOE_ERR_WORKSPACE, "%s: forward workspace of %zu bytes expected, got %zu", fn, F.total,
                    fwd_ws_bytes);
    const BwdLayout L = bwd_layout(s);
    rc = ws_check(ws, ws_bytes, L.total, fn);
    if (rc) return rc;

    hipStream_t st = (hipStream_t)stream;
    const int dt = dt_of(s->act_dtype), wdt = dt_of(s->w_dtype);
    const int64_t T = s->T, TK = T * s->topk;
    const int d = s->d, I = s->inter, a_sz = esize(s->act_dtype);
    const char *Fw = (const char *)fwd_ws;
    char *W = (char *)ws;
    const float *scores = (const float *)(Fw + F.scores);
    const int32_t *idx = (const int32_t *)(Fw + F.idx);
    const float *tw = (const float *)(Fw + F.w);
    const int32_t *offsets = (const int32_t *)(Fw + F.offsets);
    const int32_t *perm = (const int32_t *)(Fw + F.perm);
    const int32_t *inv = (const int32_t *)(Fw + F.inv);
    char *dy = W + L.dy, *dh = W + L.dh, *dab = W + L.dab, *dx = W + L.dx;
    float *dg = dtopk_w ? dtopk_w : (float *)(W + L.dg);
    float *dz = (float *)(W + L.dz);
    char *dh_s = dh + (size_t)TK * I * a_sz, *dab_s = dab + (size_t)TK * 2 * I * a_sz, *dx_s = dx + (size_t)TK * d * a_sz;
    auto U8 = [&](size_t o) { return (uint8_t *)(W + o); };
    auto F32 = [&](size_t o) { return (float *)(W + o); };

    auto mark = [&](int i) -> hipError_t {
        return (ev && ev[i]) ? hipEventRecord((hipEvent_t)ev[i], st) : hipSuccess;
    };
    HIPCHK(mark(0));
    // 1. combine: dY rows and gate gradients
    // e4m3 layers: the Dgrad inputs dY and dO also in 1 x 128 tiles along their reduction
    // (d), written by the same kernel from the bf16 values it stores
    HIPCHK(launch_bwd_combine(dt, dout, Fw + F.yperm, inv, tw, T, d, s->topk, dy, dg, fp8 ? U8(L.dyq) : nullptr,
                              fp8 ? F32(L.dys) : nullptr, fp8 && Ns ? U8(L.doq) : nullptr,
                              fp8 && Ns ? F32(L.dos) : nullptr, st));
    HIPCHK(mark(1));
    // 2. dH = dY . W_down (transposed copies [n][I][d])
    FfnProblem p[2] = {}, q[2] = {};
    p[0].n_exp = s->n_routed;
    p[0].offsets = offsets;
    p[0].x = fp8 ? (const void *)U8(L.dyq) : dy;
    p[0].xs = fp8 ? F32(L.dys) : nullptr;
    p[0].w0 = routed_wt[0];
    p[0].s0 = fp8 ? routed_wt_s[0] : nullptr;
    p[0].out = dh;
    if (Ns) {
        p[1].n_exp = Ns;
        p[1].rows_fixed = T;
        p[1].x_local = 1;
        p[1].x = fp8 ? (const void *)U8(L.doq) : dout;
        p[1].xs = fp8 ? F32(L.dos) : nullptr;
        p[1].w0 = shared_wt[0];
        p[1].s0 = fp8 ? shared_wt_s[0] : nullptr;
        p[1].out = dh_s;
    }
    FfnArgs fa{};
    fa.nprob = Ns ? 2 : 1;
    fa.ctr = (int *)(W + L.fq);
    fa.K = d;
    fa.F = I;
    for (int i = 0; i < fa.nprob; ++i) fa.p[i] = p[fa.nprob - 1 - i];
    HIPCHK(launch_ffn(wdt, FFN_BWD_DH, fa, st));
    HIPCHK(mark(2));
    // 3. gate/up recomputed from u (e4m3: the forward's 1 x 128 tiles of u); SwiGLU gradient -> [dA | dB]
    const void *xin = fp8 ? (const void *)(Fw + F.uq) : u;
    const float *xsin = fp8 ? (const float *)(Fw + F.us) : nullptr;
    q[0].n_exp = s->n_routed;
    q[0].offsets = offsets;
    q[0].gather = perm;
    q[0].x = xin;
    q[0].xs = xsin;
    q[0].w0 = routed_w[0];
    q[0].w1 = routed_w[1];
    q[0].s0 = fp8 ? routed_s[0] : nullptr;
    q[0].s1 = fp8 ? routed_s[1] : nullptr;
    q[0].dh = dh;
    q[0].out = dab;
    q[0].out_ld = 2 * I;
    if (Ns) {
        q[1].n_exp = Ns;
        q[1].rows_fixed = T;
        q[1].x_local = 1;
        q[1].x = xin;
        q[1].xs = xsin;
        q[1].w0 = shared_w[0];
        q[1].w1 = shared_w[1];
        q[1].s0 = fp8 ? shared_s[0] : nullptr;
        q[1].s1 = fp8 ? shared_s[1] : nullptr;
        q[1].dh = dh_s;
        q[1].out = dab_s;
        q[1].out_ld = 2 * I;
    }
    if (s->flags & MOE_SAVE_SWIGLU_INPUTS) {
        // the forward kept a | b for the routed rows and then the shared rows, as dh and dab lie
        // (e4m3 layers: with the 1 x 128 tiles of [dA dB], the Dgrad input of dX)
        HIPCHK(launch_swiglu_grad(wdt == DT_F32 ? DT_F32 : DT_BF16, dh, (const float *)(Fw + F.ab), dab,
                                  TK + T * Ns, I, fp8 ? U8(L.abq) : nullptr, fp8 ? F32(L.abs_) : nullptr, st));
    } else {
        for (int i = 0; i < fa.nprob; ++i) fa.p[i] = q[fa.nprob - 1 - i];
        HIPCHK(launch_ffn(wdt, FFN_GATEUP_BWD, fa, st));
        if (fp8) HIPCHK(launch_quant_rows(dt, dab, nullptr, TK + T * Ns, 2 * I, U8(L.abq), F32(L.abs_), st));
    }
    HIPCHK(mark(3));
    // 4. dX = [dA | dB] . [W_gate ; W_up] (transposed copies [n][d][2I])
    FfnProblem r[2] = {};
    r[0].n_exp = s->n_routed;
    r[0].offsets = offsets;
    r[0].x = fp8 ? (const void *)U8(L.abq) : dab;
    r[0].xs = fp8 ? F32(L.abs_) : nullptr;
    r[0].w0 = routed_wt[1];
    r[0].s0 = fp8 ? routed_wt_s[1] : nullptr;
    r[0].out = dx;
    if (Ns) {
        r[1].n_exp = Ns;
        r[1].rows_fixed = T;
        r[1].x = fp8 ? (const void *)(U8(L.abq) + (size_t)TK * 2 * I) : dab_s;
        r[1].xs = fp8 ? F32(L.abs_) + (size_t)TK * (2 * I / 128) : nullptr;
        r[1].w0 = shared_wt[1];
        r[1].s0 = fp8 ? shared_wt_s[1] : nullptr;
        r[1].out = dx_s;
    }
    fa.K = 2 * I;
    fa.F = d;
    for (int i = 0; i < fa.nprob; ++i) fa.p[i] = r[fa.nprob - 1 - i];
    HIPCHK(launch_ffn(wdt, FFN_BWD_DX, fa, st));
    HIPCHK(mark(4));
    // 5. du: dispatch sum and router chain; dz per row
    HIPCHK(launch_bwd_token(dt, dx, dx_s, Ns, inv, idx, scores, dg, gate_w, T, d, s->n_routed, s->topk,
                            s->routed_scale, du, dz, st));
    HIPCHK(mark(5));
    // 6. centroid gradient
    if (dgate_w) HIPCHK(launch_dgate(dt, u, perm, offsets, dz, s->n_routed, d, dgate_w, st));
    HIPCHK(mark(6));
    // 7. weight gradients: down (dY rows x H rows), then gate/up ([dA | dB] rows x gathered u rows);
    // e4m3: both operands of both passes re-tiled 128 x 1 along the expert's rows first
    const bool wgr = d_routed_w || (Ns && d_shared_w);
    int32_t *bbase = fp8 ? (int32_t *)(W + L.bbase) : nullptr;
    const uint8_t *hq = (const uint8_t *)(Fw + F.h), *hsq = (const uint8_t *)(Fw + F.hsh);
    const float *hs = (const float *)(Fw + F.hs), *hss = (const float *)(Fw + F.hshs);
    if (fp8 && wgr) {
        const uint8_t *uq = (const uint8_t *)(Fw + F.uq);
        const float *us = (const float *)(Fw + F.us);
        if (d_routed_w) {
            HIPCHK(launch_block_base(offsets, s->n_routed, bbase, st));
            HIPCHK(launch_quant_cols(DT_BF16, dy, nullptr, nullptr, offsets, bbase, 0, s->n_routed, L.rblk, d,
                                     U8(L.p1q), F32(L.p1s), st));
            HIPCHK(launch_quant_cols(DT_E4M3, hq, hs, nullptr, offsets, bbase, 0, s->n_routed, L.rblk, I,
                                     U8(L.q1q), F32(L.q1s), st));
            HIPCHK(launch_quant_cols(DT_BF16, dab, nullptr, nullptr, offsets, bbase, 0, s->n_routed, L.rblk, 2 * I,
                                     U8(L.p2q), F32(L.p2s), st));
            HIPCHK(launch_quant_cols(DT_E4M3, uq, us, perm, offsets, bbase, 0, s->n_routed, L.rblk, d, U8(L.q2q),
                                     F32(L.q2s), st));
        }
        if (Ns && d_shared_w) {
            HIPCHK(launch_quant_cols(DT_BF16, dout, nullptr, nullptr, nullptr, nullptr, T, 1, L.sblk, d,
                                     U8(L.sp1q), F32(L.sp1s), st));
            HIPCHK(launch_quant_cols(DT_E4M3, hsq, hss, nullptr, nullptr, nullptr, T, Ns, Ns * L.sblk, I,
                                     U8(L.sq1q), F32(L.sq1s), st));
            HIPCHK(launch_quant_cols(DT_BF16, dab_s, nullptr, nullptr, nullptr, nullptr, T, Ns, Ns * L.sblk, 2 * I,
                                     U8(L.sp2q), F32(L.sp2s), st));
            HIPCHK(launch_quant_cols(DT_E4M3, uq, us, nullptr, nullptr, nullptr, T, 1, L.sblk, d, U8(L.sq2q),
                                     F32(L.sq2s), st));
        }
    }
    HIPCHK(mark(7));
    if (wgr) {
        // shared experts first: their long reductions start early, spread over every XCD
        const int64_t hint = (TK + s->n_routed - 1) / s->n_routed;
        WgradArgs wa{};
        int np = 0;
        if (Ns && d_shared_w) {
            WgradProblem &w = wa.p[np++];
            w.n_exp = Ns;
            w.rows_fixed = T;
            w.rows_hint = T;
            w.p_local = 1;
            w.P = fp8 ? (const void *)U8(L.sp1q) : dout;
            w.Ps = fp8 ? F32(L.sp1s) : nullptr;
            w.P_ld = d;
            w.Q = fp8 ? (const void *)U8(L.sq1q) : (const void *)hsq;
            w.Qs = fp8 ? F32(L.sq1s) : nullptr;
            w.Q_ld = I;
            w.Pdim = d;
            w.Qdim = I;
            w.split = d;
            w.out0 = d_shared_w[2];
        }
        if (d_routed_w) {
            WgradProblem &w = wa.p[np++];
            w.n_exp = s->n_routed;
            w.offsets = offsets;
            w.bbase = bbase;
            w.rows_hint = hint;
            w.P = fp8 ? (const void *)U8(L.p1q) : dy;
            w.Ps = fp8 ? F32(L.p1s) : nullptr;
            w.P_ld = d;
            w.Q = fp8 ? (const void *)U8(L.q1q) : (const void *)hq;
            w.Qs = fp8 ? F32(L.q1s) : nullptr;
            w.Q_ld = I;
            w.Pdim = d;
            w.Qdim = I;
            w.split = d;
            w.out0 = d_routed_w[2];
        }
        wa.nprob = np;
        HIPCHK(launch_wgrad(wdt, 0, wa, st));
        HIPCHK(mark(8));
        np = 0;
        if (Ns && d_shared_w) {
            WgradProblem &w = wa.p[np++];
            w = WgradProblem{};
            w.n_exp = Ns;
            w.rows_fixed = T;
            w.rows_hint = T;
            w.q_local = 1;
            w.P = fp8 ? (const void *)U8(L.sp2q) : dab_s;
            w.Ps = fp8 ? F32(L.sp2s) : nullptr;
            w.P_ld = 2 * I;
            w.Q = fp8 ? (const void *)U8(L.sq2q) : u;
            w.Qs = fp8 ? F32(L.sq2s) : nullptr;
            w.Q_ld = d;
            w.Pdim = 2 * I;
            w.Qdim = d;
            w.split = I;
            w.out0 = d_shared_w[0];
            w.out1 = d_shared_w[1];
        }
        if (d_routed_w) {
            WgradProblem &w = wa.p[np++];
            w = WgradProblem{};
            w.n_exp = s->n_routed;
            w.offsets = offsets;
            w.bbase = bbase;
            w.rows_hint = hint;
            w.P = fp8 ? (const void *)U8(L.p2q) : dab;
            w.Ps = fp8 ? F32(L.p2s) : nullptr;
            w.P_ld = 2 * I;
            w.Q = fp8 ? (const void *)U8(L.q2q) : u;
            w.Qs = fp8 ? F32(L.q2s) : nullptr;
            w.Q_ld = d;
            w.q_gather = fp8 ? nullptr : perm;   // e4m3: the 128 x 1 copy is already gathered
            w.Pdim = 2 * I;
            w.Qdim = d;
            w.split = I;
            w.out0 = d_routed_w[0];
            w.out1 = d_routed_w[1];
        }
        wa.nprob = np;
        HIPCHK(launch_wgrad(wdt, 1, wa, st));
    } else {
        HIPCHK(mark(8));
    }
    HIPCHK(mark(9));
    return MOE_OK;
}

int moe_backward(const moe_shape *s, const void *u, const void *gate_w, const void *const *routed_w,
                 const float *const *routed_s, const void *const *routed_wt, const float *const *routed_wt_s,
                 const void *const *shared_w, const float *const *shared_s, const void *const *shared_wt,
                 const float *const *shared_wt_s, const void *fwd_ws, size_t fwd_ws_bytes, const void *dout, void *du,
                 float *dgate_w, void *const *d_routed_w, void *const *d_shared_w, float *dtopk_w, void *ws,
                 size_t ws_bytes, void *stream) {
    return backward_impl(s, u, gate_w, routed_w, routed_s, routed_wt, routed_wt_s, shared_w, shared_s, shared_wt,
                         shared_wt_s, fwd_ws, fwd_ws_bytes, dout, du, dgate_w, d_routed_w, d_shared_w, dtopk_w, ws,
                         ws_bytes, stream, nullptr);
}

int moe_backward_timed(const moe_shape *s, const void *u, const void *gate_w, const void *const *routed_w,
                       const float *const *routed_s, const void *const *routed_wt, const float *const *routed_wt_s,
                       const void *const *shared_w, const float *const *shared_s, const void *const *shared_wt,
                       const float *const *shared_wt_s, const void *fwd_ws, size_t fwd_ws_bytes, const void *dout,
                       void *du, float *dgate_w, void *const *d_routed_w, void *const *d_shared_w, float *dtopk_w,
                       void *ws, size_t ws_bytes, void *stream, void *const *stage_events) {
    return backward_impl(s, u, gate_w, routed_w, routed_s, routed_wt, routed_wt_s, shared_w, shared_s, shared_wt,
                         shared_wt_s, fwd_ws, fwd_ws_bytes, dout, du, dgate_w, d_routed_w, d_shared_w, dtopk_w, ws,
                         ws_bytes, stream, stage_events);
}

size_t moe_seq_balance_workspace_bytes(const moe_shape *s, int64_t seq_len) {
    if (check_shape(s, "moe_seq_balance_workspace_bytes") != MOE_OK) return 0;
    if (seq_len < 1) { fail(MOE_ERR_INVALID_ARG, "moe_seq_balance_workspace_bytes: seq_len < 1"); return 0; }
    const int64_t n_seq = (s->T + seq_len - 1) / seq_len;
    const size_t rows = (size_t)(n_seq * balance_blocks_per_seq(s->T, seq_len));
    return align256(rows * s->n_routed * 4) * 2;
}

int moe_seq_balance(const moe_shape *s, const float *scores, const int32_t *topk_idx, int64_t seq_len, float alpha,
                    float *loss, int32_t *counts, float *share, void *ws, size_t ws_bytes, void *stream) {
    const char *fn = "moe_seq_balance";
    int rc = check_shape(s, fn);
    if (rc) return rc;
    if (seq_len < 1) return fail(MOE_ERR_INVALID_ARG, "%s: seq_len = %lld must be >= 1", fn, (long long)seq_len);
    if (s->T == 0) return MOE_OK;
    NEED(scores);
    NEED(topk_idx);
    NEED(loss);
    rc = ws_check(ws, ws_bytes, moe_seq_balance_workspace_bytes(s, seq_len), fn);
    if (rc) return rc;
    const int64_t n_seq = (s->T + seq_len - 1) / seq_len;
    const size_t rows = (size_t)(n_seq * balance_blocks_per_seq(s->T, seq_len));
    float *ps = (float *)ws;
    int32_t *pc = (int32_t *)((char *)ws + align256(rows * s->n_routed * 4));
    HIPCHK(launch_seq_balance(scores, topk_idx, s->T, s->n_routed, s->topk, seq_len, alpha, loss, counts, share, ps, pc,
                              (hipStream_t)stream));
    return MOE_OK;
}

int moe_bias_update(const moe_shape *s, const int32_t *counts, float *bias, float gamma, void *stream) {
    const char *fn = "moe_bias_update";
    int rc = check_shape(s, fn);
    if (rc) return rc;
    NEED(counts);
    NEED(bias);
    HIPCHK(launch_bias_update(counts, bias, s->T, s->topk, s->n_routed, gamma, (hipStream_t)stream));
    return MOE_OK;
}

int moe_quantize_1x128(int64_t rows, int32_t cols, int32_t x_dtype, const void *x, uint8_t *q, float *sc,
                       void *stream) {
    const char *fn = "moe_quantize_1x128";
    if (rows < 0 || cols <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: bad size", fn);
    if (cols % 128) return fail(MOE_ERR_UNSUPPORTED, "%s: cols = %d is not a multiple of 128", fn, cols);
    if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "%s: x_dtype %d", fn, x_dtype);
    NEED(x);
    NEED(q);
    NEED(sc);
    HIPCHK(launch_quant_rows(dt_of(x_dtype), x, nullptr, rows, cols, q, sc, (hipStream_t)stream));
    return MOE_OK;
}

int moe_quantize_weights_128x128(int64_t nmat, int32_t rows, int32_t cols, int32_t w_dtype, const void *w,
                                 uint8_t *q, float *sc, void *stream) {
    const char *fn = "moe_quantize_weights_128x128";
    if (nmat < 0 || rows <= 0 || cols <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: bad size", fn);
    if (rows % 128 || cols % 128) return fail(MOE_ERR_UNSUPPORTED, "%s: rows and cols must be multiples of 128", fn);
    if (w_dtype != MOE_F32 && w_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "%s: w_dtype %d", fn, w_dtype);
    if (nmat * (rows / 128) * (int64_t)(cols / 128) >= (1ll << 31))
        return fail(MOE_ERR_UNSUPPORTED, "%s: too many blocks for one call", fn);
    NEED(w);
    NEED(q);
    NEED(sc);
    HIPCHK(launch_quant_blocks(dt_of(w_dtype), w, nmat, rows, cols, q, sc, (hipStream_t)stream));
    return MOE_OK;
}

int moe_quantize_128x1(int32_t n_seg, const int32_t *offsets, int64_t max_rows, int32_t cols, int32_t x_dtype,
                       const void *x, const float *x_s, const int32_t *gather, uint8_t *q, float *sc,
                       int32_t *block_base, void *stream) {
    const char *fn = "moe_quantize_128x1";
    if (n_seg < 0 || max_rows < 0 || cols <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: bad size", fn);
    if (cols % 128) return fail(MOE_ERR_UNSUPPORTED, "%s: cols = %d is not a multiple of 128", fn, cols);
    if (x_dtype != MOE_BF16 && x_dtype != MOE_E4M3) return fail(MOE_ERR_UNSUPPORTED, "%s: x_dtype %d", fn, x_dtype);
    if (n_seg == 0) return MOE_OK;
    NEED(offsets);
    NEED(x);
    if (x_dtype == MOE_E4M3) NEED(x_s);
    NEED(q);
    NEED(sc);
    NEED(block_base);
    const int64_t max_blocks = max_rows / 128 + n_seg;
    if (max_blocks >= (1ll << 31)) return fail(MOE_ERR_UNSUPPORTED, "%s: too many runs for one call", fn);
    const hipStream_t s = (hipStream_t)stream;
    HIPCHK(launch_block_base(offsets, n_seg, block_base, s));
    HIPCHK(launch_quant_cols(dt_of(x_dtype), x, x_s, gather, offsets, block_base, 0, n_seg, max_blocks, cols, q, sc, s));
    return MOE_OK;
}

}  // extern "C"
