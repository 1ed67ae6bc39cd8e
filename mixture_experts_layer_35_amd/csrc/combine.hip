// combine.hip -- layer output and the auxiliary-loss-free bias step
// ("DeepSeek-V3 Technical Report", §2.1.2: output = shared experts + gate-weighted
// routed experts; the per-expert bias moves by gamma against the whole-batch
// load after each step; §4.2: gamma = 0.001).
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

// A row is read and written in 16-byte chunks (8 bf16 or 4 fp32 features).  Thread
// (wave w, lane l) owns the NC chunks w*64*NC + l + 64*i (i < NC), 16 features in all,
// so each 16-byte load or store instruction of a wave covers 1 KB of one row.
template <int DT>
struct Chunk {
    static constexpr int NC = DT == DT_BF16 ? 2 : 4;    // chunks per thread
    static constexpr int FPC = DT == DT_BF16 ? 8 : 4;   // features per chunk
    __device__ static u32x4 load(const char *row, int c) { return __builtin_nontemporal_load((const u32x4 *)row + c); }
    __device__ static void get(u32x4 w, float *v) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (DT == DT_BF16) {
                v[2 * k] = __uint_as_float(w[k] << 16);
                v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
            } else {
                v[k] = __uint_as_float(w[k]);
            }
        }
    }
};

// One workgroup per token (grid-stride).  Selected rows are taken eight (fp32: two) at
// a time, and each batch's loads (with the first shared expert's) are all issued before
// any is used; fp32 accumulation in slot order, one rounding on store.
template <int DT, bool K8>
__global__ __launch_bounds__(1024) void combine_kernel(const char *__restrict__ y_perm, const int32_t *__restrict__ inv,
                                                      const float *__restrict__ topk_w, const char *__restrict__ y_sh,
                                                      int Ns, const char *__restrict__ res, int res_dt,
                                                      char *__restrict__ out, int64_t T, int d, int K) {
    typedef Chunk<DT> C;
    constexpr int NC = C::NC, FPC = C::FPC;
    constexpr int esz = DT == DT_F32 ? 4 : 2;
    constexpr int NB = DT == DT_F32 ? 2 : 8;      // rows per batch (register budget)
    if (K8) K = 8;
    const int nch = d / FPC;
    const int64_t rowb = (int64_t)d * esz;
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        const int32_t *rows = inv + t * K;
        const float *w = topk_w + t * K;
        for (int cb = (threadIdx.x >> 6) * 64 * NC + (threadIdx.x & 63); cb < nch; cb += (blockDim.x >> 6) * 64 * NC) {
            // chunk i of this thread; past the row's end a thread re-reads its first chunk and stores nothing
            auto ci = [&](int i) { return cb + 64 * i < nch ? cb + 64 * i : cb; };
            float acc[NC * FPC];
#pragma unroll
            for (int i = 0; i < NC * FPC; ++i) acc[i] = 0.0f;
            u32x4 sh[NC];
            for (int j0 = 0; j0 < K; j0 += NB) {
                u32x4 r[NB][NC];
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    if (K8 || j0 + j < K) {
                        const char *row = y_perm + (int64_t)rows[j0 + j] * rowb;
#pragma unroll
                        for (int i = 0; i < NC; ++i) r[j][i] = C::load(row, ci(i));
                    }
                if (j0 == 0 && Ns > 0)
#pragma unroll
                    for (int i = 0; i < NC; ++i) sh[i] = C::load(y_sh + t * rowb, ci(i));
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    if (K8 || j0 + j < K) {
                        const float wj = w[j0 + j];
#pragma unroll
                        for (int i = 0; i < NC; ++i) {
                            float v[FPC];
                            C::get(r[j][i], v);
#pragma unroll
                            for (int k = 0; k < FPC; ++k) acc[i * FPC + k] += wj * v[k];
                        }
                    }
                }
            }
            for (int s = 0; s < Ns; ++s) {
#pragma unroll
                for (int i = 0; i < NC; ++i) {
                    if (s > 0) sh[i] = C::load(y_sh + ((int64_t)s * T + t) * rowb, ci(i));
                    float v[FPC];
                    C::get(sh[i], v);
#pragma unroll
                    for (int k = 0; k < FPC; ++k) acc[i * FPC + k] += v[k];
                }
            }
            if (res) {
#pragma unroll
                for (int i = 0; i < NC; ++i) {
                    const int64_t f0 = t * d + (int64_t)ci(i) * FPC;   // first feature of the chunk
                    float v[FPC];
                    if (res_dt == DT_BF16) {
#pragma unroll
                        for (int k = 0; k < FPC; k += 2) {
                            const uint32_t x = ((const uint32_t *)res)[(f0 + k) / 2];
                            v[k] = __uint_as_float(x << 16);
                            v[k + 1] = __uint_as_float(x & 0xFFFF0000u);
                        }
                    } else {
#pragma unroll
                        for (int k = 0; k < FPC; k += 4) {
                            const f32x4 x = *((const f32x4 *)((const float *)res + f0 + k));
#pragma unroll
                            for (int q = 0; q < 4; ++q) v[k + q] = x[q];
                        }
                    }
#pragma unroll
                    for (int k = 0; k < FPC; ++k) acc[i * FPC + k] += v[k];
                }
            }
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                if (cb + 64 * i >= nch) continue;
                const float *a = acc + i * FPC;
                if (DT == DT_BF16)
                    *((u32x4 *)(out + t * rowb) + ci(i)) = u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                                                pack_bf16x2(a[4], a[5]), pack_bf16x2(a[6], a[7])};
                else
                    *((f32x4 *)(out + t * rowb) + ci(i)) = f32x4{a[0], a[1], a[2], a[3]};
            }
        }
    }
}

__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t *__restrict__ counts, float *__restrict__ bias,
                                                         float tk, int Nr, float gamma) {
    const float mean = tk / (float)Nr;
    for (int i = threadIdx.x; i < Nr; i += 256) {
        const float load = (float)counts[i];
        const float sgn = load < mean ? 1.0f : (load > mean ? -1.0f : 0.0f);
        bias[i] = bias[i] + gamma * sgn;
    }
}

__global__ void set_offsets_kernel(int32_t *off, int n, int64_t step) {
    for (int i = threadIdx.x; i <= n; i += blockDim.x) off[i] = (int32_t)(i * step);
}

}  // namespace

hipError_t launch_combine(int dt_out, int dt_res, const void *y_perm, const int32_t *inv_perm, const float *topk_w,
                          const void *y_shared, int Ns, const void *residual, void *out, int64_t T, int d, int K,
                          hipStream_t s) {
    if (T <= 0) return hipSuccess;
    // one thread per 16 features (whole waves, each over 1024 features), at most 1024; one
    // workgroup per token
    const int nt = min(1024, (d + 1023) / 1024 * 64);
    const unsigned grid = (unsigned)(T < (1 << 20) ? T : (1 << 20));
#define COMB(DT, K8)                                                                                                   \
    combine_kernel<DT, K8><<<grid, nt, 0, s>>>((const char *)y_perm, inv_perm, topk_w, (const char *)y_shared, Ns,     \
                                               (const char *)residual, dt_res, (char *)out, T, d, K)
    if (dt_out == DT_BF16) {
        if (K == 8) COMB(DT_BF16, true); else COMB(DT_BF16, false);
    } else {
        if (K == 8) COMB(DT_F32, true); else COMB(DT_F32, false);
    }
#undef COMB
    return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t *counts, float *bias, int64_t T, int K, int Nr, float gamma, hipStream_t s) {
    bias_update_kernel<<<1, 256, 0, s>>>(counts, bias, (float)(T * K), Nr, gamma);
    return hipGetLastError();
}

hipError_t launch_set_offsets(int32_t *offsets, int n, int64_t step, hipStream_t s) {
    set_offsets_kernel<<<1, 256, 0, s>>>(offsets, n, step);
    return hipGetLastError();
}

}  // namespace moe
