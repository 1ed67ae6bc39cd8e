// combine.hip -- layer output and the auxiliary-loss-free bias step
// ("DeepSeek-V3 Technical Report", §2.1.2: output = shared experts + gate-weighted
// routed experts; the per-expert bias moves by gamma against the whole-batch
// load after each step; §4.2: gamma = 0.001).
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

// 16 consecutive features of one row, loaded as raw 16-byte words so that all
// of a token's row loads can be in flight before the first is used.
template <int DT>
struct Raw16 {
    static constexpr int N = DT == DT_BF16 ? 2 : 4;
    u32x4 w[N];
    __device__ void load(const char *p) {
#pragma unroll
        for (int i = 0; i < N; ++i) w[i] = __builtin_nontemporal_load((const u32x4 *)p + i);
    }
    __device__ void get(float v[16]) const {
#pragma unroll
        for (int i = 0; i < N; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (DT == DT_BF16) {
                    v[8 * i + 2 * k] = __uint_as_float(w[i][k] << 16);
                    v[8 * i + 2 * k + 1] = __uint_as_float(w[i][k] & 0xFFFF0000u);
                } else {
                    v[4 * i + k] = __uint_as_float(w[i][k]);
                }
            }
    }
};

// One workgroup per token (grid-stride); each thread owns 16 consecutive
// features.  Selected rows are taken eight (fp32: four) at a time, and each batch's loads
// (with the first shared expert's) are all issued before any is used; fp32
// accumulation in slot order, one rounding on store.
template <int DT, bool K8>
__global__ __launch_bounds__(1024) void combine_kernel(const char *__restrict__ y_perm, const int32_t *__restrict__ inv,
                                                      const float *__restrict__ topk_w, const char *__restrict__ y_sh,
                                                      int Ns, const char *__restrict__ res, int res_dt,
                                                      char *__restrict__ out, int64_t T, int d, int K) {
    constexpr int esz = DT == DT_F32 ? 4 : 2;
    constexpr int NB = DT == DT_F32 ? 4 : 8;      // rows per batch (register budget)
    if (K8) K = 8;
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        const int32_t *rows = inv + t * K;
        const float *w = topk_w + t * K;
        for (int c = threadIdx.x * 16; c < d; c += blockDim.x * 16) {
            float acc[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
            Raw16<DT> sh;
            for (int j0 = 0; j0 < K; j0 += NB) {
                Raw16<DT> r[NB];
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    if (K8 || j0 + j < K) r[j].load(y_perm + ((int64_t)rows[j0 + j] * d + c) * esz);
                if (j0 == 0 && Ns > 0) sh.load(y_sh + (t * d + c) * esz);
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    if (K8 || j0 + j < K) {
                        float v[16];
                        r[j].get(v);
                        const float wj = w[j0 + j];
#pragma unroll
                        for (int i = 0; i < 16; ++i) acc[i] += wj * v[i];
                    }
                }
            }
            for (int s = 0; s < Ns; ++s) {
                float v[16];
                if (s == 0) {
                    sh.get(v);
                } else {
                    Raw16<DT> x;
                    x.load(y_sh + (((int64_t)s * T + t) * d + c) * esz);
                    x.get(v);
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] += v[i];
            }
            if (res) {
                float v[16];
                if (res_dt == DT_BF16) {
                    Raw16<DT_BF16> x;
                    x.load(res + (t * d + c) * 2);
                    x.get(v);
                } else {
                    Raw16<DT_F32> x;
                    x.load(res + (t * d + c) * 4);
                    x.get(v);
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] += v[i];
            }
            if (DT == DT_BF16) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    *(u32x4 *)(out + (t * d + c + 8 * h) * 2) =
                        u32x4{pack_bf16x2(acc[8 * h], acc[8 * h + 1]), pack_bf16x2(acc[8 * h + 2], acc[8 * h + 3]),
                              pack_bf16x2(acc[8 * h + 4], acc[8 * h + 5]), pack_bf16x2(acc[8 * h + 6], acc[8 * h + 7])};
            } else {
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    *(f32x4 *)(out + (t * d + c + 4 * h) * 4) =
                        f32x4{acc[4 * h], acc[4 * h + 1], acc[4 * h + 2], acc[4 * h + 3]};
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
    // one thread per 16 features (whole waves), at most 1024; one workgroup per token
    const int nt = min(1024, (d / 16 + 63) / 64 * 64);
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
