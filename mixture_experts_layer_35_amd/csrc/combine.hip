// combine.hip -- layer output and the auxiliary-loss-free bias step
// ("DeepSeek-V3 Technical Report", §2.1.2: output = shared experts + gate-weighted
// routed experts; the per-expert bias moves by gamma against the whole-batch
// load after each step; §4.2: gamma = 0.001).
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

template <int DT>
__device__ __forceinline__ void ld8(const char *p, float v[8]) {
    if (DT == DT_BF16) {
        u32x4 w = *(const u32x4 *)p;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
    }
}

// One workgroup per token (grid-stride); each thread owns 8 consecutive features
// per step.  fp32 accumulation, one rounding on store.
template <int DT, int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const char *__restrict__ y_perm, const int32_t *__restrict__ inv,
                                                     const float *__restrict__ topk_w, const char *__restrict__ y_sh,
                                                     int Ns, const char *__restrict__ res, int res_dt,
                                                     char *__restrict__ out, int64_t T, int d, int K) {
    constexpr int esz = DT == DT_F32 ? 4 : 2;
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        int64_t rows[KMAX];
        float w[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j < K) {
                rows[j] = inv[t * K + j];
                w[j] = topk_w[t * K + j];
            }
        }
        for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
            float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                if (j < K) {
                    float v[8];
                    ld8<DT>(y_perm + (rows[j] * d + c) * esz, v);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] += w[j] * v[i];
                }
            }
            for (int s = 0; s < Ns; ++s) {
                float v[8];
                ld8<DT>(y_sh + (((int64_t)s * T + t) * d + c) * esz, v);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += v[i];
            }
            if (res) {
                float v[8];
                if (res_dt == DT_BF16) ld8<DT_BF16>(res + (t * d + c) * 2, v);
                else ld8<DT_F32>(res + (t * d + c) * 4, v);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += v[i];
            }
            if (DT == DT_BF16) {
                *(u32x4 *)(out + (t * d + c) * 2) = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                          pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
            } else {
                *(f32x4 *)(out + (t * d + c) * 4) = f32x4{acc[0], acc[1], acc[2], acc[3]};
                *(f32x4 *)(out + (t * d + c) * 4 + 16) = f32x4{acc[4], acc[5], acc[6], acc[7]};
            }
        }
    }
}

// mean = fp32(T*K) / fp32(Nr); b_i = b_i + gamma * sign(mean - load_i), sign(0) = 0.
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
    const unsigned grid = (unsigned)(T < 16384 ? T : 16384);
#define COMB(DT, KM)                                                                                                   \
    combine_kernel<DT, KM><<<grid, 256, 0, s>>>((const char *)y_perm, inv_perm, topk_w, (const char *)y_shared, Ns,   \
                                                (const char *)residual, dt_res, (char *)out, T, d, K)
    if (dt_out == DT_BF16) {
        if (K <= 8) COMB(DT_BF16, 8); else COMB(DT_BF16, 32);
    } else {
        if (K <= 8) COMB(DT_F32, 8); else COMB(DT_F32, 32);
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
