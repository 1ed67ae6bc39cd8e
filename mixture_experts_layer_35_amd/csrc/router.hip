// router.hip -- token-to-expert affinities and auxiliary-loss-free group-limited
// top-K selection ("DeepSeek-V3 Technical Report", §2.1.2: sigmoid affinities,
// bias used for selection only, gates normalised over the selected un-biased
// affinities, node-limited routing; §4.2: 8 of 256 experts, at most 4 groups).
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kPitch = 144;  // LDS bytes per staged 128-byte row (16 bytes of padding)

// ---------------------------------------------------------------------------
// Gate GEMM + sigmoid.  Tile: 64 experts x 64 tokens, reduction staged in
// 128-byte rows through double-buffered LDS; four waves, each 32 x 32 as
// 2 x 2 blocks of 16x16 MFMA outputs with experts on the MFMA row side, so a
// lane ends up holding four consecutive experts of one token (one 16-byte
// store of fp32 scores).
// ---------------------------------------------------------------------------
template <int DT>
struct RTraits;
template <>
struct RTraits<DT_F32> {
    static constexpr int kSub = 8;   // 16x16x4 steps per 128-byte row
    typedef float frag;
    __device__ static frag load(const char *row, int s, int lane) {
        return *(const float *)(row + s * 16 + (lane >> 4) * 4);
    }
    __device__ static f32x4 mma(frag a, frag b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }
};
template <>
struct RTraits<DT_BF16> {
    static constexpr int kSub = 2;   // 16x16x32 steps per 128-byte row
    typedef bf16x8 frag;
    __device__ static frag load(const char *row, int s, int lane) {
        return *(const bf16x8 *)(row + s * 64 + (lane >> 4) * 16);
    }
    __device__ static f32x4 mma(frag a, frag b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
};

template <int DT>
__global__ __launch_bounds__(256) void router_gemm_kernel(const char *__restrict__ u, const char *__restrict__ gw,
                                                          float *__restrict__ scores, int64_t T, int d, int Nr) {
    typedef RTraits<DT> Tr;
    constexpr int esz = DT == DT_F32 ? 4 : 2;
    __shared__ __align__(16) char lds[2][128 * kPitch];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wt = wid & 1, we = wid >> 1;
    const int64_t t0 = (int64_t)blockIdx.x * 64;
    const int e0 = blockIdx.y * 64;
    const int64_t rowbytes = (int64_t)d * esz;

    // 128 rows (64 experts, then 64 tokens) x 8 chunks of 16 bytes = 4 chunks per thread
    const char *src[4];
    int dst[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        int chunk = tid + c * 256, row = chunk >> 3, col = chunk & 7;
        const char *p;
        if (row < 64) {
            int e = min(e0 + row, Nr - 1);
            p = gw + (int64_t)e * rowbytes;
        } else {
            int64_t t = min(t0 + row - 64, T - 1);
            p = u + t * rowbytes;
        }
        src[c] = p + col * 16;
        dst[c] = row * kPitch + col * 16;
    }
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

    const int KT = (int)(rowbytes / 128);
    u32x4 stage[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) stage[c] = *(const u32x4 *)(src[c]);
#pragma unroll
    for (int c = 0; c < 4; ++c) *(u32x4 *)(lds[0] + dst[c]) = stage[c];
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) {
#pragma unroll
            for (int c = 0; c < 4; ++c) stage[c] = *(const u32x4 *)(src[c] + (int64_t)(kt + 1) * 128);
        }
        const char *Es = lds[cur];
        const char *Us = lds[cur] + 64 * kPitch;
#pragma unroll
        for (int s = 0; s < Tr::kSub; ++s) {
            typename Tr::frag a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = Tr::load(Es + (we * 32 + i * 16 + (lane & 15)) * kPitch, s, lane);
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j] = Tr::load(Us + (wt * 32 + j * 16 + (lane & 15)) * kPitch, s, lane);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = Tr::mma(a[i], b[j], acc[i][j]);
        }
        if (kt + 1 < KT) {
#pragma unroll
            for (int c = 0; c < 4; ++c) *(u32x4 *)(lds[cur ^ 1] + dst[c]) = stage[c];
        }
        __syncthreads();
    }
    // epilogue: lane holds experts e0 + we*32 + i*16 + 4*(lane>>4) + {0..3} of token t0 + wt*32 + j*16 + (lane&15)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        int64_t t = t0 + wt * 32 + j * 16 + (lane & 15);
        if (t >= T) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int e = e0 + we * 32 + i * 16 + 4 * (lane >> 4);
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = 1.0f / (1.0f + expf(-acc[i][j][q]));
            float *dstp = scores + t * Nr + e;
            if (e + 3 < Nr && (Nr & 3) == 0) {
                *(f32x4 *)dstp = f32x4{v[0], v[1], v[2], v[3]};
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (e + q < Nr) dstp[q] = v[q];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Selection: one wave per token.  Lane l holds experts l, l+64, ... (R of them).
// Ordering keys pack (value, index) so that a single 64-bit max picks the
// larger value and, on equal values, the lower index.
// ---------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(256) void router_select_kernel(const float *__restrict__ scores,
                                                            const float *__restrict__ bias, int64_t T, int Nr, int G,
                                                            int Mg, int K, float routed_scale,
                                                            int32_t *__restrict__ topk_idx,
                                                            float *__restrict__ topk_w) {
    __shared__ float sb_all[4][64 * R];
    __shared__ float s_all[4][64 * R];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * 4 + wid;
    const bool live = t < T;                 // uniform per wave
    float *sb = sb_all[wid];
    float *sr = s_all[wid];
    const int gs = Nr / G;

    uint64_t key[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int i = lane + 64 * r;
        if (live && i < Nr) {
            float s = scores[t * Nr + i];
            float b = s + bias[i];              // one fp32 add; bias only steers selection
            sb[i] = b;
            sr[i] = s;
        }
    }
    __syncthreads();
    if (!live) return;

    // group scores: lane g < G scans its group: sum of the two largest biased affinities
    uint64_t gkey = 0;
    if (lane < G) {
        float m1 = -INFINITY, m2 = -INFINITY;
        for (int i = lane * gs; i < (lane + 1) * gs; ++i) {
            float v = sb[i];
            if (v > m1) { m2 = m1; m1 = v; }
            else if (v > m2) { m2 = v; }
        }
        float score = gs == 1 ? m1 : m1 + m2;
        gkey = order_key(score, lane);
    }
    uint64_t kept = 0;
    for (int r = 0; r < Mg; ++r) {
        uint64_t best = wave_max_u64(gkey);
        int g = key_index(best);
        kept |= 1ull << g;
        if (lane == g) gkey = 0;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int i = lane + 64 * r;
        key[r] = (i < Nr && ((kept >> (i / gs)) & 1ull)) ? order_key(sb[i], i) : 0ull;
    }
    int my_e = 0;
    float my_s = 0.0f;
    float den = 0.0f;
    for (int j = 0; j < K; ++j) {
        uint64_t local = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) local = key[r] > local ? key[r] : local;
        uint64_t best = wave_max_u64(local);
        int e = key_index(best);
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (r == (e >> 6) && lane == (e & 63)) key[r] = 0;
        float s = sr[e];
        den = den + s;                               // slot order, fp32
        if (lane == j) { my_e = e; my_s = s; }
    }
    if (lane < K) {
        topk_idx[t * K + lane] = my_e;
        topk_w[t * K + lane] = (my_s / den) * routed_scale;
    }
}

}  // namespace

hipError_t launch_router_gemm(int dt, const void *u, const void *gate_w, float *scores, int64_t T, int d, int Nr,
                              hipStream_t s) {
    if (T <= 0) return hipSuccess;
    dim3 grid((unsigned)((T + 63) / 64), (unsigned)((Nr + 63) / 64));
    if (dt == DT_F32)
        router_gemm_kernel<DT_F32><<<grid, 256, 0, s>>>((const char *)u, (const char *)gate_w, scores, T, d, Nr);
    else
        router_gemm_kernel<DT_BF16><<<grid, 256, 0, s>>>((const char *)u, (const char *)gate_w, scores, T, d, Nr);
    return hipGetLastError();
}

hipError_t launch_router_select(const float *scores, const float *bias, int64_t T, int Nr, int G, int Mg, int K,
                                float routed_scale, int32_t *topk_idx, float *topk_w, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    dim3 grid((unsigned)((T + 3) / 4));
    int R = (Nr + 63) / 64;
#define SEL(RR) router_select_kernel<RR><<<grid, 256, 0, s>>>(scores, bias, T, Nr, G, Mg, K, routed_scale, topk_idx, topk_w)
    if (R <= 1) SEL(1);
    else if (R <= 2) SEL(2);
    else if (R <= 4) SEL(4);
    else if (R <= 8) SEL(8);
    else SEL(16);
#undef SEL
    return hipGetLastError();
}

}  // namespace moe
