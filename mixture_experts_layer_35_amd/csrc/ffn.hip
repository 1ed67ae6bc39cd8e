// ffn.hip -- grouped SwiGLU expert FFN on MFMA ("DeepSeek-V3 Technical Report",
// §2.1.2: fine-grained routed experts plus shared experts; §3.3: FP8 GEMMs with
// 1 x 128 activation tiles and 128 x 128 weight blocks whose partial sums are
// promoted to fp32 every 128 products; §4.2: I = 2048 for every expert).
//
// One kernel, two passes:
//   gate/up pass: H[r, f] = SiLU(x_r . Wg[f]) * (x_r . Wu[f])   -> H (act dtype or e4m3 + 1x128 scales)
//   down pass:    Y[r, f] = H_r . Wd[f]                          -> y (out dtype)
// Rows are ragged per expert and only known on the device (offsets), so the
// grid is persistent and every workgroup walks a tile list derived from the
// offsets: tiles are (expert, feature block, row block) with the row blocks of
// one (expert, feature block) adjacent, so the weight tile they share is
// fetched once into the L2 of one XCD.  Up to two problems (routed experts and
// shared experts) share one launch.
//
// MFMA orientation: weights are the MFMA row operand and tokens the column
// operand, so each lane's four accumulator values are four consecutive output
// features of one token.
#include <mutex>

#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kPitch = 144;      // LDS bytes per staged 128-byte row
constexpr int kThreads = 256;

template <int DT>
struct FTraits;
template <>
struct FTraits<DT_F32> {
    static constexpr int esz = 4, kSub = 8;
    typedef float frag;
    __device__ static frag load(const char *row, int s, int lane) {
        return *(const float *)(row + s * 16 + (lane >> 4) * 4);
    }
    __device__ static f32x4 mma(frag a, frag b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }
};
template <>
struct FTraits<DT_BF16> {
    static constexpr int esz = 2, kSub = 2;
    typedef bf16x8 frag;
    __device__ static frag load(const char *row, int s, int lane) {
        return *(const bf16x8 *)(row + s * 64 + (lane >> 4) * 16);
    }
    __device__ static f32x4 mma(frag a, frag b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
};
template <>
struct FTraits<DT_E4M3> {
    // one 16x16x128 MFMA covers exactly one 128-long quantisation block
    static constexpr int esz = 1, kSub = 1;
    typedef i32x8 frag;
    __device__ static frag load(const char *row, int s, int lane) {
        return *(const i32x8 *)(row + (lane >> 4) * 32);
    }
    __device__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);   // unit E8M0 scales
    }
};

// Exclusive prefix of per-expert tile counts into pre[0..n]; pre[n] = total.
__device__ void tile_prefix(const FfnProblem &P, int bm, int ftiles, int *pre, int *scan) {
    const int tid = threadIdx.x;
    const int n = P.n_exp;
    const int per = (n + kThreads - 1) / kThreads;
    const int lo = min(tid * per, n), hi = min(lo + per, n);
    int local = 0;
    for (int e = lo; e < hi; ++e) {
        int m = P.offsets ? P.offsets[e + 1] - P.offsets[e] : (int)P.rows_fixed;
        local += (m + bm - 1) / bm * ftiles;
    }
    scan[tid] = local;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        int v = tid >= off ? scan[tid - off] : 0;
        __syncthreads();
        scan[tid] += v;
        __syncthreads();
    }
    int run = scan[tid] - local;
    for (int e = lo; e < hi; ++e) {
        pre[e] = run;
        int m = P.offsets ? P.offsets[e + 1] - P.offsets[e] : (int)P.rows_fixed;
        run += (m + bm - 1) / bm * ftiles;
    }
    if (tid == kThreads - 1) pre[n] = scan[tid];
    __syncthreads();
}

// Largest e in [0, n) with pre[e] <= t (pre non-decreasing, t < pre[n]).
__device__ __forceinline__ int find_expert(const int *pre, int n, int t) {
    int lo = 0, hi = n;   // invariant: pre[lo] <= t < pre[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (pre[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ FfnProblem pick(const FfnArgs &a, int p) { return p ? a.p[1] : a.p[0]; }

// BM: tokens per tile; WR: weight rows per tile (gate/up: WR/2 features, gate rows then up rows).
template <int DT, bool GATEUP, int BM, int WR>
__global__ __launch_bounds__(kThreads) void ffn_kernel(const FfnArgs a) {
    typedef FTraits<DT> Tr;
    constexpr int esz = Tr::esz;
    constexpr int BF = GATEUP ? WR / 2 : WR;      // output features per tile
    constexpr int ROWS = WR + BM;                 // staged rows per stage
    constexpr int NCH = ROWS * 8 / kThreads;      // 16-byte chunks per thread per stage
    static_assert(ROWS * 8 % kThreads == 0, "chunking");
    constexpr int RB = WR / 2 / 16;               // 16-row weight blocks per wave
    constexpr int TB = BM / 2 / 16;               // 16-token blocks per wave
    constexpr bool FP8 = DT == DT_E4M3;
    static_assert(!FP8 || !GATEUP || BF == 128, "fp8 H quantisation needs whole 128-feature groups per tile");
    static_assert(!FP8 || GATEUP || (WR / 2 <= 128 && 128 % (WR / 2) == 0), "fp8 down pass: one weight block per wave");

    extern __shared__ __align__(16) char smem[];
    char *stage_base = smem;                                      // [2][ROWS][kPitch]
    int *pre = (int *)(smem + 2 * ROWS * kPitch);                 // [2][kMaxExperts + 1]
    int *scan = pre + 2 * (kMaxExperts + 1);                      // [kThreads]
    float *xsc = (float *)(scan + kThreads);                      // [2][BM]    fp8 activation scales
    float *red = xsc + 2 * BM;                                    // [2][BM]    fp8 H amax exchange

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid & 1, wf = wid >> 1;
    const int K = a.K, F = a.F;
    const int ftiles = F / BF;
    const int64_t rowbytes = (int64_t)K * esz;
    const int KT = (int)(rowbytes / 128);
    const int kb_per_row = K / 128;               // fp8 scale blocks along K

    tile_prefix(a.p[0], BM, ftiles, pre, scan);
    if (a.nprob > 1) tile_prefix(a.p[1], BM, ftiles, pre + kMaxExperts + 1, scan);
    const int total0 = pre[a.p[0].n_exp];
    const int total = total0 + (a.nprob > 1 ? pre[kMaxExperts + 1 + a.p[1].n_exp] : 0);

    // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a contiguous run of tiles.
    const int G = gridDim.x;
    const int first = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

    for (int t = first; t < total; t += G) {
        const int p = t < total0 ? 0 : 1;
        const FfnProblem P = pick(a, p);
        const int *ppre = pre + p * (kMaxExperts + 1);
        const int lt = t - (p ? total0 : 0);
        const int e = find_expert(ppre, P.n_exp, lt);
        const int64_t base = P.offsets ? (int64_t)P.offsets[e] : (int64_t)e * P.rows_fixed;
        const int Me = P.offsets ? P.offsets[e + 1] - P.offsets[e] : (int)P.rows_fixed;
        const int mt = (Me + BM - 1) / BM;
        const int ln = lt - ppre[e];
        const int nt = ln / mt, mi = ln - nt * mt;
        const int r0 = mi * BM;
        const int valid = min(BM, Me - r0);
        const int n0 = nt * BF;

        // source of every chunk this thread stages (rows clamp to the last valid token)
        const char *src[NCH];
        int dst[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int chunk = tid + c * kThreads, row = chunk >> 3, col = chunk & 7;
            const char *ptr;
            if (row < WR) {
                const char *w = (const char *)((GATEUP && row >= BF) ? P.w1 : P.w0);
                const int f = n0 + ((GATEUP && row >= BF) ? row - BF : row);
                ptr = w + ((int64_t)e * F + f) * rowbytes;
            } else {
                const int r = min(row - WR, valid - 1);
                const int64_t R = base + r0 + r;
                const int64_t xr = P.gather ? (int64_t)P.gather[R] : (P.x_local ? (int64_t)(r0 + r) : R);
                ptr = (const char *)P.x + xr * rowbytes;
            }
            src[c] = ptr + col * 16;
            dst[c] = row * kPitch + col * 16;
        }
        // fp8: the activation scale row of the token this thread stages scales for
        const float *xs_row = nullptr;
        if (FP8 && tid < BM) {
            const int r = min(tid, valid - 1);
            const int64_t R = base + r0 + r;
            const int64_t xr = P.gather ? (int64_t)P.gather[R] : (P.x_local ? (int64_t)(r0 + r) : R);
            xs_row = P.xs + xr * kb_per_row;
        }
        // fp8: weight block-scale rows for this wave (gate/up: one gate and one up block; down: one block)
        const float *ws0 = nullptr, *ws1 = nullptr;
        if (FP8) {
            const int fb = GATEUP ? n0 / 128 : (n0 + wf * (WR / 2)) / 128;
            ws0 = P.s0 + ((int64_t)e * (F / 128) + fb) * kb_per_row;
            ws1 = GATEUP ? P.s1 + ((int64_t)e * (F / 128) + fb) * kb_per_row : ws0;
        }

        f32x4 acc[RB][TB];
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < TB; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

        __syncthreads();   // previous tile's readers are done with the stage buffers
        u32x4 stage[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) stage[c] = *(const u32x4 *)src[c];
#pragma unroll
        for (int c = 0; c < NCH; ++c) *(u32x4 *)(stage_base + dst[c]) = stage[c];
        if (FP8 && tid < BM) xsc[tid] = xs_row[0];
        __syncthreads();

        for (int kt = 0; kt < KT; ++kt) {
            const int cur = kt & 1;
            float xs_next = 0.0f;
            if (kt + 1 < KT) {
#pragma unroll
                for (int c = 0; c < NCH; ++c) stage[c] = *(const u32x4 *)(src[c] + (int64_t)(kt + 1) * 128);
                if (FP8 && tid < BM) xs_next = xs_row[kt + 1];
            }
            const char *Ws = stage_base + cur * ROWS * kPitch;
            const char *Xs = Ws + WR * kPitch;
#pragma unroll
            for (int s = 0; s < Tr::kSub; ++s) {
                typename Tr::frag af[RB], bfr[TB];
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    // gate/up: first half of the wave's blocks are gate rows, second half the matching up rows
                    const int wrow = GATEUP ? ((i < RB / 2) ? wf * (BF / 2) + i * 16 : BF + wf * (BF / 2) + (i - RB / 2) * 16)
                                            : wf * (WR / 2) + i * 16;
                    af[i] = Tr::load(Ws + (wrow + (lane & 15)) * kPitch, s, lane);
                }
#pragma unroll
                for (int j = 0; j < TB; ++j) bfr[j] = Tr::load(Xs + (wm * (BM / 2) + j * 16 + (lane & 15)) * kPitch, s, lane);
                if (FP8) {
                    const float sw0 = ws0[kt], sw1 = ws1[kt];
#pragma unroll
                    for (int j = 0; j < TB; ++j) {
                        const float sa = xsc[cur * BM + wm * (BM / 2) + j * 16 + (lane & 15)];
                        const float c0 = sa * sw0, c1 = sa * sw1;
#pragma unroll
                        for (int i = 0; i < RB; ++i) {
                            const f32x4 part = Tr::mma(af[i], bfr[j], f32x4{0, 0, 0, 0});
                            const float cc = (GATEUP && i >= RB / 2) ? c1 : c0;
#pragma unroll
                            for (int q = 0; q < 4; ++q) acc[i][j][q] += part[q] * cc;
                        }
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < RB; ++i)
#pragma unroll
                        for (int j = 0; j < TB; ++j) acc[i][j] = Tr::mma(af[i], bfr[j], acc[i][j]);
                }
            }
            if (kt + 1 < KT) {
                char *nxt = stage_base + (cur ^ 1) * ROWS * kPitch;
#pragma unroll
                for (int c = 0; c < NCH; ++c) *(u32x4 *)(nxt + dst[c]) = stage[c];
                if (FP8 && tid < BM) xsc[(cur ^ 1) * BM + tid] = xs_next;
            }
            __syncthreads();
        }

        // ---- epilogue ----
        if (GATEUP) {
            // h for gate block i pairs with up block i + RB/2 (same features)
            float h[RB / 2][TB][4];
#pragma unroll
            for (int i = 0; i < RB / 2; ++i)
#pragma unroll
                for (int j = 0; j < TB; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float g = acc[i][j][q], u = acc[i + RB / 2][j][q];
                        h[i][j][q] = __fdividef(g, 1.0f + __expf(-g)) * u;
                    }
            if (FP8) {
                // 1 x 128 groups of H along features: this tile's 128 features of a token live in
                // 4 lanes x (RB/2) blocks x 4 values of two waves (wf = 0, 1)
                float am[TB];
#pragma unroll
                for (int j = 0; j < TB; ++j) {
                    float m = 0.0f;
#pragma unroll
                    for (int i = 0; i < RB / 2; ++i)
#pragma unroll
                        for (int q = 0; q < 4; ++q) m = fmaxf(m, fabsf(h[i][j][q]));
                    m = fmaxf(m, __shfl_xor(m, 16, 64));
                    m = fmaxf(m, __shfl_xor(m, 32, 64));
                    am[j] = m;
                    if (lane < 16) red[wf * BM + wm * (BM / 2) + j * 16 + lane] = m;
                }
                __syncthreads();
#pragma unroll
                for (int j = 0; j < TB; ++j) {
                    const int tok = wm * (BM / 2) + j * 16 + (lane & 15);
                    const float amax = fmaxf(am[j], red[(wf ^ 1) * BM + tok]);
                    const float scale = quant_scale(amax);
                    if (tok >= valid) continue;
                    const int64_t R = base + r0 + tok;
                    uint8_t *orow = (uint8_t *)P.out + R * F;
#pragma unroll
                    for (int i = 0; i < RB / 2; ++i) {
                        const int f = n0 + wf * (BF / 2) + i * 16 + 4 * (lane >> 4);
                        *(uint32_t *)(orow + f) = pack_e4m3x4(clamp448(h[i][j][0] / scale), clamp448(h[i][j][1] / scale),
                                                              clamp448(h[i][j][2] / scale), clamp448(h[i][j][3] / scale));
                    }
                    if (wf == 0 && lane < 16) P.out_s[R * (F / 128) + n0 / 128] = scale;
                }
            } else {
#pragma unroll
                for (int j = 0; j < TB; ++j) {
                    const int tok = wm * (BM / 2) + j * 16 + (lane & 15);
                    if (tok >= valid) continue;
                    const int64_t R = base + r0 + tok;
#pragma unroll
                    for (int i = 0; i < RB / 2; ++i) {
                        const int f = n0 + wf * (BF / 2) + i * 16 + 4 * (lane >> 4);
                        if (DT == DT_F32) {
                            *(f32x4 *)((float *)P.out + R * F + f) = f32x4{h[i][j][0], h[i][j][1], h[i][j][2], h[i][j][3]};
                        } else {
                            *(u32x2 *)((uint16_t *)P.out + R * F + f) =
                                u32x2{pack_bf16x2(h[i][j][0], h[i][j][1]), pack_bf16x2(h[i][j][2], h[i][j][3])};
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const int tok = wm * (BM / 2) + j * 16 + (lane & 15);
                if (tok >= valid) continue;
                const int64_t R = base + r0 + tok;
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    const int f = n0 + wf * (WR / 2) + i * 16 + 4 * (lane >> 4);
                    if (DT == DT_F32) {
                        *(f32x4 *)((float *)P.out + R * F + f) = acc[i][j];
                    } else {
                        *(u32x2 *)((uint16_t *)P.out + R * F + f) =
                            u32x2{pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
                    }
                }
            }
        }
    }
}

template <int DT, bool GATEUP, int BM, int WR>
hipError_t run(const FfnArgs &a, int occupancy, hipStream_t s) {
    constexpr int ROWS = WR + BM;
    const size_t shmem = 2 * ROWS * kPitch + sizeof(int) * (2 * (kMaxExperts + 1) + kThreads) + sizeof(float) * 4 * BM;
    static std::once_flag once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(once, [&] {
        attr_err = hipFuncSetAttribute((const void *)ffn_kernel<DT, GATEUP, BM, WR>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    });
    if (attr_err != hipSuccess) return attr_err;
    int grid = device_cus() * occupancy;
    grid = (grid + 7) / 8 * 8;
    ffn_kernel<DT, GATEUP, BM, WR><<<grid, kThreads, shmem, s>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn(int dt, bool gateup, const FfnArgs &a, hipStream_t s) {
    if (dt == DT_F32) return gateup ? run<DT_F32, true, 64, 128>(a, 2, s) : run<DT_F32, false, 64, 128>(a, 2, s);
    if (dt == DT_BF16) return gateup ? run<DT_BF16, true, 64, 128>(a, 2, s) : run<DT_BF16, false, 64, 128>(a, 2, s);
    return gateup ? run<DT_E4M3, true, 64, 256>(a, 1, s) : run<DT_E4M3, false, 64, 128>(a, 2, s);
}

}  // namespace moe
