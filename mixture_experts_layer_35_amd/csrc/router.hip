// router.hip -- token-to-expert affinities and auxiliary-loss-free group-limited
// top-K selection ("DeepSeek-V3 Technical Report", §2.1.2: sigmoid affinities,
// bias used for selection only, gates normalised over the selected un-biased
// affinities, node-limited routing; §4.2: 8 of 256 experts, at most 4 groups).
#include <mutex>

#include "common.h"
#include "internal.h"
#include "lds_ring.h"

namespace moe {

namespace {

// ---------------------------------------------------------------------------
// Gate GEMM + sigmoid.  Tile: 64 experts x RT (64 or 128) tokens per
// 512-thread workgroup; the larger token tile halves the centroid traffic per
// token once the batch has enough tiles to fill the chip.  Both operands
// stream through an LDS ring of 128-byte reduction steps (64 centroid rows,
// then RT token rows) filled by direct global->LDS loads, each wave issuing
// (64+RT)/64 1 KB loads per step, so each CU keeps about 100 KB of loads in
// flight.  Eight waves form a 4 (experts) x 2 (tokens) grid of 16 x RT/2
// outputs.  Experts are the MFMA row operand, so a lane holds
// four consecutive experts of one token (one 16-byte store of fp32 scores).
// The four expert tiles of a token tile run on one XCD and share its rows
// through that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int RG_E = 64;                           // experts per tile
constexpr int RG_NT = 512;                         // threads per workgroup
constexpr int RG_LDS = 128 * 1024;                 // ring bytes

template <int RT>
struct RgTile {
    static constexpr int STAGE = (RT + RG_E) * 128;   // bytes per slot
    static constexpr int S = RG_LDS / STAGE;          // ring slots
    static constexpr int NQ = (RT + RG_E) / 64;       // 1 KB loads per wave per step
    static constexpr int TB = RT / 32;                // 16-token blocks per wave
};

template <int DT, int RT>
__global__ __launch_bounds__(RG_NT) void router_gemm_kernel(const char *__restrict__ u, const char *__restrict__ gw,
                                                           float *__restrict__ scores, int64_t T, int d, int Nr,
                                                           int etiles) {
    typedef FTraits<DT> Tr;
    typedef Frag<DT> Fr;
    typedef RgTile<RT> Tl;
    constexpr int RG_S = Tl::S, RG_STAGE = Tl::STAGE, NQ = Tl::NQ;
    extern __shared__ __align__(1024) char ring[];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int we = wid & 3, wt = wid >> 2;
    // XCD-aware order: workgroup b runs on XCD b % 8; each XCD takes a contiguous run of tiles
    const int G = gridDim.x;
    const int lin = (G & 7) == 0 ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
    const int64_t t0 = (int64_t)(lin / etiles) * RT;
    const int e0 = (lin % etiles) * RG_E;
    const int64_t rowbytes = (int64_t)d * Tr::esz;
    const int KT = (int)(rowbytes / 128);

    // this wave's NQ loads per step: instruction ins = NQ*wid + q fills staged rows
    // 8*ins .. 8*ins+7 (rows 0-63 centroids, then RT tokens); lane l takes row
    // 8*ins + l/8 and fills its chunk slot l%8 with the row's chunk (l%8) ^ swz(row).
    const char *src[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int row = 8 * (NQ * wid + q) + (lane >> 3);
        const int chunk = (lane & 7) ^ swz<128>(row);
        const char *p;
        if (row < RG_E) p = gw + (int64_t)min(e0 + row, Nr - 1) * rowbytes;
        else p = u + min(t0 + row - RG_E, T - 1) * rowbytes;
        src[q] = p + chunk * 16;
    }
    auto issue = [&](int ks) {
        char *st = ring + (ks % RG_S) * RG_STAGE;
#pragma unroll
        for (int q = 0; q < NQ; ++q) dma16(src[q] + (int64_t)ks * 128, st + (NQ * wid + q) * 1024);
    };

    f32x4 acc[Tl::TB];
#pragma unroll
    for (int j = 0; j < Tl::TB; ++j) acc[j] = f32x4{0, 0, 0, 0};
    for (int ks = 0; ks < RG_S - 1 && ks < KT; ++ks) issue(ks);
    for (int kt = 0; kt < KT; ++kt) {
        // step kt has landed once at most the later steps' loads are outstanding
        if (kt + RG_S - 2 < KT) wait_vmcnt<NQ * (RG_S - 2)>();
        else wait_vmcnt<0>();
        cta_barrier();   // every wave's loads of step kt have landed; step kt-1's slot is free
        if (kt + RG_S - 1 < KT) issue(kt + RG_S - 1);
        const char *st = ring + (kt % RG_S) * RG_STAGE;
#pragma unroll
        for (int s = 0; s < Fr::kSub; ++s) {
            const typename Fr::t a = Fr::load(st, we * 16 + (lane & 15), s, lane);
#pragma unroll
            for (int j = 0; j < Tl::TB; ++j) {
                const typename Fr::t b = Fr::load(st, RG_E + wt * (RT / 2) + j * 16 + (lane & 15), s, lane);
                acc[j] = Tr::mma(a, b, acc[j]);
            }
        }
    }
    // lane holds experts e0 + we*16 + 4*(lane>>4) + {0..3} of token t0 + wt*RT/2 + j*16 + (lane&15)
#pragma unroll
    for (int j = 0; j < Tl::TB; ++j) {
        const int64_t t = t0 + wt * (RT / 2) + j * 16 + (lane & 15);
        if (t >= T) continue;
        const int e = e0 + we * 16 + 4 * (lane >> 4);
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = 1.0f / (1.0f + expf(-acc[j][q]));
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

// ---------------------------------------------------------------------------
// Selection: one wave per token.  Lane l holds experts l, l+64, ... (R of
// them) in registers.  A group's score (the sum of its two largest biased
// affinities) comes from a butterfly top-2 merge over the group's lanes when
// groups are aligned power-of-two lane segments, else from a serial scan of
// the staged scores.  Ordering keys pack (value, index) so that a single
// 64-bit max picks the larger value and, on equal values, the lower index.
// ---------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(256) void router_select_kernel(const float *__restrict__ scores,
                                                            const float *__restrict__ bias, int64_t T, int Nr, int G,
                                                            int Mg, int K, float routed_scale,
                                                            int32_t *__restrict__ topk_idx,
                                                            float *__restrict__ topk_w) {
    __shared__ float sb_all[4][64 * R];   // serial-scan fallback: biased scores
    __shared__ float gs_all[4][64];       // group scores
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * 4 + wid;
    if (t >= T) return;                   // uniform per wave; nothing below synchronises waves
    const int gs = Nr / G;
    float sv[R], bv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = lane + 64 * r;
        sv[r] = i < Nr ? scores[t * Nr + i] : 0.0f;
        bv[r] = i < Nr ? sv[r] + bias[i] : -INFINITY;   // one fp32 add; bias only steers selection
    }
    float *gsc = gs_all[wid];
    if (gs <= 64 && (gs & (gs - 1)) == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float m1 = bv[r], m2 = -INFINITY;
            for (int off = 1; off < gs; off <<= 1) {
                const float o1 = __shfl_xor(m1, off, 64), o2 = __shfl_xor(m2, off, 64);
                const float n2 = fmaxf(fminf(m1, o1), fmaxf(m2, o2));
                m1 = fmaxf(m1, o1);
                m2 = n2;
            }
            const int i = lane + 64 * r;
            if (i < Nr && (lane & (gs - 1)) == 0) gsc[i / gs] = gs == 1 ? m1 : m1 + m2;
        }
    } else {
        float *sb = sb_all[wid];
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (lane + 64 * r < Nr) sb[lane + 64 * r] = bv[r];
        __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        if (lane < G) {
            float m1 = -INFINITY, m2 = -INFINITY;
            for (int i = lane * gs; i < (lane + 1) * gs; ++i) {
                const float v = sb[i];
                if (v > m1) { m2 = m1; m1 = v; }
                else if (v > m2) { m2 = v; }
            }
            gsc[lane] = m1 + m2;
        }
    }
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
    __builtin_amdgcn_wave_barrier();
    uint64_t gkey = lane < G ? order_key(gsc[lane], lane) : 0ull;
    uint64_t kept = 0;
    for (int r = 0; r < Mg; ++r) {
        const uint64_t best = wave_max_u64(gkey);
        const int g = key_index(best);
        kept |= 1ull << g;
        if (lane == g) gkey = 0;
    }
    uint64_t key[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = lane + 64 * r;
        key[r] = (i < Nr && ((kept >> (i / gs)) & 1ull)) ? order_key(bv[r], i) : 0ull;
    }
    int my_e = 0;
    float my_s = 0.0f;
    float den = 0.0f;
    for (int j = 0; j < K; ++j) {
        uint64_t local = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) local = key[r] > local ? key[r] : local;
        const uint64_t best = wave_max_u64(local);
        const int e = key_index(best);
        float mine = sv[0];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r == (e >> 6)) {
                mine = sv[r];
                if (lane == (e & 63)) key[r] = 0;
            }
        }
        const float s = __shfl(mine, e & 63, 64);   // the un-biased affinity of the pick
        den = den + s;                               // slot order, fp32
        if (lane == j) { my_e = e; my_s = s; }
    }
    if (lane < K) {
        topk_idx[t * K + lane] = my_e;
        topk_w[t * K + lane] = (my_s / den) * routed_scale;
    }
}

template <int DT, int RT>
hipError_t run_router_gemm(const void *u, const void *gate_w, float *scores, int64_t T, int d, int Nr, hipStream_t s) {
    static std::once_flag once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(once, [&] {
        attr_err = hipFuncSetAttribute((const void *)router_gemm_kernel<DT, RT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, RG_LDS);
    });
    if (attr_err != hipSuccess) return attr_err;
    const int etiles = (Nr + RG_E - 1) / RG_E;
    const int64_t tiles = (T + RT - 1) / RT * etiles;
    router_gemm_kernel<DT, RT><<<(unsigned)tiles, RG_NT, RG_LDS, s>>>((const char *)u, (const char *)gate_w, scores, T,
                                                                      d, Nr, etiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_router_gemm(int dt, const void *u, const void *gate_w, float *scores, int64_t T, int d, int Nr,
                              hipStream_t s) {
    if (T <= 0) return hipSuccess;
    // 128-token tiles once they alone give every CU two tiles
    const bool wide = (T + 127) / 128 * ((Nr + RG_E - 1) / RG_E) >= 2 * device_cus();
    if (dt == DT_F32)
        return wide ? run_router_gemm<DT_F32, 128>(u, gate_w, scores, T, d, Nr, s)
                    : run_router_gemm<DT_F32, 64>(u, gate_w, scores, T, d, Nr, s);
    return wide ? run_router_gemm<DT_BF16, 128>(u, gate_w, scores, T, d, Nr, s)
                : run_router_gemm<DT_BF16, 64>(u, gate_w, scores, T, d, Nr, s);
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
