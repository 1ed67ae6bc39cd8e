// router.hip -- token-to-expert affinities and auxiliary-loss-free group-limited
// top-K selection ("DeepSeek-V3 Technical Report", §2.1.2: sigmoid affinities,
// bias used for selection only, gates normalised over the selected un-biased
// affinities, node-limited routing; §4.2: 8 of 256 experts, at most 4 groups).
#include <algorithm>
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

// ---------------------------------------------------------------------------
// Split-K gate GEMM over all 256 experts.  At the V3 shape the single-pass
// kernel above re-reads every centroid row once per 64-token tile (about 235
// MB of L2 -> LDS traffic at T = 4096) and meets at a barrier 112 times per
// tile for a few MFMAs each.  Here a workgroup owns RT tokens x all experts x
// one of KS chunks of the hidden dimension: the centroids cross into LDS once
// per RT tokens, a reduction step carries RT*256*64*2 flops, and KS chunks
// give the chip enough workgroups.  Each chunk's fp32 partial products go to
// part[c][t][e]; router_finish_kernel sums them in chunk order.  Workgroups
// of one chunk run on one XCD, so that chunk of the centroids is fetched into
// its L2 once.
// ---------------------------------------------------------------------------
constexpr int RP_E = 256;                          // experts per tile (all of them)
constexpr int RP_LDS = 144 * 1024;

template <int RT>
struct RpTile {
    static constexpr int ROWS = RT + RP_E;            // staged rows per step
    static constexpr int STAGE = ROWS * 128;          // bytes per slot
    static constexpr int S = RP_LDS / STAGE;          // ring slots
    static constexpr int NQ = ROWS / 64;              // 1 KB loads per wave per step
    static constexpr int WT = RT >= 128 ? 2 : 1;      // wave grid: token x expert
    static_assert(ROWS % 64 == 0, "whole 1 KB loads per wave");
    static constexpr int WE = 8 / WT;
    static constexpr int TBW = RT / WT / 16;          // 16-token blocks per wave
    static constexpr int EBW = RP_E / WE / 16;        // 16-expert blocks per wave
};

template <int RT>
__global__ __launch_bounds__(RG_NT) void router_partial_kernel(const char *__restrict__ u, const char *__restrict__ gw,
                                                              float *__restrict__ part, int64_t T, int d, int ntiles,
                                                              int ks_count, int steps_per_chunk) {
    typedef FTraits<DT_BF16> Tr;
    typedef Frag<DT_BF16> Fr;
    typedef RpTile<RT> Tl;
    constexpr int S = Tl::S, STAGE = Tl::STAGE, NQ = Tl::NQ;
    extern __shared__ __align__(1024) char ring[];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wt = wid / Tl::WE, we = wid % Tl::WE;
    // XCD-aware order: workgroup b runs on XCD b % 8; consecutive ids share a chunk
    const int G = gridDim.x;
    const int lin = (G & 7) == 0 ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
    const int chunk = lin / ntiles, tile = lin % ntiles;
    const int64_t t0 = (int64_t)tile * RT;
    const int64_t rowbytes = (int64_t)d * 2;
    const int KT = (int)(rowbytes / 128);
    const int k0 = chunk * steps_per_chunk, k1 = min(KT, k0 + steps_per_chunk);
    const int nk = max(k1 - k0, 0);

    // instruction q of this wave fills staged rows 8*(NQ*wid+q) .. +7: centroid rows
    // first (RP_E), then the RT token rows; lane l takes row 8*ins + l/8, chunk slot l%8
    const char *src[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int row = 8 * (NQ * wid + q) + (lane >> 3);
        const int c = (lane & 7) ^ swz<128>(row);
        const char *p = row < RP_E ? gw + (int64_t)row * rowbytes : u + min(t0 + row - RP_E, T - 1) * rowbytes;
        src[q] = p + (int64_t)k0 * 128 + c * 16;
    }
    // token rows are read by this workgroup alone: nontemporal, so that L2 keeps the
    // centroid chunk that every token tile on the XCD reads
    const int uw = __builtin_amdgcn_readfirstlane(wid);
    auto issue = [&](int k) {
        char *st = ring + (k % S) * STAGE;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (8 * (NQ * uw + q) >= RP_E) dma16_stream(src[q] + (int64_t)k * 128, st + (NQ * wid + q) * 1024);
            else dma16(src[q] + (int64_t)k * 128, st + (NQ * wid + q) * 1024);
        }
    };
    f32x4 acc[Tl::EBW][Tl::TBW];
#pragma unroll
    for (int i = 0; i < Tl::EBW; ++i)
#pragma unroll
        for (int j = 0; j < Tl::TBW; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
    for (int k = 0; k < S - 1 && k < nk; ++k) issue(k);
    for (int k = 0; k < nk; ++k) {
        if (k + S - 2 < nk) wait_vmcnt<NQ * (S - 2)>();
        else wait_vmcnt<0>();
        cta_barrier();
        if (k + S - 1 < nk) issue(k + S - 1);
        const char *st = ring + (k % S) * STAGE;
#pragma unroll
        for (int sub = 0; sub < Fr::kSub; ++sub) {
            typename Fr::t a[Tl::EBW], b[Tl::TBW];
#pragma unroll
            for (int i = 0; i < Tl::EBW; ++i) a[i] = Fr::load(st, (we * Tl::EBW + i) * 16 + (lane & 15), sub, lane);
#pragma unroll
            for (int j = 0; j < Tl::TBW; ++j)
                b[j] = Fr::load(st, RP_E + (wt * Tl::TBW + j) * 16 + (lane & 15), sub, lane);
#pragma unroll
            for (int i = 0; i < Tl::EBW; ++i)
#pragma unroll
                for (int j = 0; j < Tl::TBW; ++j) acc[i][j] = Tr::mma(a[i], b[j], acc[i][j]);
        }
    }
    // a lane holds experts (we*EBW + i)*16 + 4*(lane>>4) + {0..3} of token (wt*TBW + j)*16 + (lane&15).
    // The tile goes through LDS (rows padded by 16 bytes, so the 16 tokens of a write land in
    // distinct bank groups) and leaves as whole 1 KB token rows, one 16-byte chunk per lane:
    // stored straight from the accumulators, each instruction wrote 64-byte pieces of 16 rows.
    constexpr int PITCH = RP_E * 4 + 16;
    static_assert(RT * PITCH <= RP_LDS, "the staged partial tile fits the ring");
    __syncthreads();   // every wave is done with the ring (no load is in flight after the last step)
#pragma unroll
    for (int j = 0; j < Tl::TBW; ++j) {
        const int tl = (wt * Tl::TBW + j) * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < Tl::EBW; ++i)
            *(f32x4 *)(ring + tl * PITCH + ((we * Tl::EBW + i) * 16 + 4 * (lane >> 4)) * 4) = acc[i][j];
    }
    __syncthreads();
    float *pc = part + (int64_t)chunk * T * RP_E;
    for (int r = wid; r < RT; r += RG_NT / 64) {
        const int64_t t = t0 + r;
        if (t >= T) break;
        *(f32x4 *)(pc + t * RP_E + 4 * lane) = *(const f32x4 *)(ring + r * PITCH + 16 * lane);
    }
}

// ---- 16-lane row operations on DPP (no LDS round trip) ----------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_XOR1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int DPP_ROR4 = 0x124;   // row_ror:4
constexpr int DPP_ROR8 = 0x128;   // row_ror:8 (lane i ^ 8 within the row)
constexpr int DPP_ROR12 = 0x12C;  // row_ror:12

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) { return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v))); }
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}
// the value of lane i ^ 4 within the row (ror4_is_xor4: row_ror:4 brings lane i ^ 4 to this lane,
// else row_ror:12 does)
__device__ __forceinline__ float xor4_f32(float v, bool ror4_is_xor4) {
    const float a = dpp_f32<DPP_ROR4>(v), b = dpp_f32<DPP_ROR12>(v);
    return ror4_is_xor4 ? a : b;
}
// maximum over the 16 lanes of a row, in every lane of it
__device__ __forceinline__ uint64_t row_max_u64(uint64_t v) {
    uint64_t o = dpp_u64<DPP_XOR1>(v);
    v = o > v ? o : v;
    o = dpp_u64<DPP_XOR2>(v);
    v = o > v ? o : v;
    o = dpp_u64<DPP_ROR4>(v);     // max of this quad and the next (either direction)
    v = o > v ? o : v;
    o = dpp_u64<DPP_ROR8>(v);     // and of the quads two away: all four
    v = o > v ? o : v;
    return v;
}

// ---------------------------------------------------------------------------
// Affinities and selection, 16 lanes per token (four tokens per wave): lane l
// of a token's row holds experts 16l .. 16l+15.  z is the sum of the KS chunk
// partials in chunk order (or, with given affinities, s is read as it is);
// s = sigmoid(z) is stored, s' = s + b; a group (a segment of gs/16 lanes)
// scores the sum of its two largest s'; the top-Mg groups and then the top-K
// experts among them are picked by repeated 16-lane maxima of (value, index)
// keys, so every tie goes to the lower index; gates as in router_select_kernel.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_finish_kernel(const float *__restrict__ part, int ks_count,
                                                            const float *__restrict__ scores_in,
                                                            float *__restrict__ scores_out,
                                                            const float *__restrict__ bias, int64_t T, int G, int Mg,
                                                            int K, float routed_scale, int32_t *__restrict__ topk_idx,
                                                            float *__restrict__ topk_w) {
    constexpr int V = 16, NR = 256;
    const int lane = threadIdx.x & 63, r = lane & 15;
    const int64_t t = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const bool live = t < T;
    const int64_t tt = live ? t : T - 1;            // dead rows shadow the last token and store nothing
    const int e0 = r * V;
    float sv[V];
    if (scores_in) {
#pragma unroll
        for (int q = 0; q < V / 4; ++q) {
            const f32x4 x = *(const f32x4 *)(scores_in + tt * NR + e0 + 4 * q);
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[4 * q + i] = x[i];
        }
    } else {
        float z[V];
#pragma unroll
        for (int q = 0; q < V / 4; ++q) {
            const f32x4 x = __builtin_nontemporal_load((const f32x4 *)(part + tt * NR + e0 + 4 * q));
#pragma unroll
            for (int i = 0; i < 4; ++i) z[4 * q + i] = x[i];
        }
        for (int c = 1; c < ks_count; ++c) {
            const float *pc = part + ((int64_t)c * T + tt) * NR + e0;
#pragma unroll
            for (int q = 0; q < V / 4; ++q) {
                const f32x4 x = __builtin_nontemporal_load((const f32x4 *)(pc + 4 * q));
#pragma unroll
                for (int i = 0; i < 4; ++i) z[4 * q + i] += x[i];
            }
        }
#pragma unroll
        for (int i = 0; i < V; ++i) sv[i] = 1.0f / (1.0f + expf(-z[i]));
        if (scores_out && live) {
#pragma unroll
            for (int q = 0; q < V / 4; ++q)
                *(f32x4 *)(scores_out + t * NR + e0 + 4 * q) = f32x4{sv[4 * q], sv[4 * q + 1], sv[4 * q + 2], sv[4 * q + 3]};
        }
    }
    float bv[V];
#pragma unroll
    for (int q = 0; q < V / 4; ++q) {
        const f32x4 b = *(const f32x4 *)(bias + e0 + 4 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) bv[4 * q + i] = sv[4 * q + i] + b[i];   // one fp32 add; selection only
    }
    // which way row_ror:4 turns, from the lane ids themselves
    const bool ror4_is_xor4 = (int)dpp_u32<DPP_ROR4>((uint32_t)r) == (r ^ 4);
    // group score: the two largest s' of the group's lanes
    const int gs = NR / G, glanes = gs / V;
    float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const float x = bv[i];
        m2 = fmaxf(m2, fminf(m1, x));
        m1 = fmaxf(m1, x);
    }
    auto merge = [&](float o1, float o2) {
        const float n2 = fmaxf(fminf(m1, o1), fmaxf(m2, o2));
        m1 = fmaxf(m1, o1);
        m2 = n2;
    };
    if (glanes >= 2) merge(dpp_f32<DPP_XOR1>(m1), dpp_f32<DPP_XOR1>(m2));
    if (glanes >= 4) merge(dpp_f32<DPP_XOR2>(m1), dpp_f32<DPP_XOR2>(m2));
    if (glanes >= 8) {
        const float o1 = xor4_f32(m1, ror4_is_xor4), o2 = xor4_f32(m2, ror4_is_xor4);
        merge(o1, o2);
    }
    if (glanes >= 16) merge(dpp_f32<DPP_ROR8>(m1), dpp_f32<DPP_ROR8>(m2));
    const int g = r / glanes;                       // this lane's group
    const float gscore = m1 + m2;                   // 16 | gs: a group has at least two experts
    // top-Mg groups: the lane of each group that heads it carries its key
    uint64_t gkey = (r % glanes) == 0 ? order_key(gscore, g) : 0ull;
    uint32_t kept = 0;
    for (int k = 0; k < Mg; ++k) {
        const uint64_t best = row_max_u64(gkey);
        const int gb = key_index(best);
        kept |= 1u << gb;
        if (g == gb) gkey = 0;
    }
    // top-K experts of the kept groups
    const bool mine = (kept >> g) & 1u;
    uint64_t key[V];
#pragma unroll
    for (int i = 0; i < V; ++i) key[i] = mine ? order_key(bv[i], e0 + i) : 0ull;
    uint64_t local = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) local = key[i] > local ? key[i] : local;
    int my_e = 0;
    float my_s = 0.0f, den = 0.0f;
    for (int j = 0; j < K; ++j) {
        const uint64_t best = row_max_u64(local);
        const int e = key_index(best);
        const int owner = e / V;
        float s_e = 0.0f;
        if (r == owner) {
#pragma unroll
            for (int i = 0; i < V; ++i)
                if (e0 + i == e) { s_e = sv[i]; key[i] = 0; }
            local = 0;
#pragma unroll
            for (int i = 0; i < V; ++i) local = key[i] > local ? key[i] : local;
        }
        // the un-biased affinity of the pick, from its owner lane, to the whole row
        float s_b = r == owner ? s_e : -INFINITY;
        s_b = fmaxf(s_b, dpp_f32<DPP_XOR1>(s_b));
        s_b = fmaxf(s_b, dpp_f32<DPP_XOR2>(s_b));
        s_b = fmaxf(s_b, dpp_f32<DPP_ROR4>(s_b));
        s_b = fmaxf(s_b, dpp_f32<DPP_ROR8>(s_b));
        den = den + s_b;                            // slot order, fp32
        if (r == j) { my_e = e; my_s = s_b; }
    }
    if (live && r < K) {
        topk_idx[t * K + r] = my_e;
        topk_w[t * K + r] = (my_s / den) * routed_scale;
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

bool router_splitk_ok(int dt, int Nr, int G, int K) {
    return dt == DT_BF16 && Nr == RP_E && G >= 1 && (Nr / G) % 16 == 0 && K <= 16;
}

namespace {
// Token tile and chunk count: about one workgroup per CU of an MI355X (256), the tile as
// wide as that allows.  A function of the shape alone, so workspace sizes need no device.
void splitk_plan(int64_t T, int d, int *rt, int *ks, int *spc) {
    const int cus = 256;
    *rt = T >= 2048 ? 128 : 64;
    const int64_t ntiles = (T + *rt - 1) / *rt;
    const int KT = d * 2 / 128;
    int k = (int)std::max<int64_t>(1, std::min<int64_t>(16, (cus + ntiles - 1) / ntiles));
    k = std::min(k, KT);
    *spc = (KT + k - 1) / k;
    *ks = (KT + *spc - 1) / *spc;
}
}  // namespace

size_t router_partial_bytes(int64_t T, int d, int Nr) {
    int rt, ks, spc;
    splitk_plan(T, d, &rt, &ks, &spc);
    return (size_t)ks * (size_t)T * Nr * 4;
}

hipError_t launch_router_splitk(const void *u, const void *gate_w, float *part, float *scores, const float *bias,
                                int64_t T, int d, int G, int Mg, int K, float routed_scale, int32_t *topk_idx,
                                float *topk_w, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    int rt, ks, spc;
    splitk_plan(T, d, &rt, &ks, &spc);
    const int ntiles = (int)((T + rt - 1) / rt);
    const unsigned grid = (unsigned)(ntiles * ks);
    static std::once_flag once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(once, [&] {
        attr_err = hipFuncSetAttribute((const void *)router_partial_kernel<128>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, RP_LDS);
        if (attr_err == hipSuccess)
            attr_err = hipFuncSetAttribute((const void *)router_partial_kernel<64>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, RP_LDS);
    });
    if (attr_err != hipSuccess) return attr_err;
    if (rt == 128)
        router_partial_kernel<128><<<grid, RG_NT, RP_LDS, s>>>((const char *)u, (const char *)gate_w, part, T, d, ntiles,
                                                               ks, spc);
    else
        router_partial_kernel<64><<<grid, RG_NT, RP_LDS, s>>>((const char *)u, (const char *)gate_w, part, T, d, ntiles,
                                                              ks, spc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    router_finish_kernel<<<(unsigned)((T + 15) / 16), 256, 0, s>>>(part, ks, nullptr, scores, bias, T, G, Mg, K,
                                                                   routed_scale, topk_idx, topk_w);
    return hipGetLastError();
}

hipError_t launch_router_select(const float *scores, const float *bias, int64_t T, int Nr, int G, int Mg, int K,
                                float routed_scale, int32_t *topk_idx, float *topk_w, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (Nr == RP_E && G >= 1 && (Nr / G) % 16 == 0 && K <= 16) {
        // given affinities: the 16-lane selection of the split-K path
        router_finish_kernel<<<(unsigned)((T + 15) / 16), 256, 0, s>>>(nullptr, 0, scores, nullptr, bias, T, G, Mg, K,
                                                                       routed_scale, topk_idx, topk_w);
        return hipGetLastError();
    }
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
