// ffn.hip -- grouped SwiGLU expert FFN on MFMA ("DeepSeek-V3 Technical Report",
// §2.1.2: fine-grained routed experts plus shared experts; §3.3: FP8 GEMMs with
// 1 x 128 activation tiles and 128 x 128 weight blocks whose partial sums are
// promoted to fp32 every 128 products; §4.2: I = 2048 for every expert).
//
// One kernel, two passes:
//   gate/up pass: H[r, f] = SiLU(x_r . Wg[f]) * (x_r . Wu[f])   -> H (act dtype or e4m3 + 1x128 scales)
//   down pass:    Y[r, f] = H_r . Wd[f]                          -> y (out dtype)
//
// Scheduling.  Rows are ragged per expert and only known on the device, so the
// grid is persistent (one 512-thread workgroup per CU) and every workgroup
// takes tiles from a list derived from the row offsets.  A tile is (expert,
// block of 256 weight rows, block of up to 256 tokens); row blocks of one
// (expert, weight block) are adjacent in the list, then the weight blocks of
// the expert.  The list is cut into eight ranges of about equal cost, one per
// XCD, and the workgroups of an XCD take its tiles in order through a counter,
// so the tiles in flight on an XCD are always list neighbours: a weight block
// shared by several row blocks, and the token rows shared by the weight
// blocks, are fetched once into that XCD's L2 even though tiles take unequal
// times.  Up to two problems (e.g. shared and routed experts) share a launch.
//
// Data movement.  The reduction dimension is walked in 128-byte steps.  Each
// step's weight rows and token rows are copied from global memory straight
// into an LDS ring by global_load_lds (no register staging), 16 bytes per lane,
// into XOR-swizzled rows.  Four producer waves (one per SIMD) issue all loads;
// each waits with an exact vmcnt for its own loads of the step about to be
// consumed, then the workgroup meets at a fence-free barrier.  The ring depth
// is chosen per tile: a tile stages only its valid token rows when that leaves
// three or more slots, and loads a whole step ahead right after the barrier;
// otherwise (large token blocks, two slots) it stages whole 32-token blocks and
// spreads each step's loads over the producer's products.  The next tile's
// first steps are loaded while the current tile's results are written.
//
// MFMA orientation: weights are the MFMA row operand and tokens the column
// operand, so a lane's four accumulators are four consecutive output features
// of one token.  Eight waves (two per SIMD) form a 2 (tokens) x 4 (weight rows)
// grid; each wave owns 64 weight rows x 128 tokens.
#include <mutex>
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "lds_ring.h"

namespace moe {

namespace {

// Exclusive prefix of per-expert tile counts into pre[0..n]; pre[n] = total.
// scan: NT ints of scratch.
template <int NT>
__device__ void tile_prefix(const FfnProblem &P, int bm, int ftiles, int *pre, int *scan) {
    const int tid = threadIdx.x;
    const int n = P.n_exp;
    const int per = (n + NT - 1) / NT;
    const int lo = min(tid * per, n), hi = min(lo + per, n);
    int local = 0;
    for (int e = lo; e < hi; ++e) {
        int m = P.offsets ? P.offsets[e + 1] - P.offsets[e] : (int)P.rows_fixed;
        local += (m + bm - 1) / bm * ftiles;
    }
    scan[tid] = local;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
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
    if (tid == NT - 1) pre[n] = scan[tid];
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

constexpr int BM = 256;                 // tokens per tile
constexpr int WR = 256;                 // weight rows per tile
constexpr int WM = 2, WF = 4;           // wave grid: token x weight-row
constexpr int NW = WM * WF;             // waves per workgroup
constexpr int NT = 64 * NW;             // threads per workgroup
constexpr int WRW = WR / WF;            // weight rows per wave (64)
constexpr int RB = WRW / 16;            // 16-row weight blocks per wave (4)
constexpr int TB = BM / WM / 16;        // 16-token blocks per wave (8)
constexpr int SCL_BYTES = 2048;         // fp8: per-stage scale area (BM activation + 2 weight scales)
constexpr int LDS_TOTAL = 160 * 1024;

// LDS bytes besides the ring: tile prefixes of both problems (n_exp + 1 each),
// then the tile queues' bounds and the next-tile slots (SCHED_INTS ints).
constexpr int SCHED_INTS = 16;
constexpr int NQ = 8;                   // tile queues, one per XCD
constexpr int TILE_COST_W = 128;        // a tile's weight streaming, in token rows (queue balance)
__host__ __device__ inline int prefix_bytes(int n0, int n1) {
    return ((n0 + 1 + n1 + 1 + SCHED_INTS) * 4 + 255) & ~255;
}

// Tile queues.  The tile list is cut into NQ contiguous ranges of about equal
// estimated cost (a tile of v token rows costs v + TILE_COST_W), one per XCD:
// workgroups on XCD x take the tiles of range x in list order through a counter
// (ctr[x]), so the tiles running at any moment on one XCD are neighbours in the
// list and share their weight block and token rows through that XCD's L2 however
// long each tile takes; a workgroup whose range is used up takes tiles from the
// next ranges.  bounds[0..NQ]: first tile of each range, bounds[NQ] = total.
// Expert e of a problem (m rows, mt = ceil(m / bm) row blocks, ftiles feature
// blocks) costs ftiles * (m + mt * TILE_COST_W).  scan: NT int64 of scratch.
template <int NT>
__device__ void queue_bounds(const FfnArgs &a, int bm, int ftiles, const int *pre, const int *pre1, int total0,
                             int total, long long *scan, int *bounds) {
    const int tid = threadIdx.x;
    const int n0 = a.p[0].n_exp, n = n0 + (a.nprob > 1 ? a.p[1].n_exp : 0);
    const int per = (n + NT - 1) / NT;
    const int lo = min(tid * per, n), hi = min(lo + per, n);
    auto expert = [&](int g, long long &cost, int &tile0, int &ntiles) {
        const FfnProblem &P = g < n0 ? a.p[0] : a.p[1];
        const int e = g < n0 ? g : g - n0;
        const int m = P.offsets ? P.offsets[e + 1] - P.offsets[e] : (int)P.rows_fixed;
        const int mt = (m + bm - 1) / bm;
        cost = (long long)ftiles * ((long long)m + (long long)mt * TILE_COST_W);
        tile0 = g < n0 ? pre[e] : total0 + pre1[e];
        ntiles = mt * ftiles;
    };
    long long local = 0;
    for (int g = lo; g < hi; ++g) {
        long long c;
        int t0, nt;
        expert(g, c, t0, nt);
        local += c;
    }
    scan[tid] = local;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
        const long long v = tid >= off ? scan[tid - off] : 0;
        __syncthreads();
        scan[tid] += v;
        __syncthreads();
    }
    const long long ctot = scan[NT - 1];
    long long c0 = scan[tid] - local;
    if (tid == 0) {
        bounds[0] = 0;
        bounds[NQ] = total;
    }
    // the thread whose experts hold cost position B_x = x * ctot / NQ places boundary x
    for (int g = lo; g < hi; ++g) {
        long long c;
        int t0, nt;
        expert(g, c, t0, nt);
        for (int x = 1; x < NQ; ++x) {
            const long long B = ctot * x / NQ;
            if (c > 0 && B >= c0 && B < c0 + c) bounds[x] = t0 + (int)((B - c0) * nt / c);
        }
        c0 += c;
    }
    if (ctot == 0 && tid > 0 && tid < NQ) bounds[tid] = 0;
    __syncthreads();
}

// One grab from the tile queues by a single lane: *qpos (in LDS) is how many
// queues, in the order xcd, xcd + 1, ..., this workgroup has used up.  Returns
// the tile, or -1 once every queue is used up.  Waits for each counter value.
__device__ __forceinline__ int grab_tile(int *ctr, const int *bounds, int xcd, int *qpos) {
    int q = *qpos;
    int t = -1;
    for (; q < NQ; ++q) {
        const int qq = (xcd + q) & (NQ - 1);
        t = bounds[qq] + atomicAdd(ctr + qq, 1);
        if (t < bounds[qq + 1]) break;
        t = -1;
    }
    *qpos = q;
    return t;
}

// One 128-byte reduction step of the tile: products of the wave's RB weight
// blocks with its first NTB token blocks.  A producer wave (PROD) also issues
// the NDMA loads of a later step, spread over the step's product groups (one
// group per token block and sub-step): group g issues loads
// [g*NDMA/NG, (g+1)*NDMA/NG).  A load that has to wait for room in the memory
// pipeline then stalls the wave between products instead of ahead of them.
template <int DT, bool GATEUP, int NTB, bool PROD, int NDMA, class Dma>
__device__ __forceinline__ void compute_step(const char *st, const float *sc, f32x4 (&acc)[RB][TB], int wm, int wf,
                                             int lane, const Dma &dma) {
    typedef FTraits<DT> Tr;
    typedef Frag<DT> Fr;
    constexpr int BF = GATEUP ? WR / 2 : WR;
    constexpr int NG = Fr::kSub * NTB;
    auto group_dma = [&](int g) {
        if (PROD) {
#pragma unroll
            for (int q = g * NDMA / NG; q < (g + 1) * NDMA / NG; ++q) dma(q);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if constexpr (DT == DT_E4M3) {
        constexpr int CB = Fr::CB;
        // Fragment addresses: a lane reads chunks c = 2 (lane >> 4) and c + 1 of its row, in
        // slots c ^ swz(row) and (c ^ swz(row)) ^ 1.  swz depends on row bits 0-3 only, so the
        // 16-row blocks of a wave share one pair of lane offsets and differ by constants.
        const int r15 = lane & 15, c2 = 2 * (lane >> 4);
        const int arow = (GATEUP ? wf * (BF / WF) : wf * WRW) + r15, brow = WR + wm * 16 + r15;
        const int alo = arow * CB + ((c2 ^ swz<CB>(arow)) << 4), blo = brow * CB + ((c2 ^ swz<CB>(brow)) << 4);
        const char *a0 = st + alo, *a1 = st + (alo ^ 16), *b0 = st + blo, *b1 = st + (blo ^ 16);
        auto frag = [](const char *lo, const char *hi, int delta) {
            const i32x4 x = *(const i32x4 *)(lo + delta), y = *(const i32x4 *)(hi + delta);
            return i32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        };
        i32x8 af[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            // gate/up: first half of the wave's blocks are gate rows, second half the matching up rows
            const int drow = GATEUP ? ((i < RB / 2) ? i * 16 : BF + (i - RB / 2) * 16) : i * 16;
            af[i] = frag(a0, a1, drow * CB);
        }
        const float sw0 = sc[BM], sw1 = sc[BM + 1];
        // down: the wave's rows sit in the first or the second 128-row block
        const float swd = ((wf * WRW) >= 128) ? sw1 : sw0;
        const float *scb = sc + wm * 16 + r15;
#pragma unroll
        for (int j = 0; j < NTB; ++j) {
            const i32x8 bfr = frag(b0, b1, j * WM * 16 * CB);
            const float sa = scb[j * WM * 16];
            // the block's products first, then their scaling: the scaling of one
            // product then waits only for that product, not for a chain of them
            f32x4 part[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i) part[i] = Tr::mma(af[i], bfr, f32x4{0, 0, 0, 0});
            const float c0 = sa * sw0, c1 = sa * sw1, cd = sa * swd;
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const float cc = GATEUP ? ((i >= RB / 2) ? c1 : c0) : cd;
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[i][j][q] += part[i][q] * cc;
            }
            group_dma(j);
        }
        return;
    }
    if constexpr (DT == DT_BF16) {
        constexpr int CB = Fr::CB;
        // As for e4m3: a lane reads chunk g = lane >> 4 (sub-step 0) and g + 4 (sub-step 1),
        // in slots g ^ swz(row) and (g ^ swz(row)) ^ 4, one lane offset per operand and sub-step.
        const int r15 = lane & 15, g = lane >> 4;
        const int arow = (GATEUP ? wf * (BF / WF) : wf * WRW) + r15, brow = WR + wm * 16 + r15;
        const int alo = arow * CB + ((g ^ swz<CB>(arow)) << 4), blo = brow * CB + ((g ^ swz<CB>(brow)) << 4);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const char *as = st + (s ? (alo ^ 64) : alo), *bs = st + (s ? (blo ^ 64) : blo);
            bf16x8 af[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const int drow = GATEUP ? ((i < RB / 2) ? i * 16 : BF + (i - RB / 2) * 16) : i * 16;
                af[i] = *(const bf16x8 *)(as + drow * CB);
            }
            bf16x8 bfr[NTB];
#pragma unroll
            for (int j = 0; j < NTB; ++j) bfr[j] = *(const bf16x8 *)(bs + j * WM * 16 * CB);
            // every read above stays ahead of the first product; LDS returns in order, so each
            // group of products waits only for its own operands
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NTB; ++j) {
#pragma unroll
                for (int i = 0; i < RB; ++i) acc[i][j] = Tr::mma(af[i], bfr[j], acc[i][j]);
                group_dma(s * NTB + j);
            }
        }
        return;
    }
#pragma unroll
    for (int s = 0; s < Fr::kSub; ++s) {
        typename Fr::t af[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            // gate/up: first half of the wave's blocks are gate rows, second half the matching up rows
            const int wrow = GATEUP ? ((i < RB / 2) ? wf * (BF / WF) + i * 16 : BF + wf * (BF / WF) + (i - RB / 2) * 16)
                                    : wf * WRW + i * 16;
            af[i] = Fr::load(st, wrow + (lane & 15), s, lane);
        }
        // fp32 (bf16 and e4m3 take the paths above)
        typename Fr::t bfr[NTB];
#pragma unroll
        for (int j = 0; j < NTB; ++j) bfr[j] = Fr::load(st, WR + (j * WM + wm) * 16 + (lane & 15), s, lane);
        // every read above stays ahead of the first product; LDS returns in order, so each
        // group of products waits only for its own operands
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NTB; ++j) {
#pragma unroll
            for (int i = 0; i < RB; ++i) acc[i][j] = Tr::mma(af[i], bfr[j], acc[i][j]);
            group_dma(s * NTB + j);
        }
    }
}

// LDS bytes of the fp8 H-quantisation scratch (per-wave row maxima), kept
// apart from the ring so the next tile's loads can land during the epilogue.
template <int DT, int MODE>
__host__ __device__ constexpr int red_bytes() {
    return (DT == DT_E4M3 && (MODE == FFN_GATEUP || MODE == FFN_GATEUP_SAVE)) ? WF * BM * 4 : 0;
}


template <int DT, int MODE>
__global__ __launch_bounds__(NT, 1) void ffn_kernel(const FfnArgs a, int ring_bytes) {
    constexpr bool GATEUP = MODE == FFN_GATEUP || MODE == FFN_GATEUP_SAVE || MODE == FFN_GATEUP_BWD;   // two weight matrices
    // Weight rows that one tile alone reads load with the nontemporal policy, so that L2
    // keeps the token rows the expert's other weight-block tiles read again.  That is the
    // case for the tiles of experts with one row block; the row blocks of a larger expert
    // share its weight rows through L2.  In bf16 a tile's reduction loop is instantiated
    // per policy; the e4m3 and fp32 kernels spilled with two, so they keep one policy per
    // pass (nontemporal in gate/up, cached otherwise).
    constexpr bool WS_TILE = DT == DT_BF16;
    constexpr bool SAVEAB = MODE == FFN_GATEUP_SAVE;    // epilogue also stores the SwiGLU inputs to P.ab
    constexpr bool SWBWD = MODE == FFN_GATEUP_BWD;      // epilogue: SwiGLU gradient from dH
    constexpr int esz = FTraits<DT>::esz;
    constexpr int CB = Frag<DT>::CB;              // staged bytes per row per reduction step
    constexpr int RPI = 1024 / CB;                // rows per 1 KB DMA instruction
    constexpr int NP = 4;                         // producer waves (issue every load)
    constexpr int QW = WR / RPI / NP;             // weight DMA instructions per producer per step
    constexpr int QX = BM / RPI / NP;             // token DMA instructions per producer per step, at most
    constexpr int BF = GATEUP ? WR / 2 : WR;      // output features per tile
    constexpr bool FP8 = DT == DT_E4M3;
    static_assert(!FP8 || !GATEUP || BF == 128, "fp8 H quantisation needs whole 128-feature groups per tile");
    static_assert(!FP8 || 128 % (GATEUP ? WRW / 2 : WRW) == 0, "fp8: a wave's rows sit in one weight block");

    extern __shared__ __align__(1024) char smem[];
    const int pbytes = prefix_bytes(a.p[0].n_exp, a.nprob > 1 ? a.p[1].n_exp : 0);
    int *pre = (int *)smem;                                            // [n0 + 1] then [n1 + 1]
    float *red = (float *)(smem + pbytes);                             // fp8 gate/up: [WF][BM]
    char *ring = smem + pbytes + red_bytes<DT, MODE>();
    int *scan = (int *)ring;                                           // start-up scratch, aliases the ring

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid % WM, wf = wid / WM;
    const int K = a.K, F = a.F;
    const int ftiles = (F + BF - 1) / BF;
    const int64_t rowbytes = (int64_t)K * esz;
    const int KT = (int)(rowbytes / CB);
    const int kb_per_row = K / 128;               // fp8 scale blocks along K (one per step)

    int *pre1 = pre + a.p[0].n_exp + 1;
    int *bounds = (int *)(smem + pbytes) - SCHED_INTS;                // [NQ + 1] queue bounds
    int *slot = bounds + NQ + 1;                                       // [3] tile slots, [3] grab position
    tile_prefix<NT>(a.p[0], BM, ftiles, pre, scan);
    if (a.nprob > 1) tile_prefix<NT>(a.p[1], BM, ftiles, pre1, scan);
    const int total0 = pre[a.p[0].n_exp];
    const int total = total0 + (a.nprob > 1 ? pre1[a.p[1].n_exp] : 0);
    queue_bounds<NT>(a, BM, ftiles, pre, pre1, total0, total, (long long *)ring, bounds);

    // Loads are issued by the NP producer waves only (one per SIMD), so each
    // SIMD always has a consumer wave free to run MFMAs while its producer
    // waits on a full load queue.  Instruction i (issued by producer i % NP)
    // fills staged rows RPI*i .. RPI*i+RPI-1; lane l covers row
    // RPI*i + l/(CB/16) and stores into chunk slot l%(CB/16), which holds the
    // row's chunk slot ^ swz(row).
    const bool producer = wid < NP;
    // a scalar copy of the wave id for load addresses (LDS destinations, row offsets); the
    // divergent one keeps the compiler's loop structure around the producer branches
    const int uwid = __builtin_amdgcn_readfirstlane(wid);
    const int csub = lane / (CB / 16), cslot = lane % (CB / 16);
    const int wrow0 = RPI * wid + csub;
    // Loads go through buffer descriptors: a lane's byte offset within the tile
    // stays fixed for the whole tile (a vector register), and the step's offset
    // is a scalar, so issuing a load costs no vector instruction.
    // (e4m3 tiles use 64-bit addresses from a wave-uniform base instead: their kernel has no
    // scalar registers to spare for descriptors)
    constexpr bool BUFDMA = DT != DT_E4M3;
    const int wchunk = (cslot ^ swz<CB>(wrow0)) << 4;
    const uint32_t woff = (uint32_t)(wrow0 * rowbytes) + wchunk;

    // Everything one tile's loads and stores need (wave-uniform except the
    // per-lane offsets).
    struct Tile {
        int p, valid, r0, n0, ntb, S, stage_bytes, srows, qmax, nextra;
        int nx;                       // token instructions of this producer per step
        bool spread;                  // double-buffered: loads spread over the products
        bool xfar;                    // this producer's token rows span 4 GiB or more: 64-bit addresses
        int64_t base;                 // first row of the tile's expert
        __amdgpu_buffer_rsrc_t rw0, rw1;   // buffer loads: the tile's weight rows (gate and up, or down)
        __amdgpu_buffer_rsrc_t rx;         // buffer loads: token rows from this producer's lowest one
        const char *wbase0, *wbase1;       // 64-bit loads: this producer's first weight row
        const char *xb;                    // 64-bit loads: this producer's lowest token row (wave-uniform)
        const float *xssrc, *wssrc;   // fp8 scale sources
        bool xs_live;
        uint32_t xoff[QX];            // byte offsets of this producer's token rows in rx (row index if xfar)
    };
    auto wave_min = [](uint32_t v) {
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, m, 64));
        return (uint32_t)__builtin_amdgcn_readfirstlane(v);
    };
    auto wave_max = [](uint32_t v) {
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m, 64));
        return (uint32_t)__builtin_amdgcn_readfirstlane(v);
    };
    constexpr int RSRC_FLAGS = 0x00020000;
    auto rsrc = [](const void *p, uint64_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0,
                                                 (int)(bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes),
                                                 RSRC_FLAGS);
    };
    auto setup = [&](int t, Tile &T) {
        t = __builtin_amdgcn_readfirstlane(t);
        T.p = t < total0 ? 0 : 1;
        const FfnProblem P = pick(a, T.p);
        const int *ppre = T.p ? pre1 : pre;
        const int lt = t - (T.p ? total0 : 0);
        const int e = __builtin_amdgcn_readfirstlane(find_expert(ppre, P.n_exp, lt));
        const int pe = __builtin_amdgcn_readfirstlane(ppre[e]);
        int Me;
        if (P.offsets) {
            const int o0 = __builtin_amdgcn_readfirstlane(P.offsets[e]);
            Me = __builtin_amdgcn_readfirstlane(P.offsets[e + 1]) - o0;
            T.base = o0;
        } else {
            Me = (int)P.rows_fixed;
            T.base = (int64_t)e * P.rows_fixed;
        }
        // the expert's rows are split evenly over its row blocks, so row blocks that share
        // a weight block take equally long and stay close enough to share it through L2
        const int mt = (Me + BM - 1) / BM;
        const int ln = lt - pe;
        const int nt = ln / mt, mi = ln - nt * mt;
        const int mq = Me / mt, mr = Me - mq * mt;
        T.r0 = mi * mq + min(mi, mr);
        T.valid = mq + (mi < mr ? 1 : 0);
        T.n0 = nt * BF;
        // Token blocks this tile needs per wave: NTB = ceil(valid / (16*WM)), so the specialised
        // loops below cover 32, 64, ..., 256 tokens (padding under 32 rows per tile).  Stage
        // layout: WR weight rows, then the token rows, then (fp8) the scales.  Staging only the
        // valid rows (rounded to whole instructions) keeps stages small; the token blocks then
        // read up to `over` bytes past the last slot, which the ring keeps free.  When that
        // still leaves only two slots, the stage holds all 32*NTB token rows instead (rows past
        // the valid ones repeat the last valid token and are never stored) so that every
        // producer issues the same loads each step, spread over its products.
        T.ntb = min(TB, (T.valid + 16 * WM - 1) / (16 * WM));
        {
            const int tmin = (T.valid + RPI - 1) / RPI * RPI, tfull = T.ntb * 16 * WM;
            const int over = (tfull - tmin) * CB;
            const int smin = min((ring_bytes - over) / ((WR + tmin) * CB + (FP8 ? SCL_BYTES : 0)), 8);
            T.spread = smin < 3;
            const int trows = T.spread ? tfull : tmin;
            T.srows = WR + trows;
            T.stage_bytes = T.srows * CB + (FP8 ? SCL_BYTES : 0);
            T.S = T.spread ? min(ring_bytes / T.stage_bytes, 8) : smin;
            T.nx = 0;
#pragma unroll
            for (int q = 0; q < QX; ++q) T.nx += RPI * (q * NP + wid) < trows ? 1 : 0;
        }
        // the tile's expert has one row block: its reduction loop streams the weight rows
        if (WS_TILE && mt == 1) T.ntb += 16;
        // weight rows: instruction q < QW of this producer covers row RPI*(q*NP+wid) + csub
        // of the tile; in a ragged last tile (F - n0 < WR) the instructions past F re-read
        // the last full instruction's rows
        if (BUFDMA) {
            const uint64_t wbytes = (uint64_t)(F - T.n0) * rowbytes;
            T.rw0 = rsrc((const char *)P.w0 + ((int64_t)e * F + T.n0) * rowbytes, wbytes);
            T.rw1 = GATEUP ? rsrc((const char *)P.w1 + ((int64_t)e * F + T.n0) * rowbytes, wbytes) : T.rw0;
        } else {
            T.wbase0 = (const char *)P.w0 + ((int64_t)e * F + T.n0 + wrow0) * rowbytes + wchunk;
            T.wbase1 = GATEUP ? (const char *)P.w1 + ((int64_t)e * F + T.n0 + wrow0) * rowbytes + wchunk : T.wbase0;
        }
        T.qmax = GATEUP ? QW / 2 - 1 : min(QW, (F - T.n0) / (RPI * NP)) - 1;
        T.nextra = 0;
        T.xfar = false;
        T.xs_live = false;
        T.xssrc = T.wssrc = nullptr;
        if (uwid >= NP) return;   // producers only (tested on the scalar wave id: the rest stays uniform)
        // token rows: instruction q of this producer covers token RPI*(q*NP+wid) + csub
        {
        uint32_t xr[QX];
#pragma unroll
        for (int q = 0; q < QX; ++q) {
            const int r = min(RPI * (q * NP + wid) + csub, T.valid - 1);
            const int64_t R = T.base + T.r0 + r;
            xr[q] = (uint32_t)(P.gather ? P.gather[R] : (P.x_local ? (int64_t)(T.r0 + r) : R));
        }
        uint32_t lo = xr[0], hi = xr[0];
#pragma unroll
        for (int q = 1; q < QX; ++q) {
            lo = min(lo, xr[q]);
            hi = max(hi, xr[q]);
        }
        lo = wave_min(lo);
        hi = wave_max(hi);
        const uint64_t span = (uint64_t)(hi - lo + 1) * (uint64_t)rowbytes;
        T.xfar = span > 0xFFFFFFFFull;
        if (BUFDMA) T.rx = rsrc((const char *)P.x + (int64_t)lo * rowbytes, span);
        else T.xb = (const char *)P.x + (T.xfar ? 0 : (int64_t)lo * rowbytes);
#pragma unroll
        for (int q = 0; q < QX; ++q) {
            const int row = WR + RPI * (q * NP + wid) + csub;
            T.xoff[q] = T.xfar ? xr[q] : (uint32_t)((xr[q] - lo) * (uint64_t)rowbytes) + ((cslot ^ swz<CB>(row)) << 4);
        }
        }
        // fp8 scales, 4-byte loads into the stage's scale area: producer w stages the
        // activation scales of tokens 64w .. 64w+63 (while any is valid); producer 0 also
        // stages the two weight block scales at slots BM, BM+1 (gate/up: gate and up
        // block; down: first and second 128-row block)
        if (FP8) {
            const int r = min(wid * 64 + lane, T.valid - 1);
            const int64_t R = T.base + T.r0 + r;
            const int64_t xr = P.gather ? (int64_t)P.gather[R] : (P.x_local ? (int64_t)(T.r0 + r) : R);
            T.xssrc = P.xs + xr * kb_per_row;
            T.xs_live = wid * 64 < T.valid;
            const int nb = F / 128;
            if (GATEUP) {
                const float *sbase = (lane & 1) ? P.s1 : P.s0;
                T.wssrc = sbase + ((int64_t)e * nb + T.n0 / 128) * kb_per_row;
            } else {
                const int fb = min(T.n0 / 128 + (lane & 1), nb - 1);
                T.wssrc = P.s0 + ((int64_t)e * nb + fb) * kb_per_row;
            }
            T.nextra = (T.xs_live ? 1 : 0) + (wid == 0 ? 1 : 0);
        }
    };
    // Load q of one step by this producer: q < QW are weight instructions, the
    // rest token instructions (NTB of them cover 32*NTB token rows).
    auto dma_one = [&](const Tile &T, int q, int ks, char *st, auto farc, auto wsc) {
        constexpr bool FAR = decltype(farc)::value;
        constexpr bool WSTREAM = decltype(wsc)::value;
        if (!BUFDMA) {
            // a wave-uniform base plus the step's offset (scalar), plus the lane's fixed
            // 32-bit offset: one 64-bit vector add per load
            // an opaque copy of the row stride keeps the per-instruction offsets from being
            // hoisted out of the reduction loop into registers held for the whole tile
            int64_t rb = rowbytes;
            asm volatile("" : "+s"(rb));
            if (q < QW) {
                const bool up = GATEUP && q >= QW / 2;
                const int qq = min(GATEUP ? (up ? q - QW / 2 : q) : q, T.qmax);
                const char *src = (up ? T.wbase1 : T.wbase0) + (int64_t)qq * (RPI * NP) * rb + (int64_t)ks * CB;
                if (WSTREAM) dma16_stream(src, st + (q * NP + wid) * 1024);
                else dma16(src, st + (q * NP + wid) * 1024);
            } else {
                const int qx = q - QW;
                const int ins = qx * NP + uwid;
                char *dst = st + (WR / RPI + ins) * 1024;
                // far rows (a loop of their own): xoff holds the row itself; the chunk slot of
                // every token row this lane fills equals that of its weight rows (the swizzle
                // sees row bits 0-3 only)
                if (FAR) dma16(T.xb + (int64_t)T.xoff[qx] * rb + (int64_t)ks * CB + wchunk, dst);
                else dma16(T.xb + (int64_t)(ks * CB) + T.xoff[qx], dst);
            }
            return;
        }
        if (q < QW) {
            // gate/up: instructions q < QW/2 read gate rows, the rest the matching up rows
            const bool up = GATEUP && q >= QW / 2;
            const int qq = min(GATEUP ? (up ? q - QW / 2 : q) : q, T.qmax);
            const int soff = qq * (RPI * NP) * (int)rowbytes + ks * CB;
            if (WSTREAM) buffer_dma16_stream(up ? T.rw1 : T.rw0, woff, soff, st + (q * NP + uwid) * 1024);
            else buffer_dma16(up ? T.rw1 : T.rw0, woff, soff, st + (q * NP + uwid) * 1024);
        } else {
            const int qx = q - QW;
            const int ins = qx * NP + uwid;
            char *dst = st + (WR / RPI + ins) * 1024;
            if (!T.xfar) buffer_dma16(T.rx, T.xoff[qx], ks * CB, dst);
            else dma16((const char *)pick(a, T.p).x + (int64_t)T.xoff[qx] * rowbytes + (int64_t)ks * CB + wchunk, dst);
        }
    };
    auto dma_scales = [&](const Tile &T, int ks, char *st) {
        if (FP8) {
            if (T.xs_live) dma4(T.xssrc + ks, st + T.srows * CB + uwid * 256);
            if (wid == 0) dma4(T.wssrc + ks, st + T.srows * CB + BM * 4);
        }
    };
    // The first S-1 steps of a tile (issued while the ring is otherwise idle).
    auto prologue = [&](const Tile &T) {
        if (!producer) return;
        const int ndma = QW + T.nx;
        for (int ks = 0; ks < T.S - 1 && ks < KT; ++ks) {
            char *st = ring + ks * T.stage_bytes;
            dma_scales(T, ks, st);
#pragma unroll
            for (int q = 0; q < QW + QX; ++q)
                if (q < ndma) {
                    if (!BUFDMA && T.xfar) dma_one(T, q, ks, st, std::true_type{}, std::integral_constant<bool, GATEUP>{});
                    else dma_one(T, q, ks, st, std::false_type{}, std::integral_constant<bool, GATEUP>{});
                }
        }
    };

    // Tiles come from the queues (workgroup b runs on XCD b % 8).  One lane grabs,
    // one tile ahead: right after a tile's last barrier it takes the tile after
    // next, while the other waves start the next tile's loads and write results.
    // Tile ids pass through three LDS slots: the tile of iteration k is in slot k % 3.
    const int xcd = blockIdx.x & (NQ - 1);
    const bool grabber = wid == NW - 1 && lane == 0;
    if (grabber) {
        slot[3] = 0;
        slot[0] = grab_tile(a.ctr, bounds, xcd, slot + 3);
        slot[1] = grab_tile(a.ctr, bounds, xcd, slot + 3);
    }
    __syncthreads();
    const int first = __builtin_amdgcn_readfirstlane(slot[0]);
    Tile cur, nxt;
    if (first >= 0) {
        setup(first, cur);
        cta_barrier();   // the start-up scratch in the ring is no longer read
        prologue(cur);
    }

    int it = 0;   // iteration k, kept as k % 3
    for (int t = first; t >= 0;) {
        f32x4 acc[RB][TB];
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < TB; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

        // The reduction loop, specialised on how many of the wave's token blocks
        // (j*WM + wm, j < NTB) can hold valid tokens.  Step kt sits in ring slot
        // kt % S; the loads of step kt+S-1 go to the slot step kt-1 used, which
        // every wave has finished with once it passes step kt's barrier.  The
        // first S-1 steps were loaded before the previous tile's epilogue, whose
        // stores are younger than them in this wave's memory counter: waiting
        // for at most (S-2) steps outstanding covers them conservatively.
        const int S = cur.S, stage_bytes = cur.stage_bytes, srows = cur.srows;
        auto kloop = [&](auto ntb, auto spread, auto farc, auto wsc) {
            constexpr int NTB = decltype(ntb)::value;
            constexpr bool SPREAD = decltype(spread)::value;
            constexpr int NDMA = QW + NTB * 16 * WM / RPI / NP;   // loads per producer per step, at most
            const int nlive = QW + cur.nx + cur.nextra;
            const int kmain = KT - (S - 1);   // steps during which a later step is loaded
            int slot = 0;
            for (int kt = 0; kt < KT; ++kt) {
                // step kt has landed once at most the later steps' loads are outstanding
                if (producer) {
                    if (kt + S - 2 < KT) wait_vmcnt_dyn(__builtin_amdgcn_readfirstlane(nlive * (S - 2)));
                    else wait_vmcnt<0>();
                }
                cta_barrier();
                const char *st = ring + slot * stage_bytes;
                const float *sc = (const float *)(st + srows * CB);
                if (producer && kt < kmain) {
                    char *dst = ring + (slot == 0 ? S - 1 : slot - 1) * stage_bytes;
                    const int ks = kt + S - 1;
                    dma_scales(cur, ks, dst);
                    if (!SPREAD) {
                        // a deeper ring has room to load ahead: issue the whole step first
#pragma unroll
                        for (int q = 0; q < NDMA; ++q)
                            if (q < QW + cur.nx) dma_one(cur, q, ks, dst, farc, wsc);
                        compute_step<DT, GATEUP, NTB, false, NDMA>(st, sc, acc, wm, wf, lane, [](int) {});
                    } else {
                        // double buffering: spread the loads over the products so this
                        // wave's share of the products is not held up behind them
                        compute_step<DT, GATEUP, NTB, true, NDMA>(st, sc, acc, wm, wf, lane,
                                                                  [&](int q) { dma_one(cur, q, ks, dst, farc, wsc); });
                    }
                } else {
                    compute_step<DT, GATEUP, NTB, false, NDMA>(st, sc, acc, wm, wf, lane, [](int) {});
                }
                slot = slot + 1 == S ? 0 : slot + 1;
            }
        };
        auto kloop_p = [&](auto ntb, auto wsc) {
            if (!BUFDMA && cur.xfar) {
                // e4m3 tiles whose token rows span 4 GiB or more: 64-bit row addresses
                if (cur.spread) kloop(ntb, std::true_type{}, std::true_type{}, wsc);
                else kloop(ntb, std::false_type{}, std::true_type{}, wsc);
            } else {
                if (cur.spread) kloop(ntb, std::true_type{}, std::false_type{}, wsc);
                else kloop(ntb, std::false_type{}, std::false_type{}, wsc);
            }
        };
        auto kloop_s = [&](auto ntb) {
            if constexpr (WS_TILE) {
                if (cur.ntb >= 16) kloop_p(ntb, std::true_type{});
                else kloop_p(ntb, std::false_type{});
            } else {
                kloop_p(ntb, std::integral_constant<bool, GATEUP>{});
            }
        };
        switch (cur.ntb & 15) {
            case 1: kloop_s(std::integral_constant<int, 1>{}); break;
            case 2: kloop_s(std::integral_constant<int, 2>{}); break;
            case 3: kloop_s(std::integral_constant<int, 3>{}); break;
            case 4: kloop_s(std::integral_constant<int, 4>{}); break;
            case 5: kloop_s(std::integral_constant<int, 5>{}); break;
            case 6: kloop_s(std::integral_constant<int, 6>{}); break;
            case 7: kloop_s(std::integral_constant<int, 7>{}); break;
            default: kloop_s(std::integral_constant<int, TB>{}); break;
        }

        // Every wave is done with the ring: start the next tile's loads, then
        // write this tile's results while they are in flight.
        cta_barrier();
        const int it1 = it == 2 ? 0 : it + 1, it2 = it1 == 2 ? 0 : it1 + 1;
        const int tn = __builtin_amdgcn_readfirstlane(slot[it1]);
        if (grabber && tn >= 0) {
            // slot it2 was last read at the end of the previous iteration, before this
            // tile's barriers; it is read at the end of the next tile, after its barriers
            slot[it2] = grab_tile(a.ctr, bounds, xcd, slot + 3);
            wait_lgkm0();
        } else if (grabber) {
            slot[it2] = -1;
            wait_lgkm0();
        }
        it = it1;
        if (tn >= 0) {
            setup(tn, nxt);
            prologue(nxt);
        }

        // ---- epilogue ----
        const FfnProblem P = pick(a, cur.p);
        const int valid = cur.valid, n0 = cur.n0;
        const int64_t rbase = cur.base + cur.r0;
        // h for gate block i pairs with up block i + RB/2 (same features); it is
        // recomputed from the accumulators per 16-token block to keep registers low.
        auto hval = [&](int i, int j, int q) {
            const float g = acc[i][j][q], u = acc[i + RB / 2][j][q];
            return __fdividef(g, 1.0f + __expf(-g)) * u;
        };
        const int64_t ld = P.out_ld ? P.out_ld : F;
        if (SWBWD) {
            // a, b recomputed in the accumulators; dH of the same features from the forward's
            // gradient: da = dh * b * SiLU'(a), db = dh * SiLU(a), SiLU'(a) = s (1 + a (1 - s))
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const int tok = (j * WM + wm) * 16 + (lane & 15);
                if (tok >= valid) continue;
                const int64_t R = rbase + tok;
#pragma unroll
                for (int i = 0; i < RB / 2; ++i) {
                    const int f = n0 + wf * (BF / WF) + i * 16 + 4 * (lane >> 4);
                    float dh[4], da[4], db[4];
                    if (DT == DT_F32) {
                        const f32x4 v = *(const f32x4 *)((const float *)P.dh + R * F + f);
#pragma unroll
                        for (int q = 0; q < 4; ++q) dh[q] = v[q];
                    } else {
                        const u32x2 v = *(const u32x2 *)((const uint16_t *)P.dh + R * F + f);
                        dh[0] = __uint_as_float(v[0] << 16);
                        dh[1] = __uint_as_float(v[0] & 0xFFFF0000u);
                        dh[2] = __uint_as_float(v[1] << 16);
                        dh[3] = __uint_as_float(v[1] & 0xFFFF0000u);
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) swiglu_grad(dh[q], acc[i][j][q], acc[i + RB / 2][j][q], da[q], db[q]);
                    if (DT == DT_F32) {
                        *(f32x4 *)((float *)P.out + R * ld + f) = f32x4{da[0], da[1], da[2], da[3]};
                        *(f32x4 *)((float *)P.out + R * ld + F + f) = f32x4{db[0], db[1], db[2], db[3]};
                    } else {
                        *(u32x2 *)((uint16_t *)P.out + R * ld + f) = u32x2{pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3])};
                        *(u32x2 *)((uint16_t *)P.out + R * ld + F + f) =
                            u32x2{pack_bf16x2(db[0], db[1]), pack_bf16x2(db[2], db[3])};
                    }
                }
            }
        } else if (GATEUP) {
            if (SAVEAB) {
                // the SwiGLU inputs for a backward that reads them instead of recomputing
#pragma unroll
                for (int j = 0; j < TB; ++j) {
                    const int tok = (j * WM + wm) * 16 + (lane & 15);
                    if (tok >= valid) continue;
                    float *abrow = P.ab + (rbase + tok) * (2 * (int64_t)F);
#pragma unroll
                    for (int i = 0; i < RB / 2; ++i) {
                        const int f = n0 + wf * (BF / WF) + i * 16 + 4 * (lane >> 4);
                        *(f32x4 *)(abrow + f) = acc[i][j];
                        *(f32x4 *)(abrow + F + f) = acc[i + RB / 2][j];
                    }
                }
            }
            if (FP8) {
                // 1 x 128 groups of H along features: the tile's 128 features of a token live in
                // 4 lanes x (RB/2) blocks x 4 values in each of the WF waves of its token column
#pragma unroll
                for (int j = 0; j < TB; ++j) {
                    float m = 0.0f;
#pragma unroll
                    for (int i = 0; i < RB / 2; ++i)
#pragma unroll
                        for (int q = 0; q < 4; ++q) m = fmaxf(m, fabsf(hval(i, j, q)));
                    m = fmaxf(m, __shfl_xor(m, 16, 64));
                    m = fmaxf(m, __shfl_xor(m, 32, 64));
                    if (lane < 16) red[wf * BM + (j * WM + wm) * 16 + lane] = m;
                }
                wait_lgkm0();
                cta_barrier();
#pragma unroll
                for (int j = 0; j < TB; ++j) {
                    if ((j * WM + wm) * 16 >= valid) continue;
                    const int tok = (j * WM + wm) * 16 + (lane & 15);
                    float amax = 0.0f;
#pragma unroll
                    for (int o = 0; o < WF; ++o) amax = fmaxf(amax, red[o * BM + tok]);
                    const float scale = quant_scale(amax);
                    if (tok >= valid) continue;
                    const int64_t R = rbase + tok;
                    uint8_t *orow = (uint8_t *)P.out + R * ld;
#pragma unroll
                    for (int i = 0; i < RB / 2; ++i) {
                        const int f = n0 + wf * (BF / WF) + i * 16 + 4 * (lane >> 4);
                        *(uint32_t *)(orow + f) =
                            pack_e4m3x4(clamp448(hval(i, j, 0) / scale), clamp448(hval(i, j, 1) / scale),
                                        clamp448(hval(i, j, 2) / scale), clamp448(hval(i, j, 3) / scale));
                    }
                    if (wf == 0 && lane < 16) P.out_s[R * (F / 128) + n0 / 128] = scale;
                }
            } else {
#pragma unroll
                for (int j = 0; j < TB; ++j) {
                    const int tok = (j * WM + wm) * 16 + (lane & 15);
                    if (tok >= valid) continue;
                    const int64_t R = rbase + tok;
                    if (DT == DT_F32) {
#pragma unroll
                        for (int i = 0; i < RB / 2; ++i) {
                            const int f = n0 + wf * (BF / WF) + i * 16 + 4 * (lane >> 4);
                            *(f32x4 *)((float *)P.out + R * ld + f) =
                                f32x4{hval(i, j, 0), hval(i, j, 1), hval(i, j, 2), hval(i, j, 3)};
                        }
                    } else {
                        static_assert(RB % 4 == 0, "bf16 H stores pair blocks");
#pragma unroll
                        for (int i = 0; i < RB / 2; i += 2) {
                            const float ha[4] = {hval(i, j, 0), hval(i, j, 1), hval(i, j, 2), hval(i, j, 3)};
                            const float hb[4] = {hval(i + 1, j, 0), hval(i + 1, j, 1), hval(i + 1, j, 2),
                                                 hval(i + 1, j, 3)};
                            store_pair_bf16((uint16_t *)P.out + R * ld, n0 + wf * (BF / WF) + i * 16, ha, hb, lane, F);
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const int tok = (j * WM + wm) * 16 + (lane & 15);
                if (tok >= valid) continue;
                const int64_t R = rbase + tok;
                if (DT == DT_F32) {
#pragma unroll
                    for (int i = 0; i < RB; ++i) {
                        const int f = n0 + wf * WRW + i * 16 + 4 * (lane >> 4);
                        if (f < F) *(f32x4 *)((float *)P.out + R * ld + f) = acc[i][j];
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < RB; i += 2) {
                        const float ya[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                        const float yb[4] = {acc[i + 1][j][0], acc[i + 1][j][1], acc[i + 1][j][2], acc[i + 1][j][3]};
                        store_pair_bf16((uint16_t *)P.out + R * ld, n0 + wf * WRW + i * 16, ya, yb, lane, F);
                    }
                }
            }
        }
        cur = nxt;
        t = tn;
    }
}

// SwiGLU gradient from the forward's saved fp32 (a, b): one thread per four
// consecutive features of a row, the epilogue's arithmetic (swiglu_grad).  With QUANT
// (bf16 storage, e4m3 layers) the thread also writes the 1 x 128 tiles of the bf16
// values it stores (q, qs: codes and scales of [dA dB] rows, 32 threads per tile, the
// quantiser's arithmetic), so they need not be read back.
template <int DT, bool QUANT>
__global__ __launch_bounds__(256) void swiglu_grad_kernel(const void *__restrict__ dh, const float *__restrict__ ab,
                                                          void *__restrict__ dab, int64_t quads, int F,
                                                          uint8_t *__restrict__ q8, float *__restrict__ qs) {
    static_assert(!QUANT || DT == DT_BF16, "the fused quantisation reads bf16 values");
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    // F % 128 == 0 with QUANT, so a 32-thread tile lies in one row and is wholly in range or out
    if (q >= quads) return;
    const int fq = F / 4;
    const int64_t r = q / fq;
    const int f = (int)(q - r * fq) * 4;
    float dv[4], da[4], db[4];
    if (DT == DT_F32) {
        const f32x4 v = *(const f32x4 *)((const float *)dh + r * F + f);
#pragma unroll
        for (int k = 0; k < 4; ++k) dv[k] = v[k];
    } else {
        const u32x2 v = *(const u32x2 *)((const uint16_t *)dh + r * F + f);
        dv[0] = __uint_as_float(v[0] << 16);
        dv[1] = __uint_as_float(v[0] & 0xFFFF0000u);
        dv[2] = __uint_as_float(v[1] << 16);
        dv[3] = __uint_as_float(v[1] & 0xFFFF0000u);
    }
    const f32x4 av = __builtin_nontemporal_load((const f32x4 *)(ab + r * 2 * F + f));
    const f32x4 bv = __builtin_nontemporal_load((const f32x4 *)(ab + r * 2 * F + F + f));
#pragma unroll
    for (int k = 0; k < 4; ++k) swiglu_grad(dv[k], av[k], bv[k], da[k], db[k]);
    if (DT == DT_F32) {
        *(f32x4 *)((float *)dab + r * 2 * F + f) = f32x4{da[0], da[1], da[2], da[3]};
        *(f32x4 *)((float *)dab + r * 2 * F + F + f) = f32x4{db[0], db[1], db[2], db[3]};
    } else {
        const u32x2 pa = u32x2{pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3])};
        const u32x2 pb = u32x2{pack_bf16x2(db[0], db[1]), pack_bf16x2(db[2], db[3])};
        *(u32x2 *)((uint16_t *)dab + r * 2 * F + f) = pa;
        *(u32x2 *)((uint16_t *)dab + r * 2 * F + F + f) = pb;
        if (QUANT) {
            const int sub = threadIdx.x & 31, ntile = 2 * F / 128;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x2 p = h ? pb : pa;
                const float v[4] = {__uint_as_float(p[0] << 16), __uint_as_float(p[0] & 0xFFFF0000u),
                                    __uint_as_float(p[1] << 16), __uint_as_float(p[1] & 0xFFFF0000u)};
                float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
                for (int m = 16; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 32));
                const float scale = quant_scale(amax);
                const int64_t col = (int64_t)h * F + f;
                *(uint32_t *)(q8 + r * 2 * F + col) = pack_e4m3x4(clamp448(v[0] / scale), clamp448(v[1] / scale),
                                                                  clamp448(v[2] / scale), clamp448(v[3] / scale));
                if (sub == 0) qs[r * ntile + col / 128] = scale;
            }
        }
    }
}

// The tile-queue counters start at zero in every launch.
__global__ void zero_queues_kernel(int *ctr) {
    if (threadIdx.x < NQ) ctr[threadIdx.x] = 0;
}

template <int DT, int MODE>
hipError_t run(const FfnArgs &a, hipStream_t s) {
    if (!a.ctr) return hipErrorInvalidValue;
    static std::once_flag once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(once, [&] {
        attr_err = hipFuncSetAttribute((const void *)ffn_kernel<DT, MODE>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       LDS_TOTAL);
    });
    if (attr_err != hipSuccess) return attr_err;
    const int pb = prefix_bytes(a.p[0].n_exp, a.nprob > 1 ? a.p[1].n_exp : 0);
    const int ring = LDS_TOTAL - pb - red_bytes<DT, MODE>();
    // the ring must hold two stages of any tile
    constexpr int CB = Frag<DT>::CB;
    if (ring < 2 * ((WR + BM) * CB + (DT == DT_E4M3 ? SCL_BYTES : 0))) return hipErrorInvalidValue;
    int grid = device_cus();
    grid = (grid + 7) / 8 * 8;
    zero_queues_kernel<<<1, 64, 0, s>>>(a.ctr);
    ffn_kernel<DT, MODE><<<grid, NT, LDS_TOTAL, s>>>(a, ring);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn(int dt, int mode, const FfnArgs &a, hipStream_t s) {
    if (mode == FFN_GATEUP_BWD || mode == FFN_BWD_DH || mode == FFN_BWD_DX) {
        if (mode == FFN_GATEUP_BWD)
            return dt == DT_F32 ? run<DT_F32, FFN_GATEUP_BWD>(a, s)
                                : dt == DT_BF16 ? run<DT_BF16, FFN_GATEUP_BWD>(a, s) : run<DT_E4M3, FFN_GATEUP_BWD>(a, s);
        if (mode == FFN_BWD_DH)
            return dt == DT_F32 ? run<DT_F32, FFN_BWD_DH>(a, s)
                                : dt == DT_BF16 ? run<DT_BF16, FFN_BWD_DH>(a, s) : run<DT_E4M3, FFN_BWD_DH>(a, s);
        return dt == DT_F32 ? run<DT_F32, FFN_BWD_DX>(a, s)
                            : dt == DT_BF16 ? run<DT_BF16, FFN_BWD_DX>(a, s) : run<DT_E4M3, FFN_BWD_DX>(a, s);
    }
    if (mode == FFN_GATEUP_SAVE)
        return dt == DT_F32 ? run<DT_F32, FFN_GATEUP_SAVE>(a, s)
                            : dt == DT_BF16 ? run<DT_BF16, FFN_GATEUP_SAVE>(a, s) : run<DT_E4M3, FFN_GATEUP_SAVE>(a, s);
    const bool gateup = mode == FFN_GATEUP;
    if (dt == DT_F32) return gateup ? run<DT_F32, FFN_GATEUP>(a, s) : run<DT_F32, FFN_DOWN>(a, s);
    if (dt == DT_BF16) return gateup ? run<DT_BF16, FFN_GATEUP>(a, s) : run<DT_BF16, FFN_DOWN>(a, s);
    return gateup ? run<DT_E4M3, FFN_GATEUP>(a, s) : run<DT_E4M3, FFN_DOWN>(a, s);
}

hipError_t launch_swiglu_grad(int dt, const void *dh, const float *ab, void *dab, int64_t rows, int F, uint8_t *q8,
                              float *qs, hipStream_t s) {
    const int64_t quads = rows * (F / 4);
    if (quads <= 0) return hipSuccess;
    if (q8 && (dt != DT_BF16 || F % 128)) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)((quads + 255) / 256);
    if (dt == DT_F32) swiglu_grad_kernel<DT_F32, false><<<grid, 256, 0, s>>>(dh, ab, dab, quads, F, nullptr, nullptr);
    else if (q8) swiglu_grad_kernel<DT_BF16, true><<<grid, 256, 0, s>>>(dh, ab, dab, quads, F, q8, qs);
    else swiglu_grad_kernel<DT_BF16, false><<<grid, 256, 0, s>>>(dh, ab, dab, quads, F, nullptr, nullptr);
    return hipGetLastError();
}

}  // namespace moe
