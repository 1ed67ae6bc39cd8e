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
// walks a tile list derived from the row offsets.  A tile is (expert, block of
// 256 weight rows, block of up to 256 tokens); row blocks of one (expert,
// weight block) are adjacent in the list and consecutive tiles run on one XCD,
// so a weight tile shared by several row blocks is fetched once into that
// XCD's L2.  Up to two problems (routed and shared experts) share a launch.
//
// Data movement.  The reduction dimension is walked in 128-byte steps.  Each
// step's weight rows and token rows are copied from global memory straight
// into an LDS ring by global_load_lds (no register staging), 16 bytes per lane,
// into XOR-swizzled rows.  Only the tile's valid token rows are staged, so the
// ring depth is chosen per tile from the LDS that the stage size leaves: three
// steps deep for a typical expert.  Loads complete in order, so each wave waits
// with an exact vmcnt for its own loads of the step it consumes, then the
// workgroup meets at a fence-free barrier.
//
// MFMA orientation: weights are the MFMA row operand and tokens the column
// operand, so a lane's four accumulators are four consecutive output features
// of one token.  Eight waves (two per SIMD) form a 2 (tokens) x 4 (weight rows)
// grid; each wave owns 64 weight rows x 128 tokens.
#include <mutex>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace moe {

namespace {

template <int DT>
struct FTraits;
template <>
struct FTraits<DT_F32> {
    static constexpr int esz = 4;
    __device__ static f32x4 mma(float a, float b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }
};
template <>
struct FTraits<DT_BF16> {
    static constexpr int esz = 2;
    __device__ static f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct FTraits<DT_E4M3> {
    // one 16x16x128 MFMA covers exactly one 128-long quantisation block
    static constexpr int esz = 1;
    __device__ static f32x4 mma(i32x8 a, i32x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);   // unit E8M0 scales
    }
};

// Staged rows hold CB bytes of the reduction dimension (128: one e4m3 MFMA
// step, two bf16 steps, eight fp32 steps), as CB/16 chunks of 16 bytes in
// XOR-permuted slots.  Lanes 0-15 of a fragment read take one chunk
// column of 16 consecutive rows; the permutations put those reads in distinct
// banks whether the LDS serves 8 or 16 such reads per cycle.
template <int CB>
__device__ __forceinline__ int swz(int row) {
    if (CB == 128) return (row & 7) ^ ((row >> 3) & 1);
    return ((row >> 1) ^ (row >> 3)) & 3;
}

template <int DT>
struct Frag;
template <>
struct Frag<DT_F32> {
    static constexpr int CB = 128, kSub = 8;  // 16x16x4 steps per 128-byte row
    typedef float t;
    __device__ static t load(const char *stage, int row, int s, int lane) {
        return *(const float *)(stage + row * CB + ((s ^ swz<CB>(row)) << 4) + (lane >> 4) * 4);
    }
};
template <>
struct Frag<DT_BF16> {
    static constexpr int CB = 128, kSub = 2;  // 16x16x32 steps per 128-byte row
    typedef bf16x8 t;
    __device__ static t load(const char *stage, int row, int s, int lane) {
        return *(const bf16x8 *)(stage + row * CB + (((s * 4 + (lane >> 4)) ^ swz<CB>(row)) << 4));
    }
};
template <>
struct Frag<DT_E4M3> {
    static constexpr int CB = 128, kSub = 1;  // one 16x16x128 step per 128-byte row
    typedef i32x8 t;
    __device__ static t load(const char *stage, int row, int s, int lane) {
        const int c = 2 * (lane >> 4);
        const i32x4 lo = *(const i32x4 *)(stage + row * CB + ((c ^ swz<CB>(row)) << 4));
        const i32x4 hi = *(const i32x4 *)(stage + row * CB + (((c + 1) ^ swz<CB>(row)) << 4));
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
};

// Fence-free workgroup barrier: the ring is filled by direct global->LDS loads
// whose completion each wave establishes with an explicit vmcnt wait.
__device__ __forceinline__ void cta_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt vmcnt(n) for a wave-uniform n (the immediate is encoded per case;
// counts above 47 wait for everything, which is only more conservative).
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
    switch (n) {
#define MOE_VMCNT_CASE(k) case k: wait_vmcnt<k>(); break;
        MOE_VMCNT_CASE(1) MOE_VMCNT_CASE(2) MOE_VMCNT_CASE(3) MOE_VMCNT_CASE(4) MOE_VMCNT_CASE(5)
        MOE_VMCNT_CASE(6) MOE_VMCNT_CASE(7) MOE_VMCNT_CASE(8) MOE_VMCNT_CASE(9) MOE_VMCNT_CASE(10)
        MOE_VMCNT_CASE(11) MOE_VMCNT_CASE(12) MOE_VMCNT_CASE(13) MOE_VMCNT_CASE(14) MOE_VMCNT_CASE(15)
        MOE_VMCNT_CASE(16) MOE_VMCNT_CASE(17) MOE_VMCNT_CASE(18) MOE_VMCNT_CASE(19) MOE_VMCNT_CASE(20)
        MOE_VMCNT_CASE(21) MOE_VMCNT_CASE(22) MOE_VMCNT_CASE(23) MOE_VMCNT_CASE(24) MOE_VMCNT_CASE(25)
        MOE_VMCNT_CASE(26) MOE_VMCNT_CASE(27) MOE_VMCNT_CASE(28) MOE_VMCNT_CASE(29) MOE_VMCNT_CASE(30)
        MOE_VMCNT_CASE(31) MOE_VMCNT_CASE(32) MOE_VMCNT_CASE(33) MOE_VMCNT_CASE(34) MOE_VMCNT_CASE(35)
        MOE_VMCNT_CASE(36) MOE_VMCNT_CASE(37) MOE_VMCNT_CASE(38) MOE_VMCNT_CASE(39) MOE_VMCNT_CASE(40)
        MOE_VMCNT_CASE(41) MOE_VMCNT_CASE(42) MOE_VMCNT_CASE(43) MOE_VMCNT_CASE(44) MOE_VMCNT_CASE(45)
        MOE_VMCNT_CASE(46) MOE_VMCNT_CASE(47)
#undef MOE_VMCNT_CASE
        default: wait_vmcnt<0>(); break;
    }
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void *g, void *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)l, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *g, void *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)l, 4, 0, 0);
}

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

// LDS bytes besides the ring: tile prefixes of both problems (n_exp + 1 each).
__host__ __device__ inline int prefix_bytes(int n0, int n1) { return ((n0 + 1 + n1 + 1) * 4 + 255) & ~255; }

// One 128-byte reduction step of the tile: products of the wave's RB weight
// blocks with its first NTB token blocks.
// Token blocks past the staged rows read whatever follows the stage in the
// ring (the ring depth leaves room for it); those columns are never stored.
template <int DT, bool GATEUP, int NTB>
__device__ __forceinline__ void compute_step(const char *st, const float *sc, int trows, f32x4 (&acc)[RB][TB],
                                             int wm, int wf, int lane) {
    typedef FTraits<DT> Tr;
    typedef Frag<DT> Fr;
    constexpr int BF = GATEUP ? WR / 2 : WR;
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
        if (DT == DT_E4M3) {
#pragma unroll
            for (int j = 0; j < NTB; ++j) {
                const int tok = (j * WM + wm) * 16 + (lane & 15);
                const typename Fr::t bfr = Fr::load(st, WR + tok, s, lane);
                const float sa = sc[tok];
                const float c0 = sa * sc[BM], c1 = sa * sc[BM + 1];
                // down: the wave's rows sit in the first or the second 128-row block
                const float cdown = ((wf * WRW) >= 128) ? c1 : c0;
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    const f32x4 part = Tr::mma(af[i], bfr, f32x4{0, 0, 0, 0});
                    const float cc = GATEUP ? ((i >= RB / 2) ? c1 : c0) : cdown;
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[i][j][q] += part[q] * cc;
                }
            }
        } else {
            typename Fr::t bfr[NTB];
#pragma unroll
            for (int j = 0; j < NTB; ++j) bfr[j] = Fr::load(st, WR + (j * WM + wm) * 16 + (lane & 15), s, lane);
            // every read above stays ahead of the first product; LDS returns in order, so each
            // group of products waits only for its own operands
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NTB; ++j)
#pragma unroll
                for (int i = 0; i < RB; ++i) acc[i][j] = Tr::mma(af[i], bfr[j], acc[i][j]);
        }
    }
}

template <int DT, bool GATEUP>
__global__ __launch_bounds__(NT, 1) void ffn_kernel(const FfnArgs a, int ring_bytes) {
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
    int *pre = (int *)smem;                                            // [n0 + 1] then [n1 + 1]
    char *ring = smem + prefix_bytes(a.p[0].n_exp, a.nprob > 1 ? a.p[1].n_exp : 0);
    int *scan = (int *)ring;                                           // start-up scratch, aliases the ring
    float *red = (float *)ring;                                        // fp8 epilogue scratch, aliases the ring

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid % WM, wf = wid / WM;
    const int K = a.K, F = a.F;
    const int ftiles = (F + BF - 1) / BF;
    const int64_t rowbytes = (int64_t)K * esz;
    const int KT = (int)(rowbytes / CB);
    const int kb_per_row = K / 128;               // fp8 scale blocks along K (one per step)

    int *pre1 = pre + a.p[0].n_exp + 1;
    tile_prefix<NT>(a.p[0], BM, ftiles, pre, scan);
    if (a.nprob > 1) tile_prefix<NT>(a.p[1], BM, ftiles, pre1, scan);
    const int total0 = pre[a.p[0].n_exp];
    const int total = total0 + (a.nprob > 1 ? pre1[a.p[1].n_exp] : 0);

    // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a contiguous run of tiles.
    const int G = gridDim.x;
    const int first = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

    for (int t = first; t < total; t += G) {
        const int p = t < total0 ? 0 : 1;
        const FfnProblem P = pick(a, p);
        const int *ppre = p ? pre1 : pre;
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

        // Stage layout: WR weight rows, then the valid token rows rounded up to
        // whole DMA instructions, then (fp8) the scales.  The ring holds as many
        // stages as fit.
        const int trows = (valid + RPI - 1) / RPI * RPI;
        const int srows = WR + trows;
        const int stage_bytes = srows * CB + (FP8 ? SCL_BYTES : 0);
        // token blocks this tile needs per wave: NTB = ceil(valid / (16*WM)) rounded up to an even
        // count, so the specialised loops below cover 64, 128, 192 or 256 tokens; the last slot's
        // blocks may read up to `over` bytes past the staged rows
        const int ntb = min(TB, ((valid + 16 * WM - 1) / (16 * WM) + 1) & ~1);
        const int over = max(0, ntb * 16 * WM - trows) * CB;
        const int S = min((ring_bytes - over) / stage_bytes, 8);

        // Loads are issued by the NP producer waves only (one per SIMD), so each
        // SIMD always has a consumer wave free to run MFMAs while its producer
        // waits on a full load queue.  Instruction i (issued by producer i % NP)
        // fills staged rows RPI*i .. RPI*i+RPI-1; lane l covers row
        // RPI*i + l/(CB/16) and stores into chunk slot l%(CB/16), which holds the
        // row's chunk slot ^ swz(row).  Weight rows past F clamp to F-1.
        const bool producer = wid < NP;
        const int csub = lane / (CB / 16), cslot = lane % (CB / 16);
        // weight rows: instruction q < QW of this producer covers row RPI*(q*NP+wid) + csub.  The
        // chunk permutation does not depend on q (RPI*NP rows apart), so one base pointer per
        // weight matrix plus a per-instruction row stride addresses them all; in a ragged last
        // tile (F - n0 < WR) the instructions past F re-read the last full instruction's rows.
        const int wrow0 = RPI * wid + csub;
        const int wchunk = (cslot ^ swz<CB>(wrow0)) << 4;
        const char *wbase0 = (const char *)P.w0 + ((int64_t)e * F + n0 + wrow0) * rowbytes + wchunk;
        const char *wbase1 = GATEUP ? (const char *)P.w1 + ((int64_t)e * F + n0 + wrow0) * rowbytes + wchunk : wbase0;
        const int qmax = GATEUP ? QW / 2 - 1 : min(QW, (F - n0) / (RPI * NP)) - 1;
        // token rows: instruction q of this producer covers token RPI*(q*NP+wid) + csub
        int xrow[QX];
        int nxq = 0;
#pragma unroll
        for (int q = 0; q < QX; ++q) {
            const int tr = RPI * (q * NP + wid) + csub;
            const int r = min(tr, valid - 1);
            const int64_t R = base + r0 + r;
            xrow[q] = P.gather ? P.gather[R] : (int)(P.x_local ? (int64_t)(r0 + r) : R);
            nxq += RPI * (q * NP + wid) < trows ? 1 : 0;
        }
        int nlive = producer ? QW + nxq : 0;
        // fp8 scales, 4-byte DMAs into the stage's scale area: producer w stages
        // the activation scales of tokens 64w .. 64w+63 (while any is valid);
        // producer 0 also stages the two weight block scales at slots BM, BM+1
        // (gate/up: gate and up block; down: first and second 128-row block).
        const float *xssrc = nullptr, *wssrc = nullptr;
        bool xs_live = false;
        if (FP8 && producer) {
            const int r = min(wid * 64 + lane, valid - 1);
            const int64_t R = base + r0 + r;
            const int64_t xr = P.gather ? (int64_t)P.gather[R] : (P.x_local ? (int64_t)(r0 + r) : R);
            xssrc = P.xs + xr * kb_per_row;
            xs_live = wid * 64 < valid;
            const int nb = F / 128;
            if (GATEUP) {
                const float *sbase = (lane & 1) ? P.s1 : P.s0;
                wssrc = sbase + ((int64_t)e * nb + n0 / 128) * kb_per_row;
            } else {
                const int fb = min(n0 / 128 + (lane & 1), nb - 1);
                wssrc = P.s0 + ((int64_t)e * nb + fb) * kb_per_row;
            }
            nlive += (xs_live ? 1 : 0) + (wid == 0 ? 1 : 0);
        }
        const char *xbase = (const char *)P.x;

        int slot_issue = 0;   // ring slot of the next stage issued
        auto issue = [&](int ks) {
            char *st = ring + slot_issue * stage_bytes;
            if (producer) {
                // an opaque copy of the row stride keeps the per-instruction addresses
                // from being hoisted out of the reduction loop (they would occupy
                // ~32 VGPRs for the whole tile); recomputing them costs a few SALU/VALU ops
                int64_t rb = rowbytes;
                asm volatile("" : "+s"(rb));
#pragma unroll
                for (int q = 0; q < QW; ++q) {
                    // gate/up: instructions q < QW/2 read gate rows, the rest the matching up rows
                    const bool up = GATEUP && q >= QW / 2;
                    const int qq = min(GATEUP ? (up ? q - QW / 2 : q) : q, qmax);
                    const char *src = (up ? wbase1 : wbase0) + (int64_t)qq * (RPI * NP) * rb + (int64_t)ks * CB;
                    dma16(src, st + (q * NP + wid) * 1024);
                }
#pragma unroll
                for (int q = 0; q < QX; ++q) {
                    const int ins = q * NP + wid;
                    if (RPI * ins >= trows) continue;
                    const int row = WR + RPI * ins + csub;
                    const char *src = xbase + (int64_t)xrow[q] * rb + (int64_t)ks * CB + ((cslot ^ swz<CB>(row)) << 4);
                    dma16(src, st + (WR / RPI + ins) * 1024);
                }
                if (FP8) {
                    if (xs_live) dma4(xssrc + ks, st + srows * CB + wid * 256);
                    if (wid == 0) dma4(wssrc + ks, st + srows * CB + BM * 4);
                }
            }
            slot_issue = slot_issue + 1 == S ? 0 : slot_issue + 1;
        };

        f32x4 acc[RB][TB];
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < TB; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

        cta_barrier();   // every wave is done with the ring (previous tile, start-up or epilogue scratch)
        for (int ks = 0; ks < S - 1 && ks < KT; ++ks) issue(ks);

        // The reduction loop, specialised on how many of the wave's token blocks
        // (j*WM + wm, j < NTB) can hold valid tokens.
        auto kloop = [&](auto ntb) {
            constexpr int NTB = decltype(ntb)::value;
            int slot = 0;
            for (int kt = 0; kt < KT; ++kt) {
                // step kt has landed once at most the later steps' loads are outstanding
                if (producer) {
                    if (kt + S - 2 < KT) wait_vmcnt_dyn(nlive * (S - 2));
                    else wait_vmcnt<0>();
                }
                cta_barrier();
                if (kt + S - 1 < KT) issue(kt + S - 1);
                const char *st = ring + slot * stage_bytes;
                const float *sc = (const float *)(st + srows * CB);
                compute_step<DT, GATEUP, NTB>(st, sc, trows, acc, wm, wf, lane);
                slot = slot + 1 == S ? 0 : slot + 1;
            }
        };
        if (ntb == 2) kloop(std::integral_constant<int, 2>{});
        else if (ntb == 4) kloop(std::integral_constant<int, 4>{});
        else if (ntb == 6) kloop(std::integral_constant<int, 6>{});
        else kloop(std::integral_constant<int, TB>{});

        // ---- epilogue ----
        // h for gate block i pairs with up block i + RB/2 (same features); it is
        // recomputed from the accumulators per 16-token block to keep registers low.
        auto hval = [&](int i, int j, int q) {
            const float g = acc[i][j][q], u = acc[i + RB / 2][j][q];
            return __fdividef(g, 1.0f + __expf(-g)) * u;
        };
        if (GATEUP) {
            if (FP8) {
                // 1 x 128 groups of H along features: the tile's 128 features of a token live in
                // 4 lanes x (RB/2) blocks x 4 values in each of the WF waves of its token column
                cta_barrier();   // the ring is free: every wave has finished its last step
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
                __syncthreads();
#pragma unroll
                for (int j = 0; j < TB; ++j) {
                    if ((j * WM + wm) * 16 >= valid) continue;
                    const int tok = (j * WM + wm) * 16 + (lane & 15);
                    float amax = 0.0f;
#pragma unroll
                    for (int o = 0; o < WF; ++o) amax = fmaxf(amax, red[o * BM + tok]);
                    const float scale = quant_scale(amax);
                    if (tok >= valid) continue;
                    const int64_t R = base + r0 + tok;
                    uint8_t *orow = (uint8_t *)P.out + R * F;
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
                    const int64_t R = base + r0 + tok;
#pragma unroll
                    for (int i = 0; i < RB / 2; ++i) {
                        const int f = n0 + wf * (BF / WF) + i * 16 + 4 * (lane >> 4);
                        const float h0 = hval(i, j, 0), h1 = hval(i, j, 1), h2 = hval(i, j, 2), h3 = hval(i, j, 3);
                        if (DT == DT_F32) {
                            *(f32x4 *)((float *)P.out + R * F + f) = f32x4{h0, h1, h2, h3};
                        } else {
                            *(u32x2 *)((uint16_t *)P.out + R * F + f) = u32x2{pack_bf16x2(h0, h1), pack_bf16x2(h2, h3)};
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const int tok = (j * WM + wm) * 16 + (lane & 15);
                if (tok >= valid) continue;
                const int64_t R = base + r0 + tok;
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    const int f = n0 + wf * WRW + i * 16 + 4 * (lane >> 4);
                    if (f >= F) continue;
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

template <int DT, bool GATEUP>
hipError_t run(const FfnArgs &a, hipStream_t s) {
    static std::once_flag once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(once, [&] {
        attr_err = hipFuncSetAttribute((const void *)ffn_kernel<DT, GATEUP>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       LDS_TOTAL);
    });
    if (attr_err != hipSuccess) return attr_err;
    const int pb = prefix_bytes(a.p[0].n_exp, a.nprob > 1 ? a.p[1].n_exp : 0);
    const int ring = LDS_TOTAL - pb;
    // the ring must hold two stages of any tile plus its read past the last slot (at most 56 rows)
    constexpr int CB = Frag<DT>::CB;
    if (ring < 2 * ((WR + BM) * CB + (DT == DT_E4M3 ? SCL_BYTES : 0)) + 56 * CB) return hipErrorInvalidValue;
    int grid = device_cus();
    grid = (grid + 7) / 8 * 8;
    ffn_kernel<DT, GATEUP><<<grid, NT, LDS_TOTAL, s>>>(a, ring);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn(int dt, bool gateup, const FfnArgs &a, hipStream_t s) {
    if (dt == DT_F32) return gateup ? run<DT_F32, true>(a, s) : run<DT_F32, false>(a, s);
    if (dt == DT_BF16) return gateup ? run<DT_BF16, true>(a, s) : run<DT_BF16, false>(a, s);
    return gateup ? run<DT_E4M3, true>(a, s) : run<DT_E4M3, false>(a, s);
}

}  // namespace moe
