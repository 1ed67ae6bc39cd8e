// backward.hip -- gradient of the DeepSeekMoE layer ("DeepSeek-V3 Technical
// Report", §2.1.2) for the selection the forward made (the selection is
// piecewise constant; the bias receives no gradient).  With upstream gradient
// dO of the layer output:
//   dy_{t,j} = g_{t,j} dO_t,  dg_{t,j} = dO_t . y_{t,j}      (combine)
//   per expert row: dh = W_down^T dy, dW_down += dy h^T        (down)
//     da = dh b SiLU'(a), db = dh SiLU(a)                       (SwiGLU, in the expert kernel)
//     dx = W_gate^T da + W_up^T db, dW_gate += da x^T, dW_up += db x^T
//   g_j = rs s_j / D: ds_k = rs (dg_k / D - (sum_j dg_j s_j) / D^2), dz = ds s (1 - s)
//   du_t = sum_j dx_{t,j} + dx_shared + sum_k dz_k e_k,  de_k += dz_k u_t.
// The input-gradient products run in the grouped expert kernel with
// transposed weight copies; this file holds the memory-bound token passes,
// the centroid gradient, the weight-gradient GEMM and the weight transpose.
#include "common.h"
#include "internal.h"
#include "lds_ring.h"

#include <mutex>
#include <type_traits>

namespace moe {

namespace {

template <int DT>
__device__ __forceinline__ float ld1(const void *p, int64_t i) {
    if (DT == DT_F32) return ((const float *)p)[i];
    return __uint_as_float((uint32_t)((const uint16_t *)p)[i] << 16);
}

// 8 consecutive elements from (DT storage) p + i
template <int DT>
__device__ __forceinline__ void ld8v(const void *p, int64_t i, float v[8]) {
    if (DT == DT_BF16) {
        const u32x4 w = *(const u32x4 *)((const uint16_t *)p + i);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(w[k] << 16);
            v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
    } else {
        const f32x4 a = *(const f32x4 *)((const float *)p + i), b = *(const f32x4 *)((const float *)p + i + 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) { v[k] = a[k]; v[4 + k] = b[k]; }
    }
}

template <int DT>
__device__ __forceinline__ void st8v(void *p, int64_t i, const float v[8]) {
    if (DT == DT_BF16) {
        *(u32x4 *)((uint16_t *)p + i) =
            u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
    } else {
        *(f32x4 *)((float *)p + i) = f32x4{v[0], v[1], v[2], v[3]};
        *(f32x4 *)((float *)p + i + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
}

constexpr int BW_NT = 256;

// ---- weight transpose: dst[m][c][col0 + r] = src[m][r][c] (64 x 64 tiles) ----
template <int ESZ>
__global__ __launch_bounds__(256) void transpose_kernel(const char *__restrict__ src, int rows, int cols,
                                                       char *__restrict__ dst, int dst_ld, int col0) {
    typedef typename std::conditional<ESZ == 1, uint8_t,
                                      typename std::conditional<ESZ == 2, uint16_t, uint32_t>::type>::type E;
    __shared__ E tile[64][65];
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const int64_t tiles_c = cols / 64, tiles_per = (int64_t)(rows / 64) * tiles_c;
    const int64_t m = blockIdx.x / tiles_per, tt = blockIdx.x % tiles_per;
    const int r0 = (int)(tt / tiles_c) * 64, c0 = (int)(tt % tiles_c) * 64;
    const E *s = (const E *)src + (size_t)m * rows * cols;
    E *d = (E *)dst + (size_t)m * cols * dst_ld;
#pragma unroll
    for (int k = 0; k < 16; ++k) tile[ty + 4 * k][tx] = s[(size_t)(r0 + ty + 4 * k) * cols + c0 + tx];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) d[(size_t)(c0 + ty + 4 * k) * dst_ld + col0 + r0 + tx] = tile[tx][ty + 4 * k];
}

// 1 x 128 tile of eight stored values per lane (16 lanes of one tile): the scale and
// the four-byte code pairs, the arithmetic of quant_rows_kernel on the same values
__device__ __forceinline__ void quant8_tile(const float v[8], uint8_t *q, float *sc, int sub) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
    const float scale = quant_scale(amax);
    *(u32x2 *)q = u32x2{pack_e4m3x4(clamp448(v[0] / scale), clamp448(v[1] / scale), clamp448(v[2] / scale),
                                    clamp448(v[3] / scale)),
                        pack_e4m3x4(clamp448(v[4] / scale), clamp448(v[5] / scale), clamp448(v[6] / scale),
                                    clamp448(v[7] / scale))};
    if (sub == 0) *sc = scale;
}

// ---- combine backward: one workgroup per token ----
// dY[inv(t,j)] = g_{t,j} dO_t (rounded to the act dtype); dg_{t,j} = dO_t . y[inv(t,j)]
// With QUANT (bf16, for e4m3 layers) the kernel also writes the 1 x 128 tiles of dY
// (dyq, dys) and, when doq is set, of dO: the codes quant_rows_kernel would make from
// the stored bf16 values, without reading them back.
template <int DT, int KMAX, bool QUANT>
__global__ __launch_bounds__(BW_NT) void bwd_combine_kernel(const void *__restrict__ dout, const void *__restrict__ y,
                                                            const int32_t *__restrict__ inv,
                                                            const float *__restrict__ topk_w, int64_t T, int d, int K,
                                                            void *__restrict__ dy, float *__restrict__ dg,
                                                            uint8_t *__restrict__ dyq, float *__restrict__ dys,
                                                            uint8_t *__restrict__ doq, float *__restrict__ dos) {
    static_assert(!QUANT || DT == DT_BF16, "the fused quantisation reads bf16 values");
    static_assert(BW_NT % 16 == 0, "a 1 x 128 tile is 16 consecutive threads");
    __shared__ float red[BW_NT / 64][KMAX];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        float part[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) part[j] = 0.0f;
        for (int c = threadIdx.x * 8; c < d; c += BW_NT * 8) {
            float o[8];
            ld8v<DT>(dout, t * d + c, o);
            const int sub = threadIdx.x & 15, ntile = d >> 7;
            if (QUANT && doq) quant8_tile(o, doq + t * d + c, dos + t * ntile + (c >> 7), sub);
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                if (j >= K) break;
                const int64_t row = inv[t * K + j];
                const float g = topk_w[t * K + j];
                float v[8], w[8];
                ld8v<DT>(y, row * d + c, v);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    part[j] += o[q] * v[q];
                    w[q] = g * o[q];
                }
                st8v<DT>(dy, row * d + c, w);
                if (QUANT) {
                    float wb[8];   // the stored bf16 values
#pragma unroll
                    for (int q = 0; q < 8; q += 2) {
                        const uint32_t pk = pack_bf16x2(w[q], w[q + 1]);
                        wb[q] = __uint_as_float(pk << 16);
                        wb[q + 1] = __uint_as_float(pk & 0xFFFF0000u);
                    }
                    quant8_tile(wb, dyq + row * d + c, dys + row * ntile + (c >> 7), sub);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j >= K) break;
            float v = part[j];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            if (lane == 0) red[wid][j] = v;
        }
        __syncthreads();
        if ((int)threadIdx.x < K) {
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < BW_NT / 64; ++w) v += red[w][threadIdx.x];
            dg[t * K + threadIdx.x] = v;
        }
        __syncthreads();
    }
}

// ---- token backward: dispatch sum + router chain, one workgroup per token ----
// du_t = sum_j dXr[inv(t,j)] + sum_s dXs[s][t] + sum_j dz_j e_{sel_j};  dz also per row.
template <int DT, int KMAX>
__global__ __launch_bounds__(BW_NT) void bwd_token_kernel(const void *__restrict__ dxr, const void *__restrict__ dxs,
                                                          int Ns, const int32_t *__restrict__ inv,
                                                          const int32_t *__restrict__ idx,
                                                          const float *__restrict__ scores,
                                                          const float *__restrict__ dg,
                                                          const void *__restrict__ gate_w, int64_t T, int d, int Nr,
                                                          int K, float rs, void *__restrict__ du,
                                                          float *__restrict__ dz_row) {
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        // gate chain (every thread, identical arithmetic): D in slot order as the forward summed it
        float s[KMAX], dz[KMAX];
        float den = 0.0f, sdg = 0.0f;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j >= K) break;
            s[j] = scores[t * Nr + idx[t * K + j]];
            den = den + s[j];
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j >= K) break;
            sdg += dg[t * K + j] * s[j];
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j >= K) break;
            dz[j] = rs * (dg[t * K + j] / den - sdg / (den * den)) * s[j] * (1.0f - s[j]);
        }
        if ((int)threadIdx.x < K) {
#pragma unroll
            for (int j = 0; j < KMAX; ++j)
                if (j == (int)threadIdx.x) dz_row[inv[t * K + j]] = dz[j];
        }
        for (int c = threadIdx.x * 8; c < d; c += BW_NT * 8) {
            float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                if (j >= K) break;
                float v[8], e[8];
                ld8v<DT>(dxr, (int64_t)inv[t * K + j] * d + c, v);
                ld8v<DT>(gate_w, (int64_t)idx[t * K + j] * d + c, e);
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[q] += v[q] + dz[j] * e[q];
            }
            for (int q0 = 0; q0 < Ns; ++q0) {
                float v[8];
                ld8v<DT>(dxs, ((int64_t)q0 * T + t) * d + c, v);
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[q] += v[q];
            }
            st8v<DT>(du, t * d + c, acc);
        }
    }
}

// ---- centroid gradient: de_i[c] = sum over expert i's rows r (in order) of dz_row[r] u[perm[r]][c] ----
template <int DT>
__global__ __launch_bounds__(BW_NT) void dgate_kernel(const void *__restrict__ u, const int32_t *__restrict__ perm,
                                                      const int32_t *__restrict__ offsets,
                                                      const float *__restrict__ dz_row, int d, int chunks,
                                                      float *__restrict__ dgate) {
    const int i = blockIdx.x / chunks, ch = blockIdx.x % chunks;
    const int c = (ch * BW_NT + (int)threadIdx.x) * 8;
    if (c >= d) return;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int r = offsets[i]; r < offsets[i + 1]; ++r) {
        const float z = dz_row[r];
        float v[8];
        ld8v<DT>(u, (int64_t)perm[r] * d + c, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += z * v[q];
    }
    *(f32x4 *)(dgate + (int64_t)i * d + c) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *(f32x4 *)(dgate + (int64_t)i * d + c + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

// ---- weight-gradient tile order ---------------------------------------------
// A tile is (problem, expert, 128-wide p tile, group of 128-wide q tiles); the
// group size wg_qgroup keeps roughly 32 reduction steps (of the kernel's
// step_rows rows) per workgroup.  Tiles
// of a fixed-rows problem (the shared experts: every token, long reductions)
// come first, one per workgroup in launch order so they spread over all XCDs
// and start early; the routed experts' tiles follow in contiguous ranges per
// XCD (workgroup b runs on XCD b % 8), so an expert's activations are read
// into one or two L2s rather than all eight.
__host__ __device__ inline int wg_qgroup(const WgradProblem &P) {
    const int nqt = P.Qdim / 128;
    const int64_t steps = (P.rows_hint + P.step_rows - 1) / P.step_rows;
    const int g = steps >= 32 ? 1 : (int)(32 / (steps > 0 ? steps : 1));
    return g < nqt ? g : nqt;
}
__host__ __device__ inline int64_t wg_tiles(const WgradProblem &P) {
    const int nqt = P.Qdim / 128, g = wg_qgroup(P);
    return (int64_t)P.n_exp * (P.Pdim / P.p_tile) * ((nqt + g - 1) / g);
}

struct WgTile {
    int pi, e, p0, qt0, nq;
};

// workgroup b -> tile; false for a workgroup with no tile
__device__ inline bool wg_decode(const WgradArgs &a, int64_t nlead, int64_t ntiles, int64_t b, WgTile &T) {
    int64_t t;
    const int64_t nlead8 = (nlead + 7) / 8 * 8;
    if (b < nlead) {
        t = b;
    } else if (b < nlead8) {
        return false;
    } else {
        const int64_t c = b - nlead8, per_xcd = (ntiles - nlead + 7) / 8;
        t = nlead + (c & 7) * per_xcd + (c >> 3);
        if (t >= ntiles) return false;
    }
    T.pi = 0;
    const int64_t t0 = wg_tiles(a.p[0]);
    if (a.nprob > 1 && t >= t0) {
        t -= t0;
        T.pi = 1;
    }
    const WgradProblem &P = T.pi ? a.p[1] : a.p[0];
    const int ptiles = P.Pdim / P.p_tile, nqt = P.Qdim / 128, g = wg_qgroup(P);
    const int ngroups = (nqt + g - 1) / g;
    T.e = (int)(t / ((int64_t)ptiles * ngroups));
    const int r = (int)(t - (int64_t)T.e * ptiles * ngroups);
    T.p0 = (r / ngroups) * P.p_tile;
    T.qt0 = (r % ngroups) * g;
    T.nq = min(g, nqt - T.qt0);
    return true;
}

// ---- weight gradient: C[p][q] = sum over an expert's rows r of P[r][p] Q[qrow(r)][q] ----
// fp32 layers.  A workgroup (4 waves, 2 x 2 of 64 x 64) owns one tile of the
// order above, walked in 32-row reduction steps per q tile.
// Every step stages 32 rows x 128 values of P and of Q transposed in LDS
// ([value][row], rows contiguous), so MFMA fragments (8 consecutive rows per
// lane) are two 8-byte reads.  Half the threads stage P and half Q: a thread
// loads a 4-row x 8-value patch (four 16-byte loads, coalesced along the row)
// and writes its eight 4-row columns as 8-byte stores; the 4-row group's slot
// inside an LDS row is XOR-swizzled by the row index so that neither the
// stores nor the fragment reads pile onto a few banks.  Two LDS buffers: the
// global loads of step i+1 are in flight while step i runs its MFMAs.  Q is
// the MFMA row operand (a lane's four results are four consecutive q of one
// p).  All of an expert's rows are reduced in one tile, in order: no
// cross-tile reduction, deterministic.
constexpr int WG_T = 128, WG_R = 32;

template <int DT>
struct WgLds {
    static constexpr int LDW = DT == DT_BF16 ? 20 : 36;   // dwords per LDS row (32 rows of the step + pad)
    static constexpr int GW = DT == DT_BF16 ? 2 : 4;      // dwords per 4-row group
};

__device__ __forceinline__ int wg_swz(int p) { return (p ^ (p >> 4)) & 7; }

template <int DT>
struct WgPatch {
    // 4 rows x 8 values as raw bits: bf16 in v[k][0], fp32 in v[k][0..1]
    u32x4 v[4][DT == DT_BF16 ? 1 : 2];
};

// PASS only separates the down and gate/up instantiations in profiles.
template <int DT, int PASS>
__global__ __launch_bounds__(BW_NT) void wgrad_kernel(const WgradArgs a, int64_t nlead, int64_t ntiles) {
    constexpr int LDW = WgLds<DT>::LDW, GW = WgLds<DT>::GW;
    __shared__ __align__(16) uint32_t lds[2][2][WG_T * LDW];   // [buffer][P, Q][value][row]
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wp = wid >> 1, wq = wid & 1;

    WgTile T;
    if (!wg_decode(a, nlead, ntiles, blockIdx.x, T)) return;
    const WgradProblem &P = T.pi ? a.p[1] : a.p[0];
    const int e = T.e, p0 = T.p0, qt0 = T.qt0, nq = T.nq;
    const int64_t rb = P.offsets ? (int64_t)P.offsets[e] : (int64_t)e * P.rows_fixed;
    const int64_t M = P.offsets ? (int64_t)P.offsets[e + 1] - rb : P.rows_fixed;
    const int nsteps = (int)((M + WG_R - 1) / WG_R);
    const int total = nq * nsteps;

    // output rows of this lane: p = p0 + wp*64 + j*16 + (lane&15); columns q = q0 + wq*64 + i*16 + 4*(lane>>4)
    const int split_rows = P.split < P.Pdim ? P.split : P.Pdim;
    auto store_tile = [&](int q0, const f32x4 (&acc)[4][4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p = p0 + wp * 64 + j * 16 + (lane & 15);
            void *out = p < P.split ? P.out0 : P.out1;
            const int prow = p < P.split ? p : p - P.split;
            const int64_t base = ((int64_t)e * split_rows + prow) * P.Qdim;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = q0 + wq * 64 + i * 16 + 4 * (lane >> 4);
                if (DT == DT_BF16) {
                    *(u32x2 *)((uint16_t *)out + base + q) =
                        u32x2{pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
                } else {
                    *(f32x4 *)((float *)out + base + q) = acc[i][j];
                }
            }
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
    if (total == 0) {   // an expert without rows: its gradient is zero
        for (int q = 0; q < nq; ++q) store_tile((qt0 + q) * WG_T, acc);
        return;
    }

    // staging role: threads 0..127 stage P, 128..255 stage Q; patch (rg, cg) = rows 4rg..4rg+3, values 8cg..8cg+7
    const int op = tid >> 7, pt = tid & 127, cg = pt & 15, rg = pt >> 4;
    auto load = [&](int it, WgPatch<DT> &x) {
        const int q0 = (qt0 + it / nsteps) * WG_T;
        const int64_t r0 = (int64_t)(it % nsteps) * WG_R + rg * 4;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t r = r0 + k;
            if (r < M) {
                const int64_t R = rb + r;
                const char *src;
                if (op == 0) {
                    src = (const char *)P.P + ((P.p_local ? r : R) * P.P_ld + p0 + cg * 8) * (DT == DT_BF16 ? 2 : 4);
                } else {
                    const int64_t QR = P.q_gather ? (int64_t)P.q_gather[R] : (P.q_local ? r : R);
                    src = (const char *)P.Q + (QR * P.Q_ld + q0 + cg * 8) * (DT == DT_BF16 ? 2 : 4);
                }
                x.v[k][0] = *(const u32x4 *)src;
                if (DT != DT_BF16) x.v[k][DT == DT_BF16 ? 0 : 1] = *(const u32x4 *)(src + 16);
            } else {
                x.v[k][0] = {};
                x.v[k][DT == DT_BF16 ? 0 : 1] = {};
            }
        }
    };
    auto stage = [&](int buf, const WgPatch<DT> &x) {
        uint32_t *dst = lds[buf][op];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int v = cg * 8 + c;
            uint32_t *d = dst + v * LDW + GW * (rg ^ wg_swz(v));
            if (DT == DT_BF16) {
                const int w = c >> 1;
                uint32_t r4[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) r4[k] = x.v[k][0][w];
                const uint32_t lo = (c & 1) ? ((r4[0] >> 16) | (r4[1] & 0xFFFF0000u))
                                            : ((r4[0] & 0xFFFFu) | (r4[1] << 16));
                const uint32_t hi = (c & 1) ? ((r4[2] >> 16) | (r4[3] & 0xFFFF0000u))
                                            : ((r4[2] & 0xFFFFu) | (r4[3] << 16));
                *(u32x2 *)d = u32x2{lo, hi};
            } else {
                uint32_t f4[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) f4[k] = x.v[k][(c >> 2) & (DT == DT_BF16 ? 0 : 1)][c & 3];
                *(u32x4 *)d = u32x4{f4[0], f4[1], f4[2], f4[3]};
            }
        }
    };
    auto compute = [&](int buf) {
        const uint32_t *Ps = lds[buf][0], *Qs = lds[buf][1];
        if (DT == DT_BF16) {
            // 16x16x32: lane supplies rows 8*(lane>>4) .. +7 = 4-row groups g0, g0 + 1
            const int g0 = 2 * (lane >> 4);
            bf16x8 qa[4], pb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int v = wq * 64 + i * 16 + (lane & 15);
                const uint32_t *row = Qs + v * LDW;
                const u32x2 x0 = *(const u32x2 *)(row + 2 * (g0 ^ wg_swz(v)));
                const u32x2 x1 = *(const u32x2 *)(row + 2 * ((g0 + 1) ^ wg_swz(v)));
                const u32x4 w = u32x4{x0[0], x0[1], x1[0], x1[1]};
                qa[i] = __builtin_bit_cast(bf16x8, w);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int v = wp * 64 + j * 16 + (lane & 15);
                const uint32_t *row = Ps + v * LDW;
                const u32x2 x0 = *(const u32x2 *)(row + 2 * (g0 ^ wg_swz(v)));
                const u32x2 x1 = *(const u32x2 *)(row + 2 * ((g0 + 1) ^ wg_swz(v)));
                const u32x4 w = u32x4{x0[0], x0[1], x1[0], x1[1]};
                pb[j] = __builtin_bit_cast(bf16x8, w);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[i], pb[j], acc[i][j], 0, 0, 0);
        } else {
            // 16x16x4 f32: k step g covers rows 4g .. 4g+3 (one group), lane supplies row 4g + (lane>>4)
#pragma unroll
            for (int g = 0; g < WG_R / 4; ++g) {
                float qa[4], pb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int v = wq * 64 + i * 16 + (lane & 15);
                    qa[i] = __uint_as_float(Qs[v * LDW + 4 * (g ^ wg_swz(v)) + (lane >> 4)]);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int v = wp * 64 + j * 16 + (lane & 15);
                    pb[j] = __uint_as_float(Ps[v * LDW + 4 * (g ^ wg_swz(v)) + (lane >> 4)]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i], pb[j], acc[i][j], 0, 0, 0);
            }
        }
    };

    WgPatch<DT> x;
    load(0, x);
    stage(0, x);
    __syncthreads();
    for (int it = 0; it < total; ++it) {
        const bool more = it + 1 < total;
        if (more) load(it + 1, x);
        compute(it & 1);
        if (it % nsteps == nsteps - 1) {
            store_tile((qt0 + it / nsteps) * WG_T, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
        }
        if (more) stage((it + 1) & 1, x);
        __syncthreads();
    }
}

// ---- bf16 weight gradient through an LDS ring --------------------------------
// One workgroup per (expert, 128-wide p tile); it walks every 128-wide q tile
// in 32-row reduction steps.  Four MFMA waves (2 x 2 of 64 x 64) and two
// producer waves.  The producers copy each step's operand rows into an LDS
// ring as they lie in memory ([row][value], 256 bytes per 128 values) with
// direct global->LDS loads, S steps ahead, and each waits only for its own loads;
// the MFMA waves never wait on the vector-memory counter, so their output
// stores stay in flight while later steps run.  The two roles run separate
// loops that meet at one barrier per step, which also keeps the compiler from
// guarding the MFMA waves' LDS reads against loads they never issue.
//
// MFMA fragments come from the LDS transpose read: in each group of 16 lanes,
// lane 4a+b receives value b of the 8-byte pieces addressed by lanes a, 4+a,
// 8+a and 12+a.  When lane 4j+a of group g addresses row kb + j at values
// c0 + 4a .. c0 + 4a + 3, lane L of the group receives rows kb .. kb+3 of
// value c0 + L: two such reads (kb = 8g, 8g + 4) give the eight consecutive
// rows a 16x16x32 operand lane holds.  The 16-byte chunks of a staged row sit
// in XOR-permuted slots (wgb_h) so that the 16 rows one read touches spread
// over all banks.  For a gathered Q operand the row indices of a step travel
// in the ring S - 1 steps ahead of their step, so the producer reads them from
// LDS instead of waiting on global memory.
// PW = 2: the p tile is 256 wide (two 128-value halves staged side by side, eight MFMA
// waves), which cuts the operand rows each output value costs by a quarter; it is used
// when every p dimension and split of the launch is a multiple of 256.
// Ring stages, and steps consumed per barrier (the rest of the ring is in flight): the
// 256-wide tile takes two 32-row steps per barrier from six stages, or four from eight
// when its P is resident and short enough; the 128-wide one a step per barrier from four.
// Each barrier costs about as much as a step's loads and products, so fewer is faster.
template <int PW> constexpr int wgb_s() { return PW == 2 ? 6 : 4; }
template <int PW> constexpr int wgb_sb() { return PW == 2 ? 2 : 1; }
constexpr int WGB_S4 = 8, WGB_SB4 = 4, WGB_NS4 = 5;   // eight stages, four per barrier: P of <= 5 steps
constexpr int WGB_PB = WG_R * WG_T * 2;                   // one operand half's rows of a step (8 KB)
constexpr int WGB_IDX = 256;                              // gather indices of a later step
template <int PW> constexpr int wgb_stage() { return (PW + 1) * WGB_PB + WGB_IDX; }
template <int PW> constexpr int wgb_lds() { return wgb_s<PW>() * wgb_stage<PW>(); }
template <int PW> constexpr int wgb_nt() { return 64 * (4 * PW + 2); }
// P-resident tiles (256-wide p tile only): an expert of at most WGB_NSR steps keeps its
// whole P operand in LDS, loaded once per workgroup, and only Q (plus gather indices)
// passes through the ring; a q tile then stages a third of the bytes.
constexpr int WGB_NSR = 6;
constexpr int WGB_QSTAGE = WGB_PB + WGB_IDX;
template <int PW> constexpr int wgb_res_lds() {
    return PW == 2 ? max(WGB_NSR * PW * WGB_PB + wgb_s<PW>() * WGB_QSTAGE, WGB_NS4 * PW * WGB_PB + WGB_S4 * WGB_QSTAGE) : 0;
}
template <int PW> constexpr int wgb_lds_all() { return wgb_lds<PW>() > wgb_res_lds<PW>() ? wgb_lds<PW>() : wgb_res_lds<PW>(); }

// slot permutation of a staged row's 16 chunks (an even XOR keeps chunk pairs together)
__device__ __forceinline__ int wgb_h(int k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }

typedef short wgb_v4s __attribute__((ext_vector_type(4)));
typedef short wgb_v8s __attribute__((ext_vector_type(8)));

__device__ __forceinline__ wgb_v4s lds_tr16(const char *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) wgb_v4s *)p);
}

// Four LDS words read in an asm block that also waits for them.
__device__ __forceinline__ void lds_u32_x4(uint32_t (&v)[4], uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
    asm volatile(
        "ds_read_b32 %0, %4\n"
        "ds_read_b32 %1, %5\n"
        "ds_read_b32 %2, %6\n"
        "ds_read_b32 %3, %7\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
        : "memory");
}

// PASS only separates the down and gate/up instantiations in profiles.
template <int PASS, int PW>
__global__ __launch_bounds__(wgb_nt<PW>()) void wgrad_bf16_kernel(const WgradArgs a, int64_t nlead, int64_t ntiles) {
    extern __shared__ __align__(1024) char wsm[];
    constexpr int STAGE = wgb_stage<PW>(), QB = PW * WGB_PB;   // Q rows follow the PW halves of P
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const bool producer = wid >= 4 * PW;
    const int wp = (wid >> 1) & (2 * PW - 1), wq = wid & 1;

    WgTile T;
    if (!wg_decode(a, nlead, ntiles, blockIdx.x, T)) return;
    const int pi = T.pi;
    // the problem's fields, read once (the asm blocks below clobber memory)
    const WgradProblem &Pr = pi ? a.p[1] : a.p[0];
    const uint16_t *const Pp = (const uint16_t *)Pr.P, *const Qp = (const uint16_t *)Pr.Q;
    const int64_t P_ld = Pr.P_ld, Q_ld = Pr.Q_ld;
    const int32_t *const qg = Pr.q_gather;
    const bool p_local = Pr.p_local != 0, q_local = Pr.q_local != 0;
    const int Pdim = Pr.Pdim, Qdim = Pr.Qdim, split = Pr.split;
    const int e = T.e, p0 = T.p0, qt0 = T.qt0, nq = T.nq;
    const int64_t rb = Pr.offsets ? (int64_t)Pr.offsets[e] : (int64_t)e * Pr.rows_fixed;
    const int M = (int)(Pr.offsets ? (int64_t)Pr.offsets[e + 1] - rb : Pr.rows_fixed);
    const int nsteps = (M + WG_R - 1) / WG_R;
    const int total = nq * nsteps;
    // LDS: P-resident, [P of steps 0 .. nsteps-1, PW halves each] then S stages of
    // [Q | gather indices]; otherwise S stages of [P halves | Q | gather indices]
    const bool res = PW == 2 && nsteps <= WGB_NSR;
    const bool four = res && nsteps <= WGB_NS4;
    const int ring_s = four ? WGB_S4 : wgb_s<PW>(), SB = four ? WGB_SB4 : wgb_sb<PW>();   // stages, steps per barrier
    const int D = ring_s - SB;                                   // steps in flight past the ones consumed
    const int qa0 = res ? nsteps * PW * WGB_PB : QB;   // Q of stage 0
    const int qss = res ? WGB_QSTAGE : STAGE;           // Q stage stride

    if (producer) {
        if (total == 0) return;
        // instruction n (0..7) of an operand covers rows 4n .. 4n+3 of the step; producer k issues
        // n = 2m + k.  This lane: row 4n + lane/16, chunk slot lane%16 holding data chunk
        // (lane%16) ^ h(row).  Row pointers are formed once and advanced by a uniform offset per step.
        const int k = wid - 4 * PW, drow = lane >> 4, pchunk = lane & 15;
        const bool gather = qg != nullptr;
        const int32_t *const qgb = gather ? qg + rb : nullptr;
        const int64_t prb = p_local ? 0 : rb, qrb = q_local ? 0 : rb;
        int cofs[4];
        const uint16_t *pbase[4], *qbase[4], *plast[4], *qlast[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int n = 2 * m + k, kr = 4 * n + drow;
            cofs[m] = 8 * (pchunk ^ wgb_h(kr));
            pbase[m] = Pp + (prb + kr) * P_ld + p0 + cofs[m];
            qbase[m] = Qp + (qrb + kr) * Q_ld + cofs[m];
            plast[m] = Pp + (prb + M - 1) * P_ld + p0 + cofs[m];   // rows past the expert repeat its last
            qlast[m] = Qp + (qrb + M - 1) * Q_ld + cofs[m];
        }
        auto nops = [&](int y) { return 4 * (res ? 1 : PW + 1) + ((k == 0 && gather && y + D < total) ? 1 : 0); };
        int yq = 0, ys = 0;   // q tile and step of the next step to issue
        // step y into ring slot y % S; qrow: gathered Q rows of this lane's 4 rows (if gather)
        auto issue = [&](int y, const int (&qrow)[4]) {
            char *slot = wsm + (y % ring_s) * STAGE;
            char *qslot = wsm + qa0 + (y % ring_s) * qss;
            const int q0 = (qt0 + yq) * WG_T, r0 = ys * WG_R;
            const bool ragged = r0 + WG_R > M;
            const int64_t po = (int64_t)r0 * P_ld, qo = (int64_t)r0 * Q_ld + q0;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int n = 2 * m + k;
                const bool past = ragged && r0 + 4 * n + drow >= M;
                if (!res)
#pragma unroll
                    for (int h = 0; h < PW; ++h)
                        dma16((past ? plast[m] : pbase[m] + po) + h * WG_T, slot + h * WGB_PB + n * 1024);
                const uint16_t *qs;
                if (gather) qs = Qp + (int64_t)qrow[m] * Q_ld + q0 + cofs[m];
                else qs = past ? qlast[m] + q0 : qbase[m] + qo;
                dma16(qs, qslot + n * 1024);
            }
            if (k == 0 && gather && y + D < total) {
                // row indices of step y + D ride along (64 words, the first 32 used)
                const int ys2 = (ys + D) % nsteps;
                dma4(qgb + min(ys2 * WG_R + (lane & 31), M - 1), qslot + WGB_PB);
            }
            if (++ys == nsteps) { ys = 0; ++yq; }
        };
        if (res) {
            // the expert's whole P operand, ahead of every Q step (older in the memory counter)
            for (int st = 0; st < nsteps; ++st) {
                const int r0 = st * WG_R;
                const bool ragged = r0 + WG_R > M;
                const int64_t po = (int64_t)r0 * P_ld;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int n = 2 * m + k;
                    const bool past = ragged && r0 + 4 * n + drow >= M;
#pragma unroll
                    for (int h = 0; h < PW; ++h)
                        dma16((past ? plast[m] : pbase[m] + po) + h * WG_T, wsm + (st * PW + h) * WGB_PB + n * 1024);
                }
            }
        }
        int qrow[4] = {0, 0, 0, 0};
        for (int y = 0; y < D && y < total; ++y) {
            if (gather)
#pragma unroll
                for (int m = 0; m < 4; ++m) qrow[m] = qgb[min(ys * WG_R + 4 * (2 * m + k) + drow, M - 1)];
            issue(y, qrow);
        }
        for (int x = 0; x < total; x += SB) {
            // steps x .. x+SB-1 have landed once at most the later steps' loads are outstanding
            int after = 0;
            for (int y = x + SB; y <= min(x + D - 1, total - 1); ++y) after += nops(y);
            wait_vmcnt_dyn(after);
            cta_barrier();   // steps x .. x+SB-1 landed; every MFMA wave is done with the slots of x-SB .. x-1
            for (int j = 0; j < SB; ++j) {
                const int y = x + D + j;   // into the slot of step x - SB + j
                if (y < total) {
                    if (gather) {
                        const uint32_t ib = (uint32_t)(uintptr_t)(wsm + qa0 + ((x + j) % ring_s) * qss + WGB_PB);
                        uint32_t v[4];
                        lds_u32_x4(v, ib + 4 * (4 * k + drow), ib + 4 * (4 * (2 + k) + drow),
                                   ib + 4 * (4 * (4 + k) + drow), ib + 4 * (4 * (6 + k) + drow));
#pragma unroll
                        for (int m = 0; m < 4; ++m) qrow[m] = (int)v[m];
                    }
                    issue(y, qrow);
                }
            }
        }
        return;
    }

    // ---- MFMA waves ----
    const int split_rows = split < Pdim ? split : Pdim;   // a p tile lies on one side of the split
    uint16_t *const out = (uint16_t *)(p0 < split ? Pr.out0 : Pr.out1);
    const int prow0 = p0 < split ? p0 : p0 - split;
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
    // output rows of this lane: p = p0 + wp*64 + j*16 + (lane&15); columns q = q0 + wq*64 + i*16 + 4*(lane>>4)
    // (pairs of 16-column blocks leave as one 16-byte store per lane: 128 bytes of a row per 8 lanes)
    auto store_tile = [&](int q0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int prow = prow0 + wp * 64 + j * 16 + (lane & 15);
            uint16_t *orow = out + ((int64_t)e * split_rows + prow) * Qdim;
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const float ya[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                const float yb[4] = {acc[i + 1][j][0], acc[i + 1][j][1], acc[i + 1][j][2], acc[i + 1][j][3]};
                store_pair_bf16(orow, q0 + wq * 64 + i * 16, ya, yb, lane, Qdim);
            }
        }
    };
    if (total == 0) {   // an expert without rows: its gradient is zero
        for (int q = 0; q < nq; ++q) store_tile((qt0 + q) * WG_T);
        return;
    }
    // per-lane byte offsets (in a stage) of the fragment reads: rows 8g + jj and 8g + 4 + jj
    // of values col0 + 4aa .. +3, for the 4 Q and 4 P fragments of this wave
    const int g = lane >> 4, jj = (lane >> 2) & 3, aa = lane & 3;
    int ofs[16];
#pragma unroll
    for (int f = 0; f < 8; ++f) {
        // P values of this wave: half wp / 2 of the staged p tile, columns (wp % 2) * 64 ..
        const int col0 = f < 4 ? wq * 64 + f * 16 : (wp & 1) * 64 + (f - 4) * 16;
        const int c = (col0 + 4 * aa) >> 3, off = 8 * (aa & 1);
        const int k0 = 8 * g + jj, k1 = k0 + 4;
        const int base = f < 4 ? 0 : (wp >> 1) * WGB_PB;
        ofs[2 * f] = base + k0 * 256 + ((c ^ wgb_h(k0)) << 4) + off;
        ofs[2 * f + 1] = base + k1 * 256 + ((c ^ wgb_h(k1)) << 4) + off;
    }
    const int vlast = M - (nsteps - 1) * WG_R;   // valid rows of an expert's last step
    // A q tile's results leave during the next q tile's steps, two 16-byte stores per
    // lane per step (packed to bf16 when the tile ends), instead of as one burst that
    // the ring's next loads queue behind: pv holds them, pn counts those already out.
    u32x4 pv[8];
    int pq0 = 0, pn = 8;
    auto pack_tile = [&](int q0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const float ya[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                const float yb[4] = {acc[i + 1][j][0], acc[i + 1][j][1], acc[i + 1][j][2], acc[i + 1][j][3]};
                pv[j * 2 + i / 2] = pair_bf16_value(ya, yb, lane);
            }
        pq0 = q0;
        pn = 0;
    };
    // pv[2j] and pv[2j+1] hold the wave's 64 columns of row block j for the lane's row; the
    // lanes of rows r and r ^ 8 swap halves so that each of the two 16-byte stores writes
    // 128 contiguous bytes of 8 rows (64 bytes of 16 rows before)
    auto store_pair = [&](int j) {
        const bool hi = (lane >> 3) & 1;
        const u32x4 send = hi ? pv[2 * j] : pv[2 * j + 1];
        u32x4 recv;
#pragma unroll
        for (int k = 0; k < 4; ++k) recv[k] = (uint32_t)__shfl_xor((int)send[k], 8, 64);
        const u32x4 va = hi ? recv : pv[2 * j], vb = hi ? pv[2 * j + 1] : recv;
        const int rbase = prow0 + wp * 64 + j * 16 + (lane & 7);
        uint16_t *ra = out + ((int64_t)e * split_rows + rbase) * Qdim;
        uint16_t *rb = ra + 8 * (int64_t)Qdim;
        const int f = pair_bf16_col(pq0 + wq * 64 + (hi ? 32 : 0), lane);
        if (f < Qdim) {
            *(u32x4 *)(ra + f) = va;
            *(u32x4 *)(rb + f) = vb;
        }
    };
    auto store_some = [&](int upto) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (2 * j >= pn && 2 * j < upto) store_pair(j);
        pn = upto > pn ? upto : pn;
    };
    int qt = 0, st = 0, slot = 0, sbn = 0;
    for (int x = 0; x < total; ++x) {
        if (sbn == 0) cta_barrier();             // steps x .. x+SB-1 have landed
        sbn = sbn + 1 == SB ? 0 : sbn + 1;
        const char *qsb = wsm + qa0 + slot * qss;
        const char *psb = res ? wsm + st * (PW * WGB_PB) : wsm + slot * STAGE;
        wgb_v4s r[16];
#pragma unroll
        for (int f = 0; f < 16; ++f) r[f] = lds_tr16((f < 8 ? qsb : psb) + ofs[f]);
        bf16x8 qa[4], pb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            qa[i] = __builtin_bit_cast(bf16x8, (wgb_v8s)__builtin_shufflevector(r[2 * i], r[2 * i + 1], 0, 1, 2, 3,
                                                                                 4, 5, 6, 7));
        const bool ragged = st == nsteps - 1 && vlast < WG_R;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            wgb_v8s v = __builtin_shufflevector(r[8 + 2 * j], r[8 + 2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
            if (ragged) {
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    if (8 * g + q >= vlast) v[q] = 0;
            }
            pb[j] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[i], pb[j], acc[i][j], 0, 0, 0);
        slot = slot + 1 == ring_s ? 0 : slot + 1;
        if (pn < 8) store_some(pn + 2 < 8 ? pn + 2 : 8);
        if (++st == nsteps) {
            store_some(8);
            pack_tile((qt0 + qt) * WG_T);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
            st = 0;
            ++qt;
        }
    }
    store_some(8);
}

// ---- FP8 backward helpers ------------------------------------------------------
// Block-scale grids of transposed weights: dst[m][c][col0 + r] = src[m][r][c].
__global__ __launch_bounds__(256) void scale_transpose_kernel(const float *__restrict__ src, int64_t nmat, int rows,
                                                              int cols, float *__restrict__ dst, int dst_ld,
                                                              int col0) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nmat * rows * (int64_t)cols) return;
    const int64_t m = i / ((int64_t)rows * cols);
    const int rc = (int)(i - m * rows * (int64_t)cols), r = rc / cols, c = rc - r * cols;
    dst[(m * cols + c) * dst_ld + col0 + r] = src[i];
}

// bbase[e] = sum over e' < e of ceil(len(e') / 128): the first 128-row run of expert e
// among all experts' runs (bbase[n] = the total).
__global__ void block_base_kernel(const int32_t *__restrict__ offsets, int n, int32_t *__restrict__ bbase) {
    if (threadIdx.x != 0) return;
    int32_t acc = 0;
    for (int e = 0; e < n; ++e) {
        bbase[e] = acc;
        acc += (offsets[e + 1] - offsets[e] + 127) / 128;
    }
    bbase[n] = acc;
}

// 128 x 1 tiles along the rows of segments (the FP8 weight-gradient operands):
// workgroup (b, chunk) takes 128-row run b and 2048 columns, eight adjacent
// columns per thread (16-byte bf16 or 8-byte e4m3 loads, four rows in flight).
// Segment e owns rows offsets[e] .. offsets[e+1] (or e*seg_rows .. +seg_rows);
// its runs start at its first row and are numbered from bbase[e] (or
// e*ceil(seg_rows/128)).  List row r reads source row gather[r] (or r), bf16, or
// e4m3 with 1 x 128 scales (decoded to fp32 first).  Scale = amax / 448 (1 for an
// all-zero column), codes = e4m3(clamp(v / scale)), nearest even.  The run is read
// once: a workgroup keeps its 128 rows x 128 columns in registers.
constexpr int QC_COLS = 8;                  // columns per thread
constexpr int QC_CHUNK = 16 * QC_COLS;      // columns per workgroup (16 threads per row, 16 row groups)
template <int IN>
__global__ __launch_bounds__(256) void quant_cols_kernel(const void *__restrict__ src, const float *__restrict__ src_s,
                                                         const int32_t *__restrict__ gather,
                                                         const int32_t *__restrict__ offsets,
                                                         const int32_t *__restrict__ bbase, int64_t seg_rows,
                                                         int n_seg, int cols, uint8_t *__restrict__ q,
                                                         float *__restrict__ sc) {
    const int64_t b = blockIdx.x;
    int64_t r0, r1;
    if (offsets) {
        if (b >= bbase[n_seg]) return;
        int lo = 0, hi = n_seg - 1;   // the segment whose runs include b
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (bbase[mid] <= b) lo = mid;
            else hi = mid - 1;
        }
        r0 = offsets[lo] + (b - bbase[lo]) * 128;
        r1 = min(r0 + 128, (int64_t)offsets[lo + 1]);
    } else {
        const int64_t nbs = (seg_rows + 127) / 128;
        if (b >= n_seg * nbs) return;
        const int64_t e = b / nbs, j = b - e * nbs;
        r0 = e * seg_rows + j * 128;
        r1 = min(r0 + 128, (e + 1) * seg_rows);
    }
    // one pass: thread (g, t) = (threadIdx.x / 16, threadIdx.x % 16) holds rows r0 + 8g .. r0 + 8g + 7
    // of columns c .. c + 7 in registers; the run's column maxima are combined across the
    // 16 row groups (shuffles inside a wave, then LDS across the four waves)
    __shared__ float red[4][16][QC_COLS];
    const int t = threadIdx.x & 15, g = threadIdx.x >> 4, wv = threadIdx.x >> 6;
    const int c = blockIdx.y * QC_CHUNK + t * QC_COLS;
    auto load = [&](int64_t r, float (&v)[QC_COLS]) {
        const int64_t xr = gather ? (int64_t)gather[r] : r;
        if (IN == DT_E4M3) {
            const u32x2 w = *(const u32x2 *)((const uint8_t *)src + xr * cols + c);
            const float s = src_s[xr * (cols / 128) + c / 128];
#pragma unroll
            for (int k = 0; k < QC_COLS; ++k)
                v[k] = __builtin_amdgcn_cvt_f32_fp8((int)((w[k >> 2] >> (8 * (k & 3))) & 0xFF), 0) * s;
        } else {
            const u32x4 w = *(const u32x4 *)((const uint16_t *)src + xr * cols + c);
#pragma unroll
            for (int k = 0; k < QC_COLS; k += 2) {
                v[k] = __uint_as_float(w[k >> 1] << 16);
                v[k + 1] = __uint_as_float(w[k >> 1] & 0xFFFF0000u);
            }
        }
    };
    float v[8][QC_COLS];
    float amax[QC_COLS];
#pragma unroll
    for (int k = 0; k < QC_COLS; ++k) amax[k] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t r = r0 + 8 * g + i;
        load(min(r, r1 - 1), v[i]);   // rows past the run repeat its last (no effect on the maxima)
#pragma unroll
        for (int k = 0; k < QC_COLS; ++k) amax[k] = fmaxf(amax[k], fabsf(v[i][k]));
    }
#pragma unroll
    for (int k = 0; k < QC_COLS; ++k) {
        amax[k] = fmaxf(amax[k], __shfl_xor(amax[k], 16, 64));
        amax[k] = fmaxf(amax[k], __shfl_xor(amax[k], 32, 64));
    }
    if ((threadIdx.x & 63) < 16)
#pragma unroll
        for (int k = 0; k < QC_COLS; ++k) red[wv][t][k] = amax[k];
    __syncthreads();
    float scale[QC_COLS];
#pragma unroll
    for (int k = 0; k < QC_COLS; ++k)
        scale[k] = quant_scale(fmaxf(fmaxf(red[0][t][k], red[1][t][k]), fmaxf(red[2][t][k], red[3][t][k])));
    if (g == 0) {
        *(f32x4 *)(sc + b * cols + c) = f32x4{scale[0], scale[1], scale[2], scale[3]};
        *(f32x4 *)(sc + b * cols + c + 4) = f32x4{scale[4], scale[5], scale[6], scale[7]};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t r = r0 + 8 * g + i;
        if (r >= r1) break;
        u32x2 o;
#pragma unroll
        for (int h = 0; h < 2; ++h)
            o[h] = pack_e4m3x4(clamp448(v[i][4 * h] / scale[4 * h]), clamp448(v[i][4 * h + 1] / scale[4 * h + 1]),
                               clamp448(v[i][4 * h + 2] / scale[4 * h + 2]), clamp448(v[i][4 * h + 3] / scale[4 * h + 3]));
        *(u32x2 *)(q + r * cols + c) = o;
    }
}

// ---- FP8 weight gradient -----------------------------------------------------------
// C[p][q] = sum over an expert's 128-row runs of (sum_r Pq[r][p] Qq[r][q]) * sP[run][p] * sQ[run][q],
// with both operands in 128 x 1 tiles along the rows (codes Pq, Qq, scales sP, sQ).  The
// structure is the bf16 kernel's: one workgroup per (expert, 128-wide p tile, q group),
// two producer waves filling an LDS ring with direct loads, four MFMA waves.  A step is
// one 128-row run, i.e. one 16x16x128 e4m3 MFMA per 16 x 16 output block; its fp32
// partial is scaled by the run's two column scales and added.  Fragments come from the
// 8-bit LDS transpose read: in each 16-lane group, lane 8a+b receives byte b of the
// 8-byte pieces addressed by lanes 2j+a (j = 0..7); four reads give a lane the 32
// consecutive rows of its operand.  Staged rows are 128 bytes; their 16-byte chunks sit
// in slots XOR-permuted by wf8_h so the 32 rows of one read spread over all banks.
// ring stages: two (two workgroups per CU), three for the 256-wide tile (one per CU)
template <int PW> constexpr int wf8_s() { return PW == 2 ? 3 : 2; }
constexpr int WF8_R = 128;                                 // rows per step (one quantisation run)
constexpr int WF8_PB = WF8_R * WG_T;                       // one operand's codes of a step (16 KB)
// PW = 2: 256-wide p tiles as in the bf16 kernel (two staged halves, eight MFMA waves).
// Scale area per stage: [P half 0 | Q | P half 1 | unused], 512 bytes each.
template <int PW> constexpr int wf8_stage() { return (PW + 1) * WF8_PB + PW * 2 * WG_T * 4; }
template <int PW> constexpr int wf8_lds() { return wf8_s<PW>() * wf8_stage<PW>(); }
template <int PW> constexpr int wf8_nt() { return 64 * (4 * PW + 2); }

__device__ __forceinline__ int wf8_h(int r) { return ((r >> 1) & 3) | (((r >> 5) & 1) << 2); }

typedef int wf8_v2i __attribute__((ext_vector_type(2)));

__device__ __forceinline__ wf8_v2i lds_tr8(const char *p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) wf8_v2i *)p);
}

template <int PASS, int PW>
__global__ __launch_bounds__(wf8_nt<PW>(), 3) void wgrad_fp8_kernel(const WgradArgs a, int64_t nlead, int64_t ntiles) {
    extern __shared__ __align__(1024) char wsm[];
    constexpr int STAGE = wf8_stage<PW>(), QB = PW * WF8_PB, SB = (PW + 1) * WF8_PB;   // Q codes, scales
    constexpr int WF8_S = wf8_s<PW>();
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const bool producer = wid >= 4 * PW;
    const int wp = (wid >> 1) & (2 * PW - 1), wq = wid & 1;
    WgTile T;
    if (!wg_decode(a, nlead, ntiles, blockIdx.x, T)) return;
    const WgradProblem &Pr = T.pi ? a.p[1] : a.p[0];
    const uint8_t *const Pp = (const uint8_t *)Pr.P, *const Qp = (const uint8_t *)Pr.Q;
    const float *const Ps = Pr.Ps, *const Qs = Pr.Qs;
    const int64_t P_ld = Pr.P_ld, Q_ld = Pr.Q_ld;
    const bool p_local = Pr.p_local != 0, q_local = Pr.q_local != 0;
    const int Pdim = Pr.Pdim, Qdim = Pr.Qdim, split = Pr.split;
    const int e = T.e, p0 = T.p0, qt0 = T.qt0, nq = T.nq;
    const int64_t rb = Pr.offsets ? (int64_t)Pr.offsets[e] : (int64_t)e * Pr.rows_fixed;
    const int M = (int)(Pr.offsets ? (int64_t)Pr.offsets[e + 1] - rb : Pr.rows_fixed);
    const int nsteps = (M + WF8_R - 1) / WF8_R;
    const int total = nq * nsteps;
    // first 128-row run of this expert among the operand's runs
    const int64_t bb = Pr.offsets ? (int64_t)Pr.bbase[e] : (int64_t)e * ((Pr.rows_fixed + 127) / 128);
    const int64_t pbb = p_local ? 0 : bb, qbb = q_local ? 0 : bb;

    if (producer) {
        if (total == 0) return;
        // instruction n (0..15) of an operand covers rows 8n .. 8n+7 of the step; producer k
        // issues n = 2m + k.  This lane: row 8n + lane/8, slot lane%8 holding data chunk
        // (lane%8) ^ h(row).  The run's scales: lanes 0-31 take P's 128, lanes 32-63 Q's.
        const int k = wid - 4 * PW, drow = lane >> 3, pchunk = lane & 7;
        const int64_t prb = p_local ? 0 : rb, qrb = q_local ? 0 : rb;
        int yq = 0, ys = 0;
        auto issue = [&](int y) {
            char *slot = wsm + (y % WF8_S) * STAGE;
            const int q0 = (qt0 + yq) * WG_T, r0 = ys * WF8_R;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int n = 2 * m + k, kr = 8 * n + drow;
                const int r = min(r0 + kr, M - 1);   // rows past the expert repeat its last (masked)
                const int cofs = 16 * (pchunk ^ wf8_h(kr));
#pragma unroll
                for (int h = 0; h < PW; ++h) dma16(Pp + (prb + r) * P_ld + p0 + h * WG_T + cofs, slot + h * WF8_PB + n * 1024);
                dma16(Qp + (qrb + r) * Q_ld + q0 + cofs, slot + QB + n * 1024);
            }
            if (k == 0) {
                const float *src = lane < 32 ? Ps + (pbb + ys) * Pdim + p0 + 4 * lane
                                             : Qs + (qbb + ys) * Qdim + q0 + 4 * (lane - 32);
                dma16(src, slot + SB);
            } else if (PW == 2) {
                // P half 1's scales (the upper lanes repeat them into the unused quarter)
                dma16(Ps + (pbb + ys) * Pdim + p0 + WG_T + 4 * (lane & 31), slot + SB + 2 * WG_T * 4);
            }
            if (++ys == nsteps) { ys = 0; ++yq; }
        };
        const int nops = 8 * (PW + 1) + ((k == 0 || PW == 2) ? 1 : 0);
        for (int y = 0; y < WF8_S - 1 && y < total; ++y) issue(y);
        for (int x = 0; x < total; ++x) {
            wait_vmcnt_dyn(nops * (min(x + WF8_S - 2, total - 1) - x));
            cta_barrier();
            if (x + WF8_S - 1 < total) issue(x + WF8_S - 1);
        }
        return;
    }

    const int split_rows = split < Pdim ? split : Pdim;
    uint16_t *const out = (uint16_t *)(p0 < split ? Pr.out0 : Pr.out1);
    const int prow0 = p0 < split ? p0 : p0 - split;
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
    auto store_tile = [&](int q0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int prow = prow0 + wp * 64 + j * 16 + (lane & 15);
            uint16_t *orow = out + ((int64_t)e * split_rows + prow) * Qdim;
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const float ya[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                const float yb[4] = {acc[i + 1][j][0], acc[i + 1][j][1], acc[i + 1][j][2], acc[i + 1][j][3]};
                store_pair_bf16(orow, q0 + wq * 64 + i * 16, ya, yb, lane, Qdim);
            }
        }
    };
    if (total == 0) {
        for (int q = 0; q < nq; ++q) store_tile((qt0 + q) * WG_T);
        return;
    }
    // fragment reads: lane (group g, L = 2jj + aa) addresses row 32g + 8t + jj, bytes col0 + 8aa .. +7
    const int g = lane >> 4, jj = (lane & 15) >> 1, aa = lane & 1;
    // wf8_h(r) reads row bits 1, 2 and 5, which the read index t (rows 8t apart) leaves
    // alone: one offset per fragment, the four reads 8 rows (1 KB) apart
    int ofs[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) {
        // P values of this wave: half wp / 2 of the staged p tile, columns (wp % 2) * 64 ..
        const int col0 = f < 4 ? wq * 64 + f * 16 : (wp & 1) * 64 + (f - 4) * 16;
        const int base = f < 4 ? QB : (wp >> 1) * WF8_PB;
        const int r = 32 * g + jj;
        ofs[f] = base + r * WG_T + (((col0 >> 4) ^ wf8_h(r)) << 4) + 8 * aa;
    }
    const int vlast = M - (nsteps - 1) * WF8_R;
    int qt = 0, st = 0, slot = 0;
    for (int x = 0; x < total; ++x) {
        cta_barrier();
        const char *sb = wsm + slot * STAGE;
        auto frag = [&](int f) {
            wf8_v2i v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = lds_tr8(sb + ofs[f] + 8 * t * WG_T);
            return i32x8{v[0][0], v[0][1], v[1][0], v[1][1], v[2][0], v[2][1], v[3][0], v[3][1]};
        };
        // P fragments for the whole step, Q fragments one at a time below
        i32x8 fp[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) fp[j] = frag(4 + j);
        if (st == nsteps - 1 && vlast < WF8_R) {
            // rows past the expert: zero P's bytes (lane holds rows 32g .. 32g+31, low byte first)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    const int r = 32 * g + 4 * w;
                    uint32_t m = 0;
#pragma unroll
                    for (int bt = 0; bt < 4; ++bt)
                        if (r + bt < vlast) m |= 0xFFu << (8 * bt);
                    fp[j][w] &= (int)m;
                }
        }
        // scales: [P half 0 | Q | P half 1 | unused], 128 floats each
        const float *scq = (const float *)(sb + SB) + WG_T, *scp = (const float *)(sb + SB) + 2 * WG_T * (wp >> 1);
        float sp[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sp[j] = scp[(wp & 1) * 64 + j * 16 + (lane & 15)];
        // one row of four products at a time, then its scaling: four partial sums live
        // instead of sixteen, which keeps the kernel at three waves per SIMD
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const i32x8 fq = frag(i);
            f32x4 part[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) part[j] = FTraits<DT_E4M3>::mma(fq, fp[j], f32x4{0, 0, 0, 0});
            const f32x4 sq = *(const f32x4 *)(scq + wq * 64 + i * 16 + 4 * (lane >> 4));
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[i][j][v] += part[j][v] * (sq[v] * sp[j]);
        }
        slot = slot + 1 == WF8_S ? 0 : slot + 1;
        if (++st == nsteps) {
            store_tile((qt0 + qt) * WG_T);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
            st = 0;
            ++qt;
        }
    }
}

}  // namespace

hipError_t launch_transpose(int dt, const void *src, int64_t nmat, int rows, int cols, void *dst, int dst_ld, int col0,
                            hipStream_t s) {
    const int64_t blocks = nmat * (rows / 64) * (int64_t)(cols / 64);
    if (blocks <= 0) return hipSuccess;
    if (dt == DT_F32)
        transpose_kernel<4><<<(unsigned)blocks, 256, 0, s>>>((const char *)src, rows, cols, (char *)dst, dst_ld, col0);
    else if (dt == DT_BF16)
        transpose_kernel<2><<<(unsigned)blocks, 256, 0, s>>>((const char *)src, rows, cols, (char *)dst, dst_ld, col0);
    else
        transpose_kernel<1><<<(unsigned)blocks, 256, 0, s>>>((const char *)src, rows, cols, (char *)dst, dst_ld, col0);
    return hipGetLastError();
}

hipError_t launch_transpose_scales(const float *src, int64_t nmat, int rows, int cols, float *dst, int dst_ld, int col0,
                                   hipStream_t s) {
    const int64_t n = nmat * rows * (int64_t)cols;
    if (n <= 0) return hipSuccess;
    scale_transpose_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(src, nmat, rows, cols, dst, dst_ld, col0);
    return hipGetLastError();
}

hipError_t launch_block_base(const int32_t *offsets, int n, int32_t *bbase, hipStream_t s) {
    block_base_kernel<<<1, 64, 0, s>>>(offsets, n, bbase);
    return hipGetLastError();
}

hipError_t launch_quant_cols(int in_dt, const void *src, const float *src_s, const int32_t *gather,
                             const int32_t *offsets, const int32_t *bbase, int64_t seg_rows, int n_seg, int64_t max_blocks,
                             int cols, uint8_t *q, float *sc, hipStream_t s) {
    if (max_blocks <= 0 || n_seg <= 0) return hipSuccess;
    if (max_blocks >= (1ll << 31)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)max_blocks, (unsigned)((cols + QC_CHUNK - 1) / QC_CHUNK));
    if (in_dt == DT_E4M3)
        quant_cols_kernel<DT_E4M3><<<grid, 256, 0, s>>>(src, src_s, gather, offsets, bbase, seg_rows, n_seg, cols, q,
                                                        sc);
    else
        quant_cols_kernel<DT_BF16><<<grid, 256, 0, s>>>(src, src_s, gather, offsets, bbase, seg_rows, n_seg, cols, q,
                                                        sc);
    return hipGetLastError();
}

hipError_t launch_bwd_combine(int dt, const void *dout, const void *y, const int32_t *inv, const float *topk_w, int64_t T,
                              int d, int K, void *dy, float *dg, uint8_t *dyq, float *dys, uint8_t *doq, float *dos,
                              hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (dyq && (dt != DT_BF16 || d % 128)) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)(T < (1 << 20) ? T : (1 << 20));
#define BC(DT, KM, Q)                                                                                                \
    bwd_combine_kernel<DT, KM, Q><<<grid, BW_NT, 0, s>>>(dout, y, inv, topk_w, T, d, K, dy, dg, dyq, dys, doq, dos)
    if (dt == DT_F32) { if (K <= 8) BC(DT_F32, 8, false); else BC(DT_F32, 32, false); }
    else if (dyq) { if (K <= 8) BC(DT_BF16, 8, true); else BC(DT_BF16, 32, true); }
    else { if (K <= 8) BC(DT_BF16, 8, false); else BC(DT_BF16, 32, false); }
#undef BC
    return hipGetLastError();
}

hipError_t launch_bwd_token(int dt, const void *dxr, const void *dxs, int Ns, const int32_t *inv, const int32_t *idx,
                            const float *scores, const float *dg, const void *gate_w, int64_t T, int d, int Nr, int K,
                            float rs, void *du, float *dz_row, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const unsigned grid = (unsigned)(T < (1 << 20) ? T : (1 << 20));
#define BT(DT, KM)                                                                                                     \
    bwd_token_kernel<DT, KM><<<grid, BW_NT, 0, s>>>(dxr, dxs, Ns, inv, idx, scores, dg, gate_w, T, d, Nr, K, rs, du, \
                                                    dz_row)
    if (dt == DT_F32) { if (K <= 8) BT(DT_F32, 8); else BT(DT_F32, 32); }
    else { if (K <= 8) BT(DT_BF16, 8); else BT(DT_BF16, 32); }
#undef BT
    return hipGetLastError();
}

hipError_t launch_dgate(int dt, const void *u, const int32_t *perm, const int32_t *offsets, const float *dz_row, int Nr,
                        int d, float *dgate, hipStream_t s) {
    const int chunks = (d / 8 + BW_NT - 1) / BW_NT;
    if (dt == DT_F32)
        dgate_kernel<DT_F32><<<(unsigned)(Nr * chunks), BW_NT, 0, s>>>(u, perm, offsets, dz_row, d, chunks, dgate);
    else
        dgate_kernel<DT_BF16><<<(unsigned)(Nr * chunks), BW_NT, 0, s>>>(u, perm, offsets, dz_row, d, chunks, dgate);
    return hipGetLastError();
}

hipError_t launch_wgrad(int dt, int pass, const WgradArgs &args, hipStream_t s) {
    WgradArgs a = args;
    for (int i = 0; i < a.nprob; ++i) {
        a.p[i].step_rows = dt == DT_E4M3 ? WF8_R : 32;
        a.p[i].p_tile = 128;
    }
    int64_t tiles = 0;
    for (int i = 0; i < a.nprob; ++i) tiles += wg_tiles(a.p[i]);
    if (tiles <= 0) return hipSuccess;
    // a leading fixed-rows problem is spread over all XCDs (see wg_decode)
    int64_t nlead = (a.nprob > 1 && !a.p[0].offsets) ? wg_tiles(a.p[0]) : 0;
    int64_t grid = (nlead + 7) / 8 * 8 + (tiles - nlead + 7) / 8 * 8;
    if (grid >= (1ll << 31)) return hipErrorInvalidValue;
    if (dt == DT_F32) {
        if (pass) wgrad_kernel<DT_F32, 1><<<(unsigned)grid, BW_NT, 0, s>>>(a, nlead, tiles);
        else wgrad_kernel<DT_F32, 0><<<(unsigned)grid, BW_NT, 0, s>>>(a, nlead, tiles);
    } else if (dt == DT_E4M3) {
        // the 256-wide p tile needs every p dimension and split of the launch on 256-value boundaries
        bool wide = true;
        for (int i = 0; i < a.nprob; ++i) wide = wide && a.p[i].Pdim % 256 == 0 && a.p[i].split % 256 == 0;
        if (wide) {
            for (int i = 0; i < a.nprob; ++i) a.p[i].p_tile = 256;
            tiles = 0;
            for (int i = 0; i < a.nprob; ++i) tiles += wg_tiles(a.p[i]);
            nlead = (a.nprob > 1 && !a.p[0].offsets) ? wg_tiles(a.p[0]) : 0;
            grid = (nlead + 7) / 8 * 8 + (tiles - nlead + 7) / 8 * 8;
        }
        static std::once_flag once8;
        static hipError_t attr8 = hipSuccess;
        std::call_once(once8, [] {
            const void *k[4] = {(const void *)wgrad_fp8_kernel<0, 1>, (const void *)wgrad_fp8_kernel<1, 1>,
                                (const void *)wgrad_fp8_kernel<0, 2>, (const void *)wgrad_fp8_kernel<1, 2>};
            const int lds[4] = {wf8_lds<1>(), wf8_lds<1>(), wf8_lds<2>(), wf8_lds<2>()};
            for (int i = 0; i < 4 && attr8 == hipSuccess; ++i)
                attr8 = hipFuncSetAttribute(k[i], hipFuncAttributeMaxDynamicSharedMemorySize, lds[i]);
        });
        if (attr8 != hipSuccess) return attr8;
        if (wide) {
            if (pass) wgrad_fp8_kernel<1, 2><<<(unsigned)grid, wf8_nt<2>(), wf8_lds<2>(), s>>>(a, nlead, tiles);
            else wgrad_fp8_kernel<0, 2><<<(unsigned)grid, wf8_nt<2>(), wf8_lds<2>(), s>>>(a, nlead, tiles);
        } else {
            if (pass) wgrad_fp8_kernel<1, 1><<<(unsigned)grid, wf8_nt<1>(), wf8_lds<1>(), s>>>(a, nlead, tiles);
            else wgrad_fp8_kernel<0, 1><<<(unsigned)grid, wf8_nt<1>(), wf8_lds<1>(), s>>>(a, nlead, tiles);
        }
    } else {
        // the 256-wide p tile needs every p dimension and split of the launch on 256-value boundaries
        bool wide = true;
        for (int i = 0; i < a.nprob; ++i) wide = wide && a.p[i].Pdim % 256 == 0 && a.p[i].split % 256 == 0;
        if (wide) {
            for (int i = 0; i < a.nprob; ++i) a.p[i].p_tile = 256;
            tiles = 0;
            for (int i = 0; i < a.nprob; ++i) tiles += wg_tiles(a.p[i]);
            nlead = (a.nprob > 1 && !a.p[0].offsets) ? wg_tiles(a.p[0]) : 0;
            grid = (nlead + 7) / 8 * 8 + (tiles - nlead + 7) / 8 * 8;
        }
        static std::once_flag once;
        static hipError_t attr = hipSuccess;
        std::call_once(once, [] {
            const void *k[4] = {(const void *)wgrad_bf16_kernel<0, 1>, (const void *)wgrad_bf16_kernel<1, 1>,
                                (const void *)wgrad_bf16_kernel<0, 2>, (const void *)wgrad_bf16_kernel<1, 2>};
            const int lds[4] = {wgb_lds_all<1>(), wgb_lds_all<1>(), wgb_lds_all<2>(), wgb_lds_all<2>()};
            for (int i = 0; i < 4 && attr == hipSuccess; ++i)
                attr = hipFuncSetAttribute(k[i], hipFuncAttributeMaxDynamicSharedMemorySize, lds[i]);
        });
        if (attr != hipSuccess) return attr;
        if (wide) {
            if (pass) wgrad_bf16_kernel<1, 2><<<(unsigned)grid, wgb_nt<2>(), wgb_lds_all<2>(), s>>>(a, nlead, tiles);
            else wgrad_bf16_kernel<0, 2><<<(unsigned)grid, wgb_nt<2>(), wgb_lds_all<2>(), s>>>(a, nlead, tiles);
        } else {
            if (pass) wgrad_bf16_kernel<1, 1><<<(unsigned)grid, wgb_nt<1>(), wgb_lds_all<1>(), s>>>(a, nlead, tiles);
            else wgrad_bf16_kernel<0, 1><<<(unsigned)grid, wgb_nt<1>(), wgb_lds_all<1>(), s>>>(a, nlead, tiles);
        }
    }
    return hipGetLastError();
}

}  // namespace moe
