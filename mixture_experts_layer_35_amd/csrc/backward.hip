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
    typedef typename std::conditional<ESZ == 2, uint16_t, uint32_t>::type E;
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

// ---- combine backward: one workgroup per token ----
// dY[inv(t,j)] = g_{t,j} dO_t (rounded to the act dtype); dg_{t,j} = dO_t . y[inv(t,j)]
template <int DT, int KMAX>
__global__ __launch_bounds__(BW_NT) void bwd_combine_kernel(const void *__restrict__ dout, const void *__restrict__ y,
                                                            const int32_t *__restrict__ inv,
                                                            const float *__restrict__ topk_w, int64_t T, int d, int K,
                                                            void *__restrict__ dy, float *__restrict__ dg) {
    __shared__ float red[BW_NT / 64][KMAX];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        float part[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) part[j] = 0.0f;
        for (int c = threadIdx.x * 8; c < d; c += BW_NT * 8) {
            float o[8];
            ld8v<DT>(dout, t * d + c, o);
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

// ---- weight gradient: C[p][q] = sum over an expert's rows r of P[r][p] Q[qrow(r)][q] ----
// Tile 128 (p) x 128 (q) per 256-thread workgroup (2 x 2 waves of 64 x 64).  Each
// 32-row step stages P and Q transposed in LDS ([p][r], [q][r], rows padded), so
// MFMA fragments (8 consecutive r per lane) are single 16-byte reads.  Q is the
// MFMA row operand: a lane's four results are four consecutive q of one p, one
// store into C's row p.  All of an expert's rows are reduced in one tile, in
// order: no cross-tile reduction, deterministic.
constexpr int WG_T = 128, WG_R = 32, WG_LD = WG_R + 8;   // LDS row: 32 values + pad

template <int DT>
__global__ __launch_bounds__(BW_NT) void wgrad_kernel(const WgradArgs a) {
    typedef typename std::conditional<DT == DT_BF16, uint16_t, float>::type E;
    __shared__ E Pt[WG_T][WG_LD];
    __shared__ E Qt[WG_T][WG_LD];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wp = wid >> 1, wq = wid & 1;

    // tile -> (problem, expert, p-tile, q-tile)
    int64_t t = blockIdx.x;
    int pi = 0;
    const int64_t per0 = (int64_t)(a.p[0].Pdim / WG_T) * (a.p[0].Qdim / WG_T);
    if (a.nprob > 1 && t >= (int64_t)a.p[0].n_exp * per0) { t -= (int64_t)a.p[0].n_exp * per0; pi = 1; }
    const WgradProblem &P = pi ? a.p[1] : a.p[0];
    const int ptiles = P.Pdim / WG_T, qtiles = P.Qdim / WG_T;
    const int e = (int)(t / ((int64_t)ptiles * qtiles));
    const int64_t tt = t % ((int64_t)ptiles * qtiles);
    const int p0 = (int)(tt / qtiles) * WG_T, q0 = (int)(tt % qtiles) * WG_T;
    const int64_t rb = P.offsets ? (int64_t)P.offsets[e] : (int64_t)e * P.rows_fixed;
    const int64_t M = P.offsets ? (int64_t)P.offsets[e + 1] - rb : P.rows_fixed;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

    for (int64_t r0 = 0; r0 < M; r0 += WG_R) {
        // stage: 32 rows x 128 values of P and of Q; thread takes 16 values of each (2 x 8)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int id = tid + BW_NT * h;         // 0..511: row id / 16, 8 values at (id % 16) * 8
            const int rr = id >> 4, cc = (id & 15) * 8;
            const int64_t r = r0 + rr;
            float pv[8], qv[8];
            if (r < M) {
                const int64_t R = rb + r;
                ld8v<DT>(P.P, (P.p_local ? r : R) * P.P_ld + p0 + cc, pv);
                const int64_t QR = P.q_gather ? (int64_t)P.q_gather[R] : (P.q_local ? r : R);
                ld8v<DT>(P.Q, QR * P.Q_ld + q0 + cc, qv);
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) { pv[q] = 0.0f; qv[q] = 0.0f; }
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (DT == DT_BF16) {
                    Pt[cc + q][rr] = (E)(__float_as_uint(pv[q]) >> 16);   // exact: the values are bf16
                    Qt[cc + q][rr] = (E)(__float_as_uint(qv[q]) >> 16);
                } else {
                    Pt[cc + q][rr] = pv[q];
                    Qt[cc + q][rr] = qv[q];
                }
            }
        }
        __syncthreads();
        if (DT == DT_BF16) {
            bf16x8 qa[4], pb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                qa[i] = *(const bf16x8 *)&Qt[wq * 64 + i * 16 + (lane & 15)][8 * (lane >> 4)];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                pb[j] = *(const bf16x8 *)&Pt[wp * 64 + j * 16 + (lane & 15)][8 * (lane >> 4)];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[i], pb[j], acc[i][j], 0, 0, 0);
        } else {
#pragma unroll
            for (int s = 0; s < WG_R / 4; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            (float)Qt[wq * 64 + i * 16 + (lane & 15)][4 * s + (lane >> 4)],
                            (float)Pt[wp * 64 + j * 16 + (lane & 15)][4 * s + (lane >> 4)], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
    // lane: q = q0 + wq*64 + i*16 + 4*(lane>>4) + {0..3}, p = p0 + wp*64 + j*16 + (lane&15)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int p = p0 + wp * 64 + j * 16 + (lane & 15);
        void *out = p < P.split ? P.out0 : P.out1;
        const int prow = p < P.split ? p : p - P.split;
        const int64_t base = ((int64_t)e * (P.split < P.Pdim ? P.split : P.Pdim) + prow) * P.Qdim;
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
}

}  // namespace

hipError_t launch_transpose(int dt, const void *src, int64_t nmat, int rows, int cols, void *dst, int dst_ld, int col0,
                            hipStream_t s) {
    const int64_t blocks = nmat * (rows / 64) * (int64_t)(cols / 64);
    if (blocks <= 0) return hipSuccess;
    if (dt == DT_F32)
        transpose_kernel<4><<<(unsigned)blocks, 256, 0, s>>>((const char *)src, rows, cols, (char *)dst, dst_ld, col0);
    else
        transpose_kernel<2><<<(unsigned)blocks, 256, 0, s>>>((const char *)src, rows, cols, (char *)dst, dst_ld, col0);
    return hipGetLastError();
}

hipError_t launch_bwd_combine(int dt, const void *dout, const void *y, const int32_t *inv, const float *topk_w, int64_t T,
                              int d, int K, void *dy, float *dg, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const unsigned grid = (unsigned)(T < (1 << 20) ? T : (1 << 20));
#define BC(DT, KM) bwd_combine_kernel<DT, KM><<<grid, BW_NT, 0, s>>>(dout, y, inv, topk_w, T, d, K, dy, dg)
    if (dt == DT_F32) { if (K <= 8) BC(DT_F32, 8); else BC(DT_F32, 32); }
    else { if (K <= 8) BC(DT_BF16, 8); else BC(DT_BF16, 32); }
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

hipError_t launch_wgrad(int dt, const WgradArgs &a, hipStream_t s) {
    int64_t tiles = 0;
    for (int i = 0; i < a.nprob; ++i)
        tiles += (int64_t)a.p[i].n_exp * (a.p[i].Pdim / WG_T) * (a.p[i].Qdim / WG_T);
    if (tiles <= 0) return hipSuccess;
    if (tiles >= (1ll << 31)) return hipErrorInvalidValue;
    if (dt == DT_F32) wgrad_kernel<DT_F32><<<(unsigned)tiles, BW_NT, 0, s>>>(a);
    else wgrad_kernel<DT_BF16><<<(unsigned)tiles, BW_NT, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
