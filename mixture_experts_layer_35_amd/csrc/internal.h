// internal.h -- launchers shared between the libmoe translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

enum { DT_F32 = 0, DT_BF16 = 1, DT_E4M3 = 2 };

// Number of compute units of the current device (cached per device).
int device_cus();

// ---- router ----------------------------------------------------------------
// scores[T][Nr] = sigmoid(u[T][d] . gate_w[Nr][d]^T), fp32 accumulation.
hipError_t launch_router_gemm(int dt, const void *u, const void *gate_w, float *scores, int64_t T, int d, int Nr,
                              hipStream_t s);
// Split-K gate GEMM over all experts (bf16, Nr == 256, groups of a multiple of 16
// experts, K <= 16): chunk partials to part (router_partial_bytes), then affinities
// (to scores, when not null), selection and gates in one finishing kernel.
bool router_splitk_ok(int dt, int Nr, int G, int K);
size_t router_partial_bytes(int64_t T, int d, int Nr);
hipError_t launch_router_splitk(const void *u, const void *gate_w, float *part, float *scores, const float *bias,
                                int64_t T, int d, int G, int Mg, int K, float routed_scale, int32_t *topk_idx,
                                float *topk_w, hipStream_t s);
// Group-limited biased top-K selection and normalised gates from fp32 scores.
hipError_t launch_router_select(const float *scores, const float *bias, int64_t T, int Nr, int G, int Mg, int K,
                                float routed_scale, int32_t *topk_idx, float *topk_w, hipStream_t s);

// ---- dispatch --------------------------------------------------------------
// Block histogram (64 tokens per block) -> blockcounts[nb][Nr].
hipError_t launch_perm_hist(const int32_t *topk_idx, int64_t T, int K, int Nr, int32_t *blockcounts,
                            hipStream_t s);
// counts, offsets, per-block row bases (in place in blockcounts).
hipError_t launch_perm_scan(int32_t *blockcounts, int64_t T, int Nr, int32_t *counts, int32_t *offsets,
                            hipStream_t s);
// perm_token / inv_perm from topk_idx and per-block row bases.
hipError_t launch_perm_scatter(const int32_t *topk_idx, const int32_t *blockbase, int64_t T, int K, int Nr,
                               int32_t *perm_token, int32_t *inv_perm, hipStream_t s);
inline int64_t perm_blocks(int64_t T) { return (T + 63) / 64; }

// dst[r] = src[idx ? idx[r] : r] for r < rows, row = cols elements of dtype dt (copy).
hipError_t launch_gather_rows(int dt, const void *src, const int32_t *idx, int64_t rows, int cols, void *dst,
                              hipStream_t s);
// q[r], sc[r] = Q_1x128(src[idx ? idx[r] : r]); src dtype dt (F32 / BF16).
hipError_t launch_quant_rows(int dt, const void *src, const int32_t *idx, int64_t rows, int cols, uint8_t *q,
                             float *sc, hipStream_t s);
// 128x128 block quantisation of nmat [rows][cols] matrices.
hipError_t launch_quant_blocks(int dt, const void *w, int64_t nmat, int rows, int cols, uint8_t *q, float *sc,
                               hipStream_t s);

// ---- grouped FFN -------------------------------------------------------------
struct FfnProblem {
    int n_exp;              // experts
    int x_local;            // x row of local row r is r (shared experts over u)
    const int32_t *offsets; // [n_exp+1] device row offsets, or null: expert e owns rows [e*rows_fixed, +rows_fixed)
    int64_t rows_fixed;
    const int32_t *gather;  // x row of problem row R is gather[R] (null: R, or local r when x_local)
    const void *x;          // activations, rows of K elements
    const float *xs;        // E4M3: [rows][K/128] scales
    const void *w0;         // gate (gate/up pass) or down weights, [n_exp][F][K]
    const void *w1;         // up weights (gate/up pass)
    const float *s0, *s1;   // E4M3 block scales [n_exp][F/128][K/128]
    void *out;              // gate/up: H [rows][F]; down: y [rows][F]
    float *out_s;           // E4M3 gate/up: H scales [rows][F/128]
    int64_t out_ld;         // elements between output rows (0: F)
    const void *dh;         // gate/up gradient pass: dH [rows][F] (act dtype)
    float *ab;              // FFN_GATEUP_SAVE: the SwiGLU inputs a | b as fp32 [rows][2F]
};
struct FfnArgs {
    FfnProblem p[2];
    int nprob;
    int K;      // reduction length
    int F;      // output features (I for gate/up, d for down)
    int *ctr;   // FFN_QUEUE_INTS device ints of tile-queue counters (zeroed by launch_ffn)
};
constexpr int FFN_QUEUE_INTS = 8;
constexpr int kMaxExperts = 1024;
// mode: FFN_DOWN (out = x . w^T), FFN_GATEUP (out = SiLU(x . w0^T) * (x . w1^T)),
// FFN_GATEUP_BWD (a = x . w0^T, b = x . w1^T recomputed; with dh read from P.dh,
// out[:, 0:F] = dh * b * SiLU'(a) and out[:, F:2F] = dh * SiLU(a); out_ld = 2F).
// FFN_BWD_DH / FFN_BWD_DX: the plain product of FFN_DOWN for the backward's dH = dY W_down and
// dX = [dA | dB] [W_gate ; W_up] passes, instantiated apart so that profiles tell the passes apart.
// FFN_GATEUP_SAVE: FFN_GATEUP that also stores a | b to P.ab, a mode of its own so that the
// plain forward kernel carries no extra registers for it.
enum { FFN_DOWN = 0, FFN_GATEUP = 1, FFN_GATEUP_BWD = 2, FFN_BWD_DH = 3, FFN_BWD_DX = 4, FFN_GATEUP_SAVE = 5 };
hipError_t launch_ffn(int dt, int mode, const FfnArgs &a, hipStream_t s);
// SwiGLU gradient from saved inputs: for rows x F features, dab[r][f] = da and
// dab[r][F + f] = db from dh [rows][F] and ab [rows][2F] (fp32); dh and dab are fp32
// for dt = DT_F32 and bf16 otherwise, as in the FFN_GATEUP_BWD epilogue.
hipError_t launch_swiglu_grad(int dt, const void *dh, const float *ab, void *dab, int64_t rows, int F, uint8_t *q8,
                              float *qs, hipStream_t s);

// ---- backward ----------------------------------------------------------------
// Weight-gradient problem: for each expert e with rows r (offsets, or rows_fixed
// each), C_e[p][q] = sum_r P[prow(r)][p] * Q[qrow(r)][q] over the expert's rows r:
// qrow(r) = q_gather[r], else r within the expert when q_local, else the global
// row (prow likewise with p_local).  Rows p < split go to out0 [n][split][Qdim],
// the rest to out1 [n][Pdim - split][Qdim].
struct WgradProblem {
    int n_exp;
    const int32_t *offsets;
    int64_t rows_fixed;
    const void *P;
    int64_t P_ld;
    const void *Q;
    int64_t Q_ld;
    const int32_t *q_gather;
    int p_local, q_local;   // row r of the expert reads P / Q row r (not base + r): an input shared by experts
    int Pdim, Qdim, split;
    void *out0, *out1;
    int64_t rows_hint;      // typical rows per expert (sizes the work per workgroup)
    int step_rows;          // rows per reduction step of the kernel (set by launch_wgrad)
    int p_tile;             // width of a workgroup's p tile, 128 or 256 (set by launch_wgrad)
    // e4m3 operands: 128 x 1 column scales per 128-row run ([run][Pdim], [run][Qdim]); the
    // expert's first run is bbase[e] (offsets problems) or e * ceil(rows_fixed / 128); an
    // operand read with p_local / q_local starts at run 0
    const float *Ps, *Qs;
    const int32_t *bbase;
};
struct WgradArgs {
    WgradProblem p[2];
    int nprob;
};
hipError_t launch_transpose(int dt, const void *src, int64_t nmat, int rows, int cols, void *dst, int dst_ld, int col0,
                            hipStream_t s);
hipError_t launch_transpose_scales(const float *src, int64_t nmat, int rows, int cols, float *dst, int dst_ld, int col0,
                                   hipStream_t s);
hipError_t launch_block_base(const int32_t *offsets, int n, int32_t *bbase, hipStream_t s);
// 128 x 1 tiles along segment rows (segments: device offsets with run bases bbase, or n_seg
// runs of seg_rows rows); in_dt DT_BF16, or DT_E4M3 with 1 x 128 scales src_s.
hipError_t launch_quant_cols(int in_dt, const void *src, const float *src_s, const int32_t *gather,
                             const int32_t *offsets, const int32_t *bbase, int64_t seg_rows, int n_seg, int64_t max_blocks,
                             int cols, uint8_t *q, float *sc, hipStream_t s);
hipError_t launch_bwd_combine(int dt, const void *dout, const void *y, const int32_t *inv, const float *topk_w, int64_t T,
                              int d, int K, void *dy, float *dg, uint8_t *dyq, float *dys, uint8_t *doq, float *dos,
                              hipStream_t s);
hipError_t launch_bwd_token(int dt, const void *dxr, const void *dxs, int Ns, const int32_t *inv, const int32_t *idx,
                            const float *scores, const float *dg, const void *gate_w, int64_t T, int d, int Nr, int K,
                            float rs, void *du, float *dz_row, hipStream_t s);
hipError_t launch_dgate(int dt, const void *u, const int32_t *perm, const int32_t *offsets, const float *dz_row, int Nr,
                        int d, float *dgate, hipStream_t s);
// pass: 0 for dW_down, 1 for dW_gate / dW_up (separate instantiations, same code)
hipError_t launch_wgrad(int dt, int pass, const WgradArgs &a, hipStream_t s);

// ---- combine / bias ----------------------------------------------------------
hipError_t launch_combine(int dt_out, int dt_res, const void *y_perm, const int32_t *inv_perm, const float *topk_w,
                          const void *y_shared, int Ns, const void *residual, void *out, int64_t T, int d, int K,
                          hipStream_t s);
// Sequence-wise balance statistic; part_share / part_count hold
// n_seq * balance_blocks_per_seq(T, seq_len) rows of Nr partials each.
int64_t balance_blocks_per_seq(int64_t T, int64_t seq_len);
hipError_t launch_seq_balance(const float *scores, const int32_t *idx, int64_t T, int Nr, int K, int64_t seq_len,
                              float alpha, float *loss, int32_t *counts, float *share, float *part_share,
                              int32_t *part_count, hipStream_t s);
hipError_t launch_bias_update(const int32_t *counts, float *bias, int64_t T, int K, int Nr, float gamma,
                              hipStream_t s);
hipError_t launch_set_offsets(int32_t *offsets, int n, int64_t step, hipStream_t s);

}  // namespace moe
