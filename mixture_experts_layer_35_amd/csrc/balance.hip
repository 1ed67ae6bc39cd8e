// balance.hip -- complementary sequence-wise balance statistic ("DeepSeek-V3
// Technical Report", §2.1.2: a tiny loss alpha * sum_i f_i P_i per sequence,
// kept next to the auxiliary-loss-free bias; §4.2: alpha = 0.0001).
//
// For a sequence of Ts tokens: f_i = N_r / (K * Ts) * (slots routed to expert
// i) and P_i = mean over the sequence of s_{i,t} / sum_k s_{k,t}.
//
// Two passes, both in a fixed order so the result is deterministic:
//   1. one workgroup per 64-token block of a sequence: per-expert sums of the
//      affinity shares and slot counts of its tokens;
//   2. one workgroup per sequence: the blocks' partials in order, f_i and
//      P_i, and the tree-reduced sum of f_i * P_i.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int BAL_TOK = 64;   // tokens per block
constexpr int BAL_NT = 256;   // threads per workgroup

// Lane l of each wave holds experts l, l+64, ... (R of them).
template <int R>
__global__ __launch_bounds__(BAL_NT) void balance_partial_kernel(const float *__restrict__ scores,
                                                                 const int32_t *__restrict__ idx, int64_t T,
                                                                 int Nr, int K, int64_t seq_len, int bps,
                                                                 float *__restrict__ part_share,
                                                                 int32_t *__restrict__ part_count) {
    __shared__ float ssh[BAL_NT / 64][64 * R];
    __shared__ int scnt[BAL_NT / 64][64 * R];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int64_t b = blockIdx.x;
    const int64_t q = b / bps, j = b % bps;
    const int64_t seq_end = min(T, (q + 1) * seq_len);
    const int64_t t0 = q * seq_len + j * BAL_TOK;
    const int64_t t1 = min(seq_end, t0 + BAL_TOK);
    float share[R];
    int cnt[R];
#pragma unroll
    for (int r = 0; r < R; ++r) { share[r] = 0.0f; cnt[r] = 0; }
    for (int64_t t = t0 + wid; t < t1; t += BAL_NT / 64) {
        float s[R];
        float row = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = lane + 64 * r;
            s[r] = i < Nr ? scores[t * Nr + i] : 0.0f;
            row += s[r];
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) row += __shfl_xor(row, off, 64);
#pragma unroll
        for (int r = 0; r < R; ++r) share[r] += s[r] / row;
        for (int k = 0; k < K; ++k) {
            const int e = idx[t * K + k];
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (e == lane + 64 * r) cnt[r] += 1;
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        ssh[wid][lane + 64 * r] = share[r];
        scnt[wid][lane + 64 * r] = cnt[r];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < Nr; i += BAL_NT) {
        float sum = 0.0f;
        int c = 0;
#pragma unroll
        for (int w = 0; w < BAL_NT / 64; ++w) {
            sum += ssh[w][i];
            c += scnt[w][i];
        }
        part_share[b * Nr + i] = sum;
        part_count[b * Nr + i] = c;
    }
}

__global__ __launch_bounds__(BAL_NT) void balance_final_kernel(const float *__restrict__ part_share,
                                                               const int32_t *__restrict__ part_count, int64_t T,
                                                               int Nr, int K, int64_t seq_len, int bps, float alpha,
                                                               float *__restrict__ loss, int32_t *__restrict__ counts,
                                                               float *__restrict__ share) {
    __shared__ float red[BAL_NT];
    const int64_t q = blockIdx.x;
    const int64_t Ts = min(T, (q + 1) * seq_len) - q * seq_len;
    const int nb = (int)((Ts + BAL_TOK - 1) / BAL_TOK);
    float acc = 0.0f;
    for (int i = threadIdx.x; i < Nr; i += BAL_NT) {
        float s = 0.0f;
        int c = 0;
        for (int j = 0; j < nb; ++j) {
            s += part_share[(q * bps + j) * Nr + i];
            c += part_count[(q * bps + j) * Nr + i];
        }
        const float f = (float)Nr / ((float)K * (float)Ts) * (float)c;
        const float P = s / (float)Ts;
        acc += f * P;
        if (counts) counts[q * Nr + i] = c;
        if (share) share[q * Nr + i] = P;
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = BAL_NT / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) loss[q] = alpha * red[0];
}

}  // namespace

int64_t balance_blocks_per_seq(int64_t T, int64_t seq_len) {
    return (min(T, seq_len) + BAL_TOK - 1) / BAL_TOK;
}

hipError_t launch_seq_balance(const float *scores, const int32_t *idx, int64_t T, int Nr, int K, int64_t seq_len,
                              float alpha, float *loss, int32_t *counts, float *share, float *part_share,
                              int32_t *part_count, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const int64_t n_seq = (T + seq_len - 1) / seq_len;
    const int bps = (int)balance_blocks_per_seq(T, seq_len);
    const unsigned grid = (unsigned)(n_seq * bps);
    const int R = (Nr + 63) / 64;
#define BP(RR)                                                                                                          \
    balance_partial_kernel<RR><<<grid, BAL_NT, 0, s>>>(scores, idx, T, Nr, K, seq_len, bps, part_share, part_count)
    if (R <= 1) BP(1);
    else if (R <= 2) BP(2);
    else if (R <= 4) BP(4);
    else if (R <= 8) BP(8);
    else BP(16);
#undef BP
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    balance_final_kernel<<<(unsigned)n_seq, BAL_NT, 0, s>>>(part_share, part_count, T, Nr, K, seq_len, bps, alpha, loss,
                                                           counts, share);
    return hipGetLastError();
}

}  // namespace moe
