// permute.hip -- dispatch of tokens to experts and fine-grained FP8 quantisation.
//
// Dispatch ("DeepSeek-V3 Technical Report", §2.1.2: no token is dropped; the
// whole-batch load of an expert is the number of (token, slot) pairs routed to
// it): a per-block histogram, a scan over (expert, block), and a scatter whose
// in-block ranks come from per-expert lane bitmasks, so rows of one expert are
// in increasing token order without any ordering by atomics.
//
// Quantisation (§3.3: 1 x 128 activation tiles, 128 x 128 weight blocks, one
// fp32 scale per group): scale = amax / 448 (1 for an all-zero group); code =
// E4M3FN nearest-even of clamp(x / scale) with an IEEE fp32 division.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

// ---- dispatch ----------------------------------------------------------------

// One wave per block of 64 tokens: LDS histogram of the block's (token, slot) pairs.
__global__ __launch_bounds__(64) void perm_hist_kernel(const int32_t *__restrict__ idx, int64_t T, int K, int Nr,
                                                      int32_t *__restrict__ blockcounts) {
    __shared__ int hist[kMaxExperts];
    const int lane = threadIdx.x;
    for (int e = lane; e < Nr; e += 64) hist[e] = 0;
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * 64 + lane;
    if (t < T)
        for (int j = 0; j < K; ++j) atomicAdd(&hist[idx[t * K + j]], 1);
    __syncthreads();
    int32_t *out = blockcounts + (int64_t)blockIdx.x * Nr;
    for (int e = lane; e < Nr; e += 64) out[e] = hist[e];
}

// One workgroup: counts[e] = sum over blocks; offsets = exclusive scan of counts;
// blockcounts[b][e] becomes the first row of block b's pairs for expert e.
// Thread (part, e) walks a contiguous range of blocks of expert e (P = 1024/Nr
// parts per expert; neighbouring threads read neighbouring experts of one
// block), 16 independent loads at a time.
constexpr int SCAN_NT = 1024;
constexpr int SCAN_UNROLL = 16;

__global__ __launch_bounds__(SCAN_NT) void perm_scan_kernel(int32_t *__restrict__ bc, int64_t nb, int Nr,
                                                           int32_t *__restrict__ counts, int32_t *__restrict__ offsets) {
    __shared__ int part_sum[SCAN_NT];     // [part][e]: block-range sums, then their exclusive prefix
    __shared__ int sums[SCAN_NT];
    const int tid = threadIdx.x;
    const int P = SCAN_NT / Nr;           // Nr <= 1024
    const int e = tid % Nr, part = tid / Nr;
    const bool active = part < P;
    const int64_t chunk = (nb + P - 1) / P;
    const int64_t lo = active ? min(nb, (int64_t)part * chunk) : 0, hi = active ? min(nb, lo + chunk) : 0;

    int local = 0;
    for (int64_t b0 = lo; b0 < hi; b0 += SCAN_UNROLL) {
        int v[SCAN_UNROLL];
#pragma unroll
        for (int u = 0; u < SCAN_UNROLL; ++u) v[u] = b0 + u < hi ? bc[(b0 + u) * Nr + e] : 0;
#pragma unroll
        for (int u = 0; u < SCAN_UNROLL; ++u) local += v[u];
    }
    if (active) part_sum[part * Nr + e] = local;
    __syncthreads();
    int total = 0;
    if (tid < Nr) {
        for (int p = 0; p < P; ++p) {     // exclusive prefix over the parts of expert tid
            const int c = part_sum[p * Nr + tid];
            part_sum[p * Nr + tid] = total;
            total += c;
        }
    }
    sums[tid] = tid < Nr ? total : 0;
    __syncthreads();
    // Hillis-Steele inclusive scan over the expert totals
    for (int off = 1; off < SCAN_NT; off <<= 1) {
        const int v = tid >= off ? sums[tid - off] : 0;
        __syncthreads();
        sums[tid] += v;
        __syncthreads();
    }
    if (tid < Nr) {
        counts[tid] = total;
        offsets[tid] = sums[tid] - total;  // exclusive
        if (tid == Nr - 1) offsets[Nr] = sums[tid];
    }
    if (!active) return;
    // first row of this thread's first block for expert e: the expert's exclusive
    // offset plus the pairs of the earlier parts
    int run = (e > 0 ? sums[e - 1] : 0) + part_sum[part * Nr + e];
    for (int64_t b0 = lo; b0 < hi; b0 += SCAN_UNROLL) {
        int v[SCAN_UNROLL];
#pragma unroll
        for (int u = 0; u < SCAN_UNROLL; ++u) v[u] = b0 + u < hi ? bc[(b0 + u) * Nr + e] : 0;
#pragma unroll
        for (int u = 0; u < SCAN_UNROLL; ++u) {
            if (b0 + u < hi) bc[(b0 + u) * Nr + e] = run;
            run += v[u];
        }
    }
}

// One wave per block of 64 tokens.  mask[e] has bit l set when lane l's token
// routes to e; the rank of a pair inside its expert is the number of lower
// lanes in that mask (a token routes to an expert at most once).
__global__ __launch_bounds__(64) void perm_scatter_kernel(const int32_t *__restrict__ idx,
                                                         const int32_t *__restrict__ blockbase, int64_t T, int K,
                                                         int Nr, int32_t *__restrict__ perm_token,
                                                         int32_t *__restrict__ inv_perm) {
    __shared__ unsigned long long mask[kMaxExperts];
    const int lane = threadIdx.x;
    for (int e = lane; e < Nr; e += 64) mask[e] = 0ull;
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * 64 + lane;
    const bool live = t < T;
    if (live)
        for (int j = 0; j < K; ++j) atomicOr(&mask[idx[t * K + j]], 1ull << lane);
    __syncthreads();
    if (!live) return;
    const int32_t *base = blockbase + (int64_t)blockIdx.x * Nr;
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int j = 0; j < K; ++j) {
        int e = idx[t * K + j];
        int row = base[e] + __popcll(mask[e] & below);
        perm_token[row] = (int32_t)t;
        inv_perm[t * K + j] = row;
    }
}

// ---- row gather / quantisation ------------------------------------------------

// dst row r = src row (idx ? idx[r] : r); 16-byte chunks, grid-stride over rows.
__global__ __launch_bounds__(256) void gather_rows_kernel(const char *__restrict__ src, const int32_t *__restrict__ idx,
                                                         int64_t rows, int64_t rowbytes, char *__restrict__ dst) {
    const int64_t chunks = rowbytes >> 4;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const int64_t sr = idx ? idx[r] : r;
        const u32x4 *s = (const u32x4 *)(src + sr * rowbytes);
        u32x4 *d = (u32x4 *)(dst + r * rowbytes);
        for (int64_t c = threadIdx.x; c < chunks; c += 256) d[c] = s[c];
    }
}

template <int DT>
__device__ __forceinline__ void load8(const char *p, float v[8]) {
    if (DT == DT_BF16) {
        u32x4 w = *(const u32x4 *)p;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
    }
}

// 16 lanes per 1 x 128 tile (8 elements per lane); grid-stride over (row, tile).
template <int DT>
__global__ __launch_bounds__(256) void quant_rows_kernel(const char *__restrict__ src, const int32_t *__restrict__ idx,
                                                        int64_t rows, int cols, uint8_t *__restrict__ q,
                                                        float *__restrict__ sc) {
    constexpr int esz = DT == DT_F32 ? 4 : 2;
    const int ntile = cols >> 7;
    const int64_t total = rows * ntile;
    const int sub = threadIdx.x & 15;
    // the loop bound is uniform over the workgroup, so every lane reaches the shuffles
    for (int64_t gbase = (int64_t)blockIdx.x * 16; gbase < total; gbase += (int64_t)gridDim.x * 16) {
        const int64_t g = gbase + (threadIdx.x >> 4);
        const bool live = g < total;
        const int64_t gg = live ? g : total - 1;
        const int64_t r = gg / ntile;
        const int tile = (int)(gg - r * ntile);
        const int64_t sr = idx ? idx[r] : r;
        float v[8];
        load8<DT>(src + (sr * cols + tile * 128 + sub * 8) * esz, v);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
        const float scale = quant_scale(amax);
        u32x2 out;
        out[0] = pack_e4m3x4(clamp448(v[0] / scale), clamp448(v[1] / scale), clamp448(v[2] / scale),
                             clamp448(v[3] / scale));
        out[1] = pack_e4m3x4(clamp448(v[4] / scale), clamp448(v[5] / scale), clamp448(v[6] / scale),
                             clamp448(v[7] / scale));
        if (live) {
            *(u32x2 *)(q + r * cols + tile * 128 + sub * 8) = out;
            if (sub == 0) sc[r * ntile + tile] = scale;
        }
    }
}

// One workgroup per 128 x 128 block: thread t covers row t/2, columns (t%2)*64 .. +64.
template <int DT>
__global__ __launch_bounds__(256) void quant_blocks_kernel(const char *__restrict__ w, int rows, int cols,
                                                          uint8_t *__restrict__ q, float *__restrict__ sc) {
    constexpr int esz = DT == DT_F32 ? 4 : 2;
    __shared__ float red[4];
    const int rb = rows >> 7, cb = cols >> 7;
    const int64_t blk = blockIdx.x;
    const int64_t m = blk / ((int64_t)rb * cb);
    const int bi = (int)((blk / cb) % rb), bj = (int)(blk % cb);
    const int tid = threadIdx.x;
    const int r = bi * 128 + (tid >> 1);
    const int c0 = bj * 128 + (tid & 1) * 64;
    const int64_t base = (m * rows + r) * (int64_t)cols + c0;
    float v[64];
#pragma unroll
    for (int i = 0; i < 8; ++i) load8<DT>(w + (base + i * 8) * esz, v + i * 8);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = wave_max_f32(amax);
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float scale = quant_scale(amax);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float *x = v + i * 16 + k * 4;
            o[k] = pack_e4m3x4(clamp448(x[0] / scale), clamp448(x[1] / scale), clamp448(x[2] / scale),
                               clamp448(x[3] / scale));
        }
        *(u32x4 *)(q + base + i * 16) = o;
    }
    if (tid == 0) sc[(m * rb + bi) * cb + bj] = scale;
}

}  // namespace

hipError_t launch_perm_hist(const int32_t *topk_idx, int64_t T, int K, int Nr, int32_t *blockcounts, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    perm_hist_kernel<<<(unsigned)perm_blocks(T), 64, 0, s>>>(topk_idx, T, K, Nr, blockcounts);
    return hipGetLastError();
}

hipError_t launch_perm_scan(int32_t *blockcounts, int64_t T, int Nr, int32_t *counts, int32_t *offsets, hipStream_t s) {
    perm_scan_kernel<<<1, 1024, 0, s>>>(blockcounts, perm_blocks(T), Nr, counts, offsets);
    return hipGetLastError();
}

hipError_t launch_perm_scatter(const int32_t *topk_idx, const int32_t *blockbase, int64_t T, int K, int Nr,
                               int32_t *perm_token, int32_t *inv_perm, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    perm_scatter_kernel<<<(unsigned)perm_blocks(T), 64, 0, s>>>(topk_idx, blockbase, T, K, Nr, perm_token, inv_perm);
    return hipGetLastError();
}

hipError_t launch_gather_rows(int dt, const void *src, const int32_t *idx, int64_t rows, int cols, void *dst,
                              hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    const int64_t rowbytes = (int64_t)cols * (dt == DT_F32 ? 4 : dt == DT_BF16 ? 2 : 1);
    const int64_t grid = rows < 8192 ? rows : 8192;
    gather_rows_kernel<<<(unsigned)grid, 256, 0, s>>>((const char *)src, idx, rows, rowbytes, (char *)dst);
    return hipGetLastError();
}

hipError_t launch_quant_rows(int dt, const void *src, const int32_t *idx, int64_t rows, int cols, uint8_t *q,
                             float *sc, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    const int64_t groups = rows * (cols / 128);
    int64_t grid = (groups + 15) / 16;
    if (grid > 16384) grid = 16384;
    if (dt == DT_F32)
        quant_rows_kernel<DT_F32><<<(unsigned)grid, 256, 0, s>>>((const char *)src, idx, rows, cols, q, sc);
    else
        quant_rows_kernel<DT_BF16><<<(unsigned)grid, 256, 0, s>>>((const char *)src, idx, rows, cols, q, sc);
    return hipGetLastError();
}

hipError_t launch_quant_blocks(int dt, const void *w, int64_t nmat, int rows, int cols, uint8_t *q, float *sc,
                               hipStream_t s) {
    const int64_t blocks = nmat * (rows / 128) * (int64_t)(cols / 128);
    if (blocks <= 0) return hipSuccess;
    if (dt == DT_F32)
        quant_blocks_kernel<DT_F32><<<(unsigned)blocks, 256, 0, s>>>((const char *)w, rows, cols, q, sc);
    else
        quant_blocks_kernel<DT_BF16><<<(unsigned)blocks, 256, 0, s>>>((const char *)w, rows, cols, q, sc);
    return hipGetLastError();
}

}  // namespace moe
