// Radix top-k over block-score rows for gfx950.
//
// One workgroup of 256 threads per row; thread t owns the KPT consecutive entries [t*KPT, t*KPT + KPT) so that the
// final compaction runs in index order. Scores become order-preserving uint32 keys (-0.0 folded onto +0.0; -inf
// and a key of 0 mark an ineligible entry). Four passes find the k-th largest key one 8-bit digit at a time, each
// with a 256-bin LDS histogram and a workgroup prefix scan over the bins (no serial walk over the bins). Keys
// above that threshold are all kept; keys equal to it are kept lowest index first until k are taken.
#include "qsa_internal.h"

namespace qsa {

__device__ __forceinline__ uint32_t score_key(float f)
{
    if (f == -INFINITY) return 0u;
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;  // -0.0 ranks with +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the 256 threads of the workgroup; `total` receives the sum over all threads.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *sh_wave, uint32_t &total)
{
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) sh_wave[wave] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < 4; w++) {
        const uint32_t t = sh_wave[w];
        before += (w < wave) ? t : 0u;
        all += t;
    }
    __syncthreads();
    total = all;
    return before + x - v;
}

template <int KPT>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ scores, int32_t width, int32_t k,
                                                   int32_t *__restrict__ ids, int32_t *__restrict__ counts)
{
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh_wave[4];
    __shared__ uint32_t sh_digit, sh_remaining;
    __shared__ bool sh_whole;
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const float *src = scores + row * width;
    const int32_t i0 = tid * KPT;

    uint32_t key[KPT];
    uint32_t mine = 0;
#pragma unroll
    for (int e = 0; e < KPT; e++) {
        const int32_t idx = i0 + e;
        key[e] = idx < width ? score_key(src[idx]) : 0u;
        mine += key[e] != 0u;
    }
    uint32_t n_elig;
    block_exclusive_scan(mine, sh_wave, n_elig);
    const uint32_t kk = n_elig < (uint32_t)k ? n_elig : (uint32_t)k;

    uint32_t T, take_eq = 0;
    if (kk == 0) {
        T = 0xFFFFFFFFu;  // nothing is above it
    } else if (kk == n_elig) {
        T = 0u;           // every eligible key is above it
    } else {
        uint32_t prefix = 0, mask = 0, remaining = kk;
        bool done_early = false;
#pragma unroll 1
        for (int pass = 0; pass < 4; pass++) {
            const int shift = 24 - 8 * pass;
            hist[tid] = 0;
            __syncthreads();
#pragma unroll
            for (int e = 0; e < KPT; e++)
                if (key[e] != 0u && (key[e] & mask) == prefix) atomicAdd(&hist[(key[e] >> shift) & 255u], 1u);
            __syncthreads();
            // thread t looks at digit 255 - t: cum = number of matching keys whose digit is >= 255 - t
            const uint32_t v = hist[255 - tid];
            uint32_t tot;
            const uint32_t cum = block_exclusive_scan(v, sh_wave, tot) + v;
            if (cum >= remaining && cum - v < remaining) {
                sh_digit = 255u - (uint32_t)tid;
                sh_remaining = remaining - (cum - v);
                sh_whole = (remaining - (cum - v)) == v;   // the whole bin is taken
            }
            __syncthreads();
            prefix |= sh_digit << shift;
            mask |= 255u << shift;
            remaining = sh_remaining;
            const bool whole = sh_whole;
            __syncthreads();
            if (whole) {  // every key with this prefix is kept: keep all keys >= prefix, no tie to break
                done_early = true;
                break;
            }
        }
        if (done_early) {
            T = prefix == 0u ? 0u : prefix - 1u;
            take_eq = 0;
        } else {
            T = prefix;
            take_eq = remaining;
        }
    }

    // compaction in index order: keys > T, then the first take_eq keys == T
    uint32_t n_eq = 0;
#pragma unroll
    for (int e = 0; e < KPT; e++) n_eq += (key[e] != 0u && key[e] == T);
    uint32_t tot_eq;
    uint32_t eq_rank = block_exclusive_scan(n_eq, sh_wave, tot_eq);
    bool sel[KPT];
    uint32_t n_sel = 0;
#pragma unroll
    for (int e = 0; e < KPT; e++) {
        const bool eq = key[e] != 0u && key[e] == T;
        sel[e] = (key[e] != 0u && key[e] > T) || (eq && eq_rank < take_eq);
        eq_rank += eq;
        n_sel += sel[e];
    }
    uint32_t tot_sel;
    uint32_t at = block_exclusive_scan(n_sel, sh_wave, tot_sel);
    int32_t *dst = ids + row * k;
#pragma unroll
    for (int e = 0; e < KPT; e++)
        if (sel[e]) dst[at++] = i0 + e;
    for (int32_t jj = (int32_t)kk + tid; jj < k; jj += 256) dst[jj] = -1;
    if (tid == 0) counts[row] = (int32_t)kk;
}

}  // namespace qsa

using namespace qsa;

extern "C" size_t qsa_topk_scratch_bytes(int32_t n_rows, int32_t width, int32_t k)
{
    (void)n_rows; (void)width; (void)k;
    return 0;
}

extern "C" qsa_status qsa_topk(const float *scores, int32_t n_rows, int32_t width, int32_t k, int32_t *ids,
                               int32_t *counts, void *scratch, size_t scratch_bytes, qsa_stream_t stream)
{
    (void)scratch; (void)scratch_bytes;
    if (!scores || !ids || !counts) return QSA_ERR_NULL;
    if (n_rows < 0 || width < 0) return QSA_ERR_SHAPE;
    if (k < 1 || k > width) return QSA_ERR_RANGE;
    if (width > 256 * 64) return QSA_ERR_UNSUPPORTED;
    if (n_rows == 0) return QSA_OK;
    hipStream_t s = (hipStream_t)stream;
    dim3 grid(n_rows);
    const int kpt = (width + 255) / 256;
#define QSA_TOPK(K) topk_kernel<K><<<grid, 256, 0, s>>>(scores, width, k, ids, counts)
    if (kpt <= 1) QSA_TOPK(1);
    else if (kpt <= 2) QSA_TOPK(2);
    else if (kpt <= 4) QSA_TOPK(4);
    else if (kpt <= 8) QSA_TOPK(8);
    else if (kpt <= 16) QSA_TOPK(16);
    else if (kpt <= 32) QSA_TOPK(32);
    else QSA_TOPK(64);
#undef QSA_TOPK
    return launch_status();
}
