// Radix top-k over one row of block scores held by a workgroup (the selection's arithmetic, shared by the top-k and
// selection kernels and by the chunk kernel's fused selection): order-preserving uint32 keys (-0.0 folded onto +0.0;
// -inf and a key of 0 mark an ineligible entry), up to four passes of 8-bit digits, each with a 256-bin LDS histogram
// and a prefix scan over the bins, then an index-order compaction. Keys above the k-th largest are all kept; keys
// equal to it are kept lowest index first until k are taken.
#pragma once

#include "qsa_internal.h"

namespace qsa {

__device__ __forceinline__ uint32_t score_key(float f)
{
    if (f == -INFINITY) return 0u;
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;  // -0.0 ranks with +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (a few cycles each, no LDS round trips): shifts
// by 1, 2, 4, 8 within each row of 16 lanes, then the last lane of row 0 / rows 0-1 is broadcast into the later rows.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x)
{
    int v = (int)x;
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1 and 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2 and 3
    return (uint32_t)v;
}

// Exclusive prefix sum over the NW waves of the workgroup; `total` receives the sum over all threads.
template <int NW>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *sh_wave, uint32_t &total)
{
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    const uint32_t x = wave_inclusive_scan(v);
    if (lane == 63) sh_wave[wave] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; w++) {
        const uint32_t t = sh_wave[w];
        before += (w < wave) ? t : 0u;
        all += t;
    }
    __syncthreads();
    total = all;
    return before + x - v;
}

// Top-k over one row of keys held KPT per thread (thread t owns entries [t KPT, t KPT + KPT)); writes the k ids
// (index order, -1 padded) and the count. Every thread of the 64 * NW-thread workgroup must call it.
template <int KPT, int NW>
__device__ __forceinline__ void radix_topk(const uint32_t (&key)[KPT], int32_t k, int32_t *__restrict__ dst,
                                           int32_t *__restrict__ count)
{
    static_assert(NW >= 4, "the 256 histogram bins are cleared one per thread");
    constexpr int NTH = 64 * NW;
    __shared__ uint32_t hist[2][256];
    __shared__ uint32_t sh_wave[NW];
    __shared__ uint32_t sh_digit, sh_remaining, sh_kk;
    __shared__ bool sh_whole, sh_all;
    const int tid = threadIdx.x;
    const int32_t i0 = tid * KPT;

    // The first digit pass counts every eligible key, so its histogram total is the eligible count: kk = min(count,
    // k) comes out of that pass, and when every eligible key is kept (or none exists) no threshold is needed.
    uint32_t prefix = 0, mask = 0, remaining = 0, kk = 0, T = 0, take_eq = 0;
    bool settled = false;
    if (tid < 256) hist[0][tid] = 0;
    __syncthreads();
    // Two histograms alternate (the next one is cleared while the current one fills), and one wave scans the 256
    // bins, so a pass costs two barriers.
#pragma unroll 1
    for (int pass = 0; pass < 4; pass++) {
        const int shift = 24 - 8 * pass;
        uint32_t *hc = hist[pass & 1];
#pragma unroll
        for (int e = 0; e < KPT; e++)
            if (key[e] != 0u && (key[e] & mask) == prefix) atomicAdd(&hc[(key[e] >> shift) & 255u], 1u);
        if (tid < 256) hist[(pass + 1) & 1][tid] = 0;
        __syncthreads();
        if (tid < 64) {
            // lane l holds digits 255 - 4l - e (e = 0..3), highest first; cum counts the matching keys whose digit
            // is at least the current one
            uint32_t c[4];
#pragma unroll
            for (int e = 0; e < 4; e++) c[e] = hc[255 - 4 * tid - e];
            const uint32_t lsum = (c[0] + c[1]) + (c[2] + c[3]);
            const uint32_t incl = wave_inclusive_scan(lsum);
            uint32_t rem = remaining;
            if (pass == 0) {
                const uint32_t n_elig = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
                rem = n_elig < (uint32_t)k ? n_elig : (uint32_t)k;
                if (tid == 0) {
                    sh_kk = rem;
                    sh_all = rem == n_elig;
                }
            }
            uint32_t cum = incl - lsum;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const uint32_t before = cum;
                cum += c[e];
                if (cum >= rem && before < rem) {
                    sh_digit = 255u - 4u * (uint32_t)tid - (uint32_t)e;
                    sh_remaining = rem - before;
                    sh_whole = (rem - before) == c[e];   // the whole bin is taken
                }
            }
        }
        __syncthreads();
        if (pass == 0) {
            kk = sh_kk;
            if (sh_all) {   // keep every eligible key: nothing (kk = 0) or everything is above the threshold
                T = kk == 0 ? 0xFFFFFFFFu : 0u;
                settled = true;
                break;
            }
        }
        prefix |= sh_digit << shift;
        mask |= 255u << shift;
        remaining = sh_remaining;
        if (sh_whole) {  // every key with this prefix is kept: keep all keys >= prefix, no tie to break
            T = prefix == 0u ? 0u : prefix - 1u;
            settled = true;
            break;
        }
    }
    if (!settled) {
        T = prefix;
        take_eq = remaining;
    }

    // compaction in index order: every key > T, then the first take_eq keys == T. One scan of the packed per-thread
    // counts (greater << 16 | equal; a row has at most 16,384 keys, so neither field carries) gives each thread the
    // number of greater and of equal keys before its own; the position of a kept key is the greater keys before it
    // plus the kept equal keys before it.
    uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
    for (int e = 0; e < KPT; e++) {
        n_gt += key[e] != 0u && key[e] > T;
        n_eq += key[e] != 0u && key[e] == T;
    }
    uint32_t tot;
    const uint32_t pre = block_exclusive_scan<NW>((n_gt << 16) | n_eq, sh_wave, tot);
    uint32_t gt_b = pre >> 16, eq_b = pre & 0xFFFFu;
#pragma unroll
    for (int e = 0; e < KPT; e++) {
        const bool gt = key[e] != 0u && key[e] > T, eq = key[e] != 0u && key[e] == T;
        if (gt || (eq && eq_b < take_eq)) dst[gt_b + (eq_b < take_eq ? eq_b : take_eq)] = i0 + e;
        gt_b += gt;
        eq_b += eq;
    }
    for (int32_t jj = (int32_t)kk + tid; jj < k; jj += NTH) dst[jj] = -1;
    if (tid == 0) *count = (int32_t)kk;
}

}  // namespace qsa
