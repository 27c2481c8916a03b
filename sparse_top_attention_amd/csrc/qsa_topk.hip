// Radix top-k over block-score rows for gfx950.
//
// One workgroup of 64 * NW threads per row (4 waves up to 256 entries, else 16 for qsa_topk and 8 for the fused
// selection); thread t owns the KPT consecutive entries [t*KPT, t*KPT + KPT) so that the final compaction runs in
// index order. Scores become order-preserving uint32 keys (-0.0 folded onto +0.0; -inf and a key of 0 mark an
// ineligible entry). Up to four passes find the k-th largest key one 8-bit digit at a time, each
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

template <int KPT, int NW>
__global__ __launch_bounds__(64 * NW) void topk_kernel(const float *__restrict__ scores, int32_t width, int32_t k,
                                                   int32_t *__restrict__ ids, int32_t *__restrict__ counts)
{
    const int64_t row = blockIdx.x;
    const float *src = scores + row * width;
    const int32_t i0 = threadIdx.x * KPT;
    uint32_t key[KPT];
#pragma unroll
    for (int e = 0; e < KPT; e++) {
        const int32_t idx = i0 + e;
        key[e] = idx < width ? score_key(src[idx]) : 0u;
    }
    radix_topk<KPT, NW>(key, k, ids + row * k, counts + row);
}

// ------------------------------------------------------------------------------- fused block scores + top-k
// One workgroup of NW waves per (KV head g, row i) of a decode layer: the row's q heads of g are summed, every
// block's score qsum . index[g][b] is computed (the same arithmetic, in the same order, as the block-score kernel:
// 8-dim fmaf chains per lane, then a DPP sum over the D/8 lanes of a block) into LDS, and the radix top-k selects
// from them. The index rows are fetched in batches whose loads are all in flight before the first wait (16 steps of
// NW * BPS blocks), so a wide row (more than 256 blocks) takes 8 waves: twice the bytes in flight per batch of a
// 4-wave workgroup.
template <int D, int KPT, int NW>
__global__ __launch_bounds__(64 * NW) void select_kernel(const SelectArgs a)
{
    constexpr int LPB = D / 8, BPS = 64 / LPB;       // lanes per block, blocks per wave step
    constexpr int T = 64 * NW, SB = NW * BPS;         // threads, blocks per workgroup step
    static_assert(T >= D, "one thread per dim sums q");
    __shared__ float sqs[D];
    __shared__ float ssc[T * KPT];
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int32_t g = blockIdx.x, i = blockIdx.y;
    // Loads first, in the order their values are needed: the per-row words (lane 0 pos[i], lane 1 the pool index;
    // without row_pool lane 1 reads pos[i] too and the value is ignored) and the q rows of the sum, then the index
    // rows. Without row_pool the pool is known from the arguments alone, so the index loads do not wait for a
    // round trip.
    const bool mp = a.row_pool != nullptr;
    const int32_t words = *(lane == 1 && mp ? a.row_pool + i : a.pos + i);
    float qh[8];
    {
        const int d = tid < D ? tid : 0;
        const float *qd = a.q + ((int64_t)i * a.n_qh + g * a.G) * D + d;
#pragma unroll
        for (int h = 0; h < 8; h++) qh[h] = qd[(int64_t)(h < a.G ? h : a.G - 1) * D];
    }
    bool pool_ok = true;
    PoolArg P = a.pools[0];   // fixed argument offsets: read with the other arguments, no wait for the words
    if (mp) {
        const int32_t pidx = __builtin_amdgcn_readlane(words, 1);
        pool_ok = pidx >= 0 && pidx < a.n_pools;
        if (pool_ok && pidx != 0) P = a.pools[pidx];
    }
    const int32_t n_valid = pool_ok ? P.n_valid : 0;
    const int32_t stride = (P.capacity + QSA_BLOCK - 1) / QSA_BLOCK;

    const int rb = lane / LPB, s = lane % LPB;
    const float *idx_g = P.index + (int64_t)g * stride * D + 8 * s;
    const int32_t n_live = min(a.width, (int32_t)((n_valid + QSA_BLOCK - 1) / QSA_BLOCK));
    // batches of NST steps of SB blocks each. Loads are unconditional (a dead block reads block 0 and is zeroed
    // afterwards) so a whole batch is in flight before the first wait.
    constexpr int NST = 16;
    float rv[NST][8];
    auto load_step = [&](int32_t base, int st) {
        const int32_t b = base + st * SB + wave * BPS + rb;
        const float4 *src = reinterpret_cast<const float4 *>(idx_g + (int64_t)(b < n_live ? b : 0) * D);
        const float4 u = src[0], w = src[1];
        rv[st][0] = u.x; rv[st][1] = u.y; rv[st][2] = u.z; rv[st][3] = u.w;
        rv[st][4] = w.x; rv[st][5] = w.y; rv[st][6] = w.z; rv[st][7] = w.w;
    };
    // only blocks below n_live hold a score; the rest of the row is -inf without a load
    const int32_t b_end = min(T * KPT, (n_live + NST * SB - 1) / (NST * SB) * (NST * SB));
    if (b_end > 0) {
#pragma unroll
        for (int st = 0; st < NST; st++) load_step(0, st);
    }
    const int32_t p = __builtin_amdgcn_readlane(words, 0);
    for (int e = tid; e < T * KPT; e += T)
        if (e >= b_end) {
            ssc[e] = -INFINITY;
            if (a.scores && e < a.width) a.scores[((int64_t)i * a.n_kv + g) * a.width + e] = -INFINITY;
        }

    // qsum over the row's q heads of g, summed in head order (heads past G re-read the last head, not added)
    if (tid < D) {
        float acc = 0.f;
#pragma unroll
        for (int h = 0; h < 8; h++)
            if (h < a.G) acc += qh[h];
        sqs[tid] = acc;
    }
    __syncthreads();
    float qt[8];
#pragma unroll
    for (int e = 0; e < 8; e++) qt[e] = sqs[8 * s + e];
    // one batch of index rows in registers at a time: each step's registers take the next batch's rows as soon as
    // its score is done
#pragma unroll 1
    for (int32_t base = 0; base < b_end; base += NST * SB) {
        const int32_t next = base + NST * SB;
#pragma unroll
        for (int st = 0; st < NST; st++) {
            const int32_t b = base + st * SB + wave * BPS + rb;
            const bool live = b < n_live;
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) dot = fmaf(qt[e], live ? rv[st][e] : 0.f, dot);
            dot = group_sum<LPB>(dot);
            if (s == 0 && b < T * KPT) {
                const int64_t first = (int64_t)b * QSA_BLOCK;
                const float sc = (b < a.width && first <= p && first < n_valid) ? dot : -INFINITY;
                ssc[b] = sc;
                if (a.scores && b < a.width) a.scores[((int64_t)i * a.n_kv + g) * a.width + b] = sc;
            }
            if (next < b_end) load_step(next, st);
        }
    }
    __syncthreads();
    uint32_t key[KPT];
#pragma unroll
    for (int e = 0; e < KPT; e++) key[e] = score_key(ssc[tid * KPT + e]);   // past the width: -inf, key 0
    const int64_t row = (int64_t)i * a.n_kv + g;
    radix_topk<KPT, NW>(key, a.k, a.ids + row * a.k, a.counts + row);
}

}  // namespace qsa

using namespace qsa;

qsa_status qsa::topk_launch(const float *scores, int32_t n_rows, int32_t width, int32_t k, int32_t *ids,
                            int32_t *counts, hipStream_t s)
{
    dim3 grid(n_rows);
    const int kpt = (width + 1023) / 1024;
#define QSA_TOPK(K, W) topk_kernel<K, W><<<grid, 64 * W, 0, s>>>(scores, width, k, ids, counts)
    if (width <= 256) QSA_TOPK(1, 4);
    else if (kpt <= 1) QSA_TOPK(1, 16);
    else if (kpt <= 2) QSA_TOPK(2, 16);
    else if (kpt <= 4) QSA_TOPK(4, 16);
    else if (kpt <= 8) QSA_TOPK(8, 16);
    else QSA_TOPK(16, 16);
#undef QSA_TOPK
    return launch_status();
}

qsa_status qsa::select_launch(const SelectArgs &a, int32_t n_rows, int32_t n_kv, int32_t head_dim, hipStream_t s)
{
    if (a.scores && select_splits(a)) {
        // wide rows: the score rows in one launch spread over many CUs, then the top-k over them (the fused kernel
        // would stream each row's index rows through a single CU)
        const qsa_status st = select_scores_launch(a, n_rows, n_kv, head_dim, s);
        if (st != QSA_OK) return st;
        return topk_launch(a.scores, n_rows * n_kv, a.width, a.k, a.ids, a.counts, s);
    }
    dim3 grid(n_kv, n_rows);
    // up to 256 columns: 4 waves, one column per thread; wider rows: 8 waves, KPT = 1..32 columns per thread
    const int kpt = (a.width + 511) / 512;
#define QSA_SEL(DD, K, W) select_kernel<DD, K, W><<<grid, 64 * W, 0, s>>>(a)
#define QSA_SEL_D(DD)                                                                                               \
    do {                                                                                                          \
        if (a.width <= 256) QSA_SEL(DD, 1, 4);                                                                    \
        else if (kpt <= 1) QSA_SEL(DD, 1, 8);                                                                     \
        else if (kpt <= 2) QSA_SEL(DD, 2, 8);                                                                     \
        else if (kpt <= 4) QSA_SEL(DD, 4, 8);                                                                     \
        else if (kpt <= 8) QSA_SEL(DD, 8, 8);                                                                     \
        else if (kpt <= 16) QSA_SEL(DD, 16, 8);                                                                   \
        else QSA_SEL(DD, 32, 8);                                                                                  \
    } while (0)
    switch (head_dim) {
    case 64: QSA_SEL_D(64); break;
    case 128: QSA_SEL_D(128); break;
    default: QSA_SEL_D(256); break;
    }
#undef QSA_SEL_D
#undef QSA_SEL
    return launch_status();
}

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
    return topk_launch(scores, n_rows, width, k, ids, counts, (hipStream_t)stream);
}
