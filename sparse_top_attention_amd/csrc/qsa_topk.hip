// Radix top-k over block-score rows for gfx950.
//
// One workgroup of 64 * NW threads per row (4 waves up to 256 entries, else 16 for qsa_topk and 8 for the fused
// selection); thread t owns the KPT consecutive entries [t*KPT, t*KPT + KPT) so that the final compaction runs in
// index order. Scores become order-preserving uint32 keys (-0.0 folded onto +0.0; -inf and a key of 0 mark an
// ineligible entry). Up to four passes find the k-th largest key one 8-bit digit at a time, each
// with a 256-bin LDS histogram and a workgroup prefix scan over the bins (no serial walk over the bins). Keys
// above that threshold are all kept; keys equal to it are kept lowest index first until k are taken.
#include "qsa_radix.h"

namespace qsa {

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
    constexpr int DL = lane_dims<D>(), LPB = DL / 8, BPS = 64 / LPB;   // lanes per block, blocks per wave step
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
    const int32_t stride = ceil_div(P.capacity, QSA_BLOCK);

    const int rb = lane / LPB, s0 = lane % LPB;
    const bool sl = DL == D || 8 * s0 < D;   // the lane's 8 dims are dims of the row (else it adds zeros)
    const int s = sl ? s0 : 0;
    const float *idx_g = P.index + (int64_t)g * stride * D + 8 * s;
    const int32_t n_live = min(a.width, ceil_div(n_valid, QSA_BLOCK));
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
    for (int e = 0; e < 8; e++) qt[e] = sl ? sqs[8 * s + e] : 0.f;
    // one batch of index rows in registers at a time: each step's registers take the next batch's rows as soon as
    // its score is done
#pragma unroll 1
    for (int32_t base = 0; base < b_end; base += NST * SB) {
        const int32_t next = base + NST * SB;
#pragma unroll
        for (int st = 0; st < NST; st++) {
            const int32_t b = base + st * SB + wave * BPS + rb;
            const bool live = b < n_live && sl;
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) dot = fmaf(qt[e], live ? rv[st][e] : 0.f, dot);
            dot = group_sum<LPB>(dot);
            if (s0 == 0 && b < T * KPT) {
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
    case 192: QSA_SEL_D(192); break;
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
