// Decode-path kernels of libqsa for gfx950: block index, block scores, split-K chunk attention and the
// log-sum-exp merge. All four stream int8 codes / fp32 rows from HBM with 16-byte coalesced loads; per cell the
// work is a few hundred FMAs against 272 bytes, so HBM and the fp32 VALU are the ceilings. With 4 or more q heads
// per KV head at d = 128 the chunk kernel runs both of its products on the matrix cores (fp16 MFMA with exact K and V
// codes and two-term splits of q and p * v_scale), on the VALU otherwise.
//
// Lane layout shared by the index and chunk kernels ("cell x slice"): a cell's D dims are cut into D/16 slices of
// 16 dims (one 16-byte load of int8 codes), so a wave covers 64 / (D/16) cells per step; lane = cell_slot * LPC +
// slice. A slice never straddles a 64-dim scale group. The index kernel finishes its per-cell sums with a DPP sum
// over the LPC lanes of the cell; the chunk kernel finishes its G per-cell dot products with a reduce-scatter over
// those lanes, so that each (cell, head) logit ends in one lane.
#include "qsa_internal.h"
#include "qsa_radix.h"

#include <math.h>

#include <mutex>

namespace qsa {

constexpr float LOG2E = 1.4426950408889634f;

constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ void unpack16(const int4 w, float (&x)[16])
{
    const int32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
        x[4 * j + 0] = sbyte_f<0>(ws[j]);
        x[4 * j + 1] = sbyte_f<1>(ws[j]);
        x[4 * j + 2] = sbyte_f<2>(ws[j]);
        x[4 * j + 3] = sbyte_f<3>(ws[j]);
    }
}

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4v __attribute__((ext_vector_type(4)));

// Eight signed int8 codes (two dwords, byte j of the pair = element j) as exact fp16: the byte b + 128 is put under
// the fp16 exponent of 1024 (0x64 high byte, spacing 1), giving 1024 + 128 + b, and 1152 is subtracted.
__device__ __forceinline__ h8 codes_h8(const v2i w)
{
    h8 r;
    const h2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
    for (int q = 0; q < 2; q++) {
        const uint32_t u = (uint32_t)w[q] ^ 0x80808080u;
        const h2 a = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) + bias;
        const h2 b = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) + bias;
        r[4 * q] = a[0]; r[4 * q + 1] = a[1]; r[4 * q + 2] = b[0]; r[4 * q + 3] = b[1];
    }
    return r;
}

// Eight bytes of signed 4-bit code pairs (byte j: the codes of two adjacent dims of element j, the even dim in the
// low nibble) as two sets of exact fp16, the even dims and the odd dims (the nibble n ^ 8 under the exponent of
// 1024, minus 1032).
__device__ __forceinline__ void nibbles_h8(const v2i w, h8 &even, h8 &odd)
{
    const h2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
#pragma unroll
    for (int q = 0; q < 2; q++) {
        const uint32_t u = (uint32_t)w[q] ^ 0x88888888u;
        const uint32_t ev = u & 0x0F0F0F0Fu, od = (u >> 4) & 0x0F0F0F0Fu;
        const h2 e0 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, ev, 0x04010400u)) + bias;
        const h2 e1 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, ev, 0x04030402u)) + bias;
        const h2 o0 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, od, 0x04010400u)) + bias;
        const h2 o1 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, od, 0x04030402u)) + bias;
        even[4 * q] = e0[0]; even[4 * q + 1] = e0[1]; even[4 * q + 2] = e1[0]; even[4 * q + 3] = e1[1];
        odd[4 * q] = o0[0]; odd[4 * q + 1] = o0[1]; odd[4 * q + 2] = o1[0]; odd[4 * q + 3] = o1[1];
    }
}

// x = hi + lo with hi, lo fp16 (22 significant bits): hi is x with its float mantissa cut to 10 bits (exact in fp16
// when |x| is in fp16's normal range), lo the exact remainder rounded to fp16.
__device__ __forceinline__ void split_h2(const float x, _Float16 &hi, _Float16 &lo)
{
    const float xh = __uint_as_float(__float_as_uint(x) & 0xFFFFE000u);
    hi = (_Float16)xh;
    lo = (_Float16)(x - xh);
}

// Reduce-scatter over the LPC lanes of a cell (LPC = 4, 8 or 16, lane bits = s): every lane enters with NV partial
// values, value v belonging to slot v, and lane s leaves with the sums over the LPC lanes of slots s, s + LPC, ...
// in v[0], v[LPC], ... Stage m pairs the positions p and p | m: the lane whose bit m is set keeps slot p | m, the
// other slot p, each adding what its partner (bit m flipped, the bits above m equal: the quad swaps below 4, the
// 8- and 16-lane mirrors at 4 and 8) sends for it, and the result goes to position p.
template <int LPC, int NV>
__device__ __forceinline__ void reduce_scatter(float (&v)[NV], int s)
{
#pragma unroll
    for (int m = LPC / 2; m >= 1; m /= 2) {
        // the per-lane choice is a bit select on a lane mask held in a vector register (no scalar lane masks)
        const uint32_t hi = (s & m) ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int p = 0; p < NV; p++) {
            if ((p & m) || (p & (LPC - 1) & ~(2 * m - 1))) continue;   // not the low position of a live pair
            const uint32_t lo_b = __float_as_uint(v[p]), hi_b = __float_as_uint(v[p | m]);
            const float keep = __uint_as_float((hi_b & hi) | (lo_b & ~hi));
            const float send = __uint_as_float((lo_b & hi) | (hi_b & ~hi));
            float recv;
            if (m == 8) recv = dpp_f<DPP_ROW_MIRROR>(send);
            else if (m == 4) recv = dpp_f<DPP_ROW_HALF_MIRROR>(send);
            else if (m == 2) recv = dpp_f<DPP_QUAD_XOR2>(send);
            else recv = dpp_f<DPP_QUAD_XOR1>(send);
            v[p] = keep + recv;
        }
    }
}

// --------------------------------------------------------------------------------------------- block index
// index[g][b][:] = mean of the dequantised keys of block b's valid cells, computed by one wave.
template <int D>
__device__ __forceinline__ void block_mean(const int8_t *__restrict__ k, const float *__restrict__ ks, int32_t cap,
                                           int32_t n_valid, int32_t g, int32_t b, int32_t blk_stride,
                                           float *__restrict__ index)
{
    constexpr int LPC = D / 16, CPS = 64 / LPC, STEPS = QSA_BLOCK / CPS, NG = D / QSA_GROUP;
    const int lane = threadIdx.x % 64, r = lane / LPC, s = lane % LPC, grp = (16 * s) / QSA_GROUP;
    const int32_t c0 = b * QSA_BLOCK;
    float acc[16];
#pragma unroll
    for (int e = 0; e < 16; e++) acc[e] = 0.f;
#pragma unroll
    for (int st = 0; st < STEPS; st++) {
        const int32_t c = c0 + st * CPS + r;
        if (c < n_valid) {
            const int64_t cell = (int64_t)g * cap + c;
            const int4 w = *reinterpret_cast<const int4 *>(k + cell * D + 16 * s);
            const float sc = ks[cell * NG + grp];
            float x[16];
            unpack16(w, x);
#pragma unroll
            for (int e = 0; e < 16; e++) acc[e] = fmaf(sc, x[e], acc[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < 16; e++) acc[e] = strided_sum<LPC>(acc[e]);
    int32_t nb = n_valid - c0;
    nb = nb < 0 ? 0 : (nb > QSA_BLOCK ? QSA_BLOCK : nb);
    const float inv = nb > 0 ? 1.0f / (float)nb : 0.f;
    if (r == 0) {
        float4 *dst = reinterpret_cast<float4 *>(index + ((int64_t)g * blk_stride + b) * D + 16 * s);
#pragma unroll
        for (int j = 0; j < 4; j++)
            dst[j] = make_float4(acc[4 * j] * inv, acc[4 * j + 1] * inv, acc[4 * j + 2] * inv, acc[4 * j + 3] * inv);
    }
}

// One wave per (block, KV head).
template <int D>
__global__ __launch_bounds__(64) void block_index_kernel(const int8_t *__restrict__ k, const float *__restrict__ ks,
                                                         int32_t cap, int32_t n_valid, int32_t b_first,
                                                         int32_t blk_stride, float *__restrict__ index)
{
    block_mean<D>(k, ks, cap, n_valid, blockIdx.y, b_first + blockIdx.x, blk_stride, index);
}

// ----------------------------------------------------------------------------------------------------- append
// Write side of the int8 pool: row i encodes its new K and V rows into cell cells[i] of pool pools[row_pool[i]]
// (every KV head), then the index rows of the blocks holding new cells are recomputed. One wave per (row, KV head);
// in the encoder lane l holds dim l + 64 t of scale group t, so a group's absmax is one wave-wide max.
struct AppendArgs {
    PoolArg pools[QSA_MAX_POOLS];
    int32_t n_pools;
    const int32_t *row_pool;
    const float *k_new;
    const float *v_new;
    const int32_t *cells;
    int32_t n_kv;
};

__device__ __forceinline__ bool append_row(const AppendArgs &a, int32_t i, PoolArg &P, int32_t &c)
{
    const int32_t pidx = a.row_pool ? a.row_pool[i] : 0;
    if (pidx < 0 || pidx >= a.n_pools) return false;
    P = a.pools[pidx];
    c = a.cells[i];
    return c >= 0 && c < P.n_valid;
}

// Encode of one 64-dim group held one value per lane, with QMAX = 2^(bits-1) - 1 (127 for int8, 7 for the 4-bit V
// of a K8V4 pool): amax = max |x|, scale = amax / QMAX, code = rint(x * (QMAX / amax)) clamped to [-QMAX, QMAX]
// (all fp32, correctly rounded); amax = 0 gives zeros. 4-bit codes are packed two per byte, dim 2j in the low
// nibble: the even lane of each pair takes its odd partner's code and writes the byte.
template <int D, int VB>
__global__ __launch_bounds__(64) void append_encode_kernel(const AppendArgs a)
{
    constexpr int NG = D / QSA_GROUP;
    const int lane = threadIdx.x;
    const int32_t i = blockIdx.x, g = blockIdx.y;
    PoolArg P;
    int32_t c;
    if (!append_row(a, i, P, c)) return;
    const int64_t src = ((int64_t)i * a.n_kv + g) * D, dst = (int64_t)g * P.capacity + c;
#pragma unroll
    for (int which = 0; which < 2; which++) {
        const bool v4 = which == 1 && VB == 4;
        const float qmax = v4 ? 7.0f : 127.0f;
        const float *x = (which ? a.v_new : a.k_new) + src;
        int8_t *codes = const_cast<int8_t *>(which ? P.v : P.k) + dst * (v4 ? D / 2 : D);
        float *scales = const_cast<float *>(which ? P.vs : P.ks) + dst * NG;
        float xv[NG];
#pragma unroll
        for (int t = 0; t < NG; t++) xv[t] = x[QSA_GROUP * t + lane];
#pragma unroll
        for (int t = 0; t < NG; t++) {
            const float amax = group_max<64>(fabsf(xv[t]));
            float code = 0.f;
            if (amax > 0.f) code = fminf(fmaxf(rintf(xv[t] * (qmax / amax)), -qmax), qmax);
            const int32_t ci = (int32_t)code;
            if (v4) {
                const int32_t hi = __shfl_xor(ci, 1);
                if (!(lane & 1)) codes[(QSA_GROUP * t + lane) / 2] = (int8_t)((ci & 15) | ((hi & 15) << 4));
            } else {
                codes[QSA_GROUP * t + lane] = (int8_t)ci;
            }
            if (lane == 0) scales[t] = amax / qmax;
        }
    }
}

template <int D>
__global__ __launch_bounds__(64) void append_index_kernel(const AppendArgs a)
{
    const int32_t i = blockIdx.x, g = blockIdx.y;
    PoolArg P;
    int32_t c;
    if (!append_row(a, i, P, c) || !P.index) return;
    block_mean<D>(P.k, P.ks, P.capacity, P.n_valid, g, c / QSA_BLOCK, (P.capacity + QSA_BLOCK - 1) / QSA_BLOCK,
                  const_cast<float *>(P.index));
}

// -------------------------------------------------------------------------------------------- block scores
// scores[i][g][b] = qsum[i][g] . index[g][b]. Lanes: LPB = D/8 lanes per block (8 dims each), BPS = 64/LPB blocks
// per step, NSTEP steps per wave; the index rows are loaded once and reused for every query row.
template <int D>
__global__ __launch_bounds__(64) void block_scores_kernel(const float *__restrict__ q, const int32_t *__restrict__ pos,
                                                          int32_t n_rows, int32_t n_qh, int32_t n_kv, int32_t G,
                                                          const float *__restrict__ index, int32_t blk_stride,
                                                          int32_t n_valid, int32_t n_blocks,
                                                          float *__restrict__ scores)
{
    constexpr int LPB = D / 8, BPS = 64 / LPB, NSTEP = 4;
    const int lane = threadIdx.x, rb = lane / LPB, s = lane % LPB;
    const int32_t g = blockIdx.y;
    const int32_t bw = blockIdx.x * (BPS * NSTEP);
    float rv[NSTEP][8];
    int32_t bidx[NSTEP];
    // unconditional loads (a dead block reads block 0, then counts as zeros), so all are issued before any wait
    const int32_t n_live = min(n_blocks, (int32_t)(((int64_t)n_valid + QSA_BLOCK - 1) / QSA_BLOCK));
#pragma unroll
    for (int st = 0; st < NSTEP; st++) {
        const int32_t b = bw + st * BPS + rb;
        bidx[st] = b;
        const bool live = b < n_live;
        const float4 *src =
            reinterpret_cast<const float4 *>(index + ((int64_t)g * blk_stride + (live ? b : 0)) * D + 8 * s);
        const float4 u = src[0], w = src[1];
        rv[st][0] = u.x; rv[st][1] = u.y; rv[st][2] = u.z; rv[st][3] = u.w;
        rv[st][4] = w.x; rv[st][5] = w.y; rv[st][6] = w.z; rv[st][7] = w.w;
#pragma unroll
        for (int e = 0; e < 8; e++) rv[st][e] = live ? rv[st][e] : 0.f;
    }
    for (int32_t i0 = 0; i0 < n_rows; i0 += 8) {
        const int nr = min(8, n_rows - i0);
        float qt[8][8];
#pragma unroll
        for (int rr = 0; rr < 8; rr++) {
#pragma unroll
            for (int e = 0; e < 8; e++) qt[rr][e] = 0.f;
            if (rr < nr) {
                // the row's G heads in head order; all 8 loads are issued together (heads past G re-read the last)
                float4 u[8], w[8];
#pragma unroll
                for (int h = 0; h < 8; h++) {
                    const float4 *src = reinterpret_cast<const float4 *>(
                        q + ((int64_t)(i0 + rr) * n_qh + g * G + (h < G ? h : G - 1)) * D + 8 * s);
                    u[h] = src[0];
                    w[h] = src[1];
                }
#pragma unroll
                for (int h = 0; h < 8; h++) {
                    if (h < G) {
                        qt[rr][0] += u[h].x; qt[rr][1] += u[h].y; qt[rr][2] += u[h].z; qt[rr][3] += u[h].w;
                        qt[rr][4] += w[h].x; qt[rr][5] += w[h].y; qt[rr][6] += w[h].z; qt[rr][7] += w[h].w;
                    }
                }
            }
        }
#pragma unroll
        for (int rr = 0; rr < 8; rr++) {
            if (rr >= nr) break;
            const int32_t i = i0 + rr;
            const int32_t p = pos[i];
#pragma unroll
            for (int st = 0; st < NSTEP; st++) {
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < 8; e++) dot = fmaf(qt[rr][e], rv[st][e], dot);
                dot = group_sum<LPB>(dot);
                const int32_t b = bidx[st];
                const int64_t first = (int64_t)b * QSA_BLOCK;
                if (s == 0 && b < n_blocks)
                    scores[((int64_t)i * n_kv + g) * n_blocks + b] = (first <= p && first < n_valid) ? dot : -INFINITY;
            }
        }
    }
}

// The score rows of a whole decode window in one launch, for the two-launch selection of wide rows (the fused kernel
// streams a row's index through one CU): the block-score kernel's arithmetic, in the same order, over every pool of
// the window. Workgroup (block range, g, p) scores the rows whose row_pool is p against pool p's index rows; pool 0's
// workgroups also write -inf rows for the rows whose pool index is out of range, which then select nothing.
constexpr int SCORE_STEPS = 2;   // steps of blocks per wave of the score-row kernel (more waves beat fewer, wider)

template <int D>
__global__ __launch_bounds__(64) void select_scores_kernel(const SelectArgs a)
{
    // one wave per (tile of BPS * NSTEP blocks, KV head g, row i): the row's words and q rows, then the tile's index
    // rows of the row's pool (the block-score arithmetic: 8-dim fmaf chains per lane, a DPP sum over the block's
    // lanes); blocks past the pool's valid cells, and every block of a row whose pool index is out of range, are -inf
    constexpr int LPB = D / 8, BPS = 64 / LPB, NSTEP = SCORE_STEPS;
    const int lane = threadIdx.x, rb = lane / LPB, s = lane % LPB;
    const int32_t g = blockIdx.y, i = blockIdx.z;
    const int32_t bw = blockIdx.x * (BPS * NSTEP);
    const int32_t rp = a.row_pool ? a.row_pool[i] : 0;
    const int32_t p = a.pos[i];
    // the row's G q heads of g summed in head order (heads past G re-read the last one and are not added)
    float4 u[8], w[8];
#pragma unroll
    for (int h = 0; h < 8; h++) {
        const float4 *src = reinterpret_cast<const float4 *>(
            a.q + ((int64_t)i * a.n_qh + g * a.G + (h < a.G ? h : a.G - 1)) * D + 8 * s);
        u[h] = src[0];
        w[h] = src[1];
    }
    const bool bad = rp < 0 || rp >= a.n_pools;
    const PoolArg P = a.pools[bad ? 0 : rp];
    const int32_t stride = (P.capacity + QSA_BLOCK - 1) / QSA_BLOCK;
    const int32_t n_live = bad ? 0 : min(a.width, (int32_t)(((int64_t)P.n_valid + QSA_BLOCK - 1) / QSA_BLOCK));
    float rv[NSTEP][8];
#pragma unroll
    for (int st = 0; st < NSTEP; st++) {
        const int32_t b = bw + st * BPS + rb;
        const bool live = b < n_live;
        const float4 *src =
            reinterpret_cast<const float4 *>(P.index + ((int64_t)g * stride + (live ? b : 0)) * D + 8 * s);
        const float4 x = src[0], y = src[1];
        rv[st][0] = x.x; rv[st][1] = x.y; rv[st][2] = x.z; rv[st][3] = x.w;
        rv[st][4] = y.x; rv[st][5] = y.y; rv[st][6] = y.z; rv[st][7] = y.w;
#pragma unroll
        for (int e = 0; e < 8; e++) rv[st][e] = live ? rv[st][e] : 0.f;
    }
    float qt[8];
#pragma unroll
    for (int e = 0; e < 8; e++) qt[e] = 0.f;
#pragma unroll
    for (int h = 0; h < 8; h++) {
        if (h < a.G) {
            qt[0] += u[h].x; qt[1] += u[h].y; qt[2] += u[h].z; qt[3] += u[h].w;
            qt[4] += w[h].x; qt[5] += w[h].y; qt[6] += w[h].z; qt[7] += w[h].w;
        }
    }
#pragma unroll
    for (int st = 0; st < NSTEP; st++) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++) dot = fmaf(qt[e], rv[st][e], dot);
        dot = group_sum<LPB>(dot);
        const int32_t b = bw + st * BPS + rb;
        const int64_t first = (int64_t)b * QSA_BLOCK;
        if (s == 0 && b < a.width)
            a.scores[((int64_t)i * a.n_kv + g) * a.width + b] = (b < n_live && first <= p) ? dot : -INFINITY;
    }
}

// ---------------------------------------------------------------------------------------- chunk attention
struct ChunkArgs {
    const float *q;
    const int32_t *pos;
    const int32_t *row_pool;
    const int32_t *ids;
    const int32_t *counts;
    float *m_out;
    float *l_out;
    float *o_out;
    uint8_t *empty_out;
    PoolArg pools[QSA_MAX_POOLS];
    int32_t n_pools;
    int32_t n_qh;
    int32_t n_kv;
    int32_t G;
    int32_t topk;
    int32_t bpc;
    int32_t n_chunks;
    int32_t max_chunks;
    float qscale;  // sm_scale * log2(e): logits are kept in base-2 units inside the kernel
    // fused selection (scores != NULL): every workgroup takes the top-k of its (row, KV head)'s score row of `width`
    // columns itself (ids and counts are not read); the first chunk's workgroup stores them in ids_out and
    // counts_out when those are given
    int32_t width;
    const float *scores;
    int32_t *ids_out;
    int32_t *counts_out;
};

// One workgroup of CW waves per CW / wpc consecutive chunks of one (KV head g, row i), wpc waves per chunk; every
// wave handles all G q heads of the KV head, so each K/V byte is converted once for all of them. A chunk's blocks
// are cut into pieces of PC cells; its sub-wave s takes pieces s, s + wpc, ... and keeps a running (max, sum,
// output) per head over them.
//
// q . k runs in the "cell x slice" layout (LPC lanes per cell, 16 dims each), and a reduce-scatter over the cell's
// lanes leaves the logit of head s in the cell's lane s, so the softmax work runs once per (cell, head). p . v runs
// in a "lane owns dims" layout: the piece's V codes go from HBM straight into the wave's LDS (global_load_lds,
// 16-byte chunks swizzled by cell), and ds_read_b64_tr_b8 hands each lane 8 cells of one dim per read; p * v_scale
// per (cell, scale group, head) is written to LDS by the head's lane of the cell and read back as a broadcast. Each
// lane then owns D/64 output dims of every head, so nothing is summed across lanes at the end. In the MFMA form
// (MPV below) a lane of 16-lane group G4 holds one head's logits of 8 cells, which are its A operand for p . v, the
// transposing reads of the same cells are the B operands, and a lane owns one dim of 4 heads per 16-dim tile. The
// waves of a chunk are combined through LDS with a log-sum-exp rescale (a one-wave chunk stores its partial
// directly).
constexpr int CW = 4;

//
// VB is the V code width: 8 (int8) or 4 (K8V4: two signed 4-bit codes per byte, dim 2j in the low nibble). A V row
// is RB = D * VB / 8 bytes; a 16-byte chunk of it holds DPC = 128 / VB dims, so a transposing read gives each lane
// 8 / VB dims of 8 cells and a lane makes NT = DPL * VB / 8 reads per 8 cells. The K side is the same for both.
template <int D, int G, int VB, int WPC, bool FZ>
__device__ __forceinline__ void attn_chunk_body(const ChunkArgs &a)
{
    static_assert(VB == 8 || (VB == 4 && D >= 128), "K8V4 needs head_dim >= 128");
    constexpr int PC = D <= 128 ? 32 : 16;           // cells per piece
    constexpr int LPC = D / 16, CPS = 64 / LPC, STEPS = PC / CPS, NG = D / QSA_GROUP;
    constexpr int DPL = D / 64;                      // output dims per lane
    constexpr int RB = D * VB / 8;                   // V bytes per cell row
    constexpr int NPB = 8 / VB;                      // V codes per byte
    constexpr int NT = DPL / NPB;                    // transposing reads per lane per 8 cells
    constexpr int DPC = 16 * NPB;                    // dims per 16-byte chunk
    constexpr int CPG = QSA_GROUP / DPC;             // 16-byte chunks per scale group
    constexpr int SUBS = 4 / NG;                     // 16-lane subgroups per scale group in the p . v layout
    constexpr int CHUNKS = RB / 16;                  // 16-byte chunks per V row
    constexpr int SWZ = (CHUNKS < 8 ? CHUNKS : 8) - 1;
    constexpr int VCH = PC * RB / 1024;              // 1 KB global -> LDS copies per piece
    constexpr int GP = (G + 3) & ~3;                 // p * v_scale row padded to float4s
    static_assert(CPG == SUBS * NT && VCH * 1024 == PC * RB, "p . v lane layout");
    // Both products on the matrix cores (int8 K and V, d = 128, 4 or more heads; MPV): the logits of the piece's 32
    // cells as S[cell][head] = K q^T per 64-dim scale group, and per 16-dim output tile O[head][dim] +=
    // P[head][cell] V[cell][dim], all with v_mfma_f32_16x16x32_f16 (heads padded to 16 rows). K and V codes are exact
    // in fp16; q and p * v_scale go in as two fp16 terms (hi + lo, 22 significant bits) scaled by powers of two that
    // keep them in fp16's range, both terms accumulating into the same fp32 tile.
    constexpr bool MPV = D == 128 && G >= 4;
    constexpr int NTL = D / 16;                      // 16-dim output tiles (MPV)
    static_assert(!MPV || (NG == 2 && PC == 32), "MFMA form: d = 128, 32-cell pieces");
    // MFMA form: output tile t's lane jl holds dim 16 t + jl (int8 V); with 4-bit V a transposing read of 16-byte
    // chunk c gives dims 32 c + 2 jl (low nibbles, tile 2 c) and 32 c + 2 jl + 1 (high nibbles, tile 2 c + 1)
    auto tile_dim = [](int t, int l) { return VB == 8 ? 16 * t + l : 32 * (t >> 1) + 2 * l + (t & 1); };
    __shared__ __align__(16) int8_t sv[CW][PC * RB]; // the wave's V piece: [cell][RB], chunk c of row r at c ^ swizzle(r)
    // p * v_scale rows [cell][group][head] of the VALU p . v (the MFMA form keeps p in registers)
    __shared__ __align__(16) float sp[CW][MPV ? 4 : PC * NG * GP];
    __shared__ float sm[CW][G], sl[CW][G];
    __shared__ __align__(16) float so[CW][G + (MPV ? 1 : 0)][D];   // MPV: row G takes the padding heads' stores
    // MPV's V swizzle: the 8 rows of one transposing read (cells 4 G4 + e and 16 + 4 G4 + e) land on 8 distinct
    // 16-byte positions
    auto mswz = [](int c) { return (c + 4 * (c >> 4)) & SWZ; };
    __shared__ __align__(16) float sq[G * D];        // the G q rows of (row i, KV head g)
    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int r = lane / LPC, s = lane % LPC, grp_s = s / (LPC / NG);
    const int G4 = lane >> 4, jl = lane & 15;
    const int grp_v = G4 / SUBS, sub_v = G4 % SUBS;  // the p . v lane's scale group and subgroup
    // wave -> (chunk j of the workgroup's CW / wpc chunks, sub-wave sub of the chunk's wpc waves)
    constexpr int wpc = WPC, cpw = CW / WPC;
    const int sub = wave % wpc;
    const int32_t j0c = blockIdx.x * cpw;                 // the workgroup's first chunk
    const int32_t j = j0c + wave / wpc, g = blockIdx.y, i = blockIdx.z;
    const bool chunk_ok = j < a.n_chunks;                 // the last workgroup may hold fewer chunks
    const int32_t h0 = g * G;

    // Prologue: the workgroup's G q rows (one 16-byte load per thread), then the per-row words in one vector load
    // (lane 0 pos[i], lane 1 the pool index, lane 2 the block count; a missing row_pool or id list reads pos[i]
    // instead, a valid word whose value is then ignored) and the id list, so one round trip brings them all. The q
    // rows go through LDS: every wave needs all of them, and one copy per workgroup keeps them off the load-return
    // path that the K and V bytes take. The pool's fields follow.
    constexpr int QV4 = G * D / 4, QPT = (QV4 + 64 * CW - 1) / (64 * CW);
    float4 qld[QPT];
    {
        const float4 *qsrc = reinterpret_cast<const float4 *>(a.q + ((int64_t)i * a.n_qh + h0) * D);
#pragma unroll
        for (int u = 0; u < QPT; u++) {
            const int e = tid + 64 * CW * u;
            qld[u] = qsrc[e < QV4 ? e : 0];
        }
    }
    const int64_t row_kv = (int64_t)i * a.n_kv + g;
    constexpr bool fz = FZ;                               // fused selection: a.scores holds the score rows
    const bool sel = a.ids != nullptr || fz, mp = a.row_pool != nullptr;
    const int32_t *p_pidx = mp ? a.row_pool + i : a.pos + i;
    const int32_t *p_cnt = sel && !fz ? a.counts + row_kv : a.pos + i;
    const int32_t *blist = sel && !fz ? a.ids + row_kv * a.topk : a.pos + i;
    const int32_t words = *(lane == 1 ? p_pidx : (lane == 2 ? p_cnt : a.pos + i));
    const int32_t idv = blist[sel && !fz && lane < a.topk ? lane : 0];   // k <= 64: the whole id list, one per lane
    // fused selection: the score row's keys, one column per thread up to 256 columns, else 4 consecutive columns
    // per thread (rows of up to 1,024 columns)
    __shared__ int32_t s_ids[FUSED_TOPK_MAX_K];
    __shared__ int32_t s_cnt;
    uint32_t key[4];
    const bool one_key = a.width <= 64 * CW;
    if (fz) {
        const float *srow = a.scores + row_kv * a.width;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int32_t c = one_key ? (e == 0 ? tid : a.width) : 4 * tid + e;
            key[e] = c < a.width ? score_key(srow[c]) : 0u;
        }
    }
#pragma unroll
    for (int u = 0; u < QPT; u++) {
        const int e = tid + 64 * CW * u;
        if (e < QV4) reinterpret_cast<float4 *>(sq)[e] = qld[u];
    }
    __syncthreads();
    int32_t cnt_fz = 0;
    if (fz) {
        // the same top-k as the selection kernels (the result is unique: the k largest keys, ties to the lower
        // column, in column order), into LDS; the first chunk's workgroup also stores it
        if (one_key) {
            const uint32_t key1[1] = {key[0]};
            radix_topk<1, CW>(key1, a.topk, s_ids, &s_cnt);
        } else {
            radix_topk<4, CW>(key, a.topk, s_ids, &s_cnt);
        }
        __syncthreads();
        cnt_fz = __builtin_amdgcn_readfirstlane(s_cnt);
        if (blockIdx.x == 0) {
            if (a.ids_out)
                for (int e = tid; e < a.topk; e += 64 * CW) a.ids_out[row_kv * a.topk + e] = s_ids[e];
            if (a.counts_out && tid == 0) a.counts_out[row_kv] = cnt_fz;
        }
    }
    float qv[G][16];
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float4 *src = reinterpret_cast<const float4 *>(sq + h * D + 16 * s);
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
            const float4 u = src[jj];
            qv[h][4 * jj + 0] = u.x;
            qv[h][4 * jj + 1] = u.y;
            qv[h][4 * jj + 2] = u.z;
            qv[h][4 * jj + 3] = u.w;
        }
    }
    // MFMA form: q as B operands of the logits' products, lane (G4, jl): head jl (0 for the padding heads past G),
    // dims 64 gi + 16 G4 + 8 ks + e, times 2^sqe (per head: its largest |q| times 2^sqe stays below 2^14) as hi + lo
    // fp16; qsh = sm_scale log2(e) 2^-sqe undoes the scale on the logits
    h8 qb[NG][2][2];   // [scale group][k step][hi, lo]
    float qsh = 0.f;
    // (made on the wave's first piece, after its loads are issued, so that this work overlaps their latency)
    auto make_qb = [&]() {
        float qx[NG][16];
        float qmax = 0.f;
        const int hq = jl < G ? jl : G - 1;
#pragma unroll
        for (int gi = 0; gi < NG; gi++) {
            const float4 *src = reinterpret_cast<const float4 *>(sq + hq * D + 64 * gi + 16 * G4);
#pragma unroll
            for (int jj = 0; jj < 4; jj++) {
                const float4 u = src[jj];
                const float uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    qx[gi][4 * jj + e] = jl < G ? uu[e] : 0.f;
                    qmax = fmaxf(qmax, fabsf(qx[gi][4 * jj + e]));
                }
            }
        }
        qmax = max32(max16(qmax));
        const int sqe = 14 - __builtin_amdgcn_frexp_expf(qmax);
        qsh = __builtin_amdgcn_ldexpf(a.qscale, -sqe);
#pragma unroll
        for (int gi = 0; gi < NG; gi++)
#pragma unroll
            for (int ks = 0; ks < 2; ks++)
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    _Float16 hi, lo;
                    split_h2(__builtin_amdgcn_ldexpf(qx[gi][8 * ks + e], sqe), hi, lo);
                    qb[gi][ks][0][e] = hi;
                    qb[gi][ks][1][e] = lo;
                }
    };
    bool qready = false;
    const int32_t posi = __builtin_amdgcn_readlane(words, 0);
    const int32_t cnt_raw = fz ? cnt_fz : __builtin_amdgcn_readlane(words, 2);
    bool pool_ok = true;
    PoolArg P = a.pools[0];   // fixed argument offsets: read with the other arguments, no wait for the words
    if (mp) {
        const int32_t pidx = __builtin_amdgcn_readlane(words, 1);
        pool_ok = pidx >= 0 && pidx < a.n_pools;
        if (pool_ok && pidx != 0) P = a.pools[pidx];
    }
    const int32_t limit = pool_ok ? min(P.n_valid - 1, posi) : -1;  // visible cells: c <= limit
    const int32_t cnt = cnt_raw < 0 ? 0 : (cnt_raw > a.topk ? a.topk : cnt_raw);
    const int32_t base = sel ? cnt / a.n_chunks : a.bpc, rem = sel ? cnt % a.n_chunks : 0;
    const int32_t n_blk = chunk_ok ? base + (j < rem ? 1 : 0) : 0;
    const int32_t first = j * base + (j < rem ? j : rem);

    // after the logits' reduce-scatter lane (r, s) holds heads s, s + LPC, ... (HPL slots) of its cell; the running
    // max and sum of head h live in the lanes of slot h, the output accumulators in every lane
    constexpr int HPL = (G + LPC - 1) / LPC, NV = HPL * LPC;
    float mrun[HPL], lpart[HPL], o[G][DPL];
#pragma unroll
    for (int k = 0; k < HPL; k++) {
        mrun[k] = -INFINITY;
        lpart[k] = 0.f;
    }
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int t = 0; t < DPL; t++) o[h][t] = 0.f;
    // MFMA form: tile T's accumulator; lane (G4, jl) holds dim 16 T + jl of heads 4 G4 .. 4 G4 + 3, in units of
    // 2^-srun (srun only decreases, so a rescale never grows the accumulators)
    f4v oacc[NTL];
#pragma unroll
    for (int t = 0; t < NTL; t++) oacc[t] = f4v{0.f, 0.f, 0.f, 0.f};
    int32_t srun = 1000;

    const int8_t *kbase = P.k + (int64_t)g * P.capacity * D + 16 * s;
    const int8_t *vbase = P.v + (int64_t)g * P.capacity * RB;
    const float *ksbase = P.ks + (int64_t)g * P.capacity * NG + grp_s;
    const float *vsbase = P.vs + (int64_t)g * P.capacity * NG;
    const int8_t *kmu = P.k + (int64_t)g * P.capacity * D;   // MFMA form: K and key scales of KV head g
    const float *ksm = P.ks + (int64_t)g * P.capacity * NG;
    int8_t *svw = sv[wave];
    constexpr int PPB = QSA_BLOCK / PC;              // pieces per block

    for (int32_t pc = sub; pc < n_blk * PPB; pc += wpc) {
        const int32_t t_blk = first + pc / PPB;
        const int32_t b = !sel ? t_blk
                                : fz ? __builtin_amdgcn_readfirstlane(s_ids[t_blk])
                                     : (a.topk <= 64 ? __builtin_amdgcn_readlane(idv, t_blk) : blist[t_blk]);
        // negative id, or no visible valid cell in the piece (64-bit: ids past the pool may be huge)
        if (b < 0 || (int64_t)b * QSA_BLOCK + (pc % PPB) * PC > limit) continue;
        const int32_t cb = b * QSA_BLOCK + (pc % PPB) * PC;

        if constexpr (MPV) {
            // ---- loads: the K rows as A operands (lane (G4, jl): cell 16 ct + jl, dims 64 gi + 16 G4 .. + 15), the
            // key and value scales of the lane's logit cells 16 ct + 4 G4 + e, the V piece into LDS
            // (64-bit bases of the piece in scalar registers, 32-bit lane offsets from them; cells past the limit
            // read the last visible cell)
            int4 kq[2][NG];
            float2 ksv[2][4], vsv[2][4];
            const int32_t lr = limit - cb;   // >= 0: the piece holds a visible cell
            const int8_t *kp = kmu + (int64_t)cb * D;
            const float *ksp = ksm + (int64_t)cb * NG, *vsp = vsbase + (int64_t)cb * NG;
            const int8_t *vp = vbase + (int64_t)cb * RB;
#pragma unroll
            for (int ct = 0; ct < 2; ct++) {
                const uint32_t ck = min(16 * ct + jl, lr);
#pragma unroll
                for (int gi = 0; gi < NG; gi++)
                    kq[ct][gi] = *reinterpret_cast<const int4 *>(kp + (ck * D + 64 * gi + 16 * G4));
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const uint32_t cs = min(16 * ct + 4 * G4 + e, lr);
                    ksv[ct][e] = *reinterpret_cast<const float2 *>(reinterpret_cast<const char *>(ksp) + cs * 8u);
                    vsv[ct][e] = *reinterpret_cast<const float2 *>(reinterpret_cast<const char *>(vsp) + cs * 8u);
                }
            }
#pragma unroll
            for (int q = 0; q < VCH; q++) {
                const int slot = 64 * q + lane, cell = slot / CHUNKS, pch = slot % CHUNKS;
                const uint32_t c = min(cell, lr);
                load_lds16(vp + (c * RB + 16 * (pch ^ mswz(cell))), lds_addr(svw + 1024 * q));
            }
            __builtin_amdgcn_sched_barrier(0);   // every copy is in flight before the logits start
            if (!qready) {
                make_qb();
                qready = true;
            }

            // ---- logits: S[cell][head] per scale group on the matrix cores (both q terms into one tile), then
            // t = sum over groups of k_scale * S in base-2 units; lane (G4, jl) ends with head jl's logits of cells
            // 16 ct + 4 G4 + e (masked past the limit)
            float t[2][4];
            float mb = -INFINITY;
#pragma unroll
            for (int ct = 0; ct < 2; ct++) {
                f4v sacc[NG];
#pragma unroll
                for (int gi = 0; gi < NG; gi++) {
                    const h8 k0 = codes_h8(v2i{kq[ct][gi].x, kq[ct][gi].y});
                    const h8 k1 = codes_h8(v2i{kq[ct][gi].z, kq[ct][gi].w});
                    f4v acc = {0.f, 0.f, 0.f, 0.f};
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, qb[gi][0][0], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, qb[gi][1][0], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, qb[gi][0][1], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, qb[gi][1][1], acc, 0, 0, 0);
                    sacc[gi] = acc;
                }
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const bool vis = cb + 16 * ct + 4 * G4 + e <= limit;
                    const float x = fmaf(ksv[ct][e].y, sacc[1][e], ksv[ct][e].x * sacc[0][e]) * qsh;
                    t[ct][e] = vis ? x : -INFINITY;
                    mb = fmaxf(mb, t[ct][e]);
                }
            }
            // ---- running max of head jl over the piece (the 4 lane groups), p = 2^(t - max)
            mb = max32(max16(mb));                // the piece holds a visible cell, so mb is finite
            const float mnew = fmaxf(mrun[0], mb);
            const float alpha = __builtin_amdgcn_exp2f(mrun[0] - mnew);  // 0 on the first piece
            mrun[0] = mnew;
            lpart[0] *= alpha;
#pragma unroll
            for (int ct = 0; ct < 2; ct++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    t[ct][e] = __builtin_amdgcn_exp2f(t[ct][e] - mnew);   // masked cells: 2^-inf = 0
                    lpart[0] += t[ct][e];
                }

            // ---- the piece's power-of-two scale: 2^snew times its largest |v_scale| (visible cells) stays below
            // 2^14; srun only decreases, and the accumulators take the change with the heads' rescale
            float vmax = 0.f;
#pragma unroll
            for (int ct = 0; ct < 2; ct++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const bool vis = cb + 16 * ct + 4 * G4 + e <= limit;
                    vmax = fmaxf(vmax, vis ? fmaxf(fabsf(vsv[ct][e].x), fabsf(vsv[ct][e].y)) : 0.f);
                }
            vmax = max32(max16(vmax));
            const int32_t snew = __builtin_amdgcn_readfirstlane(min(srun, 14 - __builtin_amdgcn_frexp_expf(vmax)));
            const int32_t dsh = snew - srun;   // <= 0
            const bool fresh = srun == 1000;   // the accumulators are still 0
            srun = snew;
            // rescale, when some head's max or the scale moved (a wave-uniform test): head h's factor is in lane h;
            // lane (G4, jl) holds heads 4 G4 + e, and heads past G (padding rows) get 0
            float ah[G];
            bool moved = dsh != 0;
#pragma unroll
            for (int h = 0; h < G; h++) {
                ah[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), h));
                moved = moved || ah[h] != 1.f;
            }
            if (!fresh && moved) {
                float fac[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int h = 0; h < G; h++) {
                    const float f = __builtin_amdgcn_ldexpf(ah[h], dsh);
                    if (h < 4) fac[h] = G4 == 0 ? f : fac[h];
                    else fac[h - 4] = G4 == 1 ? f : fac[h - 4];
                }
#pragma unroll
                for (int tt = 0; tt < NTL; tt++)
#pragma unroll
                    for (int e = 0; e < 4; e++) oacc[tt][e] *= fac[e];
            }

            // ---- p . v: A operands are the lane's own p values (head jl; element 4 ct + e = cell 16 ct + 4 G4 + e)
            // times v_scale of each group and 2^snew, as hi + lo fp16 (masked cells 0: their v_scale may be
            // anything); the B operands come from transposing reads whose 8 rows are those same cells
            h8 ahi[NG], alo[NG];
#pragma unroll
            for (int e8 = 0; e8 < 8; e8++) {
                const int ct = e8 >> 2, e = e8 & 3;
                const bool vis = cb + 16 * ct + 4 * G4 + e <= limit;
#pragma unroll
                for (int gi = 0; gi < NG; gi++) {
                    const float x = vis ? __builtin_amdgcn_ldexpf(t[ct][e] * (gi ? vsv[ct][e].y : vsv[ct][e].x), snew) : 0.f;
                    _Float16 hi, lo;
                    split_h2(x, hi, lo);
                    ahi[gi][e8] = hi;
                    alo[gi][e8] = lo;
                }
            }
            __builtin_amdgcn_s_waitcnt(0);   // the V piece has landed (this wave's copies)
            const int i8 = jl >> 1;
            const int vcell = 4 * G4 + (i8 & 3) + 16 * (i8 >> 2);
            if constexpr (VB == 8) {
#pragma unroll
                for (int tt = 0; tt < NTL; tt++) {
                    const h8 bv = codes_h8(__builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (QSA_LDS v2i *)(svw + vcell * RB + 16 * (tt ^ mswz(vcell)) + 8 * (jl & 1))));
                    oacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[tt / (NTL / NG)], bv, oacc[tt], 0, 0, 0);
                    oacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[tt / (NTL / NG)], bv, oacc[tt], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int c = 0; c < CHUNKS; c++) {
                    h8 bv0, bv1;
                    nibbles_h8(__builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                   (QSA_LDS v2i *)(svw + vcell * RB + 16 * (c ^ mswz(vcell)) + 8 * (jl & 1))),
                               bv0, bv1);
                    const int t0 = 2 * c, t1 = 2 * c + 1;
                    oacc[t0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[t0 / (NTL / NG)], bv0, oacc[t0], 0, 0, 0);
                    oacc[t1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[t1 / (NTL / NG)], bv1, oacc[t1], 0, 0, 0);
                    oacc[t0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[t0 / (NTL / NG)], bv0, oacc[t0], 0, 0, 0);
                    oacc[t1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[t1 / (NTL / NG)], bv1, oacc[t1], 0, 0, 0);
                }
            }
        } else {
            // ---- loads: K slices and scales into registers, the V piece into LDS
            int4 kw[STEPS];
            float ksc[STEPS], vsc[STEPS][NG];
#pragma unroll
            for (int st = 0; st < STEPS; st++) {
                const int32_t c = min(cb + st * CPS + r, limit);
                kw[st] = *reinterpret_cast<const int4 *>(kbase + (int64_t)c * D);
                ksc[st] = ksbase[(int64_t)c * NG] * a.qscale;   // sm_scale * log2(e) rides on the key scale
                const float *vsrc = vsbase + (int64_t)c * NG;   // all NG group scales of the cell, one load
                if constexpr (NG == 4) {
                    const float4 u = *reinterpret_cast<const float4 *>(vsrc);
                    vsc[st][0] = u.x; vsc[st][1] = u.y; vsc[st][2] = u.z; vsc[st][3] = u.w;
                } else if constexpr (NG == 2) {
                    const float2 u = *reinterpret_cast<const float2 *>(vsrc);
                    vsc[st][0] = u.x; vsc[st][1] = u.y;
                } else {
                    vsc[st][0] = vsrc[0];
                }
            }
#pragma unroll
            for (int q = 0; q < VCH; q++) {
                const int slot = 64 * q + lane, cell = slot / CHUNKS, pch = slot % CHUNKS;
                const int32_t c = min(cb + cell, limit);
                load_lds16(vbase + (int64_t)c * RB + 16 * (pch ^ (cell & SWZ)), lds_addr(svw + 1024 * q));
            }
            __builtin_amdgcn_sched_barrier(0);   // every copy is in flight before the logits start

            // ---- logits (base-2 units), masked past the limit: the G dot products of the lane's 16 dims, then a
            // reduce-scatter over the cell's lanes, so each (cell, head) logit is finished in one lane only
            float lg[STEPS][HPL];
#pragma unroll
            for (int st = 0; st < STEPS; st++) {
                const bool vis = cb + st * CPS + r <= limit;
                float x[16];
                unpack16(kw[st], x);
                float d[NV];
#pragma unroll
                for (int h = 0; h < NV; h++) {
                    float dot = 0.f;
                    if (h < G) {
#pragma unroll
                        for (int e = 0; e < 16; e++) dot = fmaf(qv[h < G ? h : 0][e], x[e], dot);
                    }
                    d[h] = dot * ksc[st];
                }
                reduce_scatter<LPC, NV>(d, s);
#pragma unroll
                for (int k = 0; k < HPL; k++) lg[st][k] = vis ? d[LPC * k] : -INFINITY;
            }

            // ---- running max per head over the piece's cells (lanes of one slot), p = 2^(logit - max); the output
            // accumulators take every head's rescale, read from the head's slot lane
            float alpha[HPL];
#pragma unroll
            for (int k = 0; k < HPL; k++) {
                float mb = lg[0][k];
#pragma unroll
                for (int st = 1; st < STEPS; st++) mb = fmaxf(mb, lg[st][k]);
                mb = strided_max<LPC>(mb);            // the piece holds a visible cell, so mb is finite
                const float mnew = fmaxf(mrun[k], mb);
                alpha[k] = __builtin_amdgcn_exp2f(mrun[k] - mnew);  // 0 on the first piece
                mrun[k] = mnew;
                lpart[k] *= alpha[k];
#pragma unroll
                for (int st = 0; st < STEPS; st++) {
                    const float p = __builtin_amdgcn_exp2f(lg[st][k] - mnew);   // masked cells: 2^-inf = 0
                    lpart[k] += p;
                    lg[st][k] = p;
                }
            }
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float ah = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[h / LPC]), h % LPC));
#pragma unroll
                for (int t = 0; t < DPL; t++) o[h][t] *= ah;
            }
            // p * v_scale per (cell, scale group, head) to LDS, written by the head's slot lane of each cell; masked
            // cells have p = 0 but their v_scale may be anything (even NaN): their entries are zeroed
#pragma unroll
            for (int st = 0; st < STEPS; st++) {
                const bool vis = cb + st * CPS + r <= limit;
#pragma unroll
                for (int k = 0; k < HPL; k++) {
                    const int h = s + LPC * k;
                    if (h < G) {
#pragma unroll
                        for (int gi = 0; gi < NG; gi++) sp[wave][((st * CPS + r) * NG + gi) * GP + h] = vis ? lg[st][k] * vsc[st][gi] : 0.f;
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0);   // the V piece has landed and the p rows are written (this wave only)

            // ---- o[h][dim] += sum over cells of (p * v_scale)[cell][h] * v[cell][dim]. Each cell's p * v_scale row
            // feeds only G * DPL FMAs, so the rows are read PWD cells ahead (a ring of registers) and the next 8-cell
            // block's transposing V reads are issued half a block early: the LDS latency stays behind the FMAs.
            const int i8 = jl >> 1, hh = jl & 1;
            constexpr int PWD = 3;                           // p * v_scale rows in flight
            constexpr int GR = (G + 3) / 4;                  // float4 reads per row (heads past G are not read)
            auto read_row = [&](int c, float4 (&dst)[GR]) {
                const float *prow = &sp[wave][(c * NG + grp_v) * GP];
#pragma unroll
                for (int u = 0; u < GR; u++) dst[u] = *reinterpret_cast<const float4 *>(prow + 4 * u);
            };
            auto read_v = [&](int co, v2i (&dst)[NT]) {
#pragma unroll
                for (int t = 0; t < NT; t++) {
                    const int lc = CPG * grp_v + sub_v + SUBS * t;   // logical 16-byte chunk of the lane's dims
                    const int cell = 8 * co + i8;
                    dst[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (QSA_LDS v2i *)(svw + cell * RB + 16 * (lc ^ (cell & SWZ)) + 8 * hh));
                }
            };
            float4 ring[PWD][GR];
            v2i vb[2][NT];
            read_v(0, vb[0]);
#pragma unroll
            for (int c = 0; c < PWD - 1; c++) read_row(c, ring[c]);
#pragma unroll
            for (int c = 0; c < PC; c++) {
                const int co = c / 8, ci = c % 8;
                if (c + PWD - 1 < PC) read_row(c + PWD - 1, ring[(c + PWD - 1) % PWD]);
                if (ci == 4 && co + 1 < PC / 8) read_v(co + 1, vb[(co + 1) & 1]);
                float pw[4 * GR];
#pragma unroll
                for (int u = 0; u < GR; u++) {
                    pw[4 * u] = ring[c % PWD][u].x; pw[4 * u + 1] = ring[c % PWD][u].y;
                    pw[4 * u + 2] = ring[c % PWD][u].z; pw[4 * u + 3] = ring[c % PWD][u].w;
                }
#pragma unroll
                for (int t = 0; t < NT; t++) {
                    const int32_t word = ci < 4 ? vb[co & 1][t][0] : vb[co & 1][t][1];
#pragma unroll
                    for (int n = 0; n < NPB; n++) {
                        // signed field of VB bits at bit 8 * (ci & 3) + VB * n
                        const float x = (float)((word << (32 - VB - 8 * (ci & 3) - VB * n)) >> (32 - VB));
#pragma unroll
                        for (int h = 0; h < G; h++) o[h][NPB * t + n] = fmaf(pw[h], x, o[h][NPB * t + n]);
                    }
                }
            }
        }
    }

    // the sum of a head over its lanes: the cell's slot lanes, or in the MFMA form the head's 4 lane groups; either
    // way lane h (< G) then holds head h's max and sum in slot 0
#pragma unroll
    for (int k = 0; k < HPL; k++) lpart[k] = MPV ? strided_sum<16>(lpart[k]) : strided_sum<LPC>(lpart[k]);
    if constexpr (WPC == 1) {
        // one wave per chunk: its partial is the chunk's, stored straight from registers (no LDS fold, no barrier;
        // the same values the fold would produce, since a single term's weight is 2^0 = 1)
        if (!chunk_ok) return;
        const int64_t row0 = ((int64_t)i * a.n_qh + h0) * a.max_chunks + j;
        // a chunk without a visible cell ran no piece, so its accumulators are still 0
        if constexpr (MPV) {
#pragma unroll
            for (int t = 0; t < NTL; t++) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int h = 4 * G4 + e;
                    if (h < G)
                        a.o_out[(row0 + (int64_t)h * a.max_chunks) * D + tile_dim(t, jl)] =
                            __builtin_amdgcn_ldexpf(oacc[t][e], -srun);
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < NT; t++) {
#pragma unroll
                for (int n = 0; n < NPB; n++) {
                    const int d = DPC * (CPG * grp_v + sub_v + SUBS * t) + NPB * jl + n;
#pragma unroll
                    for (int h = 0; h < G; h++)
                        a.o_out[(row0 + (int64_t)h * a.max_chunks) * D + d] = o[h][NPB * t + n];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < HPL; k++) {
            const int h = lane + LPC * k;   // lanes 0 .. LPC - 1 (the first cell's) hold every head once
            if (lane < LPC && h < G) {
                const int64_t idx = row0 + (int64_t)h * a.max_chunks;
                const bool empty = mrun[k] == -INFINITY;
                a.m_out[idx] = empty ? -INFINITY : mrun[k] * LN2;
                a.l_out[idx] = empty ? 0.f : lpart[k];
                a.empty_out[idx] = empty ? 1 : 0;
            }
        }
        return;
    }

    // ---- hand the wave's partial to LDS: the first cell's slot lanes the maxima and sums, every lane its own dims
    // of o
#pragma unroll
    for (int k = 0; k < HPL; k++) {
        const int h = lane + LPC * k;
        if (lane < LPC && h < G) {
            sm[wave][h] = mrun[k];
            sl[wave][h] = lpart[k];
        }
    }
    if constexpr (MPV) {
#pragma unroll
        for (int t = 0; t < NTL; t++) {
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int h = 4 * G4 + e;
                so[wave][h < G ? h : G][tile_dim(t, jl)] = __builtin_amdgcn_ldexpf(oacc[t][e], -srun);
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < NT; t++) {
#pragma unroll
            for (int n = 0; n < NPB; n++) {
                const int d = DPC * (CPG * grp_v + sub_v + SUBS * t) + NPB * jl + n;
#pragma unroll
                for (int h = 0; h < G; h++) so[wave][h][d] = o[h][NPB * t + n];
            }
        }
    }
    __syncthreads();

    // combine the wpc waves of each chunk: M = max m_w, out = sum e^(m_w - M) o_w (waves without a cell have
    // m_w = -inf). A thread takes four consecutive dims of one (chunk, head), so their weights are computed once and
    // the values move as 16-byte LDS reads and stores; every LDS value a round needs is read before the arithmetic,
    // which runs without branches. The (m, l, empty) of the chunks' G heads are written by the first cpw * G threads.
    constexpr int n_out4 = cpw * G * D / 4;   // float4 outputs
    constexpr int ROUNDS = (n_out4 + 64 * CW - 1) / (64 * CW);
    float hm[CW], hl[CW];
    {
        const int cc = tid < cpw * G ? tid / G : 0, h = tid < cpw * G ? tid % G : 0;
#pragma unroll
        for (int k = 0; k < CW; k++) {
            const int w = min(cc * wpc + k, CW - 1);
            hm[k] = k < wpc ? sm[w][h] : -INFINITY;
            hl[k] = sl[w][h];
        }
    }
    auto combine = [](const float (&mw)[CW], const float (&xw)[CW], float &M) {
        M = mw[0];
#pragma unroll
        for (int w = 1; w < CW; w++) M = fmaxf(M, mw[w]);
        float num = 0.f;
#pragma unroll
        for (int w = 0; w < CW; w++) {
            const float t = fmaf(__builtin_amdgcn_exp2f(mw[w] - M), xw[w], num);
            num = mw[w] != -INFINITY ? t : num;
        }
        return M != -INFINITY ? num : 0.f;
    };
#pragma unroll
    for (int r0 = 0; r0 < ROUNDS; r0++) {
        const int q4 = tid + 64 * CW * r0;
        const int qq = min(q4, n_out4 - 1);
        const int cc = qq / (G * D / 4), rem4 = qq % (G * D / 4), h = rem4 / (D / 4), d4 = rem4 % (D / 4);
        float mw[CW];
        float4 ow[CW];
#pragma unroll
        for (int k = 0; k < CW; k++) {
            const int w = min(cc * wpc + k, CW - 1);   // k >= wpc is masked
            mw[k] = k < wpc ? sm[w][h] : -INFINITY;
            ow[k] = *reinterpret_cast<const float4 *>(&so[w][h][4 * d4]);
        }
        float M = mw[0];
#pragma unroll
        for (int k = 1; k < CW; k++) M = fmaxf(M, mw[k]);
        float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int k = 0; k < CW; k++) {
            const float wk = __builtin_amdgcn_exp2f(mw[k] - M);
            const bool live = mw[k] != -INFINITY;
            num.x = live ? fmaf(wk, ow[k].x, num.x) : num.x;
            num.y = live ? fmaf(wk, ow[k].y, num.y) : num.y;
            num.z = live ? fmaf(wk, ow[k].z, num.z) : num.z;
            num.w = live ? fmaf(wk, ow[k].w, num.w) : num.w;
        }
        if (M == -INFINITY) num = make_float4(0.f, 0.f, 0.f, 0.f);
        if (q4 < n_out4 && j0c + cc < a.n_chunks)
            *reinterpret_cast<float4 *>(
                a.o_out + (((int64_t)i * a.n_qh + h0 + h) * a.max_chunks + j0c + cc) * D + 4 * d4) = num;
    }
    if (tid < cpw * G && j0c + tid / G < a.n_chunks) {
        float M;
        const float L = combine(hm, hl, M);
        const int64_t idx = ((int64_t)i * a.n_qh + h0 + tid % G) * a.max_chunks + j0c + tid / G;
        const bool empty = M == -INFINITY;
        a.m_out[idx] = empty ? -INFINITY : M * LN2;
        a.l_out[idx] = L;
        a.empty_out[idx] = empty ? 1 : 0;
    }
}

// The chunk kernel from given ids (or dense), and the decode layer's form that takes each row's top-k itself from its
// score row: two kernels, so that neither carries the other's code.
template <int D, int G, int VB, int WPC>
__global__ __launch_bounds__(64 * CW) void attn_chunk_kernel(const ChunkArgs a)
{
    attn_chunk_body<D, G, VB, WPC, false>(a);
}

template <int D, int G, int VB, int WPC>
__global__ __launch_bounds__(64 * CW) void attn_chunk_select_kernel(const ChunkArgs a)
{
    attn_chunk_body<D, G, VB, WPC, true>(a);
}

// ---------------------------------------------------------------------------------------------------- merge
// One workgroup of NW waves per (row, q head); each wave takes a contiguous 1/NW of the active chunks. A wave reads
// the (m, l, empty) of up to 64 of its chunks at once, one chunk per lane, so the max M over the non-empty chunks,
// the weights e^(m_j - M) and the weighted sum of l_j take one round of loads and a few cross-lane steps. The o_j
// rows (lanes own D/64 consecutive dims) are loaded U chunks at a time with every load in flight before the first
// use, and are added in chunk order with the weight read from the chunk's lane. Empty chunks are skipped by select,
// never multiplied (their l and o may hold anything). The waves' parts are combined through LDS.
template <int D, int NW, int U, int DS>
__global__ __launch_bounds__(64 * NW) void attn_merge_kernel(const float *__restrict__ m, const float *__restrict__ l,
                                                         const float *__restrict__ o, const uint8_t *__restrict__ em,
                                                         int32_t max_chunks, int32_t n_chunks,
                                                         const int32_t *__restrict__ n_active, int32_t n_qh,
                                                         float *__restrict__ out, float *__restrict__ lse)
{
    constexpr int DW = D / DS;                    // dims of this workgroup's slice of the row
    static_assert(DW % 64 == 0 || DW == 32, "lanes own whole dims");
    // a slice of 32 dims: lanes 0-31 take the even chunks of each row step, lanes 32-63 the odd ones
    constexpr int CPL = DW < 64 ? 2 : 1;          // chunks per row step
    constexpr int VPL = DW < 64 ? 1 : DW / 64;
    const int sub = CPL == 2 ? (int)(threadIdx.x % 64) / 32 : 0, dl = (int)(threadIdx.x % 64) % (64 / CPL);
    __shared__ float sM[NW], sL[NW];
    __shared__ float sO[NW][DW];
    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int32_t row = blockIdx.x;               // = i * n_qh + h
    const int32_t dsl = blockIdx.y;               // dim slice: dims [dsl * DW, dsl * DW + DW)
    o += dsl * DW;
    out += dsl * DW;
    const int32_t i = row / n_qh;
    int32_t na = n_active ? n_active[i] : n_chunks;
    na = na < 0 ? 0 : (na > n_chunks ? n_chunks : na);
    const int32_t j0 = (int32_t)(((int64_t)na * wave) / NW), j1 = (int32_t)(((int64_t)na * (wave + 1)) / NW);
    const int64_t base = (int64_t)row * max_chunks;
    const int32_t nq = j1 - j0;                   // chunks of this wave
    const int32_t jlast = n_chunks - 1;           // n_chunks >= 1: every clamped index is in bounds
    auto clamp_j = [&](int32_t jj) { return jj < jlast ? jj : jlast; };

    // the first batch (up to 64 chunks, one per lane, and the first U row steps of o), all loads before any wait
    float ov0[U][VPL];
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int c = CPL * u + sub;
        const float *src = o + (base + clamp_j(j0 + (c < nq ? c : 0))) * D + VPL * dl;
#pragma unroll
        for (int e = 0; e < VPL; e++) ov0[u][e] = src[e];
    }
    const int32_t jc = clamp_j(j0 + (lane < nq ? lane : 0));
    const float mv0 = m[base + jc], lv0 = l[base + jc];
    const uint8_t ev0 = em[base + jc];
    __builtin_amdgcn_sched_barrier(0);            // keep every load above ahead of the first wait
    const bool live0 = lane < nq && !ev0;

    // pass 1: M over the wave's non-empty chunks
    float M = live0 ? mv0 : -INFINITY;
    for (int32_t jb = j0 + 64; jb < j1; jb += 64) {
        const int32_t jj = jb + lane;
        const int32_t jcb = jj < j1 ? jj : jb;
        const float mv = m[base + jcb];
        const bool live = jj < j1 && !em[base + jcb];
        M = live ? fmaxf(M, mv) : M;
    }
    M = group_max<64>(M);
    if (lane == 0) sM[wave] = M;
    __syncthreads();
    M = sM[0];
#pragma unroll
    for (int w = 1; w < NW; w++) M = fmaxf(M, sM[w]);

    // pass 2: L = sum e^(m_j - M) l_j and acc = sum e^(m_j - M) o_j, in chunk order; the first batch of 64 chunks
    // uses the preloaded values
    float L = 0.f, acc[VPL];
#pragma unroll
    for (int e = 0; e < VPL; e++) acc[e] = 0.f;
    auto add_rows = [&](const float (&ov)[U][VPL], int32_t c0, int32_t nb, int32_t flag, float wgt) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            if constexpr (CPL == 1) {
                const int c = c0 + u;
                if (c < nb && __builtin_amdgcn_readlane(flag, c)) {
                    const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), c));
#pragma unroll
                    for (int e = 0; e < VPL; e++) acc[e] = fmaf(wu, ov[u][e], acc[e]);
                }
            } else {
                // the even and the odd chunk of the step; a lane takes its half's, and skips it by select when it
                // is past the batch or empty (an empty chunk's row may hold anything)
                const int c = c0 + 2 * u;
                if (c < nb) {
                    const int c1 = c + 1 < 64 ? c + 1 : 63;
                    const bool l0 = __builtin_amdgcn_readlane(flag, c) != 0;
                    const bool l1 = c + 1 < nb && __builtin_amdgcn_readlane(flag, c1) != 0;
                    const float w0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), c));
                    const float w1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), c1));
                    const float t = fmaf(sub ? w1 : w0, ov[u][0], acc[0]);
                    acc[0] = (sub ? l1 : l0) ? t : acc[0];
                }
            }
        }
    };
    auto batch = [&](int32_t jb, float mv, float lv, bool live, bool first) {
        const int32_t nb = min(64, j1 - jb);
        const float wgt = live ? expf(mv - M) : 0.f;
        L += group_sum<64>(live ? wgt * lv : 0.f);
        const int32_t flag = live ? 1 : 0;
        int32_t c0 = 0;
        if (first) {
            add_rows(ov0, 0, nb, flag, wgt);
            c0 = CPL * U;
        }
        for (; c0 < nb; c0 += CPL * U) {
            float ov[U][VPL];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const float *src = o + (base + jb + min(c0 + CPL * u + sub, nb - 1)) * D + VPL * dl;
#pragma unroll
                for (int e = 0; e < VPL; e++) ov[u][e] = src[e];
            }
            add_rows(ov, c0, nb, flag, wgt);
        }
    };
    if (M != -INFINITY && nq > 0) {
        batch(j0, mv0, lv0, live0, true);
        for (int32_t jb = j0 + 64; jb < j1; jb += 64) {
            const int32_t jcb = jb + lane < j1 ? jb + lane : jb;
            const float mv = m[base + jcb], lv = l[base + jcb];
            const bool live = jb + lane < j1 && !em[base + jcb];
            batch(jb, mv, lv, live, false);
        }
    }
    if (lane == 0) sL[wave] = L;
    if constexpr (CPL == 2) acc[0] = sum32(acc[0]);   // the even and odd chunks' sums of dim dl
#pragma unroll
    for (int e = 0; e < VPL; e++)
        if (sub == 0) sO[wave][VPL * dl + e] = acc[e];
    __syncthreads();
    if (wave == 0) {
        float Lt = sL[0];
#pragma unroll
        for (int w = 1; w < NW; w++) Lt += sL[w];
        const bool none = M == -INFINITY;
#pragma unroll
        for (int e = 0; e < VPL; e++) {
            const int d = VPL * dl + e;
            float num = sO[0][d];
#pragma unroll
            for (int w = 1; w < NW; w++) num += sO[w][d];
            if (sub == 0) out[(int64_t)row * D + d] = none ? 0.f : num / Lt;
        }
        if (lse && lane == 0 && dsl == 0) lse[row] = none ? -INFINITY : M + logf(Lt);
    }
}

}  // namespace qsa

using namespace qsa;

// ======================================================================================== C entry points
extern "C" qsa_status qsa_block_index(const qsa_pool *pool, qsa_dims dims, int32_t cell_begin, int32_t cell_end,
                                      float *index, qsa_stream_t stream)
{
    qsa_status st = check_dims(dims);
    if (st != QSA_OK) return st;
    if ((st = check_pool(pool, false)) != QSA_OK) return st;
    if (!index) return QSA_ERR_NULL;
    if (cell_begin < 0 || cell_end < cell_begin || cell_end > pool->capacity) return QSA_ERR_RANGE;
    if (cell_end == cell_begin) return QSA_OK;
    const int32_t b0 = cell_begin / QSA_BLOCK, b1 = ceil_div(cell_end, QSA_BLOCK);
    const int32_t stride = ceil_div(pool->capacity, QSA_BLOCK);
    dim3 grid(b1 - b0, dims.n_kv_heads);
    hipStream_t s = (hipStream_t)stream;
    switch (dims.head_dim) {
    case 64: block_index_kernel<64><<<grid, 64, 0, s>>>(pool->k, pool->k_scale, pool->capacity, pool->n_valid, b0, stride, index); break;
    case 128: block_index_kernel<128><<<grid, 64, 0, s>>>(pool->k, pool->k_scale, pool->capacity, pool->n_valid, b0, stride, index); break;
    default: block_index_kernel<256><<<grid, 64, 0, s>>>(pool->k, pool->k_scale, pool->capacity, pool->n_valid, b0, stride, index); break;
    }
    return launch_status();
}

extern "C" qsa_status qsa_kv_append(const qsa_pool *pools, int32_t n_pools, const int32_t *row_pool, qsa_dims dims,
                                    const float *k_new, const float *v_new, const int32_t *cells, int32_t n_rows,
                                    qsa_stream_t stream)
{
    qsa_status st = check_dims(dims);
    if (st != QSA_OK) return st;
    if (!pools || !k_new || !v_new || !cells) return QSA_ERR_NULL;
    if (n_rows < 0 || n_pools <= 0) return QSA_ERR_SHAPE;
    if (n_pools > QSA_MAX_POOLS) return QSA_ERR_UNSUPPORTED;
    for (int32_t p = 0; p < n_pools; p++)
        if ((st = check_pool(&pools[p], true)) != QSA_OK) return st;
    const int vb = common_v_bits(pools, n_pools, dims.head_dim);
    if (!vb) return QSA_ERR_UNSUPPORTED;
    if (n_rows == 0) return QSA_OK;
    if (n_rows > 65535) return QSA_ERR_UNSUPPORTED;
    AppendArgs a{};
    for (int32_t p = 0; p < n_pools; p++)
        a.pools[p] = PoolArg{pools[p].k, pools[p].k_scale, pools[p].v, pools[p].v_scale, pools[p].capacity,
                             pools[p].n_valid, pools[p].index};
    a.n_pools = row_pool ? n_pools : 1;
    a.row_pool = row_pool; a.k_new = k_new; a.v_new = v_new; a.cells = cells; a.n_kv = dims.n_kv_heads;
    dim3 grid(n_rows, dims.n_kv_heads);
    hipStream_t s = (hipStream_t)stream;
    switch (dims.head_dim * (vb == 4 ? -1 : 1)) {
    case 64: append_encode_kernel<64, 8><<<grid, 64, 0, s>>>(a); break;
    case 128: append_encode_kernel<128, 8><<<grid, 64, 0, s>>>(a); break;
    case -128: append_encode_kernel<128, 4><<<grid, 64, 0, s>>>(a); break;
    case -256: append_encode_kernel<256, 4><<<grid, 64, 0, s>>>(a); break;
    default: append_encode_kernel<256, 8><<<grid, 64, 0, s>>>(a); break;
    }
    switch (dims.head_dim) {
    case 64: append_index_kernel<64><<<grid, 64, 0, s>>>(a); break;
    case 128: append_index_kernel<128><<<grid, 64, 0, s>>>(a); break;
    default: append_index_kernel<256><<<grid, 64, 0, s>>>(a); break;
    }
    return launch_status();
}

qsa_status qsa::select_scores_launch(const SelectArgs &a, int32_t n_rows, int32_t n_kv, int32_t head_dim,
                                     hipStream_t s)
{
    const int32_t per_wave = (64 / (head_dim / 8)) * SCORE_STEPS;
    dim3 grid(ceil_div(a.width, per_wave), n_kv, n_rows);
    switch (head_dim) {
    case 64: select_scores_kernel<64><<<grid, 64, 0, s>>>(a); break;
    case 128: select_scores_kernel<128><<<grid, 64, 0, s>>>(a); break;
    default: select_scores_kernel<256><<<grid, 64, 0, s>>>(a); break;
    }
    return launch_status();
}

extern "C" qsa_status qsa_block_scores(const float *q, const int32_t *pos, int32_t n_rows, const qsa_pool *pool,
                                       qsa_dims dims, int32_t n_blocks, float *scores, qsa_stream_t stream)
{
    qsa_status st = check_dims(dims);
    if (st != QSA_OK) return st;
    if ((st = check_pool(pool, false)) != QSA_OK) return st;
    if (!q || !pos || !scores || !pool->index) return QSA_ERR_NULL;
    if (n_rows < 0 || n_blocks < 0) return QSA_ERR_SHAPE;
    const int32_t stride = ceil_div(pool->capacity, QSA_BLOCK);
    if (n_blocks > stride) return QSA_ERR_RANGE;
    if (n_rows == 0 || n_blocks == 0) return QSA_OK;
    const int32_t G = dims.n_q_heads / dims.n_kv_heads;
    const int32_t per_wave = (64 / (dims.head_dim / 8)) * 4;
    dim3 grid(ceil_div(n_blocks, per_wave), dims.n_kv_heads);
    hipStream_t s = (hipStream_t)stream;
#define QSA_SCORES(DD) block_scores_kernel<DD><<<grid, 64, 0, s>>>(q, pos, n_rows, dims.n_q_heads, dims.n_kv_heads, G, pool->index, stride, pool->n_valid, n_blocks, scores)
    switch (dims.head_dim) {
    case 64: QSA_SCORES(64); break;
    case 128: QSA_SCORES(128); break;
    default: QSA_SCORES(256); break;
    }
#undef QSA_SCORES
    return launch_status();
}

namespace {
template <int D, int VB, int W>
void launch_chunk_g(int G, dim3 grid, hipStream_t s, const ChunkArgs &a)
{
#define QSA_CHUNK(GG)                                                                                              \
    do {                                                                                                           \
        if (a.scores) attn_chunk_select_kernel<D, GG, VB, W><<<grid, 64 * CW, 0, s>>>(a);                          \
        else attn_chunk_kernel<D, GG, VB, W><<<grid, 64 * CW, 0, s>>>(a);                                          \
    } while (0)
    switch (G) {
    case 1: QSA_CHUNK(1); break;
    case 2: QSA_CHUNK(2); break;
    case 3: QSA_CHUNK(3); break;
    case 4: QSA_CHUNK(4); break;
    case 5: QSA_CHUNK(5); break;
    case 6: QSA_CHUNK(6); break;
    case 7: QSA_CHUNK(7); break;
    default: QSA_CHUNK(8); break;
    }
#undef QSA_CHUNK
}

template <int D, int VB>
void launch_chunk(int G, int wpc, dim3 grid, hipStream_t s, const ChunkArgs &a)
{
    if (wpc == CW) launch_chunk_g<D, VB, CW>(G, grid, s, a);
    else if (wpc == 2) launch_chunk_g<D, VB, 2>(G, grid, s, a);
    else launch_chunk_g<D, VB, 1>(G, grid, s, a);
}

// Waves per chunk: CW when a chunk is expected to hold at least CW pieces of 32 cells (16 at d = 256); otherwise
// small chunks (a dense 64-cell chunk is two pieces) share a workgroup instead of leaving waves idle: 2 waves per
// chunk while the grid fits the chip in one round of two workgroups per CU (the kernel's register use), else 1, so
// that a wave walks its chunk's pieces itself rather than waiting for a second round.
int chunk_wpc(int32_t D, int64_t blocks_per_chunk, int64_t n_chunks, int64_t n_groups)
{
    const int64_t pieces = blocks_per_chunk * (QSA_BLOCK / (D <= 128 ? 32 : 16));
    if (pieces >= CW) return CW;
    const int64_t wgs = (n_chunks + 1) / 2 * n_groups;   // workgroups with 2 waves per chunk
    return wgs <= 2 * 256 ? 2 : 1;
}

// vb is the pools' common V width from common_v_bits (4 only with D >= 128).
void launch_chunk_d(int D, int vb, int G, int wpc, dim3 grid, hipStream_t s, const ChunkArgs &a)
{
    if (vb == 4) {
        if (D == 128) launch_chunk<128, 4>(G, wpc, grid, s, a);
        else launch_chunk<256, 4>(G, wpc, grid, s, a);
        return;
    }
    switch (D) {
    case 64: launch_chunk<64, 8>(G, wpc, grid, s, a); break;
    case 128: launch_chunk<128, 8>(G, wpc, grid, s, a); break;
    default: launch_chunk<256, 8>(G, wpc, grid, s, a); break;
    }
}
}  // namespace

extern "C" qsa_status qsa_attn_chunk(const float *q, const int32_t *pos, int32_t n_rows, const qsa_pool *pools,
                                     int32_t n_pools, const int32_t *row_pool, qsa_dims dims, const int32_t *ids,
                                     const int32_t *counts, int32_t k, int32_t blocks_per_chunk, int32_t n_chunks,
                                     float sm_scale, const qsa_partials *out, qsa_stream_t stream)
{
    qsa_status st = check_dims(dims);
    if (st != QSA_OK) return st;
    if (!q || !pos || !pools || !out) return QSA_ERR_NULL;
    if (!out->m || !out->l || !out->o || !out->empty) return QSA_ERR_NULL;
    if (n_rows < 0 || n_pools <= 0) return QSA_ERR_SHAPE;
    if (n_pools > QSA_MAX_POOLS) return QSA_ERR_UNSUPPORTED;
    for (int32_t p = 0; p < n_pools; p++)
        if ((st = check_pool(&pools[p], true)) != QSA_OK) return st;
    const int vb = common_v_bits(pools, n_pools, dims.head_dim);
    if (!vb) return QSA_ERR_UNSUPPORTED;
    if (ids) {
        if (!counts) return QSA_ERR_NULL;
        if (k <= 0) return QSA_ERR_RANGE;
    } else if (blocks_per_chunk <= 0) {
        return QSA_ERR_RANGE;
    }
    if (n_chunks <= 0) return QSA_ERR_RANGE;
    if (n_chunks > out->max_chunks) return QSA_ERR_SCRATCH;
    if (n_rows == 0) return QSA_OK;
    if (n_rows > 65535) return QSA_ERR_UNSUPPORTED;

    ChunkArgs a{};
    a.q = q; a.pos = pos; a.row_pool = row_pool; a.ids = ids; a.counts = counts;
    a.m_out = out->m; a.l_out = out->l; a.o_out = out->o; a.empty_out = out->empty;
    for (int32_t p = 0; p < n_pools; p++)
        a.pools[p] = PoolArg{pools[p].k, pools[p].k_scale, pools[p].v, pools[p].v_scale, pools[p].capacity,
                             pools[p].n_valid};
    a.n_pools = row_pool ? n_pools : 1;
    a.n_qh = dims.n_q_heads; a.n_kv = dims.n_kv_heads; a.G = dims.n_q_heads / dims.n_kv_heads;
    a.topk = k; a.bpc = blocks_per_chunk; a.n_chunks = n_chunks; a.max_chunks = out->max_chunks;
    a.qscale = sm_scale * LOG2E;
    const int wpc = chunk_wpc(dims.head_dim, ids ? ceil_div(k, n_chunks) : blocks_per_chunk, n_chunks,
                              (int64_t)dims.n_kv_heads * n_rows);
    dim3 grid(ceil_div(n_chunks, CW / wpc), dims.n_kv_heads, n_rows);
    hipStream_t s = (hipStream_t)stream;
    launch_chunk_d(dims.head_dim, vb, a.G, wpc, grid, s, a);
    return launch_status();
}

qsa_status qsa::merge_launch(const float *m, const float *l, const float *o, const uint8_t *empty, int32_t max_chunks,
                             int32_t n_chunks, const int32_t *n_active, int32_t n_rows, int32_t n_qh,
                             int32_t head_dim, float *out, float *lse, hipStream_t s)
{
    const uint32_t rows = (uint32_t)n_rows * (uint32_t)n_qh;
    // a few chunks: 4 waves, 8 rows in flight each, one workgroup per (row, head); many (a dense window): 16 waves,
    // 16 steps of two chunks in flight each, and the head's dims split over D/32 workgroups of 32 dims, so more CUs
    // stream the o rows (each re-reads the chunks' m, l and empty marks)
#define QSA_MERGE(DD)                                                                                              \
    do {                                                                                                           \
        if (n_chunks <= 64)                                                                                        \
            attn_merge_kernel<DD, 4, 8, 1><<<dim3(rows, 1), 256, 0, s>>>(m, l, o, empty, max_chunks, n_chunks,      \
                                                                       n_active, n_qh, out, lse);                 \
        else                                                                                                       \
            attn_merge_kernel<DD, 16, 16, DD / 32><<<dim3(rows, DD / 32), 1024, 0, s>>>(                          \
                m, l, o, empty, max_chunks, n_chunks, n_active, n_qh, out, lse);                                  \
    } while (0)
    switch (head_dim) {
    case 64: QSA_MERGE(64); break;
    case 128: QSA_MERGE(128); break;
    default: QSA_MERGE(256); break;
    }
#undef QSA_MERGE
    return launch_status();
}

extern "C" qsa_status qsa_attn_merge(const qsa_partials *in, int32_t n_rows, qsa_dims dims, int32_t n_chunks,
                                     const int32_t *n_active, float *out, float *lse, qsa_stream_t stream)
{
    qsa_status st = check_dims(dims);
    if (st != QSA_OK) return st;
    if (!in || !out) return QSA_ERR_NULL;
    if (!in->m || !in->l || !in->o || !in->empty) return QSA_ERR_NULL;
    if (n_rows < 0) return QSA_ERR_SHAPE;
    if (n_chunks < 1) return QSA_ERR_RANGE;   // the merge kernel reads chunk n_chunks - 1 as its clamp target
    if (n_chunks > in->max_chunks) return QSA_ERR_SCRATCH;
    if (n_rows == 0) return QSA_OK;
    return merge_launch(in->m, in->l, in->o, in->empty, in->max_chunks, n_chunks, n_active, n_rows, dims.n_q_heads,
                        dims.head_dim, out, lse, (hipStream_t)stream);
}

// ======================================================================================= fused decode layer
namespace {
struct LayerScratch {
    size_t m, l, e, o, ids, counts, scores, total;
};

LayerScratch layer_layout(int32_t n_rows, const qsa_dims &d, int32_t n_blocks, int32_t k, int32_t n_chunks)
{
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t rh = (size_t)n_rows * d.n_q_heads * n_chunks;
    const size_t rk = (size_t)n_rows * d.n_kv_heads;
    LayerScratch s{};
    size_t off = 0;
    s.m = off; off += al(rh * sizeof(float));
    s.l = off; off += al(rh * sizeof(float));
    s.e = off; off += al(rh);
    s.o = off; off += al(rh * d.head_dim * sizeof(float));
    s.ids = off; off += al(rk * k * sizeof(int32_t));
    s.counts = off; off += al(rk * sizeof(int32_t));
    s.scores = off; off += al(rk * n_blocks * sizeof(float));
    s.total = off;
    return s;
}
}  // namespace

namespace {
// Shared argument checks and pool marshalling of the fused selection.
qsa_status select_setup(const float *q, const int32_t *pos, int32_t n_rows, const qsa_pool *pools, int32_t n_pools,
                        const int32_t *row_pool, const qsa_dims &dims, int32_t n_blocks, int32_t k, SelectArgs &sa)
{
    qsa_status st = check_dims(dims);
    if (st != QSA_OK) return st;
    if (!q || !pos || !pools) return QSA_ERR_NULL;
    if (n_rows < 0 || n_pools <= 0 || n_blocks < 0) return QSA_ERR_SHAPE;
    if (n_pools > QSA_MAX_POOLS) return QSA_ERR_UNSUPPORTED;
    for (int32_t p = 0; p < n_pools; p++) {
        if ((st = check_pool(&pools[p], true)) != QSA_OK) return st;
        if (!pools[p].index) return QSA_ERR_NULL;
        if (n_blocks > ceil_div(pools[p].capacity, QSA_BLOCK)) return QSA_ERR_RANGE;
    }
    if (k < 1 || k > n_blocks) return QSA_ERR_RANGE;
    if (n_blocks > 256 * 64) return QSA_ERR_UNSUPPORTED;
    if (n_rows > 65535) return QSA_ERR_UNSUPPORTED;
    sa = SelectArgs{};
    sa.q = q; sa.pos = pos; sa.row_pool = row_pool;
    for (int32_t p = 0; p < n_pools; p++)
        sa.pools[p] = PoolArg{pools[p].k, pools[p].k_scale, pools[p].v, pools[p].v_scale, pools[p].capacity,
                              pools[p].n_valid, pools[p].index};
    sa.n_pools = row_pool ? n_pools : 1;
    sa.n_qh = dims.n_q_heads; sa.n_kv = dims.n_kv_heads; sa.G = dims.n_q_heads / dims.n_kv_heads;
    sa.width = n_blocks; sa.k = k;
    return QSA_OK;
}
}  // namespace

extern "C" qsa_status qsa_decode_select(const float *q, const int32_t *pos, int32_t n_rows, const qsa_pool *pools,
                                        int32_t n_pools, const int32_t *row_pool, qsa_dims dims, int32_t n_blocks,
                                        int32_t k, float *scores, int32_t *ids, int32_t *counts, qsa_stream_t stream)
{
    SelectArgs sa;
    qsa_status st = select_setup(q, pos, n_rows, pools, n_pools, row_pool, dims, n_blocks, k, sa);
    if (st != QSA_OK) return st;
    if (!ids || !counts) return QSA_ERR_NULL;
    if (n_rows == 0) return QSA_OK;
    sa.ids = ids; sa.counts = counts; sa.scores = scores;
    return select_launch(sa, n_rows, dims.n_kv_heads, dims.head_dim, (hipStream_t)stream);
}

extern "C" size_t qsa_decode_layer_scratch_bytes(int32_t n_rows, qsa_dims dims, int32_t n_blocks, int32_t k,
                                                 int32_t n_chunks)
{
    if (n_rows <= 0 || n_blocks <= 0 || k <= 0 || n_chunks <= 0 || check_dims(dims) != QSA_OK) return 0;
    return layer_layout(n_rows, dims, n_blocks, k, n_chunks).total;
}

namespace {
// Host-side checks of qsa_decode_layer's arguments (everything but the scratch buffer); fills sa and vb.
qsa_status layer_setup(const float *q, const int32_t *pos, int32_t n_rows, const qsa_pool *pools, int32_t n_pools,
                       const int32_t *row_pool, const qsa_dims &dims, int32_t n_blocks, int32_t k, int32_t n_chunks,
                       const float *out, SelectArgs &sa, int &vb)
{
    qsa_status st = select_setup(q, pos, n_rows, pools, n_pools, row_pool, dims, n_blocks, k, sa);
    if (st != QSA_OK) return st;
    if (!out) return QSA_ERR_NULL;
    if (n_chunks < 1) return QSA_ERR_RANGE;
    vb = common_v_bits(pools, n_pools, dims.head_dim);
    if (!vb) return QSA_ERR_UNSUPPORTED;
    return QSA_OK;
}

// The three launches of the decode layer over a scratch region `base` already checked to hold layer_layout's total.
qsa_status layer_launch(const float *q, const int32_t *pos, int32_t n_rows, const qsa_pool *pools, int32_t n_pools,
                        const int32_t *row_pool, const qsa_dims &dims, int32_t n_blocks, int32_t k, int32_t n_chunks,
                        float sm_scale, float *out, float *lse, float *scores, int32_t *ids, int32_t *counts,
                        SelectArgs &sa, int vb, char *base, hipStream_t s)
{
    qsa_status st;
    const LayerScratch lay = layer_layout(n_rows, dims, n_blocks, k, n_chunks);

    sa.ids = ids ? ids : reinterpret_cast<int32_t *>(base + lay.ids);
    sa.counts = counts ? counts : reinterpret_cast<int32_t *>(base + lay.counts);
    // Rows of up to FUSED_TOPK_MAX_WIDTH columns: the score rows in one launch over many CUs, and every chunk
    // workgroup takes its row's top-k itself (no selection launch of one workgroup per row). Wider rows: the
    // selection launches (through the score rows when they have many live blocks), then the chunks read the ids.
    const bool fuse = n_blocks <= FUSED_TOPK_MAX_WIDTH && k <= FUSED_TOPK_MAX_K;
    sa.scores = scores ? scores : reinterpret_cast<float *>(base + lay.scores);
    if (!fuse && !scores && !select_splits(sa)) sa.scores = nullptr;
    if (fuse) st = select_scores_launch(sa, n_rows, dims.n_kv_heads, dims.head_dim, s);
    else st = select_launch(sa, n_rows, dims.n_kv_heads, dims.head_dim, s);
    if (st != QSA_OK) return st;

    ChunkArgs a{};
    a.q = q; a.pos = pos; a.row_pool = row_pool;
    if (fuse) {
        a.scores = sa.scores; a.width = n_blocks; a.ids_out = ids; a.counts_out = counts;
    } else {
        a.ids = sa.ids; a.counts = sa.counts;
    }
    a.m_out = reinterpret_cast<float *>(base + lay.m);
    a.l_out = reinterpret_cast<float *>(base + lay.l);
    a.o_out = reinterpret_cast<float *>(base + lay.o);
    a.empty_out = reinterpret_cast<uint8_t *>(base + lay.e);
    for (int32_t p = 0; p < n_pools; p++) a.pools[p] = sa.pools[p];
    a.n_pools = sa.n_pools;
    a.n_qh = dims.n_q_heads; a.n_kv = dims.n_kv_heads; a.G = sa.G;
    a.topk = k; a.bpc = 0; a.n_chunks = n_chunks; a.max_chunks = n_chunks;
    a.qscale = sm_scale * LOG2E;
    const int wpc = chunk_wpc(dims.head_dim, ceil_div(k, n_chunks), n_chunks, (int64_t)dims.n_kv_heads * n_rows);
    launch_chunk_d(dims.head_dim, vb, a.G, wpc, dim3(ceil_div(n_chunks, CW / wpc), dims.n_kv_heads, n_rows), s, a);
    if ((st = launch_status()) != QSA_OK) return st;
    return merge_launch(a.m_out, a.l_out, a.o_out, a.empty_out, n_chunks, n_chunks, nullptr, n_rows, dims.n_q_heads,
                        dims.head_dim, out, lse, s);
}
}  // namespace

extern "C" qsa_status qsa_decode_layer(const float *q, const int32_t *pos, int32_t n_rows, const qsa_pool *pools,
                                       int32_t n_pools, const int32_t *row_pool, qsa_dims dims, int32_t n_blocks,
                                       int32_t k, int32_t n_chunks, float sm_scale, float *out, float *lse,
                                       float *scores, int32_t *ids, int32_t *counts, void *scratch,
                                       size_t scratch_bytes, qsa_stream_t stream)
{
    SelectArgs sa;
    int vb = 0;
    qsa_status st = layer_setup(q, pos, n_rows, pools, n_pools, row_pool, dims, n_blocks, k, n_chunks, out, sa, vb);
    if (st != QSA_OK) return st;
    if (n_rows == 0) return QSA_OK;
    if (!scratch) return QSA_ERR_NULL;
    if (scratch_bytes < layer_layout(n_rows, dims, n_blocks, k, n_chunks).total) return QSA_ERR_SCRATCH;
    return layer_launch(q, pos, n_rows, pools, n_pools, row_pool, dims, n_blocks, k, n_chunks, sm_scale, out, lse,
                        scores, ids, counts, sa, vb, static_cast<char *>(scratch), (hipStream_t)stream);
}

// ============================================================================ decode layer without allocation
// The scratch of qsa_decode_layer_noalloc: one file-scope device array, so callers that cannot allocate (code under
// graph capture, serving loops that forbid it) pass only their inputs and outputs. Each GPU the library runs on holds
// its own copy for the life of the process. On the host the array's name is a stand-in, not a device address: the
// device address comes from hipGetSymbolAddress, once per device, and only that address is handed to kernels.
namespace {
static __device__ __align__(256) char layer_scratch_static[QSA_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex static_scratch_mutex;
char *static_scratch_ptr[MAX_DEVICES];   // per device, set on the first call on that device

qsa_status static_scratch(char **ptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return QSA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(static_scratch_mutex);
    if (!static_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(layer_scratch_static)) != hipSuccess || !p) return QSA_ERR_LAUNCH;
        static_scratch_ptr[dev] = static_cast<char *>(p);
    }
    *ptr = static_scratch_ptr[dev];
    return QSA_OK;
}
}  // namespace

extern "C" qsa_status qsa_decode_layer_noalloc(const float *q, const int32_t *pos, int32_t n_rows,
                                               const qsa_pool *pools, int32_t n_pools, const int32_t *row_pool,
                                               qsa_dims dims, int32_t n_blocks, int32_t k, int32_t n_chunks,
                                               float sm_scale, float *out, float *lse, float *scores, int32_t *ids,
                                               int32_t *counts, qsa_stream_t stream)
{
    SelectArgs sa;
    int vb = 0;
    qsa_status st = layer_setup(q, pos, n_rows, pools, n_pools, row_pool, dims, n_blocks, k, n_chunks, out, sa, vb);
    if (st != QSA_OK) return st;
    if (n_rows == 0) return QSA_OK;
    if (layer_layout(n_rows, dims, n_blocks, k, n_chunks).total > (size_t)QSA_NOALLOC_SCRATCH_BYTES)
        return QSA_ERR_SCRATCH;
    char *base = nullptr;
    if ((st = static_scratch(&base)) != QSA_OK) return st;
    return layer_launch(q, pos, n_rows, pools, n_pools, row_pool, dims, n_blocks, k, n_chunks, sm_scale, out, lse,
                        scores, ids, counts, sa, vb, base, (hipStream_t)stream);
}

extern "C" const char *qsa_status_str(qsa_status status)
{
    switch (status) {
    case QSA_OK: return "ok";
    case QSA_ERR_NULL: return "null pointer";
    case QSA_ERR_SHAPE: return "inconsistent shape";
    case QSA_ERR_UNSUPPORTED: return "unsupported shape";
    case QSA_ERR_SCRATCH: return "scratch or partials too small";
    case QSA_ERR_RANGE: return "argument out of range";
    case QSA_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}
