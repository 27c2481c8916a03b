// Decode-path kernels of libqsa for gfx950: block index, block scores, the log-sum-exp merge and the append path,
// and the host side of every decode call (the split-K chunk attention kernels live in qsa_chunk.h and are
// instantiated per head dim and V width in qsa_chunk_d*.hip). The kernels stream int8 codes / fp32 rows from HBM
// with 16-byte coalesced loads; per cell the work is a few hundred FMAs against 272 bytes, so HBM and the fp32 VALU
// are the ceilings. With 4 or more q heads
// per KV head at d = 128 the chunk kernel runs both of its products on the matrix cores (fp16 MFMA with exact K and V
// codes and two-term splits of q and p * v_scale), on the VALU otherwise.
//
// Lane layout shared by the index and chunk kernels ("cell x slice"): a cell's D dims are cut into D/16 slices of
// 16 dims (one 16-byte load of int8 codes), so a wave covers 64 / (D/16) cells per step; lane = cell_slot * LPC +
// slice. A slice never straddles a 64-dim scale group. The index kernel finishes its per-cell sums with a DPP sum
// over the LPC lanes of the cell; the chunk kernel finishes its G per-cell dot products with a reduce-scatter over
// those lanes, so that each (cell, head) logit ends in one lane. Head dim 192 uses the lane layouts of 256, its lanes
// past dim 191 idle (lane_dims).
#include "qsa_chunk.h"
#include "qsa_internal.h"
#include "qsa_radix.h"

#include <math.h>

#include <mutex>

namespace qsa {
// --------------------------------------------------------------------------------------------- block index
// index[g][b][:] = mean of the dequantised keys of block b's valid cells, computed by one wave.
template <int D>
__device__ __forceinline__ void block_mean(const int8_t *__restrict__ k, const float *__restrict__ ks, int32_t cap,
                                           int32_t n_valid, int32_t g, int32_t b, int32_t blk_stride,
                                           float *__restrict__ index)
{
    constexpr int DL = lane_dims<D>(), LPC = DL / 16, CPS = 64 / LPC, STEPS = QSA_BLOCK / CPS, NG = D / QSA_GROUP;
    const int lane = threadIdx.x % 64, r = lane / LPC, s = lane % LPC, grp = (16 * s) / QSA_GROUP;
    const bool sl = DL == D || 16 * s < D;        // the lane's slice holds dims of the row
    const int64_t c0 = (int64_t)b * QSA_BLOCK;   // 64-bit: a capacity near INT32_MAX
    float acc[16];
#pragma unroll
    for (int e = 0; e < 16; e++) acc[e] = 0.f;
#pragma unroll
    for (int st = 0; st < STEPS; st++) {
        const int64_t c = c0 + st * CPS + r;
        if (c < n_valid && sl) {
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
    const int64_t left = n_valid - c0;
    const int32_t nb = left < 0 ? 0 : (left > QSA_BLOCK ? QSA_BLOCK : (int32_t)left);
    const float inv = nb > 0 ? 1.0f / (float)nb : 0.f;
    if (r == 0 && sl) {
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
    block_mean<D>(P.k, P.ks, P.capacity, P.n_valid, g, c / QSA_BLOCK, ceil_div(P.capacity, QSA_BLOCK),
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
    constexpr int DL = lane_dims<D>(), LPB = DL / 8, BPS = 64 / LPB, NSTEP = 4;
    const int lane = threadIdx.x, rb = lane / LPB, s0 = lane % LPB;
    const bool sl = DL == D || 8 * s0 < D;   // the lane's 8 dims are dims of the row (else it adds zeros)
    const int s = sl ? s0 : 0;
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
        const bool live = b < n_live && sl;
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
                    if (h < G && sl) {
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
                if (s0 == 0 && b < n_blocks)
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
    constexpr int DL = lane_dims<D>(), LPB = DL / 8, BPS = 64 / LPB, NSTEP = SCORE_STEPS;
    const int lane = threadIdx.x, rb = lane / LPB, s0 = lane % LPB;
    const bool sl = DL == D || 8 * s0 < D;   // the lane's 8 dims are dims of the row (else it adds zeros)
    const int s = sl ? s0 : 0;
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
    const int32_t stride = ceil_div(P.capacity, QSA_BLOCK);
    const int32_t n_live = bad ? 0 : min(a.width, (int32_t)(((int64_t)P.n_valid + QSA_BLOCK - 1) / QSA_BLOCK));
    float rv[NSTEP][8];
#pragma unroll
    for (int st = 0; st < NSTEP; st++) {
        const int32_t b = bw + st * BPS + rb;
        const bool live = b < n_live && sl;
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
        if (h < a.G && sl) {
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
        if (s0 == 0 && b < a.width)
            a.scores[((int64_t)i * a.n_kv + g) * a.width + b] = (b < n_live && first <= p) ? dot : -INFINITY;
    }
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
    case 192: block_index_kernel<192><<<grid, 64, 0, s>>>(pool->k, pool->k_scale, pool->capacity, pool->n_valid, b0, stride, index); break;
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
    case 192: append_encode_kernel<192, 8><<<grid, 64, 0, s>>>(a); break;
    case -192: append_encode_kernel<192, 4><<<grid, 64, 0, s>>>(a); break;
    case -256: append_encode_kernel<256, 4><<<grid, 64, 0, s>>>(a); break;
    default: append_encode_kernel<256, 8><<<grid, 64, 0, s>>>(a); break;
    }
    switch (dims.head_dim) {
    case 64: append_index_kernel<64><<<grid, 64, 0, s>>>(a); break;
    case 128: append_index_kernel<128><<<grid, 64, 0, s>>>(a); break;
    case 192: append_index_kernel<192><<<grid, 64, 0, s>>>(a); break;
    default: append_index_kernel<256><<<grid, 64, 0, s>>>(a); break;
    }
    return launch_status();
}

qsa_status qsa::select_scores_launch(const SelectArgs &a, int32_t n_rows, int32_t n_kv, int32_t head_dim,
                                     hipStream_t s)
{
    const int32_t per_wave = (64 / (lane_dims(head_dim) / 8)) * SCORE_STEPS;
    dim3 grid(ceil_div(a.width, per_wave), n_kv, n_rows);
    switch (head_dim) {
    case 64: select_scores_kernel<64><<<grid, 64, 0, s>>>(a); break;
    case 128: select_scores_kernel<128><<<grid, 64, 0, s>>>(a); break;
    case 192: select_scores_kernel<192><<<grid, 64, 0, s>>>(a); break;
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
    const int32_t per_wave = (64 / (lane_dims(dims.head_dim) / 8)) * 4;
    dim3 grid(ceil_div(n_blocks, per_wave), dims.n_kv_heads);
    hipStream_t s = (hipStream_t)stream;
#define QSA_SCORES(DD) block_scores_kernel<DD><<<grid, 64, 0, s>>>(q, pos, n_rows, dims.n_q_heads, dims.n_kv_heads, G, pool->index, stride, pool->n_valid, n_blocks, scores)
    switch (dims.head_dim) {
    case 64: QSA_SCORES(64); break;
    case 128: QSA_SCORES(128); break;
    case 192: QSA_SCORES(192); break;
    default: QSA_SCORES(256); break;
    }
#undef QSA_SCORES
    return launch_status();
}

namespace {
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
        if (D == 128) launch_chunk_128_4(G, wpc, grid, s, a);
        else if (D == 192) launch_chunk_192_4(G, wpc, grid, s, a);
        else launch_chunk_256_4(G, wpc, grid, s, a);
        return;
    }
    switch (D) {
    case 64: launch_chunk_64_8(G, wpc, grid, s, a); break;
    case 128: launch_chunk_128_8(G, wpc, grid, s, a); break;
    case 192: launch_chunk_192_8(G, wpc, grid, s, a); break;
    default: launch_chunk_256_8(G, wpc, grid, s, a); break;
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
    if (n_chunks <= 0 || !scale_ok(sm_scale)) return QSA_ERR_RANGE;
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
    case 192: QSA_MERGE(192); break;
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
    if ((int64_t)n_rows * dims.n_q_heads > INT32_MAX) return QSA_ERR_UNSUPPORTED;   // one workgroup per (row, head)
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
                       float sm_scale, const float *out, SelectArgs &sa, int &vb)
{
    qsa_status st = select_setup(q, pos, n_rows, pools, n_pools, row_pool, dims, n_blocks, k, sa);
    if (st != QSA_OK) return st;
    if (!out) return QSA_ERR_NULL;
    if (n_chunks < 1 || !scale_ok(sm_scale)) return QSA_ERR_RANGE;
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
    qsa_status st =
        layer_setup(q, pos, n_rows, pools, n_pools, row_pool, dims, n_blocks, k, n_chunks, sm_scale, out, sa, vb);
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
    qsa_status st =
        layer_setup(q, pos, n_rows, pools, n_pools, row_pool, dims, n_blocks, k, n_chunks, sm_scale, out, sa, vb);
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
