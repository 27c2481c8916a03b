// Split-K chunk attention of libqsa's decode path (gfx950): the kernel templates, shared by the translation units
// that instantiate them per head dim and V width (qsa_chunk_d*.hip) so that the instantiations build in parallel, and
// by qsa_decode.hip, which launches them.
//
// Lane layout ("cell x slice"): a cell's D dims are cut into D/16 slices of 16 dims (one 16-byte load of int8
// codes), so a wave covers 64 / (D/16) cells per step; lane = cell_slot * LPC + slice. A slice never straddles a
// 64-dim scale group. The chunk kernel finishes its G per-cell dot products with a reduce-scatter over those lanes,
// so that each (cell, head) logit ends in one lane.
#pragma once

#include "qsa_internal.h"
#include "qsa_radix.h"

#include <math.h>

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
    // DL: the lane layout's dims (head_dim 192 runs on 256's; its lanes past dim 191 hold zeros and store nothing)
    constexpr int DL = lane_dims<D>();
    constexpr int PC = D <= 128 ? 32 : 16;           // cells per piece
    constexpr int LPC = DL / 16, CPS = 64 / LPC, STEPS = PC / CPS, NG = DL / QSA_GROUP;
    constexpr int NGM = D / QSA_GROUP;               // scale groups stored per cell
    constexpr int DPL = DL / 64;                     // output dims per lane
    constexpr int RB = D * VB / 8;                   // V bytes per cell row in the pool
    constexpr int RBL = DL * VB / 8;                 // V bytes per cell row in LDS
    constexpr int NPB = 8 / VB;                      // V codes per byte
    constexpr int NT = DPL / NPB;                    // transposing reads per lane per 8 cells
    constexpr int DPC = 16 * NPB;                    // dims per 16-byte chunk
    constexpr int CPG = QSA_GROUP / DPC;             // 16-byte chunks per scale group
    constexpr int SUBS = 4 / NG;                     // 16-lane subgroups per scale group in the p . v layout
    constexpr int CHUNKS = RBL / 16;                 // 16-byte chunks per V row in LDS
    constexpr int MCH = RB / 16;                     // the pool row's chunks (the rest of an LDS row is not read)
    constexpr int SWZ = (CHUNKS < 8 ? CHUNKS : 8) - 1;
    constexpr int VCH = PC * RBL / 1024;             // 1 KB global -> LDS copies per piece
    constexpr int GP = (G + 3) & ~3;                 // p * v_scale row padded to float4s
    static_assert(CPG == SUBS * NT && VCH * 1024 == PC * RBL, "p . v lane layout");
    // Both products on the matrix cores (int8 K and V, d = 128, 4 or more heads; MPV): the logits of the piece's 32
    // cells as S[cell][head] = K q^T per 64-dim scale group, and per 16-dim output tile O[head][dim] +=
    // P[head][cell] V[cell][dim], all with v_mfma_f32_16x16x32_f16 (heads padded to 16 rows). K and V codes are exact
    // in fp16; q and p * v_scale go in as two fp16 terms (hi + lo, 22 significant bits) scaled by powers of two that
    // keep them in fp16's range, both terms accumulating into the same fp32 tile.
    constexpr bool MPV = D == 128 && G >= 4;
    constexpr int NTL = D / 16;                      // 16-dim output tiles (MPV)
    static_assert(!MPV || (NG == 2 && PC == 32 && DL == D), "MFMA form: d = 128, 32-cell pieces");
    // MFMA form: output tile t's lane jl holds dim 16 t + jl (int8 V); with 4-bit V a transposing read of 16-byte
    // chunk c gives dims 32 c + 2 jl (low nibbles, tile 2 c) and 32 c + 2 jl + 1 (high nibbles, tile 2 c + 1)
    auto tile_dim = [](int t, int l) { return VB == 8 ? 16 * t + l : 32 * (t >> 1) + 2 * l + (t & 1); };
    __shared__ __align__(16) int8_t sv[CW][PC * RBL];   // the wave's V piece: [cell][RBL], chunk c of row r at c ^ swizzle(r)
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
    const int r = lane / LPC, s = lane % LPC;
    const bool s_in = DL == D || 16 * s < D;         // the lane's slice holds dims of the row
    const int s_ld = s_in ? s : 0;                   // the slice it loads (padding slices load slice 0, unused)
    const int grp_s = s_ld / (LPC / NG);
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
        const float4 *src = reinterpret_cast<const float4 *>(sq + h * D + 16 * s_ld);
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
            const float4 u = s_in ? src[jj] : make_float4(0.f, 0.f, 0.f, 0.f);
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

    const int8_t *kbase = P.k + (int64_t)g * P.capacity * D + 16 * s_ld;
    const int8_t *vbase = P.v + (int64_t)g * P.capacity * RB;
    const float *ksbase = P.ks + (int64_t)g * P.capacity * NGM + grp_s;
    const float *vsbase = P.vs + (int64_t)g * P.capacity * NGM;
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
            // the piece's matrix-core section runs at raised wave priority (its MFMAs issue ahead of the other waves'
            // VALU work on the SIMD)
            __builtin_amdgcn_s_setprio(1);
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
            __builtin_amdgcn_s_setprio(0);
        } else {
            // ---- loads: K slices and scales into registers, the V piece into LDS
            int4 kw[STEPS];
            float ksc[STEPS], vsc[STEPS][NG];
#pragma unroll
            for (int st = 0; st < STEPS; st++) {
                const int32_t c = min(cb + st * CPS + r, limit);
                kw[st] = *reinterpret_cast<const int4 *>(kbase + (int64_t)c * D);
                ksc[st] = ksbase[(int64_t)c * NGM] * a.qscale;  // sm_scale * log2(e) rides on the key scale
                const float *vsrc = vsbase + (int64_t)c * NGM;  // all group scales of the cell, one load
                if constexpr (NGM == 3) {
                    vsc[st][0] = vsrc[0]; vsc[st][1] = vsrc[1]; vsc[st][2] = vsrc[2]; vsc[st][3] = 0.f;
                } else if constexpr (NG == 4) {
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
                const int mc = pch ^ (cell & SWZ);      // the pool chunk this LDS position holds
                load_lds16(vbase + (int64_t)c * RB + 16 * (RB == RBL || mc < MCH ? mc : 0), lds_addr(svw + 1024 * q));
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
                        (QSA_LDS v2i *)(svw + cell * RBL + 16 * (lc ^ (cell & SWZ)) + 8 * hh));
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
                    if (DL != D && d >= D) continue;
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
                if (DL != D && d >= D) continue;
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

// Launch of the chunk kernels for one head dim and V width, by q heads per KV head (G) and waves per chunk (wpc).
// Each instantiating translation unit defines one of these.
void launch_chunk_64_8(int G, int wpc, dim3 grid, hipStream_t s, const ChunkArgs &a);
void launch_chunk_128_8(int G, int wpc, dim3 grid, hipStream_t s, const ChunkArgs &a);
void launch_chunk_128_4(int G, int wpc, dim3 grid, hipStream_t s, const ChunkArgs &a);
void launch_chunk_192_8(int G, int wpc, dim3 grid, hipStream_t s, const ChunkArgs &a);
void launch_chunk_192_4(int G, int wpc, dim3 grid, hipStream_t s, const ChunkArgs &a);
void launch_chunk_256_8(int G, int wpc, dim3 grid, hipStream_t s, const ChunkArgs &a);
void launch_chunk_256_4(int G, int wpc, dim3 grid, hipStream_t s, const ChunkArgs &a);

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

}  // namespace qsa
