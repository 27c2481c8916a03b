// Prompt-chunk attention on gfx950 int8 matrix cores (v_mfma_i32_16x16x64_i8).
//
// Both products run on the int8 K/V codes as stored. The other operand of each product is split into exact signed
// bytes, so every int32 sum is exact and only the recombination is fp32:
//   q    : one scale per (query, head) maps max |q| to 127 * 2^16; X = rint(q * scale) = 2^16 h + 2^8 l + m.
//   p*vs : p = 2^(t - m_ref) <= 1 and w = vs * 127 * 2^24 / VS[g] (VS[g] = max v_scale over the cells the call
//          sees, w made per tile in LDS), X = p * w rounded to an integer = 2^24 d3 + 2^16 d2 + 2^8 d1 + d0.
//          Four bytes (31 bits) rather than three because one scale covers a whole row: most cells sit far below
//          the row maximum, and with 24 bits their rounding alone reached 1e-5 relative at a 32K context.
//
// Orientation. With row = (query, q head) and lane l of a wave owning row l % 16:
//   S^T[cell][row] = K[cell][:] . Q^T        (A = K codes from LDS, B = q digits from LDS)
//   O^T[dim][row]  = V^T[dim][cell] . P^T    (A = V^T read from LDS with transposing loads, B = p digits)
// The 16x16 result of an MFMA puts rows 4*(l/16) + v (v = 0..3) of column l % 16 in lane l. In S^T block b the
// A-row 4G + v is loaded with cell 16G + 4b + v, so after the four blocks of a 64-cell tile lane l holds the 16
// cells 16G .. 16G + 15 (G = l / 16) of its row -- exactly the k-slots lane l must supply as the B operand of the
// PV product, and the cells the lane's V^T operand holds. P never leaves registers.
//
// Tiles go from HBM straight into LDS (global_load_lds, no staging registers), triple-buffered; bank swizzles are
// applied by choosing which 16-byte chunk each lane fetches. V stays [cell][dim] in LDS; ds_read_b64_tr_b8 (within
// each 16-lane group, lane j receives byte i of the 8 bytes addressed by lane 2i + (j >= 8), at byte j mod 8) turns
// two reads per 16-dim block into the V^T operand.
//
// The PV int32 sums are accumulated across tiles while the reference max m_ref of a row does not move; when a tile's
// row max exceeds m_ref, the wave folds the int32 sums into fp32 (rescaled by 2^(m_old - m_new)) and restarts them,
// with m_ref set DELTA above the new max so that later small increases need no fold.
//
// K8V4 pools (4-bit V codes, two per byte) take the same kernel: the packed V tile is copied into LDS and widened to
// int8 codes there (exact), after which every product and split is the one of an int8 pool.
#include "qsa_internal.h"

#include <stdint.h>

#include <type_traits>

namespace qsa {


constexpr int PD = 128;          // head dim of the prompt kernel
constexpr int PT = 64;           // cells per tile
constexpr int PW = 4;            // waves per workgroup
constexpr int PROWS = 16 * PW;   // rows (query, head) per workgroup
constexpr int NBUF = 3;          // K/V tile buffers
constexpr float PLOG2E = 1.4426950408889634f;
constexpr float PLN2 = 0.6931471805599453f;
constexpr float PDELTA = 4.0f;   // headroom (log2 units) added to the reference max at a fold
constexpr float QMAX = 127.0f * 65536.0f;          // largest q digit value
constexpr float PMAX = 127.0f * 16777216.0f;       // largest p * w digit value
// (uint32)(p * w + PBIAS) = X + 0x808080: bytes 0..2 hold d0 + 128, d1 + 128, d2 + 128 and byte 3 holds d3 in
// [0, 127] (X <= 127 * 2^24 keeps the sum below 2^31). The conversion truncates; below 2^24 the fractional part is
// dropped, an error of at most one unit in 2^31 of the row's largest term.
constexpr float PBIAS = 8421504.0f;                // 0x808080
constexpr int FOLD_EVERY = 1024;                   // tiles between forced folds (int32 sums stay below 2^31)
constexpr int NCU = 256;                            // compute units of an MI355X
constexpr int VS_SLICES = 32;

// 16-byte chunk swizzles of the LDS tiles (rows of 128 B): K chunks for the plain 16-byte operand reads, V chunks
// for the 8-byte transposing reads (consecutive cells land on different banks).
__device__ __forceinline__ int swz_k(int cell) { return (cell & 3) | ((cell >> 2) & 4); }
__device__ __forceinline__ int swz_v(int cell) { return cell & 7; }

__device__ __forceinline__ uint32_t bperm(uint32_t s0, uint32_t s1, uint32_t sel)
{
    return __builtin_amdgcn_perm(s0, s1, sel);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int WAIT_VM0_LGKM0 = 0x0070;   // all vector memory and LDS operations done
constexpr int WAIT_VM5_LGKM0 = 0x0075;   // all but the 5 newest vector memory operations done, LDS done
constexpr int WAIT_VM4_LGKM0 = 0x0074;   // all but the 4 newest

// ---------------------------------------------------------------------------------------------- q digits
// One wave per (query, q head), four per workgroup: qd[g][r][plane][d] int8 with r = query * G + head-in-group,
// plane 0/1/2 = h/l/m, and qs[g][r] = max|q| / (127 * 65536) * |sm_scale| * log2(e) so that
// q . k * sm_scale * log2(e) = qs * (X . k): the digits are those of sign(sm_scale) * q, so the logit scale of a row
// is never negative (the attention kernel floors it at a tiny positive value).
__device__ __forceinline__ void prompt_qsplit(const float *__restrict__ q, int32_t n_qh, int32_t G, int32_t R,
                                              int64_t n_rows, float qscale, int8_t *__restrict__ qd,
                                              float *__restrict__ qs, uint32_t wg)
{
    const int lane = threadIdx.x % 64;
    const int64_t row = (int64_t)wg * 4 + threadIdx.x / 64;   // = query * n_qh + head
    if (row >= n_rows) return;                                          // whole waves leave together
    const int32_t qi = (int32_t)(row / n_qh), h = (int32_t)(row % n_qh);
    const int32_t g = h / G, r = qi * G + h % G;
    const float2 x = reinterpret_cast<const float2 *>(q + row * PD)[lane];
    const float amax = group_max<64>(fmaxf(fabsf(x.x), fabsf(x.y)));
    const float s = amax > 0.f ? copysignf(QMAX / amax, qscale) : 0.f;
    const int32_t X[2] = {(int32_t)rintf(x.x * s), (int32_t)rintf(x.y * s)};
    int32_t dg[3][2];
#pragma unroll
    for (int e = 0; e < 2; e++) {
        const int32_t m = (X[e] << 24) >> 24;
        const int32_t x1 = (X[e] - m) >> 8;
        const int32_t l = (x1 << 24) >> 24;
        dg[2][e] = m;
        dg[1][e] = l;
        dg[0][e] = (x1 - l) >> 8;
    }
    int8_t *dst = qd + ((int64_t)g * R + r) * 3 * PD;
#pragma unroll
    for (int p = 0; p < 3; p++) {
        const uint16_t pair = (uint16_t)((dg[p][0] & 255) | ((dg[p][1] & 255) << 8));
        reinterpret_cast<uint16_t *>(dst + p * PD)[lane] = pair;
    }
    if (lane == 0) qs[(int64_t)g * R + r] = amax > 0.f ? amax / QMAX * fabsf(qscale) : 0.f;
}

// ------------------------------------------------------------------------------------------ V-scale bound
// Partial maxima of v_scale (both 64-dim groups) over the cells any query of the call can see: each workgroup
// reduces one of VS_SLICES slices of KV head g's cells; the attention kernel folds the slices.
__device__ __forceinline__ void prompt_vsmax(const float *__restrict__ vs, int32_t cap, int32_t n_cells,
                                             float *__restrict__ VSp, int32_t g, int32_t sl)
{
    __shared__ float red[4];
    const int32_t per = (n_cells + VS_SLICES - 1) / VS_SLICES;
    const int32_t e0 = 2 * min(n_cells, sl * per), e1 = 2 * min(n_cells, (sl + 1) * per);
    float m = 0.f;
    for (int32_t e = e0 + threadIdx.x; e < e1; e += 256) m = fmaxf(m, vs[(int64_t)g * cap * 2 + e]);
    m = group_max<64>(m);
    if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = m;
    __syncthreads();
    if (threadIdx.x == 0) VSp[g * VS_SLICES + sl] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Both preparation steps in one launch (they are independent): the first nvb = n_kv * VS_SLICES workgroups reduce
// the v_scale slices (dispatched first, so they run beside the q split rather than after it), the rest split q.
__global__ __launch_bounds__(256) void prompt_prep_kernel(const float *__restrict__ q, int32_t n_qh, int32_t G,
                                                          int32_t R, int64_t n_rows, float qscale,
                                                          int8_t *__restrict__ qd, float *__restrict__ qs, uint32_t nvb,
                                                          const float *__restrict__ vs, int32_t cap, int32_t n_cells,
                                                          float *__restrict__ VSp)
{
    if (blockIdx.x < nvb)
        prompt_vsmax(vs, cap, n_cells, VSp, (int32_t)(blockIdx.x / VS_SLICES), (int32_t)(blockIdx.x % VS_SLICES));
    else
        prompt_qsplit(q, n_qh, G, R, n_rows, qscale, qd, qs, blockIdx.x - nvb);
}

// VS[g] from its VS_SLICES partial maxima, one per lane (lanes past them hold 0): a wave max.
__device__ __forceinline__ float head_vs(float part)
{
    static_assert(VS_SLICES <= 64, "one slice per lane");
    const float VS = group_max<64>(part);
    return VS > 0.f ? VS : 1.f;
}

// ------------------------------------------------------------------------------------------- main kernel
struct PromptArgs {
    const int8_t *qd;
    const float *qs;
    const float *VSp;  // [n_kv][VS_SLICES] partial maxima of v_scale
    PoolArg pool;
    float *m_out;
    float *l_out;
    float *o_out;
    uint8_t *e_out;
    float *out;       // written directly when S == 1
    int32_t n_q;
    int32_t pos0;
    int32_t n_qh;
    int32_t G;
    int32_t R;        // rows per KV head = n_q * G
    int32_t S;        // cell chunks per row block
};

constexpr int QROW = 3 * PD + 16;  // LDS bytes per row of q digits (padded: consecutive rows start 4 banks apart)

struct __align__(16) PromptTile {
    int8_t k[PT * PD];     // [cell][128], 16-byte chunk p of row c holds chunk p ^ swz_k(c)
    int8_t v[PT * PD];     // [cell][128], 16-byte chunk p of row c holds chunk p ^ swz_v(c)
    float ks[PT * 2];      // [cell][grp]
    float vs[PT * 2];      // [cell][grp], scaled in LDS to w = v_scale * 127 * 2^24 / VS[g]
};

// K8V4 pools: wave w stages the packed 4-bit V codes of the tile's cells 16w .. 16w + 15 (1,024 bytes, lane l holds
// cell 16w + l/4, dims 32 (l & 3) .. + 31) at the start of its own 2,048-byte share of the V slot, and once its copies
// have landed expands them in place into the int8 layout of the slot: two 16-byte chunks of the cell's row per lane.
// Every byte a wave reads lies in the rows it writes, and a wave's reads complete before its writes, so the expansion
// needs no barrier of its own; the step's barrier publishes it.
__device__ __forceinline__ uint32_t s4_lo(uint32_t u)   // signed low nibbles of the 4 bytes -> 4 int8
{
    return (((u & 0x0F0F0F0Fu) ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
}
__device__ __forceinline__ void expand_v4(int8_t *tv, int wave, int lane)
{
    const int cell = 16 * wave + (lane >> 2), pos = lane & 3;
    const v4i pk = *reinterpret_cast<const v4i *>(tv + 2048 * wave + 16 * lane);
    uint32_t o[8];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t lo = s4_lo((uint32_t)pk[k]), hi = s4_lo((uint32_t)pk[k] >> 4);   // dims 8k + 2j, 8k + 2j + 1
        o[2 * k] = bperm(hi, lo, 0x05010400u);
        o[2 * k + 1] = bperm(hi, lo, 0x07030602u);
    }
    int8_t *row = tv + cell * PD;
    *reinterpret_cast<v4i *>(row + 16 * ((2 * pos) ^ swz_v(cell))) =
        v4i{(int32_t)o[0], (int32_t)o[1], (int32_t)o[2], (int32_t)o[3]};
    *reinterpret_cast<v4i *>(row + 16 * ((2 * pos + 1) ^ swz_v(cell))) =
        v4i{(int32_t)o[4], (int32_t)o[5], (int32_t)o[6], (int32_t)o[7]};
}

template <int VB>
__global__ __launch_bounds__(256, 2) void prompt_attn_kernel(const PromptArgs a)
{
    __shared__ PromptTile tile[NBUF];
    __shared__ __align__(16) int8_t sq[PROWS * QROW];  // q digits of the workgroup's rows: [row][plane][128]
    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // scalar: LDS destinations of the tile copies
    const int n16 = lane & 15, G4 = lane >> 4;
    const int32_t g = blockIdx.z, j = blockIdx.y;
    const int32_t row0 = blockIdx.x * PROWS;
    const PoolArg P = a.pool;

    // this lane's row and its causal limit (last visible cell)
    const int32_t r = row0 + 16 * wave + n16;
    const bool row_ok = r < a.R;
    const int32_t qi = row_ok ? r / a.G : 0;
    const int32_t lim = row_ok ? min(a.pos0 + qi, P.n_valid - 1) : -1;
    // smallest limit over the wave's rows: tiles ending at or before it need no mask
    const int32_t wr0 = row0 + 16 * wave;
    const int32_t wave_lim = (wr0 + 15 < a.R) ? min(a.pos0 + wr0 / a.G, P.n_valid - 1) : -1;

    // cells the workgroup's last row can see, cut into S chunks of whole tiles
    const int32_t rlast = min(row0 + PROWS - 1, a.R - 1);
    // (64-bit: the last query may sit at position INT32_MAX)
    const int32_t c_end = (int32_t)min((int64_t)P.n_valid, (int64_t)a.pos0 + rlast / a.G + 1);
    const int32_t n_tiles = c_end > 0 ? (c_end + PT - 1) / PT : 0;
    const int32_t t0 = (int32_t)(((int64_t)n_tiles * j) / a.S), t1 = (int32_t)(((int64_t)n_tiles * (j + 1)) / a.S);
    const int32_t c_last = c_end - 1;

    // Prologue loads, all issued at once (they land while the first tiles' copies are issued): the q digits of the
    // workgroup's rows (B operands of S^T, stored to LDS below; rows past R are zero), the row's logit scale and one
    // partial maximum of v_scale per lane.
    constexpr int QV = PROWS * (3 * PD / 16) / 256;   // 16-byte q-digit loads per thread
    static_assert(QV * 256 == PROWS * (3 * PD / 16), "whole loads per thread");
    // (every load is unconditional, from a clamped index, so none waits behind a branch)
    int4 qv[QV];
#pragma unroll
    for (int u = 0; u < QV; u++) {
        const int e = tid + 256 * u, rr = e / (3 * PD / 16), k16 = e % (3 * PD / 16);
        const int32_t rg = min(row0 + rr, a.R - 1);
        qv[u] = *reinterpret_cast<const int4 *>(a.qd + ((int64_t)g * a.R + rg) * 3 * PD + 16 * k16);
    }
    const float qs_ld = a.qs[(int64_t)g * a.R + min(r, a.R - 1)];
    const float vs_ld = a.VSp[g * VS_SLICES + lane % VS_SLICES];
    const int8_t *qrow_lds = sq + (16 * wave + n16) * QROW + 16 * G4;
    // set in the prologue below: the row's logit scale (a floor keeps -inf * crow = -inf for all-zero q rows, whose
    // logits are all 0), the value of one unit of the p * w digits, and w = v_scale * vsc
    float crow = 0.f, sw = 0.f, vsc = 0.f;

    v4i acc[4][8];   // PV int32 sums per digit plane (weights 2^24, 2^16, 2^8, 1)
#pragma unroll
    for (int db = 0; db < 8; db++) acc[0][db] = acc[1][db] = acc[2][db] = acc[3][db] = v4i{0, 0, 0, 0};
    // The fp32 sums (the lane's 32 outputs of its row) change only at folds, so they live in the row's output slot
    // in global memory rather than in registers: the out row itself with one chunk, the chunk's partial otherwise.
    const int32_t hq = g * a.G + (r % a.G);
    const int64_t orow_idx = ((int64_t)qi * a.n_qh + hq) * a.S + j;
    float *const orow = (a.S == 1 ? a.out : a.o_out) + orow_idx * PD + 4 * G4;
    bool have_o = false;
    // O = (O + sum_planes acc * 2^(8 plane) * sw) * alpha, restarting the int32 sums
    auto fold = [&](float alpha, float4 (&o)[8]) {
#pragma unroll
        for (int db = 0; db < 8; db++)
            o[db] = have_o ? *reinterpret_cast<const float4 *>(orow + 16 * db) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int db = 0; db < 8; db++) {
            float part[4];
#pragma unroll
            for (int v = 0; v < 4; v++)
                part[v] = fmaf((float)acc[0][db][v], 16777216.f,
                               fmaf((float)acc[1][db][v], 65536.f, fmaf((float)acc[2][db][v], 256.f, (float)acc[3][db][v])));
            o[db] = make_float4(fmaf(part[0], sw, o[db].x) * alpha, fmaf(part[1], sw, o[db].y) * alpha,
                                fmaf(part[2], sw, o[db].z) * alpha, fmaf(part[3], sw, o[db].w) * alpha);
            acc[0][db] = acc[1][db] = acc[2][db] = acc[3][db] = v4i{0, 0, 0, 0};
        }
    };
    float lsum = 0.f, mref = -INFINITY;

    // ---- tile staging, straight from HBM into LDS: per 64-cell tile, 8 KB of K codes, 8 KB of V codes (4 KB packed
    // for K8V4) and 512 B of each scale; wave w issues 16-byte slots [128 w, 128 w + 128) of K and of V (slots
    // [64 w, 64 w + 64) of packed V) and one 64-float half of a scale array
    constexpr int VROW = VB == 8 ? PD : PD / 2;   // V bytes per cell
    constexpr int NCOPY = VB == 8 ? 5 : 4;        // copies each wave issues per tile
    constexpr int WAIT_TILE = VB == 8 ? WAIT_VM5_LGKM0 : WAIT_VM4_LGKM0;   // all but the newest tile's copies done
    static_assert((WAIT_TILE & 15) == NCOPY, "the tile wait counts one tile's copies");
    const int8_t *kg = P.k + (int64_t)g * P.capacity * PD;
    const int8_t *vg = P.v + (int64_t)g * P.capacity * VROW;
    const float *ksg = P.ks + (int64_t)g * P.capacity * 2;
    const float *vsg = P.vs + (int64_t)g * P.capacity * 2;
    // The tile's base address is wave-uniform (scalar registers); a lane's byte offset within a full tile is the
    // same for every tile, and only a tile that runs past the last cell clamps its cells.
    uint32_t koff[2], voff[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int slot = 128 * wave + 64 * h + lane;
        const int cell = slot >> 3, pos = slot & 7;
        koff[h] = cell * PD + 16 * (pos ^ swz_k(cell));
        voff[h] = cell * PD + 16 * (pos ^ swz_v(cell));
    }
    const int se = 64 * (wave & 1) + lane;   // float se of the tile's [cell][grp] scales
    // (each wave issues NCOPY copies per tile)
    auto stage = [&](int32_t t, int buf) {
        const int32_t cb = t * PT;
        PromptTile &T = tile[buf];
        const int8_t *kt = kg + (int64_t)cb * PD;
        const int8_t *vt = vg + (int64_t)cb * VROW;
        const float *st = (wave < 2 ? ksg : vsg) + (int64_t)cb * 2;
        float *sdst = (wave < 2 ? T.ks : T.vs) + 64 * (wave & 1);
        const int32_t nfull = c_last - cb;   // cells past nfull re-read cell nfull
        if (nfull >= PT - 1) {
#pragma unroll
            for (int h = 0; h < 2; h++) {
                copy_lds16(kt, koff[h], lds_addr(T.k + 1024 * (2 * wave + h)));
                if constexpr (VB == 8) copy_lds16(vt, voff[h], lds_addr(T.v + 1024 * (2 * wave + h)));
            }
            if constexpr (VB == 4) copy_lds16(vt, 1024 * wave + 16 * lane, lds_addr(T.v + 2048 * wave));
            copy_lds4(st, 4 * se, lds_addr(sdst));
        } else {
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int slot = 128 * wave + 64 * h + lane;
                const int cell = slot >> 3, pos = slot & 7, c = min(cell, nfull);
                copy_lds16(kt, c * PD + 16 * (pos ^ swz_k(cell)), lds_addr(T.k + 1024 * (2 * wave + h)));
                if constexpr (VB == 8)
                    copy_lds16(vt, c * PD + 16 * (pos ^ swz_v(cell)), lds_addr(T.v + 1024 * (2 * wave + h)));
            }
            if constexpr (VB == 4)
                copy_lds16(vt, min(16 * wave + (lane >> 2), nfull) * VROW + 16 * (lane & 3),
                           lds_addr(T.v + 2048 * wave));
            copy_lds4(st, 4 * (2 * min(se >> 1, nfull) + (se & 1)), lds_addr(sdst));
        }
    };
    // Once this wave's copies of a tile have landed (the compiler barrier keeps the LDS reads after the wait): the
    // waves that copied the v_scale halves turn them into w, and for K8V4 every wave widens its share of the V codes.
    // No branch (the K-scale waves rewrite theirs times 1), so the step's scheduler can interleave it with the
    // exponentials that follow.
    auto finish = [&](int buf) {
        PromptTile &T = tile[buf];
        asm volatile("" ::: "memory");
        float *sc = (wave < 2 ? T.ks : T.vs) + se;
        *sc = *sc * (wave >= 2 ? vsc : 1.f);
        if constexpr (VB == 4) expand_v4(T.v, wave, lane);
    };

    // Tiles are triple-buffered and prefetched two ahead: tile t lives in buffer (t - t0) % 3, its copies are issued
    // at the start of step t - 2, and each wave waits for its own in the middle of step t - 1 and finishes its share.
    if (t0 < t1) stage(t0, 0);
    if (t0 + 1 < t1) stage(t0 + 1, 1);
#pragma unroll
    for (int u = 0; u < QV; u++) {   // (the q loads are older than the copies: they land first)
        const int e = tid + 256 * u, rr = e / (3 * PD / 16), k16 = e % (3 * PD / 16);
        *reinterpret_cast<int4 *>(sq + rr * QROW + 16 * k16) = row0 + rr < a.R ? qv[u] : make_int4(0, 0, 0, 0);
    }
    crow = fmaxf(row_ok ? qs_ld : 0.f, 1e-30f);
    {
        const float VS = head_vs(lane < VS_SLICES ? vs_ld : 0.f);
        sw = VS / PMAX;
        vsc = PMAX / VS;
    }
    if (t0 + 1 < t1) __builtin_amdgcn_s_waitcnt(WAIT_TILE);   // tile t0 has landed
    else __builtin_amdgcn_s_waitcnt(WAIT_VM0_LGKM0);
    if (t0 < t1) finish(0);
    __syncthreads();

    // Tiles before t_mask end at or before the wave's smallest limit and need no causal mask; the loop is split so
    // the mask compares only run on the last tiles. Every iteration has one barrier, so the waves stay matched.
    const int32_t t_mask = wave_lim < PT - 1 ? 0 : (wave_lim - (PT - 1)) / PT + 1;
    // BUF_TAG is tile t's buffer when known at compile time (the unrolled loop), or -1: constant buffer indexes turn
    // every LDS address of the step into a loop-invariant register plus an immediate offset.
    auto step = [&](int32_t t, auto masked_tag, auto buf_tag) {
        constexpr bool masked = decltype(masked_tag)::value;
        constexpr int BUF = decltype(buf_tag)::value;
        const int buf = BUF >= 0 ? BUF : (t - t0) % NBUF;
        const int buf1 = BUF >= 0 ? (BUF + 1) % NBUF : (buf + 1 == NBUF ? 0 : buf + 1);
        const int buf2 = BUF >= 0 ? (BUF + 2) % NBUF : (buf1 + 1 == NBUF ? 0 : buf1 + 1);
        // tile t + 2 into the buffer tile t - 1 used; past the last tile the last one is copied again into a buffer
        // nobody reads any more, so that every step waits and finishes the same way, without a branch
        stage(min(t + 2, t1 - 1), buf2);
        const PromptTile &T = tile[buf];
        const int32_t cb = t * PT;

        // ---- S^T = K . Q^T, four 16-cell blocks; lane l ends with cells 16*G4 + 4b + v of row n16
        float t2[4][4];
        __builtin_amdgcn_s_setprio(1);   // MFMA sections get issue priority over the other waves' VALU work
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const int cellA = 16 * (n16 >> 2) + 4 * b + (n16 & 3);
            v4i hacc[2], lmacc[2];
#pragma unroll
            for (int grp = 0; grp < 2; grp++) {
                const int chunk = 4 * grp + G4;
                const v4i ka = *reinterpret_cast<const v4i *>(T.k + cellA * PD + 16 * (chunk ^ swz_k(cellA)));
                const v4i qh = *reinterpret_cast<const v4i *>(qrow_lds + 0 * PD + 64 * grp);
                const v4i ql = *reinterpret_cast<const v4i *>(qrow_lds + 1 * PD + 64 * grp);
                const v4i qm = *reinterpret_cast<const v4i *>(qrow_lds + 2 * PD + 64 * grp);
                hacc[grp] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka, qh, v4i{0, 0, 0, 0}, 0, 0, 0);
                v4i lm = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka, ql, v4i{0, 0, 0, 0}, 0, 0, 0);
                lm = lm << 8;
                lmacc[grp] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka, qm, lm, 0, 0, 0);
            }
            const int cl0 = 16 * G4 + 4 * b;
            const float4 ksa = *reinterpret_cast<const float4 *>(&T.ks[2 * cl0]);
            const float4 ksb = *reinterpret_cast<const float4 *>(&T.ks[2 * cl0 + 4]);
            const float k0[4] = {ksa.x, ksa.z, ksb.x, ksb.z}, k1[4] = {ksa.y, ksa.w, ksb.y, ksb.w};
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const float a0 = fmaf((float)hacc[0][v], 65536.f, (float)lmacc[0][v]);
                const float a1 = fmaf((float)hacc[1][v], 65536.f, (float)lmacc[1][v]);
                float tv = fmaf(a1, k1[v], a0 * k0[v]);   // logit / crow
                if constexpr (masked) {
                    if (cb + cl0 + v > lim) tv = -INFINITY;
                }
                t2[b][v] = tv;
            }
        }

        __builtin_amdgcn_s_setprio(0);
        // ---- row max over the tile; fold the int32 PV sums when it passes the reference
        float rm = t2[0][0];
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int v = 0; v < 4; v++) rm = fmaxf(rm, t2[b][v]);
        rm = max16(rm);
        rm = max32(rm) * crow;                       // row max in log2 units (crow > 0)
        const bool need = rm > mref;
        const bool force = ((t - t0) % FOLD_EVERY) == FOLD_EVERY - 1;   // wave-uniform
        if (__any(need) || force) {
            const float mnew = need ? rm + PDELTA : mref;
            // a row whose reference is still -inf has summed nothing (every p was 0): it only takes the reference
            const bool fold_row = (need || force) && row_ok;
            const bool store = fold_row && mref != -INFINITY;
            if (store) {   // both sums are relative to the old reference
                const float alpha = need ? __builtin_amdgcn_exp2f(mref - mnew) : 1.f;
                float4 o[8];
                fold(alpha, o);
#pragma unroll
                for (int db = 0; db < 8; db++) *reinterpret_cast<float4 *>(orow + 16 * db) = o[db];
                have_o = true;
                lsum *= alpha;
            }
            if (fold_row) mref = mnew;
            // the fold's stores are not left behind the tile copies
            if (__any(store)) __builtin_amdgcn_s_waitcnt(WAIT_VM0_LGKM0);
        }
        const float mexp = mref == -INFINITY ? 0.f : mref;

        // ---- tile t + 1, whose copies were issued a step ago, is finished here so that the exponentials and
        // splits below hide the LDS round trips (its buffer is not read before the step's closing barrier)
        __builtin_amdgcn_s_waitcnt(WAIT_TILE);
        finish(buf1);

        // ---- p = 2^(t - m_ref); the digits of p * w, per scale group, are the B operands of O^T += V^T . P^T,
        // run over the group's four 16-dim blocks. V^T rows come from two transposing reads per block.
        float p[4][4];
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                p[b][v] = __builtin_amdgcn_exp2f(fmaf(t2[b][v], crow, -mexp));
                lsum += p[b][v];
            }
        const int i = n16 >> 1, hh = n16 & 1;
        const int c0 = 16 * G4 + i, c1 = c0 + 8;   // (c & 7) == i for both
        v4i pd[2][4];   // [group][digit plane d3, d2, d1, d0] of the lane's 16 cells
#pragma unroll
        for (int grp = 0; grp < 2; grp++) {
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const int cl0 = 16 * G4 + 4 * b;
                const float4 wa = *reinterpret_cast<const float4 *>(&T.vs[2 * cl0]);
                const float4 wb = *reinterpret_cast<const float4 *>(&T.vs[2 * cl0 + 4]);
                const float wv[4] = {grp ? wa.y : wa.x, grp ? wa.w : wa.z, grp ? wb.y : wb.x, grp ? wb.w : wb.z};
                uint32_t u[4];
#pragma unroll
                for (int v = 0; v < 4; v++) u[v] = (uint32_t)fmaf(p[b][v], wv[v], PBIAS);
                const uint32_t A01 = bperm(u[1], u[0], 0x05010400u), B01 = bperm(u[1], u[0], 0x07030602u);
                const uint32_t A23 = bperm(u[3], u[2], 0x05010400u), B23 = bperm(u[3], u[2], 0x07030602u);
                pd[grp][3][b] = (int32_t)(bperm(A23, A01, 0x05040100u) ^ 0x80808080u);
                pd[grp][2][b] = (int32_t)(bperm(A23, A01, 0x07060302u) ^ 0x80808080u);
                pd[grp][1][b] = (int32_t)(bperm(B23, B01, 0x05040100u) ^ 0x80808080u);
                pd[grp][0][b] = (int32_t)bperm(B23, B01, 0x07060302u);
            }
        }
        // Both groups' splits first, then the 32 MFMAs as one burst: MFMA and VALU work of one wave do not overlap on
        // this chip, those of two waves on a SIMD do, so a long MFMA run gives the SIMD's other wave room to issue
        // its VALU work meanwhile.
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int grp = 0; grp < 2; grp++) {
#pragma unroll
            for (int dq = 0; dq < 4; dq++) {
                const int db = 4 * grp + dq, ch = 2 * db + hh;   // 8-byte chunk of the cell's 128-byte row
                const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (QSA_LDS v2i *)(T.v + c0 * PD + 8 * (ch ^ (2 * i))));
                const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (QSA_LDS v2i *)(T.v + c1 * PD + 8 * (ch ^ (2 * i))));
                const v4i va = v4i{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                for (int pl = 0; pl < 4; pl++)
                    acc[pl][db] = __builtin_amdgcn_mfma_i32_16x16x64_i8(va, pd[grp][pl], acc[pl][db], 0, 0, 0);
            }
        }

        __builtin_amdgcn_s_setprio(0);
        __syncthreads();
    };
    using runtime_buf = std::integral_constant<int, -1>;
    int32_t t = t0;
    const int32_t t_plain = min(t_mask, t1);
    static_assert(NBUF == 3, "the plain loop is unrolled once per buffer");
    for (; t + NBUF <= t_plain; t += NBUF) {   // (t - t0) % NBUF == 0 here
        step(t, std::false_type{}, std::integral_constant<int, 0>{});
        step(t + 1, std::false_type{}, std::integral_constant<int, 1>{});
        step(t + 2, std::false_type{}, std::integral_constant<int, 2>{});
    }
    for (; t < t_plain; t++) step(t, std::false_type{}, runtime_buf{});
    for (; t < t1; t++) step(t, std::true_type{}, runtime_buf{});
    __builtin_amdgcn_s_waitcnt(WAIT_VM0_LGKM0);   // the repeated copies of the last steps have landed

    // ---- final fold and output
    lsum = sum16(lsum);
    lsum = sum32(lsum);
    if (!row_ok) return;
    const bool empty = mref == -INFINITY;
    float4 o[8];
    fold(1.f, o);
    if (a.S == 1) {
        const float inv = empty ? 0.f : 1.f / lsum;
#pragma unroll
        for (int db = 0; db < 8; db++)
            *reinterpret_cast<float4 *>(orow + 16 * db) =
                make_float4(o[db].x * inv, o[db].y * inv, o[db].z * inv, o[db].w * inv);
    } else {
#pragma unroll
        for (int db = 0; db < 8; db++)
            *reinterpret_cast<float4 *>(orow + 16 * db) = empty ? make_float4(0.f, 0.f, 0.f, 0.f) : o[db];
        if (G4 == 0) {
            a.m_out[orow_idx] = empty ? -INFINITY : mref * PLN2;
            a.l_out[orow_idx] = empty ? 0.f : lsum;
            a.e_out[orow_idx] = empty ? 1 : 0;
        }
    }
}

// ------------------------------------------------------------------------------------------- chunk merge
// The S cell chunks of each (query, q head) row folded as the decode merge folds them: M over the non-empty chunks,
// weights e^(m_j - M) added in chunk order, empty chunks skipped by select (their o may hold anything), a row with
// none gets zeros. 32 lanes per row with four dims each, 8 rows per 256-thread workgroup, no cross-lane work. Up to
// NS = 4 chunks every load of a row is issued before the first use; more chunks (small calls) take a loop.
constexpr int MAX_S = 32;   // cell chunks per row block at most

template <int NS>
__global__ __launch_bounds__(256) void prompt_merge_kernel(const float *__restrict__ m, const float *__restrict__ l,
                                                           const uint8_t *__restrict__ em, const float *__restrict__ o,
                                                           int32_t S, int64_t rows, float *__restrict__ out)
{
    const int64_t row = (int64_t)blockIdx.x * 8 + threadIdx.x / 32;
    if (row >= rows) return;
    const int dl = threadIdx.x % 32;
    if constexpr (NS == 0) {
        // lane dl of the row holds chunk dl's (m, l, empty) (S <= MAX_S = 32 lanes): M and the weights in one round
        // of loads and a 32-lane max; the o rows are then loaded eight chunks at a time, every load unconditional
        // (an empty chunk's row is read but skipped by select)
        static_assert(MAX_S <= 32, "one chunk per lane of the row's 32");
        const bool in = dl < S;
        const int64_t e0 = row * S;
        const float mj = in ? m[e0 + dl] : -INFINITY;
        const float lj = in ? l[e0 + dl] : 0.f;
        const bool live = in && em[e0 + dl] == 0;
        const float M = max16(group_max<16>(live ? mj : -INFINITY));   // over the row's 32 lanes
        const float w = live ? expf(mj - M) : 0.f;
        const float L = sum16(group_sum<16>(live ? w * lj : 0.f));
        const int base = threadIdx.x & 32;   // the row's first lane in the wave
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int32_t j0 = 0; j0 < S; j0 += 8) {
            float4 ov[8];
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const int32_t jj = j0 + u < S ? j0 + u : S - 1;
                ov[u] = *reinterpret_cast<const float4 *>(o + (e0 + jj) * PD + 4 * dl);
            }
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const int src = base + ((j0 + u) & 31);
                const float wu = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * src, __float_as_int(w)));
                const bool lu = j0 + u < S && wu > 0.f;
                acc = lu ? make_float4(fmaf(wu, ov[u].x, acc.x), fmaf(wu, ov[u].y, acc.y), fmaf(wu, ov[u].z, acc.z),
                                       fmaf(wu, ov[u].w, acc.w))
                         : acc;
            }
        }
        *reinterpret_cast<float4 *>(out + row * PD + 4 * dl) = M == -INFINITY
            ? make_float4(0.f, 0.f, 0.f, 0.f) : make_float4(acc.x / L, acc.y / L, acc.z / L, acc.w / L);
        return;
    }
    constexpr int N = NS > 0 ? NS : 1;
    float4 ov[N];
    float mv[N], lv[N];
    bool live[N];
#pragma unroll
    for (int j = 0; j < N; j++) {
        if (j < S) {
            const int64_t e = row * S + j;
            ov[j] = *reinterpret_cast<const float4 *>(o + e * PD + 4 * dl);
            mv[j] = m[e];
            lv[j] = l[e];
            live[j] = em[e] == 0;
        } else {
            ov[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            mv[j] = lv[j] = 0.f;
            live[j] = false;
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < N; j++) M = live[j] ? fmaxf(M, mv[j]) : M;
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < N; j++) {
        if (live[j]) {
            const float w = expf(mv[j] - M);
            L = fmaf(w, lv[j], L);
            acc = make_float4(fmaf(w, ov[j].x, acc.x), fmaf(w, ov[j].y, acc.y), fmaf(w, ov[j].z, acc.z),
                              fmaf(w, ov[j].w, acc.w));
        }
    }
    const bool none = M == -INFINITY;
    *reinterpret_cast<float4 *>(out + row * PD + 4 * dl) =
        none ? make_float4(0.f, 0.f, 0.f, 0.f) : make_float4(acc.x / L, acc.y / L, acc.z / L, acc.w / L);
}

// Cell chunks per row block (at most MAX_S): the S that minimises rounds of workgroups (two per CU) times the tiles a
// workgroup walks, plus two tiles' worth of start-up and store per workgroup, the smaller S on a tie. `last` (pos0 +
// n_q) stands for the cells the call sees, so the choice and the scratch size depend on the arguments alone. The
// 2,048-query chunk at a 32K context gets 2 (three full rounds); a handful of queries gets up to 32, so its few
// row blocks still spread over the chip.
int prompt_chunks(int32_t n_q, int64_t last, const qsa_dims &d)
{
    const int64_t R = (int64_t)n_q * (d.n_q_heads / d.n_kv_heads);
    const int64_t wg = d.n_kv_heads * ((R + PROWS - 1) / PROWS);
    if (wg <= 0) return 1;
    const int64_t slots = 2 * NCU, tiles = (last + PT - 1) / PT;
    int best = 1;
    int64_t best_cost = INT64_MAX;
    for (int S = 1; S <= MAX_S; S++) {
        const int64_t rounds = (wg * S + slots - 1) / slots;
        const int64_t cost = rounds * ((tiles + S - 1) / S + 2);
        if (cost < best_cost) {
            best_cost = cost;
            best = S;
        }
    }
    return best;
}

struct PromptScratch {
    size_t qd, qs, vs, m, l, o, e, total;
};

PromptScratch prompt_layout(int32_t n_q, int64_t last, const qsa_dims &d)
{
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t rows = (size_t)n_q * d.n_q_heads;
    const int S = prompt_chunks(n_q, last, d);
    PromptScratch s{};
    size_t off = 0;
    s.qd = off; off += al(rows * 3 * PD);
    s.qs = off; off += al(rows * sizeof(float));
    s.vs = off; off += al((size_t)d.n_kv_heads * VS_SLICES * sizeof(float));
    if (S > 1) {
        s.m = off; off += al(rows * S * sizeof(float));
        s.l = off; off += al(rows * S * sizeof(float));
        s.e = off; off += al(rows * S);
        s.o = off; off += al(rows * S * PD * sizeof(float));
    }
    s.total = off;
    return s;
}

// ------------------------------------------------------------------------------------------- other head dims
// The matrix-core kernel above covers head_dim 128 (int8 and K8V4 pools). The other head dims the decode kernels
// support (64 and 256, K8V4 at 256) take the chunk attention kernel in dense mode -- query i as a row at position
// pos0 + i over blocks of its visible cells, split in up to FB_MAX_CHUNKS chunks -- and the log-sum-exp merge,
// FB_BATCH queries at a time so that the partials stay small. Same result (softmax attention over the visible cells),
// on the VALU or the fp16 matrix cores instead of the int8 digit products, and every query reads its own cells, so it
// is much slower.
constexpr int32_t FB_BATCH = 64, FB_MAX_CHUNKS = 32;

struct DenseLayout {
    size_t pos, m, l, e, o, total;
    int32_t batch, chunks;   // queries per batch, chunk slots per row
};

DenseLayout dense_layout(int32_t n_q, int64_t n_cells, const qsa_dims &d)
{
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    DenseLayout s{};
    s.batch = n_q < FB_BATCH ? n_q : FB_BATCH;
    const int64_t n_blocks = (n_cells + QSA_BLOCK - 1) / QSA_BLOCK;
    s.chunks = (int32_t)(n_blocks < 1 ? 1 : (n_blocks < FB_MAX_CHUNKS ? n_blocks : FB_MAX_CHUNKS));
    const size_t rh = (size_t)s.batch * d.n_q_heads * s.chunks;
    size_t off = 0;
    s.pos = off; off += al((size_t)n_q * sizeof(int32_t));
    s.m = off; off += al(rh * sizeof(float));
    s.l = off; off += al(rh * sizeof(float));
    s.e = off; off += al(rh);
    s.o = off; off += al(rh * d.head_dim * sizeof(float));
    s.total = off;
    return s;
}

__global__ __launch_bounds__(256) void prompt_pos_kernel(int32_t *__restrict__ pos, int32_t n_q, int32_t pos0)
{
    const int32_t i = (int32_t)(blockIdx.x * 256 + threadIdx.x);
    if (i < n_q) pos[i] = pos0 + i;
}

// Validated by qsa_prompt_attn (dims, pool, pointers, n_q > 0, positions in range).
qsa_status prompt_dense(const float *q, int32_t n_q, int32_t pos0, const qsa_pool *pool, const qsa_dims &dims,
                        float sm_scale, float *out, void *scratch, size_t scratch_bytes, hipStream_t s)
{
    const int64_t last = (int64_t)pos0 + n_q;
    const DenseLayout lay = dense_layout(n_q, last, dims);
    if (!scratch) return QSA_ERR_NULL;
    if (scratch_bytes < lay.total) return QSA_ERR_SCRATCH;
    // chunks over the blocks holding the cells the call can see: balanced runs of blocks, at most lay.chunks of them
    const int64_t n_cells = last < pool->n_valid ? last : pool->n_valid;
    const int32_t n_blocks = (int32_t)((n_cells + QSA_BLOCK - 1) / QSA_BLOCK);
    const int32_t want = n_blocks < 1 ? 1 : (n_blocks < lay.chunks ? n_blocks : lay.chunks);
    const int32_t bpc = n_blocks < 1 ? 1 : (n_blocks + want - 1) / want;
    const int32_t n_chunks = n_blocks < 1 ? 1 : (n_blocks + bpc - 1) / bpc;
    char *base = static_cast<char *>(scratch);
    int32_t *pos = reinterpret_cast<int32_t *>(base + lay.pos);
    qsa_partials parts{reinterpret_cast<float *>(base + lay.m), reinterpret_cast<float *>(base + lay.l),
                       reinterpret_cast<float *>(base + lay.o), reinterpret_cast<uint8_t *>(base + lay.e), lay.chunks};
    prompt_pos_kernel<<<dim3((uint32_t)((n_q + 255) / 256)), 256, 0, s>>>(pos, n_q, pos0);
    qsa_status st = launch_status();
    const int64_t row = (int64_t)dims.n_q_heads * dims.head_dim;
    for (int32_t b0 = 0; b0 < n_q && st == QSA_OK; b0 += lay.batch) {
        const int32_t nb = n_q - b0 < lay.batch ? n_q - b0 : lay.batch;
        st = qsa_attn_chunk(q + b0 * row, pos + b0, nb, pool, 1, nullptr, dims, nullptr, nullptr, 0, bpc, n_chunks,
                            sm_scale, &parts, s);
        if (st == QSA_OK) st = qsa_attn_merge(&parts, nb, dims, n_chunks, nullptr, out + b0 * row, nullptr, s);
    }
    return st;
}

}  // namespace qsa

using namespace qsa;

extern "C" size_t qsa_prompt_scratch_bytes(int32_t n_q, int32_t pos0, qsa_dims dims)
{
    if (n_q <= 0 || pos0 < 0 || check_dims(dims) != QSA_OK) return 0;
    if ((int64_t)n_q * dims.n_q_heads > INT32_MAX) return 0;
    const int64_t last = (int64_t)pos0 + n_q;
    // head_dim 128 runs the matrix-core kernel (int8 or K8V4 pools alike), the other head dims the dense chunk path
    return dims.head_dim == PD ? prompt_layout(n_q, last, dims).total : dense_layout(n_q, last, dims).total;
}

extern "C" qsa_status qsa_prompt_attn(const float *q, int32_t n_q, int32_t pos0, const qsa_pool *pool, qsa_dims dims,
                                      float sm_scale, float *out, void *scratch, size_t scratch_bytes,
                                      qsa_stream_t stream)
{
    qsa_status st = check_dims(dims);
    if (st != QSA_OK) return st;
    if ((st = check_pool(pool, true)) != QSA_OK) return st;
    if (!q || !out) return QSA_ERR_NULL;
    if (n_q < 0 || pos0 < 0 || (int64_t)pos0 + n_q - 1 > INT32_MAX || !scale_ok(sm_scale)) return QSA_ERR_RANGE;
    if (!common_v_bits(pool, 1, dims.head_dim)) return QSA_ERR_UNSUPPORTED;   // K8V4 needs head_dim >= 128
    if ((int64_t)n_q * dims.n_q_heads > INT32_MAX) return QSA_ERR_UNSUPPORTED;   // (query, head) rows index grids
    if (n_q == 0) return QSA_OK;
    if (!scratch) return QSA_ERR_NULL;
    // the size qsa_prompt_scratch_bytes reports, whatever the pool's V format
    if (scratch_bytes < qsa_prompt_scratch_bytes(n_q, pos0, dims)) return QSA_ERR_SCRATCH;
    if (dims.head_dim != PD)
        return prompt_dense(q, n_q, pos0, pool, dims, sm_scale, out, scratch, scratch_bytes, (hipStream_t)stream);
    const int64_t last = (int64_t)pos0 + n_q;
    const int32_t n_cells = (int32_t)(last < pool->n_valid ? last : pool->n_valid);
    const PromptScratch lay = prompt_layout(n_q, last, dims);
    const int32_t G = dims.n_q_heads / dims.n_kv_heads;
    const int64_t R = (int64_t)n_q * G;
    if (R > (int64_t)1 << 30) return QSA_ERR_UNSUPPORTED;
    const int S = prompt_chunks(n_q, last, dims);
    char *base = static_cast<char *>(scratch);
    hipStream_t s = (hipStream_t)stream;

    int8_t *qd = reinterpret_cast<int8_t *>(base + lay.qd);
    float *qs = reinterpret_cast<float *>(base + lay.qs);
    float *VSp = reinterpret_cast<float *>(base + lay.vs);
    const int64_t n_rows = (int64_t)n_q * dims.n_q_heads;
    const uint32_t nvb = (uint32_t)dims.n_kv_heads * VS_SLICES;
    prompt_prep_kernel<<<dim3(nvb + (uint32_t)((n_rows + 3) / 4)), 256, 0, s>>>(
        q, dims.n_q_heads, G, (int32_t)R, n_rows, sm_scale * PLOG2E, qd, qs, nvb, pool->v_scale, pool->capacity,
        n_cells, VSp);

    PromptArgs a{};
    a.qd = qd; a.qs = qs; a.VSp = VSp;
    a.pool = PoolArg{pool->k, pool->k_scale, pool->v, pool->v_scale, pool->capacity, pool->n_valid};
    a.out = out;
    a.n_q = n_q; a.pos0 = pos0; a.n_qh = dims.n_q_heads; a.G = G; a.R = (int32_t)R; a.S = S;
    if (S > 1) {
        a.m_out = reinterpret_cast<float *>(base + lay.m);
        a.l_out = reinterpret_cast<float *>(base + lay.l);
        a.e_out = reinterpret_cast<uint8_t *>(base + lay.e);
        a.o_out = reinterpret_cast<float *>(base + lay.o);
    }
    dim3 grid((uint32_t)((R + PROWS - 1) / PROWS), S, dims.n_kv_heads);
    if (v_bits_of(*pool) == 8) prompt_attn_kernel<8><<<grid, 256, 0, s>>>(a);
    else prompt_attn_kernel<4><<<grid, 256, 0, s>>>(a);
    if ((st = launch_status()) != QSA_OK) return st;
    if (S > 1) {
        const int64_t rows = (int64_t)n_q * dims.n_q_heads;
        const dim3 mgrid((uint32_t)((rows + 7) / 8));
        if (S <= 4) prompt_merge_kernel<4><<<mgrid, 256, 0, s>>>(a.m_out, a.l_out, a.e_out, a.o_out, S, rows, out);
        else prompt_merge_kernel<0><<<mgrid, 256, 0, s>>>(a.m_out, a.l_out, a.e_out, a.o_out, S, rows, out);
        return launch_status();
    }
    return QSA_OK;
}
