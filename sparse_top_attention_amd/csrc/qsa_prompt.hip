// Prompt-chunk attention on gfx950 int8 matrix cores (v_mfma_i32_16x16x64_i8).
//
// Both products run on the int8 K/V codes as stored. The other operand of each product is split into three
// exact signed bytes (X = 65536 h + 256 l + m), so every int32 sum is exact and only the recombination is fp32:
//   q    : one scale per (query, head) maps max |q| to 127, X = rint(q * 127 * 65536 / max|q|);
//   p*vs : p = 2^(t - m_ref) <= 1 and vs <= VS[g][grp] (max over the visible cells), X = rint(p vs 127 65536 / VS).
//
// Orientation. With row = (query, q head) and lane l of a wave owning row l % 16:
//   S^T[cell][row] = K[cell][:] . Q^T        (A = K codes from LDS, B = q digits from LDS)
//   O^T[dim][row]  = V^T[dim][cell] . P^T    (A = V^T from LDS,      B = p digits straight from S^T's registers)
// The 16x16 result of an MFMA puts rows 4*(l/16) + v (v = 0..3) of column l % 16 in lane l. In S^T block b the
// A-row 4G + v is loaded with cell 16G + 4b + v, so after the four blocks of a 64-cell tile lane l holds the 16
// cells 16G .. 16G + 15 (G = l / 16) of its row -- exactly the k-slots lane l must supply as the B operand of the
// PV product, and the same cells V^T's row chunk G holds. P never leaves registers.
//
// The PV int32 sums are accumulated across tiles while the reference max m_ref of a row does not move; when a tile's
// row max exceeds m_ref, the wave folds the int32 sums into fp32 (rescaled by 2^(m_old - m_new)) and restarts them,
// with m_ref set DELTA above the new max so that later small increases need no fold.
#include "qsa_internal.h"

namespace qsa {

typedef int32_t v4i __attribute__((ext_vector_type(4)));

constexpr int PD = 128;          // head dim of the prompt kernel
constexpr int PT = 64;           // cells per tile
constexpr int PW = 4;            // waves per workgroup
constexpr int PROWS = 16 * PW;   // rows (query, head) per workgroup
constexpr float PLOG2E = 1.4426950408889634f;
constexpr float PLN2 = 0.6931471805599453f;
constexpr float PDELTA = 2.0f;   // headroom (log2 units) added to the reference max at a fold
constexpr float MAGIC = 8388608.0f;                 // 2^23: fp32 with ulp 1 on [2^23, 2^24)
constexpr uint32_t MAGIC_BIAS = 0x4A7F7F80u;        // bits(2^23) - 0x808080
constexpr int NCU = 256;                            // compute units of an MI355X

// 16-byte chunk swizzles for the LDS tiles (K rows of 128 B, V^T rows of 64 B)
__device__ __forceinline__ int swz_k(int cell) { return (cell & 3) | ((cell >> 2) & 4); }
__device__ __forceinline__ int swz_v(int dim) { return (dim >> 1) & 3; }

__device__ __forceinline__ uint32_t bperm(uint32_t s0, uint32_t s1, uint32_t sel)
{
    return __builtin_amdgcn_perm(s0, s1, sel);
}

// ---------------------------------------------------------------------------------------------- q digits
// One wave per (query, q head): qd[g][r][plane][d] int8 with r = query * G + head-in-group, plane 0/1/2 = h/l/m,
// and qs[g][r] = max|q| / (127 * 65536) * sm_scale * log2(e) so that q . k * sm_scale * log2(e) = qs * (X . k).
__global__ __launch_bounds__(64) void prompt_qsplit_kernel(const float *__restrict__ q, int32_t n_qh, int32_t G,
                                                           int32_t R, float qscale, int8_t *__restrict__ qd,
                                                           float *__restrict__ qs)
{
    const int lane = threadIdx.x;
    const int32_t qi = blockIdx.x / n_qh, h = blockIdx.x % n_qh;
    const int32_t g = h / G, r = qi * G + h % G;
    const float2 x = reinterpret_cast<const float2 *>(q + (int64_t)blockIdx.x * PD)[lane];
    const float amax = group_max<64>(fmaxf(fabsf(x.x), fabsf(x.y)));
    const float s = amax > 0.f ? (127.0f * 65536.0f) / amax : 0.f;
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
    if (lane == 0) qs[(int64_t)g * R + r] = amax > 0.f ? amax / (127.0f * 65536.0f) * qscale : 0.f;
}

// ------------------------------------------------------------------------------------------ V-scale bound
// VS[g][grp] = max of v_scale over the cells any query of the call can see (1 when there is none).
__global__ __launch_bounds__(256) void prompt_vsmax_kernel(const float *__restrict__ vs, int32_t cap, int32_t n_cells,
                                                           float *__restrict__ VS)
{
    __shared__ float red[4];
    const int32_t g = blockIdx.x / 2, grp = blockIdx.x % 2;
    float m = 0.f;
    for (int32_t c = threadIdx.x; c < n_cells; c += 256) m = fmaxf(m, vs[((int64_t)g * cap + c) * 2 + grp]);
    m = group_max<64>(m);
    if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        const float t = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        VS[blockIdx.x] = t > 0.f ? t : 1.f;
    }
}

// ------------------------------------------------------------------------------------------- main kernel
struct PromptArgs {
    const int8_t *qd;
    const float *qs;
    const float *VS;
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
    int8_t k[PT * PD];     // [cell][128], 16-byte chunks swizzled by swz_k(cell)
    int8_t vt[PD * PT];    // [dim][64],   16-byte chunks swizzled by swz_v(dim)
    float ks[PT * 2];      // [cell][grp]
    float vs[PT * 2];      // [cell][grp], scaled by 127 * 65536 / VS[grp]
};

__global__ __launch_bounds__(256, 2) void prompt_attn_kernel(const PromptArgs a)
{
    __shared__ PromptTile tile[2];
    __shared__ __align__(16) int8_t sq[PROWS * QROW];  // q digits of the workgroup's rows: [row][plane][128]
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
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
    const int32_t c_end = min(P.n_valid, a.pos0 + rlast / a.G + 1);
    const int32_t n_tiles = c_end > 0 ? (c_end + PT - 1) / PT : 0;
    const int32_t t0 = (int32_t)(((int64_t)n_tiles * j) / a.S), t1 = (int32_t)(((int64_t)n_tiles * (j + 1)) / a.S);
    const int32_t c_last = c_end - 1;

    // q digits of the workgroup's rows (B operands of S^T) into LDS; rows past R are zero
    for (int e = tid; e < PROWS * (3 * PD / 16); e += 256) {
        const int rr = e / (3 * PD / 16), k16 = e % (3 * PD / 16);
        const int32_t rg = row0 + rr;
        int4 v = make_int4(0, 0, 0, 0);
        if (rg < a.R) v = *reinterpret_cast<const int4 *>(a.qd + ((int64_t)g * a.R + rg) * 3 * PD + 16 * k16);
        *reinterpret_cast<int4 *>(sq + rr * QROW + 16 * k16) = v;
    }
    const int8_t *qrow_lds = sq + (16 * wave + n16) * QROW + 16 * G4;
    const float crow = row_ok ? a.qs[(int64_t)g * a.R + r] : 0.f;
    const float VS0 = a.VS[2 * g], VS1 = a.VS[2 * g + 1];
    const float vsc0 = (127.0f * 65536.0f) / VS0, vsc1 = (127.0f * 65536.0f) / VS1;
    const float sw0 = VS0 / (127.0f * 65536.0f), sw1 = VS1 / (127.0f * 65536.0f);

    v4i accH[8], accL[8], accM[8];
    float O[8][4];
#pragma unroll
    for (int db = 0; db < 8; db++) {
        accH[db] = accL[db] = accM[db] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int v = 0; v < 4; v++) O[db][v] = 0.f;
    }
    float lsum = 0.f, mref = -INFINITY;

    // ---- tile staging: registers first (global loads in flight), then LDS
    const int8_t *kg = P.k + (int64_t)g * P.capacity * PD;
    const int8_t *vg = P.v + (int64_t)g * P.capacity * PD;
    const float *ksg = P.ks + (int64_t)g * P.capacity * 2;
    const float *vsg = P.vs + (int64_t)g * P.capacity * 2;
    int4 kst[2];
    int2 vst[4];
    float2 kss, vss;
    auto stage = [&](int32_t t) {
        const int32_t cb = t * PT;
        {
            const int32_t c = min(cb + tid / 4, c_last);
            const int4 *src = reinterpret_cast<const int4 *>(kg + (int64_t)c * PD + 32 * (tid % 4));
            kst[0] = src[0];
            kst[1] = src[1];
        }
#pragma unroll
        for (int k4 = 0; k4 < 4; k4++) {
            const int32_t c = min(cb + 4 * (tid % 16) + k4, c_last);
            vst[k4] = *reinterpret_cast<const int2 *>(vg + (int64_t)c * PD + 8 * (tid / 16));
        }
        if (tid < PT) {
            const int32_t c = min(cb + tid, c_last);
            kss = *reinterpret_cast<const float2 *>(ksg + (int64_t)c * 2);
            vss = *reinterpret_cast<const float2 *>(vsg + (int64_t)c * 2);
        }
    };
    auto commit = [&](int buf) {
        PromptTile &T = tile[buf];
        {
            const int cell = tid / 4;
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int chunk = 2 * (tid % 4) + h;
                *reinterpret_cast<int4 *>(T.k + cell * PD + 16 * (chunk ^ swz_k(cell))) = kst[h];
            }
        }
        {
            // 4 cells x 8 dims -> 8 dwords of 4 cells each (one per dim)
            uint32_t lo[4], hi[4];
#pragma unroll
            for (int k4 = 0; k4 < 4; k4++) {
                lo[k4] = (uint32_t)vst[k4].x;
                hi[k4] = (uint32_t)vst[k4].y;
            }
            uint32_t dcol[8];
#pragma unroll
            for (int half = 0; half < 2; half++) {
                const uint32_t *w = half ? hi : lo;
                const uint32_t A01 = bperm(w[1], w[0], 0x05010400u), C01 = bperm(w[1], w[0], 0x07030602u);
                const uint32_t A23 = bperm(w[3], w[2], 0x05010400u), C23 = bperm(w[3], w[2], 0x07030602u);
                dcol[4 * half + 0] = bperm(A23, A01, 0x05040100u);
                dcol[4 * half + 1] = bperm(A23, A01, 0x07060302u);
                dcol[4 * half + 2] = bperm(C23, C01, 0x05040100u);
                dcol[4 * half + 3] = bperm(C23, C01, 0x07060302u);
            }
            const int cell0 = 4 * (tid % 16), chunk = cell0 / 16, within = cell0 % 16;
#pragma unroll
            for (int dd = 0; dd < 8; dd++) {
                const int dim = 8 * (tid / 16) + dd;
                *reinterpret_cast<uint32_t *>(T.vt + dim * PT + 16 * (chunk ^ swz_v(dim)) + within) = dcol[dd];
            }
        }
        if (tid < PT) {
            T.ks[2 * tid] = kss.x;
            T.ks[2 * tid + 1] = kss.y;
            T.vs[2 * tid] = vss.x * vsc0;
            T.vs[2 * tid + 1] = vss.y * vsc1;
        }
    };

    if (t0 < t1) {
        stage(t0);
        commit(0);
    }
    __syncthreads();

    for (int32_t t = t0; t < t1; t++) {
        const int buf = (t - t0) & 1;
        if (t + 1 < t1) stage(t + 1);
        const PromptTile &T = tile[buf];
        const int32_t cb = t * PT;
        const bool masked = cb + PT - 1 > wave_lim;

        // ---- S^T = K . Q^T, four 16-cell blocks; lane l ends with cells 16*G4 + 4b + v of row n16
        float t2[4][4];
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
                float tv = fmaf(a1, k1[v], a0 * k0[v]) * crow;
                if (masked && cb + cl0 + v > lim) tv = -INFINITY;
                t2[b][v] = tv;
            }
        }

        // ---- row max over the tile; fold the int32 PV sums when it passes the reference
        float rm = t2[0][0];
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int v = 0; v < 4; v++) rm = fmaxf(rm, t2[b][v]);
        rm = max16(rm);
        rm = max32(rm);
        const bool need = rm > mref;
        if (__any(need)) {
            const float mnew = need ? rm + PDELTA : mref;
            const float alpha = need ? __builtin_amdgcn_exp2f(mref - mnew) : 1.f;
#pragma unroll
            for (int db = 0; db < 8; db++) {
                const float sw = db < 4 ? sw0 : sw1;
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    const float part = fmaf((float)accH[db][v], 65536.f,
                                            fmaf((float)accL[db][v], 256.f, (float)accM[db][v]));
                    O[db][v] = fmaf(part, sw, O[db][v]) * alpha;   // both are relative to the old reference
                }
                accH[db] = accL[db] = accM[db] = v4i{0, 0, 0, 0};
            }
            lsum *= alpha;
            mref = mnew;
        }
        const float mexp = mref == -INFINITY ? 0.f : mref;

        // ---- p, its digits per scale group, packed as the B operands of O^T
        v4i ph[2], pl[2], pm[2];
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const int cl0 = 16 * G4 + 4 * b;
            const float4 vsa = *reinterpret_cast<const float4 *>(&T.vs[2 * cl0]);
            const float4 vsb = *reinterpret_cast<const float4 *>(&T.vs[2 * cl0 + 4]);
            const float w0[4] = {vsa.x, vsa.z, vsb.x, vsb.z}, w1[4] = {vsa.y, vsa.w, vsb.y, vsb.w};
            uint32_t u0[4], u1[4];
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const float p = __builtin_amdgcn_exp2f(t2[b][v] - mexp);
                lsum += p;
                u0[v] = __float_as_uint(fmaf(p, w0[v], MAGIC)) - MAGIC_BIAS;
                u1[v] = __float_as_uint(fmaf(p, w1[v], MAGIC)) - MAGIC_BIAS;
            }
#pragma unroll
            for (int grp = 0; grp < 2; grp++) {
                const uint32_t *u = grp ? u1 : u0;
                const uint32_t A01 = bperm(u[1], u[0], 0x05010400u), B01 = bperm(u[1], u[0], 0x0c0c0602u);
                const uint32_t A23 = bperm(u[3], u[2], 0x05010400u), B23 = bperm(u[3], u[2], 0x0c0c0602u);
                pm[grp][b] = (int32_t)(bperm(A23, A01, 0x05040100u) ^ 0x80808080u);
                pl[grp][b] = (int32_t)(bperm(A23, A01, 0x07060302u) ^ 0x80808080u);
                ph[grp][b] = (int32_t)(bperm(B23, B01, 0x05040100u) ^ 0x80808080u);
            }
        }

        // ---- O^T += V^T . P^T over 8 blocks of 16 dims
#pragma unroll
        for (int db = 0; db < 8; db++) {
            const int grp = db >> 2, dim = 16 * db + n16;
            const v4i va = *reinterpret_cast<const v4i *>(T.vt + dim * PT + 16 * (G4 ^ swz_v(dim)));
            accH[db] = __builtin_amdgcn_mfma_i32_16x16x64_i8(va, ph[grp], accH[db], 0, 0, 0);
            accL[db] = __builtin_amdgcn_mfma_i32_16x16x64_i8(va, pl[grp], accL[db], 0, 0, 0);
            accM[db] = __builtin_amdgcn_mfma_i32_16x16x64_i8(va, pm[grp], accM[db], 0, 0, 0);
        }

        if (t + 1 < t1) commit(buf ^ 1);
        __syncthreads();
    }

    // ---- final fold and output
#pragma unroll
    for (int db = 0; db < 8; db++) {
        const float sw = db < 4 ? sw0 : sw1;
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const float part = fmaf((float)accH[db][v], 65536.f, fmaf((float)accL[db][v], 256.f, (float)accM[db][v]));
            O[db][v] = fmaf(part, sw, O[db][v]);
        }
    }
    lsum = sum16(lsum);
    lsum = sum32(lsum);
    if (!row_ok) return;
    const int32_t h = g * a.G + (r % a.G);
    const bool empty = mref == -INFINITY;
    if (a.S == 1) {
        const float inv = empty ? 0.f : 1.f / lsum;
        float *dst = a.out + ((int64_t)qi * a.n_qh + h) * PD;
#pragma unroll
        for (int db = 0; db < 8; db++)
            *reinterpret_cast<float4 *>(dst + 16 * db + 4 * G4) =
                make_float4(O[db][0] * inv, O[db][1] * inv, O[db][2] * inv, O[db][3] * inv);
    } else {
        const int64_t idx = ((int64_t)qi * a.n_qh + h) * a.S + j;
        float *dst = a.o_out + idx * PD;
#pragma unroll
        for (int db = 0; db < 8; db++)
            *reinterpret_cast<float4 *>(dst + 16 * db + 4 * G4) =
                empty ? make_float4(0.f, 0.f, 0.f, 0.f) : make_float4(O[db][0], O[db][1], O[db][2], O[db][3]);
        if (G4 == 0) {
            a.m_out[idx] = empty ? -INFINITY : mref * PLN2;
            a.l_out[idx] = empty ? 0.f : lsum;
            a.e_out[idx] = empty ? 1 : 0;
        }
    }
}

// Cell chunks per row block: enough workgroups to fill the chip in whole rounds of two per CU.
int prompt_chunks(int32_t n_q, const qsa_dims &d)
{
    const int64_t R = (int64_t)n_q * (d.n_q_heads / d.n_kv_heads);
    const int64_t wg = d.n_kv_heads * ((R + PROWS - 1) / PROWS);
    if (wg <= 0) return 1;
    const int64_t slots = 2 * NCU;
    int best = 1;
    double best_eff = 0.0;
    for (int S = 1; S <= 4; S++) {
        const int64_t n = wg * S;
        const double eff = (double)n / (double)(((n + slots - 1) / slots) * slots);
        if (eff > best_eff + 0.05) {
            best_eff = eff;
            best = S;
        }
    }
    return best;
}

struct PromptScratch {
    size_t qd, qs, vs, m, l, o, e, total;
};

PromptScratch prompt_layout(int32_t n_q, const qsa_dims &d)
{
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t rows = (size_t)n_q * d.n_q_heads;
    const int S = prompt_chunks(n_q, d);
    PromptScratch s{};
    size_t off = 0;
    s.qd = off; off += al(rows * 3 * PD);
    s.qs = off; off += al(rows * sizeof(float));
    s.vs = off; off += al((size_t)d.n_kv_heads * 2 * sizeof(float));
    if (S > 1) {
        s.m = off; off += al(rows * S * sizeof(float));
        s.l = off; off += al(rows * S * sizeof(float));
        s.e = off; off += al(rows * S);
        s.o = off; off += al(rows * S * PD * sizeof(float));
    }
    s.total = off;
    return s;
}

}  // namespace qsa

using namespace qsa;

extern "C" size_t qsa_prompt_scratch_bytes(int32_t n_q, qsa_dims dims)
{
    if (n_q <= 0 || check_dims(dims) != QSA_OK || dims.head_dim != PD) return 0;
    return prompt_layout(n_q, dims).total;
}

extern "C" qsa_status qsa_prompt_attn(const float *q, int32_t n_q, int32_t pos0, const qsa_pool *pool, qsa_dims dims,
                                      float sm_scale, float *out, void *scratch, size_t scratch_bytes,
                                      qsa_stream_t stream)
{
    qsa_status st = check_dims(dims);
    if (st != QSA_OK) return st;
    if ((st = check_pool(pool, true)) != QSA_OK) return st;
    if (!q || !out) return QSA_ERR_NULL;
    if (n_q < 0 || pos0 < 0) return QSA_ERR_RANGE;
    if (dims.head_dim != PD) return QSA_ERR_UNSUPPORTED;
    if (n_q == 0) return QSA_OK;
    const PromptScratch lay = prompt_layout(n_q, dims);
    if (!scratch) return QSA_ERR_NULL;
    if (scratch_bytes < lay.total) return QSA_ERR_SCRATCH;
    const int32_t G = dims.n_q_heads / dims.n_kv_heads;
    const int64_t R = (int64_t)n_q * G;
    if (R > (int64_t)1 << 30) return QSA_ERR_UNSUPPORTED;
    const int S = prompt_chunks(n_q, dims);
    char *base = static_cast<char *>(scratch);
    hipStream_t s = (hipStream_t)stream;

    int8_t *qd = reinterpret_cast<int8_t *>(base + lay.qd);
    float *qs = reinterpret_cast<float *>(base + lay.qs);
    float *VS = reinterpret_cast<float *>(base + lay.vs);
    prompt_qsplit_kernel<<<dim3((uint32_t)n_q * dims.n_q_heads), 64, 0, s>>>(q, dims.n_q_heads, G, (int32_t)R,
                                                                             sm_scale * PLOG2E, qd, qs);
    const int64_t last = (int64_t)pos0 + n_q;
    const int32_t n_cells = (int32_t)(last < pool->n_valid ? last : pool->n_valid);
    prompt_vsmax_kernel<<<dim3(dims.n_kv_heads * 2), 256, 0, s>>>(pool->v_scale, pool->capacity, n_cells, VS);

    PromptArgs a{};
    a.qd = qd; a.qs = qs; a.VS = VS;
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
    prompt_attn_kernel<<<grid, 256, 0, s>>>(a);
    if ((st = launch_status()) != QSA_OK) return st;
    if (S > 1) return merge_launch(a.m_out, a.l_out, a.o_out, a.e_out, S, S, nullptr, n_q, dims.n_q_heads, PD, out,
                                   nullptr, s);
    return QSA_OK;
}
