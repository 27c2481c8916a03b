// Internal helpers shared by libqsa's translation units: status plumbing on the host, and wave64 cross-lane
// primitives (DPP within a row of 16 lanes, permlane swaps across rows) on the device. gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "qsa.h"

#define QSA_BLOCK 64  // cells per selection block
#define QSA_GROUP 64  // dims per int8 scale group
#define QSA_MAX_POOLS 8

namespace qsa {

// The lane layouts cut a cell's dims into 16-dim slices (8-dim slices for the index rows) and reduce across a cell's
// slices with power-of-two cross-lane steps. head_dim 192 (12 slices) therefore runs on the layouts of 256: the lanes
// of slices past dim 191 load nothing of the row and add exact zeros.
template <int D>
constexpr int lane_dims() { return D == 192 ? 256 : D; }
inline int lane_dims(int d) { return d == 192 ? 256 : d; }

// ------------------------------------------------------------------------------------------------ host side
inline bool dims_supported(const qsa_dims &d)
{
    if (d.block_cells != QSA_BLOCK) return false;
    if (d.head_dim != 64 && d.head_dim != 128 && d.head_dim != 192 && d.head_dim != 256) return false;
    if (d.n_kv_heads <= 0 || d.n_q_heads <= 0 || d.n_q_heads % d.n_kv_heads != 0) return false;
    if (d.n_q_heads / d.n_kv_heads > 8) return false;
    if (d.n_kv_heads > 65535) return false;   // KV heads index a launch grid's y dimension
    return true;
}

inline qsa_status check_dims(const qsa_dims &d)
{
    if (d.n_q_heads <= 0 || d.n_kv_heads <= 0 || d.head_dim <= 0 || d.block_cells <= 0) return QSA_ERR_SHAPE;
    if (d.n_q_heads % d.n_kv_heads != 0) return QSA_ERR_SHAPE;
    return dims_supported(d) ? QSA_OK : QSA_ERR_UNSUPPORTED;
}

inline qsa_status check_pool(const qsa_pool *p, bool need_v)
{
    if (!p) return QSA_ERR_NULL;
    if (!p->k || !p->k_scale) return QSA_ERR_NULL;
    if (need_v && (!p->v || !p->v_scale)) return QSA_ERR_NULL;
    if (p->capacity < 0 || p->n_valid < 0) return QSA_ERR_SHAPE;
    if (p->n_valid > p->capacity) return QSA_ERR_RANGE;
    if (p->v_bits != 0 && p->v_bits != 8 && p->v_bits != 4) return QSA_ERR_UNSUPPORTED;
    return QSA_OK;
}

// A softmax scale the kernels can use (any finite value, negative and zero included).
inline bool scale_ok(float s) { return __builtin_isfinite(s); }

// V bits of a pool (0 means 8).
inline int v_bits_of(const qsa_pool &p) { return p.v_bits == 4 ? 4 : 8; }

// The V format shared by the pools of one call, or 0 when they differ or K8V4 meets an unsupported head_dim.
inline int common_v_bits(const qsa_pool *pools, int32_t n_pools, int32_t head_dim)
{
    const int vb = v_bits_of(pools[0]);
    for (int32_t p = 1; p < n_pools; p++)
        if (v_bits_of(pools[p]) != vb) return 0;
    if (vb == 4 && head_dim == 64) return 0;
    return vb;
}

// ceil(a / b) for a >= 0, b > 0, in 64 bits so that counts near INT32_MAX do not wrap.
__host__ __device__ inline int32_t ceil_div(int32_t a, int32_t b) { return (int32_t)(((int64_t)a + b - 1) / b); }

inline qsa_status launch_status()
{
    return hipGetLastError() == hipSuccess ? QSA_OK : QSA_ERR_LAUNCH;
}

// Kernel-argument copy of a pool (device pointers only).
struct PoolArg {
    const int8_t *k;
    const float *ks;
    const int8_t *v;
    const float *vs;
    int32_t capacity;
    int32_t n_valid;
    const float *index;   // block index (selection only; may be null elsewhere)
};

// Fused block scores + top-k of a decode layer: one workgroup per (KV head, row).
struct SelectArgs {
    const float *q;
    const int32_t *pos;
    const int32_t *row_pool;
    PoolArg pools[QSA_MAX_POOLS];
    int32_t n_pools;
    int32_t n_qh;
    int32_t n_kv;
    int32_t G;
    int32_t width;       // score columns (blocks) per row
    int32_t k;
    int32_t *ids;        // [n_rows][n_kv][k]
    int32_t *counts;     // [n_rows][n_kv]
    float *scores;       // optional [n_rows][n_kv][width]
};
qsa_status select_launch(const SelectArgs &a, int32_t n_rows, int32_t n_kv, int32_t head_dim, hipStream_t s);
// The score rows alone (all pools, one launch) and the radix top-k over score rows: the two launches that replace the
// fused selection kernel when a score buffer is at hand and some pool has more than SELECT_SPLIT_WIDTH live blocks
// (blocks below both the row width and the pool's valid cells; the fused kernel loads no others).
constexpr int32_t SELECT_SPLIT_WIDTH = 256;
// The decode layer's chunk kernel takes the top-k itself (from score rows written by the score launch) for rows of
// up to FUSED_TOPK_MAX_WIDTH columns and k up to FUSED_TOPK_MAX_K.
constexpr int32_t FUSED_TOPK_MAX_WIDTH = 1024, FUSED_TOPK_MAX_K = 256;
inline bool select_splits(const SelectArgs &a)
{
    int32_t live = 0;
    for (int32_t p = 0; p < a.n_pools; p++)
        live = std::max(live, std::min(a.width, ceil_div(a.pools[p].n_valid, QSA_BLOCK)));
    return live > SELECT_SPLIT_WIDTH;
}
qsa_status select_scores_launch(const SelectArgs &a, int32_t n_rows, int32_t n_kv, int32_t head_dim, hipStream_t s);
qsa_status topk_launch(const float *scores, int32_t n_rows, int32_t width, int32_t k, int32_t *ids, int32_t *counts,
                       hipStream_t s);

// Launches the log-sum-exp merge of chunk partials laid out [n_rows][n_qh][max_chunks] (+[head_dim] for o).
qsa_status merge_launch(const float *m, const float *l, const float *o, const uint8_t *empty, int32_t max_chunks,
                        int32_t n_chunks, const int32_t *n_active, int32_t n_rows, int32_t n_qh, int32_t head_dim,
                        float *out, float *lse, hipStream_t stream);

// ---------------------------------------------------------------------------------------------- device side
typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef int32_t v2i __attribute__((ext_vector_type(2)));
#define QSA_LDS __attribute__((address_space(3)))

// Global -> LDS copies (global_load_lds): lane l's bytes land at lds + size * l; lds must be wave-uniform. Written
// as inline assembly so that the compiler does not track them: it would otherwise wait for every such load (and
// for every vector load issued with them) before the next use of any loaded register or LDS byte. Kernels wait for
// them themselves with s_waitcnt vmcnt; vector loads return in issue order, so a wait the compiler emits for its
// own loads stays correct (it only becomes stricter) when these copies are in flight too.
__device__ __forceinline__ void load_lds16(const void *src, uint32_t lds)
{
    asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void load_lds4(const void *src, uint32_t lds)
{
    asm volatile("global_load_lds_dword %0, off" : : "v"(src), "{m0}"(lds) : "memory");
}
// The same copies from a wave-uniform base (scalar registers) plus a 32-bit per-lane byte offset.
__device__ __forceinline__ void copy_lds16(const void *base, uint32_t off, uint32_t lds)
{
    asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void copy_lds4(const void *base, uint32_t off, uint32_t lds)
{
    asm volatile("global_load_lds_dword %0, %1" : : "v"(off), "s"(base), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const QSA_LDS void *)p;
}

// DPP controls (gfx9 encoding).
constexpr int DPP_QUAD_XOR1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane i of each 8 -> 7 - i
constexpr int DPP_ROW_MIRROR = 0x140;       // lane i of each 16 -> 15 - i

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Pairwise combine with the lane 16 apart (within each 32) or 32 apart, via the gfx950 permlane swaps. With both
// operands equal, the swap leaves {own value, partner value} in the two result registers of every lane (which
// register holds which depends on the half), so a commutative op on the pair gives the same bits in both lanes.
__device__ __forceinline__ float sum16(float v)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}
__device__ __forceinline__ float max16(float v)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
    return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float sum32(float v)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}
__device__ __forceinline__ float max32(float v)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

// Sum / max over aligned groups of N lanes (N in {2, 4, 8, 16, 32, 64}); every lane of the group gets the result.
template <int N>
__device__ __forceinline__ float group_sum(float v)
{
    if constexpr (N >= 2) v += dpp_f<DPP_QUAD_XOR1>(v);
    if constexpr (N >= 4) v += dpp_f<DPP_QUAD_XOR2>(v);
    if constexpr (N >= 8) v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
    if constexpr (N >= 16) v += dpp_f<DPP_ROW_MIRROR>(v);
    if constexpr (N >= 32) v = sum16(v);
    if constexpr (N >= 64) v = sum32(v);
    return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v)
{
    if constexpr (N >= 2) v = fmaxf(v, dpp_f<DPP_QUAD_XOR1>(v));
    if constexpr (N >= 4) v = fmaxf(v, dpp_f<DPP_QUAD_XOR2>(v));
    if constexpr (N >= 8) v = fmaxf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
    if constexpr (N >= 16) v = fmaxf(v, dpp_f<DPP_ROW_MIRROR>(v));
    if constexpr (N >= 32) v = max16(v);
    if constexpr (N >= 64) v = max32(v);
    return v;
}

// Sum over lanes that are STRIDE apart (lanes l, l + STRIDE, l + 2 STRIDE, ... up to 64): every lane gets the
// sum over its residue class mod STRIDE. STRIDE in {1, 2, 4, 8, 16, 32, 64}.
template <int STRIDE>
__device__ __forceinline__ float strided_sum(float v)
{
    if constexpr (STRIDE <= 1) v += dpp_f<DPP_QUAD_XOR1>(v);
    if constexpr (STRIDE <= 2) v += dpp_f<DPP_QUAD_XOR2>(v);
    if constexpr (STRIDE <= 4) v += __shfl_xor(v, 4);
    if constexpr (STRIDE <= 8) v += __shfl_xor(v, 8);
    if constexpr (STRIDE <= 16) v = sum16(v);
    if constexpr (STRIDE <= 32) v = sum32(v);
    return v;
}

template <int STRIDE>
__device__ __forceinline__ float strided_max(float v)
{
    if constexpr (STRIDE <= 1) v = fmaxf(v, dpp_f<DPP_QUAD_XOR1>(v));
    if constexpr (STRIDE <= 2) v = fmaxf(v, dpp_f<DPP_QUAD_XOR2>(v));
    if constexpr (STRIDE <= 4) v = fmaxf(v, __shfl_xor(v, 4));
    if constexpr (STRIDE <= 8) v = fmaxf(v, __shfl_xor(v, 8));
    if constexpr (STRIDE <= 16) v = max16(v);
    if constexpr (STRIDE <= 32) v = max32(v);
    return v;
}

// Signed byte j of a dword, as float.
template <int J>
__device__ __forceinline__ float sbyte_f(int32_t w)
{
    return (float)((w << (24 - 8 * J)) >> 24);
}

}  // namespace qsa
