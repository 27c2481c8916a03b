// Prompt-chunk attention on int8 matrix cores (gfx950). Not implemented yet: the call validates its arguments and
// reports QSA_ERR_UNSUPPORTED without launching anything.
#include "qsa_internal.h"

using namespace qsa;

extern "C" size_t qsa_prompt_scratch_bytes(int32_t n_q, qsa_dims dims)
{
    (void)n_q; (void)dims;
    return 0;
}

extern "C" qsa_status qsa_prompt_attn(const float *q, int32_t n_q, int32_t pos0, const qsa_pool *pool, qsa_dims dims,
                                      float sm_scale, float *out, void *scratch, size_t scratch_bytes,
                                      qsa_stream_t stream)
{
    (void)sm_scale; (void)scratch; (void)scratch_bytes; (void)stream;
    qsa_status st = check_dims(dims);
    if (st != QSA_OK) return st;
    if ((st = check_pool(pool, true)) != QSA_OK) return st;
    if (!q || !out) return QSA_ERR_NULL;
    if (n_q < 0 || pos0 < 0) return QSA_ERR_RANGE;
    return QSA_ERR_UNSUPPORTED;
}
