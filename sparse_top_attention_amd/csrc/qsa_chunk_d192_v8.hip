// Instantiations of the chunk kernels for head dim 192 with 8-bit V codes.
#include "qsa_chunk.h"

namespace qsa {
void launch_chunk_192_8(int G, int wpc, dim3 grid, hipStream_t s, const ChunkArgs &a)
{
    launch_chunk<192, 8>(G, wpc, grid, s, a);
}
}  // namespace qsa
