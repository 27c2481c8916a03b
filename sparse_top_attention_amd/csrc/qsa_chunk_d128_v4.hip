// Instantiations of the chunk kernels for head dim 128 with 4-bit V codes.
#include "qsa_chunk.h"

namespace qsa {
void launch_chunk_128_4(int G, int wpc, dim3 grid, hipStream_t s, const ChunkArgs &a)
{
    launch_chunk<128, 4>(G, wpc, grid, s, a);
}
}  // namespace qsa
