// The entropy chunk pass as a launch of its own: grid (chunks, rows), each
// block reduces one chunk of one logit row to (max, sum 2^u, sum u 2^u,
// argmax) in the caller's partials (entropy_ops.hpp; hyper.ai summary of
// WeDLM, "Method": the fill rule ranks positions by their predictive entropy).
//
// Compiled without NaN semantics, as the attention launch that carries the
// same chunk blocks: the logits are taken to be finite, so the maxima need no
// quieting of their operands.
#include "entropy_ops.hpp"

namespace wedlm {

template <typename T, bool VEC>
__global__ void __launch_bounds__(kEntThreads)
k_entropy_partial(const T* __restrict__ logits, int V, int chunk_elems, int n_chunks,
                  EntPartial* __restrict__ part) {
  __shared__ EntPartial red[kEntThreads / kWave];
  entropy_chunk_block<T, VEC>(logits, V, chunk_elems, n_chunks, part, blockIdx.x, blockIdx.y,
                              red);
}

}  // namespace wedlm

using namespace wedlm;

void wedlm::launch_entropy_partials(int dtype, int B, int W, int V, const void* logits,
                                    const EntPlan& pl, EntPartial* part, hipStream_t s) {
  const dim3 grid(pl.n_chunks, B * W);
  if (dtype == WEDLM_BF16) {
    const uint16_t* z = static_cast<const uint16_t*>(logits);
    if (pl.vec)
      hipLaunchKernelGGL((k_entropy_partial<uint16_t, true>), grid, dim3(kEntThreads), 0, s, z, V,
                         pl.chunk_elems, pl.n_chunks, part);
    else
      hipLaunchKernelGGL((k_entropy_partial<uint16_t, false>), grid, dim3(kEntThreads), 0, s, z, V,
                         pl.chunk_elems, pl.n_chunks, part);
  } else {
    const float* z = static_cast<const float*>(logits);
    if (pl.vec)
      hipLaunchKernelGGL((k_entropy_partial<float, true>), grid, dim3(kEntThreads), 0, s, z, V,
                         pl.chunk_elems, pl.n_chunks, part);
    else
      hipLaunchKernelGGL((k_entropy_partial<float, false>), grid, dim3(kEntThreads), 0, s, z, V,
                         pl.chunk_elems, pl.n_chunks, part);
  }
}

