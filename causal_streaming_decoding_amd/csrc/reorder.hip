// Topological reorder of the sliding window: one 64-lane wavefront per sequence.
//
// hyper.ai summary of WeDLM, "Method": filled (observed) tokens are placed
// physically before the mask tokens and every token keeps its logical
// position; the streaming decoder does this to its W-slot window each step.
//
// Lane i owns slot i. A ballot over the filled flags gives the whole window as
// one 64-bit mask; a slot's physical index is then a popcount of the flags
// below it (filled slots) or n_obs plus the popcount of the masks below it
// (mask slots), which is the stable partition. The leading filled run, used by
// the commit, is the count of trailing ones of the ballot. Under the block
// rule (the stop-and-wait baseline that the same summary contrasts with
// streaming: a block is cached only once finalised) the run counts only when
// it covers the whole window, and is 0 otherwise.
#include "window_ops.hpp"

namespace wedlm {

constexpr int kReorderWaves = 4;

__global__ void __launch_bounds__(kWave * kReorderWaves)
k_window_reorder(int B, int W, int block_rule, const uint8_t* __restrict__ filled,
                 const int32_t* __restrict__ prefix_len, int32_t* __restrict__ perm,
                 int32_t* __restrict__ inv_perm, int32_t* __restrict__ pos,
                 int32_t* __restrict__ n_obs, int32_t* __restrict__ run_len) {
  const int lane = threadIdx.x & (kWave - 1);
  const int b = blockIdx.x * kReorderWaves + (threadIdx.x >> 6);
  if (b >= B) return;  // uniform per wavefront
  const bool f = lane < W && filled[b * W + lane] != 0;
  wave_reorder(b, W, lane, f, max(prefix_len[b], 0), block_rule, perm, inv_perm, pos, n_obs,
               run_len);
}

}  // namespace wedlm

static int launch_reorder(int B, int W, int block_rule, const uint8_t* filled,
                          const int32_t* prefix_len, int32_t* perm, int32_t* inv_perm, int32_t* pos,
                          int32_t* n_obs, int32_t* run_len, void* stream) {
  using namespace wedlm;
  if (B <= 0 || W <= 0 || W > WEDLM_MAX_WINDOW) return WEDLM_ERR_INVALID;
  if (!filled || !prefix_len || !perm || !inv_perm || !pos || !n_obs || !run_len)
    return WEDLM_ERR_INVALID;
  const int blocks = ceil_div(B, kReorderWaves);
  hipLaunchKernelGGL(k_window_reorder, dim3(blocks), dim3(kWave * kReorderWaves), 0,
                     as_stream(stream), B, W, block_rule, filled, prefix_len, perm, inv_perm, pos,
                     n_obs, run_len);
  return launch_status();
}

extern "C" int wedlm_window_reorder(int B, int W, const uint8_t* filled, const int32_t* prefix_len,
                                    int32_t* perm, int32_t* inv_perm, int32_t* pos, int32_t* n_obs,
                                    int32_t* run_len, void* stream) {
  return launch_reorder(B, W, 0, filled, prefix_len, perm, inv_perm, pos, n_obs, run_len, stream);
}

extern "C" int wedlm_window_reorder_rule(int B, int W, int commit_rule, const uint8_t* filled,
                                         const int32_t* prefix_len, int32_t* perm,
                                         int32_t* inv_perm, int32_t* pos, int32_t* n_obs,
                                         int32_t* run_len, void* stream) {
  if (commit_rule != WEDLM_COMMIT_STREAM && commit_rule != WEDLM_COMMIT_BLOCK)
    return WEDLM_ERR_INVALID;
  return launch_reorder(B, W, commit_rule == WEDLM_COMMIT_BLOCK ? 1 : 0, filled, prefix_len, perm,
                        inv_perm, pos, n_obs, run_len, stream);
}
