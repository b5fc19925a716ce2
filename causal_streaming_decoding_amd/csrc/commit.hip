// Commit of the leftmost filled run into the paged cache, and window refill.
//
// hyper.ai summary of WeDLM, "Method": the leftmost contiguous filled prefix of
// the window is committed to the cache right away - under the causal mask its
// KV depends only on earlier tokens - and new masks are appended so the window
// stays W wide. The cache is paged (PagedAttention, mlsanity.com page,
// "Builds on").
//
// Two kernels on the caller's stream:
//   k_commit_rows  grid (sequence x kv head, layer): copies the c committed rows of
//                  k_phys / v_phys (physical rows 0..c-1 are slots 0..c-1) into
//                  the pages at positions L..L+c-1 (commit_rows_block,
//                  commit_ops.hpp; the fp32 attention launch runs the same
//                  function in blocks of its own to append its rows).
//   k_commit_state one wavefront per sequence: cache slots, window shift with
//                  the new fills, mask refill, prefix_len += c. It runs after
//                  the copies (same stream), which read the old prefix_len.
#include "commit_ops.hpp"

#include <cmath>
#include <type_traits>

namespace wedlm {

constexpr int kCommitThreads = 256;

template <typename T, bool kRope>
__global__ void __launch_bounds__(kCommitThreads)
k_commit_rows(int B, int W, int Hkv, int D, int P, int num_pages, int max_pages,
              const int32_t* __restrict__ run_len, const int32_t* __restrict__ prefix_len,
              const T* __restrict__ k_phys, const T* __restrict__ v_phys,
              const int32_t* __restrict__ block_table, T* __restrict__ k_cache,
              T* __restrict__ v_cache, long long cache_layer_stride, CommitRope rope,
              const int32_t* __restrict__ rot_pos) {
  commit_rows_block<T, kRope>(B, W, Hkv, D, P, num_pages, max_pages, run_len, prefix_len, k_phys,
                              v_phys, block_table, k_cache, v_cache, cache_layer_stride,
                              rope.omega, rot_pos, blockIdx.x / Hkv, blockIdx.x % Hkv, blockIdx.y,
                              threadIdx.x, kCommitThreads);
}

__global__ void __launch_bounds__(kWave)
k_commit_state(int W, int P, int num_pages, int max_pages, const int32_t* __restrict__ run_len,
               const uint8_t* __restrict__ selected, const int32_t* __restrict__ argmax_tok,
               const int32_t* __restrict__ block_table, int32_t* __restrict__ tokens,
               uint8_t* __restrict__ filled, int32_t* __restrict__ prefix_len,
               int32_t* __restrict__ commit_len, int32_t* __restrict__ cache_slot,
               int32_t mask_id) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  bool f = false, sel = false;
  int tok = mask_id, am = 0;
  if (i < W) {
    const int row = b * W + i;
    f = filled[row] != 0;
    tok = tokens[row];
    sel = selected[row] != 0;
    am = argmax_tok[row];
  }
  bool f_new;
  wave_commit_state(b, W, i, P, num_pages, max_pages, run_len[b], f, tok, sel, am, block_table,
                    tokens, filled, prefix_len, commit_len, cache_slot, mask_id, f_new);
}

}  // namespace wedlm

using namespace wedlm;

static int launch_commit(bool rope, int dtype, int n_layers, int B, int W, int Hkv, int D,
                         int page_size, int num_pages, int max_pages, double theta,
                         const int32_t* run_len, const uint8_t* selected,
                         const int32_t* argmax_tok, const void* k_rows, const void* v_rows,
                         const int32_t* block_table, void* k_cache, void* v_cache, int32_t* tokens,
                         uint8_t* filled, int32_t* prefix_len, int32_t* commit_len,
                         int32_t* cache_slot, int32_t mask_id, void* stream) {
  if (!valid_dtype(dtype)) return WEDLM_ERR_UNSUPPORTED;
  if (n_layers <= 0 || B <= 0 || W <= 0 || W > WEDLM_MAX_WINDOW || Hkv <= 0 || D <= 0 ||
      page_size <= 0 || num_pages <= 0 || max_pages <= 0)
    return WEDLM_ERR_INVALID;
  if (rope && !(theta > 0.0)) return WEDLM_ERR_INVALID;
  const int X = 16 / static_cast<int>(elt_size(dtype));
  if (D % X != 0 || page_size != 16) return WEDLM_ERR_UNSUPPORTED;
  if (rope && (D % (2 * X) != 0 || D > kCommitMaxD)) return WEDLM_ERR_UNSUPPORTED;
  // fused form: k and v both NULL means the rows were appended already (by
  // wedlm_window_attn_rope with commit_run); only the window state is updated
  const bool rows = !(rope && k_rows == nullptr && v_rows == nullptr);
  if (!run_len || !selected || !argmax_tok || (rows && (!k_rows || !v_rows)) || !block_table ||
      !k_cache || !v_cache || !tokens || !filled || !prefix_len || !commit_len || !cache_slot)
    return WEDLM_ERR_INVALID;
  if (n_layers > 65535) return WEDLM_ERR_UNSUPPORTED;
  if (1LL * B * Hkv > 0x7fffffffLL) return WEDLM_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  const long long stride = 1LL * num_pages * Hkv * D * page_size;
  CommitRope tab{};
  if (rope)
    for (int j = 0; j < D / 2; ++j) tab.omega[j] = std::pow(theta, -2.0 * j / D);
  const dim3 grid(B * Hkv, n_layers);
  auto go = [&](auto kernel, auto* tag) {
    using T = std::remove_pointer_t<decltype(tag)>;
    hipLaunchKernelGGL(kernel, grid, dim3(kCommitThreads), 0, s, B, W, Hkv, D, page_size,
                       num_pages, max_pages, run_len, prefix_len, static_cast<const T*>(k_rows),
                       static_cast<const T*>(v_rows), block_table, static_cast<T*>(k_cache),
                       static_cast<T*>(v_cache), stride, tab, nullptr);
  };
  if (rows) {
    if (dtype == WEDLM_BF16) {
      uint16_t* tag = nullptr;
      rope ? go(k_commit_rows<uint16_t, true>, tag) : go(k_commit_rows<uint16_t, false>, tag);
    } else {
      float* tag = nullptr;
      rope ? go(k_commit_rows<float, true>, tag) : go(k_commit_rows<float, false>, tag);
    }
    const int st = launch_status();
    if (st != WEDLM_OK) return st;
  }
  hipLaunchKernelGGL(k_commit_state, dim3(B), dim3(kWave), 0, s, W, page_size, num_pages,
                     max_pages, run_len, selected, argmax_tok, block_table, tokens, filled,
                     prefix_len, commit_len, cache_slot, mask_id);
  return launch_status();
}

extern "C" int wedlm_commit_prefix(int dtype, int n_layers, int B, int W, int Hkv, int D,
                                   int page_size, int num_pages, int max_pages,
                                   const int32_t* run_len, const uint8_t* selected,
                                   const int32_t* argmax_tok, const void* k_phys,
                                   const void* v_phys, const int32_t* block_table, void* k_cache,
                                   void* v_cache, int32_t* tokens, uint8_t* filled,
                                   int32_t* prefix_len, int32_t* commit_len, int32_t* cache_slot,
                                   int32_t mask_id, void* stream) {
  return launch_commit(false, dtype, n_layers, B, W, Hkv, D, page_size, num_pages, max_pages, 0.0,
                       run_len, selected, argmax_tok, k_phys, v_phys, block_table, k_cache,
                       v_cache, tokens, filled, prefix_len, commit_len, cache_slot, mask_id,
                       stream);
}

extern "C" int wedlm_commit_prefix_rope(int dtype, int n_layers, int B, int W, int Hkv, int D,
                                        int page_size, int num_pages, int max_pages, double theta,
                                        const int32_t* run_len, const uint8_t* selected,
                                        const int32_t* argmax_tok, const void* k, const void* v,
                                        const int32_t* block_table, void* k_cache, void* v_cache,
                                        int32_t* tokens, uint8_t* filled, int32_t* prefix_len,
                                        int32_t* commit_len, int32_t* cache_slot,
                                        int32_t mask_id, void* stream) {
  return launch_commit(true, dtype, n_layers, B, W, Hkv, D, page_size, num_pages, max_pages,
                       theta, run_len, selected, argmax_tok, k, v, block_table, k_cache, v_cache,
                       tokens, filled, prefix_len, commit_len, cache_slot, mask_id, stream);
}
