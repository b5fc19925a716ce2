// Commit of the leftmost filled run into the paged cache, and window refill.
//
// hyper.ai summary of WeDLM, "Method": the leftmost contiguous filled prefix of
// the window is committed to the cache right away - under the causal mask its
// KV depends only on earlier tokens - and new masks are appended so the window
// stays W wide. The cache is paged (PagedAttention, mlsanity.com page,
// "Builds on").
//
// Two kernels on the caller's stream:
//   k_commit_rows  grid (sequence, layer): copies the c committed rows of
//                  k_phys / v_phys (physical rows 0..c-1 are slots 0..c-1) into
//                  the pages at positions L..L+c-1.
//   k_commit_state one wavefront per sequence: cache slots, window shift with
//                  the new fills, mask refill, prefix_len += c. It runs after
//                  the copies (same stream), which read the old prefix_len.
#include "common.hpp"

namespace wedlm {

constexpr int kCommitThreads = 256;

__device__ __forceinline__ int commit_length(int run, int L, int W, int max_pages, int P) {
  int c = min(max(run, 0), W);
  const int room = max(max_pages * P - L, 0);
  return min(c, room);
}

template <typename T>
__global__ void __launch_bounds__(kCommitThreads)
k_commit_rows(int B, int W, int Hkv, int D, int P, int num_pages, int max_pages,
              const int32_t* __restrict__ run_len, const int32_t* __restrict__ prefix_len,
              const T* __restrict__ k_phys, const T* __restrict__ v_phys,
              const int32_t* __restrict__ block_table, T* __restrict__ k_cache,
              T* __restrict__ v_cache, long long cache_layer_stride) {
  constexpr int X = 16 / sizeof(T);  // elements per 16-byte key slice
  const int b = blockIdx.x;
  const int layer = blockIdx.y;
  const int L = max(prefix_len[b], 0);
  const int c = commit_length(run_len[b], L, W, max_pages, P);
  if (c == 0) return;
  const int32_t* bt = block_table + static_cast<size_t>(b) * max_pages;
  const size_t lb = static_cast<size_t>(layer) * B + b;
  T* kcl = k_cache + static_cast<size_t>(layer) * cache_layer_stride;
  T* vcl = v_cache + static_cast<size_t>(layer) * cache_layer_stride;
  const int slices = D / X;
  // keys: one 16-byte slice per task
  const int ktasks = c * Hkv * slices;
  for (int task = threadIdx.x; task < ktasks; task += kCommitThreads) {
    const int sl = task % slices;
    const int kvh = (task / slices) % Hkv;
    const int j = task / (slices * Hkv);
    const int t = L + j;
    const int pid = min(max(bt[t / P], 0), num_pages - 1);
    const T* src = k_phys + ((lb * W + j) * Hkv + kvh) * D + sl * X;
    T* dst = kcl + ((static_cast<size_t>(pid) * Hkv + kvh) * slices + sl) * P * X + (t % P) * X;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
  // values: the page stores each dimension's P positions contiguously
  const int vtasks = c * Hkv * D;
  for (int task = threadIdx.x; task < vtasks; task += kCommitThreads) {
    const int d = task % D;
    const int kvh = (task / D) % Hkv;
    const int j = task / (D * Hkv);
    const int t = L + j;
    const int pid = min(max(bt[t / P], 0), num_pages - 1);
    vcl[((static_cast<size_t>(pid) * Hkv + kvh) * D + d) * P + (t % P)] =
        v_phys[((lb * W + j) * Hkv + kvh) * D + d];
  }
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
  const bool in_window = i < W;
  const int L = max(prefix_len[b], 0);
  const int c = commit_length(run_len[b], L, W, max_pages, P);
  int f = 0, tok = mask_id;
  if (in_window) {
    const int row = b * W + i;
    const bool sel = selected[row] != 0;
    f = (filled[row] != 0 || sel) ? 1 : 0;
    tok = sel ? argmax_tok[row] : tokens[row];
  }
  // every lane has read its slot; shift left by c within the wavefront
  const int src = i + c;
  const int f_in = __shfl(f, src < kWave ? src : 0, kWave);
  const int t_in = __shfl(tok, src < kWave ? src : 0, kWave);
  if (in_window) {
    const int row = b * W + i;
    const bool keep = src < W;
    filled[row] = keep ? static_cast<uint8_t>(f_in) : static_cast<uint8_t>(0);
    tokens[row] = keep ? t_in : mask_id;
    int slot = -1;
    if (i < c) {
      const int t = L + i;
      const int pid = min(max(block_table[static_cast<size_t>(b) * max_pages + t / P], 0),
                          num_pages - 1);
      slot = pid * P + t % P;
    }
    cache_slot[row] = slot;
  }
  if (i == 0) {
    commit_len[b] = c;
    prefix_len[b] = L + c;
  }
}

}  // namespace wedlm

using namespace wedlm;

extern "C" int wedlm_commit_prefix(int dtype, int n_layers, int B, int W, int Hkv, int D,
                                   int page_size, int num_pages, int max_pages,
                                   const int32_t* run_len, const uint8_t* selected,
                                   const int32_t* argmax_tok, const void* k_phys,
                                   const void* v_phys, const int32_t* block_table, void* k_cache,
                                   void* v_cache, int32_t* tokens, uint8_t* filled,
                                   int32_t* prefix_len, int32_t* commit_len, int32_t* cache_slot,
                                   int32_t mask_id, void* stream) {
  if (!valid_dtype(dtype)) return WEDLM_ERR_UNSUPPORTED;
  if (n_layers <= 0 || B <= 0 || W <= 0 || W > WEDLM_MAX_WINDOW || Hkv <= 0 || D <= 0 ||
      page_size <= 0 || num_pages <= 0 || max_pages <= 0)
    return WEDLM_ERR_INVALID;
  const int X = 16 / static_cast<int>(elt_size(dtype));
  if (D % X != 0) return WEDLM_ERR_UNSUPPORTED;
  if (!run_len || !selected || !argmax_tok || !k_phys || !v_phys || !block_table || !k_cache ||
      !v_cache || !tokens || !filled || !prefix_len || !commit_len || !cache_slot)
    return WEDLM_ERR_INVALID;
  if (n_layers > 65535) return WEDLM_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  const long long stride = 1LL * num_pages * Hkv * D * page_size;
  const dim3 grid(B, n_layers);
  if (dtype == WEDLM_BF16)
    hipLaunchKernelGGL(k_commit_rows<uint16_t>, grid, dim3(kCommitThreads), 0, s, B, W, Hkv, D,
                       page_size, num_pages, max_pages, run_len, prefix_len,
                       static_cast<const uint16_t*>(k_phys), static_cast<const uint16_t*>(v_phys),
                       block_table, static_cast<uint16_t*>(k_cache),
                       static_cast<uint16_t*>(v_cache), stride);
  else
    hipLaunchKernelGGL(k_commit_rows<float>, grid, dim3(kCommitThreads), 0, s, B, W, Hkv, D,
                       page_size, num_pages, max_pages, run_len, prefix_len,
                       static_cast<const float*>(k_phys), static_cast<const float*>(v_phys),
                       block_table, static_cast<float*>(k_cache), static_cast<float*>(v_cache),
                       stride);
  int st = launch_status();
  if (st != WEDLM_OK) return st;
  hipLaunchKernelGGL(k_commit_state, dim3(B), dim3(kWave), 0, s, W, page_size, num_pages,
                     max_pages, run_len, selected, argmax_tok, block_table, tokens, filled,
                     prefix_len, commit_len, cache_slot, mask_id);
  return launch_status();
}
