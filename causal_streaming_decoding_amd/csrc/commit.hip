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
//                  the pages at positions L..L+c-1.
//   k_commit_state one wavefront per sequence: cache slots, window shift with
//                  the new fills, mask refill, prefix_len += c. It runs after
//                  the copies (same stream), which read the old prefix_len.
#include "window_ops.hpp"

#include <cmath>
#include <type_traits>

namespace wedlm {

constexpr int kCommitThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Committed rows are written as whole 64-byte lines: a line holds 4 keys of
// one 16-byte K slice, or 16 keys of 64 / (16 * sizeof(T)) value dimensions.
// Each line touched by the commit is read, the committed keys are merged in
// registers (static indices, so nothing goes to scratch) and the line is
// stored back in full - partial-line stores would make the memory system
// read-modify-write every 2- or 16-byte piece. One thread owns one line; one
// block covers one (sequence, kv head, layer), so a commit of c <= 16 rows
// touches at most 5 x D/8 key lines and 2 x D/2 value lines per block: one
// round of 256 threads for D = 128.
constexpr int kCommitMaxD = 256;

// RoPE frequencies theta^(-2j/D) for the fused variant (host-computed).
struct CommitRope {
  double omega[kCommitMaxD / 2];
};

// kRope: k_phys / v_phys are the window rows in slot order before RoPE (the
// committed rows 0..c-1 are slots 0..c-1 either way); each committed key is
// rotated as it is written, at rot_pos[b][j] when rot_pos is given (the
// positions an attention call rotated the same rows at), else at its logical
// position L + j. The two agree when rot_pos comes from the window reorder.
template <typename T, bool kRope>
__global__ void __launch_bounds__(kCommitThreads)
k_commit_rows(int B, int W, int Hkv, int D, int P, int num_pages, int max_pages,
              const int32_t* __restrict__ run_len, const int32_t* __restrict__ prefix_len,
              const T* __restrict__ k_phys, const T* __restrict__ v_phys,
              const int32_t* __restrict__ block_table, T* __restrict__ k_cache,
              T* __restrict__ v_cache, long long cache_layer_stride, CommitRope rope,
              const int32_t* __restrict__ rot_pos) {
  constexpr int X = 16 / sizeof(T);         // elements per 16-byte K slice
  constexpr int kLineElems = 64 / sizeof(T);
  constexpr int kDimsPerLine = kLineElems / 16;  // value dimensions per line (P = 16)
  const int b = blockIdx.x / Hkv;
  const int kvh = blockIdx.x % Hkv;
  const int layer = blockIdx.y;
  const int L = max(prefix_len[b], 0);
  const int c = commit_length(run_len[b], L, W, max_pages, P);
  if (c == 0) return;
  const int32_t* bt = block_table + static_cast<size_t>(b) * max_pages;
  const size_t lb = static_cast<size_t>(layer) * B + b;
  T* kcl = k_cache + static_cast<size_t>(layer) * cache_layer_stride;
  T* vcl = v_cache + static_cast<size_t>(layer) * cache_layer_stride;
  const int slices = D / X;
  const int end = L + c;  // committed positions are L .. end-1

  // keys: lines of 4 positions within one slice of one page
  const int line0 = L / 4, nlines = (end - 1) / 4 - line0 + 1;
  const int ktasks = nlines * slices;
  for (int task = threadIdx.x; task < ktasks; task += kCommitThreads) {
    const int sl = task % slices;
    const int t0 = (line0 + task / slices) * 4;
    const int pid = min(max(bt[t0 / P], 0), num_pages - 1);
    u32x4* dst = reinterpret_cast<u32x4*>(
        kcl + ((static_cast<size_t>(pid) * Hkv + kvh) * slices + sl) * P * X + (t0 % P) * X);
    u32x4 line[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) line[e] = dst[e];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = t0 + e;
      if (t >= L && t < end) {
        const T* krow = k_phys + ((lb * W + (t - L)) * Hkv + kvh) * D;
        line[e] = *reinterpret_cast<const u32x4*>(krow + sl * X);
        if constexpr (kRope) {
          // rotate-half: slice sl pairs with sl +- slices/2
          const int hs = slices / 2;
          const bool lower = sl < hs;
          const int j0 = (lower ? sl : sl - hs) * X;  // first frequency index
          union {
            u32x4 v;
            T e[X];
          } own, mate, out;
          own.v = line[e];
          mate.v = *reinterpret_cast<const u32x4*>(krow + (lower ? sl + hs : sl - hs) * X);
          const double tr = rot_pos ? static_cast<double>(rot_pos[b * W + (t - L)])
                                    : static_cast<double>(t);
#pragma unroll
          for (int x = 0; x < X; ++x) {
            float c, sn;
            rope_cos_sin(tr, rope.omega[j0 + x], c, sn);
            const float a = Elt<T>::load(&own.e[x]), m = Elt<T>::load(&mate.e[x]);
            // lower half: a cos - mate sin; upper half: a cos + mate sin
            Elt<T>::store(&out.e[x], lower ? a * c - m * sn : a * c + m * sn);
          }
          line[e] = out.v;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = line[e];
  }

  // values: lines of kDimsPerLine dimensions x 16 positions of one page
  const int pg0 = L / P, npg = (end - 1) / P - pg0 + 1;
  const int groups = D / kDimsPerLine;
  const int vtasks = npg * groups;
  for (int task = threadIdx.x; task < vtasks; task += kCommitThreads) {
    const int dg = task % groups;
    const int pg = pg0 + task / groups;
    const int pid = min(max(bt[pg], 0), num_pages - 1);
    T* dst = vcl + ((static_cast<size_t>(pid) * Hkv + kvh) * D + dg * kDimsPerLine) * P;
    union {
      u32x4 v[4];
      T e[kLineElems];
    } line;
#pragma unroll
    for (int i = 0; i < 4; ++i) line.v[i] = reinterpret_cast<const u32x4*>(dst)[i];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = pg * P + e;
      if (t >= L && t < end) {
        const T* src = v_phys + ((lb * W + (t - L)) * Hkv + kvh) * D + dg * kDimsPerLine;
#pragma unroll
        for (int dd = 0; dd < kDimsPerLine; ++dd) line.e[dd * 16 + e] = src[dd];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) reinterpret_cast<u32x4*>(dst)[i] = line.v[i];
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

// Rows part of the fused commit (used by the f32 attention path, which has no
// rows of its own to append): rotated keys and values of rows 0..c-1, the keys
// rotated at rot_pos[b][j] (the attention's positions).
int wedlm::commit_rows_rope(int dtype, int n_layers, int B, int W, int Hkv, int D, int page_size,
                            int num_pages, int max_pages, double theta, const int32_t* run_len,
                            const int32_t* prefix_len, const int32_t* rot_pos, const void* k_rows,
                            const void* v_rows, const int32_t* block_table, void* k_cache,
                            void* v_cache, hipStream_t s) {
  const int X = 16 / static_cast<int>(elt_size(dtype));
  if (D % (2 * X) != 0 || D > kCommitMaxD || page_size != 16) return WEDLM_ERR_UNSUPPORTED;
  const long long stride = 1LL * num_pages * Hkv * D * page_size;
  CommitRope tab{};
  for (int j = 0; j < D / 2; ++j) tab.omega[j] = std::pow(theta, -2.0 * j / D);
  const dim3 grid(B * Hkv, n_layers);
  if (dtype == WEDLM_BF16)
    hipLaunchKernelGGL((k_commit_rows<uint16_t, true>), grid, dim3(kCommitThreads), 0, s, B, W,
                       Hkv, D, page_size, num_pages, max_pages, run_len, prefix_len,
                       static_cast<const uint16_t*>(k_rows), static_cast<const uint16_t*>(v_rows),
                       block_table, static_cast<uint16_t*>(k_cache),
                       static_cast<uint16_t*>(v_cache), stride, tab, rot_pos);
  else
    hipLaunchKernelGGL((k_commit_rows<float, true>), grid, dim3(kCommitThreads), 0, s, B, W, Hkv,
                       D, page_size, num_pages, max_pages, run_len, prefix_len,
                       static_cast<const float*>(k_rows), static_cast<const float*>(v_rows),
                       block_table, static_cast<float*>(k_cache), static_cast<float*>(v_cache),
                       stride, tab, rot_pos);
  return launch_status();
}

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
