// Rows half of the commit (a5): the c committed window rows of a sequence
// written into its cache pages at positions L .. L+c-1, shared by the commit
// kernel and the fp32 attention launch that appends them.
//
// hyper.ai summary of WeDLM, "Method": the leftmost contiguous filled prefix
// of the window is committed to the cache right away. The cache is paged
// (PagedAttention, mlsanity.com page, "Builds on").
#pragma once

#include "window_ops.hpp"

namespace wedlm {

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
// One call moves the rows of one (sequence b, kv head kvh, layer) with the
// nthreads threads of a block (tid: this thread's index); omega holds the D/2
// rotation frequencies.
template <typename T, bool kRope>
__device__ __forceinline__ void commit_rows_block(
    int B, int W, int Hkv, int D, int P, int num_pages, int max_pages,
    const int32_t* __restrict__ run_len, const int32_t* __restrict__ prefix_len,
    const T* __restrict__ k_phys, const T* __restrict__ v_phys,
    const int32_t* __restrict__ block_table, T* __restrict__ k_cache, T* __restrict__ v_cache,
    long long cache_layer_stride, const double* omega, const int32_t* __restrict__ rot_pos, int b,
    int kvh, int layer, int tid, int nthreads) {
  constexpr int X = 16 / sizeof(T);         // elements per 16-byte K slice
  constexpr int kLineElems = 64 / sizeof(T);
  constexpr int kDimsPerLine = kLineElems / 16;  // value dimensions per line (P = 16)
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
  for (int task = tid; task < ktasks; task += nthreads) {
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
            rope_cos_sin(tr, omega[j0 + x], c, sn);
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
  for (int task = tid; task < vtasks; task += nthreads) {
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

}  // namespace wedlm
