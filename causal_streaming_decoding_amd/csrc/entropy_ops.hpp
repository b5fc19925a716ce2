// Chunk pass of the full-vocabulary entropy (one block per chunk of a logit
// row), shared by the entropy kernels and by the attention kernel, whose
// launch can carry the chunk blocks of the same step after its own
// workgroups.
//
// Entropy of softmax(z) in one streaming pass, in base-2 units: with
// u = (z - m) log2(e), s = sum 2^u and t = sum u 2^u, H = ln2 (log2 s - t / s).
// Each thread keeps (m, s, t) for its strided 16-byte vectors; when a pass
// raises the running max the sums are rescaled by 2^(m_old - m_new) (exact
// identity: t' = (t + d s) 2^d with d = (m_old - m_new) log2 e). For the
// argmax each thread keeps only the first index of the lowest vector holding
// its max; the block's reduction keeps the lowest such vector among the holders
// of the block's max (vectors do not overlap, so it holds the lowest index of
// the max), and one thread finds the max inside that one 16-byte vector.
#pragma once

#include "common.hpp"

namespace wedlm {

constexpr int kEntThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct EVec {
  static constexpr int N = 16 / sizeof(T);
  union {
    u32x4 raw;
    T e[N];
  };
};

// Vectors (16 bytes, or single elements when !VEC) per thread per block: all
// of a thread's loads are issued before any is reduced.
constexpr int kEntIter = 8;

// One pass of a thread over kEntIter vectors of N elements starting at
// element base (+ the thread's offset), folded into its running (m, s, t) and
// best (first index of the lowest vector holding m). GUARD: vectors at or past
// end are skipped (the chunk's last, partial pass); without it every vector is
// in range and no lane masking is emitted. All of the pass's loads are issued
// before any is reduced; then the vector maxima, the pass maximum and the
// lowest vector holding it, one rescale of the running sums, and the sums of
// every element against that one reference.
template <typename T, int N, bool GUARD>
__device__ __forceinline__ void entropy_pass(const T* __restrict__ z, int base, int end,
                                             float& m, float& s, float& t, int& best) {
  EVec<T> vv[kEntIter];
  // byte offsets from the row's (uniform) start: one 32-bit add per load
  const char* zb = reinterpret_cast<const char*>(z);
  const uint32_t off0 = static_cast<uint32_t>(base + threadIdx.x * N) * sizeof(T);
#pragma unroll
  for (int it = 0; it < kEntIter; ++it) {
    const int i0 = base + (it * kEntThreads + threadIdx.x) * N;
    if constexpr (N > 1) {
      const u32x4* src = reinterpret_cast<const u32x4*>(
          zb + (off0 + static_cast<uint32_t>(it * kEntThreads * N * sizeof(T))));
      if (GUARD)
        vv[it].raw = i0 < end ? *src : u32x4{0u, 0u, 0u, 0u};
      else
        vv[it].raw = *src;
    } else {
      vv[it].raw = u32x4{0u, 0u, 0u, 0u};
      if (!GUARD || i0 < end) vv[it].e[0] = z[i0];
    }
  }
  float mv[kEntIter];
#pragma unroll
  for (int it = 0; it < kEntIter; ++it) {
    float mz = Elt<T>::load(&vv[it].e[0]);
#pragma unroll
    for (int e = 1; e < N; ++e) mz = fmaxf(mz, Elt<T>::load(&vv[it].e[e]));
    // a skipped vector can neither raise the maximum nor be chosen for it
    if (GUARD && base + (it * kEntThreads + threadIdx.x) * N >= end) mz = -INFINITY;
    mv[it] = mz;
  }
  float mpass = mv[0];
#pragma unroll
  for (int it = 1; it < kEntIter; ++it) mpass = fmaxf(mpass, mv[it]);
  if (mpass > m) {
    // the lowest vector holding the pass maximum (one of them holds it exactly)
    int bi = kEntIter - 1;
#pragma unroll
    for (int it = kEntIter - 2; it >= 0; --it) bi = mv[it] == mpass ? it : bi;
    best = base + (bi * kEntThreads + threadIdx.x) * N;
    // rescale the running sums to the new reference
    const float d = (m - mpass) * kLog2eF;
    const float f = __builtin_amdgcn_exp2f(d);
    t = (t + d * s) * f;
    s = s * f;
    m = mpass;
  }
  const float mb = m * kLog2eF;
#pragma unroll
  for (int it = 0; it < kEntIter; ++it) {
    if (GUARD && base + (it * kEntThreads + threadIdx.x) * N >= end) continue;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      const float u = fmaf(Elt<T>::load(&vv[it].e[e]), kLog2eF, -mb);
      const float p = __builtin_amdgcn_exp2f(u);
      s += p;
      t = fmaf(p, u, t);
    }
  }
}

// Chunk `chunk` of logit row `row` reduced to (m, s, t, argmax) by a block of
// kEntThreads threads, written to part[row * n_chunks + chunk]; red is the
// block's LDS scratch. VEC: rows are 16-byte aligned and V is a multiple of
// the vector width.
template <typename T, bool VEC>
__device__ __forceinline__ void entropy_chunk_block(const T* __restrict__ logits, int V,
                                                    int chunk_elems, int n_chunks,
                                                    EntPartial* __restrict__ part, int chunk,
                                                    int row, EntPartial* red) {
  constexpr int N = VEC ? EVec<T>::N : 1;
  constexpr int kPassElems = kEntThreads * kEntIter * N;
  const int begin = chunk * chunk_elems;
  const int end = min(V, begin + chunk_elems);
  const T* z = logits + static_cast<size_t>(row) * V;
  float m = kNegBig, s = 0.f, t = 0.f;
  int best = -1;
  // one pass when VEC (a chunk is exactly kEntIter vectors per thread),
  // 16 / sizeof(T) passes of single elements otherwise; the test is uniform
  for (int base = begin; base < end; base += kPassElems) {
    if (end - base >= kPassElems)
      entropy_pass<T, N, false>(z, base, end, m, s, t, best);
    else
      entropy_pass<T, N, true>(z, base, end, m, s, t, best);
  }
  // idx: first index of the thread's vector, refined to the element below
  EntPartial acc{m, s, t, best >= 0 ? best : 0x7fffffff};
  // wavefront then block reduction
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    EntPartial o;
    o.m = __shfl_xor(acc.m, off, kWave);
    o.s = __shfl_xor(acc.s, off, kWave);
    o.t = __shfl_xor(acc.t, off, kWave);
    o.idx = __shfl_xor(acc.idx, off, kWave);
    merge(acc, o);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    EntPartial r = red[0];
    for (int w = 1; w < kEntThreads / kWave; ++w) merge(r, red[w]);
    if (N > 1 && r.idx != 0x7fffffff) {
      // the lowest element of that vector equal to the max (it holds one)
      EVec<T> bv;
      bv.raw = *reinterpret_cast<const u32x4*>(z + r.idx);
      int e0 = N - 1;
#pragma unroll
      for (int e = N - 2; e >= 0; --e)
        if (Elt<T>::load(&bv.e[e]) == r.m) e0 = e;
      r.idx += e0;
    }
    part[static_cast<size_t>(row) * n_chunks + chunk] = r;
  }
}

// Chunking of the rows: kEntIter 16-byte vectors per thread (the same element
// count on the single-element path, so the workspace does not depend on
// alignment).
struct EntPlan {
  int chunk_elems, n_chunks;
  bool vec;
};

inline EntPlan plan_entropy(int dtype, int B, int W, int V) {
  EntPlan pl{};
  const int N = 16 / static_cast<int>(elt_size(dtype));
  pl.vec = (V % N) == 0;
  // a chunk is kEntIter 16-byte vectors per thread (the same element count on
  // the single-element path, so the workspace does not depend on alignment)
  pl.chunk_elems = kEntThreads * kEntIter * N;
  pl.n_chunks = ceil_div(V, pl.chunk_elems);
  (void)B;
  (void)W;
  return pl;
}

// Host side (entropy.hip): the chunk pass as a launch of its own (grid
// n_chunks x B*W of k_entropy_partial) over pl's chunking, enqueued on s.
void launch_entropy_partials(int dtype, int B, int W, int V, const void* logits,
                             const EntPlan& pl, EntPartial* part, hipStream_t s);

}  // namespace wedlm
