// Causal GQA window attention over [paged KV prefix ; reordered window].
//
// hyper.ai summary of WeDLM, "Method": one causal forward pass over the
// reordered window, conditioned on the persistent KV cache; sai.science review,
// "Strengths": the causal mask is the plain one. FlashAttention's online softmax
// and PagedAttention's block table (mlsanity.com page, "Builds on") are the
// prior art; this kernel is written for CDNA4 from scratch.
//
// bf16 path (D = 128, page P = 16). One workgroup of 4 wavefronts per (layer,
// sequence, kv head, key-range split, part of 4 row tiles); each wavefront
// owns one 16-row tile of the group's M = W*g query rows (physical row p,
// query head h of the group), and the parts of one group run on one XCD. The
// group's key pages stream through an LDS ring, one page (16 keys, 8 KB of K
// and V) per stage, filled by global->LDS DMA: 4 stages, 4 workgroups per CU.
// The waves take
// two pages per barrier; the barrier both publishes them and frees the two
// stages computed before them, which are refilled at once: all but two stages
// are in flight while the waves compute. Each key byte is read from HBM once
// per workgroup.
//
//   S^T (16 keys x 16 rows)  = K (16 x 128) . Q^T         v_mfma_f32_16x16x32_bf16
//   O^T (16 dims x 16 rows) += V^T (x2) . [P_hi; P_lo]^T  v_mfma_f32_16x16x32_bf16
//
// P is split into a bf16 hi and lo part so that rounding the probabilities
// costs no accuracy: the PV MFMA's 32 K slots take the 16 keys' hi parts and
// then their lo parts, against the page's 16 V rows twice.
//
// Cache page layouts (16-byte vectors, contiguous per wave instruction):
//   K page [Hkv][D/8][P][8]: 16-byte slices of the 16 keys side by side, so a
//     page of one kv head is 4 KB contiguous and a DMA instruction moves 1 KB;
//   V page [Hkv][D][P]: each value dimension's 16 keys contiguous (32 B), so a
//     lane reads 8 consecutive keys of one dimension as one 16-byte vector.
// The score MFMA leaves 4 consecutive keys of one query row in each lane; two
// row-swap permutes regroup them into 8-key runs for the PV product. Row max
// and row sum need two cross-lane steps (the 4 lanes holding one row).
//
// When there are too few groups to fill the GPU, a group's pages are split
// across workgroups; each split writes (max, sum, unnormalised O) and a combine
// kernel merges them. The splits follow the live prefix lengths: each
// (layer, kv head) gets a fixed number of workgroups, and each sequence as
// many of them as its pages need, so a ragged batch's longest sequence is not
// the long pole (find_split). The window's own keys are processed by the last
// split with the causal rule (row p sees window rows 0..p), staged into LDS in
// the same page layout.
#include "attn_combine.hpp"
#include "attn_device.hpp"
#include "attn_tile32.hpp"
#include "commit_ops.hpp"
#include "common.hpp"
#include "entropy_ops.hpp"

#include <cmath>

namespace wedlm {

// LDS ring (one 8 KB page per stage) per workgroup size. A CU holds 4
// workgroups of 4 waves (4 wavefronts per SIMD); the ring keeps 8 pages
// (64 KB) in flight per CU while the waves compute. The launches use 4-wave
// workgroups only; the 8-wave configuration (2 per CU, 7 stages) is kept as a
// measured alternative. Every ring advances two pages per barrier (attend_pages2):
// against one page per barrier with 3 stages at 5 workgroups per CU, this
// took the 36-layer streaming launch from 5.49 to 5.64 TB/s and the
// dual-stream forward with 16-key blocks from 2.31 to 2.16 ms (5 workgroups
// per CU with 4 stages, the RoPE frequencies kept in a free stage, and 3 per
// CU with 6 stages both measured slower on those shapes).
template <int NW>
struct Ring {
  static_assert(NW == 4 || NW == 8, "4- or 8-wave workgroups");
  static constexpr int kWavesPerSimd = 4;
  static constexpr int kWgPerCu = NW == 4 ? 4 : 2;
  static constexpr int kStages = NW == 4 ? 4 : 7;
  static constexpr bool kPair = true;
  static constexpr int kAhead = kStages - (kPair ? 2 : 1);  // pages in flight during compute
};

struct AttnArgs {
  // physical order and rotated; with RoPE fused: slot order, before RoPE
  const uint16_t* q;   // [nl][B][W][Hq][D]
  const uint16_t* k;   // [nl][B][W][Hkv][D]
  const uint16_t* v;
  const uint16_t* kc;  // [nl][num_pages][Hkv][D/8][P][8]
  const uint16_t* vc;  // [nl][num_pages][Hkv][D][P]
  const int32_t* block_table;
  const int32_t* prefix_len;
  uint16_t* out;       // [nl][B][W][Hq][D]
  // split partials, one slot per workgroup: slot = (layer*Hkv + kvh)*cols + j
  float* ws_o;         // [n_layers*Hkv*cols][M][D]
  float* ws_ml;        // [n_layers*Hkv*cols][M][2]
  int2* ws_plan;       // [groups]: first slot and number of splits of each group
  int B, W, Hq, Hkv, g, M;
  int num_pages, max_pages, max_prefix_len;
  int cols;            // work units per (layer, kv head): B, or S > B when split
  int parts;           // workgroups per work unit, each taking part_rows of the M rows
  int part_rows;
  long long units;     // n_layers * Hkv * cols
  int split;           // key ranges split across workgroups (partials + combine)
  int min_pages;       // no split takes fewer pages than this (unless it is all there is)
  long long cache_layer_stride;  // elements per layer of one cache
  float scale_log2;
  // RoPE fused into the loads (else unused): physical row -> slot, logical
  // position of each physical row, and the D/2 rotation frequencies
  const int32_t* perm;
  const int32_t* pos;
  double omega[kHeadDim / 2];
  // optional append of the committed rows (RoPE fused path): run length per
  // sequence, and the caches as writable pointers; null when not appending
  const int32_t* commit_run;
  uint16_t* kc_w;
  uint16_t* vc_w;
  // optional entropy chunk pass of the same step, carried by the workgroups
  // past the attention's (wedlm_window_attn_rope_entropy): bf16 logits
  // [rows][V], ent_chunks chunks of ent_chunk_elems per row, partials out
  long long attn_blocks;  // workgroups of the attention itself
  const uint16_t* ent_logits;
  EntPartial* ent_part;
  int ent_V, ent_chunk_elems, ent_chunks, ent_vec;
};



struct RowState {
  f32x4 o[8];  // O^T accumulators per 16-dim tile: lane holds dims 4q..4q+3 of row (lane & 15)
  float m;     // reference max of scaled scores (log2 units)
  float l;     // sum of probabilities against m
};

// Wait states between an MFMA that writes a VGPR and the first VALU or memory
// instruction that reads it (or a VALU that overwrites its SrcC). The compiler
// inserts them inside one basic block, but misses them when the reader sits in
// a successor block reached by a branch (here: the masking branch right after
// the score MFMAs), and a too-early read sees a partial accumulation. Sixteen
// wait states cover every MFMA used here; the tied operands pin the order.
__device__ __forceinline__ void mfma_result_guard(f32x4& x) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(x));
}
__device__ __forceinline__ void mfma_result_guard(f32x4 (&o)[8]) {
  asm volatile("s_nop 7\n\ts_nop 7"
               : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]), "+v"(o[4]), "+v"(o[5]),
                 "+v"(o[6]), "+v"(o[7]));
}

// Reductions over the four lanes holding one query row (lanes c, c+16, c+32,
// c+48) with the gfx950 row-swap permutes (row_swap16 / row_swap32): applied
// to two copies of x, every lane ends up holding the values of both rows of
// its pair, in the same two registers. Every lane therefore combines the same
// operands in the same order, and all four lanes of a row get bitwise equal
// results.
__device__ __forceinline__ float row_max4(float x) {
  float a = x, b = x;
  row_swap16(a, b);
  float c = fmaxf(a, b), d = c;
  row_swap32(c, d);
  return fmaxf(c, d);
}
__device__ __forceinline__ float row_sum4(float x) {
  float a = x, b = x;
  row_swap16(a, b);
  float c = a + b, d = c;
  row_swap32(c, d);
  return c + d;
}

// Regroups the bf16 probability pairs for the PV product. On entry lane group
// G (lanes 16G..16G+15) holds, for its query row, the hi parts (h01, h23) and
// lo parts (l01, l23) of keys 4G..4G+3. On exit the four registers of group 0
// hold the hi parts of keys 0..7, group 1 the hi parts of keys 8..15, group 2
// the lo parts of keys 0..7 and group 3 the lo parts of keys 8..15: the B
// operand whose K slots match a V^T operand holding 8 consecutive keys of one
// value dimension (keys 8*(G & 1)..+7), one 16-byte LDS read with no copies.
// The 32-lane swap moves the lo parts of groups 0-1 up and the hi parts of
// groups 2-3 down; the 16-lane swap then pairs neighbouring groups. Two wait
// states separate each VALU write from the permute that reads it.
__device__ __forceinline__ void pv_regroup(uint32_t& h01, uint32_t& h23, uint32_t& l01,
                                           uint32_t& l23) {
  asm("s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %2\n\t"
      "v_permlane32_swap_b32 %1, %3\n\t"
      "s_nop 1\n\t"
      "v_permlane16_swap_b32 %0, %2\n\t"
      "v_permlane16_swap_b32 %1, %3"
      : "+v"(h01), "+v"(h23), "+v"(l01), "+v"(l23));
}

// Keys past a partial last prefix page have p = 0, but 0 * NaN and 0 * Inf are
// NaN in the PV product: cache positions a sequence has not written yet may
// hold any bits. On such a page (lim < 16, wave-uniform) the V operand's
// elements of keys >= lim are cleared. A lane holds keys 8*(grp & 1) .. +7 of
// one value dimension, two keys per 32-bit word.
__device__ __forceinline__ u32x4 v_key_mask(int lim, int grp) {
  const int nv = min(max(lim - (grp & 1) * 8, 0), 8);  // valid keys of this lane's 8
  u32x4 m;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    m[w] = (2 * w < nv ? 0x0000ffffu : 0u) | (2 * w + 1 < nv ? 0xffff0000u : 0u);
  return m;
}

// Scores, online softmax and PV for one 16-key stage.
//
// S^T = K Q^T (four v_mfma_f32_16x16x32_bf16 over the 128 dimensions) leaves
// keys 4q..4q+3 of one query row in each lane. After the probabilities are
// split and regrouped (pv_regroup), the v_mfma_f32_16x16x32_bf16 that forms
// O^T += V^T P^T takes in each lane 8 keys' hi or lo parts against the
// 16 bytes holding the same 8 keys of one value dimension in the transposed V
// page. Row max and row sum take two row-swap permutes (the 4 lanes holding a
// row).
//
// Softmax: scores are scaled into log2 units inside one FMA. The reference
// max m is raised only when a row's new max exceeds it by more than
// kRescaleLog2 (then O and l are rescaled by 2^(m_old - m_new)); otherwise
// probabilities are taken against the stale m and stay below 2^kRescaleLog2.
// Numerator and denominator share the reference, so the result is exact up
// to rounding, and the rescale runs only in the rare stages that need it.
//
// P enters the PV product as a bf16 pair hi + lo (hi = RNE(p), lo = RNE(p - hi)),
// so the probabilities carry ~16 mantissa bits instead of bf16's 8.
//
// lim: keys kk < lim of the stage are visible to this lane's row. vlim: keys
// kk >= vlim (wave-uniform) are cleared from the V operand as well; a prefix
// page passes vlim = lim, a window chunk kPage (its rows are window inputs, or
// zero past W).
__device__ __forceinline__ void attend_page(RowState& st, const bf16x8 (&qr)[4], const Stage& sg,
                                            int lane, int lim, int vlim, float scale_log2) {
  const int col = lane & 15, grp = lane >> 4;
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const u32x4 kk = *reinterpret_cast<const u32x4*>(&sg.k[s * 512 + lane * 8]);
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kk), qr[s], sc, 0, 0, 0);
  }
  // also separates the previous stage's PV MFMAs from the rescale below
  mfma_result_guard(sc);
  // sc[i] is key 4*grp + i of the page for query row `col`
  float x[4] = {sc[0], sc[1], sc[2], sc[3]};
  if (lim < kPage) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (grp * 4 + i >= lim) x[i] = -INFINITY;
  }
  const float mx = row_max4(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  const float mc = mx * scale_log2;  // candidate max in log2 units (-inf if no visible key)
  const bool raise = mc > st.m + kRescaleLog2;
  if (__ballot(raise)) {
    const float m_new = raise ? mc : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);  // 0 when st.m = -inf
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] *= alpha;
    st.m = m_new;
  }
  const float base = st.m == -INFINITY ? 0.f : st.m;
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(x[i], scale_log2, -base));
  st.l += row_sum4((p[0] + p[1]) + (p[2] + p[3]));
  uint32_t h01 = pack_bf16x2(p[0], p[1]), h23 = pack_bf16x2(p[2], p[3]);
  uint32_t l01 = pack_bf16x2(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
  uint32_t l23 = pack_bf16x2(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
  pv_regroup(h01, h23, l01, l23);
  const u32x4 pb = {h01, h23, l01, l23};
  if (vlim < kPage) {
    const u32x4 vm = v_key_mask(vlim, grp);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const u32x4 va =
          *reinterpret_cast<const u32x4*>(&sg.v[(dt * 16 + col) * kPage + (grp & 1) * 8]) & vm;
      st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(pb), st.o[dt], 0, 0, 0);
    }
    return;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    // keys 8*(grp & 1) .. +7 of value dimension dt*16 + col: one 16-byte read
    const u32x4 va =
        *reinterpret_cast<const u32x4*>(&sg.v[(dt * 16 + col) * kPage + (grp & 1) * 8]);
    st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(pb), st.o[dt], 0, 0, 0);
  }
}

// P^T for the PV product of one page from a lane's 4 probabilities (hi and lo
// bf16 parts, regrouped as in attend_page), then O^T += V^T P^T over the page;
// V elements of keys >= vlim are cleared (a partial last prefix page).
__device__ __forceinline__ void pv_page(RowState& st, const Stage& sg, int col, int grp,
                                        float p0, float p1, float p2, float p3, int vlim) {
  uint32_t h01 = pack_bf16x2(p0, p1), h23 = pack_bf16x2(p2, p3);
  uint32_t l01 = pack_bf16x2(p0 - bf16_lo(h01), p1 - bf16_hi(h01));
  uint32_t l23 = pack_bf16x2(p2 - bf16_lo(h23), p3 - bf16_hi(h23));
  pv_regroup(h01, h23, l01, l23);
  const u32x4 pb = {h01, h23, l01, l23};
  if (vlim < kPage) {
    const u32x4 vm = v_key_mask(vlim, grp);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const u32x4 va =
          *reinterpret_cast<const u32x4*>(&sg.v[(dt * 16 + col) * kPage + (grp & 1) * 8]) & vm;
      st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(pb), st.o[dt], 0, 0, 0);
    }
    return;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const u32x4 va =
        *reinterpret_cast<const u32x4*>(&sg.v[(dt * 16 + col) * kPage + (grp & 1) * 8]);
    st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(pb), st.o[dt], 0, 0, 0);
  }
}

// Two 16-key stages at once (the deep rings): the two score products are
// independent MFMA chains, and the row max, the rescale decision and the row
// sum are taken once over the pair's 32 keys. Otherwise as attend_page; the
// PV products are accumulated in page order.
__device__ __forceinline__ void attend_pages2(RowState& st, const bf16x8 (&qr)[4],
                                              const Stage& s0, const Stage& s1, int lane,
                                              int lim0, int lim1, float scale_log2) {
  const int col = lane & 15, grp = lane >> 4;
  f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const u32x4 ka = *reinterpret_cast<const u32x4*>(&s0.k[s * 512 + lane * 8]);
    const u32x4 kb = *reinterpret_cast<const u32x4*>(&s1.k[s * 512 + lane * 8]);
    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka), qr[s], sa, 0, 0, 0);
    sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kb), qr[s], sb, 0, 0, 0);
  }
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(sa), "+v"(sb));  // as mfma_result_guard
  float x[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
  if (lim0 < kPage) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (grp * 4 + i >= lim0) x[i] = -INFINITY;
  }
  if (lim1 < kPage) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (grp * 4 + i >= lim1) x[4 + i] = -INFINITY;
  }
  const float m8 = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                         fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  const float mc = row_max4(m8) * scale_log2;
  const bool raise = mc > st.m + kRescaleLog2;
  if (__ballot(raise)) {
    const float m_new = raise ? mc : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);  // 0 when st.m = -inf
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] *= alpha;
    st.m = m_new;
  }
  const float base = st.m == -INFINITY ? 0.f : st.m;
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(x[i], scale_log2, -base));
  st.l += row_sum4(((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
  pv_page(st, s0, col, grp, p[0], p[1], p[2], p[3], lim0);
  pv_page(st, s1, col, grp, p[4], p[5], p[6], p[7], lim1);
}



template <int NW>
struct DmaShape {
  static constexpr int kPerWave = kPageVecs / (kWave * NW) > 0 ? kPageVecs / (kWave * NW) : 1;
  static constexpr int kIssuers = kPageVecs / (kWave * kPerWave);  // waves that issue
};

// DMA of one page (K then V of kv head kvh) into a ring stage; id_raw is the
// page's block-table entry (clamped to the pool here).
template <int NW, bool kNt>
__device__ __forceinline__ void stage_dma(Stage& sg, int wave, int lane, int id_raw,
                                          int num_pages, int Hkv, int kvh,
                                          const uint16_t* kc_layer, const uint16_t* vc_layer) {
  constexpr size_t page_elems = static_cast<size_t>(kHeadDim) * kPage;
  using S = DmaShape<NW>;
  if (wave >= S::kIssuers) return;  // wave-uniform
  // generic -> LDS address space: the 32-bit LDS byte address of the stage
  const uint32_t lds_base = static_cast<uint32_t>(
      reinterpret_cast<size_t>((__attribute__((address_space(3))) char*)(&sg)));
  // the page id is wave-uniform: keep it in SGPRs
  const int pid = __builtin_amdgcn_readfirstlane(min(max(id_raw, 0), num_pages - 1));
  const size_t off = (static_cast<size_t>(pid) * Hkv + kvh) * page_elems;
  const uint32_t voff = static_cast<uint32_t>(lane) * 16u;  // lane's 16 bytes of 1 KB
#pragma unroll
  for (int i = 0; i < S::kPerWave; ++i) {
    const int v0 = (i * S::kIssuers + wave) * kWave;  // first vector (wave-uniform)
    // vectors 0..255 are the K part, 256..511 the V part of the page
    const uint16_t* part = (v0 < 256 ? kc_layer : vc_layer) + off + (v0 % 256) * 8;
    const uint64_t sbase = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(
                                static_cast<uint32_t>(reinterpret_cast<uint64_t>(part) >> 32)))
                            << 32) |
                           static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
                               static_cast<uint32_t>(reinterpret_cast<uint64_t>(part))));
    lds_dma_16<kNt>(sbase, voff, __builtin_amdgcn_readfirstlane(lds_base + v0 * 16));
  }
}

// Wait until at most N of this thread's vector-memory operations are in
// flight, then synchronise the workgroup. The memory clobber keeps the
// compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void stage_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}


// Wait for the oldest in-flight stage when `behind` (<= N) later stages,
// kDma DMAs each, may stay in flight, then synchronise the workgroup. The
// count must be an immediate, hence the chain over 0..N.
template <int kDma, int N>
__device__ __forceinline__ void stage_wait_behind(int behind) {
  if constexpr (N == 0) {
    stage_wait_barrier<0>();
  } else {
    if (behind >= N)
      stage_wait_barrier<N * kDma>();
    else
      stage_wait_behind<kDma, N - 1>(behind);
  }
}


// Appends the committed window rows held by the staged chunk (physical rows
// kw0 .. kw0+15, rotated) to the caches: rows 0..c-1 go to positions
// L..L+c-1, with c the run length clamped to the window and to the pages the
// table holds (the commit rule of the commit step). Keys as 16-byte slices,
// values as 2-byte elements of the transposed page; positions of the page
// other than the appended ones are not touched. have_ids: pre0 / pre1 are
// already the block-table entries of the chunk's two pages.
__device__ __forceinline__ void append_committed(const AttnArgs& a, const Stage& sg,
                                                 const int32_t* bt, int b, int layer, int kvh,
                                                 int kw0, int tid, int nthreads, bool have_ids,
                                                 int pre0, int pre1) {
  const int Lc = max(a.prefix_len[b], 0);
  int c = min(max(a.commit_run[b], 0), a.W);
  c = min(c, max(a.max_pages * kPage - Lc, 0));
  const int rows = min(c - kw0, kPage);  // rows of this chunk to append (none if <= 0)
  if (rows <= 0) return;
  uint16_t* kcl = a.kc_w + static_cast<size_t>(layer) * a.cache_layer_stride;
  uint16_t* vcl = a.vc_w + static_cast<size_t>(layer) * a.cache_layer_stride;
  // the chunk's rows lie in at most two pages: their ids once, as scalars
  const int pg0 = (Lc + kw0) / kPage;
  int id0 = pre0, id1 = pre1;  // chunk 0: fetched at the start of the workgroup
  if (!have_ids)
    load_page_ids2(page_entry(bt, pg0, a.max_pages), page_entry(bt, pg0 + 1, a.max_pages), id0,
                   id1);
  id0 = min(max(id0, 0), a.num_pages - 1);
  id1 = min(max(id1, 0), a.num_pages - 1);
  constexpr int kTasksPerRow = 16 + kHeadDim;  // 16 key slices, 128 value elements
  for (int idx = tid; idx < rows * kTasksPerRow; idx += nthreads) {
    const int j = idx / kTasksPerRow, r = idx % kTasksPerRow;
    const int t = Lc + kw0 + j;
    const int pid = t / kPage == pg0 ? id0 : id1;
    const size_t page = (static_cast<size_t>(pid) * a.Hkv + kvh) * kPartElems;
    if (r < 16) {
      *reinterpret_cast<u32x4*>(kcl + page + (r * kPage + t % kPage) * 8) =
          *reinterpret_cast<const u32x4*>(&sg.k[(r * kPage + j) * 8]);
    } else {
      const int d = r - 16;
      vcl[page + d * kPage + t % kPage] = sg.v[d * kPage + j];
    }
  }
}

// ---- key-range splits of a ragged batch ----------------------------------
// In split mode each (layer, kv head) column has S = cols workgroups. The
// work of sequence b is u_b = its prefix pages + its window's 16-key chunks
// (the last split also attends to the window). With a split size of K units,
// sequence b takes ceil(u_b / K) consecutive workgroups of the column, split s
// covering pages [s K, (s+1) K) of its prefix. K is the smallest value, not
// below min_pages, for which the sequences' split counts fit in S: it lies in
// [ceil(P / S), ceil((P - B) / (S - B))] with P = sum u_b, and the upper end
// always fits (ceil(u/K) <= (u - 1)/K + 1 for u >= 1), so a binary search over
// that interval finds it. The first wave of the workgroup evaluates it and
// shares the result through LDS; workgroups past the last split return at
// once.
struct SplitSlot {
  int b;        // sequence, or -1 when this workgroup has no split
  int split;    // index of this split within its sequence
  int n_split;  // splits of the sequence
  int first;    // workgroup index (within the column) of the sequence's split 0
  int K;        // units per split
};

__device__ __forceinline__ int seq_units(const AttnArgs& a, int b) {
  const int L = min(max(a.prefix_len[b], 0), a.max_prefix_len);
  return (L + kPage - 1) / kPage + (a.W + kPage - 1) / kPage;
}

// Inclusive prefix sum over the 64 lanes with DPP (no LDS traffic): shifts
// by 1, 2, 4, 8 lanes within each 16-lane row, then each row adds the last
// lane of the row before it (rows 1 and 3 from rows 0 and 2), then rows 2
// and 3 add lane 31. Lanes whose DPP source lies outside the row add 0.
__device__ __forceinline__ unsigned wave_incl_scan(unsigned x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

__device__ __forceinline__ long long wave_sum_ll(long long x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// sum over sequences of ceil(u_b / K) (K = 1 gives sum u_b)
__device__ __forceinline__ long long split_total(const AttnArgs& a, int K, int lane) {
  long long n = 0;
  for (int b0 = 0; b0 < a.B; b0 += kWave) {
    const int b = b0 + lane;
    const unsigned u = b < a.B ? static_cast<unsigned>(seq_units(a, b)) : 0u;
    n += wave_sum_ll(static_cast<long long>((u + K - 1) / static_cast<unsigned>(K)));
  }
  return n;
}

__device__ SplitSlot find_split(const AttnArgs& a, int j, int lane) {
  const long long S = a.cols, Bn = a.B;  // S > B in split mode
  // a batch of at most one wavefront's sequences keeps each lane's units in a
  // register, and while every count stays below 2^25 (64 of them sum below
  // 2^31) the sums are 32-bit DPP scans: the search below reads prefix_len
  // once and touches no LDS
  const unsigned u_own = (a.B <= kWave && lane < a.B) ? static_cast<unsigned>(seq_units(a, lane)) : 0u;
  const bool one = a.B <= kWave && __ballot(u_own >= (1u << 25)) == 0;
  const unsigned u_lane = one ? u_own : 0u;
  auto total = [&](int K) -> long long {
    if (one)
      return static_cast<long long>(__builtin_amdgcn_readlane(
          wave_incl_scan((u_lane + K - 1) / static_cast<unsigned>(K)), kWave - 1));
    return split_total(a, K, lane);
  };
  const long long P = total(1);
  long long lo = max(static_cast<long long>(a.min_pages), (P + S - 1) / S);
  long long hi = max(lo, (P - Bn + (S - Bn) - 1) / (S - Bn));
  while (lo < hi) {
    const long long mid = (lo + hi) / 2;
    if (total(static_cast<int>(mid)) <= S)
      hi = mid;
    else
      lo = mid + 1;
  }
  const int K = static_cast<int>(lo);
  SplitSlot r{-1, 0, 1, 0, K};
  long long base = 0;  // workgroups taken by the sequences before this chunk
  for (int b0 = 0; b0 < a.B; b0 += kWave) {
    const int b = b0 + lane;
    const int u = one ? static_cast<int>(u_lane) : (b < a.B ? seq_units(a, b) : 0);
    const int n = b < a.B ? (u + K - 1) / K : 0;
    // inclusive prefix sum over the chunk's lanes (split counts are at most
    // S, so the chunk's sum fits in 32 bits)
    const int incl = static_cast<int>(wave_incl_scan(static_cast<unsigned>(n)));
    const long long lo_j = base + incl - n;
    const unsigned long long hit = __ballot(n > 0 && j >= lo_j && j < base + incl);
    if (hit) {
      const int src = __ffsll(static_cast<long long>(hit)) - 1;
      r.b = b0 + src;
      r.first = static_cast<int>(base) + __shfl(incl - n, src, kWave);
      r.n_split = __shfl(n, src, kWave);
      r.split = j - r.first;
      return r;
    }
    base += __shfl(incl, kWave - 1, kWave);
  }
  return r;
}

// NW wavefronts per workgroup, one 16-row tile each. kRope: q, k, v are in
// slot order before RoPE; each query row and window key is gathered through
// perm and rotated at its logical position as it is loaded.
template <int NW, bool kRope, bool kNt>
__global__ void __launch_bounds__(kWave * NW)
__attribute__((amdgpu_waves_per_eu(Ring<NW>::kWavesPerSimd, Ring<NW>::kWavesPerSimd)))
k_window_attn_bf16(AttnArgs a) {
  touch_kernargs<sizeof(AttnArgs)>();
  constexpr int kDma = DmaShape<NW>::kPerWave;  // DMA instructions per issuing thread per stage
  constexpr int kStages = Ring<NW>::kStages;
  constexpr int kAhead = Ring<NW>::kAhead;
  __shared__ Stage stage[kStages];
  __shared__ double s_omega[kRope ? kHeadDim / 2 : 1];
  // the sequence's window order (physical row -> slot, clamped) and logical
  // positions, read once from HBM
  __shared__ int s_perm[kRope ? WEDLM_MAX_WINDOW : 1];
  __shared__ int s_pos[kRope ? WEDLM_MAX_WINDOW : 1];
  __shared__ int s_split[4];

  if (blockIdx.x >= a.attn_blocks) {
    // one chunk of one logit row (4 waves = kEntThreads threads)
    __shared__ EntPartial red[kEntThreads / kWave];
    const long long e = blockIdx.x - a.attn_blocks;
    const int chunk = static_cast<int>(e % a.ent_chunks);
    const int row = static_cast<int>(e / a.ent_chunks);
    if (a.ent_vec)
      entropy_chunk_block<uint16_t, true>(a.ent_logits, a.ent_V, a.ent_chunk_elems, a.ent_chunks,
                                          a.ent_part, chunk, row, red);
    else
      entropy_chunk_block<uint16_t, false>(a.ent_logits, a.ent_V, a.ent_chunk_elems,
                                           a.ent_chunks, a.ent_part, chunk, row, red);
    return;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int col = lane & 15, grp = lane >> 4;

  // Consecutive workgroups go to different XCDs (round robin). With the
  // sequence as the fastest index after the split, each XCD streams every kv
  // head of its sequences; with the kv head there (Hkv = 8), XCD x would read
  // only the x-th 4 KB of every page record, which leaves HBM channels unevenly
  // loaded when pages are allocated in order (measured 4.5 against 5.2 TB/s).
  int bid = blockIdx.x;
  int part = 0;
  if (a.parts > 1) {
    // the row parts of one work unit are kNumXcds ids apart: same XCD, dispatched
    // together, so the second reads the unit's pages from that XCD's L2
    const int xcd = bid % kNumXcds;
    const int rest = bid / kNumXcds;
    part = rest % a.parts;
    bid = (rest / a.parts) * kNumXcds + xcd;
    if (bid >= a.units) return;  // padding of the last XCD round
  }
  // sequence, or (sequence, split) in split mode; a split launch rotates the
  // column's slots by the column index, so that the last splits of the
  // groups (those that also attend to the window) fall on different XCDs
  const int j = a.split ? (bid % a.cols + bid / a.cols) % a.cols : bid % a.cols;
  bid /= a.cols;
  const int kvh = bid % a.Hkv;
  const int layer = bid / a.Hkv;
  int b = j, split = 0, n_split = 1, K = 0;
  if (a.split) {
    if (wave == 0) {
      const SplitSlot sl = find_split(a, j, lane);
      if (lane == 0) {
        s_split[0] = sl.b;
        s_split[1] = sl.split;
        s_split[2] = sl.n_split;
        s_split[3] = sl.K;
      }
    }
    __syncthreads();
    b = __builtin_amdgcn_readfirstlane(s_split[0]);
    if (b < 0) return;  // every wave of the workgroup takes this branch
    split = __builtin_amdgcn_readfirstlane(s_split[1]);
    n_split = __builtin_amdgcn_readfirstlane(s_split[2]);
    K = __builtin_amdgcn_readfirstlane(s_split[3]);
  }
  const int group = (layer * a.B + b) * a.Hkv + kvh;
  const size_t slot = static_cast<size_t>(layer * a.Hkv + kvh) * a.cols + j;

  // The prefix length, the window order and positions, the rotation
  // frequencies and the block-table entries of the first pages are all
  // requested before any of them is used, and complete together at one wait
  // in the prologue below: one round trip, where taking each value as it was
  // loaded made four in a row. The entries are those of the split's first
  // pages, which do not depend on the prefix length (page_entry clamps the
  // index; a split that starts past the prefix requests no page).
  int pl_b = a.prefix_len[b];  // read once: the append's pages need it too
  const int pg_first = a.split ? split * K : 0;
  const bool with_window = split == n_split - 1;
  if (a.split && split == 0 && part == 0 && tid == 0)
    a.ws_plan[group] = make_int2(static_cast<int>(slot), n_split);

  // ---- this wave's 16 query rows (B operand of S^T = K Q^T) ---------------
  // Loaded through asm, before the first pages' DMAs, and retired below with
  // an explicit vmcnt that lets those DMAs stay in flight. (Rows past M read
  // row 0 of the group - valid memory - and are never stored.)
  const size_t lb = static_cast<size_t>(layer) * a.B + b;
  const int row0 = part * a.part_rows;  // first row of this workgroup's part
  const int row = row0 + wave * 16 + col;
  const bool row_ok = row < a.M && wave * 16 < a.part_rows;
  const int prow = row / a.g, hh = row % a.g;
  int qslot = row_ok ? prow : 0;  // window row holding this query row
  int qpos = 0;
  const int32_t* bt = a.block_table + static_cast<size_t>(b) * a.max_pages;
  const uint16_t* kc_layer = a.kc + static_cast<size_t>(layer) * a.cache_layer_stride;
  const uint16_t* vc_layer = a.vc + static_cast<size_t>(layer) * a.cache_layer_stride;
  // set in the prologue, once the prefix length has arrived
  int L, npages, pg_begin, pg_end, npg, pro;
  // The first min(kAhead, npg) pages are requested before the loop; their
  // block-table entries are fetched (scalar loads) while the window order
  // is on its way. The entries of the pages the first chunk of committed
  // rows is appended to (positions L, L + 1, ...) follow the first DMAs.
  constexpr int kAhead2 = (kAhead + 1) / 2 * 2;
  int id_pro[kAhead2];
  const bool appends = kRope && a.commit_run != nullptr && part == 0 && with_window;
  int app_id0 = 0, app_id1 = 0;
  u32x4 qv[4];
  {
    int pm = 0, ps = 0;
    double om = 0.0;
    if constexpr (kRope) {
      if (tid < a.W) {
        pm = a.perm[b * a.W + tid];
        ps = a.pos[b * a.W + tid];
      }
      if (tid < kHeadDim / 2) om = a.omega[tid];
    }
#pragma unroll
    for (int q = 0; q < kAhead2; q += 2)
      load_page_ids2(page_entry(bt, pg_first + q, a.max_pages),
                     page_entry(bt, pg_first + q + 1, a.max_pages), id_pro[q], id_pro[q + 1]);
    // Every load above is in flight: the values are taken here, together
    // (the compiler would otherwise wait for each right after its load, to
    // start the arithmetic on it).
    asm volatile("" : "+v"(pl_b), "+v"(pm), "+v"(ps), "+v"(om));
    pl_b = __builtin_amdgcn_readfirstlane(pl_b);
    L = min(max(pl_b, 0), a.max_prefix_len);
    npages = (L + kPage - 1) / kPage;
    pg_begin = a.split ? min(npages, pg_first) : 0;
    pg_end = a.split ? min(npages, pg_begin + K) : npages;
    npg = pg_end - pg_begin;
    pro = min(kAhead, npg);
    if constexpr (kRope) {
      // frequencies, window order and positions to LDS, all before any
      // asynchronous load is issued (the waits the compiler adds for these
      // are then free)
      if (tid < kHeadDim / 2) s_omega[tid] = om;
      if (tid < a.W) {
        s_perm[tid] = min(max(pm, 0), a.W - 1);
        s_pos[tid] = ps;
      }
      __syncthreads();
      qslot = s_perm[qslot];
      qpos = s_pos[row_ok ? prow : 0];
    }
    {
      // Loaded through asm, before the first pages' DMAs, and retired below
      // with an explicit vmcnt that lets those DMAs stay in flight. (Rows
      // past M read row 0 of the group - valid memory - and are never stored.)
      const uint16_t* qrow =
          a.q + ((lb * a.W + qslot) * a.Hq + kvh * a.g + (row_ok ? hh : 0)) * kHeadDim;
      // qpos is an input so that its load has completed before the query loads
#pragma unroll
      for (int s = 0; s < 4; ++s)
        asm volatile("global_load_dwordx4 %0, %1, off"
                     : "=v"(qv[s])
                     : "v"(qrow + s * 32 + grp * 8), "v"(qpos)
                     : "memory");
    }
#pragma unroll
    for (int j = 0; j < kAhead; ++j)
      if (j < pro)
        stage_dma<NW, kNt>(stage[j], wave, lane, id_pro[j], a.num_pages, a.Hkv, kvh, kc_layer,
                           vc_layer);
    if (appends) {
      const int Lc = max(pl_b, 0);
      load_page_ids2(page_entry(bt, Lc / kPage, a.max_pages),
                     page_entry(bt, Lc / kPage + 1, a.max_pages), app_id0, app_id1);
    }
    // Retire the query loads: only the kAhead stages issued after them may
    // remain. Waves that issue no DMA (none with 4 or 8 waves), and every
    // wave when the split has fewer than kAhead pages, wait for everything
    // first; that asm has no register operands, so nothing touches the query
    // registers before the tied wait below.
    if (wave >= DmaShape<NW>::kIssuers || pro < kAhead)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt vmcnt(%4)"
                 : "+v"(qv[0]), "+v"(qv[1]), "+v"(qv[2]), "+v"(qv[3])
                 : "n"(kAhead * kDma));
  }
  RowState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // waves past the part's last row tile only move data
  const bool computes = wave * 16 < a.part_rows && row0 + wave * 16 < a.M;
  if constexpr (kRope) {
    // this lane holds dims s*32 + grp*8 .. +7: slices s and s+2 are a RoPE pair
    rope_pair(qv[0], qv[2], static_cast<double>(qpos), s_omega, grp * 8);
    rope_pair(qv[1], qv[3], static_cast<double>(qpos), s_omega, 32 + grp * 8);
  }
  bf16x8 qr[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) qr[s] = as_bf16x8(qv[s]);

  // Ring of kStages stages. The prologue requested pages 0 .. kAhead-1. At
  // iteration i each thread waits for its own DMAs of page i and one barrier
  // makes every wave's part visible; every wave has then also finished
  // computing page i-1 (its LDS reads retired before it reached the barrier),
  // so that stage is refilled with page i+kAhead right away: kAhead pages are
  // in flight while the waves compute, one barrier per page.
  // The deep rings (kPair) take pages i and i+1 per barrier and refill the two
  // stages computed before them (kAhead = kStages - 2); an odd last page is
  // taken alone.
  // The first window chunk's rows are requested by DMA once no page is left
  // to request, into the two stages the last pages no longer need: raw keys
  // (gathered through the window order, slice-major as a page's K part) into
  // stage win_a, raw values in the same order into stage win_b's K part. After
  // the ring the keys are rotated in place and the values transposed into
  // win_a's V part, with no global access left in the window phase.
  const int row_stride = a.Hkv * kHeadDim;
  const uint16_t* kwin = a.k + lb * a.W * row_stride + kvh * kHeadDim;
  const uint16_t* vwin = a.v + lb * a.W * row_stride + kvh * kHeadDim;
  constexpr bool kPrefetchWin = kRope && NW == 4;
  int win_a = 0, win_b = 1;
  bool win_issued = false;
  // x: the first page taken at this barrier; pages x-2 and x-1 (stages
  // (x+2)%4 and (x+3)%4) were computed before it and no page is refilled
  auto prefetch_window = [&](int x) {
    if constexpr (kPrefetchWin) {
      if (!with_window || win_issued) return;
      win_issued = true;
      win_a = (x + 2) % kStages;
      win_b = (x + 3) % kStages;
      // wave w moves slices 4w .. 4w+3 of the 16 keys: K, then V
      const int j = lane & 15, sl = wave * 4 + (lane >> 4);
      const int slot = s_perm[min(j, a.W - 1)];  // keys past W: a valid row, never used
      const uint16_t* kr = kwin + slot * row_stride + sl * 8;
      const uint16_t* vr = vwin + slot * row_stride + sl * 8;
      const uint32_t la = static_cast<uint32_t>(
          reinterpret_cast<size_t>((__attribute__((address_space(3))) char*)(&stage[win_a])));
      const uint32_t lb_ = static_cast<uint32_t>(
          reinterpret_cast<size_t>((__attribute__((address_space(3))) char*)(&stage[win_b])));
      uint32_t saved;
      asm volatile(
          "s_mov_b32 %0, m0\n\t"
          "s_mov_b32 m0, %3\n\t"
          "global_load_lds_dwordx4 %1, off\n\t"
          "s_mov_b32 m0, %4\n\t"
          "global_load_lds_dwordx4 %2, off\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(saved)
          : "v"(kr), "v"(vr), "s"(__builtin_amdgcn_readfirstlane(la + wave * 1024)),
            "s"(__builtin_amdgcn_readfirstlane(lb_ + wave * 1024))
          : "memory");
    }
  };
  int i0 = 0;
  if constexpr (Ring<NW>::kPair) {
    for (; i0 + 1 < npg; i0 += 2) {
      const int pg = pg_begin + i0;
      // pages requested after page i0+1: up to kAhead-2, fewer near the end
      stage_wait_behind<kDma, kAhead - 2>(min(kAhead - 2, npg - 2 - i0));
      if (i0 + kAhead >= npg) prefetch_window(i0);  // after the last page's DMA
      if (i0 + kAhead < npg) {
        // both pages' block-table entries with one scalar wait
        int id0, id1;
        load_page_ids2(page_entry(bt, pg + kAhead, a.max_pages),
                       page_entry(bt, pg + kAhead + 1, a.max_pages), id0, id1);
        stage_dma<NW, kNt>(stage[(i0 + kAhead) % kStages], wave, lane, id0, a.num_pages, a.Hkv,
                           kvh, kc_layer, vc_layer);
        if (i0 + kAhead + 1 < npg)
          stage_dma<NW, kNt>(stage[(i0 + kAhead + 1) % kStages], wave, lane, id1, a.num_pages,
                             a.Hkv, kvh, kc_layer, vc_layer);
      }
      if (computes)
        attend_pages2(st, qr, stage[i0 % kStages], stage[(i0 + 1) % kStages], lane,
                      L - pg * kPage, L - (pg + 1) * kPage, a.scale_log2);
    }
  }
  for (int i = i0; i < npg; ++i) {
    const int pg = pg_begin + i;
    // pages requested after page i: up to kAhead-1, fewer near the end
    stage_wait_behind<kDma, kAhead - 1>(min(kAhead - 1, npg - 1 - i));
    if (i + kAhead >= npg) prefetch_window(i);
    if (i + kAhead < npg)
      stage_dma<NW, kNt>(stage[(i + kAhead) % kStages], wave, lane,
                         load_page_id(page_entry(bt, pg + kAhead, a.max_pages)), a.num_pages,
                         a.Hkv, kvh, kc_layer, vc_layer);
    if (computes)
      attend_page(st, qr, stage[i % kStages], lane, L - pg * kPage, L - pg * kPage, a.scale_log2);
  }
  // The window reuses stage 0: every DMA must have landed before it is
  // overwritten (and none may be in flight when the workgroup ends). The
  // compiler does not see the asm DMAs, so a plain __syncthreads() would not
  // wait for them.
  stage_wait_barrier<0>();

  // ---- the window's own keys, causal over physical order -------------------
  if (with_window) {
    if (kPrefetchWin && !win_issued) {
      // no page at all: every stage is free
      prefetch_window(0);
      stage_wait_barrier<0>();
    }
    for (int kw0 = 0; kw0 < a.W; kw0 += kPage) {
      Stage& sg = stage[win_a];
      // 16 keys x 16 slices of 8 dims: K goes to [slice][key][8], V is transposed
      auto put = [&](int j, int sl, u32x4 kv, u32x4 vv) {
        *reinterpret_cast<u32x4*>(&sg.k[(sl * kPage + j) * 8]) = kv;
        uint16_t* vt = &sg.v[(sl * 8) * kPage + j];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          vt[(2 * w) * kPage] = static_cast<uint16_t>(vv[w]);
          vt[(2 * w + 1) * kPage] = static_cast<uint16_t>(vv[w] >> 16);
        }
      };
      if constexpr (kRope) {
        // keys, gathered through perm: one task per (key, slice pair sl / sl+8,
        // 32-bit word), the two dims of the word rotated with their partners
        // (small tasks keep the registers of the running O free)
        uint32_t* kw = reinterpret_cast<uint32_t*>(sg.k);
        // chunk 0 was moved in raw by DMA: keys in place in sg.k, values in
        // stage win_b's K part; every (key, slice pair, word) task reads and
        // writes only its own two words
        const bool pre = kPrefetchWin && kw0 == 0;
        const uint32_t* vraw = reinterpret_cast<const uint32_t*>(stage[win_b].k);
        for (int idx = tid; idx < kPage * 8 * 4; idx += kWave * NW) {
          const int j = idx >> 5, sl = (idx >> 2) & 7, w = idx & 3;
          const int key = kw0 + j;
          uint32_t lo = 0u, hi = 0u;
          if (key < a.W) {
            uint32_t x, y;
            if (pre) {
              x = kw[((sl * kPage + j) * 8) / 2 + w];
              y = kw[(((sl + 8) * kPage + j) * 8) / 2 + w];
            } else {
              const int slot = s_perm[key];
              const uint16_t* kr = kwin + slot * row_stride + sl * 8 + 2 * w;
              x = *reinterpret_cast<const uint32_t*>(kr);
              y = *reinterpret_cast<const uint32_t*>(kr + kHeadDim / 2);
            }
            const double t = static_cast<double>(s_pos[key]);
            float c0, s0, c1, s1;
            rope_cos_sin(t, s_omega[sl * 8 + 2 * w], c0, s0);
            rope_cos_sin(t, s_omega[sl * 8 + 2 * w + 1], c1, s1);
            const float a0 = bf16_lo(x), a1 = bf16_hi(x), h0 = bf16_lo(y), h1 = bf16_hi(y);
            lo = pack_bf16x2(a0 * c0 - h0 * s0, a1 * c1 - h1 * s1);
            hi = pack_bf16x2(h0 * c0 + a0 * s0, h1 * c1 + a1 * s1);
          }
          kw[((sl * kPage + j) * 8) / 2 + w] = lo;
          kw[(((sl + 8) * kPage + j) * 8) / 2 + w] = hi;
        }
        // values, gathered through perm
        for (int idx = tid; idx < kPage * 16; idx += kWave * NW) {
          const int j = idx >> 4, sl = idx & 15;
          const int key = kw0 + j;
          u32x4 vv = {0u, 0u, 0u, 0u};
          if (key < a.W)
            vv = pre ? *reinterpret_cast<const u32x4*>(vraw + (sl * kPage + j) * 4)
                     : *reinterpret_cast<const u32x4*>(vwin + s_perm[key] * row_stride + sl * 8);
          uint16_t* vt = &sg.v[(sl * 8) * kPage + j];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vt[(2 * e) * kPage] = static_cast<uint16_t>(vv[e]);
            vt[(2 * e + 1) * kPage] = static_cast<uint16_t>(vv[e] >> 16);
          }
        }
      } else {
        for (int idx = tid; idx < kPage * 16; idx += kWave * NW) {
          const int j = idx >> 4, sl = idx & 15;
          const int key = kw0 + j;
          u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
          if (key < a.W) {
            kv = *reinterpret_cast<const u32x4*>(kwin + key * row_stride + sl * 8);
            vv = *reinterpret_cast<const u32x4*>(vwin + key * row_stride + sl * 8);
          }
          put(j, sl, kv, vv);
        }
      }
      lds_barrier();
      if constexpr (kRope) {
        if (appends)
          append_committed(a, sg, bt, b, layer, kvh, kw0, tid, kWave * NW, kw0 == 0, app_id0,
                           app_id1);
      }
      // the appended rows' stores may still be in flight at the barrier below:
      // it only protects the stage for the next chunk
      if (computes) {
        const int lim = min(a.W, prow + 1) - kw0;  // window key kw0 + kk visible iff kk < lim
        attend_page(st, qr, sg, lane, lim, kPage, a.scale_log2);
      }
      lds_barrier();
    }
  }

  // ---- write out ------------------------------------------------------------
  mfma_result_guard(st.o);
  if (!row_ok) return;
  if (!a.split) {
    const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
    uint16_t* orow = a.out + ((lb * a.W + prow) * a.Hq + kvh * a.g + hh) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const u32x2 w = {pack_bf16x2(st.o[dt][0] * inv, st.o[dt][1] * inv),
                       pack_bf16x2(st.o[dt][2] * inv, st.o[dt][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + dt * 16 + grp * 4) = w;
    }
  } else {
    float* o = a.ws_o + (slot * a.M + row) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<float4*>(o + dt * 16 + grp * 4) =
          make_float4(st.o[dt][0], st.o[dt][1], st.o[dt][2], st.o[dt][3]);
    if (grp == 0) {
      float* ml = a.ws_ml + (slot * a.M + row) * 2;
      ml[0] = st.m;
      ml[1] = st.l;
    }
  }
}

// ---------------------------------------------------------------------------
// Wide groups: M = W*g of 129..256 query rows (g = 7 with W = 32, g = 4 with
// W = 64, ...). One workgroup of 8 wavefronts per (layer, sequence, kv head,
// key-range split) takes all M rows with the 32-row tiles of attn_tile32.hpp
// (wavefront w: rows 32w .. 32w+31, row = physical row * g + head), so every
// page is read once per split; the 16-row kernel runs such a group as several
// 4-wave row parts, each reading every page (at the g = 7, W = 32 shape the
// page stream alone, with no compute, took 56 us for 4 parts). The split's
// pages come in 64-key tiles through a 3-stage LDS ring (one workgroup per
// CU, two tiles in flight while one is computed); the last split stages the
// window's own keys once into a tile of its own - gathered through the
// window order and rotated at their logical positions, the committed rows
// appended to the cache from there - and attends to them causally in
// physical order. Split plan, partial layout and merge are the 16-row
// kernel's (find_split, ws_o / ws_ml / ws_plan, combine_quad).
// ---------------------------------------------------------------------------
constexpr int kWideStages = 3;
constexpr int kWideAhead = kWideStages - 1;  // tiles in flight while one is computed
static_assert(kWideAhead == 2, "tile_wait_barrier covers one tile behind the computed one");

template <bool kRope, bool kNt>
__global__ void __launch_bounds__(kTileThreads) k_window_attn_wide(AttnArgs a) {
  touch_kernargs<sizeof(AttnArgs)>();
  __shared__ Tile ring[kWideStages];
  __shared__ Tile own;  // the window's own keys (W <= 64): K rotated, V plain then fp16
  __shared__ double s_omega[kRope ? kHeadDim / 2 : 1];
  __shared__ int s_perm[kRope ? WEDLM_MAX_WINDOW : 1];
  __shared__ int s_pos[kRope ? WEDLM_MAX_WINDOW : 1];
  __shared__ int s_split[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, h = lane >> 5;

  int bid = blockIdx.x;
  // sequence, or (sequence, split) in split mode; a split launch rotates the
  // column's slots by the column index, so that the last splits of the
  // groups (those that also attend to the window) fall on different XCDs
  const int j = a.split ? (bid % a.cols + bid / a.cols) % a.cols : bid % a.cols;
  bid /= a.cols;
  const int kvh = bid % a.Hkv;
  const int layer = bid / a.Hkv;
  int b = j, split = 0, n_split = 1;
  int K = 0;
  if (a.split) {
    if (wave == 0) {
      const SplitSlot sl = find_split(a, j, lane);
      if (lane == 0) {
        s_split[0] = sl.b;
        s_split[1] = sl.split;
        s_split[2] = sl.n_split;
        s_split[3] = sl.K;
      }
    }
    __syncthreads();
    b = __builtin_amdgcn_readfirstlane(s_split[0]);
    if (b < 0) return;  // every wave of the workgroup takes this branch
    split = __builtin_amdgcn_readfirstlane(s_split[1]);
    n_split = __builtin_amdgcn_readfirstlane(s_split[2]);
    K = __builtin_amdgcn_readfirstlane(s_split[3]);
  }
  const int group = (layer * a.B + b) * a.Hkv + kvh;
  const size_t slot = static_cast<size_t>(layer * a.Hkv + kvh) * a.cols + j;
  const int pl_b = a.prefix_len[b];
  const int L = min(max(pl_b, 0), a.max_prefix_len);
  const int npages = (L + kPage - 1) / kPage;
  const int pg_begin = a.split ? min(npages, split * K) : 0;
  const int pg_end = a.split ? min(npages, pg_begin + K) : npages;
  const bool with_window = split == n_split - 1;
  if (a.split && split == 0 && tid == 0)
    a.ws_plan[group] = make_int2(static_cast<int>(slot), n_split);
  // the split's keys: positions key_begin .. key_end - 1
  const int key_begin = pg_begin * kPage;
  const int key_end = min(L, pg_end * kPage);
  const int n_tiles = max(key_end - key_begin, 0) / kTileKeys +
                      (max(key_end - key_begin, 0) % kTileKeys != 0 ? 1 : 0);
  const bool appends = kRope && a.commit_run != nullptr && with_window;

  // this lane's query row (rows past M take row 0's inputs and are never stored)
  const size_t lb = static_cast<size_t>(layer) * a.B + b;
  const int r = wave * 32 + li;
  const bool row_ok = r < a.M;
  const int rr = row_ok ? r : 0;
  const int prow = rr / a.g, hh = rr % a.g;
  const int32_t* bt = a.block_table + static_cast<size_t>(b) * a.max_pages;
  const uint16_t* kc_layer = a.kc + static_cast<size_t>(layer) * a.cache_layer_stride;
  const uint16_t* vc_layer = a.vc + static_cast<size_t>(layer) * a.cache_layer_stride;

  if constexpr (kRope) {
    if (tid < kHeadDim / 2) s_omega[tid] = a.omega[tid];
    if (tid < a.W) {
      s_perm[tid] = min(max(a.perm[b * a.W + tid], 0), a.W - 1);
      s_pos[tid] = a.pos[b * a.W + tid];
    }
  }
  __syncthreads();

  auto issue_tile = [&](int t) {
    int id[kTilePages];  // pages past the split: valid memory, cleared below
    load_page_ids4(bt, pg_begin + t * kTilePages, a.max_pages, id);
    tile_dma<kNt>(ring[t % kWideStages], id, kc_layer, vc_layer, a.Hkv, kvh, a.num_pages, wave,
                  lane);
  };
  // The DMAs are issued before the plain loads below: those complete in
  // order after them, so every wait the compiler places for its own loads
  // also covers the DMAs, and the ring's explicit counts start from zero.
  for (int t = 0; t < kWideAhead && t < n_tiles; ++t) issue_tile(t);

  // (cos, sin) of the window rows' positions at every frequency, formed once
  // into ring stage kWideAhead, which no DMA fills before the ring's first
  // barrier
  static_assert(sizeof(Tile) >= WEDLM_MAX_WINDOW * (kHeadDim / 2) * sizeof(f32x2),
                "RoPE table size");
  const f32x2* cs_tab = reinterpret_cast<const f32x2*>(&ring[kWideAhead]);
  if constexpr (kRope) {
    f32x2* tab = reinterpret_cast<f32x2*>(&ring[kWideAhead]);
    for (int e = tid; e < a.W * (kHeadDim / 2); e += kTileThreads) {
      float c, sn;
      rope_cos_sin(static_cast<double>(s_pos[e >> 6]), s_omega[e & 63], c, sn);
      tab[e] = f32x2{c, sn};
    }
    __syncthreads();
  }

  // query rows: lane half h holds dims 16 s + 8 h .. +7 (B operand of K-step s)
  bf16x8 qr[8];
  {
    const int qslot = kRope ? s_perm[prow] : prow;
    const uint16_t* qrow =
        a.q + ((lb * a.W + qslot) * a.Hq + static_cast<size_t>(kvh) * a.g + hh) * kHeadDim;
    u32x4 qv[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qv[ks] = *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * h);
    if constexpr (kRope) {
      // dims 16 ks + 8 h + e and 16 (ks + 4) + 8 h + e are a rotate-half pair
      const f32x2* cs = cs_tab + prow * (kHeadDim / 2);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) rope_pair_tab(qv[ks], qv[ks + 4], cs, 16 * ks + 8 * h);
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qr[ks] = as_bf16x8(qv[ks]);
  }

  RowState32 st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[dt][e] = 0.f;

  // ---- the window's own keys, causal over physical order -------------------
  if (with_window) {
    const int row_stride = a.Hkv * kHeadDim;
    const uint16_t* kwin = a.k + lb * a.W * row_stride + kvh * kHeadDim;
    const uint16_t* vwin = a.v + lb * a.W * row_stride + kvh * kHeadDim;
    {
      // keys: one (key, slice pair) per thread, rotated at the key's position
      const int kk = tid & 63, sl = tid >> 6;
      u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
      if (kk < a.W) {
        const uint16_t* krow = kwin + (kRope ? s_perm[kk] : kk) * row_stride;
        lo = *reinterpret_cast<const u32x4*>(krow + sl * 8);
        hi = *reinterpret_cast<const u32x4*>(krow + kHeadDim / 2 + sl * 8);
        if constexpr (kRope) rope_pair_tab(lo, hi, cs_tab + kk * (kHeadDim / 2), sl * 8);
      }
      Stage& pg = own.pg[kk >> 4];
      *reinterpret_cast<u32x4*>(&pg.k[(sl * kPage + (kk & 15)) * 8]) = lo;
      *reinterpret_cast<u32x4*>(&pg.k[((sl + 8) * kPage + (kk & 15)) * 8]) = hi;
    }
    // values, plain [dim][key] bf16 (the layout the committed-row append reads)
    for (int task = tid; task < kTileKeys * 16; task += kTileThreads) {
      const int kk = task & 63, dv = task >> 6;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (kk < a.W)
        val = *reinterpret_cast<const u32x4*>(vwin + (kRope ? s_perm[kk] : kk) * row_stride +
                                              dv * 8);
      uint16_t* vt = &own.pg[kk >> 4].v[(dv * 8) * kPage + (kk & 15)];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        vt[(2 * w) * kPage] = static_cast<uint16_t>(val[w] & 0xffffu);
        vt[(2 * w + 1) * kPage] = static_cast<uint16_t>(val[w] >> 16);
      }
    }
    __syncthreads();
    if constexpr (kRope) {
      if (appends) {
        for (int kw0 = 0; kw0 < a.W; kw0 += kPage)
          append_committed(a, own.pg[kw0 / kPage], bt, b, layer, kvh, kw0, tid, kTileThreads,
                           false, 0, 0);
        __syncthreads();  // the append's LDS reads are done before V is rewritten
      }
    }
    {
      // values to fp16, in the vslot order: dimension d of page p (its two
      // 16-byte vectors, keys 0..7 and 8..15) per thread
      const int p = tid >> 7, d = tid & 127;
      uint16_t* v = own.pg[p].v;
      u32x4 w0 = *reinterpret_cast<const u32x4*>(v + (2 * d) * 8);
      u32x4 w1 = *reinterpret_cast<const u32x4*>(v + (2 * d + 1) * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0[e] = bf16x2_to_f16x2(w0[e]);
        w1[e] = bf16x2_to_f16x2(w1[e]);
      }
      *reinterpret_cast<u32x4*>(v + vslot(d, 0) * 8) = w0;
      *reinterpret_cast<u32x4*>(v + vslot(d, 1) * 8) = w1;
    }
    __syncthreads();
    // window key kk is visible to physical row prow iff kk <= prow (and kk < W)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int pa = 32 * hf;
      const int hi = min(prow + 1, a.W) - pa;
      if (!__ballot(hi > 0)) continue;  // wave-uniform
      attend32(st, qr, own.pg[2 * hf], own.pg[2 * hf + 1], lane, 0, hi, 0, hi - kPage,
               a.scale_log2);
    }
  }

  // ---- the split's cache tiles ------------------------------------------------
  // Tile t + 1's values are converted to fp16 while tile t is computed, so one
  // barrier per tile both publishes them and frees the stage tile t + 2 takes.
  // In each tile the keys past the split (pages past it, or positions past
  // the prefix) are cleared from the values and masked from the scores.
  auto tile_keys = [&](int t) { return key_end - (key_begin + t * kTileKeys); };
  if (n_tiles > 0) {
    tile_wait_barrier(min(kWideAhead - 1, n_tiles - 1));  // tile 0 has landed
    tile_v_to_f16(ring[0], tid, tile_keys(0));
  }
  for (int t = 0; t < n_tiles; ++t) {
    // only tile t + 1's DMAs can be in flight here: after this barrier it has
    // landed everywhere, tile t's values are fp16 everywhere, and tile t - 1's
    // stage is free
    tile_wait_barrier(0);
    if (t + kWideAhead < n_tiles) issue_tile(t + kWideAhead);
    if (t + 1 < n_tiles) tile_v_to_f16(ring[(t + 1) % kWideStages], tid, tile_keys(t + 1));
    const Tile& tl = ring[t % kWideStages];
    const int nv = tile_keys(t);  // every row sees the keys of the tile below nv
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int pa = 32 * hf;
      if (nv <= pa) continue;  // workgroup-uniform
      attend32(st, qr, tl.pg[2 * hf], tl.pg[2 * hf + 1], lane, 0, nv - pa, 0, nv - pa - kPage,
               a.scale_log2);
    }
  }
  // no DMA may be in flight when the workgroup ends (n_tiles = 0: none issued)

  // ---- write out ----------------------------------------------------------------
  mfma32_guard(st.o[0]);
  mfma32_guard(st.o[1]);
  mfma32_guard(st.o[2]);
  mfma32_guard(st.o[3]);
  st.l = half_sum(st.l);  // every lane takes part in the swap
  if (!row_ok) return;
  if (!a.split) {
    const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
    uint16_t* orow =
        a.out + ((lb * a.W + prow) * a.Hq + static_cast<size_t>(kvh) * a.g + hh) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 w = {pack_bf16x2(st.o[dt][4 * q] * inv, st.o[dt][4 * q + 1] * inv),
                         pack_bf16x2(st.o[dt][4 * q + 2] * inv, st.o[dt][4 * q + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + dt * 32 + 8 * q + 4 * h) = w;
      }
  } else {
    float* o = a.ws_o + (slot * a.M + r) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(o + dt * 32 + 8 * q + 4 * h) =
            make_float4(st.o[dt][4 * q], st.o[dt][4 * q + 1], st.o[dt][4 * q + 2],
                        st.o[dt][4 * q + 3]);
    if (h == 0) {
      float* ml = a.ws_ml + (slot * a.M + r) * 2;
      ml[0] = st.m;
      ml[1] = st.l;
    }
  }
}

// Merge of the per-split partials (combine_quad, attn_combine.hpp): one
// thread per (group, row, 4 value dimensions).
__global__ void __launch_bounds__(256) k_window_attn_combine(CombineArgs c) {
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx < c.threads) combine_quad(c, idx);
}

// ---------------------------------------------------------------------------
// f32 path (small shapes): one wavefront per (layer, sequence, query head,
// physical row); 64 keys per step, one key per lane for the scores, then every
// lane accumulates its own output dimensions. K page [Hkv][D/4][P][4],
// V page [Hkv][D][P] as for bf16 with 16-byte slices of 4 floats.
// ---------------------------------------------------------------------------
constexpr int kF32MaxD = 256;

// RoPE inputs of the fused f32 path: row -> slot, positions, D/2 frequencies.
struct RopeF32 {
  const int32_t* perm;
  const int32_t* pos;
  double omega[kF32MaxD / 2];
};

// kSmall (D <= 64): each lane holds one output dimension, and every key's
// value for it is requested before the keys' scores are formed, so the
// value loads wait alongside the key loads instead of after the softmax.
template <bool kRope, bool kSmall>
__global__ void __launch_bounds__(kWave)
k_window_attn_f32(const float* __restrict__ q, const float* __restrict__ k,
                  const float* __restrict__ v, const float* __restrict__ kc,
                  const float* __restrict__ vc, const int32_t* __restrict__ block_table,
                  const int32_t* __restrict__ prefix_len, float* __restrict__ out, int B, int W,
                  int Hq, int Hkv, int D, int num_pages, int max_pages, int max_prefix_len,
                  long long cache_layer_stride, float scale_log2, RopeF32 rp,
                  long long attn_blocks, const int32_t* __restrict__ commit_run,
                  float* __restrict__ kc_w, float* __restrict__ vc_w) {
  __shared__ float qs[kF32MaxD];
  const int lane = threadIdx.x;
  if constexpr (kRope) {
    // blocks past the attention's append the committed rows (commit_run given):
    // one block per (layer, sequence, kv head), at positions the attention
    // does not read (L and beyond), rotated at the attention's positions
    if (static_cast<long long>(blockIdx.x) >= attn_blocks) {
      const long long e = blockIdx.x - attn_blocks;
      const int kvh_c = static_cast<int>(e % Hkv);
      const int b_c = static_cast<int>((e / Hkv) % B);
      const int layer_c = static_cast<int>(e / (1LL * Hkv * B));
      commit_rows_block<float, true>(B, W, Hkv, D, kPage, num_pages, max_pages, commit_run,
                                     prefix_len, k, v, block_table, kc_w, vc_w,
                                     cache_layer_stride, rp.omega, rp.pos, b_c, kvh_c, layer_c,
                                     lane, kWave);
      return;
    }
  }
  int bid = blockIdx.x;
  const int p = bid % W;
  bid /= W;
  const int h = bid % Hq;
  bid /= Hq;
  const int b = bid % B;
  const int layer = bid / B;
  const int g = Hq / Hkv, kvh = h / g;
  const size_t lb = static_cast<size_t>(layer) * B + b;
  const int half = D / 2;
  // kRope: window rows are gathered through perm and rotated at their
  // logical position as they are read
  auto slot_of = [&](int row) { return kRope ? min(max(rp.perm[b * W + row], 0), W - 1) : row; };
  if constexpr (kRope) {
    const float* qr = q + ((lb * W + slot_of(p)) * Hq + h) * D;
    const double tq = static_cast<double>(rp.pos[b * W + p]);
    for (int j = lane; j < half; j += kWave) {
      float c, sn;
      rope_cos_sin(tq, rp.omega[j], c, sn);
      qs[j] = qr[j] * c - qr[j + half] * sn;
      qs[j + half] = qr[j + half] * c + qr[j] * sn;
    }
  } else {
    for (int d = lane; d < D; d += kWave) qs[d] = q[((lb * W + p) * Hq + h) * D + d];
  }
  // kSmall: the rotations of window rows 0..p, (cos, sin) per frequency,
  // computed once by all lanes rather than per key by the lane holding it
  __shared__ float2 s_cs[kSmall && kRope ? WEDLM_MAX_WINDOW * (kWave / 2) : 1];
  if constexpr (kSmall && kRope) {
    for (int e = lane; e < (p + 1) * half; e += kWave) {
      const int r = e / half, j = e % half;
      float c, sn;
      rope_cos_sin(static_cast<double>(rp.pos[b * W + r]), rp.omega[j], c, sn);
      s_cs[e] = make_float2(c, sn);
    }
  }
  __syncthreads();
  const int L = min(max(prefix_len[b], 0), max_prefix_len);
  const int nkeys = L + p + 1;
  const int32_t* bt = block_table + static_cast<size_t>(b) * max_pages;
  const float* kcl = kc + static_cast<size_t>(layer) * cache_layer_stride;
  const float* vcl = vc + static_cast<size_t>(layer) * cache_layer_stride;
  const size_t page_elems = static_cast<size_t>(D) * kPage;
  float m = -INFINITY, l = 0.f;
  float o[kF32MaxD / kWave];
#pragma unroll
  for (int i = 0; i < kF32MaxD / kWave; ++i) o[i] = 0.f;
  for (int k0 = 0; k0 < nkeys; k0 += kWave) {
    const int key = k0 + lane;
    const int nk = min(kWave, nkeys - k0);
    float vk[kSmall ? kWave : 1];
    if constexpr (kSmall) {
#pragma unroll
      for (int j = 0; j < kWave; ++j) {
        const int kj = k0 + min(j, nk - 1);  // keys past nk: a valid row, weight 0 below
        const float* src;
        int stride = 1;
        if (kj < L) {
          const int pid = min(max(bt[kj / kPage], 0), num_pages - 1);
          src = vcl + (static_cast<size_t>(pid) * Hkv + kvh) * page_elems + kj % kPage;
          stride = kPage;
        } else {
          src = v + ((lb * W + slot_of(kj - L)) * Hkv + kvh) * D;
        }
        vk[j] = lane < D ? src[lane * stride] : 0.f;
      }
    }
    float sc = -INFINITY;
    if (key < nkeys) {
      float dot = 0.f;
      // 16-byte loads, unrolled so that several are in flight at once
      const float4* q4 = reinterpret_cast<const float4*>(qs);
      if (key < L) {
        const int pid = min(max(bt[key / kPage], 0), num_pages - 1);
        const float4* kp4 = reinterpret_cast<const float4*>(
                                kcl + (static_cast<size_t>(pid) * Hkv + kvh) * page_elems) +
                            key % kPage;
#pragma unroll 4
        for (int d4 = 0; d4 < D / 4; ++d4) {
          const float4 kv = kp4[d4 * kPage], qv = q4[d4];
          dot += qv.x * kv.x + qv.y * kv.y + qv.z * kv.z + qv.w * kv.w;
        }
      } else if constexpr (kRope) {
        const int r = key - L;
        const float4* kr4 =
            reinterpret_cast<const float4*>(k + ((lb * W + slot_of(r)) * Hkv + kvh) * D);
        const double tk = static_cast<double>(rp.pos[b * W + r]);
#pragma unroll 2
        for (int j4 = 0; j4 < half / 4; ++j4) {
          const float4 lo = kr4[j4], hi = kr4[j4 + half / 4];
          const float4 ql = q4[j4], qh = q4[j4 + half / 4];
          const float al[4] = {lo.x, lo.y, lo.z, lo.w}, ah[4] = {hi.x, hi.y, hi.z, hi.w};
          const float bl[4] = {ql.x, ql.y, ql.z, ql.w}, bh[4] = {qh.x, qh.y, qh.z, qh.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float c, sn;
            if constexpr (kSmall) {
              const float2 cs = s_cs[r * half + 4 * j4 + e];
              c = cs.x;
              sn = cs.y;
            } else {
              rope_cos_sin(tk, rp.omega[4 * j4 + e], c, sn);
            }
            dot += bl[e] * (al[e] * c - ah[e] * sn) + bh[e] * (ah[e] * c + al[e] * sn);
          }
        }
      } else {
        const float4* kr4 =
            reinterpret_cast<const float4*>(k + ((lb * W + (key - L)) * Hkv + kvh) * D);
#pragma unroll 4
        for (int d4 = 0; d4 < D / 4; ++d4) {
          const float4 kv = kr4[d4], qv = q4[d4];
          dot += qv.x * kv.x + qv.y * kv.y + qv.z * kv.z + qv.w * kv.w;
        }
      }
      sc = dot * scale_log2;
    }
    const float mx = wave_max(sc);
    const float m_new = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    const float pk = key < nkeys ? __builtin_amdgcn_exp2f(sc - m_new) : 0.f;
    l = l * alpha + wave_sum(pk);
    m = m_new;
#pragma unroll
    for (int i = 0; i < kF32MaxD / kWave; ++i) o[i] *= alpha;
    if constexpr (kSmall) {
      // the values are in registers: accumulate in key order
#pragma unroll
      for (int j = 0; j < kWave; ++j) {
        const float pj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pk), j));
        if (j < nk) o[0] += pj * vk[j];
      }
      continue;
    }
    // PV over this step's keys, kPvBatch keys at a time: the batch's values
    // are all requested before any is used (one key at a time left a chain of
    // dependent block-table and value loads per key), then accumulated in key
    // order.
    constexpr int kPvBatch = 8;
    for (int j0 = 0; j0 < nk; j0 += kPvBatch) {
      float pj[kPvBatch];
      float vv[kPvBatch][kF32MaxD / kWave];
#pragma unroll
      for (int u = 0; u < kPvBatch; ++u) {
        const int j = j0 + u;
        pj[u] = __shfl(pk, min(j, kWave - 1), kWave);
        const int kj = k0 + j;
        const float* src = nullptr;
        int stride = 1;
        if (j < nk) {
          if (kj < L) {
            const int pid = min(max(bt[kj / kPage], 0), num_pages - 1);
            src = vcl + (static_cast<size_t>(pid) * Hkv + kvh) * page_elems + kj % kPage;
            stride = kPage;
          } else {
            src = v + ((lb * W + slot_of(kj - L)) * Hkv + kvh) * D;
          }
        }
#pragma unroll
        for (int i = 0; i < kF32MaxD / kWave; ++i) {
          const int d = lane + i * kWave;
          vv[u][i] = (src != nullptr && d < D) ? src[d * stride] : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < kPvBatch; ++u) {
        if (j0 + u >= nk) break;
#pragma unroll
        for (int i = 0; i < kF32MaxD / kWave; ++i)
          if (lane + i * kWave < D) o[i] += pj[u] * vv[u][i];
      }
    }
  }
  const float inv = 1.f / l;
  float* orow = out + ((lb * W + p) * Hq + h) * D;
#pragma unroll
  for (int i = 0; i < kF32MaxD / kWave; ++i) {
    const int d = lane + i * kWave;
    if (d < D) orow[d] = o[i] * inv;
  }
}

// ---- launch planning -------------------------------------------------------
struct AttnPlan {
  int cols;   // work units per (layer, kv head)
  int parts;  // workgroups per work unit (row parts)
  int part_rows;
  bool split;
  int min_pages;
  int waves;  // wavefronts per workgroup: 4 (one 16-row tile each), or 8 for wide groups
  bool wide;  // 129..256 rows: k_window_attn_wide, all rows in one workgroup (32-row tiles)
  size_t ws_o_bytes, ws_ml_bytes, ws_plan_bytes;
};

static AttnPlan plan_bf16(int n_layers, int B, int W, int Hq, int Hkv, int max_prefix_len) {
  AttnPlan pl{};
  const int g = Hq / Hkv;
  const int M = W * g;
  const int tiles = ceil_div(M, 16);
  // Up to 128 rows: 16-row tiles, one 4-wave workgroup per 4 tiles of the
  // work unit (row parts on one XCD for more than 64 rows; larger workgroups
  // of 16-row tiles measured slower: for the dual-stream prediction blocks
  // 2.36 / 2.37 ms with one 8-wave workgroup (32-key blocks) or two (64-key
  // blocks) against 2.18 / 2.22 ms, 3.13 ms with one 16-wave workgroup).
  // 129..256 rows: one 8-wave workgroup of 32-row tiles takes the whole group
  // (k_window_attn_wide), one workgroup per CU.
  pl.wide = M > 128 && M <= 256;
  pl.waves = pl.wide ? 8 : 4;
  pl.parts = pl.wide ? 1 : ceil_div(tiles, 4);
  pl.part_rows = pl.wide ? M : ceil_div(tiles, pl.parts) * 16;
  const long long groups = 1LL * n_layers * B * Hkv;
  const long long columns = 1LL * n_layers * Hkv;
  // aim for one full round of workgroups (every CU holding as many as its
  // registers allow) but keep >= 6 pages per split (bs1, L = 2048: 8 pages
  // per split took 21.2 us per chained step, 6 pages 20.7, 4 pages 22.8 as
  // the merge of the split partials grows);
  // how the column's workgroups are shared out follows the live prefix
  // lengths on the device (find_split)
  const int wg_per_cu = pl.wide ? 1 : Ring<4>::kWgPerCu;
  const long long target = 1LL * kNumCUs * wg_per_cu / pl.parts;  // work units per round
  pl.min_pages = 6;
  const int npages = ceil_div(max(max_prefix_len, 1), kPage);
  pl.cols = B;
  pl.split = false;
  if (groups < target) {
    long long S = (target + columns - 1) / columns;
    S = std::min(S, 1LL * B * max(1, npages / pl.min_pages));
    if (S > B) {
      pl.cols = static_cast<int>(S);
      pl.split = true;
    }
  }
  if (pl.split) {
    const size_t slots = static_cast<size_t>(columns) * pl.cols;
    pl.ws_o_bytes = slots * M * kHeadDim * sizeof(float);
    pl.ws_ml_bytes = slots * M * 2 * sizeof(float);
    pl.ws_plan_bytes = static_cast<size_t>(groups) * sizeof(int2);
  }
  return pl;
}

// The merge of a split launch: its partials and plan in the workspace
// (layout of plan_bf16), the output rows it writes.
static CombineArgs combine_of(const AttnPlan& pl, const AttnArgs& a, long long groups) {
  CombineArgs c{};
  c.ws_o = a.ws_o;
  c.ws_ml = a.ws_ml;
  c.ws_plan = a.ws_plan;
  c.out = a.out;
  c.n_groups = static_cast<int>(groups);
  c.M = a.M;
  c.W = a.W;
  c.Hq = a.Hq;
  c.Hkv = a.Hkv;
  c.g = a.g;
  c.cols = pl.cols;
  c.n_slots = a.units;
  c.threads = pl.split ? groups * a.M * (kHeadDim / 4) : 0;
  return c;
}

}  // namespace wedlm

using namespace wedlm;

static int validate_attn(int dtype, int n_layers, int B, int W, int Hq, int Hkv, int D,
                         int page_size, int max_prefix_len) {
  if (!valid_dtype(dtype)) return WEDLM_ERR_UNSUPPORTED;
  if (n_layers <= 0 || B <= 0 || W <= 0 || W > WEDLM_MAX_WINDOW || Hq <= 0 || Hkv <= 0 || D <= 0)
    return WEDLM_ERR_INVALID;
  if (Hq % Hkv != 0 || max_prefix_len < 0) return WEDLM_ERR_INVALID;
  // keeps every launch-plan product (layers x sequences x heads x rows) in range
  if (n_layers > kMaxShapeDim || B > kMaxShapeDim || Hq > kMaxShapeDim) return WEDLM_ERR_UNSUPPORTED;
  if (page_size != kPage) return WEDLM_ERR_UNSUPPORTED;
  if (dtype == WEDLM_BF16) {
    if (D != kHeadDim) return WEDLM_ERR_UNSUPPORTED;
    if (W * (Hq / Hkv) > kMaxRows) return WEDLM_ERR_UNSUPPORTED;
  } else {
    if (D % 4 != 0 || D > kF32MaxD) return WEDLM_ERR_UNSUPPORTED;
  }
  return WEDLM_OK;
}

extern "C" size_t wedlm_window_attn_workspace_size(int dtype, int n_layers, int B, int W, int Hq,
                                                   int Hkv, int D, int page_size,
                                                   int max_prefix_len) {
  if (validate_attn(dtype, n_layers, B, W, Hq, Hkv, D, page_size, max_prefix_len) != WEDLM_OK)
    return 0;
  if (dtype != WEDLM_BF16) return 0;
  const AttnPlan pl = plan_bf16(n_layers, B, W, Hq, Hkv, max_prefix_len);
  return pl.ws_o_bytes + pl.ws_ml_bytes + pl.ws_plan_bytes;
}

// Shared by both entry points; `rope` selects the fused-RoPE kernels (q, k, v
// in slot order before RoPE, perm / pos / theta used), else q, k, v are the
// rotated physical-order rows and perm / pos / theta are ignored.
static int launch_attn(bool rope, int dtype, int n_layers, int B, int W, int Hq, int Hkv, int D,
                       int page_size, int num_pages, int max_pages, int max_prefix_len, float scale,
                       double theta, const void* q, const void* k, const void* v,
                       const int32_t* perm, const int32_t* pos, const void* k_cache,
                       const void* v_cache, const int32_t* block_table, const int32_t* prefix_len,
                       const int32_t* commit_run, void* out_phys, void* workspace,
                       size_t workspace_bytes, int flags, void* stream, int V = 0,
                       const void* logits = nullptr, void* ent_workspace = nullptr,
                       size_t ent_workspace_bytes = 0) {
  int st = validate_attn(dtype, n_layers, B, W, Hq, Hkv, D, page_size, max_prefix_len);
  if (st != WEDLM_OK) return st;
  if ((flags & ~(WEDLM_ATTN_SHARED_PAGES | WEDLM_ATTN_DEFER_COMBINE)) != 0) return WEDLM_ERR_INVALID;
  if (num_pages <= 0 || max_pages <= 0 || static_cast<long long>(max_pages) * page_size <
                                               static_cast<long long>(max_prefix_len))
    return WEDLM_ERR_INVALID;
  if (!q || !k || !v || !k_cache || !v_cache || !block_table || !prefix_len || !out_phys)
    return WEDLM_ERR_INVALID;
  if (rope && (!perm || !pos || !(theta > 0.0) || D % 2 != 0)) return WEDLM_ERR_INVALID;
  // the fused f32 kernel rotates window keys four dimension pairs at a time
  // (float4 halves), as the f32 commit does
  if (rope && dtype == WEDLM_F32 && D % 8 != 0) return WEDLM_ERR_UNSUPPORTED;
  if (!(scale > 0.f)) return WEDLM_ERR_INVALID;
  hipStream_t s = as_stream(stream);
  const long long cache_layer_stride = 1LL * num_pages * Hkv * D * page_size;
  const float scale_log2 = scale * kLog2e;
  // rotation frequencies theta^(-2j/D), formed once on the host in double
  double omega[kF32MaxD / 2] = {};
  if (rope)
    for (int j = 0; j < D / 2; ++j) omega[j] = std::pow(theta, -2.0 * j / D);
  if (dtype == WEDLM_F32) {
    const long long attn_blocks = 1LL * n_layers * B * Hq * W;
    // the committed rows are appended by blocks of the same launch
    const long long blocks = attn_blocks + (rope && commit_run ? 1LL * n_layers * B * Hkv : 0);
    if (blocks > 0x7fffffffLL) return WEDLM_ERR_UNSUPPORTED;
    RopeF32 rp{};
    rp.perm = perm;
    rp.pos = pos;
    for (int j = 0; j < kF32MaxD / 2; ++j) rp.omega[j] = omega[j];
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(blocks)), dim3(kWave), 0, s,
                         static_cast<const float*>(q), static_cast<const float*>(k),
                         static_cast<const float*>(v), static_cast<const float*>(k_cache),
                         static_cast<const float*>(v_cache), block_table, prefix_len,
                         static_cast<float*>(out_phys), B, W, Hq, Hkv, D, num_pages, max_pages,
                         max_prefix_len, cache_layer_stride, scale_log2, rp, attn_blocks,
                         commit_run, static_cast<float*>(const_cast<void*>(k_cache)),
                         static_cast<float*>(const_cast<void*>(v_cache)));
    };
    const bool small = D <= kWave;
    if (rope)
      small ? go(k_window_attn_f32<true, true>) : go(k_window_attn_f32<true, false>);
    else
      small ? go(k_window_attn_f32<false, true>) : go(k_window_attn_f32<false, false>);
    return launch_status();
  }
  const AttnPlan pl = plan_bf16(n_layers, B, W, Hq, Hkv, max_prefix_len);
  const size_t need = pl.ws_o_bytes + pl.ws_ml_bytes + pl.ws_plan_bytes;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return WEDLM_ERR_WORKSPACE;
  AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.kc = static_cast<const uint16_t*>(k_cache);
  a.vc = static_cast<const uint16_t*>(v_cache);
  a.block_table = block_table;
  a.prefix_len = prefix_len;
  a.out = static_cast<uint16_t*>(out_phys);
  a.ws_o = need ? static_cast<float*>(workspace) : nullptr;
  a.ws_ml = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.ws_o_bytes) : nullptr;
  a.ws_plan = need ? reinterpret_cast<int2*>(static_cast<char*>(workspace) + pl.ws_o_bytes +
                                             pl.ws_ml_bytes)
                   : nullptr;
  a.B = B;
  a.W = W;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.g = Hq / Hkv;
  a.M = W * a.g;
  a.num_pages = num_pages;
  a.max_pages = max_pages;
  a.max_prefix_len = max_prefix_len;
  a.cols = pl.cols;
  a.parts = pl.parts;
  a.part_rows = pl.part_rows;
  a.units = 1LL * n_layers * Hkv * pl.cols;
  a.split = pl.split ? 1 : 0;
  a.min_pages = pl.min_pages;
  a.cache_layer_stride = cache_layer_stride;
  a.scale_log2 = scale_log2;
  a.perm = perm;
  a.pos = pos;
  for (int j = 0; j < kHeadDim / 2; ++j) a.omega[j] = omega[j];
  a.commit_run = commit_run;
  a.kc_w = commit_run ? static_cast<uint16_t*>(const_cast<void*>(k_cache)) : nullptr;
  a.vc_w = commit_run ? static_cast<uint16_t*>(const_cast<void*>(v_cache)) : nullptr;
  const long long groups = 1LL * n_layers * B * Hkv;
  const long long attn_blocks =
      pl.parts == 1 ? a.units : (a.units + kNumXcds - 1) / kNumXcds * kNumXcds * pl.parts;
  a.attn_blocks = attn_blocks;
  a.ent_logits = static_cast<const uint16_t*>(logits);
  a.ent_part = static_cast<EntPartial*>(ent_workspace);
  a.ent_V = 0;
  a.ent_chunk_elems = 0;
  a.ent_chunks = 1;
  a.ent_vec = 0;
  long long ent_blocks = 0;
  if (logits != nullptr) {
    EntPlan ep = plan_entropy(dtype, B, W, V);
    if (reinterpret_cast<uintptr_t>(logits) % 16 != 0) ep.vec = false;
    a.ent_V = V;
    a.ent_chunk_elems = ep.chunk_elems;
    a.ent_chunks = ep.n_chunks;
    a.ent_vec = ep.vec ? 1 : 0;
    ent_blocks = 1LL * B * W * ep.n_chunks;
  }
  // Pages that several rows share are read more than once per launch: then
  // the DMA keeps the default cache policy, otherwise it streams (kNt).
  const bool nt = (flags & WEDLM_ATTN_SHARED_PAGES) == 0;
  if (pl.wide) {
    // one workgroup per CU: the entropy chunk blocks (small, many per CU)
    // would inherit its LDS and run one per CU, so the chunk pass is a launch
    // of its own (the same chunk function, bitwise the same partials)
    if (a.units > 0x7fffffffLL) return WEDLM_ERR_UNSUPPORTED;
    a.attn_blocks = a.units;
    const dim3 wgrid(static_cast<unsigned>(a.units));
    auto gw = [&](auto kernel) { hipLaunchKernelGGL(kernel, wgrid, dim3(kTileThreads), 0, s, a); };
    if (rope) {
      if (nt) gw(k_window_attn_wide<true, true>); else gw(k_window_attn_wide<true, false>);
    } else {
      if (nt) gw(k_window_attn_wide<false, true>); else gw(k_window_attn_wide<false, false>);
    }
    st = launch_status();
    if (st == WEDLM_OK && logits != nullptr) {
      EntPlan ep = plan_entropy(dtype, B, W, V);
      if (reinterpret_cast<uintptr_t>(logits) % 16 != 0) ep.vec = false;
      launch_entropy_partials(dtype, B, W, V, logits, ep, static_cast<EntPartial*>(ent_workspace),
                              s);
      st = launch_status();
    }
  } else {
  const long long blocks = attn_blocks + ent_blocks;
  if (blocks > 0x7fffffffLL) return WEDLM_ERR_UNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(blocks));
  auto go = [&](auto kernel, int waves) {
    hipLaunchKernelGGL(kernel, grid, dim3(kWave * waves), 0, s, a);
  };
  auto pick = [&](auto k_nt, auto k_cached, int waves) { nt ? go(k_nt, waves) : go(k_cached, waves); };
  rope ? pick(k_window_attn_bf16<4, true, true>, k_window_attn_bf16<4, true, false>, pl.waves)
       : pick(k_window_attn_bf16<4, false, true>, k_window_attn_bf16<4, false, false>, pl.waves);
  st = launch_status();
  }
  // a deferred merge is launched by the step tail (wedlm_select_commit_reorder_combine)
  if (st != WEDLM_OK || !pl.split || (flags & WEDLM_ATTN_DEFER_COMBINE)) return st;
  CombineArgs c = combine_of(pl, a, groups);
  hipLaunchKernelGGL(k_window_attn_combine, dim3(static_cast<unsigned>((c.threads + 255) / 256)),
                     dim3(256), 0, s, c);
  return launch_status();
}

int wedlm::attn_combine_args(int dtype, int n_layers, int B, int W, int Hq, int Hkv, int D,
                             int page_size, int max_prefix_len, const void* workspace,
                             size_t workspace_bytes, void* out, CombineArgs* c) {
  *c = CombineArgs{};
  const int st = validate_attn(dtype, n_layers, B, W, Hq, Hkv, D, page_size, max_prefix_len);
  if (st != WEDLM_OK) return st;
  if (dtype != WEDLM_BF16) return WEDLM_OK;  // the f32 path never splits
  const AttnPlan pl = plan_bf16(n_layers, B, W, Hq, Hkv, max_prefix_len);
  if (!pl.split) return WEDLM_OK;
  const size_t need = pl.ws_o_bytes + pl.ws_ml_bytes + pl.ws_plan_bytes;
  if (workspace == nullptr || workspace_bytes < need) return WEDLM_ERR_WORKSPACE;
  if (out == nullptr) return WEDLM_ERR_INVALID;
  AttnArgs a{};
  char* ws = static_cast<char*>(const_cast<void*>(workspace));
  a.ws_o = reinterpret_cast<float*>(ws);
  a.ws_ml = reinterpret_cast<float*>(ws + pl.ws_o_bytes);
  a.ws_plan = reinterpret_cast<int2*>(ws + pl.ws_o_bytes + pl.ws_ml_bytes);
  a.out = static_cast<uint16_t*>(out);
  a.W = W;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.g = Hq / Hkv;
  a.M = W * a.g;
  a.units = 1LL * n_layers * Hkv * pl.cols;
  *c = combine_of(pl, a, 1LL * n_layers * B * Hkv);
  return WEDLM_OK;
}

extern "C" int wedlm_window_attn(int dtype, int n_layers, int B, int W, int Hq, int Hkv, int D,
                                 int page_size, int num_pages, int max_pages, int max_prefix_len,
                                 float scale, const void* q_phys, const void* k_phys,
                                 const void* v_phys, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* prefix_len,
                                 void* out_phys, void* workspace, size_t workspace_bytes,
                                 int flags, void* stream) {
  return launch_attn(false, dtype, n_layers, B, W, Hq, Hkv, D, page_size, num_pages, max_pages,
                     max_prefix_len, scale, 0.0, q_phys, k_phys, v_phys, nullptr, nullptr, k_cache,
                     v_cache, block_table, prefix_len, nullptr, out_phys, workspace,
                     workspace_bytes, flags, stream);
}

extern "C" int wedlm_window_attn_rope_entropy(
    int dtype, int n_layers, int B, int W, int Hq, int Hkv, int D, int page_size, int num_pages,
    int max_pages, int max_prefix_len, float scale, double theta, const void* q, const void* k,
    const void* v, const int32_t* perm, const int32_t* pos, void* k_cache, void* v_cache,
    const int32_t* block_table, const int32_t* prefix_len, const int32_t* commit_run,
    void* out_phys, void* workspace, size_t workspace_bytes, int flags, int V,
    const void* logits, void* ent_workspace, size_t ent_workspace_bytes, void* stream) {
  if (dtype != WEDLM_BF16) return WEDLM_ERR_UNSUPPORTED;  // the chunk blocks read bf16
  if (V <= 0 || logits == nullptr) return WEDLM_ERR_INVALID;
  if (B > 0 && W > 0 && 1LL * B * W > 65535) return WEDLM_ERR_UNSUPPORTED;
  if (B > 0 && W > 0 && W <= WEDLM_MAX_WINDOW) {
    const EntPlan ep = plan_entropy(dtype, B, W, V);
    const size_t need = static_cast<size_t>(B) * W * ep.n_chunks * sizeof(EntPartial);
    if (ent_workspace == nullptr || ent_workspace_bytes < need) return WEDLM_ERR_WORKSPACE;
  }
  return launch_attn(true, dtype, n_layers, B, W, Hq, Hkv, D, page_size, num_pages, max_pages,
                     max_prefix_len, scale, theta, q, k, v, perm, pos, k_cache, v_cache,
                     block_table, prefix_len, commit_run, out_phys, workspace, workspace_bytes,
                     flags, stream, V, logits, ent_workspace, ent_workspace_bytes);
}

extern "C" int wedlm_window_attn_rope(int dtype, int n_layers, int B, int W, int Hq, int Hkv,
                                      int D, int page_size, int num_pages, int max_pages,
                                      int max_prefix_len, float scale, double theta, const void* q,
                                      const void* k, const void* v, const int32_t* perm,
                                      const int32_t* pos, void* k_cache, void* v_cache,
                                      const int32_t* block_table, const int32_t* prefix_len,
                                      const int32_t* commit_run, void* out_phys, void* workspace,
                                      size_t workspace_bytes, int flags, void* stream) {
  return launch_attn(true, dtype, n_layers, B, W, Hq, Hkv, D, page_size, num_pages, max_pages,
                     max_prefix_len, scale, theta, q, k, v, perm, pos, k_cache, v_cache,
                     block_table, prefix_len, commit_run, out_phys, workspace, workspace_bytes,
                     flags, stream);
}
