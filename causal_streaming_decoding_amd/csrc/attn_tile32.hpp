// 32-row MFMA tiles of the attention kernels that give every wavefront 32
// query rows and stream keys in 64-key tiles of four 16-key pages: the block
// attention (block_attn.hip, the dual-stream forward) and the wide-group
// window attention (attn.hip, groups of more than 128 query rows).
//
// Per 32 keys and wavefront:
//   S^T (32 keys x 32 rows)  = K . Q^T   v_mfma_f32_32x32x16_bf16, 8 K-steps of 16 dims
//   O^T (32 dims x 32 rows) += V^T . P^T  v_mfma_f32_32x32x16_f16, per page and 32-dim tile
// The score accumulator leaves 16 keys of one query row in each lane; with
// the K rows loaded in a permuted order (kperm) they are 8 consecutive keys
// of each page per lane half, the B operand of the PV product as they stand,
// against one 16-byte run of V^T per lane read from a bank-swizzled V page
// (vslot). A row's max and sum take one swap of the two lane halves. The
// online softmax is the window kernel's (scores in log2 units, the reference
// max raised lazily).
//
// The PV product runs in fp16: each tile's values are converted in LDS once
// (bf16 -> fp16 is exact for magnitudes in [2^-14, 65504]), and each
// probability p in [0, 1] is rounded once to fp16 (relative error <= 2^-11),
// the row sum l being accumulated from the fp32 probabilities. The output
// then differs from the exact softmax average by at most 2^-11 max|v| (the
// largest value magnitude the row attends to): 2e-3 for |v| <= 4. The 16-row
// window kernel carries 16 bits of p as a bf16 hi + lo pair instead, which
// costs a second PV MFMA per page and three VALU operations per score; a
// single bf16 part (2^-9) would not meet that bound.
//
// Workgroups of 8 wavefronts (512 threads) move a tile with one DMA
// instruction per page and wavefront: wavefronts 0-3 the K part, 4-7 the V
// part, whose 16-byte vectors the lane addresses place in the vslot order.
#pragma once

#include "attn_device.hpp"
#include "common.hpp"

namespace wedlm {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f16x8 as_f16x8(u32x4 u) { return __builtin_bit_cast(f16x8, u); }

// Two floats to fp16, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), f16x2));
}

// A 32-bit word of two bf16 values as two fp16 values: exact for magnitudes
// in [2^-14, 65504] (fp16 holds every 8-bit significand there); below, fp16
// subnormals keep it within 2^-25.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) { return pack_f16x2(bf16_lo(w), bf16_hi(w)); }

constexpr int kTileKeys = 64;
constexpr int kTilePages = kTileKeys / kPage;  // 4
constexpr int kTileThreads = 512;              // 8 wavefronts
constexpr int kTileDma = kTilePages * kPageVecs / kTileThreads;  // DMA instructions per thread per tile
static_assert(kTileDma == kTilePages, "one DMA instruction per page of a tile and wavefront");

struct Tile {
  Stage pg[kTilePages];
};

struct RowState32 {
  f32x16 o[4];  // O^T per 32-dim tile: register r of lane l holds dim 32*dt + 8*(r/4) + 4*(l/32) + r%4 of row l % 32
  float m;      // reference max of scaled scores (log2 units), equal in lanes l and l ^ 32
  float l;      // this lane's share of the row sum (its 16 keys of each 32-key block)
};

// Wait states after an 8-pass MFMA before a VALU reads its result in a later
// basic block: the compiler places them inside one block only (the masking
// branch below follows the score MFMAs). The tied operands pin the order.
__device__ __forceinline__ void mfma32_guard(f32x16& x) { asm volatile("s_nop 7\n\ts_nop 7" : "+v"(x)); }

// max / sum over the two lanes holding one row (l and l ^ 32): the same
// operands in the same order in both
__device__ __forceinline__ float half_max(float x) {
  float a = x, b = x;
  row_swap32(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float half_sum(float x) {
  float a = x, b = x;
  row_swap32(a, b);
  return a + b;
}

// Key order of the score product: A row i of a 32-key block holds key
// kperm(i), i with bits 2 and 3 swapped. The accumulator's register r of lane
// half h then holds key 16 (r / 8) + 8 h + r % 8: the B operand of the PV
// K-step over page r / 8 is 8 consecutive keys per lane half, matched by one
// 16-byte run of V^T.
__device__ __forceinline__ int kperm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// 16-byte LDS slot of value dimension d, keys 8 hv .. 8 hv + 7, in a V page:
// the two halves of the dimensions with bit 3 set trade places, so that the
// 16 lanes of one read (16 consecutive dimensions, one half) fall in 16
// different bank groups. The cache page's vector 2 d + hv lands in slot
// vslot(d, hv) = its index with bit 0 flipped when bit 4 is set.
__device__ __forceinline__ int vslot(int d, int hv) { return 2 * d + (hv ^ ((d >> 3) & 1)); }

// One block of 32 keys: keys 0..15 are page pa, 16..31 page pb. Key kk of
// page A is visible to this lane's row iff loa <= kk < hia (page B: lob, hib).
// The values of keys no row may see hold zeros (cache positions not written
// yet may hold any bits, and 0 * NaN is NaN): the caller clears them.
__device__ __forceinline__ void attend32(RowState32& st, const bf16x8 (&qr)[8], const Stage& pa,
                                         const Stage& pb, int lane, int loa, int hia, int lob,
                                         int hib, float scale_log2) {
  const int li = lane & 31, h = lane >> 5;
  // A operand of the scores: lane l reads key li (page li / 16) at dims
  // 16 s + 8 h .. +7 (slice 2 s + h of the K page)
  const uint16_t* kb = (li < kPage ? pa.k : pb.k) + (h * kPage + (kperm(li) & 15)) * 8;
  f32x16 sc;
#pragma unroll
  for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const u32x4 kk = *reinterpret_cast<const u32x4*>(kb + s * 2 * kPage * 8);
    sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kk), qr[s], sc, 0, 0, 0);
  }
  mfma32_guard(sc);
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = sc[r];
  if (__ballot(loa > 0 || hia < kPage || lob > 0 || hib < kPage)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 16 * (r >> 3) + 8 * h + (r & 7);
      const bool vis = key < kPage ? (key >= loa && key < hia)
                                   : (key - kPage >= lob && key - kPage < hib);
      if (!vis) x[r] = -INFINITY;
    }
  }
  float m16 = x[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) m16 = fmaxf(m16, x[r]);
  const float mc = half_max(m16) * scale_log2;  // -inf if no visible key
  const bool raise = mc > st.m + kRescaleLog2;
  if (__ballot(raise)) {
    const float m_new = raise ? mc : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);  // 0 while st.m = -inf
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st.o[dt] *= alpha;
    st.m = m_new;
  }
  const float base = st.m == -INFINITY ? 0.f : st.m;
  float p[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(x[r], scale_log2, -base));
  st.l += (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]))) +
          (((p[8] + p[9]) + (p[10] + p[11])) + ((p[12] + p[13]) + (p[14] + p[15])));
  // B operands of the PV product (fp16): K-step kk (page kk) takes registers
  // 8kk .. 8kk+7
  u32x4 bp[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int w = 0; w < 4; ++w) bp[kk][w] = pack_f16x2(p[8 * kk + 2 * w], p[8 * kk + 2 * w + 1]);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const Stage& sg = kk == 0 ? pa : pb;
    // lane (dim li of the tile, half h): keys 8h .. 8h+7, one 16-byte read
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const u32x4 va = *reinterpret_cast<const u32x4*>(sg.v + vslot(dt * 32 + li, h) * 8);
      st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(va), as_f16x8(bp[kk]), st.o[dt],
                                                        0, 0, 0);
    }
  }
}

// rope_pair with the cosines and sines of the row's position taken from a
// table: cs[f] = (cos, sin) of frequency f at that position.
__device__ __forceinline__ void rope_pair_tab(u32x4& lo, u32x4& hi, const f32x2* cs, int j0) {
  u32x4 ylo, yhi;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f32x2 t0 = cs[j0 + 2 * w], t1 = cs[j0 + 2 * w + 1];
    const float a0 = bf16_lo(lo[w]), a1 = bf16_hi(lo[w]);
    const float h0 = bf16_lo(hi[w]), h1 = bf16_hi(hi[w]);
    ylo[w] = pack_bf16x2(a0 * t0[0] - h0 * t0[1], a1 * t1[0] - h1 * t1[1]);
    yhi[w] = pack_bf16x2(h0 * t0[0] + a0 * t0[1], h1 * t1[0] + a1 * t1[1]);
  }
  lo = ylo;
  hi = yhi;
}

// DMA of one 64-key tile of kv head kvh (pages id[0..3], clamped to the pool)
// into dst by a 512-thread workgroup: instruction i of wavefront w moves
// vectors 64 w .. 64 w + 63 of page i (K for w < 4, V for w >= 4; the V
// vectors through the vslot swizzle). kNt: the non-temporal hint.
template <bool kNt>
__device__ __forceinline__ void tile_dma(Tile& dst, const int (&id)[kTilePages],
                                         const uint16_t* kc, const uint16_t* vc, int Hkv, int kvh,
                                         int num_pages, int wave, int lane) {
  constexpr size_t kPageElems = static_cast<size_t>(kHeadDim) * kPage;
  const int v0 = wave * kWave;  // this wavefront's first vector of a page (wave-uniform)
  const uint32_t vlane =
      16u * static_cast<uint32_t>(v0 < 256 ? lane : (lane ^ ((lane >> 4) & 1)));
#pragma unroll
  for (int i = 0; i < kTilePages; ++i) {
    const int pid = __builtin_amdgcn_readfirstlane(min(max(id[i], 0), num_pages - 1));
    const size_t off = (static_cast<size_t>(pid) * Hkv + kvh) * kPageElems;
    const uint16_t* part = (v0 < 256 ? kc : vc) + off + (v0 % 256) * 8;
    const uint64_t sbase =
        (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(
             static_cast<uint32_t>(reinterpret_cast<uint64_t>(part) >> 32)))
         << 32) |
        static_cast<uint32_t>(
            __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uint64_t>(part))));
    const uint32_t lds = static_cast<uint32_t>(
        reinterpret_cast<size_t>((__attribute__((address_space(3))) char*)(&dst.pg[i])));
    lds_dma_16<kNt>(sbase, vlane, __builtin_amdgcn_readfirstlane(lds + v0 * 16));
  }
}

// The values of a landed tile to fp16 in place (2 of its 1024 16-byte V
// vectors per thread of 512); the keys at or past nv (positions no row sees,
// which may not be written) are cleared. The caller synchronises before and
// after.
__device__ __forceinline__ void tile_v_to_f16(Tile& tl, int tid, int nv) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int u = c * kTileThreads + tid;
    const int slot = u & 255;
    u32x4* vp = reinterpret_cast<u32x4*>(&tl.pg[u >> 8].v[slot * 8]);
    u32x4 w = *vp;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = bf16x2_to_f16x2(w[e]);
    if (nv < kTileKeys) {
      // vector slot holds keys 8 hv .. 8 hv + 7 of page u >> 8 (vslot inverted)
      const int key0 = (u >> 8) * kPage + 8 * ((slot & 1) ^ ((slot >> 4) & 1));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] &= (key0 + 2 * e < nv ? 0x0000ffffu : 0u) | (key0 + 2 * e + 1 < nv ? 0xffff0000u : 0u);
    }
    *vp = w;
  }
}

// Wait until at most `behind` (<= 1) later tiles' DMAs are in flight for
// this thread, then synchronise the workgroup.
__device__ __forceinline__ void tile_wait_barrier(int behind) {
  if (behind >= 1)
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(kTileDma) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace wedlm
