// Device helpers shared by the window attention (attn.hip) and the block
// attention (block_attn.hip): bf16 vector types, the cache page layout, the
// global -> LDS page DMA, block-table reads through the scalar cache, the
// gfx950 row-swap permutes and the RoPE rotation of a row slice pair.
#pragma once

#include "common.hpp"

namespace wedlm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;
constexpr int kPage = 16;
constexpr int kMaxRows = 256;       // M = W*g rows: at most four 4-wave row parts
constexpr int kPageVecs = 512;      // 16-byte vectors of one page of one kv head (K 4 KB + V 4 KB)
constexpr int kPartElems = 2048;    // bf16 elements of one 4 KB page part
constexpr int kNumCUs = 256;        // MI355X compute units
constexpr int kNumXcds = 8;         // MI355X: 8 XCDs of 32 CUs, workgroups dealt round-robin

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// One stage of the ring: one page of one kv head in the cache layout.
struct Stage {
  uint16_t k[kPartElems];  // [D/8][16 keys][8]
  uint16_t v[kPartElems];  // [D][16 keys]
};

// Swaps between lane groups of two registers (gfx950): v_permlane16_swap
// exchanges the odd 16-lane rows of one register with the even rows of
// another, v_permlane32_swap the upper 32 lanes of one with the lower 32 of
// another. Issued from asm because the compiler's builtins treat the two
// results as one value; the s_nop gives the wait states between a VALU write
// and a permute read.
__device__ __forceinline__ void row_swap16(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void row_swap32(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// Asynchronous page staging: global -> LDS DMA (global_load_lds_dwordx4).
// Each instruction moves 64 lanes x 16 B = 1 KB: lane l's 16 bytes land at
// M0 + 16 l in LDS. A stage is 512 vectors (K then V of one page); wavefront w
// issues instructions for vectors (i*NW + w)*64 .. +63 (two each for 4 waves,
// one each for 8).
// The DMA is issued from inline asm so that the compiler does not add its own
// conservative vmcnt waits before every LDS read of the ring; the waits are
// explicit (stage_wait_barrier) and counted per thread in issue order.
// M0 is a reserved register: it is saved and restored around the DMA.
// kNt: the loads carry the non-temporal hint (nt). When every page is read
// once per launch (each sequence owns its pages, as in decoding), the pages
// should not displace other lines on their way through the caches: on the
// 36-layer streaming shape this took the launch from 5.1 to 5.5 TB/s (the
// scope bits sc0 / sc1 on top of it changed nothing). When block-table rows
// share pages (the dual-stream forward: every block of a sample reads the
// sample's memory rows), the re-reads hit in the caches only without the
// hint (2.9 against 2.3 ms for the 16-key-block forward).
template <bool kNt>
__device__ __forceinline__ void lds_dma_16(uint64_t sbase, uint32_t voff, uint32_t lds_byte_addr) {
  // scalar base + per-lane 32-bit offset: no 64-bit address arithmetic per
  // lane and page
  uint32_t saved;
  if constexpr (kNt)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "global_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds_byte_addr)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds_byte_addr)
        : "memory");
}

// Workgroup barrier for LDS reuse only: this thread's LDS accesses have
// completed; its global memory operations (DMAs, stores) may still be in
// flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A wave-uniform block-table entry through the scalar cache (read only).
// Scalar loads count against lgkmcnt, not vmcnt, so reading the table never
// waits for the DMAs in flight.
__device__ __forceinline__ int load_page_id(const int32_t* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint64_t su =
      (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32))) << 32) |
      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u)));
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(su) : "memory");
  return v;
}

// Two block-table entries with one wait (both scalar loads in flight together).
__device__ __forceinline__ void load_page_ids2(const int32_t* p0, const int32_t* p1, int& v0,
                                               int& v1) {
  auto su = [](const int32_t* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    return (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32)))
            << 32) |
           static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u)));
  };
  asm volatile(
      "s_load_dword %0, %2, 0x0\n\t"
      "s_load_dword %1, %3, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(v0), "=&s"(v1)
      : "s"(su(p0)), "s"(su(p1))
      : "memory");
}

// The block-table entries of logical pages pg .. pg+3 (a 64-key tile) of a
// table row holding max_pages entries, each clamped into the row: one 16-byte
// scalar load when the four lie inside the row, else four clamped loads; one
// wait either way. Scalar loads count against lgkmcnt, not vmcnt.
typedef uint32_t su32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load_page_ids4(const int32_t* bt, int pg, int max_pages,
                                               int (&id)[4]) {
  auto su = [](const int32_t* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    return (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32)))
            << 32) |
           static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u)));
  };
  pg = __builtin_amdgcn_readfirstlane(pg);
  if (pg >= 0 && pg + 3 < max_pages) {
    su32x4 v;
    asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)"
                 : "=s"(v)
                 : "s"(su(bt + pg))
                 : "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) id[i] = static_cast<int>(v[i]);
  } else {
    const int32_t* p0 = bt + min(max(pg, 0), max_pages - 1);
    const int32_t* p1 = bt + min(max(pg + 1, 0), max_pages - 1);
    const int32_t* p2 = bt + min(max(pg + 2, 0), max_pages - 1);
    const int32_t* p3 = bt + min(max(pg + 3, 0), max_pages - 1);
    asm volatile(
        "s_load_dword %0, %4, 0x0\n\t"
        "s_load_dword %1, %5, 0x0\n\t"
        "s_load_dword %2, %6, 0x0\n\t"
        "s_load_dword %3, %7, 0x0\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&s"(id[0]), "=&s"(id[1]), "=&s"(id[2]), "=&s"(id[3])
        : "s"(su(p0)), "s"(su(p1)), "s"(su(p2)), "s"(su(p3))
        : "memory");
  }
}

// Block-table entry of logical page pg of a sequence's table row, the page
// index clamped to the table and the entry to the pool: the id a DMA reads.
__device__ __forceinline__ const int32_t* page_entry(const int32_t* bt, int pg, int max_pages) {
  return bt + __builtin_amdgcn_readfirstlane(min(max(pg, 0), max_pages - 1));
}

// Rotates a 16-byte slice pair of one row by RoPE: lo holds dims j0..j0+7,
// hi dims j0+64..j0+71 (rotate-half pairing, D = 128), position t.
__device__ __forceinline__ void rope_pair(u32x4& lo, u32x4& hi, double t, const double* omega,
                                          int j0) {
  u32x4 ylo, yhi;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float c0, s0, c1, s1;
    rope_cos_sin(t, omega[j0 + 2 * w], c0, s0);
    rope_cos_sin(t, omega[j0 + 2 * w + 1], c1, s1);
    const float a0 = bf16_lo(lo[w]), a1 = bf16_hi(lo[w]);
    const float h0 = bf16_lo(hi[w]), h1 = bf16_hi(hi[w]);
    ylo[w] = pack_bf16x2(a0 * c0 - h0 * s0, a1 * c1 - h1 * s1);
    yhi[w] = pack_bf16x2(h0 * c0 + a0 * s0, h1 * c1 + a1 * s1);
  }
  lo = ylo;
  hi = yhi;
}

}  // namespace wedlm
