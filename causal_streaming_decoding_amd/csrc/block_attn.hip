// Block attention: the windows of a sequence laid end to end over the
// sequence's own paged cache, in workgroups shaped like a prefill.
//
// hyper.ai summary of WeDLM, "Method": training pairs a clean memory stream
// with a masked prediction stream over the same logical positions; the
// prediction stream is cut into blocks that are reordered inside, and a
// block's tokens attend to the memory stream's context before the block and,
// inside the block, causally. Each stream's attention is a batch of windows
// of the window step whose windows are the consecutive W-position blocks of
// one sample: window j of sample s has the prefix 0 .. jW-1 of the sample's
// cache (one block-table row per sample) and attends to its own W keys,
// causally in physical order (the window order perm, the logical positions
// pos). That is what wedlm_window_attn_rope computes for such a batch; the
// window kernel serves each window by itself (at most 64 query rows per pass
// over its prefix, a 16-row tile per wavefront), while here 256 query rows of
// consecutive windows share every key tile read into LDS, and each
// wavefront's 32 rows share every K and V operand it reads.
//
// Workgroup: 8 wavefronts (two per SIMD, one workgroup per CU) and 256 query
// rows: 256 / g consecutive positions x the g query heads of one kv head
// (row r: position r / g, head r % g); wavefront w owns rows 32w .. 32w+31.
// Keys come in tiles of 64 (four 16-key pages, 32 KB of K and V):
//   - own tiles: the windows' own keys, read from the step inputs through
//     the window order and rotated at their logical positions into one LDS
//     tile (the prologue, while the first cache tiles are in flight); a row
//     sees the keys of its own window up to its own physical row;
//   - cache tiles: positions 0 .. jhi*W - 1 (jhi: the last window the
//     workgroup touches), through a 3-stage LDS ring filled by global->LDS
//     DMA, two tiles in flight while one is computed; a row of window j sees
//     the positions below jW. Workgroups are launched longest prefix first.
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
// largest value magnitude the row attends to): 2e-3 for |v| <= 4. The window
// kernel carries 16 bits of p as a bf16 hi + lo pair instead, which costs a
// second PV MFMA per page and three VALU operations per score; a single bf16
// part (2^-9) would not meet that bound.
#include "attn_device.hpp"
#include "common.hpp"

#include <cmath>

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

constexpr int kBlkWaves = 8;
constexpr int kBlkThreads = kBlkWaves * kWave;  // 512
constexpr int kBlkRows = 32 * kBlkWaves;        // query rows per workgroup
constexpr int kTileKeys = 64;
constexpr int kTilePages = kTileKeys / kPage;   // 4
constexpr int kBlkStages = 3;                   // ring tiles (96 KB)
constexpr int kBlkAhead = kBlkStages - 1;       // cache tiles in flight while one is computed
constexpr int kBlkDma = kTilePages * kPageVecs / kBlkThreads;  // DMA instructions per thread per tile
constexpr int kMaxOwn = kBlkRows + WEDLM_MAX_WINDOW;  // own keys of a workgroup, at most
static_assert(kBlkDma == kTilePages, "one DMA instruction per page of a tile and wavefront");

struct Tile {
  Stage pg[kTilePages];
};

struct BlockAttnArgs {
  const uint16_t* q;  // [S*nb][W][Hq][D]: slot order, before RoPE
  const uint16_t* k;  // [S*nb][W][Hkv][D]
  const uint16_t* v;
  const int32_t* perm;  // [S*nb][W]: physical row -> slot
  const int32_t* pos;   // [S*nb][W]: logical position of each physical row
  const uint16_t* kc;   // [num_pages][Hkv][D/8][P][8]
  const uint16_t* vc;   // [num_pages][Hkv][D][P]
  const int32_t* block_table;  // [S][max_pages]
  uint16_t* out;               // [S*nb][W][Hq][D], physical order
  int S, N, W, nb, Hq, Hkv, g;
  int pos_per_wg;  // positions per workgroup: kBlkRows / g
  int n_groups;    // workgroups per (sample, kv head)
  int num_pages, max_pages;
  float scale_log2;
  double omega[kHeadDim / 2];
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

// Wait until at most `behind` (<= 1) later tiles' DMAs are in flight for
// this thread, then synchronise the workgroup.
__device__ __forceinline__ void tile_wait_barrier(int behind) {
  if (behind >= 1)
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(kBlkDma) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
static_assert(kBlkAhead == 2, "tile_wait_barrier covers one tile behind the computed one");

__global__ void __launch_bounds__(kBlkThreads) k_block_attn_bf16(BlockAttnArgs a) {
  __shared__ Tile ring[kBlkStages];
  __shared__ Tile own;
  __shared__ double s_omega[kHeadDim / 2];
  __shared__ int s_perm[kMaxOwn];  // own key i (position own_begin + i): its slot, clamped
  __shared__ int s_pos[kMaxOwn];   // and its logical position

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, h = lane >> 5;

  // longest prefix first: the workgroups of the last positions of every
  // (sample, kv head) come first
  const int sh_count = a.S * a.Hkv;
  const int sh = static_cast<int>(blockIdx.x % sh_count);
  const int grp = a.n_groups - 1 - static_cast<int>(blockIdx.x / sh_count);
  const int s = sh / a.Hkv, kvh = sh % a.Hkv;
  const int R0 = grp * a.pos_per_wg;  // positions R0 .. R_end-1 of sample s
  const int R_end = min(a.N, R0 + a.pos_per_wg);
  const int j_lo = R0 / a.W, j_hi = (R_end - 1) / a.W;
  const int own_begin = j_lo * a.W;    // own keys: positions own_begin .. R_end-1
  const int n_own = R_end - own_begin;  // <= pos_per_wg + W - 1 <= kMaxOwn
  const int n_cache = j_hi * a.W;       // cache positions seen by some row
  const int n_tiles = (n_cache + kTileKeys - 1) / kTileKeys;

  // this lane's query row (rows past the sample's end take the first row's
  // inputs and are never stored)
  const int r = wave * 32 + li;
  const int R = R0 + r / a.g;
  const int hh = r % a.g;
  const bool row_ok = R < R_end;
  const int Rc = row_ok ? R : R0;
  const int j = Rc / a.W, p = Rc % a.W;
  const size_t bwin = static_cast<size_t>(s) * a.nb + j;
  const int lim = j * a.W;  // cache positions below lim are visible to this row

  if (tid < kHeadDim / 2) s_omega[tid] = a.omega[tid];
  for (int i = tid; i < n_own; i += kBlkThreads) {
    const int Rk = own_begin + i;
    const size_t e = (static_cast<size_t>(s) * a.nb + Rk / a.W) * a.W + Rk % a.W;
    s_perm[i] = min(max(a.perm[e], 0), a.W - 1);
    s_pos[i] = a.pos[e];
  }
  __syncthreads();

  // cache tile t -> ring stage t % kBlkStages: instruction i of every
  // wavefront moves 1 KB of page i of the tile (wavefronts 0-3 the K part,
  // 4-7 the V part)
  const int32_t* bt = a.block_table + static_cast<size_t>(s) * a.max_pages;
  constexpr size_t kPageElems = static_cast<size_t>(kHeadDim) * kPage;
  const int v0 = wave * kWave;  // this wavefront's first vector of a page (wave-uniform)
  // source of this lane's 16 bytes: K in order, V through the slot swizzle
  const uint32_t vlane =
      16u * static_cast<uint32_t>(v0 < 256 ? lane : (lane ^ ((lane >> 4) & 1)));
  auto issue_tile = [&](int t) {
    int id[kTilePages];
    load_page_ids2(page_entry(bt, 4 * t, a.max_pages), page_entry(bt, 4 * t + 1, a.max_pages),
                   id[0], id[1]);
    load_page_ids2(page_entry(bt, 4 * t + 2, a.max_pages),
                   page_entry(bt, 4 * t + 3, a.max_pages), id[2], id[3]);
    Tile& dst = ring[t % kBlkStages];
#pragma unroll
    for (int i = 0; i < kTilePages; ++i) {
      const int pid = __builtin_amdgcn_readfirstlane(min(max(id[i], 0), a.num_pages - 1));
      const size_t off = (static_cast<size_t>(pid) * a.Hkv + kvh) * kPageElems;
      const uint16_t* part = (v0 < 256 ? a.kc : a.vc) + off + (v0 % 256) * 8;
      const uint64_t sbase =
          (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(
               static_cast<uint32_t>(reinterpret_cast<uint64_t>(part) >> 32)))
           << 32) |
          static_cast<uint32_t>(
              __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uint64_t>(part))));
      const uint32_t lds = static_cast<uint32_t>(
          reinterpret_cast<size_t>((__attribute__((address_space(3))) char*)(&dst.pg[i])));
      lds_dma_16<false>(sbase, vlane,
                        __builtin_amdgcn_readfirstlane(lds + v0 * 16));
    }
  };
  // The DMAs are issued before the plain loads below: those complete in
  // order after them, so every wait the compiler places for its own loads
  // also covers the DMAs, and the ring's explicit counts start from zero.
  for (int t = 0; t < kBlkAhead && t < n_tiles; ++t) issue_tile(t);

  // RoPE of the query rows and own keys: when the own positions fit one
  // tile (64 positions), their (cos, sin) at every frequency are formed once
  // into ring stage kBlkAhead, which no DMA fills before the ring's first
  // barrier; otherwise each row computes its own.
  static_assert(kBlkAhead < kBlkStages, "the RoPE table needs a ring stage the prologue leaves free");
  const bool tab = n_own <= kTileKeys;  // workgroup-uniform
  f32x2* cs_tab = reinterpret_cast<f32x2*>(&ring[kBlkAhead]);  // [64 positions][64 frequencies]
  static_assert(sizeof(Tile) >= kTileKeys * (kHeadDim / 2) * sizeof(f32x2), "RoPE table size");
  if (tab) {
    for (int e = tid; e < n_own * (kHeadDim / 2); e += kBlkThreads) {
      float c, sn;
      rope_cos_sin(static_cast<double>(s_pos[e >> 6]), s_omega[e & 63], c, sn);
      cs_tab[e] = f32x2{c, sn};
    }
    __syncthreads();
  }

  // query rows: lane half h holds dims 16 s + 8 h .. +7 (B operand of K-step s)
  bf16x8 qr[8];
  {
    const int slot = s_perm[Rc - own_begin];
    const uint16_t* qrow =
        a.q + ((bwin * a.W + slot) * a.Hq + static_cast<size_t>(kvh) * a.g + hh) * kHeadDim;
    u32x4 qv[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qv[ks] = *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * h);
    // dims 16 ks + 8 h + e and 16 (ks + 4) + 8 h + e are a rotate-half pair
    if (tab) {
      const f32x2* cs = cs_tab + (Rc - own_begin) * (kHeadDim / 2);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) rope_pair_tab(qv[ks], qv[ks + 4], cs, 16 * ks + 8 * h);
    } else {
      const double t = static_cast<double>(s_pos[Rc - own_begin]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) rope_pair(qv[ks], qv[ks + 4], t, s_omega, 16 * ks + 8 * h);
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

  // ---- own tiles: keys own_begin + 64 ot .. +63 ------------------------------
  const int n_own_tiles = (n_own + kTileKeys - 1) / kTileKeys;
  for (int ot = 0; ot < n_own_tiles; ++ot) {
    if (ot > 0) __syncthreads();  // every wavefront is done with the previous own tile
    {
      // keys: one (key, slice pair) per thread, rotated at the key's position
      const int kk = tid & 63, sl = tid >> 6;
      const int i = ot * kTileKeys + kk;
      u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
      if (i < n_own) {
        const int Rk = own_begin + i;
        const size_t e = (static_cast<size_t>(s) * a.nb + Rk / a.W) * a.W + s_perm[i];
        const uint16_t* krow = a.k + (e * a.Hkv + kvh) * kHeadDim;
        lo = *reinterpret_cast<const u32x4*>(krow + sl * 8);
        hi = *reinterpret_cast<const u32x4*>(krow + 64 + sl * 8);
        if (tab)
          rope_pair_tab(lo, hi, cs_tab + i * (kHeadDim / 2), sl * 8);
        else
          rope_pair(lo, hi, static_cast<double>(s_pos[i]), s_omega, sl * 8);
      }
      Stage& pg = own.pg[kk >> 4];
      *reinterpret_cast<u32x4*>(&pg.k[(sl * kPage + (kk & 15)) * 8]) = lo;
      *reinterpret_cast<u32x4*>(&pg.k[((sl + 8) * kPage + (kk & 15)) * 8]) = hi;
    }
    // values, transposed to [dim][key]: one (key, 8 dims) per task
    for (int task = tid; task < kTileKeys * 16; task += kBlkThreads) {
      const int kk = task & 63, dv = task >> 6;
      const int i = ot * kTileKeys + kk;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (i < n_own) {
        const int Rk = own_begin + i;
        const size_t e = (static_cast<size_t>(s) * a.nb + Rk / a.W) * a.W + s_perm[i];
        val = *reinterpret_cast<const u32x4*>(a.v + (e * a.Hkv + kvh) * kHeadDim + dv * 8);
      }
      Stage& pg = own.pg[kk >> 4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int key = kk & 15;
        const uint32_t hw = bf16x2_to_f16x2(val[w]);
        pg.v[vslot(dv * 8 + 2 * w, key >> 3) * 8 + (key & 7)] = static_cast<uint16_t>(hw & 0xffffu);
        pg.v[vslot(dv * 8 + 2 * w + 1, key >> 3) * 8 + (key & 7)] = static_cast<uint16_t>(hw >> 16);
      }
    }
    __syncthreads();
    // this row sees own positions j W .. Rc (its window, up to itself)
    const int key0 = own_begin + ot * kTileKeys;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int pa = key0 + 32 * hf;
      const int lo = lim - pa, hi = Rc + 1 - pa;  // visible: lo <= key < hi of the 32
      if (!__ballot(lo < 32 && hi > 0)) continue;  // wave-uniform
      attend32(st, qr, own.pg[2 * hf], own.pg[2 * hf + 1], lane, lo, hi, lo - kPage, hi - kPage,
               a.scale_log2);
    }
  }

  // ---- cache tiles: positions 64 t .. 64 t + 63 ------------------------------
  for (int t = 0; t < n_tiles; ++t) {
    tile_wait_barrier(min(kBlkAhead - 1, n_tiles - 1 - t));
    if (t + kBlkAhead < n_tiles) issue_tile(t + kBlkAhead);
    Tile& tl = ring[t % kBlkStages];
    // the tile's values to fp16 in place, 2 of its 1024 16-byte V vectors per
    // thread; in the last tile, positions >= n_cache (no row sees them; they
    // may not be written) are cleared
    const int nv = n_cache - t * kTileKeys;  // keys of the tile below n_cache (workgroup-uniform)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int u = c * kBlkThreads + tid;
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
    lds_barrier();
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int pa = t * kTileKeys + 32 * hf;
      if (!__ballot(lim > pa)) continue;  // no row of this wavefront sees these keys
      attend32(st, qr, tl.pg[2 * hf], tl.pg[2 * hf + 1], lane, 0, lim - pa, 0, lim - pa - kPage,
               a.scale_log2);
    }
  }

  // ---- write out ----------------------------------------------------------------
  mfma32_guard(st.o[0]);
  mfma32_guard(st.o[1]);
  mfma32_guard(st.o[2]);
  mfma32_guard(st.o[3]);
  st.l = half_sum(st.l);  // every lane takes part in the swap
  if (!row_ok) return;
  const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
  uint16_t* orow =
      a.out + ((bwin * a.W + p) * a.Hq + static_cast<size_t>(kvh) * a.g + hh) * kHeadDim;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x2 w = {pack_bf16x2(st.o[dt][4 * q] * inv, st.o[dt][4 * q + 1] * inv),
                       pack_bf16x2(st.o[dt][4 * q + 2] * inv, st.o[dt][4 * q + 3] * inv)};
      *reinterpret_cast<u32x2*>(orow + dt * 32 + 8 * q + 4 * h) = w;
    }
}

}  // namespace wedlm

using namespace wedlm;

extern "C" int wedlm_block_attn_rope(int dtype, int S, int N, int W, int Hq, int Hkv, int D,
                                     int page_size, int num_pages, int max_pages, float scale,
                                     double theta, const void* q, const void* k, const void* v,
                                     const int32_t* perm, const int32_t* pos, const void* k_cache,
                                     const void* v_cache, const int32_t* block_table, void* out,
                                     void* stream) {
  if (!valid_dtype(dtype)) return WEDLM_ERR_UNSUPPORTED;
  if (S <= 0 || N <= 0 || W <= 0 || W > WEDLM_MAX_WINDOW || Hq <= 0 || Hkv <= 0 || D <= 0)
    return WEDLM_ERR_INVALID;
  if (N % W != 0 || Hq % Hkv != 0) return WEDLM_ERR_INVALID;
  if (!q || !k || !v || !perm || !pos || !k_cache || !v_cache || !block_table || !out)
    return WEDLM_ERR_INVALID;
  if (!(scale > 0.f) || !(theta > 0.0)) return WEDLM_ERR_INVALID;
  const int g = Hq / Hkv;
  if (dtype != WEDLM_BF16 || D != kHeadDim || page_size != kPage || kBlkRows % g != 0)
    return WEDLM_ERR_UNSUPPORTED;
  // the last window's prefix must fit the table and the table the pool
  if (num_pages <= 0 || max_pages <= 0 ||
      static_cast<long long>(max_pages) * page_size < static_cast<long long>(N) - W)
    return WEDLM_ERR_INVALID;
  BlockAttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.perm = perm;
  a.pos = pos;
  a.kc = static_cast<const uint16_t*>(k_cache);
  a.vc = static_cast<const uint16_t*>(v_cache);
  a.block_table = block_table;
  a.out = static_cast<uint16_t*>(out);
  a.S = S;
  a.N = N;
  a.W = W;
  a.nb = N / W;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.g = g;
  a.pos_per_wg = kBlkRows / g;
  a.n_groups = ceil_div(N, a.pos_per_wg);
  a.num_pages = num_pages;
  a.max_pages = max_pages;
  a.scale_log2 = scale * kLog2e;
  // rotation frequencies theta^(-2j/D), formed once on the host in double
  for (int jj = 0; jj < kHeadDim / 2; ++jj) a.omega[jj] = std::pow(theta, -2.0 * jj / kHeadDim);
  const long long blocks = 1LL * S * Hkv * a.n_groups;
  if (blocks > 0x7fffffffLL) return WEDLM_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(k_block_attn_bf16, dim3(static_cast<unsigned>(blocks)), dim3(kBlkThreads), 0,
                     as_stream(stream), a);
  return launch_status();
}
