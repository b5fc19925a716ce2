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
// Per 32 keys and wavefront the 32-row tile of attn_tile32.hpp: bf16 scores,
// the fp16 PV product, K rows in the permuted order and the V page swizzled
// for conflict-free operand reads.
#include "attn_device.hpp"
#include "attn_tile32.hpp"
#include "common.hpp"

#include <cmath>

namespace wedlm {

constexpr int kBlkWaves = 8;
constexpr int kBlkThreads = kBlkWaves * kWave;  // 512
constexpr int kBlkRows = 32 * kBlkWaves;        // query rows per workgroup
constexpr int kBlkStages = 3;                   // ring tiles (96 KB)
constexpr int kBlkAhead = kBlkStages - 1;       // cache tiles in flight while one is computed
constexpr int kMaxOwn = kBlkRows + WEDLM_MAX_WINDOW;  // own keys of a workgroup, at most
static_assert(kBlkThreads == kTileThreads, "the tile helpers assume 512 threads");

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
  auto issue_tile = [&](int t) {
    int id[kTilePages];
    load_page_ids4(bt, 4 * t, a.max_pages, id);
    tile_dma<false>(ring[t % kBlkStages], id, a.kc, a.vc, a.Hkv, kvh, a.num_pages, wave, lane);
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
  // Tile t + 1's values are converted to fp16 while tile t is computed, so one
  // barrier per tile both publishes them and frees the stage tile t + 2
  // takes; in the last tile, positions >= n_cache (no row sees them; they may
  // not be written) are cleared.
  if (n_tiles > 0) {
    tile_wait_barrier(min(kBlkAhead - 1, n_tiles - 1));  // tile 0 has landed
    tile_v_to_f16(ring[0], tid, n_cache);
  }
  for (int t = 0; t < n_tiles; ++t) {
    // only tile t + 1's DMAs can be in flight here: after this barrier it has
    // landed everywhere, tile t's values are fp16 everywhere, and tile t - 1's
    // stage is free
    tile_wait_barrier(0);
    if (t + kBlkAhead < n_tiles) issue_tile(t + kBlkAhead);
    if (t + 1 < n_tiles)
      tile_v_to_f16(ring[(t + 1) % kBlkStages], tid, n_cache - (t + 1) * kTileKeys);
    const Tile& tl = ring[t % kBlkStages];
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
