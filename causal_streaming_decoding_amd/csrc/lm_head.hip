// Vocabulary projection fused with the softmax entropy, argmax and selection.
//
// hyper.ai summary of WeDLM, "Method": each step runs one causal forward pass
// over the window, whose predictions feed a distance-penalised entropy rule;
// the last operation of that pass is the projection of each slot's final
// hidden state onto the vocabulary, z = h W^T (a plain linear layer here: no
// bias, no soft cap). This kernel forms z in registers and reduces it straight
// to the (max, sum, weighted sum, argmax) partials of the entropy pass, so the
// [B*W][V] logits never reach HBM.
//
// Product (D = A B, v_mfma_f32_32x32x16_bf16): A = 32 vocabulary rows of W
// (16 hidden elements each), B = 32 hidden-state rows; the accumulator lane l
// then holds, for hidden row l % 32, 16 vocabulary entries 8*(r/4) + 4*(l/32)
// + r%4, so a row's softmax partial needs one swap of the two lane halves.
//
// Workgroup: 4 wavefronts, 256 vocabulary entries (64 per wavefront, two
// 32-row A blocks) x up to 128 hidden rows (RB blocks of 32; more rows take
// more workgroups, dispatched next to each other so that the repeated W tile
// comes from the shared last-level cache). The hidden dimension streams in
// chunks of 64 through a 3-stage LDS ring filled by global->LDS DMA two
// chunks ahead, one barrier per chunk: a stage holds the chunk of the 256 W
// rows and of the hidden rows. Both are 128-byte lines whose 16-byte units are
// XOR-swizzled by row, so the 16 consecutive rows an MFMA operand read touches
// fall in different banks. The K order inside a chunk is free as long as A and
// B agree: lane half kg takes hidden elements kg*32 + 8*ks .. +7 at K-step ks.
#include "common.hpp"

#include <type_traits>

namespace wedlm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kLmThreads = 256;                      // 4 wavefronts
constexpr int kLmVB = 2;                             // 32-row vocabulary blocks per wavefront
constexpr int kLmVocabTile = 4 * kLmVB * 32;         // vocabulary entries per workgroup
constexpr int kLmKC = 64;                            // hidden elements per chunk
constexpr int kLmKSteps = kLmKC / 16;                // MFMA K-steps per chunk
constexpr int kLmStages = 3;                         // h chunks in the LDS ring
constexpr int kLmMaxRB = 4;                          // 32-row blocks of hidden rows per workgroup

__device__ __forceinline__ bf16x8_t as_bf16x8_t(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

// LDS unit (16 bytes) holding unit u of tile row r of an h chunk.
__device__ __forceinline__ int h_swz(int r, int u) { return u ^ (((r >> 1) & 7) ^ ((r & 1) << 2)); }

// global -> LDS DMA of 64 lanes x 16 bytes: lane l's bytes land at M0 + 16 l.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_byte_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(lds_byte_addr)
      : "memory");
}

struct LmArgs {
  const uint16_t* h;   // [rows][hidden]
  const uint16_t* w;   // [V][hidden]
  EntPartial* part;    // [rows][n_tiles]
  int rows, hidden, V, n_tiles;
};

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

template <int RB>
__global__ void __launch_bounds__(kLmThreads)
k_lm_head_partial(LmArgs a) {
  constexpr int kTileRows = 32 * RB;
  constexpr int kDmaH = RB;                   // h DMA instructions per wavefront per chunk (8 rows each)
  constexpr int kDmaW = kLmVocabTile / 32;    // W DMA instructions per wavefront per chunk
  constexpr int kGroup = kDmaH + kDmaW;       // DMAs per wavefront per chunk
  constexpr int kStageElems = (kLmVocabTile + kTileRows) * kLmKC;
  __shared__ uint16_t ring[kLmStages][kStageElems];  // [W rows | hidden rows][64], swizzled
  __shared__ EntPartial red[4][kTileRows];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, kg = lane >> 5;
  const int v_wg = blockIdx.y * kLmVocabTile;
  const int r0 = blockIdx.x * kTileRows;
  const int nk = a.hidden / kLmKC;

  // DMA sources: instruction j of this wavefront moves stage lines
  // (j*4 + wave)*8 .. +7; lane l takes line l/8, 16-byte unit l%8 of the
  // swizzled line. Lines 0..255 are W rows (clamped to V - 1; entries past V
  // are masked at the end), the rest hidden rows (clamped to rows - 1; never
  // stored).
  const uint16_t* wsrc[kDmaW];
  const uint16_t* hsrc[kDmaH];
#pragma unroll
  for (int j = 0; j < kDmaW; ++j) {
    const int line = (j * 4 + wave) * 8 + (lane >> 3);
    const int v = min(v_wg + line, a.V - 1);
    wsrc[j] = a.w + static_cast<size_t>(v) * a.hidden + h_swz(line, lane & 7) * 8;
  }
#pragma unroll
  for (int j = 0; j < kDmaH; ++j) {
    const int line = (j * 4 + wave) * 8 + (lane >> 3);
    const int row = min(r0 + line, a.rows - 1);
    hsrc[j] = a.h + static_cast<size_t>(row) * a.hidden + h_swz(line, lane & 7) * 8;
  }
  const uint32_t ring_base = static_cast<uint32_t>(
      reinterpret_cast<size_t>((__attribute__((address_space(3))) char*)(&ring[0][0])));
  auto issue = [&](int c) {
    const int k0 = c * kLmKC;
    const uint32_t stage = ring_base + (c % kLmStages) * (kStageElems * 2);
#pragma unroll
    for (int j = 0; j < kDmaW; ++j)
      dma16(wsrc[j] + k0, __builtin_amdgcn_readfirstlane(stage + (j * 4 + wave) * 8 * kLmKC * 2));
#pragma unroll
    for (int j = 0; j < kDmaH; ++j)
      dma16(hsrc[j] + k0, __builtin_amdgcn_readfirstlane(
                              stage + (kLmVocabTile + (j * 4 + wave) * 8) * kLmKC * 2));
  };

  f32x16 acc[kLmVB][RB];
#pragma unroll
  for (int vb = 0; vb < kLmVB; ++vb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[vb][rb][e] = 0.f;

  issue(0);
  if (nk > 1) issue(1);
  for (int c = 0; c < nk; ++c) {
    // this thread's DMAs of chunk c have landed (chunk c + 1's may remain);
    // the barrier publishes every wave's part and frees the stage of chunk
    // c - 1, which is refilled with chunk c + 2
    if (c + 1 < nk)
      wait_vm_barrier<kGroup>();
    else
      wait_vm_barrier<0>();
    if (c + 2 < nk) issue(c + 2);
    const uint16_t* st = &ring[c % kLmStages][0];
#pragma unroll
    for (int ks = 0; ks < kLmKSteps; ++ks) {
      const int u = kg * 4 + ks;
      u32x4_t wa[kLmVB];
#pragma unroll
      for (int vb = 0; vb < kLmVB; ++vb) {
        const int line = wave * 64 + vb * 32 + li;
        wa[vb] = *reinterpret_cast<const u32x4_t*>(st + line * kLmKC + h_swz(line, u) * 8);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int line = kLmVocabTile + rb * 32 + li;
        const u32x4_t hb = *reinterpret_cast<const u32x4_t*>(st + line * kLmKC + h_swz(line, u) * 8);
#pragma unroll
        for (int vb = 0; vb < kLmVB; ++vb)
          acc[vb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8_t(wa[vb]), as_bf16x8_t(hb),
                                                               acc[vb][rb], 0, 0, 0);
      }
    }
  }
  // the last MFMAs complete before their results are read (a sleep of ~128
  // clocks exceeds every MFMA's latency; the scheduling barriers keep the
  // reads after it)
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_sleep(2);
  __builtin_amdgcn_sched_barrier(0);

  // ---- softmax partial of each hidden row over this wavefront's 64 entries ----
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    EntPartial p{kNegBig, 0.f, 0.f, 0x7fffffff};
#pragma unroll
    for (int vb = 0; vb < kLmVB; ++vb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = v_wg + wave * 64 + vb * 32 + 8 * (r >> 2) + 4 * kg + (r & 3);
        const float z = acc[vb][rb][r];
        if (v < a.V && (z > p.m || (z == p.m && v < p.idx))) {
          p.m = z;
          p.idx = v;
        }
      }
    const float mb = p.m * kLog2eF;
#pragma unroll
    for (int vb = 0; vb < kLmVB; ++vb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = v_wg + wave * 64 + vb * 32 + 8 * (r >> 2) + 4 * kg + (r & 3);
        const float u = fmaf(acc[vb][rb][r], kLog2eF, -mb);
        const float e = v < a.V ? __builtin_amdgcn_exp2f(u) : 0.f;
        p.s += e;
        p.t = fmaf(e, u, p.t);
      }
    EntPartial o;
    o.m = __shfl_xor(p.m, 32, kWave);
    o.s = __shfl_xor(p.s, 32, kWave);
    o.t = __shfl_xor(p.t, 32, kWave);
    o.idx = __shfl_xor(p.idx, 32, kWave);
    // the same order in both halves, so both hold the same result
    if (kg == 0) {
      merge(p, o);
      red[wave][rb * 32 + li] = p;
    }
  }
  __syncthreads();
  if (tid < kTileRows && r0 + tid < a.rows) {
    EntPartial p = red[0][tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) merge(p, red[w][tid]);
    a.part[static_cast<size_t>(r0 + tid) * a.n_tiles + blockIdx.y] = p;
  }
}

// Merge of a row's tile partials, in tile order per thread and then a fixed
// tree: one workgroup per row, one partial per row out.
__global__ void __launch_bounds__(kLmThreads)
k_entropy_merge_rows(const EntPartial* __restrict__ part, int n_tiles, EntPartial* __restrict__ out) {
  const int row = blockIdx.x;
  const EntPartial* pr = part + static_cast<size_t>(row) * n_tiles;
  EntPartial acc{kNegBig, 0.f, 0.f, 0x7fffffff};
  for (int c = threadIdx.x; c < n_tiles; c += kLmThreads) merge(acc, pr[c]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    EntPartial o;
    o.m = __shfl_xor(acc.m, off, kWave);
    o.s = __shfl_xor(acc.s, off, kWave);
    o.t = __shfl_xor(acc.t, off, kWave);
    o.idx = __shfl_xor(acc.idx, off, kWave);
    merge(acc, o);
  }
  __shared__ EntPartial red[kLmThreads / kWave];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    EntPartial r = red[0];
#pragma unroll
    for (int w = 1; w < kLmThreads / kWave; ++w) merge(r, red[w]);
    out[row] = r;
  }
}

struct LmPlan {
  int rb, n_tiles, row_groups;
  size_t part_bytes, merged_bytes;
};

static LmPlan plan_lm_head(int rows, int V) {
  LmPlan pl{};
  pl.rb = rows <= 32 ? 1 : (rows <= 64 ? 2 : kLmMaxRB);
  pl.row_groups = ceil_div(rows, 32 * pl.rb);
  pl.n_tiles = ceil_div(V, kLmVocabTile);
  // partial offsets stay 256-byte aligned
  pl.part_bytes = (static_cast<size_t>(rows) * pl.n_tiles * sizeof(EntPartial) + 255) & ~size_t(255);
  pl.merged_bytes = static_cast<size_t>(rows) * sizeof(EntPartial);
  return pl;
}

static int validate_lm_head(int dtype, int B, int W, int hidden, int V) {
  if (!valid_dtype(dtype)) return WEDLM_ERR_UNSUPPORTED;
  if (B <= 0 || W <= 0 || W > WEDLM_MAX_WINDOW || hidden <= 0 || V <= 0) return WEDLM_ERR_INVALID;
  if (dtype != WEDLM_BF16 || hidden % kLmKC != 0) return WEDLM_ERR_UNSUPPORTED;
  if (1LL * B * W > 65535 || ceil_div(V, kLmVocabTile) > 65535) return WEDLM_ERR_UNSUPPORTED;
  return WEDLM_OK;
}

}  // namespace wedlm

using namespace wedlm;

extern "C" size_t wedlm_lm_head_select_workspace_size(int dtype, int B, int W, int hidden, int V) {
  if (validate_lm_head(dtype, B, W, hidden, V) != WEDLM_OK) return 0;
  const LmPlan pl = plan_lm_head(B * W, V);
  return pl.part_bytes + pl.merged_bytes;
}

extern "C" int wedlm_lm_head_select(int dtype, int B, int W, int hidden, int V,
                                    const void* hidden_states, const void* w_vocab,
                                    const uint8_t* filled, float lambda, float tau, int min_fill,
                                    float* entropy, float* score, int32_t* argmax_tok,
                                    uint8_t* selected, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  const int st0 = validate_lm_head(dtype, B, W, hidden, V);
  if (st0 != WEDLM_OK) return st0;
  if (min_fill != 0 && min_fill != 1) return WEDLM_ERR_INVALID;
  if (lambda != lambda || tau != tau) return WEDLM_ERR_INVALID;  // NaN
  if (!hidden_states || !w_vocab || !filled || !entropy || !score || !argmax_tok || !selected)
    return WEDLM_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(hidden_states) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(w_vocab) % 16 != 0)
    return WEDLM_ERR_INVALID;
  const int rows = B * W;
  const LmPlan pl = plan_lm_head(rows, V);
  if (workspace == nullptr || workspace_bytes < pl.part_bytes + pl.merged_bytes)
    return WEDLM_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  EntPartial* part = static_cast<EntPartial*>(workspace);
  EntPartial* merged =
      reinterpret_cast<EntPartial*>(static_cast<char*>(workspace) + pl.part_bytes);
  LmArgs a;
  a.h = static_cast<const uint16_t*>(hidden_states);
  a.w = static_cast<const uint16_t*>(w_vocab);
  a.part = part;
  a.rows = rows;
  a.hidden = hidden;
  a.V = V;
  a.n_tiles = pl.n_tiles;
  const dim3 grid(pl.row_groups, pl.n_tiles);
  switch (pl.rb) {
    case 1: hipLaunchKernelGGL(k_lm_head_partial<1>, grid, dim3(kLmThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_lm_head_partial<2>, grid, dim3(kLmThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL(k_lm_head_partial<4>, grid, dim3(kLmThreads), 0, s, a); break;
    default: hipLaunchKernelGGL(k_lm_head_partial<4>, grid, dim3(kLmThreads), 0, s, a); break;
  }
  int st = launch_status();
  if (st != WEDLM_OK) return st;
  hipLaunchKernelGGL(k_entropy_merge_rows, dim3(rows), dim3(kLmThreads), 0, s, part, pl.n_tiles,
                     merged);
  st = launch_status();
  if (st != WEDLM_OK) return st;
  return launch_entropy_select(merged, 1, B, W, filled, lambda, tau, min_fill, entropy, score,
                               argmax_tok, selected, s);
}
