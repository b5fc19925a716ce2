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
// 32-row A blocks) x up to 256 hidden rows (RB blocks of 32: the 256 rows'
// accumulators fill the accumulation registers; more rows take more
// workgroups, dispatched next to each other). The hidden dimension
// streams in chunks of 64:
//   - W, packed once by wedlm_lm_head_pack into 4 KB tiles (32 rows x 64, in
//     MFMA operand order): each wavefront loads its own tiles straight into
//     registers (nothing to share), one contiguous KB per load instruction,
//     three chunks ahead, in four rotating register buffers (the loop runs in
//     whole rotations, so that each buffer is a fixed set of registers);
//   - h: every row's chunk is shared by the 4 wavefronts through a 4-stage LDS
//     ring filled by global->LDS DMA, one barrier per chunk. Rows are 128-byte
//     lines whose 16-byte units are XOR-swizzled by row, so the 16
//     consecutive rows an operand read touches fall in different banks.
// The K order inside a chunk is free as long as A and B agree: lane half kg
// takes hidden elements kg*32 + 8*ks .. +7 at K-step ks.
#include "common.hpp"

#include <type_traits>

namespace wedlm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kLmThreads = 256;                      // 4 wavefronts
constexpr int kLmMaxVB = 2;                          // 32-row vocabulary blocks per wavefront (at most)
constexpr int kLmKC = 64;                            // hidden elements per chunk
constexpr int kLmKSteps = kLmKC / 16;                // MFMA K-steps per chunk
constexpr int kLmTileElems = 32 * kLmKC;             // one packed W tile: 32 rows x 64 (4 KB)
constexpr int kLmAhead = 3;                          // chunks requested ahead of the one computed
constexpr int kLmStages = kLmAhead + 1;              // h ring stages and W register buffers
constexpr int kLmMaxRB = 8;                          // 32-row blocks of hidden rows per workgroup
constexpr int kNumXcds = 8;  // MI355X: 8 XCDs of 32 CUs, each with its own L2

__device__ __forceinline__ bf16x8_t as_bf16x8_t(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

// LDS unit (16 bytes) holding unit u of tile row r of an h chunk.
__device__ __forceinline__ int h_swz(int r, int u) { return u ^ (((r >> 1) & 7) ^ ((r & 1) << 2)); }

// One 16-byte load per lane into registers through asm, so that the
// compiler adds no wait of its own (the waits are explicit and counted, and
// name the loaded registers; the build's assembly audit, isa_audit.py, checks
// that no instruction reads, copies or reuses them before that wait). It reads the packed projection, which streams
// through once per launch (a second row group on the same XCD finds it in
// L2 all the same): the non-temporal hint (nt) took the 16-row shape from
// 250 to 221 us and helped every other shape too.
__device__ __forceinline__ void load16(u32x4_t& dst, const void* p) {
  asm volatile("global_load_dwordx4 %0, %1, off nt" : "=v"(dst) : "v"(p) : "memory");
}

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
  const uint16_t* w;   // packed: [v_blocks][hidden / 64][4 K-steps][2][32 rows][8]
  EntPartial* part;    // [rows][n_tiles]
  int rows, hidden, V, n_tiles, v_blocks, row_groups;
};

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

// Wait until at most `behind` (<= N) later chunks' operations, kPer each, are
// in flight, then synchronise the workgroup (the count must be an immediate).
template <int kPer, int N>
__device__ __forceinline__ void wait_chunks_behind(int behind) {
  if constexpr (N == 0) {
    wait_vm_barrier<0>();
  } else {
    if (behind >= N)
      wait_vm_barrier<N * kPer>();
    else
      wait_chunks_behind<kPer, N - 1>(behind);
  }
}

template <int RB, int VB>
__global__ void __launch_bounds__(kLmThreads)
k_lm_head_partial(LmArgs a) {
  static_assert(VB == 1 || VB == 2, "vocabulary blocks per wavefront");
  constexpr int kTileRows = 32 * RB;
  constexpr int kWaveVocab = 32 * VB;         // vocabulary entries per wavefront
  constexpr int kDmaH = RB;                   // h DMA instructions per wavefront per chunk (8 rows each)
  constexpr int kPer = VB * kLmKSteps + kDmaH;  // vector-memory operations per wavefront per chunk
  constexpr int kStageElems = kTileRows * kLmKC;
  __shared__ uint16_t ring[kLmStages][kStageElems];  // hidden rows [row][64], swizzled
  __shared__ EntPartial red[4][kTileRows];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, kg = lane >> 5;
  // Workgroups are dealt to the 8 XCDs round-robin by linear id; the row
  // groups of one vocabulary tile are given ids on the same XCD, one after
  // the other, so they run together and share the tile's projection through
  // that XCD's L2 (with one row group this is the identity).
  const int xcd = blockIdx.x % kNumXcds;
  const int slot = blockIdx.x / kNumXcds;
  const int tile = (slot / a.row_groups) * kNumXcds + xcd;
  const int rg = slot % a.row_groups;
  if (tile >= a.n_tiles) return;  // padding of the last round of 8 tiles (whole workgroup)
  const int v_wg = tile * 4 * kWaveVocab;
  const int r0 = rg * kTileRows;
  const int nk = a.hidden / kLmKC;  // a multiple of 4 on this path

  // this lane's W: the packed tiles of its two 32-row vocabulary blocks (the
  // packed rows past V are zeros and their entries are masked at the end);
  // at K-step ks the lane reads 16 bytes at (ks*2 + kg)*32 + li of a tile,
  // so each load instruction reads 1 KB of contiguous memory
  const uint16_t* wtile[VB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) {
    const int blk = min((v_wg + wave * kWaveVocab) / 32 + vb, a.v_blocks - 1);
    wtile[vb] = a.w + static_cast<size_t>(blk) * nk * kLmTileElems + (kg * 32 + li) * 8;
  }
  // DMA sources: instruction j of this wavefront moves ring lines
  // (j*4 + wave)*8 .. +7; lane l takes line l/8, 16-byte unit l%8 of the
  // swizzled line (rows clamped to rows - 1; never stored). Instructions are
  // 32 lines apart, which leaves the swizzle unchanged.
  const int line0 = wave * 8 + (lane >> 3);
  const int hcol0 = h_swz(line0, lane & 7) * 8;
  const uint32_t ring_base = static_cast<uint32_t>(
      reinterpret_cast<size_t>((__attribute__((address_space(3))) char*)(&ring[0][0])));
  // B operand addresses: row blocks are 32 lines apart, which leaves the
  // swizzle (a function of line % 16) unchanged, so a block adds an immediate
  // offset to one of four per-lane bases (one per K-step)
  int hoff[kLmKSteps];
#pragma unroll
  for (int ks = 0; ks < kLmKSteps; ++ks) hoff[ks] = li * kLmKC + h_swz(li, kg * 4 + ks) * 8;

  typedef u32x4_t WBuf[VB][kLmKSteps];
  WBuf wbuf[kLmStages];
  // chunk c's W loads (asm, waits explicit) then its h DMAs into ring stage c % 4
  auto issue = [&](int c, auto stage_c, WBuf& wb) {
    constexpr int T = decltype(stage_c)::value;
    const int k0 = c * kLmKC;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
      for (int ks = 0; ks < kLmKSteps; ++ks)
        load16(wb[vb][ks], wtile[vb] + static_cast<size_t>(c) * kLmTileElems + ks * 512);
#pragma unroll
    for (int j = 0; j < kDmaH; ++j) {
      const int row = min(r0 + line0 + 32 * j, a.rows - 1);
      dma16(a.h + static_cast<size_t>(row) * a.hidden + hcol0 + k0,
            __builtin_amdgcn_readfirstlane(ring_base + T * (kStageElems * 2) +
                                           (j * 4 + wave) * 8 * kLmKC * 2));
    }
  };
  f32x16 acc[VB][RB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[vb][rb][e] = 0.f;

  // Chunk c (c % 4 == S): wait until only `behind` later chunks' operations
  // are in flight - this thread's W registers and DMAs of chunk c have landed;
  // the wait names the W registers so nothing reads them earlier - and
  // synchronise: every wave's h rows are visible and every wave is done with
  // chunk c - 1, whose stage and buffer take chunk c + 3 (when kIssue).
  auto step = [&](auto s_c, auto behind_c, auto issue_c, int c) {
    constexpr int S = decltype(s_c)::value;
    constexpr int kBehind = decltype(behind_c)::value;
    WBuf& wb = wbuf[S];
    if constexpr (VB == 2)
      asm volatile("s_waitcnt vmcnt(%8) lgkmcnt(0)\n\ts_barrier"
                   : "+v"(wb[0][0]), "+v"(wb[0][1]), "+v"(wb[0][2]), "+v"(wb[0][3]),
                     "+v"(wb[1][0]), "+v"(wb[1][1]), "+v"(wb[1][2]), "+v"(wb[1][3])
                   : "n"(kBehind * kPer)
                   : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%4) lgkmcnt(0)\n\ts_barrier"
                   : "+v"(wb[0][0]), "+v"(wb[0][1]), "+v"(wb[0][2]), "+v"(wb[0][3])
                   : "n"(kBehind * kPer)
                   : "memory");
    if constexpr (decltype(issue_c)::value)
      issue(c + kLmAhead, std::integral_constant<int, (S + kLmAhead) % kLmStages>{},
            wbuf[(S + kLmAhead) % kLmStages]);
    const uint16_t* st = &ring[S][0];
    // the B operands of K-step ks + 1 are read while those of ks feed the MFMAs
    u32x4_t hb[2][RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      hb[0][rb] = *reinterpret_cast<const u32x4_t*>(st + hoff[0] + rb * 32 * kLmKC);
#pragma unroll
    for (int ks = 0; ks < kLmKSteps; ++ks) {
      if (ks + 1 < kLmKSteps) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          hb[(ks + 1) & 1][rb] =
              *reinterpret_cast<const u32x4_t*>(st + hoff[ks + 1] + rb * 32 * kLmKC);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int vb = 0; vb < VB; ++vb)
          acc[vb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              as_bf16x8_t(wb[vb][ks]), as_bf16x8_t(hb[ks & 1][rb]), acc[vb][rb], 0, 0, 0);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using Yes = std::true_type;
  using No = std::false_type;
  issue(0, I0{}, wbuf[0]);
  issue(1, I1{}, wbuf[1]);
  issue(2, I2{}, wbuf[2]);
  // whole rotations: every step issues, two later chunks are in flight at each wait
  int c = 0;
  for (; c + 8 <= nk; c += 4) {
    step(I0{}, I2{}, Yes{}, c);
    step(I1{}, I2{}, Yes{}, c + 1);
    step(I2{}, I2{}, Yes{}, c + 2);
    step(I3{}, I2{}, Yes{}, c + 3);
  }
  // the last four chunks (c = nk - 4): only the first still issues
  step(I0{}, I2{}, Yes{}, c);
  step(I1{}, I2{}, No{}, c + 1);
  step(I2{}, I1{}, No{}, c + 2);
  step(I3{}, I0{}, No{}, c + 3);
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
    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = v_wg + wave * kWaveVocab + vb * 32 + 8 * (r >> 2) + 4 * kg + (r & 3);
        const float z = acc[vb][rb][r];
        if (v < a.V && (z > p.m || (z == p.m && v < p.idx))) {
          p.m = z;
          p.idx = v;
        }
      }
    const float mb = p.m * kLog2eF;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = v_wg + wave * kWaveVocab + vb * 32 + 8 * (r >> 2) + 4 * kg + (r & 3);
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
    // one row block at a time: only its 32 accumulators are moved out of the
    // accumulation registers at once
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  if (tid < kTileRows && r0 + tid < a.rows) {
    EntPartial p = red[0][tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) merge(p, red[w][tid]);
    a.part[static_cast<size_t>(r0 + tid) * a.n_tiles + tile] = p;
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
  int rb, vb, n_tiles, row_groups;
  size_t part_bytes, merged_bytes;
};

static LmPlan plan_lm_head(int rows, int V) {
  LmPlan pl{};
  // up to 256 rows: groups of at most 128 rows (two groups on one XCD share
  // each tile through L2: 434 against 450 us for one 256-row group at 256
  // rows); above that 256-row groups (four 128-row groups measured slower)
  pl.rb = rows <= 32 ? 1 : (rows <= 64 ? 2 : (rows <= 256 ? 4 : kLmMaxRB));
  // two blocks per wavefront: one block (twice the tiles, a smaller last
  // round) measured slower for 256 and 512 rows
  pl.vb = kLmMaxVB;
  pl.row_groups = ceil_div(rows, 32 * pl.rb);
  pl.n_tiles = ceil_div(V, 4 * 32 * pl.vb);
  // partial offsets stay 256-byte aligned
  pl.part_bytes = (static_cast<size_t>(rows) * pl.n_tiles * sizeof(EntPartial) + 255) & ~size_t(255);
  pl.merged_bytes = static_cast<size_t>(rows) * sizeof(EntPartial);
  return pl;
}

// hidden: whole 4-chunk rotations of the main loop (a multiple of 256)
static int validate_shape(int dtype, int hidden, int V) {
  if (!valid_dtype(dtype)) return WEDLM_ERR_UNSUPPORTED;
  if (hidden <= 0 || V <= 0) return WEDLM_ERR_INVALID;
  if (dtype != WEDLM_BF16 || hidden % (kLmKC * kLmStages) != 0) return WEDLM_ERR_UNSUPPORTED;
  if (ceil_div(V, 4 * 32) > 65535 || 1LL * ceil_div(V, 32) * 32 * hidden > (1LL << 40))
    return WEDLM_ERR_UNSUPPORTED;
  return WEDLM_OK;
}

static int validate_lm_head(int dtype, int B, int W, int hidden, int V) {
  const int st = validate_shape(dtype, hidden, V);
  if (st != WEDLM_OK) return st;
  if (B <= 0 || W <= 0 || W > WEDLM_MAX_WINDOW) return WEDLM_ERR_INVALID;
  if (1LL * B * W > 65535) return WEDLM_ERR_UNSUPPORTED;
  return WEDLM_OK;
}

// Packs w [V][hidden] into 4 KB tiles, one thread per 16-byte vector of the
// packed array: tile (block b, chunk c) holds rows 32b .. 32b+31 and hidden
// elements 64c .. 64c+63 as [K-step ks][half kg][row li][8], where the 8
// elements are hidden 64c + 32kg + 8ks .. +7. Rows past V are zeros.
__global__ void __launch_bounds__(256)
k_lm_head_pack(const uint16_t* __restrict__ w, uint16_t* __restrict__ out, int V, int hidden,
               long long n_vec) {
  const long long o = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (o >= n_vec) return;
  const int nk = hidden / kLmKC;
  const int li = static_cast<int>(o & 31);
  const int kg = static_cast<int>((o >> 5) & 1);
  const int ks = static_cast<int>((o >> 6) & 3);
  const long long tile = o >> 8;
  const int c = static_cast<int>(tile % nk);
  const long long b = tile / nk;
  const long long v = b * 32 + li;
  u32x4_t x = {0u, 0u, 0u, 0u};
  if (v < V)
    x = *reinterpret_cast<const u32x4_t*>(w + v * hidden + c * kLmKC + kg * 32 + ks * 8);
  *reinterpret_cast<u32x4_t*>(out + o * 8) = x;
}

}  // namespace wedlm

using namespace wedlm;

extern "C" size_t wedlm_lm_head_packed_size(int dtype, int hidden, int V) {
  if (validate_shape(dtype, hidden, V) != WEDLM_OK) return 0;
  return static_cast<size_t>(ceil_div(V, 32)) * 32 * hidden * elt_size(dtype);
}

extern "C" int wedlm_lm_head_pack(int dtype, int hidden, int V, const void* w_vocab, void* w_packed,
                                  void* stream) {
  const int st = validate_shape(dtype, hidden, V);
  if (st != WEDLM_OK) return st;
  if (!w_vocab || !w_packed || reinterpret_cast<uintptr_t>(w_vocab) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(w_packed) % 16 != 0)
    return WEDLM_ERR_INVALID;
  const long long n_vec = 1LL * ceil_div(V, 32) * 32 * hidden / 8;
  const long long blocks = (n_vec + 255) / 256;
  if (blocks > 0x7fffffffLL) return WEDLM_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(k_lm_head_pack, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     as_stream(stream), static_cast<const uint16_t*>(w_vocab),
                     static_cast<uint16_t*>(w_packed), V, hidden, n_vec);
  return launch_status();
}

extern "C" size_t wedlm_lm_head_select_workspace_size(int dtype, int B, int W, int hidden, int V) {
  if (validate_lm_head(dtype, B, W, hidden, V) != WEDLM_OK) return 0;
  const LmPlan pl = plan_lm_head(B * W, V);
  return pl.part_bytes + pl.merged_bytes;
}

extern "C" int wedlm_lm_head_select(int dtype, int B, int W, int hidden, int V,
                                    const void* hidden_states, const void* w_packed,
                                    const uint8_t* filled, float lambda, float tau, int min_fill,
                                    float* entropy, float* score, int32_t* argmax_tok,
                                    uint8_t* selected, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  const int st0 = validate_lm_head(dtype, B, W, hidden, V);
  if (st0 != WEDLM_OK) return st0;
  if (min_fill != 0 && min_fill != 1) return WEDLM_ERR_INVALID;
  if (lambda != lambda || tau != tau) return WEDLM_ERR_INVALID;  // NaN
  if (!hidden_states || !w_packed || !filled || !entropy || !score || !argmax_tok || !selected)
    return WEDLM_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(hidden_states) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(w_packed) % 16 != 0)
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
  a.w = static_cast<const uint16_t*>(w_packed);
  a.part = part;
  a.rows = rows;
  a.hidden = hidden;
  a.V = V;
  a.n_tiles = pl.n_tiles;
  a.v_blocks = ceil_div(V, 32);
  a.row_groups = pl.row_groups;
  const dim3 grid(pl.row_groups * ceil_div(pl.n_tiles, kNumXcds) * kNumXcds);
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(kLmThreads), 0, s, a); };
  if (pl.rb == 1) go(k_lm_head_partial<1, 2>);
  else if (pl.rb == 2) go(k_lm_head_partial<2, 2>);
  else if (pl.rb == 4) go(k_lm_head_partial<4, 2>);
  else go(k_lm_head_partial<8, 2>);
  int st = launch_status();
  if (st != WEDLM_OK) return st;
  hipLaunchKernelGGL(k_entropy_merge_rows, dim3(rows), dim3(kLmThreads), 0, s, part, pl.n_tiles,
                     merged);
  st = launch_status();
  if (st != WEDLM_OK) return st;
  return launch_entropy_select(merged, 1, B, W, filled, lambda, tau, min_fill, entropy, score,
                               argmax_tok, selected, s);
}
