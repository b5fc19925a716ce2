// Per-sequence operations of the window step, one wavefront per sequence
// (lane i holds slot i, W <= 64). The separate kernels (reorder, selection,
// state commit) and the fused step tail all run these same functions, so both
// forms give bitwise equal results.
//
// hyper.ai summary of WeDLM, "Method": filled slots are moved before the masks
// with their logical positions kept; positions are filled by a
// distance-penalised entropy rule; the leftmost contiguous filled run is
// committed and masks are appended. sai.science review, "Weaknesses": the
// adjusted-entropy equation is missing (read as entropy + lambda * slot);
// "Reproducibility & code": a None threshold decodes one token per step.
#pragma once

#include "common.hpp"

namespace wedlm {

// Tokens the commit takes: the run, clamped to the window and to the pages the
// table holds beyond L.
__device__ __forceinline__ int commit_length(int run, int L, int W, int max_pages, int P) {
  int c = min(max(run, 0), W);
  const int room = max(max_pages * P - L, 0);
  return min(c, room);
}

// (a4) Merges row (b, i)'s n_chunks entropy partials in chunk order, forms the
// entropy H = ln2 (log2 s - t / s), argmax and score = H + lambda * i (fp32:
// the product rounded, then the sum), writes them, and returns whether the
// slot is selected: a mask slot (cand) whose score is below tau, or - when no
// slot of the sequence clears tau and min_fill is 1 - the candidate with the
// lowest score (lowest slot on equal scores). Every lane of the wavefront
// must call it. argmax_out receives the slot's argmax (lanes past W: 0).
__device__ __forceinline__ bool wave_select(const EntPartial* __restrict__ part, int n_chunks,
                                            int b, int W, int i, bool cand_in, float lambda,
                                            float tau, int min_fill, float* __restrict__ entropy,
                                            float* __restrict__ score,
                                            int32_t* __restrict__ argmax_tok,
                                            uint8_t* __restrict__ selected, int& argmax_out) {
  const bool in_window = i < W;
  float sc = INFINITY;
  bool cand = false;
  argmax_out = 0;
  if (in_window) {
    const int row = b * W + i;
    const EntPartial* pr = part + static_cast<size_t>(row) * n_chunks;
    EntPartial acc = pr[0];
    // partials are loaded 8 at a time so that their latencies overlap, and
    // merged in chunk order
    for (int c0 = 1; c0 < n_chunks; c0 += 8) {
      EntPartial buf[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (c0 + k < n_chunks) buf[k] = pr[c0 + k];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (c0 + k < n_chunks) merge(acc, buf[k]);
    }
    const float H = kLn2F * (log2f(acc.s) - acc.t / acc.s);
    // product rounded, then the sum: no fused multiply-add
    sc = __fadd_rn(H, __fmul_rn(lambda, static_cast<float>(i)));
    entropy[row] = H;
    score[row] = sc;
    argmax_tok[row] = acc.idx;
    argmax_out = acc.idx;
    cand = cand_in;
  }
  bool sel = cand && sc < tau;
  const uint64_t any_sel = __ballot(sel);
  const uint64_t any_cand = __ballot(cand);
  if (any_sel == 0 && any_cand != 0 && min_fill == 1) {
    // lowest score among candidates, lowest slot on equal scores
    float best = cand ? sc : INFINITY;
    int who = cand ? i : kWave;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ob = __shfl_xor(best, off, kWave);
      const int ow = __shfl_xor(who, off, kWave);
      if (ob < best || (ob == best && ow < who)) {
        best = ob;
        who = ow;
      }
    }
    sel = (i == who);
  }
  if (in_window) selected[b * W + i] = sel ? 1 : 0;
  return sel;
}

// (a5, window state) Commits c = commit_length(run) tokens: lane i's new slot
// is old slot i + c with this step's fills applied (filled |= selected, token
// = argmax where selected), the last c slots become masks, L grows by c, and
// the cache slots of the committed positions L .. L+c-1 are recorded
// (page id * P + offset, -1 past c). f_in / tok_in are the lane's
// forward-time flag and token. Every lane must call it; returns the new L and
// sets f_out to the lane's new filled flag.
__device__ __forceinline__ int wave_commit_state(int b, int W, int i, int P, int num_pages,
                                                 int max_pages, int run, bool f_in, int tok_in,
                                                 bool sel, int argmax,
                                                 const int32_t* __restrict__ block_table,
                                                 int32_t* __restrict__ tokens,
                                                 uint8_t* __restrict__ filled,
                                                 int32_t* __restrict__ prefix_len,
                                                 int32_t* __restrict__ commit_len,
                                                 int32_t* __restrict__ cache_slot, int32_t mask_id,
                                                 bool& f_out) {
  const bool in_window = i < W;
  const int L = max(prefix_len[b], 0);
  const int c = commit_length(run, L, W, max_pages, P);
  int f = 0, tok = mask_id;
  if (in_window) {
    f = (f_in || sel) ? 1 : 0;
    tok = sel ? argmax : tok_in;
  }
  // every lane has its slot; shift left by c within the wavefront
  const int src = i + c;
  const int f_sh = __shfl(f, src < kWave ? src : 0, kWave);
  const int t_sh = __shfl(tok, src < kWave ? src : 0, kWave);
  f_out = false;
  if (in_window) {
    const int row = b * W + i;
    const bool keep = src < W;
    f_out = keep && f_sh != 0;
    filled[row] = f_out ? 1 : 0;
    tokens[row] = keep ? t_sh : mask_id;
    int slot = -1;
    if (i < c) {
      const int t = L + i;
      const int pid = min(max(block_table[static_cast<size_t>(b) * max_pages + t / P], 0),
                          num_pages - 1);
      slot = pid * P + t % P;
    }
    cache_slot[row] = slot;
  }
  if (i == 0) {
    commit_len[b] = c;
    prefix_len[b] = L + c;
  }
  return L + c;
}

// (a1) Topological reorder of one window from the lanes' filled flags: a
// ballot gives the window as one 64-bit mask; a slot's physical index is a
// popcount of the flags below it (filled) or n_obs plus the popcount of the
// masks below it (masks) - the stable partition; slot i has logical position
// L + i. run_len is the leading filled run (the trailing ones of the ballot),
// or under the block rule W when the whole window is filled and 0 otherwise.
// Every lane must call it.
__device__ __forceinline__ void wave_reorder(int b, int W, int lane, bool f, int L, int block_rule,
                                             int32_t* __restrict__ perm,
                                             int32_t* __restrict__ inv_perm,
                                             int32_t* __restrict__ pos, int32_t* __restrict__ n_obs,
                                             int32_t* __restrict__ run_len) {
  const bool in_window = lane < W;
  const bool fl = in_window && f;
  const uint64_t fm = __ballot(fl);
  const uint64_t window = (W == kWave) ? ~0ull : ((1ull << W) - 1ull);
  const uint64_t mm = ~fm & window;
  const uint64_t below = (1ull << lane) - 1ull;  // lane < 64, so the shift is defined
  const int nobs = __popcll(fm);
  const int phys = fl ? __popcll(fm & below) : nobs + __popcll(mm & below);
  if (in_window) {
    inv_perm[b * W + lane] = phys;
    perm[b * W + phys] = lane;
    pos[b * W + phys] = L + lane;
  }
  if (lane == 0) {
    n_obs[b] = nobs;
    // lanes >= W contribute 0 bits, so the first zero is at most W
    const uint64_t zeros = ~fm;
    const int run = zeros == 0 ? kWave : __builtin_ctzll(zeros);
    run_len[b] = block_rule ? (run == W ? W : 0) : run;
  }
}

}  // namespace wedlm
