// Merge of the key-range split partials of the bf16 window attention.
//
// When a group's keys are split across workgroups (few groups for the GPU),
// each split leaves (max m_s, sum l_s, unnormalised O_s) of its keys, in log2
// units, and the output is
//   out = sum_s O_s 2^(m_s - m) / sum_s l_s 2^(m_s - m),  m = max_s m_s
// (FlashAttention's online-softmax merge, mlsanity.com page on WeDLM,
// "Builds on"). One thread per (group, row, 4 value dimensions) makes one pass
// over the group's splits (the plan entry its split 0 wrote: first slot,
// count) with a running reference max, reading kCombineBatch splits at a time
// with every load of a batch issued before any is used.
//
// The merge runs either in a kernel of its own right after the attention
// (wedlm_window_attn*) or, when the attention call defers it, in the launch of
// the step tail (wedlm_select_commit_reorder_combine), as extra workgroups
// beside the per-sequence tail: both read the partials the attention left.
#pragma once

#include "common.hpp"

namespace wedlm {

struct CombineArgs {
  const float* ws_o;     // [slots][M][128] unnormalised partial outputs
  const float* ws_ml;    // [slots][M][2] (m, l)
  const int2* ws_plan;   // [groups]: first slot and number of splits
  uint16_t* out;         // [n_layers][B][W][Hq][128] bf16, physical rows
  int n_groups, M, W, Hq, Hkv, g, cols;
  long long n_slots;
  long long threads;     // n_groups * M * 32; 0: nothing to merge
};

constexpr int kCombineBatch = 8;
constexpr int kCombineDim = 128;

__device__ __forceinline__ void combine_quad(const CombineArgs& c, long long idx) {
  const int quads = kCombineDim / 4;
  const int d4 = static_cast<int>(idx % quads);
  const int row = static_cast<int>((idx / quads) % c.M);
  const int group = static_cast<int>(idx / (static_cast<long long>(quads) * c.M));
  int2 plan = c.ws_plan[group];
  // the plan entry is device data: keep its slots inside the partials (a
  // column holds cols of them), whatever it holds
  plan.x = static_cast<int>(min(max(static_cast<long long>(plan.x), 0LL), c.n_slots - 1));
  const int n_splits = static_cast<int>(
      min(static_cast<long long>(min(max(plan.y, 0), c.cols)), c.n_slots - plan.x));
  float m = -INFINITY, lsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < n_splits; s0 += kCombineBatch) {
    float2 ml[kCombineBatch];
    float4 o[kCombineBatch];
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      const int s = s0 + k;
      const size_t part = (static_cast<size_t>(plan.x) + s) * c.M + row;
      ml[k] = s < n_splits ? reinterpret_cast<const float2*>(c.ws_ml)[part]
                           : make_float2(-INFINITY, 0.f);
      o[k] = s < n_splits ? *reinterpret_cast<const float4*>(c.ws_o + part * kCombineDim + d4 * 4)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // a split with no keys (l = 0, m = -inf) contributes nothing
    float bm = m;
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k)
      if (ml[k].y != 0.f) bm = fmaxf(bm, ml[k].x);
    if (bm > m) {
      const float r = __builtin_amdgcn_exp2f(m - bm);  // 0 while m = -inf
      acc.x *= r;
      acc.y *= r;
      acc.z *= r;
      acc.w *= r;
      lsum *= r;
      m = bm;
    }
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      if (ml[k].y == 0.f) continue;
      const float w = __builtin_amdgcn_exp2f(ml[k].x - m);
      acc.x += o[k].x * w;
      acc.y += o[k].y * w;
      acc.z += o[k].z * w;
      acc.w += o[k].w * w;
      lsum += ml[k].y * w;
    }
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const int kvh = group % c.Hkv;
  const int lbi = group / c.Hkv;  // layer * B + b
  const int p = row / c.g, hh = row % c.g;
  uint16_t* orow = c.out + ((static_cast<size_t>(lbi) * c.W + p) * c.Hq + kvh * c.g + hh) * kCombineDim;
  uint2 w;
  w.x = pack_bf16x2(acc.x * inv, acc.y * inv);
  w.y = pack_bf16x2(acc.z * inv, acc.w * inv);
  *reinterpret_cast<uint2*>(orow + d4 * 4) = w;
}

// Host side (attn.hip): the merge of an attention call with these shapes and
// workspace, as wedlm_window_attn* would launch it. c->threads = 0 when that
// call does not split key ranges. Returns a WEDLM status (shape checks as the
// attention's; WEDLM_ERR_WORKSPACE when the workspace is smaller than the
// call's).
int attn_combine_args(int dtype, int n_layers, int B, int W, int Hq, int Hkv, int D,
                      int page_size, int max_prefix_len, const void* workspace,
                      size_t workspace_bytes, void* out, CombineArgs* c);

}  // namespace wedlm
