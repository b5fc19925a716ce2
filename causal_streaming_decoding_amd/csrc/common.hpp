// Shared device/host helpers of the wedlm HIP library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wedlm.h"

namespace wedlm {

constexpr int kWave = 64;

// ---- bf16 storage as raw 16-bit words --------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// float -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.f));
}

// Low / high bf16 of a packed 32-bit word, as float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Element load/store through float for the f32 / bf16 template paths.
template <typename T> struct Elt;
template <> struct Elt<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float x) { *p = x; }
};
template <> struct Elt<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(uint16_t* p, float x) { *p = f32_to_bf16(x); }
};

// ---- kernel arguments ------------------------------------------------------

// The compiler reads each kernel argument where it is first used, and each
// read of a new 64-byte line of the argument segment waits for that line (a
// launch-latency cost on short kernels: several such waits in a row before the
// first global load). This touches every line of the first kBytes bytes (all
// inside the kernel's explicit arguments) with scalar loads issued together
// before one wait, so the later reads hit the scalar cache.
template <int kBytes>
__device__ __forceinline__ void touch_kernargs() {
  const __attribute__((address_space(4))) uint32_t* ka =
      (const __attribute__((address_space(4))) uint32_t*)__builtin_amdgcn_kernarg_segment_ptr();
  uint32_t x = 0;
#pragma unroll
  for (int o = 0; o + 4 <= kBytes; o += 64) x ^= ka[o / 4];
  asm volatile("" ::"s"(x));
}

// ---- RoPE angle ---------------------------------------------------------------

// cos and sin of t * omega radians (RoFormer rotation, mlsanity.com page on
// WeDLM, "Builds on"). The angle is formed in double precision and reduced by
// multiples of pi/2 (a two-part pi/2, so the remainder keeps ~1e-16 absolute
// accuracy for angles up to 1e6 rad; an fp32 angle at position 1e4 would be
// off by milliradians). On the remainder, |r| <= pi/4, the Taylor series of
// sin to r^9 and of cos to r^10 are below 1e-8 of truncation error, and are
// evaluated in fp32; the quadrant n mod 4 then rotates (sin, cos).
__device__ __forceinline__ void rope_cos_sin(double t, double omega, float& c, float& s) {
  constexpr double k2OverPi = 0.6366197723675814;
  constexpr double kPiHalfHi = 1.5707963267948966;     // nearest double to pi/2
  constexpr double kPiHalfLo = 6.123233995736766e-17;  // pi/2 - kPiHalfHi
  const double a = t * omega;
  const double n = rint(a * k2OverPi);
  const float r = static_cast<float>(fma(-n, kPiHalfHi, a) - n * kPiHalfLo);
  const float r2 = r * r;
  const float sr =
      r * fmaf(r2, fmaf(r2, fmaf(r2, fmaf(r2, 2.7557319e-6f, -1.9841270e-4f), 8.3333333e-3f),
                        -1.6666667e-1f),
               1.f);
  const float cr = fmaf(
      r2,
      fmaf(r2, fmaf(r2, fmaf(r2, fmaf(r2, -2.7557319e-7f, 2.4801587e-5f), -1.3888889e-3f),
                    4.1666668e-2f),
           -0.5f),
      1.f);
  const int q = static_cast<int>(static_cast<long long>(n) & 3);
  // sin(r + q pi/2) and cos(r + q pi/2)
  s = q == 0 ? sr : (q == 1 ? cr : (q == 2 ? -sr : -cr));
  c = q == 0 ? cr : (q == 1 ? -sr : (q == 2 ? -cr : sr));
}

// ---- wave reductions (64 lanes) --------------------------------------------

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// ---- softmax entropy partials ----------------------------------------------

constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLn2F = 0.6931471805599453f;
// A start value below any finite logit that keeps (m_old - m_new) * log2e finite.
constexpr float kNegBig = -1.0e30f;

// Reduction state of softmax entropy over part of a row of logits z, in base
// 2: m = max z, s = sum 2^u and t = sum u 2^u with u = (z - m) log2(e); idx is
// the lowest index holding m. Entropy in nats is ln2 (log2 s - t / s).
struct EntPartial {
  float m, s, t;
  int idx;
};

// a <- a (+) b: both sums are moved to the larger reference max by the exact
// identity t' = (t + d s) 2^d, s' = s 2^d with d = (m_old - m_new) log2(e);
// ties of the max keep the lower index.
__device__ __forceinline__ void merge(EntPartial& a, const EntPartial& b) {
  const float mn = fmaxf(a.m, b.m);
  const float da = (a.m - mn) * kLog2eF, db = (b.m - mn) * kLog2eF;
  const float fa = __builtin_amdgcn_exp2f(da), fb = __builtin_amdgcn_exp2f(db);
  const float s = a.s * fa + b.s * fb;
  const float t = (a.t + da * a.s) * fa + (b.t + db * b.s) * fb;
  int idx;
  if (a.m > b.m) idx = a.idx;
  else if (b.m > a.m) idx = b.idx;
  else idx = min(a.idx, b.idx);
  a.m = mn;
  a.s = s;
  a.t = t;
  a.idx = idx;
}

// ---- host helpers -----------------------------------------------------------

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? WEDLM_OK : WEDLM_ERR_HIP;
}

inline size_t elt_size(int dtype) { return dtype == WEDLM_BF16 ? 2 : 4; }

inline bool valid_dtype(int dtype) { return dtype == WEDLM_F32 || dtype == WEDLM_BF16; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Largest layer, sequence and head counts the host-side launch plans take.
constexpr int kMaxShapeDim = 65535;

// ceil(a / b) for b > 0, without forming a + b - 1 (no overflow near INT_MAX)
inline int ceil_div(int a, int b) { return a / b + (a % b > 0 ? 1 : 0); }

// Internal: the selection half of wedlm_entropy_select over n_chunks partials
// per row ([B * W][n_chunks], in vocabulary order), enqueued on `s`. Defined
// in entropy.hip.
int launch_entropy_select(const EntPartial* part, int n_chunks, int B, int W,
                          const uint8_t* filled, float lambda, float tau, int min_fill,
                          float* entropy, float* score, int32_t* argmax_tok, uint8_t* selected,
                          hipStream_t s);

}  // namespace wedlm
