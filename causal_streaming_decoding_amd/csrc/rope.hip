// RoPE at logical positions, gathered into physical order.
//
// RoFormer rotation (mlsanity.com page on WeDLM, "Builds on") at the logical
// position each window token keeps through the reordering (hyper.ai summary,
// "Method"). Rotate-half pairing: dimension j turns with j + D/2 by
// pos * theta^(-2j/D).
//
// One workgroup per (physical row p, sequence b, group of layers). The D/2
// angles of the row are formed and their sine/cosine taken in double precision
// once per workgroup (they do not depend on the layer or head), then kept in
// LDS as fp32. Every head's pair of 16-byte half-vectors (dims j..j+X-1 and
// j+D/2..) is read, rotated in fp32 and rounded once to the storage type. Values
// are only gathered. The gather reads the slot perm[p] and writes row p, so
// reads and writes are both whole contiguous head rows.
#include "common.hpp"

namespace wedlm {

constexpr int kRopeThreads = 256;
constexpr int kRopeLayersPerBlock = 4;

template <typename T>
struct Vec16 {
  static constexpr int N = 16 / sizeof(T);
  union {
    uint4 raw;
    T e[N];
  };
};

template <typename T, bool VEC>
__global__ void __launch_bounds__(kRopeThreads)
k_rope_logical(int n_layers, int B, int W, int Hq, int Hkv, int D, double log2_theta,
               const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
               const int32_t* __restrict__ perm, const int32_t* __restrict__ pos,
               T* __restrict__ q_phys, T* __restrict__ k_phys, T* __restrict__ v_phys) {
  __shared__ float cs[128];
  __shared__ float sn[128];
  const int p = blockIdx.x;
  const int b = blockIdx.y;
  const int l0 = blockIdx.z * kRopeLayersPerBlock;
  const int l1 = min(n_layers, l0 + kRopeLayersPerBlock);
  const int half = D / 2;
  const int slot = min(max(perm[b * W + p], 0), W - 1);
  const double t = static_cast<double>(pos[b * W + p]);
  for (int j = threadIdx.x; j < half; j += kRopeThreads) {
    const double omega = exp2(-(2.0 * j / D) * log2_theta);
    double s, c;
    sincos(t * omega, &s, &c);
    cs[j] = static_cast<float>(c);
    sn[j] = static_cast<float>(s);
  }
  __syncthreads();

  constexpr int N = VEC ? Vec16<T>::N : 1;
  const int nvec = half / N;  // half-vectors per head
  const int rot_tasks = (Hq + Hkv) * nvec;
  const int copy_tasks = Hkv * (D / N);
  for (int layer = l0; layer < l1; ++layer) {
    const size_t lb = static_cast<size_t>(layer) * B + b;
    const T* qs = q + (lb * W + slot) * Hq * D;
    const T* ks = k + (lb * W + slot) * Hkv * D;
    T* qd = q_phys + (lb * W + p) * Hq * D;
    T* kd = k_phys + (lb * W + p) * Hkv * D;
    for (int task = threadIdx.x; task < rot_tasks + copy_tasks; task += kRopeThreads) {
      if (task < rot_tasks) {
        const int head = task / nvec;
        const int j0 = (task % nvec) * N;
        const T* src = head < Hq ? qs + head * D : ks + (head - Hq) * D;
        T* dst = head < Hq ? qd + head * D : kd + (head - Hq) * D;
        if constexpr (VEC) {
          Vec16<T> lo, hi, ylo, yhi;
          lo.raw = *reinterpret_cast<const uint4*>(src + j0);
          hi.raw = *reinterpret_cast<const uint4*>(src + j0 + half);
#pragma unroll
          for (int e = 0; e < N; ++e) {
            const float a = Elt<T>::load(&lo.e[e]);
            const float h = Elt<T>::load(&hi.e[e]);
            const float c = cs[j0 + e], s = sn[j0 + e];
            Elt<T>::store(&ylo.e[e], a * c - h * s);
            Elt<T>::store(&yhi.e[e], h * c + a * s);
          }
          *reinterpret_cast<uint4*>(dst + j0) = ylo.raw;
          *reinterpret_cast<uint4*>(dst + j0 + half) = yhi.raw;
        } else {
          const float a = Elt<T>::load(src + j0);
          const float h = Elt<T>::load(src + j0 + half);
          const float c = cs[j0], s = sn[j0];
          Elt<T>::store(dst + j0, a * c - h * s);
          Elt<T>::store(dst + j0 + half, h * c + a * s);
        }
      } else {
        const int e0 = (task - rot_tasks) * N;  // element offset inside the Hkv*D row
        const T* vs = v + (lb * W + slot) * Hkv * D + e0;
        T* vd = v_phys + (lb * W + p) * Hkv * D + e0;
        if constexpr (VEC) {
          *reinterpret_cast<uint4*>(vd) = *reinterpret_cast<const uint4*>(vs);
        } else {
          *vd = *vs;
        }
      }
    }
  }
}

template <typename T>
static void launch_rope(int n_layers, int B, int W, int Hq, int Hkv, int D, double theta,
                        const void* q, const void* k, const void* v, const int32_t* perm,
                        const int32_t* pos, void* q_phys, void* k_phys, void* v_phys,
                        hipStream_t stream) {
  const dim3 grid(W, B, ceil_div(n_layers, kRopeLayersPerBlock));
  const double log2_theta = log2(theta);
  const bool vec = ((D / 2) % Vec16<T>::N) == 0;
  auto args = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kRopeThreads), 0, stream, n_layers, B, W, Hq, Hkv, D,
                       log2_theta, static_cast<const T*>(q), static_cast<const T*>(k),
                       static_cast<const T*>(v), perm, pos, static_cast<T*>(q_phys),
                       static_cast<T*>(k_phys), static_cast<T*>(v_phys));
  };
  if (vec)
    args(k_rope_logical<T, true>);
  else
    args(k_rope_logical<T, false>);
}

}  // namespace wedlm

extern "C" int wedlm_rope_logical(int dtype, int n_layers, int B, int W, int Hq, int Hkv, int D,
                                  double theta, const void* q, const void* k, const void* v,
                                  const int32_t* perm, const int32_t* pos, void* q_phys,
                                  void* k_phys, void* v_phys, void* stream) {
  using namespace wedlm;
  if (!valid_dtype(dtype)) return WEDLM_ERR_UNSUPPORTED;
  if (n_layers <= 0 || B <= 0 || W <= 0 || W > WEDLM_MAX_WINDOW || Hq <= 0 || Hkv <= 0 || D <= 0)
    return WEDLM_ERR_INVALID;
  if (Hq % Hkv != 0 || D % 2 != 0 || !(theta > 0.0)) return WEDLM_ERR_INVALID;
  if (D > 256) return WEDLM_ERR_UNSUPPORTED;
  if (!q || !k || !v || !perm || !pos || !q_phys || !k_phys || !v_phys) return WEDLM_ERR_INVALID;
  if (B > 65535 || n_layers > 65535 * kRopeLayersPerBlock) return WEDLM_ERR_UNSUPPORTED;
  if (dtype == WEDLM_BF16)
    launch_rope<uint16_t>(n_layers, B, W, Hq, Hkv, D, theta, q, k, v, perm, pos, q_phys, k_phys,
                          v_phys, as_stream(stream));
  else
    launch_rope<float>(n_layers, B, W, Hq, Hkv, D, theta, q, k, v, perm, pos, q_phys, k_phys,
                       v_phys, as_stream(stream));
  return launch_status();
}
