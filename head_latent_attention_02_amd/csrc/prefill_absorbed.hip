// Absorbed-form prefill: the setup that lets the split-KV decode kernels run
// every query row of a forward pass as its own sequence.
//
// In the absorbed form ("A Training-Memory Regression in MLA Sequence
// Parallelism ... LAGA" (Pith review), Fig. 2 "Absorbed (B2)") a query is
// carried into latent space and attends to the latent rows c_kv || R(k_pe)
// directly, with the latent rows as values; the per-head output is the
// merged latent accumulator times the value part of W_kv_b.  That is the
// decode step's arithmetic with one query per sequence, so the prefill
// reuses it: query row i of batch entry b becomes sequence b * Sq + i, all
// rows of one batch entry share that entry's latent rows, and a row's causal
// limit becomes its cache length.  This file builds those latent rows and
// the per-row lengths and RoPE positions.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace {

// rotate-half RoPE of a key pair at an absolute position; the angle is formed
// and reduced to [-pi, pi] in fp64 so that large positions keep their
// accuracy, then rotated with the fp32 sine and cosine of the reduced angle
__device__ __forceinline__ void rope_sc(double pos, int m, int dr, float base, float& s, float& c) {
  constexpr double TWO_PI_HI = 6.283185307179586, TWO_PI_LO = 2.4492935982947064e-16;
  const double theta = exp(-2.0 * (double)m / (double)dr * log((double)base));
  const double ang = pos * theta;
  const double k = rint(ang * (1.0 / TWO_PI_HI));
  sincosf((float)fma(-k, TWO_PI_LO, fma(-k, TWO_PI_HI, ang)), &s, &c);
}

template <mla_dtype DT>
__global__ void __launch_bounds__(256)
latent_cache_kernel(ExplicitArgs a, void* __restrict__ cache, int32_t* __restrict__ cache_len,
                    int64_t* __restrict__ q_pos) {
  const int dlat = a.dkv + a.dr, half = a.dr / 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // latent rows [B, Skv, dkv + dr]: c_kv copied, k_pe rotated at kv_pos0 + j
  const int64_t n_elem = (int64_t)a.B * a.Skv * dlat;
  for (int64_t e = first; e < n_elem; e += stride) {
    const int64_t r = e / dlat;
    const int c = (int)(e - r * dlat);
    float v;
    if (c < a.dkv) {
      v = load_elem<DT>(a.c_kv, r * a.dkv + c);
    } else {
      const int m = c - a.dkv, mp = m < half ? m : m - half;
      const int64_t j = r % a.Skv;
      float s, co;
      rope_sc((double)(a.kv_pos0 + j), mp, a.dr, a.rope_base, s, co);
      const float lo = load_elem<DT>(a.k_pe, r * a.dr + mp), hi = load_elem<DT>(a.k_pe, r * a.dr + mp + half);
      v = m < half ? lo * co - hi * s : hi * co + lo * s;
    }
    store_elem<DT>(cache, e, v);
  }
  // per query row: visible keys (a prefix of the entry's rows) and position
  const int64_t n_rows = (int64_t)a.B * a.Sq;
  for (int64_t e = first; e < n_rows; e += stride) {
    const int64_t i = e % a.Sq;
    int64_t lim = a.Skv;
    if (a.causal) lim = max((int64_t)0, min(a.q_pos0 + i - a.kv_pos0 + 1, (int64_t)a.Skv));
    cache_len[e] = (int32_t)lim;
    q_pos[e] = a.q_pos0 + i;
  }
}

}  // namespace

hipError_t launch_latent_cache(const ExplicitArgs& a, void* cache, int32_t* cache_len, int64_t* q_pos,
                               hipStream_t stream) {
  const int64_t n = std::max((int64_t)a.B * a.Skv * (a.dkv + a.dr), (int64_t)a.B * a.Sq);
  if (n == 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 8192);
  if (a.in_dt == MLA_BF16)
    hipLaunchKernelGGL(latent_cache_kernel<MLA_BF16>, dim3(blocks), dim3(256), 0, stream, a, cache, cache_len,
                       q_pos);
  else
    hipLaunchKernelGGL(latent_cache_kernel<MLA_FP32>, dim3(blocks), dim3(256), 0, stream, a, cache, cache_len,
                       q_pos);
  return hipGetLastError();
}
