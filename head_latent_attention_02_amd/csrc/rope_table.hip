// RoPE cos/sin table for the decoupled band (rotate-half pairing, angle =
// position * base^(-2m/d_rope)).  Angles and their sines are formed in fp64 so
// that positions in the tens of thousands keep full fp32 accuracy; the table
// itself is fp32.
#include "common.h"
#include "kernels.h"

__global__ void rope_table_kernel(float2* __restrict__ table, int64_t pos0, int n, int half,
                                  double log_base, int dr) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n * half) return;
  int p = (int)(idx / half);
  int m = (int)(idx % half);
  double theta = exp(-2.0 * (double)m / (double)dr * log_base);
  double ang = (double)(pos0 + p) * theta;
  double s, c;
  sincos(ang, &s, &c);
  table[idx] = make_float2((float)c, (float)s);
}

hipError_t launch_rope_table(float2* table, int64_t pos0, int n, int dr, float base,
                             hipStream_t stream) {
  int half = dr / 2;
  int64_t total = (int64_t)n * half;
  if (total == 0) return hipSuccess;
  int threads = 256;
  int blocks = (int)((total + threads - 1) / threads);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(threads), 0, stream, table, pos0, n,
                     half, log((double)base), dr);
  return hipGetLastError();
}

// The query table and the rotated key band in one launch (the MFMA paths):
// threads [0, nq * half) write the query table; the rest cover (b, j, m) of
// the key band R(k_pe[b, j], kv_pos0 + j) in fp16 for j < s_pad (zeros for
// j >= s_vis), forming each key angle as rope_table_kernel does.  The key
// table is written too (batch entry 0) when ktab is not null.
__global__ void rope_band_kernel(float2* __restrict__ qtab, float2* __restrict__ ktab,
                                 uint16_t* __restrict__ krot, const uint16_t* __restrict__ k_pe, int64_t q_pos0,
                                 int nq, int64_t kv_pos0, int Skv, int s_vis, int s_pad, int nb, double log_base,
                                 int dr) {
  const int half = dr / 2;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nqe = (int64_t)nq * half;
  if (idx < nqe) {
    const int p = (int)(idx / half), m = (int)(idx % half);
    const double theta = exp(-2.0 * (double)m / (double)dr * log_base);
    double s, c;
    sincos((double)(q_pos0 + p) * theta, &s, &c);
    qtab[idx] = make_float2((float)c, (float)s);
    return;
  }
  idx -= nqe;
  if (idx >= (int64_t)nb * s_pad * half) return;
  const int m = (int)(idx % half);
  const int64_t bj = idx / half;
  const int j = (int)(bj % s_pad), b = (int)(bj / s_pad);
  float ylo = 0.f, yhi = 0.f;
  if (j < s_vis) {
    const double theta = exp(-2.0 * (double)m / (double)dr * log_base);
    double s, c;
    sincos((double)(kv_pos0 + j) * theta, &s, &c);
    const float cf = (float)c, sf = (float)s;
    if (ktab != nullptr && b == 0) ktab[(int64_t)j * half + m] = make_float2(cf, sf);
    const int64_t src = ((int64_t)b * Skv + j) * dr;
    const float lo = bf16_bits_to_float(k_pe[src + m]), hi = bf16_bits_to_float(k_pe[src + m + half]);
    ylo = lo * cf - hi * sf;
    yhi = hi * cf + lo * sf;
  }
  const int64_t dst = ((int64_t)b * s_pad + j) * dr;
  krot[dst + m] = float_to_f16_bits(ylo);
  krot[dst + m + half] = float_to_f16_bits(yhi);
}

hipError_t launch_rope_band(const ExplicitArgs& a, float2* qtab, float2* ktab, uint16_t* krot,
                            hipStream_t stream) {
  const int half = a.dr / 2;
  const int64_t total = ((int64_t)a.Sq + (int64_t)a.B * a.s_pad) * half;
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const int blocks = (int)((total + threads - 1) / threads);
  hipLaunchKernelGGL(rope_band_kernel, dim3(blocks), dim3(threads), 0, stream, qtab, ktab, krot,
                     static_cast<const uint16_t*>(a.k_pe), a.q_pos0, a.Sq, a.kv_pos0, a.Skv, a.s_vis, a.s_pad,
                     a.B, log((double)a.rope_base), a.dr);
  return hipGetLastError();
}
