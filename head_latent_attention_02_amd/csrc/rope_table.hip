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
