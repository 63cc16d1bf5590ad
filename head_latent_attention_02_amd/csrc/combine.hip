// Log-sum-exp merge of the split-KV partials followed by the un-absorb
// projection.  The merge rescales each chunk's normalised partial by
// exp(lse_k - lse) and sums, which reproduces the softmax over the whole
// sequence ("Helix Parallelism ..." (Pith review), "What carries the
// argument"); the merged latent accumulator is then mapped to d_v through the
// value part of W_kv_b ("A Training-Memory Regression in MLA Sequence
// Parallelism ... LAGA" (Pith review), Fig. 2 "Absorbed (B2)", un-absorb).
//
// One block per (head, group of CB sequences): the head's W_UV rows are read
// once per group while the group's merged accumulators sit in LDS.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int CB = 8;         // sequences per block
constexpr int CTHREADS = 256;

template <mla_dtype WT, mla_dtype OT>
__global__ void __launch_bounds__(CTHREADS)
combine_kernel(DecodeArgs a, const float* __restrict__ lse_part, const float* __restrict__ o_part) {
  extern __shared__ float olat[];            // [CB][dkv]
  __shared__ float wk[CB][64];               // chunk weights (n_splits <= 64)
  __shared__ float lse_s[CB];
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * CB;
  const int nb = min(CB, a.B - b0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ns = a.n_splits;

  // chunk weights: one wave per sequence
  for (int bi = wave; bi < nb; bi += CTHREADS / 64) {
    int b = b0 + bi;
    float l = (lane < ns) ? lse_part[((int64_t)b * ns + lane) * a.H + h] : -INFINITY;
    float m = wave_max(l);
    float e = (l == -INFINITY) ? 0.f : expf(l - m);
    float tot = wave_sum(e);
    if (lane < ns) wk[bi][lane] = (tot > 0.f) ? e / tot : 0.f;
    if (lane == 0) lse_s[bi] = (tot > 0.f) ? m + logf(tot) : -INFINITY;
  }
  __syncthreads();
  for (int e = tid; e < nb * a.dkv; e += CTHREADS) {
    int bi = e / a.dkv, c = e % a.dkv, b = b0 + bi;
    float acc = 0.f;
    for (int k = 0; k < ns; ++k) {
      float wgt = wk[bi][k];
      if (wgt != 0.f) acc += wgt * o_part[(((int64_t)b * ns + k) * a.H + h) * a.dkv + c];
    }
    olat[bi * a.dkv + c] = acc;
  }
  __syncthreads();
  // out[b,h,v] = W_UV[h][v] . o_lat[b]: one wave per row v, lanes over c
  const int64_t wrow0 = (int64_t)h * (a.dn + a.dv) + a.dn;
  for (int v = wave; v < a.dv; v += CTHREADS / 64) {
    float acc[CB];
#pragma unroll
    for (int bi = 0; bi < CB; ++bi) acc[bi] = 0.f;
    for (int c = lane; c < a.dkv; c += 64) {
      float wv = load_elem<WT>(a.w, (wrow0 + v) * a.dkv + c);
#pragma unroll
      for (int bi = 0; bi < CB; ++bi) acc[bi] += wv * olat[(bi < nb ? bi : 0) * a.dkv + c];
    }
#pragma unroll
    for (int bi = 0; bi < CB; ++bi) {
      float r = wave_sum(acc[bi]);
      if (lane == 0 && bi < nb) store_elem<OT>(a.out, ((int64_t)(b0 + bi) * a.H + h) * a.dv + v, r);
    }
  }
  if (a.lse != nullptr && tid < nb) a.lse[(int64_t)(b0 + tid) * a.H + h] = lse_s[tid];
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, const float* lse_part, const float* o_part,
                          hipStream_t stream) {
  dim3 grid(a.H, (a.B + CB - 1) / CB);
  size_t smem = sizeof(float) * CB * a.dkv;
  if (a.in_dt == MLA_BF16) {
    if (a.out_dt == MLA_BF16)
      hipLaunchKernelGGL((combine_kernel<MLA_BF16, MLA_BF16>), grid, dim3(CTHREADS), smem, stream, a,
                         lse_part, o_part);
    else
      hipLaunchKernelGGL((combine_kernel<MLA_BF16, MLA_FP32>), grid, dim3(CTHREADS), smem, stream, a,
                         lse_part, o_part);
  } else {
    if (a.out_dt == MLA_BF16)
      hipLaunchKernelGGL((combine_kernel<MLA_FP32, MLA_BF16>), grid, dim3(CTHREADS), smem, stream, a,
                         lse_part, o_part);
    else
      hipLaunchKernelGGL((combine_kernel<MLA_FP32, MLA_FP32>), grid, dim3(CTHREADS), smem, stream, a,
                         lse_part, o_part);
  }
  return hipGetLastError();
}
