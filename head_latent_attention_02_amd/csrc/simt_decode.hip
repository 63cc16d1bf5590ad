// SIMT (fp32 arithmetic) absorbed split-KV decode: query absorption and the
// per-chunk partial attention.  Steps follow the absorbed form of "A
// Training-Memory Regression in MLA Sequence Parallelism ... LAGA" (Pith
// review), Fig. 2 "Absorbed (B2)", and the chunk partials plus log-sum-exp of
// "Helix Parallelism ..." (Pith review), "What carries the argument".
#include "common.h"
#include "kernels.h"

namespace {

// q~[b,h,c] = sum_n W[h*(dn+dv)+n, c] q_nope[b,h,n] for c < dkv;
// q~[b,h,dkv+m] = R(q_pe[b,h], L_b - 1)[m].  One block per (b, h).
template <mla_dtype DT>
__global__ void __launch_bounds__(256)
simt_absorb_kernel(DecodeArgs a, float* __restrict__ qt) {
  extern __shared__ float qs[];  // [dn]
  const int b = blockIdx.y, h = blockIdx.x;
  const int64_t bh = (int64_t)b * a.H + h;
  const int dlat = a.dkv + a.dr, half = a.dr / 2;
  for (int n = threadIdx.x; n < a.dn; n += blockDim.x) qs[n] = load_elem<DT>(a.q_nope, bh * a.dn + n);
  __syncthreads();
  const int64_t wrow = (int64_t)h * (a.dn + a.dv);
  for (int c = threadIdx.x; c < a.dkv; c += blockDim.x) {
    float acc = 0.f;
    for (int n = 0; n < a.dn; ++n) acc += load_elem<DT>(a.w, (wrow + n) * a.dkv + c) * qs[n];
    qt[bh * dlat + c] = acc;
  }
  int L = min(max(a.cache_len[b], 0), a.max_len);
  double pos = a.q_pos != nullptr ? (double)a.q_pos[b] : (double)(L > 0 ? L - 1 : 0);
  for (int m = threadIdx.x; m < half; m += blockDim.x) {
    double theta = exp(-2.0 * (double)m / (double)a.dr * log((double)a.rope_base));
    double s, c;
    sincos(pos * theta, &s, &c);
    float lo = load_elem<DT>(a.q_pe, bh * a.dr + m), hi = load_elem<DT>(a.q_pe, bh * a.dr + m + half);
    qt[bh * dlat + a.dkv + m] = lo * (float)c - hi * (float)s;
    qt[bh * dlat + a.dkv + m + half] = hi * (float)c + lo * (float)s;
  }
}

constexpr int SK_T = 256;  // tokens per tile

// One block per (head, chunk, batch): online softmax over the chunk's tokens.
template <mla_dtype DT>
__global__ void __launch_bounds__(256)
simt_splitkv_kernel(DecodeArgs a, const float* __restrict__ qt, float* __restrict__ lse_part,
                    float* __restrict__ o_part) {
  extern __shared__ float sm[];
  const int dlat = a.dkv + a.dr;
  float* qs = sm;               // [dlat]
  float* ps = qs + dlat;        // [SK_T]
  float* red = ps + SK_T;       // [8]
  const int h = blockIdx.x, k = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t bh = (int64_t)b * a.H + h;
  int L = min(max(a.cache_len[b], 0), a.max_len);
  int csz = (L + a.n_splits - 1) / a.n_splits;
  int t0 = min(L, k * csz), t1 = min(L, (k + 1) * csz);
  for (int d = tid; d < dlat; d += 256) qs[d] = qt[bh * dlat + d];
  __syncthreads();
  // each thread owns latent columns c = tid + 256*u
  constexpr int MAXU = 4;   // dkv <= 1024
  float acc[MAXU] = {0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const uint8_t* base = static_cast<const uint8_t*>(a.cache);
  const int esz = (DT == MLA_BF16) ? 2 : 4;
  for (int tt = t0; tt < t1; tt += SK_T) {
    int t = tt + tid;
    float s = -INFINITY;
    if (t < t1) {
      const void* row = base + ((int64_t)(b / a.seq_per_cache) * a.cache_stride + (int64_t)t * dlat) * esz;
      float dot = 0.f;
      for (int d = 0; d < dlat; ++d) dot += qs[d] * load_elem<DT>(row, d);
      s = dot * a.scale;
    }
    // block max
    float mx = wave_max(s);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float m_new = fmaxf(m_run, mx);
    float p = (s == -INFINITY) ? 0.f : expf(s - m_new);
    ps[tid] = p;
    float sm_ = wave_sum(p);
    __syncthreads();
    if ((tid & 63) == 0) red[4 + (tid >> 6)] = sm_;
    __syncthreads();
    float tile_sum = red[4] + red[5] + red[6] + red[7];
    float alpha = (m_run == -INFINITY) ? 0.f : expf(m_run - m_new);
    l_run = l_run * alpha + tile_sum;
    m_run = m_new;
    int nt = min(SK_T, t1 - tt);
    for (int u = 0; u < MAXU; ++u) {
      int c = tid + 256 * u;
      if (c >= a.dkv) break;
      float o = acc[u] * alpha;
      for (int q = 0; q < nt; ++q) {
        const void* row = base + ((int64_t)(b / a.seq_per_cache) * a.cache_stride + (int64_t)(tt + q) * dlat) * esz;
        o += ps[q] * load_elem<DT>(row, c);
      }
      acc[u] = o;
    }
    __syncthreads();
  }
  const int64_t pidx = ((int64_t)b * a.n_splits + k) * a.H + h;
  for (int u = 0; u < MAXU; ++u) {
    int c = tid + 256 * u;
    if (c >= a.dkv) break;
    o_part[pidx * a.dkv + c] = (l_run > 0.f) ? acc[u] / l_run : 0.f;
  }
  if (tid == 0) lse_part[pidx] = (l_run > 0.f) ? m_run + logf(l_run) : -INFINITY;
}

}  // namespace

hipError_t launch_simt_absorb(const DecodeArgs& a, float* qt, hipStream_t stream) {
  dim3 grid(a.H, a.B);
  size_t smem = sizeof(float) * a.dn;
  if (a.in_dt == MLA_BF16)
    hipLaunchKernelGGL(simt_absorb_kernel<MLA_BF16>, grid, dim3(256), smem, stream, a, qt);
  else
    hipLaunchKernelGGL(simt_absorb_kernel<MLA_FP32>, grid, dim3(256), smem, stream, a, qt);
  return hipGetLastError();
}

hipError_t launch_simt_splitkv(const DecodeArgs& a, const float* qt, float* lse_part, float* o_part,
                               hipStream_t stream) {
  dim3 grid(a.H, a.n_splits, a.B);
  size_t smem = sizeof(float) * (a.dkv + a.dr + SK_T + 8);
  if (a.in_dt == MLA_BF16)
    hipLaunchKernelGGL(simt_splitkv_kernel<MLA_BF16>, grid, dim3(256), smem, stream, a, qt, lse_part,
                       o_part);
  else
    hipLaunchKernelGGL(simt_splitkv_kernel<MLA_FP32>, grid, dim3(256), smem, stream, a, qt, lse_part,
                       o_part);
  return hipGetLastError();
}
