// SIMT (fp32 arithmetic) explicit-form MLA forward.  It serves any head
// geometry the MFMA kernels do not cover and the fp32 storage dtype, with fp32
// accumulation throughout.  Steps follow the explicit form of "A
// Training-Memory Regression in MLA Sequence Parallelism ... LAGA" (Pith
// review), "What carries the argument" and Fig. 2: up-project the latent into
// per-head K_nope / V, rotate the RoPE bands, causal softmax attention.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int UP_TILE = 64;   // output tile (rows x cols) of the up-projection
constexpr int UP_K = 16;      // reduction step

// C[j, n] = sum_c c_kv[b, j, c] * W[n, c] for j < s_vis, n < H*(dn+dv);
// column n of head h = n / (dn+dv) goes to Kn (first dn) or V (rest).
template <mla_dtype DT>
__global__ void __launch_bounds__(256)
simt_upproj_kernel(const void* __restrict__ c_kv, const void* __restrict__ w, float* __restrict__ kn,
                   float* __restrict__ v, int Skv, int s_vis, int H, int dkv, int dn, int dv) {
  __shared__ float As[UP_K][UP_TILE + 1];
  __shared__ float Bs[UP_K][UP_TILE + 1];
  const int b = blockIdx.z;
  const int j0 = blockIdx.y * UP_TILE;
  const int n0 = blockIdx.x * UP_TILE;
  const int N = H * (dn + dv);
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  const int64_t cbase = (int64_t)b * Skv * dkv;
  for (int k0 = 0; k0 < dkv; k0 += UP_K) {
    for (int e = threadIdx.x; e < UP_K * UP_TILE; e += 256) {
      int r = e / UP_K, kk = e % UP_K;
      int j = j0 + r, n = n0 + r, k = k0 + kk;
      As[kk][r] = (j < s_vis && k < dkv) ? load_elem<DT>(c_kv, cbase + (int64_t)j * dkv + k) : 0.f;
      Bs[kk][r] = (n < N && k < dkv) ? load_elem<DT>(w, (int64_t)n * dkv + k) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < UP_K; ++kk) {
      float a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int i = 0; i < 4; ++i) bb[i] = Bs[kk][tx * 4 + i];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] += a[i] * bb[q];
    }
    __syncthreads();
  }
  const int dh = dn + dv;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int j = j0 + ty * 4 + i;
    if (j >= s_vis) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int n = n0 + tx * 4 + q;
      if (n >= N) continue;
      int h = n / dh, m = n % dh;
      int64_t bh = (int64_t)b * H + h;
      if (m < dn) kn[(bh * s_vis + j) * dn + m] = acc[i][q];
      else v[(bh * s_vis + j) * dv + (m - dn)] = acc[i][q];
    }
  }
}

// krot[b, j, :] = R(k_pe[b, j, :], kv_pos0 + j) using the k table.
template <mla_dtype DT>
__global__ void simt_krot_kernel(const void* __restrict__ k_pe, const float2* __restrict__ ktab,
                                 float* __restrict__ krot, int Skv, int s_vis, int dr) {
  const int half = dr / 2;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int b = blockIdx.y;
  if (idx >= (int64_t)s_vis * half) return;
  int j = (int)(idx / half), m = (int)(idx % half);
  int64_t src = ((int64_t)b * Skv + j) * dr;
  float lo = load_elem<DT>(k_pe, src + m), hi = load_elem<DT>(k_pe, src + m + half);
  float2 cs = ktab[(int64_t)j * half + m];
  int64_t dst = ((int64_t)b * s_vis + j) * dr;
  krot[dst + m] = lo * cs.x - hi * cs.y;
  krot[dst + m + half] = hi * cs.x + lo * cs.y;
}

constexpr int AT_Q = 16;   // query rows per block
constexpr int AT_K = 16;   // keys per tile

// One block per (16 query rows, head, batch).  Online softmax over key tiles.
template <mla_dtype DT, mla_dtype OT>
__global__ void __launch_bounds__(256)
simt_attention_kernel(ExplicitArgs a, const float* __restrict__ kn, const float* __restrict__ v,
                      const float* __restrict__ krot, const float2* __restrict__ qtab) {
  extern __shared__ float smem[];
  const int dqk = a.dn + a.dr, dv = a.dv, half = a.dr / 2;
  float* Qs = smem;                       // [AT_Q][dqk]
  float* Ks = Qs + AT_Q * dqk;            // [AT_K][dqk]
  float* Vs = Ks + AT_K * dqk;            // [AT_K][dv]
  float* Os = Vs + AT_K * dv;             // [AT_Q][dv]
  float* Ss = Os + AT_Q * dv;             // [AT_Q][AT_K]
  float* Ms = Ss + AT_Q * AT_K;           // [AT_Q]
  float* Ls = Ms + AT_Q;                  // [AT_Q]
  float* Al = Ls + AT_Q;                  // [AT_Q]

  const int i0 = blockIdx.x * AT_Q, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t bh = (int64_t)b * a.H + h;

  // Q rows: [q_nope ; R(q_pe, q_pos0 + i)]
  for (int e = tid; e < AT_Q * dqk; e += 256) {
    int r = e / dqk, d = e % dqk, i = i0 + r;
    float val = 0.f;
    if (i < a.Sq) {
      int64_t row = ((int64_t)b * a.Sq + i) * a.H + h;
      if (d < a.dn) {
        val = load_elem<DT>(a.q_nope, row * a.dn + d);
      } else {
        int m = d - a.dn, mm = m % half;
        float lo = load_elem<DT>(a.q_pe, row * a.dr + mm);
        float hi = load_elem<DT>(a.q_pe, row * a.dr + mm + half);
        float2 cs = qtab[(int64_t)i * half + mm];
        val = (m < half) ? lo * cs.x - hi * cs.y : hi * cs.x + lo * cs.y;
      }
    }
    Qs[e] = val;
  }
  for (int e = tid; e < AT_Q * dv; e += 256) Os[e] = 0.f;
  if (tid < AT_Q) { Ms[tid] = -INFINITY; Ls[tid] = 0.f; }
  __syncthreads();

  // keys visible to the last query row of this block
  int i_last = min(i0 + AT_Q, a.Sq) - 1;
  int64_t kend64 = a.causal ? (a.q_pos0 + i_last - a.kv_pos0 + 1) : (int64_t)a.Skv;
  int kend = (int)max((int64_t)0, min(kend64, (int64_t)a.s_vis));

  for (int j0 = 0; j0 < kend; j0 += AT_K) {
    for (int e = tid; e < AT_K * dqk; e += 256) {
      int r = e / dqk, d = e % dqk, j = j0 + r;
      float val = 0.f;
      if (j < kend) val = (d < a.dn) ? kn[(bh * a.s_vis + j) * a.dn + d]
                                     : krot[((int64_t)b * a.s_vis + j) * a.dr + (d - a.dn)];
      Ks[e] = val;
    }
    for (int e = tid; e < AT_K * dv; e += 256) {
      int r = e / dv, d = e % dv, j = j0 + r;
      Vs[e] = (j < kend) ? v[(bh * a.s_vis + j) * dv + d] : 0.f;
    }
    __syncthreads();
    {
      int r = tid / AT_K, c = tid % AT_K;
      int i = i0 + r, j = j0 + c;
      float s = -INFINITY;
      bool vis = (i < a.Sq) && (j < kend) && (!a.causal || a.kv_pos0 + j <= a.q_pos0 + i);
      if (vis) {
        float dot = 0.f;
        for (int d = 0; d < dqk; ++d) dot += Qs[r * dqk + d] * Ks[c * dqk + d];
        s = dot * a.scale;
      }
      Ss[r * AT_K + c] = s;
    }
    __syncthreads();
    if (tid < AT_Q) {
      float m_old = Ms[tid], mx = m_old;
      for (int c = 0; c < AT_K; ++c) mx = fmaxf(mx, Ss[tid * AT_K + c]);
      float alpha = 1.f, sum = 0.f;
      if (mx == -INFINITY) {
        for (int c = 0; c < AT_K; ++c) Ss[tid * AT_K + c] = 0.f;
      } else {
        alpha = (m_old == -INFINITY) ? 0.f : expf(m_old - mx);
        for (int c = 0; c < AT_K; ++c) {
          float s = Ss[tid * AT_K + c];
          float p = (s == -INFINITY) ? 0.f : expf(s - mx);
          Ss[tid * AT_K + c] = p;
          sum += p;
        }
      }
      Ls[tid] = Ls[tid] * alpha + sum;
      Ms[tid] = mx;
      Al[tid] = alpha;
    }
    __syncthreads();
    for (int e = tid; e < AT_Q * dv; e += 256) {
      int r = e / dv, d = e % dv;
      float acc = Os[e] * Al[r];
      for (int c = 0; c < AT_K; ++c) acc += Ss[r * AT_K + c] * Vs[c * dv + d];
      Os[e] = acc;
    }
    __syncthreads();
  }

  for (int e = tid; e < AT_Q * dv; e += 256) {
    int r = e / dv, d = e % dv, i = i0 + r;
    if (i >= a.Sq) continue;
    float l = Ls[r];
    float o = (l > 0.f) ? Os[e] / l : 0.f;
    store_elem<OT>(a.out, (((int64_t)b * a.Sq + i) * a.H + h) * dv + d, o);
  }
  if (a.lse != nullptr && tid < AT_Q && i0 + tid < a.Sq) {
    float l = Ls[tid];
    a.lse[bh * a.Sq + i0 + tid] = (l > 0.f) ? Ms[tid] + logf(l) : -INFINITY;
  }
}

template <mla_dtype DT>
hipError_t launch_simt_explicit_dt(const ExplicitArgs& a, float* kn, float* v, float* krot,
                                   const float2* qtab, const float2* ktab, hipStream_t stream) {
  if (a.s_vis > 0) {
    dim3 grid((a.H * (a.dn + a.dv) + UP_TILE - 1) / UP_TILE, (a.s_vis + UP_TILE - 1) / UP_TILE, a.B);
    hipLaunchKernelGGL(simt_upproj_kernel<DT>, grid, dim3(256), 0, stream, a.c_kv, a.w, kn, v,
                       a.Skv, a.s_vis, a.H, a.dkv, a.dn, a.dv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int64_t n = (int64_t)a.s_vis * (a.dr / 2);
    dim3 g2((unsigned)((n + 255) / 256), a.B);
    hipLaunchKernelGGL(simt_krot_kernel<DT>, g2, dim3(256), 0, stream, a.k_pe, ktab, krot, a.Skv,
                       a.s_vis, a.dr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.Sq == 0) return hipSuccess;
  const int dqk = a.dn + a.dr;
  size_t smem = sizeof(float) * ((size_t)AT_Q * dqk + AT_K * dqk + AT_K * a.dv + AT_Q * a.dv +
                                 AT_Q * AT_K + 3 * AT_Q);
  dim3 grid((a.Sq + AT_Q - 1) / AT_Q, a.H, a.B);
  if (a.out_dt == MLA_BF16)
    hipLaunchKernelGGL((simt_attention_kernel<DT, MLA_BF16>), grid, dim3(256), smem, stream, a, kn, v,
                       krot, qtab);
  else
    hipLaunchKernelGGL((simt_attention_kernel<DT, MLA_FP32>), grid, dim3(256), smem, stream, a, kn, v,
                       krot, qtab);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_simt_explicit(const ExplicitArgs& a, float* kn, float* v, float* krot,
                                const float2* qtab, const float2* ktab, hipStream_t stream) {
  if (a.in_dt == MLA_BF16) return launch_simt_explicit_dt<MLA_BF16>(a, kn, v, krot, qtab, ktab, stream);
  return launch_simt_explicit_dt<MLA_FP32>(a, kn, v, krot, qtab, ktab, stream);
}
