// SIMT (fp32 arithmetic) backward of the explicit-form MLA forward: the
// gradient of sum(d_out * out) with respect to q_nope, q_pe, c_kv, k_pe and
// W_kv_b.  The training setting of "A Training-Memory Regression in MLA
// Sequence Parallelism ... LAGA" (Pith review): "If this is right" (equal
// parameter gradients for LAGA and the explicit form) and the Fig. 5 caption.
//
// Every kernel computes one output element (or one rotated pair) by a plain
// loop over its reduction, from the definitions:
//   P_ij = exp(s_ij - LSE_i) on visible keys (0 elsewhere), s from the forward
//   dP_ij = dO_i . V_j,  D_i = dO_i . O_i,  dS_ij = P_ij (dP_ij - D_i)
//   dq_nope_i = sigma sum_j dS_ij K_j,   dq_pe_i = R^T(sigma sum_j dS_ij krot_j)
//   dK_j = sigma sum_i dS_ij q_nope_i,   dV_j = sum_i P_ij dO_i
//   dk_pe_j = R^T(sigma sum_h sum_i dS_ij qrot_i)
//   dc_kv_j = sum_h W_UK[h]^T dK_j + W_UV[h]^T dV_j,  dW rows = sum_j dKV_j c_j^T
// where R^T, the transpose of the RoPE rotation, rotates by the negative
// angle.  It keeps P and dS for every (head, query, visible key), so it is
// meant for small problems and for head geometries the MFMA path does not
// take.
#include "common.h"
#include "kernels.h"

namespace {

__device__ __forceinline__ bool visible(const ExplicitArgs& f, int i, int j) {
  return !f.causal || f.kv_pos0 + j <= f.q_pos0 + i;
}

// qrot[b, i, h, :] = R(q_pe[b, i, h, :], q_pos0 + i)
template <mla_dtype DT>
__global__ void qrot_kernel(ExplicitArgs f, const float2* __restrict__ qtab, float* __restrict__ qrot) {
  const int half = f.dr / 2;
  const int64_t n = (int64_t)f.B * f.Sq * f.H * half;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int m = (int)(idx % half);
  const int64_t row = idx / half;                  // (b, i, h)
  const int i = (int)((row / f.H) % f.Sq);
  const float lo = load_elem<DT>(f.q_pe, row * f.dr + m), hi = load_elem<DT>(f.q_pe, row * f.dr + m + half);
  const float2 cs = qtab[(int64_t)i * half + m];
  qrot[row * f.dr + m] = lo * cs.x - hi * cs.y;
  qrot[row * f.dr + m + half] = hi * cs.x + lo * cs.y;
}

// P and dS of one (b, h, i, j), j < s_vis
template <mla_dtype DT, mla_dtype OT>
__global__ void p_ds_kernel(BackwardArgs a, SimtBwdWorkspace w) {
  const ExplicitArgs& f = a.f;
  const int64_t n = (int64_t)f.B * f.H * f.Sq * f.s_vis;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int j = (int)(idx % f.s_vis);
  const int64_t bhi = idx / f.s_vis;
  const int i = (int)(bhi % f.Sq);
  const int64_t bh = bhi / f.Sq;
  const int h = (int)(bh % f.H), b = (int)(bh / f.H);
  const float lse = a.lse[bh * f.Sq + i];
  float p = 0.f, ds = 0.f;
  if (visible(f, i, j) && lse != -INFINITY) {
    const int64_t qrow = ((int64_t)b * f.Sq + i) * f.H + h;
    float s = 0.f;
    for (int d = 0; d < f.dn; ++d) s += load_elem<DT>(f.q_nope, qrow * f.dn + d) * w.kn[(bh * f.s_vis + j) * f.dn + d];
    for (int d = 0; d < f.dr; ++d) s += w.qrot[qrow * f.dr + d] * w.krot[((int64_t)b * f.s_vis + j) * f.dr + d];
    p = expf(s * f.scale - lse);
    float dp = 0.f, dd = 0.f;
    for (int d = 0; d < f.dv; ++d) {
      const float g = load_elem<OT>(a.d_out, qrow * f.dv + d);
      dp += g * w.v[(bh * f.s_vis + j) * f.dv + d];
      dd += g * load_elem<OT>(a.out, qrow * f.dv + d);
    }
    ds = p * (dp - dd);
  }
  w.p[idx] = p;
  w.ds[idx] = ds;
}

// dq_nope[b, i, h, d] = sigma sum_j dS K_nope
__global__ void dq_nope_kernel(BackwardArgs a, SimtBwdWorkspace w) {
  const ExplicitArgs& f = a.f;
  const int64_t n = (int64_t)f.B * f.Sq * f.H * f.dn;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int d = (int)(idx % f.dn);
  const int64_t row = idx / f.dn;                  // (b, i, h)
  const int h = (int)(row % f.H);
  const int i = (int)((row / f.H) % f.Sq), b = (int)(row / ((int64_t)f.H * f.Sq));
  const int64_t bh = (int64_t)b * f.H + h;
  const float* ds = w.ds + (bh * f.Sq + i) * f.s_vis;
  float acc = 0.f;
  for (int j = 0; j < f.s_vis; ++j) acc += ds[j] * w.kn[(bh * f.s_vis + j) * f.dn + d];
  a.dq_nope[idx] = f.scale * acc;
}

// dq_pe[b, i, h, (m, m + half)] = R^T(sigma sum_j dS krot_j) at q_pos0 + i
__global__ void dq_pe_kernel(BackwardArgs a, SimtBwdWorkspace w) {
  const ExplicitArgs& f = a.f;
  const int half = f.dr / 2;
  const int64_t n = (int64_t)f.B * f.Sq * f.H * half;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int m = (int)(idx % half);
  const int64_t row = idx / half;
  const int h = (int)(row % f.H);
  const int i = (int)((row / f.H) % f.Sq), b = (int)(row / ((int64_t)f.H * f.Sq));
  const int64_t bh = (int64_t)b * f.H + h;
  const float* ds = w.ds + (bh * f.Sq + i) * f.s_vis;
  float lo = 0.f, hi = 0.f;
  for (int j = 0; j < f.s_vis; ++j) {
    const float* kr = w.krot + ((int64_t)b * f.s_vis + j) * f.dr;
    lo += ds[j] * kr[m];
    hi += ds[j] * kr[m + half];
  }
  lo *= f.scale;
  hi *= f.scale;
  const float2 cs = w.qtab[(int64_t)i * half + m];
  a.dq_pe[row * f.dr + m] = lo * cs.x + hi * cs.y;
  a.dq_pe[row * f.dr + m + half] = hi * cs.x - lo * cs.y;
}

// dKn[b, h, j, d] = sigma sum_i dS q_nope;  dV[b, h, j, d] = sum_i P dO
template <mla_dtype DT, mla_dtype OT>
__global__ void dk_dv_kernel(BackwardArgs a, SimtBwdWorkspace w) {
  const ExplicitArgs& f = a.f;
  const int dkv = f.dn + f.dv;
  const int64_t n = (int64_t)f.B * f.H * f.s_vis * dkv;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int d = (int)(idx % dkv);
  const int64_t bhj = idx / dkv;
  const int j = (int)(bhj % f.s_vis);
  const int64_t bh = bhj / f.s_vis;
  const int h = (int)(bh % f.H), b = (int)(bh / f.H);
  float acc = 0.f;
  for (int i = 0; i < f.Sq; ++i) {
    const int64_t qrow = ((int64_t)b * f.Sq + i) * f.H + h;
    const int64_t e = (bh * f.Sq + i) * f.s_vis + j;
    if (d < f.dn) acc += w.ds[e] * load_elem<DT>(f.q_nope, qrow * f.dn + d);
    else acc += w.p[e] * load_elem<OT>(a.d_out, qrow * f.dv + (d - f.dn));
  }
  if (d < f.dn) w.dkn[bhj * f.dn + d] = f.scale * acc;
  else w.dv[bhj * f.dv + (d - f.dn)] = acc;
}

// dk_pe[b, j, (m, m + half)] = R^T(sigma sum_h sum_i dS qrot) at kv_pos0 + j;
// zero for rows no query sees
__global__ void dk_pe_kernel(BackwardArgs a, SimtBwdWorkspace w) {
  const ExplicitArgs& f = a.f;
  const int half = f.dr / 2;
  const int64_t n = (int64_t)f.B * f.Skv * half;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int m = (int)(idx % half);
  const int64_t bj = idx / half;
  const int j = (int)(bj % f.Skv), b = (int)(bj / f.Skv);
  float lo = 0.f, hi = 0.f;
  if (j < f.s_vis) {
    for (int h = 0; h < f.H; ++h) {
      const int64_t bh = (int64_t)b * f.H + h;
      for (int i = 0; i < f.Sq; ++i) {
        const float ds = w.ds[(bh * f.Sq + i) * f.s_vis + j];
        const float* qr = w.qrot + (((int64_t)b * f.Sq + i) * f.H + h) * f.dr;
        lo += ds * qr[m];
        hi += ds * qr[m + half];
      }
    }
    lo *= f.scale;
    hi *= f.scale;
    const float2 cs = w.ktab[(int64_t)j * half + m];
    const float l2 = lo * cs.x + hi * cs.y, h2 = hi * cs.x - lo * cs.y;
    lo = l2;
    hi = h2;
  }
  a.dk_pe[bj * f.dr + m] = lo;
  a.dk_pe[bj * f.dr + m + half] = hi;
}

// dc_kv[b, j, c] = sum_h sum_n dKV[b, h, j, n] W[h (dn+dv) + n, c]; zero past s_vis
template <mla_dtype DT>
__global__ void dc_kernel(BackwardArgs a, SimtBwdWorkspace w) {
  const ExplicitArgs& f = a.f;
  const int64_t n = (int64_t)f.B * f.Skv * f.dkv;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int c = (int)(idx % f.dkv);
  const int64_t bj = idx / f.dkv;
  const int j = (int)(bj % f.Skv), b = (int)(bj / f.Skv);
  float acc = 0.f;
  if (j < f.s_vis) {
    const int dh = f.dn + f.dv;
    for (int h = 0; h < f.H; ++h) {
      const int64_t bh = (int64_t)b * f.H + h;
      for (int m = 0; m < f.dn; ++m)
        acc += w.dkn[(bh * f.s_vis + j) * f.dn + m] * load_elem<DT>(f.w, ((int64_t)h * dh + m) * f.dkv + c);
      for (int m = 0; m < f.dv; ++m)
        acc += w.dv[(bh * f.s_vis + j) * f.dv + m] * load_elem<DT>(f.w, ((int64_t)h * dh + f.dn + m) * f.dkv + c);
    }
  }
  a.dc_kv[idx] = acc;
}

// dW[h (dn+dv) + m, c] = sum_b sum_j dKV[b, h, j, m] c_kv[b, j, c]
template <mla_dtype DT>
__global__ void dw_kernel(BackwardArgs a, SimtBwdWorkspace w) {
  const ExplicitArgs& f = a.f;
  const int dh = f.dn + f.dv;
  const int64_t n = (int64_t)f.H * dh * f.dkv;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int c = (int)(idx % f.dkv);
  const int64_t r = idx / f.dkv;
  const int h = (int)(r / dh), m = (int)(r % dh);
  float acc = 0.f;
  for (int b = 0; b < f.B; ++b) {
    const int64_t bh = (int64_t)b * f.H + h;
    for (int j = 0; j < f.s_vis; ++j) {
      const float g = m < f.dn ? w.dkn[(bh * f.s_vis + j) * f.dn + m] : w.dv[(bh * f.s_vis + j) * f.dv + (m - f.dn)];
      acc += g * load_elem<DT>(f.c_kv, ((int64_t)b * f.Skv + j) * f.dkv + c);
    }
  }
  a.dw[idx] = acc;
}

dim3 grid_for(int64_t n) { return dim3((unsigned)((n + 255) / 256)); }

template <mla_dtype DT, mla_dtype OT>
hipError_t launch_dt(const BackwardArgs& a, const SimtBwdWorkspace& w, hipStream_t s) {
  const ExplicitArgs& f = a.f;
  const int half = f.dr / 2;
  hipError_t e;
#define MLA_LAUNCH(kern, n)                                                       \
  do {                                                                            \
    const int64_t n_ = (n);                                                       \
    if (n_ > 0) {                                                                 \
      hipLaunchKernelGGL(kern, grid_for(n_), dim3(256), 0, s, a, w);              \
      if ((e = hipGetLastError()) != hipSuccess) return e;                        \
    }                                                                             \
  } while (0)
  if ((int64_t)f.B * f.Sq * f.H * half > 0) {
    hipLaunchKernelGGL(qrot_kernel<DT>, grid_for((int64_t)f.B * f.Sq * f.H * half), dim3(256), 0, s, f, w.qtab,
                       w.qrot);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  MLA_LAUNCH((p_ds_kernel<DT, OT>), (int64_t)f.B * f.H * f.Sq * f.s_vis);
  MLA_LAUNCH(dq_nope_kernel, (int64_t)f.B * f.Sq * f.H * f.dn);
  MLA_LAUNCH(dq_pe_kernel, (int64_t)f.B * f.Sq * f.H * half);
  MLA_LAUNCH((dk_dv_kernel<DT, OT>), (int64_t)f.B * f.H * f.s_vis * (f.dn + f.dv));
  MLA_LAUNCH(dk_pe_kernel, (int64_t)f.B * f.Skv * half);
  MLA_LAUNCH(dc_kernel<DT>, (int64_t)f.B * f.Skv * f.dkv);
  MLA_LAUNCH(dw_kernel<DT>, (int64_t)f.H * (f.dn + f.dv) * f.dkv);
#undef MLA_LAUNCH
  return hipSuccess;
}

}  // namespace

hipError_t launch_simt_backward(const BackwardArgs& a, const SimtBwdWorkspace& w, hipStream_t stream) {
  const bool in_bf16 = a.f.in_dt == MLA_BF16, out_bf16 = a.f.out_dt == MLA_BF16;
  if (in_bf16) return out_bf16 ? launch_dt<MLA_BF16, MLA_BF16>(a, w, stream) : launch_dt<MLA_BF16, MLA_FP32>(a, w, stream);
  return out_bf16 ? launch_dt<MLA_FP32, MLA_BF16>(a, w, stream) : launch_dt<MLA_FP32, MLA_FP32>(a, w, stream);
}
