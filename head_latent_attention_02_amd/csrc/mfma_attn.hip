// Causal MLA attention in head dimension on fp16 MFMA (fp32 accumulate).
//
// Computes, per head h and query i,
//   logit_j = softmax_scale * ( [q_nope ; R(q_pe, q_pos0+i)] . [K_nope_j ; R(k_pe_j)] )
//   out_i = sum_j softmax(logit)_j V_j           over keys with kv_pos0+j <= q_pos0+i
// the head-dimension attention of the explicit / LAGA form in "A
// Training-Memory Regression in MLA Sequence Parallelism ... LAGA" (Pith
// review), "What carries the argument" and Fig. 2; the Fig. 5 caption is the
// page's case for a fused (online-softmax) kernel over an eager one.
//
// Layout of the work: a workgroup owns 256 query rows of one (batch, head) and
// 8 waves of 32 rows each.  Each wave keeps its Q^T block (192 x 32) in
// registers as the B operand and computes S^T = K Q^T, so every lane holds one
// query's scores: the row max needs one swap with the partner lane, and the
// rescale of the O^T accumulator (128 x 32) is a per-lane multiply.  P then
// feeds O^T += V^T P^T directly from registers: the keys inside each 16-wide
// reduction step are taken in the order the lanes already hold them, and the
// V^T rows are read from LDS in that same order.  K (64 x 192) and V^T
// (128 x 64) tiles are double-buffered in LDS with a register prefetch of the
// next tile.  Only the diagonal tiles are masked; tiles past a wave's last
// visible key are skipped.  Workgroups are dealt so that all query tiles of
// one head run on the same XCD (its L2 holds that head's K/V), longest first.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int QW = 32;            // query rows per wave
constexpr int NW = 8;             // waves per workgroup
constexpr int QT = QW * NW;       // query rows per workgroup
constexpr int KT = 64;            // keys per tile
constexpr int DN = 128, DR = 64, DQK = 192, DV = 128;
constexpr int KP = DQK + 8;       // K tile pitch (fp16)
constexpr int VP = KT + 12;       // V^T tile pitch (fp16): 8-byte aligned rows, measured
                                  // free of bank conflicts for the 8-byte reads below
constexpr int NTHREADS = NW * 64;
constexpr float RESCALE_TAU = 8.f;   // log2 units

template <mla_dtype OT>
__global__ void __launch_bounds__(NTHREADS)
mfma_attention_kernel(ExplicitArgs a, const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vt,
                      const uint16_t* __restrict__ krot, const float2* __restrict__ qtab, int nqt) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][DV * VP];

  const int P = a.B * a.H;
  const int n = blockIdx.x;
  const int xcd = n & 7, slot = n >> 3;
  const int p = xcd + 8 * (slot / nqt);
  const int qt = nqt - 1 - (slot % nqt);
  if (p >= P) return;
  const int b = p / a.H, h = p % a.H;
  const int64_t bh = (int64_t)b * a.H + h;
  const int i0 = qt * QT;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hb = lane >> 5;
  const int iw0 = i0 + wave * QW;
  const int i = iw0 + l32;                 // this lane's query row
  const bool row_ok = i < a.Sq;

  // ---- Q^T operand in registers (fp16) ------------------------------------
  f16x8_t qf[DQK / 16];
  {
    const int64_t qrow = ((int64_t)b * a.Sq + (row_ok ? i : 0)) * a.H + h;
    const uint16_t* qn = static_cast<const uint16_t*>(a.q_nope) + qrow * DN;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q_pe) + qrow * DR;
#pragma unroll
    for (int ks = 0; ks < DN / 16; ++ks) {
      u32x4_t raw = row_ok ? *reinterpret_cast<const u32x4_t*>(qn + ks * 16 + hb * 8)
                           : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[ks][2 * e] = (_Float16)bf16_bits_to_float((uint16_t)(raw[e] & 0xffff));
        qf[ks][2 * e + 1] = (_Float16)bf16_bits_to_float((uint16_t)(raw[e] >> 16));
      }
    }
    // rope band: elements m = 16*(ks-8) + 8*hb + e of R(q_pe, q_pos0 + i)
#pragma unroll
    for (int ks = DN / 16; ks < DQK / 16; ++ks) {
      const int m0 = 16 * (ks - DN / 16) + 8 * hb;       // 0..56, a run of 8 within one half
      const int mlo = m0 & 31;                            // pair index of the run's first element
      u32x4_t rlo = row_ok ? *reinterpret_cast<const u32x4_t*>(qp + mlo) : u32x4_t{0u, 0u, 0u, 0u};
      u32x4_t rhi = row_ok ? *reinterpret_cast<const u32x4_t*>(qp + mlo + 32) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t wl = rlo[e >> 1], wh = rhi[e >> 1];
        float lo = bf16_bits_to_float((uint16_t)((e & 1) ? (wl >> 16) : (wl & 0xffff)));
        float hi = bf16_bits_to_float((uint16_t)((e & 1) ? (wh >> 16) : (wh & 0xffff)));
        float2 cs = row_ok ? qtab[(int64_t)i * 32 + mlo + e] : make_float2(1.f, 0.f);
        float r = (m0 < 32) ? (lo * cs.x - hi * cs.y) : (hi * cs.x + lo * cs.y);
        qf[ks][e] = (_Float16)r;
      }
    }
  }

  // ---- key range ------------------------------------------------------------
  const int i_last_wg = min(i0 + QT, a.Sq) - 1;
  auto limit = [&](int qi) -> int {        // keys [0, limit) visible to query qi
    if (!a.causal) return a.s_vis;
    int64_t lim = a.q_pos0 + qi - a.kv_pos0 + 1;
    return (int)max((int64_t)0, min(lim, (int64_t)a.s_vis));
  };
  const int kend_wg = limit(i_last_wg);
  const int ntile = (kend_wg + KT - 1) / KT;
  const bool wave_has_rows = iw0 < a.Sq;
  const int kend_w = wave_has_rows ? limit(min(iw0 + QW, a.Sq) - 1) : 0;
  const int kfull_w = wave_has_rows ? limit(iw0) : 0;
  const int lim_i = row_ok ? limit(i) : 0;

  // ---- tile loads: 5 chunks of 16 B per thread -------------------------------
  const uint16_t* kn_bh = kn + bh * (int64_t)a.s_pad * DN;
  const uint16_t* vt_bh = vt + bh * (int64_t)DV * a.s_pad;
  const uint16_t* kr_b = krot + (int64_t)b * a.s_pad * DR;
  u32x4_t pre[5];
  auto gload = [&](int j0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int q = tid + NTHREADS * u;
      int row = q >> 4, c16 = q & 15;
      pre[u] = *reinterpret_cast<const u32x4_t*>(kn_bh + (int64_t)(j0 + row) * DN + c16 * 8);
    }
    {
      int row = tid >> 3, c = tid & 7;
      pre[2] = *reinterpret_cast<const u32x4_t*>(kr_b + (int64_t)(j0 + row) * DR + c * 8);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int q = tid + NTHREADS * u;
      int row = q >> 3, c = q & 7;
      pre[3 + u] = *reinterpret_cast<const u32x4_t*>(vt_bh + (int64_t)row * a.s_pad + j0 + c * 8);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int q = tid + NTHREADS * u;
      int row = q >> 4, c16 = q & 15;
      *reinterpret_cast<u32x4_t*>(&Ks[buf][row * KP + c16 * 8]) = pre[u];
    }
    {
      int row = tid >> 3, c = tid & 7;
      *reinterpret_cast<u32x4_t*>(&Ks[buf][row * KP + DN + c * 8]) = pre[2];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int q = tid + NTHREADS * u;
      int row = q >> 3, c = q & 7;
      u32x2_t* dst = reinterpret_cast<u32x2_t*>(&Vs[buf][row * VP + c * 8]);
      dst[0] = u32x2_t{pre[3 + u][0], pre[3 + u][1]};
      dst[1] = u32x2_t{pre[3 + u][2], pre[3 + u][3]};
    }
  };

  const float c_log2 = a.scale * MLA_LOG2E;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t oacc[DV / 32];
#pragma unroll
  for (int v = 0; v < DV / 32; ++v)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[v][e] = 0.f;

  if (ntile > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int t = 0; t < ntile; ++t) {
    const int j0 = t * KT;
    const int buf = t & 1;
    if (t + 1 < ntile) gload(j0 + KT);

    if (j0 < kend_w) {
      const bool masked = (j0 + KT > kfull_w);
      f32x16_t sacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < DQK / 16; ++ks) {
          f16x8_t kf = *reinterpret_cast<const f16x8_t*>(&Ks[buf][(kt * 32 + l32) * KP + ks * 16 + hb * 8]);
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], sacc[kt], 0, 0, 0);
        }
      }
      // scale (log2 domain), mask, row max
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = sacc[kt][e] * c_log2;
          if (masked) {
            int j = j0 + kt * 32 + 8 * (e >> 2) + 4 * hb + (e & 3);
            if (j >= lim_i) x = -INFINITY;
          }
          sacc[kt][e] = x;
          mx = fmaxf(mx, x);
        }
      mx = half_pair_max(mx);
      // The reference max only moves when the tile exceeds it by more than
      // RESCALE_TAU (log2 units); P then stays below 2^RESCALE_TAU and the O^T
      // rescale is skipped on almost every tile.  A row that has seen no
      // visible key keeps m_run = -inf and uses 0 as its reference.
      const bool move = mx > m_run + RESCALE_TAU;
      if (__ballot(move) != 0ull) {
        const float alpha = move ? fast_exp2(m_run - mx) : 1.f;   // 0 when m_run was -inf
        const float m_new = move ? mx : m_run;
        l_run *= alpha;
        m_run = m_new;
#pragma unroll
        for (int v = 0; v < DV / 32; ++v)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[v][e] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float rs = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float pv = fast_exp2(sacc[kt][e] - m_use);
          sacc[kt][e] = pv;
          rs += pv;
        }
      l_run += rs;
      // O^T += V^T P^T
#pragma unroll
      for (int ps = 0; ps < KT / 16; ++ps) {
        const int kt = ps >> 1, g0 = 2 * (ps & 1);
        f16x8_t pf;
#pragma unroll
        for (int u = 0; u < 8; ++u) pf[u] = (_Float16)sacc[kt][4 * (g0 + (u >> 2)) + (u & 3)];
        const int key0 = kt * 32 + 16 * (ps & 1) + 4 * hb;
#pragma unroll
        for (int v = 0; v < DV / 32; ++v) {
          const uint16_t* vrow = &Vs[buf][(v * 32 + l32) * VP + key0];
          f16x4_t lo = *reinterpret_cast<const f16x4_t*>(vrow);
          f16x4_t hi = *reinterpret_cast<const f16x4_t*>(vrow + 8);
          f16x8_t vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[v] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf, oacc[v], 0, 0, 0);
        }
      }
    }

    if (t + 1 < ntile) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ---------------------------------------------------------------
  const float l = half_pair_sum(l_run);
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  if (row_ok) {
    const int64_t orow = (((int64_t)b * a.Sq + i) * a.H + h) * DV;
#pragma unroll
    for (int v = 0; v < DV / 32; ++v)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = v * 32 + 8 * g + 4 * hb;
        float o0 = oacc[v][4 * g] * inv, o1 = oacc[v][4 * g + 1] * inv;
        float o2 = oacc[v][4 * g + 2] * inv, o3 = oacc[v][4 * g + 3] * inv;
        if constexpr (OT == MLA_FP32) {
          *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + orow + d) = f32x4_t{o0, o1, o2, o3};
        } else {
          u32x2_t v2;
          v2[0] = pack_bf16x2(o0, o1);
          v2[1] = pack_bf16x2(o2, o3);
          *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(a.out) + orow + d) = v2;
        }
      }
    if (a.lse != nullptr && hb == 0)
      a.lse[bh * a.Sq + i] = (l > 0.f) ? (m_run + __log2f(l)) * MLA_LN2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_mfma_attention(const ExplicitArgs& a, const uint16_t* kn, const uint16_t* vt,
                                 const uint16_t* krot, const float2* qtab, hipStream_t stream) {
  if (a.Sq == 0) return hipSuccess;
  const int P = a.B * a.H;
  const int nqt = (a.Sq + QT - 1) / QT;
  const int P8 = (P + 7) & ~7;
  dim3 grid((unsigned)(P8 * nqt));
  if (a.out_dt == MLA_BF16)
    hipLaunchKernelGGL(mfma_attention_kernel<MLA_BF16>, grid, dim3(NTHREADS), 0, stream, a, kn, vt, krot,
                       qtab, nqt);
  else
    hipLaunchKernelGGL(mfma_attention_kernel<MLA_FP32>, grid, dim3(NTHREADS), 0, stream, a, kn, vt, krot,
                       qtab, nqt);
  return hipGetLastError();
}
