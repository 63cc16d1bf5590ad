// Absorbed split-KV decode on bf16 MFMA: query absorption and the per-chunk
// partial attention over the latent cache.
//
// Absorbed form: "A Training-Memory Regression in MLA Sequence Parallelism ...
// LAGA" (Pith review), "What carries the argument" (the absorbed query is the
// transpose of W_kv_b's key part times q_nope) and Fig. 2 "Absorbed (B2)";
// the cache row is the 576-wide latent plus RoPE band of "TPLA ..." (Pith
// review), "If this is right".  The chunk partials with their log-sum-exp are
// those of "Helix Parallelism ..." (Pith review), "What carries the argument";
// they are merged by the separate combine kernel.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int DC = 512, DRP = 64, DLAT = 576, DN = 128, DV = 128;

// ---------------------------------------------------------------------------
// q~[b,h,:512] = W_UK[h]^T q_nope[b,h] (fp32 accumulate, bf16 result) and
// q~[b,h,512:] = R(q_pe[b,h], L_b - 1).  One block per (head, 16 sequences);
// each thread owns 2 latent columns for the 16 sequences.
constexpr int AB = 16;
__global__ void __launch_bounds__(256)
absorb_bf16_kernel(DecodeArgs a, uint16_t* __restrict__ qt) {
  __shared__ float qs[AB][DN];
  const int h = blockIdx.x, b0 = blockIdx.y * AB;
  const int nb = min(AB, a.B - b0);
  const int tid = threadIdx.x;
  const uint16_t* qn = static_cast<const uint16_t*>(a.q_nope);
  const uint16_t* w = static_cast<const uint16_t*>(a.w);
  for (int e = tid; e < AB * DN; e += 256) {
    int bi = e / DN, n = e % DN;
    qs[bi][n] = (bi < nb) ? bf16_bits_to_float(qn[((int64_t)(b0 + bi) * a.H + h) * DN + n]) : 0.f;
  }
  __syncthreads();
  float acc[AB][2];
#pragma unroll
  for (int bi = 0; bi < AB; ++bi) acc[bi][0] = acc[bi][1] = 0.f;
  const uint16_t* wrow = w + (int64_t)h * (DN + DV) * DC + 2 * tid;
  for (int n = 0; n < DN; ++n) {
    uint32_t w2 = *reinterpret_cast<const uint32_t*>(wrow + (int64_t)n * DC);
    float w0 = bf16_bits_to_float((uint16_t)(w2 & 0xffff)), w1 = bf16_bits_to_float((uint16_t)(w2 >> 16));
#pragma unroll
    for (int bi = 0; bi < AB; ++bi) {
      float q = qs[bi][n];
      acc[bi][0] += q * w0;
      acc[bi][1] += q * w1;
    }
  }
#pragma unroll
  for (int bi = 0; bi < AB; ++bi)
    if (bi < nb)
      *reinterpret_cast<uint32_t*>(qt + ((int64_t)(b0 + bi) * a.H + h) * DLAT + 2 * tid) =
          pack_bf16x2(acc[bi][0], acc[bi][1]);
  // RoPE band of the query at the new token's position
  const uint16_t* qp = static_cast<const uint16_t*>(a.q_pe);
  for (int e = tid; e < nb * 32; e += 256) {
    int bi = e >> 5, m = e & 31, b = b0 + bi;
    int L = min(max(a.cache_len[b], 0), a.max_len);
    double pos = (double)(L > 0 ? L - 1 : 0);
    double theta = exp(-2.0 * (double)m / (double)DRP * log((double)a.rope_base));
    double s, c;
    sincos(pos * theta, &s, &c);
    const int64_t row = (int64_t)b * a.H + h;
    float lo = bf16_bits_to_float(qp[row * DRP + m]), hi = bf16_bits_to_float(qp[row * DRP + m + 32]);
    qt[row * DLAT + DC + m] = float_to_bf16_bits(lo * (float)c - hi * (float)s);
    qt[row * DLAT + DC + m + 32] = float_to_bf16_bits(hi * (float)c + lo * (float)s);
  }
}

// ---------------------------------------------------------------------------
// Split-KV partial attention.  One workgroup per (chunk, sequence), 8 waves;
// wave w owns heads 16w .. 16w+15 (heads beyond H idle).  Per 32-token tile:
//   S^T[t][h] = C[t][:576] . q~[h]      (16x16x32 MFMAs, q~ held in registers)
//   online softmax per head (each lane owns one head of its 16)
//   O^T[d][h] += C^T[d][t] P^T[t][h]    (16x16x32 MFMAs, P from registers)
// The tile is staged twice in LDS: row-major C for the first product and
// transposed C^T (built by a 4x8 register transpose on the way in) for the
// second, both double-buffered with a register prefetch of the next tile.
constexpr int TT = 32;               // tokens per tile
constexpr int CP = DLAT + 8;         // C tile pitch (bf16)
constexpr int CTP = TT + 8;          // C^T tile pitch (bf16)
constexpr int NTHREADS = 512;

__global__ void __launch_bounds__(NTHREADS)
mfma_splitkv_kernel(DecodeArgs a, const uint16_t* __restrict__ qt, float* __restrict__ lse_part,
                    float* __restrict__ o_part) {
  __shared__ __attribute__((aligned(16))) uint16_t Cs[2][TT * CP];
  __shared__ __attribute__((aligned(16))) uint16_t Cts[2][DC * CTP];

  const int k = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int h = wave * 16 + l16;
  const bool wave_active = wave * 16 < a.H;

  const int L = min(max(a.cache_len[b], 0), a.max_len);
  const int csz = (L + a.n_splits - 1) / a.n_splits;
  const int t0 = min(L, k * csz), t1 = min(L, (k + 1) * csz);
  const int ntile = (t1 - t0 + TT - 1) / TT;

  // q~ operand in registers: lane holds q~[h][32ks + 8q4 .. +8]
  bf16x8_t qf[DLAT / 32];
  if (wave_active) {
    const uint16_t* qrow = qt + ((int64_t)b * a.H + h) * DLAT;
#pragma unroll
    for (int ks = 0; ks < DLAT / 32; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 32 + q4 * 8);
  }

  const uint16_t* cbase = static_cast<const uint16_t*>(a.cache) + (int64_t)b * a.cache_stride;
  // load roles: c-part 4 rows x 8 columns per thread; rope part one 16 B chunk
  const int tq = tid >> 6, db = tid & 63;
  const int rtok = (tid & 255) >> 3, rc = tid & 7;
  u32x4_t pre[5];
  auto gload = [&](int tt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int tok = tt + 4 * tq + r;
      pre[r] = (tok < t1) ? *reinterpret_cast<const u32x4_t*>(cbase + (int64_t)tok * DLAT + 8 * db)
                          : u32x4_t{0u, 0u, 0u, 0u};
    }
    int tok = tt + rtok;
    pre[4] = (tid < 256 && tok < t1)
                 ? *reinterpret_cast<const u32x4_t*>(cbase + (int64_t)tok * DLAT + DC + 8 * rc)
                 : u32x4_t{0u, 0u, 0u, 0u};
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<u32x4_t*>(&Cs[buf][(4 * tq + r) * CP + 8 * db]) = pre[r];
    if (tid < 256) *reinterpret_cast<u32x4_t*>(&Cs[buf][rtok * CP + DC + 8 * rc]) = pre[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) ? 16 : 0;
      uint32_t x0 = (pre[0][e >> 1] >> sh) & 0xffffu, x1 = (pre[1][e >> 1] >> sh) & 0xffffu;
      uint32_t x2 = (pre[2][e >> 1] >> sh) & 0xffffu, x3 = (pre[3][e >> 1] >> sh) & 0xffffu;
      u32x2_t v2;
      v2[0] = x0 | (x1 << 16);
      v2[1] = x2 | (x3 << 16);
      *reinterpret_cast<u32x2_t*>(&Cts[buf][(8 * db + e) * CTP + 4 * tq]) = v2;
    }
  };

  const float c_log2 = a.scale * MLA_LOG2E;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t oacc[DC / 16];
#pragma unroll
  for (int d = 0; d < DC / 16; ++d) oacc[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (ntile > 0) {
    gload(t0);
    lstore(0);
  }
  __syncthreads();

  for (int t = 0; t < ntile; ++t) {
    const int tt = t0 + t * TT;
    const int buf = t & 1;
    if (t + 1 < ntile) gload(tt + TT);

    if (wave_active) {
      f32x4_t sacc[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        sacc[st] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DLAT / 32; ++ks) {
          bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(&Cs[buf][(st * 16 + l16) * CP + ks * 32 + q4 * 8]);
          sacc[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[ks], sacc[st], 0, 0, 0);
        }
      }
      // sacc[st][r]: token tt + 16st + 4q4 + r, head h
      const bool tail = (tt + TT > t1);
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = sacc[st][r] * c_log2;
          if (tail && (tt + 16 * st + 4 * q4 + r >= t1)) x = -INFINITY;
          sacc[st][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float rs = 0.f;
      bf16x8_t pf;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float pv = fast_exp2(sacc[st][r] - m_use);
          rs += pv;
          pf[4 * st + r] = __builtin_bit_cast(__bf16, float_to_bf16_bits(pv));
        }
      l_run = l_run * alpha + rs;
      m_run = m_new;
      if (__ballot(alpha != 1.f) != 0ull) {
#pragma unroll
        for (int d = 0; d < DC / 16; ++d) oacc[d] *= alpha;
      }
#pragma unroll
      for (int d = 0; d < DC / 16; ++d) {
        const uint16_t* crow = &Cts[buf][(d * 16 + l16) * CTP + 4 * q4];
        u32x2_t lo = *reinterpret_cast<const u32x2_t*>(crow);
        u32x2_t hi = *reinterpret_cast<const u32x2_t*>(crow + 16);
        u32x4_t raw = {lo[0], lo[1], hi[0], hi[1]};
        bf16x8_t af = __builtin_bit_cast(bf16x8_t, raw);
        oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, pf, oacc[d], 0, 0, 0);
      }
    }

    if (t + 1 < ntile) lstore(buf ^ 1);
    __syncthreads();
  }

  if (!wave_active || h >= a.H) return;
  float l = l_run + __shfl_xor(l_run, 16, 64);
  l += __shfl_xor(l, 32, 64);
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  const int64_t pidx = ((int64_t)b * a.n_splits + k) * a.H + h;
  float* dst = o_part + pidx * DC;
#pragma unroll
  for (int d = 0; d < DC / 16; ++d)
    *reinterpret_cast<f32x4_t*>(dst + d * 16 + 4 * q4) = oacc[d] * inv;
  if (q4 == 0) lse_part[pidx] = (l > 0.f) ? (m_run + __log2f(l)) * MLA_LN2 : -INFINITY;
}

}  // namespace

hipError_t launch_absorb_bf16(const DecodeArgs& a, uint16_t* qt, hipStream_t stream) {
  dim3 grid(a.H, (a.B + AB - 1) / AB);
  hipLaunchKernelGGL(absorb_bf16_kernel, grid, dim3(256), 0, stream, a, qt);
  return hipGetLastError();
}

hipError_t launch_mfma_splitkv(const DecodeArgs& a, const uint16_t* qt, float* lse_part, float* o_part,
                               hipStream_t stream) {
  dim3 grid(a.n_splits, a.B);
  hipLaunchKernelGGL(mfma_splitkv_kernel, grid, dim3(NTHREADS), 0, stream, a, qt, lse_part, o_part);
  return hipGetLastError();
}
