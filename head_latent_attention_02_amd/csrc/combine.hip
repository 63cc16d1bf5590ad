// Log-sum-exp merge of the split-KV partials followed by the un-absorb
// projection.  The merge rescales each chunk's normalised partial by
// exp(lse_k - lse) and sums, which reproduces the softmax over the whole
// sequence ("Helix Parallelism ..." (Pith review), "What carries the
// argument"); the merged latent accumulator is then mapped to d_v through the
// value part of W_kv_b ("A Training-Memory Regression in MLA Sequence
// Parallelism ... LAGA" (Pith review), Fig. 2 "Absorbed (B2)", un-absorb).
//
// One block per (head, group of CB sequences), 256 threads.
//   1. chunk weights w_k = exp(lse_k - lse) per sequence (one wave each);
//   2. merge: each thread owns 16-byte column groups of the group's latent rows and
//      issues the loads of all chunks of a column before combining them, so
//      a whole chunk row is in flight at once (the step is bandwidth-bound);
//   3. un-absorb: thread (v, half) computes out[b, h, v] for half of the
//      group's sequences from W_UV[h] row v (read once per block, 16 bytes at
//      a time) and the merged rows in LDS.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int CB = 16;         // sequences per block (the un-absorb MFMA's 16 columns)
constexpr int CTHREADS = 256;
constexpr int MAXNS = 64;      // chunk limit (checked on the host)
constexpr int KBATCH = 16;     // chunk loads in flight per column

template <mla_dtype WT>
__device__ __forceinline__ void load8(const void* w, int64_t idx, float (&f)[8]) {
  if constexpr (WT == MLA_BF16) {
    u32x4_t raw = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(w) + idx);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = bf16_bits_to_float((uint16_t)(raw[e] & 0xffff));
      f[2 * e + 1] = bf16_bits_to_float((uint16_t)(raw[e] >> 16));
    }
  } else {
    const f32x4_t* p = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(w) + idx);
    f32x4_t a = p[0], b = p[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = a[e];
      f[4 + e] = b[e];
    }
  }
}

template <mla_dtype WT, mla_dtype OT, bool HALFP>
__global__ void __launch_bounds__(CTHREADS) __attribute__((amdgpu_waves_per_eu(2)))
combine_kernel(DecodeArgs a, const float* __restrict__ lse_part, const void* __restrict__ o_part) {
  extern __shared__ __attribute__((aligned(16))) float olat[];   // [CB][dkv]
  __shared__ float wk[CB][MAXNS];
  __shared__ float lse_s[CB];
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * CB;
  const int nb = min(CB, a.B - b0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ns = a.n_splits, dkv = a.dkv;
  auto lse_index = [&](int bb) -> int64_t {
    return a.lse_seq > 0 ? ((int64_t)(bb / a.lse_seq) * a.H + h) * a.lse_seq + bb % a.lse_seq
                         : (int64_t)bb * a.H + h;
  };

  // The MFMA un-absorb (step 3, bf16 weights, d_v = 128, d_kv = 512) takes
  // its W_UV fragments in registers: the first half is loaded here, so that
  // its latency passes during the merge, the second half at the start of
  // step 3, while the first half is multiplied.
  constexpr int UKS = 512 / 32;                 // k-steps of the MFMA un-absorb
  const bool mfma_unabsorb = WT == MLA_BF16 && a.dv == 2 * 16 * (CTHREADS / 64) && dkv == 32 * UKS;
  const int64_t wrow0 = (int64_t)h * (a.dn + a.dv) + a.dn;
  const int l16 = lane & 15, q4 = lane >> 4;
  bf16x8_t wfr[UKS][2];
  const uint16_t* wv = static_cast<const uint16_t*>(a.w) + (wrow0 + 32 * wave + l16) * dkv + 8 * q4;
  auto load_w = [&](int ks0) {
#pragma unroll
    for (int ks = ks0; ks < ks0 + UKS / 2; ++ks)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
        wfr[ks][vb] = *reinterpret_cast<const bf16x8_t*>(wv + (int64_t)16 * vb * dkv + 32 * ks);
  };
  if constexpr (WT == MLA_BF16) {
    if (mfma_unabsorb) load_w(0);
  }

  // 1. chunk weights
  for (int bi = wave; bi < nb; bi += CTHREADS / 64) {
    const int b = b0 + bi;
    const float l = (lane < ns) ? lse_part[((int64_t)b * ns + lane) * a.H + h] : -INFINITY;
    const float m = wave_max(l);
    const float e = (l == -INFINITY) ? 0.f : expf(l - m);
    const float tot = wave_sum(e);
    if (lane < ns) wk[bi][lane] = (tot > 0.f) ? e / tot : 0.f;
    if (lane == 0) lse_s[bi] = (tot > 0.f) ? m + logf(tot) : -INFINITY;
  }
  __syncthreads();

  // 2. merge: G columns per thread (16-byte loads: 4 fp32 or 8 fp16 partial
  // elements; dkv is a multiple of 8 on the fp16 path and of 4 otherwise)
  constexpr int G = HALFP ? 8 : 4;
  const int cgn = dkv / G;
  const int64_t kstride = (int64_t)a.H * dkv;             // elements between chunks
  for (int it = tid; it < nb * cgn; it += CTHREADS) {
    const int bi = it / cgn, cg = it - bi * cgn, b = b0 + bi;
    const int64_t src = ((int64_t)b * ns * a.H + h) * dkv + G * cg;
    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < ns; k0 += KBATCH) {
      u32x4_t v[KBATCH];
#pragma unroll
      for (int j = 0; j < KBATCH; ++j) {
        const int64_t idx = src + (k0 + j) * kstride;
        v[j] = (k0 + j >= ns) ? u32x4_t{0u, 0u, 0u, 0u}
               : HALFP ? *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(o_part) + idx)
                       : *reinterpret_cast<const u32x4_t*>(static_cast<const float*>(o_part) + idx);
      }
#pragma unroll
      for (int j = 0; j < KBATCH; ++j) {
        if (k0 + j >= ns) continue;
        const float wj = wk[bi][k0 + j];
        if constexpr (HALFP) {
          const f16x8_t hv = __builtin_bit_cast(f16x8_t, v[j]);
          acc0 += f32x4_t{(float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]} * wj;
          acc1 += f32x4_t{(float)hv[4], (float)hv[5], (float)hv[6], (float)hv[7]} * wj;
        } else {
          acc0 += __builtin_bit_cast(f32x4_t, v[j]) * wj;
        }
      }
    }
    *reinterpret_cast<f32x4_t*>(&olat[bi * dkv + G * cg]) = acc0;
    if constexpr (HALFP) *reinterpret_cast<f32x4_t*>(&olat[bi * dkv + G * cg + 4]) = acc1;
  }
  __syncthreads();

  // 3. un-absorb: out[b, h, v] = W_UV[h][v] . o_lat[b]
  if constexpr (WT == MLA_BF16) {
    if (mfma_unabsorb) {
      // On 16x16x32 bf16 MFMA: out^T[v][s] = W_UV[h][v][:] . o_lat[s][:], 16 rows
      // v x 16 sequence columns per product; wave w owns v-blocks 2w
      // and 2w+1.  A lane holds 8 consecutive latent columns of one W row (the
      // 16 lanes of a k-group read 16 rows, 64 contiguous bytes each), and the
      // fp32 o_lat enters as two bf16 terms, hi = bf16(x) and lo = bf16(x - hi),
      // so the product keeps about 16 bits of o_lat.
      f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
      load_w(UKS / 2);
#pragma unroll
      for (int ks = 0; ks < UKS; ++ks) {
        bf16x8_t bhi = {}, blo = {};
        if (l16 < nb) {
          const f32x4_t* o = reinterpret_cast<const f32x4_t*>(&olat[l16 * dkv + 32 * ks + 8 * q4]);
          const f32x4_t o0 = o[0], o1 = o[1];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = (e < 4) ? o0[e] : o1[e - 4];
            const __bf16 hi = (__bf16)x;
            bhi[e] = hi;
            blo[e] = (__bf16)(x - (float)hi);
          }
        }
#pragma unroll
        for (int vb = 0; vb < 2; ++vb) {
          acc[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfr[ks][vb], bhi, acc[vb], 0, 0, 0);
          acc[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfr[ks][vb], blo, acc[vb], 0, 0, 0);
        }
      }
      // lane holds out^T[v = 32 wave + 16 vb + 4 q4 + r][s = l16]
      if (l16 < nb) {
#pragma unroll
        for (int vb = 0; vb < 2; ++vb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            store_elem<OT>(a.out, ((int64_t)(b0 + l16) * a.H + h) * a.dv + 32 * wave + 16 * vb + 4 * q4 + r,
                           acc[vb][r]);
      }
      if (a.lse != nullptr && tid < nb) a.lse[lse_index(b0 + tid)] = lse_s[tid];
      return;
    }
  }
  constexpr int HALF = CB / 2;
  for (int it = tid; it < a.dv * 2; it += CTHREADS) {
    const int v = it % a.dv, half = it / a.dv;
    float acc[HALF];
#pragma unroll
    for (int j = 0; j < HALF; ++j) acc[j] = 0.f;
    const int64_t wbase = (wrow0 + v) * dkv;
    for (int c = 0; c < dkv; c += 8) {
      float w[8];
      load8<WT>(a.w, wbase + c, w);
#pragma unroll
      for (int j = 0; j < HALF; ++j) {
        const int bi = half * HALF + j;
        const f32x4_t* o = reinterpret_cast<const f32x4_t*>(&olat[(bi < nb ? bi : 0) * dkv + c]);
        const f32x4_t o0 = o[0], o1 = o[1];
        acc[j] += w[0] * o0[0] + w[1] * o0[1] + w[2] * o0[2] + w[3] * o0[3] +
                  w[4] * o1[0] + w[5] * o1[1] + w[6] * o1[2] + w[7] * o1[3];
      }
    }
#pragma unroll
    for (int j = 0; j < HALF; ++j) {
      const int bi = half * HALF + j;
      if (bi < nb) store_elem<OT>(a.out, ((int64_t)(b0 + bi) * a.H + h) * a.dv + v, acc[j]);
    }
  }
  if (a.lse != nullptr && tid < nb) a.lse[lse_index(b0 + tid)] = lse_s[tid];
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, const float* lse_part, const void* o_part, bool half_parts,
                          hipStream_t stream) {
  dim3 grid(a.H, (a.B + CB - 1) / CB);
  size_t smem = sizeof(float) * CB * a.dkv;
#define MLA_COMBINE(WT, OT)                                                                                    \
  if (half_parts)                                                                                              \
    hipLaunchKernelGGL((combine_kernel<WT, OT, true>), grid, dim3(CTHREADS), smem, stream, a, lse_part, o_part); \
  else                                                                                                         \
    hipLaunchKernelGGL((combine_kernel<WT, OT, false>), grid, dim3(CTHREADS), smem, stream, a, lse_part, o_part);
  if (a.in_dt == MLA_BF16) {
    if (a.out_dt == MLA_BF16) {
      MLA_COMBINE(MLA_BF16, MLA_BF16)
    } else {
      MLA_COMBINE(MLA_BF16, MLA_FP32)
    }
  } else {
    if (a.out_dt == MLA_BF16) {
      MLA_COMBINE(MLA_FP32, MLA_BF16)
    } else {
      MLA_COMBINE(MLA_FP32, MLA_FP32)
    }
  }
#undef MLA_COMBINE
  return hipGetLastError();
}
