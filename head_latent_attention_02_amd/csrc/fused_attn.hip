// Explicit-form MLA attention with the latent up-projection fused in: K_nope
// and V are computed tile by tile from c_kv and W_kv_b inside the attention
// workgroup and never stored to HBM.  "A Training-Memory Regression in MLA
// Sequence Parallelism ... LAGA" (Pith review) names this fusion as future
// work ("Where Pith is reading between the lines"); its Fig. 3 caption is the
// cost side: the up-projection is then repeated by every query block that
// reads a key tile instead of running once as one large GEMM.
//
// One workgroup per (b, h, 256 queries): 8 waves of 32 queries.  Per tile of
// 128 keys:
//   up-projection  [K_nope^T ; V] of the tile from c_kv (bf16 MFMA 32x32x16,
//                  fp32 accumulate, rounded to fp16 like the materialised
//                  path).  Wave w computes the d-block w%4 of K_nope^T and of
//                  V for key blocks 2(w/4), 2(w/4)+1; the c_kv tile streams
//                  through a two-slot LDS ring in chunks of 64 latent columns,
//                  the W_kv_b fragments of the head go from global memory
//                  straight into registers, two k-steps ahead.
//   attention      S^T = K Q^T (fp16 MFMA), online softmax per query, O^T +=
//                  V^T P^T, over 32-key blocks of the tile, as in the
//                  materialised kernel.
// The rotated key band is read from the small fp16 band buffer that the
// materialised path also uses (shared by all heads).
//
// Operand order (as in the backward kernels): K rows of a 32-key block sit in
// LDS in the order rho -> key with bits 2 and 3 swapped, so that accumulator
// elements 8u .. 8u+7 of a lane are keys 16u + 8x .. 16u + 8x + 7 (x the lane
// half): the P fragments of the next MFMA without any data movement.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int DN = 128, DR = 64, DQK = 192, DV = 128, DKV = 512, HD = DN + DV;
constexpr int NW = 8, NT = 64 * NW, QW = 32, QB = NW * QW;   // 256 queries per workgroup
constexpr int KT = 128;                                       // keys per tile
constexpr int KCH = 64;                                       // latent columns per chunk
constexpr int NCH = DKV / KCH;                                // chunks per tile
constexpr int KS = DQK / 16;                                  // k-steps of S
constexpr float TAU = 8.f;                                    // rescale threshold (log2 units)
// LDS (16-bit elements); padded rows keep the 16-byte fragment reads of 16
// consecutive rows on distinct banks
constexpr int K_LD = DQK + 8;                                 // K tile: [KT][K_LD]
constexpr int VT_LD = KT + 8;                                 // V^T tile: [DV][VT_LD]
constexpr int C_ELEMS = KT * KCH;                             // one c_kv chunk [KT][KCH], swizzled
constexpr int CH_UNITS = C_ELEMS / 8;                         // 16-byte units per chunk
constexpr int CU_PER_T = CH_UNITS / NT;                       // units per thread per chunk
static_assert(CH_UNITS % NT == 0, "chunk copy");
constexpr int KR_UNITS = KT * DR / 8;                         // 16-byte units of the key band per tile
constexpr int KR_PER_T = KR_UNITS / NT;
static_assert(KR_UNITS % NT == 0, "band copy");

__device__ __forceinline__ f32x16_t mfma_h(f16x8_t a, f16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma_b(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// index inside a 32-block <-> LDS row: swap bits 2 and 3 (an involution)
__device__ __forceinline__ int perm32(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
// 16-byte unit swizzle of a 128-byte chunk row
__device__ __forceinline__ int csw(int row) { return (row >> 1) & 7; }

template <mla_dtype OT>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
fused_attention_kernel(ExplicitArgs a, const uint16_t* __restrict__ krot, const float2* __restrict__ qtab, int nqt) {
  __shared__ __attribute__((aligned(16))) uint16_t Kt[KT * K_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[DV * VT_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Cr[2 * C_ELEMS];

  // heads on XCDs (blockIdx.x % 8), two at a time, longest query blocks
  // first alternating between the two
  const int P = a.B * a.H;
  const int n = blockIdx.x;
  const int xcd = n & 7, slot = n >> 3;
  const int grp = slot / (2 * nqt), r = slot % (2 * nqt);
  const int p = xcd + 8 * (2 * grp + (r & 1));
  const int qt = nqt - 1 - (r >> 1);
  if (p >= P) return;
  const int b = p / a.H, h = p % a.H;
  const int64_t bh = (int64_t)b * a.H + h;
  const int i0 = qt * QB;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hb = lane >> 5;
  const int iw0 = i0 + wave * QW;
  const float c_log2 = a.scale * MLA_LOG2E;

  auto limit = [&](int qi) __attribute__((always_inline)) -> int {   // keys [0, limit) visible to query qi
    if (!a.causal) return a.s_vis;
    int64_t lim = a.q_pos0 + qi - a.kv_pos0 + 1;
    return (int)max((int64_t)0, min(lim, (int64_t)a.s_vis));
  };
  const int kend_wg = limit(min(i0 + QB, a.Sq) - 1);
  const int ntile = (kend_wg + KT - 1) / KT;                 // tiles end at or before s_pad
  const bool wave_has_rows = iw0 < a.Sq;
  const int kend_w = wave_has_rows ? limit(min(iw0 + QW, a.Sq) - 1) : 0;
  const int kfull_w = wave_has_rows ? limit(iw0) : 0;
  const int i_me = iw0 + l32;
  const int lim_me = (i_me < a.Sq) ? limit(i_me) : 0;

  // ---- up-projection operands ------------------------------------------------
  // Wave (kq, di): K_nope^T rows 32di.. and V columns 32di.. of W_kv_b's head
  // block, key blocks 2kq and 2kq+1 of the tile.
  const int kq = wave >> 2, di = wave & 3;
  const uint16_t* wbase = static_cast<const uint16_t*>(a.w) + (int64_t)h * HD * DKV;
  const uint16_t* wuk = wbase + (int64_t)(32 * di + l32) * DKV + 8 * hb;
  const uint16_t* wuv = wbase + (int64_t)(DN + 32 * di + l32) * DKV + 8 * hb;
  const uint16_t* cbase = static_cast<const uint16_t*>(a.c_kv) + (int64_t)b * a.Skv * DKV;
  const uint16_t* kbase = krot + (int64_t)b * a.s_pad * DR;
  const int nchunk = ntile * NCH;

  // chunk g = NCH t + c: keys 128t .., latent columns 64c ..; unit q of the
  // chunk (row q/8, stored unit q%8) holds latent unit (q%8) ^ csw(row).
  // one staging set: chunk g+1 is stored before chunk g+2 is loaded into it
  u32x4_t cst[CU_PER_T];
  auto load_chunk = [&](int g) __attribute__((always_inline)) {
    const int t = g / NCH, c = g % NCH;
#pragma unroll
    for (int k = 0; k < CU_PER_T; ++k) {
      const int q = tid + NT * k, row = q >> 3, u = (q & 7) ^ csw(row);
      // rows past the last latent row repeat it: finite K and V for keys
      // that the mask removes (a zero P times a non-finite V would not vanish)
      const int key = min(t * KT + row, a.Skv - 1);
      cst[k] = *reinterpret_cast<const u32x4_t*>(cbase + (int64_t)key * DKV + c * KCH + 8 * u);
    }
  };
  auto store_chunk = [&](int g) __attribute__((always_inline)) {
    uint16_t* dst = Cr + (g & 1) * C_ELEMS;
#pragma unroll
    for (int k = 0; k < CU_PER_T; ++k) *reinterpret_cast<u32x4_t*>(dst + 8 * (tid + NT * k)) = cst[k];
  };
  // W fragments, two k-steps ahead: k-step z (16 latent columns, counted
  // across chunks and tiles) uses slot z % 2, which is then refilled for z + 2
  bf16x8_t wf[2][2];
  auto load_w = [&](int slot_, int z) __attribute__((always_inline)) {
    const int col = (z % (DKV / 16)) * 16;
    wf[slot_][0] = *reinterpret_cast<const bf16x8_t*>(wuk + col);
    wf[slot_][1] = *reinterpret_cast<const bf16x8_t*>(wuv + col);
  };
  // the rotated key band of a tile: loaded during the previous tile's
  // attention, stored into the K rows once every wave is past that attention
  u32x4_t kst[KR_PER_T];
  auto store_band = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < KR_PER_T; ++k) {
      const int q = tid + NT * k, rho = q >> 3, u = q & 7;
      *reinterpret_cast<u32x4_t*>(Kt + rho * K_LD + DN + 8 * u) = kst[k];
    }
  };
  auto load_band = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < KR_PER_T; ++k) {
      const int q = tid + NT * k, rho = q >> 3, u = q & 7;
      const int key = t * KT + (rho & ~31) + perm32(rho & 31);
      kst[k] = *reinterpret_cast<const u32x4_t*>(kbase + (int64_t)key * DR + 8 * u);
    }
  };

  // chunk 0 goes to slot 0 before the loop; chunk 1 and the W fragments of
  // chunk 0 are on their way while Q is loaded
  if (nchunk > 0) {
    load_band(0);
    load_chunk(0);
    store_chunk(0);
    store_band();
    if (nchunk > 1) load_chunk(1);
    load_w(0, 0);
    load_w(1, 1);
  }

  // ---- Q^T operand (fp16): lane (l32, hb) holds query row l32 of the wave,
  // k-slots 8hb .. 8hb+7 of every k-step (q_nope, then R(q_pe)) ------------------
  f16x8_t qf[KS];
  {
    const int ic = i_me < a.Sq ? i_me : a.Sq - 1;
    const int64_t qrow = ((int64_t)b * a.Sq + ic) * a.H + h;
    const u32x4_t* qn = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.q_nope) + qrow * DN);
    const uint16_t* qp = static_cast<const uint16_t*>(a.q_pe) + qrow * DR;
    const float2* qt2 = qtab + (int64_t)ic * (DR / 2);
#pragma unroll
    for (int ks = 0; ks < DN / 16; ++ks) {
      const u32x4_t r = qn[2 * ks + hb];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[ks][2 * e] = (_Float16)bf16_bits_to_float((uint16_t)(r[e] & 0xffff));
        qf[ks][2 * e + 1] = (_Float16)bf16_bits_to_float((uint16_t)(r[e] >> 16));
      }
    }
    // band element m (0..63) of R(q_pe): pairs (m, m+32) turn by the angle of m % 32
#pragma unroll
    for (int ks = DN / 16; ks < KS; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int m = 16 * (ks - DN / 16) + 8 * hb + e, mm = m & 31;
        const float lo = bf16_bits_to_float(qp[mm]), hi = bf16_bits_to_float(qp[mm + 32]);
        const float2 cs = qt2[mm];
        qf[ks][e] = (_Float16)(m < 32 ? lo * cs.x - hi * cs.y : hi * cs.x + lo * cs.y);
      }
    }
  }

  f32x16_t oacc[DV / 32];
#pragma unroll
  for (int db = 0; db < DV / 32; ++db) oacc[db] = f32x16_t{};
  float m_ref = -INFINITY, l_run = 0.f;

  for (int t = 0; t < ntile; ++t) {
    // ---- up-projection of tile t ----------------------------------------------
    f32x16_t kacc[2] = {}, vacc[2] = {};
    for (int c = 0; c < NCH; c += 2) {
      // two chunks per trip so that the staging set is a compile-time index
      auto chunk = [&](auto sc, int g) __attribute__((always_inline)) {
        constexpr int S = decltype(sc)::value;                 // == g & 1
        __syncthreads();                                       // chunk g stored; slot (g+1)&1 free
        if (g + 1 < nchunk) store_chunk(g + 1);
        if (g + 2 < nchunk) load_chunk(g + 2);
        const uint16_t* cs = Cr + S * C_ELEMS;
#pragma unroll
        for (int ks = 0; ks < KCH / 16; ++ks) {
          const int u = 2 * ks + hb;
          const int r0 = 64 * kq + l32, r1 = r0 + 32;
          const bf16x8_t c0 = *reinterpret_cast<const bf16x8_t*>(cs + r0 * KCH + 8 * (u ^ csw(r0)));
          const bf16x8_t c1 = *reinterpret_cast<const bf16x8_t*>(cs + r1 * KCH + 8 * (u ^ csw(r1)));
          kacc[0] = mfma_b(wf[ks & 1][0], c0, kacc[0]);
          kacc[1] = mfma_b(wf[ks & 1][0], c1, kacc[1]);
          vacc[0] = mfma_b(c0, wf[ks & 1][1], vacc[0]);
          vacc[1] = mfma_b(c1, wf[ks & 1][1], vacc[1]);
          const int z = g * (KCH / 16) + ks + 2;
          if (z < nchunk * (KCH / 16)) load_w(ks & 1, z);
        }
      };
      chunk(std::integral_constant<int, 0>{}, t * NCH + c);
      chunk(std::integral_constant<int, 1>{}, t * NCH + c + 1);
    }
    // every wave is past the previous tile's attention (barriers above):
    // K_nope^T block (rows d, columns keys) -> K rows rho = perm(key), 4 d per store
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int kb = 2 * kq + x;
      uint16_t* krow = Kt + (32 * kb + perm32(l32)) * K_LD + 32 * di + 4 * hb;
      uint16_t* vcol = Vt + (32 * di + l32) * VT_LD + 32 * kb + 4 * hb;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f16x4_t kv4, vv4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          kv4[r] = (_Float16)kacc[x][4 * g4 + r];
          vv4[r] = (_Float16)vacc[x][4 * g4 + r];
        }
        *reinterpret_cast<f16x4_t*>(krow + 8 * g4) = kv4;
        *reinterpret_cast<f16x4_t*>(vcol + 8 * g4) = vv4;
      }
    }
    __syncthreads();
    if (t + 1 < ntile) load_band(t + 1);

    // ---- attention over the 32-key blocks of tile t ------------------------------
#pragma unroll 1
    for (int j = 0; j < KT / 32; ++j) {
      const int k0 = t * KT + 32 * j;
      if (k0 >= kend_w) break;
      f32x16_t sacc = {};
      const uint16_t* kr = Kt + (32 * j + l32) * K_LD + 8 * hb;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sacc = mfma_h(*reinterpret_cast<const f16x8_t*>(kr + 16 * ks), qf[ks], sacc);
      // element e: key k0 + perm(8(e/4) + 4hb + e%4), query i_me
      float tv[16];
      const bool full = k0 + 32 <= kfull_w;
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + perm32(8 * (e >> 2) + 4 * hb + (e & 3));
        tv[e] = (full || key < lim_me) ? sacc[e] * c_log2 : -INFINITY;
        mx = fmaxf(mx, tv[e]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool need = mx > m_ref + TAU;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float alpha = need ? ((m_ref == -INFINITY) ? 0.f : fast_exp2(m_ref - mx)) : 1.f;
        if (need) m_ref = mx;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DV / 32; ++db) oacc[db] *= alpha;
      }
      const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
      f16x8_t pb[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = fast_exp2(tv[e] - m_use);
        l_run += pv;
        pb[e >> 3][e & 7] = (_Float16)pv;
      }
      const uint16_t* vr = Vt + l32 * VT_LD + 32 * j + 8 * hb;
#pragma unroll
      for (int db = 0; db < DV / 32; ++db)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          oacc[db] = mfma_h(*reinterpret_cast<const f16x8_t*>(vr + 32 * db * VT_LD + 16 * u), pb[u], oacc[db]);
    }
    if (t + 1 < ntile) {
      __syncthreads();                                   // every wave is done with tile t's K rows
      store_band();
    }
  }

  // ---- epilogue: O = O^T / l, LSE --------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (i_me >= a.Sq) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t orow = (((int64_t)b * a.Sq + i_me) * a.H + h) * DV;
#pragma unroll
  for (int db = 0; db < DV / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = 32 * db + 8 * g4 + 4 * hb;
      f32x4_t o4;
#pragma unroll
      for (int r = 0; r < 4; ++r) o4[r] = oacc[db][4 * g4 + r] * inv;
      if constexpr (OT == MLA_BF16) {
        u32x2_t w2;
        w2[0] = (uint32_t)float_to_bf16_bits(o4[0]) | ((uint32_t)float_to_bf16_bits(o4[1]) << 16);
        w2[1] = (uint32_t)float_to_bf16_bits(o4[2]) | ((uint32_t)float_to_bf16_bits(o4[3]) << 16);
        *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(a.out) + orow + d) = w2;
      } else {
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + orow + d) = o4;
      }
    }
  if (a.lse != nullptr && hb == 0) {
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    a.lse[bh * a.Sq + i_me] = (l_tot > 0.f) ? (m_use + __log2f(l_tot)) * MLA_LN2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_fused_attention(const ExplicitArgs& a, const uint16_t* krot, const float2* qtab,
                                  hipStream_t stream) {
  if (a.Sq == 0) return hipSuccess;
  const int nqt = (a.Sq + QB - 1) / QB;
  const int P = a.B * a.H;
  const dim3 grid(16 * ((P + 15) / 16) * nqt);         // whole pairs of heads on every XCD
  if (a.out_dt == MLA_BF16)
    hipLaunchKernelGGL(fused_attention_kernel<MLA_BF16>, grid, dim3(NT), 0, stream, a, krot, qtab, nqt);
  else
    hipLaunchKernelGGL(fused_attention_kernel<MLA_FP32>, grid, dim3(NT), 0, stream, a, krot, qtab, nqt);
  return hipGetLastError();
}
