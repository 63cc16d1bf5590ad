// Backward of the explicit-form MLA forward on fp16 MFMA (fp32 accumulate),
// for d_kv 512, d_nope 128, d_rope 64, d_v 128 and bf16 inputs: the gradient
// of sum(d_out * out) with respect to q_nope, q_pe, c_kv, k_pe and W_kv_b (the
// training setting of "A Training-Memory Regression in MLA Sequence
// Parallelism ... LAGA" (Pith review); "If this is right" on gradients).
//
// With sigma the softmax scale, P the softmax of the forward (recomputed from
// its LSE), D_i = d_out_i . out_i:
//   dS = P (dO V^T - D),  dV = P^T dO,  dK = sigma dS^T Q,  dQ = sigma dS K
// over the 192-wide [q_nope ; R(q_pe)] / [K_nope ; R(k_pe)] and the 128-wide V,
// then dc_kv = dKV W (dKV = [dK_nope | dV] per head), dW = dKV^T c_kv, and the
// RoPE bands rotated back (the transpose of a rotation turns by the negative
// angle), the key band summed over heads.
//
// Kernels (one launch each):
//   prep_q      fp16 Q = [q_nope ; R(q_pe)] and dO in row layout [bh][i][d] and
//               transposed layout [bh][d][i] (query rows padded to 128 with
//               zeros), and D = dO . out in fp32.
//   transpose   K_nope^T, the rotated key band transposed, W^T and c_kv^T
//               (fp16); V comes from the up-projection in rows [bh][key][128].
//   kv          per (b, h, 128 keys): 8 waves, two per 32-key block sharing a
//               SIMD: one holds K and computes S = Q K^T, P and dV^T += dO^T P,
//               the other holds V and computes dP = dO V^T, dS and
//               dK^T += Q^T dS, P passing between them through LDS; the two
//               alternate MFMA and vector phases in opposite order.  32-query
//               tiles of Q, dO, Q^T, dO^T stream through LDS.  Writes dKV in
//               both row and column layouts (fp16, for the two GEMMs) and the
//               per-head key-band gradient.
//   dq          per (b, h, 128 queries): 8 waves, two per 32-query block
//               sharing a SIMD: one holds Q^T and computes S^T = K Q^T, P and
//               the RoPE band of dQ^T += K^T dS^T, the other holds dO^T and
//               computes dP^T = V dO^T, dS and the nope part of dQ^T; P and
//               dS pass between them through LDS.  32-key tiles of K, V and
//               K^T stream through LDS.  Writes dq_nope and the rotated-back
//               dq_pe.
//   Both attention kernels deal the heads over the XCDs (all blocks of a
//   head on one XCD at once, walking the streamed tiles in the same order),
//   so each streamed tile is fetched into that XCD's L2 once for all of them.
//   dk_pe       the head sum of the key-band gradient, rotated back.
//   gemm_nt     C = A B^T with A, B fp16 row-major and fp32 C: dc_kv and dW.
//
// Operand order.  Rows of the streamed Q / dO (kv kernel) and K / V (dq
// kernel) tiles sit in LDS in the permuted order rho -> (rho with bits 2 and
// 3 swapped): the accumulator row that lane half x holds in element 4g + r is
// 8g + 4x + r, and with that order the 8 elements 8u .. 8u+7 of a lane are the
// 8 consecutive indices 16u + 8x .. 16u + 8x + 7 that it supplies as the
// k-slots of the next MFMA, so P and dS go from accumulators to MFMA operands
// inside the lane.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int DN = 128, DR = 64, DQK = 192, DV = 128, DKV = 512;
constexpr int HD = DN + DV;          // rows of W_kv_b per head

typedef _Float16 f16;

__device__ __forceinline__ f32x16_t mfma(f16x8_t a, f16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// rho <-> index inside a 32-block: swap bits 2 and 3 (an involution)
__device__ __forceinline__ int perm32(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
__device__ __forceinline__ uint16_t h_bits(float x) { return float_to_f16_bits(x); }

// ---------------------------------------------------------------- prep_q --
// One block per (b, h, 32 query rows); thread t handles element columns.
template <mla_dtype OT>
__global__ void __launch_bounds__(256)
prep_q_kernel(BackwardArgs a, const float2* __restrict__ qtab, uint16_t* __restrict__ qf, uint16_t* __restrict__ qft,
              uint16_t* __restrict__ dof, uint16_t* __restrict__ doft, float* __restrict__ dvec,
              float* __restrict__ lsdt, int sq_pad) {
  __shared__ __attribute__((aligned(16))) uint16_t Qs[32][DQK + 8];
  __shared__ __attribute__((aligned(16))) uint16_t Ds[32][DV + 8];
  __shared__ float red[32][9];
  const ExplicitArgs& f = a.f;
  const int i0 = blockIdx.x * 32, h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * f.H + h;
  const int tid = threadIdx.x;
  // rows: r = tid / 8 (32 rows), 8 threads per row
  const int r = tid >> 3, c8 = tid & 7;
  const int i = i0 + r;
  const bool live = i < f.Sq;
  const int64_t row = ((int64_t)b * f.Sq + (live ? i : 0)) * f.H + h;
  // q_nope: 16 columns per thread (two 16-byte loads, two 16-byte LDS stores)
  {
    u32x4_t v[2] = {u32x4_t{0u, 0u, 0u, 0u}, u32x4_t{0u, 0u, 0u, 0u}};
    if (live) {
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(f.q_nope) + row * DN + c8 * 16);
      v[0] = src[0];
      v[1] = src[1];
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      u32x4_t o;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        const uint32_t x = v[hh][w2];
        o[w2] = (uint32_t)h_bits(bf16_bits_to_float((uint16_t)(x & 0xffff))) |
                ((uint32_t)h_bits(bf16_bits_to_float((uint16_t)(x >> 16))) << 16);
      }
      *reinterpret_cast<u32x4_t*>(&Qs[r][c8 * 16 + 8 * hh]) = o;
    }
  }
  // rope pairs (m, m + 32), m = 4 c8 .. 4 c8 + 3: 8-byte loads of both halves
  {
    u32x2_t xl = {0u, 0u}, xh = {0u, 0u};
    f32x4_t cs[2] = {f32x4_t{1.f, 0.f, 1.f, 0.f}, f32x4_t{1.f, 0.f, 1.f, 0.f}};
    if (live) {
      const uint16_t* qp = static_cast<const uint16_t*>(f.q_pe) + row * DR + 4 * c8;
      xl = *reinterpret_cast<const u32x2_t*>(qp);
      xh = *reinterpret_cast<const u32x2_t*>(qp + 32);
      const f32x4_t* ct = reinterpret_cast<const f32x4_t*>(qtab + (int64_t)i * 32 + 4 * c8);
      cs[0] = ct[0];
      cs[1] = ct[1];
    }
    u32x2_t lo2, hi2;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float x0 = bf16_bits_to_float((uint16_t)((xl[k >> 1] >> (16 * (k & 1))) & 0xffff));
      const float x1 = bf16_bits_to_float((uint16_t)((xh[k >> 1] >> (16 * (k & 1))) & 0xffff));
      const float c = cs[k >> 1][2 * (k & 1)], sn = cs[k >> 1][2 * (k & 1) + 1];
      const uint32_t lo = h_bits(live ? x0 * c - x1 * sn : 0.f), hi = h_bits(live ? x1 * c + x0 * sn : 0.f);
      if (k & 1) {
        lo2[k >> 1] |= lo << 16;
        hi2[k >> 1] |= hi << 16;
      } else {
        lo2[k >> 1] = lo;
        hi2[k >> 1] = hi;
      }
    }
    *reinterpret_cast<u32x2_t*>(&Qs[r][DN + 4 * c8]) = lo2;
    *reinterpret_cast<u32x2_t*>(&Qs[r][DN + 32 + 4 * c8]) = hi2;
  }
  // dO and D = dO . out (16 columns per thread, summed in column order)
  float dsum = 0.f;
  {
    float g[16], o[16];
    if constexpr (OT == MLA_BF16) {
      u32x4_t gv[2] = {}, ov[2] = {};
      if (live) {
        const u32x4_t* gs = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.d_out) + row * DV + c8 * 16);
        const u32x4_t* os = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.out) + row * DV + c8 * 16);
        gv[0] = gs[0]; gv[1] = gs[1];
        ov[0] = os[0]; ov[1] = os[1];
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        g[k] = bf16_bits_to_float((uint16_t)((gv[k >> 3][(k & 7) >> 1] >> (16 * (k & 1))) & 0xffff));
        o[k] = bf16_bits_to_float((uint16_t)((ov[k >> 3][(k & 7) >> 1] >> (16 * (k & 1))) & 0xffff));
      }
    } else {
      f32x4_t gv[4] = {}, ov[4] = {};
      if (live) {
        const f32x4_t* gs = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(a.d_out) + row * DV + c8 * 16);
        const f32x4_t* os = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(a.out) + row * DV + c8 * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          gv[q] = gs[q];
          ov[q] = os[q];
        }
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        g[k] = gv[k >> 2][k & 3];
        o[k] = ov[k >> 2][k & 3];
      }
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) dsum += g[k] * o[k];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      u32x4_t pk;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2)
        pk[w2] = (uint32_t)h_bits(g[8 * hh + 2 * w2]) | ((uint32_t)h_bits(g[8 * hh + 2 * w2 + 1]) << 16);
      *reinterpret_cast<u32x4_t*>(&Ds[r][c8 * 16 + 8 * hh]) = pk;
    }
  }
  red[r][c8] = dsum;
  __syncthreads();
  if (c8 == 0) {
    float s = 0.f;
    for (int k = 0; k < 8; ++k) s += red[r][k];
    dvec[bh * sq_pad + i] = live ? s : 0.f;
    // the key-parallel kernel's copy of this tile: LSE then D at the LDS row
    // of query r (rows past S_q get an infinite LSE, so P = 0 there)
    float* t64 = lsdt + (bh * (sq_pad / 32) + blockIdx.x) * 64;
    t64[perm32(r)] = live ? a.lse[bh * f.Sq + i] : INFINITY;
    t64[32 + perm32(r)] = live ? s : 0.f;
  }
  // row layouts: 192 / 128 fp16 per row, 16-byte pieces
  for (int c = tid; c < 32 * (DQK / 8); c += 256) {
    const int rr = c / (DQK / 8), cc = c % (DQK / 8);
    *reinterpret_cast<u32x4_t*>(qf + (bh * sq_pad + i0 + rr) * DQK + cc * 8) =
        *reinterpret_cast<const u32x4_t*>(&Qs[rr][cc * 8]);
  }
  for (int c = tid; c < 32 * (DV / 8); c += 256) {
    const int rr = c / (DV / 8), cc = c % (DV / 8);
    *reinterpret_cast<u32x4_t*>(dof + (bh * sq_pad + i0 + rr) * DV + cc * 8) =
        *reinterpret_cast<const u32x4_t*>(&Ds[rr][cc * 8]);
  }
  // transposed layouts: column d, 32 queries (8 per 16-byte piece)
  for (int c = tid; c < DQK * 4; c += 256) {
    const int d = c >> 2, q8 = (c & 3) * 8;
    u32x4_t v;
    for (int e = 0; e < 4; ++e) v[e] = (uint32_t)Qs[q8 + 2 * e][d] | ((uint32_t)Qs[q8 + 2 * e + 1][d] << 16);
    *reinterpret_cast<u32x4_t*>(qft + (bh * DQK + d) * sq_pad + i0 + q8) = v;
  }
  for (int c = tid; c < DV * 4; c += 256) {
    const int d = c >> 2, q8 = (c & 3) * 8;
    u32x4_t v;
    for (int e = 0; e < 4; ++e) v[e] = (uint32_t)Ds[q8 + 2 * e][d] | ((uint32_t)Ds[q8 + 2 * e + 1][d] << 16);
    *reinterpret_cast<u32x4_t*>(doft + (bh * DV + d) * sq_pad + i0 + q8) = v;
  }
}

// ------------------------------------------------------------- transpose --
// out[z][c][r] = in[z][r][c] for r < rows_valid (0 for rows_valid <= r < rows),
// fp16 out, in fp16 or bf16 bits.  in: row stride in_ld, batch stride in_bs;
// out: row stride out_ld, batch stride out_bs.  32 x 32 tiles.
template <bool IN_BF16>
__global__ void __launch_bounds__(256)
transpose_kernel(const uint16_t* __restrict__ in, uint16_t* __restrict__ out, int rows, int rows_valid, int cols,
                 int64_t in_ld, int64_t in_bs, int64_t out_ld, int64_t out_bs) {
  __shared__ uint16_t T[32][34];
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32, z = blockIdx.z;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;    // 32 x 8
  for (int k = 0; k < 32; k += 8) {
    const int r = r0 + ty + k, c = c0 + tx;
    uint16_t v = 0;
    if (r < rows_valid && c < cols) {
      v = in[z * in_bs + (int64_t)r * in_ld + c];
      if (IN_BF16) v = h_bits(bf16_bits_to_float(v));
    }
    T[ty + k][tx] = v;
  }
  __syncthreads();
  for (int k = 0; k < 32; k += 8) {
    const int c = c0 + ty + k, r = r0 + tx;
    if (c < cols && r < rows) out[z * out_bs + (int64_t)c * out_ld + r] = T[tx][ty + k];
  }
}

// The same with 64 x 64 tiles moved in 16-byte pieces; rows and cols must be
// multiples of 8 (row r reads as 0 for rows_valid <= r < rows).
template <bool IN_BF16>
__global__ void __launch_bounds__(256)
transpose64_kernel(const uint16_t* __restrict__ in, uint16_t* __restrict__ out, int rows, int rows_valid, int cols,
                   int64_t in_ld, int64_t in_bs, int64_t out_ld, int64_t out_bs) {
  __shared__ __attribute__((aligned(16))) uint16_t T[64][64 + 8];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64, z = blockIdx.z;
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = tid + 256 * k, rr = q >> 3, cc = (q & 7) * 8;     // row rr, columns cc .. cc+7 of the tile
    const int r = r0 + rr, c = c0 + cc;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (r < rows_valid && c < cols) {
      v = *reinterpret_cast<const u32x4_t*>(in + z * in_bs + (int64_t)r * in_ld + c);
      if (IN_BF16) {
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2)
          v[w2] = (uint32_t)h_bits(bf16_bits_to_float((uint16_t)(v[w2] & 0xffff))) |
                  ((uint32_t)h_bits(bf16_bits_to_float((uint16_t)(v[w2] >> 16))) << 16);
      }
    }
    *reinterpret_cast<u32x4_t*>(&T[rr][cc]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = tid + 256 * k, cc = q >> 3, rr = (q & 7) * 8;     // column cc, rows rr .. rr+7 of the tile
    const int c = c0 + cc, r = r0 + rr;
    if (c < cols && r < rows) {
      u32x4_t v;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) v[w2] = (uint32_t)T[rr + 2 * w2][cc] | ((uint32_t)T[rr + 2 * w2 + 1][cc] << 16);
      *reinterpret_cast<u32x4_t*>(out + z * out_bs + (int64_t)c * out_ld + r) = v;
    }
  }
}

// -------------------------------------------------------------------- kv --
// Key-parallel kernel: per (b, h, 128 keys), 8 waves; the work of each
// 32-key block is split between two waves that share a SIMD:
//   wave A (waves 0-3) holds K and dV^T:  S = Q K^T, P, dV^T += dO^T P
//   wave B (waves 4-7) holds V and dK^T:  dP = dO V^T, dS = P (dP - D),
//                                         dK^T += Q^T dS
// P goes from A to B through LDS (fp32, lane to the same lane, since dP and S
// share the accumulator layout).  Each wave alternates an MFMA phase and a
// vector phase, one barrier apart, and the B waves run one phase behind the A
// waves, so on every SIMD one wave issues MFMAs while the other does its
// exponentials, LDS exchange and tile copies:
//   M_A(t): dV(t) and S(t+1)       V_A(t): P(t), its copy to LDS
//   M_B(t): dK(t) and dP(t+1)      V_B(t): P(t) from LDS, dS(t)
// Query tiles stream through two rings of 3 stages: the early part (Q and dO
// rows, LSE and D), copied by the A waves two tiles ahead, and the late part
// (Q^T, dO^T), copied by the B waves two tiles ahead (the late part of a
// tile is read one tile later than its early part).
// Stage parts in 16-byte chunks; rows padded so that 16-byte fragment reads of
// 16 consecutive rows fall in distinct banks, each part starting at a multiple
// of 64 chunks so that one copy instruction reads one buffer:
//   early: Qp [32][192+8] and dOp [32][128+8] fp16 (rows in permuted order),
//          LSE and D [32] fp32 (permuted order)
//   late:  QT [192][32+8] and dOT [128][32+8] fp16
// Padding chunks are filled with a copy of some chunk of the same part.
constexpr int QP_LD = DQK + 8, DOP_LD = DV + 8, QT_LD = 40;
constexpr int KE_QP0 = 0, KE_DOP0 = 832, KE_LSD0 = 1408, KE_CH = 1472;   // early stage (16-byte chunks)
constexpr int KL_QT0 = 0, KL_DOT0 = 960, KL_CH = 1600;                   // late stage
constexpr int KE_INSTR = KE_CH / 64, KL_INSTR = KL_CH / 64;               // copy instructions per stage (23, 25)
constexpr int KE_STAGE_B = KE_CH * 16, KL_STAGE_B = KL_CH * 16;
constexpr int KV_NST = 3;
constexpr int KV_PEX0 = KV_NST * (KE_STAGE_B + KL_STAGE_B);             // P exchange: [key block][4][64 lanes] f32x4
constexpr int KV_LDS = KV_PEX0 + 4 * 4 * 64 * 16;
static_assert(KV_LDS <= 160 * 1024, "LDS");
static_assert(KE_CH % 64 == 0 && KL_CH % 64 == 0 && KE_DOP0 % 64 == 0 && KE_LSD0 % 64 == 0 && KL_DOT0 % 64 == 0,
              "part alignment");
static_assert(KE_QP0 + 32 * QP_LD / 8 <= KE_DOP0 && KE_DOP0 + 32 * DOP_LD / 8 <= KE_LSD0 && KE_LSD0 + 16 <= KE_CH &&
              KL_QT0 + DQK * QT_LD / 8 <= KL_DOT0 && KL_DOT0 + DV * QT_LD / 8 <= KL_CH, "stage parts");
constexpr int KV_PRIO_M = 2;
constexpr int KV_MPF = 4;                     // operand fragments read ahead in an MFMA phase

// LDS writes of this wave are complete, then the workgroup barrier; no memory
// access moves across it
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// byte offset of the lane's chunk pch of an early (E) or late (L) stage in its
// source tensor (tile 0); padding chunks copy chunk 0 of their row
__device__ __forceinline__ int kv_src_early(int pch) {
  if (pch < KE_DOP0) {
    int rho = pch / (QP_LD / 8), c = pch % (QP_LD / 8);
    if (rho >= 32 || c >= DQK / 8) rho = c = 0;
    return (perm32(rho) * DQK + 8 * c) * 2;
  }
  if (pch < KE_LSD0) {
    const int p2 = pch - KE_DOP0;
    int rho = p2 / (DOP_LD / 8), c = p2 % (DOP_LD / 8);
    if (rho >= 32 || c >= DV / 8) rho = c = 0;
    return (perm32(rho) * DV + 8 * c) * 2;
  }
  const int p2 = pch - KE_LSD0;
  return (p2 < 16 ? p2 : 0) * 16;
}
__device__ __forceinline__ int kv_src_late(int pch, int sq_pad) {
  const int p2 = pch < KL_DOT0 ? pch : pch - KL_DOT0;
  const int d = p2 / (QT_LD / 8);
  int c = p2 % (QT_LD / 8);
  if (c >= 4) c = 0;
  return (d * sq_pad + 8 * c) * 2;
}

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
kv_kernel(BackwardArgs a, const uint16_t* __restrict__ qf, const uint16_t* __restrict__ qft,
          const uint16_t* __restrict__ dof, const uint16_t* __restrict__ doft, const float* __restrict__ lsdt,
          const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vrow, const uint16_t* __restrict__ krot,
          uint16_t* __restrict__ dkv, uint16_t* __restrict__ dkvt, float* __restrict__ dkr, int sq_pad, int n_kb,
          int xcd_deal) {
  __shared__ __attribute__((aligned(16))) uint8_t sm[KV_LDS];
  const ExplicitArgs& f = a.f;
  // XCD x (= blockIdx.x % 8) takes heads x, x + 8, ...: all key blocks of a
  // head run on one XCD at the same time, key block 0 (the longest) first;
  // they all walk the query tiles from the last one down, so a tile is
  // fetched once into that XCD's L2 and read there by every key block
  int kbi, bhi;
  if (xcd_deal) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    bhi = xcd + 8 * (slot / n_kb);
    kbi = slot % n_kb;
  } else {
    kbi = blockIdx.x % n_kb;
    bhi = blockIdx.x / n_kb;
  }
  const int b = bhi / f.H, h = bhi % f.H;
  const int64_t bh = (int64_t)b * f.H + h;
  const int kb = kbi * 128;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave >> 2, kw = wave & 3;          // role 0: A, 1: B; key block kw of 32 keys
  const int l32 = lane & 31, hb = lane >> 5;
  const int key = kb + kw * 32 + l32;                 // this lane's key (accumulator column)
  const float c2 = f.scale * MLA_LOG2E;

  int qt0 = 0;
  if (f.causal) {
    const int64_t first = (int64_t)kb + f.kv_pos0 - f.q_pos0;     // first query that sees key kb
    qt0 = (int)max((int64_t)0, min(first, (int64_t)sq_pad) / 32);
  }
  const int nt = sq_pad / 32 - qt0;                   // query tiles of this workgroup
  const int qlast = sq_pad / 32 - 1;                  // step r handles query tile qlast - r

  const uint32_t sm_lds = (uint32_t)(uintptr_t)(LDS_AS void*)&sm[0];
  auto est = [&](int r) __attribute__((always_inline)) { return sm + (r % KV_NST) * KE_STAGE_B; };
  auto lst = [&](int r) __attribute__((always_inline)) {
    return sm + KV_NST * KE_STAGE_B + (r % KV_NST) * KL_STAGE_B;
  };
  f32x4_t* pex = reinterpret_cast<f32x4_t*>(sm + KV_PEX0) + kw * 4 * 64;   // [4][64 lanes]

  // the B operands of the two products of each role, loaded once; then every
  // later vector-memory operation of the wave is a tile copy
  const int kk = min(key, f.s_pad - 1);
  if (role == 0) {
    // ================================ A ==================================
    f16x8_t kb_[DQK / 16];
    {
      const uint16_t* kr = kn + (bh * f.s_pad + kk) * DN;
#pragma unroll
      for (int ks = 0; ks < DN / 16; ++ks) kb_[ks] = *reinterpret_cast<const f16x8_t*>(kr + 16 * ks + 8 * hb);
      const uint16_t* rr = krot + ((int64_t)b * f.s_pad + kk) * DR;
#pragma unroll
      for (int ks = 0; ks < DR / 16; ++ks)
        kb_[DN / 16 + ks] = *reinterpret_cast<const f16x8_t*>(rr + 16 * ks + 8 * hb);
    }
    wait_vmcnt<0>();
    int voff[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) voff[i] = kv_src_early(64 * (4 * i + kw) + lane);
    const i32x4_t rs_qp = make_rsrc_uniform(qf + bh * sq_pad * DQK, (uint32_t)sq_pad * DQK * 2);
    const i32x4_t rs_dop = make_rsrc_uniform(dof + bh * sq_pad * DV, (uint32_t)sq_pad * DV * 2);
    const i32x4_t rs_lsd = make_rsrc_uniform(lsdt + bh * (sq_pad / 32) * 64, (uint32_t)(sq_pad / 32) * 256);
    const int n_mine = kw < 3 ? 6 : 5;                 // early copy instructions of this wave
    auto issue_w = [&](auto wc, int r) __attribute__((always_inline)) {
      constexpr int W = decltype(wc)::value;
      const int qt = qlast - r;
      const uint32_t st = __builtin_amdgcn_readfirstlane(sm_lds + (uint32_t)((r % KV_NST) * KE_STAGE_B));
      static_for<6>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value, n = 4 * i + W, c0 = 64 * n;
        if constexpr (n < KE_INSTR) {
          constexpr int part = c0 < KE_DOP0 ? 0 : c0 < KE_LSD0 ? 1 : 2;
          const i32x4_t& rs = part == 0 ? rs_qp : part == 1 ? rs_dop : rs_lsd;
          const int so = part == 0 ? qt * 32 * DQK * 2 : part == 1 ? qt * 32 * DV * 2 : qt * 256;
          lds_dma_b128(rs, st + (uint32_t)c0 * 16, voff[i], __builtin_amdgcn_readfirstlane(so));
        }
      });
    };
    auto issue = [&](int r) __attribute__((always_inline)) {
      if (r >= nt) return;
      if (kw == 0) issue_w(std::integral_constant<int, 0>{}, r);
      else if (kw == 1) issue_w(std::integral_constant<int, 1>{}, r);
      else if (kw == 2) issue_w(std::integral_constant<int, 2>{}, r);
      else issue_w(std::integral_constant<int, 3>{}, r);
    };
    // copies of tile r have landed given that those of tile r + 1 may be in flight
    auto wait_for = [&](int r) __attribute__((always_inline)) {
      if (r + 1 < nt) {
        if (n_mine == 6) wait_vmcnt<6>();
        else wait_vmcnt<5>();
      } else {
        wait_vmcnt<0>();
      }
    };

    f32x16_t dvt[DV / 32];
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) dvt[d] = f32x16_t{};
    f32x16_t sacc = f32x16_t{};
    auto s_mfmas = [&](int r) __attribute__((always_inline)) {
      const uint16_t* Qp = reinterpret_cast<const uint16_t*>(est(r) + KE_QP0 * 16);
      sacc = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < DQK / 16; ++ks)
        sacc = mfma(*reinterpret_cast<const f16x8_t*>(Qp + l32 * QP_LD + 16 * ks + 8 * hb), kb_[ks], sacc);
    };
    const int key_last = kb + kw * 32 + 31;
    const int dpos = (int)max((int64_t)-(1 << 30), min((int64_t)(1 << 30), f.q_pos0 - f.kv_pos0));
    f16x8_t pb[2];
    // V_A(r): P = exp2(S c2 - LSE log2 e), branch free (a masked pair gets the
    // exponent -inf); fp16 copy for dV, fp32 copy to LDS for B
    auto v_phase = [&](int r) __attribute__((always_inline)) {
      const float* lsd = reinterpret_cast<const float*>(est(r) + KE_LSD0 * 16);
      const int q0 = (qlast - r) * 32;
      const bool full = key_last < f.s_vis && q0 + 31 < f.Sq && (!f.causal || key_last - q0 <= dpos);
      f32x4_t l4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) l4[g] = *reinterpret_cast<const f32x4_t*>(lsd + 8 * g + 4 * hb);
      float p[16];
      if (__builtin_amdgcn_readfirstlane((int)full)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) p[e] = fast_exp2(sacc[e] * c2 - l4[e >> 2][e & 3] * MLA_LOG2E);
      } else {
        const bool key_ok = key < f.s_vis;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int rho = 8 * (e >> 2) + 4 * hb + (e & 3);
          const int i = q0 + perm32(rho);
          const bool vis = key_ok & (i < f.Sq) & (!f.causal | (key - i <= dpos));
          const float x = sacc[e] * c2 - l4[e >> 2][e & 3] * MLA_LOG2E;
          p[e] = fast_exp2(vis ? x : -INFINITY);
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) pb[e >> 3][e & 7] = (f16)p[e];
#pragma unroll
      for (int q = 0; q < 4; ++q) pex[q * 64 + lane] = f32x4_t{p[4 * q], p[4 * q + 1], p[4 * q + 2], p[4 * q + 3]};
    };
    // M_A(r): dV(r) += dO^T P and S(r+1) as one MFMA stream (the S chain
    // interleaved with the independent dV products), operand fragments read
    // KV_MPF ahead
    auto m_stream = [&](auto with_s, int r) __attribute__((always_inline)) {
      constexpr bool WS = decltype(with_s)::value;
      constexpr int NOPS = WS ? 20 : 8;
      const uint16_t* dOT = reinterpret_cast<const uint16_t*>(lst(r) + KL_DOT0 * 16);
      const uint16_t* Qp = reinterpret_cast<const uint16_t*>(est(r + 1) + KE_QP0 * 16);
      auto s_of = [](int k) constexpr { return !WS ? -1 : k < 16 ? ((k & 1) ? -1 : k >> 1) : k - 8; };
      auto v_of = [](int k) constexpr { return !WS ? k : k < 16 ? ((k & 1) ? k >> 1 : -1) : -1; };
      auto frag = [&](auto kc) __attribute__((always_inline)) -> f16x8_t {
        constexpr int k = decltype(kc)::value, js = s_of(k), jv = v_of(k);
        if constexpr (js >= 0) return *reinterpret_cast<const f16x8_t*>(Qp + l32 * QP_LD + 16 * js + 8 * hb);
        else return *reinterpret_cast<const f16x8_t*>(dOT + ((jv & 3) * 32 + l32) * QT_LD + 16 * (jv >> 2) + 8 * hb);
      };
      f16x8_t fr[KV_MPF + 1];
      static_for<KV_MPF>([&](auto c) __attribute__((always_inline)) {
        constexpr int k = decltype(c)::value;
        if constexpr (k < NOPS) fr[k] = frag(std::integral_constant<int, k>{});
      });
      static_for<NOPS>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value, js = s_of(k), jv = v_of(k);
        if constexpr (k + KV_MPF < NOPS)
          fr[(k + KV_MPF) % (KV_MPF + 1)] = frag(std::integral_constant<int, k + KV_MPF>{});
        if constexpr (js >= 0)
          sacc = mfma(fr[k % (KV_MPF + 1)], kb_[js], js == 0 ? f32x16_t{} : sacc);
        else
          dvt[jv & 3] = mfma(fr[k % (KV_MPF + 1)], pb[jv >> 2], dvt[jv & 3]);
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    auto iteration = [&](auto with_s, int r) __attribute__((always_inline)) {
      barrier_only();
      issue(r + 2);
      v_phase(r);
      wait_for(r + 1);
      barrier_lds();
      __builtin_amdgcn_s_setprio(KV_PRIO_M);
      m_stream(with_s, r);
      __builtin_amdgcn_s_setprio(0);
    };

    issue(0);
    issue(1);
    wait_for(0);
    __syncthreads();
    if (nt > 0) s_mfmas(0);
    // the last iteration is peeled so that the loop body holds one MFMA stream
    for (int r = 0; r + 1 < nt; ++r) iteration(std::true_type{}, r);
    if (nt > 0) iteration(std::false_type{}, nt - 1);
    barrier_only();                                   // the B waves' last phase
    // dV^T -> dKV columns DN .. DN+127 (row and column layouts)
    if (key < f.s_pad) {
      uint16_t* rowp = dkv + ((int64_t)b * f.s_pad + key) * ((int64_t)f.H * HD) + (int64_t)h * HD;
      const int64_t ncol = (int64_t)f.B * f.s_pad;
#pragma unroll
      for (int db = 0; db < DV / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + 8 * g + 4 * hb;
          u32x2_t pk;
          pk[0] = pack_f16x2(dvt[db][4 * g], dvt[db][4 * g + 1]);
          pk[1] = pack_f16x2(dvt[db][4 * g + 2], dvt[db][4 * g + 3]);
          *reinterpret_cast<u32x2_t*>(rowp + DN + d) = pk;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            dkvt[((int64_t)h * HD + DN + d + rr) * ncol + (int64_t)b * f.s_pad + key] = h_bits(dvt[db][4 * g + rr]);
        }
    }
  } else {
    // ================================ B ==================================
    f16x8_t vb_[DV / 16];
    {
      const uint16_t* vr = vrow + (bh * f.s_pad + kk) * DV;
#pragma unroll
      for (int ks = 0; ks < DV / 16; ++ks) vb_[ks] = *reinterpret_cast<const f16x8_t*>(vr + 16 * ks + 8 * hb);
    }
    wait_vmcnt<0>();
    int voff[7];
#pragma unroll
    for (int i = 0; i < 7; ++i) voff[i] = kv_src_late(64 * (4 * i + kw) + lane, sq_pad);
    const uint32_t q_bytes = (uint32_t)sq_pad * DQK * 2, o_bytes = (uint32_t)sq_pad * DV * 2;
    const i32x4_t rs_qt = make_rsrc_uniform(qft + bh * DQK * sq_pad, q_bytes);
    const i32x4_t rs_dot = make_rsrc_uniform(doft + bh * DV * sq_pad, o_bytes);
    const int n_mine = kw == 0 ? 7 : 6;                // late copy instructions of this wave
    auto issue_w = [&](auto wc, int r) __attribute__((always_inline)) {
      constexpr int W = decltype(wc)::value;
      const int qt = qlast - r;
      const uint32_t st =
          __builtin_amdgcn_readfirstlane(sm_lds + (uint32_t)(KV_NST * KE_STAGE_B + (r % KV_NST) * KL_STAGE_B));
      static_for<7>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value, n = 4 * i + W, c0 = 64 * n;
        if constexpr (n < KL_INSTR) {
          constexpr int part = c0 < KL_DOT0 ? 0 : 1;
          const i32x4_t& rs = part == 0 ? rs_qt : rs_dot;
          lds_dma_b128(rs, st + (uint32_t)c0 * 16, voff[i], __builtin_amdgcn_readfirstlane(qt * 64));
        }
      });
    };
    auto issue = [&](int r) __attribute__((always_inline)) {
      if (r >= nt) return;
      if (kw == 0) issue_w(std::integral_constant<int, 0>{}, r);
      else if (kw == 1) issue_w(std::integral_constant<int, 1>{}, r);
      else if (kw == 2) issue_w(std::integral_constant<int, 2>{}, r);
      else issue_w(std::integral_constant<int, 3>{}, r);
    };
    auto wait_for = [&](int r) __attribute__((always_inline)) {
      if (r + 1 < nt) {
        if (n_mine == 7) wait_vmcnt<7>();
        else wait_vmcnt<6>();
      } else {
        wait_vmcnt<0>();
      }
    };

    f32x16_t dkt[DQK / 32];
#pragma unroll
    for (int d = 0; d < DQK / 32; ++d) dkt[d] = f32x16_t{};
    f32x16_t pacc = f32x16_t{};
    auto dp_mfmas = [&](int r) __attribute__((always_inline)) {
      const uint16_t* dOp = reinterpret_cast<const uint16_t*>(est(r) + KE_DOP0 * 16);
      pacc = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < DV / 16; ++ks)
        pacc = mfma(*reinterpret_cast<const f16x8_t*>(dOp + l32 * DOP_LD + 16 * ks + 8 * hb), vb_[ks], pacc);
    };
    f16x8_t sb[2];
    // V_B(r): dS = P (dP - D) with P from the A wave of this key block
    auto v_phase = [&](int r) __attribute__((always_inline)) {
      const float* lsd = reinterpret_cast<const float*>(est(r) + KE_LSD0 * 16);
      f32x4_t d4[4], p4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        d4[g] = *reinterpret_cast<const f32x4_t*>(lsd + 32 + 8 * g + 4 * hb);
        p4[g] = pex[g * 64 + lane];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) sb[e >> 3][e & 7] = (f16)(p4[e >> 2][e & 3] * (pacc[e] - d4[e >> 2][e & 3]));
    };
    // M_B(r): dK(r) += Q^T dS and dP(r+1) as one MFMA stream (the dP chain
    // interleaved with the dK products), fragments read KV_MPF ahead
    auto m_stream = [&](auto with_p, int r) __attribute__((always_inline)) {
      constexpr bool WP = decltype(with_p)::value;
      constexpr int NOPS = WP ? 20 : 12;
      const uint16_t* QT = reinterpret_cast<const uint16_t*>(lst(r) + KL_QT0 * 16);
      const uint16_t* dOp = reinterpret_cast<const uint16_t*>(est(r + 1) + KE_DOP0 * 16);
      auto p_of = [](int k) constexpr { return !WP ? -1 : k < 16 ? ((k & 1) ? k >> 1 : -1) : -1; };
      auto k_of = [](int k) constexpr { return !WP ? k : k < 16 ? ((k & 1) ? -1 : k >> 1) : k - 8; };
      auto frag = [&](auto kc) __attribute__((always_inline)) -> f16x8_t {
        constexpr int k = decltype(kc)::value, jp = p_of(k), jk = k_of(k);
        if constexpr (jp >= 0) return *reinterpret_cast<const f16x8_t*>(dOp + l32 * DOP_LD + 16 * jp + 8 * hb);
        else return *reinterpret_cast<const f16x8_t*>(QT + ((jk % 6) * 32 + l32) * QT_LD + 16 * (jk / 6) + 8 * hb);
      };
      f16x8_t fr[KV_MPF + 1];
      static_for<KV_MPF>([&](auto c) __attribute__((always_inline)) {
        constexpr int k = decltype(c)::value;
        if constexpr (k < NOPS) fr[k] = frag(std::integral_constant<int, k>{});
      });
      static_for<NOPS>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value, jp = p_of(k), jk = k_of(k);
        if constexpr (k + KV_MPF < NOPS)
          fr[(k + KV_MPF) % (KV_MPF + 1)] = frag(std::integral_constant<int, k + KV_MPF>{});
        if constexpr (jp >= 0)
          pacc = mfma(fr[k % (KV_MPF + 1)], vb_[jp], jp == 0 ? f32x16_t{} : pacc);
        else
          dkt[jk % 6] = mfma(fr[k % (KV_MPF + 1)], sb[jk / 6], dkt[jk % 6]);
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    auto iteration = [&](auto with_p, int r) __attribute__((always_inline)) {
      barrier_only();
      issue(r + 2);
      v_phase(r);
      wait_for(r + 1);
      barrier_lds();                                  // P(r) read before the A wave writes P(r+1)
      __builtin_amdgcn_s_setprio(KV_PRIO_M);
      m_stream(with_p, r);
      __builtin_amdgcn_s_setprio(0);
    };

    issue(0);
    issue(1);
    wait_for(0);
    __syncthreads();
    barrier_only();                                   // one phase behind the A waves
    if (nt > 0) dp_mfmas(0);
    for (int r = 0; r + 1 < nt; ++r) iteration(std::true_type{}, r);
    if (nt > 0) iteration(std::false_type{}, nt - 1);
    // dK^T -> dKV columns 0 .. DN-1 (both layouts) and the key-band gradient
    if (key < f.s_pad) {
      uint16_t* rowp = dkv + ((int64_t)b * f.s_pad + key) * ((int64_t)f.H * HD) + (int64_t)h * HD;
      const int64_t ncol = (int64_t)f.B * f.s_pad;
#pragma unroll
      for (int db = 0; db < DQK / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + 8 * g + 4 * hb;
          float v[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) v[rr] = f.scale * dkt[db][4 * g + rr];
          if (d < DN) {
            u32x2_t pk;
            pk[0] = pack_f16x2(v[0], v[1]);
            pk[1] = pack_f16x2(v[2], v[3]);
            *reinterpret_cast<u32x2_t*>(rowp + d) = pk;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              dkvt[((int64_t)h * HD + d + rr) * ncol + (int64_t)b * f.s_pad + key] = h_bits(v[rr]);
          } else {
            *reinterpret_cast<f32x4_t*>(dkr + (bh * f.s_pad + key) * DR + (d - DN)) = f32x4_t{v[0], v[1], v[2], v[3]};
          }
        }
    }
  }
}

// -------------------------------------------------------------------- dq --
// Query-parallel kernel: per (b, h, 128 queries), 8 waves; the work of each
// 32-query block is split between two waves that share a SIMD:
//   wave A (waves 0-3) holds Q^T:  S^T = K Q^T, P, and dQ^T of the RoPE band
//                                  (+= K_rope^T dS^T, one tile late)
//   wave B (waves 4-7) holds dO^T: dP^T = V dO^T, dS = P (dP - D), and dQ^T
//                                  of the nope part (+= K_nope^T dS^T)
// P goes from A to B and dS from B to A through LDS, lane to the same lane.
// The waves alternate MFMA and vector phases, B one phase behind A:
//   M_A(t): dQ_rope(t-1), S(t+1)      V_A(t): P(t), its copy to LDS
//   M_B(t): dQ_nope(t), dP(t+1)       V_B(t): P(t) from LDS, dS(t) and its copy
// Key tiles stream through two rings of 3 stages: the early part (K_nope,
// rotated band and V rows), copied by the A waves two tiles ahead, and the
// late part (K_nope^T, band^T), copied by the B waves one tile ahead.
// Stage parts in 16-byte chunks (rows padded against bank conflicts, parts
// on 64-chunk boundaries, padding chunks copies of a chunk of the same part):
//   early: Kn [32][128+8], Kr [32][64+8], Vp [32][128+8] fp16, rows in
//          permuted key order
//   late:  KTn [128][32+8], KTr [64][32+8] fp16 (natural key order)
constexpr int KN_LD = DN + 8, KR_LD = DR + 8, VP_LD = DV + 8, KT_LD = 40;
constexpr int QE_KN0 = 0, QE_KR0 = 576, QE_VP0 = 896, QE_CH = 1472;
constexpr int QL_KTN0 = 0, QL_KTR0 = 640, QL_CH = 960;
constexpr int QE_INSTR = QE_CH / 64, QL_INSTR = QL_CH / 64;   // 23, 15
constexpr int QE_STAGE_B = QE_CH * 16, QL_STAGE_B = QL_CH * 16;
constexpr int DQ_NST = 3;
constexpr int DQ_PEX0 = DQ_NST * (QE_STAGE_B + QL_STAGE_B);    // P: [query block][4][64 lanes] f32x4
constexpr int DQ_SEX0 = DQ_PEX0 + 4 * 4 * 64 * 16;             // dS: [2][query block][2][64 lanes] f16x8
constexpr int DQ_LDS = DQ_SEX0 + 2 * 4 * 2 * 64 * 16;
static_assert(DQ_LDS <= 160 * 1024, "LDS");
static_assert(QE_KN0 + 32 * KN_LD / 8 <= QE_KR0 && QE_KR0 + 32 * KR_LD / 8 <= QE_VP0 &&
              QE_VP0 + 32 * VP_LD / 8 <= QE_CH && QL_KTN0 + DN * KT_LD / 8 <= QL_KTR0 &&
              QL_KTR0 + DR * KT_LD / 8 <= QL_CH, "stage parts");
static_assert(QE_KR0 % 64 == 0 && QE_VP0 % 64 == 0 && QE_CH % 64 == 0 && QL_KTR0 % 64 == 0 && QL_CH % 64 == 0,
              "part alignment");

__device__ __forceinline__ int dq_src_early(int pch) {
  if (pch < QE_KR0) {
    int rho = pch / (KN_LD / 8), c = pch % (KN_LD / 8);
    if (rho >= 32 || c >= DN / 8) rho = c = 0;
    return (perm32(rho) * DN + 8 * c) * 2;
  }
  if (pch < QE_VP0) {
    const int p2 = pch - QE_KR0;
    int rho = p2 / (KR_LD / 8), c = p2 % (KR_LD / 8);
    if (rho >= 32 || c >= DR / 8) rho = c = 0;
    return (perm32(rho) * DR + 8 * c) * 2;
  }
  const int p2 = pch - QE_VP0;
  int rho = p2 / (VP_LD / 8), c = p2 % (VP_LD / 8);
  if (rho >= 32 || c >= DV / 8) rho = c = 0;
  return (perm32(rho) * DV + 8 * c) * 2;
}
__device__ __forceinline__ int dq_src_late(int pch, int s_pad) {
  const int p2 = pch < QL_KTR0 ? pch : pch - QL_KTR0;
  const int d = p2 / (KT_LD / 8);
  int c = p2 % (KT_LD / 8);
  if (c >= 4) c = 0;
  return (d * s_pad + 8 * c) * 2;
}

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
dq_kernel(BackwardArgs a, const uint16_t* __restrict__ qf, const uint16_t* __restrict__ dof,
          const float* __restrict__ dvec, const uint16_t* __restrict__ kn, const uint16_t* __restrict__ krot,
          const uint16_t* __restrict__ vrow, const uint16_t* __restrict__ knt, const uint16_t* __restrict__ krt,
          const float2* __restrict__ qtab, int sq_pad, int n_qb, int xcd_deal) {
  __shared__ __attribute__((aligned(16))) uint8_t sm[DQ_LDS];
  const ExplicitArgs& f = a.f;
  // longest first: the last query block sees the most keys.  XCD x (=
  // blockIdx.x % 8) takes heads x, x + 8, ...: all query blocks of a head run
  // on one XCD at the same time and walk the key tiles in the same order, so
  // a key tile is fetched once into that XCD's L2 for all of them
  int qbi, bhi;
  if (xcd_deal) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    bhi = xcd + 8 * (slot / n_qb);
    qbi = n_qb - 1 - slot % n_qb;
  } else {
    qbi = n_qb - 1 - (int)(blockIdx.x % n_qb);
    bhi = blockIdx.x / n_qb;
  }
  const int b = bhi / f.H, h = bhi % f.H;
  const int64_t bh = (int64_t)b * f.H + h;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave >> 2, qw = wave & 3;          // role 0: A, 1: B; query block qw of 32
  const int l32 = lane & 31, hb = lane >> 5;
  const int i = qbi * 128 + qw * 32 + l32;            // this lane's query (accumulator column)
  const float c2 = f.scale * MLA_LOG2E;

  // key tiles visible to the block's last query
  int kend = f.s_vis;
  if (f.causal) {
    const int i_last = min(qbi * 128 + 127, f.Sq - 1);
    const int64_t lim = f.q_pos0 + i_last - f.kv_pos0 + 1;
    kend = (int)max((int64_t)0, min(lim, (int64_t)f.s_vis));
  }
  const int nkt = (kend + 31) / 32;

  const uint32_t sm_lds = (uint32_t)(uintptr_t)(LDS_AS void*)&sm[0];
  auto est = [&](int kt) __attribute__((always_inline)) { return sm + (kt % DQ_NST) * QE_STAGE_B; };
  auto lst = [&](int kt) __attribute__((always_inline)) {
    return sm + DQ_NST * QE_STAGE_B + (kt % DQ_NST) * QL_STAGE_B;
  };
  f32x4_t* pex = reinterpret_cast<f32x4_t*>(sm + DQ_PEX0) + qw * 4 * 64;                 // [4][64 lanes]
  auto sex = [&](int kt) __attribute__((always_inline)) {                                  // [2][64 lanes]
    return reinterpret_cast<f16x8_t*>(sm + DQ_SEX0) + ((kt & 1) * 4 + qw) * 2 * 64;
  };
  const uint32_t sp = (uint32_t)f.s_pad;

  if (role == 0) {
    // ================================ A ==================================
    f16x8_t qb_[DQK / 16];                             // B operand: lane = query, k-slots 16 ks + 8 hb ..
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks)
      qb_[ks] = *reinterpret_cast<const f16x8_t*>(qf + (bh * sq_pad + i) * DQK + 16 * ks + 8 * hb);
    const float lse = (i < f.Sq) ? a.lse[bh * f.Sq + i] : -INFINITY;
    // a row with an infinite LSE sees no key; its P is 0 through row_ok
    const bool row_ok = i < f.Sq && lse != -INFINITY;
    const float lse_l2 = row_ok ? lse * MLA_LOG2E : 0.f;
    const int dpos = (int)max((int64_t)-(1 << 30), min((int64_t)(1 << 30), f.q_pos0 - f.kv_pos0));
    // keys [0, kfull) are visible to every query of this block
    int kfull = f.s_vis;
    if (f.causal) {
      const int64_t lim = f.q_pos0 + (qbi * 128 + qw * 32) - f.kv_pos0 + 1;
      kfull = (int)max((int64_t)0, min(lim, (int64_t)f.s_vis));
    }
    const bool rows_live = qbi * 128 + qw * 32 + 31 < f.Sq;
    wait_vmcnt<0>();                                   // later vector-memory operations are tile copies
    int voff[6];
#pragma unroll
    for (int k = 0; k < 6; ++k) voff[k] = dq_src_early(64 * (4 * k + qw) + lane);
    const i32x4_t rs_kn = make_rsrc_uniform(kn + bh * f.s_pad * DN, sp * DN * 2);
    const i32x4_t rs_kr = make_rsrc_uniform(krot + (int64_t)b * f.s_pad * DR, sp * DR * 2);
    const i32x4_t rs_vp = make_rsrc_uniform(vrow + bh * f.s_pad * DV, sp * DV * 2);
    const int n_mine = qw < 3 ? 6 : 5;                 // early copy instructions of this wave
    auto issue_w = [&](auto wc, int kt) __attribute__((always_inline)) {
      constexpr int W = decltype(wc)::value;
      const uint32_t st = __builtin_amdgcn_readfirstlane(sm_lds + (uint32_t)((kt % DQ_NST) * QE_STAGE_B));
      static_for<6>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value, n = 4 * k + W, c0 = 64 * n;
        if constexpr (n < QE_INSTR) {
          constexpr int part = c0 < QE_KR0 ? 0 : c0 < QE_VP0 ? 1 : 2;
          const i32x4_t& rs = part == 0 ? rs_kn : part == 1 ? rs_kr : rs_vp;
          const int so = part == 0 ? kt * 32 * DN * 2 : part == 1 ? kt * 32 * DR * 2 : kt * 32 * DV * 2;
          lds_dma_b128(rs, st + (uint32_t)c0 * 16, voff[k], __builtin_amdgcn_readfirstlane(so));
        }
      });
    };
    auto issue = [&](int kt) __attribute__((always_inline)) {
      if (kt >= nkt) return;
      if (qw == 0) issue_w(std::integral_constant<int, 0>{}, kt);
      else if (qw == 1) issue_w(std::integral_constant<int, 1>{}, kt);
      else if (qw == 2) issue_w(std::integral_constant<int, 2>{}, kt);
      else issue_w(std::integral_constant<int, 3>{}, kt);
    };
    // copies of tile kt have landed given that those of tile kt + 1 may be in flight
    auto wait_for = [&](int kt) __attribute__((always_inline)) {
      if (kt + 1 < nkt) {
        if (n_mine == 6) wait_vmcnt<6>();
        else wait_vmcnt<5>();
      } else {
        wait_vmcnt<0>();
      }
    };

    f32x16_t dqr[DR / 32];                             // dQ^T of the RoPE band
#pragma unroll
    for (int d = 0; d < DR / 32; ++d) dqr[d] = f32x16_t{};
    f32x16_t sacc = f32x16_t{};
    auto s_mfmas = [&](int kt) __attribute__((always_inline)) {
      const uint8_t* st = est(kt);
      const uint16_t* Kn = reinterpret_cast<const uint16_t*>(st + QE_KN0 * 16);
      const uint16_t* Kr = reinterpret_cast<const uint16_t*>(st + QE_KR0 * 16);
      sacc = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < DQK / 16; ++ks) {
        const uint16_t* ap = ks < DN / 16 ? Kn + l32 * KN_LD + 16 * ks : Kr + l32 * KR_LD + 16 * (ks - DN / 16);
        sacc = mfma(*reinterpret_cast<const f16x8_t*>(ap + 8 * hb), qb_[ks], sacc);
      }
    };
    // dQ^T_rope += K_rope^T dS^T of tile kt (k-slots: keys 16u + 8hb .. in natural order)
    auto dqr_mfmas = [&](int kt) __attribute__((always_inline)) {
      const uint16_t* KTr = reinterpret_cast<const uint16_t*>(lst(kt) + QL_KTR0 * 16);
      const f16x8_t* ds = sex(kt);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const f16x8_t sbu = ds[u * 64 + lane];
#pragma unroll
        for (int db = 0; db < DR / 32; ++db)
          dqr[db] = mfma(*reinterpret_cast<const f16x8_t*>(KTr + (db * 32 + l32) * KT_LD + 16 * u + 8 * hb), sbu,
                         dqr[db]);
      }
    };
    // V_A(kt): P^T = exp2(S^T c2 - LSE log2 e), branch free (a masked pair
    // gets the exponent -inf), to LDS for B
    auto v_phase = [&](int kt) __attribute__((always_inline)) {
      const bool fast = __builtin_amdgcn_readfirstlane((int)(rows_live && kt * 32 + 32 <= kfull));
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float p[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int e = 4 * g + rr;
          const float x = sacc[e] * c2 - lse_l2;
          if (fast) {
            p[rr] = fast_exp2(x);
          } else {
            const int j = kt * 32 + perm32(8 * g + 4 * hb + rr);
            const bool vis = row_ok & (j < f.s_vis) & (!f.causal | (j - i <= dpos));
            p[rr] = fast_exp2(vis ? x : -INFINITY);
          }
        }
        pex[g * 64 + lane] = f32x4_t{p[0], p[1], p[2], p[3]};
      }
    };
    // M_A(kt): dQ_rope(kt-1) (with_r) and S(kt+1) (with_s) as one MFMA
    // stream, the S chain interleaved with the rope products, operand
    // fragments read KV_MPF ahead
    auto m_stream = [&](auto with_r, auto with_s, int kt) __attribute__((always_inline)) {
      constexpr bool WR = decltype(with_r)::value, WS = decltype(with_s)::value;
      constexpr int NR = WR ? 4 : 0, NS = WS ? 12 : 0, NOPS = NR + NS;
      const uint8_t* st = est(WS ? kt + 1 : kt);
      const uint16_t* Kn = reinterpret_cast<const uint16_t*>(st + QE_KN0 * 16);
      const uint16_t* Kr = reinterpret_cast<const uint16_t*>(st + QE_KR0 * 16);
      const uint16_t* KTr = reinterpret_cast<const uint16_t*>(lst(WR ? kt - 1 : kt) + QL_KTR0 * 16);
      // op k: rope product k/2 for odd k < 2 NR when both run, else the S chain
      auto r_of = [](int k) constexpr { return !WR ? -1 : !WS ? k : (k < 2 * NR && (k & 1)) ? k >> 1 : -1; };
      auto s_of = [](int k) constexpr {
        return !WS ? -1 : !WR ? k : k < 2 * NR ? ((k & 1) ? -1 : k >> 1) : k - NR;
      };
      auto frag = [&](auto kc) __attribute__((always_inline)) -> f16x8_t {
        constexpr int k = decltype(kc)::value, jr = r_of(k), js = s_of(k);
        if constexpr (jr >= 0) {
          // rope product jr: u = jr / 2, d-block jr % 2
          return *reinterpret_cast<const f16x8_t*>(KTr + ((jr & 1) * 32 + l32) * KT_LD + 16 * (jr >> 1) + 8 * hb);
        } else {
          const uint16_t* ap = js < DN / 16 ? Kn + l32 * KN_LD + 16 * js : Kr + l32 * KR_LD + 16 * (js - DN / 16);
          return *reinterpret_cast<const f16x8_t*>(ap + 8 * hb);
        }
      };
      f16x8_t dsu[2];
      if constexpr (WR) {
        const f16x8_t* ds = sex(kt - 1);
        dsu[0] = ds[lane];
        dsu[1] = ds[64 + lane];
      }
      f16x8_t fr[KV_MPF + 1];
      static_for<KV_MPF>([&](auto c) __attribute__((always_inline)) {
        constexpr int k = decltype(c)::value;
        if constexpr (k < NOPS) fr[k] = frag(std::integral_constant<int, k>{});
      });
      static_for<NOPS>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value, jr = r_of(k), js = s_of(k);
        if constexpr (k + KV_MPF < NOPS)
          fr[(k + KV_MPF) % (KV_MPF + 1)] = frag(std::integral_constant<int, k + KV_MPF>{});
        if constexpr (jr >= 0)
          dqr[jr & 1] = mfma(fr[k % (KV_MPF + 1)], dsu[jr >> 1], dqr[jr & 1]);
        else
          sacc = mfma(fr[k % (KV_MPF + 1)], qb_[js], js == 0 ? f32x16_t{} : sacc);
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    auto iteration = [&](auto with_r, auto with_s, int kt) __attribute__((always_inline)) {
      barrier_only();
      issue(kt + 2);
      v_phase(kt);
      wait_for(kt + 1);
      barrier_lds();
      __builtin_amdgcn_s_setprio(KV_PRIO_M);
      m_stream(with_r, with_s, kt);
      __builtin_amdgcn_s_setprio(0);
    };

    issue(0);
    issue(1);
    wait_for(0);
    __syncthreads();
    if (nkt > 0) s_mfmas(0);
    // the first and the last iterations are peeled so that the loop body
    // holds one MFMA stream
    if (nkt == 1) iteration(std::false_type{}, std::false_type{}, 0);
    if (nkt > 1) iteration(std::false_type{}, std::true_type{}, 0);
    for (int kt = 1; kt + 1 < nkt; ++kt) iteration(std::true_type{}, std::true_type{}, kt);
    if (nkt > 1) iteration(std::true_type{}, std::false_type{}, nkt - 1);
    barrier_only();                                   // dS of the last tile is in LDS
    if (nkt > 0) dqr_mfmas(nkt - 1);
    // dq_pe: rows 128 + m (block 0) and 128 + m + 32 (block 1) sit in the same
    // lane and element; rotated back by the negative angle
    if (i < f.Sq) {
      const int64_t row = ((int64_t)b * f.Sq + i) * f.H + h;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 8 * g + 4 * hb + r;
          const float lo = f.scale * dqr[0][4 * g + r], hi = f.scale * dqr[1][4 * g + r];
          const float2 cs = qtab[(int64_t)i * 32 + m];
          a.dq_pe[row * DR + m] = lo * cs.x + hi * cs.y;
          a.dq_pe[row * DR + m + 32] = hi * cs.x - lo * cs.y;
        }
    }
  } else {
    // ================================ B ==================================
    f16x8_t ob_[DV / 16];                              // B operand: lane = query
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
      ob_[ks] = *reinterpret_cast<const f16x8_t*>(dof + (bh * sq_pad + i) * DV + 16 * ks + 8 * hb);
    const float dd = dvec[bh * sq_pad + i];
    wait_vmcnt<0>();
    int voff[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) voff[k] = dq_src_late(64 * (4 * k + qw) + lane, f.s_pad);
    const i32x4_t rs_ktn = make_rsrc_uniform(knt + bh * DN * f.s_pad, sp * DN * 2);
    const i32x4_t rs_ktr = make_rsrc_uniform(krt + (int64_t)b * DR * f.s_pad, sp * DR * 2);
    const int n_mine = qw < 3 ? 4 : 3;                 // late copy instructions of this wave
    auto issue_w = [&](auto wc, int kt) __attribute__((always_inline)) {
      constexpr int W = decltype(wc)::value;
      const uint32_t st =
          __builtin_amdgcn_readfirstlane(sm_lds + (uint32_t)(DQ_NST * QE_STAGE_B + (kt % DQ_NST) * QL_STAGE_B));
      static_for<4>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value, n = 4 * k + W, c0 = 64 * n;
        if constexpr (n < QL_INSTR) {
          constexpr int part = c0 < QL_KTR0 ? 0 : 1;
          const i32x4_t& rs = part == 0 ? rs_ktn : rs_ktr;
          lds_dma_b128(rs, st + (uint32_t)c0 * 16, voff[k], __builtin_amdgcn_readfirstlane(kt * 64));
        }
      });
    };
    auto issue = [&](int kt) __attribute__((always_inline)) {
      if (kt >= nkt) return;
      if (qw == 0) issue_w(std::integral_constant<int, 0>{}, kt);
      else if (qw == 1) issue_w(std::integral_constant<int, 1>{}, kt);
      else if (qw == 2) issue_w(std::integral_constant<int, 2>{}, kt);
      else issue_w(std::integral_constant<int, 3>{}, kt);
    };
    auto wait_for = [&](int kt) __attribute__((always_inline)) {
      if (kt + 1 < nkt) {
        if (n_mine == 4) wait_vmcnt<4>();
        else wait_vmcnt<3>();
      } else {
        wait_vmcnt<0>();
      }
    };

    f32x16_t dqn[DN / 32];                             // dQ^T of the nope part
#pragma unroll
    for (int d = 0; d < DN / 32; ++d) dqn[d] = f32x16_t{};
    f32x16_t pacc = f32x16_t{};
    auto dp_mfmas = [&](int kt) __attribute__((always_inline)) {
      const uint16_t* Vp = reinterpret_cast<const uint16_t*>(est(kt) + QE_VP0 * 16);
      pacc = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < DV / 16; ++ks)
        pacc = mfma(*reinterpret_cast<const f16x8_t*>(Vp + l32 * VP_LD + 16 * ks + 8 * hb), ob_[ks], pacc);
    };
    f16x8_t sb[2];
    // V_B(kt): dS^T = P^T (dP^T - D) with P from the A wave of this block
    auto v_phase = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4_t p4 = pex[g * 64 + lane];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int e = 4 * g + rr;
          sb[e >> 3][e & 7] = (f16)(p4[rr] * (pacc[e] - dd));
        }
      }
      f16x8_t* ds = sex(kt);
      ds[lane] = sb[0];
      ds[64 + lane] = sb[1];
    };
    // M_B(kt): dQ_nope(kt) and dP(kt+1) as one MFMA stream (the dP chain
    // interleaved with the nope products), fragments read KV_MPF ahead
    auto m_stream = [&](auto with_p, int kt) __attribute__((always_inline)) {
      constexpr bool WP = decltype(with_p)::value;
      constexpr int NOPS = WP ? 16 : 8;
      const uint16_t* KTn = reinterpret_cast<const uint16_t*>(lst(kt) + QL_KTN0 * 16);
      const uint16_t* Vp = reinterpret_cast<const uint16_t*>(est(kt + 1) + QE_VP0 * 16);
      auto n_of = [](int k) constexpr { return !WP ? k : (k & 1) ? -1 : k >> 1; };
      auto p_of = [](int k) constexpr { return !WP ? -1 : (k & 1) ? k >> 1 : -1; };
      auto frag = [&](auto kc) __attribute__((always_inline)) -> f16x8_t {
        constexpr int k = decltype(kc)::value, jn = n_of(k), jp = p_of(k);
        if constexpr (jn >= 0)   // nope product jn: u = jn / 4, d-block jn % 4
          return *reinterpret_cast<const f16x8_t*>(KTn + ((jn & 3) * 32 + l32) * KT_LD + 16 * (jn >> 2) + 8 * hb);
        else
          return *reinterpret_cast<const f16x8_t*>(Vp + l32 * VP_LD + 16 * jp + 8 * hb);
      };
      f16x8_t fr[KV_MPF + 1];
      static_for<KV_MPF>([&](auto c) __attribute__((always_inline)) {
        constexpr int k = decltype(c)::value;
        if constexpr (k < NOPS) fr[k] = frag(std::integral_constant<int, k>{});
      });
      static_for<NOPS>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value, jn = n_of(k), jp = p_of(k);
        if constexpr (k + KV_MPF < NOPS)
          fr[(k + KV_MPF) % (KV_MPF + 1)] = frag(std::integral_constant<int, k + KV_MPF>{});
        if constexpr (jn >= 0)
          dqn[jn & 3] = mfma(fr[k % (KV_MPF + 1)], sb[jn >> 2], dqn[jn & 3]);
        else
          pacc = mfma(fr[k % (KV_MPF + 1)], ob_[jp], jp == 0 ? f32x16_t{} : pacc);
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    auto iteration = [&](auto with_p, int kt) __attribute__((always_inline)) {
      barrier_only();
      issue(kt + 1);
      v_phase(kt);
      wait_for(kt);
      barrier_lds();                                  // P(kt) read and dS(kt) written before A goes on
      __builtin_amdgcn_s_setprio(KV_PRIO_M);
      m_stream(with_p, kt);
      __builtin_amdgcn_s_setprio(0);
    };

    issue(0);
    wait_vmcnt<0>();
    __syncthreads();
    barrier_only();                                   // one phase behind the A waves
    if (nkt > 0) dp_mfmas(0);
    for (int kt = 0; kt + 1 < nkt; ++kt) iteration(std::true_type{}, kt);
    if (nkt > 0) iteration(std::false_type{}, nkt - 1);
    if (i < f.Sq) {
      const int64_t row = ((int64_t)b * f.Sq + i) * f.H + h;
#pragma unroll
      for (int db = 0; db < DN / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + 8 * g + 4 * hb;
          *reinterpret_cast<f32x4_t*>(a.dq_nope + row * DN + d) =
              f32x4_t{f.scale * dqn[db][4 * g], f.scale * dqn[db][4 * g + 1], f.scale * dqn[db][4 * g + 2],
                      f.scale * dqn[db][4 * g + 3]};
        }
    }
  }
}

// ------------------------------------------------------------------ dk_pe --
// dk_pe[b, j, (m, m+32)] = R^T(sum_h dkr[b, h, j, :]); zero for j >= s_vis
__global__ void dk_pe_kernel(BackwardArgs a, const float* __restrict__ dkr, const float2* __restrict__ ktab) {
  const ExplicitArgs& f = a.f;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)f.B * f.Skv * 32) return;
  const int m = (int)(idx & 31);
  const int64_t bj = idx >> 5;
  const int j = (int)(bj % f.Skv), b = (int)(bj / f.Skv);
  float lo = 0.f, hi = 0.f;
  if (j < f.s_vis) {
    for (int h = 0; h < f.H; ++h) {
      const float* g = dkr + (((int64_t)b * f.H + h) * f.s_pad + j) * DR;
      lo += g[m];
      hi += g[m + 32];
    }
    const float2 cs = ktab[(int64_t)j * 32 + m];
    const float l2 = lo * cs.x + hi * cs.y, h2 = hi * cs.x - lo * cs.y;
    lo = l2;
    hi = h2;
  }
  a.dk_pe[bj * DR + m] = lo;
  a.dk_pe[bj * DR + m + 32] = hi;
}

// ---------------------------------------------------------------- gemm_nt --
// C[m][n] = sum_k A[m][k] B[n][k]: dc_kv = dKV W and dW = dKV^T c_kv.  A [M][K]
// and B [N][K] fp16 row-major, M, N multiples of 256, K a multiple of 32.
// Tile 256 x 256, one workgroup of 8 waves (two per SIMD); wave w computes rows
// 128 (w & 1) .. +127 and columns 64 (w >> 1) .. +63 of the tile on 32x32x16
// MFMAs with the accumulators in AGPRs.  The reduction streams in steps of 32
// through a ring of 4 LDS stages (16 KB of A rows + 16 KB of B rows), filled
// by buffer->LDS copies: waves 0-3 issue theirs at the start of a step, waves
// 4-7 after their first 8 MFMAs of it, so one wave of each SIMD keeps the
// matrix unit busy while the other is held issuing.  Rows of 32 elements
// (4 chunks of 16 bytes) hold chunk c at c ^ ((r >> 2) & 3).
// With ksplit > 1 the reduction is cut into ksplit slices of kchunk; slice s
// writes its fp32 sum to part[s] (row-major M x N) and gemm_reduce_kernel adds
// the slices.  Otherwise the result goes straight to C, row m at
// (m / map_div) * map_stride + m % map_div (a batch of row blocks stored with
// their own stride) and only rows with m % map_div < m_store.
// Workgroups: the n_tn column tiles of one (row tile, slice) run on one XCD
// (blockIdx.x % 8, the dispatcher's order), so its A block reaches that XCD's
// L2 once for all of them.
constexpr int GT = 256, GKS = 32, GNST = 4;
constexpr int G_REG = GT * GKS * 2;                 // one operand region of a stage (16 KB)
constexpr int G_STAGE = 2 * G_REG;
constexpr int G_THREADS = 512;
__global__ void __launch_bounds__(G_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_nt_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, float* __restrict__ C,
               float* __restrict__ part, int M, int N, int K, int kchunk, int ksplit, int m_store, int64_t ldc,
               int64_t map_div, int64_t map_stride) {
  __shared__ __attribute__((aligned(16))) uint16_t Ls[GNST * G_STAGE / 2];
  const int n_tm = M / GT, n_tn = N / GT;
  const int n_groups = n_tm * ksplit;                // (row tile, slice) pairs
  int tm, tn, sl;
  {
    int gi;
    if (n_groups % 8 == 0) {
      const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
      gi = xcd + 8 * (slot / n_tn);
      tn = slot % n_tn;
    } else {
      gi = blockIdx.x / n_tn;
      tn = blockIdx.x % n_tn;
    }
    tm = gi % n_tm;
    sl = gi / n_tm;
  }
  const int m0 = tm * GT, n0 = tn * GT, k0 = sl * kchunk;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hb = lane >> 5;
  const int wr = 128 * (wave & 1), wc = 64 * (wave >> 1);

  // copy instruction i (0, 1) of an operand covers stage slot 512 i + tid:
  // row 128 i + tid / 4, physical chunk tid & 3, which holds logical chunk
  // (tid & 3) ^ ((tid >> 4) & 3) of that row
  const int v_lane = (tid >> 2) * (K * 2) + (((tid & 3) ^ ((tid >> 4) & 3)) * 16);
  const i32x4_t ra = make_rsrc_uniform(A + (int64_t)m0 * K, (uint32_t)GT * K * 2);
  const i32x4_t rb = make_rsrc_uniform(B + (int64_t)n0 * K, (uint32_t)GT * K * 2);
  const uint32_t ls_lds = (uint32_t)(uintptr_t)(LDS_AS void*)&Ls[0];
  auto issue_step = [&](int g) __attribute__((always_inline)) {
    const uint32_t dst = ls_lds + (uint32_t)((g % GNST) * G_STAGE) + (uint32_t)wave * 1024u;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int so = __builtin_amdgcn_readfirstlane(i * 128 * (K * 2) + (k0 + g * GKS) * 2);
      lds_dma_b128(ra, dst + i * (G_THREADS * 16), v_lane, so);
      lds_dma_b128(rb, dst + G_REG + i * (G_THREADS * 16), v_lane, so);
    }
  };
  constexpr int LOADS = 4;                           // copies per wave per step
  const int sw = (l32 >> 2) & 3;
  const int fo0 = l32 * (GKS * 2) + ((0 + hb) ^ sw) * 16;
  const int fo1 = l32 * (GKS * 2) + ((2 + hb) ^ sw) * 16;

  f32x16_t acc[4][2];
  const int nk = kchunk / GKS;
  for (int g = 0; g < GNST - 1 && g < nk; ++g) issue_step(g);
  for (int g = 0; g < nk; ++g) {
    // the copies of step g have landed (later steps may still be in flight)
    const int newer = min(GNST - 2, nk - 1 - g);
    if (newer >= 2) wait_vmcnt<2 * LOADS>();
    else if (newer == 1) wait_vmcnt<LOADS>();
    else wait_vmcnt<0>();
    __syncthreads();                                 // ... for every wave; the stage of step g-1 is free
    const bool issue_now = g + GNST - 1 < nk;
    if (wave < 4 && issue_now) issue_step(g + GNST - 1);
    const char* st = reinterpret_cast<const char*>(Ls) + (g % GNST) * G_STAGE;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int fo = kk ? fo1 : fo0;
      f16x8_t fa[4], fb[2];
#pragma unroll
      for (int x = 0; x < 4; ++x) fa[x] = *reinterpret_cast<const f16x8_t*>(st + (wr + 32 * x) * (GKS * 2) + fo);
#pragma unroll
      for (int y = 0; y < 2; ++y)
        fb[y] = *reinterpret_cast<const f16x8_t*>(st + G_REG + (wc + 32 * y) * (GKS * 2) + fo);
      if (kk == 0 && g == 0) {
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int y = 0; y < 2; ++y)
            asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=a"(acc[x][y]) : "v"(fa[x]), "v"(fb[y]));
      } else {
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int y = 0; y < 2; ++y)
            asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc[x][y]) : "v"(fa[x]), "v"(fb[y]));
      }
      if (kk == 0 && wave >= 4 && issue_now) issue_step(g + GNST - 1);
    }
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::);
  // D element e of block (x, y): row wr + 32x + 8(e/4) + 4hb + e%4, column wc + 32y + l32
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      asm volatile("" : "+a"(acc[x][y]));
      const int n = n0 + wc + 32 * y + l32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wr + 32 * x + 8 * (e >> 2) + 4 * hb + (e & 3);
        if (ksplit > 1) {
          part[((int64_t)sl * M + m) * N + n] = acc[x][y][e];
        } else {
          const int64_t mb = m / map_div, mr = m % map_div;
          if (mr < m_store) C[(mb * map_stride + mr) * ldc + n] = acc[x][y][e];
        }
      }
    }
}

// C (row map as in gemm_nt_kernel) = sum over the ksplit slices of part,
// four columns per thread
__global__ void __launch_bounds__(256)
gemm_reduce_kernel(const float* __restrict__ part, float* __restrict__ C, int M, int N, int ksplit, int m_store,
                   int64_t ldc, int64_t map_div, int64_t map_stride) {
  const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i4 >= (int64_t)M * N / 4) return;
  const int64_t m = i4 * 4 / N, n = i4 * 4 % N;
  const int64_t mb = m / map_div, mr = m % map_div;
  if (mr >= m_store) return;
  f32x4_t s = *reinterpret_cast<const f32x4_t*>(part + m * N + n);
  for (int k = 1; k < ksplit; ++k) s += *reinterpret_cast<const f32x4_t*>(part + ((int64_t)k * M + m) * N + n);
  *reinterpret_cast<f32x4_t*>(C + (mb * map_stride + mr) * ldc + n) = s;
}

}  // namespace

size_t mfma_backward_workspace(const ExplicitArgs& f, MfmaBwdWorkspace* w, char* base) {
  const size_t B = f.B, H = f.H, sq_pad = (size_t)(f.Sq + 127) / 128 * 128, sp = f.s_pad;
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    const size_t o = off;
    off = (off + bytes + 255) / 256 * 256;
    return base == nullptr ? nullptr : base + o;
  };
  char* p;
  p = take(8 * (size_t)f.Sq * 32);             if (w) w->qtab = reinterpret_cast<float2*>(p);
  p = take(8 * sp * 32);                       if (w) w->ktab = reinterpret_cast<float2*>(p);
  p = take(2 * B * H * sp * DN);               if (w) w->kn = reinterpret_cast<uint16_t*>(p);
  p = take(2 * B * sp * DR);                   if (w) w->krot = reinterpret_cast<uint16_t*>(p);
  p = take(2 * B * H * sq_pad * DQK);          if (w) w->qf = reinterpret_cast<uint16_t*>(p);
  p = take(2 * B * H * DQK * sq_pad);          if (w) w->qft = reinterpret_cast<uint16_t*>(p);
  p = take(2 * B * H * sq_pad * DV);           if (w) w->dof = reinterpret_cast<uint16_t*>(p);
  p = take(2 * B * H * DV * sq_pad);           if (w) w->doft = reinterpret_cast<uint16_t*>(p);
  p = take(4 * B * H * sq_pad);                if (w) w->dvec = reinterpret_cast<float*>(p);
  p = take(4 * B * H * sq_pad * 2);            if (w) w->lsdt = reinterpret_cast<float*>(p);
  p = take(2 * B * H * sp * DV);               if (w) w->vrow = reinterpret_cast<uint16_t*>(p);
  p = take(2 * B * H * DN * sp);               if (w) w->knt = reinterpret_cast<uint16_t*>(p);
  p = take(2 * B * DR * sp);                   if (w) w->krt = reinterpret_cast<uint16_t*>(p);
  p = take(2 * B * sp * H * HD);               if (w) w->dkv = reinterpret_cast<uint16_t*>(p);
  p = take(2 * H * HD * B * sp);               if (w) w->dkvt = reinterpret_cast<uint16_t*>(p);
  p = take(4 * B * H * sp * DR);               if (w) w->dkr = reinterpret_cast<float*>(p);
  p = take(2 * (size_t)DKV * H * HD);          if (w) w->wt = reinterpret_cast<uint16_t*>(p);
  p = take(2 * (size_t)DKV * B * sp);          if (w) w->ct = reinterpret_cast<uint16_t*>(p);
  if (w) w->sq_pad = (int)sq_pad;
  return off;
}

namespace {
// out[z][c][r] = in[z][r][c] over rows x cols (rows >= rows_valid read as 0)
template <bool IN_BF16>
hipError_t transpose(const uint16_t* in, uint16_t* out, int rows, int rows_valid, int cols, int64_t in_ld,
                     int64_t in_bs, int64_t out_ld, int64_t out_bs, int nbatch, hipStream_t s) {
  if (rows == 0 || cols == 0 || nbatch == 0) return hipSuccess;
  // 16-byte pieces need 8-element multiples and 16-byte aligned rows
  const bool wide = rows % 8 == 0 && cols % 8 == 0 && in_ld % 8 == 0 && in_bs % 8 == 0 && out_ld % 8 == 0 &&
                    out_bs % 8 == 0 && reinterpret_cast<uintptr_t>(in) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(out) % 16 == 0;
  if (wide)
    hipLaunchKernelGGL(transpose64_kernel<IN_BF16>, dim3((cols + 63) / 64, (rows + 63) / 64, nbatch), dim3(256), 0, s,
                       in, out, rows, rows_valid, cols, in_ld, in_bs, out_ld, out_bs);
  else
    hipLaunchKernelGGL(transpose_kernel<IN_BF16>, dim3((cols + 31) / 32, (rows + 31) / 32, nbatch), dim3(256), 0, s,
                       in, out, rows, rows_valid, cols, in_ld, in_bs, out_ld, out_bs);
  return hipGetLastError();
}

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t rows, int64_t row_len, int64_t skip_rows,
                                 int64_t batch_rows) {
  // zero rows [skip_rows, batch_rows) of each batch of batch_rows rows
  const int64_t per = (batch_rows - skip_rows) * row_len;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * per) return;
  const int64_t z = idx / per, r = idx % per;
  p[z * batch_rows * row_len + skip_rows * row_len + r] = 0.f;
}
}  // namespace

hipError_t launch_bwd_prep(const BackwardArgs& a, const MfmaBwdWorkspace& w, hipStream_t s) {
  const ExplicitArgs& f = a.f;
  const int sp = f.s_pad, B = f.B, H = f.H;
  hipError_t e;
  if (w.sq_pad > 0) {
    if (f.out_dt == MLA_BF16)
      hipLaunchKernelGGL(prep_q_kernel<MLA_BF16>, dim3(w.sq_pad / 32, H, B), dim3(256), 0, s, a, w.qtab, w.qf, w.qft,
                         w.dof, w.doft, w.dvec, w.lsdt, w.sq_pad);
    else
      hipLaunchKernelGGL(prep_q_kernel<MLA_FP32>, dim3(w.sq_pad / 32, H, B), dim3(256), 0, s, a, w.qtab, w.qf, w.qft,
                         w.dof, w.doft, w.dvec, w.lsdt, w.sq_pad);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // (V comes from the up-projection in the row layout vrow[bh][key][d].)
  // K_nope columns: kn[bh][key][d] -> knt[bh][d][key]
  if ((e = transpose<false>(w.kn, w.knt, sp, sp, DN, DN, (int64_t)sp * DN, sp, (int64_t)DN * sp, B * H, s)) != hipSuccess)
    return e;
  // rotated key band: krot[b][key][d] -> krt[b][d][key]
  if ((e = transpose<false>(w.krot, w.krt, sp, sp, DR, DR, (int64_t)sp * DR, sp, (int64_t)DR * sp, B, s)) != hipSuccess)
    return e;
  // W^T [512][H*256] (fp16)
  if ((e = transpose<true>(static_cast<const uint16_t*>(f.w), w.wt, H * HD, H * HD, DKV, DKV, 0, (int64_t)H * HD, 0, 1,
                           s)) != hipSuccess)
    return e;
  // c_kv^T [512][B*sp] (fp16), rows past the visible keys zero
  return transpose<true>(static_cast<const uint16_t*>(f.c_kv), w.ct, sp, f.s_vis, DKV, DKV, (int64_t)f.Skv * DKV,
                         (int64_t)B * sp, sp, B, s);
}

hipError_t launch_bwd_kv(const BackwardArgs& a, const MfmaBwdWorkspace& w, hipStream_t s) {
  const ExplicitArgs& f = a.f;
  if (f.s_pad == 0) return hipSuccess;
  const int n_kb = f.s_pad / 128;
  const int xcd_deal = (f.B * f.H) % 8 == 0 ? 1 : 0;
  hipLaunchKernelGGL(kv_kernel, dim3(f.B * f.H * n_kb), dim3(512), 0, s, a, w.qf, w.qft, w.dof, w.doft, w.lsdt, w.kn,
                     w.vrow, w.krot, w.dkv, w.dkvt, w.dkr, w.sq_pad, n_kb, xcd_deal);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BackwardArgs& a, const MfmaBwdWorkspace& w, hipStream_t s) {
  const ExplicitArgs& f = a.f;
  if (f.Sq == 0) return hipSuccess;
  const int n_qb = w.sq_pad / 128;
  const int xcd_deal = (f.B * f.H) % 8 == 0 ? 1 : 0;
  hipLaunchKernelGGL(dq_kernel, dim3(f.B * f.H * n_qb), dim3(512), 0, s, a, w.qf, w.dof, w.dvec, w.kn, w.krot, w.vrow,
                     w.knt, w.krt, w.qtab, w.sq_pad, n_qb, xcd_deal);
  return hipGetLastError();
}

hipError_t launch_bwd_dkpe(const BackwardArgs& a, const MfmaBwdWorkspace& w, hipStream_t s) {
  const ExplicitArgs& f = a.f;
  const int64_t n = (int64_t)f.B * f.Skv * 32;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(dk_pe_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, w.dkr, w.ktab);
  return hipGetLastError();
}

namespace {
// C = A B^T on gemm_nt_kernel.  When the 256 x 256 tiles alone cannot fill the
// CUs, the reduction is cut into up to 8 slices whose fp32 sums go to the
// workspace's fp16 query operands (qf, dead once the two attention-backward
// kernels have run) and are added by gemm_reduce_kernel.
hipError_t gemm_nt(const uint16_t* A, const uint16_t* Bm, float* C, int M, int N, int K, int m_store, int64_t ldc,
                   int64_t map_div, int64_t map_stride, const MfmaBwdWorkspace& w, const ExplicitArgs& f,
                   hipStream_t s) {
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n_cu = 256;
  const int n_tiles = (M / GT) * (N / GT);
  const size_t part_room = 2 * (size_t)f.B * f.H * w.sq_pad * DQK;   // bytes of qf
  int ksplit = 1;
  while (ksplit < 8 && n_tiles * ksplit * 2 <= n_cu && K % (2 * ksplit * GKS) == 0 && K / (2 * ksplit) >= 256 &&
         (size_t)2 * ksplit * M * N * 4 <= part_room)
    ksplit *= 2;
  float* part = ksplit > 1 ? reinterpret_cast<float*>(w.qf) : nullptr;
  hipLaunchKernelGGL(gemm_nt_kernel, dim3((unsigned)(n_tiles * ksplit)), dim3(G_THREADS), 0, s, A, Bm, C, part, M, N,
                     K, K / ksplit, ksplit, m_store, ldc, map_div, map_stride);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ksplit == 1) return e;
  const int64_t n4 = (int64_t)M * N / 4;
  hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, part, C, M, N, ksplit,
                     m_store, ldc, map_div, map_stride);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_bwd_gemms(const BackwardArgs& a, const MfmaBwdWorkspace& w, hipStream_t s) {
  const ExplicitArgs& f = a.f;
  const int B = f.B, H = f.H, sp = f.s_pad;
  hipError_t e;
  // dc_kv rows of each batch entry past the computed ones (keys no query sees)
  if (f.Skv > sp) {
    const int64_t n = (int64_t)B * (f.Skv - sp) * DKV;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.dc_kv, (int64_t)B,
                       (int64_t)DKV, (int64_t)sp, (int64_t)f.Skv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (sp > 0) {
    // dc_kv[b][j][c] = sum_k dKV[b sp + j][k] W^T[c][k]   (rows j < min(sp, Skv) of each entry)
    if ((e = gemm_nt(w.dkv, w.wt, a.dc_kv, B * sp, DKV, H * HD, min(sp, f.Skv), (int64_t)DKV, (int64_t)sp,
                     (int64_t)f.Skv, w, f, s)) != hipSuccess)
      return e;
    // dW[r][c] = sum_{b, j} dKV^T[r][b sp + j] c^T[c][b sp + j]
    const int Mw = H * HD;
    return gemm_nt(w.dkvt, w.ct, a.dw, Mw, DKV, B * sp, Mw, (int64_t)DKV, (int64_t)Mw, (int64_t)Mw, w, f, s);
  }
  // no visible key: every weight gradient is zero
  const int64_t n = (int64_t)H * HD * DKV;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.dw, (int64_t)1, n,
                     (int64_t)0, (int64_t)1);
  return hipGetLastError();
}
