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
// Layout of the work: a workgroup owns 256 query rows of one (batch, head),
// 4 waves of 64 rows each, one wave per SIMD with the whole register file.
// A wave computes S^T = K Q^T on 32x32x16 MFMAs for two 32-row query blocks,
// so every K fragment read from LDS feeds two MFMAs (and every V^T fragment
// of O^T += V^T P^T as well): LDS traffic per MFMA is half of what 32 rows
// per wave need, which is what bounds this loop on gfx950.  Q^T (192 x 64,
// fp16) and the O^T accumulators
// (128 x 64) live in AGPRs; the S^T accumulators of two tiles live in VGPRs,
// where the softmax reads them.
//
// Key order.  Inside each 32-key block the K rows sit in LDS in a permuted
// order: LDS row 8g + 4x + r (the accumulator row that lane half x holds in
// element 4g + r) carries key 16(g/2) + 8x + 4(g%2) + r.  The 8 scores a lane
// holds in elements 8u .. 8u+7 are then the keys 16u + 8x .. 16u + 8x + 7,
// contiguous, which is exactly the k-slot run the lane supplies to the
// O^T += V^T P^T MFMA.  P therefore goes from the S accumulator to the B
// operand of the next product inside the lane.
//
// Tiles.  K (64 x 192, as a K_nope part and a rope part) and V^T (128 x 64)
// tiles are copied from global memory straight into LDS (buffer loads to LDS,
// 16 bytes per lane, 10 per lane per tile) through a ring of 4 stages.  In
// every tile row the 16-byte chunks are XOR-swizzled by row so that the
// 16-byte operand reads of 16 consecutive lanes fall in distinct banks.
//
// Schedule.  Iteration T issues, as one MFMA stream, the S of tile T+1 (48
// MFMAs) and the PV of tile T (32 MFMAs), and spreads the softmax of tile T
// over that stream in 72 small units, one after each of the first 72 MFMAs
// (an exponential, a row-sum add and every other step a 3-way max, or the
// fp16 packing of 8 probabilities): the matrix unit and the vector ALU of the
// SIMD work at the same time inside the one wave.  The softmax of a key step
// is done before the PV MFMAs of that step.
//
// Softmax reference.  A row's reference max is the max of its first tile
// with a visible key; P = exp2(s - ref) stays below 2^tau in fp16.  A tile
// whose max exceeds the reference by more than tau flags the workgroup, which
// then recomputes all its rows from their exact maxima (seen by the first
// pass), so the accumulators are only ever touched by MFMAs.
//
// Workgroups are dealt so that all query tiles of one head run on the same
// XCD (its L2 holds that head's K/V), longest first.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int QW = 64;            // query rows per wave (two 32-row blocks)
constexpr int NW = 4;             // waves per workgroup
constexpr int QT = QW * NW;       // query rows per workgroup
constexpr int KT = 64;            // keys per tile
constexpr int DN = 128, DR = 64, DQK = 192, DV = 128;
constexpr int NTHREADS = NW * 64;
constexpr int KS = DQK / 16;      // S k-steps (12)
// Ring stage layout (16-byte chunks, 128-byte rows whose chunks are
// XOR-swizzled by row):
//   K_nope part  [2 halves][64 rows][8 chunks]   chunks    0 .. 1023
//   rope part    [64 rows][8 chunks]             chunks 1024 .. 1535
//   V^T          [128 rows][8 chunks]            chunks 1536 .. 2559
// (half x of a K_nope row holds d = 64x .. 64x+63).  With one row length the
// operand reads of every k-step take one of four per-lane offsets plus a
// constant.
// Copy instruction g (64 lanes x 16 bytes) fills chunks 64g .. 64g+63, so each
// instruction reads one source tensor only; wave w issues g = 4u + w for
// u = 0 .. 9, so the tensor of copy u is the same for every wave (u < 4:
// K_nope, u < 6: rope, else V^T).
constexpr int N_SLOTS = KT * (DN / 8);    // 1024
constexpr int R_SLOTS = KT * (DR / 8);    // 512
constexpr int V_SLOTS = DV * (KT / 8);    // 1024
constexpr int R0 = N_SLOTS * 8, V0 = (N_SLOTS + R_SLOTS) * 8;    // fp16 offsets of the parts
constexpr int LPW = (N_SLOTS + R_SLOTS + V_SLOTS) / (64 * NW);  // copies per lane per tile (10)
constexpr int STAGE = (N_SLOTS + R_SLOTS + V_SLOTS) * 8;        // fp16 elements per ring stage
constexpr int NSTAGE = 4;
constexpr float TAU = 12.f;       // log2 units: P < 2^12 in fp16
constexpr int MPF = 4;            // operand fragments read ahead (each feeds two MFMAs)
constexpr int N_S_OPS = KS * 2 * 2;                   // S MFMAs of a tile (k-step x key block x query block)
constexpr int N_PV_OPS = (KT / 16) * (DV / 32) * 2;   // PV MFMAs of a tile (key step x d block x query block)
static_assert(LPW * 64 * NW == N_SLOTS + R_SLOTS + V_SLOTS, "tile chunks must split evenly over the waves");
static_assert(N_SLOTS % (64 * NW) == 0 && R_SLOTS % (64 * NW) == 0, "a copy round must not straddle two parts");
static_assert(LPW * 2 < 64, "vmcnt range");

// MFMAs with the register files pinned: S^T = K Q^T with Q^T in AGPRs and the
// result in VGPRs; O^T += V^T P^T with O^T in AGPRs.  Inline assembly keeps the
// compiler from moving these accumulators between the two files.  VGPR
// operands written by VALU instructions reach these MFMAs only after an
// s_nop or many instructions, and their results are read after mfma_drain().
__device__ __forceinline__ void mfma_s_first(f32x16_t& d, f16x8_t k, const f16x8_t& q) {
  // early clobber: the result must not take the registers of the K operand
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(k), "a"(q));
}
__device__ __forceinline__ void mfma_s(f32x16_t& d, f16x8_t k, const f16x8_t& q) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(k), "a"(q));
}
__device__ __forceinline__ void mfma_pv(f32x16_t& o, f16x8_t v, f16x8_t p) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
}
__device__ __forceinline__ void mfma_pv_nop(f32x16_t& o, f16x8_t v, f16x8_t p) {   // after fresh P
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
}
// zeroes o in place (the registers it already holds); the result is final
// when the statement ends, since the compiler may copy it right after
__device__ __forceinline__ void mfma_zero(f32x16_t& o) {
  const f16x8_t z = {};
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_f16 %0, %1, %1, 0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o) : "v"(z));
}
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::); }
// compiler-generated reads of acc cannot move above this point
__device__ __forceinline__ void agpr_fence(f32x16_t& acc) { asm volatile("" : "+a"(acc)); }
// v is held in AGPRs from here on (Q^T operand)
__device__ __forceinline__ void agpr_fence(f16x8_t& v) { asm volatile("s_nop 4" : "+a"(v)); }

// Chunk swizzle (stored chunk = logical chunk ^ swizzle(row)), measured free of
// LDS bank conflicts for the 16-byte reads below, where 16 consecutive lanes
// read 16 consecutive 128-byte rows (two rows per bank sweep, so 8 distinct
// chunks per row parity).
__device__ __forceinline__ int sw_8(int row) { return (row >> 1) & 7; }

// key offset (inside its 32-key block) carried by LDS row rho of that block
__device__ __forceinline__ int key_of_row(int rho) {
  const int g = rho >> 3, x = (rho >> 2) & 1, r = rho & 3;
  return 16 * (g >> 1) + 8 * x + 4 * (g & 1) + r;
}

template <mla_dtype OT>
__global__ void __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_attention_kernel(ExplicitArgs a, const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vt,
                      const uint16_t* __restrict__ krot, const float2* __restrict__ qtab, int nqt) {
  __shared__ __attribute__((aligned(16))) uint16_t Ls[NSTAGE * STAGE];

  const int P = a.B * a.H;
  const int n = blockIdx.x;
  const int xcd = n & 7, slot = n >> 3;
  const int p = xcd + 8 * (slot / nqt);
  const int qt = nqt - 1 - (slot % nqt);
  if (p >= P) return;
  const int b = p / a.H, h = p % a.H;
  const int64_t bh = (int64_t)b * a.H + h;
  const int i0 = qt * QT;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hb = lane >> 5;
  const int iw0 = i0 + wave * QW;
  const float c_log2 = a.scale * MLA_LOG2E;

  // ---- key ranges ------------------------------------------------------------
  auto limit = [&](int qi) __attribute__((always_inline)) -> int {   // keys [0, limit) visible to query qi
    if (!a.causal) return a.s_vis;
    int64_t lim = a.q_pos0 + qi - a.kv_pos0 + 1;
    return (int)max((int64_t)0, min(lim, (int64_t)a.s_vis));
  };
  const int i_last_wg = min(i0 + QT, a.Sq) - 1;
  const int kend_wg = limit(i_last_wg);
  int ntile = (kend_wg + KT - 1) / KT;              // tiles end at or before s_pad
  const bool wave_has_rows = iw0 < a.Sq;
  const int kend_w = wave_has_rows ? limit(min(iw0 + QW, a.Sq) - 1) : 0;
  const int kfull_w = wave_has_rows ? limit(iw0) : 0;
  int lim_i[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int i = iw0 + 32 * qb + l32;
    lim_i[qb] = (i < a.Sq) ? limit(i) : 0;
  }
  int t_full = min(kfull_w / KT, ntile);                 // tiles with every key visible
  int t_end = min((kend_w + KT - 1) / KT, ntile);        // tiles with any key visible

  // ---- tile copies: copy u of this wave is instruction g = NW*u + wave ---------
  // Byte offsets of tile 0; tile t adds t * (bytes per tile of that tensor).
  const i32x4_t rs_n = make_rsrc(kn + bh * a.s_pad * DN, (uint32_t)a.s_pad * DN * 2);
  const i32x4_t rs_r = make_rsrc(krot + (int64_t)b * a.s_pad * DR, (uint32_t)a.s_pad * DR * 2);
  const i32x4_t rs_v = make_rsrc(vt + bh * DV * a.s_pad, (uint32_t)a.s_pad * DV * 2);
  // Every copy of one part is the part's first copy moved by a constant
  // (worked out from the slot maps below), so a lane keeps one global offset
  // per part and the rest goes into the uniform offset:
  //   K_nope copy u (0..3):  slot s = 64(4u+w) + lane, half s/512, row (s%512)/8
  //   rope copy u (4, 5):    slot s - 1024, row (s-1024)/8
  //   V^T copy u (6..9):     slot s - 1536, row d = (s-1536)/8
  // Rows of the K parts carry keys in the permuted order of key_of_row.
  int goff_n, goff_r, goff_v;
  {
    const int rho = 8 * wave + (lane >> 3);          // row within the first 32 of a part
    const int c = (lane & 7) ^ sw_8(rho);
    goff_n = key_of_row(rho) * (DN * 2) + 16 * c;    // half 0, rows 0..31
    goff_r = key_of_row(rho) * (DR * 2) + 16 * c;
    goff_v = rho * (a.s_pad * 2) + 16 * c;
  }
  const uint32_t ls_lds = (uint32_t)(uintptr_t)(LDS_AS void*)&Ls[0];
  int vrow32 = 32 * a.s_pad * 2;                   // bytes of 32 V^T rows
  // Copy u of tile t into its ring stage.
  auto issue_copy = [&](auto uc, int t) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
    constexpr int part = (NW * u < N_SLOTS / 64) ? 0 : (NW * u < (N_SLOTS + R_SLOTS) / 64) ? 1 : 2;
    constexpr int st = part == 0 ? KT * DN * 2 : part == 1 ? KT * DR * 2 : KT * 2;
    // K_nope: copy u has rows 32(u%2) .. of half u/2; rope: rows 32(u-4) ..; V^T: d rows 32(u-6) ..
    constexpr int cu = part == 0 ? (u & 1) * 32 * (DN * 2) + (u >> 1) * (DN / 2 * 2)
                     : part == 1 ? (u - 4) * 32 * (DR * 2) : 0;
    const i32x4_t& rs = part == 0 ? rs_n : part == 1 ? rs_r : rs_v;
    const int voff = part == 0 ? goff_n : part == 1 ? goff_r : goff_v;
    int so = t * st + cu;
    if constexpr (part == 2) so += (u - 6) * vrow32;
    // the stage base is opaque to the optimizer, which would otherwise keep
    // one precomputed address per copy in scalar registers
    uint32_t base = __builtin_amdgcn_readfirstlane(ls_lds + (uint32_t)((t % NSTAGE) * STAGE * 2 + wave * 1024));
    asm volatile("" : "+s"(base));
    lds_dma_b128(rs, base + u * NW * 1024, voff, __builtin_amdgcn_readfirstlane(so));
  };
  auto issue_all = [&](int t) __attribute__((always_inline)) {
    if (t < ntile) static_for<LPW>([&](auto uc) __attribute__((always_inline)) { issue_copy(uc, t); });
  };

  // the first tiles of the first pass are on their way while Q is loaded
  for (int t = 0; t < NSTAGE - 1; ++t) issue_all(t);

  // ---- Q^T operand (fp16), query block qb ------------------------------------
  // Lane (l32, hb) supplies query row l32 of the block, k-slots 8hb .. 8hb+7 of
  // every k-step: elements 16ks + 8hb .. +7 of q_nope (ks < 8) and elements
  // m0 .. m0+7, m0 = 16(ks-8) + 8hb, of R(q_pe) (ks >= 8).  Rows past the end
  // load a valid row (their results are never stored).  The loads of both blocks are issued
  // before any arithmetic (and after the first tile copies, which they
  // overlap).
  u32x4_t rn[2][DN / 16], rp[2][4];
  f32x4_t ct[2][8];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int i = iw0 + 32 * qb + l32;
    const int ic = i < a.Sq ? i : a.Sq - 1;
    const int64_t qrow = ((int64_t)b * a.Sq + ic) * a.H + h;
    const u32x4_t* qn = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.q_nope) + qrow * DN);
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.q_pe) + qrow * DR);
    const f32x4_t* qt4 = reinterpret_cast<const f32x4_t*>(qtab + (int64_t)ic * (DR / 2));
#pragma unroll
    for (int ks = 0; ks < DN / 16; ++ks) rn[qb][ks] = qn[2 * ks + hb];
    // the rope run starts at pair mlo = 16r + 8hb (k-steps 8 + r and 10 + r)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int mlo = 16 * r + 8 * hb;
      rp[qb][2 * r] = qp[mlo / 8];             // elements mlo .. mlo+7
      rp[qb][2 * r + 1] = qp[mlo / 8 + 4];     // elements mlo+32 .. mlo+39
#pragma unroll
      for (int c = 0; c < 4; ++c) ct[qb][4 * r + c] = qt4[mlo / 2 + c];   // (cos, sin) of pairs mlo+2c, mlo+2c+1
    }
  }
  f16x8_t qf[2][KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int ks = 0; ks < DN / 16; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[qb][ks][2 * e] = (_Float16)bf16_bits_to_float((uint16_t)(rn[qb][ks][e] & 0xffff));
        qf[qb][ks][2 * e + 1] = (_Float16)bf16_bits_to_float((uint16_t)(rn[qb][ks][e] >> 16));
      }
#pragma unroll
    for (int ks = DN / 16; ks < KS; ++ks) {
      const int r = (ks - DN / 16) & 1;
      const bool second_half = ks - DN / 16 >= 2;     // output elements 32 .. 63
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wl = rp[qb][2 * r][e >> 1], wh = rp[qb][2 * r + 1][e >> 1];
        const float lo = bf16_bits_to_float((uint16_t)((e & 1) ? (wl >> 16) : (wl & 0xffff)));
        const float hi = bf16_bits_to_float((uint16_t)((e & 1) ? (wh >> 16) : (wh & 0xffff)));
        const float cs = ct[qb][4 * r + (e >> 1)][2 * (e & 1)], sn = ct[qb][4 * r + (e >> 1)][2 * (e & 1) + 1];
        const float v = second_half ? (hi * cs + lo * sn) : (lo * cs - hi * sn);
        qf[qb][ks][e] = (_Float16)v;
      }
    }
  }
  // Q^T lives in AGPRs from here on
  static_for<2>([&](auto qbc) __attribute__((always_inline)) {
    static_for<KS>([&](auto ksc) __attribute__((always_inline)) {
      agpr_fence(qf[decltype(qbc)::value][decltype(ksc)::value]);
    });
  });

  // ---- per-lane LDS read offsets (fp16 elements within a stage) -----------------
  // A lane reads row l32 of a 32-row block at logical chunk 2q + hb, q = 0..3:
  //   K_nope, k-step ks < 8:  half ks/4, q = ks % 4
  //   rope,   k-step ks >= 8: q = ks - 8
  //   V^T,    key step ps:    q = ps
  // so one offset per q serves all three parts.
  int rofs[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) rofs[q] = l32 * 64 + 8 * ((2 * q + hb) ^ sw_8(l32));
  // S op k (0..47): k-step k/4, key block (k/2)%2, query block k%2
  auto kfrag = [&](const uint16_t* st, int k) __attribute__((always_inline)) -> f16x8_t {
    const int ks = k >> 2, kt = (k >> 1) & 1;
    const int off = (ks < DN / 16) ? rofs[ks & 3] + (ks >> 2) * (KT * 64) + kt * (32 * 64)
                                   : R0 + rofs[ks - DN / 16] + kt * (32 * 64);
    return *reinterpret_cast<const f16x8_t*>(st + off);
  };
  // PV op k (0..31): key step k/8, d block (k/2)%4, query block k%2
  auto vfrag = [&](const uint16_t* st, int k) __attribute__((always_inline)) -> f16x8_t {
    const int ps = k >> 3, db = (k >> 1) & 3;
    return *reinterpret_cast<const f16x8_t*>(st + V0 + rofs[ps] + db * (32 * 64));
  };

  f32x16_t oacc[DV / 32][2];               // O^T [d block][query block], AGPRs
  static_for<DV / 32>([&](auto dbc) __attribute__((always_inline)) {
    mfma_zero(oacc[decltype(dbc)::value][0]);
    mfma_zero(oacc[decltype(dbc)::value][1]);
  });
  // S^T of two tiles [key block][query block]: the one whose softmax runs and
  // the next one, whose MFMAs are issued meanwhile (they swap every iteration)
  f32x16_t sa[2][2], sb[2][2];
  f16x8_t pk[KT / 16][2];                  // P [key step][query block]
  float m_ref[2] = {-INFINITY, -INFINITY}, m_max[2] = {-INFINITY, -INFINITY};
  // m_ref and m_max are in score units; m_usec = m_ref * c_log2 (0 while a
  // row has no reference) is what p = exp2(s * c_log2 - m_usec) subtracts
  float l_run[2] = {0.f, 0.f}, m_usec[2] = {0.f, 0.f};

  // Before a tile's stream (uniform branches, rarely taken): the causal mask
  // on the wave's diagonal tiles, and the reference of rows whose first
  // visible key lies in this tile, which is their row max over the tile.
  auto prepare = [&](bool masked, f32x16_t (&sc)[2][2], int j0) __attribute__((always_inline)) {
    if (masked) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int g = e >> 2, r = e & 3;
            const int key = j0 + kt * 32 + 16 * (g >> 1) + 8 * hb + 4 * (g & 1) + r;
            if (key >= lim_i[qb]) sc[kt][qb][e] = -INFINITY;
          }
    }
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) need |= m_ref[qb] == -INFINITY && lim_i[qb] > j0;
    if (__ballot(need) != 0ull) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float m = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) m = fmaxf(m, sc[kt][qb][e]);
        m = half_pair_max(m);
        if (m_ref[qb] == -INFINITY) m_ref[qb] = m;
        // a row that has seen no visible key keeps the reference -inf and uses 0
        m_usec[qb] = (m_ref[qb] == -INFINITY) ? 0.f : m_ref[qb] * c_log2;
      }
    }
  };

  // Softmax unit u (0 .. 71) of a tile, issued right after MFMA u of the
  // stream.  Units 9c .. 9c+8 handle the 8 scores of combination c = 2 ps + qb
  // (key step ps, query block qb); unit 9c + j, j < 8, forms p_j =
  // exp2((s_j - ref) log2(e) scale), adds p_(j-1) to the row sum and, for even j, takes the running max
  // over s_j, s_(j+1); unit 9c + 8 adds p_7 and packs the 8 values to fp16 P.
  // Each unit is at most about one MFMA long.  The P of key step ps is
  // complete at unit 18 ps + 17, before its first PV MFMA (48 + 8 ps).
  auto unit = [&](auto u_c, f32x16_t (&sc)[2][2]) __attribute__((always_inline)) {
    constexpr int u = decltype(u_c)::value;
    if constexpr (u < 72) {
      constexpr int c = u / 9, j = u % 9, ps = c >> 1, qb = c & 1, kt = ps >> 1, e0 = 8 * (ps & 1);
      if constexpr (j < 8) {
        if constexpr (j % 2 == 0) m_max[qb] = max3(m_max[qb], sc[kt][qb][e0 + j], sc[kt][qb][e0 + j + 1]);
        if constexpr (j > 0) l_run[qb] += sc[kt][qb][e0 + j - 1];
        sc[kt][qb][e0 + j] = fast_exp2(fmaf(sc[kt][qb][e0 + j], c_log2, -m_usec[qb]));
      } else {
        // P elements 8u'..8u'+7 of block kt feed PV key step ps = 2kt + u'
        l_run[qb] += sc[kt][qb][e0 + 7];
#pragma unroll
        for (int x = 0; x < 8; ++x) pk[ps][qb][x] = (_Float16)sc[kt][qb][e0 + x];
      }
    }
  };

  // One iteration: the S MFMAs of the next tile (into sn) and the PV MFMAs
  // of the current tile, one softmax unit of the current tile (sc) after each
  // MFMA: an MFMA holds the wave's issue until the matrix unit takes it, so
  // the vector work goes between consecutive MFMAs to run beside them.  In
  // the wave's last iteration the S MFMAs read a stale stage and their result
  // is never used: one stream serves every iteration.
  auto iteration = [&](bool masked, int T, f32x16_t (&sc)[2][2], f32x16_t (&sn)[2][2])
                       __attribute__((always_inline)) {
    const uint16_t* stk = Ls + ((T + 1) % NSTAGE) * STAGE;   // stage of tile T+1 (its K)
    const uint16_t* stv = Ls + (T % NSTAGE) * STAGE;         // stage of tile T (its V^T)
    constexpr int NOPS = N_S_OPS + N_PV_OPS;
    // op pair (2i, 2i+1) (query blocks 0, 1) shares one fragment: K fragment i
    // for 2i < 48, V^T fragment i - 24 after; fragments are read MPF pairs ahead
    auto frag = [&](int k) __attribute__((always_inline)) -> f16x8_t {
      return (k < N_S_OPS) ? kfrag(stk, k) : vfrag(stv, k - N_S_OPS);
    };
    f16x8_t fr[MPF + 1];
    static_for<MPF>([&](auto c) __attribute__((always_inline)) {
      fr[decltype(c)::value] = frag(2 * decltype(c)::value);
    });
    // the copies of tile T+3 (each holds the wave's issue for tens of cycles:
    // the first operand reads land meanwhile)
    issue_all(T + 3);
    mfma_drain();                                  // sc was produced by MFMAs
    prepare(masked, sc, T * KT);
    static_for<NOPS>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value, i = k >> 1, qb = k & 1;
      if constexpr (qb == 0 && 2 * (i + MPF) < NOPS) fr[(i + MPF) % (MPF + 1)] = frag(2 * (i + MPF));
      const f16x8_t f = fr[i % (MPF + 1)];
      if constexpr (k < N_S_OPS) {
        constexpr int ks = k >> 2, kt = (k >> 1) & 1;
        if constexpr (ks == 0) mfma_s_first(sn[kt][qb], f, qf[qb][ks]);
        else mfma_s(sn[kt][qb], f, qf[qb][ks]);
      } else {
        constexpr int kk = k - N_S_OPS, ps = kk >> 3, db = (kk >> 1) & 3;
        if constexpr ((kk & 7) == 0) mfma_pv_nop(oacc[db][qb], f, pk[ps][qb]);
        else mfma_pv(oacc[db][qb], f, pk[ps][qb]);
      }
      unit(kc, sc);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---- main loop -------------------------------------------------------------------
  // Ring of 4 stages: at the top of iteration T the copies of tile T+1 have
  // landed for every wave (its S is computed now), tile T is resident (its PV
  // is computed now), and tile T-1 was read for the last time in iteration
  // T-1, so the copy of tile T+3 takes its stage.  Every wave passes the same
  // barriers.
  auto step = [&](int T, f32x16_t (&sc)[2][2], f32x16_t (&sn)[2][2]) __attribute__((always_inline)) {
    // tile T+1 has landed once at most the copies of tile T+2 are in flight
    if (T + 2 < ntile) wait_vmcnt<LPW>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (T < t_end) iteration(T >= t_full, T, sc, sn);
    else issue_all(T + 3);
  };

  for (int pass = 0; pass < 2; ++pass) {
    // Values that stay the same over the whole pass are made opaque here:
    // otherwise the optimizer derives many constants from them before the
    // pass loop and keeps them all in scalar registers through the main loop.
    asm volatile("" : "+s"(ntile), "+s"(t_end), "+s"(t_full), "+s"(vrow32));
    if (pass > 0)
      for (int t = 0; t < NSTAGE - 1; ++t) issue_all(t);
    // prologue: S of tile 0
    if (ntile > 0) {
      if (ntile > 2) wait_vmcnt<2 * LPW>();
      else if (ntile > 1) wait_vmcnt<LPW>();
      else wait_vmcnt<0>();
      __syncthreads();
      if (t_end > 0) {
        const uint16_t* stk = Ls;
        f16x8_t fr[MPF + 1];
        static_for<MPF>([&](auto c) __attribute__((always_inline)) {
          fr[decltype(c)::value] = kfrag(stk, 2 * decltype(c)::value);
        });
        static_for<N_S_OPS / 2>([&](auto ic) __attribute__((always_inline)) {
          constexpr int i = decltype(ic)::value, k = 2 * i;
          if constexpr (k + 2 * MPF < N_S_OPS) fr[(i + MPF) % (MPF + 1)] = kfrag(stk, k + 2 * MPF);
          const f16x8_t f = fr[i % (MPF + 1)];
          constexpr int ks = k >> 2, kt = (k >> 1) & 1;
          if constexpr (ks == 0) {
            mfma_s_first(sa[kt][0], f, qf[0][ks]);
            mfma_s_first(sa[kt][1], f, qf[1][ks]);
          } else {
            mfma_s(sa[kt][0], f, qf[0][ks]);
            mfma_s(sa[kt][1], f, qf[1][ks]);
          }
          __builtin_amdgcn_sched_barrier(0);
        });
      }
    }
    // two iterations per trip so that the two S^T sets keep fixed registers
    for (int T = 0; T < ntile; T += 2) {
      step(T, sa, sb);
      if (T + 1 < ntile) step(T + 1, sb, sa);
    }
    // a second pass (rare): every wave learns whether any row of the
    // workgroup saw a tile exceed its reference by more than tau
    __syncthreads();                               // the ring is free again
    int* flags = reinterpret_cast<int*>(Ls);
    bool exceeded = false;
    // the reference is fixed after a row's first visible tile, so the running
    // max tells whether any tile went past it by more than tau
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
      exceeded |= m_ref[qb] != -INFINITY && (m_max[qb] - m_ref[qb]) * c_log2 > TAU;
    const bool wave_exceeded = __ballot(exceeded) != 0ull;
    flags[wave] = wave_exceeded ? 1 : 0;           // every lane stores the same value
    __syncthreads();
    const int redo = flags[0] | flags[1] | flags[2] | flags[3];
    __syncthreads();                               // flags read before the ring is refilled
    if (pass == 1 || !__builtin_amdgcn_readfirstlane(redo)) break;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      m_ref[qb] = half_pair_max(m_max[qb]);       // the exact row max
      m_usec[qb] = (m_ref[qb] == -INFINITY) ? 0.f : m_ref[qb] * c_log2;
      l_run[qb] = 0.f;
    }
    mfma_drain();
    static_for<DV / 32>([&](auto dbc) __attribute__((always_inline)) {
      mfma_zero(oacc[decltype(dbc)::value][0]);
      mfma_zero(oacc[decltype(dbc)::value][1]);
    });
  }

  // ---- epilogue ---------------------------------------------------------------
  // O = O^T / l goes row-major through this wave's part of the idle ring (rows
  // padded by 16 bytes against bank conflicts), so that every store to global
  // memory covers whole output rows.
  constexpr int OB = (OT == MLA_FP32) ? 4 : 2;                 // bytes per output element
  constexpr int OROW = DV * OB, OSTR = OROW + 16;              // row bytes, LDS row stride
  static_assert(NW * QW * OSTR <= NSTAGE * STAGE * 2, "output staging must fit in the ring");
  // The lane index is formed afresh: a value kept from the start would live
  // through the main loop, where registers are scarce.
  int lane_e;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
  const int l32e = lane_e & 31, hbe = lane_e >> 5;
  uint8_t* ob = reinterpret_cast<uint8_t*>(Ls) + wave * QW * OSTR;
  mfma_drain();
  float lsum[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = half_pair_sum(l_run[qb]);
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    lsum[qb] = l;
    uint8_t* orow = ob + (32 * qb + l32e) * OSTR;
#pragma unroll
    for (int v = 0; v < DV / 32; ++v) {
      agpr_fence(oacc[v][qb]);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = v * 32 + 8 * g + 4 * hbe;
        const float o0 = oacc[v][qb][4 * g] * inv, o1 = oacc[v][qb][4 * g + 1] * inv;
        const float o2 = oacc[v][qb][4 * g + 2] * inv, o3 = oacc[v][qb][4 * g + 3] * inv;
        if constexpr (OT == MLA_FP32) {
          *reinterpret_cast<f32x4_t*>(orow + d * 4) = f32x4_t{o0, o1, o2, o3};
        } else {
          u32x2_t v2;
          v2[0] = pack_bf16x2(o0, o1);
          v2[1] = pack_bf16x2(o2, o3);
          *reinterpret_cast<u32x2_t*>(orow + d * 2) = v2;
        }
      }
    }
  }
  // a wave reads back only what it wrote itself
  constexpr int CPR = OROW / 16;                               // 16-byte chunks per row
#pragma unroll
  for (int it = 0; it < QW * CPR / 64; ++it) {
    const int cidx = it * 64 + lane_e, row = cidx / CPR, c = cidx % CPR;
    const int i = iw0 + row;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ob + row * OSTR + 16 * c);
    if (i < a.Sq)
      *reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(a.out) +
                                  (((int64_t)b * a.Sq + i) * a.H + h) * OROW + 16 * c) = v;
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int i = iw0 + 32 * qb + l32e;
    const float l = lsum[qb];
    if (a.lse != nullptr && hbe == 0 && i < a.Sq)
      a.lse[bh * a.Sq + i] = (l > 0.f) ? (m_ref[qb] * c_log2 + __log2f(l)) * MLA_LN2 : -INFINITY;
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
