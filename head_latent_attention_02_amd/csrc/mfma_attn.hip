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
// runs 8 waves of 32 rows each, two waves per SIMD.  A wave computes
// S^T = K Q^T and O^T += V^T P^T on 32x32x16 MFMAs with Q^T (192 x 32, fp16)
// and O^T (128 x 32, fp32) held in AGPRs and K / V^T fragments read from LDS.
//
// Ping-pong.  The waves form two groups (waves 0-3 and 4-7; each SIMD holds
// one wave of each).  A wave alternates two phases separated by workgroup
// barriers:
//   M(t): the MFMA stream of S(t+1) = K(t+1) Q^T (24 MFMAs) and of
//         O^T += V^T(t) P^T(t) (16 MFMAs);
//   V(t): the softmax of S(t) into P(t) (exponentials, row sums, running
//         maxima, fp16 packing) and half of a tile's copies.
// Group 1 starts one barrier late, so while one wave of a SIMD issues MFMAs
// the other does its vector work and memory instructions: the matrix unit is
// fed by one wave while the other's exponentials and copy issues (which hold
// their wave for tens of cycles each) run beside it.  The M phase raises its
// wave's issue priority.
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
// 16 bytes per lane) through a ring of 4 stages.  Each wave issues 5 of a
// tile's 40 copies in its V phase: group 0 two tiles ahead, group 1 (one
// phase behind) three, so both halves of a tile have two phases to land.
// Split this way, neither group's V phase outgrows the M phase it faces.
// In every tile row the 16-byte chunks are XOR-swizzled by row so that the
// 16-byte operand reads of 16 consecutive lanes fall in distinct banks.
//
// Softmax reference.  A row's reference max is the max of its first tile
// with a visible key; P = exp2(s - ref) stays below 2^tau in fp16.  A tile
// whose max exceeds the reference by more than tau flags the workgroup, which
// then recomputes all its rows from their exact maxima (seen by the first
// pass), so the accumulators are only ever touched by MFMAs.
//
// Workgroups are dealt so that all query tiles of one head run on the same
// XCD (its L2 holds that head's K/V), two heads at a time, longest first.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int QW = 32;            // query rows per wave
constexpr int NW = 8;             // waves per workgroup (two per SIMD)
constexpr int NWC = 4;            // waves per group
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
// instruction reads one source tensor only; copy u = 0 .. 9 of a tile is
// g = 4u + w for the wave w (0..3) of its group, so the tensor of copy u is the
// same for all four (u < 4: K_nope, u < 6: rope, else V^T).  Group 0 issues
// u = 0 .. 4, group 1 u = 5 .. 9.
constexpr int N_SLOTS = KT * (DN / 8);    // 1024
constexpr int R_SLOTS = KT * (DR / 8);    // 512
constexpr int V_SLOTS = DV * (KT / 8);    // 1024
constexpr int R0 = N_SLOTS * 8, V0 = (N_SLOTS + R_SLOTS) * 8;    // fp16 offsets of the parts
constexpr int LPW = (N_SLOTS + R_SLOTS + V_SLOTS) / (64 * NWC); // copies per wave index per tile (10)
constexpr int HPW = LPW / 2;      // copies per wave per tile (5), one half per group
constexpr int STAGE = (N_SLOTS + R_SLOTS + V_SLOTS) * 8;        // fp16 elements per ring stage
constexpr int NSTAGE = 4;
constexpr int LOOKAHEAD = 2;      // group 0's copies of tile t + 2 go out in V(t), group 1's of t + 3
constexpr float TAU = 12.f;       // log2 units: P < 2^12 in fp16
constexpr int MPF = 4;            // operand fragments read ahead in the M phase
constexpr int PRIO_M = 2;         // issue priority of a wave in its M phase
constexpr int N_S_OPS = KS * 2;                   // S MFMAs of a tile (k-step x key block)
constexpr int N_PV_OPS = (KT / 16) * (DV / 32);   // PV MFMAs of a tile (key step x d block)
static_assert(LPW * 64 * NWC == N_SLOTS + R_SLOTS + V_SLOTS, "tile chunks must split evenly over the copy waves");
static_assert(N_SLOTS % (64 * NWC) == 0 && R_SLOTS % (64 * NWC) == 0, "a copy round must not straddle two parts");
static_assert(LPW * 2 < 64, "vmcnt range");
// stage reuse: V(t) of group 0 writes the stage of tile t+2 = tile t-2, whose
// last reader (group 1's M(t-2)) ran two barriers earlier; V(t) of group 1
// writes that of tile t+3 = tile t-1, whose last reader (group 1's own
// M(t-1)) ran in the previous interval
static_assert(NSTAGE == LOOKAHEAD + 2, "ring length and copy lookahead go together");

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
__device__ __forceinline__ void barrier() { __builtin_amdgcn_s_barrier(); }

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
__global__ void __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
mfma_attention_kernel(ExplicitArgs a, const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vt,
                      const uint16_t* __restrict__ krot, const float2* __restrict__ qtab, int nqt) {
  __shared__ __attribute__((aligned(16))) uint16_t Ls[NSTAGE * STAGE];

  // XCD x (= blockIdx.x % 8, the order the dispatcher deals workgroups)
  // takes the (batch, head) pairs p = x, x + 8, ... two at a time; within a
  // pair the query tiles go longest first, alternating between the two
  // heads, so the long tiles of the last pair do not start last.
  const int P = a.B * a.H;
  const int n = blockIdx.x;
  const int xcd = n & 7, slot = n >> 3;
  const int grp = slot / (2 * nqt), r = slot % (2 * nqt);
  const int p = xcd + 8 * (2 * grp + (r & 1));
  const int qt = nqt - 1 - (r >> 1);
  if (p >= P) return;
  const int b = p / a.H, h = p % a.H;
  const int64_t bh = (int64_t)b * a.H + h;
  const int i0 = qt * QT;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool lead = wave < NWC;                    // group 0 (runs one phase ahead of group 1)
  const int cw = wave & (NWC - 1);                   // index within the group
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
  const int i_me = iw0 + l32;
  const int lim_me = (i_me < a.Sq) ? limit(i_me) : 0;
  int t_full = min(kfull_w / KT, ntile);                 // tiles with every key visible
  int t_end = min((kend_w + KT - 1) / KT, ntile);        // tiles with any key visible

  // ---- tile copies: copy u of copy wave cw is instruction g = NWC*u + cw ---------
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
    const int rho = 8 * cw + (lane >> 3);            // row within the first 32 of a part
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
    constexpr int part = (NWC * u < N_SLOTS / 64) ? 0 : (NWC * u < (N_SLOTS + R_SLOTS) / 64) ? 1 : 2;
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
    uint32_t base = __builtin_amdgcn_readfirstlane(ls_lds + (uint32_t)((t % NSTAGE) * STAGE * 2 + cw * 1024));
    asm volatile("" : "+s"(base));
    lds_dma_b128(rs, base + u * NWC * 1024, voff, __builtin_amdgcn_readfirstlane(so));
  };
  // group 0 issues copies 0 .. HPW-1 of a tile, group 1 copies HPW .. LPW-1
  auto issue_half = [&](int t) __attribute__((always_inline)) {
    if (t >= ntile) return;
    if (lead) static_for<HPW>([&](auto uc) __attribute__((always_inline)) { issue_copy(uc, t); });
    else static_for<HPW>([&](auto uc) __attribute__((always_inline)) {
      issue_copy(std::integral_constant<int, decltype(uc)::value + HPW>{}, t);
    });
  };
  // group 0 is LOOKAHEAD tiles ahead, group 1 one more
  auto issue_prologue = [&]() __attribute__((always_inline)) {
    for (int t = 0; t < LOOKAHEAD + (lead ? 0 : 1); ++t) issue_half(t);
  };

  // the first tiles of the first pass are on their way while Q is loaded
  issue_prologue();

  // ---- Q^T operand (fp16) ------------------------------------------------------
  // Lane (l32, hb) supplies query row l32 of the wave, k-slots 8hb .. 8hb+7 of
  // every k-step: elements 16ks + 8hb .. +7 of q_nope (ks < 8) and elements
  // m0 .. m0+7, m0 = 16(ks-8) + 8hb, of R(q_pe) (ks >= 8).  Rows past the end
  // load a valid row (their results are never stored).
  f16x8_t qf[KS];
  {
    u32x4_t rn[DN / 16], rp[4];
    f32x4_t ct[8];
    const int ic = i_me < a.Sq ? i_me : a.Sq - 1;
    const int64_t qrow = ((int64_t)b * a.Sq + ic) * a.H + h;
    const u32x4_t* qn = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.q_nope) + qrow * DN);
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.q_pe) + qrow * DR);
    const f32x4_t* qt4 = reinterpret_cast<const f32x4_t*>(qtab + (int64_t)ic * (DR / 2));
#pragma unroll
    for (int ks = 0; ks < DN / 16; ++ks) rn[ks] = qn[2 * ks + hb];
    // the rope run starts at pair mlo = 16r + 8hb (k-steps 8 + r and 10 + r)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int mlo = 16 * r + 8 * hb;
      rp[2 * r] = qp[mlo / 8];             // elements mlo .. mlo+7
      rp[2 * r + 1] = qp[mlo / 8 + 4];     // elements mlo+32 .. mlo+39
#pragma unroll
      for (int c = 0; c < 4; ++c) ct[4 * r + c] = qt4[mlo / 2 + c];   // (cos, sin) of pairs mlo+2c, mlo+2c+1
    }
#pragma unroll
    for (int ks = 0; ks < DN / 16; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[ks][2 * e] = (_Float16)bf16_bits_to_float((uint16_t)(rn[ks][e] & 0xffff));
        qf[ks][2 * e + 1] = (_Float16)bf16_bits_to_float((uint16_t)(rn[ks][e] >> 16));
      }
#pragma unroll
    for (int ks = DN / 16; ks < KS; ++ks) {
      const int r = (ks - DN / 16) & 1;
      const bool second_half = ks - DN / 16 >= 2;     // output elements 32 .. 63
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wl = rp[2 * r][e >> 1], wh = rp[2 * r + 1][e >> 1];
        const float lo = bf16_bits_to_float((uint16_t)((e & 1) ? (wl >> 16) : (wl & 0xffff)));
        const float hi = bf16_bits_to_float((uint16_t)((e & 1) ? (wh >> 16) : (wh & 0xffff)));
        const float cs = ct[4 * r + (e >> 1)][2 * (e & 1)], sn = ct[4 * r + (e >> 1)][2 * (e & 1) + 1];
        const float v = second_half ? (hi * cs + lo * sn) : (lo * cs - hi * sn);
        qf[ks][e] = (_Float16)v;
      }
    }
  }
  // Q^T lives in AGPRs from here on
  static_for<KS>([&](auto ksc) __attribute__((always_inline)) { agpr_fence(qf[decltype(ksc)::value]); });

  // ---- per-lane LDS read offsets (fp16 elements within a stage) -----------------
  // A lane reads row l32 of a 32-row block at logical chunk 2q + hb, q = 0..3:
  //   K_nope, k-step ks < 8:  half ks/4, q = ks % 4
  //   rope,   k-step ks >= 8: q = ks - 8
  //   V^T,    key step ps:    q = ps
  // so one offset per q serves all three parts.
  int rofs[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) rofs[q] = l32 * 64 + 8 * ((2 * q + hb) ^ sw_8(l32));
  // S op k (0..23): k-step k/2, key block k%2
  auto kfrag = [&](const uint16_t* st, int k) __attribute__((always_inline)) -> f16x8_t {
    const int ks = k >> 1, kt = k & 1;
    const int off = (ks < DN / 16) ? rofs[ks & 3] + (ks >> 2) * (KT * 64) + kt * (32 * 64)
                                   : R0 + rofs[ks - DN / 16] + kt * (32 * 64);
    return *reinterpret_cast<const f16x8_t*>(st + off);
  };
  // PV op k (0..15): key step k/4, d block k%4
  auto vfrag = [&](const uint16_t* st, int k) __attribute__((always_inline)) -> f16x8_t {
    const int ps = k >> 2, db = k & 3;
    return *reinterpret_cast<const f16x8_t*>(st + V0 + rofs[ps] + db * (32 * 64));
  };

  f32x16_t oacc[DV / 32];                  // O^T [d block], AGPRs
  static_for<DV / 32>([&](auto dbc) __attribute__((always_inline)) { mfma_zero(oacc[decltype(dbc)::value]); });
  float m_ref = -INFINITY, m_max = -INFINITY;
  // m_ref and m_max are in score units; m_usec = m_ref * c_log2 (0 while a
  // row has no reference) is what p = exp2(s * c_log2 - m_usec) subtracts
  float l_run = 0.f, m_usec = 0.f;

  // One pass over the tiles; a second one only when some row's logits went
  // past its reference by more than tau.  S^T and P are scoped to a pass so
  // that nothing but O^T, Q^T and the row statistics is live across the pass
  // boundary.
  for (int pass = 0; pass < 2; ++pass) {
    // Values that stay the same over the whole pass are made opaque here:
    // otherwise the optimizer derives many constants from them before the
    // pass loop and keeps them all in scalar registers through the main loop.
    asm volatile("" : "+s"(ntile), "+s"(t_end), "+s"(t_full), "+s"(vrow32));
    f32x16_t sacc[2];                      // S^T [key block]
    f16x8_t pk[KT / 16];                   // P [key step]

    // M(t): S of tile t+1 (if the wave sees it) and PV of tile t (if it sees it),
    // as one MFMA stream whose operand reads run MPF fragments ahead across
    // the switch from K to V^T fragments
    auto m_stream = [&](auto first_c, auto last_c, int T) __attribute__((always_inline)) {
      constexpr int F = decltype(first_c)::value, L = decltype(last_c)::value;   // ops [F, L)
      const uint16_t* stk = Ls + ((T + 1) % NSTAGE) * STAGE;        // stage of tile T+1 (its K)
      const uint16_t* stv = Ls + ((T + NSTAGE) % NSTAGE) * STAGE;   // stage of tile T (its V^T)
      auto frag = [&](int k) __attribute__((always_inline)) -> f16x8_t {
        return (k < N_S_OPS) ? kfrag(stk, k) : vfrag(stv, k - N_S_OPS);
      };
      f16x8_t fr[MPF + 1];
      static_for<MPF>([&](auto c) __attribute__((always_inline)) {
        constexpr int k = F + decltype(c)::value;
        if constexpr (k < L) fr[k % (MPF + 1)] = frag(k);
      });
      static_for<L - F>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = F + decltype(kc)::value;
        if constexpr (k + MPF < L) fr[(k + MPF) % (MPF + 1)] = frag(k + MPF);
        if constexpr (k < N_S_OPS) {
          constexpr int ks = k >> 1, kt = k & 1;
          if constexpr (ks == 0) mfma_s_first(sacc[kt], fr[k % (MPF + 1)], qf[ks]);
          else mfma_s(sacc[kt], fr[k % (MPF + 1)], qf[ks]);
        } else {
          constexpr int kk = k - N_S_OPS, ps = kk >> 2, db = kk & 3;
          if constexpr (kk == 0) asm volatile("s_nop 4" ::);   // P was written by vector instructions
          mfma_pv(oacc[db], fr[k % (MPF + 1)], pk[ps]);
        }
      });
    };
    using I0 = std::integral_constant<int, 0>;
    using IS = std::integral_constant<int, N_S_OPS>;
    using IE = std::integral_constant<int, N_S_OPS + N_PV_OPS>;
    // M(-1) is S of tile 0 alone.  In the wave's last tile the S MFMAs read a
    // stage that holds no tile of this wave and their result is never used:
    // one stream serves every other M phase.
    auto m_phase = [&](int T) __attribute__((always_inline)) {
      if (T >= t_end) return;
      __builtin_amdgcn_s_setprio(PRIO_M);
      if (T < 0) m_stream(I0{}, IS{}, T);
      else m_stream(I0{}, IE{}, T);
      __builtin_amdgcn_s_setprio(0);
    };

    // V(t): causal mask and reference (diagonal / first tiles only), then the
    // exponentials, row sums, running maximum and fp16 packing of S(t)
    auto v_phase = [&](int T) __attribute__((always_inline)) {
      if (T >= t_end) return;
      mfma_drain();                        // S(T) was produced by MFMAs
      const int j0 = T * KT;
      if (T >= t_full) {
        // Each compare goes through VCC right before its select: written as
        // plain selects, the compiler would form all the masks first and hold
        // them in scalar registers.
        const float ninf = -INFINITY;
        const int rel = lim_me - j0 - 8 * hb;         // masked iff key offset >= rel
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int g = e >> 2, r = e & 3;
            const int off = kt * 32 + 16 * (g >> 1) + 4 * (g & 1) + r;
            asm volatile("v_cmp_le_i32 vcc, %1, %2\n\tv_cndmask_b32 %0, %0, %3, vcc"
                         : "+v"(sacc[kt][e])
                         : "v"(rel), "n"(off), "v"(ninf)
                         : "vcc");
          }
      }
      // the reference of rows whose first visible key lies in this tile
      const bool need = m_ref == -INFINITY && lim_me > j0;
      if (__ballot(need) != 0ull) {
        float m = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) m = max2(m, sacc[kt][e]);
        m = half_pair_max(m);
        if (m_ref == -INFINITY) m_ref = m;
        // a row that has seen no visible key keeps the reference -inf and uses 0
        m_usec = (m_ref == -INFINITY) ? 0.f : m_ref * c_log2;
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; e += 2) m_max = max3(m_max, sacc[kt][e], sacc[kt][e + 1]);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          sacc[kt][e] = fast_exp2(fmaf(sacc[kt][e], c_log2, -m_usec));
          l_run += sacc[kt][e];
        }
      // P elements 8u..8u+7 of block kt feed PV key step ps = 2kt + u
#pragma unroll
      for (int ps = 0; ps < KT / 16; ++ps)
#pragma unroll
        for (int x = 0; x < 8; ++x) pk[ps][x] = (_Float16)sacc[ps >> 1][8 * (ps & 1) + x];
    };

    // ---- phases ---------------------------------------------------------------
    // Interval k (between two consecutive barriers) runs phase k of group 0 and
    // phase k-1 of group 1.  Phase 0 is M(-1) (S of tile 0), then V(t), M(t)
    // for t = 0 .. ntile-1.  Tile t is first read by group 0's M(t-1), in
    // interval 2t.  Group 0's half goes out in its V(t-2) (interval 2t-3) and
    // is waited for at the end of its V(t-1); group 1's half goes out in its
    // V(t-3) (interval 2t-4) and is waited for at the end of its M(t-2)
    // (interval 2t-1).  The first tiles go out before the pass.
    if (pass > 0) issue_prologue();
    // tile 0 has landed: at most the wave's copies of tiles 1 .. are in flight
    if (lead) {
      if (ntile > 1) wait_vmcnt<HPW>();
      else wait_vmcnt<0>();
    } else {
      if (ntile > 2) wait_vmcnt<2 * HPW>();
      else if (ntile > 1) wait_vmcnt<HPW>();
      else wait_vmcnt<0>();
    }
    __syncthreads();                       // tile 0 has landed; the ring's old contents are dead
    if (!lead) barrier();                // group 1 runs one phase behind
    m_phase(-1);
    // group 1: its half of tile 1 (read by group 0's M(0), in the next interval)
    if (!lead) {
      if (ntile > 2) wait_vmcnt<HPW>();
      else wait_vmcnt<0>();
    }
    for (int T = 0; T < ntile; ++T) {
      barrier();
      issue_half(T + LOOKAHEAD + (lead ? 0 : 1));
      v_phase(T);
      // group 0: its half of tile T+1 has landed once at most its copies of
      // tile T+2 are in flight
      if (lead) {
        if (T + LOOKAHEAD < ntile) wait_vmcnt<HPW>();
        else wait_vmcnt<0>();
      }
      barrier();
      m_phase(T);
      // group 1: its half of tile T+2 (first read by group 0's M(T+1), in the
      // next interval) has landed once at most its copies of tile T+3 are in flight
      if (!lead) {
        if (T + LOOKAHEAD + 1 < ntile) wait_vmcnt<HPW>();
        else wait_vmcnt<0>();
      }
    }
    if (lead) barrier();                 // group 0 catches up
    // a second pass (rare): every wave learns whether any row of the
    // workgroup saw a tile exceed its reference by more than tau
    __syncthreads();                       // every wave is done with the ring
    int* flags = reinterpret_cast<int*>(Ls);
    // the reference is fixed after a row's first visible tile, so the running
    // max tells whether any tile went past it by more than tau
    const bool exceeded = m_ref != -INFINITY && (m_max - m_ref) * c_log2 > TAU;
    const bool wave_exceeded = __ballot(exceeded) != 0ull;
    flags[wave] = wave_exceeded ? 1 : 0;   // every lane stores the same value
    __syncthreads();
    int redo = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) redo |= flags[w];
    __syncthreads();                       // flags read before the ring is refilled
    if (pass == 1 || !__builtin_amdgcn_readfirstlane(redo)) break;
    m_ref = half_pair_max(m_max);          // the exact row max
    m_usec = (m_ref == -INFINITY) ? 0.f : m_ref * c_log2;
    l_run = 0.f;
    mfma_drain();
    static_for<DV / 32>([&](auto dbc) __attribute__((always_inline)) { mfma_zero(oacc[decltype(dbc)::value]); });
  }

  // ---- epilogue ---------------------------------------------------------------
  // O = O^T / l goes row-major through this wave's part of the idle ring (rows
  // padded by 16 bytes against bank conflicts), so that every store to global
  // memory covers whole output rows.  The stores are non-temporal: the output
  // is not read again here, and the K/V tiles the XCD's other query tiles
  // still read keep their place in its L2.
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
  const float lsum = half_pair_sum(l_run);
  {
    const float inv = (lsum > 0.f) ? 1.f / lsum : 0.f;
    uint8_t* orow = ob + l32e * OSTR;
#pragma unroll
    for (int v = 0; v < DV / 32; ++v) {
      agpr_fence(oacc[v]);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = v * 32 + 8 * g + 4 * hbe;
        const float o0 = oacc[v][4 * g] * inv, o1 = oacc[v][4 * g + 1] * inv;
        const float o2 = oacc[v][4 * g + 2] * inv, o3 = oacc[v][4 * g + 3] * inv;
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
  // a wave reads back only what its own lanes wrote
  lds_wave_fence();
  constexpr int CPR = OROW / 16;                               // 16-byte chunks per row
#pragma unroll
  for (int it = 0; it < QW * CPR / 64; ++it) {
    const int cidx = it * 64 + lane_e, row = cidx / CPR, c = cidx % CPR;
    const int i = iw0 + row;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ob + row * OSTR + 16 * c);
    if (i < a.Sq)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(a.out) +
                                                                (((int64_t)b * a.Sq + i) * a.H + h) * OROW + 16 * c));
  }
  {
    const int i = iw0 + l32e;
    if (a.lse != nullptr && hbe == 0 && i < a.Sq)
      a.lse[bh * a.Sq + i] = (lsum > 0.f) ? (m_ref * c_log2 + __log2f(lsum)) * MLA_LN2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_mfma_attention(const ExplicitArgs& a, const uint16_t* kn, const uint16_t* vt,
                                 const uint16_t* krot, const float2* qtab, hipStream_t stream) {
  if (a.Sq == 0) return hipSuccess;
  const int P = a.B * a.H;
  const int nqt = (a.Sq + QT - 1) / QT;
  const int P16 = (P + 15) & ~15;                    // whole pairs of heads on every XCD
  dim3 grid((unsigned)(P16 * nqt));
  if (a.out_dt == MLA_BF16)
    hipLaunchKernelGGL(mfma_attention_kernel<MLA_BF16>, grid, dim3(NTHREADS), 0, stream, a, kn, vt, krot,
                       qtab, nqt);
  else
    hipLaunchKernelGGL(mfma_attention_kernel<MLA_FP32>, grid, dim3(NTHREADS), 0, stream, a, kn, vt, krot,
                       qtab, nqt);
  return hipGetLastError();
}
