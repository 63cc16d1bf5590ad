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
// 8 waves of 32 rows each (2 waves per SIMD).  Each wave keeps its Q^T block
// (192 x 32, fp16, pre-multiplied by softmax_scale * log2(e)) in registers as
// the B operand and computes S^T = K Q^T on 32x32x16 MFMAs, so every lane holds
// one query's scores: the row max needs one swap with the partner lane and the
// rescale of the O^T accumulator (128 x 32) is a per-lane multiply.
//
// Key order.  Inside each 32-key block the K rows sit in LDS in a permuted
// order: LDS row 8g + 4x + r (the accumulator row that lane half x holds in
// element 4g + r) carries key 16(g/2) + 8x + 4(g%2) + r.  The 8 scores a lane
// holds in elements 8u .. 8u+7 are then the keys 16u + 8x .. 16u + 8x + 7,
// contiguous, which is exactly the k-slot run the lane supplies to the
// O^T += V^T P^T MFMA.  P therefore goes from the S accumulator to the B
// operand of the next product inside the lane, and the matching V^T operand is
// one aligned 16-byte read.
//
// Tiles.  K (64 x 192, as a K_nope part and a rope part) and V^T (128 x 64)
// tiles are copied from global memory straight into LDS (buffer loads to LDS,
// 16 bytes per lane, 5 per wave per tile) through a ring of 4 stages, two
// tiles ahead of the one whose S is computed.  In every tile row the 16-byte
// chunks are XOR-swizzled by row so that the 16-byte operand reads of 16
// consecutive lanes fall in distinct banks.
//
// Schedule.  The waves form two groups with one wave of each on every SIMD;
// the groups run half an iteration apart, so that on each SIMD one wave issues
// MFMAs (the PV of the previous tile and the S of the current one) while the
// other computes a softmax on the vector ALU.
//
// Only the diagonal tiles are masked; tiles past a wave's last visible key are
// skipped.  The reference max of a row only
// moves when a tile exceeds it by more than 8 (log2 units), which skips the
// O^T rescale on almost every tile (P stays below 2^8, inside fp16's range).
// The row sum is taken on the fp16 P the MFMA consumes (v_dot2 with ones).
// Workgroups are dealt so that all query tiles of one head run on the same XCD
// (its L2 holds that head's K/V), longest first.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int QW = 32;            // query rows per wave
constexpr int NW = 8;             // waves per workgroup
constexpr int QT = QW * NW;       // query rows per workgroup
constexpr int KT = 64;            // keys per tile
constexpr int DN = 128, DR = 64, DQK = 192, DV = 128;
constexpr int NTHREADS = NW * 64;
// Ring stage layout (16-byte chunks; every row's chunks XOR-swizzled by row & 7):
//   K_nope part  [64 rows][16 chunks]   chunks    0 .. 1023
//   rope part    [64 rows][ 8 chunks]   chunks 1024 .. 1535
//   V^T          [128 rows][8 chunks]   chunks 1536 .. 2559
// Copy instruction g (64 lanes x 16 bytes) fills chunks 64g .. 64g+63, so each
// instruction reads one source tensor only.
constexpr int N_SLOTS = KT * (DN / 8);    // 1024
constexpr int R_SLOTS = KT * (DR / 8);    // 512
constexpr int V_SLOTS = DV * (KT / 8);    // 1024
constexpr int R0 = N_SLOTS * 8, V0 = (N_SLOTS + R_SLOTS) * 8;    // fp16 offsets of the parts
constexpr int LPW = (N_SLOTS + R_SLOTS + V_SLOTS) / (64 * NW);  // copies per wave per tile (5)
constexpr int STAGE = (N_SLOTS + R_SLOTS + V_SLOTS) * 8;        // fp16 elements per ring stage
constexpr int NSTAGE = 4;
constexpr float RESCALE_TAU = 8.f;   // log2 units
constexpr int MPF = 4;               // MFMA operand fragments read ahead
static_assert(LPW * 64 * NW == N_SLOTS + R_SLOTS + V_SLOTS, "tile chunks must split evenly over the waves");
static_assert(N_SLOTS % 64 == 0 && R_SLOTS % 64 == 0, "a copy must not straddle two parts");

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

// Chunk swizzles (stored chunk = logical chunk ^ swizzle(row)), measured free of
// LDS bank conflicts for the 16-byte reads below, where 16 consecutive lanes
// read 16 consecutive rows: 256-byte rows need 16 distinct chunks over those
// rows, 128-byte rows (two per bank sweep) 8 distinct chunks per row parity.
__device__ __forceinline__ int sw_n(int row) { return row & 15; }
__device__ __forceinline__ int sw_8(int row) { return (row >> 1) & 7; }

// key offset (inside its 32-key block) carried by LDS row rho of that block
__device__ __forceinline__ int key_of_row(int rho) {
  const int g = rho >> 3, x = (rho >> 2) & 1, r = rho & 3;
  return 16 * (g >> 1) + 8 * x + 4 * (g & 1) + r;
}

template <mla_dtype OT>
__global__ void __launch_bounds__(NTHREADS)
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
  const int i = iw0 + l32;                 // this lane's query row
  const bool row_ok = i < a.Sq;
  const float c_log2 = a.scale * MLA_LOG2E;

  // ---- Q^T operand in registers (fp16, scaled into the log2 domain) ----------
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
        qf[ks][2 * e] = (_Float16)(bf16_bits_to_float((uint16_t)(raw[e] & 0xffff)) * c_log2);
        qf[ks][2 * e + 1] = (_Float16)(bf16_bits_to_float((uint16_t)(raw[e] >> 16)) * c_log2);
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
        qf[ks][e] = (_Float16)(r * c_log2);
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
  const int ntile = (kend_wg + KT - 1) / KT;        // tiles end at or before s_pad
  const bool wave_has_rows = iw0 < a.Sq;
  const int kend_w = wave_has_rows ? limit(min(iw0 + QW, a.Sq) - 1) : 0;
  const int kfull_w = wave_has_rows ? limit(iw0) : 0;
  const int lim_i = row_ok ? limit(i) : 0;

  // ---- tile copies: copy u of this wave is instruction g = wave*LPW + u -------
  // Byte offsets of tile 0; tile t adds t * (bytes per tile of that tensor).
  const i32x4_t rs_n = make_rsrc(kn + bh * a.s_pad * DN, (uint32_t)a.s_pad * DN * 2);
  const i32x4_t rs_r = make_rsrc(krot + (int64_t)b * a.s_pad * DR, (uint32_t)a.s_pad * DR * 2);
  const i32x4_t rs_v = make_rsrc(vt + bh * DV * a.s_pad, (uint32_t)a.s_pad * DV * 2);
  int goff[LPW];
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int s = (wave * LPW + u) * 64 + lane;
    if (s < N_SLOTS) {
      const int rho = s >> 4, c = (s & 15) ^ sw_n(rho);
      goff[u] = (32 * (rho >> 5) + key_of_row(rho & 31)) * (DN * 2) + 16 * c;
    } else if (s < N_SLOTS + R_SLOTS) {
      const int sr = s - N_SLOTS, rho = sr >> 3, c = (sr & 7) ^ sw_8(rho);
      goff[u] = (32 * (rho >> 5) + key_of_row(rho & 31)) * (DR * 2) + 16 * c;
    } else {
      const int sv = s - N_SLOTS - R_SLOTS, d = sv >> 3, c = (sv & 7) ^ sw_8(d);
      goff[u] = d * (a.s_pad * 2) + 16 * c;
    }
  }
  // resource and per-tile byte stride of each copy (wave-uniform)
  i32x4_t rs_u[LPW];
  int st_u[LPW];
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int g = wave * LPW + u;
    const bool isn = g < N_SLOTS / 64, isr = !isn && g < (N_SLOTS + R_SLOTS) / 64;
    rs_u[u] = isn ? rs_n : (isr ? rs_r : rs_v);
    st_u[u] = isn ? KT * DN * 2 : (isr ? KT * DR * 2 : KT * 2);
  }
  int issue_stage = 0, issue_tile = 0;
  auto issue = [&]() {                      // next tile in order, into the next ring stage
    LDS_AS uint16_t* dst = (LDS_AS uint16_t*)(Ls + issue_stage * STAGE + wave * LPW * 512);
#pragma unroll
    for (int u = 0; u < LPW; ++u)
      mla_raw_buffer_load_lds(rs_u[u], (LDS_AS void*)(dst + u * 512), 16, goff[u], issue_tile * st_u[u], 0, 0);
    issue_stage = (issue_stage == NSTAGE - 1) ? 0 : issue_stage + 1;
    ++issue_tile;
  };

  // ---- per-lane LDS read pointers ----------------------------------------------
  // A lane reads rows kt*32 + l32 (K parts) or v*32 + l32 (V^T) at logical
  // chunk 2q + hb:
  //   K_nope, k-step ks < 8:  16-chunk rows, q = ks      (kp[ks])
  //   rope,   k-step ks >= 8: 8-chunk rows,  q = ks - 8  (rp[q])
  //   V^T,    key step ps:    8-chunk rows,  q = ps      (vp[q])
  // The row swizzles depend only on l32's low bits, shared by all those rows.
  // kp/rp address the stage of the next tile whose S is computed, vp the stage
  // of the next tile whose PV is computed; each advances with its tile.
  LDS_AS const uint16_t* kp[DN / 16];
  LDS_AS const uint16_t* rp[4];
  LDS_AS const uint16_t* vp[4];
#pragma unroll
  for (int q = 0; q < DN / 16; ++q) kp[q] = (LDS_AS const uint16_t*)Ls + l32 * DN + 8 * ((2 * q + hb) ^ sw_n(l32));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int x = 8 * ((2 * q + hb) ^ sw_8(l32));
    rp[q] = (LDS_AS const uint16_t*)Ls + R0 + l32 * DR + x;
    vp[q] = (LDS_AS const uint16_t*)Ls + V0 + l32 * KT + x;
  }
  int kstage = 0, vstage = 0;
  auto ring_step = [](int& st) {
    const int step = (st == NSTAGE - 1) ? -(NSTAGE - 1) * STAGE : STAGE;
    st = (st == NSTAGE - 1) ? 0 : st + 1;
    return step;
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t oacc[DV / 32];
#pragma unroll
  for (int v = 0; v < DV / 32; ++v)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[v][e] = 0.f;
  f32x16_t sacc[2];             // S^T of the tile between its MFMA phase and its softmax
  f16x8_t pk[KT / 16];          // P of the tile between its softmax and its PV
#pragma unroll
  for (int ps = 0; ps < KT / 16; ++ps)
#pragma unroll
    for (int e = 0; e < 8; ++e) pk[ps][e] = (_Float16)0.f;
  const h2_t ones = {(_Float16)1.f, (_Float16)1.f};

  const int t_full = min(kfull_w / KT, ntile);                 // tiles with every key visible
  const int t_end = min((kend_w + KT - 1) / KT, ntile);        // tiles with any key visible

  // MFMA phase of tile T: O^T += V^T P^T for tile T-1 (16 MFMAs), then
  // S^T = K Q^T for tile T (24 MFMAs, the two 32-key blocks interleaved as two
  // accumulation chains).  The 40 operand fragments come from LDS; each is
  // read MPF MFMAs ahead of its use, a software pipeline that hides the LDS
  // latency inside the wave (the other wave of the SIMD is busy with its
  // softmax meanwhile).  The scheduling fences keep the compiler from hoisting
  // more reads than that, which would cost registers.
  auto mfma_phase = [&](int T) {
    // op k: k < 16 -> PV step ps = k/4, d-block v = k%4;  k >= 16 -> S k-step (k-16)/2, block (k-16)%2
    auto frag = [&](int k) -> f16x8_t {
      if (k < 16) return *(LDS_AS const f16x8_t*)(vp[k >> 2] + (k & 3) * 32 * KT);
      const int ks = (k - 16) >> 1, kt = (k - 16) & 1;
      LDS_AS const uint16_t* src = (ks < DN / 16) ? kp[ks] + kt * 32 * DN : rp[ks - DN / 16] + kt * 32 * DR;
      return *(LDS_AS const f16x8_t*)src;
    };
    // One straight-line variant serves every tile up to the wave's last: the PV
    // of T = 0 multiplies tile 0's V^T (loaded, finite) by P = 0, and the S
    // computed at T = t_end (possibly from a stage holding no tile) is never
    // used.  Past that the wave only copies.  Without any tile nothing runs, so
    // no LDS data that was never written can reach O.
    if (T <= t_end && ntile > 0) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.f;
      constexpr int NOPS = 16 + 2 * (DQK / 16);
      f16x8_t fr[MPF + 1];
#pragma unroll
      for (int k = 0; k < MPF; ++k) fr[k] = frag(k);
#pragma unroll
      for (int k = 0; k < NOPS; ++k) {
        if (k + MPF < NOPS) fr[(k + MPF) % (MPF + 1)] = frag(k + MPF);
        if (k < 16) {
          oacc[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fr[k % (MPF + 1)], pk[k >> 2], oacc[k & 3], 0, 0, 0);
        } else {
          const int ks = (k - 16) >> 1, kt = (k - 16) & 1;
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fr[k % (MPF + 1)], qf[ks], sacc[kt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (T >= 1) {
      const int st = ring_step(vstage);
#pragma unroll
      for (int q = 0; q < 4; ++q) vp[q] += st;
    }
    if (T < ntile) {
      const int st = ring_step(kstage);
#pragma unroll
      for (int q = 0; q < DN / 16; ++q) kp[q] += st;
#pragma unroll
      for (int q = 0; q < 4; ++q) rp[q] += st;
    }
  };

  // Softmax phase of tile T: mask (diagonal tiles), lazy reference max, P in fp16.
  auto softmax_phase = [&](int T) {
    if (T < 0 || T >= t_end) return;
    if (T >= t_full) {
      const int j0 = T * KT;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int g = e >> 2, r = e & 3;
          const int j = j0 + kt * 32 + 16 * (g >> 1) + 8 * hb + 4 * (g & 1) + r;
          if (j >= lim_i) sacc[kt][e] = -INFINITY;
        }
    }
    // Short dependency chains throughout: this runs on a SIMD whose other wave
    // keeps the matrix unit busy, so its latency is what counts.
    float m8[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int kt = c >> 2, e = 4 * (c & 3);
      m8[c] = fmaxf(fmaxf(sacc[kt][e], sacc[kt][e + 1]), fmaxf(sacc[kt][e + 2], sacc[kt][e + 3]));
    }
    float mx = fmaxf(fmaxf(fmaxf(m8[0], m8[1]), fmaxf(m8[2], m8[3])), fmaxf(fmaxf(m8[4], m8[5]), fmaxf(m8[6], m8[7])));
    mx = half_pair_max(mx);
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
    // A row that has seen no visible key keeps m_run = -inf and uses 0.
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float pv[32];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) pv[16 * kt + e] = fast_exp2(sacc[kt][e] - m_use);
    // P elements 8u..8u+7 of block kt feed PV step ps = 2kt + u
#pragma unroll
    for (int ps = 0; ps < KT / 16; ++ps)
#pragma unroll
      for (int e = 0; e < 8; ++e) pk[ps][e] = (_Float16)pv[8 * ps + e];
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ps = 0; ps < KT / 16; ++ps)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const h2_t pr = {pk[ps][2 * e], pk[ps][2 * e + 1]};
        ls[e] = __builtin_amdgcn_fdot2(pr, ones, ls[e], false);
      }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };

  // ---- main loop -----------------------------------------------------------------
  // Two wave groups, one wave of each per SIMD, run half an iteration apart:
  // while one group issues the MFMAs of a tile the other computes a softmax, so
  // each SIMD keeps its matrix unit and its vector ALU busy at the same time.
  //   group 0, iteration T:  MFMA(T)       | barrier | softmax(T)
  //   group 1, iteration T:  softmax(T-1)  | barrier | MFMA(T)
  // Every wave passes the same 2*(ntile+1) barriers.  At the top of iteration T
  // the copies of tile T have landed for every wave, and the last reads of tile
  // T-2 (its PV, in MFMA(T-1)) are done, so the copy of tile T+2 can take its
  // stage: a ring of 4 stages with two tiles in flight.
  auto top = [&](int T) {
    if (T < ntile) {
      if (T + 1 < ntile) wait_vmcnt<LPW>();
      else wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    if (T + 2 < ntile) issue();
  };
  if (ntile > 0) issue();
  if (ntile > 1) issue();
  if (wave < NW / 2) {
    for (int T = 0; T <= ntile; ++T) {
      top(T);
      mfma_phase(T);
      __builtin_amdgcn_s_barrier();
      softmax_phase(T);
    }
  } else {
    for (int T = 0; T <= ntile; ++T) {
      top(T);
      softmax_phase(T - 1);
      __builtin_amdgcn_s_barrier();
      mfma_phase(T);
    }
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
