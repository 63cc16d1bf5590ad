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
// 16 bytes per lane, 5 per wave per tile) through a ring of 3 stages, two
// tiles ahead of the one being consumed.  In every tile row the 16-byte chunks
// are XOR-swizzled with row & 7, so the 16-byte operand reads of a lane group
// fall in distinct banks.
//
// Only the diagonal tiles run the masked variant of the tile code; tiles past
// a wave's last visible key are skipped.  The reference max of a row only
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
constexpr int NSTAGE = 3;
constexpr float RESCALE_TAU = 8.f;   // log2 units
static_assert(LPW * 64 * NW == N_SLOTS + R_SLOTS + V_SLOTS, "tile chunks must split evenly over the waves");
static_assert(N_SLOTS % 64 == 0 && R_SLOTS % 64 == 0, "a copy must not straddle two parts");

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

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
  const int sw = l32 & 7;                  // row swizzle of every row this lane reads
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
      const int rho = s >> 4, c = (s & 15) ^ (rho & 7);
      goff[u] = (32 * (rho >> 5) + key_of_row(rho & 31)) * (DN * 2) + 16 * c;
    } else if (s < N_SLOTS + R_SLOTS) {
      const int sr = s - N_SLOTS, rho = sr >> 3, c = (sr & 7) ^ (rho & 7);
      goff[u] = (32 * (rho >> 5) + key_of_row(rho & 31)) * (DR * 2) + 16 * c;
    } else {
      const int sv = s - N_SLOTS - R_SLOTS, d = sv >> 3, c = (sv & 7) ^ (d & 7);
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

  // ---- per-lane LDS read offsets (fp16 elements within a stage) --------------
  // A lane reads rows kt*32 + l32 (K parts) or v*32 + l32 (V^T), all with row
  // swizzle sw, at logical chunk 2q + hb of an 8-chunk group q:
  //   K_nope, k-step ks < 8:  row pitch 16 chunks, group ks/4, q = ks%4
  //   rope,   k-step ks >= 8: row pitch 8 chunks, q = ks-8
  //   V^T,    key step ps:    row pitch 8 chunks, q = ps (keys 16ps + 8hb .. +7)
  // The pointers address the stage of the tile being consumed and advance with it.
  LDS_AS const uint16_t* np[4];
  LDS_AS const uint16_t* rp[4];             // V^T: rp[q] + (V0 - R0), since l32*KT = l32*DR
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int x = 8 * ((2 * q + hb) ^ sw);
    np[q] = (LDS_AS const uint16_t*)Ls + l32 * DN + x;
    rp[q] = (LDS_AS const uint16_t*)Ls + R0 + l32 * DR + x;
  }
  static_assert(KT == DR, "V^T and rope rows share the per-lane offsets");

  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t oacc[DV / 32];
#pragma unroll
  for (int v = 0; v < DV / 32; ++v)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[v][e] = 0.f;
  const h2_t ones = {(_Float16)1.f, (_Float16)1.f};

  auto tile = [&](int j0, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    // S^T = K Q^T: the two 32-key blocks are independent accumulation chains,
    // interleaved; K fragments are read KPF k-steps ahead of their MFMAs (the
    // scheduling fence keeps the compiler from hoisting all 24 reads, which
    // would need 96 more registers)
    constexpr int KPF = 1;
    auto kread = [&](int ks, int kt) {
      LDS_AS const uint16_t* src = (ks < DN / 16) ? np[ks & 3] + kt * 32 * DN + 64 * (ks >> 2)
                                                  : rp[ks - DN / 16] + kt * 32 * DR;
      return *(LDS_AS const f16x8_t*)src;
    };
    f32x16_t sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.f;
    f16x8_t kfr[KPF + 1][2];
#pragma unroll
    for (int ks = 0; ks < KPF; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) kfr[ks][kt] = kread(ks, kt);
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks) {
      if (ks + KPF < DQK / 16) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) kfr[(ks + KPF) % (KPF + 1)][kt] = kread(ks + KPF, kt);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kfr[ks % (KPF + 1)][kt], qf[ks], sacc[kt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if constexpr (MASKED) {
          const int g = e >> 2, r = e & 3;
          const int j = j0 + kt * 32 + 16 * (g >> 1) + 8 * hb + 4 * (g & 1) + r;
          if (j >= lim_i) sacc[kt][e] = -INFINITY;
        }
        mx = fmaxf(mx, sacc[kt][e]);
      }
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
    // O^T += V^T P^T, 16 keys per step: elements 8u..8u+7 of block kt
#pragma unroll
    for (int ps = 0; ps < KT / 16; ++ps) {
      const int kt = ps >> 1, u = ps & 1;
      f16x8_t pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = (_Float16)fast_exp2(sacc[kt][8 * u + e] - m_use);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const h2_t pr = {pf[2 * e], pf[2 * e + 1]};
        l_run = __builtin_amdgcn_fdot2(pr, ones, l_run, false);
      }
      f16x8_t vf[DV / 32];
#pragma unroll
      for (int v = 0; v < DV / 32; ++v) vf[v] = *(LDS_AS const f16x8_t*)(rp[ps] + (V0 - R0) + v * 32 * KT);
#pragma unroll
      for (int v = 0; v < DV / 32; ++v)
        oacc[v] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[v], pf, oacc[v], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- main loop: ring of NSTAGE tiles, two in flight ------------------------
  if (ntile > 0) issue();
  if (ntile > 1) issue();
  // Every wave passes the same ntile barriers; its own tiles split into the
  // unmasked ones, the diagonal ones (masked) and those past its last key
  // (copies only), each in a loop of its own so that the accumulators keep
  // their registers across iterations.
  int stage = 0;
  auto next_tile = [&](int t) {
    // this wave's copies of tile t have landed (tile t+1's may still run); the
    // barrier extends that to every wave and also retires all reads of tile t-1,
    // whose stage the copy of tile t+2 overwrites
    if (t + 1 < ntile) wait_vmcnt<LPW>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (t + 2 < ntile) issue();
  };
  auto advance = [&]() {
    const int step = (stage == NSTAGE - 1) ? -(NSTAGE - 1) * STAGE : STAGE;
    stage = (stage == NSTAGE - 1) ? 0 : stage + 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      np[q] += step;
      rp[q] += step;
    }
  };
  const int t_full = min(kfull_w / KT, ntile);                 // tiles with every key visible
  const int t_end = min((kend_w + KT - 1) / KT, ntile);        // tiles with any key visible
  int t = 0;
  for (; t < t_full; ++t) {
    next_tile(t);
    tile(t * KT, std::false_type{});
    advance();
  }
  for (; t < t_end; ++t) {
    next_tile(t);
    tile(t * KT, std::true_type{});
    advance();
  }
  for (; t < ntile; ++t) next_tile(t);

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
