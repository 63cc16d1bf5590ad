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

typedef short lds_v4s __attribute__((__vector_size__(4 * sizeof(short))));

__device__ __forceinline__ bf16x8_t cat_bf16(lds_v4s lo, lds_v4s hi) {
  u32x2_t a = __builtin_bit_cast(u32x2_t, lo), b = __builtin_bit_cast(u32x2_t, hi);
  u32x4_t r = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8_t, r);
}

// ---------------------------------------------------------------------------
// q~[b,h,:512] = W_UK[h]^T q_nope[b,h] (fp32 accumulate, bf16 result) and
// q~[b,h,512:] = R(q_pe[b,h], L_b - 1).
//
// Per head this is a small GEMM, q~^T[c][b] = sum_n W[h*256+n][c] q_nope[b][n],
// run on 16x16x32 bf16 MFMA.  A workgroup takes one head, 256 latent columns
// and 64 sequences: it copies the head's 128 x 256 block of W (rows n, which
// is c-contiguous in memory) into LDS and reads it back with the transposed
// LDS read, which hands each lane 4 consecutive n of one column c; q_nope is
// read from global memory in the same n order.  In a 32-wide k-step, k-slot
// 8q4 + u stands for n = 4q4 + u (u < 4) or 16 + 4q4 + u - 4 (u >= 4) on both
// operands.  Each lane ends with 4 consecutive latent columns of one sequence.
constexpr int AM = 64;                  // sequences per workgroup
constexpr int AN = 256;                 // latent columns per workgroup
constexpr int AWSTR = AN * 2 + 8;       // LDS row stride in bytes (padded against bank conflicts)
static_assert(DN * (AN / 8) % 256 == 0, "W block chunks must split evenly over the threads");
__global__ void __launch_bounds__(256)
absorb_mfma_kernel(DecodeArgs a, uint16_t* __restrict__ qt) {
  __shared__ __attribute__((aligned(16))) uint8_t Ws[DN * AWSTR];
  const int h = blockIdx.x, c0 = blockIdx.y * AN, b0 = blockIdx.z * AM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const uint16_t* w = static_cast<const uint16_t*>(a.w);
  const uint16_t* qn = static_cast<const uint16_t*>(a.q_nope);
  // W rows h*256 + n, columns c0 .. c0+255 -> LDS row n (16-byte chunks; all
  // loads are issued before the first LDS write)
  constexpr int WCH = DN * (AN / 8) / 256;          // chunks per thread (16)
  u32x4_t wv[WCH];
#pragma unroll
  for (int it = 0; it < WCH; ++it) {
    const int i = tid + 256 * it, n = i / (AN / 8), ch = i % (AN / 8);
    wv[it] = *reinterpret_cast<const u32x4_t*>(w + ((int64_t)h * (DN + DV) + n) * DC + c0 + 8 * ch);
  }
#pragma unroll
  for (int it = 0; it < WCH; ++it) {
    const int i = tid + 256 * it, n = i / (AN / 8), ch = i % (AN / 8);
    *reinterpret_cast<u32x2_t*>(Ws + n * AWSTR + 16 * ch) = u32x2_t{wv[it][0], wv[it][1]};
    *reinterpret_cast<u32x2_t*>(Ws + n * AWSTR + 16 * ch + 8) = u32x2_t{wv[it][2], wv[it][3]};
  }
  // q_nope^T as the B operand: lane holds sequence b0 + 16 mb + l16 (rows past
  // the batch read the last sequence and are not stored)
  bf16x8_t qb[AM / 16][DN / 32];
#pragma unroll
  for (int mb = 0; mb < AM / 16; ++mb) {
    const int bc = min(b0 + 16 * mb + l16, a.B - 1);
    const uint16_t* row = qn + ((int64_t)bc * a.H + h) * DN;
#pragma unroll
    for (int ks = 0; ks < DN / 32; ++ks) {
      const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(row + 32 * ks + 4 * q4);
      const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(row + 32 * ks + 16 + 4 * q4);
      qb[mb][ks] = __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
    }
  }
  __syncthreads();
  // wave w: latent columns c0 + 64w .. +63 (4 blocks of 16) for all 64 sequences
  f32x4_t acc[4][AM / 16];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < AM / 16; ++mb) acc[nb][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < DN / 32; ++ks) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      // rows n = 32ks + 4q4 + l16/4 (+16), 4 columns from 64w + 16nb + 4(l16&3):
      // transposed, lane l16 receives column 64w + 16nb + l16
      const uint8_t* src = Ws + (32 * ks + 4 * q4 + (l16 >> 2)) * AWSTR + 2 * (64 * wave + 16 * nb + 4 * (l16 & 3));
      const lds_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS lds_v4s*)(src));
      const lds_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS lds_v4s*)(src + 16 * AWSTR));
      const bf16x8_t wf = cat_bf16(lo, hi);
#pragma unroll
      for (int mb = 0; mb < AM / 16; ++mb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, qb[mb][ks], acc[nb][mb], 0, 0, 0);
    }
  }
  // lane holds q~^T[c = c0 + 64w + 16nb + 4q4 + r][b = b0 + 16mb + l16]
#pragma unroll
  for (int mb = 0; mb < AM / 16; ++mb) {
    const int b = b0 + 16 * mb + l16;
    if (b >= a.B) continue;
    uint16_t* dst = qt + ((int64_t)b * a.H + h) * DLAT + c0 + 64 * wave + 4 * q4;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      *reinterpret_cast<u32x2_t*>(dst + 16 * nb) =
          u32x2_t{pack_bf16x2(acc[nb][mb][0], acc[nb][mb][1]), pack_bf16x2(acc[nb][mb][2], acc[nb][mb][3])};
  }
  // RoPE band of the query at the new token's position
  // (both column blocks of the head share the work; a thread's pair index m
  // is fixed, so its frequency is formed once).  The angle is formed and
  // reduced to [-pi, pi] in fp64 (so large positions lose no accuracy), then
  // the fp32 sine and cosine of the reduced angle carry a few fp32 ulps.
  const uint16_t* qp = static_cast<const uint16_t*>(a.q_pe);
  constexpr double TWO_PI_HI = 6.283185307179586, TWO_PI_LO = 2.4492935982947064e-16;
  const int m = tid & 31;
  const double theta = exp(-2.0 * (double)m / (double)DRP * log((double)a.rope_base));
  for (int e = tid + 256 * blockIdx.y; e < AM * 32; e += 256 * gridDim.y) {
    const int b = b0 + (e >> 5);
    if (b >= a.B) break;
    int L = min(max(a.cache_len[b], 0), a.max_len);
    const double ang = (a.q_pos != nullptr ? (double)a.q_pos[b] : (double)(L > 0 ? L - 1 : 0)) * theta;
    const double k = rint(ang * (1.0 / TWO_PI_HI));
    const float r = (float)fma(-k, TWO_PI_LO, fma(-k, TWO_PI_HI, ang));
    float s, c;
    sincosf(r, &s, &c);
    const int64_t row = (int64_t)b * a.H + h;
    float lo = bf16_bits_to_float(qp[row * DRP + m]), hi = bf16_bits_to_float(qp[row * DRP + m + 32]);
    qt[row * DLAT + DC + m] = float_to_bf16_bits(lo * (float)c - hi * (float)s);
    qt[row * DLAT + DC + m + 32] = float_to_bf16_bits(hi * (float)c + lo * (float)s);
  }
}

// ---------------------------------------------------------------------------
// Split-KV partial attention.
//
// One workgroup of 4 waves (one per SIMD, the whole register file each) per
// (chunk, sequence).  The chunk's cache rows stream through a ring of 4 LDS
// tile buffers of 32 tokens x 576 latent columns, filled by direct
// buffer->LDS loads (every lane issues 9 loads of 16 bytes per tile; 2 to 3
// tiles are in flight while one is computed).  The loads carry the
// non-temporal hint: each cache row is read once, and the step's small
// operands (q~, W_kv_b, the partials) then stay in the caches.  Each tile goes through two
// products:
//
//   scores: wave w owns head groups 2w and 2w+1 (32 heads, q~ in VGPRs) and
//     computes S^T[t][h] = C[t][:576] . q~[h] on 16x16x32 bf16 MFMA, then the
//     softmax in the log2 domain (each lane owns one head of each group);
//     P^T (bf16) goes to LDS;
//   values: wave w owns latent columns 128w .. 128w+127 of every head and
//     accumulates O^T[d][h] += C^T[d][t] P^T[t][h] (16x16x32 bf16 MFMA,
//     accumulators in AGPRs).
//
// Splitting the value product by latent column means the tile's 512 value
// columns are read from LDS once per tile in total (with the transposed LDS
// read, ds_read_b64_tr_b16), and P^T for all heads is only 8 KB; the score
// product reads the tile once per 32 heads.
//
// Schedule: iteration T issues the score MFMAs of tile T+1 and then the value
// MFMAs of tile T as one instruction stream, with the softmax of tile T+1 cut
// into 24 small units placed between the value MFMAs, so the vector ALU works
// while the matrix unit does.  P^T is double-buffered in LDS (tile T's is read
// while tile T+1's is written), which leaves one barrier per tile.
//
// Softmax reference: a head's reference is the max of its first tile;
// P = exp2((s - ref) log2(e) scale) stays below 2^8.  A tile whose max
// exceeds the reference by more than 8 (log2 units) flags the pass, and the
// workgroup then recomputes its chunk from the chunk max seen by the first
// pass, so the accumulators are only ever touched by MFMAs.
//
// The score result layout (token rows 4q4 + r of each 16-token half) is kept
// as the k-slot order of the value product: P^T slot 8q4 + u of a head is
// token 4q4 + u (u < 4) or 16 + 4q4 + u - 4 (u >= 4), and the transposed
// reads of C^T use the same permutation, so a score lane writes its 8
// probabilities as one 16-byte chunk that a value lane reads back unchanged.
// Inside a tile row the 16-byte chunks are XOR-swizzled by row&7, measured
// free of LDS bank conflicts for both the row reads and the transposed reads.
constexpr int TT = 32;                   // tokens per tile
constexpr int NBUF = 4;                  // tile ring depth
constexpr int CHUNKS = DLAT / 8;         // 16-byte chunks per row (72)
constexpr int NTHREADS = 256;
constexpr int NW = NTHREADS / 64;        // waves
constexpr int MAXG = 8;                  // head groups of 16 (128 heads)
constexpr int LOADS = TT * CHUNKS / NTHREADS;         // loads per lane per tile (9)
constexpr int DT_W = DC / 16 / NW;       // value-product d-tiles per wave (8)
constexpr int KS = DLAT / 32;            // score k-steps (18)
constexpr int SPF = 4;                   // score fragments read ahead of their MFMAs
constexpr float TAU = 8.f;               // log2 units: a tile past the reference by more flags a redo

// 16-byte chunk swizzle of a tile row (measured free of LDS bank conflicts for
// both the row reads and the transposed reads below)
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

// acc += A B on the 16x16x32 bf16 MFMA, with the accumulator held in AGPRs.
// Written as inline assembly so that the value-product accumulators (256
// registers) stay in the AGPR file while the score accumulators, which the
// softmax reads, are VGPRs.  Every compiler-generated access to these AGPRs
// (zeroing, the final read) is separated from the MFMAs by a
// barrier or an explicit s_nop, which covers the MFMA result latency.
__device__ __forceinline__ void mfma_agpr(f32x4_t& acc, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::); }
// Marks acc as produced here: compiler-generated reads of the accumulator
// (AGPR -> VGPR copies) cannot move above this point, which follows the drain.
__device__ __forceinline__ void agpr_fence(f32x4_t& acc) { asm volatile("" : "+a"(acc)); }
// acc = 0 (0 x 0 + 0 on the same MFMA, so the accumulator never leaves the
// AGPRs).  The zero operand is written by VALU moves that the compiler may
// place right before this statement; the s_nop gives the MFMA the wait states
// that a VALU write needs before an MFMA reads the register.
__device__ __forceinline__ void mfma_agpr_zero(f32x4_t& acc) {
  const bf16x8_t z = {};
  asm volatile("s_nop 4\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(z));
}

// max / sum over the 4 lanes l16 + 16 q4 (q4 = 0..3) that share a head
__device__ __forceinline__ float quad_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  return half_pair_max(v);
}
__device__ __forceinline__ float quad_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  return half_pair_sum(v);
}

template <int NHT>       // head groups of 16 (H = 16 NHT)
__global__ void __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_splitkv_kernel(DecodeArgs a, const uint16_t* __restrict__ qt, float* __restrict__ lse_part,
                    uint16_t* __restrict__ o_part) {
  // 4 x 36 KB tile ring + 2 x 8 KB of P^T: the whole 160 KB.  The end-of-pass
  // flags and the final 1/l go through ring memory once the ring is idle.
  __shared__ __attribute__((aligned(16))) uint16_t Cs[NBUF][TT * DLAT];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[2][MAXG * 16 * TT];   // P^T [h][k-slot]

  const int k = blockIdx.x, b = a.reverse ? a.B - 1 - (int)blockIdx.y : (int)blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int hg0 = 2 * wave;                     // first head group of this wave's scores

  const int L = min(max(a.cache_len[b], 0), a.max_len);
  const int csz = (L + a.n_splits - 1) / a.n_splits;
  const int t0 = min(L, k * csz), t1 = min(L, (k + 1) * csz);
  const int ntile = (t1 - t0 + TT - 1) / TT;

  // Tile loads: lane instruction i fills tile slot s = (wave*9 + i)*64 + lane,
  // i.e. row s/72 and swizzled chunk s%72.  The buffer range ends at the
  // chunk's last row, so rows past it read as zero.
  const uint16_t* cbase = static_cast<const uint16_t*>(a.cache) + (int64_t)(b / a.seq_per_cache) * a.cache_stride;
  const i32x4_t rsrc = make_rsrc(cbase, (uint32_t)t1 * (DLAT * 2));
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);      // wave index as a scalar
  const uint32_t cs_lds = (uint32_t)(uintptr_t)(LDS_AS void*)&Cs[0][0];
  // byte offset inside a tile of the lane's 9 slots (< 36864, two per register)
  uint32_t slot_off[(LOADS + 1) / 2];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int slot = (wave * LOADS + i) * 64 + lane;
    const int r = slot / CHUNKS, pc = slot - r * CHUNKS;
    const uint32_t off = (uint32_t)(r * (DLAT * 2) + swz(r, pc) * 16);
    if (i & 1) slot_off[i >> 1] |= off << 16;
    else slot_off[i >> 1] = off;
  }
  auto issue_tile = [&](int tile) {
    const int tbyte = __builtin_amdgcn_readfirstlane((t0 + tile * TT) * (DLAT * 2));
    const uint32_t dst = cs_lds + (uint32_t)((tile & (NBUF - 1)) * (TT * DLAT * 2) + wave_s * (LOADS * 1024));
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int voff_i = (int)((i & 1) ? (slot_off[i >> 1] >> 16) : (slot_off[i >> 1] & 0xffffu));
      lds_dma_b128_nt(rsrc, dst + i * 1024, voff_i, tbyte);
    }
  };
  // wait until the loads of tile `tile` (issued in order) have landed, given
  // that tiles up to `last_issued` have been issued
  auto wait_tile = [&](int tile, int last_issued) {
    const int after = last_issued - tile;
    if (after >= 3) wait_vmcnt<3 * LOADS>();
    else if (after == 2) wait_vmcnt<2 * LOADS>();
    else if (after == 1) wait_vmcnt<LOADS>();
    else wait_vmcnt<0>();
  };

  // q~ as the B operand: lane holds q~[h][32ks + 8q4 .. +8] for h = 16g + l16
  // of groups g = hg0, hg0 + 1 (zero for a group past H)
  for (int i = 0; i < NBUF - 1 && i < ntile; ++i) issue_tile(i);
  bf16x8_t qf[2][KS];
#pragma unroll
  for (int hg = 0; hg < 2; ++hg) {
    const int g = hg0 + hg;
    const uint16_t* qrow = qt + ((int64_t)b * a.H + 16 * min(g, NHT - 1) + l16) * DLAT + q4 * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 32);
      qf[hg][ks] = (g < NHT) ? v : bf16x8_t{};
    }
  }
  // The first tiles go out before q~ is loaded, so that both latencies
  // overlap; after this wait vmcnt counts tile loads only.
  wait_vmcnt<0>();

  // Score-product row reads.  The read for k-step ks is logical chunk 4ks + q4
  // of row l16 (+16 for the second token half, which shares the swizzle); with
  // s = l16 & 7 that is physical chunk 4(ks ^ s/4) + (q4 ^ s%4), so even and
  // odd k-steps each walk a fixed base in steps of 8 chunks.
  int soff_e, soff_o;
  {
    const int rsw = l16 & 7;
    const int rp = l16 * DLAT + 8 * (q4 ^ (rsw & 3));
    soff_e = rp + 32 * (rsw >> 2);
    soff_o = rp + 32 * (1 - (rsw >> 2));
  }
  auto sfrag = [&](const uint16_t* C, int s) -> bf16x8_t {   // s = 2 ks + st
    const int ks = s >> 1, st = s & 1;
    const int off = ((ks & 1) ? soff_o : soff_e) + 64 * (ks >> 1) + st * 16 * DLAT;
    return *reinterpret_cast<const bf16x8_t*>(C + off);
  };
  // Value-product transposed reads.  Lane (row d = 16dt + l16, k-slots 8q4 + u)
  // holds C[token][d] for tokens 4q4 + u (u < 4) and 16 + 4q4 + u - 4 (u >= 4):
  // two reads of 4 rows x 16 columns per 16-lane group, rows ra and ra + 16
  // (same swizzle).  Element 16dt + 4(l16&3) sits in chunk 2dt + x,
  // x = (l16&3)>>1, which the row swizzle s maps to 2(dt ^ s/2) + (x ^ s%2);
  // this wave's d-tiles are dt = 8 wave + i, so dt & 3 = i & 3 and
  // dt >> 2 = 2 wave + i/4.
  int voff[4];
  {
    const int ra = 4 * q4 + (l16 >> 2);
    const int sa = ra & 7;
    const int x = (l16 & 3) >> 1, w4 = 4 * (l16 & 1);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      voff[m] = ra * DLAT + 8 * (2 * (m ^ (sa >> 1)) + (x ^ (sa & 1))) + w4 + 128 * wave;
  }
  auto vfrag = [&](const uint16_t* Cv, int i) -> bf16x8_t {    // C^T fragment of d-tile 8 wave + i
    const int off = voff[i & 3] + 64 * (i >> 2);
    lds_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS lds_v4s*)(Cv + off));
    lds_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS lds_v4s*)(Cv + off + 16 * DLAT));
    return cat_bf16(lo, hi);
  };
  auto pfrag = [&](const uint16_t* Pv, int g) -> bf16x8_t {    // P^T fragment of head group g
    return *reinterpret_cast<const bf16x8_t*>(&Pv[(16 * g + l16) * TT + 8 * q4]);
  };

  const float c_log2 = a.scale * MLA_LOG2E;
  // m_ref / m_max in score units; mc = m_ref * c_log2 (0 while unset)
  float m_ref[2] = {-INFINITY, -INFINITY}, m_max[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  float mc[2] = {0.f, 0.f};
  bool exceeded = false;
  f32x4_t oacc[DT_W][NHT];                      // [d-tile of this wave][head group]
  f32x4_t sacc[2][2];                           // [token half][head group]

  // Score product of the tile in Csc: S^T[t][h] for 32 tokens x this wave's
  // 32 heads, 72 MFMAs in four accumulation chains; fragments are read SPF
  // ahead of their MFMAs.
  auto score_phase = [&](const uint16_t* Csc) {
    bf16x8_t af[SPF + 1];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int hg = 0; hg < 2; ++hg) sacc[st][hg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < SPF; ++s) af[s] = sfrag(Csc, s);
#pragma unroll
    for (int s = 0; s < 2 * KS; ++s) {
      if (s + SPF < 2 * KS) af[(s + SPF) % (SPF + 1)] = sfrag(Csc, s + SPF);
      const int ks = s >> 1, st = s & 1;
#pragma unroll
      for (int hg = 0; hg < 2; ++hg)
        sacc[st][hg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s % (SPF + 1)], qf[hg][ks], sacc[st][hg], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Softmax of the tile whose scores are in sacc (first token tt), against
  // the pass's reference: P^T = exp2((s - m_ref) c_log2) in bf16 to Pn, row
  // sums to l_run.  The reference is the row max of the first tile (or, on a
  // second pass, the chunk's max); a later tile whose max exceeds it by more
  // than tau flags the pass for a redo, so the accumulators are only ever
  // touched by MFMAs and P stays below 2^tau.  Unit j of head group hg is
  // 12 hg + j; the units run between the value MFMAs of the previous tile.
  float sm8[2], rs[2], pv_prev[2];
  bf16x8_t pf[2];
  auto softmax_unit = [&](auto j_c, int tt, uint16_t* Pn) __attribute__((always_inline)) {
    constexpr int jj = decltype(j_c)::value, hg = jj / 12, j = jj % 12;
    if constexpr (j == 0) {
      if (hg == 0 && tt + TT > t1) {      // tail tile: tokens past the chunk end get no weight
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (tt + 16 * st + 4 * q4 + r >= t1) sacc[st][h2][r] = -INFINITY;
      }
      sm8[hg] = max3(max3(sacc[0][hg][0], sacc[0][hg][1], sacc[0][hg][2]),
                     max3(sacc[0][hg][3], sacc[1][hg][0], sacc[1][hg][1]), max2(sacc[1][hg][2], sacc[1][hg][3]));
    } else if constexpr (j == 1) {
      auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(sm8[hg]), __float_as_uint(sm8[hg]), false, false);
      sm8[hg] = max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
    } else if constexpr (j == 2) {
      auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sm8[hg]), __float_as_uint(sm8[hg]), false, false);
      const float mx = max2(__uint_as_float(r2[0]), __uint_as_float(r2[1]));   // the head's max over the tile
      m_max[hg] = max2(m_max[hg], mx);
      if (m_ref[hg] == -INFINITY) m_ref[hg] = mx;        // first tile of the first pass
      else exceeded |= (mx - m_ref[hg]) * c_log2 > TAU;
      mc[hg] = (m_ref[hg] == -INFINITY) ? 0.f : m_ref[hg] * c_log2;
      rs[hg] = 0.f;
    } else if constexpr (j < 11) {
      constexpr int e = j - 3, st = e >> 2, r = e & 3;
      const float p = fast_exp2(fmaf(sacc[st][hg][r], c_log2, -mc[hg]));
      if constexpr (e > 0) rs[hg] += pv_prev[hg];
      pv_prev[hg] = p;
      pf[hg][e] = (__bf16)p;         // round to nearest even
    } else {
      l_run[hg] += rs[hg] + pv_prev[hg];
      const int h = 16 * (hg0 + hg) + l16;
      *reinterpret_cast<bf16x8_t*>(&Pn[h * TT + 8 * q4]) = pf[hg];
    }
  };
  constexpr int N_UNITS = 24;

  // Iteration T: the score product of tile T+1 and then the value product of
  // tile T, as one instruction stream, with the softmax of tile T+1 in units
  // between the value MFMAs.  Tile T+1 past the last one reads a stale ring
  // stage; all its tokens are past the chunk end, so it adds nothing.
  auto iteration = [&](int T) __attribute__((always_inline)) {
    const uint16_t* Cv = &Cs[T & (NBUF - 1)][0];
    const uint16_t* Cn = &Cs[(T + 1) & (NBUF - 1)][0];
    const uint16_t* Pv = &Ps[T & 1][0];
    uint16_t* Pn = &Ps[(T + 1) & 1][0];
    const int tt = t0 + (T + 1) * TT;
    bf16x8_t cf[DT_W], pg[2];
#pragma unroll
    for (int j = 0; j < DT_W / 2; ++j) cf[j] = vfrag(Cv, j);
    pg[0] = pfrag(Pv, 0);
    score_phase(Cn);
#pragma unroll
    for (int j = DT_W / 2; j < DT_W; ++j) cf[j] = vfrag(Cv, j);
    // value MFMA v = DT_W g + j (head group major, so each P^T fragment is read
    // once); a softmax unit after every second one
    static_for<NHT>([&](auto gc) __attribute__((always_inline)) {
      constexpr int g = decltype(gc)::value;
      if constexpr (g + 1 < NHT) pg[(g + 1) & 1] = pfrag(Pv, g + 1);
      static_for<DT_W>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        mfma_agpr(oacc[j][g], cf[j], pg[g & 1]);
        constexpr int v = DT_W * g + j;
        if constexpr (v % 2 == 0 && v / 2 < N_UNITS) softmax_unit(std::integral_constant<int, v / 2>{}, tt, Pn);
        __builtin_amdgcn_sched_barrier(0);
      });
    });
    // units the value product had no room for (few head groups)
    static_for<N_UNITS>([&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      if constexpr (u >= DT_W * NHT / 2) softmax_unit(uc, tt, Pn);
    });
  };

  // Prologue of a pass: scores and softmax of tile 0 (into Ps[0]).  Loop:
  // at the top of iteration T tile T+1 has landed, P^T of tile T is in
  // Ps[T&1] for every head, and every wave is done with iteration T-1, so
  // tile T+3 takes the ring stage of tile T-1.  A redo (second pass) starts
  // from the chunk max seen by the first pass, which no tile exceeds.
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int i = 0; i < DT_W; ++i)
#pragma unroll
      for (int g = 0; g < NHT; ++g) mfma_agpr_zero(oacc[i][g]);
    l_run[0] = l_run[1] = 0.f;
    if (pass > 0)
      for (int i = 0; i < NBUF - 1 && i < ntile; ++i) issue_tile(i);
    if (ntile > 0) {
      wait_tile(0, min(NBUF - 2, ntile - 1));
      __syncthreads();
      score_phase(&Cs[0][0]);
      static_for<N_UNITS>([&](auto uc) __attribute__((always_inline)) { softmax_unit(uc, t0, &Ps[0][0]); });
    }
    for (int T = 0; T < ntile; ++T) {
      if (T + 1 < ntile) wait_tile(T + 1, min(T + NBUF - 2, ntile - 1));
      __syncthreads();
      if (T + NBUF - 1 < ntile) issue_tile(T + NBUF - 1);
      iteration(T);
    }
    // end of pass: did any head of any wave exceed its reference?
    __syncthreads();                             // the ring is idle
    int* flags = reinterpret_cast<int*>(&Cs[0][0]);
    flags[wave] = (__ballot(exceeded) != 0ull) ? 1 : 0;    // every lane stores the same value
    __syncthreads();
    const int redo = flags[0] | flags[1] | flags[2] | flags[3];
    __syncthreads();                             // flags read before the ring is refilled
    if (!__builtin_amdgcn_readfirstlane(redo)) break;
    m_ref[0] = m_max[0];
    m_ref[1] = m_max[1];
    mc[0] = (m_ref[0] == -INFINITY) ? 0.f : m_ref[0] * c_log2;
    mc[1] = (m_ref[1] == -INFINITY) ? 0.f : m_ref[1] * c_log2;
    exceeded = false;
    mfma_drain();
  }

  // The ring is idle now.  Each wave stages its O^T block as rows of heads
  // (fp16, rows padded by 16 bytes against bank conflicts) in its own 34 KB of
  // ring memory, then stores whole 256-byte row pieces of o_part; 1/l per head
  // sits after the four staging areas.
  constexpr int OSTR = 128 * 2 + 16;                      // staging row stride (bytes)
  uint8_t* ring = reinterpret_cast<uint8_t*>(&Cs[0][0]);
  static_assert(4 * MAXG * 16 * OSTR + MAXG * 16 * 4 <= NBUF * TT * DLAT * 2, "staging fits in the ring");
  float* linv_s = reinterpret_cast<float*>(ring + 4 * MAXG * 16 * OSTR);
#pragma unroll
  for (int hg = 0; hg < 2; ++hg) {
    if (hg0 + hg >= NHT) break;
    const float l = quad_sum(l_run[hg]);
    const int h = 16 * (hg0 + hg) + l16;
    if (q4 == 0) {
      linv_s[h] = (l > 0.f) ? 1.f / l : 0.f;
      lse_part[((int64_t)b * a.n_splits + k) * a.H + h] =
          (l > 0.f) ? (m_ref[hg] * c_log2 + __log2f(l)) * MLA_LN2 : -INFINITY;
    }
  }
  __syncthreads();
  mfma_drain();
  // lane holds O^T[d = 16 (8 wave + i) + 4q4 + r][h = 16g + l16]
  // (fp16: the normalised partial is a convex combination of cache rows)
  uint8_t* stg = ring + wave * (MAXG * 16 * OSTR);
#pragma unroll
  for (int g = 0; g < NHT; ++g) {
    const int hh = 16 * g + l16;
    const float inv = linv_s[hh];
#pragma unroll
    for (int i = 0; i < DT_W; ++i) {
      agpr_fence(oacc[i][g]);
      const f32x4_t v = oacc[i][g] * inv;
      *reinterpret_cast<u32x2_t*>(stg + hh * OSTR + (16 * i + 4 * q4) * 2) =
          u32x2_t{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
    }
  }
  // a wave reads back only the rows its own lanes wrote: 4 heads x 256 bytes
  // per instruction
  lds_wave_fence();
  uint16_t* dst = o_part + ((int64_t)b * a.n_splits + k) * a.H * DC + 128 * wave;
#pragma unroll
  for (int it = 0; it < 4 * NHT; ++it) {
    const int row = 4 * it + (lane >> 4), c = lane & 15;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + row * OSTR + 16 * c);
    *reinterpret_cast<u32x4_t*>(dst + (int64_t)row * DC + 8 * c) = v;
  }
}

}  // namespace

hipError_t launch_absorb_bf16(const DecodeArgs& a, uint16_t* qt, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  dim3 grid(a.H, DC / AN, (a.B + AM - 1) / AM);
  hipLaunchKernelGGL(absorb_mfma_kernel, grid, dim3(256), 0, stream, a, qt);
  return hipGetLastError();
}

hipError_t launch_mfma_splitkv(const DecodeArgs& a, const uint16_t* qt, float* lse_part, uint16_t* o_part,
                               hipStream_t stream) {
  dim3 grid(a.n_splits, a.B);
  switch (a.H >> 4) {
#define MLA_SPLITKV_CASE(n)                                                                               \
  case n:                                                                                                 \
    hipLaunchKernelGGL(mfma_splitkv_kernel<n>, grid, dim3(NTHREADS), 0, stream, a, qt, lse_part, o_part); \
    break;
    MLA_SPLITKV_CASE(1)
    MLA_SPLITKV_CASE(2)
    MLA_SPLITKV_CASE(3)
    MLA_SPLITKV_CASE(4)
    MLA_SPLITKV_CASE(5)
    MLA_SPLITKV_CASE(6)
    MLA_SPLITKV_CASE(7)
    MLA_SPLITKV_CASE(8)
#undef MLA_SPLITKV_CASE
    default:
      return hipErrorInvalidValue;   // excluded by the host-side eligibility check
  }
  return hipGetLastError();
}
