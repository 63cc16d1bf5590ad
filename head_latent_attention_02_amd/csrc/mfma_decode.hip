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
// Split-KV partial attention.
//
// One workgroup per (chunk, sequence); 8 waves, wave w owns heads 16w ..
// 16w+15 (heads past H idle).  The chunk's cache rows stream through a ring of
// 4 LDS tile buffers of 32 tokens x 576 latent columns (direct buffer->LDS
// loads by 4 loader waves, 3 tiles in flight).  Per tile each wave computes
//   S^T[t][h] = C[t][:576] . q~[h]          (16x16x32 bf16 MFMA, q~ in VGPRs)
//   online softmax in the log2 domain       (each lane owns one head)
//   O^T[d][h] += C^T[d][t] P^T[t][h]        (16x16x32 bf16 MFMA, P in VGPRs)
// so P never leaves registers: the first product's result layout (token rows
// 4q4 + r of each 16-token half) is the k-slot layout the second product needs
// once C^T is read with the LDS transpose read (ds_read_b64_tr_b16).
// The reference max of a head only moves when a tile exceeds it by more than
// 8 (log2 units), which skips the accumulator rescale on most tiles; the
// result is exact either way because l and O share the same reference.
// Inside a tile row the 16-byte chunks are XOR-swizzled by row&7, measured
// free of LDS bank conflicts for both the row reads and the transposed reads.
constexpr int TT = 32;                   // tokens per tile
constexpr int NBUF = 4;                  // tile ring depth
constexpr int CHUNKS = DLAT / 8;         // 16-byte chunks per row (72)
constexpr int NTHREADS = 512;
constexpr int LOADERS = 4;               // waves that issue the tile loads
constexpr int LOADS = TT * CHUNKS / (LOADERS * 64);   // loads per loader wave per tile (9)
constexpr float RESCALE_TAU = 8.f;       // log2 units

typedef short lds_v4s __attribute__((__vector_size__(4 * sizeof(short))));

// 16-byte chunk swizzle of a tile row (measured free of LDS bank conflicts for
// both the row reads and the transposed reads below)
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

__device__ __forceinline__ bf16x8_t cat_bf16(lds_v4s lo, lds_v4s hi) {
  u32x2_t a = __builtin_bit_cast(u32x2_t, lo), b = __builtin_bit_cast(u32x2_t, hi);
  u32x4_t r = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8_t, r);
}

__global__ void __launch_bounds__(NTHREADS)
mfma_splitkv_kernel(DecodeArgs a, const uint16_t* __restrict__ qt, float* __restrict__ lse_part,
                    float* __restrict__ o_part) {
  __shared__ __attribute__((aligned(16))) uint16_t Cs[NBUF][TT * DLAT];

  const int k = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int h = wave * 16 + l16;
  const bool wave_active = wave * 16 < a.H;     // H is a multiple of 16

  const int L = min(max(a.cache_len[b], 0), a.max_len);
  const int csz = (L + a.n_splits - 1) / a.n_splits;
  const int t0 = min(L, k * csz), t1 = min(L, (k + 1) * csz);
  const int ntile = (t1 - t0 + TT - 1) / TT;

  // q~ as the B operand: lane holds q~[h][32ks + 8q4 .. +8]
  bf16x8_t qf[DLAT / 32];
  {
    const uint16_t* qrow = qt + ((int64_t)b * a.H + (wave_active ? h : 0)) * DLAT;
#pragma unroll
    for (int ks = 0; ks < DLAT / 32; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 32 + q4 * 8);
  }

  // Tile loads: loader wave w, instruction i fills tile slots (w*LOADS+i)*64 +
  // lane, i.e. row slot/72 and swizzled chunk slot%72.  The buffer range ends
  // at the chunk's last row, so rows past it read as zero.
  const uint16_t* cbase = static_cast<const uint16_t*>(a.cache) + (int64_t)b * a.cache_stride;
  const i32x4_t rsrc = make_rsrc(cbase, (uint32_t)t1 * (DLAT * 2));
  int voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int slot = ((wave & (LOADERS - 1)) * LOADS + i) * 64 + lane;
    const int r = slot / CHUNKS, pc = slot - r * CHUNKS;
    voff[i] = r * (DLAT * 2) + swz(r, pc) * 16;
  }
  auto issue_tile = [&](int tile) {
    if (wave >= LOADERS) return;
    const int tbyte = (t0 + tile * TT) * (DLAT * 2);
    uint16_t* dst = &Cs[tile & (NBUF - 1)][0];
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      mla_raw_buffer_load_lds(rsrc, (LDS_AS void*)(dst + (wave * LOADS + i) * 512), 16, voff[i] + tbyte, 0, 0, 0);
  };

  const float c_log2 = a.scale * MLA_LOG2E;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t oacc[DC / 16];
#pragma unroll
  for (int d = 0; d < DC / 16; ++d) oacc[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int i = 0; i < NBUF - 1 && i < ntile; ++i) issue_tile(i);

  for (int t = 0; t < ntile; ++t) {
    const int ahead = min(NBUF - 2, ntile - 1 - t);       // tiles issued after tile t
    if (ahead >= 2) wait_vmcnt<2 * LOADS>();
    else if (ahead == 1) wait_vmcnt<LOADS>();
    else wait_vmcnt<0>();
    // own loads of tile t have landed; the barrier makes that true for all
    // waves and also fences the reuse of the buffer read in iteration t-1
    __builtin_amdgcn_s_barrier();
    if (t + NBUF - 1 < ntile) issue_tile(t + NBUF - 1);
    if (!wave_active) continue;

    const uint16_t* C = &Cs[t & (NBUF - 1)][0];
    const int tt = t0 + t * TT;

    // S^T = C q~^T: sacc[st][r] is head h, token 16st + 4q4 + r.  The row read
    // for k-step ks is chunk (4ks + q4) ^ sw(row); since q4 < 4 this is
    // 4*(ks ^ sw/4) + (q4 ^ sw%4), so even and odd k-steps each walk a fixed
    // base in steps of 8 chunks.
    f32x4_t sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    const uint16_t* pe[2];
    const uint16_t* po[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int row = st * 16 + l16;
      const int rsw = row & 7;
      const uint16_t* rp = C + row * DLAT + 8 * (q4 ^ (rsw & 3));
      pe[st] = rp + 32 * (rsw >> 2);          // chunk group of even k-steps
      po[st] = rp + 32 * (1 - (rsw >> 2));    // and of odd ones
    }
    // the two 16-token halves are independent accumulation chains; interleave them
#pragma unroll
    for (int ks = 0; ks < DLAT / 32; ++ks)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint16_t* ap = ((ks & 1) ? po[st] : pe[st]) + 64 * (ks >> 1);
        bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(ap);
        sacc[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[ks], sacc[st], 0, 0, 0);
      }

    // online softmax (log2 domain) with a lazily moved reference max
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
    const bool move = mx > m_run + RESCALE_TAU;         // always true on the first tile
    if (__ballot(move) != 0ull) {
      const float alpha = move ? fast_exp2(m_run - mx) : 1.f;   // 0 on the first tile
      const float m_new = move ? mx : m_run;
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < DC / 16; ++d) oacc[d] *= alpha;
    }
    bf16x8_t pf;
    float rs = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float pv = fast_exp2(sacc[st][r] - m_run);
        rs += pv;
        pf[4 * st + r] = __builtin_bit_cast(__bf16, float_to_bf16_bits(pv));
      }
    l_run += rs;

    // O^T += C^T P^T.  Lane (row d = 16dt + l16, k-slots 8q4 + u) holds
    // C[token][d] for tokens 4q4 + u (u < 4) and 16 + 4q4 + u - 4 (u >= 4):
    // two transposed reads of 4 rows x 16 columns per 16-lane group.
    // Element e0 = 16dt + 4(l16&3) sits in chunk 2dt + x, x = (l16&3)>>1, which
    // the row swizzle s maps to 2(dt ^ s/2) + (x ^ s%2): within each group of 4
    // d-tiles the order is permuted, so 4 bases per row walk in steps of 8 chunks.
    const int ra = 4 * q4 + (l16 >> 2), rb = ra + 16;
    const int sa = ra & 7, sb = rb & 7;
    const int x = (l16 & 3) >> 1, w = 4 * (l16 & 1);
    const uint16_t* pa[4];
    const uint16_t* pb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      pa[m] = C + ra * DLAT + 8 * (2 * (m ^ (sa >> 1)) + (x ^ (sa & 1))) + w;
      pb[m] = C + rb * DLAT + 8 * (2 * (m ^ (sb >> 1)) + (x ^ (sb & 1))) + w;
    }
#pragma unroll
    for (int dt = 0; dt < DC / 16; ++dt) {
      const int m = dt & 3, j = dt >> 2;
      lds_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS lds_v4s*)(pa[m] + 64 * j));
      lds_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS lds_v4s*)(pb[m] + 64 * j));
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cat_bf16(lo, hi), pf, oacc[dt], 0, 0, 0);
    }
  }

  if (!wave_active) return;
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
