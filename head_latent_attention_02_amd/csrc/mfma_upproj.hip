// Latent up-projection on bf16 MFMA (fp32 accumulate, fp16 results).
//
// Explicit form of "A Training-Memory Regression in MLA Sequence Parallelism
// ... LAGA" (Pith review), "What carries the argument" and Fig. 2: per-head
// K_nope and V are the latent rows times the shared linear map W_kv_b.  The
// Fig. 3 caption notes that splitting this product into per-head-shard GEMMs
// made it slower at equal FLOPs, so it runs here as one GEMM over all heads:
//   C[j, n] = sum_c c_kv[b, j, c] * W[n, c],   j < s_vis, n < H * 256.
// Both operands are contiguous along c (W is stored one row per output
// feature), which is the MFMA operand layout, so nothing is transposed on
// the way in.
//
// Outputs (fp16): Kn [B, H, s_pad, 128] and V^T [B, H, 128, s_pad] (key index
// fastest, the layout the attention kernel's P.V product reads), or, for the
// backward, V in rows [B, H, s_pad, 128] like Kn.
//
// Persistent kernel, one workgroup of 8 waves per CU (two waves per SIMD:
// while one is held issuing its tile copies, the other keeps the SIMD's
// matrix unit busy; waves 0-3 issue theirs at the start of a reduction step,
// waves 4-7 after their first 8 MFMAs of it).  A tile is 256 latent rows x the 256 output columns of
// one head; waves 0-3 produce its K_nope half (W rows as the A operand, so
// each lane ends with 4 consecutive features of one key) and waves 4-7 its V
// half (latent rows as the A operand, so each lane ends with 4 consecutive
// keys of one feature), 128 x 64 per wave on 32x32x16 MFMA with the
// accumulators in AGPRs.  The reduction over the 512 latent columns
// streams in steps of 32 through a ring of 4 LDS stages (16 KB of latent
// rows + 16 KB of W rows each) filled by direct buffer->LDS loads; the ring
// runs across tile boundaries, so the next tile's first steps are in flight
// while a tile's results are converted and stored.  Tiles are dealt so that
// the 32 CUs of an XCD work on 4 heads x 8 key tiles at a time (1 MB of W and
// 2 MB of latent rows, inside that XCD's L2).
#include "common.h"
#include "kernels.h"

namespace {

constexpr int TJ = 256;          // latent rows per tile
constexpr int TN = 256;          // output columns per tile (= one head)
constexpr int TK = 32;           // reduction step
constexpr int DKV = 512;
constexpr int NKS = DKV / TK;    // reduction steps per tile (16)
constexpr int NSTAGE = 4;        // LDS ring depth
constexpr int NTHREADS = 512;
constexpr int REG_BYTES = TJ * TK * 2;       // one operand region of a stage (16 KB)
constexpr int STAGE_BYTES = 2 * REG_BYTES;   // latent rows then W rows
constexpr int LOADS = 2 * REG_BYTES / 16 / NTHREADS;   // 16-byte copies per lane per step (4)
constexpr int COPY_ROWS = NTHREADS / 4;                 // 64-byte rows one copy instruction fills (128)
constexpr int STG_BYTES = 16 * 256;                     // output staging per wave: 16 rows of 256 bytes

// acc += A B on the 32x32x16 bf16 MFMA with the accumulator held in AGPRs
// (the 128 accumulator registers stay in AGPRs; operands stay in VGPRs).
__device__ __forceinline__ void mfma32_agpr(f32x16_t& acc, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// acc = A B (the first product of a tile starts the accumulation)
__device__ __forceinline__ void mfma32_agpr_first(f32x16_t& acc, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::); }
// Marks acc as produced here: compiler-generated reads of the accumulator
// (AGPR -> VGPR copies) cannot move above this point, which follows the
// drain.  Used for one column of blocks at a time, so that only those blocks
// are copied out at once.
__device__ __forceinline__ void agpr_fence(f32x16_t& acc) { asm volatile("" : "+a"(acc)); }

// tile id -> (batch*head, key tile)
__device__ __forceinline__ void tile_coords(int tile, int n_jt, bool xcd_deal, int& bh, int& jt) {
  if (xcd_deal) {
    // 256 consecutive tile ids = 8 groups of 32 (one per XCD); group c covers
    // heads 4(c/2) .. 4(c/2)+3 and key tiles 8(c%2) .. 8(c%2)+7 of a 16-tile row
    const int step = tile >> 8, w = tile & 255;
    const int xcd = w & 7, m = w >> 3;
    const int c = step * 8 + xcd;
    bh = 4 * (c >> 1) + (m >> 3);
    jt = 8 * (c & 1) + (m & 7);
  } else {
    bh = tile / n_jt;
    jt = tile - bh * n_jt;
  }
}

__global__ void __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
mfma_upproj_kernel(const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ w,
                   uint16_t* __restrict__ kn, uint16_t* __restrict__ vt, int B, int H, int Skv,
                   int s_vis, int s_pad, int n_jt, int n_tiles, int xcd_deal, int v_rows) {
  // the copy ring, then the output staging of the 8 waves
  __shared__ __attribute__((aligned(16))) uint16_t Ls[(NSTAGE * STAGE_BYTES + NTHREADS / 64 * STG_BYTES) / 2];
  uint8_t* const stg_all = reinterpret_cast<uint8_t*>(Ls) + NSTAGE * STAGE_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hb = lane >> 5;
  const int part = wave >> 2;          // 0: K_nope columns, 1: V columns
  const int jq = (wave >> 1) & 1;      // 128-row half of the A side
  const int nh = wave & 1;             // 64-row half of the B side
  const int G = gridDim.x;
  const int my_tiles = (n_tiles - (int)blockIdx.x + G - 1) / G;
  const int total_steps = my_tiles * NKS;

  // Stage layout: rows of 32 bf16 (64 bytes = 4 chunks of 16 bytes); chunk c
  // of row r sits at chunk c ^ ((r >> 2) & 3), which spreads the 16 rows that
  // a 16-lane group reads over all 64 banks.
  // Copies: lane instruction i covers slot s = 512 i + tid of a region, i.e.
  // row 128 i + tid/4, physical chunk tid & 3 (the swizzle only depends on
  // tid, so one per-lane offset serves every row block, step and tile).
  const int v_lane = (tid >> 2) * (DKV * 2) + (((tid & 3) ^ ((tid >> 4) & 3)) * 16);
  const uint32_t ls_lds = (uint32_t)(uintptr_t)(LDS_AS void*)&Ls[0];

  // fragment reads: A/B operand of the 32x32x16 MFMA = 8 consecutive bf16
  // (logical chunk 2kk + hb) of row l32 of a 32-row block; rows 32x + l32 of
  // a 128-row group share the swizzle (l32 >> 2) & 3
  const int sw = (l32 >> 2) & 3;
  const int frag_off0 = l32 * (TK * 2) + ((0 + hb) ^ sw) * 16;   // kk = 0
  const int frag_off1 = l32 * (TK * 2) + ((2 + hb) ^ sw) * 16;   // kk = 1
  // first (A) and second (B) operand regions of this wave, byte offsets in a stage
  // With v_rows the V half is formed like the K_nope half (W rows 128..255 as
  // the A operand) and stored as rows [B, H, s_pad, 128] into vt.
  const bool row_form = part == 0 || v_rows != 0;
  const int a_rows = row_form ? (REG_BYTES + part * 128 * TK * 2) : (jq * 128 * TK * 2);
  const int b_rows = row_form ? ((jq * 128 + nh * 64) * TK * 2) : (REG_BYTES + (128 + nh * 64) * TK * 2);

  // Copy-issue state: the step issued next is step is_ks of the block's
  // tile is_t, into ring stage is_stage; ra / rb address that tile's latent
  // rows and W rows and change only when the issue moves on to a new tile, so
  // the per-step issue is the copies alone.
  int is_t = 0, is_ks = 0, is_stage = 0;
  i32x4_t ra, rb;
  auto set_issue_tile = [&](int t) {
    int bh, jt;
    tile_coords((int)blockIdx.x + t * G, n_jt, xcd_deal != 0, bh, jt);
    const int h = bh % H, b = bh / H;
    const int j0 = jt * TJ;
    const int rows = max(0, min(TJ, s_vis - j0));
    ra = make_rsrc_uniform(c_kv + ((int64_t)b * Skv + j0) * DKV, (uint32_t)rows * (DKV * 2));
    rb = make_rsrc_uniform(w + (int64_t)h * TN * DKV, (uint32_t)TN * (DKV * 2));
  };
  auto issue_next = [&]() {
    const uint32_t dst = ls_lds + (uint32_t)(is_stage * STAGE_BYTES) + (uint32_t)wave * 1024u;
#pragma unroll
    for (int i = 0; i < LOADS / 2; ++i) {
      const int so = i * COPY_ROWS * (DKV * 2) + is_ks * (TK * 2);
      lds_dma_b128(ra, dst + i * (NTHREADS * 16), v_lane, so);
      lds_dma_b128(rb, dst + REG_BYTES + i * (NTHREADS * 16), v_lane, so);
    }
  };
  auto advance_issue = [&]() {
    is_stage = (is_stage + 1) & (NSTAGE - 1);
    if (++is_ks == NKS) {
      is_ks = 0;
      if (++is_t < my_tiles) set_issue_tile(is_t);
    }
  };
  static_assert((NSTAGE & (NSTAGE - 1)) == 0, "ring depth is a power of two");

  f32x16_t acc[4][2];
  const int ahead = min(NSTAGE - 1, total_steps);
  if (my_tiles > 0) set_issue_tile(0);
  for (int g = 0; g < ahead; ++g) { issue_next(); advance_issue(); }

  for (int t = 0; t < my_tiles; ++t) {
    for (int ks = 0; ks < NKS; ++ks) {
      const int g = t * NKS + ks;
      // copies of step g have landed (later steps may still be in flight)
      const int newer = min(NSTAGE - 2, total_steps - 1 - g);
      static_assert(NSTAGE - 2 <= 3, "wait counts below cover up to 3 newer steps");
      if (newer >= 3) wait_vmcnt<3 * LOADS>();
      else if (newer == 2) wait_vmcnt<2 * LOADS>();
      else if (newer == 1) wait_vmcnt<LOADS>();
      else wait_vmcnt<0>();
      __syncthreads();           // ... for every wave; stage g-1 is free again
      const bool issue_now = g + NSTAGE - 1 < total_steps;
      if (wave < 4 && issue_now) issue_next();

      const char* st = reinterpret_cast<const char*>(Ls) + (g % NSTAGE) * STAGE_BYTES;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int fo = kk ? frag_off1 : frag_off0;
        bf16x8_t fa[4], fb[2];
#pragma unroll
        for (int x = 0; x < 4; ++x)
          fa[x] = *reinterpret_cast<const bf16x8_t*>(st + a_rows + x * 32 * (TK * 2) + fo);
#pragma unroll
        for (int y = 0; y < 2; ++y)
          fb[y] = *reinterpret_cast<const bf16x8_t*>(st + b_rows + y * 32 * (TK * 2) + fo);
        if (kk == 0 && ks == 0) {
#pragma unroll
          for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) mfma32_agpr_first(acc[x][y], fa[x], fb[y]);
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) mfma32_agpr(acc[x][y], fa[x], fb[y]);
        }
        // waves 4-7 issue theirs while waves 0-3 (one per SIMD) run their MFMAs
        if (kk == 0 && wave >= 4 && issue_now) issue_next();
      }
      if (issue_now) advance_issue();
    }

    // epilogue (the next tile's first steps are already in flight): the
    // wave's 64 output rows (keys of K_nope, features of V^T) go out in four
    // rounds of 16 rows, each staged in the wave's 4 KB of LDS so that every
    // store writes whole 256-byte row segments.  The stores are non-temporal,
    // so that the 4 MB an XCD writes per round of tiles does not push the
    // latent rows, which the XCD's next tiles read again, out of its L2.  In a 32x32 block lane
    // (l32, hb) holds, for each group g, 4 consecutive outputs of row l32 at
    // column 8g + 4hb of the block; a staged row's 16-byte chunks are
    // XOR-swizzled by the row, which keeps both the 8-byte writes and the
    // 16-byte reads free of bank conflicts.
    int bh, jt;
    tile_coords((int)blockIdx.x + t * G, n_jt, xcd_deal != 0, bh, jt);
    const int j0 = jt * TJ;
    uint8_t* stg = stg_all + wave * STG_BYTES;
    mfma_drain();
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      uint32_t wd[4][4][2];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        agpr_fence(acc[x][y]);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          wd[x][g][0] = pack_f16x2(acc[x][y][4 * g + 0], acc[x][y][4 * g + 1]);
          wd[x][g][1] = pack_f16x2(acc[x][y][4 * g + 2], acc[x][y][4 * g + 3]);
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if ((l32 >> 4) == h) {
          const int rr = l32 & 15;
#pragma unroll
          for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int g = 0; g < 4; ++g)
              *reinterpret_cast<u32x2_t*>(stg + rr * 256 + (((4 * x + g) ^ rr) * 16) + 8 * hb) =
                  u32x2_t{wd[x][g][0], wd[x][g][1]};
        }
        // other lanes' writes are read below: no access moves across, and the
        // writes are complete
        lds_wave_fence();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 4 * i + (lane >> 4), c = lane & 15;
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + rr * 256 + ((c ^ rr) * 16));
          const int row = nh * 64 + y * 32 + 16 * h + rr;   // within the tile's 256 rows / 128 features
          if (row_form) {
            // K_nope (or V) row of key j0 + jq*128 + row, features 8c .. 8c+7
            uint16_t* dst = (part == 0 ? kn : vt) + ((int64_t)bh * s_pad + j0 + jq * 128 + row) * 128 + 8 * c;
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst));
          } else {
            // V^T row of feature row, keys j0 + jq*128 + 8c .. +7
            uint16_t* dst = vt + ((int64_t)bh * 128 + row) * s_pad + j0 + jq * 128 + 8 * c;
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst));
          }
        }
        lds_wave_fence();                   // the reads are done before the next round's writes
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

}  // namespace

hipError_t launch_mfma_upproj(const ExplicitArgs& a, uint16_t* kn, uint16_t* vt, hipStream_t stream, bool v_rows) {
  if (a.s_vis == 0) return hipSuccess;
  const int n_jt = a.s_pad / TJ;
  const int n_tiles = a.B * a.H * n_jt;
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n_cu = 256;
  int grid = n_cu;                                   // one workgroup per CU
  if (grid > n_tiles) grid = n_tiles;
  // the XCD-aware dealing needs whole rounds of 256 tiles over 256 CUs,
  // heads in groups of 4 and key rows in tiles of 16
  const int xcd_deal = (grid == 256 && n_tiles % 256 == 0 && n_jt == 16 && (a.B * a.H) % 4 == 0) ? 1 : 0;
  hipLaunchKernelGGL(mfma_upproj_kernel, dim3(grid), dim3(NTHREADS), 0, stream,
                     static_cast<const uint16_t*>(a.c_kv), static_cast<const uint16_t*>(a.w), kn, vt,
                     a.B, a.H, a.Skv, a.s_vis, a.s_pad, n_jt, n_tiles, xcd_deal, v_rows ? 1 : 0);
  return hipGetLastError();
}
