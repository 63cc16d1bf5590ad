// Latent up-projection on bf16 MFMA (fp32 accumulate, fp16 results).
//
// Explicit form of "A Training-Memory Regression in MLA Sequence Parallelism
// ... LAGA" (Pith review), "What carries the argument" and Fig. 2: per-head
// K_nope and V are the latent rows times the shared linear map W_kv_b.  The
// Fig. 3 caption notes that splitting this product into per-head-shard GEMMs
// made it slower at equal FLOPs, so it runs here as one GEMM over all heads:
//   C[j, n] = sum_c c_kv[b, j, c] * W[n, c],   j < s_vis, n < H * 256.
// Both operands are contiguous along c (W is stored one row per output
// feature), which is what the MFMA operand layout wants, so no transpose is
// needed on the way in.
//
// Outputs (fp16): Kn [B, H, s_pad, 128] and V^T [B, H, 128, s_pad] (key index
// fastest, the layout the attention kernel's P.V product reads).
//
// Tiling: 256 latent rows x 256 output columns (one head) per tile, 4 waves of
// 128 x 128 (one wave per SIMD, accumulators in the extended register file);
// waves 0-1 produce the K_nope half (operands swapped so each lane ends with 4
// consecutive features of one key), waves 2-3 the V half (each lane ends with
// 4 consecutive keys of one feature).  The reduction runs in 8 steps of 64
// staged through LDS with a register prefetch of the next step.  The grid is
// persistent: each workgroup walks tiles so that the stores of one tile drain
// while the next one computes, and tiles are dealt so that the 32 CUs of one
// XCD work on neighbouring tiles of the same heads (shared L2).
#include "common.h"
#include "kernels.h"

namespace {

constexpr int TJ = 256;          // latent rows per tile
constexpr int TN = 256;          // output columns per tile (= one head)
constexpr int TK = 64;           // reduction step
constexpr int DKV = 512;
constexpr int PITCH = TK + 8;    // bf16 elements per LDS row (bank spread)
constexpr int NTHREADS = 256;

__global__ void __launch_bounds__(NTHREADS)
mfma_upproj_kernel(const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ w,
                   uint16_t* __restrict__ kn, uint16_t* __restrict__ vt, int B, int H, int Skv,
                   int s_vis, int s_pad, int n_jt, int n_tiles) {
  // rows 0..TJ-1: latent rows (A); rows TJ..TJ+TN-1: W rows of the head (B)
  __shared__ __attribute__((aligned(16))) uint16_t Ls[(TJ + TN) * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int part = wave >> 1;          // 0: K_nope columns, 1: V columns
  const int jq = wave & 1;             // 128-row half of the tile
  const int l32 = lane & 31, hb = lane >> 5;
  // Every wave computes acc[i][k] = mfma(F_i, S_k) over 4 x 4 fragments.  For
  // K_nope waves F are W rows and S latent rows (D[n][j]); for V waves F are
  // latent rows and S W rows (D[j][n]).
  const int f_row0 = (part == 0) ? TJ : jq * 128;
  const int s_row0 = (part == 0) ? jq * 128 : TJ + 128;

  // tile dealing: consecutive tile ids go to the same XCD
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int per_xcd = G >> 3;          // grid is a multiple of 8
  const int local = blockIdx.x >> 3;

  for (int step = 0;; ++step) {
    int tile = step * G + xcd * per_xcd + local;
    if (tile >= n_tiles) break;
    const int jt = tile % n_jt;
    const int bh = tile / n_jt;
    const int h = bh % H, b = bh / H;
    const int j0 = jt * TJ;

    const uint16_t* abase = c_kv + ((int64_t)b * Skv) * DKV;
    const uint16_t* bbase = w + (int64_t)h * TN * DKV;

    f32x16_t acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[x][y][e] = 0.f;

    u32x4_t pa[8], pb[8];
    auto gload = [&](int k0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int q = tid + NTHREADS * i;      // 2048 chunks of 16 B per operand
        int row = q >> 3, c16 = q & 7;
        // rows past the last visible one repeat it: their results land in
        // the padding rows, which the attention kernel never lets through
        int j = min(j0 + row, s_vis - 1);
        pa[i] = *reinterpret_cast<const u32x4_t*>(abase + (int64_t)j * DKV + k0 + c16 * 8);
        pb[i] = *reinterpret_cast<const u32x4_t*>(bbase + (int64_t)row * DKV + k0 + c16 * 8);
      }
    };
    auto lstore = [&]() {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int q = tid + NTHREADS * i;
        int row = q >> 3, c16 = q & 7;
        *reinterpret_cast<u32x4_t*>(&Ls[row * PITCH + c16 * 8]) = pa[i];
        *reinterpret_cast<u32x4_t*>(&Ls[(TJ + row) * PITCH + c16 * 8]) = pb[i];
      }
    };

    gload(0);
    for (int ks = 0; ks < DKV / TK; ++ks) {
      __syncthreads();
      lstore();
      __syncthreads();
      if (ks + 1 < DKV / TK) gload((ks + 1) * TK);
#pragma unroll
      for (int kk = 0; kk < TK / 16; ++kk) {
        bf16x8_t ff[4], sf[4];
#pragma unroll
        for (int x = 0; x < 4; ++x)
          ff[x] = *reinterpret_cast<const bf16x8_t*>(&Ls[(f_row0 + x * 32 + l32) * PITCH + kk * 16 + hb * 8]);
#pragma unroll
        for (int y = 0; y < 4; ++y)
          sf[y] = *reinterpret_cast<const bf16x8_t*>(&Ls[(s_row0 + y * 32 + l32) * PITCH + kk * 16 + hb * 8]);
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int y = 0; y < 4; ++y)
            acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ff[x], sf[y], acc[x][y], 0, 0, 0);
      }
    }

    // epilogue: fp16 stores straight from the accumulators
    const int64_t head = (int64_t)b * H + h;
    if (part == 0) {
      // acc[x][y] holds D[n][j]: n = x*32 + 8g + 4hb + r, j = jq*128 + y*32 + l32
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        int j = j0 + jq * 128 + y * 32 + l32;
        uint16_t* dst = kn + (head * s_pad + j) * 128;
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            int n = x * 32 + 8 * g + 4 * hb;
            u32x2_t v2;
            v2[0] = pack_f16x2(acc[x][y][4 * g + 0], acc[x][y][4 * g + 1]);
            v2[1] = pack_f16x2(acc[x][y][4 * g + 2], acc[x][y][4 * g + 3]);
            *reinterpret_cast<u32x2_t*>(dst + n) = v2;
          }
      }
    } else {
      // acc[x][y] holds D[j][n]: j = jq*128 + x*32 + 8g + 4hb + r, n = y*32 + l32
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        int n = y * 32 + l32;
        uint16_t* dst = vt + (head * 128 + n) * s_pad + j0 + jq * 128;
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            int j = x * 32 + 8 * g + 4 * hb;
            u32x2_t v2;
            v2[0] = pack_f16x2(acc[x][y][4 * g + 0], acc[x][y][4 * g + 1]);
            v2[1] = pack_f16x2(acc[x][y][4 * g + 2], acc[x][y][4 * g + 3]);
            *reinterpret_cast<u32x2_t*>(dst + j) = v2;
          }
      }
    }
  }
}

// krot[b, j, :] = R(k_pe[b, j, :], kv_pos0 + j) in fp16 for j < s_pad
// (zeros for j >= s_vis).  One thread per rotation pair.
__global__ void krot_f16_kernel(const uint16_t* __restrict__ k_pe, const float2* __restrict__ ktab,
                                uint16_t* __restrict__ krot, int Skv, int s_vis, int s_pad) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int b = blockIdx.y;
  if (idx >= (int64_t)s_pad * 32) return;
  int j = (int)(idx >> 5), m = (int)(idx & 31);
  float ylo = 0.f, yhi = 0.f;
  if (j < s_vis) {
    int64_t src = ((int64_t)b * Skv + j) * 64;
    float lo = bf16_bits_to_float(k_pe[src + m]), hi = bf16_bits_to_float(k_pe[src + m + 32]);
    float2 cs = ktab[(int64_t)j * 32 + m];
    ylo = lo * cs.x - hi * cs.y;
    yhi = hi * cs.x + lo * cs.y;
  }
  int64_t dst = ((int64_t)b * s_pad + j) * 64;
  krot[dst + m] = float_to_f16_bits(ylo);
  krot[dst + m + 32] = float_to_f16_bits(yhi);
}

}  // namespace

hipError_t launch_mfma_upproj(const ExplicitArgs& a, uint16_t* kn, uint16_t* vt, hipStream_t stream) {
  if (a.s_vis == 0) return hipSuccess;
  int n_jt = a.s_pad / TJ;
  int n_tiles = a.B * a.H * n_jt;
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n_cu = 256;
  int grid = n_cu;                                   // one workgroup per CU
  if (grid > n_tiles) grid = n_tiles;
  grid = (grid + 7) & ~7;                            // multiple of 8 for the XCD dealing
  hipLaunchKernelGGL(mfma_upproj_kernel, dim3(grid), dim3(NTHREADS), 0, stream,
                     static_cast<const uint16_t*>(a.c_kv), static_cast<const uint16_t*>(a.w), kn, vt,
                     a.B, a.H, a.Skv, a.s_vis, a.s_pad, n_jt, n_tiles);
  return hipGetLastError();
}

hipError_t launch_krot_f16(const ExplicitArgs& a, const float2* ktab, uint16_t* krot,
                           hipStream_t stream) {
  if (a.s_pad == 0) return hipSuccess;
  int64_t n = (int64_t)a.s_pad * 32;
  dim3 grid((unsigned)((n + 255) / 256), a.B);
  hipLaunchKernelGGL(krot_f16_kernel, grid, dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a.k_pe), ktab, krot, a.Skv, a.s_vis, a.s_pad);
  return hipGetLastError();
}
