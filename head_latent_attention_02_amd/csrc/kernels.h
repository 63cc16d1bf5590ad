// Internal launch interface between the C-ABI layer (mla_api.hip) and the
// kernel translation units.  Each launcher enqueues its kernel(s) on `stream`
// and returns the launch status; shapes have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

struct ExplicitArgs {
  int B, Sq, Skv, H, dkv, dn, dr, dv;
  int64_t q_pos0, kv_pos0;
  int causal;
  float scale, rope_base;
  mla_dtype in_dt, out_dt;
  int s_vis;      // latent rows visible to at least one query
  int s_pad;      // s_vis rounded up to the MFMA key tile
  const void *q_nope, *q_pe, *c_kv, *k_pe, *w;
  void* out;
  float* lse;
};

// Explicit-form backward: the forward's arguments plus its saved output and
// LSE, the output gradient and the five fp32 input gradients.
struct BackwardArgs {
  ExplicitArgs f;             // f.out / f.lse unused; f.out_dt is the dtype of out and d_out
  const void* out;            // [B, Sq, H, dv]
  const float* lse;           // [B, H, Sq]
  const void* d_out;          // [B, Sq, H, dv]
  float *dq_nope, *dq_pe, *dc_kv, *dk_pe, *dw;   // gradients, same shapes as the inputs
};

struct DecodeArgs {
  int B, H, dkv, dn, dr, dv;
  int max_len;
  int64_t cache_stride;
  int n_splits;
  float scale, rope_base;
  mla_dtype in_dt, out_dt;
  const void *q_nope, *q_pe, *cache, *w;
  const int32_t* cache_len;
  void* out;
  float* lse;
  // Absorbed prefill runs every query row as its own sequence (defaults keep
  // the decode step's meaning):
  int seq_per_cache = 1;            // consecutive sequences sharing one cache entry
  const int64_t* q_pos = nullptr;   // RoPE position per sequence (nullptr: cache_len - 1)
  int reverse = 0;                  // split-KV takes sequences last to first
  int lse_seq = 0;                  // > 0: lse is [B / lse_seq, H, lse_seq], else [B, H]
};

// Absorbed prefill: latent cache rows cache[b][j] = c_kv[b][j] || R(k_pe[b][j],
// kv_pos0 + j) (in_dt), and per query row i of batch entry b (sequence
// b * Sq + i) its visible key count and RoPE position.
hipError_t launch_latent_cache(const ExplicitArgs& a, void* cache, int32_t* cache_len, int64_t* q_pos,
                               hipStream_t stream);

// RoPE cos/sin table: table[p*(dr/2)+m] = (cos, sin)((pos0+p) * base^(-2m/dr)),
// angles formed in fp64.
hipError_t launch_rope_table(float2* table, int64_t pos0, int n, int dr, float base,
                             hipStream_t stream);

// ---- SIMT (fp32 arithmetic) explicit path --------------------------------
// Workspace: Kn fp32 [B,H,s_vis,dn], V fp32 [B,H,s_vis,dv], krot fp32
// [B,s_vis,dr], q table [Sq,dr/2], k table [s_vis,dr/2].
hipError_t launch_simt_explicit(const ExplicitArgs& a, float* kn, float* v, float* krot,
                                const float2* qtab, const float2* ktab, hipStream_t stream);

// ---- MFMA explicit path ---------------------------------------------------
// kn fp16 [B,H,s_pad,128], vt fp16 [B,H,128,s_pad] (or, with v_rows, V in
// rows [B,H,s_pad,128]), krot fp16 [B,s_pad,64].
hipError_t launch_mfma_upproj(const ExplicitArgs& a, uint16_t* kn, uint16_t* vt,
                              hipStream_t stream, bool v_rows = false);
// The query RoPE table qtab [S_q][d_r/2] and the rotated key band krot in one
// launch (the key table ktab [s_vis][d_r/2] as well when ktab is not null).
hipError_t launch_rope_band(const ExplicitArgs& a, float2* qtab, float2* ktab, uint16_t* krot,
                            hipStream_t stream);
hipError_t launch_mfma_attention(const ExplicitArgs& a, const uint16_t* kn, const uint16_t* vt,
                                 const uint16_t* krot, const float2* qtab, hipStream_t stream);
// Attention with the up-projection fused in: reads c_kv and w directly.
hipError_t launch_fused_attention(const ExplicitArgs& a, const uint16_t* krot, const float2* qtab,
                                  hipStream_t stream);

// ---- explicit-form backward ----------------------------------------------
// SIMT path.  Workspace (fp32): Kn [B,H,s_vis,dn], V [B,H,s_vis,dv], krot
// [B,s_vis,dr], qrot [B,Sq,H,dr], P and dS [B,H,Sq,s_vis], dKn [B,H,s_vis,dn],
// dV [B,H,s_vis,dv]; q / k rope tables.
struct SimtBwdWorkspace {
  float *kn, *v, *krot, *qrot, *p, *ds, *dkn, *dv;
  const float2 *qtab, *ktab;
};
hipError_t launch_simt_backward(const BackwardArgs& a, const SimtBwdWorkspace& w, hipStream_t stream);

// MFMA path (bf16 inputs, d_kv 512, d_nope 128, d_rope 64, d_v 128).  fp16
// workspace tensors: the up-projection's kn [bh][s_pad][128] and vrow
// [bh][s_pad][128] (V in rows), krot [b][s_pad][64]; Q = [q_nope ; R(q_pe)] as qf [bh][sq_pad][192] and
// qft [bh][192][sq_pad]; dO as dof [bh][sq_pad][128] and doft
// [bh][128][sq_pad]; knt [bh][128][s_pad]; krt
// [b][64][s_pad]; dkv [b][s_pad][H*256] and dkvt [H*256][b*s_pad] ([dK_nope |
// dV] per head, scaled); wt [512][H*256]; ct [512][b*s_pad].  fp32: dvec
// [bh][sq_pad] (dO . out), dkr [bh][s_pad][64].  sq_pad = s_q rounded up to 128.
struct MfmaBwdWorkspace {
  float2 *qtab, *ktab;
  uint16_t *kn, *krot, *qf, *qft, *dof, *doft, *vrow, *knt, *krt, *dkv, *dkvt, *wt, *ct;
  float *dvec, *dkr;
  float* lsdt;        // per 32-query tile: LSE then D, 32 each, in the permuted row order
  int sq_pad;
};
// Bytes of workspace (base == nullptr) or the carving of `base` into `w`.
size_t mfma_backward_workspace(const ExplicitArgs& f, MfmaBwdWorkspace* w, char* base);
hipError_t launch_bwd_prep(const BackwardArgs& a, const MfmaBwdWorkspace& w, hipStream_t stream);
hipError_t launch_bwd_kv(const BackwardArgs& a, const MfmaBwdWorkspace& w, hipStream_t stream);
hipError_t launch_bwd_dq(const BackwardArgs& a, const MfmaBwdWorkspace& w, hipStream_t stream);
hipError_t launch_bwd_dkpe(const BackwardArgs& a, const MfmaBwdWorkspace& w, hipStream_t stream);
hipError_t launch_bwd_gemms(const BackwardArgs& a, const MfmaBwdWorkspace& w, hipStream_t stream);

// ---- decode ---------------------------------------------------------------
// q~ is fp32 [B,H,dkv+dr] (SIMT) or bf16 (MFMA); lse_part fp32 [B,ns,H];
// o_part [B,ns,H,dkv] fp32 (SIMT) or fp16 (MFMA).
hipError_t launch_simt_absorb(const DecodeArgs& a, float* qt, hipStream_t stream);
hipError_t launch_simt_splitkv(const DecodeArgs& a, const float* qt, float* lse_part,
                               float* o_part, hipStream_t stream);
hipError_t launch_absorb_bf16(const DecodeArgs& a, uint16_t* qt, hipStream_t stream);
hipError_t launch_mfma_splitkv(const DecodeArgs& a, const uint16_t* qt, float* lse_part,
                               uint16_t* o_part, hipStream_t stream);
hipError_t launch_combine(const DecodeArgs& a, const float* lse_part, const void* o_part, bool half_parts,
                          hipStream_t stream);
