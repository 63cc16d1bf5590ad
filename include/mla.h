/*
 * mla.h -- C ABI of libmla: the Multi-head Latent Attention (MLA) forward hot
 * path on AMD MI355X (gfx950).
 *
 * Pages this interface follows (Pith review pages):
 *   [LAGA]  "A Training-Memory Regression in MLA Sequence Parallelism: Why
 *            Megatron-Core Forbids Absorption, and LAGA -- a
 *            Communication-Efficient Fix"
 *   [TPLA]  "TPLA: Tensor Parallel Latent Attention for Efficient
 *            Disaggregated Prefill and Decode Inference"
 *   [Helix] "Helix Parallelism: Rethinking Sharding Strategies for
 *            Interactive Multi-Million-Token LLM Decoding"
 *
 * Two operations:
 *   mla_fwd_explicit     the explicit (training / LAGA per-rank) form: the
 *                        latent c_KV is up-projected through W_kv_b into
 *                        per-head K_nope and V, the decoupled RoPE band is
 *                        rotated, and causal softmax attention runs in head
 *                        dimension ([LAGA] "What carries the argument" and the
 *                        Fig. 2 caption, flows "Explicit (B1)" and "LAGA").
 *   mla_decode_absorbed  the absorbed decode form: each query is absorbed into
 *                        latent space, attends to the 576-wide latent cache
 *                        rows directly, the KV sequence is split in chunks
 *                        whose partial outputs are merged by log-sum-exp
 *                        rescaling, and the merged latent output is
 *                        up-projected to d_v ([LAGA] "What carries the
 *                        argument" and Fig. 2 "Absorbed (B2)"; [TPLA] "If this
 *                        is right" for the 576-wide cache row; [Helix] "What
 *                        carries the argument" for the LSE merge).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers unless a comment says otherwise.
 *     Tensors are dense row-major with the shapes given below, 16-byte
 *     aligned.  The caller owns and allocates every buffer, including the
 *     workspace; the library never allocates, frees or synchronises.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     runs asynchronously; the call returns once the kernels are enqueued.
 *   - Arguments are validated on the host before anything is enqueued.  On a
 *     validation failure the call returns a non-zero status and launches
 *     nothing.  A failed kernel launch returns MLA_ERR_HIP.  No C++ exception
 *     crosses this interface.
 *   - Weight layout (reading of the pages, which give only the 512 x (128*256)
 *     map): W_kv_b is the linear map from d_kv to H*(d_nope+d_v) stored one
 *     row per output feature, i.e. [H*(d_nope+d_v), d_kv].  Rows
 *     h*(d_nope+d_v) .. h*(d_nope+d_v)+d_nope-1 are head h's key part W_UK[h],
 *     the next d_v rows its value part W_UV[h].  This is the transpose of a
 *     d_kv-major [d_kv, H*(d_nope+d_v)] layout that the literal "512 x
 *     (128*256)" would also allow; it is chosen because the LAGA page ("What
 *     carries the argument") writes the absorbed query as the transpose of
 *     W_kv_b applied to q_nope, which under this layout is W_UK[h]^T q with
 *     no reshuffle, and because a head shard is then one contiguous block of
 *     rows.  A caller holding the d_kv-major form passes its transpose.
 *   - RoPE: rotate-half pairs (m, m + d_rope/2), theta_m = base^(-2m/d_rope),
 *     angle = absolute position * theta_m, angles formed in fp64.
 *   - LSE outputs are natural logs of the sum of exp of the scaled logits;
 *     a query that sees no key gets O = 0 and LSE = -inf.
 *   - Calls are reentrant.  Apart from the optional per-thread timing records
 *     (mla_timing_*), the library keeps no state between calls.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, non-positive size, bad enum   */
  MLA_ERR_UNSUPPORTED = 2,        /* valid request the library does not implement */
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,
  MLA_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed  */
} mla_status;

typedef enum { MLA_BF16 = 0, MLA_FP32 = 1 } mla_dtype;

typedef enum {
  MLA_ALGO_AUTO = 0,     /* MFMA kernels when the shape allows, else SIMT      */
  MLA_ALGO_SIMT = 1,     /* fp32 SIMT kernels, any supported shape or dtype     */
  MLA_ALGO_MFMA = 2,     /* MFMA kernels; MLA_ERR_UNSUPPORTED if not eligible   */
  MLA_ALGO_FUSED = 3     /* explicit forward only: the MFMA attention with the
                            latent up-projection fused in, so K_nope and V
                            never reach device memory (MFMA eligibility; the
                            other entry points return MLA_ERR_UNSUPPORTED)    */
} mla_algo;

/* ------------------------------------------------------------------------ */
/* Explicit form                                                             */
/* ------------------------------------------------------------------------ */
typedef struct {
  int32_t batch;        /* B >= 1                                              */
  int32_t s_q;          /* query rows per sequence, >= 0                       */
  int32_t s_kv;         /* latent rows per sequence, >= 0                      */
  int32_t n_heads;      /* H >= 1                                              */
  int32_t d_kv;         /* latent width (512 at DeepSeek-V2/V3 dims)           */
  int32_t d_nope;       /* per-head non-rotary q/k width (128)                 */
  int32_t d_rope;       /* decoupled RoPE band width, even (64)                */
  int32_t d_v;          /* per-head value width (128)                          */
  int64_t q_pos0;       /* absolute position of query row 0                    */
  int64_t kv_pos0;      /* absolute position of latent row 0                   */
  int32_t causal;       /* 1: key j visible to query i iff kv_pos0+j <= q_pos0+i */
  float softmax_scale;  /* multiplies the whole logit; usually 1/sqrt(d_nope+d_rope).
                           Finite and > 0, else MLA_ERR_INVALID_ARGUMENT        */
  float rope_base;      /* RoPE base, > 1 (10000)                              */
  mla_dtype in_dtype;   /* dtype of q_nope, q_pe, c_kv, k_pe, w_kv_b            */
  mla_dtype out_dtype;  /* dtype of out (lse is always fp32)                   */
  mla_algo algo;        /* kernel family.  MFMA and FUSED need bf16 inputs,
                           d_kv 512, d_nope 128, d_rope 64, d_v 128, and at
                           most 2^22 visible latent rows per sequence        */
} mla_explicit_desc;

/* Bytes of device workspace mla_fwd_explicit needs for `desc`; 0 if the
 * descriptor is invalid or unsupported. */
size_t mla_fwd_explicit_workspace_size(const mla_explicit_desc* desc);

/* Explicit-form forward ([LAGA] "What carries the argument", Fig. 2 B1/LAGA):
 *   K_nope[j,h] = W_UK[h] c_kv[j],  V[j,h] = W_UV[h] c_kv[j]
 *   logit[h,i,j] = softmax_scale * ( q_nope[i,h].K_nope[j,h]
 *                   + R(q_pe[i,h], q_pos0+i) . R(k_pe[j], kv_pos0+j) )
 *   out[i,h] = sum_j softmax_j(logit)[h,i,j] V[j,h] over visible keys.
 * k_pe is one band per latent row, shared by all heads.
 *
 *   q_nope [B, s_q, H, d_nope]     q_pe [B, s_q, H, d_rope]  (un-rotated)
 *   c_kv   [B, s_kv, d_kv]         k_pe [B, s_kv, d_rope]    (un-rotated)
 *   w_kv_b [H*(d_nope+d_v), d_kv]
 *   out    [B, s_q, H, d_v]        (out_dtype)
 *   lse    [B, H, s_q] fp32, or NULL when not wanted
 *   workspace: device buffer of at least mla_fwd_explicit_workspace_size()
 *   bytes; its contents on entry are ignored and on exit are unspecified
 *   (see mla_fwd_explicit_workspace_layout for the MFMA path's intermediates).
 * Latent rows no query can see (causal) are neither up-projected nor read.
 * With algo MLA_ALGO_FUSED the up-projection runs inside the attention
 * kernel, once per 256-query block that reads a key tile ([LAGA] "Where Pith
 * is reading between the lines": the fused kernel as future work; Fig. 3
 * caption: the repeated up-projection is its cost), and the workspace holds
 * only the RoPE tables and the rotated key band (2 * B * s_vis' * 64 bytes,
 * s_vis' the visible rows rounded up to 256) instead of the
 * B * H * s_vis' * 512 bytes of fp16 K_nope and V^T. */
mla_status mla_fwd_explicit(const mla_explicit_desc* desc,
                            const void* q_nope, const void* q_pe,
                            const void* c_kv, const void* k_pe,
                            const void* w_kv_b,
                            void* out, float* lse,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/* Where the MFMA path leaves its intermediates inside the workspace, for
 * testing the up-projection on its own.  Writes byte offsets (host memory,
 * offsets[4]):
 *   [0] K_nope  fp16 [B, H, s_kv_pad, d_nope]
 *   [1] V^T     fp16 [B, H, d_v, s_kv_pad]   (key index fastest)
 *   [2] R(k_pe) fp16 [B, s_kv_pad, d_rope]
 *   [3] s_kv_pad (an element count, not an offset)
 * Only rows below the last visible key are written.  Returns
 * MLA_ERR_UNSUPPORTED when `desc` would not take the MFMA path. */
mla_status mla_fwd_explicit_workspace_layout(const mla_explicit_desc* desc,
                                             size_t offsets[4]);

/* ------------------------------------------------------------------------ */
/* Absorbed split-KV decode                                                  */
/* ------------------------------------------------------------------------ */
typedef struct {
  int32_t batch;             /* B >= 1                                         */
  int32_t n_heads;           /* H >= 1                                         */
  int32_t d_kv, d_nope, d_rope, d_v;
  int32_t max_cache_len;     /* host-side upper bound of cache_len[b] (grid sizing) */
  int64_t cache_batch_stride;/* elements between sequences in kv_cache,
                                >= max_cache_len * (d_kv + d_rope)             */
  int32_t n_splits;          /* chunks per sequence, >= 1                       */
  float softmax_scale;       /* finite and > 0, else MLA_ERR_INVALID_ARGUMENT   */
  float rope_base;
  mla_dtype in_dtype;        /* dtype of q_nope, q_pe, kv_cache, w_kv_b         */
  mla_dtype out_dtype;
  mla_algo algo;
} mla_decode_desc;

size_t mla_decode_absorbed_workspace_size(const mla_decode_desc* desc);

/* One decode step in absorbed form ([LAGA] Fig. 2 B2; [Helix] "What carries
 * the argument"):
 *   p = cache_len[b] - 1 (the new token's position; its row is in the cache)
 *   q~[b,h] = [ W_UK[h]^T q_nope[b,h] ; R(q_pe[b,h], p) ]      (d_kv+d_rope)
 *   logit_t = softmax_scale * q~[b,h] . kv_cache[b,t]        for t < cache_len[b]
 *   chunk size c = ceil(cache_len[b] / n_splits), chunk k = [k c, min(L,(k+1)c));
 *   per chunk a partial latent output normalised within the chunk plus its
 *   LSE; the partials are merged by LSE rescaling into o_lat[b,h] (d_kv);
 *   out[b,h] = W_UV[h] o_lat[b,h].
 *
 *   q_nope   [B, H, d_nope]             q_pe [B, H, d_rope] (un-rotated)
 *   kv_cache [B, *, d_kv + d_rope] with row stride d_kv+d_rope and sequence
 *            stride cache_batch_stride; each row is the latent c_kv then the
 *            already-rotated k_pe band
 *   cache_len [B] int32, device: rows attended per sequence, 0..max_cache_len
 *   w_kv_b   [H*(d_nope+d_v), d_kv]
 *   out      [B, H, d_v] (out_dtype)    lse [B, H] fp32 or NULL
 * cache_len values outside [0, max_cache_len] are clamped to that range on
 * the device.  A sequence with cache_len 0 gets out = 0 and lse = -inf.
 * Limits: d_kv a multiple of 8 and at most 1024, n_splits at most 64
 * (MLA_ERR_UNSUPPORTED otherwise); w_kv_b and workspace 16-byte aligned. */
mla_status mla_decode_absorbed(const mla_decode_desc* desc,
                               const void* q_nope, const void* q_pe,
                               const void* kv_cache, const int32_t* cache_len,
                               const void* w_kv_b,
                               void* out, float* lse,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/* Offsets of the decode intermediates inside the workspace (host memory,
 * offsets[4]):
 *   [0] q~        [B, H, d_kv+d_rope]  (bf16 on the MFMA path, fp32 on SIMT)
 *   [1] lse_part  fp32 [B, n_splits, H]
 *   [2] o_part    [B, n_splits, H, d_kv]   (normalised within the chunk):
 *                 fp16 on the MFMA path, fp32 on SIMT.  Each row is a convex
 *                 combination of cache rows, so on the MFMA path the cache's
 *                 latent values must lie within fp16 range (|x| < 65504).
 *   [3] bytes per q~ and per o_part element (2 on the MFMA path, 4 on SIMT) */
mla_status mla_decode_absorbed_workspace_layout(const mla_decode_desc* desc,
                                                size_t offsets[4]);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the decode
 * step of mla_decode_absorbed with the same arguments and results, minus the
 * workspace.  Its intermediates (q~, chunk LSEs, partials: the bytes that
 * mla_decode_absorbed_workspace_size reports) go to a fixed device array of
 * MLA_DECODE_NOALLOC_MAX_BYTES bytes (64 MiB) inside the library, one per
 * GPU, held until the process ends.  The call allocates and frees
 * nothing.
 *   - A step whose intermediates exceed that size returns
 *     MLA_ERR_WORKSPACE_TOO_SMALL (mla_last_error gives both sizes) and
 *     launches nothing.  At 128 heads and 16 splits one sequence needs about
 *     2.3 MB, so up to 28 sequences fit.
 *   - Every call on one GPU uses that GPU's one array.  Calls whose execution
 *     overlaps on one GPU (other streams, other threads) race on it and give
 *     undefined results; serialize them.  The kernels write every
 *     intermediate before reading it, so nothing needs clearing between calls.
 *   - The array's device address is looked up on the first call made with a
 *     device current (a runtime symbol lookup, no allocation). */
#define MLA_DECODE_NOALLOC_MAX_BYTES ((size_t)64 << 20)

mla_status mla_decode_absorbed_noalloc(const mla_decode_desc* desc,
                                       const void* q_nope, const void* q_pe,
                                       const void* kv_cache, const int32_t* cache_len,
                                       const void* w_kv_b,
                                       void* out, float* lse,
                                       void* stream);

/* ------------------------------------------------------------------------ */
/* Absorbed-form forward of the explicit problem                            */
/* ------------------------------------------------------------------------ */

/* The forward of mla_fwd_explicit computed in absorbed form ("A
 * Training-Memory Regression in MLA Sequence Parallelism ... LAGA" (Pith
 * review), Fig. 2 "Absorbed (B2)"): each query is carried into latent space,
 * q~ = [W_UK[h]^T q_nope ; R(q_pe, q_pos0 + i)], attends to the latent rows
 * [c_kv[j] ; R(k_pe[j], kv_pos0 + j)] with c_kv[j] as the values, and the
 * merged latent accumulator is mapped to d_v by W_UV[h].  Mathematically the
 * same result as the explicit form (equal up to rounding).
 *
 * Arguments, layouts, ownership, validation and errors are those of
 * mla_fwd_explicit: out [B, s_q, H, d_v], lse [B, H, s_q] or NULL.  It runs
 * the decode path with every query row as its own sequence (one KV chunk
 * each, longest rows first), so its eligibility for the MFMA kernels is the
 * decode step's (bf16, d_kv 512, d_nope 128, d_rope 64, d_v 128, n_heads a
 * multiple of 16 up to 128); other shapes take the SIMT kernels.
 *
 * Workspace (mla_fwd_absorbed_workspace_size bytes, 16-byte aligned): the
 * decode intermediates for B * s_q sequences (q~, lse_part, o_part) followed
 * by the latent rows [B, s_kv, d_kv + d_rope] (in_dtype) and each row's
 * visible-key count and RoPE position. */
size_t mla_fwd_absorbed_workspace_size(const mla_explicit_desc* desc);

mla_status mla_fwd_absorbed(const mla_explicit_desc* desc,
                            const void* q_nope, const void* q_pe,
                            const void* c_kv, const void* k_pe,
                            const void* w_kv_b,
                            void* out, float* lse,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/* ------------------------------------------------------------------------ */
/* Backward of the explicit form                                             */
/* ------------------------------------------------------------------------ */

/* Gradients of sum(d_out * out) with respect to the five inputs of
 * mla_fwd_explicit, given the forward's output and LSE ("A Training-Memory
 * Regression in MLA Sequence Parallelism ... LAGA" (Pith review): the
 * training setting; "If this is right" states that LAGA's parameter gradients
 * equal the explicit form's).  With P the softmax of the forward's logits,
 *   dV = P^T d_out,  dP = d_out V^T,  dS = P (dP - rowsum(d_out * out)),
 *   dq_nope = s dS K_nope,  dK_nope = s dS^T q_nope  (s = softmax_scale),
 *   dq_pe = R^T(s dS R(k_pe)),  dk_pe = R^T(s sum_h dS^T R(q_pe)),
 *   dc_kv = sum_h dK_nope W_UK[h] + dV W_UV[h],  dW_UK[h] = dK_nope^T c_kv,
 *   dW_UV[h] = dV^T c_kv,
 * where R^T, the transpose of the RoPE rotation, rotates by the negative
 * angle.
 *
 *   desc, q_nope, q_pe, c_kv, k_pe, w_kv_b: as given to mla_fwd_explicit
 *   out   [B, s_q, H, d_v] (desc->out_dtype): the forward's output
 *   lse   [B, H, s_q] fp32: the forward's LSE
 *   d_out [B, s_q, H, d_v] (desc->out_dtype): gradient with respect to out
 *   dq_nope [B, s_q, H, d_nope], dq_pe [B, s_q, H, d_rope], dc_kv [B, s_kv, d_kv],
 *   dk_pe [B, s_kv, d_rope], dw_kv_b [H*(d_nope+d_v), d_kv]: fp32 outputs,
 *   fully written (latent rows no query sees get zero gradients).
 * Workspace: mla_bwd_explicit_workspace_size() bytes, 16-byte aligned.
 * MLA_ALGO_MFMA (the default where eligible) takes the forward's MFMA shapes
 * (bf16 inputs, d_kv 512, d_nope 128, d_rope 64, d_v 128) with batch * padded
 * key and query rows below 2^30; it runs the products on fp16 MFMA with fp32
 * accumulation and keeps fp16 copies of Q, d_out, K, V and of [dK_nope | dV]
 * in the workspace (all pointers 16-byte aligned).  The SIMT kernels (any
 * head geometry, fp32 arithmetic) keep the probabilities and their gradients
 * for every visible pair: at most 2^31 pairs per call (B * H * s_q * visible
 * keys), else MLA_ERR_UNSUPPORTED. */
size_t mla_bwd_explicit_workspace_size(const mla_explicit_desc* desc);

mla_status mla_bwd_explicit(const mla_explicit_desc* desc,
                            const void* q_nope, const void* q_pe,
                            const void* c_kv, const void* k_pe,
                            const void* w_kv_b,
                            const void* out, const float* lse, const void* d_out,
                            float* dq_nope, float* dq_pe, float* dc_kv, float* dk_pe,
                            float* dw_kv_b,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/* ------------------------------------------------------------------------ */
/* Per-kernel timing (profiling aid; not needed for computing)               */
/* ------------------------------------------------------------------------ */
/* Between mla_timing_begin() and mla_timing_end() on the calling thread, each
 * kernel (or fixed group of kernels) the entry points above enqueue is
 * bracketed by two HIP events recorded on the call's stream.  The launches
 * themselves are unchanged.  mla_timing_end() waits for the recorded events
 * and adds each launch's elapsed time to a per-name total, which
 * mla_timing_get() reports until mla_timing_reset().  Events are created by
 * the library the first time they are needed and reused afterwards.
 * Errors: MLA_ERR_HIP if an event call fails; MLA_ERR_INVALID_ARGUMENT for an
 * index out of range or a NULL output pointer. */
mla_status mla_timing_begin(void);
mla_status mla_timing_end(void);
mla_status mla_timing_reset(void);
int32_t mla_timing_count(void);
/* name: static string owned by the library; total_ms: summed duration;
 * launches: number of bracketed launches (host memory outputs). */
mla_status mla_timing_get(int32_t index, const char** name, double* total_ms, int64_t* launches);

/* Static description of a status code. */
const char* mla_status_string(mla_status status);

/* Text of the last HIP error seen by this thread (empty if none). */
const char* mla_last_error(void);

/* Build information: offload target and kernel families compiled in. */
const char* mla_build_info(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H */
