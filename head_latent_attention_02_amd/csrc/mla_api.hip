// C ABI of libmla: argument validation, workspace carving and the launch
// sequence of each entry point.  Every check runs on the host before the first
// launch, so an invalid call enqueues nothing.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

constexpr size_t kAlign = 256;
constexpr int kUpTile = 256;        // latent-row tile of the MFMA up-projection

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_dtype(mla_dtype d) { return d == MLA_BF16 || d == MLA_FP32; }
bool valid_algo(mla_algo a) {
  return a == MLA_ALGO_AUTO || a == MLA_ALGO_SIMT || a == MLA_ALGO_MFMA || a == MLA_ALGO_FUSED;
}

mla_status hip_fail(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return MLA_ERR_HIP;
}

// ---------------------------------------------------------------- timing --
struct TimingTotal {
  const char* name;
  double ms;
  int64_t launches;
};
struct PendingLaunch {
  const char* name;
  hipEvent_t start, stop;
};
struct TimingState {
  bool active = false;
  std::vector<hipEvent_t> pool;
  std::vector<PendingLaunch> pending;
  std::vector<TimingTotal> totals;
};
thread_local TimingState g_timing;

hipEvent_t timing_event() {
  if (!g_timing.pool.empty()) {
    hipEvent_t e = g_timing.pool.back();
    g_timing.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one launcher call with events when timing is active.
class TimedLaunch {
 public:
  TimedLaunch(const char* name, hipStream_t s) : name_(name), stream_(s) {
    if (!g_timing.active) return;
    start_ = timing_event();
    if (start_ != nullptr) (void)hipEventRecord(start_, stream_);
  }
  ~TimedLaunch() {
    if (!g_timing.active || start_ == nullptr) return;
    hipEvent_t stop = timing_event();
    if (stop == nullptr) return;
    (void)hipEventRecord(stop, stream_);
    g_timing.pending.push_back({name_, start_, stop});
  }

 private:
  const char* name_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr;
};

// ---------------------------------------------------------------- explicit --
struct ExplicitPlan {
  bool mfma = false;
  bool fused = false;     // MFMA attention with the up-projection fused in
  int s_vis = 0, s_pad = 0;
  size_t off_qtab = 0, off_ktab = 0, off_kn = 0, off_v = 0, off_krot = 0, total = 0;
};

bool explicit_shape_ok(const mla_explicit_desc* d) {
  if (d == nullptr) return false;
  if (d->batch < 1 || d->n_heads < 1 || d->s_q < 0 || d->s_kv < 0) return false;
  if (d->d_kv < 1 || d->d_nope < 1 || d->d_v < 1 || d->d_rope < 2 || (d->d_rope & 1)) return false;
  if (d->causal != 0 && d->causal != 1) return false;
  if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype) || !valid_algo(d->algo)) return false;
  // the MFMA kernels take the row max of raw scores, which equals the max of
  // the scaled logits only for a positive scale
  if (!std::isfinite(d->softmax_scale) || !(d->softmax_scale > 0.f)) return false;
  if (!std::isfinite(d->rope_base) || !(d->rope_base > 0.f)) return false;
  // element counts must stay addressable with 64-bit offsets and 32-bit grids
  const int64_t B = d->batch, H = d->n_heads;
  if (B * d->s_q * H > (int64_t)1 << 40 || B * d->s_kv > (int64_t)1 << 36) return false;
  if (H * (int64_t)(d->d_nope + d->d_v) > (int64_t)1 << 24) return false;
  return true;
}

constexpr int kMaxMfmaKeys = 1 << 22;    // visible keys (rounded up) on the MFMA path

bool explicit_mfma_eligible(const mla_explicit_desc* d) {
  return d->in_dtype == MLA_BF16 && d->d_kv == 512 && d->d_nope == 128 && d->d_rope == 64 &&
         d->d_v == 128;
}

bool explicit_simt_supported(const mla_explicit_desc* d) {
  return d->d_nope + d->d_rope + d->d_v <= 448 && d->d_rope <= 256;
}

// Returns MLA_OK and fills `plan`, or the status that the call must return.
mla_status make_explicit_plan(const mla_explicit_desc* d, ExplicitPlan* plan) {
  if (!explicit_shape_ok(d)) return MLA_ERR_INVALID_ARGUMENT;
  ExplicitPlan p;
  if (d->s_q == 0) {
    p.s_vis = 0;
  } else if (d->causal) {
    int64_t lim = d->q_pos0 + (int64_t)d->s_q - 1 - d->kv_pos0 + 1;
    p.s_vis = (int)std::max<int64_t>(0, std::min<int64_t>(lim, d->s_kv));
  } else {
    p.s_vis = d->s_kv;
  }
  p.s_pad = (p.s_vis + kUpTile - 1) / kUpTile * kUpTile;
  // the MFMA attention addresses one head's K_nope / V^T rows with 32-bit
  // byte offsets: s_pad * 256 bytes must stay below 2^31
  const bool mfma_ok = explicit_mfma_eligible(d) && p.s_pad <= kMaxMfmaKeys;
  bool mfma;
  if (d->algo == MLA_ALGO_MFMA || d->algo == MLA_ALGO_FUSED) {
    if (!mfma_ok) return MLA_ERR_UNSUPPORTED;
    mfma = true;
  } else if (d->algo == MLA_ALGO_SIMT) {
    mfma = false;
  } else {
    mfma = mfma_ok;
  }
  if (!mfma && !explicit_simt_supported(d)) return MLA_ERR_UNSUPPORTED;
  const bool fused = d->algo == MLA_ALGO_FUSED;
  p.mfma = mfma && !fused;
  p.fused = fused;
  const size_t B = d->batch, H = d->n_heads, half = d->d_rope / 2;
  size_t off = 0;
  p.off_qtab = off; off = align_up(off + sizeof(float2) * (size_t)d->s_q * half);
  p.off_ktab = off; off = align_up(off + sizeof(float2) * (size_t)p.s_vis * half);
  if (fused) {
    p.off_krot = off; off = align_up(off + 2 * B * (size_t)p.s_pad * 64);
  } else if (mfma) {
    p.off_kn = off;   off = align_up(off + 2 * B * H * (size_t)p.s_pad * 128);
    p.off_v = off;    off = align_up(off + 2 * B * H * 128 * (size_t)p.s_pad);
    p.off_krot = off; off = align_up(off + 2 * B * (size_t)p.s_pad * 64);
  } else {
    p.off_kn = off;   off = align_up(off + 4 * B * H * (size_t)p.s_vis * d->d_nope);
    p.off_v = off;    off = align_up(off + 4 * B * H * (size_t)p.s_vis * d->d_v);
    p.off_krot = off; off = align_up(off + 4 * B * (size_t)p.s_vis * d->d_rope);
  }
  p.total = off;
  *plan = p;
  return MLA_OK;
}

// ------------------------------------------------------------------ decode --
struct DecodePlan {
  bool mfma = false;
  size_t off_qt = 0, off_lse = 0, off_opart = 0, qt_elem = 0, total = 0;
};

bool decode_shape_ok(const mla_decode_desc* d) {
  if (d == nullptr) return false;
  if (d->batch < 1 || d->n_heads < 1 || d->max_cache_len < 0 || d->n_splits < 1) return false;
  if (d->d_kv < 1 || d->d_nope < 1 || d->d_v < 1 || d->d_rope < 2 || (d->d_rope & 1)) return false;
  if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype) || !valid_algo(d->algo)) return false;
  // the MFMA kernels take the row max of raw scores, which equals the max of
  // the scaled logits only for a positive scale
  if (!std::isfinite(d->softmax_scale) || !(d->softmax_scale > 0.f)) return false;
  if (!std::isfinite(d->rope_base) || !(d->rope_base > 0.f)) return false;
  const int64_t row = (int64_t)d->d_kv + d->d_rope;
  if (d->cache_batch_stride < (int64_t)d->max_cache_len * row) return false;
  if ((int64_t)d->batch * d->n_heads > (int64_t)1 << 30) return false;
  return true;
}

bool decode_mfma_eligible(const mla_decode_desc* d) {
  // tile loads use 32-bit byte offsets within one sequence's rows
  return d->in_dtype == MLA_BF16 && d->d_kv == 512 && d->d_nope == 128 && d->d_rope == 64 &&
         d->d_v == 128 && d->n_heads % 16 == 0 && d->n_heads <= 128 && d->cache_batch_stride % 8 == 0 &&
         (int64_t)d->max_cache_len * (d->d_kv + d->d_rope) * 2 < ((int64_t)1 << 31);
}

bool decode_simt_supported(const mla_decode_desc* d) { return d->d_kv <= 1024 && d->d_rope <= 256; }

mla_status make_decode_plan(const mla_decode_desc* d, DecodePlan* plan) {
  if (!decode_shape_ok(d)) return MLA_ERR_INVALID_ARGUMENT;
  if (d->n_splits > 64 || d->algo == MLA_ALGO_FUSED) return MLA_ERR_UNSUPPORTED;
  // the combine keeps 8 merged rows in LDS and reads rows 8 elements at a time
  if (d->d_kv > 1024 || d->d_kv % 8 != 0) return MLA_ERR_UNSUPPORTED;
  bool mfma;
  if (d->algo == MLA_ALGO_MFMA) {
    if (!decode_mfma_eligible(d)) return MLA_ERR_UNSUPPORTED;
    mfma = true;
  } else if (d->algo == MLA_ALGO_SIMT) {
    mfma = false;
  } else {
    mfma = decode_mfma_eligible(d);
  }
  if (!mfma && !decode_simt_supported(d)) return MLA_ERR_UNSUPPORTED;
  DecodePlan p;
  p.mfma = mfma;
  const size_t B = d->batch, H = d->n_heads, ns = d->n_splits, dlat = d->d_kv + d->d_rope;
  p.qt_elem = mfma ? 2 : 4;
  size_t off = 0;
  p.off_qt = off;    off = align_up(off + p.qt_elem * B * H * dlat);
  p.off_lse = off;   off = align_up(off + 4 * B * ns * H);
  // the MFMA path keeps its partials in fp16 (their values lie in the cache's range)
  p.off_opart = off; off = align_up(off + p.qt_elem * B * ns * H * (size_t)d->d_kv);
  p.total = off;
  *plan = p;
  return MLA_OK;
}


void fill_decode_args(const mla_decode_desc* desc, const void* q_nope, const void* q_pe, const void* kv_cache,
                      const int32_t* cache_len, const void* w_kv_b, void* out, float* lse, DecodeArgs* pa) {
  DecodeArgs& a = *pa;
  a.B = desc->batch; a.H = desc->n_heads; a.dkv = desc->d_kv; a.dn = desc->d_nope;
  a.dr = desc->d_rope; a.dv = desc->d_v; a.max_len = desc->max_cache_len;
  a.cache_stride = desc->cache_batch_stride; a.n_splits = desc->n_splits;
  a.scale = desc->softmax_scale; a.rope_base = desc->rope_base;
  a.in_dt = desc->in_dtype; a.out_dt = desc->out_dtype;
  a.q_nope = q_nope; a.q_pe = q_pe; a.cache = kv_cache; a.w = w_kv_b; a.cache_len = cache_len;
  a.out = out; a.lse = lse;
}

// absorb, split-KV and combine for a validated plan
mla_status run_decode(const DecodePlan& p, const DecodeArgs& a, char* ws, hipStream_t s) {
  float* lse_part = reinterpret_cast<float*>(ws + p.off_lse);
  void* o_part = ws + p.off_opart;
  hipError_t e;
  if (p.mfma) {
    uint16_t* qt = reinterpret_cast<uint16_t*>(ws + p.off_qt);
    {
      TimedLaunch t("absorb", s);
      e = launch_absorb_bf16(a, qt, s);
    }
    if (e != hipSuccess) return hip_fail(e, "query absorption");
    {
      TimedLaunch t("mfma_split_kv", s);
      e = launch_mfma_splitkv(a, qt, lse_part, static_cast<uint16_t*>(o_part), s);
    }
    if (e != hipSuccess) return hip_fail(e, "mfma split-KV attention");
  } else {
    float* qt = reinterpret_cast<float*>(ws + p.off_qt);
    {
      TimedLaunch t("simt_absorb", s);
      e = launch_simt_absorb(a, qt, s);
    }
    if (e != hipSuccess) return hip_fail(e, "query absorption");
    {
      TimedLaunch t("simt_split_kv", s);
      e = launch_simt_splitkv(a, qt, lse_part, static_cast<float*>(o_part), s);
    }
    if (e != hipSuccess) return hip_fail(e, "simt split-KV attention");
  }
  {
    TimedLaunch t("lse_combine", s);
    e = launch_combine(a, lse_part, o_part, p.mfma, s);
  }
  if (e != hipSuccess) return hip_fail(e, "LSE combine");
  return MLA_OK;
}

// ----------------------------------------------------- explicit backward --
struct BackwardPlan {
  ExplicitPlan fwd;                 // the forward's plan (s_vis, tables)
  bool mfma = false;
  size_t off_qtab = 0, off_ktab = 0, off_kn = 0, off_v = 0, off_krot = 0, off_qrot = 0, off_p = 0,
         off_ds = 0, off_dkn = 0, off_dv = 0, total = 0;
};

// The SIMT backward keeps P and dS for every visible pair; its workspace is
// bounded here so that a call cannot ask for an absurd allocation.
constexpr size_t kMaxSimtBwdPairs = size_t(1) << 31;

ExplicitArgs explicit_args(const mla_explicit_desc* desc, const ExplicitPlan& p) {
  ExplicitArgs f{};
  f.B = desc->batch; f.Sq = desc->s_q; f.Skv = desc->s_kv; f.H = desc->n_heads;
  f.dkv = desc->d_kv; f.dn = desc->d_nope; f.dr = desc->d_rope; f.dv = desc->d_v;
  f.q_pos0 = desc->q_pos0; f.kv_pos0 = desc->kv_pos0; f.causal = desc->causal;
  f.scale = desc->softmax_scale; f.rope_base = desc->rope_base;
  f.in_dt = desc->in_dtype; f.out_dt = desc->out_dtype;
  f.s_vis = p.s_vis; f.s_pad = p.s_pad;
  return f;
}

mla_status make_backward_plan(const mla_explicit_desc* d, BackwardPlan* plan) {
  if (d != nullptr && d->algo == MLA_ALGO_FUSED) {
    if (!explicit_shape_ok(d)) return MLA_ERR_INVALID_ARGUMENT;
    return MLA_ERR_UNSUPPORTED;
  }
  BackwardPlan p;
  mla_explicit_desc fd = *d;
  // the MFMA backward takes the forward's MFMA shapes, with its GEMM
  // dimensions (B * s_pad keys, H * 256 weight rows) within 32-bit ints
  mla_explicit_desc md = *d;
  md.algo = MLA_ALGO_MFMA;
  ExplicitPlan mp;
  const bool mfma_ok = d->algo != MLA_ALGO_SIMT && make_explicit_plan(&md, &mp) == MLA_OK && mp.mfma &&
                       (int64_t)d->batch * mp.s_pad < ((int64_t)1 << 30) &&
                       (int64_t)d->batch * ((d->s_q + 127) / 128 * 128) < ((int64_t)1 << 30);
  if (d->algo == MLA_ALGO_MFMA && !mfma_ok) {
    if (!explicit_shape_ok(d)) return MLA_ERR_INVALID_ARGUMENT;
    return MLA_ERR_UNSUPPORTED;
  }
  if (mfma_ok) {
    p.fwd = mp;
    p.mfma = true;
    p.total = mfma_backward_workspace(explicit_args(d, mp), nullptr, nullptr);
    *plan = p;
    return MLA_OK;
  }
  fd.algo = MLA_ALGO_SIMT;
  mla_status st = make_explicit_plan(&fd, &p.fwd);
  if (st != MLA_OK) return st;
  const size_t B = d->batch, H = d->n_heads, Sq = d->s_q, sv = p.fwd.s_vis, half = d->d_rope / 2;
  if (B * H * Sq * sv > kMaxSimtBwdPairs) return MLA_ERR_UNSUPPORTED;
  size_t off = 0;
  p.off_qtab = off; off = align_up(off + sizeof(float2) * Sq * half);
  p.off_ktab = off; off = align_up(off + sizeof(float2) * sv * half);
  p.off_kn = off;   off = align_up(off + 4 * B * H * sv * d->d_nope);
  p.off_v = off;    off = align_up(off + 4 * B * H * sv * d->d_v);
  p.off_krot = off; off = align_up(off + 4 * B * sv * d->d_rope);
  p.off_qrot = off; off = align_up(off + 4 * B * Sq * H * d->d_rope);
  p.off_p = off;    off = align_up(off + 4 * B * H * Sq * sv);
  p.off_ds = off;   off = align_up(off + 4 * B * H * Sq * sv);
  p.off_dkn = off;  off = align_up(off + 4 * B * H * sv * d->d_nope);
  p.off_dv = off;   off = align_up(off + 4 * B * H * sv * d->d_v);
  p.total = off;
  *plan = p;
  return MLA_OK;
}

// ------------------------------------------------------- absorbed prefill --
// The decode problem that an absorbed-form forward maps to: one sequence per
// query row (B * Sq of them), one chunk each, the batch entry's latent rows
// as every one of its rows' cache.
struct AbsorbedPlan {
  mla_decode_desc dd{};
  DecodePlan dec;
  size_t off_cache = 0, off_len = 0, off_pos = 0, total = 0;
};

mla_status make_absorbed_plan(const mla_explicit_desc* d, AbsorbedPlan* plan) {
  if (!explicit_shape_ok(d)) return MLA_ERR_INVALID_ARGUMENT;
  AbsorbedPlan p;
  const int64_t rows = (int64_t)d->batch * d->s_q;
  if (rows > (int64_t)1 << 30 || (int64_t)d->s_kv > ((int64_t)1 << 31) - 1) return MLA_ERR_UNSUPPORTED;
  if (rows == 0) {
    *plan = p;
    return MLA_OK;
  }
  const int64_t dlat = (int64_t)d->d_kv + d->d_rope;
  p.dd.batch = (int32_t)rows;
  p.dd.n_heads = d->n_heads; p.dd.d_kv = d->d_kv; p.dd.d_nope = d->d_nope; p.dd.d_rope = d->d_rope;
  p.dd.d_v = d->d_v; p.dd.max_cache_len = d->s_kv; p.dd.cache_batch_stride = (int64_t)d->s_kv * dlat;
  p.dd.n_splits = 1;
  p.dd.softmax_scale = d->softmax_scale; p.dd.rope_base = d->rope_base;
  p.dd.in_dtype = d->in_dtype; p.dd.out_dtype = d->out_dtype; p.dd.algo = d->algo;
  mla_status st = make_decode_plan(&p.dd, &p.dec);
  if (st != MLA_OK) return st;
  const size_t esz = d->in_dtype == MLA_BF16 ? 2 : 4;
  size_t off = p.dec.total;
  p.off_cache = off; off = align_up(off + esz * (size_t)d->batch * d->s_kv * dlat);
  p.off_len = off;   off = align_up(off + 4 * (size_t)rows);
  p.off_pos = off;   off = align_up(off + 8 * (size_t)rows);
  p.total = off;
  *plan = p;
  return MLA_OK;
}
// ------------------------------------------------- allocation-free decode --
// Fixed scratch for mla_decode_absorbed_noalloc: the decode intermediates (q~,
// chunk LSEs and partials) live here instead of in a caller workspace.  Each
// GPU the library runs on holds its own copy for the life of the process.  In
// host code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, once per device, and only that address is ever handed
// to kernels.
constexpr size_t kScratchBytes = MLA_DECODE_NOALLOC_MAX_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up on the
// first call made on that device.
mla_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    g_last_error = "device index beyond the scratch table";
    return MLA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) {
      g_last_error = "hipGetSymbolAddress(scratch) returned a null address";
      return MLA_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}
}  // namespace

extern "C" {

size_t mla_fwd_explicit_workspace_size(const mla_explicit_desc* desc) {
  ExplicitPlan p;
  if (make_explicit_plan(desc, &p) != MLA_OK) return 0;
  return p.total;
}

mla_status mla_fwd_explicit_workspace_layout(const mla_explicit_desc* desc, size_t offsets[4]) {
  if (offsets == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  ExplicitPlan p;
  mla_status st = make_explicit_plan(desc, &p);
  if (st != MLA_OK) return st;
  if (!p.mfma) return MLA_ERR_UNSUPPORTED;
  offsets[0] = p.off_kn;
  offsets[1] = p.off_v;
  offsets[2] = p.off_krot;
  offsets[3] = (size_t)p.s_pad;
  return MLA_OK;
}

mla_status mla_fwd_explicit(const mla_explicit_desc* desc, const void* q_nope, const void* q_pe,
                            const void* c_kv, const void* k_pe, const void* w_kv_b, void* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  ExplicitPlan p;
  mla_status st = make_explicit_plan(desc, &p);
  if (st != MLA_OK) return st;
  const bool has_q = desc->s_q > 0, has_kv = desc->s_kv > 0;
  if (w_kv_b == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  if (has_q && (q_nope == nullptr || q_pe == nullptr || out == nullptr)) return MLA_ERR_INVALID_ARGUMENT;
  if (has_kv && (c_kv == nullptr || k_pe == nullptr)) return MLA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < p.total) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (p.total > 0 && workspace == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  if (p.mfma || p.fused) {
    const void* ptrs[] = {q_nope, q_pe, c_kv, k_pe, w_kv_b, out, workspace};
    for (const void* q : ptrs)
      if (q != nullptr && !aligned16(q)) return MLA_ERR_INVALID_ARGUMENT;
  }
  if (!has_q) return MLA_OK;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  ExplicitArgs a;
  a.B = desc->batch; a.Sq = desc->s_q; a.Skv = desc->s_kv; a.H = desc->n_heads;
  a.dkv = desc->d_kv; a.dn = desc->d_nope; a.dr = desc->d_rope; a.dv = desc->d_v;
  a.q_pos0 = desc->q_pos0; a.kv_pos0 = desc->kv_pos0; a.causal = desc->causal;
  a.scale = desc->softmax_scale; a.rope_base = desc->rope_base;
  a.in_dt = desc->in_dtype; a.out_dt = desc->out_dtype;
  a.s_vis = p.s_vis; a.s_pad = p.s_pad;
  a.q_nope = q_nope; a.q_pe = q_pe; a.c_kv = c_kv; a.k_pe = k_pe; a.w = w_kv_b;
  a.out = out; a.lse = lse;

  float2* qtab = reinterpret_cast<float2*>(ws + p.off_qtab);
  float2* ktab = reinterpret_cast<float2*>(ws + p.off_ktab);
  hipError_t e;
  if (p.fused || p.mfma) {
    // the query table and the rotated key band (the key table is not needed)
    TimedLaunch t("rope_band", s);
    e = launch_rope_band(a, qtab, nullptr, reinterpret_cast<uint16_t*>(ws + p.off_krot), s);
  } else {
    TimedLaunch t("rope_tables", s);
    e = launch_rope_table(qtab, a.q_pos0, a.Sq, a.dr, a.rope_base, s);
    if (e == hipSuccess) e = launch_rope_table(ktab, a.kv_pos0, a.s_vis, a.dr, a.rope_base, s);
  }
  if (e != hipSuccess) return hip_fail(e, "rope tables");
  if (p.fused) {
    uint16_t* kr = reinterpret_cast<uint16_t*>(ws + p.off_krot);
    {
      TimedLaunch t("fused_attention", s);
      e = launch_fused_attention(a, kr, qtab, s);
    }
    if (e != hipSuccess) return hip_fail(e, "fused attention");
  } else if (p.mfma) {
    uint16_t* kn = reinterpret_cast<uint16_t*>(ws + p.off_kn);
    uint16_t* vt = reinterpret_cast<uint16_t*>(ws + p.off_v);
    uint16_t* kr = reinterpret_cast<uint16_t*>(ws + p.off_krot);
    {
      TimedLaunch t("mfma_up_projection", s);
      e = launch_mfma_upproj(a, kn, vt, s);
    }
    if (e != hipSuccess) return hip_fail(e, "mfma up-projection");
    {
      TimedLaunch t("mfma_attention", s);
      e = launch_mfma_attention(a, kn, vt, kr, qtab, s);
    }
    if (e != hipSuccess) return hip_fail(e, "mfma attention");
  } else {
    TimedLaunch t("simt_explicit", s);
    e = launch_simt_explicit(a, reinterpret_cast<float*>(ws + p.off_kn), reinterpret_cast<float*>(ws + p.off_v),
                             reinterpret_cast<float*>(ws + p.off_krot), qtab, ktab, s);
    if (e != hipSuccess) return hip_fail(e, "simt explicit forward");
  }
  return MLA_OK;
}

size_t mla_decode_absorbed_workspace_size(const mla_decode_desc* desc) {
  DecodePlan p;
  if (make_decode_plan(desc, &p) != MLA_OK) return 0;
  return p.total;
}

mla_status mla_decode_absorbed_workspace_layout(const mla_decode_desc* desc, size_t offsets[4]) {
  if (offsets == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  DecodePlan p;
  mla_status st = make_decode_plan(desc, &p);
  if (st != MLA_OK) return st;
  offsets[0] = p.off_qt;
  offsets[1] = p.off_lse;
  offsets[2] = p.off_opart;
  offsets[3] = p.qt_elem;
  return MLA_OK;
}

mla_status mla_decode_absorbed(const mla_decode_desc* desc, const void* q_nope, const void* q_pe,
                               const void* kv_cache, const int32_t* cache_len, const void* w_kv_b, void* out,
                               float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  DecodePlan p;
  mla_status st = make_decode_plan(desc, &p);
  if (st != MLA_OK) return st;
  if (q_nope == nullptr || q_pe == nullptr || cache_len == nullptr || w_kv_b == nullptr || out == nullptr)
    return MLA_ERR_INVALID_ARGUMENT;
  if (desc->max_cache_len > 0 && kv_cache == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < p.total) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (workspace == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  if (!aligned16(w_kv_b) || !aligned16(workspace)) return MLA_ERR_INVALID_ARGUMENT;
  if (p.mfma) {
    const void* ptrs[] = {q_nope, q_pe, kv_cache, out};
    for (const void* q : ptrs)
      if (q != nullptr && !aligned16(q)) return MLA_ERR_INVALID_ARGUMENT;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  DecodeArgs a;
  fill_decode_args(desc, q_nope, q_pe, kv_cache, cache_len, w_kv_b, out, lse, &a);
  return run_decode(p, a, static_cast<char*>(workspace), s);
}

mla_status mla_decode_absorbed_noalloc(const mla_decode_desc* desc, const void* q_nope, const void* q_pe,
                                       const void* kv_cache, const int32_t* cache_len, const void* w_kv_b,
                                       void* out, float* lse, void* stream) {
  DecodePlan p;
  mla_status st = make_decode_plan(desc, &p);
  if (st != MLA_OK) return st;
  if (q_nope == nullptr || q_pe == nullptr || cache_len == nullptr || w_kv_b == nullptr || out == nullptr)
    return MLA_ERR_INVALID_ARGUMENT;
  if (desc->max_cache_len > 0 && kv_cache == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  if (p.total > kScratchBytes) {
    g_last_error = "decode intermediates need " + std::to_string(p.total) + " bytes; the fixed scratch holds " +
                   std::to_string(kScratchBytes);
    return MLA_ERR_WORKSPACE_TOO_SMALL;
  }
  if (!aligned16(w_kv_b)) return MLA_ERR_INVALID_ARGUMENT;
  if (p.mfma) {
    const void* ptrs[] = {q_nope, q_pe, kv_cache, out};
    for (const void* q : ptrs)
      if (q != nullptr && !aligned16(q)) return MLA_ERR_INVALID_ARGUMENT;
  }
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != MLA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  DecodeArgs a;
  fill_decode_args(desc, q_nope, q_pe, kv_cache, cache_len, w_kv_b, out, lse, &a);
  return run_decode(p, a, static_cast<char*>(ws), s);
}

size_t mla_bwd_explicit_workspace_size(const mla_explicit_desc* desc) {
  BackwardPlan p;
  if (make_backward_plan(desc, &p) != MLA_OK) return 0;
  return std::max<size_t>(p.total, 1);
}

mla_status mla_bwd_explicit(const mla_explicit_desc* desc, const void* q_nope, const void* q_pe,
                            const void* c_kv, const void* k_pe, const void* w_kv_b, const void* out,
                            const float* lse, const void* d_out, float* dq_nope, float* dq_pe, float* dc_kv,
                            float* dk_pe, float* dw_kv_b, void* workspace, size_t workspace_bytes,
                            void* stream) {
  BackwardPlan p;
  mla_status st = make_backward_plan(desc, &p);
  if (st != MLA_OK) return st;
  const bool has_q = desc->s_q > 0, has_kv = desc->s_kv > 0;
  if (w_kv_b == nullptr || dw_kv_b == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  if (has_q && (q_nope == nullptr || q_pe == nullptr || out == nullptr || lse == nullptr || d_out == nullptr ||
                dq_nope == nullptr || dq_pe == nullptr))
    return MLA_ERR_INVALID_ARGUMENT;
  if (has_kv && (c_kv == nullptr || k_pe == nullptr || dc_kv == nullptr || dk_pe == nullptr))
    return MLA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < p.total) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (workspace == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  BackwardArgs a;
  a.f = explicit_args(desc, p.fwd);
  ExplicitArgs& f = a.f;
  f.q_nope = q_nope; f.q_pe = q_pe; f.c_kv = c_kv; f.k_pe = k_pe; f.w = w_kv_b;
  f.out = nullptr; f.lse = nullptr;
  a.out = out; a.lse = lse; a.d_out = d_out;
  a.dq_nope = dq_nope; a.dq_pe = dq_pe; a.dc_kv = dc_kv; a.dk_pe = dk_pe; a.dw = dw_kv_b;
  hipError_t e;
  if (p.mfma) {
    const void* ptrs[] = {q_nope, q_pe, c_kv, k_pe, w_kv_b, out, d_out, dq_nope, dq_pe, dc_kv, dk_pe, dw_kv_b, workspace};
    for (const void* q : ptrs)
      if (q != nullptr && !aligned16(q)) return MLA_ERR_INVALID_ARGUMENT;
    MfmaBwdWorkspace w;
    mfma_backward_workspace(f, &w, ws);
    {
      // both tables (the key table turns the key band's gradient back) and the key band
      TimedLaunch t("rope_band", s);
      e = launch_rope_band(f, w.qtab, w.ktab, w.krot, s);
    }
    if (e != hipSuccess) return hip_fail(e, "rope tables");
    {
      TimedLaunch t("mfma_up_projection", s);
      e = launch_mfma_upproj(f, w.kn, w.vrow, s, /*v_rows=*/true);   // V straight in the row layout
    }
    if (e != hipSuccess) return hip_fail(e, "mfma up-projection");
    {
      TimedLaunch t("bwd_prep", s);
      e = launch_bwd_prep(a, w, s);
    }
    if (e != hipSuccess) return hip_fail(e, "backward operand layouts");
    {
      TimedLaunch t("bwd_kv", s);
      e = launch_bwd_kv(a, w, s);
    }
    if (e != hipSuccess) return hip_fail(e, "backward key/value gradients");
    {
      TimedLaunch t("bwd_dq", s);
      e = launch_bwd_dq(a, w, s);
    }
    if (e != hipSuccess) return hip_fail(e, "backward query gradients");
    {
      TimedLaunch t("bwd_dk_pe", s);
      e = launch_bwd_dkpe(a, w, s);
    }
    if (e != hipSuccess) return hip_fail(e, "backward key band gradient");
    {
      TimedLaunch t("bwd_gemms", s);
      e = launch_bwd_gemms(a, w, s);
    }
    if (e != hipSuccess) return hip_fail(e, "backward latent and weight gradients");
    return MLA_OK;
  }
  SimtBwdWorkspace w;
  w.qtab = reinterpret_cast<float2*>(ws + p.off_qtab);
  w.ktab = reinterpret_cast<float2*>(ws + p.off_ktab);
  w.kn = reinterpret_cast<float*>(ws + p.off_kn);
  w.v = reinterpret_cast<float*>(ws + p.off_v);
  w.krot = reinterpret_cast<float*>(ws + p.off_krot);
  w.qrot = reinterpret_cast<float*>(ws + p.off_qrot);
  w.p = reinterpret_cast<float*>(ws + p.off_p);
  w.ds = reinterpret_cast<float*>(ws + p.off_ds);
  w.dkn = reinterpret_cast<float*>(ws + p.off_dkn);
  w.dv = reinterpret_cast<float*>(ws + p.off_dv);
  {
    TimedLaunch t("rope_tables", s);
    e = launch_rope_table(const_cast<float2*>(w.qtab), f.q_pos0, f.Sq, f.dr, f.rope_base, s);
    if (e == hipSuccess) e = launch_rope_table(const_cast<float2*>(w.ktab), f.kv_pos0, f.s_vis, f.dr, f.rope_base, s);
  }
  if (e != hipSuccess) return hip_fail(e, "rope tables");
  {
    // K_nope, V and the rotated key band, as in the forward (no query rows)
    TimedLaunch t("simt_up_projection", s);
    ExplicitArgs up = f;
    up.Sq = 0;
    e = launch_simt_explicit(up, w.kn, w.v, w.krot, w.qtab, w.ktab, s);
  }
  if (e != hipSuccess) return hip_fail(e, "simt up-projection");
  {
    TimedLaunch t("simt_backward", s);
    e = launch_simt_backward(a, w, s);
  }
  if (e != hipSuccess) return hip_fail(e, "simt backward");
  return MLA_OK;
}

size_t mla_fwd_absorbed_workspace_size(const mla_explicit_desc* desc) {
  AbsorbedPlan p;
  if (make_absorbed_plan(desc, &p) != MLA_OK) return 0;
  return std::max<size_t>(p.total, 1);
}

mla_status mla_fwd_absorbed(const mla_explicit_desc* desc, const void* q_nope, const void* q_pe,
                            const void* c_kv, const void* k_pe, const void* w_kv_b, void* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  AbsorbedPlan p;
  mla_status st = make_absorbed_plan(desc, &p);
  if (st != MLA_OK) return st;
  const bool has_q = desc->s_q > 0, has_kv = desc->s_kv > 0;
  if (w_kv_b == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  if (has_q && (q_nope == nullptr || q_pe == nullptr || out == nullptr)) return MLA_ERR_INVALID_ARGUMENT;
  if (has_kv && (c_kv == nullptr || k_pe == nullptr)) return MLA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < p.total) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (p.total > 0 && workspace == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  if (!has_q) return MLA_OK;
  if (!aligned16(w_kv_b) || !aligned16(workspace)) return MLA_ERR_INVALID_ARGUMENT;
  if (p.dec.mfma) {
    const void* ptrs[] = {q_nope, q_pe, out};
    for (const void* q : ptrs)
      if (!aligned16(q)) return MLA_ERR_INVALID_ARGUMENT;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  ExplicitArgs ea{};
  ea.B = desc->batch; ea.Sq = desc->s_q; ea.Skv = desc->s_kv; ea.H = desc->n_heads;
  ea.dkv = desc->d_kv; ea.dn = desc->d_nope; ea.dr = desc->d_rope; ea.dv = desc->d_v;
  ea.q_pos0 = desc->q_pos0; ea.kv_pos0 = desc->kv_pos0; ea.causal = desc->causal;
  ea.scale = desc->softmax_scale; ea.rope_base = desc->rope_base;
  ea.in_dt = desc->in_dtype; ea.out_dt = desc->out_dtype;
  ea.c_kv = c_kv; ea.k_pe = k_pe;
  void* cache = ws + p.off_cache;
  int32_t* len = reinterpret_cast<int32_t*>(ws + p.off_len);
  int64_t* pos = reinterpret_cast<int64_t*>(ws + p.off_pos);
  hipError_t e;
  {
    TimedLaunch t("latent_cache", s);
    e = launch_latent_cache(ea, cache, len, pos, s);
  }
  if (e != hipSuccess) return hip_fail(e, "latent rows");
  DecodeArgs a;
  fill_decode_args(&p.dd, q_nope, q_pe, cache, len, w_kv_b, out, lse, &a);
  a.seq_per_cache = desc->s_q;
  a.q_pos = pos;
  a.reverse = 1;          // longest rows first
  a.lse_seq = desc->s_q;  // lse [B, H, s_q] as in the explicit form
  return run_decode(p.dec, a, ws, s);
}

mla_status mla_timing_begin(void) {
  g_timing.active = true;
  return MLA_OK;
}

mla_status mla_timing_end(void) {
  g_timing.active = false;
  mla_status st = MLA_OK;
  for (const PendingLaunch& p : g_timing.pending) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(p.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.start, p.stop);
    if (e != hipSuccess) {
      st = hip_fail(e, "timing");
    } else {
      bool found = false;
      for (TimingTotal& t : g_timing.totals)
        if (std::strcmp(t.name, p.name) == 0) {
          t.ms += ms;
          t.launches += 1;
          found = true;
        }
      if (!found) g_timing.totals.push_back({p.name, (double)ms, 1});
    }
    g_timing.pool.push_back(p.start);
    g_timing.pool.push_back(p.stop);
  }
  g_timing.pending.clear();
  return st;
}

mla_status mla_timing_reset(void) {
  g_timing.totals.clear();
  return MLA_OK;
}

int32_t mla_timing_count(void) { return (int32_t)g_timing.totals.size(); }

mla_status mla_timing_get(int32_t index, const char** name, double* total_ms, int64_t* launches) {
  if (index < 0 || index >= (int32_t)g_timing.totals.size() || name == nullptr || total_ms == nullptr ||
      launches == nullptr)
    return MLA_ERR_INVALID_ARGUMENT;
  const TimingTotal& t = g_timing.totals[index];
  *name = t.name;
  *total_ms = t.ms;
  *launches = t.launches;
  return MLA_OK;
}

const char* mla_status_string(mla_status status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARGUMENT: return "MLA_ERR_INVALID_ARGUMENT";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

const char* mla_build_info(void) {
  return "libmla: target gfx950; kernels: rope_table, simt (explicit, decode), mfma (up-projection, "
         "attention, absorb, split-KV), lse combine";
}

}  // extern "C"
