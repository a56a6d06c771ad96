// C ABI of the jagged HSTU attention library: argument validation, workspace
// carve-up and the launch sequence of each call. Every check runs before the
// first launch, so an error never leaves an output half written.
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "../../include/hstu_attn.h"
#include "internal.h"

using namespace hstu;

namespace {

thread_local std::string g_last_error;

hstu_status fail(hstu_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

hstu_status ok() {
  g_last_error.clear();
  return HSTU_OK;
}

}  // namespace

int hstu::set_error(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

namespace {

hstu_status hip_fail(hipError_t e, const char* what) {
  return fail(HSTU_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int elem_bytes(int32_t dtype) { return dtype == HSTU_DTYPE_BF16 ? 2 : 4; }

// Largest input row stride (elements): 64 rows of 4-byte elements must stay
// below 2^31 bytes.
constexpr int64_t kMaxStride = (int64_t)1 << 22;

// Shape checks shared by every attention entry point.
hstu_status check_desc(const hstu_attn_desc* d) {
  if (!d) return fail(HSTU_EINVAL, "desc is NULL");
  if (d->batch < 0) return fail(HSTU_EINVAL, "batch %d < 0", d->batch);
  if (d->heads < 1) return fail(HSTU_EINVAL, "heads %d < 1", d->heads);
  if (d->dtype != HSTU_DTYPE_BF16 && d->dtype != HSTU_DTYPE_FP32)
    return fail(HSTU_EINVAL, "unknown dtype %d", d->dtype);
  if (d->d_qk != d->d_v)
    return fail(HSTU_EUNSUPPORTED, "d_qk (%d) != d_v (%d) is not supported", d->d_qk, d->d_v);
  const bool dim_ok = d->d_qk == 32 || d->d_qk == 64 || d->d_qk == 128;
  if (!dim_ok)
    return fail(HSTU_EUNSUPPORTED, "head dim %d is not supported for dtype %d", d->d_qk, d->dtype);
  if (d->max_len < 1 || d->max_len > (1 << 30)) return fail(HSTU_EINVAL, "max_len %d out of range", d->max_len);
  if (d->n_time_buckets < 0 || d->n_time_buckets > 1024)
    return fail(HSTU_EINVAL, "n_time_buckets %d outside [0, 1024]", d->n_time_buckets);
  if (d->deterministic != 0 && d->deterministic != 1)
    return fail(HSTU_EINVAL, "deterministic %d must be 0 or 1", d->deterministic);
  if (d->rab_heads != 1 && d->rab_heads != d->heads)
    return fail(HSTU_EINVAL, "rab_heads %d must be 1 or heads (%d)", d->rab_heads, d->heads);
  if (d->total_tokens < 0 || d->total_tokens >= ((int64_t)1 << 31))
    return fail(HSTU_EINVAL, "total_tokens %lld outside [0, 2^31)", (long long)d->total_tokens);
  if ((double)d->total_tokens * d->heads * d->d_qk >= 4.0e18)
    return fail(HSTU_EINVAL, "total_tokens * heads * d overflows the index range");
  const int64_t hd = (int64_t)d->heads * d->d_qk;
  const int vec = 16 / elem_bytes(d->dtype);
  const int64_t strides[4] = {d->stride_q, d->stride_k, d->stride_v, d->stride_u};
  const char* names[4] = {"stride_q", "stride_k", "stride_v", "stride_u"};
  for (int i = 0; i < 4; ++i) {
    if (i == 3 && strides[i] == 0) continue;  // u may be absent
    if (strides[i] < hd) return fail(HSTU_EINVAL, "%s %lld < heads*d (%lld)", names[i], (long long)strides[i], (long long)hd);
    if (strides[i] % vec) return fail(HSTU_EINVAL, "%s %lld must be a multiple of %d", names[i], (long long)strides[i], vec);
    // the kernels address a 64-row tile of an input through a buffer
    // resource whose range is a 32-bit byte count
    if (strides[i] > kMaxStride)
      return fail(HSTU_EUNSUPPORTED, "%s %lld above %lld", names[i], (long long)strides[i], (long long)kMaxStride);
  }
  return HSTU_OK;
}

AttnParams base_params(const hstu_attn_desc* d, const int64_t* seq_offsets, const int64_t* num_targets,
                       const int64_t* timestamps, const float* rab_pos, const float* rab_time,
                       const void* q, const void* k, const void* v, const void* u) {
  AttnParams p = {};
  p.B = d->batch;
  p.H = d->heads;
  p.D = d->d_qk;
  p.max_len = d->max_len;
  p.n_time_buckets = rab_time ? d->n_time_buckets : 0;
  p.rab_heads = d->rab_heads;
  p.det = d->deterministic;
  p.n_time_room = d->n_time_buckets;
  p.T = d->total_tokens;
  p.sq = d->stride_q;
  p.sk = d->stride_k;
  p.sv = d->stride_v;
  p.su = d->stride_u;
  p.seq_offsets = seq_offsets;
  p.num_targets = num_targets;
  p.timestamps = rab_time ? timestamps : nullptr;
  p.rab_pos = rab_pos;
  p.rab_time = rab_time;
  p.q = q;
  p.k = k;
  p.v = v;
  p.u = u;
  return p;
}

hstu_status check_inputs(const hstu_attn_desc* d, const int64_t* seq_offsets, const int64_t* timestamps,
                         const float* rab_time, const void* q, const void* k, const void* v,
                         const void* u) {
  if (d->batch > 0 && !seq_offsets) return fail(HSTU_EINVAL, "seq_offsets is NULL");
  if (rab_time && d->n_time_buckets < 1)
    return fail(HSTU_EINVAL, "rab_time given but n_time_buckets is %d", d->n_time_buckets);
  if (rab_time && !timestamps) return fail(HSTU_EINVAL, "rab_time given without timestamps");
  if (d->total_tokens > 0) {
    if (!q || !k || !v) return fail(HSTU_EINVAL, "q, k and v are required");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || (u && !aligned(u, 16)))
      return fail(HSTU_EINVAL, "q, k, v, u must be 16-byte aligned");
    if (u && d->stride_u == 0) return fail(HSTU_EINVAL, "u given with stride_u 0");
  }
  return HSTU_OK;
}

template <typename T>
hipError_t dispatch_fwd(const AttnParams& p, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_fwd<T, 32>(p, s);
    case 64: return launch_fwd<T, 64>(p, s);
    case 128: return launch_fwd<T, 128>(p, s);
    default: return hipErrorInvalidValue;
  }
}
template <>
hipError_t dispatch_fwd<bf16>(const AttnParams& p, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_fwd<bf16, 32>(p, s);
    case 64: return launch_fwd<bf16, 64>(p, s);
    case 128: return launch_fwd<bf16, 128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t dispatch_fwd_cand(const AttnParams& p, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_fwd_cand<T, 32>(p, s);
    case 64: return launch_fwd_cand<T, 64>(p, s);
    case 128: return launch_fwd_cand<T, 128>(p, s);
    default: return hipErrorInvalidValue;
  }
}
template <>
hipError_t dispatch_fwd_cand<bf16>(const AttnParams& p, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_fwd_cand<bf16, 32>(p, s);
    case 64: return launch_fwd_cand<bf16, 64>(p, s);
    case 128: return launch_fwd_cand<bf16, 128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// Joined row count of a cached-history call (candidates + history rows).
hstu_status check_hist_tokens(const hstu_attn_desc* d, int64_t hist_tokens) {
  if (hist_tokens < 0) return fail(HSTU_EINVAL, "hist_tokens %lld < 0", (long long)hist_tokens);
  if (d->total_tokens + hist_tokens >= ((int64_t)1 << 31))
    return fail(HSTU_EINVAL, "total_tokens + hist_tokens = %lld outside [0, 2^31)",
                (long long)(d->total_tokens + hist_tokens));
  if ((double)(d->total_tokens + hist_tokens) * d->heads * d->d_qk >= 4.0e18)
    return fail(HSTU_EINVAL, "(total_tokens + hist_tokens) * heads * d overflows the index range");
  return HSTU_OK;
}

template <typename T>
hipError_t dispatch_bwd(const AttnParams& p, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_bwd<T, 32>(p, s);
    case 64: return launch_bwd<T, 64>(p, s);
    case 128: return launch_bwd<T, 128>(p, s);
    default: return hipErrorInvalidValue;
  }
}
template <>
hipError_t dispatch_bwd<bf16>(const AttnParams& p, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_bwd_k16<32>(p, s);
    case 64: return launch_bwd_k16<64>(p, s);
    case 128: return launch_bwd_k16<128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t dispatch_dq(const AttnParams& p, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_dq<T, 32>(p, s);
    case 64: return launch_dq<T, 64>(p, s);
    case 128: return launch_dq<T, 128>(p, s);
    default: return hipErrorInvalidValue;
  }
}
template <>
hipError_t dispatch_dq<bf16>(const AttnParams& p, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_dq<bf16, 32>(p, s);
    case 64: return launch_dq<bf16, 64>(p, s);
    case 128: return launch_dq<bf16, 128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t dispatch_dq_ds(const AttnParams& p, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_dq_ds<32>(p, s);
    case 64: return launch_dq_ds<64>(p, s);
    case 128: return launch_dq_ds<128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// After the prep and dA' / dU: dK / dV / d_rab per key block, then dQ per
// query block (its own schedule, the forward's). With the dS export (bf16),
// the schedule's count of exported sequences splits the dQ work between the
// two dQ kernels.
template <typename T>
hipError_t run_bwd_main(const AttnParams& p, hipStream_t s) {
  hipError_t e = dispatch_bwd<T>(p, s);
  if (e == hipSuccess) e = launch_rab_reduce(p, s);
  AttnParams pq = p;                             // the dQ pass walks query blocks
  pq.items = p.items_q;
  if (e == hipSuccess) e = dispatch_dq<T>(pq, s);
  if (e == hipSuccess && p.ds != nullptr) e = dispatch_dq_ds(pq, s);
  return e;
}

}  // namespace

extern "C" {

hstu_status hstu_attn_fwd_workspace_size(const hstu_attn_desc* desc, size_t* bytes) {
  hstu_status st = check_desc(desc);
  if (st != HSTU_OK) return st;
  if (!bytes) return fail(HSTU_EINVAL, "bytes is NULL");
  AttnParams p = base_params(desc, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                             nullptr, nullptr);
  *bytes = carve_workspace(p, nullptr, false, elem_bytes(desc->dtype), false);
  return ok();
}

hstu_status hstu_attn_bwd_workspace_size(const hstu_attn_desc* desc, size_t* bytes) {
  hstu_status st = check_desc(desc);
  if (st != HSTU_OK) return st;
  if (!bytes) return fail(HSTU_EINVAL, "bytes is NULL");
  AttnParams p = base_params(desc, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                             nullptr, nullptr);
  *bytes = carve_workspace(p, nullptr, true, elem_bytes(desc->dtype), true);
  return ok();
}

hstu_status hstu_attn_bwd_workspace_size_min(const hstu_attn_desc* desc, size_t* bytes) {
  hstu_status st = check_desc(desc);
  if (st != HSTU_OK) return st;
  if (!bytes) return fail(HSTU_EINVAL, "bytes is NULL");
  AttnParams p = base_params(desc, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                             nullptr, nullptr);
  *bytes = carve_workspace(p, nullptr, true, elem_bytes(desc->dtype), false);
  return ok();
}

hstu_status hstu_attn_fwd(const hstu_attn_desc* desc, const int64_t* seq_offsets,
                          const int64_t* num_targets, const int64_t* timestamps,
                          const float* rab_pos, const float* rab_time, const void* q,
                          const void* k, const void* v, const void* u, void* o, float* a_saved,
                          void* workspace, size_t workspace_bytes, void* stream) {
  hstu_status st = check_desc(desc);
  if (st != HSTU_OK) return st;
  st = check_inputs(desc, seq_offsets, timestamps, rab_time, q, k, v, u);
  if (st != HSTU_OK) return st;
  if (desc->total_tokens > 0) {
    if (!o) return fail(HSTU_EINVAL, "o is NULL");
    if (!aligned(o, 16) || (a_saved && !aligned(a_saved, 16)))
      return fail(HSTU_EINVAL, "o and a_saved must be 16-byte aligned");
  }
  AttnParams p = base_params(desc, seq_offsets, num_targets, timestamps, rab_pos, rab_time, q, k,
                             v, u);
  p.o = o;
  p.a_saved = a_saved;
  const size_t need = carve_workspace(p, nullptr, false, elem_bytes(desc->dtype), false);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(HSTU_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                workspace_bytes);
  carve_workspace(p, workspace, false, elem_bytes(desc->dtype), false);
  if (p.T == 0 || p.B == 0) return ok();
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_fwd_prep(p, s);         // sequence prep and work list
  if (e == hipSuccess)
    e = desc->dtype == HSTU_DTYPE_BF16 ? dispatch_fwd<bf16>(p, s) : dispatch_fwd<float>(p, s);
  if (e != hipSuccess) return hip_fail(e, "hstu_attn_fwd launch");
  return ok();
}

hstu_status hstu_attn_fwd_cached_workspace_size(const hstu_attn_desc* desc, int64_t hist_tokens,
                                                 size_t* bytes) {
  hstu_status st = check_desc(desc);
  if (st != HSTU_OK) return st;
  st = check_hist_tokens(desc, hist_tokens);
  if (st != HSTU_OK) return st;
  if (!bytes) return fail(HSTU_EINVAL, "bytes is NULL");
  AttnParams p = base_params(desc, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                             nullptr, nullptr);
  p.T = desc->total_tokens + hist_tokens;
  p.m_rows = desc->total_tokens;
  p.kv_splits = cand_kv_splits(p.m_rows, hist_tokens, p.B, p.H);
  CandArgs c = {};
  *bytes = carve_workspace_cand(p, c, nullptr);
  return ok();
}

hstu_status hstu_attn_fwd_cached(const hstu_attn_desc* desc, const int64_t* cand_offsets,
                                 const int64_t* cand_first, const int64_t* n_cands,
                                 const int64_t* hist_offsets, int64_t hist_tokens,
                                 const int64_t* ts_hist, const int64_t* ts_cand,
                                 const float* rab_pos, const float* rab_time, const void* q,
                                 const void* k, const void* v, const void* u, const void* k_hist,
                                 const void* v_hist, int64_t stride_kh, int64_t stride_vh, void* o,
                                 float* a_saved, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  hstu_status st = check_desc(desc);
  if (st != HSTU_OK) return st;
  st = check_hist_tokens(desc, hist_tokens);
  if (st != HSTU_OK) return st;
  if (desc->batch > 0 && (!cand_offsets || !cand_first || !n_cands || !hist_offsets))
    return fail(HSTU_EINVAL, "cand_offsets, cand_first, n_cands and hist_offsets are required");
  if (rab_time && desc->n_time_buckets < 1)
    return fail(HSTU_EINVAL, "rab_time given but n_time_buckets is %d", desc->n_time_buckets);
  // a call without candidate rows computes nothing, so needs no tensors
  if (desc->total_tokens > 0) {
    if (rab_time && (!ts_cand || (hist_tokens > 0 && !ts_hist)))
      return fail(HSTU_EINVAL, "rab_time given without ts_cand / ts_hist");
    // the candidate tensors as the forward's inputs
    st = check_inputs(desc, cand_offsets, ts_cand, rab_time, q, k, v, u);
    if (st != HSTU_OK) return st;
  }
  if (hist_tokens > 0 && desc->total_tokens > 0) {
    if (!k_hist || !v_hist) return fail(HSTU_EINVAL, "k_hist and v_hist are required");
    if (!aligned(k_hist, 16) || !aligned(v_hist, 16))
      return fail(HSTU_EINVAL, "k_hist and v_hist must be 16-byte aligned");
    const int64_t hd = (int64_t)desc->heads * desc->d_qk;
    const int vec = 16 / elem_bytes(desc->dtype);
    if (stride_kh < hd || stride_vh < hd || stride_kh % vec || stride_vh % vec)
      return fail(HSTU_EINVAL, "stride_kh %lld / stride_vh %lld must be >= heads*d (%lld) and multiples of %d",
                  (long long)stride_kh, (long long)stride_vh, (long long)hd, vec);
  }
  if (desc->total_tokens > 0) {
    if (!o) return fail(HSTU_EINVAL, "o is NULL");
    if (!aligned(o, 16) || (a_saved && !aligned(a_saved, 16)))
      return fail(HSTU_EINVAL, "o and a_saved must be 16-byte aligned");
  }
  AttnParams p = base_params(desc, nullptr, nullptr, nullptr, rab_pos, rab_time, q, k, v, u);
  p.T = desc->total_tokens + hist_tokens;
  p.m_rows = desc->total_tokens;
  p.kv_splits = cand_kv_splits(p.m_rows, hist_tokens, p.B, p.H);
  p.o = o;
  p.a_saved = a_saved;
  p.k_hist = k_hist;
  p.v_hist = v_hist;
  p.skh = stride_kh;
  p.svh = stride_vh;
  CandArgs c = {cand_offsets, cand_first, n_cands, hist_offsets, ts_hist, ts_cand, nullptr, nullptr};
  const size_t need = carve_workspace_cand(p, c, nullptr);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(HSTU_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                workspace_bytes);
  carve_workspace_cand(p, c, workspace);
  p.cand = c.cand;
  p.timestamps = rab_time ? c.ts_joined : nullptr;   // the joined numbering's timestamps
  if (desc->total_tokens == 0 || p.B == 0) return ok();
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_prep_cand(p, c, s);     // sequence prep and work list
  if (e == hipSuccess)
    e = desc->dtype == HSTU_DTYPE_BF16 ? dispatch_fwd_cand<bf16>(p, s) : dispatch_fwd_cand<float>(p, s);
  if (e != hipSuccess) return hip_fail(e, "hstu_attn_fwd_cached launch");
  return ok();
}

hstu_status hstu_attn_bwd(const hstu_attn_desc* desc, const int64_t* seq_offsets,
                          const int64_t* num_targets, const int64_t* timestamps,
                          const float* rab_pos, const float* rab_time, const void* q,
                          const void* k, const void* v, const void* u, const float* a_saved,
                          const void* d_o, void* dq, void* dk, void* dv, void* du,
                          float* d_rab_pos, float* d_rab_time, void* workspace,
                          size_t workspace_bytes, void* stream) {
  hstu_status st = check_desc(desc);
  if (st != HSTU_OK) return st;
  st = check_inputs(desc, seq_offsets, timestamps, rab_time, q, k, v, u);
  if (st != HSTU_OK) return st;
  if (rab_pos && !d_rab_pos) return fail(HSTU_EINVAL, "rab_pos given but d_rab_pos is NULL");
  if (rab_time && !d_rab_time) return fail(HSTU_EINVAL, "rab_time given but d_rab_time is NULL");
  if (desc->total_tokens > 0) {
    if (!d_o || !dq || !dk || !dv) return fail(HSTU_EINVAL, "d_o, dq, dk and dv are required");
    if (u && (!du || !a_saved)) return fail(HSTU_EINVAL, "a gated call needs du and a_saved");
    if (!aligned(d_o, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
        (du && !aligned(du, 16)) || (a_saved && !aligned(a_saved, 16)))
      return fail(HSTU_EINVAL, "gradient buffers must be 16-byte aligned");
  }
  AttnParams p = base_params(desc, seq_offsets, num_targets, timestamps, rab_pos, rab_time, q, k,
                             v, u);
  p.a_in = a_saved;
  p.d_o = d_o;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.du = du;
  p.d_rab_pos = rab_pos ? d_rab_pos : nullptr;
  p.d_rab_time = rab_time ? d_rab_time : nullptr;
  const int eb = elem_bytes(desc->dtype);
  const size_t need = carve_workspace(p, nullptr, true, eb, false);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(HSTU_EWORKSPACE, "workspace needs at least %zu bytes, 256-byte aligned (got %zu)",
                need, workspace_bytes);
  // the dS export when the workspace holds its room, else the recompute pass
  const bool ds_room = workspace_bytes >= carve_workspace(p, nullptr, true, eb, true);
  carve_workspace(p, workspace, true, eb, ds_room);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (p.T > 0 && p.B > 0) {
    // work lists, sequence prep (which also clears d_rab_pos / d_rab_time)
    // and dA', dU in one launch
    e = desc->dtype == HSTU_DTYPE_BF16 ? launch_bwd_prep<bf16>(p, s) : launch_bwd_prep<float>(p, s);
    if (e == hipSuccess)
      e = desc->dtype == HSTU_DTYPE_BF16 ? run_bwd_main<bf16>(p, s) : run_bwd_main<float>(p, s);
  } else {
    // nothing to attend over: the rab gradients are still overwritten
    if (p.d_rab_pos)
      e = launch_fill_f32(p.d_rab_pos, (int64_t)desc->rab_heads * (2 * (int64_t)desc->max_len - 1), 0.f, s);
    if (e == hipSuccess && p.d_rab_time)
      e = launch_fill_f32(p.d_rab_time, (int64_t)desc->rab_heads * desc->n_time_buckets, 0.f, s);
  }
  if (e != hipSuccess) return hip_fail(e, "hstu_attn_bwd launch");
  return ok();
}

hstu_status hstu_rab_bucketize(const hstu_attn_desc* desc, const int64_t* seq_offsets,
                               const int64_t* num_targets, const int64_t* timestamps,
                               const int64_t* pair_offsets, uint16_t* bp_out, uint8_t* bt_out,
                               void* stream) {
  if (!desc) return fail(HSTU_EINVAL, "desc is NULL");
  if (desc->batch < 0) return fail(HSTU_EINVAL, "batch %d < 0", desc->batch);
  if (desc->max_len < 1 || desc->max_len > 32768)
    return fail(HSTU_EINVAL, "max_len %d outside [1, 32768] for a uint16 position bucket", desc->max_len);
  if (desc->batch > 0 && (!seq_offsets || !pair_offsets))
    return fail(HSTU_EINVAL, "seq_offsets and pair_offsets are required");
  if (bt_out && (!timestamps || desc->n_time_buckets < 1 || desc->n_time_buckets > 256))
    return fail(HSTU_EINVAL, "bt_out needs timestamps and 1 <= n_time_buckets <= 256");
  AttnParams p = {};
  p.B = desc->batch;
  p.max_len = desc->max_len;
  p.n_time_buckets = desc->n_time_buckets;
  p.seq_offsets = seq_offsets;
  p.num_targets = num_targets;
  p.timestamps = timestamps;
  hipError_t e = launch_bucketize(p, pair_offsets, bp_out, bt_out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hstu_rab_bucketize launch");
  return ok();
}

hstu_status hstu_rab_pair_offsets(const hstu_attn_desc* desc, const int64_t* seq_offsets,
                                  const int64_t* num_targets, int64_t* pair_offsets, void* stream) {
  if (!desc) return fail(HSTU_EINVAL, "desc is NULL");
  if (desc->batch < 0) return fail(HSTU_EINVAL, "batch %d < 0", desc->batch);
  if (!pair_offsets || (desc->batch > 0 && !seq_offsets))
    return fail(HSTU_EINVAL, "seq_offsets and pair_offsets are required");
  hipError_t e = launch_pair_offsets(seq_offsets, num_targets, desc->batch, pair_offsets,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hstu_rab_pair_offsets launch");
  return ok();
}

hstu_status hstu_linear(int64_t M, int64_t K, int64_t N, const void* x, int64_t ldx, const void* w,
                        const float* bias, void* y, int32_t apply_silu, void* stream) {
  if (M < 0 || K <= 0 || N <= 0) return fail(HSTU_EINVAL, "bad sizes M=%lld K=%lld N=%lld", (long long)M, (long long)K, (long long)N);
  if (K % 32 || N % 128) return fail(HSTU_EUNSUPPORTED, "K must be a multiple of 32 and N of 128");
  if (ldx < K || ldx % 8) return fail(HSTU_EINVAL, "ldx %lld must be >= K and a multiple of 8", (long long)ldx);
  if (M > 0 && (!x || !w || !y)) return fail(HSTU_EINVAL, "x, w and y are required");
  if (!aligned(x, 16) || !aligned(w, 16)) return fail(HSTU_EINVAL, "x and w must be 16-byte aligned");
  hipError_t e = launch_linear(M, K, N, x, ldx, w, bias, y, apply_silu, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hstu_linear launch");
  return ok();
}

hstu_status hstu_layernorm_gate(int64_t M, int64_t N, const float* a, const void* u, int64_t ldu,
                                float eps, void* out, void* stream) {
  if (M < 0 || N <= 0 || N % 64 || N > 4096) return fail(HSTU_EINVAL, "N must be a positive multiple of 64, <= 4096");
  if (ldu < N || ldu % 4) return fail(HSTU_EINVAL, "ldu %lld must be >= N and a multiple of 4", (long long)ldu);
  if (!(eps >= 0.f)) return fail(HSTU_EINVAL, "eps must be >= 0");
  if (M > 0 && (!a || !u || !out)) return fail(HSTU_EINVAL, "a, u and out are required");
  if (!aligned(a, 16) || !aligned(u, 8) || !aligned(out, 8)) return fail(HSTU_EINVAL, "misaligned buffer");
  hipError_t e = launch_layernorm_gate(M, N, a, u, ldu, eps, out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hstu_layernorm_gate launch");
  return ok();
}

// ---------------------------------------------------------------- FP8 projection
hstu_status hstu_fp8_quantize_rows(int64_t M, int64_t K, const void* x, int64_t ldx, void* q,
                                   float* scale, void* stream) {
  if (M < 0 || K <= 0) return fail(HSTU_EINVAL, "bad sizes M=%lld K=%lld", (long long)M, (long long)K);
  if (K % 16) return fail(HSTU_EUNSUPPORTED, "K must be a multiple of 16");
  if (ldx < K || ldx % 8) return fail(HSTU_EINVAL, "ldx %lld must be >= K and a multiple of 8", (long long)ldx);
  if (M > 0 && (!x || !q || !scale)) return fail(HSTU_EINVAL, "x, q and scale are required");
  if (!aligned(x, 16) || !aligned(q, 16)) return fail(HSTU_EINVAL, "x and q must be 16-byte aligned");
  hipError_t e = launch_fp8_quantize_rows(M, K, x, ldx, q, scale, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hstu_fp8_quantize_rows launch");
  return ok();
}

hstu_status hstu_fp8_prepare_weight(int64_t K, int64_t N, const void* w, void* q, float* scale,
                                    void* stream) {
  if (K <= 0 || N < 0) return fail(HSTU_EINVAL, "bad sizes K=%lld N=%lld", (long long)K, (long long)N);
  if (K % 16) return fail(HSTU_EUNSUPPORTED, "K must be a multiple of 16");
  if (N > 0 && (!w || !q || !scale)) return fail(HSTU_EINVAL, "w, q and scale are required");
  if (!aligned(w, 2) || !aligned(q, 16)) return fail(HSTU_EINVAL, "misaligned w or q");
  hipError_t e = launch_fp8_prepare_weight(K, N, w, q, scale, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hstu_fp8_prepare_weight launch");
  return ok();
}

hstu_status hstu_fp8_linear(int64_t M, int64_t K, int64_t N, const void* xq, const float* x_scale,
                            const void* wq, const float* w_scale, const float* bias, void* y,
                            int32_t apply_silu, void* stream) {
  if (M < 0 || K <= 0 || N < 0) return fail(HSTU_EINVAL, "bad sizes M=%lld K=%lld N=%lld", (long long)M, (long long)K, (long long)N);
  if (K % 16) return fail(HSTU_EUNSUPPORTED, "K must be a multiple of 16");
  if (M > 0 && N > 0 && (!xq || !x_scale || !wq || !w_scale || !y))
    return fail(HSTU_EINVAL, "xq, x_scale, wq, w_scale and y are required");
  if (!aligned(xq, 16) || !aligned(wq, 16)) return fail(HSTU_EINVAL, "xq and wq must be 16-byte aligned");
  hipError_t e = launch_fp8_linear(M, K, N, xq, x_scale, wq, w_scale, bias, y, apply_silu, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hstu_fp8_linear launch");
  return ok();
}

hstu_status hstu_layernorm_gate_fp8(int64_t M, int64_t N, const float* a, const void* u, int64_t ldu,
                                    float eps, void* q, float* scale, void* stream) {
  if (M < 0 || N <= 0 || N % 64 || N > 4096) return fail(HSTU_EINVAL, "N must be a positive multiple of 64, <= 4096");
  if (u && (ldu < N || ldu % 4)) return fail(HSTU_EINVAL, "ldu %lld must be >= N and a multiple of 4", (long long)ldu);
  if (!(eps >= 0.f)) return fail(HSTU_EINVAL, "eps must be >= 0");
  if (M > 0 && (!a || !q || !scale)) return fail(HSTU_EINVAL, "a, q and scale are required");
  if (!aligned(a, 16) || !aligned(u, 8) || !aligned(q, 4)) return fail(HSTU_EINVAL, "misaligned buffer");
  hipError_t e = launch_layernorm_gate_fp8(M, N, a, u, ldu, eps, q, scale, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hstu_layernorm_gate_fp8 launch");
  return ok();
}

// ---------------------------------------------------------------- layer backward
namespace {

struct LayerBwdWs {
  void *pre, *z, *dz, *da, *du, *dq, *dk, *dv, *d_pre, *attn;
  float* part;                                   // split partial sums of the weight gradients
  float* cpart;                                  // per-band column sums (bias gradients)
  size_t attn_bytes;
};

// Carve-up of the layer backward's workspace (base == nullptr: sizes only).
hstu_status layer_bwd_carve(int64_t M, int32_t batch, int32_t d_model, int32_t heads,
                            int32_t head_dim, int32_t max_len, void* base, LayerBwdWs* w,
                            size_t* bytes) {
  const int64_t HD = (int64_t)heads * head_dim, W = 4 * HD;
  hstu_attn_desc ad = {};
  ad.batch = batch; ad.heads = heads; ad.d_qk = head_dim; ad.d_v = head_dim;
  ad.max_len = max_len > 0 ? max_len : 1;
  ad.n_time_buckets = 0; ad.rab_heads = 1; ad.dtype = HSTU_DTYPE_BF16; ad.total_tokens = M;
  ad.stride_q = ad.stride_k = ad.stride_v = W; ad.stride_u = 0;
  // max_len 0 (no bound): the attention's minimum workspace, whose dQ pass
  // recomputes dS; otherwise room for the dS export
  size_t attn = 0;
  hstu_status st = max_len > 0 ? hstu_attn_bwd_workspace_size(&ad, &attn)
                               : hstu_attn_bwd_workspace_size_min(&ad, &attn);
  if (st != HSTU_OK) return st;
  size_t off = 0;
  auto take = [&](size_t b) {
    const size_t at = off;
    off += (b + 255) & ~(size_t)255;
    return base ? (void*)((char*)base + at) : nullptr;
  };
  const size_t e = 2;                            // bf16
  w->pre = take(e * M * W);
  w->z = take(e * M * HD);
  w->dz = take(e * M * HD);
  w->da = take(e * M * HD);
  w->du = take(e * M * HD);
  w->dq = take(e * M * HD);
  w->dk = take(e * M * HD);
  w->dv = take(e * M * HD);
  w->d_pre = take(e * M * W);
  auto part_bytes = [&](int64_t m, int64_t n) {
    const int sp = wgrad_splits(m, n, M);
    return sp > 1 ? (size_t)sp * m * n * sizeof(float) : (size_t)0;
  };
  const size_t p2 = part_bytes(HD, d_model), p1 = part_bytes(d_model, W);
  w->part = static_cast<float*>(take(p1 > p2 ? p1 : p2));
  w->cpart = static_cast<float*>(take(sizeof(float) * colsum_bands(M) * (W > d_model ? W : d_model)));
  w->attn = take(attn);
  w->attn_bytes = attn;
  *bytes = off;
  return HSTU_OK;
}

hstu_status layer_bwd_check(int64_t M, int32_t batch, int32_t d_model, int32_t heads, int32_t head_dim,
                            int32_t max_len) {
  if (M < 0 || M >= ((int64_t)1 << 31) || batch < 0 || heads < 1)
    return fail(HSTU_EINVAL, "bad sizes M=%lld batch=%d heads=%d", (long long)M, batch, heads);
  if (max_len < 0 || max_len > (1 << 30)) return fail(HSTU_EINVAL, "max_len %d out of range", max_len);
  if (head_dim != 32 && head_dim != 64 && head_dim != 128)
    return fail(HSTU_EUNSUPPORTED, "head_dim %d is not supported", head_dim);
  if (d_model <= 0 || d_model % 128 || ((int64_t)heads * head_dim) % 128)
    return fail(HSTU_EUNSUPPORTED, "d_model (%d) and heads*head_dim (%d) must be multiples of 128",
                d_model, heads * head_dim);
  return HSTU_OK;
}

}  // namespace

hstu_status hstu_layer_bwd_workspace_size(int64_t M, int32_t batch, int32_t d_model, int32_t heads,
                                          int32_t head_dim, int32_t max_len, size_t* bytes) {
  hstu_status st = layer_bwd_check(M, batch, d_model, heads, head_dim, max_len);
  if (st != HSTU_OK) return st;
  if (!bytes) return fail(HSTU_EINVAL, "bytes is NULL");
  LayerBwdWs w;
  st = layer_bwd_carve(M, batch, d_model, heads, head_dim, max_len, nullptr, &w, bytes);
  if (st != HSTU_OK) return st;
  return ok();
}

hstu_status hstu_layer_bwd(int64_t M, int32_t batch, int32_t d_model, int32_t heads,
                           int32_t head_dim, int32_t max_len, const int64_t* seq_offsets,
                           const int64_t* num_targets,
                           const void* x, const void* w1, const float* b1, const void* w2,
                           const void* uvqk, const float* a, float eps, const void* dy, void* dx,
                           float* dw1, float* db1, float* dw2, float* db2, void* workspace,
                           size_t workspace_bytes, void* stream) {
  hstu_status st = layer_bwd_check(M, batch, d_model, heads, head_dim, max_len);
  if (st != HSTU_OK) return st;
  if (!(eps >= 0.f)) return fail(HSTU_EINVAL, "eps must be >= 0");
  if (batch > 0 && !seq_offsets) return fail(HSTU_EINVAL, "seq_offsets is NULL");
  if (!dw1 || !db1 || !dw2 || !db2 || !w1 || !w2)
    return fail(HSTU_EINVAL, "w1, w2, dw1, db1, dw2 and db2 are required");
  if (M > 0 && (!x || !uvqk || !a || !dy || !dx))
    return fail(HSTU_EINVAL, "x, uvqk, a, dy and dx are required");
  const void* al[] = {x, w1, w2, uvqk, a, dy, dx, dw1, dw2};
  for (const void* q : al)
    if (!aligned(q, 16)) return fail(HSTU_EINVAL, "layer backward buffers must be 16-byte aligned");
  LayerBwdWs w;
  size_t need = 0;
  st = layer_bwd_carve(M, batch, d_model, heads, head_dim, max_len, nullptr, &w, &need);
  if (st != HSTU_OK) return st;
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(HSTU_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                workspace_bytes);
  layer_bwd_carve(M, batch, d_model, heads, head_dim, max_len, workspace, &w, &need);
  hipStream_t s = (hipStream_t)stream;
  const int64_t HD = (int64_t)heads * head_dim, W = 4 * HD;
  if (M == 0) {                                  // no tokens: every gradient is 0
    hipError_t z = launch_fill_f32(dw1, (int64_t)d_model * W, 0.f, s);
    if (z == hipSuccess) z = launch_fill_f32(db1, W, 0.f, s);
    if (z == hipSuccess) z = launch_fill_f32(dw2, HD * d_model, 0.f, s);
    if (z == hipSuccess) z = launch_fill_f32(db2, d_model, 0.f, s);
    if (z != hipSuccess) return hip_fail(z, "hstu_layer_bwd launch");
    return ok();
  }
  const bf16* uv = reinterpret_cast<const bf16*>(uvqk);
  hipError_t e = hipSuccess;
  auto run = [&](hipError_t r) { if (e == hipSuccess) e = r; };
  // Z = LayerNorm(A) * U; dW2 = Z^T dY, db2 = colsum dY; dZ = dY W2^T
  run(launch_linear(M, d_model, W, x, d_model, w1, b1, w.pre, 0, s));         // Pre = X W1 + b1
  run(launch_layernorm_gate(M, HD, a, uv, W, eps, w.z, s));
  run(launch_wgrad(HD, d_model, M, w.z, HD, dy, d_model, dw2, w.part, s));
  run(launch_colsum(M, d_model, dy, d_model, db2, w.cpart, s));
  run(launch_linear_nt(M, d_model, HD, dy, d_model, w2, d_model, w.dz, s));
  // dU = dZ * LN(A), dA = LayerNorm'(A)^T (dZ * U)
  run(launch_layernorm_gate_bwd(M, HD, a, uv, W, eps, w.dz, w.da, w.du, s));
  if (e != hipSuccess) return hip_fail(e, "hstu_layer_bwd launch");
  // attention backward (no gate, no bias) with dO = dA
  if (M > 0 && batch > 0) {
    hstu_attn_desc ad = {};
    ad.batch = batch; ad.heads = heads; ad.d_qk = head_dim; ad.d_v = head_dim;
  ad.max_len = max_len > 0 ? max_len : 1;
    ad.n_time_buckets = 0; ad.rab_heads = 1; ad.dtype = HSTU_DTYPE_BF16; ad.total_tokens = M;
    ad.stride_q = ad.stride_k = ad.stride_v = W; ad.stride_u = 0;
    st = hstu_attn_bwd(&ad, seq_offsets, num_targets, nullptr, nullptr, nullptr, uv + 2 * HD,
                       uv + 3 * HD, uv + HD, nullptr, nullptr, w.da, w.dq, w.dk, w.dv, nullptr,
                       nullptr, nullptr, w.attn, w.attn_bytes, stream);
    if (st != HSTU_OK) return st;
  }
  // dPre = [dU, dV, dQ, dK] * SiLU'(Pre); db1 = colsum dPre; dW1 = X^T dPre; dX = dPre W1^T
  run(launch_silu_bwd_uvqk(M, M, HD, w.pre, w.du, w.dv, w.dq, w.dk, w.d_pre, s));
  run(launch_colsum(M, W, w.d_pre, W, db1, w.cpart, s));
  run(launch_wgrad(d_model, W, M, x, d_model, w.d_pre, W, dw1, w.part, s));
  run(launch_linear_nt(M, W, d_model, w.d_pre, W, w1, W, dx, s));
  if (e != hipSuccess) return hip_fail(e, "hstu_layer_bwd launch");
  return ok();
}

hstu_status hstu_attn_bwd_report(const hstu_attn_desc* desc, const void* workspace,
                                 size_t workspace_bytes, hstu_attn_bwd_info* info, void* stream) {
  hstu_status st = check_desc(desc);
  if (st != HSTU_OK) return st;
  if (!info) return fail(HSTU_EINVAL, "info is NULL");
  AttnParams p = base_params(desc, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                             nullptr, nullptr);
  const int eb = elem_bytes(desc->dtype);
  const size_t need = carve_workspace(p, nullptr, true, eb, false);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(HSTU_EWORKSPACE, "workspace needs at least %zu bytes, 256-byte aligned (got %zu)",
                need, workspace_bytes);
  const bool ds_room = workspace_bytes >= carve_workspace(p, nullptr, true, eb, true);
  carve_workspace(p, const_cast<void*>(workspace), true, eb, ds_room);
  info->dq_from_ds = 0;
  info->rab_deterministic = 0;
  info->ds_sequences = 0;
  if (p.T == 0 || p.B == 0) {
    info->rab_deterministic = p.det;             // nothing summed: trivially repeatable
    return ok();
  }
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  // the dS-export and deterministic flags are adjacent (ds_on, det_on)
  int32_t flags[2] = {0, 0};
  const int32_t* dev_flags = p.ds_on ? p.ds_on : (p.det_on ? p.det_on - 1 : nullptr);
  if (e == hipSuccess && dev_flags) e = hipMemcpy(flags, dev_flags, sizeof(flags), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hstu_attn_bwd_report");
  // flags[0]: the leading sequences whose dS tiles fit the room
  info->ds_sequences = p.ds_on ? flags[0] : 0;
  info->dq_from_ds = info->ds_sequences == p.B ? 1 : 0;
  info->rab_deterministic = p.det_on ? flags[1] : 0;
  return ok();
}

const char* hstu_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
