// C ABI of libpg.so: argument checks, error text, the layout's device copy,
// and dispatch to the HIP launchers. Exceptions never cross this boundary.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

#include "pg_internal.h"

namespace {
thread_local std::string g_last_error;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

pg_status hip_fail(hipError_t e, const char* what) {
  return pg_fail(PG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Device-side checks shared by the compute entry points.
pg_status check_device_layout(const pg_layout* L) {
  if (!L) return pg_fail(PG_ERR_INVALID_ARG, "layout is NULL");
  if (!L->dev_buf && L->T > 0)
    return pg_fail(PG_ERR_STATE, "layout has no device copy (call pg_layout_upload)");
  if (L->T > 0) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev != L->device)
      return pg_fail(PG_ERR_STATE, "layout lives on device %d, current device is %d", L->device, dev);
  }
  return PG_OK;
}
}  // namespace

pg_status pg_fail(pg_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  try {
    g_last_error = buf;
  } catch (...) {
  }
  return s;
}

void pg_clear_error() { g_last_error.clear(); }

extern "C" {

const char* pg_status_string(pg_status s) {
  switch (s) {
    case PG_OK: return "ok";
    case PG_ERR_INVALID_ARG: return "invalid argument";
    case PG_ERR_UNSUPPORTED: return "unsupported";
    case PG_ERR_HIP: return "HIP error";
    case PG_ERR_OOM: return "out of memory";
    case PG_ERR_STATE: return "bad state";
  }
  return "unknown status";
}

const char* pg_last_error(void) { return g_last_error.c_str(); }

pg_status pg_build_layout_host(int32_t num_groups, const int32_t* prefix_lens,
                               const int32_t* suffix_counts, const int32_t* suffix_lens,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               double rope_theta, pg_layout** out) {
  if (!out) return pg_fail(PG_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  pg_clear_error();
  pg_layout* L = new (std::nothrow) pg_layout();
  if (!L) return pg_fail(PG_ERR_OOM, "host allocation failed");
  pg_status s = pg_layout_build_host(*L, num_groups, prefix_lens, suffix_counts, suffix_lens,
                                     num_q_heads, num_kv_heads, head_dim, rope_theta);
  if (s != PG_OK) {
    delete L;
    return s;
  }
  *out = L;
  return PG_OK;
}

pg_status pg_layout_upload(pg_layout* L, hipStream_t stream) {
  if (!L) return pg_fail(PG_ERR_INVALID_ARG, "layout is NULL");
  if (L->dev_buf || L->T == 0) {
    if (L->T == 0 && L->device < 0) {
      hipError_t e = hipGetDevice(&L->device);
      if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    }
    return PG_OK;
  }
  const size_t A = 256;
  const size_t T = size_t(L->T);
  const size_t off_g0 = 0;
  const size_t off_pe = align_up(off_g0 + 4 * T, A);
  const size_t off_ss = align_up(off_pe + 4 * T, A);
  const size_t off_it = align_up(off_ss + 4 * T, A);
  const size_t off_sp = align_up(off_it + sizeof(pg_work_item) * L->items.size(), A);
  const size_t off_fr = align_up(off_sp + sizeof(pg_key_span) * L->spans.size(), A);
  const size_t off_kv = align_up(off_fr + sizeof(double) * L->inv_freq.size(), A);
  const size_t G = L->group_off.size() - 1, N = L->suffix_lens.size();
  const size_t off_ow = align_up(off_kv + sizeof(pg_kv_item) * L->kv_items.size(), A);
  const size_t off_go = align_up(off_ow + 4 * T, A);
  const size_t off_pl = align_up(off_go + 4 * (G + 1), A);
  const size_t off_so = align_up(off_pl + 4 * G, A);
  const size_t off_sg = align_up(off_so + 4 * L->seg_off.size(), A);
  const size_t off_sl = align_up(off_sg + 4 * N, A);
  const size_t off_di = align_up(off_sl + 4 * N, A);
  const size_t off_dro = align_up(off_di + sizeof(pg_dec_item) * L->dec_items.size(), A);
  const size_t off_dr = align_up(off_dro + 4 * L->dec_ref_off.size(), A);
  const size_t bytes = align_up(off_dr + 4 * L->dec_refs.size(), A);
  hipError_t e = hipGetDevice(&L->device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  pg_slot* slot = nullptr;
  pg_status st = pg_slot_acquire(L->device, bytes, &slot);
  if (st != PG_OK) return st;
  unsigned char* h = slot->host;
  std::memcpy(h + off_g0, L->tok_g0.data(), 4 * T);
  std::memcpy(h + off_pe, L->tok_pe.data(), 4 * T);
  std::memcpy(h + off_ss, L->tok_ss.data(), 4 * T);
  if (!L->items.empty())
    std::memcpy(h + off_it, L->items.data(), sizeof(pg_work_item) * L->items.size());
  if (!L->spans.empty())
    std::memcpy(h + off_sp, L->spans.data(), sizeof(pg_key_span) * L->spans.size());
  std::memcpy(h + off_fr, L->inv_freq.data(), sizeof(double) * L->inv_freq.size());
  if (!L->kv_items.empty())
    std::memcpy(h + off_kv, L->kv_items.data(), sizeof(pg_kv_item) * L->kv_items.size());
  std::memcpy(h + off_ow, L->tok_owner.data(), 4 * T);
  std::memcpy(h + off_go, L->group_off.data(), 4 * (G + 1));
  if (G) std::memcpy(h + off_pl, L->prefix_lens.data(), 4 * G);
  std::memcpy(h + off_so, L->seg_off.data(), 4 * L->seg_off.size());
  if (N) {
    std::memcpy(h + off_sg, L->suffix_group.data(), 4 * N);
    std::memcpy(h + off_sl, L->suffix_lens.data(), 4 * N);
  }
  if (!L->dec_items.empty())
    std::memcpy(h + off_di, L->dec_items.data(), sizeof(pg_dec_item) * L->dec_items.size());
  if (!L->dec_ref_off.empty())
    std::memcpy(h + off_dro, L->dec_ref_off.data(), 4 * L->dec_ref_off.size());
  if (!L->dec_refs.empty())
    std::memcpy(h + off_dr, L->dec_refs.data(), 4 * L->dec_refs.size());
  void* d = slot->dev;
  e = hipMemcpyAsync(d, h, bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) {
    pg_slot_release(slot);
    return hip_fail(e, "hipMemcpyAsync");
  }
  pg_slot_note_use(slot, stream);
  L->slot = slot;
  unsigned char* b = static_cast<unsigned char*>(d);
  L->dev_buf = d;
  L->d_g0 = reinterpret_cast<const int32_t*>(b + off_g0);
  L->d_pe = reinterpret_cast<const int32_t*>(b + off_pe);
  L->d_ss = reinterpret_cast<const int32_t*>(b + off_ss);
  L->d_items = reinterpret_cast<const pg_work_item*>(b + off_it);
  L->d_spans = reinterpret_cast<const pg_key_span*>(b + off_sp);
  L->d_inv_freq = reinterpret_cast<const double*>(b + off_fr);
  L->d_kv_items = reinterpret_cast<const pg_kv_item*>(b + off_kv);
  L->d_owner = reinterpret_cast<const int32_t*>(b + off_ow);
  L->d_group_off = reinterpret_cast<const int32_t*>(b + off_go);
  L->d_prefix_lens = reinterpret_cast<const int32_t*>(b + off_pl);
  L->d_seg_off = reinterpret_cast<const int32_t*>(b + off_so);
  L->d_suffix_group = reinterpret_cast<const int32_t*>(b + off_sg);
  L->d_suffix_lens = reinterpret_cast<const int32_t*>(b + off_sl);
  L->d_dec_items = reinterpret_cast<const pg_dec_item*>(b + off_di);
  L->d_dec_ref_off = reinterpret_cast<const int32_t*>(b + off_dro);
  L->d_dec_refs = reinterpret_cast<const int32_t*>(b + off_dr);
  return PG_OK;
}

pg_status pg_build_layout(int32_t num_groups, const int32_t* prefix_lens,
                          const int32_t* suffix_counts, const int32_t* suffix_lens,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          double rope_theta, hipStream_t stream, pg_layout** out) {
  pg_status s = pg_build_layout_host(num_groups, prefix_lens, suffix_counts, suffix_lens,
                                     num_q_heads, num_kv_heads, head_dim, rope_theta, out);
  if (s != PG_OK) return s;
  s = pg_layout_upload(*out, stream);
  if (s != PG_OK) {
    pg_layout_destroy(*out);
    *out = nullptr;
  }
  return s;
}

pg_status pg_layout_info(const pg_layout* L, pg_layout_summary* info) {
  if (!L || !info) return pg_fail(PG_ERR_INVALID_ARG, "NULL argument");
  info->total_tokens = L->T;
  info->num_groups = L->G;
  info->num_segments = L->num_segments;
  info->max_position = L->max_position;
  info->num_items = int32_t(L->items.size());
  info->num_spans = int32_t(L->spans.size());
  info->block_tokens = L->block_tokens;
  info->heads_per_item = L->heads_per_item;
  info->device_ready = (L->dev_buf != nullptr || (L->T == 0 && L->device >= 0)) ? 1 : 0;
  info->useful_pairs = L->useful_pairs;
  info->unpacked_pairs = L->unpacked_pairs;
  info->max_item_cost = L->max_item_cost;
  info->max_xcd_cost = 0;
  for (int64_t c : L->xcd_load) info->max_xcd_cost = c > info->max_xcd_cost ? c : info->max_xcd_cost;
  info->num_kv_items = int32_t(L->kv_items.size());
  info->num_dec_items = int32_t(L->dec_items.size());
  info->num_dec_refs = int64_t(L->dec_refs.size());
  info->max_group_len = L->max_group_len;
  info->reserved = 0;
  return PG_OK;
}

pg_status pg_layout_copy_offsets(const pg_layout* L, int32_t* group_off, int32_t* seg_off) {
  if (!L) return pg_fail(PG_ERR_INVALID_ARG, "layout is NULL");
  if (group_off) std::memcpy(group_off, L->group_off.data(), 4 * L->group_off.size());
  if (seg_off) std::memcpy(seg_off, L->seg_off.data(), 4 * L->seg_off.size());
  return PG_OK;
}

pg_status pg_layout_copy_tokens(const pg_layout* L, int32_t* g0, int32_t* pe, int32_t* ss) {
  if (!L) return pg_fail(PG_ERR_INVALID_ARG, "layout is NULL");
  const size_t n = 4 * size_t(L->T);
  if (g0 && n) std::memcpy(g0, L->tok_g0.data(), n);
  if (pe && n) std::memcpy(pe, L->tok_pe.data(), n);
  if (ss && n) std::memcpy(ss, L->tok_ss.data(), n);
  return PG_OK;
}

pg_status pg_layout_copy_work(const pg_layout* L, pg_work_item* items, pg_key_span* spans) {
  if (!L) return pg_fail(PG_ERR_INVALID_ARG, "layout is NULL");
  if (items && !L->items.empty())
    std::memcpy(items, L->items.data(), sizeof(pg_work_item) * L->items.size());
  if (spans && !L->spans.empty())
    std::memcpy(spans, L->spans.data(), sizeof(pg_key_span) * L->spans.size());
  return PG_OK;
}

pg_status pg_layout_copy_kv_work(const pg_layout* L, pg_kv_item* items) {
  if (!L) return pg_fail(PG_ERR_INVALID_ARG, "layout is NULL");
  if (items && !L->kv_items.empty())
    std::memcpy(items, L->kv_items.data(), sizeof(pg_kv_item) * L->kv_items.size());
  return PG_OK;
}

pg_status pg_layout_copy_decode_work(const pg_layout* L, pg_dec_item* items, int32_t* ref_off,
                                     int32_t* refs) {
  if (!L) return pg_fail(PG_ERR_INVALID_ARG, "layout is NULL");
  if (items && !L->dec_items.empty())
    std::memcpy(items, L->dec_items.data(), sizeof(pg_dec_item) * L->dec_items.size());
  if (ref_off && !L->dec_ref_off.empty())
    std::memcpy(ref_off, L->dec_ref_off.data(), 4 * L->dec_ref_off.size());
  if (refs && !L->dec_refs.empty())
    std::memcpy(refs, L->dec_refs.data(), 4 * L->dec_refs.size());
  return PG_OK;
}

void pg_layout_destroy(pg_layout* L) {
  if (!L) return;
  pg_slot_release(L->slot);   // reused only after the enqueued work that reads it
  delete L;
}

pg_status pg_position_ids(const pg_layout* L, int64_t* pos, hipStream_t stream) {
  pg_status s = check_device_layout(L);
  if (s != PG_OK) return s;
  if (L->T == 0) return PG_OK;
  if (!pos) return pg_fail(PG_ERR_INVALID_ARG, "pos is NULL");
  hipError_t e = pg_launch_positions(*L, pos, stream);
  pg_slot_note_use(L->slot, stream);
  return e == hipSuccess ? PG_OK : hip_fail(e, "position-id kernel launch");
}

pg_status pg_rope(const pg_layout* L, const int64_t* pos, const void* q_in, const void* k_in,
                  void* q_out, void* k_out, pg_dtype dtype, hipStream_t stream) {
  pg_status s = check_device_layout(L);
  if (s != PG_OK) return s;
  if (dtype != PG_F32 && dtype != PG_BF16)
    return pg_fail(PG_ERR_UNSUPPORTED, "dtype %d not supported", int(dtype));
  if (L->T == 0) return PG_OK;
  if (!pos || (!q_in != !q_out) || (!k_in != !k_out) || (!q_in && !k_in))
    return pg_fail(PG_ERR_INVALID_ARG, "NULL tensor pointer (a pair may be skipped only whole)");
  hipError_t e = pg_launch_rope(*L, pos, q_in, k_in, q_out, k_out, dtype, stream);
  pg_slot_note_use(L->slot, stream);
  return e == hipSuccess ? PG_OK : hip_fail(e, "rope kernel launch");
}

pg_status pg_attn_fwd(const pg_layout* L, const void* q, const void* k, const void* v, void* o,
                      float* lse, pg_dtype dtype, float softmax_scale, hipStream_t stream) {
  pg_status s = check_device_layout(L);
  if (s != PG_OK) return s;
  if (dtype != PG_F32 && dtype != PG_BF16)
    return pg_fail(PG_ERR_UNSUPPORTED, "dtype %d not supported", int(dtype));
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return pg_fail(PG_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (L->T == 0) return PG_OK;
  if (!q || !k || !v || !o) return pg_fail(PG_ERR_INVALID_ARG, "NULL tensor pointer");
  hipError_t e;
  if (dtype == PG_BF16 && L->d == 128)
    e = pg_launch_attn_mfma(*L, q, k, v, o, lse, softmax_scale, stream);
  else
    e = pg_launch_attn_rowwise(*L, q, k, v, o, lse, dtype, softmax_scale, stream);
  pg_slot_note_use(L->slot, stream);
  return e == hipSuccess ? PG_OK : hip_fail(e, "attention kernel launch");
}

pg_status pg_attn_bwd(const pg_layout* L, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dout, void* dq, void* dk,
                      void* dv, float* delta, pg_dtype dtype, float softmax_scale,
                      hipStream_t stream) {
  pg_status s = check_device_layout(L);
  if (s != PG_OK) return s;
  if (dtype != PG_F32 && dtype != PG_BF16)
    return pg_fail(PG_ERR_UNSUPPORTED, "dtype %d not supported", int(dtype));
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return pg_fail(PG_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (L->T == 0) return PG_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta)
    return pg_fail(PG_ERR_INVALID_ARG, "NULL tensor pointer");
  if (dq == dk || dq == dv || dk == dv)
    return pg_fail(PG_ERR_INVALID_ARG, "dq, dk, dv must be distinct buffers");
  if (L->T * L->Hq > int64_t(0x7fffffff))
    return pg_fail(PG_ERR_INVALID_ARG, "too many query rows");
  hipError_t e;
  if (dtype == PG_BF16 && L->d == 128)
    e = pg_launch_attn_bwd(*L, q, k, v, o, lse, dout, dq, dk, dv, delta, softmax_scale, stream);
  else
    e = pg_launch_bwd_rowwise(*L, q, k, v, o, lse, dout, dq, dk, dv, delta, dtype, softmax_scale,
                              stream);
  pg_slot_note_use(L->slot, stream);
  return e == hipSuccess ? PG_OK : hip_fail(e, "backward kernel launch");
}

pg_status pg_decode_workspace_size(const pg_layout* L, size_t* bytes) {
  if (!L || !bytes) return pg_fail(PG_ERR_INVALID_ARG, "NULL argument");
  *bytes = pg_decode_workspace_bytes(*L);
  return PG_OK;
}

pg_status pg_attn_decode_noalloc(const pg_layout* L, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* cur_lens, void* o, float* lse,
                                 pg_dtype dtype, float softmax_scale, hipStream_t stream) {
  pg_status s = check_device_layout(L);
  if (s != PG_OK) return s;
  if (dtype != PG_BF16 && dtype != PG_F32) return pg_fail(PG_ERR_INVALID_ARG, "bad dtype %d", int(dtype));
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return pg_fail(PG_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  const int64_t N = int64_t(L->suffix_lens.size());
  if (N == 0) return PG_OK;
  if (!q || !o || !lse || !cur_lens) return pg_fail(PG_ERR_INVALID_ARG, "NULL tensor pointer");
  if (L->T > 0 && (!k_cache || !v_cache)) return pg_fail(PG_ERR_INVALID_ARG, "NULL cache pointer");
  if (N * L->Hq > int64_t(0x7fffffff)) return pg_fail(PG_ERR_INVALID_ARG, "too many query rows");
  void* scratch = nullptr;
  if (dtype == PG_BF16 && L->d == 128) {
    const size_t need = pg_decode_workspace_bytes(*L);
    if (need > size_t(PG_DECODE_SCRATCH_BYTES))
      return pg_fail(PG_ERR_INVALID_ARG,
                     "decode step needs %zu bytes of scratch, more than the %zu of the static "
                     "array (use pg_attn_decode with a workspace)",
                     need, size_t(PG_DECODE_SCRATCH_BYTES));
    hipError_t e = pg_decode_scratch(L->device, &scratch);
    if (e != hipSuccess) return hip_fail(e, "decode scratch address");
  }
  hipError_t e = pg_launch_attn_decode(*L, q, k_cache, v_cache, cur_lens, o, lse, scratch, dtype,
                                       softmax_scale, stream);
  pg_slot_note_use(L->slot, stream);
  return e == hipSuccess ? PG_OK : hip_fail(e, "decode kernel launch");
}

pg_status pg_attn_decode(const pg_layout* L, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* cur_lens, void* o, float* lse,
                         void* workspace, size_t workspace_bytes, pg_dtype dtype,
                         float softmax_scale, hipStream_t stream) {
  pg_status s = check_device_layout(L);
  if (s != PG_OK) return s;
  if (dtype != PG_BF16 && dtype != PG_F32) return pg_fail(PG_ERR_INVALID_ARG, "bad dtype %d", int(dtype));
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return pg_fail(PG_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  const int64_t N = int64_t(L->suffix_lens.size());
  if (N == 0) return PG_OK;
  if (!q || !o || !lse || !cur_lens) return pg_fail(PG_ERR_INVALID_ARG, "NULL tensor pointer");
  if (L->T > 0 && (!k_cache || !v_cache)) return pg_fail(PG_ERR_INVALID_ARG, "NULL cache pointer");
  const bool mfma = dtype == PG_BF16 && L->d == 128;
  if (mfma) {
    const size_t need = pg_decode_workspace_bytes(*L);
    if (need > 0 && (!workspace || workspace_bytes < need))
      return pg_fail(PG_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu needed",
                     workspace ? workspace_bytes : size_t(0), need);
  }
  if (N * L->Hq > int64_t(0x7fffffff)) return pg_fail(PG_ERR_INVALID_ARG, "too many query rows");
  hipError_t e = pg_launch_attn_decode(*L, q, k_cache, v_cache, cur_lens, o, lse, workspace, dtype,
                                       softmax_scale, stream);
  pg_slot_note_use(L->slot, stream);
  return e == hipSuccess ? PG_OK : hip_fail(e, "decode kernel launch");
}

namespace {
pg_status check_padded(const pg_layout* L, int32_t max_len) {
  pg_status s = check_device_layout(L);
  if (s != PG_OK) return s;
  if (max_len < L->max_group_len)
    return pg_fail(PG_ERR_INVALID_ARG, "max_len %d shorter than the longest group row %d", max_len,
                   L->max_group_len);
  return PG_OK;
}
pg_status check_row_bytes(int64_t row_bytes) {
  if (row_bytes <= 0 || row_bytes % 4 != 0)
    return pg_fail(PG_ERR_INVALID_ARG, "row_bytes %lld must be a positive multiple of 4",
                   (long long)row_bytes);
  return PG_OK;
}
}  // namespace

pg_status pg_position_ids_padded(const pg_layout* L, int32_t max_len, int64_t* pos, uint8_t* mask,
                                 hipStream_t stream) {
  pg_status s = check_padded(L, max_len);
  if (s != PG_OK) return s;
  const int64_t G = int64_t(L->group_off.size()) - 1;
  if (G * max_len == 0) return PG_OK;
  if (!pos) return pg_fail(PG_ERR_INVALID_ARG, "pos is NULL");
  hipError_t e = pg_launch_positions_padded(*L, max_len, pos, mask, stream);
  pg_slot_note_use(L->slot, stream);
  return e == hipSuccess ? PG_OK : hip_fail(e, "padded positions kernel launch");
}

pg_status pg_pad_rows(const pg_layout* L, const void* packed, int64_t row_bytes, void* padded,
                      int32_t max_len, hipStream_t stream) {
  pg_status s = check_padded(L, max_len);
  if (s == PG_OK) s = check_row_bytes(row_bytes);
  if (s != PG_OK) return s;
  const int64_t G = int64_t(L->group_off.size()) - 1;
  if (G * max_len == 0) return PG_OK;
  if (!padded || (L->T > 0 && !packed)) return pg_fail(PG_ERR_INVALID_ARG, "NULL tensor pointer");
  hipError_t e = pg_launch_pad(*L, packed, row_bytes, padded, max_len, stream);
  pg_slot_note_use(L->slot, stream);
  return e == hipSuccess ? PG_OK : hip_fail(e, "pad kernel launch");
}

pg_status pg_unpad_rows(const pg_layout* L, const void* padded, int32_t max_len, int64_t row_bytes,
                        void* packed, hipStream_t stream) {
  pg_status s = check_padded(L, max_len);
  if (s == PG_OK) s = check_row_bytes(row_bytes);
  if (s != PG_OK) return s;
  if (L->T == 0) return PG_OK;
  if (!padded || !packed) return pg_fail(PG_ERR_INVALID_ARG, "NULL tensor pointer");
  hipError_t e = pg_launch_unpad(*L, padded, max_len, row_bytes, packed, stream);
  pg_slot_note_use(L->slot, stream);
  return e == hipSuccess ? PG_OK : hip_fail(e, "unpad kernel launch");
}

pg_status pg_pack_rows(const pg_layout* L, const void* prefix, int32_t prefix_pad,
                       const void* suffix, int32_t suffix_pad, void* packed, int64_t row_bytes,
                       hipStream_t stream) {
  pg_status s = check_device_layout(L);
  if (s != PG_OK) return s;
  if (row_bytes <= 0 || row_bytes % 4 != 0)
    return pg_fail(PG_ERR_INVALID_ARG, "row_bytes %lld must be a positive multiple of 4",
                   (long long)row_bytes);
  if (prefix_pad < L->max_prefix_len || suffix_pad < L->max_suffix_len)
    return pg_fail(PG_ERR_INVALID_ARG, "padding (%d, %d) shorter than the longest prompt %d / response %d",
                   prefix_pad, suffix_pad, L->max_prefix_len, L->max_suffix_len);
  if (L->T == 0) return PG_OK;
  if (!packed || (L->max_prefix_len > 0 && !prefix) || (L->max_suffix_len > 0 && !suffix))
    return pg_fail(PG_ERR_INVALID_ARG, "NULL tensor pointer");
  hipError_t e = pg_launch_pack(*L, prefix, prefix_pad, suffix, suffix_pad, packed, row_bytes, stream);
  pg_slot_note_use(L->slot, stream);
  return e == hipSuccess ? PG_OK : hip_fail(e, "pack kernel launch");
}

pg_status pg_unpack_rows(const pg_layout* L, const void* packed, int64_t row_bytes,
                         void* prefix_out, int32_t prefix_pad, void* suffix_out, int32_t suffix_pad,
                         hipStream_t stream) {
  pg_status s = check_device_layout(L);
  if (s != PG_OK) return s;
  if (row_bytes <= 0 || row_bytes % 4 != 0)
    return pg_fail(PG_ERR_INVALID_ARG, "row_bytes %lld must be a positive multiple of 4",
                   (long long)row_bytes);
  if ((prefix_out && prefix_pad < L->max_prefix_len) || (suffix_out && suffix_pad < L->max_suffix_len))
    return pg_fail(PG_ERR_INVALID_ARG, "padding (%d, %d) shorter than the longest prompt %d / response %d",
                   prefix_pad, suffix_pad, L->max_prefix_len, L->max_suffix_len);
  if (prefix_pad < 0 || suffix_pad < 0) return pg_fail(PG_ERR_INVALID_ARG, "negative padding");
  if ((prefix_out || suffix_out) && L->T > 0 && !packed)
    return pg_fail(PG_ERR_INVALID_ARG, "packed is NULL");
  hipError_t e = pg_launch_unpack(*L, packed, row_bytes, prefix_out, prefix_pad, suffix_out,
                                  suffix_pad, stream);
  pg_slot_note_use(L->slot, stream);
  return e == hipSuccess ? PG_OK : hip_fail(e, "unpack kernel launch");
}

}  // extern "C"
