// C ABI of the verification library: host-side validation and launch order.
// Every entry point checks its arguments, returns a status (never aborts)
// and only enqueues kernels on the caller's stream.

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "internal.h"
#include "spec_verify.h"

namespace {

thread_local std::string g_last_error;

sv_status fail(sv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sv_status ok() {
  g_last_error.clear();
  return SV_OK;
}

sv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

sv_status check_batch(const sv_batch* b, const char* who) {
  if (!b) return fail(SV_EINVAL, "%s: batch is null", who);
  if (b->B < 1) return fail(SV_EINVAL, "%s: B must be >= 1 (got %d)", who, b->B);
  if (b->max_T < 1 || b->max_T > sv::kMaxT)
    return fail(SV_ECAPACITY, "%s: max_T must be in 1..%d (got %d)", who, sv::kMaxT, b->max_T);
  if (b->total_T < b->B || static_cast<long long>(b->total_T) > static_cast<long long>(b->B) * b->max_T)
    return fail(SV_EINVAL, "%s: total_T=%d inconsistent with B=%d, max_T=%d", who, b->total_T,
                b->B, b->max_T);
  if (!b->cu_seqlens) return fail(SV_EINVAL, "%s: cu_seqlens is null", who);
  return SV_OK;
}

sv_status check_attn(const sv_batch* batch, const void* q, const void* k_new, const void* v_new,
                     void* k_cache, void* v_cache, const int32_t* block_table,
                     int32_t max_pages, int32_t num_pages, int32_t P, const int32_t* ctx_lens,
                     void* out, int32_t Hq, int32_t Hkv, int32_t D, sv_dtype dtype,
                     const char* who = "spec_verify_attention") {
  sv_status st = check_batch(batch, who);
  if (st != SV_OK) return st;
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !block_table || !ctx_lens || !out)
    return fail(SV_EINVAL, "%s: a required pointer is null", who);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(SV_EINVAL, "%s: Hq=%d must be a positive multiple of Hkv=%d", who, Hq, Hkv);
  if (P < 1 || max_pages < 1 || num_pages < 1)
    return fail(SV_EINVAL, "%s: page_size, max_pages_per_seq, num_pages must be >= 1", who);
  if (dtype == SV_BF16) {
    if (D != 64 && D != 128) return fail(SV_EDTYPE, "%s: bf16 path needs D in {64,128} (got %d)", who, D);
    if (P < 16 || (P & (P - 1)) != 0)
      return fail(SV_EINVAL, "%s: page_size %d must be a power of two >= 16", who, P);
    if (batch->B > 2048)
      return fail(SV_ECAPACITY, "%s: the bf16 path takes at most 2048 sequences (got %d)", who,
                  batch->B);
    if ((Hq / Hkv) * batch->max_T > 64)
      return fail(SV_ECAPACITY, "%s: (Hq/Hkv)*max_T = %d exceeds 64 query rows", who,
                  (Hq / Hkv) * batch->max_T);
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_new) |
         reinterpret_cast<uintptr_t>(v_new) | reinterpret_cast<uintptr_t>(k_cache) |
         reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(out)) & 15)
      return fail(SV_EINVAL, "%s: bf16 tensors must be 16-byte aligned", who);
  } else if (dtype == SV_F32) {
    if (D < 1 || D > 128) return fail(SV_EDTYPE, "%s: fp32 path needs 1 <= D <= 128 (got %d)", who, D);
  } else {
    return fail(SV_EDTYPE, "%s: unsupported dtype %d", who, static_cast<int>(dtype));
  }
  return SV_OK;
}

// The checks of spec_verify_attention_kv8 beyond those of the bf16 path.
sv_status check_attn_kv8(const float* k_scale, const float* v_scale, const char* who) {
  if (!k_scale || !v_scale) return fail(SV_EINVAL, "%s: k_scale and v_scale are required", who);
  if ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 15)
    return fail(SV_EINVAL, "%s: scales must be 16-byte aligned", who);
  return SV_OK;
}

sv_status check_attn_workspace(const sv_batch* batch, int32_t Hq, int32_t Hkv, int32_t D,
                               int32_t max_pages, int32_t P, sv_dtype dtype,
                               const void* workspace, size_t workspace_bytes, const char* who) {
  const size_t need =
      sv::attn_workspace_bytes(batch->B, batch->total_T, Hq, Hkv, D, max_pages, P, dtype);
  if (need && (!workspace || workspace_bytes < need))
    return fail(SV_EWORKSPACE, "%s: workspace needs %zu bytes (got %zu)", who, need,
                workspace ? workspace_bytes : size_t(0));
  return SV_OK;
}

sv::AttnArgs make_attn_args(const sv_batch* batch, const void* q, const void* k_new,
                            const void* v_new, void* k_cache, void* v_cache,
                            const int32_t* block_table, int32_t max_pages, int32_t num_pages,
                            int32_t P, const int32_t* ctx_lens, void* out, int32_t Hq,
                            int32_t Hkv, int32_t D, sv_dtype dtype, float scale, int32_t write_kv,
                            void* ws, int32_t* err, const float* k_scale = nullptr,
                            const float* v_scale = nullptr) {
  sv::AttnArgs a{};
  a.B = batch->B;
  a.total_T = batch->total_T;
  a.max_T = batch->max_T;
  a.cu = batch->cu_seqlens;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.P = P;
  a.ctx_lens = ctx_lens;
  a.out = out;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.scale = scale == 0.f ? 1.f / std::sqrt(static_cast<float>(D)) : scale;
  a.write_kv = write_kv ? 1 : 0;
  a.err = err;
  a.kv8 = k_scale != nullptr;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  if (dtype == SV_BF16) {
    a.n_wg = sv::attn_stream_grid(D, Hq / Hkv, a.max_T, a.kv8 != 0);
    sv::attn_workspace_carve(ws, a.B, Hkv, D, a.n_wg, &a.seg_meta, &a.part_o, &a.part_ml);
  }
  return a;
}

// true for a pointer the 16-byte vector loads cannot take (null passes)
bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

sv_status check_gdn_common(const sv_batch* batch, void* state, sv_dtype state_dtype,
                           int32_t num_slots, sv_dtype io_dtype, int32_t H, int32_t dk,
                           int32_t dv, const char* who) {
  sv_status st = check_batch(batch, who);
  if (st != SV_OK) return st;
  if (!state) return fail(SV_EINVAL, "%s: state is null", who);
  if (state_dtype != SV_F32 && state_dtype != SV_F16)
    return fail(SV_EDTYPE, "%s: unsupported state dtype %d", who, static_cast<int>(state_dtype));
  if (num_slots < 1) return fail(SV_EINVAL, "%s: num_slots must be >= 1", who);
  if (io_dtype != SV_F32 && io_dtype != SV_BF16)
    return fail(SV_EDTYPE, "%s: unsupported io dtype %d", who, static_cast<int>(io_dtype));
  if (dk != 64 && dk != 128) return fail(SV_EDTYPE, "%s: dk must be 64 or 128 (got %d)", who, dk);
  if (dv < 64 || dv > 256 || dv % 64 != 0)
    return fail(SV_EDTYPE, "%s: dv must be a multiple of 64 up to 256 (got %d)", who, dv);
  if (H < 1) return fail(SV_EINVAL, "%s: H must be >= 1", who);
  if (reinterpret_cast<uintptr_t>(state) & 15)
    return fail(SV_EINVAL, "%s: state must be 16-byte aligned", who);
  return SV_OK;
}

// Every acceptance argument except the workspace.
sv_status check_accept_args(const sv_batch* batch, const sv_accept_args* acc,
                            const int32_t* result, const char* who) {
  sv_status st = check_batch(batch, who);
  if (st != SV_OK) return st;
  const sv_accept_mode mode = acc->mode;
  if (mode != SV_ACCEPT_GREEDY && mode != SV_ACCEPT_REJECTION)
    return fail(SV_EINVAL, "%s: unknown mode %d", who, static_cast<int>(mode));
  if (acc->logit_dtype != SV_F32 && acc->logit_dtype != SV_BF16)
    return fail(SV_EDTYPE, "%s: unsupported logit dtype %d", who,
                static_cast<int>(acc->logit_dtype));
  const int32_t V = acc->V;
  if (V < 1) return fail(SV_EINVAL, "%s: V must be >= 1", who);
  if (!acc->target_logits || !result)
    return fail(SV_EINVAL, "%s: target_logits and result are required", who);
  if (batch->total_T > batch->B && !acc->draft_tokens)
    return fail(SV_EINVAL, "%s: draft_tokens is required when there are drafts", who);
  if (mode == SV_ACCEPT_REJECTION &&
      (!acc->u_final || (batch->total_T > batch->B && !acc->u_accept)))
    return fail(SV_EINVAL, "%s: rejection needs u_accept and u_final", who);
  return SV_OK;
}

sv_status check_accept(const sv_batch* batch, const sv_accept_args* acc, const int32_t* result,
                       const void* workspace, size_t workspace_bytes, const char* who) {
  sv_status st = check_accept_args(batch, acc, result, who);
  if (st != SV_OK) return st;
  const size_t need = sv::accept_workspace_bytes(batch->B, batch->total_T, acc->V, acc->mode);
  if (!workspace || workspace_bytes < need)
    return fail(SV_EWORKSPACE, "%s: workspace needs %zu bytes (got %zu)", who, need,
                workspace ? workspace_bytes : size_t(0));
  return SV_OK;
}

sv_status check_gdn_call(const sv_batch* batch, sv_gdn_mode mode, const void* state,
                         sv_dtype state_dtype, const int32_t* state_slot, int32_t num_slots,
                         const void* q, const void* k, const void* v, sv_dtype io_dtype,
                         const float* alpha, const float* beta, const int32_t* commit_len,
                         const void* out, int32_t H, int32_t dk, int32_t dv,
                         const sv_gdn_pending* pending, const char* who) {
  sv_status st = check_gdn_common(batch, const_cast<void*>(state), state_dtype, num_slots,
                                  io_dtype, H, dk, dv, who);
  if (st != SV_OK) return st;
  if (mode != SV_GDN_VERIFY_COMMIT && mode != SV_GDN_VERIFY_ONLY && mode != SV_GDN_COMMIT_ONLY)
    return fail(SV_EINVAL, "%s: unknown mode %d", who, static_cast<int>(mode));
  if (!k || !v || !alpha || !beta) return fail(SV_EINVAL, "%s: k, v, alpha, beta are required", who);
  if (mode != SV_GDN_COMMIT_ONLY && (!q || !out))
    return fail(SV_EINVAL, "%s: q and out are required unless COMMIT_ONLY", who);
  if (mode != SV_GDN_VERIFY_ONLY && !commit_len)
    return fail(SV_EINVAL, "%s: commit_len is required unless VERIFY_ONLY", who);
  if (!state_slot && num_slots < batch->B)
    return fail(SV_EINVAL, "%s: without state_slot, num_slots must be >= B", who);
  if (misaligned16(q) || misaligned16(k) || misaligned16(v) ||
      (pending && (misaligned16(pending->k) || misaligned16(pending->v))))
    return fail(SV_EINVAL, "%s: q, k, v must be 16-byte aligned", who);
  if (pending) {
    st = check_batch(&pending->batch, who);
    if (st != SV_OK) return st;
    if (pending->batch.B != batch->B)
      return fail(SV_EINVAL, "%s: pending batch has B=%d, this batch B=%d", who,
                  pending->batch.B, batch->B);
    if (!pending->k || !pending->v || !pending->alpha || !pending->beta || !pending->commit_len)
      return fail(SV_EINVAL, "%s: pending k, v, alpha, beta, commit_len are required", who);
  }
  return SV_OK;
}

sv_status launch_accept_checked(const sv_batch* batch, const sv_accept_args* acc,
                                int32_t* result, int32_t* commit_len_out,
                                int32_t* ctx_lens_inout, void* workspace, int32_t* err,
                                hipStream_t stream, const char* who);

sv_status accept_impl(const sv_batch* batch, const sv_accept_args* acc, int32_t* result,
                      int32_t* commit_len_out, int32_t* ctx_lens_inout, void* workspace,
                      size_t workspace_bytes, int32_t* err, hipStream_t stream, const char* who) {
  sv_status st = check_accept(batch, acc, result, workspace, workspace_bytes, who);
  if (st != SV_OK) return st;
  return launch_accept_checked(batch, acc, result, commit_len_out, ctx_lens_inout, workspace,
                               err, stream, who);
}

sv_status launch_accept_checked(const sv_batch* batch, const sv_accept_args* acc,
                                int32_t* result, int32_t* commit_len_out,
                                int32_t* ctx_lens_inout, void* workspace, int32_t* err,
                                hipStream_t stream, const char* who) {
  const sv_accept_mode mode = acc->mode;
  const int32_t V = acc->V;
  sv::AcceptArgs a{};
  a.B = batch->B;
  a.total_T = batch->total_T;
  a.max_T = batch->max_T;
  a.cu = batch->cu_seqlens;
  a.mode = mode;
  a.target = acc->target_logits;
  a.draft = mode == SV_ACCEPT_REJECTION ? acc->draft_logits : nullptr;
  a.V = V;
  a.draft_tokens = acc->draft_tokens;
  a.u_accept = acc->u_accept;
  a.u_final = acc->u_final;
  a.bonus = acc->bonus_tokens;
  a.result = result;
  a.commit_len_out = commit_len_out;
  a.ctx_lens = ctx_lens_inout;
  a.err = err;
  a.ws = workspace;
  return hip_status(sv::launch_accept(a, acc->logit_dtype, stream), who);
}

}  // namespace

extern "C" {

const char* sv_last_error(void) { return g_last_error.c_str(); }

const char* sv_version(void) { return "specverify 0.2 gfx950"; }

int32_t sv_read_device_error(const int32_t* err, hipStream_t stream) {
  if (!err) {
    fail(SV_EINVAL, "sv_read_device_error: err is null");
    return -1;
  }
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, err, sizeof(v), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    hip_status(e, "sv_read_device_error");
    return -1;
  }
  ok();
  return v;
}

sv_status sv_clear_device_error(int32_t* err, hipStream_t stream) {
  if (!err) return fail(SV_EINVAL, "sv_clear_device_error: err is null");
  return hip_status(sv::launch_fill_i32(err, 1, 0, stream), "sv_clear_device_error");
}

size_t sv_workspace_bytes(int32_t B, int32_t max_T, int32_t Hq, int32_t D, int32_t V,
                          int32_t max_pages_per_seq) {
  if (B < 1 || max_T < 1 || max_T > sv::kMaxT || Hq < 1 || D < 1 || V < 1 ||
      max_pages_per_seq < 1)
    return 0;
  const int32_t total_T = B * max_T;
  // the attention workspace grows with the KV heads: Hq bounds them
  size_t need = sv::attn_workspace_bytes(B, total_T, Hq, Hq, D, max_pages_per_seq, 16, SV_BF16);
  need = std::max(need, sv::accept_workspace_bytes(B, total_T, V, SV_ACCEPT_GREEDY));
  need = std::max(need, sv::accept_workspace_bytes(B, total_T, V, SV_ACCEPT_REJECTION));
  return need;
}

size_t spec_verify_attention_workspace_bytes(int32_t B, int32_t total_T, int32_t Hq, int32_t Hkv,
                                             int32_t D, int32_t max_pages_per_seq,
                                             int32_t page_size, sv_dtype dtype) {
  if (B < 1 || total_T < 1 || Hq < 1 || Hkv < 1 || D < 1 || max_pages_per_seq < 1 || page_size < 1)
    return 0;
  return sv::attn_workspace_bytes(B, total_T, Hq, Hkv, D, max_pages_per_seq, page_size, dtype);
}

sv_status spec_verify_attention(const sv_batch* batch, const void* q, const void* k_new,
                                const void* v_new, void* k_cache, void* v_cache,
                                const int32_t* block_table, int32_t max_pages_per_seq,
                                int32_t num_pages, int32_t page_size, const int32_t* ctx_lens,
                                void* out, int32_t Hq, int32_t Hkv, int32_t D, sv_dtype dtype,
                                float scale, int32_t write_kv, void* workspace,
                                size_t workspace_bytes, int32_t* err, hipStream_t stream) {
  sv_status st = check_attn(batch, q, k_new, v_new, k_cache, v_cache, block_table,
                            max_pages_per_seq, num_pages, page_size, ctx_lens, out, Hq, Hkv, D,
                            dtype);
  if (st != SV_OK) return st;
  st = check_attn_workspace(batch, Hq, Hkv, D, max_pages_per_seq, page_size, dtype, workspace,
                            workspace_bytes, "spec_verify_attention");
  if (st != SV_OK) return st;
  sv::AttnArgs a = make_attn_args(batch, q, k_new, v_new, k_cache, v_cache, block_table,
                                  max_pages_per_seq, num_pages, page_size, ctx_lens, out, Hq, Hkv,
                                  D, dtype, scale, write_kv, workspace, err);
  return hip_status(sv::launch_attention(a, dtype, stream), "spec_verify_attention");
}

sv_status spec_verify_attention_kv8(const sv_batch* batch, const void* q, const void* k_new,
                                    const void* v_new, int8_t* k_cache, int8_t* v_cache,
                                    const float* k_scale, const float* v_scale,
                                    const int32_t* block_table, int32_t max_pages_per_seq,
                                    int32_t num_pages, int32_t page_size,
                                    const int32_t* ctx_lens, void* out, int32_t Hq, int32_t Hkv,
                                    int32_t D, float scale, void* workspace,
                                    size_t workspace_bytes, int32_t* err, hipStream_t stream) {
  const char* who = "spec_verify_attention_kv8";
  sv_status st = check_attn(batch, q, k_new, v_new, k_cache, v_cache, block_table,
                            max_pages_per_seq, num_pages, page_size, ctx_lens, out, Hq, Hkv, D,
                            SV_BF16, who);
  if (st != SV_OK) return st;
  st = check_attn_kv8(k_scale, v_scale, who);
  if (st != SV_OK) return st;
  st = check_attn_workspace(batch, Hq, Hkv, D, max_pages_per_seq, page_size, SV_BF16, workspace,
                            workspace_bytes, who);
  if (st != SV_OK) return st;
  sv::AttnArgs a = make_attn_args(batch, q, k_new, v_new, k_cache, v_cache, block_table,
                                  max_pages_per_seq, num_pages, page_size, ctx_lens, out, Hq, Hkv,
                                  D, SV_BF16, scale, 1, workspace, err, k_scale, v_scale);
  return hip_status(sv::launch_attention(a, SV_BF16, stream), who);
}

sv_status gdn_verify_commit(const sv_batch* batch, sv_gdn_mode mode, void* state,
                            sv_dtype state_dtype, const int32_t* state_slot, int32_t num_slots,
                            const void* q,
                            const void* k, const void* v, sv_dtype io_dtype, const float* alpha,
                            const float* beta, const int32_t* commit_len, void* out, int32_t H,
                            int32_t dk, int32_t dv, const sv_gdn_pending* pending, int32_t* err,
                            hipStream_t stream) {
  const char* who = "gdn_verify_commit";
  sv_status st = check_gdn_call(batch, mode, state, state_dtype, state_slot, num_slots, q, k, v,
                                io_dtype, alpha, beta, commit_len, out, H, dk, dv, pending, who);
  if (st != SV_OK) return st;
  sv::GdnScalars s{};
  s.B = batch->B;
  s.total_T = batch->total_T;
  s.max_T = batch->max_T;
  s.cu = batch->cu_seqlens;
  s.mode = mode;
  s.state_slot = state_slot;
  s.num_slots = num_slots;
  s.commit_len = commit_len;
  s.H = H;
  s.dk = dk;
  s.dv = dv;
  s.err = err;
  sv::GdnFullPtrs p{};
  p.state = state;
  p.q = q;
  p.k = k;
  p.v = v;
  p.alpha = alpha;
  p.beta = beta;
  p.out = out;
  if (pending) {
    s.has_pending = 1;
    s.p_total_T = pending->batch.total_T;
    s.p_max_T = pending->batch.max_T;
    s.p_cu = pending->batch.cu_seqlens;
    s.p_commit = pending->commit_len;
    p.pk = pending->k;
    p.pv = pending->v;
    p.palpha = pending->alpha;
    p.pbeta = pending->beta;
  }
  return hip_status(sv::launch_gdn(s, p, io_dtype, state_dtype, stream), who);
}

sv_status short_conv_verify_commit(const sv_batch* batch, sv_gdn_mode mode, void* state,
                                   const int32_t* state_slot, int32_t num_slots, const void* x,
                                   const float* weight, const float* bias, sv_dtype io_dtype,
                                   int32_t activation, const int32_t* commit_len, void* out,
                                   int32_t C, int32_t K, const sv_conv_pending* pending,
                                   int32_t* err, hipStream_t stream) {
  const char* who = "short_conv_verify_commit";
  sv_status st = check_batch(batch, who);
  if (st != SV_OK) return st;
  if (mode != SV_GDN_VERIFY_COMMIT && mode != SV_GDN_VERIFY_ONLY && mode != SV_GDN_COMMIT_ONLY)
    return fail(SV_EINVAL, "%s: unknown mode %d", who, static_cast<int>(mode));
  if (io_dtype != SV_F32 && io_dtype != SV_BF16)
    return fail(SV_EDTYPE, "%s: unsupported io dtype %d", who, static_cast<int>(io_dtype));
  if (K < 2 || K > 8) return fail(SV_EINVAL, "%s: K must be in 2..8 (got %d)", who, K);
  if (C < 1) return fail(SV_EINVAL, "%s: C must be >= 1", who);
  if (activation != SV_ACT_NONE && activation != SV_ACT_SILU)
    return fail(SV_EINVAL, "%s: unknown activation %d", who, activation);
  if (!state || !x || !weight) return fail(SV_EINVAL, "%s: state, x and weight are required", who);
  if (num_slots < 1) return fail(SV_EINVAL, "%s: num_slots must be >= 1", who);
  if (!state_slot && num_slots < batch->B)
    return fail(SV_EINVAL, "%s: without state_slot, num_slots must be >= B", who);
  if (mode != SV_GDN_COMMIT_ONLY && !out)
    return fail(SV_EINVAL, "%s: out is required unless COMMIT_ONLY", who);
  if (mode != SV_GDN_VERIFY_ONLY && !commit_len)
    return fail(SV_EINVAL, "%s: commit_len is required unless VERIFY_ONLY", who);
  sv::ConvArgs a{};
  a.B = batch->B;
  a.total_T = batch->total_T;
  a.max_T = batch->max_T;
  a.cu = batch->cu_seqlens;
  a.mode = mode;
  a.state_slot = state_slot;
  a.num_slots = num_slots;
  a.commit_len = commit_len;
  a.C = C;
  a.K = K;
  a.activation = activation;
  a.state = state;
  a.x = x;
  a.weight = weight;
  a.bias = bias;
  a.out = out;
  a.err = err;
  if (pending) {
    st = check_batch(&pending->batch, "short_conv_verify_commit (pending)");
    if (st != SV_OK) return st;
    if (pending->batch.B != batch->B)
      return fail(SV_EINVAL, "%s: pending batch has B=%d, this batch B=%d", who,
                  pending->batch.B, batch->B);
    if (!pending->x || !pending->commit_len)
      return fail(SV_EINVAL, "%s: pending x and commit_len are required", who);
    a.has_pending = 1;
    a.p_total_T = pending->batch.total_T;
    a.p_max_T = pending->batch.max_T;
    a.p_cu = pending->batch.cu_seqlens;
    a.p_commit = pending->commit_len;
    a.px = pending->x;
  }
  return hip_status(sv::launch_conv(a, io_dtype, stream), who);
}

namespace {

constexpr int32_t kMaxWindow = 64;  // checkpoint slots per sequence

sv_status check_window(const sv_batch* batch, int32_t window, const char* who) {
  if (window < batch->max_T || window > kMaxWindow)
    return fail(SV_EINVAL, "%s: window must be in max_T..%d (got %d, max_T %d)", who, kMaxWindow,
                window, batch->max_T);
  return SV_OK;
}

sv::GdnScalars gdn_scalars(const sv_batch* batch, int mode, const int32_t* state_slot,
                           int32_t num_slots, const int32_t* commit_len, int32_t H, int32_t dk,
                           int32_t dv, int32_t window, int32_t* err) {
  sv::GdnScalars s{};
  s.B = batch->B;
  s.total_T = batch->total_T;
  s.max_T = batch->max_T;
  s.cu = batch->cu_seqlens;
  s.mode = mode;
  s.state_slot = state_slot;
  s.num_slots = num_slots;
  s.commit_len = commit_len;
  s.H = H;
  s.dk = dk;
  s.dv = dv;
  s.window = window;
  s.err = err;
  return s;
}

sv_status check_conv_common(const sv_batch* batch, const void* state, const int32_t* state_slot,
                            int32_t num_slots, sv_dtype io_dtype, int32_t C, int32_t K,
                            const char* who) {
  sv_status st = check_batch(batch, who);
  if (st != SV_OK) return st;
  if (io_dtype != SV_F32 && io_dtype != SV_BF16)
    return fail(SV_EDTYPE, "%s: unsupported io dtype %d", who, static_cast<int>(io_dtype));
  if (K < 2 || K > 8) return fail(SV_EINVAL, "%s: K must be in 2..8 (got %d)", who, K);
  if (C < 1) return fail(SV_EINVAL, "%s: C must be >= 1", who);
  if (!state) return fail(SV_EINVAL, "%s: state is required", who);
  if (num_slots < 1) return fail(SV_EINVAL, "%s: num_slots must be >= 1", who);
  if (!state_slot && num_slots < batch->B)
    return fail(SV_EINVAL, "%s: without state_slot, num_slots must be >= B", who);
  return SV_OK;
}

// The short convolution of a GDN layer inside the step.
sv_status check_step_conv(const sv_batch* batch, const sv_gdn_config* g, const sv_gdn_layer& L,
                          const sv_gdn_layer* P, const char* who) {
  if (g->conv_C < 1) return SV_OK;
  if (g->conv_K < 2 || g->conv_K > 8)
    return fail(SV_EINVAL, "%s: conv_K must be in 2..8 (got %d)", who, g->conv_K);
  if (g->conv_activation != SV_ACT_NONE && g->conv_activation != SV_ACT_SILU)
    return fail(SV_EINVAL, "%s: unknown conv activation %d", who, g->conv_activation);
  if (!L.conv_state || !L.conv_x || !L.conv_out || !L.conv_weight)
    return fail(SV_EINVAL, "%s: conv_state, conv_x, conv_out and conv_weight are required", who);
  if (P && !P->conv_x) return fail(SV_EINVAL, "%s: the pending conv_x is required", who);
  (void)batch;
  return SV_OK;
}

sv::ConvArgs step_conv_args(const sv_batch* batch, const sv_gdn_config* g, int mode,
                            const int32_t* commit_len, int32_t* err) {
  sv::ConvArgs a{};
  a.B = batch->B;
  a.total_T = batch->total_T;
  a.max_T = batch->max_T;
  a.cu = batch->cu_seqlens;
  a.mode = mode;
  a.state_slot = g->state_slot;
  a.num_slots = g->num_slots;
  a.commit_len = commit_len;
  a.C = g->conv_C;
  a.K = g->conv_K;
  a.activation = g->conv_activation;
  a.err = err;
  return a;
}

// COMMIT_ONLY of the first commit_len[b] tokens of every layer (and its short
// convolution when gcfg->conv_C > 0) in batched launches; arguments checked.
sv_status commit_layers(const sv_batch* batch, const sv_gdn_config* gcfg,
                        const sv_gdn_layer* layers, int n_gdn, const int32_t* commit_len,
                        int32_t* err, hipStream_t stream, const char* who) {
  sv::GdnScalars s{};
  s.B = batch->B;
  s.total_T = batch->total_T;
  s.max_T = batch->max_T;
  s.cu = batch->cu_seqlens;
  s.mode = SV_GDN_COMMIT_ONLY;
  s.state_slot = gcfg->state_slot;
  s.num_slots = gcfg->num_slots;
  s.commit_len = commit_len;
  s.H = gcfg->H;
  s.dk = gcfg->dk;
  s.dv = gcfg->dv;
  s.err = err;
  for (int l0 = 0; l0 < n_gdn; l0 += sv::kGdnLayersPerLaunch) {
    const int nl = std::min(sv::kGdnLayersPerLaunch, n_gdn - l0);
    sv::GdnCommitTable t{};
    for (int i = 0; i < nl; ++i) {
      const sv_gdn_layer& G = layers[l0 + i];
      t.l[i] = sv::GdnCommitPtrs{G.state, G.k, G.v, G.alpha, G.beta};
      t.c[i] = sv::ConvCommitPtrs{G.conv_state, G.conv_x};
    }
    const sv::ConvArgs c = step_conv_args(batch, gcfg, SV_GDN_COMMIT_ONLY, commit_len, err);
    const sv_status st =
        hip_status(sv::launch_gdn_commit_multi(s, t, nl, gcfg->io_dtype, gcfg->state_dtype, stream,
                                               gcfg->conv_C > 0 ? &c : nullptr),
                   who);
    if (st != SV_OK) return st;
  }
  return SV_OK;
}

}  // namespace

sv_status gdn_verify_checkpoint(const sv_batch* batch, const void* state, sv_dtype state_dtype,
                                const int32_t* state_slot, int32_t num_slots, const void* q,
                                const void* k, const void* v, sv_dtype io_dtype,
                                const float* alpha, const float* beta, void* out,
                                void* checkpoints, int32_t window, int32_t H, int32_t dk,
                                int32_t dv, int32_t* err, hipStream_t stream) {
  const char* who = "gdn_verify_checkpoint";
  sv_status st = check_gdn_common(batch, const_cast<void*>(state), state_dtype, num_slots,
                                  io_dtype, H, dk, dv, who);
  if (st != SV_OK) return st;
  st = check_window(batch, window, who);
  if (st != SV_OK) return st;
  if (!q || !k || !v || !alpha || !beta || !out || !checkpoints)
    return fail(SV_EINVAL, "%s: q, k, v, alpha, beta, out and checkpoints are required", who);
  if (reinterpret_cast<uintptr_t>(checkpoints) & 15)
    return fail(SV_EINVAL, "%s: checkpoints must be 16-byte aligned", who);
  if (misaligned16(q) || misaligned16(k) || misaligned16(v))
    return fail(SV_EINVAL, "%s: q, k, v must be 16-byte aligned", who);
  if (!state_slot && num_slots < batch->B)
    return fail(SV_EINVAL, "%s: without state_slot, num_slots must be >= B", who);
  const sv::GdnScalars s = gdn_scalars(batch, SV_GDN_VERIFY_ONLY, state_slot, num_slots, nullptr,
                                       H, dk, dv, window, err);
  sv::GdnFullPtrs p{};
  p.state = const_cast<void*>(state);  // read only: VERIFY_ONLY without pending tokens
  p.q = q;
  p.k = k;
  p.v = v;
  p.alpha = alpha;
  p.beta = beta;
  p.out = out;
  p.ckpt = checkpoints;
  return hip_status(sv::launch_gdn(s, p, io_dtype, state_dtype, stream), who);
}

sv_status gdn_commit_prefix(const sv_batch* batch, void* state, sv_dtype state_dtype,
                            const int32_t* state_slot, int32_t num_slots, const void* checkpoints,
                            int32_t window, const int32_t* commit_len, int32_t H, int32_t dk,
                            int32_t dv, int32_t* err, hipStream_t stream) {
  const char* who = "gdn_commit_prefix";
  sv_status st =
      check_gdn_common(batch, state, state_dtype, num_slots, SV_F32, H, dk, dv, who);
  if (st != SV_OK) return st;
  st = check_window(batch, window, who);
  if (st != SV_OK) return st;
  if (!checkpoints || !commit_len)
    return fail(SV_EINVAL, "%s: checkpoints and commit_len are required", who);
  if (reinterpret_cast<uintptr_t>(checkpoints) & 15)
    return fail(SV_EINVAL, "%s: checkpoints must be 16-byte aligned", who);
  if (!state_slot && num_slots < batch->B)
    return fail(SV_EINVAL, "%s: without state_slot, num_slots must be >= B", who);
  const sv::GdnScalars s = gdn_scalars(batch, SV_GDN_COMMIT_ONLY, state_slot, num_slots,
                                       commit_len, H, dk, dv, window, err);
  return hip_status(sv::launch_gdn_commit_prefix(s, checkpoints, state, state_dtype, stream), who);
}

sv_status short_conv_verify_checkpoint(const sv_batch* batch, const void* state,
                                       const int32_t* state_slot, int32_t num_slots,
                                       const void* x, const float* weight, const float* bias,
                                       sv_dtype io_dtype, int32_t activation, void* out,
                                       void* prefix_states, int32_t window, int32_t C, int32_t K,
                                       int32_t* err, hipStream_t stream) {
  const char* who = "short_conv_verify_checkpoint";
  sv_status st = check_conv_common(batch, state, state_slot, num_slots, io_dtype, C, K, who);
  if (st != SV_OK) return st;
  st = check_window(batch, window, who);
  if (st != SV_OK) return st;
  if (activation != SV_ACT_NONE && activation != SV_ACT_SILU)
    return fail(SV_EINVAL, "%s: unknown activation %d", who, activation);
  if (!x || !weight || !out || !prefix_states)
    return fail(SV_EINVAL, "%s: x, weight, out and prefix_states are required", who);
  sv::ConvArgs a{};
  a.B = batch->B;
  a.total_T = batch->total_T;
  a.max_T = batch->max_T;
  a.cu = batch->cu_seqlens;
  a.mode = SV_GDN_VERIFY_ONLY;
  a.state_slot = state_slot;
  a.num_slots = num_slots;
  a.C = C;
  a.K = K;
  a.activation = activation;
  a.state = const_cast<void*>(state);  // read only: VERIFY_ONLY without pending tokens
  a.x = x;
  a.weight = weight;
  a.bias = bias;
  a.out = out;
  a.series = prefix_states;
  a.window = window;
  a.err = err;
  return hip_status(sv::launch_conv(a, io_dtype, stream), who);
}

sv_status short_conv_commit_prefix(const sv_batch* batch, void* state, const int32_t* state_slot,
                                   int32_t num_slots, const void* prefix_states, int32_t window,
                                   const int32_t* commit_len, sv_dtype io_dtype, int32_t C,
                                   int32_t K, int32_t* err, hipStream_t stream) {
  const char* who = "short_conv_commit_prefix";
  sv_status st = check_conv_common(batch, state, state_slot, num_slots, io_dtype, C, K, who);
  if (st != SV_OK) return st;
  st = check_window(batch, window, who);
  if (st != SV_OK) return st;
  if (!prefix_states || !commit_len)
    return fail(SV_EINVAL, "%s: prefix_states and commit_len are required", who);
  sv::ConvArgs a{};
  a.B = batch->B;
  a.total_T = batch->total_T;
  a.max_T = batch->max_T;
  a.cu = batch->cu_seqlens;
  a.mode = SV_GDN_COMMIT_ONLY;
  a.state_slot = state_slot;
  a.num_slots = num_slots;
  a.commit_len = commit_len;
  a.C = C;
  a.K = K;
  a.state = state;
  a.series = const_cast<void*>(prefix_states);
  a.window = window;
  a.err = err;
  return hip_status(sv::launch_conv_commit_prefix(a, io_dtype, stream), who);
}

size_t spec_accept_workspace_bytes(int32_t B, int32_t total_T, int32_t V, sv_accept_mode mode) {
  if (B < 1 || total_T < 1 || V < 1) return 0;
  return sv::accept_workspace_bytes(B, total_T, V, mode);
}

sv_status spec_accept(const sv_batch* batch, sv_accept_mode mode, const void* target_logits,
                      const void* draft_logits, sv_dtype logit_dtype, int32_t V,
                      const int32_t* draft_tokens, const float* u_accept, const float* u_final,
                      int32_t* result, int32_t* commit_len_out, int32_t* ctx_lens_inout,
                      void* workspace, size_t workspace_bytes, int32_t* err,
                      hipStream_t stream) {
  sv_accept_args acc{};
  acc.mode = mode;
  acc.logit_dtype = logit_dtype;
  acc.V = V;
  acc.target_logits = target_logits;
  acc.draft_logits = draft_logits;
  acc.draft_tokens = draft_tokens;
  acc.u_accept = u_accept;
  acc.u_final = u_final;
  acc.bonus_tokens = nullptr;
  return accept_impl(batch, &acc, result, commit_len_out, ctx_lens_inout, workspace,
                     workspace_bytes, err, stream, "spec_accept");
}

sv_status spec_accept_args(const sv_batch* batch, const sv_accept_args* acc, int32_t* result,
                           int32_t* commit_len_out, int32_t* ctx_lens_inout, void* workspace,
                           size_t workspace_bytes, int32_t* err, hipStream_t stream) {
  if (!acc) return fail(SV_EINVAL, "spec_accept_args: acc is null");
  return accept_impl(batch, acc, result, commit_len_out, ctx_lens_inout, workspace,
                     workspace_bytes, err, stream, "spec_accept_args");
}

sv_status spec_accept_noalloc(const sv_batch* batch, const sv_accept_args* acc, int32_t* result,
                              int32_t* commit_len_out, int32_t* ctx_lens_inout, int32_t* err,
                              hipStream_t stream) {
  const char* who = "spec_accept_noalloc";
  if (!acc) return fail(SV_EINVAL, "%s: acc is null", who);
  sv_status st = check_accept_args(batch, acc, result, who);
  if (st != SV_OK) return st;
  const size_t need = sv::accept_workspace_bytes(batch->B, batch->total_T, acc->V, acc->mode);
  if (need > sv::kAcceptScratchBytes)
    return fail(SV_ECAPACITY, "%s: this batch needs %zu bytes of scratch, the library holds %zu",
                who, need, sv::kAcceptScratchBytes);
  void* scratch_ptr = nullptr;
  st = hip_status(sv::accept_scratch(&scratch_ptr), who);
  if (st != SV_OK) return st;
  return launch_accept_checked(batch, acc, result, commit_len_out, ctx_lens_inout, scratch_ptr,
                               err, stream, who);
}

size_t spec_verify_step_workspace_bytes(const sv_batch* batch, const sv_attn_config* acfg,
                                        const sv_accept_args* acc) {
  if (!batch || batch->B < 1 || batch->total_T < 1) return 0;
  size_t need = 0;
  if (acfg)
    need = std::max(need, sv::attn_workspace_bytes(batch->B, batch->total_T, acfg->Hq, acfg->Hkv,
                                                   acfg->D, acfg->max_pages_per_seq,
                                                   acfg->page_size, acfg->dtype));
  if (acc && acc->V >= 1)
    need = std::max(need, sv::accept_workspace_bytes(batch->B, batch->total_T, acc->V, acc->mode));
  return need;
}

sv_status spec_verify_step(const sv_batch* batch, int32_t n_layers, const uint8_t* layer_kind,
                           const sv_attn_config* acfg, const sv_attn_layer* attn,
                           const sv_gdn_config* gcfg, const sv_gdn_layer* gdn,
                           const sv_accept_args* acc, int32_t* ctx_lens, int32_t* result,
                           int32_t* commit_len, sv_schedule schedule,
                           const sv_step_pending* pending, void* workspace,
                           size_t workspace_bytes, int32_t* err, hipStream_t stream) {
  const char* who = "spec_verify_step";
  sv_status st = check_batch(batch, who);
  if (st != SV_OK) return st;
  if (n_layers < 0 || (n_layers > 0 && !layer_kind))
    return fail(SV_EINVAL, "%s: layer_kind is required", who);
  if (!acc || !ctx_lens || !result || !commit_len)
    return fail(SV_EINVAL, "%s: accept args, ctx_lens, result and commit_len are required", who);
  if (schedule != SV_SCHEDULE_TWO_PHASE && schedule != SV_SCHEDULE_DEFERRED)
    return fail(SV_EINVAL, "%s: unknown schedule %d", who, static_cast<int>(schedule));
  int n_attn = 0, n_gdn = 0;
  for (int l = 0; l < n_layers; ++l) {
    if (layer_kind[l] == 1) ++n_attn;
    else if (layer_kind[l] == 0) ++n_gdn;
    else return fail(SV_EINVAL, "%s: layer_kind[%d] = %d is neither 0 nor 1", who, l, layer_kind[l]);
  }
  if (n_attn && (!acfg || !attn)) return fail(SV_EINVAL, "%s: attention config/layers missing", who);
  if (n_gdn && (!gcfg || !gdn)) return fail(SV_EINVAL, "%s: GDN config/layers missing", who);
  if (n_attn && acfg->kv_format != SV_KV_PLAIN && acfg->kv_format != SV_KV_INT8)
    return fail(SV_EINVAL, "%s: unknown kv_format %d", who, static_cast<int>(acfg->kv_format));
  if (n_attn && acfg->kv_format == SV_KV_INT8 && acfg->dtype != SV_BF16)
    return fail(SV_EDTYPE, "%s: INT8 KV pages take bf16 activations", who);
  if (pending && schedule != SV_SCHEDULE_DEFERRED)
    return fail(SV_EINVAL, "%s: pending tokens are only used by the deferred schedule", who);
  if (pending && (!pending->layers || !pending->commit_len))
    return fail(SV_EINVAL, "%s: pending layers and commit_len are required", who);
  const size_t need = spec_verify_step_workspace_bytes(batch, n_attn ? acfg : nullptr, acc);
  if (!workspace || workspace_bytes < need)
    return fail(SV_EWORKSPACE, "%s: workspace needs %zu bytes (got %zu)", who, need,
                workspace ? workspace_bytes : size_t(0));

  // 0. every argument of every layer and of the acceptance is checked before
  // the first launch, so a refused call has changed no page, state or length
  // (a retry after fixing it must not replay pending tokens twice)
  {
    char what[64];
    int ia = 0, ig = 0;
    for (int l = 0; l < n_layers; ++l) {
      std::snprintf(what, sizeof(what), "%s: layer %d", who, l);
      if (layer_kind[l] == 1) {
        const sv_attn_layer& L = attn[ia++];
        const sv_dtype dt = acfg->kv_format == SV_KV_INT8 ? SV_BF16 : acfg->dtype;
        st = check_attn(batch, L.q, L.k_new, L.v_new, L.k_cache, L.v_cache, acfg->block_table,
                        acfg->max_pages_per_seq, acfg->num_pages, acfg->page_size, ctx_lens,
                        L.out, acfg->Hq, acfg->Hkv, acfg->D, dt, what);
        if (st == SV_OK && acfg->kv_format == SV_KV_INT8)
          st = check_attn_kv8(L.k_scale, L.v_scale, what);
      } else {
        const sv_gdn_layer& G = gdn[ig];
        sv_gdn_pending pg{};
        if (pending) {
          const sv_gdn_layer& P = pending->layers[ig];
          pg = sv_gdn_pending{pending->batch, P.k, P.v, P.alpha, P.beta, pending->commit_len};
        }
        ++ig;
        st = check_gdn_call(batch, SV_GDN_VERIFY_ONLY, G.state, gcfg->state_dtype,
                            gcfg->state_slot, gcfg->num_slots, G.q, G.k, G.v, gcfg->io_dtype,
                            G.alpha, G.beta, nullptr, G.out, gcfg->H, gcfg->dk, gcfg->dv,
                            pending ? &pg : nullptr, what);
        if (st == SV_OK)
          st = check_step_conv(batch, gcfg, G, pending ? &pending->layers[ig - 1] : nullptr,
                               what);
      }
      if (st != SV_OK) return st;
    }
    st = check_accept(batch, acc, result, workspace, workspace_bytes, who);
    if (st != SV_OK) return st;
  }

  // 1. verify every layer in model order
  int ia = 0, ig = 0;
  for (int l = 0; l < n_layers; ++l) {
    if (layer_kind[l] == 1) {
      const sv_attn_layer& L = attn[ia++];
      if (acfg->kv_format == SV_KV_INT8) {
        st = spec_verify_attention_kv8(
            batch, L.q, L.k_new, L.v_new, static_cast<int8_t*>(L.k_cache),
            static_cast<int8_t*>(L.v_cache), L.k_scale, L.v_scale, acfg->block_table,
            acfg->max_pages_per_seq, acfg->num_pages, acfg->page_size, ctx_lens, L.out, acfg->Hq,
            acfg->Hkv, acfg->D, acfg->scale, workspace, workspace_bytes, err, stream);
      } else {
        st = spec_verify_attention(batch, L.q, L.k_new, L.v_new, L.k_cache, L.v_cache,
                                   acfg->block_table, acfg->max_pages_per_seq, acfg->num_pages,
                                   acfg->page_size, ctx_lens, L.out, acfg->Hq, acfg->Hkv, acfg->D,
                                   acfg->dtype, acfg->scale, 1, workspace, workspace_bytes, err,
                                   stream);
      }
    } else {
      const sv_gdn_layer& G = gdn[ig];
      sv_gdn_pending pg{};
      const sv_gdn_pending* pp = nullptr;
      if (pending) {
        const sv_gdn_layer& P = pending->layers[ig];
        pg.batch = pending->batch;
        pg.k = P.k;
        pg.v = P.v;
        pg.alpha = P.alpha;
        pg.beta = P.beta;
        pg.commit_len = pending->commit_len;
        pp = &pg;
      }
      if (gcfg->conv_C > 0) {
        // the layer's GDN verify and its short convolution in one launch
        sv::GdnScalars s{};
        s.B = batch->B;
        s.total_T = batch->total_T;
        s.max_T = batch->max_T;
        s.cu = batch->cu_seqlens;
        s.mode = SV_GDN_VERIFY_ONLY;
        s.state_slot = gcfg->state_slot;
        s.num_slots = gcfg->num_slots;
        s.H = gcfg->H;
        s.dk = gcfg->dk;
        s.dv = gcfg->dv;
        s.err = err;
        sv::GdnFullPtrs p{};
        p.state = G.state;
        p.q = G.q;
        p.k = G.k;
        p.v = G.v;
        p.alpha = G.alpha;
        p.beta = G.beta;
        p.out = G.out;
        sv::ConvArgs c = step_conv_args(batch, gcfg, SV_GDN_VERIFY_ONLY, nullptr, err);
        c.state = G.conv_state;
        c.x = G.conv_x;
        c.weight = G.conv_weight;
        c.bias = G.conv_bias;
        c.out = G.conv_out;
        if (pending) {
          s.has_pending = 1;
          s.p_total_T = pending->batch.total_T;
          s.p_max_T = pending->batch.max_T;
          s.p_cu = pending->batch.cu_seqlens;
          s.p_commit = pending->commit_len;
          p.pk = pg.k;
          p.pv = pg.v;
          p.palpha = pg.alpha;
          p.pbeta = pg.beta;
          c.has_pending = 1;
          c.p_total_T = pending->batch.total_T;
          c.p_max_T = pending->batch.max_T;
          c.p_cu = pending->batch.cu_seqlens;
          c.p_commit = pending->commit_len;
          c.px = pending->layers[ig].conv_x;
        }
        st = hip_status(sv::launch_gdn_conv(s, p, c, gcfg->io_dtype, gcfg->state_dtype, stream),
                        who);
        ++ig;
      } else {
        ++ig;
        st = gdn_verify_commit(batch, SV_GDN_VERIFY_ONLY, G.state, gcfg->state_dtype,
                               gcfg->state_slot, gcfg->num_slots, G.q, G.k, G.v,
                               gcfg->io_dtype, G.alpha, G.beta, nullptr, G.out, gcfg->H,
                               gcfg->dk, gcfg->dv, pp, err, stream);
      }
    }
    if (st != SV_OK) return st;
  }
  // 2. acceptance (ctx_lens is advanced by a+1 here, after every attention layer)
  st = accept_impl(batch, acc, result, commit_len, ctx_lens, workspace, workspace_bytes, err,
                   stream, who);
  if (st != SV_OK) return st;
  // 3. two-phase: commit the first a+1 tokens of every GDN layer
  // (every layer's state, k, v and gates were checked in step 0)
  if (schedule == SV_SCHEDULE_TWO_PHASE && n_gdn > 0) {
    st = commit_layers(batch, gcfg, gdn, n_gdn, commit_len, err, stream, who);
    if (st != SV_OK) return st;
  }
  return ok();
}

sv_status spec_verify_flush(int32_t n_gdn, const sv_gdn_config* gcfg,
                            const sv_step_pending* pending, int32_t* err, hipStream_t stream) {
  const char* who = "spec_verify_flush";
  if (n_gdn < 0) return fail(SV_EINVAL, "%s: n_gdn must be >= 0 (got %d)", who, n_gdn);
  if (!pending) return fail(SV_EINVAL, "%s: pending is required", who);
  if (n_gdn == 0) return ok();
  if (!gcfg || !pending->layers || !pending->commit_len)
    return fail(SV_EINVAL, "%s: gdn config, pending layers and commit_len are required", who);
  const sv_batch* batch = &pending->batch;
  // every layer is checked before the first launch
  char what[64];
  for (int l = 0; l < n_gdn; ++l) {
    std::snprintf(what, sizeof(what), "%s: layer %d", who, l);
    const sv_gdn_layer& G = pending->layers[l];
    sv_status st = check_gdn_call(batch, SV_GDN_COMMIT_ONLY, G.state, gcfg->state_dtype,
                                  gcfg->state_slot, gcfg->num_slots, nullptr, G.k, G.v,
                                  gcfg->io_dtype, G.alpha, G.beta, pending->commit_len,
                                  nullptr, gcfg->H, gcfg->dk, gcfg->dv, nullptr, what);
    if (st != SV_OK) return st;
    if (gcfg->conv_C > 0) {
      if (gcfg->conv_K < 2 || gcfg->conv_K > 8)
        return fail(SV_EINVAL, "%s: conv_K must be in 2..8 (got %d)", what, gcfg->conv_K);
      if (!G.conv_state || !G.conv_x)
        return fail(SV_EINVAL, "%s: conv_state and conv_x are required", what);
    }
  }
  return commit_layers(batch, gcfg, pending->layers, n_gdn, pending->commit_len, err, stream,
                       who);
}

}  // extern "C"
