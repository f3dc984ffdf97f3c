// Host-side launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {

constexpr int kMaxT = 8;                 // verify tokens per sequence
constexpr int kGdnLayersPerLaunch = 48;  // layers in one batched commit launch

// ---------------------------------------------------------------- GDN
struct GdnScalars {
  int B, total_T, max_T;
  const int32_t* cu;            // [B+1]
  int mode;                     // sv_gdn_mode
  const int32_t* state_slot;    // [B] or null
  int num_slots;
  const int32_t* commit_len;    // [B] or null (VERIFY_ONLY)
  int H, dk, dv;
  int has_pending;
  int p_total_T, p_max_T;
  const int32_t* p_cu;          // [B+1]
  const int32_t* p_commit;      // [B]
  int window;                   // checkpoint series slots (checkpoint calls)
  int32_t* err;
};

struct ConvArgs {
  int B, total_T, max_T;
  const int32_t* cu;            // [B+1]
  int mode;                     // sv_gdn_mode
  const int32_t* state_slot;    // [B] or null
  int num_slots;
  const int32_t* commit_len;    // [B] or null (VERIFY_ONLY)
  int C, K, activation;
  void* state;                  // [num_slots][K-1][C] io dtype
  const void* x;                // [total_T][C]
  const float* weight;          // [C][K]
  const float* bias;            // [C] or null
  void* out;                    // [total_T][C]
  int has_pending;
  int p_total_T, p_max_T;
  const int32_t* p_cu;          // [B+1]
  const int32_t* p_commit;      // [B]
  const void* px;               // [p_total_T][C]
  void* series;                 // [B][window][K-1][C] prefix states, or null
  int window;
  int32_t* err;
};
hipError_t launch_conv(const ConvArgs& a, sv_dtype io_dtype, hipStream_t stream);
// CommitPrefix of the conv: state[slot_b] = series[b][c_b - 1] where c_b >= 1.
hipError_t launch_conv_commit_prefix(const ConvArgs& a, sv_dtype io_dtype, hipStream_t stream);

struct GdnFullPtrs {
  void* state;                  // fp32 or fp16 [num_slots][H][dv][dk]
  const void* q; const void* k; const void* v;
  const float* alpha; const float* beta;
  void* out;
  const void* pk; const void* pv; const float* palpha; const float* pbeta;
  void* ckpt;                   // checkpoint series [B][window][H][dv][dk], or null
};

struct GdnCommitPtrs {
  void* state;
  const void* k; const void* v;
  const float* alpha; const float* beta;
};

struct ConvCommitPtrs {
  void* state;                  // [num_slots][K-1][C]
  const void* x;                // [total_T][C]
};

struct GdnCommitTable {
  GdnCommitPtrs l[kGdnLayersPerLaunch];
  ConvCommitPtrs c[kGdnLayersPerLaunch];  // used when the launch commits convs too
};

hipError_t launch_gdn(const GdnScalars& s, const GdnFullPtrs& p, sv_dtype io,
                      sv_dtype state_dtype, hipStream_t stream);
// CommitPrefix: state[slot_b] = ckpt[b][window - T_b + c_b - 1] where c_b >= 1.
hipError_t launch_gdn_commit_prefix(const GdnScalars& s, const void* ckpt, void* state,
                                    sv_dtype state_dtype, hipStream_t stream);
// COMMIT_ONLY over n_layers (<= kGdnLayersPerLaunch) layers in one launch;
// with conv (its scalars; state and x per layer from t.c) the layers' short
// convolutions are committed in the same launch.
hipError_t launch_gdn_commit_multi(const GdnScalars& s, const GdnCommitTable& t,
                                   int n_layers, sv_dtype io, sv_dtype state_dtype,
                                   hipStream_t stream, const ConvArgs* conv = nullptr);
// The GDN verify / commit of a layer and its short convolution in one launch
// (the conv's blocks after the GDN's; they share no data).
hipError_t launch_gdn_conv(const GdnScalars& s, const GdnFullPtrs& p, const ConvArgs& conv,
                           sv_dtype io, sv_dtype state_dtype, hipStream_t stream);

// ---------------------------------------------------------------- attention
struct AttnArgs {
  int B, total_T, max_T;
  const int32_t* cu;
  const void* q; const void* k_new; const void* v_new;
  void* k_cache; void* v_cache;
  const int32_t* block_table;
  int max_pages, num_pages, P;
  const int32_t* ctx_lens;
  void* out;
  int Hq, Hkv, D;
  float scale;                  // already resolved (never 0)
  int write_kv;
  // INT8 pages: k_cache / v_cache hold int8 codes, scales fp32 [Hkv][D]
  int kv8;
  const float* k_scale;
  const float* v_scale;
  int32_t* err;
  // stream-kernel grid and the pieces of segments cut by range boundaries
  int n_wg;                     // workgroups (grid.x)
  int* seg_meta;                // [B * Hkv][2]: first and last workgroup of a segment,
                                // then the launch's count of cost units
  float* part_o;                // [(B * Hkv + n_wg) * 64 rows][D]
  float* part_ml;               // [(B * Hkv + n_wg) * 64 rows][2]
};

// Workspace of one attention call: [segment meta | partial O | partial (m, l)].
size_t attn_workspace_bytes(int B, int total_T, int Hq, int Hkv, int D,
                            int max_pages, int P, sv_dtype dtype);
void attn_workspace_carve(void* ws, int B, int Hkv, int D, int n_wg, int** seg_meta,
                          float** part_o, float** part_ml);
// Grid of the stream kernel for these shapes on the current device.
int attn_stream_grid(int D, int G, int max_T, bool kv8);
hipError_t launch_attention(const AttnArgs& a, sv_dtype dtype,
                            hipStream_t stream);

// ---------------------------------------------------------------- accept
struct AcceptArgs {
  int B, total_T, max_T;
  const int32_t* cu;
  int mode;                     // sv_accept_mode
  const void* target; const void* draft;
  int V;
  const int32_t* draft_tokens;
  const float* u_accept; const float* u_final;
  const int32_t* bonus;         // [B] supplied bonus tokens, or null
  int32_t* result;
  int32_t* commit_len_out;
  int32_t* ctx_lens;
  int32_t* err;
  void* ws;
};

size_t accept_workspace_bytes(int B, int total_T, int V, int mode);
// Scratch of the allocation-free acceptance: a device array of the library,
// one per GPU.  accept_scratch gives the current device's address (looked up
// once per device with that device current).
constexpr size_t kAcceptScratchBytes = size_t(8) << 20;
hipError_t accept_scratch(void** ptr);
// Fill n int32 words with v on the stream (a kernel, so it can be captured).
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t stream);
hipError_t launch_accept(const AcceptArgs& a, sv_dtype dtype,
                         hipStream_t stream);

}  // namespace sv
