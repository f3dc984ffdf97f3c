// One block of the short causal convolution: 256 channels of one sequence
// (shared by the standalone launch and the launch that runs it beside the
// GDN verify of the same layer).
//
// The packed varlen operator of onnxruntime-genai pull request 2457 (commit
// message on the VarlenCausalConvWithState prefix states) keeps a rolling
// state of the last K-1 inputs per sequence.  Per channel c, with
// z = [state_0 .. state_{K-2}, x_0 .. x_{T-1}] (oldest first):
//   y_t[c] = act( sum_{i<K} w[c, i] z_{t+i}[c] + bias[c] ),   act = id or SiLU
// Commit keeps the last K-1 rows of [state, x_0 .. x_{c_b-1}]; with pending
// tokens (deferred schedule) the window first advances over the previous
// step's c_b pending inputs and that state is stored.  One thread per
// (sequence, channel): the window lives in registers, every access is a
// coalesced row of C channels, and the stored state is a copy of inputs.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace sv {

constexpr int kConvThreads = 256;

template <typename IO, int K, bool CKPT>
__device__ __forceinline__ void conv_block(const ConvArgs& a, int b, int cblk) {
  using L = io<IO>;
  const int c = cblk * kConvThreads + threadIdx.x;
  const bool report = cblk == 0 && threadIdx.x == 0;
  // ---- validate the sequence (uniform over the block).  Every per-sequence
  // value is loaded before any is checked (the guards depend on kernel
  // arguments only), so the block waits one round trip for all of them.
  const bool has_commit = a.mode != SV_GDN_VERIFY_ONLY;
  const int x0 = a.cu[b];
  const int x1 = a.cu[b + 1];
  const int slot = a.state_slot ? a.state_slot[b] : b;
  const int cm_in = has_commit ? a.commit_len[b] : 0;
  const int p0 = a.has_pending ? a.p_cu[b] : 0;
  const int p1 = a.has_pending ? a.p_cu[b + 1] : 1;
  const int pc_in = a.has_pending ? a.p_commit[b] : 0;
  const int T = x1 - x0;
  const int pT = p1 - p0;
  int bad = 0;
  if (T < 1 || T > a.max_T || x0 < 0 || x0 + T > a.total_T) bad = SV_DERR_SEQLEN;
  else if (slot < 0 || slot >= a.num_slots) bad = SV_DERR_SLOT;
  else if (cm_in < 0 || cm_in > T) bad = SV_DERR_COMMIT;
  else if (a.has_pending && (pT < 1 || pT > a.p_max_T || p0 < 0 || p0 + pT > a.p_total_T))
    bad = SV_DERR_SEQLEN;
  else if (pc_in < 0 || pc_in > pT) bad = SV_DERR_COMMIT;
  if (bad) {
    if (report) flag_error(a.err, bad);
    return;
  }
  const int cm = cm_in;
  const int px0 = p0, pc = pc_in;
  if (c >= a.C) return;
  const int C = a.C;
  const size_t srow = static_cast<size_t>(slot) * (K - 1);

  // ---- every input this thread reads, loaded before any is used (rows
  // clamped into the sequence, the surplus masked afterwards): the window,
  // the pending inputs, this call's inputs
  const bool verify = a.mode != SV_GDN_COMMIT_ONLY;
  const int n = verify ? T : cm;  // current tokens read
  float win[K - 1];
#pragma unroll
  for (int i = 0; i < K - 1; ++i) win[i] = L::load(a.state, (srow + i) * C + c);
  float pin[kMaxT];
  if (a.has_pending) {
#pragma unroll
    for (int t = 0; t < kMaxT; ++t)
      pin[t] = L::load(a.px, static_cast<size_t>(px0 + min(t, pT - 1)) * C + c);
  }
  float z[K - 1 + kMaxT];
#pragma unroll
  for (int t = 0; t < kMaxT; ++t)
    z[K - 1 + t] = L::load(a.x, static_cast<size_t>(x0 + min(t, T - 1)) * C + c);
#pragma unroll
  for (int t = 0; t < kMaxT; ++t)
    if (t >= n) z[K - 1 + t] = 0.f;

  // ---- the window: the last K-1 inputs, then the pending ones shifted in
  if (a.has_pending) {
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) {
      if (t < pc) {
#pragma unroll
        for (int i = 0; i < K - 2; ++i) win[i] = win[i + 1];
        win[K - 2] = pin[t];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < K - 1; ++i) z[i] = win[i];

  if (verify) {
    float w[K];
#pragma unroll
    for (int i = 0; i < K; ++i) w[i] = a.weight[static_cast<size_t>(c) * K + i];
    const float bias = a.bias ? a.bias[c] : 0.f;
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) {
      if (t >= T) break;
      float u = 0.f;
#pragma unroll
      for (int i = 0; i < K; ++i) u = fmaf(w[i], z[t + i], u);
      u += bias;
      if (a.activation == SV_ACT_SILU) u = u / (1.f + expf(-u));
      L::store(a.out, static_cast<size_t>(x0 + t) * C + c, u);
    }
  }

  if constexpr (CKPT) {  // the window after every token, front-aligned
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) {
      if (t >= T) break;
#pragma unroll
      for (int i = 0; i < K - 1; ++i)
        L::store(a.series, ((static_cast<size_t>(b) * a.window + t) * (K - 1) + i) * C + c,
                 z[t + 1 + i]);
    }
  }

  // ---- store the committed window (a copy of inputs: exact)
  if (a.mode == SV_GDN_VERIFY_ONLY) {
    if (pc > 0) {
#pragma unroll
      for (int i = 0; i < K - 1; ++i) L::store(a.state, (srow + i) * C + c, win[i]);
    }
  } else if (pc > 0 || cm > 0) {
#pragma unroll
    for (int i = 0; i < K - 1; ++i) {
      float v = z[0];
#pragma unroll
      for (int s = 0; s <= kMaxT; ++s)  // z[cm + i] with cm a runtime value
        if (s == cm) v = z[s + i];
      L::store(a.state, (srow + i) * C + c, v);
    }
  }
}


// conv_block with the width K chosen at run time (2..8).
template <typename IO>
__device__ __forceinline__ void conv_block_any(const ConvArgs& a, int b, int cblk) {
  switch (a.K) {
    case 2: conv_block<IO, 2, false>(a, b, cblk); break;
    case 3: conv_block<IO, 3, false>(a, b, cblk); break;
    case 4: conv_block<IO, 4, false>(a, b, cblk); break;
    case 5: conv_block<IO, 5, false>(a, b, cblk); break;
    case 6: conv_block<IO, 6, false>(a, b, cblk); break;
    case 7: conv_block<IO, 7, false>(a, b, cblk); break;
    default: conv_block<IO, 8, false>(a, b, cblk); break;
  }
}

}  // namespace sv
