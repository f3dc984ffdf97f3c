// Short causal convolution of the linear-attention layers: verify and commit.
//
// The packed varlen operator of onnxruntime-genai pull request 2457 (commit
// message on the VarlenCausalConvWithState prefix states) keeps a rolling
// state of the last K-1 inputs per sequence and publishes the state after
// every token (slot j = state after local token j).  Per channel c, with
// z = [state_0 .. state_{K-2}, x_0 .. x_{T-1}] (oldest first):
//   y_t[c] = act( sum_{i<K} w[c, i] z_{t+i}[c] + bias[c] ),   act = id or SiLU
// Commit keeps the last K-1 rows of [state, x_0 .. x_{c_b-1}]: the state a run
// over only the accepted prefix leaves; rejected tokens are never applied.
// With pending tokens (deferred schedule) the window first advances over the
// previous step's c_b pending inputs and that state is stored.
//
// With a prefix-state series (the operator's prefix_states output, slot j =
// the window after local token j) the verify also writes every token's
// window; CommitPrefix then copies slot c_b - 1 into the state.
//
// One thread per (sequence, channel): the window lives in registers, every
// access is a coalesced row of C channels, and the stored state is a copy of
// inputs (no arithmetic), so it is exact.

#include "conv_block.h"

namespace sv {
namespace {

constexpr int kThreads = kConvThreads;

template <typename IO, int K, bool CKPT>
__global__ __launch_bounds__(kThreads) void conv_kernel(ConvArgs a) {
  conv_block<IO, K, CKPT>(a, blockIdx.y, blockIdx.x);
}

template <typename IO, bool CKPT>
void launch_conv_k(const ConvArgs& a, hipStream_t stream) {
  const dim3 grid((a.C + kThreads - 1) / kThreads, a.B);
  switch (a.K) {
    case 2: hipLaunchKernelGGL((conv_kernel<IO, 2, CKPT>), grid, dim3(kThreads), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((conv_kernel<IO, 3, CKPT>), grid, dim3(kThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((conv_kernel<IO, 4, CKPT>), grid, dim3(kThreads), 0, stream, a); break;
    case 5: hipLaunchKernelGGL((conv_kernel<IO, 5, CKPT>), grid, dim3(kThreads), 0, stream, a); break;
    case 6: hipLaunchKernelGGL((conv_kernel<IO, 6, CKPT>), grid, dim3(kThreads), 0, stream, a); break;
    case 7: hipLaunchKernelGGL((conv_kernel<IO, 7, CKPT>), grid, dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL((conv_kernel<IO, 8, CKPT>), grid, dim3(kThreads), 0, stream, a); break;
  }
}

template <typename IO>
hipError_t launch_conv_io(const ConvArgs& a, hipStream_t stream) {
  if (a.series) launch_conv_k<IO, true>(a, stream);
  else launch_conv_k<IO, false>(a, stream);
  return hipGetLastError();
}

// CommitPrefix: one thread per (sequence, channel) copies the K - 1 rows of
// slot c_b - 1 (c_b = 0 keeps the state).
template <typename IO>
__global__ __launch_bounds__(kThreads) void conv_commit_prefix_kernel(ConvArgs a) {
  using E = typename io<IO>::storage;
  const int b = blockIdx.y;
  const int c = blockIdx.x * kThreads + threadIdx.x;
  const bool report = blockIdx.x == 0 && threadIdx.x == 0;
  const int x0 = a.cu[b];
  const int T = a.cu[b + 1] - x0;
  if (T < 1 || T > a.max_T || x0 < 0 || x0 + T > a.total_T) {
    if (report) flag_error(a.err, SV_DERR_SEQLEN);
    return;
  }
  const int slot = a.state_slot ? a.state_slot[b] : b;
  if (slot < 0 || slot >= a.num_slots) {
    if (report) flag_error(a.err, SV_DERR_SLOT);
    return;
  }
  const int cm = a.commit_len[b];
  if (cm < 0 || cm > T) {
    if (report) flag_error(a.err, SV_DERR_COMMIT);
    return;
  }
  if (cm == 0 || c >= a.C) return;
  const int Km1 = a.K - 1;
  const E* src = static_cast<const E*>(a.series) +
                 (static_cast<size_t>(b) * a.window + (cm - 1)) * Km1 * a.C;
  E* dst = static_cast<E*>(a.state) + static_cast<size_t>(slot) * Km1 * a.C;
  for (int i = 0; i < Km1; ++i) dst[static_cast<size_t>(i) * a.C + c] = src[static_cast<size_t>(i) * a.C + c];
}

}  // namespace

hipError_t launch_conv(const ConvArgs& a, sv_dtype io_dt, hipStream_t stream) {
  return io_dt == SV_BF16 ? launch_conv_io<bf16_t>(a, stream) : launch_conv_io<float>(a, stream);
}

hipError_t launch_conv_commit_prefix(const ConvArgs& a, sv_dtype io_dt, hipStream_t stream) {
  const dim3 grid((a.C + kThreads - 1) / kThreads, a.B);
  if (io_dt == SV_BF16)
    hipLaunchKernelGGL(conv_commit_prefix_kernel<bf16_t>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(conv_commit_prefix_kernel<float>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sv
