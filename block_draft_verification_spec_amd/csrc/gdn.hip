// Gated delta-net (GDN) recurrent-state verify and commit.
//
// Gated delta rule (Yang, Kautz & Hatamizadeh, ICLR 2025), per sequence b and
// head h, with the dv x dk state stored V-major in fp32 (onnxruntime-genai
// pull request 2457, GatedDeltaNet state layout) and fp32 gates:
//   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t
// Written per state row i (s_i is row i, a dk-vector):
//   u_i = s_i . k_t,   w_i = beta_t (v_{t,i} - alpha_t u_i),
//   s_i <- alpha_t s_i + w_i k_t,   o_{t,i} = alpha_t (s_i . q_t) + w_i (k_t . q_t)
// (the last line is s_i' . q_t expanded, so both dot products read the state
// before the update and reduce together).  Rows never interact, so a block
// owns 64 rows of one (b, h) tile and keeps them in registers for all tokens:
// the state is read once and written at most once, right after the last token
// whose effect is kept (lmdeploy pull request 5019, "Two fixes" item 2: the
// commit runs after acceptance; onnxruntime-genai pull request 2457:
// CommitPrefix keeps the accepted prefix without a snapshot).
//
// Layout of a block: 256 threads = 16 row groups x 16 column lanes.  Thread
// (row group rg, lane c) holds rows rg + 16 r (r < 4) and, of each row, the
// elements 64 v + 4 c .. 64 v + 4 c + 3 (v < dk / 64): sixteen consecutive
// lanes read one 256-byte half row per instruction, fully coalesced.  Token
// inputs (at most 8 pending + 8 current) are staged in LDS as fp32.

#include "device_common.h"
#include "internal.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = 64;
constexpr int kRowsPerThread = 4;
constexpr int kMaxTok = 2 * kMaxT;

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot4(const float4& a, const float4& b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

template <int DK>
struct GdnSmem {
  float k_s[kMaxTok][DK];
  float q_s[kMaxT][DK];
  float v_s[kMaxTok][kRowsPerBlock];
  float a_s[kMaxTok];
  float b_s[kMaxTok];
  float o_s[kMaxT][kRowsPerBlock];
};

// COMMIT_ONLY_NP: compile-time COMMIT_ONLY without pending tokens (the
// batched commit of the two-phase step); q, out and the pending pointers are
// then never touched.
template <typename IO, int DK, bool COMMIT_ONLY_NP>
__device__ __forceinline__ void gdn_tile(
    GdnSmem<DK>& sm, const GdnScalars& s, float* __restrict__ state, const void* q,
    const void* k, const void* v, const float* __restrict__ alpha,
    const float* __restrict__ beta, void* out, const void* pk, const void* pv,
    const float* __restrict__ palpha, const float* __restrict__ pbeta, int b,
    int h, int rb, bool report) {
  using L = io<IO>;
  constexpr int NV4 = DK / 64;
  auto& k_s = sm.k_s;
  auto& q_s = sm.q_s;
  auto& v_s = sm.v_s;
  auto& a_s = sm.a_s;
  auto& b_s = sm.b_s;
  auto& o_s = sm.o_s;

  const int tid = threadIdx.x;
  // ---- validate the sequence (uniform over the block)
  const int x0 = s.cu[b];
  const int T = s.cu[b + 1] - x0;
  if (T < 1 || T > s.max_T || x0 < 0 || x0 + T > s.total_T) {
    if (report && tid == 0) flag_error(s.err, SV_DERR_SEQLEN);
    return;
  }
  const int slot = s.state_slot ? s.state_slot[b] : b;
  if (slot < 0 || slot >= s.num_slots) {
    if (report && tid == 0) flag_error(s.err, SV_DERR_SLOT);
    return;
  }
  int c = 0;
  if (s.mode != SV_GDN_VERIFY_ONLY) {
    c = s.commit_len[b];
    if (c < 0 || c > T) {
      if (report && tid == 0) flag_error(s.err, SV_DERR_COMMIT);
      return;
    }
  }
  int px0 = 0, pc = 0;
  if (!COMMIT_ONLY_NP && s.has_pending) {
    px0 = s.p_cu[b];
    const int pT = s.p_cu[b + 1] - px0;
    if (pT < 1 || pT > s.p_max_T || px0 < 0 || px0 + pT > s.p_total_T) {
      if (report && tid == 0) flag_error(s.err, SV_DERR_SEQLEN);
      return;
    }
    pc = s.p_commit[b];
    if (pc < 0 || pc > pT) {
      if (report && tid == 0) flag_error(s.err, SV_DERR_COMMIT);
      return;
    }
  }
  const bool verify = !COMMIT_ONLY_NP && s.mode != SV_GDN_COMMIT_ONLY;
  const int n_cur = verify ? T : c;
  const int n_tot = pc + n_cur;
  // Index of the last token whose effect is stored; -1: nothing is stored.
  const int store_at = (s.mode == SV_GDN_VERIFY_ONLY) ? pc - 1 : pc + c - 1;
  if (!verify && store_at < 0) return;

  const int H = s.H;
  const int DV = s.dv;
  const int row0 = rb * kRowsPerBlock;
  const int cl = tid & 15;
  const int rg = tid >> 4;
  float* tile = state + (static_cast<size_t>(slot) * H + h) * DV * DK;

  // ---- issue the state loads first: they are the long-latency traffic
  float4 sr[kRowsPerThread][NV4];
#pragma unroll
  for (int r = 0; r < kRowsPerThread; ++r) {
    const float* rowp = tile + static_cast<size_t>(row0 + rg + 16 * r) * DK;
#pragma unroll
    for (int vv = 0; vv < NV4; ++vv)
      sr[r][vv] = *reinterpret_cast<const float4*>(rowp + vv * 64 + 4 * cl);
  }

  // ---- stage token inputs as fp32
  for (int i = tid; i < n_tot * DK; i += kThreads) {
    const int t = i / DK, e = i - t * DK;
    k_s[t][e] = t < pc ? L::load(pk, (static_cast<size_t>(px0 + t) * H + h) * DK + e)
                       : L::load(k, (static_cast<size_t>(x0 + t - pc) * H + h) * DK + e);
  }
  if (verify) {
    for (int i = tid; i < T * DK; i += kThreads) {
      const int t = i / DK, e = i - t * DK;
      q_s[t][e] = L::load(q, (static_cast<size_t>(x0 + t) * H + h) * DK + e);
    }
  }
  for (int i = tid; i < n_tot * kRowsPerBlock; i += kThreads) {
    const int t = i / kRowsPerBlock, r = i - t * kRowsPerBlock;
    v_s[t][r] = t < pc ? L::load(pv, (static_cast<size_t>(px0 + t) * H + h) * DV + row0 + r)
                       : L::load(v, (static_cast<size_t>(x0 + t - pc) * H + h) * DV + row0 + r);
  }
  if (tid < n_tot) {
    const int t = tid;
    const size_t gi = t < pc ? static_cast<size_t>(px0 + t) * H + h
                             : static_cast<size_t>(x0 + t - pc) * H + h;
    a_s[t] = t < pc ? palpha[gi] : alpha[gi];
    b_s[t] = t < pc ? pbeta[gi] : beta[gi];
  }
  __syncthreads();

  // ---- the recurrence, one token at a time
  for (int i = 0; i < n_tot; ++i) {
    const bool emit = verify && i >= pc;
    float4 kk[NV4];
#pragma unroll
    for (int vv = 0; vv < NV4; ++vv)
      kk[vv] = *reinterpret_cast<const float4*>(&k_s[i][vv * 64 + 4 * cl]);
    float uk[kRowsPerThread], uq[kRowsPerThread];
    float kq = 0.f;
#pragma unroll
    for (int r = 0; r < kRowsPerThread; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int vv = 0; vv < NV4; ++vv) acc += dot4(sr[r][vv], kk[vv]);
      uk[r] = acc;
    }
    if (emit) {
      float4 qq[NV4];
#pragma unroll
      for (int vv = 0; vv < NV4; ++vv)
        qq[vv] = *reinterpret_cast<const float4*>(&q_s[i - pc][vv * 64 + 4 * cl]);
#pragma unroll
      for (int vv = 0; vv < NV4; ++vv) kq += dot4(kk[vv], qq[vv]);
#pragma unroll
      for (int r = 0; r < kRowsPerThread; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int vv = 0; vv < NV4; ++vv) acc += dot4(sr[r][vv], qq[vv]);
        uq[r] = acc;
      }
    }
    // full-row dot products: sum over the 16 lanes that share the rows
#pragma unroll
    for (int r = 0; r < kRowsPerThread; ++r) uk[r] = row16_sum(uk[r]);
    if (emit) {
      kq = row16_sum(kq);
#pragma unroll
      for (int r = 0; r < kRowsPerThread; ++r) uq[r] = row16_sum(uq[r]);
    }
    const float al = a_s[i];
    const float be = b_s[i];
#pragma unroll
    for (int r = 0; r < kRowsPerThread; ++r) {
      const int rl = rg + 16 * r;
      const float w = be * (v_s[i][rl] - al * uk[r]);
#pragma unroll
      for (int vv = 0; vv < NV4; ++vv) {
        sr[r][vv].x = al * sr[r][vv].x + w * kk[vv].x;
        sr[r][vv].y = al * sr[r][vv].y + w * kk[vv].y;
        sr[r][vv].z = al * sr[r][vv].z + w * kk[vv].z;
        sr[r][vv].w = al * sr[r][vv].w + w * kk[vv].w;
      }
      if (emit && cl == 0) o_s[i - pc][rl] = al * uq[r] + w * kq;
    }
    if (i == store_at) {
#pragma unroll
      for (int r = 0; r < kRowsPerThread; ++r) {
        float* rowp = tile + static_cast<size_t>(row0 + rg + 16 * r) * DK;
#pragma unroll
        for (int vv = 0; vv < NV4; ++vv) {
          // streaming store: this launch does not read the state again
          const f32x4_t t = {sr[r][vv].x, sr[r][vv].y, sr[r][vv].z, sr[r][vv].w};
          __builtin_nontemporal_store(t, reinterpret_cast<f32x4_t*>(rowp + vv * 64 + 4 * cl));
        }
      }
    }
  }

  if (verify) {
    __syncthreads();
    for (int i = tid; i < T * kRowsPerBlock; i += kThreads) {
      const int t = i / kRowsPerBlock, r = i - t * kRowsPerBlock;
      L::store(out, (static_cast<size_t>(x0 + t) * H + h) * DV + row0 + r, o_s[t][r]);
    }
  }
}

template <typename IO, int DK>
__global__ __launch_bounds__(kThreads) void gdn_kernel(GdnScalars s, GdnFullPtrs p) {
  __shared__ GdnSmem<DK> sm;
  const int rb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  gdn_tile<IO, DK, false>(sm, s, p.state, p.q, p.k, p.v, p.alpha, p.beta, p.out, p.pk,
                   p.pv, p.palpha, p.pbeta, b, h, rb, rb == 0 && h == 0);
}

template <typename IO, int DK>
__global__ __launch_bounds__(kThreads) void gdn_commit_multi_kernel(GdnScalars s,
                                                                    GdnCommitTable t) {
  const int rb = blockIdx.x, h = blockIdx.y;
  const int b = blockIdx.z % s.B;
  const int layer = blockIdx.z / s.B;
  const GdnCommitPtrs& p = t.l[layer];
  __shared__ GdnSmem<DK> sm;
  gdn_tile<IO, DK, true>(sm, s, p.state, p.k, p.k, p.v, p.alpha, p.beta, p.state,
                         p.k, p.v, p.alpha, p.beta, b, h, rb,
                   rb == 0 && h == 0 && layer == 0);
}

}  // namespace

hipError_t launch_gdn(const GdnScalars& s, const GdnFullPtrs& p, sv_dtype io_dt,
                      hipStream_t stream) {
  dim3 grid(s.dv / kRowsPerBlock, s.H, s.B);
  dim3 block(kThreads);
  if (io_dt == SV_BF16) {
    if (s.dk == 128) hipLaunchKernelGGL((gdn_kernel<bf16_t, 128>), grid, block, 0, stream, s, p);
    else hipLaunchKernelGGL((gdn_kernel<bf16_t, 64>), grid, block, 0, stream, s, p);
  } else {
    if (s.dk == 128) hipLaunchKernelGGL((gdn_kernel<float, 128>), grid, block, 0, stream, s, p);
    else hipLaunchKernelGGL((gdn_kernel<float, 64>), grid, block, 0, stream, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_gdn_commit_multi(const GdnScalars& s, const GdnCommitTable& t,
                                   int n_layers, sv_dtype io_dt, hipStream_t stream) {
  dim3 grid(s.dv / kRowsPerBlock, s.H, s.B * n_layers);
  dim3 block(kThreads);
  if (io_dt == SV_BF16) {
    if (s.dk == 128) hipLaunchKernelGGL((gdn_commit_multi_kernel<bf16_t, 128>), grid, block, 0, stream, s, t);
    else hipLaunchKernelGGL((gdn_commit_multi_kernel<bf16_t, 64>), grid, block, 0, stream, s, t);
  } else {
    if (s.dk == 128) hipLaunchKernelGGL((gdn_commit_multi_kernel<float, 128>), grid, block, 0, stream, s, t);
    else hipLaunchKernelGGL((gdn_commit_multi_kernel<float, 64>), grid, block, 0, stream, s, t);
  }
  return hipGetLastError();
}

}  // namespace sv
