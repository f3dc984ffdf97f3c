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
// Layout of a block: 256 threads = 32 row groups x 8 column lanes.  Thread
// (row group rg, lane c) holds rows rg and rg + 32 and, of each row, the
// elements 32 j + 4 c .. 32 j + 4 c + 3 (j < dk / 32): eight consecutive
// lanes read one 128-byte line of a row per instruction, and a row's dot
// products reduce over 8 lanes in three DPP steps.  Token inputs (at most 8
// pending + 8 current) are staged in LDS as fp32.
//
// The decay costs no per-element multiply: the registers hold S / g with a
// block-uniform scale g (the product of the alphas since the last fold), so
//   S_t = alpha g S' + w k^T = (alpha g) (S' + (w / (alpha g)) k^T),
// i.e. g <- alpha g and one FMA per element.  If alpha g falls below 2^-20
// (alpha = 0 included) the decay is applied to the registers instead.  The
// scale is folded back (g = 1) after the last replayed pending token, so the
// current tokens run exactly as from the committed state loaded afresh; the
// stored state is g S' and storing never changes the registers, so outputs
// do not depend on where (or whether) the state is stored.

#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "conv_block.h"
#include "device_common.h"
#include "internal.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = 64;
constexpr int kRowsPerThread = 2;
constexpr int kLanesPerRow = 8;
constexpr float kMinScale = 0x1p-20f;  // below it the decay is applied, not deferred
constexpr int kMaxTok = 2 * kMaxT;

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// The state is stored as fp32, or as fp16 (rounded to nearest even once per
// store; all arithmetic stays in fp32).
typedef _Float16 h16x4_t __attribute__((ext_vector_type(4)));

template <typename ST>
__device__ __forceinline__ float4 load_state4(const ST* p);
// streaming loads: a launch reads each state element once, and keeping the
// state out of the caches measured 10 % faster once the bank exceeds them
template <>
__device__ __forceinline__ float4 load_state4<float>(const float* p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
template <>
__device__ __forceinline__ float4 load_state4<_Float16>(const _Float16* p) {
  const h16x4_t v = __builtin_nontemporal_load(reinterpret_cast<const h16x4_t*>(p));
  return make_float4(static_cast<float>(v.x), static_cast<float>(v.y),
                     static_cast<float>(v.z), static_cast<float>(v.w));
}

// streaming store: this launch does not read the state again
template <typename ST>
__device__ __forceinline__ void store_state4(ST* p, float x, float y, float z, float w);
template <>
__device__ __forceinline__ void store_state4<float>(float* p, float x, float y, float z,
                                                    float w) {
  const f32x4_t t = {x, y, z, w};
  __builtin_nontemporal_store(t, reinterpret_cast<f32x4_t*>(p));
}
// fp32 -> fp16 of a value already rounded to fp32.  The empty asm pins x in
// a register: otherwise a product feeding the conversion may be contracted
// into one mixed-precision multiply-add that rounds only once (to fp16), and
// the replayed and the stored state would then differ in the last bit.
__device__ __forceinline__ _Float16 to_f16(float x) {
  asm volatile("" : "+v"(x));
  return static_cast<_Float16>(x);
}
template <>
__device__ __forceinline__ void store_state4<_Float16>(_Float16* p, float x, float y, float z,
                                                       float w) {
  const h16x4_t t = {to_f16(x), to_f16(y), to_f16(z), to_f16(w)};
  __builtin_nontemporal_store(t, reinterpret_cast<h16x4_t*>(p));
}

// the value a store and a fresh load would give back
template <typename ST>
__device__ __forceinline__ float as_stored(float x);
template <>
__device__ __forceinline__ float as_stored<float>(float x) {
  return x;
}
template <>
__device__ __forceinline__ float as_stored<_Float16>(float x) {
  return static_cast<float>(to_f16(x));
}

// acc + a . b as a chain of fused multiply-adds
__device__ __forceinline__ float fma4(const float4& a, const float4& b, float acc) {
  acc = fmaf(a.x, b.x, acc);
  acc = fmaf(a.y, b.y, acc);
  acc = fmaf(a.z, b.z, acc);
  return fmaf(a.w, b.w, acc);
}

// Sum over aligned groups of 8 lanes, result in every lane of the group:
// mirror within the half row, then swap lane pairs 2 apart and 1 apart.
__device__ __forceinline__ float lane8_sum(float v) {
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x4e>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0xb1>(v);   // quad_perm [1,0,3,2]
  return v;
}

// One 16-byte chunk of token inputs to fp32 in LDS (dst 16-byte aligned):
// eight bf16 values or four fp32 values.
template <typename LS>
__device__ __forceinline__ void chunk_to_f32(const uint4& r, float* dst);
template <>
__device__ __forceinline__ void chunk_to_f32<uint16_t>(const uint4& r, float* dst) {
  float4* d = reinterpret_cast<float4*>(dst);
  d[0] = make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                     __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
  d[1] = make_float4(__uint_as_float(r.z << 16), __uint_as_float(r.z & 0xffff0000u),
                     __uint_as_float(r.w << 16), __uint_as_float(r.w & 0xffff0000u));
}
template <>
__device__ __forceinline__ void chunk_to_f32<float>(const uint4& r, float* dst) {
  *reinterpret_cast<float4*>(dst) = make_float4(__uint_as_float(r.x), __uint_as_float(r.y),
                                                __uint_as_float(r.z), __uint_as_float(r.w));
}

template <int DK>
struct GdnSmem {
  float k_s[kMaxTok][DK];
  float q_s[kMaxT][DK];
  float v_s[kMaxTok][kRowsPerBlock];
  float a_s[kMaxTok];
  float b_s[kMaxTok];
  float o_s[kMaxT][kRowsPerBlock];
  float kq_s[kMaxT];  // k_t . q_t of the current tokens
};

// COMMIT_ONLY_NP: compile-time COMMIT_ONLY without pending tokens (the
// batched commit of the two-phase step); q, out and the pending pointers are
// then never touched.
// CKPT: verify (mode VERIFY_ONLY, no pending) that also writes the state after
// every token into the checkpoint series, end-aligned: token i of a T-token
// sequence goes to slot window - T + i of ckpt [B][window][H][dv][dk].
template <typename IO, typename ST, int DK, bool COMMIT_ONLY_NP, bool CKPT = false>
__device__ __forceinline__ void gdn_tile(
    GdnSmem<DK>& sm, const GdnScalars& s, void* __restrict__ state, const void* q,
    const void* k, const void* v, const float* __restrict__ alpha,
    const float* __restrict__ beta, void* out, const void* pk, const void* pv,
    const float* __restrict__ palpha, const float* __restrict__ pbeta, int b,
    int h, int rb, bool report, void* __restrict__ ckpt = nullptr) {
  using L = io<IO>;
  constexpr int NV4 = DK / 32;  // float4 per row per thread
  auto& k_s = sm.k_s;
  auto& q_s = sm.q_s;
  auto& v_s = sm.v_s;
  auto& a_s = sm.a_s;
  auto& b_s = sm.b_s;
  auto& o_s = sm.o_s;
  auto& kq_s = sm.kq_s;

  const int tid = threadIdx.x;
  // ---- validate the sequence (uniform over the block).  Every per-sequence
  // value is loaded before any is checked (the guards depend on kernel
  // arguments only), so the block waits one round trip for all of them.
  const bool has_commit = s.mode != SV_GDN_VERIFY_ONLY;
  const bool has_pend = !COMMIT_ONLY_NP && s.has_pending;
  const int x0 = s.cu[b];
  const int x1 = s.cu[b + 1];
  const int slot = s.state_slot ? s.state_slot[b] : b;
  const int c_in = has_commit ? s.commit_len[b] : 0;
  const int p0 = has_pend ? s.p_cu[b] : 0;
  const int p1 = has_pend ? s.p_cu[b + 1] : 1;
  const int pc_in = has_pend ? s.p_commit[b] : 0;
  const int T = x1 - x0;
  const int pT = p1 - p0;
  int bad = 0;
  if (T < 1 || T > s.max_T || x0 < 0 || x0 + T > s.total_T) bad = SV_DERR_SEQLEN;
  else if (slot < 0 || slot >= s.num_slots) bad = SV_DERR_SLOT;
  else if (c_in < 0 || c_in > T) bad = SV_DERR_COMMIT;
  else if (has_pend && (pT < 1 || pT > s.p_max_T || p0 < 0 || p0 + pT > s.p_total_T))
    bad = SV_DERR_SEQLEN;
  else if (pc_in < 0 || pc_in > pT) bad = SV_DERR_COMMIT;
  if (bad) {
    if (report && tid == 0) flag_error(s.err, bad);
    return;
  }
  const int c = c_in;
  const int px0 = p0, pc = pc_in;
  const bool verify = !COMMIT_ONLY_NP && s.mode != SV_GDN_COMMIT_ONLY;
  const int n_cur = verify ? T : c;
  const int n_tot = pc + n_cur;
  // Index of the last token whose effect is stored; -1: nothing is stored.
  const int store_at = (s.mode == SV_GDN_VERIFY_ONLY) ? pc - 1 : pc + c - 1;
  if (!verify && store_at < 0) return;

  const int H = s.H;
  const int DV = s.dv;
  const int row0 = rb * kRowsPerBlock;
  const int cl = tid & (kLanesPerRow - 1);
  const int rg = tid / kLanesPerRow;
  constexpr int kRowStride = kThreads / kLanesPerRow;  // rows rg + kRowStride r
  ST* tile = static_cast<ST*>(state) + (static_cast<size_t>(slot) * H + h) * DV * DK;

  // ---- token inputs: a fixed set of 16-byte loads per thread (chunks of the
  // k and q rows and of this block's slice of the v rows), all issued before
  // any is used, so the block waits one memory round trip for all of them; a
  // chunk past the last token reads token 0 again and is not stored.  Rows are
  // 16-byte aligned (the entry points require aligned q, k, v).
  using LS = typename L::storage;
  constexpr int EPC = 16 / sizeof(LS);                    // elements per chunk
  constexpr int KCH = DK / EPC;                           // chunks per k or q row
  constexpr int VCH = kRowsPerBlock / EPC;                // chunks per v row slice
  constexpr int KN = (kMaxTok * KCH + kThreads - 1) / kThreads;
  constexpr int QN = (kMaxT * KCH + kThreads - 1) / kThreads;
  constexpr int VN = (kMaxTok * VCH + kThreads - 1) / kThreads;
  const LS* kp = static_cast<const LS*>(k);
  const LS* pkp = static_cast<const LS*>(pk);
  const LS* vp = static_cast<const LS*>(v);
  const LS* pvp = static_cast<const LS*>(pv);
  // token t of the stream (replayed pending tokens, then this call's)
  auto tok = [&](int t, const LS* pend, const LS* cur, int width) __attribute__((always_inline)) {
    return t < pc ? pend + (static_cast<size_t>(px0 + t) * H + h) * width
                  : cur + (static_cast<size_t>(x0 + t - pc) * H + h) * width;
  };
  uint4 kr[KN], qr[QN], vr[VN];
#pragma unroll
  for (int i = 0; i < KN; ++i) {
    const int idx = tid + kThreads * i, t = idx / KCH;
    kr[i] = *reinterpret_cast<const uint4*>(tok(t < n_tot ? t : 0, pkp, kp, DK) +
                                            (idx % KCH) * EPC);
  }
  if (verify) {
#pragma unroll
    for (int i = 0; i < QN; ++i) {
      const int idx = tid + kThreads * i, t = idx / KCH;
      qr[i] = *reinterpret_cast<const uint4*>(
          static_cast<const LS*>(q) + (static_cast<size_t>(x0 + (t < T ? t : 0)) * H + h) * DK +
          (idx % KCH) * EPC);
    }
  }
#pragma unroll
  for (int i = 0; i < VN; ++i) {
    const int idx = tid + kThreads * i, t = idx / VCH;
    vr[i] = *reinterpret_cast<const uint4*>(tok(t < n_tot ? t : 0, pvp, vp, DV) + row0 +
                                            (idx % VCH) * EPC);
  }
  float ar = 0.f, br = 0.f;
  if (tid < n_tot) {
    const int t = tid;
    const size_t gi = t < pc ? static_cast<size_t>(px0 + t) * H + h
                             : static_cast<size_t>(x0 + t - pc) * H + h;
    ar = t < pc ? palpha[gi] : alpha[gi];
    br = t < pc ? pbeta[gi] : beta[gi];
  }

  // ---- the state loads: the long-latency traffic
  float4 sr[kRowsPerThread][NV4];
#pragma unroll
  for (int r = 0; r < kRowsPerThread; ++r) {
    const ST* rowp = tile + static_cast<size_t>(row0 + rg + kRowStride * r) * DK;
#pragma unroll
    for (int j = 0; j < NV4; ++j) sr[r][j] = load_state4<ST>(rowp + 32 * j + 4 * cl);
  }

  // ---- token inputs to LDS as fp32
#pragma unroll
  for (int i = 0; i < KN; ++i) {
    const int idx = tid + kThreads * i, t = idx / KCH;
    if (t < n_tot) chunk_to_f32<LS>(kr[i], &k_s[t][(idx % KCH) * EPC]);
  }
  if (verify) {
#pragma unroll
    for (int i = 0; i < QN; ++i) {
      const int idx = tid + kThreads * i, t = idx / KCH;
      if (t < T) chunk_to_f32<LS>(qr[i], &q_s[t][(idx % KCH) * EPC]);
    }
  }
#pragma unroll
  for (int i = 0; i < VN; ++i) {
    const int idx = tid + kThreads * i, t = idx / VCH;
    if (t < n_tot) chunk_to_f32<LS>(vr[i], &v_s[t][(idx % VCH) * EPC]);
  }
  if (tid < n_tot) {
    a_s[tid] = ar;
    b_s[tid] = br;
  }
  __syncthreads();
  // k_t . q_t of every current token, once per block: 16 lanes per token
  if (verify && tid < 16 * T) {
    const int t = tid >> 4, c16 = tid & 15;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < DK / 16; ++e)
      acc = fmaf(k_s[pc + t][16 * e + c16], q_s[t][16 * e + c16], acc);
    acc = row16_sum(acc);
    if (c16 == 0) kq_s[t] = acc;
  }
  __syncthreads();

  // ---- the recurrence, one token at a time (registers hold S / g)
  float g = 1.f;
  for (int i = 0; i < n_tot; ++i) {
    const bool emit = verify && i >= pc;
    // Dot products of both rows with k_t (and q_t), one float4 of k / q at
    // a time so that few registers besides the state are live.
    float uk[kRowsPerThread], uq[kRowsPerThread];
    float kq = 0.f;
#pragma unroll
    for (int r = 0; r < kRowsPerThread; ++r) uk[r] = uq[r] = 0.f;
    if (emit) {
#pragma unroll
      for (int j = 0; j < NV4; ++j) {
        const float4 kj = *reinterpret_cast<const float4*>(&k_s[i][32 * j + 4 * cl]);
        const float4 qj = *reinterpret_cast<const float4*>(&q_s[i - pc][32 * j + 4 * cl]);
#pragma unroll
        for (int r = 0; r < kRowsPerThread; ++r) {
          uk[r] = fma4(sr[r][j], kj, uk[r]);
          uq[r] = fma4(sr[r][j], qj, uq[r]);
        }
      }
      kq = kq_s[i - pc];
#pragma unroll
      for (int r = 0; r < kRowsPerThread; ++r) uq[r] = lane8_sum(uq[r]);
    } else {
#pragma unroll
      for (int j = 0; j < NV4; ++j) {
        const float4 kj = *reinterpret_cast<const float4*>(&k_s[i][32 * j + 4 * cl]);
#pragma unroll
        for (int r = 0; r < kRowsPerThread; ++r) uk[r] = fma4(sr[r][j], kj, uk[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < kRowsPerThread; ++r) uk[r] = lane8_sum(uk[r]);
    const float al = a_s[i];
    const float be = b_s[i];
    float g_new = al * g;  // scale of S_t
    float w[kRowsPerThread];
#pragma unroll
    for (int r = 0; r < kRowsPerThread; ++r) {
      const int rl = rg + kRowStride * r;
      w[r] = be * (v_s[i][rl] - al * (g * uk[r]));
      // o_t = S_t q_t = alpha S_{t-1} q_t + w (k_t . q_t)
      if (emit && cl == 0) o_s[i - pc][rl] = g_new * uq[r] + w[r] * kq;
    }
    if (g_new < kMinScale) {  // block-uniform and rare: apply the decay now
#pragma unroll
      for (int r = 0; r < kRowsPerThread; ++r)
#pragma unroll
        for (int j = 0; j < NV4; ++j) {
          sr[r][j].x *= g_new;
          sr[r][j].y *= g_new;
          sr[r][j].z *= g_new;
          sr[r][j].w *= g_new;
        }
      g_new = 1.f;
    }
    // any fixed reciprocal keeps S = g S' consistent: the hardware one
    const float inv_g = __builtin_amdgcn_rcpf(g_new);
    float wg[kRowsPerThread];
#pragma unroll
    for (int r = 0; r < kRowsPerThread; ++r) wg[r] = w[r] * inv_g;
#pragma unroll
    for (int j = 0; j < NV4; ++j) {
      const float4 kj = *reinterpret_cast<const float4*>(&k_s[i][32 * j + 4 * cl]);
#pragma unroll
      for (int r = 0; r < kRowsPerThread; ++r) {
        sr[r][j].x = fmaf(wg[r], kj.x, sr[r][j].x);
        sr[r][j].y = fmaf(wg[r], kj.y, sr[r][j].y);
        sr[r][j].z = fmaf(wg[r], kj.z, sr[r][j].z);
        sr[r][j].w = fmaf(wg[r], kj.w, sr[r][j].w);
      }
    }
    g = g_new;
    if (i == pc - 1) {  // end of the replayed tokens: fold the scale (and the
                        // storage rounding, so the current tokens run from
                        // exactly the committed state)
#pragma unroll
      for (int r = 0; r < kRowsPerThread; ++r)
#pragma unroll
        for (int j = 0; j < NV4; ++j) {
          sr[r][j].x = as_stored<ST>(sr[r][j].x * g);
          sr[r][j].y = as_stored<ST>(sr[r][j].y * g);
          sr[r][j].z = as_stored<ST>(sr[r][j].z * g);
          sr[r][j].w = as_stored<ST>(sr[r][j].w * g);
        }
      g = 1.f;
    }
    if (i == store_at) {
#pragma unroll
      for (int r = 0; r < kRowsPerThread; ++r) {
        ST* rowp = tile + static_cast<size_t>(row0 + rg + kRowStride * r) * DK;
#pragma unroll
        for (int j = 0; j < NV4; ++j)
          store_state4<ST>(rowp + 32 * j + 4 * cl, g * sr[r][j].x, g * sr[r][j].y,
                           g * sr[r][j].z, g * sr[r][j].w);
      }
    }
    if constexpr (CKPT) {
      ST* ctile = static_cast<ST*>(ckpt) +
                  ((static_cast<size_t>(b) * s.window + (s.window - T + i)) * H + h) * DV * DK;
#pragma unroll
      for (int r = 0; r < kRowsPerThread; ++r) {
        ST* rowp = ctile + static_cast<size_t>(row0 + rg + kRowStride * r) * DK;
#pragma unroll
        for (int j = 0; j < NV4; ++j)
          store_state4<ST>(rowp + 32 * j + 4 * cl, g * sr[r][j].x, g * sr[r][j].y,
                           g * sr[r][j].z, g * sr[r][j].w);
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

template <typename IO, typename ST, int DK, bool CKPT>
__global__ __launch_bounds__(kThreads) void gdn_kernel(GdnScalars s, GdnFullPtrs p) {
  __shared__ GdnSmem<DK> sm;
  const int rb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  gdn_tile<IO, ST, DK, false, CKPT>(sm, s, p.state, p.q, p.k, p.v, p.alpha, p.beta, p.out,
                                    p.pk, p.pv, p.palpha, p.pbeta, b, h, rb,
                                    rb == 0 && h == 0, p.ckpt);
}

// CommitPrefix over the checkpoint series: the slot of the accepted prefix
// becomes the state (c_b = 0 keeps it).  One workgroup per (head, sequence),
// a plain 16-byte copy of the dv x dk tile.
template <typename ST>
__global__ __launch_bounds__(256) void gdn_commit_prefix_kernel(GdnScalars s, const void* ckpt,
                                                                void* state) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const bool report = h == 0 && tid == 0;
  const int x0 = s.cu[b];
  const int T = s.cu[b + 1] - x0;
  if (T < 1 || T > s.max_T || x0 < 0 || x0 + T > s.total_T) {
    if (report) flag_error(s.err, SV_DERR_SEQLEN);
    return;
  }
  const int slot = s.state_slot ? s.state_slot[b] : b;
  if (slot < 0 || slot >= s.num_slots) {
    if (report) flag_error(s.err, SV_DERR_SLOT);
    return;
  }
  const int c = s.commit_len[b];
  if (c < 0 || c > T) {
    if (report) flag_error(s.err, SV_DERR_COMMIT);
    return;
  }
  if (c == 0) return;
  const size_t n16 = static_cast<size_t>(s.dv) * s.dk * sizeof(ST) / 16;
  const uint4* src = static_cast<const uint4*>(ckpt) +
                     ((static_cast<size_t>(b) * s.window + (s.window - T + c - 1)) * s.H + h) * n16;
  uint4* dst = static_cast<uint4*>(state) + (static_cast<size_t>(slot) * s.H + h) * n16;
  for (size_t i = tid; i < n16; i += 256) dst[i] = src[i];
}

// The batched two-phase commit: one block per (64-row block, head,
// sequence, layer), the row block fastest; with CONV, the layers' short
// convolutions follow as blocks of 256 channels per (sequence, layer).
template <typename IO, typename ST, int DK, bool CONV>
__global__ __launch_bounds__(kThreads) void gdn_commit_multi_kernel(GdnScalars s, GdnCommitTable t,
                                                                    ConvArgs c, int n_gdn_blocks) {
  const int blk = blockIdx.x;
  if (CONV && blk >= n_gdn_blocks) {
    const int ncb = (c.C + kConvThreads - 1) / kConvThreads;
    const int r = blk - n_gdn_blocks;
    const int cblk = r % ncb, b = (r / ncb) % c.B, layer = r / (ncb * c.B);
    ConvArgs cl = c;
    cl.state = t.c[layer].state;
    cl.x = t.c[layer].x;
    conv_block_any<IO>(cl, b, cblk);
    return;
  }
  const int nrb = s.dv / kRowsPerBlock;
  const int rb = blk % nrb, h = (blk / nrb) % s.H;
  const int z = blk / (nrb * s.H);
  const int b = z % s.B, layer = z / s.B;
  const GdnCommitPtrs& p = t.l[layer];
  __shared__ GdnSmem<DK> sm;
  gdn_tile<IO, ST, DK, true>(sm, s, p.state, p.k, p.k, p.v, p.alpha, p.beta, p.state,
                         p.k, p.v, p.alpha, p.beta, b, h, rb,
                   rb == 0 && h == 0 && layer == 0);
}

// A layer's GDN verify / commit and its short convolution in one launch.  The
// conv's blocks (256 channels of one sequence each: a few dependent memory
// round trips, little traffic) are spread evenly among the GDN's (row block
// fastest, as in gdn_kernel; bound by the state traffic), so their latency
// overlaps the GDN's streaming instead of trailing it: block i is the conv
// block floor(i Nc / N) when floor((i + 1) Nc / N) moves past it.
template <typename IO, typename ST, int DK>
__global__ __launch_bounds__(kThreads) void gdn_conv_kernel(GdnScalars s, GdnFullPtrs p,
                                                            ConvArgs c, int n_gdn_blocks) {
  const int ncb = (c.C + kConvThreads - 1) / kConvThreads;
  const long long n_conv = static_cast<long long>(ncb) * c.B;
  const long long n_all = n_conv + n_gdn_blocks;
  const long long i = blockIdx.x;
  const int c_lo = static_cast<int>(i * n_conv / n_all);
  const int c_hi = static_cast<int>((i + 1) * n_conv / n_all);
  if (c_hi > c_lo) {
    conv_block_any<IO>(c, c_lo / ncb, c_lo % ncb);
    return;
  }
  const int blk = static_cast<int>(i) - c_lo;  // GDN blocks before this one
  __shared__ GdnSmem<DK> sm;
  const int nrb = s.dv / kRowsPerBlock;
  const int rb = blk % nrb, h = (blk / nrb) % s.H, b = blk / (nrb * s.H);
  gdn_tile<IO, ST, DK, false, false>(sm, s, p.state, p.q, p.k, p.v, p.alpha, p.beta, p.out,
                                     p.pk, p.pv, p.palpha, p.pbeta, b, h, rb,
                                     rb == 0 && h == 0);
}

// Resident blocks per CU of the dk = 128 launches over an fp32 state bank.
// Registers and LDS admit eight; measured on MI355X (32 heads, dk = dv =
// 128; 64 sequences with 4 verify tokens, 256 with 2 to 8), holding a CU to
// five by padding each block's LDS makes a layer 1.5-2 % faster in verify +
// commit and 2-4 % faster in the deferred replay + verify (four: the same;
// three: 7-20 % slower).  With eight, the resident blocks load, compute and
// store in step, and the state traffic pauses while they compute.  An fp16
// bank is bound by its VALU work instead and runs 9 % slower at five, so it
// keeps eight.
constexpr int kGdnBlocksPerCU = 5;

// Dynamic LDS that leaves at most kGdnBlocksPerCU blocks of `kernel` (static
// LDS `fixed` bytes, 256 threads) on a CU of the current device, checked
// with the occupancy query; 0 if the device does not report its LDS size.
size_t gdn_lds_pad(const void* kernel, size_t fixed) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, size_t> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, kernel);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int lds = 0, per_block = 0;
  size_t pad = 0;
  if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) ==
          hipSuccess &&
      hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) ==
          hipSuccess &&
      lds > 0 && per_block > 0) {
    const size_t share = static_cast<size_t>(lds) / kGdnBlocksPerCU;
    const size_t cap = static_cast<size_t>(per_block);
    pad = share > fixed ? ((std::min(share, cap) - fixed) & ~size_t(255)) : 0;
    // the allocation granule may fit one block more or fewer: step the pad
    // until the occupancy query agrees (bounded)
    for (int k = 0; k < 64; ++k) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kThreads, pad) != hipSuccess)
        break;
      if (n > kGdnBlocksPerCU && fixed + pad + 256 <= cap) pad += 256;
      else if (n < kGdnBlocksPerCU && pad >= 256) pad -= 256;
      else break;
    }
  }
  cache[key] = pad;
  return pad;
}

template <typename ST, typename K>
size_t pad_for(K* kernel, int dk) {
  return dk == 128 && std::is_same<ST, float>::value
             ? gdn_lds_pad(reinterpret_cast<const void*>(kernel), sizeof(GdnSmem<128>))
             : 0;
}

template <typename IO, typename ST>
void launch_gdn_t(const GdnScalars& s, const GdnFullPtrs& p, hipStream_t stream) {
  const dim3 grid(s.dv / kRowsPerBlock, s.H, s.B);
  if (p.ckpt) {
    if (s.dk == 128)
      hipLaunchKernelGGL((gdn_kernel<IO, ST, 128, true>), grid, dim3(kThreads), 0, stream, s, p);
    else
      hipLaunchKernelGGL((gdn_kernel<IO, ST, 64, true>), grid, dim3(kThreads), 0, stream, s, p);
  } else {
    if (s.dk == 128)
      hipLaunchKernelGGL((gdn_kernel<IO, ST, 128, false>), grid, dim3(kThreads),
                         pad_for<ST>(&gdn_kernel<IO, ST, 128, false>, 128), stream, s, p);
    else
      hipLaunchKernelGGL((gdn_kernel<IO, ST, 64, false>), grid, dim3(kThreads), 0, stream, s, p);
  }
}

// kernel arguments of the batched commit stay within the 4 KiB argument block
static_assert(sizeof(GdnScalars) + sizeof(GdnCommitTable) + sizeof(ConvArgs) + sizeof(int) + 64 <=
                  4096,
              "batched commit arguments exceed 4 KiB");

template <typename IO, typename ST>
void launch_commit_t(const GdnScalars& s, const GdnCommitTable& t, int n_layers,
                     hipStream_t stream, const ConvArgs* conv) {
  const int n_gdn = (s.dv / kRowsPerBlock) * s.H * s.B * n_layers;
  ConvArgs c{};
  int n_conv = 0;
  if (conv) {
    c = *conv;
    n_conv = (c.C + kConvThreads - 1) / kConvThreads * c.B * n_layers;
  }
  const dim3 grid(n_gdn + n_conv);
  if (conv) {
    if (s.dk == 128)
      hipLaunchKernelGGL((gdn_commit_multi_kernel<IO, ST, 128, true>), grid, dim3(kThreads),
                         pad_for<ST>(&gdn_commit_multi_kernel<IO, ST, 128, true>, 128), stream, s, t,
                         c, n_gdn);
    else
      hipLaunchKernelGGL((gdn_commit_multi_kernel<IO, ST, 64, true>), grid, dim3(kThreads), 0,
                         stream, s, t, c, n_gdn);
  } else {
    if (s.dk == 128)
      hipLaunchKernelGGL((gdn_commit_multi_kernel<IO, ST, 128, false>), grid, dim3(kThreads),
                         pad_for<ST>(&gdn_commit_multi_kernel<IO, ST, 128, false>, 128), stream, s,
                         t, c, n_gdn);
    else
      hipLaunchKernelGGL((gdn_commit_multi_kernel<IO, ST, 64, false>), grid, dim3(kThreads), 0,
                         stream, s, t, c, n_gdn);
  }
}

template <typename IO, typename ST>
void launch_gdn_conv_t(const GdnScalars& s, const GdnFullPtrs& p, const ConvArgs& c,
                       hipStream_t stream) {
  const int n_gdn = (s.dv / kRowsPerBlock) * s.H * s.B;
  const int n_conv = (c.C + kConvThreads - 1) / kConvThreads * c.B;
  const dim3 grid(n_gdn + n_conv);
  if (s.dk == 128)
    hipLaunchKernelGGL((gdn_conv_kernel<IO, ST, 128>), grid, dim3(kThreads),
                       pad_for<ST>(&gdn_conv_kernel<IO, ST, 128>, 128), stream, s, p, c, n_gdn);
  else
    hipLaunchKernelGGL((gdn_conv_kernel<IO, ST, 64>), grid, dim3(kThreads), 0, stream, s, p, c,
                       n_gdn);
}

}  // namespace

hipError_t launch_gdn(const GdnScalars& s, const GdnFullPtrs& p, sv_dtype io_dt,
                      sv_dtype state_dt, hipStream_t stream) {
  const bool h = state_dt == SV_F16;
  if (io_dt == SV_BF16) {
    if (h) launch_gdn_t<bf16_t, _Float16>(s, p, stream);
    else launch_gdn_t<bf16_t, float>(s, p, stream);
  } else {
    if (h) launch_gdn_t<float, _Float16>(s, p, stream);
    else launch_gdn_t<float, float>(s, p, stream);
  }
  return hipGetLastError();
}

hipError_t launch_gdn_commit_multi(const GdnScalars& s, const GdnCommitTable& t,
                                   int n_layers, sv_dtype io_dt, sv_dtype state_dt,
                                   hipStream_t stream, const ConvArgs* conv) {
  const bool h = state_dt == SV_F16;
  if (io_dt == SV_BF16) {
    if (h) launch_commit_t<bf16_t, _Float16>(s, t, n_layers, stream, conv);
    else launch_commit_t<bf16_t, float>(s, t, n_layers, stream, conv);
  } else {
    if (h) launch_commit_t<float, _Float16>(s, t, n_layers, stream, conv);
    else launch_commit_t<float, float>(s, t, n_layers, stream, conv);
  }
  return hipGetLastError();
}

hipError_t launch_gdn_conv(const GdnScalars& s, const GdnFullPtrs& p, const ConvArgs& c,
                           sv_dtype io_dt, sv_dtype state_dt, hipStream_t stream) {
  const bool h = state_dt == SV_F16;
  if (io_dt == SV_BF16) {
    if (h) launch_gdn_conv_t<bf16_t, _Float16>(s, p, c, stream);
    else launch_gdn_conv_t<bf16_t, float>(s, p, c, stream);
  } else {
    if (h) launch_gdn_conv_t<float, _Float16>(s, p, c, stream);
    else launch_gdn_conv_t<float, float>(s, p, c, stream);
  }
  return hipGetLastError();
}

hipError_t launch_gdn_commit_prefix(const GdnScalars& s, const void* ckpt, void* state,
                                    sv_dtype state_dt, hipStream_t stream) {
  const dim3 grid(s.H, s.B);
  if (state_dt == SV_F16)
    hipLaunchKernelGGL(gdn_commit_prefix_kernel<_Float16>, grid, dim3(256), 0, stream, s, ckpt,
                       state);
  else
    hipLaunchKernelGGL(gdn_commit_prefix_kernel<float>, grid, dim3(256), 0, stream, s, ckpt,
                       state);
  return hipGetLastError();
}

}  // namespace sv
