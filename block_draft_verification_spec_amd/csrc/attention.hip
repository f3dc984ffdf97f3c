// Paged verification attention with KV write-through, split over the context.
//
// lmdeploy pull request 5019 (feature list): the target checks a fixed chain
// of drafts in one pass with paged verification attention, so verify token j
// of sequence b attends to the L_b cached positions and to the in-flight
// positions L_b .. L_b + j (plain causal mask).  Logical position p lives in
// page block_table[b, p / P] at slot p % P of a [num_pages, Hkv, P, D] pool
// (the dense read-back of such a sequence is the flatten_kv_cache gather of
// lmdeploy pull request 3945).  In-flight K/V come from k_new / v_new and are
// written through into their slots (onnxruntime-genai pull request 2457: the
// KV append is an idempotent in-place write; the length update happens after
// acceptance).
//
// bf16 path (one workgroup = 4 waves per (split, kv head, sequence)):
//   * the G = Hq / Hkv query heads of a KV head and the T_b verify tokens form
//     M = G * T_b query rows (row m = token m / G, head m % G), padded to
//     16-row tiles; one KV read serves all of them;
//   * the page ids a split touches are read once into LDS, so a tile's K/V
//     loads never wait on a block-table load;
//   * a 64-key tile of K and V is loaded with coalesced 16-byte loads into a
//     ring of register buffers (up to 3 tiles ahead), K is stored row-major
//     in LDS and V transposed (4 keys x 8 dims per thread, transposed in
//     registers);
//   * wave w owns keys 16 w .. 16 w + 15 of every tile:
//       S^T (16 keys x 16 rows) = K Q^T   with mfma_f32_16x16x32_bf16
//       O^T (16 dims x 16 rows) += V^T P^T with mfma_f32_16x16x16bf16_1k
//     so the online-softmax state of a query row and its output columns sit
//     in the same lane and the rescale needs no shuffle;
//   * the 4 waves merge their (max, sum, O) in LDS in a fixed order, and the
//     split writes a partial (fp32) or, if it is the only split of its
//     sequence, the final output;
//   * a combine kernel merges the splits with the log-sum-exp rule
//       m = max_s m_s, l = sum_s e^(m_s - m) l_s, o = sum_s e^(m_s - m) O_s / l.
// fp32 path: one wave per (query token, head), plain VALU online softmax.

#include "device_common.h"
#include "internal.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kKT = 64;  // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short short4_t;
typedef __attribute__((ext_vector_type(4))) float float4_t;

union U16x8 {
  uint4 u;
  bf16x8_t v;
  uint16_t h[8];
};

// 16-bit element e (0..7, a compile-time constant after unrolling) of a
// 16-byte vector, as the low half of a 32-bit value.
__device__ __forceinline__ uint32_t half16(const uint4& u, int e) {
  const uint32_t w = e < 2 ? u.x : (e < 4 ? u.y : (e < 6 ? u.z : u.w));
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

__device__ __forceinline__ int seq_tiles(int L, int T) { return (L + T + kKT - 1) / kKT; }

// Validate a sequence for attention.  Returns false (and maybe flags) if the
// whole sequence must be skipped.
__device__ __forceinline__ bool attn_seq_ok(const AttnArgs& a, int b, int* x0, int* T, int* L,
                                            bool report) {
  *x0 = a.cu[b];
  *T = a.cu[b + 1] - *x0;
  *L = a.ctx_lens[b];
  if (*T < 1 || *T > a.max_T || *x0 < 0 || *x0 + *T > a.total_T || *L < 0) {
    if (report) flag_error(a.err, SV_DERR_SEQLEN);
    return false;
  }
  if (static_cast<long long>(*L) + *T > static_cast<long long>(a.max_pages) * a.P) {
    if (report) flag_error(a.err, SV_DERR_CAPACITY);
    return false;
  }
  return true;
}

// Element offset of (position p, kv head g, dim d0) in the pool, or -1 if the
// page id is outside the pool.
__device__ __forceinline__ long long page_offset(const AttnArgs& a, int b, int g, int p, int d0) {
  const int page = a.block_table[static_cast<size_t>(b) * a.max_pages + p / a.P];
  if (page < 0 || page >= a.num_pages) return -1;
  return ((static_cast<long long>(page) * a.Hkv + g) * a.P + (p % a.P)) * a.D + d0;
}

// --------------------------------------------------------------------------
// bf16 MFMA split kernel
// --------------------------------------------------------------------------
constexpr int kMaxTilesPerSplit = 16;
constexpr int kMaxSplitPages = 72;  // pages a split may touch (tiles_per_split <= 16, P >= 16)

// PF: tiles in flight per workgroup (a ring of register buffers).  Registers
// are the largest staging store of a CU, so the loads of PF tiles are kept
// outstanding while the current tile is computed from LDS.
template <int D, int NQT, int PF>
__global__ __launch_bounds__(kThreads) void attn_split_bf16(AttnArgs a) {
  constexpr int CPK = D / 8;        // 16-byte chunks per key row
  constexpr int KPT = CPK / 4;      // keys per thread per tile (4 or 2)
  constexpr int KS = D + 8;         // K row stride in LDS (bf16 elements)
  constexpr int VS = kKT + 4;       // V^T row stride in LDS
  constexpr int NDT = D / 16;       // 16-dim output tiles
  constexpr int NKS = D / 32;       // k-steps of the QK^T product
  constexpr int ROWS = 16 * NQT;
  __shared__ __attribute__((aligned(16))) uint16_t lds[kKT * KS + D * VS];
  __shared__ float wm[4][ROWS];
  __shared__ float wl[4][ROWS];
  __shared__ int s_pages[kMaxSplitPages];
  uint16_t* Ks = lds;
  uint16_t* Vt = lds + kKT * KS;

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  int x0, T, L;
  if (!attn_seq_ok(a, b, &x0, &T, &L, split == 0 && g == 0 && tid == 0)) return;
  const int ntiles = seq_tiles(L, T);
  const int t_begin = split * a.tiles_per_split;
  if (t_begin >= ntiles) return;
  const int t_end = min(ntiles, t_begin + a.tiles_per_split);
  const int nsplit_b = (ntiles + a.tiles_per_split - 1) / a.tiles_per_split;
  const int G = a.Hq / a.Hkv;
  const int M = G * T;
  const int P = a.P;

  // ---- the split's page ids, read once: positions t_begin*64 .. pos_end-1
  const int pos_end = min(t_end * kKT, L + T);
  const int first_page = (t_begin * kKT) / P;
  const int n_pages = (pos_end - 1) / P - first_page + 1;
  bool bad_page = false;
  if (tid < n_pages) {
    int pid = a.block_table[static_cast<size_t>(b) * a.max_pages + first_page + tid];
    if (pid < 0 || pid >= a.num_pages) {
      bad_page = true;
      pid = -1;
    }
    s_pages[tid] = pid;
  }

  // ---- Q fragments (B operand of S^T = K Q^T): row 16 nt + lr, dims
  // 32 s + 8 lg .. + 7.
  bf16x8_t qf[NQT][NKS];
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    const int m = 16 * nt + lr;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      U16x8 t;
      if (m < M) {
        const int j = m / G, hh = m - j * G;
        const size_t off = (static_cast<size_t>(x0 + j) * a.Hq + g * G + hh) * D + 32 * s + 8 * lg;
        t.u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + off);
      } else {
        t.u = make_uint4(0, 0, 0, 0);
      }
      qf[nt][s] = t.v;
    }
  }
  __syncthreads();

  // ---- per-thread slice of a tile: keys KPT*kb .. +KPT-1, dims 8*dc .. +7
  const int dc = tid % CPK, kb = tid / CPK;
  // Branch-free tile load: every thread issues the same 2 * KPT loads for
  // every tile, so the compiler's wait counts stay exact across the ring.
  // Keys at or past the split's end (pos_end) read a valid dummy row (an
  // in-flight row of the sequence) and are zeroed; they are also masked.
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const uint16_t* kn = static_cast<const uint16_t*>(a.k_new);
  const uint16_t* vn = static_cast<const uint16_t*>(a.v_new);
  auto load_tile = [&](int tile, uint4 (&kreg)[KPT], uint4 (&vreg)[KPT]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int p = tile * kKT + KPT * kb + i;
      const int pc = min(p, pos_end - 1);
      const int pid = s_pages[pc / P - first_page];
      const bool in_ctx = p < L && p < pos_end && pid >= 0;
      const bool in_new = p >= L && p < pos_end;
      const size_t off_c =
          ((static_cast<size_t>(max(pid, 0)) * a.Hkv + g) * P + (pc % P)) * D + 8 * dc;
      const size_t off_n =
          (static_cast<size_t>(x0 + min(max(p - L, 0), T - 1)) * a.Hkv + g) * D + 8 * dc;
      uint4 kv = *reinterpret_cast<const uint4*>(in_ctx ? kc + off_c : kn + off_n);
      uint4 vv = *reinterpret_cast<const uint4*>(in_ctx ? vc + off_c : vn + off_n);
      // zero by mask, not by select: a select lets the compiler move the
      // load under a branch, which breaks the exact wait counts
      const uint32_t keep = (in_ctx || in_new) ? 0xffffffffu : 0u;
      kreg[i] = make_uint4(kv.x & keep, kv.y & keep, kv.z & keep, kv.w & keep);
      vreg[i] = make_uint4(vv.x & keep, vv.y & keep, vv.z & keep, vv.w & keep);
    }
  };

  // Write-through of the in-flight K/V rows into their slots, by the split
  // that owns those positions (reads of them come from k_new / v_new).
  if (a.write_kv) {
    for (int idx = tid; idx < T * CPK; idx += kThreads) {
      const int j = idx / CPK, c = idx - j * CPK;
      const int p = L + j;
      if (p < t_begin * kKT || p >= pos_end) continue;
      const int pid = s_pages[p / P - first_page];
      if (pid < 0) continue;
      const size_t off_c = ((static_cast<size_t>(pid) * a.Hkv + g) * P + (p % P)) * D + 8 * c;
      const size_t off_n = (static_cast<size_t>(x0 + j) * a.Hkv + g) * D + 8 * c;
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.k_cache) + off_c) =
          *reinterpret_cast<const uint4*>(kn + off_n);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.v_cache) + off_c) =
          *reinterpret_cast<const uint4*>(vn + off_n);
    }
  }

  float4_t oacc[NQT][NDT];
  float m_run[NQT], l_run[NQT];
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[nt][dt] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
  const float sl2 = a.scale * kLog2e;

  auto write_lds = [&](const uint4 (&kreg)[KPT], const uint4 (&vreg)[KPT]) __attribute__((always_inline)) {
      // K rows: 16-byte stores; V transposed: KPT keys of one dim per store.
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        *reinterpret_cast<uint4*>(Ks + (KPT * kb + i) * KS + 8 * dc) = kreg[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t hv[KPT];
#pragma unroll
        for (int i = 0; i < KPT; ++i) hv[i] = half16(vreg[i], e);
        uint16_t* dst = Vt + (8 * dc + e) * VS + KPT * kb;
        if constexpr (KPT == 4) {
          uint2 pk;
          pk.x = hv[0] | (hv[1] << 16);
          pk.y = hv[2] | (hv[3] << 16);
          *reinterpret_cast<uint2*>(dst) = pk;
        } else {
          *reinterpret_cast<uint32_t*>(dst) = hv[0] | (hv[1] << 16);
        }
      }
  };
  auto compute_tile = [&](int tile) __attribute__((always_inline)) {
      const int kbase = tile * kKT + 16 * w;  // first key of this wave
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt) {
        float4_t s = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          U16x8 af;
          af.u = *reinterpret_cast<const uint4*>(Ks + (16 * w + lr) * KS + 32 * ks + 8 * lg);
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af.v, qf[nt][ks], s, 0, 0, 0);
        }
        // lane holds S^T[key 4 lg + r][row lr]
        const int m = 16 * nt + lr;
        const int j = m / G;
        const int lim = (m < M) ? L + j : -1;  // last visible position
        float sv[4];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int p = kbase + 4 * lg + r;
          sv[r] = (p <= lim && p < pos_end) ? s[r] * sl2 : -INFINITY;
          tmax = fmaxf(tmax, sv[r]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run[nt], tmax);
        short4_t pf;
        float psum = 0.f;
        if (m_new == -INFINITY) {
          pf = short4_t{0, 0, 0, 0};
        } else {
          const float alpha = exp2f(m_run[nt] - m_new);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint16_t hb = f32_to_bf16(exp2f(sv[r] - m_new));
            pf[r] = static_cast<short>(hb);
            psum += bf16_to_f32(hb);
          }
          l_run[nt] = l_run[nt] * alpha + psum;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) oacc[nt][dt] *= alpha;
          m_run[nt] = m_new;
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const short4_t vf =
              *reinterpret_cast<const short4_t*>(Vt + (16 * dt + lr) * VS + 16 * w + 4 * lg);
          oacc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pf, oacc[nt][dt], 0, 0, 0);
        }
      }
  };
  // one tile: LDS store of its buffer, refill the buffer PF tiles ahead,
  // compute from LDS
  auto consume = [&](int tile, uint4 (&kreg)[KPT], uint4 (&vreg)[KPT]) __attribute__((always_inline)) {
    __syncthreads();  // previous tile's LDS reads are done
    write_lds(kreg, vreg);
    __syncthreads();
    load_tile(tile + PF, kreg, vreg);
    compute_tile(tile);
  };
  // The ring runs a whole number of PF-tile rounds; tiles past t_end are
  // fully masked and read only the dummy row.
  uint4 kr0[KPT], vr0[KPT], kr1[KPT], vr1[KPT], kr2[KPT], vr2[KPT], kr3[KPT], vr3[KPT];
  load_tile(t_begin, kr0, vr0);
  if constexpr (PF > 1) load_tile(t_begin + 1, kr1, vr1);
  if constexpr (PF > 2) load_tile(t_begin + 2, kr2, vr2);
  if constexpr (PF > 3) load_tile(t_begin + 3, kr3, vr3);
  // Fully unrolled (no loop back edge: the compiler would drain every
  // outstanding load there); uniform early exit once the split is done.
#pragma unroll
  for (int round = 0; round < kMaxTilesPerSplit / PF; ++round) {
    const int tile = t_begin + round * PF;
    if (tile >= t_end) break;
    consume(tile, kr0, vr0);
    if constexpr (PF > 1) consume(tile + 1, kr1, vr1);
    if constexpr (PF > 2) consume(tile + 2, kr2, vr2);
    if constexpr (PF > 3) consume(tile + 3, kr3, vr3);
  }
  if (bad_page) flag_error(a.err, SV_DERR_PAGE);

  // ---- merge the four waves in a fixed order
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    float l = l_run[nt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (lg == 0) {
      wm[w][16 * nt + lr] = m_run[nt];
      wl[w][16 * nt + lr] = l;
    }
  }
  __syncthreads();  // also: all LDS tile reads are done
  float* R = reinterpret_cast<float*>(lds);  // [ROWS][D] fp32 (fits in the tile space)
  float scale_w[NQT];
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    const int m = 16 * nt + lr;
    float mm = fmaxf(fmaxf(wm[0][m], wm[1][m]), fmaxf(wm[2][m], wm[3][m]));
    scale_w[nt] = (wm[w][m] == -INFINITY) ? 0.f : exp2f(wm[w][m] - mm);
  }
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          float4* dst = reinterpret_cast<float4*>(R + (16 * nt + lr) * D + 16 * dt + 4 * lg);
          const float4_t v = oacc[nt][dt] * scale_w[nt];
          if (ww == 0) {
            *dst = make_float4(v[0], v[1], v[2], v[3]);
          } else {
            float4 c = *dst;
            *dst = make_float4(c.x + v[0], c.y + v[1], c.z + v[2], c.w + v[3]);
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- this split's result: row m -> (token j, head g*G + hh)
  for (int i = tid; i < M * (D / 4); i += kThreads) {
    const int m = i / (D / 4), d4 = (i - m * (D / 4)) * 4;
    const float mm = fmaxf(fmaxf(wm[0][m], wm[1][m]), fmaxf(wm[2][m], wm[3][m]));
    float ls = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww)
      if (wm[ww][m] != -INFINITY) ls += wl[ww][m] * exp2f(wm[ww][m] - mm);
    const int j = m / G, hh = m - j * G;
    const size_t row = static_cast<size_t>(x0 + j) * a.Hq + g * G + hh;
    const float4 o = *reinterpret_cast<const float4*>(R + m * D + d4);
    if (nsplit_b == 1) {
      const float inv = 1.f / ls;
      uint2 pk;
      pk.x = f32_to_bf16(o.x * inv) | (static_cast<uint32_t>(f32_to_bf16(o.y * inv)) << 16);
      pk.y = f32_to_bf16(o.z * inv) | (static_cast<uint32_t>(f32_to_bf16(o.w * inv)) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * D + d4) = pk;
    } else {
      const size_t pi = row * a.nsplit + split;
      *reinterpret_cast<float4*>(a.part_o + pi * D + d4) = o;
      if (d4 == 0) {
        a.part_ml[2 * pi] = mm;
        a.part_ml[2 * pi + 1] = ls;
      }
    }
  }
}

// --------------------------------------------------------------------------
// log-sum-exp combine of the splits (bf16 path).  A separate launch: the
// kernel boundary makes every split's partial visible, where a device-scope
// fence inside the split kernel would write back and invalidate the whole L2
// of an XCD once per workgroup.
// --------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attn_combine_bf16(AttnArgs a) {
  const int h = blockIdx.x, j = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  int x0, T, L;
  if (!attn_seq_ok(a, b, &x0, &T, &L, false)) return;
  if (j >= T) return;
  const int ntiles = seq_tiles(L, T);
  const int ns = (ntiles + a.tiles_per_split - 1) / a.tiles_per_split;
  if (ns == 1) return;  // written by the split kernel
  const size_t row = static_cast<size_t>(x0 + j) * a.Hq + h;
  const size_t pbase = row * a.nsplit;
  float mm = -INFINITY;
  for (int s = 0; s < ns; ++s) mm = fmaxf(mm, a.part_ml[2 * (pbase + s)]);
  float acc[D / 64];
#pragma unroll
  for (int e = 0; e < D / 64; ++e) acc[e] = 0.f;
  float ls = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float ms = a.part_ml[2 * (pbase + s)];
    if (ms == -INFINITY) continue;
    const float f = exp2f(ms - mm);
    ls += f * a.part_ml[2 * (pbase + s) + 1];
#pragma unroll
    for (int e = 0; e < D / 64; ++e) acc[e] += f * a.part_o[(pbase + s) * D + lane + 64 * e];
  }
  const float inv = 1.f / ls;
#pragma unroll
  for (int e = 0; e < D / 64; ++e)
    static_cast<uint16_t*>(a.out)[row * D + lane + 64 * e] = f32_to_bf16(acc[e] * inv);
}

// --------------------------------------------------------------------------
// fp32 path: one wave per (head, token, sequence)
// --------------------------------------------------------------------------
__global__ __launch_bounds__(64) void attn_f32(AttnArgs a) {
  const int h = blockIdx.x, j = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  int x0, T, L;
  if (!attn_seq_ok(a, b, &x0, &T, &L, h == 0 && j == 0 && lane == 0)) return;
  if (j >= T) return;
  const int D = a.D;
  const int G = a.Hq / a.Hkv;
  const int g = h / G;
  const float* q = static_cast<const float*>(a.q) + (static_cast<size_t>(x0 + j) * a.Hq + h) * D;
  const float* kn = static_cast<const float*>(a.k_new);
  const float* vn = static_cast<const float*>(a.v_new);
  const float* kc = static_cast<const float*>(a.k_cache);
  const float* vc = static_cast<const float*>(a.v_cache);
  __shared__ float qs[128];
  __shared__ float ws[64];
  __shared__ long long offs[64];
  for (int d = lane; d < D; d += 64) qs[d] = q[d];
  // write-through of this token's K/V, once per KV head
  if (a.write_kv && h % G == 0) {
    const long long po = page_offset(a, b, g, L + j, 0);
    if (po >= 0) {
      for (int d = lane; d < D; d += 64) {
        static_cast<float*>(a.k_cache)[po + d] = kn[(static_cast<size_t>(x0 + j) * a.Hkv + g) * D + d];
        static_cast<float*>(a.v_cache)[po + d] = vn[(static_cast<size_t>(x0 + j) * a.Hkv + g) * D + d];
      }
    } else if (lane == 0) {
      flag_error(a.err, SV_DERR_PAGE);
    }
  }
  __syncthreads();
  const int n = L + j + 1;
  float m_run = -INFINITY, l_run = 0.f;
  float o[2] = {0.f, 0.f};
  bool bad = false;
  for (int base = 0; base < n; base += 64) {
    const int p = base + lane;
    float s = -INFINITY;
    long long off = -2;  // -2: in flight, -1: bad page
    if (p < n) {
      const float* kr;
      if (p < L) {
        off = page_offset(a, b, g, p, 0);
        kr = off >= 0 ? kc + off : nullptr;
        if (off < 0) bad = true;
      } else {
        kr = kn + (static_cast<size_t>(x0 + p - L) * a.Hkv + g) * D;
      }
      if (kr) {
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc += qs[d] * kr[d];
        s = acc * a.scale;
      }
    }
    offs[lane] = off;
    const float bm = group_max<64>(s);
    const float m_new = fmaxf(m_run, bm);
    const float alpha = (m_run == -INFINITY) ? 0.f : __expf(m_run - m_new);
    const float pw = (s == -INFINITY) ? 0.f : __expf(s - m_new);
    ws[lane] = pw;
    l_run = l_run * alpha + group_sum<64>(pw);
    __syncthreads();
    o[0] *= alpha;
    o[1] *= alpha;
    const int cnt = min(64, n - base);
    for (int i = 0; i < cnt; ++i) {
      const float wgt = ws[i];
      const long long vo = offs[i];
      const int p2 = base + i;
      const float* vr = vo >= 0 ? vc + vo
                     : (vo == -2 ? vn + (static_cast<size_t>(x0 + p2 - L) * a.Hkv + g) * D : nullptr);
      if (!vr) continue;
      if (lane < D) o[0] += wgt * vr[lane];
      if (lane + 64 < D) o[1] += wgt * vr[lane + 64];
    }
    m_run = m_new;
    __syncthreads();
  }
  if (bad) flag_error(a.err, SV_DERR_PAGE);
  float* out = static_cast<float*>(a.out) + (static_cast<size_t>(x0 + j) * a.Hq + h) * D;
  const float inv = 1.f / l_run;
  if (lane < D) out[lane] = o[0] * inv;
  if (lane + 64 < D) out[lane + 64] = o[1] * inv;
}

template <int D, int NQT>
void launch_bf16(const AttnArgs& a, hipStream_t stream) {
  // deeper prefetch where the accumulators leave room for it
  constexpr int PF = NQT == 1 ? 3 : (NQT == 2 ? 2 : 1);
  hipLaunchKernelGGL((attn_split_bf16<D, NQT, PF>), dim3(a.nsplit, a.Hkv, a.B), dim3(kThreads), 0,
                     stream, a);
}

}  // namespace

void attn_split_plan(int B, int Hkv, int max_pages, int P, int* nsplit, int* tiles_per_split) {
  const long long max_pos = static_cast<long long>(max_pages) * P;
  const int max_tiles = static_cast<int>((max_pos + kKT - 1) / kKT);
  const long long pairs = static_cast<long long>(B) * Hkv;
  const int want = static_cast<int>(std::max<long long>(1, (2048 + pairs - 1) / pairs));
  int tps = (max_tiles + want - 1) / want;
  tps = std::min(kMaxTilesPerSplit, std::max(4, tps));
  *tiles_per_split = tps;
  *nsplit = std::max(1, (max_tiles + tps - 1) / tps);
}

size_t attn_workspace_bytes(int B, int total_T, int Hq, int Hkv, int D, int max_pages, int P,
                            sv_dtype dtype) {
  if (dtype != SV_BF16) return 0;
  int ns, tps;
  attn_split_plan(B, Hkv, max_pages, P, &ns, &tps);
  const size_t rows = static_cast<size_t>(total_T) * Hq * ns;
  const size_t o_bytes = (rows * D * sizeof(float) + 255) & ~size_t(255);
  return o_bytes + rows * 2 * sizeof(float);
}

void attn_workspace_carve(void* ws, int total_T, int Hq, int D, int nsplit, float** part_o,
                          float** part_ml) {
  const size_t rows = static_cast<size_t>(total_T) * Hq * nsplit;
  const size_t o_bytes = (rows * D * sizeof(float) + 255) & ~size_t(255);
  *part_o = static_cast<float*>(ws);
  *part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + o_bytes);
}

hipError_t launch_attention(const AttnArgs& a, sv_dtype dtype, hipStream_t stream) {
  if (dtype == SV_F32) {
    hipLaunchKernelGGL(attn_f32, dim3(a.Hq, a.max_T, a.B), dim3(64), 0, stream, a);
    return hipGetLastError();
  }
  const int G = a.Hq / a.Hkv;
  const int rows = G * a.max_T;
  const int nqt = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
  if (a.D == 128) {
    if (nqt == 1) launch_bf16<128, 1>(a, stream);
    else if (nqt == 2) launch_bf16<128, 2>(a, stream);
    else launch_bf16<128, 4>(a, stream);
  } else {
    if (nqt == 1) launch_bf16<64, 1>(a, stream);
    else if (nqt == 2) launch_bf16<64, 2>(a, stream);
    else launch_bf16<64, 4>(a, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.D == 128)
    hipLaunchKernelGGL((attn_combine_bf16<128>), dim3(a.Hq, a.max_T, a.B), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_combine_bf16<64>), dim3(a.Hq, a.max_T, a.B), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sv
