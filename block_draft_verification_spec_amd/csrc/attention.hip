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
// bf16 path (workgroups of 4 waves streaming balanced tile ranges, see the
// stream kernel below):
//   * the G = Hq / Hkv query heads of a KV head and the T_b verify tokens form
//     M = G * T_b query rows (row m = token m / G, head m % G), padded to
//     16-row tiles; one KV read serves all of them;
//   * the page ids of up to 256 tiles are staged in LDS at a time, so a
//     tile's K/V loads never wait on a block-table load;
//   * a 64-key tile of K and V is loaded with coalesced 16-byte streaming
//     loads into registers one tile ahead of the compute (three workgroups
//     per CU keep enough tiles in flight), K is stored row-major in LDS and
//     V transposed (4 keys x 8 dims per thread, transposed in registers);
//   * wave w owns keys 16 w .. 16 w + 15 of every tile:
//       S^T (16 keys x 16 rows) = K Q^T   with mfma_f32_16x16x32_bf16
//       O^T (16 dims x 16 rows) += V^T P^T with mfma_f32_16x16x16bf16_1k
//     so the online-softmax state of a query row and its output columns sit
//     in the same lane and the rescale needs no shuffle;
//   * the 4 waves merge their (max, sum, O) in LDS in a fixed order.
// INT8 pages (bf16 activations; the main model's kv_cache_quant_type =
// int8_per_channel in the onnxruntime-genai pull request 2457 commit message on
// the MTP head): code = clamp(rint(x / s), -127, 127) with a static fp32 scale
// s per (KV head, channel) for K and for V.  A small kernel first writes the
// in-flight rows' codes into their slots; the stream kernel then reads every
// position from the pages (8 KiB per 64-key tile at D = 128, half the bf16
// bytes), widens each code c to the fp16 value 1152 + c (exact) on the way
// into LDS, the constant taken off once per output, and runs the
// same tiles with fp16 MFMAs: the K scale is folded into Q (q_d s_d rounded to
// fp16), the V scale applied to the accumulated output channel.
// fp32 path: one wave per (query token, head), plain VALU online softmax.

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kKT = 64;  // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(4))) short short4_t;
typedef __attribute__((ext_vector_type(4))) float float4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

union U16x8 {
  uint4 u;
  bf16x8_t v;
  uint16_t h[8];
};

// 16-bit element e (0..7, a compile-time constant after unrolling) of a
// 16-byte vector, as the low half of a 32-bit value.
__device__ __forceinline__ uint32_t half16(u32x4_t u, int e) {
  const uint32_t w = u[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// Four int8 codes (one 32-bit word) -> four fp16 values 1152 + c, exactly:
// the byte with its sign bit flipped is u = c + 128 in 0..255, and placed
// under the fp16 exponent of 1024 it reads 1024 + u.  The constant is never
// subtracted per code: in the scores it adds 1152 sum_d q_d s_d to every key
// of a query row, which the softmax ignores, and in the PV product it adds
// 1152 times the row's weight sum, which the epilogue takes off once.
constexpr float kCodeBias = 1152.f;
__device__ __forceinline__ void i8x4_to_f16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = w ^ 0x80808080u;
  lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// Two fp32 values rounded to nearest even into bf16 or fp16 (element 0 in
// the low half) by one packed conversion, and each half read back as fp32.
typedef __attribute__((ext_vector_type(2))) float float2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
template <bool F16>
__device__ __forceinline__ uint32_t round2_t(float2_t x) {
  if constexpr (F16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2_t));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}
template <bool F16>
__device__ __forceinline__ float lo16_to_f32(uint32_t u) {
  if constexpr (F16)
    return f16_bits_to_f32(static_cast<uint16_t>(u & 0xffffu));
  else
    return __uint_as_float(u << 16);
}
template <bool F16>
__device__ __forceinline__ float hi16_to_f32(uint32_t u) {
  if constexpr (F16)
    return f16_bits_to_f32(static_cast<uint16_t>(u >> 16));
  else
    return __uint_as_float(u & 0xffff0000u);
}

__device__ __forceinline__ int seq_tiles(int L, int T) { return (L + T + kKT - 1) / kKT; }

// Validate a sequence (first row x0, T verify tokens, L cached tokens) for
// attention.  Returns false (and maybe flags) if the whole sequence must be
// skipped.
__device__ __forceinline__ bool attn_seq_valid(const AttnArgs& a, int x0, int T, int L,
                                               bool report) {
  if (T < 1 || T > a.max_T || x0 < 0 || x0 + T > a.total_T || L < 0) {
    if (report) flag_error(a.err, SV_DERR_SEQLEN);
    return false;
  }
  if (static_cast<long long>(L) + T > static_cast<long long>(a.max_pages) * a.P) {
    if (report) flag_error(a.err, SV_DERR_CAPACITY);
    return false;
  }
  return true;
}

__device__ __forceinline__ bool attn_seq_ok(const AttnArgs& a, int b, int* x0, int* T, int* L,
                                            bool report) {
  *x0 = a.cu[b];
  *T = a.cu[b + 1] - *x0;
  *L = a.ctx_lens[b];
  return attn_seq_valid(a, *x0, *T, *L, report);
}

// Element offset of (position p, kv head g, dim d0) in the pool, or -1 if the
// page id is outside the pool.
__device__ __forceinline__ long long page_offset(const AttnArgs& a, int b, int g, int p, int d0) {
  const int page = a.block_table[static_cast<size_t>(b) * a.max_pages + p / a.P];
  if (page < 0 || page >= a.num_pages) return -1;
  return ((static_cast<long long>(page) * a.Hkv + g) * a.P + (p % a.P)) * a.D + d0;
}

// --------------------------------------------------------------------------
// bf16 MFMA stream kernel
// --------------------------------------------------------------------------
// Work split: the (sequence, KV head) segments are laid end to end as one
// sequence of N 64-key tiles (segment s = b * Hkv + g holds the tiles of
// sequence b, head g, in position order).  Each segment is priced at its
// tiles plus piece_cost() units for the set-up of a piece (bounds, Q, page
// ids, a first tile with none in flight, and the write of its result);
// the U units are split evenly over the W workgroups, workgroup w taking
// units [U w / W, U (w + 1) / W), and a unit range maps to the tiles it
// covers (unit r of a segment is its tile max(r - piece_cost, 0)).  So each
// workgroup's share of the cost is fixed whatever the context lengths: one
// that starts more segments streams fewer tiles.  A segment cut by range
// boundaries is computed in pieces; piece (s, w) of a segment writes its
// partial (max, sum, O) to slot s + w (distinct for every piece, since
// segments advance with w) and the workgroup that owns the segment's first
// tile records which workgroups cover the segment; a combine kernel merges
// the pieces.  A segment covered by one workgroup is written directly.
constexpr int kMaxB = 2048;        // sequences per call on the bf16 path
constexpr int kChunkTiles = 256;   // tiles whose page ids are staged at once
constexpr int kRound = 12;         // tiles per unrolled round (a multiple of PF)
constexpr int kMaxRows = 64;       // query rows per (sequence, KV head)
// Wave priority while a wave issues the next tile's loads (0 while it
// computes), so a CU's waves issue their loads ahead of each other's compute:
// INT8 pages 2.5 % faster per layer, bf16 unchanged.
constexpr int kLoadPrio = 3;

// Split parameters, measured on MI355X (64 sequences of 2048 to 8192 keys,
// 32q/8kv heads, D = 128, 4 verify tokens; 32 sequences of 512 to 4096
// keys; 256 sequences of 16384 to 32768 keys with 2 to 8 verify tokens).
//
// Profile 0, bf16 pages: at most two workgroups per CU (with one 16-row
// query tile the register budget is that of three; see wg_per_cu_cap) and
// a piece set-up priced at 7 tiles, 6 where the workgroups average 32 tiles
// or more (the 64-sequence layer 0.8 % faster at 6; the 32-sequence call,
// at 18 tiles per workgroup, 1.5 % slower at 6): 0.227-0.231 ms per
// 64-sequence layer against 0.239-0.241 ms at three workgroups per CU, and
// 61.6-63.3 against 67-68 us for the 32-sequence call.  One tile in flight
// per workgroup at two workgroups streams faster than at three: a CU's
// memory path is shared, and the third workgroup mostly lengthened the
// queue (a 2-deep register ring at two per CU measured 0.237 ms, one per CU
// 0.270 ms).  The 256-sequence layer (32-row tiles, two per CU by
// registers) measured the same under either profile.
//
// Profile 1, INT8 pages: three workgroups per CU (their tiles carry more
// VALU work per byte; at two per CU they ran 0.136-0.155 against
// 0.132-0.140 ms) and a 3-tile piece set-up.  Shorter ranges for the
// workgroups of later dispatch rounds (a CU's older waves win its
// arbitration) once measured 1 % faster for INT8 pages; with the kernel as
// it is now they measured no faster, and the per-workgroup arithmetic of a
// weighted split slowed every launch's start-up (bf16 pages 0.5-1 %, the
// 32-sequence call 1.5 %), so every profile splits evenly.
// 16-row MFMA tiles of query rows per (sequence, KV head): G max_T rows.
__host__ __device__ constexpr int nqt_for(int G, int max_T) {
  return G * max_T <= 16 ? 1 : (G * max_T <= 32 ? 2 : 4);
}
__host__ __device__ constexpr int split_profile(bool kv8) { return kv8 ? 1 : 0; }
template <int PROF>
constexpr int piece_cost() { return PROF == 0 ? 7 : 3; }
// First unit of workgroup w: U w / W.
__host__ __device__ inline int wg_unit(int w, int W, int U) {
  return static_cast<int>(static_cast<long long>(U) * w / W);
}

// One tile's slice of K and V held by a thread.
template <int KPT>
struct TileRegs {
  u32x4_t k[KPT];
  u32x4_t v[KPT];
};

__host__ __device__ inline int piece_wg(int u, int W, int U) {
  // the workgroup whose range [wg_unit(w), wg_unit(w + 1)) holds unit u: the
  // last w with U w < (u + 1) W
  return min(static_cast<int>(((static_cast<long long>(u) + 1) * W - 1) / U), W - 1);
}

// PF: tiles in flight per workgroup (a ring of register buffers; registers
// are the largest staging store of a CU).
// KV8: INT8 pages (fp16 tiles in LDS and fp16 MFMAs) instead of bf16 pages.
template <int D, int NQT, int PF, bool KV8>
__device__ __forceinline__ void attn_stream_body(const AttnArgs& a) {
  constexpr int DPC = KV8 ? 16 : 8;  // dims per 16-byte chunk
  constexpr int kProf = split_profile(KV8);
  constexpr int kPC = piece_cost<kProf>();  // a piece's set-up, in tiles
  constexpr int CPK = D / DPC;      // 16-byte chunks per key row
  constexpr int KPT = CPK / 4;      // keys per thread per tile (4, 2 or 1)
  constexpr int KS = D + 8;         // K row stride in LDS (16-bit elements)
  constexpr int VS = kKT + 4;       // V^T row stride in LDS
  constexpr int NDT = D / 16;       // 16-dim output tiles
  constexpr int NKS = D / 32;       // k-steps of the QK^T product
  constexpr int ROWS = 16 * NQT;
  static_assert(kRound % PF == 0, "round must hold whole ring turns");
  __shared__ __attribute__((aligned(16))) uint16_t lds[kKT * KS + D * VS];
  __shared__ float wm[4][ROWS];
  __shared__ float wl[4][ROWS];
  // the sequence holding t_lo, its first tile and unit; t_lo, t_hi; that
  // sequence's first verify row, verify tokens and context length
  __shared__ int s_first[8];
  __shared__ int s_ids[kChunkTiles * 4];     // page ids of the current chunk
  __shared__ int s_scan[2][kThreads / 64];
  uint16_t* Ks = lds;
  uint16_t* Vt = lds + kKT * KS;
  // V^T column swizzle: key k of row r sits at column k ^ vswz(r), a multiple
  // of 4 (8 for INT8) that depends on r / 16 only, so the transposed stores
  // of a wave spread over the banks and a read of 4 keys stays contiguous
  auto vswz = [](int r) __attribute__((always_inline)) { return (KV8 ? 8 : 4) * (r >> 4); };

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int B = a.B, Hkv = a.Hkv, G = a.Hq / a.Hkv, P = a.P;

  // ---- tiles of every sequence and their prefix over segments.  Thread tid
  // owns sequences tid * kPer .. tid * kPer + kPer - 1; their cu_seqlens and
  // ctx_lens entries are all loaded (indices clamped) before any is used.
  constexpr int kPer = (kMaxB + kThreads - 1) / kThreads;
  int cuv[kPer + 1], lv[kPer];
#pragma unroll
  for (int i = 0; i <= kPer; ++i) cuv[i] = a.cu[min(tid * kPer + i, B)];
#pragma unroll
  for (int i = 0; i < kPer; ++i) lv[i] = a.ctx_lens[min(tid * kPer + i, B - 1)];
  // one wait for all of them here (the uses below sit in branches, into which
  // the compiler would otherwise move a load and its wait)
#pragma unroll
  for (int i = 0; i <= kPer; ++i) asm volatile("" : "+v"(cuv[i]));
#pragma unroll
  for (int i = 0; i < kPer; ++i) asm volatile("" : "+v"(lv[i]));
  int nts[kPer];  // tiles per segment of each sequence (0: no tiles)
  int run = 0, srun = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = tid * kPer + i;
    nts[i] = 0;
    if (b < B && attn_seq_valid(a, cuv[i], cuv[i + 1] - cuv[i], lv[i], blockIdx.x == 0))
      nts[i] = seq_tiles(lv[i], cuv[i + 1] - cuv[i]);
    run += nts[i] * Hkv;
    srun += nts[i] > 0 ? Hkv : 0;  // segments with tiles
  }
  // inclusive scans of the per-thread tile and segment counts: within each wave
  // by shuffles, then the totals of the waves before it
  int inc = run, sinc = srun;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(inc, off, 64), ys = __shfl_up(sinc, off, 64);
    if (lane >= off) {
      inc += y;
      sinc += ys;
    }
  }
  if (lane == 63) {
    s_scan[0][w] = inc;
    s_scan[1][w] = sinc;
  }
  __syncthreads();
  int excl = inc - run, sexcl = sinc - srun;
  for (int ww = 0; ww < w; ++ww) {
    excl += s_scan[0][ww];
    sexcl += s_scan[1][ww];
  }
  const int N = s_scan[0][0] + s_scan[0][1] + s_scan[0][2] + s_scan[0][3];
  const int NS = s_scan[1][0] + s_scan[1][1] + s_scan[1][2] + s_scan[1][3];
  const int W = gridDim.x, wg = blockIdx.x;
  // the piece set-up in tiles: one less for bf16 pages with long ranges
  const int pc = (kProf == 0 && N >= 32 * W) ? kPC - 1 : kPC;
  const int U = N + pc * NS;
  const int uexcl = excl + pc * sexcl;
  if (wg == 0 && tid == 0) a.seg_meta[2 * B * Hkv] = U;  // for the combine launch
  const int u_lo = wg_unit(wg, W, U);
  const int u_hi = wg_unit(wg + 1, W, U);
  // the sequences whose units hold u_lo and u_hi: their owners map them to
  // tiles (sequences without tiles own no units and never match; unit U maps
  // to tile N)
  {
    int pre = excl, upre = uexcl;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int nt = nts[i], uend = upre + (nt > 0 ? (nt + pc) * Hkv : 0);
      auto tile_of = [&](int u) {
        const int r = u - upre, h = r / (nt + pc);
        return pre + h * nt + max(r - h * (nt + pc) - pc, 0);
      };
      if (u_lo >= upre && u_lo < uend) {
        s_first[0] = tid * kPer + i;
        s_first[1] = pre;
        s_first[2] = upre;
        s_first[3] = tile_of(u_lo);
        s_first[5] = cuv[i];
        s_first[6] = cuv[i + 1] - cuv[i];
        s_first[7] = lv[i];
      }
      if (u_hi >= upre && u_hi < uend) s_first[4] = tile_of(u_hi);
      pre += nt * Hkv;
      upre = uend;
    }
  }
  __syncthreads();
  const int t_lo = u_lo < U ? s_first[3] : N;
  const int t_hi = u_hi < U ? s_first[4] : N;

  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const uint16_t* kn = static_cast<const uint16_t*>(a.k_new);
  const uint16_t* vn = static_cast<const uint16_t*>(a.v_new);
  const int8_t* kc8 = static_cast<const int8_t*>(a.k_cache);
  const int8_t* vc8 = static_cast<const int8_t*>(a.v_cache);
  const int dc = tid % CPK, kb = tid / CPK;  // thread's slice: keys KPT*kb.., dims DPC*dc..
  const float sl2 = a.scale * kLog2e;
  bool bad_page = false;

  // State of the current piece and chunk (function scope, read by the
  // always-inlined helpers below).
  int b = 0, g = 0, x0 = 0, T = 1, L = 0, M = 1, pos_end = 1, first_page = 0;
  int last_tile = 0, last_pg = 0;   // of the current chunk
  const int ps = __builtin_ctz(P);  // the page size is a power of two
  const int toff = KPT * kb;        // the thread's first key in a tile
  using QF = std::conditional_t<KV8, f16x8_t, bf16x8_t>;
  QF qf[NQT][NKS];
  float4_t oacc[NQT][NDT];
  float m_run[NQT], l_run[NQT];

  // Tile load: every thread issues the same 2 * KPT loads for every tile,
  // so the compiler's wait counts stay exact; the page lookup and address are
  // computed once per tile (a thread's keys share one page).  A key at or
  // past pos_end is masked in the scores, so it gets probability exactly 0;
  // what it reads must only be finite: an in-flight row (bf16) or any code
  // (INT8).  Nothing is done to the loaded values before they are stored to
  // LDS, so no instruction waits on a load earlier than the tile's own turn.
  auto load_tile = [&](int tile) __attribute__((always_inline)) {
    TileRegs<KPT> r;
    if (tile > last_tile) {  // prefetch past the chunk, never computed: read
                             // the sequence's first in-flight row (small, hot)
      const size_t off_n = (static_cast<size_t>(x0) * Hkv + g) * D + 8 * dc;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        r.k[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kn + off_n));
        r.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vn + off_n));
      }
      return r;
    }
    // the thread's KPT keys share one page (P >= 16 >= KPT and pos is a
    // multiple of KPT)
    const int pos = tile * kKT + toff;
    const int pid = s_ids[min((pos >> ps) - first_page, last_pg)];
    // every id is inside the pool: a sequence with a bad one is skipped
    const size_t base =
        ((static_cast<size_t>(max(pid, 0)) * Hkv + g) * P + (pos & (P - 1))) * D + DPC * dc;
    if constexpr (KV8) {
      // every position, in-flight ones included, is read from the pages
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        r.k[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kc8 + base + i * D));
        r.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vc8 + base + i * D));
      }
      return r;
    }
    if (tile * kKT + kKT <= L) {  // context keys only (block-uniform)
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        r.k[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kc + base + i * D));
        r.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vc + base + i * D));
      }
      return r;
    }
    // in-flight keys come from k_new / v_new (past the end: a valid row,
    // masked in the scores)
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int p = pos + i;
      const bool in_ctx = p < L && pid >= 0;
      const size_t off_n =
          (static_cast<size_t>(x0 + min(max(p - L, 0), T - 1)) * Hkv + g) * D + DPC * dc;
      r.k[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(in_ctx ? kc + base + i * D : kn + off_n));
      r.v[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(in_ctx ? vc + base + i * D : vn + off_n));
    }
    return r;
  };
  // K rows: 16-byte stores; V transposed: KPT keys of one dim per store.
  auto write_lds = [&](const TileRegs<KPT>& r) __attribute__((always_inline)) {
    if constexpr (KV8) {
      // 16 codes per register quad -> 16 fp16 values (two quads)
      u32x4_t kh[KPT][2], vh[KPT][2];
#pragma unroll
      for (int i = 0; i < KPT; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint32_t lo, hi;
          i8x4_to_f16(r.k[i][c], lo, hi);
          kh[i][c >> 1][2 * (c & 1)] = lo;
          kh[i][c >> 1][2 * (c & 1) + 1] = hi;
          i8x4_to_f16(r.v[i][c], lo, hi);
          vh[i][c >> 1][2 * (c & 1)] = lo;
          vh[i][c >> 1][2 * (c & 1) + 1] = hi;
        }
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(Ks + (KPT * kb + i) * KS + 16 * dc);
        dst[0] = kh[i][0];
        dst[1] = kh[i][1];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        uint16_t* dst = Vt + (16 * dc + e) * VS + ((KPT * kb) ^ vswz(16 * dc + e));
        if constexpr (KPT == 2) {
          *reinterpret_cast<uint32_t*>(dst) =
              half16(vh[0][e >> 3], e & 7) | (half16(vh[1][e >> 3], e & 7) << 16);
        } else {
          *dst = static_cast<uint16_t>(half16(vh[0][e >> 3], e & 7));
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      *reinterpret_cast<u32x4_t*>(Ks + (KPT * kb + i) * KS + 8 * dc) = r.k[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t hv[KPT];
#pragma unroll
      for (int i = 0; i < KPT; ++i) hv[i] = half16(r.v[i], e);
      uint16_t* dst = Vt + (8 * dc + e) * VS + ((KPT * kb) ^ vswz(8 * dc + e));
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
  // wave w owns keys 16 w .. 16 w + 15 of the tile
  auto compute_tile = [&](int tile) __attribute__((always_inline)) {
    const int kbase = tile * kKT + 16 * w;
    // a tile of context keys below pos_end needs only the padding-row mask
    const bool inner = (tile + 1) * kKT <= min(L, pos_end);
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
      float4_t sacc = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const u32x4_t araw =
            *reinterpret_cast<const u32x4_t*>(Ks + (16 * w + lr) * KS + 32 * ks + 8 * lg);
        if constexpr (KV8)
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, araw),
                                                        qf[nt][ks], sacc, 0, 0, 0);
        else
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, araw),
                                                         qf[nt][ks], sacc, 0, 0, 0);
      }
      // lane holds S^T[key 4 lg + r][row lr]
      const int m = 16 * nt + lr;
      float sv[4];
      float tmax = -INFINITY;
      if (inner) {  // every key visible to every query row of the sequence
        const bool row_ok = m < M;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sv[r] = row_ok ? sacc[r] * sl2 : -INFINITY;
          tmax = fmaxf(tmax, sv[r]);
        }
      } else {
        const int lim = (m < M) ? L + m / G : -1;  // last visible position
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int p = kbase + 4 * lg + r;
          sv[r] = (p <= lim && p < pos_end) ? sacc[r] * sl2 : -INFINITY;
          tmax = fmaxf(tmax, sv[r]);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run[nt], tmax);
      short4_t pf;
      if (m_new == -INFINITY) {
        pf = short4_t{0, 0, 0, 0};
      } else {
        // 2^x by the hardware instruction (arguments <= 0; -inf gives 0)
        const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_new);
        float2_t e01, e23;
        e01[0] = __builtin_amdgcn_exp2f(sv[0] - m_new);
        e01[1] = __builtin_amdgcn_exp2f(sv[1] - m_new);
        e23[0] = __builtin_amdgcn_exp2f(sv[2] - m_new);
        e23[1] = __builtin_amdgcn_exp2f(sv[3] - m_new);
        // the weights rounded to nearest even, two per conversion; the
        // rounded weight enters both the PV product and the normaliser
        const uint32_t w01 = round2_t<KV8>(e01), w23 = round2_t<KV8>(e23);
        pf = __builtin_bit_cast(short4_t, make_uint2(w01, w23));
        float psum = lo16_to_f32<KV8>(w01);
        psum += hi16_to_f32<KV8>(w01);
        psum += lo16_to_f32<KV8>(w23);
        psum += hi16_to_f32<KV8>(w23);
        l_run[nt] = l_run[nt] * alpha + psum;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {  // skip when no row's max moved
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) oacc[nt][dt] *= alpha;
        }
        m_run[nt] = m_new;
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const short4_t vf =
            *reinterpret_cast<const short4_t*>(Vt + (16 * dt + lr) * VS +
                                               ((16 * w + 4 * lg) ^ vswz(16 * dt)));
        if constexpr (KV8)
          oacc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(
              __builtin_bit_cast(f16x4_t, vf), __builtin_bit_cast(f16x4_t, pf), oacc[nt][dt], 0, 0,
              0);
        else
          oacc[nt][dt] =
              __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pf, oacc[nt][dt], 0, 0, 0);
      }
    }
  };
  // one tile: LDS store of its buffer, refill the buffer PF tiles ahead,
  // compute from LDS
  auto consume = [&](int tile, TileRegs<KPT>& slot) __attribute__((always_inline)) {
    __syncthreads();  // previous tile's LDS reads are done
    write_lds(slot);
    __syncthreads();
    __builtin_amdgcn_s_setprio(kLoadPrio);  // the next tile's loads issue first
    slot = load_tile(tile + PF);
    __builtin_amdgcn_s_setprio(0);
    compute_tile(tile);
  };

  TileRegs<KPT> r0, r1, r2;

  // Pieces in order: sequence cb (its first tile is cbase) and its Hkv
  // segments of nt_b tiles; past its last tile the next sequence with tiles.
  int cb = t_lo < t_hi ? s_first[0] : B, cbase = t_lo < t_hi ? s_first[1] : 0;
  int ucbase = t_lo < t_hi ? s_first[2] : 0;  // sequence cb's first unit
  int nt_b = 0;
  bool next_seq = true;
  if (t_lo < t_hi) {  // the first sequence's bounds, as the start-up scan read them
    x0 = s_first[5];
    T = s_first[6];
    L = s_first[7];
    nt_b = seq_tiles(L, T);
    next_seq = false;
  }
  for (int t = t_lo; t < t_hi;) {
    if (next_seq) {
      for (; cb < B; ++cb) {  // skipped: sequences that failed validation
        x0 = a.cu[cb];
        T = a.cu[cb + 1] - x0;
        L = a.ctx_lens[cb];
        if (attn_seq_valid(a, x0, T, L, false)) break;
      }
      if (cb >= B) break;  // not reached: tiles before N belong to valid sequences
      nt_b = seq_tiles(L, T);
      next_seq = false;
    }
    // ---- the piece: segment (b, g) tiles [lt_begin, lt_end)
    b = cb;
    g = (t - cbase) / nt_b;
    const int seg_start = cbase + g * nt_b;
    const int lt_begin = t - seg_start;
    const int lt_end = min(t_hi, seg_start + nt_b) - seg_start;
    const int s = b * Hkv + g;
    const bool whole = lt_begin == 0 && lt_end == nt_b;
    M = G * T;
    // the segment's last tile is its unit kPC + nt_b - 1
    const int seg_last_wg =
        piece_wg(ucbase + g * (nt_b + pc) + pc + nt_b - 1, W, U);
    t = seg_start + lt_end;
    if (t == cbase + Hkv * nt_b) {
      cbase = t;
      ucbase += Hkv * (nt_b + pc);
      ++cb;
      next_seq = true;
    }

    // The first chunk's page ids (the first 4 * kThreads of the sequence, four
    // per thread) are loaded before the Q fragments, so that the two round
    // trips overlap; the staging below uses them.
    const int* bt = a.block_table + static_cast<size_t>(b) * a.max_pages;
    const int npg = (L + T - 1) / P + 1;  // pages the sequence uses
    int pid0[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) pid0[u] = bt[min(u * kThreads + tid, npg - 1)];

    // Q fragments (B operand of S^T = K Q^T): row 16 nt + lr, dims 32 s + 8 lg ..
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
      const int m = 16 * nt + lr;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        U16x8 tq;
        if (m < M) {
          const int j = m / G, hh = m - j * G;
          const size_t off =
              (static_cast<size_t>(x0 + j) * a.Hq + g * G + hh) * D + 32 * ks + 8 * lg;
          tq.u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + off);
        } else {
          tq.u = make_uint4(0, 0, 0, 0);
        }
        if constexpr (KV8) {
          // fold the K channel scales into q: q_d s_d, rounded to fp16
          const float* ksc = a.k_scale + static_cast<size_t>(g) * D + 32 * ks + 8 * lg;
          const float4 s0 = *reinterpret_cast<const float4*>(ksc);
          const float4 s1 = *reinterpret_cast<const float4*>(ksc + 4);
          const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
          f16x8_t qh;
#pragma unroll
          for (int e = 0; e < 8; ++e) qh[e] = static_cast<_Float16>(bf16_to_f32(tq.h[e]) * sc[e]);
          qf[nt][ks] = qh;
        } else {
          qf[nt][ks] = tq.v;
        }
      }
    }
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
      m_run[nt] = -INFINITY;
      l_run[nt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[nt][dt] = float4_t{0.f, 0.f, 0.f, 0.f};
    }

    bool seq_bad = false;
    for (int c0 = lt_begin; c0 < lt_end; c0 += kChunkTiles) {
      const int c1 = min(lt_end, c0 + kChunkTiles);
      pos_end = min(c1 * kKT, L + T);  // keys at or past it are masked
      first_page = (c0 * kKT) / P;
      const int n_pages = (pos_end - 1) / P - first_page + 1;
      last_tile = (pos_end - 1) / kKT;
      last_pg = n_pages - 1;
      __syncthreads();  // the previous chunk is done with s_ids and the tile LDS
      if (c0 == lt_begin) {
        // The piece's first chunk checks every page id the sequence uses
        // (positions 0 .. L + T - 1) while it stages its own: a sequence with
        // an id outside the pool is skipped by all of its pieces (no output,
        // no append) and flagged.  Four loads per thread are issued before
        // any is used.
        int bad = 0;
        auto check = [&](int i0, const int (&pid)[4]) __attribute__((always_inline)) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * kThreads + tid, li = i - first_page;
            if (i < npg) {
              bad |= (pid[u] < 0 || pid[u] >= a.num_pages) ? 1 : 0;
              if (li >= 0 && li < n_pages) s_ids[li] = pid[u];
            }
          }
        };
        check(0, pid0);
        for (int i0 = 4 * kThreads; i0 < npg; i0 += 4 * kThreads) {
          int pid[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) pid[u] = bt[min(i0 + u * kThreads + tid, npg - 1)];
          check(i0, pid);
        }
        // one flag per wave (s_scan is free after the start-up), one barrier
        const bool wave_bad = __builtin_amdgcn_ballot_w64(bad != 0) != 0;
        if (lane == 0) s_scan[0][w] = wave_bad ? 1 : 0;
        __syncthreads();
        seq_bad = (s_scan[0][0] | s_scan[0][1] | s_scan[0][2] | s_scan[0][3]) != 0;
        if (lt_begin == 0 && tid == 0) {  // the combine's record of the segment
          // first > last: nothing to merge (a skipped sequence)
          a.seg_meta[2 * s] = seq_bad ? 1 : wg;
          a.seg_meta[2 * s + 1] = seq_bad ? 0 : seg_last_wg;
        }
        if (seq_bad) break;
      } else {  // later chunks of a long piece: ids already checked
        for (int i = tid; i < n_pages; i += kThreads) s_ids[i] = bt[first_page + i];
        __syncthreads();
      }

      r0 = load_tile(c0);
      if constexpr (PF > 1) r1 = load_tile(c0 + 1);
      if constexpr (PF > 2) r2 = load_tile(c0 + 2);
      // Rounds of kRound tiles are unrolled: inside a round the ring's wait
      // counts are exact; the compiler drains outstanding loads only at the
      // round's back edge, which the PF-deep prefetch has already covered.
      for (int tile = c0; tile < c1; tile += kRound) {
#pragma unroll
        for (int u = 0; u < kRound; u += PF) {
          if (tile + u >= c1) break;
          consume(tile + u, r0);
          if constexpr (PF > 1) {
            if (tile + u + 1 >= c1) break;
            consume(tile + u + 1, r1);
          }
          if constexpr (PF > 2) {
            if (tile + u + 2 >= c1) break;
            consume(tile + u + 2, r2);
          }
        }
      }
      // write-through of the in-flight K/V rows that fall in this chunk (after
      // its tiles: their reads of those positions come from k_new / v_new, so
      // no tile load waits behind these copies)
      if (!KV8 && a.write_kv) {
        for (int idx = tid; idx < T * CPK; idx += kThreads) {
          const int j = idx / CPK, c = idx - j * CPK;
          const int p = L + j;
          if (p < c0 * kKT || p >= pos_end) continue;
          const int pid = s_ids[p / P - first_page];
          if (pid < 0) continue;
          const size_t off_c = ((static_cast<size_t>(pid) * Hkv + g) * P + (p % P)) * D + 8 * c;
          const size_t off_n = (static_cast<size_t>(x0 + j) * Hkv + g) * D + 8 * c;
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.k_cache) + off_c) =
              *reinterpret_cast<const uint4*>(kn + off_n);
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.v_cache) + off_c) =
              *reinterpret_cast<const uint4*>(vn + off_n);
        }
      }
    }

    if (seq_bad) {
      if (tid == 0) bad_page = true;
      continue;
    }

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
      const float mm = fmaxf(fmaxf(wm[0][m], wm[1][m]), fmaxf(wm[2][m], wm[3][m]));
      scale_w[nt] = (wm[w][m] == -INFINITY) ? 0.f : exp2f(wm[w][m] - mm);
    }
    // One 16-row tile: each wave writes its rows to a region of its own (the
    // four fit in the tile space) and the result loop scales and adds them in
    // wave order, behind one barrier; more tiles: the waves scale and add into
    // one region in turn.  Either way the sum is
    // fma(O3, s3, fma(O2, s2, fma(O1, s1, O0 * s0))).
    constexpr bool kOwnRegions = NQT == 1;
    static_assert(!kOwnRegions || 4 * 16 * D * 4 <= (kKT * KS + D * VS) * 2,
                  "four waves' rows fit in the tile space");
    if constexpr (kOwnRegions) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        float4* dst = reinterpret_cast<float4*>(R + (w * 16 + lr) * D + 16 * dt + 4 * lg);
        const float4_t v = oacc[0][dt];
        *dst = make_float4(v[0], v[1], v[2], v[3]);
      }
      __syncthreads();
    } else {
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
                const float4 c = *dst;
                const float4_t o = oacc[nt][dt];
                const float sw = scale_w[nt];
                *dst = make_float4(fmaf(o[0], sw, c.x), fmaf(o[1], sw, c.y), fmaf(o[2], sw, c.z),
                                   fmaf(o[3], sw, c.w));
              }
            }
          }
        }
        __syncthreads();
      }
    }

    // ---- the piece's result: row m -> (token m / G, head g * G + m % G)
    for (int i = tid; i < M * (D / 4); i += kThreads) {
      const int m = i / (D / 4), d4 = (i - m * (D / 4)) * 4;
      const float mm = fmaxf(fmaxf(wm[0][m], wm[1][m]), fmaxf(wm[2][m], wm[3][m]));
      float ls = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww)
        if (wm[ww][m] != -INFINITY) ls += wl[ww][m] * exp2f(wm[ww][m] - mm);
      float4 o = *reinterpret_cast<const float4*>(R + m * D + d4);
      if constexpr (kOwnRegions) {
        const float s0 = (wm[0][m] == -INFINITY) ? 0.f : exp2f(wm[0][m] - mm);
        o = make_float4(o.x * s0, o.y * s0, o.z * s0, o.w * s0);
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
          const float sw = (wm[ww][m] == -INFINITY) ? 0.f : exp2f(wm[ww][m] - mm);
          const float4 c = *reinterpret_cast<const float4*>(R + (ww * 16 + m) * D + d4);
          o = make_float4(fmaf(c.x, sw, o.x), fmaf(c.y, sw, o.y), fmaf(c.z, sw, o.z),
                          fmaf(c.w, sw, o.w));
        }
      }
      if constexpr (KV8) {  // the codes' bias (weight sum ls), then the V channel scales
        const float4 vs = *reinterpret_cast<const float4*>(a.v_scale + static_cast<size_t>(g) * D + d4);
        const float bias = kCodeBias * ls;
        o = make_float4((o.x - bias) * vs.x, (o.y - bias) * vs.y, (o.z - bias) * vs.z,
                        (o.w - bias) * vs.w);
      }
      if (whole) {
        const int j = m / G, hh = m - j * G;
        const size_t row = static_cast<size_t>(x0 + j) * a.Hq + g * G + hh;
        const float inv = 1.f / ls;
        uint2 pk;
        pk.x = f32_to_bf16(o.x * inv) | (static_cast<uint32_t>(f32_to_bf16(o.y * inv)) << 16);
        pk.y = f32_to_bf16(o.z * inv) | (static_cast<uint32_t>(f32_to_bf16(o.w * inv)) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * D + d4) = pk;
      } else {
        const size_t pi = static_cast<size_t>(s + wg) * kMaxRows + m;
        *reinterpret_cast<float4*>(a.part_o + pi * D + d4) = o;
        if (d4 == 0) {
          a.part_ml[2 * pi] = mm;
          a.part_ml[2 * pi + 1] = ls;
        }
      }
    }
  }
  if (bad_page) flag_error(a.err, SV_DERR_PAGE);
}

// WPE: waves per SIMD the register allocation is held to (workgroups per
// CU; the LDS of three fits in one CU).
template <int D, int NQT, int PF, int WPE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void attn_stream_bf16(AttnArgs a) {
  attn_stream_body<D, NQT, PF, false>(a);
}

template <int D, int NQT, int PF, int WPE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void attn_stream_kv8(AttnArgs a) {
  attn_stream_body<D, NQT, PF, true>(a);
}

// --------------------------------------------------------------------------
// INT8 pages: the in-flight rows' codes, written before the stream kernel
// reads them.  One workgroup per (verify token, sequence); four channels per
// thread: code = clamp(rint(x / s), -127, 127) with the fp32 quotient.
// --------------------------------------------------------------------------
__device__ __forceinline__ uint32_t quant4(uint2 x, float4 s) {
  const float xs[4] = {bf16_to_f32(x.x & 0xffffu), bf16_to_f32(x.x >> 16),
                       bf16_to_f32(x.y & 0xffffu), bf16_to_f32(x.y >> 16)};
  const float ss[4] = {s.x, s.y, s.z, s.w};
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float c = fminf(fmaxf(rintf(xs[e] / ss[e]), -127.f), 127.f);
    w |= (static_cast<uint32_t>(static_cast<int>(c)) & 0xffu) << (8 * e);
  }
  return w;
}

// True if every page id sequence b uses for positions 0 .. n - 1 (n >= 1) is
// inside the pool.  Block-wide (every thread of the block calls it); each
// wave reduces by ballot, the waves through LDS.
__device__ bool seq_pages_ok(const AttnArgs& a, int b, int n) {
  __shared__ int wave_bad[4];
  const int tid = threadIdx.x, nw = (blockDim.x + 63) / 64;
  const int npg = (n - 1) / a.P + 1;
  const int* bt = a.block_table + static_cast<size_t>(b) * a.max_pages;
  int bad = 0;
  for (int i = tid; i < npg; i += blockDim.x) {
    const int pid = bt[i];
    bad |= (pid < 0 || pid >= a.num_pages) ? 1 : 0;
  }
  const bool wb = __builtin_amdgcn_ballot_w64(bad != 0) != 0;
  if ((tid & 63) == 0) wave_bad[tid >> 6] = wb ? 1 : 0;
  __syncthreads();
  int any = 0;
  for (int i = 0; i < nw; ++i) any |= wave_bad[i];
  __syncthreads();  // the flags may be written again by a later call
  return any == 0;
}

__global__ __launch_bounds__(256) void attn_append_kv8(AttnArgs a) {
  const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int x0, T, L;
  if (!attn_seq_ok(a, b, &x0, &T, &L, false)) return;  // the stream kernel flags it
  if (j >= T) return;
  // a sequence with a page id outside the pool is not appended (the stream
  // kernel flags and skips it)
  if (!seq_pages_ok(a, b, L + T)) return;
  const int p = L + j;
  const int pid = a.block_table[static_cast<size_t>(b) * a.max_pages + p / a.P];
  const int HD = a.Hkv * a.D;
  const size_t src = static_cast<size_t>(x0 + j) * HD;
  for (int c4 = tid; c4 < HD / 4; c4 += 256) {
    const int idx = 4 * c4, g = idx / a.D, d = idx - g * a.D;
    const size_t dst = ((static_cast<size_t>(pid) * a.Hkv + g) * a.P + (p % a.P)) * a.D + d;
    const uint2 kx = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.k_new) + src + idx);
    const uint2 vx = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.v_new) + src + idx);
    *reinterpret_cast<uint32_t*>(static_cast<int8_t*>(a.k_cache) + dst) =
        quant4(kx, *reinterpret_cast<const float4*>(a.k_scale + idx));
    *reinterpret_cast<uint32_t*>(static_cast<int8_t*>(a.v_cache) + dst) =
        quant4(vx, *reinterpret_cast<const float4*>(a.v_scale + idx));
  }
}

// --------------------------------------------------------------------------
// log-sum-exp merge of the pieces of a segment (bf16 path).  A separate
// launch: the kernel boundary makes every piece visible, where a
// device-scope fence inside the stream kernel would write back and
// invalidate the whole L2 of an XCD once per workgroup.
//   m = max_i m_i, l = sum_i e^(m_i - m) l_i, o = sum_i e^(m_i - m) O_i / l
// --------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void attn_combine_bf16(AttnArgs a) {
  // blocks (KV head, sequence, z) share the segment's M = G T_b query rows
  // by 256-float4 slices, one float4 of one row per thread
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x + blockIdx.z * kThreads;
  const int G = a.Hq / a.Hkv;
  const int s = b * a.Hkv + g;
  // the segment's piece record and the sequence bounds are fetched together,
  // with one wait before the first branch (the record is used only once the
  // sequence is known to be valid)
  int wf = a.seg_meta[2 * s], wl_ = a.seg_meta[2 * s + 1];
  int Units = a.seg_meta[2 * a.B * a.Hkv];
  int x0 = a.cu[b], x1 = a.cu[b + 1], L = a.ctx_lens[b];
  asm volatile("" : "+s"(wf), "+s"(wl_), "+s"(Units), "+s"(x0), "+s"(x1), "+s"(L));
  const int T = x1 - x0;
  if (!attn_seq_valid(a, x0, T, L, false)) return;
  if (wf >= wl_) return;  // one piece: written by the stream kernel
  // With few cost units some ranges [wg_unit(w), wg_unit(w + 1)) are empty
  // (never when every workgroup's share U w_r / S(W) is a unit or more); such
  // a workgroup between wf and wl wrote no piece (its slot holds another
  // call's data) and is skipped.  Between the units of the segment's first and
  // last tiles every unit is a tile, so a non-empty unit range there is a
  // non-empty piece.
  const int W = a.n_wg;
  const bool sparse = Units < W;
  constexpr int kFew = 4;  // pieces fetched at once (one round trip)
  int pws[kFew], np = 0;
  for (int w = wf; w <= wl_; ++w) {
    if (sparse && wg_unit(w, W, Units) == wg_unit(w + 1, W, Units)) continue;
    if (np < kFew) pws[np] = w;
    ++np;
  }
  const int M = G * T;
  for (int i = tid; i < M * (D / 4); i += kThreads * gridDim.z) {
    const int m = i / (D / 4), d4 = (i - m * (D / 4)) * 4;
    float mm = -INFINITY, ls = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    auto add = [&](float pm, float pl, float4 po) __attribute__((always_inline)) {
      if (pm == -INFINITY) return;
      const float mn = fmaxf(mm, pm);
      const float fo = mm == -INFINITY ? 0.f : exp2f(mm - mn), fp = exp2f(pm - mn);
      ls = ls * fo + pl * fp;
      acc = make_float4(acc.x * fo + po.x * fp, acc.y * fo + po.y * fp, acc.z * fo + po.z * fp,
                        acc.w * fo + po.w * fp);
      mm = mn;
    };
    if (np <= kFew) {
      float2 ml[kFew];
      float4 po[kFew];
#pragma unroll
      for (int q = 0; q < kFew; ++q) {  // pieces past np re-read piece 0, unused
        const size_t pi = static_cast<size_t>(s + pws[q < np ? q : 0]) * kMaxRows + m;
        ml[q] = *reinterpret_cast<const float2*>(a.part_ml + 2 * pi);
        po[q] = *reinterpret_cast<const float4*>(a.part_o + pi * D + d4);
      }
#pragma unroll
      for (int q = 0; q < kFew; ++q)
        if (q < np) add(ml[q].x, ml[q].y, po[q]);
    } else {
      for (int w = wf; w <= wl_; ++w) {
        if (sparse && wg_unit(w, W, Units) == wg_unit(w + 1, W, Units)) continue;
        const size_t pi = static_cast<size_t>(s + w) * kMaxRows + m;
        const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + 2 * pi);
        add(ml.x, ml.y, *reinterpret_cast<const float4*>(a.part_o + pi * D + d4));
      }
    }
    // row m -> (token m / G, head g G + m % G)
    const int j = m / G, hh = m - j * G;
    const size_t row = static_cast<size_t>(x0 + j) * a.Hq + g * G + hh;
    const float inv = 1.f / ls;
    uint2 pk;
    pk.x = f32_to_bf16(acc.x * inv) | (static_cast<uint32_t>(f32_to_bf16(acc.y * inv)) << 16);
    pk.y = f32_to_bf16(acc.z * inv) | (static_cast<uint32_t>(f32_to_bf16(acc.w * inv)) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * D + d4) = pk;
  }
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
  // a sequence with a page id outside the pool is flagged and skipped: no
  // output, no append
  if (!seq_pages_ok(a, b, L + T)) {
    if (h == 0 && j == 0 && lane == 0) flag_error(a.err, SV_DERR_PAGE);
    return;
  }
  for (int d = lane; d < D; d += 64) qs[d] = q[d];
  // write-through of this token's K/V, once per KV head
  if (a.write_kv && h % G == 0) {
    const long long po = page_offset(a, b, g, L + j, 0);
    for (int d = lane; d < D; d += 64) {
      static_cast<float*>(a.k_cache)[po + d] = kn[(static_cast<size_t>(x0 + j) * a.Hkv + g) * D + d];
      static_cast<float*>(a.v_cache)[po + d] = vn[(static_cast<size_t>(x0 + j) * a.Hkv + g) * D + d];
    }
  }
  __syncthreads();
  const int n = L + j + 1;
  float m_run = -INFINITY, l_run = 0.f;
  float o[2] = {0.f, 0.f};
  for (int base = 0; base < n; base += 64) {
    const int p = base + lane;
    float s = -INFINITY;
    long long off = -2;  // -2: in flight
    if (p < n) {
      const float* kr;
      if (p < L) {
        off = page_offset(a, b, g, p, 0);  // inside the pool (checked above)
        kr = kc + off;
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
  float* out = static_cast<float*>(a.out) + (static_cast<size_t>(x0 + j) * a.Hq + h) * D;
  const float inv = 1.f / l_run;
  if (lane < D) out[lane] = o[0] * inv;
  if (lane + 64 < D) out[lane + 64] = o[1] * inv;
}

// One tile in flight per workgroup.  The register budget is that of three
// resident workgroups per CU (a fourth, at 128 registers, was 10 % slower at
// the 64-sequence hybrid shape); INT8 pages launch three per CU, bf16 pages
// two (wg_per_cu_cap), and a deeper ring in fewer workgroups measured slower
// for both.
template <int D, int NQT>
constexpr int ring_depth() {
  return 1;
}
template <int D, int NQT>
constexpr int waves_per_simd() {
  return NQT == 1 ? 3 : (NQT == 2 ? 2 : 1);
}
// Workgroups launched per CU, at most: split profile 0 (bf16 pages) runs
// two per CU, also where three fit.
constexpr int wg_per_cu_cap(bool kv8) { return split_profile(kv8) == 0 ? 2 : 8; }

template <int D, int NQT, bool KV8>
const void* stream_kernel() {
  if constexpr (KV8)
    return reinterpret_cast<const void*>(
        &attn_stream_kv8<D, NQT, ring_depth<D, NQT>(), waves_per_simd<D, NQT>()>);
  else
    return reinterpret_cast<const void*>(
        &attn_stream_bf16<D, NQT, ring_depth<D, NQT>(), waves_per_simd<D, NQT>()>);
}


template <bool KV8>
const void* stream_kernel_for(int D, int nqt) {
  if (D == 128) {
    if (nqt == 1) return stream_kernel<128, 1, KV8>();
    if (nqt == 2) return stream_kernel<128, 2, KV8>();
    return stream_kernel<128, 4, KV8>();
  }
  if (nqt == 1) return stream_kernel<64, 1, KV8>();
  if (nqt == 2) return stream_kernel<64, 2, KV8>();
  return stream_kernel<64, 4, KV8>();
}

// Resident workgroups of one stream-kernel instance on the current device:
// the grid that keeps every CU busy without a second wave of workgroups.
int stream_grid(int D, int nqt, bool kv8) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, bool>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(dev, D, nqt, kv8);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const void* fn = kv8 ? stream_kernel_for<true>(D, nqt) : stream_kernel_for<false>(D, nqt);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  per_cu = std::min(per_cu, wg_per_cu_cap(kv8));
  const int n = cus * per_cu;
  cache[key] = n;
  return n;
}

// The workspace holds the pieces of the largest grid of either page format.
int stream_grid_max(int D) {
  int n = 0;
  for (int kv8 = 0; kv8 < 2; ++kv8)
    for (int nqt : {1, 2, 4}) n = std::max(n, stream_grid(D, nqt, kv8 != 0));
  return n;
}

template <int D, int NQT>
void launch_stream(const AttnArgs& a, hipStream_t stream) {
  if (a.kv8)
    hipLaunchKernelGGL((attn_stream_kv8<D, NQT, ring_depth<D, NQT>(), waves_per_simd<D, NQT>()>),
                       dim3(a.n_wg), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_stream_bf16<D, NQT, ring_depth<D, NQT>(), waves_per_simd<D, NQT>()>),
                       dim3(a.n_wg), dim3(kThreads), 0, stream, a);
}

}  // namespace

size_t attn_workspace_bytes(int B, int total_T, int Hq, int Hkv, int D, int max_pages, int P,
                            sv_dtype dtype) {
  (void)total_T;
  (void)Hq;
  (void)max_pages;
  (void)P;
  if (dtype != SV_BF16) return 0;
  const size_t slots = static_cast<size_t>(B) * Hkv + stream_grid_max(D);
  const size_t meta = ((static_cast<size_t>(B) * Hkv * 2 + 1) * sizeof(int) + 255) & ~size_t(255);
  const size_t o_bytes = (slots * kMaxRows * D * sizeof(float) + 255) & ~size_t(255);
  return meta + o_bytes + slots * kMaxRows * 2 * sizeof(float);
}

void attn_workspace_carve(void* ws, int B, int Hkv, int D, int n_wg, int** seg_meta,
                          float** part_o, float** part_ml) {
  (void)n_wg;
  const size_t slots = static_cast<size_t>(B) * Hkv + stream_grid_max(D);
  const size_t meta = ((static_cast<size_t>(B) * Hkv * 2 + 1) * sizeof(int) + 255) & ~size_t(255);
  const size_t o_bytes = (slots * kMaxRows * D * sizeof(float) + 255) & ~size_t(255);
  char* base = static_cast<char*>(ws);
  *seg_meta = reinterpret_cast<int*>(base);
  *part_o = reinterpret_cast<float*>(base + meta);
  *part_ml = reinterpret_cast<float*>(base + meta + o_bytes);
}

int attn_stream_grid(int D, int G, int max_T, bool kv8) {
  return stream_grid(D, nqt_for(G, max_T), kv8);
}

// Blocks of the combine per segment: one float4 of the segment's rows per
// thread (G max_T rows of D / 4 float4s).
int combine_z(const AttnArgs& a, int D) {
  const int items = (a.Hq / a.Hkv) * a.max_T * (D / 4);
  return (items + kThreads - 1) / kThreads;
}

hipError_t launch_attention(const AttnArgs& a, sv_dtype dtype, hipStream_t stream) {
  if (dtype == SV_F32) {
    hipLaunchKernelGGL(attn_f32, dim3(a.Hq, a.max_T, a.B), dim3(64), 0, stream, a);
    return hipGetLastError();
  }
  if (a.kv8) {
    hipLaunchKernelGGL(attn_append_kv8, dim3(a.max_T, a.B), dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nqt = nqt_for(a.Hq / a.Hkv, a.max_T);
  if (a.D == 128) {
    if (nqt == 1) launch_stream<128, 1>(a, stream);
    else if (nqt == 2) launch_stream<128, 2>(a, stream);
    else launch_stream<128, 4>(a, stream);
  } else {
    if (nqt == 1) launch_stream<64, 1>(a, stream);
    else if (nqt == 2) launch_stream<64, 2>(a, stream);
    else launch_stream<64, 4>(a, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.D == 128)
    hipLaunchKernelGGL((attn_combine_bf16<128>), dim3(a.Hkv, a.B, combine_z(a, 128)), dim3(kThreads),
                       0, stream, a);
  else
    hipLaunchKernelGGL((attn_combine_bf16<64>), dim3(a.Hkv, a.B, combine_z(a, 64)), dim3(kThreads),
                       0, stream, a);
  return hipGetLastError();
}

}  // namespace sv
