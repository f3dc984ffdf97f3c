// Acceptance of the verified drafts: greedy and rejection sampling.
//
// Greedy (onnxruntime-genai pull request 2457, greedy MTP step and the device
// argmax of all verify rows read back once): g_i = argmax of target row i,
// lowest index on ties; a = leading run of drafts equal to g_i; y = g_a.
// Rejection sampling (Leviathan, Kalman & Matias 2023, Algorithm 1; Chen et
// al. 2023), temperature 1: draft x_i passes iff u_i q_i(x_i) < p_i(x_i); at
// the first failure y is drawn from max(0, p_i - q_i) (from p_i if that is all
// zero), and after k passes from p_k, by inverse CDF in vocabulary order with
// the supplied uniform: y = first index whose running sum exceeds u * total.
// Output rows follow the lmdeploy reject sampler (pull request 3945, review of
// reject_sampler.py): accepted drafts, then y, padded with -1.  As there,
// the draft distribution may be absent (point mass on the draft token:
// accept iff u < p(x), residual p without x) and the bonus token may be
// supplied (used when every draft passes, in place of the last row's argmax
// or draw).
//
// Kernels (all reductions that decide an integer run in fp64, so that the
// decisions agree with an fp64 reference except on a set of uniforms of
// measure ~1e-16 per decision):
//   greedy:    row_argmax_partial  (chunk x row)  -> decide_greedy (sequence)
//   rejection: row_stats_partial   (chunk x row)  -> decide_reject (sequence)
//              -> residual_partial (chunk x seq)  -> final_draw    (sequence)
// A chunk is 4096 vocabulary entries read by 256 threads: with 16-byte loads
// when the rows are 16-byte aligned and V is a multiple of the entries of one
// load, otherwise with coalesced stride-256 element loads, so any V and any
// row alignment is supported.

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "exp2_table.h"
#include "internal.h"

namespace sv {

// Scratch of spec_accept_noalloc: kAcceptScratchBytes in every GPU's copy of
// this code object, kept until the process ends.  Host code never passes the
// array's name to a kernel (on the host it names a stand-in, not device
// memory): accept_scratch() returns the device address of the current GPU's
// copy.  Every call on one GPU shares it; calls that overlap on a GPU race.
static __device__ __align__(256) unsigned char scratch[kAcceptScratchBytes];

hipError_t accept_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {  // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}
namespace {

constexpr int kChunk = 4096;
constexpr int kThreads = 256;
constexpr int kPerThread = kChunk / kThreads;

__host__ __device__ inline int n_chunks(int V) { return (V + kChunk - 1) / kChunk; }

// Whether chunk `chunk` of a row reaches past V (only the row's last chunk
// can): its entries past V are loaded from inside the row and must be masked.
__device__ __forceinline__ bool chunk_has_tail(int chunk, int V) { return (chunk + 1) * kChunk > V; }

// exp(x) for x <= 0 in fp64 for the per-entry work, by the table-driven
// method of P. T. P. Tang (ACM TOMS 15(2), 1989): with k the integer nearest
// to x * 256 / ln 2 and r = x - k ln2 / 256 (|r| <= ln2 / 512, taken in two
// fma steps with ln 2 split into a double and its remainder),
//   exp(x) = 2^(k >> 8) * 2^((k & 255) / 256) * (1 + p(r)),
// p the degree-4 Taylor polynomial of exp(r) - 1, whose remainder
// r^5 / 120 stays below 3.8e-17 relative (a third of an ulp of 1; on 4e7
// host-checked points of [-707, 0] the result is within 1.33 ulp of exp).
// Each block copies the 256 entries 2^(j/256) (correctly rounded doubles,
// exp2_table.h) into LDS.
// Every step is a full-rate fp64 or integer operation: adding 1.5 * 2^52 to
// x * 256 / ln 2 (in one fma) rounds it to the nearest integer, ties to even,
// and leaves that integer in the low word of the sum; the power 2^(k >> 8)
// is applied with one ldexp, exact while the result is normal (x above about
// -708) and rounded once below, so the result underflows gradually to 0
// near -745.  x is first clamped to -800, which maps -inf and NaN to 0.
constexpr int kExpTab = 256;

__device__ __forceinline__ void exp_table_init(double* tab) {
  for (int j = threadIdx.x; j < kExpTab; j += blockDim.x) tab[j] = kExp2Tab[j];
}

struct ExpReduced {
  double pr;   // p(r)
  uint32_t k;  // k, two's complement
};

__device__ __forceinline__ ExpReduced exp_reduce(double xc) {
  constexpr double kShift = 0x1.8p52;
  constexpr double kInvStep = 256.0 / 0.693147180559945309417232121458176568;
  constexpr double kStepHi = 0x1.62e42fefa39efp-1 / 256.0;   // ln 2 rounded to double, / 256
  constexpr double kStepLo = 2.319046813846299558e-17 / 256.0;  // ln 2 minus that double, / 256
  const double ks = fma(xc, kInvStep, kShift);
  const uint32_t ki = static_cast<uint32_t>(__double_as_longlong(ks));
  const double k = ks - kShift;
  double r = fma(-k, kStepHi, xc);
  r = fma(-k, kStepLo, r);
  const double pr = r * fma(r, fma(r, fma(r, 1.0 / 24.0, 1.0 / 6.0), 0.5), 1.0);
  return {pr, ki};
}

__device__ __forceinline__ double exp_nonpos(double x, const double* tab) {
  const ExpReduced e = exp_reduce(fmax(x, -800.0));
  const double t = tab[e.k & (kExpTab - 1)];
  return ldexp(fma(t, e.pr, t), static_cast<int>(e.k) >> 8);
}

// The variant for the row sums.  x is clamped to -707 instead, so every
// result is a normal number and 2^(k >> 8) can go into the table entry's
// exponent field by one integer add: the table (exp_table_init_biased) holds
// 2^(j/256) with j << 12 taken off its high word, and adding k << 12 to that
// word puts j's bits back and adds k >> 8 to the exponent (both exact in
// arithmetic mod 2^32, since k << 12 = ((k >> 8) << 20) + ((k & 255) << 12)).
// On [-707, 0] the result equals exp_nonpos bit for bit.  Below -707 (also
// -inf) it is e^-707, about 9e-308 instead of a smaller value: a chunk sum
// also holds the entry at the chunk's maximum, e^0 = 1, so these terms are
// lost in its rounding.
__device__ __forceinline__ void exp_table_init_biased(uint2* tab) {
  for (int j = threadIdx.x; j < kExpTab; j += blockDim.x) {
    const unsigned long long b = static_cast<unsigned long long>(__double_as_longlong(kExp2Tab[j]));
    tab[j] = make_uint2(static_cast<uint32_t>(b),
                        static_cast<uint32_t>(b >> 32) - (static_cast<uint32_t>(j) << 12));
  }
}

__device__ __forceinline__ double exp_nonpos_sum(double x, const uint2* tab_biased) {
  const ExpReduced e = exp_reduce(fmax(x, -707.0));
  const uint2 w = tab_biased[e.k & (kExpTab - 1)];
  const double t = __hiloint2double(static_cast<int>(w.y + (e.k << 12)), static_cast<int>(w.x));
  return fma(t, e.pr, t);
}

// Workspace layout (byte offsets are 256-aligned).
struct AcceptWs {
  size_t keys, stats, dec, fin, csum, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline AcceptWs accept_ws_layout(int B, int total_T, int V, int mode) {
  AcceptWs w{};
  const int nc = n_chunks(V);
  size_t off = 0;
  w.keys = off;   // greedy: uint64 [total_T][nc]
  if (mode == SV_ACCEPT_GREEDY) off += align256(sizeof(unsigned long long) * size_t(total_T) * nc);
  w.stats = off;  // rejection: double2 {chunk max, chunk sum} [rows][nc]
  const int rows = 2 * total_T - B;
  if (mode == SV_ACCEPT_REJECTION) off += align256(sizeof(double2) * size_t(rows) * nc);
  w.dec = off;    // int4 per sequence {a, kind, target row, draft row}
  off += align256(sizeof(int4) * size_t(B));
  w.fin = off;    // double4 per sequence {Mt, Zt, Md, Zd}
  off += align256(sizeof(double4) * size_t(B));
  w.csum = off;   // double [B][nc]
  off += align256(sizeof(double) * size_t(B) * nc);
  w.total = off;
  return w;
}

template <typename T>
__device__ __forceinline__ float ld(const void* base, size_t i) {
  return io<T>::load(base, i);
}

__device__ __forceinline__ unsigned long long argmax_key(float f, int idx) {
  uint32_t u = __float_as_uint(f);
  if (f == 0.f) u = 0;  // -0 == +0
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(ord) << 32) |
         static_cast<unsigned long long>(0xffffffffu - static_cast<uint32_t>(idx));
}

__device__ __forceinline__ int key_index(unsigned long long key) {
  return static_cast<int>(0xffffffffu - static_cast<uint32_t>(key & 0xffffffffu));
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sequence validation shared by the per-sequence kernels.
__device__ __forceinline__ bool seq_ok(const AcceptArgs& a, int b, int* x0, int* T) {
  *x0 = a.cu[b];
  *T = a.cu[b + 1] - *x0;
  // the k_b = T_b - 1 drafts sit at rows x0 - b .. x0 - b + T_b - 2
  return *T >= 1 && *T <= a.max_T && *x0 >= b && *x0 + *T <= a.total_T &&
         *x0 - b + *T - 1 <= a.total_T - a.B;
}

__device__ void write_outputs(const AcceptArgs& a, int b, int x0, int acc, int y) {
  const int d0 = x0 - b;
  int32_t* row = a.result + a.B + static_cast<size_t>(b) * a.max_T;
  // the accepted drafts, every load issued before the first store (indices
  // clamped into the draft array, which is non-empty whenever acc > 0)
  const int n_drafts = a.total_T - a.B;
  int tok[kMaxT] = {};
  if (n_drafts > 0) {
#pragma unroll
    for (int j = 0; j < kMaxT; ++j) tok[j] = a.draft_tokens[min(d0 + j, n_drafts - 1)];
  }
#pragma unroll
  for (int j = 0; j < kMaxT; ++j)
    if (j < a.max_T) row[j] = j < acc ? tok[j] : (j == acc ? y : -1);
  a.result[b] = acc;
  if (a.commit_len_out) a.commit_len_out[b] = acc + 1;
  if (a.ctx_lens) a.ctx_lens[b] += acc + 1;
}

// A skipped sequence (bad lengths, a draft or bonus id outside the
// vocabulary): accept_len -1, a row of -1 and commit length 0, so a commit
// that follows keeps its recurrent state; its ctx_lens entry is not changed.
__device__ void skip_outputs(const AcceptArgs& a, int b) {
  int32_t* row = a.result + a.B + static_cast<size_t>(b) * a.max_T;
  for (int j = 0; j < a.max_T; ++j) row[j] = -1;
  a.result[b] = -1;
  if (a.commit_len_out) a.commit_len_out[b] = 0;
}

// ------------------------------------------------------- chunk loads
// Entries of one 16-byte load.
template <typename T>
constexpr int kVecN = 16 / static_cast<int>(sizeof(typename io<T>::storage));

// Vocabulary index of a thread's entry e of a chunk.  VEC (rows 16-byte
// aligned and V a multiple of kVecN<T>, checked by the launcher): 16-byte
// group l * kThreads + tid of the chunk holds entries l * kVecN .. of the
// thread; otherwise entry e sits at stride kThreads.
template <typename T, bool VEC>
__device__ __forceinline__ int chunk_entry(int chunk, int tid, int e) {
  constexpr int NV = VEC ? kVecN<T> : 1;
  return chunk * kChunk + ((e / NV) * kThreads + tid) * NV + e % NV;
}

// A thread's kPerThread entries of one chunk of row `row` as loaded (raw
// bits, so that holding them in flight needs no wait), every load issued
// before any is used; an entry past V reads a valid entry of the row and is
// masked by the caller.
template <typename T, bool VEC>
struct ChunkRaw {
  using S = typename io<T>::storage;
  static constexpr int NV = VEC ? kVecN<T> : 1;
  static constexpr int N = VEC ? kPerThread / NV : kPerThread;
  using R = std::conditional_t<VEC, uint4, S>;
  R raw[N];
};

template <typename T, bool VEC>
__device__ __forceinline__ void load_chunk_raw(const void* src, int row, int V, int chunk, int tid,
                                               ChunkRaw<T, VEC>& c) {
  using S = typename io<T>::storage;
  if constexpr (VEC) {
    constexpr int NV = kVecN<T>;
    const uint4* p =
        reinterpret_cast<const uint4*>(static_cast<const S*>(src) + static_cast<size_t>(row) * V);
    const int last = V / NV - 1;
#pragma unroll
    for (int l = 0; l < kPerThread / NV; ++l)
      c.raw[l] = p[min(chunk * (kChunk / NV) + l * kThreads + tid, last)];
  } else {
    const S* p = static_cast<const S*>(src) + static_cast<size_t>(row) * V;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      c.raw[e] = p[min(chunk_entry<T, false>(chunk, tid, e), V - 1)];
  }
}

// The entries as fp32 values (bf16 widens exactly).
template <typename T, bool VEC>
__device__ __forceinline__ void unpack_chunk(const ChunkRaw<T, VEC>& c, float* out) {
  if constexpr (VEC) {
    constexpr int NV = kVecN<T>;
#pragma unroll
    for (int l = 0; l < kPerThread / NV; ++l) {
      const uint32_t w[4] = {c.raw[l].x, c.raw[l].y, c.raw[l].z, c.raw[l].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (NV == 8) {  // two bf16 entries per word, the lower first
          out[l * NV + 2 * q] = __uint_as_float(w[q] << 16);
          out[l * NV + 2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
        } else {
          out[l * NV + q] = __uint_as_float(w[q]);
        }
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if constexpr (std::is_same<T, float>::value) out[e] = c.raw[e];
      else out[e] = bf16_to_f32(c.raw[e]);
    }
  }
}

template <typename T, bool VEC>
__device__ __forceinline__ void load_chunk(const void* src, int row, int V, int chunk, int tid,
                                           float* out) {
  ChunkRaw<T, VEC> c;
  load_chunk_raw<T, VEC>(src, row, V, chunk, tid, c);
  unpack_chunk<T, VEC>(c, out);
}

// ------------------------------------------------------------------ greedy
// The row kernels below are persistent: block i takes the (row, chunk) items
// i, i + grid, ... (chunk fastest) and issues the next item's loads before it
// reduces the current one, so a block always has a chunk in flight.
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void row_argmax_partial(AcceptArgs a, int n_items) {
  const int tid = threadIdx.x;
  const int nc = n_chunks(a.V);
  __shared__ unsigned long long red[kThreads / 64];
  const AcceptWs L = accept_ws_layout(a.B, a.total_T, a.V, a.mode);
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(static_cast<char*>(a.ws) + L.keys);
  ChunkRaw<T, VEC> nxt;
  int item = blockIdx.x;
  if (item < n_items) load_chunk_raw<T, VEC>(a.target, item / nc, a.V, item % nc, tid, nxt);
  for (; item < n_items; item += gridDim.x) {
    const int row = item / nc, chunk = item - row * nc;
    float vals[kPerThread];
    unpack_chunk<T, VEC>(nxt, vals);
    const int next = item + gridDim.x;
    if (next < n_items) load_chunk_raw<T, VEC>(a.target, next / nc, a.V, next % nc, tid, nxt);
    unsigned long long best = 0;
    if (chunk_has_tail(chunk, a.V)) {
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) {  // the key orders ties by index
        const int idx = chunk_entry<T, VEC>(chunk, tid, e);
        const unsigned long long key = idx < a.V ? argmax_key(vals[e], idx) : 0ull;
        best = key > best ? key : best;
      }
    } else {
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) {
        const unsigned long long key = argmax_key(vals[e], chunk_entry<T, VEC>(chunk, tid, e));
        best = key > best ? key : best;
      }
    }
    best = wave_max_u64(best);
    if ((tid & 63) == 0) red[tid >> 6] = best;
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < kThreads / 64; ++w) best = red[w] > best ? red[w] : best;
      keys[static_cast<size_t>(row) * nc + chunk] = best;
    }
    __syncthreads();  // red is written again by the next item
  }
}

__global__ __launch_bounds__(64) void decide_greedy(AcceptArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  int x0, T;
  if (!seq_ok(a, b, &x0, &T)) {
    if (lane == 0) {
      flag_error(a.err, SV_DERR_SEQLEN);
      skip_outputs(a, b);
    }
    return;
  }
  const int nc = n_chunks(a.V);
  const AcceptWs L = accept_ws_layout(a.B, a.total_T, a.V, a.mode);
  const unsigned long long* keys =
      reinterpret_cast<const unsigned long long*>(static_cast<const char*>(a.ws) + L.keys);
  const int d0 = x0 - b;
  // every draft id of the sequence must be in the vocabulary
  const int xd = lane < T - 1 ? a.draft_tokens[d0 + lane] : 0;
  if (__builtin_amdgcn_ballot_w64(xd < 0 || xd >= a.V) != 0) {
    if (lane == 0) {
      flag_error(a.err, SV_DERR_TOKEN);
      skip_outputs(a, b);
    }
    return;
  }
  int acc = 0, y = -1;
  for (int i = 0; i < T; ++i) {
    unsigned long long best = 0;
    for (int c = lane; c < nc; c += 64) {
      const unsigned long long k = keys[static_cast<size_t>(x0 + i) * nc + c];
      best = k > best ? k : best;
    }
    best = wave_max_u64(best);
    const int g = key_index(best);
    if (i == T - 1 || a.draft_tokens[d0 + i] != g) {
      acc = i;
      y = g;
      break;
    }
  }
  if (acc == T - 1 && a.bonus) {  // every draft accepted: the supplied bonus
    y = a.bonus[b];
    if (y < 0 || y >= a.V) {
      if (lane == 0) {
        flag_error(a.err, SV_DERR_TOKEN);
        skip_outputs(a, b);
      }
      return;
    }
  }
  if (lane == 0) write_outputs(a, b, x0, acc, y);
}

// ------------------------------------------------------------------ rejection
// Row r < total_T: target row r; otherwise draft row r - total_T.
// VEC: 16-byte row loads (see chunk_entry).
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void row_stats_partial(AcceptArgs a, int n_items) {
  const int tid = threadIdx.x;
  const int nc = n_chunks(a.V);
  __shared__ float redm[kThreads / 64];
  __shared__ double reds[kThreads / 64];
  __shared__ uint2 tab[kExpTab];
  exp_table_init_biased(tab);  // read after the first barrier below
  const AcceptWs L = accept_ws_layout(a.B, a.total_T, a.V, a.mode);
  double2* stats = reinterpret_cast<double2*>(static_cast<char*>(a.ws) + L.stats);
  auto load = [&](int it, ChunkRaw<T, VEC>& c) __attribute__((always_inline)) {
    const int r = it / nc;
    load_chunk_raw<T, VEC>(r < a.total_T ? a.target : a.draft,
                           r < a.total_T ? r : r - a.total_T, a.V, it - r * nc, tid, c);
  };
  ChunkRaw<T, VEC> nxt;
  int item = blockIdx.x;
  if (item < n_items) load(item, nxt);
  for (; item < n_items; item += gridDim.x) {
    const int r = item / nc, chunk = item - r * nc;
    float vals[kPerThread];
    unpack_chunk<T, VEC>(nxt, vals);
    if (item + static_cast<int>(gridDim.x) < n_items) load(item + gridDim.x, nxt);
    if (chunk_has_tail(chunk, a.V)) {
#pragma unroll
      for (int e = 0; e < kPerThread; ++e)
        if (chunk_entry<T, VEC>(chunk, tid, e) >= a.V) vals[e] = -INFINITY;
    }
    float m = vals[0];
#pragma unroll
    for (int e = 1; e < kPerThread; ++e) m = fmaxf(m, vals[e]);
    m = wave_max_f32(m);
    if ((tid & 63) == 0) redm[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(redm[0], redm[1]), fmaxf(redm[2], redm[3]));
    double sum = 0.0;
    if (m > -INFINITY) {
#pragma unroll
      for (int e = 0; e < kPerThread; ++e)
        sum += exp_nonpos_sum(static_cast<double>(vals[e]) - static_cast<double>(m), tab);
    }
    sum = wave_sum_f64(sum);
    if ((tid & 63) == 0) reds[tid >> 6] = sum;
    __syncthreads();
    if (tid == 0)
      stats[static_cast<size_t>(r) * nc + chunk] =
          make_double2(static_cast<double>(m), reds[0] + reds[1] + reds[2] + reds[3]);
  }
}

// Combine the chunk statistics of one row: M = max, Z = sum_c z_c e^(m_c - M).
__device__ double2 row_norm(const double2* stats, int row, int nc, int lane) {
  double M = -INFINITY;
  for (int c = lane; c < nc; c += 64) M = fmax(M, stats[static_cast<size_t>(row) * nc + c].x);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmax(M, __shfl_xor(M, o, 64));
  double Z = 0.0;
  for (int c = lane; c < nc; c += 64) {
    const double2 st = stats[static_cast<size_t>(row) * nc + c];
    if (st.y > 0.0) Z += st.y * exp(st.x - M);
  }
  Z = wave_sum_f64(Z);
  return make_double2(M, Z);
}

// Per sequence, 256 threads: every input of the decisions is fetched in
// parallel (draft tokens, uniforms and the logits at the drafts by wave 0,
// the row normalisers by the four waves in turn), then thread 0 runs the
// sequential accept test from LDS.
template <typename T>
__global__ __launch_bounds__(kThreads) void decide_reject(AcceptArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const AcceptWs L = accept_ws_layout(a.B, a.total_T, a.V, a.mode);
  int4* dec = reinterpret_cast<int4*>(static_cast<char*>(a.ws) + L.dec);
  int x0, tn;
  if (!seq_ok(a, b, &x0, &tn)) {
    if (tid == 0) {
      flag_error(a.err, SV_DERR_SEQLEN);
      dec[b] = make_int4(-1, -1, -1, -1);
      skip_outputs(a, b);
    }
    return;
  }
  const int d0 = x0 - b;
  const int nd = tn - 1;  // drafts
  __shared__ int xs[kMaxT];
  __shared__ float lt_s[kMaxT], lq_s[kMaxT], u_s[kMaxT];
  __shared__ double2 nt_s[kMaxT], nd_s[kMaxT];
  __shared__ int bad_s;
  if (tid == 0) bad_s = 0;
  __syncthreads();
  if (w == 0 && lane < nd) {
    const int x = a.draft_tokens[d0 + lane];
    const float u = a.u_accept[d0 + lane];
    const bool ok = x >= 0 && x < a.V;
    const int xc = ok ? x : 0;
    const float lt = ld<T>(a.target, static_cast<size_t>(x0 + lane) * a.V + xc);
    const float lq = a.draft ? ld<T>(a.draft, static_cast<size_t>(d0 + lane) * a.V + xc) : 0.f;
    xs[lane] = x;
    u_s[lane] = u;
    lt_s[lane] = lt;
    lq_s[lane] = lq;
    if (!ok) bad_s = 1;
  }
  const int nc = n_chunks(a.V);
  const double2* stats = reinterpret_cast<const double2*>(static_cast<const char*>(a.ws) + L.stats);
  // rows: target rows 0..nd (the last one for the bonus draw), then draft rows
  const int n_rows = tn + (a.draft ? nd : 0);
  for (int r = w; r < n_rows; r += kThreads / 64) {
    const int row = r < tn ? x0 + r : a.total_T + d0 + (r - tn);
    const double2 v = row_norm(stats, row, nc, lane);
    if (lane == 0) {
      if (r < tn) nt_s[r] = v;
      else nd_s[r - tn] = v;
    }
  }
  __syncthreads();
  if (tid != 0) return;
  if (bad_s) {
    flag_error(a.err, SV_DERR_TOKEN);
    dec[b] = make_int4(-1, -1, -1, -1);
    skip_outputs(a, b);
    return;
  }
  double4* fin = reinterpret_cast<double4*>(static_cast<char*>(a.ws) + L.fin);
  for (int i = 0; i < nd; ++i) {
    const double2 nt = nt_s[i];
    const double p = exp(static_cast<double>(lt_s[i]) - nt.x) / nt.y;
    double q = 1.0;  // point-mass draft distribution when no draft logits are given
    double2 ndv = make_double2(0.0, 0.0);
    if (a.draft) {
      ndv = nd_s[i];
      q = exp(static_cast<double>(lq_s[i]) - ndv.x) / ndv.y;
    }
    const double u = static_cast<double>(u_s[i]);
    if (!(u * q < p)) {
      // kind 1: residual max(0, p - q); kind 2: p without the draft token
      dec[b] = a.draft ? make_int4(i, 1, x0 + i, d0 + i) : make_int4(i, 2, x0 + i, xs[i]);
      fin[b] = make_double4(nt.x, nt.y, ndv.x, ndv.y);
      return;
    }
  }
  if (a.bonus) {  // every draft accepted: the supplied bonus, no draw
    const int y = a.bonus[b];
    if (y < 0 || y >= a.V) {
      flag_error(a.err, SV_DERR_TOKEN);
      skip_outputs(a, b);
    } else {
      write_outputs(a, b, x0, tn - 1, y);
    }
    dec[b] = make_int4(-1, -1, -1, -1);
    return;
  }
  const double2 nt = nt_s[tn - 1];
  dec[b] = make_int4(tn - 1, 0, x0 + tn - 1, -1);   // kind 0: target row
  fin[b] = make_double4(nt.x, nt.y, 0.0, 0.0);
}

// Logits of vocabulary entry y (clamped into the row, so the load is always
// in bounds and never waits on a branch) for the final draw of a sequence:
// the target row rt and, with DRAFT (kind 1), the draft row rd.
template <typename T, bool DRAFT>
__device__ __forceinline__ float2 draw_logits(const AcceptArgs& a, int rt, int rd, int y) {
  const int yc = min(y, a.V - 1);
  const float lt = ld<T>(a.target, static_cast<size_t>(rt) * a.V + yc);
  const float lq = DRAFT ? ld<T>(a.draft, static_cast<size_t>(rd) * a.V + yc) : 0.f;
  return make_float2(lt, lq);
}

// The logits of entries y0 + stride * e, e < kPerThread, every load issued
// before any is used.
template <typename T>
__device__ __forceinline__ void load_draw_logits(const AcceptArgs& a, int kind, int rt, int rd,
                                                 int y0, int stride, float2* lg) {
  if (kind == 1) {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) lg[e] = draw_logits<T, true>(a, rt, rd, y0 + stride * e);
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) lg[e] = draw_logits<T, false>(a, rt, rd, y0 + stride * e);
  }
}

// Weight of vocabulary entry y < V from its logits; rz holds the reciprocals
// of the two normalisers (f.y, f.w).  KIND 0: p; 1: max(p - q, 0); 2: p
// with the point-mass draft at rd taken out.
template <int KIND>
__device__ __forceinline__ double draw_weight_k(int rd, const double4& f, const double2& rz, int y,
                                                float2 lg, const double* tab) {
  const double p = exp_nonpos(static_cast<double>(lg.x) - f.x, tab) * rz.x;
  if constexpr (KIND == 0) {
    return p;
  } else if constexpr (KIND == 2) {
    return y == rd ? 0.0 : p;
  } else {
    const double q = exp_nonpos(static_cast<double>(lg.y) - f.z, tab) * rz.y;
    return fmax(p - q, 0.0);
  }
}

// The same for any kind and any y; entries past the vocabulary weigh 0.
__device__ __forceinline__ double draw_weight(const AcceptArgs& a, int kind, int rd,
                                              const double4& f, const double2& rz, int y,
                                              float2 lg, const double* tab) {
  if (y >= a.V) return 0.0;
  if (kind == 0) return draw_weight_k<0>(rd, f, rz, y, lg, tab);
  if (kind == 2) return draw_weight_k<2>(rd, f, rz, y, lg, tab);
  return draw_weight_k<1>(rd, f, rz, y, lg, tab);
}

// A thread's sum of the weights of its kPerThread entries of a chunk, in
// entry order (as draw_weight would give them: a masked entry adds 0).
template <int KIND, typename T, bool VEC>
__device__ __forceinline__ double residual_thread_sum(const AcceptArgs& a, int rd, const double4& f,
                                                      const double2& rz, int chunk, int tid,
                                                      const float2* lg, const double* tab) {
  double s = 0.0;
  if (chunk_has_tail(chunk, a.V)) {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int y = chunk_entry<T, VEC>(chunk, tid, e);
      if (y < a.V) s += draw_weight_k<KIND>(rd, f, rz, y, lg[e], tab);
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      s += draw_weight_k<KIND>(rd, f, rz, chunk_entry<T, VEC>(chunk, tid, e), lg[e], tab);
  }
  return s;
}

// VEC: as for row_stats_partial.
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void residual_partial(AcceptArgs a) {
  const int chunk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const AcceptWs L = accept_ws_layout(a.B, a.total_T, a.V, a.mode);
  const int4 d = reinterpret_cast<const int4*>(static_cast<const char*>(a.ws) + L.dec)[b];
  const double4 f = reinterpret_cast<const double4*>(static_cast<const char*>(a.ws) + L.fin)[b];
  if (d.x < 0) return;
  const double2 rz = make_double2(1.0 / f.y, 1.0 / f.w);
  float2 lg[kPerThread];
  {
    float pt[kPerThread], pq[kPerThread];
    load_chunk<T, VEC>(a.target, d.z, a.V, chunk, tid, pt);
    if (d.y == 1) {  // the residual p - q needs the draft row
      load_chunk<T, VEC>(a.draft, d.w, a.V, chunk, tid, pq);
    } else {
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) pq[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) lg[e] = make_float2(pt[e], pq[e]);
  }
  __shared__ double tab[kExpTab];
  __shared__ double red[kThreads / 64];
  exp_table_init(tab);
  __syncthreads();
  double s;
  if (d.y == 1) s = residual_thread_sum<1, T, VEC>(a, d.w, f, rz, chunk, tid, lg, tab);
  else if (d.y == 2) s = residual_thread_sum<2, T, VEC>(a, d.w, f, rz, chunk, tid, lg, tab);
  else s = residual_thread_sum<0, T, VEC>(a, d.w, f, rz, chunk, tid, lg, tab);
  s = wave_sum_f64(s);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    s = red[0];
    for (int w = 1; w < kThreads / 64; ++w) s += red[w];
    reinterpret_cast<double*>(static_cast<char*>(a.ws) + L.csum)
        [static_cast<size_t>(b) * gridDim.x + chunk] = s;
  }
}

// Inverse-CDF search inside one chunk: returns the first y of the chunk whose
// running sum (starting at `base`) exceeds t, or -1.  Block-wide, 256 threads;
// each thread owns kPerThread consecutive entries.
template <typename T>
__device__ int chunk_search(const AcceptArgs& a, int kind, int rt, int rd, const double4& f,
                            const double2& rz, const double* tab, int chunk, double base,
                            double t, int* last_pos) {
  const int tid = threadIdx.x;
  __shared__ double pre[kThreads];
  __shared__ int found;
  __shared__ int lastp;
  double w[kPerThread];
  double s = 0.0;
  const int y0 = chunk * kChunk + tid * kPerThread;
  float2 lg[kPerThread];
  load_draw_logits<T>(a, kind, rt, rd, y0, 1, lg);
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    w[e] = draw_weight(a, kind, rd, f, rz, y0 + e, lg[e], tab);
    s += w[e];
  }
  pre[tid] = s;
  if (tid == 0) {
    found = 0x7fffffff;
    lastp = -1;
  }
  __syncthreads();
  if (tid == 0) {   // exclusive prefix over the 256 thread sums, in order
    double run = base;
    for (int i = 0; i < kThreads; i += 8) {  // eight LDS reads in flight
      double v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = pre[i + j];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pre[i + j] = run;
        run += v[j];
      }
    }
  }
  __syncthreads();
  double run = pre[tid];
  int hit = -1, lastpos = -1;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    run += w[e];
    if (w[e] > 0.0) lastpos = y0 + e;
    if (hit < 0 && run > t && w[e] > 0.0) hit = y0 + e;
  }
  if (hit >= 0) atomicMin(&found, hit);
  if (lastpos >= 0) atomicMax(&lastp, lastpos);
  __syncthreads();
  *last_pos = lastp;
  return found == 0x7fffffff ? -1 : found;
}

// Thread 0 walks v[0..n) in index order, staged through LDS 256 entries at a
// time (every thread loads one), so the walk reads LDS rather than waiting on
// one global load per entry.  Without t: returns the sum.  With t: returns the
// first index c whose running sum before it plus v[c] exceeds t with v[c] > 0
// (-1 if none), and that running sum in *base.  The result is valid in
// thread 0; block-wide call.
__device__ double ordered_walk(const double* v, int n, double* stage, bool search, double t,
                               int* found, double* base) {
  const int tid = threadIdx.x;
  double run = 0.0;
  bool done = false;
  if (tid == 0) *found = -1;
  for (int c0 = 0; c0 < n; c0 += kThreads) {
    const int m = min(kThreads, n - c0);
    if (tid < m) stage[tid] = v[c0 + tid];
    __syncthreads();
    if (tid == 0 && !done) {
      for (int i = 0; i < m; ++i) {
        const double x = stage[i];
        if (search && run + x > t && x > 0.0) {
          *found = c0 + i;
          *base = run;
          done = true;
          break;
        }
        run += x;
      }
    }
    __syncthreads();
  }
  return run;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void final_draw(AcceptArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const AcceptWs L = accept_ws_layout(a.B, a.total_T, a.V, a.mode);
  // the decision record, the normalisers and (up to kThreads chunks) the
  // chunk sums are fetched together, in one round trip
  int4 d = reinterpret_cast<const int4*>(static_cast<const char*>(a.ws) + L.dec)[b];
  const float u_fin = a.u_final[b];
  const double4 f = reinterpret_cast<const double4*>(static_cast<const char*>(a.ws) + L.fin)[b];
  const int nc = n_chunks(a.V);
  double* csum = reinterpret_cast<double*>(static_cast<char*>(a.ws) + L.csum) + static_cast<size_t>(b) * nc;
  const bool one_stage = nc <= kThreads;
  const double cv = one_stage ? csum[min(tid, nc - 1)] : 0.0;
  if (d.x < 0) return;
  const double2 rz = make_double2(1.0 / f.y, 1.0 / f.w);
  __shared__ double tab[kExpTab];
  exp_table_init(tab);
  __shared__ double total_s;
  __shared__ double stage[kThreads];
  __shared__ int chunk_s;
  __shared__ double base_s;
  {
    double tot = 0.0;
    if (one_stage) {  // the staged sums, added in index order by thread 0
      stage[tid] = cv;
      __syncthreads();
      if (tid == 0)
        for (int c = 0; c < nc; ++c) tot += stage[c];
    } else {
      tot = ordered_walk(csum, nc, stage, false, 0.0, &chunk_s, &base_s);
    }
    if (tid == 0) total_s = tot;
  }
  __syncthreads();
  double total = total_s;
  bool staged = one_stage;  // stage[] still holds csum
  if (d.y != 0 && !(total > 0.0)) {
    staged = false;
    // p == q up to rounding: the residual is empty, draw from p instead.
    d.y = 0;
    __syncthreads();
    for (int c = 0; c < nc; ++c) {
      double s = 0.0;
      for (int e = 0; e < kPerThread; ++e) {
        const int y = c * kChunk + e * kThreads + tid;
        s += draw_weight(a, 0, d.w, f, rz, y, draw_logits<T, false>(a, d.z, d.w, y), tab);
      }
      s = wave_sum_f64(s);
      __shared__ double red[kThreads / 64];
      if ((tid & 63) == 0) red[tid >> 6] = s;
      __syncthreads();
      if (tid == 0) {
        double v = red[0];
        for (int w = 1; w < kThreads / 64; ++w) v += red[w];
        csum[c] = v;
      }
      __syncthreads();
    }
    {
      const double tot = ordered_walk(csum, nc, stage, false, 0.0, &chunk_s, &base_s);
      if (tid == 0) total_s = tot;
    }
    __syncthreads();
    total = total_s;
  }
  const double t = static_cast<double>(u_fin) * total;
  // chunk whose inclusive running sum first exceeds t
  if (staged) {
    if (tid == 0) {
      double run = 0.0, base = 0.0;
      int found = -1;
      for (int c = 0; c < nc; ++c) {
        const double x = stage[c];
        if (run + x > t && x > 0.0) {
          found = c;
          base = run;
          break;
        }
        run += x;
      }
      chunk_s = found;
      base_s = base;
    }
  } else {
    if (tid == 0) base_s = 0.0;
    ordered_walk(csum, nc, stage, true, t, &chunk_s, &base_s);
  }
  __syncthreads();
  int y = -1;
  int chunk = chunk_s;
  if (chunk < 0) {
    // rounding left no crossing: last index with positive weight
    for (int c = nc - 1; c >= 0 && y < 0; --c) {
      if (!(csum[c] > 0.0)) continue;
      int lastp;
      chunk_search<T>(a, d.y, d.z, d.w, f, rz, tab, c, 0.0, INFINITY, &lastp);
      y = lastp;
    }
  } else {
    int lastp;
    y = chunk_search<T>(a, d.y, d.z, d.w, f, rz, tab, chunk, base_s, t, &lastp);
    if (y < 0) y = lastp;
  }
  if (tid == 0) write_outputs(a, b, d.z - d.x, d.x, y);  // d.z - d.x = first row x0
}

// Blocks of the persistent row kernels: eight per compute unit.
int row_blocks() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  return 8 * cus;
}

template <typename T>
hipError_t launch_typed(const AcceptArgs& a, hipStream_t stream) {
  const int nc = n_chunks(a.V);
  using S = typename io<T>::storage;
  // 16-byte row loads: rows 16-byte aligned and V a multiple of the load's entries
  const bool vec = (static_cast<size_t>(a.V) * sizeof(S)) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(a.target) % 16 == 0 &&
                   (!a.draft || reinterpret_cast<uintptr_t>(a.draft) % 16 == 0);
  if (a.mode == SV_ACCEPT_GREEDY) {
    const int n_items = nc * a.total_T;
    const dim3 grid(std::min(n_items, row_blocks()));
    if (vec)
      hipLaunchKernelGGL((row_argmax_partial<T, true>), grid, dim3(kThreads), 0, stream, a, n_items);
    else
      hipLaunchKernelGGL((row_argmax_partial<T, false>), grid, dim3(kThreads), 0, stream, a, n_items);
    hipLaunchKernelGGL(decide_greedy, dim3(a.B), dim3(64), 0, stream, a);
  } else {
    const int rows = a.draft ? 2 * a.total_T - a.B : a.total_T;
    const int n_items = nc * rows;
    const dim3 grid(std::min(n_items, row_blocks()));
    if (vec)
      hipLaunchKernelGGL((row_stats_partial<T, true>), grid, dim3(kThreads), 0, stream, a, n_items);
    else
      hipLaunchKernelGGL((row_stats_partial<T, false>), grid, dim3(kThreads), 0, stream, a, n_items);
    hipLaunchKernelGGL((decide_reject<T>), dim3(a.B), dim3(kThreads), 0, stream, a);
    if (vec)
      hipLaunchKernelGGL((residual_partial<T, true>), dim3(nc, a.B), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((residual_partial<T, false>), dim3(nc, a.B), dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL((final_draw<T>), dim3(a.B), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_i32(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32, dim3((n + 255) / 256), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

size_t accept_workspace_bytes(int B, int total_T, int V, int mode) {
  return accept_ws_layout(B, total_T, V, mode).total;
}

hipError_t launch_accept(const AcceptArgs& a, sv_dtype dtype, hipStream_t stream) {
  return dtype == SV_BF16 ? launch_typed<bf16_t>(a, stream) : launch_typed<float>(a, stream);
}

}  // namespace sv
