// Top-k Markov drafting (DSparkSpeculator API page, _sample_sequential_topk).
//
// The candidates of every (request, step) row are the k largest of that
// step's base logits, chosen once for all steps. Each step then applies the
// Markov bias at those columns only, through k gathered rows of w2; every
// other entry of the row is -inf, and the row goes through the same sampler
// and cache write as the dense loop (so verification reads it unchanged).
//
// Three launches on the caller's stream:
//  1. topk_chunk_kernel, one work-group per 8192-column chunk of a row:
//     streams the chunk's base logits, writes -inf over the same cache
//     columns, and keeps the chunk's k largest entries.
//  2. topk_merge_kernel, one work-group per row: the k largest of the
//     chunks' survivors, in increasing column order.
//  3. topk_chain_kernel, one work-group per request: the K sequential steps,
//     each over the k candidates of its row.
//
// Selection order: the winner rule's total order (NaN above every number,
// -0 == +0, the lower column first among equal values), encoded in the
// 64-bit winner key ord(value) << 32 | ~column, so that "the k largest keys"
// is the whole rule and every key is distinct. Key 0 means "no entry".
#include "mds_device.h"
#include "mds_internal.h"

namespace mds {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kTopkChunk / kThreads;  // 32 base logits per thread

// -------------------------------------------------- block radix select --
// Block-wide (256 threads) search for the k largest of n distinct keys held
// in LDS, most significant byte first. On return, the selected keys are
// exactly those with (key & mask) >= prefix. Requires n >= k >= 1.
struct SelectState {
  unsigned long long prefix;
  int need, done;
};

__device__ void block_select_top(const unsigned long long* keys, int n, int k, unsigned* hist, unsigned* wtot,
                                 SelectState* st, unsigned long long& prefix, unsigned long long& mask) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  prefix = 0;
  mask = 0;
  int need = k;  // keys still to take among those whose masked bits equal prefix
  for (int shift = 56; shift >= 0; shift -= 8) {
    hist[t] = 0u;
    __syncthreads();
    for (int i = t; i < n; i += kThreads) {
      const unsigned long long key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // s = keys in digit bins >= t (suffix sum over the 256 bins)
    const unsigned h = hist[t];
    unsigned s = h;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned o = __shfl_down(s, off);
      if (lane + off < 64) s += o;
    }
    if (lane == 0) wtot[w] = s;
    __syncthreads();
    for (int u = w + 1; u < kThreads / 64; ++u) s += wtot[u];
    if (s >= (unsigned)need && s - h < (unsigned)need) {  // the bin holding the need-th largest key
      const int rest = need - (int)(s - h);
      st->prefix = prefix | ((unsigned long long)t << shift);
      st->need = rest;
      st->done = (int)h == rest;
    }
    __syncthreads();
    prefix = st->prefix;
    need = st->need;
    mask |= 0xFFull << shift;
    if (st->done) break;  // every key of the bin is taken
  }
}

// ------------------------------------------------------------ loads --
// Four base logits of a chunk; the vector form is non-temporal (each base
// row is read once here, and the chain reads only its candidates)
template <bool BF16>
__device__ __forceinline__ void load4(const void* row, int c, int V, bool vec, float v[4]) {
  if (vec && c + 3 < V) {
    if (BF16) {
      const u32x2 x = __builtin_nontemporal_load((const u32x2*)((const uint16_t*)row + c));
      v[0] = __uint_as_float(x.x << 16);
      v[1] = __uint_as_float(x.x & 0xFFFF0000u);
      v[2] = __uint_as_float(x.y << 16);
      v[3] = __uint_as_float(x.y & 0xFFFF0000u);
    } else {
      const f32x4 x = __builtin_nontemporal_load((const f32x4*)((const float*)row + c));
      v[0] = x.x;
      v[1] = x.y;
      v[2] = x.z;
      v[3] = x.w;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = 0.0f;
    if (c + i < V)
      v[i] = BF16 ? bf16_bits_to_f32(((const uint16_t*)row)[c + i]) : ((const float*)row)[c + i];
  }
}

template <bool BF16>
__device__ __forceinline__ void store_neg_inf4(void* row, int c, int V, bool vec) {
  if (vec && c + 3 < V) {
    if (BF16)
      *(u32x2*)((uint16_t*)row + c) = u32x2{0xFF80FF80u, 0xFF80FF80u};
    else
      *(f32x4*)((float*)row + c) = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (c + i < V) {
      if (BF16)
        ((uint16_t*)row)[c + i] = 0xFF80u;
      else
        ((float*)row)[c + i] = -INFINITY;
    }
  }
}

__device__ __forceinline__ int row_slot(const TopkArgs& a, int b, int k, uint32_t* status) {
  return draft_slot(a.idx_map, a.row_map, a.B, a.K, a.n_slots, a.n_rows, status, b, k);
}
__device__ __forceinline__ int slot_cache_row(const TopkArgs& a, int b, int s) {
  return !a.idx_map ? b : (a.row_map ? a.row_map[s] : s);
}

// Lane i's copy of lane i ^ m's word: DPP quad permutations for m = 1, 2,
// the LDS swizzle's bit mode (within 32 lanes) for m = 4..16, a permute for 32.
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int m) {
  if (m == 1) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  if (m == 2) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  if (m == 4) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (4 << 10));
  if (m == 8) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (8 << 10));
  if (m == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (16 << 10));
  return (uint32_t)__shfl_xor((int)v, m);
}

// The 64 keys of a wave in decreasing order over the lanes (lane i: the
// (i+1)-th largest), by a bitonic network of lane exchanges.
__device__ __forceinline__ unsigned long long wave_sort_desc(unsigned long long x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const unsigned long long y =
          ((unsigned long long)lane_xor((uint32_t)(x >> 32), stride) << 32) | lane_xor((uint32_t)x, stride);
      // runs of `size` lanes alternate direction, the last one decreasing;
      // the lower lane of a pair keeps the smaller key in an increasing run
      const bool keep_min = ((lane & stride) == 0) == ((lane & size) != 0);
      x = keep_min ? (y < x ? y : x) : (y > x ? y : x);
    }
  }
  return x;
}

// Keys of a decreasing list of 64 greater than x.
__device__ __forceinline__ int count_above(const unsigned long long* list, unsigned long long x) {
  int pos = list[63] > x ? 64 : 0;
#pragma unroll
  for (int step = 32; step >= 1; step >>= 1)
    if (pos < 64 && list[pos + step - 1] > x) pos += step;
  return pos;
}

// ------------------------------------------------- 1. chunk selection --
// Thread t holds columns c0 + 1024 j + 4 t + i (j < 8, i < 4). The k-th
// largest of the 256 per-thread maxima, t0, is a lower bound of the chunk's
// k-th largest key, and only the k threads whose maximum reaches t0 can hold
// keys >= t0: at most 32 k survivors go to LDS for the exact selection. A
// thread's maximum is t0 when exactly k - 1 maxima exceed it (the keys are
// distinct): each wave sorts its 64 maxima, and every thread counts the
// larger ones by binary search in the four sorted lists.
template <bool BBF16, bool CBF16>
__global__ __launch_bounds__(kThreads) void topk_chunk_kernel(TopkArgs a) {
  extern __shared__ unsigned long long s_keys[];  // [32 * topk]
  __shared__ unsigned long long s_tmax[kThreads];
  __shared__ unsigned s_hist[256];
  __shared__ unsigned s_wtot[4];
  __shared__ SelectState s_st;
  __shared__ unsigned long long s_t0;
  __shared__ int s_n, s_out;
  const int chunk = blockIdx.x % a.NC;
  const int row = blockIdx.x / a.NC;
  const int b = row / a.K, k = row - b * a.K;
  const int sl = row_slot(a, b, k, nullptr);
  if (sl < 0) return;  // inert row: no cache write, no candidates (uniform over the block)
  const int tid = threadIdx.x;
  const int V = a.V;
  const int c0 = chunk * kTopkChunk;
  const void* brow = BBF16 ? (const void*)((const uint16_t*)a.base + b * a.base_rs + k * a.base_ss)
                           : (const void*)((const float*)a.base + b * a.base_rs + k * a.base_ss);
  const long long crow_off = (long long)slot_cache_row(a, b, sl) * a.cache_rs + (long long)k * a.cache_ss;
  void* crow = CBF16 ? (void*)((uint16_t*)a.cache + crow_off) : (void*)((float*)a.cache + crow_off);
  if (tid == 0) {
    s_t0 = 0ull;
    s_n = 0;
    s_out = 0;
  }
  float v[kPerThread];
#pragma unroll
  for (int j = 0; j < kPerThread / 4; ++j) load4<BBF16>(brow, c0 + 1024 * j + 4 * tid, V, a.vec_base != 0, v + 4 * j);
#pragma unroll
  for (int j = 0; j < kPerThread / 4; ++j) store_neg_inf4<CBF16>(crow, c0 + 1024 * j + 4 * tid, V, a.vec_cache != 0);

  unsigned long long tmax = 0ull;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int c = c0 + 1024 * (j >> 2) + 4 * tid + (j & 3);
    const unsigned long long key = c < V ? win_key(v[j], (uint32_t)c) : 0ull;
    tmax = key > tmax ? key : tmax;
  }
  s_tmax[tid] = wave_sort_desc(tmax);  // wave w's maxima, decreasing, at s_tmax[64 w ..]
  __syncthreads();
  int above = 0;  // thread maxima larger than this thread's
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) above += count_above(s_tmax + 64 * w, tmax);
  if (tmax != 0ull && above == a.topk - 1) s_t0 = tmax;  // distinct nonzero keys: one writer at most
  __syncthreads();
  const unsigned long long t0 = s_t0 ? s_t0 : 1ull;
  const int cap = kPerThread * a.topk;
  if (tmax >= t0) {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int c = c0 + 1024 * (j >> 2) + 4 * tid + (j & 3);
      const unsigned long long key = c < V ? win_key(v[j], (uint32_t)c) : 0ull;
      if (key >= t0) {
        const int i = atomicAdd(&s_n, 1);
        if (i < cap) s_keys[i] = key;
      }
    }
  }
  __syncthreads();
  const int n = min(s_n, cap);
  unsigned long long* out = a.ckeys + ((size_t)row * a.NC + chunk) * a.topk;
  if (n <= a.topk) {  // every survivor is kept; the rest of the slots say "none"
    for (int i = tid; i < a.topk; i += kThreads) out[i] = i < n ? s_keys[i] : 0ull;
    return;
  }
  unsigned long long prefix, mask;
  block_select_top(s_keys, n, a.topk, s_hist, s_wtot, &s_st, prefix, mask);
  for (int i = tid; i < n; i += kThreads) {
    const unsigned long long key = s_keys[i];
    if ((key & mask) >= prefix) {
      const int i2 = atomicAdd(&s_out, 1);
      if (i2 < a.topk) out[i2] = key;
    }
  }
}

// ------------------------------------------------------- 2. row merge --
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(TopkArgs a) {
  __shared__ unsigned long long s_keys[kTopkMergeKeys];
  __shared__ unsigned long long s_sel[kTopkMax];
  __shared__ unsigned s_hist[256];
  __shared__ unsigned s_wtot[4];
  __shared__ SelectState s_st;
  __shared__ int s_n;
  const int row = blockIdx.x;
  const int b = row / a.K, k = row - b * a.K;
  if (row_slot(a, b, k, nullptr) < 0) return;
  const int tid = threadIdx.x;
  const int n = a.NC * a.topk;
  const unsigned long long* in = a.ckeys + (size_t)row * n;
  for (int i = tid; i < n; i += kThreads) s_keys[i] = in[i];
  if (tid == 0) s_n = 0;
  __syncthreads();
  unsigned long long prefix = 0ull, mask = 0ull;  // n == topk: every key is taken
  if (n > a.topk) block_select_top(s_keys, n, a.topk, s_hist, s_wtot, &s_st, prefix, mask);
  for (int i = tid; i < n; i += kThreads) {
    const unsigned long long key = s_keys[i];
    if (key != 0ull && (key & mask) >= prefix) {
      const int i2 = atomicAdd(&s_n, 1);
      if (i2 < a.topk) s_sel[i2] = key;
    }
  }
  __syncthreads();
  // increasing column order: a candidate's rank is the number of lower
  // columns (m == topk, as a row has V >= topk entries; a shortfall would
  // leave -1, "no candidate")
  const int m = min(s_n, a.topk);
  if (tid < m) {
    const uint32_t c = win_col(s_sel[tid]);
    int rank = 0;
    for (int u = 0; u < m; ++u) rank += win_col(s_sel[u]) < c;
    a.cand[(size_t)row * a.topk + rank] = (int32_t)c;
  } else if (tid < a.topk) {
    a.cand[(size_t)row * a.topk + tid] = -1;
  }
}

// ------------------------------------------------------ 3. the chain --
// Winner of two (score, column) entries under the winner rule; col < 0 is
// "no entry".
template <typename S>
__device__ __forceinline__ void better(S& s, int& c, S s2, int c2) {
  bool take;
  if (c2 < 0)
    take = false;
  else if (c < 0)
    take = true;
  else if (s2 != s2 || s != s)
    take = (s2 != s2) && (s == s || c2 < c);
  else
    take = s2 > s || (s2 == s && c2 < c);
  s = take ? s2 : s;
  c = take ? c2 : c;
}

// The chain's winner over a wave by the DPP row operations of the shared
// wave reductions (the winner order is associative and commutative).
template <typename S>
__device__ __forceinline__ void row_better(S& s, int& c) {
  better(s, c, dpp_val<kDppXor1>(s), dpp_val<kDppXor1>(c));
  better(s, c, dpp_val<kDppXor2>(s), dpp_val<kDppXor2>(c));
  better(s, c, dpp_val<kDppRor4>(s), dpp_val<kDppRor4>(c));
  better(s, c, dpp_val<kDppRor8>(s), dpp_val<kDppRor8>(c));
}
template <typename S>
__device__ __forceinline__ void wave_better_dpp(S& s, int& c) {
  row_better(s, c);
  S s0 = lane_val(s, 0);
  int c0 = lane_val(c, 0);
#pragma unroll
  for (int l = 16; l < 64; l += 16) better(s0, c0, lane_val(s, l), lane_val(c, l));
  s = s0;
  c = c0;
}
__device__ __forceinline__ float dot8(u32x4 w, const float* e) {
  float acc = 0.0f;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const uint32_t x = h == 0 ? w.x : (h == 1 ? w.y : (h == 2 ? w.z : w.w));
    acc = __builtin_fmaf(__uint_as_float(x << 16), e[2 * h], acc);
    acc = __builtin_fmaf(__uint_as_float(x & 0xFFFF0000u), e[2 * h + 1], acc);
  }
  return acc;
}

constexpr int kChainBatch = 8;  // 16-byte w2 chunks a thread loads per step
constexpr int kMaxSteps = 32;   // K <= 32 (checked at the boundary)

template <bool BBF16, bool CBF16, bool F64>
__global__ __launch_bounds__(kThreads) void topk_chain_kernel(TopkArgs a, int tpc) {
  using Score = typename std::conditional<F64, double, float>::type;
  __shared__ float s_e[512];
  // per-wave results: a wave writes the next step's only after the next
  // step's embedding barrier, which every wave reaches after reading these
  __shared__ Score s_ws[4];
  __shared__ int s_wc[4];
  __shared__ float s_wm[4], s_wsum[4];
  __shared__ int s_wnan[4];
  __shared__ int s_sl[kMaxSteps];
  __shared__ float s_T[kMaxSteps];
  __shared__ unsigned long long s_seed[kMaxSteps], s_pos[kMaxSteps];
  const int b = blockIdx.x, K = a.K;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = a.r, nch = r >> 3;
  const int ci = tid / tpc, part = tid - ci * tpc;
  auto cand_of = [&](int k) { return ci < a.topk ? a.cand[((size_t)b * K + k) * a.topk + ci] : -1; };

  // A step's loads: the w2 rows of this thread's candidate and its base
  // logit, the embedding row of the previous token (a row past V reads row 0
  // and is flagged when the step is live), and the next step's candidate.
  // They are issued as soon as the previous token is known, so they fly
  // while the previous step finishes its log-sum-exp and this step draws
  // its noise.
  int cc = -1, cc_next = cand_of(0);
  u32x4 wch[kChainBatch];
  u32x4 ew = {0u, 0u, 0u, 0u};
  float bv = 0.0f;
  bool tk_bad = false;
  auto issue = [&](int k, long long tk) {
    cc = cc_next;
    if (k + 1 < K) cc_next = cand_of(k + 1);
    const bool has = cc >= 0 && cc < a.V;
    const int col = has ? cc : 0;
    const uint16_t* w2row = a.w2 + (size_t)col * r;
#pragma unroll
    for (int q = 0; q < kChainBatch; ++q) {
      const int j = part + q * tpc;
      if (has && j < nch) wch[q] = *(const u32x4*)(w2row + 8 * j);
    }
    bv = 0.0f;
    if (has && part == 0) {
      bv = BBF16 ? bf16_bits_to_f32(((const uint16_t*)a.base)[b * a.base_rs + k * a.base_ss + col])
                 : ((const float*)a.base)[b * a.base_rs + k * a.base_ss + col];
    }
    tk_bad = tk < 0 || tk >= a.V;
    if (tk_bad) tk = 0;
    if (tid < nch) ew = *(const u32x4*)(a.w1 + (size_t)tk * r + 8 * tid);  // r <= 512: one chunk per thread
  };
  // step 0's loads go out with the per-step state: slots, temperatures,
  // seeds and sample positions, one thread per step
  issue(0, (long long)a.anchor[b]);
  if (tid < K) {
    const int sl = row_slot(a, b, tid, a.status);
    s_sl[tid] = sl;
    const int ss = sl < 0 ? 0 : sl;
    s_T[tid] = a.temp[ss];
    s_seed[tid] = (unsigned long long)a.seeds[ss];
    s_pos[tid] = (unsigned long long)(a.sample_pos[b * K + tid] - 1);
  }
  __syncthreads();
  for (int k = 0; k < K; ++k) {
    const int row = b * K + k;
    const int sl = s_sl[k];
    if (sl < 0) {  // inert step: no sample, no cache write; the next step has no previous token
      if (tid == 0) {
        a.tokens[row] = -1;
        if (a.lse) a.lse[row] = NAN;
      }
      if (k + 1 < K) issue(k + 1, -1);
      continue;
    }
    if (tk_bad && tid == 0) set_status(a.status, kStatusBadAnchor);
    const float T = s_T[k];
    const bool samp = T > 0.0f;
    const float invT = samp ? 1.0f / T : 1.0f;
    const bool has = cc >= 0 && cc < a.V;
    const bool mine = has && part == 0;  // this thread scores the candidate
    const int col = has ? cc : 0;
    // the noise at the candidate, while the loads are in flight
    Score g = (Score)0;
    if (mine && samp) {
      const unsigned long long seed = s_seed[k], pos = s_pos[k];
      const Philox4 w = philox4x32_10((uint32_t)col >> 2, (uint32_t)pos, (uint32_t)(pos >> 32), kSaltDraft,
                                      (uint32_t)seed, (uint32_t)(seed >> 32));
      const uint32_t sel = col & 3;
      const uint32_t wd = sel == 0 ? w.x0 : (sel == 1 ? w.x1 : (sel == 2 ? w.x2 : w.x3));
      if constexpr (F64)
        g = gumbel64_from_word(wd);
      else
        g = gumbel_from_word(wd);
    }
    if (tid < nch) {
      const uint32_t xs[4] = {ew.x, ew.y, ew.z, ew.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        s_e[8 * tid + 2 * h] = __uint_as_float(xs[h] << 16);
        s_e[8 * tid + 2 * h + 1] = __uint_as_float(xs[h] & 0xFFFF0000u);
      }
    }
    __syncthreads();  // the embedding is in s_e
    const uint16_t* w2row = a.w2 + (size_t)col * r;
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < kChainBatch; ++q) {
      const int j = part + q * tpc;
      if (has && j < nch) acc += dot8(wch[q], s_e + 8 * j);
    }
    for (int j = part + kChainBatch * tpc; has && j < nch; j += tpc)
      acc += dot8(*(const u32x4*)(w2row + 8 * j), s_e + 8 * j);
    for (int off = tpc >> 1; off >= 1; off >>= 1) acc += __uint_as_float(lane_xor(__float_as_uint(acc), off));

    // biased logit, cache write, score and log-sum-exp terms at the candidate
    Score s = (Score)0;
    int c = -1;
    float x = -INFINITY;
    int xnan = 0;
    if (mine) {
      const float z = bv + acc;
      const long long off = (long long)slot_cache_row(a, b, sl) * a.cache_rs + (long long)k * a.cache_ss + col;
      float cv = z;
      if (CBF16) {
        const uint32_t hb = f32_to_bf16_bits(z);
        ((uint16_t*)a.cache)[off] = (uint16_t)hb;
        cv = bf16_bits_to_f32(hb);
      } else {
        ((float*)a.cache)[off] = z;
      }
      c = col;
      if (samp) {
        if constexpr (F64)
          s = (Score)((double)z / (double)T + g);
        else
          s = (Score)(div_t(z, T, invT) + g);
        x = div_t(cv, T, invT);
        xnan = x != x;
        if (xnan) x = -INFINITY;
      } else {
        s = (Score)z;
      }
    }
    // winner, and max / NaN flag of cache / T
    wave_better_dpp(s, c);
    float m = wave_max_dpp(x);
    int anynan = __any(xnan) ? 1 : 0;
    if (lane == 0) {
      s_ws[wv] = s;
      s_wc[wv] = c;
      s_wm[wv] = m;
      s_wnan[wv] = anynan;
    }
    __syncthreads();  // every thread merges the four waves' results
    Score sw = s_ws[0];
    int cw = s_wc[0];
    m = s_wm[0];
    anynan = s_wnan[0];
    for (int u = 1; u < 4; ++u) {
      better(sw, cw, s_ws[u], s_wc[u]);
      m = fmaxf(m, s_wm[u]);
      anynan |= s_wnan[u];
    }
    // an all -inf row: every column ties at -inf and the first column wins
    const int token = (cw < 0 || (sw == -(Score)INFINITY)) ? 0 : cw;
    // the next step's loads (also for an inert step, which keeps the
    // candidate prefetch in order), before this step's log-sum-exp
    if (k + 1 < K) issue(k + 1, token);
    float lse = NAN;
    if (samp && !anynan && (m == INFINITY || m == -INFINITY)) {
      lse = m;
    } else if (samp && !anynan) {
      float e = (mine && x > -INFINITY) ? __expf(x - m) : 0.0f;
      e = wave_sum_dpp(e);
      if (lane == 0) s_wsum[wv] = e;
      __syncthreads();
      lse = m + __logf(s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3]);
    }
    if (tid == 0) {
      a.tokens[row] = token;
      if (a.lse) a.lse[row] = lse;
    }
  }
}

template <bool BBF16, bool CBF16>
hipError_t launch_select_t(const TopkArgs& a, hipStream_t st) {
  const size_t lds = topk_chunk_lds(a.topk);
  if (lds + 4096 > 65536) {  // with the kernel's static LDS
    const hipError_t e = hipFuncSetAttribute((const void*)topk_chunk_kernel<BBF16, CBF16>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((topk_chunk_kernel<BBF16, CBF16>), dim3(a.NC * a.B * a.K), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <bool BBF16, bool CBF16, bool F64>
hipError_t launch_chain_t(const TopkArgs& a, hipStream_t st) {
  // threads per candidate: a power of two, at most a wave and at most the
  // rank's 16-byte chunks
  int kp = 1;
  while (kp < a.topk) kp <<= 1;
  int tpc = kThreads / kp;
  if (tpc > 64) tpc = 64;
  while (tpc > 1 && tpc > (a.r >> 3)) tpc >>= 1;
  hipLaunchKernelGGL((topk_chain_kernel<BBF16, CBF16, F64>), dim3(a.B), dim3(kThreads), 0, st, a, tpc);
  return hipGetLastError();
}

template <bool F64>
hipError_t launch_chain_f(const TopkArgs& a, hipStream_t st) {
  if (a.base_bf16)
    return a.cache_bf16 ? launch_chain_t<true, true, F64>(a, st) : launch_chain_t<true, false, F64>(a, st);
  return a.cache_bf16 ? launch_chain_t<false, true, F64>(a, st) : launch_chain_t<false, false, F64>(a, st);
}

}  // namespace

size_t topk_chunk_lds(int topk) { return (size_t)kPerThread * topk * sizeof(unsigned long long); }

hipError_t launch_topk_select(const TopkArgs& a, hipStream_t st) {
  if (a.base_bf16) return a.cache_bf16 ? launch_select_t<true, true>(a, st) : launch_select_t<true, false>(a, st);
  return a.cache_bf16 ? launch_select_t<false, true>(a, st) : launch_select_t<false, false>(a, st);
}

hipError_t launch_topk_merge(const TopkArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(topk_merge_kernel, dim3(a.B * a.K), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_topk_chain(const TopkArgs& a, hipStream_t st) {
  return a.fp64 ? launch_chain_f<true>(a, st) : launch_chain_f<false>(a, st);
}

}  // namespace mds
