// Rejection-sampling verification kernels (gfx950).
//
// PR #65007 (Part 2) describes the stock rejection sampler as per-block
// kernels over 8192-column statistics blocks whose partials per-request
// kernels combine, plus residual-mass and resample kernels. Here, without
// top-p, three launches do the whole pass:
//   stats_wave_kernel  one wave per (row, kStatsChunk-column block) streams
//                    the target rows (and the draft cache rows when the draft
//                    loop gave no log-normalisers): (max, sum exp) of
//                    logit / T for sampled requests, the winner key of the
//                    raw logits for greedy ones (PR #63554, Notes: greedy
//                    verification compares with the target argmax and never
//                    reads the draft cache), one plain partial store per
//                    block;
//   combine_kernel   one wave per request combines the partials and runs the
//                    K accept tests p(x) >= u * q(x);
//   residual_kernel  one work-group per (request, 2048-column block) draws
//                    over its block with Gumbel-max from the normalised
//                    residual max(0, p - q) of the first rejected row, or
//                    from p for the bonus token; the last one of a request
//                    writes the output tokens.
// With top-p the same statistics pass and combine (without the accept tests)
// come first; top_p_kernel (topp.hip) then finds the kept sets from the row
// maxima, decide_kernel runs the accept tests, then the residual pass.
//
// Cross-work-group hand-off inside a launch (the residual pass): winner keys
// are published with device-scope atomics whose completion the publishing
// thread waits for before it bumps the request's arrival counter; the last
// arrival reads them back with read-modify-writes. Every counter returns to
// zero before the call ends.
#include "mds_device.h"
#include "mds_internal.h"

#include <type_traits>

namespace mds {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxK = 32;

__device__ __forceinline__ float load_f32_or_bf16(const void* p, long long off, int bf16) {
  return bf16 ? bf16_bits_to_f32(((const uint16_t*)p)[off]) : ((const float*)p)[off];
}

// Wait until every vector memory operation of this thread has completed
// (returning atomics included); the "memory" clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ unsigned long long pack_ms(float m, float s) {
  return ((unsigned long long)__float_as_uint(s) << 32) | __float_as_uint(m);
}
__device__ __forceinline__ float unpack_m(unsigned long long p) { return __uint_as_float((uint32_t)p); }
__device__ __forceinline__ float unpack_s(unsigned long long p) { return __uint_as_float((uint32_t)(p >> 32)); }

__device__ __forceinline__ unsigned long long block_max_key(unsigned long long key) {
  __shared__ unsigned long long sk[4];
  key = wave_max_key(key);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sk[wave] = key;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) key = sk[w] > key ? sk[w] : key;
  }
  return key;
}

__device__ __forceinline__ bool kept(const TopP& tp, float t, int v) {
  if (!tp.on) return true;
  const uint32_t o = ord_f32(t);
  return o > tp.tau || (o == tp.tau && v <= tp.cut);
}

// Per-request statistics staged in LDS for the decision.
struct ReqLds {
  float m[kMaxK + 1], lz[kMaxK + 1], lq[kMaxK], qm[kMaxK];
  unsigned long long key[kMaxK + 1], qkey[kMaxK];
  int acc[kMaxK];
  int x[kMaxK];             // draft tokens (sampled requests: clamped into [0, V))
  float tx[kMaxK], cx[kMaxK];  // target and cache logits at the draft tokens
  unsigned long long seed;     // the request's seed and anchor position, loaded ahead by the caller
  long long pos0;
};

// Draft token k of request b (state slot s) and the target / cache logits at
// it. -1 is a placeholder (no draft from here on; the logits are not read);
// any other token outside [0, V) is replaced by 0 and flagged in the status
// word.
__device__ __forceinline__ void draft_point(const VerifyArgs& a, int b, int s, int k, int& x, float& tx, float& cx) {
  x = a.draft[b * a.K + k];
  tx = cx = 0.0f;
  if (x == -1) return;
  if (x < 0 || x >= a.V) {
    set_status(a.status, kStatusBadDraft);
    x = 0;
  }
  tx = a.target[(long long)(b * (a.K + 1) + k) * a.target_rs + x];
  cx = load_f32_or_bf16(a.cache, (long long)verify_cache_row(a, b, s) * a.cache_rs + (long long)k * a.cache_ss + x,
                        a.cache_bf16);
}

// A padding request: every output token -1, none accepted, no residual draw.
__device__ void finish_padding(const VerifyArgs& a, int b) {
  const int lane = threadIdx.x & 63;
  if (lane <= a.K) a.out_tokens[(size_t)b * (a.K + 1) + lane] = -1;
  if (lane == 0) {
    a.num_accepted[b] = 0;
    ReqState r{};
    r.mode = 2;
    a.req[b] = r;
  }
}

constexpr int kStage = 1024;  // partials a combining wave stages in LDS at a time

// Orders the LDS accesses of one wave around it (a wave's LDS operations
// execute in issue order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave combines nrows consecutive rows of NC packed partials, partial
// (row, chunk) at p[chunk * cstride + row]: the max of the words (keys) or
// their (max, sum exp) merge. Partials are plain loads (stored by the
// statistics launch before), staged in LDS a page at a time (all loads of a
// page in flight together); each row of the page is then merged by a group of lanes (a
// power of two) and the group's results by shuffles. Results go to
// om / os / okey [row].
__device__ void wave_combine(const unsigned long long* p, size_t cstride, int nrows, int NC, bool keys,
                             unsigned long long* stage, float* om, float* os, unsigned long long* okey) {
  const int lane = threadIdx.x & 63;
  const int cpp = NC < kStage ? NC : kStage;  // chunks per page
  const int rpp = kStage / cpp;               // rows per page, >= 1
  for (int r0 = 0; r0 < nrows; r0 += rpp) {
    const int nr = nrows - r0 < rpp ? nrows - r0 : rpp;
    // lanes per row: the largest power of two with nr * lpr <= 64 (1 if nr > 32)
    int lpr = 64;
    while (lpr > 1 && lpr * nr > 64) lpr >>= 1;
    const int grp = lane / lpr, sub = lane - grp * lpr;  // lane's row of the page, and its place in the group
    float m = -INFINITY, s = 0.0f;
    unsigned long long key = 0ull;
    for (int c0 = 0; c0 < NC; c0 += cpp) {
      const int nc = NC - c0 < cpp ? NC - c0 : cpp;
      const int n = nr * nc;
      for (int t0 = 0; t0 < n; t0 += 64 * 16) {
        unsigned long long w[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (t0 + u * 64 < n) {  // wave-uniform: only batches holding some partial
            int t = t0 + u * 64 + lane;
            t = t < n ? t : n - 1;
            const int rr = t / nc, cc = t - rr * nc;
            const unsigned long long* q = p + (size_t)(c0 + cc) * cstride + (r0 + rr);
            w[u] = *q;
          }
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int t = t0 + u * 64 + lane;
          if (t0 + u * 64 < n && t < n) stage[t] = w[u];
        }
      }
      wave_lds_sync();
      if (grp < nr) {  // nr <= 33 rows, so every row has a group of its own
        for (int cc = sub; cc < nc; cc += lpr) {
          const unsigned long long x = stage[grp * nc + cc];
          if (keys)
            key = x > key ? x : key;
          else
            lse_merge(m, s, unpack_m(x), unpack_s(x));
        }
      }
      wave_lds_sync();
    }
    // merge the lpr lanes of each group (xor within the aligned group)
    for (int off = 1; off < lpr; off <<= 1) {
      const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
      const unsigned long long k2 = __shfl_xor(key, off);
      lse_merge(m, s, m2, s2);
      key = k2 > key ? k2 : key;
    }
    if (sub == 0 && grp < nr) {
      om[r0 + grp] = m;
      os[r0 + grp] = s;
      okey[r0 + grp] = key;
    }
  }
  wave_lds_sync();
}

// The K accept tests of request b (independent; the first failure ends the
// run), then ReqState for the residual draw. Greedy requests are finished
// here: the final token is the argmax of row n_acc. Run by one wave with L
// filled.
__device__ void decide(const VerifyArgs& a, int b, int sl, ReqLds& L) {
  const int K = a.K, V = a.V;
  const int lane = threadIdx.x & 63;
  const float T = a.temp[sl];
  const bool greedy = !(T > 0.0f);
  const float invT = greedy ? 1.0f : 1.0f / T;
  // the drafts end at the first -1 placeholder
  int mb = K;
  for (int k = K - 1; k >= 0; --k)
    if (L.x[k] == -1) mb = k;
  if (lane < mb) {
    const int k = lane;
    const int x = L.x[k];
    bool ok;
    if (greedy) {
      ok = x == (int32_t)win_col(L.key[k]);
    } else {
      const int row = b * (K + 1) + k;
      const float tx = L.tx[k];
      float logp = -INFINITY;
      if (!a.topp || kept(a.topp[row], tx, x)) logp = div_t(tx, T, invT) - L.m[k] - L.lz[k];
      float p = expf(logp);
      float q = expf(div_t(L.cx[k], T, invT) - L.lq[k]);
      // a row with no finite logit (max -inf) has the one-hot at column 0 as
      // its distribution, the column the winner rule gives it
      if (L.m[k] == -INFINITY) p = x == 0 ? 1.0f : 0.0f;
      if (L.lq[k] == -INFINITY) q = x == 0 ? 1.0f : 0.0f;
      const unsigned long long sd = L.seed;
      const unsigned long long pk = (unsigned long long)(L.pos0 + k);
      const Philox4 w = philox4x32_10(0u, (uint32_t)pk, (uint32_t)(pk >> 32), kSaltAccept, (uint32_t)sd,
                                      (uint32_t)(sd >> 32));
      const float u = uniform24(w.x0);
      ok = p >= u * q;  // a NaN q rejects
    }
    L.acc[k] = ok;
  }
  wave_lds_sync();
  int n = 0;
  while (n < mb && L.acc[n]) ++n;
  if (greedy && lane <= K) {
    const int i = lane;
    int v = -1;
    if (i < n) {
      v = a.draft[b * K + i];
      if (v < 0 || v >= V) v = 0;
    } else if (i == n) {
      v = (int)win_col(L.key[n]);
    }
    a.out_tokens[(size_t)b * (K + 1) + i] = v;
  }
  if (lane == 0) {
    ReqState r;
    r.n_acc = n;
    r.mode = greedy ? 2 : (n < mb ? ((L.lq[n] != L.lq[n]) ? 3 : 1) : 0);
    r.M = L.m[n];
    r.LZ = L.lz[n];
    r.LQ = r.mode == 1 ? L.lq[n] : 0.0f;
    r.pad = 0;
    r.tp = a.topp ? a.topp[b * (K + 1) + n] : TopP{0u, 0, 0.0f, 0};
    if (r.tp.on) r.LZ = r.tp.log_z;
    a.req[b] = r;
    a.rkey[verify_key_index(b)] = 0ull;
    if (greedy) a.num_accepted[b] = n;
  }
}

// Combine every partial of request b, write the row statistics and, without
// top-p, decide. Run by one wave after the whole statistics pass; block 0 of
// each target row has recorded the target and cache logits at the draft
// tokens.
__device__ void combine_request(const VerifyArgs& a, int b, int sl, ReqLds& L, unsigned long long* stage) {
  const int K = a.K, NC = a.NC;
  const int lane = threadIdx.x & 63;
  if (sl < 0) {  // padding request: nothing was published
    if (a.decide) finish_padding(a, b);
    return;
  }
  // every load goes out together: temperature, draft tokens, draft
  // normalisers, seed and position, the logits at the draft tokens (recorded
  // by block 0 of each target row) and the partials
  const float T = a.temp[sl];
  int x0 = 0;
  float lq0 = 0.0f;
  if (lane < K) {
    x0 = a.draft[b * K + lane];
    if (a.draft_lse) lq0 = a.draft_lse[b * K + lane];
  }
  if (a.decide && lane == 0) {  // only the decision reads them (the top-p debug entry passes neither)
    L.seed = (unsigned long long)a.seeds[sl];
    L.pos0 = a.anchor_pos[b];
  }
  const bool greedy = !(T > 0.0f);
  if (lane < K) {
    if (greedy) {
      L.x[lane] = x0;
    } else {
      const unsigned long long w = a.tq[b * K + lane];
      L.x[lane] = (x0 == -1) ? -1 : ((x0 < 0 || x0 >= a.V) ? 0 : x0);
      L.tx[lane] = unpack_m(w);
      L.cx[lane] = unpack_s(w);
    }
  }
  wave_combine(a.tpart + (size_t)b * (K + 1), (size_t)a.B * (K + 1), K + 1, NC, greedy, stage, L.m, L.lz, L.key);
  if (lane <= K) {
    const float s = L.lz[lane];
    const float lz = (s != s) ? NAN : __logf(s);
    L.lz[lane] = lz;
    a.rowstat[b * (K + 1) + lane] = RowStat{L.m[lane], lz, L.key[lane]};
  }
  if (a.qpart && !greedy) {
    wave_combine(a.qpart + (size_t)b * K, (size_t)a.B * K, K, NC, false, stage, L.qm, L.lq, L.qkey);
    if (lane < K) {
      const float s = L.lq[lane];
      const float lq = (s != s) ? NAN : L.qm[lane] + __logf(s);
      L.lq[lane] = lq;
      a.qlse[b * K + lane] = lq;
    }
  } else if (lane < K) {
    const float lq = greedy ? 0.0f : lq0;
    L.lq[lane] = lq;
    a.qlse[b * K + lane] = lq;
  }
  wave_lds_sync();
  if (a.decide) decide(a, b, sl, L);
}

// ---- statistics: one wave per (row, block) ----
constexpr int kWavePer = kStatsChunk / 64;  // values per lane: columns c0 + 256 i + 4 lane + e

// The lane's kWavePer values of one block; when the whole block exists and
// vector access is allowed (a wave-uniform test) every load is issued before
// any value is used.
template <bool BF16>
__device__ __forceinline__ void load_wave_block(const void* rowp, int V, int c0, bool vec, float (&v)[kWavePer]) {
  // a buffer over the row: 32-bit offsets from one base, and loads past the
  // row's V elements return 0 (the pad of a partial block) without a test
  constexpr int kEs = BF16 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)rowp, (short)0, V * kEs, 0x00020000);  // raw, byte-addressed
  const int tc = c0 + (int)(threadIdx.x & 63) * 4;
  if (vec && c0 + kStatsChunk <= V) {
#pragma unroll
    for (int i = 0; i < kWavePer / 4; ++i) {
      if (BF16) {
        const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (tc + i * 256) * kEs, 0, 2));
        v[4 * i + 0] = bf16_bits_to_f32(w.x & 0xFFFFu);
        v[4 * i + 1] = bf16_bits_to_f32(w.x >> 16);
        v[4 * i + 2] = bf16_bits_to_f32(w.y & 0xFFFFu);
        v[4 * i + 3] = bf16_bits_to_f32(w.y >> 16);
      } else {
        const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (tc + i * 256) * kEs, 0, 2));
        v[4 * i + 0] = __uint_as_float(w.x);
        v[4 * i + 1] = __uint_as_float(w.y);
        v[4 * i + 2] = __uint_as_float(w.z);
        v[4 * i + 3] = __uint_as_float(w.w);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kWavePer / 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int off = (tc + i * 256 + e) * kEs;
        v[4 * i + e] = BF16 ? bf16_bits_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 2))
                            : __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 2));
      }
  }
}

// (max, sum exp) of x = v / T of the whole block in every lane of the wave:
// the lane's own pair, then the wave maximum, each lane's sum rescaled to it
// once, and a wave sum. A NaN anywhere makes the sum NaN.
__device__ __forceinline__ void wave_block_stats(float (&v)[kWavePer], int c0, int V, float T, float invT, float& M,
                                                 float& S) {
  const int tc = c0 + (int)(threadIdx.x & 63) * 4;
  float m = -INFINITY, s = 0.0f;
  bool has_nan = false;
#pragma unroll
  for (int j = 0; j < kWavePer; ++j) {
    const bool valid = tc + (j >> 2) * 256 + (j & 3) < V;
    const float x = valid ? div_t(v[j], T, invT) : -INFINITY;
    has_nan |= x != x;
    v[j] = (x == x) ? x : -INFINITY;
    m = fmaxf(m, v[j]);
  }
  if (m != -INFINITY) {
#pragma unroll
    for (int j = 0; j < kWavePer; ++j) s += fast_exp(v[j] - m);
  }
  M = wave_max_dpp(m);
  float sc = m == -INFINITY ? 0.0f : s * fast_exp(m - M);
  if (has_nan) sc = NAN;
  S = wave_sum_dpp(sc);
}

// winner key of the raw values over the block, in every lane
__device__ __forceinline__ unsigned long long wave_block_key(const float (&v)[kWavePer], int c0, int V) {
  const int tc = c0 + (int)(threadIdx.x & 63) * 4;
  float bv = -INFINITY;
  int bi = -1;
#pragma unroll
  for (int j = 0; j < kWavePer; ++j) {
    const int c = tc + (j >> 2) * 256 + (j & 3);  // increasing in j
    if (c < V) win_update(bv, bi, v[j], c);
  }
  return wave_max_u64(bi >= 0 ? win_key(bv, (uint32_t)bi) : 0ull);
}

// Grid (ceil(NC / 4), rows): wave w of work-group x takes block 4 x + w of
// the row; rows = B(K+1) target rows, then B*K cache rows when draft_lse is
// null (split over y and z, y at most 32768). One plain store per block;
// combine_kernel follows.
__global__ __launch_bounds__(kThreads) void stats_wave_kernel(VerifyArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = (int)blockIdx.x * 4 + wave;
  const int row = (int)blockIdx.z * (int)gridDim.y + (int)blockIdx.y;
  const int K = a.K, V = a.V, NC = a.NC;
  const int n_t = a.B * (K + 1);
  const int n_rows = n_t + (a.qpart ? a.B * K : 0);
  if (row >= n_rows || chunk >= NC) return;
  const bool is_target = row < n_t;
  const int b = is_target ? row / (K + 1) : (row - n_t) / K;
  const int sl = verify_slot(a, b);
  if (sl < 0) return;  // padding request: combine_kernel reads nothing of it
  const int c0 = chunk * kStatsChunk;
  float v[kWavePer];
  if (is_target) {
    // the row's loads go out first: nothing about them depends on T
    load_wave_block<false>(a.target + (long long)row * a.target_rs, V, c0, a.vec_target != 0, v);
    asm volatile("" ::: "memory");
    const float T = a.temp[sl];
    unsigned long long word;
    if (!(T > 0.0f)) {
      word = wave_block_key(v, c0, V);
    } else {
      float m, s;
      wave_block_stats(v, c0, V, T, 1.0f / T, m, s);
      word = pack_ms(m, s);
    }
    if (lane == 0) {
      a.tpart[(size_t)chunk * n_t + row] = word;
      // block 0 of target row k < K of a sampled request also records the
      // target and cache logits at draft token k, for the accept test
      const int k = row - b * (K + 1);
      if (chunk == 0 && k < K && T > 0.0f) {
        int x;
        float tx, cx;
        draft_point(a, b, sl, k, x, tx, cx);
        a.tq[b * K + k] = pack_ms(tx, cx);
      }
    }
  } else {
    const float T = a.temp[sl];
    if (!(T > 0.0f)) return;  // greedy requests never read the cache
    const int q = row - n_t, k = q - b * K;
    const long long off = (long long)verify_cache_row(a, b, sl) * a.cache_rs + (long long)k * a.cache_ss;
    if (a.cache_bf16)
      load_wave_block<true>((const uint16_t*)a.cache + off, V, c0, a.vec_cache != 0, v);
    else
      load_wave_block<false>((const float*)a.cache + off, V, c0, a.vec_cache != 0, v);
    float m, s;
    wave_block_stats(v, c0, V, T, 1.0f / T, m, s);
    if (lane == 0) a.qpart[(size_t)chunk * ((size_t)a.B * K) + q] = pack_ms(m, s);
  }
}

// After a statistics pass without arrival counting: one wave per request.
__global__ __launch_bounds__(64) void combine_kernel(VerifyArgs a) {
  __shared__ ReqLds L;
  __shared__ unsigned long long stage[kStage];
  const int b = blockIdx.x;
  combine_request(a, b, verify_slot(a, b), L, stage);
}

// With top-p: one wave per request after the top-p kernel.
__global__ __launch_bounds__(64) void decide_kernel(VerifyArgs a) {
  __shared__ ReqLds L;
  const int b = blockIdx.x, K = a.K;
  const int j = threadIdx.x;
  const int sl = verify_slot(a, b);
  if (sl < 0) {
    finish_padding(a, b);
    return;
  }
  if (j == 0) {
    L.seed = (unsigned long long)a.seeds[sl];
    L.pos0 = a.anchor_pos[b];
  }
  if (j <= K) {
    const RowStat rs = a.rowstat[b * (K + 1) + j];
    const TopP tp = a.topp ? a.topp[b * (K + 1) + j] : TopP{0u, 0, 0.0f, 0};
    L.m[j] = rs.m;
    L.lz[j] = tp.on ? tp.log_z : rs.lz;
    L.key[j] = rs.key;
    if (j < K) {
      L.lq[j] = a.qlse[b * K + j];
      if (a.temp[sl] > 0.0f) {
        draft_point(a, b, sl, j, L.x[j], L.tx[j], L.cx[j]);
      } else {
        L.x[j] = a.draft[b * K + j];
      }
    }
  }
  wave_lds_sync();
  decide(a, b, sl, L);
}

// Score of column c for the final draw: log residual + g (mode 1; only a
// positive residual is a candidate, with a finite score), else log p + g.
struct DrawCtx {
  float T, invT, M, LZ, LQ;
  TopP tp;
  uint32_t pk0, pk1, sk0, sk1;
  bool p_onehot, q_onehot;  // target / draft row without a finite logit: one-hot at column 0
};

__device__ __forceinline__ float draw_logp(const DrawCtx& d, float t, int c) {
  if (d.p_onehot) return c == 0 ? 0.0f : -INFINITY;
  return kept(d.tp, t, c) ? div_t(t, d.T, d.invT) - d.M - d.LZ : -INFINITY;
}
// the same for rows known to hold a finite logit
__device__ __forceinline__ float draw_logp_finite(const DrawCtx& d, float t, int c) {
  return kept(d.tp, t, c) ? div_t(t, d.T, d.invT) - d.M - d.LZ : -INFINITY;
}

// Gumbel-max over log p of a whole target row by one wave (lanes 0..63): the
// draw when the residual of the rejected row is empty everywhere.
__device__ unsigned long long wave_draw_p(const VerifyArgs& a, const float* trow, const DrawCtx& d) {
  const int lane = threadIdx.x & 63, V = a.V;
  float bv = -INFINITY;
  int bi = -1;
  for (int c = lane * 4; c < V; c += 256) {
    const Philox4 w = philox4x32_10((uint32_t)(c >> 2), d.pk0, d.pk1, kSaltResample, d.sk0, d.sk1);
    const uint32_t wd[4] = {w.x0, w.x1, w.x2, w.x3};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c + e < V) win_update(bv, bi, draw_logp(d, trow[c + e], c + e) + gumbel_from_word(wd[e]), c + e);
  }
  return wave_max_u64(bi >= 0 ? win_key(bv, (uint32_t)bi) : 0ull);
}

// One work-group per (request, kResCols-column block): the block's winner of
// the final draw is merged into the request's key with one atomic max; the
// last block of the request writes the output tokens. In mode 1 only the
// residual is scored; if it turns out empty everywhere (key 0) the last block
// draws from p over the whole row instead.
template <bool CBF16>
__global__ __launch_bounds__(kThreads) void residual_kernel(VerifyArgs a) {
  constexpr int kPer = kResCols / kThreads;  // columns c0 + 1024 i + 4 tid + e
  const int chunk = blockIdx.x, b = blockIdx.y;
  const ReqState rq = a.req[b];
  if (rq.mode == 2) return;
  const int K = a.K, V = a.V;
  const int j = rq.n_acc, mode = rq.mode;
  const int sl = verify_slot(a, b);  // live: padding requests are in mode 2
  DrawCtx d;
  d.T = a.temp[sl];
  d.invT = 1.0f / d.T;
  d.M = rq.M;
  d.LZ = rq.LZ;
  d.LQ = rq.LQ;
  d.tp = rq.tp;
  d.p_onehot = rq.M == -INFINITY;
  d.q_onehot = rq.LQ == -INFINITY;
  const unsigned long long sd = (unsigned long long)a.seeds[sl];
  const unsigned long long pk = (unsigned long long)(a.anchor_pos[b] + j);
  d.pk0 = (uint32_t)pk;
  d.pk1 = (uint32_t)(pk >> 32);
  d.sk0 = (uint32_t)sd;
  d.sk1 = (uint32_t)(sd >> 32);
  const bool resid = mode == 1;
  const float* trow = a.target + (long long)(b * (K + 1) + j) * a.target_rs;
  const long long crow = (long long)verify_cache_row(a, b, sl) * a.cache_rs + (long long)j * a.cache_ss;
  const int c0 = chunk * kResCols;
  const int tc = c0 + (int)threadIdx.x * 4;
  float tv[kPer], cv[kPer];
  if (a.vec_target && c0 + kResCols <= V) {  // block-uniform: all loads issued before any use
#pragma unroll
    for (int i = 0; i < kPer / 4; ++i) {
      const f32x4 w = __builtin_nontemporal_load((const f32x4*)(trow + tc + i * 1024));
      tv[4 * i + 0] = w.x;
      tv[4 * i + 1] = w.y;
      tv[4 * i + 2] = w.z;
      tv[4 * i + 3] = w.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int c = tc + (q >> 2) * 1024 + (q & 3);
      tv[q] = c < V ? trow[c] : 0.0f;
    }
  }
  // bf16 cache words stay packed until they are used, so no unpacking
  // waits on a load before the next one is issued
  uint32_t cw[kPer / 2];
  if (resid) {
    if (a.vec_cache && c0 + kResCols <= V) {
#pragma unroll
      for (int i = 0; i < kPer / 4; ++i) {
        if (CBF16) {
          const u32x2 w = __builtin_nontemporal_load((const u32x2*)((const uint16_t*)a.cache + crow + tc + i * 1024));
          cw[2 * i + 0] = w.x;
          cw[2 * i + 1] = w.y;
        } else {
          const f32x4 w = __builtin_nontemporal_load((const f32x4*)((const float*)a.cache + crow + tc + i * 1024));
          cv[4 * i + 0] = w.x;
          cv[4 * i + 1] = w.y;
          cv[4 * i + 2] = w.z;
          cv[4 * i + 3] = w.w;
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int c = tc + (q >> 2) * 1024 + (q & 3);
        if (CBF16) {
          const uint32_t h = c < V ? ((const uint16_t*)a.cache)[crow + c] : 0u;
          cw[q >> 1] = (q & 1) ? (cw[q >> 1] | (h << 16)) : h;
        } else {
          cv[q] = c < V ? ((const float*)a.cache)[crow + c] : 0.0f;
        }
      }
    }
  }
  float bv = -INFINITY;
  int bi = -1;
  // residual draw: the thread's winner of log r + g = log(r / (ln 2 * E2)),
  // E2 = -log2 u, found by comparing r / E2 across its columns (cross-
  // multiplied, strict: the lower column keeps a tie); its score then takes
  // the same float operations as in the bonus draw
  float rb = 0.0f, eb = 1.0f;
  // DEG: the target or the draft row has no finite logit (a request-uniform
  // case), so p or q is the one-hot at column 0
  auto scan = [&](auto deg_tag) {
    constexpr bool DEG = decltype(deg_tag)::value;
#pragma unroll
    for (int i = 0; i < kPer / 4; ++i) {
      const int c = tc + i * 1024;
      if (c >= V) break;
      const Philox4 w = philox4x32_10((uint32_t)(c >> 2), d.pk0, d.pk1, kSaltResample, d.sk0, d.sk1);
      const uint32_t wd[4] = {w.x0, w.x1, w.x2, w.x3};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (c + e < V) {
          const float logp = DEG ? draw_logp(d, tv[4 * i + e], c + e) : draw_logp_finite(d, tv[4 * i + e], c + e);
          if (resid) {
            const int q = 4 * i + e;
            const float cq = CBF16 ? bf16_bits_to_f32((q & 1) ? (cw[q >> 1] >> 16) : (cw[q >> 1] & 0xFFFFu)) : cv[q];
            float qv = __expf(div_t(cq, d.T, d.invT) - d.LQ);
            if (DEG && d.q_onehot) qv = c + e == 0 ? 1.0f : 0.0f;
            const float rv = __expf(logp) - qv;
            const float e2 = neg_log2_uniform(wd[e]);
            const bool take = rv > 0.0f && (bi < 0 || rv * eb > rb * e2);
            rb = take ? rv : rb;
            eb = take ? e2 : eb;
            bi = take ? c + e : bi;
          } else {
            win_update(bv, bi, logp + gumbel_from_word(wd[e]), c + e);
          }
        }
      }
    }
  };
  if (d.p_onehot || (resid && d.q_onehot))
    scan(std::integral_constant<bool, true>());
  else
    scan(std::integral_constant<bool, false>());
  if (resid && bi >= 0) bv = fmaxf(__logf(rb), -0x1.fffffep+127f) + gumbel_from_e2(eb);
  const unsigned long long key = block_max_key(bi >= 0 ? win_key(bv, (uint32_t)bi) : 0ull);
  // waves 1..3 are done; wave 0 publishes and, if last, finishes the request
  if (threadIdx.x >= 64) return;
  unsigned long long* rk = a.rkey + verify_key_index(b);
  unsigned* cnt = a.cnt + verify_counter_index(b);
  int last = 0;
  if (threadIdx.x == 0) {
    const unsigned long long prev = atomicMax(rk, key);
    asm volatile("" ::"v"(prev));  // keep the returning form
    wait_vmem();
    last = atomicAdd(cnt, 1u) == (unsigned)a.NR - 1u;
  }
  last = __shfl(last, 0);
  if (!last) return;
  // every block of the request has published: read and clear the key
  unsigned long long KEY = 0ull;
  if (threadIdx.x == 0) {
    KEY = atomicExch(rk, 0ull);
    atomicExch(cnt, 0u);
  }
  KEY = __shfl(KEY, 0);
  if (resid && KEY == 0ull) KEY = wave_draw_p(a, trow, d);
  const int token = (int)win_col(KEY);
  const int i = threadIdx.x;
  if (i <= K) {
    int v = -1;
    if (i < j) {
      v = a.draft[b * K + i];
      if (v < 0 || v >= V) v = 0;
    } else if (i == j) {
      v = token;
    }
    a.out_tokens[(size_t)b * (K + 1) + i] = v;
  }
  if (i == 0) a.num_accepted[b] = j;
}

__global__ void debug_noise_kernel(int n, const int32_t* cols, long long seed, long long pos, uint32_t salt,
                                   uint32_t* words, float* g) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int c = cols[i];
  const unsigned long long sd = (unsigned long long)seed, pk = (unsigned long long)pos;
  const Philox4 w = philox4x32_10((uint32_t)c >> 2, (uint32_t)pk, (uint32_t)(pk >> 32), salt, (uint32_t)sd,
                                  (uint32_t)(sd >> 32));
  const uint32_t wd[4] = {w.x0, w.x1, w.x2, w.x3};
  const uint32_t word = wd[c & 3];
  words[i] = word;
  g[i] = gumbel_from_word(word);
}

__global__ void debug_gumbel_kernel(int n, const uint32_t* words, float* g) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) g[i] = gumbel_from_word(words[i]);
}

}  // namespace

hipError_t launch_verify_stats(const VerifyArgs& a, hipStream_t st) {
  const int rows = a.B * (a.K + 1) + (a.qpart ? a.B * a.K : 0);
  const int gy = rows < 32768 ? rows : 32768;
  const int gz = (rows + gy - 1) / gy;
  hipLaunchKernelGGL(stats_wave_kernel, dim3((a.NC + 3) / 4, gy, gz), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_combine(const VerifyArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(combine_kernel, dim3(a.B), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decide(const VerifyArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(decide_kernel, dim3(a.B), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_residual(const VerifyArgs& a, hipStream_t st) {
  if (a.cache_bf16)
    hipLaunchKernelGGL(residual_kernel<true>, dim3(a.NR, a.B), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(residual_kernel<false>, dim3(a.NR, a.B), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_debug_noise(int n, const int32_t* cols, long long seed, long long pos, uint32_t salt,
                              uint32_t* words, float* g, hipStream_t st) {
  hipLaunchKernelGGL(debug_noise_kernel, dim3((n + 255) / 256), dim3(256), 0, st, n, cols, seed, pos, salt, words, g);
  return hipGetLastError();
}

hipError_t launch_debug_gumbel(int n, const uint32_t* words, float* g, hipStream_t st) {
  hipLaunchKernelGGL(debug_gumbel_kernel, dim3((n + 255) / 256), dim3(256), 0, st, n, words, g);
  return hipGetLastError();
}

}  // namespace mds
