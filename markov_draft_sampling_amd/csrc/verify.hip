// Rejection-sampling verification kernels (gfx950).
//
// PR #65007 (Part 2) describes the stock rejection sampler as per-block
// kernels over 8192-column statistics blocks whose partials per-request
// kernels combine, plus residual-mass and resample kernels. Here:
//   target_stats_kernel  one work-group per (target row, 8192-column block):
//                        (max, sum exp) of logit / T for sampled requests,
//                        the winner key of the raw logits for greedy ones
//                        (PR #63554, Notes: greedy verification compares with
//                        the target argmax and never reads the draft cache);
//   draft_stats_kernel   the same (max, sum exp) over the draft cache rows,
//                        only when the draft loop did not provide them;
//   residual_kernel      one work-group per (request, block): every group
//                        first combines its request's partials and runs the
//                        K accept tests p(x) >= u * q(x) itself (a few scalar
//                        loads), then draws over its block with Gumbel-max
//                        from the normalised residual max(0, p - q) of the
//                        first rejected row, or from p for the bonus token;
//   verify_finalize_kernel  combines the per-block draws and writes tokens.
#include "mds_device.h"
#include "mds_internal.h"

namespace mds {

namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kStatsChunk / kThreads;  // 32 columns

__device__ __forceinline__ float load_f32_or_bf16(const void* p, long long off, int bf16) {
  return bf16 ? bf16_bits_to_f32(((const uint16_t*)p)[off]) : ((const float*)p)[off];
}

// block-wide merge of (m, s) and of a winner key over 4 waves
__device__ __forceinline__ void block_merge(float& m, float& s, unsigned long long& key, float* sm, float* ss,
                                            unsigned long long* sk) {
  wave_lse_merge(m, s);
  key = wave_max_u64(key);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sm[wave] = m;
    ss[wave] = s;
    sk[wave] = key;
  }
  __syncthreads();
  m = sm[0];
  s = ss[0];
  key = sk[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) {
    lse_merge(m, s, sm[w], ss[w]);
    key = sk[w] > key ? sk[w] : key;
  }
}

// (max, sum exp) of x = v / T and the raw winner key over one 8192-column block
template <bool BF16>
__device__ void row_block_stats(const void* rowp, int V, int c_begin, bool vec, float T, float invT, bool want_stats,
                                bool want_key, StatPart* out) {
  __shared__ float sm[4], ss[4];
  __shared__ unsigned long long sk[4];
  float vals[kPerThread];
  int cols[kPerThread / 4];
#pragma unroll
  for (int i = 0; i < kPerThread / 4; ++i) {
    const int c = c_begin + (i * kThreads + threadIdx.x) * 4;
    cols[i] = c;
    const int n = V - c >= 4 ? 4 : (V - c > 0 ? V - c : 0);
    if (vec && n == 4) {
      if (BF16) {
        const u32x2 w = __builtin_nontemporal_load((const u32x2*)((const uint16_t*)rowp + c));
        vals[4 * i + 0] = bf16_bits_to_f32(w.x & 0xFFFFu);
        vals[4 * i + 1] = bf16_bits_to_f32(w.x >> 16);
        vals[4 * i + 2] = bf16_bits_to_f32(w.y & 0xFFFFu);
        vals[4 * i + 3] = bf16_bits_to_f32(w.y >> 16);
      } else {
        const f32x4 w = __builtin_nontemporal_load((const f32x4*)((const float*)rowp + c));
        vals[4 * i + 0] = w.x;
        vals[4 * i + 1] = w.y;
        vals[4 * i + 2] = w.z;
        vals[4 * i + 3] = w.w;
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) vals[4 * i + t] = t < n ? load_f32_or_bf16(rowp, c + t, BF16) : -INFINITY;
    }
  }
  float m = -INFINITY, s = 0.0f;
  bool has_nan = false;
  unsigned long long key = 0ull;
  if (want_stats) {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const bool valid = cols[j >> 2] + (j & 3) < V;
      const float x = valid ? div_t(vals[j], T, invT) : -INFINITY;
      has_nan |= valid && (x != x);
      vals[j] = (x == x) ? x : -INFINITY;
      m = fmaxf(m, vals[j]);
    }
    if (m != -INFINITY) {
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) s += fast_exp(vals[j] - m);
    }
    if (has_nan) s = NAN;
  }
  if (want_key) {
    float bv = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < kPerThread / 4; ++i) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (cols[i] + t < V) win_update(bv, bi, vals[4 * i + t], cols[i] + t);
    }
    key = bi >= 0 ? win_key(bv, (uint32_t)bi) : 0ull;
  }
  block_merge(m, s, key, sm, ss, sk);
  if (threadIdx.x == 0) {
    out->m = m;
    out->s = s;
    out->key = key;
  }
}

__global__ __launch_bounds__(kThreads) void target_stats_kernel(VerifyArgs a) {
  const int chunk = blockIdx.x, row = blockIdx.y;
  const int b = row / (a.K + 1);
  const float T = a.temp[b];
  const bool greedy = !(T > 0.0f);
  const float* rowp = a.target + (long long)row * a.target_rs;
  row_block_stats<false>(rowp, a.V, chunk * kStatsChunk, a.vec_target, greedy ? 1.0f : T, greedy ? 1.0f : 1.0f / T,
                         !greedy, greedy, a.tpart + (size_t)row * a.NC + chunk);
}

__global__ __launch_bounds__(kThreads) void draft_stats_kernel(VerifyArgs a) {
  const int chunk = blockIdx.x, row = blockIdx.y;  // row = b*K + k
  const int b = row / a.K, k = row - b * a.K;
  const float T = a.temp[b];
  StatPart* out = a.qpart + (size_t)row * a.NC + chunk;
  if (!(T > 0.0f)) {
    if (threadIdx.x == 0) *out = StatPart{-INFINITY, 0.0f, 0ull};
    return;
  }
  const long long off = (long long)b * a.cache_rs + (long long)k * a.cache_ss;
  if (a.cache_bf16)
    row_block_stats<true>((const uint16_t*)a.cache + off, a.V, chunk * kStatsChunk, a.vec_cache, T, 1.0f / T, true,
                          false, out);
  else
    row_block_stats<false>((const float*)a.cache + off, a.V, chunk * kStatsChunk, a.vec_cache, T, 1.0f / T, true,
                           false, out);
}

// combine NC partials of `parts` with one wave; returns (m, s) and key in lane 0..63
__device__ __forceinline__ void combine_parts(const StatPart* parts, int NC, float& m, float& s,
                                              unsigned long long& key) {
  const int lane = threadIdx.x & 63;
  m = -INFINITY;
  s = 0.0f;
  key = 0ull;
  for (int i = lane; i < NC; i += 64) {
    const StatPart p = parts[i];
    lse_merge(m, s, p.m, p.s);
    key = p.key > key ? p.key : key;
  }
  wave_lse_merge(m, s);
  key = wave_max_u64(key);
}

__device__ __forceinline__ bool kept(const TopP& tp, float t, int v) {
  if (!tp.on) return true;
  const uint32_t o = ord_f32(t);
  return o > tp.tau || (o == tp.tau && v <= tp.cut);
}

constexpr int kMaxK = 32;

__global__ __launch_bounds__(kThreads) void residual_kernel(VerifyArgs a) {
  __shared__ float s_m[kMaxK + 1], s_lz[kMaxK + 1], s_lq[kMaxK];
  __shared__ unsigned long long s_key[kMaxK + 1];
  __shared__ int s_n, s_mode, s_acc[kMaxK];
  __shared__ float sm[4], ss[4];
  __shared__ unsigned long long sk[4];
  const int chunk = blockIdx.x, b = blockIdx.y;
  const int K = a.K, V = a.V;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float T = a.temp[b];
  const bool greedy = !(T > 0.0f);
  const float invT = greedy ? 1.0f : 1.0f / T;

  // per-row statistics of this request
  for (int j = wave; j <= K; j += 4) {
    float m, s;
    unsigned long long key;
    combine_parts(a.tpart + (size_t)(b * (K + 1) + j) * a.NC, a.NC, m, s, key);
    if (lane == 0) {
      s_m[j] = m;
      s_lz[j] = (a.topp && a.topp[b * (K + 1) + j].on) ? a.topp[b * (K + 1) + j].log_z : __logf(s);
      s_key[j] = key;
    }
  }
  if (!greedy) {
    if (a.qpart) {
      for (int k = wave; k < K; k += 4) {
        float m, s;
        unsigned long long key;
        combine_parts(a.qpart + (size_t)(b * K + k) * a.NC, a.NC, m, s, key);
        if (lane == 0) s_lq[k] = (s != s) ? NAN : m + __logf(s);
      }
    } else {
      for (int k = threadIdx.x; k < K; k += kThreads) s_lq[k] = a.draft_lse[b * K + k];
    }
  }
  __syncthreads();

  // the K accept tests are independent; the first failing one ends the run
  for (int k = threadIdx.x; k < K; k += kThreads) {
    int x = a.draft[b * K + k];
    bool ok;
    if (greedy) {
      ok = x == (int32_t)win_col(s_key[k]);
    } else {
      if (x < 0 || x >= V) {
        set_status(a.status, kStatusBadDraft);
        x = 0;
      }
      const long long rowoff = (long long)(b * (K + 1) + k) * a.target_rs;
      const float tx = a.target[rowoff + x];
      float logp = -INFINITY;
      if (!a.topp || kept(a.topp[b * (K + 1) + k], tx, x)) logp = div_t(tx, T, invT) - s_m[k] - s_lz[k];
      const float p = expf(logp);
      const long long coff = (long long)b * a.cache_rs + (long long)k * a.cache_ss + x;
      const float cx = load_f32_or_bf16(a.cache, coff, a.cache_bf16);
      const float q = expf(div_t(cx, T, invT) - s_lq[k]);
      const unsigned long long sd = (unsigned long long)a.seeds[b];
      const unsigned long long pk = (unsigned long long)(a.anchor_pos[b] + k);
      const Philox4 w = philox4x32_10(0u, (uint32_t)pk, (uint32_t)(pk >> 32), kSaltAccept, (uint32_t)sd,
                                      (uint32_t)(sd >> 32));
      const float u = uniform24(w.x0);
      ok = p >= u * q;  // a NaN q rejects
    }
    s_acc[k] = ok;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    while (n < K && s_acc[n]) ++n;
    const int mode = greedy ? 2 : (n < K ? ((s_lq[n] != s_lq[n]) ? 3 : 1) : 0);
    s_n = n;
    s_mode = mode;
    if (chunk == 0) a.req[b] = ReqState{n, n, mode, greedy ? (int)win_col(s_key[n]) : -1};
  }
  __syncthreads();
  const int n = s_n, mode = s_mode;
  if (mode == 2) return;

  // Gumbel-max over this block of row n: log residual, and log p as fallback / bonus
  const int j = n;
  const float M = s_m[j], LZ = s_lz[j];
  const float LQ = mode == 1 ? s_lq[j] : 0.0f;
  const TopP tp = a.topp ? a.topp[b * (K + 1) + j] : TopP{0u, 0, 0.0f, 0};
  const float* trow = a.target + (long long)(b * (K + 1) + j) * a.target_rs;
  const long long crow = (long long)b * a.cache_rs + (long long)j * a.cache_ss;
  const unsigned long long sd = (unsigned long long)a.seeds[b];
  const unsigned long long pk = (unsigned long long)(a.anchor_pos[b] + j);
  float bvr = -INFINITY, bvp = -INFINITY, sum_r = 0.0f;
  int bir = -1, bip = -1;
  const int c_begin = chunk * kStatsChunk;
#pragma unroll 2
  for (int i = 0; i < kPerThread / 4; ++i) {
    const int c = c_begin + (i * kThreads + threadIdx.x) * 4;
    const int nv = V - c >= 4 ? 4 : (V - c > 0 ? V - c : 0);
    if (nv == 0) continue;
    float tv[4], cv[4];
    if (a.vec_target && nv == 4) {
      const f32x4 w = __builtin_nontemporal_load((const f32x4*)(trow + c));
      tv[0] = w.x;
      tv[1] = w.y;
      tv[2] = w.z;
      tv[3] = w.w;
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) tv[t] = t < nv ? trow[c + t] : 0.0f;
    }
    if (mode == 1) {
      if (a.vec_cache && nv == 4) {
        if (a.cache_bf16) {
          const u32x2 w = __builtin_nontemporal_load((const u32x2*)((const uint16_t*)a.cache + crow + c));
          cv[0] = bf16_bits_to_f32(w.x & 0xFFFFu);
          cv[1] = bf16_bits_to_f32(w.x >> 16);
          cv[2] = bf16_bits_to_f32(w.y & 0xFFFFu);
          cv[3] = bf16_bits_to_f32(w.y >> 16);
        } else {
          const f32x4 w = __builtin_nontemporal_load((const f32x4*)((const float*)a.cache + crow + c));
          cv[0] = w.x;
          cv[1] = w.y;
          cv[2] = w.z;
          cv[3] = w.w;
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) cv[t] = t < nv ? load_f32_or_bf16(a.cache, crow + c + t, a.cache_bf16) : 0.0f;
      }
    }
    const Philox4 w = philox4x32_10((uint32_t)(c >> 2), (uint32_t)pk, (uint32_t)(pk >> 32), kSaltResample,
                                    (uint32_t)sd, (uint32_t)(sd >> 32));
    const uint32_t wd[4] = {w.x0, w.x1, w.x2, w.x3};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t >= nv) break;
      const float g = gumbel_from_word(wd[t]);
      const float logp = kept(tp, tv[t], c + t) ? div_t(tv[t], T, invT) - M - LZ : -INFINITY;
      win_update(bvp, bip, logp + g, c + t);
      if (mode == 1) {
        const float pv = __expf(logp);
        const float qv = __expf(div_t(cv[t], T, invT) - LQ);
        const float rv = pv - qv;
        const float sr = rv > 0.0f ? __logf(rv) + g : -INFINITY;
        sum_r += rv > 0.0f ? rv : 0.0f;
        win_update(bvr, bir, sr, c + t);
      }
    }
  }
  unsigned long long kr = bir >= 0 ? win_key(bvr, (uint32_t)bir) : 0ull;
  unsigned long long kp = bip >= 0 ? win_key(bvp, (uint32_t)bip) : 0ull;
  kr = wave_max_u64(kr);
  kp = wave_max_u64(kp);
  sum_r = wave_sum_f32(sum_r);
  if (lane == 0) {
    sk[wave] = kr;
    sm[wave] = sum_r;
  }
  __shared__ unsigned long long skp[4];
  if (lane == 0) skp[wave] = kp;
  __syncthreads();
  if (threadIdx.x == 0) {
    ResPart out{0ull, 0ull, 0.0f, 0.0f};
    for (int wv = 0; wv < 4; ++wv) {
      out.key_r = sk[wv] > out.key_r ? sk[wv] : out.key_r;
      out.key_p = skp[wv] > out.key_p ? skp[wv] : out.key_p;
      out.sum_r += sm[wv];
    }
    a.rpart[(size_t)b * a.NC + chunk] = out;
  }
}

__global__ __launch_bounds__(kThreads) void verify_finalize_kernel(VerifyArgs a) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= a.B) return;
  const ReqState rq = a.req[b];
  int token = rq.token;
  if (rq.mode != 2) {
    unsigned long long kr = 0ull, kp = 0ull;
    float sr = 0.0f;
    for (int i = lane; i < a.NC; i += 64) {
      const ResPart p = a.rpart[(size_t)b * a.NC + i];
      kr = p.key_r > kr ? p.key_r : kr;
      kp = p.key_p > kp ? p.key_p : kp;
      sr += p.sum_r;
    }
    kr = wave_max_u64(kr);
    kp = wave_max_u64(kp);
    sr = wave_sum_f32(sr);
    token = (int)win_col((rq.mode == 1 && sr > 0.0f) ? kr : kp);
  }
  const int K = a.K;
  for (int i = lane; i <= K; i += 64) {
    int v = -1;
    if (i < rq.n_acc) {
      v = a.draft[b * K + i];
      if (v < 0 || v >= a.V) v = 0;
    } else if (i == rq.n_acc) {
      v = token;
    }
    a.out_tokens[(size_t)b * (K + 1) + i] = v;
  }
  if (lane == 0) a.num_accepted[b] = rq.n_acc;
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

hipError_t launch_target_stats(const VerifyArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(target_stats_kernel, dim3(a.NC, a.B * (a.K + 1)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_draft_stats(const VerifyArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(draft_stats_kernel, dim3(a.NC, a.B * a.K), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_residual(const VerifyArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(residual_kernel, dim3(a.NC, a.B), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_verify_finalize(const VerifyArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(verify_finalize_kernel, dim3((a.B + 3) / 4), dim3(kThreads), 0, st, a);
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
