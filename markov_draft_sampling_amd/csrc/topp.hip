// Exact, deterministic top-p over target rows (gfx950).
//
// PR #65007, Part 2: the kept set is the shortest prefix of the columns
// ordered by logit (descending) then token id (ascending) whose probability
// mass reaches p, plus the row maximum; masses are summed in 64-bit fixed
// point so every run keeps the same set. Greedy rows skip it.
//
// One 1024-thread work-group per row:
//   * w = exp(x - max) with x = logit / T is quantised to Q = floor(w * 2^40)
//     (w <= 1, so a row of < 2^24 columns sums below 2^64); the target mass
//     is TQ = ceil(p * sum Q) (at least 1, so the maximum is always kept);
//   * the order key is ord(logit) (monotone in the logit), the id breaks ties;
//   * first the columns are binned by how far x lies below the row maximum
//     M (known from the statistics pass), 1/128 of a logit unit per bin:
//     the bins are monotone in the logit and spread the columns evenly, so
//     their LDS histogram of (mass, count) takes few colliding atomics, and
//     every column with zero quantised mass falls into one last bin that is
//     never counted; when the crossing bin holds too many columns (dense
//     ties) the crossing is instead narrowed over the 32-bit key in levels of
//     12, 12 and 8 bits, one pass over the row per level;
//   * as soon as the crossing bin holds at most kCap columns they are gathered
//     into LDS, sorted by (key desc, id asc) and prefix-summed exactly;
//   * if a single key value holds more than kCap columns (ties), all of them
//     carry the same Q and the cut is the n-th smallest id of that value.
// The result per row is (tau, cut): a column is kept iff ord(t) > tau, or
// ord(t) == tau and id <= cut; log_z is the log of the kept mass.
#include "mds_device.h"
#include "mds_internal.h"

namespace mds {

namespace {

constexpr int kTp = 1024;
constexpr int kCap = 4096;
constexpr int kNB0 = 4096;             // bins below the row maximum
constexpr float kBinScale = 128.0f;    // bins per unit of x

// bin of x below the maximum M: floor((M - x) * 128), 4095 for x at least
// 32 below M (exp(-32) < 2^-40: quantised mass 0), -inf and NaN
__device__ __forceinline__ int max_bin(float x, float M) {
  const float f = (M - x) * kBinScale;  // >= 0: M is the maximum of the same x
  return f < (float)(kNB0 - 1) ? (f > 0.0f ? (int)f : 0) : kNB0 - 1;
}

__device__ __forceinline__ unsigned long long quantise(float w) {
  return (unsigned long long)(w * 1099511627776.0f);  // floor(w * 2^40), w in [0, 1]
}

// exclusive prefix sum over the 1024 threads of the block
__device__ unsigned long long block_excl_scan(unsigned long long v, unsigned long long* scratch,
                                              unsigned long long* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) scratch[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long run = 0;
    for (int w = 0; w < kTp / 64; ++w) {
      const unsigned long long t = scratch[w];
      scratch[w] = run;
      run += t;
    }
    scratch[kTp / 64] = run;
  }
  __syncthreads();
  const unsigned long long res = scratch[wave] + inc - v;
  if (total) *total = scratch[kTp / 64];
  __syncthreads();
  return res;
}

struct RowCtx {
  const float* t;
  int V;
  bool vec;
  float T, invT, M;
};

// visit every column of the row with (column, logit); columns ascend per
// thread. Whole batches of kRowBatch vector loads go out before any of their
// values is used (one load in flight per thread would leave the pass bound
// by memory latency); the rest of the row follows one load at a time.
constexpr int kRowBatch = 4;
template <class F>
__device__ __forceinline__ void for_row(const RowCtx& r, F&& f) {
  constexpr int kStep = kTp * 4;
  int c0 = threadIdx.x * 4;
  if (r.vec) {
    for (; c0 + (kRowBatch - 1) * kStep + 4 <= r.V; c0 += kRowBatch * kStep) {
      f32x4 w[kRowBatch];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) w[u] = *(const f32x4*)(r.t + c0 + u * kStep);
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        const int c = c0 + u * kStep;
        f(c, w[u].x);
        f(c + 1, w[u].y);
        f(c + 2, w[u].z);
        f(c + 3, w[u].w);
      }
    }
  }
  for (int c = c0; c < r.V; c += kStep) {
    const int n = r.V - c >= 4 ? 4 : r.V - c;
    if (r.vec && n == 4) {
      const f32x4 w = *(const f32x4*)(r.t + c);
      f(c, w.x);
      f(c + 1, w.y);
      f(c + 2, w.z);
      f(c + 3, w.w);
    } else {
      for (int i = 0; i < n; ++i) f(c + i, r.t[c + i]);
    }
  }
}

__global__ __launch_bounds__(kTp) void top_p_kernel(VerifyArgs a) {
  __shared__ unsigned long long h_mass[4096];
  __shared__ unsigned int h_cnt[4096];
  __shared__ unsigned long long c_key[kCap];
  __shared__ unsigned long long c_q[kCap];
  __shared__ unsigned long long scratch[kTp / 64 + 1];
  __shared__ unsigned long long s_sumq, s_above, s_tq;
  __shared__ unsigned int s_digit, s_cnt, s_ncand;
  __shared__ float s_M;
  __shared__ int s_found_i;

  const int row = blockIdx.x;
  const int b = row / (a.K + 1);
  const int sl = verify_slot(a, b);
  const float T = sl >= 0 ? a.temp[sl] : 0.0f;  // padding requests: off
  const float p = sl >= 0 ? a.top_p[sl] : 1.0f;
  TopP* out = a.topp + row;
  if (!(T > 0.0f) || !(p < 1.0f)) {
    if (threadIdx.x == 0) *out = TopP{0u, 0, 0.0f, 0};
    return;
  }
  const int tid = threadIdx.x;
  if (tid == 0) s_M = a.rowstat[row].m;
  __syncthreads();
  if (s_M == -INFINITY) {  // no finite logit: only the first column (the row maximum by rule) is kept
    if (tid == 0) *out = TopP{ord_f32(-INFINITY), 0, -INFINITY, 1};
    return;
  }
  RowCtx rc{a.target + (long long)row * a.target_rs, a.V, a.vec_target != 0, T, 1.0f / T, s_M};

  // total quantised mass and the histogram of the bins below the maximum
  for (int i = tid; i < kNB0; i += kTp) {
    h_mass[i] = 0;
    h_cnt[i] = 0;
  }
  __syncthreads();
  {
    unsigned long long sumq = 0;
    for_row(rc, [&](int, float t) {
      const float x = div_t(t, rc.T, rc.invT);
      const unsigned long long q = quantise(fast_exp(x - rc.M));
      const int d = max_bin(x, rc.M);
      if (d < kNB0 - 1) {  // the last bin holds mass 0 only: never the crossing
        if (q) atomicAdd(&h_mass[d], q);
        atomicAdd(&h_cnt[d], 1u);
      }
      sumq += q;
    });
    unsigned long long tot;
    block_excl_scan(sumq, scratch, &tot);
    if (tid == 0) {
      s_sumq = tot;
      unsigned long long tq = (unsigned long long)ceil((double)p * (double)tot);
      if (tq < 1) tq = 1;
      if (tq > tot) tq = tot;
      s_tq = tq;
      s_digit = kNB0;
      s_cnt = 0;
      s_above = 0;
    }
    __syncthreads();
    // crossing bin, in ascending bin (descending logit) order
    unsigned long long loc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) loc += h_mass[tid * 4 + j];
    const unsigned long long ex = block_excl_scan(loc, scratch, nullptr);
    const unsigned long long need = s_tq;
    unsigned long long run = ex;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = tid * 4 + j;
      const unsigned long long mass = h_mass[d];
      if (run < need && need <= run + mass) {
        s_digit = (unsigned int)d;
        s_above = run;
        s_cnt = h_cnt[d];
      }
      run += mass;
    }
    __syncthreads();
  }
  const int bin0 = (int)s_digit;  // kNB0 if no bin crossed (cannot happen for finite rows)
  unsigned long long above = s_above;
  unsigned int cnt = s_cnt;
  // filter of the crossing bin's columns for the gather below: the bin below
  // the maximum, or (after narrowing) the key prefix
  bool by_bin = bin0 < kNB0 && cnt <= (unsigned int)kCap;
  unsigned int prefix = 0;
  int pbits = 0;
  if (!by_bin) {
    above = 0;
    cnt = 0;
    // narrowing levels: (shift, width) of the digit below the fixed prefix
    const int shifts[3] = {20, 8, 0};
    const int widths[3] = {12, 12, 8};
    for (int lvl = 0; lvl < 3; ++lvl) {
      const int nb = 1 << widths[lvl], sh = shifts[lvl];
      for (int i = tid; i < nb; i += kTp) {
        h_mass[i] = 0;
        h_cnt[i] = 0;
      }
      __syncthreads();
      unsigned long long sumq = 0;
      const unsigned int pf = prefix;
      const int pb = pbits;
      for_row(rc, [&](int, float t) {
        const uint32_t o = ord_f32(t);
        if (pb && (o >> (32 - pb)) != pf) return;
        const float x = div_t(t, rc.T, rc.invT);
        const unsigned long long q = quantise(fast_exp(x - rc.M));
        const unsigned int d = (o >> sh) & (nb - 1);
        atomicAdd(&h_mass[d], q);
        atomicAdd(&h_cnt[d], 1u);
        sumq += q;
      });
      if (lvl == 0) {
        unsigned long long tot;
        block_excl_scan(sumq, scratch, &tot);
        if (tid == 0) {
          s_sumq = tot;
          unsigned long long tq = (unsigned long long)ceil((double)p * (double)tot);
          if (tq < 1) tq = 1;
          if (tq > tot) tq = tot;
          s_tq = tq;
        }
      }
      __syncthreads();
      // crossing bin, scanning digits from the top
      if (tid == 0) {
        s_digit = 0;
        s_cnt = 0;
        s_above = above;
      }
      __syncthreads();
      unsigned long long loc = 0;
      const int d0 = nb - 1 - tid * 4;
      for (int j = 0; j < 4; ++j)
        if (d0 - j >= 0) loc += h_mass[d0 - j];
      const unsigned long long ex = block_excl_scan(loc, scratch, nullptr);
      {
        const unsigned long long need = s_tq - above;
        unsigned long long run = ex;
        for (int j = 0; j < 4; ++j) {
          const int d = d0 - j;
          if (d < 0) break;
          const unsigned long long mass = h_mass[d];
          if (run < need && need <= run + mass) {
            s_digit = (unsigned int)d;
            s_above = above + run;
            s_cnt = h_cnt[d];
          }
          run += mass;
        }
      }
      __syncthreads();
      prefix = (prefix << widths[lvl]) | s_digit;
      pbits += widths[lvl];
      above = s_above;
      cnt = s_cnt;
      __syncthreads();
      if (cnt <= (unsigned int)kCap) break;
    }

  }

  const unsigned long long tq = s_tq;
  uint32_t tau;
  int cut;
  unsigned long long kept_mass;
  if (cnt <= (unsigned int)kCap) {
    // gather the crossing bin, sort it exactly, prefix-sum its masses
    if (tid == 0) s_ncand = 0;
    __syncthreads();
    const unsigned int pf = prefix;
    const int pb = pbits;
    for_row(rc, [&](int c, float t) {
      const uint32_t o = ord_f32(t);
      const float x = div_t(t, rc.T, rc.invT);
      if (by_bin ? max_bin(x, rc.M) != bin0 : (o >> (32 - pb)) != pf) return;
      const unsigned int slot = atomicAdd(&s_ncand, 1u);
      if (slot < (unsigned int)kCap) {
        c_key[slot] = ((unsigned long long)o << 32) | (uint32_t)(~(uint32_t)c);
        c_q[slot] = quantise(fast_exp(x - rc.M));
      }
    });
    __syncthreads();
    const int n = (int)min(s_ncand, (unsigned int)kCap);
    if (n == 0) {  // no crossing found (cannot happen for finite rows): keep every column
      if (tid == 0) *out = TopP{0u, 0, 0.0f, 0};
      return;
    }
    int P = 1;
    while (P < n) P <<= 1;
    for (int i = n + tid; i < P; i += kTp) {
      c_key[i] = 0ull;
      c_q[i] = 0ull;
    }
    __syncthreads();
    // bitonic sort, descending by key (column order: logit desc, id asc)
    for (int k = 2; k <= P; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P; i += kTp) {
          const int l = i ^ j;
          if (l > i) {
            const bool desc = (i & k) == 0;
            const unsigned long long ki = c_key[i], kl = c_key[l];
            if (desc ? (ki < kl) : (ki > kl)) {
              c_key[i] = kl;
              c_key[l] = ki;
              const unsigned long long q = c_q[i];
              c_q[i] = c_q[l];
              c_q[l] = q;
            }
          }
        }
        __syncthreads();
      }
    }
    // first sorted position whose inclusive prefix reaches the target
    unsigned long long loc = 0;
    for (int j = 0; j < 4; ++j)
      if (tid * 4 + j < n) loc += c_q[tid * 4 + j];
    const unsigned long long ex = block_excl_scan(loc, scratch, nullptr);
    if (tid == 0) s_found_i = -1;
    __syncthreads();
    {
      const unsigned long long need = tq - above;
      unsigned long long run = ex;
      for (int j = 0; j < 4; ++j) {
        const int i = tid * 4 + j;
        if (i >= n) break;
        const unsigned long long q = c_q[i];
        if (run < need && need <= run + q) {
          s_found_i = i;
          s_above = above + run + q;
        }
        run += q;
      }
    }
    __syncthreads();
    const int fi = s_found_i >= 0 ? s_found_i : n - 1;
    tau = (uint32_t)(c_key[fi] >> 32);
    cut = (int)(~(uint32_t)c_key[fi]);
    kept_mass = s_found_i >= 0 ? s_above : above;
  } else {
    // one key value holds more than kCap columns: they all carry the same
    // mass; keep the n smallest ids of that value
    tau = prefix;
    unsigned long long qtie = 0;
    for_row(rc, [&](int, float t) {
      if (ord_f32(t) == tau && qtie == 0) qtie = quantise(fast_exp(div_t(t, rc.T, rc.invT) - rc.M));
    });
    // any thread that saw the value knows q; share it
    if (tid == 0) s_sumq = 0;
    __syncthreads();
    if (qtie) atomicMax(&s_sumq, qtie);
    __syncthreads();
    qtie = s_sumq;
    const unsigned long long need = tq - above;
    const unsigned long long nkeep = (need + qtie - 1) / qtie;
    const int span = (a.V + kTp - 1) / kTp;
    const int lo = tid * span, hi = min(a.V, lo + span);
    unsigned long long c = 0;
    for (int v = lo; v < hi; ++v) c += ord_f32(rc.t[v]) == tau;
    const unsigned long long ex = block_excl_scan(c, scratch, nullptr);
    if (tid == 0) s_found_i = a.V - 1;
    __syncthreads();
    if (ex < nkeep && nkeep <= ex + c) {
      unsigned long long run = ex;
      for (int v = lo; v < hi; ++v) {
        if (ord_f32(rc.t[v]) == tau && ++run == nkeep) {
          s_found_i = v;
          break;
        }
      }
    }
    __syncthreads();
    cut = s_found_i;
    kept_mass = above + nkeep * qtie;
  }
  if (tid == 0) {
    const double z = (double)kept_mass * 0x1p-40;
    *out = TopP{tau, cut, (float)log(z), 1};
  }
}

__global__ void debug_top_p_out_kernel(int rows, const TopP* tp, uint32_t* tau, int32_t* cut, float* log_z,
                                       int32_t* on) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= rows) return;
  tau[i] = tp[i].tau;
  cut[i] = tp[i].cut;
  log_z[i] = tp[i].log_z;
  on[i] = tp[i].on;
}

}  // namespace

hipError_t launch_debug_top_p_out(int rows, const TopP* tp, uint32_t* tau, int32_t* cut, float* log_z, int32_t* on,
                                  hipStream_t st) {
  hipLaunchKernelGGL(debug_top_p_out_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, rows, tp, tau, cut, log_z,
                     on);
  return hipGetLastError();
}

hipError_t launch_top_p(const VerifyArgs& a, hipStream_t st) {
  if (a.B * (a.K + 1) == 0) return hipSuccess;
  hipLaunchKernelGGL(top_p_kernel, dim3(a.B * (a.K + 1)), dim3(kTp), 0, st, a);
  return hipGetLastError();
}

}  // namespace mds
