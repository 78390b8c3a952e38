// Markov draft loop kernels (gfx950).
//
// One launch of draft_step_kernel runs one step of the sequential loop of the
// DSparkSpeculator API page (_sample_markov_chain: Markov embedding of the
// previous token -> Markov bias -> biased logits -> _sample_logits) for every
// request at once, fused:
//   * w2 [V, r] bf16 is streamed once per step and projected against the
//     embeddings of all requests of the batch tile with bf16 MFMA
//     (v_mfma_f32_16x16x32_bf16: M = 16 vocabulary columns, N = 16 requests,
//     K = 32 of the rank), fp32 accumulation;
//   * the epilogue works straight from the accumulator layout (lane l holds
//     four consecutive columns of request l % 16): z = base + bias, store of
//     the draft-logits cache, z / T, Philox-keyed Gumbel noise, a running
//     first-NaN/first-max winner and the (max, sum exp) of cache / T that the
//     verifier needs for q;
//   * per work-group winners are merged with one 64-bit atomic max per
//     request (the key orders values by the winner rule and breaks ties by the
//     lower column), which replaces the pages' per-1024-column block maxima
//     and their cross-block pass: the rule composes over any column
//     partition (PR #65007, Part 1, step 4).
// The next step reads the winner of the previous one as its previous token;
// the kernel boundary orders the steps.
#include "mds_device.h"
#include "mds_internal.h"

namespace mds {

namespace {

// LDS row stride of the embedding tile in bf16 elements: r plus 8 (16 bytes)
// so that the 16 rows a ds_read_b128 touches start on different banks.
__device__ __forceinline__ int emb_stride(int r) { return r + 8; }

template <bool BF16>
__device__ __forceinline__ void load4(const void* p, long long off, int n, bool vec, float (&v)[4]) {
  if (BF16) {
    const uint16_t* q = (const uint16_t*)p + off;
    if (vec && n == 4) {
      const u32x2 w = __builtin_nontemporal_load((const u32x2*)q);
      v[0] = bf16_bits_to_f32(w.x & 0xFFFFu);
      v[1] = bf16_bits_to_f32(w.x >> 16);
      v[2] = bf16_bits_to_f32(w.y & 0xFFFFu);
      v[3] = bf16_bits_to_f32(w.y >> 16);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = t < n ? bf16_bits_to_f32(q[t]) : 0.0f;
    }
  } else {
    const float* q = (const float*)p + off;
    if (vec && n == 4) {
      const f32x4 w = __builtin_nontemporal_load((const f32x4*)q);
      v[0] = w.x;
      v[1] = w.y;
      v[2] = w.z;
      v[3] = w.w;
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = t < n ? q[t] : 0.0f;
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void store4(void* p, long long off, int n, bool vec, const float (&z)[4], float (&stored)[4]) {
  if (BF16) {
    uint32_t h[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      h[t] = f32_to_bf16_bits(z[t]);
      stored[t] = bf16_bits_to_f32(h[t]);
    }
    uint16_t* q = (uint16_t*)p + off;
    if (vec && n == 4) {
      u32x2 w;
      w.x = h[0] | (h[1] << 16);
      w.y = h[2] | (h[3] << 16);
      __builtin_nontemporal_store(w, (u32x2*)q);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t < n) q[t] = (uint16_t)h[t];
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) stored[t] = z[t];
    float* q = (float*)p + off;
    if (vec && n == 4) {
      const f32x4 w = {z[0], z[1], z[2], z[3]};
      __builtin_nontemporal_store(w, (f32x4*)q);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t < n) q[t] = z[t];
    }
  }
}

// RKT: r / 32 when known at compile time, 0 for a runtime rank (<= 512).
template <int NB, int RKT>
__global__ __launch_bounds__(256) void draft_step_kernel(DraftStepArgs a) {
  constexpr int NT = NB / 16;
  constexpr int RKMAX = RKT > 0 ? RKT : 16;
  const int RK = RKT > 0 ? RKT : (a.r >> 5);
  extern __shared__ __align__(16) unsigned char smem[];
  const int rs = emb_stride(a.r);
  uint16_t* s_e = (uint16_t*)smem;                             // [NB][rs]
  int* s_prev = (int*)(smem + (size_t)NB * rs * 2);           // [NB]
  unsigned long long* s_key = (unsigned long long*)(s_prev + NB);  // [4][NB]
  float* s_qm = (float*)(s_key + 4 * NB);                      // [4][NB]
  float* s_qs = s_qm + 4 * NB;                                 // [4][NB]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Work-groups are dealt round-robin to the 8 XCDs by linear id. When the
  // slab count is a multiple of 8, the batch tiles of one column slab are
  // given ids on the same XCD so its w2 rows are re-read from that XCD's L2.
  int g, bt;
  {
    const int id = blockIdx.x;
    if ((a.G & 7) == 0) {
      const int xcd = id & 7, local = id >> 3;
      g = (local / a.BT) * 8 + xcd;
      bt = local - (local / a.BT) * a.BT;
    } else {
      g = id % a.G;
      bt = id / a.G;
    }
  }
  const int b0 = bt * NB;
  const int k = a.k;

  // previous token of every request of the tile
  for (int i = tid; i < NB; i += 256) {
    const int b = b0 + i;
    int prev = 0;
    if (b < a.B) {
      long long t = (k == 0) ? (long long)a.anchor[b] : (long long)win_col(a.keys[(size_t)(k - 1) * a.B + b]);
      if (t < 0 || t >= a.V) {
        set_status(a.status, kStatusBadAnchor);
        t = 0;
      }
      prev = (int)t;
    }
    s_prev[i] = prev;
  }
  __syncthreads();
  // Markov embeddings w1[prev] -> LDS (zero rows past the batch)
  {
    const int cpr = a.r >> 3;  // 16-byte chunks per row
    for (int i = tid; i < NB * cpr; i += 256) {
      const int row = i / cpr, ch = i - row * cpr;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (b0 + row < a.B) v = *(const uint4*)(a.w1 + (size_t)s_prev[row] * a.r + ch * 8);
      *(uint4*)(s_e + row * rs + ch * 8) = v;
    }
  }
  __syncthreads();

  // per-lane request parameters for each 16-request sub-tile
  const int lrow = lane & 15, lgrp = lane >> 4;
  bool rv[NT];
  float Tv[NT], invT[NT];
  uint32_t sk0[NT], sk1[NT], pk0[NT], pk1[NT];
  long long rbase[NT], rcache[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int b = b0 + nt * 16 + lrow;
    rv[nt] = b < a.B;
    const int bb = rv[nt] ? b : 0;
    Tv[nt] = a.temp[bb];
    invT[nt] = Tv[nt] > 0.0f ? 1.0f / Tv[nt] : 0.0f;
    const unsigned long long sd = (unsigned long long)a.seeds[bb];
    const unsigned long long pk = (unsigned long long)(a.anchor_pos[bb] + k);
    sk0[nt] = (uint32_t)sd;
    sk1[nt] = (uint32_t)(sd >> 32);
    pk0[nt] = (uint32_t)pk;
    pk1[nt] = (uint32_t)(pk >> 32);
    rbase[nt] = (long long)bb * a.base_rs + (long long)k * a.base_ss;
    rcache[nt] = (long long)bb * a.cache_rs + (long long)k * a.cache_ss;
  }

  float bv[NT], qm[NT], qs[NT];
  int bi[NT];
  bool qnan[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    bv[nt] = -INFINITY;
    bi[nt] = -1;
    qm[nt] = -INFINITY;
    qs[nt] = 0.0f;
    qnan[nt] = false;
  }

  const int mt_begin = (int)(((long long)g * a.nMT) / a.G);
  const int mt_end = (int)(((long long)(g + 1) * a.nMT) / a.G);
  const int V = a.V, r = a.r;

  for (int mt = mt_begin + wave; mt < mt_end; mt += 4) {
    const int c0 = mt * 16;
    // A operand: 16 rows of w2 (vocabulary columns c0..c0+15), 32 ranks per step
    bf16x8 afr[RKMAX];
    {
      const int v = c0 + lrow;
      const uint16_t* wp = a.w2 + (size_t)(v < V ? v : 0) * r + lgrp * 8;
#pragma unroll
      for (int s = 0; s < RKMAX; ++s) {
        if (s < RK) {
          bf16x8 t = *(const bf16x8*)(wp + s * 32);
          if (v >= V) t = bf16x8{};
          afr[s] = t;
        }
      }
    }
    // epilogue inputs: four consecutive columns of request (nt*16 + lrow)
    const int c = c0 + lgrp * 4;
    const int n = V - c >= 4 ? 4 : (V - c > 0 ? V - c : 0);
    float bz[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (rv[nt] && n > 0) {
        if (a.base_bf16)
          load4<true>(a.base, rbase[nt] + c, n, a.vec_base, bz[nt]);
        else
          load4<false>(a.base, rbase[nt] + c, n, a.vec_base, bz[nt]);
      }
    }
    // projection: bias[c0 + i][request j] for the tile
    floatx4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < RKMAX; ++s) {
      if (s < RK) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const bf16x8 bfr = *(const bf16x8*)(s_e + (nt * 16 + lrow) * rs + s * 32 + lgrp * 8);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[s], bfr, acc[nt], 0, 0, 0);
        }
      }
    }
    if (n == 0) continue;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (!rv[nt]) continue;
      float z[4], cv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) z[t] = bz[nt][t] + acc[nt][t];
      if (a.cache_bf16)
        store4<true>(a.cache, rcache[nt] + c, n, a.vec_cache, z, cv);
      else
        store4<false>(a.cache, rcache[nt] + c, n, a.vec_cache, z, cv);
      if (Tv[nt] > 0.0f) {
        const Philox4 w = philox4x32_10((uint32_t)(c >> 2), pk0[nt], pk1[nt], kSaltDraft, sk0[nt], sk1[nt]);
        const uint32_t wd[4] = {w.x0, w.x1, w.x2, w.x3};
        float x[4];
        float xm = -INFINITY;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float sv = div_t(z[t], Tv[nt], invT[nt]) + gumbel_from_word(wd[t]);
          if (t < n) win_update(bv[nt], bi[nt], sv, c + t);
          const float xv = div_t(cv[t], Tv[nt], invT[nt]);
          qnan[nt] |= (t < n) && (xv != xv);
          x[t] = (t < n && xv == xv) ? xv : -INFINITY;
          xm = fmaxf(xm, x[t]);
        }
        const float mn = fmaxf(qm[nt], xm);
        if (mn != -INFINITY) {
          float acc_s = qs[nt] * fast_exp(qm[nt] - mn);
#pragma unroll
          for (int t = 0; t < 4; ++t) acc_s += fast_exp(x[t] - mn);
          qs[nt] = acc_s;
          qm[nt] = mn;
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (t < n) win_update(bv[nt], bi[nt], z[t], c + t);
      }
    }
  }

  // merge the four lanes of each request, then the four waves, then publish
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    uint64_t key = bi[nt] >= 0 ? win_key(bv[nt], (uint32_t)bi[nt]) : 0ull;
    key = max_over_groups16(key);
    float m = qm[nt], s = qnan[nt] ? NAN : qs[nt];
    {
      float m2 = __shfl_xor(m, 16), s2 = __shfl_xor(s, 16);
      lse_merge(m, s, m2, s2);
      m2 = __shfl_xor(m, 32);
      s2 = __shfl_xor(s, 32);
      lse_merge(m, s, m2, s2);
    }
    if (lgrp == 0) {
      s_key[wave * NB + nt * 16 + lrow] = key;
      s_qm[wave * NB + nt * 16 + lrow] = m;
      s_qs[wave * NB + nt * 16 + lrow] = s;
    }
  }
  __syncthreads();
  for (int i = tid; i < NB; i += 256) {
    const int b = b0 + i;
    if (b >= a.B) continue;
    unsigned long long key = s_key[i];
    float m = s_qm[i], s = s_qs[i];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const unsigned long long k2 = s_key[w * NB + i];
      key = k2 > key ? k2 : key;
      lse_merge(m, s, s_qm[w * NB + i], s_qs[w * NB + i]);
    }
    if (key) atomicMax(&a.keys[(size_t)k * a.B + b], key);
    a.qpart[((size_t)k * a.B + b) * a.G + g] = make_float2(m, s);
  }
}

__global__ __launch_bounds__(256) void draft_init_kernel(unsigned long long* keys, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) keys[i] = 0ull;
}

// Draft tokens from the winner keys, and log-sum-exp of cache / T per row
// from the per-work-group partials; one wave per (request, step).
__global__ __launch_bounds__(256) void draft_finalize_kernel(DraftFinalArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.B * a.K) return;
  const int b = row / a.K, k = row - b * a.K;
  if (lane == 0) a.tokens[row] = (int32_t)win_col(a.keys[(size_t)k * a.B + b]);
  if (!a.lse) return;
  float m = -INFINITY, s = 0.0f;
  const float2* qp = a.qpart + ((size_t)k * a.B + b) * a.G;
  for (int i = lane; i < a.G; i += 64) {
    const float2 p = qp[i];
    lse_merge(m, s, p.x, p.y);
  }
  wave_lse_merge(m, s);
  if (lane == 0) {
    float out;
    if (!(a.temp[b] > 0.0f) || s != s)
      out = NAN;
    else
      out = m + __logf(s);
    a.lse[row] = out;
  }
}

template <int NB, int RKT>
hipError_t launch_step(const DraftStepArgs& a, int bt, hipStream_t st) {
  const size_t lds = (size_t)NB * (a.r + 8) * 2 + NB * 4 + 4 * NB * 8 + 8 * NB * 4;
  DraftStepArgs b = a;
  b.BT = bt;
  hipLaunchKernelGGL((draft_step_kernel<NB, RKT>), dim3(a.G * bt), dim3(256), lds, st, b);
  return hipGetLastError();
}

template <int NB>
hipError_t launch_step_nb(const DraftStepArgs& a, int bt, hipStream_t st) {
  switch (a.r) {
    case 64: return launch_step<NB, 2>(a, bt, st);
    case 128: return launch_step<NB, 4>(a, bt, st);
    case 192: return launch_step<NB, 6>(a, bt, st);
    case 256: return launch_step<NB, 8>(a, bt, st);
    default: return launch_step<NB, 0>(a, bt, st);
  }
}

}  // namespace

int draft_nb(int B, int r) {
  // batch tile: 16 or 32 requests (larger tiles exceed the register file
  // with the epilogue state of every request a lane carries)
  (void)r;
  return B <= 16 ? 16 : 32;
}

hipError_t launch_draft_init(unsigned long long* keys, int n, hipStream_t st) {
  hipLaunchKernelGGL(draft_init_kernel, dim3((n + 255) / 256), dim3(256), 0, st, keys, n);
  return hipGetLastError();
}

hipError_t launch_draft_step(const DraftStepArgs& a, hipStream_t st) {
  const int nb = draft_nb(a.B, a.r);
  const int bt = (a.B + nb - 1) / nb;
  return nb == 16 ? launch_step_nb<16>(a, bt, st) : launch_step_nb<32>(a, bt, st);
}

hipError_t launch_draft_finalize(const DraftFinalArgs& a, hipStream_t st) {
  const int rows = a.B * a.K;
  hipLaunchKernelGGL(draft_finalize_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace mds
