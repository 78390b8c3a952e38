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

size_t draft_step_lds(int NB, int r) {
  return (size_t)64 * r * 2 + (size_t)NB * (r + 8) * 2 + (size_t)NB * (64 + 4) * 4 + NB * 4 + 4 * NB * 8 + 8 * NB * 4;
}

namespace {

// LDS row stride of the embedding tile in bf16 elements: r plus 8 (16 bytes)
// so that the 16 rows a ds_read_b128 touches start on different banks.
__device__ __forceinline__ int emb_stride(int r) { return r + 8; }

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
      *(u32x2*)q = w;
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
      *(f32x4*)q = w;
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t < n) q[t] = z[t];
    }
  }
}

// Geometry of one step kernel work-group: NB requests x CW = 64 columns per
// chunk; each of the 4 waves owns one 16-column MFMA tile of the chunk.
constexpr int kCW = 64;

template <bool BF16>
__device__ __forceinline__ void load_row4(const void* p, long long off, int n, bool vec, float (&v)[4]) {
  if (BF16) {
    const uint16_t* q = (const uint16_t*)p + off;
    if (vec && n == 4) {
      const u32x2 w = *(const u32x2*)q;
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
      const f32x4 w = *(const f32x4*)q;
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

// The chunk's w2 rows [c0, c0 + 64) x r are loaded with coalesced 16-byte
// loads and stored in LDS row-major with the 16-byte column chunks of row rho
// XOR-permuted by (rho & 7): the MFMA operand reads (16 rows, same chunk)
// then hit 8 distinct bank groups.
template <int NB, int RKT>
__global__ __launch_bounds__(256) void draft_step_kernel(DraftStepArgs a) {
  constexpr int NT = NB / 16;     // 16-request MFMA tiles
  constexpr int EPT = NB * kCW / 4 / 256;  // float4 groups of the epilogue per thread
  constexpr int RKMAX = RKT > 0 ? RKT : 16;
  constexpr int WLMAX = RKMAX;    // 16-byte w2 loads per thread per chunk = 64 * r / 8 / 256 = r / 32
  const int RK = RKT > 0 ? RKT : (a.r >> 5);
  const int r = a.r, V = a.V, k = a.k;
  const int cpr = r >> 3;                 // 16-byte chunks per w2 row
  const int xmask = (cpr & 7) ? 3 : 7;  // keeps the permuted chunk inside its row
  extern __shared__ __align__(16) unsigned char smem[];
  const int rs = emb_stride(r);
  uint16_t* s_w = (uint16_t*)smem;                                   // [64][r] swizzled w2 stage
  uint16_t* s_e = s_w + kCW * r;                                     // [NB][rs] embeddings
  float* s_bias = (float*)(s_e + NB * rs);                           // [NB][kCW + 4]
  int* s_prev = (int*)(s_bias + NB * (kCW + 4));                     // [NB]
  unsigned long long* s_key = (unsigned long long*)(s_prev + NB);    // [4][NB]
  float* s_qm = (float*)(s_key + 4 * NB);                            // [4][NB]
  float* s_qs = s_qm + 4 * NB;                                       // [4][NB]
  constexpr int BST = kCW + 4;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Work-groups are dealt round-robin to the 8 XCDs by linear id. When the
  // slab count is a multiple of 8, the batch tiles of one column slab get ids
  // on the same XCD so its w2 rows are re-read from that XCD's L2.
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

  // this work-group's columns: 16-column tiles [mt_begin, mt_end)
  const int mt_begin = (int)(((long long)g * a.nMT) / a.G);
  const int mt_end = (int)(((long long)(g + 1) * a.nMT) / a.G);
  const int c_begin = mt_begin * 16, c_end = min(mt_end * 16, V);
  const int nchunks = (mt_end - mt_begin + 3) >> 2;

  // epilogue ownership: float4 group j = tid + 256*e -> request row j / 16, columns 4*(j % 16)
  int erow[EPT], ecol[EPT];
  bool ev[EPT];
  float Tv[EPT], invT[EPT];
  uint32_t sk0[EPT], sk1[EPT], pk0[EPT], pk1[EPT];
  long long rbase[EPT], rcache[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int j = tid + 256 * e;
    erow[e] = j / (kCW / 4);
    ecol[e] = (j % (kCW / 4)) * 4;
    const int b = b0 + erow[e];
    const int sl = draft_slot(a, b);  // -1: past the batch or inert at this step
    ev[e] = sl >= 0;
    const int bb = b < a.B ? b : 0;
    const int ss = ev[e] ? sl : 0;
    Tv[e] = a.temp[ss];
    invT[e] = Tv[e] > 0.0f ? 1.0f / Tv[e] : 0.0f;
    const unsigned long long sd = (unsigned long long)a.seeds[ss];
    const unsigned long long pk = (unsigned long long)draft_pos_key(a, bb);
    sk0[e] = (uint32_t)sd;
    sk1[e] = (uint32_t)(sd >> 32);
    pk0[e] = (uint32_t)pk;
    pk1[e] = (uint32_t)(pk >> 32);
    rbase[e] = (long long)bb * a.base_rs + (long long)k * a.base_ss;
    rcache[e] = (long long)(ev[e] ? draft_cache_row(a, b, sl) : 0) * a.cache_rs + (long long)k * a.cache_ss;
  }
  float bv[EPT], qm[EPT], qs[EPT];
  int bi[EPT];
  bool qnan[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    bv[e] = -INFINITY;
    bi[e] = -1;
    qm[e] = -INFINITY;
    qs[e] = 0.0f;
    qnan[e] = false;
  }

  // chunk loaders (w2 rows into registers, base into registers)
  u32x4 wreg[WLMAX];
  float bz[EPT][4], bzn[EPT][4];
  // Rows past V are read from row 0 instead: they only feed bias columns
  // past V (row m of the product depends on w2 row m alone), which the
  // epilogue never uses. No select on the loaded data, so the loads of the
  // next chunk stay in flight while this one is computed.
  auto load_w2 = [&](int c0) {
#pragma unroll
    for (int i = 0; i < WLMAX; ++i) {
      if (i < RK) {
        const int q = tid + 256 * i;  // 16-byte chunk of the 64-row block
        const int row = q / cpr;
        const int v = c0 + row;
        const uint16_t* p = a.w2 + (size_t)(v < V ? v : 0) * r + (q - row * cpr) * 8;
        wreg[i] = *(const u32x4*)p;
      }
    }
  };
  auto store_w2 = [&]() {
#pragma unroll
    for (int i = 0; i < WLMAX; ++i) {
      if (i < RK) {
        const int q = tid + 256 * i;
        const int row = q / cpr, ch = q - row * cpr;
        *(u32x4*)(s_w + row * r + ((ch ^ (row & xmask)) * 8)) = wreg[i];
      }
    }
  };
  auto load_base = [&](int c0, float (&dst)[EPT][4]) {
    if (!a.base_bf16 && a.vec_base && c0 + kCW <= c_end) {
      // whole chunk inside the slab (a block-uniform test): unconditional
      // vector loads (rows past the batch read request 0 and are never used)
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const f32x4 w = *(const f32x4*)((const float*)a.base + rbase[e] + c0 + ecol[e]);
        dst[e][0] = w.x;
        dst[e][1] = w.y;
        dst[e][2] = w.z;
        dst[e][3] = w.w;
      }
      return;
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int c = c0 + ecol[e];
      const int n = c_end - c >= 4 ? 4 : (c_end - c > 0 ? c_end - c : 0);
      if (ev[e] && n > 0) {
        if (a.base_bf16)
          load_row4<true>(a.base, rbase[e] + c, n, a.vec_base, dst[e]);
        else
          load_row4<false>(a.base, rbase[e] + c, n, a.vec_base, dst[e]);
      }
    }
  };

  // the first chunk's loads go out before the previous tokens and the
  // embedding gather, whose latency they then overlap
  if (nchunks > 0) {
    load_w2(c_begin);
    load_base(c_begin, bz);
  }
  // previous token of every request of the tile
  for (int i = tid; i < NB; i += 256) {
    const int b = b0 + i;
    int prev = -1;  // rows that are not served get a zero embedding
    if (draft_slot(a, b) >= 0) {
      long long t = (k == 0) ? (long long)a.anchor[b] : (long long)(int32_t)win_col(a.keys[key_index(k - 1, a.B, b)]);
      if (t < 0 || t >= V) {
        set_status(a.status, kStatusBadAnchor);
        t = 0;
      }
      prev = (int)t;
    }
    s_prev[i] = prev;
  }
  __syncthreads();
  // Markov embeddings w1[prev] -> LDS
  for (int i = tid; i < NB * cpr; i += 256) {
    const int row = i / cpr, ch = i - row * cpr;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (s_prev[row] >= 0) v = *(const u32x4*)(a.w1 + (size_t)s_prev[row] * r + ch * 8);
    *(u32x4*)(s_e + row * rs + ch * 8) = v;
  }

  if (nchunks > 0) store_w2();
  __syncthreads();

  const int lrow = lane & 15, lgrp = lane >> 4;
  for (int ci = 0; ci < nchunks; ++ci) {
    const int c0 = c_begin + ci * kCW;
    const bool more = ci + 1 < nchunks;
    if (more) {
      load_w2(c0 + kCW);
      load_base(c0 + kCW, bzn);
    }
    // projection of this wave's 16 columns for all NB requests
    if (c0 + wave * 16 < c_end) {
      floatx4 acc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      const int arow = wave * 16 + lrow;
#pragma unroll
      for (int s = 0; s < RKMAX; ++s) {
        if (s < RK) {
          const int ch = s * 4 + lgrp;
          const bf16x8 afr = *(const bf16x8*)(s_w + arow * r + ((ch ^ (arow & xmask)) * 8));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const bf16x8 bfr = *(const bf16x8*)(s_e + (nt * 16 + lrow) * rs + s * 32 + lgrp * 8);
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr, acc[nt], 0, 0, 0);
          }
        }
      }
      // lane holds bias of columns wave*16 + 4*lgrp + t for request nt*16 + lrow
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const f32x4 v = {acc[nt][0], acc[nt][1], acc[nt][2], acc[nt][3]};
        *(f32x4*)(s_bias + (nt * 16 + lrow) * BST + wave * 16 + lgrp * 4) = v;
      }
    }
    __syncthreads();
    // epilogue: bias + base -> cache, temperature, Gumbel noise, winner, q statistics
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int c = c0 + ecol[e];
      const int n = c_end - c >= 4 ? 4 : (c_end - c > 0 ? c_end - c : 0);
      if (!ev[e] || n == 0) continue;
      const f32x4 bias = *(const f32x4*)(s_bias + erow[e] * BST + ecol[e]);
      float z[4], cv[4];
      z[0] = bz[e][0] + bias.x;
      z[1] = bz[e][1] + bias.y;
      z[2] = bz[e][2] + bias.z;
      z[3] = bz[e][3] + bias.w;
      if (a.cache_bf16)
        store4<true>(a.cache, rcache[e] + c, n, a.vec_cache, z, cv);
      else
        store4<false>(a.cache, rcache[e] + c, n, a.vec_cache, z, cv);
      if (Tv[e] > 0.0f) {
        const Philox4 w = philox4x32_10((uint32_t)(c >> 2), pk0[e], pk1[e], kSaltDraft, sk0[e], sk1[e]);
        const uint32_t wd[4] = {w.x0, w.x1, w.x2, w.x3};
        float x[4];
        float xm = -INFINITY;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float sv = div_t(z[t], Tv[e], invT[e]) + gumbel_from_word(wd[t]);
          if (t < n) win_update(bv[e], bi[e], sv, c + t);
          const float xv = div_t(cv[t], Tv[e], invT[e]);
          qnan[e] |= (t < n) && (xv != xv);
          x[t] = (t < n && xv == xv) ? xv : -INFINITY;
          xm = fmaxf(xm, x[t]);
        }
        const float mn = fmaxf(qm[e], xm);
        if (mn != -INFINITY) {
          float acc_s = qs[e] * fast_exp(qm[e] - mn);
#pragma unroll
          for (int t = 0; t < 4; ++t) acc_s += fast_exp(x[t] - mn);
          qs[e] = acc_s;
          qm[e] = mn;
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (t < n) win_update(bv[e], bi[e], z[t], c + t);
      }
    }
    if (more) {
      store_w2();
#pragma unroll
      for (int e = 0; e < EPT; ++e)
#pragma unroll
        for (int t = 0; t < 4; ++t) bz[e][t] = bzn[e][t];
    }
    __syncthreads();
  }

  // merge: the 16 threads of one request row are 16 consecutive lanes
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    unsigned long long key = bi[e] >= 0 ? win_key(bv[e], (uint32_t)bi[e]) : 0ull;
    float m = qm[e], s = qnan[e] ? NAN : qs[e];
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const unsigned long long k2 = __shfl_xor(key, off);
      key = k2 > key ? k2 : key;
      const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
      lse_merge(m, s, m2, s2);
    }
    if ((lane & 15) == 0) {
      s_key[erow[e]] = key;
      s_qm[erow[e]] = m;
      s_qs[erow[e]] = s;
    }
  }
  __syncthreads();
  for (int i = tid; i < NB; i += 256) {
    const int b = b0 + i;
    if (draft_slot(a, b) < 0) continue;  // no winner and no partial for rows that are not served
    const unsigned long long key = s_key[i];
    if (key) atomicMax(&a.keys[key_index(k, a.B, b)], key);
    a.qpart[((size_t)k * a.B + b) * a.Gq + g] = make_float2(s_qm[i], s_qs[i]);
  }
}

__global__ __launch_bounds__(256) void draft_init_kernel(unsigned long long* keys, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) keys[(size_t)i * kKeyStride] = 0ull;
}

// Draft tokens from the winner keys, and log-sum-exp of cache / T per row
// from the per-work-group partials; one wave per (request, step).
__global__ __launch_bounds__(256) void draft_finalize_kernel(DraftFinalArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.B * a.K) return;
  const int b = row / a.K, k = row - b * a.K;
  // inert rows keep key 0, i.e. token -1; the key is left cleared for the
  // next call on this workspace
  if (lane == 0) {
    unsigned long long* kp = a.keys + key_index(k, a.B, b);
    a.tokens[row] = key_col(*kp, a.fp64 != 0);
    *kp = 0ull;
  }
  if (!a.lse) return;
  const int sl = draft_slot(a.idx_map, a.row_map, a.B, a.K, a.n_slots, a.n_rows, nullptr, b, k);
  if (sl < 0) {
    if (lane == 0) a.lse[row] = NAN;
    return;
  }
  const float T = a.temp[sl];  // in flight with the partials
  float m = -INFINITY, s = 0.0f;
  const float2* qp = a.qpart + ((size_t)k * a.B + b) * a.Gq;
  const int n = k == 0 ? a.G0 : a.G;
  // four partials a lane in flight at a time (an empty one merges as a no-op)
  for (int i0 = lane; i0 < n; i0 += 256) {
    float2 p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] = i0 + 64 * u < n ? qp[i0 + 64 * u] : make_float2(-INFINITY, 0.0f);
#pragma unroll
    for (int u = 0; u < 4; ++u) lse_merge(m, s, p[u].x, p[u].y);
  }
  wave_lse_merge_dpp(m, s);
  if (lane == 0) {
    float out;
    if (!(T > 0.0f) || s != s)
      out = NAN;
    else
      out = m + __logf(s);
    a.lse[row] = out;
  }
}

template <int NB, int RKT>
hipError_t launch_step(const DraftStepArgs& a, int bt, hipStream_t st) {
  const size_t lds = draft_step_lds(NB, a.r);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute((const void*)draft_step_kernel<NB, RKT>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
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
