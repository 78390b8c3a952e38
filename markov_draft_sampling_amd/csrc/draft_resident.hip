// Persistent Markov draft loop with w2 resident on chip (gfx950).
//
// The sequential loop of the DSparkSpeculator API page (_sample_markov_chain)
// reads the whole Markov projection w2 [V, r] once per step (PR #65007,
// Part 1: the loop is memory bound on exactly that). On MI355X the register
// files (256 CUs x 512 KiB) and LDS (256 x 160 KiB) of the chip together
// exceed w2 (102 MB at V = 200064, r = 256), so one launch runs all K steps:
//   * one work-group per CU owns a contiguous slab of 16-column tiles; at
//     start it loads its slab of w2 once: the first 4*RMT tiles into
//     registers (each wave keeps RMT tiles as MFMA A operands, 256 registers
//     per lane), the rest into LDS (coalesced loads, rows XOR-swizzled by
//     16-byte chunk so the operand reads are bank-conflict free);
//   * every step then streams only the base logits and the cache: for each
//     32-request tile, embeddings w1[prev] go to LDS, each wave projects its
//     tiles with v_mfma_f32_16x16x32_bf16 and runs the epilogue from the
//     accumulator layout (bias + base -> cache, temperature, Philox Gumbel,
//     running winner, q statistics) with the next tile's base rows in flight;
//   * per-request winners merge by a 64-bit atomic max; between steps all
//     work-groups meet at a grid barrier (arrival counter per step) whose
//     wait is bounded: on a timeout the kernel sets a sticky status bit and an
//     abort flag that makes every work-group return.
// All work-groups must be resident at once: the launch uses one work-group per
// CU and enough LDS that no second one fits on a CU.
#include "mds_device.h"
#include "mds_internal.h"

namespace mds {

namespace {

constexpr int kNB = 32;        // requests per batch tile
constexpr int kThreads = 256;  // 4 waves, one per SIMD
constexpr unsigned kSpinLimit = 1u << 21;
constexpr int kDepth = 4;      // base-row tiles in flight per wave (register ring)

__device__ __forceinline__ size_t fixed_lds(int r) {
  return (size_t)kNB * (r + 8) * 2 + kNB * 4 + 4 * kNB * 8 + 8 * kNB * 4 + 64;
}

// Wait until `target` work-groups have arrived at `counter`. Returns false
// when the wait was abandoned (timeout here or elsewhere). The only data the
// next step reads across work-groups are the winner keys, written by
// device-scope atomics that have returned (so are performed) before this
// barrier and read back with device-scope atomic loads; no cache maintenance
// is needed (a release fence here would write back the L2, full of cache rows).
__device__ bool grid_barrier(unsigned* counter, unsigned target, unsigned* abort_flag, uint32_t* status,
                             int* s_flag) {
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(counter, 1u);
    int ok = 1;
    unsigned spins = 0;
    // poll with relaxed device-scope loads (served past the non-coherent L2,
    // no cache maintenance per poll), then one acquire fence after the wait
    while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        ok = 0;
        break;
      }
      if (++spins > kSpinLimit) {
        set_status(status, kStatusBarrierTimeout);
        atomicExch(abort_flag, 1u);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    *s_flag = ok;
  }
  __syncthreads();
  return *s_flag != 0;
}

template <bool BF16>
__device__ __forceinline__ void load_col4(const void* p, long long off, int n, bool vec, float (&v)[4]) {
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

template <bool BF16>
__device__ __forceinline__ void store_col4(void* p, long long off, int n, bool vec, const float (&z)[4],
                                           float (&stored)[4]) {
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

// RK = r / 32 (MFMA k-steps per tile), RMT = register-resident tiles per wave
// (a multiple of kDepth, so the base-row ring index stays static across the
// register tiles and the LDS tiles that follow them).
template <int RK, int RMT, bool BBF16, bool CBF16>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void draft_resident_kernel(
    DraftStepArgs a) {
  static_assert(RMT % kDepth == 0, "register tiles per wave must be a multiple of the ring depth");
  static_assert(kNB == 32, "the projection is written for two 16-request MFMA tiles");
  constexpr int NT = kNB / 16;
  constexpr int R = RK * 32;
  constexpr int CPR = R / 8;  // 16-byte chunks per w2 row
  constexpr int XMASK = (CPR & 7) ? 3 : 7;
  constexpr int RS = R + 8;   // embedding row stride (bf16)
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* s_e = (uint16_t*)smem;                                   // [32][RS]
  int* s_prev = (int*)(s_e + kNB * RS);                              // [32]
  unsigned long long* s_key = (unsigned long long*)(s_prev + kNB);   // [4][32]
  float* s_qm = (float*)(s_key + 4 * kNB);                           // [4][32]
  float* s_qs = s_qm + 4 * kNB;                                      // [4][32]
  int* s_flag = (int*)(s_qs + 4 * kNB);
  uint16_t* s_w = (uint16_t*)(smem + fixed_lds(R));                  // [n_lds][16][R] swizzled

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int g = blockIdx.x, G = a.G, V = a.V, B = a.B;
  const int mt_begin = (int)(((long long)g * a.nMT) / G);
  const int mt_end = (int)(((long long)(g + 1) * a.nMT) / G);
  const int n_my = mt_end - mt_begin;
  const int n_reg = n_my < 4 * RMT ? n_my : 4 * RMT;  // tiles held in registers by the 4 waves
  const int n_lds = n_my - n_reg;                      // tiles held in LDS (<= a.n_lds_tiles)

  // ---- load this work-group's slab of w2 once ----
  bf16x8 wr[RMT][RK];
#pragma unroll
  for (int j = 0; j < RMT; ++j) {
    const int t = wave + 4 * j;
    const int v = (mt_begin + t) * 16 + lrow;
    const bool ok = t < n_reg && v < V;
    const uint16_t* p = a.w2 + (size_t)(ok ? v : 0) * R + lgrp * 8;
#pragma unroll
    for (int s = 0; s < RK; ++s) {
      bf16x8 x = *(const bf16x8*)(p + s * 32);
      if (!ok) x = bf16x8{};
      wr[j][s] = x;
    }
  }
  for (int q = tid; q < n_lds * 16 * CPR; q += kThreads) {
    const int tile = q / (16 * CPR);
    const int rem = q - tile * 16 * CPR;
    const int row = rem / CPR, ch = rem - row * CPR;
    const int v = (mt_begin + n_reg + tile) * 16 + row;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (v < V) x = *(const u32x4*)(a.w2 + (size_t)v * R + ch * 8);
    *(u32x4*)(s_w + (tile * 16 + row) * R + ((ch ^ (row & XMASK)) * 8)) = x;
  }

  // tiles of this wave: register tiles j < R_w, then LDS tiles wave, wave+4, ...
  // (LDS tiles exist only when every wave holds RMT register tiles)
  int R_w = 0;
#pragma unroll
  for (int j = 0; j < RMT; ++j) R_w += (wave + 4 * j < n_reg) ? 1 : 0;
  const int L_w = n_lds > wave ? (n_lds - wave + 3) / 4 : 0;
  const int T_w = R_w + L_w;
  const int last = T_w > 0 ? T_w - 1 : 0;

  const int BT = (B + kNB - 1) / kNB;
  for (int k = 0; k < a.K; ++k) {
    if (k > 0 && !grid_barrier(a.bar + (k - 1), (unsigned)G, a.abort_flag, a.status, s_flag)) return;
    for (int bt = 0; bt < BT; ++bt) {
      const int b0 = bt * kNB;
      __syncthreads();  // the previous tile's LDS reads are done
      if (tid < kNB) {
        const int b = b0 + tid;
        int prev = 0;
        if (b < B) {
          long long t;
          if (k == 0) {
            t = a.anchor[b];
          } else {
            const unsigned long long key =
                __hip_atomic_load(&a.keys[key_index(k - 1, B, b)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            t = (long long)win_col(key);
          }
          if (t < 0 || t >= V) {
            set_status(a.status, kStatusBadAnchor);
            t = 0;
          }
          prev = (int)t;
        }
        s_prev[tid] = prev;
      }
      __syncthreads();
      for (int i = tid; i < kNB * CPR; i += kThreads) {
        const int row = i / CPR, ch = i - row * CPR;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (b0 + row < B) v = *(const u32x4*)(a.w1 + (size_t)s_prev[row] * R + ch * 8);
        *(u32x4*)(s_e + row * RS + ch * 8) = v;
      }
      __syncthreads();
      // embedding operands (16 requests x 32 ranks per MFMA) are read from
      // LDS at every tile, all of a tile's reads ahead of its MFMAs; the
      // runtime-zero offset keeps the compiler from hoisting them into 64
      // more registers next to the resident w2
      const uint16_t* ebase = s_e + lrow * RS + lgrp * 8;

      // per-lane request parameters (rows nt*16 + lrow of the tile)
      bool rv[NT];
      float Tv[NT], invT[NT], bv[NT], qm[NT], qs[NT];
      int bi[NT];
      bool qnan[NT];
      uint32_t sk0[NT], sk1[NT], pk0[NT], pk1[NT];
      long long rbase[NT], rcache[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int b = b0 + nt * 16 + lrow;
        rv[nt] = b < B;
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
        bv[nt] = -INFINITY;
        bi[nt] = -1;
        qm[nt] = -INFINITY;
        qs[nt] = 0.0f;
        qnan[nt] = false;
      }
      bool all_fast = a.vec_base && a.vec_cache, all_t1 = true;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        all_fast &= rv[nt] && Tv[nt] > 0.0f;
        all_t1 &= Tv[nt] == 1.0f;
      }
      const bool fast_req = __all(all_fast);
      const bool t1 = __all(all_t1);

      auto tile_col = [&](int t) -> int {  // first column of this wave's t-th tile
        return t < R_w ? (mt_begin + wave + 4 * t) * 16 : (mt_begin + n_reg + wave + 4 * (t - R_w)) * 16;
      };
      // base rows of this wave's tiles: a ring of kDepth tiles, kDepth - 1
      // ahead; the last tiles are requested again at the end (cache hits),
      // so every load is unconditional and in order
      auto load_base = [&](int t, float (&dst)[NT][4]) {
        const int c = tile_col(t) + lgrp * 4;
        if (fast_req && c + 4 <= V) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) load_col4<BBF16>(a.base, rbase[nt] + c, 4, true, dst[nt]);
        } else {
          const int n = V - c >= 4 ? 4 : (V - c > 0 ? V - c : 0);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[nt][i] = 0.0f;
            if (rv[nt] && n > 0) load_col4<BBF16>(a.base, rbase[nt] + c, n, a.vec_base, dst[nt]);
          }
        }
      };
      // epilogue of one tile from the accumulator layout: lane holds columns
      // c .. c+3 of request 16 nt + lrow
      auto epilogue = [&](int t, const floatx4 (&acc)[NT], const float (&bz)[NT][4]) {
        const int c = tile_col(t) + lgrp * 4;
        if (fast_req && tile_col(t) + 16 <= V) {
          // straight-line form: every request of the tile exists and samples,
          // full tile, vector stores; a NaN among the q values rides the sum
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            float z[4], cv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) z[i] = bz[nt][i] + acc[nt][i];
            store_col4<CBF16>(a.cache, rcache[nt] + c, 4, true, z, cv);
            const Philox4 w = philox4x32_10((uint32_t)(c >> 2), pk0[nt], pk1[nt], kSaltDraft, sk0[nt], sk1[nt]);
            const uint32_t wd[4] = {w.x0, w.x1, w.x2, w.x3};
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float y = t1 ? z[i] : div_t(z[i], Tv[nt], invT[nt]);
              x[i] = CBF16 ? (t1 ? cv[i] : div_t(cv[i], Tv[nt], invT[nt])) : y;
              const float sv = y + gumbel_from_word(wd[i]);
              const bool take = (sv > bv[nt]) || ((sv != sv) && (bv[nt] == bv[nt])) || (bi[nt] < 0);
              bv[nt] = take ? sv : bv[nt];
              bi[nt] = take ? c + i : bi[nt];
            }
            const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));  // NaN-ignoring max
            const float mn = fmaxf(qm[nt], mx);
            const float sub = mn == -INFINITY ? 0.0f : mn;
            float s_acc = qs[nt] * fast_exp(qm[nt] - sub);
#pragma unroll
            for (int i = 0; i < 4; ++i) s_acc += fast_exp(x[i] - sub);
            qs[nt] = s_acc;
            qm[nt] = mn;
          }
          return;
        }
        const int n = V - c >= 4 ? 4 : (V - c > 0 ? V - c : 0);
        if (n == 0) return;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (!rv[nt]) continue;
          float z[4], cv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) z[i] = bz[nt][i] + acc[nt][i];
          store_col4<CBF16>(a.cache, rcache[nt] + c, n, a.vec_cache, z, cv);
          if (Tv[nt] > 0.0f) {
            const Philox4 w = philox4x32_10((uint32_t)(c >> 2), pk0[nt], pk1[nt], kSaltDraft, sk0[nt], sk1[nt]);
            const uint32_t wd[4] = {w.x0, w.x1, w.x2, w.x3};
            float x[4];
            float xm = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float sv = div_t(z[i], Tv[nt], invT[nt]) + gumbel_from_word(wd[i]);
              if (i < n) win_update(bv[nt], bi[nt], sv, c + i);
              const float xv = div_t(cv[i], Tv[nt], invT[nt]);
              qnan[nt] |= (i < n) && (xv != xv);
              x[i] = (i < n && xv == xv) ? xv : -INFINITY;
              xm = fmaxf(xm, x[i]);
            }
            const float mn = fmaxf(qm[nt], xm);
            if (mn != -INFINITY) {
              float acc_s = qs[nt] * fast_exp(qm[nt] - mn);
#pragma unroll
              for (int i = 0; i < 4; ++i) acc_s += fast_exp(x[i] - mn);
              qs[nt] = acc_s;
              qm[nt] = mn;
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (i < n) win_update(bv[nt], bi[nt], z[i], c + i);
          }
        }
      };

      auto bfrag = [&](int sidx, int nt, int t) -> bf16x8 {
        return *(const bf16x8*)(ebase + nt * 16 * RS + sidx * 32 + a.zero * t);
      };
      auto project = [&](int t, floatx4 (&acc)[NT]) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        if (t < R_w) {
          // register-resident tile t: every case names its tile statically so
          // wr[][] stays in registers
          switch (t) {
#define MDS_REG_TILE(J)                                                                                  \
  case J:                                                                                                \
    if constexpr (J < RMT) {                                                                             \
      bf16x8 e0 = bfrag(0, 0, t), e1 = bfrag(0, 1, t);                                                   \
      _Pragma("unroll") for (int sidx = 0; sidx < RK; ++sidx) {                                          \
        bf16x8 n0 = e0, n1 = e1;                                                                         \
        if (sidx + 1 < RK) {                                                                             \
          n0 = bfrag(sidx + 1, 0, t);                                                                    \
          n1 = bfrag(sidx + 1, 1, t);                                                                    \
        }                                                                                                \
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wr[J][sidx], e0, acc[0], 0, 0, 0);              \
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wr[J][sidx], e1, acc[1], 0, 0, 0);              \
        e0 = n0;                                                                                         \
        e1 = n1;                                                                                         \
      }                                                                                                  \
      /* one slice of embedding reads ahead of the MFMAs that use them */                                \
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                                                 \
      _Pragma("unroll") for (int sidx = 0; sidx + 1 < RK; ++sidx) {                                      \
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                                               \
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                               \
      }                                                                                                  \
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                                 \
    }                                                                                                    \
    break;
            MDS_REG_TILE(0) MDS_REG_TILE(1) MDS_REG_TILE(2) MDS_REG_TILE(3) MDS_REG_TILE(4) MDS_REG_TILE(5)
            MDS_REG_TILE(6) MDS_REG_TILE(7) MDS_REG_TILE(8) MDS_REG_TILE(9) MDS_REG_TILE(10) MDS_REG_TILE(11)
            MDS_REG_TILE(12) MDS_REG_TILE(13) MDS_REG_TILE(14) MDS_REG_TILE(15) MDS_REG_TILE(16) MDS_REG_TILE(17)
            MDS_REG_TILE(18) MDS_REG_TILE(19) MDS_REG_TILE(20) MDS_REG_TILE(21) MDS_REG_TILE(22) MDS_REG_TILE(23)
            MDS_REG_TILE(24) MDS_REG_TILE(25) MDS_REG_TILE(26) MDS_REG_TILE(27) MDS_REG_TILE(28) MDS_REG_TILE(29)
            MDS_REG_TILE(30) MDS_REG_TILE(31)
#undef MDS_REG_TILE
            default: break;
          }
        } else {
          const int L = wave + 4 * (t - R_w);
          const uint16_t* wrow = s_w + (L * 16 + lrow) * R;
          bf16x8 f = *(const bf16x8*)(wrow + ((lgrp ^ (lrow & XMASK)) * 8));
          bf16x8 e0 = bfrag(0, 0, t), e1 = bfrag(0, 1, t);
#pragma unroll
          for (int sidx = 0; sidx < RK; ++sidx) {
            bf16x8 nf = f, n0 = e0, n1 = e1;
            if (sidx + 1 < RK) {
              const int ch = (sidx + 1) * 4 + lgrp;
              nf = *(const bf16x8*)(wrow + ((ch ^ (lrow & XMASK)) * 8));
              n0 = bfrag(sidx + 1, 0, t);
              n1 = bfrag(sidx + 1, 1, t);
            }
            acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f, e0, acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f, e1, acc[1], 0, 0, 0);
            f = nf;
            e0 = n0;
            e1 = n1;
          }
          // one slice of w2 and embedding reads ahead of the MFMAs that use them
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
          for (int sidx = 0; sidx + 1 < RK; ++sidx) {
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
      };

      float ring[kDepth][NT][4];
#pragma unroll
      for (int u = 0; u < kDepth - 1; ++u) load_base(min(u, last), ring[u]);
      for (int t0 = 0; t0 < T_w; t0 += kDepth) {
#pragma unroll
        for (int u = 0; u < kDepth; ++u) {
          const int t = t0 + u;
          if (t < T_w) {
            load_base(min(t + kDepth - 1, last), ring[(u + kDepth - 1) % kDepth]);
            floatx4 acc[NT];
            project(t, acc);
            epilogue(t, acc, ring[u]);
          }
        }
      }

      // merge the four lanes of each request, then the four waves, then publish
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        uint64_t key = bi[nt] >= 0 ? win_key(bv[nt], (uint32_t)bi[nt]) : 0ull;
        key = max_over_groups16(key);
        float m = qm[nt], s = qnan[nt] ? NAN : qs[nt];
        float m2 = __shfl_xor(m, 16), s2 = __shfl_xor(s, 16);
        lse_merge(m, s, m2, s2);
        m2 = __shfl_xor(m, 32);
        s2 = __shfl_xor(s, 32);
        lse_merge(m, s, m2, s2);
        if (lgrp == 0) {
          s_key[wave * kNB + nt * 16 + lrow] = key;
          s_qm[wave * kNB + nt * 16 + lrow] = m;
          s_qs[wave * kNB + nt * 16 + lrow] = s;
        }
      }
      __syncthreads();
      if (tid < kNB) {
        const int b = b0 + tid;
        if (b < B) {
          unsigned long long key = s_key[tid];
          float m = s_qm[tid], s = s_qs[tid];
#pragma unroll
          for (int w = 1; w < 4; ++w) {
            const unsigned long long k2 = s_key[w * kNB + tid];
            key = k2 > key ? k2 : key;
            lse_merge(m, s, s_qm[w * kNB + tid], s_qs[w * kNB + tid]);
          }
          // the returned value makes the wave wait until the atomic is performed
          const unsigned long long prev = key ? atomicMax(&a.keys[key_index(k, B, b)], key) : 0ull;
          s_flag[1] = (int)(prev >> 63);
          a.qpart[((size_t)k * B + b) * G + g] = make_float2(m, s);
        }
      }
    }
  }
}

template <int RK, int RMT, bool BBF16, bool CBF16>
hipError_t launch_res_t(const DraftStepArgs& a, size_t lds, hipStream_t st) {
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute((const void*)draft_resident_kernel<RK, RMT, BBF16, CBF16>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((draft_resident_kernel<RK, RMT, BBF16, CBF16>), dim3(a.G), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <int RK, int RMT>
hipError_t launch_res(const DraftStepArgs& a, size_t lds, hipStream_t st) {
  if (a.base_bf16)
    return a.cache_bf16 ? launch_res_t<RK, RMT, true, true>(a, lds, st) : launch_res_t<RK, RMT, true, false>(a, lds, st);
  return a.cache_bf16 ? launch_res_t<RK, RMT, false, true>(a, lds, st) : launch_res_t<RK, RMT, false, false>(a, lds, st);
}

// register tiles per wave for rank r: about 256 registers of w2 per lane
// (RMT tiles x RK k-steps x 4), RMT a multiple of the ring depth
int res_rmt(int r) {
  const int rmt = 64 / (r / 32);
  return rmt - rmt % kDepth;
}

}  // namespace

hipError_t draft_resident_plan(int V, int r, int G, size_t lds_limit, int* n_lds_tiles, size_t* lds_bytes) {
  if (r != 64 && r != 128 && r != 192 && r != 256) return hipErrorNotSupported;
  if (G < 1) return hipErrorNotSupported;
  const int nMT = (V + 15) / 16;
  const int per_wg = (nMT + G - 1) / G;
  const int n_lds = per_wg - 4 * res_rmt(r);
  const size_t fixed = (size_t)kNB * (r + 8) * 2 + kNB * 4 + 4 * kNB * 8 + 8 * kNB * 4 + 64;
  const size_t tile = (size_t)16 * r * 2;
  const size_t need = fixed + (size_t)(n_lds > 0 ? n_lds : 0) * tile;
  if (need > lds_limit) return hipErrorNotSupported;
  // one work-group per CU: ask for more than half of the CU's LDS
  const size_t lds = need > lds_limit / 2 + 1 ? need : lds_limit / 2 + 1024;
  *n_lds_tiles = n_lds > 0 ? n_lds : 0;
  *lds_bytes = lds;
  return hipSuccess;
}

hipError_t launch_draft_resident(const DraftStepArgs& a, size_t lds, hipStream_t st) {
  switch (a.r) {
    case 64: return launch_res<2, 32>(a, lds, st);
    case 128: return launch_res<4, 16>(a, lds, st);
    case 192: return launch_res<6, 8>(a, lds, st);
    case 256: return launch_res<8, 8>(a, lds, st);
    default: return hipErrorNotSupported;
  }
}

}  // namespace mds
