// Draft LM head (DSparkSpeculator API page, _sample_sequential and
// _sample_sequential_topk: compute_draft_logits turns the gathered hidden
// state of every (request, step) row into that row's base draft logits before
// the Markov loop).
//
// logits[m, v] = sum_h hidden[m, h] * lm_head[v, h]: bf16 inputs, float32
// accumulation on the matrix cores (v_mfma_f32_16x16x32_bf16), row m = b*K + k
// written to the base-logit layout the draft loop reads.
//
// With B*K rows in the low hundreds the product is bound by memory traffic:
// the lm_head stream (V*H*2 bytes, 1.64 GB at V = 200064, H = 4096, read once)
// plus every work-group's re-read of its M tile's hidden rows (from L2). Each
// work-group therefore owns as many vocabulary rows as its accumulators allow
// (256 for up to 224 rows of M, in eight waves of 32 rows: 112 float
// accumulators a lane, two waves per SIMD), one work-group per CU. H is
// walked in chunks of 128 columns:
//  - hidden rows: copied straight into LDS (buffer loads with the LDS flag, no
//    registers; instruction q of wave w fills 4 rows, 4 NW q + 4 w ..),
//    double buffered, 16-byte slots XOR-swizzled by row so the fragment reads
//    of 16 consecutive rows hit distinct banks;
//  - lm_head rows: each wave reads its own rows row-contiguously (whole 128-byte
//    lines; a direct load in MFMA operand layout touches 16 rows per
//    instruction and streams markedly slower), two chunks deep in registers,
//    and stages each half chunk through a private LDS area into operand layout;
//  - copies go out a few per slice of 32 columns and one barrier ends a chunk;
//  - work-groups start at different chunks, so that they do not all read the
//    same columns of the hidden rows (the same memory channels) at once.
#include "mds_device.h"
#include "mds_internal.h"

namespace mds {
namespace {

constexpr int kKC = 128;  // H columns per chunk (4 slices of 32, 256 bytes a row)
constexpr int kStagger = 7;  // chunk offset between consecutive work-groups

// Work-group barrier once this wave's hidden-chunk copies have landed in LDS:
// s_waitcnt vmcnt(N) lgkmcnt(0) (at most N newer loads, lm_head rows in
// flight, stay outstanding; every LDS access of the wave has completed), then
// s_barrier. No release fence: that would wait for every load in flight.
template <int N>
__device__ __forceinline__ void chunk_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Fused form: step 0 of the Markov draft loop on the work-group's vocabulary
// rows (the DSparkSpeculator API page, _sample_sequential: the first step
// consumes compute_draft_logits' first row), run on the LM head's own logits
// instead of a stored base row. Requests b < B <= 32 are served by lanes
// lr (b = 16 nt + lr), as in the loop's step kernel: the anchors' w1 rows and
// the wave's w2 rows give the Markov bias by MFMA (the same slices in the same
// order as the step kernel), st0 holds the wave's logits of the requests'
// step-0 rows ([32 requests][16 NBW columns], in the base dtype's precision),
// then the step epilogue: cache row 0, the draft noise, the running winner
// and the q statistics, merged over the lanes, then over the waves in LDS
// (xs: 16 NW * 32 bytes), into one atomic max and one q partial (slot gidx)
// per request.
constexpr int kS0RK = 8;  // rank slices of 32 of the fused step 0 (r <= 256)

// The fused step's loads, all independent of each other: the per-request
// parameters, the anchors' w1 rows (the tokens were read at the kernel's
// start) and the wave's w2 rows.
template <int NBW>
struct Step0In {
  float T[2];
  unsigned long long sd[2], pk[2];
  bf16x8 Er[2][kS0RK];
  u32x4 A[NBW][kS0RK];
};

__device__ __forceinline__ int step0_token(const DraftStepArgs& d, int nt) {
  const int b = nt * 16 + (threadIdx.x & 15);
  return d.anchor[b < d.B ? b : d.B - 1];
}

template <int NBW>
__device__ __forceinline__ void step0_load(const DraftStepArgs& d, int vw, const int (&tk)[2], Step0In<NBW>& in) {
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int V = d.V, r = d.r, RK = r >> 5;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int b = nt * 16 + lr;
    const int bb = b < d.B ? b : d.B - 1;
    in.T[nt] = d.temp[bb];
    in.sd[nt] = (unsigned long long)d.seeds[bb];
    in.pk[nt] = (unsigned long long)draft_pos_key(d, bb);
    const int t = tk[nt] < 0 || tk[nt] >= V ? 0 : tk[nt];
#pragma unroll
    for (int s = 0; s < kS0RK; ++s)
      in.Er[nt][s] = *(const bf16x8*)(d.w1 + (size_t)t * r + (s < RK ? s : 0) * 32 + lg * 8);
  }
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int v = vw + nb * 16 + lr;
    const uint16_t* p = d.w2 + (size_t)(v < V ? v : V - 1) * r + lg * 8;
#pragma unroll
    for (int s = 0; s < kS0RK; ++s) in.A[nb][s] = *(const u32x4*)(p + (s < RK ? s : RK - 1) * 32);
  }
}

template <int NBW, int NW, bool CBF16>
__device__ void fused_step0(const DraftStepArgs& d, int vw, int gidx, const float* st0, unsigned char* xs, int m0,
                            int mt, const int (&tk)[2], const Step0In<NBW>& in) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int V = d.V, RK = d.r >> 5;
  bool valid[2];
  float Tv[2], invT[2];
  uint32_t sk0[2], sk1[2], pk0[2], pk1[2];
  long long rc[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int b = nt * 16 + lr;
    // served here: the request's step-0 row lies in this work-group's M tile
    valid[nt] = b < d.B && b * d.K >= m0 && b * d.K < m0 + mt;
    const int bb = b < d.B ? b : d.B - 1;
    Tv[nt] = in.T[nt];
    invT[nt] = Tv[nt] > 0.0f ? 1.0f / Tv[nt] : 0.0f;
    sk0[nt] = (uint32_t)in.sd[nt];
    sk1[nt] = (uint32_t)(in.sd[nt] >> 32);
    pk0[nt] = (uint32_t)in.pk[nt];
    pk1[nt] = (uint32_t)(in.pk[nt] >> 32);
    rc[nt] = (long long)bb * d.cache_rs;
    if ((tk[nt] < 0 || tk[nt] >= V) && valid[nt]) set_status(d.status, kStatusBadAnchor);
  }
  // Markov bias: D[column 4 lg + i of block nb][request 16 nt + lr]
  floatx4 bias[NBW][2];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) bias[nb][nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < kS0RK; ++s)
      if (s < RK)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          bias[nb][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, in.A[nb][s]), in.Er[nt][s],
                                                                 bias[nb][nt], 0, 0, 0);
  }
  unsigned long long* s_key = (unsigned long long*)xs;  // [NW][32]
  float* s_qm = (float*)(s_key + NW * 32);              // [NW][32]
  float* s_qs = s_qm + NW * 32;                         // [NW][32]
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int b = nt * 16 + lr;
    // the lane's columns in increasing order; the winner starts at the first (value -inf)
    const int c_first = vw + lg * 4;
    float bv = -INFINITY, qm = -INFINITY, qs = 0.0f;
    int bi = c_first < V ? c_first : -1;
    bool qnan = false;
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int c = vw + nb * 16 + lg * 4;
      const int n = V - c >= 4 ? 4 : (V - c > 0 ? V - c : 0);
      const f32x4 bz = *(const f32x4*)(st0 + b * (16 * NBW) + nb * 16 + lg * 4);
      float z[4] = {bz.x + bias[nb][nt][0], bz.y + bias[nb][nt][1], bz.z + bias[nb][nt][2], bz.w + bias[nb][nt][3]};
      if (!valid[nt] || n == 0) continue;
      float cv[4];
      if (CBF16) {
        uint32_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[i] = f32_to_bf16_bits(z[i]);
          cv[i] = bf16_bits_to_f32(h[i]);
        }
        uint16_t* q = (uint16_t*)d.cache + rc[nt] + c;
        if (d.vec_cache && n == 4) {
          *(u32x2*)q = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i < n) q[i] = (uint16_t)h[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) cv[i] = z[i];
        float* q = (float*)d.cache + rc[nt] + c;
        if (d.vec_cache && n == 4) {
          *(f32x4*)q = f32x4{z[0], z[1], z[2], z[3]};
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i < n) q[i] = z[i];
        }
      }
      if (Tv[nt] > 0.0f) {
        const Philox4 wv = philox4x32_10((uint32_t)(c >> 2), pk0[nt], pk1[nt], kSaltDraft, sk0[nt], sk1[nt]);
        const uint32_t wd[4] = {wv.x0, wv.x1, wv.x2, wv.x3};
        float x[4];
        float xm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sv = div_t(z[i], Tv[nt], invT[nt]) + gumbel_from_word(wd[i]);
          if (i < n) win_update(bv, bi, sv, c + i);
          const float xv = div_t(cv[i], Tv[nt], invT[nt]);
          qnan |= (i < n) && (xv != xv);
          x[i] = (i < n && xv == xv) ? xv : -INFINITY;
          xm = fmaxf(xm, x[i]);
        }
        const float mn = fmaxf(qm, xm);
        if (mn != -INFINITY) {
          float s_acc = qs * fast_exp(qm - mn);
#pragma unroll
          for (int i = 0; i < 4; ++i) s_acc += fast_exp(x[i] - mn);
          qs = s_acc;
          qm = mn;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < n) win_update(bv, bi, z[i], c + i);
      }
    }
    // the 4 lanes of the request row, then the waves
    unsigned long long key = bi >= 0 ? win_key_of(bv, (uint32_t)bi) : 0ull;
    float m = qm, sq = qnan ? NAN : qs;
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
      const unsigned long long k2 = __shfl_xor(key, off);
      key = k2 > key ? k2 : key;
      const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(sq, off);
      lse_merge(m, sq, m2, s2);
    }
    if (lg == 0) {
      s_key[w * 32 + b] = key;
      s_qm[w * 32 + b] = m;
      s_qs[w * 32 + b] = sq;
    }
  }
  __syncthreads();
  if (tid < 32 && tid < d.B && tid * d.K >= m0 && tid * d.K < m0 + mt) {
    const int b = tid;
    unsigned long long key = s_key[b];
    float m = s_qm[b], sq = s_qs[b];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
      const unsigned long long k2 = s_key[i * 32 + b];
      key = k2 > key ? k2 : key;
      lse_merge(m, sq, s_qm[i * 32 + b], s_qs[i * 32 + b]);
    }
    if (key) atomicMax(&d.keys[key_index(0, d.B, b)], key);
    d.qpart[(size_t)b * d.Gq + gidx] = make_float2(m, sq);
  }
}

// MB: 16-row blocks of the M tile; NBW: 16-row vocabulary blocks per wave; NW:
// waves (the work-group covers 16 NBW NW rows from vocabulary row v0 on); S0:
// 0, or the fused step 0 with a float32 (1) or bf16 (2) cache
template <int MB, int NBW, int NW, bool OBF16, int S0>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void lm_head_kernel(
    LmHeadArgs a, int v0, DraftStepArgs d, int gbase) {
  constexpr int kNBW = NBW;
  constexpr int kVT = NW * kNBW * 16;
  constexpr int MT = MB * 16;
  // hidden chunks, double buffered; 16-byte slot j of row R holds the row's slot j ^ (R & 15)
  __shared__ __attribute__((aligned(16))) uint16_t s_h0[MT * kKC];
  __shared__ __attribute__((aligned(16))) uint16_t s_h1[MT * kKC];
  // each wave's lm_head rows for half a chunk (64 columns), staged from the row-contiguous loads
  // into the MFMA operand layout; 16-byte slot t of row R sits at slot t ^ ((R / 2) % 8)
  __shared__ __attribute__((aligned(16))) uint16_t s_a[NW][16 * kNBW * 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int m0 = blockIdx.y * MT;
  const int vw = v0 + blockIdx.x * kVT + w * kNBW * 16;  // first vocabulary row of this wave
  int tk0[2] = {0, 0};  // fused step 0: the anchors of requests lr and 16 + lr, read at once
  if constexpr (S0 != 0) {
    tk0[0] = step0_token(d, 0);
    tk0[1] = step0_token(d, 1);
  }
  const int S = a.H >> 5;                          // 32-wide slices of H (a multiple of 2 * 4)
  const int NC = S / 4;                            // chunks of four slices
  // this work-group's chunk order: coff, coff + 1, ... (mod NC)
  const int coff = (int)((blockIdx.x * (unsigned)kStagger) % (unsigned)NC);

  // hidden chunk c into LDS: wave w's instruction p fills rows R = 4 NW p + 4 w .. + 3 (1 KB), lane
  // l landing in row R + l / 16, slot l % 16, so it fetches that row's slot (l % 16) ^ ((4 w + l / 16) % 16).
  // Buffer loads from the tile's first row: per-lane byte offsets (rows past M repeat row M - 1),
  // the chunk's column offset as the scalar offset.
  const int Mt = min(MT, a.M - m0);
  const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.hidden + (size_t)m0 * a.hidden_rs), (short)0, (int)((size_t)Mt * a.hidden_rs * 2),
      0x00020000);  // descriptor word 3: raw byte-addressed access (32-bit data format)
  constexpr int kQ = (MT + 4 * NW - 1) / (4 * NW);  // copy instructions per wave and chunk
  const int R0 = w * 4 + (lane >> 4);
  const int gsl = ((lane & 15) ^ (R0 & 15)) * 16;
  auto dma_one = [&](uint16_t* buf, int c, int p) {
    if (MT % (4 * NW) != 0 && p * 4 * NW + w * 4 >= MT) return;
    const int voff = min(p * 4 * NW + R0, Mt - 1) * a.hidden_rs * 2 + gsl;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(hrs, (__attribute__((address_space(3))) void*)(buf + (p * 4 * NW + w * 4) * kKC),
                                             16, voff, (c + coff >= NC ? c + coff - NC : c + coff) * kKC * 2, 0, 0);
  };
  auto dma = [&](uint16_t* buf, int c) {
#pragma unroll
    for (int p = 0; p < kQ; ++p) dma_one(buf, c, p);
  };

  // lm_head rows of this wave: 16 NBW rows from vw on, read row-contiguously (half a chunk is
  // 2 NBW loads of eight 128-byte row segments each: lane l takes row 8 i + l / 8, slot l % 8),
  // rows past V repeat row V - 1; buffer loads from the work-group's first row, non-temporal
  const int vt0 = v0 + blockIdx.x * kVT;
  const int nrows = min(kVT, a.V - vt0);
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.lm_head + (size_t)vt0 * a.H), (short)0, (int)((size_t)nrows * a.H * 2), 0x00020000);
  constexpr int kAL = 2 * kNBW;  // loads per half chunk
  int aoff[kAL];
#pragma unroll
  for (int i = 0; i < kAL; ++i) aoff[i] = min(w * 16 * kNBW + i * 8 + (lane >> 3), nrows - 1) * a.H * 2 + (lane & 7) * 16;
  auto aload = [&](int c, int h, int i) {
    return __builtin_amdgcn_raw_buffer_load_b128(ars, aoff[i], (c + coff >= NC ? c + coff - NC : c + coff) * 256 + h * 128, 2);
  };
  uint16_t* sa = s_a[w];
  // staging slot of load i's lane: row 8 i + lane / 8, slot (lane % 8) ^ ((4 i + lane / 16) % 8)
  int soff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) soff[i] = (lane >> 3) * 64 + (((lane & 7) ^ ((i * 4 + (lane >> 4)) & 7)) * 8);
  // operand read of slice q of a half: row 16 nb + lr, slot (4 q + lg) ^ ((lr / 2) % 8)
  int roff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) roff[q] = lr * 64 + (((q * 4 + lg) ^ ((lr >> 1) & 7)) * 8);
  floatx4 acc[kNBW][MB];
#pragma unroll
  for (int nb = 0; nb < kNBW; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  // lm_head ring of two chunks. Per chunk c the copies go out before the slices' operand reads:
  // lm_head half 0 of chunk c + 1 (slice 0), the two halves of hidden chunk c + 1 (slices 1
  // and 2), lm_head half 1 of chunk c + 1 (slice 3). The wait for the hidden chunk at the end of
  // chunk c leaves those last lm_head loads in flight (first staged at slice 2 of chunk c + 1).
  dma(s_h0, 0);
  u32x4 A[2][2][kAL];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < kAL; ++i) A[0][h][i] = aload(0, h, i);
  chunk_barrier<0>();

#pragma nounroll
  for (int c0 = 0; c0 < NC; c0 += 2) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int c = c0 + cc;  // chunk c: ring slot and LDS buffer cc (NC is even: H is a multiple of 256)
      {
        uint16_t* cur = cc ? s_h1 : s_h0;
        uint16_t* nxt = cc ? s_h0 : s_h1;
        // the last chunk is requested again at the end (L2 hits, never used)
        const int ch = min(c + 1, NC - 1);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          if (p == 0 || p == 3) {
#pragma unroll
            for (int i = 0; i < kAL; ++i) A[cc ^ 1][p == 3][i] = aload(ch, p == 3, i);
          } else {
#pragma unroll
            for (int q = 0; q < kQ; ++q)
              if ((q < (kQ + 1) / 2) == (p == 1)) dma_one(nxt, ch, q);
          }
          __builtin_amdgcn_sched_barrier(0);
          if ((p & 1) == 0) {
            // this half's lm_head rows into the wave's staging area (LDS operations of a wave
            // complete in order: the previous half's operand reads are done before these land)
#pragma unroll
            for (int i = 0; i < kAL; ++i) *(u32x4*)(sa + i * 8 * 64 + soff[i & 1]) = A[cc][p >> 1][i];
          }
          const uint16_t* hb = cur + lr * kKC + (((p * 4 + lg) ^ lr) * 8);
          bf16x8 af[kNBW];
#pragma unroll
          for (int nb = 0; nb < kNBW; ++nb) af[nb] = *(const bf16x8*)(sa + nb * 16 * 64 + roff[p & 1]);
          // all of the slice's hidden fragments first, so their LDS reads overlap
          bf16x8 bfr[MB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) bfr[mb] = *(const bf16x8*)(hb + mb * 16 * kKC);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < kNBW; ++nb)
              acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[nb], bfr[mb], acc[nb][mb], 0, 0, 0);
          if ((p & 1) == 0) __builtin_amdgcn_sched_group_barrier(0x200, kAL, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, MB + kNBW, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, kNBW * MB, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // hidden chunk c + 1 has landed in LDS (only lm_head half 1 of chunk c + 1 may be in flight)
        chunk_barrier<kAL>();
      }
    }
  }
  // D layout: lane holds vocabulary rows 4 lg .. 4 lg + 3 of its block for row lr of the M block
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m0 + mb * 16 + lr;
    if (m >= a.M) continue;
    const int b = m / a.K, k = m - b * a.K;
    const long long off = (long long)b * a.out_rs + (long long)k * a.out_ss;
#pragma unroll
    for (int nb = 0; nb < kNBW; ++nb) {
      const int v = vw + nb * 16 + lg * 4;
      const floatx4 z = acc[nb][mb];
      if (S0 && k == 0) {
        // step-0 row: kept for the fused step, in the base dtype's precision
        float* o = (float*)s_a[w] + b * (16 * kNBW) + nb * 16 + lg * 4;
        if (OBF16)
          *(f32x4*)o = f32x4{bf16_bits_to_f32(f32_to_bf16_bits(z[0])), bf16_bits_to_f32(f32_to_bf16_bits(z[1])),
                             bf16_bits_to_f32(f32_to_bf16_bits(z[2])), bf16_bits_to_f32(f32_to_bf16_bits(z[3]))};
        else
          *(f32x4*)o = f32x4{z[0], z[1], z[2], z[3]};
        continue;
      }
      if (OBF16) {
        uint16_t* o = (uint16_t*)a.out + off + v;
        const uint32_t h0 = f32_to_bf16_bits(z[0]), h1 = f32_to_bf16_bits(z[1]);
        const uint32_t h2 = f32_to_bf16_bits(z[2]), h3 = f32_to_bf16_bits(z[3]);
        if (a.vec_out && v + 3 < a.V) {
          *(u32x2*)o = u32x2{h0 | (h1 << 16), h2 | (h3 << 16)};
        } else {
          const uint32_t hh[4] = {h0, h1, h2, h3};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (v + i < a.V) o[i] = (uint16_t)hh[i];
        }
      } else {
        float* o = (float*)a.out + off + v;
        if (a.vec_out && v + 3 < a.V) {
          *(f32x4*)o = f32x4{z[0], z[1], z[2], z[3]};
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (v + i < a.V) o[i] = z[i];
        }
      }
    }
  }
  if constexpr (S0 != 0) {
    // (issued once the accumulators are stored: holding these registers during
    // the stores would spill; the anchors were read at the start, so none of
    // these loads waits on another)
    Step0In<kNBW> in0;
    step0_load<kNBW>(d, vw, tk0, in0);
    fused_step0<kNBW, NW, S0 == 2>(d, vw, gbase + blockIdx.x, (const float*)s_a[w], (unsigned char*)s_h1, m0, MT, tk0,
                                   in0);
  }
}

template <int MB, int NBW, int NW, int S0>
hipError_t launch_mbs(const LmHeadArgs& a, int v0, int n_tiles, int m_tiles, const DraftStepArgs& d, int gbase,
                      hipStream_t st) {
  const dim3 grid(n_tiles, m_tiles);
  if (a.out_bf16)
    hipLaunchKernelGGL((lm_head_kernel<MB, NBW, NW, true, S0>), grid, dim3(NW * 64), 0, st, a, v0, d, gbase);
  else
    hipLaunchKernelGGL((lm_head_kernel<MB, NBW, NW, false, S0>), grid, dim3(NW * 64), 0, st, a, v0, d, gbase);
  return hipGetLastError();
}

template <int MB, int NBW, int NW>
hipError_t launch_mb(const LmHeadArgs& a, int v0, int n_tiles, int m_tiles, const DraftStepArgs* d, int gbase,
                     hipStream_t st) {
  if (!d) return launch_mbs<MB, NBW, NW, 0>(a, v0, n_tiles, m_tiles, DraftStepArgs{}, 0, st);
  if (d->cache_bf16) return launch_mbs<MB, NBW, NW, 2>(a, v0, n_tiles, m_tiles, *d, gbase, st);
  return launch_mbs<MB, NBW, NW, 1>(a, v0, n_tiles, m_tiles, *d, gbase, st);
}

// One work-group per CU: the 256-row tiles (eight waves of 32 rows, two per
// SIMD; four of 64 for a 13-block M tile, whose eight-wave form would spill)
// run in rounds of `cus`; M tiles of 15 or 16 blocks take 128-row tiles (four
// waves of 32 rows) to keep their accumulators in registers. A last partial
// round (whose few work-groups would each still stream their whole lm_head
// tile, and re-read every hidden row, through one CU while the others idle) is
// instead covered by tail work-groups of 64 vocabulary rows by 64 rows of M
// (four waves of 16 rows); a vocabulary too small for one round takes only
// tail work-groups.
template <int MB>
int split_tiles(const LmHeadArgs& a, int m_tiles, int& full, int& tail) {
  constexpr int NWM = (MB <= 14 && MB != 13) ? 8 : 4;
  constexpr int NBW = MB <= 14 ? 256 / 16 / NWM : 2;
  constexpr int ROWS = 16 * NBW * NWM;
  const int tiles = (a.V + ROWS - 1) / ROWS;
  const int cus = a.cus > 0 ? a.cus : tiles;
  full = m_tiles == 1 ? (tiles / cus) * cus : tiles;
  tail = full == tiles ? 0 : (a.V - full * ROWS + 63) / 64;
  return ROWS;
}

// d: the fused step 0 (null: the plain LM head); its q partials take slots
// 0 .. full + tail - 1 (the work-groups of both launches)
template <int MB>
hipError_t launch_split(const LmHeadArgs& a, int m_tiles, const DraftStepArgs* d, hipStream_t st) {
  constexpr int NWM = (MB <= 14 && MB != 13) ? 8 : 4;
  constexpr int NBW = MB <= 14 ? 256 / 16 / NWM : 2;
  constexpr int MBT = MB < 4 ? MB : 4;
  int full, tail;
  const int rows = split_tiles<MB>(a, m_tiles, full, tail);
  if (full > 0) {
    const hipError_t e = launch_mb<MB, NBW, NWM>(a, 0, full, m_tiles, d, 0, st);
    if (e != hipSuccess || tail == 0) return e;
  }
  // a tail exists only with one M tile of at most 256 rows
  return launch_mb<MBT, 1, 4>(a, full * rows, tail, (a.M + 16 * MBT - 1) / (16 * MBT), d, full, st);
}

}  // namespace

hipError_t launch_lm_head(const LmHeadArgs& a, hipStream_t st, const DraftStepArgs* step0) {
  const int M = a.M;
  const int mb = M >= 256 ? 16 : (M + 15) / 16;
  const int m_tiles = (M + 255) / 256;
  switch (mb) {
    case 1: return launch_split<1>(a, m_tiles, step0, st);
    case 2: return launch_split<2>(a, m_tiles, step0, st);
    case 3: return launch_split<3>(a, m_tiles, step0, st);
    case 4: return launch_split<4>(a, m_tiles, step0, st);
    case 5: return launch_split<5>(a, m_tiles, step0, st);
    case 6: return launch_split<6>(a, m_tiles, step0, st);
    case 7: return launch_split<7>(a, m_tiles, step0, st);
    case 8: return launch_split<8>(a, m_tiles, step0, st);
    case 9: return launch_split<9>(a, m_tiles, step0, st);
    case 10: return launch_split<10>(a, m_tiles, step0, st);
    case 11: return launch_split<11>(a, m_tiles, step0, st);
    case 12: return launch_split<12>(a, m_tiles, step0, st);
    case 13: return launch_split<13>(a, m_tiles, step0, st);
    case 14: return launch_split<14>(a, m_tiles, step0, st);
    case 15: return launch_split<15>(a, m_tiles, step0, st);
    default: return launch_split<16>(a, m_tiles, step0, st);
  }
}

int lm_head_work_groups(const LmHeadArgs& a) {
  int full = 0, tail = 0;
  const int M = a.M;
  const int mb = M >= 256 ? 16 : (M + 15) / 16;
  const int m_tiles = (M + 255) / 256;
  switch (mb) {
    case 13: split_tiles<13>(a, m_tiles, full, tail); break;
    case 15: split_tiles<15>(a, m_tiles, full, tail); break;
    case 16: split_tiles<16>(a, m_tiles, full, tail); break;
    default: split_tiles<14>(a, m_tiles, full, tail); break;  // every other M tile takes 256-row tiles
  }
  return full + tail;
}

}  // namespace mds
