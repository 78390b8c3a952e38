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

// MB: 16-row blocks of the M tile; NBW: 16-row vocabulary blocks per wave; NW:
// waves (the work-group covers 16 NBW NW rows from vocabulary row v0 on)
template <int MB, int NBW, int NW, bool OBF16>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void lm_head_kernel(LmHeadArgs a, int v0) {
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
}

template <int MB, int NBW, int NW>
hipError_t launch_mb(const LmHeadArgs& a, int v0, int n_tiles, int m_tiles, hipStream_t st) {
  const dim3 grid(n_tiles, m_tiles);
  if (a.out_bf16)
    hipLaunchKernelGGL((lm_head_kernel<MB, NBW, NW, true>), grid, dim3(NW * 64), 0, st, a, v0);
  else
    hipLaunchKernelGGL((lm_head_kernel<MB, NBW, NW, false>), grid, dim3(NW * 64), 0, st, a, v0);
  return hipGetLastError();
}

// One work-group per CU: the 256-row tiles (eight waves of 32 rows, two per
// SIMD; four of 64 for a 13-block M tile, whose eight-wave form would spill)
// run in rounds of `cus`; M tiles of 15 or 16 blocks take 128-row tiles (four
// waves of 32 rows) to keep their accumulators in registers. A last partial
// round (whose few work-groups would each still stream their whole lm_head
// tile through one CU while the others idle) is instead covered by 64-row
// tiles (four waves of 16 rows); a vocabulary too small for one round uses
// 64-row tiles throughout.
template <int MB>
hipError_t launch_split(const LmHeadArgs& a, int m_tiles, hipStream_t st) {
  constexpr int NWM = (MB <= 14 && MB != 13) ? 8 : 4;
  constexpr int NBW = MB <= 14 ? 256 / 16 / NWM : 2;
  constexpr int ROWS = 16 * NBW * NWM;
  const int tiles = (a.V + ROWS - 1) / ROWS;
  const int cus = a.cus > 0 ? a.cus : tiles;
  const int full = m_tiles == 1 ? (tiles / cus) * cus : tiles;
  if (full == tiles) return launch_mb<MB, NBW, NWM>(a, 0, tiles, m_tiles, st);
  if (full > 0) {
    const hipError_t e = launch_mb<MB, NBW, NWM>(a, 0, full, m_tiles, st);
    if (e != hipSuccess) return e;
  }
  const int v0 = full * ROWS;
  return launch_mb<MB, 1, 4>(a, v0, (a.V - v0 + 63) / 64, m_tiles, st);
}

}  // namespace

hipError_t launch_lm_head(const LmHeadArgs& a, hipStream_t st) {
  const int M = a.M;
  const int mb = M >= 256 ? 16 : (M + 15) / 16;
  const int m_tiles = (M + 255) / 256;
  switch (mb) {
    case 1: return launch_split<1>(a, m_tiles, st);
    case 2: return launch_split<2>(a, m_tiles, st);
    case 3: return launch_split<3>(a, m_tiles, st);
    case 4: return launch_split<4>(a, m_tiles, st);
    case 5: return launch_split<5>(a, m_tiles, st);
    case 6: return launch_split<6>(a, m_tiles, st);
    case 7: return launch_split<7>(a, m_tiles, st);
    case 8: return launch_split<8>(a, m_tiles, st);
    case 9: return launch_split<9>(a, m_tiles, st);
    case 10: return launch_split<10>(a, m_tiles, st);
    case 11: return launch_split<11>(a, m_tiles, st);
    case 12: return launch_split<12>(a, m_tiles, st);
    case 13: return launch_split<13>(a, m_tiles, st);
    case 14: return launch_split<14>(a, m_tiles, st);
    case 15: return launch_split<15>(a, m_tiles, st);
    default: return launch_split<16>(a, m_tiles, st);
  }
}

}  // namespace mds
