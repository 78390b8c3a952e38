// Draft LM head (DSparkSpeculator API page, _sample_sequential and
// _sample_sequential_topk: compute_draft_logits turns the gathered hidden
// state of every (request, step) row into that row's base draft logits before
// the Markov loop).
//
// logits[m, v] = sum_h hidden[m, h] * lm_head[v, h]: bf16 inputs, float32
// accumulation on the matrix cores (v_mfma_f32_16x16x32_bf16), row m = b*K + k
// written to the base-logit layout the draft loop reads.
//
// With B*K rows in the low hundreds the product is bound by the lm_head
// stream (V*H*2 bytes, 1.64 GB at V = 200064, H = 4096), so each work-group
// owns 128 vocabulary rows for all rows of its M tile (up to 256) and lm_head
// is read from HBM once. One work-group per CU (accumulators in AGPRs, the
// VGPRs free for deep prefetch): each of the four waves streams its own 32
// vocabulary rows straight into MFMA A operands, two chunks of four 32-wide
// slices of H ahead in registers, a row's 256 bytes of a chunk requested
// together, with non-temporal loads (read once: they should not evict the
// hidden rows, which every work-group re-reads, from L2). The M tile's hidden rows go through LDS in 128-wide
// chunks (double buffered; rows padded to 272 bytes so the 16-byte fragment
// reads of 16 consecutive rows hit distinct banks), loaded into registers a
// whole chunk ahead. One barrier per chunk of four slices.
#include "mds_device.h"
#include "mds_internal.h"

namespace mds {
namespace {

constexpr int kNBW = 2;                   // 16-row vocabulary blocks per wave
constexpr int kVT = 4 * kNBW * 16;        // vocabulary rows per work-group (128)
constexpr int kKC = 128;                  // H columns per hidden chunk (4 slices)
constexpr int kRS = kKC + 8;              // LDS row stride of a hidden chunk (bf16)

// hidden chunk c of the M tile: thread t covers row 16 p + t / 16, 16-byte part t % 16.
// Rows past M repeat row M - 1 (their results are never stored): every load
// is unconditional, so the compiler can count outstanding loads exactly
// instead of draining them at a branch.
template <int MB>
__device__ __forceinline__ void chunk_load(const LmHeadArgs& a, int m0, int c, int tid, u32x4 (&hs)[MB]) {
#pragma unroll
  for (int p = 0; p < MB; ++p) {
    const int m = min(m0 + p * 16 + (tid >> 4), a.M - 1);
    hs[p] = *(const u32x4*)(a.hidden + (size_t)m * a.hidden_rs + c * kKC + (tid & 15) * 8);
  }
}

template <int MB>
__device__ __forceinline__ void chunk_store(uint16_t* buf, int tid, const u32x4 (&hs)[MB]) {
#pragma unroll
  for (int p = 0; p < MB; ++p) *(u32x4*)(buf + (p * 16 + (tid >> 4)) * kRS + (tid & 15) * 8) = hs[p];
}

template <int MB, bool OBF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void lm_head_kernel(LmHeadArgs a) {
  constexpr int MT = MB * 16;
  extern __shared__ __attribute__((aligned(16))) uint16_t s_h[];  // [2][MT * kRS]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int m0 = blockIdx.y * MT;
  const int vw = blockIdx.x * kVT + w * kNBW * 16;  // first vocabulary row of this wave
  const int S = a.H >> 5;                          // 32-wide slices of H (a multiple of 2 * 4)

  // A operands: vocabulary row vw + 16 nb + lr (clamped into range), elements 8 lg .. 8 lg + 7 of a slice
  const uint16_t* arow[kNBW];
#pragma unroll
  for (int nb = 0; nb < kNBW; ++nb) {
    const int v = min(vw + nb * 16 + lr, a.V - 1);
    arow[nb] = a.lm_head + (size_t)v * a.H + lg * 8;
  }
  // A ring: three chunks of four slices; chunk c + 2 is requested while chunk c
  // is multiplied, each row's 256 bytes of a chunk in one burst
  u32x4 A[3][4][kNBW];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int nb = 0; nb < kNBW; ++nb)
        A[r][p][nb] = __builtin_nontemporal_load((const u32x4*)(arow[nb] + (r * 4 + p) * 32));

  floatx4 acc[kNBW][MB];
#pragma unroll
  for (int nb = 0; nb < kNBW; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  u32x4 hs[MB];
  chunk_load<MB>(a, m0, 0, tid, hs);
  chunk_store<MB>(s_h, tid, hs);
  __syncthreads();

  const int NC = S / 4;  // chunks of four slices
  for (int c0 = 0; c0 < NC; c0 += 6) {
#pragma unroll
    for (int cc = 0; cc < 6; ++cc) {
      const int c = c0 + cc;  // chunk c: ring slot cc % 3, hidden rows in LDS buffer cc % 2
      if (c < NC) {
        // next hidden chunk first, then the A chunk two ahead: waiting for the
        // former at the end of this chunk does not wait for the latter (the
        // last chunks are requested again at the end: L2 hits, never used)
        chunk_load<MB>(a, m0, min(c + 1, NC - 1), tid, hs);
        const int cn = min(c + 2, NC - 1);
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
          for (int nb = 0; nb < kNBW; ++nb)
            A[(cc + 2) % 3][p][nb] = __builtin_nontemporal_load((const u32x4*)(arow[nb] + (cn * 4 + p) * 32));
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint16_t* hb = s_h + (cc & 1) * MT * kRS + lr * kRS + p * 32 + lg * 8;
          const bf16x8 a0 = __builtin_bit_cast(bf16x8, A[cc % 3][p][0]);
          const bf16x8 a1 = __builtin_bit_cast(bf16x8, A[cc % 3][p][1]);
          // all of the slice's hidden fragments first, so their LDS reads overlap
          bf16x8 bfr[MB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) bfr[mb] = *(const bf16x8*)(hb + mb * 16 * kRS);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            acc[0][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bfr[mb], acc[0][mb], 0, 0, 0);
            acc[1][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bfr[mb], acc[1][mb], 0, 0, 0);
          }
          // schedule: the slice's LDS reads all go out first, then the MFMAs
          // (the scheduler would otherwise wait on each read before its two
          // MFMAs, or chain one accumulator's MFMAs across slices)
          __builtin_amdgcn_sched_group_barrier(0x100, MB, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * MB, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        chunk_store<MB>(s_h + ((cc + 1) & 1) * MT * kRS, tid, hs);
        __syncthreads();
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

template <int MB>
hipError_t launch_mb(const LmHeadArgs& a, int m_tiles, hipStream_t st) {
  const dim3 grid((a.V + kVT - 1) / kVT, m_tiles);
  const size_t lds = (size_t)2 * MB * 16 * kRS * sizeof(uint16_t);
  const void* fn = a.out_bf16 ? (const void*)lm_head_kernel<MB, true> : (const void*)lm_head_kernel<MB, false>;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (a.out_bf16)
    hipLaunchKernelGGL((lm_head_kernel<MB, true>), grid, dim3(256), lds, st, a);
  else
    hipLaunchKernelGGL((lm_head_kernel<MB, false>), grid, dim3(256), lds, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lm_head(const LmHeadArgs& a, hipStream_t st) {
  const int M = a.M;
  const int mb = M >= 256 ? 16 : (M + 15) / 16;
  const int m_tiles = (M + 255) / 256;
  switch (mb) {
    case 1: return launch_mb<1>(a, m_tiles, st);
    case 2: return launch_mb<2>(a, m_tiles, st);
    case 3: return launch_mb<3>(a, m_tiles, st);
    case 4: return launch_mb<4>(a, m_tiles, st);
    case 5: return launch_mb<5>(a, m_tiles, st);
    case 6: return launch_mb<6>(a, m_tiles, st);
    case 7: return launch_mb<7>(a, m_tiles, st);
    case 8: return launch_mb<8>(a, m_tiles, st);
    case 9: return launch_mb<9>(a, m_tiles, st);
    case 10: return launch_mb<10>(a, m_tiles, st);
    case 11: return launch_mb<11>(a, m_tiles, st);
    case 12: return launch_mb<12>(a, m_tiles, st);
    case 13: return launch_mb<13>(a, m_tiles, st);
    case 14: return launch_mb<14>(a, m_tiles, st);
    case 15: return launch_mb<15>(a, m_tiles, st);
    default: return launch_mb<16>(a, m_tiles, st);
  }
}

}  // namespace mds
