// Markov draft step, wave-independent streaming variant (gfx950, rank <= 256).
//
// The same fused step as draft_step_kernel (one step of the sequential loop of
// the DSparkSpeculator API page: Markov embedding of the previous token ->
// Markov bias -> biased logits -> Gumbel-max sample, plus the draft-logits
// cache and its (max, sum exp) for q), laid out so that the four waves of a
// work-group never wait for each other inside the column loop:
//   * wave w of slab g walks the 16-column tiles mt_begin + w, + 4, + 8, ...;
//   * the 16 w2 rows of a tile are loaded straight into the MFMA A operand
//     (v_mfma_f32_16x16x32_bf16, lane l: row l % 16, rank elements
//     8 (l / 16) + 32 s of slice s), and the next tile's rows and base logits
//     are in flight while the current tile is computed;
//   * the embeddings of the batch tile (the B operand) are read once: into
//     LDS by the work-group, or, on the fast path, by each wave straight into
//     registers (previous tokens, then embedding rows, then the first tiles,
//     so that this dependent chain has no other load queued ahead of it);
//   * the epilogue runs in the accumulator layout: lane l owns request
//     16 nt + l % 16 and the 4 consecutive columns 4 (l / 16) .. + 3 of the
//     tile, so base loads and cache stores are 16-byte vector accesses.
// Winners and q statistics are merged across the 4 lanes of a request row,
// then across the waves in LDS, then across work-groups with one 64-bit
// atomic max per request (PR #65007, Part 1, step 4: the first-max rule
// composes over any column partition).
#include "mds_device.h"
#include "mds_internal.h"

#include <type_traits>

namespace mds {

namespace {

// The fp64 option's float64 score of column col: the column's noise word
// again, then z / T + (-ln(-ln u)) in float64 (T = 1: z itself). Kept out of
// line: the fast loop calls it for the few columns that can still win.
__device__ __noinline__ double score64_of(float z, float T, int t1, uint32_t col, uint32_t pk0, uint32_t pk1,
                                          uint32_t sk0, uint32_t sk1) {
  const Philox4 w = philox4x32_10(col >> 2, pk0, pk1, kSaltDraft, sk0, sk1);
  const uint32_t sel = col & 3u;
  const uint32_t wd = sel == 0 ? w.x0 : (sel == 1 ? w.x1 : (sel == 2 ? w.x2 : w.x3));
  return (t1 ? (double)z : (double)z / (double)T) + gumbel64_from_word(wd);
}

constexpr int kRKMax = 8;  // rank slices of 32 (r <= 256)
constexpr int kRing = 2;   // ring entries (tiles in flight + the tile in use) per wave in the fast loop

// F64: the fp64 Gumbel option (scores and the running winner in float64).
// FL: compile the fixed-count fast loop; it raises the register count to one
// wave per SIMD, so it is used when the grid has one work-group per CU (up to
// kDraftFastTiles batch tiles, their slabs filling the CUs once) and left out
// otherwise.
template <int NB, bool BBF16, bool CBF16, bool F64, bool FL>
__global__ __launch_bounds__(256) void draft_wave_kernel(DraftStepArgs a) {
  using Score = typename std::conditional<F64, double, float>::type;
  constexpr int NT = NB / 16;
  const int r = a.r, V = a.V, k = a.k;
  const int RK = r >> 5;
  const int rs = r + 8;  // LDS row stride of the embeddings (bf16 elements)
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* s_e = (uint16_t*)smem;                                   // [NB][rs]
  int* s_prev = (int*)(s_e + NB * rs);                               // [NB]
  unsigned long long* s_key = (unsigned long long*)(s_prev + NB);    // [4][NB]
  float* s_qm = (float*)(s_key + 4 * NB);                            // [4][NB]
  float* s_qs = s_qm + 4 * NB;                                       // [4][NB]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  // Work-groups are dealt round-robin to the 8 XCDs by linear id; when the
  // slab count is a multiple of 8 the batch tiles of one slab share an XCD.
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
  const int mt_begin = (int)(((long long)g * a.nMT) / a.G);
  const int mt_end = (int)(((long long)(g + 1) * a.nMT) / a.G);

  // The previous tokens of the lane's requests, for the fast path: their
  // loads depend on nothing, so they go out ahead of the per-request
  // parameters and the two round trips overlap (the tokens, and then the
  // embedding rows, are the kernel's dependent chain).
  unsigned long long tkw[NT];
  if (FL) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int b = b0 + nt * 16 + lr;
      const int bb = b < a.B ? b : a.B - 1;
      tkw[nt] = (k == 0) ? (unsigned long long)(long long)a.anchor[bb] : a.keys[key_index(k - 1, a.B, bb)];
    }
    asm volatile("" ::: "memory");
  }

  // the requests this lane serves: 16 nt + lr of the batch tile
  bool valid[NT];
  float Tv[NT], invT[NT];
  uint32_t sk0[NT], sk1[NT], pk0[NT], pk1[NT];
  long long rbase[NT], rcache[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int b = b0 + nt * 16 + lr;
    const int sl = draft_slot(a, b);  // -1: past the batch or inert at this step
    valid[nt] = sl >= 0;
    const int bb = b < a.B ? b : a.B - 1;
    const int ss = valid[nt] ? sl : 0;  // a readable slot for rows that are not served
    Tv[nt] = a.temp[ss];
    invT[nt] = Tv[nt] > 0.0f ? 1.0f / Tv[nt] : 0.0f;
    const unsigned long long sd = (unsigned long long)a.seeds[ss];
    const unsigned long long pk = (unsigned long long)draft_pos_key(a, bb);
    sk0[nt] = (uint32_t)sd;
    sk1[nt] = (uint32_t)(sd >> 32);
    pk0[nt] = (uint32_t)pk;
    pk1[nt] = (uint32_t)(pk >> 32);
    rbase[nt] = (long long)bb * a.base_rs + (long long)k * a.base_ss;
    rcache[nt] = (long long)(valid[nt] ? draft_cache_row(a, b, sl) : 0) * a.cache_rs + (long long)k * a.cache_ss;
  }

  // Tile loaders. Row-major w2: a load covers 64 bytes of each of 16 rows,
  // and rows past V are read from row V - 1 (they only feed bias columns
  // past V, which the epilogue never uses). Tiled w2 (tile_w2_kernel): the
  // same operands in load order, so a load covers 1 KB of one tile, and the
  // last tile is padded. No select touches the loaded data, so the next
  // tile's loads stay in flight.
  const bool tiled = a.w2_tiled != 0;
  const int sstep = tiled ? 512 : 32;  // elements from one rank slice to the next
  auto a_lane = [&](int t) {
    const int v = t * 16 + lr;
    return tiled ? a.w2 + (size_t)t * 16 * r + lane * 8 : a.w2 + (size_t)(v < V ? v : V - 1) * r + lg * 8;
  };
  auto load_a = [&](int t, u32x4 (&A)[kRKMax]) {
    const uint16_t* p = a_lane(t);
#pragma unroll
    for (int s = 0; s < kRKMax; ++s) A[s] = *(const u32x4*)(p + (s < RK ? s : RK - 1) * sstep);
  };
  // The fast loop's loader, with the layout a constant (the slice offsets
  // then fold into the load instructions); FULL: rank r = 32 kRKMax, every
  // slice real.
  auto load_a_fixed = [&](auto tiled_tag, auto full_tag, int t, u32x4 (&A)[kRKMax]) {
    constexpr bool TL = decltype(tiled_tag)::value;
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr int SS = TL ? 512 : 32;
    const int v = t * 16 + lr;
    const uint16_t* p = TL ? a.w2 + (size_t)t * 16 * (FULL ? 32 * kRKMax : r) + lane * 8
                           : a.w2 + (size_t)(v < V ? v : V - 1) * (FULL ? 32 * kRKMax : r) + lg * 8;
#pragma unroll
    for (int s = 0; s < kRKMax; ++s) A[s] = *(const u32x4*)(p + (FULL ? s : (s < RK ? s : RK - 1)) * SS);
  };
  auto load_base_vec = [&](int t, float (&bz)[NT][4]) {
    const int c = t * 16 + lg * 4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (BBF16) {
        const u32x2 w = *(const u32x2*)((const uint16_t*)a.base + rbase[nt] + c);
        bz[nt][0] = bf16_bits_to_f32(w.x & 0xFFFFu);
        bz[nt][1] = bf16_bits_to_f32(w.x >> 16);
        bz[nt][2] = bf16_bits_to_f32(w.y & 0xFFFFu);
        bz[nt][3] = bf16_bits_to_f32(w.y >> 16);
      } else {
        const f32x4 w = *(const f32x4*)((const float*)a.base + rbase[nt] + c);
        bz[nt][0] = w.x;
        bz[nt][1] = w.y;
        bz[nt][2] = w.z;
        bz[nt][3] = w.w;
      }
    }
  };
  auto load_base = [&](int t, float (&bz)[NT][4]) {
    const int c = t * 16 + lg * 4;
    if (a.vec_base && t * 16 + 16 <= V) {  // whole tile inside V: a wave-uniform test
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (BBF16) {
          const u32x2 w = *(const u32x2*)((const uint16_t*)a.base + rbase[nt] + c);
          bz[nt][0] = bf16_bits_to_f32(w.x & 0xFFFFu);
          bz[nt][1] = bf16_bits_to_f32(w.x >> 16);
          bz[nt][2] = bf16_bits_to_f32(w.y & 0xFFFFu);
          bz[nt][3] = bf16_bits_to_f32(w.y >> 16);
        } else {
          const f32x4 w = *(const f32x4*)((const float*)a.base + rbase[nt] + c);
          bz[nt][0] = w.x;
          bz[nt][1] = w.y;
          bz[nt][2] = w.z;
          bz[nt][3] = w.w;
        }
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const long long off = rbase[nt] + c + i;
          bz[nt][i] = c + i < V ? (BBF16 ? bf16_bits_to_f32(((const uint16_t*)a.base)[off])
                                         : ((const float*)a.base)[off])
                                : 0.0f;
        }
    }
  };

  const int t_first = mt_begin + wave;
  u32x4 A[kRKMax], An[kRKMax];
  float bz[NT][4], bzn[NT][4];

  // Running winner and q statistics per served request. The winner starts
  // at the lane's first column (value -inf), so a later column replaces it
  // only when strictly larger or the first NaN: the first-max rule.
  const int c_first = t_first * 16 + lg * 4;
  Score bv[NT];
  float qm[NT], qs[NT];
  int bi[NT];
  bool qnan[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    bv[nt] = -INFINITY;
    bi[nt] = (t_first < mt_end && c_first < V) ? c_first : -1;
    qm[nt] = -INFINITY;
    qs[nt] = 0.0f;
    qnan[nt] = false;
  }
  // Fast epilogue for full tiles when every served request of the batch tile
  // samples (T > 0), with vector cache stores (none for the rows that are not
  // served: padding past the batch, or inert at this step); T == 1 skips the
  // division.
  bool all_sampled = true, all_t1 = true;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    all_sampled &= !valid[nt] || Tv[nt] > 0.0f;
    all_t1 &= !valid[nt] || Tv[nt] == 1.0f;
  }
  // the same value in every wave of the work-group (the waves serve the same requests)
  const bool fast_req = a.vec_cache && __all(all_sampled);
  const bool t1 = __all(all_t1);

  // Fast loop: the full tiles of a work-group whose requests all exist and
  // sample, with vector base loads and cache stores. Its body has a fixed
  // number of memory operations (the next tile's loads, then this tile's
  // stores), so the wait for the next tile leaves this tile's stores in
  // flight; the remaining tiles (a partial last tile, other work-groups) take
  // the general loop below.
  int t_gen = t_first;
  if (FL && fast_req && a.vec_base) {
    // Direct path. Each wave reads the embedding rows of its lanes'
    // requests' previous tokens (loaded at the start) straight into MFMA B
    // operands (request 16 nt + lr, rank elements 8 lg + 32 s of slice s),
    // then the first tiles. Loads complete in issue order, so nothing is
    // queued ahead of this dependent chain, and no work-group barrier waits
    // for it.
    int pv[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // rows that are not served read a request's token (an address inside
      // the arrays) and keep a zero token without a status bit
      long long tk = (k == 0) ? (long long)tkw[nt] : (long long)key_col(tkw[nt], F64);
      if (tk < 0 || tk >= V) {
        if (valid[nt]) set_status(a.status, kStatusBadAnchor);
        tk = 0;
      }
      pv[nt] = valid[nt] ? (int)tk : 0;
    }
    const int full_end = mt_end < V / 16 ? mt_end : V / 16;  // tiles [mt_begin, full_end) lie inside V
    // the embedding operands are the same for every tile: read once, kept in
    // registers for the whole loop (one wave per SIMD leaves room)
    bf16x8 Er[NT][kRKMax];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int s = 0; s < kRKMax; ++s)
        Er[nt][s] = *(const bf16x8*)(a.w1 + (size_t)pv[nt] * r + (s < RK ? s : 0) * 32 + lg * 8);
    asm volatile("" ::: "memory");  // the tile loads stay behind the embedding loads
    // fp64 option: every element's float32 score comes first (within ~1e-5
    // of its float64 score), and a lane scores in float64 only the elements
    // that can still win. It keeps its two best float32 scores per request
    // tile (stable: an equal later score does not displace an earlier one);
    // an element that leaves or never enters them while within the margin of
    // the running maximum is scored at once, and anything below the margin is
    // beaten, in float64 too, by the element holding that maximum. After the
    // loop the two kept are scored, and all are merged by the winner rule:
    // the first NaN, else the largest score, the lower column on a tie. An
    // element whose float32 score overflowed (a finite logit over a tiny
    // temperature) is scored at once.
    float k2s[NT][2], k2z[NT][2];
    int k2c[NT][2], nanc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      nanc[nt] = -1;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        k2s[nt][j] = -INFINITY;
        k2z[nt][j] = 0.0f;
        k2c[nt][j] = -1;
      }
    }
    auto margin = [](float m) { return m - (1e-4f + 1e-5f * fabsf(m)); };
    auto exact = [&](auto t1_tag, int nt, float zz, int col) {
      const double sv = score64_of(zz, Tv[nt], decltype(t1_tag)::value, (uint32_t)col, pk0[nt], pk1[nt], sk0[nt],
                                   sk1[nt]);
      const double b = (double)bv[nt];
      const bool take = sv != sv ? (b == b || col < bi[nt]) : (b == b && (sv > b || (sv == b && col < bi[nt])));
      bv[nt] = take ? (Score)sv : bv[nt];
      bi[nt] = take ? col : bi[nt];
    };
    // One full tile of the fast loop: bias by MFMA from the ring entry's w2
    // rows, then the branch-free epilogue.
    // MASK: some row of the batch tile is not served (its cache stores are skipped)
    auto fast_tile = [&](auto t1_tag, auto full_tag, auto mask_tag, int t, const u32x4 (&Ab)[kRKMax],
                         const float (&bzb)[NT][4]) {
      constexpr bool T1 = decltype(t1_tag)::value;
      constexpr bool FULL = decltype(full_tag)::value;
      constexpr bool MASK = decltype(mask_tag)::value;
      floatx4 acc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < kRKMax; ++s) {
        if (FULL || s < RK) {
          const bf16x8 afr = __builtin_bit_cast(bf16x8, Ab[s]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, Er[nt][s], acc[nt], 0, 0, 0);
        }
      }
      const int c = t * 16 + lg * 4;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float z[4], cv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = bzb[nt][i] + acc[nt][i];
        if (CBF16) {
          uint32_t h[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            h[i] = f32_to_bf16_bits(z[i]);
            cv[i] = bf16_bits_to_f32(h[i]);
          }
          u32x2 w;
          w.x = h[0] | (h[1] << 16);
          w.y = h[2] | (h[3] << 16);
          if (!MASK || valid[nt]) *(u32x2*)((uint16_t*)a.cache + rcache[nt] + c) = w;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) cv[i] = z[i];
          if (!MASK || valid[nt]) *(f32x4*)((float*)a.cache + rcache[nt] + c) = f32x4{z[0], z[1], z[2], z[3]};
        }
        const Philox4 w = philox4x32_10((uint32_t)(c >> 2), pk0[nt], pk1[nt], kSaltDraft, sk0[nt], sk1[nt]);
        const uint32_t wd[4] = {w.x0, w.x1, w.x2, w.x3};
        float y[4], x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y[i] = T1 ? z[i] : div_t(z[i], Tv[nt], invT[nt]);
          x[i] = CBF16 ? (T1 ? cv[i] : div_t(cv[i], Tv[nt], invT[nt])) : y[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (F64) {
            const float s32 = y[i] + gumbel_from_word(wd[i]);
            const bool up0 = s32 > k2s[nt][0], up1 = s32 > k2s[nt][1];
            // the element that leaves the two (or never enters): an old
            // second, or this one; NaN goes to nanc, -inf can never win
            const float ds = up1 ? k2s[nt][1] : s32;
            const float dz = up1 ? k2z[nt][1] : z[i];
            const int dc = up1 ? k2c[nt][1] : c + i;
            k2s[nt][1] = up0 ? k2s[nt][0] : (up1 ? s32 : k2s[nt][1]);
            k2z[nt][1] = up0 ? k2z[nt][0] : (up1 ? z[i] : k2z[nt][1]);
            k2c[nt][1] = up0 ? k2c[nt][0] : (up1 ? c + i : k2c[nt][1]);
            k2s[nt][0] = up0 ? s32 : k2s[nt][0];
            k2z[nt][0] = up0 ? z[i] : k2z[nt][0];
            k2c[nt][0] = up0 ? c + i : k2c[nt][0];
            if (s32 != s32 && nanc[nt] < 0) nanc[nt] = c + i;
            if (dc >= 0 && ds > -INFINITY && ds >= margin(k2s[nt][0])) exact(t1_tag, nt, dz, dc);
            // a finite logit whose float32 score overflowed (z / T past the
            // float32 range) has a finite float64 score the filter cannot
            // rank: it is scored at once
            if (!T1 && fabsf(s32) == INFINITY && fabsf(z[i]) < INFINITY) exact(t1_tag, nt, z[i], c + i);
          } else {
            const Score sv = y[i] + gumbel_from_word(wd[i]);
            // the winner rule as one mask: a held NaN stays; otherwise a NaN
            // or a strictly larger score replaces it
            const bool take = (bv[nt] == bv[nt]) & !(sv <= bv[nt]);
            bv[nt] = take ? sv : bv[nt];
            bi[nt] = take ? c + i : bi[nt];
          }
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
    };
    // The loop keeps kRing tiles in flight per wave: ring entry i holds tile
    // t + 4 i. Entries are refilled right after their tile is computed, with
    // the tile kRing steps ahead, so a load has kRing - 1 tiles of compute
    // to arrive. The loop is unrolled over the ring (no register copies,
    // which would wait for the loads) and runs whole turns only; the last
    // partial turn computes the entries already loaded.
    auto run_fast = [&](auto t1_tag, auto full_tag, auto mask_tag, auto tiled_tag) {
      auto load = [&](int tt, u32x4 (&Ab)[kRKMax]) { load_a_fixed(tiled_tag, full_tag, tt, Ab); };
      int t = t_first;
      if (t < full_end) {
        const int t_lastf = t_first + ((full_end - 1 - t_first) / 4) * 4;
        const int n_tiles = (t_lastf - t_first) / 4 + 1;
        const int n_turns = n_tiles / kRing;
        u32x4 Ar[kRing][kRKMax];
        float bzr[kRing][NT][4];
#pragma unroll
        for (int e = 0; e < kRing; ++e) {
          const int te = t + 4 * e <= t_lastf ? t + 4 * e : t_lastf;  // past the last tile: that tile again (cache hits)
          load(te, Ar[e]);
          load_base_vec(te, bzr[e]);
        }
        for (int turn = 0; turn < n_turns; ++turn) {
#pragma unroll
          for (int e = 0; e < kRing; ++e) {
            fast_tile(t1_tag, full_tag, mask_tag, t + 4 * e, Ar[e], bzr[e]);
            const int tn = t + 4 * (e + kRing) <= t_lastf ? t + 4 * (e + kRing) : t_lastf;
            load(tn, Ar[e]);
            load_base_vec(tn, bzr[e]);
          }
          t += 4 * kRing;
        }
        const int rest = n_tiles - n_turns * kRing;
#pragma unroll
        for (int e = 0; e < kRing - 1; ++e)
          if (e < rest) fast_tile(t1_tag, full_tag, mask_tag, t + 4 * e, Ar[e], bzr[e]);
        t += 4 * rest;
        if constexpr (F64) {  // the kept two and the first NaN join the lane's winner
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
              if (k2c[nt][j] >= 0) exact(t1_tag, nt, k2z[nt][j], k2c[nt][j]);
            if (nanc[nt] >= 0) {
              const double b = (double)bv[nt];
              if (b == b || nanc[nt] < bi[nt]) {
                bv[nt] = (Score)NAN;
                bi[nt] = nanc[nt];
              }
            }
          }
        }
      }
      return t;
    };
    using True = std::integral_constant<bool, true>;
    using False = std::integral_constant<bool, false>;
    auto fast = [&](auto t1_tag, auto full_tag, auto mask_tag) {  // the w2 layout a constant of the loop
      return tiled ? run_fast(t1_tag, full_tag, mask_tag, True()) : run_fast(t1_tag, full_tag, mask_tag, False());
    };
    bool all_valid = true;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) all_valid &= valid[nt];
    if (!__all(all_valid))  // padding rows (small batches): one general instance (the division by T = 1 is exact)
      t_gen = fast(False(), False(), True());
    else if (RK == kRKMax)
      t_gen = t1 ? fast(True(), True(), False()) : fast(False(), True(), False());
    else
      t_gen = t1 ? fast(True(), False(), False()) : fast(False(), False(), False());
    if (V & 15) {  // some work-group has a partial last tile: the general loop reads the embeddings from LDS
      if (wave == 0) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int s = 0; s < kRKMax; ++s)
            if (s < RK) *(bf16x8*)(s_e + (nt * 16 + lr) * rs + s * 32 + lg * 8) = Er[nt][s];
      }
      __syncthreads();
    }
    if (t_gen < mt_end) {  // the partial last tile, for the general loop
      load_a(t_gen, A);
      load_base(t_gen, bz);
    }
  } else {
    // the first tile's loads go out before the previous tokens and the
    // embedding gather, whose latency they then overlap
    if (t_first < mt_end) {
      load_a(t_first, A);
      load_base(t_first, bz);
    }
    // previous token of every request of the tile
    const int cpr = r >> 3;  // 16-byte chunks per embedding row
    for (int i = tid; i < NB; i += 256) {
      const int b = b0 + i;
      int prev = -1;  // rows that are not served get a zero embedding
      if (draft_slot(a, b) >= 0) {
        // the previous step's winner (key 0, i.e. -1, when that step was inert)
        long long tk = (k == 0) ? (long long)a.anchor[b] : (long long)key_col(a.keys[key_index(k - 1, a.B, b)], F64);
        if (tk < 0 || tk >= V) {
          set_status(a.status, kStatusBadAnchor);
          tk = 0;
        }
        prev = (int)tk;
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
    __syncthreads();
  }

  // the wave's last tile: the prefetch past it requests that tile again
  const int t_last = t_gen < mt_end ? t_gen + ((mt_end - 1 - t_gen) / 4) * 4 : t_gen;
  for (int t = t_gen; t < mt_end; t += 4) {
    {
      const int tn = t + 4 < mt_end ? t + 4 : t_last;
      load_a(tn, An);
      load_base(tn, bzn);
    }
    // bias of this tile: D[column][request] for the NT request tiles
    floatx4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < kRKMax; ++s) {
      if (s < RK) {
        const bf16x8 afr = __builtin_bit_cast(bf16x8, A[s]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const bf16x8 bfr = *(const bf16x8*)(s_e + (nt * 16 + lr) * rs + s * 32 + lg * 8);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr, acc[nt], 0, 0, 0);
        }
      }
    }
    // epilogue: lane holds columns c .. c+3 of request 16 nt + lr
    const int c = t * 16 + lg * 4;
    // Straight-line form: no per-element branches. A NaN among the q values
    // is carried by the sum itself (NaN stays NaN through every later merge).
    auto epi_fast = [&](auto t1_tag) {
      constexpr bool T1 = decltype(t1_tag)::value;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float z[4], cv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = bz[nt][i] + acc[nt][i];
        if (CBF16) {
          uint32_t h[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            h[i] = f32_to_bf16_bits(z[i]);
            cv[i] = bf16_bits_to_f32(h[i]);
          }
          u32x2 w;
          w.x = h[0] | (h[1] << 16);
          w.y = h[2] | (h[3] << 16);
          if (valid[nt]) *(u32x2*)((uint16_t*)a.cache + rcache[nt] + c) = w;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) cv[i] = z[i];
          if (valid[nt]) *(f32x4*)((float*)a.cache + rcache[nt] + c) = f32x4{z[0], z[1], z[2], z[3]};
        }
        const Philox4 w = philox4x32_10((uint32_t)(c >> 2), pk0[nt], pk1[nt], kSaltDraft, sk0[nt], sk1[nt]);
        const uint32_t wd[4] = {w.x0, w.x1, w.x2, w.x3};
        float y[4], x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y[i] = T1 ? z[i] : div_t(z[i], Tv[nt], invT[nt]);
          x[i] = CBF16 ? (T1 ? cv[i] : div_t(cv[i], Tv[nt], invT[nt])) : y[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Score sv;
          if (F64)
            sv = (T1 ? (double)z[i] : (double)z[i] / (double)Tv[nt]) + gumbel64_from_word(wd[i]);
          else
            sv = y[i] + gumbel_from_word(wd[i]);
          const bool take = (bv[nt] == bv[nt]) & !(sv <= bv[nt]);
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
    };
    if (fast_req && t * 16 + 16 <= V) {
      if (t1)
        epi_fast(std::integral_constant<bool, true>());
      else
        epi_fast(std::integral_constant<bool, false>());
    } else {
    const int n = V - c >= 4 ? 4 : (V - c > 0 ? V - c : 0);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (!valid[nt] || n == 0) continue;
      float z[4], cv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = bz[nt][i] + acc[nt][i];
      if (CBF16) {
        uint32_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[i] = f32_to_bf16_bits(z[i]);
          cv[i] = bf16_bits_to_f32(h[i]);
        }
        uint16_t* q = (uint16_t*)a.cache + rcache[nt] + c;
        if (a.vec_cache && n == 4) {
          u32x2 w;
          w.x = h[0] | (h[1] << 16);
          w.y = h[2] | (h[3] << 16);
          *(u32x2*)q = w;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i < n) q[i] = (uint16_t)h[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) cv[i] = z[i];
        float* q = (float*)a.cache + rcache[nt] + c;
        if (a.vec_cache && n == 4) {
          *(f32x4*)q = f32x4{z[0], z[1], z[2], z[3]};
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i < n) q[i] = z[i];
        }
      }
      if (Tv[nt] > 0.0f) {
        const Philox4 w = philox4x32_10((uint32_t)(c >> 2), pk0[nt], pk1[nt], kSaltDraft, sk0[nt], sk1[nt]);
        const uint32_t wd[4] = {w.x0, w.x1, w.x2, w.x3};
        float x[4];
        float xm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Score sv;
          if (F64)
            sv = (double)z[i] / (double)Tv[nt] + gumbel64_from_word(wd[i]);
          else
            sv = div_t(z[i], Tv[nt], invT[nt]) + gumbel_from_word(wd[i]);
          if (i < n) win_update(bv[nt], bi[nt], sv, c + i);
          const float xv = div_t(cv[i], Tv[nt], invT[nt]);
          qnan[nt] |= (i < n) && (xv != xv);
          x[i] = (i < n && xv == xv) ? xv : -INFINITY;
          xm = fmaxf(xm, x[i]);
        }
        const float mn = fmaxf(qm[nt], xm);
        if (mn != -INFINITY) {
          float s_acc = qs[nt] * fast_exp(qm[nt] - mn);
#pragma unroll
          for (int i = 0; i < 4; ++i) s_acc += fast_exp(x[i] - mn);
          qs[nt] = s_acc;
          qm[nt] = mn;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < n) win_update(bv[nt], bi[nt], (Score)z[i], c + i);
      }
    }
    }
#pragma unroll
    for (int s = 0; s < kRKMax; ++s) A[s] = An[s];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) bz[nt][i] = bzn[nt][i];
  }

  // merge the 4 lanes of each request row (lanes lr, lr + 16, lr + 32, lr + 48)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    unsigned long long key = bi[nt] >= 0 ? win_key_of(bv[nt], (uint32_t)bi[nt]) : 0ull;
    float m = qm[nt], s = qnan[nt] ? NAN : qs[nt];
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
      const unsigned long long k2 = __shfl_xor(key, off);
      key = k2 > key ? k2 : key;
      const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
      lse_merge(m, s, m2, s2);
    }
    if (lg == 0) {
      s_key[wave * NB + nt * 16 + lr] = key;
      s_qm[wave * NB + nt * 16 + lr] = m;
      s_qs[wave * NB + nt * 16 + lr] = s;
    }
  }
  __syncthreads();
  for (int i = tid; i < NB; i += 256) {
    const int b = b0 + i;
    if (draft_slot(a, b) < 0) continue;  // no winner and no partial for rows that are not served
    unsigned long long key = s_key[i];
    float m = s_qm[i], s = s_qs[i];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const unsigned long long k2 = s_key[w * NB + i];
      key = k2 > key ? k2 : key;
      lse_merge(m, s, s_qm[w * NB + i], s_qs[w * NB + i]);
    }
    if (key) atomicMax(&a.keys[key_index(k, a.B, b)], key);
    a.qpart[((size_t)k * a.B + b) * a.Gq + g] = make_float2(m, s);
  }
}

template <int NB, bool BBF16, bool CBF16, bool F64>
hipError_t launch_wave(const DraftStepArgs& a, int bt, hipStream_t st) {
  DraftStepArgs b = a;
  b.BT = bt;
  if (bt <= kDraftFastTiles)
    hipLaunchKernelGGL((draft_wave_kernel<NB, BBF16, CBF16, F64, true>), dim3(a.G * bt), dim3(256),
                       draft_wave_lds(NB, a.r), st, b);
  else
    hipLaunchKernelGGL((draft_wave_kernel<NB, BBF16, CBF16, F64, false>), dim3(a.G * bt), dim3(256),
                       draft_wave_lds(NB, a.r), st, b);
  return hipGetLastError();
}

template <int NB, bool F64>
hipError_t launch_wave_nb(const DraftStepArgs& a, int bt, hipStream_t st) {
  if (a.base_bf16)
    return a.cache_bf16 ? launch_wave<NB, true, true, F64>(a, bt, st) : launch_wave<NB, true, false, F64>(a, bt, st);
  return a.cache_bf16 ? launch_wave<NB, false, true, F64>(a, bt, st) : launch_wave<NB, false, false, F64>(a, bt, st);
}

// The tiled order of w2 that the step kernel reads with 1 KB loads. Tile t
// (rows 16 t .. 16 t + 15) takes 16 r consecutive elements; in it, rank
// slice s (elements 32 s .. 32 s + 31) takes 512, and the 8 elements at
// 8 l hold elements 32 s + 8 g .. + 7 of row 16 t + m, l = m + 16 g: lane
// l's piece of the A operand of the 16x16x32 MFMA for that slice. Rows past
// V are zero. One thread per 16-byte piece.
__global__ __launch_bounds__(256) void tile_w2_kernel(const uint16_t* __restrict__ w2, uint16_t* __restrict__ out,
                                                      int V, int r, long long n) {
  const long long c = (long long)blockIdx.x * 256 + threadIdx.x;
  if (c >= n) return;
  const int per_tile = 2 * r;  // 16-byte pieces per tile
  const long long t = c / per_tile;
  const int q = (int)(c - t * per_tile);
  const int l = q & 63;
  const long long v = t * 16 + (l & 15);
  u32x4 x = {0u, 0u, 0u, 0u};
  if (v < V) x = *(const u32x4*)(w2 + v * r + 32 * (q >> 6) + 8 * (l >> 4));
  *(u32x4*)(out + c * 8) = x;
}

}  // namespace

hipError_t launch_tile_w2(const uint16_t* w2, uint16_t* out, int V, int r, hipStream_t st) {
  const long long n = (long long)w2_tiled_elems(V, r) / 8;
  hipLaunchKernelGGL(tile_w2_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, w2, out, V, r, n);
  return hipGetLastError();
}

size_t draft_wave_lds(int NB, int r) {
  return (size_t)NB * (r + 8) * 2 + (size_t)NB * 4 + (size_t)4 * NB * 8 + (size_t)8 * NB * 4;
}

hipError_t launch_draft_wave(const DraftStepArgs& a, hipStream_t st) {
  if (a.r > 32 * kRKMax) return hipErrorNotSupported;
  const int nb = draft_nb(a.B, a.r);
  const int bt = (a.B + nb - 1) / nb;
  if (a.fp64)
    return nb == 16 ? launch_wave_nb<16, true>(a, bt, st) : launch_wave_nb<32, true>(a, bt, st);
  return nb == 16 ? launch_wave_nb<16, false>(a, bt, st) : launch_wave_nb<32, false>(a, bt, st);
}

}  // namespace mds
