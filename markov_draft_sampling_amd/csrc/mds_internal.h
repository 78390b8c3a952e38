// Host/device interface between the C-ABI layer (abi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mds {

// ------------------------------------------------------------ draft loop --
constexpr int kDraftMaxSlabs = 1024;    // column slabs (work-groups) per batch tile and step
constexpr int kDraftMinTilesPerSlab = 8;  // 16-column tiles per slab, at least
// Winner keys sit one 128-byte line apart: every work-group of a step merges
// into every request's key, and atomics on keys sharing a line serialise.
constexpr int kKeyStride = 16;  // u64 words from one (step, request) key to the next
__host__ __device__ __forceinline__ size_t key_index(int k, int B, int b) {
  return ((size_t)k * B + b) * kKeyStride;
}
// Every draft and top-k workspace starts with a region of kFixedKeys winner
// keys that each call leaves at zero (the finalize pass clears the keys it
// reads, and nothing else writes there), so a streaming call with
// K * B <= kFixedKeys needs no clearing launch whatever the workspace held
// before; larger calls keep theirs elsewhere and clear them first.
constexpr int kFixedKeys = 4096;

struct DraftStepArgs {
  int B, K, V, r, k, G, nMT, BT;
  int base_bf16, cache_bf16, vec_base, vec_cache;
  const void* base;
  long long base_rs, base_ss;
  const uint16_t* w1;
  const uint16_t* w2;
  const int32_t* anchor;
  const long long* anchor_pos;
  const float* temp;
  const long long* seeds;
  void* cache;
  long long cache_rs, cache_ss;
  unsigned long long* keys;  // [K][B] winner keys at key_index(k, B, b)
  float2* qpart;             // [K][B][Gq] (max, sum exp) of cache / T per slab
  int Gq;                    // partials per (step, request) row of qpart (>= G)
  uint32_t* status;
  int zero;                  // always 0 (an offset the compiler cannot fold)
  // request-state indexing (all null / B for the plain call)
  const int32_t* idx_map;    // [B][K] state slot of row b at step k, < 0 inert; null: slot = b
  const int32_t* row_map;    // [n_slots] cache row of a slot; null: row = slot
  const long long* sample_pos;  // [B][K] predicted position P (draw keyed by P - 1); null: anchor_pos + k
  int n_slots, n_rows;
  int fp64;                  // fp64 Gumbel option: float64 scores, 64-bit keys of the fp64 format
  int w2_tiled;              // w2 in the 16-row tile order of tile_w2_kernel (step kernels for r <= 256 only)
};

struct DraftFinalArgs {
  int B, K, G;               // G: q partials of each step after the first
  unsigned long long* keys;  // read, then cleared
  const float2* qpart;       // [K][B][Gq]
  const float* temp;
  int32_t* tokens;
  float* lse;
  const int32_t* idx_map;
  const int32_t* row_map;
  int n_slots, n_rows;
  int fp64;  // keys in the fp64 format
  int G0;    // q partials of step 0
  int Gq;    // partials per (step, request) row of qpart
};

// The state slot of batch row b at draft step k, or -1 when the row is inert
// there (past the batch, a negative slot, or a slot / cache row out of range,
// the last two flagged in the status word).
__device__ __forceinline__ int draft_slot(const int32_t* idx_map, const int32_t* row_map, int B, int K, int n_slots,
                                          int n_rows, uint32_t* status, int b, int k) {
  if (b >= B) return -1;
  if (!idx_map) return b;
  const int s = idx_map[(size_t)b * K + k];
  if (s < 0) return -1;
  const int row = s < n_slots ? (row_map ? row_map[s] : s) : -1;
  if (row < 0 || row >= n_rows) {
    if (status) atomicOr(status, 8u);
    return -1;
  }
  return s;
}
__device__ __forceinline__ int draft_slot(const DraftStepArgs& a, int b) {
  return draft_slot(a.idx_map, a.row_map, a.B, a.K, a.n_slots, a.n_rows, a.status, b, a.k);
}
// cache row of a live slot s of batch row b
__device__ __forceinline__ int draft_cache_row(const DraftStepArgs& a, int b, int s) {
  return !a.idx_map ? b : (a.row_map ? a.row_map[s] : s);
}
// key of the draw of batch row b (< B) at step k: the position before the predicted token
__device__ __forceinline__ long long draft_pos_key(const DraftStepArgs& a, int b) {
  return a.sample_pos ? a.sample_pos[(size_t)b * a.K + a.k] - 1 : a.anchor_pos[b] + a.k;
}

int draft_nb(int B, int r);
int draft_slabs(int V, int cus);
// Batch tiles up to which the wave kernel runs one work-group per CU over
// all of them (the fixed-count fast loop needs the CU to itself).
constexpr int kDraftFastTiles = 4;
int draft_wave_slabs(int V, int cus, int bt);
hipError_t launch_draft_init(unsigned long long* keys, int n, hipStream_t st);
hipError_t launch_draft_step(const DraftStepArgs& a, hipStream_t st);
// Wave-independent streaming step (rank <= 256); hipErrorNotSupported
// (nothing launched) for a larger rank.
size_t draft_wave_lds(int NB, int r);
// w2 [V, r] row-major -> the tiled order the step kernels read with 1 KB loads
// (w2_tiled_elems(V, r) bf16 elements, rows past V zero)
__host__ __forceinline__ size_t w2_tiled_elems(int V, int r) { return (size_t)((V + 15) / 16) * 16 * r; }
hipError_t launch_tile_w2(const uint16_t* w2, uint16_t* out, int V, int r, hipStream_t st);
hipError_t launch_draft_wave(const DraftStepArgs& a, hipStream_t st);
hipError_t launch_draft_finalize(const DraftFinalArgs& a, hipStream_t st);

// ------------------------------------------------- top-k Markov drafting --
constexpr int kTopkMax = 256;             // candidates per row, at most
constexpr int kTopkChunk = 8192;          // base-logit columns per selection work-group
constexpr int kTopkMergeKeys = 7168;      // chunk keys a row's merge holds on chip (chunks * k)

struct TopkArgs {
  int B, K, V, r, topk, NC;  // NC = chunks per row
  int base_bf16, cache_bf16, vec_base, vec_cache;
  const void* base;
  long long base_rs, base_ss;
  const uint16_t* w1;
  const uint16_t* w2;
  const int32_t* anchor;
  const float* temp;
  const long long* seeds;
  void* cache;
  long long cache_rs, cache_ss;
  int32_t* tokens;
  float* lse;
  unsigned long long* ckeys;  // [B*K][NC][topk] each chunk's k largest selection keys (0 = none)
  int32_t* cand;              // [B*K][topk] a row's candidate columns, increasing
  uint32_t* status;
  const int32_t* idx_map;     // as in DraftStepArgs
  const int32_t* row_map;
  const long long* sample_pos;  // [B][K], required
  int n_slots, n_rows;
  int fp64;
};
size_t topk_chunk_lds(int topk);

// ------------------------------------------------------ draft LM head --
struct LmHeadArgs {
  int M, K, V, H;             // rows M = B*K (row m = b*K + k), vocabulary, hidden size (a multiple of 256)
  const uint16_t* hidden;     // [M][H] bf16, row stride hidden_rs elements
  long long hidden_rs;
  const uint16_t* lm_head;    // [V][H] bf16, contiguous
  void* out;                  // row (b, k) at b*out_rs + k*out_ss elements, float32 or bf16
  long long out_rs, out_ss;
  int out_bf16, vec_out;
  int cus;                    // compute units of the device (the launch splits its last partial round)
};
// step0 non-null: the LM head also runs step 0 of the draft loop (M = B*K
// <= 256, B <= 32, rank <= 256, the fp32 Gumbel): the step-0 logit rows are not
// stored, and the q partials of step 0 take lm_head_work_groups(a) slots
hipError_t launch_lm_head(const LmHeadArgs& a, hipStream_t st, const DraftStepArgs* step0 = nullptr);
int lm_head_work_groups(const LmHeadArgs& a);
hipError_t launch_topk_select(const TopkArgs& a, hipStream_t st);
hipError_t launch_topk_merge(const TopkArgs& a, hipStream_t st);
hipError_t launch_topk_chain(const TopkArgs& a, hipStream_t st);

// ---------------------------------------------------------- verification --
// columns per statistics block: the pages' sampler uses 8192-column blocks;
// the block size only orders the summation, and 4096 measured faster here
// (37.1 against 38.7 us for the pass at V = 200064, B = 32, K = 7)
constexpr int kStatsChunk = 4096;

// Partials of one (row, block) are published as one 64-bit word: for a
// sampled row (max, sum exp) of x = logit / T as two floats (max in the low
// half), for a greedy row the winner key of the raw logits.
struct RowStat {  // combined statistics of one target row
  float m;        // max of x = logit / T (sampled rows)
  float lz;       // log of sum exp(x - m); NaN if the row held NaN
  unsigned long long key;  // winner key of the raw logits (greedy rows)
};

struct TopP {  // kept set of one target row: ord(t) > tau, or == tau and id <= cut
  uint32_t tau;
  int cut;
  float log_z;  // log of the kept mass sum exp(x - m)
  int on;
};

struct ReqState {  // the accept decision of one request, read by the residual draw
  int n_acc;   // accepted drafts; the final token is drawn from row n_acc
  int mode;    // 0 bonus from p_K, 1 residual of row n_acc, 2 greedy (done), 3 residual empty -> p
  float M, LZ; // row n_acc: max of logit / T and log of its (kept) mass
  float LQ;    // draft row n_acc: log sum exp of cache / T (mode 1)
  int pad;
  TopP tp;     // kept set of row n_acc (tp.on == 0 when no top-p)
};

// The kVerifyCounterBytes after the verify workspace's 256-byte status block
// hold one arrival counter and one 64-bit winner key per request. Every call
// leaves them at zero, so they sit at a fixed offset whatever (B, K, V) a
// call uses. The block is 2048 lines of 512 bytes: request b uses line
// b mod 2048, its counter is 32-bit word b / 2048 of the line's first 128
// bytes, its key 64-bit word b / 2048 of bytes [128, 384). With b < 65536
// (the largest batch a call accepts) b / 2048 < 32, so no key overlaps a
// counter and nothing leaves the line. Requests b and b + 2048 i share a
// line; any other two do not (many work-groups bumping counters of one line
// serialise on it).
constexpr size_t kVerifyCounterOffset = 256;
constexpr int kVerifyLines = 2048;
constexpr int kVerifyLineBytes = 512;
constexpr size_t kVerifyCounterBytes = (size_t)kVerifyLines * kVerifyLineBytes;
constexpr int kVerifyMaxB = kVerifyLines * 32;  // b / 2048 < 32
// index in 32-bit words from the start of the block
__host__ __device__ constexpr int verify_counter_index(int b) {
  return (b & (kVerifyLines - 1)) * (kVerifyLineBytes / 4) + (b >> 11);
}
// index in 64-bit words from the start of the block
__host__ __device__ constexpr int verify_key_index(int b) {
  return (b & (kVerifyLines - 1)) * (kVerifyLineBytes / 8) + 16 + (b >> 11);
}

struct VerifyArgs {
  int B, K, V, NC;
  const float* target;
  long long target_rs;
  const void* cache;
  int cache_bf16, vec_cache;
  long long cache_rs, cache_ss;
  const float* draft_lse;  // [B*K], or null: then the statistics pass also reads the cache rows
  const int32_t* draft;
  const float* temp;
  const float* top_p;
  const long long* seeds;
  const long long* anchor_pos;
  int32_t* out_tokens;
  int32_t* num_accepted;
  unsigned long long* tpart;  // [NC][B*(K+1)] packed partials of the target rows
  unsigned long long* qpart;  // [NC][B*K] packed partials of the cache rows (draft_lse null)
  RowStat* rowstat;           // [B*(K+1)]
  float* qlse;                // [B*K] draft log-normalisers (copied or combined)
  unsigned long long* tq;     // [B*K] (target, cache) logits at the draft tokens, packed
  TopP* topp;                 // [B*(K+1)] or null
  ReqState* req;              // [B]
  unsigned long long* rkey;   // winner keys of the final draws, at verify_key_index(b)
  unsigned* cnt;              // [B] arrival counters (zero between calls)
  uint32_t* status;
  int vec_target;
  int decide;                 // the statistics pass also takes the accept decision (no top-p)
  int NR;                     // residual blocks per request (kResCols columns each)
  // request-state indexing (null / B for the plain call)
  const int32_t* idx_map;     // [B] state slot of request b, < 0 padding; null: slot = b
  const int32_t* row_map;     // [n_slots] cache row of a slot; null: row = slot
  int n_slots, n_rows;
};

// The state slot of request b, or -1 for a padding request (a negative slot,
// or a slot / cache row out of range, the latter flagged in the status word).
__device__ __forceinline__ int verify_slot(const VerifyArgs& a, int b) {
  if (!a.idx_map) return b;
  const int s = a.idx_map[b];
  if (s < 0) return -1;
  const int row = s < a.n_slots ? (a.row_map ? a.row_map[s] : s) : -1;
  if (row < 0 || row >= a.n_rows) {
    if (a.status) atomicOr(a.status, 8u);
    return -1;
  }
  return s;
}
__device__ __forceinline__ int verify_cache_row(const VerifyArgs& a, int b, int s) {
  return !a.idx_map ? b : (a.row_map ? a.row_map[s] : s);
}

constexpr int kResCols = 2048;  // columns per residual work-group

// The statistics pass; launch_combine must follow it (it also decides when
// a.decide, i.e. without top-p).
hipError_t launch_verify_stats(const VerifyArgs& a, hipStream_t st);
hipError_t launch_combine(const VerifyArgs& a, hipStream_t st);
hipError_t launch_top_p(const VerifyArgs& a, hipStream_t st);
hipError_t launch_decide(const VerifyArgs& a, hipStream_t st);
hipError_t launch_residual(const VerifyArgs& a, hipStream_t st);

// ----------------------------------------------------------------- debug --
hipError_t launch_debug_noise(int n, const int32_t* cols, long long seed, long long pos, uint32_t salt,
                              uint32_t* words, float* g, hipStream_t st);
hipError_t launch_debug_gumbel(int n, const uint32_t* words, float* g, hipStream_t st);
hipError_t launch_debug_top_p_out(int rows, const TopP* tp, uint32_t* tau, int32_t* cut, float* log_z, int32_t* on,
                                  hipStream_t st);

}  // namespace mds
