// extern "C" entry points of libmds.so: argument validation on the host,
// workspace layout, and the kernel sequence on the caller's stream. See
// include/mds.h for the contract of each call.
#include <mutex>
#include <string>

#include "../../include/mds.h"
#include "mds_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int ok() {
  g_last_error.clear();
  return MDS_OK;
}

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int kMaxBatch = 65535;
static_assert(kMaxBatch < mds::kVerifyMaxB, "the verify counter block must hold every request of a call");

int check_sizes(int B, int K, int V) {
  if (B < 1 || B > kMaxBatch) return fail(MDS_ERR_INVALID_ARG, "B must be in [1, 65535]");
  if (K < 1 || K > 32) return fail(MDS_ERR_INVALID_ARG, "K must be in [1, 32]");
  if (V < 2 || V >= (1 << 24)) return fail(MDS_ERR_INVALID_ARG, "V must be in [2, 2^24)");
  return MDS_OK;
}

int check_rank(int r) {
  if (r < 32 || r > 512) return fail(MDS_ERR_INVALID_ARG, "r must be in [32, 512]");
  if (r % 32) return fail(MDS_ERR_UNSUPPORTED, "r must be a multiple of 32");
  return MDS_OK;
}

// rows (b, k) of a [B, K, V] view must not overlap when written
bool rows_disjoint(int B, int K, int V, long long rs, long long ss) {
  if (rs < 0 || ss < 0) return false;
  if (B == 1 && K == 1) return true;
  if (B == 1) return ss >= V;
  if (K == 1) return rs >= V;
  return (ss >= V && rs >= (long long)(K - 1) * ss + V) || (rs >= V && ss >= (long long)(B - 1) * rs + V);
}

bool vec_ok(const void* p, int dtype, long long rs, long long ss) {
  return aligned(p, dtype == MDS_BF16 ? 8 : 16) && rs % 4 == 0 && ss % 4 == 0;
}

// Draft workspace: [status | kFixedKeys winner keys, one per 128-byte line,
// kept at zero between calls | the call's keys when K*B > kFixedKeys |
// per-slab (max, sum exp) partials K*B*kDraftMaxSlabs]. Sized without the
// device so the query needs no GPU.
struct DraftLayout {
  int nMT;
  bool fixed_keys;  // the keys sit in the zero-kept region
  size_t keys, qpart, total;
};

size_t fixed_keys_bytes() { return up((size_t)mds::kFixedKeys * 8 * mds::kKeyStride); }

DraftLayout draft_layout(int B, int K, int V) {
  DraftLayout L;
  L.nMT = (V + 15) / 16;
  size_t o = kAlign + fixed_keys_bytes();
  L.fixed_keys = (size_t)K * B <= (size_t)mds::kFixedKeys;
  if (L.fixed_keys) {
    L.keys = kAlign;
  } else {
    L.keys = o;
    o += up((size_t)K * B * 8 * mds::kKeyStride);
  }
  L.qpart = o;
  L.total = L.qpart + up((size_t)K * B * mds::kDraftMaxSlabs * sizeof(float2));
  return L;
}

struct VerifyLayout {
  int NC;
  size_t tpart, qpart, rowstat, qlse, tq, topp, req, total;
};

// [status block][per-request counters, fixed size][partials and per-row state]
VerifyLayout verify_layout(int B, int K, int V, bool top_p, bool has_lse) {
  VerifyLayout L;
  L.NC = (V + mds::kStatsChunk - 1) / mds::kStatsChunk;
  size_t o = mds::kVerifyCounterOffset + mds::kVerifyCounterBytes;
  L.tpart = o;
  o += up((size_t)B * (K + 1) * L.NC * 8);
  L.qpart = has_lse ? 0 : o;
  if (!has_lse) o += up((size_t)B * K * L.NC * 8);
  L.rowstat = o;
  o += up((size_t)B * (K + 1) * sizeof(mds::RowStat));
  L.qlse = o;
  o += up((size_t)B * K * sizeof(float));
  L.tq = o;
  o += up((size_t)B * K * 8);
  L.topp = top_p ? o : 0;
  if (top_p) o += up((size_t)B * (K + 1) * sizeof(mds::TopP));
  L.req = o;
  o += up((size_t)B * sizeof(mds::ReqState));
  L.total = o;
  return L;
}

void verify_workspace_args(mds::VerifyArgs& a, unsigned char* ws, const VerifyLayout& L, bool top_p, bool has_lse) {
  a.NC = L.NC;
  a.status = (uint32_t*)ws;
  a.cnt = (unsigned*)(ws + mds::kVerifyCounterOffset);
  a.tpart = (unsigned long long*)(ws + L.tpart);
  a.qpart = has_lse ? nullptr : (unsigned long long*)(ws + L.qpart);
  a.rowstat = (mds::RowStat*)(ws + L.rowstat);
  a.qlse = (float*)(ws + L.qlse);
  a.tq = (unsigned long long*)(ws + L.tq);
  a.topp = top_p ? (mds::TopP*)(ws + L.topp) : nullptr;
  a.req = (mds::ReqState*)(ws + L.req);
  a.rkey = (unsigned long long*)(ws + mds::kVerifyCounterOffset);
  a.decide = !top_p;
  a.NR = (a.V + mds::kResCols - 1) / mds::kResCols;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(MDS_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

// Request-state indexing of a call (all null for the plain entry points).
struct Indexing {
  const int32_t* idx_map = nullptr;
  const int32_t* row_map = nullptr;
  const int64_t* sample_pos = nullptr;
  int n_slots = 0, n_rows = 0;
  uint32_t flags = 0;
};

int check_indexing(const Indexing& ix) {
  if (ix.flags & ~(MDS_DRAFT_FP64_GUMBEL | MDS_DRAFT_W2_TILED)) return fail(MDS_ERR_INVALID_ARG, "unknown flag bits");
  if (!ix.idx_map) return MDS_OK;
  if (ix.n_slots < 1 || ix.n_rows < 1) return fail(MDS_ERR_INVALID_ARG, "n_slots and n_cache_rows must be >= 1");
  return MDS_OK;
}

int draft_impl(int B, int K, int V, int r, const void* base, int base_dtype, int64_t base_rs, int64_t base_ss,
               const void* w1, const void* w2, const int32_t* anchor, const int64_t* anchor_pos,
               const float* temperature, const int64_t* seeds, void* cache, int cache_dtype, int64_t cache_rs,
               int64_t cache_ss, int32_t* draft_tokens, float* draft_lse, void* workspace, size_t ws_bytes,
               void* stream, void* ev_begin, void* ev_end, int* n_launches, const Indexing& ix = Indexing(),
               uint32_t* status = nullptr, const mds::LmHeadArgs* lm = nullptr) {
  int rc;
  if ((rc = check_sizes(B, K, V)) || (rc = check_rank(r)) || (rc = check_indexing(ix))) return rc;
  if (!base || !w1 || !w2 || !anchor || (!anchor_pos && !ix.sample_pos) || !temperature || !seeds || !cache ||
      !draft_tokens || !workspace)
    return fail(MDS_ERR_INVALID_ARG, "a required pointer is NULL");
  if ((base_dtype != MDS_F32 && base_dtype != MDS_BF16) || (cache_dtype != MDS_F32 && cache_dtype != MDS_BF16))
    return fail(MDS_ERR_INVALID_ARG, "dtype must be MDS_F32 or MDS_BF16");
  if (base_rs < 0 || base_ss < 0) return fail(MDS_ERR_INVALID_ARG, "base strides must be >= 0");
  const int n_rows = ix.idx_map ? ix.n_rows : B;
  if (!rows_disjoint(n_rows, K, V, cache_rs, cache_ss))
    return fail(MDS_ERR_INVALID_ARG, "cache strides make rows overlap or are shorter than V");
  const bool fp64 = (ix.flags & MDS_DRAFT_FP64_GUMBEL) != 0;
  if (fp64 && r > 256) return fail(MDS_ERR_UNSUPPORTED, "the fp64 Gumbel option needs r <= 256");
  const bool tiled = (ix.flags & MDS_DRAFT_W2_TILED) != 0;
  if (tiled && r > 256) return fail(MDS_ERR_UNSUPPORTED, "tiled w2 needs r <= 256");
  if (!aligned(w1, 16) || !aligned(w2, 16)) return fail(MDS_ERR_INVALID_ARG, "w1 and w2 must be 16-byte aligned");
  if (!aligned(workspace, kAlign)) return fail(MDS_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const DraftLayout L = draft_layout(B, K, V);
  if (ws_bytes < L.total) return fail(MDS_ERR_WORKSPACE, "workspace too small for the draft loop");
  unsigned char* ws = (unsigned char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  mds::DraftStepArgs a{};
  a.B = B;
  a.K = K;
  a.V = V;
  a.r = r;
  a.nMT = L.nMT;
  a.base_bf16 = base_dtype == MDS_BF16;
  a.cache_bf16 = cache_dtype == MDS_BF16;
  a.vec_base = vec_ok(base, base_dtype, base_rs, base_ss);
  a.vec_cache = vec_ok(cache, cache_dtype, cache_rs, cache_ss);
  a.base = base;
  a.base_rs = base_rs;
  a.base_ss = base_ss;
  a.w1 = (const uint16_t*)w1;
  a.w2 = (const uint16_t*)w2;
  a.anchor = anchor;
  a.anchor_pos = (const long long*)anchor_pos;
  a.temp = temperature;
  a.seeds = (const long long*)seeds;
  a.cache = cache;
  a.cache_rs = cache_rs;
  a.cache_ss = cache_ss;
  a.keys = (unsigned long long*)(ws + L.keys);
  a.qpart = (float2*)(ws + L.qpart);
  a.status = status ? status : (uint32_t*)ws;
  a.idx_map = ix.idx_map;
  a.row_map = ix.idx_map ? ix.row_map : nullptr;
  a.sample_pos = (const long long*)ix.sample_pos;
  a.n_slots = ix.idx_map ? ix.n_slots : B;
  a.n_rows = n_rows;
  a.fp64 = fp64;
  a.w2_tiled = tiled;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "device query");
  const bool wave_kernel = r <= 256;
  const int nb = mds::draft_nb(B, r);
  a.G = wave_kernel ? mds::draft_wave_slabs(V, cus, (B + nb - 1) / nb) : mds::draft_slabs(V, cus);
  a.Gq = a.G;
  // lm: step 0 runs in the draft LM head's work-groups, one q partial each
  const int G0 = lm ? mds::lm_head_work_groups(*lm) : a.G;
  if (G0 > a.Gq) a.Gq = G0;
  // keys in the zero-kept region need no clearing
  if (!L.fixed_keys) {
    if ((e = mds::launch_draft_init(a.keys, K * B, st)) != hipSuccess) return hip_fail(e, "draft init launch");
  }
  if (ev_begin && (e = hipEventRecord((hipEvent_t)ev_begin, st)) != hipSuccess) return hip_fail(e, "event record");
  for (int k = 0; k < K; ++k) {
    a.k = k;
    if (k == 0 && lm)
      e = mds::launch_lm_head(*lm, st, &a);
    else
      e = wave_kernel ? mds::launch_draft_wave(a, st) : mds::launch_draft_step(a, st);
    if (e != hipSuccess) return hip_fail(e, "draft step launch");
  }
  if (ev_end && (e = hipEventRecord((hipEvent_t)ev_end, st)) != hipSuccess) return hip_fail(e, "event record");
  if (n_launches) *n_launches = K;
  mds::DraftFinalArgs f{B, K, a.G, a.keys, a.qpart, temperature, draft_tokens, draft_lse,
                        a.idx_map, a.row_map, a.n_slots, a.n_rows, a.fp64, G0, a.Gq};
  if ((e = mds::launch_draft_finalize(f, st)) != hipSuccess) return hip_fail(e, "draft finalize launch");
  return ok();
}

int verify_impl(int B, int K, int V, const float* target, int64_t target_row_stride, const void* cache,
                int cache_dtype, int64_t cache_req_stride, int64_t cache_step_stride, const float* draft_lse,
                const int32_t* draft_tokens, const float* temperature, const float* top_p, const int64_t* seeds,
                const int64_t* anchor_pos, int32_t* out_tokens, int32_t* num_accepted, void* workspace,
                size_t workspace_bytes, void* stream, const Indexing& ix) {
  int rc;
  if ((rc = check_sizes(B, K, V)) || (rc = check_indexing(ix))) return rc;
  if (!target || !cache || !draft_tokens || !temperature || !seeds || !anchor_pos || !out_tokens || !num_accepted ||
      !workspace)
    return fail(MDS_ERR_INVALID_ARG, "a required pointer is NULL");
  if (cache_dtype != MDS_F32 && cache_dtype != MDS_BF16)
    return fail(MDS_ERR_INVALID_ARG, "cache dtype must be MDS_F32 or MDS_BF16");
  if (target_row_stride < V) return fail(MDS_ERR_INVALID_ARG, "target_row_stride must be >= V");
  if (cache_req_stride < 0 || cache_step_stride < 0) return fail(MDS_ERR_INVALID_ARG, "cache strides must be >= 0");
  const int n_rows = ix.idx_map ? ix.n_rows : B;
  if (!aligned(workspace, kAlign)) return fail(MDS_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const VerifyLayout L = verify_layout(B, K, V, top_p != nullptr, draft_lse != nullptr);
  if (workspace_bytes < L.total) return fail(MDS_ERR_WORKSPACE, "workspace too small for verification");
  unsigned char* ws = (unsigned char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  mds::VerifyArgs a{};
  a.B = B;
  a.K = K;
  a.V = V;
  a.target = target;
  a.target_rs = target_row_stride;
  a.vec_target = aligned(target, 16) && target_row_stride % 4 == 0;
  a.cache = cache;
  a.cache_bf16 = cache_dtype == MDS_BF16;
  a.vec_cache = vec_ok(cache, cache_dtype, cache_req_stride, cache_step_stride);
  a.cache_rs = cache_req_stride;
  a.cache_ss = cache_step_stride;
  a.draft_lse = draft_lse;
  a.draft = draft_tokens;
  a.temp = temperature;
  a.top_p = top_p;
  a.seeds = (const long long*)seeds;
  a.anchor_pos = (const long long*)anchor_pos;
  a.out_tokens = out_tokens;
  a.num_accepted = num_accepted;
  verify_workspace_args(a, ws, L, top_p != nullptr, draft_lse != nullptr);
  a.idx_map = ix.idx_map;
  a.row_map = ix.idx_map ? ix.row_map : nullptr;
  a.n_slots = ix.idx_map ? ix.n_slots : B;
  a.n_rows = n_rows;
  hipError_t e;
  // The statistics pass only streams; one wave per request then combines
  // (and, without top-p, decides); with top-p the decision waits for the
  // top-p pass.
  if ((e = mds::launch_verify_stats(a, st)) != hipSuccess) return hip_fail(e, "verify stats launch");
  if ((e = mds::launch_combine(a, st)) != hipSuccess) return hip_fail(e, "combine launch");
  if (top_p) {
    if ((e = mds::launch_top_p(a, st)) != hipSuccess) return hip_fail(e, "top-p launch");
    if ((e = mds::launch_decide(a, st)) != hipSuccess) return hip_fail(e, "decide launch");
  }
  if ((e = mds::launch_residual(a, st)) != hipSuccess) return hip_fail(e, "residual launch");
  return ok();
}

// Top-k drafting workspace: [status | the draft workspace's zero-kept key
// region, untouched (so either kind of call may share a workspace) | chunk
// keys B*K*NC*topk u64 | candidate columns B*K*topk int32]
struct TopkLayout {
  int NC;
  size_t ckeys, cand, total;
};

TopkLayout topk_layout(int B, int K, int V, int topk) {
  TopkLayout L;
  L.NC = (V + mds::kTopkChunk - 1) / mds::kTopkChunk;
  L.ckeys = kAlign + fixed_keys_bytes();
  L.cand = L.ckeys + up((size_t)B * K * L.NC * topk * 8);
  L.total = L.cand + up((size_t)B * K * topk * 4);
  return L;
}

int check_topk(int B, int K, int V, int topk) {
  if (topk < 1 || topk > mds::kTopkMax || topk > V) return fail(MDS_ERR_INVALID_ARG, "topk must be in [1, min(256, V)]");
  const long long NC = (V + mds::kTopkChunk - 1) / mds::kTopkChunk;
  if (NC * topk > mds::kTopkMergeKeys)
    return fail(MDS_ERR_UNSUPPORTED, "ceil(V / 8192) * topk must be <= 7168");
  if (NC * B * K > 0x7FFFFFFFLL) return fail(MDS_ERR_UNSUPPORTED, "too many selection work-groups");
  return MDS_OK;
}

int topk_impl(int B, int K, int V, int r, int topk, const void* base, int base_dtype, int64_t base_rs,
              int64_t base_ss, const void* w1, const void* w2, const int32_t* anchor, const float* temperature,
              const int64_t* seeds, void* cache, int cache_dtype, int64_t cache_rs, int64_t cache_ss,
              int32_t* draft_tokens, float* draft_lse, void* workspace, size_t ws_bytes, void* stream,
              void* ev_begin, void* ev_end, const Indexing& ix) {
  int rc;
  if ((rc = check_sizes(B, K, V)) || (rc = check_rank(r)) || (rc = check_indexing(ix)) ||
      (rc = check_topk(B, K, V, topk)))
    return rc;
  if (ix.flags & MDS_DRAFT_W2_TILED) return fail(MDS_ERR_UNSUPPORTED, "top-k drafting reads row-major w2");
  if (!base || !w1 || !w2 || !anchor || !ix.sample_pos || !temperature || !seeds || !cache || !draft_tokens ||
      !workspace)
    return fail(MDS_ERR_INVALID_ARG, "a required pointer is NULL");
  if ((base_dtype != MDS_F32 && base_dtype != MDS_BF16) || (cache_dtype != MDS_F32 && cache_dtype != MDS_BF16))
    return fail(MDS_ERR_INVALID_ARG, "dtype must be MDS_F32 or MDS_BF16");
  if (base_rs < 0 || base_ss < 0) return fail(MDS_ERR_INVALID_ARG, "base strides must be >= 0");
  const int n_rows = ix.idx_map ? ix.n_rows : B;
  if (!rows_disjoint(n_rows, K, V, cache_rs, cache_ss))
    return fail(MDS_ERR_INVALID_ARG, "cache strides make rows overlap or are shorter than V");
  if (!aligned(w1, 16) || !aligned(w2, 16)) return fail(MDS_ERR_INVALID_ARG, "w1 and w2 must be 16-byte aligned");
  if (!aligned(workspace, kAlign)) return fail(MDS_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const TopkLayout L = topk_layout(B, K, V, topk);
  if (ws_bytes < L.total) return fail(MDS_ERR_WORKSPACE, "workspace too small for top-k drafting");
  unsigned char* ws = (unsigned char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  mds::TopkArgs a{};
  a.B = B;
  a.K = K;
  a.V = V;
  a.r = r;
  a.topk = topk;
  a.NC = L.NC;
  a.base_bf16 = base_dtype == MDS_BF16;
  a.cache_bf16 = cache_dtype == MDS_BF16;
  a.vec_base = vec_ok(base, base_dtype, base_rs, base_ss);
  a.vec_cache = vec_ok(cache, cache_dtype, cache_rs, cache_ss);
  a.base = base;
  a.base_rs = base_rs;
  a.base_ss = base_ss;
  a.w1 = (const uint16_t*)w1;
  a.w2 = (const uint16_t*)w2;
  a.anchor = anchor;
  a.temp = temperature;
  a.seeds = (const long long*)seeds;
  a.cache = cache;
  a.cache_rs = cache_rs;
  a.cache_ss = cache_ss;
  a.tokens = draft_tokens;
  a.lse = draft_lse;
  a.ckeys = (unsigned long long*)(ws + L.ckeys);
  a.cand = (int32_t*)(ws + L.cand);
  a.status = (uint32_t*)ws;
  a.idx_map = ix.idx_map;
  a.row_map = ix.idx_map ? ix.row_map : nullptr;
  a.sample_pos = (const long long*)ix.sample_pos;
  a.n_slots = ix.idx_map ? ix.n_slots : B;
  a.n_rows = n_rows;
  a.fp64 = (ix.flags & MDS_DRAFT_FP64_GUMBEL) != 0;
  hipError_t e;
  if (ev_begin && (e = hipEventRecord((hipEvent_t)ev_begin, st)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = mds::launch_topk_select(a, st)) != hipSuccess) return hip_fail(e, "top-k selection launch");
  if (ev_end && (e = hipEventRecord((hipEvent_t)ev_end, st)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = mds::launch_topk_merge(a, st)) != hipSuccess) return hip_fail(e, "top-k merge launch");
  if ((e = mds::launch_topk_chain(a, st)) != hipSuccess) return hip_fail(e, "top-k chain launch");
  return ok();
}

// ------------------------------------------------ allocation-free draft call --
// mds_markov_draft_loop_noalloc keeps its workspace in this array instead of
// a caller's buffer: status block | the zero-kept winner-key region | per-slab
// partials of at most kNoAllocMaxRows (request, step) rows. Every device the
// library runs on holds its own copy until the process ends. In host code
// `scratch` names a host-side stand-in: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr int kNoAllocMaxRows = 1024;  // K * B
constexpr size_t kNoAllocScratchBytes =
    kAlign + (size_t)mds::kFixedKeys * 8 * mds::kKeyStride + (size_t)kNoAllocMaxRows * mds::kDraftMaxSlabs * 8;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchState {
  unsigned char* ptr = nullptr;  // device address of this device's scratch
  bool keys_zero = false;        // its winner-key region is known to be zero
};
std::mutex g_scratch_mu;
ScratchState g_scratch[kMaxDevices];

// Checks the LM head's arguments and fills a (with the device's CU count).
int lm_head_args(int B, int K, int V, int H, const void* hidden, int64_t hidden_row_stride, const void* lm_head,
                 void* out, int out_dtype, int64_t out_req_stride, int64_t out_step_stride, mds::LmHeadArgs& a) {
  int rc;
  if ((rc = check_sizes(B, K, V))) return rc;
  if (H < 256 || H > 65536 || H % 256) return fail(MDS_ERR_UNSUPPORTED, "H must be a multiple of 256 in [256, 65536]");
  if (!hidden || !lm_head || !out) return fail(MDS_ERR_INVALID_ARG, "a required pointer is NULL");
  if (out_dtype != MDS_F32 && out_dtype != MDS_BF16) return fail(MDS_ERR_INVALID_ARG, "out dtype must be MDS_F32 or MDS_BF16");
  if (hidden_row_stride < H || hidden_row_stride % 8)
    return fail(MDS_ERR_INVALID_ARG, "hidden_row_stride must be >= H and a multiple of 8");
  if (!aligned(hidden, 16) || !aligned(lm_head, 16))
    return fail(MDS_ERR_INVALID_ARG, "hidden and lm_head must be 16-byte aligned");
  if (!rows_disjoint(B, K, V, out_req_stride, out_step_stride))
    return fail(MDS_ERR_INVALID_ARG, "out strides make rows overlap or are shorter than V");
  a = mds::LmHeadArgs{};
  a.M = B * K;
  a.K = K;
  a.V = V;
  a.H = H;
  a.hidden = (const uint16_t*)hidden;
  a.hidden_rs = hidden_row_stride;
  a.lm_head = (const uint16_t*)lm_head;
  a.out = out;
  a.out_rs = out_req_stride;
  a.out_ss = out_step_stride;
  a.out_bf16 = out_dtype == MDS_BF16;
  a.vec_out = vec_ok(out, out_dtype, out_req_stride, out_step_stride);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&a.cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "device query");
  return MDS_OK;
}

}  // namespace

namespace mds {
// Streaming kernel: two work-groups per CU (what its LDS and registers allow),
// fewer for small vocabularies, a multiple of the 8 XCDs when large.
int draft_slabs(int V, int cus) {
  const int nMT = (V + 15) / 16;
  int G = (nMT + kDraftMinTilesPerSlab - 1) / kDraftMinTilesPerSlab;
  const int cap = cus > 0 ? 2 * cus : kDraftMaxSlabs;
  if (G > cap) G = cap;
  if (G > kDraftMaxSlabs) G = kDraftMaxSlabs;
  if (G > 64) G &= ~7;
  return G < 1 ? 1 : G;
}

// Wave-independent kernel: one work-group per CU (measured best against two
// per CU for the V = 200064, B = 32 step), at least 8 tiles per slab. With up
// to kDraftFastTiles batch tiles the slabs of all tiles together fill the CUs
// once (V = 200064: B = 128 as 64 slabs x 4 tiles, 92 against 102 us per
// launch for 256 x 4 two per CU; B = 96 as 80 x 3, 75 against 83 us).
int draft_wave_slabs(int V, int cus, int bt) {
  const int nMT = (V + 15) / 16;
  int G = (nMT + kDraftMinTilesPerSlab - 1) / kDraftMinTilesPerSlab;
  const int cap = cus > 0 ? cus / (bt <= kDraftFastTiles ? bt : 1) : kDraftMaxSlabs;
  if (G > cap) G = cap;
  if (G > kDraftMaxSlabs) G = kDraftMaxSlabs;
  if (G > 64) G &= ~7;
  return G < 1 ? 1 : G;
}
}  // namespace mds

extern "C" {

int mds_abi_version(void) { return MDS_ABI_VERSION; }

const char* mds_status_string(int status) {
  switch (status) {
    case MDS_OK: return "ok";
    case MDS_ERR_INVALID_ARG: return "invalid argument";
    case MDS_ERR_UNSUPPORTED: return "unsupported argument";
    case MDS_ERR_WORKSPACE: return "workspace too small";
    case MDS_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* mds_last_error(void) { return g_last_error.c_str(); }

int mds_draft_workspace_bytes(int B, int K, int V, int r, size_t* out_bytes) {
  int rc;
  if ((rc = check_sizes(B, K, V)) || (rc = check_rank(r))) return rc;
  if (!out_bytes) return fail(MDS_ERR_INVALID_ARG, "out_bytes is NULL");
  *out_bytes = draft_layout(B, K, V).total;
  return ok();
}

int mds_markov_w2_tiled_bytes(int V, int r, size_t* out_bytes) {
  int rc;
  if ((rc = check_sizes(1, 1, V)) || (rc = check_rank(r))) return rc;
  if (!out_bytes) return fail(MDS_ERR_INVALID_ARG, "out_bytes is NULL");
  *out_bytes = mds::w2_tiled_elems(V, r) * 2;
  return ok();
}

int mds_tile_markov_w2(int V, int r, const void* w2, void* w2_tiled, size_t w2_tiled_bytes, void* stream) {
  int rc;
  if ((rc = check_sizes(1, 1, V)) || (rc = check_rank(r))) return rc;
  if (!w2 || !w2_tiled) return fail(MDS_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(w2, 16) || !aligned(w2_tiled, 16)) return fail(MDS_ERR_INVALID_ARG, "w2 and w2_tiled must be 16-byte aligned");
  const size_t need = mds::w2_tiled_elems(V, r) * 2;
  if (w2_tiled_bytes < need) return fail(MDS_ERR_INVALID_ARG, "w2_tiled is smaller than mds_markov_w2_tiled_bytes");
  const uintptr_t i0 = (uintptr_t)w2, i1 = i0 + (size_t)V * r * 2, o0 = (uintptr_t)w2_tiled, o1 = o0 + need;
  if (i0 < o1 && o0 < i1) return fail(MDS_ERR_INVALID_ARG, "w2 and w2_tiled overlap");
  const hipError_t e = mds::launch_tile_w2((const uint16_t*)w2, (uint16_t*)w2_tiled, V, r, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tile launch");
  return ok();
}

int mds_draft_topk_workspace_bytes(int B, int K, int V, int r, int topk, size_t* out_bytes) {
  int rc;
  if ((rc = check_sizes(B, K, V)) || (rc = check_rank(r)) || (rc = check_topk(B, K, V, topk))) return rc;
  if (!out_bytes) return fail(MDS_ERR_INVALID_ARG, "out_bytes is NULL");
  *out_bytes = topk_layout(B, K, V, topk).total;
  return ok();
}

int mds_markov_draft_loop_topk(int B, int K, int V, int r, int topk, const void* base, int base_dtype,
                               int64_t base_req_stride, int64_t base_step_stride, const void* w1, const void* w2,
                               const int32_t* anchor_tokens, const int32_t* idx_map, const int64_t* sample_pos,
                               int n_slots, const float* temperature, const int64_t* seeds,
                               const int32_t* row_mapping, int n_cache_rows, void* cache, int cache_dtype,
                               int64_t cache_row_stride, int64_t cache_step_stride, int32_t* draft_tokens,
                               float* draft_lse, uint32_t flags, void* workspace, size_t workspace_bytes,
                               void* stream, void* ev_begin, void* ev_end) {
  if (!idx_map && (row_mapping || n_slots < B || n_cache_rows < B))
    return fail(MDS_ERR_INVALID_ARG, "without idx_map: no row_mapping, n_slots >= B and n_cache_rows >= B");
  Indexing ix;
  ix.idx_map = idx_map;
  ix.row_map = row_mapping;
  ix.sample_pos = sample_pos;
  ix.n_slots = n_slots;
  ix.n_rows = n_cache_rows;
  ix.flags = flags;
  return topk_impl(B, K, V, r, topk, base, base_dtype, base_req_stride, base_step_stride, w1, w2, anchor_tokens,
                   temperature, seeds, cache, cache_dtype, cache_row_stride, cache_step_stride, draft_tokens,
                   draft_lse, workspace, workspace_bytes, stream, ev_begin, ev_end, ix);
}

int mds_draft_lm_head(int B, int K, int V, int H, const void* hidden, int64_t hidden_row_stride, const void* lm_head,
                      void* out, int out_dtype, int64_t out_req_stride, int64_t out_step_stride, void* stream,
                      void* ev_begin, void* ev_end) {
  mds::LmHeadArgs a;
  int rc;
  if ((rc = lm_head_args(B, K, V, H, hidden, hidden_row_stride, lm_head, out, out_dtype, out_req_stride,
                         out_step_stride, a)))
    return rc;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (ev_begin && (e = hipEventRecord((hipEvent_t)ev_begin, st)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = mds::launch_lm_head(a, st)) != hipSuccess) return hip_fail(e, "LM head launch");
  if (ev_end && (e = hipEventRecord((hipEvent_t)ev_end, st)) != hipSuccess) return hip_fail(e, "event record");
  return ok();
}

int mds_markov_draft_loop_from_hidden(int B, int K, int V, int r, int H, const void* hidden, int64_t hidden_row_stride,
                                      const void* lm_head, void* base, int base_dtype, int64_t base_req_stride,
                                      int64_t base_step_stride, const void* w1, const void* w2,
                                      const int32_t* anchor_tokens, const int64_t* anchor_pos,
                                      const float* temperature, const int64_t* seeds, void* cache, int cache_dtype,
                                      int64_t cache_req_stride, int64_t cache_step_stride, int32_t* draft_tokens,
                                      float* draft_lse, void* workspace, size_t workspace_bytes, void* stream,
                                      void* ev_begin, void* ev_end) {
  mds::LmHeadArgs lm;
  int rc;
  if ((rc = lm_head_args(B, K, V, H, hidden, hidden_row_stride, lm_head, base, base_dtype, base_req_stride,
                         base_step_stride, lm)))
    return rc;
  // step 0 inside the LM head's work-groups when one M tile holds every row
  // (B*K <= 256), the step kernel's batch tile holds every request (B <= 32),
  // the rank takes the streaming step kernel and the LM head's work-groups fit
  // the q partial slots; otherwise the LM head and the loop run one after
  // the other
  const bool fused = B <= 32 && B * K <= 256 && r <= 256 && mds::lm_head_work_groups(lm) <= mds::kDraftMaxSlabs;
  if (fused)
    return draft_impl(B, K, V, r, base, base_dtype, base_req_stride, base_step_stride, w1, w2, anchor_tokens,
                      anchor_pos, temperature, seeds, cache, cache_dtype, cache_req_stride, cache_step_stride,
                      draft_tokens, draft_lse, workspace, workspace_bytes, stream, ev_begin, ev_end, nullptr,
                      Indexing(), nullptr, &lm);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (ev_begin && (e = hipEventRecord((hipEvent_t)ev_begin, st)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = mds::launch_lm_head(lm, st)) != hipSuccess) return hip_fail(e, "LM head launch");
  return draft_impl(B, K, V, r, base, base_dtype, base_req_stride, base_step_stride, w1, w2, anchor_tokens,
                    anchor_pos, temperature, seeds, cache, cache_dtype, cache_req_stride, cache_step_stride,
                    draft_tokens, draft_lse, workspace, workspace_bytes, stream, nullptr, ev_end, nullptr);
}

int mds_verify_workspace_bytes(int B, int K, int V, int has_top_p, int has_draft_lse, size_t* out_bytes) {
  int rc;
  if ((rc = check_sizes(B, K, V))) return rc;
  if (!out_bytes) return fail(MDS_ERR_INVALID_ARG, "out_bytes is NULL");
  *out_bytes = verify_layout(B, K, V, has_top_p != 0, has_draft_lse != 0).total;
  return ok();
}

int mds_markov_draft_loop(int B, int K, int V, int r, const void* base, int base_dtype, int64_t base_req_stride,
                          int64_t base_step_stride, const void* w1, const void* w2, const int32_t* anchor_tokens,
                          const int64_t* anchor_pos, const float* temperature, const int64_t* seeds, void* cache,
                          int cache_dtype, int64_t cache_req_stride, int64_t cache_step_stride,
                          int32_t* draft_tokens, float* draft_lse, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return draft_impl(B, K, V, r, base, base_dtype, base_req_stride, base_step_stride, w1, w2, anchor_tokens,
                    anchor_pos, temperature, seeds, cache, cache_dtype, cache_req_stride, cache_step_stride,
                    draft_tokens, draft_lse, workspace, workspace_bytes, stream, nullptr, nullptr, nullptr);
}

int mds_markov_draft_loop_timed(int B, int K, int V, int r, const void* base, int base_dtype,
                                int64_t base_req_stride, int64_t base_step_stride, const void* w1, const void* w2,
                                const int32_t* anchor_tokens, const int64_t* anchor_pos, const float* temperature,
                                const int64_t* seeds, void* cache, int cache_dtype, int64_t cache_req_stride,
                                int64_t cache_step_stride, int32_t* draft_tokens, float* draft_lse, void* workspace,
                                size_t workspace_bytes, void* stream, void* ev_begin, void* ev_end,
                                int* n_step_launches) {
  if (!ev_begin || !ev_end) return fail(MDS_ERR_INVALID_ARG, "events must not be NULL");
  return draft_impl(B, K, V, r, base, base_dtype, base_req_stride, base_step_stride, w1, w2, anchor_tokens,
                    anchor_pos, temperature, seeds, cache, cache_dtype, cache_req_stride, cache_step_stride,
                    draft_tokens, draft_lse, workspace, workspace_bytes, stream, ev_begin, ev_end, n_step_launches);
}

int mds_rejection_verify(int B, int K, int V, const float* target, int64_t target_row_stride, const void* cache,
                         int cache_dtype, int64_t cache_req_stride, int64_t cache_step_stride,
                         const float* draft_lse, const int32_t* draft_tokens, const float* temperature,
                         const float* top_p, const int64_t* seeds, const int64_t* anchor_pos, int32_t* out_tokens,
                         int32_t* num_accepted, void* workspace, size_t workspace_bytes, void* stream) {
  return verify_impl(B, K, V, target, target_row_stride, cache, cache_dtype, cache_req_stride, cache_step_stride,
                     draft_lse, draft_tokens, temperature, top_p, seeds, anchor_pos, out_tokens, num_accepted,
                     workspace, workspace_bytes, stream, Indexing());
}

int mds_rejection_verify_indexed(int B, int K, int V, const float* target, int64_t target_row_stride,
                                 const void* cache, int cache_dtype, int64_t cache_row_stride,
                                 int64_t cache_step_stride, int n_cache_rows, const float* draft_lse,
                                 const int32_t* draft_tokens, const int32_t* idx_map, int n_slots,
                                 const float* temperature, const float* top_p, const int64_t* seeds,
                                 const int32_t* row_mapping, const int64_t* anchor_pos, int32_t* out_tokens,
                                 int32_t* num_accepted, void* workspace, size_t workspace_bytes, void* stream) {
  if (!idx_map) return fail(MDS_ERR_INVALID_ARG, "idx_map is NULL");
  Indexing ix;
  ix.idx_map = idx_map;
  ix.row_map = row_mapping;
  ix.n_slots = n_slots;
  ix.n_rows = n_cache_rows;
  return verify_impl(B, K, V, target, target_row_stride, cache, cache_dtype, cache_row_stride, cache_step_stride,
                     draft_lse, draft_tokens, temperature, top_p, seeds, anchor_pos, out_tokens, num_accepted,
                     workspace, workspace_bytes, stream, ix);
}

int mds_markov_draft_loop_ex(int B, int K, int V, int r, const void* base, int base_dtype, int64_t base_req_stride,
                             int64_t base_step_stride, const void* w1, const void* w2, const int32_t* anchor_tokens,
                             const int32_t* idx_map, const int64_t* sample_pos, int n_slots, const float* temperature,
                             const int64_t* seeds, const int32_t* row_mapping, int n_cache_rows, void* cache,
                             int cache_dtype, int64_t cache_row_stride, int64_t cache_step_stride,
                             int32_t* draft_tokens, float* draft_lse, uint32_t flags, void* workspace,
                             size_t workspace_bytes, void* stream, void* ev_begin, void* ev_end,
                             int* n_step_launches) {
  if (!sample_pos) return fail(MDS_ERR_INVALID_ARG, "sample_pos must not be NULL");
  if (!idx_map && (row_mapping || n_slots < B || n_cache_rows < B))
    return fail(MDS_ERR_INVALID_ARG, "without idx_map: no row_mapping, n_slots >= B and n_cache_rows >= B");
  Indexing ix;
  ix.idx_map = idx_map;
  ix.row_map = row_mapping;
  ix.sample_pos = sample_pos;
  ix.n_slots = n_slots;
  ix.n_rows = n_cache_rows;
  ix.flags = flags;
  return draft_impl(B, K, V, r, base, base_dtype, base_req_stride, base_step_stride, w1, w2, anchor_tokens, nullptr,
                    temperature, seeds, cache, cache_dtype, cache_row_stride, cache_step_stride, draft_tokens,
                    draft_lse, workspace, workspace_bytes, stream, ev_begin, ev_end, n_step_launches, ix);
}

int mds_debug_noise(int n, const int32_t* cols, int64_t seed, int64_t pos_key, uint32_t salt, uint32_t* words,
                    float* gumbel, void* stream) {
  if (n < 0) return fail(MDS_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return ok();
  if (!cols || !words || !gumbel) return fail(MDS_ERR_INVALID_ARG, "a required pointer is NULL");
  hipError_t e = mds::launch_debug_noise(n, cols, seed, pos_key, salt, words, gumbel, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "debug noise launch");
}

int mds_debug_top_p(int rows, int V, const float* target, int64_t row_stride, const float* temperature,
                    const float* top_p, uint32_t* tau, int32_t* cut, float* log_z, int32_t* on, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int rc;
  if ((rc = check_sizes(rows, 1, V))) return rc;
  if (!target || !temperature || !top_p || !tau || !cut || !log_z || !on || !workspace)
    return fail(MDS_ERR_INVALID_ARG, "a required pointer is NULL");
  if (row_stride < V) return fail(MDS_ERR_INVALID_ARG, "row_stride must be >= V");
  if (!aligned(workspace, kAlign)) return fail(MDS_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const VerifyLayout L = verify_layout(rows, 1, V, true, true);
  if (workspace_bytes < L.total) return fail(MDS_ERR_WORKSPACE, "workspace too small");
  unsigned char* ws = (unsigned char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  // every row is its own request with K = 0: row b*(K+1)+j is just b
  mds::VerifyArgs a{};
  a.B = rows;
  a.K = 0;
  a.V = V;
  a.target = target;
  a.target_rs = row_stride;
  a.vec_target = aligned(target, 16) && row_stride % 4 == 0;
  a.temp = temperature;
  a.top_p = top_p;
  verify_workspace_args(a, ws, L, true, true);
  hipError_t e;
  if ((e = mds::launch_verify_stats(a, st)) != hipSuccess) return hip_fail(e, "verify stats launch");
  if ((e = mds::launch_combine(a, st)) != hipSuccess) return hip_fail(e, "combine launch");
  if ((e = mds::launch_top_p(a, st)) != hipSuccess) return hip_fail(e, "top-p launch");
  if ((e = mds::launch_debug_top_p_out(rows, a.topp, tau, cut, log_z, on, st)) != hipSuccess)
    return hip_fail(e, "top-p output launch");
  return ok();
}

int mds_markov_draft_loop_noalloc(int B, int K, int V, int r, const void* base, int base_dtype,
                                  int64_t base_req_stride, int64_t base_step_stride, const void* w1, const void* w2,
                                  const int32_t* anchor_tokens, const int64_t* anchor_pos, const float* temperature,
                                  const int64_t* seeds, void* cache, int cache_dtype, int64_t cache_req_stride,
                                  int64_t cache_step_stride, int32_t* draft_tokens, float* draft_lse,
                                  uint32_t* status, void* stream) {
  int rc;
  if ((rc = check_sizes(B, K, V))) return rc;
  if ((long long)K * B > kNoAllocMaxRows)
    return fail(MDS_ERR_UNSUPPORTED, "mds_markov_draft_loop_noalloc needs K * B <= 1024 (its scratch is fixed)");
  if (!status) return fail(MDS_ERR_INVALID_ARG, "status is NULL");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "device query");
  if (dev < 0 || dev >= kMaxDevices) return fail(MDS_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchState& S = g_scratch[dev];
  if (!S.ptr) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return hip_fail(e, "scratch address");
    S.ptr = (unsigned char*)p;
  }
  hipStream_t st = (hipStream_t)stream;
  if (!S.keys_zero) {  // first call on this device, or a launch failed since the region was last known zero
    if ((e = mds::launch_draft_init((unsigned long long*)(S.ptr + kAlign), mds::kFixedKeys, st)) != hipSuccess)
      return hip_fail(e, "scratch clear launch");
    S.keys_zero = true;
  }
  rc = draft_impl(B, K, V, r, base, base_dtype, base_req_stride, base_step_stride, w1, w2, anchor_tokens, anchor_pos,
                  temperature, seeds, cache, cache_dtype, cache_req_stride, cache_step_stride, draft_tokens, draft_lse,
                  S.ptr, kNoAllocScratchBytes, stream, nullptr, nullptr, nullptr, Indexing(), status);
  if (rc == MDS_ERR_HIP) S.keys_zero = false;  // launched steps may have left winner keys behind
  return rc;
}

int mds_verify_slot_offsets(int b, size_t* counter_offset, size_t* key_offset) {
  if (b < 0 || b >= kMaxBatch) return fail(MDS_ERR_INVALID_ARG, "b must be in [0, 65535)");
  if (!counter_offset || !key_offset) return fail(MDS_ERR_INVALID_ARG, "a required pointer is NULL");
  *counter_offset = mds::kVerifyCounterOffset + (size_t)mds::verify_counter_index(b) * 4;
  *key_offset = mds::kVerifyCounterOffset + (size_t)mds::verify_key_index(b) * 8;
  return ok();
}

int mds_debug_gumbel(int n, const uint32_t* words, float* gumbel, void* stream) {
  if (n < 0) return fail(MDS_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return ok();
  if (!words || !gumbel) return fail(MDS_ERR_INVALID_ARG, "a required pointer is NULL");
  hipError_t e = mds::launch_debug_gumbel(n, words, gumbel, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "debug gumbel launch");
}

}  // extern "C"
