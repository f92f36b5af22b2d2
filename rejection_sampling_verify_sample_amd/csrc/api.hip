// C ABI of the verify library: argument checks, workspace layout, launches.
// Every argument error is found here, on the host, before any HIP call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/spec_verify.h"
#include "params.hpp"

#define SPEC_EXPORT extern "C" __attribute__((visibility("default")))

namespace sv {
hipError_t launch_ngram_sample(const NgramSampleParams& P, bool bf16, hipStream_t stream);
hipError_t launch_pool_fill(int32_t* pool, int64_t n, hipStream_t stream);
hipError_t launch_pool_insert(const PoolParams& P, hipStream_t stream);
hipError_t launch_pool_lookup(const PoolParams& P, hipStream_t stream);
hipError_t launch_cache_fill(int32_t* cache, int64_t seq_elems, int64_t n, hipStream_t stream);
hipError_t launch_cache_insert(const CacheParams& P, hipStream_t stream);
hipError_t launch_cache_lookup(const CacheParams& P, hipStream_t stream);
hipError_t launch_sample(const SampleParams& P, bool bf16, bool filtered, int phases, hipStream_t stream);
hipError_t launch_greedy(const GreedyParams& P, bool bf16, hipStream_t stream);
hipError_t launch_philox(uint64_t seed, uint64_t round, int32_t B, int32_t K, float* out, hipStream_t stream);
hipError_t launch_row_stats(const RowStatsParams& P, bool bf16, hipStream_t stream);
}  // namespace sv

namespace {

using sv::GreedyLayout;
using sv::SampleLayout;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Most segments a row may be split into: bounds the partials the workspace holds.
int32_t seg_max(int64_t rows, int64_t V, int64_t cap = 64) {
  int64_t s = ceil_div(65536, std::max<int64_t>(rows, 1));
  s = std::min<int64_t>(s, cap);
  s = std::min<int64_t>(s, std::max<int64_t>(1, V / 256));
  return static_cast<int32_t>(std::max<int64_t>(s, 1));
}

// Segments per row: enough workgroups to fill the 256 CUs (target_blocks), but
// segments of at least `min_seg` elements. SPECVERIFY_S<n> overrides (tuning).
int32_t seg_choice(int64_t rows, int64_t V, int64_t target_blocks, int64_t min_seg, int32_t smax,
                   const char* env) {
  int64_t s = ceil_div(target_blocks, std::max<int64_t>(rows, 1));
  s = std::min<int64_t>(s, std::max<int64_t>(1, V / min_seg));
  if (const char* e = std::getenv(env)) {
    const long v = std::strtol(e, nullptr, 10);
    if (v > 0) s = v;
  }
  return static_cast<int32_t>(std::clamp<int64_t>(s, 1, smax));
}

bool sample_shape_ok(int32_t B, int32_t K, int32_t V) {
  if (B < 0 || K < 0 || K > SPEC_MAX_K || V < 1 || V > SPEC_MAX_V) return false;
  return static_cast<int64_t>(B) * (2 * static_cast<int64_t>(K) + 1) <= SPEC_MAX_ROWS;
}

// A pass-1 schedule: strictly increasing stage ends in [1, K], the last one K
// (K = 0: no stage).
bool stages_ok(int32_t K, const int32_t* ends, int32_t n) {
  if (K == 0) return n == 0;
  if (!ends || n < 1 || n > SPEC_MAX_STAGES) return false;
  int32_t prev = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (ends[i] <= prev || ends[i] > K) return false;
    prev = ends[i];
  }
  return prev == K;
}

bool greedy_shape_ok(int32_t B, int32_t G, int32_t N, int32_t V) {
  if (B < 0 || G < 1 || N < 2 || N > SPEC_MAX_K + 1 || V < 1 || V > SPEC_MAX_V) return false;
  if (static_cast<int64_t>(G) * N > sv::kMaxGreedyRowsPerBatch) return false;
  return static_cast<int64_t>(B) * G * N <= SPEC_MAX_ROWS;
}

SampleLayout sample_layout(int32_t B, int32_t K, int32_t V) {
  SampleLayout L{};
  const int64_t rows1 = static_cast<int64_t>(B) * 2 * K;
  L.S1max = seg_max(rows1, V);
  L.S2max = seg_max(B, V, 256);
  L.S1 = seg_choice(rows1, V, 1024, 8192, L.S1max, "SPECVERIFY_S1");
  L.S2 = seg_choice(B, V, sv::kMassThreads / sv::kMassBlock, 1024, L.S2max, "SPECVERIFY_S2");
  size_t off = 0;
  const size_t p1 = static_cast<size_t>(rows1) * L.S1max;
  L.off_p1m = off; off = align256(off + p1 * sizeof(float));
  L.off_p1s = off; off = align256(off + p1 * sizeof(double));
  L.off_p1x = off; off = align256(off + static_cast<size_t>(rows1) * sizeof(float));
  L.off_info_n = off; off = align256(off + static_cast<size_t>(B) * sizeof(int32_t));
  L.off_info_R = off; off = align256(off + static_cast<size_t>(B) * 2 * sizeof(float));
  L.off_info_S = off; off = align256(off + static_cast<size_t>(B) * 2 * sizeof(double));
  // pass-2 chunks: 64 16-byte vectors each, plus the head and the tail of the row
  // (at most ceil(V/256) + 2 for fp32 rows, fewer for bf16)
  L.NCmax = static_cast<int32_t>(ceil_div(V, 256) + 2);
  const size_t p2 = static_cast<size_t>(B) * L.NCmax;
  L.off_p2cm = off; off = align256(off + p2 * sizeof(float));
  L.off_p2cs = off; off = align256(off + p2 * sizeof(double));
  L.off_alive = off; off = align256(off + static_cast<size_t>(B) * sizeof(int32_t));
  // filtered entry point: one (reference, kept mass, threshold) per logit row
  const size_t rows = static_cast<size_t>(B) * (2 * static_cast<size_t>(K) + 1);
  L.off_fR = off; off = align256(off + rows * sizeof(float));
  L.off_fS = off; off = align256(off + rows * sizeof(double));
  L.off_fthr = off; off = align256(off + rows * sizeof(uint32_t));
  L.off_fflag = off; off = align256(off + rows * sizeof(uint32_t));
  L.off_infoT = off; off = align256(off + static_cast<size_t>(B) * 2 * sizeof(uint32_t));
  L.total = std::max<size_t>(off, 256);
  return L;
}


GreedyLayout greedy_layout(int32_t B, int32_t G, int32_t N, int32_t V) {
  GreedyLayout L{};
  const int64_t rows = static_cast<int64_t>(B) * G * N;
  L.S3max = seg_max(rows, V);
  L.S3 = seg_choice(rows, V, 3072, 8192, L.S3max, "SPECVERIFY_S3");
  size_t off = 0;
  const size_t p3 = static_cast<size_t>(rows) * L.S3max;
  L.off_p3v = off; off = align256(off + p3 * sizeof(float));
  L.off_p3i = off; off = align256(off + p3 * sizeof(int32_t));
  L.total = std::max<size_t>(off, 256);
  return L;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

}  // namespace

SPEC_EXPORT int32_t spec_abi_version(void) { return SPEC_ABI_VERSION; }

SPEC_EXPORT const char* spec_status_string(int32_t status) {
  switch (status) {
    case SPEC_OK: return "ok";
    case SPEC_ERR_NULL: return "a required pointer is NULL";
    case SPEC_ERR_SHAPE: return "a size is out of range";
    case SPEC_ERR_TEMPERATURE: return "temperature must be finite and > 0";
    case SPEC_ERR_DTYPE: return "unknown dtype";
    case SPEC_ERR_WORKSPACE: return "workspace too small";
    case SPEC_ERR_HIP: return "HIP launch failed";
    case SPEC_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case SPEC_ERR_PHASE: return "phase mask outside 1..15";
    case SPEC_ERR_FILTER_V: return "vocabulary too large for the filtered verify";
    case SPEC_ERR_STAGES: return "invalid stage schedule (strictly increasing ends in [1, K], the last K)";
    case SPEC_ERR_POOL: return "n-gram pool buffer smaller than spec_ngram_pool_bytes / spec_ngram_cache_bytes";
    default: return "unknown status";
  }
}

SPEC_EXPORT size_t spec_verify_sample_workspace_size(int32_t B, int32_t K, int32_t V) {
  if (!sample_shape_ok(B, K, V)) return 0;
  return sample_layout(B, K, V).total;
}

SPEC_EXPORT size_t spec_verify_sample_filtered_workspace_size(int32_t B, int32_t K, int32_t V) {
  if (!sample_shape_ok(B, K, V) || V > sv::kMaxFilterV) return 0;
  return sample_layout(B, K, V).total;
}

SPEC_EXPORT size_t spec_verify_greedy_workspace_size(int32_t B, int32_t G, int32_t N, int32_t V) {
  if (!greedy_shape_ok(B, G, N, V)) return 0;
  return greedy_layout(B, G, N, V).total;
}

namespace {
spec_status verify_sample_phases(const void* target_logits, const void* draft_logits, int32_t dtype,
                                 const int32_t* draft_tokens, const float* uniforms, int32_t B, int32_t K,
                                 int32_t V, float temperature, int32_t* out_tokens, int32_t* out_num_accepted,
                                 float* out_probs, void* workspace, size_t workspace_bytes, void* stream,
                                 int phases, bool filtered = false, const int32_t* top_k = nullptr,
                                 const float* top_p = nullptr, int32_t* out_kept = nullptr,
                                 const int32_t* stage_ends = nullptr, int32_t num_stages = -1,
                                 bool check_only = false) {
  if (!sample_shape_ok(B, K, V)) return SPEC_ERR_SHAPE;
  if (num_stages >= 0 && !stages_ok(K, stage_ends, num_stages)) return SPEC_ERR_STAGES;
  if (filtered && V > sv::kMaxFilterV) return SPEC_ERR_FILTER_V;
  if (phases < 1 || phases > sv::kPhaseAll) return SPEC_ERR_PHASE;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
  if (!(std::isfinite(temperature) && temperature > 0.f)) return SPEC_ERR_TEMPERATURE;
  const float c = static_cast<float>(1.4426950408889634074 / static_cast<double>(temperature));
  if (!std::isfinite(c)) return SPEC_ERR_TEMPERATURE;
  if (B == 0) return SPEC_OK;
  if (!target_logits || !uniforms || !out_tokens || !out_num_accepted || !workspace) return SPEC_ERR_NULL;
  if (K > 0 && (!draft_logits || !draft_tokens)) return SPEC_ERR_NULL;
  const size_t es = dtype == SPEC_BF16 ? 2 : 4;
  if (!aligned(target_logits, es) || (K > 0 && !aligned(draft_logits, es)) ||
      (K > 0 && !aligned(draft_tokens, 4)) || !aligned(uniforms, 4) || !aligned(out_tokens, 4) ||
      !aligned(out_num_accepted, 4) || (out_probs && !aligned(out_probs, 4)) || !aligned(workspace, 8))
    return SPEC_ERR_ALIGN;
  if ((top_k && !aligned(top_k, 4)) || (top_p && !aligned(top_p, 4)) || (out_kept && !aligned(out_kept, 4)))
    return SPEC_ERR_ALIGN;
  const SampleLayout L = sample_layout(B, K, V);
  if (workspace_bytes < L.total) return SPEC_ERR_WORKSPACE;
  if (check_only) return SPEC_OK;

  sv::SampleParams P{};
  P.target = target_logits;
  P.draft = draft_logits;
  P.tokens = draft_tokens;
  P.uniforms = uniforms;
  P.B = B;
  P.K = K;
  P.V = V;
  P.c = c;
  P.S1 = L.S1;
  P.S2 = L.S2;
  P.S1max = L.S1max;
  if (num_stages > 0) {
    // early exit: per-stage segment counts from the stage's own row count
    P.nstage = num_stages;
    int32_t a = 0;
    for (int32_t st = 0; st < num_stages; ++st) {
      P.stage_end[st] = stage_ends[st];
      // a later stage reads only the batch rows still walking: its segments are sized
      // as if a quarter of them were, so that few survivors still spread over the chip
      const int64_t rows = static_cast<int64_t>(B) * 2 * (stage_ends[st] - a);
      P.stage_S1[st] = seg_choice(st == 0 ? rows : ceil_div(rows, 4), V, 1024, 8192, L.S1max,
                                  st == 0 ? "SPECVERIFY_S1" : "SPECVERIFY_S1L");
      a = stage_ends[st];
    }
    P.probs_past_n = num_stages == 1;
  } else {
    P.nstage = 1;
    P.stage_end[0] = K;
    P.stage_S1[0] = L.S1;
    P.probs_past_n = 1;
  }
  P.out_tokens = out_tokens;
  P.out_n = out_num_accepted;
  P.out_probs = out_probs;
  P.p1_m = at<float>(workspace, L.off_p1m);
  P.p1_s = at<double>(workspace, L.off_p1s);
  P.info_n = at<int32_t>(workspace, L.off_info_n);
  P.info_R = at<float>(workspace, L.off_info_R);
  P.info_S = at<double>(workspace, L.off_info_S);
  P.NCmax = L.NCmax;
  P.p1_x = at<float>(workspace, L.off_p1x);
  P.p2_cm = at<float>(workspace, L.off_p2cm);
  P.p2_cs = at<double>(workspace, L.off_p2cs);
  P.stage_alive = at<int32_t>(workspace, L.off_alive);
  if (filtered) {
    P.top_k = top_k;
    P.top_p = top_p;
    P.out_kept = out_kept;
    P.f_R = at<float>(workspace, L.off_fR);
    P.f_S = at<double>(workspace, L.off_fS);
    P.f_thr = at<uint32_t>(workspace, L.off_fthr);
    P.f_flag = at<uint32_t>(workspace, L.off_fflag);
    // SPECVERIFY_FILTER=multi sends every row to the multi-pass select (tuning, testing)
    const char* fm = std::getenv("SPECVERIFY_FILTER");
    P.filt_multi = (fm && std::strcmp(fm, "multi") == 0) ? 1 : 0;
    P.info_T = at<uint32_t>(workspace, L.off_infoT);
  }
  const hipError_t e =
      sv::launch_sample(P, dtype == SPEC_BF16, filtered, phases, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}
}  // namespace

#define SPEC_SAMPLE_ARGS                                                                                     \
  const void *target_logits, const void *draft_logits, int32_t dtype, const int32_t *draft_tokens,           \
      const float *uniforms, int32_t B, int32_t K, int32_t V, float temperature, int32_t *out_tokens,        \
      int32_t *out_num_accepted, float *out_probs, void *workspace, size_t workspace_bytes, void *stream
#define SPEC_SAMPLE_FWD                                                                                      \
  target_logits, draft_logits, dtype, draft_tokens, uniforms, B, K, V, temperature, out_tokens,              \
      out_num_accepted, out_probs, workspace, workspace_bytes, stream

SPEC_EXPORT spec_status spec_verify_sample(SPEC_SAMPLE_ARGS) {
  return verify_sample_phases(SPEC_SAMPLE_FWD, sv::kPhaseAll);
}
// ---------------------------------------------------------------- the verify without a caller workspace

// The workspace of spec_verify_sample_noalloc: one fixed device array per GPU,
// held until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory: the device address comes from hipGetSymbolAddress, once per
// device, and only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (null on a HIP error).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

SPEC_EXPORT size_t spec_verify_sample_noalloc_max_bytes(void) { return SPEC_NOALLOC_SCRATCH_BYTES; }

SPEC_EXPORT spec_status spec_verify_sample_noalloc(const void* target_logits, const void* draft_logits,
                                                   int32_t dtype, const int32_t* draft_tokens,
                                                   const float* uniforms, int32_t B, int32_t K, int32_t V,
                                                   float temperature, int32_t* out_tokens,
                                                   int32_t* out_num_accepted, float* out_probs, void* stream) {
  // every argument check first, with a stand-in workspace, so that no HIP call precedes an argument error
  if (!sample_shape_ok(B, K, V)) return SPEC_ERR_SHAPE;
  if (sample_layout(B, K, V).total > SPEC_NOALLOC_SCRATCH_BYTES) return SPEC_ERR_WORKSPACE;
  static double probe_ws;  // a valid, aligned host pointer: only checked, never passed to a kernel
  const spec_status st = verify_sample_phases(target_logits, draft_logits, dtype, draft_tokens, uniforms, B, K, V,
                                              temperature, out_tokens, out_num_accepted, out_probs, &probe_ws,
                                              SPEC_NOALLOC_SCRATCH_BYTES, stream, sv::kPhaseAll, false, nullptr,
                                              nullptr, nullptr, nullptr, -1, /*check_only=*/true);
  if (st != SPEC_OK || B == 0) return st;
  void* ws = scratch_on_current_device();
  if (!ws) return SPEC_ERR_HIP;
  return verify_sample_phases(target_logits, draft_logits, dtype, draft_tokens, uniforms, B, K, V, temperature,
                              out_tokens, out_num_accepted, out_probs, ws, SPEC_NOALLOC_SCRATCH_BYTES, stream,
                              sv::kPhaseAll);
}

SPEC_EXPORT spec_status spec_verify_sample_phases(SPEC_SAMPLE_ARGS, int32_t phases) {
  return verify_sample_phases(SPEC_SAMPLE_FWD, phases);
}

SPEC_EXPORT spec_status spec_verify_sample_staged(SPEC_SAMPLE_ARGS, const int32_t* stage_ends, int32_t num_stages) {
  if (num_stages < 0) return SPEC_ERR_STAGES;
  return verify_sample_phases(SPEC_SAMPLE_FWD, sv::kPhaseAll, false, nullptr, nullptr, nullptr, stage_ends,
                              num_stages);
}

#define SPEC_FILTER_ARGS const int32_t *top_k, const float *top_p, int32_t *out_kept
SPEC_EXPORT spec_status spec_verify_sample_filtered(SPEC_SAMPLE_ARGS, SPEC_FILTER_ARGS) {
  return verify_sample_phases(SPEC_SAMPLE_FWD, sv::kPhaseAll, true, top_k, top_p, out_kept);
}
SPEC_EXPORT spec_status spec_verify_sample_filtered_phases(SPEC_SAMPLE_ARGS, SPEC_FILTER_ARGS, int32_t phases) {
  return verify_sample_phases(SPEC_SAMPLE_FWD, phases, true, top_k, top_p, out_kept);
}

SPEC_EXPORT spec_status spec_verify_greedy(const void* target_logits, int32_t dtype, const int32_t* cand_tokens,
                                           int32_t B, int32_t G, int32_t N, int32_t V, int32_t* out_tokens,
                                           int32_t* out_accept_len, int32_t* out_best_cand, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  if (!greedy_shape_ok(B, G, N, V)) return SPEC_ERR_SHAPE;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
  if (B == 0) return SPEC_OK;
  if (!target_logits || !cand_tokens || !out_tokens || !out_accept_len || !out_best_cand || !workspace)
    return SPEC_ERR_NULL;
  const size_t es = dtype == SPEC_BF16 ? 2 : 4;
  if (!aligned(target_logits, es) || !aligned(cand_tokens, 4) || !aligned(out_tokens, 4) ||
      !aligned(out_accept_len, 4) || !aligned(out_best_cand, 4) || !aligned(workspace, 8))
    return SPEC_ERR_ALIGN;
  const GreedyLayout L = greedy_layout(B, G, N, V);
  if (workspace_bytes < L.total) return SPEC_ERR_WORKSPACE;

  sv::GreedyParams P{};
  P.logits = target_logits;
  P.cand = cand_tokens;
  P.B = B;
  P.G = G;
  P.N = N;
  P.V = V;
  P.S3 = L.S3;
  // SPECVERIFY_SELECT=block keeps the workgroup select for every shape (tests, tuning)
  const char* sel = std::getenv("SPECVERIFY_SELECT");
  P.select_block = (sel && std::strcmp(sel, "block") == 0) ? 1 : 0;
  P.out_tokens = out_tokens;
  P.out_len = out_accept_len;
  P.out_best = out_best_cand;
  P.p3_v = at<float>(workspace, L.off_p3v);
  P.p3_i = at<int32_t>(workspace, L.off_p3i);
  const hipError_t e = sv::launch_greedy(P, dtype == SPEC_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

SPEC_EXPORT spec_status spec_fill_uniforms(uint64_t seed, uint64_t round, int32_t B, int32_t K, float* out,
                                           void* stream) {
  if (B < 0 || K < 0 || K > SPEC_MAX_K || static_cast<int64_t>(B) * (K + 1) > SPEC_MAX_ROWS)
    return SPEC_ERR_SHAPE;
  if (B == 0) return SPEC_OK;
  if (!out) return SPEC_ERR_NULL;
  if (!aligned(out, 4)) return SPEC_ERR_ALIGN;
  const hipError_t e = sv::launch_philox(seed, round, B, K, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

// ---------------------------------------------------------------- n-gram pool

namespace {

// Elements of a pool, or -1 for invalid sizes (or a size that does not fit in size_t).
int64_t pool_elems(int32_t B, int32_t V, int32_t G, int32_t N) {
  if (B < 0 || V < 1 || V > SPEC_MAX_V || G < 1 || G > SPEC_MAX_POOL_G || N < 2 || N > SPEC_MAX_POOL_N) return -1;
  const unsigned __int128 n = static_cast<unsigned __int128>(B) * V * G * (N - 1);
  if (n * 4 > static_cast<unsigned __int128>(INT64_MAX)) return -1;
  return static_cast<int64_t>(n);
}

spec_status pool_check(const void* pool, size_t pool_bytes, int32_t B, int32_t V, int32_t G, int32_t N) {
  const int64_t n = pool_elems(B, V, G, N);
  if (n < 0) return SPEC_ERR_SHAPE;
  if (B == 0) return SPEC_OK;
  if (!pool) return SPEC_ERR_NULL;
  if (!aligned(pool, 16)) return SPEC_ERR_ALIGN;
  if (pool_bytes < static_cast<size_t>(n) * 4) return SPEC_ERR_POOL;
  return SPEC_OK;
}

}  // namespace

SPEC_EXPORT size_t spec_ngram_pool_bytes(int32_t B, int32_t V, int32_t G, int32_t N) {
  const int64_t n = pool_elems(B, V, G, N);
  return n < 0 ? 0 : static_cast<size_t>(n) * 4;
}

SPEC_EXPORT spec_status spec_ngram_pool_init(void* pool, size_t pool_bytes, int32_t B, int32_t V, int32_t G,
                                             int32_t N, void* stream) {
  const spec_status st = pool_check(pool, pool_bytes, B, V, G, N);
  if (st != SPEC_OK || B == 0) return st;
  const hipError_t e = sv::launch_pool_fill(static_cast<int32_t*>(pool), pool_elems(B, V, G, N),
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

SPEC_EXPORT spec_status spec_ngram_pool_insert(void* pool, size_t pool_bytes, int32_t B, int32_t V, int32_t G,
                                               int32_t N, const int32_t* ngrams, int32_t W, int32_t* out_skipped,
                                               void* stream) {
  if (W < 0 || W > SPEC_MAX_POOL_W) return SPEC_ERR_SHAPE;
  const spec_status st = pool_check(pool, pool_bytes, B, V, G, N);
  if (st != SPEC_OK || B == 0) return st;
  if (W > 0 && !ngrams) return SPEC_ERR_NULL;
  if (!aligned(ngrams, 4) || !aligned(out_skipped, 4)) return SPEC_ERR_ALIGN;
  sv::PoolParams P{};
  P.pool = static_cast<int32_t*>(pool);
  P.B = B;
  P.V = V;
  P.G = G;
  P.N = N;
  P.W = W;
  P.ngrams = ngrams;
  P.out_skipped = out_skipped;
  const hipError_t e = sv::launch_pool_insert(P, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

SPEC_EXPORT spec_status spec_ngram_pool_lookup(const void* pool, size_t pool_bytes, int32_t B, int32_t V, int32_t G,
                                               int32_t N, const int32_t* last_tokens, int32_t* out_cand,
                                               int32_t* out_count, void* stream) {
  const spec_status st = pool_check(pool, pool_bytes, B, V, G, N);
  if (st != SPEC_OK || B == 0) return st;
  if (!last_tokens || !out_cand || !out_count) return SPEC_ERR_NULL;
  if (!aligned(last_tokens, 4) || !aligned(out_cand, 4) || !aligned(out_count, 4)) return SPEC_ERR_ALIGN;
  sv::PoolParams P{};
  P.pool = const_cast<int32_t*>(static_cast<const int32_t*>(pool));
  P.B = B;
  P.V = V;
  P.G = G;
  P.N = N;
  P.last = last_tokens;
  P.out_cand = out_cand;
  P.out_count = out_count;
  const hipError_t e = sv::launch_pool_lookup(P, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

// ---------------------------------------------------------------- hashed n-gram pool

namespace {

struct CacheGeometry {
  int64_t seq_elems = -1;  // int32 per sequence; -1 for invalid sizes
  int64_t elems = -1;      // int32 in all
  int32_t set_elems = 0;
  int32_t set_shift = 32;
};

CacheGeometry cache_geometry(int32_t B, int32_t sets, int32_t ways, int32_t G, int32_t N) {
  CacheGeometry g;
  if (B < 0 || sets < 1 || sets > SPEC_MAX_CACHE_SETS || (sets & (sets - 1)) != 0 || ways < 1 ||
      ways > SPEC_MAX_CACHE_WAYS || G < 1 || G > SPEC_MAX_POOL_G || N < 2 || N > SPEC_MAX_POOL_N)
    return g;
  const int64_t set_elems = 2 * static_cast<int64_t>(ways) + static_cast<int64_t>(ways) * G * (N - 1);
  const int64_t seq_elems = (4 + sets * set_elems + 3) / 4 * 4;
  const unsigned __int128 n = static_cast<unsigned __int128>(B) * static_cast<uint64_t>(seq_elems);
  if (n * 4 > static_cast<unsigned __int128>(INT64_MAX) || n * 4 > static_cast<unsigned __int128>(SIZE_MAX)) return g;
  g.seq_elems = seq_elems;
  g.elems = static_cast<int64_t>(n);
  g.set_elems = static_cast<int32_t>(set_elems);
  int log2 = 0;
  while ((1 << log2) < sets) ++log2;
  g.set_shift = 32 - log2;
  return g;
}

spec_status cache_check(const void* cache, size_t cache_bytes, const CacheGeometry& g, int32_t B) {
  if (g.elems < 0) return SPEC_ERR_SHAPE;
  if (B == 0) return SPEC_OK;
  if (!cache) return SPEC_ERR_NULL;
  if (!aligned(cache, 16)) return SPEC_ERR_ALIGN;
  if (cache_bytes < static_cast<size_t>(g.elems) * 4) return SPEC_ERR_POOL;
  return SPEC_OK;
}

sv::CacheParams cache_params(void* cache, const CacheGeometry& g, int32_t B, int32_t V, int32_t sets, int32_t ways,
                             int32_t G, int32_t N) {
  sv::CacheParams P{};
  P.cache = static_cast<int32_t*>(cache);
  P.seq_elems = g.seq_elems;
  P.set_elems = g.set_elems;
  P.set_shift = g.set_shift;
  P.B = B;
  P.V = V;
  P.sets = sets;
  P.ways = ways;
  P.G = G;
  P.N = N;
  return P;
}

}  // namespace

SPEC_EXPORT size_t spec_ngram_cache_bytes(int32_t B, int32_t sets, int32_t ways, int32_t G, int32_t N) {
  const CacheGeometry g = cache_geometry(B, sets, ways, G, N);
  return g.elems < 0 ? 0 : static_cast<size_t>(g.elems) * 4;
}

SPEC_EXPORT spec_status spec_ngram_cache_init(void* cache, size_t cache_bytes, int32_t B, int32_t sets, int32_t ways,
                                              int32_t G, int32_t N, void* stream) {
  const CacheGeometry g = cache_geometry(B, sets, ways, G, N);
  const spec_status st = cache_check(cache, cache_bytes, g, B);
  if (st != SPEC_OK || B == 0) return st;
  const hipError_t e = sv::launch_cache_fill(static_cast<int32_t*>(cache), g.seq_elems, g.elems,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

SPEC_EXPORT spec_status spec_ngram_cache_insert(void* cache, size_t cache_bytes, int32_t B, int32_t V, int32_t sets,
                                                int32_t ways, int32_t G, int32_t N, const int32_t* ngrams, int32_t W,
                                                int32_t* out_skipped, void* stream) {
  if (W < 0 || W > SPEC_MAX_POOL_W || V < 1 || V > SPEC_MAX_V) return SPEC_ERR_SHAPE;
  const CacheGeometry g = cache_geometry(B, sets, ways, G, N);
  const spec_status st = cache_check(cache, cache_bytes, g, B);
  if (st != SPEC_OK || B == 0) return st;
  if (W > 0 && !ngrams) return SPEC_ERR_NULL;
  if (!aligned(ngrams, 4) || !aligned(out_skipped, 4)) return SPEC_ERR_ALIGN;
  sv::CacheParams P = cache_params(cache, g, B, V, sets, ways, G, N);
  P.W = W;
  P.ngrams = ngrams;
  P.out_skipped = out_skipped;
  const hipError_t e = sv::launch_cache_insert(P, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

SPEC_EXPORT spec_status spec_ngram_cache_lookup(const void* cache, size_t cache_bytes, int32_t B, int32_t V,
                                                int32_t sets, int32_t ways, int32_t G, int32_t N,
                                                const int32_t* last_tokens, int32_t* out_cand, int32_t* out_count,
                                                void* stream) {
  if (V < 1 || V > SPEC_MAX_V) return SPEC_ERR_SHAPE;
  const CacheGeometry g = cache_geometry(B, sets, ways, G, N);
  const spec_status st = cache_check(cache, cache_bytes, g, B);
  if (st != SPEC_OK || B == 0) return st;
  if (!last_tokens || !out_cand || !out_count) return SPEC_ERR_NULL;
  if (!aligned(last_tokens, 4) || !aligned(out_cand, 4) || !aligned(out_count, 4)) return SPEC_ERR_ALIGN;
  sv::CacheParams P = cache_params(const_cast<void*>(cache), g, B, V, sets, ways, G, N);
  P.last = last_tokens;
  P.out_cand = out_cand;
  P.out_count = out_count;
  const hipError_t e = sv::launch_cache_lookup(P, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

// ---------------------------------------------------------------- sampling verify of one-hot n-grams

namespace {

bool ngram_sample_shape_ok(int32_t B, int32_t G, int32_t N, int32_t V) {
  if (B < 0 || G < 1 || G > SPEC_MAX_POOL_G || N < 2 || N > SPEC_MAX_K + 1 || V < 1 || V > SPEC_MAX_NGRAM_SAMPLE_V)
    return false;
  if (G * N > SPEC_MAX_NGRAM_SAMPLE_GN) return false;
  return static_cast<int64_t>(B) * G * N <= SPEC_MAX_ROWS;
}

struct NgsLayout {
  int32_t S1, S1max, nbmax;
  size_t off_m, off_s, off_gx, off_blk, total;
};

NgsLayout ngs_layout(int32_t B, int32_t G, int32_t N, int32_t V) {
  NgsLayout L{};
  const int64_t rows = static_cast<int64_t>(B) * G * N;
  L.S1max = seg_max(rows, V);
  L.S1 = seg_choice(rows, V, 1024, 8192, L.S1max, "SPECVERIFY_S4");
  size_t off = 0;
  const size_t p1 = static_cast<size_t>(rows) * L.S1max;
  L.off_m = off; off = align256(off + p1 * sizeof(float));
  L.off_s = off; off = align256(off + p1 * sizeof(double));
  L.off_gx = off; off = align256(off + static_cast<size_t>(B) * G * (N - 1) * G * sizeof(float));
  // blocks per row: at most ceil(V / (4 * kNgsBlkVecs)), fp32 holding 4 entries per vector
  L.nbmax = static_cast<int32_t>(ceil_div(V, 4 * sv::kNgsBlkVecs));
  L.off_blk = off; off = align256(off + static_cast<size_t>(rows) * L.nbmax * 2 * sizeof(float));
  L.total = std::max<size_t>(off, 256);
  return L;
}

}  // namespace

SPEC_EXPORT size_t spec_verify_ngram_sample_workspace_size(int32_t B, int32_t G, int32_t N, int32_t V) {
  if (!ngram_sample_shape_ok(B, G, N, V)) return 0;
  return ngs_layout(B, G, N, V).total;
}

SPEC_EXPORT spec_status spec_verify_ngram_sample(const void* target_logits, int32_t dtype, const int32_t* cand_tokens,
                                                 const float* uniforms, int32_t B, int32_t G, int32_t N, int32_t V,
                                                 float temperature, int32_t* out_tokens, int32_t* out_accept_len,
                                                 int32_t* out_rows, void* workspace, size_t workspace_bytes,
                                                 void* stream) {
  if (!ngram_sample_shape_ok(B, G, N, V)) return SPEC_ERR_SHAPE;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
  if (!(std::isfinite(temperature) && temperature > 0.f)) return SPEC_ERR_TEMPERATURE;
  const float c = static_cast<float>(1.4426950408889634074 / static_cast<double>(temperature));
  if (!std::isfinite(c)) return SPEC_ERR_TEMPERATURE;
  if (B == 0) return SPEC_OK;
  if (!target_logits || !cand_tokens || !uniforms || !out_tokens || !out_accept_len || !out_rows || !workspace)
    return SPEC_ERR_NULL;
  const size_t es = dtype == SPEC_BF16 ? 2 : 4;
  if (!aligned(target_logits, es) || !aligned(cand_tokens, 4) || !aligned(uniforms, 4) || !aligned(out_tokens, 4) ||
      !aligned(out_accept_len, 4) || !aligned(out_rows, 4) || !aligned(workspace, 8))
    return SPEC_ERR_ALIGN;
  const NgsLayout L = ngs_layout(B, G, N, V);
  if (workspace_bytes < L.total) return SPEC_ERR_WORKSPACE;
  sv::NgramSampleParams P{};
  P.logits = target_logits;
  P.cand = cand_tokens;
  P.uniforms = uniforms;
  P.B = B;
  P.G = G;
  P.N = N;
  P.V = V;
  P.c = c;
  P.S1 = L.S1;
  P.S1max = L.S1max;
  P.out_tokens = out_tokens;
  P.out_len = out_accept_len;
  P.out_rows = out_rows;
  P.p1_m = at<float>(workspace, L.off_m);
  P.p1_s = at<double>(workspace, L.off_s);
  P.gx = at<float>(workspace, L.off_gx);
  P.blk = at<float2>(workspace, L.off_blk);
  P.nbmax = L.nbmax;
  const hipError_t e = sv::launch_ngram_sample(P, dtype == SPEC_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

// ---------------------------------------------------------------- softmax statistics of rows

namespace {

struct RowStatsLayout {
  int32_t S;
  size_t off_m, off_s, total;
};

RowStatsLayout row_stats_layout(int32_t rows, int32_t V) {
  RowStatsLayout L{};
  L.S = seg_choice(rows, V, 1024, 8192, seg_max(rows, V), "SPECVERIFY_S1");
  const size_t p = static_cast<size_t>(rows) * seg_max(rows, V);
  size_t off = 0;
  L.off_m = off; off = align256(off + p * sizeof(float));
  L.off_s = off; off = align256(off + p * sizeof(double));
  L.total = std::max<size_t>(off, 256);
  return L;
}

bool row_stats_shape_ok(int32_t rows, int32_t V) {
  return rows >= 0 && rows <= SPEC_MAX_ROWS && V >= 1 && V <= SPEC_MAX_V;
}

}  // namespace

SPEC_EXPORT size_t spec_row_stats_workspace_size(int32_t rows, int32_t V) {
  if (!row_stats_shape_ok(rows, V)) return 0;
  return row_stats_layout(rows, V).total;
}

SPEC_EXPORT spec_status spec_row_stats(const void* logits, int32_t dtype, int32_t rows, int32_t V, float temperature,
                                       float* out_max, double* out_sum, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (!row_stats_shape_ok(rows, V)) return SPEC_ERR_SHAPE;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
  if (!(std::isfinite(temperature) && temperature > 0.f)) return SPEC_ERR_TEMPERATURE;
  const float c = static_cast<float>(1.4426950408889634074 / static_cast<double>(temperature));
  if (!std::isfinite(c)) return SPEC_ERR_TEMPERATURE;
  if (rows == 0) return SPEC_OK;
  if (!logits || !out_max || !out_sum || !workspace) return SPEC_ERR_NULL;
  const size_t es = dtype == SPEC_BF16 ? 2 : 4;
  if (!aligned(logits, es) || !aligned(out_max, 4) || !aligned(out_sum, 8) || !aligned(workspace, 8))
    return SPEC_ERR_ALIGN;
  const RowStatsLayout L = row_stats_layout(rows, V);
  if (workspace_bytes < L.total) return SPEC_ERR_WORKSPACE;
  sv::RowStatsParams P{};
  P.logits = logits;
  P.rows = rows;
  P.V = V;
  P.c = c;
  P.S = L.S;
  P.pm = at<float>(workspace, L.off_m);
  P.ps = at<double>(workspace, L.off_s);
  P.out_max = out_max;
  P.out_sum = out_sum;
  const hipError_t e = sv::launch_row_stats(P, dtype == SPEC_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}
