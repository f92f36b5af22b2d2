// Launch parameters, workspace layout and segment choices (host and device).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace sv {

// ---------------------------------------------------------------- sampling verify

constexpr int kMaxStages = 8;  // pass-1 stages of the early-exit verify

struct SampleParams {
  const void* target;      // [B, K+1, V]
  const void* draft;       // [B, K, V]
  const int32_t* tokens;   // [B, K]
  const float* uniforms;   // [B, K+1, 2]
  int32_t B, K, V;
  float c;                 // log2(e) / T, rounded to fp32
  int32_t S1, S2;          // segments per row in pass 1 (the widest stage) / workgroups per batch row in pass 2
  int32_t S1max;           // partial slots per logit row
  // Pass 1 in stages over the draft positions (early exit): stage s reads positions
  // [stage_end[s-1], stage_end[s]) with stage_S1[s] segments per row, only for batch
  // rows that accepted every earlier position. One stage: every position at once.
  int32_t nstage;
  int32_t stage_end[kMaxStages];
  int32_t stage_S1[kMaxStages];
  int32_t probs_past_n;    // out_probs after the first rejection: 1 = computed, 0 = NaN (not every row is read)
  int32_t* stage_alive;    // [B] 1 when the walk accepted every position before the current stage
  int32_t* out_tokens;     // [B, K+1]
  int32_t* out_n;          // [B]
  float* out_probs;        // [B, K, 2] or null
  // workspace (written by one kernel, read by a later one: no counters, no clearing)
  int32_t NCmax;           // chunk slots per batch row in p2_cm / p2_cs
  float* p1_m;             // [S1max][B*2K] segment maxima (row statistics), segment-major
  double* p1_s;            // [S1max][B*2K] segment sums against fl(m*c)
  float* p1_x;             // [B*2K] logit of the draft token in each row (NaN if the token is out of range)
  int32_t* info_n;         // [B] first rejection n, K when all accepted, -1 on a fault (accept decisions)
  float* info_R;           // [B, 2] reference exponents of target row n, draft row n
  double* info_S;          // [B, 2] softmax denominators of those rows
  float* p2_cm;            // [B*NCmax] per-chunk maximum (bonus draw)
  double* p2_cs;           // [B*NCmax] per-chunk mass (residual, or bonus mass against fl(max*c))
  // top-k / top-p filtering (filtered entry point only; null / 0 otherwise)
  const int32_t* top_k;    // [B] or null: k of each batch row (off unless 0 < k < V)
  const float* top_p;      // [B] or null: p of each batch row (off unless p < 1)
  int32_t* out_kept;       // [B, 2K+1] or null: kept entries of target rows 0..K, then draft rows 0..K-1
  float* f_R;              // [B*(2K+1)] reference exponent of each row's masses (same row order as out_kept)
  double* f_S;             // [B*(2K+1)] kept mass against f_R (0: the row has no finite logit)
  uint32_t* f_thr;         // [B*(2K+1)] a row keeps the entries whose order key is >= this
  uint32_t* f_flag;        // [B*(2K+1)] 1: the row needs the multi-pass select (written for every row)
  int32_t filt_multi;      // 1: every row takes the multi-pass select (no one-read path)
  uint32_t* info_T;        // [B, 2] thresholds of the rows the draw reads
};


// Kernels of the sampling verify, in stream order.
enum SamplePhase : int {
  kPhaseRowStats = 1,  // pass 1: online max / sum-exp of target and draft rows 0..K-1
  kPhaseAccept = 2,    // accept tests, first rejection, accepted prefix
  kPhaseMass = 4,      // pass 2: residual / bonus mass per segment of the row(s) the draw needs
  kPhaseDraw = 8,      // inverse-CDF search inside the chosen segment
  kPhaseAll = 15
};

// Threads per pass-2 workgroup. Pass 2 is sized to about 2^18 threads in all
// (SampleLayout::S2 workgroups per batch row).
#ifndef SV_MASS_BLOCK
#define SV_MASS_BLOCK 256
#endif
constexpr int kMassBlock = SV_MASS_BLOCK;
constexpr int kMassThreads = 1 << 18;

struct SampleLayout {
  int32_t S1, S2, S1max, S2max;
  int32_t NCmax;
  size_t off_p1m, off_p1s, off_p1x, off_info_n, off_info_R, off_info_S, off_p2cm, off_p2cs, off_alive;
  size_t off_fR, off_fS, off_fthr, off_fflag, off_infoT;  // filtered entry point only
  size_t total;
};

// Filtered verify: masses are summed in fixed point, round(m * 2^40) per entry with
// m <= 1, in 64-bit integers, so a row may hold at most 2^24 entries.
constexpr int64_t kMaxFilterV = int64_t(1) << 24;

// ---------------------------------------------------------------- softmax statistics of rows

struct RowStatsParams {
  const void* logits;      // [rows, V]
  int32_t rows, V;
  float c;                 // log2(e) / T, rounded to fp32
  int32_t S;               // segments per row
  float* pm;               // [S][rows] segment maxima
  double* ps;              // [S][rows] segment sums against fl(m*c)
  float* out_max;          // [rows]
  double* out_sum;         // [rows]
};

// ---------------------------------------------------------------- greedy verify

struct GreedyParams {
  const void* logits;      // [B, G, N, V]
  const int32_t* cand;     // [B, G, N-1]
  int32_t B, G, N, V;
  int32_t S3;
  int32_t select_block;    // 1: the workgroup select for every shape (SPECVERIFY_SELECT=block; tests)
  int32_t* out_tokens;     // [B, N]
  int32_t* out_len;        // [B]
  int32_t* out_best;       // [B]
  float* p3_v;             // [B*G*N*S3] segment maxima
  int32_t* p3_i;           // [B*G*N*S3] lowest index attaining them (-1 if none finite)
};

struct GreedyLayout {
  int32_t S3, S3max;
  size_t off_p3v, off_p3i, total;
};

constexpr int32_t kMaxGreedyRowsPerBatch = 8192;  // G*N: argmaxes of one batch row held in LDS

// ---------------------------------------------------------------- sampling verify of one-hot n-grams

struct NgramSampleParams {
  const void* logits;      // [B, G, N, V]
  const int32_t* cand;     // [B, G, N-1]
  const float* uniforms;   // [B, N, G+1]
  int32_t B, G, N, V;
  float c;                 // log2(e) / T, rounded to fp32
  int32_t S1, S1max;       // segments per row / partial slots per row
  int32_t* out_tokens;     // [B, N]
  int32_t* out_len;        // [B]
  int32_t* out_rows;       // [B]
  float* p1_m;             // [S1max][B*G*N] segment maxima, segment-major
  double* p1_s;            // [S1max][B*G*N] segment sums against fl(m*c)
  float* gx;               // [B*G*(N-1)*G] logit of candidate h's token at position i in row (g, i)
  float2* blk;             // [B*G*N*nbmax] per block of kNgsBlkVecs vectors: (R, sum of 2^(x*c - R))
  int32_t nbmax;           // block slots per row
};

// 16-byte vectors per block of the n-gram sampling verify's pass 1 (the macro
// exists for measured sweeps).
#ifndef SV_NGS_BLK_VECS
#define SV_NGS_BLK_VECS 256
#endif
constexpr int kNgsBlkVecs = SV_NGS_BLK_VECS;

// ---------------------------------------------------------------- n-gram pool

struct PoolParams {
  int32_t* pool;           // [B][V][G][N-1]
  int32_t B, V, G, N, W;
  const int32_t* ngrams;   // [B, W, N] (insert)
  int32_t* out_skipped;    // [B] or null (insert)
  const int32_t* last;     // [B] (lookup)
  int32_t* out_cand;       // [B, G, N-1] (lookup)
  int32_t* out_count;      // [B] (lookup)
};

// ---------------------------------------------------------------- hashed n-gram pool

struct CacheParams {
  int32_t* cache;          // B sequences of seq_elems int32: the clock, then `sets` sets
  int64_t seq_elems;       // int32 per sequence: 4 + sets * set_elems, rounded up to a multiple of 4
  int32_t set_elems;       // int32 per set: keys[ways], stamps[ways], slots[ways][G][N-1]
  int32_t set_shift;       // 32 - log2(sets); 32 when there is one set
  int32_t B, V, sets, ways, G, N, W;
  const int32_t* ngrams;   // [B, W, N] (insert)
  int32_t* out_skipped;    // [B] or null (insert)
  const int32_t* last;     // [B] (lookup)
  int32_t* out_cand;       // [B, G, N-1] (lookup)
  int32_t* out_count;      // [B] (lookup)
};

}  // namespace sv
