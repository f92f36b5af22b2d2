// Launch parameters, workspace layout and segment choices (host and device).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace sv {

// ---------------------------------------------------------------- sampling verify

struct SampleParams {
  const void* target;      // [B, K+1, V]
  const void* draft;       // [B, K, V]
  const int32_t* tokens;   // [B, K]
  const float* uniforms;   // [B, K+1, 2]
  int32_t B, K, V;
  float c;                 // log2(e) / T, rounded to fp32
  int32_t S1, S2;          // segments per row in pass 1 / pass 2
  int32_t* out_tokens;     // [B, K+1]
  int32_t* out_n;          // [B]
  float* out_probs;        // [B, K, 2] or null
  // workspace
  float* p1_m;             // [B*2K*S1] segment maxima
  double* p1_s;            // [B*2K*S1] segment sums against fl(m*c)
  uint32_t* cnt1;          // [B] pass-1 arrivals
  int32_t* info_n;         // [B] first rejection n, K when all accepted, -1 on a fault
  float* info_R;           // [B, 2] reference exponents of target row n, draft row n
  double* info_S;          // [B, 2] softmax denominators of those rows
  float* p2_m;             // [B*S2]
  double* p2_s;            // [B*S2]
  uint32_t* cnt2;          // [B] pass-2 arrivals
};

struct SampleLayout {
  int32_t S1, S2, S1max, S2max;
  size_t off_p1m, off_p1s, off_cnt1, off_info_n, off_info_R, off_info_S, off_p2m, off_p2s, off_cnt2, total;
};

// ---------------------------------------------------------------- greedy verify

struct GreedyParams {
  const void* logits;      // [B, G, N, V]
  const int32_t* cand;     // [B, G, N-1]
  int32_t B, G, N, V;
  int32_t S3;
  int32_t* out_tokens;     // [B, N]
  int32_t* out_len;        // [B]
  int32_t* out_best;       // [B]
  float* p3_v;             // [B*G*N*S3] segment maxima
  int32_t* p3_i;           // [B*G*N*S3] lowest index attaining them (-1 if none finite)
  uint32_t* cnt3;          // [B]
};

struct GreedyLayout {
  int32_t S3, S3max;
  size_t off_p3v, off_p3i, off_cnt3, total;
};

constexpr int32_t kMaxGreedyRowsPerBatch = 8192;  // G*N: argmaxes of one batch row held in LDS

}  // namespace sv
