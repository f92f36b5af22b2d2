// Softmax statistics of logit rows (gfx950): the row maximum m and the denominator
// S = sum_v 2^(fl(x_v * c - fl(m * c))), c = fl(log2(e) / T), so that
// p_v = 2^(x_v * c - fl(m * c)) / S is row v's softmax at temperature T
// ("Speculative Decoding —— LLM推理优化技术（一）" §4: the temperature divides the
// logits; kwkr.cn/news/620797 notes §3.2: probabilities in fp32 at least).
//
// The same streaming reduction as the verify's pass 1 (rowstats.hpp): one
// workgroup per (row, segment) keeps an online (max, sum) over 16-byte
// nontemporal loads, and a second kernel merges a row's segment partials.
#include "../../include/spec_verify.h"
#include "common.hpp"
#include "params.hpp"
#include "rowstats.hpp"

namespace sv {

template <typename T>
__global__ __launch_bounds__(kRowBlock) void k_row_stats_partial(RowStatsParams P) {
  touch_kernargs(P);
  const int64_t ntask = static_cast<int64_t>(P.rows) * P.S;
  for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) {
    int64_t r;
    int seg;
    split_task(task, P.S, r, seg);
    const T* row = static_cast<const T*>(P.logits) + r * P.V;
    Online o;
    o.init();
    online_segment<kRowBlock>(row, P.V, seg, P.S, P.c, o);
    float m;
    double s;
    block_online<kRowBlock>(o, P.c, m, s);
    if (threadIdx.x == 0) {
      P.pm[seg * static_cast<int64_t>(P.rows) + r] = m;
      P.ps[seg * static_cast<int64_t>(P.rows) + r] = s;
    }
    __syncthreads();  // shared memory is reused by the next task
  }
}

constexpr int kMergeBlock = 256;

__global__ __launch_bounds__(kMergeBlock) void k_row_stats_merge(RowStatsParams P) {
  touch_kernargs(P);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kMergeBlock;
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * kMergeBlock + threadIdx.x; r < P.rows; r += stride) {
    float M;
    double S;
    merge_partials(P.pm + r, P.ps + r, P.rows, P.S, P.c, M, S);
    P.out_max[r] = M;
    P.out_sum[r] = S;
  }
}

hipError_t launch_row_stats(const RowStatsParams& P, bool bf16, hipStream_t stream) {
  const int64_t tasks = static_cast<int64_t>(P.rows) * P.S;
  const dim3 grid(static_cast<uint32_t>(tasks < (1 << 20) ? tasks : (1 << 20)));
  if (bf16)
    hipLaunchKernelGGL(k_row_stats_partial<bf16_t>, grid, dim3(kRowBlock), 0, stream, P);
  else
    hipLaunchKernelGGL(k_row_stats_partial<float>, grid, dim3(kRowBlock), 0, stream, P);
  const int64_t mg = (static_cast<int64_t>(P.rows) + kMergeBlock - 1) / kMergeBlock;
  hipLaunchKernelGGL(k_row_stats_merge, dim3(static_cast<uint32_t>(mg < 4096 ? mg : 4096)), dim3(kMergeBlock), 0,
                     stream, P);
  return hipGetLastError();
}

}  // namespace sv
