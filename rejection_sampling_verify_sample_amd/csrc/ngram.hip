// The n-gram pool that feeds the greedy verify with candidates (gfx950).
//
// Source: "Lookahead Decoding 完全拆解:Jacobi 迭代与 N-gram 池", sections "Lookahead
// 分支" (every step the window yields W new n-grams of length N, gathered into a
// pool), "N-gram 池与身份判定" (only n-grams whose first token equals the last
// generated token are verified) and "验证分支" (n-grams not adopted stay in the pool).
//
// Layout: one pool per sequence, direct-indexed by the first token (the key):
//   pool[b][key][slot][N-1] int32,
// a key's slots holding its continuations newest first, compacted, empty slots
// with -1 in every token. A key keeps its G most recently inserted distinct
// continuations; a continuation inserted again becomes the newest.
//
// Kernels:
//   k_pool_fill    marks every slot empty (16-byte stores, grid-stride).
//   k_pool_insert  one workgroup per sequence. The call's W n-grams are staged
//                  in LDS; every wave finds each n-gram's key itself, one per lane,
//                  and wave w takes n-grams w, w + 16, ... An n-gram whose key has
//                  no later valid n-gram in the call leads that key (distinct keys
//                  are distinct buckets, so no two waves touch one), and its wave
//                  rebuilds the key's bucket lane-parallel: the call's continuations of the key, each at
//                  its last occurrence, newest first, then the old slots they do
//                  not repeat, cut to G. This equals inserting the n-grams one by
//                  one in window order.
//   k_pool_lookup  one wave per sequence: the slots of the last token's key.
#include "../../include/spec_verify.h"
#include "common.hpp"
#include "params.hpp"
#include "pool_bucket.hpp"

namespace sv {

__device__ __forceinline__ int32_t* bucket(const PoolParams& P, int b, int key) {
  return P.pool + ((static_cast<int64_t>(b) * P.V + key) * P.G) * (P.N - 1);
}

// ---------------------------------------------------------------- fill

__global__ __launch_bounds__(256) void k_pool_fill(int32_t* pool, int64_t n) {
  const int64_t nvec = n / 4;
  u32x4* v = reinterpret_cast<u32x4*>(pool);
  const u32x4 empty = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nvec; i += stride) v[i] = empty;
  for (int64_t i = nvec * 4 + static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    pool[i] = -1;
}

// ---------------------------------------------------------------- insert

constexpr int kPoolWaves = 16;
constexpr int kPoolBlock = 64 * kPoolWaves;

struct PoolShared {
  int32_t ng[SPEC_MAX_POOL_W * SPEC_MAX_POOL_N];  // the call's n-grams, [W][N]
};

__global__ __launch_bounds__(kPoolBlock) void k_pool_insert(PoolParams P) {
  touch_kernargs(P);
  __shared__ PoolShared sh;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int W = P.W, N = P.N, G = P.G;
  for (int64_t task = blockIdx.x; task < P.B; task += gridDim.x) {
    const int b = static_cast<int>(task);
    for (int i = threadIdx.x; i < W * N; i += kPoolBlock) sh.ng[i] = P.ngrams[static_cast<int64_t>(b) * W * N + i];
    __syncthreads();
    // every wave finds each n-gram's key itself (lane w: n-gram w; -1 when skipped),
    // so the waves need no second barrier
    int myk = -1;
    if (lane < W) {
      bool valid = true;
      for (int i = 0; i < N; ++i) {
        const int t = sh.ng[lane * N + i];
        valid = valid && t >= 0 && t < P.V;
      }
      myk = valid ? sh.ng[lane * N] : -1;
    }
    if (wave == 0) {
      const uint64_t bad = __ballot(lane < W && myk < 0);
      if (lane == 0 && P.out_skipped) P.out_skipped[b] = __popcll(bad);
    }
    // wave `wave` takes n-grams wave, wave + 16, ...; an n-gram leads its key (and
    // its wave rebuilds the key's bucket) when no later n-gram of the call has that
    // key. Distinct keys are distinct buckets, so no two waves touch one.
    for (int li = wave; li < W; li += kPoolWaves) {
      const int key = __builtin_amdgcn_readlane(myk, li);
      if (key < 0) continue;  // skipped n-gram
      const uint64_t same = __ballot(lane < W && myk == key);  // the call's n-grams of this key
      if (same >> li >> 1) continue;                             // a later one leads
      rebuild_bucket(sh.ng, N, G, lane, same, bucket(P, b, key), true);
    }
    __syncthreads();  // LDS is reused by the next sequence
  }
}

// ---------------------------------------------------------------- lookup

__global__ __launch_bounds__(64) void k_pool_lookup(PoolParams P) {
  touch_kernargs(P);
  const int lane = threadIdx.x & 63;
  const int G = P.G, N = P.N;
  for (int64_t task = blockIdx.x; task < P.B; task += gridDim.x) {
    const int b = static_cast<int>(task);
    const int key = P.last[b];
    const bool in = key >= 0 && key < P.V;
    int32_t* oc = P.out_cand + static_cast<int64_t>(b) * G * (N - 1);
    bool full = false;
    if (lane < G) {
      const int32_t* bk = in ? bucket(P, b, key) + lane * (N - 1) : nullptr;
      for (int i = 0; i < N - 1; ++i) {
        const int32_t t = in ? bk[i] : -1;
        oc[lane * (N - 1) + i] = t;
        if (i == 0) full = t >= 0;
      }
    }
    const uint64_t fm = __ballot(full);
    if (lane == 0) P.out_count[b] = __popcll(fm);
  }
}

// ---------------------------------------------------------------- launch

static dim3 pool_grid(int64_t tasks) { return dim3(static_cast<uint32_t>(tasks < (1 << 20) ? tasks : (1 << 20))); }

hipError_t launch_pool_fill(int32_t* pool, int64_t n, hipStream_t stream) {
  const int64_t blocks = (n / 4 + 255) / 256;
  hipLaunchKernelGGL(k_pool_fill, pool_grid(blocks > 0 ? blocks : 1), dim3(256), 0, stream, pool, n);
  return hipGetLastError();
}

hipError_t launch_pool_insert(const PoolParams& P, hipStream_t stream) {
  hipLaunchKernelGGL(k_pool_insert, pool_grid(P.B), dim3(kPoolBlock), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_pool_lookup(const PoolParams& P, hipStream_t stream) {
  hipLaunchKernelGGL(k_pool_lookup, pool_grid(P.B), dim3(64), 0, stream, P);
  return hipGetLastError();
}

}  // namespace sv
