// The hashed n-gram pool: the pool of ngram.hip held in a bounded per-sequence hash
// table, so its memory follows what it holds instead of the vocabulary (gfx950).
//
// Source: "Lookahead Decoding 完全拆解:Jacobi 迭代与 N-gram 池", sections "Lookahead
// 分支", "N-gram 池与身份判定" and "验证分支", as for the direct pool. The page leaves
// the pool's capacity open; this table bounds it:
//   * a sequence has `sets` sets (a power of two) of `ways` entries; a key lives in
//     the set named by the top log2(sets) bits of key * 2654435769 mod 2^32 (Knuth's
//     multiplicative hashing; the constant is floor(2^32 / golden ratio));
//   * every inserted n-gram takes the next value of its sequence's clock and a key's
//     stamp is the value of its newest n-gram; a new key in a full set takes the
//     entry of the key with the oldest stamp, continuations and all;
//   * within a key the direct pool's rule holds (pool_bucket.hpp).
//
// Layout, per sequence (seq_elems int32, a multiple of 4, so every sequence starts
// 16-byte aligned):
//   [0]                    the clock (uint32); [1..3] zero
//   [4 + s * set_elems]    set s: keys[ways] int32 (-1: empty way),
//                          stamps[ways] uint32,
//                          slots[ways][G][N-1] int32 (newest first, -1 empty).
// A lookup reads one set's keys with one load per lane and then one way's slots.
//
// Kernels:
//   k_cache_fill    every clock 0, everything else -1 (16-byte stores).
//   k_cache_insert  one workgroup per sequence. The call's n-grams are staged in LDS;
//                   the wave that takes a set's last n-gram of the call runs that set
//                   (n-grams of one set never meet another wave). One lane per way,
//                   it replays the set's n-grams in window order on the set's keys
//                   (a hit refreshes the stamp, a miss takes an empty way, else the
//                   way with the oldest stamp), remembering in which n-gram each
//                   way's key arrived. Then it rebuilds each way the call touched
//                   from that n-gram on, keeping the old slots only for a key held
//                   before the call that never left it, and writes keys and stamps.
//   k_cache_lookup  one wave per sequence: the home set's keys one per lane, then the
//                   slots of the way that holds the token.
#include "../../include/spec_verify.h"
#include "common.hpp"
#include "params.hpp"
#include "pool_bucket.hpp"

namespace sv {

constexpr uint32_t kGoldenMul = 2654435769u;  // floor(2^32 / golden ratio)

__device__ __forceinline__ int home_set(const CacheParams& P, int key) {
  if (P.set_shift >= 32) return 0;
  return static_cast<int>((static_cast<uint32_t>(key) * kGoldenMul) >> P.set_shift);
}

__device__ __forceinline__ int32_t* cache_seq(const CacheParams& P, int b) {
  return P.cache + static_cast<int64_t>(b) * P.seq_elems;
}

__device__ __forceinline__ int32_t* cache_set(const CacheParams& P, int32_t* seq, int s) {
  return seq + 4 + static_cast<int64_t>(s) * P.set_elems;
}

// ---------------------------------------------------------------- fill

__global__ __launch_bounds__(256) void k_cache_fill(int32_t* cache, int64_t seq_vecs, int64_t nvec) {
  u32x4* v = reinterpret_cast<u32x4*>(cache);
  const u32x4 empty = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  const u32x4 header = {0u, 0u, 0u, 0u};
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nvec; i += stride)
    v[i] = (i % seq_vecs == 0) ? header : empty;
}

// ---------------------------------------------------------------- insert

constexpr int kCacheWaves = 16;
constexpr int kCacheBlock = 64 * kCacheWaves;

struct CacheShared {
  int32_t ng[SPEC_MAX_POOL_W * SPEC_MAX_POOL_N];  // the call's n-grams, [W][N]
};

// The way (lane < ways) whose stamp is the oldest: the largest age new_clock - stamp,
// taken modulo 2^32; the lowest such lane. Whole wave.
__device__ __forceinline__ int oldest_way(uint32_t wstamp, uint32_t new_clock, int lane, int ways) {
  const uint32_t age = lane < ways ? new_clock - wstamp : 0u;
  uint32_t m = age;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), o, 64)));
  const uint64_t at = __ballot(lane < ways && age == m);
  return __ffsll(static_cast<unsigned long long>(at)) - 1;
}

__global__ __launch_bounds__(kCacheBlock) void k_cache_insert(CacheParams P) {
  touch_kernargs(P);
  __shared__ CacheShared sh;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int W = P.W, N = P.N, G = P.G, ways = P.ways;
  for (int64_t task = blockIdx.x; task < P.B; task += gridDim.x) {
    const int b = static_cast<int>(task);
    int32_t* seq = cache_seq(P, b);
    // every thread reads the clock before the barrier; it is written after the last one
    const uint32_t clock = static_cast<uint32_t>(seq[0]);
    for (int i = threadIdx.x; i < W * N; i += kCacheBlock) sh.ng[i] = P.ngrams[static_cast<int64_t>(b) * W * N + i];
    __syncthreads();
    // every wave finds each n-gram's key and set itself (lane w: n-gram w; -1 when skipped)
    int myk = -1, mys = -1;
    if (lane < W) {
      bool valid = true;
      for (int i = 0; i < N; ++i) {
        const int t = sh.ng[lane * N + i];
        valid = valid && t >= 0 && t < P.V;
      }
      if (valid) {
        myk = sh.ng[lane * N];
        mys = home_set(P, myk);
      }
    }
    const uint64_t validm = __ballot(myk >= 0);
    const uint32_t new_clock = clock + static_cast<uint32_t>(__popcll(validm));
    if (wave == 0 && lane == 0 && P.out_skipped) P.out_skipped[b] = W - __popcll(validm);
    // wave `wave` takes n-grams wave, wave + 16, ...; the wave holding a set's last
    // n-gram of the call runs that set
    for (int li = wave; li < W; li += kCacheWaves) {
      const int s = __builtin_amdgcn_readlane(mys, li);
      if (s < 0) continue;                          // skipped n-gram
      const uint64_t inset = __ballot(mys == s);    // the call's n-grams of this set
      if (inset >> li >> 1) continue;               // a later one leads
      int32_t* set = cache_set(P, seq, s);
      int32_t* keys = set;
      uint32_t* stamps = reinterpret_cast<uint32_t*>(set + ways);
      int32_t* slots = set + 2 * ways;
      int wkey = -1;
      uint32_t wstamp = 0u;
      int wborn = -1;  // the n-gram of this call in which the way's key arrived; -1: held before
      bool wtouched = false;
      if (lane < ways) {
        wkey = keys[lane];
        wstamp = stamps[lane];
      }
      // replay the set's n-grams in window order
      for (uint64_t m = inset; m != 0ull; m &= m - 1ull) {
        const int j = __ffsll(static_cast<unsigned long long>(m)) - 1;
        const int k = __builtin_amdgcn_readlane(myk, j);
        const uint32_t st = clock + static_cast<uint32_t>(__popcll(validm & ((1ull << j) - 1ull)));
        const uint64_t hit = __ballot(lane < ways && wkey == k);
        int t;
        if (hit) {
          t = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        } else {
          const uint64_t empty = __ballot(lane < ways && wkey < 0);
          t = empty ? __ffsll(static_cast<unsigned long long>(empty)) - 1 : oldest_way(wstamp, new_clock, lane, ways);
          if (lane == t) {
            wkey = k;
            wborn = j;
          }
        }
        if (lane == t) {
          wstamp = st;
          wtouched = true;
        }
      }
      // rebuild every touched way from the n-gram its key arrived in
      for (uint64_t tm = __ballot(wtouched); tm != 0ull; tm &= tm - 1ull) {
        const int t = __ffsll(static_cast<unsigned long long>(tm)) - 1;
        const int key = __builtin_amdgcn_readlane(wkey, t);
        const int born = __builtin_amdgcn_readlane(wborn, t);
        uint64_t same = __ballot(myk == key);
        if (born >= 0) same &= ~((1ull << born) - 1ull);
        rebuild_bucket(sh.ng, N, G, lane, same, slots + static_cast<int64_t>(t) * G * (N - 1), born < 0);
      }
      if (wtouched) {
        keys[lane] = wkey;
        stamps[lane] = wstamp;
      }
    }
    __syncthreads();  // the clock has been read everywhere; LDS is reused by the next sequence
    if (threadIdx.x == 0) seq[0] = static_cast<int32_t>(new_clock);
  }
}

// ---------------------------------------------------------------- lookup

__global__ __launch_bounds__(64) void k_cache_lookup(CacheParams P) {
  touch_kernargs(P);
  const int lane = threadIdx.x & 63;
  const int G = P.G, N = P.N, ways = P.ways;
  for (int64_t task = blockIdx.x; task < P.B; task += gridDim.x) {
    const int b = static_cast<int>(task);
    const int key = P.last[b];
    int way = -1;
    const int32_t* slots = nullptr;
    if (key >= 0 && key < P.V) {
      const int32_t* set = cache_set(P, cache_seq(P, b), home_set(P, key));
      const int32_t wk = lane < ways ? set[lane] : -1;
      const uint64_t hit = __ballot(lane < ways && wk == key);
      if (hit) {
        way = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        slots = set + 2 * ways + static_cast<int64_t>(way) * G * (N - 1);
      }
    }
    int32_t* oc = P.out_cand + static_cast<int64_t>(b) * G * (N - 1);
    bool full = false;
    if (lane < G) {
      for (int i = 0; i < N - 1; ++i) {
        const int32_t t = way >= 0 ? slots[lane * (N - 1) + i] : -1;
        oc[lane * (N - 1) + i] = t;
        if (i == 0) full = t >= 0;
      }
    }
    const uint64_t fm = __ballot(full);
    if (lane == 0) P.out_count[b] = __popcll(fm);
  }
}

// ---------------------------------------------------------------- launch

static dim3 cache_grid(int64_t tasks) { return dim3(static_cast<uint32_t>(tasks < (1 << 20) ? tasks : (1 << 20))); }

hipError_t launch_cache_fill(int32_t* cache, int64_t seq_elems, int64_t n, hipStream_t stream) {
  const int64_t nvec = n / 4;
  const int64_t blocks = (nvec + 255) / 256;
  hipLaunchKernelGGL(k_cache_fill, cache_grid(blocks > 0 ? blocks : 1), dim3(256), 0, stream, cache, seq_elems / 4,
                     nvec);
  return hipGetLastError();
}

hipError_t launch_cache_insert(const CacheParams& P, hipStream_t stream) {
  hipLaunchKernelGGL(k_cache_insert, cache_grid(P.B), dim3(kCacheBlock), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_cache_lookup(const CacheParams& P, hipStream_t stream) {
  hipLaunchKernelGGL(k_cache_lookup, cache_grid(P.B), dim3(64), 0, stream, P);
  return hipGetLastError();
}

}  // namespace sv
