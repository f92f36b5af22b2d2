// Block-wide scans and the inverse-CDF search shared by the verify kernels (gfx950).
#pragma once

#include "common.hpp"

namespace sv {

// ---------------------------------------------------------------- block utilities

template <int BS>
__device__ __forceinline__ double block_sum(double v) {
  constexpr int W = BS / 64;
  __shared__ double sh[W];
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < W; ++i) t += sh[i];
  __syncthreads();
  return t;
}

__device__ __forceinline__ double wave_inclusive_scan(double v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

// Inclusive prefix sum over the block (thread order), fp64. Also returns the block total.
template <int BS>
__device__ __forceinline__ double block_inclusive_scan(double v, double& total) {
  constexpr int W = BS / 64;
  __shared__ double sh[W];
  const int w = threadIdx.x >> 6;
  v = wave_inclusive_scan(v);
  if ((threadIdx.x & 63) == 63) sh[w] = v;
  __syncthreads();
  double before = 0.0;
  total = 0.0;
  for (int i = 0; i < W; ++i) {
    if (i < w) before += sh[i];
    total += sh[i];
  }
  __syncthreads();
  return before + v;
}

// Lowest thread index whose predicate holds (BS if none), in every thread.
template <int BS>
__device__ __forceinline__ int block_first(bool pred) {
  constexpr int W = BS / 64;
  __shared__ uint64_t sh[W];
  const uint64_t bal = __ballot(pred);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = bal;
  __syncthreads();
  int first = BS;
  for (int i = W - 1; i >= 0; --i)
    if (sh[i]) first = i * 64 + (__ffsll(static_cast<unsigned long long>(sh[i])) - 1);
  __syncthreads();
  return first;
}

template <int BS>
__device__ __forceinline__ int64_t block_max_i64(int64_t v) {
  constexpr int W = BS / 64;
  __shared__ int64_t sh[W];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int64_t y = __shfl_xor(v, o, 64);
    v = y > v ? y : v;
  }
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  int64_t t = sh[0];
  for (int i = 1; i < W; ++i) t = sh[i] > t ? sh[i] : t;
  __syncthreads();
  return t;
}

// Inverse-CDF search over elements [lo, hi) with weights w(e), by the whole block:
// the smallest k with (sum of w over [lo, k]) > tau. Each chunk of the range gives
// every thread kSearchE contiguous elements, held in registers; chunk masses and
// thread offsets are fp64, the run inside a thread fp32. If rounding leaves no
// crossing, returns the last element with w > 0 (lo if none). Used for the rare
// zero-residual fallback, which draws from p_n over the whole row.
constexpr int kSearchE = 8;

template <int BS, typename W>
__device__ int64_t block_search(int64_t lo, int64_t hi, double tau, const W& w) {
  __shared__ int64_t sh_k;
  double base = 0.0;
  int64_t last_pos = -1;
  for (int64_t c0 = lo; c0 < hi; c0 += static_cast<int64_t>(BS) * kSearchE) {
    const int64_t e0 = c0 + static_cast<int64_t>(threadIdx.x) * kSearchE;
    float wv[kSearchE];
    float ts = 0.f;
#pragma unroll
    for (int k = 0; k < kSearchE; ++k) {
      const int64_t e = e0 + k;
      wv[k] = (e < hi) ? w(e) : 0.f;
      ts += wv[k];
      if (wv[k] > 0.f) last_pos = e;
    }
    double total;
    const double incl = block_inclusive_scan<BS>(static_cast<double>(ts), total);
    if (base + total > tau) {
      const double excl = incl - static_cast<double>(ts);
      const int t = block_first<BS>(base + incl > tau);
      if (static_cast<int>(threadIdx.x) == t) {
        int64_t k_found = -1, k_lastpos = -1;
        float run = 0.f;
#pragma unroll
        for (int k = 0; k < kSearchE; ++k) {
          run += wv[k];
          if (wv[k] > 0.f) k_lastpos = e0 + k;
          if (k_found < 0 && base + excl + static_cast<double>(run) > tau) k_found = e0 + k;
        }
        sh_k = (k_found >= 0) ? k_found : (k_lastpos >= 0 ? k_lastpos : e0);
      }
      __syncthreads();
      const int64_t k = sh_k;
      __syncthreads();
      return k;
    }
    base += total;
  }
  const int64_t lp = block_max_i64<BS>(last_pos);
  return lp >= 0 ? lp : lo;
}

// Chunks of a row: chunk 0 holds the elements before the first 16-byte boundary,
// chunks 1..nvc hold 64 vectors each (the last one possibly fewer), chunk nvc+1
// the ragged tail. One wave reads one vector chunk with one load per lane.
constexpr int kChunkVecs = 64;

struct Chunks {
  int64_t h, nvec;
  int nvc;
  __device__ __forceinline__ int count() const { return nvc + 2; }
};

template <typename T>
__device__ __forceinline__ Chunks chunks_of(const T* row, int64_t V) {
  Chunks ch;
  ch.h = head_elems(row, V);
  ch.nvec = (V - ch.h) / Elem<T>::kVec;
  ch.nvc = static_cast<int>((ch.nvec + kChunkVecs - 1) / kChunkVecs);
  return ch;
}

// Element range [lo, hi) of scalar chunk 0 (head) or nvc+1 (tail).
template <typename T>
__device__ __forceinline__ void scalar_chunk_range(const Chunks& ch, int c, int64_t V, int64_t& lo, int64_t& hi) {
  if (c == 0) {
    lo = 0;
    hi = ch.h;
  } else {
    lo = ch.h + ch.nvec * Elem<T>::kVec;
    hi = V;
  }
}

}  // namespace sv
