// Device helpers shared by the verify kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kBlock = 256;             // threads per workgroup: 4 waves of 64
constexpr int kWaves = kBlock / 64;

// bf16 storage type: the upper 16 bits of an IEEE float.
struct bf16_t {
  uint16_t bits;
};

// ---------------------------------------------------------------- element access

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int kVec = 4;  // elements per 16-byte load
  __device__ __forceinline__ static float get(const float* p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void vec(const float* p, float (&x)[4]) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
};

template <>
struct Elem<bf16_t> {
  static constexpr int kVec = 8;
  __device__ __forceinline__ static float get(const bf16_t* p, size_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i].bits) << 16);
  }
  __device__ __forceinline__ static void vec(const bf16_t* p, float (&x)[8]) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
};

// Elements before the first 16-byte boundary of a row (clamped to V).
template <typename T>
__device__ __forceinline__ int64_t head_elems(const T* row, int64_t V) {
  const uintptr_t mis = reinterpret_cast<uintptr_t>(row) & 15u;
  const int64_t h = mis ? static_cast<int64_t>((16u - mis) / sizeof(T)) : 0;
  return h < V ? h : V;
}

// ---------------------------------------------------------------- segment geometry
//
// A row of V elements is split into S segments along its 16-byte vectors:
// elements before the first 16-byte boundary belong to segment 0, the ragged
// tail after the last whole vector to segment S-1.
struct SegRange {
  int64_t head, v0, v1;   // head elements; vector range [v0, v1) counted from the first boundary
  int64_t lo, hi;         // element range [lo, hi) of the whole segment
};

template <typename T>
__device__ __forceinline__ SegRange seg_range(const T* row, int64_t V, int seg, int S) {
  constexpr int VEC = Elem<T>::kVec;
  SegRange r;
  r.head = head_elems(row, V);
  const int64_t nvec = (V - r.head) / VEC;
  r.v0 = nvec * seg / S;
  r.v1 = nvec * (seg + 1) / S;
  r.lo = (seg == 0) ? 0 : r.head + r.v0 * VEC;
  r.hi = (seg == S - 1) ? V : r.head + r.v1 * VEC;
  return r;
}

// ---------------------------------------------------------------- math

// 2^t on the hardware exponential unit (v_exp_f32; 2^-inf = 0).
__device__ __forceinline__ float exp2_hw(float t) { return __builtin_amdgcn_exp2f(t); }

// ---------------------------------------------------------------- wave / block reductions

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_sumf(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------- online softmax state
//
// A partial softmax denominator over some elements x, kept against the
// reference exponent R = fl(m * c) of its running maximum m (c = log2(e) / T):
//   s = sum 2^(fl(x*c - R)),   one fused multiply-add per element.
// Every partial uses the same rounding of m * c for its reference, so partials
// combine exactly up to the rounding of the rescale factors.
struct Online {
  float m;  // running maximum of the raw logits (-inf when none is finite)
  float R;  // fl(m * c); 0 while m == -inf, so -inf logits still give 2^-inf = 0
  float s;

  __device__ __forceinline__ void init() {
    m = -INFINITY;
    R = 0.f;
    s = 0.f;
  }
  // Raise the reference to a new maximum mt > m.
  __device__ __forceinline__ void raise(float mt, float c) {
    const float Rn = mt * c;
    s = (s > 0.f) ? s * exp2_hw(R - Rn) : 0.f;
    m = mt;
    R = Rn;
  }
  __device__ __forceinline__ void add(float x, float c) { s += exp2_hw(fmaf(x, c, -R)); }
};

// ---------------------------------------------------------------- coherent scratch access
//
// Partials written by one workgroup and read by the last-arriving workgroup of
// a group travel through device memory with agent-scope atomics, so no
// per-XCD L2 can serve a stale copy.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(double* p, double v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), static_cast<uint64_t>(__double_as_longlong(v)),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ double ld_agent(const double* p) {
  return __longlong_as_double(static_cast<long long>(
      __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
}
__device__ __forceinline__ int32_t ld_agent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrive at a group counter after this workgroup's partial is stored. Returns
// true (in every thread) for the last of `expected` arrivals, which also
// resets the counter to zero for the next call.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected) {
  __shared__ int s_last;
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const int last = (prev == expected - 1);
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  const bool last = s_last != 0;
  if (last) __threadfence();
  return last;
}

}  // namespace sv
