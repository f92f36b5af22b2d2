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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load with the nontemporal hint: the streamed logits are read once, so
// they should not displace cache lines that are reused.
__device__ __forceinline__ u32x4 load_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// A raw buffer resource over [base, base + bytes), bytes < 2^31: a 16-byte load at
// an offset past the end returns zero without a memory access (the hardware's
// range check), so loads need no per-lane guard.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

// 16-byte nontemporal load of vector `vi` of a buffer resource (zero past its end).
__device__ __forceinline__ u32x4 load_stream_buf(__amdgpu_buffer_rsrc_t r, int vi) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, vi * 16, 0, 2);
}

// ---------------------------------------------------------------- element access

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int kVec = 4;  // elements per 16-byte load
  __device__ __forceinline__ static float get(const float* p, size_t i) { return p[i]; }
  // element e in [0, 4) of a raw vector (e may differ across lanes)
  __device__ __forceinline__ static float lane_elem(const u32x4& v, int e) {
    return __uint_as_float(e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w);
  }
  __device__ __forceinline__ static void unpack(const u32x4& v, float (&x)[4]) {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  }
  template <bool NT = true>
  __device__ __forceinline__ static void vec(const float* p, float (&x)[4]) {
    const u32x4 v = NT ? load_stream(p) : *reinterpret_cast<const u32x4*>(p);
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  }
};

template <>
struct Elem<bf16_t> {
  static constexpr int kVec = 8;
  __device__ __forceinline__ static float get(const bf16_t* p, size_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i].bits) << 16);
  }
  // element e in [0, 8) of a raw vector (e may differ across lanes)
  __device__ __forceinline__ static float lane_elem(const u32x4& v, int e) {
    const int j = e >> 1;
    const uint32_t w = j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  __device__ __forceinline__ static void unpack(const u32x4& v, float (&x)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
  template <bool NT = true>
  __device__ __forceinline__ static void vec(const bf16_t* p, float (&x)[8]) {
    const u32x4 v = NT ? load_stream(p) : *reinterpret_cast<const u32x4*>(p);
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

// Order key of a logit: keys compare as unsigned integers exactly as the logits
// compare as floats (-0 takes the key of +0, so equal values have equal keys;
// -inf has the smallest key of any non-NaN value).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

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

// ---------------------------------------------------------------- DPP wave scans
//
// Inclusive scans across the 64 lanes of a wave with gfx9 DPP moves (row_shr
// 1/2/4/8 inside each row of 16 lanes, then row_bcast 15 and 31 across rows):
// six dependent register moves instead of LDS-routed shuffles. Every lane of the
// wave must be active. Lanes outside a move's source range receive the identity.
namespace dpp {
constexpr int kShr1 = 0x111, kShr2 = 0x112, kShr4 = 0x114, kShr8 = 0x118, kBcast15 = 0x142, kBcast31 = 0x143;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t mov(uint32_t v, uint32_t identity) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(identity), static_cast<int>(v), CTRL,
                                                           ROW_MASK, 0xf, false));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float movf(float v, float identity) {
  return __uint_as_float(mov<CTRL, ROW_MASK>(__float_as_uint(v), __float_as_uint(identity)));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double movd(double v) {  // identity +0.0
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = mov<CTRL, ROW_MASK>(static_cast<uint32_t>(u), 0u);
  const uint32_t hi = mov<CTRL, ROW_MASK>(static_cast<uint32_t>(u >> 32), 0u);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}
}  // namespace dpp

// Inclusive prefix sum over the lanes of a wave (lane order), fp64.
__device__ __forceinline__ double wave_scan_add(double v) {
  v += dpp::movd<dpp::kShr1, 0xf>(v);
  v += dpp::movd<dpp::kShr2, 0xf>(v);
  v += dpp::movd<dpp::kShr4, 0xf>(v);
  v += dpp::movd<dpp::kShr8, 0xf>(v);
  v += dpp::movd<dpp::kBcast15, 0xa>(v);
  v += dpp::movd<dpp::kBcast31, 0xc>(v);
  return v;
}

// Inclusive prefix sum over the lanes of a wave, fp32.
__device__ __forceinline__ float wave_scan_addf(float v) {
  v += dpp::movf<dpp::kShr1, 0xf>(v, 0.f);
  v += dpp::movf<dpp::kShr2, 0xf>(v, 0.f);
  v += dpp::movf<dpp::kShr4, 0xf>(v, 0.f);
  v += dpp::movf<dpp::kShr8, 0xf>(v, 0.f);
  v += dpp::movf<dpp::kBcast15, 0xa>(v, 0.f);
  v += dpp::movf<dpp::kBcast31, 0xc>(v, 0.f);
  return v;
}

// Inclusive prefix maximum over the lanes of a wave, fp32 (lane 63 holds the maximum).
__device__ __forceinline__ float wave_scan_maxf(float v) {
  v = fmaxf(v, dpp::movf<dpp::kShr1, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp::movf<dpp::kShr2, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp::movf<dpp::kShr4, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp::movf<dpp::kShr8, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp::movf<dpp::kBcast15, 0xa>(v, -INFINITY));
  v = fmaxf(v, dpp::movf<dpp::kBcast31, 0xc>(v, -INFINITY));
  return v;
}

// Value of lane `l` (uniform across the wave) in every lane.
__device__ __forceinline__ float lane_f(float v, int l) {
  return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(__float_as_uint(v)), l)));
}
__device__ __forceinline__ int lane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ double lane_d(double v, int l) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u)), l));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u >> 32)), l));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Lowest lane whose predicate holds (64 if none); highest such lane (-1 if none).
__device__ __forceinline__ int first_lane(bool pred) {
  const uint64_t m = __ballot(pred);
  return m ? __ffsll(static_cast<unsigned long long>(m)) - 1 : 64;
}
__device__ __forceinline__ int last_lane(bool pred) {
  const uint64_t m = __ballot(pred);
  return m ? 63 - __clzll(static_cast<long long>(m)) : -1;
}

// A kernel's parameter block is read with scalar loads where each field is
// first used, often several dependent rounds apart, and a cold line costs its
// round a scalar-cache miss. One round at kernel entry that touches every
// 64-byte line of the block (dwords 48 bytes apart, and the grid size just past
// it) makes the later rounds hits.
template <typename Params>
__device__ __forceinline__ void touch_kernargs(const Params& P) {
  static_assert(sizeof(Params) % 4 == 0, "whole dwords");
  const char* base = reinterpret_cast<const char*>(&P);
  auto dword = [&](size_t i) {
    uint32_t v;
    __builtin_memcpy(&v, base + 4 * i, 4);
    return v;
  };
#pragma unroll
  for (size_t i = 0; i < sizeof(Params) / 4; i += 12) asm volatile("" ::"s"(dword(i)));
  asm volatile("" ::"s"(dword(sizeof(Params) / 4 - 1)), "s"(gridDim.x));
}

// Quotient and remainder of a workgroup-uniform task index by d > 0. A 64-bit
// division is a scalar sequence of about a hundred instructions, each on the
// short kernels' critical path, so indices below 2^31 take the 32-bit one.
__device__ __forceinline__ void split_task(int64_t task, int d, int64_t& q, int& r) {
  if (task < (int64_t{1} << 31)) {
    const uint32_t t = static_cast<uint32_t>(task), ud = static_cast<uint32_t>(d);
    const uint32_t qq = t / ud;
    q = qq;
    r = static_cast<int>(t - qq * ud);
  } else {
    q = task / d;
    r = static_cast<int>(task - q * d);
  }
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

// Combine the per-thread online states of a block. Result valid in thread 0:
// m = block maximum, s = sum against fl(m * c). Each thread rescales its own
// partial to the block reference in fp32 (exactly as a raise does); the sums
// across lanes and waves are fp64.
template <int BS>
__device__ __forceinline__ void block_online(const Online& o, float c, float& m_out, double& s_out) {
  constexpr int W = BS / 64;
  __shared__ float sh_m[W];
  __shared__ double sh_s[W];
  const int w = threadIdx.x >> 6;
  const float mw = wave_max(o.m);
  if ((threadIdx.x & 63) == 0) sh_m[w] = mw;
  __syncthreads();
  float M = sh_m[0];
#pragma unroll
  for (int i = 1; i < W; ++i) M = fmaxf(M, sh_m[i]);
  const float RM = M * c;
  const float sl = (o.s > 0.f) ? o.s * exp2_hw(o.R - RM) : 0.f;
  const double sw = wave_sum(static_cast<double>(sl));
  if ((threadIdx.x & 63) == 0) sh_s[w] = sw;
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < W; ++i) s += sh_s[i];
    m_out = M;
    s_out = s;
  }
}

}  // namespace sv
