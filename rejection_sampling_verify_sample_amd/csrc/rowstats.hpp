// Streaming row statistics shared by the verify kernels (gfx950): the online
// (max, sum of 2^(x*c - R)) of a row segment, and the merge of a row's segment
// partials.
#pragma once

#include "common.hpp"

namespace sv {

// ---------------------------------------------------------------- online softmax over a segment

// Launch geometry, chosen by measured sweeps on gfx950 (the macros exist for such sweeps).
#ifndef SV_ROW_BLOCK
#define SV_ROW_BLOCK 256
#endif
#ifndef SV_ROW_UNROLL
#define SV_ROW_UNROLL 3
#endif
constexpr int kRowBlock = SV_ROW_BLOCK;  // threads per row-statistics workgroup
constexpr int kUnroll = SV_ROW_UNROLL;   // 16-byte vectors in flight per thread per step

template <int BS, typename T>
__device__ __forceinline__ void online_scalar(const T* row, int64_t lo, int64_t hi, float c, Online& o) {
  for (int64_t e = lo + threadIdx.x; e < hi; e += BS) {
    const float x = Elem<T>::get(row, e);
    if (x > o.m) o.raise(x, c);
    o.add(x, c);
  }
}

// The online (max, sum) of a segment's whole vectors: the software-pipelined loop
// reads through a raw buffer resource over the segment (bytes < 2^31), so the next
// step's loads are issued before this step is reduced and need no per-lane guard
// (past the segment they read nothing); only the segment's last step masks.
template <int BS, typename T>
__device__ __forceinline__ void online_vectors_pipelined(const T* vb, int nv, float c, Online& o) {
  constexpr int VEC = Elem<T>::kVec;
  constexpr int U = kUnroll;
  const __amdgpu_buffer_rsrc_t rs = buffer_over(vb, static_cast<int64_t>(nv) * 16);
  const int t = threadIdx.x;
  u32x4 cur[U], nxt[U];
#pragma unroll
  for (int u = 0; u < U; ++u) cur[u] = load_stream_buf(rs, t + u * BS);
  for (int base = 0; base < nv; base += U * BS) {
#pragma unroll
    for (int u = 0; u < U; ++u) nxt[u] = load_stream_buf(rs, base + U * BS + t + u * BS);
    float x[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) Elem<T>::unpack(cur[u], x[u]);
    if (base + U * BS > nv) {  // the segment's last step
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool in = base + t + u * BS < nv;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          if (!in) x[u][e] = -INFINITY;
      }
    }
    float mt = x[0][0];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) mt = fmaxf(mt, x[u][e]);
    if (mt > o.m) o.raise(mt, c);
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float a = exp2_hw(fmaf(x[u][0], c, -o.R));
#pragma unroll
      for (int e = 1; e < VEC; ++e) a += exp2_hw(fmaf(x[u][e], c, -o.R));
      acc += a;
    }
    o.s += acc;
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
  }
}

// The same over vectors [v0, v1) of a segment too large for a buffer resource.
template <int BS, typename T>
__device__ __forceinline__ void online_vectors_plain(const T* vb, int64_t v0, int64_t v1, float c, Online& o) {
  constexpr int VEC = Elem<T>::kVec;
  int64_t v = v0 + threadIdx.x;
  for (; v + (kUnroll - 1) * BS < v1; v += kUnroll * BS) {
    float x[kUnroll][VEC];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) Elem<T>::vec(vb + (v + u * BS) * VEC, x[u]);
    float mt = x[0][0];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) mt = fmaxf(mt, x[u][e]);
    if (mt > o.m) o.raise(mt, c);
    float t = 0.f;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float a = exp2_hw(fmaf(x[u][0], c, -o.R));
#pragma unroll
      for (int e = 1; e < VEC; ++e) a += exp2_hw(fmaf(x[u][e], c, -o.R));
      t += a;
    }
    o.s += t;
  }
  for (; v < v1; v += BS) {
    float x[VEC];
    Elem<T>::vec(vb + v * VEC, x);
    float mt = x[0];
#pragma unroll
    for (int e = 1; e < VEC; ++e) mt = fmaxf(mt, x[e]);
    if (mt > o.m) o.raise(mt, c);
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) a += exp2_hw(fmaf(x[e], c, -o.R));
    o.s += a;
  }
}

template <int BS, typename T>
__device__ __forceinline__ void online_segment(const T* row, int64_t V, int seg, int S, float c, Online& o) {
  constexpr int VEC = Elem<T>::kVec;
  const SegRange r = seg_range(row, V, seg, S);
  if (seg == 0) online_scalar<BS>(row, 0, r.head, c, o);
  const T* vb = row + r.head;
  // the pipelined loop's byte offsets reach two steps past the segment's end
  if ((r.v1 - r.v0) * 16 < (int64_t(1) << 31) - 32 * kUnroll * BS)
    online_vectors_pipelined<BS>(vb + r.v0 * VEC, static_cast<int>(r.v1 - r.v0), c, o);
  else
    online_vectors_plain<BS>(vb, r.v0, r.v1, c, o);
  if (seg == S - 1) online_scalar<BS>(row, r.head + ((V - r.head) / VEC) * VEC, V, c, o);
}

// Merge segment partials (m_j, s_j) = (pm[j*stride], ps[j*stride]) of one row, in
// segment order (the partial arrays are segment-major, so a one-segment layout
// packs the rows' partials densely). Each partial is
// rescaled from its reference fl(m_j * c) to the row's by 2^d, with d the exact
// fp64 difference of the two references and 2^d from the hardware unit (about
// 1e-7 relative, the order of the fp32 sums inside each partial); the partial
// holding the maximum needs no rescale.
// Up to kMergeRegs partials are loaded at once (one round of loads, held in
// registers); a row split into more segments is read in a loop.
constexpr int kMergeRegs = 16;

__device__ __forceinline__ double rescaled_partial(double sj, float Rj, float RMf) {
  if (!(sj > 0.0)) return 0.0;
  return (Rj == RMf) ? sj
                     : sj * static_cast<double>(exp2_hw(static_cast<float>(static_cast<double>(Rj) -
                                                                           static_cast<double>(RMf))));
}

__device__ __forceinline__ void merge_partials(const float* pm, const double* ps, int64_t stride, int S, float c,
                                               float& M, double& Ssum) {
  M = -INFINITY;
  Ssum = 0.0;
  if (S == 1) {  // one segment: the same values as the general merge below, without its loop
    const float m0 = pm[0];
    const double s0 = ps[0];
    M = fmaxf(M, m0);
    // m0 == M unless m0 is NaN, whose rescale factor leaves a NaN sum
    Ssum = (s0 > 0.0) ? ((m0 == M) ? s0 : static_cast<double>(__builtin_nanf(""))) : 0.0;
    return;
  }
  if (S <= kMergeRegs) {
    float mv[kMergeRegs];
    double sv[kMergeRegs];
#pragma unroll
    for (int j = 0; j < kMergeRegs; ++j) {
      const bool in = j < S;
      mv[j] = in ? pm[j * stride] : -INFINITY;
      sv[j] = in ? ps[j * stride] : 0.0;
    }
#pragma unroll
    for (int j = 0; j < kMergeRegs; ++j) M = fmaxf(M, mv[j]);
    const float RMf = M * c;
#pragma unroll
    for (int j = 0; j < kMergeRegs; ++j) Ssum += rescaled_partial(sv[j], mv[j] * c, RMf);
    return;
  }
  for (int j = 0; j < S; ++j) M = fmaxf(M, pm[j * stride]);
  const float RMf = M * c;
  for (int j = 0; j < S; ++j) Ssum += rescaled_partial(ps[j * stride], pm[j * stride] * c, RMf);
}

}  // namespace sv
