// Greedy (temperature 0) verify of G disjoint candidate n-grams (gfx950).
//
// Method ("Lookahead Decoding 完全拆解:Jacobi 迭代与 N-gram 池,不靠草稿模型的投机解码",
// section "验证分支:输出分布不变性", eq. (1)): the i-th token of a candidate must equal
// the target's argmax at position i; the longest matched prefix among the
// candidates wins, followed by the argmax right after it.
//
// k_greedy_argmax: one workgroup per (logit row, segment) streams its segment with
// 16-byte loads and keeps the running (maximum, lowest index attaining it) per
// thread, visiting its elements in increasing index order; a block reduction on
// (value desc, index asc) gives the segment's first argmax.
// k_greedy_select (launched after it, so no cross-workgroup synchronisation):
// one workgroup per batch row merges the segments in index order, matches every
// candidate's prefix, and picks the longest (lowest candidate index on ties).
#include "common.hpp"
#include "params.hpp"

namespace sv {

struct ArgMax {
  float v;
  int64_t i;  // -1: no element seen yet
  // Elements arrive in increasing index order, so a tie keeps the earlier index.
  __device__ __forceinline__ void take(float x, int64_t e) {
    if (i < 0 || x > v) {
      v = x;
      i = e;
    }
  }
  template <int VEC>
  __device__ __forceinline__ void take_vec(const float (&x)[VEC], int64_t base) {
    float m = x[0];
#pragma unroll
    for (int e = 1; e < VEC; ++e) m = fmaxf(m, x[e]);
    if (i < 0 || m > v) {
      int first = VEC - 1;
#pragma unroll
      for (int e = VEC - 1; e >= 0; --e)
        if (x[e] == m) first = e;  // lowest e attaining m
      v = m;
      i = base + first;
    }
  }
};

// (value desc, index asc) merge of two candidates; i < 0 means empty.
__device__ __forceinline__ void argmax_merge(float& v, int64_t& i, float v2, int64_t i2) {
  if (i2 < 0) return;
  if (i < 0 || v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

// Launch shape, chosen by measured sweeps on gfx950 (the macros exist for such sweeps).
#ifndef SV_ARG_BLOCK
#define SV_ARG_BLOCK 256
#endif
#ifndef SV_ARG_UNROLL
#define SV_ARG_UNROLL 3
#endif
constexpr int kArgBlock = SV_ARG_BLOCK;    // threads per argmax workgroup
constexpr int kArgUnroll = SV_ARG_UNROLL;  // 16-byte vectors per thread per step

// The segment's whole vectors [0, nv) from vb, software-pipelined through a raw
// buffer resource (bytes < 2^31): the next step's loads are issued before this step
// is reduced, and loads past the segment read nothing. base_e is the row index of
// vb's first element. Every thread visits its elements in increasing index order.
template <int BS, typename T>
__device__ __forceinline__ void argmax_vectors_pipelined(const T* vb, int nv, int64_t base_e, ArgMax& a) {
  constexpr int VEC = Elem<T>::kVec;
  constexpr int U = kArgUnroll;
  const __amdgpu_buffer_rsrc_t rs = buffer_over(vb, static_cast<int64_t>(nv) * 16);
  const int t = threadIdx.x;
  u32x4 cur[U], nxt[U];
#pragma unroll
  for (int u = 0; u < U; ++u) cur[u] = load_stream_buf(rs, t + u * BS);
  for (int base = 0; base < nv; base += U * BS) {
#pragma unroll
    for (int u = 0; u < U; ++u) nxt[u] = load_stream_buf(rs, base + U * BS + t + u * BS);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = base + t + u * BS;
      if (v < nv) {
        float x[VEC];
        Elem<T>::unpack(cur[u], x);
        a.take_vec(x, base_e + static_cast<int64_t>(v) * VEC);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
  }
}

template <int BS, typename T, bool NT = true>
__device__ __forceinline__ void argmax_segment(const T* row, int64_t V, int seg, int S, ArgMax& a) {
  constexpr int VEC = Elem<T>::kVec;
  const SegRange r = seg_range(row, V, seg, S);
  if (seg == 0)
    for (int64_t e = threadIdx.x; e < r.head; e += BS) a.take(Elem<T>::get(row, e), e);
  const T* vb = row + r.head;
  // the pipelined loop's byte offsets reach two steps past the segment's end
  if (NT && (r.v1 - r.v0) * 16 < (int64_t(1) << 31) - 32 * kArgUnroll * BS) {
    argmax_vectors_pipelined<BS>(vb + r.v0 * VEC, static_cast<int>(r.v1 - r.v0), r.head + r.v0 * VEC, a);
    if (seg == S - 1)
      for (int64_t e = r.head + ((V - r.head) / VEC) * VEC + threadIdx.x; e < V; e += BS)
        a.take(Elem<T>::get(row, e), e);
    return;
  }
  int64_t v = r.v0 + threadIdx.x;
  for (; v + BS < r.v1; v += 2 * BS) {
    float x0[VEC], x1[VEC];
    Elem<T>::template vec<NT>(vb + v * VEC, x0);
    Elem<T>::template vec<NT>(vb + (v + BS) * VEC, x1);
    a.take_vec(x0, r.head + v * VEC);
    a.take_vec(x1, r.head + (v + BS) * VEC);
  }
  for (; v < r.v1; v += BS) {
    float x0[VEC];
    Elem<T>::template vec<NT>(vb + v * VEC, x0);
    a.take_vec(x0, r.head + v * VEC);
  }
  if (seg == S - 1)
    for (int64_t e = r.head + ((V - r.head) / VEC) * VEC + threadIdx.x; e < V; e += BS)
      a.take(Elem<T>::get(row, e), e);
}

template <int BS>
__device__ __forceinline__ void block_argmax(float& v, int64_t& i) {
  constexpr int W = BS / 64;
  __shared__ float sh_v[W];
  __shared__ int64_t sh_i[W];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(v, o, 64);
    const int64_t i2 = __shfl_xor(i, o, 64);
    argmax_merge(v, i, v2, i2);
  }
  if ((threadIdx.x & 63) == 0) {
    sh_v[threadIdx.x >> 6] = v;
    sh_i[threadIdx.x >> 6] = i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < W; ++w) argmax_merge(v, i, sh_v[w], sh_i[w]);
  }
}

template <typename T, int BS, bool NT>
__device__ __forceinline__ void greedy_argmax_task(const GreedyParams& P, const int64_t task) {
  const int S = P.S3;
  int64_t rq;
  int seg;
  split_task(task, S, rq, seg);
  const int row = static_cast<int>(rq);  // in [0, B*G*N)
  const T* rp = static_cast<const T*>(P.logits) + static_cast<int64_t>(row) * P.V;
  ArgMax a{-INFINITY, -1};
  argmax_segment<BS, T, NT>(rp, P.V, seg, S, a);
  float v = a.v;
  int64_t i = a.i;
  block_argmax<BS>(v, i);
  if (threadIdx.x == 0) {
    // a segment whose maximum is -inf holds no finite logit: report it as empty
    P.p3_v[static_cast<int64_t>(row) * S + seg] = v;
    P.p3_i[static_cast<int64_t>(row) * S + seg] = isfinite(v) ? static_cast<int32_t>(i) : -1;
  }
}

template <typename T, int BS = kArgBlock, bool NT = true>
__global__ __launch_bounds__(BS) void k_greedy_argmax(GreedyParams P) {
  touch_kernargs(P);
  const int64_t ntask = static_cast<int64_t>(P.B) * P.G * P.N * P.S3;
  for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) {
    greedy_argmax_task<T, BS, NT>(P, task);
    __syncthreads();  // shared memory is reused by the next task
  }
}

__device__ __forceinline__ void greedy_select_task(const GreedyParams& P, const int64_t task) {
  const int S = P.S3, N = P.N, G = P.G;
  const int GN = G * N;
  const int b = static_cast<int>(task);
  extern __shared__ int32_t sh_amax[];  // [G*N] argmax per row of this batch row
  __shared__ int sh_fault;
  __shared__ uint32_t sh_key;
  if (threadIdx.x == 0) {
    sh_fault = 0;
    sh_key = 0;
  }
  __syncthreads();
  for (int r = threadIdx.x; r < GN; r += kBlock) {
    const int64_t base = (static_cast<int64_t>(b) * GN + r) * S;
    float bv = -INFINITY;
    int32_t bi = -1;
    for (int j = 0; j < S; ++j) {  // segments in index order: strict > keeps the lowest index
      const int32_t ij = P.p3_i[base + j];
      const float vj = P.p3_v[base + j];
      if (ij >= 0 && (bi < 0 || vj > bv)) {
        bv = vj;
        bi = ij;
      }
    }
    sh_amax[r] = bi;
    if (bi < 0) atomicOr(&sh_fault, 1);
  }
  __syncthreads();
  const int32_t* cb = P.cand + static_cast<int64_t>(b) * G * (N - 1);
  for (int g = threadIdx.x; g < G; g += kBlock) {
    int L = 0;
    bool run = true;
    for (int t = 0; t < N - 1; ++t) {
      const int32_t ct = cb[g * (N - 1) + t];
      if (ct < 0 || ct >= P.V) atomicOr(&sh_fault, 1);
      if (run && ct == sh_amax[g * N + t]) ++L;
      else run = false;
    }
    // key: longer prefix first, then lower candidate index
    atomicMax(&sh_key, (static_cast<uint32_t>(L) << 16) | static_cast<uint32_t>(0xFFFF - g));
  }
  __syncthreads();
  const bool fault = sh_fault != 0;
  const uint32_t key = sh_key;
  const int L = static_cast<int>(key >> 16);
  const int best = 0xFFFF - static_cast<int>(key & 0xFFFF);
  int32_t* ot = P.out_tokens + static_cast<int64_t>(b) * N;
  for (int t = threadIdx.x; t < N; t += kBlock) {
    int32_t tok = -1;
    if (!fault) {
      if (t < L) tok = cb[best * (N - 1) + t];
      else if (t == L) tok = sh_amax[best * N + L];
    }
    ot[t] = tok;
  }
  if (threadIdx.x == 0) {
    P.out_len[b] = fault ? -1 : L;
    P.out_best[b] = fault ? -1 : best;
  }
}

__global__ __launch_bounds__(kBlock) void k_greedy_select(GreedyParams P) {
  touch_kernargs(P);
  const int64_t ntask = P.B;
  for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) {
    greedy_select_task(P, task);
    __syncthreads();  // shared memory is reused by the next task
  }
}

constexpr int kSelectMaxT = 16;  // candidate tokens the one-wave select holds per lane

// The select of batch row b by one wave with no barrier, when its G*N rows fit the
// wave (lane r holds row r's argmax): one round of loads (the rows' segment partials
// and the candidates), shuffles for the prefix matches, a wave maximum of the
// (prefix length, lowest candidate) key. The same results as greedy_select_task.
__device__ __forceinline__ void greedy_select_wave(const GreedyParams& P, const int b) {
  const int S = P.S3, N = P.N, G = P.G;
  const int GN = G * N;
  const int lane = threadIdx.x & 63;
  // candidate lane g's tokens (N - 1 <= kSelectMaxT of them), issued with the partials
  const int32_t* cb = P.cand + static_cast<int64_t>(b) * G * (N - 1);
  int32_t ct[kSelectMaxT];
#pragma unroll
  for (int t = 0; t < kSelectMaxT; ++t) ct[t] = (lane < G && t < N - 1) ? cb[lane * (N - 1) + t] : 0;
  // row r = lane: its segments in index order (strict > keeps the lowest index)
  float bv = -INFINITY;
  int32_t bi = -1;
  if (lane < GN) {
    const int64_t base = (static_cast<int64_t>(b) * GN + lane) * S;
    for (int j = 0; j < S; ++j) {
      const int32_t ij = P.p3_i[base + j];
      const float vj = P.p3_v[base + j];
      if (ij >= 0 && (bi < 0 || vj > bv)) {
        bv = vj;
        bi = ij;
      }
    }
  }
  bool bad = lane < GN && bi < 0;
  // candidate g = lane: its matched prefix against the argmaxes of its rows
  int L = 0;
  bool run = true;
#pragma unroll
  for (int t = 0; t < kSelectMaxT; ++t) {
    if (t >= N - 1) break;  // wave-uniform
    const int32_t am = __shfl(bi, min(lane, G - 1) * N + t, 64);  // every lane takes part
    if (lane < G) {
      const int32_t c = ct[t];
      bad = bad || c < 0 || c >= P.V;
      if (run && c == am) ++L;
      else run = false;
    }
  }
  const bool fault = __ballot(bad) != 0;
  // longer prefix first, then the lower candidate index
  uint32_t key = lane < G ? (static_cast<uint32_t>(L) << 16) | static_cast<uint32_t>(0xFFFF - lane) : 0u;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) key = max(key, static_cast<uint32_t>(__shfl_xor(static_cast<int>(key), o, 64)));
  const int Lb = static_cast<int>(key >> 16);
  const int best = 0xFFFF - static_cast<int>(key & 0xFFFF);
  const int32_t bonus = __shfl(bi, best * N + Lb, 64);  // the argmax right after the prefix
  int32_t* ot = P.out_tokens + static_cast<int64_t>(b) * N;
  if (lane < N) {
    int32_t tok = -1;
    if (!fault) {
      if (lane < Lb) tok = cb[best * (N - 1) + lane];
      else if (lane == Lb) tok = bonus;
    }
    ot[lane] = tok;
  }
  if (lane == 0) {
    P.out_len[b] = fault ? -1 : Lb;
    P.out_best[b] = fault ? -1 : best;
  }
}

constexpr int kSelectWaveBlock = 64;  // one wave per batch row

__global__ __launch_bounds__(kSelectWaveBlock) void k_greedy_select_wave(GreedyParams P) {
  touch_kernargs(P);
  for (int64_t task = blockIdx.x; task < P.B; task += gridDim.x) greedy_select_wave(P, static_cast<int>(task));
}

constexpr int64_t kMaxGrid = 1 << 20;  // workgroups per launch; kernels loop over their tasks

inline dim3 grid_for(int64_t tasks) { return dim3(static_cast<uint32_t>(tasks < kMaxGrid ? tasks : kMaxGrid)); }

template <typename T>
static hipError_t launch_greedy_t(const GreedyParams& P, hipStream_t stream) {
  const int64_t g = static_cast<int64_t>(P.B) * P.G * P.N * P.S3;
  hipLaunchKernelGGL((k_greedy_argmax<T>), grid_for(g), dim3(kArgBlock), 0, stream, P);
  if (static_cast<int64_t>(P.G) * P.N <= 64 && P.N - 1 <= kSelectMaxT && !P.select_block) {
    hipLaunchKernelGGL(k_greedy_select_wave, grid_for(P.B), dim3(kSelectWaveBlock), 0, stream, P);
  } else {
    const size_t lds = static_cast<size_t>(P.G) * P.N * sizeof(int32_t);
    hipLaunchKernelGGL(k_greedy_select, grid_for(P.B), dim3(kBlock), lds, stream, P);
  }
  return hipGetLastError();
}

hipError_t launch_greedy(const GreedyParams& P, bool bf16, hipStream_t stream) {
  return bf16 ? launch_greedy_t<bf16_t>(P, stream) : launch_greedy_t<float>(P, stream);
}

}  // namespace sv
