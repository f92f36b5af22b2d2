// Rejection-sampling verify kernels (gfx950).
//
// Method ("Speculative Decoding —— LLM推理优化技术（一）" §2.1-2.3; kwkr.cn/news/620797
// notes §3.1-3.4): p_i = softmax(target_i / T), q_i = softmax(draft_i / T) in fp32;
// accept x_i iff r_i < min(1, p_i(x_i) / q_i(x_i)); stop at the first rejection n
// and draw from norm(max(0, p_n - q_n)); if all K are accepted draw a bonus token
// from p_K.
//
// Kernels, in stream order; each reads what the previous ones wrote, so no
// workgroup waits for another and no cross-workgroup atomics or fences are needed:
//   k_sample_rowstats  one workgroup per (batch row b, logit row j < 2K, segment): one
//                      streaming pass with 16-byte nontemporal loads keeps an online
//                      maximum and a sum of 2^(x*c - R) (c = log2(e)/T) per thread; a
//                      wave shuffle and an LDS step combine the block. Segment 0 also
//                      fetches the logit of the row's draft token. The bonus row is not
//                      read here: it is needed only when all K drafts are accepted.
//   k_sample_mass      one workgroup per (b, segment). It first takes the accept
//                      decisions of batch row b (merging the row statistics, alpha_i,
//                      and the first rejection from one 64-lane ballot); segment 0
//                      writes them out. Then it reads only the row(s) the draw needs --
//                      target and draft row n after a rejection, or the bonus row K --
//                      and records the draw mass of every chunk of 64 vectors (one wave
//                      load): max(0, p - q) summed, or for the bonus row the chunk's
//                      maximum and its softmax sum against that maximum.
//   k_sample_draw      one workgroup per b: scans the chunk masses in fp64, picks the
//                      chunk where u*Z falls, and one wave rereads that chunk (1 KB,
//                      cache-hot) and finds the token with a lane prefix sum.
// k_sample_accept runs the decisions alone, for callers that run the phases apart.
#include "common.hpp"
#include "params.hpp"

namespace sv {

// ---------------------------------------------------------------- online softmax over a segment

constexpr int kRowBlock = 128;  // threads per row-statistics workgroup (measured best on gfx950)
constexpr int kUnroll = 4;      // 16-byte vectors in flight per thread per step

template <int BS, typename T>
__device__ __forceinline__ void online_scalar(const T* row, int64_t lo, int64_t hi, float c, Online& o) {
  for (int64_t e = lo + threadIdx.x; e < hi; e += BS) {
    const float x = Elem<T>::get(row, e);
    if (x > o.m) o.raise(x, c);
    o.add(x, c);
  }
}

template <int BS, typename T>
__device__ __forceinline__ void online_segment(const T* row, int64_t V, int seg, int S, float c, Online& o) {
  constexpr int VEC = Elem<T>::kVec;
  const SegRange r = seg_range(row, V, seg, S);
  if (seg == 0) online_scalar<BS>(row, 0, r.head, c, o);
  const T* vb = row + r.head;
  int64_t v = r.v0 + threadIdx.x;
  for (; v + (kUnroll - 1) * BS < r.v1; v += kUnroll * BS) {
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
  for (; v < r.v1; v += BS) {
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
  if (seg == S - 1) online_scalar<BS>(row, r.head + ((V - r.head) / VEC) * VEC, V, c, o);
}

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

// Merge segment partials (m_j, s_j) of one row, in segment order.
__device__ __forceinline__ void merge_partials(const float* pm, const double* ps, int S, float c, float& M,
                                               double& Ssum) {
  M = -INFINITY;
  for (int j = 0; j < S; ++j) M = fmaxf(M, pm[j]);
  const double RM = static_cast<double>(M * c);
  Ssum = 0.0;
  for (int j = 0; j < S; ++j) {
    const double sj = ps[j];
    if (sj > 0.0) Ssum += sj * exp2(static_cast<double>(pm[j] * c) - RM);
  }
}

template <typename T>
__device__ __forceinline__ const T* target_row(const SampleParams& P, int b, int i) {
  return static_cast<const T*>(P.target) + (static_cast<int64_t>(b) * (P.K + 1) + i) * P.V;
}
template <typename T>
__device__ __forceinline__ const T* draft_row(const SampleParams& P, int b, int i) {
  return static_cast<const T*>(P.draft) + (static_cast<int64_t>(b) * P.K + i) * P.V;
}

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

// ---------------------------------------------------------------- row statistics (pass 1)

template <typename T>
__device__ __forceinline__ void sample_rowstats_task(const SampleParams& P, const int64_t task) {
  const int K = P.K, S = P.S1;
  const int seg = static_cast<int>(task % S);
  // tasks walk the target rows of every batch row, then the draft rows, in memory order
  const int t = static_cast<int>(task / S);
  const bool is_draft = t >= P.B * K;
  const int tb = is_draft ? t - P.B * K : t;
  const int b = tb / K;
  const int pos = tb - b * K;
  const int j = is_draft ? K + pos : pos;
  const int row = b * 2 * K + j;  // partial slot: j < K target row j, else draft row j-K
  const T* rp = (j < K) ? target_row<T>(P, b, j) : draft_row<T>(P, b, pos);
  // segment 0 fetches the draft token's logit; issued first, consumed after the stream
  float xl = __builtin_nanf("");
  if (seg == 0 && threadIdx.x == 0) {
    const int x = P.tokens[static_cast<int64_t>(b) * K + pos];
    if (x >= 0 && x < P.V) xl = Elem<T>::get(rp, x);
  }
  Online o;
  o.init();
  online_segment<kRowBlock>(rp, P.V, seg, S, P.c, o);
  float m;
  double s;
  block_online<kRowBlock>(o, P.c, m, s);
  if (threadIdx.x == 0) {
    P.p1_m[static_cast<int64_t>(row) * S + seg] = m;
    P.p1_s[static_cast<int64_t>(row) * S + seg] = s;
    if (seg == 0) P.p1_x[row] = xl;
  }
}

template <typename T>
__global__ __launch_bounds__(kRowBlock) void k_sample_rowstats(SampleParams P) {
  const int64_t ntask = static_cast<int64_t>(P.B) * 2 * P.K * P.S1;
  for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) {
    sample_rowstats_task<T>(P, task);
    __syncthreads();  // shared memory is reused by the next task
  }
}

// ---------------------------------------------------------------- accept tests and first rejection

// Accept decisions of batch row b, computed by a whole workgroup (blockDim.x >= 64
// and >= 2K). One round of independent loads: the row statistics, the draft
// tokens' logits (fetched in pass 1), the tokens and the accept uniforms. Every
// thread returns with d.n (K when all K are accepted) and d.fault; the statistics
// of the 2K rows stay in d. With `write`, the workgroup also writes the accepted
// prefix, out_num_accepted, out_probs and the draw descriptor.
struct Decision {
  float R[2 * 64];
  double S[2 * 64];
  float prob[2 * 64];
  int n, fault;
};

__device__ __forceinline__ void decide_block(const SampleParams& P, const int b, const bool write, Decision& d) {
  const int K = P.K, S = P.S1;
  const int tid = threadIdx.x;
  if (tid < 2 * K) {
    float M;
    double Ssum;
    const int64_t r = static_cast<int64_t>(b) * 2 * K + tid;
    merge_partials(P.p1_m + r * S, P.p1_s + r * S, S, P.c, M, Ssum);
    const float R = M * P.c;
    const float xl = P.p1_x[r];
    d.R[tid] = R;
    d.S[tid] = Ssum;
    const bool ok = isfinite(M) && Ssum > 0.0 && isfinite(Ssum) && !isnan(xl);
    // p_i(x_i) (tid < K) or q_i(x_i) (tid >= K); NaN marks a row that cannot be used
    d.prob[tid] = ok ? exp2_hw(fmaf(xl, P.c, -R)) / static_cast<float>(Ssum) : __builtin_nanf("");
  }
  __syncthreads();
  if (tid < 64) {
    bool stop = false, fault = false;
    if (tid < K) {
      const int x = P.tokens[static_cast<int64_t>(b) * K + tid];
      const float p = d.prob[tid], q = d.prob[K + tid];
      if (x >= 0 && x < P.V && !isnan(p) && !isnan(q)) {
        // alpha = min(1, p/q), truncated to 1 without dividing when p >= q; 0 when p = 0
        const float alpha = (p == 0.f) ? 0.f : ((p >= q) ? 1.f : p / q);
        const float r = P.uniforms[(static_cast<int64_t>(b) * (K + 1) + tid) * 2];
        stop = !(r < alpha);
      } else {
        stop = true;
        fault = true;
      }
      if (write && P.out_probs) {
        P.out_probs[(static_cast<int64_t>(b) * K + tid) * 2] = p;
        P.out_probs[(static_cast<int64_t>(b) * K + tid) * 2 + 1] = q;
      }
    }
    const uint64_t stops = __ballot(stop);
    const uint64_t faults = __ballot(fault);
    if (tid == 0) {
      const int n = stops ? (__ffsll(static_cast<unsigned long long>(stops)) - 1) : K;
      d.n = n;
      d.fault = (n < K) && ((faults >> n) & 1ull);
    }
  }
  __syncthreads();
  if (!write) return;
  const int n = d.n;
  const bool fault = d.fault != 0;
  int32_t* ot = P.out_tokens + static_cast<int64_t>(b) * (K + 1);
  for (int i = tid; i <= K; i += blockDim.x) {
    if (fault || i > n) ot[i] = -1;
    else if (i < n) ot[i] = P.tokens[static_cast<int64_t>(b) * K + i];
  }
  if (tid == 0) {
    P.out_n[b] = fault ? -1 : n;
    P.info_n[b] = fault ? -1 : n;
    if (!fault && n < K) {
      P.info_R[2 * b] = d.R[n];
      P.info_R[2 * b + 1] = d.R[K + n];
      P.info_S[2 * b] = d.S[n];
      P.info_S[2 * b + 1] = d.S[K + n];
    }
  }
}

constexpr int kAcceptBlock = 128;  // one thread per logit row (2K <= 128)

__global__ __launch_bounds__(kAcceptBlock) void k_sample_accept(SampleParams P) {
  __shared__ Decision d;
  for (int64_t task = blockIdx.x; task < P.B; task += gridDim.x) {
    decide_block(P, static_cast<int>(task), true, d);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- pass 2: chunk masses

// Residual weight max(0, p - q) of one vocabulary entry, from the raw logits.
struct Residual {
  float c, Rt, Rq, it, iq;
  __device__ __forceinline__ float operator()(float xt, float xq) const {
    const float pt = exp2_hw(fmaf(xt, c, -Rt)) * it;
    const float pq = exp2_hw(fmaf(xq, c, -Rq)) * iq;
    return fmaxf(pt - pq, 0.f);
  }
};

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

// Pass-2 descriptor of batch row b: n in [0, K] (K = bonus draw), or false on a fault
// (also for a descriptor out of range, so a draw without its accept pass reads nothing).
__device__ __forceinline__ bool draw_row(const SampleParams& P, int b, int& n) {
  if (P.K == 0) {
    n = 0;
    return true;
  }
  n = P.info_n[b];
  return n >= 0 && n <= P.K;
}

__device__ __forceinline__ Residual residual_of(const SampleParams& P, int b) {
  Residual r;
  r.c = P.c;
  r.Rt = P.info_R[2 * b];
  r.Rq = P.info_R[2 * b + 1];
  r.it = static_cast<float>(1.0 / P.info_S[2 * b]);
  r.iq = static_cast<float>(1.0 / P.info_S[2 * b + 1]);
  return r;
}

// Draw weights of vector chunk c for this lane: the VEC weights of the lane's
// vector (zeros past the row), for the residual (two rows) or the bonus row
// (against the reference R).
template <typename T>
__device__ __forceinline__ void chunk_lane_weights(const T* tr, const T* dr, bool paired, const Chunks& ch, int c,
                                                   bool bonus, const Residual& res, float cscale, float R,
                                                   float (&w)[Elem<T>::kVec]) {
  constexpr int VEC = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int64_t vi = static_cast<int64_t>(c - 1) * kChunkVecs + lane;
  if (vi >= ch.nvec) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) w[e] = 0.f;
    return;
  }
  float xt[VEC];
  Elem<T>::vec(tr + ch.h + vi * VEC, xt);
  if (bonus) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) w[e] = exp2_hw(fmaf(xt[e], cscale, -R));
    return;
  }
  float xq[VEC];
  if (paired) {
    Elem<T>::vec(dr + ch.h + vi * VEC, xq);
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) xq[e] = Elem<T>::get(dr, ch.h + vi * VEC + e);
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) w[e] = res(xt[e], xq[e]);
}

// The mass of scalar chunk c (the head or the tail, fewer than VEC elements),
// computed by one wave; lane 0 stores (chunk max, chunk mass). Bonus chunks are
// summed against fl(chunk max * c); residual chunks store max -inf.
template <typename T>
__device__ __forceinline__ void wave_scalar_chunk_mass(const SampleParams& P, const T* tr, const T* dr,
                                                       const Chunks& ch, int c, bool bonus, const Residual& res,
                                                       float* cm, double* cs) {
  const int lane = threadIdx.x & 63;
  int64_t lo, hi;
  scalar_chunk_range<T>(ch, c, P.V, lo, hi);
  const int64_t e = lo + lane;
  const bool in = e < hi;
  const float xt = in ? Elem<T>::get(tr, e) : -INFINITY;
  float mx = -INFINITY, a = 0.f;
  if (bonus) {
    mx = wave_max(xt);
    a = (in && mx > -INFINITY) ? exp2_hw(fmaf(xt, P.c, -(mx * P.c))) : 0.f;
  } else {
    a = in ? res(xt, Elem<T>::get(dr, e)) : 0.f;
  }
  const float sum = wave_sumf(a);
  if (lane == 0) {
    cm[c] = mx;
    cs[c] = sum;
  }
}

// The masses of vector chunks c, c + cstride, ..., (CU of them, below cend),
// computed by one wave: the loads of all of them are issued before any is
// reduced, so a wave keeps CU (or 2*CU) 16-byte loads per lane in flight. Lane 0
// stores (chunk max, chunk mass).
constexpr int kChunksPerWave = 1;

template <typename T>
__device__ __forceinline__ void wave_vector_chunks_mass(const SampleParams& P, const T* tr, const T* dr,
                                                        bool paired, const Chunks& ch, int c, int cstride, int cend,
                                                        bool bonus, const Residual& res, float* cm, double* cs) {
  constexpr int VEC = Elem<T>::kVec;
  constexpr int CU = kChunksPerWave;
  const int lane = threadIdx.x & 63;
  float xt[CU][VEC], xq[CU][VEC];
#pragma unroll
  for (int u = 0; u < CU; ++u) {
    const int cu = c + u * cstride;
    const int64_t vi = static_cast<int64_t>(cu - 1) * kChunkVecs + lane;
    const bool in = (cu < cend) && vi < ch.nvec;
    if (in) {
      Elem<T>::vec(tr + ch.h + vi * VEC, xt[u]);
      if (!bonus) {
        if (paired) {
          Elem<T>::vec(dr + ch.h + vi * VEC, xq[u]);
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) xq[u][e] = Elem<T>::get(dr, ch.h + vi * VEC + e);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) xt[u][e] = xq[u][e] = -INFINITY;  // zero weight either way
    }
  }
#pragma unroll
  for (int u = 0; u < CU; ++u) {
    const int cu = c + u * cstride;
    if (cu >= cend) break;
    float mx = -INFINITY, a = 0.f;
    if (bonus) {
      float lm = xt[u][0];
#pragma unroll
      for (int e = 1; e < VEC; ++e) lm = fmaxf(lm, xt[u][e]);
      mx = wave_max(lm);
      if (mx > -INFINITY) {  // a chunk with no finite logit carries no mass
        const float R = mx * P.c;
#pragma unroll
        for (int e = 0; e < VEC; ++e) a += exp2_hw(fmaf(xt[u][e], P.c, -R));
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) a += res(xt[u][e], xq[u][e]);
    }
    const float sum = wave_sumf(a);
    if (lane == 0) {
      cm[cu] = mx;
      cs[cu] = sum;
    }
  }
}

// Pass 2 over the chunks of segment `seg`. With FUSE_ACCEPT the workgroup first
// takes the accept decisions of its batch row itself (segment 0 also writes them
// out), so no separate accept launch precedes it.
template <typename T, bool FUSE_ACCEPT>
__device__ __forceinline__ void sample_mass_task(const SampleParams& P, const int64_t task) {
  const int K = P.K, S = P.S2;
  const int seg = static_cast<int>(task % S);
  const int b = static_cast<int>(task / S);
  __shared__ Decision d;
  Residual res{};
  int n;
  if (FUSE_ACCEPT) {
    decide_block(P, b, seg == 0, d);  // with K = 0: n = 0, the bonus draw
    n = d.n;
    if (d.fault) return;
    if (n < K) {
      res.c = P.c;
      res.Rt = d.R[n];
      res.Rq = d.R[K + n];
      res.it = static_cast<float>(1.0 / d.S[n]);
      res.iq = static_cast<float>(1.0 / d.S[K + n]);
    }
  } else {
    if (!draw_row(P, b, n)) return;  // fault: nothing to draw
    if (n < K) res = residual_of(P, b);
  }
  const bool bonus = (n == K);
  const T* tr = target_row<T>(P, b, n);
  const T* dr = bonus ? tr : draft_row<T>(P, b, n);
  const Chunks ch = chunks_of(tr, P.V);
  const bool paired = bonus || head_elems(dr, P.V) == ch.h;
  float* cm = P.p2_cm + static_cast<int64_t>(b) * P.NCmax;
  double* cs = P.p2_cs + static_cast<int64_t>(b) * P.NCmax;
  // vector chunks [c0, c1) of this segment; segment 0 adds the head, the last one the tail
  const int c0 = 1 + static_cast<int>(static_cast<int64_t>(ch.nvc) * seg / S);
  const int c1 = 1 + static_cast<int>(static_cast<int64_t>(ch.nvc) * (seg + 1) / S);
  const int wave = threadIdx.x >> 6;
  constexpr int W = kBlock / 64;
  if (seg == 0 && wave == 0) wave_scalar_chunk_mass<T>(P, tr, dr, ch, 0, bonus, res, cm, cs);
  if (seg == S - 1 && wave == W - 1) wave_scalar_chunk_mass<T>(P, tr, dr, ch, ch.nvc + 1, bonus, res, cm, cs);
  for (int c = c0 + wave; c < c1; c += W * kChunksPerWave)
    wave_vector_chunks_mass<T>(P, tr, dr, paired, ch, c, W, c1, bonus, res, cm, cs);
}

template <typename T, bool FUSE_ACCEPT>
__global__ __launch_bounds__(kBlock) void k_sample_mass(SampleParams P) {
  const int64_t ntask = static_cast<int64_t>(P.B) * P.S2;
  for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) {
    sample_mass_task<T, FUSE_ACCEPT>(P, task);
    __syncthreads();  // shared memory is reused by the next task
  }
}

// ---------------------------------------------------------------- pass 2: the draw

// Inverse-CDF search over elements [lo, hi) with weights w(e), by the whole block:
// the smallest k with (sum of w over [lo, k]) > tau. Each chunk of the range gives
// every thread kSearchE contiguous elements, held in registers; chunk masses and
// thread offsets are fp64, the run inside a thread fp32. If rounding leaves no
// crossing, returns the last element with w > 0 (lo if none). Used for the rare
// zero-residual fallback, which draws from p_n over the whole row.
constexpr int kSearchE = 8;

template <typename W>
__device__ int64_t block_search(int64_t lo, int64_t hi, double tau, const W& w) {
  __shared__ int64_t sh_k;
  double base = 0.0;
  int64_t last_pos = -1;
  for (int64_t c0 = lo; c0 < hi; c0 += static_cast<int64_t>(kBlock) * kSearchE) {
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
    const double incl = block_inclusive_scan<kBlock>(static_cast<double>(ts), total);
    if (base + total > tau) {
      const double excl = incl - static_cast<double>(ts);
      const int t = block_first<kBlock>(base + incl > tau);
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
  const int64_t lp = block_max_i64<kBlock>(last_pos);
  return lp >= 0 ? lp : lo;
}

template <typename T>
__device__ __forceinline__ void sample_draw_task(const SampleParams& P, const int64_t task) {
  constexpr int VEC = Elem<T>::kVec;
  const int K = P.K;
  const int b = static_cast<int>(task);
  const int tid = threadIdx.x;
  int n;
  if (!draw_row(P, b, n)) return;  // the accept pass already wrote the fault outputs
  const bool bonus = (n == K);
  const T* tr = target_row<T>(P, b, n);
  const T* dr = bonus ? tr : draft_row<T>(P, b, n);
  const Chunks ch = chunks_of(tr, P.V);
  const int NC = ch.count();
  const float* cm = P.p2_cm + static_cast<int64_t>(b) * P.NCmax;
  const double* cs = P.p2_cs + static_cast<int64_t>(b) * P.NCmax;
  const float u = P.uniforms[(static_cast<int64_t>(b) * (K + 1) + n) * 2 + 1];
  __shared__ float sh_max[kWaves];
  __shared__ int sh_chunk;
  __shared__ double sh_tau;
  // each thread owns a contiguous run of chunks
  const int per = (NC + kBlock - 1) / kBlock;
  const int j0 = min(tid * per, NC);
  const int j1 = min(j0 + per, NC);
  float M = 0.f;
  if (bonus) {
    float lm = -INFINITY;
    for (int j = j0; j < j1; ++j) lm = fmaxf(lm, cm[j]);
    lm = wave_max(lm);
    if ((tid & 63) == 0) sh_max[tid >> 6] = lm;
    __syncthreads();
    M = sh_max[0];
    for (int i = 1; i < kWaves; ++i) M = fmaxf(M, sh_max[i]);
  }
  const double RM = static_cast<double>(M * P.c);
  auto mass = [&](int j) -> double {
    const double s = cs[j];
    if (!bonus) return s;
    return s > 0.0 ? s * exp2(static_cast<double>(cm[j] * P.c) - RM) : 0.0;
  };
  double mine = 0.0;
  int last_pos = -1;
  for (int j = j0; j < j1; ++j) {
    const double mj = mass(j);
    mine += mj;
    if (mj > 0.0) last_pos = j;
  }
  double Z;
  const double incl = block_inclusive_scan<kBlock>(mine, Z);  // chunk order, fp64
  // 0: search a chunk; 1: zero residual mass -> draw from p_n; 2: bonus row fault
  int mode = 0;
  if (bonus && !(isfinite(M) && Z > 0.0 && isfinite(Z))) mode = 2;
  else if (!bonus && !(Z > 0.0 && isfinite(Z))) mode = 1;
  int32_t* ot = P.out_tokens + static_cast<int64_t>(b) * (K + 1);
  if (mode == 2) {
    for (int i = tid; i <= K; i += kBlock) ot[i] = -1;
    if (tid == 0) P.out_n[b] = -1;
    return;
  }
  if (mode == 1) {
    // zero residual mass: draw from p_n over the whole row
    const Residual res = residual_of(P, b);
    const float c = P.c, Rt = res.Rt, it = res.it;
    auto pw = [&](int64_t e) { return exp2_hw(fmaf(Elem<T>::get(tr, e), c, -Rt)) * it; };
    float a = 0.f;
    for (int64_t e = tid; e < P.V; e += kBlock) a += pw(e);
    const double Zp = block_sum<kBlock>(static_cast<double>(a));
    const int64_t k = block_search(0, P.V, static_cast<double>(u) * Zp, pw);
    if (tid == 0) ot[n] = static_cast<int32_t>(k);
    return;
  }
  // the chunk where u*Z falls
  const double target = static_cast<double>(u) * Z;
  const int t = block_first<kBlock>(incl > target);
  if (t < kBlock) {
    if (tid == t) {
      double run = incl - mine;
      int jstar = -1;
      double tau = 0.0;
      for (int j = j0; j < j1; ++j) {
        const double mj = mass(j);
        if (run + mj > target) {
          jstar = j;
          tau = target - run;
          break;
        }
        run += mj;
      }
      if (jstar < 0) {  // rounding inside this thread's run: its last chunk with mass
        jstar = last_pos >= 0 ? last_pos : j0;
        tau = INFINITY;
      }
      sh_chunk = jstar;
      sh_tau = tau;
    }
  } else {  // rounding put u*Z at the very end: the last chunk holding mass
    const int64_t jl = block_max_i64<kBlock>(last_pos);
    if (tid == 0) {
      sh_chunk = jl >= 0 ? static_cast<int>(jl) : 0;
      sh_tau = INFINITY;
    }
  }
  __syncthreads();
  const int jstar = min(max(sh_chunk, 0), NC - 1);
  double tau = sh_tau;
  float R = 0.f;
  if (bonus) {
    R = cm[jstar] * P.c;
    tau *= exp2(RM - static_cast<double>(R));  // into the chunk's own reference
  }
  if (tid >= 64) return;  // one wave searches the chunk
  const Residual res = bonus ? Residual{} : residual_of(P, b);
  int64_t k;
  if (jstar == 0 || jstar == ch.nvc + 1) {
    int64_t lo, hi;
    scalar_chunk_range<T>(ch, jstar, P.V, lo, hi);
    if (tid != 0) return;
    float run = 0.f;
    int64_t kf = -1, kl = -1;
    for (int64_t e = lo; e < hi; ++e) {
      const float xt = Elem<T>::get(tr, e);
      const float wv = bonus ? exp2_hw(fmaf(xt, P.c, -R)) : res(xt, Elem<T>::get(dr, e));
      run += wv;
      if (wv > 0.f) kl = e;
      if (kf < 0 && static_cast<double>(run) > tau) kf = e;
    }
    k = kf >= 0 ? kf : (kl >= 0 ? kl : lo);
  } else {
    const bool paired = bonus || head_elems(dr, P.V) == ch.h;
    float w[VEC];
    chunk_lane_weights<T>(tr, dr, paired, ch, jstar, bonus, res, P.c, R, w);
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) ls += w[e];
    const double lincl = wave_inclusive_scan(static_cast<double>(ls));
    const uint64_t hit = __ballot(lincl > tau);
    const int64_t base_e = ch.h + static_cast<int64_t>(jstar - 1) * kChunkVecs * VEC;
    if (hit) {
      const int lane = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      if (tid != lane) return;
      const double excl = lincl - static_cast<double>(ls);
      float run = 0.f;
      int kk = -1, kl = -1;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        run += w[e];
        if (w[e] > 0.f) kl = e;
        if (kk < 0 && excl + static_cast<double>(run) > tau) kk = e;
      }
      k = base_e + static_cast<int64_t>(lane) * VEC + (kk >= 0 ? kk : (kl >= 0 ? kl : 0));
    } else {
      // rounding left no crossing: the last element of the chunk with weight > 0
      int kl = -1;
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        if (w[e] > 0.f) kl = e;
      int64_t best = kl >= 0 ? base_e + static_cast<int64_t>(tid) * VEC + kl : -1;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const int64_t y = __shfl_xor(best, o, 64);
        best = y > best ? y : best;
      }
      if (tid != 0) return;
      k = best >= 0 ? best : base_e;
    }
  }
  ot[n] = static_cast<int32_t>(k);
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_sample_draw(SampleParams P) {
  for (int64_t task = blockIdx.x; task < P.B; task += gridDim.x) {
    sample_draw_task<T>(P, task);
    __syncthreads();  // shared memory is reused by the next task
  }
}

// ---------------------------------------------------------------- launch

// Workgroups per launch are capped (a dispatch holds fewer than 2^32 work-items);
// every kernel loops over its tasks with a workgroup stride.
constexpr int64_t kMaxGrid = 1 << 20;

inline dim3 grid_for(int64_t tasks) { return dim3(static_cast<uint32_t>(tasks < kMaxGrid ? tasks : kMaxGrid)); }

template <typename T>
static hipError_t launch_sample_t(const SampleParams& P, int phases, hipStream_t stream) {
  if ((phases & kPhaseRowStats) && P.K > 0) {
    const int64_t g = static_cast<int64_t>(P.B) * 2 * P.K * P.S1;
    hipLaunchKernelGGL(k_sample_rowstats<T>, grid_for(g), dim3(kRowBlock), 0, stream, P);
  }
  const int64_t gm = static_cast<int64_t>(P.B) * P.S2;
  if ((phases & kPhaseAccept) && (phases & kPhaseMass)) {
    hipLaunchKernelGGL((k_sample_mass<T, true>), grid_for(gm), dim3(kBlock), 0, stream, P);
  } else if (phases & kPhaseAccept) {
    hipLaunchKernelGGL(k_sample_accept, grid_for(P.B), dim3(kAcceptBlock), 0, stream, P);
  } else if (phases & kPhaseMass) {
    hipLaunchKernelGGL((k_sample_mass<T, false>), grid_for(gm), dim3(kBlock), 0, stream, P);
  }
  if (phases & kPhaseDraw) hipLaunchKernelGGL(k_sample_draw<T>, grid_for(P.B), dim3(kBlock), 0, stream, P);
  return hipGetLastError();
}

// phases: a mask of SamplePhase bits, run in order.
hipError_t launch_sample(const SampleParams& P, bool bf16, int phases, hipStream_t stream) {
  return bf16 ? launch_sample_t<bf16_t>(P, phases, stream) : launch_sample_t<float>(P, phases, stream);
}

}  // namespace sv
