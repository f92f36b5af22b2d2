// Rejection-sampling verify kernels (gfx950).
//
// Method ("Speculative Decoding —— LLM推理优化技术（一）" §2.1-2.3; kwkr.cn/news/620797
// notes §3.1-3.4): p_i = softmax(target_i / T), q_i = softmax(draft_i / T) in fp32;
// accept x_i iff r_i < min(1, p_i(x_i) / q_i(x_i)); stop at the first rejection n
// and draw from norm(max(0, p_n - q_n)); if all K are accepted draw a bonus token
// from p_K.
//
// Pass 1 (k_sample_pass1): one workgroup per (batch row b, logit row j, segment).
// It streams its segment once with 16-byte loads and keeps an online maximum and
// sum of 2^(x*c - R) (c = log2(e)/T) per thread; a wave shuffle and an LDS step
// combine the block. The last workgroup of batch row b (arrival counter) merges
// the segments of all 2K rows, gathers the draft token's logits, computes alpha_i,
// and finds the first rejection with one 64-lane ballot over the K positions.
// The bonus row is not read in pass 1: it is needed only when all K accept.
//
// Pass 2 (k_sample_pass2): one workgroup per (b, segment) reads only the row(s)
// the draw needs -- target row n and draft row n after a rejection, or the bonus
// row K -- and sums the residual mass max(0, p - q) (or the online softmax mass of
// the bonus row) per segment. The last workgroup of b scans the segment masses in
// fp64, picks the segment where u*Z falls, rereads that segment (cache-hot) and
// searches it with a block prefix sum.
#include "common.hpp"
#include "params.hpp"

namespace sv {

// ---------------------------------------------------------------- online softmax over a segment

constexpr int kUnroll = 4;  // 16-byte vectors in flight per thread per step

template <typename T>
__device__ __forceinline__ void online_scalar(const T* row, int64_t lo, int64_t hi, float c, Online& o) {
  for (int64_t e = lo + threadIdx.x; e < hi; e += kBlock) {
    const float x = Elem<T>::get(row, e);
    if (x > o.m) o.raise(x, c);
    o.add(x, c);
  }
}

template <typename T>
__device__ __forceinline__ void online_segment(const T* row, int64_t V, int seg, int S, float c, Online& o) {
  constexpr int VEC = Elem<T>::kVec;
  const SegRange r = seg_range(row, V, seg, S);
  if (seg == 0) online_scalar(row, 0, r.head, c, o);
  const T* vb = row + r.head;
  int64_t v = r.v0 + threadIdx.x;
  for (; v + (kUnroll - 1) * kBlock < r.v1; v += kUnroll * kBlock) {
    float x[kUnroll][VEC];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) Elem<T>::vec(vb + (v + u * kBlock) * VEC, x[u]);
    float mt = x[0][0];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) mt = fmaxf(mt, x[u][e]);
    if (mt > o.m) o.raise(mt, c);
    float part[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float a = exp2_hw(fmaf(x[u][0], c, -o.R));
#pragma unroll
      for (int e = 1; e < VEC; ++e) a += exp2_hw(fmaf(x[u][e], c, -o.R));
      part[u] = a;
    }
    o.s += (part[0] + part[1]) + (part[2] + part[3]);
  }
  for (; v < r.v1; v += kBlock) {
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
  if (seg == S - 1) online_scalar(row, r.head + ((V - r.head) / VEC) * VEC, V, c, o);
}

// Combine the per-thread online states of a block. Result valid in thread 0:
// m = block maximum, s = sum against fl(m * c) in fp64.
__device__ __forceinline__ void block_online(const Online& o, float c, float& m_out, double& s_out) {
  __shared__ float sh_m[kWaves];
  __shared__ double sh_s[kWaves];
  const float mw = wave_max(o.m);
  const float Rw = mw * c;
  const float sl = (o.s > 0.f) ? o.s * exp2_hw(o.R - Rw) : 0.f;
  const double sw = wave_sum(static_cast<double>(sl));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh_m[w] = mw;
    sh_s[w] = sw;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = sh_m[0];
    for (int i = 1; i < kWaves; ++i) M = fmaxf(M, sh_m[i]);
    const double RM = static_cast<double>(M * c);
    double s = 0.0;
    for (int i = 0; i < kWaves; ++i)
      if (sh_s[i] > 0.0) s += sh_s[i] * exp2(static_cast<double>(sh_m[i] * c) - RM);
    m_out = M;
    s_out = s;
  }
}

// Merge segment partials (m_j, s_j) of one row, in segment order.
__device__ __forceinline__ void merge_partials(const float* pm, const double* ps, int S, float c, float& M,
                                               double& Ssum) {
  M = -INFINITY;
  for (int j = 0; j < S; ++j) M = fmaxf(M, ld_agent(pm + j));
  const double RM = static_cast<double>(M * c);
  Ssum = 0.0;
  for (int j = 0; j < S; ++j) {
    const double sj = ld_agent(ps + j);
    if (sj > 0.0) Ssum += sj * exp2(static_cast<double>(ld_agent(pm + j) * c) - RM);
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

// ---------------------------------------------------------------- pass 1

template <typename T>
__global__ __launch_bounds__(kBlock) void k_sample_pass1(SampleParams P) {
  const int K = P.K, S = P.S1;
  const int seg = blockIdx.x % S;
  const int row = blockIdx.x / S;  // in [0, B*2K): j < K target row j, else draft row j-K
  const int b = row / (2 * K);
  const int j = row - b * 2 * K;
  const T* rp = (j < K) ? target_row<T>(P, b, j) : draft_row<T>(P, b, j - K);

  Online o;
  o.init();
  online_segment(rp, P.V, seg, S, P.c, o);
  float m;
  double s;
  block_online(o, P.c, m, s);
  if (threadIdx.x == 0) {
    st_agent(P.p1_m + static_cast<int64_t>(row) * S + seg, m);
    st_agent(P.p1_s + static_cast<int64_t>(row) * S + seg, s);
  }
  if (!arrive_last(P.cnt1 + b, static_cast<uint32_t>(2 * K * S))) return;

  // ---- epilogue of batch row b: accept tests and the first rejection
  __shared__ float sh_M[2 * 64];
  __shared__ float sh_R[2 * 64];
  __shared__ double sh_S[2 * 64];
  __shared__ int sh_n, sh_fault;
  const int tid = threadIdx.x;
  if (tid < 2 * K) {
    float M;
    double Ssum;
    const int64_t r0 = (static_cast<int64_t>(b) * 2 * K + tid) * S;
    merge_partials(P.p1_m + r0, P.p1_s + r0, S, P.c, M, Ssum);
    sh_M[tid] = M;
    sh_R[tid] = M * P.c;
    sh_S[tid] = Ssum;
  }
  __syncthreads();
  if (tid < 64) {
    bool stop = false, fault = false;
    if (tid < K) {
      float p = __builtin_nanf(""), q = __builtin_nanf("");
      const int x = P.tokens[static_cast<int64_t>(b) * K + tid];
      const float Mt = sh_M[tid], Mq = sh_M[K + tid];
      const double St = sh_S[tid], Sq = sh_S[K + tid];
      const bool ok = x >= 0 && x < P.V && isfinite(Mt) && isfinite(Mq) && St > 0.0 && Sq > 0.0 &&
                      isfinite(St) && isfinite(Sq);
      if (ok) {
        const float xt = Elem<T>::get(target_row<T>(P, b, tid), x);
        const float xq = Elem<T>::get(draft_row<T>(P, b, tid), x);
        p = exp2_hw(fmaf(xt, P.c, -sh_R[tid])) / static_cast<float>(St);
        q = exp2_hw(fmaf(xq, P.c, -sh_R[K + tid])) / static_cast<float>(Sq);
        // alpha = min(1, p/q), truncated to 1 without dividing when p >= q; 0 when p = 0
        const float alpha = (p == 0.f) ? 0.f : ((p >= q) ? 1.f : p / q);
        const float r = P.uniforms[(static_cast<int64_t>(b) * (K + 1) + tid) * 2];
        stop = !(r < alpha);
      } else {
        stop = true;
        fault = true;
      }
      if (P.out_probs) {
        P.out_probs[(static_cast<int64_t>(b) * K + tid) * 2] = p;
        P.out_probs[(static_cast<int64_t>(b) * K + tid) * 2 + 1] = q;
      }
    }
    const uint64_t stops = __ballot(stop);
    const uint64_t faults = __ballot(fault);
    if (tid == 0) {
      const int n = stops ? (__ffsll(static_cast<unsigned long long>(stops)) - 1) : K;
      sh_n = n;
      sh_fault = (n < K) && ((faults >> n) & 1ull);
    }
  }
  __syncthreads();
  const int n = sh_n;
  const bool fault = sh_fault != 0;
  int32_t* ot = P.out_tokens + static_cast<int64_t>(b) * (K + 1);
  for (int i = tid; i <= K; i += kBlock) {
    if (fault || i > n) ot[i] = -1;
    else if (i < n) ot[i] = P.tokens[static_cast<int64_t>(b) * K + i];
  }
  if (tid == 0) {
    P.out_n[b] = fault ? -1 : n;
    P.info_n[b] = fault ? -1 : n;
    if (!fault && n < K) {
      P.info_R[2 * b] = sh_R[n];
      P.info_R[2 * b + 1] = sh_R[K + n];
      P.info_S[2 * b] = sh_S[n];
      P.info_S[2 * b + 1] = sh_S[K + n];
    }
  }
}

// ---------------------------------------------------------------- pass 2

// Residual weight max(0, p - q) of one vocabulary entry, from the raw logits.
struct Residual {
  float c, Rt, Rq, it, iq;
  __device__ __forceinline__ float operator()(float xt, float xq) const {
    const float pt = exp2_hw(fmaf(xt, c, -Rt)) * it;
    const float pq = exp2_hw(fmaf(xq, c, -Rq)) * iq;
    return fmaxf(pt - pq, 0.f);
  }
};

template <typename T>
__device__ __forceinline__ float residual_segment(const T* tr, const T* dr, int64_t V, int seg, int S,
                                                  const Residual& w) {
  constexpr int VEC = Elem<T>::kVec;
  const SegRange r = seg_range(tr, V, seg, S);
  float acc = 0.f;
  const bool paired = head_elems(dr, V) == r.head;
  if (paired) {
    if (seg == 0)
      for (int64_t e = threadIdx.x; e < r.head; e += kBlock) acc += w(Elem<T>::get(tr, e), Elem<T>::get(dr, e));
    const T* tb = tr + r.head;
    const T* db = dr + r.head;
    int64_t v = r.v0 + threadIdx.x;
    for (; v + kBlock < r.v1; v += 2 * kBlock) {
      float xt[2][VEC], xq[2][VEC];
      Elem<T>::vec(tb + v * VEC, xt[0]);
      Elem<T>::vec(db + v * VEC, xq[0]);
      Elem<T>::vec(tb + (v + kBlock) * VEC, xt[1]);
      Elem<T>::vec(db + (v + kBlock) * VEC, xq[1]);
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        a0 += w(xt[0][e], xq[0][e]);
        a1 += w(xt[1][e], xq[1][e]);
      }
      acc += a0 + a1;
    }
    for (; v < r.v1; v += kBlock) {
      float xt[VEC], xq[VEC];
      Elem<T>::vec(tb + v * VEC, xt);
      Elem<T>::vec(db + v * VEC, xq);
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) a += w(xt[e], xq[e]);
      acc += a;
    }
    if (seg == S - 1)
      for (int64_t e = r.head + ((V - r.head) / VEC) * VEC + threadIdx.x; e < V; e += kBlock)
        acc += w(Elem<T>::get(tr, e), Elem<T>::get(dr, e));
  } else {
    // the two rows sit at different 16-byte phases: element loads
    for (int64_t e = r.lo + threadIdx.x; e < r.hi; e += kBlock) acc += w(Elem<T>::get(tr, e), Elem<T>::get(dr, e));
  }
  return acc;
}

__device__ __forceinline__ double block_sum(double v) {
  __shared__ double sh[kWaves];
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < kWaves; ++i) t += sh[i];
  __syncthreads();
  return t;
}

// Inclusive prefix sum over the block (thread order), fp64. Also returns the block total.
__device__ __forceinline__ double block_inclusive_scan(double v, double& total) {
  __shared__ double sh[kWaves];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) sh[w] = v;
  __syncthreads();
  double before = 0.0;
  total = 0.0;
  for (int i = 0; i < kWaves; ++i) {
    if (i < w) before += sh[i];
    total += sh[i];
  }
  __syncthreads();
  return before + v;
}

// Lowest thread index whose predicate holds (kBlock if none), in every thread.
__device__ __forceinline__ int block_first(bool pred) {
  __shared__ uint64_t sh[kWaves];
  const uint64_t bal = __ballot(pred);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = bal;
  __syncthreads();
  int first = kBlock;
  for (int i = kWaves - 1; i >= 0; --i)
    if (sh[i]) first = i * 64 + (__ffsll(static_cast<unsigned long long>(sh[i])) - 1);
  __syncthreads();
  return first;
}

__device__ __forceinline__ int64_t block_max_i64(int64_t v) {
  __shared__ int64_t sh[kWaves];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int64_t y = __shfl_xor(v, o, 64);
    v = y > v ? y : v;
  }
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  int64_t t = sh[0];
  for (int i = 1; i < kWaves; ++i) t = sh[i] > t ? sh[i] : t;
  __syncthreads();
  return t;
}

// Inverse-CDF search over elements [lo, hi) with weights w(e): the smallest k
// with (sum of w over [lo, k]) > tau. Each chunk gives every thread E contiguous
// elements; chunk masses and thread offsets are in fp64, the run inside a
// thread in fp32 (the same order as its chunk sum). If rounding leaves no
// crossing, returns the last element with w > 0 (lo if there is none).
constexpr int kSearchE = 16;

template <typename W>
__device__ int64_t block_search(int64_t lo, int64_t hi, double tau, const W& w) {
  __shared__ int64_t sh_k;
  double base = 0.0;
  int64_t last_pos = -1;
  for (int64_t c0 = lo; c0 < hi; c0 += static_cast<int64_t>(kBlock) * kSearchE) {
    const int64_t e0 = c0 + static_cast<int64_t>(threadIdx.x) * kSearchE;
    float ts = 0.f;
    for (int k = 0; k < kSearchE; ++k) {
      const int64_t e = e0 + k;
      if (e < hi) {
        const float wv = w(e);
        ts += wv;
        if (wv > 0.f) last_pos = e;
      }
    }
    double total;
    const double incl = block_inclusive_scan(static_cast<double>(ts), total);
    if (base + total > tau) {
      const double excl = incl - static_cast<double>(ts);
      const int t = block_first(base + incl > tau);
      if (static_cast<int>(threadIdx.x) == t) {
        int64_t k_found = -1, k_lastpos = -1;
        float run = 0.f;
        for (int k = 0; k < kSearchE; ++k) {
          const int64_t e = e0 + k;
          if (e >= hi) break;
          const float wv = w(e);
          run += wv;
          if (wv > 0.f) k_lastpos = e;
          if (base + excl + static_cast<double>(run) > tau) {
            k_found = e;
            break;
          }
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
  const int64_t lp = block_max_i64(last_pos);
  return lp >= 0 ? lp : lo;
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_sample_pass2(SampleParams P) {
  const int K = P.K, S = P.S2;
  const int seg = blockIdx.x % S;
  const int b = blockIdx.x / S;
  int n = K;
  bool fault = false;
  if (K > 0) {
    const int ni = P.info_n[b];
    fault = ni < 0 || ni > K;  // a descriptor out of range (no matching pass 1) draws nothing
    n = fault ? 0 : ni;
  }
  const bool bonus = (n == K);
  float pm = 0.f;
  double ps = 0.0;
  Residual res{};
  if (!fault) {
    if (bonus) {
      Online o;
      o.init();
      online_segment(target_row<T>(P, b, K), P.V, seg, S, P.c, o);
      block_online(o, P.c, pm, ps);
    } else {
      res.c = P.c;
      res.Rt = P.info_R[2 * b];
      res.Rq = P.info_R[2 * b + 1];
      res.it = static_cast<float>(1.0 / P.info_S[2 * b]);
      res.iq = static_cast<float>(1.0 / P.info_S[2 * b + 1]);
      const float a = residual_segment(target_row<T>(P, b, n), draft_row<T>(P, b, n), P.V, seg, S, res);
      ps = block_sum(static_cast<double>(a));
    }
  }
  if (threadIdx.x == 0) {
    st_agent(P.p2_m + static_cast<int64_t>(b) * S + seg, pm);
    st_agent(P.p2_s + static_cast<int64_t>(b) * S + seg, ps);
  }
  if (!arrive_last(P.cnt2 + b, static_cast<uint32_t>(S))) return;
  if (fault) return;  // pass 1 already wrote the fault outputs

  // ---- epilogue of batch row b: choose the segment, then search inside it
  __shared__ int sh_seg, sh_mode;
  __shared__ double sh_tau;
  __shared__ float sh_Rseg;
  const float u = P.uniforms[(static_cast<int64_t>(b) * (K + 1) + n) * 2 + 1];
  if (threadIdx.x == 0) {
    const float* qm = P.p2_m + static_cast<int64_t>(b) * S;
    const double* qs = P.p2_s + static_cast<int64_t>(b) * S;
    float M = -INFINITY;
    double RM = 0.0;
    if (bonus) {
      for (int j = 0; j < S; ++j) M = fmaxf(M, ld_agent(qm + j));
      RM = static_cast<double>(M * P.c);
    }
    double Z = 0.0;
    for (int j = 0; j < S; ++j) {
      const double sj = ld_agent(qs + j);
      Z += bonus ? (sj > 0.0 ? sj * exp2(static_cast<double>(ld_agent(qm + j) * P.c) - RM) : 0.0) : sj;
    }
    int mode = 0;  // 0: search a segment, 1: residual mass is zero -> draw from p_n, 2: bonus row fault
    if (bonus && !(isfinite(M) && Z > 0.0 && isfinite(Z))) mode = 2;
    else if (!bonus && !(Z > 0.0)) mode = 1;
    int jstar = -1;
    double tau = 0.0;
    float Rseg = 0.f;
    if (mode == 0) {
      const double target = static_cast<double>(u) * Z;
      double Pj = 0.0;
      int jlast = -1;
      for (int j = 0; j < S; ++j) {
        const double sj = ld_agent(qs + j);
        const double mj = bonus ? (sj > 0.0 ? sj * exp2(static_cast<double>(ld_agent(qm + j) * P.c) - RM) : 0.0) : sj;
        if (mj > 0.0) jlast = j;
        if (jstar < 0 && Pj + mj > target) {
          jstar = j;
          tau = target - Pj;
          if (bonus) {
            Rseg = ld_agent(qm + j) * P.c;
            tau *= exp2(RM - static_cast<double>(Rseg));  // into the segment's own reference
          }
        }
        Pj += mj;
      }
      if (jstar < 0) {  // rounding: u*Z at the very end; take the last segment holding mass
        jstar = jlast;
        tau = INFINITY;
        if (bonus) Rseg = ld_agent(qm + jlast) * P.c;
      }
    }
    sh_mode = mode;
    sh_seg = jstar;
    sh_tau = tau;
    sh_Rseg = Rseg;
  }
  __syncthreads();
  const int mode = sh_mode;
  int32_t* ot = P.out_tokens + static_cast<int64_t>(b) * (K + 1);
  if (mode == 2) {
    for (int i = threadIdx.x; i <= K; i += kBlock) ot[i] = -1;
    if (threadIdx.x == 0) P.out_n[b] = -1;
    return;
  }
  int64_t k;
  if (mode == 0) {
    const int j = sh_seg;
    const double tau = sh_tau;
    if (bonus) {
      const T* br = target_row<T>(P, b, K);
      const SegRange r = seg_range(br, P.V, j, S);
      const float c = P.c, R = sh_Rseg;
      k = block_search(r.lo, r.hi, tau, [&](int64_t e) { return exp2_hw(fmaf(Elem<T>::get(br, e), c, -R)); });
    } else {
      const T* tr = target_row<T>(P, b, n);
      const T* dr = draft_row<T>(P, b, n);
      const SegRange r = seg_range(tr, P.V, j, S);
      k = block_search(r.lo, r.hi, tau,
                       [&](int64_t e) { return res(Elem<T>::get(tr, e), Elem<T>::get(dr, e)); });
    }
  } else {
    // zero residual mass: draw from p_n over the whole row
    const T* tr = target_row<T>(P, b, n);
    const float c = P.c, Rt = res.Rt, it = res.it;
    auto pw = [&](int64_t e) { return exp2_hw(fmaf(Elem<T>::get(tr, e), c, -Rt)) * it; };
    float a = 0.f;
    for (int64_t e = threadIdx.x; e < P.V; e += kBlock) a += pw(e);
    const double Zp = block_sum(static_cast<double>(a));
    k = block_search(0, P.V, static_cast<double>(u) * Zp, pw);
  }
  if (threadIdx.x == 0) {
    ot[n] = static_cast<int32_t>(k);
    if (K == 0) P.out_n[b] = 0;
  }
}

// ---------------------------------------------------------------- launch

template <typename T>
static hipError_t launch_sample_t(const SampleParams& P, int phases, hipStream_t stream) {
  if ((phases & 1) && P.K > 0) {
    const int64_t g1 = static_cast<int64_t>(P.B) * 2 * P.K * P.S1;
    hipLaunchKernelGGL(k_sample_pass1<T>, dim3(static_cast<uint32_t>(g1)), dim3(kBlock), 0, stream, P);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & 2) {
    const int64_t g2 = static_cast<int64_t>(P.B) * P.S2;
    hipLaunchKernelGGL(k_sample_pass2<T>, dim3(static_cast<uint32_t>(g2)), dim3(kBlock), 0, stream, P);
    return hipGetLastError();
  }
  return hipSuccess;
}

// phases: bit 0 = pass 1 (accept tests), bit 1 = pass 2 (the draw).
hipError_t launch_sample(const SampleParams& P, bool bf16, int phases, hipStream_t stream) {
  return bf16 ? launch_sample_t<bf16_t>(P, phases, stream) : launch_sample_t<float>(P, phases, stream);
}

}  // namespace sv
