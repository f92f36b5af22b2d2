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
//   k_sample_mass      one workgroup per (b, segment). Wave 0 first takes the accept
//                      decisions of batch row b (merging the row statistics, alpha_i,
//                      and the first rejection from one 64-lane ballot) and shares the
//                      draw descriptor through LDS; wave 0 of segment 0 also writes the
//                      decisions out. Then every wave reads only
//                      the row(s) the draw needs -- target and draft row n after a
//                      rejection, or the bonus row K -- and records the draw mass of every
//                      chunk of 64 vectors (one wave load): max(0, p - q) summed, or for
//                      the bonus row the chunk's maximum and its softmax sum against it.
//   k_sample_draw      one wave per b: an fp64 DPP lane scan of the chunk masses picks the
//                      chunk where u*Z falls; the wave rereads that chunk (one 16-byte
//                      vector per lane and row) and a second lane scan finds the token.
// These short kernels are latency-bound: each dependent step (a memory round, an
// LDS round trip, a barrier) shows in the round time, so the decision and the draw
// keep to registers, DPP moves and ballots.
// k_sample_accept runs the decisions alone, for callers that run the phases apart.
#include <type_traits>

#include "../../include/spec_verify.h"
#include "common.hpp"
#include "params.hpp"
#include "rowstats.hpp"
#include "search.hpp"

namespace sv {

template <typename T>
__device__ __forceinline__ const T* target_row(const SampleParams& P, int b, int i) {
  return static_cast<const T*>(P.target) + (static_cast<int64_t>(b) * (P.K + 1) + i) * P.V;
}
template <typename T>
__device__ __forceinline__ const T* draft_row(const SampleParams& P, int b, int i) {
  return static_cast<const T*>(P.draft) + (static_cast<int64_t>(b) * P.K + i) * P.V;
}

// ---------------------------------------------------------------- row statistics (pass 1)

// Segments per row of the pass-1 stage that holds draft position `pos`.
// Rows of the pass-1 partial arrays: the stride between their segments.
__device__ __forceinline__ int64_t p1_rows(const SampleParams& P) { return static_cast<int64_t>(P.B) * 2 * P.K; }

__device__ __forceinline__ int stage_segments(const SampleParams& P, int pos) {
  int S = P.stage_S1[0];
  for (int s = 1; s < P.nstage; ++s)
    if (pos >= P.stage_end[s - 1]) S = P.stage_S1[s];
  return S;
}

// Task `task` of pass-1 stage `stage`: positions [a, e) of every batch row, target
// rows then draft rows, in memory order.
template <typename T>
__device__ __forceinline__ void rowstats_row(const SampleParams& P, const int b, const int pos, const bool is_draft,
                                             const int seg, const int S) {
  const int K = P.K;
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
    P.p1_m[seg * p1_rows(P) + row] = m;
    P.p1_s[seg * p1_rows(P) + row] = s;
    if (seg == 0) P.p1_x[row] = xl;
  }
}


// ---------------------------------------------------------------- accept tests and first rejection

// Accept decisions of batch row b, taken by one wave with no barrier; every lane
// returns the same n and fault. One round of independent loads: the row
// statistics, the draft tokens' logits (fetched in pass 1), the tokens and the
// accept uniforms. Lane l holds logit rows j = l and j = l + 64 (j < 2K; row j < K
// is target row j, else draft row j - K). With `write`, the wave also writes the
// accepted prefix, out_num_accepted, out_probs and the draw descriptor.
struct WaveDecision {
  int n;          // first rejection, K when all K are accepted (wave-uniform)
  bool fault;     // wave-uniform
  float R[2];     // per lane: reference exponents of the lane's two rows
  double S[2];    // softmax denominators (filtered rows: kept masses)
  uint32_t T[2];  // key thresholds of the filtered rows
  // values of logit row j (wave-uniform j < 2K)
  __device__ __forceinline__ float rowR(int j) const { return lane_f(j >= 64 ? R[1] : R[0], j & 63); }
  __device__ __forceinline__ double rowS(int j) const { return lane_d(j >= 64 ? S[1] : S[0], j & 63); }
  __device__ __forceinline__ uint32_t rowT(int j) const {
    return static_cast<uint32_t>(lane_i(static_cast<int>(j >= 64 ? T[1] : T[0]), j & 63));
  }
};

// Row j (< K: target row j, else draft row j - K) of batch row b in the filtered
// row order: target rows 0..K, then draft rows 0..K-1.
__device__ __forceinline__ int64_t filt_row(const SampleParams& P, int b, int j) {
  return static_cast<int64_t>(b) * (2 * P.K + 1) + (j < P.K ? j : j + 1);
}

// FILT: the rows' laws are the top-k / top-p filtered ones, described by the
// filter kernel's (reference, kept mass, key threshold) per row.
// klim < K replays the walk over positions [0, klim) only (a pass-1 stage asking
// whether its batch row is still needed): n = klim when none of them stops it.
template <bool FILT>
__device__ __forceinline__ void decide_wave(const SampleParams& P, const int b, const bool write, WaveDecision& d,
                                            const int klim) {
  const int K = P.K;
  const int lane = threadIdx.x & 63;
  // the draft token and accept uniform of position `lane`, fetched with the row statistics
  int x = 0;
  float r_acc = 0.f;
  if (lane < klim) {
    x = P.tokens[static_cast<int64_t>(b) * K + lane];
    r_acc = P.uniforms[(static_cast<int64_t>(b) * (K + 1) + lane) * 2];
  }
  float prob[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = lane + 64 * h;
    const int posj = j < K ? j : j - K;
    prob[h] = __builtin_nanf("");
    d.R[h] = 0.f;
    d.S[h] = 0.0;
    d.T[h] = 0u;
    if (j < 2 * K && posj < klim) {
      const int64_t r = static_cast<int64_t>(b) * 2 * K + j;
      const float xl = P.p1_x[r];
      if constexpr (FILT) {
        const int64_t fr = filt_row(P, b, j);
        const float R = P.f_R[fr];
        const double Ssum = P.f_S[fr];
        const uint32_t thr = P.f_thr[fr];
        d.R[h] = R;
        d.S[h] = Ssum;
        d.T[h] = thr;
        const bool ok = Ssum > 0.0 && isfinite(Ssum) && !isnan(xl);
        // p'_i(x_i) or q'_i(x_i): 0 outside the row's kept set
        prob[h] = !ok ? __builtin_nanf("")
                      : (order_key(xl) >= thr ? exp2_hw(fmaf(xl, P.c, -R)) / static_cast<float>(Ssum) : 0.f);
      } else {
        float M;
        double Ssum;
        merge_partials(P.p1_m + r, P.p1_s + r, p1_rows(P), stage_segments(P, posj), P.c, M, Ssum);
        const float R = M * P.c;
        d.R[h] = R;
        d.S[h] = Ssum;
        const bool ok = isfinite(M) && Ssum > 0.0 && isfinite(Ssum) && !isnan(xl);
        // p_i(x_i) (j < K) or q_i(x_i) (j >= K); NaN marks a row that cannot be used
        prob[h] = ok ? exp2_hw(fmaf(xl, P.c, -R)) / static_cast<float>(Ssum) : __builtin_nanf("");
      }
    }
  }
  // position i = lane: p_i(x_i) is the lane's first row, q_i(x_i) is row K + i
  const int jq = K + lane;
  const float q0 = __shfl(prob[0], jq & 63, 64);
  const float q1 = __shfl(prob[1], jq & 63, 64);
  const float p = prob[0];
  const float q = (jq < 64) ? q0 : q1;
  bool stop = false, flt = false;
  if (lane < klim) {
    if (x >= 0 && x < P.V && !isnan(p) && !isnan(q)) {
      // alpha = min(1, p/q), truncated to 1 without dividing when p >= q; 0 when p = 0
      const float alpha = (p == 0.f) ? 0.f : ((p >= q) ? 1.f : p / q);
      stop = !(r_acc < alpha);
    } else {
      stop = true;
      flt = true;
    }
  }
  const uint64_t stops = __ballot(stop);
  const uint64_t faults = __ballot(flt);
  const int n = stops ? (__ffsll(static_cast<unsigned long long>(stops)) - 1) : klim;
  const bool fault = (n < klim) && ((faults >> n) & 1ull);
  d.n = n;
  d.fault = fault;
  if (!write) return;
  int32_t* ot = P.out_tokens + static_cast<int64_t>(b) * (K + 1);
  for (int i = lane; i <= K; i += 64) {
    if (fault || i > n) ot[i] = -1;
    else if (i < n) ot[i] = x;  // i < n <= K <= 64, so i is this lane's position
  }
  if (P.out_probs && lane < K) {
    // positions after the first rejection: NaN when pass 1 may not have read them
    const bool known = P.probs_past_n || lane <= n;
    P.out_probs[(static_cast<int64_t>(b) * K + lane) * 2] = known ? p : __builtin_nanf("");
    P.out_probs[(static_cast<int64_t>(b) * K + lane) * 2 + 1] = known ? q : __builtin_nanf("");
  }
  // the draw descriptor: references and denominators of the rows the draw reads
  float R0 = 0.f, R1 = 0.f;
  double S0 = 0.0, S1 = 0.0;
  uint32_t T0 = 0u, T1 = 0u;
  if (!fault && n < K) {
    R0 = d.rowR(n);
    R1 = d.rowR(K + n);
    S0 = d.rowS(n);
    S1 = d.rowS(K + n);
    if constexpr (FILT) {
      T0 = d.rowT(n);
      T1 = d.rowT(K + n);
    }
  }
  if (lane == 0) {
    P.out_n[b] = fault ? -1 : n;
    P.info_n[b] = fault ? -1 : n;
    if (!fault && n < K) {
      P.info_R[2 * b] = R0;
      P.info_R[2 * b + 1] = R1;
      P.info_S[2 * b] = S0;
      P.info_S[2 * b + 1] = S1;
      if constexpr (FILT) {
        P.info_T[2 * b] = T0;
        P.info_T[2 * b + 1] = T1;
      }
    } else if (FILT && !fault) {  // the bonus draw from the filtered last row: no draft side
      const int64_t fr = static_cast<int64_t>(b) * (2 * K + 1) + K;
      P.info_R[2 * b] = P.f_R[fr];
      P.info_R[2 * b + 1] = 0.f;
      P.info_S[2 * b] = P.f_S[fr];
      P.info_S[2 * b + 1] = 0.0;
      P.info_T[2 * b] = P.f_thr[fr];
      P.info_T[2 * b + 1] = 0xFFFFFFFFu;
    }
  }
}

constexpr int kAcceptBlock = 64;  // one wave per batch row

template <bool FILT>
__global__ __launch_bounds__(kAcceptBlock) void k_sample_accept(SampleParams P) {
  touch_kernargs(P);
  for (int64_t task = blockIdx.x; task < P.B; task += gridDim.x) {
    WaveDecision d;
    decide_wave<FILT>(P, static_cast<int>(task), true, d, P.K);
  }
}

// ---------------------------------------------------------------- pass-1 kernel

// Pass 1, or its first stage: positions [0, e) of every batch row, target rows
// then draft rows, in memory order.
template <typename T>
__global__ __launch_bounds__(kRowBlock) void k_sample_rowstats(SampleParams P, int stage) {
  touch_kernargs(P);
  const int e = P.stage_end[stage];
  const int S = P.stage_S1[stage];
  const int64_t ntask = static_cast<int64_t>(P.B) * 2 * e * S;
  for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) {
    int64_t tq;
    int seg;
    split_task(task, S, tq, seg);
    const int t = static_cast<int>(tq);
    const bool is_draft = t >= P.B * e;
    const int tb = is_draft ? t - P.B * e : t;
    const int b = tb / e;
    rowstats_row<T>(P, b, tb - b * e, is_draft, seg, S);
    __syncthreads();  // shared memory is reused by the next task
  }
}

// Before a later stage: one wave per batch row replays the accept walk over the
// positions before the stage (from their statistics) and flags the rows it did
// not stop.
constexpr int kAliveBlock = 1024;

__global__ __launch_bounds__(kAliveBlock) void k_stage_alive(SampleParams P, int a) {
  touch_kernargs(P);
  const int64_t b = static_cast<int64_t>(blockIdx.x) * (kAliveBlock / 64) + (threadIdx.x >> 6);
  if (b >= P.B) return;  // b is uniform across the wave
  WaveDecision d;
  decide_wave<false>(P, static_cast<int>(b), false, d, a);
  if ((threadIdx.x & 63) == 0) P.stage_alive[b] = (!d.fault && d.n == a) ? 1 : 0;
}

// The li-th flagged batch row (wave-uniform; -1 past the last).
__device__ __forceinline__ int nth_alive(const SampleParams& P, int64_t li) {
  const int lane = threadIdx.x & 63;
  for (int64_t b0 = 0; b0 < P.B; b0 += 64) {
    const int64_t bb = b0 + lane;
    uint64_t m = __ballot(bb < P.B && P.stage_alive[bb] != 0);
    const int c = __popcll(m);
    if (li < c) {
      for (int64_t k = 0; k < li; ++k) m &= m - 1;
      return static_cast<int>(b0 + __ffsll(static_cast<unsigned long long>(m)) - 1);
    }
    li -= c;
  }
  return -1;
}

// A later pass-1 stage: positions [a, e) of the flagged batch rows only, their
// segments spread over a fixed grid (the count of flagged rows is known only on
// the device).
template <typename T>
__global__ __launch_bounds__(kRowBlock) void k_sample_rowstats_alive(SampleParams P, int stage) {
  touch_kernargs(P);
  const int a = P.stage_end[stage - 1];
  const int npos = P.stage_end[stage] - a;
  const int S = P.stage_S1[stage];
  const int lane = threadIdx.x & 63;
  int64_t count = 0;
  for (int64_t b0 = 0; b0 < P.B; b0 += 64) {
    const int64_t bb = b0 + lane;
    count += __popcll(__ballot(bb < P.B && P.stage_alive[bb] != 0));
  }
  const int64_t per_row = static_cast<int64_t>(2) * npos * S;
  const int64_t ntask = count * per_row;
  for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int b = nth_alive(P, task / per_row);
    const int r = static_cast<int>(task % per_row);
    const int seg = r % S;
    const int t = r / S;
    const bool is_draft = t >= npos;
    rowstats_row<T>(P, b, a + (is_draft ? t - npos : t), is_draft, seg, S);
    __syncthreads();  // shared memory is reused by the next task
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
  __device__ __forceinline__ float target(float xt) const { return exp2_hw(fmaf(xt, c, -Rt)) * it; }
};

// The same on the filtered laws: an entry outside a row's kept set (order key
// below the row's threshold) has weight 0 on that side.
struct ResidualF {
  float c, Rt, Rq, it, iq;
  uint32_t kt, kq;
  __device__ __forceinline__ float target(float xt) const {
    return order_key(xt) >= kt ? exp2_hw(fmaf(xt, c, -Rt)) * it : 0.f;
  }
  // max(0, pt - q'(xq)), pt the entry's p' value
  __device__ __forceinline__ float residual(float pt, float xq) const {
    const float pq = order_key(xq) >= kq ? exp2_hw(fmaf(xq, c, -Rq)) * iq : 0.f;
    return fmaxf(pt - pq, 0.f);
  }
  __device__ __forceinline__ float operator()(float xt, float xq) const { return residual(target(xt), xq); }
  // The kept target law p' alone (no draft side): the draw's weights when the
  // residual has no mass, and those of the filtered bonus draw.
  __device__ __forceinline__ ResidualF target_only() const {
    ResidualF r = *this;
    r.Rq = 0.f;
    r.iq = 0.f;
    r.kq = 0xFFFFFFFFu;
    return r;
  }
};

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

__device__ __forceinline__ float inv_or_zero(double s) { return s > 0.0 ? static_cast<float>(1.0 / s) : 0.f; }

__device__ __forceinline__ ResidualF residual_of_f(const SampleParams& P, int b) {
  ResidualF r;
  r.c = P.c;
  r.Rt = P.info_R[2 * b];
  r.Rq = P.info_R[2 * b + 1];
  r.it = inv_or_zero(P.info_S[2 * b]);
  r.iq = inv_or_zero(P.info_S[2 * b + 1]);
  r.kt = P.info_T[2 * b];
  r.kq = P.info_T[2 * b + 1];
  return r;
}

template <bool FILT>
using ResOf = typename std::conditional<FILT, ResidualF, Residual>::type;

// Draw weights of vector chunk c for this lane: the VEC weights of the lane's
// vector (zeros past the row), for the residual (two rows) or the bonus row
// (against the reference R).
template <typename T, typename Res>
__device__ __forceinline__ void chunk_lane_weights(const T* tr, const T* dr, bool paired, const Chunks& ch, int c,
                                                   bool bonus, const Res& res, float cscale, float R,
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
// summed against fl(chunk max * c); residual chunks store max -inf, except on the
// filtered laws, whose residual chunks store the chunk's mass of p' in place of the
// maximum (the draw's weights when the residual has no mass).
template <typename T, typename Res>
__device__ __forceinline__ void wave_scalar_chunk_mass(const SampleParams& P, const T* tr, const T* dr,
                                                       const Chunks& ch, int c, bool bonus, const Res& res,
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
  } else if constexpr (std::is_same<Res, ResidualF>::value) {
    const float pt = in ? res.target(xt) : 0.f;
    a = in ? res.residual(pt, Elem<T>::get(dr, e)) : 0.f;
    mx = wave_sumf(pt);
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
// reduced (kept as raw 16-byte vectors, so 2*CU loads per lane cost 8*CU
// registers), and lane 63 stores (chunk max, chunk mass); on the filtered laws a
// residual chunk stores its mass of p' in place of the maximum, as above. Two chunks per wave
// measured best on gfx950 (two rounds of loads per wave at the 64 x 128k shape;
// one, three or four chunks per round were 0.3-0.5 us slower per verify round).
#ifndef SV_CHUNKS_PER_WAVE
#define SV_CHUNKS_PER_WAVE 2
#endif
constexpr int kChunksPerWave = SV_CHUNKS_PER_WAVE;

template <typename T, typename Res>
__device__ __forceinline__ void wave_vector_chunks_mass(const SampleParams& P, const T* tr, const T* dr,
                                                        bool paired, const Chunks& ch, int c, int cstride, int cend,
                                                        bool bonus, const Res& res, float* cm, double* cs) {
  constexpr int VEC = Elem<T>::kVec;
  constexpr int CU = kChunksPerWave;
  const int lane = threadIdx.x & 63;
  // raw 16-byte vectors: every load of the CU chunks is issued before any is unpacked
  u32x4 rt[CU], rq[CU];
  const u32x4 none = {0u, 0u, 0u, 0u};  // placeholder for a vector that is not read (never unpacked as data)
#pragma unroll
  for (int u = 0; u < CU; ++u) {
    const int cu = c + u * cstride;
    const int64_t vi = static_cast<int64_t>(cu - 1) * kChunkVecs + lane;
    const bool in = (cu < cend) && vi < ch.nvec;
    rt[u] = in ? load_stream(tr + ch.h + vi * VEC) : none;
    rq[u] = (in && !bonus && paired) ? load_stream(dr + ch.h + vi * VEC) : none;
  }
#pragma unroll
  for (int u = 0; u < CU; ++u) {
    const int cu = c + u * cstride;
    if (cu >= cend) break;
    const int64_t vi = static_cast<int64_t>(cu - 1) * kChunkVecs + lane;
    const bool in = vi < ch.nvec;
    float xt[VEC], xq[VEC];
    Elem<T>::unpack(rt[u], xt);
    if (!in) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) xt[e] = -INFINITY;  // zero weight either way
    }
    float mx = -INFINITY, a = 0.f;
    if (bonus) {
      float lm = xt[0];
#pragma unroll
      for (int e = 1; e < VEC; ++e) lm = fmaxf(lm, xt[e]);
      mx = lane_f(wave_scan_maxf(lm), 63);
      if (mx > -INFINITY) {  // a chunk with no finite logit carries no mass
        const float R = mx * P.c;
#pragma unroll
        for (int e = 0; e < VEC; ++e) a += exp2_hw(fmaf(xt[e], P.c, -R));
      }
    } else {
      if (paired) {
        Elem<T>::unpack(rq[u], xq);
      } else if (in) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) xq[e] = Elem<T>::get(dr, ch.h + vi * VEC + e);
      }
      if (!in) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) xq[e] = -INFINITY;
      }
      if constexpr (std::is_same<Res, ResidualF>::value) {
        float ap = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float pt = res.target(xt[e]);
          ap += pt;
          a += res.residual(pt, xq[e]);
        }
        mx = wave_scan_addf(ap);  // lane 63: the chunk's mass of p'
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) a += res(xt[e], xq[e]);
      }
    }
    const float sum = wave_scan_addf(a);  // lane 63 holds the chunk's total
    if (lane == 63) {
      cm[cu] = mx;
      cs[cu] = sum;
    }
  }
}

// Pass 2 over the chunks of segment `seg`. With FUSE_ACCEPT the workgroup first
// takes the accept decisions of its batch row itself (segment 0 also writes them
// out), so no separate accept launch precedes it.
// FILT: the filtered laws; the bonus draw is then a residual with no draft side
// (its weights are the kept target masses), so no chunk maxima are needed.
template <bool FILT>
struct MassTask {
  bool run;          // false: a fault, nothing was streamed and nothing is drawn
  int n;             // the draw's position (K: the bonus draw)
  ResOf<FILT> res;   // the draw weights (residual, or the filtered bonus row)
};

// The draw weights of batch row b after its decisions d (n = d.n, no fault).
template <bool FILT>
__device__ __forceinline__ ResOf<FILT> mass_residual(const SampleParams& P, int b, const WaveDecision& d, int K) {
  ResOf<FILT> res{};
  const int n = d.n;
  if (n < K) {
    res.c = P.c;
    res.Rt = d.rowR(n);
    res.Rq = d.rowR(K + n);
    if constexpr (FILT) {
      res.it = inv_or_zero(d.rowS(n));
      res.iq = inv_or_zero(d.rowS(K + n));
      res.kt = d.rowT(n);
      res.kq = d.rowT(K + n);
    } else {
      res.it = static_cast<float>(1.0 / d.rowS(n));
      res.iq = static_cast<float>(1.0 / d.rowS(K + n));
    }
  } else if constexpr (FILT) {
    const int64_t fr = static_cast<int64_t>(b) * (2 * K + 1) + K;
    res.c = P.c;
    res.Rt = P.f_R[fr];
    res.it = inv_or_zero(P.f_S[fr]);
    res.kt = P.f_thr[fr];
    res.Rq = 0.f;
    res.iq = 0.f;
    res.kq = 0xFFFFFFFFu;
  }
  return res;
}

template <typename T, bool FUSE_ACCEPT, bool FILT, int BS = kMassBlock>
__device__ __forceinline__ MassTask<FILT> sample_mass_task(const SampleParams& P, const int b, const int seg,
                                                           const int S) {
  const int K = P.K;
  const int wave = threadIdx.x >> 6;
  MassTask<FILT> mt{false, 0, {}};
  ResOf<FILT>& res = mt.res;
  int n;
  if (FUSE_ACCEPT) {
    // Wave 0 takes the decisions (segment 0 also writes them out) and shares them
    // through LDS: deciding in every wave measured 0.9 us slower per round, the
    // CU's SIMDs issuing four copies of the same serial decision.
    __shared__ ResOf<FILT> sh_res;
    __shared__ int sh_n, sh_fault;
    if (wave == 0) {
      WaveDecision d;
      decide_wave<FILT>(P, b, seg == 0, d, K);  // with K = 0: n = 0, the bonus draw
      n = d.n;
      if (!d.fault) res = mass_residual<FILT>(P, b, d, K);
      if ((threadIdx.x & 63) == 0) {
        sh_n = n;
        sh_fault = d.fault;
        sh_res = res;
      }
    }
    __syncthreads();
    n = sh_n;
    const bool fault = sh_fault != 0;
    res = sh_res;
    __syncthreads();  // the shared values are rewritten by the next task
    if (fault) return mt;
  } else {
    if (!draw_row(P, b, n)) return mt;  // fault: nothing to draw
    if constexpr (FILT) res = residual_of_f(P, b);
    else if (n < K) res = residual_of(P, b);
  }
  mt.run = true;
  mt.n = n;
  const bool bonus = !FILT && (n == K);
  const T* tr = target_row<T>(P, b, n);
  const T* dr = (n == K) ? tr : draft_row<T>(P, b, n);
  const Chunks ch = chunks_of(tr, P.V);
  const bool paired = (n == K) || head_elems(dr, P.V) == ch.h;
  float* cm = P.p2_cm + static_cast<int64_t>(b) * P.NCmax;
  double* cs = P.p2_cs + static_cast<int64_t>(b) * P.NCmax;
  // vector chunks [c0, c1) of this segment; segment 0 adds the head, the last one the tail
  const int c0 = 1 + static_cast<int>(static_cast<int64_t>(ch.nvc) * seg / S);
  const int c1 = 1 + static_cast<int>(static_cast<int64_t>(ch.nvc) * (seg + 1) / S);
  constexpr int W = BS / 64;
  if (seg == 0 && wave == 0) wave_scalar_chunk_mass<T>(P, tr, dr, ch, 0, bonus, res, cm, cs);
  if (seg == S - 1 && wave == W - 1) wave_scalar_chunk_mass<T>(P, tr, dr, ch, ch.nvc + 1, bonus, res, cm, cs);
  for (int c = c0 + wave; c < c1; c += W * kChunksPerWave)
    wave_vector_chunks_mass<T>(P, tr, dr, paired, ch, c, W, c1, bonus, res, cm, cs);
  return mt;
}

template <typename T, bool FUSE_ACCEPT, bool FILT>
__global__ __launch_bounds__(kMassBlock) void k_sample_mass(SampleParams P) {
  touch_kernargs(P);
  const int64_t ntask = static_cast<int64_t>(P.B) * P.S2;
  for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) {
    int64_t b;
    int seg;
    split_task(task, P.S2, b, seg);
    sample_mass_task<T, FUSE_ACCEPT, FILT>(P, static_cast<int>(b), seg, P.S2);
  }
}

// ---------------------------------------------------------------- pass 2: the draw

// block_search for one wave, with no barrier: the smallest k in [lo, hi) with
// (sum of w over [lo, k]) > tau; chunk and lane offsets fp64, the run inside a
// lane fp32; the last element with w > 0 (lo if none) when rounding leaves no crossing.
__device__ __forceinline__ int64_t wave_max_i64(int64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int64_t y = __shfl_xor(v, o, 64);
    v = y > v ? y : v;
  }
  return v;
}

template <typename W>
__device__ int64_t wave_search(int64_t lo, int64_t hi, double tau, const W& w) {
  const int lane = threadIdx.x & 63;
  double base = 0.0;
  int64_t last_pos = -1;
  for (int64_t c0 = lo; c0 < hi; c0 += 64 * kSearchE) {
    const int64_t e0 = c0 + static_cast<int64_t>(lane) * kSearchE;
    float wv[kSearchE];
    float ts = 0.f;
#pragma unroll
    for (int k = 0; k < kSearchE; ++k) {
      const int64_t e = e0 + k;
      wv[k] = (e < hi) ? w(e) : 0.f;
      ts += wv[k];
      if (wv[k] > 0.f) last_pos = e;
    }
    const double incl = wave_scan_add(static_cast<double>(ts));
    const double total = lane_d(incl, 63);
    if (base + total > tau) {
      const int t = first_lane(base + incl > tau);
      const double excl = incl - static_cast<double>(ts);
      int64_t k_found = -1, k_lastpos = -1;
      float run = 0.f;
#pragma unroll
      for (int k = 0; k < kSearchE; ++k) {
        run += wv[k];
        if (wv[k] > 0.f) k_lastpos = e0 + k;
        if (k_found < 0 && base + excl + static_cast<double>(run) > tau) k_found = e0 + k;
      }
      const int64_t mine = (k_found >= 0) ? k_found : (k_lastpos >= 0 ? k_lastpos : e0);
      return __shfl(mine, t < 64 ? t : 63, 64);
    }
    base += total;
  }
  const int64_t lp = wave_max_i64(last_pos);
  return lp >= 0 ? lp : lo;
}

constexpr int kDrawBlock = 64;      // one wave per batch row
constexpr int kDrawRegChunks = 10;  // chunk masses a lane keeps in registers (enough for V up to 163840)

// A lane's contiguous run of the chunk masses of one batch row, held in registers
// by the draw (lane l owns chunks [l*per, l*per + per), per = ceil(NC / 64)).
struct DrawMasses {
  int NC;  // chunk count the runs were laid out for
  float cm[kDrawRegChunks];
  double cs[kDrawRegChunks];
};

__device__ __forceinline__ void load_draw_masses(const SampleParams& P, const int b, const int NC, DrawMasses& dm) {
  const int lane = threadIdx.x & 63;
  const float* cm = P.p2_cm + static_cast<int64_t>(b) * P.NCmax;
  const double* cs = P.p2_cs + static_cast<int64_t>(b) * P.NCmax;
  const int per = (NC + 63) / 64;
  const int j0 = min(lane * per, NC);
  const int j1 = min(j0 + per, NC);
  dm.NC = NC;
#pragma unroll
  for (int i = 0; i < kDrawRegChunks; ++i) {
    const bool in = j0 + i < j1;
    dm.cm[i] = in ? cm[j0 + i] : -INFINITY;
    dm.cs[i] = in ? cs[j0 + i] : 0.0;
  }
}

// The inverse-CDF draw of batch row b at position n (K: the bonus draw), by one
// wave with no barrier on its usual path: an fp64 lane scan of the chunk masses
// picks the chunk where u*Z falls, one reload of that chunk (one 16-byte vector
// per lane and row) and a second lane scan pick the token. `res` holds the draw
// weights (unused by the unfiltered bonus draw); `dm` the lanes' runs of chunk
// masses when they were laid out for this row's chunk count (else they are read
// again from the workspace).
template <typename T, bool FILT>
__device__ __forceinline__ void draw_core(const SampleParams& P, const int b, const int n, const float u,
                                          const ResOf<FILT>& res, const DrawMasses& dm) {
  constexpr int VEC = Elem<T>::kVec;
  const int K = P.K;
  const int lane = threadIdx.x & 63;
  const float* cm = P.p2_cm + static_cast<int64_t>(b) * P.NCmax;
  const double* cs = P.p2_cs + static_cast<int64_t>(b) * P.NCmax;
  const float (&cmr)[kDrawRegChunks] = dm.cm;
  const double (&csr)[kDrawRegChunks] = dm.cs;
  const int NC0 = dm.NC;
  const bool is_bonus = (n == K);
  const bool bonus = !FILT && is_bonus;  // chunk masses against chunk maxima (unfiltered bonus only)
  const T* tr = target_row<T>(P, b, n);
  const T* dr = is_bonus ? tr : draft_row<T>(P, b, n);
  const Chunks ch = chunks_of(tr, P.V);
  const int NC = ch.count();
  // each lane owns a contiguous run of chunks [j0, j1)
  const int per = (NC + 63) / 64;
  const int j0 = min(lane * per, NC);
  const int j1 = min(j0 + per, NC);
  // `cached`: the run is the one loaded above and fits the registers (wave-uniform)
  const bool cached = (NC == NC0) && (per <= kDrawRegChunks);
  float RMf = 0.f;
  if (bonus) {
    float lm = -INFINITY;
    if (cached) {
#pragma unroll
      for (int i = 0; i < kDrawRegChunks; ++i) lm = fmaxf(lm, cmr[i]);
    } else {
      for (int j = j0; j < j1; ++j) lm = fmaxf(lm, cm[j]);
    }
    const float M = lane_f(wave_scan_maxf(lm), 63);
    RMf = M * P.c;
    if (!isfinite(M)) {  // the bonus row has no finite logit
      int32_t* ot = P.out_tokens + static_cast<int64_t>(b) * (K + 1);
      for (int i = lane; i <= K; i += 64) ot[i] = -1;
      if (lane == 0) P.out_n[b] = -1;
      return;
    }
  }
  // Bonus chunks are rescaled from their own reference fl(max_j * c) to the row's:
  // the exponent difference is exact in fp64, 2^d comes from the hardware unit.
  auto factor = [&](float cmj) -> float {
    return exp2_hw(static_cast<float>(static_cast<double>(cmj * P.c) - static_cast<double>(RMf)));
  };
  // usep (filtered laws, wave-uniform): the residual has no mass, so the draw takes
  // p'_n, whose chunk masses pass 2 left in place of the chunk maxima
  bool usep = false;
  auto mass_of = [&](float cmj, double csj) -> double {
    if (FILT && usep) return cmj > 0.f ? static_cast<double>(cmj) : 0.0;
    if (!bonus) return csj;
    return csj > 0.0 ? csj * static_cast<double>(factor(cmj)) : 0.0;
  };
  double mine, incl, Z;
  int last_pos;
  float cm_last;
  auto totals = [&]() {
    mine = 0.0;
    last_pos = -1;
    cm_last = 0.f;
    if (cached) {
#pragma unroll
      for (int i = 0; i < kDrawRegChunks; ++i) {
        const double mj = mass_of(cmr[i], csr[i]);  // 0 past the run
        mine += mj;
        if (mj > 0.0) {
          last_pos = j0 + i;
          cm_last = cmr[i];
        }
      }
    } else {
      for (int j = j0; j < j1; ++j) {
        const double mj = mass_of(cm[j], cs[j]);
        mine += mj;
        if (mj > 0.0) last_pos = j;
      }
    }
    incl = wave_scan_add(mine);  // chunk order, fp64
    Z = lane_d(incl, 63);
  };
  totals();
  ResOf<FILT> rw = res;  // the in-chunk weights
  if constexpr (FILT) {
    if (!is_bonus && !(Z > 0.0 && isfinite(Z))) {
      usep = true;
      rw = res.target_only();
      totals();
    }
  }
  int32_t* ot = P.out_tokens + static_cast<int64_t>(b) * (K + 1);
  if (is_bonus && !(Z > 0.0 && isfinite(Z))) {  // a bonus row with no mass: fault
    for (int i = lane; i <= K; i += 64) ot[i] = -1;
    if (lane == 0) P.out_n[b] = -1;
    return;
  }
  if (!is_bonus && !(Z > 0.0 && isfinite(Z))) {
    // zero residual mass: draw from p_n over the whole row (filtered laws reach this
    // only when p'_n's chunk masses hold none either)
    auto pw = [&](int64_t e) { return res.target(Elem<T>::get(tr, e)); };
    float a = 0.f;
    for (int64_t e = lane; e < P.V; e += 64) a += pw(e);
    const double Zp = lane_d(wave_scan_add(static_cast<double>(a)), 63);
    const int64_t k = wave_search(0, P.V, static_cast<double>(u) * Zp, pw);
    if (lane == 0) ot[n] = static_cast<int32_t>(k);
    return;
  }
  // the chunk where u*Z falls: the first lane whose inclusive mass passes it
  const double target = static_cast<double>(u) * Z;
  const int t = first_lane(incl > target);
  int jstar;
  double tau;
  float cmx;
  if (t < 64) {
    // every lane walks its own run; lane t's result is the one used
    double run = incl - mine;
    int js = -1;
    double ta = 0.0;
    float cx = 0.f;
    if (cached) {
#pragma unroll
      for (int i = 0; i < kDrawRegChunks; ++i) {
        if (js < 0 && j0 + i < j1) {
          const double mj = mass_of(cmr[i], csr[i]);
          if (run + mj > target) {
            js = j0 + i;
            ta = target - run;
            cx = cmr[i];
          } else {
            run += mj;
          }
        }
      }
    } else if (lane == t) {
      for (int j = j0; j < j1; ++j) {
        const double mj = mass_of(cm[j], cs[j]);
        if (run + mj > target) {
          js = j;
          ta = target - run;
          cx = cm[j];
          break;
        }
        run += mj;
      }
    }
    if (js < 0 && lane == t) {  // rounding inside the run: its last chunk with mass
      js = last_pos >= 0 ? last_pos : j0;
      ta = INFINITY;
      cx = cached ? cm_last : cm[min(max(js, 0), NC - 1)];
    }
    jstar = lane_i(js, t);
    tau = lane_d(ta, t);
    cmx = lane_f(cx, t);
  } else {  // rounding put u*Z at the very end: the last chunk holding mass
    const int lw = last_lane(last_pos >= 0);
    jstar = lw >= 0 ? lane_i(last_pos, lw) : 0;
    tau = INFINITY;
    cmx = (lw >= 0 && cached) ? lane_f(cm_last, lw) : cm[min(max(jstar, 0), NC - 1)];
  }
  jstar = min(max(jstar, 0), NC - 1);
  float R = 0.f;
  if (bonus) {
    R = cmx * P.c;
    tau = tau / static_cast<double>(factor(cmx));  // into the chunk's own reference
  }
  int64_t k;
  if (jstar == 0 || jstar == ch.nvc + 1) {
    int64_t lo, hi;
    scalar_chunk_range<T>(ch, jstar, P.V, lo, hi);
    if (lane != 0) return;
    float run = 0.f;
    int64_t kf = -1, kl = -1;
    for (int64_t e = lo; e < hi; ++e) {
      const float xt = Elem<T>::get(tr, e);
      const float wv = bonus ? exp2_hw(fmaf(xt, P.c, -R)) : rw(xt, Elem<T>::get(dr, e));
      run += wv;
      if (wv > 0.f) kl = e;
      if (kf < 0 && static_cast<double>(run) > tau) kf = e;
    }
    k = kf >= 0 ? kf : (kl >= 0 ? kl : lo);
  } else {
    const bool paired = is_bonus || head_elems(dr, P.V) == ch.h;
    float w[VEC];
    chunk_lane_weights<T>(tr, dr, paired, ch, jstar, bonus, rw, P.c, R, w);
    float ls = 0.f;
    int kl = -1;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      ls += w[e];
      if (w[e] > 0.f) kl = e;
    }
    const double lincl = wave_scan_add(static_cast<double>(ls));
    const int hl = first_lane(lincl > tau);
    const int64_t base_e = ch.h + static_cast<int64_t>(jstar - 1) * kChunkVecs * VEC;
    if (hl < 64) {
      if (lane != hl) return;
      const double excl = lincl - static_cast<double>(ls);
      float run = 0.f;
      int kk = -1;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        run += w[e];
        if (kk < 0 && excl + static_cast<double>(run) > tau) kk = e;
      }
      k = base_e + static_cast<int64_t>(lane) * VEC + (kk >= 0 ? kk : (kl >= 0 ? kl : 0));
    } else {
      // rounding left no crossing: the last element of the chunk with weight > 0
      const int lw = last_lane(kl >= 0);
      if (lane != 0) return;
      k = lw >= 0 ? base_e + static_cast<int64_t>(lw) * VEC + lane_i(kl, lw) : base_e;
    }
  }
  ot[n] = static_cast<int32_t>(k);
}

// The draw as its own kernel: one round of loads that do not depend on the row
// the draw reads (the descriptor, every draw uniform, and the lane's run of chunk
// masses). Chunk geometry depends only on the 16-byte phase of the row, which
// every row of batch row b shares when a row is a whole number of 16-byte
// vectors; otherwise draw_core reads the masses again once the row is known.
template <typename T, bool FILT>
__device__ __forceinline__ void sample_draw_task(const SampleParams& P, const int b) {
  const int K = P.K;
  const int lane = threadIdx.x & 63;
  const int n_raw = (K == 0) ? 0 : P.info_n[b];
  const float u_lane = P.uniforms[(static_cast<int64_t>(b) * (K + 1) + min(lane, K)) * 2 + 1];
  const float dR0 = P.info_R[2 * b], dR1 = P.info_R[2 * b + 1];
  const double dS0 = P.info_S[2 * b], dS1 = P.info_S[2 * b + 1];
  uint32_t dT0 = 0u, dT1 = 0u;
  if constexpr (FILT) {
    dT0 = P.info_T[2 * b];
    dT1 = P.info_T[2 * b + 1];
  }
  DrawMasses dm;
  load_draw_masses(P, b, chunks_of(target_row<T>(P, b, 0), P.V).count(), dm);
  const int n = __builtin_amdgcn_readfirstlane(n_raw);
  if (n < 0 || n > K) return;  // the accept pass already wrote the fault outputs
  const float u = (n < 64) ? lane_f(u_lane, n) : P.uniforms[(static_cast<int64_t>(b) * (K + 1) + n) * 2 + 1];
  ResOf<FILT> res{};
  res.c = P.c;
  res.Rt = dR0;
  res.Rq = dR1;
  if constexpr (FILT) {
    res.it = inv_or_zero(dS0);
    res.iq = inv_or_zero(dS1);
    res.kt = dT0;
    res.kq = dT1;
  } else if (n < K) {
    res.it = static_cast<float>(1.0 / dS0);
    res.iq = static_cast<float>(1.0 / dS1);
  }
  draw_core<T, FILT>(P, b, n, u, res, dm);
}

template <typename T, bool FILT>
__global__ __launch_bounds__(kDrawBlock) void k_sample_draw(SampleParams P) {
  touch_kernargs(P);
  for (int64_t task = blockIdx.x; task < P.B; task += gridDim.x) sample_draw_task<T, FILT>(P, static_cast<int>(task));
}

// ---------------------------------------------------------------- launch

// Workgroups per launch are capped (a dispatch holds fewer than 2^32 work-items);
// every kernel loops over its tasks with a workgroup stride.
constexpr int64_t kMaxGrid = 1 << 20;

constexpr int64_t kAliveGrid = 2048;  // workgroups of a later pass-1 stage (one wave of them on the chip)

inline dim3 grid_for(int64_t tasks) { return dim3(static_cast<uint32_t>(tasks < kMaxGrid ? tasks : kMaxGrid)); }

hipError_t launch_filter_rows(const SampleParams& P, bool bf16, hipStream_t stream);

// FILT: the row-statistics phase is the filter kernel (all 2K+1 rows of each batch row).
template <typename T, bool FILT>
static hipError_t launch_sample_t(const SampleParams& P, int phases, hipStream_t stream) {
  if (phases & kPhaseRowStats) {
    if (FILT) {
      const hipError_t e = launch_filter_rows(P, sizeof(T) == 2, stream);
      if (e != hipSuccess) return e;
    } else if (P.K > 0) {
      hipLaunchKernelGGL(k_sample_rowstats<T>, grid_for(static_cast<int64_t>(P.B) * 2 * P.stage_end[0] * P.stage_S1[0]),
                         dim3(kRowBlock), 0, stream, P, 0);
      for (int st = 1; st < P.nstage; ++st) {
        const int a = P.stage_end[st - 1];
        hipLaunchKernelGGL(k_stage_alive, grid_for((static_cast<int64_t>(P.B) + 15) / 16), dim3(kAliveBlock), 0,
                           stream, P, a);
        const int64_t g = static_cast<int64_t>(P.B) * 2 * (P.stage_end[st] - a) * P.stage_S1[st];
        hipLaunchKernelGGL(k_sample_rowstats_alive<T>, grid_for(g < kAliveGrid ? g : kAliveGrid), dim3(kRowBlock), 0,
                           stream, P, st);
      }
    }
  }
  const int64_t gm = static_cast<int64_t>(P.B) * P.S2;
  if ((phases & kPhaseAccept) && (phases & kPhaseMass)) {
    hipLaunchKernelGGL((k_sample_mass<T, true, FILT>), grid_for(gm), dim3(kMassBlock), 0, stream, P);
  } else if (phases & kPhaseAccept) {
    hipLaunchKernelGGL(k_sample_accept<FILT>, grid_for(P.B), dim3(kAcceptBlock), 0, stream, P);
  } else if (phases & kPhaseMass) {
    hipLaunchKernelGGL((k_sample_mass<T, false, FILT>), grid_for(gm), dim3(kMassBlock), 0, stream, P);
  }
  if (phases & kPhaseDraw)
    hipLaunchKernelGGL((k_sample_draw<T, FILT>), grid_for(P.B), dim3(kDrawBlock), 0, stream, P);
  return hipGetLastError();
}

// phases: a mask of SamplePhase bits, run in order; filtered: the top-k / top-p verify.
hipError_t launch_sample(const SampleParams& P, bool bf16, bool filtered, int phases, hipStream_t stream) {
  if (filtered)
    return bf16 ? launch_sample_t<bf16_t, true>(P, phases, stream) : launch_sample_t<float, true>(P, phases, stream);
  return bf16 ? launch_sample_t<bf16_t, false>(P, phases, stream) : launch_sample_t<float, false>(P, phases, stream);
}

}  // namespace sv
