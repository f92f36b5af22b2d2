// Sampling verify of greedy-drafted (one-hot) n-gram candidates (gfx950).
//
// Method ("Lookahead Decoding 完全拆解:Jacobi 迭代与 N-gram 池", section "采样模式的
// 验证"; "Speculative Decoding —— LLM推理优化技术（一）" §2.1): a candidate token x
// drafted greedily has the one-hot law q = delta_x, so it is accepted with
// probability min(1, p(x) / 1) = p(x), and a rejection leaves the residual
// norm(max(0, p - delta_x)): p with x removed. With G disjoint candidates the
// active ones (whose prefix matches the tokens accepted so far) are tried in
// index order at each position, on the law of the lowest active candidate's row;
// each rejection removes its token; an acceptance keeps the candidates carrying
// the token; when every try fails the token is drawn from the remaining mass;
// after N-1 accepted tokens a bonus token is drawn from row N-1.
//
// Kernels, in stream order:
//   k_ngs_rowstats  one workgroup per (row, segment) of all B*G*N target rows:
//                   the online (max, sum 2^(x*c - R)) of the segment, and the sum of
//                   every block of 256 16-byte vectors with its reference R; segment 0
//                   of a row (g, i < N-1) also gathers the logits of every
//                   candidate's token at position i, so the walk needs no further
//                   look at a row. A row of at most 16 blocks (64 KB) is read in one
//                   shot, every load issued at once; longer ones block after block.
//   k_ngs_verify    one workgroup per sequence. One round of loads stages the
//                   sequence's row statistics, candidates, uniforms and gathered
//                   logits in LDS; wave 0 walks the positions and tries (a few dozen
//                   scalar steps); the draw then takes the block masses from pass 1,
//                   reloads only the blocks holding a rejected token, picks the block
//                   and reloads it to find the token.
#include "../../include/spec_verify.h"
#include "common.hpp"
#include "params.hpp"
#include "rowstats.hpp"
#include "search.hpp"

namespace sv {

__device__ __forceinline__ int64_t ngs_row(const NgramSampleParams& P, int b, int g, int i) {
  return (static_cast<int64_t>(b) * P.G + g) * P.N + i;
}

template <typename T>
__device__ __forceinline__ const T* ngs_row_ptr(const NgramSampleParams& P, int64_t row) {
  return static_cast<const T*>(P.logits) + row * P.V;
}

// ---------------------------------------------------------------- row blocks

// Blocks of a row: kNgsBlkVecs 16-byte vectors each (the last one possibly fewer),
// counted from the row's first 16-byte boundary. The scalar head before that
// boundary and the scalar tail after the last whole vector belong to no block.
struct RowBlocks {
  int64_t h;        // head elements
  int64_t nvec;     // whole vectors after the head
  int64_t tail_lo;  // first tail element
  int nb;           // vector blocks
};

template <typename T>
__device__ __forceinline__ RowBlocks blocks_of(const T* row, int64_t V) {
  RowBlocks rb;
  rb.h = head_elems(row, V);
  rb.nvec = (V - rb.h) / Elem<T>::kVec;
  rb.tail_lo = rb.h + rb.nvec * Elem<T>::kVec;
  rb.nb = static_cast<int>((rb.nvec + kNgsBlkVecs - 1) / kNgsBlkVecs);
  return rb;
}

constexpr int kBlkChunks = kNgsBlkVecs / 64;  // one coalesced 16-byte load per lane each
static_assert(kBlkChunks * 64 == kNgsBlkVecs, "a block is a whole number of wave loads");

// The lane's raw vectors of vector block k (zero past the row's last whole vector),
// through a buffer resource over the row's whole vectors (V <= 2^20 keeps its
// bytes below 2^31).
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t vectors_of(const T* rp, const RowBlocks& rb) {
  return buffer_over(rp + rb.h, rb.nvec * 16);
}

__device__ __forceinline__ void load_block(__amdgpu_buffer_rsrc_t rs, int64_t k, u32x4 (&raw)[kBlkChunks]) {
  const int v0 = static_cast<int>(k) * kNgsBlkVecs + (threadIdx.x & 63);
#pragma unroll
  for (int u = 0; u < kBlkChunks; ++u) raw[u] = load_stream_buf(rs, v0 + u * 64);
}

// ---------------------------------------------------------------- pass 1

// One workgroup per (row, segment); a segment is a run of whole blocks (segment 0
// also takes the head, the last segment the tail). Each wave takes every
// kNgsRowWaves-th block, issuing the next block's kBlkChunks loads before it reduces
// the current one. A ballot spots a new maximum, whose wave reduction then raises
// the wave's running reference R = fl(m*c); the block's sum of 2^(x*c - R) is stored
// with that R, so any later reference R' recovers the block's mass as
// sum * 2^(R - R'). The waves' running (m, sum) then merge into the segment's
// partial, as the online softmax does.
#ifndef SV_NGS_ROW_WAVES
#define SV_NGS_ROW_WAVES 4
#endif
constexpr int kNgsRowWaves = SV_NGS_ROW_WAVES;
constexpr int kNgsRowBlock = 64 * kNgsRowWaves;

// A row of at most kNgsShotBlocks blocks per wave is read in one shot: every wave
// issues the loads of all its blocks at once (the whole row is in flight), takes its
// maximum over them, fixes R = fl(m*c) and then sums each block against that R.
#ifndef SV_NGS_SHOT_BLOCKS
#define SV_NGS_SHOT_BLOCKS 4
#endif
constexpr int kNgsShotBlocks = SV_NGS_SHOT_BLOCKS;

// Raw words that widen to -inf: two bf16 -inf, or one fp32 -inf.
template <typename T>
__device__ __forceinline__ uint32_t neg_inf_word();
template <>
__device__ __forceinline__ uint32_t neg_inf_word<bf16_t>() { return 0xFF80FF80u; }
template <>
__device__ __forceinline__ uint32_t neg_inf_word<float>() { return 0xFF800000u; }

// The wave's (m, sum of 2^(x*c - fl(m*c))) over its blocks wave, wave + kNgsRowWaves, ...
// of a row with rb.nb <= kNgsShotBlocks * kNgsRowWaves, and the scalar entries xs (-inf
// where a lane holds none); each block's sum is stored with that reference.
template <typename T>
__device__ __forceinline__ void ngs_row_shot(__amdgpu_buffer_rsrc_t rs, const RowBlocks& rb, int wave, float xs,
                                             float c, float2* bs, float& m_out, double& s_out) {
  constexpr int VEC = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int nvec = static_cast<int>(rb.nvec);  // < 2^31: the row's bytes fit a buffer resource
  u32x4 raw[kNgsShotBlocks][kBlkChunks];
#pragma unroll
  for (int j = 0; j < kNgsShotBlocks; ++j) {
    const int k = wave + j * kNgsRowWaves;
    load_block(rs, k < rb.nb ? k : rb.nb, raw[j]);  // past the row: reads zeros, replaced below
  }
  // vectors past the row's last whole one (the last block's tail, and every block past
  // the row) become -inf words, so the passes below need no mask
#pragma unroll
  for (int j = 0; j < kNgsShotBlocks; ++j) {
    const int k = wave + j * kNgsRowWaves;
    if ((k + 1) * kNgsBlkVecs > nvec) {  // wave-uniform
#pragma unroll
      for (int u = 0; u < kBlkChunks; ++u) {
        const bool in = k * kNgsBlkVecs + u * 64 + lane < nvec;
        const uint32_t ni = neg_inf_word<T>();
        raw[j][u] = in ? raw[j][u] : u32x4{ni, ni, ni, ni};
      }
    }
  }
  float mt = xs;
#pragma unroll
  for (int j = 0; j < kNgsShotBlocks; ++j)
#pragma unroll
    for (int u = 0; u < kBlkChunks; ++u) {
      float x[VEC];
      Elem<T>::unpack(raw[j][u], x);
#pragma unroll
      for (int e = 0; e < VEC; ++e) mt = fmaxf(mt, x[e]);
    }
  const float m = lane_f(wave_scan_maxf(mt), 63);
  const float R = (m > -INFINITY) ? m * c : 0.f;  // 0 while the wave holds no number: every term is 0
  // the sums widen the raw words again rather than keep every widened entry alive
  // from the maximum's pass (which would double the registers)
#pragma unroll
  for (int j = 0; j < kNgsShotBlocks; ++j)
#pragma unroll
    for (int u = 0; u < kBlkChunks; ++u) asm volatile("" : "+v"(raw[j][u]));
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < kNgsShotBlocks; ++j) {
    const int k = wave + j * kNgsRowWaves;
    float a = 0.f;
#pragma unroll
    for (int u = 0; u < kBlkChunks; ++u) {
      float x[VEC];
      Elem<T>::unpack(raw[j][u], x);
#pragma unroll
      for (int e = 0; e < VEC; ++e) a += exp2_hw(fmaf(x[e], c, -R));
    }
    const float sb = lane_f(wave_scan_addf(a), 63);
    s += static_cast<double>(sb);
    if (lane == 0 && k < rb.nb) bs[k] = make_float2(R, sb);
  }
  if (wave == 0) s += static_cast<double>(lane_f(wave_scan_addf(exp2_hw(fmaf(xs, c, -R))), 63));
  m_out = m;
  s_out = s;
}

// The wave's (m, sum of 2^(x*c - fl(m*c))) over its blocks of segment seg of S, read
// block after block (the next block's loads issued before this one is reduced), and
// the scalar entries xs; each block's sum is stored with the reference it was summed
// against.
template <typename T>
__device__ __forceinline__ void ngs_row_pipelined(__amdgpu_buffer_rsrc_t rs, const RowBlocks& rb, int seg, int S,
                                                  int wave, float xs, float c, float2* bs, float& m_out,
                                                  double& s_out) {
  constexpr int VEC = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;  // the wave's running maximum; R = fl(m*c), 0 while m == -inf
  float R = 0.f;
  double s = 0.0;
  const int64_t b0 = static_cast<int64_t>(rb.nb) * seg / S, b1 = static_cast<int64_t>(rb.nb) * (seg + 1) / S;
  // software pipeline: the next block's loads are issued before this block is
  // reduced; past the segment they aim past the row's end, which reads nothing
  u32x4 raw[kBlkChunks], nxt[kBlkChunks];
  int64_t k = b0 + wave;
  load_block(rs, k < b1 ? k : rb.nb, raw);
  for (; k < b1; k += kNgsRowWaves) {
    load_block(rs, k + kNgsRowWaves < b1 ? k + kNgsRowWaves : rb.nb, nxt);
    float x[kBlkChunks][VEC];
#pragma unroll
    for (int u = 0; u < kBlkChunks; ++u) Elem<T>::unpack(raw[u], x[u]);
    if ((k + 1) * kNgsBlkVecs > rb.nvec) {  // the row's last block, not whole
#pragma unroll
      for (int u = 0; u < kBlkChunks; ++u) {
        const bool in = k * kNgsBlkVecs + u * 64 + lane < rb.nvec;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          if (!in) x[u][e] = -INFINITY;
      }
    }
    float mt = x[0][0];
#pragma unroll
    for (int u = 0; u < kBlkChunks; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) mt = fmaxf(mt, x[u][e]);
    if (__ballot(mt > m)) {  // a new running maximum (the wave reduction only then)
      const float bm = lane_f(wave_scan_maxf(mt), 63);
      const float Rn = bm * c;
      s = (s > 0.0) ? s * static_cast<double>(exp2_hw(static_cast<float>(static_cast<double>(R) - Rn))) : 0.0;
      m = bm;
      R = Rn;
    }
    float a = 0.f;
#pragma unroll
    for (int u = 0; u < kBlkChunks; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) a += exp2_hw(fmaf(x[u][e], c, -R));
    const float sb = lane_f(wave_scan_addf(a), 63);
    s += static_cast<double>(sb);
    if (lane == 0) bs[k] = make_float2(R, sb);
#pragma unroll
    for (int u = 0; u < kBlkChunks; ++u) raw[u] = nxt[u];
  }
  if (wave == 0) {
    const float bm = lane_f(wave_scan_maxf(xs), 63);
    if (bm > m) {
      const float Rn = bm * c;
      s = (s > 0.0) ? s * static_cast<double>(exp2_hw(static_cast<float>(static_cast<double>(R) - Rn))) : 0.0;
      m = bm;
      R = Rn;
    }
    s += static_cast<double>(lane_f(wave_scan_addf(exp2_hw(fmaf(xs, c, -R))), 63));
  }
  m_out = m;
  s_out = s;
}

template <typename T>
__global__ __launch_bounds__(kNgsRowBlock) void k_ngs_rowstats(NgramSampleParams P) {
  touch_kernargs(P);
  __shared__ float sh_m[kNgsRowWaves];
  __shared__ double sh_s[kNgsRowWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int S = P.S1;
  const float c = P.c;
  const int64_t rows = static_cast<int64_t>(P.B) * P.G * P.N;
  for (int64_t task = blockIdx.x; task < rows * S; task += gridDim.x) {
    int64_t row, bg, bq;
    int seg, i, g;
    split_task(task, S, row, seg);
    split_task(row, P.N, bg, i);
    split_task(bg, P.G, bq, g);  // b = bg / G
    const int b = static_cast<int>(bq);
    const T* rp = ngs_row_ptr<T>(P, row);
    const RowBlocks rb = blocks_of(rp, P.V);
    // segment 0 gathers the logits at every candidate's token for this position
    float xg = __builtin_nanf("");
    const int h = threadIdx.x;
    if (seg == 0 && i < P.N - 1 && h < P.G) {
      const int x = P.cand[(static_cast<int64_t>(b) * P.G + h) * (P.N - 1) + i];
      if (x >= 0 && x < P.V) xg = Elem<T>::get(rp, x);
    }
    // the segment's scalar elements, in wave 0: lanes 0-7 the head, lanes 8-15 the tail
    float xs = -INFINITY;
    if (wave == 0) {
      if (seg == 0 && lane < rb.h) xs = Elem<T>::get(rp, lane);
      if (seg == S - 1 && lane >= 8 && lane - 8 < P.V - rb.tail_lo) xs = Elem<T>::get(rp, rb.tail_lo + lane - 8);
    }
    float m;
    double s;
    float2* bs = P.blk + row * P.nbmax;
    const __amdgpu_buffer_rsrc_t rs = vectors_of(rp, rb);
    if (S == 1 && rb.nb <= kNgsShotBlocks * kNgsRowWaves)
      ngs_row_shot<T>(rs, rb, wave, xs, c, bs, m, s);
    else
      ngs_row_pipelined<T>(rs, rb, seg, S, wave, xs, c, bs, m, s);
    if (lane == 0) {
      sh_m[wave] = m;
      sh_s[wave] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float M = sh_m[0];
#pragma unroll
      for (int w = 1; w < kNgsRowWaves; ++w) M = fmaxf(M, sh_m[w]);
      const float RM = M * c;
      double Ssum = 0.0;
#pragma unroll
      for (int w = 0; w < kNgsRowWaves; ++w) Ssum += rescaled_partial(sh_s[w], sh_m[w] * c, RM);
      P.p1_m[seg * rows + row] = M;
      P.p1_s[seg * rows + row] = Ssum;
    }
    if (seg == 0 && i < P.N - 1 && h < P.G) P.gx[(bg * (P.N - 1) + i) * P.G + h] = xg;
    __syncthreads();  // shared memory is reused by the next task
  }
}

// ---------------------------------------------------------------- the walk and the draw

constexpr int kNgsBlock = 1024;
// the gathered logits of a sequence are staged in LDS when they fit this many floats
constexpr int kNgsGxStage = 4096;

struct NgsShared {
  // staged inputs of the sequence (G*N <= SPEC_MAX_NGRAM_SAMPLE_GN)
  float M[SPEC_MAX_NGRAM_SAMPLE_GN];               // row maximum, rows (g, i) at g*N + i
  double Z[SPEC_MAX_NGRAM_SAMPLE_GN];              // row sum of 2^(x*c - fl(M*c))
  int cand[SPEC_MAX_NGRAM_SAMPLE_GN];              // [G][N-1]
  float uni[SPEC_MAX_NGRAM_SAMPLE_GN + SPEC_MAX_K + 1];  // [N][G+1]
  float gx[kNgsGxStage];                           // [G][N-1][G] when it fits
  // the walk's result
  int n_acc;       // accepted tokens; -1 on a fault
  int rows;        // candidate whose rows the draw reads
  int ntried;      // tokens rejected at the draw's position (excluded from its law)
  int tried[SPEC_MAX_POOL_G];
  int prefix[SPEC_MAX_K + 1];
  float R;         // reference exponent and softmax denominator of the draw row
  double S;
  float u;
};

// Stage the sequence's inputs in LDS with the whole workgroup (one round of loads):
// every row's merged statistics, the candidates, the uniforms and, when they fit,
// the gathered logits. Returns true when a candidate token is outside [0, V).
__device__ __forceinline__ bool ngs_stage(const NgramSampleParams& P, int b, NgsShared& sh) {
  const int G = P.G, N = P.N;
  const int64_t nc = static_cast<int64_t>(G) * (N - 1);
  const int64_t ngx = nc * G;
  bool bad = false;
  for (int r = threadIdx.x; r < G * N; r += kNgsBlock) {
    const int64_t row = static_cast<int64_t>(b) * G * N + r;
    float M;
    double Z;
    merge_partials(P.p1_m + row, P.p1_s + row, static_cast<int64_t>(P.B) * G * N, P.S1, P.c, M, Z);
    sh.M[r] = M;
    sh.Z[r] = Z;
  }
  for (int e = threadIdx.x; e < nc; e += kNgsBlock) {
    const int x = P.cand[static_cast<int64_t>(b) * nc + e];
    bad = bad || x < 0 || x >= P.V;
    sh.cand[e] = x;
  }
  for (int e = threadIdx.x; e < N * (G + 1); e += kNgsBlock)
    sh.uni[e] = P.uniforms[static_cast<int64_t>(b) * N * (G + 1) + e];
  if (ngx <= kNgsGxStage)
    for (int e = threadIdx.x; e < ngx; e += kNgsBlock) sh.gx[e] = P.gx[static_cast<int64_t>(b) * ngx + e];
  return __syncthreads_or(bad) != 0;
}

// The walk of batch row b by one wave from the staged inputs; every lane holds the
// same values (the positions and tries run in order; lane h holds candidate h's data).
__device__ __forceinline__ void ngs_walk(const NgramSampleParams& P, int b, NgsShared& sh) {
  const int lane = threadIdx.x & 63;
  const int G = P.G, N = P.N;
  const bool gx_staged = static_cast<int64_t>(G) * (N - 1) * G <= kNgsGxStage;
  uint64_t active = (G == 64) ? ~0ull : ((1ull << G) - 1);
  int i = 0;
  for (;;) {
    const int g0 = __ffsll(static_cast<unsigned long long>(active)) - 1;
    const float M = sh.M[g0 * N + i];
    const double Ssum = sh.Z[g0 * N + i];
    // lane h: candidate h's token at i, its logit in row (g0, i), its accept uniform
    int x = -1;
    float xl = 0.f, r = 1.f;
    if (i < N - 1 && lane < G) {
      x = sh.cand[lane * (N - 1) + i];
      const int64_t gi = (static_cast<int64_t>(g0) * (N - 1) + i) * G + lane;
      xl = gx_staged ? sh.gx[gi] : P.gx[static_cast<int64_t>(b) * G * (N - 1) * G + gi];
      r = sh.uni[i * (G + 1) + lane];
    }
    const float u_draw = sh.uni[i * (G + 1) + G];
    if (!(isfinite(M) && Ssum > 0.0 && isfinite(Ssum))) {
      if (lane == 0) sh.n_acc = -1;  // a consulted row with no finite logit
      return;
    }
    const float R = M * P.c;
    const float inv = static_cast<float>(1.0 / Ssum);
    if (i == N - 1) {  // every candidate token accepted: the bonus draw
      if (lane == 0) {
        sh.n_acc = i;
        sh.rows = g0;
        sh.ntried = 0;
        sh.R = R;
        sh.S = Ssum;
        sh.u = u_draw;
      }
      return;
    }
    const float px = (lane < G) ? exp2_hw(fmaf(xl, P.c, -R)) * inv : 0.f;
    // the tries, in candidate order (wave-uniform scalar loop); lane t keeps the t-th
    // token rejected at this position
    double removed = 0.0;
    int ntried = 0;
    int my_tried = -1;
    int accepted = -1;
    for (uint64_t m = active; m; m &= m - 1) {
      const int h = __ffsll(static_cast<unsigned long long>(m)) - 1;
      const int xh = lane_i(x, h);
      const bool seen = __ballot(lane < ntried && my_tried == xh) != 0;
      const double pxh = static_cast<double>(lane_f(px, h));
      const double left = 1.0 - removed;
      // alpha = p_cur(x) / q(x) with q = delta_x: p(x) renormalised over the untried tokens
      const double alpha = (seen || !(left > 0.0)) ? 0.0 : pxh / left;
      if (static_cast<double>(lane_f(r, h)) < alpha) {
        accepted = xh;
        break;
      }
      if (!seen) {
        removed += pxh;
        if (lane == ntried) my_tried = xh;
        ++ntried;
      }
    }
    if (accepted < 0) {  // every try failed: draw from the remaining mass
      if (lane < ntried) sh.tried[lane] = my_tried;
      if (lane == 0) {
        sh.n_acc = i;
        sh.rows = g0;
        sh.ntried = ntried;
        sh.R = R;
        sh.S = Ssum;
        sh.u = u_draw;
      }
      return;
    }
    if (lane == 0) sh.prefix[i] = accepted;
    active &= __ballot(lane < G && x == accepted);
    ++i;
  }
}

// The draw from row `row` by the whole workgroup: p with the tokens rejected at
// this position removed (none for the bonus draw). The masses of the row's blocks
// come from pass 1's block sums, except the blocks that hold a rejected token,
// which the waves reload and sum without it (one block per wave, with the row's
// scalar head and tail in the last wave): one round of loads. Wave 0 scans the
// block masses in fp64, picks the block where u*Z falls, reloads it and finds the
// token with chunk and lane scans. Zero remaining mass (rounding only) samples p;
// rounding past the end takes the last weight > 0.
constexpr int kNgsWaves = kNgsBlock / 64;
// block masses held in LDS: the vector blocks of a row of SPEC_MAX_NGRAM_SAMPLE_V fp32
// entries (4 per vector), plus the scalar head and tail
constexpr int kNgsMaxBlocks = SPEC_MAX_NGRAM_SAMPLE_V / (kNgsBlkVecs * 4) + 2;
static_assert(kNgsMaxBlocks <= 64 * 32, "the block scan gives each lane at most 32 blocks");

// Rejected tokens among this lane's elements of vector block k: bit u*VEC + e for
// element e of its vector in chunk u.
template <typename T>
__device__ __forceinline__ uint64_t block_excl_mask(const RowBlocks& rb, int64_t k, const NgsShared& sh, int ntried) {
  constexpr int VEC = Elem<T>::kVec;
  static_assert(kBlkChunks * VEC <= 64, "one mask bit per element of a lane");
  const int lane = threadIdx.x & 63;
  uint64_t mask = 0;
  for (int t = 0; t < ntried; ++t) {
    const int64_t off = static_cast<int64_t>(sh.tried[t]) - rb.h - k * kNgsBlkVecs * VEC;
    if (off >= 0 && off < static_cast<int64_t>(kNgsBlkVecs) * VEC) {
      const int v = static_cast<int>(off / VEC);
      if ((v & 63) == lane) mask |= 1ull << ((v >> 6) * VEC + static_cast<int>(off % VEC));
    }
  }
  return mask;
}

// This lane's weights 2^(x*c - R) / S in vector block k, 0 for masked elements and
// past the last whole vector.
template <typename T>
__device__ __forceinline__ void block_weights(__amdgpu_buffer_rsrc_t rs, const RowBlocks& rb, int64_t k, float c,
                                              float R, float inv, uint64_t mask,
                                              float (&w)[kBlkChunks][Elem<T>::kVec]) {
  constexpr int VEC = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  u32x4 raw[kBlkChunks];
  load_block(rs, k, raw);
#pragma unroll
  for (int u = 0; u < kBlkChunks; ++u) {
    float x[VEC];
    Elem<T>::unpack(raw[u], x);
    const bool in = k * kNgsBlkVecs + u * 64 + lane < rb.nvec;
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      w[u][e] = (in && !((mask >> (u * VEC + e)) & 1ull)) ? exp2_hw(fmaf(x[e], c, -R)) * inv : 0.f;
  }
}

// This lane's weight in the scalar head (tail == false) or tail: element e = lo + lane.
template <typename T>
__device__ __forceinline__ float scalar_weight(const T* rp, const RowBlocks& rb, int64_t V, bool tail, float c,
                                               float R, float inv, bool excl, const NgsShared& sh, int ntried,
                                               int64_t& e) {
  const int lane = threadIdx.x & 63;
  const int64_t lo = tail ? rb.tail_lo : 0, hi = tail ? V : rb.h;
  e = lo + lane;
  bool out = e >= hi;
  if (excl && !out)
    for (int t = 0; t < ntried; ++t) out = out || sh.tried[t] == e;
  return out ? 0.f : exp2_hw(fmaf(Elem<T>::get(rp, e), c, -R)) * inv;
}

template <typename T>
__device__ int64_t ngs_draw(const NgramSampleParams& P, int64_t row, const T* rp, const NgsShared& sh) {
  constexpr int VEC = Elem<T>::kVec;
  __shared__ double sh_bm[kNgsMaxBlocks];  // [0] head, [1 + k] vector block k, [nb + 1] tail
  __shared__ double sh_xm[SPEC_MAX_POOL_G];
  __shared__ int sh_xk[SPEC_MAX_POOL_G];
  __shared__ int sh_blk, sh_ok;
  __shared__ double sh_tau;
  __shared__ int64_t sh_k;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t V = P.V;
  const float c = P.c, R = sh.R;
  const float inv = static_cast<float>(1.0 / sh.S);
  const int ntried = sh.ntried;
  const RowBlocks rb = blocks_of(rp, V);
  const int nb = rb.nb, NB = rb.nb + 2;
  const float2* bs = P.blk + row * P.nbmax;
  for (int pass = 0; pass < 2; ++pass) {
    const bool excl = pass == 0 && ntried > 0;  // pass 1 (zero remaining mass) samples p itself
    // pass 1's block sums, rescaled to the row's reference
    for (int k = threadIdx.x; k < nb; k += kNgsBlock) {
      const float2 st = bs[k];
      sh_bm[1 + k] = (st.y > 0.f) ? static_cast<double>(st.y) *
                                        static_cast<double>(exp2_hw(static_cast<float>(static_cast<double>(st.x) - R))) *
                                        static_cast<double>(inv)
                                  : 0.0;
    }
    if (wave < kNgsWaves - 1) {
      // the blocks holding a rejected token, each summed by the wave of its first one
      for (int t = wave; excl && t < ntried; t += kNgsWaves - 1) {
        const int64_t e = sh.tried[t];
        int64_t k = (e >= rb.h && e < rb.tail_lo) ? (e - rb.h) / (static_cast<int64_t>(kNgsBlkVecs) * VEC) : -1;
        for (int t2 = 0; k >= 0 && t2 < t; ++t2) {
          const int64_t e2 = sh.tried[t2];
          if (e2 >= rb.h && e2 < rb.tail_lo && (e2 - rb.h) / (static_cast<int64_t>(kNgsBlkVecs) * VEC) == k) k = -1;
        }
        double mass = 0.0;
        if (k >= 0) {
          float w[kBlkChunks][VEC];
          block_weights<T>(vectors_of(rp, rb), rb, k, c, R, inv, block_excl_mask<T>(rb, k, sh, ntried), w);
          float ls = 0.f;
#pragma unroll
          for (int u = 0; u < kBlkChunks; ++u)
#pragma unroll
            for (int x = 0; x < VEC; ++x) ls += w[u][x];
          mass = lane_d(wave_scan_add(static_cast<double>(ls)), 63);
        }
        if (lane == 0) {
          sh_xm[t] = mass;
          sh_xk[t] = static_cast<int>(k);
        }
      }
    } else {
      int64_t e;
      const float wh = scalar_weight(rp, rb, V, false, c, R, inv, excl, sh, ntried, e);
      const float wt = scalar_weight(rp, rb, V, true, c, R, inv, excl, sh, ntried, e);
      const double mh = lane_d(wave_scan_add(static_cast<double>(wh)), 63);
      const double mt = lane_d(wave_scan_add(static_cast<double>(wt)), 63);
      if (lane == 0) {
        sh_bm[0] = mh;
        sh_bm[nb + 1] = mt;
      }
    }
    __syncthreads();
    if (excl && static_cast<int>(threadIdx.x) < ntried && sh_xk[threadIdx.x] >= 0)
      sh_bm[1 + sh_xk[threadIdx.x]] = sh_xm[threadIdx.x];
    __syncthreads();
    if (wave == 0) {
      // block scan in fp64: lane l owns the contiguous blocks [l*per, l*per + per)
      const int per = (NB + 63) / 64;
      const int j0 = min(lane * per, NB), j1 = min(j0 + per, NB);
      double mine = 0.0;
      int last = -1;
      for (int j = j0; j < j1; ++j) {
        mine += sh_bm[j];
        if (sh_bm[j] > 0.0) last = j;
      }
      const double incl = wave_scan_add(mine);
      const double Z = lane_d(incl, 63);
      const bool ok = Z > 0.0 && isfinite(Z);
      if (ok) {
        const double tau = static_cast<double>(sh.u) * Z;
        const int t = first_lane(incl > tau);
        if (t < 64) {
          if (lane == t) {
            double run = incl - mine;
            int js = -1;
            for (int j = j0; j < j1 && js < 0; ++j) {
              if (run + sh_bm[j] > tau) js = j;
              else run += sh_bm[j];
            }
            sh_blk = js >= 0 ? js : (last >= 0 ? last : j0);
            sh_tau = js >= 0 ? tau - run : INFINITY;
          }
        } else {  // rounding put u*Z at the very end: the last block with mass
          const int lw = last_lane(last >= 0);
          if (lane == 0) {
            sh_blk = lw >= 0 ? lane_i(last, lw) : 0;
            sh_tau = INFINITY;
          }
        }
      }
      if (lane == 0) sh_ok = ok;
    }
    __syncthreads();
    if (!sh_ok) {
      if (pass == 0) continue;
      return 0;  // unreachable for a row with a finite logit
    }
    if (wave == 0) {
      const int j = sh_blk;
      const double tau = sh_tau;
      int64_t found = -1, lastpos = -1;
      if (j == 0 || j == nb + 1) {
        // the scalar head or tail: lane l holds element lo + l
        int64_t e;
        const float w = scalar_weight(rp, rb, V, j != 0, c, R, inv, excl, sh, ntried, e);
        const double incl = wave_scan_add(static_cast<double>(w));
        const int hl = first_lane(incl > tau);
        const int lw = last_lane(w > 0.f);
        const int64_t lo = (j == 0) ? 0 : rb.tail_lo;
        if (hl < 64) found = lo + hl;
        else if (lw >= 0) lastpos = lo + lw;
        if (found < 0 && lastpos < 0) found = lo;
      } else {
        // vector block k: chunk by chunk (64 vectors each, in token order), then the lane
        const int64_t k = j - 1;
        float w[kBlkChunks][VEC];
        block_weights<T>(vectors_of(rp, rb), rb, k, c, R, inv, excl ? block_excl_mask<T>(rb, k, sh, ntried) : 0ull, w);
        double before = 0.0;  // mass of the block's chunks before chunk u
#pragma unroll
        for (int u = 0; u < kBlkChunks; ++u) {
          float ls = 0.f;
          int kl = -1;
#pragma unroll
          for (int x = 0; x < VEC; ++x) {
            ls += w[u][x];
            if (w[u][x] > 0.f) kl = x;
          }
          const double incl = wave_scan_add(static_cast<double>(ls));
          const int lw = last_lane(kl >= 0);
          if (lw >= 0) lastpos = rb.h + (k * kNgsBlkVecs + u * 64 + lw) * VEC + lane_i(kl, lw);
          if (found < 0) {
            const int hl = first_lane(before + incl > tau);
            if (hl < 64) {
              const double pre = before + incl - static_cast<double>(ls);
              float run = 0.f;
              int kk = -1;
#pragma unroll
              for (int x = 0; x < VEC; ++x) {
                run += w[u][x];
                if (kk < 0 && pre + static_cast<double>(run) > tau) kk = x;
              }
              const int pick = kk >= 0 ? kk : (kl >= 0 ? kl : 0);
              found = rb.h + (k * kNgsBlkVecs + u * 64 + hl) * VEC + lane_i(pick, hl);
            }
          }
          before += lane_d(incl, 63);
        }
        if (found < 0 && lastpos < 0) found = rb.h + k * kNgsBlkVecs * VEC;
      }
      if (lane == 0) sh_k = found >= 0 ? found : lastpos;
    }
    __syncthreads();
    const int64_t k = sh_k;
    __syncthreads();
    return k;
  }
  return 0;
}

template <typename T>
__global__ __launch_bounds__(kNgsBlock) void k_ngs_verify(NgramSampleParams P) {
  touch_kernargs(P);
  __shared__ NgsShared sh;
  const int N = P.N;
  for (int64_t task = blockIdx.x; task < P.B; task += gridDim.x) {
    const int b = static_cast<int>(task);
    if (ngs_stage(P, b, sh)) {
      if (threadIdx.x == 0) sh.n_acc = -1;  // a candidate token outside [0, V)
    } else if (threadIdx.x < 64) {
      ngs_walk(P, b, sh);
    }
    __syncthreads();
    const int L = sh.n_acc;
    int32_t* ot = P.out_tokens + static_cast<int64_t>(b) * N;
    if (L < 0) {
      for (int t = threadIdx.x; t < N; t += kNgsBlock) ot[t] = -1;
      if (threadIdx.x == 0) {
        P.out_len[b] = -1;
        P.out_rows[b] = -1;
      }
      __syncthreads();
      continue;
    }
    const int64_t drow = ngs_row(P, b, sh.rows, L);
    const int64_t k = ngs_draw<T>(P, drow, ngs_row_ptr<T>(P, drow), sh);
    for (int t = threadIdx.x; t < N; t += kNgsBlock) ot[t] = t < L ? sh.prefix[t] : (t == L ? static_cast<int32_t>(k) : -1);
    if (threadIdx.x == 0) {
      P.out_len[b] = L;
      P.out_rows[b] = sh.rows;
    }
    __syncthreads();  // shared memory is reused by the next sequence
  }
}

// ---------------------------------------------------------------- launch

hipError_t launch_ngram_sample(const NgramSampleParams& P, bool bf16, hipStream_t stream) {
  const int64_t tasks = static_cast<int64_t>(P.B) * P.G * P.N * P.S1;
  const dim3 g1(static_cast<uint32_t>(tasks < (1 << 20) ? tasks : (1 << 20)));
  const dim3 g2(static_cast<uint32_t>(P.B < (1 << 20) ? P.B : (1 << 20)));
  if (bf16) {
    hipLaunchKernelGGL(k_ngs_rowstats<bf16_t>, g1, dim3(kNgsRowBlock), 0, stream, P);
    hipLaunchKernelGGL(k_ngs_verify<bf16_t>, g2, dim3(kNgsBlock), 0, stream, P);
  } else {
    hipLaunchKernelGGL(k_ngs_rowstats<float>, g1, dim3(kNgsRowBlock), 0, stream, P);
    hipLaunchKernelGGL(k_ngs_verify<float>, g2, dim3(kNgsBlock), 0, stream, P);
  }
  return hipGetLastError();
}

}  // namespace sv
