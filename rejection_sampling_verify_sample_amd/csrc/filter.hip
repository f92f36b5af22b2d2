// Top-k / top-p filtering of the logit rows of a verify round (gfx950).
//
// Method (kwkr.cn/news/620797 engineering notes, §3.4): the temperature rescales
// both sides before p and q are formed; a top-k or top-p truncation uses the same
// parameter on the draft and the target side, and the correction is drawn only
// inside the kept set. Each row keeps the entries whose logit is >= a threshold:
//   top-k (0 < k < V): every entry with fewer than k entries strictly above it;
//   top-p (p < 1), on the law left by top-k and renormalised: an entry whose
//     strictly-larger kept entries hold mass < p, and always the row's largest.
// The verify then runs unchanged on the renormalised kept laws p', q'.
//
// k_filter_rows: one 256-thread workgroup per logit row (target rows 0..K and
// draft rows 0..K-1 of every batch row) finds the threshold exactly by a radix
// select on the 32-bit order key of the logits (digits of 11, 11 and 10 bits;
// bf16 keys are resolved after two digits). Each digit is one pass over the row
// that builds an LDS histogram of the digit over the entries still in play: the
// count of entries and their mass 2^(x*c - R) in fixed point (round(m * 2^40)
// in 64-bit integers), so every sum is exact and independent of the order the
// atomics land in. Pass one also keeps the online maximum, which fixes R. The
// row is re-read from cache by the later passes (plain loads, not streaming).
// Per row the kernel leaves the reference R, the kept mass against it, the key
// threshold and the kept count; the accept, mass and draw kernels apply them.
#include "common.hpp"
#include "params.hpp"

namespace sv {

constexpr int kFiltBlock = 256;
constexpr int kFiltUnroll = 2;
constexpr int kHistBins = 2048;
constexpr int kFixBits = 40;

// round(m * 2^40) for 0 <= m <= 1, from the bits of m (integer arithmetic only).
__device__ __forceinline__ uint64_t to_fixed(float m) {
  const uint32_t b = __float_as_uint(m);
  const int ex = static_cast<int>(b >> 23);
  if (ex == 0) return 0;
  const uint64_t mant = (b & 0x7FFFFFu) | 0x800000u;  // m = mant * 2^(ex - 150)
  const int sh = ex - (150 - kFixBits);
  if (sh >= 0) return mant << sh;
  const int rs = -sh;
  if (rs > 24) return 0;
  return (mant + (uint64_t(1) << (rs - 1))) >> rs;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Exclusive prefix sum over the block in thread order; also the block total.
__device__ __forceinline__ uint64_t block_excl_u64(uint64_t v, uint64_t& total) {
  constexpr int W = kFiltBlock / 64;
  __shared__ uint64_t sh[W];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint64_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  uint64_t before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    if (i < w) before += sh[i];
    total += sh[i];
  }
  __syncthreads();
  return before + inc - v;
}

__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v) {
  uint64_t t;
  block_excl_u64(v, t);
  return t;
}

struct FiltShared {
  uint32_t cnt[kHistBins];
  unsigned long long mass[kHistBins];
  // the bin a scan picked, with the count and mass of the bins above it and in it
  uint32_t pick_bin;
  uint64_t pick_above_cnt, pick_above_mass, pick_cnt, pick_mass;
  float M;
  double S;
};

__device__ __forceinline__ void clear_hist(FiltShared& sh) {
  for (int i = threadIdx.x; i < kHistBins; i += kFiltBlock) {
    sh.cnt[i] = 0;
    sh.mass[i] = 0;
  }
  __syncthreads();
}

// Entry e of a 16-byte vector held as raw words.
template <typename T>
__device__ __forceinline__ float vec_elem(const u32x4& v, int e);
template <>
__device__ __forceinline__ float vec_elem<float>(const u32x4& v, int e) {
  return __uint_as_float(v[e]);
}
template <>
__device__ __forceinline__ float vec_elem<bf16_t>(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}

// Visit every entry of a row with f(x): 16-byte vectors where aligned,
// kFiltUnroll of them in flight per thread, held raw and widened one entry at a
// time. Plain (cached) loads: the row is read again by the next pass.
template <typename T, typename F>
__device__ __forceinline__ void visit_row(const T* row, int64_t V, F&& f) {
  constexpr int VEC = Elem<T>::kVec;
  constexpr int BS = kFiltBlock, U = kFiltUnroll;
  const int64_t h = head_elems(row, V);
  for (int64_t e = threadIdx.x; e < h; e += BS) f(Elem<T>::get(row, e));
  const int64_t nvec = (V - h) / VEC;
  const u32x4* vb = reinterpret_cast<const u32x4*>(row + h);
  int64_t v = threadIdx.x;
  for (; v + (U - 1) * BS < nvec; v += U * BS) {
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = vb[v + u * BS];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) f(vec_elem<T>(w[u], e));
  }
  for (; v < nvec; v += BS) {
    const u32x4 w = vb[v];
#pragma unroll
    for (int e = 0; e < VEC; ++e) f(vec_elem<T>(w, e));
  }
  for (int64_t e = h + nvec * VEC + threadIdx.x; e < V; e += BS) f(Elem<T>::get(row, e));
}

// Scan the histogram's nb bins from the top and pick the first bin that
//   (COUNT) brings the count of entries down to it to >= r   (r >= 1), or
//   (MASS)  holds entries and brings A0 + the mass down to it to >= P
//           (with P <= 0: the first bin that holds entries).
// The pick lands in sh.pick_*; bins above it give pick_above_cnt / _mass. Both
// modes report the masses (the kept mass of a top-k cut comes from them).
template <bool MASS>
__device__ void scan_hist(FiltShared& sh, int nb, uint64_t r, double P, uint64_t A0) {
  const int per = nb / kFiltBlock;
  const int t = threadIdx.x;
  uint64_t tc = 0, tm = 0;
  for (int i = 0; i < per; ++i) {
    const int b = nb - 1 - (t * per + i);
    tc += sh.cnt[b];
    tm += sh.mass[b];
  }
  uint64_t total;
  const uint64_t ec = block_excl_u64(tc, total);
  const uint64_t em = block_excl_u64(tm, total);
  bool mine;
  if (MASS) {
    mine = (P <= 0.0) ? (tc > 0 && ec == 0) : (static_cast<double>(A0 + em) < P &&
                                                 static_cast<double>(A0 + em + tm) >= P);
  } else {
    mine = ec < r && ec + tc >= r;
  }
  if (mine) {
    uint64_t c_above = ec, m_above = em;
    for (int i = 0; i < per; ++i) {
      const int b = nb - 1 - (t * per + i);
      const uint64_t c = sh.cnt[b];
      const uint64_t m = sh.mass[b];
      const bool hit = MASS ? (c > 0 && (P <= 0.0 || static_cast<double>(A0 + m_above + m) >= P))
                            : (c_above + c >= r);
      if (hit) {
        sh.pick_bin = static_cast<uint32_t>(b);
        sh.pick_above_cnt = c_above;
        sh.pick_above_mass = m_above;
        sh.pick_cnt = c;
        sh.pick_mass = m;
        break;
      }
      c_above += c;
      m_above += m;
    }
  }
  __syncthreads();
}

// One refinement pass: histogram of the digit (key >> dshift) & (nb - 1) over the
// entries with key in [max(lo, rlo), rhi]; entries with key > rhi (and >= lo) are
// counted, with their mass, in ab_cnt / ab_mass.
template <typename T>
__device__ void refine_pass(FiltShared& sh, const T* row, int64_t V, float c, float Rf, uint32_t lo, uint32_t rlo,
                            uint32_t rhi, int dshift, int nb, uint64_t& ab_cnt, uint64_t& ab_mass) {
  clear_hist(sh);
  const uint32_t rl = rlo > lo ? rlo : lo;
  uint64_t acnt = 0, amass = 0;
  visit_row(row, V, [&](float x) {
    const uint32_t k = order_key(x);
    if (k < lo) return;
    if (k > rhi) {
      acnt += 1;
      amass += to_fixed(fminf(exp2_hw(fmaf(x, c, -Rf)), 1.f));
    } else if (k >= rl) {
      const int b = static_cast<int>((k >> dshift) & static_cast<uint32_t>(nb - 1));
      atomicAdd(&sh.cnt[b], 1u);
      atomicAdd(&sh.mass[b], static_cast<unsigned long long>(to_fixed(fminf(exp2_hw(fmaf(x, c, -Rf)), 1.f))));
    }
  });
  __syncthreads();
  ab_cnt = block_sum_u64(acnt);
  ab_mass = block_sum_u64(amass);
}

template <typename T>
__device__ void filter_row_task(const SampleParams& P, const int64_t task, FiltShared& sh) {
  const int K = P.K;
  const int64_t V = P.V;
  const int64_t ntgt = static_cast<int64_t>(P.B) * (K + 1);
  int b, j, tok_slot = -1;
  const T* row;
  if (task < ntgt) {  // target rows first, in memory order
    b = static_cast<int>(task / (K + 1));
    j = static_cast<int>(task - static_cast<int64_t>(b) * (K + 1));
    row = static_cast<const T*>(P.target) + task * V;
    if (j < K) tok_slot = j;
  } else {
    const int64_t t = task - ntgt;
    b = static_cast<int>(t / K);
    const int i = static_cast<int>(t - static_cast<int64_t>(b) * K);
    j = K + 1 + i;
    row = static_cast<const T*>(P.draft) + t * V;
    tok_slot = K + i;
  }
  const int64_t fr = static_cast<int64_t>(b) * (2 * K + 1) + j;
  const int kk = P.top_k ? P.top_k[b] : 0;
  const float pp = P.top_p ? P.top_p[b] : 1.f;
  const bool k_on = kk > 0 && kk < V;
  const bool p_on = pp < 1.f;  // false for NaN
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int L = kBf16 ? 2 : 3;
  const float c = P.c;

  float xl = __builtin_nanf("");
  if (tok_slot >= 0 && threadIdx.x == 0) {
    const int x = P.tokens[static_cast<int64_t>(b) * K + (tok_slot < K ? tok_slot : tok_slot - K)];
    if (x >= 0 && x < V) xl = Elem<T>::get(row, x);
  }

  // pass 1: online maximum and sum; with top-k also the histogram of the top digit
  if (k_on) clear_hist(sh);
  Online o;
  o.init();
  visit_row(row, V, [&](float x) {
    if (x > o.m) o.raise(x, c);
    o.add(x, c);
    if (k_on) atomicAdd(&sh.cnt[order_key(x) >> 21], 1u);
  });
  {
    float M;
    double S;
    block_online<kFiltBlock>(o, c, M, S);
    if (threadIdx.x == 0) {
      sh.M = M;
      sh.S = S;
    }
    __syncthreads();
  }
  const float M = sh.M;
  const double S = sh.S;
  if (!(M > -INFINITY)) {  // no finite logit: the row keeps nothing
    if (threadIdx.x == 0) {
      P.f_R[fr] = 0.f;
      P.f_S[fr] = 0.0;
      P.f_thr[fr] = 0xFFFFFFFFu;
      if (P.out_kept) P.out_kept[fr] = 0;
      if (tok_slot >= 0) P.p1_x[static_cast<int64_t>(b) * 2 * K + tok_slot] = xl;
    }
    __syncthreads();
    return;
  }
  // masses 2^(x*c - Rf) against Rf = fl(M*c) + 1 stay <= 1 (the largest is about 1/2)
  const float R = M * c;
  const float Rf = R + 1.f;
  uint32_t thr = 0;
  uint64_t kept_n = static_cast<uint64_t>(V), kept_m = 0;
  bool fixed_mass = false;

  if (k_on) {
    scan_hist<false>(sh, kHistBins, static_cast<uint64_t>(kk), 0.0, 0);
    uint32_t prefix = sh.pick_bin;
    uint64_t r = static_cast<uint64_t>(kk) - sh.pick_above_cnt;
    __syncthreads();
    for (int lev = 1; lev < L; ++lev) {
      const int shift = lev == 1 ? 21 : 10;
      const int dshift = lev == 1 ? 10 : 0;
      const int nb = lev == 1 ? kHistBins : 1024;
      const uint32_t rlo = prefix << shift, rhi = rlo | ((1u << shift) - 1u);
      uint64_t ab_cnt, ab_mass;
      refine_pass(sh, row, V, c, Rf, 0u, rlo, rhi, dshift, nb, ab_cnt, ab_mass);
      scan_hist<false>(sh, nb, r, 0.0, 0);
      r -= sh.pick_above_cnt;
      prefix = (prefix << (lev == 1 ? 11 : 10)) | sh.pick_bin;
      if (lev == L - 1) {
        thr = prefix << (kBf16 ? 10 : 0);
        kept_n = ab_cnt + sh.pick_above_cnt + sh.pick_cnt;
        kept_m = ab_mass + sh.pick_above_mass + sh.pick_mass;
        fixed_mass = true;
      }
      __syncthreads();
    }
  }
  if (p_on) {
    const uint32_t lo = thr;
    uint64_t ab_cnt = 0, ab_mass = 0;
    refine_pass(sh, row, V, c, Rf, lo, 0u, 0xFFFFFFFFu, 21, kHistBins, ab_cnt, ab_mass);
    uint64_t zt = 0;
    for (int i = threadIdx.x; i < kHistBins; i += kFiltBlock) zt += sh.mass[i];
    const uint64_t Z = block_sum_u64(zt);
    const double Pm = static_cast<double>(pp) * static_cast<double>(Z);
    scan_hist<true>(sh, kHistBins, 0, Pm, 0);
    uint32_t prefix = sh.pick_bin;
    __syncthreads();
    for (int lev = 1; lev < L; ++lev) {
      const int shift = lev == 1 ? 21 : 10;
      const int dshift = lev == 1 ? 10 : 0;
      const int nb = lev == 1 ? kHistBins : 1024;
      const uint32_t rlo = prefix << shift, rhi = rlo | ((1u << shift) - 1u);
      refine_pass(sh, row, V, c, Rf, lo, rlo, rhi, dshift, nb, ab_cnt, ab_mass);
      scan_hist<true>(sh, nb, 0, Pm, ab_mass);
      prefix = (prefix << (lev == 1 ? 11 : 10)) | sh.pick_bin;
      if (lev == L - 1) {
        thr = prefix << (kBf16 ? 10 : 0);
        kept_n = ab_cnt + sh.pick_above_cnt + sh.pick_cnt;
        kept_m = ab_mass + sh.pick_above_mass + sh.pick_mass;
        fixed_mass = true;
      }
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) {
    P.f_R[fr] = Rf;
    // without a filter the online sum serves, moved from reference R to Rf
    P.f_S[fr] = fixed_mass ? static_cast<double>(kept_m) * 0x1p-40
                           : S * exp2(static_cast<double>(R) - static_cast<double>(Rf));
    P.f_thr[fr] = thr;
    if (P.out_kept) P.out_kept[fr] = static_cast<int32_t>(kept_n);
    if (tok_slot >= 0) P.p1_x[static_cast<int64_t>(b) * 2 * K + tok_slot] = xl;
  }
  __syncthreads();
}

template <typename T>
__global__ __launch_bounds__(kFiltBlock) void k_filter_rows(SampleParams P) {
  __shared__ FiltShared sh;
  const int64_t ntask = static_cast<int64_t>(P.B) * (2 * P.K + 1);
  for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) filter_row_task<T>(P, task, sh);
}

hipError_t launch_filter_rows(const SampleParams& P, bool bf16, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(P.B) * (2 * P.K + 1);
  const dim3 grid(static_cast<uint32_t>(rows < (1 << 20) ? rows : (1 << 20)));
  if (bf16)
    hipLaunchKernelGGL(k_filter_rows<bf16_t>, grid, dim3(kFiltBlock), 0, stream, P);
  else
    hipLaunchKernelGGL(k_filter_rows<float>, grid, dim3(kFiltBlock), 0, stream, P);
  return hipGetLastError();
}

}  // namespace sv
