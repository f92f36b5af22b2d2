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
// The multi-pass select: one 256-thread workgroup per logit row (target rows 0..K
// and draft rows 0..K-1 of every batch row) finds the threshold exactly by a radix
// select on the 32-bit order key of the logits (digits of 11, 11 and 10 bits;
// bf16 keys are resolved after two digits). Each digit is one pass over the row
// that builds an LDS histogram of the digit over the entries still in play: the
// count of entries and their mass 2^(x*c - R) in fixed point (round(m * 2^40)
// in 64-bit integers), so every sum is exact and independent of the order the
// atomics land in. Pass one also keeps the online maximum, which fixes R. The
// row is re-read from cache by the later passes (plain loads, not streaming).
// Per row it leaves the reference R, the kept mass against it, the key threshold
// and the kept count; the accept, mass and draw kernels apply them.
//
// k_filter reads most rows once instead, one workgroup per row, with the same
// fixed-point masses against the same reference, so its results are the multi-pass
// select's. With top-k on and k <= 64 every thread publishes its running maximum in
// LDS, and the k-th largest of those 256 maxima (each the maximum of a disjoint part
// of the row) is a lower bound of the row's k-th largest logit; entries at or above
// it go to an LDS buffer, one wave finds the k-th largest key by a bitwise search and
// sorts the kept keys, and the top-p group comes from an exact scan of their masses.
// Rows with top-p on, or top-k > 64, take a bound from the first step of the read and
// keep the entries above it in a buffer or, for long bf16 rows with top-p alone, count
// entries per key; a long fp32 row with top-p alone whose nucleus outgrows the buffer
// is read twice (bin counts bound the cut to a band, then exact masses and the band's
// keys). Details stand above each route. A bf16 row none of them finishes takes the
// multi-pass select in the same workgroup; an fp32 row is flagged for it and
// k_filter_rows, launched after k_filter, runs it (it skips the rows finished before).
#include "common.hpp"
#include "params.hpp"

namespace sv {

constexpr int kFiltBlock = 256;
constexpr int kFiltUnroll = 4;
constexpr int kHistBins = 2048;
constexpr int kFixBits = 40;
constexpr int kFiltCap = 2048;   // candidate buffer of the one-pass top-k path (a power of two)
constexpr int kFiltFastK = 64;   // the largest k it takes: one running maximum per lane
#ifndef SV_FAST_MINB
#define SV_FAST_MINB 5  // workgroups per CU the one-pass kernel is compiled for (register budget)
#endif
#ifndef SV_FAST_UNROLL
#define SV_FAST_UNROLL 4
#endif
constexpr int kFastUnroll = SV_FAST_UNROLL;  // 16-byte vectors per thread per step of the one-pass read
#ifndef SV_WIDE_UNROLL
#define SV_WIDE_UNROLL 3
#endif
constexpr int kWideUnroll = SV_WIDE_UNROLL;  // the same for the top-p / large top-k read (its sample is one step)

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

// 2^d for a double d of moderate size: the hardware exponential of the fraction,
// then an exact scaling by the integer part (exact when d is an integer). Its
// relative error is that of one fp32 exponential.
__device__ __forceinline__ double pow2d(double d) {
  const double n = floor(d);
  return ldexp(static_cast<double>(exp2_hw(static_cast<float>(d - n))), static_cast<int>(n));
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

// The one-pass top-k path's shared memory.
struct FastBuf {
  uint32_t key[kFiltCap];   // candidates: logits while collecting, then their order keys, sorted
  uint32_t kept[64];        // the wave-level cut's kept keys
  uint32_t res_thr, res_n;  // its results
  unsigned long long res_m;
  uint32_t nbuf;
  uint32_t lmax[kFiltBlock];  // every thread's running maximum (float bits), published for the bound
  float wmax[kFiltBlock / 64];
  int32_t wmin[kFiltBlock / 64];
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
template <typename Visit>
__device__ void refine_pass(FiltShared& sh, Visit&& visit, float c, float Rf, uint32_t lo, uint32_t rlo,
                            uint32_t rhi, int dshift, int nb, uint64_t& ab_cnt, uint64_t& ab_mass) {
  clear_hist(sh);
  const uint32_t rl = rlo > lo ? rlo : lo;
  uint64_t acnt = 0, amass = 0;
  visit([&](float x) {
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

// ---------------------------------------------------------------- one-pass top-k candidates

// Lower bound of the k-th largest key of a row from 256 of its entries (k <= 64),
// four per lane: the largest key t, searched over its top 16 bits, with at least k
// of them at or above it, so at least k entries of the row are >= t.
__device__ __forceinline__ uint32_t kth_bound(const float (&v)[kFiltBlock / 64], int k) {
  uint32_t key[kFiltBlock / 64];
#pragma unroll
  for (int o = 0; o < kFiltBlock / 64; ++o) key[o] = order_key(v[o]);
  uint32_t t = 0;
#pragma unroll
  for (int bit = 31; bit >= 16; --bit) {
    const uint32_t cand = t | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int o = 0; o < kFiltBlock / 64; ++o) cnt += __popcll(__ballot(key[o] >= cand));
    if (cnt >= k) t = cand;
  }
  return t;
}

// The float f with x >= f exactly when order_key(x) >= t (x not NaN); every value
// when t is at or below the key of -inf.
__device__ __forceinline__ float key_floor_value(uint32_t t) {
  constexpr uint32_t kKeyNegInf = 0x007FFFFFu;
  if (t <= kKeyNegInf) return -INFINITY;
  return __uint_as_float((t & 0x80000000u) ? (t & 0x7FFFFFFFu) : ~t);
}

// Inclusive prefix sum of 32-bit counts over the lanes of a wave (DPP moves).
__device__ __forceinline__ uint32_t wave_scan_add_u32(uint32_t v) {
  v += dpp::mov<dpp::kShr1, 0xf>(v, 0u);
  v += dpp::mov<dpp::kShr2, 0xf>(v, 0u);
  v += dpp::mov<dpp::kShr4, 0xf>(v, 0u);
  v += dpp::mov<dpp::kShr8, 0xf>(v, 0u);
  v += dpp::mov<dpp::kBcast15, 0xa>(v, 0u);
  v += dpp::mov<dpp::kBcast31, 0xc>(v, 0u);
  return v;
}

// Reserve room for `cnt` values of every lane of the wave (lane order): one wave
// scan and one LDS atomic. Returns the lane's first slot. Every lane takes part.
__device__ __forceinline__ uint32_t reserve_slots(uint32_t& nbuf, uint32_t cnt) {
  const int lane = threadIdx.x & 63;
  const uint32_t incl = wave_scan_add_u32(cnt);
  uint32_t base = 0;
  if (lane == 63 && incl) base = atomicAdd(&nbuf, incl);
  base = __builtin_amdgcn_readlane(base, 63);
  return base + incl - cnt;
}

// Append the lane's values whose bit is set in `take` (bit i for x[i]).
template <int N>
__device__ __forceinline__ void append_masked(FastBuf& fb, const float (&x)[N], uint32_t take) {
  uint32_t pos = reserve_slots(fb.nbuf, static_cast<uint32_t>(__popc(take)));
#pragma unroll
  for (int i = 0; i < N; ++i)
    if ((take >> i) & 1u) {
      if (pos < static_cast<uint32_t>(kFiltCap)) fb.key[pos] = __float_as_uint(x[i]);
      ++pos;
    }
}

// Read the row once: its maximum, and into fb.key every entry at or above a running
// lower bound of the k-th largest key (k <= kFiltFastK), which includes every entry
// top-k keeps. Returns the number of candidates (more than kFiltCap: overflow).
template <typename T>
__device__ uint32_t collect_candidates(const T* row, int64_t V, int kk, FastBuf& fb, float& rowmax, uint32_t& lbound) {
  constexpr int VEC = Elem<T>::kVec;
  constexpr int BS = kFiltBlock, U = kFastUnroll, W = kFiltBlock / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x == 0) fb.nbuf = 0;
  __atomic_store_n(&fb.lmax[threadIdx.x], __float_as_uint(-INFINITY), __ATOMIC_RELAXED);
  __syncthreads();
  float m = -INFINITY;  // this thread's running maximum
  uint32_t thr = 0u;
  float thrf = -INFINITY;
  const int64_t h = head_elems(row, V);
  const int64_t nvec = (V - h) / VEC;
  const u32x4* vb = reinterpret_cast<const u32x4*>(row + h);
  // steps of U*BS vectors taken by every thread together (the loop bound is uniform:
  // the wave scans and ballots below need every lane)
  int64_t base = 0;
  int it = 0;
  for (; base + U * BS <= nvec; base += U * BS, ++it) {
    const int64_t v = base + threadIdx.x;
    u32x4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) raw[u] = load_stream(vb + v + u * BS);
    float im = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float y[VEC];
      Elem<T>::unpack(raw[u], y);
#pragma unroll
      for (int e = 0; e < VEC; ++e) im = fmaxf(im, y[e]);
    }
    m = fmaxf(m, im);
    __atomic_store_n(&fb.lmax[threadIdx.x], __float_as_uint(m), __ATOMIC_RELAXED);
    if ((it & (it + 1)) == 0 || (it & 3) == 3) {  // steps 0, 1, 3, then every 4th
      // any published maximum is an entry of its thread's part of the row
      float pub[W];
#pragma unroll
      for (int o = 0; o < W; ++o) pub[o] = __uint_as_float(__atomic_load_n(&fb.lmax[lane + 64 * o], __ATOMIC_RELAXED));
      const uint32_t t = kth_bound(pub, kk);
      if (t > thr) {
        thr = t;
        thrf = key_floor_value(t);
      }
    }
    if (__ballot(im >= thrf)) {  // rare once the bound has risen
      // each vector's take bits, then one slot reservation and a loop over the set
      // bits (few after the first steps; a fully unrolled store of every entry
      // would hold all of them in registers)
      uint32_t tk[U];
      uint32_t cnt = 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float y[VEC];
        Elem<T>::unpack(raw[u], y);
        uint32_t t = 0;
#pragma unroll
        for (int e = 0; e < VEC; ++e) t |= (y[e] >= thrf ? 1u : 0u) << e;
        tk[u] = t;
        cnt += __popc(t);
      }
      uint32_t pos = reserve_slots(fb.nbuf, cnt);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        for (uint32_t t = tk[u]; t != 0u; t &= t - 1u) {
          if (pos < static_cast<uint32_t>(kFiltCap))
            fb.key[pos] = __float_as_uint(Elem<T>::lane_elem(raw[u], __ffs(t) - 1));
          ++pos;
        }
      }
    }
  }
  // the last vectors, one per thread, then the scalar head (lanes 0-7 of wave 0) and
  // tail (lanes 8-15): every lane of each wave takes part in the appends
  for (; base < nvec; base += BS) {
    const int64_t vr = base + threadIdx.x;
    float x[VEC];
    const bool in = vr < nvec;
    if (in) {
      Elem<T>::unpack(load_stream(vb + vr), x);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) x[e] = -INFINITY;
    }
    uint32_t take = 0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      m = fmaxf(m, x[e]);
      take |= (in && x[e] >= thrf ? 1u : 0u) << e;
    }
    append_masked(fb, x, take);
  }
  if (w == 0) {
    const int64_t tail_lo = h + nvec * VEC;
    const int64_t e = lane < 8 ? lane : tail_lo + (lane - 8);
    const bool in = lane < 8 ? lane < h : (lane < 16 && e < V);
    float x[1];
    x[0] = in ? Elem<T>::get(row, e) : -INFINITY;
    m = fmaxf(m, x[0]);
    append_masked(fb, x, in ? 1u : 0u);
  }
  const float wm = wave_max(m);
  if (lane == 0) fb.wmax[w] = wm;
  __syncthreads();
  float M = fb.wmax[0];
#pragma unroll
  for (int o = 1; o < W; ++o) M = fmaxf(M, fb.wmax[o]);
  rowmax = M;
  lbound = thr;
  return fb.nbuf;
}

// Sort key[0..npad) in descending order (bitonic network; npad a power of two).
__device__ void sort_keys_desc(uint32_t* key, int npad) {
  for (int size = 2; size <= npad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < npad / 2; i += kFiltBlock) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint32_t a = key[lo], b = key[hi];
        if ((a < b) == up) {
          key[lo] = b;
          key[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

// Smallest value over the block, every thread gets it (wmin: one slot per wave).
__device__ __forceinline__ int32_t block_min_i32(int32_t* wmin, int32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) wmin[threadIdx.x >> 6] = v;
  __syncthreads();
  int32_t r = wmin[0];
#pragma unroll
  for (int o = 1; o < kFiltBlock / 64; ++o) r = min(r, wmin[o]);
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------- the cut

// Top-k then top-p thresholds over the entries `visit` presents (every entry of the
// row, or a candidate buffer holding every entry top-k keeps). With top-k on, the
// histogram of the top key digit must already be in sh.cnt.
template <bool kBf16, typename Visit>
__device__ __forceinline__ void cut_row(FiltShared& sh, Visit&& visit, int kk, float pp, bool k_on, bool p_on, float c, float Rf,
                        uint32_t& thr, uint64_t& kept_n, uint64_t& kept_m, bool& fixed_mass) {
  constexpr int L = kBf16 ? 2 : 3;
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
      refine_pass(sh, visit, c, Rf, 0u, rlo, rhi, dshift, nb, ab_cnt, ab_mass);
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
    refine_pass(sh, visit, c, Rf, lo, 0u, 0xFFFFFFFFu, 21, kHistBins, ab_cnt, ab_mass);
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
      refine_pass(sh, visit, c, Rf, lo, rlo, rhi, dshift, nb, ab_cnt, ab_mass);
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
}

// A logit row of the round: target rows 0..K of every batch row first (memory
// order), then draft rows 0..K-1. fr indexes the per-row filter results.
struct FiltRow {
  int b, tok_slot;  // tok_slot: slot of the row's draft-token logit in p1_x, -1 for the bonus row
  int64_t fr;
  const void* row;
};

__device__ __forceinline__ FiltRow filt_row(const SampleParams& P, int64_t task, size_t esize) {
  const int K = P.K;
  const int64_t ntgt = static_cast<int64_t>(P.B) * (K + 1);
  FiltRow r;
  int j;
  r.tok_slot = -1;
  if (task < ntgt) {
    int64_t q;
    split_task(task, K + 1, q, j);
    r.b = static_cast<int>(q);
    r.row = static_cast<const char*>(P.target) + task * P.V * static_cast<int64_t>(esize);
    if (j < K) r.tok_slot = j;
  } else {
    const int64_t t = task - ntgt;
    int64_t q;
    int i;
    split_task(t, K, q, i);
    r.b = static_cast<int>(q);
    j = K + 1 + i;
    r.row = static_cast<const char*>(P.draft) + t * P.V * static_cast<int64_t>(esize);
    r.tok_slot = K + i;
  }
  r.fr = static_cast<int64_t>(r.b) * (2 * K + 1) + j;
  return r;
}

// The draft-token logit of the row (thread 0; NaN if the token is out of range).
template <typename T>
__device__ __forceinline__ float filt_token_logit(const SampleParams& P, const FiltRow& r) {
  float xl = __builtin_nanf("");
  if (r.tok_slot >= 0 && threadIdx.x == 0) {
    const int K = P.K;
    const int x = P.tokens[static_cast<int64_t>(r.b) * K + (r.tok_slot < K ? r.tok_slot : r.tok_slot - K)];
    if (x >= 0 && x < P.V) xl = Elem<T>::get(static_cast<const T*>(r.row), x);
  }
  return xl;
}

__device__ __forceinline__ void filt_write(const SampleParams& P, const FiltRow& r, float Rf, double fS, uint32_t thr,
                                           uint64_t kept_n, float xl) {
  if (threadIdx.x == 0) {
    P.f_R[r.fr] = Rf;
    P.f_S[r.fr] = fS;
    P.f_thr[r.fr] = thr;
    if (P.out_kept) P.out_kept[r.fr] = static_cast<int32_t>(kept_n);
    if (r.tok_slot >= 0) P.p1_x[static_cast<int64_t>(r.b) * 2 * P.K + r.tok_slot] = xl;
  }
}

// The logit with order key k (k the key of a number).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// The value of lane ^ S. Strides inside a row of 16 lanes take two DPP row shifts
// (lane + S for lanes with bit S clear, lane - S for the others, both inside the
// row); 16 and 32 take an LDS-routed shuffle.
template <int S>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (S <= 8) {
    const uint32_t up = dpp::mov<0x100 + S, 0xf>(v, v);  // row_shl:S, lane + S
    const uint32_t dn = dpp::mov<0x110 + S, 0xf>(v, v);  // row_shr:S, lane - S
    return (threadIdx.x & S) ? dn : up;
  } else {
    return static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), S, 64));
  }
}

template <int SIZE, int STRIDE>
__device__ __forceinline__ uint32_t bitonic_step(uint32_t v) {
  const int lane = threadIdx.x & 63;
  const uint32_t o = lane_xor<STRIDE>(v);
  const bool up = (lane & SIZE) == 0;
  const bool first = (lane & STRIDE) == 0;
  return (first == up) ? max(v, o) : min(v, o);
}

template <int SIZE, int STRIDE>
__device__ __forceinline__ uint32_t bitonic_merge(uint32_t v) {
  v = bitonic_step<SIZE, STRIDE>(v);
  if constexpr (STRIDE > 1) v = bitonic_merge<SIZE, STRIDE / 2>(v);
  return v;
}

// Descending bitonic sort of one key per lane across the wave (every lane active).
__device__ __forceinline__ uint32_t wave_sort_desc(uint32_t v) {
  v = bitonic_merge<2, 1>(v);
  v = bitonic_merge<4, 2>(v);
  v = bitonic_merge<8, 4>(v);
  v = bitonic_merge<16, 8>(v);
  v = bitonic_merge<32, 16>(v);
  v = bitonic_merge<64, 32>(v);
  return v;
}

// The cut by wave 0 alone when the candidates fit its registers (n <= 512) and
// top-k keeps at most 64 entries: the k-th largest key by a bitwise search, the
// kept keys sorted one per lane, and the top-p group from an exact fp64 lane scan
// of their fixed-point masses (integers below 2^47). False (nothing written) when
// it does not apply.
template <bool kBf16, typename MassF>
__device__ bool wave_cut(FastBuf& fb, int n, int kk, float pp, MassF&& mass, uint32_t lo, uint32_t hi) {
  constexpr int R = 8;
  const int lane = threadIdx.x & 63;
  uint32_t kr[R];
#pragma unroll
  for (int j = 0; j < R; ++j) kr[j] = (j * 64 + lane < n) ? order_key(__uint_as_float(fb.key[j * 64 + lane])) : 0u;
  // The k-th largest key t lies in [lo, hi], so it has their common leading bits:
  // the bitwise search starts below them. bf16 keys end in 16 zero bits (sign bit
  // set) or 16 one bits (clear), so their search stops at bit 16.
  constexpr int kBottom = kBf16 ? 16 : 0;
  uint32_t tk = lo;
  int top = -1;
  if (lo != hi) {
    top = 31 - __clz(lo ^ hi);
    tk = (top == 31) ? 0u : (lo & ~((2u << top) - 1u));
  }
#pragma unroll 1
  for (int bit = top; bit >= kBottom; --bit) {
    const uint32_t cand = tk | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < R; ++j) cnt += __popcll(__ballot(kr[j] >= cand));
    if (cnt >= kk) tk = cand;
  }
  if (kBf16) tk = (tk & 0xFFFF0000u) | ((tk & 0x80000000u) ? 0u : 0xFFFFu);
  int c = 0;
#pragma unroll
  for (int j = 0; j < R; ++j) c += __popcll(__ballot(kr[j] >= tk));
  if (c > 64) return false;
  int at = 0;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const uint64_t bal = __ballot(kr[j] >= tk);
    if (kr[j] >= tk) fb.kept[at + __popcll(bal & ((1ull << lane) - 1))] = kr[j];
    at += __popcll(bal);
  }
  // the wave reads what its own lanes wrote
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint32_t key = wave_sort_desc(lane < c ? fb.kept[lane] : 0u);
  const double m = lane < c ? static_cast<double>(mass(key)) : 0.0;
  const double incl = wave_scan_add(m);
  const double Z = lane_d(incl, 63);
  uint32_t tp = tk;
  if (pp < 1.f) {
    const double Pm = static_cast<double>(pp) * Z;
    const int j = first_lane(lane < c && incl >= Pm);
    tp = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(key), j < 64 ? j : 0));
  }
  const bool kept = lane < c && key >= tp;
  const double km = lane_d(wave_scan_add(kept ? m : 0.0), 63);
  const uint32_t kn = static_cast<uint32_t>(__popcll(__ballot(kept)));
  if (lane == 0) {
    fb.res_thr = tp;
    fb.res_n = kn;
    fb.res_m = static_cast<unsigned long long>(km);
  }
  return true;
}

// The cut of a one-pass row from its candidates (n <= kFiltCap order keys in fb.key;
// M the row maximum).
template <typename T>
__device__ void cut_candidates(const SampleParams& P, const FiltRow& r, FastBuf& fb, int n, float M, int kk,
                               float pp, float xl, uint32_t lbound) {
  if (!(M > -INFINITY)) {  // no finite logit: the row keeps nothing
    filt_write(P, r, 0.f, 0.0, 0xFFFFFFFFu, 0, xl);
    __syncthreads();
    return;
  }
  const float c = P.c;
  const float Rf = M * c + 1.f;  // masses 2^(x*c - Rf) stay <= 1, as in the multi-pass path
  auto mass = [&](uint32_t key) {
    return to_fixed(fminf(exp2_hw(fmaf(key_value(key), c, -Rf)), 1.f));
  };
  if (n <= 512) {  // the common case: wave 0 alone, on the raw candidates
    __shared__ int wave_done;
    if (threadIdx.x < 64) {
      // wave 0's final bound is at most the k-th largest key, the row maximum at least
      const bool done = wave_cut<sizeof(T) == 2>(fb, n, kk, pp, mass, lbound, order_key(M));
      if (threadIdx.x == 0) wave_done = done;
    }
    __syncthreads();
    if (wave_done) {
      uint32_t thr = fb.res_thr;
      if (sizeof(T) == 2) thr &= ~0x3FFu;
      filt_write(P, r, Rf, static_cast<double>(fb.res_m) * 0x1p-40, thr, fb.res_n, xl);
      __syncthreads();  // shared memory is reused by the next row
      return;
    }
  }
  // otherwise the whole workgroup sorts the candidates, as order keys padded with 0
  // (below the key of every number) to a power of two; n >= k, since at least k
  // entries reach the final bound
  int npad = 1;
  while (npad < n) npad <<= 1;
  for (int i = threadIdx.x; i < npad; i += kFiltBlock) fb.key[i] = i < n ? order_key(__uint_as_float(fb.key[i])) : 0u;
  __syncthreads();
  sort_keys_desc(fb.key, npad);
  // each thread takes a contiguous run of sorted positions
  const int per = (npad + kFiltBlock - 1) / kFiltBlock;
  const int i0 = min(static_cast<int>(threadIdx.x) * per, npad), i1 = min(i0 + per, npad);
  // top-k: the k-th largest key; the row keeps every entry at or above it
  const uint32_t tk = fb.key[kk - 1];
  uint64_t ms = 0, cn = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = fb.key[i];
    if (key >= tk) {
      ms += mass(key);
      ++cn;
    }
  }
  uint64_t Z;
  const uint64_t before = block_excl_u64(ms, Z);
  uint32_t thr = tk;
  uint64_t kept_n = block_sum_u64(cn), kept_m = Z;
  if (pp < 1.f) {
    // top-p on the top-k law: the first key group (descending) whose running mass
    // reaches p * Z, and every key above it (p <= 0: the largest key's group)
    const double Pm = static_cast<double>(pp) * static_cast<double>(Z);
    int32_t first = INT32_MAX;
    uint64_t run = before;
    for (int i = i0; i < i1; ++i) {
      const uint32_t key = fb.key[i];
      if (key < tk) break;
      run += mass(key);
      if (static_cast<double>(run) >= Pm) {
        first = i;
        break;
      }
    }
    // a crossing always exists (the last kept entry brings the run to Z >= p * Z); the
    // clamp only guards the index
    const uint32_t tp = fb.key[min(block_min_i32(fb.wmin, first), npad - 1)];
    uint64_t ms2 = 0, cn2 = 0;
    for (int i = i0; i < i1; ++i) {
      const uint32_t key = fb.key[i];
      if (key >= tp) {
        ms2 += mass(key);
        ++cn2;
      }
    }
    thr = tp;
    kept_m = block_sum_u64(ms2);
    kept_n = block_sum_u64(cn2);
  }
  // bf16 keys carry 16 bits: the threshold the multi-pass select gives has its low 10 bits clear
  if (sizeof(T) == 2) thr &= ~0x3FFu;
  filt_write(P, r, Rf, static_cast<double>(kept_m) * 0x1p-40, thr, kept_n, xl);
  __syncthreads();  // shared memory is reused by the next row
}

// One-pass top-k path of a row (0 < k <= 64): the candidates, then the cut. False
// (nothing written) when the candidates overflow the buffer.
template <typename T>
__device__ __forceinline__ bool filter_row_fast(const SampleParams& P, const FiltRow& r, FastBuf& fb, int kk, float pp, float xl) {
  float M;
  uint32_t lbound;
  const uint32_t n = collect_candidates(static_cast<const T*>(r.row), P.V, kk, fb, M, lbound);
  if (n > static_cast<uint32_t>(kFiltCap)) {
    __syncthreads();  // shared memory is reused by the multi-pass select
    return false;
  }
  cut_candidates<T>(P, r, fb, static_cast<int>(n), M, kk, pp, xl, lbound);
  return true;
}

// ---------------------------------------------------------------- one-read top-p and large top-k
//
// A row with top-p on, or with top-k and k > 64, is read once as well. The first
// step of the read (kFastUnroll * 256 16-byte vectors) doubles as a sample: a
// histogram of its entries by their distance below the sample maximum, in bins of
// half a doubling of the tempered mass, gives a bound L meant to lie below the
// row's cut. Top-p alone takes the smallest L whose sample mass above it reaches
// (1 + p) / 2 of the sample's mass; top-k the smallest L whose sample count above
// it, scaled to the row, reaches 1.25k + 16. The read then keeps every entry >= L
// in an LDS buffer as an order key and, for top-p alone, sums the mass of the
// others. The cut runs on the buffer: a radix select over the key span of the
// candidates, with the masses of the multi-pass select (the same fixed point
// against the same reference). It is exact whenever the buffer holds the cut: top-k
// needs k candidates; top-p alone needs the candidates' mass to reach p * Z, where
// Z adds the rest of the row's mass. A row that fails either test, whose buffer
// overflows, or whose sample predicts an overflow, takes the multi-pass select.

constexpr int kWideWords = 6144;  // candidate buffer: 24 KB of keys (16-bit keys for bf16 rows, 32-bit for fp32)
constexpr int kSampleBins = 64;   // half-doubling bins below the sample maximum
constexpr int kWideBins = 256;    // radix digit of the cut
constexpr uint32_t kNoPick = 0xFFFFFFFFu;
static_assert(kWideBins == kFiltBlock, "one bin per thread in the scans");

// Stored keys of the buffer. fp32 rows: the 32-bit order key.
template <typename T>
struct WideKey {
  static constexpr int kCap = kWideWords;
  __device__ __forceinline__ static uint32_t get(const uint32_t* w, int i) { return w[i]; }
  __device__ __forceinline__ static void put(uint32_t* w, uint32_t i, float x) { w[i] = order_key(x); }
  __device__ __forceinline__ static uint32_t full(uint32_t k) { return k; }
  __device__ __forceinline__ static uint32_t thr(uint32_t k) { return k; }
};
// bf16 rows: the upper half of the order key (the lower half is 0 for a value with
// its sign clear, all ones otherwise), so twice as many fit; the threshold takes the
// form the multi-pass select gives bf16 rows (low 10 bits clear).
template <>
struct WideKey<bf16_t> {
  static constexpr int kCap = 2 * kWideWords;
  __device__ __forceinline__ static uint32_t get(const uint32_t* w, int i) {
    return reinterpret_cast<const uint16_t*>(w)[i];
  }
  __device__ __forceinline__ static void put(uint32_t* w, uint32_t i, float x) {
    reinterpret_cast<uint16_t*>(w)[i] = static_cast<uint16_t>(order_key(x) >> 16);
  }
  __device__ __forceinline__ static uint32_t full(uint32_t k) { return (k << 16) | ((k & 0x8000u) ? 0u : 0xFFFFu); }
  __device__ __forceinline__ static uint32_t thr(uint32_t k) { return full(k) & ~0x3FFu; }
};

constexpr int kHistKeys = 4096;   // long bf16 rows: one count per key, over 32 binades
constexpr int kHighRoom = 256;    // the counted keys reach two binades above the sample maximum
constexpr int kHighCap = 256;     // entries above them, kept as keys

struct WideBuf {
  union {
    uint32_t key[kWideWords];  // candidate keys
    struct {
      uint32_t cnt[kHistKeys];  // entries per bf16 key, from the bottom key up
      uint32_t high[kHighCap];  // keys above the counted ones
    } h;
  };
  uint32_t cnt[kWideBins];
  unsigned long long mass[kWideBins];
  uint32_t nbuf;
  float L;  // the candidate bound (-inf: every entry)
  int go;   // 0: the sample predicts more candidates than the buffer holds
  uint32_t pick_bin;
  uint64_t pick_above_cnt, pick_above_mass;
  float wmax[kFiltBlock / 64];
  int32_t wmin[kFiltBlock / 64];
  uint32_t wkey[2][kFiltBlock / 64];
  double wsum[kFiltBlock / 64];
};

// The candidate bound from the sample: every thread's vectors of the first step.
template <typename T, int U>
__device__ void wide_bound(WideBuf& wb, const u32x4 (&raw)[U], int64_t V, int kk, bool k_on, float pp, float c) {
  constexpr int VEC = Elem<T>::kVec;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float sm = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float y[VEC];
    Elem<T>::unpack(raw[u], y);
#pragma unroll
    for (int e = 0; e < VEC; ++e) sm = fmaxf(sm, y[e]);
  }
  sm = wave_max(sm);
  wb.cnt[threadIdx.x] = 0;
  wb.mass[threadIdx.x] = 0;
  if (lane == 0) wb.wmax[w] = sm;
  __syncthreads();
  float Ms = wb.wmax[0];
#pragma unroll
  for (int o = 1; o < kFiltBlock / 64; ++o) Ms = fmaxf(Ms, wb.wmax[o]);
  if (Ms > -INFINITY) {
    const float c2 = 2.f * c;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float y[VEC];
      Elem<T>::unpack(raw[u], y);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float d = (Ms - y[e]) * c2;  // NaN and +inf fail the test
        if (d < static_cast<float>(kSampleBins)) {
          const int j = static_cast<int>(d);
          atomicAdd(&wb.cnt[j], 1u);
          // the sample's masses against its maximum, in units of 2^-24 (deterministic sums)
          atomicAdd(&wb.mass[j], static_cast<unsigned long long>(exp2_hw((y[e] - Ms) * c) * 16777216.f + 0.5f));
        }
      }
    }
  }
  __syncthreads();
  if (w == 0) {
    float L = -INFINITY;
    int go = V <= WideKey<T>::kCap;
    if (Ms > -INFINITY) {
      const double cn = wave_scan_add(static_cast<double>(wb.cnt[lane]));  // bins 0..lane: within (lane+1)/2 doublings
      const double ms = wave_scan_add(static_cast<double>(wb.mass[lane]));
      const double scale = static_cast<double>(V) / static_cast<double>(U * kFiltBlock * VEC);
      // top-k: the sample count expected above the k-th largest, plus three of its
      // standard deviations and a little more; top-p: half of the way from p to 1
      const double a = static_cast<double>(kk) / scale;
      const bool hit = k_on ? cn >= a + 3.0 * sqrt(a) + 4.0
                            : ms >= 0.5 * (1.0 + static_cast<double>(fmaxf(pp, 0.f))) * lane_d(ms, 63);
      const int j = first_lane(hit);
      if (j < 64) {
        L = Ms - static_cast<float>(j + 1) * 0.5f / c;
        go = lane_d(cn, j) * scale <= 0.9 * static_cast<double>(WideKey<T>::kCap);
      }
    }
    if (lane == 0) {
      wb.L = L;
      wb.go = go;
    }
  }
  __syncthreads();
}

// Append the lane's values whose bit is set in `take` to the buffer (lane order).
template <typename T, int N>
__device__ __forceinline__ void wide_append(WideBuf& wb, const float (&x)[N], uint32_t take) {
  uint32_t pos = reserve_slots(wb.nbuf, static_cast<uint32_t>(__popc(take)));
#pragma unroll
  for (int i = 0; i < N; ++i)
    if ((take >> i) & 1u) {
      if (pos < static_cast<uint32_t>(WideKey<T>::kCap)) WideKey<T>::put(wb.key, pos, x[i]);
      ++pos;
    }
}

// Read a wide-path row once: its maximum, the candidates (every entry >= L, as keys
// in wb.key; n_out of them, more than the buffer holds on an overflow) and, with
// need_rest, each thread's sum of 2^(x*c - fl(L*c)) over its other entries. False
// when the sample sends the row to the multi-pass select.
template <typename T, bool need_rest>
__device__ bool wide_collect(const T* row, int64_t V, WideBuf& wb, int kk, bool k_on, float pp, float c,
                             float& rowmax, float& L_out, double& rest_out, uint32_t& n_out) {
  constexpr int VEC = Elem<T>::kVec;
  constexpr int BS = kFiltBlock, U = kWideUnroll, W = kFiltBlock / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x == 0) wb.nbuf = 0;
  const int64_t h = head_elems(row, V);
  const int64_t nvec = (V - h) / VEC;
  const u32x4* vb = reinterpret_cast<const u32x4*>(row + h);
  const int64_t nsteps = nvec / (U * BS);
  // a row longer than the buffer has at least one whole step (V > 8192 entries
  // leaves more than 2047 vectors, and a step is 1024), which is the sample
  const bool sampling = V > WideKey<T>::kCap;
  float L = -INFINITY, Lc = -INFINITY;
  float m = -INFINITY;
  double rest = 0.0;
  if (!sampling) __syncthreads();  // nbuf = 0 before any append (the sample's barriers order it otherwise)
  for (int64_t s = 0; s < nsteps; ++s) {
    u32x4 cur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = load_stream(vb + s * (U * BS) + threadIdx.x + u * BS);
    if (s == 0 && sampling) {
      wide_bound<T, U>(wb, cur, V, kk, k_on, pp, c);
      if (!wb.go) return false;  // uniform
      L = wb.L;
      Lc = L * c;
    }
    uint32_t tk[U];
    uint32_t cnt = 0;
    float rs = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float y[VEC];
      Elem<T>::unpack(cur[u], y);
      uint32_t t = 0;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        m = fmaxf(m, y[e]);
        t |= (y[e] >= L ? 1u : 0u) << e;
        if (need_rest) rs += (y[e] < L) ? exp2_hw(fmaf(y[e], c, -Lc)) : 0.f;
      }
      tk[u] = t;
      cnt += __popc(t);
    }
    rest += static_cast<double>(rs);
    uint32_t pos = reserve_slots(wb.nbuf, cnt);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      for (uint32_t t = tk[u]; t != 0u; t &= t - 1u) {
        if (pos < static_cast<uint32_t>(WideKey<T>::kCap))
          WideKey<T>::put(wb.key, pos, Elem<T>::lane_elem(cur[u], __ffs(t) - 1));
        ++pos;
      }
    }
  }
  // the last vectors, one per thread, then the scalar head (lanes 0-7 of wave 0) and
  // tail (lanes 8-15): every lane of each wave takes part in the appends
  for (int64_t base = nsteps * (U * BS); base < nvec; base += BS) {
    const int64_t vr = base + threadIdx.x;
    const bool in = vr < nvec;
    float x[VEC];
    if (in) {
      Elem<T>::unpack(load_stream(vb + vr), x);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) x[e] = -INFINITY;
    }
    uint32_t take = 0;
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      m = fmaxf(m, x[e]);
      take |= (in && x[e] >= L ? 1u : 0u) << e;
      if (need_rest) rs += (in && x[e] < L) ? exp2_hw(fmaf(x[e], c, -Lc)) : 0.f;
    }
    rest += static_cast<double>(rs);
    wide_append<T>(wb, x, take);
  }
  if (w == 0) {
    const int64_t tail_lo = h + nvec * VEC;
    const int64_t e = lane < 8 ? lane : tail_lo + (lane - 8);
    const bool in = lane < 8 ? lane < h : (lane < 16 && e < V);
    float x[1];
    x[0] = in ? Elem<T>::get(row, e) : -INFINITY;
    m = fmaxf(m, x[0]);
    if (need_rest && in && x[0] < L) rest += static_cast<double>(exp2_hw(fmaf(x[0], c, -Lc)));
    wide_append<T>(wb, x, (in && x[0] >= L) ? 1u : 0u);
  }
  const float wm = wave_max(m);
  if (lane == 0) wb.wmax[w] = wm;
  __syncthreads();
  float M = wb.wmax[0];
#pragma unroll
  for (int o = 1; o < W; ++o) M = fmaxf(M, wb.wmax[o]);
  rowmax = M;
  L_out = L;
  rest_out = rest;
  n_out = wb.nbuf;
  return true;
}

// Sum of one fp64 value per thread over the block, in a fixed order (every thread gets it).
__device__ __forceinline__ double block_sum_f64(WideBuf& wb, double v) {
  const double s = wave_sum(v);
  if ((threadIdx.x & 63) == 0) wb.wsum[threadIdx.x >> 6] = s;
  __syncthreads();
  double t = wb.wsum[0];
#pragma unroll
  for (int o = 1; o < kFiltBlock / 64; ++o) t += wb.wsum[o];
  __syncthreads();
  return t;
}

// Histogram of the digit (key - base) >> shift & 255 over the candidates with key >=
// lo whose digits above it equal `prefix` (every candidate at the top level); with
// MASS also their fixed-point masses. The scan's pick is reset to kNoPick.
template <typename T, bool MASS, typename MassF>
__device__ void hist_wide(WideBuf& wb, int n, uint32_t base, int shift, bool top, uint32_t prefix, uint32_t lo,
                          MassF&& mass) {
  wb.cnt[threadIdx.x] = 0;
  wb.mass[threadIdx.x] = 0;
  if (threadIdx.x == 0) wb.pick_bin = kNoPick;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kFiltBlock) {
    const uint32_t k = WideKey<T>::get(wb.key, i);
    const uint32_t d = k - base;
    // below the top level shift + 8 <= 24
    if (k < lo || (!top && (d >> (shift + 8)) != prefix)) continue;
    const int b = static_cast<int>((d >> shift) & 255u);
    atomicAdd(&wb.cnt[b], 1u);
    if (MASS) atomicAdd(&wb.mass[b], static_cast<unsigned long long>(mass(k)));
  }
  __syncthreads();
}

// Scan the 256 bins from the top (thread t holds bin 255 - t) and pick, as
// scan_hist does, the bin where the count from the top reaches r (COUNT) or the
// first bin holding entries where A0 plus the mass from the top reaches P (MASS;
// P <= 0: the first bin holding entries). No bin qualifies: the pick stays kNoPick.
template <bool MASS>
__device__ void scan_wide(WideBuf& wb, uint64_t r, double P, uint64_t A0) {
  const int b = kWideBins - 1 - static_cast<int>(threadIdx.x);
  const uint64_t c = wb.cnt[b], m = wb.mass[b];
  uint64_t total;
  const uint64_t ec = block_excl_u64(c, total);
  const uint64_t em = block_excl_u64(m, total);
  bool mine;
  if (MASS) {
    mine = c > 0 && ((P <= 0.0) ? ec == 0
                                : (static_cast<double>(A0 + em) < P && static_cast<double>(A0 + em + m) >= P));
  } else {
    mine = ec < r && ec + c >= r;
  }
  if (mine) {
    wb.pick_bin = static_cast<uint32_t>(b);
    wb.pick_above_cnt = ec;
    wb.pick_above_mass = em;
  }
  __syncthreads();
}

// The cut of a wide-path row from its n candidates: top-k (the k-th largest key),
// then top-p on the top-k law, or on the whole row when top-k is off (the row's mass
// outside the buffer is Zrest). False (nothing written) when the buffer does not
// hold the cut. Results as in the multi-pass select.
// With Aabove > 0 (top-p alone), the buffer holds a band of keys and Nabove entries of
// mass Aabove lie above it: the cut runs from that mass on, and those entries are kept.
template <typename T>
__device__ bool wide_cut(WideBuf& wb, int n, int kk, bool k_on, float pp, bool p_on, float c, float Rf,
                         uint64_t Zrest, uint32_t& thr_out, uint64_t& kept_n, uint64_t& kept_m,
                         uint64_t Aabove = 0, uint64_t Nabove = 0) {
  using WK = WideKey<T>;
  const int w = threadIdx.x >> 6;
  auto mass = [&](uint32_t k) { return to_fixed(fminf(exp2_hw(fmaf(key_value(WK::full(k)), c, -Rf)), 1.f)); };
  // the key span of the candidates sets the digits: (key - kmin) in as few 8-bit digits as it needs
  uint32_t lo_k = 0xFFFFFFFFu, hi_k = 0u;
  for (int i = threadIdx.x; i < n; i += kFiltBlock) {
    const uint32_t k = WK::get(wb.key, i);
    lo_k = min(lo_k, k);
    hi_k = max(hi_k, k);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo_k = min(lo_k, static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo_k), o, 64)));
    hi_k = max(hi_k, static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi_k), o, 64)));
  }
  if ((threadIdx.x & 63) == 0) {
    wb.wkey[0][w] = lo_k;
    wb.wkey[1][w] = hi_k;
  }
  __syncthreads();
  uint32_t kmin = wb.wkey[0][0], kmax = wb.wkey[1][0];
#pragma unroll
  for (int o = 1; o < kFiltBlock / 64; ++o) {
    kmin = min(kmin, wb.wkey[0][o]);
    kmax = max(kmax, wb.wkey[1][o]);
  }
  const uint32_t span = kmax - kmin;
  const int levels = span ? (32 - __clz(static_cast<int>(span)) + 7) / 8 : 1;
  uint32_t lo = 0;
  if (k_on) {
    if (n < kk) return false;  // uniform
    uint32_t prefix = 0;
    uint64_t r = static_cast<uint64_t>(kk);
    for (int lev = 0; lev < levels; ++lev) {
      hist_wide<T, false>(wb, n, kmin, 8 * (levels - 1 - lev), lev == 0, prefix, 0u, mass);
      scan_wide<false>(wb, r, 0.0, 0);
      const uint32_t pb = wb.pick_bin;
      r -= wb.pick_above_cnt;
      __syncthreads();  // every thread has read the pick before the next level resets it
      if (pb == kNoPick) return false;
      prefix = (prefix << 8) | pb;
    }
    lo = kmin + prefix;
  }
  uint32_t thr = lo;
  if (p_on) {
    uint64_t zc = 0;
    for (int i = threadIdx.x; i < n; i += kFiltBlock) {
      const uint32_t k = WK::get(wb.key, i);
      if (k >= lo) zc += mass(k);
    }
    const uint64_t Zc = block_sum_u64(zc);
    const double Pm = static_cast<double>(pp) * static_cast<double>(Zc + Zrest + Aabove);
    if (static_cast<double>(Zc + Aabove) < Pm) return false;  // the cut lies below the bound
    if (Aabove > 0 && static_cast<double>(Aabove) >= Pm) return false;  // above the band
    uint32_t prefix = 0;
    uint64_t A0 = Aabove;
    for (int lev = 0; lev < levels; ++lev) {
      hist_wide<T, true>(wb, n, kmin, 8 * (levels - 1 - lev), lev == 0, prefix, lo, mass);
      scan_wide<true>(wb, 0, Pm, A0);
      const uint32_t pb = wb.pick_bin;
      A0 += wb.pick_above_mass;
      __syncthreads();
      if (pb == kNoPick) return false;
      prefix = (prefix << 8) | pb;
    }
    thr = kmin + prefix;
  }
  uint64_t cn = 0, ms = 0;
  for (int i = threadIdx.x; i < n; i += kFiltBlock) {
    const uint32_t k = WK::get(wb.key, i);
    if (k >= thr) {
      ++cn;
      ms += mass(k);
    }
  }
  kept_n = block_sum_u64(cn) + Nabove;
  kept_m = block_sum_u64(ms) + Aabove;
  thr_out = WK::thr(thr);
  return true;
}

// ---------------------------------------------------------------- long bf16 rows: a count per key
//
// A bf16 logit takes one of 2^16 keys, and entries with equal keys have equal
// masses, so counts per key describe the top of a row exactly, whatever the number
// of entries there. A long bf16 row takes that route instead of the buffer: the
// sample maximum's key, plus two binades, is the top of kHistKeys bins of one key
// each (32 binades), and the read adds each entry to its bin. Entries above the bins
// (a peak the sample missed) go to a short list of keys; entries below them add their
// mass to the rest (top-p alone). The cut scans the list, sorted, then the bins from
// the top; the mass of a bin is its count times the fixed-point mass of its key, the
// sum the multi-pass select forms entry by entry.

// bf16 key (upper half of the order key) of a widened bf16 value, and its value.
__device__ __forceinline__ uint32_t key16(float x) { return order_key(x) >> 16; }
__device__ __forceinline__ float key16_value(uint32_t k) { return key_value(WideKey<bf16_t>::full(k)); }
constexpr uint32_t kKey16NegInf = 0x007Fu;  // the smallest key of a number

// One thread's entries of a bf16 row: two per 32-bit word, `valid` marking the
// words that hold entries. Keys are formed two at a time (a negative half flips all
// 16 bits, a positive one its sign bit; -0 takes the key 0x7FFF, merged into +0's
// bin after the read). Each entry goes to its bin, to the high list (above the
// bins, rare: a wave-uniform slow path) or, for top-p alone, to the rest sum.
template <int NW>
__device__ __forceinline__ void hist16_words(WideBuf& wb, const uint32_t (&w)[NW], uint32_t valid, uint32_t bottom,
                                             float hiV, float loV, float c, float Lc, bool need_rest, float& m,
                                             float& rs) {
  float vmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    if (!((valid >> j) & 1u)) continue;
    const uint32_t k2 = w[j] ^ ((((w[j] >> 15) & 0x00010001u) * 0x7FFFu) | 0x80008000u);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint32_t k = half ? (k2 >> 16) : (k2 & 0xFFFFu);
      const float y = __uint_as_float(half ? (w[j] & 0xFFFF0000u) : (w[j] << 16));
      vmax = fmaxf(vmax, y);
      // keys bottom .. bottom + 4095 are counted (NaN keys lie outside: see hist16_collect)
      const uint32_t d = k - bottom;
      if (d < static_cast<uint32_t>(kHistKeys)) atomicAdd(&wb.h.cnt[d], 1u);
      if (need_rest) rs += (y < loV) ? exp2_hw(fmaf(y, c, -Lc)) : 0.f;
    }
  }
  m = fmaxf(m, vmax);
  if (__ballot(vmax > hiV)) {  // rare: entries above the counted keys
    uint32_t take = 0;
#pragma unroll
    for (int j = 0; j < NW; ++j)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const float y = __uint_as_float(half ? (w[j] & 0xFFFF0000u) : (w[j] << 16));
        take |= (((valid >> j) & 1u) && y > hiV ? 1u : 0u) << (2 * j + half);
      }
    uint32_t pos = reserve_slots(wb.nbuf, static_cast<uint32_t>(__popc(take)));
#pragma unroll
    for (int e = 0; e < 2 * NW; ++e)
      if ((take >> e) & 1u) {
        const uint32_t x = (e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16);
        if (pos < static_cast<uint32_t>(kHighCap)) wb.h.high[pos] = key16(__uint_as_float(x));
        ++pos;
      }
  }
}

// Read a long bf16 row once into the key counts. False when the row needs the
// multi-pass select (a sample with no finite logit). Outputs: the row maximum, the
// bottom key, each thread's rest sum 2^(x*c - fl(loV*c)) (need_rest) and loV, the
// value of the bottom key (-inf when every number is counted).
__device__ bool hist16_collect(const bf16_t* row, int64_t V, WideBuf& wb, float c, bool need_rest, float& rowmax,
                               uint32_t& bottom_out, float& loV_out, double& rest_out) {
  constexpr int VEC = 8, BS = kFiltBlock, U = kWideUnroll, W = kFiltBlock / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t h = head_elems(row, V);
  const int64_t nvec = (V - h) / VEC;
  const u32x4* vb = reinterpret_cast<const u32x4*>(row + h);
  const int64_t nsteps = nvec / (U * BS);  // >= 1: the caller takes rows longer than the buffer
  if (threadIdx.x == 0) wb.nbuf = 0;
  for (int i = threadIdx.x; i < kHistKeys; i += BS) wb.h.cnt[i] = 0;
  u32x4 cur[U];
#pragma unroll
  for (int u = 0; u < U; ++u) cur[u] = load_stream(vb + threadIdx.x + u * BS);
  float sm = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float y[VEC];
    Elem<bf16_t>::unpack(cur[u], y);
#pragma unroll
    for (int e = 0; e < VEC; ++e) sm = fmaxf(sm, y[e]);
  }
  sm = wave_max(sm);
  if (lane == 0) wb.wmax[w] = sm;
  __syncthreads();
  float Ms = wb.wmax[0];
#pragma unroll
  for (int o = 1; o < W; ++o) Ms = fmaxf(Ms, wb.wmax[o]);
  __syncthreads();  // wmax is written again at the end
  if (!(Ms > -INFINITY)) return false;  // uniform
  // counted keys: bottom .. bottom + 4095, topped kHighRoom keys above the sample
  // maximum's key; bottom >= the key of -inf and the top <= the key of +inf, so no
  // NaN key is counted
  const uint32_t top0 = min(key16(Ms) + static_cast<uint32_t>(kHighRoom), 0xFF80u);
  uint32_t bottom = max(top0 >= static_cast<uint32_t>(kHistKeys - 1) ? top0 - (kHistKeys - 1) : 0u, kKey16NegInf);
  // -0 (key 0x7FFF) and +0 (key 0x8000) fall on the same side of each end of the range
  if (bottom == 0x8000u) bottom = 0x7FFFu;
  if (bottom + (kHistKeys - 1) == 0x7FFFu) bottom += 1;
  const uint32_t top = bottom + (kHistKeys - 1);
  // above the counted keys: y > hiV; below them: y < loV
  const float hiV = top < 0xFF80u ? key16_value(top) : INFINITY;  // 0xFF80: the key of +inf
  const float loV = bottom <= kKey16NegInf ? -INFINITY : key16_value(bottom);
  const float Lc = loV * c;
  float m = -INFINITY;
  double rest = 0.0;
  for (int64_t s = 0; s < nsteps; ++s) {
    if (s > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = load_stream(vb + s * (U * BS) + threadIdx.x + u * BS);
    }
    float rs = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t wd[4] = {cur[u].x, cur[u].y, cur[u].z, cur[u].w};
      hist16_words(wb, wd, 0xFu, bottom, hiV, loV, c, Lc, need_rest, m, rs);
    }
    rest += static_cast<double>(rs);
  }
  // the last vectors, one per thread, then the scalar head (lanes 0-7 of wave 0) and
  // tail (lanes 8-15): every lane of each wave takes part
  for (int64_t base = nsteps * (U * BS); base < nvec; base += BS) {
    const int64_t vr = base + threadIdx.x;
    const bool in = vr < nvec;
    const u32x4 v = in ? load_stream(vb + vr) : u32x4{0u, 0u, 0u, 0u};
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
    float rs = 0.f;
    hist16_words(wb, wd, in ? 0xFu : 0u, bottom, hiV, loV, c, Lc, need_rest, m, rs);
    rest += static_cast<double>(rs);
  }
  if (w == 0) {
    // one entry per lane, in the low half of a word whose high half is a NaN (not counted)
    const int64_t tail_lo = h + nvec * VEC;
    const int64_t e = lane < 8 ? lane : tail_lo + (lane - 8);
    const bool in = lane < 8 ? lane < h : (lane < 16 && e < V);
    const uint32_t wd[1] = {in ? (0x7FC00000u | static_cast<uint32_t>(row[e].bits)) : 0u};
    float rs = 0.f;
    hist16_words(wb, wd, in ? 1u : 0u, bottom, hiV, loV, c, Lc, need_rest, m, rs);
    rest += static_cast<double>(rs);
  }
  __syncthreads();
  // -0 was counted under key 0x7FFF: it belongs to +0 (key 0x8000; both or neither are counted)
  if (threadIdx.x == 0 && bottom <= 0x7FFFu && 0x8000u <= top) {
    wb.h.cnt[0x8000u - bottom] += wb.h.cnt[0x7FFFu - bottom];
    wb.h.cnt[0x7FFFu - bottom] = 0;
  }
  const float wm = wave_max(m);
  if (lane == 0) wb.wmax[w] = wm;
  __syncthreads();
  float M = wb.wmax[0];
#pragma unroll
  for (int o = 1; o < W; ++o) M = fmaxf(M, wb.wmax[o]);
  rowmax = M;
  bottom_out = bottom;
  loV_out = loV;
  rest_out = rest;
  return true;
}

// Scan the key counts from the top bin down to bin lo (thread t holds bins 4095 - 16t
// down to 4080 - 16t) and pick, as scan_hist does, the bin where the count from the
// top reaches r (COUNT) or the first bin holding entries where A0 plus the mass from
// the top reaches P (MASS; P <= 0: the first bin holding entries). No bin qualifies:
// the pick stays kNoPick.
template <bool MASS, typename FM>
__device__ void hist16_scan(WideBuf& wb, int lo, uint64_t r, double P, uint64_t A0, FM&& fm) {
  constexpr int per = kHistKeys / kFiltBlock;
  const int hi = kHistKeys - 1 - per * static_cast<int>(threadIdx.x);
  if (threadIdx.x == 0) wb.pick_bin = kNoPick;
  uint64_t tc = 0, tm = 0;
#pragma unroll 1
  for (int i = 0; i < per && hi - i >= lo; ++i) {
    const uint64_t n = wb.h.cnt[hi - i];
    tc += n;
    if (MASS && n) tm += n * fm(hi - i);
  }
  uint64_t total;
  const uint64_t ec = block_excl_u64(tc, total);
  const uint64_t em = MASS ? block_excl_u64(tm, total) : 0;
  bool mine;
  if (MASS) {
    mine = tc > 0 && ((P <= 0.0) ? ec == 0
                                 : (static_cast<double>(A0 + em) < P && static_cast<double>(A0 + em + tm) >= P));
  } else {
    mine = ec < r && ec + tc >= r;
  }
  if (mine) {
    uint64_t ca = ec, ma = em;
  #pragma unroll 1
  for (int i = 0; i < per && hi - i >= lo; ++i) {
      const uint64_t n = wb.h.cnt[hi - i];
      const uint64_t mm = (MASS && n) ? n * fm(hi - i) : 0;
      const bool hit = MASS ? (n > 0 && (P <= 0.0 || static_cast<double>(A0 + ma + mm) >= P)) : (ca + n >= r);
      if (hit) {
        wb.pick_bin = static_cast<uint32_t>(hi - i);
        wb.pick_above_cnt = ca;
        wb.pick_above_mass = ma;
        break;
      }
      ca += n;
      ma += mm;
    }
  }
  __syncthreads();
}

// The top-p cut of a long bf16 row from its key counts and high list (nh keys);
// Zrest is the mass below the counted keys. False (nothing written) when they do not
// hold the cut.
__device__ bool hist16_cut(WideBuf& wb, uint32_t nh, uint32_t bottom, float pp, float c, float Rf, uint64_t Zrest,
                           uint32_t& thr_out, uint64_t& kept_n, uint64_t& kept_m) {
  constexpr int per = kHistKeys / kFiltBlock;
  auto fmk = [&](uint32_t k) -> uint64_t { return to_fixed(fminf(exp2_hw(fmaf(key16_value(k), c, -Rf)), 1.f)); };
  auto fm = [&](int b) -> uint64_t { return fmk(bottom + static_cast<uint32_t>(b)); };
  // the high list, sorted descending (padded with key 0, below every number)
  int npad = 1;
  while (npad < static_cast<int>(nh)) npad <<= 1;
  if (nh > 1) {
    for (int i = static_cast<int>(nh) + threadIdx.x; i < npad; i += kFiltBlock) wb.h.high[i] = 0u;
    __syncthreads();
    sort_keys_desc(wb.h.high, npad);
  }
  const int t = threadIdx.x;
  // the list's masses wait in wb.mass (unused on this path): few registers stay live
  wb.mass[t] = t < static_cast<int>(nh) ? fmk(wb.h.high[t]) : 0u;
  const uint64_t Hm = block_sum_u64(wb.mass[t]);
  uint64_t zb = 0;
#pragma unroll 1
  for (int i = 0; i < per; ++i) {
    const int b = kHistKeys - 1 - per * t - i;
    const uint64_t n = wb.h.cnt[b];
    if (n) zb += n * fm(b);
  }
  const double Pm = static_cast<double>(pp) * static_cast<double>(Hm + block_sum_u64(zb) + Zrest);
  uint32_t thr;
  if (nh > 0 && (Pm <= 0.0 || static_cast<double>(Hm) >= Pm)) {
    // the cut is in the high list: the first entry (descending) whose running mass reaches p * Z
    uint64_t Ht;
    const uint64_t hbefore = block_excl_u64(wb.mass[t], Ht);  // list mass above entry t
    const bool hit = t < static_cast<int>(nh) && (Pm <= 0.0 || static_cast<double>(hbefore + wb.mass[t]) >= Pm);
    const int j = block_min_i32(wb.wmin, hit ? t : INT32_MAX);
    if (j == INT32_MAX) return false;
    thr = wb.h.high[j];
  } else {
    hist16_scan<true>(wb, 0, 0, Pm, Hm, fm);
    const uint32_t pb = wb.pick_bin;
    __syncthreads();
    if (pb == kNoPick) return false;  // the cut lies below the counted keys
    thr = bottom + pb;
  }
  // kept entries: the list's and the bins' at or above the threshold
  const bool hkept = t < static_cast<int>(nh) && wb.h.high[t] >= thr;
  uint64_t cn = hkept ? 1u : 0u, ms = hkept ? wb.mass[t] : 0u;
#pragma unroll 1
  for (int i = 0; i < per; ++i) {
    const int b = kHistKeys - 1 - per * t - i;
    if (bottom + static_cast<uint32_t>(b) < thr) break;
    const uint64_t n = wb.h.cnt[b];
    cn += n;
    if (n) ms += n * fm(b);
  }
  kept_n = block_sum_u64(cn);
  kept_m = block_sum_u64(ms);
  thr_out = WideKey<bf16_t>::thr(thr);
  return true;
}

// The mass of entries outside the buffer or the counted keys, summed by each
// thread against fl(L*c), moved to Rf in the fixed-point unit.
__device__ __forceinline__ uint64_t rest_fixed(WideBuf& wb, double rest, float L, float c, float Rf) {
  const double rt = block_sum_f64(wb, rest);
  return static_cast<uint64_t>(llrint(rt * pow2d(static_cast<double>(L * c) - static_cast<double>(Rf) + kFixBits)));
}

// The buffer route of a row (fp32 rows, short bf16 rows, top-k rows). False
// (nothing written) when it does not finish the row.
template <typename T>
__device__ __forceinline__ bool buffer_row(const SampleParams& P, const FiltRow& r, WideBuf& wb, int kk, bool k_on,
                                           float pp, bool p_on, float xl) {
  const float c = P.c;
  const bool need_rest = p_on && !k_on;
  float M, L;
  double rest;
  uint32_t n;
  const bool read = need_rest ? wide_collect<T, true>(static_cast<const T*>(r.row), P.V, wb, kk, k_on, pp, c, M, L, rest, n)
                              : wide_collect<T, false>(static_cast<const T*>(r.row), P.V, wb, kk, k_on, pp, c, M, L, rest, n);
  if (!read) {
    __syncthreads();
    return false;
  }
  if (!(M > -INFINITY)) {  // no finite logit: the row keeps nothing
    filt_write(P, r, 0.f, 0.0, 0xFFFFFFFFu, 0, xl);
    __syncthreads();
    return true;
  }
  if (n == 0 || n > static_cast<uint32_t>(WideKey<T>::kCap)) {
    __syncthreads();
    return false;
  }
  const float Rf = M * c + 1.f;  // as in the multi-pass select
  const uint64_t Zrest = (need_rest && L > -INFINITY) ? rest_fixed(wb, rest, L, c, Rf) : 0u;
  uint32_t thr;
  uint64_t kn, km;
  const bool ok = wide_cut<T>(wb, static_cast<int>(n), kk, k_on, pp, p_on, c, Rf, Zrest, thr, kn, km);
  if (ok) filt_write(P, r, Rf, static_cast<double>(km) * 0x1p-40, thr, kn, xl);
  __syncthreads();  // shared memory is reused by the next row
  return ok;
}

// The key-count route of a long bf16 row with top-p alone. False (nothing written)
// when it does not finish the row.
__device__ __forceinline__ bool hist16_row(const SampleParams& P, const FiltRow& r, WideBuf& wb, float pp, float xl) {
  const float c = P.c;
  constexpr bool need_rest = true;
  float M, L;
  double rest;
  uint32_t bottom;
  if (!hist16_collect(static_cast<const bf16_t*>(r.row), P.V, wb, c, need_rest, M, bottom, L, rest)) {
    __syncthreads();
    return false;
  }
  const uint32_t nh = wb.nbuf;
  if (nh > static_cast<uint32_t>(kHighCap)) {
    __syncthreads();
    return false;
  }
  const float Rf = M * c + 1.f;  // as in the multi-pass select
  const uint64_t Zrest = L > -INFINITY ? rest_fixed(wb, rest, L, c, Rf) : 0u;
  uint32_t thr;
  uint64_t kn, km;
  const bool ok = hist16_cut(wb, nh, bottom, pp, c, Rf, Zrest, thr, kn, km);
  if (ok) filt_write(P, r, Rf, static_cast<double>(km) * 0x1p-40, thr, kn, xl);
  __syncthreads();  // shared memory is reused by the next row
  return ok;
}

// ---------------------------------------------------------------- long fp32 rows with top-p alone: counts, then a band
//
// An fp32 row whose nucleus is larger than the buffer (a flat row with top-p alone)
// is read twice instead of going to the multi-pass select. The first read counts its
// entries in 4096 bins of 1/128 of a doubling of mass each (32 doublings), from one
// doubling above the first step's maximum down (entries above are kept as keys, those
// below summed as the rest), and finds the row maximum. A bin's entries take masses
// between those of its edges, so the counts bound the mass above every bin, and the
// bins where the cut can lie form a band. The second read sums every entry's fixed-point mass exactly, the
// whole row and the part above the band, and keeps the band's entries as keys; the cut
// then runs on them from the mass above the band. The masses and the reference are the
// multi-pass select's, so are the results. A bin index is a monotone function of the
// value computed the same way in both reads, so the band holds whole ties.

constexpr int kMassBins = 4096;       // bins of the first read (the bf16 route's key counts' memory)
#ifndef SV_F32_BINS_PER_DOUBLING
#define SV_F32_BINS_PER_DOUBLING 128
#endif
constexpr float kBinsPerDoubling = SV_F32_BINS_PER_DOUBLING;
constexpr double kRestSlack = 1e-5;   // relative bound on the rounding of the first read's rest sum
static_assert(kMassBins <= kHistKeys, "the bins use the key counts' memory");

// Bin of x: -1 above mref (the high list), kMassBins below the counted bins (or NaN).
__device__ __forceinline__ int mass_bin(float x, float mref, float s) {
  if (x > mref) return -1;
  const float d = (mref - x) * s;
  return d < static_cast<float>(kMassBins) ? static_cast<int>(d) : kMassBins;
}

// The entries of 16-byte vector v of an fp32 row (those whose bit is set in `valid`)
// in the first read: the maximum, the bin counts, the high list, the rest.
__device__ __forceinline__ void f32_count_vec(WideBuf& wb, const u32x4& v, uint32_t valid, float mref, float s,
                                              float c, float Lc, float& m, float& rs) {
  const float x[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
  float vmax = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (!((valid >> e) & 1u)) continue;
    vmax = fmaxf(vmax, x[e]);
    const float d = (mref - x[e]) * s;  // NaN for a NaN entry: no bin, no rest
    if (d >= 0.f && d < static_cast<float>(kMassBins)) atomicAdd(&wb.h.cnt[static_cast<int>(d)], 1u);
    rs += (d >= static_cast<float>(kMassBins)) ? exp2_hw(fmaf(x[e], c, -Lc)) : 0.f;
  }
  m = fmaxf(m, vmax);
  if (__ballot(vmax > mref)) {  // rare: entries above the counted bins, kept as full keys
    uint32_t take = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) take |= (((valid >> e) & 1u) && x[e] > mref ? 1u : 0u) << e;
    uint32_t pos = reserve_slots(wb.nbuf, static_cast<uint32_t>(__popc(take)));
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((take >> e) & 1u) {
        if (pos < static_cast<uint32_t>(kHighCap)) wb.h.high[pos] = order_key(x[e]);
        ++pos;
      }
  }
}

// Visit every entry of a long fp32 row with 16-byte loads, kWideUnroll per thread per
// step: f(vector, valid mask) for the whole vectors, then the scalar head (lanes 0-3 of
// wave 0) and tail (lanes 4-7) as vectors with one valid entry; every lane of each
// wave takes part in every call.
template <typename F>
__device__ __forceinline__ void f32_visit(const float* row, int64_t V, F&& f) {
  constexpr int VEC = 4, BS = kFiltBlock, U = kWideUnroll;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t h = head_elems(row, V);
  const int64_t nvec = (V - h) / VEC;
  const u32x4* vb = reinterpret_cast<const u32x4*>(row + h);
  const int64_t nsteps = nvec / (U * BS);
  for (int64_t st = 0; st < nsteps; ++st) {
    u32x4 cur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = load_stream(vb + st * (U * BS) + threadIdx.x + u * BS);
#pragma unroll
    for (int u = 0; u < U; ++u) f(cur[u], 0xFu);
  }
  for (int64_t base = nsteps * (U * BS); base < nvec; base += BS) {
    const int64_t vr = base + threadIdx.x;
    const bool in = vr < nvec;
    f(in ? load_stream(vb + vr) : u32x4{0u, 0u, 0u, 0u}, in ? 0xFu : 0u);
  }
  if (w == 0) {
    const int64_t tail_lo = h + nvec * VEC;
    const int64_t e = lane < 4 ? lane : tail_lo + (lane - 4);
    const bool in = lane < 4 ? lane < h : (lane < 8 && e < V);
    f(u32x4{in ? __float_as_uint(row[e]) : 0u, 0u, 0u, 0u}, in ? 1u : 0u);
  }
}

// The first read of a long fp32 row (V > the buffer): bin counts in wb.h.cnt, the
// entries above mref as keys in wb.h.high (wb.nbuf of them), each thread's rest sum
// 2^(x*c - fl(loV*c)) over the entries below the bins, and the row maximum. False
// when the row needs the multi-pass select (a first step with no finite logit).
__device__ bool f32_count(const float* row, int64_t V, WideBuf& wb, float c, float& rowmax, float& mref_out,
                          float& s_out, float& loV_out, double& rest_out) {
  constexpr int BS = kFiltBlock, U = kWideUnroll, W = kFiltBlock / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x == 0) wb.nbuf = 0;
  for (int i = threadIdx.x; i < kMassBins; i += BS) wb.h.cnt[i] = 0;
  // the first step's maximum places the bins
  const u32x4* vb = reinterpret_cast<const u32x4*>(row + head_elems(row, V));
  float sm = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const u32x4 v = load_stream(vb + threadIdx.x + u * BS);  // V > the buffer: a whole first step
    sm = fmaxf(sm, fmaxf(fmaxf(__uint_as_float(v.x), __uint_as_float(v.y)),
                         fmaxf(__uint_as_float(v.z), __uint_as_float(v.w))));
  }
  sm = wave_max(sm);
  if (lane == 0) wb.wmax[w] = sm;
  __syncthreads();
  float Ms = wb.wmax[0];
#pragma unroll
  for (int o = 1; o < W; ++o) Ms = fmaxf(Ms, wb.wmax[o]);
  __syncthreads();  // wmax is written again at the end
  if (!(Ms > -INFINITY) || !(Ms < INFINITY)) return false;  // uniform
  const float s = c * kBinsPerDoubling;                        // bins per unit of logit
  const float mref = Ms + 1.f / c;                             // one doubling of mass above
  const float loV = mref - static_cast<float>(kMassBins) / s;  // about where the bins end
  if (!(mref < INFINITY) || !(loV > -INFINITY)) return false;
  const float Lc = loV * c;
  float m = -INFINITY, rs = 0.f;
  double rest = 0.0;
  int k = 0;
  f32_visit(row, V, [&](u32x4 v, uint32_t valid) {
    f32_count_vec(wb, v, valid, mref, s, c, Lc, m, rs);
    if (++k == 8) {  // the rest into double every few vectors
      rest += static_cast<double>(rs);
      rs = 0.f;
      k = 0;
    }
  });
  rest += static_cast<double>(rs);
  __syncthreads();
  const float wm = wave_max(m);
  if (lane == 0) wb.wmax[w] = wm;
  __syncthreads();
  float M = wb.wmax[0];
#pragma unroll
  for (int o = 1; o < W; ++o) M = fmaxf(M, wb.wmax[o]);
  rowmax = M;
  mref_out = mref;
  s_out = s;
  loV_out = loV;
  rest_out = rest;
  return true;
}

// The largest value x with mass_bin(x) >= J (+inf for J <= -1). The bin index falls
// as the value rises, so mass_bin(x) < J exactly when x > this value (x not NaN); a
// bisection over the order keys from -inf (bin kMassBins >= J) finds it.
__device__ __forceinline__ float bin_floor_value(int J, float mref, float s) {
  if (J <= -1) return INFINITY;
  uint32_t lo = order_key(-INFINITY), hi = order_key(INFINITY);
  while (lo < hi) {
    const uint32_t mid = lo + (hi - lo + 1u) / 2u;
    if (mass_bin(key_value(mid), mref, s) >= J) {
      lo = mid;
    } else {
      hi = mid - 1u;
    }
  }
  return key_value(lo);
}

// One thread's fixed-point sums of the second read: the whole row, above the band, in
// the band (from the kept entries, after the read), and the count above it.
struct F32Sums {
  uint64_t zt = 0, za = 0, zb = 0, na = 0;
  double dt = 0.0, da = 0.0;  // whole numbers below 2^53, moved to zt/za
  __device__ __forceinline__ void flush() {
    zt += static_cast<uint64_t>(dt);
    za += static_cast<uint64_t>(da);
    dt = da = 0.0;
  }
};

// The fixed-point mass of x, round(m * 2^40) with m = min(2^(x*c - Rf), 1) rounded
// half up as to_fixed does, as a double: m * 2^40 is exact in fp32, and adding 1/2 to
// it is exact in fp64 (at most 24 significant bits, none below 2^-45).
__device__ __forceinline__ double fixed_mass_f64(float x, float c, float Rf) {
  const float m = fminf(exp2_hw(fmaf(x, c, -Rf)), 1.f);
  return floor(static_cast<double>(m * 0x1p40f) + 0.5);
}

// The second read keeps the band's entries in four parts of the buffer, one per wave,
// each wave counting its own entries in a register: a position of a step where some
// lane holds a band entry costs one ballot, a lane count and a store, no atomic.
constexpr int kBandWaves = kFiltBlock / 64;
constexpr uint32_t kBandPart = WideKey<float>::kCap / kBandWaves;  // entries per wave

// The entries of a 16-byte vector of the second read (those whose bit is set in
// `valid`; the same mask on every lane except at the row's ends): their sums, and the
// band's entries as raw bits in the wave's part `part`, n counting them (uniform; past
// kBandPart they are counted, not stored).
__device__ __forceinline__ void f32_band_vec(const u32x4& v, uint32_t valid, float c, float Rf, float Xa, float Xb,
                                             F32Sums& sm, uint32_t* part, uint32_t& n) {
  const float x[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool ok = (valid >> e) & 1u;
    const double q = ok ? fixed_mass_f64(x[e], c, Rf) : 0.0;
    const bool above = ok && x[e] > Xa, in_band = ok && x[e] > Xb && x[e] <= Xa;  // NaN: neither
    sm.dt += q;
    sm.da += above ? q : 0.0;
    sm.na += above ? 1u : 0u;
    const uint64_t bm = __ballot(in_band);
    if (bm != 0ull) {  // uniform
      if (in_band) {
        const uint32_t rank = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bm >> 32),
                                                        __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bm), 0u));
        if (n + rank < kBandPart) part[n + rank] = __float_as_uint(x[e]);
      }
      n += static_cast<uint32_t>(__popcll(bm));
    }
  }
}

// The second read of a long fp32 row: every entry's fixed-point mass summed (the row,
// above the band) and the band's entries kept, then gathered to wb.key[0..nb) as keys
// in wave order, their masses summed on the way. Whole steps of kWideUnroll vectors
// per thread, then the last vectors, the scalar head (lanes 0-3 of wave 0) and tail
// (lanes 4-7); every lane of each wave takes part in each vector. False (uniform)
// when a wave's part overflowed.
__device__ bool f32_band_read(const float* row, int64_t V, WideBuf& wb, float c, float Rf, float Xa, float Xb,
                              F32Sums& sm, uint32_t& nb) {
  constexpr int BS = kFiltBlock, U = kWideUnroll;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t h = head_elems(row, V);
  const int64_t nvec = (V - h) / 4;
  const u32x4* vb = reinterpret_cast<const u32x4*>(row + h);
  const int64_t nsteps = nvec / (U * BS);
  uint32_t* part = wb.key + w * kBandPart;
  uint32_t n = 0;
  int k = 0;
  for (int64_t st = 0; st < nsteps; ++st) {
    u32x4 cur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = load_stream(vb + st * (U * BS) + threadIdx.x + u * BS);
#pragma unroll
    for (int u = 0; u < U; ++u) f32_band_vec(cur[u], 0xFu, c, Rf, Xa, Xb, sm, part, n);
    if (++k == 256) {  // 3072 entries of at most 2^40 each: the sums stay whole below 2^53
      sm.flush();
      k = 0;
    }
  }
  for (int64_t base = nsteps * (U * BS); base < nvec; base += BS) {
    const int64_t vr = base + threadIdx.x;
    const bool in = vr < nvec;
    f32_band_vec(in ? load_stream(vb + vr) : u32x4{0u, 0u, 0u, 0u}, in ? 0xFu : 0u, c, Rf, Xa, Xb, sm, part, n);
  }
  if (w == 0) {
    const int64_t tail_lo = h + nvec * 4;
    const int64_t e = lane < 4 ? lane : tail_lo + (lane - 4);
    const bool in = lane < 4 ? lane < h : (lane < 8 && e < V);
    f32_band_vec(u32x4{in ? __float_as_uint(row[e]) : 0u, 0u, 0u, 0u}, in ? 1u : 0u, c, Rf, Xa, Xb, sm, part, n);
  }
  sm.flush();
  // gather the parts: wave o's entries go to [off[o], off[o] + cnt[o])
  if (lane == 0) wb.wkey[0][w] = n;
  __syncthreads();
  uint32_t cnt[kBandWaves], off[kBandWaves];
  uint32_t total = 0;
  bool over = false;
#pragma unroll
  for (int o = 0; o < kBandWaves; ++o) {
    cnt[o] = wb.wkey[0][o];
    over = over || cnt[o] > kBandPart;
    off[o] = total;
    total += cnt[o];
  }
  nb = total;
  if (over) return false;  // uniform
  constexpr int kPer = WideKey<float>::kCap / kFiltBlock;
  uint32_t tmp[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t i = threadIdx.x + static_cast<uint32_t>(j * kFiltBlock);
    tmp[j] = 0u;
    if (i < total) {
      int o = 0;
#pragma unroll
      for (int q = 1; q < kBandWaves; ++q) o += (i >= off[q]) ? 1 : 0;
      uint32_t base_o = off[0];
#pragma unroll
      for (int q = 1; q < kBandWaves; ++q) base_o = (o == q) ? off[q] : base_o;
      const float x = __uint_as_float(wb.key[o * kBandPart + (i - base_o)]);
      tmp[j] = order_key(x);
      sm.zb += static_cast<uint64_t>(fixed_mass_f64(x, c, Rf));
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t i = threadIdx.x + static_cast<uint32_t>(j * kFiltBlock);
    if (i < total) wb.key[i] = tmp[j];
  }
  __syncthreads();
  return true;
}

// Top-p alone on a long fp32 row in two reads (see above). False (nothing written)
// when the counts cannot place the cut in a band that fits the buffer: the row then
// takes the multi-pass select.
__device__ __forceinline__ bool f32_topp_row(const SampleParams& P, const FiltRow& r, WideBuf& wb, float pp,
                                             float xl) {
  const float c = P.c;
  const float* row = static_cast<const float*>(r.row);
  const int64_t V = P.V;
  if (!(pp > 0.f)) return false;  // uniform: p <= 0 keeps the largest logit's entries (the multi-pass select)
  float M, mref, s, loV;
  double rest;
  if (!f32_count(row, V, wb, c, M, mref, s, loV, rest)) {
    __syncthreads();
    return false;
  }
  const uint32_t nh = wb.nbuf;
  if (nh > static_cast<uint32_t>(kHighCap) || !(M > -INFINITY)) {
    __syncthreads();
    return false;
  }
  const float Rf = M * c + 1.f;  // as in the multi-pass select
  auto fmv = [&](float x) -> uint64_t { return to_fixed(fminf(exp2_hw(fmaf(x, c, -Rf)), 1.f)); };
  const int t = threadIdx.x;
  // exact masses of the high list; the rest approximately, with its bounds
  const uint64_t Hm = block_sum_u64(t < static_cast<int>(nh) ? fmv(key_value(wb.h.high[t])) : 0u);
  const uint64_t Zr = rest_fixed(wb, rest, loV, c, Rf);
  const double rlo = fmax(0.0, static_cast<double>(Zr) * (1.0 - kRestSlack) - static_cast<double>(V));
  const double rhi = static_cast<double>(Zr) * (1.0 + kRestSlack) + static_cast<double>(V);
  // bounds of a bin's entry masses: its edges, widened past the rounding of the bin
  // index and of the edges (a few units in the last place of mref, in bins) and of the
  // hardware exponential (relative 1e-6)
  const float slack = 1e-3f + fabsf(mref) * s * 4e-7f;
  auto bin_lo = [&](int j) -> uint64_t {
    const uint64_t f = fmv(mref - (static_cast<float>(j) + 1.f + slack) / s);
    return f > f / 1000000u + 1u ? f - f / 1000000u - 1u : 0u;
  };
  auto bin_hi = [&](int j) -> uint64_t {
    const uint64_t f = fmv(mref - (static_cast<float>(j) - slack) / s);
    return f + f / 1000000u + 1u;
  };
  // thread t holds bins 16t .. 16t + 15 (j grows as the value falls)
  constexpr int per = kMassBins / kFiltBlock;
  const int j0 = per * t;
  uint64_t tl = 0, tu = 0;
#pragma unroll 1
  for (int i = 0; i < per; ++i) {
    const uint64_t n = wb.h.cnt[j0 + i];
    if (n) {
      tl += n * bin_lo(j0 + i);
      tu += n * bin_hi(j0 + i);
    }
  }
  uint64_t Ltot, Utot;
  const uint64_t le = block_excl_u64(tl, Ltot);  // the bins above thread t's (threads before t)
  const uint64_t ue = block_excl_u64(tu, Utot);
  const double Plo = static_cast<double>(pp) * (static_cast<double>(Hm + Ltot) + rlo);
  const double Phi = static_cast<double>(pp) * (static_cast<double>(Hm + Utot) + rhi);
  // the band [ja, jb]: the cut's bin j* is the first whose mass from the top reaches
  // p * Z, so ja <= j* with ja the first bin whose upper bound reaches Plo, and j* <= jb
  // with jb the first bin whose lower bound reaches Phi; bin -1 is the high list
  int ja = kMassBins, jb = kMassBins;
  {
    uint64_t cu = Hm + ue, cl = Hm + le;
#pragma unroll 1
    for (int i = 0; i < per; ++i) {
      const uint64_t n = wb.h.cnt[j0 + i];
      if (n) {
        cu += n * bin_hi(j0 + i);
        cl += n * bin_lo(j0 + i);
      }
      if (ja == kMassBins && static_cast<double>(cu) >= Plo) ja = j0 + i;
      if (jb == kMassBins && static_cast<double>(cl) >= Phi) jb = j0 + i;
    }
  }
  ja = block_min_i32(wb.wmin, ja);
  jb = block_min_i32(wb.wmin, jb);
  if (static_cast<double>(Hm) >= Plo) ja = -1;  // the cut may lie in the high list
  if (static_cast<double>(Hm) >= Phi) jb = -1;  // it does
  if (jb >= kMassBins || ja > jb) {  // the cut may lie below the counted bins
    __syncthreads();
    return false;
  }
  uint64_t nbt = (t == 0 && ja < 0) ? nh : 0u;
#pragma unroll 1
  for (int i = 0; i < per; ++i)
    if (j0 + i >= ja && j0 + i <= jb) nbt += wb.h.cnt[j0 + i];
  const uint64_t nband = block_sum_u64(nbt);
  if (nband == 0 || nband > static_cast<uint64_t>(WideKey<float>::kCap)) {
    __syncthreads();
    return false;
  }
  __syncthreads();  // every count has been read: the buffer reuses their memory
  if (t == 0) wb.nbuf = 0;
  __syncthreads();
  // second read: exact masses, the band's entries as keys
  const float Xa = bin_floor_value(ja, mref, s);      // above the band: x > Xa
  const float Xb = bin_floor_value(jb + 1, mref, s);  // in the band: Xb < x <= Xa
  F32Sums sums;
  uint32_t nb = 0;
  if (!f32_band_read(row, V, wb, c, Rf, Xa, Xb, sums, nb)) {
    __syncthreads();
    return false;
  }
  const uint64_t Zt = block_sum_u64(sums.zt), A = block_sum_u64(sums.za), Zb = block_sum_u64(sums.zb);
  const uint64_t Na = block_sum_u64(sums.na);
  if (nb != nband) {  // uniform; the two reads see the same row, so this does not happen
    __syncthreads();
    return false;
  }
  uint32_t thr;
  uint64_t kn, km;
  const bool ok =
      wide_cut<float>(wb, static_cast<int>(nb), 0, false, pp, true, c, Rf, Zt - A - Zb, thr, kn, km, A, Na);
  if (ok) filt_write(P, r, Rf, static_cast<double>(km) * 0x1p-40, thr, kn, xl);
  __syncthreads();  // shared memory is reused by the next row
  return ok;
}

// The one-read path of a row with top-p on, or with top-k and k > 64: top-p alone on
// a long bf16 row goes through the key counts, every other row through the buffer.
// False (nothing written) when the row needs the multi-pass select.
template <typename T>
__device__ __forceinline__ bool filter_row_wide(const SampleParams& P, const FiltRow& r, WideBuf& wb, int kk,
                                                bool k_on, float pp, bool p_on, float xl) {
  if constexpr (sizeof(T) == 2) {
    if (!k_on && P.V > WideKey<T>::kCap) return hist16_row(P, r, wb, pp, xl);
  }
  if (buffer_row<T>(P, r, wb, kk, k_on, pp, p_on, xl)) return true;
  if constexpr (sizeof(T) == 4) {
    // a long fp32 row whose nucleus the buffer cannot hold: two reads
    if (!k_on && p_on && P.V > WideKey<T>::kCap) return f32_topp_row(P, r, wb, pp, xl);
  }
  return false;
}

// The multi-pass select of a row (any filter setting): a radix select over the
// whole row, one pass per digit.
template <typename T>
__device__ __forceinline__ void filter_row_task(const SampleParams& P, const FiltRow& r, FiltShared& sh, int kk, float pp, float xl) {
  const int64_t V = P.V;
  const T* row = static_cast<const T*>(r.row);
  const bool k_on = kk > 0 && kk < V;
  const bool p_on = pp < 1.f;  // false for NaN
  const float c = P.c;

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
    filt_write(P, r, 0.f, 0.0, 0xFFFFFFFFu, 0, xl);
    __syncthreads();
    return;
  }
  // masses 2^(x*c - Rf) against Rf = fl(M*c) + 1 stay <= 1 (the largest is about 1/2)
  const float R = M * c;
  const float Rf = R + 1.f;
  uint32_t thr = 0;
  uint64_t kept_n = static_cast<uint64_t>(V), kept_m = 0;
  bool fixed_mass = false;
  auto visit_all = [&](auto&& f) { visit_row(row, V, f); };
  cut_row<sizeof(T) == 2>(sh, visit_all, kk, pp, k_on, p_on, c, Rf, thr, kept_n, kept_m, fixed_mass);
  // without a filter the online sum serves, moved from reference R to Rf
  filt_write(P, r, Rf,
             fixed_mass ? static_cast<double>(kept_m) * 0x1p-40 : S * exp2(static_cast<double>(R) - static_cast<double>(Rf)),
             thr, kept_n, xl);
  __syncthreads();
}

// A row with no filter: its maximum and softmax denominator, one read.
template <typename T>
__device__ __forceinline__ void filter_row_plain(const SampleParams& P, const FiltRow& r, float xl) {
  const float c = P.c;
  Online o;
  o.init();
  visit_row(static_cast<const T*>(r.row), static_cast<int64_t>(P.V), [&](float x) {
    if (x > o.m) o.raise(x, c);
    o.add(x, c);
  });
  float M;
  double S;
  block_online<kFiltBlock>(o, c, M, S);  // valid in thread 0, the only writer
  if (threadIdx.x == 0) {
    if (!(M > -INFINITY)) {
      filt_write(P, r, 0.f, 0.0, 0xFFFFFFFFu, 0, xl);
    } else {
      const float R = M * c;
      const float Rf = R + 1.f;  // as in the multi-pass select
      filt_write(P, r, Rf, S * pow2d(static_cast<double>(R) - static_cast<double>(Rf)), 0u,
                 static_cast<uint64_t>(P.V), xl);
    }
  }
  __syncthreads();
}

// Shared memory of the row paths (a workgroup runs one at a time).
union FiltLds {
  FastBuf fast;
  WideBuf wide;
  FiltShared multi;  // the multi-pass select of a bf16 row the one-read paths leave
};

#ifndef SV_FILT_ROWS_GRID
#define SV_FILT_ROWS_GRID 512  // workgroups of the multi-pass kernel (fp32 rows)
#endif
#ifndef SV_FILT_MINB
#define SV_FILT_MINB 5  // workgroups per CU the one-read kernel is compiled for (its LDS allows five)
#endif

// One workgroup per logit row, read once: no filter, top-k with k <= 64, or top-p /
// larger top-k. A bf16 row these paths do not finish takes the multi-pass select in
// the same workgroup; an fp32 row is flagged (f_flag = 1) for k_filter_rows. Every
// row's flag is written.
// The grid is two-dimensional, one workgroup per row (no loop over rows: values
// derived from the thread index are not kept live across rows).
template <typename T>
__global__ __launch_bounds__(kFiltBlock, SV_FILT_MINB) void k_filter(SampleParams P) {
  touch_kernargs(P);
  __shared__ FiltLds lds;
  const int64_t ntask = static_cast<int64_t>(P.B) * (2 * P.K + 1);
  const int64_t task = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
  if (task < ntask) {
    const FiltRow r = filt_row(P, task, sizeof(T));
    const int kk = P.top_k ? P.top_k[r.b] : 0;
    const float pp = P.top_p ? P.top_p[r.b] : 1.f;
    const bool k_on = kk > 0 && kk < P.V;
    const bool p_on = pp < 1.f;  // false for NaN
    bool done = false;
    const float xl = filt_token_logit<T>(P, r);
    if (!P.filt_multi) {
      if (k_on && kk <= kFiltFastK) {
        done = filter_row_fast<T>(P, r, lds.fast, kk, pp, xl);
      } else if (k_on || p_on) {
        done = filter_row_wide<T>(P, r, lds.wide, kk, k_on, pp, p_on, xl);
      } else {
        filter_row_plain<T>(P, r, xl);
        done = true;
      }
    }
    if constexpr (sizeof(T) == 2) {
      // bf16 rows save the second launch; fp32 rows keep it (with this call inlined, the
      // fp32 kernel's one-read paths measured slower)
      if (!done) {
        __syncthreads();  // the one-read path's shared memory is reused
        filter_row_task<T>(P, r, lds.multi, kk, pp, xl);
        done = true;
      }
    }
    if (threadIdx.x == 0) P.f_flag[r.fr] = done ? 0u : 1u;
  }
}

// The multi-pass select of the flagged fp32 rows. Workgroup w takes rows w, w + G, ...;
// each batch of 256 of its rows reads their flags at once.
template <typename T>
__global__ __launch_bounds__(kFiltBlock) void k_filter_rows(SampleParams P) {
  touch_kernargs(P);
  __shared__ FiltShared sh;
  __shared__ uint64_t flagged[kFiltBlock / 64];
  const int64_t ntask = static_cast<int64_t>(P.B) * (2 * P.K + 1);
  const int64_t G = gridDim.x;
  for (int64_t base = blockIdx.x; base < ntask; base += G * kFiltBlock) {
    const int64_t mine = base + static_cast<int64_t>(threadIdx.x) * G;
    bool f = false;
    if (mine < ntask) {
      const FiltRow r = filt_row(P, mine, sizeof(T));
      f = P.f_flag[r.fr] != 0u;
    }
    const uint64_t bal = __ballot(f);
    if ((threadIdx.x & 63) == 0) flagged[threadIdx.x >> 6] = bal;
    __syncthreads();
    for (int wv = 0; wv < kFiltBlock / 64; ++wv) {
      for (uint64_t bits = flagged[wv]; bits != 0; bits &= bits - 1) {
        const int64_t task = base + static_cast<int64_t>(wv * 64 + __ffsll(static_cast<unsigned long long>(bits)) - 1) * G;
        const FiltRow r = filt_row(P, task, sizeof(T));
        const int kk = P.top_k ? P.top_k[r.b] : 0;
        const float pp = P.top_p ? P.top_p[r.b] : 1.f;
        filter_row_task<T>(P, r, sh, kk, pp, filt_token_logit<T>(P, r));
      }
    }
    __syncthreads();  // the flags of the next batch overwrite these
  }
}

static dim3 filt_grid(int64_t tasks, int64_t cap) { return dim3(static_cast<uint32_t>(tasks < cap ? tasks : cap)); }

// One workgroup per row: x up to 2^16, y the rest.
static dim3 filt_grid_2d(int64_t tasks) {
  const int64_t x = tasks < 65536 ? tasks : 65536;
  return dim3(static_cast<uint32_t>(x), static_cast<uint32_t>((tasks + x - 1) / x));
}

hipError_t launch_filter_rows(const SampleParams& P, bool bf16, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(P.B) * (2 * P.K + 1);
  // the multi-pass kernel of fp32 rows: every row when the one-read paths are off,
  // else a few workgroups, since flagged rows are rare
  const int64_t g2 = P.filt_multi ? rows : (SV_FILT_ROWS_GRID);
  if (bf16) {
    hipLaunchKernelGGL(k_filter<bf16_t>, filt_grid_2d(rows), dim3(kFiltBlock), 0, stream, P);
  } else {
    hipLaunchKernelGGL(k_filter<float>, filt_grid_2d(rows), dim3(kFiltBlock), 0, stream, P);
    hipLaunchKernelGGL(k_filter_rows<float>, filt_grid(rows, g2), dim3(kFiltBlock), 0, stream, P);
  }
  return hipGetLastError();
}

}  // namespace sv
