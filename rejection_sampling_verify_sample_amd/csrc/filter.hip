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
//
// With top-k on and k <= 64 the row is read once instead (k_filter_fast): every
// thread publishes its running maximum in LDS, and the k-th largest of those 256
// maxima (each the maximum of a disjoint part of the row) is a lower bound of the
// row's k-th largest logit. Entries at or above the bound (every entry top-k
// keeps, plus a few hundred others) go to an LDS buffer. One wave then finds the
// k-th largest key by a bitwise search and sorts the kept keys, and the top-p
// group comes from an exact scan of the same fixed-point masses, so the results
// are those of the multi-pass select. A row whose candidates overflow the buffer
// (many entries tied at the top), and every other filtered row, take the
// multi-pass select (k_filter_rows, which skips the rows finished before it).
#include "common.hpp"
#include "params.hpp"

namespace sv {

constexpr int kFiltBlock = 256;
constexpr int kFiltUnroll = 2;
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
__device__ __forceinline__ uint32_t reserve_slots(FastBuf& fb, uint32_t cnt) {
  const int lane = threadIdx.x & 63;
  const uint32_t incl = wave_scan_add_u32(cnt);
  uint32_t base = 0;
  if (lane == 63 && incl) base = atomicAdd(&fb.nbuf, incl);
  base = __builtin_amdgcn_readlane(base, 63);
  return base + incl - cnt;
}

// Append the lane's values whose bit is set in `take` (bit i for x[i]).
template <int N>
__device__ __forceinline__ void append_masked(FastBuf& fb, const float (&x)[N], uint32_t take) {
  uint32_t pos = reserve_slots(fb, static_cast<uint32_t>(__popc(take)));
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
      uint32_t pos = reserve_slots(fb, cnt);
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

// Smallest value over the block (thread 0's argument order is irrelevant).
__device__ __forceinline__ int32_t block_min_i32(FastBuf& fb, int32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) fb.wmin[threadIdx.x >> 6] = v;
  __syncthreads();
  int32_t r = fb.wmin[0];
#pragma unroll
  for (int o = 1; o < kFiltBlock / 64; ++o) r = min(r, fb.wmin[o]);
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

// Top-k with a small k reads the row once.
__device__ __forceinline__ bool fast_eligible(const SampleParams& P, int b) {
  const int kk = P.top_k ? P.top_k[b] : 0;
  return kk > 0 && kk < P.V && kk <= kFiltFastK;
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
    const uint32_t tp = fb.key[min(block_min_i32(fb, first), npad - 1)];
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

// One-pass path of a row: the candidates, then the cut. The candidate count goes to
// f_cnt, so that k_filter_rows skips the rows finished here.
template <typename T>
__device__ void filter_row_fast(const SampleParams& P, int64_t task, FastBuf& fb) {
  const FiltRow r = filt_row(P, task, sizeof(T));
  if (!fast_eligible(P, r.b)) return;
  const int kk = P.top_k[r.b];
  const float pp = P.top_p ? P.top_p[r.b] : 1.f;
  const float xl = filt_token_logit<T>(P, r);
  float M;
  uint32_t lbound;
  const uint32_t n = collect_candidates(static_cast<const T*>(r.row), P.V, kk, fb, M, lbound);
  if (threadIdx.x == 0) P.f_cnt[r.fr] = n;
  if (n > static_cast<uint32_t>(kFiltCap)) {
    __syncthreads();  // the buffer is reused by the next row
    return;
  }
  cut_candidates<T>(P, r, fb, static_cast<int>(n), M, kk, pp, xl, lbound);
}

// The multi-pass select of a row the one-pass path does not finish (no small top-k,
// or a half whose candidates overflowed).
template <typename T>
__device__ void filter_row_task(const SampleParams& P, int64_t task, FiltShared& sh) {
  const FiltRow r = filt_row(P, task, sizeof(T));
  if (fast_eligible(P, r.b) && P.f_cnt[r.fr] <= static_cast<uint32_t>(kFiltCap)) return;
  const int64_t V = P.V;
  const T* row = static_cast<const T*>(r.row);
  const int kk = P.top_k ? P.top_k[r.b] : 0;
  const float pp = P.top_p ? P.top_p[r.b] : 1.f;
  const bool k_on = kk > 0 && kk < V;
  const bool p_on = pp < 1.f;  // false for NaN
  const float c = P.c;
  const float xl = filt_token_logit<T>(P, r);

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

template <typename T>
__global__ __launch_bounds__(kFiltBlock, SV_FAST_MINB) void k_filter_fast(SampleParams P) {
  touch_kernargs(P);
  __shared__ FastBuf fb;
  const int64_t ntask = static_cast<int64_t>(P.B) * (2 * P.K + 1);
  for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) filter_row_fast<T>(P, task, fb);
}

template <typename T>
__global__ __launch_bounds__(kFiltBlock) void k_filter_rows(SampleParams P) {
  touch_kernargs(P);
  __shared__ FiltShared sh;
  const int64_t ntask = static_cast<int64_t>(P.B) * (2 * P.K + 1);
  for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) filter_row_task<T>(P, task, sh);
}

static dim3 filt_grid(int64_t tasks) { return dim3(static_cast<uint32_t>(tasks < (1 << 20) ? tasks : (1 << 20))); }

hipError_t launch_filter_rows(const SampleParams& P, bool bf16, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(P.B) * (2 * P.K + 1);
  if (bf16) {
    hipLaunchKernelGGL(k_filter_fast<bf16_t>, filt_grid(rows), dim3(kFiltBlock), 0, stream, P);
    hipLaunchKernelGGL(k_filter_rows<bf16_t>, filt_grid(rows), dim3(kFiltBlock), 0, stream, P);
  } else {
    hipLaunchKernelGGL(k_filter_fast<float>, filt_grid(rows), dim3(kFiltBlock), 0, stream, P);
    hipLaunchKernelGGL(k_filter_rows<float>, filt_grid(rows), dim3(kFiltBlock), 0, stream, P);
  }
  return hipGetLastError();
}

}  // namespace sv
