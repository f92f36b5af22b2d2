// One key's bucket of the n-gram pools (the direct table and the hashed one), rebuilt
// by one wave from the n-grams of an insert call (gfx950).
//
// Source: "Lookahead Decoding 完全拆解:Jacobi 迭代与 N-gram 池", sections "Lookahead
// 分支" and "N-gram 池与身份判定". A key keeps its G most recently inserted distinct
// continuations, newest first; a continuation inserted again becomes the newest.
#pragma once

#include "../../include/spec_verify.h"
#include "common.hpp"

namespace sv {

// Do n-grams w1 and w2 of the staged call (ng, [W][N] int32) carry the same continuation?
__device__ __forceinline__ bool same_cont(const int32_t* ng, int N, int w1, int w2) {
  for (int i = 1; i < N; ++i)
    if (ng[w1 * N + i] != ng[w2 * N + i]) return false;
  return true;
}

// Rebuild the bucket at bk (G slots of N-1 int32, newest first, compacted, an empty slot
// -1 throughout). `same` marks the call's n-grams of the key (bit w: n-gram w of ng); they
// enter at their last occurrence, the newest (highest w) first, followed, when keep_old,
// by the bucket's old slots that none of them repeats, in their order; the result is cut
// to G. This equals inserting those n-grams one by one in window order. With keep_old
// false the old slots are not read (the bucket belongs to a key new to it).
// Called by a whole wave with `same` and keep_old uniform; lane g handles slot g and
// n-gram g of the call.
__device__ __forceinline__ void rebuild_bucket(const int32_t* ng, int N, int G, int lane, uint64_t same, int32_t* bk,
                                               bool keep_old) {
  // the old slot `lane` (lanes < G), loaded before the continuations are compared
  int32_t old[SPEC_MAX_POOL_N - 1];
  bool held = false;
  if (keep_old && lane < G) {
#pragma unroll
    for (int i = 0; i < SPEC_MAX_POOL_N - 1; ++i) old[i] = (i < N - 1) ? bk[lane * (N - 1) + i] : -1;
    held = old[0] >= 0;
  }
  // the key's n-grams of this call at their last occurrence, newest (highest w) first
  bool fresh = false;
  if ((same >> lane) & 1ull) {
    fresh = true;
    for (uint64_t later = same >> lane >> 1; later != 0ull; later &= later - 1ull) {
      const int w2 = lane + 1 + __ffsll(static_cast<unsigned long long>(later)) - 1;
      if (same_cont(ng, N, lane, w2)) {
        fresh = false;
        break;
      }
    }
  }
  const uint64_t freshm = __ballot(fresh);
  const int nfresh = __popcll(freshm);
  // rank among the fresh ones: the fresh n-grams after this one come first
  const int rank = __popcll(freshm >> lane) - 1;
  // the old slot `lane` is kept when no fresh continuation repeats it
  bool keep = held;
  for (uint64_t f = freshm; f != 0ull && keep; f &= f - 1ull) {
    const int w2 = __ffsll(static_cast<unsigned long long>(f)) - 1;
    bool eq = true;
#pragma unroll
    for (int i = 0; i < SPEC_MAX_POOL_N - 1; ++i)
      if (i < N - 1) eq = eq && ng[w2 * N + i + 1] == old[i];
    keep = !eq;
  }
  const uint64_t keepm = __ballot(keep);
  const int okeep = __popcll(keepm & ((1ull << lane) - 1));  // kept old slots before this one
  const int total = min(nfresh + __popcll(keepm), G);
  // every old slot is read above, before any slot is written (the wave runs in lockstep)
  __builtin_amdgcn_wave_barrier();
  if (fresh && rank < G)
    for (int i = 1; i < N; ++i) bk[rank * (N - 1) + (i - 1)] = ng[lane * N + i];
  if (keep && nfresh + okeep < G) {
#pragma unroll
    for (int i = 0; i < SPEC_MAX_POOL_N - 1; ++i)
      if (i < N - 1) bk[(nfresh + okeep) * (N - 1) + i] = old[i];
  }
  if (lane >= total && lane < G)
    for (int i = 0; i < N - 1; ++i) bk[lane * (N - 1) + i] = -1;
}

}  // namespace sv
