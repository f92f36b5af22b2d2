// Verify uniforms from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64 products on a
// 128-bit counter, the 64-bit key bumped by two Weyl constants between rounds.
// One thread per (b, i); counter (i, b, round lo, round hi), key (seed lo, seed hi);
// words 0 and 1 become the accept uniform r and the draw uniform u as
// (w >> 8) * 2^-24, exact in fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

__global__ __launch_bounds__(256) void k_philox_uniforms(uint32_t k0, uint32_t k1, uint32_t r0, uint32_t r1,
                                                          int32_t B, int32_t Kp1, float* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(B) * Kp1) return;
  const uint32_t b = static_cast<uint32_t>(idx / Kp1);
  const uint32_t i = static_cast<uint32_t>(idx % Kp1);
  uint32_t c0 = i, c1 = b, c2 = r0, c3 = r1;
  uint32_t key0 = k0, key1 = k1;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round) {
      key0 += 0x9E3779B9u;
      key1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
    c0 = hi1 ^ c1 ^ key0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ key1;
    c3 = lo0;
  }
  constexpr float kScale = 1.0f / 16777216.0f;  // 2^-24
  out[idx * 2] = static_cast<float>(c0 >> 8) * kScale;
  out[idx * 2 + 1] = static_cast<float>(c1 >> 8) * kScale;
}

hipError_t launch_philox(uint64_t seed, uint64_t round, int32_t B, int32_t K, float* out, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(B) * (K + 1);
  const uint32_t blocks = static_cast<uint32_t>((n + 255) / 256);
  hipLaunchKernelGGL(k_philox_uniforms, dim3(blocks), dim3(256), 0, stream, static_cast<uint32_t>(seed),
                     static_cast<uint32_t>(seed >> 32), static_cast<uint32_t>(round),
                     static_cast<uint32_t>(round >> 32), B, K + 1, out);
  return hipGetLastError();
}

}  // namespace sv
