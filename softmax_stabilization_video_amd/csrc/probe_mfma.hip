// probe_mfma.hip -- the bf16 matrix-core rate this GPU sustains.
//
// A loop of independent v_mfma_f32_32x32x16_bf16 (the instruction of the
// attention kernels) with no memory traffic, on every SIMD, in two forms:
//  - constant operands (small values, the same for every MFMA): the rate at
//    the highest clock the chip reaches, close to the published peak;
//  - random operands (bf16 values of a hashed counter, about unit scale, a
//    different register set for each of the four accumulator chains, so every
//    MFMA reads other data than the one before): the chip is power-limited,
//    and switching data lowers the clock it holds; this rate is the ceiling
//    an attention kernel, whose operands change at every MFMA, can reach.
// Built as its own library (libclis_probe.so), used only for measurement; not
// part of the attention path.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kChains = 4;  // independent accumulators per wave

// A 32-bit integer hash (two multiply-xorshift rounds).
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// A value of about unit scale from a counter: the sum of the hash's four
// bytes, centred.
__device__ __forceinline__ float hashed_value(uint32_t key) {
  const uint32_t h = mix32(key);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += (float)((h >> (8 * i)) & 255u) * (1.f / 255.f) - 0.5f;
  return 1.7f * s;
}

template <bool RANDOM>
__global__ void __launch_bounds__(kThreads) mfma_loop(float* __restrict__ out, int iters) {
  bf16x8 a[kChains], b[kChains];
  const uint32_t lane = blockIdx.x * kThreads + threadIdx.x;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (RANDOM) {
        a[c][i] = (__bf16)hashed_value(lane * 64u + 8u * c + i);
        b[c][i] = (__bf16)hashed_value(0x9e3779b9u ^ (lane * 64u + 8u * c + i));
      } else {
        a[c][i] = (__bf16)(0.001f * (float)(threadIdx.x + i));
        b[c][i] = (__bf16)(0.002f * (float)(i + 1));
      }
    }
  floatx16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[c], acc[c], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;  // keeps the loop live
}

}  // namespace

extern "C" {

// Enqueues `blocks` workgroups of 256 threads, each wave running `iters` x 4
// MFMAs (32x32x16 bf16, 32768 FLOP each) on `stream` (a hipStream_t as void*),
// with constant operands (random == 0) or random ones (random != 0).  `out` is
// a device buffer of blocks * 256 floats.  Returns 0, or a HIP error code
// (nothing enqueued for bad arguments).
int clis_probe_mfma(float* out, int blocks, int iters, int random, void* stream) {
  if (!out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (random)
    mfma_loop<true><<<blocks, kThreads, 0, s>>>(out, iters);
  else
    mfma_loop<false><<<blocks, kThreads, 0, s>>>(out, iters);
  return (int)hipGetLastError();
}

// FLOPs one clis_probe_mfma call performs.
double clis_probe_mfma_flops(int blocks, int iters) {
  return (double)blocks * (kThreads / 64) * (double)iters * kChains * 32768.0;
}

}  // extern "C"
