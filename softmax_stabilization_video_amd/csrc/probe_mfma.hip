// probe_mfma.hip -- the bf16 matrix-core rate this GPU sustains.
//
// A loop of independent v_mfma_f32_32x32x16_bf16 (the instruction of the
// attention kernels) with no memory traffic, on every SIMD.  Its rate is the
// practical ceiling of those kernels under the same clock and power limits,
// reported beside the published peak.  Built as its own library
// (libclis_probe.so), used only for measurement; not part of the attention
// path.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kChains = 4;  // independent accumulators per wave

__global__ void __launch_bounds__(kThreads) mfma_loop(float* __restrict__ out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(threadIdx.x + i));
    b[i] = (__bf16)(0.002f * (float)(i + 1));
  }
  floatx16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
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
// MFMAs (32x32x16 bf16, 32768 FLOP each) on `stream` (a hipStream_t as void*).
// `out` is a device buffer of blocks * 256 floats.  Returns 0, or a HIP error
// code (nothing enqueued for bad arguments).
int clis_probe_mfma(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  mfma_loop<<<blocks, kThreads, 0, static_cast<hipStream_t>(stream)>>>(out, iters);
  return (int)hipGetLastError();
}

// FLOPs one clis_probe_mfma call performs.
double clis_probe_mfma_flops(int blocks, int iters) {
  return (double)blocks * (kThreads / 64) * (double)iters * kChains * 32768.0;
}

}  // extern "C"
