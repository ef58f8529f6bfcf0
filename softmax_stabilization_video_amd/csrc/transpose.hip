// transpose.hip -- the V^T copy that the bf16 attention kernels read their
// P.V operands from (layout: see the V^T paragraph of attn_bf16.hip).
//
// V [BH][Nk][D] -> V^T tiles [BH][Nk_pad / 64][D][kVtRow] bf16, Nk_pad =
// vt_pad(Nk): row c of tile t holds channel c of keys 64t .. 64t + 63, zeros
// past the last key, then 8 zeros of padding (the kernels' LDS row stride, so
// a tile loads into LDS as one contiguous copy).  Within every 16-key group
// the keys are stored in the order {0-3, 8-11, 4-7, 12-15} (vt_pos): a lane's
// P.V operand, keys 4g..4g+3 and 8+4g..8+4g+3 of a 16-key step (g = lane /
// 32), is then contiguous.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace clis {
namespace {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

constexpr int kTK = 64;  // keys per block (also the max |V| block)

// Position of key k within its 16-key group in V^T: swap bits 2 and 3.
__device__ __forceinline__ int vt_pos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// One block transposes keys blk*64 .. blk*64+63 of head bh (block index
// bh * nblk + blk, a 1-D grid so the head count is not bound by a grid
// dimension) through LDS: coalesced 16-byte reads along channels, coalesced
// 16-byte writes along keys.  With vmax_blk set it also writes the block's
// max |V| (NaN kept) to vmax_blk[bh * nblk + blk], so certification need not
// read V again.
template <int D>
__global__ void __launch_bounds__(256)
transpose_v(const uint16_t* __restrict__ V, uint16_t* __restrict__ Vt, int Nk, int nblk,
            float* __restrict__ vmax_blk) {
  __shared__ uint16_t t[D][kTK + 2];  // [channel][key position]; +2 breaks bank strides
  const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk, kt = blk * kTK;
  const uint16_t* src = V + (size_t)bh * Nk * D;
  uint16_t* dst = Vt + (size_t)blockIdx.x * D * kVtRow;  // tile blk of head bh
  constexpr int CPR = D / 8;
  float vmax = 0.f;
  for (int i = threadIdx.x; i < kTK * CPR; i += 256) {
    const int r = i / CPR, ch = i % CPR, key = kt + r;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (key < Nk)  // V is read once here: a nontemporal (streaming) load
      u = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(src + (size_t)key * D + ch * 8)));
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    if (vmax_blk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float((w[e] & 0x7fffu) << 16), hi = __uint_as_float(w[e] & 0x7fff0000u);
        vmax = (lo > vmax || lo != lo) ? lo : vmax;
        vmax = (hi > vmax || hi != hi) ? hi : vmax;
      }
    }
    const int pos = vt_pos(r);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t[ch * 8 + 2 * e][pos] = (uint16_t)(w[e] & 0xffffu);
      t[ch * 8 + 2 * e + 1][pos] = (uint16_t)(w[e] >> 16);
    }
  }
  if (vmax_blk) {  // the block's max |V|: waves, then the four wave results
    __shared__ float red[4];
    for (int off = 32; off > 0; off >>= 1) {
      const float o = __shfl_xor(vmax, off);
      vmax = (o > vmax || o != o) ? o : vmax;
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = vmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      float m = red[0];
      for (int i = 1; i < 4; ++i) m = (red[i] > m || red[i] != red[i]) ? red[i] : m;
      vmax_blk[(size_t)bh * nblk + blk] = m;
    }
  }
  __syncthreads();
  constexpr int QPR = kVtRow / 8;  // 16-byte pieces per tile row, the last one padding
  static_assert(kVtRow == kTK + 8, "a V^T tile row: the block's keys and one 16-byte pad");
  for (int i = threadIdx.x; i < D * QPR; i += 256) {
    const int c = i / QPR, q = i % QPR;
    uint32_t w[4] = {0, 0, 0, 0};
    if (q < kTK / 8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (uint32_t)t[c][q * 8 + 2 * e] | ((uint32_t)t[c][q * 8 + 2 * e + 1] << 16);
    }
    *reinterpret_cast<uint4*>(dst + i * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

hipError_t launch_transpose_v(const void* v, void* vt, int BH, int Nk, int d, hipStream_t s, float* vmax_blk) {
  const int nblk = vt_pad(Nk) / kTK;
  const long long blocks = (long long)BH * nblk;
  if (blocks <= 0 || blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const uint16_t* src = static_cast<const uint16_t*>(v);
  uint16_t* dst = static_cast<uint16_t*>(vt);
  if (d == 128) transpose_v<128><<<(unsigned)blocks, 256, 0, s>>>(src, dst, Nk, nblk, vmax_blk);
  else if (d == 64) transpose_v<64><<<(unsigned)blocks, 256, 0, s>>>(src, dst, Nk, nblk, vmax_blk);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace clis
