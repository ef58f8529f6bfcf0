// attn_fp32.hip -- fp32 attention forward for fp32 inputs, where the result
// must stay within fp32 accuracy of softmax attention.  bf16 MFMA would round
// the operands, so this path runs fp32 FMAs on the VALU; it serves small fp32
// problems, not the throughput workloads.  The softmax forms are those of the
// bf16 kernel ("CLiS: Plug-and-Play Attention Acceleration for Video
// Diffusion on TPUs via Certified Stabilization", abstract and Figure 5(a)):
// fixed stabilizer (with its key-shard form, o_acc / l_acc), online softmax,
// and online softmax with lazy rescaling; each can also write the row
// log-sum-exp.
//
// One workgroup = 64 threads = 64 query rows of one head; each thread owns a
// row (its output accumulator in registers, its query row in LDS).  Key and
// value tiles of 32 rows are staged in LDS and read as broadcasts.
#include <hip/hip_runtime.h>
#include <math.h>

#include "internal.h"

namespace clis {
namespace {

constexpr int kRows = 64;
constexpr int kTile = 32;

template <int D, bool FIXED, bool CAUSAL, bool LAZY>
__global__ void __launch_bounds__(kRows)
attn_fwd_fp32(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
              float* __restrict__ O, const float* __restrict__ mu, const int32_t* __restrict__ head_list,
              const int32_t* __restrict__ head_count, int Nq, int Nk, float c2, float* __restrict__ lse,
              float* __restrict__ o_acc, float* __restrict__ l_acc, int accumulate, int kv_offset) {
  __shared__ float Qs[kRows][D + 1];
  __shared__ float Ks[kTile][D];
  __shared__ float Vs[kTile][D];
  const int n_qt = (Nq + kRows - 1) / kRows;
  const int slot = blockIdx.x / n_qt;
  const int qt = blockIdx.x % n_qt;
  int bh = slot;
  if (head_list) {
    if (slot >= *head_count) return;
    bh = head_list[slot];
  }
  const int t = threadIdx.x;
  const int qrow = qt * kRows + t;
  const bool qvalid = qrow < Nq;
  const float* Qh = Q + (size_t)bh * Nq * D;
  const float* Kh = K + (size_t)bh * Nk * D;
  const float* Vh = V + (size_t)bh * Nk * D;

  for (int i = t; i < kRows * D; i += kRows) {
    const int r = i / D, c = i % D, qr = qt * kRows + r;
    Qs[r][c] = (qr < Nq) ? Qh[(size_t)qr * D + c] : 0.f;
  }

  float o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) o[c] = 0.f;
  float m = FIXED ? (qvalid ? mu[(size_t)bh * Nq + qrow] : 0.f) : -INFINITY;
  float l = 0.f;
  if (FIXED && o_acc && accumulate && qvalid) {  // continue the sums of earlier key shards
    const float* arow = o_acc + ((size_t)bh * Nq + qrow) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] = arow[c];
    l = l_acc[(size_t)bh * Nq + qrow];
  }

  // local keys this block needs (the causal mask compares global indices)
  const int kv_end = CAUSAL ? max(0, min(Nk, (qt + 1) * kRows - kv_offset)) : Nk;
  for (int kt = 0; kt < kv_end; kt += kTile) {
    __syncthreads();
    for (int i = t; i < kTile * D; i += kRows) {
      const int r = i / D, c = i % D, key = kt + r;
      Ks[r][c] = (key < Nk) ? Kh[(size_t)key * D + c] : 0.f;
      Vs[r][c] = (key < Nk) ? Vh[(size_t)key * D + c] : 0.f;
    }
    __syncthreads();
    float x[kTile];
#pragma unroll 4
    for (int j = 0; j < kTile; ++j) {
      float s = 0.f;
#pragma unroll 16
      for (int c = 0; c < D; ++c) s = fmaf(Qs[t][c], Ks[j][c], s);
      const int key = kt + j;
      const bool ok = key < Nk && (!CAUSAL || kv_offset + key <= qrow);
      x[j] = ok ? (FIXED ? fmaf(s, c2, -m) : s * c2) : -INFINITY;
    }
    if constexpr (LAZY) {
      // conditional rescaling: the stabilizer moves only when the tile
      // maximum exceeds it by more than 8 (log2 units); weights stay <= 256
      float tmax = -INFINITY;
      for (int j = 0; j < kTile; ++j) tmax = fmaxf(tmax, x[j]);
      if (tmax > m + 8.f) {
        const float alpha = __builtin_amdgcn_exp2f(m - tmax);  // 0 while m = -inf
        l *= alpha;
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] *= alpha;
        m = tmax;
      }
      const float msub = (m == -INFINITY) ? 0.f : m;
      for (int j = 0; j < kTile; ++j) x[j] -= msub;
    } else if constexpr (!FIXED) {
      float tmax = -INFINITY;
      for (int j = 0; j < kTile; ++j) tmax = fmaxf(tmax, x[j]);
      const float mnew = fmaxf(m, tmax);
      const bool none = (mnew == -INFINITY);
      const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m - mnew);
      const float msub = none ? 0.f : mnew;
      l *= alpha;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] *= alpha;
      for (int j = 0; j < kTile; ++j) x[j] -= msub;
      m = mnew;
    }
    for (int j = 0; j < kTile; ++j) {
      const float p = __builtin_amdgcn_exp2f(x[j]);
      l += p;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = fmaf(p, Vs[j][c], o[c]);
    }
  }
  if (FIXED && o_acc) {  // key shard: the unnormalized sums
    if (qvalid) {
      float* arow = o_acc + ((size_t)bh * Nq + qrow) * D;
#pragma unroll
      for (int c = 0; c < D; ++c) arow[c] = o[c];
      l_acc[(size_t)bh * Nq + qrow] = l;
    }
    return;
  }
  if (qvalid) {
    const float inv = 1.f / l;
    if (lse) lse[(size_t)bh * Nq + qrow] = 0.693147180559945309f * (m + log2f(l));
    float* orow = O + ((size_t)bh * Nq + qrow) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) orow[c] = o[c] * inv;
  }
}

template <int D, bool FIXED, bool CAUSAL, bool LAZY = false>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  const int n_qt = (a.Nq + kRows - 1) / kRows;
  const long long blocks = (long long)n_qt * a.n_slots;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  attn_fwd_fp32<D, FIXED, CAUSAL, LAZY><<<(unsigned)blocks, kRows, 0, s>>>(
      static_cast<const float*>(a.q), static_cast<const float*>(a.k), static_cast<const float*>(a.v),
      static_cast<float*>(a.o), a.mu, a.head_list, a.head_count, a.Nq, a.Nk, a.c2, a.lse, a.o_acc, a.l_acc,
      a.accumulate, a.kv_offset);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, bool fixed, hipStream_t s) {
  if (fixed) return a.causal ? launch_t<D, true, true>(a, s) : launch_t<D, true, false>(a, s);
  if (a.lazy) return a.causal ? launch_t<D, false, true, true>(a, s) : launch_t<D, false, false, true>(a, s);
  return a.causal ? launch_t<D, false, true>(a, s) : launch_t<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_attn_fp32(const AttnArgs& a, bool fixed, hipStream_t s) {
  if (a.d == 128) return launch_d<128>(a, fixed, s);
  if (a.d == 64) return launch_d<64>(a, fixed, s);
  return hipErrorInvalidValue;
}

}  // namespace clis
