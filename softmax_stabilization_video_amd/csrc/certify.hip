// certify.hip -- per-head certification pre-pass for CLiS attention on gfx950.
//
// Implements Algorithm 1 of "CLiS: Plug-and-Play Attention Acceleration for
// Video Diffusion on TPUs via Certified Stabilization" (steps 1-7) plus the
// fixed per-row stabilizer.  The pass is HBM-bound (it reads K twice and Q
// and V once), so its arithmetic is fp64: cheap here, and it keeps the flag
// decision B_h <= C in the same precision as an fp64 reference.
//
// Kernels, in stream order:
//   1. cert_keys_values: per (head, key split) partial column sums of K and
//      partial max |V|                                   (steps 1 and 5)
//   2. cert_kbar: kbar = (sum of partials in split order) / Nk      (step 1)
//      (when the bf16 attention path has already transposed V, that pass
//      wrote max |V| per 64-key block; cert_keys_values then skips V and
//      cert_kbar folds the block maxima into the first split's partial)
//   3. cert_norms: key splits -> partial max ||k - kbar||^2 (steps 2-3);
//      query splits -> partial max ||q||^2 and mu_r = c (q_r . kbar)
//   4. cert_finalize: kappa, B_h, G, A, C, flag per head         (steps 3-7)
// With one key split and one query split (short sequences) cert_small runs
// the four passes for a head in one block: one launch instead of four.
// Every reduction has a fixed order (no atomics), so results are bitwise
// reproducible.  Maxima propagate NaN so that a NaN input never certifies.
#include <hip/hip_runtime.h>
#include <math.h>

#include "internal.h"

namespace clis {
namespace {

constexpr int kThreads = 256;

// max that keeps NaN once seen (fmax would drop it).
__device__ __forceinline__ double max_keep_nan(double acc, double x) {
  return (x > acc || x != x) ? x : acc;
}

// Elements per 16-byte vector load.
template <typename T> struct Vec;
template <> struct Vec<uint16_t> { static constexpr int n = 8; };
template <> struct Vec<float> { static constexpr int n = 4; };

// 16 bytes of a row that this pass reads once: a nontemporal load (the
// streaming hint keeps the single-use rows from displacing cached data;
// measured 7-9% faster certification on the long workloads).
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 stream_load16(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(static_cast<const u32x4v*>(p)));
}

// Rows in flight per lane in the streaming loops (loads issued before use):
// enough that a CU keeps 64 KB or more of reads outstanding.
constexpr int kUnroll = 8;

// 16 bytes of row elements, widened to fp64.
template <typename T>
__device__ __forceinline__ void widen(const uint4 u, double* out) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = (double)__uint_as_float(w[i] << 16);
      out[2 * i + 1] = (double)__uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    out[0] = (double)__uint_as_float(u.x);
    out[1] = (double)__uint_as_float(u.y);
    out[2] = (double)__uint_as_float(u.z);
    out[3] = (double)__uint_as_float(u.w);
  }
}

__device__ __forceinline__ void split_range(int n, int splits, int s, int* lo, int* hi) {
  const long long per = ((long long)n + splits - 1) / splits;
  long long a = per * s, b = a + per;
  if (a > n) a = n;
  if (b > n) b = n;
  *lo = (int)a;
  *hi = (int)b;
}

// Block-wide NaN-keeping max over NTH threads; every thread gets the result.
template <int NTH = kThreads>
__device__ double block_max(double x, double* red) {
  for (int off = 32; off > 0; off >>= 1) x = max_keep_nan(x, __shfl_xor(x, off));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  double r = red[0];
  for (int i = 1; i < NTH / 64; ++i) r = max_keep_nan(r, red[i]);
  return r;
}

// Step 1 (partial column sums of K) and step 5 (partial max |V|).
// (one block of NTH threads: head bh, key split `split`)
template <typename T, int D, bool WITH_V, int NTH = kThreads>
__device__ __forceinline__ void keys_values_block(const T* __restrict__ K, const T* __restrict__ V, int Nk, int Sk,
                                                  double* out, double* vmax_out, int bh, int split) {
  constexpr int VEC = Vec<T>::n, TPR = D / VEC, RPI = NTH / TPR;
  __shared__ double colsum[RPI][D];
  __shared__ double red[NTH / 64];
  int lo, hi;
  split_range(Nk, Sk, split, &lo, &hi);
  const int tr = threadIdx.x / TPR, tc = threadIdx.x % TPR;
  const T* kb = K + (size_t)bh * Nk * D;
  const T* vb = WITH_V ? V + (size_t)bh * Nk * D : nullptr;  // without: max |V| comes from the transpose
  double acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
  double vmax = 0.0;
  // UN rows per lane in flight; the sums still run in row order
  constexpr int UN = WITH_V ? kUnroll / 2 : kUnroll;
  for (int j0 = lo + tr; j0 < hi; j0 += UN * RPI) {
    uint4 uk[UN], uv[WITH_V ? UN : 1];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * RPI;
      uk[u] = make_uint4(0, 0, 0, 0);
      if constexpr (WITH_V) uv[u] = make_uint4(0, 0, 0, 0);
      if (j < hi) {
        uk[u] = stream_load16(kb + (size_t)j * D + tc * VEC);
        if constexpr (WITH_V) uv[u] = stream_load16(vb + (size_t)j * D + tc * VEC);
      }
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      if (j0 + u * RPI >= hi) break;
      double x[VEC];
      widen<T>(uk[u], x);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += x[e];
      if constexpr (WITH_V) {
        widen<T>(uv[u], x);
#pragma unroll
        for (int e = 0; e < VEC; ++e) vmax = max_keep_nan(vmax, fabs(x[e]));
      }
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) colsum[tr][tc * VEC + e] = acc[e];
  vmax = block_max<NTH>(vmax, red);  // contains __syncthreads
  for (int c = threadIdx.x; c < D; c += NTH) {
    double s = 0.0;
    for (int r = 0; r < RPI; ++r) s += colsum[r][c];  // fixed row-group order
    out[c] = s;
  }
  if (threadIdx.x == 0) *vmax_out = vmax;
}

template <typename T, int D, bool WITH_V>
__global__ void __launch_bounds__(kThreads)
cert_keys_values(const T* __restrict__ K, const T* __restrict__ V, int Nk, int Sk,
                 double* __restrict__ ksum_part, double* __restrict__ vmax_part) {
  // 1-D grid: any head count
  keys_values_block<T, D, WITH_V>(K, V, Nk, Sk, ksum_part + (size_t)blockIdx.x * D, vmax_part + blockIdx.x,
                                  blockIdx.x / Sk, blockIdx.x % Sk);
}

// Step 1: kbar from the split partials, summed in split order (threads c <
// D of the block; every thread reaches the barrier).  The head's partial sums
// `sums` ([Sk][D]) -> kbar ([D], and kbar_copy if set); with vmax_blk (the
// head's nblk block maxima of |V|) their maximum goes to *vmax_out (split 0's
// partial).
template <int D>
__device__ __forceinline__ void kbar_block_impl(const double* sums, int Nk, int Sk, double* __restrict__ kbar,
                                                double* kbar_copy, const float* __restrict__ vmax_blk, int nblk,
                                                double* vmax_out, double* red) {
  const int c = threadIdx.x;
  if (vmax_blk) {
    double m = 0.0;
    if (c < D) {
      // eight loads in flight per lane (a maximum does not depend on the order)
      for (int i0 = c; i0 < nblk; i0 += 8 * D) {
        float t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = i0 + u * D < nblk ? vmax_blk[i0 + u * D] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) m = max_keep_nan(m, (double)t[u]);
      }
    }
    for (int off = 32; off > 0; off >>= 1) m = max_keep_nan(m, __shfl_xor(m, off));
    if (c < D && (c & 63) == 0) red[c >> 6] = m;
    __syncthreads();
    if (c == 0) {
      double r = red[0];
      for (int w = 1; w < (D + 63) / 64; ++w) r = max_keep_nan(r, red[w]);
      *vmax_out = r;
    }
  }
  if (c < D) {
    const double* p = sums + c;
    double s = 0.0;
    int i = 0;
    for (; i + 8 <= Sk; i += 8) {  // eight loads in flight, then the adds in split order
      double t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = p[(size_t)(i + u) * D];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += t[u];
    }
    for (; i < Sk; ++i) s += p[(size_t)i * D];
    kbar[c] = s / (double)Nk;
    if (kbar_copy) kbar_copy[c] = s / (double)Nk;
  }
}

template <int D>
__device__ __forceinline__ void kbar_block(const double* __restrict__ ksum_part, int Nk, int Sk,
                                           double* __restrict__ kbar, const float* __restrict__ vmax_blk, int nblk,
                                           double* __restrict__ vmax_part, int bh) {
  __shared__ double red[(D + 63) / 64];
  kbar_block_impl<D>(ksum_part + (size_t)bh * Sk * D, Nk, Sk, kbar + (size_t)bh * D, nullptr,
                     vmax_blk ? vmax_blk + (size_t)bh * nblk : nullptr, nblk, vmax_part + (size_t)bh * Sk, red);
}

template <int D>
__global__ void __launch_bounds__(D)
cert_kbar(const double* __restrict__ ksum_part, int Nk, int Sk, double* __restrict__ kbar,
          const float* __restrict__ vmax_blk, int nblk, double* __restrict__ vmax_part) {
  kbar_block<D>(ksum_part, Nk, Sk, kbar, vmax_blk, nblk, vmax_part, blockIdx.x);
}

// One fp64 value from another lane of the same row of 16 lanes (a DPP move
// of both halves; the pattern CTRL never selects a lane outside the row).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_mov_dpp((int)(unsigned)u, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(unsigned)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Sum over the 8 consecutive lanes that hold one row: pairs (xor 1), quads
// (xor 2), then the two quads (lane i with 7 - i); every lane of the group
// ends with the same value.  DPP moves stay in the VALU.
__device__ __forceinline__ double row8_sum(double x) {
  x += dpp_f64<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f64<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f64<0x141>(x);  // row_half_mirror
  return x;
}

// Steps 2-3 on key splits; ||q||^2 and the stabilizers on query splits.
// Eight lanes hold a row: lane t of the group its 16-byte chunks t, t + 8,
// ... (contiguous 128 bytes of the row per load across the group).
template <typename T, int D>
__device__ __forceinline__ void norms_block(const T* __restrict__ Q, const T* __restrict__ K,
                                            const double* __restrict__ kbar, int Nq, int Nk, int Sk, int Sq,
                                            double c2, float* __restrict__ mu, double* __restrict__ kap_part,
                                            double* __restrict__ qss_part, int bh, int part) {
  constexpr int VEC = Vec<T>::n, TPR = 8, RPI = kThreads / TPR;
  constexpr int NL = D / VEC / TPR;  // 16-byte loads per lane per row
  constexpr int UN = kUnroll / 2;  // rows per lane in flight (more measured slower: registers)
  static_assert(D % (VEC * TPR) == 0, "whole chunks per lane");
  __shared__ double red[kThreads / 64];
  const int tr = threadIdx.x / TPR, tc = threadIdx.x % TPR;
  double kb[NL][VEC];
#pragma unroll
  for (int i = 0; i < NL; ++i)
#pragma unroll
    for (int e = 0; e < VEC; ++e) kb[i][e] = kbar[(size_t)bh * D + (tc + TPR * i) * VEC + e];
  double best = 0.0;
  const bool keys = part < Sk;
  const int split = keys ? part : part - Sk;
  const int n = keys ? Nk : Nq;
  int lo, hi;
  split_range(n, keys ? Sk : Sq, split, &lo, &hi);
  const T* base = (keys ? K : Q) + (size_t)bh * n * D;
  // every lane of a row group runs the same trip count, so the DPP partners
  // are always active
  for (int j0 = lo; j0 < hi; j0 += UN * RPI) {
    uint4 ld[UN][NL];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * RPI + tr;
#pragma unroll
      for (int i = 0; i < NL; ++i)
        ld[u][i] = j < hi ? stream_load16(base + (size_t)j * D + (tc + TPR * i) * VEC)
                          : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * RPI + tr;
      double ss = 0.0, dot = 0.0;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        double x[VEC];
        widen<T>(ld[u][i], x);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          if (keys) {
            const double t = x[e] - kb[i][e];
            ss += t * t;
          } else {
            ss += x[e] * x[e];
            dot += x[e] * kb[i][e];
          }
        }
      }
      ss = row8_sum(ss);
      if (!keys) dot = row8_sum(dot);
      if (j < hi) {
        best = max_keep_nan(best, ss);
        if (!keys && tc == 0) mu[(size_t)bh * Nq + j] = (float)(c2 * dot);
      }
    }
  }
  best = block_max(best, red);
  if (threadIdx.x == 0) (keys ? kap_part[(size_t)bh * Sk + split] : qss_part[(size_t)bh * Sq + split]) = best;
}

template <typename T, int D>
__global__ void __launch_bounds__(kThreads)
cert_norms(const T* __restrict__ Q, const T* __restrict__ K, const double* __restrict__ kbar,
           int Nq, int Nk, int Sk, int Sq, double c2, float* __restrict__ mu,
           double* __restrict__ kap_part, double* __restrict__ qss_part) {
  // 1-D grid: any head count.  Heads in reverse order: the keys that
  // cert_keys_values read last are the ones still cached (measured 2-3%
  // faster than forward order on the long workloads; results do not depend
  // on the order, each block writes its own partial).
  const unsigned b = gridDim.x - 1 - blockIdx.x;
  norms_block<T, D>(Q, K, kbar, Nq, Nk, Sk, Sq, c2, mu, kap_part, qss_part, b / (Sk + Sq), b % (Sk + Sq));
}

// ceil(log2 x) for finite x >= 1, exactly.
__device__ __forceinline__ int ceil_log2_f64(double x) {
  int e;
  const double f = frexp(x, &e);
  return (f == 0.5) ? e - 1 : e;
}

// Steps 3-7 and the flag for head h from its maxima (one thread).
__device__ __forceinline__ void finalize_values(double vmax, double kap2, double qss, int Nk, double c2,
                                                int32_t* __restrict__ cert, clis_head_stats_t* __restrict__ stats,
                                                int h) {
  const double kappa = sqrt(kap2);
  const double qmax = sqrt(qss);
  const double bound = (c2 * qmax) * kappa;
  // step 5; a non-finite max |V| gets G = 128 so that C < 0
  const int G = isfinite(vmax) ? ceil_log2_f64(vmax > 1.0 ? vmax : 1.0) : 128;
  // step 6: ceil(log2 Nk) for Nk >= 1
  const int L = (Nk <= 1) ? 0 : 32 - __clz(Nk - 1);
  const int A = L + G;
  // step 7 with the Figure 3 limits of fp32 accumulators and bf16/fp32 exp2
  // outputs: log2 of the largest finite value is 127.99... in both formats,
  // so floor(U_exp) = 127 and ceil(U_acc - A) - 1 = 127 - A for integer A.
  const int C = min(127, 127 - A);
  const int ok = (isfinite(bound) && bound <= (double)C) ? 1 : 0;
  cert[h] = ok;
  clis_head_stats_t st;
  st.kappa = kappa;
  st.qnorm_max = qmax;
  st.bound = bound;
  st.maxabs_v = vmax;
  st.G = G;
  st.L = L;
  st.A = A;
  st.C = C;
  st.cert = ok;
  st.reserved = 0;
  stats[h] = st;
}

// The same from the split partials, one wave per head: lane i takes splits
// i, i + 64, ... and the lanes' maxima meet by shuffles (a maximum does not
// depend on the order, and a NaN is kept whichever lane holds it).
constexpr int kFinalizeHeads = kThreads / 64;  // heads per block

__global__ void __launch_bounds__(kThreads)
cert_finalize(const double* __restrict__ vmax_part, const double* __restrict__ kap_part,
              const double* __restrict__ qss_part, int BH, int Nk, int Sk, int Sq, double c2,
              int32_t* __restrict__ cert, clis_head_stats_t* __restrict__ stats) {
  const int lane = threadIdx.x & 63;
  const long long h = (long long)blockIdx.x * kFinalizeHeads + threadIdx.x / 64;
  if (h >= BH) return;  // whole waves
  double vmax = 0.0, kap2 = 0.0, qss = 0.0;
  for (int i = lane; i < Sk; i += 64) {
    vmax = max_keep_nan(vmax, vmax_part[h * Sk + i]);
    kap2 = max_keep_nan(kap2, kap_part[h * Sk + i]);
  }
  for (int i = lane; i < Sq; i += 64) qss = max_keep_nan(qss, qss_part[h * Sq + i]);
  for (int off = 32; off > 0; off >>= 1) {
    vmax = max_keep_nan(vmax, __shfl_xor(vmax, off));
    kap2 = max_keep_nan(kap2, __shfl_xor(kap2, off));
    qss = max_keep_nan(qss, __shfl_xor(qss, off));
  }
  if (lane == 0) finalize_values(vmax, kap2, qss, Nk, c2, cert, stats, (int)h);
}

// Shapes with one key split and one query split: the four passes for one
// head in one block, in the same order and with the same arithmetic as the
// four kernels (so the results are bitwise theirs), one launch instead of
// four.
// Steps 2-3 for short sequences: the key norms and the query norms with the
// stabilizers in one pass over the rows [K; Q] of head bh (the same per-row
// arithmetic as norms_block); the two maxima go to *kap2 and *qss.
template <typename T, int D, int NTH>
__device__ __forceinline__ void norms_both_block(const T* __restrict__ Q, const T* __restrict__ K,
                                                 const double* kbar_head, int Nq, int Nk, double c2,
                                                 float* __restrict__ mu, int bh, double* kap2, double* qss) {
  constexpr int VEC = Vec<T>::n, TPR = 8, RPI = NTH / TPR;
  constexpr int NL = D / VEC / TPR;  // 16-byte loads per lane per row
  constexpr int UN = NL > 2 ? kUnroll / 4 : kUnroll / 2;  // rows per lane in flight
  static_assert(D % (VEC * TPR) == 0, "whole chunks per lane");
  __shared__ double red[NTH / 64];
  const int tr = threadIdx.x / TPR, tc = threadIdx.x % TPR;
  double kb[NL][VEC];
#pragma unroll
  for (int i = 0; i < NL; ++i)
#pragma unroll
    for (int e = 0; e < VEC; ++e) kb[i][e] = kbar_head[(tc + TPR * i) * VEC + e];
  const T* kbase = K + (size_t)bh * Nk * D;
  const T* qbase = Q + (size_t)bh * Nq * D;
  const int n = Nk + Nq;  // rows 0 .. Nk-1 are keys, the rest queries
  double best_k = 0.0, best_q = 0.0;
  // all lanes of a row group take the same row and trip count, so the DPP
  // partners are always active
  for (int j0 = 0; j0 < n; j0 += UN * RPI) {
    uint4 ld[UN][NL];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * RPI + tr;
      const T* row = j < Nk ? kbase + (size_t)j * D : qbase + (size_t)(j - Nk) * D;
#pragma unroll
      for (int i = 0; i < NL; ++i)
        ld[u][i] = j < n ? stream_load16(row + (tc + TPR * i) * VEC) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * RPI + tr;
      const bool key = j < Nk;
      double ss = 0.0, dot = 0.0;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        double x[VEC];
        widen<T>(ld[u][i], x);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          if (key) {
            const double t = x[e] - kb[i][e];
            ss += t * t;
          } else {
            ss += x[e] * x[e];
            dot += x[e] * kb[i][e];
          }
        }
      }
      ss = row8_sum(ss);
      dot = row8_sum(dot);
      if (key) {
        best_k = max_keep_nan(best_k, ss);
      } else if (j < n) {
        best_q = max_keep_nan(best_q, ss);
        if (tc == 0) mu[(size_t)bh * Nq + (j - Nk)] = (float)(c2 * dot);
      }
    }
  }
  *kap2 = block_max<NTH>(best_k, red);
  *qss = block_max<NTH>(best_q, red);
}

// Certification of one head per block of kSmallThreads threads, for one key
// split and one query split: column sums, kbar, the norm pass over keys and
// queries together, and the flag -- one launch instead of four.
constexpr int kSmallThreads = 1024;

template <typename T, int D, bool WITH_V>
__global__ void __launch_bounds__(kSmallThreads)
cert_small(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, int Nq, int Nk, double c2,
           const float* __restrict__ vmax_blk, int nblk, double* __restrict__ kbar, float* __restrict__ mu,
           int32_t* __restrict__ cert, clis_head_stats_t* __restrict__ stats) {
  static_assert(D <= kSmallThreads, "kbar: one thread per channel");
  // the head's column sums, kbar and max |V| stay in LDS between the passes
  __shared__ double sums[D], kb[D], red[(D + 63) / 64], vmax;
  const int bh = blockIdx.x;
  keys_values_block<T, D, WITH_V, kSmallThreads>(K, V, Nk, 1, sums, &vmax, bh, 0);
  __syncthreads();  // the column sums are in LDS
  kbar_block_impl<D>(sums, Nk, 1, kbar + (size_t)bh * D, kb, vmax_blk ? vmax_blk + (size_t)bh * nblk : nullptr,
                     nblk, &vmax, red);
  __syncthreads();  // kbar (and max |V|) are in LDS
  double kap2, qss;
  norms_both_block<T, D, kSmallThreads>(Q, K, kb, Nq, Nk, c2, mu, bh, &kap2, &qss);
  if (threadIdx.x == 0) finalize_values(vmax, kap2, qss, Nk, c2, cert, stats, bh);
}

__global__ void __launch_bounds__(64)
route_heads(const int32_t* __restrict__ cert, int mode, int BH, int32_t* __restrict__ lists,
            int32_t* __restrict__ counts, int32_t* __restrict__ route_out) {
  // One wave compacts the heads in index order: ballot + prefix popcount.
  const int lane = threadIdx.x;
  int nf = 0, no = 0, nsplit = 0;
  for (int base = 0; base < BH; base += 64) {
    const int h = base + lane;
    int fixed = 0;
    if (h < BH) fixed = (mode == CLIS_MODE_FIXED) || (mode == CLIS_MODE_AUTO && cert[h] != 0);
    const unsigned long long fm = __ballot(h < BH && fixed);
    const unsigned long long om = __ballot(h < BH && !fixed);
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (h < BH) {
      if (fixed) lists[nf + __popcll(fm & below)] = h;
      else lists[BH + no + __popcll(om & below)] = h;
      if (route_out) route_out[h] = fixed;
    }
    if (base == 0) nsplit = __popcll(fm & ((1ull << kSplitHeads) - 1));  // heads 0 .. kSplitHeads-1
    nf += __popcll(fm);
    no += __popcll(om);
  }
  if (lane == 0) {
    counts[0] = nf;
    counts[1] = no;
    counts[2] = 0;  // work counters of the attention kernels that follow
    counts[3] = 0;
    counts[4] = nsplit;
  }
}

template <typename T, int D>
hipError_t certify_typed(const CertifyArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  const int Sk = cert_splits(a.Nk), Sq = cert_splits(a.Nq);
  const double c2 = (double)a.scale * kLog2e;
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  if ((long long)BH * (Sk + Sq) > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (Sk == 1 && Sq == 1) {
    // without V when max |V| came with the V transpose
    auto kern = a.vmax_blk ? cert_small<T, D, false> : cert_small<T, D, true>;
    kern<<<(unsigned)BH, kSmallThreads, 0, s>>>(q, k, v, a.Nq, a.Nk, c2, a.vmax_blk, a.vmax_nblk, a.kbar, a.mu,
                                                a.cert, a.stats);
    return hipGetLastError();
  }
  if (a.vmax_blk)  // max |V| came with the V transpose
    cert_keys_values<T, D, false><<<(unsigned)(BH * Sk), kThreads, 0, s>>>(k, v, a.Nk, Sk, a.ksum_part, a.vmax_part);
  else
    cert_keys_values<T, D, true><<<(unsigned)(BH * Sk), kThreads, 0, s>>>(k, v, a.Nk, Sk, a.ksum_part, a.vmax_part);
  cert_kbar<D><<<BH, D, 0, s>>>(a.ksum_part, a.Nk, Sk, a.kbar, a.vmax_blk, a.vmax_nblk, a.vmax_part);
  cert_norms<T, D><<<(unsigned)(BH * (Sk + Sq)), kThreads, 0, s>>>(q, k, a.kbar, a.Nq, a.Nk, Sk, Sq, c2, a.mu,
                                                                    a.kap_part, a.qss_part);
  const int fb = (int)(((long long)BH + kFinalizeHeads - 1) / kFinalizeHeads);
  cert_finalize<<<fb, kThreads, 0, s>>>(a.vmax_part, a.kap_part, a.qss_part, BH, a.Nk, Sk, Sq, c2,
                                        a.cert, a.stats);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_certify(const CertifyArgs& a, hipStream_t s) {
  if (a.dtype == CLIS_BF16) {
    if (a.d == 128) return certify_typed<uint16_t, 128>(a, s);
    if (a.d == 64) return certify_typed<uint16_t, 64>(a, s);
  } else {
    if (a.d == 128) return certify_typed<float, 128>(a, s);
    if (a.d == 64) return certify_typed<float, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_route(const int32_t* cert, int mode, int BH, int32_t* lists, int32_t* counts,
                        int32_t* route_out, hipStream_t s) {
  route_heads<<<1, 64, 0, s>>>(cert, mode, BH, lists, counts, route_out);
  return hipGetLastError();
}

}  // namespace clis
