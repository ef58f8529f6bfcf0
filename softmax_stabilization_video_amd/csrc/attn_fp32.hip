// attn_fp32.hip -- attention forward for fp32 inputs, on the fp32 matrix
// cores (v_mfma_f32_32x32x2_f32): Q, K, V, the weights P and the sums all stay
// fp32, so the result keeps fp32 accuracy.  The softmax forms are those of
// the bf16 kernels ("CLiS: Plug-and-Play Attention Acceleration for Video
// Diffusion on TPUs via Certified Stabilization", abstract and Figure 5(a)):
// fixed stabilizer (with its key-shard form, o_acc / l_acc), online softmax,
// and online softmax with lazy rescaling; each can also write the row
// log-sum-exp.  The FP32 exp2 limits of Figure 3 enter through C, which the
// certificate compares against.
//
// One workgroup = 32 query rows of one head and four waves.  The 32-key tiles
// are dealt to the waves in turn (tile t to wave t mod 4); each wave keeps its
// own partial sums, and the four partials are combined in LDS in wave order at
// the end, so the result does not depend on timing.  A wave computes the
// transposed score tile S^T = K Q^T (32 keys x 32 queries): a lane then holds
// 16 keys of one query, and its 16 weights are, register for register, the B
// operand of O^T += V^T P^T; P never leaves the registers.  The dot products
// of S^T run over the head dim in the order lane half 0 takes dims [0, d/2)
// and lane half 1 dims [d/2, d); the key order inside a P.V step is the one
// the score tile's layout gives (lane half h, register r: key 8 (r / 4) +
// 4 h + r mod 4).  K and V go from memory (mostly L2) to registers with no
// LDS staging: the wave reads each tile once, one tile ahead of its use.
//
// Routing: the kernel takes the route of each head itself (fixed when the
// call forces it or, in auto mode, when the head's certificate flag is set),
// so a certified fp32 call is one attention launch after certification; the
// choice is uniform over a workgroup.
#include <hip/hip_runtime.h>
#include <math.h>

#include "internal.h"

namespace clis {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kRows = 32;   // query rows per workgroup
constexpr int kTile = 32;   // keys per tile
constexpr int kWaves = 4;   // waves per workgroup, each on every 4th key tile
constexpr int kThreads = 64 * kWaves;

// Route of the kernel's heads: every head online, every head fixed, or per head
// from the certificate flags.
enum Route { kOnline = 0, kFixed = 1, kAuto = 2 };

__device__ __forceinline__ floatx16 mfma32(float a, float b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Key of register r of a score tile in lane half h (the MFMA's output layout).
__device__ __forceinline__ int tile_key(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// One key tile's operands for a lane: its K row half (dims h*d/2 ...) and, for
// each P.V step s and dim block t, V[key of step s][32 t + column].  Keys past
// Nk read as zeros.
template <int D>
struct TileRegs {
  float k[D / 2];
  float v[D / 32][16];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& R, const float* __restrict__ Kh,
                                          const float* __restrict__ Vh, int kt, int Nk, int h, int col) {
  const int key = kt + col;
  if (key < Nk) {
    const float4* src = reinterpret_cast<const float4*>(Kh + (size_t)key * D + h * (D / 2));
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const float4 x = src[i];
      R.k[4 * i] = x.x;
      R.k[4 * i + 1] = x.y;
      R.k[4 * i + 2] = x.z;
      R.k[4 * i + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < D / 2; ++i) R.k[i] = 0.f;
  }
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int vk = kt + tile_key(s, h);
#pragma unroll
    for (int t = 0; t < D / 32; ++t) R.v[t][s] = vk < Nk ? Vh[(size_t)vk * D + 32 * t + col] : 0.f;
  }
}

template <int D, int ROUTE, bool CAUSAL, bool LAZY>
__global__ void __launch_bounds__(kThreads)
attn_fwd_fp32(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
              float* __restrict__ O, const float* __restrict__ mu, const int32_t* __restrict__ cert,
              int32_t* __restrict__ route_out, int Nq, int Nk, float c2, float* __restrict__ lse,
              float* __restrict__ o_acc, float* __restrict__ l_acc, int accumulate, int kv_offset) {
  // No implicit fusing of a product into a following add: each route computes
  // the operations as written (explicit fmaf where one rounding is meant), so
  // its results do not depend on which other routes the instance can take --
  // auto mode equals the forced route bitwise.
#pragma clang fp contract(off)
  constexpr int NT = D / 32;   // 32-dim blocks of O^T
  constexpr int OST = D + 4;   // LDS row stride of a wave's partial O (floats)
  __shared__ __attribute__((aligned(16))) float part_o[kWaves][kRows][OST];
  __shared__ float part_l[kWaves][kRows];
  __shared__ float part_m[kWaves][kRows];

  const int n_qt = (Nq + kRows - 1) / kRows;
  const int bh = blockIdx.x / n_qt;
  // causal: the longest query tiles (most keys) first
  const int qt = CAUSAL ? n_qt - 1 - blockIdx.x % n_qt : blockIdx.x % n_qt;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int q0 = qt * kRows;
  const int qrow = q0 + col;  // this lane's query
  const bool qvalid = qrow < Nq;
  // the row's stabilizer is read whenever the head may run fixed, before the
  // flag is known, so that the two loads are in flight together
  const float mu_row = (ROUTE != kOnline && qvalid) ? mu[(size_t)bh * Nq + qrow] : 0.f;
  const bool FIXED = ROUTE == kFixed || (ROUTE == kAuto && cert[bh] != 0);
  if (route_out && blockIdx.x % n_qt == 0 && threadIdx.x == 0) route_out[bh] = FIXED ? 1 : 0;
  const float* Kh = K + (size_t)bh * Nk * D;
  const float* Vh = V + (size_t)bh * Nk * D;

  // this lane's half of its query row: dims h*d/2 ...
  float qf[D / 2];
  if (qvalid) {
    const float4* src = reinterpret_cast<const float4*>(Q + ((size_t)bh * Nq + qrow) * D + h * (D / 2));
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const float4 x = src[i];
      qf[4 * i] = x.x;
      qf[4 * i + 1] = x.y;
      qf[4 * i + 2] = x.z;
      qf[4 * i + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < D / 2; ++i) qf[i] = 0.f;
  }

  floatx16 o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m = FIXED ? mu_row : -INFINITY;
  float l = 0.f;  // this lane's 16 keys of every tile; the halves are added at the end

  // local keys this block needs (the causal mask compares global indices)
  const int kv_end = CAUSAL ? max(0, min(Nk, q0 + kRows - kv_offset)) : Nk;
  const int n_kt = (kv_end + kTile - 1) / kTile;
  TileRegs<D> cur;
  if (wave < n_kt) load_tile<D>(cur, Kh, Vh, wave * kTile, Nk, h, col);
  for (int it = wave; it < n_kt; it += kWaves) {
    const int kt = it * kTile;
    // the next tile (the wave's last tile loads itself again, unused)
    TileRegs<D> nxt;
    load_tile<D>(nxt, Kh, Vh, it + kWaves < n_kt ? kt + kWaves * kTile : kt, Nk, h, col);

    floatx16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int i = 0; i < D / 2; ++i) s = mfma32(cur.k[i], qf[i], s);

    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kt + tile_key(r, h);
      const bool ok = key < Nk && (!CAUSAL || kv_offset + key <= qrow);
      x[r] = ok ? (FIXED ? fmaf(s[r], c2, -m) : s[r] * c2) : -INFINITY;
    }
    if (!FIXED) {
      float tmax = x[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, x[r]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));  // both halves of the query's keys
      float msub;
      if constexpr (LAZY) {
        // conditional rescaling: the stabilizer moves only when the tile
        // maximum exceeds it by more than 8 (log2 units); weights stay <= 256
        if (tmax > m + 8.f) {
          const float alpha = __builtin_amdgcn_exp2f(m - tmax);  // 0 while m = -inf
          l *= alpha;
#pragma unroll
          for (int t = 0; t < NT; ++t) o[t] *= alpha;
          m = tmax;
        }
        msub = (m == -INFINITY) ? 0.f : m;
      } else {
        const float mnew = fmaxf(m, tmax);
        const bool none = (mnew == -INFINITY);
        const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m - mnew);
        msub = none ? 0.f : mnew;
        l *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) o[t] *= alpha;
        m = mnew;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] -= msub;
    }
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(x[r]);
      l += p[r];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) o[t] = mfma32(cur.v[t][r], p[r], o[t]);
    cur = nxt;
  }

  // this wave's partial: O^T register r of block t is dim 32 t + tile_key(r, h)
  l += __shfl_xor(l, 32);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<float4*>(&part_o[wave][col][32 * t + 8 * a + 4 * h]) =
          make_float4(o[t][4 * a], o[t][4 * a + 1], o[t][4 * a + 2], o[t][4 * a + 3]);
  if (h == 0) {
    part_l[wave][col] = l;
    part_m[wave][col] = m;
  }
  __syncthreads();

  // combine the waves in order; a thread takes 4 dims of one row at a time
  for (int e = threadIdx.x; e < kRows * (D / 4); e += kThreads) {
    const int r = e / (D / 4), c4 = (e % (D / 4)) * 4;
    const int row = q0 + r;
    if (row >= Nq) continue;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float lt = 0.f, mt = FIXED ? part_m[0][r] : -INFINITY;
    if (FIXED) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float4 y = *reinterpret_cast<const float4*>(&part_o[w][r][c4]);
        acc.x += y.x; acc.y += y.y; acc.z += y.z; acc.w += y.w;
        lt += part_l[w][r];
      }
    } else {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) mt = fmaxf(mt, part_m[w][r]);
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = part_m[w][r];
        const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - mt);
        const float4 y = *reinterpret_cast<const float4*>(&part_o[w][r][c4]);
        acc.x = fmaf(f, y.x, acc.x); acc.y = fmaf(f, y.y, acc.y);
        acc.z = fmaf(f, y.z, acc.z); acc.w = fmaf(f, y.w, acc.w);
        lt = fmaf(f, part_l[w][r], lt);
      }
    }
    const size_t orow = (size_t)bh * Nq + row;
    if (FIXED && o_acc) {  // key shard: the unnormalized sums, continued from earlier shards
      float4* dst = reinterpret_cast<float4*>(o_acc + orow * D + c4);
      if (accumulate) {
        const float4 y = *dst;
        acc.x = y.x + acc.x; acc.y = y.y + acc.y; acc.z = y.z + acc.z; acc.w = y.w + acc.w;
      }
      *dst = acc;
      if (c4 == 0) l_acc[orow] = accumulate ? l_acc[orow] + lt : lt;
      continue;
    }
    const float inv = 1.f / lt;
    *reinterpret_cast<float4*>(O + orow * D + c4) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (lse && c4 == 0) lse[orow] = 0.693147180559945309f * (mt + log2f(lt));
  }
}

template <int D, int ROUTE, bool CAUSAL, bool LAZY = false>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  const int n_qt = (a.Nq + kRows - 1) / kRows;
  const long long blocks = (long long)n_qt * a.n_slots;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  attn_fwd_fp32<D, ROUTE, CAUSAL, LAZY><<<(unsigned)blocks, kThreads, 0, s>>>(
      static_cast<const float*>(a.q), static_cast<const float*>(a.k), static_cast<const float*>(a.v),
      static_cast<float*>(a.o), a.mu, a.cert, a.route_out, a.Nq, a.Nk, a.c2, a.lse, a.o_acc, a.l_acc,
      a.accumulate, a.kv_offset);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, bool fixed, hipStream_t s) {
  if (a.cert) return a.causal ? launch_t<D, kAuto, true>(a, s) : launch_t<D, kAuto, false>(a, s);
  if (fixed) return a.causal ? launch_t<D, kFixed, true>(a, s) : launch_t<D, kFixed, false>(a, s);
  if (a.lazy) return a.causal ? launch_t<D, kOnline, true, true>(a, s) : launch_t<D, kOnline, false, true>(a, s);
  return a.causal ? launch_t<D, kOnline, true>(a, s) : launch_t<D, kOnline, false>(a, s);
}

}  // namespace

hipError_t launch_attn_fp32(const AttnArgs& a, bool fixed, hipStream_t s) {
  if (a.head_list) return hipErrorInvalidValue;  // the fp32 kernel routes by itself
  if ((a.cert || fixed) && !a.mu) return hipErrorInvalidValue;  // the kernel reads mu on these routes
  if (a.d == 128) return launch_d<128>(a, fixed, s);
  if (a.d == 64) return launch_d<64>(a, fixed, s);
  return hipErrorInvalidValue;
}

}  // namespace clis
