// attn_bf16.hip -- fused attention forward on gfx950 bf16 MFMA.  One kernel
// template covers three softmax forms:
//   FIXED  -- CLiS: each query row's stabilizer mu_i is fixed before the key
//             loop, so the loop has no running maximum, no cross-lane step
//             and no accumulator rescaling ("CLiS: Plug-and-Play Attention
//             Acceleration for Video Diffusion on TPUs via Certified
//             Stabilization", abstract and Figure 5(a));
//   ONLINE -- online softmax: per key tile a running row maximum and a
//             rescale factor alpha for the row sum and the output accumulator
//             (the baseline those pages compare against);
//   ONLINE, LAZY -- online softmax with conditional rescaling (the form of
//             FlashAttention-4, which those pages name as a comparator): the
//             stabilizer in use moves, and the accumulators are rescaled, only
//             when a row's tile maximum exceeds it by more than kLazyTau (log2
//             units), under a wave-uniform branch; weights stay <= 2^kLazyTau.
// The fixed form has two more switches: PARTIAL (key shards: fp32
// unnormalized sums in and out) and, for the dense non-shard form, the
// last-round key splits below.  Every fixed form evaluates the exp2 argument
// as x = fma(s, c, -mu) in fp32 from the fp32 score s = q.k and the exact bf16
// inputs, so x stays within fp32 rounding of c q.k - mu: the quantity the
// certificate bounds.  The fixed and online forms use
// independently tuned workgroup sizes (the pages tune tiles per method too,
// Table 7 caption).
//
// Work decomposition.  A workgroup of WAVES waves owns 32*H*WAVES query rows
// of one (batch, head); each wave owns H 32-row halves (H = 2 in the fixed
// forms at d = 128, H = 1 otherwise), and two waves share a SIMD.  K and
// V^T tiles of 64 keys stream through an LDS ring, loaded with buffer loads
// that write LDS directly (buffer_load_dword[x4] ... lds), one barrier per
// tile.  Both products use v_mfma_f32_32x32x16_bf16 with fp32 accumulation,
// oriented so that every lane owns one query row of each half:
//   S^T = K Q^T   A = K rows from LDS (ds_read_b128), B = Q fragments held in
//                 registers for the whole loop; lane l holds the scores of
//                 query l%32 for 16 of every 32 keys (register r of a 32-key
//                 block: key 8(r/4) + 4g + r%4, g = l/32); the other 16 keys
//                 sit in lane l^32.
//   O^T = V^T P^T A = V^T fragments from LDS (one ds_read_b128 each), B = P
//                 straight from the S^T accumulators, converted to bf16.
// Per-row quantities (mu, m, l, alpha) are therefore per lane; a row meets
// lane l^32 only for the online tile maximum and the final row sum.
//
// Two halves per wave (H = 2).  Each K or V^T fragment read from LDS then
// feeds two products, which halves the LDS reads per MFMA.  The 64 rows'
// output accumulators (128 registers) live in AGPRs and the tile work is
// generated asm (gen_tile_h2.py -> tile_h2.inc) in fixed registers.  The two
// waves of a SIMD run the same chain of parts (scores, weights, products of
// the tile's two 32-key blocks) half a tile apart, so that one's weights
// (VALU only) overlap the other's products; a window between barriers then
// reads two tiles while the next loads, hence three LDS stages.  The next
// tile's loads are issued from inside the asm, spread between products.
//
// V^T.  The P.V operand needs, per lane, eight keys of one channel: keys
// 4g..4g+3 and 8+4g..8+4g+3 of a 16-key step.  transpose_v (transpose.hip)
// writes V^T as 64-key tiles [d][kVtRow] (a tile's 64 keys per channel, then
// 8 zeros) with each 16-key group stored as {0-3, 8-11, 4-7, 12-15}, which
// makes those eight keys contiguous, so one ds_read_b128 fetches an operand
// (instead of two LDS transpose reads from a row-major V tile; on gfx950 the
// LDS read issue rate bounds a 32-row MFMA attention).  Nk_pad is a multiple
// of 128; keys past Nk are zero.
//
// Outputs.  Normally O = O_acc / l in bf16, and optionally each row's
// log-sum-exp ln 2 * (m + log2 l), where m is the fixed mu_i or the final
// running maximum (both in log2 units).  With o_acc set (fixed variant
// only, for key-value shards) the kernel instead starts from, or overwrites,
// fp32 unnormalized sums o_acc and l_acc: with a fixed stabilizer the sums
// over disjoint key ranges simply add.  kv_offset is the global index of key 0
// (the causal mask compares global key and query indices).
//
// Work pool (dense forms).  A grid of W workgroups runs in rounds of the
// workgroups resident at once, and the XCDs of one GPU run at different clocks
// under this load, so with the hardware's fixed round-robin deal of
// workgroups to XCDs the slowest XCD finishes last, and a partial last round
// leaves most CUs idle.  The last tenth of the items (at least the partial
// round) is instead a pool claimed from a device counter by the workgroups
// that follow the others: whole items, and in the fixed form then items cut
// into 8 key splits that write fp32 unnormalized sums to the workspace, added
// in split order and normalized by tail_combine (with a fixed stabilizer the
// parts simply add).  XCDs that run faster reach the pool earlier and claim
// more of it.  The counters are zeroed by the route kernel that precedes
// every launch.
//
// LDS layouts.  Compiled tile code (H = 1): rows unpadded, with 16-byte
// chunks XOR-swizzled per row, so the 16 lanes that read one chunk position of
// 16 rows hit distinct banks; the swizzle is applied when loading (lane i of a
// load-to-LDS instruction writes slot base+16i, so each lane fetches the
// global chunk that belongs there) and each lane keeps its fragment offsets.
// Generated code (H = 2): rows padded by 16 bytes (a 272-byte K row, a
// 144-byte V^T row, as the V^T tiles are stored), which also spreads 16 rows
// over all banks and makes every fragment one base register plus an
// immediate.  K rows past the last key read as zeros (the buffer descriptor's
// range check) and their weights are masked to 0.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "internal.h"
#include "tile_h2.inc"

namespace clis {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Waves per workgroup of each variant (measured best on MI355X).
#ifndef CLIS_FIXED_WAVES
#define CLIS_FIXED_WAVES 8
#endif
#ifndef CLIS_ONLINE_WAVES
#define CLIS_ONLINE_WAVES 4
#endif
#ifndef CLIS_CAUSAL_GROUP
#define CLIS_CAUSAL_GROUP 2
#endif
#ifndef CLIS_FIXED_CAUSAL_WAVES
#define CLIS_FIXED_CAUSAL_WAVES CLIS_FIXED_WAVES
#endif
// 32-row halves of queries per wave in the fixed forms that return O
#ifndef CLIS_FIXED_HALVES
#define CLIS_FIXED_HALVES 2
#endif
#ifndef CLIS_FIXED_CAUSAL_HALVES
#define CLIS_FIXED_CAUSAL_HALVES CLIS_FIXED_HALVES
#endif

constexpr int kBN = 64;                   // keys per tile
constexpr int kXcds = 8;                  // MI355X: workgroups are dealt round-robin to 8 XCDs
constexpr int kBufferFlags = 0x00020000;  // raw buffer descriptor word 3 (untyped 32-bit data)

// A raw buffer descriptor as four words (for asm operands): base, no stride,
// num_records bytes in range.  The arguments are wave-uniform.
__device__ __forceinline__ u32x4 buffer_words(const void* base, uint32_t num_records) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const auto u = [](uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); };
  return u32x4{u((uint32_t)a), u((uint32_t)(a >> 32) & 0xFFFFu), u(num_records), (uint32_t)kBufferFlags};
}
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLazyTau = 8.f;  // log2 units: lazy-rescale weights stay <= 256
constexpr int kMaxSplit = kTailSplits;  // key splits per split item
#ifndef CLIS_POOL_DIV
#define CLIS_POOL_DIV 10         // pool: at least 1 / CLIS_POOL_DIV of the items (0: the last round only)
#endif
#ifndef CLIS_POOL_OVER
#define CLIS_POOL_OVER 50        // pool workgroups launched beyond one per claim, in percent
#endif

// Work of the dense forms: `active` items (query tiles of the routed heads).
// In the fixed form the last query tile of each of the first S listed heads
// whose index is below kSplitHeads (S is counted by the route kernel) is cut
// into kTailSplits key splits (fp32 partial sums in the tail buffers, added
// in split order by tail_combine); which items are cut is a function of the
// head alone, so a head's output bits do not depend on the other heads routed
// with it.  Of the W = active - S whole items, the first F run one workgroup
// each, in XCD-local order; the last P1 whole items and then the S * 8 splits
// form a pool.  The workgroups after the first F each claim one pool entry
// from a device counter when they start, and exit if none is left (or at once
// when the pool is empty, e.g. when no head is routed to the kernel).  There
// are more of them than entries, and an XCD reaches its share of them once
// its own items are under way, so XCDs that run faster (the XCDs of one GPU
// run at different clocks under load) claim more of the pool; the splits at
// its end even out the last round.
struct PoolPlan {
  int F, P1, S;
};
__host__ __device__ inline PoolPlan pool_plan(int active, int conc, int S) {
  if (conc <= 0 || active <= 0) return PoolPlan{active, 0, 0};
  const int W = active - S;
  const int P = max(active % conc, CLIS_POOL_DIV > 0 ? active / CLIS_POOL_DIV : 0);
  const int P1 = min(W, max(0, P - S));
  return PoolPlan{W - P1, P1, S};
}

// Whole item w (0 <= w < active - S) -> (slot in the head list, query tile):
// the first S heads contribute their first n_qt - 1 tiles, the others all.
__device__ __forceinline__ void whole_item(int w, int S, int n_qt, int* slot, int* qt) {
  const int a = S * (n_qt - 1);
  if (w < a) {
    *slot = w / (n_qt - 1);
    *qt = w % (n_qt - 1);
  } else {
    const int x = w - a;
    *slot = S + x / n_qt;
    *qt = x % n_qt;
  }
}

__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// Logical block id for physical id `bid` when the first `active` blocks are
// live: each XCD gets one contiguous range of logical ids, so the query tiles
// of a head (which share its keys and values) stay within one XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int active) {
  const int x = bid % kXcds, i = bid / kXcds;
  const int base = active / kXcds, rem = active % kXcds;
  return (x < rem) ? x * (base + 1) + i : rem * (base + 1) + (x - rem) * base + i;
}

template <int D, int WAVES, int H = 1>
struct Geo {
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BM = 32 * H * WAVES;             // query rows per workgroup (H 32-row halves per wave)
  static constexpr int NS = D / 16;                     // k-steps of the S product
  static constexpr int NC = D / 32;                     // 32-channel output blocks
  // LDS tile rows: padded by 16 bytes for the generated two-half code (a
  // fragment is then one base register plus an immediate); unpadded, with
  // the 16-byte chunks of a row XOR-swizzled, for compiled code (per-lane
  // chunk offsets; fewer registers for the load sources)
  static constexpr bool PADDED = H == 2;
  static constexpr int KSTR = D * 2 + (PADDED ? 16 : 0);    // LDS bytes per K tile row (a key)
  static constexpr int VSTR = kBN * 2 + (PADDED ? 16 : 0);  // LDS bytes per V^T tile row (a channel)
  static constexpr int KTILE = kBN * KSTR;              // one K tile in LDS
  static constexpr int VTILE = D * VSTR;                // one V^T tile in LDS
  static constexpr int VTILE_G = D * kVtRow * 2;        // one V^T tile in memory (rows of kVtRow bf16)
  static constexpr int KCH = KTILE / 1024, VCH = VTILE / 1024;  // 1 KB load-to-LDS chunks per tile
  static constexpr int KL = (KCH + WAVES - 1) / WAVES;  // chunks per wave (at most) per tile
  static constexpr int VL = (VCH + WAVES - 1) / WAVES;
  // LDS stages: two (double buffering); three where the two waves of a SIMD
  // run half a tile apart and so read two tiles at a time (H = 2)
  static constexpr int NSTAGE = H == 2 ? 3 : 2;
  static constexpr int LDS_BYTES = NSTAGE * (KTILE + VTILE);
  // LDS map: the V^T stages, then the K stages
  static constexpr int voff(int stage) { return stage * VTILE; }
  static constexpr int koff(int stage) { return NSTAGE * VTILE + stage * KTILE; }
  static_assert(KTILE % 1024 == 0 && VTILE % 1024 == 0, "tiles are whole 1 KB load chunks");
  static_assert(!PADDED || VTILE == VTILE_G, "a padded V^T tile loads as one contiguous copy");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS of one workgroup");
};

// Unpadded tiles: the chunk swizzle of a row, for conflict-free 16-row reads.
// K tile row = one key (2D bytes).
template <int D>
__device__ __forceinline__ int swz_k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
// V^T tile row = one channel (128 bytes): two rows per 256 bytes of banks.
__device__ __forceinline__ int swz_v(int row) { return (row >> 1) & 7; }

// Byte offset, from a load's base, of the global data that lane `lane` of
// 1 KB chunk `ch` writes into a padded LDS tile of rows of `row_bytes` bytes
// (stride `stride` in LDS, `gstride` in memory); pad bytes read out of range,
// i.e. zeros, with no memory access.
__device__ __forceinline__ uint32_t chunk_src(int ch, int lane, int stride, int row_bytes, uint32_t gstride) {
  const int p = ch * 1024 + 16 * lane, r = p / stride, cb = p % stride;
  return cb < row_bytes ? (uint32_t)r * gstride + (uint32_t)cb : 0xFFFFFF00u;
}

// One wave's share of the K and V^T tiles at key kt, written to LDS by
// buffer loads of 1 KB chunks wave, wave + WAVES, ... of each LDS tile, each
// lane 16 bytes from the per-lane sources gk / gv (a padded V^T tile, H = 2,
// is one contiguous block laid out as in LDS: every lane's source is 16 x
// lane, the chunk's offset goes in the scalar offset).  Keys at and past Nk
// read as zeros.
template <int D, int WAVES, int H>
__device__ __forceinline__ void load_tiles(const char* Kh, const char* Vth, int kt, int Nk, char* lds, int stage,
                                           int wave, const uint32_t* gk, const uint32_t* gv) {
  using G = Geo<D, WAVES, H>;
  const int kbytes = min(Nk - kt, kBN) * D * 2;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(Kh + (size_t)kt * D * 2), 0, kbytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(Vth + (size_t)(kt / kBN) * G::VTILE_G), 0, G::VTILE_G, kBufferFlags);
  char* vdst = lds + G::voff(stage) + wave * 1024;
#pragma unroll
  for (int j = 0; j < G::VL; ++j)
    if (G::VCH % WAVES == 0 || j * WAVES + wave < G::VCH)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vdst + j * WAVES * 1024), 16, gv[H == 2 ? 0 : j],
                                               H == 2 ? (j * WAVES + wave) * 1024 : 0, 0, 0);
  char* kdst = lds + G::koff(stage) + wave * 1024;
#pragma unroll
  for (int j = 0; j < G::KL; ++j)
    if (G::KCH % WAVES == 0 || j * WAVES + wave < G::KCH)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kdst + j * WAVES * 1024), 16, gk[j], 0, 0, 0);
}

template <int D, bool FIXED, bool CAUSAL, int WAVES, bool PARTIAL, bool LAZY, int H>
__global__ void __launch_bounds__(64 * WAVES, WAVES >= 8 ? 1 : 2)
attn_fwd_bf16(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
              const uint16_t* __restrict__ Vt, uint16_t* __restrict__ O,
              const float* __restrict__ mu, const int32_t* __restrict__ head_list,
              const int32_t* __restrict__ head_count, int n_slots, int Nq, int Nk, int Nk_pad, float c2,
              float* __restrict__ lse, float* __restrict__ o_acc, float* __restrict__ l_acc, int accumulate,
              int kv_offset_arg, float* __restrict__ tail_o, float* __restrict__ tail_l, int pool_conc,
              int* __restrict__ sched, const int32_t* __restrict__ split_heads) {
  static_assert(FIXED || !PARTIAL, "key shards use the fixed stabilizer");
  static_assert(!(FIXED && LAZY), "lazy rescaling is an online-softmax form");
  static_assert(H == 1 || (H == 2 && FIXED), "two row halves per wave: fixed path");
  using G = Geo<D, WAVES, H>;
  constexpr bool PAD = H == 2;  // padded LDS tile rows (else swizzled)
  const int kv_offset = PARTIAL ? kv_offset_arg : 0;  // global index of key 0
  constexpr int NS = G::NS, NC = G::NC, BM = G::BM;
  __shared__ __attribute__((aligned(1024))) char lds[G::LDS_BYTES];  // V^T and K tiles, two stages each

  constexpr bool TAIL = FIXED && !PARTIAL && !CAUSAL;  // key splits of the pool
  const int n_qt = (Nq + BM - 1) / BM;
  const int n_heads = head_list ? *head_count : n_slots;
  const int active = n_heads * n_qt;
  int split = -1, nsplit = 1;  // split: this workgroup's slot in the tail buffers
  static_assert(!TAIL || BM <= kTailRows, "tail buffers hold kTailRows rows per workgroup");
  int slot, qt;
  if (!PARTIAL && !CAUSAL && sched) {  // pooled work (file comment)
    const int S = (TAIL && tail_o) ? (split_heads ? *split_heads : head_list ? 0 : min(n_slots, kSplitHeads)) : 0;
    const PoolPlan pp = pool_plan(active, pool_conc, S);
    const int b = blockIdx.x;
    int w;  // whole item, or -1 for a key split
    if (b < pp.F) {
      w = xcd_remap(b, pp.F);
    } else {  // pool workgroup: claim one entry
      const int entries = pp.P1 + pp.S * kMaxSplit;
      if (entries == 0) return;  // nothing pooled (no head routed to this kernel)
      // broadcast through LDS stage 1, which the second tile's load first
      // writes after a barrier every wave reaches past this read (a separate
      // LDS variable makes hipcc wait for each tile load before the next
      // product).  The counter only grows, so once a plain read shows the
      // pool drained the claim is skipped: it would fail, and thousands of
      // claims on one address cost more than the reads.
      int* claim = reinterpret_cast<int*>(lds + G::voff(1));
      if (threadIdx.x == 0) {
        const int seen = __hip_atomic_load(sched, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *claim = seen < entries ? atomicAdd(sched, 1) : seen;
      }
      __syncthreads();
      const int c = *claim;
      if (c < pp.P1) {  // a whole item
        w = pp.F + c;
      } else {
        split = c - pp.P1;  // a key split: its slot in the tail buffers
        if (!TAIL || split >= pp.S * kMaxSplit) return;
        nsplit = kMaxSplit;
        w = -1;
      }
    }
    if (w >= 0) {
      whole_item(w, pp.S, n_qt, &slot, &qt);
    } else {
      slot = split / kMaxSplit;
      qt = n_qt - 1;
    }
  } else {
    if ((int)blockIdx.x >= active) return;
    const int lid = xcd_remap(blockIdx.x, active);
    if constexpr (CAUSAL) {
      // Longest query tiles first, with heads taken in groups of G.  An XCD
      // deals consecutive workgroups round-robin to its four shader engines and
      // waits, in order, for a free CU in the next one, so every four
      // consecutive workgroups should be of (nearly) equal length and each
      // engine's total work equal: the G heads of a group advance together,
      // through their query tiles in blocks of M = 4 / G, every other block in
      // reverse.
      constexpr int G = CLIS_CAUSAL_GROUP, M = 4 / G;
      static_assert(G == 1 || G == 2 || G == 4, "heads per group: 1, 2 or 4");
      const int heads = active / n_qt, grp = lid / (G * n_qt);
      const int width = min(G, heads - G * grp), r = lid - G * n_qt * grp;
      slot = G * grp + r % width;
      const int p = r / width, blk = p / M, e = p % M, top = n_qt - 1 - M * blk;
      qt = (blk % 2 == 1 && blk < n_qt / M) ? top - (M - 1) + e : top - e;
    } else {
      slot = lid / n_qt;
      qt = lid % n_qt;
    }
  }
  const int bh = head_list ? head_list[slot] : slot;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int g = lane >> 5, ln = lane & 31;
  const int row0 = qt * BM + wave * 32 * H;  // first query row of this wave
  int qrow[H];
  bool qvalid[H];
  size_t qoff[H];
  auto set_rows = [&](int lane_) {
    g = lane_ >> 5;
    ln = lane_ & 31;
#pragma unroll
    for (int h = 0; h < H; ++h) {  // half h: rows row0 + 32h .. + 31, one per lane pair (l, l^32)
      qrow[h] = row0 + 32 * h + ln;
      qvalid[h] = qrow[h] < Nq;
      qoff[h] = ((size_t)bh * Nq + (qvalid[h] ? qrow[h] : 0)) * D;
    }
  };
  set_rows(lane);
  const char* Kh = reinterpret_cast<const char*>(K + (size_t)bh * Nk * D);
  const char* Vth = reinterpret_cast<const char*>(Vt) + (size_t)bh * (Nk_pad / kBN) * G::VTILE_G;

  // keys this workgroup covers: all of them, or its split's range of tiles
  int nkl = Nk;
  if (TAIL && split >= 0) {
    const int nt = (Nk + kBN - 1) / kBN, s = split % nsplit;
    const int t0 = s * nt / nsplit, t1 = (s + 1) * nt / nsplit;
    Kh += (size_t)t0 * kBN * D * 2;
    Vth += (size_t)t0 * G::VTILE_G;
    nkl = max(0, min(Nk - t0 * kBN, (t1 - t0) * kBN));
  }
  const int kv_end = CAUSAL ? max(0, min(Nk, (qt + 1) * BM - kv_offset)) : nkl;  // local keys needed
  const int ntiles = (kv_end + kBN - 1) / kBN;

  // ---- per-lane, loop-invariant offsets
  // load-to-LDS sources within a tile (lane's 16 bytes of chunk j * WAVES +
  // wave), and fragment addresses: the K fragment of (32-key block kb,
  // k-step s) is row 32kb + ln, bytes 16(2s + g) .. +15 of the key; the V^T
  // fragment of (block kb, 16-key step t, channel block c) is row 32c + ln,
  // V^T positions 32kb + 16t + 8g .. +7.  Padded tiles: one per-lane base
  // (kaddr, vaddr) plus a constant; swizzled tiles: per-lane offsets kro, vro.
  uint32_t gk[G::KL], gv[PAD ? 1 : G::VL];
  uint32_t kro[PAD ? 1 : NS], vro[PAD ? 1 : 4];
  const uint32_t kaddr = (uint32_t)(ln * G::KSTR + g * 16);
  const uint32_t vaddr = (uint32_t)(ln * G::VSTR + g * 16);
  if constexpr (PAD) {
#pragma unroll
    for (int j = 0; j < G::KL; ++j) gk[j] = chunk_src(j * WAVES + wave, lane, G::KSTR, D * 2, D * 2);
    gv[0] = 16 * lane;
  } else {
#pragma unroll
    for (int j = 0; j < G::KL; ++j) {
      const int c = (j * WAVES + wave) * 64 + lane, krow = c / (D / 8), kp = c % (D / 8);
      gk[j] = (uint32_t)(krow * D + (kp ^ swz_k<D>(krow)) * 8) * 2;
    }
#pragma unroll
    for (int j = 0; j < G::VL; ++j) {
      const int c = (j * WAVES + wave) * 64 + lane, vrow = c / (kBN / 8), vp = c % (kBN / 8);
      gv[j] = (uint32_t)(vrow * kVtRow * 2 + (vp ^ swz_v(vrow)) * 16);
    }
#pragma unroll
    for (int st = 0; st < NS; ++st) kro[st] = (uint32_t)(ln * D + (((2 * st + g) ^ swz_k<D>(ln)) * 8)) * 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) vro[q] = (uint32_t)(ln * kBN * 2 + (((2 * q + g) ^ swz_v(ln)) * 16));
  }
  auto kfrag = [&](const char* Ks, int kb, int st) {
    return *reinterpret_cast<const bf16x8*>(Ks + kb * 32 * G::KSTR +
                                            (PAD ? st * 32 + kaddr : kro[PAD ? 0 : st]));
  };
  auto vfrag = [&](const char* Vs, int kb, int t, int c) {
    return *reinterpret_cast<const bf16x8*>(Vs + c * 32 * G::VSTR +
                                            (PAD ? (4 * kb + 2 * t) * 16 + vaddr : vro[PAD ? 0 : 2 * kb + t]));
  };

  auto load_tile = [&](int kt, int stage) {
    load_tiles<D, WAVES, H>(Kh, Vth, kt, nkl, lds, stage, wave, gk, gv);
  };
  if (ntiles > 0) load_tile(0, 0);  // first tile in flight before anything else

  bf16x8 qf[H][NS];
  float mrow[H], negmu[H], lsum[H];
  floatx16 oacc[H][NC];
#pragma unroll
  for (int h = 0; h < H; ++h) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (qvalid[h]) u = *reinterpret_cast<const uint4*>(Q + qoff[h] + 16 * s + 8 * g);
      qf[h][s] = __builtin_bit_cast(bf16x8, u);
    }
    mrow[h] = FIXED ? (qvalid[h] ? mu[(size_t)bh * Nq + qrow[h]] : 0.f) : -INFINITY;
    negmu[h] = -mrow[h];
    lsum[h] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[h][c][r] = 0.f;
  }
  if (PARTIAL && accumulate) {  // continue the sums of earlier key shards
#pragma unroll
    for (int h = 0; h < H; ++h) {
      if (!qvalid[h]) continue;
      const float* arow = o_acc + qoff[h];
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const float4 t = *reinterpret_cast<const float4*>(arow + c * 32 + 8 * rq + 4 * g);
          oacc[h][c][4 * rq + 0] = t.x;
          oacc[h][c][4 * rq + 1] = t.y;
          oacc[h][c][4 * rq + 2] = t.z;
          oacc[h][c][4 * rq + 3] = t.w;
        }
      if (g == 0) lsum[h] = l_acc[(size_t)bh * Nq + qrow[h]];
    }
  }


  // S^T of one 32-key block for row half h
  auto qk = [&](const char* Ks, int kb, int h) {
    floatx16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      acc = mfma32(kfrag(Ks, kb, s), qf[h][s], acc);
    return acc;
  };
  auto visible = [&](int kt, int kb, int r, int h) {
    const int key = kt + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
    return key < nkl && (!CAUSAL || kv_offset + key <= qrow[h]);
  };
  // bf16 weights of one block packed for the product, and the row sum.  The
  // fixed forms add the fp32 weights, register by register (as the
  // generated two-half code does, so that a one-shard call is bitwise the
  // dense fixed call); the online forms add the rounded weights with v_dot2
  // (which holds the matrix pipeline while it runs, but measured faster in
  // this compiled code than plain adds)
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  auto pack = [&](const float* p, uint32_t* pw, int h) {
    if constexpr (FIXED) {
#pragma unroll
      for (int r = 0; r < 16; ++r) lsum[h] += p[r];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pw[e] = pack_bf16(p[2 * e], p[2 * e + 1]);
      if constexpr (!FIXED)
        lsum[h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[e]), ones, lsum[h], false);
    }
  };
  // O^T += V^T P^T for one 32-key block
  auto pv = [&](const char* Vs, int kb, const uint32_t* pw, int h) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(pw[4 * t], pw[4 * t + 1], pw[4 * t + 2], pw[4 * t + 3]));
#pragma unroll
      for (int c = 0; c < NC; ++c)
        oacc[h][c] = mfma32(vfrag(Vs, kb, t, c), pf, oacc[h][c]);
    }
  };

  auto tile = [&](int it, auto stage_tag, auto mask_tag, bool need_mask) {
    constexpr int ST = decltype(stage_tag)::value;
    constexpr bool MASK = decltype(mask_tag)::value;
    const int kt = it * kBN;
    const char* Ks = lds + G::koff(ST);
    const char* Vs = lds + G::voff(ST);
    if constexpr (FIXED) {
      // no running maximum: x = c s - mu with mu fixed, weights 2^x
      (void)need_mask;
      auto weights = [&](const floatx16& sacc, int kb, int h, uint32_t* pw) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = __builtin_amdgcn_exp2f(fmaf(sacc[r], c2, negmu[h]));
          if constexpr (MASK) p[r] = visible(kt, kb, r, h) ? p[r] : 0.f;
        }
        pack(p, pw, h);
      };
      // (the score products follow the closure above in source order: the
      // other order schedules into 256 VGPRs with spills on hipcc 7.2)
      const floatx16 s0 = qk(Ks, 0, 0);
      const floatx16 s1 = qk(Ks, 1, 0);
      uint32_t pw0[8], pw1[8];
      weights(s0, 0, 0, pw0);
      weights(s1, 1, 0, pw1);
      pv(Vs, 0, pw0, 0);
      pv(Vs, 1, pw1, 0);
    } else {
      const floatx16 s0 = qk(Ks, 0, 0);
      const floatx16 s1 = qk(Ks, 1, 0);
      // online softmax: the tile maximum must be known before any weight,
      // and every weight waits for it (c > 0, so the maximum of c s is c
      // times the maximum of s)
      float x[2][16];
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[0][r] = s0[r];
        x[1][r] = s1[r];
        if (need_mask) {
          x[0][r] = visible(kt, 0, r, 0) ? x[0][r] : -INFINITY;
          x[1][r] = visible(kt, 1, r, 0) ? x[1][r] : -INFINITY;
        }
        tmax = fmaxf(tmax, fmaxf(x[0][r], x[1][r]));
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * c2;
      float msub;
      auto rescale = [&](float alpha) {
        lsum[0] *= alpha;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[0][c][r] *= alpha;
      };
      if constexpr (LAZY) {
        // a row moves its stabilizer only past a growth of kLazyTau; the
        // rescale runs when any row of the wave moved (-inf: no key seen yet)
        const bool grow = tmax > mrow[0] + kLazyTau;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float mnew = grow ? tmax : mrow[0];
          rescale(grow ? __builtin_amdgcn_exp2f(mrow[0] - mnew) : 1.f);
          mrow[0] = mnew;
        }
        msub = (mrow[0] == -INFINITY) ? 0.f : mrow[0];
      } else {
        const float mnew = fmaxf(mrow[0], tmax);
        const bool none = (mnew == -INFINITY);  // no visible key yet
        rescale(none ? 1.f : __builtin_amdgcn_exp2f(mrow[0] - mnew));
        msub = none ? 0.f : mnew;
        mrow[0] = mnew;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[0][r] = __builtin_amdgcn_exp2f(fmaf(x[0][r], c2, -msub));
        x[1][r] = __builtin_amdgcn_exp2f(fmaf(x[1][r], c2, -msub));
      }
      uint32_t pw0[8], pw1[8];
      pack(x[0], pw0, 0);
      pack(x[1], pw1, 0);
      pv(Vs, 0, pw0, 0);
      pv(Vs, 1, pw1, 0);
    }
  };

  auto step = [&](int it, auto stage_tag) {
    constexpr int ST = decltype(stage_tag)::value;
    const int kt = it * kBN;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile `it` is in LDS; nobody still reads the other stage
    if (it + 1 < ntiles) load_tile(kt + kBN, ST ^ 1);
    const bool need_mask = (kt + kBN > nkl) || (CAUSAL && kv_offset + kt + kBN - 1 > row0);
    if constexpr (FIXED) {
      // one straight-line body per mask case
      if (need_mask) tile(it, stage_tag, std::true_type{}, true);
      else tile(it, stage_tag, std::false_type{}, false);
    } else {
      tile(it, stage_tag, std::false_type{}, need_mask);
    }
  };

  // Tiles this wave computes.  Under the causal mask the last ones of the
  // workgroup can lie wholly above this wave's rows; the wave still takes part
  // in their barriers and loads, in a loop of its own after the compute loop
  // (a skip inside the compute loop makes hipcc copy the output accumulators
  // at every tile).
  int nt_wave = ntiles;
  if constexpr (CAUSAL) {
    const int x = row0 + 32 * H - kv_offset;  // local keys up to this wave's last row, plus one
    nt_wave = x <= 0 ? 0 : min(ntiles, (x + kBN - 1) / kBN);
  }
  if constexpr (H == 1) {
    for (int it = 0; it < nt_wave; it += 2) {
      step(it, std::integral_constant<int, 0>{});
      if (it + 1 < nt_wave) step(it + 1, std::integral_constant<int, 1>{});
    }
  } else {
    // Two row halves per wave: the tile work is generated asm (tile_h2.inc),
    // one site, so the output accumulators stay in the same AGPRs throughout.
    // Waves w and w + WAVES/2 share a SIMD.  Both run the chain
    //   qk0 sm0 pv0 qk1 sm1 pv1 | qk0 ... (scores, weights, products of the
    //   two 32-key blocks of each tile)
    // but the window between two barriers starts at a different point of it:
    //   first wave:  pv1(t-1) qk0 sm0 pv0 qk1 sm1
    //   second wave: sm1(t-1) pv1(t-1) qk0 sm0 pv0 qk1
    // so that the one's weights (VALU only) overlap the other's products.
    // Window t reads tiles t-1 and t while tile t+1 loads: three LDS stages.
    // The scores / packed weights of the part in flight stay in v82..v113
    // from one window to the next.
    static_assert(D == 128, "the two-half tile body is generated for d = 128");
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)lds;
    const int pair = wave >= WAVES / 2 ? 1 : 0;
    floatx16 sc0 = {}, sc1 = {};
    // a masked tile keeps the weight of (block kb, register r) of half h iff
    // the key index 32kb + 8(r/4) + 4g + (r%4) from the tile start is below
    // lim_h + 4g: the tile's keys below Nk, and under the causal mask those up
    // to the row's own index.  lim_h drops by 64 a tile, so tile t - 1's
    // limits are lim_h + 64.  Without the causal mask both halves share one.
    int lim0 = nkl, lim1 = nkl;
    if constexpr (CAUSAL) {
      lim0 = min(lim0, qrow[0] - kv_offset + 1);
      lim1 = min(lim1, qrow[H - 1] - kv_offset + 1);
    }
    lim0 -= 4 * g;
    lim1 -= 4 * g;
    int st = 0;  // stage of tile w
    // the wave's share of each tile's loads, issued from inside the asm
    // between its products (see gen_tile_h2.py): key rows 8w .. 8w + 7 and
    // V^T chunks w, w + 8, w + 16
    static_assert(WAVES == 8 && kBN / WAVES == 8 && G::VCH == 18, "the generated loads' shares");
    const uint32_t l4k = 4 * lane + 8 * wave * D * 2, l16 = 16 * lane + 1024 * wave;
    for (int w = 0; w <= ntiles; ++w) {
      const int kt = w * kBN, pst = st == 0 ? 2 : st - 1, nst = st == 2 ? 0 : st + 1;
      if (w < ntiles) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // tile w is in LDS; nobody still reads tile w - 2
      }
      {
        // tile w + 1 into stage nst, if there is one (nld: which loads the
        // wave issues: 0 none, 2 all but a third V^T chunk, 3 all)
        const int nld = __builtin_amdgcn_readfirstlane(w + 1 < ntiles ? (wave < G::VCH - 2 * WAVES ? 3 : 2) : 0);
        const u32x4 rk = buffer_words(Kh + (size_t)(kt + kBN) * D * 2, (uint32_t)max(0, min(nkl - kt - kBN, kBN)) * D * 2);
        const u32x4 rv = buffer_words(Vth + (size_t)(w + 1) * G::VTILE_G, (uint32_t)G::VTILE_G);
        const uint32_t kdst = __builtin_amdgcn_readfirstlane(lds_base + G::koff(nst) + 8 * wave * G::KSTR);
        const uint32_t vdst = __builtin_amdgcn_readfirstlane(lds_base + G::voff(nst) + 1024 * wave);
        // variant: 0/1 a whole window, 2/3 the first tile's, 4/5 the drain
        // after this wave's last tile (first / second wave of the pair), 6
        // only the loads (past the drain).  The asm runs every window, so the
        // compiler sees one straight path for the accumulators.
        const int kind = __builtin_amdgcn_readfirstlane(
            (w > nt_wave || nt_wave == 0) ? 6 : (w == 0 ? 2 : w < nt_wave ? 0 : 4) + pair);
        // wave-uniform scalars of the asm block, in SGPRs
        const uint32_t ks = __builtin_amdgcn_readfirstlane(lds_base + G::koff(st));
        const uint32_t vs = __builtin_amdgcn_readfirstlane(lds_base + G::voff(st));
        const uint32_t vsp = __builtin_amdgcn_readfirstlane(lds_base + G::voff(pst));
        // mask flags of tiles w and w - 1
        const int mf = __builtin_amdgcn_readfirstlane(
            ((kt + kBN > nkl) || (CAUSAL && kv_offset + kt + kBN - 1 > row0)) ? 1 : 0);
        const int mfp = __builtin_amdgcn_readfirstlane(
            ((kt > nkl) || (CAUSAL && kv_offset + kt - 1 > row0)) ? 1 : 0);
        asm volatile(CLIS_TILE_H2_WINDOW
                     : [o00] "+a"(oacc[0][0]), [o01] "+a"(oacc[0][1]), [o02] "+a"(oacc[0][2]), [o03] "+a"(oacc[0][3]),
                       [o10] "+a"(oacc[H - 1][0]), [o11] "+a"(oacc[H - 1][1]), [o12] "+a"(oacc[H - 1][2]),
                       [o13] "+a"(oacc[H - 1][3]), [l0] "+v"(lsum[0]), [l1] "+v"(lsum[H - 1]),
                       [sc0] "+{v[82:97]}"(sc0), [sc1] "+{v[98:113]}"(sc1)
                     : [q00] "v"(qf[0][0]), [q01] "v"(qf[0][1]), [q02] "v"(qf[0][2]), [q03] "v"(qf[0][3]),
                       [q04] "v"(qf[0][4]), [q05] "v"(qf[0][5]), [q06] "v"(qf[0][6]), [q07] "v"(qf[0][7]),
                       [q10] "v"(qf[H - 1][0]), [q11] "v"(qf[H - 1][1]), [q12] "v"(qf[H - 1][2]),
                       [q13] "v"(qf[H - 1][3]), [q14] "v"(qf[H - 1][4]), [q15] "v"(qf[H - 1][5]),
                       [q16] "v"(qf[H - 1][6]), [q17] "v"(qf[H - 1][7]), [nm0] "v"(negmu[0]),
                       [nm1] "v"(negmu[H - 1]), [kad] "v"(kaddr), [vad] "v"(vaddr), [ks] "s"(ks), [vs] "s"(vs),
                       [vsp] "s"(vsp), [c2] "s"(c2), [mf] "s"(mf), [mfp] "s"(mfp), [kind] "s"(kind),
                       [lim0] "v"(lim0), [lim1] "v"(CAUSAL ? lim1 : lim0), [rk] "s"(rk), [rv] "s"(rv),
                       [kdst] "s"(kdst), [vdst] "s"(vdst), [l4k] "v"(l4k), [l16] "v"(l16), [nld] "s"(nld)
                     : CLIS_TILE_H2_CLOBBERS);
      }
      st = nst;
      lim0 -= kBN;
      lim1 -= kBN;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the last (empty) loads have landed
    // The rows' indices again, from a lane id the compiler cannot reuse from
    // before the loop (keeping them would cost registers in it)
    set_rows(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
  }
  if constexpr (CAUSAL && H == 1) {
    for (int it = nt_wave; it < ntiles; ++it) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (it + 1 < ntiles) load_tile((it + 1) * kBN, (it + 1) & 1);
    }
  }

  // ---- epilogue: the row sum's two lane halves meet, then O = O_acc / l
#pragma unroll
  for (int h = 0; h < H; ++h) lsum[h] += __shfl_xor(lsum[h], 32);
  if (TAIL && split >= 0) {  // one key split: unnormalized sums for tail_combine
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const int r = wave * 32 * H + 32 * h + ln;  // row within the workgroup
      float* arow = tail_o + ((size_t)split * kTailRows + r) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          *reinterpret_cast<float4*>(arow + c * 32 + 8 * rq + 4 * g) = make_float4(
              oacc[h][c][4 * rq], oacc[h][c][4 * rq + 1], oacc[h][c][4 * rq + 2], oacc[h][c][4 * rq + 3]);
      if (g == 0) tail_l[(size_t)split * kTailRows + r] = lsum[h];
    }
    return;
  }
  if constexpr (PARTIAL) {  // key shard: the unnormalized sums
#pragma unroll
    for (int h = 0; h < H; ++h) {
      if (!qvalid[h]) continue;
      float* arow = o_acc + qoff[h];
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          *reinterpret_cast<float4*>(arow + c * 32 + 8 * rq + 4 * g) = make_float4(
              oacc[h][c][4 * rq], oacc[h][c][4 * rq + 1], oacc[h][c][4 * rq + 2], oacc[h][c][4 * rq + 3]);
      if (g == 0) l_acc[(size_t)bh * Nq + qrow[h]] = lsum[h];
    }
    return;
  }
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const float inv = 1.f / lsum[h];
    if (qvalid[h] && lse && g == 0)
      lse[(size_t)bh * Nq + qrow[h]] = kLn2 * ((FIXED ? -negmu[h] : mrow[h]) + log2f(lsum[h]));
    if (qvalid[h]) {
      uint16_t* orow = O + qoff[h];
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          uint2 w;
          w.x = pack_bf16(oacc[h][c][4 * rq + 0] * inv, oacc[h][c][4 * rq + 1] * inv);
          w.y = pack_bf16(oacc[h][c][4 * rq + 2] * inv, oacc[h][c][4 * rq + 3] * inv);
          *reinterpret_cast<uint2*>(orow + c * 32 + 8 * rq + 4 * g) = w;
        }
    }
  }
}

// Finishes the pool's key splits: the kMaxSplit parts of the t-th split item
// (the last query tile of list slot t) are summed in split order, then
// O = sum o / sum l (and the log-sum-exp when asked), for the rows that
// exist.  Workgroup t * (BM / kCombineRows) + c takes rows c * kCombineRows ...
// of item t; 256 threads, each 4 channels of one row per pass.
constexpr int kCombineRows = 32;

template <int D, int BM>
__global__ void __launch_bounds__(256)
tail_combine(const float* __restrict__ tail_o, const float* __restrict__ tail_l, uint16_t* __restrict__ O,
             const float* __restrict__ mu, float* __restrict__ lse, const int32_t* __restrict__ head_list,
             const int32_t* __restrict__ split_heads, int n_slots, int Nq) {
  constexpr int GROUPS = D / 4, ROWS = 256 / GROUPS;  // rows per pass
  constexpr int CHUNKS = BM / kCombineRows;
  static_assert(BM % kCombineRows == 0 && kCombineRows % ROWS == 0, "whole passes per chunk");
  const int n_qt = (Nq + BM - 1) / BM;
  const int S = split_heads ? *split_heads : head_list ? 0 : min(n_slots, kSplitHeads);
  const int t = blockIdx.x / CHUNKS, chunk = blockIdx.x % CHUNKS;
  if (t >= S) return;
  const int slot = t, qt = n_qt - 1;
  const int bh = head_list ? head_list[slot] : slot;
  const int cg = threadIdx.x % GROUPS, r0 = threadIdx.x / GROUPS;
  for (int r = chunk * kCombineRows + r0; r < (chunk + 1) * kCombineRows; r += ROWS) {
    const int qrow = qt * BM + r;
    if (qrow >= Nq) break;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float l = 0.f;
    for (int s = 0; s < kMaxSplit; ++s) {
      const size_t part = (size_t)(t * kMaxSplit + s) * kTailRows + r;
      const float4 a = *reinterpret_cast<const float4*>(tail_o + part * D + 4 * cg);
      acc.x += a.x; acc.y += a.y; acc.z += a.z; acc.w += a.w;
      l += tail_l[part];
    }
    const float inv = 1.f / l;
    const size_t row = (size_t)bh * Nq + qrow;
    uint2 w;
    w.x = pack_bf16(acc.x * inv, acc.y * inv);
    w.y = pack_bf16(acc.z * inv, acc.w * inv);
    *reinterpret_cast<uint2*>(O + row * D + 4 * cg) = w;
    if (lse && cg == 0) lse[row] = kLn2 * (mu[row] + log2f(l));
  }
}

// Compute units of the current device (cached per device; 0 if unknown).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D, bool FIXED, bool CAUSAL, bool PARTIAL = false, bool LAZY = false>
hipError_t launch_t(const AttnArgs& a, const uint16_t* vt, int nk_pad, hipStream_t s) {
  constexpr int WAVES = FIXED ? (CAUSAL ? CLIS_FIXED_CAUSAL_WAVES : CLIS_FIXED_WAVES) : CLIS_ONLINE_WAVES;
  constexpr int H = (FIXED && D == 128) ? (CAUSAL ? CLIS_FIXED_CAUSAL_HALVES : CLIS_FIXED_HALVES) : 1;
  using G = Geo<D, WAVES, H>;
  const int n_qt = (a.Nq + G::BM - 1) / G::BM;
  // pooled work of the dense forms (file comment): conc workgroups are
  // resident at a time; the pool's workgroups follow the others and exit once
  // it is empty.  The causal forms keep their static order: claims from all
  // XCDs interleave and would undo its balance across shader engines.
  constexpr bool TAIL = FIXED && !PARTIAL && !CAUSAL;
  const bool splits = TAIL && a.tail_o;
  const int conc = (!PARTIAL && !CAUSAL && a.sched) ? min(cu_count(), kPoolWorkers) * (WAVES >= 8 ? 1 : 2) : 0;
  long long blocks = (long long)n_qt * a.n_slots;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (conc > 0) {
    // Pool workgroups.  With active <= blocks items of which S are split, the
    // first F = active - S - P1 workgroups run whole items and the rest claim
    // from P1 + S * kMaxSplit entries, so blocks + (kMaxSplit - 1) * Smax
    // workgroups cover every entry for any active and S <= Smax =
    // min(n_slots, kSplitHeads), with P1 <= pmax = min(blocks, max(conc - 1,
    // blocks / CLIS_POOL_DIV)).  CLIS_POOL_OVER percent more of every entry's
    // worth lets faster XCDs claim more.
    const long long div = CLIS_POOL_DIV > 0 ? blocks / CLIS_POOL_DIV : 0;
    const long long pmax = std::min<long long>(blocks, std::max<long long>(conc - 1, div));
    const long long smax = splits ? std::min<long long>(a.n_slots, kSplitHeads) : 0;
    blocks += (kMaxSplit - 1) * smax + (pmax + kMaxSplit * smax) * CLIS_POOL_OVER / 100;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  }
  attn_fwd_bf16<D, FIXED, CAUSAL, WAVES, PARTIAL, LAZY, H><<<(unsigned)blocks, G::THREADS, 0, s>>>(
      static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k), vt, static_cast<uint16_t*>(a.o),
      a.mu, a.head_list, a.head_count, a.n_slots, a.Nq, a.Nk, nk_pad, a.c2, a.lse, a.o_acc, a.l_acc,
      a.accumulate, a.kv_offset, a.tail_o, a.tail_l, conc, conc > 0 ? a.sched : nullptr, a.split_heads);
  if constexpr (TAIL) {
    if (conc > 0 && splits) {  // workgroups for every row chunk of every possible split item
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      tail_combine<D, G::BM><<<(unsigned)(kSplitHeads * (G::BM / kCombineRows)), 256, 0, s>>>(
          a.tail_o, a.tail_l, static_cast<uint16_t*>(a.o), a.mu, a.lse, a.head_list, a.split_heads, a.n_slots,
          a.Nq);
    }
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, bool fixed, const uint16_t* vt, int nk_pad, hipStream_t s) {
  if (a.o_acc) {  // key shard
    if (!fixed) return hipErrorInvalidValue;
    return a.causal ? launch_t<D, true, true, true>(a, vt, nk_pad, s) : launch_t<D, true, false, true>(a, vt, nk_pad, s);
  }
  if (fixed) return a.causal ? launch_t<D, true, true>(a, vt, nk_pad, s) : launch_t<D, true, false>(a, vt, nk_pad, s);
  if (a.lazy)
    return a.causal ? launch_t<D, false, true, false, true>(a, vt, nk_pad, s)
                    : launch_t<D, false, false, false, true>(a, vt, nk_pad, s);
  return a.causal ? launch_t<D, false, true>(a, vt, nk_pad, s) : launch_t<D, false, false>(a, vt, nk_pad, s);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, bool fixed, const void* vt, hipStream_t s) {
  const int nk_pad = vt_pad(a.Nk);
  const uint16_t* v = static_cast<const uint16_t*>(vt);
  if (a.d == 128) return launch_d<128>(a, fixed, v, nk_pad, s);
  if (a.d == 64) return launch_d<64>(a, fixed, v, nk_pad, s);
  return hipErrorInvalidValue;
}

}  // namespace clis
