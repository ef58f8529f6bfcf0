// internal.h -- kernel launchers and workspace layout shared by the library's
// translation units (not part of the public ABI; see include/clis.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "clis.h"

namespace clis {

// log2(e) in fp64; the exp2 arguments of the kernels are c = scale * log2(e)
// times a dot product, so that exp2 (the gfx950 v_exp_f32) replaces exp.
constexpr double kLog2e = 1.442695040888963407359924681001892137;

// Rows of one head handled by one certification block: heads are split so
// that a launch has enough blocks to cover the chip (the split counts are a
// pure function of the shape, so the workspace size is too).
inline int cert_splits(int n) {
  int s = (n + 1023) / 1024;
  return s < 1 ? 1 : (s > 64 ? 64 : s);
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Byte offsets of every region inside the caller's workspace.
struct WsLayout {
  size_t ksum_part;  // [BH][Sk][d] fp64   partial key column sums
  size_t vmax_part;  // [BH][Sk]    fp64   partial max |V|
  size_t kap_part;   // [BH][Sk]    fp64   partial max ||k - kbar||^2
  size_t qss_part;   // [BH][Sq]    fp64   partial max ||q||^2
  size_t kbar;       // [BH][d]     fp64
  size_t stats;      // [BH]        clis_head_stats_t
  size_t mu;         // [BH][Nq]    fp32   stabilizers when the caller gave none
  size_t cert;       // [BH]        int32
  size_t lists;      // [2][BH]     int32  heads routed fixed / online
  size_t counts;     // [8]         int32  list lengths, work counters, split heads
  size_t vt;         // [BH][Nk_pad / 64][d][kVtRow] bf16  V^T tiles for the bf16 attention kernels
  size_t vmax_blk;   // [BH][vt_pad(Nk) / 64] fp32  max |V| per 64-key block, from the V transpose
  size_t tail_o;     // [kTailSlots][kTailRows][d] fp32  key-split partial sums of the pool
  size_t tail_l;     // [kTailSlots][kTailRows]    fp32
  size_t total;
};

// Key splits at the end of the fixed kernel's pool of work items: at most
// kTailSlots splits of kTailRows query rows each; kPoolWorkers caps the
// workgroups resident at once that the pool is sized for.  The items cut into
// kTailSplits key splits are the last query tiles of the heads with index
// below kSplitHeads that the kernel runs: a function of the head alone, so a
// head's result does not depend on which other heads are routed with it.
constexpr int kTailSlots = 128;
constexpr int kTailRows = 512;
constexpr int kPoolWorkers = 256;
constexpr int kTailSplits = 8;
constexpr int kSplitHeads = kTailSlots / kTailSplits;

// Keys of the V^T copy, padded to whole 128-key tiles (either tile size).
inline int vt_pad(int Nk) { return (Nk + 127) / 128 * 128; }
// The V^T copy is stored as 64-key tiles, each d rows (channels) of kVtRow
// bf16: the tile's 64 keys, then 8 zeros.  A tile is then one contiguous
// block laid out exactly as the kernels keep it in LDS.
constexpr int kVtRow = 72;
inline size_t vt_bytes(int BH, int Nk, int d) { return (size_t)BH * (vt_pad(Nk) / 64) * d * kVtRow * 2; }

inline WsLayout ws_layout(int B, int H, int Nq, int Nk, int d) {
  const size_t BH = (size_t)B * H, Sk = cert_splits(Nk), Sq = cert_splits(Nq);
  WsLayout w{};
  size_t o = 0;
  w.ksum_part = o; o = align256(o + BH * Sk * d * sizeof(double));
  w.vmax_part = o; o = align256(o + BH * Sk * sizeof(double));
  w.kap_part = o;  o = align256(o + BH * Sk * sizeof(double));
  w.qss_part = o;  o = align256(o + BH * Sq * sizeof(double));
  w.kbar = o;      o = align256(o + BH * d * sizeof(double));
  w.stats = o;     o = align256(o + BH * sizeof(clis_head_stats_t));
  w.mu = o;        o = align256(o + BH * (size_t)Nq * sizeof(float));
  w.cert = o;      o = align256(o + BH * sizeof(int32_t));
  w.lists = o;     o = align256(o + 2 * BH * sizeof(int32_t));
  w.counts = o;    o = align256(o + 8 * sizeof(int32_t));
  w.vt = o;        o = align256(o + vt_bytes((int)BH, Nk, d));
  w.vmax_blk = o;  o = align256(o + BH * (size_t)(vt_pad(Nk) / 64) * sizeof(float));
  w.tail_o = o;    o = align256(o + (size_t)kTailSlots * kTailRows * d * sizeof(float));
  w.tail_l = o;    o = align256(o + (size_t)kTailSlots * kTailRows * sizeof(float));
  w.total = o;
  return w;
}

struct CertifyArgs {
  const void* q; const void* k; const void* v;
  int B, H, Nq, Nk, d;
  float scale;
  int dtype;
  float* mu;                 // [BH][Nq]
  int32_t* cert;             // [BH]
  clis_head_stats_t* stats;  // [BH] (never NULL here: workspace copy if the caller gave none)
  double* kbar;              // [BH][d]
  double* ksum_part; double* vmax_part; double* kap_part; double* qss_part;
  // If set: max |V| per 64-key block, already computed by the V transpose
  // (vmax_nblk blocks per head); certification then does not read V.
  const float* vmax_blk = nullptr;
  int vmax_nblk = 0;
};

hipError_t launch_certify(const CertifyArgs& a, hipStream_t s);

// Builds the fixed / online head lists from cert and mode (one tiny kernel);
// counts[0..1] receive the list lengths, counts[2..3] (work counters) zero,
// counts[4] the number of fixed-routed heads with index < kSplitHeads.
hipError_t launch_route(const int32_t* cert, int mode, int BH, int32_t* lists, int32_t* counts,
                        int32_t* route_out, hipStream_t s);

struct AttnArgs {
  const void* q; const void* k; const void* v; void* o;
  const float* mu;            // fixed path only
  const int32_t* head_list;   // NULL: every head, in order
  const int32_t* head_count;  // device count of head_list entries
  int n_slots;                // heads the grid covers (B*H)
  int Nq, Nk, d;
  float c2;                   // scale * log2(e), rounded to fp32
  int causal;
  float* lse = nullptr;       // [BH][Nq] natural-log row log-sum-exp, or NULL
  // Key-shard form (fixed path): unnormalized fp32 sums instead of O.
  float* o_acc = nullptr;     // [BH][Nq][d], or NULL for the normal output
  float* l_acc = nullptr;     // [BH][Nq]
  int accumulate = 0;         // 1: add to o_acc / l_acc; 0: overwrite them
  int kv_offset = 0;          // global index of key 0 (causal mask)
  int lazy = 0;               // online path: conditional (lazy) rescaling
  // Last-round key splits (dense fixed path): workspace for the partial sums.
  float* tail_o = nullptr;    // [kTailSlots][kTailRows][d], or NULL: no splits
  float* tail_l = nullptr;    // [kTailSlots][kTailRows]
  int* sched = nullptr;       // pool counter, zero at launch, or NULL: no pool
  const int32_t* split_heads = nullptr;  // device count of listed heads < kSplitHeads
  // fp32 kernel only (it takes no head list): if cert is set, each head runs
  // fixed when cert[head] != 0 and online otherwise (auto mode); route_out
  // (or NULL) receives 1 for a fixed head, 0 for an online one.
  const int32_t* cert = nullptr;
  int32_t* route_out = nullptr;
};

// bf16 kernels: V is read through a transposed copy [BH][vt_pad(Nk) / 64]
// [d][kVtRow] that launch_transpose_v writes.
// vmax_blk (or NULL): also writes max |V| of every 64-key block, [BH][vt_pad(Nk) / 64].
hipError_t launch_transpose_v(const void* v, void* vt, int BH, int Nk, int d, hipStream_t s,
                              float* vmax_blk = nullptr);
hipError_t launch_attn_bf16(const AttnArgs& a, bool fixed, const void* vt, hipStream_t s);
// fp32 kernel: every head of the grid (no head list); routes as AttnArgs::cert
// says, else fixed or online as `fixed` says.
hipError_t launch_attn_fp32(const AttnArgs& a, bool fixed, hipStream_t s);

// O = o_acc / l (bf16 or fp32), and lse = ln 2 (mu + log2 l) if lse is set.
hipError_t launch_combine(const float* o_acc, const float* l_acc, void* o, int dtype_bf16, const float* mu,
                          float* lse, long long rows, int d, hipStream_t s);

}  // namespace clis
