/*
 * clis.h -- C ABI of the CLiS attention-forward library for AMD MI355X (gfx950).
 *
 * CLiS (Certified Loop-invariant Stabilization) is described on the pages
 * "CLiS: Plug-and-Play Attention Acceleration for Video Diffusion on TPUs via
 * Certified Stabilization" (cited below as [CLiS ...]).  Per the abstract, it
 * fixes each query row's softmax stabilizer before the key/value loop, so the
 * loop needs no running maximum and no accumulator rescaling; it certifies
 * per head that this is numerically safe, and heads that fail fall back to
 * online softmax.  The output is ordinary softmax attention
 *     O = softmax(scale * Q K^T [+ causal mask]) V
 * so the library drops in where a fused attention forward was called.
 *
 * Layout.  Q [B, H, Nq, d], K and V [B, H, Nk, d], O [B, H, Nq, d]: dense,
 * row-major, d innermost, one element type for all four (bf16 or fp32).
 * Stabilizers mu [B, H, Nq] fp32, flags cert and routes [B, H] int32.
 *
 * Ownership.  The caller owns every buffer.  All pointers except `stream`
 * are DEVICE pointers; q, k, v, o, o_acc must be 16-byte aligned, ws
 * 256-byte aligned, stats and kbar 8-byte aligned, and the other fp32 and
 * int32 arrays 4-byte aligned.  The library never allocates or frees memory;
 * scratch space comes from the caller's workspace `ws` of at least
 * clis_workspace_bytes(...) bytes.  `stream` is a hipStream_t passed as void*
 * (NULL: the null stream).
 *
 * Execution.  Every call only enqueues kernels on `stream` and returns; there
 * is no host synchronisation and no device-to-host copy, also in auto mode,
 * where each head's route is read on the device.  Results are valid once the
 * stream has reached them, and are bitwise reproducible run to run (fixed
 * reduction orders, no floating-point atomics).  Calls on distinct streams
 * may overlap if their workspaces and outputs are disjoint.
 *
 * Errors.  Every entry point returns a clis_status_t.  A nonzero status means
 * nothing was enqueued (except CLIS_ERR_HIP, which reports a failed launch);
 * clis_last_error() then gives a thread-local description.  No C++ exception
 * or abort crosses the ABI.
 *
 * Shapes.  d must be 64 or 128.  B, H, Nq may be 0 (nothing is enqueued and
 * CLIS_OK is returned); a call with at least one query row needs Nk >= 1.
 * causal needs Nq == Nk (query i sees keys 0..i), except for key shards
 * (clis_attn_fwd_partial).  scale must be finite and
 * > 0.  Every dimension must fit in int32, B*H*N*d in int64, and one head's
 * keys must span less than 2 GiB (d * Nk * 2 bytes, Nk rounded up to 128).
 */
#ifndef CLIS_H
#define CLIS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { CLIS_BF16 = 0, CLIS_FP32 = 1 } clis_dtype_t;

/* How clis_attn_fwd picks each head's kernel [CLiS abstract]. */
typedef enum {
  CLIS_MODE_AUTO = 0,   /* certified heads: fixed stabilizer; the rest: online softmax */
  CLIS_MODE_FIXED = 1,  /* every head on the fixed-stabilizer kernel (testing tool: an
                           uncertified head may overflow to Inf/NaN) */
  CLIS_MODE_ONLINE = 2,  /* every head on the online-softmax kernel */
  CLIS_MODE_ONLINE_LAZY = 3  /* every head on online softmax with conditional rescaling: the
                                stabilizer in use moves, and the accumulators are rescaled, only
                                when a row's tile maximum exceeds it by more than 8 (log2 units),
                                as FlashAttention-4 does (a comparator the CLiS pages name) */
} clis_mode_t;

typedef enum {
  CLIS_OK = 0,
  CLIS_ERR_NULL = 1,        /* a required pointer is NULL */
  CLIS_ERR_SHAPE = 2,       /* bad dimension, scale, or causal with Nq != Nk */
  CLIS_ERR_UNSUPPORTED = 3, /* d not in {64, 128}, or unknown dtype / mode */
  CLIS_ERR_ALIGN = 4,       /* a pointer below its alignment (see Ownership) */
  CLIS_ERR_WORKSPACE = 5,   /* ws missing or smaller than clis_workspace_bytes() */
  CLIS_ERR_HIP = 6          /* a HIP launch failed; see clis_last_error() */
} clis_status_t;

/* Per-head certification record, the quantities of [CLiS Algorithm 1]. */
typedef struct {
  double kappa;     /* step 3: max_r ||k_r - kbar||_2, fp64 */
  double qnorm_max; /* max_r ||q_r||_2, fp64 */
  double bound;     /* step 4: B_h = scale*log2(e) * qnorm_max * kappa */
  double maxabs_v;  /* step 5: max |V| over the head */
  int32_t G;        /* step 5: ceil(log2 max(1, maxabs_v)); 128 if non-finite */
  int32_t L;        /* step 6: ceil(log2 Nk) */
  int32_t A;        /* step 6: L + G */
  int32_t C;        /* step 7: 127 - A */
  int32_t cert;     /* 1 iff bound is finite and bound <= C */
  int32_t reserved;
} clis_head_stats_t;

/* Workspace bytes any entry point of this library needs for these shapes, a
 * pure function of them (256 if any is <= 0):
 *   - certification scratch, stabilizers, flags and route lists (small);
 *   - a transposed copy of V for the bf16 attention kernels (about the size
 *     of V, keys rounded up to 128) and its max |V| per 64 keys;
 *   - fp32 partial sums for the fixed kernel's last-round key splits:
 *     256 x 256 rows x (d + 1) floats, about 32 MiB at d = 128. */
size_t clis_workspace_bytes(int B, int H, int Nq, int Nk, int d);

/*
 * Certify every (b, h) head and compute its fixed stabilizers
 * [CLiS Algorithm 1, steps 1-7; abstract].  Per head, in fp64 with fixed
 * reduction orders:
 *   kbar = mean of the key rows;  kappa = max_r ||k_r - kbar||_2;
 *   B_h = scale*log2(e) * max_r ||q_r||_2 * kappa  (Cauchy-Schwarz bound on
 *         every exp2 argument scale*log2(e) * q.(k - kbar));
 *   G = ceil(log2 max(1, max|V|)),  A = ceil(log2 Nk) + G,  C = 127 - A
 *   (the exp2 and fp32-accumulator limits of [CLiS Figure 3]: floor(U_exp)
 *   = 127 and ceil(U_acc - A) - 1 = 127 - A for fp32/bf16);
 *   cert = B_h finite and B_h <= C;
 *   mu_r = scale*log2(e) * (q_r . kbar), rounded to fp32 (log2 units).
 * Inputs containing Inf or NaN make the head uncertified.
 *   q, k, v    device inputs, layout above; dtype clis_dtype_t.
 *   mu_out     device [B, H, Nq] fp32, required.
 *   cert_out   device [B, H] int32, required (1 certified, 0 not).
 *   stats_out  device [B, H] clis_head_stats_t, or NULL.
 *   kbar_out   device [B, H, d] fp64, or NULL.
 *   ws         device workspace of ws_bytes >= clis_workspace_bytes().
 */
int clis_certify(const void* q, const void* k, const void* v,
                 int B, int H, int Nq, int Nk, int d, float scale, int dtype,
                 float* mu_out, int32_t* cert_out, clis_head_stats_t* stats_out,
                 double* kbar_out, void* ws, size_t ws_bytes, void* stream);

/*
 * CLiS attention forward [CLiS abstract; Figure 5(a)].  Heads routed to the
 * fixed path evaluate, with no running maximum and no rescaling,
 *   o_i = sum_j 2^{x_ij} v_j / sum_j 2^{x_ij},
 *   x_ij = scale*log2(e) * (q_i . k_j) - mu_i,
 * which equals softmax attention exactly in real arithmetic; heads routed to
 * the online path run online softmax (the kernel of online_attn_fwd).
 *   o          device output [B, H, Nq, d], same dtype as the inputs.
 *   mode       clis_mode_t.
 *   mu, cert   device results of clis_certify for these inputs, or NULL: if
 *              the mode needs them (auto: both, fixed: mu) and either is NULL,
 *              certification runs first inside this call, into ws.
 *   route_out  device [B, H] int32 (1 fixed, 0 online), or NULL.
 *   lse_out    device [B, H, Nq] fp32, or NULL: each row's log-sum-exp
 *              ln sum_j exp(scale * q_i . k_j) over its visible keys (natural
 *              log), the statistic a backward pass of fused attention needs.
 *              The fixed path gets it as ln 2 * (mu_i + log2 l_i) from its
 *              row sum l_i, the online path as ln 2 * (m_i + log2 l_i) from its
 *              final running maximum; no extra pass over the keys.
 *   ws         device workspace (clis_workspace_bytes()); may be NULL only if
 *              mode is online or online_lazy, dtype is fp32 and route_out is
 *              NULL.
 * Output dtype equals input dtype: fp32 accumulation, bf16 stored with round
 * to nearest even; on the bf16 path the exp2 weights are rounded to bf16
 * (nearest even) before the P.V product; the row sums (hence lse) add the
 * fp32 weights on the fixed path and the rounded weights on the online path.
 * fp32 inputs run one kernel that takes each head's route from cert itself.
 */
int clis_attn_fwd(const void* q, const void* k, const void* v, void* o,
                  int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                  int mode, const float* mu, const int32_t* cert, int32_t* route_out,
                  float* lse_out, void* ws, size_t ws_bytes, void* stream);

/* Bytes of the device scratch that clis_attn_fwd_noalloc uses: 128 MiB. */
#define CLIS_NOALLOC_SCRATCH_BYTES (128u << 20)

/*
 * clis_attn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation, arguments and results as clis_attn_fwd, bitwise,
 * without the ws / ws_bytes arguments.  Its scratch is a static device array
 * of CLIS_NOALLOC_SCRATCH_BYTES inside this library, one copy per GPU, held
 * until the process ends; its address is looked up on the first call on each
 * device.  No allocation happens in this call.
 *   Limit: shapes whose clis_workspace_bytes(B, H, Nq, Nk, d) exceeds
 *   CLIS_NOALLOC_SCRATCH_BYTES are rejected with CLIS_ERR_WORKSPACE (nothing
 *   enqueued), e.g. B*H*Nk up to about 350,000 keys at d = 128 with bf16.
 *   Concurrency: every call on one GPU shares that GPU's scratch, which keeps
 *   the last call's contents (each call writes everything it reads before
 *   reading it).  Calls that overlap on one GPU -- on different streams or
 *   from different threads without ordering -- race and must not be issued.
 */
int clis_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                          int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                          int mode, const float* mu, const int32_t* cert, int32_t* route_out,
                          float* lse_out, void* stream);

/*
 * Online-softmax attention forward for every head: the tuned baseline and the
 * fallback path [CLiS abstract: running row maxima and accumulator
 * rescaling].  Per key tile: m' = max(m, tile max of c*s), alpha = 2^{m-m'},
 * l = alpha*l + sum 2^{c*s-m'}, O = alpha*O + P.V.  Bitwise equal to
 * clis_attn_fwd with CLIS_MODE_ONLINE (lse_out as there, or NULL).  The bf16
 * kernels read V through a transposed copy kept in ws (clis_workspace_bytes());
 * ws may be NULL for fp32.
 */
int online_attn_fwd(const void* q, const void* k, const void* v, void* o,
                    int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                    float* lse_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Key-sharded attention with a fixed stabilizer [CLiS Figure 5(a)]: with mu_i
 * fixed for the whole key loop, the unnormalized sums of disjoint key ranges
 *   o_acc_i = sum_j 2^{x_ij} v_j,   l_i = sum_j 2^{x_ij},
 *   x_ij = scale*log2(e) * (q_i . k_j) - mu_i,
 * simply add, with no max or rescale merge.  One call processes one shard of
 * keys (k, v are [B, H, Nk, d] holding global keys kv_offset .. kv_offset+Nk-1)
 * against all queries:
 *   mu          device [B, H, Nq] fp32 stabilizers, required: from
 *               clis_certify on the whole key set (a certified head's mu
 *               keeps every shard's sums in range; an uncertified head may
 *               overflow, as in CLIS_MODE_FIXED).
 *   kv_offset   global index of this shard's first key, >= 0; only the
 *               causal mask uses it (query i sees global keys 0..i; Nq need
 *               not equal Nk here).
 *   accumulate  0: overwrite o_acc and l_acc; 1: add this shard to them.
 *   o_acc       device [B, H, Nq, d] fp32 (16-byte aligned), l_acc device
 *               [B, H, Nq] fp32: unnormalized sums, caller-owned.
 *   ws          device workspace of clis_workspace_bytes(B, H, Nq, Nk, d)
 *               bytes (the shard's V^T); may be NULL for fp32.
 * Shards may be any partition of the keys, in any order.  Finish with
 * clis_attn_combine.
 */
int clis_attn_fwd_partial(const void* q, const void* k, const void* v,
                          int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                          const float* mu, int kv_offset, int accumulate,
                          float* o_acc, float* l_acc, void* ws, size_t ws_bytes, void* stream);

/*
 * Finishes key-sharded attention: o = o_acc / l per row in the output dtype
 * (bf16 round to nearest even, or fp32), and, if lse_out is set, each row's
 * log-sum-exp ln 2 * (mu_i + log2 l_i) (mu then required).  o is
 * [B, H, Nq, d], 16-byte aligned; a row whose l is 0 (it saw no key) gives
 * Inf/NaN, as softmax over no keys is undefined.
 */
int clis_attn_combine(const float* o_acc, const float* l_acc, void* o,
                      int B, int H, int Nq, int d, int dtype,
                      const float* mu, float* lse_out, void* stream);

/* Static text for a status code. */
const char* clis_status_string(int status);

/* Thread-local description of this thread's last failed call ("" if none). */
const char* clis_last_error(void);

/* ABI version of this header: 2. */
int clis_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CLIS_H */
