// api.hip -- the C ABI of include/clis.h: argument checks, workspace carving,
// routing and kernel launches.  Host code only; no allocation, no host
// synchronisation, no device-to-host traffic.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "internal.h"

namespace {

// Scratch of clis_attn_fwd_noalloc, for callers that cannot allocate: one
// copy per GPU, held until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: every use goes through the
// device address that scratch_address() looks up once per device.
__device__ __align__(256) unsigned char scratch[CLIS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's `scratch` (looked up on the first
// call on each device, with that device current).
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(CLIS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape, scale and dtype checks shared by every entry point.  Returns
// CLIS_OK, or an error status with the message set.  *empty is set when
// there is no query row to compute (nothing should be enqueued).
int check_common(int B, int H, int Nq, int Nk, int d, float scale, int dtype, int causal, bool* empty) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
    return fail(CLIS_ERR_SHAPE, "negative dimension (B=%d H=%d Nq=%d Nk=%d)", B, H, Nq, Nk);
  if (dtype != CLIS_BF16 && dtype != CLIS_FP32) return fail(CLIS_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (d != 64 && d != 128) return fail(CLIS_ERR_UNSUPPORTED, "head dim %d not in {64, 128}", d);
  if (!(scale > 0.f) || !isfinite(scale)) return fail(CLIS_ERR_SHAPE, "scale must be finite and > 0");
  if (causal && Nq != Nk) return fail(CLIS_ERR_SHAPE, "causal attention needs Nq == Nk (%d vs %d)", Nq, Nk);
  *empty = (B == 0 || H == 0 || Nq == 0);
  if (*empty) return CLIS_OK;
  if (Nk < 1) return fail(CLIS_ERR_SHAPE, "Nk must be >= 1 when there are query rows");
  const long long BH = (long long)B * H;
  if (BH > 0x7fffffffLL) return fail(CLIS_ERR_SHAPE, "B*H exceeds int32");
  const long long nmax = Nq > Nk ? Nq : Nk;
  if (BH * nmax > (0x7fffffffffffffffLL / 4) / d) return fail(CLIS_ERR_SHAPE, "tensor too large");
  if ((long long)d * clis::vt_pad(Nk) * 2 >= 0x7fffffffLL)
    return fail(CLIS_ERR_SHAPE, "Nk=%d too large: one head's keys must span < 2 GiB", Nk);
  return CLIS_OK;
}

int check_io(const void* q, const void* k, const void* v, const void* o, bool need_o) {
  if (!q || !k || !v || (need_o && !o)) return fail(CLIS_ERR_NULL, "q, k, v%s must be non-NULL", need_o ? ", o" : "");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || (need_o && !aligned(o, 16)))
    return fail(CLIS_ERR_ALIGN, "q, k, v, o must be 16-byte aligned");
  return CLIS_OK;
}

// Pointer checks of the attention entry points (q, k, v, o and the
// optional per-row / per-head arrays).
int check_attn_io(const void* q, const void* k, const void* v, const void* o, const float* mu,
                  const int32_t* cert, const int32_t* route_out, const float* lse_out) {
  int st = check_io(q, k, v, o, true);
  if (st != CLIS_OK) return st;
  if ((lse_out && !aligned(lse_out, 4)) || (mu && !aligned(mu, 4)) || (cert && !aligned(cert, 4)) ||
      (route_out && !aligned(route_out, 4)))
    return fail(CLIS_ERR_ALIGN, "mu, cert, route_out and lse_out must be 4-byte aligned");
  return CLIS_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Enqueue certification into caller buffers (workspace for the partials).
int do_certify(const void* q, const void* k, const void* v, int B, int H, int Nq, int Nk, int d,
               float scale, int dtype, float* mu, int32_t* cert, clis_head_stats_t* stats,
               double* kbar, void* ws, hipStream_t s, const float* vmax_blk = nullptr) {
  const clis::WsLayout L = clis::ws_layout(B, H, Nq, Nk, d);
  clis::CertifyArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.B = B; a.H = H; a.Nq = Nq; a.Nk = Nk; a.d = d;
  a.scale = scale;
  a.dtype = dtype;
  a.mu = mu;
  a.cert = cert;
  a.stats = stats ? stats : at<clis_head_stats_t>(ws, L.stats);
  a.kbar = kbar ? kbar : at<double>(ws, L.kbar);
  a.ksum_part = at<double>(ws, L.ksum_part);
  a.vmax_part = at<double>(ws, L.vmax_part);
  a.kap_part = at<double>(ws, L.kap_part);
  a.qss_part = at<double>(ws, L.qss_part);
  a.vmax_blk = vmax_blk;
  a.vmax_nblk = clis::vt_pad(Nk) / 64;
  const hipError_t e = clis::launch_certify(a, s);
  if (e != hipSuccess) return hip_fail(e, "certify launch");
  return CLIS_OK;
}

int check_ws(void* ws, size_t ws_bytes, int B, int H, int Nq, int Nk, int d) {
  if (!ws) return fail(CLIS_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(CLIS_ERR_ALIGN, "workspace must be 256-byte aligned");
  const size_t need = clis::ws_layout(B, H, Nq, Nk, d).total;
  if (ws_bytes < need) return fail(CLIS_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  return CLIS_OK;
}

clis::AttnArgs attn_args(const void* q, const void* k, const void* v, void* o, int B, int H, int Nq,
                         int Nk, int d, float scale, int causal) {
  clis::AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.n_slots = B * H;
  a.Nq = Nq; a.Nk = Nk; a.d = d;
  a.c2 = (float)((double)scale * clis::kLog2e);
  a.causal = causal ? 1 : 0;
  return a;
}

hipError_t launch_attn(const clis::AttnArgs& a, int dtype, bool fixed, const void* vt, hipStream_t s) {
  if (dtype != CLIS_BF16) return clis::launch_attn_fp32(a, fixed, s);
  return clis::launch_attn_bf16(a, fixed, vt, s);
}

// The bf16 kernels read V through a transposed copy in the workspace.
bool needs_vt(int dtype) { return dtype == CLIS_BF16; }

}  // namespace

extern "C" {

size_t clis_workspace_bytes(int B, int H, int Nq, int Nk, int d) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return 256;
  return clis::ws_layout(B, H, Nq, Nk, d).total;
}

int clis_certify(const void* q, const void* k, const void* v, int B, int H, int Nq, int Nk, int d,
                 float scale, int dtype, float* mu_out, int32_t* cert_out, clis_head_stats_t* stats_out,
                 double* kbar_out, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  bool empty = false;
  int st = check_common(B, H, Nq, Nk, d, scale, dtype, 0, &empty);
  if (st != CLIS_OK || empty) return st;
  if ((st = check_io(q, k, v, nullptr, false)) != CLIS_OK) return st;
  if (!mu_out || !cert_out) return fail(CLIS_ERR_NULL, "mu_out and cert_out must be non-NULL");
  if (!aligned(mu_out, 4) || !aligned(cert_out, 4) || !aligned(stats_out, 8) || !aligned(kbar_out, 8))
    return fail(CLIS_ERR_ALIGN, "mu_out and cert_out must be 4-byte, stats_out and kbar_out 8-byte aligned");
  if ((st = check_ws(ws, ws_bytes, B, H, Nq, Nk, d)) != CLIS_OK) return st;
  return do_certify(q, k, v, B, H, Nq, Nk, d, scale, dtype, mu_out, cert_out, stats_out, kbar_out, ws,
                    static_cast<hipStream_t>(stream));
}

int clis_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int Nq, int Nk,
                  int d, float scale, int causal, int dtype, int mode, const float* mu,
                  const int32_t* cert, int32_t* route_out, float* lse_out, void* ws, size_t ws_bytes,
                  void* stream) {
  g_err[0] = 0;
  if (mode != CLIS_MODE_AUTO && mode != CLIS_MODE_FIXED && mode != CLIS_MODE_ONLINE &&
      mode != CLIS_MODE_ONLINE_LAZY)
    return fail(CLIS_ERR_UNSUPPORTED, "unknown mode %d", mode);
  const bool all_online = (mode == CLIS_MODE_ONLINE || mode == CLIS_MODE_ONLINE_LAZY);
  bool empty = false;
  int st = check_common(B, H, Nq, Nk, d, scale, dtype, causal, &empty);
  if (st != CLIS_OK || empty) return st;
  if ((st = check_attn_io(q, k, v, o, mu, cert, route_out, lse_out)) != CLIS_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  clis::AttnArgs a = attn_args(q, k, v, o, B, H, Nq, Nk, d, scale, causal);
  a.lse = lse_out;
  a.lazy = (mode == CLIS_MODE_ONLINE_LAZY);
  // fp32 online needs no workspace: one kernel; every bf16 call routes first
  // (the route kernel also zeroes the kernels' work counters)
  const bool plain_online = (all_online && !route_out && !needs_vt(dtype));
  if (!plain_online || needs_vt(dtype)) {
    if ((st = check_ws(ws, ws_bytes, B, H, Nq, Nk, d)) != CLIS_OK) return st;
  }
  const clis::WsLayout L = clis::ws_layout(B, H, Nq, Nk, d);
  const int BH = B * H;
  const bool need_cert = (mode == CLIS_MODE_AUTO && (!cert || !mu)) || (mode == CLIS_MODE_FIXED && !mu);
  hipError_t e;
  void* vt = nullptr;
  float* vmax_blk = nullptr;  // the transpose also takes certification's max |V|
  if (needs_vt(dtype)) {
    vt = at<void>(ws, L.vt);
    if (need_cert) vmax_blk = at<float>(ws, L.vmax_blk);
    if ((e = clis::launch_transpose_v(v, vt, BH, Nk, d, s, vmax_blk)) != hipSuccess)
      return hip_fail(e, "V transpose launch");
  }
  if (plain_online) {
    e = launch_attn(a, dtype, false, vt, s);
    return e == hipSuccess ? CLIS_OK : hip_fail(e, "online attention launch");
  }

  const float* mu_use = mu;
  const int32_t* cert_use = cert;
  if (need_cert) {
    float* mu_ws = at<float>(ws, L.mu);
    int32_t* cert_ws = at<int32_t>(ws, L.cert);
    st = do_certify(q, k, v, B, H, Nq, Nk, d, scale, dtype, mu_ws, cert_ws, nullptr, nullptr, ws, s, vmax_blk);
    if (st != CLIS_OK) return st;
    mu_use = mu_ws;
    cert_use = cert_ws;
  }
  if (!needs_vt(dtype)) {  // fp32: one launch that routes each head itself
    clis::AttnArgs f = a;
    f.mu = mu_use;
    f.route_out = route_out;
    if (mode == CLIS_MODE_AUTO) f.cert = cert_use;
    if ((e = launch_attn(f, dtype, mode == CLIS_MODE_FIXED, vt, s)) != hipSuccess)
      return hip_fail(e, "attention launch");
    return CLIS_OK;
  }
  int32_t* lists = at<int32_t>(ws, L.lists);
  int32_t* counts = at<int32_t>(ws, L.counts);
  e = clis::launch_route(cert_use, mode, BH, lists, counts, route_out, s);
  if (e != hipSuccess) return hip_fail(e, "route launch");

  // Each kernel's grid covers every head; slots past its list's count exit
  // at once, so the routing needs no host round trip.
  if (!all_online) {
    clis::AttnArgs f = a;
    f.tail_o = at<float>(ws, L.tail_o);
    f.tail_l = at<float>(ws, L.tail_l);
    f.sched = counts + 2;  // zeroed by the route kernel above
    f.split_heads = counts + 4;
    f.mu = mu_use;
    f.head_list = lists;
    f.head_count = counts;
    if ((e = launch_attn(f, dtype, true, vt, s)) != hipSuccess) return hip_fail(e, "fixed attention launch");
  }
  if (mode != CLIS_MODE_FIXED) {
    clis::AttnArgs g = a;
    g.head_list = lists + BH;
    g.head_count = counts + 1;
    g.sched = counts + 3;  // zeroed by the route kernel above
    if ((e = launch_attn(g, dtype, false, vt, s)) != hipSuccess) return hip_fail(e, "online attention launch");
  }
  return CLIS_OK;
}

int clis_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, int B, int H, int Nq, int Nk,
                          int d, float scale, int causal, int dtype, int mode, const float* mu,
                          const int32_t* cert, int32_t* route_out, float* lse_out, void* stream) {
  g_err[0] = 0;
  if (mode != CLIS_MODE_AUTO && mode != CLIS_MODE_FIXED && mode != CLIS_MODE_ONLINE &&
      mode != CLIS_MODE_ONLINE_LAZY)
    return fail(CLIS_ERR_UNSUPPORTED, "unknown mode %d", mode);
  bool empty = false;
  int st = check_common(B, H, Nq, Nk, d, scale, dtype, causal, &empty);
  if (st != CLIS_OK || empty) return st;
  if ((st = check_attn_io(q, k, v, o, mu, cert, route_out, lse_out)) != CLIS_OK) return st;
  const size_t need = clis::ws_layout(B, H, Nq, Nk, d).total;
  if (need > (size_t)CLIS_NOALLOC_SCRATCH_BYTES)
    return fail(CLIS_ERR_WORKSPACE, "shape needs %zu bytes of scratch, more than the %zu of clis_attn_fwd_noalloc "
                "(use clis_attn_fwd with a workspace)", need, (size_t)CLIS_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e, "scratch address");
  return clis_attn_fwd(q, k, v, o, B, H, Nq, Nk, d, scale, causal, dtype, mode, mu, cert, route_out, lse_out, ws,
                       (size_t)CLIS_NOALLOC_SCRATCH_BYTES, stream);
}

int online_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int Nq, int Nk,
                    int d, float scale, int causal, int dtype, float* lse_out, void* ws, size_t ws_bytes,
                    void* stream) {
  return clis_attn_fwd(q, k, v, o, B, H, Nq, Nk, d, scale, causal, dtype, CLIS_MODE_ONLINE, nullptr,
                       nullptr, nullptr, lse_out, ws, ws_bytes, stream);
}

int clis_attn_fwd_partial(const void* q, const void* k, const void* v, int B, int H, int Nq, int Nk, int d,
                          float scale, int causal, int dtype, const float* mu, int kv_offset, int accumulate,
                          float* o_acc, float* l_acc, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  bool empty = false;
  // a causal shard need not be square: the mask compares global indices
  int st = check_common(B, H, Nq, Nk, d, scale, dtype, 0, &empty);
  if (st != CLIS_OK || empty) return st;
  if ((st = check_io(q, k, v, nullptr, false)) != CLIS_OK) return st;
  if (!mu || !o_acc || !l_acc) return fail(CLIS_ERR_NULL, "mu, o_acc and l_acc must be non-NULL");
  if (!aligned(o_acc, 16) || !aligned(l_acc, 4) || !aligned(mu, 4))
    return fail(CLIS_ERR_ALIGN, "o_acc must be 16-byte, l_acc and mu 4-byte aligned");
  if (kv_offset < 0 || (long long)kv_offset + Nk > 0x7fffffffLL)
    return fail(CLIS_ERR_SHAPE, "kv_offset %d out of range", kv_offset);
  if (accumulate != 0 && accumulate != 1) return fail(CLIS_ERR_SHAPE, "accumulate must be 0 or 1");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  void* vt = nullptr;
  if (needs_vt(dtype)) {
    if ((st = check_ws(ws, ws_bytes, B, H, Nq, Nk, d)) != CLIS_OK) return st;
    vt = at<void>(ws, clis::ws_layout(B, H, Nq, Nk, d).vt);
    if ((e = clis::launch_transpose_v(v, vt, B * H, Nk, d, s)) != hipSuccess) return hip_fail(e, "V transpose launch");
  }
  clis::AttnArgs a = attn_args(q, k, v, nullptr, B, H, Nq, Nk, d, scale, causal);
  a.mu = mu;
  a.o_acc = o_acc;
  a.l_acc = l_acc;
  a.accumulate = accumulate;
  a.kv_offset = kv_offset;
  if ((e = launch_attn(a, dtype, true, vt, s)) != hipSuccess) return hip_fail(e, "key-shard attention launch");
  return CLIS_OK;
}

int clis_attn_combine(const float* o_acc, const float* l_acc, void* o, int B, int H, int Nq, int d, int dtype,
                      const float* mu, float* lse_out, void* stream) {
  g_err[0] = 0;
  if (B < 0 || H < 0 || Nq < 0) return fail(CLIS_ERR_SHAPE, "negative dimension (B=%d H=%d Nq=%d)", B, H, Nq);
  if (dtype != CLIS_BF16 && dtype != CLIS_FP32) return fail(CLIS_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (d != 64 && d != 128) return fail(CLIS_ERR_UNSUPPORTED, "head dim %d not in {64, 128}", d);
  const long long rows = (long long)B * H * Nq;
  if (rows == 0) return CLIS_OK;
  if (rows > (0x7fffffffffffffffLL / 4) / d) return fail(CLIS_ERR_SHAPE, "tensor too large");
  if (!o_acc || !l_acc || !o) return fail(CLIS_ERR_NULL, "o_acc, l_acc and o must be non-NULL");
  if (lse_out && !mu) return fail(CLIS_ERR_NULL, "lse_out needs mu");
  if (!aligned(o_acc, 16) || !aligned(o, 16) || !aligned(l_acc, 4) || (lse_out && !aligned(lse_out, 4)) ||
      (mu && !aligned(mu, 4)))
    return fail(CLIS_ERR_ALIGN, "o_acc and o must be 16-byte, l_acc, mu and lse_out 4-byte aligned");
  const hipError_t e = clis::launch_combine(o_acc, l_acc, o, dtype == CLIS_BF16, mu, lse_out, rows, d,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CLIS_OK : hip_fail(e, "combine launch");
}

const char* clis_status_string(int status) {
  switch (status) {
    case CLIS_OK: return "ok";
    case CLIS_ERR_NULL: return "null pointer";
    case CLIS_ERR_SHAPE: return "invalid shape or scale";
    case CLIS_ERR_UNSUPPORTED: return "unsupported head dim, dtype or mode";
    case CLIS_ERR_ALIGN: return "misaligned pointer";
    case CLIS_ERR_WORKSPACE: return "workspace missing or too small";
    case CLIS_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

const char* clis_last_error(void) { return g_err; }

int clis_abi_version(void) { return 2; }

}  // extern "C"
