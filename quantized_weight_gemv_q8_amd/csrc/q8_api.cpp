// q8_api.cpp -- the C ABI: argument validation, device check, dispatch.
//
// Every entry point validates all of its arguments before touching the HIP
// runtime, so a bad call fails synchronously with nothing enqueued (and can
// be tested on a host without a GPU). Then it checks, once per device, that
// the current device is gfx950 (memra wiki: fail early when the binary does
// not match the device), and enqueues kernels on the caller's stream.
#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>

#include "q8gemv.h"

#include <climits>
#include "q8_internal.h"

using q8::DevInfo;
using q8::HBank;
using q8::HMat;

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
DevInfo g_info[kMaxDevices];
int g_info_rc[kMaxDevices];

void probe(int dev) {
  DevInfo& d = g_info[dev];
  d.device = dev;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    g_info_rc[dev] = Q8_ERR_DEVICE;
    return;
  }
  d.cus = prop.multiProcessorCount;
  d.lds_per_block = prop.sharedMemPerBlock;
  d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  g_info_rc[dev] = d.gfx950 ? Q8_OK : Q8_ERR_DEVICE;
}

// Current device's cached properties; Q8_ERR_DEVICE unless it is gfx950.
int current_device(const DevInfo** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return Q8_ERR_DEVICE;
  std::call_once(g_once[dev], probe, dev);
  if (g_info_rc[dev] != Q8_OK) return g_info_rc[dev];
  *out = &g_info[dev];
  return Q8_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t dt_size(int dt) { return dt == Q8_DT_F16 ? 2 : dt == Q8_DT_F32 ? 4 : 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int check_matrix(const q8_matrix* W) {
  if (!W || !W->qs || !W->d) return Q8_ERR_NULL;
  if (W->format != Q8_FMT_Q8_0 && W->format != Q8_FMT_Q4_0) return Q8_ERR_DTYPE;
  if (W->M < 1 || W->M > INT32_MAX || W->K < 32 || W->K % 32 || W->K > (1LL << 24))
    return Q8_ERR_SHAPE;
  const int64_t row_bytes = W->format == Q8_FMT_Q4_0 ? W->K / 2 : W->K;
  if (W->ld_qs < row_bytes || W->ld_d < W->K / 32) return Q8_ERR_SHAPE;
  if (W->ld_qs % 16 || W->ld_d % 8 || !aligned(W->qs, 16) || !aligned(W->d, 16))
    return Q8_ERR_ALIGN;
  return Q8_OK;
}

int check_bank(const q8_bank* B) {
  if (!B) return Q8_ERR_NULL;
  int rc = check_matrix(&B->e0);
  if (rc) return rc;
  if (B->E < 1) return Q8_ERR_SHAPE;
  if (B->E > 1 && (B->stride_qs < B->e0.M * B->e0.ld_qs || B->stride_d < B->e0.M * B->e0.ld_d))
    return Q8_ERR_SHAPE;
  if (B->stride_qs % 16 || B->stride_d % 8) return Q8_ERR_ALIGN;
  return Q8_OK;
}

HMat to_h(const q8_matrix* W) {
  return HMat{W->qs, W->d, W->M, W->K, W->ld_qs, W->ld_d,
              W->format == Q8_FMT_Q4_0 ? q8::kFmtQ4 : q8::kFmtQ8};
}

HBank to_hb(const q8_bank* B) {
  return HBank{to_h(&B->e0), B->stride_qs, B->stride_d, (int)B->E};
}

int launch_rc(hipError_t e) { return e == hipSuccess ? Q8_OK : Q8_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* q8_status_str(int status) {
  switch (status) {
    case Q8_OK: return "ok";
    case Q8_ERR_NULL: return "null pointer";
    case Q8_ERR_SHAPE: return "bad shape";
    case Q8_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case Q8_ERR_DTYPE: return "unsupported dtype";
    case Q8_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case Q8_ERR_DEVICE: return "device is not gfx950 (or no device)";
    case Q8_ERR_LAUNCH: return "kernel launch failed";
    case Q8_ERR_ALIAS: return "output overlaps an input";
  }
  return "unknown status";
}

int q8_device_check(int device) {
  if (device < 0 || device >= kMaxDevices) return Q8_ERR_DEVICE;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device >= n) return Q8_ERR_DEVICE;
  std::call_once(g_once[device], probe, device);
  return g_info_rc[device];
}

// ------------------------------------------------------------ packing
int q8_pack_layout(int64_t M, int64_t K, int64_t* ld_qs, int64_t* ld_d, size_t* qs_bytes,
                   size_t* d_bytes) {
  if (M < 1 || K < 32 || K % 32) return Q8_ERR_SHAPE;
  const int64_t lq = K;
  const int64_t ld = (K / 32 + 7) / 8 * 8;
  if (ld_qs) *ld_qs = lq;
  if (ld_d) *ld_d = ld;
  if (qs_bytes) *qs_bytes = (size_t)M * (size_t)lq;
  if (d_bytes) *d_bytes = (size_t)M * (size_t)ld * 2;
  return Q8_OK;
}

int q8_pack_host(const void* blocks, int64_t M, int64_t K, int8_t* qs, int64_t ld_qs, uint16_t* d,
                 int64_t ld_d) {
  if (!blocks || !qs || !d) return Q8_ERR_NULL;
  if (M < 1 || K < 32 || K % 32) return Q8_ERR_SHAPE;
  if (ld_qs < K || ld_d < K / 32) return Q8_ERR_SHAPE;
  if (ld_qs % 16 || ld_d % 8) return Q8_ERR_ALIGN;
  const uint8_t* src = (const uint8_t*)blocks;
  const int64_t nb = K / 32;
  for (int64_t m = 0; m < M; ++m) {
    int8_t* qrow = qs + m * ld_qs;
    uint16_t* drow = d + m * ld_d;
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t* blk = src + (m * nb + b) * 34;
      drow[b] = (uint16_t)(blk[0] | ((uint16_t)blk[1] << 8));
      memcpy(qrow + b * 32, blk + 2, 32);
    }
    if (ld_qs > K) memset(qrow + K, 0, (size_t)(ld_qs - K));
    for (int64_t b = nb; b < ld_d; ++b) drow[b] = 0;
  }
  return Q8_OK;
}

int q8_unpack_host(const int8_t* qs, int64_t ld_qs, const uint16_t* d, int64_t ld_d, int64_t M,
                   int64_t K, void* blocks) {
  if (!blocks || !qs || !d) return Q8_ERR_NULL;
  if (M < 1 || K < 32 || K % 32) return Q8_ERR_SHAPE;
  if (ld_qs < K || ld_d < K / 32) return Q8_ERR_SHAPE;
  uint8_t* dst = (uint8_t*)blocks;
  const int64_t nb = K / 32;
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t b = 0; b < nb; ++b) {
      uint8_t* blk = dst + (m * nb + b) * 34;
      const uint16_t v = d[m * ld_d + b];
      blk[0] = (uint8_t)(v & 0xff);
      blk[1] = (uint8_t)(v >> 8);
      memcpy(blk + 2, qs + m * ld_qs + b * 32, 32);
    }
  }
  return Q8_OK;
}

// ------------------------------------------------------------ Q4_0 packing
int q8_pack_q4_0_layout(int64_t M, int64_t K, int64_t* ld_qs, int64_t* ld_d, size_t* qs_bytes,
                        size_t* d_bytes) {
  if (M < 1 || K < 32 || K % 32) return Q8_ERR_SHAPE;
  const int64_t lq = K / 2;
  const int64_t ld = (K / 32 + 7) / 8 * 8;
  if (ld_qs) *ld_qs = lq;
  if (ld_d) *ld_d = ld;
  if (qs_bytes) *qs_bytes = (size_t)M * (size_t)lq;
  if (d_bytes) *d_bytes = (size_t)M * (size_t)ld * 2;
  return Q8_OK;
}

int q8_pack_q4_0_host(const void* blocks, int64_t M, int64_t K, uint8_t* qs, int64_t ld_qs,
                      uint16_t* d, int64_t ld_d) {
  if (!blocks || !qs || !d) return Q8_ERR_NULL;
  if (M < 1 || K < 32 || K % 32) return Q8_ERR_SHAPE;
  if (ld_qs < K / 2 || ld_d < K / 32) return Q8_ERR_SHAPE;
  if (ld_qs % 16 || ld_d % 8) return Q8_ERR_ALIGN;
  const uint8_t* src = (const uint8_t*)blocks;
  const int64_t nb = K / 32;
  for (int64_t m = 0; m < M; ++m) {
    uint8_t* qrow = qs + m * ld_qs;
    uint16_t* drow = d + m * ld_d;
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t* blk = src + (m * nb + b) * 18;
      drow[b] = (uint16_t)(blk[0] | ((uint16_t)blk[1] << 8));
      memcpy(qrow + b * 16, blk + 2, 16);
    }
    if (ld_qs > K / 2) memset(qrow + K / 2, 0, (size_t)(ld_qs - K / 2));
    for (int64_t b = nb; b < ld_d; ++b) drow[b] = 0;
  }
  return Q8_OK;
}

int q8_unpack_q4_0_host(const uint8_t* qs, int64_t ld_qs, const uint16_t* d, int64_t ld_d,
                        int64_t M, int64_t K, void* blocks) {
  if (!blocks || !qs || !d) return Q8_ERR_NULL;
  if (M < 1 || K < 32 || K % 32) return Q8_ERR_SHAPE;
  if (ld_qs < K / 2 || ld_d < K / 32) return Q8_ERR_SHAPE;
  uint8_t* dst = (uint8_t*)blocks;
  const int64_t nb = K / 32;
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t b = 0; b < nb; ++b) {
      uint8_t* blk = dst + (m * nb + b) * 18;
      const uint16_t v = d[m * ld_d + b];
      blk[0] = (uint8_t)(v & 0xff);
      blk[1] = (uint8_t)(v >> 8);
      memcpy(blk + 2, qs + m * ld_qs + b * 16, 16);
    }
  }
  return Q8_OK;
}

// ------------------------------------------------------------ dense GEMV
// The next launch of a call over N tokens in passes of per_pass, from token
// n0: its pass size nt and the number of such passes it runs. Where the
// 9..16-token kernel does not apply (multi), every remaining full pass
// goes into one launch (the one-group kernels run them as slices of one
// grid); otherwise one pass per launch.
static void next_launch(int N, int n0, int per_pass, bool multi, int* nt, int* slices) {
  *nt = N - n0 < per_pass ? N - n0 : per_pass;
  *slices = multi && *nt == per_pass ? (N - n0) / per_pass : 1;
}

static int gemv_impl(const q8_matrix* Wa, const q8_matrix* Wb, const void* x, int x_dt, void* ya,
                     void* yb, int y_dt, int N, void* stream) {
  int rc = check_matrix(Wa);
  if (rc) return rc;
  if (Wb) {
    rc = check_matrix(Wb);
    if (rc) return rc;
    if (Wb->K != Wa->K) return Q8_ERR_SHAPE;
    if (Wb->format != Wa->format) return Q8_ERR_DTYPE;
  }
  if (!x || !ya || (Wb && !yb)) return Q8_ERR_NULL;
  if (N < 1) return Q8_ERR_SHAPE;
  const size_t xs = dt_size(x_dt), ys = dt_size(y_dt);
  if (!xs || !ys) return Q8_ERR_DTYPE;
  if (!aligned(x, 16) || !aligned(ya, ys) || (Wb && !aligned(yb, ys))) return Q8_ERR_ALIGN;
  const size_t xbytes = (size_t)N * Wa->K * xs;
  const size_t yabytes = (size_t)N * Wa->M * ys;
  if (overlap(x, xbytes, ya, yabytes)) return Q8_ERR_ALIAS;
  if (Wb) {
    const size_t ybbytes = (size_t)N * Wb->M * ys;
    if (overlap(x, xbytes, yb, ybbytes) || overlap(ya, yabytes, yb, ybbytes)) return Q8_ERR_ALIAS;
  }
  const DevInfo* dev = nullptr;
  rc = current_device(&dev);
  if (rc) return rc;
  const bool xf = x_dt == Q8_DT_F32;
  const int64_t rows = Wa->M + (Wb ? Wb->M : 0);
  const bool wide = q8::wide_pass_applies(*dev, Wa->format, Wa->K, xf, rows);
  const int per_pass = wide ? q8::max_tokens_per_pass_wide(*dev, Wa->K, xf)
                            : q8::max_tokens_per_pass(*dev, Wa->K, xf);
  if (per_pass < 1) return Q8_ERR_SHAPE;
  const HMat A = to_h(Wa);
  HMat B;
  if (Wb) B = to_h(Wb);
  for (int n0 = 0, nt, slices; n0 < N; n0 += nt * slices) {
    next_launch(N, n0, per_pass, !wide, &nt, &slices);
    const char* xp = (const char*)x + (size_t)n0 * Wa->K * xs;
    char* yap = (char*)ya + (size_t)n0 * Wa->M * ys;
    char* ybp = Wb ? (char*)yb + (size_t)n0 * Wb->M * ys : nullptr;
    hipError_t e = q8::launch_gemv(*dev, A, Wb ? &B : nullptr, xp, xf, Wa->K, yap, ybp,
                                   y_dt == Q8_DT_F16, nt, (hipStream_t)stream, nullptr, slices);
    if (e != hipSuccess) return Q8_ERR_LAUNCH;
  }
  return Q8_OK;
}

int q8_gemv(const q8_matrix* W, const void* x, int x_dt, void* y, int y_dt, int N, void* stream) {
  return gemv_impl(W, nullptr, x, x_dt, y, nullptr, y_dt, N, stream);
}

int q8_gemv_pair(const q8_matrix* Wa, const q8_matrix* Wb, const void* x, int x_dt, void* ya,
                 void* yb, int y_dt, int N, void* stream) {
  if (!Wb) return Q8_ERR_NULL;
  return gemv_impl(Wa, Wb, x, x_dt, ya, yb, y_dt, N, stream);
}

int q8_gemv_pair_silu(const q8_matrix* Wg, const q8_matrix* Wu, const void* x, int x_dt, void* h,
                      int h_dt, int N, void* stream) {
  int rc = check_matrix(Wg);
  if (rc) return rc;
  if ((rc = check_matrix(Wu))) return rc;
  if (Wu->M != Wg->M || Wu->K != Wg->K) return Q8_ERR_SHAPE;
  if (Wu->format != Wg->format) return Q8_ERR_DTYPE;
  if (!x || !h) return Q8_ERR_NULL;
  if (N < 1) return Q8_ERR_SHAPE;
  const size_t xs = dt_size(x_dt), hs = dt_size(h_dt);
  if (!xs || !hs) return Q8_ERR_DTYPE;
  if (!aligned(x, 16) || !aligned(h, hs)) return Q8_ERR_ALIGN;
  if (overlap(x, (size_t)N * Wg->K * xs, h, (size_t)N * Wg->M * hs)) return Q8_ERR_ALIAS;
  const DevInfo* dev = nullptr;
  rc = current_device(&dev);
  if (rc) return rc;
  const bool xf = x_dt == Q8_DT_F32;
  const bool wide = q8::wide_pass_applies(*dev, Wg->format, Wg->K, xf, 2 * Wg->M);
  const int per_pass = wide ? q8::max_tokens_per_pass_wide(*dev, Wg->K, xf)
                            : q8::max_tokens_per_pass(*dev, Wg->K, xf);
  if (per_pass < 1) return Q8_ERR_SHAPE;
  const HMat G = to_h(Wg), U = to_h(Wu);
  for (int n0 = 0, nt, slices; n0 < N; n0 += nt * slices) {
    next_launch(N, n0, per_pass, !wide, &nt, &slices);
    hipError_t e = q8::launch_glu(*dev, G, U, (const char*)x + (size_t)n0 * Wg->K * xs, xf,
                                  (char*)h + (size_t)n0 * Wg->M * hs, h_dt == Q8_DT_F16, nt,
                                  (hipStream_t)stream, nullptr, nullptr, slices);
    if (e != hipSuccess) return Q8_ERR_LAUNCH;
  }
  return Q8_OK;
}

// ------------------------------------------------------------ LM head
size_t q8_lmhead_ws_bytes(int64_t V, int N) {
  (void)N;
  return q8::lmhead_ws_bytes(V);
}

static int lmhead_impl(const q8_matrix* W, const int32_t* row_ids, const void* x, int x_dt,
                       float* logits, int32_t* ids, int N, void* ws, size_t ws_bytes,
                       void* stream) {
  int rc = check_matrix(W);
  if (rc) return rc;
  if (!x || !ids) return Q8_ERR_NULL;
  if (N < 1) return Q8_ERR_SHAPE;
  const size_t xs = dt_size(x_dt);
  if (!xs) return Q8_ERR_DTYPE;
  if (!aligned(x, 16) || !aligned(ids, 4) || (logits && !aligned(logits, 4)) ||
      (row_ids && !aligned(row_ids, 4)))
    return Q8_ERR_ALIGN;
  if (!ws || !aligned(ws, 16) || ws_bytes < q8_lmhead_ws_bytes(W->M, N)) return Q8_ERR_WORKSPACE;
  const size_t xbytes = (size_t)N * W->K * xs;
  const size_t lbytes = logits ? (size_t)N * W->M * 4 : 0;
  const size_t rbytes = row_ids ? (size_t)W->M * 4 : 0;
  if ((logits && overlap(x, xbytes, logits, lbytes)) || overlap(x, xbytes, ids, 4 * (size_t)N) ||
      (logits && overlap(logits, lbytes, ids, 4 * (size_t)N)) ||
      overlap(ws, ws_bytes, x, xbytes) || overlap(ws, ws_bytes, ids, 4 * (size_t)N) ||
      (logits && overlap(ws, ws_bytes, logits, lbytes)) ||
      (row_ids && (overlap(row_ids, rbytes, ids, 4 * (size_t)N) ||
                   overlap(row_ids, rbytes, ws, ws_bytes) ||
                   (logits && overlap(row_ids, rbytes, logits, lbytes)))))
    return Q8_ERR_ALIAS;
  const DevInfo* dev = nullptr;
  rc = current_device(&dev);
  if (rc) return rc;
  const bool xf = x_dt == Q8_DT_F32;
  const int per_pass = q8::lmhead_max_tokens_per_pass(*dev, W->K, xf);
  if (per_pass < 1) return Q8_ERR_SHAPE;
  const HMat A = to_h(W);
  for (int n0 = 0; n0 < N; n0 += per_pass) {
    const int nt = N - n0 < per_pass ? N - n0 : per_pass;
    const char* xp = (const char*)x + (size_t)n0 * W->K * xs;
    float* lp = logits ? logits + (size_t)n0 * W->M : nullptr;
    hipError_t e = q8::launch_lmhead(*dev, A, row_ids, xp, xf, lp, W->M, ids + n0, (char*)ws, nt,
                                     (hipStream_t)stream);
    if (e != hipSuccess) return Q8_ERR_LAUNCH;
  }
  return Q8_OK;
}

int q8_lmhead_argmax(const q8_matrix* W, const void* x, int x_dt, float* logits, int32_t* ids,
                     int N, void* ws, size_t ws_bytes, void* stream) {
  return lmhead_impl(W, nullptr, x, x_dt, logits, ids, N, ws, ws_bytes, stream);
}

int q8_lmhead_argmax_rows(const q8_matrix* W, const int32_t* row_ids, const void* x, int x_dt,
                          float* logits, int32_t* ids, int N, void* ws, size_t ws_bytes,
                          void* stream) {
  if (!row_ids) return Q8_ERR_NULL;
  return lmhead_impl(W, row_ids, x, x_dt, logits, ids, N, ws, ws_bytes, stream);
}

// ------------------------------------------------------------ routed experts
size_t q8_moe_ws_bytes(int E, int T, int topk, int64_t F, int64_t M) {
  if (E < 1 || T < 1 || topk < 1 || F < 0 || M < 0) return 0;
  size_t off[q8::kMoeWsAreas];
  return q8::moe_ws_layout(E, T, topk, F, M, off);
}

int q8_moe_ws_layout(int E, int T, int topk, int64_t F, int64_t M, size_t offsets[7]) {
  if (!offsets) return Q8_ERR_NULL;
  if (E < 1 || T < 1 || topk < 1 || topk > E || F < 0 || M < 0) return Q8_ERR_SHAPE;
  size_t off[q8::kMoeWsAreas];
  q8::moe_ws_layout(E, T, topk, F, M, off);
  for (int i = 0; i < 7; ++i) offsets[i] = off[i];
  return Q8_OK;
}

static q8::MoeWs moe_ws_ptrs(void* ws, int E, int T, int topk, int64_t F, int64_t M) {
  size_t off[q8::kMoeWsAreas];
  q8::moe_ws_layout(E, T, topk, F, M, off);
  char* b = (char*)ws;
  q8::MoeWs w;
  w.counts = (int32_t*)(b + off[0]);
  w.offsets = (int32_t*)(b + off[1]);
  w.pairs = (int32_t*)(b + off[2]);
  w.active = (int32_t*)(b + off[3]);
  w.n_active = (int32_t*)(b + off[4]);
  w.n_vslots = w.n_active + 1;
  w.n_bad_ids = w.n_active + 2;
  w.h = F > 0 ? (float*)(b + off[5]) : nullptr;
  w.y_pair = (float*)(b + off[6]);
  w.vslots = (int32_t*)(b + off[7]);
  return w;
}

static int check_routing(const int32_t* ids, const float* gate_w, int T, int topk, int E,
                         bool need_gate) {
  if (!ids || (need_gate && !gate_w)) return Q8_ERR_NULL;
  if (T < 1 || topk < 1 || topk > E || (int64_t)T * topk > 8192) return Q8_ERR_SHAPE;
  if (!aligned(ids, 4) || (gate_w && !aligned(gate_w, 4))) return Q8_ERR_ALIGN;
  return Q8_OK;
}

int q8_moe_gemv(const q8_bank* W, const int32_t* expert_ids, const float* gate_w, const void* x,
                int x_dt, int x_per_pair, float* y, int T, int topk, void* ws, size_t ws_bytes,
                void* stream) {
  int rc = check_bank(W);
  if (rc) return rc;
  if (W->E > 4096) return Q8_ERR_SHAPE;
  rc = check_routing(expert_ids, gate_w, T, topk, W->E, false);
  if (rc) return rc;
  if (!x || !y) return Q8_ERR_NULL;
  const size_t xs = dt_size(x_dt);
  if (!xs) return Q8_ERR_DTYPE;
  if (!aligned(x, 16) || !aligned(y, 4)) return Q8_ERR_ALIGN;
  const int P = T * topk;
  const int64_t M = W->e0.M, K = W->e0.K;
  // the routed row space (virtual slots x rows) is indexed in 32 bits
  if ((int64_t)q8::moe_max_vslots(W->E, P) * M > INT32_MAX) return Q8_ERR_SHAPE;
  if (!ws || !aligned(ws, 16) || ws_bytes < q8_moe_ws_bytes(W->E, T, topk, 0, M))
    return Q8_ERR_WORKSPACE;
  const size_t xbytes = (size_t)(x_per_pair ? P : T) * K * xs;
  const size_t ybytes = (size_t)(gate_w ? T : P) * M * 4;
  if (overlap(x, xbytes, y, ybytes) || overlap(ws, ws_bytes, x, xbytes) ||
      overlap(ws, ws_bytes, y, ybytes))
    return Q8_ERR_ALIAS;
  const DevInfo* dev = nullptr;
  rc = current_device(&dev);
  if (rc) return rc;
  const bool xf = x_dt == Q8_DT_F32;
  if (!q8::moe_fits(*dev, K, xf)) return Q8_ERR_SHAPE;
  q8::MoeWs w = moe_ws_ptrs(ws, W->E, T, topk, 0, M);
  float* yp = gate_w ? w.y_pair : y;
  hipStream_t s = (hipStream_t)stream;
  const q8::RouteReq route{expert_ids, W->E, P, gate_w ? nullptr : y, M};
  if (q8::launch_moe_gemv(*dev, to_hb(W), w, topk, x, xf, x_per_pair != 0, yp, route, s) !=
      hipSuccess)
    return Q8_ERR_LAUNCH;
  if (gate_w)
    return launch_rc(q8::launch_moe_combine(expert_ids, W->E, gate_w, yp, y, T, topk, M, s));
  return Q8_OK;
}

// The routed FFN on a workspace ws of ws_bytes; no_alloc: ws is the
// library's scratch array (its size is checked here, before the runtime is
// touched, and it cannot alias the caller's buffers).
static int moe_ffn_impl(const q8_bank* gate, const q8_bank* up, const q8_bank* down,
                        const int32_t* expert_ids, const float* gate_w, const void* x, int x_dt,
                        float* out, int T, int topk, void* ws, size_t ws_bytes, bool no_alloc,
                        void* stream) {
  int rc = check_bank(gate);
  if (rc) return rc;
  if ((rc = check_bank(up)) || (rc = check_bank(down))) return rc;
  const int E = gate->E;
  if (up->E != E || down->E != E || E > 4096) return Q8_ERR_SHAPE;
  const int64_t F = gate->e0.M, H = gate->e0.K;
  if (up->e0.M != F || up->e0.K != H || down->e0.M != H || down->e0.K != F) return Q8_ERR_SHAPE;
  if (up->e0.format != gate->e0.format) return Q8_ERR_DTYPE;
  rc = check_routing(expert_ids, gate_w, T, topk, E, true);
  if (rc) return rc;
  if ((int64_t)q8::moe_max_vslots(E, T * topk) * (2 * F > H ? 2 * F : H) > INT32_MAX)
    return Q8_ERR_SHAPE;
  if (!x || !out) return Q8_ERR_NULL;
  const size_t xs = dt_size(x_dt);
  if (!xs) return Q8_ERR_DTYPE;
  if (!aligned(x, 16) || !aligned(out, 4)) return Q8_ERR_ALIGN;
  const size_t need = q8_moe_ws_bytes(E, T, topk, F, H);
  if (no_alloc) {
    if (need > q8::kNoAllocScratchBytes) return Q8_ERR_WORKSPACE;
  } else if (!ws || !aligned(ws, 16) || ws_bytes < need) {
    return Q8_ERR_WORKSPACE;
  }
  const size_t xbytes = (size_t)T * H * xs, obytes = (size_t)T * H * 4;
  if (overlap(x, xbytes, out, obytes) ||
      (!no_alloc && (overlap(ws, ws_bytes, x, xbytes) || overlap(ws, ws_bytes, out, obytes))))
    return Q8_ERR_ALIAS;
  const DevInfo* dev = nullptr;
  rc = current_device(&dev);
  if (rc) return rc;
  if (no_alloc && q8::noalloc_scratch(dev->device, &ws) != hipSuccess) return Q8_ERR_DEVICE;
  const bool xf = x_dt == Q8_DT_F32;
  if (!q8::moe_fits(*dev, H, xf) || !q8::moe_fits(*dev, F, true)) return Q8_ERR_SHAPE;
  const int P = T * topk;
  q8::MoeWs w = moe_ws_ptrs(ws, E, T, topk, F, H);
  hipStream_t s = (hipStream_t)stream;
  const q8::RouteReq route{expert_ids, E, P, nullptr, 0};
  const q8::RouteReq routed{nullptr, E, P, nullptr, 0};  // the workspace holds it by then
  if (q8::launch_moe_gate_up(*dev, to_hb(gate), to_hb(up), w, topk, x, xf, w.h, route, s) !=
      hipSuccess)
    return Q8_ERR_LAUNCH;
  if (q8::launch_moe_gemv(*dev, to_hb(down), w, topk, w.h, true, true, w.y_pair, routed, s) !=
      hipSuccess)
    return Q8_ERR_LAUNCH;
  return launch_rc(q8::launch_moe_combine(expert_ids, E, gate_w, w.y_pair, out, T, topk, H, s));
}

int q8_moe_ffn(const q8_bank* gate, const q8_bank* up, const q8_bank* down,
               const int32_t* expert_ids, const float* gate_w, const void* x, int x_dt,
               float* out, int T, int topk, void* ws, size_t ws_bytes, void* stream) {
  return moe_ffn_impl(gate, up, down, expert_ids, gate_w, x, x_dt, out, T, topk, ws, ws_bytes,
                      false, stream);
}

size_t q8_noalloc_scratch_bytes(void) { return q8::kNoAllocScratchBytes; }

int q8_moe_ffn_noalloc(const q8_bank* gate, const q8_bank* up, const q8_bank* down,
                       const int32_t* expert_ids, const float* gate_w, const void* x, int x_dt,
                       float* out, int T, int topk, void* stream) {
  return moe_ffn_impl(gate, up, down, expert_ids, gate_w, x, x_dt, out, T, topk, nullptr, 0,
                      true, stream);
}

// ------------------------------------------------------------ shared expert
// Workspace: h [T][F] and the expert's output [T][H], fp32, each area
// 256-byte aligned.
static void shared_ws_layout(int64_t F, int64_t H, int T, size_t off[2], size_t* total) {
  (void)H;
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  off[0] = 0;                            // h [T][F] fp32
  off[1] = up((size_t)T * F * 4);        // gate dots [T] fp32
  *total = off[1] + up((size_t)T * 4);
}

size_t q8_moe_shared_ws_bytes(int64_t F, int64_t H, int T) {
  if (F < 1 || H < 1 || T < 1) return 0;
  size_t off[2], total;
  shared_ws_layout(F, H, T, off, &total);
  return total;
}

int q8_moe_shared_expert(const q8_matrix* Wg, const q8_matrix* Wu, const q8_matrix* Wd,
                         const q8_matrix* Wsg, const void* x, int x_dt, int T, float* out,
                         void* ws, size_t ws_bytes, void* stream) {
  int rc = check_matrix(Wg);
  if (rc) return rc;
  if ((rc = check_matrix(Wu)) || (rc = check_matrix(Wd)) || (rc = check_matrix(Wsg))) return rc;
  const int64_t F = Wg->M, H = Wg->K;
  if (Wu->M != F || Wu->K != H || Wd->M != H || Wd->K != F || Wsg->M != 1 || Wsg->K != H)
    return Q8_ERR_SHAPE;
  if (Wu->format != Wg->format || Wsg->format != Wg->format) return Q8_ERR_DTYPE;
  if (!x || !out) return Q8_ERR_NULL;
  if (T < 1) return Q8_ERR_SHAPE;
  const size_t xs = dt_size(x_dt);
  if (!xs) return Q8_ERR_DTYPE;
  if (!aligned(x, 16) || !aligned(out, 4)) return Q8_ERR_ALIGN;
  if (!ws || !aligned(ws, 16) || ws_bytes < q8_moe_shared_ws_bytes(F, H, T))
    return Q8_ERR_WORKSPACE;
  const size_t xbytes = (size_t)T * H * xs, obytes = (size_t)T * H * 4;
  if (overlap(x, xbytes, out, obytes) || overlap(ws, ws_bytes, x, xbytes) ||
      overlap(ws, ws_bytes, out, obytes))
    return Q8_ERR_ALIAS;
  const DevInfo* dev = nullptr;
  rc = current_device(&dev);
  if (rc) return rc;
  const bool xf = x_dt == Q8_DT_F32;
  const int pass_h = q8::max_tokens_per_pass(*dev, H, xf);
  const int pass_f = q8::max_tokens_per_pass(*dev, F, true);
  if (pass_h < 1 || pass_f < 1) return Q8_ERR_SHAPE;
  size_t off[2], total;
  shared_ws_layout(F, H, T, off, &total);
  float* h = (float*)((char*)ws + off[0]);
  float* gd = (float*)((char*)ws + off[1]);
  const HMat G = to_h(Wg), U = to_h(Wu), D = to_h(Wd), SG = to_h(Wsg);
  hipStream_t s = (hipStream_t)stream;
  // Two kinds of launch per pass: the gate/up pair with the gate row as an
  // extra row (h and the gate dots), then the down projection whose
  // epilogue adds sigmoid(gate dot) * (Wd h) into out.
  for (int n0 = 0, nt, slices; n0 < T; n0 += nt * slices) {
    next_launch(T, n0, pass_h, true, &nt, &slices);
    const char* xp = (const char*)x + (size_t)n0 * H * xs;
    if (q8::launch_glu(*dev, G, U, xp, xf, h + (size_t)n0 * F, false, nt, s, &SG, gd + n0,
                       slices) != hipSuccess)
      return Q8_ERR_LAUNCH;
  }
  for (int n0 = 0, nt, slices; n0 < T; n0 += nt * slices) {
    next_launch(T, n0, pass_f, true, &nt, &slices);
    if (q8::launch_gemv(*dev, D, nullptr, h + (size_t)n0 * F, true, F, out + (size_t)n0 * H,
                        nullptr, false, nt, s, gd + n0, slices) != hipSuccess)
      return Q8_ERR_LAUNCH;
  }
  return Q8_OK;
}

// ------------------------------------------------------------ router
static int check_topk(const float* logits, int T, int E, int topk, const int32_t* ids,
                      const float* gate_w) {
  if (!logits || !ids || !gate_w) return Q8_ERR_NULL;
  if (T < 1 || E < 1 || E > q8::kRouterMaxE || topk < 1 || topk > E || topk > q8::kRouterMaxK)
    return Q8_ERR_SHAPE;
  if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(gate_w, 4)) return Q8_ERR_ALIGN;
  const size_t lb = (size_t)T * E * 4, ob = (size_t)T * topk * 4;
  if (overlap(logits, lb, ids, ob) || overlap(logits, lb, gate_w, ob) || overlap(ids, ob, gate_w, ob))
    return Q8_ERR_ALIAS;
  return Q8_OK;
}

int q8_moe_topk_softmax(const float* logits, int T, int E, int topk, int32_t* expert_ids,
                        float* gate_w, void* stream) {
  int rc = check_topk(logits, T, E, topk, expert_ids, gate_w);
  if (rc) return rc;
  const DevInfo* dev = nullptr;
  rc = current_device(&dev);
  if (rc) return rc;
  return launch_rc(
      q8::launch_topk_softmax(logits, T, E, topk, expert_ids, gate_w, (hipStream_t)stream));
}

int q8_moe_router(const q8_matrix* Wr, const void* x, int x_dt, int T, int topk, float* logits,
                  int32_t* expert_ids, float* gate_w, void* stream) {
  int rc = check_matrix(Wr);
  if (rc) return rc;
  if (!x) return Q8_ERR_NULL;
  rc = check_topk(logits, T, (int)Wr->M, topk, expert_ids, gate_w);
  if (rc) return rc;
  const size_t xs = dt_size(x_dt);
  if (!xs) return Q8_ERR_DTYPE;
  const size_t xb = (size_t)T * Wr->K * xs, ob = (size_t)T * topk * 4;
  if (overlap(x, xb, expert_ids, ob) || overlap(x, xb, gate_w, ob)) return Q8_ERR_ALIAS;
  if (!aligned(x, 16)) return Q8_ERR_ALIGN;
  if (overlap(x, xb, logits, (size_t)T * Wr->M * 4)) return Q8_ERR_ALIAS;
  // The GEMV (all its passes in one launch where it can), then the top-k.
  rc = gemv_impl(Wr, nullptr, x, x_dt, logits, nullptr, Q8_DT_F32, T, stream);
  if (rc) return rc;
  return launch_rc(q8::launch_topk_softmax(logits, T, (int)Wr->M, topk, expert_ids, gate_w,
                                           (hipStream_t)stream));
}

}  // extern "C"
