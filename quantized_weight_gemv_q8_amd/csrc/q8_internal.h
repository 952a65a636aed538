// q8_internal.h -- host-side interface between the C ABI (q8_api.cpp) and
// the kernel launchers (*.hip). Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "q8_format.h"

namespace q8 {

// Tokens per pass of the dense GEMV, the pair and the SiLU pair (passes of
// 9..16 tokens run a kernel with a runtime token count; other kernels take
// passes of at most 8).
constexpr int kMaxNTWide = 16;

struct DevInfo {
  int device;
  int cus;             // compute units
  size_t lds_per_block;  // bytes of dynamic LDS a workgroup may use
  bool gfx950;
};

struct HMat {  // host view of one packed matrix
  const int8_t* qs;
  const uint16_t* d;
  int64_t M, K, ld_qs, ld_d;
  int fmt;  // kFmtQ8 or kFmtQ4
};

struct HBank {
  HMat e0;
  int64_t stride_qs, stride_d;
  int E;
};

// Lanes per row team for a given K (K only: keeps per-token results
// independent of N and of the kernel that runs the row). Chosen from the
// number of 16-byte chunks, K/16 for Q8_0.
int lanes_per_row(int64_t K);
inline int lanes_for(int fmt, int64_t K) { return lanes_per_row(fmt == kFmtQ4 ? K / 2 : K); }

// Calls fn(F, LPR, XF32) with the runtime format, lane count and x type as
// compile-time constants (std::integral_constant values).
template <class Fn>
inline hipError_t dispatch_chunks(int fmt, int lpr, bool x_f32, Fn&& fn) {
  auto by_x = [&](auto f, auto l) -> hipError_t {
    if (x_f32) return fn(f, l, std::true_type{});
    return fn(f, l, std::false_type{});
  };
  auto by_l = [&](auto f) -> hipError_t {
    if (lpr == 64) return by_x(f, std::integral_constant<int, 64>{});
    if (lpr == 32) return by_x(f, std::integral_constant<int, 32>{});
    return by_x(f, std::integral_constant<int, 16>{});
  };
  if (fmt == kFmtQ4) return by_l(std::integral_constant<int, kFmtQ4>{});
  return by_l(std::integral_constant<int, kFmtQ8>{});
}

// Resident workgroups of kernel `fn` per compute unit at `lds` bytes of
// dynamic LDS and `threads` threads per workgroup, from the runtime's
// occupancy calculator; cached per (kernel, lds, threads). Persistent grids
// launch cus * this many blocks.
int blocks_per_cu(const void* fn, size_t lds, int threads);
// Lets kernel fn take `bytes` of dynamic LDS (above the default 64 KiB);
// the attribute is set once per kernel and size, not on every launch.
hipError_t allow_dynamic_lds(const void* fn, size_t bytes);

// LDS bytes for x of one pass of nt tokens of K activations.
inline size_t x_lds_bytes(int nt, int64_t K, bool x_f32) {
  return (size_t)nt * (size_t)K * (x_f32 ? 4 : 2);
}

// Largest token count per pass that fits the LDS limit (<= 8), 0 if none.
int max_tokens_per_pass(const DevInfo& dev, int64_t K, bool x_f32);
// The same for the dense GEMV, the pair and the SiLU pair, whose passes of
// 9..16 tokens run one kernel with the token count as a runtime value
// (<= 16), when wide_pass_applies.
int max_tokens_per_pass_wide(const DevInfo& dev, int64_t K, bool x_f32);
// Whether passes of 9..16 tokens over `rows` rows (2M for the SiLU pair)
// take the wide kernel; otherwise passes are of at most 8 tokens.
bool wide_pass_applies(const DevInfo& dev, int fmt, int64_t K, bool x_f32, int64_t rows);

// y[n] = A x[n] (and yb[n] = B x[n] when B != nullptr) for nt <= 16 tokens.
// With gate set (fp32 y, no B): y[n] += sigmoid(gate[n]) * (A x[n]).
// slices > 1 (nt <= 8): that many passes of nt tokens (slices * nt tokens,
// x and y advancing by nt rows per pass), in one launch where the
// one-group kernel applies, else one launch per pass.
hipError_t launch_gemv(const DevInfo& dev, const HMat& A, const HMat* B, const void* x,
                       bool x_f32, int64_t ldx, void* ya, void* yb, bool y_f16, int nt,
                       hipStream_t s, const float* gate = nullptr, int slices = 1);

// LM head pass: logits (may be null) and ids [nt]. The workspace holds the
// argmax slots and counters; it must be zero before the first pass and is
// zero again after each completed pass.
size_t lmhead_ws_bytes(int64_t V);
// Tokens per LM-head pass: the x image of a pass plus the fused kernel's
// static LDS fit one workgroup's LDS (<= 8; 0 if not even one token fits).
int lmhead_max_tokens_per_pass(const DevInfo& dev, int64_t K, bool x_f32);
hipError_t launch_lmhead(const DevInfo& dev, const HMat& W, const int32_t* row_ids, const void* x,
                         bool x_f32, float* logits, int64_t ld_logits, int32_t* ids, char* ws,
                         int nt, hipStream_t s);

// The scratch array of the entry points that allocate nothing: its
// address on device `device`, which must be the current device (taken
// once per device with hipGetSymbolAddress, q8_noalloc.hip).
// kNoAllocScratchBytes is its size.
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
hipError_t noalloc_scratch(int device, void** ptr);

// Routed experts.
struct MoeWs {
  int32_t* counts;   // [E]
  int32_t* offsets;  // [E+1]
  int32_t* pairs;    // [P]
  int32_t* active;   // [E]
  int32_t* n_active; // [1]
  int32_t* n_vslots; // [1], after n_active
  int32_t* n_bad_ids; // [1], after n_vslots: pairs with an out-of-range expert id
  float* h;          // [P][F] or null
  float* y_pair;     // [P][Mout] or null
  int32_t* vslots;   // [moe_max_vslots(E, P)][8]: expert, token count, pair ids
};

// Areas of the workspace: the seven documented ones, then the slot records.
constexpr int kMoeWsAreas = 8;
size_t moe_ws_layout(int E, int T, int topk, int64_t F, int64_t M, size_t off[kMoeWsAreas]);
int moe_max_vslots(int E, int P);
// Whether a routed workgroup's LDS image of activations (the rows of the
// tokens of the virtual slots it stages at once) fits for this K.
bool moe_fits(const DevInfo& dev, int64_t K, bool x_f32);

hipError_t launch_moe_route(const int32_t* ids, int E, int P, const MoeWs& ws, float* zero_rows,
                            int64_t zero_ld, hipStream_t s);
// The routing a routed launch needs first: ids null when the workspace
// already holds it (a later kernel of the same layer); otherwise the
// launch routes (inside the kernel when its LDS has room, else with a
// separate route launch before it) and zeroes the zero_rows rows of pairs
// with out-of-range expert ids.
struct RouteReq {
  const int32_t* ids;
  int E, P;
  float* zero_rows;
  int64_t zero_ld;
};
// Routed GEMV over a bank: y_pair[p] = W[e_p] x[src(p)]; src(p) = p / topk
// (x_per_pair false) or p. x fp16 or fp32.
hipError_t launch_moe_gemv(const DevInfo& dev, const HBank& W, const MoeWs& ws, int topk,
                           const void* x, bool x_f32, bool x_per_pair, float* y_pair,
                           const RouteReq& rq, hipStream_t s);
// h[p] = silu(Wg[e_p] x_t) * (Wu[e_p] x_t), x fp16 [T][H].
hipError_t launch_moe_gate_up(const DevInfo& dev, const HBank& G, const HBank& U,
                              const MoeWs& ws, int topk, const void* x, bool x_f32, float* h,
                              const RouteReq& rq, hipStream_t s);
// h[n][m] = silu(G x_n)[m] * (U x_n)[m]; G, U of one shape; h fp32 or fp16.
// With extra (one row of the same K and format): xdot[n] = extra . x_n too,
// in the same launch.
// slices as for launch_gemv.
hipError_t launch_glu(const DevInfo& dev, const HMat& G, const HMat& U, const void* x,
                      bool x_f32, void* h, bool h_f16, int nt, hipStream_t s,
                      const HMat* extra = nullptr, float* xdot = nullptr, int slices = 1);
// Router: ids [T][topk] and softmax weights [T][topk] from logits [T][E].
constexpr int kRouterMaxE = 4096;  // 64 experts per lane of the token's wave
constexpr int kRouterMaxK = 64;    // one picked logit per lane
hipError_t launch_topk_softmax(const float* logits, int T, int E, int topk, int32_t* ids,
                               float* gate_w, hipStream_t s);
// out[t] = sum_j gate_w[t][j] * y_pair[t*topk + j] (slots with invalid ids skipped).
hipError_t launch_moe_combine(const int32_t* ids, int E, const float* gate_w,
                              const float* y_pair, float* out, int T, int topk, int64_t M,
                              hipStream_t s);

}  // namespace q8
