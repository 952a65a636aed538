// q8_moe.hip -- routed-expert Q8_0 GEMVs with expert-major CSR dispatch.
//
// Decode-time MoE touches only the experts the router picked; the pages
// batch the routed (token, slot) pairs by expert so each active expert's
// weights stream once for all of its tokens (memra wiki, feature list:
// "MoE ... expert-major CSR batching"), keep routing and lengths on the
// device so the step stays graph-replayable ("graph-replayable
// device-length counters"), and require a token's outputs not to depend on
// its co-arrivals (memra performance, serving exactness arc).
//
// Kernels:
//  route    one workgroup: counts, offsets, expert-major pair list (stable:
//           ascending pair id inside an expert) and the active-expert list.
//  gate_up  grid (active-expert slot, row tile): the gate and up rows of the
//           same output index are a team's two rows, so the epilogue has
//           both sums in one lane and writes h = silu(g) * u.
//  rows     grid (active-expert slot, row tile): y_pair[p] = W[e] x_p for a
//           bank (the down projection, or a single routed GEMV).
//  combine  out[t] = sum_j gate_w[t][j] * y_pair[t*topk + j], ascending j.
// Per-(row, token) arithmetic is the engine's, which does not depend on
// how many tokens an expert received, so a token's result is independent
// of the rest of the batch.
#include "q8_engine.hpp"
#include "q8_internal.h"

namespace q8 {

__global__ __launch_bounds__(1024) void moe_route_kernel(const int32_t* ids, int E, int P,
                                                         MoeWs ws, float* zero_rows,
                                                         int64_t zero_ld) {
  extern __shared__ int32_t sm[];
  int32_t* cnt = sm;              // [E]
  int32_t* off = sm + E;          // [E+1]
  int32_t* sid = sm + 2 * E + 1;  // [P]
  const int tid = threadIdx.x, nth = blockDim.x;
  for (int e = tid; e < E; e += nth) cnt[e] = 0;
  for (int p = tid; p < P; p += nth) sid[p] = ids[p];
  __syncthreads();
  for (int p = tid; p < P; p += nth) {
    const int e = sid[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int o = 0, na = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = o;
      o += cnt[e];
      if (cnt[e] > 0) ws.active[na++] = e;
    }
    off[E] = o;
    *ws.n_active = na;
  }
  __syncthreads();
  for (int e = tid; e < E; e += nth) {
    ws.counts[e] = cnt[e];
    ws.offsets[e] = off[e];
  }
  if (tid == 0) ws.offsets[E] = off[E];
  for (int p = tid; p < P; p += nth) {
    const int e = sid[p];
    if (e >= 0 && e < E) {
      int rank = 0;
      for (int q = 0; q < p; ++q) rank += (sid[q] == e);
      ws.pairs[off[e] + rank] = p;
    } else if (zero_rows) {
      for (int64_t m = 0; m < zero_ld; ++m) zero_rows[(int64_t)p * zero_ld + m] = 0.0f;
    }
  }
}

// ---------------------------------------------------------------- shared pieces
struct ExpertMat {
  const int8_t* qs;
  const uint16_t* d;
  int64_t ld_qs, ld_d;
};

__device__ __forceinline__ ExpertMat expert_of(const HBank& b, int e) {
  ExpertMat m;
  m.qs = b.e0.qs + (int64_t)e * b.stride_qs;
  m.d = b.e0.d + (int64_t)e * b.stride_d;
  m.ld_qs = b.e0.ld_qs;
  m.ld_d = b.e0.ld_d;
  return m;
}

struct SingleMap {
  ExpertMat w;
  int64_t M;      // rows of the expert matrix
  int64_t r_end;  // end of this workgroup's row tile
  __device__ __forceinline__ bool row(int64_t i, const int8_t*& q, const uint16_t*& d) const {
    q = w.qs + i * w.ld_qs;
    d = w.d + i * w.ld_d;
    return i < r_end;
  }
};

// virtual row i = 2*rho + s: s = 0 gate row rho, s = 1 up row rho
struct GateUpMap {
  ExpertMat g, u;
  int64_t r_end;  // end (virtual rows) of this tile
  __device__ __forceinline__ bool row(int64_t i, const int8_t*& q, const uint16_t*& d) const {
    const int64_t rho = i >> 1;
    const bool up = (i & 1) != 0;
    q = up ? u.qs + rho * u.ld_qs : g.qs + rho * g.ld_qs;
    d = up ? u.d + rho * u.ld_d : g.d + rho * g.ld_d;
    return i < r_end;
  }
};

struct PairOutEpi {  // y[pid[n]][row] = v
  float* y;
  int64_t ld;
  int64_t r_end;
  const int32_t* pid;  // LDS, [NT]
  template <int NT, int R, int CNT>
  __device__ __forceinline__ void emit(int64_t rbase, int base, bool owner, const float* v) {
    if (!owner) return;
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = base + i;
      if (idx >= NT * R) continue;
      const int n = idx / R, r = idx - (idx / R) * R;
      const int64_t row = rbase + r;
      if (row >= r_end) continue;
      y[(int64_t)pid[n] * ld + row] = v[i];
    }
  }
};

struct SiluMulEpi {  // values come in (gate, up) pairs for one token
  float* h;
  int64_t ld;
  int64_t r_end;  // virtual rows
  const int32_t* pid;
  template <int NT, int R, int CNT>
  __device__ __forceinline__ void emit(int64_t rbase, int base, bool owner, const float* v) {
    static_assert(R == 2 && CNT == 2, "gate/up pairs");
    if (!owner) return;
    const int n = base / 2;
    if (n >= NT || rbase >= r_end) return;
    const float g = v[0], u = v[1];
    const float sg = g / (1.0f + expf(-g));
    h[(int64_t)pid[n] * ld + (rbase >> 1)] = sg * u;
  }
};

template <int NT, bool XF32, class Map, class Epi, int R, int MINC, int LPR>
__device__ __forceinline__ void expert_pass(const Map& map, Epi& epi, const char* x,
                                            int64_t ldx_bytes, bool x_per_pair, int topk,
                                            const int32_t* pid_lds, int C, int64_t r_begin,
                                            int64_t r_end, uint4* lds) {
  const char* rows[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int p = pid_lds[n];
    const int src = x_per_pair ? p : p / topk;
    rows[n] = x + (int64_t)src * ldx_bytes;
  }
  stage_x<NT, XF32>(rows, C, lds);
  __syncthreads();
  constexpr int G = (kWave / LPR) * R;
  const int64_t n_groups = (r_end - r_begin + G - 1) / G;
  run_rows<NT, LPR, R, MINC, XF32>(map, epi, lds, C, n_groups, threadIdx.x / kWave,
                                   kWavesPerBlock, r_begin);
  __syncthreads();
}

// Token-count dispatch inside one workgroup (the count is per expert and
// only known on the device).
template <bool XF32, class Map, class Epi, int MINC, int LPR, int RFIX>
__device__ __forceinline__ void expert_tokens(const Map& map, Epi& epi, const char* x,
                                              int64_t ldx_bytes, bool x_per_pair, int topk,
                                              int32_t* pid_lds, const int32_t* pairs, int ne,
                                              int C, int64_t r_begin, int64_t r_end, uint4* lds) {
  for (int t0 = 0; t0 < ne; t0 += kMaxNT) {
    const int nt = ne - t0 < kMaxNT ? ne - t0 : kMaxNT;
    if (threadIdx.x < nt) pid_lds[threadIdx.x] = pairs[t0 + threadIdx.x];
    __syncthreads();
    epi.pid = pid_lds;
#define Q8_CASE(K_)                                                                        \
  case K_:                                                                                 \
    expert_pass<K_, XF32, Map, Epi, (RFIX ? RFIX : (K_ <= 2 ? 2 : 4)), MINC, LPR>(         \
        map, epi, x, ldx_bytes, x_per_pair, topk, pid_lds, C, r_begin, r_end, lds);        \
    break;
    switch (nt) {
      Q8_CASE(1) Q8_CASE(2) Q8_CASE(3) Q8_CASE(4) Q8_CASE(5) Q8_CASE(6) Q8_CASE(7) Q8_CASE(8)
    }
#undef Q8_CASE
  }
}

struct MoeGrid {
  int64_t rows_per_tile;  // rows of one tile (virtual rows for gate/up)
};

template <int LPR, bool XF32>
__global__ __launch_bounds__(kBlock) void moe_rows_kernel(HBank W, MoeWs ws, int topk,
                                                         const char* x, int64_t ldx_bytes,
                                                         int x_per_pair, float* y,
                                                         int64_t rows_per_tile) {
  extern __shared__ uint4 lds_x[];
  __shared__ int32_t pid_lds[kMaxNT];
  const int slot = blockIdx.x;
  if (slot >= *ws.n_active) return;
  const int e = ws.active[slot];
  const int o0 = ws.offsets[e];
  const int ne = ws.offsets[e + 1] - o0;
  const int64_t M = W.e0.M;
  const int64_t r_begin = (int64_t)blockIdx.y * rows_per_tile;
  if (r_begin >= M) return;
  const int64_t r_end = r_begin + rows_per_tile < M ? r_begin + rows_per_tile : M;
  SingleMap map;
  map.w = expert_of(W, e);
  map.M = M;
  map.r_end = r_end;
  PairOutEpi epi;
  epi.y = y;
  epi.ld = M;
  epi.r_end = r_end;
  epi.pid = pid_lds;
  const int C = (int)(W.e0.K / 16);
  expert_tokens<XF32, SingleMap, PairOutEpi, 1, LPR, 0>(map, epi, x, ldx_bytes, x_per_pair != 0,
                                                         topk, pid_lds, ws.pairs + o0, ne, C,
                                                         r_begin, r_end, lds_x);
}

template <int LPR, bool XF32>
__global__ __launch_bounds__(kBlock) void moe_gate_up_kernel(HBank Gb, HBank Ub, MoeWs ws,
                                                            int topk, const char* x,
                                                            int64_t ldx_bytes, float* h,
                                                            int64_t rows_per_tile) {
  extern __shared__ uint4 lds_x[];
  __shared__ int32_t pid_lds[kMaxNT];
  const int slot = blockIdx.x;
  if (slot >= *ws.n_active) return;
  const int e = ws.active[slot];
  const int o0 = ws.offsets[e];
  const int ne = ws.offsets[e + 1] - o0;
  const int64_t F = Gb.e0.M;
  const int64_t VR = 2 * F;  // virtual rows
  const int64_t r_begin = (int64_t)blockIdx.y * rows_per_tile;
  if (r_begin >= VR) return;
  const int64_t r_end = r_begin + rows_per_tile < VR ? r_begin + rows_per_tile : VR;
  GateUpMap map;
  map.g = expert_of(Gb, e);
  map.u = expert_of(Ub, e);
  map.r_end = r_end;
  SiluMulEpi epi;
  epi.h = h;
  epi.ld = F;
  epi.r_end = r_end;
  epi.pid = pid_lds;
  const int C = (int)(Gb.e0.K / 16);
  expert_tokens<XF32, GateUpMap, SiluMulEpi, 2, LPR, 2>(map, epi, x, ldx_bytes, false, topk,
                                                         pid_lds, ws.pairs + o0, ne, C, r_begin,
                                                         r_end, lds_x);
}

__global__ __launch_bounds__(256) void moe_combine_kernel(const int32_t* ids, int E,
                                                         const float* gate_w, const float* yp,
                                                         float* out, int topk, int64_t M) {
  const int t = blockIdx.y;
  const int64_t m = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  float acc = 0.0f;
  for (int j = 0; j < topk; ++j) {
    const int e = ids[t * topk + j];
    if (e < 0 || e >= E) continue;
    acc = __builtin_fmaf(gate_w[t * topk + j], yp[((int64_t)t * topk + j) * M + m], acc);
  }
  out[(int64_t)t * M + m] = acc;
}

// ---------------------------------------------------------------- host side
static int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

size_t moe_ws_layout(int E, int T, int topk, int64_t F, int64_t M, size_t off[7]) {
  const int64_t P = (int64_t)T * topk;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = (size_t)round_up((int64_t)(o + bytes), 256);
    return at;
  };
  off[0] = take(4 * (size_t)E);
  off[1] = take(4 * (size_t)(E + 1));
  off[2] = take(4 * (size_t)P);
  off[3] = take(4 * (size_t)E);
  off[4] = take(4);
  off[5] = take(F > 0 ? 4 * (size_t)P * (size_t)F : 0);
  off[6] = take(4 * (size_t)P * (size_t)M);
  return o;
}

hipError_t launch_moe_route(const int32_t* ids, int E, int P, const MoeWs& ws, float* zero_rows,
                            int64_t zero_ld, hipStream_t s) {
  const size_t lds = 4 * (size_t)(2 * E + 1 + P);
  int threads = 256;
  if (P > 256 || E > 256) threads = 1024;
  MoeWs w = ws;
  void* args[] = {(void*)&ids, &E, &P, &w, &zero_rows, &zero_ld};
  return hipLaunchKernel((const void*)moe_route_kernel, dim3(1), dim3(threads), args, lds, s);
}

static int64_t tiles_for(const DevInfo& dev, int slots, int64_t rows, int64_t row_quantum) {
  int64_t tiles = (4LL * dev.cus + slots - 1) / slots;
  if (tiles < 1) tiles = 1;
  const int64_t max_tiles = (rows + row_quantum - 1) / row_quantum;
  if (tiles > max_tiles) tiles = max_tiles;
  return tiles;
}

template <int LPR, bool XF32>
static hipError_t moe_rows_t(const DevInfo& dev, const HBank& W, const MoeWs& ws, int P, int topk,
                             const char* x, int64_t ldx_bytes, int x_per_pair, float* y,
                             hipStream_t s) {
  const int slots = P < W.E ? P : W.E;
  const int64_t M = W.e0.M;
  const int64_t quantum = (int64_t)kWavesPerBlock * (kWave / LPR) * 4;
  const int64_t tiles = tiles_for(dev, slots, M, quantum);
  int64_t rpt = round_up((M + tiles - 1) / tiles, (kWave / LPR) * 4);
  const size_t lds = (size_t)kMaxNT * (W.e0.K / 16) * 16 * XPlanes<XF32>::P;
  auto fn = moe_rows_kernel<LPR, XF32>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  HBank w = W;
  MoeWs wsv = ws;
  void* args[] = {&w, &wsv, &topk, (void*)&x, &ldx_bytes, &x_per_pair, &y, &rpt};
  const int64_t ty = (M + rpt - 1) / rpt;
  return hipLaunchKernel((const void*)fn, dim3((unsigned)slots, (unsigned)ty), dim3(kBlock), args,
                         lds, s);
}

hipError_t launch_moe_gemv(const DevInfo& dev, const HBank& W, const MoeWs& ws, int P, int topk,
                           const void* x, bool x_f32, bool x_per_pair, float* y_pair,
                           hipStream_t s) {
  const int64_t ldx_bytes = W.e0.K * (x_f32 ? 4 : 2);
  const char* xp = (const char*)x;
  const int lpr = lanes_per_row(W.e0.K);
  const int xpp = x_per_pair ? 1 : 0;
  if (x_f32) {
    if (lpr == 64) return moe_rows_t<64, true>(dev, W, ws, P, topk, xp, ldx_bytes, xpp, y_pair, s);
    if (lpr == 32) return moe_rows_t<32, true>(dev, W, ws, P, topk, xp, ldx_bytes, xpp, y_pair, s);
    return moe_rows_t<16, true>(dev, W, ws, P, topk, xp, ldx_bytes, xpp, y_pair, s);
  }
  if (lpr == 64) return moe_rows_t<64, false>(dev, W, ws, P, topk, xp, ldx_bytes, xpp, y_pair, s);
  if (lpr == 32) return moe_rows_t<32, false>(dev, W, ws, P, topk, xp, ldx_bytes, xpp, y_pair, s);
  return moe_rows_t<16, false>(dev, W, ws, P, topk, xp, ldx_bytes, xpp, y_pair, s);
}

template <int LPR, bool XF32>
static hipError_t moe_gu_t(const DevInfo& dev, const HBank& G, const HBank& U, const MoeWs& ws,
                           int P, int topk, const char* x, int64_t ldx_bytes, float* h,
                           hipStream_t s) {
  const int slots = P < G.E ? P : G.E;
  const int64_t VR = 2 * G.e0.M;
  const int64_t quantum = (int64_t)kWavesPerBlock * (kWave / LPR) * 2;
  const int64_t tiles = tiles_for(dev, slots, VR, quantum);
  int64_t rpt = round_up((VR + tiles - 1) / tiles, (kWave / LPR) * 2);
  const size_t lds = (size_t)kMaxNT * (G.e0.K / 16) * 16 * XPlanes<XF32>::P;
  auto fn = moe_gate_up_kernel<LPR, XF32>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  HBank g = G, u = U;
  MoeWs wsv = ws;
  void* args[] = {&g, &u, &wsv, &topk, (void*)&x, &ldx_bytes, &h, &rpt};
  const int64_t ty = (VR + rpt - 1) / rpt;
  return hipLaunchKernel((const void*)fn, dim3((unsigned)slots, (unsigned)ty), dim3(kBlock), args,
                         lds, s);
}

hipError_t launch_moe_gate_up(const DevInfo& dev, const HBank& G, const HBank& U,
                              const MoeWs& ws, int P, int topk, const void* x, bool x_f32,
                              float* h, hipStream_t s) {
  const int64_t ldx_bytes = G.e0.K * (x_f32 ? 4 : 2);
  const char* xp = (const char*)x;
  const int lpr = lanes_per_row(G.e0.K);
  if (x_f32) {
    if (lpr == 64) return moe_gu_t<64, true>(dev, G, U, ws, P, topk, xp, ldx_bytes, h, s);
    if (lpr == 32) return moe_gu_t<32, true>(dev, G, U, ws, P, topk, xp, ldx_bytes, h, s);
    return moe_gu_t<16, true>(dev, G, U, ws, P, topk, xp, ldx_bytes, h, s);
  }
  if (lpr == 64) return moe_gu_t<64, false>(dev, G, U, ws, P, topk, xp, ldx_bytes, h, s);
  if (lpr == 32) return moe_gu_t<32, false>(dev, G, U, ws, P, topk, xp, ldx_bytes, h, s);
  return moe_gu_t<16, false>(dev, G, U, ws, P, topk, xp, ldx_bytes, h, s);
}

hipError_t launch_moe_combine(const int32_t* ids, int E, const float* gate_w,
                              const float* y_pair, float* out, int T, int topk, int64_t M,
                              hipStream_t s) {
  void* args[] = {(void*)&ids, &E, (void*)&gate_w, (void*)&y_pair, &out, &topk, &M};
  const unsigned gx = (unsigned)((M + 255) / 256);
  return hipLaunchKernel((const void*)moe_combine_kernel, dim3(gx, (unsigned)T), dim3(256), args, 0,
                         s);
}

}  // namespace q8
