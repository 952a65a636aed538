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

constexpr int kRouteThreads = 1024;

// Block-wide exclusive scan of one int per thread (kRouteThreads threads).
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int t = threadIdx.x;
  tmp[t] = v;
  __syncthreads();
  for (int off = 1; off < kRouteThreads; off <<= 1) {
    const int add = t >= off ? tmp[t - off] : 0;
    __syncthreads();
    tmp[t] += add;
    __syncthreads();
  }
  const int incl = tmp[t];
  *total = tmp[kRouteThreads - 1];
  __syncthreads();
  return incl - v;
}

// Expert-major CSR of the routed pairs in one workgroup: counts by LDS
// atomics, offsets and the active list by block scans, pairs scattered by
// atomic cursors and then put in ascending pair order inside each expert,
// so the result does not depend on the order the atomics happened in.
__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(const int32_t* ids, int E, int P,
                                                                 MoeWs ws, float* zero_rows,
                                                                 int64_t zero_ld) {
  extern __shared__ int32_t sm[];
  __shared__ int scan_tmp[kRouteThreads];
  int32_t* cnt = sm;              // [E]
  int32_t* off = cnt + E;         // [E+1]
  int32_t* cur = off + E + 1;     // [E]
  int32_t* sid = cur + E;         // [P]
  int32_t* tmp = sid + P;         // [P]
  const int t = threadIdx.x;
  for (int e = t; e < E; e += kRouteThreads) cnt[e] = 0;
  for (int p = t; p < P; p += kRouteThreads) {
    const int e = ids[p];
    sid[p] = (e >= 0 && e < E) ? e : -1;
  }
  __syncthreads();
  for (int p = t; p < P; p += kRouteThreads)
    if (sid[p] >= 0) atomicAdd(&cnt[sid[p]], 1);
  __syncthreads();
  // each thread owns a contiguous run of experts
  const int per = (E + kRouteThreads - 1) / kRouteThreads;
  const int e0 = t * per, e1 = e0 + per < E ? e0 + per : E;
  int sum = 0, act = 0;
  for (int e = e0; e < e1; ++e) {
    sum += cnt[e];
    act += cnt[e] > 0;
  }
  int total_pairs, total_active;
  const int base = block_exclusive_scan(sum, scan_tmp, &total_pairs);
  const int abase = block_exclusive_scan(act, scan_tmp, &total_active);
  {
    int o = base, a = abase;
    for (int e = e0; e < e1; ++e) {
      off[e] = o;
      cur[e] = o;
      ws.counts[e] = cnt[e];
      ws.offsets[e] = o;
      if (cnt[e] > 0) ws.active[a++] = e;
      o += cnt[e];
    }
  }
  if (t == 0) {
    off[E] = total_pairs;
    ws.offsets[E] = total_pairs;
    *ws.n_active = total_active;
  }
  __syncthreads();
  for (int p = t; p < P; p += kRouteThreads) {
    const int e = sid[p];
    if (e >= 0) {
      tmp[atomicAdd(&cur[e], 1)] = p;
    } else if (zero_rows) {
      for (int64_t m = 0; m < zero_ld; ++m) zero_rows[(int64_t)p * zero_ld + m] = 0.0f;
    }
  }
  __syncthreads();
  for (int e = t; e < E; e += kRouteThreads) {
    const int lo = off[e], hi = off[e + 1];
    for (int i = lo + 1; i < hi; ++i) {  // insertion sort: segments are short
      const int v = tmp[i];
      int j = i - 1;
      while (j >= lo && tmp[j] > v) {
        tmp[j + 1] = tmp[j];
        --j;
      }
      tmp[j + 1] = v;
    }
    for (int i = lo; i < hi; ++i) ws.pairs[i] = tmp[i];
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

struct PairOutEpi {  // y[pid[n]][row] = v for live tokens n < nt
  float* y;
  int64_t ld;
  int64_t r_end;
  const int32_t* pid;  // LDS, [nt]
  int nt;
  template <int NT, int R, int CNT>
  __device__ __forceinline__ void emit(int64_t rbase, int base, bool owner, const float* v) {
    if (!owner) return;
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = base + i;
      if (idx >= NT * R) continue;
      const int n = idx / R, r = idx - (idx / R) * R;
      const int64_t row = rbase + r;
      if (n >= nt || row >= r_end) continue;
      y[(int64_t)pid[n] * ld + row] = v[i];
    }
  }
};

struct SiluMulEpi {  // values come in (gate, up) pairs for one token
  float* h;
  int64_t ld;
  int64_t r_end;  // virtual rows
  const int32_t* pid;  // LDS, [nt]
  int nt;
  template <int NT, int R, int CNT>
  __device__ __forceinline__ void emit(int64_t rbase, int base, bool owner, const float* v) {
    static_assert(R == 2 && CNT == 2, "gate/up pairs");
    if (!owner) return;
    const int n = base / 2;
    if (n >= nt || rbase >= r_end) return;
    const float g = v[0], u = v[1];
    const float sg = g / (1.0f + expf(-g));
    h[(int64_t)pid[n] * ld + (rbase >> 1)] = sg * u;
  }
};

// Tokens per pass for routed experts (most experts receive one or two
// tokens: 128 pairs over ~80 active experts). An expert with more tokens
// takes several passes over its tile, the later ones served from L2. The
// load window is one chunk (D = 1). Both were picked by same-process A/B
// on MI355X for the 128-expert top-8 T=16 layer (184 -> 134 us against a
// 2-token pass with D = 4; wider passes and other tile sizes were slower).
constexpr int kMoeNT = 4;

template <int NT, bool XF32, int R, int D, int MINC, int LPR, class Map, class Epi>
__device__ __forceinline__ void expert_pass(const Map& map, Epi& epi, const char* x,
                                            int64_t ldx_bytes, bool x_per_pair, int topk,
                                            const int32_t* pid_lds, int C, int64_t r_begin,
                                            int64_t r_end, uint4* lds, int nt) {
  constexpr int G = (kWave / LPR) * R;
  const int64_t n_groups = (r_end - r_begin + G - 1) / G;
  auto stage = [=]() {
    const char* rows[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int p = n < nt ? pid_lds[n] : 0;
      const int src = x_per_pair ? p : p / topk;
      rows[n] = x + (int64_t)src * ldx_bytes;
    }
    stage_x<NT, XF32>(rows, C, lds, nt);
    __syncthreads();
  };
  run_rows<NT, LPR, R, D, MINC, XF32>(map, epi, lds, C, n_groups, threadIdx.x / kWave,
                                      kWavesPerBlock, r_begin, stage, nt);
}

// Persistent loop over work items (active-expert slot, row tile); for each,
// passes of up to kMoeNT of the expert's routed pairs.
template <bool XF32, int MINC, int LPR, int RFIX, class MakeMap, class Epi>
__device__ __forceinline__ void expert_items(const MoeWs& ws, int64_t tiles, int64_t rows_per_tile,
                                             int64_t rows_total, const MakeMap& make_map, Epi& epi,
                                             const char* x, int64_t ldx_bytes, bool x_per_pair,
                                             int topk, int C, int32_t* pid_lds, uint4* lds) {
  const int64_t items = (int64_t)__builtin_amdgcn_readfirstlane(*ws.n_active) * tiles;
  for (int64_t wi = blockIdx.x; wi < items; wi += gridDim.x) {
    const int slot = (int)(wi / tiles);
    const int64_t tile = wi - (int64_t)slot * tiles;
    const int e = __builtin_amdgcn_readfirstlane(ws.active[slot]);
    const int o0 = __builtin_amdgcn_readfirstlane(ws.offsets[e]);
    const int ne = __builtin_amdgcn_readfirstlane(ws.offsets[e + 1]) - o0;
    const int64_t r_begin = tile * rows_per_tile;
    const int64_t r_end = r_begin + rows_per_tile < rows_total ? r_begin + rows_per_tile : rows_total;
    const auto map = make_map(e, r_end);
    epi.r_end = r_end;
    for (int t0 = 0; t0 < ne; t0 += kMoeNT) {
      const int nt = ne - t0 < kMoeNT ? ne - t0 : kMoeNT;
      __syncthreads();  // previous pass done with pid_lds and the LDS x image
      if (threadIdx.x < nt) pid_lds[threadIdx.x] = ws.pairs[o0 + t0 + threadIdx.x];
      __syncthreads();
      epi.pid = pid_lds;
      epi.nt = nt;
      expert_pass<kMoeNT, XF32, (RFIX ? RFIX : Tune<kMoeNT, false>::R), 1, MINC, LPR>(
          map, epi, x, ldx_bytes, x_per_pair, topk, pid_lds, C, r_begin, r_end, lds, nt);
    }
  }
}

template <int LPR, bool XF32>
__global__ __launch_bounds__(kBlock) void moe_rows_kernel(HBank W, MoeWs ws, int topk,
                                                         const char* x, int64_t ldx_bytes,
                                                         int x_per_pair, float* y, int64_t tiles,
                                                         int64_t rows_per_tile) {
  extern __shared__ uint4 lds_x[];
  __shared__ int32_t pid_lds[kMoeNT];
  const int64_t M = W.e0.M;
  PairOutEpi epi;
  epi.y = y;
  epi.ld = M;
  epi.pid = pid_lds;
  auto make_map = [&](int e, int64_t r_end) {
    SingleMap m;
    m.w = expert_of(W, e);
    m.M = M;
    m.r_end = r_end;
    return m;
  };
  expert_items<XF32, 1, LPR, 0>(ws, tiles, rows_per_tile, M, make_map, epi, x, ldx_bytes,
                                x_per_pair != 0, topk, (int)(W.e0.K / 16), pid_lds, lds_x);
}

template <int LPR, bool XF32>
__global__ __launch_bounds__(kBlock) void moe_gate_up_kernel(HBank Gb, HBank Ub, MoeWs ws,
                                                            int topk, const char* x,
                                                            int64_t ldx_bytes, float* h,
                                                            int64_t tiles, int64_t rows_per_tile) {
  extern __shared__ uint4 lds_x[];
  __shared__ int32_t pid_lds[kMoeNT];
  const int64_t F = Gb.e0.M;
  SiluMulEpi epi;
  epi.h = h;
  epi.ld = F;
  epi.pid = pid_lds;
  auto make_map = [&](int e, int64_t r_end) {
    GateUpMap m;
    m.g = expert_of(Gb, e);
    m.u = expert_of(Ub, e);
    m.r_end = r_end;
    return m;
  };
  expert_items<XF32, 2, LPR, 2>(ws, tiles, rows_per_tile, 2 * F, make_map, epi, x, ldx_bytes,
                                false, topk, (int)(Gb.e0.K / 16), pid_lds, lds_x);
}

__global__ __launch_bounds__(256) void moe_combine_kernel(const int32_t* ids, int E,
                                                         const float* gate_w, const float* yp,
                                                         float* out, int topk, int64_t M) {
  const int t = blockIdx.y;
  const int64_t m0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (m0 >= M) return;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j = 0; j < topk; ++j) {
    const int e = ids[t * topk + j];
    if (e < 0 || e >= E) continue;
    const float w = gate_w[t * topk + j];
    const float* row = yp + ((int64_t)t * topk + j) * M;
    if ((M & 3) == 0) {
      const float4 v = *reinterpret_cast<const float4*>(row + m0);
      acc[0] = __builtin_fmaf(w, v.x, acc[0]);
      acc[1] = __builtin_fmaf(w, v.y, acc[1]);
      acc[2] = __builtin_fmaf(w, v.z, acc[2]);
      acc[3] = __builtin_fmaf(w, v.w, acc[3]);
    } else {
      for (int i = 0; i < 4 && m0 + i < M; ++i) acc[i] = __builtin_fmaf(w, row[m0 + i], acc[i]);
    }
  }
  for (int i = 0; i < 4 && m0 + i < M; ++i) out[(int64_t)t * M + m0 + i] = acc[i];
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
  const size_t lds = 4 * (size_t)(3 * E + 1 + 2 * P);
  MoeWs w = ws;
  void* args[] = {(void*)&ids, &E, &P, &w, &zero_rows, &zero_ld};
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)moe_route_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  return hipLaunchKernel((const void*)moe_route_kernel, dim3(1), dim3(kRouteThreads), args, lds, s);
}

// Row tiles per expert: enough work items (active experts x tiles) to give
// each resident workgroup several, each tile at least one group per wave.
static void plan_tiles(int64_t blocks, int slots, int64_t rows, int64_t group_rows, int64_t* tiles,
                       int64_t* rows_per_tile) {
  const int64_t min_rows = group_rows * kWavesPerBlock;
  int64_t t = (6 * blocks + slots - 1) / slots;
  const int64_t max_t = (rows + min_rows - 1) / min_rows;
  if (t > max_t) t = max_t;
  if (t < 1) t = 1;
  int64_t rpt = (rows + t - 1) / t;
  rpt = round_up(rpt, group_rows);
  *rows_per_tile = rpt;
  *tiles = (rows + rpt - 1) / rpt;
}

template <int LPR, bool XF32>
static hipError_t moe_rows_t(const DevInfo& dev, const HBank& W, const MoeWs& ws, int P, int topk,
                             const char* x, int64_t ldx_bytes, int x_per_pair, float* y,
                             hipStream_t s) {
  const int slots = P < W.E ? P : W.E;
  const int64_t M = W.e0.M;
  const size_t lds = (size_t)kMoeNT * (W.e0.K / 16) * 16 * XPlanes<XF32>::P;
  auto fn = moe_rows_kernel<LPR, XF32>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t blocks = (int64_t)dev.cus * blocks_per_cu((const void*)fn, lds);
  int64_t tiles, rpt;
  plan_tiles(blocks, slots, M, (kWave / LPR) * Tune<kMoeNT, false>::R, &tiles, &rpt);
  int64_t grid = slots * tiles < blocks ? slots * tiles : blocks;
  HBank w = W;
  MoeWs wsv = ws;
  void* args[] = {&w, &wsv, &topk, (void*)&x, &ldx_bytes, &x_per_pair, &y, &tiles, &rpt};
  return hipLaunchKernel((const void*)fn, dim3((unsigned)grid), dim3(kBlock), args, lds, s);
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
  const size_t lds = (size_t)kMoeNT * (G.e0.K / 16) * 16 * XPlanes<XF32>::P;
  auto fn = moe_gate_up_kernel<LPR, XF32>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t blocks = (int64_t)dev.cus * blocks_per_cu((const void*)fn, lds);
  int64_t tiles, rpt;
  plan_tiles(blocks, slots, VR, (kWave / LPR) * 2, &tiles, &rpt);
  int64_t grid = slots * tiles < blocks ? slots * tiles : blocks;
  HBank g = G, u = U;
  MoeWs wsv = ws;
  void* args[] = {&g, &u, &wsv, &topk, (void*)&x, &ldx_bytes, &h, &tiles, &rpt};
  return hipLaunchKernel((const void*)fn, dim3((unsigned)grid), dim3(kBlock), args, lds, s);
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
  const unsigned gx = (unsigned)(((M + 3) / 4 + 255) / 256);
  return hipLaunchKernel((const void*)moe_combine_kernel, dim3(gx, (unsigned)T), dim3(256), args, 0,
                         s);
}

}  // namespace q8
