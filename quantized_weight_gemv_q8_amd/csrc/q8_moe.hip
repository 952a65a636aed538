// q8_moe.hip -- routed-expert Q8_0 GEMVs with expert-major CSR dispatch.
//
// Decode-time MoE touches only the experts the router picked; the pages
// batch the routed (token, slot) pairs by expert so each active expert's
// weights stream once for all of its tokens (memra wiki, feature list, the
// MoE item: routed tokens batched per expert in CSR form), keep routing and
// lengths on the device so that the step stays replayable as a graph (same
// item: lengths counted on the device), and require a token's outputs not
// to depend on
// its co-arrivals (memra performance, serving exactness arc).
//
// Kernels:
//  route    one workgroup: counts, offsets, expert-major pair list (stable:
//           ascending pair id inside an expert), the active-expert list and
//           the virtual slots: an active expert with up to kMoeNT of its
//           pairs (an expert with more pairs gets several slots). Pairs
//           whose expert id is out of range are left out, and their number
//           is written to the workspace error word (a failure the caller
//           can read, not a silent fallback).
//  gate_up  the rows of all virtual slots form one row space (a team's two
//           rows are the gate and up rows of one output index, so the
//           epilogue has both sums in one lane and writes h = silu(g) * u);
//           each persistent workgroup streams one contiguous, equal slice
//           of it, with the activations of the slots it touches staged once.
//  rows     the same over a bank: y_pair[p] = W[e] x_p (the down
//           projection, or a single routed GEMV).
//  combine  out[t] = sum_j gate_w[t][j] * y_pair[t*topk + j], ascending j.
// Per-(row, token) arithmetic is the engine's, which does not depend on
// how many tokens an expert received or which slot they landed in, so a
// token's result is independent of the rest of the batch.
#include "q8_engine.hpp"
#include "q8_internal.h"

namespace q8 {

constexpr int kRouteThreads = 1024;

// Tokens per virtual slot. Most experts receive one or two tokens (128
// pairs over ~90 active experts at 128 experts, top-8, 16 tokens); an
// expert with more takes several slots, the later ones re-reading its rows.
// Two per slot was the fastest of 1, 2, 3 and 4 in same-process A/B on
// MI355X for that layer (95 us against 113 us for 4: the smaller
// accumulator set raises occupancy by more than the re-reads cost).
constexpr int kMoeNT = 2;
// Virtual slot record: [0] expert, [1] token count, [2 .. 2+kMoeNT) pair
// ids; 32 bytes.
constexpr int kVSlotInts = 8;
static_assert(2 + kMoeNT <= kVSlotInts, "slot record");
// Slots staged together by one workgroup (a slice no longer than one
// slot's rows touches at most two).
constexpr int kSegV = 2;

// Block-wide exclusive scan of three ints per thread (WAVES waves):
// inclusive scans inside each wave by shuffles, then the wave totals from
// LDS. Two barriers in all.
template <int WAVES>
__device__ __forceinline__ void block_exclusive_scan3(int v[3], int (*wtot)[3], int total[3]) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int incl[3] = {v[0], v[1], v[2]};
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int o = __shfl_up(incl[i], off, kWave);
      if (lane >= off) incl[i] += o;
    }
  }
  if (lane == kWave - 1) {
#pragma unroll
    for (int i = 0; i < 3; ++i) wtot[wave][i] = incl[i];
  }
  __syncthreads();
  int before[3] = {0, 0, 0};
#pragma unroll
  for (int i = 0; i < 3; ++i) total[i] = 0;
  for (int w = 0; w < WAVES; ++w) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (w < wave) before[i] += wtot[w][i];
      total[i] += wtot[w][i];
    }
  }
  __syncthreads();  // wtot may be reused
#pragma unroll
  for (int i = 0; i < 3; ++i) v[i] = before[i] + incl[i] - v[i];
}

// Expert-major CSR of the routed pairs in one workgroup: counts by LDS
// atomics, offsets and the active list by block scans, pairs scattered by
// atomic cursors and then put in ascending pair order inside each expert,
// so the result does not depend on the order the atomics happened in.
// sm: route_scratch_ints(E, P) int32 of LDS. The slot records go to
// vslots_out and their count to *nv_out (global or LDS); with write_ws the
// workspace areas (counts, offsets, pairs, active, n_active, n_vslots and,
// if vslots_out is elsewhere, the slot records) are written too, and the
// rows of pairs whose expert id is out of range are zeroed in zero_rows.
// Ends with a barrier: the records are visible to the whole workgroup.
__host__ __device__ constexpr int route_scratch_ints(int E, int P) { return 3 * E + 1 + 2 * P; }

template <int THREADS>
__device__ __forceinline__ void route_block(const int32_t* ids, int E, int P, int32_t* sm,
                                            const MoeWs& ws, bool write_ws, int32_t* vslots_out,
                                            int32_t* nv_out, float* zero_rows, int64_t zero_ld) {
  __shared__ int wtot[THREADS / kWave][3];
  __shared__ int n_bad;
  int32_t* cnt = sm;              // [E]
  int32_t* off = cnt + E;         // [E+1]
  int32_t* cur = off + E + 1;     // [E]
  int32_t* sid = cur + E;         // [P]
  int32_t* tmp = sid + P;         // [P]
  const int t = threadIdx.x;
  if (t == 0) n_bad = 0;
  for (int e = t; e < E; e += THREADS) cnt[e] = 0;
  int my_bad = 0;
  for (int p = t; p < P; p += THREADS) {
    const int e = ids[p];
    const bool ok = e >= 0 && e < E;
    sid[p] = ok ? e : -1;
    my_bad += ok ? 0 : 1;
  }
  __syncthreads();
  if (my_bad) atomicAdd(&n_bad, my_bad);
  for (int p = t; p < P; p += THREADS)
    if (sid[p] >= 0) atomicAdd(&cnt[sid[p]], 1);
  __syncthreads();
  // Each thread owns a contiguous run of experts: its pairs, its active
  // experts and its virtual slots are placed after those of lower runs.
  const int per = (E + THREADS - 1) / THREADS;
  const int e0 = t * per < E ? t * per : E, e1 = e0 + per < E ? e0 + per : E;
  int v[3] = {0, 0, 0};  // pairs, active experts, virtual slots
  for (int e = e0; e < e1; ++e) {
    v[0] += cnt[e];
    v[1] += cnt[e] > 0;
    v[2] += (cnt[e] + kMoeNT - 1) / kMoeNT;
  }
  int total[3];
  block_exclusive_scan3<THREADS / kWave>(v, wtot, total);
  {
    int o = v[0], a = v[1];
    for (int e = e0; e < e1; ++e) {
      off[e] = o;
      cur[e] = o;
      if (write_ws) {
        ws.counts[e] = cnt[e];
        ws.offsets[e] = o;
        if (cnt[e] > 0) ws.active[a++] = e;
      }
      o += cnt[e];
    }
  }
  if (t == 0) {
    off[E] = total[0];
    *nv_out = total[2];
    if (write_ws) {
      ws.offsets[E] = total[0];
      *ws.n_active = total[1];
      *ws.n_vslots = total[2];
      *ws.n_bad_ids = n_bad;  // the workspace error word: written by every routed call
    }
  }
  __syncthreads();
  for (int p = t; p < P; p += THREADS) {
    const int e = sid[p];
    if (e >= 0) {
      tmp[atomicAdd(&cur[e], 1)] = p;
    } else if (write_ws && zero_rows) {
      for (int64_t m = 0; m < zero_ld; ++m) zero_rows[(int64_t)p * zero_ld + m] = 0.0f;
    }
  }
  __syncthreads();
  // Ascending pair order inside each expert, so the result does not depend
  // on the order the atomics happened in (insertion sort: segments are
  // short). The owner of a run sorts it, then writes its pairs and slots.
  for (int e = e0; e < e1; ++e) {
    const int lo = off[e], hi = off[e + 1];
    for (int i = lo + 1; i < hi; ++i) {
      const int x = tmp[i];
      int j = i - 1;
      while (j >= lo && tmp[j] > x) {
        tmp[j + 1] = tmp[j];
        --j;
      }
      tmp[j + 1] = x;
    }
    if (write_ws)
      for (int i = lo; i < hi; ++i) ws.pairs[i] = tmp[i];
  }
  const bool also_ws = write_ws && vslots_out != ws.vslots;
  int vs = v[2];
  for (int e = e0; e < e1; ++e) {
    for (int k = 0; k < cnt[e]; k += kMoeNT) {
      int rec[kVSlotInts];
      const int nt = cnt[e] - k < kMoeNT ? cnt[e] - k : kMoeNT;
      rec[0] = e;
      rec[1] = nt;
#pragma unroll
      for (int n = 0; n < kVSlotInts - 2; ++n) rec[2 + n] = n < nt ? tmp[off[e] + k + n] : -1;
      const int4 r0 = make_int4(rec[0], rec[1], rec[2], rec[3]);
      const int4 r1 = make_int4(rec[4], rec[5], rec[6], rec[7]);
      int4* dst = reinterpret_cast<int4*>(vslots_out + (size_t)vs * kVSlotInts);
      dst[0] = r0;
      dst[1] = r1;
      if (also_ws) {
        int4* g = reinterpret_cast<int4*>(ws.vslots + (size_t)vs * kVSlotInts);
        g[0] = r0;
        g[1] = r1;
      }
      ++vs;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(const int32_t* ids, int E, int P,
                                                                 MoeWs ws, float* zero_rows,
                                                                 int64_t zero_ld) {
  extern __shared__ int32_t sm[];
  route_block<kRouteThreads>(ids, E, P, sm, ws, true, ws.vslots, ws.n_vslots, zero_rows, zero_ld);
}

// Routing computed inside a routed kernel (no separate launch): every
// workgroup builds the slot records in its own LDS, after the activations'
// image, and workgroup 0 also writes the workspace for the kernels that
// follow and for inspection.
struct InlineRoute {
  const int32_t* ids;  // null: the slot records are in the workspace already
  int E, P;
  float* zero_rows;
  int64_t zero_ld;
};

// LDS layout after the activations' image: the route scratch (rounded up to
// 16 bytes), the record count (one 16-byte piece), the 16-byte-aligned
// records.
__host__ __device__ constexpr int inline_route_scratch(int E, int P) {
  return (route_scratch_ints(E, P) + 3) / 4 * 4;
}
__host__ __device__ constexpr size_t inline_route_lds(int E, int P, int max_vslots) {
  return 4 * ((size_t)inline_route_scratch(E, P) + 4 + (size_t)max_vslots * kVSlotInts);
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

// ---------------------------------------------------------------- routed stream
// The row engine's inner loop, over the groups [g_begin, g_end) of the
// virtual-slot row space (group g covers rows (g % gpv) * G .. of slot
// g / gpv; rows at or past rpv are dead). Each group takes its expert, its
// token count and the LDS image of its tokens from the segment tables:
// slot v0 + j has expert seg_e[j], seg_nt[j] tokens, pair ids
// seg_pid[j * NT ..], and its tokens' activations at LDS block j * NT.
// Same per-lane chunk order, accumulation and team reduction as the dense
// engine, so each (row, token) result is the dense result.
template <int F, int NT, int LPR, int R, int D, int MINC, bool XF32, class RowOf, class Epi,
          class Stage>
__device__ __forceinline__ void run_routed(const RowOf& rowof, Epi& epi, const uint4* lds, int C,
                                           int g_begin, int g_end, int gpv, int rpv, int v0,
                                           const int32_t* seg_e, const int32_t* seg_nt,
                                           const int32_t* seg_pid, Stage&& stage) {
  constexpr int RPW = kWave / LPR;
  constexpr int G = RPW * R;
  constexpr int V = NT * R;
  constexpr int VP = Pow2<V>::value;
  using Shape = ReduceShape<LPR, VP, MINC>;
  constexpr int P = ChunkPlanes<F, XF32>::P;
  constexpr int S = kWavesPerBlock;  // waves of the workgroup take groups in turn

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int p = lane % LPR;
  const int team = lane / LPR;
  const int CPL = (C + LPR - 1) / LPR;

  const int g_first = g_begin + wave;
  const int my_groups = g_first < g_end ? (g_end - g_first + S - 1) / S : 0;
  const int total = my_groups * CPL;
  const int padded = (total + D - 1) / D * D;

  Slot<R> slot[D];
  // issue cursor: group ig = slot iv, group il inside the slot, chunk ij
  int ig = g_first, iv = g_first / gpv, il = g_first - (g_first / gpv) * gpv, ij = 0;
  const int8_t* iq[R];
  const uint16_t* id[R];
  bool iok[R];
  auto refresh = [&]() {
    const bool live = ig < g_end;
    const int e = live ? seg_e[iv - v0] : 0;
    const int rb = il * G + team * R;
#pragma unroll
    for (int r = 0; r < R; ++r) iok[r] = live && rb + r < rpv && rowof(e, rb + r, iq[r], id[r]);
  };
  refresh();
  auto issue = [&](Slot<R>& sl) {
    const int c = p + LPR * ij;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (iok[r] && c < C) {
        sl.q[r] = load_stream16(iq[r] + (int64_t)c * 16);
        sl.d[r] = id[r][c >> Fmt<F>::kScaleShift];
      } else {
        sl.q[r] = make_uint4(0, 0, 0, 0);
        sl.d[r] = 0;
      }
    }
    if (++ij == CPL) {
      ij = 0;
      ig += S;
      il += S;
      while (il >= gpv) {
        il -= gpv;
        ++iv;
      }
      refresh();
    }
  };

#pragma unroll
  for (int s = 0; s < D; ++s) issue(slot[s]);
  stage();

  float acc[VP];
#pragma unroll
  for (int i = 0; i < VP; ++i) acc[i] = 0.0f;
  // compute cursor and the group's token context
  int cg = g_first, cv = iv, cl = 0, cj = 0;
  cv = g_first / gpv;
  cl = g_first - cv * gpv;
  int nt = 0;
  const uint4* xb = lds;
  auto context = [&]() {
    if (cg < g_end) {
      const int j = cv - v0;
      nt = __builtin_amdgcn_readfirstlane(seg_nt[j]);
      xb = lds + (size_t)j * NT * P * C;
    }
  };
  context();

  for (int it = 0; it < padded; it += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int c = p + LPR * cj;
      if (c < C) chunk_fma<F, NT, R, XF32>(slot[s].q, slot[s].d, xb, C, c, nt, acc);
      issue(slot[s]);
      if (++cj == CPL) {
        if (cg < g_end) {
          int base = 0;
          TeamReduce<VP, MINC, LPR / 2, swap_reduce<F, LPR, XF32>()>::run(acc, p, base);
          const bool owner = (p & Shape::OWNER_MASK) == 0;
          epi.pid = seg_pid + (cv - v0) * NT;
          epi.nt = nt;
          epi.template emit<NT, R, Shape::CNT>(cl * G + team * R, base, owner, acc);
        }
#pragma unroll
        for (int i = 0; i < VP; ++i) acc[i] = 0.0f;
        cj = 0;
        cg += S;
        cl += S;
        while (cl >= gpv) {
          cl -= gpv;
          ++cv;
        }
        context();
      }
    }
  }
}

// Workgroup b streams groups [b*n/grid, (b+1)*n/grid) of the n = n_vslots *
// gpv groups, in segments of at most kSegV virtual slots: load the
// segments' slot records, issue the first weight loads, stage the
// activations of their tokens (x row p / topk, or p when x holds one row
// per pair), then stream.
template <int F, int NT, int LPR, int R, int MINC, bool XF32, class RowOf, class Epi>
__device__ __forceinline__ void routed_slices(const int32_t* vslots, int nv, const RowOf& rowof,
                                              Epi& epi, const char* x, int64_t ldx_bytes,
                                              bool x_per_pair, int topk, int C, int rpv,
                                              uint4* lds) {
  __shared__ int32_t seg_e[kSegV], seg_nt[kSegV], seg_pid[kSegV * NT];
  static_assert(NT == kMoeNT, "slot records hold kMoeNT pairs");
  constexpr int G = (kWave / LPR) * R;
  const int gpv = (rpv + G - 1) / G;
  nv = __builtin_amdgcn_readfirstlane(nv);
  const int n_groups = nv * gpv;
  const int g_lo = (int)((int64_t)blockIdx.x * n_groups / gridDim.x);
  const int g_hi = (int)((int64_t)(blockIdx.x + 1) * n_groups / gridDim.x);
  for (int g = g_lo; g < g_hi;) {
    const int v0 = g / gpv;
    const int v1 = v0 + kSegV < nv ? v0 + kSegV : nv;
    const int seg_end = g_hi < v1 * gpv ? g_hi : v1 * gpv;
    __syncthreads();  // the previous segment is done with the tables and the LDS image
    if (threadIdx.x < kSegV) {
      const int j = threadIdx.x;
      const int v = v0 + j;
      int4 a = make_int4(0, 0, -1, -1), b = make_int4(-1, -1, -1, -1);
      if (v < v1) {
        const int4* rec = reinterpret_cast<const int4*>(vslots + (size_t)v * kVSlotInts);
        a = rec[0];
        b = rec[1];
      }
      const int r[kVSlotInts] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      seg_e[j] = r[0];
      seg_nt[j] = r[1];
#pragma unroll
      for (int n = 0; n < NT; ++n) seg_pid[j * NT + n] = n < r[1] ? r[2 + n] : -1;
    }
    __syncthreads();
    auto stage = [&]() {
      const char* rows[kSegV * NT];
#pragma unroll
      for (int i = 0; i < kSegV * NT; ++i) {
        const int pid = __builtin_amdgcn_readfirstlane(seg_pid[i]);
        const int src = x_per_pair ? pid : pid / topk;
        rows[i] = pid < 0 ? nullptr : x + (int64_t)src * ldx_bytes;
      }
      stage_fmt<F, kSegV * NT, XF32, 1>(rows, C, lds);
      __syncthreads();
    };
    run_routed<F, NT, LPR, R, 1, MINC, XF32>(rowof, epi, lds, C, g, seg_end, gpv, rpv, v0, seg_e,
                                          seg_nt, seg_pid, stage);
    g = seg_end;
  }
}

// Occupancy request: 6 waves per SIMD (80 VGPRs) for Q8_0 with fp16
// activations, which the kernels meet without spilling (measured faster
// than the 5 waves the allocator picks unasked); 4 (128 VGPRs) for the
// heavier fp32 or Q4_0 variants. For the fp32-activation down projection
// of the E = 128 top-8 layer, 5 and 6 waves took the layer from 89.8 us
// to 95.5 and 124.4 us (same-process A/B on MI355X).
template <int F, bool XF32>
constexpr int moe_waves() {
  return (XF32 || F == kFmtQ4) ? 4 : 6;
}

// The slot records for a routed kernel: computed here (rt.ids set) into
// LDS after the activations' image of lds_x_bytes, or read from the
// workspace.
__device__ __forceinline__ const int32_t* routed_records(const MoeWs& ws, const InlineRoute& rt,
                                                         uint4* lds_x, size_t lds_x_bytes,
                                                         int& nv) {
  if (rt.ids == nullptr) {
    nv = *ws.n_vslots;
    return ws.vslots;
  }
  int32_t* sm = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(lds_x) + lds_x_bytes);
  int32_t* nv_lds = sm + inline_route_scratch(rt.E, rt.P);
  int32_t* vs_lds = nv_lds + 4;
  route_block<kBlock>(rt.ids, rt.E, rt.P, sm, ws, blockIdx.x == 0, vs_lds, nv_lds, rt.zero_rows,
                      rt.zero_ld);
  nv = *nv_lds;
  return vs_lds;
}

template <int F, int LPR, bool XF32>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(moe_waves<F, XF32>()))) void moe_rows_kernel(HBank W, MoeWs ws, int topk,
                                                         const char* x, int64_t ldx_bytes,
                                                         int x_per_pair, float* y,
                                                         InlineRoute rt, int64_t lds_x_bytes) {
  extern __shared__ uint4 lds_x[];
  int nv;
  const int32_t* vslots = routed_records(ws, rt, lds_x, (size_t)lds_x_bytes, nv);
  const int M = (int)W.e0.M;
  PairOutEpi epi;
  epi.y = y;
  epi.ld = M;
  epi.r_end = M;
  epi.pid = nullptr;
  epi.nt = 0;
  auto rowof = [W](int e, int i, const int8_t*& q, const uint16_t*& d) {
    q = W.e0.qs + (int64_t)e * W.stride_qs + (int64_t)i * W.e0.ld_qs;
    d = W.e0.d + (int64_t)e * W.stride_d + (int64_t)i * W.e0.ld_d;
    return true;
  };
  routed_slices<F, kMoeNT, LPR, Tune<kMoeNT, false>::R, 1, XF32>(
      vslots, nv, rowof, epi, x, ldx_bytes, x_per_pair != 0, topk, (int)chunks_per_row(F, W.e0.K),
      M, lds_x);
}

// virtual row i = 2*rho + s: s = 0 gate row rho, s = 1 up row rho
template <int FM, int LPR, bool XF32>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(moe_waves<FM, XF32>()))) void moe_gate_up_kernel(HBank Gb, HBank Ub, MoeWs ws,
                                                            int topk, const char* x,
                                                            int64_t ldx_bytes, float* h,
                                                            InlineRoute rt, int64_t lds_x_bytes) {
  extern __shared__ uint4 lds_x[];
  int nv;
  const int32_t* vslots = routed_records(ws, rt, lds_x, (size_t)lds_x_bytes, nv);
  const int F = (int)Gb.e0.M;
  SiluMulEpi epi;
  epi.h = h;
  epi.ld = F;
  epi.r_end = 2 * F;
  epi.pid = nullptr;
  epi.nt = 0;
  auto rowof = [Gb, Ub](int e, int i, const int8_t*& q, const uint16_t*& d) {
    const int64_t rho = i >> 1;
    const bool up = (i & 1) != 0;
    const int8_t* q0 = up ? Ub.e0.qs : Gb.e0.qs;
    const uint16_t* d0 = up ? Ub.e0.d : Gb.e0.d;
    const int64_t sq = up ? Ub.stride_qs : Gb.stride_qs;
    const int64_t sd = up ? Ub.stride_d : Gb.stride_d;
    const int64_t lq = up ? Ub.e0.ld_qs : Gb.e0.ld_qs;
    const int64_t ld = up ? Ub.e0.ld_d : Gb.e0.ld_d;
    q = q0 + (int64_t)e * sq + rho * lq;
    d = d0 + (int64_t)e * sd + rho * ld;
    return true;
  };
  routed_slices<FM, kMoeNT, LPR, 2, 2, XF32>(vslots, nv, rowof, epi, x, ldx_bytes, false, topk,
                                             (int)chunks_per_row(FM, Gb.e0.K), 2 * F, lds_x);
}

// The pairs of token t are taken eight at a time: their ids, gate weights
// and rows are all loaded before the first FMA (one memory round trip per
// eight pairs instead of one per pair), then folded in ascending j, a pair
// with an out-of-range expert leaving the sum as it is.
__global__ __launch_bounds__(256) void moe_combine_kernel(const int32_t* ids, int E,
                                                         const float* gate_w, const float* yp,
                                                         float* out, int topk, int64_t M) {
  constexpr int U = 8;
  const int t = blockIdx.y;
  const int64_t m0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (m0 >= M) return;
  const bool vec = (M & 3) == 0;
  const int nv = vec ? 4 : (int)(M - m0 < 4 ? M - m0 : 4);
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j0 = 0; j0 < topk; j0 += U) {
    bool ok[U];
    float w[U];
    float v[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u < topk ? j0 + u : topk - 1;  // in range; unused past topk
      const int e = ids[t * topk + j];
      ok[u] = j0 + u < topk && e >= 0 && e < E;
      w[u] = gate_w[t * topk + j];
      const float* row = yp + ((int64_t)t * topk + j) * M + m0;
      if (vec) {
        const float4 r = *reinterpret_cast<const float4*>(row);
        v[u][0] = r.x;
        v[u][1] = r.y;
        v[u][2] = r.z;
        v[u][3] = r.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[u][i] = i < nv ? row[i] : 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = ok[u] ? __builtin_fmaf(w[u], v[u][i], acc[i]) : acc[i];
  }
  for (int i = 0; i < nv; ++i) out[(int64_t)t * M + m0 + i] = acc[i];
}

// ---------------------------------------------------------------- host side
static int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

static size_t moe_lds_bytes(int64_t K, bool x_f32) {
  return (size_t)kSegV * kMoeNT * (size_t)(K / 16) * 16 * (x_f32 ? 4 : 2);
}

// The segment tables and the engine's other static LDS take well under 1 KiB.
bool moe_fits(const DevInfo& dev, int64_t K, bool x_f32) {
  return moe_lds_bytes(K, x_f32) + 1024 <= dev.lds_per_block;
}

int moe_max_vslots(int E, int P) { return (E < P ? E : P) + P / kMoeNT + 1; }

size_t moe_ws_layout(int E, int T, int topk, int64_t F, int64_t M, size_t off[kMoeWsAreas]) {
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
  off[4] = take(12);  // n_active, n_vslots, n_bad_ids (the error word)
  off[5] = take(F > 0 ? 4 * (size_t)P * (size_t)F : 0);
  off[6] = take(4 * (size_t)P * (size_t)M);
  off[7] = take(4 * (size_t)kVSlotInts * (size_t)moe_max_vslots(E, (int)P));
  return o;
}

hipError_t launch_moe_route(const int32_t* ids, int E, int P, const MoeWs& ws, float* zero_rows,
                            int64_t zero_ld, hipStream_t s) {
  const size_t lds = 4 * (size_t)route_scratch_ints(E, P);
  MoeWs w = ws;
  void* args[] = {(void*)&ids, &E, &P, &w, &zero_rows, &zero_ld};
  if (hipError_t e = allow_dynamic_lds((const void*)moe_route_kernel, lds)) return e;
  return hipLaunchKernel((const void*)moe_route_kernel, dim3(1), dim3(kRouteThreads), args, lds, s);
}

template <class Fn>
static hipError_t moe_launch(Fn fn, size_t lds, void** args, hipStream_t s, const DevInfo& dev) {
  if (hipError_t e = allow_dynamic_lds((const void*)fn, lds)) return e;
  const int64_t blocks = (int64_t)dev.cus * blocks_per_cu((const void*)fn, lds, kBlock);
  return hipLaunchKernel((const void*)fn, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(kBlock),
                         args, lds, s);
}

// A routed kernel computes the routing itself when its LDS has room for the
// route's scratch and records next to the activations' image; otherwise
// the route runs as its own launch first. Measured on MI355X (128 experts,
// top-8, 16 tokens): the separate route launch costs 5.2 us of a 92.5 us
// layer.
static bool route_inline(const DevInfo& dev, int64_t K, bool x_f32, const RouteReq& rq) {
  return rq.ids != nullptr && moe_lds_bytes(K, x_f32) + inline_route_lds(rq.E, rq.P,
                                                                         moe_max_vslots(rq.E, rq.P)) +
                                  1024 <= dev.lds_per_block;
}

static hipError_t route_first(const DevInfo& dev, int64_t K, bool x_f32, const RouteReq& rq,
                              const MoeWs& ws, InlineRoute& rt, size_t& lds, hipStream_t s) {
  rt = InlineRoute{nullptr, 0, 0, nullptr, 0};
  lds = moe_lds_bytes(K, x_f32);
  if (rq.ids == nullptr) return hipSuccess;
  if (route_inline(dev, K, x_f32, rq)) {
    rt = InlineRoute{rq.ids, rq.E, rq.P, rq.zero_rows, rq.zero_ld};
    lds += inline_route_lds(rq.E, rq.P, moe_max_vslots(rq.E, rq.P));
    return hipSuccess;
  }
  return launch_moe_route(rq.ids, rq.E, rq.P, ws, rq.zero_rows, rq.zero_ld, s);
}

template <int F, int LPR, bool XF32>
static hipError_t moe_rows_t(const DevInfo& dev, const HBank& W, const MoeWs& ws, int topk,
                             const char* x, int64_t ldx_bytes, int x_per_pair, float* y,
                             const RouteReq& rq, hipStream_t s) {
  InlineRoute rt;
  size_t lds;
  hipError_t e = route_first(dev, W.e0.K, XF32, rq, ws, rt, lds, s);
  if (e != hipSuccess) return e;
  HBank w = W;
  MoeWs wsv = ws;
  int64_t lds_x = (int64_t)moe_lds_bytes(W.e0.K, XF32);
  void* args[] = {&w, &wsv, &topk, (void*)&x, &ldx_bytes, &x_per_pair, &y, &rt, &lds_x};
  return moe_launch(moe_rows_kernel<F, LPR, XF32>, lds, args, s, dev);
}

hipError_t launch_moe_gemv(const DevInfo& dev, const HBank& W, const MoeWs& ws, int topk,
                           const void* x, bool x_f32, bool x_per_pair, float* y_pair,
                           const RouteReq& rq, hipStream_t s) {
  const int64_t ldx_bytes = W.e0.K * (x_f32 ? 4 : 2);
  const char* xp = (const char*)x;
  const int xpp = x_per_pair ? 1 : 0;
  return dispatch_chunks(W.e0.fmt, lanes_for(W.e0.fmt, W.e0.K), x_f32,
                         [&](auto f, auto l, auto xf) {
    return moe_rows_t<decltype(f)::value, decltype(l)::value, decltype(xf)::value>(
        dev, W, ws, topk, xp, ldx_bytes, xpp, y_pair, rq, s);
  });
}

template <int F, int LPR, bool XF32>
static hipError_t moe_gu_t(const DevInfo& dev, const HBank& G, const HBank& U, const MoeWs& ws,
                           int topk, const char* x, int64_t ldx_bytes, float* h,
                           const RouteReq& rq, hipStream_t s) {
  InlineRoute rt;
  size_t lds;
  hipError_t e = route_first(dev, G.e0.K, XF32, rq, ws, rt, lds, s);
  if (e != hipSuccess) return e;
  HBank g = G, u = U;
  MoeWs wsv = ws;
  int64_t lds_x = (int64_t)moe_lds_bytes(G.e0.K, XF32);
  void* args[] = {&g, &u, &wsv, &topk, (void*)&x, &ldx_bytes, &h, &rt, &lds_x};
  return moe_launch(moe_gate_up_kernel<F, LPR, XF32>, lds, args, s, dev);
}

hipError_t launch_moe_gate_up(const DevInfo& dev, const HBank& G, const HBank& U,
                              const MoeWs& ws, int topk, const void* x, bool x_f32, float* h,
                              const RouteReq& rq, hipStream_t s) {
  const int64_t ldx_bytes = G.e0.K * (x_f32 ? 4 : 2);
  const char* xp = (const char*)x;
  // Teams of at most 32 lanes: a wave then works on two gate/up row pairs
  // (2.5% faster than 64-lane teams at K = 2048 in same-process A/B).
  const int lpr0 = lanes_for(G.e0.fmt, G.e0.K);
  const int lpr = lpr0 < 32 ? lpr0 : 32;
  return dispatch_chunks(G.e0.fmt, lpr, x_f32, [&](auto f, auto l, auto xf) -> hipError_t {
    if constexpr (decltype(l)::value == 64) {
      return hipErrorInvalidValue;  // never chosen: teams are capped at 32 lanes
    } else {
      return moe_gu_t<decltype(f)::value, decltype(l)::value, decltype(xf)::value>(
          dev, G, U, ws, topk, xp, ldx_bytes, h, rq, s);
    }
  });
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
