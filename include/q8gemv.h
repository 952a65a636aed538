/*
 * q8gemv.h -- C ABI of the MI355X (gfx950) Q8_0 weight-only GEMV library.
 *
 * What the library computes. A Q8_0 weight matrix W [M][K] is stored as
 * blocks of 32 consecutive elements along K; each block holds one fp16
 * scale d and 32 int8 quants q, and the weight is d*q. This is the GGUF
 * Q8_0 format that the memra engine loads and runs through its decode
 * matvecs (memra wiki, feature list: the item on NVFP4, Q4_0 and Q8_0
 * decode, which names repacked split-plane matvecs chosen per shape; and
 * the loaders item).
 * For N tokens x [N][K]:
 *
 *     y[n][m] = sum_k d[m][k/32] * q[m][k] * x[n][k]
 *
 * N = 1 is plain decode; N = 2..8 is the batched K+1 verify of speculative
 * decoding (memra wiki, feature list: the item on MTP speculative decoding,
 * whose K drafted tokens plus one are verified in one batched pass).
 * Accuracy contract: every output is within
 * 1e-3 * sum_k |d*q*x| of the exact value (fp32 accumulation); the result
 * for token n is bitwise independent of N and of the other tokens' values
 * (the pages require verify logits to equal plain decode exactly: memra
 * wiki, gate paragraph, the self-consistency gate over K = 1..8; bw24
 * README, where no logit may differ).
 *
 * Conventions for every entry point:
 *  - Pointers marked [dev] are device memory (hipMalloc or a torch
 *    tensor's data pointer) owned by the caller; [host] are host memory.
 *    The library allocates nothing and keeps no per-call state; it caches
 *    only per-device properties, once, thread-safely.
 *  - Inputs are never written; outputs are fully overwritten.
 *  - `stream` is a hipStream_t (NULL = the null stream). Hot-path calls
 *    only enqueue kernels on it: no allocation, no synchronisation, no
 *    host<->device copy, so they can be captured in a HIP graph (the pages
 *    run one graph replay per decoded token: memra wiki, feature list,
 *    the graph-decode item).
 *  - Errors: arguments are validated before anything is enqueued; a
 *    negative q8_status is returned and nothing is launched. A launch
 *    failure reported by the HIP runtime returns Q8_ERR_LAUNCH. Faults
 *    inside a kernel surface at the caller's next synchronisation, like any
 *    HIP call. Unsupported inputs are refused, never silently routed to a
 *    slow path (topairepos memra listing, which prefers a clear failure to a
 *    quiet fallback).
 *  - Sizes: a pass's activations are held in the LDS of one workgroup
 *    (160 KiB on MI355X), so a K for which not even one token fits is
 *    refused with Q8_ERR_SHAPE. q8_gemv, the pairs, the router and the
 *    shared expert need K*2 bytes (fp16 x) or K*4 (fp32 x): K <= 81920 or
 *    40960 on MI355X (the shared expert's down projection reads fp32 h, so
 *    F <= 40960). The LM heads keep 1 KiB of their own: K <= 81408 or
 *    40704. The routed experts stage four tokens' rows next to 1 KiB of
 *    tables: K <= 20352 or 10176 (the FFN's down projection reads fp32 h,
 *    so F <= 10176). Routed calls take E <= 4096 and T*topk <= 8192 pairs,
 *    with (min(E, T*topk) + T*topk/2 + 1) * M < 2^31 (their row space is
 *    indexed in 32 bits). A matrix has at most 2^31 - 1 rows. Weights and
 *    outputs are addressed in 64 bits.
 *  - The library runs only on gfx950; on any other device every hot-path
 *    call returns Q8_ERR_DEVICE (memra wiki: the engine verifies at start-up
 *    that the binary matches the device and fails early otherwise).
 */
#ifndef Q8GEMV_H
#define Q8GEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    Q8_OK = 0,
    Q8_ERR_NULL = -1,      /* a required pointer is NULL */
    Q8_ERR_SHAPE = -2,     /* M, K, N, E, T or topk out of range, K % 32 != 0 */
    Q8_ERR_ALIGN = -3,     /* a pointer or leading dimension breaks 16-byte alignment */
    Q8_ERR_DTYPE = -4,     /* unsupported dtype code */
    Q8_ERR_WORKSPACE = -5, /* workspace NULL, misaligned or too small */
    Q8_ERR_DEVICE = -6,    /* current device is not gfx950, or no device */
    Q8_ERR_LAUNCH = -7,    /* the HIP runtime rejected a launch */
    Q8_ERR_ALIAS = -8      /* an output overlaps an input it must not */
} q8_status;

typedef enum { Q8_DT_F16 = 1, Q8_DT_F32 = 2 } q8_dtype;

/* Weight formats of a packed matrix (q8_matrix.format). */
typedef enum { Q8_FMT_Q8_0 = 0, Q8_FMT_Q4_0 = 1 } q8_format;

/* One packed matrix [M][K], rows = outputs, blocks of 32 weights along K,
 * in the split-plane layout written by the packers: a quant plane and a
 * scale plane, every row starting on a 16-byte boundary.
 *   format Q8_FMT_Q8_0 (q8_pack_host): qs [dev] int8 [M][ld_qs], row m
 *     holds q[m][0..K-1] in K order; ld_qs >= K.
 *   format Q8_FMT_Q4_0 (q8_pack_q4_0_host): qs [dev] bytes [M][ld_qs], row
 *     m holds the 16 data bytes of each GGUF Q4_0 block in K order;
 *     ld_qs >= K/2.
 *   d [dev] fp16 bit patterns [M][ld_d]: row m holds the K/32 scales.
 *   K % 32 == 0, M >= 1, ld_qs % 16 == 0, ld_d >= K/32 and ld_d % 8 == 0,
 *   qs and d 16-byte aligned. A zero-initialised struct is Q8_0.
 * Every entry point below accepts either format (matrices combined in one
 * call, e.g. a pair, must share it); another format value is Q8_ERR_DTYPE.
 * Any layout with these strides is accepted; e.g. one interleaved Q8_0
 * buffer per row ([K quants][K/32 scales]) is qs = base, d = base + K,
 * ld_qs = K + K/16 bytes, ld_d = ld_qs / 2, valid when K % 256 == 0. */
typedef struct q8_matrix {
    const int8_t *qs;
    const uint16_t *d;
    int64_t M, K;
    int64_t ld_qs; /* bytes */
    int64_t ld_d;  /* fp16 elements */
    int32_t format; /* q8_format */
} q8_matrix;

/* E experts of identical shape: expert e's matrix is e0 with
 * qs + e*stride_qs and d + e*stride_d. Strides keep 16-byte alignment
 * (stride_qs % 16 == 0, stride_d % 8 == 0). */
typedef struct q8_bank {
    q8_matrix e0;
    int64_t stride_qs; /* bytes */
    int64_t stride_d;  /* fp16 elements */
    int32_t E;
} q8_bank;

/* Human-readable name of a status code: a static string, never NULL
 * ("unknown status" for a value outside q8_status). Every failure of this
 * library is a named status the caller can report, never a silent
 * fallback (topairepos memra listing, which asks for useful failures over
 * silent fallbacks). No device is touched; callable on any host. */
const char *q8_status_str(int status);

/* Q8_OK iff HIP device `device` (an index as for hipSetDevice) exists and
 * is a gfx950 part; Q8_ERR_DEVICE otherwise. The answer is probed once per
 * device and cached (thread-safe). Call it at start-up to fail early, as
 * the pages' engine does when its binary does not match the GPU (memra
 * wiki: it checks the device at start-up and refuses to run on a
 * mismatch); every hot-path call makes the same check on the current
 * device. */
int q8_device_check(int device);

/* ------------------------------------------------------------ packing (host)
 * Load-time repack of GGUF Q8_0 blocks into the split-plane layout (memra
 * wiki, feature list: the split-plane repack; the onboarding CLI packs models
 * into the engine's own layout, topairepos memra listing, memra-cli row).
 *
 * q8_pack_layout: leading dimensions and plane sizes for an [M][K] matrix:
 *   ld_qs = K (bytes), ld_d = round_up(K/32, 8) (fp16 elements),
 *   qs_bytes = M*ld_qs, d_bytes = 2*M*ld_d. Any output pointer may be NULL.
 * q8_pack_host: blocks [host] = M rows of K/32 blocks of 34 bytes
 *   (little-endian fp16 scale, then 32 int8) -> qs [host] [M][ld_qs],
 *   d [host] [M][ld_d]. Padding is written as zero. Byte-exact: unpacking
 *   gives the input back.
 * q8_unpack_host: the inverse. */
int q8_pack_layout(int64_t M, int64_t K, int64_t *ld_qs, int64_t *ld_d,
                   size_t *qs_bytes, size_t *d_bytes);
int q8_pack_host(const void *blocks, int64_t M, int64_t K,
                 int8_t *qs, int64_t ld_qs, uint16_t *d, int64_t ld_d);
int q8_unpack_host(const int8_t *qs, int64_t ld_qs, const uint16_t *d, int64_t ld_d,
                   int64_t M, int64_t K, void *blocks);

/* ------------------------------------------------------------ dense GEMV
 * y[n][m] = sum_k d[m][k/32]*q[m][k]*x[n][k] for n < N, m < W->M.
 *   x [dev] [N][W->K], dtype x_dt (Q8_DT_F16 or Q8_DT_F32), contiguous,
 *     16-byte aligned.
 *   y [dev] [N][W->M], dtype y_dt (Q8_DT_F32, or Q8_DT_F16 rounded to
 *     nearest even), contiguous; must not overlap x.
 *   N >= 1. Tokens run in passes, every weight byte read once per pass:
 *   passes of up to 16 tokens for Q8_0 weights and fp16 x with rows of
 *   64 lanes (K a multiple of 1024, e.g. 5120) and at least 12 row groups
 *   of 4 rows per CU (rows >= 12288 on a 256-CU MI355X; the 9..16-token
 *   verify of the pages' K+1 speculative step, memra wiki feature list),
 *   passes of up to 8 tokens otherwise, all full passes of 4 or more
 *   tokens in one launch where the one-group kernel applies (the pass is
 *   the workgroup's y index; later passes find most weights in the L2);
 *   fewer if the x image of a pass would not fit the LDS. Per-token
 *   results are bitwise identical to N = 1 whatever the pass size. */
int q8_gemv(const q8_matrix *W, const void *x, int x_dt, void *y, int y_dt, int N,
            void *stream);

/* Fused pair: ya = Wa x and yb = Wb x in one launch sharing one staging of
 * x: the gate and up projections of a SiLU-gated MLP, which the pages'
 * decode runs as one fused matvec (memra performance, the qwen/silu MLP
 * class of the decode kernels). Wa->K == Wb->K; M may differ; both
 * matrices have one format.
 *   x [dev] [N][K] of x_dt, contiguous, 16-byte aligned;
 *   ya [dev] [N][Wa->M], yb [dev] [N][Wb->M], both of y_dt, must not
 *   overlap x or each other (Q8_ERR_ALIAS).
 * Results are bitwise equal to two q8_gemv calls (same per-row
 * arithmetic). No activation is applied (q8_gemv_pair_silu applies it).
 * N >= 1, passes as for q8_gemv (rows = Wa->M + Wb->M). */
int q8_gemv_pair(const q8_matrix *Wa, const q8_matrix *Wb, const void *x, int x_dt,
                 void *ya, void *yb, int y_dt, int N, void *stream);

/* Fused gate+up pair with the MLP activation (the SiLU-gated MLP of the
 * pages' qwen/silu model class, memra performance):
 *   h[n][m] = silu(g) * u,  g = (Wg x_n)[m], u = (Wu x_n)[m],
 *   silu(z) = z / (1 + exp(-z)) in fp32 (expf).
 * g and u are bitwise the ya and yb of q8_gemv_pair; only h is stored
 * (fp32, or fp16 rounded to nearest even), so the MLP's down projection
 * reads N*M values instead of 2*N*M. Wg and Wu have the same M and K.
 * x [dev] [N][K] of x_dt; h [dev] [N][M] of h_dt, must not overlap x.
 * N >= 1 (passes as for q8_gemv with rows = 2 * M; per-token results
 * N-invariant). */
int q8_gemv_pair_silu(const q8_matrix *Wg, const q8_matrix *Wu, const void *x, int x_dt,
                      void *h, int h_dt, int N, void *stream);

/* ------------------------------------------------------------ Q4_0
 * The same GEMV family over GGUF Q4_0 weights (memra wiki, feature list:
 * the item on NVFP4, Q4_0 and Q8_0 decode with split-plane matvecs). A Q4_0
 * block is 18 bytes: little-endian fp16 d, then 16 bytes whose low nibbles
 * are elements 0..15 and high nibbles elements 16..31, each stored as
 * q + 8 (q in [-8, 7]); the weight is d * q. The packed matrix is a
 * q8_matrix whose qs is the nibble plane: the 16 data bytes of each block,
 * in GGUF order, rows of ld_qs >= K/2 bytes (a multiple of 16), 16-byte
 * aligned; d is the scale plane as for Q8_0.
 *
 * q8_pack_q4_0_layout / q8_pack_q4_0_host / q8_unpack_q4_0_host: as the
 * Q8_0 packer (ld_qs = K/2, ld_d = K/32 rounded up to 8, padding zeroed,
 * byte-exact round trip), for blocks [host] of 18 bytes.
 * A Q4_0 matrix (format = Q8_FMT_Q4_0) runs through every entry point
 * (q8_gemv, pairs, LM heads, routed experts, router) with the same
 * arguments, pass structure, N-invariance and errors as Q8_0. */
int q8_pack_q4_0_layout(int64_t M, int64_t K, int64_t *ld_qs, int64_t *ld_d, size_t *qs_bytes,
                        size_t *d_bytes);
int q8_pack_q4_0_host(const void *blocks, int64_t M, int64_t K, uint8_t *qs, int64_t ld_qs,
                      uint16_t *d, int64_t ld_d);
int q8_unpack_q4_0_host(const uint8_t *qs, int64_t ld_qs, const uint16_t *d, int64_t ld_d,
                        int64_t M, int64_t K, void *blocks);

/* ------------------------------------------------------------ LM head
 * logits[n][v] = W x_n (as q8_gemv with fp32 output) and
 * ids[n] = the smallest v with logits[n][v] == max_v logits[n][v]
 * (ties go to the lowest index; -0 and +0 compare equal). The argmax is
 * taken over the same fp32 values that are written to logits, so ids is
 * always consistent with logits. logits may be NULL (only ids are written,
 * so the caller copies back 4 bytes per token, as the pages' graph decode
 * does: memra wiki, feature list, the graph-decode item).
 *   x [dev] fp16 or fp32 [N][K]; logits [dev] fp32 [N][V] or NULL;
 *   ids [dev] int32 [N]; N >= 1 (passes of up to 8 tokens).
 *   ws [dev] workspace of at least q8_lmhead_ws_bytes(V, N) bytes
 *   (4608 bytes plus 8 * V rounded up to 256; it grows with V, so size it
 *   for the largest vocabulary it will serve), 16-byte aligned, owned by
 *   the caller. It must be zero-filled once before its first use: it holds
 *   the argmax slots, the counters that let the last workgroup finish the
 *   argmax, and scratch logits for calls without logits; every completed
 *   call leaves it all zero again, so the same workspace can be reused
 *   (and captured in a graph) without clearing it. Keep it for LM-head
 *   calls only; concurrent calls must use distinct workspaces.
 * Launches: for a pass of 2 tokens, or of 1 token over a large enough
 * matrix (from about 150 MB of weights with logits, 280 MB without), the
 * GEMV writes the logits (the caller's, else the workspace's scratch) and
 * a second, short launch takes the argmax over them (and zeroes the
 * scratch); other passes run GEMV and argmax fused in one launch. Results
 * are the same either way. */
size_t q8_lmhead_ws_bytes(int64_t V, int N);
int q8_lmhead_argmax(const q8_matrix *W, const void *x, int x_dt, float *logits,
                     int32_t *ids, int N, void *ws, size_t ws_bytes, void *stream);

/* Draft LM head over a ranked subset of the vocabulary (the pages' MTP
 * drafting reads a vocab-masked head of a few tens of thousands of rows
 * instead of the whole vocabulary; memra wiki, feature list, MTP
 * speculative decoding). W holds the S subset rows, packed at load time
 * (gathered from the full head's blocks in subset order); row_ids [dev]
 * int32 [S] is the vocabulary id of each row. As q8_lmhead_argmax over W,
 * except ids[n] = row_ids[s*] where s* is the first maximum in subset
 * order (equal logits go to the earlier subset position); logits, if not
 * NULL, are [N][S] in subset order and bitwise equal to the full head's
 * logits at those rows. row_ids values are copied, never dereferenced.
 * Same workspace contract as q8_lmhead_argmax. */
int q8_lmhead_argmax_rows(const q8_matrix *W, const int32_t *row_ids, const void *x, int x_dt,
                          float *logits, int32_t *ids, int N, void *ws, size_t ws_bytes,
                          void *stream);

/* ------------------------------------------------------------ routed experts
 * Expert-major CSR batching of routed experts (memra wiki, feature list,
 * the MoE item, which batches routed tokens per expert in CSR form): the routed (token, slot) pairs are
 * grouped by expert on the device, and each active expert's weights are
 * streamed once for all tokens routed to it. Routing never leaves the
 * device (graph-replayable device-side lengths, memra wiki, feature list).
 * A token's outputs never depend on which other tokens share the batch
 * (memra performance, serving exactness arc).
 *
 * expert_ids [dev] int32 [T][topk]: expert of slot j of token t; the
 *   topk ids of one token must be distinct and in [0, E). Checking them on
 *   the host would need a synchronisation, so the check runs on the
 *   device: a pair whose id is out of range is left out (its per-pair
 *   output row is zero and it adds nothing to the combine), and the number
 *   of such pairs is written to the workspace error word (below). Every
 *   call writes the word (0 for valid ids), so it needs no clearing, also
 *   under graph replay; read it after the call to detect bad routing.
 * gate_w [dev] fp32 [T][topk]: combine weights (e.g. softmax router output).
 * Pair p = t*topk + j.
 *
 * Workspace layout (q8_moe_ws_layout gives byte offsets; all int32 unless
 * noted): [0] counts[E], [1] offsets[E+1], [2] pairs[T*topk] (pair ids in
 * expert-major order, ascending p inside an expert), [3] active[E]
 * (experts with count > 0, ascending), [4] n_active, then (int32 [1] of
 * area [4]) the routed-slot count, then (int32 [2] of area [4]) the error
 * word: the number of pairs whose expert id was out of range, [5] h fp32
 * [T*topk][F] (q8_moe_ffn only), [6] y_pair fp32 [T*topk][Mout].
 * The caller may read these after the call for inspection. */

/* Routed GEMV over one bank W (E experts of [M][K]):
 *   y_pair[p] = W[e_p] x_{src(p)}, src(p) = t if x_per_pair == 0 (x is
 *   [T][K]), else p (x is [T*topk][K]).
 *   gate_w == NULL: y [dev] fp32 [T*topk][M] receives y_pair.
 *   gate_w != NULL: y [dev] fp32 [T][M] receives
 *     sum_{j ascending} gate_w[t][j] * y_pair[t*topk + j].
 * x_dt is Q8_DT_F16 or Q8_DT_F32. ws >= q8_moe_ws_bytes(E, T, topk, 0, M). */
size_t q8_moe_ws_bytes(int E, int T, int topk, int64_t F, int64_t M);
int q8_moe_ws_layout(int E, int T, int topk, int64_t F, int64_t M, size_t offsets[7]);
int q8_moe_gemv(const q8_bank *W, const int32_t *expert_ids, const float *gate_w,
                const void *x, int x_dt, int x_per_pair, float *y, int T, int topk,
                void *ws, size_t ws_bytes, void *stream);

/* Routed SiLU-gated expert FFN (the qwen/silu MoE class of the pages,
 * memra performance, grouped expert lane):
 *   h_p   = silu(Wg[e_p] x_t) * (Wu[e_p] x_t)            fp32 [F]
 *   out_t = sum_{j ascending} gate_w[t][j] * Wd[e_p] h_p  fp32 [H]
 * with silu(z) = z / (1 + exp(-z)). gate, up: banks of [F][H]; down: bank
 * of [H][F]; the three banks have the same E. x [dev] fp16 [T][H];
 * out [dev] fp32 [T][H]. ws >= q8_moe_ws_bytes(E, T, topk, F, H). */
int q8_moe_ffn(const q8_bank *gate, const q8_bank *up, const q8_bank *down,
               const int32_t *expert_ids, const float *gate_w, const void *x, int x_dt,
               float *out, int T, int topk, void *ws, size_t ws_bytes, void *stream);

/* The same routed FFN for callers that cannot allocate or hand over a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the workspace is the library's own scratch array
 * of q8_noalloc_scratch_bytes() bytes (8 MiB) per GPU, a static device
 * array allocated with the library's code object on each GPU it runs on
 * and held until the process ends. The call allocates nothing and calls
 * no allocating routine. Arguments, results and errors are those of
 * q8_moe_ffn (bitwise the same outputs), except:
 *   - Q8_ERR_WORKSPACE when the workspace this shape needs,
 *     q8_moe_ws_bytes(E, T, topk, F, H), exceeds the scratch size
 *     (e.g. E = 128, F = 768, H = 2048, top-8: up to 88 tokens);
 *   - all calls on one GPU share that GPU's array, which keeps the last
 *     call's contents: calls that overlap on one GPU (concurrent streams,
 *     threads) race and must be serialised by the caller. Every call
 *     rewrites everything it reads, so nothing needs clearing. */
size_t q8_noalloc_scratch_bytes(void);
int q8_moe_ffn_noalloc(const q8_bank *gate, const q8_bank *up, const q8_bank *down,
                       const int32_t *expert_ids, const float *gate_w, const void *x, int x_dt,
                       float *out, int T, int topk, void *stream);

/* ------------------------------------------------------------ router
 * The step upstream of the routed experts, kept on the device so the
 * routed layer replays as a graph with no host round-trip (memra wiki,
 * feature list: graph-replayable device-length counters; one graph replay
 * per token), and computed one token at a time so a token's experts never
 * depend on its co-arrivals (memra performance, serving exactness arc:
 * m-invariant router kernels). The pages do not spell out the router's
 * arithmetic; the library's reading: per token t,
 *   expert_ids[t][0..topk) = the topk experts with the largest logits, in
 *     descending order of logit; equal logits go to the lower expert index
 *     first; -0 and +0 compare equal;
 *   gate_w[t][j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the picked
 *     logits l_0 >= l_1 >= ... (fp32 expf; equal to a softmax over all
 *     experts renormalised to the picked ones).
 * logits [dev] fp32 [T][E], finite (a NaN gives an unspecified pick, no
 * fault); expert_ids [dev] int32 [T][topk]; gate_w [dev] fp32 [T][topk];
 * 1 <= E <= 4096, 1 <= topk <= min(E, 64); T >= 1. No workspace. The
 * outputs feed q8_moe_gemv / q8_moe_ffn directly. */
int q8_moe_topk_softmax(const float *logits, int T, int E, int topk, int32_t *expert_ids,
                        float *gate_w, void *stream);

/* Router from a Q8_0 router matrix Wr [E][K]: logits = Wr x (as q8_gemv
 * with fp32 output, so bitwise independent of T), then
 * q8_moe_topk_softmax. x [dev] [T][K] of x_dt; logits [dev] fp32 [T][E]
 * (written, caller-owned). Launches: the GEMV's (all its passes in one
 * launch where the one-group kernel applies), then the top-k launch. */
int q8_moe_router(const q8_matrix *Wr, const void *x, int x_dt, int T, int topk, float *logits,
                  int32_t *expert_ids, float *gate_w, void *stream);

/* ------------------------------------------------------------ shared expert
 * The dense expert that a routed layer runs on every token beside the
 * routed ones, scaled per token by its own sigmoid gate and added to the
 * routed output (the pages' MoE decode computes that per-layer gate as one
 * fused dot: memra wiki, board notes on the 35B MoE decode; memra
 * performance, flip history). For every token t:
 *   out[t] += sigmoid(Wsg x_t) * Wd (silu(Wg x_t) * (Wu x_t))
 * Wg, Wu [F][H] and Wsg [1][H] (the gate row) share one format, Wd [H][F]
 * any: Q8_0 or Q4_0 (Q8_ERR_DTYPE if Wg, Wu and Wsg differ). x [dev]
 * [T][H] of x_dt; out [dev] fp32 [T][H], read and written (pass the routed
 * output of q8_moe_ffn, or zeros); T >= 1.
 * h = silu(g) * u is kept in fp32 and fed to Wd as fp32 activations; the
 * gate dot Wsg x_t is a GEMV row like any other (the same per-row
 * arithmetic), its sigmoid 1 / (1 + expf(-g)) in fp32, and each output is
 * out = fma(sigmoid, (Wd h)[m], out). Each output is within the bound the
 * oracle propagates from the GEMV bounds (sigma' <= 1/4).
 *   ws [dev] at least q8_moe_shared_ws_bytes(F, H, T) bytes, 16-byte
 *   aligned, caller-owned scratch (h and the gate dots; no zero-fill
 *   needed). Two launches for all full passes of up to 8 tokens (one more
 *   of each for a ragged last pass): the SiLU pair with the gate row as
 *   one more row (the fused gate dot), then the down GEMV whose epilogue
 *   applies the gate and adds into out. */
size_t q8_moe_shared_ws_bytes(int64_t F, int64_t H, int T);
int q8_moe_shared_expert(const q8_matrix *Wg, const q8_matrix *Wu, const q8_matrix *Wd,
                         const q8_matrix *Wsg, const void *x, int x_dt, int T, float *out,
                         void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* Q8GEMV_H */
