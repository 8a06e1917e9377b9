/*
 * pisa.h -- C ABI of the PISA hot path on AMD Instinct MI355X (gfx950).
 *
 * PISA ("Block Sparse Attention with Log-Linear Complexity") selects, for every
 * query, K key blocks of C tokens by a coarse-to-fine top-K descent over a
 * mean-pooled key pyramid, scoring blocks by log-sum-exp, then runs softmax
 * attention over the raw keys and values of the selected blocks.  Citations
 * refer to the hyper.ai page of the paper (the only page with definitions),
 * by section:
 *   [BSA] block-sparse attention (o_t equation; flat selection cost)
 *   [PYR] pyramid key-block hierarchy (level sizes, Concat, mean pooling)
 *   [SEL] coarse-to-fine top-K selection (initial set, expansion, gK bound,
 *         keep-all rule, LSE block score)
 *   [KER] kernel implementation (GQA score sum, two-stage train/prefill
 *         kernels, query clusters and Q_tile, fused decode kernel)
 *
 * Conventions (all entry points):
 *   - Pointers are DEVICE memory unless stated.  The caller owns every buffer;
 *     the library never allocates device memory, never synchronises the
 *     stream, and launches only on `stream` (asynchronously).
 *   - Tensors are dense row-major.  q: [B][Hq][N][D]; k, v: [B][Hkv][cap][D]
 *     (cap = problem.cap, or N when cap is 0); o: [B][Hq][N][D].
 *   - Element types: PISA_F32 (float) or PISA_BF16 (bfloat16 bit patterns,
 *     uint16_t).  All accumulation is fp32; summaries are stored in fp32.
 *   - Query head h' belongs to KV head h' / G_Q with G_Q = Hq / Hkv.
 *   - Indices are 0-based.  Leaf j holds tokens [jC, min(jC + C, N)).
 *   - Causal problems: a block at any level is valid for query t iff its first
 *     token is <= t; keys i > t are masked in leaf scores and attention.
 *   - Ties in every top-K are broken toward the lower block index.
 *   - Arguments are validated on the host before any launch; an invalid one
 *     returns PISA_ERR_INVALID_ARG, an unsupported shape PISA_ERR_UNSUPPORTED,
 *     a too-small workspace PISA_ERR_WORKSPACE, a HIP launch failure
 *     PISA_ERR_HIP.  Outputs are undefined unless PISA_OK is returned.
 *     pisa_last_error() then describes the problem (thread-local string).
 *   - Supported in this version: g == 2 (the page's merge factor), D in
 *     {64, 128}, G_Q in {1, 2, 4, 8, 16}, 1 <= K <= 32, 1 <= C <= 128,
 *     N < 2^26, B * Hkv * N * K < 2^31, and the summary rows of one head
 *     times D below 2^31 (rows = sum over levels of ceil(cap / (C 2^(l-1))),
 *     about 2 cap / C: cap / C below about 8.4M at D = 128), so that every
 *     element offset inside a head's summaries fits 32 bits.
 */
#ifndef PISA_H_
#define PISA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PISA_OK = 0,
  PISA_ERR_INVALID_ARG = 1,
  PISA_ERR_UNSUPPORTED = 2,
  PISA_ERR_WORKSPACE = 3,
  PISA_ERR_HIP = 4
} pisa_status;

typedef enum { PISA_F32 = 0, PISA_BF16 = 1 } pisa_dtype;

/* Selection schedule; every schedule returns identical results. */
typedef enum {
  PISA_SELECT_AUTO = 0,      /* two-stage                                     */
  PISA_SELECT_TWO_STAGE = 1, /* [KER] stage 1 routing, query clusters, MFMA
                                leaf scoring, final top-K                    */
  PISA_SELECT_FUSED = 2      /* one program per (query, KV head) walks every
                                level and scores raw leaf keys itself ([KER]
                                decode design)                               */
} pisa_select_algo;

/* Attention schedule; both return the same result (up to fp32 rounding). */
typedef enum {
  PISA_ATTN_AUTO = 0,        /* leaf-major                                    */
  PISA_ATTN_LEAF_MAJOR = 1,  /* kept (query, leaf) pairs grouped by leaf; one
                                workgroup streams a leaf's queries through
                                MFMA and a merge pass combines the partials  */
  PISA_ATTN_QUERY_MAJOR = 2  /* one wave per (query, KV head); no workspace   */
} pisa_attn_algo;

typedef struct {
  int32_t B, N, Hq, Hkv, D; /* batch, tokens, query heads, KV heads, head dim */
  int32_t C;                /* leaf block size (the first merge factor, [PYR]) */
  int32_t g;                /* merge factor above the leaves; must be 2        */
  int32_t K;                /* blocks kept per level ([SEL])                   */
  int32_t causal;           /* 0 or 1                                          */
  int32_t dtype;            /* pisa_dtype of q, k, v, o                         */
  float scale;              /* logit scale; 0 => 1/sqrt(D)                      */
  int32_t q_tile;           /* stage-2 queries that share one read of a key
                               fragment: 16/G_Q (one 16-column MFMA tile) or
                               32/G_Q (two tiles; bf16 with C = 32, 64 or 128);
                               0 => 32/G_Q where allowed, else 16/G_Q.  Only
                               changes the schedule, never the result
                               ([KER] Q_tile).  Other values:
                               PISA_ERR_UNSUPPORTED.                            */
  int32_t cap;              /* token capacity of k/v rows and of the pyramid;
                               0 => N.  Must be >= N.                           */
  int32_t select_algo;      /* pisa_select_algo                                 */
  int32_t attn_algo;        /* pisa_attn_algo                                   */
} pisa_problem;

/* ---- key pyramid [PYR] ------------------------------------------------- *
 * Layout: float pyr[B][Hkv][R][D], then a block-floating-point copy read by
 * the bf16 routing kernel: fp16 f16[B][Hkv][R][D] = row * 2^-ex[row] and
 * int32 ex[B][Hkv][R] (the row's largest magnitude scaled into [2^14, 2^15));
 * pisa_pyramid_bytes covers all three.
 * R = sum over levels l = 1..L(cap) of
 * M_l(cap), M_1(n) = ceil(n / C), M_{l+1} = ceil(M_l / 2), L(n) the first
 * level with one block.  Level l of head (b, h) starts at row
 * sum_{l' < l} M_{l'}(cap).  Level 1 holds leaf means of raw keys; level l+1
 * holds the mean of each block's existing children (a ragged parent averages
 * its children's summaries, the mean-pooling equation taken literally).     */
size_t pisa_pyramid_bytes(const pisa_problem* p);
int32_t pisa_levels(int64_t n, int32_t C);                 /* L(n)            */
int64_t pisa_level_rows(int64_t n, int32_t C, int32_t l);  /* M_l(n) for 1 <= l <= 62
                                                              (1 above L(n)); 0 for
                                                              arguments out of range */
int64_t pisa_level_offset(int64_t cap, int32_t C, int32_t l); /* first row    */

/* Builds levels 1..L(N) of every (b, h) from k[b][h][0..N) (row stride cap).
 * [PYR] level-0 equation, level-size ceiling equation, mean-pooling equation.
 * Rows beyond M_l(N) are left untouched.                                      */
pisa_status pisa_build_pyramid(const pisa_problem* p, const void* k, float* pyr,
                               hipStream_t stream);

/* ---- selection [SEL], [KER] --------------------------------------------- *
 * For every (b, h, t): start from the coarsest level's single block; at each
 * level drop invalid blocks, keep all if <= K remain, else score each block
 * by sum over the G_Q query heads of h of the log-sum-exp over its valid
 * children of q . child_summary * scale (at level 1 the children are the raw
 * keys: the exact raw-key LSE), keep the top K and expand them into their
 * children.  Output: idx[B][Hkv][N][K] int32 leaf indices, ascending, -1
 * padded; score (may be NULL) the GQA-summed leaf LSE of each kept leaf
 * (-inf padded).  Reads pyr built by pisa_build_pyramid for the same k.
 * ws: device workspace of at least pisa_select_workspace_bytes(p) bytes
 * (256-byte aligned); its contents on entry do not matter.  After a
 * two-stage call (select_algo AUTO or TWO_STAGE) has completed, the first
 * B*Hkv*N*K int32 of ws hold the stage-1 result: per (b, h, t) the level-2
 * blocks kept by the descent ([B][Hkv][N][K], -1 padded), whose children are
 * the candidate leaves stage 2 scored.  Exposed so a caller can check the
 * final set against those candidates; a fused call leaves ws unspecified.  */
size_t pisa_select_workspace_bytes(const pisa_problem* p);
pisa_status pisa_select(const pisa_problem* p, const void* q, const void* k, const float* pyr,
                        int32_t* idx, float* score, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* ---- selection without a caller workspace --------------------------------- *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, kernels and results as pisa_select, with the workspace taken
 * from a scratch array of PISA_NOALLOC_SCRATCH_BYTES that the library holds
 * on each GPU it runs on (from the first call on that GPU until the process
 * ends).  The call allocates and frees nothing.  A problem whose
 * pisa_select_workspace_bytes exceeds PISA_NOALLOC_SCRATCH_BYTES returns
 * PISA_ERR_WORKSPACE before anything is launched (128 MiB holds, e.g.,
 * N = 32768 with 8 KV heads and K = 16).  The scratch needs no clearing:
 * like pisa_select's workspace, its contents on entry do not matter.  Every
 * call on one GPU uses that GPU's one array, so calls that overlap on a GPU
 * (other streams, other host threads) race; serialise them.  Other errors
 * as pisa_select.                                                          */
#define PISA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
pisa_status pisa_select_noalloc(const pisa_problem* p, const void* q, const void* k, const float* pyr,
                                int32_t* idx, float* score, hipStream_t stream);

/* ---- block-sparse attention [BSA] --------------------------------------- *
 * o[b][h'][t] = sum_i softmax_i(q . k_i * scale) v_i over the keys i of the
 * leaves idx[b][h'/G_Q][t][*] (entries < 0 or >= ceil(N/C) ignored; keys
 * i > t masked when causal).  o has the input dtype; lse (may be NULL) is float [B][Hq][N], the
 * log-sum-exp of the attended logits.  A query with no attended key gets
 * o = 0 and lse = -inf.  ws: at least pisa_attn_workspace_bytes(p) bytes,
 * 256-byte aligned (query-major: 256).  For the leaf-major schedule it holds
 * the partial outputs of a chunk of KV heads, B*Hkv*N*K*G*(D*elem + 8) bytes
 * capped near 24 GiB (about 18 GB for N = 131072, K = 16, 8 KV heads of
 * G = 4, D = 128, bf16), plus the clusters.                                 */
size_t pisa_attn_workspace_bytes(const pisa_problem* p);
pisa_status pisa_sparse_attn(const pisa_problem* p, const void* q, const void* k, const void* v,
                             const int32_t* idx, void* o, float* lse, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* ---- backward of the sparse attention [BSA] o_t equation ----------------- *
 * Gradients of L = sum_t dout_t . o_t for the attention of pisa_sparse_attn
 * over the FIXED selection idx (index-valued: no gradient flows through the
 * selection).  With p = softmax(z), z_i = q_t . k_i * scale over the keys of
 * the kept leaves (i <= t when causal) and D_t = dout_t . o_t:
 *   dq_t = scale sum_i p_i (dout_t . v_i - D_t) k_i,
 *   dk_i = scale sum_t p_i (dout_t . v_i - D_t) q_t,   dv_i = sum_t p_i dout_t.
 * q, dout, dq: [B][Hq][N][D]; k, v, dk, dv: [B][Hkv][cap][D] (rows >= N of dk,
 * dv are not written); idx: [B][Hkv][N][K] as from pisa_select; o and lse:
 * the outputs of pisa_sparse_attn for the same inputs (lse fp32 [B][Hq][N],
 * required).  Element types follow dtype; accumulation is fp32 (bf16 inputs:
 * p and dS are rounded to bf16 for the matrix products).  ws: at least
 * pisa_attn_backward_workspace_bytes(p) bytes, 256-byte aligned.  fp32
 * inputs with D = 128 need C <= 64 (a leaf's K, V and K^T tiles must fit
 * the LDS): otherwise PISA_ERR_UNSUPPORTED, and the workspace size is 0.   */
size_t pisa_attn_backward_workspace_bytes(const pisa_problem* p);
pisa_status pisa_sparse_attn_backward(const pisa_problem* p, const void* q, const void* k, const void* v,
                                      const int32_t* idx, const void* o, const float* lse, const void* dout,
                                      void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                                      hipStream_t stream);

/* ---- flat single-level selector (measurement baseline) [BSA] ------------ *
 * Scores every valid leaf j by sum over the G_Q query heads of
 * q_{h',t} . P_1[j] * scale and keeps the top K (same order and output
 * format as pisa_select).  Reads level 1 of pyr.                            */
size_t pisa_flat_workspace_bytes(const pisa_problem* p);
pisa_status pisa_flat_select(const pisa_problem* p, const void* q, const float* pyr, int32_t* idx,
                             float* score, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- decode [KER] decode paragraph --------------------------------------- *
 * One generated token per sequence.  For each sequence s with n = len[s]
 * cached tokens (n < cap): writes k_new/v_new at row n of the caches,
 * recomputes the mean of leaf n / C and of its ancestors (growing a level when
 * the leaf count crosses a power of two), then selects for the new query at
 * t = n (every block of the n + 1 tokens is valid) with one fused program per
 * (s, h), runs attention over the selected leaves into o[s][h'][D] and finally
 * sets len[s] = n + 1.  The pyramid must hold the pyramid of the first n
 * tokens (pisa_build_pyramid with N = n, cap = cap initialises it).
 * k_cache, v_cache: [S][Hkv][cap][D]; pyr: [S][Hkv][R(cap)][D] fp32;
 * len: [S] int32 (device); q_new: [S][Hq][D]; k_new, v_new: [S][Hkv][D];
 * o: [S][Hq][D]; idx: [S][Hkv][K] (may be NULL); score likewise.
 * err (may be NULL): device int32 set to 1 if some len[s] >= cap (that
 * sequence is then left untouched); never cleared by the library.          */
typedef struct {
  int32_t S, cap, Hq, Hkv, D;
  int32_t C, g, K;
  int32_t dtype;
  float scale; /* 0 => 1/sqrt(D) */
} pisa_decode_problem;

pisa_status pisa_decode_step(const pisa_decode_problem* p, void* k_cache, void* v_cache, float* pyr,
                             int32_t* len, const void* q_new, const void* k_new, const void* v_new,
                             void* o, int32_t* idx, float* score, int32_t* err, hipStream_t stream);

/* ---- diagnostics ----------------------------------------------------------- *
 * Per-kernel timer.  pisa_timer_enable(1) clears earlier records and makes
 * every kernel launch of the library record a HIP event pair on its launch
 * stream (a few microseconds of overhead per launch); pisa_timer_enable(0)
 * stops and clears.  pisa_timer_report waits for the recorded events, writes
 * one line "kernel<TAB>launches<TAB>total_ms" per kernel name into buf (host
 * memory, NUL-terminated, truncated to cap bytes), clears the records and
 * returns the number of kernel names.  Process-wide, not for use from several
 * host threads at once.                                                      */
void pisa_timer_enable(int32_t on);
int32_t pisa_timer_report(char* buf, size_t cap);

/* Work counters of the bf16 stage-1 routing kernel (the same kernel as
 * pisa_select's stage 1, with counting enabled): adds to the device uint64
 * counts[6] (caller-zeroed) the number of (query, KV head) routed, the
 * candidates scored at levels >= 2, the valid child summary rows read, the
 * levels scored, the kept level-2 blocks, and the valid child rows among
 * those read from device memory (the rest come from the coarse levels the
 * kernel stages in LDS).  ws: at least
 * pisa_select_workspace_bytes(p) bytes (its first part receives the kept
 * level-2 blocks).  For measurement only; not part of the hot path.          */
pisa_status pisa_route_counts(const pisa_problem* p, const void* q, const void* k, const float* pyr,
                              uint64_t* counts, void* ws, size_t ws_bytes, hipStream_t stream);

/* Measurement probe, not part of the method: gathers tiles of 16 fp16 rows
 * of D elements at pseudo-random rows of a table, loaded the way stage-1
 * routing loads the child summaries it does not hold in LDS (128-byte pieces
 * of a row per eight lanes, then through an LDS tile into the MFMA operand
 * layout), so that a benchmark can time the on-chip gather rate stage 1 is
 * bounded by.
 * table: device fp16 [heads][rows_per_head][D] (D 64 or 128); workgroups of
 * 16 waves, workgroup i reading head i % heads; every wave gathers
 * tiles_per_wave tiles (a multiple of 4), i.e. tiles_per_wave * 16 * D * 2
 * bytes; sink: device uint32 [workgroups * 16 * 64] receives checksums.
 * Returns PISA_ERR_INVALID_ARG for a bad argument (nothing launched).       */
pisa_status pisa_probe_gather(const void* table, int64_t rows_per_head, int32_t heads, int32_t D,
                              int32_t workgroups, int64_t tiles_per_wave, uint32_t* sink, hipStream_t stream);

/* Measurement probe, not part of the method: plain 16-byte streams over a
 * device buffer, so that a benchmark can time the HBM rate the memory-bound
 * kernels are compared with.  mode 0 reads `bytes` of src and writes one
 * checksum word per thread to sink (device uint32 [workgroups * 256]);
 * mode 1 copies `bytes` of src to dst (sink unused).  bytes is a positive
 * multiple of 16 and src / dst are 16-byte aligned device pointers; the
 * grid is `workgroups` workgroups of 256 threads striding over the buffer.
 * Returns PISA_ERR_INVALID_ARG for a bad argument (nothing launched).       */
pisa_status pisa_probe_stream(const void* src, void* dst, int64_t bytes, int32_t mode, int32_t workgroups,
                              uint32_t* sink, hipStream_t stream);

/* Thread-local description of the last non-OK status ("" if none). */
const char* pisa_last_error(void);
/* Library version string (static storage). */
const char* pisa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PISA_H_ */
