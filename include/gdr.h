/*
 * gdr.h -- C ABI of the MI355X (gfx950) chunked gated-delta-rule library.
 *
 * The library computes the chunked prefill of the gated delta rule, the
 * linear-attention recurrence of Gated DeltaNet (GDN):
 *
 *     S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * with an fp32 [K, V] state per value head, in the chunked (WY) form whose
 * forward and backward passes the FlashQLA pages fuse and accelerate
 * (FlashQLA curated summary, sections "核心亮點" and
 * "GDN Chunked Prefill的效率問題").  The argument lists follow that page's
 * low-level forward/backward listing (section "使用方式與需求"):
 *   forward:  q, k, v, g, beta, scale, initial_state, cu_seqlens
 *             -> g (processed), A, o, final_state
 *   backward: q, k, v, g, beta, A, do, dht, scale, initial_state, cu_seqlens
 *             -> dq, dk, dv, dbeta, dg, dh0
 * Variable-length packing and state continuation follow the Tongyi page
 * "FlashQLA - Tongyi Labsがオープンソース化した高性能線形アテンション演算子ライブラリ",
 * sections "FlashQLAの主な機能" and "FlashQLAの使い方".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers: every tensor pointer is a DEVICE pointer, except arguments whose
 *   name ends in _host (host memory).  Device pointers must be 16-byte
 *   aligned.  The library never allocates or frees device memory, never
 *   synchronises the device and never writes its inputs; it enqueues kernels
 *   on `stream` (a hipStream_t; NULL = the null stream) and returns.
 * Layouts (row-major, dense):
 *   q, k, dq, dk      [B, T, Hq, K]   dtype of the call
 *   v, o, do, dv      [B, T, Hv, V]   dtype of the call
 *   g, beta, dg, dbeta, g_cum        [B, T, Hv]  fp32
 *   A                 [B, T, Hv, 64]  fp32: row of the chunk's A for each token
 *   initial_state, final_state, dht, dh0   [N, Hv, K, V]  fp32
 *   cu_seqlens        [N + 1] int32 token offsets (packed mode, B must be 1)
 *   N = B without cu_seqlens, N = shape->num_seqs with it.
 * Heads: value head h reads query/key head h / (Hv / Hq) (contiguous groups).
 * Gate: g is the per-token log-gate (decay exp(g)); g <= 0 is expected.  A
 *   head with any g > 0 is still computed exactly, but never from a warmup
 *   (see the context-parallel options below).
 * Chunks: 64 tokens, restarting at every sequence start; the last chunk of a
 *   sequence may be short.
 * Supported: K, V in {32, 64, 128} with K == V; Hv a multiple of Hq;
 *   dtype bf16 (q, k, v, o, do, dq, dk, dv in bfloat16) or fp32; fp32 needs
 *   K <= 64 in the forward and K == 32 in the backward.
 * Errors: arguments are validated on the host before anything is enqueued; a
 *   negative status is returned and gdr_last_error() describes it.  Launch
 *   failures map to GDR_ERR_HIP.  Faults inside kernels surface at the
 *   caller's next synchronisation, as usual for HIP.
 * Threads: calls are thread-safe; gdr_last_error() is per thread.
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDR_OK = 0,
  GDR_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, bad shape, bad cu_seqlens_host */
  GDR_ERR_UNSUPPORTED = -2,   /* shape or dtype outside the supported set */
  GDR_ERR_WORKSPACE = -3,     /* workspace too small (see *_workspace_size) */
  GDR_ERR_HIP = -4            /* a HIP launch/runtime call failed */
} gdr_status;

typedef enum { GDR_BF16 = 0, GDR_F32 = 1 } gdr_dtype;

typedef struct {
  int32_t B, T;      /* batch, tokens per batch row (packed: B = 1, T = total) */
  int32_t Hq, Hv;    /* query/key heads, value heads (Hv % Hq == 0) */
  int32_t K, V;      /* key and value head dimensions */
  int32_t num_seqs;  /* N in packed mode (cu_seqlens given); ignored otherwise */
  gdr_dtype dtype;   /* element type of q, k, v, o, do, dq, dk, dv */
} gdr_shape;

/* Intra-card context parallelism (the pages' automatic single-card CP:
 * FlashQLA curated summary, section "平衡解決方案：雙核心融合與自動CP";
 * Tongyi page, section "FlashQLAの技術原則").  When (sequence, head) units are
 * too few to fill the GPU, each sequence is cut into segments of
 * `cp_segment_chunks` chunks; a segment's start state is rebuilt from zero over
 * the `cp_warmup_chunks` chunks before it, which is exact up to a factor
 * exp(sum of g over those chunks) as long as every token transition is a
 * contraction (g <= 0 and 0 <= beta |k|^2 <= 2).  A head is certified, and
 * uses the segments, when every token of the sequence meets those two
 * conditions and every warmup window has sum(g) <= cp_log_eps; each segment
 * of it then warms up over the fewest of those chunks
 * (counted back from its start) whose sum(g) already reaches cp_log_eps, which
 * keeps the same bound.  Any other head (for example one with g = 0) gets its segment
 * start states exactly instead: the map from a segment's start state to its
 * end state is affine, h_out = M h_in + b (the correction matrix the Tongyi
 * page describes for CP), so every segment's (M, b) is computed in parallel,
 * the start states follow from a short scan, and the segments then run from
 * them; with cp_serial_fallback = 1 such heads run serially instead.  Results
 * never depend on an uncertified warmup.  The bf16 backward uses the same
 * segments for both of its serial passes: the recomputed chunk states as
 * above, and the reverse pass over the state gradient, whose segments start
 * at their ends after up to cp_warmup_chunks chunks of warmup, again the
 * fewest that reach cp_log_eps (the reverse map is the transposed M plus an
 * offset); its certificate also covers the windows after every segment end.  The fp32 backward runs each head whole.
 * Pass NULL for the defaults; a zero-initialised struct also gives the
 * defaults. */
typedef enum { GDR_CP_AUTO = 0, GDR_CP_OFF = 1, GDR_CP_FORCE = 2 } gdr_cp_mode;

typedef struct {
  gdr_cp_mode cp_mode;       /* default GDR_CP_AUTO */
  int32_t cp_segment_chunks; /* GDR_CP_FORCE: chunks per segment (>= 1) */
  int32_t cp_warmup_chunks;  /* most warmup chunks before each segment; default 8 */
  float cp_log_eps;          /* certificate threshold on sum(g); default ln(1e-6) */
  int32_t cp_serial_fallback;/* 1: uncertified heads run serially; 0 (default): exact segment states */
  int32_t precise_vnew;      /* 1: the bf16 forward's output pass takes Vnew = A''(V - Gamma K h) as two
                              * bf16 terms (hi + lo) in its two products, P Vnew and the state update
                              * K^T (d * Vnew), instead of one bf16 rounding: for strongly coupled keys
                              * (nearly parallel keys without decay, where the chunk system I + L is
                              * badly conditioned), at the cost of one more MFMA per product; see the
                              * notes on precision.  0 (default): one bf16 operand.  Ignored in fp32
                              * and by the backward's recomputation. */
} gdr_options;

/* What the planner chose for a forward call (for tests and reporting). */
typedef struct {
  int32_t num_seqs;          /* N */
  int32_t total_chunks;      /* sum over sequences of ceil(len / 64) */
  int32_t max_chunks;        /* longest sequence, in chunks */
  int32_t v_blocks;          /* state column blocks per workgroup of the state pass */
  int32_t segment_chunks;    /* chunks per CP segment (>= max_chunks: no CP) */
  int32_t warmup_chunks;     /* most warmup chunks per segment (0 without CP) */
  int32_t total_segments;    /* sum over sequences of ceil(chunks / segment_chunks) */
  int32_t state_workgroups;  /* workgroups of the state pass */
} gdr_plan_info;

/* Bytes of device workspace gdr_chunk_fwd needs for this problem.
 * cu_seqlens_host is required in packed mode (num_seqs + 1 int32 values).
 * Returns 0 and sets gdr_last_error() on invalid arguments. */
size_t gdr_chunk_fwd_workspace_size(const gdr_shape* shape, const gdr_options* opts,
                                    const int32_t* cu_seqlens_host);

/* Forward chunked prefill.
 *   q, k, v, g, beta, scale   inputs as laid out above; scale > 0 finite.
 *   initial_state             nullable: zero initial state.
 *   cu_seqlens                nullable: B rows of T tokens; else packed mode,
 *                             with cu_seqlens_host its host copy (must match).
 *   o                         output [B, T, Hv, V] (call dtype).
 *   final_state               nullable: not written.
 *   g_cum_out                 nullable: chunk-local inclusive cumsum of g.
 *   A_out                     nullable: per-chunk A = (I + L)^-1 rows, where
 *                             L_ij = beta_i exp(gcum_i - gcum_j) k_i.k_j, i > j.
 *   workspace                 >= gdr_chunk_fwd_workspace_size() bytes, owned by
 *                             the caller, contents ignored and clobbered.
 */
gdr_status gdr_chunk_fwd(const gdr_shape* shape, const gdr_options* opts,
                         const void* q, const void* k, const void* v,
                         const float* g, const float* beta, float scale,
                         const float* initial_state,
                         const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                         void* o, float* final_state, float* g_cum_out, float* A_out,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the library-owned scratch that gdr_chunk_fwd_noalloc uses as its
 * workspace (128 MiB, held on every device that loads the library until the
 * process ends). */
#define GDR_NOALLOC_SCRATCH_BYTES (128u << 20)

/* gdr_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the workspace is the library's own
 * scratch on the current device, and the call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine).  Arguments, layouts and
 * results are those of gdr_chunk_fwd; `stream` must belong to the current
 * device.  Problems whose gdr_chunk_fwd_workspace_size() exceeds
 * GDR_NOALLOC_SCRATCH_BYTES are rejected with GDR_ERR_WORKSPACE (for example
 * the long-context shape B=1, T=65536, Hv=8, K=V=128 needs 114 MiB and fits).
 * Every call on one device shares that device's scratch: calls that overlap
 * in time on one device (concurrent streams or host threads) race and must
 * be serialised by the caller; calls in stream order are safe.  The first
 * call on a device looks up the scratch's device address there. */
gdr_status gdr_chunk_fwd_noalloc(const gdr_shape* shape, const gdr_options* opts,
                                 const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, float scale,
                                 const float* initial_state,
                                 const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                 void* o, float* final_state, float* g_cum_out, float* A_out,
                                 void* stream);

/* Planner decision for the forward (host only, nothing is enqueued). */
gdr_status gdr_chunk_fwd_plan(const gdr_shape* shape, const gdr_options* opts,
                              const int32_t* cu_seqlens_host, gdr_plan_info* out);

/* Bytes of device workspace gdr_chunk_bwd needs. */
size_t gdr_chunk_bwd_workspace_size(const gdr_shape* shape, const gdr_options* opts,
                                    const int32_t* cu_seqlens_host);

/* Backward of gdr_chunk_fwd for the loss <o, d_o> + <final_state, dht>.
 *   g                         the RAW log-gate (not g_cum).
 *   A                         nullable: the forward's A_out; recomputed if NULL.
 *   d_o                       [B, T, Hv, V] (call dtype).
 *   dht                       nullable: zero.
 *   initial_state             nullable: zero.
 *   dq, dk, dv                outputs (call dtype); dq, dk sum over each group.
 *   dbeta, dg                 outputs fp32 [B, T, Hv]; dg is w.r.t. raw g.
 *   dh0                       nullable output [N, Hv, K, V] (gradient at the
 *                             initial state, zero state if none was given).
 */
gdr_status gdr_chunk_bwd(const gdr_shape* shape, const gdr_options* opts,
                         const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const float* A,
                         const void* d_o, const float* dht, float scale,
                         const float* initial_state,
                         const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                         void* dq, void* dk, void* dv, float* dbeta, float* dg, float* dh0,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* gdr_last_error(void);

/* ---- kernel timing (diagnostics) ------------------------------------------
 * When enabled, every kernel the library enqueues is bracketed by a pair of
 * HIP events recorded on the launch stream.  gdr_timing_collect() waits for
 * the recorded events, folds their durations into per-kernel totals and
 * returns the number of distinct kernels seen; gdr_timing_entry() reads them.
 * Timing adds two event records per launch; it is off by default. */
void gdr_timing_enable(int enable);
int gdr_timing_collect(void);
int gdr_timing_entry(int i, const char** name, double* total_ms, int32_t* launches);
void gdr_timing_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
