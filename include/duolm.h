/*
 * duolm.h -- C ABI of the MI355X (gfx950) DuoLM online ranker forward with
 * multi-item scoring (MIS).
 *
 * What the library computes.  A request carries a shared user-history prefix
 * of ids (instruction tokens, then per history item a marker token, one
 * virtual-token-ID (VID) item vector and its feedback tokens) and K candidate
 * VIDs.  The ranker (a Qwen3-0.6B-shaped decoder) prefills the prefix once;
 * every candidate occupies one position, sits at logical position L (the
 * prefix length) and attends to the prefix and to itself only, through a tree
 * mask; a shared linear head turns the candidate's final hidden state into a
 * score s = w^T h.  Nothing is decoded.  Sources:
 *   - "DuoLM: Fast and Effective Personalized Recommendation with Language
 *     Models" (paper.rainbus.top digest), sections 核心方法 (ranker input, shared
 *     head, tree mask and unified position ids, the exactness identity) and
 *     方法步骤详情 steps 3-5 (FP16 GPU-resident item table behind virtual ids
 *     V + iota(i); requests carry only ids; prefix KV prefilled once and shared;
 *     K scores returned in input order; graph replay of the segmented prefill);
 *   - "DuoLM은 아이템 벡터 재사용과 공유 프리픽스로 LLM 추천 서빙을 가속한다"
 *     (onedev.kr), sections 어떻게 동작하나 (input template, last hidden state,
 *     no attention between candidates) and 어떻게 쓰나 (VID table appended after
 *     the vocabulary V, packing after the shared prefix, tree mask plus
 *     position-id rule, one prefill of the prefix KV per request).
 *
 * Conventions for every entry point:
 *   - Return value: DUOLM_OK (0) or a negative duolm_status.  On error a
 *     message is available from duolm_last_error() (thread-local), and no
 *     output buffer has been written.
 *   - The caller owns every buffer it passes; the library never keeps a
 *     pointer to caller memory past the call.
 *   - A ranker handle is used by one thread at a time.  Calls on one handle
 *     are serialised on its stream.
 *   - Scoring calls are synchronous: when they return, the scores are in the
 *     output buffer.
 */
#ifndef DUOLM_H
#define DUOLM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct duolm_ranker duolm_ranker; /* opaque, owned by the library */

typedef enum {
  DUOLM_OK = 0,
  DUOLM_EINVAL = -1, /* bad argument: NULL pointer, K < 1, L < 1, length over a limit, bad option */
  DUOLM_ERANGE = -2, /* an id outside [0, V + N) */
  DUOLM_ENOMEM = -3, /* device or pinned-host allocation failed */
  DUOLM_EHIP = -4,   /* a HIP runtime call failed */
  DUOLM_EIO = -5,    /* weights file missing, short or malformed */
  DUOLM_ESTATE = -6  /* call not valid in the handle's current state */
} duolm_status;

/* Model dimensions, read back from a loaded ranker. */
typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab;
  float rms_eps, rope_base;
  int64_t n_vid;      /* rows of the VID table now loaded (0 if none) */
  int32_t max_prefix; /* largest accepted prefix length L */
  int32_t max_rows;   /* largest number of rows one forward launch handles */
} duolm_dims;

/*
 * Load ranker weights from a file written by this package's weights writer
 * (magic "DUOLMW01", a 64-byte header with the dimensions, then the tensors in
 * the canonical order, each 64-byte aligned; matrices bf16 [out, in], norm
 * gains and the head vector fp32).  Weights are copied to device `hip_device`
 * and re-laid-out for the kernels; the file is not kept open.
 *   path   : NUL-terminated file path (host).
 *   out    : receives the new handle; free it with duolm_free_ranker().
 * Errors: EINVAL (NULL, unsupported dimensions), EIO, ENOMEM, EHIP.
 */
int duolm_load_ranker(const char* path, int hip_device, duolm_ranker** out);

/* Same as duolm_load_ranker, from a host buffer holding the file's bytes. */
int duolm_load_ranker_mem(const void* blob, uint64_t nbytes, int hip_device, duolm_ranker** out);

/*
 * Load (or replace) the item table D: n_rows fp16 rows of d_model values,
 * row-major, host memory.  Row iota answers id V + iota (digest, 方法步骤详情
 * step 3).  The rows are copied into a GPU-resident table.
 * Errors: EINVAL (NULL, n_rows < 1, V + n_rows over INT32_MAX), ENOMEM, EHIP.
 */
int duolm_load_vid_table(duolm_ranker* r, const uint16_t* rows_fp16, int64_t n_rows);

int duolm_get_dims(const duolm_ranker* r, duolm_dims* out);

/*
 * One request: prefix ids, then its candidate ids (host pointers).
 *
 * inline_vecs (optional): instead of looking item vectors up in the table,
 * ship them in the request -- the alternative the pages compare VID ids
 * against ([digest] 实验结果: ids cut the request size by 99% and raise
 * throughput).  When non-NULL it holds one fp16 row of d_model values for
 * every position whose id is >= V, in prefix-then-candidates order, and
 * those ids only mark the positions (any value >= V); no table is needed.
 *
 * cand_len (optional, 0 means 1): ids per candidate.  An item spread over m
 * vectors (the pages' FIR m = 8 rating service, [digest] 实验结果; 未来方向
 * (2)) is a candidate branch of m rows at logical positions L .. L + m - 1,
 * causal inside the branch and blind to other candidates; it is scored at
 * its last row.  cand_ids then holds n_cand * cand_len ids, candidate-major.
 */
typedef struct {
  const int32_t* ids;          /* prefix_len ids, each in [0, V + N) (or >= V with inline_vecs) */
  int32_t prefix_len;          /* L >= 1 */
  const int32_t* cand_ids;     /* n_cand * max(cand_len, 1) ids in [0, V + N) (VIDs in practice) */
  int32_t n_cand;              /* K >= 1 candidates */
  const uint16_t* inline_vecs; /* NULL, or fp16 [number of ids >= V][d_model] */
  int32_t cand_len;            /* m: 0 or 1 (one row per candidate), up to DUOLM_MAX_CAND_LEN */
} duolm_request;

#define DUOLM_MAX_CAND_LEN 64

typedef enum {
  DUOLM_MODE_MIS = 0,        /* packed: prefix once, K one-row branches under the tree mask */
  DUOLM_MODE_INDEPENDENT = 1 /* each candidate appended alone to the prefix, full causal forward */
} duolm_mode;

typedef struct {
  int32_t mode;      /* duolm_mode */
  int32_t use_graph; /* nonzero: replay a captured HIP graph for the batch's shape bucket */
  void* hip_stream;  /* hipStream_t to order the work on, or NULL for the handle's own stream */
  int32_t max_lanes; /* 0 or 2: a call of >= 2048 rows over >= 2 sequences runs as two halves side
                        by side on two streams (the second is the handle's own); 1: one launch */
  int32_t reserved;  /* 0 */
} duolm_opts;

/*
 * Score a batch of requests (MIS by default).
 *   reqs, n_req : n_req >= 1 requests (host).
 *   scores      : host buffer of sum(n_cand) floats, written request-major,
 *                 candidates in input order (digest, 方法步骤详情 step 4).
 *   opts        : NULL means MIS with graph replay on the handle's stream.
 * Ids are validated on the host before any device work.  In independent
 * mode a candidate of m ids is appended alone to its prefix as m causal rows.
 * Errors: EINVAL (also cand_len outside [0, DUOLM_MAX_CAND_LEN]), ERANGE,
 * ESTATE (a VID id with no table loaded), ENOMEM, EHIP.
 */
int duolm_score_batch(duolm_ranker* r, const duolm_request* reqs, int32_t n_req, float* scores,
                      const duolm_opts* opts);

/*
 * Device-resident variant: the ids are already in device memory (item
 * vectors always come from the table here).
 *   prefix_len, n_cand : host arrays of n_req lengths.
 *   cand_len           : host array of n_req ids-per-candidate (as in
 *                        duolm_request), or NULL for one id per candidate.
 *   d_ids              : device, int32, the requests concatenated as
 *                        [prefix_0, cands_0, prefix_1, cands_1, ...].
 *   d_scores           : device, sum(n_cand) floats, request-major.
 * Ids are range-checked on the device: an out-of-range id makes the call
 * return ERANGE with d_scores untouched.
 */
int duolm_score_batch_dev(duolm_ranker* r, const int32_t* prefix_len, const int32_t* n_cand,
                          const int32_t* cand_len, int32_t n_req, const int32_t* d_ids, float* d_scores,
                          const duolm_opts* opts);

/*
 * duolm_score_batch_dev without any allocation, for callers that cannot
 * allocate memory (code running under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments and results as
 * duolm_score_batch_dev, but the call's activations, descriptor block and
 * scores live in a fixed scratch array of 112 MiB per GPU, built into the
 * library (each GPU the library runs on holds it until the process ends), and
 * the call makes no device or pinned allocation.  The forward runs as one
 * eager launch on the call's stream (opts->use_graph and opts->max_lanes are
 * ignored).
 *   Limit: the call's rows (sum of L + K*m in MIS mode, of K*(L + m) in
 *   independent mode) must fit the scratch: 24,580 bytes per row for the
 *   0.6B shape, about 4,700 rows, and one launch; larger calls return EINVAL
 *   and write nothing.
 *   Every call on one GPU shares that GPU's scratch, which keeps the last
 *   call's contents: calls that overlap on one GPU (from several threads, or
 *   several rankers on different streams) race and must be serialised by the
 *   caller.
 * Errors: as duolm_score_batch_dev, plus EINVAL for a call over the limit and
 * ESTATE if the scratch could not be located when the ranker was loaded.
 */
int duolm_score_batch_dev_noalloc(duolm_ranker* r, const int32_t* prefix_len, const int32_t* n_cand,
                                  const int32_t* cand_len, int32_t n_req, const int32_t* d_ids, float* d_scores,
                                  const duolm_opts* opts);

/*
 * Offline export of item vectors -- the step that fills the item table
 * before serving ([digest] 一句话总结 and 核心方法: the continuous-input
 * interface RMS-normalises the encoder's item representation a, calibrates it
 * by the reference scale rho of the ranker's native word embeddings and
 * multiplies a learnable gain e^gamma; 方法步骤详情 step 3: the frozen
 * vectors are written once as FP16 into the GPU-resident table; onedev.kr
 * digest, 어떻게 동작하나).  Per row
 *     z = e^gamma * rho * a / sqrt(mean_k a_k^2 + eps),
 * evaluated in float64 and rounded once to IEEE binary16 (nearest, ties to
 * even; magnitudes from 65520 up become +-inf).  A row whose mean square plus
 * eps is 0 exports as zeros.  eps = 0 is the bare RMS.
 */
typedef enum { DUOLM_DTYPE_F32 = 0, DUOLM_DTYPE_BF16 = 1, DUOLM_DTYPE_F16 = 2 } duolm_dtype;
#define DUOLM_MAX_EXPORT_DIM 8192

/*
 * Export on the current HIP device, stream-ordered (returns once the work is
 * enqueued on hip_stream; NULL is the null stream).
 *   d_a    : device, n_rows x d values of a_dtype, row-major, 16-byte aligned.
 *   d       : row length, a multiple of 8 in [8, DUOLM_MAX_EXPORT_DIM].
 *   rho, gamma, eps : finite; eps >= 0.
 *   d_z    : device, n_rows x d fp16 outputs, 16-byte aligned (caller-owned).
 * n_rows = 0 is a no-op.  Both buffers must be device memory of the current
 * device; a pointer that is not, or whose enclosing allocation is shorter than
 * the stated bytes, is rejected (an overrun inside a larger allocation, as
 * from a caching allocator's pool, cannot be seen and is the caller's).
 * Errors: EINVAL (bad dtype, d, n_rows, scale arguments, or a buffer that is
 * not such device memory), EHIP.
 */
int duolm_export_item_vectors(const void* d_a, int32_t a_dtype, int64_t n_rows, int32_t d, double rho,
                              double gamma, double eps, uint16_t* d_z, void* hip_stream);

/*
 * Export n_rows encoder outputs (device, [n_rows][d_model] of a_dtype) straight
 * into the ranker's item table, replacing any previous table: row iota answers
 * id V + iota, as with duolm_load_vid_table.  Synchronous.
 * Errors: as duolm_export_item_vectors, plus EINVAL for n_rows < 1 or
 * V + n_rows over INT32_MAX, ENOMEM.
 */
int duolm_export_vid_table(duolm_ranker* r, const void* d_a, int32_t a_dtype, int64_t n_rows, double rho,
                           double gamma, double eps);

/*
 * rho: the root mean square over every entry of the ranker's token embedding
 * matrix (its "native word embeddings"), accumulated in float64 in a fixed
 * order (the same value on every call).  Synchronous.
 * Errors: EINVAL (NULL), ENOMEM, EHIP.
 */
int duolm_reference_scale(duolm_ranker* r, double* rho);

/*
 * Host input packer.  A request carries only item ids and feedback; the
 * runtime assembles the ranker input from them ([digest] 方法步骤详情 step 4).
 * The input reads: the instruction, then for every history item a marker
 * token, the item's vector(s) and its feedback text, then the candidate
 * header, then the candidates' vectors ([onedev] 어떻게 동작하나; packing after
 * the shared prefix: 어떻게 쓰나).  The pages found this CPU-side input
 * compilation to be the bottleneck of their runtime near 200 requests/s
 * ([digest] 实验结果); here it is plain id copying in C++, optionally spread
 * over threads.  Feedback text arrives as token ids: nothing is tokenised.
 * Host only: no GPU work, and ids are not range-checked (scoring checks them).
 */
typedef struct {
  const int32_t* instruction; /* n_instruction ids opening every request */
  int32_t n_instruction;
  int32_t marker;             /* id opening every history item */
  const int32_t* cand_header; /* n_cand_header ids after the history, before the candidates */
  int32_t n_cand_header;
} duolm_template;

typedef struct {
  int32_t n_items;             /* history items, oldest first (>= 0) */
  int32_t item_len;            /* VIDs per history item: 0 or 1 means one, up to DUOLM_MAX_CAND_LEN */
  const int32_t* item_vids;    /* n_items * max(item_len, 1) VIDs, item-major */
  const int32_t* feedback;     /* the items' feedback ids, concatenated */
  const int32_t* feedback_off; /* n_items + 1 non-decreasing offsets into feedback, starting at 0 */
  const int32_t* cand_vids;    /* n_cand * max(cand_len, 1) VIDs, candidate-major */
  int32_t n_cand;              /* >= 1 */
  int32_t cand_len;            /* VIDs per candidate, as in duolm_request */
} duolm_history;

/* Number of ids duolm_pack_requests writes for these requests.
 * Errors: EINVAL (NULL, n_req < 1, a malformed request or template). */
int duolm_packed_size(const duolm_template* t, const duolm_history* reqs, int32_t n_req, int64_t* n_ids);

/*
 * Assemble n_req requests into ids (host, ids_cap int32) as
 * [prefix_0, cands_0, prefix_1, cands_1, ...], and write each request's
 * prefix length, candidate count and ids per candidate (host arrays of
 * n_req): the inputs of duolm_score_packed, or of duolm_score_batch_dev once
 * ids are on the device.  n_threads 0 or 1 packs on the calling thread; more
 * (up to 64, and at most one per 65,536 ids of work, since starting a thread
 * costs about as much as copying that many ids) splits the requests into
 * contiguous ranges of about equal id counts, packed in parallel; the output
 * is the same.
 * Errors: EINVAL (as duolm_packed_size, or ids_cap too small, or NULL outputs).
 */
int duolm_pack_requests(const duolm_template* t, const duolm_history* reqs, int32_t n_req, int32_t n_threads,
                        int32_t* ids, int64_t ids_cap, int32_t* prefix_len, int32_t* n_cand, int32_t* cand_len);

/*
 * Score a packed batch held in host memory (as duolm_pack_requests writes it):
 * ids are range-checked while being copied into the handle's page-locked
 * staging buffer and go up by DMA from there; scores come back the same way
 * into `scores` (host, sum(n_cand) floats).  cand_len may be NULL.
 * Synchronous.  Errors: as duolm_score_batch.
 */
int duolm_score_packed(duolm_ranker* r, const int32_t* prefix_len, const int32_t* n_cand, const int32_t* cand_len,
                       int32_t n_req, const int32_t* ids, float* scores, const duolm_opts* opts);

/*
 * Sessions: a user's prefix whose K and V stay on the GPU between calls, so
 * that a newly arrived history item appends its rows' K and V instead of the
 * whole prefix being prefilled again -- the pages' in-session incremental
 * personalisation ([digest] 未来方向 (3): only the new item's vectors and KV
 * are appended).  With causal attention the rows already computed do not
 * depend on later rows, so appending is exact: a session's scores are, bit
 * for bit, those of scoring its whole prefix in one call (same kernels, same
 * reduction order).  Sharing one item's KV across different users' prefixes
 * (未来方向 (5)) would change results and is not offered.
 *
 * K and V live in a pool of pages of 64 prefix rows x all layers
 * (2 * n_layers * 64 * n_kv_heads * head_dim bf16 values per page: 7.3 MB
 * for the 0.6B shape), reserved once per handle; sessions take pages as they
 * grow and return them when freed.
 */
typedef struct duolm_session duolm_session; /* opaque, owned by the library */

/* Reserve the pool for max_rows prefix rows in total over all sessions (in
 * pages of 64).  Replaces an earlier pool; fails with ESTATE while sessions
 * exist.  Errors: EINVAL, ENOMEM, ESTATE, EHIP. */
int duolm_kv_pool_init(duolm_ranker* r, int64_t max_rows);

/* Pages of the pool not held by any session. */
int duolm_kv_pool_free_pages(const duolm_ranker* r, int64_t* n_free);

/* A new empty session (prefix length 0).  Errors: EINVAL, ESTATE (no pool). */
int duolm_session_create(duolm_ranker* r, duolm_session** out);

/* Prefix rows the session holds. */
int duolm_session_length(const duolm_session* s, int32_t* prefix_len);

/* Returns the session's pages to the pool and frees it.  NULL is a no-op.
 * Sessions still alive when their ranker is freed are freed with it. */
void duolm_session_free(duolm_session* s);

/*
 * One call over n distinct sessions of this ranker.  Session i first appends
 * n_new[i] prefix ids (at positions L_i .. L_i + n_new[i] - 1, attending to
 * its cached rows and causally among themselves), then scores n_cand[i]
 * candidates (0: none) of cand_len[i] ids each against its whole prefix,
 * exactly as duolm_score_batch scores a request whose prefix is everything
 * the session has appended so far.
 *   ids    : host, per session [new ids, candidate ids], sessions in order.
 *   scores : host, sum(n_cand) floats, session-major, candidates in order
 *            (may be NULL when no candidates are scored).
 *   cand_len : host array or NULL, as in duolm_request.
 * On success each session's length grows by n_new[i]; on error no session
 * length changes.  MIS mode only.  Synchronous.
 * Errors: EINVAL (bad counts, a session twice or of another ranker, prefix
 * over the maximum, candidates with an empty prefix), ERANGE, ESTATE,
 * ENOMEM (the pool has too few free pages), EHIP.
 */
int duolm_session_step(duolm_ranker* r, duolm_session* const* sessions, int32_t n, const int32_t* n_new,
                       const int32_t* n_cand, const int32_t* cand_len, const int32_t* ids, float* scores,
                       const duolm_opts* opts);

/* Kernel classes for the profiling counters. */
typedef enum {
  DUOLM_K_EMBED = 0,      /* VID-aware embedding gather */
  DUOLM_K_RMSNORM = 1,    /* input / post-attention RMSNorm */
  DUOLM_K_GEMM_QKV = 2,   /* fused Q,K,V projection */
  DUOLM_K_QK_ROPE = 3,    /* per-head q/k RMSNorm + rotary embedding */
  DUOLM_K_ATTN_PREFIX = 4,/* causal attention over each prefix */
  DUOLM_K_ATTN_BRANCH = 5,/* candidate-branch attention over the shared prefix KV + self */
  DUOLM_K_GEMM_O = 6,     /* output projection + residual */
  DUOLM_K_GEMM_GATEUP = 7,/* gate/up projection + SwiGLU */
  DUOLM_K_GEMM_DOWN = 8,  /* down projection + residual */
  DUOLM_K_HEAD = 9,       /* final RMSNorm + score head */
  DUOLM_K_COUNT = 10
} duolm_kernel_class;

typedef struct {
  int64_t launches;   /* launches timed since the last reset */
  double total_ms;    /* device time they ran: per call, the union of their intervals between HIP
                         events (the sum of their durations unless launches overlap, as the two
                         concurrent halves of a large batch do) */
  double flops;       /* algorithmic FLOPs of those launches (useful work only) */
  double bytes;       /* algorithmic HBM bytes of those launches */
} duolm_kernel_stats;

/*
 * Time launches of the kernel classes in `class_mask` (bit i = class i) with
 * HIP events recorded on the launching stream, eager or inside captured
 * graphs (as event-record nodes).  0 turns timing off.  Resets the counters.
 * A call of at least 2048 rows over two or more sequences runs as two
 * halves on two streams, side by side; its timed launches of one class may
 * then overlap, and total_ms counts the time they ran once.
 */
int duolm_set_profiling(duolm_ranker* r, uint32_t class_mask);
int duolm_get_kernel_stats(duolm_ranker* r, int32_t kernel_class, duolm_kernel_stats* out);

/* Message for the last non-OK status on this thread ("" if none). */
const char* duolm_last_error(void);

/* Frees weights, table, workspace, graphs and the handle.  NULL is a no-op. */
void duolm_free_ranker(duolm_ranker* r);

#ifdef __cplusplus
}
#endif
#endif /* DUOLM_H */
