/*
 * wave_index.h -- C ABI of the MI355X (gfx950) wave-index library (libwave_index.so).
 *
 * The wave index is the attention-aware vector index of RetroInfer ("RetroInfer: A Vector Storage
 * Engine for Scalable Long-Context LLM Inference"; technical summaries on gist.science, Spanish
 * page section 2.A and Arabic page section 2.a).  Each decode query's attention is split into
 *   - a steady zone: the first `sink` and the last `window` positions, attended exactly;
 *   - a retrieval zone: the tokens of the top_k clusters of a spherical-k-means index whose
 *     centroids score highest against the query, attended exactly;
 *   - an estimation zone: every other non-empty cluster c, approximated from its mean key mu_c,
 *     its size n_c and its value sum SV_c: numerator += n_c * exp(s_c) * SV_c / n_c,
 *     denominator += n_c * exp(s_c), with s_c = <q, mu_c> * scale;
 * and the three partial softmax states are merged with log-sum-exp.  The index is built at
 * prefill by spherical k-means run separately on consecutive segments of the sequence (Spanish
 * page section 3, "Clustering Segmentado"; Arabic page section 2.a, last paragraph).
 *
 * Conventions shared by every entry point
 *   - Pointers are device pointers unless marked (host).  All device buffers are caller-allocated
 *     and caller-owned; the library never allocates or frees device memory.  Only a wave buffer
 *     (below) keeps state between calls: its cache lives in device memory the caller provides,
 *     and its host state in memory wi_wavebuf_create allocates.
 *   - Layout is row-major and contiguous, heads-major: [B, H, tokens, d].  Query head h reads KV
 *     head h / (Hq / Hkv).
 *   - `stream` is a hipStream_t (0 = the null stream).  Calls enqueue work and return; they never
 *     synchronise, except that a wave-buffer call waits for the access log of the call two
 *     before it and wi_wavebuf_stats for every pending log.  Asynchronous faults surface at the
 *     caller's next synchronisation.
 *   - d must be 128.  Element types are fp32 (WI_F32) or bfloat16 (WI_BF16); arithmetic is fp32
 *     (fast paths) and fp64 (every decision that must be reproducible: k-means assignments and
 *     sums, top-k ties).
 *   - Invalid arguments are rejected on the host before anything is enqueued: the call returns a
 *     negative wi_status, sets the thread-local wi_last_error() string and has no side effect.
 *   - NaN or Inf inputs are not checked; they propagate to the outputs.
 */
#ifndef WAVE_INDEX_H_
#define WAVE_INDEX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WI_OK = 0,
  WI_ERR_INVALID_ARG = -1, /* bad shape, null required pointer, inconsistent parameters      */
  WI_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels implement (d != 128, ...)     */
  WI_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the *_workspace_bytes figure   */
  WI_ERR_HIP = -4          /* a HIP launch or query failed; see wi_last_error()               */
} wi_status;

typedef enum { WI_F32 = 0, WI_BF16 = 1 } wi_dtype;

/* Parameters of an index build.  The clustered range of each (b, g) is positions
 * [sink, N - window) (empty when sink + window >= N); it is cut into consecutive segments of
 * seg_len tokens (the last may be shorter; seg_len = 0 means one segment), and segment s owns
 * cluster ids [s * clusters_per_seg, (s + 1) * clusters_per_seg).  Segments hold at most 65536
 * tokens.  iters >= 1 Lloyd iterations (assign, then update) run on every segment. */
typedef struct {
  int32_t B, Hkv, N, d;
  int32_t sink, window;
  int32_t seg_len;
  int32_t clusters_per_seg;
  int32_t iters;
  int32_t dtype;   /* wi_dtype of K, V and of the stored index */
  uint64_t seed;   /* seeds the per-segment initialisation     */
} wi_build_params;

/* The index: every pointer is caller-allocated device memory, sized by wi_index_shapes_for().
 *   centroids   [B,Hkv,C,d]   dtype  mean key of each cluster (0 for an empty cluster)
 *   value_sums  [B,Hkv,C,d]   dtype  sum of member values (0 for an empty cluster)
 *   sizes       [B,Hkv,C]     int32  member count n_c
 *   offsets     [B,Hkv,C+1]   int32  exclusive prefix sum of sizes: cluster c owns rows
 *                                    [offsets[c], offsets[c+1]) of k_perm / v_perm
 *   perm        [B,Hkv,Nc]    int32  absolute token position of each k_perm row
 *   k_perm      [B,Hkv,Nc,d]  dtype  clustered keys, cluster after cluster, ascending position
 *   v_perm      [B,Hkv,Nc,d]  dtype  the matching values
 *   k_steady    [B,Hkv,NS,d]  dtype  keys of the steady zone, ascending position
 *   v_steady    [B,Hkv,NS,d]  dtype  the matching values
 * where C = nseg * clusters_per_seg, Nc = clustered tokens, NS = min(N, sink + window).
 * wi_decode only reads an index, so several streams may decode the same index concurrently. */
typedef struct {
  void *centroids, *value_sums;
  int32_t *sizes, *offsets, *perm;
  void *k_perm, *v_perm;
  void *k_steady, *v_steady;
} wi_index_view;

/* Sizes (in elements, except build_workspace_bytes) of every index buffer. */
typedef struct {
  int64_t C, Nc, n_steady, nseg;
  int64_t centroids, value_sums, sizes, offsets, perm, k_perm, v_perm, k_steady, v_steady;
  int64_t build_workspace_bytes;
} wi_index_shapes;

/* Parameters of one batched GQA decode step over an index built with matching B, Hkv, d and
 * dtype.  n_steady, C and Nc are the figures wi_index_shapes_for() returned.  top_k >= 0 clusters
 * are retrieved per query head (clamped to the head's number of non-empty clusters).  scale
 * multiplies every logit (1/sqrt(d) for standard attention). */
typedef struct {
  int32_t B, Hq, Hkv, d;
  int32_t n_steady, C, Nc;
  int32_t top_k;
  float scale;
  int32_t dtype;
} wi_decode_params;

/* (host) Fill *out with the buffer sizes of an index for *p.  Host only; enqueues nothing.
 * Errors: WI_ERR_INVALID_ARG for null pointers or out-of-range fields, WI_ERR_UNSUPPORTED for
 * d != 128, a segment longer than 65536 tokens, more than 4096 clusters per segment or more
 * than 2^31 rows in one index buffer. */
wi_status wi_index_shapes_for(const wi_build_params *p, wi_index_shapes *out);

/* Build the wave index of K, V ([B,Hkv,N,d], dtype) into *out (segmented spherical k-means;
 * RetroInfer Spanish summary section 3 and Arabic summary section 2.a).
 * Per segment: initial centroid directions are unit-normalised key rows chosen by a partial
 * Fisher-Yates shuffle driven by SplitMix64 (Steele, Lea, Flood, OOPSLA 2014) seeded from
 * (seed, b, g, s); then `iters` times: assign every key to the centroid direction of highest
 * inner product (ties to the lower id; decided in fp64), and replace every non-empty cluster's
 * direction by its normalised fp64 member sum (kept when the cluster is empty).  The last
 * assignment defines sizes, offsets, perm, the copies, centroids (mean key) and value sums.
 * The result is a deterministic function of (K, V, parameters).  `workspace` must hold
 * build_workspace_bytes (256-byte aligned).  K and V may be freed once the build completes. */
wi_status wi_build_index(const wi_build_params *p, const void *k, const void *v,
                         const wi_index_view *out, void *workspace, size_t ws_bytes,
                         void *stream);

/* Grow an index by one segment: the L = seg_len tokens that have left the local window since
 * `prev` was built are clustered as a new segment (segmented clustering: RetroInfer Spanish
 * summary section 3 "Clustering Segmentado", Arabic summary section 2.a last paragraph; the
 * segments are clustered independently, each from its own seed).
 *   p     the parameters of the grown context (N tokens); seg_len >= 1 and the clustered range
 *         N - sink - window must be a positive multiple of seg_len.  `prev` is the index of the
 *         first N - seg_len tokens with the same sink, window, seg_len, clusters_per_seg, iters,
 *         seed and dtype (so it holds only full segments).
 *   k, v  [B,Hkv,N,d] the grown context (the new segment's rows and the steady zone are read).
 *   out   the index of the grown context, with the shapes of wi_index_shapes_for(p); it must not
 *         overlap `prev`.  Its first segments are copied from `prev`, the last one is clustered,
 *         and the steady-zone copies are taken from k, v.
 * The result equals wi_build_index(p, k, v) bit for bit.  Workspace: build_workspace_bytes of p.
 * Errors: as wi_build_index, and WI_ERR_INVALID_ARG for a clustered range that is not a positive
 * multiple of seg_len, seg_len 0, null pointers in either view, or overlapping buffers. */
wi_status wi_index_append_segment(const wi_build_params *p, const void *k, const void *v,
                                  const wi_index_view *prev, const wi_index_view *out,
                                  void *workspace, size_t ws_bytes, void *stream);

/* (host) Workspace bytes wi_decode needs for *p.  Host only. */
wi_status wi_decode_workspace_bytes(const wi_decode_params *p, size_t *bytes);

/* One decode step for every (b, query head) (RetroInfer Spanish summary section 2.A items 1-3,
 * Arabic summary section 2.a):
 *   q        [B,Hq,d]      dtype  the queries
 *   out      [B,Hq,d]      fp32   attention output
 *   lse      [B,Hq]        fp32   log-sum-exp of the merged softmax state (nullable)
 *   sel_ids  [B,Hq,top_k]  int32  retrieved cluster ids in ascending order, -1 padded (nullable)
 * The retrieval zone of a head is the min(top_k, #non-empty) non-empty clusters that come first
 * in the order (-sigma_c, c), sigma_c = <q, mu_c> with exact products summed in fp64 in ascending
 * coordinate order: higher score first, lower id on equal scores.  `workspace` must hold
 * wi_decode_workspace_bytes (256-byte aligned); calls that share a workspace must not overlap.
 * Errors: WI_ERR_INVALID_ARG for inconsistent parameters or null required pointers,
 * WI_ERR_WORKSPACE for a short or misaligned workspace, WI_ERR_UNSUPPORTED for d != 128, a
 * group size other than 1, 2, 4 or 8, more than 262144 clusters or 2^23 tokens per KV head, or
 * B * Hkv above 65535. */
wi_status wi_decode(const wi_decode_params *p, const wi_index_view *idx, const void *q,
                    float *out, float *lse, int32_t *sel_ids, void *workspace, size_t ws_bytes,
                    void *stream);

/* wi_decode for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the workspace is a static array of the
 * library's own, 64 MiB on every device the library runs on (held until the process ends), so
 * the call takes no workspace argument and allocates nothing.  Every other argument, the result
 * and the errors are those of wi_decode; also WI_ERR_UNSUPPORTED when wi_decode_workspace_bytes
 * exceeds 64 MiB (e.g. batch 16 at 128K tokens).  All calls on one device share its array:
 * calls that overlap on one device (on different streams, or from different threads without
 * ordering) race and give wrong results. */
wi_status wi_decode_noalloc(const wi_decode_params *p, const wi_index_view *idx, const void *q,
                            float *out, float *lse, int32_t *sel_ids, void *stream);

/* One decode step that attends over the previous step's zones where the queries barely moved
 * (FreeKV Spanish summary, section A items 1-2: speculative retrieval, and a fine-grained
 * correction that selects again for the KV heads whose consecutive queries have a cosine below a
 * threshold tau).  For every (b, KV head): if every one of its query heads has
 * cos(q, q_prev) >= tau, where cos = <q, q'> / (|q| |q'|) from exact products summed in fp64 in
 * ascending coordinate order, with IEEE fp64 square roots and division, and 0 when either query
 * is zero, each of those heads takes its retrieval zone from sel_prev; otherwise the heads select
 * as wi_decode does.  The scores of the current query are computed for every head either way: the
 * estimation zone (every non-empty cluster outside the zone) uses them.
 *   q_prev    [B,Hq,d]     dtype  the previous step's queries
 *   sel_prev  [B,Hq,top_k] int32  the zones to keep; entries outside [0, C) are skipped and
 *                                 repeats count once
 *   tau                           the threshold (> 1 never reuses, <= 0 reuses any pair)
 *   sel_ids   [B,Hq,top_k] int32  the zone each head attended over, ascending, -1 padded
 *                                 (required when top_k > 0)
 *   reused    [B,Hkv]      int32  1 where the KV head kept sel_prev (nullable)
 * The call also keeps the reuse flags in the workspace for wi_select_refresh.  Feeding sel_ids
 * to the next step keeps a zone for as long as the queries stay within tau of their predecessor;
 * calling wi_select_refresh first gives FreeKV's scheme, in which a kept zone is one step old.
 * Everything else, and the errors, as wi_decode; also WI_ERR_INVALID_ARG for a null q_prev or
 * sel_prev, a NaN tau, a null sel_ids with top_k > 0, or sel_prev overlapping sel_ids. */
wi_status wi_decode_gated(const wi_decode_params *p, const wi_index_view *idx, const void *q,
                          const void *q_prev, const int32_t *sel_prev, float tau, float *out,
                          float *lse, int32_t *sel_ids, int32_t *reused, void *workspace,
                          size_t ws_bytes, void *stream);

/* The selection that wi_decode_gated postponed (FreeKV Spanish summary, section A items 1-2: for
 * the heads that were not corrected, retrieval is deferred and overlapped with other work for the
 * next step).  For every (b, KV head) that the last wi_decode_gated call on this workspace
 * marked reused, overwrites its heads' sel_ids rows with the top-k of the current queries, as
 * wi_decode selects them; other rows are left as they are.  p, idx, q, sel_ids and the workspace
 * must be those of that call, and the workspace must not have been used since; the call may be
 * enqueued later or on another stream, ordered after that call.  After a wi_decode call on the
 * workspace it does nothing.  Errors: as wi_decode for the shared arguments; WI_ERR_INVALID_ARG
 * for a null sel_ids with top_k > 0. */
wi_status wi_select_refresh(const wi_decode_params *p, const wi_index_view *idx, const void *q,
                            int32_t *sel_ids, void *workspace, size_t ws_bytes, void *stream);

/* Per-cluster data of the estimation error bound of an index (the pages promise a controlled
 * error for the estimation zone without a formula: RetroInfer technical summary, section 2.A
 * item 3; Arabic summary, section 2.a).  With |x|^2 the sum over coordinates in ascending order
 * of fp64 squares (differences rounded to fp64 first, no fused multiply-add) and sqrt_up(y) the
 * smallest float f >= 0 with f * f >= y:
 *   radius [B,Hkv,C] float  sqrt_up(max over the members i of c of |k_i - mu_c|^2), mu_c the
 *                           stored centroid; 0 for an empty cluster (nullable when C = 0)
 *   vnorm  [B,Hkv,C] float  sqrt_up(max over the members of |v_i|^2); 0 for an empty cluster
 *                           (nullable when C = 0)
 *   vmax   [B,Hkv]   float  sqrt_up(max |v|^2 over every token, steady zone included)
 * p gives B, Hkv, d, dtype, n_steady, C and Nc as for wi_decode (Hq, top_k and scale are not
 * read).  The index is only read; the outputs are caller-allocated device buffers.  Errors:
 * WI_ERR_INVALID_ARG for null pointers or inconsistent sizes, WI_ERR_UNSUPPORTED as wi_decode. */
wi_status wi_bound_data(const wi_decode_params *p, const wi_index_view *idx, float *radius,
                        float *vnorm, float *vmax, void *stream);

/* One decode step whose retrieval zone is sized per query head to meet an error bound (the
 * pages promise a controlled error for the estimation zone without a formula: RetroInfer
 * technical summary, section 2.A item 3; Arabic summary, section 2.a).  With s = scale, |q| the
 * query norm, sigma_c the query-centroid score, m* the largest s sigma_c of the head, and the
 * bound data of wi_bound_data (r_c = radius, V_c = vnorm, V_all = vmax), every non-empty cluster
 * has w_c = n_c exp(s sigma_c - m*), x_c = s |q| r_c and
 *   err_c = w_c (exp(x_c) - 1) (V_c + (1 + u) V_all) + w_c u V_c,   lo_c = w_c exp(-x_c),
 * u the relative rounding bound of the stored value sums (2^-8 + 2^-23 for bf16, 2^-24 for
 * fp32).  A zone made of the k first non-empty clusters in the order (-sigma_c, c) bounds
 * |out - dense attention| by A(k) = (sum of err_c outside the zone) / (sum of every lo_c).  The
 * zone is the smallest k in [0, min(top_k, #non-empty)] with A(k) <= eps (the cap if none), with
 * every term and A(k) taken on canonical fp64 scores; its clusters are then the top k exactly as
 * wi_decode selects them.  Each head first decides on fp32 scores and terms and keeps that
 * decision when rigorous bounds on their rounding (and on the clusters whose fp32 order may
 * differ from the canonical one) show A(k) <= eps and A(k - 1) > eps; otherwise it recomputes
 * every non-empty cluster's terms in fp64 from canonical scores and decides on those.  The size
 * is therefore the fp64 decision unless some A(j) lies within fp64 rounding of eps.
 *   radius, vnorm [B,Hkv,C], vmax [B,Hkv]  float  from wi_bound_data for this index
 *   eps                                     >= 0 (inf: the smallest zone, k = 0)
 *   sel_ids   [B,Hq,top_k] int32  the zone, ascending, -1 padded (nullable)
 *   k_used    [B,Hq]       int32  the zone size of each head (nullable)
 *   err_bound [B,Hq]       float  the bound after attention (nullable): the same sums outside
 *             the zone with |out| in place of (1 + u) V_all and, in the denominator, the exact
 *             part's total plus the estimated clusters' lo_c; 0 when nothing is estimated
 *   n_exact   [1]          uint32 device counter (nullable), incremented once for every head
 *             that decided in fp64; the caller zeroes it
 * Everything else, and the errors, as wi_decode; also WI_ERR_INVALID_ARG for a null radius,
 * vnorm (C > 0) or vmax, or eps < 0 or NaN, and WI_ERR_UNSUPPORTED for top_k > 2048. */
wi_status wi_decode_bounded(const wi_decode_params *p, const wi_index_view *idx, const float *radius,
                            const float *vnorm, const float *vmax, const void *q, float eps,
                            float *out, float *lse, int32_t *sel_ids, int32_t *k_used,
                            float *err_bound, uint32_t *n_exact, void *workspace, size_t ws_bytes,
                            void *stream);

/* ---------------------------------------------------------------------------------------
 * Wave buffer (RetroInfer technical summary, section 2.B; Arabic summary, section 2.b): decode
 * over an index whose cluster-major K/V copies (wi_index_view.k_perm / v_perm) live in host
 * memory, with a GPU cache of KV blocks managed from the host off the attention's critical path
 * and an execution buffer for the blocks the cache misses.
 *
 * The clustered rows of each (b, KV head) are cut into blocks of 16 rows.  One device pool holds
 * cache_blocks cached blocks and exec_blocks execution-buffer blocks.  Each wi_decode_wavebuf
 * call, in stream order: applies the admissions the host decided from the previous call (copying
 * the previous call's staged misses into cache slots); scores and selects as wi_decode; for every
 * block a head's retrieval zone touches, uses the cached copy, or copies the block from host
 * memory into the execution buffer, or, when the execution buffer is full, leaves it in host
 * memory for the attention kernel to read there; attends and merges.  The call's access log goes
 * back to the host on a stream of the wave buffer's own while attention runs.  The host decides
 * from each call's log two calls later (logs and execution buffer are double-buffered, so the
 * host never waits for the call just enqueued), in call order: it updates the LRU order, the
 * hits first, then the staged misses, each in ascending (b, KV head, block) order; every staged
 * miss not cached since is admitted, into a free slot or in place of the least recently used
 * block.  The admissions decided from call t take effect at call t + 2.  Blocks read from host
 * memory in place are not admitted.  Results equal wi_decode's bit for bit whatever the cache
 * holds.
 *
 * Requirements: k_perm and v_perm must be host memory the device can read (hipHostMalloc);
 * every other index buffer, q, out, lse, sel_ids and the workspace are device memory.  The
 * device memory of the wave buffer (wi_wavebuf_device_bytes: the cache, two execution-buffer
 * regions of exec_blocks, directory, logs; 256-byte aligned) is caller-
 * allocated and must outlive it; the host state (the LRU, a pinned copy of the log, a stream
 * and two events) is allocated by wi_wavebuf_create and freed by wi_wavebuf_destroy.  One
 * wave buffer serves one index (same B, Hkv, Nc and dtype) and one stream at a time; its calls
 * must not overlap and cannot be captured in a graph (the host acts between them).  The pool
 * (cache_blocks + 2 * exec_blocks blocks of 16 rows) holds at most 2^29 rows.  After any error
 * from wi_decode_wavebuf, destroy the wave buffer (its host state may have advanced past the
 * device's).  Errors: WI_ERR_INVALID_ARG for null or negative arguments or a wave buffer of
 * another index, WI_ERR_UNSUPPORTED as wi_decode and for a pool beyond 2^29 rows,
 * WI_ERR_WORKSPACE for too little device memory. */
typedef struct wi_wavebuf wi_wavebuf;

wi_status wi_wavebuf_device_bytes(const wi_decode_params *p, int32_t cache_blocks,
                                  int32_t exec_blocks, size_t *bytes);
wi_status wi_wavebuf_create(const wi_decode_params *p, int32_t cache_blocks, int32_t exec_blocks,
                            void *device_mem, size_t bytes, void *stream, wi_wavebuf **out);
wi_status wi_decode_wavebuf(wi_wavebuf *wb, const wi_decode_params *p, const wi_index_view *idx,
                            const void *q, float *out, float *lse, int32_t *sel_ids,
                            void *workspace, size_t ws_bytes, void *stream);
/* (host) Waits for every pending log and decides from them (the decisions still take effect two
 * calls after the call they come from), then fills stats[6]: calls, hits, misses staged in the
 * execution buffer, blocks read from host memory in place, admissions, evictions (blocks are
 * counted once per call however many heads touch them). */
wi_status wi_wavebuf_stats(wi_wavebuf *wb, int64_t *stats);
wi_status wi_wavebuf_destroy(wi_wavebuf *wb);

/* Stages timed by the profiling hook below (one entry per kernel the entry points launch). */
typedef enum {
  WI_STAGE_SCORE = 0,     /* decode: query-centroid scores (MFMA), per-tile summaries       */
  WI_STAGE_SELECT = 1,    /* decode: per-head top-k and retrieval lists, and beside them the
                             estimation over all non-empty clusters                          */
  WI_STAGE_ATTEND = 2,    /* decode: exact attention over steady + retrieved rows and the
                             retrieved clusters' estimation terms                            */
  WI_STAGE_MERGE = 3,     /* decode: log-sum-exp merge into out and lse                      */
  WI_STAGE_PREP = 4,      /* build: steady-zone copies, key norms                           */
  WI_STAGE_INIT = 5,      /* build: seeded initial centroid directions                      */
  WI_STAGE_ASSIGN = 6,    /* build: k-means assignment (MFMA), all iterations               */
  WI_STAGE_RESCORE = 7,   /* build: fp64 re-decision of uncertain assignments               */
  WI_STAGE_CSR = 8,       /* build: sizes, offsets, permutation                             */
  WI_STAGE_UPDATE = 9,    /* build: centroid directions from member sums                    */
  WI_STAGE_FINAL = 10,    /* build: mean keys, value sums, cluster-major copies             */
  WI_STAGE_REFRESH = 11,  /* wi_select_refresh: the postponed top-k of reused groups        */
  WI_NUM_STAGES = 12
} wi_stage;

/* (host) Profiling hook for measurement tools.  While enabled, wi_decode and wi_build_index
 * record a pair of HIP events around each kernel they launch, on the call's stream (this adds
 * event records between the kernels; leave it disabled for production timing).  Enabling clears
 * the accumulated figures.  Not thread-safe against concurrent calls on several threads.
 * enable = 0 turns the hook off, 1 times every launch once; enable = R > 1 additionally launches
 * each decode kernel R times back to back between its two events (the decode kernels are pure
 * functions of their inputs, so the repeats leave the results unchanged), which measures the
 * per-launch duration without the cost of the event records themselves.  Negative values:
 * WI_ERR_INVALID_ARG. */
wi_status wi_profile_enable(int enable);

/* (host) Profiling hook for measurement tools: while wi_profile_enable(R) with R > 1 repeats each
 * decode kernel, repeat r reads the index through views[r mod n] instead of the call's own index
 * (the queries, workspace and outputs stay the call's).  The views must be bit-identical copies
 * of the index the calls decode, so that every repeat computes the same results; placed at other
 * HBM addresses, they keep a repeat's reads from hitting in the last-level cache, as they would
 * not in a run that decodes many sequences.  The array is copied; n = 0 clears the list.
 * Wave-buffer calls ignore it.  Errors: WI_ERR_INVALID_ARG for n < 0, or null views with n > 0. */
wi_status wi_profile_rotate(const wi_index_view *views, int n);

/* (host) Wait for the recorded events and return, per stage, the summed kernel time in
 * milliseconds and the number of launches (repeats included) since the hook was enabled.  Both arrays hold
 * WI_NUM_STAGES entries.  Synchronises on the recorded events only. */
wi_status wi_profile_read(double *total_ms, int64_t *launches);

/* (host) Static description of a status code. */
const char *wi_status_string(wi_status s);

/* (host) Detail of the last error raised on the calling thread ("" if none). */
const char *wi_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WAVE_INDEX_H_ */
