/*
 * hstu.h - C ABI of the MI355X (gfx950) jagged HSTU ranking encoder.
 *
 * What it computes. One DLRMv3/HSTU-style ranking-encoder stack over a jagged
 * batch of users, as described on the page "DLRMv3: MLPerf Inference generative
 * recommendation benchmark" (section "Model selection"): per layer a fused D->4D
 * projection, attention Mask(SiLU(Q K^T)) V with an absolute position bias added
 * to Q, K and V, and a post-attention GEMM of 3*D*D multiply-adds per token. The
 * user interaction history (UIH) is encoded once per request and shared by every
 * candidate; a user's history keys/values persist across consecutive timestamps
 * (same section). Candidates are target-aware (the multi-stage sequence model
 * page, "Target-Aware Multi-Head Attention"): they attend to the whole history
 * and to themselves, never to other candidates, and history rows never see
 * candidates, so the history's representation does not depend on the candidate
 * set. Jagged batches are concatenated rows plus offsets, the exclusive running
 * sum of per-user lengths (TorchRec DLRM tutorial page, section 2.1).
 *
 * Per layer l, for user b with m cached, n new history rows and c candidates:
 *   Xn = (X - mean(X)) / sqrt(var(X) + 1e-6)     (per row over its D features)
 *   S = SiLU(Xn W1_l) = [U | V | Q | K]          (each D wide)
 *   V += P_l[pos, 0:D]; Q += P_l[pos, D:2D]; K += P_l[pos, 2D:3D]
 *        new history row i has pos = m + i; every candidate has pos = m + n
 *   history row i:  O_i = (1/max_len) * sum_{key j <= m+i} SiLU(q_i . k_j) v_j
 *   candidate r:    O_r = (1/max_len) * (sum_{all m+n history keys j} SiLU(q_r . k_j) v_j
 *                                        + SiLU(q_r . k_r) v_r)
 *        (per head h: the columns [h*dh, (h+1)*dh), dh = D / heads)
 *   X_{l+1} = X_l + [U | O | U*O] W2_l
 * The position bias P_l is optional; a layer may instead (or also) carry a relative
 * table rel_l, and then every weight SiLU(q_i . k_j) gains rel_l[h][pos_i - pos_j]
 * (see hstu_layer_weights). The new history rows' K, V (after bias) are appended to
 * the cache. Entry points around the encoder: hstu_pack_uih builds the history
 * tokens from per-event context and action embeddings, hstu_score turns candidate
 * rows into outcome probabilities, and hstu_pool_* manage the pages of a paged
 * cache for time-ordered request replay.
 *
 * bfloat16 mode: storage is bfloat16, accumulation float32; results are rounded
 * to bfloat16 (nearest, ties to even) at U,V,Q,K; at each attention weight SiLU(q.k)
 * (plus the relative bias, when there is one); at each attention output; at the gate
 * U*O; and at X + Z. The normalisation is applied to the projection's float32 product,
 * so Xn is never rounded.
 * float32 mode: float32 storage and arithmetic throughout.
 *
 * Conventions for every entry point:
 *  - Host pointers are read during the call only. Device pointers must stay valid
 *    until the work enqueued on `stream` has completed.
 *  - Nothing is allocated on the device or in pinned host memory by the library;
 *    scratch memory is the caller's workspace. The per-call work plan (a few bytes
 *    per user and per attention work item) is computed on the host, in host memory
 *    the calling thread keeps for its next calls, and reaches the workspace inside
 *    the arguments of small copy kernels, which the runtime captures when they are
 *    enqueued.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 *    stream). There is no device or host synchronisation inside a call.
 *  - Every argument is validated on the host before anything is enqueued. On a
 *    validation error nothing is launched and no host array is modified.
 *  - Calls may run concurrently from several host threads if each uses its own
 *    workspace, outputs and cache slots.
 *  - Inputs, outputs, workspace and cache must not overlap.
 */
#ifndef HSTU_H_
#define HSTU_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSTU_ABI_VERSION 9

/* Element type of every device tensor of a call. */
enum hstu_dtype { HSTU_F32 = 0, HSTU_BF16 = 1 };

/* Status codes. No exception or abort ever crosses the ABI. */
enum hstu_status_code {
  HSTU_OK = 0,
  HSTU_ERR_NULL = 1,       /* a required pointer is NULL                                  */
  HSTU_ERR_SHAPE = 2,      /* unsupported dims/dtype (see hstu_dims), B < 0, or a user   */
                           /* with 2^30 or more history rows or candidates              */
  HSTU_ERR_OFFSETS = 3,    /* offsets do not start at 0 or decrease                        */
  HSTU_ERR_CAPACITY = 4,   /* m+n >= max_len, cache capacity < m+n, bad or repeated slot,   */
                           /* cached_len < 0, or one user's keys of one layer span 2 GiB or */
                           /* more ((m+n) * row pitch in bytes; the pitch is D elements with */
                           /* a cache, 3D without); paged: a bad page_rows, pages or        */
                           /* pages_per_user, too few pages per user, or a pool of 2 GiB    */
  HSTU_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than hstu_workspace_size()          */
  HSTU_ERR_HIP = 6,        /* a HIP runtime call failed; outputs and cache are undefined    */
  HSTU_ERR_ALIGN = 7,      /* a device pointer is not 16-byte aligned                       */
  HSTU_ERR_TOO_LARGE = 8   /* hstu_encode_static: the batch exceeds its fixed scratch       */
};
typedef int32_t hstu_status;

/* Model dimensions, fixed for a model.
 *  layers  >= 1
 *  d_model  D; heads H (at most 127) with dh = D / H.
 *           float32:  D % 64 == 0 and dh in {32, 64, 128}
 *           bfloat16: D % 128 == 0 and dh in {32, 64, 128}
 *  max_len  rows of each position-bias table; every user needs m + n + 1 <= max_len
 *           (history positions 0..m+n-1 plus the candidate slot m+n). The attention
 *           scale is 1/max_len. A table has fewer than 2^31 elements:
 *           max_len * 3 * D < 2^31.
 *  dtype    enum hstu_dtype.
 *  weight_layout  enum hstu_weight_layout: how hstu_encode and hstu_encode_static
 *           read w_uvqk and w_out (hstu_layer_weights); every entry point that takes
 *           dims rejects other values with HSTU_ERR_SHAPE. */
typedef struct hstu_dims {
  int32_t layers;
  int32_t d_model;
  int32_t heads;
  int32_t max_len;
  int32_t dtype;
  int32_t weight_layout;
} hstu_dims;

/* Layout of the two weight matrices of a layer.
 *  HSTU_WEIGHTS_PREPARED  w_uvqk [4D][D], w_out [D][3D]: each output feature's weights
 *                         in one row, as the GEMMs read them (hstu_transpose_weights
 *                         makes them from the other layout once per model).
 *  HSTU_WEIGHTS_MATH      w_uvqk [D][4D] (W1, column blocks U, V, Q, K) and w_out
 *                         [3D][D] (W2, row blocks U, O, U*O), as the projection X W1 and
 *                         the output GEMM [U | O | U*O] W2 are written. Each call then
 *                         transposes both into its workspace first (7 D^2 elements a
 *                         layer, counted in hstu_workspace_size; two launches for up to
 *                         16 layers): 29 MB and about 40 us a call at D = 512 and 8
 *                         layers, 1% of that call. */
typedef enum hstu_weight_layout { HSTU_WEIGHTS_PREPARED = 0, HSTU_WEIGHTS_MATH = 1 } hstu_weight_layout;

/* One layer's parameters: device pointers, row-major, in the call's dtype.
 *  w_uvqk   HSTU_WEIGHTS_PREPARED: [4D][D], output feature j of the projection in row j
 *           (the transpose of W1 [D][4D]); row blocks U, V, Q, K.
 *           HSTU_WEIGHTS_MATH: W1 itself, [D][4D].
 *  w_out    HSTU_WEIGHTS_PREPARED: [D][3D], output feature j of the output GEMM in row
 *           j (the transpose of W2 [3D][D]); column blocks U, O, U*O.
 *           HSTU_WEIGHTS_MATH: W2 itself, [3D][D].
 *  pos_bias [max_len][3D]: row p is the absolute bias of position p, added to V, Q, K
 *           after the SiLU (column blocks V, Q, K); NULL: no absolute bias.
 *  rel_bias [H][max_len]: rel_bias[h][d] is added to every attention weight
 *           SiLU(q_i . k_j) of head h whose relative position pos_i - pos_j is d
 *           (the original HSTU form Mask(SiLU(Q K^T) + bias) V from the DLRMv3
 *           page's "Model selection" section); NULL: no relative bias.
 * w_uvqk, w_out and any non-NULL table are 16-byte aligned. In bfloat16 each call widens
 * a layer's relative table to float32 in its workspace (H * max_len * 4 bytes, counted in
 * hstu_workspace_size) before that layer's attention. */
typedef struct hstu_layer_weights {
  const void* w_uvqk;
  const void* w_out;
  const void* pos_bias;
  const void* rel_bias;
} hstu_layer_weights;

/* Streaming key/value cache (caller-owned): user b's history keys / values (after
 * position bias) at positions 0..cached_len[b]-1, in one of two layouts.
 *  cached_len    host [B], in/out: m_b on entry; m_b + n_b after a successful call.
 *  page_rows == 0: slot layout.
 *    k, v          device, each [layers][slots][capacity][D] in the call's dtype; user b's
 *                  position p is row p of slot slot_of_user[b].
 *    slot_of_user  host [B]; distinct slots in [0, slots). m_b + n_b <= capacity.
 *  page_rows == 64: paged layout (the pages field set, slots/capacity/slot_of_user
 *                  unused). The cache holds each user's rows in pages of 64, so the
 *                  memory a user holds grows with its history, 64 rows at a time.
 *    k, v          device, each [layers][pages][64][D] in the call's dtype.
 *    page_table    DEVICE int32 [B][pages_per_user] (4-byte aligned): user b's position
 *                  p is row p % 64 of page page_table[b][p / 64]. Entries
 *                  0..ceil((m_b+n_b)/64)-1 of each row must hold page ids in [0, pages),
 *                  no page used by two users (or twice) of one call. The library cannot
 *                  check device contents: a page id outside [0, pages) reads as zeros
 *                  and takes no writes (results are then wrong, but no memory outside
 *                  the pool is touched). ceil((m_b+n_b)/64) <= pages_per_user, and one
 *                  layer's pool spans under 2 GiB (pages * 64 * D * element size).
 * The call reads positions 0..m_b-1 and writes positions m_b..m_b+n_b-1 of each layer.
 * Candidates are never appended. */
typedef struct hstu_kv_cache {
  void* k;
  void* v;
  int32_t slots;
  int32_t capacity;
  const int32_t* slot_of_user;
  int32_t* cached_len;
  int32_t page_rows;
  int32_t pages;
  int32_t pages_per_user;
  const int32_t* page_table;
} hstu_kv_cache;

/* HSTU_ABI_VERSION of the loaded library. */
int32_t hstu_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* hstu_status_string(hstu_status s);

/* Bytes of device workspace hstu_encode needs for this batch (host-only; launches
 * nothing). uih_offsets / cand_offsets: host int32 [B+1], starting at 0,
 * non-decreasing; user b owns history rows uih_offsets[b]..uih_offsets[b+1]-1 and
 * candidate rows cand_offsets[b]..cand_offsets[b+1]-1. */
hstu_status hstu_workspace_size(const hstu_dims* d, int32_t B, const int32_t* uih_offsets,
                                 const int32_t* cand_offsets, size_t* bytes);

/* Work of one hstu_encode call (host-only integer arithmetic).
 *  algorithmic_flops: 2 x the multiply-adds the method needs over all layers: both
 *    GEMMs for every new history row and candidate, q.k and a*v for every masked pair
 *    (history row i of user b sees m_b+i+1 keys; a candidate sees m_b+n_b keys plus
 *    itself). Per layer and user: 14*(n+c)*D^2 + 4*D*(n*m + n(n+1)/2 + c*(m+n+1)).
 *  formula_flops: the benchmark page's expression
 *    2*layers*(N*N*D/2 + N*D*D*4 + N*D*D*3) with N = m+n, summed over users.
 * cached_len may be NULL (all m = 0). Either output pointer may be NULL.
 * Errors: those of hstu_workspace_size's arguments, HSTU_ERR_CAPACITY for a negative
 * cached_len, HSTU_ERR_SHAPE when either count exceeds 2^64 - 1 (possible only for
 * batches hstu_encode would refuse: it bounds every user by max_len). */
hstu_status hstu_flops(const hstu_dims* d, int32_t B, const int32_t* uih_offsets,
                       const int32_t* cand_offsets, const int32_t* cached_len,
                       uint64_t* algorithmic_flops, uint64_t* formula_flops);

/* The attention's work plan of one hstu_encode call (host-only; launches nothing), for
 * inspection and tests. A work item is (user, head, up to Q query rows of one kind) with
 * Q = 128 in bfloat16 and 64 in float32. Items of one (user, head) go whole to one of
 * 8 bins (one per XCD; workgroup w runs on XCD w % 8), groups largest first on the least
 * loaded bin, and inside a bin the items run longest first. Writes *grid (the
 * attention's workgroup count, 8 x the longest bin) and, when codes is not NULL and
 * capacity >= *grid, codes[w] for workgroup w: -1 for no work, else
 * (user << 32) | (query block << 8) | (head << 1) | is_candidate, the query block
 * counting Q-row blocks of the user's history (or candidate) rows. cached_len may be
 * NULL (all m = 0). Errors: as hstu_workspace_size; HSTU_ERR_WORKSPACE if codes is not
 * NULL and capacity < *grid (then *grid is still written). */
hstu_status hstu_attention_plan(const hstu_dims* d, int32_t B, const int32_t* uih_offsets,
                                const int32_t* cand_offsets, const int32_t* cached_len, int32_t* grid,
                                int64_t* codes, int64_t capacity);

/* Encode one jagged batch through all layers.
 *  uih        device [uih_offsets[B]][D]   new history tokens of every user
 *  cand       device [cand_offsets[B]][D]  candidate tokens
 *  w          host array of d->layers entries (device pointers inside)
 *  kv         NULL (no earlier history: m_b = 0, nothing appended) or a cache
 *  uih_out    device [uih_offsets[B]][D]   final-layer rows of the new history tokens
 *  cand_out   device [cand_offsets[B]][D]  final-layer rows of the candidates
 *  workspace  device, >= hstu_workspace_size() bytes, 256-byte aligned
 * Users with n_b = 0 and/or c_b = 0, and B = 0, are valid. Device pointers must be
 * 16-byte aligned. On HSTU_OK, kv->cached_len[b] has been advanced by n_b. */
hstu_status hstu_encode(const hstu_dims* d, int32_t B, const int32_t* uih_offsets,
                        const int32_t* cand_offsets, const void* uih, const void* cand,
                        const hstu_layer_weights* w, hstu_kv_cache* kv, void* uih_out,
                        void* cand_out, void* workspace, size_t workspace_bytes, void* stream);

/* hstu_encode for callers that cannot allocate (code under HIP graph capture, serving
 * loops, harnesses that forbid allocation): the same arguments without the workspace,
 * the same plan, kernels and results (bit for bit). It calls no hipMalloc, hipFree or
 * other allocating routine, on the device or the host, and never records timing events.
 *  - Its workspace is a fixed device array of 64 MiB in the library (file-scope, one copy
 *    per GPU, held from the GPU's first call until the process ends); the planner works
 *    in fixed host arrays. Batches whose workspace (hstu_workspace_size) exceeds 64 MiB,
 *    with more than 1024 users or more than 16384 attention work items (per head,
 *    ceil(n_b/128) + ceil(c_b/128) summed over users, bfloat16; 64-row items in float32)
 *    are rejected with HSTU_ERR_TOO_LARGE before anything is enqueued. 64 MiB holds about
 *    9000 rows (history plus candidates) at D = 512 in bfloat16.
 *  - Every call on one GPU shares that GPU's array, and a later call overwrites what an
 *    earlier one left there: calls that overlap on one GPU (concurrent streams, or host
 *    threads with different streams) race, so the caller orders them (e.g. one stream).
 *    Host threads are serialised around the planning inside the call.
 *  - The stream must belong to the current device. Errors as hstu_encode, plus
 *    HSTU_ERR_TOO_LARGE; HSTU_ERR_HIP also when the array's device address cannot be
 *    looked up. */
hstu_status hstu_encode_static(const hstu_dims* d, int32_t B, const int32_t* uih_offsets,
                               const int32_t* cand_offsets, const void* uih, const void* cand,
                               const hstu_layer_weights* w, hstu_kv_cache* kv, void* uih_out, void* cand_out,
                               void* stream);

/* History tokens from per-event context and action embeddings: the two input forms
 * of the DLRMv3 page's action-embedding paragraph (section "Model selection"). The
 * original HSTU weaves each event's context features and its action into the
 * sequence as two tokens, doubling its length; DLRMv3 merges the two embeddings of
 * an event into one token instead (read here as their sum).
 *  events   E >= 0: rows of context and action, every user's events concatenated in
 *           the jagged order of the history offsets
 *  mode     HSTU_PACK_SUM: uih [E][D], row e = context[e] + action[e], added in float32
 *             and rounded once to the dtype (nearest, ties to even)
 *           HSTU_PACK_INTERLEAVE: uih [2E][D], rows 2e and 2e+1 = context[e] and
 *             action[e]; user b's tokens are rows 2*o[b] .. 2*o[b+1]-1 for event offsets
 *             o, so hstu_encode takes the offsets 2*o (and a user with m cached events
 *             has 2m cached tokens)
 *  context, action  device [E][D] in the dims' dtype; uih device output, which must
 *           not overlap them. All three 16-byte aligned.
 * Only d_model and dtype matter, but the dims are checked as for hstu_encode.
 * Errors: HSTU_ERR_SHAPE (dims, E < 0, unknown mode, or an output of 2^31 or more
 * 16-byte chunks), HSTU_ERR_NULL (a device pointer is NULL while E > 0),
 * HSTU_ERR_ALIGN, HSTU_ERR_HIP (the launch failed). E = 0 launches nothing.
 * Enqueued on `stream` like hstu_encode; the two can share a stream. */
enum hstu_pack_mode { HSTU_PACK_SUM = 0, HSTU_PACK_INTERLEAVE = 1 };
hstu_status hstu_pack_uih(const hstu_dims* d, int32_t events, int32_t mode, const void* context,
                          const void* action, void* uih, void* stream);

/* Weights from the layout the method writes them in to the layout hstu_encode reads,
 * once per model (e.g. at load time): dst[c][r] = src[r][c] for a device matrix src
 * [rows][cols], row-major, in dtype (HSTU_F32 or HSTU_BF16); elements are copied bit for
 * bit. The projection X W1 with W1 [D][4D] (column blocks U, V, Q, K) gives w_uvqk
 * [4D][D] from rows = D, cols = 4D; the output GEMM [U | O | U*O] W2 with W2 [3D][D]
 * (row blocks U, O, U*O) gives w_out [D][3D] from rows = 3D, cols = D. The DLRMv3 page's
 * FLOP formula (section "Model selection") names the two GEMMs; this only changes where
 * each weight sits.
 *  src, dst  device, element-aligned, not overlapping
 * Errors: HSTU_ERR_SHAPE (unknown dtype, rows or cols < 0, rows * cols >= 2^31, or the
 * two matrices overlap), HSTU_ERR_NULL (a pointer is NULL while rows * cols > 0),
 * HSTU_ERR_ALIGN, HSTU_ERR_HIP (the launch failed). An empty matrix launches nothing.
 * Enqueued on `stream` like hstu_encode. */
hstu_status hstu_transpose_weights(int32_t dtype, int32_t rows, int32_t cols, const void* src, void* dst,
                                   void* stream);

/* Candidate scoring head: the probability of each predicted outcome for every
 * candidate row. The DLRMv3 page keeps a top-layer MLP for the final prediction
 * (section "Model selection"); the TorchRec tutorial page (section 1.1, the final
 * output) takes the probability as the sigmoid of the top MLP's output.
 *  x        device [rows][D] in the dims' dtype: candidate rows, e.g. hstu_encode's
 *           cand_out
 *  head     host array of head_layers (1..8) layers; layer l maps its input h (width
 *           D for l = 0, else layer l-1's out_features) to h W^T + b, followed by
 *           ReLU on every layer but the last:
 *             weight  device [out_features][in] row-major, in the dtype
 *             bias    device [out_features], in the dtype
 *           hidden out_features: multiples of 128 in [128, 512]; the last layer's
 *           out_features (the outcomes): 1..16; D <= 512
 *  prob     device float32 [rows][outcomes]: sigmoid of the last layer's outputs
 * bfloat16: products accumulate in float32; hidden activations are rounded to
 * bfloat16 (nearest even) after ReLU; logits and probabilities are not rounded.
 * float32: float32 throughout. All device pointers 16-byte aligned.
 * Errors: HSTU_ERR_SHAPE (dims, widths, layer count, rows < 0), HSTU_ERR_NULL,
 * HSTU_ERR_ALIGN, HSTU_ERR_HIP. rows = 0 launches nothing. Enqueued on `stream`. */
typedef struct hstu_head_layer {
  const void* weight;
  const void* bias;
  int32_t out_features;
} hstu_head_layer;
hstu_status hstu_score(const hstu_dims* d, int32_t rows, const void* x, const hstu_head_layer* head,
                       int32_t head_layers, float* prob, void* stream);

/* Streaming replay: a host-side manager of a paged hstu_kv_cache (page_rows 64).
 * Requests are replayed in time order (the DLRMv3 page, section "Dataset selection")
 * and a user's history keys/values are reused across its consecutive requests (section
 * "Model selection"); cached state goes stale (the multi-stage sequence model page, its
 * limitations section: invalidation and TTL design). Per request the pool decides
 * whether the user's cached rows are extended or its history is encoded again, and
 * which pages hold the user's rows: a user holds ceil(rows / 64) pages of the cache, so
 * the memory it takes follows its history. Host only: it launches nothing and touches
 * no device memory (the caller copies each batch's page table to the device).
 *
 * hstu_pool_create: a pool of `pages` (>= 1) pages, the `pages` of the hstu_kv_cache it
 *   manages; `max_rows` (>= 1): most rows one user may hold (use at most max_len - 1,
 *   so that a user's history also fits the position tables); `ttl` (>= 0): cached rows
 *   last committed more than ttl time units before a request are stale. Errors:
 *   ERR_NULL, ERR_SHAPE, ERR_HIP (the host allocation failed).
 * hstu_pool_assign: one batch of B requests from distinct users (ids >= 0) at time
 *   `now`; user b brings new_events[b] (>= 0) events since its last request, and
 *   would resend window[b] (0..max_rows) events, its latest, if its history must be
 *   encoded again. For each user it writes cached_len[b] and rebuild[b]:
 *     0  the user's fresh rows can take the new events (cached + new <= max_rows):
 *        send only the new events, after cached_len[b] cached rows;
 *     1  cached_len[b] = 0: send the latest window[b] events, as new rows;
 *   and row b of page_table (host int32 [B][pages_per_user]): the user's pages in
 *   position order for its rows after the call (hits keep their pages and get more,
 *   a rebuild reuses the user's pages), -1 past them. When too few pages are free,
 *   the least recently committed users outside the batch and not pending are evicted
 *   (all their pages freed), oldest first. Every user of the batch is pending until
 *   hstu_pool_commit or hstu_pool_abort; a pending user may not be assigned again.
 *   Errors (the pool and the output arrays unchanged): ERR_NULL, ERR_SHAPE (B < 0,
 *   pages_per_user < 1, an id < 0, repeated or pending, new_events < 0, window out of
 *   range), ERR_CAPACITY (a user would need more than pages_per_user pages, or the
 *   batch does not fit even after evicting every user it may evict).
 * hstu_pool_commit: after hstu_encode succeeded for the batch: user b now holds
 *   total_len[b] rows (cached_len + rows sent), last used at `now`; pages beyond its
 *   rows are freed. Errors (nothing changed): ERR_SHAPE (a user not pending),
 *   ERR_CAPACITY (a length below the cached length, above max_rows or its pages).
 * hstu_pool_abort: after a failed encode: the users' pages are freed, the users
 *   forgotten.
 * hstu_pool_stats: counters indexed by enum hstu_pool_stat.
 * hstu_pool_lookup: a user's committed rows and the pages it holds (0, 0 if absent).
 * A pool is not synchronised: calls on one pool from several threads need the
 * caller's lock. */
typedef struct hstu_kv_pool hstu_kv_pool;
enum hstu_pool_stat {
  HSTU_POOL_HITS = 0,            /* cached rows extended                          */
  HSTU_POOL_REBUILD_NEW = 1,     /* user had no cached rows                       */
  HSTU_POOL_REBUILD_STALE = 2,   /* cached rows older than ttl                    */
  HSTU_POOL_REBUILD_FULL = 3,    /* no room for the new events under max_rows     */
  HSTU_POOL_EVICTIONS = 4,       /* users whose pages were taken for other users  */
  HSTU_POOL_PAGES_IN_USE = 5,    /* pages held now                                */
  HSTU_POOL_PAGES_PEAK = 6,      /* most pages held after any assign              */
  HSTU_POOL_STATS = 7
};
hstu_status hstu_pool_create(int32_t pages, int32_t max_rows, int64_t ttl, hstu_kv_pool** pool);
void hstu_pool_destroy(hstu_kv_pool* pool);
hstu_status hstu_pool_assign(hstu_kv_pool* pool, int32_t B, const int64_t* user, const int32_t* new_events,
                             const int32_t* window, int64_t now, int32_t pages_per_user, int32_t* page_table,
                             int32_t* cached_len, int32_t* rebuild);
hstu_status hstu_pool_commit(hstu_kv_pool* pool, int32_t B, const int64_t* user, const int32_t* total_len,
                             int64_t now);
hstu_status hstu_pool_abort(hstu_kv_pool* pool, int32_t B, const int64_t* user);
hstu_status hstu_pool_stats(const hstu_kv_pool* pool, int64_t* stats, int32_t n);
hstu_status hstu_pool_lookup(const hstu_kv_pool* pool, int64_t user, int32_t* len, int32_t* pages);

/* Measurement aid: device time of each kernel that hstu_encode, hstu_pack_uih and
 * hstu_score launch, taken with HIP events recorded on the caller's stream
 * immediately before and after every launch while timing is enabled (calls on one
 * device at a time).
 *  hstu_timing_enable(1) discards earlier records and starts recording;
 *  hstu_timing_enable(0) stops recording (records are kept).
 *  hstu_timing_select(mask) restricts the events to the kernel kinds k whose bit
 *  (1 << k) is set (all kinds until called; kept across enable/disable). Each timed
 *  launch adds two event records to the stream, and they cost device time between
 *  kernels: timing a subset of kinds costs less.
 *  hstu_timing_read waits for the recorded events, then writes, per kernel kind k <
 *  kinds (enum hstu_kernel_kind), the summed milliseconds total_ms[k] and the number
 *  of launches[k] recorded since enabling; it consumes the records. */
enum hstu_kernel_kind {
  HSTU_KERNEL_PLAN = 0,       /* jagged row planner                      */
  HSTU_KERNEL_UVQK = 1,       /* projection GEMM + SiLU + bias + append  */
  HSTU_KERNEL_ATTENTION = 2,  /* target-aware causal SiLU attention      */
  HSTU_KERNEL_OUT = 3,        /* gated output GEMM + residual            */
  HSTU_KERNEL_NORM = 4,       /* normalisation work: float32 models normalise each  */
                              /* layer's input rows; bfloat16 models run two passes  */
                              /* per call (W1 column sums, first-layer row sums) and */
                              /* normalise inside the projection                     */
  HSTU_KERNEL_PACK = 5,       /* hstu_pack_uih                           */
  HSTU_KERNEL_SCORE = 6,      /* hstu_score                              */
  HSTU_KERNEL_KINDS = 7
};
hstu_status hstu_timing_enable(int32_t enable);
hstu_status hstu_timing_select(uint32_t kinds_mask);
hstu_status hstu_timing_read(double* total_ms, int64_t* launches, int32_t kinds);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_H_ */
