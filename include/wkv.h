/*
 * wkv.h -- C ABI of libwkv, the KV-memory hot path of WorldKV-style
 * autoregressive video world models, hand-written HIP for gfx950 (MI355X).
 *
 * Sources, cited by page title and section:
 *   [WorldKV]   "WorldKV: Efficient World Memory with World Retrieval and
 *               Compression": Sec. 4.2 World Retrieval, Sec. 4.3 World
 *               Compression, Sec. 5.1 Implementation Details.
 *   [WorldPager] WorldPager summary: abstract and Fig. 2 (int4 KV store in
 *               pinned host memory, retrieval from the extrapolated camera
 *               pose, no stall on a miss).
 *   [WorldAttention] WorldAttention breakdown: scaled dot-product attention of
 *               the current chunk over visible keys; the index-mapping and
 *               contiguous-copy stages of its kernel section; page scores as
 *               the dot product of the mean query and the mean key.
 *
 * Conventions for every call:
 *   - bf16 tensors are passed as uint16_t bit patterns. K / V / Q tensors are
 *     token-major and contiguous: [rows][H][D], one row = H*D*2 bytes.
 *   - Pointers are DEVICE memory unless marked [host]. Every device pointer
 *     must be 16-byte aligned. The caller allocates and owns every buffer; the
 *     library never allocates and never frees device memory.
 *   - Every call enqueues its kernels on the given stream (a hipStream_t; NULL
 *     = the default stream) and returns without synchronising. WKV_OK means
 *     "enqueued". A device-side fault surfaces at the caller's next
 *     synchronisation, as with any HIP launch.
 *   - All argument checks run on the host before anything is enqueued. A
 *     non-OK status from a check enqueues nothing and leaves every output
 *     untouched; the reason is available from wkv_last_error() (thread-local
 *     text). WKV_ERR_HIP reports a runtime failure of an enqueue, after which
 *     the call's earlier work may already be enqueued.
 *   - Calls are stateless and reentrant; ordering is the stream's. The host
 *     tier's slot table is state the caller owns and passes in.
 *   - Supported shapes: D in {64, 128}; H >= 1; H*D <= 8192.
 */
#ifndef WKV_H_
#define WKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WKV_ABI_VERSION 3

typedef void* wkv_stream_t; /* hipStream_t */

typedef enum {
  WKV_OK = 0,
  WKV_ERR_NULL = 1,        /* a required pointer is NULL                     */
  WKV_ERR_SHAPE = 2,       /* a size is out of range or inconsistent         */
  WKV_ERR_RATIO = 3,       /* keep ratio outside [0, 1] or NaN               */
  WKV_ERR_K = 4,           /* top-k count < 1 or pose history not 1 or 2     */
  WKV_ERR_ALIGN = 5,       /* a device pointer is not 16-byte aligned        */
  WKV_ERR_WORKSPACE = 6,   /* workspace too small                            */
  WKV_ERR_UNSUPPORTED = 7, /* head dim / dtype not supported                 */
  WKV_ERR_HIP = 8          /* the HIP runtime rejected a launch              */
} wkv_status;

/* Camera pose of a chunk: translation and yaw (radians). [WorldKV] Sec. 4.2
 * indexes each stored chunk by the camera state at its generation time. */
typedef struct {
  float x, y, z, yaw;
} wkv_pose;

/* Camera pose with a full rotation: translation and a quaternion (w, x, y,
 * z) of any non-zero norm ([WorldKV] Sec. 5.1 "geodesic distance in
 * rotation"). 32 bytes; pad is ignored. */
typedef struct {
  float x, y, z;
  float qw, qx, qy, qz;
  float pad;
} wkv_pose_q;

/* A run of window rows: k, v bf16 [n][H][D] (device). n may be 0 (then k, v
 * may be NULL). */
typedef struct {
  const uint16_t* k;
  const uint16_t* v;
  int32_t n;
} wkv_segment;

enum { WKV_BANK_BF16 = 0, WKV_BANK_INT4_G32 = 1 };

/* The store of compressed chunks ([WorldKV] Sec. 4.2: evicted chunks are kept
 * in memory, each indexed by its camera state). M chunks of Lc rows each.
 *   WKV_BANK_BF16:     k, v = bf16 [M][Lc][H][D]; k_scale, v_scale unused.
 *   WKV_BANK_INT4_G32: k, v = uint8 [M][Lc][H][D/2], element d of a (row,
 *                      head) in byte d/2, low nibble for even d, read as a
 *                      signed 4-bit integer q in [-8, 7]; k_scale, v_scale =
 *                      bf16 [M][Lc][H][D/32], one scale per 32 consecutive
 *                      elements along D. Value = bf16_RNE(float(q) * scale).
 *                      ([WorldPager] abstract / Fig. 2: the KV memory is
 *                      stored as int4.) */
typedef struct {
  int32_t dtype;
  int32_t M;
  int32_t Lc;
  const void* k;
  const void* v;
  const uint16_t* k_scale;
  const uint16_t* v_scale;
} wkv_bank;

/* ABI version of the loaded library (WKV_ABI_VERSION). */
int32_t wkv_abi_version(void);

/* Text of the last non-OK status returned on the calling thread. */
const char* wkv_last_error(void);

/* ------------------------------------------------------------------------
 * World Compression ([WorldKV] Sec. 4.3 "World Compression Mechanism").
 *
 * A unit is one evicted chunk at one layer: F frames x T tokens, frame 0 is
 * the anchor. For every non-anchor token (frame f >= 1, position j) the score
 * is, in float64, with cos = 0 when a norm is 0:
 *   WKV_SCORE_POSITION     s[(f-1)*T + j] = (1/H) sum_h cos(K[f,j,h,:], K[0,j,h,:])
 *                          the head-mean cosine to the anchor key at the same
 *                          position;
 *   WKV_SCORE_ANCHOR_MEAN  s[(f-1)*T + j] = (1/H) sum_h (1/T) sum_i cos(K[f,j,h,:], K[0,i,h,:])
 *                          the section's equation as printed: the mean cosine
 *                          to every anchor-frame key, averaged over heads.
 * The n_keep = wkv_keep_count(F, T, r)
 * lowest (score, pooled index) pairs are retained (ties go to the lower
 * index, NaN orders last). The compressed unit is the T anchor rows followed
 * by the retained rows in ascending source order, for K and V alike.
 * ------------------------------------------------------------------------ */

/* [host] n_keep = round-half-away(r * (F-1) * T) in float64, clamped to
 * [0, (F-1)*T]. Returns -1 for invalid arguments. Rows per compressed unit
 * are T + n_keep. */
int32_t wkv_keep_count(int32_t F, int32_t T, float r);

enum { WKV_SCORE_POSITION = 0, WKV_SCORE_ANCHOR_MEAN = 1 };

/* [host] Workspace bytes wkv_compress_chunk (or _int4) needs for B units
 * with the given score mode, with key_mean != 0 when the call is given a
 * key_mean output (an upper bound for every keep ratio: a call that is given
 * its scores output, or that needs no score at r = 0 or 1, uses less). 0 for
 * invalid arguments. */
size_t wkv_compress_workspace_bytes(int32_t B, int32_t F, int32_t T, int32_t H,
                                    int32_t D, int32_t score_mode, int32_t key_mean);

/* [host] Diagnostic: anchor-frame tokens each block of the compression score
 * kernel covers for a call on B units of T tokens and H heads with the given
 * score mode, int4 != 0 for wkv_compress_chunk_int4. The tile starts at one
 * pass of (token, head) pairs and, where each block carries fixed work that
 * more tokens amortise (the int4 store, the anchor-mean score), doubles while
 * the grid keeps >= 2048 blocks. It changes no result; tests use it to reach
 * every tile size. -1 for invalid arguments. */
int32_t wkv_compress_score_tile(int32_t B, int32_t T, int32_t H, int32_t score_mode,
                                int32_t int4);

/* Compress B contiguous units.
 *   k, v       bf16 [B][F*T][H][D]            inputs
 *   k_out,
 *   v_out      bf16 [B][Lc][H][D]             outputs, Lc = T + n_keep
 *   kept_idx   int32 [B][Lc]                  output: in-unit source row of
 *                                             every output row, ascending
 *   score_mode WKV_SCORE_POSITION or WKV_SCORE_ANCHOR_MEAN
 *   scores     double [B][(F-1)*T] or NULL    optional output
 *   key_mean   double [B][H][D] or NULL       optional output: the mean key of
 *                                             each compressed unit, the
 *                                             float64 mean of its Lc K rows
 *                                             per (head, dim), as query-based
 *                                             retrieval scores stored chunks
 *                                             (wkv_query_topk); equal to
 *                                             wkv_mean_rows of k_out up to
 *                                             the order of the float64 sums;
 *                                             bitwise reproducible
 *   ws         >= wkv_compress_workspace_bytes(B, F, T, H, D, score_mode,
 *              key_mean != NULL) bytes (may be NULL when that is 0)
 * Limits: 1 <= B <= 65535; 2 <= F <= 4; 1 <= T; (F-1)*T <= 8192; 0 <= r <= 1.
 * Errors: WKV_ERR_UNSUPPORTED for an unknown score_mode. */
wkv_status wkv_compress_chunk(const uint16_t* k, const uint16_t* v, int32_t B,
                              int32_t F, int32_t T, int32_t H, int32_t D,
                              float r, int32_t score_mode, uint16_t* k_out, uint16_t* v_out,
                              int32_t* kept_idx, double* scores, double* key_mean, void* ws,
                              size_t ws_bytes, wkv_stream_t stream);

/* wkv_compress_chunk without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The workspace is a static device array
 * of 64 MiB that every GPU the library runs on holds until the process ends;
 * its address on a device is resolved on the first call on that device
 * (make that first call outside graph capture). The call allocates nothing.
 * A call whose workspace (wkv_compress_workspace_bytes with key_mean = 0,
 * less the scores when given) exceeds 64 MiB is refused with
 * WKV_ERR_WORKSPACE. It has no key_mean output. Every call on one
 * GPU shares that GPU's array, which keeps the last call's contents: calls
 * that overlap on one GPU (on different streams, or concurrently enqueued by
 * other threads) race and must be ordered by the caller. Arguments, outputs,
 * limits and other errors as wkv_compress_chunk. */
wkv_status wkv_compress_chunk_noalloc(const uint16_t* k, const uint16_t* v, int32_t B,
                                      int32_t F, int32_t T, int32_t H, int32_t D, float r,
                                      int32_t score_mode, uint16_t* k_out, uint16_t* v_out,
                                      int32_t* kept_idx, double* scores, wkv_stream_t stream);

/* Compress B contiguous units and store the compressed rows in the int4
 * format of the bank (wkv_bank with WKV_BANK_INT4_G32): the int4 KV store of
 * [WorldPager] (abstract, Fig. 2) written at eviction time. Selection and
 * kept_idx / scores are exactly those of wkv_compress_chunk; every output row
 * is then encoded per group of 32 consecutive elements of one (row, head):
 *     scale = bf16_RNE(max|x| / 7)      (float32 division, correctly rounded)
 *     q     = clamp(rint(x / scale), -8, 7), q = 0 when scale == 0
 * with rint rounding half to even; element d is the low nibble of byte d/2
 * when d is even, the high nibble when d is odd.
 *   k_packed,
 *   v_packed   uint8 [B][Lc][H][D/2]           outputs
 *   k_scale,
 *   v_scale    bf16  [B][Lc][H][D/32]          outputs
 *   key_mean   double [B][H][D] or NULL        optional output: the mean of the
 *                                              unit's retained K rows as read
 *                                              (before encoding), exactly as
 *                                              wkv_compress_chunk gives it
 * Other arguments, limits and errors as wkv_compress_chunk. Inputs must be
 * finite: the codes of a group holding an Inf or NaN are unspecified. */
wkv_status wkv_compress_chunk_int4(const uint16_t* k, const uint16_t* v, int32_t B,
                                   int32_t F, int32_t T, int32_t H, int32_t D, float r,
                                   int32_t score_mode, uint8_t* k_packed, uint8_t* v_packed,
                                   uint16_t* k_scale, uint16_t* v_scale, int32_t* kept_idx,
                                   double* scores, double* key_mean, void* ws, size_t ws_bytes,
                                   wkv_stream_t stream);

/* ------------------------------------------------------------------------
 * World Retrieval by camera pose ([WorldKV] Sec. 4.2 retrieval equation
 * R = Top-k(sim(a_cur, a_i)); Sec. 5.1: distance = squared L2 translation +
 * geodesic rotation, each normalised over the candidate set, smallest first).
 *
 * For every stored chunk i, in float64:
 *   dt_i = (x_i-x_q)^2 + (y_i-y_q)^2 + (z_i-z_q)^2
 *   dr_i = |wrap(yaw_i - yaw_q)|, wrap into (-pi, pi]
 *   D_i  = minmax(dt)_i + minmax(dr)_i    (a term is 0 when its range is 0)
 * The k_eff = min(k, M) smallest (D_i, i) pairs are returned, sorted by
 * ascending chunk index.
 *
 * The query pose: n_hist = 1 -> query_hist[0]; n_hist = 2 -> extrapolated
 * linearly from query_hist[0] (previous) and query_hist[1] (last):
 * q = last + (last - prev), yaw = wrap(yaw_l + wrap(yaw_l - yaw_p)), formed
 * in float64 and stored as float ([WorldPager] Fig. 2: prefetch for the
 * next chunk is driven by a linearly extrapolated pose).
 *   bank_poses  wkv_pose [M]          device, 1 <= M <= 8192
 *   query_hist  wkv_pose [n_hist]     [host]
 *   out_idx     int32 [k_eff]         output, ascending chunk ids
 *   out_dist    double [k_eff]        optional output (NULL ok): D_i
 *   out_query   wkv_pose [1]          optional output (NULL ok): query used
 * ------------------------------------------------------------------------ */
wkv_status wkv_pose_topk(const wkv_pose* bank_poses, int32_t M,
                         const wkv_pose* query_hist, int32_t n_hist, int32_t k,
                         int32_t* out_idx, double* out_dist,
                         wkv_pose* out_query, wkv_stream_t stream);

/* [host] The query pose extrapolated one chunk ahead ([WorldPager] Fig. 2:
 * next-chunk retrieval runs on a linearly extrapolated pose):
 * translation last + (last - prev), yaw wrap(yaw_l + wrap(yaw_l - yaw_p)),
 * in float64, rounded to float. wkv_pose_topk with n_hist = 2 uses it. */
wkv_pose wkv_pose_extrapolate(wkv_pose prev, wkv_pose last);

/* [host] wkv_pose_topk evaluated on the host, for planning: the host tier
 * chooses the next chunk's staging set from the extrapolated pose while the
 * GPU still works on the current chunk ([WorldPager] Fig. 2: the pose is an
 * input known before compute). Same float64 operation sequence, result and
 * order as wkv_pose_topk; bank_poses, query_hist, out_idx [min(k, M)] and
 * out_dist (NULL ok) are host memory. */
wkv_status wkv_pose_topk_host(const wkv_pose* bank_poses, int32_t M, const wkv_pose* query_hist,
                              int32_t n_hist, int32_t k, int32_t* out_idx, double* out_dist);

/* Pose top-k with full rotations: as wkv_pose_topk with the rotation term
 *   dr_i = 2 * atan2(|r_xyz|, |r_w|),  r = conj(q_i) * q_query
 * (the SO(3) geodesic angle, float64 from the float32 values), min-max
 * normalised with the translation term. The query is given (no history).
 *   bank_poses  wkv_pose_q [M]   device, 1 <= M <= 8192
 *   query       wkv_pose_q [1]   [host]
 *   out_idx     int32 [min(k, M)], out_dist double [min(k, M)] (NULL ok) */
wkv_status wkv_pose_topk_so3(const wkv_pose_q* bank_poses, int32_t M, const wkv_pose_q* query,
                             int32_t k, int32_t* out_idx, double* out_dist,
                             wkv_stream_t stream);

/* ------------------------------------------------------------------------
 * Query-based World Retrieval ([WorldKV] Sec. 4.2: sim(a_cur, a_i) may be a
 * query-based importance score; [WorldAttention] pipeline: a page is scored
 * by the dot product of the current mean query and the page's mean key).
 *
 * A stored chunk is summarised by the float64 mean of its key rows, the
 * current chunk by the mean of its query rows (wkv_mean_rows), per (head,
 * dim). The score of chunk m is, in float64,
 *     s_m = sum_h sum_d key_means[m][h][d] * query_mean[h][d]
 * and the k_eff = min(k, M) largest (s_m, lower index first; NaN orders
 * last) are returned in ascending chunk index.
 * ------------------------------------------------------------------------ */

/* [host] Workspace bytes wkv_mean_rows needs for B units of L rows. */
size_t wkv_mean_rows_workspace_bytes(int32_t B, int32_t L, int32_t H, int32_t D);

/* out[b][h][d] = (1/L) * sum_i x[b][rows[b][i]][h][d] in float64.
 *   x      bf16 [B][L_in][H][D]                 input rows
 *   rows   int32 [B][L] or NULL                 rows averaged (NULL: the
 *                                               first L = L_in rows); an id
 *                                               outside [0, L_in) adds zeros
 *   out    double [B][H][D]                     output
 *   ws     >= wkv_mean_rows_workspace_bytes(B, L, H, D) bytes
 * Limits: 1 <= B <= 65535; 1 <= L <= 4194240; L <= L_in when rows is NULL;
 * H*D <= 8192, D in {64, 128}. Bitwise reproducible (fixed summation order). */
wkv_status wkv_mean_rows(const uint16_t* x, int32_t B, int32_t L_in, const int32_t* rows,
                         int32_t L, int32_t H, int32_t D, double* out, void* ws,
                         size_t ws_bytes, wkv_stream_t stream);

/* Top-k stored chunks by query score.
 *   key_means   double [M][H][D]    mean key of each stored chunk
 *   query_mean  double [H][D]       mean query of the current chunk
 *   out_idx     int32 [min(k, M)]   ascending chunk index
 *   scores      double [M]          output: every chunk's score (required)
 * Limits: 1 <= M <= 8192; k >= 1 (k > M is clamped). */
wkv_status wkv_query_topk(const double* key_means, int32_t M, const double* query_mean,
                          int32_t H, int32_t D, int32_t k, int32_t* out_idx, double* scores,
                          wkv_stream_t stream);

/* ------------------------------------------------------------------------
 * Host tier ([WorldKV] Sec. 4.2: evicted chunks are stored in GPU/CPU
 * memory; [WorldPager] abstract and Fig. 2: the int4 store lives in pinned
 * host memory, the next chunk's retrieval set is staged from the
 * extrapolated pose, and a retrieved chunk that is not staged is replaced
 * by staged data instead of stalling).
 *
 * A staging bank in HBM (a wkv_bank of n_slots chunks, same dtype and Lc as
 * the host bank) holds the chunks most recently requested. The table below
 * lives on the host and is owned by the caller; the library keeps no state.
 * Planning rule: the request gets a new stamp; an id already staged keeps
 * its slot; each other id, in request order, takes the slot with the
 * smallest (last-use stamp, slot index) among the slots holding no id of
 * the request, and is copied there.
 * ------------------------------------------------------------------------ */

#define WKV_TIER_MAX_SLOTS 64

typedef struct {
  int32_t n_slots;
  int32_t chunk[WKV_TIER_MAX_SLOTS];       /* chunk id held by each slot, -1 = empty */
  uint64_t last_use[WKV_TIER_MAX_SLOTS];   /* stamp of the last request using it, 0 = never */
  uint64_t clock;                          /* last stamp handed out */
} wkv_tier;

/* [host] Empty table of n_slots (1..WKV_TIER_MAX_SLOTS) slots. */
wkv_status wkv_tier_init(wkv_tier* t, int32_t n_slots);

/* [host] Plan a request without copying: ids (host, distinct, 1 <= n <=
 * n_slots, each >= 0). keep_ids [n_keep] (host, NULL when 0) name chunks
 * whose slots must not be evicted, because an enqueued chunk still reads
 * them. Writes slot_of[n], and the chunks to copy as copy_ids / copy_slots
 * [*n_copies] (host arrays of n entries). Updates t; a request that cannot
 * fit beside the kept chunks is WKV_ERR_SHAPE and changes neither t nor any
 * output. */
wkv_status wkv_tier_plan(wkv_tier* t, const int32_t* ids, int32_t n, const int32_t* keep_ids,
                         int32_t n_keep, int32_t* slot_of, int32_t* copy_ids,
                         int32_t* copy_slots, int32_t* n_copies);

/* How wkv_tier_prefetch moves chunks.
 *   WKV_TIER_COPY_KERNEL: one kernel reads the pinned host bank through its
 *     device mapping (host_bank must come from hipHostMalloc). It waits on
 *     the device for anything ordered before it on `stream`, but holds a few
 *     CUs while it runs.
 *   WKV_TIER_COPY_ENGINE: copy-engine transfers (hipMemcpyAsync), no CUs.
 *     Use it on a stream with no waits on other streams' events (order the
 *     staging by keep_ids and double-buffered tables instead): otherwise the
 *     runtime may block the host until those events complete. */
enum { WKV_TIER_COPY_KERNEL = 0, WKV_TIER_COPY_ENGINE = 1 };

/* Plan a request (as wkv_tier_plan, with keep_ids) and enqueue on `stream`,
 * in order: the copies of the chunks it needs from host_bank (pinned host
 * memory; ids < host_bank->M) into their staging slots, by copy_mode (a
 * kernel copy needs a device mapping of host_bank, else
 * WKV_ERR_UNSUPPORTED), then a small kernel writing the table's chunk
 * ids to dev_slot_chunk [n_slots] and each id's slot to dev_pred_slot [n]
 * (device; values captured at enqueue). The caller orders `stream` after
 * the last reader of the staging bank and its readers after this call's
 * work (events). *n_copies (host) receives the number of chunks copied.
 * staging->M must equal t->n_slots. On WKV_ERR_HIP the slots this request
 * was filling are marked empty in t (their contents are not to be trusted). */
wkv_status wkv_tier_prefetch(wkv_tier* t, const int32_t* ids, int32_t n, const int32_t* keep_ids,
                             int32_t n_keep, const wkv_bank* host_bank, const wkv_bank* staging,
                             int32_t H, int32_t D, int32_t copy_mode, int32_t* dev_slot_chunk,
                             int32_t* dev_pred_slot, int32_t* n_copies, wkv_stream_t stream);

/* For each retrieved chunk actual_idx[j] (device, j < n <= 64): out_slot[j]
 * = the slot of slot_chunk [n_slots] holding it (a hit). The misses (a
 * negative id is one), in rank order, take the entries of pred_slot [n]
 * (the predicted request's slots, rank order) that no hit uses, so a chunk
 * is never placed twice and the window never waits for a copy.
 * out_miss[0] = number of misses (device; NULL ok). out_slot then indexes
 * the staging bank in wkv_assemble_window. */
wkv_status wkv_tier_resolve(const int32_t* actual_idx, int32_t n, const int32_t* slot_chunk,
                            int32_t n_slots, const int32_t* pred_slot, int32_t* out_slot,
                            int32_t* out_miss, wkv_stream_t stream);

/* ------------------------------------------------------------------------
 * Window assembly ([WorldKV] Sec. 4.2: retrieved KV is inserted back into the
 * native attention window without re-encoding; Sec. 5.1: the window is
 * sink | retrieval | recent | denoising; [WorldAttention] kernel section:
 * selected KV is copied into one contiguous buffer before attention).
 *
 * Writes win_k / win_v bf16 [Nk][H][D] with
 *   rows [0, n_s)                          = sink
 *   rows [n_s + i*Lc, n_s + (i+1)*Lc)      = bank chunk retrieved_idx[i],
 *                                            i = 0..n_ret-1 (int4 banks are
 *                                            dequantised on the fly)
 *   then recent[0], ..., recent[n_recent-1], then current,
 * Nk = n_s + n_ret*Lc + sum(recent[].n) + current.n, which must not exceed
 * win_rows nor 2^26 - 1 (one 64-lane wave copies each row and a launch holds
 * fewer than 2^32 lanes): WKV_ERR_SHAPE otherwise. A retrieved id outside
 * [0, M) yields zero rows (no fault).
 *   sink, current  [host] wkv_segment
 *   bank           [host] wkv_bank (device arrays inside)
 *   retrieved_idx  int32 [n_ret] device (e.g. out_idx of wkv_pose_topk)
 *   recent         [host] wkv_segment [n_recent], 0 <= n_recent <= 14
 * ------------------------------------------------------------------------ */
/* [host] Rows of the window wkv_assemble_window writes for these pieces:
 * sink->n + n_ret * Lc + sum(recent[i].n) + current->n (the caller sizes
 * win_k / win_v with it). -1 for a NULL piece, a negative count or more than
 * 14 recent segments (the reason is in wkv_last_error()). */
int64_t wkv_window_rows(const wkv_segment* sink, int32_t n_ret, int32_t Lc,
                        const wkv_segment* recent, int32_t n_recent, const wkv_segment* current);

wkv_status wkv_assemble_window(const wkv_segment* sink, const wkv_bank* bank,
                               const int32_t* retrieved_idx, int32_t n_ret,
                               const wkv_segment* recent, int32_t n_recent,
                               const wkv_segment* current, int32_t H, int32_t D,
                               uint16_t* win_k, uint16_t* win_v,
                               int64_t win_rows, wkv_stream_t stream);

/* ------------------------------------------------------------------------
 * Chunk attention ([WorldAttention]: scaled dot-product attention of the
 * current chunk's Nq queries over Nk visible keys, 1/sqrt(d) scaling,
 * repeated at every denoising step; [WorldKV] Sec. 1 / 5.2: the denoising
 * chunk attends to the assembled window).
 *   O[i,h,:] = sum_j softmax_j(scale * <Q[i,h,:], K[j,h,:]>) V[j,h,:]
 * No mask; query and key head counts are equal. bf16 MFMA products with
 * float32 accumulation and softmax; O is rounded to bf16 (RNE).
 *   q    bf16 [Nq][H][D];  k, v  bf16 [Nk][H][D];  out  bf16 [Nq][H][D]
 *   lse  float [H][Nq] optional (NULL ok): natural-log log-sum-exp of the
 *        scaled scores of every query row
 *   scale <= 0 selects 1/sqrt(D)
 *   ws   workspace for split-key partials; wkv_attention_workspace_bytes()
 *        gives the size for the library's preferred split. With less (or
 *        NULL) the call uses as many splits as fit, down to none.
 * Limits: 1 <= Nq, 1 <= Nk, Nk < 2^31 / H.
 * ------------------------------------------------------------------------ */
size_t wkv_attention_workspace_bytes(int32_t Nq, int32_t Nk, int32_t H,
                                     int32_t D);

wkv_status wkv_chunk_attention(const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, int32_t Nq, int32_t Nk,
                               int32_t H, int32_t D, float scale,
                               uint16_t* out, float* lse, void* ws,
                               size_t ws_bytes, wkv_stream_t stream);

/* ------------------------------------------------------------------------
 * Chunk attention over the window read in place ([WorldAttention] kernel
 * section: the contiguous KV copy before attention is a large share of its
 * latency; [WorldKV] Sec. 4.2 / 5.1: the window is sink | retrieval | recent
 * | denoising). Computes what wkv_assemble_window followed by
 * wkv_chunk_attention computes, without writing the window: the kernel reads
 * each 64-key tile straight from its piece (the sink, bank chunk
 * retrieved_idx[i], a recent segment, or the current chunk).
 *   q, Nq, H, D, scale, out, lse   as for wkv_chunk_attention
 *   sink, bank, retrieved_idx, n_ret, recent, n_recent, current
 *                                  as for wkv_assemble_window; the bank
 *                                  must be WKV_BANK_BF16 (an int4 bank is
 *                                  WKV_ERR_UNSUPPORTED: its rows need the
 *                                  dequantising gather). A retrieved id
 *                                  outside [0, M) reads as zero rows, as in
 *                                  the assembled window.
 *   ws, ws_bytes   device workspace: a table of the window's 64-key tiles
 *                  (64 bytes per tile, rounded up to 256 bytes; required,
 *                  WKV_ERR_WORKSPACE otherwise), then split-key partials.
 *                  wkv_attention_window_workspace_bytes() gives the size
 *                  with the preferred split; with less, fewer splits. The
 *                  call writes the table on its stream, so concurrent calls
 *                  need separate workspaces.
 * Each piece is padded to whole 64-key tiles and its padding is masked, so
 * the result equals the assembled path's up to the order of the fp32
 * additions. Limits: at most 32 pieces (n_ret + n_recent + 2), the padded
 * key count Nk_pad = sum of 64 * ceil(n / 64) over the pieces is >= 1 and
 * Nk_pad * H * D < 2^31.
 * ------------------------------------------------------------------------ */
size_t wkv_attention_window_workspace_bytes(int32_t Nq, int64_t Nk_pad, int32_t H,
                                            int32_t D);

wkv_status wkv_chunk_attention_window(const uint16_t* q, int32_t Nq,
                                      const wkv_segment* sink, const wkv_bank* bank,
                                      const int32_t* retrieved_idx, int32_t n_ret,
                                      const wkv_segment* recent, int32_t n_recent,
                                      const wkv_segment* current, int32_t H, int32_t D,
                                      float scale, uint16_t* out, float* lse, void* ws,
                                      size_t ws_bytes, wkv_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* WKV_H_ */
