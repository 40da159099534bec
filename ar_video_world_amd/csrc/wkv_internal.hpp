// Internal launcher interface between the C ABI layer (api.cpp) and the
// kernel translation units. Not installed; no torch types anywhere.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace wkv {

constexpr int kMaxSegments = 16;  // sink + up to 14 recent + current
constexpr int64_t kMaxWindowRows = (1LL << 26) - 1;  // one 64-lane block per row, < 2^32 lanes

// ---- compression
int compress_score_tile(int B, int T, int H, bool grow);
int compress_mean_slices(int B, int T, int H);  // anchor-token slices of the anchor-mean sums
size_t compress_score_lds_bytes(int B, int F, int T, int H, int D, bool mean, bool q4);
size_t compress_anchor_lds_bytes(int H, int D, bool q4);  // the anchor-mean kernel
// Destination of the compressed rows: bf16 rows (k, v) when k_packed is
// null, else int4 codes (k_packed, v_packed: [B][Lc][H][D/2]) with bf16 group
// scales (k_scale, v_scale: [B][Lc][H][D/32]).
struct CompressDst {
  uint16_t* k;
  uint16_t* v;
  uint8_t* k_packed;
  uint8_t* v_packed;
  uint16_t* k_scale;
  uint16_t* v_scale;
};
// The mean key of each compressed unit (float64 [B][H][D]), when key_mean is
// given: araw [B][H][slices][D] holds the anchor-row sums of the anchor-mean
// score's kernel (slices as for that score; used with the anchor-mean score
// only), ksum [B][runs][H*D] the sums of the summing gather's runs.
struct KeyMeanWs {
  double* key_mean;
  double* araw;
  double* ksum;
};
// Column slices and runs of the summing gather for `rows` K rows per unit,
// and the most runs any keep ratio and score mode give (rows <= F*T): ksum
// holds B * compress_key_runs_max * H*D doubles.
int compress_key_slices(int cpr);
int compress_key_runs(int B, int rows, int cpr);
int compress_key_runs_max(int B, int F, int T, int cpr);
// mean_part [B][H][slices][D] and abar [B][H][D] (float64) are used, and must
// be given, for the anchor-mean score only; abar == nullptr selects the
// position-aligned score.
hipError_t compress_launch(const uint16_t* k, const uint16_t* v, int B, int F, int T,
                           int H, int D, int n_keep, const CompressDst& dst,
                           int32_t* kept_idx, double* scores, bool need_scores,
                           double* mean_part, double* abar, const KeyMeanWs& km, hipStream_t s);

// The compression workspace of callers that cannot allocate: a file-scope
// device array of compress_scratch_bytes() bytes per GPU. compress_scratch()
// gives its address on the current device (resolved on the first call per
// device and kept).
size_t compress_scratch_bytes();
hipError_t compress_scratch(void** ptr);

// ---- query retrieval
int mean_rows_slices(int L);
// part: [B][slices][H*D] float64 workspace; rows may be null (all rows).
hipError_t mean_rows_launch(const uint16_t* x, int B, int L_in, const int32_t* rows, int L,
                            int HD, double* part, double* out, hipStream_t s);
hipError_t query_topk_launch(const double* key_means, int M, const double* query_mean, int HD,
                             int k_eff, int32_t* out_idx, double* scores, hipStream_t s);

// ---- pose top-k
hipError_t pose_topk_launch(const void* poses, int M, const float* last,
                            const float* prev, int n_hist, int k_eff, int32_t* out_idx,
                            double* out_dist, void* out_query, hipStream_t s);

// poses: 32-byte records (x, y, z, qw, qx, qy, qz, pad); query: 7 floats.
hipError_t pose_topk_so3_launch(const void* poses, int M, const float* query, int k_eff,
                                int32_t* out_idx, double* out_dist, hipStream_t s);

// ---- host tier (device side)
constexpr int kTierMaxSlots = 64;
struct TierTable {
  int32_t chunk[kTierMaxSlots];
  int32_t pred[kTierMaxSlots];
  int32_t n_slots;
  int32_t n_pred;
};
hipError_t tier_table_launch(const TierTable& t, int32_t* slot_chunk, int32_t* pred_slot,
                             hipStream_t s);
// Copies of whole chunks: array a (K, V and, for int4, their scales) moves
// bytes[a] from src[a] + id[j]*bytes[a] (device mapping of pinned host
// memory) to dst[a] + slot[j]*bytes[a]; every bytes[a] is a multiple of 4.
struct TierCopy {
  const uint8_t* src[4];
  uint8_t* dst[4];
  size_t bytes[4];
  int32_t id[kTierMaxSlots];
  int32_t slot[kTierMaxSlots];
  int32_t narr;
  int32_t n;
};
hipError_t tier_copy_launch(const TierCopy& c, hipStream_t s);
hipError_t tier_resolve_launch(const int32_t* actual, int n, const int32_t* slot_chunk,
                               int n_slots, const int32_t* pred_slot, int32_t* out_slot,
                               int32_t* out_miss, hipStream_t s);

// ---- window assembly
struct AssemblePlan {
  const uint16_t* seg_k[kMaxSegments];
  const uint16_t* seg_v[kMaxSegments];
  int64_t seg_start[kMaxSegments + 1];
  int nseg;
  const void* bank_k;
  const void* bank_v;
  const uint16_t* bank_ks;
  const uint16_t* bank_vs;
  const int32_t* idx;
  int M, Lc, n_ret, int4;
  int64_t ret_off;
  int64_t Nk;
  int cpr;  // 16-byte chunks per bf16 output row (H*D/8)
};
hipError_t assemble_launch(const AssemblePlan& p, uint16_t* win_k, uint16_t* win_v,
                           hipStream_t s);

// ---- chunk attention
struct AttnPlan {
  int splits;       // key splits (1 = write O directly)
  int keys_per_split;
};
AttnPlan attention_plan(int Nq, int Nk, int H, int D, int num_cus);
size_t attention_ws_bytes(const AttnPlan& p, int Nq, int H, int D);
hipError_t attention_launch(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            int Nq, int Nk, int H, int D, float scale, uint16_t* out,
                            float* lse, const AttnPlan& plan, void* ws, hipStream_t s);

// The window read in place: its pieces (sink, retrieved bank chunks, recent
// segments, current) in window order, each padded to whole 64-key tiles.
// Piece p covers tiles [tile0[p], tile0[p+1]) and n[p] rows; a piece with
// slot[p] >= 0 is bank chunk idx[slot[p]] (k[p], v[p] then hold the bank
// base, and an id outside [0, M) reads as zero rows).
constexpr int kMaxWinPieces = 32;
struct WinPieces {
  const uint16_t* k[kMaxWinPieces];
  const uint16_t* v[kMaxWinPieces];
  int32_t n[kMaxWinPieces];
  int32_t slot[kMaxWinPieces];
  int32_t tile0[kMaxWinPieces + 1];
  const int32_t* idx;
  int32_t M, Lc, npieces;
};
// ws holds the per-tile table (attention_window_table_bytes) and then the
// split partials (attention_ws_bytes).
size_t attention_window_table_bytes(int ntiles);
hipError_t attention_window_launch(const uint16_t* q, const WinPieces& w, int Nq, int H, int D,
                                   float scale, uint16_t* out, float* lse, const AttnPlan& plan,
                                   void* ws, hipStream_t s);

}  // namespace wkv
