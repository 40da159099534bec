// C ABI of libwkv: argument validation on the host (before anything is
// enqueued), workspace sizing and launch planning. The operations themselves
// are defined in include/wkv.h and run in the kernel translation units.
#include "../../include/wkv.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

#include "wkv_internal.hpp"

static_assert(sizeof(wkv_pose) == 16, "wkv_pose is read as one float4 per pose");
static_assert(sizeof(wkv_pose_q) == 32, "wkv_pose_q is read as two float4 per pose");

namespace {

thread_local char g_err[512] = "";

wkv_status fail(wkv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

wkv_status hip_fail(hipError_t e, const char* what) {
  return fail(WKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

wkv_status check_hd(int32_t H, int32_t D) {
  if (D != 64 && D != 128) return fail(WKV_ERR_UNSUPPORTED, "head dim D=%d (supported: 64, 128)", D);
  if (H < 1 || (int64_t)H * D > 8192) return fail(WKV_ERR_SHAPE, "heads H=%d out of range (1..%d)", H, 8192 / D);
  return WKV_OK;
}

// An attribute of the current device, cached per device id.
template <hipDeviceAttribute_t ATTR>
int device_attr(int fallback) {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fallback;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, ATTR, dev) != hipSuccess || n <= 0) n = fallback;
    cache[dev] = n;
  }
  return cache[dev];
}

int num_cus() { return device_attr<hipDeviceAttributeMultiprocessorCount>(256); }
int max_lds_per_block() { return device_attr<hipDeviceAttributeMaxSharedMemoryPerBlock>(65536); }

int64_t keep_count(int32_t F, int32_t T, float r) {
  const int64_t N = (int64_t)(F - 1) * T;
  const double x = (double)r * (double)N;
  int64_t n = (int64_t)x;
  if (x - (double)n >= 0.5) ++n;
  if (n < 0) n = 0;
  if (n > N) n = N;
  return n;
}

// Largest grid y / z extent: the batch and row-slice counts ride on those axes.
constexpr int kMaxGridYZ = 65535;

constexpr size_t kWsAlign = 256;
size_t round_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Workspace layout, float64, each part 256-byte aligned:
//   [scores B*N]                        when the caller gives no scores output
//   [anchor-mean partials B*H*slices*D] [abar B*H*D]   anchor-mean score
//   [anchor-row sums B*H*slices*D]      mean key with the anchor-mean score
//   [kept-row run sums B*runs*H*D]      mean key
struct CompressWsLayout {
  size_t scores, part, abar, araw, ksum, total;
};
CompressWsLayout compress_ws_layout(int32_t B, int32_t F, int32_t T, int32_t H, int32_t D,
                                    bool mean, bool scores_in_ws, bool key_mean) {
  CompressWsLayout L{};
  const size_t slices = (size_t)B * H * wkv::compress_mean_slices(B, T, H) * D * sizeof(double);
  L.scores = 0;
  L.part = scores_in_ws ? round_up((size_t)B * (size_t)(F - 1) * (size_t)T * sizeof(double)) : 0;
  L.abar = L.part + (mean ? round_up(slices) : 0);
  L.araw = L.abar + (mean ? round_up((size_t)B * H * D * sizeof(double)) : 0);
  L.ksum = L.araw + (key_mean && mean ? round_up(slices) : 0);
  L.total = L.ksum + (key_mean ? round_up((size_t)B * wkv::compress_key_runs_max(B, F, T, H * D / 8) *
                                          (size_t)H * D * sizeof(double))
                               : 0);
  return L;
}

// Validation and launch shared by the bf16 and int4 compression entry points
// (their output pointers are checked by the callers).
wkv_status compress_common(const char* fn, const uint16_t* k, const uint16_t* v, int32_t B,
                           int32_t F, int32_t T, int32_t H, int32_t D, float r,
                           int32_t score_mode, const wkv::CompressDst& dst, int32_t* kept_idx,
                           double* scores, double* key_mean, void* ws, size_t ws_bytes,
                           wkv_stream_t stream) {
  if (!k || !v || !kept_idx)
    return fail(WKV_ERR_NULL, "%s: k, v and kept_idx are required", fn);
  if (wkv_status st = check_hd(H, D)) return st;
  if (B < 1 || B > kMaxGridYZ || F < 2 || F > 4 || T < 1)
    return fail(WKV_ERR_SHAPE, "%s: need 1<=B<=%d, 2<=F<=4, T>=1 (B=%d F=%d T=%d)", fn,
                kMaxGridYZ, B, F, T);
  if ((int64_t)(F - 1) * T > 8192)
    return fail(WKV_ERR_SHAPE, "%s: (F-1)*T=%lld exceeds 8192", fn, (long long)(F - 1) * T);
  if ((int64_t)B * F * T * H * D >= ((int64_t)1 << 40))
    return fail(WKV_ERR_SHAPE, "%s: batch too large", fn);
  if (!(r >= 0.0f && r <= 1.0f)) return fail(WKV_ERR_RATIO, "%s: r=%g not in [0,1]", fn, (double)r);
  if (score_mode != WKV_SCORE_POSITION && score_mode != WKV_SCORE_ANCHOR_MEAN)
    return fail(WKV_ERR_UNSUPPORTED, "%s: score_mode=%d (supported: 0, 1)", fn, score_mode);
  if (!aligned16(k) || !aligned16(v) || !aligned16(kept_idx) || (scores && !aligned16(scores)) ||
      (key_mean && !aligned16(key_mean)) || (ws && !aligned16(ws)))
    return fail(WKV_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
  const int n_keep = (int)keep_count(F, T, r);
  const int N = (F - 1) * T;
  const bool need_scores = scores != nullptr;
  const bool score = need_scores || (n_keep > 0 && n_keep < N);
  const bool mean = score_mode == WKV_SCORE_ANCHOR_MEAN && score;
  const CompressWsLayout L =
      compress_ws_layout(B, F, T, H, D, mean, score && !scores, key_mean != nullptr);
  if (L.total > 0 && (!ws || ws_bytes < L.total))
    return fail(WKV_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn,
                ws ? ws_bytes : (size_t)0, L.total);
  if (score && wkv::compress_score_lds_bytes(B, F, T, H, D, mean, dst.k_packed != nullptr) >
                   (size_t)max_lds_per_block())
    return fail(WKV_ERR_SHAPE, "%s: H*D too large for the score kernel's LDS", fn);
  if (mean &&
      wkv::compress_anchor_lds_bytes(H, D, dst.k_packed != nullptr) > (size_t)max_lds_per_block())
    return fail(WKV_ERR_SHAPE, "%s: H*D too large for the anchor kernel's LDS", fn);
  char* wsb = static_cast<char*>(ws);
  double* sbuf = scores ? scores : (score ? reinterpret_cast<double*>(wsb + L.scores) : nullptr);
  double* part = mean ? reinterpret_cast<double*>(wsb + L.part) : nullptr;
  double* abar = mean ? reinterpret_cast<double*>(wsb + L.abar) : nullptr;
  const wkv::KeyMeanWs km{key_mean,
                          key_mean && mean ? reinterpret_cast<double*>(wsb + L.araw) : nullptr,
                          key_mean ? reinterpret_cast<double*>(wsb + L.ksum) : nullptr};
  hipError_t e = wkv::compress_launch(k, v, B, F, T, H, D, n_keep, dst, kept_idx, sbuf,
                                      need_scores, part, abar, km, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return WKV_OK;
}

}  // namespace

extern "C" {

int32_t wkv_abi_version(void) { return WKV_ABI_VERSION; }

const char* wkv_last_error(void) { return g_err; }

int32_t wkv_keep_count(int32_t F, int32_t T, float r) {
  if (F < 2 || T < 1 || !(r >= 0.0f && r <= 1.0f)) return -1;
  if ((int64_t)(F - 1) * T > (int64_t)INT32_MAX) return -1;
  return (int32_t)keep_count(F, T, r);
}

int32_t wkv_compress_score_tile(int32_t B, int32_t T, int32_t H, int32_t score_mode,
                                int32_t int4) {
  if (B < 1 || T < 1 || H < 1) return -1;
  if (score_mode != WKV_SCORE_POSITION && score_mode != WKV_SCORE_ANCHOR_MEAN) return -1;
  return wkv::compress_score_tile(B, T, H, int4 != 0 || score_mode == WKV_SCORE_ANCHOR_MEAN);
}

size_t wkv_compress_workspace_bytes(int32_t B, int32_t F, int32_t T, int32_t H, int32_t D,
                                    int32_t score_mode, int32_t key_mean) {
  if (B < 1 || F < 2 || T < 1 || H < 1 || D < 1) return 0;
  if (score_mode != WKV_SCORE_POSITION && score_mode != WKV_SCORE_ANCHOR_MEAN) return 0;
  return compress_ws_layout(B, F, T, H, D, score_mode == WKV_SCORE_ANCHOR_MEAN, true,
                            key_mean != 0)
      .total;
}

wkv_status wkv_compress_chunk(const uint16_t* k, const uint16_t* v, int32_t B, int32_t F,
                              int32_t T, int32_t H, int32_t D, float r, int32_t score_mode,
                              uint16_t* k_out, uint16_t* v_out, int32_t* kept_idx, double* scores,
                              double* key_mean, void* ws, size_t ws_bytes, wkv_stream_t stream) {
  if (!k_out || !v_out)
    return fail(WKV_ERR_NULL, "wkv_compress_chunk: k, v, k_out, v_out and kept_idx are required");
  if (!aligned16(k_out) || !aligned16(v_out))
    return fail(WKV_ERR_ALIGN, "wkv_compress_chunk: device pointers must be 16-byte aligned");
  return compress_common("wkv_compress_chunk", k, v, B, F, T, H, D, r, score_mode,
                         wkv::CompressDst{k_out, v_out, nullptr, nullptr, nullptr, nullptr},
                         kept_idx, scores, key_mean, ws, ws_bytes, stream);
}

wkv_status wkv_compress_chunk_noalloc(const uint16_t* k, const uint16_t* v, int32_t B,
                                      int32_t F, int32_t T, int32_t H, int32_t D, float r,
                                      int32_t score_mode, uint16_t* k_out, uint16_t* v_out,
                                      int32_t* kept_idx, double* scores, wkv_stream_t stream) {
  static const char* fn = "wkv_compress_chunk_noalloc";
  if (!k_out || !v_out)
    return fail(WKV_ERR_NULL, "%s: k, v, k_out, v_out and kept_idx are required", fn);
  if (!aligned16(k_out) || !aligned16(v_out))
    return fail(WKV_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
  // Arguments the shared checks refuse go straight to them (with no
  // workspace), so they are reported exactly as by wkv_compress_chunk.
  if (!k || !v || !kept_idx || (D != 64 && D != 128) || H < 1 || (int64_t)H * D > 8192 ||
      B < 1 || B > kMaxGridYZ || F < 2 || F > 4 || T < 1 || (int64_t)(F - 1) * T > 8192 ||
      !(r >= 0.0f && r <= 1.0f) ||
      (score_mode != WKV_SCORE_POSITION && score_mode != WKV_SCORE_ANCHOR_MEAN))
    return compress_common(fn, k, v, B, F, T, H, D, r, score_mode,
                           wkv::CompressDst{k_out, v_out, nullptr, nullptr, nullptr, nullptr},
                           kept_idx, scores, nullptr, nullptr, 0, stream);
  const int n_keep = (int)keep_count(F, T, r);
  const int N = (F - 1) * T;
  const bool score = scores != nullptr || (n_keep > 0 && n_keep < N);
  const bool mean = score_mode == WKV_SCORE_ANCHOR_MEAN && score;
  const size_t need = compress_ws_layout(B, F, T, H, D, mean, score && !scores, false).total;
  const size_t cap = wkv::compress_scratch_bytes();
  if (need > cap)
    return fail(WKV_ERR_WORKSPACE,
                "%s: this call needs %zu bytes of workspace, more than the library's static "
                "scratch of %zu bytes (use wkv_compress_chunk with a workspace)", fn, need, cap);
  void* ws = nullptr;
  if (need > 0) {
    hipError_t e = wkv::compress_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "wkv_compress_chunk_noalloc: scratch address");
  }
  return compress_common(fn, k, v, B, F, T, H, D, r, score_mode,
                         wkv::CompressDst{k_out, v_out, nullptr, nullptr, nullptr, nullptr},
                         kept_idx, scores, nullptr, ws, need > 0 ? cap : 0, stream);
}

wkv_status wkv_compress_chunk_int4(const uint16_t* k, const uint16_t* v, int32_t B, int32_t F,
                                   int32_t T, int32_t H, int32_t D, float r, int32_t score_mode,
                                   uint8_t* k_packed, uint8_t* v_packed, uint16_t* k_scale,
                                   uint16_t* v_scale, int32_t* kept_idx, double* scores,
                                   double* key_mean, void* ws, size_t ws_bytes,
                                   wkv_stream_t stream) {
  if (!k_packed || !v_packed || !k_scale || !v_scale)
    return fail(WKV_ERR_NULL,
                "wkv_compress_chunk_int4: k, v, k_packed, v_packed, k_scale, v_scale and kept_idx "
                "are required");
  if (!aligned16(k_packed) || !aligned16(v_packed) || !aligned16(k_scale) || !aligned16(v_scale))
    return fail(WKV_ERR_ALIGN, "wkv_compress_chunk_int4: device pointers must be 16-byte aligned");
  return compress_common("wkv_compress_chunk_int4", k, v, B, F, T, H, D, r, score_mode,
                         wkv::CompressDst{nullptr, nullptr, k_packed, v_packed, k_scale, v_scale},
                         kept_idx, scores, key_mean, ws, ws_bytes, stream);
}

size_t wkv_mean_rows_workspace_bytes(int32_t B, int32_t L, int32_t H, int32_t D) {
  if (B < 1 || L < 1 || H < 1 || D < 1) return 0;
  return (size_t)B * wkv::mean_rows_slices(L) * (size_t)H * D * sizeof(double);
}

wkv_status wkv_mean_rows(const uint16_t* x, int32_t B, int32_t L_in, const int32_t* rows,
                         int32_t L, int32_t H, int32_t D, double* out, void* ws,
                         size_t ws_bytes, wkv_stream_t stream) {
  if (!x || !out || !ws) return fail(WKV_ERR_NULL, "wkv_mean_rows: x, out and ws are required");
  if (wkv_status st = check_hd(H, D)) return st;
  if (B < 1 || B > kMaxGridYZ || L < 1 || L_in < 1 || (!rows && L > L_in) ||
      wkv::mean_rows_slices(L) > kMaxGridYZ)
    return fail(WKV_ERR_SHAPE, "wkv_mean_rows: B=%d L_in=%d L=%d (B <= %d, L <= %d)", B, L_in, L,
                kMaxGridYZ, kMaxGridYZ * 64);
  if ((int64_t)B * L_in * H * D >= ((int64_t)1 << 40) || (int64_t)B * L >= ((int64_t)1 << 31))
    return fail(WKV_ERR_SHAPE, "wkv_mean_rows: input too large");
  if (!aligned16(x) || !aligned16(out) || !aligned16(ws) || (rows && !aligned16(rows)))
    return fail(WKV_ERR_ALIGN, "wkv_mean_rows: device pointers must be 16-byte aligned");
  const size_t need = wkv_mean_rows_workspace_bytes(B, L, H, D);
  if (ws_bytes < need)
    return fail(WKV_ERR_WORKSPACE, "wkv_mean_rows: workspace %zu bytes < %zu needed", ws_bytes, need);
  hipError_t e = wkv::mean_rows_launch(x, B, L_in, rows, L, H * D, static_cast<double*>(ws), out,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "wkv_mean_rows launch");
  return WKV_OK;
}

wkv_status wkv_query_topk(const double* key_means, int32_t M, const double* query_mean,
                          int32_t H, int32_t D, int32_t k, int32_t* out_idx, double* scores,
                          wkv_stream_t stream) {
  if (!key_means || !query_mean || !out_idx || !scores)
    return fail(WKV_ERR_NULL, "wkv_query_topk: key_means, query_mean, out_idx and scores are required");
  if (wkv_status st = check_hd(H, D)) return st;
  if (M < 1 || M > 8192) return fail(WKV_ERR_SHAPE, "wkv_query_topk: M=%d (1..8192)", M);
  if (k < 1) return fail(WKV_ERR_K, "wkv_query_topk: k=%d", k);
  if (!aligned16(key_means) || !aligned16(query_mean) || !aligned16(out_idx) || !aligned16(scores))
    return fail(WKV_ERR_ALIGN, "wkv_query_topk: device pointers must be 16-byte aligned");
  const int k_eff = k < M ? k : M;
  hipError_t e = wkv::query_topk_launch(key_means, M, query_mean, H * D, k_eff, out_idx, scores,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "wkv_query_topk launch");
  return WKV_OK;
}

wkv_status wkv_pose_topk(const wkv_pose* bank_poses, int32_t M, const wkv_pose* query_hist,
                         int32_t n_hist, int32_t k, int32_t* out_idx, double* out_dist,
                         wkv_pose* out_query, wkv_stream_t stream) {
  if (!bank_poses || !query_hist || !out_idx)
    return fail(WKV_ERR_NULL, "wkv_pose_topk: bank_poses, query_hist and out_idx are required");
  if (M < 1 || M > 8192) return fail(WKV_ERR_SHAPE, "wkv_pose_topk: M=%d not in [1, 8192]", M);
  if (k < 1) return fail(WKV_ERR_K, "wkv_pose_topk: k=%d < 1", k);
  if (n_hist != 1 && n_hist != 2) return fail(WKV_ERR_K, "wkv_pose_topk: n_hist=%d (must be 1 or 2)", n_hist);
  if (!aligned16(bank_poses) || !aligned16(out_idx) || (out_dist && !aligned16(out_dist)) ||
      (out_query && !aligned16(out_query)))
    return fail(WKV_ERR_ALIGN, "wkv_pose_topk: device pointers must be 16-byte aligned");
  const float* last = &query_hist[n_hist - 1].x;
  const float* prev = n_hist == 2 ? &query_hist[0].x : nullptr;
  const int k_eff = k < M ? k : M;
  hipError_t e = wkv::pose_topk_launch(bank_poses, M, last, prev, n_hist, k_eff, out_idx,
                                       out_dist, out_query, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "wkv_pose_topk launch");
  return WKV_OK;
}

wkv_status wkv_pose_topk_so3(const wkv_pose_q* bank_poses, int32_t M, const wkv_pose_q* query,
                             int32_t k, int32_t* out_idx, double* out_dist,
                             wkv_stream_t stream) {
  if (!bank_poses || !query || !out_idx)
    return fail(WKV_ERR_NULL, "wkv_pose_topk_so3: bank_poses, query and out_idx are required");
  if (M < 1 || M > 8192) return fail(WKV_ERR_SHAPE, "wkv_pose_topk_so3: M=%d not in [1, 8192]", M);
  if (k < 1) return fail(WKV_ERR_K, "wkv_pose_topk_so3: k=%d < 1", k);
  if (!aligned16(bank_poses) || !aligned16(out_idx) || (out_dist && !aligned16(out_dist)))
    return fail(WKV_ERR_ALIGN, "wkv_pose_topk_so3: device pointers must be 16-byte aligned");
  const int k_eff = k < M ? k : M;
  hipError_t e = wkv::pose_topk_so3_launch(bank_poses, M, &query->x, k_eff, out_idx, out_dist,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "wkv_pose_topk_so3 launch");
  return WKV_OK;
}

wkv_status wkv_tier_init(wkv_tier* t, int32_t n_slots) {
  if (!t) return fail(WKV_ERR_NULL, "wkv_tier_init: t is NULL");
  if (n_slots < 1 || n_slots > WKV_TIER_MAX_SLOTS)
    return fail(WKV_ERR_SHAPE, "wkv_tier_init: n_slots=%d (1..%d)", n_slots, WKV_TIER_MAX_SLOTS);
  std::memset(t, 0, sizeof(*t));
  t->n_slots = n_slots;
  for (int i = 0; i < WKV_TIER_MAX_SLOTS; ++i) t->chunk[i] = -1;
  return WKV_OK;
}

wkv_status wkv_tier_plan(wkv_tier* t, const int32_t* ids, int32_t n, const int32_t* keep_ids,
                         int32_t n_keep, int32_t* slot_of, int32_t* copy_ids,
                         int32_t* copy_slots, int32_t* n_copies) {
  if (!t || !ids || !slot_of || !copy_ids || !copy_slots || !n_copies || (n_keep > 0 && !keep_ids))
    return fail(WKV_ERR_NULL, "wkv_tier_plan: null argument");
  if (n_keep < 0) return fail(WKV_ERR_SHAPE, "wkv_tier_plan: n_keep=%d", n_keep);
  if (t->n_slots < 1 || t->n_slots > WKV_TIER_MAX_SLOTS)
    return fail(WKV_ERR_SHAPE, "wkv_tier_plan: table not initialised (n_slots=%d)", t->n_slots);
  if (n < 1 || n > t->n_slots)
    return fail(WKV_ERR_SHAPE, "wkv_tier_plan: n=%d (1..n_slots=%d)", n, t->n_slots);
  for (int i = 0; i < n; ++i) {
    if (ids[i] < 0) return fail(WKV_ERR_SHAPE, "wkv_tier_plan: ids[%d]=%d < 0", i, ids[i]);
    for (int j = 0; j < i; ++j)
      if (ids[j] == ids[i]) return fail(WKV_ERR_SHAPE, "wkv_tier_plan: id %d repeated", ids[i]);
  }
  // Work on copies: a request that does not fit leaves the table and every
  // output unchanged.
  wkv_tier nt = *t;
  int32_t so[WKV_TIER_MAX_SLOTS], ci[WKV_TIER_MAX_SLOTS], cs[WKV_TIER_MAX_SLOTS];
  const uint64_t stamp = ++nt.clock;
  bool taken[WKV_TIER_MAX_SLOTS] = {};
  for (int s = 0; s < nt.n_slots; ++s)
    for (int j = 0; j < n_keep && !taken[s]; ++j)
      taken[s] = nt.chunk[s] >= 0 && nt.chunk[s] == keep_ids[j];
  for (int i = 0; i < n; ++i) {
    so[i] = -1;
    for (int s = 0; s < nt.n_slots; ++s)
      if (nt.chunk[s] == ids[i]) {
        so[i] = s;
        taken[s] = true;
        nt.last_use[s] = stamp;
        break;
      }
  }
  int nc = 0;
  for (int i = 0; i < n; ++i) {
    if (so[i] >= 0) continue;
    int v = -1;
    for (int s = 0; s < nt.n_slots; ++s)
      if (!taken[s] && (v < 0 || nt.last_use[s] < nt.last_use[v])) v = s;  // ties: lower slot
    if (v < 0)
      return fail(WKV_ERR_SHAPE, "wkv_tier_plan: %d slots cannot hold the request beside the kept chunks",
                  nt.n_slots);
    nt.chunk[v] = ids[i];
    nt.last_use[v] = stamp;
    taken[v] = true;
    so[i] = v;
    ci[nc] = ids[i];
    cs[nc] = v;
    ++nc;
  }
  *t = nt;
  std::copy(so, so + n, slot_of);
  std::copy(ci, ci + nc, copy_ids);
  std::copy(cs, cs + nc, copy_slots);
  *n_copies = nc;
  return WKV_OK;
}

wkv_status wkv_tier_prefetch(wkv_tier* t, const int32_t* ids, int32_t n, const int32_t* keep_ids,
                             int32_t n_keep, const wkv_bank* host_bank, const wkv_bank* staging,
                             int32_t H, int32_t D, int32_t copy_mode, int32_t* dev_slot_chunk,
                             int32_t* dev_pred_slot, int32_t* n_copies, wkv_stream_t stream) {
  if (!t || !ids || !host_bank || !staging || !dev_slot_chunk || !dev_pred_slot || !n_copies)
    return fail(WKV_ERR_NULL, "wkv_tier_prefetch: null argument");
  if (wkv_status st = check_hd(H, D)) return st;
  const bool q4 = host_bank->dtype == WKV_BANK_INT4_G32;
  if ((host_bank->dtype != WKV_BANK_BF16 && !q4) || staging->dtype != host_bank->dtype ||
      staging->Lc != host_bank->Lc || host_bank->Lc < 1 || host_bank->M < 1 ||
      staging->M != t->n_slots)
    return fail(WKV_ERR_SHAPE, "wkv_tier_prefetch: host bank and staging bank do not match the table");
  if (!host_bank->k || !host_bank->v || !staging->k || !staging->v ||
      (q4 && (!host_bank->k_scale || !host_bank->v_scale || !staging->k_scale || !staging->v_scale)))
    return fail(WKV_ERR_NULL, "wkv_tier_prefetch: bank pointers are required");
  for (int i = 0; i < n; ++i)
    if (ids[i] >= host_bank->M)
      return fail(WKV_ERR_SHAPE, "wkv_tier_prefetch: ids[%d]=%d >= M=%d", i, ids[i], host_bank->M);
  if (!aligned16(dev_slot_chunk) || !aligned16(dev_pred_slot))
    return fail(WKV_ERR_ALIGN, "wkv_tier_prefetch: device pointers must be 16-byte aligned");
  if (copy_mode != WKV_TIER_COPY_KERNEL && copy_mode != WKV_TIER_COPY_ENGINE)
    return fail(WKV_ERR_UNSUPPORTED, "wkv_tier_prefetch: copy_mode=%d", copy_mode);
  // Plan on a copy of the table: nothing changes unless every enqueue succeeds.
  wkv_tier nt = *t;
  int32_t slot_of[WKV_TIER_MAX_SLOTS], cid[WKV_TIER_MAX_SLOTS], cslot[WKV_TIER_MAX_SLOTS], nc = 0;
  if (wkv_status st = wkv_tier_plan(&nt, ids, n, keep_ids, n_keep, slot_of, cid, cslot, &nc))
    return st;
  // A copy that was enqueued may already be overwriting its slot: if a later
  // step fails, those slots are marked empty in the caller's table so that no
  // later request trusts their contents.
  auto abandon = [&](hipError_t e, const char* what) {
    for (int i = 0; i < nc; ++i) {
      t->chunk[cslot[i]] = -1;
      t->last_use[cslot[i]] = 0;
    }
    return hip_fail(e, what);
  };
  const size_t rows = (size_t)host_bank->Lc * H * D;
  const size_t kv_bytes = q4 ? rows / 2 : rows * 2;
  const size_t sc_bytes = q4 ? rows / 32 * 2 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nc > 0 && copy_mode == WKV_TIER_COPY_ENGINE) {
    for (int i = 0; i < nc; ++i) {
      const size_t src = (size_t)cid[i], dst = (size_t)cslot[i];
      const void* from[4] = {host_bank->k, host_bank->v, host_bank->k_scale, host_bank->v_scale};
      const void* to[4] = {staging->k, staging->v, staging->k_scale, staging->v_scale};
      for (int c = 0; c < (q4 ? 4 : 2); ++c) {
        const size_t bytes = c < 2 ? kv_bytes : sc_bytes;
        hipError_t e = hipMemcpyAsync(static_cast<char*>(const_cast<void*>(to[c])) + dst * bytes,
                                      static_cast<const char*>(from[c]) + src * bytes, bytes,
                                      hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return abandon(e, "wkv_tier_prefetch copy");
      }
    }
  } else if (nc > 0) {
    // The copies read the host bank through its device mapping (pinned
    // memory allocated with hipHostMalloc is mapped); anything else is
    // refused here rather than touched by the kernel.
    const void* hsrc[4] = {host_bank->k, host_bank->v, host_bank->k_scale, host_bank->v_scale};
    void* ddst[4] = {const_cast<void*>(staging->k), const_cast<void*>(staging->v),
                     const_cast<uint16_t*>(staging->k_scale), const_cast<uint16_t*>(staging->v_scale)};
    wkv::TierCopy c;
    std::memset(&c, 0, sizeof(c));
    c.narr = q4 ? 4 : 2;
    c.n = nc;
    for (int a = 0; a < c.narr; ++a) {
      void* dp = nullptr;
      hipError_t e = hipHostGetDevicePointer(&dp, const_cast<void*>(hsrc[a]), 0);
      if (e != hipSuccess || !dp)
        return fail(WKV_ERR_UNSUPPORTED,
                    "wkv_tier_prefetch: the host bank must be pinned, device-mapped host memory (%s)",
                    hipGetErrorString(e));
      c.src[a] = static_cast<const uint8_t*>(dp);
      c.dst[a] = static_cast<uint8_t*>(ddst[a]);
      c.bytes[a] = a < 2 ? kv_bytes : sc_bytes;
    }
    for (int i = 0; i < nc; ++i) {
      c.id[i] = cid[i];
      c.slot[i] = cslot[i];
    }
    hipError_t e = wkv::tier_copy_launch(c, s);
    if (e != hipSuccess) return abandon(e, "wkv_tier_prefetch copy");
  }
  wkv::TierTable tt;
  std::memset(&tt, 0, sizeof(tt));
  tt.n_slots = nt.n_slots;
  tt.n_pred = n;
  for (int i = 0; i < nt.n_slots; ++i) tt.chunk[i] = nt.chunk[i];
  for (int i = 0; i < n; ++i) tt.pred[i] = slot_of[i];
  hipError_t e = wkv::tier_table_launch(tt, dev_slot_chunk, dev_pred_slot, s);
  if (e != hipSuccess) return abandon(e, "wkv_tier_prefetch table");
  *t = nt;
  *n_copies = nc;
  return WKV_OK;
}

wkv_status wkv_tier_resolve(const int32_t* actual_idx, int32_t n, const int32_t* slot_chunk,
                            int32_t n_slots, const int32_t* pred_slot, int32_t* out_slot,
                            int32_t* out_miss, wkv_stream_t stream) {
  if (!actual_idx || !slot_chunk || !pred_slot || !out_slot)
    return fail(WKV_ERR_NULL, "wkv_tier_resolve: null argument");
  if (n < 1 || n > WKV_TIER_MAX_SLOTS || n_slots < 1 || n_slots > WKV_TIER_MAX_SLOTS)
    return fail(WKV_ERR_SHAPE, "wkv_tier_resolve: n=%d n_slots=%d (1..%d)", n, n_slots,
                WKV_TIER_MAX_SLOTS);
  if (!aligned16(actual_idx) || !aligned16(slot_chunk) || !aligned16(pred_slot) ||
      !aligned16(out_slot) || (out_miss && !aligned16(out_miss)))
    return fail(WKV_ERR_ALIGN, "wkv_tier_resolve: device pointers must be 16-byte aligned");
  hipError_t e = wkv::tier_resolve_launch(actual_idx, n, slot_chunk, n_slots, pred_slot, out_slot,
                                          out_miss, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "wkv_tier_resolve launch");
  return WKV_OK;
}

int64_t wkv_window_rows(const wkv_segment* sink, int32_t n_ret, int32_t Lc,
                        const wkv_segment* recent, int32_t n_recent, const wkv_segment* current) {
  if (!sink || !current || (n_recent > 0 && !recent)) {
    fail(WKV_ERR_NULL, "wkv_window_rows: sink, current (and recent when n_recent > 0) are required");
    return -1;
  }
  if (n_ret < 0 || Lc < 0 || n_recent < 0 || n_recent > wkv::kMaxSegments - 2) {
    fail(WKV_ERR_SHAPE, "wkv_window_rows: n_ret=%d Lc=%d n_recent=%d (0..%d)", n_ret, Lc,
         n_recent, wkv::kMaxSegments - 2);
    return -1;
  }
  int64_t rows = (int64_t)n_ret * Lc;
  const wkv_segment* ends[2] = {sink, current};
  for (int i = 0; i < 2 + n_recent; ++i) {
    const wkv_segment* s = i < 2 ? ends[i] : &recent[i - 2];
    if (s->n < 0) {
      fail(WKV_ERR_SHAPE, "wkv_window_rows: a segment has n=%d", s->n);
      return -1;
    }
    rows += s->n;
  }
  return rows;
}

wkv_status wkv_assemble_window(const wkv_segment* sink, const wkv_bank* bank,
                               const int32_t* retrieved_idx, int32_t n_ret,
                               const wkv_segment* recent, int32_t n_recent,
                               const wkv_segment* current, int32_t H, int32_t D,
                               uint16_t* win_k, uint16_t* win_v, int64_t win_rows,
                               wkv_stream_t stream) {
  if (!sink || !current || !win_k || !win_v)
    return fail(WKV_ERR_NULL, "wkv_assemble_window: sink, current, win_k and win_v are required");
  if (wkv_status st = check_hd(H, D)) return st;
  if (n_ret < 0 || n_recent < 0 || n_recent > wkv::kMaxSegments - 2)
    return fail(WKV_ERR_SHAPE, "wkv_assemble_window: n_ret=%d n_recent=%d (0..%d)", n_ret, n_recent,
                wkv::kMaxSegments - 2);
  if (n_ret > 0 && (!bank || !retrieved_idx))
    return fail(WKV_ERR_NULL, "wkv_assemble_window: n_ret>0 needs bank and retrieved_idx");
  if (n_recent > 0 && !recent) return fail(WKV_ERR_NULL, "wkv_assemble_window: recent is NULL");
  if (!aligned16(win_k) || !aligned16(win_v) || (retrieved_idx && !aligned16(retrieved_idx)))
    return fail(WKV_ERR_ALIGN, "wkv_assemble_window: device pointers must be 16-byte aligned");

  wkv::AssemblePlan p;
  std::memset(&p, 0, sizeof(p));
  // Segments: sink, recent..., current, in window order.
  const wkv_segment* segs[wkv::kMaxSegments];
  int ns = 0;
  segs[ns++] = sink;
  for (int i = 0; i < n_recent; ++i) segs[ns++] = &recent[i];
  segs[ns++] = current;
  for (int i = 0; i < ns; ++i) {
    const wkv_segment* s = segs[i];
    if (s->n < 0) return fail(WKV_ERR_SHAPE, "wkv_assemble_window: segment %d has n=%d", i, s->n);
    if (s->n > 0 && (!s->k || !s->v))
      return fail(WKV_ERR_NULL, "wkv_assemble_window: segment %d has n=%d but NULL k/v", i, s->n);
    if (!aligned16(s->k) || !aligned16(s->v))
      return fail(WKV_ERR_ALIGN, "wkv_assemble_window: segment %d pointers must be 16-byte aligned", i);
  }
  int Lc = 0, M = 0, int4 = 0;
  if (n_ret > 0) {
    if (bank->dtype != WKV_BANK_BF16 && bank->dtype != WKV_BANK_INT4_G32)
      return fail(WKV_ERR_UNSUPPORTED, "wkv_assemble_window: bank dtype %d", bank->dtype);
    if (bank->M < 1 || bank->Lc < 1)
      return fail(WKV_ERR_SHAPE, "wkv_assemble_window: bank M=%d Lc=%d", bank->M, bank->Lc);
    if (!bank->k || !bank->v) return fail(WKV_ERR_NULL, "wkv_assemble_window: bank k/v NULL");
    int4 = bank->dtype == WKV_BANK_INT4_G32;
    if (int4 && (!bank->k_scale || !bank->v_scale))
      return fail(WKV_ERR_NULL, "wkv_assemble_window: int4 bank needs k_scale and v_scale");
    if (!aligned16(bank->k) || !aligned16(bank->v) ||
        (int4 && (!aligned16(bank->k_scale) || !aligned16(bank->v_scale))))
      return fail(WKV_ERR_ALIGN, "wkv_assemble_window: bank pointers must be 16-byte aligned");
    Lc = bank->Lc;
    M = bank->M;
  }
  int64_t row = 0;
  p.seg_start[0] = 0;
  p.seg_k[0] = sink->k;
  p.seg_v[0] = sink->v;
  row = sink->n;
  p.ret_off = row;
  row += (int64_t)n_ret * Lc;
  for (int i = 1; i < ns; ++i) {
    p.seg_start[i] = row;
    p.seg_k[i] = segs[i]->k;
    p.seg_v[i] = segs[i]->v;
    row += segs[i]->n;
  }
  p.seg_start[ns] = row;
  p.nseg = ns;
  p.Nk = row;
  if (p.Nk > win_rows)
    return fail(WKV_ERR_SHAPE, "wkv_assemble_window: window needs %lld rows, capacity %lld",
                (long long)p.Nk, (long long)win_rows);
  if (p.Nk > wkv::kMaxWindowRows)
    return fail(WKV_ERR_SHAPE, "wkv_assemble_window: window of %lld rows exceeds %lld",
                (long long)p.Nk, (long long)wkv::kMaxWindowRows);
  if (p.Nk == 0) return WKV_OK;
  p.bank_k = n_ret ? bank->k : nullptr;
  p.bank_v = n_ret ? bank->v : nullptr;
  p.bank_ks = n_ret ? bank->k_scale : nullptr;
  p.bank_vs = n_ret ? bank->v_scale : nullptr;
  p.idx = retrieved_idx;
  p.M = M;
  p.Lc = Lc;
  p.n_ret = n_ret;
  p.int4 = int4;
  p.cpr = H * D / 8;
  hipError_t e = wkv::assemble_launch(p, win_k, win_v, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "wkv_assemble_window launch");
  return WKV_OK;
}

size_t wkv_attention_workspace_bytes(int32_t Nq, int32_t Nk, int32_t H, int32_t D) {
  if (Nq < 1 || Nk < 1 || H < 1 || (D != 64 && D != 128)) return 0;
  wkv::AttnPlan p = wkv::attention_plan(Nq, Nk, H, D, num_cus());
  return wkv::attention_ws_bytes(p, Nq, H, D);
}

wkv_status wkv_chunk_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               int32_t Nq, int32_t Nk, int32_t H, int32_t D, float scale,
                               uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                               wkv_stream_t stream) {
  if (!q || !k || !v || !out) return fail(WKV_ERR_NULL, "wkv_chunk_attention: q, k, v and out are required");
  if (wkv_status st = check_hd(H, D)) return st;
  if (Nq < 1 || Nk < 1) return fail(WKV_ERR_SHAPE, "wkv_chunk_attention: Nq=%d Nk=%d", Nq, Nk);
  if ((int64_t)Nk * H * D >= ((int64_t)1 << 31) || (int64_t)Nq * H * D >= ((int64_t)1 << 31))
    return fail(WKV_ERR_SHAPE, "wkv_chunk_attention: Nq*H*D and Nk*H*D must be < 2^31");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (lse && !aligned16(lse)) || (ws && !aligned16(ws)))
    return fail(WKV_ERR_ALIGN, "wkv_chunk_attention: device pointers must be 16-byte aligned");
  if (!(scale == scale) || std::isinf(scale))
    return fail(WKV_ERR_SHAPE, "wkv_chunk_attention: scale is not finite");
  const float sc = scale > 0.0f ? scale : 1.0f / std::sqrt((float)D);
  wkv::AttnPlan plan = wkv::attention_plan(Nq, Nk, H, D, num_cus());
  // Fewer splits when the workspace is short.
  while (plan.splits > 1 && (!ws || wkv::attention_ws_bytes(plan, Nq, H, D) > ws_bytes)) {
    const int kblocks = (Nk + 63) / 64;
    const int want = plan.splits / 2;
    const int kb_per = (kblocks + want - 1) / want;
    plan.keys_per_split = kb_per * 64;
    plan.splits = (kblocks + kb_per - 1) / kb_per;
  }
  if (plan.splits <= 1) {
    plan.splits = 1;
    plan.keys_per_split = Nk;
  }
  hipError_t e = wkv::attention_launch(q, k, v, Nq, Nk, H, D, sc, out, lse, plan, ws,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "wkv_chunk_attention launch");
  return WKV_OK;
}

size_t wkv_attention_window_workspace_bytes(int32_t Nq, int64_t Nk_pad, int32_t H, int32_t D) {
  if (Nq < 1 || Nk_pad < 1 || Nk_pad >= ((int64_t)1 << 31) || H < 1 || (D != 64 && D != 128))
    return 0;
  wkv::AttnPlan p = wkv::attention_plan(Nq, (int)Nk_pad, H, D, num_cus());
  return wkv::attention_window_table_bytes((int)((Nk_pad + 63) / 64)) +
         wkv::attention_ws_bytes(p, Nq, H, D);
}

wkv_status wkv_chunk_attention_window(const uint16_t* q, int32_t Nq, const wkv_segment* sink,
                                      const wkv_bank* bank, const int32_t* retrieved_idx,
                                      int32_t n_ret, const wkv_segment* recent, int32_t n_recent,
                                      const wkv_segment* current, int32_t H, int32_t D,
                                      float scale, uint16_t* out, float* lse, void* ws,
                                      size_t ws_bytes, wkv_stream_t stream) {
  static const char* fn = "wkv_chunk_attention_window";
  if (!q || !out || !sink || !current)
    return fail(WKV_ERR_NULL, "%s: q, out, sink and current are required", fn);
  if (wkv_status st = check_hd(H, D)) return st;
  if (Nq < 1) return fail(WKV_ERR_SHAPE, "%s: Nq=%d", fn, Nq);
  if (n_ret < 0 || n_recent < 0 || n_ret + n_recent + 2 > wkv::kMaxWinPieces)
    return fail(WKV_ERR_SHAPE, "%s: n_ret=%d n_recent=%d (at most %d pieces)", fn, n_ret,
                n_recent, wkv::kMaxWinPieces);
  if (n_ret > 0 && (!bank || !retrieved_idx))
    return fail(WKV_ERR_NULL, "%s: n_ret>0 needs bank and retrieved_idx", fn);
  if (n_recent > 0 && !recent) return fail(WKV_ERR_NULL, "%s: recent is NULL", fn);
  if (!aligned16(q) || !aligned16(out) || (lse && !aligned16(lse)) || (ws && !aligned16(ws)) ||
      (retrieved_idx && !aligned16(retrieved_idx)))
    return fail(WKV_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
  if ((int64_t)Nq * H * D >= ((int64_t)1 << 31))
    return fail(WKV_ERR_SHAPE, "%s: Nq*H*D must be < 2^31", fn);
  if (!(scale == scale) || std::isinf(scale))
    return fail(WKV_ERR_SHAPE, "%s: scale is not finite", fn);
  if (n_ret > 0) {
    if (bank->dtype == WKV_BANK_INT4_G32)
      return fail(WKV_ERR_UNSUPPORTED, "%s: an int4 bank needs wkv_assemble_window", fn);
    if (bank->dtype != WKV_BANK_BF16)
      return fail(WKV_ERR_UNSUPPORTED, "%s: bank dtype %d", fn, bank->dtype);
    if (bank->M < 1 || bank->Lc < 1)
      return fail(WKV_ERR_SHAPE, "%s: bank M=%d Lc=%d", fn, bank->M, bank->Lc);
    if (!bank->k || !bank->v) return fail(WKV_ERR_NULL, "%s: bank k/v NULL", fn);
    if (!aligned16(bank->k) || !aligned16(bank->v))
      return fail(WKV_ERR_ALIGN, "%s: bank pointers must be 16-byte aligned", fn);
  }
  // Pieces in window order: sink, retrieved slots, recent..., current.
  wkv::WinPieces w;
  std::memset(&w, 0, sizeof(w));
  int np = 0;
  int64_t tiles = 0;
  auto add = [&](const uint16_t* k, const uint16_t* v, int32_t n, int32_t slot) -> wkv_status {
    if (n < 0) return fail(WKV_ERR_SHAPE, "%s: piece %d has n=%d", fn, np, n);
    if (slot < 0 && n > 0 && (!k || !v))
      return fail(WKV_ERR_NULL, "%s: piece %d has n=%d but NULL k/v", fn, np, n);
    if (!aligned16(k) || !aligned16(v))
      return fail(WKV_ERR_ALIGN, "%s: piece %d pointers must be 16-byte aligned", fn, np);
    w.k[np] = k;
    w.v[np] = v;
    w.n[np] = n;
    w.slot[np] = slot;
    w.tile0[np] = (int32_t)tiles;
    tiles += (n + 63) / 64;
    ++np;
    return WKV_OK;
  };
  wkv_status st = add(sink->k, sink->v, sink->n, -1);
  for (int i = 0; st == WKV_OK && i < n_ret; ++i)
    st = add(static_cast<const uint16_t*>(bank->k), static_cast<const uint16_t*>(bank->v),
             bank->Lc, i);
  for (int i = 0; st == WKV_OK && i < n_recent; ++i)
    st = add(recent[i].k, recent[i].v, recent[i].n, -1);
  if (st == WKV_OK) st = add(current->k, current->v, current->n, -1);
  if (st != WKV_OK) return st;
  const int64_t nk_pad = tiles * 64;
  if (nk_pad < 1) return fail(WKV_ERR_SHAPE, "%s: the window is empty", fn);
  if (nk_pad * H * D >= ((int64_t)1 << 31))
    return fail(WKV_ERR_SHAPE, "%s: padded window of %lld keys: Nk_pad*H*D must be < 2^31", fn,
                (long long)nk_pad);
  w.tile0[np] = (int32_t)tiles;
  w.npieces = np;
  w.idx = retrieved_idx;
  w.M = n_ret > 0 ? bank->M : 0;
  w.Lc = n_ret > 0 ? bank->Lc : 0;
  const float sc = scale > 0.0f ? scale : 1.0f / std::sqrt((float)D);
  const int Nk = (int)nk_pad;
  const size_t table = wkv::attention_window_table_bytes((int)tiles);
  if (!ws || ws_bytes < table)
    return fail(WKV_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu for the tile table", fn,
                ws ? ws_bytes : (size_t)0, table);
  const size_t part_bytes = ws_bytes - table;
  wkv::AttnPlan plan = wkv::attention_plan(Nq, Nk, H, D, num_cus());
  while (plan.splits > 1 && wkv::attention_ws_bytes(plan, Nq, H, D) > part_bytes) {
    const int kblocks = Nk / 64;
    const int want = plan.splits / 2;
    const int kb_per = (kblocks + want - 1) / want;
    plan.keys_per_split = kb_per * 64;
    plan.splits = (kblocks + kb_per - 1) / kb_per;
  }
  if (plan.splits <= 1) {
    plan.splits = 1;
    plan.keys_per_split = Nk;
  }
  hipError_t e = wkv::attention_window_launch(q, w, Nq, H, D, sc, out, lse, plan, ws,
                                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "wkv_chunk_attention_window launch");
  return WKV_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Host-side retrieval planning for the host tier (WorldPager Fig. 2: the
// camera pose is an input known before the chunk is computed, so the
// retrieval set of the next chunk is chosen from the extrapolated pose while
// the GPU still works on the current one, and its copies are queued ahead).
// wkv_pose_topk_host is the pose top-k of wkv_pose_topk evaluated on the host
// for that planning: the same float64 operation sequence (contraction off
// from here to the end of the file), min-max normalisation, and (distance,
// index) order with NaN last. The retrieval feeding the window stays on the
// GPU.
#pragma clang fp contract(off)

namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;
constexpr double kPi = 3.1415926535897932384626433832795;

double wrap_angle(double a) {
  double w = a - kTwoPi * std::rint(a / kTwoPi);
  if (w <= -kPi) w = w + kTwoPi;
  if (w > kPi) w = w - kTwoPi;
  return w;
}

double minmax(double v, double lo, double hi) { return hi == lo ? 0.0 : (v - lo) / (hi - lo); }

}  // namespace


extern "C" {

wkv_status wkv_pose_topk_host(const wkv_pose* bank_poses, int32_t M, const wkv_pose* query_hist,
                              int32_t n_hist, int32_t k, int32_t* out_idx, double* out_dist) {
  if (!bank_poses || !query_hist || !out_idx)
    return fail(WKV_ERR_NULL, "wkv_pose_topk_host: bank_poses, query_hist and out_idx are required");
  if (M < 1 || M > 8192) return fail(WKV_ERR_SHAPE, "wkv_pose_topk_host: M=%d not in [1, 8192]", M);
  if (k < 1) return fail(WKV_ERR_K, "wkv_pose_topk_host: k=%d < 1", k);
  if (n_hist != 1 && n_hist != 2)
    return fail(WKV_ERR_K, "wkv_pose_topk_host: n_hist=%d (must be 1 or 2)", n_hist);
  const wkv_pose& last = query_hist[n_hist - 1];
  double qx = last.x, qy = last.y, qz = last.z, qyaw = last.yaw;
  if (n_hist == 2) {
    const wkv_pose& prev = query_hist[0];
    const double lx = last.x, ly = last.y, lz = last.z, lyaw = last.yaw;
    qx = 2.0 * lx - (double)prev.x;
    qy = 2.0 * ly - (double)prev.y;
    qz = 2.0 * lz - (double)prev.z;
    qyaw = wrap_angle(lyaw + wrap_angle(lyaw - (double)prev.yaw));
  }
  // the query is a float32 pose
  const double fx = (float)qx, fy = (float)qy, fz = (float)qz, fyaw = (float)qyaw;
  std::vector<double> dtr(M), drot(M);
  double tmin = INFINITY, tmax = -INFINITY, rmin = INFINITY, rmax = -INFINITY;
  for (int i = 0; i < M; ++i) {
    const double dx = (double)bank_poses[i].x - fx;
    const double dy = (double)bank_poses[i].y - fy;
    const double dz = (double)bank_poses[i].z - fz;
    dtr[i] = (dx * dx + dy * dy) + dz * dz;
    drot[i] = std::fabs(wrap_angle((double)bank_poses[i].yaw - fyaw));
    tmin = std::fmin(tmin, dtr[i]);
    tmax = std::fmax(tmax, dtr[i]);
    rmin = std::fmin(rmin, drot[i]);
    rmax = std::fmax(rmax, drot[i]);
  }
  std::vector<std::pair<double, int>> key(M);
  for (int i = 0; i < M; ++i) {
    const double d = minmax(dtr[i], tmin, tmax) + minmax(drot[i], rmin, rmax);
    key[i] = {std::isnan(d) ? INFINITY : d, i};
  }
  const int k_eff = k < M ? k : M;
  std::partial_sort(key.begin(), key.begin() + k_eff, key.end());
  std::vector<int> sel(k_eff);
  for (int i = 0; i < k_eff; ++i) sel[i] = key[i].second;
  std::sort(sel.begin(), sel.end());
  for (int i = 0; i < k_eff; ++i) {
    out_idx[i] = sel[i];
    if (out_dist) {
      const int j = sel[i];
      out_dist[i] = minmax(dtr[j], tmin, tmax) + minmax(drot[j], rmin, rmax);
    }
  }
  return WKV_OK;
}

wkv_pose wkv_pose_extrapolate(wkv_pose prev, wkv_pose last) {
  wkv_pose q;
  const double lx = last.x, ly = last.y, lz = last.z, lyaw = last.yaw;
  q.x = (float)(2.0 * lx - (double)prev.x);
  q.y = (float)(2.0 * ly - (double)prev.y);
  q.z = (float)(2.0 * lz - (double)prev.z);
  q.yaw = (float)wrap_angle(lyaw + wrap_angle(lyaw - (double)prev.yaw));
  return q;
}

}  // extern "C"
