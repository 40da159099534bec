// Query-based World Retrieval (WorldKV Sec. 4.2: sim(a_cur, a_i) may be a
// query-based importance score; WorldAttention pipeline: a page is scored by
// the dot product of the current mean query and its mean key, the top pages
// are kept).
//
//   mean rows  - float64 mean over token rows of bf16 [B][L_in][H][D], all
//                rows or the rows an index list names. Grid (column group of
//                512 elements, slice of 64 rows, unit): each wave loads its 16
//                rows of the slice at once as whole 1 KiB row segments (16
//                bytes per lane), accumulates 8 doubles per lane in row order,
//                and the block adds its 4 waves in a fixed order into a
//                per-slice partial; a finalize kernel adds the
//                slices in order and divides by L. No atomics: the result is
//                bitwise reproducible.
//   query top-k - one wave per stored chunk forms <mean key, mean query> in
//                float64 (fixed shuffle tree), then one block keeps the k
//                largest (score, lower index first) with the shared radix
//                select and writes them in ascending chunk order.
#include "wkv_common.hpp"
#include "wkv_internal.hpp"
#include "wkv_select.hpp"

namespace wkv {

namespace {

constexpr int kMeanBlock = 256;
constexpr int kRowsPerSlice = 64;
constexpr int kChunksPerGroup = 64;  // 16-byte column chunks per block (one per lane)

// grid: (ceil(C8 / 64), slices, B). part[b][slice][HD].
__global__ __launch_bounds__(kMeanBlock) void mean_rows_kernel(
    const uint16_t* __restrict__ x, int L_in, const int32_t* __restrict__ rows, int L, int HD,
    double* __restrict__ part) {
  __shared__ double red[kMeanBlock / 64][kChunksPerGroup][8];
  const int b = blockIdx.z, sl = blockIdx.y, cg = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int C8 = HD / 8;
  const int c = cg * kChunksPerGroup + lane;
  const bool col = c < C8;
  const int r0 = sl * kRowsPerSlice;
  const int r1 = min(L, r0 + kRowsPerSlice);
  const uint4* src = reinterpret_cast<const uint4*>(x) + (size_t)b * L_in * C8;
  const int32_t* ridx = rows ? rows + (size_t)b * L : nullptr;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  auto load = [&](int r) -> uint4 {
    const int sr = ridx ? ridx[r] : r;
    if (!col || sr < 0 || sr >= L_in) return make_uint4(0, 0, 0, 0);  // out of range: zeros
    return ld_stream(src + (size_t)sr * C8 + c);
  };
  auto add = [&](const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += (double)bf16_to_f32(w[q] & 0xFFFFu);
      acc[2 * q + 1] += (double)bf16_to_f32(w[q] >> 16);
    }
  };
  // All of a wave's rows of the slice are in flight at once (one memory
  // round trip), then added in row order.
  constexpr int kPerWave = kRowsPerSlice / (kMeanBlock / 64);
  uint4 v[kPerWave];
#pragma unroll
  for (int t = 0; t < kPerWave; ++t) {
    const int r = r0 + wave + 4 * t;
    v[t] = r < r1 ? load(r) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int t = 0; t < kPerWave; ++t) add(v[t]);
#pragma unroll
  for (int e = 0; e < 8; ++e) red[wave][lane][e] = acc[e];
  __syncthreads();
  double* dst = part + ((size_t)b * gridDim.y + sl) * HD;
  for (int i = threadIdx.x; i < kChunksPerGroup * 8; i += kMeanBlock) {
    const int ln = i / 8, e = i % 8;
    const int cc = cg * kChunksPerGroup + ln;
    if (cc >= C8) continue;
    double t = red[0][ln][e];
#pragma unroll
    for (int w = 1; w < kMeanBlock / 64; ++w) t += red[w][ln][e];
    dst[cc * 8 + e] = t;
  }
}

// grid: (ceil(HD / 256), B). out[b][i] = (sum over slices, in order) / L.
__global__ __launch_bounds__(256) void mean_rows_final_kernel(const double* __restrict__ part,
                                                               int nsl, int L, int HD,
                                                               double* __restrict__ out) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= HD) return;
  const double* p = part + (size_t)b * nsl * HD + i;
  // Loads of eight slices in flight, added in slice order.
  double t = 0.0;
  int s = 0;
  for (; s + 8 <= nsl; s += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(size_t)(s + u) * HD];
#pragma unroll
    for (int u = 0; u < 8; ++u) t += v[u];
  }
  for (; s < nsl; ++s) t += p[(size_t)s * HD];
  out[(size_t)b * HD + i] = t / (double)L;
}

// grid: ceil(M / 4), block 256: wave w scores chunk blockIdx.x * 4 + w.
__global__ __launch_bounds__(256) void query_score_kernel(const double* __restrict__ km, int M,
                                                          const double* __restrict__ qm, int HD,
                                                          double* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;  // whole wave leaves together
  const double* k = km + (size_t)m * HD;
  double acc = 0.0;
  for (int d = lane; d < HD; d += 64) acc = fma(k[d], qm[d], acc);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) scores[m] = acc;
}

// One block: the k_eff largest scores (lower index first on ties, NaN last),
// written in ascending chunk order.
template <int BLOCK, int KPT>
__global__ __launch_bounds__(BLOCK) void score_topk_kernel(const double* __restrict__ scores,
                                                           int M, int k_eff,
                                                           int32_t* __restrict__ out_idx) {
  __shared__ SelectShared sh;
  const int tid = threadIdx.x;
  uint64_t key[KPT];
  bool valid[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int p = tid * KPT + i;
    valid[i] = p < M;
    key[i] = valid[i] ? order_key(-scores[p]) : ~0ull;  // largest first; NaN keeps the top key
  }
  bool keep[KPT];
  int kc = 0;
  if (k_eff >= M) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      keep[i] = valid[i];
      kc += keep[i] ? 1 : 0;
    }
  } else {
    uint64_t prefix, mask;
    int rank;
    block_radix_select<BLOCK, KPT>(key, valid, k_eff, sh, &prefix, &mask, &rank);
    kc = block_keep_flags<BLOCK, KPT>(key, valid, prefix, mask, rank, sh, keep);
  }
  int tot;
  int pos = block_exclusive_scan<BLOCK>(kc, sh, &tot);
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (keep[i] && pos < k_eff) out_idx[pos] = tid * KPT + i;  // never past k_eff
    pos += keep[i] ? 1 : 0;
  }
}

}  // namespace

int mean_rows_slices(int L) { return (L + kRowsPerSlice - 1) / kRowsPerSlice; }

hipError_t mean_rows_launch(const uint16_t* x, int B, int L_in, const int32_t* rows, int L,
                            int HD, double* part, double* out, hipStream_t s) {
  const int nsl = mean_rows_slices(L);
  const int C8 = HD / 8;
  hipLaunchKernelGGL(mean_rows_kernel, dim3((C8 + kChunksPerGroup - 1) / kChunksPerGroup, nsl, B),
                     dim3(kMeanBlock), 0, s, x, L_in, rows, L, HD, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mean_rows_final_kernel, dim3((HD + 255) / 256, B), dim3(256), 0, s, part,
                     nsl, L, HD, out);
  return hipGetLastError();
}

hipError_t query_topk_launch(const double* km, int M, const double* qm, int HD, int k_eff,
                             int32_t* out_idx, double* scores, hipStream_t s) {
  hipLaunchKernelGGL(query_score_kernel, dim3((M + 3) / 4), dim3(256), 0, s, km, M, qm, HD,
                     scores);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (M <= 64)
    hipLaunchKernelGGL((score_topk_kernel<64, 1>), dim3(1), dim3(64), 0, s, scores, M, k_eff,
                       out_idx);
  else if (M <= 1024)
    hipLaunchKernelGGL((score_topk_kernel<256, 4>), dim3(1), dim3(256), 0, s, scores, M, k_eff,
                       out_idx);
  else
    hipLaunchKernelGGL((score_topk_kernel<1024, 8>), dim3(1), dim3(1024), 0, s, scores, M,
                       k_eff, out_idx);
  return hipGetLastError();
}

}  // namespace wkv
