// World Compression of evicted chunks (WorldKV Sec. 4.3 "World Compression
// Mechanism"): per non-anchor token, the head-mean cosine of its key to the
// anchor-frame key at the same position; keep the anchor frame plus the
// lowest-scoring fraction of the pooled non-anchor tokens; compact K and V.
//
// Three kernels per call, all on the caller's stream:
//   score  - streams every key row once (HBM-bound). 4 lanes own one
//            (token, head) slice of D elements: each loads 16-byte pieces of
//            the anchor row and of the F-1 non-anchor rows, accumulates the
//            dot product and both squared norms in float64 (bf16 products are
//            exact in float64), reduces across its 4 lanes, and stores the
//            per-head cosine in LDS; the block then averages over heads in a
//            fixed order. The anchor slice already sits in registers, so the
//            score kernel also writes the anchor rows of k_out.
//   select - one block per unit, sized to the pooled count (256, 512 or 1024
//            threads, 8 keys each): radix select of the n_keep-th smallest
//            (score, index) key, stable compaction by block scan, writes
//            kept_idx.
//   gather - one wave per output row: copies the kept K rows (non-anchor) and
//            all kept V rows with 16-byte loads and stores. Outputs and V
//            (read once) use streaming accesses; the kept K rows use the
//            default policy since the score pass has just read them.
#include "wkv_common.hpp"
#include "wkv_internal.hpp"
#include "wkv_select.hpp"

namespace wkv {

namespace {

constexpr int kScoreBlock = 256;
constexpr int kLanesPerPair = 4;
constexpr int kPairsPerPass = kScoreBlock / kLanesPerPair;  // 64

__device__ __forceinline__ void accum_sq(const uint4& x, double& acc) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    double lo = (double)bf16_to_f32(w[i] & 0xFFFFu);
    double hi = (double)bf16_to_f32(w[i] >> 16);
    acc = fma(lo, lo, acc);
    acc = fma(hi, hi, acc);
  }
}

__device__ __forceinline__ void accum_dot_sq(const uint4& x, const uint4& a,
                                             double& dot, double& sq) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  const uint32_t v[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    double xl = (double)bf16_to_f32(w[i] & 0xFFFFu);
    double xh = (double)bf16_to_f32(w[i] >> 16);
    double al = (double)bf16_to_f32(v[i] & 0xFFFFu);
    double ah = (double)bf16_to_f32(v[i] >> 16);
    sq = fma(xl, xl, sq);
    sq = fma(xh, xh, sq);
    dot = fma(xl, al, dot);
    dot = fma(xh, ah, dot);
  }
}

__device__ __forceinline__ double quad_sum(double x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  return x;
}

// grid: (ceil(T / TT), B). Dynamic LDS: TT * (F-1) * H doubles.
template <int D, int F>
__global__ __launch_bounds__(kScoreBlock) void compress_score_kernel(
    const uint16_t* __restrict__ k, int T, int H, int TT,
    double* __restrict__ scores, uint16_t* __restrict__ k_out, int Lc) {
  constexpr int NLD = D / 32;  // 16-byte loads per lane per row slice
  extern __shared__ double cosbuf[];
  const int b = blockIdx.y;
  const int j0 = blockIdx.x * TT;
  const int ntok = min(TT, T - j0);
  const int npairs = ntok * H;
  const int tid = threadIdx.x;
  const int slot = tid / kLanesPerPair;
  const int sub = tid % kLanesPerPair;
  const size_t HD = (size_t)H * D;
  const uint16_t* unit = k + (size_t)b * F * T * HD;
  uint16_t* kout_unit = k_out + (size_t)b * Lc * HD;

  // Every lane of a quad runs the same number of iterations, so the quad
  // shuffles below always see their partners.
  for (int pair = slot; pair < npairs; pair += kPairsPerPass) {
    const int jl = pair / H;
    const int h = pair - jl * H;
    const int j = j0 + jl;
    uint4 a[NLD];
    uint4 x[F - 1][NLD];
    const size_t aoff = ((size_t)j * H + h) * D + sub * 8;
#pragma unroll
    for (int i = 0; i < NLD; ++i)
      a[i] = *reinterpret_cast<const uint4*>(unit + aoff + i * 32);
#pragma unroll
    for (int f = 1; f < F; ++f) {
      const size_t off = (((size_t)f * T + j) * H + h) * D + sub * 8;
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        x[f - 1][i] = *reinterpret_cast<const uint4*>(unit + off + i * 32);
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i)
      st_stream(kout_unit + aoff + i * 32, a[i]);
    double na = 0.0;
#pragma unroll
    for (int i = 0; i < NLD; ++i) accum_sq(a[i], na);
    na = quad_sum(na);
#pragma unroll
    for (int f = 1; f < F; ++f) {
      double dt = 0.0, nk = 0.0;
#pragma unroll
      for (int i = 0; i < NLD; ++i) accum_dot_sq(x[f - 1][i], a[i], dt, nk);
      dt = quad_sum(dt);
      nk = quad_sum(nk);
      if (sub == 0) {
        const double prod = nk * na;
        const double c = (prod == 0.0) ? 0.0 : dt / sqrt(prod);
        cosbuf[(jl * (F - 1) + (f - 1)) * H + h] = c;
      }
    }
  }
  __syncthreads();
  const int N = (F - 1) * T;
  for (int t = tid; t < ntok * (F - 1); t += kScoreBlock) {
    const int jl = t / (F - 1);
    const int fm = t - jl * (F - 1);
    const double* c = cosbuf + t * H;
    double s = 0.0;
    for (int h = 0; h < H; ++h) s += c[h];
    s = s / (double)H;
    scores[(size_t)b * N + (size_t)fm * T + j0 + jl] = s;
  }
}

constexpr int kSelKPT = 8;  // N <= 8 * block size

// grid: B. Writes kept_idx[b][0..Lc).
template <int kSelBlock>
__global__ __launch_bounds__(kSelBlock) void compress_select_kernel(
    const double* __restrict__ scores, int N, int T, int n_keep,
    int32_t* __restrict__ kept_idx, int Lc) {
  __shared__ SelectShared sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t* out = kept_idx + (size_t)b * Lc;
  for (int j = tid; j < T; j += kSelBlock) out[j] = j;
  if (n_keep == 0) return;
  if (n_keep == N) {
    for (int p = tid; p < N; p += kSelBlock) out[T + p] = T + p;
    return;
  }
  uint64_t key[kSelKPT];
  bool valid[kSelKPT];
  const double* s = scores + (size_t)b * N;
#pragma unroll
  for (int i = 0; i < kSelKPT; ++i) {
    const int p = tid * kSelKPT + i;
    valid[i] = p < N;
    key[i] = valid[i] ? order_key(s[p]) : ~0ull;
  }
  uint64_t prefix, mask;
  int rank;
  block_radix_select<kSelBlock, kSelKPT>(key, valid, n_keep, sh, &prefix, &mask,
                                         &rank);
  bool keep[kSelKPT];
  const int kc = block_keep_flags<kSelBlock, kSelKPT>(key, valid, prefix, mask,
                                                      rank, sh, keep);
  int tot;
  int pos = block_exclusive_scan<kSelBlock>(kc, sh, &tot);
#pragma unroll
  for (int i = 0; i < kSelKPT; ++i) {
    if (keep[i]) {
      if (pos < n_keep) out[T + pos] = T + tid * kSelKPT + i;  // never past Lc
      ++pos;
    }
  }
}

constexpr int kGatherBlock = 256;
constexpr int kRowsPerWave = 4;  // the copy loop below is written for 4

// grid: (ceil(Lc / (waves * kRowsPerWave)), B, 2). z = 0 copies K rows (rows
// below k_skip are skipped: the score kernel already wrote them), z = 1
// copies V rows. cpr = 16-byte chunks per row.
__global__ __launch_bounds__(kGatherBlock) void compress_gather_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ kept_idx, int FT, int Lc, int cpr, int k_skip,
    uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out) {
  const int b = blockIdx.y;
  const bool isk = blockIdx.z == 0;
  const uint4* src = reinterpret_cast<const uint4*>(isk ? k : v) + (size_t)b * FT * cpr;
  uint4* dst = reinterpret_cast<uint4*>(isk ? k_out : v_out) + (size_t)b * Lc * cpr;
  const int32_t* idx = kept_idx + (size_t)b * Lc;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * (kGatherBlock / 64) + wave) * kRowsPerWave;
  const int lo = isk ? k_skip : 0;
  // Resolve each row's source once (wave-uniform), then stream its columns.
  const uint4* rs[kRowsPerWave];
  uint4* rd[kRowsPerWave];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int row = row0 + r;
    const bool act = row < Lc && row >= lo;
    rs[r] = act ? src + (size_t)idx[row] * cpr : nullptr;
    rd[r] = act ? dst + (size_t)row * cpr : nullptr;
  }
  for (int c = lane; c < cpr; c += 64) {
    uint4 b0 = rs[0] ? (isk ? rs[0][c] : ld_stream(rs[0] + c)) : make_uint4(0, 0, 0, 0);
    uint4 b1 = rs[1] ? (isk ? rs[1][c] : ld_stream(rs[1] + c)) : make_uint4(0, 0, 0, 0);
    uint4 b2 = rs[2] ? (isk ? rs[2][c] : ld_stream(rs[2] + c)) : make_uint4(0, 0, 0, 0);
    uint4 b3 = rs[3] ? (isk ? rs[3][c] : ld_stream(rs[3] + c)) : make_uint4(0, 0, 0, 0);
    if (rd[0]) st_stream(rd[0] + c, b0);
    if (rd[1]) st_stream(rd[1] + c, b1);
    if (rd[2]) st_stream(rd[2] + c, b2);
    if (rd[3]) st_stream(rd[3] + c, b3);
  }
}

template <int D, int F>
hipError_t launch_score(const uint16_t* k, int B, int T, int H, int TT,
                        double* scores, uint16_t* k_out, int Lc, hipStream_t s) {
  dim3 grid((T + TT - 1) / TT, B);
  size_t lds = (size_t)TT * (F - 1) * H * sizeof(double);
  hipLaunchKernelGGL((compress_score_kernel<D, F>), grid, dim3(kScoreBlock), lds, s,
                     k, T, H, TT, scores, k_out, Lc);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_score_F(const uint16_t* k, int B, int F, int T, int H, int TT,
                            double* scores, uint16_t* k_out, int Lc, hipStream_t s) {
  switch (F) {
    case 2: return launch_score<D, 2>(k, B, T, H, TT, scores, k_out, Lc, s);
    case 3: return launch_score<D, 3>(k, B, T, H, TT, scores, k_out, Lc, s);
    case 4: return launch_score<D, 4>(k, B, T, H, TT, scores, k_out, Lc, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Tokens per score block: at least one full pass of (token, head) pairs, and
// grown while the grid still has >= 2048 blocks.
int compress_score_tile(int B, int T, int H) {
  int tt = (kPairsPerPass + H - 1) / H;
  while (tt * 2 <= 64 && tt * 2 * H <= 512 &&
         (long long)((T + tt * 2 - 1) / (tt * 2)) * B >= 2048)
    tt *= 2;
  return tt < T ? tt : T;
}

hipError_t compress_launch(const uint16_t* k, const uint16_t* v, int B, int F,
                           int T, int H, int D, int n_keep, uint16_t* k_out,
                           uint16_t* v_out, int32_t* kept_idx, double* scores,
                           bool need_scores, hipStream_t s) {
  const int N = (F - 1) * T;
  const int Lc = T + n_keep;
  const int cpr = H * D / 8;
  const bool score = need_scores || (n_keep > 0 && n_keep < N);
  hipError_t e = hipSuccess;
  if (score) {
    const int TT = compress_score_tile(B, T, H);
    e = (D == 128) ? dispatch_score_F<128>(k, B, F, T, H, TT, scores, k_out, Lc, s)
                   : dispatch_score_F<64>(k, B, F, T, H, TT, scores, k_out, Lc, s);
    if (e != hipSuccess) return e;
  }
  if (N <= 256 * kSelKPT)
    hipLaunchKernelGGL((compress_select_kernel<256>), dim3(B), dim3(256), 0, s, scores, N, T,
                       n_keep, kept_idx, Lc);
  else if (N <= 512 * kSelKPT)
    hipLaunchKernelGGL((compress_select_kernel<512>), dim3(B), dim3(512), 0, s, scores, N, T,
                       n_keep, kept_idx, Lc);
  else
    hipLaunchKernelGGL((compress_select_kernel<1024>), dim3(B), dim3(1024), 0, s, scores, N, T,
                       n_keep, kept_idx, Lc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows_per_block = (kGatherBlock / 64) * kRowsPerWave;
  dim3 grid((Lc + rows_per_block - 1) / rows_per_block, B, 2);
  hipLaunchKernelGGL(compress_gather_kernel, grid, dim3(kGatherBlock), 0, s, k, v,
                     kept_idx, F * T, Lc, cpr, score ? T : 0, k_out, v_out);
  return hipGetLastError();
}

}  // namespace wkv
