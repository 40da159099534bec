// World Retrieval by camera pose (WorldKV Sec. 4.2 retrieval equation,
// Sec. 5.1 distance recipe; WorldPager Fig. 2 for the extrapolated query).
//
// One block sized to the bank (one wave up to 64 chunks, 256 threads up to
// 1024, 1024 threads up to 8192): every thread forms the query pose,
// computes the float64 translation and rotation distances of its stored
// chunks, the block reduces their min and max, forms the normalised sum, and
// the shared radix select keeps the k smallest (distance, index) pairs,
// written in ascending chunk order. Floating-point contraction is off in this file so
// every distance is the same sequence of correctly rounded IEEE operations
// the definition states.
#pragma clang fp contract(off)

#include "wkv_common.hpp"
#include "wkv_internal.hpp"
#include "wkv_select.hpp"

namespace wkv {

namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;
constexpr double kPi = 3.1415926535897932384626433832795;

// Angle into (-pi, pi]: a - 2pi * rint(a / 2pi), then the -pi / +pi seams.
__device__ __forceinline__ double wrap_angle(double a) {
  double w = a - kTwoPi * rint(a / kTwoPi);
  if (w <= -kPi) w = w + kTwoPi;
  if (w > kPi) w = w - kTwoPi;
  return w;
}

struct PoseArgs {
  float qx, qy, qz, qyaw;  // last (or only) pose
  float px, py, pz, pyaw;  // previous pose (n_hist == 2)
  int n_hist;
};

template <int BLOCK>
__device__ __forceinline__ double block_reduce(double v, bool is_max, double* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    double y = __shfl_xor(v, o, 64);
    v = is_max ? fmax(v, y) : fmin(v, y);
  }
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double r = red[0];
  for (int w = 1; w < BLOCK / 64; ++w) r = is_max ? fmax(r, red[w]) : fmin(r, red[w]);
  return r;
}

// Shared tail of both pose kernels: block min/max of the two terms, the
// normalised sum, the k_eff smallest (distance, index) pairs written in
// ascending chunk order.
template <int BLOCK, int KPT>
__device__ __forceinline__ void finish_topk(const double (&dtr)[KPT], const double (&drot)[KPT],
                                            const bool (&valid)[KPT], double tmin, double tmax,
                                            double rmin, double rmax, int M, int k_eff,
                                            int32_t* __restrict__ out_idx,
                                            double* __restrict__ out_dist, SelectShared& sh,
                                            double* red) {
  const int tid = threadIdx.x;
  tmin = block_reduce<BLOCK>(tmin, false, red);
  tmax = block_reduce<BLOCK>(tmax, true, red);
  rmin = block_reduce<BLOCK>(rmin, false, red);
  rmax = block_reduce<BLOCK>(rmax, true, red);
  const double trng = tmax - tmin, rrng = rmax - rmin;

  uint64_t key[KPT];
  double dist[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const double a = (tmax == tmin) ? 0.0 : (dtr[i] - tmin) / trng;
    const double r = (rmax == rmin) ? 0.0 : (drot[i] - rmin) / rrng;
    dist[i] = a + r;
    key[i] = valid[i] ? order_key(dist[i]) : ~0ull;
  }
  bool keep[KPT];
  int kc;
  if (k_eff >= M) {
    kc = 0;
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
    if (keep[i] && pos < k_eff) {  // never past the k_eff outputs
      out_idx[pos] = tid * KPT + i;
      if (out_dist) out_dist[pos] = dist[i];
    }
    pos += keep[i] ? 1 : 0;
  }
}

template <int BLOCK, int KPT>
__global__ __launch_bounds__(BLOCK) void pose_topk_kernel(
    const float4* __restrict__ poses, int M, PoseArgs qa, int k_eff,
    int32_t* __restrict__ out_idx, double* __restrict__ out_dist,
    float4* __restrict__ out_query) {
  __shared__ SelectShared sh;
  __shared__ double red[BLOCK / 64];
  const int tid = threadIdx.x;

  double qx = qa.qx, qy = qa.qy, qz = qa.qz, qyaw = qa.qyaw;
  if (qa.n_hist == 2) {
    const double lx = qa.qx, ly = qa.qy, lz = qa.qz, lyaw = qa.qyaw;
    qx = 2.0 * lx - (double)qa.px;
    qy = 2.0 * ly - (double)qa.py;
    qz = 2.0 * lz - (double)qa.pz;
    qyaw = wrap_angle(lyaw + wrap_angle(lyaw - (double)qa.pyaw));
  }
  // The query is stored as float; distances use the float value.
  const float fqx = (float)qx, fqy = (float)qy, fqz = (float)qz, fqyaw = (float)qyaw;
  if (tid == 0 && out_query) *out_query = make_float4(fqx, fqy, fqz, fqyaw);

  double dtr[KPT], drot[KPT];
  bool valid[KPT];
  double tmin = INFINITY, tmax = -INFINITY, rmin = INFINITY, rmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int p = tid * KPT + i;
    valid[i] = p < M;
    dtr[i] = 0.0;
    drot[i] = 0.0;
    if (valid[i]) {
      const float4 P = poses[p];
      const double dx = (double)P.x - (double)fqx;
      const double dy = (double)P.y - (double)fqy;
      const double dz = (double)P.z - (double)fqz;
      dtr[i] = (dx * dx + dy * dy) + dz * dz;
      drot[i] = fabs(wrap_angle((double)P.w - (double)fqyaw));
      tmin = fmin(tmin, dtr[i]);
      tmax = fmax(tmax, dtr[i]);
      rmin = fmin(rmin, drot[i]);
      rmax = fmax(rmax, drot[i]);
    }
  }
  finish_topk<BLOCK, KPT>(dtr, drot, valid, tmin, tmax, rmin, rmax, M, k_eff, out_idx, out_dist,
                          sh, red);
}

// Full-rotation variant: a pose is 32 bytes (x, y, z, qw, qx, qy, qz, pad);
// the rotation term is the SO(3) geodesic angle of r = conj(q_i) * q_query,
// 2 * atan2(|r_xyz|, |r_w|), in float64 from the float32 pose values.
struct PoseQ {
  float x, y, z, qw, qx, qy, qz, pad;
};

__device__ __forceinline__ double geodesic(double wa, double xa, double ya, double za, double wb,
                                           double xb, double yb, double zb) {
  const double w = wa * wb + ((xa * xb + ya * yb) + za * zb);
  const double vx = (wa * xb - wb * xa) - (ya * zb - za * yb);
  const double vy = (wa * yb - wb * ya) - (za * xb - xa * zb);
  const double vz = (wa * zb - wb * za) - (xa * yb - ya * xb);
  return 2.0 * atan2(sqrt((vx * vx + vy * vy) + vz * vz), fabs(w));
}

template <int BLOCK, int KPT>
__global__ __launch_bounds__(BLOCK) void pose_topk_so3_kernel(
    const float4* __restrict__ poses, int M, PoseQ q, int k_eff, int32_t* __restrict__ out_idx,
    double* __restrict__ out_dist) {
  __shared__ SelectShared sh;
  __shared__ double red[BLOCK / 64];
  const int tid = threadIdx.x;
  double dtr[KPT], drot[KPT];
  bool valid[KPT];
  double tmin = INFINITY, tmax = -INFINITY, rmin = INFINITY, rmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int p = tid * KPT + i;
    valid[i] = p < M;
    dtr[i] = 0.0;
    drot[i] = 0.0;
    if (valid[i]) {
      const float4 A = poses[2 * p], Bq = poses[2 * p + 1];
      const double dx = (double)A.x - (double)q.x;
      const double dy = (double)A.y - (double)q.y;
      const double dz = (double)A.z - (double)q.z;
      dtr[i] = (dx * dx + dy * dy) + dz * dz;
      drot[i] = geodesic(A.w, Bq.x, Bq.y, Bq.z, q.qw, q.qx, q.qy, q.qz);
      tmin = fmin(tmin, dtr[i]);
      tmax = fmax(tmax, dtr[i]);
      rmin = fmin(rmin, drot[i]);
      rmax = fmax(rmax, drot[i]);
    }
  }
  finish_topk<BLOCK, KPT>(dtr, drot, valid, tmin, tmax, rmin, rmax, M, k_eff, out_idx, out_dist,
                          sh, red);
}

}  // namespace

hipError_t pose_topk_launch(const void* poses, int M, const float* last,
                            const float* prev, int n_hist, int k_eff,
                            int32_t* out_idx, double* out_dist, void* out_query,
                            hipStream_t s) {
  PoseArgs qa;
  qa.qx = last[0]; qa.qy = last[1]; qa.qz = last[2]; qa.qyaw = last[3];
  qa.px = prev ? prev[0] : 0.f; qa.py = prev ? prev[1] : 0.f;
  qa.pz = prev ? prev[2] : 0.f; qa.pyaw = prev ? prev[3] : 0.f;
  qa.n_hist = n_hist;
  const float4* P = reinterpret_cast<const float4*>(poses);
  float4* oq = reinterpret_cast<float4*>(out_query);
  if (M <= 64)
    hipLaunchKernelGGL((pose_topk_kernel<64, 1>), dim3(1), dim3(64), 0, s, P, M, qa, k_eff,
                       out_idx, out_dist, oq);
  else if (M <= 1024)
    hipLaunchKernelGGL((pose_topk_kernel<256, 4>), dim3(1), dim3(256), 0, s, P, M, qa, k_eff,
                       out_idx, out_dist, oq);
  else
    hipLaunchKernelGGL((pose_topk_kernel<1024, 8>), dim3(1), dim3(1024), 0, s, P, M, qa, k_eff,
                       out_idx, out_dist, oq);
  return hipGetLastError();
}

}  // namespace wkv

namespace wkv {

hipError_t pose_topk_so3_launch(const void* poses, int M, const float* query, int k_eff,
                                int32_t* out_idx, double* out_dist, hipStream_t s) {
  PoseQ q;
  q.x = query[0]; q.y = query[1]; q.z = query[2];
  q.qw = query[3]; q.qx = query[4]; q.qy = query[5]; q.qz = query[6]; q.pad = 0.f;
  const float4* P = reinterpret_cast<const float4*>(poses);
  if (M <= 64)
    hipLaunchKernelGGL((pose_topk_so3_kernel<64, 1>), dim3(1), dim3(64), 0, s, P, M, q, k_eff,
                       out_idx, out_dist);
  else if (M <= 1024)
    hipLaunchKernelGGL((pose_topk_so3_kernel<256, 4>), dim3(1), dim3(256), 0, s, P, M, q, k_eff,
                       out_idx, out_dist);
  else
    hipLaunchKernelGGL((pose_topk_so3_kernel<1024, 8>), dim3(1), dim3(1024), 0, s, P, M, q,
                       k_eff, out_idx, out_dist);
  return hipGetLastError();
}

}  // namespace wkv
