// Chunk attention (WorldAttention: scaled dot-product attention of the
// current chunk's queries over the visible keys, scaled by 1/sqrt(d), run at
// every denoising step; its kernel section streams key/value tiles with an
// online softmax: running max m, denominator l, unnormalised output o).
//
// gfx950 design. One block = 4 waves = 128 queries of one head; each wave owns
// 32 queries and walks the key range in tiles of 64 keys staged in LDS
// (double-buffered, next tile's global loads in flight during the current
// tile's math).
//   * S^T = K_tile * Q^T on v_mfma_f32_32x32x16_bf16: the 32x32 accumulator
//     layout puts one query per lane column, so the softmax row statistics of
//     a query live in two lanes (lane, lane^32) and need one cross-lane op.
//   * The rows of each 32-key MFMA tile are fed in a fixed permutation of the
//     keys chosen so that accumulator elements 8m..8m+7 of a lane are exactly
//     the 8 consecutive keys that lane must supply as the B operand of the
//     P*V MFMA: P^T goes from accumulator to operand by a bf16 conversion, with
//     no shuffle. The same permutation indexes V^T, so the sum is unchanged.
//   * O^T += V^T * P^T on the same MFMA; V is transposed into LDS ([d][key])
//     when staged, so each lane reads its 8 keys as one 16-byte LDS load.
//   * K rows in LDS use an XOR swizzle of 16-byte chunks so the permuted row
//     reads are free of bank conflicts.
//   * Softmax in base 2: p = exp2(s * scale*log2e - m). The O rescale is
//     skipped (exactly) for a wave whose running max did not change.
//   * Long key ranges with few query tiles are split over blocks; each split
//     writes unnormalised fp32 partials plus (m, l) and a merge kernel
//     combines them with the log-sum-exp identity.
//   * Blocks are renumbered so that each XCD (blocks are dealt round-robin
//     over the 8 XCDs) works on a contiguous range of (head, split, q-tile):
//     tiles sharing K/V share that XCD's L2.
#include "wkv_common.hpp"
#include "wkv_internal.hpp"

namespace wkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// MFMA row rho of a 32-key tile holds key perm(rho) of that tile.
__device__ __forceinline__ int key_perm(int rho) {
  const int i = rho >> 3, gg = (rho >> 2) & 1, j = rho & 3;
  return 16 * (i >> 1) + 8 * gg + 4 * (i & 1) + j;
}

// 16-byte chunk swizzle of K rows in LDS.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  const int s = (r & 3) | (((r >> 3) & 1) << 2) | (((r >> 2) & 1) << 3);
  return s & (D / 8 - 1);
}

__device__ __forceinline__ int xcd_remap(int L, int G) {
  const int per = G / 8, rem = G % 8;
  const int xcd = L % 8, idx = L / 8;
  return (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

template <int D>
struct Smem {
  static constexpr int VP = kBN + 8;        // V^T row pitch (bf16)
  static constexpr int K_ELEMS = kBN * D;   // swizzled, no pad
  static constexpr int V_ELEMS = D * VP;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
};

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, int Nq, int Nk, int H, float c,
    uint16_t* __restrict__ O, float* __restrict__ lse, float* __restrict__ opart,
    float2* __restrict__ mlpart, int nsplit, int kps) {
  using S = Smem<D>;
  constexpr int KS = D / 16;             // k-steps of the QK product
  constexpr int DT = D / 32;             // d tiles of the PV product
  constexpr int KCH = D / 8;             // 16-byte chunks per K row
  constexpr int KLD = kBN * KCH / kThreads;  // K chunks staged per thread
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * S::BUF];

  const int ntq = (Nq + kBM - 1) / kBM;
  const int W = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = W % ntq;
  const int rest = W / ntq;
  const int split = rest % nsplit;
  const int h = rest / nsplit;
  const int kbeg = split * kps;
  const int kend = min(Nk, kbeg + kps);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const size_t HD = (size_t)H * D;

  // Q^T operand: lane holds query l32, dims ks*16 + g*8 .. +8.
  const int q = qt * kBM + wave * 32 + l32;
  bf16x8 qf[KS];
  {
    const uint16_t* qp = Q + (size_t)min(q, Nq - 1) * HD + (size_t)h * D + g * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 u = *reinterpret_cast<const uint4*>(qp + ks * 16);
      if (q >= Nq) u = make_uint4(0, 0, 0, 0);
      qf[ks] = as_bf16x8(u);
    }
  }

  // Staging assignments.
  // K: chunk cidx = r*256 + tid -> key cidx / KCH, chunk cidx % KCH.
  // V: 4 keys (4*kg .. +3) x 8 dims (8*dch .. +7) per thread.
  const int kg = tid & 15, dch = tid >> 4;
  const bool vact = dch < D / 8;
  uint4 kreg[KLD];
  uint4 vreg[4];

  auto load_tile = [&](int kb) {
#pragma unroll
    for (int r = 0; r < KLD; ++r) {
      const int cidx = r * kThreads + tid;
      const int key = cidx / KCH, ch = cidx % KCH;
      const int gk = kb + key;
      kreg[r] = (gk < kend)
                    ? *reinterpret_cast<const uint4*>(K + (size_t)gk * HD + (size_t)h * D + ch * 8)
                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int gk = kb + 4 * kg + i;
      vreg[i] = (vact && gk < kend)
                    ? *reinterpret_cast<const uint4*>(V + (size_t)gk * HD + (size_t)h * D + dch * 8)
                    : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* Ks = smem + buf * S::BUF;
    uint16_t* VT = Ks + S::K_ELEMS;
#pragma unroll
    for (int r = 0; r < KLD; ++r) {
      const int cidx = r * kThreads + tid;
      const int key = cidx / KCH, ch = cidx % KCH;
      *reinterpret_cast<uint4*>(Ks + key * D + ((ch ^ kswz<D>(key)) * 8)) = kreg[r];
    }
    if (vact) {
      const uint32_t w0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
      const uint32_t w1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
      const uint32_t w2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
      const uint32_t w3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // dims 2w (low halves) and 2w+1 (high halves) of the 4 keys
        uint2 lo, hi;
        lo.x = (w0[w] & 0xFFFFu) | (w1[w] << 16);
        lo.y = (w2[w] & 0xFFFFu) | (w3[w] << 16);
        hi.x = (w0[w] >> 16) | (w1[w] & 0xFFFF0000u);
        hi.y = (w2[w] >> 16) | (w3[w] & 0xFFFF0000u);
        const int d = dch * 8 + 2 * w;
        *reinterpret_cast<uint2*>(VT + d * S::VP + 4 * kg) = lo;
        *reinterpret_cast<uint2*>(VT + (d + 1) * S::VP + 4 * kg) = hi;
      }
    }
  };

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  float m = -INFINITY;  // running max of s*c (base-2 domain)
  float lsum = 0.f;     // this lane's share of the denominator

  // Row of the 32-key MFMA tile this lane feeds (A operand of S^T).
  const int prow = key_perm(l32);

  const int nblk = (kend - kbeg + kBN - 1) / kBN;
  load_tile(kbeg);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < nblk; ++it) {
    const int kb = kbeg + it * kBN;
    const int cur = it & 1;
    const bool has_next = it + 1 < nblk;
    if (has_next) load_tile(kb + kBN);

    const uint16_t* Ks = smem + cur * S::BUF;
    const uint16_t* VT = Ks + S::K_ELEMS;

    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kt][e] = 0.f;
      const int r = kt * 32 + prow;
      const uint16_t* krow = Ks + r * D;
      const int sw = kswz<D>(r);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(krow + (((2 * ks + g) ^ sw) * 8));
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qf[ks], s[kt], 0, 0, 0);
      }
    }

    // Mask keys past the end of this block's range (last tile only).
    if (kb + kBN > kend) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kb + kt * 32 + 16 * (e >> 3) + 8 * g + (e & 7);
          if (key >= kend) s[kt][e] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kt][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;

    bf16x8 pb[2][2];
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        f32x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * mm + e], c, -m_new));
          pv[e] = p;
          ps += p;
        }
        pb[kt][mm] = __builtin_convertvector(pv, bf16x8);
      }
    lsum = lsum * alpha + ps;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
    }

#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint4 a = *reinterpret_cast<const uint4*>(
              VT + (dt * 32 + l32) * S::VP + kt * 32 + 16 * mm + 8 * g);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), pb[kt][mm], o[dt], 0, 0, 0);
        }

    if (has_next) store_tile(cur ^ 1);
    __syncthreads();
  }

  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  if (q >= Nq) return;
  if (nsplit == 1) {
    const float inv = 1.0f / ltot;
    uint16_t* op = O + (size_t)q * HD + (size_t)h * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint2 w;
        w.x = pack_bf16x2(o[dt][4 * i + 0] * inv, o[dt][4 * i + 1] * inv);
        w.y = pack_bf16x2(o[dt][4 * i + 2] * inv, o[dt][4 * i + 3] * inv);
        *reinterpret_cast<uint2*>(op + dt * 32 + 8 * i + 4 * g) = w;
      }
    if (lse && g == 0) lse[(size_t)h * Nq + q] = (m + log2f(ltot)) * kLn2;
  } else {
    const size_t row = ((size_t)split * H + h) * Nq + q;
    float* pp = opart + row * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 w = make_float4(o[dt][4 * i + 0], o[dt][4 * i + 1], o[dt][4 * i + 2],
                               o[dt][4 * i + 3]);
        *reinterpret_cast<float4*>(pp + dt * 32 + 8 * i + 4 * g) = w;
      }
    if (g == 0) mlpart[row] = make_float2(m, ltot);
  }
}

// Combines split partials: O = sum_s 2^(m_s-M) o_s / sum_s 2^(m_s-M) l_s.
// 32 lanes per (head, query) row, 4 dims each (D = 128) or 2 (D = 64).
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(
    const float* __restrict__ opart, const float2* __restrict__ mlpart, int Nq, int H,
    int nsplit, uint16_t* __restrict__ O, float* __restrict__ lse) {
  constexpr int PER = D / 32;
  const int rowid = blockIdx.x * 8 + (threadIdx.x >> 5);
  const int sub = threadIdx.x & 31;
  if (rowid >= H * Nq) return;
  const int h = rowid / Nq, q = rowid - h * Nq;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, mlpart[((size_t)s * H + h) * Nq + q].x);
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float den = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const size_t row = ((size_t)s * H + h) * Nq + q;
    const float2 ml = mlpart[row];
    const float w = exp2f(ml.x - M);
    den += w * ml.y;
    const float* pp = opart + row * D + sub * PER;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] += w * pp[i];
  }
  const float inv = 1.0f / den;
  uint16_t* op = O + (size_t)q * H * D + (size_t)h * D + sub * PER;
#pragma unroll
  for (int i = 0; i < PER; i += 2) {
    *reinterpret_cast<uint32_t*>(op + i) = pack_bf16x2(acc[i] * inv, acc[i + 1] * inv);
  }
  if (lse && sub == 0) lse[(size_t)h * Nq + q] = (M + log2f(den)) * kLn2;
}

template <int D>
hipError_t launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, int Nq, int Nk,
                  int H, float scale, uint16_t* out, float* lse, const AttnPlan& plan,
                  void* ws, hipStream_t s) {
  const int ntq = (Nq + kBM - 1) / kBM;
  const int G = ntq * H * plan.splits;
  const float c = scale * kLog2e;
  float* opart = nullptr;
  float2* ml = nullptr;
  if (plan.splits > 1) {
    opart = reinterpret_cast<float*>(ws);
    ml = reinterpret_cast<float2*>(opart + (size_t)plan.splits * H * Nq * D);
  }
  hipLaunchKernelGGL((attn_fwd_kernel<D>), dim3(G), dim3(kThreads), 0, s, q, k, v, Nq, Nk,
                     H, c, out, lse, opart, ml, plan.splits, plan.keys_per_split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  const int rows = H * Nq;
  hipLaunchKernelGGL((attn_merge_kernel<D>), dim3((rows + 7) / 8), dim3(256), 0, s, opart,
                     ml, Nq, H, plan.splits, out, lse);
  return hipGetLastError();
}

}  // namespace

// Split the key range only when the (q-tile, head) grid cannot give every CU
// two blocks; each split keeps >= 8 key tiles.
AttnPlan attention_plan(int Nq, int Nk, int H, int D, int num_cus) {
  (void)D;
  AttnPlan p;
  const long long tiles = (long long)((Nq + kBM - 1) / kBM) * H;
  const int kblocks = (Nk + kBN - 1) / kBN;
  int splits = 1;
  while (tiles * splits < 2LL * num_cus && kblocks / (splits * 2) >= 8) splits *= 2;
  const int kb_per = (kblocks + splits - 1) / splits;
  p.keys_per_split = kb_per * kBN;
  p.splits = (kblocks + kb_per - 1) / kb_per;
  return p;
}

size_t attention_ws_bytes(const AttnPlan& p, int Nq, int H, int D) {
  if (p.splits <= 1) return 0;
  return (size_t)p.splits * H * Nq * ((size_t)D * sizeof(float) + sizeof(float2));
}

hipError_t attention_launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, int Nq,
                            int Nk, int H, int D, float scale, uint16_t* out, float* lse,
                            const AttnPlan& plan, void* ws, hipStream_t s) {
  return (D == 128) ? launch<128>(q, k, v, Nq, Nk, H, scale, out, lse, plan, ws, s)
                    : launch<64>(q, k, v, Nq, Nk, H, scale, out, lse, plan, ws, s);
}

}  // namespace wkv
