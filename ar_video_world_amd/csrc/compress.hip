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
//            score kernel also writes the anchor rows of k_out, through a
//            per-wave LDS stage so that every store writes whole lines.
//            With the anchor-mean score (the section's equation: the mean
//            cosine to all T anchor tokens) two kernels run first instead:
//            anchor-mean sums, per run of anchor tokens of one unit (all
//            heads, so rows are written whole), the unit anchor keys k/|k|
//            in float64 and writes those anchor rows of k_out; a finalize
//            kernel adds the runs in a fixed order and divides by T. The mean of the cosines to every anchor token
//            is then one dot product, <k, abar> / |k|, so the score kernel
//            reads only the non-anchor rows and abar (kept in LDS).
//   select - one block per unit, sized to the pooled count (512 threads x 4
//            keys, 1024 x 4 or 1024 x 8): radix select of the n_keep-th smallest
//            (score, index) key, stable compaction by block scan, writes
//            kept_idx.
//   gather - one wave per output row: copies the kept K rows (non-anchor) and
//            all kept V rows with 16-byte loads and stores, all streaming
//            (plain loads of the K rows, which the score pass read before,
//            were 2 % slower).
#include <algorithm>
#include <mutex>

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

// int4 encoding of one 32-element group held by the 4 lanes of a quad, 8
// consecutive elements per lane in lane order: scale = bf16_RNE(max|x| / 7),
// code = clamp(rint(x / scale), -8, 7), or 0 when the scale is 0; both
// divisions are correctly rounded float32 and rint rounds half to even.
// Returns this lane's 4 bytes (element e in bits 4e..4e+3, so the low
// nibble of each byte holds the even element); *sbits gets the scale.
__device__ __forceinline__ uint32_t int4_encode_quad(const uint4& x, uint16_t* sbits) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  float v[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = bf16_to_f32(w[q] & 0xFFFFu);
    v[2 * q + 1] = bf16_to_f32(w[q] >> 16);
  }
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
  // Max over the quad with two row permutes (DPP quad_perm [1,0,3,2], then
  // [2,3,0,1]): lanes l^1, then l^2.
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1, 0xF, 0xF, true)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x4E, 0xF, 0xF, true)));
  // m / 7 correctly rounded, as one Newton step from m * RN(1/7): the residual
  // m - 7*y0 is exact, and the corrected quotient equals the correctly
  // rounded one for every bf16 m, subnormals included (checked exhaustively).
  constexpr float kInv7 = 1.0f / 7.0f;  // RN(1/7)
  const float y0 = m * kInv7;
  const float m7 = __builtin_isinf(m) ? m : fmaf(fmaf(-y0, 7.0f, m), kInv7, y0);
  const uint16_t sb = f32_to_bf16(m7);
  const float sc = bf16_to_f32(sb);
  uint32_t out = 0;
  if (sc != 0.f) {
    // inv is the correctly rounded 1/sc. k = rint(x * inv) is the nearest
    // integer to x / sc except at exact half-integers: x and sc carry 8-bit
    // significands, so any other quotient lies at least 1/1020 from a
    // half-integer, far beyond the error of x * inv. The residual
    // r = x - k*sc is exact (k has 4 bits), and k + r*inv lands exactly on
    // the half-integer at a tie and within 0.499 of k otherwise, so its rint
    // is the round-half-even quotient in every case (checked exhaustively
    // against exact rounding for all bf16 pairs with |x / sc| <= 7.02). A
    // scale so small that 1/sc overflows, or infinite, takes the division.
    // For finite groups |x / sc| <= 7 / (1 - 2^-9) < 7.5, so every code is in
    // [-7, 7]. Adding 1.5 * 2^23 + 8 rounds k + r*inv half-to-even to an
    // integer (the spacing of floats there is 1) and leaves code + 8, in
    // [1, 15], in the low mantissa bits with bits 4..21 clear. So two codes
    // pack into a byte with one shift-or, four bytes into a word with three
    // byte permutes, and flipping bit 3 of every nibble turns code + 8 into
    // the code's two's complement.
    const float inv = __fdiv_rn(1.0f, sc);
    if (inv < 3.0e38f && inv > 0.f) {
      uint32_t t[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float k = rintf(v[e] * inv);
        t[e] = __float_as_uint(fmaf(fmaf(-k, sc, v[e]), inv, k) + 12582920.0f);
      }
      uint32_t pb[4];  // byte 0 of each: codes 2j (low nibble) and 2j + 1
#pragma unroll
      for (int j = 0; j < 4; ++j) pb[j] = (t[2 * j + 1] << 4) | t[2 * j];
      const uint32_t lo = __builtin_amdgcn_perm(pb[1], pb[0], 0x0C0C0400u);  // [pb0.b0, pb1.b0, 0, 0]
      const uint32_t hi = __builtin_amdgcn_perm(pb[3], pb[2], 0x04000C0Cu);  // [0, 0, pb2.b0, pb3.b0]
      out = (lo | hi) ^ 0x88888888u;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float q = rintf(__fdiv_rn(v[e], sc));
        out |= ((uint32_t)(int)fminf(fmaxf(q, -8.f), 7.f) & 0xFu) << (4 * e);
      }
    }
  }
  *sbits = sb;
  return out;
}

// Where compressed rows go: bf16 rows, or int4 codes + bf16 group scales.
struct CompressOut {
  uint16_t* k;     // bf16 [B][Lc][H][D]
  uint16_t* v;
  uint8_t* kq;     // int4 [B][Lc][H][D/2]
  uint8_t* vq;
  uint16_t* ks;    // bf16 [B][Lc][H][D/32]
  uint16_t* vs;
};

// Wave-staged stores of the (row, head) slices held by the 16 quads of a
// wave. The quads hold 16 consecutive (row, head) pairs, so their output is
// one contiguous run: each active quad writes its slice (bf16 rows, or int4
// codes and scales) into the wave's LDS stage, then every lane stores whole
// 16-byte pieces of the run (the int4 scales as one 8- or 4-byte piece per
// pair), so each store instruction writes whole cache lines. Storing the
// slices from the quads directly wrote 16-byte pieces at 64- or 256-byte
// strides, partial lines that cost a 300-unit call of 3 x 880 x 12 x 128
// 110-170 us.
template <int NLD, bool Q4>
struct SliceStage {
  static constexpr int SLICE = Q4 ? NLD * 16 : NLD * 64;  // bytes per slice: codes, or bf16
  static constexpr int SCALE = NLD * 2;                   // int4 scale bytes per slice
  static constexpr int BYTES = 16 * (SLICE + (Q4 ? SCALE : 0));  // one wave's stage
};

// Every lane of the wave calls this (the stores are wave-wide). `active`:
// this quad holds a slice (quad-uniform); qw: the quad's index in the wave;
// nvalid: how many of the wave's 16 pairs are stored; e0: element offset of
// the wave's first pair in the output ((row*H + h)*D).
template <int NLD, bool Q4>
__device__ __forceinline__ void stage_store(const uint4 (&a)[NLD], bool active, int qw, int sub,
                                            int lane, uint8_t* stage, int nvalid, size_t e0,
                                            uint16_t* bf, uint8_t* pk, uint16_t* sc) {
  using SS = SliceStage<NLD, Q4>;
  if (active) {
    if constexpr (!Q4) {
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        *reinterpret_cast<uint4*>(stage + qw * SS::SLICE + i * 64 + sub * 16) = a[i];
    } else {
      uint8_t* scl = stage + 16 * SS::SLICE;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        uint16_t sb;
        const uint32_t p = int4_encode_quad(a[i], &sb);
        *reinterpret_cast<uint32_t*>(stage + qw * SS::SLICE + i * 16 + sub * 4) = p;
        if (sub == 0) *reinterpret_cast<uint16_t*>(scl + qw * SS::SCALE + i * 2) = sb;
      }
    }
  }
  // The wave's LDS writes land before its reads (LDS requests of one wave
  // complete in issue order; the wait also orders them for the compiler).
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  if constexpr (!Q4) {
    uint8_t* dst = reinterpret_cast<uint8_t*>(bf) + e0 * 2;
    for (int o = lane * 16; o < nvalid * SS::SLICE; o += kWave * 16)
      st_stream(dst + o, *reinterpret_cast<const uint4*>(stage + o));
  } else {
    uint8_t* dst = pk + e0 / 2;
    for (int o = lane * 16; o < nvalid * SS::SLICE; o += kWave * 16)
      st_stream(dst + o, *reinterpret_cast<const uint4*>(stage + o));
    const uint8_t* scl = stage + 16 * SS::SLICE;
    uint8_t* sdst = reinterpret_cast<uint8_t*>(sc) + e0 / 16;  // 2 bytes per 32 elements
    if (lane < nvalid) {
      if constexpr (SS::SCALE == 8)
        *reinterpret_cast<uint2*>(sdst + lane * 8) = *reinterpret_cast<const uint2*>(scl + lane * 8);
      else
        *reinterpret_cast<uint32_t*>(sdst + lane * 4) = *reinterpret_cast<const uint32_t*>(scl + lane * 4);
    }
  }
  // Every lane has read the stage before any quad writes it again.
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
}

// The anchor-mean kernel's per-head sums sit D + 1 doubles apart, so the
// quads writing them in one instruction (different heads, 64 bytes apart
// within a head) spread over the LDS banks two lanes deep instead of
// meeting on one bank per head (a stride of D doubles is a whole number of
// bank rounds: 6.6 conflict cycles per LDS instruction on 300 units of
// 3 x 880 x 12 x 128). The slice stages follow from the next 16 bytes.
__host__ __device__ inline size_t anchor_stage_offset(int H, int D) {
  return ((size_t)H * (D + 1) * sizeof(double) + 15) / 16 * 16;
}

// Anchor-mean blocks: 256 lanes, or 512 when 256 would leave over an eighth
// more of the quads idle (40 heads: 40 of 64 quads against 120 of 128) or
// cannot hold one quad per head.
int mean_block_threads(int H) {
  const int w256 = H <= 64 ? 64 % H : 64, w512 = 128 % H;
  return 2 * w256 > w512 + 16 ? 512 : 256;
}

// Anchor tokens per anchor-mean block: whole passes, doubled while a unit has
// more than 128 slices (the finalize kernel adds them in sequence) or the grid
// keeps >= 2048 blocks at twice the size.
int compress_mean_tokens(int B, int T, int H) {
  int mt = mean_block_threads(H) / kLanesPerPair / H;
  while (mt < T && ((T + mt - 1) / mt > 128 ||
                    (long long)B * ((T + 2 * mt - 1) / (2 * mt)) >= 2048))
    mt *= 2;
  return mt;
}

// grid: (nslice, B), block NT. Sum over a slice of mt anchor tokens of the
// unit anchor keys of every head (a zero key adds nothing), float64, into
// part[b][h][slice][D]; copies those anchor rows to k_out. 4 lanes own one
// (token, head) row slice of D elements, as in the score kernel, and each quad
// keeps one head: quad q takes head q % H of token q / H of every pass of
// P = (NT/4) / H consecutive tokens. The quads of a pass therefore cover
// whole rows, so the int4 codes and scales of a token leave as full cache
// lines (a block per head wrote 64-byte and 8-byte pieces of lines shared
// with other heads' blocks: 465 against 325 us for the bf16 store on 300
// units of 3 x 880 x 12 x 128). The P quads of a head add into LDS in a fixed
// order, so the result does not depend on timing.
// SUMS: bit 0 = the unit anchor keys (the anchor-mean score) into part,
// bit 1 = the anchor keys themselves (the compressed chunk's mean key) into
// rawpart, both [B][H][slices][D].
template <int D, bool Q4, int NT, int SUMS>
__global__ __launch_bounds__(NT) void compress_anchor_mean_kernel(
    const uint16_t* __restrict__ k, int F, int T, int H, int mt, double* __restrict__ part,
    double* __restrict__ rawpart, CompressOut out, int Lc) {
  constexpr int NLD = D / 32;
  constexpr int E = NLD * 8;  // elements per lane
  constexpr bool UNIT = SUMS & 1, RAW = SUMS & 2;
  constexpr int NQ = NT / kLanesPerPair;
  extern __shared__ double red[];  // [H][D + 1], then the waves' slice stages
  const int sl = blockIdx.x, b = blockIdx.y;
  const int P = NQ / H;  // tokens per pass (H <= NQ)
  const int j0 = sl * mt;
  const int ntok = min(mt, T - j0);
  const int tid = threadIdx.x;
  const int q = tid / kLanesPerPair;
  const int sub = tid % kLanesPerPair;
  const int t = q / H, h = q - t * H;
  const size_t HD = (size_t)H * D;
  const uint16_t* unit = k + (size_t)b * F * T * HD;
  const size_t ubase = (size_t)b * Lc * HD;  // element offset of this unit's output
  double acc[UNIT ? E : 1], raw[RAW ? E : 1];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if constexpr (UNIT) acc[e] = 0.0;
    if constexpr (RAW) raw[e] = 0.0;
  }
  // Every lane of a quad runs the same iterations (quad shuffles inside);
  // the next token's slice is loaded while this one is reduced.
  uint4 an[NLD];
  auto load_row = [&](int jl) {
    const size_t off = ((size_t)(j0 + jl) * H + h) * D + sub * 8;
#pragma unroll
    for (int i = 0; i < NLD; ++i) an[i] = *reinterpret_cast<const uint4*>(unit + off + i * 32);
  };
  // Quads past the last full head set idle. Passes run together over the
  // block (pass k takes tokens kP .. kP+P-1, all heads: P*H consecutive
  // (row, head) slices), so each wave's anchor slices leave through its stage.
  uint8_t* stage = reinterpret_cast<uint8_t*>(red) + anchor_stage_offset(H, D) +
                   (tid / kWave) * SliceStage<NLD, Q4>::BYTES;
  const int qw = q % 16;
  const int wq0 = q - qw;  // the wave's first quad
  if (t < P && t < ntok) load_row(t);
  for (int k0 = 0; k0 < ntok; k0 += P) {
    const int jl = k0 + t;
    const bool act = t < P && jl < ntok;
    uint4 a[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) a[i] = an[i];
    if (act && jl + P < ntok) load_row(jl + P);
    // this wave's slices: quads wq0 .. wq0+15 of the pass, while they hold a
    // token of the block
    const int nv = min(16, min(P * H, (ntok - k0) * H) - wq0);
    if (nv > 0)
      stage_store<NLD, Q4>(a, act, qw, sub, tid % kWave, stage, nv,
                           ubase + ((size_t)(j0 + k0) * H + wq0) * D, out.k, out.kq, out.ks);
    if (!act) continue;
    if constexpr (RAW) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const uint32_t w[4] = {a[i].x, a[i].y, a[i].z, a[i].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          raw[i * 8 + 2 * c] += (double)bf16_to_f32(w[c] & 0xFFFFu);
          raw[i * 8 + 2 * c + 1] += (double)bf16_to_f32(w[c] >> 16);
        }
      }
    }
    if constexpr (UNIT) {
      double na = 0.0;
#pragma unroll
      for (int i = 0; i < NLD; ++i) accum_sq(a[i], na);
      na = quad_sum(na);
      const double inv = (na == 0.0) ? 0.0 : 1.0 / sqrt(na);
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const uint32_t w[4] = {a[i].x, a[i].y, a[i].z, a[i].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[i * 8 + 2 * c] = fma((double)bf16_to_f32(w[c] & 0xFFFFu), inv, acc[i * 8 + 2 * c]);
          acc[i * 8 + 2 * c + 1] = fma((double)bf16_to_f32(w[c] >> 16), inv, acc[i * 8 + 2 * c + 1]);
        }
      }
    }
  }
  // Pass slot 0 writes each head's D sums, slots 1..P-1 add theirs in turn;
  // then the block's sums go to its slice of the partials.
  auto combine = [&](const double (&v)[E], double* out_part) {
    for (int r = 0; r < P; ++r) {
      if (t == r) {
#pragma unroll
        for (int i = 0; i < NLD; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            double* cell = red + h * (D + 1) + i * 32 + sub * 8 + e;
            *cell = (r == 0) ? v[i * 8 + e] : *cell + v[i * 8 + e];
          }
      }
      __syncthreads();
    }
    double* dst = out_part + (size_t)b * HD * gridDim.x;
    for (int i = tid; i < (int)HD; i += NT) {
      const int hh = i / D, d = i - hh * D;
      dst[((size_t)hh * gridDim.x + sl) * D + d] = red[hh * (D + 1) + d];
    }
    __syncthreads();  // red is reused by the next combine
  };
  if constexpr (UNIT) combine(acc, part);
  if constexpr (RAW) combine(raw, rawpart);
}

// grid: (H, B), block D. abar[b][h][d] = (sum over slices, in order) / T.
__global__ void compress_anchor_mean_final_kernel(const double* __restrict__ part, int nslice,
                                                  int T, int H, double* __restrict__ abar) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x, D = blockDim.x;
  const double* src = part + ((size_t)b * H + h) * nslice * D + d;
  // Eight loads in flight per round; the sum still runs in slice order.
  double t = 0.0;
  int s = 0;
  for (; s + 8 <= nslice; s += 8) {
    double x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = src[(size_t)(s + i) * D];
#pragma unroll
    for (int i = 0; i < 8; ++i) t += x[i];
  }
  for (; s < nslice; ++s) t += src[(size_t)s * D];
  abar[((size_t)b * H + h) * D + d] = t / (double)T;
}

// grid: (ceil(T / TT), B). Dynamic LDS: TT * (F-1) * H doubles, then (MEAN)
// H rows of D + kAbarSkew doubles holding abar, or (position score) from the
// next 16-byte boundary the 4 waves' slice stages.
constexpr int kAbarSkew = 2;

__host__ __device__ inline size_t score_stage_offset(int TT, int F, int H) {
  return ((size_t)TT * (F - 1) * H * sizeof(double) + 15) / 16 * 16;
}

template <int D, int F, bool MEAN, bool Q4>
__global__ __launch_bounds__(kScoreBlock) void compress_score_kernel(
    const uint16_t* __restrict__ k, int T, int H, int TT,
    double* __restrict__ scores, CompressOut out, int Lc,
    const double* __restrict__ abar_g) {
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
  const size_t ubase = (size_t)b * Lc * HD;  // element offset of this unit's output

  if constexpr (MEAN) {
    // abar rows sit kAbarSkew doubles apart beyond D, so the quads of a
    // wave (consecutive heads) read distinct LDS banks.
    double* abar = cosbuf + (size_t)TT * (F - 1) * H;
    uint4 x[F - 1][NLD];
    auto load_rows = [&](int pr) {
      const int jl = pr / H;
      const int h = pr - jl * H;
#pragma unroll
      for (int f = 1; f < F; ++f) {
        const size_t off = (((size_t)f * T + j0 + jl) * H + h) * D + sub * 8;
#pragma unroll
        for (int i = 0; i < NLD; ++i)
          x[f - 1][i] = *reinterpret_cast<const uint4*>(unit + off + i * 32);
      }
    };
    // The first rows are in flight while abar is staged.
    if (slot < npairs) load_rows(slot);
    const double* src = abar_g + (size_t)b * HD;
    for (int i = tid; i < (int)HD; i += kScoreBlock)
      abar[(i / D) * (D + kAbarSkew) + i % D] = src[i];
    __syncthreads();
    // Every lane of a quad runs the same number of iterations (quad shuffles).
    for (int pair = slot; pair < npairs; pair += kPairsPerPass) {
      const int jl = pair / H;
      const int h = pair - jl * H;
      double av[NLD * 8];
      const double* ah = abar + h * (D + kAbarSkew) + sub * 8;
#pragma unroll
      for (int i = 0; i < NLD; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) av[i * 8 + e] = ah[i * 32 + e];
      uint4 xc[F - 1][NLD];
#pragma unroll
      for (int f = 0; f < F - 1; ++f)
#pragma unroll
        for (int i = 0; i < NLD; ++i) xc[f][i] = x[f][i];
      if (pair + kPairsPerPass < npairs) load_rows(pair + kPairsPerPass);  // next rows
#pragma unroll
      for (int f = 1; f < F; ++f) {
        double dt = 0.0, nk = 0.0;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const uint32_t w[4] = {xc[f - 1][i].x, xc[f - 1][i].y, xc[f - 1][i].z, xc[f - 1][i].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const double xl = (double)bf16_to_f32(w[q] & 0xFFFFu);
            const double xh = (double)bf16_to_f32(w[q] >> 16);
            nk = fma(xl, xl, nk);
            nk = fma(xh, xh, nk);
            dt = fma(xl, av[i * 8 + 2 * q], dt);
            dt = fma(xh, av[i * 8 + 2 * q + 1], dt);
          }
        }
        dt = quad_sum(dt);
        nk = quad_sum(nk);
        if (sub == 0) cosbuf[(jl * (F - 1) + (f - 1)) * H + h] = (nk == 0.0) ? 0.0 : dt / sqrt(nk);
      }
    }
  } else {
    // Rows of the next pair are loaded while this pair is reduced.
    uint4 a[NLD];
    uint4 x[F - 1][NLD];
    auto load_rows = [&](int pr) {
      const int jl = pr / H;
      const int h = pr - jl * H;
      const int j = j0 + jl;
      const size_t aoff = ((size_t)j * H + h) * D + sub * 8;
#pragma unroll
      for (int i = 0; i < NLD; ++i) a[i] = *reinterpret_cast<const uint4*>(unit + aoff + i * 32);
#pragma unroll
      for (int f = 1; f < F; ++f) {
        const size_t off = (((size_t)f * T + j) * H + h) * D + sub * 8;
#pragma unroll
        for (int i = 0; i < NLD; ++i)
          x[f - 1][i] = *reinterpret_cast<const uint4*>(unit + off + i * 32);
      }
    };
    if (slot < npairs) load_rows(slot);
    // Each wave walks its passes together (the anchor slices leave through
    // the wave's stage); a quad with no pair in a pass only joins the store.
    // The 4 lanes of a quad always agree, so the quad shuffles below always
    // see their partners.
    uint8_t* stage = reinterpret_cast<uint8_t*>(cosbuf) + score_stage_offset(TT, F, H) +
                     (tid / kWave) * SliceStage<NLD, Q4>::BYTES;
    const int qw = slot % 16;
    for (int pw = slot - qw; pw < npairs; pw += kPairsPerPass) {
      const int pair = pw + qw;
      const bool act = pair < npairs;
      const int jl = pair / H;
      const int h = pair - jl * H;
      uint4 ac[NLD];
      uint4 xc[F - 1][NLD];
#pragma unroll
      for (int i = 0; i < NLD; ++i) ac[i] = a[i];
#pragma unroll
      for (int f = 0; f < F - 1; ++f)
#pragma unroll
        for (int i = 0; i < NLD; ++i) xc[f][i] = x[f][i];
      if (act && pair + kPairsPerPass < npairs) load_rows(pair + kPairsPerPass);
      stage_store<NLD, Q4>(ac, act, qw, sub, tid % kWave, stage, min(16, npairs - pw),
                           ubase + ((size_t)j0 * H + pw) * D, out.k, out.kq, out.ks);
      if (!act) continue;
      double na = 0.0;
#pragma unroll
      for (int i = 0; i < NLD; ++i) accum_sq(ac[i], na);
      na = quad_sum(na);
#pragma unroll
      for (int f = 1; f < F; ++f) {
        double dt = 0.0, nk = 0.0;
#pragma unroll
        for (int i = 0; i < NLD; ++i) accum_dot_sq(xc[f - 1][i], ac[i], dt, nk);
        dt = quad_sum(dt);
        nk = quad_sum(nk);
        if (sub == 0) {
          const double prod = nk * na;
          const double c = (prod == 0.0) ? 0.0 : dt / sqrt(prod);
          cosbuf[(jl * (F - 1) + (f - 1)) * H + h] = c;
        }
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

// Select block: 512 threads with 4 keys each up to 2048 pooled tokens (short
// per-thread chains in the histogram passes: 11.3 us against 14.6 us for 256
// threads x 8 keys on one 1760-token unit), 1024 x 4 and 1024 x 8 beyond.

// grid: B. Writes kept_idx[b][0..Lc).
template <int kSelBlock, int kSelKPT>
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

// One wave per block and one output row per wave: many small blocks keep
// more rows in flight than fewer wide ones (a 300-unit batch at r = 1 copies
// at 5.9 TB/s this way, 5.3 TB/s with 4-wave blocks of 4 rows per wave).
constexpr int kGatherBlock = 64;
// 16-byte chunks each lane loads before it stores any (a whole 12 x 128 row).
constexpr int kGatherUnroll = 3;

// grid: (Lc, B, 2). z = 0 copies K rows (rows below k_skip are skipped: the
// score kernel already wrote them), z = 1 copies V rows. cpr = 16-byte chunks
// (8 elements) per row, a multiple of 4; with int4 output the 4 lanes holding
// one 32-element group encode it together. Every load and store streams
// (nontemporal): no source or output row is read again by this step. For the
// int4 store that matters most: its 4-byte code and 2-byte scale stores as
// plain stores held a 300-unit batch at r = 1 to 0.56 of HBM peak, against
// 0.70 streamed.
// z0 = 1 launches the V rows only (grid z = 1).
template <bool Q4>
__global__ __launch_bounds__(kGatherBlock) void compress_gather_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ kept_idx, int FT, int Lc, int cpr, int k_skip,
    CompressOut out, int z0) {
  const int b = blockIdx.y;
  const bool isk = blockIdx.z + z0 == 0;
  const int row = blockIdx.x;
  if (row >= Lc || (isk && row < k_skip)) return;  // whole block
  const uint4* src = reinterpret_cast<const uint4*>(isk ? k : v) +
                     ((size_t)b * FT + kept_idx[(size_t)b * Lc + row]) * cpr;
  const size_t ro = ((size_t)b * Lc + row) * cpr;  // output row, in chunks
  const int lane = threadIdx.x;
  for (int c0 = lane; c0 < cpr; c0 += 64 * kGatherUnroll) {
    uint4 x[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int c = c0 + 64 * u;
      x[u] = c < cpr ? ld_stream(src + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int c = c0 + 64 * u;
      if (c >= cpr) continue;  // uniform over each quad (cpr % 4 == 0)
      if constexpr (!Q4) {
        st_stream(reinterpret_cast<uint4*>(isk ? out.k : out.v) + ro + c, x[u]);
      } else {
        uint16_t sb;
        const uint32_t p = int4_encode_quad(x[u], &sb);  // every lane of the quad
        __builtin_nontemporal_store(p, reinterpret_cast<uint32_t*>(isk ? out.kq : out.vq) + ro + c);
        if ((c & 3) == 0) __builtin_nontemporal_store(sb, (isk ? out.ks : out.vs) + (ro + c) / 4);
      }
    }
  }
}

// K rows of the compressed chunk with their float64 sum, for the mean key.
// grid: (runs, column slices, B); kKsumWaves waves per block. A block takes
// output rows [r_first + run * kKsumWaves * rw, + kKsumWaves * rw) of its
// unit over one slice of 64 * kGatherUnroll 16-byte chunks (8 elements
// each); wave w takes every kKsumWaves-th row from the w-th, copies it to the
// output when its index is >= store_from (rows below were written by the
// score kernel: bf16, or int4 encoded as in the gather kernel) and adds it
// into float64 sums, 8 per chunk and lane. Each wave keeps its next two rows
// in flight. The waves' sums then meet in one LDS row, added in wave order,
// so ksum[b][run][chunk*8 ..] is a deterministic partial, added in run order
// by the finalize kernel.
constexpr int kKsumWaves = 4;
constexpr int kKsumBlock = kKsumWaves * kWave;

template <bool Q4>
__global__ __launch_bounds__(kKsumBlock) void compress_gather_ksum_kernel(
    const uint16_t* __restrict__ k, const int32_t* __restrict__ kept_idx, int FT, int Lc,
    int cpr, int r_first, int rw, int store_from, CompressOut out, double* __restrict__ ksum) {
  __shared__ double red[64 * kGatherUnroll * 8];
  const int run = blockIdx.x, cs = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  const int blk0 = r_first + run * kKsumWaves * rw;
  const int row1 = min(Lc, blk0 + kKsumWaves * rw);
  const int c0 = cs * 64 * kGatherUnroll + lane;
  const uint4* src_unit = reinterpret_cast<const uint4*>(k) + (size_t)b * FT * cpr;
  const int32_t* ki = kept_idx + (size_t)b * Lc;
  double acc[kGatherUnroll][8];
#pragma unroll
  for (int u = 0; u < kGatherUnroll; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[u][e] = 0.0;
  auto load = [&](int row, uint4 (&dst)[kGatherUnroll]) {
    const uint4* src = src_unit + (size_t)ki[row] * cpr;
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int c = c0 + 64 * u;
      dst[u] = c < cpr ? ld_stream(src + c) : make_uint4(0, 0, 0, 0);
    }
  };
  constexpr int S = kKsumWaves;  // row stride of a wave
  const int row0 = blk0 + wv;
  uint4 n1[kGatherUnroll], n2[kGatherUnroll];
  if (row0 < row1) load(row0, n1);
  if (row0 + S < row1) load(row0 + S, n2);
  for (int row = row0; row < row1; row += S) {
    uint4 x[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      x[u] = n1[u];
      n1[u] = n2[u];
    }
    if (row + 2 * S < row1) load(row + 2 * S, n2);
    const size_t ro = ((size_t)b * Lc + row) * cpr;
    const bool st = row >= store_from;
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int c = c0 + 64 * u;
      if (c >= cpr) continue;  // uniform over each quad (cpr % 4 == 0, slices of 192)
      if (st) {
        if constexpr (!Q4) {
          st_stream(reinterpret_cast<uint4*>(out.k) + ro + c, x[u]);
        } else {
          uint16_t sb;
          const uint32_t p = int4_encode_quad(x[u], &sb);
          __builtin_nontemporal_store(p, reinterpret_cast<uint32_t*>(out.kq) + ro + c);
          if ((c & 3) == 0) __builtin_nontemporal_store(sb, out.ks + (ro + c) / 4);
        }
      }
      const uint32_t w[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[u][2 * q] += (double)bf16_to_f32(w[q] & 0xFFFFu);
        acc[u][2 * q + 1] += (double)bf16_to_f32(w[q] >> 16);
      }
    }
  }
  // wave 0 writes its sums, waves 1 .. kKsumWaves-1 add theirs in turn
  for (int j = 0; j < kKsumWaves; ++j) {
    if (wv == j) {
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          double* cell = red + (u * 64 + lane) * 8 + e;
          *cell = (j == 0) ? acc[u][e] : *cell + acc[u][e];
        }
    }
    __syncthreads();
  }
  double* dst = ksum + ((size_t)b * gridDim.x + run) * (size_t)cpr * 8;
  const int nval = min(cpr - cs * 64 * kGatherUnroll, 64 * kGatherUnroll) * 8;
  for (int i = threadIdx.x; i < nval; i += kKsumBlock)
    dst[(size_t)cs * 64 * kGatherUnroll * 8 + i] = red[i];
}

// grid: (H, B), block D * kFinalGroups. key_mean[b][h][d] = (sum of the
// partials) / Lc, the partials being the anchor-row slices apart[b][h][s][d]
// (s < nslice) followed by the kept-row runs ksum[b][r][h*D + d] (r < nruns).
// Group g adds partials g, g + G, ... in order, four loads in flight; the
// groups' sums are then added in group order.
constexpr int kFinalGroups = 8;

__global__ __launch_bounds__(128 * kFinalGroups) void compress_key_mean_final_kernel(
    const double* __restrict__ apart, int nslice, const double* __restrict__ ksum, int nruns,
    int Lc, int H, double* __restrict__ key_mean) {
  __shared__ double red[kFinalGroups][128];
  const int h = blockIdx.x, b = blockIdx.y;
  const int D = blockDim.x / kFinalGroups;
  const int d = threadIdx.x % D, g = threadIdx.x / D;
  const size_t HD = (size_t)H * D;
  const double* ap = nslice > 0 ? apart + ((size_t)b * H + h) * nslice * D + d : nullptr;
  const double* kp = nruns > 0 ? ksum + (size_t)b * nruns * HD + (size_t)h * D + d : nullptr;
  auto part = [&](int p) { return p < nslice ? ap[(size_t)p * D] : kp[(size_t)(p - nslice) * HD]; };
  const int n = nslice + nruns;
  double t = 0.0;
  int p = g;
  for (; p + 3 * kFinalGroups < n; p += 4 * kFinalGroups) {
    double x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = part(p + i * kFinalGroups);
#pragma unroll
    for (int i = 0; i < 4; ++i) t += x[i];
  }
  for (; p < n; p += kFinalGroups) t += part(p);
  red[g][d] = t;
  __syncthreads();
  if (g > 0) return;
  double s = red[0][d];
#pragma unroll
  for (int j = 1; j < kFinalGroups; ++j) s += red[j][d];
  key_mean[((size_t)b * H + h) * D + d] = s / (double)Lc;
}

template <int D, int F>
hipError_t launch_score(const uint16_t* k, int B, int T, int H, int TT, double* scores,
                        const CompressOut& out, bool q4, int Lc, const double* abar,
                        hipStream_t s) {
  dim3 grid((T + TT - 1) / TT, B);
  const size_t cos_lds = (size_t)TT * (F - 1) * H * sizeof(double);
  const size_t stage_lds = score_stage_offset(TT, F, H);
  constexpr int NLD = D / 32;
  constexpr int W = kScoreBlock / kWave;
  if (abar) {  // the anchor-mean kernel has stored the anchor rows
    const size_t lds = cos_lds + (size_t)H * (D + kAbarSkew) * sizeof(double);
    hipLaunchKernelGGL((compress_score_kernel<D, F, true, false>), grid, dim3(kScoreBlock), lds,
                       s, k, T, H, TT, scores, out, Lc, abar);
  } else if (q4) {
    const size_t lds = stage_lds + W * SliceStage<NLD, true>::BYTES;
    hipLaunchKernelGGL((compress_score_kernel<D, F, false, true>), grid, dim3(kScoreBlock), lds,
                       s, k, T, H, TT, scores, out, Lc, abar);
  } else {
    const size_t lds = stage_lds + W * SliceStage<NLD, false>::BYTES;
    hipLaunchKernelGGL((compress_score_kernel<D, F, false, false>), grid, dim3(kScoreBlock),
                       lds, s, k, T, H, TT, scores, out, Lc, abar);
  }
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_score_F(const uint16_t* k, int B, int F, int T, int H, int TT,
                            double* scores, const CompressOut& out, bool q4, int Lc,
                            const double* abar, hipStream_t s) {
  switch (F) {
    case 2: return launch_score<D, 2>(k, B, T, H, TT, scores, out, q4, Lc, abar, s);
    case 3: return launch_score<D, 3>(k, B, T, H, TT, scores, out, q4, Lc, abar, s);
    case 4: return launch_score<D, 4>(k, B, T, H, TT, scores, out, q4, Lc, abar, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int NT, int SUMS>
void launch_anchor_mean_sums(const uint16_t* k, int B, int F, int T, int H, double* part,
                             double* rawpart, const CompressOut& out, bool q4, int Lc,
                             hipStream_t s) {
  const int mt = compress_mean_tokens(B, T, H);
  const dim3 grid((T + mt - 1) / mt, B);
  constexpr int W = NT / kWave;
  const size_t lds = anchor_stage_offset(H, D) +
                     W * (q4 ? SliceStage<D / 32, true>::BYTES : SliceStage<D / 32, false>::BYTES);
  if (q4)
    hipLaunchKernelGGL((compress_anchor_mean_kernel<D, true, NT, SUMS>), grid, dim3(NT), lds, s,
                       k, F, T, H, mt, part, rawpart, out, Lc);
  else
    hipLaunchKernelGGL((compress_anchor_mean_kernel<D, false, NT, SUMS>), grid, dim3(NT), lds, s,
                       k, F, T, H, mt, part, rawpart, out, Lc);
}

// part: unit-key sums for the anchor-mean score; rawpart: anchor key sums
// for the mean key, or null.
template <int D, int NT>
void launch_anchor_mean_nt(const uint16_t* k, int B, int F, int T, int H, double* part,
                           double* rawpart, const CompressOut& out, bool q4, int Lc,
                           hipStream_t s) {
  if (rawpart)
    launch_anchor_mean_sums<D, NT, 3>(k, B, F, T, H, part, rawpart, out, q4, Lc, s);
  else
    launch_anchor_mean_sums<D, NT, 1>(k, B, F, T, H, part, rawpart, out, q4, Lc, s);
}

template <int D>
void launch_anchor_mean(const uint16_t* k, int B, int F, int T, int H, double* part,
                        double* rawpart, const CompressOut& out, bool q4, int Lc, hipStream_t s) {
  if (mean_block_threads(H) == 512)
    launch_anchor_mean_nt<D, 512>(k, B, F, T, H, part, rawpart, out, q4, Lc, s);
  else
    launch_anchor_mean_nt<D, 256>(k, B, F, T, H, part, rawpart, out, q4, Lc, s);
}

}  // namespace

// Tokens per score block: as many as one pass of (token, head) pairs holds
// (5 at 12 heads: one unit of 880 tokens spreads over 176 blocks, each done
// in one round of loads). When each block has fixed work to spread over more
// tokens (encoding the anchor rows to int4, or staging the anchor mean in
// LDS) the tile starts from the smallest that covers a full pass and grows
// while the grid still has >= 2048 blocks. On 300 units of
// 3 x 880 x 12 x 128, growth took the int4 batch from 0.45 to 0.49 of HBM
// peak and the anchor-mean batch from 0.58 to 0.64, while the position-mode
// bf16 batch ran 1-4 % faster on the smallest tile.
int compress_score_tile(int B, int T, int H, bool grow) {
  int tt = grow ? (kPairsPerPass + H - 1) / H : (H >= kPairsPerPass ? 1 : kPairsPerPass / H);
  while (grow && tt * 2 <= 64 && tt * 2 * H <= 512 &&
         (long long)((T + tt * 2 - 1) / (tt * 2)) * B >= 2048)
    tt *= 2;
  return tt < T ? tt : T;
}

// Workspace of wkv_compress_chunk_noalloc, for callers that cannot allocate
// (code under graph capture, serving loops, harnesses that forbid it): every
// GPU the library runs on holds its own copy until the process ends. In host
// code the array's name is not a device address; its address on the current
// device comes from hipGetSymbolAddress, resolved once per device.
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kScratchDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};
}  // namespace

size_t compress_scratch_bytes() { return kScratchBytes; }

hipError_t compress_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

int compress_mean_slices(int B, int T, int H) {
  const int mt = compress_mean_tokens(B, T, H);
  return (T + mt - 1) / mt;
}

size_t compress_anchor_lds_bytes(int H, int D, bool q4) {
  const int W = mean_block_threads(H) / kWave;
  const size_t stage = D == 128 ? (q4 ? SliceStage<4, true>::BYTES : SliceStage<4, false>::BYTES)
                                : (q4 ? SliceStage<2, true>::BYTES : SliceStage<2, false>::BYTES);
  return anchor_stage_offset(H, D) + W * stage;
}

size_t compress_score_lds_bytes(int B, int F, int T, int H, int D, bool mean, bool q4) {
  const int TT = compress_score_tile(B, T, H, q4 || mean);
  if (mean) return ((size_t)TT * (F - 1) * H + (size_t)H * (D + kAbarSkew)) * sizeof(double);
  const int W = kScoreBlock / kWave;
  const size_t stage = D == 128 ? (q4 ? SliceStage<4, true>::BYTES : SliceStage<4, false>::BYTES)
                                : (q4 ? SliceStage<2, true>::BYTES : SliceStage<2, false>::BYTES);
  return score_stage_offset(TT, F, H) + W * stage;
}

int compress_key_slices(int cpr) { return (cpr + 64 * kGatherUnroll - 1) / (64 * kGatherUnroll); }

// Rows per wave of the summing gather: each block writes one partial row of
// H*D doubles, 4 / (kKsumWaves * rw) of the bytes it reads, so rw starts at 4
// and doubles (to 32) while the grid keeps >= 1024 blocks.
int compress_key_rw(int B, int rows, int cpr) {
  const long long ncs = compress_key_slices(cpr);
  int rw = 4;
  while (rw < 32 &&
         (long long)B * ncs * ((rows + 2 * kKsumWaves * rw - 1) / (2 * kKsumWaves * rw)) >= 1024)
    rw *= 2;
  return rw;
}

int compress_key_runs(int B, int rows, int cpr) {
  const int per = kKsumWaves * compress_key_rw(B, rows, cpr);
  return (rows + per - 1) / per;
}

int compress_key_runs_max(int B, int F, int T, int cpr) {
  int m = 0;
  for (int rows = 1; rows <= F * T; ++rows) m = std::max(m, compress_key_runs(B, rows, cpr));
  return m;
}

hipError_t compress_launch(const uint16_t* k, const uint16_t* v, int B, int F,
                           int T, int H, int D, int n_keep, const CompressDst& dst,
                           int32_t* kept_idx, double* scores, bool need_scores,
                           double* mean_part, double* abar, const KeyMeanWs& km,
                           hipStream_t s) {
  const bool q4 = dst.k_packed != nullptr;
  const CompressOut out{dst.k, dst.v, dst.k_packed, dst.v_packed, dst.k_scale, dst.v_scale};
  const int N = (F - 1) * T;
  const int Lc = T + n_keep;
  const int cpr = H * D / 8;
  const bool score = need_scores || (n_keep > 0 && n_keep < N);
  const bool kmean = km.key_mean != nullptr;
  hipError_t e = hipSuccess;
  // The anchor-mean score adds the anchor rows themselves beside their unit
  // keys for the mean key (no extra read); otherwise the summing gather adds
  // them, reading them again.
  const bool araw = kmean && abar != nullptr;
  if (score) {
    if (abar) {  // the anchor-mean kernel also writes the anchor rows
      if (D == 128)
        launch_anchor_mean<128>(k, B, F, T, H, mean_part, araw ? km.araw : nullptr, out, q4, Lc, s);
      else
        launch_anchor_mean<64>(k, B, F, T, H, mean_part, araw ? km.araw : nullptr, out, q4, Lc, s);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL(compress_anchor_mean_final_kernel, dim3(H, B), dim3(D), 0, s,
                         mean_part, compress_mean_slices(B, T, H), T, H, abar);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int TT = compress_score_tile(B, T, H, q4 || abar != nullptr);
    e = (D == 128) ? dispatch_score_F<128>(k, B, F, T, H, TT, scores, out, q4, Lc, abar, s)
                   : dispatch_score_F<64>(k, B, F, T, H, TT, scores, out, q4, Lc, abar, s);
    if (e != hipSuccess) return e;
  }
  if (N <= 2048)
    hipLaunchKernelGGL((compress_select_kernel<512, 4>), dim3(B), dim3(512), 0, s, scores, N, T,
                       n_keep, kept_idx, Lc);
  else if (N <= 4096)
    hipLaunchKernelGGL((compress_select_kernel<1024, 4>), dim3(B), dim3(1024), 0, s, scores, N, T,
                       n_keep, kept_idx, Lc);
  else
    hipLaunchKernelGGL((compress_select_kernel<1024, 8>), dim3(B), dim3(1024), 0, s, scores, N, T,
                       n_keep, kept_idx, Lc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int k_first = score ? T : 0;  // K rows the gather writes (the rest are anchor rows)
  if (!kmean) {
    dim3 grid(Lc, B, 2);
    if (q4)
      hipLaunchKernelGGL(compress_gather_kernel<true>, grid, dim3(kGatherBlock), 0, s, k, v,
                         kept_idx, F * T, Lc, cpr, k_first, out, 0);
    else
      hipLaunchKernelGGL(compress_gather_kernel<false>, grid, dim3(kGatherBlock), 0, s, k, v,
                         kept_idx, F * T, Lc, cpr, k_first, out, 0);
    return hipGetLastError();
  }
  // Mean key: V rows by the gather; K rows by the summing gather, which
  // copies rows from k_first on and adds rows from r_first on.
  dim3 vgrid(Lc, B, 1);
  if (q4)
    hipLaunchKernelGGL(compress_gather_kernel<true>, vgrid, dim3(kGatherBlock), 0, s, k, v,
                       kept_idx, F * T, Lc, cpr, 0, out, 1);
  else
    hipLaunchKernelGGL(compress_gather_kernel<false>, vgrid, dim3(kGatherBlock), 0, s, k, v,
                       kept_idx, F * T, Lc, cpr, 0, out, 1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int r_first = araw ? T : 0;
  const int rows = Lc - r_first;
  const int rw = compress_key_rw(B, rows, cpr);
  const int nruns = compress_key_runs(B, rows, cpr);
  if (nruns > 0) {
    dim3 kgrid(nruns, compress_key_slices(cpr), B);
    if (q4)
      hipLaunchKernelGGL(compress_gather_ksum_kernel<true>, kgrid, dim3(kKsumBlock), 0, s, k,
                         kept_idx, F * T, Lc, cpr, r_first, rw, k_first, out, km.ksum);
    else
      hipLaunchKernelGGL(compress_gather_ksum_kernel<false>, kgrid, dim3(kKsumBlock), 0, s, k,
                         kept_idx, F * T, Lc, cpr, r_first, rw, k_first, out, km.ksum);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(compress_key_mean_final_kernel, dim3(H, B), dim3(D * kFinalGroups), 0, s,
                     km.araw, araw ? compress_mean_slices(B, T, H) : 0, km.ksum, nruns, Lc, H,
                     km.key_mean);
  return hipGetLastError();
}

}  // namespace wkv
