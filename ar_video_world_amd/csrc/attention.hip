// Chunk attention (WorldAttention: scaled dot-product attention of the
// current chunk's queries over the visible keys, scaled by 1/sqrt(d), run at
// every denoising step; its kernel section streams key/value tiles with an
// online softmax: running max m, denominator l, unnormalised output o).
//
// gfx950 design. One block = 4 waves = 128 queries of one head; each wave owns
// 32 queries and walks the key range in tiles of 64 keys.
//   * K/V tiles go from global memory straight into LDS with raw buffer loads
//     (buffer_load ... lds): no register staging, no VALU, rows past the
//     window read as zero. K is staged one tile ahead of V in two K and two V
//     stages, each its own LDS array, so the compiler can see that loads in
//     flight never alias the stages being read.
//   * S^T = K_tile * Q^T on v_mfma_f32_32x32x16_bf16: the 32x32 accumulator
//     layout puts one query per lane column, so the softmax row statistics of
//     a query live in two lanes (lane, lane^32), combined by v_permlane32_swap.
//   * The rows of each 32-key MFMA tile are fed in a fixed permutation of the
//     keys chosen so that accumulator elements 8m..8m+7 of a lane are exactly
//     the 8 consecutive keys that lane must supply as the B operand of the
//     P*V MFMA: P^T goes from accumulator to operand by a bf16 conversion, with
//     no shuffle. The same permutation indexes V^T, so the sum is unchanged.
//   * O^T += V^T * P^T on the same MFMA; the V^T operand comes from row-major V
//     in LDS through transposing reads (ds_read_b64_tr_b16).
//   * K and V rows in LDS use XOR swizzles of 16-byte chunks so that the row
//     reads and the transposing reads are free of bank conflicts.
//   * Softmax in base 2 with a fixed per-row reference: p = exp2(s*c - mref),
//     c = scale*log2(e), converted to bf16, and the row sum is a bf16 dot2 of
//     exactly the weights the P*V product uses. There is no per-tile row max:
//     the first tile of a block's key range sets mref to that tile's row max
//     before the key loop (so the row sum is >= 1 from then on and cannot
//     underflow), and after
//     that a range guard on the tile's row sums (rare branch) moves mref up
//     only when some weight would approach the fp32/bf16 range. O and l
//     always share mref, so the result does not depend on where it sits.
//   * While a wave issues its P*V MFMAs it runs at raised priority, so when
//     the two waves sharing a SIMD are in different phases the MFMA-dense one
//     issues first and the other's softmax VALU fills the gaps.
//   * The S^T product of tile t+1 is issued ahead of the softmax of tile t,
//     so one wave has MFMA work independent of its VALU work.
//   * Long key ranges with few query tiles are split over blocks; each split
//     writes unnormalised fp32 partials plus (m, l) and a merge kernel
//     combines them with the log-sum-exp identity.
//   * Blocks are renumbered so that each XCD (blocks are dealt round-robin
//     over the 8 XCDs) works on a contiguous range of (head, split, q-tile):
//     tiles sharing K/V share that XCD's L2.
//   * The same kernel also reads the window in place (WorldAttention's
//     kernel section counts the contiguous KV copy among its main costs):
//     the window's pieces (sink, retrieved bank chunks, recent segments,
//     current) are padded to whole tiles, a small kernel writes one entry per
//     tile (its rows in K and V, and its real keys), and the key loop takes
//     each tile's loads from that entry instead of from one contiguous array.
#include <cstring>

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
constexpr float kBigSum = 1073741824.0f;     // 2^30: largest accepted tile row sum

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef int i32x4 __attribute__((ext_vector_type(4)));
// Raw buffer descriptor (stride 0): loads at byte offsets >= nrec return 0.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t nrec) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nrec,
                                           0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

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
struct Tile {
  static constexpr int KCH = D / 8;                       // 16-byte chunks per row
  static constexpr int ROW = D * 2;                       // bytes per row of one head
  static constexpr int BYTES = kBN * ROW;                 // one K or V tile
  static constexpr int STAGE = 2 * BYTES;                 // K tile, then V tile
  static constexpr int ROWS_PER_LOAD = 1024 / ROW;        // rows per wave-wide 1 KiB load
  static constexpr int LOADS = BYTES / 1024 / (kThreads / 64);  // per wave and operand
};

// V rows: chunk c of key r is stored at position c ^ vswz(r). The transpose
// reads of the P*V operand touch 4 consecutive keys x one 64-byte quarter of
// the row per half-wave; the rotation puts those 4 quarters on disjoint banks.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * (r & 1);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// 16 bytes per lane from global (raw buffer, zero past nrec) straight into
// LDS at lds + 16 * lane.
__device__ __forceinline__ void buffer_load_lds16(rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group the
// lanes' 4-element chunks are concatenated and lane j receives elements j,
// j+16, j+32, j+48 of that sequence.
__device__ __forceinline__ uint2 lds_read_tr(const uint8_t* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  return __builtin_bit_cast(uint2, v);
}

// max over the lane pair (l, l ^ 32) with one VALU lane swap.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One 64-key tile t of the window read in place, as two 32-byte halves. The
// first holds what iteration t of the key loop needs in one scalar load: the
// K rows of tile t+2 and the V rows of tile t+1 (head 0; the loop queues
// those two loads), how many rows their pieces still have from there (0 for
// a bank id outside the bank: the tile reads as zero rows), and how many of
// tile t's 64 keys are real (the rest is padding, masked). The second holds
// tile t's own rows, for the loads queued before the loop.
struct __attribute__((aligned(32))) TileEntry {
  const uint16_t* k_next2;
  const uint16_t* v_next1;
  int32_t rows_next2;
  int32_t rows_next1;
  int32_t nvalid;
  int32_t rows;
  const uint16_t* k;
  const uint16_t* v;
  int64_t pad[2];
};

// The piece table is the first kernel argument and is read where it lies in
// the kernel-argument segment; indexing a by-value copy at a run-time index
// would put it in scratch memory.
typedef const __attribute__((address_space(4))) WinPieces* kernarg_pieces;

// One thread per tile of the padded key space: resolves the pieces of tiles
// t, t+1 and t+2 (and their bank ids) once per call.
__device__ __forceinline__ void resolve_tile(kernarg_pieces win, int64_t HD, int t,
                                             const uint16_t** k, const uint16_t** v,
                                             int* rows, int* nvalid) {
  if (t >= win->tile0[win->npieces]) {
    *k = nullptr;
    *v = nullptr;
    *rows = 0;
    *nvalid = 0;
    return;
  }
  int pc = 0;
  while (pc + 1 < win->npieces && t >= win->tile0[pc + 1]) ++pc;
  const int row0 = (t - win->tile0[pc]) * kBN;
  int64_t r0 = row0;
  int n = win->n[pc] - row0;
  if (win->slot[pc] >= 0) {
    const int id = win->idx[win->slot[pc]];
    if (id >= 0 && id < win->M) r0 += (int64_t)id * win->Lc;
    else n = 0;
  }
  *k = win->k[pc] + r0 * HD;
  *v = win->v[pc] + r0 * HD;
  *rows = n;
  *nvalid = min(kBN, win->n[pc] - row0);
}

__global__ __launch_bounds__(256) void attn_tile_table_kernel(const WinPieces win_arg,
                                                               int64_t HD,
                                                               TileEntry* __restrict__ tab) {
  const kernarg_pieces win = (kernarg_pieces)(__builtin_amdgcn_kernarg_segment_ptr());
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= win->tile0[win->npieces]) return;
  TileEntry e;
  const uint16_t* unused;
  int nv;
  resolve_tile(win, HD, t, &e.k, &e.v, &e.rows, &e.nvalid);
  resolve_tile(win, HD, t + 2, &e.k_next2, &unused, &e.rows_next2, &nv);
  resolve_tile(win, HD, t + 1, &unused, &e.v_next1, &e.rows_next1, &nv);
  e.pad[0] = e.pad[1] = 0;
  tab[t] = e;
}

// SEG: the keys are the window's pieces read in place, each padded to whole
// tiles and described per tile by `tab`; Nk is then the padded key count, a
// multiple of 64. Otherwise K and V are one contiguous window.
template <int D, bool SEG>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, int Nq, int Nk, int H, float c,
    uint16_t* __restrict__ O, float* __restrict__ lse, float* __restrict__ opart,
    float2* __restrict__ mlpart, int nsplit, int kps, const TileEntry* __restrict__ tab) {
  using T = Tile<D>;
  constexpr int KS = D / 16;   // k-steps of the QK product
  constexpr int DT = D / 32;   // d tiles of the PV product
  constexpr int KCH = T::KCH;
  // K is staged one tile ahead of V (the S^T product of tile t+1 overlaps
  // the softmax of tile t), in two K and two V stages. Each stage is its own
  // array and every access names its array at compile time, so the compiler
  // can see that loads in flight never alias the stages being read.
  __shared__ __attribute__((aligned(1024))) uint8_t kst0[T::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kst1[T::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vst0[T::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vst1[T::BYTES];

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

  // Direct-to-LDS staging: each wave-wide load fills 1 KiB of the tile, lane
  // l writing the 16 bytes at row (l / KCH), position (l % KCH) of its rows.
  // The lane fetches the global chunk that the row's swizzle puts there.
  // Offsets are relative to the tile's first row of this head.
  uint32_t kvo[T::LOADS], vvo[T::LOADS];
#pragma unroll
  for (int r = 0; r < T::LOADS; ++r) {
    const int row = (wave * T::LOADS + r) * T::ROWS_PER_LOAD + lane / KCH;
    const int pos = lane % KCH;
    kvo[r] = (uint32_t)((row * (int)HD + (pos ^ kswz<D>(row)) * 8) * 2);
    vvo[r] = (uint32_t)((row * (int)HD + (pos ^ vswz<D>(row)) * 8) * 2);
  }
  // SEG: rows of a tile at `tile` (head 0) with `rows` left in its piece.
  auto issue_rows = [&](const uint16_t* tile, int rows, uint8_t* stage,
                        const uint32_t (&vo)[T::LOADS]) {
    const uint32_t nrec =
        rows > 0 ? (uint32_t)(((size_t)rows * HD - (size_t)h * D) * 2) : 0u;
    const rsrc_t rs = make_rsrc(tile + (size_t)h * D, nrec);
    uint8_t* dst = stage + wave * T::LOADS * 1024;
#pragma unroll
    for (int r = 0; r < T::LOADS; ++r) buffer_load_lds16(rs, dst + r * 1024, vo[r]);
  };
  auto issue = [&](bool isv, int kb, uint8_t* stage, const uint32_t (&vo)[T::LOADS]) {
    const uint16_t* src = (isv ? V : K) + (size_t)kb * HD + (size_t)h * D;
    const uint32_t nrec = (uint32_t)(((size_t)(Nk - kb) * HD - (size_t)h * D) * 2);
    const rsrc_t rs = make_rsrc(src, nrec);
    uint8_t* dst = stage + wave * T::LOADS * 1024;
#pragma unroll
    for (int r = 0; r < T::LOADS; ++r) buffer_load_lds16(rs, dst + r * 1024, vo[r]);
  };

  // LDS read offsets. S^T operand: row kt*32 + prow (prow = key_perm(l32)),
  // chunk (2ks + g) swizzled; the swizzle depends on the row's low 4 bits
  // only, so it is the same for both 32-key halves.
  const int prow = key_perm(l32);
  uint32_t koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    koff[ks] = (uint32_t)(prow * T::ROW + (((2 * ks + g) ^ kswz<D>(prow)) * 16));
  // P*V operand (transpose reads): lane i of 16-lane group G reads keys
  // kb0 + i/4 (kb0 = kt*32 + 16mm + 8g + 4h, a multiple of 4) at columns
  // dt*32 + 16*(G%2) + 4*(i%4) .. +3, so lane j gets 4 keys of column
  // dt*32 + 16*(G%2) + j = dt*32 + l32.
  const int trow = (lane & 15) >> 2;
  const int tchunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  uint32_t voff[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    voff[dt] = (uint32_t)((8 * g + trow) * T::ROW + (((4 * dt + tchunk) ^ vswz<D>(trow)) * 16) +
                          (lane & 1) * 8);

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  float mref = 0.f;    // reference for s*scale*log2(e) of this lane's query
  float lsum = 0.f;    // this lane's share of the denominator

  const int nblk = (kend - kbeg + kBN - 1) / kBN;

  // S^T of one tile from the K stage `ks_` (Q^T in registers).
  auto qk = [&](const uint8_t* ks_, f32x16 (&st)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) st[kt][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(ks_ + kt * 32 * T::ROW + koff[ks]);
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qf[ks], st[kt], 0, 0, 0);
      }
    }
  };

  // Prologue: K(0), V(0), K(1) in flight, then S^T(0).
  f32x16 sc[2];
  if constexpr (!SEG) {
    if (nblk > 0) {
      issue(false, kbeg, kst0, kvo);
      issue(true, kbeg, vst0, vvo);
    }
    if (nblk > 1) issue(false, kbeg + kBN, kst1, kvo);
  } else {
    if (nblk > 0) {
      const TileEntry& e0 = tab[kbeg / kBN];
      issue_rows(e0.k, e0.rows, kst0, kvo);
      issue_rows(e0.v, e0.rows, vst0, vvo);
    }
    if (nblk > 1) {
      const TileEntry& e1 = tab[kbeg / kBN + 1];
      issue_rows(e1.k, e1.rows, kst1, kvo);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  qk(kst0, sc);
  __syncthreads();  // kst0 is refilled by the first iteration
  // The reference starts at the first tile's row max (over its real keys),
  // so the row's largest weight so far is 1 and its sum stays >= 1: nothing
  // that dominates the row can underflow.
  if (nblk > 0) {
    int lim = kend - kbeg;
    if constexpr (SEG) lim = min(lim, tab[kbeg / kBN].nvalid);
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (kt * 32 + 16 * (e >> 3) + 8 * g + (e & 7) < lim) mx = fmaxf(mx, sc[kt][e]);
    mx = max_halves(mx) * c;
    if (mx > -INFINITY) mref = mx;
  }

  // Iteration t: loads K(t+2) and V(t+1); softmax of S(t) (registers)
  // overlapped with S^T(t+1) from K stage kc; O^T += V(t) P(t) from V stage vc.
  auto tile = [&](int it, const uint8_t* kc, const uint8_t* vc, uint8_t* kd, uint8_t* vd) {
    const int kb = kbeg + it * kBN;
    int nvalid = kBN;
    if constexpr (!SEG) {
      if (it + 2 < nblk) issue(false, kb + 2 * kBN, kd, kvo);
      if (it + 1 < nblk) issue(true, kb + kBN, vd, vvo);
    } else {
      // one 32-byte scalar load: this iteration's loads and tile it's keys
      typedef int i32x8 __attribute__((ext_vector_type(8)));
      const i32x8 e = *reinterpret_cast<const i32x8*>(tab + kb / kBN);
      const uint16_t* k2 = reinterpret_cast<const uint16_t*>(
          (uint64_t)(uint32_t)e[0] | ((uint64_t)(uint32_t)e[1] << 32));
      const uint16_t* v1 = reinterpret_cast<const uint16_t*>(
          (uint64_t)(uint32_t)e[2] | ((uint64_t)(uint32_t)e[3] << 32));
      const int r2 = e[4], r1 = e[5];
      nvalid = e[6];
      if (it + 2 < nblk) issue_rows(k2, r2, kd, kvo);
      if (it + 1 < nblk) issue_rows(v1, r1, vd, vvo);
    }

    // SEG: mask the padding after the last row of a piece.
    if constexpr (SEG) {
      if (nvalid < kBN) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (kt * 32 + 16 * (e >> 3) + 8 * g + (e & 7) >= nvalid) sc[kt][e] = -INFINITY;
      }
    }
    // Mask keys past the end of this block's range (last tile only).
    if (kb + kBN > kend) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kb + kt * 32 + 16 * (e >> 3) + 8 * g + (e & 7);
          if (key >= kend) sc[kt][e] = -INFINITY;
        }
    }

    // S^T of the next tile (its K stage landed last iteration). On the last
    // tile this reads a stale stage and the result is dropped.
    f32x16 sn[2];
    qk(kc, sn);

    // p = 2^(s*c - mref) as bf16, and the tile's row sum of exactly those
    // weights (this lane's half of the row).
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    bf16x8 pb[2][2];
    float ts = 0.f;
    auto weights = [&]() {
      ts = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          f32x8 pv;
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(sc[kt][8 * mm + e], c, -mref));
          const bf16x8 b = __builtin_convertvector(pv, bf16x8);
          pb[kt][mm] = b;
          ts = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(b, b, 0, 1), ones, ts, false);
          ts = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(b, b, 2, 3), ones, ts, false);
          ts = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(b, b, 4, 5), ones, ts, false);
          ts = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(b, b, 6, 7), ones, ts, false);
        }
    };
    weights();
    // Instruction order for this region (sched_group_barrier masks: 0x100 LDS
    // read, 0x008 MFMA, 0x002 VALU): the first 4 K reads of S^T(t+1) up
    // front, then each of its 16 MFMAs followed by the next K read and 6 of
    // the softmax VALU ops of tile t, so MFMAs never wait on a K read that
    // was just issued and the VALU work is spread between them.
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
    // Range guard. The reference mref stays where it is while every half-row
    // tile sum is <= 2^30 (no weight near the fp32/bf16 range). Otherwise the
    // row's reference moves to its max (up only, once weight has accumulated;
    // O and l are rescaled by the same factor, or reset if nothing has
    // accumulated) and the weights are recomputed. O and l always share mref,
    // so the result is the same for any reference. Both halves of a row
    // decide on row-wide quantities, so they always agree.
    if (__any(!(ts <= kBigSum))) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[kt][e]);
      mx = max_halves(mx) * c;
      const bool acc = sum_halves(lsum) > 0.f;
      float mnew = acc ? fmaxf(mref, mx) : mx;
      if (!(mnew > -INFINITY)) mnew = mref;  // every key of the row masked
      const float alpha = acc ? __builtin_amdgcn_exp2f(mref - mnew) : 0.f;
      mref = mnew;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
      weights();
    }
    lsum += ts;

    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint8_t* vb = vc + (kt * 32 + 16 * mm) * T::ROW + voff[dt];
          const uint2 lo = lds_read_tr(vb);
          const uint2 hi = lds_read_tr(vb + 4 * T::ROW);
          const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), pb[kt][mm], o[dt], 0, 0, 0);
        }
    // P*V region: each MFMA right after the two transposing reads it needs.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    }
    sc[0] = sn[0];
    sc[1] = sn[1];
    __builtin_amdgcn_s_setprio(0);

    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): K(t+2), V(t+1) have landed
    __syncthreads();
  };
  for (int it = 0; it < nblk; it += 2) {
    tile(it, kst1, vst0, kst0, vst1);
    if (it + 1 < nblk) tile(it + 1, kst0, vst1, kst1, vst0);
  }

  const float ltot = sum_halves(lsum);
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
    if (lse && g == 0) lse[(size_t)h * Nq + q] = (mref + log2f(ltot)) * kLn2;
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
    if (g == 0) mlpart[row] = make_float2(mref, ltot);
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
  float acc[PER];
  float den;
  if (nsplit == 2) {
    // Two splits (the usual case): every load of the row is in flight at once.
    const size_t r0 = (size_t)h * Nq + q, r1 = ((size_t)H + h) * Nq + q;
    const float2 m0 = mlpart[r0], m1 = mlpart[r1];
    float x0[PER], x1[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      x0[i] = opart[r0 * D + sub * PER + i];
      x1[i] = opart[r1 * D + sub * PER + i];
    }
    M = fmaxf(m0.x, m1.x);
    const float w0 = exp2f(m0.x - M), w1 = exp2f(m1.x - M);
    den = fmaf(w1, m1.y, w0 * m0.y);
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = fmaf(w1, x1[i], w0 * x0[i]);
  } else {
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, mlpart[((size_t)s * H + h) * Nq + q].x);
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    den = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const size_t row = ((size_t)s * H + h) * Nq + q;
      const float2 ml = mlpart[row];
      const float w = exp2f(ml.x - M);
      den = fmaf(w, ml.y, den);
      const float* pp = opart + row * D + sub * PER;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = fmaf(w, pp[i], acc[i]);
    }
  }
  const float inv = 1.0f / den;
  uint16_t* op = O + (size_t)q * H * D + (size_t)h * D + sub * PER;
#pragma unroll
  for (int i = 0; i < PER; i += 2) {
    *reinterpret_cast<uint32_t*>(op + i) = pack_bf16x2(acc[i] * inv, acc[i + 1] * inv);
  }
  if (lse && sub == 0) lse[(size_t)h * Nq + q] = (M + log2f(den)) * kLn2;
}

template <int D, bool SEG>
hipError_t launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, int Nq, int Nk,
                  int H, float scale, uint16_t* out, float* lse, const AttnPlan& plan,
                  void* ws, const TileEntry* tab, hipStream_t s) {
  const int ntq = (Nq + kBM - 1) / kBM;
  const int G = ntq * H * plan.splits;
  const float c = scale * kLog2e;
  float* opart = nullptr;
  float2* ml = nullptr;
  if (plan.splits > 1) {
    opart = reinterpret_cast<float*>(ws);
    ml = reinterpret_cast<float2*>(opart + (size_t)plan.splits * H * Nq * D);
  }
  hipLaunchKernelGGL((attn_fwd_kernel<D, SEG>), dim3(G), dim3(kThreads), 0, s, q, k, v, Nq, Nk,
                     H, c, out, lse, opart, ml, plan.splits, plan.keys_per_split, tab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  const int rows = H * Nq;
  hipLaunchKernelGGL((attn_merge_kernel<D>), dim3((rows + 7) / 8), dim3(256), 0, s, opart,
                     ml, Nq, H, plan.splits, out, lse);
  return hipGetLastError();
}

}  // namespace

// Two 4-wave blocks fit on a CU. The key range is split (in powers of two,
// each split keeping >= 8 key tiles) only until the grid covers about 90% of
// those resident slots: fewer splits mean less partial traffic to merge.
// A grid of more than one round of resident blocks whose last round is less
// than 3/8 full is split in two as well: its last blocks would otherwise run
// on a mostly idle chip for most of a block's time. At 40 heads and 32,760
// keys that took grids of 1.02-1.33 rounds 13-18 % faster, 2.03-2.50 rounds
// 4-11 %, 3.05-3.36 rounds 4-8 % and 4.14-4.30 rounds 4-5 %; at 3.44 rounds
// and beyond half a round the split was slower.
AttnPlan attention_plan(int Nq, int Nk, int H, int D, int num_cus) {
  (void)D;
  AttnPlan p;
  const long long tiles = (long long)((Nq + kBM - 1) / kBM) * H;
  const long long slots = 2LL * num_cus;
  const int kblocks = (Nk + kBN - 1) / kBN;
  int splits = 1;
  while (tiles * splits * 10 < slots * 9 && kblocks / (splits * 2) >= 8) splits *= 2;
  if (splits == 1 && tiles > slots && kblocks / 2 >= 8) {
    const long long rem = tiles % slots;
    if (rem > 0 && rem * 8 < slots * 3) splits = 2;
  }
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
  return (D == 128) ? launch<128, false>(q, k, v, Nq, Nk, H, scale, out, lse, plan, ws, nullptr, s)
                    : launch<64, false>(q, k, v, Nq, Nk, H, scale, out, lse, plan, ws, nullptr, s);
}

size_t attention_window_table_bytes(int ntiles) {
  return ((size_t)ntiles * sizeof(TileEntry) + 255) / 256 * 256;
}

// The window in place: the tile table goes at the start of ws, the split
// partials after it. Nk is the padded key count of the pieces.
hipError_t attention_window_launch(const uint16_t* q, const WinPieces& w, int Nq, int H, int D,
                                   float scale, uint16_t* out, float* lse, const AttnPlan& plan,
                                   void* ws, hipStream_t s) {
  const int ntiles = w.tile0[w.npieces];
  const int Nk = ntiles * kBN;
  TileEntry* tab = reinterpret_cast<TileEntry*>(ws);
  hipLaunchKernelGGL(attn_tile_table_kernel, dim3((ntiles + 255) / 256), dim3(256), 0, s, w,
                     (int64_t)H * D, tab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  void* part = static_cast<char*>(ws) + attention_window_table_bytes(ntiles);
  return (D == 128) ? launch<128, true>(q, nullptr, nullptr, Nq, Nk, H, scale, out, lse, plan,
                                        part, tab, s)
                    : launch<64, true>(q, nullptr, nullptr, Nq, Nk, H, scale, out, lse, plan,
                                       part, tab, s);
}

}  // namespace wkv
