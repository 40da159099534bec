// Window assembly (WorldKV Sec. 4.2: retrieved chunks are inserted into the
// native attention window without re-encoding; Sec. 5.1: sink | retrieval |
// recent | denoising; WorldAttention kernel section: selected KV is copied
// into one contiguous buffer so that attention runs on regular tiles).
//
// One wave per output row (a few rows per wave in flight). The row's source
// is resolved once per wave from the segment table passed by value; rows of
// the retrieved region come from bank chunk retrieved_idx[slot]. bf16 rows
// are 16-byte copies; int4 rows (WorldPager: int4 KV store) read 4 packed
// bytes and one bf16 group scale per 8 output elements and write the
// dequantised bf16 values bf16_RNE(float(q) * scale) with 16-byte stores.
#include "wkv_common.hpp"
#include "wkv_internal.hpp"

namespace wkv {

namespace {

constexpr int kBlock = 256;
constexpr int kRowsPerWave = 4;

// Output row -> source for the non-retrieved regions. Segment s covers output
// rows [start[s], start[s+1]).
struct SegTable {
  const uint16_t* k[kMaxSegments];
  const uint16_t* v[kMaxSegments];
  int64_t start[kMaxSegments + 1];
  int nseg;
};

struct BankArgs {
  const void* k;
  const void* v;
  const uint16_t* ks;
  const uint16_t* vs;
  const int32_t* idx;
  int M, Lc, n_ret;
  int64_t off;  // first output row of the retrieved region
  int int4;
};

__device__ __forceinline__ uint4 dequant8(uint32_t packed, float scale) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t byte = (packed >> (8 * i)) & 0xFFu;
    const int qlo = ((int)(byte << 28)) >> 28;   // sign-extend low nibble
    const int qhi = ((int)(byte << 24)) >> 28;   // sign-extend high nibble
    o[i] = pack_bf16x2((float)qlo * scale, (float)qhi * scale);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// grid: (ceil(Nk / (waves * kRowsPerWave)), 2); y = 0 -> K, 1 -> V.
__global__ __launch_bounds__(kBlock) void assemble_kernel(
    SegTable seg, BankArgs bank, int64_t Nk, int cpr, uint16_t* __restrict__ win_k,
    uint16_t* __restrict__ win_v) {
  const bool isk = blockIdx.y == 0;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row0 =
      ((int64_t)blockIdx.x * (kBlock / 64) + wave) * kRowsPerWave;
  uint4* dst = reinterpret_cast<uint4*>(isk ? win_k : win_v);
  const int64_t ret_end = bank.off + (int64_t)bank.n_ret * bank.Lc;

  // Resolve the source of each row (wave-uniform values).
  const uint4* src[kRowsPerWave];
  const uint32_t* psrc[kRowsPerWave];
  const uint16_t* ssrc[kRowsPerWave];
  int kind[kRowsPerWave];  // 0 none, 1 bf16 copy, 2 int4, 3 zero
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int64_t row = row0 + r;
    kind[r] = 0;
    src[r] = nullptr;
    psrc[r] = nullptr;
    ssrc[r] = nullptr;
    if (row >= Nk) continue;
    if (row >= bank.off && row < ret_end) {
      const int64_t rr = row - bank.off;
      const int slot = (int)(rr / bank.Lc);
      const int64_t inrow = rr - (int64_t)slot * bank.Lc;
      const int id = bank.idx[slot];
      if (id < 0 || id >= bank.M) {
        kind[r] = 3;
        continue;
      }
      const int64_t brow = (int64_t)id * bank.Lc + inrow;
      if (bank.int4) {
        kind[r] = 2;
        // 8 elements per 4 packed bytes: one 32-bit word per output chunk.
        psrc[r] = reinterpret_cast<const uint32_t*>(isk ? bank.k : bank.v) + brow * cpr;
        ssrc[r] = (isk ? bank.ks : bank.vs) + brow * (cpr / 4);
      } else {
        kind[r] = 1;
        src[r] = reinterpret_cast<const uint4*>(isk ? bank.k : bank.v) + brow * cpr;
      }
      continue;
    }
    int s = 0;
    while (s + 1 < seg.nseg && row >= seg.start[s + 1]) ++s;
    kind[r] = 1;
    src[r] = reinterpret_cast<const uint4*>(isk ? seg.k[s] : seg.v[s]) +
             (row - seg.start[s]) * cpr;
  }

  for (int c = lane; c < cpr; c += 64) {
    uint4 buf[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      if (kind[r] == 1) {
        buf[r] = src[r][c];
      } else if (kind[r] == 2) {
        const uint32_t p = psrc[r][c];
        const float sc = bf16_to_f32(ssrc[r][c >> 2]);
        buf[r] = dequant8(p, sc);
      } else {
        buf[r] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
      if (kind[r] != 0) dst[(row0 + r) * cpr + c] = buf[r];
  }
}

}  // namespace

hipError_t assemble_launch(const AssemblePlan& p, uint16_t* win_k, uint16_t* win_v,
                           hipStream_t s) {
  SegTable seg;
  for (int i = 0; i < kMaxSegments; ++i) {
    seg.k[i] = i < p.nseg ? p.seg_k[i] : nullptr;
    seg.v[i] = i < p.nseg ? p.seg_v[i] : nullptr;
  }
  for (int i = 0; i <= kMaxSegments; ++i) seg.start[i] = i <= p.nseg ? p.seg_start[i] : 0;
  seg.nseg = p.nseg;
  BankArgs bank;
  bank.k = p.bank_k;
  bank.v = p.bank_v;
  bank.ks = p.bank_ks;
  bank.vs = p.bank_vs;
  bank.idx = p.idx;
  bank.M = p.M;
  bank.Lc = p.Lc;
  bank.n_ret = p.n_ret;
  bank.off = p.ret_off;
  bank.int4 = p.int4;
  const int64_t rows_per_block = (kBlock / 64) * kRowsPerWave;
  dim3 grid((unsigned)((p.Nk + rows_per_block - 1) / rows_per_block), 2);
  hipLaunchKernelGGL(assemble_kernel, grid, dim3(kBlock), 0, s, seg, bank, p.Nk,
                     p.cpr, win_k, win_v);
  return hipGetLastError();
}

}  // namespace wkv
