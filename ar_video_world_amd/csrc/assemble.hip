// Window assembly (WorldKV Sec. 4.2: retrieved chunks are inserted into the
// native attention window without re-encoding; Sec. 5.1: sink | retrieval |
// recent | denoising; WorldAttention kernel section: selected KV is copied
// into one contiguous buffer so that attention runs on regular tiles).
//
// One wave per block and one output row per wave (many small blocks keep
// more rows in flight than fewer wide ones); each lane loads up to
// kUnroll 16-byte chunks of its row before it stores any. The row's source
// is resolved once per wave from the segment table passed by value; rows of
// the retrieved region come from bank chunk retrieved_idx[slot]. bf16 rows
// are 16-byte copies; int4 rows (WorldPager: int4 KV store) read 4 packed
// bytes and one bf16 group scale per 8 output elements and write the
// dequantised bf16 values bf16_RNE(float(q) * scale) with 16-byte stores.
#include "wkv_common.hpp"
#include "wkv_internal.hpp"

namespace wkv {

namespace {

constexpr int kBlock = 64;
constexpr int kUnroll = 5;  // 16-byte chunks per lane in flight (a 40 x 128 row in two rounds)

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

// grid: (Nk, 2); y = 0 -> K, 1 -> V. STREAM: bf16 source rows are read with
// nontemporal loads.
template <bool STREAM>
__global__ __launch_bounds__(kBlock) void assemble_kernel(
    SegTable seg, BankArgs bank, int64_t Nk, int cpr, uint16_t* __restrict__ win_k,
    uint16_t* __restrict__ win_v) {
  const bool isk = blockIdx.y == 0;
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  if (row >= Nk) return;  // whole block
  uint4* dst = reinterpret_cast<uint4*>(isk ? win_k : win_v) + row * cpr;
  const int64_t ret_end = bank.off + (int64_t)bank.n_ret * bank.Lc;

  // Resolve the source of the row (block-uniform values).
  const uint4* src = nullptr;
  const uint32_t* psrc = nullptr;
  const uint16_t* ssrc = nullptr;
  int kind = 1;  // 1 bf16 copy, 2 int4, 3 zero
  if (row >= bank.off && row < ret_end) {
    const int64_t rr = row - bank.off;
    const int slot = (int)(rr / bank.Lc);
    const int64_t inrow = rr - (int64_t)slot * bank.Lc;
    const int id = bank.idx[slot];
    if (id < 0 || id >= bank.M) {
      kind = 3;
    } else {
      const int64_t brow = (int64_t)id * bank.Lc + inrow;
      if (bank.int4) {
        kind = 2;
        // 8 elements per 4 packed bytes: one 32-bit word per output chunk.
        psrc = reinterpret_cast<const uint32_t*>(isk ? bank.k : bank.v) + brow * cpr;
        ssrc = (isk ? bank.ks : bank.vs) + brow * (cpr / 4);
      } else {
        src = reinterpret_cast<const uint4*>(isk ? bank.k : bank.v) + brow * cpr;
      }
    }
  } else {
    int s = 0;
    while (s + 1 < seg.nseg && row >= seg.start[s + 1]) ++s;
    src = reinterpret_cast<const uint4*>(isk ? seg.k[s] : seg.v[s]) +
          (row - seg.start[s]) * cpr;
  }

  for (int c0 = lane; c0 < cpr; c0 += 64 * kUnroll) {
    uint4 buf[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + 64 * u;
      buf[u] = make_uint4(0, 0, 0, 0);
      if (c >= cpr) continue;
      if (kind == 1) {
        buf[u] = STREAM ? ld_stream(src + c) : src[c];
      } else if (kind == 2) {
        const uint32_t p = psrc[c];
        const float sc = bf16_to_f32(ssrc[c >> 2]);
        buf[u] = dequant8(p, sc);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + 64 * u;
      if (c < cpr) dst[c] = buf[u];
    }
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
  dim3 grid((unsigned)p.Nk, 2);
  // A window larger than the 256 MB Infinity Cache cannot have been left
  // there by whatever wrote its sources, so its rows stream past the caches
  // (671 MB at 14 B class: 214 us against 234 us). A smaller one may still
  // sit there, and plain loads keep that (97 MB at 1.3 B class: 34 us
  // against 35 us).
  const bool stream = (double)p.Nk * p.cpr * 16 * 2 > 256.0 * (1 << 20);
  if (stream)
    hipLaunchKernelGGL(assemble_kernel<true>, grid, dim3(kBlock), 0, s, seg, bank, p.Nk, p.cpr,
                       win_k, win_v);
  else
    hipLaunchKernelGGL(assemble_kernel<false>, grid, dim3(kBlock), 0, s, seg, bank, p.Nk, p.cpr,
                       win_k, win_v);
  return hipGetLastError();
}

}  // namespace wkv
