// Host tier device side (WorldPager abstract and Fig. 2: the store lives in
// pinned host memory, the next retrieval set is staged from the extrapolated
// pose, and a retrieved chunk that is not staged is replaced by staged data
// instead of waiting for a copy).
//
//   table   - one wave writes the staging table (chunk id per slot) and the
//             predicted slot of each rank, passed by value: the values are
//             captured when the launch is enqueued, so the host may plan the
//             next request before this one's copies have run.
//   copy    - the staging copies as one kernel that reads the pinned host
//             bank through its device mapping: a copy engine transfer would
//             wait on the host for the stream's earlier dependencies (the last
//             reader of the staging bank), a kernel waits on the device.
//             A small fixed grid (the copy is PCIe-bound, and every CU it
//             holds is one the concurrent attention cannot use) walks all
//             copies with 16-byte loads when the chunk size allows, else
//             4-byte.
//   resolve - one wave: lane j finds the slot holding retrieved chunk j; the
//             misses, in rank order, take the predicted slots no hit uses
//             (ballots rank both lists), so no chunk is placed twice.
#include "wkv_common.hpp"
#include "wkv_internal.hpp"

namespace wkv {

namespace {

__global__ __launch_bounds__(64) void tier_table_kernel(TierTable t, int32_t* __restrict__ slot_chunk,
                                                        int32_t* __restrict__ pred_slot) {
  const int i = threadIdx.x;
  if (i < t.n_slots) slot_chunk[i] = t.chunk[i];
  if (pred_slot && i < t.n_pred) pred_slot[i] = t.pred[i];
}

__global__ __launch_bounds__(64) void tier_resolve_kernel(const int32_t* __restrict__ actual, int n,
                                                          const int32_t* __restrict__ slot_chunk,
                                                          int n_slots,
                                                          const int32_t* __restrict__ pred_slot,
                                                          int32_t* __restrict__ out_slot,
                                                          int32_t* __restrict__ out_miss) {
  __shared__ int32_t hit[64];
  const int j = threadIdx.x;
  int h = -1;
  if (j < n) {
    const int32_t a = actual[j];
    if (a >= 0)
      for (int i = 0; i < n_slots; ++i)
        if (slot_chunk[i] == a) {
          h = i;
          break;
        }
  }
  hit[j] = h;
  __syncthreads();
  // Predicted slot of rank j is spare when no hit uses it.
  bool spare = false;
  int p = -1;
  if (j < n) {
    p = pred_slot[j];
    spare = true;
    for (int i = 0; i < n; ++i) spare = spare && hit[i] != p;
  }
  const uint64_t miss_mask = __ballot(j < n && h < 0);
  const uint64_t spare_mask = __ballot(spare);
  __syncthreads();
  hit[j] = p;  // reuse: predicted slot of each rank
  __syncthreads();
  if (j < n) {
    if (h >= 0) {
      out_slot[j] = h;
    } else {
      // the r-th miss (rank order) takes the r-th spare predicted slot
      int r = __popcll(miss_mask & ((1ull << j) - 1ull));
      uint64_t m = spare_mask;
      while (r-- > 0) m &= m - 1ull;
      // Distinct predicted slots always leave enough spares; otherwise -1
      // (the window gathers zero rows for it).
      out_slot[j] = m ? hit[__ffsll((unsigned long long)m) - 1] : -1;
    }
  }
  if (j == 0 && out_miss) out_miss[0] = (int32_t)__popcll(miss_mask);
}

constexpr int kCopyBlock = 256;
constexpr int kCopyGrid = 8;  // PCIe-bound: a few CUs keep enough reads in flight

// grid: kCopyGrid blocks; block b moves every (b + kCopyGrid*i)-th 16-byte
// (or 4-byte) unit of each (chunk, array) copy, four loads in flight.
__global__ __launch_bounds__(kCopyBlock) void tier_copy_kernel(TierCopy c) {
  const size_t stride = (size_t)kCopyBlock * kCopyGrid;
  const size_t t0 = (size_t)blockIdx.x * kCopyBlock + threadIdx.x;
  for (int j = 0; j < c.n; ++j) {
    for (int a = 0; a < c.narr; ++a) {
      const size_t bytes = c.bytes[a];
      const uint8_t* src = c.src[a] + (size_t)c.id[j] * bytes;
      uint8_t* dst = c.dst[a] + (size_t)c.slot[j] * bytes;
      if (bytes % 16 == 0) {
        const uint4* s4 = reinterpret_cast<const uint4*>(src);
        uint4* d4 = reinterpret_cast<uint4*>(dst);
        const size_t n = bytes / 16;
        size_t i = t0;
        for (; i + 3 * stride < n; i += 4 * stride) {
          const uint4 x0 = s4[i], x1 = s4[i + stride], x2 = s4[i + 2 * stride],
                      x3 = s4[i + 3 * stride];
          st_stream(d4 + i, x0);
          st_stream(d4 + i + stride, x1);
          st_stream(d4 + i + 2 * stride, x2);
          st_stream(d4 + i + 3 * stride, x3);
        }
        for (; i < n; i += stride) st_stream(d4 + i, s4[i]);
      } else {
        const uint32_t* s1 = reinterpret_cast<const uint32_t*>(src);
        uint32_t* d1 = reinterpret_cast<uint32_t*>(dst);
        for (size_t i = t0; i < bytes / 4; i += stride) d1[i] = s1[i];
      }
    }
  }
}

}  // namespace

hipError_t tier_copy_launch(const TierCopy& c, hipStream_t s) {
  if (c.n < 1) return hipSuccess;
  hipLaunchKernelGGL(tier_copy_kernel, dim3(kCopyGrid), dim3(kCopyBlock), 0, s, c);
  return hipGetLastError();
}

hipError_t tier_table_launch(const TierTable& t, int32_t* slot_chunk, int32_t* pred_slot,
                             hipStream_t s) {
  hipLaunchKernelGGL(tier_table_kernel, dim3(1), dim3(64), 0, s, t, slot_chunk, pred_slot);
  return hipGetLastError();
}

hipError_t tier_resolve_launch(const int32_t* actual, int n, const int32_t* slot_chunk,
                               int n_slots, const int32_t* pred_slot, int32_t* out_slot,
                               int32_t* out_miss, hipStream_t s) {
  hipLaunchKernelGGL(tier_resolve_kernel, dim3(1), dim3(64), 0, s, actual, n, slot_chunk, n_slots,
                     pred_slot, out_slot, out_miss);
  return hipGetLastError();
}

}  // namespace wkv
