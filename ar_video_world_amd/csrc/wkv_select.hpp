// Block-wide deterministic bottom-k selection over 64-bit ordered keys, used
// by the compression select (bottom P % of pooled non-anchor tokens, WorldKV
// Sec. 4.3) and by the pose top-k (WorldKV Sec. 4.2).
//
// Keys live in registers, KPT per thread in blocked order (thread t holds the
// items t*KPT .. t*KPT+KPT-1). The k-th smallest key is found by an MSB-first
// radix select with 8-bit digits that starts below the leading bits every
// key shares (the block's min and max key give them): scores of one sign and
// magnitude range share a dozen or more leading bits, and skipping them
// halves the passes. Items are then kept when their key is below that
// threshold, plus the lowest-index items equal to it, so the kept set is
// exactly the k smallest (key, index) pairs.
#pragma once

#include "wkv_common.hpp"

namespace wkv {

struct SelectShared {
  uint32_t hist[256];
  uint64_t wmin[32];
  uint64_t wmax[32];
  int wave_tot[32];
  int bucket;
  int rank;
  int done;
};

// Exclusive block scan of one int per thread. Returns this thread's prefix;
// *total receives the block total. Contains barriers: every thread calls it.
template <int BLOCK>
__device__ __forceinline__ int block_exclusive_scan(int v, SelectShared& sh,
                                                    int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int NW = BLOCK / 64;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();  // wave_tot may still be read by a previous scan
  if (lane == 63) sh.wave_tot[wave] = x;
  __syncthreads();
  int wbase = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    int t = sh.wave_tot[w];
    wbase += (w < wave) ? t : 0;
    tot += t;
  }
  *total = tot;
  return wbase + x - v;
}

// Histogram increment with wave-level aggregation of equal digits: the few
// most common digits of the wave are counted with one atomic each (early
// radix passes see only a handful of distinct digits), the rest atomically.
__device__ __forceinline__ void hist_add(uint32_t* hist, bool pend, uint32_t d) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int it = 0; it < 3; ++it) {
    uint64_t act = __ballot(pend);
    if (act == 0) return;
    int leader = __ffsll((unsigned long long)act) - 1;
    uint32_t dl = __shfl((int)d, leader, 64);
    bool same = pend && (d == dl);
    uint64_t m = __ballot(same);
    if (lane == leader) atomicAdd(&hist[dl], (uint32_t)__popcll(m));
    if (same) pend = false;
  }
  if (pend) atomicAdd(&hist[d], 1u);
}

// Finds the k-th smallest (1 <= k <= number of valid keys) key. On return,
// *prefix / *mask describe the threshold bucket and *rank is how many of the
// items whose masked key equals *prefix are kept (lowest indices first).
template <int BLOCK, int KPT>
__device__ void block_radix_select(const uint64_t (&key)[KPT],
                                   const bool (&valid)[KPT], int k,
                                   SelectShared& sh, uint64_t* prefix_out,
                                   uint64_t* mask_out, int* rank_out) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  constexpr int NW = BLOCK / 64;
  // Leading bits shared by every valid key.
  uint64_t kmin = ~0ull, kmax = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (valid[i]) {
      kmin = key[i] < kmin ? key[i] : kmin;
      kmax = key[i] > kmax ? key[i] : kmax;
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t a = __shfl_xor(kmin, o, 64), b = __shfl_xor(kmax, o, 64);
    kmin = a < kmin ? a : kmin;
    kmax = b > kmax ? b : kmax;
  }
  __syncthreads();  // wmin / wmax may still be read by a previous call
  if (lane == 0) {
    sh.wmin[wave] = kmin;
    sh.wmax[wave] = kmax;
  }
  __syncthreads();
  kmin = sh.wmin[0];
  kmax = sh.wmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    kmin = sh.wmin[w] < kmin ? sh.wmin[w] : kmin;
    kmax = sh.wmax[w] > kmax ? sh.wmax[w] : kmax;
  }
  const uint64_t diff = kmin ^ kmax;
  if (diff == 0) {  // every valid key is equal: keep the k lowest indices
    *prefix_out = kmin;
    *mask_out = ~0ull;
    *rank_out = k;
    return;
  }
  int hi = 63 - __clzll((long long)diff);  // highest bit where keys differ
  uint64_t mask = hi == 63 ? 0ull : ~((2ull << hi) - 1ull);
  uint64_t prefix = kmin & mask;
  int rank = k;
#pragma unroll 1
  while (hi >= 0) {
    const int lo = hi >= 7 ? hi - 7 : 0;
    const uint32_t dmask = (2u << (hi - lo)) - 1u;  // 8 bits, fewer in the last pass
    for (int i = tid; i < 256; i += BLOCK) sh.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      bool m = valid[i] && ((key[i] & mask) == prefix);
      hist_add(sh.hist, m, (uint32_t)(key[i] >> lo) & dmask);
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t c0 = sh.hist[4 * tid + 0], c1 = sh.hist[4 * tid + 1];
      uint32_t c2 = sh.hist[4 * tid + 2], c3 = sh.hist[4 * tid + 3];
      int s = (int)(c0 + c1 + c2 + c3);
      int incl = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(incl, o, 64);
        if (tid >= o) incl += y;
      }
      int excl = incl - s;
      if (excl < rank && rank <= incl) {
        int r = rank - excl;
        uint32_t cs[4] = {c0, c1, c2, c3};
        int b = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (b == 0 && r <= (int)cs[q]) {
            b = q + 1;
          } else if (b == 0) {
            r -= (int)cs[q];
          }
        }
        sh.bucket = 4 * tid + (b - 1);
        sh.rank = r;
        sh.done = (r == (int)cs[b - 1]) ? 1 : 0;  // whole bucket kept
      }
    }
    __syncthreads();
    const int bucket = sh.bucket;
    rank = sh.rank;
    const int done = sh.done;
    prefix |= (uint64_t)bucket << lo;
    mask |= (uint64_t)dmask << lo;
    __syncthreads();  // sh.* is rewritten by the next pass
    if (done) break;
    hi = lo - 1;
  }
  *prefix_out = prefix;
  *mask_out = mask;
  *rank_out = rank;
}

// Keep flags for the k smallest (key, index) pairs given the select result;
// returns this thread's kept count and fills keep[]. Every thread calls it.
template <int BLOCK, int KPT>
__device__ int block_keep_flags(const uint64_t (&key)[KPT],
                                const bool (&valid)[KPT], uint64_t prefix,
                                uint64_t mask, int rank, SelectShared& sh,
                                bool (&keep)[KPT]) {
  int eqc = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    eqc += (valid[i] && (key[i] & mask) == prefix) ? 1 : 0;
  int tot;
  int er = block_exclusive_scan<BLOCK>(eqc, sh, &tot);
  int kc = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const uint64_t mk = key[i] & mask;
    bool eq = valid[i] && mk == prefix;
    bool kp = valid[i] && (mk < prefix || (eq && er < rank));
    er += eq ? 1 : 0;
    keep[i] = kp;
    kc += kp ? 1 : 0;
  }
  return kc;
}

}  // namespace wkv
