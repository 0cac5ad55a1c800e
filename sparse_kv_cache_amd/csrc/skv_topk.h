// skv_topk.h -- block-wide top-k selection of one score row, shared by the
// page_topk kernel and the decode kernel that selects in-block.  Internal to
// the library; not part of the C ABI.
//
// Selection: EntmaxKV README "How it works" (keep topk_pages per query head;
// the budget counts pages and includes the always-attended tail page);
// vortex_torch pull request "flow: add H2O sparse attention", hardware
// follow-up (the reserved leading bos and trailing eos entries are kept and
// only the window between them is ranked).
//
// Method.  Scores become order-preserving uint32 keys (-0.0 folded onto
// +0.0) held in registers, ITEMS contiguous entries per thread.  A
// most-significant-digit radix select finds the key prefix of the m-th best
// candidate: the bits every candidate shares are skipped (block OR / AND),
// each pass histograms the next BITS bits of the keys still matching the
// prefix into its own LDS histogram (atomics; every wave then finds the digit
// itself, so a pass costs one barrier), and the select stops as soon as the
// chosen bin is taken whole.  Keys above the prefix are taken; when equal keys
// must be split, the lowest indices are taken.  One block-wide prefix count of
// two values per thread (entries taken outright, entries equal to the prefix)
// gives every entry its place, so the indices are written in ascending order
// with no sort.
#pragma once

#include <limits.h>

#include "skv_device.h"

namespace skv {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;                        // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Select within one row of N scores (srow, 16-byte aligned when aligned16)
// with the whole block: writes the ascending selection to out[0, k_cap)
// (padded with -1) and, when bout is given, the selected pages' physical
// blocks btr[p] to bout; returns the selected count (every thread).  out and
// bout may point to global or LDS memory.  Ends with a block barrier unless
// SYNC_END is false (outputs that no thread of the block reads back).
// The selection from keys already in registers: key[i] is the order key of
// entry tid * ITEMS + i (entries outside the ranked window are ignored).
template <int BLOCK, int ITEMS, int BITS = 8, bool SYNC_END = true>
__device__ int topk_row_keys(const uint32_t (&key)[ITEMS], int N, int topk_pages,
                             double topk_frac, int bos, int eos,
                             const int32_t* __restrict__ btr, int64_t bt_ld,
                             int32_t* out, int32_t* bout, int k_cap);

template <int BLOCK, int ITEMS, int BITS = 8, bool SYNC_END = true>
__device__ int topk_row(const float* __restrict__ srow, bool aligned16, int N,
                        int topk_pages, double topk_frac, int bos, int eos,
                        const int32_t* __restrict__ btr, int64_t bt_ld,
                        int32_t* out, int32_t* bout, int k_cap) {
  const int lo = bos < N ? bos : N;
  int hi = N - eos > 0 ? N - eos : 0;
  if (hi < lo) hi = lo;
  const int base = threadIdx.x * ITEMS;
  uint32_t key[ITEMS];
  constexpr bool kVec = ITEMS % 4 == 0;          // 16-byte pieces per thread
  const bool vec = kVec && aligned16 && (base + ITEMS <= hi) && (base >= lo);
  if (vec) {
    if constexpr (kVec) {
#pragma unroll
      for (int i = 0; i < ITEMS; i += 4) {
        const float4 v = *reinterpret_cast<const float4*>(srow + base + i);
        key[i] = order_key(v.x); key[i + 1] = order_key(v.y);
        key[i + 2] = order_key(v.z); key[i + 3] = order_key(v.w);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int p = base + i;
      key[i] = (p >= lo && p < hi) ? order_key(srow[p]) : 0u;
    }
  }
  return topk_row_keys<BLOCK, ITEMS, BITS, SYNC_END>(key, N, topk_pages, topk_frac, bos,
                                                     eos, btr, bt_ld, out, bout, k_cap);
}

// Keys of the first row_len stored entries of srow, whatever the row's valid
// length (the selection masks by N), so the loads need not wait for N.
template <int ITEMS>
__device__ __forceinline__ void load_row_keys(const float* __restrict__ srow,
                                              bool aligned16, int64_t row_len,
                                              uint32_t (&key)[ITEMS]) {
  const int base = threadIdx.x * ITEMS;
  constexpr bool kVec = ITEMS % 4 == 0;
  if (kVec && aligned16 && base + ITEMS <= row_len) {
    if constexpr (kVec) {
#pragma unroll
      for (int i = 0; i < ITEMS; i += 4) {
        const float4 v = *reinterpret_cast<const float4*>(srow + base + i);
        key[i] = order_key(v.x); key[i + 1] = order_key(v.y);
        key[i + 2] = order_key(v.z); key[i + 3] = order_key(v.w);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int p = base + i;
      key[i] = p < row_len ? order_key(srow[p]) : 0u;
    }
  }
}

// Bits [0, x) set (x clipped to [0, 32]).
__device__ __forceinline__ uint32_t low_bits(int x) {
  return x <= 0 ? 0u : x >= 32 ? 0xffffffffu : ((1u << x) - 1u);
}

template <int BLOCK, int ITEMS, int BITS, bool SYNC_END>
__device__ int topk_row_keys(const uint32_t (&key)[ITEMS], int N, int topk_pages,
                             double topk_frac, int bos, int eos,
                             const int32_t* __restrict__ btr, int64_t bt_ld,
                             int32_t* out, int32_t* bout, int k_cap) {
  static_assert(ITEMS <= 32, "a thread's entries are tracked in 32-bit masks");
  constexpr int NW = BLOCK / 64;
  constexpr int kBits = BITS;                    // digit width
  constexpr int kBins = 1 << kBits;
  constexpr int kPasses = (32 + kBits - 1) / kBits;
  constexpr int kPerLane = kBins / 64;           // bins a lane scans
  static_assert(kPerLane % 4 == 0, "a lane scans its bins 16 bytes at a time");
  __shared__ __align__(16) int hist[kPasses][kBins];   // one histogram per pass
  __shared__ int scan_smem[2 * NW];
  __shared__ uint32_t s_or[NW], s_and[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int k = topk_pages;
  const double f = floor(topk_frac * static_cast<double>(N));
  if (f > static_cast<double>(k)) k = static_cast<int>(f);
  if (k > N) k = N;
  const int lo = bos < N ? bos : N;
  int hi = N - eos > 0 ? N - eos : 0;
  if (hi < lo) hi = lo;
  const int nres = N - (hi - lo);
  const int want = k - nres > 0 ? k - nres : 0;
  const int ncand = hi - lo;

  const int base = tid * ITEMS;
  // This thread's entries base + i as bit i: in the row (vm), in the ranked
  // window (wm), reserved (rm: in the row, outside the window).  Every
  // per-entry test below is a bit test, so the loops carry no branches.
  const uint32_t im = low_bits(ITEMS);
  const uint32_t vm = low_bits(N - base) & im;
  const uint32_t wm = low_bits(hi - base) & ~low_bits(lo - base) & im;
  const uint32_t rm = vm & ~wm;

  constexpr bool kVec = ITEMS % 4 == 0;
  // block ids of this thread's entries, fetched alongside the keys
  int32_t bid[ITEMS];
  if (bout != nullptr) {
    if (kVec && ((bt_ld & 3) == 0) && ((reinterpret_cast<uintptr_t>(btr) & 15) == 0) &&
        base + ITEMS <= N && base + ITEMS <= bt_ld) {
      if constexpr (kVec) {
#pragma unroll
        for (int i = 0; i < ITEMS; i += 4) {
          const int4 v = *reinterpret_cast<const int4*>(btr + base + i);
          bid[i] = v.x; bid[i + 1] = v.y; bid[i + 2] = v.z; bid[i + 3] = v.w;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int p = base + i;
        bid[i] = (p < N && p < bt_ld) ? btr[p] : -1;
      }
    }
  }
  for (int j = tid; j < kPasses * kBins; j += BLOCK) (&hist[0][0])[j] = 0;

  // Selection state: candidates whose (key & pmask) exceeds prefix are taken;
  // among those equal to prefix under pmask, the r_eq lowest indices.
  uint32_t prefix, pmask;
  int r_eq;
  if (want == 0) {
    prefix = 0xffffffffu; pmask = 0xffffffffu; r_eq = 0;   // reserved only
  } else if (want >= ncand) {
    prefix = 0u; pmask = 0u; r_eq = INT_MAX;               // every candidate
  } else {
    // Bits shared by every candidate need no radix pass: start the digits at
    // the highest bit where two candidates differ.
    uint32_t o = 0u, a = 0xffffffffu;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const uint32_t c = 0u - ((wm >> i) & 1u);       // all ones for a candidate
      o |= key[i] & c;
      a &= key[i] | ~c;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      o |= __shfl_xor(o, off);
      a &= __shfl_xor(a, off);
    }
    if (lane == 0) { s_or[wave] = o; s_and[wave] = a; }
    __syncthreads();                   // also orders the histogram clearing
    o = 0u; a = 0xffffffffu;
#pragma unroll
    for (int w = 0; w < NW; ++w) { o |= s_or[w]; a &= s_and[w]; }
    const uint32_t diff = o ^ a;       // bits that vary among candidates
    int top = diff ? 31 - __clz(diff) : -1;
    // bits below the lowest varying one are equal too (bf16-valued scores
    // leave the low 16 bits of every key the same)
    const int bot = diff ? __ffs(static_cast<int>(diff)) - 1 : 0;
    pmask = top >= 0 ? ~((2u << top) - 1u) : 0xffffffffu;
    if (top == 31) pmask = 0u;
    prefix = a & pmask;
    int remaining = want;
    int bin = ncand;                   // entries matching the prefix so far
    int pass = 0;
    while (remaining < bin && top >= bot) {
      int shift = top >= kBits - 1 ? top - (kBits - 1) : 0;
      if (shift < bot) shift = bot;
      const int width = top - shift + 1;
      const uint32_t dmask = (1u << width) - 1u;
      int* hp = hist[pass];
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        if (((wm >> i) & 1u) && (key[i] & pmask) == prefix)
          atomicAdd(&hp[(key[i] >> shift) & dmask], 1);
      }
      __syncthreads();
      // every wave finds the digit itself: no broadcast, no second barrier.
      // Lane l scans bins [kPerLane * l, kPerLane * (l + 1)).
      int cs[kPerLane];
#pragma unroll
      for (int j = 0; j < kPerLane; j += 4) {
        const int4 v = *reinterpret_cast<const int4*>(&hp[kPerLane * lane + j]);
        cs[j] = v.x; cs[j + 1] = v.y; cs[j + 2] = v.z; cs[j + 3] = v.w;
      }
      int sum = 0;
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) sum += cs[j];
      const int incl = skv::wave_inclusive_scan(sum);
      int above = __builtin_amdgcn_readlane(incl, 63) - incl;   // in higher digits
      int my_digit = 0, my_rem = 0, my_bin = 0;
      bool found = false;
#pragma unroll
      for (int j = kPerLane - 1; j >= 0; --j) {
        if (above < remaining && above + cs[j] >= remaining) {
          my_digit = kPerLane * lane + j;
          my_rem = remaining - above;
          my_bin = cs[j];
          found = true;
        }
        above += cs[j];
      }
      const unsigned long long ball = __ballot(found);
      const int src = __ffsll(static_cast<long long>(ball)) - 1;   // wave-uniform
      const uint32_t dg = static_cast<uint32_t>(__builtin_amdgcn_readlane(my_digit, src));
      remaining = __builtin_amdgcn_readlane(my_rem, src);
      bin = __builtin_amdgcn_readlane(my_bin, src);
      prefix |= dg << shift;
      pmask |= dmask << shift;
      top = shift - 1;
      ++pass;
    }
    r_eq = remaining;
  }

  // Entries taken outright (reserved, or above the prefix) and entries equal
  // to the prefix, as bit masks and counts, prefix-summed together: the r_eq
  // lowest-index equal entries are taken, so an entry's place is the
  // outright count before it plus min(equal count before it, r_eq).
  uint32_t om = rm, em = 0u;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const uint32_t km = key[i] & pmask;
    om |= static_cast<uint32_t>(km > prefix) << i;
    em |= static_cast<uint32_t>(km == prefix) << i;
  }
  em &= wm;
  om = (om & wm) | rm;
  const int n_out = __popc(om), n_eq = __popc(em);
  // exclusive scans of both counts: wave scans, one barrier for the wave
  // totals (the selection's own closing barrier, or the caller's, keeps the
  // totals from being overwritten before every wave has read them)
  const int ix = skv::wave_inclusive_scan(n_out);
  const int iy = skv::wave_inclusive_scan(n_eq);
  if (lane == 63) { scan_smem[wave] = ix; scan_smem[NW + wave] = iy; }
  __syncthreads();
  int out_before = ix - n_out, eq_before = iy - n_eq, out_total = 0, eq_total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int tx = scan_smem[w], ty = scan_smem[NW + w];
    if (w < wave) { out_before += tx; eq_before += ty; }
    out_total += tx;
    eq_total += ty;
  }
  const int total = out_total + (eq_total < r_eq ? eq_total : r_eq);
  // entries taken: the outright ones, and the equal ones still within r_eq
  const int eq_take = r_eq - eq_before;               // equal entries this thread may take
  uint32_t tm = om;
  if (eq_take >= n_eq) {
    tm |= em;
  } else if (eq_take > 0) {
    uint32_t e = em;
    for (int c = 0; c < eq_take; ++c) {                // lowest indices first
      tm |= e & (0u - e);
      e &= e - 1u;
    }
  }
  int pos = out_before + (eq_before < r_eq ? eq_before : r_eq);
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    if ((tm >> i) & 1u) {
      if (pos < k_cap) {
        out[pos] = base + i;
        if (bout != nullptr) bout[pos] = bid[i];
      }
      ++pos;
    }
  }
  for (int j = total + tid; j < k_cap; j += BLOCK) {
    out[j] = -1;
    if (bout != nullptr) bout[j] = -1;
  }
  if constexpr (SYNC_END) __syncthreads();
  return total < k_cap ? total : k_cap;
}

}  // namespace skv
