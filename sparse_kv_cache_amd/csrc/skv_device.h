// skv_device.h -- device helpers shared by the HIP kernels of libsparsekv
// (gfx950, wave64).  Internal to the library; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Matrix-core operand types (gfx950 bf16 MFMA).
typedef __bf16 skv_bf16x8 __attribute__((ext_vector_type(8)));
typedef short skv_short4 __attribute__((ext_vector_type(4)));
typedef float skv_f32x4 __attribute__((ext_vector_type(4)));

namespace skv {

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16
// A bf16 value is the upper half of an IEEE binary32 pattern.

__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Unpack 8 bf16 (one 16-byte vector) into floats.
__device__ __forceinline__ void unpack8(const uint4 v, float (&x)[8]) {
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
  x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
  x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// ------------------------------------------------- cross-lane reductions
// DPP moves inside a row of 16 lanes.  quad_perm [1,0,3,2] (0xB1) and
// [2,3,0,1] (0x4E) exchange within quads, row_half_mirror (0x141) reverses
// each 8-lane half, row_mirror (0x140) reverses the 16-lane row.  Each step
// adds two symmetric operands, so every lane of a group ends with the same
// bits.

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(
      0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LPR lanes (LPR = 8 or 16).
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPR == 8 || LPR == 16, "group of 8 or 16 lanes");
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  if constexpr (LPR == 16) x += dpp<0x140>(x);
  return x;
}

template <int LPR>
__device__ __forceinline__ float group_max(float x) {
  static_assert(LPR == 8 || LPR == 16, "group of 8 or 16 lanes");
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  if constexpr (LPR == 16) x = fmaxf(x, dpp<0x140>(x));
  return x;
}

// Whole-wave sum / max, the same value in every lane: DPP row reductions
// (no LDS permutes), then the four row results read into scalars.
__device__ __forceinline__ float row_lane(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  return (row_lane(x, 0) + row_lane(x, 16)) + (row_lane(x, 32) + row_lane(x, 48));
}

__device__ __forceinline__ float wave_max(float x) {
  x = group_max<16>(x);
  return fmaxf(fmaxf(row_lane(x, 0), row_lane(x, 16)), fmaxf(row_lane(x, 32), row_lane(x, 48)));
}

__device__ __forceinline__ int wave_inclusive_scan(int x) {
  // Hillis-Steele inside each 16-lane row with row_shr:1,2,4,8 (lanes with no
  // source add the 0 passed as `old`), then row_bcast:15 carries each row's
  // last lane into the next row (rows 1 and 3) and row_bcast:31 carries lane
  // 31 into rows 2 and 3.
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
  return x;
}

// Exclusive prefix sum over the block.  smem needs nwaves + 1 ints.  Every
// thread of the block must call it.
__device__ __forceinline__ int block_exclusive_scan(int x, int* total,
                                                    int* smem) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = (blockDim.x + kWave - 1) / kWave;
  int inc = wave_inclusive_scan(x);
  if (lane == kWave - 1) smem[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int w = lane < nwaves ? smem[lane] : 0;
    int wi = wave_inclusive_scan(w);
    if (lane < nwaves) smem[lane] = wi - w;
    if (lane == nwaves - 1) smem[nwaves] = wi;
  }
  __syncthreads();
  int r = inc - x + smem[wave];
  *total = smem[nwaves];
  __syncthreads();
  return r;
}

// Two exclusive prefix sums over the block at the cost of one (the same three
// barriers).  smem needs 2 * (nwaves + 1) ints.  Every thread must call it.
__device__ __forceinline__ void block_exclusive_scan2(int x, int y, int* ex, int* ey,
                                                      int* tx, int* ty, int* smem) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = (blockDim.x + kWave - 1) / kWave;
  int* sy = smem + nwaves + 1;
  const int ix = wave_inclusive_scan(x);
  const int iy = wave_inclusive_scan(y);
  if (lane == kWave - 1) { smem[wave] = ix; sy[wave] = iy; }
  __syncthreads();
  if (wave == 0) {
    const int wx = lane < nwaves ? smem[lane] : 0;
    const int wy = lane < nwaves ? sy[lane] : 0;
    const int jx = wave_inclusive_scan(wx);
    const int jy = wave_inclusive_scan(wy);
    if (lane < nwaves) { smem[lane] = jx - wx; sy[lane] = jy - wy; }
    if (lane == nwaves - 1) { smem[nwaves] = jx; sy[nwaves] = jy; }
  }
  __syncthreads();
  *ex = ix - x + smem[wave];
  *ey = iy - y + sy[wave];
  *tx = smem[nwaves];
  *ty = sy[nwaves];
  __syncthreads();
}

// log2(e) and ln(2) for base-2 exponentials.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Matrix-core operand of the 16x16x32 bf16 MFMA from 16 loaded bytes.
__device__ __forceinline__ skv_bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(skv_bf16x8, v);
}

}  // namespace skv
