// lanes.h -- lane exchanges within a 64-lane wave on gfx950 that avoid the
// LDS crossbar a general shuffle goes through (a round trip of the memory
// pipeline, ~100 cycles): DPP moves inside 16-lane rows or across the wave,
// a swizzle inside 32-lane halves, and lane reads.  Every caller runs them
// with the whole wave active.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace per {

// Lane exchanges within a wave that avoid the LDS crossbar a general
// shuffle goes through (a round trip of the memory pipeline): DPP moves
// inside 16-lane rows, a swizzle inside 32-lane halves, a lane read.
// xor_lanes(x, s): the value of lane i ^ 2^s.
__device__ __forceinline__ float xor_lanes(float x, int s) {
  const int v = __float_as_int(x);
  switch (s) {  // s is a constant wherever this is unrolled
    case 0:  // quad_perm [1,0,3,2]
      return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true));
    case 1:  // quad_perm [2,3,0,1]
      return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true));
    case 2: {  // row_half_mirror (lane i ^ 7), then quad_perm [3,2,1,0] (i ^ 3)
      const int h = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, true);
      return __int_as_float(__builtin_amdgcn_update_dpp(0, h, 0x1B, 0xF, 0xF, true));
    }
    case 3:  // row_ror:8
      return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, true));
    case 4:  // swizzle, bit mode: xor 16
      return __int_as_float(__builtin_amdgcn_ds_swizzle(v, 0x401F));
    default:
      return __shfl_xor(x, 1 << s);
  }
}

// down_lanes(x, q): the value of lane i + 2^q, for the lanes i that are
// multiples of 2^(q+1) (the only ones that use it).
__device__ __forceinline__ float down_lanes(float x, int q) {
  const int v = __float_as_int(x);
  switch (q) {  // q is a constant wherever this is unrolled
    case 0:  // row_shl:1
      return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x101, 0xF, 0xF, true));
    case 1:  // row_shl:2
      return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x102, 0xF, 0xF, true));
    case 2:  // row_shl:4
      return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0xF, true));
    case 3:  // row_shl:8
      return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x108, 0xF, 0xF, true));
    case 4:  // swizzle, bit mode: xor 16
      return __int_as_float(__builtin_amdgcn_ds_swizzle(v, 0x401F));
    default:  // lane 32, for lane 0
      return __int_as_float(__builtin_amdgcn_readlane(v, 32));
  }
}

// The value of lane i + 1 (DPP wave_shl:1; lane 63 gets 0).
__device__ __forceinline__ uint32_t next_lane(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x130, 0xF, 0xF, true);
}

// The max over the wave, the same in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int s = 0; s < 5; ++s)
    v = max(v, (uint32_t)__float_as_uint(xor_lanes(__uint_as_float(v), s)));
  return max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
             (uint32_t)__builtin_amdgcn_readlane((int)v, 32));
}

// The bitwise or over the wave, the same in every lane.
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
#pragma unroll
  for (int s = 0; s < 5; ++s) v |= (uint32_t)__float_as_uint(xor_lanes(__uint_as_float(v), s));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) |
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
}

}  // namespace per
