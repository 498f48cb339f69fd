// Wave-level helpers shared by the kernels (device code only; included by the .hip sources).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs {

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS round trips):
// within each 16-lane row by shifts of 1, 2, 4 and 8 (lanes shifted in from outside the row
// read 0), then lane 15 of each row added to the next row (rows 1 and 3) and lane 31 to the
// upper half (rows 2 and 3).
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

}  // namespace hs
