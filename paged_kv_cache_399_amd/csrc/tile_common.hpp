// Device helpers shared by the kernels that stage 64-key chunks in LDS and
// run both attention products on matrix cores (paged prefill, and decode of
// wide packs of sequences that share blocks).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkv {

// Pairwise maxima with lane swaps on the vector ALU: v_permlane32_swap
// exchanges the upper half of one register with the lower half of another;
// with both operands equal, its two results hold the values of lanes l and
// l ^ 32 (v_permlane16_swap: of 16-lane rows, l and l ^ 16), in the same
// order in every lane, so both lanes of a pair get the same bits.
__device__ __forceinline__ float pair_max32(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto x = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)x[0]), __builtin_bit_cast(float, (uint32_t)x[1]));
}
__device__ __forceinline__ float pair_max16(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto x = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)x[0]), __builtin_bit_cast(float, (uint32_t)x[1]));
}

// Key rows of a staged chunk sit in LDS unpadded, with the 16-byte piece c of
// key row k stored at piece c ^ kswz(k).  One score-fragment read covers key
// rows {8a + b (+4) : a, b < 4} (the MFMA row order that gives each lane eight
// consecutive keys) at one piece index.  With rows padded by one piece (a
// uniform stride) those rows shared banks: on gfx950 the bank-conflict
// counter (SQ_LDS_BANK_CONFLICT) showed 4 extra cycles per such read, and 0
// with this swizzle (probe kernels of the exact address patterns).  The XOR
// uses row bits 0, 1, 3 and 4; bits 2 and 5 (chain Y, second half) are not
// used, so all rows a lane reads share one swizzle.
template <int D>
__device__ __forceinline__ int kswz(int k) {
  if constexpr (D == 128) return (k & 3) | (((k >> 3) & 3) << 2);
  return ((k & 3) | (((k >> 3) & 1) << 2)) ^ (((k >> 4) & 1) * 3);
}

}  // namespace pkv
