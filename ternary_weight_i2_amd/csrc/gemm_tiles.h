// gemm_tiles.h -- pieces shared by the MFMA GEMM kernels (gemm.hip, the
// prefill tiles; gemm16.hip, the 16-token tiles).
#pragma once
#include "common.h"

#ifndef BITNET_GEMM_XCD_REMAP
#define BITNET_GEMM_XCD_REMAP 1   // group each XCD's workgroups on shared token tiles
#endif

namespace bitnet {

// Swizzle of the 16-byte pieces of a 128-byte token row in LDS: slot c' of
// row r holds piece c' ^ tok_swz(r).  A wave's fragment read takes the same
// piece of 32 consecutive rows; with this mix no two rows among 8 (128-byte
// bank window) or 16 (256-byte window) consecutive ones share a slot, where
// r & 7 left rows r and r + 8 on the same banks of a 256-byte window.
__device__ __forceinline__ int tok_swz(int r) { return (r ^ (r >> 3)) & 7; }

// The prefill matmul's path for 1..16 tokens: 16-token tiles on the 16x16x64
// MFMA (gemm16.hip); launch_gemm_mfma hands such launches over to it.
hipError_t launch_gemm16(const GemmMat *mats, int nmats, int64_t K, const int8_t *xq,
                         const float *xs, const int32_t *xsum, int64_t N, hipStream_t st);

}  // namespace bitnet
