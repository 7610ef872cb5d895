// Tiled storage of bf16 matrices that feed v_mfma_f32_16x16x32_bf16.
//
// A matrix X [rows][K] (rows a multiple of 16, K a multiple of 32) is stored
// as 16-row x 32-column tiles of 512 elements, tile (rt, kt) at element
// (rt * K/32 + kt) * 512.  Inside a tile, lane l of a wave owns the 16 bytes
// at l * 8: row rt*16 + l%16, columns kt*32 + 8*(l/16) .. +7 -- exactly the
// A (or B) operand fragment of the MFMA, so one wave-wide 16-byte load reads
// one whole tile from 1 KB of contiguous memory.
//
// Activations of a batch keep each request's rows together and padded to a
// multiple of 16: request b's token t is tiled row b * TP + t, TP = 16 *
// ceil(tokens / 16).  Padding rows are never written and never stored from.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace dmx {

// element offset of the 8-column chunk (row, col .. col+7), col % 8 == 0
__host__ __device__ __forceinline__ size_t tile_off(int row, int col, int K) {
  return ((size_t)(row >> 4) * (size_t)(K >> 5) + (size_t)(col >> 5)) * 512 + (size_t)((row & 15) + 16 * ((col >> 3) & 3)) * 8;
}

// fp32 tiles (a 16 x 32 tile is 2 KB: two 1 KB halves holding columns
// 8q..8q+3 and 8q+4..8q+7 of the lane's 8-column group): float offset of the
// first half of chunk (row, col .. col+7); the second half is 256 floats on.
__host__ __device__ __forceinline__ size_t tile_off_f32(int row, int col, int N) {
  return ((size_t)(row >> 4) * (size_t)(N >> 5) + (size_t)(col >> 5)) * 512 + (size_t)((row & 15) + 16 * ((col >> 3) & 3)) * 4;
}

__host__ __device__ __forceinline__ int padded_tokens(int tokens) { return (tokens + 15) & ~15; }

__host__ __device__ __forceinline__ bool row_valid(int prow, int tokens, int tp) { return prow % tp < tokens; }

}  // namespace dmx
