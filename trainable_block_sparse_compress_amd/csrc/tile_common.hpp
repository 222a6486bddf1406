// Helpers shared by the query-tile attention kernels (forward and the dQ
// pass of the backward): key order of the S^T tiles, LDS swizzle of staged
// [key][dim] blocks, wait-count immediates and opaque lane values.
#pragma once

#include "common.hpp"

namespace infllmv2 {

// Key held by row r of S^T key tile kt (a 64-key block has 4 tiles of 16).
// With this order the S^T accumulators of tiles 2kk and 2kk+1 are exactly
// the MFMA B operand for keys 32kk .. 32kk+31 (lane (c16, q4) holds keys
// 32kk + 8*q4 .. +7), so P^T (or dS^T) never leaves registers.
__device__ __forceinline__ int key_of(int kt, int r) {
  return 32 * (kt >> 1) + 8 * (r >> 2) + 4 * (kt & 1) + (r & 3);
}
// LDS swizzle of staged [key][dim] rows: 16-byte chunk p of row `row` sits
// at chunk p ^ swz_k(row), so the 8 rows a group of 8 lanes reads together
// map to distinct bank groups.
__device__ __forceinline__ int swz_k(int row) { return (row & 3) | ((row >> 1) & 4); }

// Opaque copy of a lane value: keeps the compiler from folding lane-constant
// address offsets into per-load invariants hoisted out of the block loops
// (which would pin dozens of 64-bit addresses in registers).
__device__ __forceinline__ int opaque(int v) {
  int r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

__device__ __forceinline__ int64_t opaque64(int64_t v) {
  const int lo = opaque((int)v), hi = opaque((int)(v >> 32));
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// s_waitcnt immediate: wait until at most n vector-memory loads are
// outstanding (vmcnt in bits 3:0 and 15:14), no wait on expcnt / lgkmcnt.
__host__ __device__ constexpr int vmcnt_imm(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

}  // namespace infllmv2
