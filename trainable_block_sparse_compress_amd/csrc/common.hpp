// Device-side building blocks shared by the gfx950 kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace infllmv2 {

constexpr int kHeadDim = 128;
constexpr int kBlock = 64;   // tokens per attention block
constexpr int kWave = 64;    // CDNA wavefront

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float floatx4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef unsigned int u32x4 __attribute__((__vector_size__(4 * sizeof(unsigned int))));

// ---------------------------------------------------------------------------
// MFMA: D(16x16 f32) += A(16x32 bf16) * B(32x16 bf16).
// Lane l holds A row (l % 16), B column (l % 16), reduction slots 8*(l/16)+v;
// D column (l % 16), rows 4*(l/16)+v.
// ---------------------------------------------------------------------------
__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void stg16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ u32x4 zero16() { return u32x4{0u, 0u, 0u, 0u}; }

// Two floats -> packed bf16 pair (round to nearest even; one v_cvt_pk_bf16_f32).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Cross-lane reductions between the two 32-lane halves and between odd and
// even 16-lane rows (gfx950 v_permlane32_swap / v_permlane16_swap).  Swapping
// a register with itself leaves each lane with its own value in one result
// and its partner's in the other, so the symmetric combination of the two
// results is the pairwise reduction in every lane.
__device__ __forceinline__ float sum_x32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_x32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_x16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Reduce-scatter of two registers across the 32-lane halves: one half ends
// with a's half-sum, the other with b's.
__device__ __forceinline__ float rs_x32(float a, float b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Same across odd/even 16-lane rows.
__device__ __forceinline__ float rs_x16(float a, float b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sequence description shared by the kernels: start row and length.
struct SeqRange {
  int start;
  int len;
};
__device__ __forceinline__ SeqRange seq_range(const int32_t* cu, const int32_t* used, int s) {
  SeqRange r;
  r.start = cu[s];
  r.len = used ? used[s] : (cu[s + 1] - cu[s]);
  if (r.start < 0 || r.len < 0) {
    r.start = 0;
    r.len = 0;
  }
  return r;
}

// Sequence of packed query row `row`, with its query and key ranges and (if
// cu_c is given) its first compressed row.  cu_q is non-decreasing with
// batch + 1 entries; the row's sequence is the last one whose query start is
// <= row.  Up to 64 sequences this costs one round of loads: lane i reads
// sequence i's entries, a ballot finds the sequence and its lane's values
// are broadcast.  Larger batches binary-search.  Every lane of the wave
// calls it with the same row.  False when the row lies in no sequence.
struct RowSeq {
  int s;
  SeqRange rq, rk;
  int c0;
};
__device__ __forceinline__ bool find_row_seq(const int32_t* cu_q, const int32_t* used_q, const int32_t* cu_k,
                                             const int32_t* used_k, const int32_t* cu_c, int batch, int64_t row,
                                             RowSeq& r) {
  if (batch <= 0) return false;
  if (batch <= 64) {
    const int lane = __lane_id();
    const bool in = lane < batch;
    const int i = in ? lane : 0;
    const int qs = cu_q[i];
    const int ql = used_q ? used_q[i] : cu_q[i + 1] - qs;
    const int ks = cu_k[i];
    const int kl = used_k ? used_k[i] : cu_k[i + 1] - ks;
    const int cc = cu_c ? cu_c[i] : 0;
    const uint64_t le = __ballot(in && (int64_t)qs <= row);
    const int s = le ? 63 - __clzll((long long)le) : 0;
    r.s = s;
    r.rq.start = __builtin_amdgcn_readlane(qs, s);
    r.rq.len = __builtin_amdgcn_readlane(ql, s);
    r.rk.start = __builtin_amdgcn_readlane(ks, s);
    r.rk.len = __builtin_amdgcn_readlane(kl, s);
    r.c0 = __builtin_amdgcn_readlane(cc, s);
    if (r.rq.start < 0 || r.rq.len < 0) r.rq = SeqRange{0, 0};
    if (r.rk.start < 0 || r.rk.len < 0) r.rk = SeqRange{0, 0};
  } else {
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu_q[mid] <= row) lo = mid;
      else hi = mid - 1;
    }
    r.s = lo;
    r.rq = seq_range(cu_q, used_q, lo);
    r.rk = seq_range(cu_k, used_k, lo);
    r.c0 = cu_c ? cu_c[lo] : 0;
  }
  return row >= r.rq.start && row < (int64_t)r.rq.start + r.rq.len;
}

}  // namespace infllmv2
