// Stage-1 block representation: parameter-free mean pooling of the keys
// (top168.com article on InfLLM-V2, section 三 "块表示的三阶段压缩": kernel
// l_C1 = B/2 and stride s_C1 = B/4; section 四 uses the same pooling with
// l_C2 = 4 l_C1, s_C2 = 4 s_C1 for the coarse keys of the LSE approximation).
//
// One thread produces 8 dims (16 bytes) of one window.  The window sum is
// accumulated in float64, which is exact for sums of bf16 values of the
// magnitudes met here, and rounded once to bf16 (nearest, ties to even), so
// the result is the correctly rounded mean.  HBM-bound.
#include "kernels.hpp"

namespace infllmv2 {

// float64 -> bf16 bits, round to nearest even, in one step (no float32 hop).
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
  uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
  if (mag == 0) return sign;
  const int e = (int)(mag >> 52) - 1023;
  if (e < -126) {
    // bf16 subnormal range: fixed quantum 2^-133 (128 lands on the smallest normal).
    const double r = rint(__longlong_as_double((long long)mag) * 0x1p133);
    return sign | (uint32_t)r;
  }
  mag += (1ull << 44) - 1ull + ((mag >> 45) & 1ull);
  const int e2 = (int)(mag >> 52) - 1023;
  if (e2 > 127) return sign | 0x7F80u;
  return sign | ((uint32_t)(e2 + 127) << 7) | ((uint32_t)(mag >> 45) & 0x7Fu);
}

__global__ __launch_bounds__(256) void compress_k_kernel(CompressArgs a) {
  const int s = blockIdx.z;
  const int g = blockIdx.y;
  const SeqRange rk = seq_range(a.cu_k, a.used_k, s);
  const int nw = rk.len >= a.kernel ? (rk.len - a.kernel) / a.stride + 1 : 0;
  const int j0 = a.cmp_begin ? a.cmp_begin[s] : 0;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int j = j0 + (idx >> 4);
  const int c = idx & 15;
  if (j < 0 || j >= nw || (a.cmp_begin && (idx >> 4) >= a.max_new)) return;
  const int64_t orow = (int64_t)a.cu_cmp[s] + j;
  if (orow < 0 || orow >= a.c_rows) return;

  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;
  const int64_t first = (int64_t)rk.start + (int64_t)a.stride * j;
  for (int u = 0; u < a.kernel; ++u) {
    const int64_t row = first + u;
    if (row < 0 || row >= a.rows_k) continue;
    const u32x4 v = ldg16(a.k + (row * a.h_kv + g) * kHeadDim + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += (double)__uint_as_float(v[i] << 16);
      acc[2 * i + 1] += (double)__uint_as_float(v[i] & 0xFFFF0000u);
    }
  }
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double lo = acc[2 * i] / (double)a.kernel;
    const double hi = acc[2 * i + 1] / (double)a.kernel;
    o[i] = f64_to_bf16_bits(lo) | (f64_to_bf16_bits(hi) << 16);
  }
  stg16(a.k_cmp + ((int64_t)g * a.c_rows + orow) * kHeadDim + 8 * c, o);
}

// Windows twice as long as their stride (both configurations of the pages:
// (32, 16) and (128, 64)) are the sum of two adjacent stride-long segments:
// every key row is read once.  Thread (window j, 16-byte chunk c) sums
// segment j; window j adds segment j + 1 from its neighbour through LDS (the
// workgroup's last window sums that segment itself).  The float64 segment
// sums are exact, so the result equals the direct window sum.
__global__ __launch_bounds__(256) void compress_k_pair_kernel(CompressArgs a) {
  __shared__ double seg[17][16][8];
  const int s = blockIdx.z;
  const int g = blockIdx.y;
  const SeqRange rk = seq_range(a.cu_k, a.used_k, s);
  const int nw = rk.len >= a.kernel ? (rk.len - a.kernel) / a.stride + 1 : 0;
  const int j0 = a.cmp_begin ? a.cmp_begin[s] : 0;
  const int jj = threadIdx.x >> 4;              // window of this thread within the workgroup
  const int c = threadIdx.x & 15;
  const int jw = blockIdx.x * 16 + jj;          // window index relative to j0
  const int j = j0 + jw;
  const int n_here = a.cmp_begin ? min(a.max_new, nw - j0) : nw;
  const bool active = j >= 0 && jw < n_here;
  auto segment = [&](int jseg, double (&acc)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0;
    const int64_t first = (int64_t)rk.start + (int64_t)a.stride * jseg;
    // Eight rows per step, all loads issued before the adds.
    for (int u0 = 0; u0 < a.stride; u0 += 8) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t row = first + u0 + u;
        v[u] = (u0 + u < a.stride && row >= 0 && row < a.rows_k)
                   ? ldg16(a.k + (row * a.h_kv + g) * kHeadDim + 8 * c) : zero16();
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += (double)__uint_as_float(v[u][i] << 16);
          acc[2 * i + 1] += (double)__uint_as_float(v[u][i] & 0xFFFF0000u);
        }
    }
  };
  double acc[8];
  if (active) segment(j, acc);
#pragma unroll
  for (int i = 0; i < 8; ++i) seg[jj][c][i] = active ? acc[i] : 0.0;
  // The segment after the workgroup's last window.
  if (jj == 15 && active) {
    double nx[8];
    segment(j + 1, nx);
#pragma unroll
    for (int i = 0; i < 8; ++i) seg[16][c][i] = nx[i];
  }
  __syncthreads();
  if (!active) return;
  // The last active window of a partial workgroup also sums its next segment.
  double nxt[8];
  if (jj < 15 && jw + 1 < n_here) {
#pragma unroll
    for (int i = 0; i < 8; ++i) nxt[i] = seg[jj + 1][c][i];
  } else if (jj < 15) {
    segment(j + 1, nxt);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) nxt[i] = seg[16][c][i];
  }
  const int64_t orow = (int64_t)a.cu_cmp[s] + j;
  if (orow < 0 || orow >= a.c_rows) return;
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double lo = (acc[2 * i] + nxt[2 * i]) / (double)a.kernel;
    const double hi = (acc[2 * i + 1] + nxt[2 * i + 1]) / (double)a.kernel;
    o[i] = f64_to_bf16_bits(lo) | (f64_to_bf16_bits(hi) << 16);
  }
  stg16(a.k_cmp + ((int64_t)g * a.c_rows + orow) * kHeadDim + 8 * c, o);
}

// V [rows_k, h_kv, 128] -> VT [h_kv, 128, batch, ld], zero past each sequence's
// length, so the attention kernels read 8 consecutive keys of one dim as one
// 16-byte load (the MFMA reduction runs over keys in P.V).
__global__ __launch_bounds__(256) void transpose_v_kernel(TransposeArgs a) {
  __shared__ uint16_t tile[64][136];
  const int s = blockIdx.z;
  const int g = blockIdx.y;
  const int key0 = blockIdx.x * 64;
  const SeqRange rk = seq_range(a.cu_k, a.used_k, s);
  if (key0 >= a.ld) return;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int key = (tid >> 4) + 16 * it;
    const int c = tid & 15;
    const int64_t row = (int64_t)rk.start + key0 + key;
    u32x4 v = zero16();
    if (key0 + key < rk.len && row < a.rows_k) v = ldg16(a.v + (row * a.h_kv + g) * kHeadDim + 8 * c);
    uint32_t* dst = reinterpret_cast<uint32_t*>(&tile[key][8 * c]);
    dst[0] = v[0];
    dst[1] = v[1];
    dst[2] = v[2];
    dst[3] = v[3];
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int dim = (tid >> 3) + 32 * it;
    const int kc = tid & 7;
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = tile[8 * kc + 2 * i][dim];
      const uint32_t hi = tile[8 * kc + 2 * i + 1][dim];
      o[i] = lo | (hi << 16);
    }
    stg16(a.vt + (((int64_t)g * kHeadDim + dim) * a.batch + s) * a.ld + key0 + 8 * kc, o);
  }
}

}  // namespace infllmv2

namespace infllmv2 {

hipError_t launch_compress(const CompressArgs& a, int batch, int max_windows, hipStream_t st) {
  const int64_t threads = (int64_t)max_windows * 16;
  dim3 grid((unsigned)((threads + 255) / 256), a.h_kv, batch);
  if (a.kernel == 2 * a.stride)
    hipLaunchKernelGGL(compress_k_pair_kernel, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(compress_k_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_transpose_v(const TransposeArgs& a, hipStream_t st) {
  dim3 grid((unsigned)(a.ld / 64), a.h_kv, a.batch);
  hipLaunchKernelGGL(transpose_v_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace infllmv2
