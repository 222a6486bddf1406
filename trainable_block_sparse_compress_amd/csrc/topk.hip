// Block selection: init ∪ local ∪ top-k (top168.com article on InfLLM-V2,
// section 七 "技术实现的创新细节": a query in block b_i always attends the fixed
// init blocks and its local blocks; top-k runs over the remaining blocks and
// the attended set is the union).
//
// One wavefront per (query row, KV group).  Candidate scores (non-negative
// floats) are held in registers as order-preserving integer keys (bits + 1,
// 0 marks an empty slot).  A radix select over 8-bit digits with a 256-bin
// LDS histogram finds the exact n_topk-th largest key T; the selected
// candidates are every key > T plus the lowest-index keys == T needed to
// reach n_topk (ties broken toward the lower block index).  Ballot prefix
// counts then emit the blocks in ascending order: init blocks, selected
// candidates, local blocks — already sorted because those ranges are
// disjoint and ordered.
#include "kernels.hpp"
#include "topk_row.hpp"

namespace infllmv2 {

namespace {

constexpr int kWavesPerWG = 4;
constexpr int kSurvCap = 512;   // candidates per wave kept in LDS on the compacted path

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

// Radix select over 8-bit digits: the exact kk-th largest of the live keys
// (every live key lies in [kmin, kmax]).  On return kk holds how many keys
// equal to the result are still to be taken.  each(f) calls f(key) for every
// non-zero key this lane holds.  The digits start right below the bits
// common to kmax and kmin.
template <class Each>
__device__ __forceinline__ uint32_t radix_kth(uint32_t* hist, int lane, uint32_t kmax, uint32_t kmin, int& kk,
                                              Each each) {
  const uint32_t diff = kmax ^ kmin;
  if (!diff) return kmax;
  const int top_bit = 31 - __clz((int)diff);
  const uint32_t above = top_bit >= 31 ? 0u : ~((2u << top_bit) - 1u);
  uint32_t prefix = kmax & above;
  uint32_t pmask = above;
  for (int hb = top_bit; hb >= 0; hb -= 8) {
    const int lob = max(0, hb - 7);
    const int width = hb - lob + 1;
    const uint32_t dmask = (1u << width) - 1u;
#pragma unroll
    for (int b = 0; b < 4; ++b) hist[lane * 4 + b] = 0;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    each([&](uint32_t k) {
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> lob) & dmask], 1u);
    });
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    // Lane l owns bins 4l .. 4l+3; count of keys in higher bins via a
    // suffix scan over lanes.
    uint32_t h4[4];
    uint32_t local = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      h4[b] = hist[lane * 4 + b];
      local += h4[b];
    }
    uint32_t suffix = local;  // inclusive: lanes >= lane
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = (uint32_t)__shfl_down((int)suffix, off);
      if (lane + off < 64) suffix += o;
    }
    uint32_t cum = suffix - local;  // keys in bins above 4l+3
    int found = -1, newk = 0;
#pragma unroll
    for (int b = 3; b >= 0; --b) {
      if (found < 0 && cum < (uint32_t)kk && (uint32_t)kk <= cum + h4[b]) {
        found = lane * 4 + b;
        newk = kk - (int)cum;
      }
      cum += h4[b];
    }
    const uint64_t ball = __ballot(found >= 0);
    const int src = __ffsll((unsigned long long)ball) - 1;
    const int digit = __shfl(found, src);
    kk = __shfl(newk, src);
    prefix |= ((uint32_t)digit & dmask) << lob;
    pmask |= dmask << lob;
    __builtin_amdgcn_wave_barrier();
  }
  return prefix;
}

// Emit the candidates of one 64-wide step in ascending order: every key
// above T, and keys equal to T while the tie budget kk lasts (lowest block
// index first).  base / eq_seen carry over between steps.
__device__ __forceinline__ void emit_step(int32_t* out, int lane, uint32_t key, int block, uint32_t T, int kk,
                                          int limit, int& base, int& eq_seen) {
  const bool gt = key > T;
  const bool eq = key == T && key != 0;
  const uint64_t eqb = __ballot(eq);
  const int eq_rank = eq_seen + __popcll(eqb & lanemask_lt(lane));
  const bool take = gt || (eq && eq_rank < kk);
  const uint64_t tb = __ballot(take);
  const int pos = base + __popcll(tb & lanemask_lt(lane));
  if (take && pos < limit) out[pos] = block;
  base += __popcll(tb);
  eq_seen += __popcll(eqb);
}

template <int PER>
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist_all[kWavesPerWG][256];
  __shared__ uint32_t surv_key_all[kWavesPerWG][kSurvCap];
  __shared__ uint16_t surv_blk_all[kWavesPerWG][kSurvCap];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // row is wave-uniform
  const int lane = threadIdx.x & 63;
  uint32_t* hist = hist_all[wave];
  const int s = blockIdx.z;
  const int g = blockIdx.y;
  const SeqRange rq = seq_range(a.cu_q, a.used_q, s);
  const SeqRange rk = seq_range(a.cu_k, a.used_k, s);
  const int i = blockIdx.x * kWavesPerWG + wave;
  if (i >= rq.len) return;
  const int64_t row = (int64_t)rq.start + i;
  if (row >= a.rows_q) return;
  const int t = rk.len - rq.len + i;
  const int bt = t / kBlock;
  const int n_sel = a.n_init + a.n_local + a.n_topk;
  int32_t* out = a.idx + ((int64_t)g * a.rows_q + row) * n_sel;
  const int lo = a.n_init;
  const int hi = (int)min((int64_t)(bt - a.n_local), a.bs_ld - 1);
  const int nc = hi - lo + 1;

  if (nc <= a.n_topk) {
    // Every causal block is attended.
    for (int e = lane; e < n_sel; e += 64) out[e] = e <= bt ? e : -1;
    return;
  }
  if (a.n_topk == 0) {
    // No top-k: the init and local blocks only.
    for (int e = lane; e < a.n_init; e += 64) out[e] = e;
    for (int r = lane; r < a.n_local; r += 64) out[a.n_init + r] = bt - a.n_local + 1 + r;
    return;
  }

  const float* row_bs = a.bs + ((int64_t)g * a.rows_q + row) * a.bs_ld + lo;
  uint32_t key[PER];
  uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
  // Every load is issued before any is used: slots past the row read its
  // last candidate (nc >= 1 here) and are cleared afterwards, so no branch
  // separates a load from the next.
#pragma unroll
  for (int p = 0; p < PER; ++p) key[p] = __float_as_uint(row_bs[min(lane + 64 * p, nc - 1)]);
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const bool in = lane + 64 * p < nc;
    key[p] = in ? key[p] + 1u : 0u;
    kmax = in ? max(kmax, key[p]) : kmax;
    kmin = in ? min(kmin, key[p]) : kmin;
  }
  // Lower bound of the n_topk-th largest key: each lane holds at least one
  // key >= its own maximum, so at least 64 keys are >= the smallest lane
  // maximum, and for n_topk <= 64 so is the n_topk-th largest (a lane with
  // no key has maximum 0, which turns the bound off).  Keys below it can
  // never be selected and are dropped (key 0 = empty).
  uint32_t lane_max = kmax;
  for (int off = 32; off >= 1; off >>= 1) {
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    lane_max = min(lane_max, (uint32_t)__shfl_xor((int)lane_max, off));
  }
  const uint32_t bound = (a.n_topk >= 1 && a.n_topk <= 64) ? lane_max : 0u;
  kmin = max(kmin, bound);
  // The live candidates, in ascending block order, go to this wave's LDS
  // list (as far as it reaches); n_live counts them all.
  uint32_t* sk = surv_key_all[wave];
  uint16_t* sb = surv_blk_all[wave];
  int n_live = 0;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const bool live = key[p] != 0u && key[p] >= bound;
    const uint64_t b = __ballot(live);
    const int pos = n_live + __popcll(b & lanemask_lt(lane));
    if (live && pos < kSurvCap) {
      sk[pos] = key[p];
      sb[pos] = (uint16_t)(lane + 64 * p);
    }
    n_live += __popcll(b);
  }
  int kk = a.n_topk;
  const int n_init_eff = min(a.n_init, bt + 1);
  const int limit = n_init_eff + a.n_topk;
  for (int e = lane; e < n_init_eff; e += 64) out[e] = e;
  int base = n_init_eff;
  int eq_seen = 0;

  if (n_live <= kSurvCap) {
    // Compacted path: the select and the emission walk only the list.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const uint32_t T = radix_kth(hist, lane, kmax, kmin, kk, [&](auto f) {
      for (int e = lane; e < n_live; e += 64) f(sk[e]);
    });
    for (int e0 = 0; e0 < n_live; e0 += 64) {
      const int e = e0 + lane;
      const bool in = e < n_live;
      emit_step(out, lane, in ? sk[e] : 0u, lo + (in ? (int)sb[e] : 0), T, kk, limit, base, eq_seen);
    }
  } else {
    // Many candidates in contention (ties or a flat score profile): the
    // select and the emission re-read the row rather than keep the keys in
    // registers across both paths.
    auto key_at = [&](int c) -> uint32_t {
      if (c >= nc) return 0u;
      const uint32_t k = __float_as_uint(row_bs[c]) + 1u;
      return k >= bound ? k : 0u;
    };
    const uint32_t T = radix_kth(hist, lane, kmax, kmin, kk, [&](auto f) {
      for (int c = lane; c < nc; c += 64) {
        const uint32_t k = key_at(c);
        if (k != 0u) f(k);
      }
    });
    for (int c0 = 0; c0 < nc; c0 += 64) emit_step(out, lane, key_at(c0 + lane), lo + c0 + lane, T, kk, limit, base, eq_seen);
  }
  base = limit;
  for (int r = lane; r < a.n_local; r += 64) out[base + r] = bt - a.n_local + 1 + r;
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, int batch, int h_kv, int max_seqlen_q, int max_blocks,
                       hipStream_t st) {
  dim3 grid((max_seqlen_q + kWavesPerWG - 1) / kWavesPerWG, h_kv, batch);
  const int need = (max_blocks + 63) / 64;
  if (need <= 8) {
    hipLaunchKernelGGL(topk_kernel<8>, grid, dim3(256), 0, st, a);
  } else if (need <= 16) {
    hipLaunchKernelGGL(topk_kernel<16>, grid, dim3(256), 0, st, a);
  } else if (need <= 32) {
    hipLaunchKernelGGL(topk_kernel<32>, grid, dim3(256), 0, st, a);
  } else if (need <= 64) {
    hipLaunchKernelGGL(topk_kernel<64>, grid, dim3(256), 0, st, a);
  } else if (need <= 128) {
    hipLaunchKernelGGL(topk_kernel<128>, grid, dim3(256), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace infllmv2

// ---------------------------------------------------------------------------
// Row path: one workgroup of 256 threads per (query row, KV group), for
// launches with few rows (decode); the selection itself is in topk_row.hpp.
// ---------------------------------------------------------------------------
namespace infllmv2 {
namespace {

template <int PER>
__global__ __launch_bounds__(kRowThreads) void topk_rows_kernel(TopkArgs a) {
  __shared__ RowSelLds sh;
  const int tid = threadIdx.x;
  uint32_t key[PER];
  row_keys_load<PER>(a, blockIdx.x, blockIdx.y, tid, key);
  RowSetup rs;
  if (!row_setup(a, blockIdx.x, blockIdx.y, tid, rs) || rs.done) return;
  row_keys_clear<PER>(rs, tid, key);
  row_select<PER>(a, rs, key, sh);
}

}  // namespace

hipError_t launch_topk_rows(const TopkArgs& a, int h_kv, int max_blocks, hipStream_t st) {
  dim3 grid((unsigned)a.rows_q, h_kv);
  const int need = (max_blocks + kRowThreads - 1) / kRowThreads;
  if (need <= 4) hipLaunchKernelGGL(topk_rows_kernel<4>, grid, dim3(kRowThreads), 0, st, a);
  else if (need <= 8) hipLaunchKernelGGL(topk_rows_kernel<8>, grid, dim3(kRowThreads), 0, st, a);
  else if (need <= 16) hipLaunchKernelGGL(topk_rows_kernel<16>, grid, dim3(kRowThreads), 0, st, a);
  else if (need <= 32) hipLaunchKernelGGL(topk_rows_kernel<32>, grid, dim3(kRowThreads), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace infllmv2
