// Top-k of one (query row, KV group) by a whole workgroup of 256 threads:
// the row path of the block selection (init blocks, top-k of the remaining
// candidates, local blocks; top168.com article on InfLLM-V2, section 七
// "技术实现的创新细节"), shared by the top-k row kernel and the split block
// scoring, whose last workgroup of a row selects that row's blocks.
// Thread i owns the PER consecutive candidates PER*i .. PER*i+PER-1, so
// candidate order is thread order; a radix select over 8-bit digits on a
// shared 256-bin histogram finds the exact n_topk-th largest key, and two
// workgroup scans (ties, then selected counts) give every thread its output
// slots.
#pragma once

#include "kernels.hpp"

namespace infllmv2 {
namespace {

constexpr int kRowThreads = 256;

// Exclusive prefix over the workgroup's threads; `total` gets the sum.
__device__ __forceinline__ int wg_exclusive_scan(int v, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  __syncthreads();   // wsum free from any earlier use
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kRowThreads / 64; ++w) {
    const int x = wsum[w];
    before += w < wave ? x : 0;
    total += x;
  }
  return before + incl - v;
}

// Shared memory of the row selection (one workgroup per (row, KV group)).
struct RowSelLds {
  uint32_t hist[256];
  int wsum[kRowThreads / 64];
  uint32_t ext[3][kRowThreads / 64];
  int pick[2];
};

// Row setup shared by the row kernels: false when the row is outside every
// sequence; otherwise the row's last block and candidate range, and rows
// that keep every candidate (or take no top-k) are emitted here (done = true).
struct RowSetup {
  int bt, lo, hi, nc, n_sel;
  int32_t* out;
  bool done;
};
__device__ __forceinline__ bool row_setup(const TopkArgs& a, int64_t row, int g, int tid, RowSetup& r) {
  RowSeq rsq;
  if (!find_row_seq(a.cu_q, a.used_q, a.cu_k, a.used_k, nullptr, a.batch, row, rsq)) return false;
  const SeqRange rq = rsq.rq, rk = rsq.rk;
  const int t = rk.len - rq.len + (int)(row - rq.start);
  if (t < 0) return false;
  r.bt = t / kBlock;
  r.n_sel = a.n_init + a.n_local + a.n_topk;
  r.out = a.idx + ((int64_t)g * a.rows_q + row) * r.n_sel;
  r.lo = a.n_init;
  r.hi = (int)min((int64_t)(r.bt - a.n_local), a.bs_ld - 1);
  r.nc = r.hi - r.lo + 1;
  r.done = true;
  if (r.nc <= a.n_topk) {
    for (int e = tid; e < r.n_sel; e += kRowThreads) r.out[e] = e <= r.bt ? e : -1;
    return true;
  }
  if (a.n_topk == 0) {
    for (int e = tid; e < a.n_init; e += kRowThreads) r.out[e] = e;
    for (int q = tid; q < a.n_local; q += kRowThreads) r.out[a.n_init + q] = r.bt - a.n_local + 1 + q;
    return true;
  }
  r.done = false;
  return true;
}

// Top-n_topk of the row's candidate keys (thread tid holds candidates
// lo + PER*tid + p as order-preserving keys, bits + 1, 0 = empty) and the
// emission of init ∪ top-k ∪ local in ascending order.
template <int PER>
__device__ __forceinline__ void row_select(const TopkArgs& a, const RowSetup& rs, uint32_t (&key)[PER],
                                           RowSelLds& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* hist = sh.hist;
  int* wsum = sh.wsum;
  auto& ext = sh.ext;
  int* pick = sh.pick;
  const int bt = rs.bt, lo = rs.lo;
  int32_t* out = rs.out;
  uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    kmax = key[p] != 0 ? max(kmax, key[p]) : kmax;
    kmin = key[p] != 0 ? min(kmin, key[p]) : kmin;
  }
  // Smallest thread maximum: a lower bound of the n_topk-th largest key for
  // n_topk <= kRowThreads (every thread holds a key >= its own maximum);
  // keys below it are dropped before the histogram passes.
  uint32_t thr_max = kmax;
  for (int off = 32; off >= 1; off >>= 1) {
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    thr_max = min(thr_max, (uint32_t)__shfl_xor((int)thr_max, off));
  }
  if (lane == 0) {
    ext[0][wave] = kmax;
    ext[1][wave] = kmin;
    ext[2][wave] = thr_max;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kRowThreads / 64; ++w) {
    kmax = max(kmax, ext[0][w]);
    kmin = min(kmin, ext[1][w]);
    thr_max = min(thr_max, ext[2][w]);
  }
  const uint32_t bound = (a.n_topk >= 1 && a.n_topk <= kRowThreads) ? thr_max : 0u;
#pragma unroll
  for (int p = 0; p < PER; ++p) key[p] = key[p] >= bound ? key[p] : 0u;
  kmin = max(kmin, bound);
  const uint32_t diff = kmax ^ kmin;
  const int top_bit = diff ? 31 - __clz((int)diff) : 0;
  uint32_t prefix = diff ? (kmax & ~((top_bit >= 31) ? 0xFFFFFFFFu : ((2u << top_bit) - 1u))) : kmax;
  uint32_t pmask = diff ? ~((top_bit >= 31) ? 0xFFFFFFFFu : ((2u << top_bit) - 1u)) : 0xFFFFFFFFu;
  int kk = a.n_topk;
  if (diff) {
    for (int hb = top_bit; hb >= 0; hb -= 8) {
      const int lob = max(0, hb - 7);
      const int width = hb - lob + 1;
      const uint32_t dmask = (1u << width) - 1u;
      hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int p = 0; p < PER; ++p)
        if (key[p] != 0 && (key[p] & pmask) == prefix) atomicAdd(&hist[(key[p] >> lob) & dmask], 1u);
      __syncthreads();
      if (wave == 0) {
        uint32_t h4[4], local = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          h4[b] = hist[lane * 4 + b];
          local += h4[b];
        }
        uint32_t suffix = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t o = (uint32_t)__shfl_down((int)suffix, off);
          if (lane + off < 64) suffix += o;
        }
        uint32_t cum = suffix - local;
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
        if (lane == src) {
          pick[0] = found;
          pick[1] = newk;
        }
      }
      __syncthreads();
      const int digit = pick[0];
      kk = pick[1];
      prefix |= ((uint32_t)digit & dmask) << lob;
      pmask |= dmask << lob;
      __syncthreads();   // hist and pick are rewritten by the next pass
    }
  }
  const uint32_t T = prefix;

  // Ties: the lowest-index kk keys equal to T are taken.
  int n_eq = 0, n_gt = 0;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    n_eq += (key[p] == T && key[p] != 0);
    n_gt += key[p] > T;
  }
  int tot;
  const int eq_before = wg_exclusive_scan(n_eq, wsum, tot);
  const int n_take = n_gt + max(0, min(n_eq, kk - eq_before));
  int pos = wg_exclusive_scan(n_take, wsum, tot);
  const int n_init_eff = min(a.n_init, bt + 1);
  for (int e = tid; e < n_init_eff; e += kRowThreads) out[e] = e;
  pos += n_init_eff;
  int eq_rank = eq_before;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const bool eq = key[p] == T && key[p] != 0;
    const bool take = key[p] > T || (eq && eq_rank < kk);
    eq_rank += eq;
    if (take) {
      if (pos < n_init_eff + a.n_topk) out[pos] = lo + PER * tid + p;
      ++pos;
    }
  }
  const int base = n_init_eff + a.n_topk;
  for (int r = tid; r < a.n_local; r += kRowThreads) out[base + r] = bt - a.n_local + 1 + r;
}

// The row's scores from its first candidate (block n_init) on, as thread
// tid's PER slots.  They depend on the row alone, so they can be read before
// (and in the same round as) the row's metadata: slots past the stored row
// read its last entry, and row_keys_clear turns the row's scores into keys
// and empties every slot past its candidates once row_setup knows them.
template <int PER>
__device__ __forceinline__ void row_keys_load(const TopkArgs& a, int64_t row, int g, int tid, uint32_t (&key)[PER]) {
  const int64_t navail = a.bs_ld - a.n_init;
  const float* row_bs = a.bs + ((int64_t)g * a.rows_q + row) * a.bs_ld + a.n_init;
  if (navail > 0) {
#pragma unroll
    for (int p = 0; p < PER; ++p) key[p] = __float_as_uint(row_bs[min((int64_t)(PER * tid + p), navail - 1)]);
  } else {
#pragma unroll
    for (int p = 0; p < PER; ++p) key[p] = 0u;
  }
}
// After row_setup with done == false (so nc > n_topk >= 1 and every one of
// the nc candidates was read): order-preserving keys (bits + 1), 0 = empty.
template <int PER>
__device__ __forceinline__ void row_keys_clear(const RowSetup& rs, int tid, uint32_t (&key)[PER]) {
#pragma unroll
  for (int p = 0; p < PER; ++p) key[p] = PER * tid + p < rs.nc ? key[p] + 1u : 0u;
}

}  // namespace
}  // namespace infllmv2
