// Backward of the block-sparse (and dense) causal attention on bf16 MFMA.
//
// The method trains through its sparse attention (reading notes
// "论文阅读：InfLLM-V2", section "训练是怎么做的": long-context fine-tuning
// with the plain next-token objective).  The block selection is a top-k,
// piecewise constant in q and k, so the gradient flows through the
// attention over the selected blocks only, with the block sets fixed.  For
// one query row and head with probabilities P over its key set and upstream
// gradient dO (chain rule through the softmax Jacobian):
//   dV_u += P_u dO,   dS_u = P_u (dO . v_u - D),   D = dO . o,
//   dQ = scale * sum_u dS_u k_u,   dK_u += scale * dS_u q.
// P is recomputed from the forward's LSE.  Passes:
//  1. prep: log2-scaled LSE and D per (row, head); Q and dO of every
//     (row, KV group) transposed to [dim][head], the layout of the
//     head-contracting products of pass 3;
//  2. masks: for each tile of 16 query rows, the 16-bit mask of its tokens
//     attending every block (the forward's sets: init, local, list entries
//     read as a set; dense: every causal block), transposed block-major;
//     token counts per block split into work items of at most kBwdChunk
//     tokens;
//  3. dK / dV, key-major: per work item two waves (half of the dims each)
//     stage its K / V block in LDS, stream the item's tokens (ascending) and
//     store their fp32 partial sums; dQ, query-major: the forward's tile layout, each block a tile's
//     tokens attend staged once in LDS;
//  4. each block's partial sums are added in item order (deterministic) and
//     rounded to bf16.
#include <algorithm>
#include <type_traits>

#include "kernels.hpp"
#include "tile_common.hpp"

namespace infllmv2 {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

// D(16x16 f32) += A(16x16 bf16) * B(16x16 bf16); lane l holds A row (l % 16)
// and B column (l % 16) with reduction slots 4*(l/16) .. +3, D column
// (l % 16) rows 4*(l/16) .. +3.
__device__ __forceinline__ floatx4 mfma16k16(s16x4 a, s16x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ s16x4 pack4(float x0, float x1, float x2, float x3) {
  uint2 w;
  w.x = pack_bf16x2(x0, x1);
  w.y = pack_bf16x2(x2, x3);
  return __builtin_bit_cast(s16x4, w);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// Pass 1: per (row, KV group) statistics and transposed operands.
// Workgroup: 4 waves, wave w takes row 4 * blockIdx.x + w of group blockIdx.y.
// Lane (h = lane / 4, quarter lane % 4) loads dims 32*quarter .. +31 of head h.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[4][2][16 * kHeadDim];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave;
  const int g = blockIdx.y;
  const bool valid = r < a.rows_q;
  const int h = lane >> 2, quarter = lane & 3;
  const bool hv = valid && h < a.G;
  const int64_t base = (r * a.h_q + (int64_t)g * a.G + h) * kHeadDim + 32 * quarter;
  float dsum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4 qv = zero16(), dv = zero16(), ov = zero16();
    if (hv) {
      qv = ldg16(a.q + base + 8 * i);
      dv = ldg16(a.dout + base + 8 * i);
      ov = ldg16(a.out + base + 8 * i);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dsum += bf16_lo(dv[j]) * bf16_lo(ov[j]) + bf16_hi(dv[j]) * bf16_hi(ov[j]);
    *reinterpret_cast<u32x4*>(&tile[wave][0][h * kHeadDim + 32 * quarter + 8 * i]) = qv;
    *reinterpret_cast<u32x4*>(&tile[wave][1][h * kHeadDim + 32 * quarter + 8 * i]) = dv;
  }
  dsum += __shfl_xor(dsum, 1);
  dsum += __shfl_xor(dsum, 2);
  if (valid && quarter == 0) {
    float l2 = __builtin_inff();     // padded heads and rows that attend nothing: P = 0
    if (h < a.G) {
      const float L = a.lse[(int64_t)(g * a.G + h) * a.rows_q + r];
      if (L > -__builtin_inff()) l2 = L * kLog2e;
    }
    a.lse2[(r * a.h_kv + g) * 16 + h] = l2;
    a.dd[(r * a.h_kv + g) * 16 + h] = h < a.G ? dsum : 0.f;
  }
  __syncthreads();
  if (!valid) return;
  // Lane l = 16*q4 + c16 writes the 32 values its MFMA operand lane reads
  // in pass 3: dims 16*dt + c16 (dt = 0..7) of heads 4*q4 .. 4*q4+3.
  const int c16 = lane & 15, q4 = lane >> 4;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    uint32_t w[16];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int hp = 0; hp < 2; ++hp) {
        const uint32_t lo = tile[wave][which][(4 * q4 + 2 * hp) * kHeadDim + 16 * dt + c16];
        const uint32_t hi = tile[wave][which][(4 * q4 + 2 * hp + 1) * kHeadDim + 16 * dt + c16];
        w[2 * dt + hp] = lo | (hi << 16);
      }
    uint16_t* dst = (which ? a.dot : a.qt) + (r * a.h_kv + g) * 2048 + (c16 * 4 + q4) * 32;
#pragma unroll
    for (int m = 0; m < 4; ++m) stg16(dst + 8 * m, u32x4{w[4 * m], w[4 * m + 1], w[4 * m + 2], w[4 * m + 3]});
  }
}

// ---------------------------------------------------------------------------
// Pass 2a: token masks of one 16-row tile for every block of the sequence.
// Grid (ntiles, h_kv, batch).  Rows are the forward's sets: init and local
// blocks by arithmetic, list entries b with 0 <= b <= b_t as a set.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_mask_kernel(BwdArgs a) {
  __shared__ uint32_t mask[kBwdMaxBlocks];
  const int tile = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x;
  const SeqRange rq = seq_range(a.cu_q, a.used_q, s);
  const SeqRange rk = seq_range(a.cu_k, a.used_k, s);
  const int pos0 = rk.len - rq.len;
  const int i0 = 16 * tile;
  const int nq = max(0, min(16, rq.len - i0));
  const bool dense = a.bidx == nullptr;
  for (int b = tid; b < a.nblk; b += 256) {
    uint32_t m = 0;
    for (int tk = 0; tk < nq; ++tk) {
      const int t = pos0 + i0 + tk;
      if (t < 0 || (int64_t)rq.start + i0 + tk >= a.rows_q) continue;
      const int bt = t / kBlock;
      const bool rel = b <= bt && (dense || b < a.n_init || b >= bt - a.n_local + 1);
      m |= (uint32_t)rel << tk;
    }
    mask[b] = m;
  }
  __syncthreads();
  if (!dense) {
    const int tk = tid >> 4;
    const int t = pos0 + i0 + tk;
    const int64_t row = (int64_t)rq.start + i0 + tk;
    if (tk < nq && t >= 0 && row < a.rows_q) {
      const int bt = t / kBlock;
      const int32_t* list = a.bidx + ((int64_t)g * a.rows_q + row) * a.n_sel;
      for (int e = tid & 15; e < a.n_sel; e += 16) {
        const int b = list[e];
        if (b >= 0 && b <= bt && b < a.nblk) atomicOr(&mask[b], 1u << tk);
      }
    }
  }
  __syncthreads();
  uint16_t* dst = a.mask_t + (((int64_t)g * a.batch + s) * a.ntiles + tile) * a.nblk;
  for (int b = tid; b < a.nblk; b += 256) dst[b] = (uint16_t)mask[b];
}

// Pass 2b: [ntiles][nblk] -> [nblk][ntiles] per (group, sequence), 64 x 64 tiles.
__global__ __launch_bounds__(256) void bwd_mask_transpose_kernel(BwdArgs a) {
  __shared__ uint16_t t[64][66];
  const int b0 = blockIdx.x * 64, t0 = blockIdx.y * 64;
  const int64_t gs = blockIdx.z;
  const uint16_t* src = a.mask_t + gs * a.ntiles * a.nblk;
  uint16_t* dst = a.mask_b + gs * a.nblk * a.ntiles;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;
    t[r][c] = (t0 + r < a.ntiles && b0 + c < a.nblk) ? src[(int64_t)(t0 + r) * a.nblk + b0 + c] : 0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;
    if (b0 + r < a.nblk && t0 + c < a.ntiles) dst[(int64_t)(b0 + r) * a.ntiles + t0 + c] = t[c][r];
  }
}

// Pass 2c: tokens per (group, sequence, block) -> work items of kBwdChunk.
__global__ __launch_bounds__(256) void bwd_count_kernel(BwdArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + wave;
  if (b >= a.nblk) return;
  const int64_t e = ((int64_t)blockIdx.y * a.batch + blockIdx.z) * a.nblk + b;
  const uint16_t* row = a.mask_b + e * a.ntiles;
  int tot = 0;
  for (int t = lane; t < a.ntiles; t += 64) tot += __builtin_popcount((uint32_t)row[t]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
  if (lane == 0) a.items[e] = (tot + kBwdChunk - 1) / kBwdChunk;
}

// Pass 2d: one workgroup lays the items out as a list (block-major).
__global__ __launch_bounds__(1024) void bwd_list_kernel(BwdArgs a) {
  __shared__ int32_t sc[1024];
  const int tid = threadIdx.x;
  const int64_t n = (int64_t)a.h_kv * a.batch * a.nblk;
  int64_t run = 0;
  for (int64_t base = 0; base < n; base += 1024) {
    const int64_t i = base + tid;
    const int c = i < n ? a.items[i] : 0;
    sc[tid] = c;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {   // inclusive scan (Hillis-Steele)
      const int v = tid >= o ? sc[tid - o] : 0;
      __syncthreads();
      sc[tid] += v;
      __syncthreads();
    }
    const int64_t excl = run + sc[tid] - c;
    if (i < n) a.item_off[i] = (int32_t)(excl < a.wmax ? excl : a.wmax);
    for (int j = 0; j < c; ++j) {
      if (excl + j < a.wmax) {
        a.work[2 * (excl + j)] = (int32_t)i;
        a.work[2 * (excl + j) + 1] = j;
      }
    }
    run += sc[1023];
    __syncthreads();
  }
  if (tid == 0) *a.nwork = (int32_t)(run < a.wmax ? run : a.wmax);
}

// ---------------------------------------------------------------------------
// Pass 3a: dK, dV of one block for the tokens of one work item.  Two waves:
// wave w owns dims 64w .. 64w+63 of the block's 64 x 128 dK and dV (128 fp32
// registers), so two such workgroups fit on a SIMD pair per slot.  Products
// with heads on the 16-wide side:
//   S  = Q K^T        (16 heads x 16 keys per MFMA, contraction over dims)
//   dP = dO V^T
//   dV += P^T dO,  dK += dS^T Q   (16 keys x 16 dims, contraction over heads)
// S and dP come out with lane (c16 = key, q4 -> heads 4*q4 .. +3), exactly
// the A layout of the head-contracting 16x16x16 products, whose B operands
// are the lane-ordered copies of Q and dO written by pass 1.  Both waves
// compute S and dP (the full contraction over dims) from the K / V block
// staged once in LDS; the item's tokens are listed in LDS first.  The
// partial sums go to the item's own slot of the workspace (no atomics).
// ---------------------------------------------------------------------------
constexpr int kDkvWaves = 2;

__global__ __launch_bounds__(64 * kDkvWaves) void bwd_dkdv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t kv[2][64 * 256];
  __shared__ int32_t toks[kBwdChunk];
  __shared__ int32_t tok_count;
  const int item = blockIdx.x;
  if (item >= *a.nwork) return;
  const int e = a.work[2 * item], chunk = a.work[2 * item + 1];
  const int b = e % a.nblk;
  const int gs = e / a.nblk;
  const int s = gs % a.batch, g = gs / a.batch;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, q4 = lane >> 4, c16 = lane & 15;
  const SeqRange rq = seq_range(a.cu_q, a.used_q, s);
  const SeqRange rk = seq_range(a.cu_k, a.used_k, s);
  const int pos0 = rk.len - rq.len;

  // K and V of block b staged in LDS as [key][dim] rows (16-byte chunk p of
  // row r at slot p ^ (r & 7), so 8 consecutive rows read together hit
  // distinct banks); keys past the sequence are zero rows.  Each wave stages
  // 8 of the 16 parts of 4 rows.
  {
    const int64_t gstride = (int64_t)a.h_kv * kHeadDim;
    const uint16_t* kb = a.k + (((int64_t)rk.start + kBlock * b) * a.h_kv + g) * kHeadDim;
    const uint16_t* vb = a.v + (((int64_t)rk.start + kBlock * b) * a.h_kv + g) * kHeadDim;
    const bool inside = kBlock * b + kBlock <= rk.len && (int64_t)rk.start + kBlock * b + kBlock <= a.rows_k;
#pragma unroll
    for (int j = 0; j < 16 / kDkvWaves; ++j) {
      const int part = wave + kDkvWaves * j;
      const int row = 4 * part + (lane >> 4);
      const int64_t off = row * gstride + 8 * ((lane & 15) ^ (row & 7));
      if (inside) {
        __builtin_amdgcn_global_load_lds(kb + off, (__attribute__((address_space(3))) void*)(kv[0] + part * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vb + off, (__attribute__((address_space(3))) void*)(kv[1] + part * 1024), 16, 0, 0);
      } else {
        const bool in = kBlock * b + row < rk.len && (int64_t)rk.start + kBlock * b + row < a.rows_k;
        const u32x4 xk = in ? ldg16(kb + off) : zero16();
        const u32x4 xv = in ? ldg16(vb + off) : zero16();
        *reinterpret_cast<u32x4*>(kv[0] + part * 1024 + 16 * lane) = xk;
        *reinterpret_cast<u32x4*>(kv[1] + part * 1024 + 16 * lane) = xv;
      }
    }
  }

  // The item's tokens (wave 0): ordinals [chunk * kBwdChunk, +kBwdChunk) of
  // the block's tokens in ascending (tile, row) order.
  if (wave == 0) {
    const uint16_t* mrow = a.mask_b + (int64_t)e * a.ntiles;
    const int ntile_s = min((rq.len + 15) / 16, a.ntiles);
    const int target = chunk * kBwdChunk, target_end = target + kBwdChunk;
    int run = 0;
    for (int tau = max(0, kBlock * b - pos0) / 16; tau < ntile_s && run < target_end; tau += 64) {
      const uint32_t m = tau + lane < ntile_s ? mrow[tau + lane] : 0u;
      const int c = __builtin_popcount(m);
      int incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      const int tot = __shfl(incl, 63);
      if (run + tot > target) {
        int ord = run + incl - c;
        uint32_t mm = m;
        while (mm != 0u) {
          const int bit = (int)__builtin_ctz(mm);
          mm &= mm - 1;
          if (ord >= target && ord < target_end) toks[ord - target] = 16 * (tau + lane) + bit;
          ++ord;
        }
      }
      run += tot;
    }
    if (lane == 0) tok_count = max(0, min(run, target_end) - target);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  const int count = tok_count;

  // B operand (key tile kt, dims 32ks + 8q4 .. +7) of row 16kt + c16.
  auto frag = [&](int which, int kt, int ks) {
    const int row = 16 * kt + c16;
    return as_bf16x8(*reinterpret_cast<const u32x4*>(kv[which] + row * 256 + (((4 * ks + q4) ^ (row & 7)) << 4)));
  };
  floatx4 dk[4][4], dv[4][4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int dl = 0; dl < 4; ++dl) {
      dk[kt][dl] = floatx4{0.f, 0.f, 0.f, 0.f};
      dv[kt][dl] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

  const bool hv = c16 < a.G;
  // Operands of one token; the next token's are in flight while the current
  // one computes.
  struct Ops {
    u32x4 qa[4], da[4];     // Q, dO as A operands (dims 32ks + 8q4 .. +7 of head c16)
    u32x4 qt[2], dt[2];     // this wave's dim tiles of Q, dO as [dim][head] B operands
    floatx4 l2, dd;         // LSE * log2(e) and D of heads 4q4 .. +3
  };
  auto load = [&](int i, Ops& o) {
    const int64_t r = (int64_t)rq.start + i;
    const int64_t qoff = (r * a.h_q + (int64_t)g * a.G + c16) * kHeadDim + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      o.qa[ks] = hv ? ldg16(a.q + qoff + 32 * ks) : zero16();
      o.da[ks] = hv ? ldg16(a.dout + qoff + 32 * ks) : zero16();
    }
    const int64_t toff = (r * a.h_kv + g) * 2048 + (c16 * 4 + q4) * 32 + 16 * wave;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      o.qt[m] = ldg16(a.qt + toff + 8 * m);
      o.dt[m] = ldg16(a.dot + toff + 8 * m);
    }
    const int64_t soff = (r * a.h_kv + g) * 16 + 4 * q4;
    o.l2 = *reinterpret_cast<const floatx4*>(a.lse2 + soff);
    o.dd = *reinterpret_cast<const floatx4*>(a.dd + soff);
  };
  auto compute = [&](int i, const Ops& o) {
    const int t = pos0 + i;
    s16x4 pa[4], dsa[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      floatx4 sc = floatx4{0.f, 0.f, 0.f, 0.f}, dp = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        sc = mfma16(as_bf16x8(o.qa[ks]), frag(0, kt, ks), sc);
        dp = mfma16(as_bf16x8(o.da[ks]), frag(1, kt, ks), dp);
      }
      const bool vis = kBlock * b + 16 * kt + c16 <= t;
      float p[4], ds[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = vis ? fast_exp2(fmaf(sc[j], a.c, -o.l2[j])) : 0.f;
        ds[j] = vis ? p[j] * (dp[j] - o.dd[j]) : 0.f;
      }
      pa[kt] = pack4(p[0], p[1], p[2], p[3]);
      dsa[kt] = pack4(ds[0], ds[1], ds[2], ds[3]);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int dl = 2 * m + h;
        const s16x4 qv = __builtin_bit_cast(s16x4, uint2{o.qt[m][2 * h], o.qt[m][2 * h + 1]});
        const s16x4 dv4 = __builtin_bit_cast(s16x4, uint2{o.dt[m][2 * h], o.dt[m][2 * h + 1]});
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          dv[kt][dl] = mfma16k16(pa[kt], dv4, dv[kt][dl]);
          dk[kt][dl] = mfma16k16(dsa[kt], qv, dk[kt][dl]);
        }
      }
    }
  };
  Ops A, B;
  if (count > 0) load(toks[0], A);
  for (int x = 0; x < count; x += 2) {
    if (x + 1 < count) load(toks[x + 1], B);
    compute(toks[x], A);
    if (x + 1 < count) {
      if (x + 2 < count) load(toks[x + 2], A);
      compute(toks[x + 1], B);
    }
  }

  // Partial sums of this item: floatx4 (which, kt, dt) of every lane,
  // lane-major; this wave holds dim tiles dt = 4*wave + dl.
  float* part = a.part + (int64_t)item * 16384 + 4 * lane;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int dl = 0; dl < 4; ++dl) {
      const int dtile = 4 * wave + dl;
      *reinterpret_cast<floatx4*>(part + (kt * 8 + dtile) * 256) = dk[kt][dl] * a.scale;
      *reinterpret_cast<floatx4*>(part + ((4 + kt) * 8 + dtile) * 256) = dv[kt][dl];
    }
}

// ---------------------------------------------------------------------------
// Pass 4: dK (blockIdx.y = 0) or dV (1) of one block: the partial sums of its
// items added in item order, rounded to bf16, written row by row.  Blocks no
// row attends get zeros.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a) {
  __shared__ float blk[64][kHeadDim + 4];
  const int e = blockIdx.x, which = blockIdx.y;
  const int b = e % a.nblk;
  const int gs = e / a.nblk;
  const int s = gs % a.batch, g = gs / a.batch;
  const SeqRange rk = seq_range(a.cu_k, a.used_k, s);
  if (kBlock * b >= rk.len) return;
  const int n_items = a.items[e], first = a.item_off[e];
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int f = tid + 256 * k;             // (kt, dt) = f / 64, lane = f % 64
    const int kt = f >> 9, dt = (f >> 6) & 7, ln = f & 63;
    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
    const float* src = a.part + (int64_t)first * 16384 + ((which * 4 + kt) * 8 + dt) * 256 + 4 * ln;
    for (int j = 0; j < n_items; ++j) acc += *reinterpret_cast<const floatx4*>(src + (int64_t)j * 16384);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) blk[16 * kt + 4 * (ln >> 4) + jj][16 * dt + (ln & 15)] = acc[jj];
  }
  __syncthreads();
  uint16_t* dst = which ? a.dv : a.dk;
  for (int c = tid; c < 64 * 16; c += 256) {
    const int row = c >> 4, ch = c & 15;
    const int key = kBlock * b + row;
    if (key >= rk.len || (int64_t)rk.start + key >= a.rows_k) continue;
    const float* x = &blk[row][8 * ch];
    stg16(dst + (((int64_t)rk.start + key) * a.h_kv + g) * kHeadDim + 8 * ch,
          u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                pack_bf16x2(x[6], x[7])});
  }
}

// ---------------------------------------------------------------------------
// Pass 3b: dQ, query-major.  Per workgroup 16 consecutive query rows of one
// sequence and one KV group, 8 waves of 2 rows, as in the forward.  The
// blocks any row attends (from the mask table) are staged once in an LDS
// ring, K and V both as [key][dim] (XOR-swizzled, direct global->LDS
// loads), in batches of two with one barrier per batch; a wave computes for
// its rows that attend the block
//   S^T = K Q^T,  dP^T = V dO^T,  dS^T = P^T (dP^T - D),  dQ^T += K^T dS^T,
// where the K^T fragments (8 consecutive keys of one dim) are gathered from
// the staged [key][dim] tile with 16-bit LDS reads.
// ---------------------------------------------------------------------------
typedef uint32_t uint32x2_t __attribute__((ext_vector_type(2)));
constexpr int kDqWaves = 8;
constexpr int kDqTPW = 2;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqWin = 2048;
constexpr int kDqRing = 4;
constexpr int kDqShareMin = 2;   // rows of the tile attending a block for the shared phase

struct DqLds {
  // Shared phase: slot r holds a K block at ring[r][0] and its V at
  // ring[r][1].  Private phase: wave w owns the 16 KB at (ring[0][0] +
  // 16 KB * w) for the K block it is streaming.
  uint8_t ring[kDqRing][2][64 * 256];
  uint32_t mask[kDqWin];
  int32_t ub[kDqWin];
  uint32_t um[kDqWin];
  int32_t cnt[kDqWin / kDqThreads][kDqWaves];
  int32_t pcnt[16];   // private blocks per tile row
  int32_t perm[16];   // tile row of each wave slot 2w + k
};

struct Dq {
  const BwdArgs& a;
  int s, g, lane, q4, c16, wave;
  SeqRange rq, rk;
  int tpos[kDqTPW], bt[kDqTPW];
  int64_t trow[kDqTPW];
  bool tval[kDqTPW];
  bf16x8 qb[kDqTPW][4], db[kDqTPW][4];
  floatx4 acc[kDqTPW][8];
  float l2[kDqTPW], dd[kDqTPW];
  int tb[kDqTPW];     // tile row (mask bit) of each of the wave's rows
  const uint16_t* kbase;
  const uint16_t* vbase;
  int64_t krow;
  int klo[2];
  int koff[4];
  int trlb, trs2;    // K^T transposed reads: lane byte base and chunk swizzle

  __device__ Dq(const BwdArgs& args) : a(args) {}

  // Mask bits of this wave's rows, gathered into bits 0 .. kDqTPW-1.
  __device__ __forceinline__ uint32_t sel_of(uint32_t v) const {
    uint32_t r = 0;
#pragma unroll
    for (int k = 0; k < kDqTPW; ++k) r |= ((v >> tb[k]) & 1u) << k;
    return r;
  }
  __device__ __forceinline__ uint32_t mine_mask() const {
    uint32_t r = 0;
#pragma unroll
    for (int k = 0; k < kDqTPW; ++k) r |= 1u << tb[k];
    return r;
  }
  // State of row k of this wave: tile row tt (query row i0 + tt).
  __device__ __forceinline__ void init_token(int k, int tt, int i0, int pos0) {
    tb[k] = tt;
    const int i = i0 + tt;
    tpos[k] = pos0 + i;
    trow[k] = (int64_t)rq.start + i;
    tval[k] = i < rq.len && trow[k] < a.rows_q && tpos[k] >= 0;
    bt[k] = tval[k] ? tpos[k] / kBlock : -1;
    const bool hv = tval[k] && c16 < a.G;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 vq = zero16(), vd = zero16();
      if (hv) {
        const int64_t o = (trow[k] * a.h_q + (int64_t)g * a.G + c16) * kHeadDim + 32 * ks + 8 * q4;
        vq = ldg16(a.q + o);
        vd = ldg16(a.dout + o);
      }
      qb[k][ks] = as_bf16x8(vq);
      db[k][ks] = as_bf16x8(vd);
    }
    l2[k] = __builtin_inff();
    dd[k] = 0.f;
    if (tval[k]) {
      l2[k] = a.lse2[(trow[k] * a.h_kv + g) * 16 + c16];
      dd[k] = a.dd[(trow[k] * a.h_kv + g) * 16 + c16];
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[k][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  __device__ __forceinline__ void init_offsets() {
    krow = (int64_t)a.h_kv * kHeadDim;
    kbase = a.k + ((int64_t)rk.start * a.h_kv + g) * kHeadDim;
    vbase = a.v + ((int64_t)rk.start * a.h_kv + g) * kHeadDim;
#pragma unroll
    for (int v = 0; v < 2; ++v)
      klo[v] = (lane >> 4) * (int)krow + 8 * ((lane & 15) ^ (((lane >> 4) & 3) | (4 * v)));
    const int key0 = 8 * (c16 >> 2) + (c16 & 3);
    const int sw = swz_k(key0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) koff[ks] = key0 * 256 + (((4 * ks + q4) ^ sw) << 4);
    // K^T fragment (dt, kk): element j is K[key 32kk + 8q4 + j][dim 16dt + c16].
    // gfx950's transposed LDS read (ds_read_b64_tr_b16) hands lane i of a
    // 16-lane group element j of the 8 bytes read by lane 4j + i/4, taken at
    // position i % 4.  So lane L of group q4 reads the 4 dims 16dt + 4(L%4) ..
    // +3 of key row 32kk + 8q4 + L/4 (+4 for elements 4..7); in the swizzled
    // tile that row's chunk (2dt + (L%4)/2) sits at chunk (2dt) ^ trs2, with
    // the row's swizzle (L/4 | 4(q4&1): the row's low bits come from L/4 and
    // q4 alone) folded into trs2.
    trlb = (8 * q4 + (c16 >> 2)) * 256 + 8 * (c16 & 1);
    trs2 = ((c16 >> 2) | ((q4 & 1) << 2)) ^ ((c16 & 3) >> 1);
  }

  static __device__ __forceinline__ bf16x8 lds16(const uint8_t* p) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(p));
  }

  __device__ __forceinline__ bool k_inside(int b) const {
    return (int64_t)rk.start + kBlock * b + kBlock <= a.rows_k;
  }
  // One 1 KB part (4 rows) of block b of tensor `base` into lt + 1024 * part,
  // rows clamped to the tensor.
  __device__ __forceinline__ void stage_part_clamped(uint8_t* lt, const uint16_t* tensor, int b, int part) const {
    const int key = 4 * part + (lane >> 4);
    int64_t r = (int64_t)rk.start + kBlock * b + key;
    r = r < a.rows_k ? r : a.rows_k - 1;
    __builtin_amdgcn_global_load_lds(tensor + (r * a.h_kv + g) * kHeadDim + 8 * ((lane & 15) ^ swz_k(key)),
                                     (__attribute__((address_space(3))) void*)(lt + part * 1024), 16, 0, 0);
  }
  // Stage K and V of block b: every wave writes two 1 KB parts of each.
  __device__ __forceinline__ void stage_issue(uint8_t* lk, uint8_t* lv, int b) const {
    if (k_inside(b)) {
      const int lo0 = opaque(klo[0]), lo1 = opaque(klo[1]);
      const uint16_t* bk = kbase + (int64_t)(kBlock * b) * krow;
      const uint16_t* bv = vbase + (int64_t)(kBlock * b) * krow;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int part = wave + kDqWaves * j;
        const int64_t o = (int64_t)(4 * part) * krow + ((part & 2) ? lo1 : lo0);
        __builtin_amdgcn_global_load_lds(bk + o, (__attribute__((address_space(3))) void*)(lk + part * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(bv + o, (__attribute__((address_space(3))) void*)(lv + part * 1024), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        stage_part_clamped(lk, a.k, b, wave + kDqWaves * j);
        stage_part_clamped(lv, a.v, b, wave + kDqWaves * j);
      }
    }
  }

  // Zero the K rows of a staged block at or past the sequence end: the K^T
  // product contracts over keys, and rows past the end may hold anything.
  __device__ __forceinline__ void zero_tail(uint8_t* lk, int b) const {
    const int first = rk.len - kBlock * b;
    for (int c = threadIdx.x; c < 64 * 16; c += kDqThreads) {
      const int row = c >> 4;
      if (row >= first) *reinterpret_cast<u32x4*>(lk + row * 256 + ((c & 15) << 4)) = zero16();
    }
  }

  // K^T fragment (dt, kk) from the staged K tile: two transposed reads,
  // keys 32kk + 8q4 + 0..3 and + 4..7 (see init_offsets).
  template <int dt, int kk>
  __device__ __forceinline__ bf16x8 kt_frag(const uint8_t* lk) const {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const uint8_t* p = lk + trlb + 16 * ((2 * dt) ^ trs2) + 8192 * kk;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 1024));
    const uint32x2_t wl = __builtin_bit_cast(uint32x2_t, lo), wh = __builtin_bit_cast(uint32x2_t, hi);
    return as_bf16x8(u32x4{wl[0], wl[1], wh[0], wh[1]});
  }

  // Private phase: this wave alone stages K block b into its LDS region
  // (16 direct global->LDS loads of 1 KB, the shared phase's layout).
  __device__ __forceinline__ void issue_k_private(uint8_t* lk, int b) const {
    if (k_inside(b)) {
      const int lo0 = opaque(klo[0]), lo1 = opaque(klo[1]);
      const uint16_t* bk = kbase + (int64_t)(kBlock * b) * krow;
#pragma unroll
      for (int part = 0; part < 16; ++part)
        __builtin_amdgcn_global_load_lds(bk + (int64_t)(4 * part) * krow + ((part & 2) ? lo1 : lo0),
                                         (__attribute__((address_space(3))) void*)(lk + part * 1024), 16, 0, 0);
    } else {
#pragma unroll
      for (int part = 0; part < 16; ++part) stage_part_clamped(lk, a.k, b, part);
    }
  }
  // Private phase: the V fragments of block b straight into registers, in
  // the A-operand layout the shared phase reads from LDS (fragment (kt, ks):
  // key row key0 + 32 (kt / 2) + 4 (kt % 2), dims 32 ks + 8 q4 .. +8), rows
  // clamped to the tensor.
  __device__ __forceinline__ void load_v_private(u32x4 (&vb)[4][4], int b) const {
    const int key0 = 8 * (c16 >> 2) + (c16 & 3);
    if (k_inside(b)) {
      const uint16_t* p = vbase + (int64_t)(kBlock * b + key0) * krow + 8 * q4;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          vb[kt][ks] = ldg16(p + (int64_t)(32 * (kt >> 1) + 4 * (kt & 1)) * krow + 32 * ks);
    } else {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        int64_t r = (int64_t)rk.start + kBlock * b + key0 + 32 * (kt >> 1) + 4 * (kt & 1);
        r = r < a.rows_k ? r : a.rows_k - 1;
        const uint16_t* p = a.v + (r * a.h_kv + g) * kHeadDim + 8 * q4;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) vb[kt][ks] = ldg16(p + 32 * ks);
      }
    }
  }
  // Zero this wave's staged K rows at or past the sequence end (see zero_tail).
  __device__ __forceinline__ void zero_tail_private(uint8_t* lk, int b) const {
    const int first = rk.len - kBlock * b;
    for (int c = lane; c < 64 * 16; c += 64) {
      const int row = c >> 4;
      if (row >= first) *reinterpret_cast<u32x4*>(lk + row * 256 + ((c & 15) << 4)) = zero16();
    }
  }

  // Private phase, block b for the rows of this wave in sel: K from the
  // wave's region, V from registers.
  __device__ __forceinline__ void consume_private(uint32_t sel, const uint8_t* lk, const u32x4 (&vb)[4][4], int b) {
#pragma unroll
    for (int k = 0; k < kDqTPW; ++k) {
      if (!((sel >> k) & 1u)) continue;
      const bool diag = b == bt[k];
      const int lim = tpos[k] - kBlock * b - 8 * q4;
      bf16x8 dsb[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float ds[2][4];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kt = 2 * kk + half;
          const int roff = 256 * (32 * (kt >> 1) + 4 * (kt & 1));
          floatx4 st = floatx4{0.f, 0.f, 0.f, 0.f}, dp = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            st = mfma16(lds16(lk + koff[ks] + roff), qb[k][ks], st);
            dp = mfma16(as_bf16x8(vb[kt][ks]), db[k][ks], dp);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool vis = !diag || 32 * (kt >> 1) + 4 * (kt & 1) + r <= lim;
            const float pr = fast_exp2(fmaf(st[r], a.c, -l2[k]));
            ds[half][r] = vis ? pr * (dp[r] - dd[k]) : 0.f;
          }
        }
        u32x4 w;
        w[0] = pack_bf16x2(ds[0][0], ds[0][1]);
        w[1] = pack_bf16x2(ds[0][2], ds[0][3]);
        w[2] = pack_bf16x2(ds[1][0], ds[1][1]);
        w[3] = pack_bf16x2(ds[1][2], ds[1][3]);
        dsb[kk] = as_bf16x8(w);
      }
      auto step = [&](auto dtc, auto kkc) {
        constexpr int dt = decltype(dtc)::value, kk = decltype(kkc)::value;
        acc[k][dt] = mfma16(kt_frag<dt, kk>(lk), dsb[kk], acc[k][dt]);
      };
      auto dts = [&](auto kkc) {
        step(std::integral_constant<int, 0>{}, kkc);
        step(std::integral_constant<int, 1>{}, kkc);
        step(std::integral_constant<int, 2>{}, kkc);
        step(std::integral_constant<int, 3>{}, kkc);
        step(std::integral_constant<int, 4>{}, kkc);
        step(std::integral_constant<int, 5>{}, kkc);
        step(std::integral_constant<int, 6>{}, kkc);
        step(std::integral_constant<int, 7>{}, kkc);
      };
      dts(std::integral_constant<int, 0>{});
      dts(std::integral_constant<int, 1>{});
    }
  }

  // Block b (K at lk, V at lv) for the rows of this wave in sel.
  __device__ __forceinline__ void consume(uint32_t sel, const uint8_t* lk, const uint8_t* lv, int b) {
    bf16x8 dsb[kDqTPW][2];
#pragma unroll
    for (int k = 0; k < kDqTPW; ++k) {
      if (!((sel >> k) & 1u)) continue;
      const bool diag = b == bt[k];
      const int lim = tpos[k] - kBlock * b - 8 * q4;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float ds[2][4];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kt = 2 * kk + half;
          const int roff = 256 * (32 * (kt >> 1) + 4 * (kt & 1));
          floatx4 st = floatx4{0.f, 0.f, 0.f, 0.f}, dp = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            st = mfma16(lds16(lk + koff[ks] + roff), qb[k][ks], st);
            dp = mfma16(lds16(lv + koff[ks] + roff), db[k][ks], dp);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool vis = !diag || 32 * (kt >> 1) + 4 * (kt & 1) + r <= lim;
            // (selects, not products: keys past the sequence may hold anything)
            const float pr = fast_exp2(fmaf(st[r], a.c, -l2[k]));
            ds[half][r] = vis ? pr * (dp[r] - dd[k]) : 0.f;
          }
        }
        u32x4 w;
        w[0] = pack_bf16x2(ds[0][0], ds[0][1]);
        w[1] = pack_bf16x2(ds[0][2], ds[0][3]);
        w[2] = pack_bf16x2(ds[1][0], ds[1][1]);
        w[3] = pack_bf16x2(ds[1][2], ds[1][3]);
        dsb[k][kk] = as_bf16x8(w);
      }
    }
    auto step = [&](auto dtc, auto kkc) {
      constexpr int dt = decltype(dtc)::value, kk = decltype(kkc)::value;
      const bf16x8 f = kt_frag<dt, kk>(lk);
#pragma unroll
      for (int k = 0; k < kDqTPW; ++k)
        if ((sel >> k) & 1u) acc[k][dt] = mfma16(f, dsb[k][kk], acc[k][dt]);
    };
    auto dts = [&](auto kkc) {
      step(std::integral_constant<int, 0>{}, kkc);
      step(std::integral_constant<int, 1>{}, kkc);
      step(std::integral_constant<int, 2>{}, kkc);
      step(std::integral_constant<int, 3>{}, kkc);
      step(std::integral_constant<int, 4>{}, kkc);
      step(std::integral_constant<int, 5>{}, kkc);
      step(std::integral_constant<int, 6>{}, kkc);
      step(std::integral_constant<int, 7>{}, kkc);
    };
    dts(std::integral_constant<int, 0>{});
    dts(std::integral_constant<int, 1>{});
  }

  // kMulti: keys beyond one window of kDqWin blocks; that instance loops over
  // windows and keeps every block in the shared phase (a loop around both
  // phases would keep their registers live at once).
  template <bool kMulti>
  __device__ void run(DqLds& sh) {
    const int tile = blockIdx.x;
    g = blockIdx.y;
    s = blockIdx.z;
    rq = seq_range(a.cu_q, a.used_q, s);
    rk = seq_range(a.cu_k, a.used_k, s);
    const int i0 = 16 * tile;
    if (i0 >= rq.len) return;
    const int pos0 = rk.len - rq.len;
    const int tid = threadIdx.x;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    lane = tid & 63;
    q4 = lane >> 4;
    c16 = lane & 15;
    init_offsets();
    // The multi-window instance keeps row 2w + k on wave w; the single-window
    // one assigns the rows once the masks are known (below).
    if constexpr (kMulti) {
#pragma unroll
      for (int k = 0; k < kDqTPW; ++k) init_token(k, wave * kDqTPW + k, i0, pos0);
    }

    const int nq = min(16, rq.len - i0);
    const int bt_last = min(max(0, pos0 + i0 + nq - 1) / kBlock, a.nblk - 1);
    const uint16_t* mrow = a.mask_t + (((int64_t)g * a.batch + s) * a.ntiles + tile) * a.nblk;
    const int w_last = kMulti ? bt_last : 0;
    for (int w0 = 0; w0 <= w_last; w0 += kDqWin) {
      const int w1 = min(bt_last + 1, w0 + kDqWin);
      const int nblk = w1 - w0;
      for (int e = tid; e < kDqWin; e += kDqThreads) sh.mask[e] = e < nblk ? mrow[w0 + e] : 0u;
      if (!kMulti && tid < 16) sh.pcnt[tid] = 0;
      __syncthreads();
      if constexpr (!kMulti) {
        // Balance the private phase: rows ranked by private block count are
        // paired heaviest with lightest, one pair per wave.
        for (int e = tid; e < nblk; e += kDqThreads) {
          const uint32_t v = sh.mask[e];
          if (v != 0u && __builtin_popcount(v) < kDqShareMin)
            for (uint32_t x = v; x != 0u; x &= x - 1u) atomicAdd(&sh.pcnt[__builtin_ctz(x)], 1);
        }
        __syncthreads();
        static_assert(kDqTPW == 2 && kDqWaves * kDqTPW == 16, "the pairing gives each wave two of 16 rows");
        if (wave == 0 && lane < 16) {
          const int c = sh.pcnt[lane];
          int rank = 0;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int cj = sh.pcnt[j];
            rank += (cj > c || (cj == c && j < lane)) ? 1 : 0;
          }
          sh.perm[rank < 8 ? kDqTPW * rank : kDqTPW * (15 - rank) + 1] = lane;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kDqTPW; ++k)
          init_token(k, __builtin_amdgcn_readfirstlane(sh.perm[wave * kDqTPW + k]), i0, pos0);
      }
      // Compact the attended blocks, ascending.
      uint64_t bal[kDqWin / kDqThreads];
#pragma unroll
      for (int j = 0; j < kDqWin / kDqThreads; ++j) {
        const int e = kDqThreads * j + tid;
        const uint32_t v = sh.mask[e];
        bal[j] = __ballot(v != 0u && (kMulti || __builtin_popcount(v) >= kDqShareMin));
        if (lane == 0) sh.cnt[j][wave] = __builtin_popcountll(bal[j]);
      }
      __syncthreads();
      int n_ent = 0;
#pragma unroll
      for (int j = 0; j < kDqWin / kDqThreads; ++j) {
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kDqWaves; ++w) {
          const int c = sh.cnt[j][w];
          before += w < wave ? c : 0;
          total += c;
        }
        if ((bal[j] >> lane) & 1ull) {
          const int e = kDqThreads * j + tid;
          const int pos = n_ent + before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[j] >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bal[j], 0u));
          sh.ub[pos] = w0 + e;
          sh.um[pos] = sh.mask[e];
        }
        n_ent += total;
      }
      __syncthreads();
      // Order the list for balance: within each run of 64 entries an entry
      // is followed by the first later one whose rows lie in other waves
      // (else by the next one), so the two blocks of a batch tend to occupy
      // different waves.  Runs are 64 entries, so batches never straddle them.
      for (int c = wave; 64 * c < n_ent; c += kDqWaves) {
        const int cnt = min(64, n_ent - 64 * c);
        const bool ok = lane < cnt;
        const int32_t ubv = ok ? sh.ub[64 * c + lane] : 0;
        const uint32_t umv = ok ? sh.um[64 * c + lane] : 0u;
        uint32_t wm = 0;
#pragma unroll
        for (int w = 0; w < kDqWaves; ++w) {
          uint32_t wb = ((1u << kDqTPW) - 1u) << (kDqTPW * w);
          if constexpr (!kMulti) {
            wb = 0;
#pragma unroll
            for (int k = 0; k < kDqTPW; ++k) wb |= 1u << sh.perm[kDqTPW * w + k];
          }
          wm |= (uint32_t)((umv & wb) != 0u) << w;
        }
        const uint64_t valid = cnt == 64 ? ~0ull : ((1ull << cnt) - 1ull);
        uint64_t used = 0;
        int dest = 0, p = 0;
        for (int i = 0; i < cnt; ++i) {
          if ((used >> i) & 1ull) continue;
          used |= 1ull << i;
          dest = lane == i ? p : dest;
          ++p;
          const uint32_t aw = __builtin_amdgcn_readlane(wm, i);
          const uint64_t later = valid & ~used & ~((2ull << i) - 1ull);
          uint64_t cand = __ballot((wm & aw) == 0u) & later;
          if (cand == 0) cand = later;
          if (cand != 0) {
            const int j = (int)__builtin_ctzll(cand);
            used |= 1ull << j;
            dest = lane == j ? p : dest;
            ++p;
          }
        }
        if (ok) {
          sh.ub[64 * c + dest] = ubv;
          sh.um[64 * c + dest] = umv;
        }
      }
      __syncthreads();
      if (n_ent > 0) {
        stage_issue(sh.ring[0][0], sh.ring[0][1], sh.ub[0]);
        if (n_ent > 1) stage_issue(sh.ring[1][0], sh.ring[1][1], sh.ub[1]);
        for (int u = 0; u < n_ent; u += 2) {
          const int half = (u >> 1) & 1;
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
          __syncthreads();
          const int b0 = __builtin_amdgcn_readfirstlane(sh.ub[u]);
          const int b1 = u + 1 < n_ent ? __builtin_amdgcn_readfirstlane(sh.ub[u + 1]) : -1;
          const bool p0 = kBlock * b0 + kBlock > rk.len;
          const bool p1 = b1 >= 0 && kBlock * b1 + kBlock > rk.len;
          if (p0 || p1) {
            if (p0) zero_tail(sh.ring[2 * half][0], b0);
            if (p1) zero_tail(sh.ring[2 * half + 1][0], b1);
            __syncthreads();
          }
          if (u + 2 < n_ent) stage_issue(sh.ring[2 * (half ^ 1)][0], sh.ring[2 * (half ^ 1)][1], sh.ub[u + 2]);
          if (u + 3 < n_ent) stage_issue(sh.ring[2 * (half ^ 1) + 1][0], sh.ring[2 * (half ^ 1) + 1][1], sh.ub[u + 3]);
          const uint32_t m0 = sel_of(__builtin_amdgcn_readfirstlane(sh.um[u]));
          if (m0) consume(m0, sh.ring[2 * half][0], sh.ring[2 * half][1], b0);
          if (b1 >= 0) {
            const uint32_t m1 = sel_of(__builtin_amdgcn_readfirstlane(sh.um[u + 1]));
            if (m1) consume(m1, sh.ring[2 * half + 1][0], sh.ring[2 * half + 1][1], b1);
          }
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      }
      // Private phase: this wave's blocks that stayed out of the shared list,
      // ascending, one block in flight (K in the wave's region, V in
      // registers) while the previous one computes.
      if constexpr (!kMulti) {
        __syncthreads();   // the ring becomes the private regions
        uint8_t* region = &sh.ring[0][0][0] + wave * (64 * 256);
        const uint32_t mine = mine_mask();
        int chunk = 0;
        uint64_t pend = 0;
        // Next private block of this wave (wave-uniform), or -1.
        auto next_block = [&](uint32_t& sel) -> int {
          while (pend == 0) {
            if (chunk * 64 >= nblk) return -1;
            const int e = chunk * 64 + lane;
            const uint32_t v = e < nblk ? sh.mask[e] : 0u;
            pend = __ballot((v & mine) != 0u && __builtin_popcount(v) < kDqShareMin);
            ++chunk;
          }
          const int e = (chunk - 1) * 64 + (int)__builtin_ctzll(pend);
          pend &= pend - 1;
          sel = sel_of(__builtin_amdgcn_readfirstlane(sh.mask[e]));
          return w0 + e;
        };
        uint32_t sc = 0;
        int bc = next_block(sc);
        u32x4 vb[4][4];
        if (bc >= 0) {
          issue_k_private(region, bc);
          load_v_private(vb, bc);
        }
        while (bc >= 0) {
          uint32_t sn = 0;
          const int bn = next_block(sn);
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // K(bc) in the region, V(bc) in registers
          if (kBlock * bc + kBlock > rk.len) zero_tail_private(region, bc);
          consume_private(sc, region, vb, bc);
          if (bn >= 0) {
            __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0): the region's K reads are done
            issue_k_private(region, bn);
            load_v_private(vb, bn);
          }
          bc = bn;
          sc = sn;
        }
      }
      __syncthreads();   // the ring and the lists are reused by the next window
    }

#pragma unroll
    for (int k = 0; k < kDqTPW; ++k) {
      if (!tval[k] || c16 >= a.G) continue;
      uint16_t* dst = a.dq + (trow[k] * a.h_q + (int64_t)g * a.G + c16) * kHeadDim + 4 * q4;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        uint2 w;
        w.x = pack_bf16x2(a.scale * acc[k][dt][0], a.scale * acc[k][dt][1]);
        w.y = pack_bf16x2(a.scale * acc[k][dt][2], a.scale * acc[k][dt][3]);
        *reinterpret_cast<uint2*>(dst + 16 * dt) = w;
      }
    }
  }
};

template <bool kMulti>
__global__ __launch_bounds__(kDqThreads) void bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) DqLds sh;
  Dq st(a);
  st.run<kMulti>(sh);
}

}  // namespace

hipError_t launch_attention_bwd(const BwdArgs& a, int max_seqlen_q, int max_seqlen_k, hipStream_t st) {
  (void)max_seqlen_k;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((a.rows_q + 3) / 4), a.h_kv), dim3(256), 0, st, a);
  hipLaunchKernelGGL(bwd_mask_kernel, dim3(a.ntiles, a.h_kv, a.batch), dim3(256), 0, st, a);
  hipLaunchKernelGGL(bwd_mask_transpose_kernel, dim3((a.nblk + 63) / 64, (a.ntiles + 63) / 64, a.h_kv * a.batch),
                     dim3(256), 0, st, a);
  hipLaunchKernelGGL(bwd_count_kernel, dim3((a.nblk + 3) / 4, a.h_kv, a.batch), dim3(256), 0, st, a);
  hipLaunchKernelGGL(bwd_list_kernel, dim3(1), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(a.wmax), dim3(64 * kDkvWaves), 0, st, a);
  const dim3 dq_grid((max_seqlen_q + 15) / 16, a.h_kv, a.batch);
  if (a.nblk <= kDqWin)
    hipLaunchKernelGGL(bwd_dq_kernel<false>, dq_grid, dim3(kDqThreads), 0, st, a);
  else
    hipLaunchKernelGGL(bwd_dq_kernel<true>, dq_grid, dim3(kDqThreads), 0, st, a);
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((int64_t)a.h_kv * a.batch * a.nblk), 2), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace infllmv2
