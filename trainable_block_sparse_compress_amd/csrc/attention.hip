// Block-sparse and dense causal attention on bf16 MFMA.
//
// The sparse path is the single unified branch of InfLLM-V2: selected blocks
// and the sliding window are one sparse attention, with the local blocks
// extended to cover the window (top168.com article on InfLLM-V2, section 七
// "技术实现的创新细节"; reading notes "论文阅读：InfLLM-V2", section "对齐计算图").
// The dense path below the length threshold is the same kernel with every
// causal block treated as shared.
//
// Per workgroup: NW waves x TPW query tokens of one sequence, one KV group.
//  - Shared phase: blocks that every token of the tile attends (init blocks,
//    and the local window, which only depends on the token's block) are
//    staged once in LDS (K as [key][dim], V^T as [dim][key], both
//    XOR-swizzled) and consumed by all waves.
//  - Per-token phase: each token's remaining (top-k) blocks come straight
//    from global memory / L2; the 16 heads of the group form the 16-wide
//    MFMA tile.
// Products are computed transposed: S^T = K Q^T (16 keys x 16 heads per
// MFMA), then O^T += V^T P^T.  With the key order chosen below, the S^T
// accumulator of two key tiles is exactly the B operand P^T of the next MFMA,
// so P never leaves registers, and V^T fragments are 8 consecutive keys of one
// dim: one 16-byte load.
#include "kernels.hpp"

namespace infllmv2 {

namespace {

// Key held by row r of S^T key tile kt (a 64-key block has 4 tiles of 16).
__device__ __forceinline__ int key_of(int kt, int r) {
  return 32 * (kt >> 1) + 8 * (r >> 2) + 4 * (kt & 1) + (r & 3);
}
// LDS swizzle of K rows: the 8 rows a group of 8 lanes reads together map to
// distinct 16-byte bank groups.
__device__ __forceinline__ int swz_k(int row) { return (row & 3) | ((row >> 1) & 4); }

// Zero the bf16 lanes of an 8-key V^T fragment whose key (first + i) >= limit.
__device__ __forceinline__ u32x4 clip_keys(u32x4 v, int first, int limit) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (first + 2 * i >= limit) v[i] &= 0xFFFF0000u;
    if (first + 2 * i + 1 >= limit) v[i] &= 0x0000FFFFu;
  }
  return v;
}

// s_waitcnt immediate: wait until at most n vector-memory loads are
// outstanding (vmcnt in bits 3:0 and 15:14), no wait on expcnt / lgkmcnt.
__host__ __device__ constexpr int vmcnt_imm(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// Lazy rescaling threshold: the running max is only raised when a block's
// max exceeds it by more than 8 in log2 units, so P <= 2^8 (exact enough in
// bf16) and most blocks skip the O rescale.
constexpr float kLazyLog2 = 8.f;

constexpr int kAttnWaves = 8;                    // waves per workgroup
constexpr int kTPW = 2;                          // query tokens per wave
constexpr int kTileTok = kAttnWaves * kTPW;      // 16 tokens per workgroup (one mask bit each)
constexpr int kThreads = 64 * kAttnWaves;
constexpr int kWin = 1024;                       // blocks per list window
constexpr int kRing = 4;                         // staged blocks: 1 computing + 3 in flight

struct AttnLds {
  uint8_t k[kRing][64 * 256];   // K block, [key][dim], swizzled (ring of staged blocks)
  uint8_t v[kRing][128 * 128];  // V^T block, [dim][key], swizzled
  uint32_t mask[kWin];          // per block of the window: which tile tokens attend it
  int32_t ub[kWin];             // compacted (block, mask) list
  uint32_t um[kWin];
  int32_t wsum[kAttnWaves];
};

// One workgroup: 16 consecutive query tokens of one sequence and one KV group.
// Every block any of them attends (init, local, top-k union; dense: all
// causal blocks) is listed once with a bit mask of its tokens, staged once
// in LDS, and consumed by exactly the tokens that attend it.
struct Attn {
  const AttnArgs& a;
  int s, g, lane, q4, c16, wave;
  SeqRange rq, rk;
  int tpos[kTPW], bt[kTPW];
  int64_t trow[kTPW];
  bool tval[kTPW];
  bf16x8 qb[kTPW][4];
  floatx4 o[kTPW][8];
  float m[kTPW], l[kTPW];

  __device__ Attn(const AttnArgs& args) : a(args) {}

  // Online-softmax update of token k with the S^T tile of block b, then pack
  // P^T as the two B operands (keys 0..31 and 32..63) of the P.V product.
  __device__ __forceinline__ void softmax_block(int k, int b, const floatx4 (&sacc)[4], bf16x8 (&pb)[2]) {
    float v[4][4];
    float mx = -__builtin_inff();
    if (b == bt[k]) {          // the query's own block: keys after it are masked
      const int lim = tpos[k] - kBlock * b;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[kt][r] = key_of(kt, 4 * q4 + r) <= lim ? sacc[kt][r] : -__builtin_inff();
          mx = fmaxf(mx, v[kt][r]);
        }
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[kt][r] = sacc[kt][r];
          mx = fmaxf(mx, v[kt][r]);
        }
      }
    }
    mx = max_x32(max_x16(mx));
    if (__ballot(mx * a.c > m[k] * a.c + kLazyLog2) != 0) {
      const float mn = fmaxf(m[k], mx);
      const float alpha = fast_exp2((m[k] - mn) * a.c);
      m[k] = mn;
      l[k] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) o[k][dt][r] *= alpha;
      }
    }
    const float mc = m[k] * a.c;
    float p[4][4];
    float ls = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kt][r] = fast_exp2(fmaf(v[kt][r], a.c, -mc));
        ls += p[kt][r];
      }
    }
    l[k] += ls;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 w;
      w[0] = pack_bf16x2(p[2 * kk][0], p[2 * kk][1]);
      w[1] = pack_bf16x2(p[2 * kk][2], p[2 * kk][3]);
      w[2] = pack_bf16x2(p[2 * kk + 1][0], p[2 * kk + 1][1]);
      w[3] = pack_bf16x2(p[2 * kk + 1][2], p[2 * kk + 1][3]);
      pb[kk] = as_bf16x8(w);
    }
  }

  __device__ __forceinline__ const uint16_t* vt_col(int dim) const {
    return a.vt + (((int64_t)g * kHeadDim + dim) * a.batch + s) * a.vt_ld;
  }

  // Stage block b into LDS with direct global->LDS 16-byte loads (no
  // registers involved): every wave writes two contiguous 1 KB parts of the
  // K tile and two of the V^T tile.  LDS slot (row, chunk p) receives global
  // chunk p ^ swizzle(row), so the tiles land swizzled.  Rows past the
  // sequence hold whatever the clamped address reads: K garbage is masked by
  // causality; a partial V^T block is zeroed by fix_partial().
  __device__ __forceinline__ void stage_issue(uint8_t* lk, uint8_t* lv, int b) const {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int part = wave + kAttnWaves * j;
      const int off = part * 1024 + lane * 16;
      const int key = off >> 8;
      const int ch = ((off >> 4) & 15) ^ swz_k(key);
      int64_t row = (int64_t)rk.start + kBlock * b + key;
      row = row < a.rows_k ? row : a.rows_k - 1;
      __builtin_amdgcn_global_load_lds(a.k + (row * a.h_kv + g) * kHeadDim + 8 * ch,
                                       (__attribute__((address_space(3))) void*)(lk + part * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int part = wave + kAttnWaves * j;
      const int off = part * 1024 + lane * 16;
      const int dim = off >> 7;
      const int ch = ((off >> 4) & 7) ^ (dim & 7);
      int64_t first = (int64_t)kBlock * b + 8 * ch;
      first = first + 8 <= a.vt_ld ? first : a.vt_ld - 8;
      __builtin_amdgcn_global_load_lds(vt_col(dim) + first,
                                       (__attribute__((address_space(3))) void*)(lv + part * 1024), 16, 0, 0);
    }
  }
  // Zero the V^T columns of keys >= len_k in a staged partial block.
  __device__ __forceinline__ void fix_partial(uint8_t* lv, int b) const {
    const int tid = threadIdx.x;
    for (int c = tid; c < 128 * 8; c += kThreads) {
      const int dim = c >> 3, p = c & 7;
      const int first = kBlock * b + 8 * (p ^ (dim & 7));
      u32x4* slot = reinterpret_cast<u32x4*>(lv + dim * 128 + (p << 4));
      *slot = clip_keys(*slot, first, rk.len);
    }
  }

  // Lane-constant LDS byte offsets of the MFMA fragments (see stage_issue
  // for the swizzles): K fragment (kt, ks) sits at koff[ks] + 256*kt_key(kt),
  // V^T fragment (dt, kk) at voff[kk] + 2048*dt.
  int koff[4], voff[2];
  __device__ __forceinline__ void init_offsets() {
    const int key0 = 8 * (c16 >> 2) + (c16 & 3);
    const int sw = swz_k(key0);   // equal for every key of this lane
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) koff[ks] = key0 * 256 + (((4 * ks + q4) ^ sw) << 4);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) voff[kk] = c16 * 128 + (((4 * kk + q4) ^ (c16 & 7)) << 4);
  }
  static __device__ __forceinline__ bf16x8 lds16(const uint8_t* p) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(p));
  }

  // Block b (staged in lk / lv) for the tokens of this wave whose bit is set
  // in sel.  All fragment loads of a product are issued before its MFMAs;
  // the V^T loads are in flight during the softmax.
  __device__ __forceinline__ void consume(uint32_t sel, const uint8_t* lk, const uint8_t* lv, int b) {
    floatx4 sacc[kTPW][4];
    {
      bf16x8 kf[4][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          kf[kt][ks] = lds16(lk + koff[ks] + 256 * (32 * (kt >> 1) + 4 * (kt & 1)));
#pragma unroll
      for (int k = 0; k < kTPW; ++k) {
        if (!((sel >> k) & 1u)) continue;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          sacc[k][kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) sacc[k][kt] = mfma16(kf[kt][ks], qb[k][ks], sacc[k][kt]);
        }
      }
    }
    bf16x8 vf[8][2];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) vf[dt][kk] = lds16(lv + voff[kk] + 2048 * dt);
    bf16x8 pb[kTPW][2];
#pragma unroll
    for (int k = 0; k < kTPW; ++k)
      if ((sel >> k) & 1u) softmax_block(k, b, sacc[k], pb[k]);
#pragma unroll
    for (int k = 0; k < kTPW; ++k) {
      if (!((sel >> k) & 1u)) continue;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) o[k][dt] = mfma16(vf[dt][kk], pb[k][kk], o[k][dt]);
    }
  }

  __device__ void run(AttnLds& sh) {
    // XCD-aware order: workgroups are dispatched round-robin over the 8
    // XCDs; remap them so each XCD walks a contiguous range of query tiles
    // (neighbouring tiles share their local window and hot blocks in L2).
    const unsigned nx = gridDim.x, ny = gridDim.y;
    const unsigned N = nx * ny * gridDim.z;
    const unsigned L = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
    const unsigned full = N - N % 8u;
    const unsigned T = L < full ? (L % 8u) * (full / 8u) + L / 8u : L;
    const int tile = (int)(T % nx);
    g = (int)((T / nx) % ny);
    s = (int)(T / (nx * ny));

    rq = seq_range(a.cu_q, a.used_q, s);
    rk = seq_range(a.cu_k, a.used_k, s);
    const int i0 = tile * kTileTok;
    if (i0 >= rq.len) return;
    const int pos0 = rk.len - rq.len;
    const int tid = threadIdx.x;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    lane = tid & 63;
    q4 = lane >> 4;
    c16 = lane & 15;
    const bool dense = a.bidx == nullptr;
    init_offsets();

#pragma unroll
    for (int k = 0; k < kTPW; ++k) {
      const int i = i0 + wave * kTPW + k;
      tpos[k] = pos0 + i;
      trow[k] = (int64_t)rq.start + i;
      tval[k] = i < rq.len && trow[k] < a.rows_q && tpos[k] >= 0;
      bt[k] = tval[k] ? tpos[k] / kBlock : -1;
      const bool hv = tval[k] && c16 < a.G;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        u32x4 v = zero16();
        if (hv) v = ldg16(a.q + (trow[k] * a.h_q + g * a.G + c16) * kHeadDim + 32 * ks + 8 * q4);
        qb[k][ks] = as_bf16x8(v);
      }
      m[k] = -1e30f;
      l[k] = 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[k][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    const int nq = min(kTileTok, rq.len - i0);
    const int bt_last = max(0, pos0 + i0 + nq - 1) / kBlock;
    for (int w0 = 0; w0 <= bt_last; w0 += kWin) {
      const int w1 = min(bt_last + 1, w0 + kWin);
      // 1. init / local (dense: every causal block), by arithmetic.
      for (int b = w0 + tid; b < w1; b += kThreads) {
        uint32_t msk = 0;
        for (int tk = 0; tk < nq; ++tk) {
          const int t = pos0 + i0 + tk;
          if (t < 0 || (int64_t)rq.start + i0 + tk >= a.rows_q) continue;
          const int btk = t / kBlock;
          const bool rel = b <= btk && (dense || b < a.n_init || b >= btk - a.n_local + 1);
          msk |= (uint32_t)rel << tk;
        }
        sh.mask[b - w0] = msk;
      }
      __syncthreads();
      // 2. top-k entries of the tile's tokens (set union; -1, repeats and
      //    blocks after the token's own are ignored).
      if (!dense) {
#pragma unroll
        for (int k = 0; k < kTPW; ++k) {
          if (!tval[k]) continue;
          const int32_t* list = a.bidx + ((int64_t)g * a.rows_q + trow[k]) * a.n_sel;
          const uint32_t bit = 1u << (wave * kTPW + k);
          for (int e = lane; e < a.n_sel; e += 64) {
            const int b = list[e];
            if (b >= 0 && b <= bt[k] && b >= w0 && b < w1 && kBlock * b + kBlock <= a.vt_ld)
              atomicOr(&sh.mask[b - w0], bit);
          }
        }
      }
      __syncthreads();
      // 3. compact the non-empty blocks, ascending.
      uint32_t mk[kWin / kThreads];
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < kWin / kThreads; ++j) {
        const int e = tid * (kWin / kThreads) + j;
        mk[j] = e < w1 - w0 ? sh.mask[e] : 0u;
        cnt += mk[j] != 0u;
      }
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      if (lane == 63) sh.wsum[wave] = incl;
      __syncthreads();
      int wbase = 0, n_ent = 0;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const int ws = sh.wsum[w];
        wbase += w < wave ? ws : 0;
        n_ent += ws;
      }
      int pos = wbase + incl - cnt;
#pragma unroll
      for (int j = 0; j < kWin / kThreads; ++j) {
        if (mk[j]) {
          sh.ub[pos] = w0 + tid * (kWin / kThreads) + j;
          sh.um[pos] = mk[j];
          ++pos;
        }
      }
      __syncthreads();
      // 4. walk the list; the next block's staging loads are in flight while
      //    the current one computes.
      if (n_ent > 0) {
        // Batches of two blocks: the ring holds the batch being consumed and
        // the next one in flight; one barrier per batch, so the per-wave load
        // imbalance of single blocks averages over two.
        stage_issue(sh.k[0], sh.v[0], sh.ub[0]);
        if (n_ent > 1) stage_issue(sh.k[1], sh.v[1], sh.ub[1]);
        for (int u = 0; u < n_ent; u += 2) {
          const int half = (u >> 1) & 1;
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // this wave's part of the batch has landed
          __syncthreads();                            // ... every wave's; the other half is free
          const int b0 = __builtin_amdgcn_readfirstlane(sh.ub[u]);
          const int b1 = u + 1 < n_ent ? __builtin_amdgcn_readfirstlane(sh.ub[u + 1]) : -1;
          const bool p0 = kBlock * b0 + kBlock > rk.len;
          const bool p1 = b1 >= 0 && kBlock * b1 + kBlock > rk.len;
          if (p0 || p1) {
            if (p0) fix_partial(sh.v[2 * half], b0);
            if (p1) fix_partial(sh.v[2 * half + 1], b1);
            __syncthreads();
          }
          if (u + 2 < n_ent) stage_issue(sh.k[2 * (half ^ 1)], sh.v[2 * (half ^ 1)], sh.ub[u + 2]);
          if (u + 3 < n_ent) stage_issue(sh.k[2 * (half ^ 1) + 1], sh.v[2 * (half ^ 1) + 1], sh.ub[u + 3]);
          const uint32_t sh_mask = (1u << kTPW) - 1u;
          const uint32_t m0 = (__builtin_amdgcn_readfirstlane(sh.um[u]) >> (wave * kTPW)) & sh_mask;
          if (m0) consume(m0, sh.k[2 * half], sh.v[2 * half], b0);
          if (b1 >= 0) {
            const uint32_t m1 = (__builtin_amdgcn_readfirstlane(sh.um[u + 1]) >> (wave * kTPW)) & sh_mask;
            if (m1) consume(m1, sh.k[2 * half + 1], sh.v[2 * half + 1], b1);
          }
        }
        __syncthreads();   // list and buffers are reused by the next window
      }
    }

#pragma unroll
    for (int k = 0; k < kTPW; ++k) {
      const float lt = sum_x16(sum_x32(l[k]));
      if (!tval[k]) continue;
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      if (c16 < a.G) {
        uint16_t* dst = a.out + (trow[k] * a.h_q + g * a.G + c16) * kHeadDim + 4 * q4;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          uint2 w;
          w.x = pack_bf16x2(o[k][dt][0] * inv, o[k][dt][1] * inv);
          w.y = pack_bf16x2(o[k][dt][2] * inv, o[k][dt][3] * inv);
          *reinterpret_cast<uint2*>(dst + 16 * dt) = w;
        }
        if (a.lse && q4 == 0)
          a.lse[(int64_t)(g * a.G + c16) * a.rows_q + trow[k]] =
              lt > 0.f ? m[k] * a.scale + logf(lt) : -__builtin_inff();
      }
    }
  }
};

__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) AttnLds sh;
  Attn st(a);
  st.run(sh);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int max_seqlen_q, hipStream_t st) {
  dim3 grid((max_seqlen_q + kTileTok - 1) / kTileTok, a.h_kv, a.batch);
  hipLaunchKernelGGL(attn_kernel, grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace infllmv2
