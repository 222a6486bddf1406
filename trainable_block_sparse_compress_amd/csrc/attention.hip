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

template <int NW, int TPW>
struct Attn {
  static constexpr int kThreads = 64 * NW;
  static constexpr int kQT = NW * TPW;

  const AttnArgs& a;
  int s, g, wave, lane, q4, c16;
  SeqRange rq, rk;
  int tpos[TPW], bt[TPW];
  int64_t trow[TPW];
  bool tval[TPW];
  bf16x8 qb[TPW][4];
  floatx4 o[TPW][8];
  float m[TPW], l[TPW];

  __device__ Attn(const AttnArgs& args) : a(args) {}

  // True when token k attends block b through the shared (init/local) set.
  __device__ __forceinline__ bool shared_rel(int k, int b, bool dense) const {
    if (!tval[k] || b > bt[k]) return false;
    if (dense) return true;
    return b < a.n_init || b >= bt[k] - a.n_local + 1;
  }

  // Online-softmax update of token k with the S^T tile of block b, then pack
  // P^T as the two B operands (keys 0..31 and 32..63) of the P.V product.
  __device__ __forceinline__ void softmax_block(int k, int b, const floatx4 (&sacc)[4], bf16x8 (&pb)[2]) {
    const bool need_mask = (b == bt[k]);
    float v[4][4];
    float mx = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key_of(kt, 4 * q4 + r);
        const bool ok = !need_mask || (kBlock * b + key <= tpos[k]);
        v[kt][r] = ok ? sacc[kt][r] : -__builtin_inff();
        mx = fmaxf(mx, v[kt][r]);
      }
    }
    mx = max_x32(max_x16(mx));
    const float mn = fmaxf(m[k], mx);
    const float alpha = fast_exp2((m[k] - mn) * a.c);
    m[k] = mn;
    const float mc = mn * a.c;
    float ls = l[k] * alpha;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) o[k][dt][r] *= alpha;
    }
    float p[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kt][r] = fast_exp2(fmaf(v[kt][r], a.c, -mc));
        ls += p[kt][r];
      }
    }
    l[k] = ls;
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

  // ---- shared phase: stage block b in LDS, every wave consumes it --------
  __device__ __forceinline__ void stage(uint8_t* lk, uint8_t* lv, int b) const {
    const int tid = threadIdx.x;
    for (int c = tid; c < 64 * 16; c += kThreads) {
      const int key = c >> 4, ch = c & 15;
      const int pos = kBlock * b + key;
      const int64_t row = (int64_t)rk.start + pos;
      u32x4 v = zero16();
      if (pos < rk.len && row < a.rows_k) v = ldg16(a.k + (row * a.h_kv + g) * kHeadDim + 8 * ch);
      *reinterpret_cast<u32x4*>(lk + key * 256 + ((ch ^ swz_k(key)) << 4)) = v;
    }
    for (int c = tid; c < 128 * 8; c += kThreads) {
      const int dim = c >> 3, ch = c & 7;
      const int first = kBlock * b + 8 * ch;
      u32x4 v = zero16();
      if (first < rk.len && first + 8 <= a.vt_ld) v = clip_keys(ldg16(vt_col(dim) + first), first, rk.len);
      *reinterpret_cast<u32x4*>(lv + dim * 128 + ((ch ^ (dim & 7)) << 4)) = v;
    }
  }

  __device__ __forceinline__ void consume_lds(const uint8_t* lk, const uint8_t* lv, int b, bool dense) {
    bool rel[TPW];
    bool any = false;
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      rel[k] = shared_rel(k, b, dense);
      any |= rel[k];
    }
    if (!any) return;
    floatx4 sacc[TPW][4];
#pragma unroll
    for (int k = 0; k < TPW; ++k)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) sacc[k][kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int key = key_of(kt, c16);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int ch = 4 * ks + q4;
        const bf16x8 af = as_bf16x8(*reinterpret_cast<const u32x4*>(lk + key * 256 + ((ch ^ swz_k(key)) << 4)));
#pragma unroll
        for (int k = 0; k < TPW; ++k)
          if (rel[k]) sacc[k][kt] = mfma16(af, qb[k][ks], sacc[k][kt]);
      }
    }
    bf16x8 pb[TPW][2];
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      if (rel[k]) softmax_block(k, b, sacc[k], pb[k]);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int dim = 16 * dt + c16;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int ch = 4 * kk + q4;
        const bf16x8 af = as_bf16x8(*reinterpret_cast<const u32x4*>(lv + dim * 128 + ((ch ^ (dim & 7)) << 4)));
#pragma unroll
        for (int k = 0; k < TPW; ++k)
          if (rel[k]) o[k][dt] = mfma16(af, pb[k][kk], o[k][dt]);
      }
    }
  }

  // ---- per-token phase: block b of token k from global memory -----------
  __device__ __forceinline__ void consume_global(int k, int b) {
    const int64_t row0 = (int64_t)rk.start + kBlock * b;
    floatx4 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) sacc[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
    bf16x8 kf[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      int64_t row = row0 + key_of(kt, c16);
      row = row < a.rows_k ? row : a.rows_k - 1;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[kt][ks] = as_bf16x8(ldg16(a.k + (row * a.h_kv + g) * kHeadDim + 32 * ks + 8 * q4));
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sacc[kt] = mfma16(kf[kt][ks], qb[k][ks], sacc[kt]);
    bf16x8 vf[8][2];
    const bool partial = kBlock * b + kBlock > rk.len;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint16_t* col = vt_col(16 * dt + c16);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int first = kBlock * b + 32 * kk + 8 * q4;
        u32x4 v = ldg16(col + first);
        if (partial) v = clip_keys(v, first, rk.len);
        vf[dt][kk] = as_bf16x8(v);
      }
    }
    bf16x8 pb[2];
    softmax_block(k, b, sacc, pb);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) o[k][dt] = mfma16(vf[dt][kk], pb[kk], o[k][dt]);
  }

  __device__ void run(uint8_t* lk, uint8_t* lv) {
    s = blockIdx.z;
    g = blockIdx.y;
    rq = seq_range(a.cu_q, a.used_q, s);
    rk = seq_range(a.cu_k, a.used_k, s);
    const int i0 = blockIdx.x * kQT;
    if (i0 >= rq.len) return;
    const int pos0 = rk.len - rq.len;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    lane = threadIdx.x & 63;
    q4 = lane >> 4;
    c16 = lane & 15;
    const bool dense = a.bidx == nullptr;

#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int i = i0 + wave * TPW + k;
      tpos[k] = pos0 + i;
      trow[k] = (int64_t)rq.start + i;
      tval[k] = i < rq.len && trow[k] < a.rows_q && tpos[k] >= 0;
      bt[k] = tpos[k] / kBlock;
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

    const int nq = min(kQT, rq.len - i0);
    const int bt_first = max(0, pos0 + i0) / kBlock;
    const int bt_last = max(0, pos0 + i0 + nq - 1) / kBlock;
    const int n_init_eff = dense ? 0 : min(a.n_init, bt_last + 1);
    const int loc_lo = dense ? 0 : max(n_init_eff, bt_first - a.n_local + 1);
    for (int idx = 0;; ++idx) {
      const int b = idx < n_init_eff ? idx : loc_lo + (idx - n_init_eff);
      if (b > bt_last) break;
      __syncthreads();
      stage(lk, lv, b);
      __syncthreads();
      consume_lds(lk, lv, b, dense);
    }

    if (!dense) {
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        if (!tval[k]) continue;
        const int32_t* list = a.bidx + ((int64_t)g * a.rows_q + trow[k]) * a.n_sel;
        const int local_lo = bt[k] - a.n_local + 1;
        int prev = -1;
        for (int e = 0; e < a.n_sel; ++e) {
          const int b = __builtin_amdgcn_readfirstlane(list[e]);
          if (b < 0 || b > bt[k] || b <= prev) continue;
          prev = b;
          if (b < a.n_init || b >= local_lo) continue;  // attended in the shared phase
          if (kBlock * b + kBlock > a.vt_ld) continue;   // outside the V^T buffer (bad metadata)
          consume_global(k, b);
        }
      }
    }

#pragma unroll
    for (int k = 0; k < TPW; ++k) {
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
          a.lse[(int64_t)(g * a.G + c16) * a.rows_q + trow[k]] = lt > 0.f ? m[k] * a.scale + logf(lt) : -__builtin_inff();
      }
    }
  }
};

template <int NW, int TPW>
__global__ __launch_bounds__(64 * NW) void attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lk[64 * 256];
  __shared__ __attribute__((aligned(16))) uint8_t lv[128 * 128];
  Attn<NW, TPW> st(a);
  st.run(lk, lv);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int max_seqlen_q, hipStream_t st) {
  constexpr int NW = 4, TPW = 4;
  dim3 grid((max_seqlen_q + NW * TPW - 1) / (NW * TPW), a.h_kv, a.batch);
  hipLaunchKernelGGL((attn_kernel<NW, TPW>), grid, dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

}  // namespace infllmv2
