// Block-sparse and dense causal attention on bf16 MFMA.
//
// The sparse path is the single unified branch of InfLLM-V2: selected blocks
// and the sliding window are one sparse attention, with the local blocks
// extended to cover the window (top168.com article on InfLLM-V2, section 七
// "技术实现的创新细节"; reading notes "论文阅读：InfLLM-V2", section "对齐计算图").
// The dense path below the length threshold is an instance of the same
// kernel in which every causal block is shared and the block list and token
// masks follow by arithmetic.
//
// Per workgroup: 16 consecutive query tokens of one sequence and one KV group,
// 8 waves of 2 tokens.  Every block the tokens attend is listed once with a
// bit mask of its tokens, then consumed in two phases:
//  - Shared phase: blocks attended by several tokens of the tile (init and
//    local blocks, popular top-k blocks; dense: every causal block) are
//    staged once in an LDS ring (K as [key][dim], V^T as [dim][key], both
//    XOR-swizzled) and consumed by the waves whose tokens attend them, one
//    workgroup barrier per batch of two blocks.
//  - Private phase: blocks attended by few tokens are streamed by the waves
//    that own those tokens, each on its own (K through a per-wave LDS region,
//    V^T straight into registers), with no workgroup barrier, so a wave that
//    owns many private blocks does not hold up the others.  Tokens are
//    assigned to waves only once the masks are known, heaviest private load
//    paired with lightest, so the waves' private phases end together.
// The 16 heads of the group form the 16-wide MFMA tile.
// Products are computed transposed: S^T = K Q^T (16 keys x 16 heads per
// MFMA), then O^T += V^T P^T.  With the key order chosen below, the S^T
// accumulator of two key tiles is exactly the B operand P^T of the next MFMA,
// so P never leaves registers, and V^T fragments are 8 consecutive keys of one
// dim: one 16-byte load.
#include "kernels.hpp"
#include "tile_common.hpp"

namespace infllmv2 {

namespace {

// Zero the bf16 lanes of an 8-key V^T fragment whose key (first + i) >= limit.
__device__ __forceinline__ u32x4 clip_keys(u32x4 v, int first, int limit) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (first + 2 * i >= limit) v[i] &= 0xFFFF0000u;
    if (first + 2 * i + 1 >= limit) v[i] &= 0x0000FFFFu;
  }
  return v;
}

// Lazy rescaling threshold: the running max is only raised when a block's
// max exceeds it by more than 8 in log2 units, so P <= 2^8 (exact enough in
// bf16) and most blocks skip the O rescale.
constexpr float kLazyLog2 = 8.f;
constexpr float kLazySum = 256.f;   // 2^kLazyLog2

constexpr int kAttnWaves = 8;                    // waves per workgroup
constexpr int kTPW = 2;                          // query tokens per wave
constexpr int kTileTok = kAttnWaves * kTPW;      // 16 tokens per workgroup (one mask bit each)
constexpr int kThreads = 64 * kAttnWaves;
constexpr int kWin = 2048;                       // blocks per list window (128K keys)
constexpr int kRing = 4;                         // shared phase: 2 blocks consumed + 2 in flight
constexpr int kShareMin = 2;                     // tokens attending a block for the shared phase

struct AttnLds {
  // Shared phase: slot r holds a K block at ring[r][0] and its V^T at
  // ring[r][1].  Private phase: wave w owns the 16 KB at (ring[0][0] + 16 KB * w)
  // for the K block it is streaming.
  uint8_t ring[kRing][2][64 * 256];
  uint32_t mask[kWin];          // per block of the window: which tile tokens attend it
  int32_t ub[kWin];             // compacted shared-phase (block, mask) list
  uint32_t um[kWin];
  int32_t cnt[kWin / kThreads][kAttnWaves];
  int32_t pcnt[kTileTok];       // private blocks per tile token
  int32_t perm[kTileTok];       // token (tile index) of each wave slot 2w + k
};
static_assert(kRing * 2 * 64 * 256 == kAttnWaves * 64 * 256, "private regions alias the ring");

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
  int tb[kTPW];                 // tile-token index (mask bit) of each of the wave's tokens
  unsigned xrank;               // the workgroup's dispatch rank on its XCD

  // Mask bits of this wave's tokens, gathered into bits 0 .. kTPW-1.
  __device__ __forceinline__ uint32_t sel_of(uint32_t v) const {
    uint32_t r = 0;
#pragma unroll
    for (int k = 0; k < kTPW; ++k) r |= ((v >> tb[k]) & 1u) << k;
    return r;
  }
  __device__ __forceinline__ uint32_t mine_mask() const {
    uint32_t r = 0;
#pragma unroll
    for (int k = 0; k < kTPW; ++k) r |= 1u << tb[k];
    return r;
  }
  // State of token k of this wave: tile token tt (query row i0 + tt).
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
      u32x4 v = zero16();
      if (hv) v = ldg16(a.q + (trow[k] * a.h_q + g * a.G + c16) * kHeadDim + 32 * ks + 8 * q4);
      qb[k][ks] = as_bf16x8(v);
    }
    m[k] = -1e30f;
    l[k] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[k][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  __device__ Attn(const AttnArgs& args) : a(args) {}

  // Online-softmax update of token k with the S^T tile of block b, then pack
  // P^T as the two B operands (keys 0..31 and 32..63) of the P.V product.
  // kSumCheck: exponentiate against the running max first, and look for the
  // block max only when some lane's sum of its 16 values exceeds 2^8.  A sum
  // bounds each of its terms, so below that no score exceeds the running max
  // by more than the lazy threshold and the values stand as computed; the
  // max reduction is skipped on almost every block.  Without it, the block
  // max is taken first (the multi-window instance, which has no registers to
  // keep the scores live across the test).  Either way a block raises the
  // running max only past the threshold, which bounds P and is not a
  // rounding decision.
  template <bool kSumCheck>
  __device__ __forceinline__ void softmax_block(int k, int b, const floatx4 (&sacc)[4], bf16x8 (&pb)[2]) {
    float v[4][4];
    if (b == bt[k]) {          // the query's own block: keys after it are masked
      // key_of(kt, 4*q4 + r) = 8*q4 + (32*(kt/2) + 4*(kt%2) + r): compare the
      // lane-free part against the limit shifted by the lane's 8*q4.
      const int lim = tpos[k] - kBlock * b - 8 * q4;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          v[kt][r] = 32 * (kt >> 1) + 4 * (kt & 1) + r <= lim ? sacc[kt][r] : -__builtin_inff();
    } else {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[kt][r] = sacc[kt][r];
    }
    float p[4][4];
    float ls = 0.f;
    const auto exponentiate = [&]() {
      const float mc = m[k] * a.c;
      ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[kt][r] = fast_exp2(fmaf(v[kt][r], a.c, -mc));
          ls += p[kt][r];
        }
    };
    // Raise the running max to the block max (rescaling l and O) when the
    // block max exceeds it by more than the lazy threshold; true if raised.
    const auto raise_max = [&]() -> bool {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, v[kt][r]);
      mx = max_x32(max_x16(mx));
      if (__ballot(mx * a.c > m[k] * a.c + kLazyLog2) == 0) return false;
      const float mn = fmaxf(m[k], mx);
      const float alpha = fast_exp2((m[k] - mn) * a.c);
      m[k] = mn;
      l[k] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[k][dt][r] *= alpha;
      return true;
    };
    if constexpr (kSumCheck) {
      exponentiate();
      // (an infinite or NaN sum, as on a token's first block, fails <=)
      if (__ballot(!(ls <= kLazySum)) != 0 && raise_max()) exponentiate();
    } else {
      raise_max();
      exponentiate();
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

  // Global addressing of K and V^T blocks: buffer loads from a wave-uniform
  // base (a buffer descriptor in scalar registers, rebuilt per block) plus a
  // uniform offset and a 32-bit lane byte offset set once by init_offsets,
  // so no load costs per-lane 64-bit address arithmetic.
  const char* kbase;       // K row 0 of this sequence, this KV group
  const char* vbase;       // V^T dim 0 of this sequence, this KV group
  int64_t krow;            // bytes between consecutive K rows
  int64_t vdim;            // bytes between consecutive V^T dims
  uint32_t klo[2];         // K staging: lane byte offset in a 4-row part, per swizzle variant
  uint32_t vlo_stage;      // V^T staging: lane byte offset in an 8-dim part
  uint32_t vlo_frag;       // V^T fragment loads: lane byte offset (dim c16, keys 8*q4)
  // v as a wave-uniform value, so that the descriptors and offsets derived
  // from it are formed in scalar registers.
  static __device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
  }
  // Raw buffer over [base, base + 4 GiB): stride 0, no record limit, the
  // gfx9-family word 3 (32-bit data format).
  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const char* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, -1, 0x00020000);
  }
  static __device__ __forceinline__ void buf_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
  }

  // K row `row` (relative to the sequence), chunk ch, clamped to the tensor.
  __device__ __forceinline__ const uint16_t* k_clamped(int row, int ch) const {
    int64_t r = (int64_t)rk.start + row;
    r = r < a.rows_k ? r : a.rows_k - 1;
    return a.k + (r * a.h_kv + g) * kHeadDim + 8 * ch;
  }
  // One 1 KB part (4 rows) of K block b into lk + 1024 * part, rows clamped
  // to the tensor (a block that reaches past its end).
  __device__ __forceinline__ void stage_k_part(uint8_t* lk, int b, int part) const {
    const int key = 4 * part + (lane >> 4);
    __builtin_amdgcn_global_load_lds(k_clamped(kBlock * b + key, (lane & 15) ^ swz_k(key)),
                                     (__attribute__((address_space(3))) void*)(lk + part * 1024), 16, 0, 0);
  }
  // True when every row of block b lies inside the K tensor.
  __device__ __forceinline__ bool k_inside(int b) const {
    return (int64_t)rk.start + kBlock * b + kBlock <= a.rows_k;
  }

  // Stage block b into LDS with direct global->LDS 16-byte loads (no
  // registers involved): every wave writes two contiguous 1 KB parts of the
  // K tile and two of the V^T tile.  LDS slot (row, chunk p) receives global
  // chunk p ^ swizzle(row), so the tiles land swizzled.  K rows past the
  // tensor read its last row and rows past the sequence read whatever follows
  // (both masked by causality); a partial V^T block is zeroed by
  // fix_partial().
  __device__ __forceinline__ void stage_issue(uint8_t* lk, uint8_t* lv, int b) const {
    if (k_inside(b)) {
      const auto r = rsrc(kbase + (int64_t)(kBlock * b) * krow);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int part = wave + kAttnWaves * j;
        buf_lds16(r, (part & 2) ? klo[1] : klo[0], (uint32_t)((4 * part) * krow), lk + part * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) stage_k_part(lk, b, wave + kAttnWaves * j);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int part = wave + kAttnWaves * j;   // dims 8*part .. 8*part+7
      buf_lds16(rsrc(vbase + (int64_t)(2 * kBlock) * b + (int64_t)(8 * part) * vdim), vlo_stage, 0u, lv + part * 1024);
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
    krow = uniform64((int64_t)a.h_kv * kHeadDim * 2);
    vdim = uniform64((int64_t)a.batch * a.vt_ld * 2);
    kbase = reinterpret_cast<const char*>(
        uniform64(reinterpret_cast<int64_t>(a.k + ((int64_t)rk.start * a.h_kv + g) * kHeadDim)));
    vbase = reinterpret_cast<const char*>(
        uniform64(reinterpret_cast<int64_t>(a.vt + ((int64_t)g * kHeadDim * a.batch + s) * a.vt_ld)));
    // (the host keeps 16 V^T dims under 4 GiB, so every offset fits 32 bits)
#pragma unroll
    for (int v = 0; v < 2; ++v)
      klo[v] = (uint32_t)((lane >> 4) * krow + 16 * ((lane & 15) ^ (((lane >> 4) & 3) | (4 * v))));
    vlo_stage = (uint32_t)((lane >> 3) * vdim + 16 * ((lane & 7) ^ ((lane >> 3) & 7)));
    vlo_frag = (uint32_t)(c16 * vdim + 16 * q4);
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

  // S^T tiles of block b (K staged at lk) for the tokens of this wave in sel.
  __device__ __forceinline__ void scores(uint32_t sel, const uint8_t* lk, floatx4 (&sacc)[kTPW][4]) const {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      bf16x8 kf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[ks] = lds16(lk + koff[ks] + 256 * (32 * (kt >> 1) + 4 * (kt & 1)));
#pragma unroll
      for (int k = 0; k < kTPW; ++k) {
        if (!((sel >> k) & 1u)) continue;
        sacc[k][kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) sacc[k][kt] = mfma16(kf[ks], qb[k][ks], sacc[k][kt]);
      }
    }
  }

  // Shared phase: block b (staged in lk / lv) for the tokens of this wave
  // whose bit is set in sel.  The V^T loads are in flight during the softmax.
  template <bool kSumCheck>
  __device__ __forceinline__ void consume(uint32_t sel, const uint8_t* lk, const uint8_t* lv, int b) {
    floatx4 sacc[kTPW][4];
    // MFMA stretches run at raised wave priority, so the other wave on the
    // SIMD fills the gaps with its softmax work rather than competing.
    __builtin_amdgcn_s_setprio(1);
    scores(sel, lk, sacc);
    __builtin_amdgcn_s_setprio(0);
    bf16x8 vf[8][2];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) vf[dt][kk] = lds16(lv + voff[kk] + 2048 * dt);
    bf16x8 pb[kTPW][2];
#pragma unroll
    for (int k = 0; k < kTPW; ++k)
      if ((sel >> k) & 1u) softmax_block<kSumCheck>(k, b, sacc[k], pb[k]);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int k = 0; k < kTPW; ++k) {
      if (!((sel >> k) & 1u)) continue;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) o[k][dt] = mfma16(vf[dt][kk], pb[k][kk], o[k][dt]);
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // Private phase: this wave alone stages K block b into its LDS region
  // (16 direct global->LDS loads of 1 KB, same swizzled layout as the ring).
  __device__ __forceinline__ void issue_k_private(uint8_t* lk, int b) const {
    if (k_inside(b)) {
      const auto r = rsrc(kbase + (int64_t)(kBlock * b) * krow);
#pragma unroll
      for (int part = 0; part < 16; ++part)
        buf_lds16(r, (part & 2) ? klo[1] : klo[0], (uint32_t)((4 * part) * krow), lk + part * 1024);
    } else {
#pragma unroll
      for (int part = 0; part < 16; ++part) stage_k_part(lk, b, part);
    }
  }
  // Private phase: V^T fragments of block b straight into registers
  // (fragment (dt, kk): dim 16*dt + c16, keys 64*b + 32*kk + 8*q4 .. +8).
  __device__ __forceinline__ void load_v_private(u32x4 (&vb)[8][2], int b) const {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const auto r = rsrc(vbase + (int64_t)(2 * kBlock) * b + (int64_t)(16 * dt) * vdim);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) vb[dt][kk] = __builtin_amdgcn_raw_buffer_load_b128(r, vlo_frag + 64 * kk, 0, 0);
    }
  }

  // Private phase, block b for the tokens of this wave in sel: K from the
  // wave's region, V^T from registers (keys past the sequence zeroed).
  template <bool kSumCheck>
  __device__ __forceinline__ void consume_private(uint32_t sel, const uint8_t* lk, u32x4 (&vb)[8][2], int b) {
    if (kBlock * b + kBlock > rk.len) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) vb[dt][kk] = clip_keys(vb[dt][kk], kBlock * b + 32 * kk + 8 * q4, rk.len);
    }
    // One token at a time (a private block rarely serves both tokens of the
    // wave): S^T, softmax and P.V of the first before the second.
#pragma unroll
    for (int k = 0; k < kTPW; ++k) {
      if (!((sel >> k) & 1u)) continue;
      floatx4 sacc[4];
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        bf16x8 kf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kf[ks] = lds16(lk + koff[ks] + 256 * (32 * (kt >> 1) + 4 * (kt & 1)));
        sacc[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) sacc[kt] = mfma16(kf[ks], qb[k][ks], sacc[kt]);
      }
      __builtin_amdgcn_s_setprio(0);
      bf16x8 pb[2];
      softmax_block<kSumCheck>(k, b, sacc, pb);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) o[k][dt] = mfma16(as_bf16x8(vb[dt][kk]), pb[kk], o[k][dt]);
      __builtin_amdgcn_s_setprio(0);
    }
  }

  // One window of blocks [w0, w1): build the token masks, run the shared
  // phase over the popular blocks, then the private phase.  kSingle: the
  // single-window kernel, which also balances the tokens over the waves and
  // orders the shared list (both left out of the multi-window kernel, whose
  // loop keeps every token on its wave and leaves no registers to spare).
  template <bool kSingle, bool kDense>
  __device__ __forceinline__ void window(AttnLds& sh, int w0, int w1, int nq, int pos0, int i0, int tid) {
    constexpr bool dense = kDense;
    const int nblk = w1 - w0;
    int n_ent = 0;
    // Dense: tile tokens [dlo, dhi) are valid (position >= 0, row inside
    // the tensor), and the shared list is every block of the window up to
    // the last valid token's own (none past the V^T row), entry u being
    // block w0 + u with its token mask by arithmetic (ent_mask below).
    const int p0 = pos0 + i0;
    const int dlo = max(0, -p0);
    const int dhi = (int)min<int64_t>(nq, a.rows_q - rq.start - i0);
    if constexpr (dense) {
      if (dlo < dhi) {
        const int last = min(min(w1, (p0 + dhi - 1) / kBlock + 1), (int)(a.vt_ld / kBlock));
        n_ent = max(0, last - w0);
      }
    } else {
      // 1. init / local, by arithmetic.
      if (tid < kTileTok) sh.pcnt[tid] = 0;
      for (int b = w0 + tid; b < w1; b += kThreads) {
        uint32_t msk = 0;
        // (a block past the V^T row would mean inconsistent lengths: skipped)
        for (int tk = 0; tk < nq && kBlock * b + kBlock <= a.vt_ld; ++tk) {
          const int t = pos0 + i0 + tk;
          if (t < 0 || (int64_t)rq.start + i0 + tk >= a.rows_q) continue;
          const int btk = t / kBlock;
          const bool rel = b <= btk && (b < a.n_init || b >= btk - a.n_local + 1);
          msk |= (uint32_t)rel << tk;
        }
        sh.mask[b - w0] = msk;
      }
      __syncthreads();
      // 2. top-k entries of the tile's tokens (set union; -1, repeats and
      //    blocks after the token's own are ignored).
      {
#pragma unroll
        for (int k = 0; k < kTPW; ++k) {
          if (!tval[k]) continue;
          const int32_t* list = a.bidx + ((int64_t)g * a.rows_q + trow[k]) * a.n_sel;
          const uint32_t bit = 1u << tb[k];
          for (int e = lane; e < a.n_sel; e += 64) {
            const int b = list[e];
            if (b >= 0 && b <= bt[k] && b >= w0 && b < w1 && kBlock * b + kBlock <= a.vt_ld)
              atomicOr(&sh.mask[b - w0], bit);
          }
        }
      }
      __syncthreads();
      // 3. compact the shared-phase blocks, ascending: entry e = 512*j + tid
      //    goes to (blocks before round j) + (blocks of earlier waves in
      //    round j) + (earlier lanes of this wave).
      uint64_t bal[kWin / kThreads];
#pragma unroll
      for (int j = 0; j < kWin / kThreads; ++j) {
        const int e = kThreads * j + tid;
        const uint32_t v = e < nblk ? sh.mask[e] : 0u;
        bal[j] = __ballot(v != 0u && __builtin_popcount(v) >= kShareMin);
        if (kSingle && v != 0u && __builtin_popcount(v) < kShareMin) {
          for (uint32_t x = v; x != 0u; x &= x - 1u) atomicAdd(&sh.pcnt[__builtin_ctz(x)], 1);
        }
        if (lane == 0) sh.cnt[j][wave] = __builtin_popcountll(bal[j]);
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kWin / kThreads; ++j) {
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) {
          const int c = sh.cnt[j][w];
          before += w < wave ? c : 0;
          total += c;
        }
        if ((bal[j] >> lane) & 1ull) {
          const int e = kThreads * j + tid;
          const int pos = n_ent + before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[j] >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bal[j], 0u));
          sh.ub[pos] = w0 + e;
          sh.um[pos] = sh.mask[e];
        }
        n_ent += total;
      }
      __syncthreads();
      // 3a. balance the private phase: the tokens ranked by private block
      //     count are paired heaviest with lightest, one pair per wave, and the
      //     waves take over their new tokens (no token has been touched yet).
      if (kSingle) {
        static_assert(kTPW == 2, "the pairing gives each wave two tokens");
        if (wave == 0 && lane < kTileTok) {
          const int c = sh.pcnt[lane];
          int rank = 0;
#pragma unroll
          for (int j = 0; j < kTileTok; ++j) {
            const int cj = sh.pcnt[j];
            rank += (cj > c || (cj == c && j < lane)) ? 1 : 0;
          }
          const int slot = rank < kTileTok / 2 ? kTPW * rank : kTPW * (kTileTok - 1 - rank) + 1;
          sh.perm[slot] = lane;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kTPW; ++k) {
          const int tt = __builtin_amdgcn_readfirstlane(sh.perm[wave * kTPW + k]);
          if (tt != tb[k]) init_token(k, tt, i0, pos0);
        }
      }
      // 3b. order the shared list for balance: within each run of 64 entries an
      //     entry is followed by the first later one whose tokens lie in other
      //     waves (else by the next one), so the two blocks of a batch tend to
      //     occupy different waves.  Runs are 64 entries, so batches of two
      //     never straddle them.
      if (kSingle) {
        for (int c = wave; 64 * c < n_ent; c += kAttnWaves) {
          const int cnt = min(64, n_ent - 64 * c);
          const bool ok = lane < cnt;
          const int32_t ubv = ok ? sh.ub[64 * c + lane] : 0;
          const uint32_t umv = ok ? sh.um[64 * c + lane] : 0u;
          uint32_t wm = 0;
#pragma unroll
          for (int w = 0; w < kAttnWaves; ++w) {
            uint32_t wb = 0;
#pragma unroll
            for (int k = 0; k < kTPW; ++k) wb |= 1u << sh.perm[kTPW * w + k];
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
      }
    }
    // 4. shared phase: walk the list; the next batch's staging loads are in
    //    flight while the current one computes.
    if (n_ent > 0) {
      // Batches of two blocks: the ring holds the batch being consumed and
      // the next one in flight; one barrier per batch, so the per-wave load
      // imbalance of single blocks averages over two.
      // Entry u of the list: its block and the tile tokens attending it.
      const auto ent_block = [&](int u) -> int {
        return dense ? w0 + u : __builtin_amdgcn_readfirstlane(sh.ub[u]);
      };
      const auto ent_mask = [&](int u, int b) -> uint32_t {
        if (!dense) return __builtin_amdgcn_readfirstlane(sh.um[u]);
        const int lo = max(dlo, kBlock * b - p0);   // tokens at positions >= 64 b
        return lo < dhi ? ((1u << dhi) - 1u) & ~((1u << lo) - 1u) : 0u;
      };
      stage_issue(sh.ring[0][0], sh.ring[0][1], ent_block(0));
      if (n_ent > 1) stage_issue(sh.ring[1][0], sh.ring[1][1], ent_block(1));
      for (int u = 0; u < n_ent; u += 2) {
        const int half = (u >> 1) & 1;
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // this wave's part of the batch has landed
        __syncthreads();                            // ... every wave's; the other half is free
        const int b0 = ent_block(u);
        const int b1 = u + 1 < n_ent ? ent_block(u + 1) : -1;
        const bool p0 = kBlock * b0 + kBlock > rk.len;
        const bool p1 = b1 >= 0 && kBlock * b1 + kBlock > rk.len;
        if (p0 || p1) {
          if (p0) fix_partial(sh.ring[2 * half][1], b0);
          if (p1) fix_partial(sh.ring[2 * half + 1][1], b1);
          __syncthreads();
        }
        if (u + 2 < n_ent) stage_issue(sh.ring[2 * (half ^ 1)][0], sh.ring[2 * (half ^ 1)][1], ent_block(u + 2));
        if (u + 3 < n_ent) stage_issue(sh.ring[2 * (half ^ 1) + 1][0], sh.ring[2 * (half ^ 1) + 1][1], ent_block(u + 3));
        const uint32_t m0 = sel_of(ent_mask(u, b0));
        if (m0) consume<kSingle>(m0, sh.ring[2 * half][0], sh.ring[2 * half][1], b0);
        if (b1 >= 0) {
          const uint32_t m1 = sel_of(ent_mask(u + 1, b1));
          if (m1) consume<kSingle>(m1, sh.ring[2 * half + 1][0], sh.ring[2 * half + 1][1], b1);
        }
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();   // the ring becomes the private regions
    }
    // 5. private phase: this wave's blocks that stayed out of the shared
    //    list, one block in flight (K in the wave's region, V^T in
    //    registers): its loads are issued once the previous block's
    //    products have read the region and registers, while the other waves
    //    compute.  The walk is ascending from a start point that advances by
    //    1/64 of the range per dispatch rank on the XCD (and wraps), so the
    //    workgroups running side by side on an XCD pass the same part of the
    //    range at about the same time and share the blocks they have in
    //    common in its L2 (-0.7% kernel time at 128K against walks that all
    //    start at block 0; the result does not depend on the order beyond
    //    rounding, and the order is fixed).
    if (!dense) {
      uint8_t* region = &sh.ring[0][0][0] + wave * (64 * 256);
      const uint32_t mine = mine_mask();
      uint64_t pend = 0;
      const int nch = (nblk + 63) / 64;
      const int start = (int)((int64_t)(xrank % 64u) * nblk / 64);
      const int c0 = start / 64;
      int step = 0, cur = 0;
      // Next private block of this wave (wave-uniform), or -1: chunks of 64
      // entries from the start point's, which is visited twice (its entries
      // from the start point on, then at the end those before it).
      auto next_block = [&](uint32_t& sel) -> int {
        while (pend == 0) {
          if (nch == 0 || step > nch) return -1;
          const int c = (c0 + step) % nch;
          const int e = c * 64 + lane;
          const uint32_t v = e < nblk ? sh.mask[e] : 0u;
          bool ok = (v & mine) != 0u && __builtin_popcount(v) < kShareMin;
          if (step == 0) ok = ok && e >= start;
          if (step == nch) ok = ok && e < start;
          pend = __ballot(ok);
          cur = c;
          ++step;
        }
        const int e = cur * 64 + (int)__builtin_ctzll(pend);
        pend &= pend - 1;
        sel = sel_of(__builtin_amdgcn_readfirstlane(sh.mask[e]));
        return w0 + e;
      };
      uint32_t sc = 0;
      int bc = next_block(sc);
      u32x4 vb[8][2];
      if (bc >= 0) {
        issue_k_private(region, bc);
        load_v_private(vb, bc);
      }
      while (bc >= 0) {
        uint32_t sn = 0;
        const int bn = next_block(sn);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // K(bc) in the region, V(bc) in registers
        consume_private<kSingle>(sc, region, vb, bc);
        if (bn >= 0) {
          __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0): the region's K reads are done
          issue_k_private(region, bn);
          load_v_private(vb, bn);
        }
        bc = bn;
        sc = sn;
      }
    }
  }

  template <bool kMulti, bool kDense>
  __device__ void run(AttnLds& sh) {
    // XCD-aware order: workgroups are dispatched round-robin over the 8
    // XCDs; remap them so each XCD walks a contiguous range of query tiles
    // (neighbouring tiles share their local window and hot blocks in L2).
    const unsigned nx = gridDim.x, ny = gridDim.y;
    const unsigned N = nx * ny * gridDim.z;
    const unsigned L = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
    unsigned T;
    if (kDense && 8u * nx > N) {
      // Dense causal over a sequence longer than one XCD's share of the
      // grid: a tile's work grows with its position, and contiguous ranges
      // left the XCDs holding the last tiles with most of the work (measured
      // 16 -> 9.4 ms at 32K).  Chunks of 32 consecutive tiles go to the XCDs
      // round-robin (L2 reuse inside a chunk), heaviest first.
      constexpr unsigned C = 32;
      const unsigned full = N - N % (8u * C);
      T = L;
      if (L < full) {
        const unsigned k = L / 8u, x = L % 8u;
        T = (8u * (k / C) + x) * C + k % C;
      }
      T = N - 1u - T;
    } else {
      const unsigned full = N - N % 8u;
      T = L < full ? (L % 8u) * (full / 8u) + L / 8u : L;
      // Last tiles first: dense causal tiles grow with their position, and
      // sparse ones up to the first |I| blocks (the launch's tail then holds
      // the light tiles).
      T = N - 1u - T;
    }
    xrank = L / 8u;
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
    init_offsets();

#pragma unroll
    for (int k = 0; k < kTPW; ++k) init_token(k, wave * kTPW + k, i0, pos0);

    const int nq = min(kTileTok, rq.len - i0);
    const int bt_last = max(0, pos0 + i0 + nq - 1) / kBlock;
    // Keys up to kWin blocks (V^T rows of at most 64 * kWin) take one
    // window, in a kernel without a loop around the phases (a loop would keep
    // both phases' address registers live at once).  Blocks past the V^T row
    // are never attended, so clamping to kWin there loses nothing.
    if constexpr (!kMulti) {
      window<true, kDense>(sh, 0, min(bt_last + 1, kWin), nq, pos0, i0, tid);
    } else {
      for (int w0 = 0; w0 <= bt_last; w0 += kWin) {
        window<false, kDense>(sh, w0, min(bt_last + 1, w0 + kWin), nq, pos0, i0, tid);
        __syncthreads();   // mask, lists and LDS are reused by the next window
      }
    }

#pragma unroll
    for (int k = 0; k < kTPW; ++k) {
      const float lt = sum_x16(sum_x32(l[k]));
      // Rows of the sequence placed before its first key attend nothing
      // (their state is untouched: out = 0, lse = -inf).
      if (trow[k] - rq.start >= rq.len || trow[k] >= a.rows_q) continue;
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

template <bool kMulti, bool kDense>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) AttnLds sh;
  Attn st(a);
  st.run<kMulti, kDense>(sh);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int max_seqlen_q, hipStream_t st) {
  dim3 grid((max_seqlen_q + kTileTok - 1) / kTileTok, a.h_kv, a.batch);
  const bool multi = a.vt_ld > (int64_t)kWin * kBlock, dense = a.bidx == nullptr;
  if (dense) {
    if (multi) hipLaunchKernelGGL((attn_kernel<true, true>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((attn_kernel<false, true>), grid, dim3(kThreads), 0, st, a);
  } else {
    if (multi) hipLaunchKernelGGL((attn_kernel<true, false>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((attn_kernel<false, false>), grid, dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace infllmv2

// ---------------------------------------------------------------------------
// Split-K path.  With few query tiles (decode: one token per sequence) the
// tile kernel above would leave most of the chip idle, each workgroup
// walking a whole block list alone.  Here a workgroup takes one query row,
// one KV group and one range of the row's (deduplicated, ascending) block
// set; its four waves take every fourth block of the range straight from
// global memory into registers, merge their online-softmax states in LDS and
// write one partial.  The merge kernel combines the partials of a row.
// ---------------------------------------------------------------------------
namespace infllmv2 {
namespace {

constexpr int kSplitWaves = 4;
constexpr int kSplitThreads = 64 * kSplitWaves;

constexpr int kWordsPerThread = 8;   // bitmap of up to 65536 blocks (4M keys)

struct SplitLds {
  uint32_t bits[kWordsPerThread * kSplitThreads];
  int32_t list[kSplitMaxSel];
  int32_t cnt[kSplitWaves];
  float pm[kSplitWaves][16];   // running max per head (the lanes of a head share it)
  float pl[kSplitWaves][16];
  float po[kSplitWaves][16 * kHeadDim];
};

__global__ __launch_bounds__(kSplitThreads, 2) void attn_split_kernel(AttnArgs a, int splits, float* part) {
  __shared__ __attribute__((aligned(16))) SplitLds sh;
  const int sp = blockIdx.x, g = blockIdx.y;
  const int64_t row = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, q4 = lane >> 4, c16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool dense = a.bidx == nullptr;
  // The row's list entries and query fragments depend on the row alone: they
  // are read in the same round as its sequence's metadata.
  int lv[kSplitMaxSel / kSplitThreads];
#pragma unroll
  for (int j = 0; j < kSplitMaxSel / kSplitThreads; ++j) {
    const int i = tid + kSplitThreads * j;
    lv[j] = (!dense && i < a.n_sel) ? a.bidx[((int64_t)g * a.rows_q + row) * a.n_sel + i] : -1;
  }
  // Query fragments (the group's heads are the 16 MFMA columns, padded).
  bf16x8 qb[4];
  {
    const bool hv = c16 < a.G;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 v = zero16();
      if (hv) v = ldg16(a.q + (row * a.h_q + g * a.G + c16) * kHeadDim + 32 * ks + 8 * q4);
      qb[ks] = as_bf16x8(v);
    }
  }
  RowSeq rsq;
  if (!find_row_seq(a.cu_q, a.used_q, a.cu_k, a.used_k, nullptr, a.batch, row, rsq)) return;
  const int s = rsq.s;
  const SeqRange rq = rsq.rq, rk = rsq.rk;
  const int t = rk.len - rq.len + (int)(row - rq.start);
  if (t < 0) return;
  const int bt = t / kBlock;
  const int nvt = (int)(a.vt_ld / kBlock);   // blocks inside a V^T row

  // The row's block set, ascending and without repeats.
  int nb;
  if (dense) {
    nb = min(bt + 1, nvt);
  } else {
    // Set of candidate blocks (the list, the init blocks, the local blocks)
    // as a bitmap over blocks 0..bt, then listed ascending.
    const int nbits = min(min(bt + 1, nvt), kWordsPerThread * kSplitThreads * 32);
    const int nwords = (nbits + 31) >> 5;
    for (int w = tid; w < nwords; w += kSplitThreads) sh.bits[w] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSplitMaxSel / kSplitThreads; ++j)
      if (lv[j] >= 0 && lv[j] < nbits) atomicOr(&sh.bits[lv[j] >> 5], 1u << (lv[j] & 31));
    for (int i = tid; i < a.n_init + a.n_local; i += kSplitThreads) {
      const int b = i < a.n_init ? i : bt - (i - a.n_init);
      if (b >= 0 && b < nbits) atomicOr(&sh.bits[b >> 5], 1u << (b & 31));
    }
    __syncthreads();
    // Thread tid owns words kWordsPerThread*tid .. +kWordsPerThread-1.
    uint32_t wv[kWordsPerThread];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kWordsPerThread; ++j) {
      const int w = kWordsPerThread * tid + j;
      wv[j] = w < nwords ? sh.bits[w] : 0u;
      cnt += __builtin_popcount(wv[j]);
    }
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) sh.cnt[wave] = incl;
    __syncthreads();
    int base = 0;
    nb = 0;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) {
      base += w < wave ? sh.cnt[w] : 0;
      nb += sh.cnt[w];
    }
    int pos = base + incl - cnt;
#pragma unroll
    for (int j = 0; j < kWordsPerThread; ++j) {
      uint32_t x = wv[j];
      while (x) {
        const int bit = __builtin_ctz(x);
        x &= x - 1u;
        sh.list[pos++] = 32 * (kWordsPerThread * tid + j) + bit;
      }
    }
    __syncthreads();
  }
  const int lo = (int)((int64_t)nb * sp / splits), hi = (int)((int64_t)nb * (sp + 1) / splits);
  floatx4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = -1e30f, l = 0.f;
  const uint16_t* vbase = a.vt + ((int64_t)g * kHeadDim * a.batch + s) * a.vt_ld;
  const int64_t vdim = (int64_t)a.batch * a.vt_ld;

  for (int r = lo + wave; r < hi; r += kSplitWaves) {
    const int b = dense ? r : sh.list[r];
    bf16x8 kf[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      int64_t krow = (int64_t)rk.start + kBlock * b + key_of(kt, c16);
      krow = krow < a.rows_k ? krow : a.rows_k - 1;
      const uint16_t* kp = a.k + (krow * a.h_kv + g) * kHeadDim + 8 * q4;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[kt][ks] = as_bf16x8(ldg16(kp + 32 * ks));
    }
    u32x4 vb[8][2];
    const uint16_t* vp = vbase + (int64_t)c16 * vdim + kBlock * b + 8 * q4;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) vb[dt][kk] = ldg16(vp + (int64_t)(16 * dt) * vdim + 32 * kk);
    floatx4 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sacc[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sacc[kt] = mfma16(kf[kt][ks], qb[ks], sacc[kt]);
    }
    // Online softmax update (keys after the query masked in its own block),
    // exponentiated against the running max first; the block max is looked
    // for only when some lane's sum passes 2^8 (see the tile kernel).
    float v[4][4];
    const int lim = t - kBlock * b - 8 * q4;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        v[kt][rr] = (b < bt || 32 * (kt >> 1) + 4 * (kt & 1) + rr <= lim) ? sacc[kt][rr] : -__builtin_inff();
    float p[4][4];
    float ls = 0.f;
    const auto exponentiate = [&]() {
      const float mc = m * a.c;
      ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          p[kt][rr] = fast_exp2(fmaf(v[kt][rr], a.c, -mc));
          ls += p[kt][rr];
        }
    };
    exponentiate();
    if (__ballot(!(ls <= kLazySum)) != 0) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) mx = fmaxf(mx, v[kt][rr]);
      mx = max_x32(max_x16(mx));
      if (__ballot(mx * a.c > m * a.c + kLazyLog2) != 0) {
        const float mn = fmaxf(m, mx);
        const float alpha = fast_exp2((m - mn) * a.c);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) o[dt][rr] *= alpha;
        exponentiate();
      }
    }
    l += ls;
    bf16x8 pb[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 w;
      w[0] = pack_bf16x2(p[2 * kk][0], p[2 * kk][1]);
      w[1] = pack_bf16x2(p[2 * kk][2], p[2 * kk][3]);
      w[2] = pack_bf16x2(p[2 * kk + 1][0], p[2 * kk + 1][1]);
      w[3] = pack_bf16x2(p[2 * kk + 1][2], p[2 * kk + 1][3]);
      pb[kk] = as_bf16x8(w);
    }
    const bool partial = kBlock * b + kBlock > rk.len;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x4 vv = partial ? clip_keys(vb[dt][kk], kBlock * b + 32 * kk + 8 * q4, rk.len) : vb[dt][kk];
        o[dt] = mfma16(as_bf16x8(vv), pb[kk], o[dt]);
      }
  }

  // Merge the four waves' states, then write the workgroup's partial.
  const float lt = sum_x16(sum_x32(l));
  if (q4 == 0) {
    sh.pm[wave][c16] = m;
    sh.pl[wave][c16] = lt;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *reinterpret_cast<floatx4*>(&sh.po[wave][c16 * kHeadDim + 16 * dt + 4 * q4]) = o[dt];
  __syncthreads();
  const int h = tid >> 4, d0 = 8 * (tid & 15);
  float M = sh.pm[0][h];
#pragma unroll
  for (int w = 1; w < kSplitWaves; ++w) M = fmaxf(M, sh.pm[w][h]);
  float L = 0.f, acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
  for (int w = 0; w < kSplitWaves; ++w) {
    const float wt = fast_exp2((sh.pm[w][h] - M) * a.c);
    L += wt * sh.pl[w][h];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += wt * sh.po[w][h * kHeadDim + d0 + i];
  }
  float* dst = part + (((int64_t)row * a.h_kv + g) * splits + sp) * kPartFloats;
#pragma unroll
  for (int i = 0; i < 8; i += 4)
    *reinterpret_cast<floatx4*>(dst + h * kHeadDim + d0 + i) = floatx4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]};
  if ((tid & 15) == 0) {
    dst[16 * kHeadDim + h] = L;
    dst[16 * kHeadDim + 16 + h] = M;
  }
}

__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int splits, const float* part) {
  __shared__ float wt[kSplitMaxSplits][16];
  __shared__ float lp[kSplitMaxSplits][16];
  __shared__ float Mh[16], Lh[16];
  const int g = blockIdx.x;
  const int64_t row = blockIdx.y;
  const int tid = threadIdx.x, h = tid >> 4, d0 = 8 * (tid & 15);
  const float* src = part + ((int64_t)row * a.h_kv + g) * splits * kPartFloats;
  // Per-split maxima of every head, then each head's weights and sum (read
  // in the same round as the row's metadata; a row outside every sequence
  // has no partials and writes nothing).
  for (int i = tid; i < 16 * splits; i += 256) {
    wt[i >> 4][i & 15] = src[(i >> 4) * kPartFloats + 16 * kHeadDim + 16 + (i & 15)];
    lp[i >> 4][i & 15] = src[(i >> 4) * kPartFloats + 16 * kHeadDim + (i & 15)];
  }
  RowSeq rsq;
  if (!find_row_seq(a.cu_q, a.used_q, a.cu_k, a.used_k, nullptr, a.batch, row, rsq)) return;
  // A row placed before its sequence's first key attends nothing (the split
  // kernel wrote no partial for it): out = 0, lse = -inf.
  const int nparts = rsq.rk.len - rsq.rq.len + (int)(row - rsq.rq.start) < 0 ? 0 : splits;
  __syncthreads();
  if (tid < 16) {
    float M = -__builtin_inff();
    for (int p = 0; p < nparts; ++p) M = fmaxf(M, wt[p][tid]);
    float L = 0.f;
    for (int p = 0; p < nparts; ++p) {
      const float w = fast_exp2((wt[p][tid] - M) * a.c);
      wt[p][tid] = w;
      L += w * lp[p][tid];
    }
    Mh[tid] = M;
    Lh[tid] = L;
  }
  __syncthreads();
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll 4
  for (int p = 0; p < nparts; ++p) {
    const float* pp = src + p * kPartFloats + h * kHeadDim + d0;
    const floatx4 x0 = *reinterpret_cast<const floatx4*>(pp);
    const floatx4 x1 = *reinterpret_cast<const floatx4*>(pp + 4);
    const float w = wt[p][h];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] += w * x0[i];
      acc[4 + i] += w * x1[i];
    }
  }
  if (h >= a.G) return;
  const float L = Lh[h];
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* dst = a.out + (row * a.h_q + g * a.G + h) * kHeadDim + d0;
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  stg16(dst, w);
  if (a.lse && (tid & 15) == 0)
    a.lse[(int64_t)(g * a.G + h) * a.rows_q + row] = L > 0.f ? Mh[h] * a.scale + logf(L) : -__builtin_inff();
}

}  // namespace

hipError_t launch_attention_split(const AttnArgs& a, int64_t rows_q, int splits, float* part,
                                  hipStream_t st) {
  hipLaunchKernelGGL(attn_split_kernel, dim3(splits, a.h_kv, (unsigned)rows_q), dim3(kSplitThreads), 0, st, a,
                     splits, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(a.h_kv, (unsigned)rows_q), dim3(256), 0, st, a, splits,
                     (const float*)part);
  return hipGetLastError();
}

}  // namespace infllmv2
