// Block scoring on bf16 MFMA: stages 2 and 3 of the three-stage block
// representation (top168.com article on InfLLM-V2, section 三 "块表示的三阶段压缩")
// with the hardware-aware two-pass scheme of section 四 "高效实现的技术突破".
//
//   pass 1 (score_lse_kernel):    L[t, h] = log sum_j exp(scale * q[t,h] . kc[g, j])
//                                  over the windows j visible to t.  Run on the
//                                  stage-1 keys it is exact; run on the coarse
//                                  keys (kernel 128, stride 64) it is the LSE
//                                  approximation.
//   pass 2 (score_blocks_kernel): p[t, h, j] = exp(scale * q[t,h] . kc1[g, j] - L[t, h]),
//                                  S[t, g, j] = sum over the group's heads of p,
//                                  score[t, g, b] = max_{j = 4b-1 .. 4b+3} S[t, g, j].
//                                  The group sum and the max pool happen in
//                                  registers; only block scores reach HBM.
//
// Tiling: a workgroup owns 16 query tokens of one sequence and one KV group
// (4 waves x 4 tokens).  For one token the 16 heads of its group are the 16
// rows of a 16x16x32 MFMA tile and 16 compressed keys its columns, so each
// lane ends up holding 4 heads of one window: the group sum is 3 in-lane adds
// plus a reduce-scatter over the four 16-lane rows, after which lane l holds
// S for window (start of its 64 windows + l) and a quad max gives the block
// score.
// Compressed-key tiles of 128 windows are staged in LDS (direct global->LDS
// loads, double-buffered: the next tile lands while this one computes) and
// shared by the 4 waves; each LDS fragment feeds 4 MFMAs (one per token).
// Within a tile the 16-window chunks are software-pipelined: one chunk's
// MFMAs are in flight while the previous chunk's exponentials run.
// Group sizes below 16 pad the head rows with zeros.
//
// Pass 1 keeps a per-row offset instead of a per-element running max: the
// first 16 windows set it to their exact max; afterwards a row's sum is only
// renormalised (by a power of two) when it exceeds 2^32, and a tile whose sum
// overflows is redone with its exact max (one test per tile for the whole
// wave).  Every exponent stays finite and the result is the same log-sum-exp,
// with one FMA, one exp and one add per score on full tiles; the offset is
// kept in log2 units (scaled by scale * log2 e), so L = m ln 2 + ln(sum).
#include "kernels.hpp"

namespace infllmv2 {

namespace {

constexpr int kQT = 16;      // query tokens per workgroup
constexpr int kTPW = 4;      // tokens per wave
constexpr int kWT = 128;     // windows per tile
constexpr int kCT = kWT / 16;  // 16-window chunks per tile

// DPP move of a float: lane i takes src from the lane the control selects;
// lanes without a source keep `old`.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), kCtrl, 0xF, 0xF, false));
}

__device__ __forceinline__ int n_visible(int t, int win_kernel, int win_stride, int nwin) {
  if (t < win_kernel - 1) return 0;
  return min(nwin, (t - win_kernel + 1) / win_stride + 1);
}

// Scheduling fence: keeps the compiler from sinking a chunk's fragment reads
// to their first use (it does so to save registers, and the MFMAs then wait
// on LDS latency).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Stage windows j0 .. j0 + kWT - 1 of one sequence's compressed keys into
// LDS with direct global->LDS loads: kWT rows of 256 bytes, 1 KB parts, part
// p written by wave p % 4.  LDS chunk c of row w receives global chunk
// c ^ (w & 7), so that 8 consecutive rows read at the same chunk hit
// distinct banks.  A wave's rows are 4 * wave + 16 * it + lane / 16 and its
// chunk swizzle is the same in every part, so the per-lane byte offset
// `voff` is loop-invariant and the tile and part advance the uniform base
// only.  Rows past the last valid one (`rmax`, relative to the sequence's
// first window) read that row instead and are masked by visibility.
__device__ __forceinline__ void stage_windows(uint8_t* lds, const uint8_t* base, int j0, int rmax,
                                              uint32_t voff, int lw, int wave) {
  if (j0 + kWT - 1 <= rmax) {
    const uint8_t* b = base + (int64_t)j0 * 256;
#pragma unroll
    for (int it = 0; it < kWT / 16; ++it)
      __builtin_amdgcn_global_load_lds(b + it * 4096 + voff,
                                       (__attribute__((address_space(3))) void*)(lds + (wave + 4 * it) * 1024),
                                       16, 0, 0);
  } else {
#pragma unroll
    for (int it = 0; it < kWT / 16; ++it) {
      const int row = min(j0 + lw + 16 * it, rmax);
      __builtin_amdgcn_global_load_lds(base + (uint32_t)(row * 256 + (voff & 255)),
                                       (__attribute__((address_space(3))) void*)(lds + (wave + 4 * it) * 1024),
                                       16, 0, 0);
    }
  }
}

__device__ __forceinline__ bf16x8 lds_window_frag(const uint8_t* lds, int w, int ch) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(lds + w * 256 + ((ch ^ (w & 7)) << 4)));
}

template <int PASS>
__device__ __forceinline__ void score_body(const ScoreArgs& a, uint8_t* lds) {
  const int s = blockIdx.z;
  const int g = blockIdx.y;
  const SeqRange rq = seq_range(a.cu_q, a.used_q, s);
  const SeqRange rk = seq_range(a.cu_k, a.used_k, s);
  // A tile's work grows with its position (causal windows): the last tiles
  // are dispatched first, so the tail of the launch holds the light ones
  // (8.58 -> 8.32 ms for selection at 128K).  PASS 3 (unfused baseline) runs
  // over one chunk of query rows at a time.
  const int i0 = (PASS == 3 ? a.chunk0 : 0) + (int)(PASS == 3 ? blockIdx.x : gridDim.x - 1 - blockIdx.x) * kQT;
  if (i0 >= rq.len) return;
  const int pos0 = rk.len - rq.len;
  const int nq = min(kQT, rq.len - i0);
  const int t_first = pos0 + i0;
  const int t_last = t_first + nq - 1;
  const int n_sel = a.n_init + a.n_local + a.n_topk;
  // Rows whose candidate count does not exceed n_topk keep every block; none
  // of them needs scores.
  if (t_last < n_sel * kBlock) return;
  const int nwin = rk.len >= a.win_kernel ? (rk.len - a.win_kernel) / a.win_stride + 1 : 0;

  int j_begin, j_end;
  if (PASS == 1) {
    j_begin = 0;
    j_end = n_visible(t_last, a.win_kernel, a.win_stride, nwin);
  } else {
    const int b_hi = t_last / kBlock - a.n_local;      // last candidate block in the tile
    j_begin = max(0, 4 * a.n_init - 1) & ~(kWT - 1);
    j_end = 4 * b_hi + 4;
  }
  if (j_end <= j_begin) return;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int q4 = lane >> 4;
  const int c16 = lane & 15;
  const int64_t c0 = a.cu_c[s];
  if (c0 < 0 || c0 >= a.c_rows) return;   // inconsistent metadata: nothing to read
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.kc + ((int64_t)g * a.c_rows + c0) * kHeadDim);
  const int rmax = (int)(a.c_rows - 1 - c0);
  const int lw = 4 * wave + q4;
  const uint32_t voff = (uint32_t)(lw * 256 + ((c16 ^ (lw & 7)) << 4));

  int tpos[kTPW], nv[kTPW], bt[kTPW];
  int64_t trow[kTPW];
  bool tval[kTPW], need[kTPW];
  bf16x8 qa[kTPW][4];
  float Lc[kTPW][4];
#pragma unroll
  for (int k = 0; k < kTPW; ++k) {
    const int i = i0 + wave * kTPW + k;
    tval[k] = i < rq.len;
    tpos[k] = pos0 + i;
    trow[k] = (int64_t)rq.start + i;
    bt[k] = tpos[k] / kBlock;
    need[k] = tval[k] && (bt[k] - a.n_local - a.n_init + 1 > a.n_topk) && trow[k] < a.rows_q;
    nv[k] = n_visible(tpos[k], a.win_kernel, a.win_stride, nwin);
    const bool hv = tval[k] && c16 < a.G && trow[k] < a.rows_q;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 v = zero16();
      if (hv) v = ldg16(a.q + (trow[k] * a.h_q + g * a.G + c16) * kHeadDim + 32 * ks + 8 * q4);
      qa[k][ks] = as_bf16x8(v);
    }
    if (PASS >= 2) {
      // Loads at clamped addresses first, the conditions after, so the four
      // loads are in flight together.
      float lraw[4];
      const int64_t lrow = min(trow[k], a.rows_q - 1);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        lraw[r] = a.lse[(int64_t)(g * a.G + min(4 * q4 + r, a.G - 1)) * a.rows_q + lrow];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool use = need[k] && 4 * q4 + r < a.G && lraw[r] > -__builtin_inff();
        Lc[k][r] = use ? lraw[r] * 1.4426950408889634f : __builtin_inff();
      }
    }
  }

  // Pass 1 row state, in the exp2 domain: offset m (scaled by c) and sum.
  // Pass 2: the last window sum of the previous 64 windows (bit pattern),
  // each token's block-score row and its last candidate block (-1: none).
  float m[kTPW][4], ssum[kTPW][4];
  int carry[kTPW], b_hi[kTPW];
  float* bs_row[kTPW];
#pragma unroll
  for (int k = 0; k < kTPW; ++k) {
    carry[k] = 0;
    b_hi[k] = need[k] ? (int)min((int64_t)(bt[k] - a.n_local), a.bs_ld - 1) : -1;
    bs_row[k] = a.bs + ((int64_t)g * a.rows_q + min(trow[k], a.rows_q - 1)) * a.bs_ld;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m[k][r] = 0.f;
      ssum[k][r] = 0.f;
    }
  }
  const int nv_first = n_visible(t_first, a.win_kernel, a.win_stride, nwin);
  const int ntiles = (j_end - j_begin + kWT - 1) / kWT;

  // B fragments of chunk ct (16 windows) and the S^T chunk (16 windows x 16
  // heads) of every token of the wave: four independent MFMA chains.
  auto frags = [&](const uint8_t* cur, int ct, bf16x8 (&b)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) b[ks] = lds_window_frag(cur, 16 * ct + c16, 4 * ks + q4);
  };
  auto mm = [&](const bf16x8 (&b)[4], floatx4 (&acc)[kTPW]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int k = 0; k < kTPW; ++k)
        acc[k] = mfma16(qa[k][ks], b[ks], ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : acc[k]);
  };
  auto chunk = [&](const uint8_t* cur, int ct, floatx4 (&acc)[kTPW]) {
    bf16x8 b[4];
    frags(cur, ct, b);
    mm(b, acc);
  };
  // Walk over the chunks of a staged tile, software-pipelined: the MFMAs of
  // chunk ct are issued (and the fragments of chunk ct + 1 read) before
  // chunk ct - 1's scores are consumed, so one chunk's exponentials run
  // while the matrix cores compute the next.
  auto walk = [&](const uint8_t* cur, auto&& consume) {
    bf16x8 b[2][4];
    floatx4 acc[2][kTPW];
    frags(cur, 0, b[0]);
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      sched_fence();
      if (ct + 1 < kCT) frags(cur, ct + 1, b[(ct + 1) & 1]);
      sched_fence();
      mm(b[ct & 1], acc[ct & 1]);
      if (ct > 0) consume(acc[(ct - 1) & 1], ct - 1);
    }
    sched_fence();
    consume(acc[(kCT - 1) & 1], kCT - 1);
  };

  stage_windows(lds, kbase, j_begin, rmax, voff, lw, wave);
  for (int it = 0; it < ntiles; ++it) {
    const int jt = j_begin + it * kWT;
    const uint8_t* cur = lds + (it & 1) * (kWT * 256);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's part of tile it has landed
    __syncthreads();                 // ... every wave's; the other buffer is free
    if (it + 1 < ntiles) stage_windows(lds + ((it + 1) & 1) * (kWT * 256), kbase, jt + kWT, rmax, voff, lw, wave);

    // Every window of the tile is visible to every token of the tile: no
    // per-score visibility test.
    const bool full = jt + kWT <= nv_first;
    if (PASS == 1) {
      if (it == 0) {
        // Offset of each row: the max over its visible windows among the
        // first 16 (every scored token sees window 0).
        floatx4 acc[kTPW];
        chunk(cur, 0, acc);
#pragma unroll
        for (int k = 0; k < kTPW; ++k)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float v = jt + c16 < nv[k] ? acc[k][r] : -__builtin_inff();
            float mt = v;   // max over the 16 windows: lanes of this 16-lane row
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off));
            m[k][r] = mt > -__builtin_inff() ? mt * a.c : 0.f;
          }
      }
      float st[kTPW][4];
      if (full) {
        walk(cur, [&](floatx4 (&acc)[kTPW], int ct) {
#pragma unroll
          for (int k = 0; k < kTPW; ++k)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float e = fast_exp2(fmaf(acc[k][r], a.c, -m[k][r]));
              st[k][r] = ct == 0 ? e : st[k][r] + e;
            }
        });
      } else {
        walk(cur, [&](floatx4 (&acc)[kTPW], int ct) {
#pragma unroll
          for (int k = 0; k < kTPW; ++k) {
            const bool ok = jt + 16 * ct + c16 < nv[k];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float e = ok ? fast_exp2(fmaf(acc[k][r], a.c, -m[k][r])) : 0.f;
              st[k][r] = ct == 0 ? e : st[k][r] + e;
            }
          }
        });
      }
      // One test per tile for the whole wave: a new sum past 2^32, or a tile
      // sum that overflowed (its new sum is then infinite).  Both are rare:
      // an overflowed tile is redone with its exact max, a large sum is
      // renormalised by a power of two.
      float ns[kTPW][4];
      float mx = 0.f;
#pragma unroll
      for (int k = 0; k < kTPW; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ns[k][r] = ssum[k][r] + st[k][r];
          mx = fmaxf(mx, ns[k][r]);
        }
      if (__ballot(!(mx <= 4294967296.f)) != 0) {
        bool bad = false;
#pragma unroll
        for (int k = 0; k < kTPW; ++k)
#pragma unroll
          for (int r = 0; r < 4; ++r) bad |= !(st[k][r] <= 3.0e38f);
        if (__ballot(bad) != 0) {
          float mt[kTPW][4];
#pragma unroll
          for (int k = 0; k < kTPW; ++k)
#pragma unroll
            for (int r = 0; r < 4; ++r) mt[k][r] = m[k][r];
#pragma unroll 1
          for (int ct = 0; ct < kCT; ++ct) {
            floatx4 acc[kTPW];
            chunk(cur, ct, acc);
#pragma unroll
            for (int k = 0; k < kTPW; ++k) {
              const bool ok = full || (jt + 16 * ct + c16 < nv[k]);
#pragma unroll
              for (int r = 0; r < 4; ++r) mt[k][r] = fmaxf(mt[k][r], ok ? acc[k][r] * a.c : mt[k][r]);
            }
          }
#pragma unroll
          for (int k = 0; k < kTPW; ++k)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              ns[k][r] = ssum[k][r] * fast_exp2(m[k][r] - mt[k][r]);
              m[k][r] = mt[k][r];
            }
#pragma unroll 1
          for (int ct = 0; ct < kCT; ++ct) {
            floatx4 acc[kTPW];
            chunk(cur, ct, acc);
#pragma unroll
            for (int k = 0; k < kTPW; ++k) {
              const bool ok = full || (jt + 16 * ct + c16 < nv[k]);
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float e = fast_exp2(fmaf(acc[k][r], a.c, -m[k][r]));
                ns[k][r] += ok ? e : 0.f;
              }
            }
          }
        }
#pragma unroll
        for (int k = 0; k < kTPW; ++k)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float sn = ns[k][r];
            if (sn > 4294967296.f) {
              const int e2 = (int)__builtin_amdgcn_logf(sn);   // log2, truncated
              ns[k][r] = ldexpf(sn, -e2);
              m[k][r] += (float)e2;
            }
          }
      }
#pragma unroll
      for (int k = 0; k < kTPW; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) ssum[k][r] = ns[k][r];
    } else if (PASS == 3) {
      // Unfused baseline: every head's probability of every visible window
      // goes to the S_C1 chunk buffer [batch][chunk_rows][h_kv][G][sc1_ld].
      float* dst[kTPW];
#pragma unroll
      for (int k = 0; k < kTPW; ++k)
        dst[k] = a.sc1 + (((int64_t)s * a.chunk_rows + (i0 - a.chunk0) + wave * kTPW + k) * a.h_kv + g) *
                             a.G * a.sc1_ld;
      walk(cur, [&](floatx4 (&acc)[kTPW], int ct) {
        const int j = jt + 16 * ct + c16;
#pragma unroll
        for (int k = 0; k < kTPW; ++k) {
          if (need[k] && j < nv[k]) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (4 * q4 + r < a.G) dst[k][(int64_t)(4 * q4 + r) * a.sc1_ld + j] = fast_exp2(fmaf(acc[k][r], a.c, -Lc[k][r]));
          }
        }
      });
    } else {
      float sct[kTPW][kCT];
      if (full) {
        walk(cur, [&](floatx4 (&acc)[kTPW], int ct) {
#pragma unroll
          for (int k = 0; k < kTPW; ++k) {
            float sum = fast_exp2(fmaf(acc[k][0], a.c, -Lc[k][0]));
#pragma unroll
            for (int r = 1; r < 4; ++r) sum += fast_exp2(fmaf(acc[k][r], a.c, -Lc[k][r]));
            sct[k][ct] = sum;
          }
        });
      } else {
        walk(cur, [&](floatx4 (&acc)[kTPW], int ct) {
#pragma unroll
          for (int k = 0; k < kTPW; ++k) {
            float sum = fast_exp2(fmaf(acc[k][0], a.c, -Lc[k][0]));
#pragma unroll
            for (int r = 1; r < 4; ++r) sum += fast_exp2(fmaf(acc[k][r], a.c, -Lc[k][r]));
            sct[k][ct] = jt + 16 * ct + c16 < nv[k] ? sum : 0.f;
          }
        });
      }
#pragma unroll
      for (int h = 0; h < kCT / 4; ++h) {
        const int jh = jt + 64 * h;
        // Block of this lane's quad, relative to the candidate range.
        const int bq = (jh >> 2) + (lane >> 2);
#pragma unroll
        for (int k = 0; k < kTPW; ++k) {
          // Reduce-scatter over the four 16-lane rows: afterwards lane l
          // holds the group sum for window jh + l.
          const float S = rs_x16(rs_x32(sct[k][4 * h], sct[k][4 * h + 2]), rs_x32(sct[k][4 * h + 1], sct[k][4 * h + 3]));
          // Quad max (windows 4b .. 4b+3) and the window before each quad
          // (4b-1; lane 0 takes the previous 64 windows' last) via DPP.  The
          // sums are non-negative floats, ordered as their bit patterns, so
          // the maxima are integer maxima.
          const int si = __float_as_int(S);
          const int q1 = max(si, __builtin_amdgcn_update_dpp(0, si, 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
          const int qm = max(q1, __builtin_amdgcn_update_dpp(0, q1, 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
          const int prev = __builtin_amdgcn_update_dpp(carry[k], si, 0x138, 0xF, 0xF, false);   // wave_shr:1
          carry[k] = __builtin_amdgcn_readlane(si, 63);
          if ((lane & 3) == 0 && bq >= a.n_init && bq <= b_hi[k])
            bs_row[k][bq] = __int_as_float(max(qm, prev));
        }
      }
    }
  }
  __syncthreads();

  if (PASS == 1) {
#pragma unroll
    for (int k = 0; k < kTPW; ++k) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float mm = m[k][r], ss = ssum[k][r];
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
          const float m2 = __shfl_xor(mm, off);
          const float s2 = __shfl_xor(ss, off);
          const float mn = fmaxf(mm, m2);
          ss = ss * fast_exp2(mm - mn) + s2 * fast_exp2(m2 - mn);
          mm = mn;
        }
        const int head = 4 * q4 + r;
        if (c16 == 0 && tval[k] && head < a.G && trow[k] < a.rows_q) {
          // m is in log2 units: L = m ln 2 + ln(sum).
          const float L = ss > 0.f ? mm * 0.6931471805599453f + logf(ss) : -__builtin_inff();
          a.lse[(int64_t)(g * a.G + head) * a.rows_q + trow[k]] = L;
        }
      }
    }
  }
}

__global__ __launch_bounds__(256, 2) void score_lse_kernel(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kWT * 256];
  score_body<1>(a, lds);
}

__global__ __launch_bounds__(256, 2) void score_blocks_kernel(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kWT * 256];
  score_body<2>(a, lds);
}

// Unfused baseline of pass 2 (the layout the fused kernel avoids): the
// per-head probabilities of one chunk of query rows reach HBM.
__global__ __launch_bounds__(256, 2) void score_probs_kernel(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kWT * 256];
  score_body<3>(a, lds);
}

// Unfused baseline, second step: one wave per (query row of the chunk, KV
// group) reads the G heads' probabilities of each candidate window from the
// chunk buffer, sums them (the group sum) and max-pools the sums into block
// scores, written in the same layout as the fused kernel's.
__global__ __launch_bounds__(256) void group_pool_kernel(ScoreArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s = blockIdx.z, g = blockIdx.y;
  const int ic = blockIdx.x * 4 + wave;              // row within the chunk
  const int i = a.chunk0 + ic;
  const SeqRange rq = seq_range(a.cu_q, a.used_q, s);
  const SeqRange rk = seq_range(a.cu_k, a.used_k, s);
  if (ic >= a.chunk_rows || i >= rq.len) return;
  const int t = rk.len - rq.len + i;
  const int64_t row = (int64_t)rq.start + i;
  if (t < 0 || row >= a.rows_q) return;
  const int bt = t / kBlock;
  if (bt - a.n_local - a.n_init + 1 <= a.n_topk) return;   // keeps every candidate
  const int nwin = rk.len >= a.win_kernel ? (rk.len - a.win_kernel) / a.win_stride + 1 : 0;
  const int nv = n_visible(t, a.win_kernel, a.win_stride, nwin);
  const int b_hi = (int)min((int64_t)(bt - a.n_local), a.bs_ld - 1);
  const float* src = a.sc1 + (((int64_t)s * a.chunk_rows + ic) * a.h_kv + g) * a.G * a.sc1_ld;
  float* bsr = a.bs + ((int64_t)g * a.rows_q + row) * a.bs_ld;
  int carry = 0;
  const int j_hi = 4 * b_hi + 4;
  for (int j0 = max(0, 4 * a.n_init - 1) & ~63; j0 < j_hi; j0 += 64) {
    const int j = j0 + lane;
    float S = 0.f;
    if (j < nv && j < a.sc1_ld)
      for (int h = 0; h < a.G; ++h) S += src[(int64_t)h * a.sc1_ld + j];
    // Non-negative sums are ordered as their bit patterns: integer maxima.
    const int si = __float_as_int(S);
    const int q1 = max(si, __builtin_amdgcn_update_dpp(0, si, 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
    const int qm = max(q1, __builtin_amdgcn_update_dpp(0, q1, 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
    const int prev = __builtin_amdgcn_update_dpp(carry, si, 0x138, 0xF, 0xF, false);    // wave_shr:1
    carry = __builtin_amdgcn_readlane(si, 63);
    const int b = (j0 >> 2) + (lane >> 2);
    if ((lane & 3) == 0 && b >= a.n_init && b <= b_hi) bsr[b] = __int_as_float(max(qm, prev));
  }
}

}  // namespace

hipError_t launch_score_lse(const ScoreArgs& a, int batch, int max_seqlen_q, hipStream_t st) {
  dim3 grid((max_seqlen_q + kQT - 1) / kQT, a.h_kv, batch);
  hipLaunchKernelGGL(score_lse_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_score_blocks(const ScoreArgs& a, int batch, int max_seqlen_q, hipStream_t st) {
  dim3 grid((max_seqlen_q + kQT - 1) / kQT, a.h_kv, batch);
  hipLaunchKernelGGL(score_blocks_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_score_unfused(const ScoreArgs& a, int batch, int max_seqlen_q, hipStream_t st) {
  for (int c0 = 0; c0 < max_seqlen_q; c0 += a.chunk_rows) {
    ScoreArgs b = a;
    b.chunk0 = c0;
    const int rows = min(a.chunk_rows, max_seqlen_q - c0);
    hipLaunchKernelGGL(score_probs_kernel, dim3((rows + kQT - 1) / kQT, a.h_kv, batch), dim3(256), 0, st, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(group_pool_kernel, dim3((rows + 3) / 4, a.h_kv, batch), dim3(256), 0, st, b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace infllmv2

// ---------------------------------------------------------------------------
// Split-K scoring.  With few query tiles (decode) a workgroup takes one query
// row, one KV group and one range of compressed keys; its waves work on
// chunks of 16 keys loaded straight into registers (the 16 heads of the group
// are the MFMA rows, 16 keys the columns).  Pass 1 keeps an exact running
// max per lane and head and writes one (max, sum) partial per range; pass 2
// merges a row's partials into its LSE and writes the block scores of its
// range, each wave walking a contiguous run of chunks so that the window
// before every quad (4b - 1) is at hand.
// ---------------------------------------------------------------------------
namespace infllmv2 {
namespace {

constexpr int kSplitScoreWaves = 4;
constexpr int kSplitDepth = 8;   // key chunks each wave keeps in flight in split pass 1
constexpr int kZDepth = 16;      // logit chunks each wave keeps in flight in split pass 2

// Row setup shared by both passes; false when the row needs no scores.
struct SplitRow {
  int s, t, bt, nv;
  int64_t c0;
};
__device__ __forceinline__ bool split_row(const ScoreArgs& a, int64_t row, SplitRow& r) {
  RowSeq rsq;
  if (!find_row_seq(a.cu_q, a.used_q, a.cu_k, a.used_k, a.cu_c, a.batch, row, rsq)) return false;
  r.s = rsq.s;
  const SeqRange rq = rsq.rq, rk = rsq.rk;
  r.t = rk.len - rq.len + (int)(row - rq.start);
  if (r.t < 0) return false;
  r.bt = r.t / kBlock;
  if (r.bt - a.n_local - a.n_init + 1 <= a.n_topk) return false;   // keeps every candidate
  const int nwin = rk.len >= a.win_kernel ? (rk.len - a.win_kernel) / a.win_stride + 1 : 0;
  r.nv = n_visible(r.t, a.win_kernel, a.win_stride, nwin);
  r.c0 = rsq.c0;
  return r.c0 >= 0 && r.c0 < a.c_rows;   // inconsistent metadata: row skipped
}

// Key fragments of the 16-key chunk j0 .. j0+15 (B operand: lane c16 holds
// key j0 + c16, dims 32 ks + 8 q4 .. +8), rows clamped to the tensor.
__device__ __forceinline__ void chunk_keys(const ScoreArgs& a, int g, int64_t c0, int j0, int c16, int q4,
                                           bf16x8 (&b)[4]) {
  int64_t rowc = c0 + j0 + c16;
  rowc = rowc < a.c_rows ? rowc : a.c_rows - 1;
  rowc = rowc > 0 ? rowc : 0;
  const uint16_t* kp = a.kc + ((int64_t)g * a.c_rows + rowc) * kHeadDim + 8 * q4;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) b[ks] = as_bf16x8(ldg16(kp + 32 * ks));
}
// S^T chunk: heads (rows) x 16 keys (columns) of one query row.
__device__ __forceinline__ floatx4 chunk_scores(const bf16x8 (&qa)[4], const bf16x8 (&b)[4]) {
  floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) acc = mfma16(qa[ks], b[ks], acc);
  return acc;
}

__device__ __forceinline__ void load_q(const ScoreArgs& a, int64_t row, int g, int c16, int q4, bf16x8 (&qa)[4]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 v = zero16();
    if (c16 < a.G) v = ldg16(a.q + (row * a.h_q + g * a.G + c16) * kHeadDim + 32 * ks + 8 * q4);
    qa[ks] = as_bf16x8(v);
  }
}

__global__ __launch_bounds__(64 * kSplitScoreWaves) void score_lse_split_kernel(ScoreArgs a) {
  __shared__ float red[kSplitScoreWaves][16][2];
  const int sp = blockIdx.x, g = blockIdx.y;
  const int64_t row = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, q4 = lane >> 4, c16 = lane & 15;
  const int wave = tid >> 6;
  bf16x8 qa[4];
  load_q(a, row, g, c16, q4, qa);   // in the same round as the row's metadata
  SplitRow r;
  if (!split_row(a, row, r)) return;
  const int nch = (r.nv + 15) >> 4;
  const int ca = (int)((int64_t)nch * sp / a.splits), cb = (int)((int64_t)nch * (sp + 1) / a.splits);
  float m[4], sm[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -__builtin_inff();
    sm[i] = 0.f;
  }
  // This wave's chunks: ca + wave, ca + wave + W, ...; DP of them in flight.
  constexpr int W = kSplitScoreWaves;
  constexpr int DP = kSplitDepth;
  bf16x8 ring[DP][4];
#pragma unroll
  for (int i = 0; i < DP; ++i)
    if (ca + wave + W * i < cb) chunk_keys(a, g, r.c0, 16 * (ca + wave + W * i), c16, q4, ring[i]);
  for (int base = ca + wave; base < cb; base += DP * W) {
#pragma unroll
    for (int i = 0; i < DP; ++i) {
      const int ch = base + W * i;
      if (ch < cb) {
        const bf16x8 b[4] = {ring[i][0], ring[i][1], ring[i][2], ring[i][3]};
        if (ch + DP * W < cb) chunk_keys(a, g, r.c0, 16 * (ch + DP * W), c16, q4, ring[i]);
        const floatx4 acc = chunk_scores(qa, b);
        const bool ok = 16 * ch + c16 < r.nv;
        if (a.zbuf != nullptr && ok && 16 * ch + c16 < a.z_ld) {
          // Exact LSE: the logits (log2 units) for the fused pass 2.
          float* zp = a.zbuf + (((int64_t)row * a.h_kv + g) * a.z_ld + 16 * ch + c16) * 16 + 4 * q4;
          *reinterpret_cast<floatx4*>(zp) = floatx4{acc[0] * a.c, acc[1] * a.c, acc[2] * a.c, acc[3] * a.c};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (ok) {
            const float mn = fmaxf(m[j], acc[j]);
            sm[j] = sm[j] * fast_exp2((m[j] - mn) * a.c) + fast_exp2((acc[j] - mn) * a.c);
            m[j] = mn;
          }
        }
      }
    }
  }
  // Combine the 16 lanes (keys) of each row group, then the waves.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float mm = m[i], ss = sm[i];
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      float m2, s2;
      if (step == 0) { m2 = dpp_f32<0xB1>(mm, mm); s2 = dpp_f32<0xB1>(ss, ss); }        // quad_perm 1,0,3,2
      else if (step == 1) { m2 = dpp_f32<0x4E>(mm, mm); s2 = dpp_f32<0x4E>(ss, ss); }   // quad_perm 2,3,0,1
      else if (step == 2) { m2 = dpp_f32<0x124>(mm, mm); s2 = dpp_f32<0x124>(ss, ss); } // row_ror:4
      else { m2 = dpp_f32<0x128>(mm, mm); s2 = dpp_f32<0x128>(ss, ss); }                // row_ror:8
      const float mn = fmaxf(mm, m2);
      ss = (mm > -__builtin_inff() ? ss * fast_exp2((mm - mn) * a.c) : 0.f) +
           (m2 > -__builtin_inff() ? s2 * fast_exp2((m2 - mn) * a.c) : 0.f);
      mm = mn;
    }
    if (c16 == 0) {
      red[wave][4 * q4 + i][0] = mm;
      red[wave][4 * q4 + i][1] = ss;
    }
  }
  __syncthreads();
  if (tid < 16) {
    float mm = red[0][tid][0], ss = red[0][tid][1];
#pragma unroll
    for (int w = 1; w < kSplitScoreWaves; ++w) {
      const float m2 = red[w][tid][0], s2 = red[w][tid][1];
      const float mn = fmaxf(mm, m2);
      ss = (mm > -__builtin_inff() ? ss * fast_exp2((mm - mn) * a.c) : 0.f) +
           (m2 > -__builtin_inff() ? s2 * fast_exp2((m2 - mn) * a.c) : 0.f);
      mm = mn;
    }
    float* dst = a.part + (((int64_t)row * a.h_kv + g) * a.splits + sp) * 32;
    dst[2 * tid] = mm;
    dst[2 * tid + 1] = ss;
  }
}

__global__ __launch_bounds__(64 * kSplitScoreWaves) void score_blocks_split_kernel(ScoreArgs a) {
  const int sp = blockIdx.x, g = blockIdx.y;
  const int64_t row = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, q4 = lane >> 4, c16 = lane & 15;
  const int wave = tid >> 6;
  SplitRow r;
  if (!split_row(a, row, r)) return;
  // Windows overlapping candidate blocks n_init .. bt - n_local: chunks of 16;
  // this wave takes a contiguous run [ca, cb) of them.
  const int b_hi = r.bt - a.n_local;
  const int cfirst = max(0, 4 * a.n_init - 1) >> 4;
  const int clast = (4 * b_hi + 3) >> 4;   // inclusive
  const int nch = clast - cfirst + 1;
  const int ca0 = cfirst + (int)((int64_t)nch * sp / a.splits);
  const int cb0 = cfirst + (int)((int64_t)nch * (sp + 1) / a.splits);
  const int ca = ca0 + (int)((int64_t)(cb0 - ca0) * wave / kSplitScoreWaves);
  const int cb = ca0 + (int)((int64_t)(cb0 - ca0) * (wave + 1) / kSplitScoreWaves);
  // Keys in flight first: the chunk before the run (its last window feeds
  // the first quad) and the first four chunks of the run.
  bf16x8 prevk[4], ring[4][4];
  if (ca < cb && ca > 0) chunk_keys(a, g, r.c0, 16 * (ca - 1), c16, q4, prevk);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (ca + i < cb) chunk_keys(a, g, r.c0, 16 * (ca + i), c16, q4, ring[i]);
  // The row's LSE partials, fetched by the whole workgroup at once.
  __shared__ float parts[kSplitMaxSplits * 32];
  {
    const float* src = a.part + ((int64_t)row * a.h_kv + g) * a.splits * 32;
    for (int i = tid; i < a.splits * 32; i += 64 * kSplitScoreWaves) parts[i] = src[i];
  }
  __syncthreads();
  if (ca >= cb) return;
  bf16x8 qa[4];
  load_q(a, row, g, c16, q4, qa);
  // LSE of the lane's four heads (log2 units, scaled).
  float Lc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * q4 + i;
    float mm = -__builtin_inff();
    for (int p = 0; p < a.splits; ++p) mm = fmaxf(mm, parts[p * 32 + 2 * h]);
    float ss = 0.f;
    for (int p = 0; p < a.splits; ++p) {
      const float m2 = parts[p * 32 + 2 * h];
      if (m2 > -__builtin_inff()) ss += parts[p * 32 + 2 * h + 1] * fast_exp2((m2 - mm) * a.c);
    }
    Lc[i] = ss > 0.f ? mm * a.c + __builtin_amdgcn_logf(ss) : __builtin_inff();
  }
  auto chunk_sum = [&](int ch, const bf16x8 (&b)[4]) -> float {
    const floatx4 acc = chunk_scores(qa, b);
    float sum = fast_exp2(fmaf(acc[0], a.c, -Lc[0]));
#pragma unroll
    for (int i = 1; i < 4; ++i) sum += fast_exp2(fmaf(acc[i], a.c, -Lc[i]));
    sum = sum_x16(sum_x32(sum));   // all heads of the group: lane c16 -> key 16 ch + c16
    return 16 * ch + c16 < r.nv ? sum : 0.f;
  };
  float carry = 0.f;
  if (ca > 0) carry = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(chunk_sum(ca - 1, prevk)), 15));
  float* bsr = a.bs + ((int64_t)g * a.rows_q + row) * a.bs_ld;
  for (int base = ca; base < cb; base += 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = base + i;
      if (ch < cb) {
        const bf16x8 b[4] = {ring[i][0], ring[i][1], ring[i][2], ring[i][3]};
        if (ch + 4 < cb) chunk_keys(a, g, r.c0, 16 * (ch + 4), c16, q4, ring[i]);   // four ahead
        const float S = chunk_sum(ch, b);
        const float q1 = fmaxf(S, dpp_f32<0xB1>(S, S));       // quad_perm 1,0,3,2
        const float qm = fmaxf(q1, dpp_f32<0x4E>(q1, q1));    // quad_perm 2,3,0,1
        const float prev = dpp_f32<0x138>(carry, S);          // wave_shr:1
        carry = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(S), 15));
        if (lane < 16 && (lane & 3) == 0) {
          const int b = 4 * ch + (lane >> 2);
          if (b >= a.n_init && b <= b_hi && b < a.bs_ld) bsr[b] = fmaxf(qm, prev);
        }
      }
    }
  }
}

// Pass 2 of the split path with the exact LSE: the same work split as
// score_blocks_split_kernel, but the logits come from pass 1's store (one
// 16-byte load per lane and window: the lane's four heads), so neither the
// stage-1 keys nor the matrix cores are needed again.
__global__ __launch_bounds__(64 * kSplitScoreWaves) void score_blocks_z_split_kernel(ScoreArgs a) {
  const int sp = blockIdx.x, g = blockIdx.y;
  const int64_t row = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, q4 = lane >> 4, c16 = lane & 15;
  const int wave = tid >> 6;
  // The row's LSE partials, fetched by the whole workgroup in the same round
  // as the row's metadata.
  __shared__ float parts[kSplitMaxSplits * 32];
  {
    const float* src = a.part + ((int64_t)row * a.h_kv + g) * a.splits * 32;
    for (int i = tid; i < a.splits * 32; i += 64 * kSplitScoreWaves) parts[i] = src[i];
  }
  SplitRow r;
  if (!split_row(a, row, r)) return;
  const int b_hi = r.bt - a.n_local;
  const int cfirst = max(0, 4 * a.n_init - 1) >> 4;
  const int clast = (4 * b_hi + 3) >> 4;   // inclusive
  const int nch = clast - cfirst + 1;
  const int ca0 = cfirst + (int)((int64_t)nch * sp / a.splits);
  const int cb0 = cfirst + (int)((int64_t)nch * (sp + 1) / a.splits);
  const int ca = ca0 + (int)((int64_t)(cb0 - ca0) * wave / kSplitScoreWaves);
  const int cb = ca0 + (int)((int64_t)(cb0 - ca0) * (wave + 1) / kSplitScoreWaves);
  // Logits of window j, heads 4 q4 .. 4 q4 + 3 (clamped into the visible
  // windows, which pass 1 wrote; the sums of windows >= nv are dropped).
  const float* zrow = a.zbuf + ((row * a.h_kv + g) * a.z_ld) * 16 + 4 * q4;
  const int jmax = max(0, min(r.nv, (int)a.z_ld) - 1);
  auto zload = [&](int ch) -> floatx4 {
    const int j = min(16 * ch + c16, jmax);
    return *reinterpret_cast<const floatx4*>(zrow + (int64_t)j * 16);
  };
  floatx4 prevz = floatx4{0.f, 0.f, 0.f, 0.f}, ring[kZDepth];
  if (ca < cb && ca > 0) prevz = zload(ca - 1);
#pragma unroll
  for (int i = 0; i < kZDepth; ++i)
    if (ca + i < cb) ring[i] = zload(ca + i);
  __syncthreads();
  if (ca >= cb) return;
  float Lc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * q4 + i;
    float mm = -__builtin_inff();
    for (int p = 0; p < a.splits; ++p) mm = fmaxf(mm, parts[p * 32 + 2 * h]);
    float ss = 0.f;
    for (int p = 0; p < a.splits; ++p) {
      const float m2 = parts[p * 32 + 2 * h];
      if (m2 > -__builtin_inff()) ss += parts[p * 32 + 2 * h + 1] * fast_exp2((m2 - mm) * a.c);
    }
    Lc[i] = (h < a.G && ss > 0.f) ? mm * a.c + __builtin_amdgcn_logf(ss) : __builtin_inff();
  }
  auto chunk_sum = [&](int ch, const floatx4& z) -> float {
    float sum = fast_exp2(z[0] - Lc[0]);
#pragma unroll
    for (int i = 1; i < 4; ++i) sum += fast_exp2(z[i] - Lc[i]);
    sum = sum_x16(sum_x32(sum));   // all heads of the group: lane c16 -> window 16 ch + c16
    return 16 * ch + c16 < r.nv ? sum : 0.f;
  };
  float carry = 0.f;
  if (ca > 0) carry = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(chunk_sum(ca - 1, prevz)), 15));
  float* bsr = a.bs + ((int64_t)g * a.rows_q + row) * a.bs_ld;
  for (int base = ca; base < cb; base += kZDepth) {
#pragma unroll
    for (int i = 0; i < kZDepth; ++i) {
      const int ch = base + i;
      if (ch < cb) {
        const floatx4 z = ring[i];
        if (ch + kZDepth < cb) ring[i] = zload(ch + kZDepth);   // kZDepth ahead
        const float S = chunk_sum(ch, z);
        const float q1 = fmaxf(S, dpp_f32<0xB1>(S, S));       // quad_perm 1,0,3,2
        const float qm = fmaxf(q1, dpp_f32<0x4E>(q1, q1));    // quad_perm 2,3,0,1
        const float prev = dpp_f32<0x138>(carry, S);          // wave_shr:1
        carry = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(S), 15));
        if (lane < 16 && (lane & 3) == 0) {
          const int b = 4 * ch + (lane >> 2);
          if (b >= a.n_init && b <= b_hi && b < a.bs_ld) bsr[b] = fmaxf(qm, prev);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_score_blocks_z_split(const ScoreArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(score_blocks_z_split_kernel, dim3(a.splits, a.h_kv, (unsigned)a.rows_q),
                     dim3(64 * kSplitScoreWaves), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_score_lse_split(const ScoreArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(score_lse_split_kernel, dim3(a.splits, a.h_kv, (unsigned)a.rows_q),
                     dim3(64 * kSplitScoreWaves), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_score_blocks_split(const ScoreArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(score_blocks_split_kernel, dim3(a.splits, a.h_kv, (unsigned)a.rows_q),
                     dim3(64 * kSplitScoreWaves), 0, st, a);
  return hipGetLastError();
}

}  // namespace infllmv2
