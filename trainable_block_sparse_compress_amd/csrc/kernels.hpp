// Kernel argument blocks and launchers of the gfx950 library.
#pragma once

#include "common.hpp"

namespace infllmv2 {

struct CompressArgs {
  const uint16_t* k;        // [rows_k, h_kv, 128]
  const int32_t* cu_k;
  const int32_t* used_k;
  int64_t rows_k;
  int h_kv;
  int kernel, stride;
  const int32_t* cu_cmp;
  const int32_t* cmp_begin;
  int max_new;
  int64_t c_rows;
  uint16_t* k_cmp;          // [h_kv, c_rows, 128]
};

struct TransposeArgs {
  const uint16_t* v;        // [rows_k, h_kv, 128]
  const int32_t* cu_k;
  const int32_t* used_k;
  int64_t rows_k;
  int h_kv, batch;
  int64_t ld;               // padded keys per sequence (multiple of 64)
  uint16_t* vt;             // [h_kv, 128, batch, ld]
};

struct ScoreArgs {
  const uint16_t* q;        // [rows_q, h_q, 128]
  const uint16_t* kc;       // [h_kv, c_rows, 128] compressed keys
  const int32_t* cu_q;
  const int32_t* used_q;
  const int32_t* cu_k;
  const int32_t* used_k;
  const int32_t* cu_c;      // first compressed row per sequence
  int64_t rows_q, c_rows;
  int h_q, h_kv, G;
  int win_kernel, win_stride;
  int n_init, n_local, n_topk;
  float scale;              // softmax scale
  float c;                  // scale * log2(e)
  float* lse;               // [h_q, rows_q], natural log
  float* bs;                // [h_kv, rows_q, bs_ld] block scores
  int64_t bs_ld;
  int batch;                // split path: sequences (row -> sequence search)
  int splits;               // split path: window ranges per (row, KV group)
  float* part;              // split path: LSE partials [rows_q, h_kv, splits, 16, 2]
  // Split path, exact LSE: pass 1 also stores every logit (scaled by c, log2
  // units) of the row's visible windows, [rows_q, h_kv, z_ld, 16] fp32, so that
  // pass 2 reads them instead of the keys.
  float* zbuf;
  int64_t z_ld;
  // Unfused baseline only: per-head probabilities of one chunk of query rows,
  // [batch, chunk_rows, h_kv, G, sc1_ld] fp32 (windows at their absolute index).
  float* sc1;
  int64_t sc1_ld;
  int chunk0, chunk_rows;
};

struct TopkArgs {
  const float* bs;          // [h_kv, rows_q, bs_ld]
  int64_t bs_ld;
  const int32_t* cu_q;
  const int32_t* used_q;
  const int32_t* cu_k;
  const int32_t* used_k;
  int64_t rows_q;
  int n_init, n_local, n_topk;
  int32_t* idx;             // [h_kv, rows_q, n_sel]
  int batch;                // row path: sequences (row -> sequence search)
};

struct AttnArgs {
  const uint16_t* q;        // [rows_q, h_q, 128]
  const uint16_t* k;        // [rows_k, h_kv, 128]
  const uint16_t* vt;       // [h_kv, 128, batch, vt_ld]
  const int32_t* cu_q;
  const int32_t* used_q;
  const int32_t* cu_k;
  const int32_t* used_k;
  int64_t rows_q, rows_k, vt_ld;
  int batch, h_q, h_kv, G;
  const int32_t* bidx;      // [h_kv, rows_q, n_sel] or nullptr (dense)
  int n_sel, n_init, n_local;
  float scale, c;
  uint16_t* out;            // [rows_q, h_q, 128]
  float* lse;               // [h_q, rows_q] or nullptr
};

// Launchers (return the launch status; no synchronisation).
hipError_t launch_compress(const CompressArgs& a, int batch, int max_windows, hipStream_t st);
hipError_t launch_transpose_v(const TransposeArgs& a, hipStream_t st);
hipError_t launch_score_lse(const ScoreArgs& a, int batch, int max_seqlen_q, hipStream_t st);
hipError_t launch_score_blocks(const ScoreArgs& a, int batch, int max_seqlen_q, hipStream_t st);
// Unfused baseline of pass 2 (the fusion ablation): per chunk of
// a.chunk_rows query rows, every head's probabilities to a.sc1, then the
// group sum and max pool from there into a.bs.
hipError_t launch_score_unfused(const ScoreArgs& a, int batch, int max_seqlen_q, hipStream_t st);
// Split-K scoring for launches with few query tiles (decode): pass 1 writes
// per-range (max, sum) partials of the LSE, pass 2 merges them and writes the
// block scores of its range.
hipError_t launch_score_lse_split(const ScoreArgs& a, hipStream_t st);
hipError_t launch_score_blocks_split(const ScoreArgs& a, hipStream_t st);
// Pass 2 of the split path with the exact LSE, from pass 1's stored logits.
hipError_t launch_score_blocks_z_split(const ScoreArgs& a, hipStream_t st);
hipError_t launch_topk(const TopkArgs& a, int batch, int h_kv, int max_seqlen_q, int max_blocks,
                       hipStream_t st);
// Top-k with a whole workgroup per (query row, KV group), for launches with
// few query rows (decode).
hipError_t launch_topk_rows(const TopkArgs& a, int h_kv, int max_blocks, hipStream_t st);
hipError_t launch_attention(const AttnArgs& a, int max_seqlen_q, hipStream_t st);

// Split-K attention for launches with few query tiles (decode): every query
// row's block set is split into `splits` ranges processed by separate
// workgroups, each writing a partial (max, sums, unnormalised output) to
// `part`; a second kernel merges the partials into out / lse.
constexpr int kSplitMaxSel = 1024;                    // list entries per row on this path
constexpr int kSplitMaxSplits = 64;                   // splits per (row, KV group)
constexpr int kPartFloats = 16 * kHeadDim + 16 + 16;   // O[16][128], l[16], m[16] per head
hipError_t launch_attention_split(const AttnArgs& a, int64_t rows_q, int splits, float* part,
                                  hipStream_t st);

// Backward of the attention (block sets held fixed).  Operands, outputs and
// the workspace buffers of the passes (see backward.hip).
constexpr int kBwdChunk = 1024;        // tokens per key-major work item
constexpr int kBwdMaxBlocks = 8192;    // blocks per sequence (LDS mask of the mask pass)

struct BwdArgs {
  const uint16_t* q;        // [rows_q, h_q, 128]
  const uint16_t* k;        // [rows_k, h_kv, 128]
  const uint16_t* v;        // [rows_k, h_kv, 128]
  const uint16_t* out;      // [rows_q, h_q, 128] forward output
  const float* lse;         // [h_q, rows_q] forward LSE (natural log)
  const uint16_t* dout;     // [rows_q, h_q, 128] upstream gradient
  const int32_t* cu_q;
  const int32_t* used_q;
  const int32_t* cu_k;
  const int32_t* used_k;
  int64_t rows_q, rows_k;
  int batch, h_q, h_kv, G;
  const int32_t* bidx;      // [h_kv, rows_q, n_sel] or nullptr (dense)
  int n_sel, n_init, n_local;
  float scale, c;           // c = scale * log2(e)
  uint16_t* dq;             // [rows_q, h_q, 128]
  uint16_t* dk;             // [rows_k, h_kv, 128]
  uint16_t* dv;
  // workspace
  float* lse2;              // [rows_q, h_kv, 16] LSE * log2(e) per padded head (+inf: no keys / pad)
  float* dd;                // [rows_q, h_kv, 16] D = dO . O per padded head
  uint16_t* qt;             // [rows_q, h_kv, 2048] Q per (row, group) in the lane order of
                            // the head-contracting MFMA operand: [c16][q4][dt][4 heads]
  uint16_t* dot;            // dO likewise
  float* part;              // [wmax, 16384] fp32 dK / dV partial sums of each work item
  uint16_t* mask_t;         // [h_kv, batch, ntiles, nblk] tokens of a 16-row tile per block
  uint16_t* mask_b;         // [h_kv, batch, nblk, ntiles] the same, block-major
  int ntiles, nblk;         // per-sequence maxima: ceil(max_q / 16), ceil(max_k / 64)
  int32_t* items;           // [h_kv, batch, nblk] work items per block
  int32_t* item_off;        // [h_kv, batch, nblk] index of each block's first item
  int32_t* work;            // [wmax, 2] (block index, item within the block)
  int32_t* nwork;           // number of work items
  int wmax;
};

hipError_t launch_attention_bwd(const BwdArgs& a, int max_seqlen_q, int max_seqlen_k, hipStream_t st);

}  // namespace infllmv2
