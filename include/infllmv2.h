/*
 * infllmv2.h — C ABI of the InfLLM-V2 sparse-attention path on MI355X (gfx950).
 *
 * The path (switch pseudocode in the reading notes "论文阅读：InfLLM-V2",
 * section "Dense-Sparse Switchable Attention"):
 *
 *   if seq_len <= threshold:  y = dense_attention(q, k, v)          -> infllmv2_dense_attn
 *   else:
 *     compressed keys (stage 1)                                    -> infllmv2_compress_k
 *     scores, group sum, max pool, init ∪ local ∪ top-k            -> infllmv2_select_blocks
 *     y = sparse attention over the selected blocks                -> infllmv2_sparse_attn
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or synchronises; it only enqueues kernels on
 *    `stream` (a hipStream_t, NULL = the null stream).  Scratch memory is a
 *    caller-provided `workspace`; passing workspace == NULL with a non-NULL
 *    `workspace_bytes` only writes the required size and returns 0 without
 *    touching the GPU.
 *  - bf16 tensors are passed as void* (bfloat16 storage, 2 bytes each).
 *  - Packed variable-length batches: sequence s's queries are rows
 *    cu_seqlens_q[s] .. cu_seqlens_q[s] + len_q(s) - 1 of q/out, its keys rows
 *    cu_seqlens_k[s] .. of k (and v).  len_q(s) = seqused_q[s] if seqused_q is
 *    not NULL, else cu_seqlens_q[s+1] - cu_seqlens_q[s]; likewise len_k(s).
 *    With seqused_* given, cu_seqlens_* needs only `batch` entries, and the
 *    sequences may be any subset of a packed buffer (this is how the
 *    dense/sparse switch hands one packed batch to both paths).
 *  - Causality is bottom-right: query i of sequence s sits at position
 *    len_k(s) - len_q(s) + i and sees keys 0 .. that position.  A decode step
 *    is the same call with len_q = 1.
 *  - Positions, blocks and compressed windows restart at each sequence.
 *  - Per-sequence metadata (cu_seqlens, seqused, cu_c*) lives on the device
 *    and is trusted: kernels clip every access to the row counts passed by
 *    value (rows_q, rows_k, c_rows), so inconsistent metadata cannot make them
 *    read or write outside the buffers, but it gives unspecified results.
 *  - Supported shapes: head_dim = 128, block_size = 64, h_q = G * h_kv with
 *    group size G in {1, 2, 4, 8, 16} (the kernels are tiled for G = 16, the
 *    GQA group size the top168.com article, section 七 "技术实现的创新细节",
 *    names as suited to block-sparse attention; smaller G is padded).
 *  - Errors: every argument is validated on the host before any HIP call.
 *    Returns INFLLMV2_OK or a negative code; infllmv2_last_error() gives a
 *    thread-local message for the last failing call on the calling thread.
 *    Calls are re-entrant; the library holds no global state besides that
 *    message.
 */
#ifndef INFLLMV2_H
#define INFLLMV2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define INFLLMV2_OK            0
#define INFLLMV2_EINVAL       (-1)  /* inconsistent or out-of-range argument */
#define INFLLMV2_EUNSUPPORTED (-2)  /* valid for the method, not implemented here */
#define INFLLMV2_EWORKSPACE   (-3)  /* workspace missing or smaller than required */
#define INFLLMV2_EHIP         (-4)  /* a HIP launch failed */

/* Static description of an error code. */
const char* infllmv2_strerror(int code);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* infllmv2_last_error(void);

/* Library version string. */
const char* infllmv2_version(void);

/*
 * infllmv2_compress_k — stage 1 of the three-stage block representation:
 * parameter-free mean pooling of the keys (top168.com article, section 三
 * "块表示的三阶段压缩": kernel l_C1 = B/2, stride s_C1 = B/4; the coarse keys of the
 * LSE approximation in section 四 use l_C2 = 4 l_C1, s_C2 = 4 s_C1).
 *
 *   k_cmp[g, cu_cmp[s] + j, :] = bf16( (1/kernel) * sum_{u < kernel} k[row(s, stride*j + u), g, :] )
 *
 * for every complete window j < N(len_k(s)) = (len_k - kernel) / stride + 1
 * (0 when len_k < kernel).  The sum is exact (float64) and rounded once to
 * bf16, to nearest even.
 *
 *   k          bf16 [rows_k, h_kv, head_dim]
 *   cu_seqlens_k, seqused_k   key rows of each sequence (seqused_k nullable)
 *   cu_cmp     int32 [batch]: first row of sequence s in k_cmp (caller computes
 *              the offsets; N() above gives each sequence's count)
 *   cmp_begin  int32 [batch] or NULL: windows j < cmp_begin[s] are left
 *              untouched (incremental use in decode: only windows completed
 *              since the last call are written)
 *   max_new    with cmp_begin: at most this many windows are written per
 *              sequence, starting at cmp_begin[s] (sizes the launch; a decode
 *              step of one token completes at most one window); ignored
 *              without cmp_begin
 *   k_cmp      bf16 [h_kv, c_rows, head_dim]  (head-major)
 *   kernel_size, stride  any positive pair; the path uses (32, 16) and (128, 64)
 */
int infllmv2_compress_k(const void* k, const int32_t* cu_seqlens_k, const int32_t* seqused_k,
                        int32_t batch, int32_t max_seqlen_k, int64_t rows_k,
                        int32_t h_kv, int32_t head_dim,
                        int32_t kernel_size, int32_t stride,
                        const int32_t* cu_cmp, const int32_t* cmp_begin, int32_t max_new,
                        int64_t c_rows, void* k_cmp, void* stream);

/*
 * infllmv2_select_blocks — block scoring and selection (top168.com article,
 * sections 三 and 四; section 七 for the union; reading notes section
 * "先看一个具体例子" for the 1 + 32 + 63 = 96-block budget of 64 tokens).
 *
 * For every query row t of KV group g:
 *   z[h, j]   = softmax_scale * q[t, h] . k_c1[g, j]           (windows visible
 *               to t: stride*j + kernel - 1 <= position)
 *   L[h]      = log sum_j exp z[h, j]   (exact: two-pass, k_c2 == NULL) or the
 *               same log-sum-exp over the coarse keys k_c2 (approximation)
 *   S[g, j]   = sum_{h in group g} exp(z[h, j] - L[h])       (group sum, fused
 *               in the score kernel; only block maxima reach memory)
 *   score[b]  = max_{j in 4b-1 .. 4b+3} S[g, j]              (max pool 5 / 4,
 *               left pad 1: the stage-1 windows overlapping block b)
 *   I(t, g)   = {0..n_init-1} ∪ {b_t-n_local+1..b_t} ∪ top-n_topk over the
 *               remaining causal blocks n_init..b_t-n_local by (score desc,
 *               block index asc); every causal block when there are no more
 *               than n_topk candidates.
 *
 *   q          bf16 [rows_q, h_q, head_dim]
 *   k_c1       bf16 [h_kv, c1_rows, head_dim] from infllmv2_compress_k(32, 16)
 *   k_c2       bf16 [h_kv, c2_rows, head_dim] from infllmv2_compress_k(128, 64),
 *              or NULL for the exact two-pass LSE
 *   cu_c1, cu_c2   int32 [batch] first compressed row per sequence (cu_c2 may
 *              be NULL iff k_c2 is NULL)
 *   block_idx  int32 [h_kv, rows_q, n_init + n_local + n_topk] (written):
 *              ascending block ids, -1 padded.  Rows of q outside every
 *              sequence are not written.
 *   workspace  >= *workspace_bytes as returned by a size query with the same
 *              shape arguments: fp32 LSE and block scores; launches with few
 *              query tiles (decode: at most 64 query rows per sequence and
 *              fewer than 512 tiles of 16 rows per KV group) add per-range
 *              LSE partials and, with the exact LSE, the logits of the first
 *              pass (64 bytes per query row, KV group and visible window)
 *              that the second pass reads back instead of the keys
 *   Supported: (c1_kernel, c1_stride) = (32, 16), (c2_kernel, c2_stride) =
 *   (128, 64), pool (5, 4, 1), n_init + n_local + n_topk >= 1 (>= 2 with
 *   k_c2, so that every row that needs scores sees a coarse window), at most
 *   8192 blocks per sequence.
 */
int infllmv2_select_blocks(const void* q, const void* k_c1, const void* k_c2,
                           const int32_t* cu_seqlens_q, const int32_t* seqused_q,
                           const int32_t* cu_seqlens_k, const int32_t* seqused_k,
                           const int32_t* cu_c1, const int32_t* cu_c2,
                           int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                           int64_t rows_q, int64_t c1_rows, int64_t c2_rows,
                           int32_t h_q, int32_t h_kv, int32_t head_dim, int32_t block_size,
                           int32_t n_init, int32_t n_local, int32_t n_topk,
                           int32_t c1_kernel, int32_t c1_stride,
                           int32_t c2_kernel, int32_t c2_stride,
                           int32_t pool_kernel, int32_t pool_stride, int32_t pool_pad,
                           float softmax_scale,
                           void* workspace, size_t* workspace_bytes,
                           int32_t* block_idx, void* stream);

/*
 * infllmv2_select_blocks_unfused — the same selection without the fused
 * group sum: the baseline of the fusion ablation (top168.com article,
 * section 四 "高效实现的技术突破": written unfused, the stage-1 scores cost
 * h_q * n^2 / s_C1 values of HBM traffic, and fusing the head-group sum
 * into the score kernel divides that by G; the hegjx.blmgzj.com repost's
 * ablation attributes part of the block-selection time to it).  Pass 2
 * writes every head's probability exp(z[h, j] - L[h]) of every visible
 * window to an fp32 buffer in HBM, in chunks of query rows; a second kernel
 * reads them back, sums each group's heads and max-pools the sums into the
 * same block scores; top-k is shared.  Same arguments, layouts, supported
 * sizes and results (up to the order of the fp32 group sum) as
 * infllmv2_select_blocks; the workspace adds the chunk buffer (at most 4 GiB:
 * batch * chunk_rows * h_q * ceil(windows / 4) * 4 floats).  Always takes
 * the tile kernels (no split-K path).  Not part of the fast path.
 */
int infllmv2_select_blocks_unfused(const void* q, const void* k_c1, const void* k_c2,
                                   const int32_t* cu_seqlens_q, const int32_t* seqused_q,
                                   const int32_t* cu_seqlens_k, const int32_t* seqused_k,
                                   const int32_t* cu_c1, const int32_t* cu_c2,
                                   int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                   int64_t rows_q, int64_t c1_rows, int64_t c2_rows,
                                   int32_t h_q, int32_t h_kv, int32_t head_dim, int32_t block_size,
                                   int32_t n_init, int32_t n_local, int32_t n_topk,
                                   int32_t c1_kernel, int32_t c1_stride,
                                   int32_t c2_kernel, int32_t c2_stride,
                                   int32_t pool_kernel, int32_t pool_stride, int32_t pool_pad,
                                   float softmax_scale,
                                   void* workspace, size_t* workspace_bytes,
                                   int32_t* block_idx, void* stream);

/*
 * infllmv2_sparse_attn — block-sparse causal attention, the single output
 * branch (reading notes section "对齐计算图"; top168.com article section 七:
 * local blocks absorb the sliding window):
 *
 *   out[t, h] = sum_{u in T} softmax_u(softmax_scale * q[t, h] . k[u, g]) v[u, g],
 *   T = {u <= position(t) : floor(u / 64) in init(t) ∪ local(t) ∪ block_idx[g, t, :]}
 *
 * with init(t) = {0..n_init-1} and local(t) = {b_t-n_local+1..b_t}.  A row
 * of block_idx is read as a set: its order does not matter, and entries
 * equal to -1, repeated, or later than b_t are skipped.  The output of
 * infllmv2_select_blocks can be passed as is, and any other block list works
 * with n_init = n_local = 0.  A row that attends no key gets out = 0 and
 * lse = -inf.
 *
 *   q, out     bf16 [rows_q, h_q, head_dim]
 *   k          bf16 [rows_k, h_kv, head_dim]
 *   v          v_seq_stride == 0: bf16 [rows_k, h_kv, head_dim] (same rows as k;
 *              the library transposes it into the workspace once per call);
 *              v_seq_stride  > 0: bf16 [h_kv, head_dim, batch, v_seq_stride]
 *              (a transposed cache: sequence s's key i at column i; the stride
 *              must be a multiple of 64; columns past len_k(s) are never used).
 *              batch x columns (v_seq_stride, or max_seqlen_k rounded up to 64)
 *              must stay below 2^27, else INFLLMV2_EUNSUPPORTED.
 *   block_idx  int32 [h_kv, rows_q, n_sel]
 *   lse_out    float [h_q, rows_q] natural-log softmax normaliser, or NULL
 *   workspace  size from a query with the same shape arguments: the
 *              transposed V (only when v_seq_stride == 0) and, for launches
 *              with few query tiles (fewer than 512 tiles of 16 rows per KV
 *              group, at most 64 query rows per sequence, at most 1024 list
 *              + init + local entries per row: decode), the split-K partials
 *              of about 8 KB per (row, KV group, split).  Zero bytes when
 *              neither applies.
 */
int infllmv2_sparse_attn(const void* q, const void* k, const void* v,
                         const int32_t* cu_seqlens_q, const int32_t* seqused_q,
                         const int32_t* cu_seqlens_k, const int32_t* seqused_k,
                         int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                         int64_t rows_q, int64_t rows_k,
                         int32_t h_q, int32_t h_kv, int32_t head_dim, int32_t block_size,
                         const int32_t* block_idx, int32_t n_sel, int32_t n_init, int32_t n_local,
                         float softmax_scale, int64_t v_seq_stride,
                         void* out, float* lse_out,
                         void* workspace, size_t* workspace_bytes, void* stream);

/*
 * infllmv2_sparse_attn_noalloc — infllmv2_sparse_attn for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, layouts, kernels and
 * results as infllmv2_sparse_attn, without the workspace: the scratch that
 * call would take from the workspace (the transposed V when v_seq_stride ==
 * 0; the split-K partials of launches with few query tiles, i.e. decode)
 * lives in a static device array of 64 MiB (67108864 bytes) that every GPU
 * the library runs on holds until the process ends.  A call whose scratch
 * would exceed it returns INFLLMV2_EUNSUPPORTED (message in
 * infllmv2_last_error) before any HIP call; e.g. the transposed V of one
 * 131072-token sequence with 2 KV heads is exactly 64 MiB, and decode at
 * batch 16 with a 128K cache needs 4.3 MB of partials.  The function
 * allocates, frees and synchronises nothing; the first call on a device
 * looks up that device's copy of the array (hipGetSymbolAddress).  Calls on
 * one GPU share its array and keep the previous call's contents: calls
 * that overlap on one GPU (different streams, or host threads) race and
 * must be ordered by the caller.  The scratch needs no clearing (every
 * element a kernel reads was written by the same call).
 */
int infllmv2_sparse_attn_noalloc(const void* q, const void* k, const void* v,
                                 const int32_t* cu_seqlens_q, const int32_t* seqused_q,
                                 const int32_t* cu_seqlens_k, const int32_t* seqused_k,
                                 int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                 int64_t rows_q, int64_t rows_k,
                                 int32_t h_q, int32_t h_kv, int32_t head_dim, int32_t block_size,
                                 const int32_t* block_idx, int32_t n_sel, int32_t n_init, int32_t n_local,
                                 float softmax_scale, int64_t v_seq_stride,
                                 void* out, float* lse_out, void* stream);

/*
 * infllmv2_dense_attn — plain causal attention over every key <= position,
 * the path short sequences take (reading notes section "Dense-Sparse
 * Switchable Attention"; dtcms.com article section 二.2.c: dense below a
 * length threshold).  Same layouts, v conventions and workspace rule as
 * infllmv2_sparse_attn.
 */
int infllmv2_dense_attn(const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_q, const int32_t* seqused_q,
                        const int32_t* cu_seqlens_k, const int32_t* seqused_k,
                        int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                        int64_t rows_q, int64_t rows_k,
                        int32_t h_q, int32_t h_kv, int32_t head_dim,
                        float softmax_scale, int64_t v_seq_stride,
                        void* out, float* lse_out,
                        void* workspace, size_t* workspace_bytes, void* stream);

/*
 * infllmv2_sparse_attn_bwd — gradients of infllmv2_sparse_attn (block_idx
 * given) or infllmv2_dense_attn (block_idx NULL) with the block sets held
 * fixed.  The method is trained through its sparse attention (reading notes
 * "论文阅读：InfLLM-V2", section "训练是怎么做的": long-context fine-tuning
 * with the plain next-token objective); the top-k selection is piecewise
 * constant in q and k, so no gradient flows into the scoring path.  With
 * P[t, h, u] the forward's probabilities over the same key sets T:
 *
 *   D[t, h]   = sum_d dout[t, h, d] * out[t, h, d]
 *   dS[t,h,u] = P[t, h, u] * (dout[t, h] . v[u, g] - D[t, h])
 *   dq[t, h]  = softmax_scale * sum_u dS[t, h, u] k[u, g]
 *   dk[u, g]  = softmax_scale * sum_{t, h in g} dS[t, h, u] q[t, h]
 *   dv[u, g]  = sum_{t, h in g} P[t, h, u] dout[t, h]
 *
 * P is recomputed from q, k and the forward's lse (lse_out of the forward
 * call, natural log).  Block lists are read exactly as the forward reads
 * them (a set per row; -1, repeats and blocks later than b_t skipped).
 *
 *   q, out, dout   bf16 [rows_q, h_q, head_dim]  (out, lse: the forward's)
 *   lse            float [h_q, rows_q]
 *   k, v           bf16 [rows_k, h_kv, head_dim]  (v in its natural layout)
 *   block_idx      int32 [h_kv, rows_q, n_sel], or NULL for dense causal
 *   dq             bf16 [rows_q, h_q, head_dim]: rows of every sequence written
 *   dk, dv         bf16 [rows_k, h_kv, head_dim]: rows of every sequence
 *                  written (zero for keys no query attends)
 *   workspace      size from a query with the same shape arguments (and the
 *                  same n_sel / n_init / n_local, or block_idx NULL): per
 *                  query row and KV group 8 KB (Q and dO re-laid out) plus
 *                  128 B of statistics; two 16-bit token-mask tables of
 *                  h_kv * batch * ceil(max_q/16) * ceil(max_k/64) entries;
 *                  64 KB of fp32 dK / dV partial sums per work item, where
 *                  every (KV group, block) with attending rows has
 *                  ceil(rows / 1024) items (bounded on the host by
 *                  h_kv * rows_q * min(n_sel + n_init + n_local, blocks) /
 *                  1024 + h_kv * batch * blocks + 1; about 1.9 GB for one
 *                  131072-token sequence at |I| = 96).
 *   Supported: head_dim 128, block_size 64, group size 1, 2, 4, 8 or 16, at
 *   most 8192 blocks per sequence and 65535 tiles of 16 query rows.  The
 *   results are deterministic (fixed summation order).
 */
int infllmv2_sparse_attn_bwd(const void* q, const void* k, const void* v,
                             const void* out, const float* lse, const void* dout,
                             const int32_t* cu_seqlens_q, const int32_t* seqused_q,
                             const int32_t* cu_seqlens_k, const int32_t* seqused_k,
                             int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                             int64_t rows_q, int64_t rows_k,
                             int32_t h_q, int32_t h_kv, int32_t head_dim, int32_t block_size,
                             const int32_t* block_idx, int32_t n_sel, int32_t n_init,
                             int32_t n_local, float softmax_scale,
                             void* dq, void* dk, void* dv,
                             void* workspace, size_t* workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* INFLLMV2_H */
