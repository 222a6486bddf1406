// Host side of the C ABI declared in include/infllmv2.h: argument validation
// (all of it before any HIP call), workspace sizing and kernel launches.  The
// library never allocates or synchronises.
#include <stdarg.h>
#include <stdio.h>

#include <cmath>
#include <mutex>
#include <string>

#include "infllmv2.h"
#include "kernels.hpp"

using namespace infllmv2;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return INFLLMV2_OK;
}

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(INFLLMV2_EHIP, "%s: %s", what, hipGetErrorString(e));
  return INFLLMV2_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
int64_t ceil_div(int64_t x, int64_t m) { return (x + m - 1) / m; }

bool group_ok(int G) { return G == 1 || G == 2 || G == 4 || G == 8 || G == 16; }

constexpr int kMaxBlocks = 8192;      // per sequence (top-k keeps <= 128 keys per lane)
constexpr int kMaxGrid = 65535;
// batch x columns of one transposed-V row: 16 such rows of bf16 stay under
// 4 GiB, the reach of the attention kernel's 32-bit offsets.
constexpr int64_t kMaxVtRow = (int64_t)1 << 27;

// Workspace of the scoring path: fp32 LSE [h_q, rows_q] + fp32 block scores
// [h_kv, rows_q, bs_ld].
// Launches with few query tiles (decode) split every row's compressed keys
// over several workgroups; pass 1 then leaves (max, sum) partials instead of
// the LSE.
struct SelectLayout {
  int64_t bs_ld;
  int splits;                 // 0: tile kernels
  size_t lse_bytes, bs_bytes, part_bytes, total;
  // Unfused baseline: per-head probabilities of chunk_rows query rows of
  // every sequence, fp32 [batch, chunk_rows, h_q, sc1_ld].
  int64_t sc1_ld = 0;
  int chunk_rows = 0;
  size_t sc1_bytes = 0;
  // Split path with the exact LSE: pass 1's stored logits, fp32
  // [rows_q, h_kv, z_ld, 16], read back by pass 2.
  int64_t z_ld = 0;
  size_t z_bytes = 0;
};
constexpr size_t kUnfusedChunkBytes = size_t(4) << 30;   // bound of the chunk buffer
// Workgroups the split scoring path aims for (measured best at batch 16:
// 512 costs 7% more, 128 costs 20% more).
constexpr int64_t kSelectTargetWgs = 256;
int select_splits(int64_t rows_q, int batch, int max_seqlen_q, int max_seqlen_k, int h_kv) {
  const int64_t tiles = ceil_div(std::max(1, max_seqlen_q), 16) * h_kv * std::max(1, batch);
  if (tiles >= 512 || max_seqlen_q > 64 || rows_q > kMaxGrid || rows_q < 1) return 0;
  const int64_t want = ceil_div(kSelectTargetWgs, rows_q * h_kv);
  const int64_t cap = std::max<int64_t>(1, ceil_div(std::max(1, max_seqlen_k), 16) / 64);   // >= 64 keys each
  return (int)std::max<int64_t>(1, std::min<int64_t>({want, cap, (int64_t)64}));
}
SelectLayout select_layout(int64_t rows_q, int batch, int max_seqlen_q, int h_q, int h_kv,
                           int max_seqlen_k, bool unfused, bool approx) {
  SelectLayout L;
  L.bs_ld = round_up(std::max<int64_t>(1, ceil_div(max_seqlen_k, kBlock)), 4);
  L.splits = unfused ? 0 : select_splits(rows_q, batch, max_seqlen_q, max_seqlen_k, h_kv);
  L.lse_bytes = align_up((size_t)h_q * (size_t)rows_q * sizeof(float));
  L.bs_bytes = align_up((size_t)h_kv * (size_t)rows_q * (size_t)L.bs_ld * sizeof(float));
  L.part_bytes = L.splits > 0 ? align_up((size_t)rows_q * h_kv * L.splits * 32 * sizeof(float)) : 0;
  if (unfused) {
    const int64_t nwin = max_seqlen_k >= 32 ? (max_seqlen_k - 32) / 16 + 1 : 1;
    L.sc1_ld = round_up(nwin, 4);
    const size_t per_row = (size_t)std::max(1, batch) * h_q * (size_t)L.sc1_ld * sizeof(float);
    const int64_t fit = std::max<int64_t>(16, (int64_t)(kUnfusedChunkBytes / per_row) / 16 * 16);
    L.chunk_rows = (int)std::min<int64_t>(fit, round_up(std::max(1, max_seqlen_q), 16));
    L.sc1_bytes = align_up(per_row * (size_t)L.chunk_rows);
  }
  if (L.splits > 0 && !approx) {
    L.z_ld = round_up(std::max<int64_t>(1, max_seqlen_k >= 32 ? (max_seqlen_k - 32) / 16 + 1 : 1), 16);
    L.z_bytes = align_up((size_t)rows_q * h_kv * (size_t)L.z_ld * 16 * sizeof(float));
  }
  L.total = L.lse_bytes + L.bs_bytes + L.part_bytes + L.sc1_bytes + L.z_bytes;
  return L;
}

// Workspace of the attention path: V transposed to [h_kv, 128, batch, ld].
size_t vt_bytes(int h_kv, int batch, int max_seqlen_k) {
  const int64_t ld = round_up(std::max(1, max_seqlen_k), kBlock);
  return align_up((size_t)h_kv * kHeadDim * (size_t)batch * (size_t)ld * 2);
}

// Launches with fewer query tiles than this take the split-K path.
constexpr int64_t kSplitTileLimit = 512;
constexpr int kSplitTargetWgs = 256;   // measured best at batch 16 (512: +3%, 128: +12%)

// Split count of the split-K attention path, or 0 for the tile kernel.
int attn_splits(int64_t rows_q, int batch, int max_seqlen_q, int max_seqlen_k, int h_kv, bool dense,
                int n_sel, int n_init, int n_local) {
  const int64_t tiles = ceil_div(std::max(1, max_seqlen_q), 16) * h_kv * std::max(1, batch);
  if (tiles >= kSplitTileLimit || max_seqlen_q > 64 || rows_q > kMaxGrid || rows_q < 1) return 0;
  if (!dense && (int64_t)n_sel + n_init + n_local > kSplitMaxSel) return 0;
  if (ceil_div(std::max(1, max_seqlen_k), kBlock) > 65536) return 0;   // block bitmap of the split path
  const int64_t blocks = dense ? ceil_div(std::max(1, max_seqlen_k), kBlock)
                               : std::min<int64_t>((int64_t)n_sel + n_init + n_local,
                                                   ceil_div(std::max(1, max_seqlen_k), kBlock));
  const int64_t want = ceil_div(kSplitTargetWgs, rows_q * h_kv);
  const int64_t cap = std::max<int64_t>(1, blocks / 4);   // at least one block per wave
  return (int)std::max<int64_t>(1, std::min<int64_t>({want, cap, (int64_t)kSplitMaxSplits}));
}

int workspace_check(void* ws, size_t* bytes, size_t need, bool* query) {
  *query = false;
  if (ws == nullptr && bytes != nullptr) {
    *bytes = need;
    *query = true;
    return ok();
  }
  if (need > 0) {
    REQUIRE(ws != nullptr, INFLLMV2_EWORKSPACE, "workspace of %zu bytes required", need);
    REQUIRE(bytes != nullptr && *bytes >= need, INFLLMV2_EWORKSPACE,
            "workspace too small: %zu < %zu bytes", bytes ? *bytes : (size_t)0, need);
  }
  return INFLLMV2_OK;
}

int common_seq_checks(int batch, int max_seqlen_q, int max_seqlen_k, int64_t rows_q, int64_t rows_k) {
  REQUIRE(batch >= 0 && batch <= kMaxGrid, INFLLMV2_EINVAL, "batch %d out of range [0, %d]", batch, kMaxGrid);
  REQUIRE(max_seqlen_q >= 0 && max_seqlen_k >= 0, INFLLMV2_EINVAL, "negative max sequence length");
  REQUIRE(max_seqlen_q <= max_seqlen_k, INFLLMV2_EINVAL,
          "max_seqlen_q %d > max_seqlen_k %d (queries are the last positions of their sequence)",
          max_seqlen_q, max_seqlen_k);
  REQUIRE(rows_q >= 0 && rows_k >= 0, INFLLMV2_EINVAL, "negative row count");
  return INFLLMV2_OK;
}

// Scratch of infllmv2_sparse_attn_noalloc: one file-scope device array per
// GPU the library runs on (held until the process ends).  Host code never
// passes the array's name to a kernel: it uses the device address that
// hipGetSymbolAddress returns, fetched once per device (with that device
// current) on the entry point's first call there.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(INFLLMV2_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  REQUIRE(dev >= 0 && dev < kMaxDevices, INFLLMV2_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(INFLLMV2_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return INFLLMV2_OK;
}

int attn_common(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                const int32_t* seqused_q, const int32_t* cu_seqlens_k, const int32_t* seqused_k,
                int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k, int64_t rows_q,
                int64_t rows_k, int32_t h_q, int32_t h_kv, int32_t head_dim, const int32_t* block_idx,
                int32_t n_sel, int32_t n_init, int32_t n_local, float softmax_scale,
                int64_t v_seq_stride, void* out, float* lse_out, void* workspace,
                size_t* workspace_bytes, void* stream, bool dense, bool noalloc = false) {
  int rc = common_seq_checks(batch, max_seqlen_q, max_seqlen_k, rows_q, rows_k);
  if (rc) return rc;
  REQUIRE(head_dim == kHeadDim, INFLLMV2_EUNSUPPORTED, "head_dim %d unsupported (128 only)", head_dim);
  REQUIRE(h_kv >= 1 && h_q >= 1 && h_q % h_kv == 0, INFLLMV2_EINVAL, "h_q %d not a multiple of h_kv %d", h_q, h_kv);
  REQUIRE(h_kv <= kMaxGrid, INFLLMV2_EINVAL, "h_kv too large");
  REQUIRE(group_ok(h_q / h_kv), INFLLMV2_EUNSUPPORTED, "group size %d unsupported (1, 2, 4, 8, 16)", h_q / h_kv);
  REQUIRE(std::isfinite(softmax_scale) && softmax_scale > 0.f, INFLLMV2_EINVAL, "softmax_scale must be finite and > 0");
  if (!dense) {
    REQUIRE(n_sel >= 1, INFLLMV2_EINVAL, "n_sel must be >= 1");
    REQUIRE(n_init >= 0 && n_local >= 0, INFLLMV2_EINVAL, "n_init and n_local must be >= 0");
  }
  REQUIRE(v_seq_stride >= 0, INFLLMV2_EINVAL, "negative v_seq_stride");
  if (v_seq_stride > 0) {
    REQUIRE(v_seq_stride % kBlock == 0, INFLLMV2_EINVAL, "v_seq_stride must be a multiple of 64");
    REQUIRE(v_seq_stride >= round_up(max_seqlen_k, kBlock), INFLLMV2_EINVAL,
            "v_seq_stride %lld < max_seqlen_k rounded to 64", (long long)v_seq_stride);
  }
  // The tile kernel addresses 16 rows of the transposed V (head-dim rows of
  // batch x columns each) with 32-bit offsets from one base.
  const int64_t vt_cols = v_seq_stride > 0 ? v_seq_stride : round_up(std::max(1, max_seqlen_k), kBlock);
  REQUIRE((int64_t)batch * vt_cols < kMaxVtRow, INFLLMV2_EUNSUPPORTED,
          "batch x transposed-V columns %lld reaches the limit of %lld",
          (long long)((int64_t)batch * vt_cols), (long long)kMaxVtRow);
  const int splits = attn_splits(rows_q, batch, max_seqlen_q, max_seqlen_k, h_kv, dense, n_sel,
                                 n_init, n_local);
  const size_t vt_need = v_seq_stride > 0 ? 0 : vt_bytes(h_kv, batch, max_seqlen_k);
  const size_t part_need =
      splits > 0 ? align_up((size_t)rows_q * h_kv * splits * kPartFloats * sizeof(float)) : 0;
  const size_t need = vt_need + part_need;
  if (noalloc) {
    REQUIRE(need <= kNoallocScratchBytes, INFLLMV2_EUNSUPPORTED,
            "needs %zu bytes of scratch (transposed V %zu, split-K partials %zu), above the static "
            "maximum of %zu bytes", need, vt_need, part_need, kNoallocScratchBytes);
  } else {
    bool query = false;
    rc = workspace_check(workspace, workspace_bytes, need, &query);
    if (rc || query) return rc;
  }
  if (batch == 0 || max_seqlen_q == 0) return ok();
  REQUIRE(rows_q >= 1 && rows_k >= 1, INFLLMV2_EINVAL, "rows_q and rows_k must be >= 1");
  REQUIRE(q && k && v && out && cu_seqlens_q && cu_seqlens_k, INFLLMV2_EINVAL, "null tensor pointer");
  REQUIRE(dense || block_idx, INFLLMV2_EINVAL, "null block_idx");
  if (noalloc && need > 0) {
    rc = scratch_address(&workspace);
    if (rc) return rc;
  }
  (void)seqused_q;
  (void)seqused_k;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint16_t* vt = reinterpret_cast<const uint16_t*>(v);
  int64_t vt_ld = v_seq_stride;
  if (v_seq_stride == 0) {
    vt_ld = round_up(std::max(1, max_seqlen_k), kBlock);
    REQUIRE(vt_ld / kBlock <= kMaxGrid, INFLLMV2_EUNSUPPORTED, "sequence too long");
    TransposeArgs t;
    t.v = reinterpret_cast<const uint16_t*>(v);
    t.cu_k = cu_seqlens_k;
    t.used_k = seqused_k;
    t.rows_k = rows_k;
    t.h_kv = h_kv;
    t.batch = batch;
    t.ld = vt_ld;
    t.vt = reinterpret_cast<uint16_t*>(workspace);
    rc = hip_status(launch_transpose_v(t, st), "transpose_v launch");
    if (rc) return rc;
    vt = t.vt;
  }
  AttnArgs a;
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.k = reinterpret_cast<const uint16_t*>(k);
  a.vt = vt;
  a.cu_q = cu_seqlens_q;
  a.used_q = seqused_q;
  a.cu_k = cu_seqlens_k;
  a.used_k = seqused_k;
  a.rows_q = rows_q;
  a.rows_k = rows_k;
  a.vt_ld = vt_ld;
  a.batch = batch;
  a.h_q = h_q;
  a.h_kv = h_kv;
  a.G = h_q / h_kv;
  a.bidx = dense ? nullptr : block_idx;
  a.n_sel = dense ? 0 : n_sel;
  a.n_init = dense ? 0 : n_init;
  a.n_local = dense ? 0 : n_local;
  a.scale = softmax_scale;
  a.c = softmax_scale * 1.4426950408889634f;
  a.out = reinterpret_cast<uint16_t*>(out);
  a.lse = lse_out;
  if (splits > 0) {
    float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + vt_need);
    rc = hip_status(launch_attention_split(a, rows_q, splits, part, st), "split attention launch");
  } else {
    rc = hip_status(launch_attention(a, max_seqlen_q, st), "attention launch");
  }
  if (rc) return rc;
  return ok();
}

// Workspace of the backward: offsets of its buffers.
struct BwdLayout {
  int64_t ntiles, nblk, wmax;
  size_t lse2, dd, qt, dot, part, mask_t, mask_b, items, item_off, work, nwork, total;
};
BwdLayout bwd_layout(int64_t rows_q, int64_t rows_k, int batch, int max_seqlen_q, int max_seqlen_k,
                     int h_kv, bool dense, int n_sel, int n_init, int n_local) {
  BwdLayout L;
  L.ntiles = std::max<int64_t>(1, ceil_div(max_seqlen_q, 16));
  L.nblk = std::max<int64_t>(1, ceil_div(max_seqlen_k, kBlock));
  const int64_t per_row = dense ? L.nblk : std::min<int64_t>(L.nblk, (int64_t)n_sel + n_init + n_local);
  // Every work item but the last of a block holds kBwdChunk tokens.
  const int64_t nb = (int64_t)h_kv * batch * L.nblk;
  L.wmax = ceil_div((int64_t)h_kv * rows_q * per_row, kBwdChunk) + nb + 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  L.lse2 = take((size_t)rows_q * h_kv * 16 * sizeof(float));
  L.dd = take((size_t)rows_q * h_kv * 16 * sizeof(float));
  L.qt = take((size_t)rows_q * h_kv * kHeadDim * 16 * 2);
  L.dot = take((size_t)rows_q * h_kv * kHeadDim * 16 * 2);
  L.part = take((size_t)L.wmax * 16384 * sizeof(float));
  L.mask_t = take((size_t)nb * L.ntiles * 2);
  L.mask_b = take((size_t)nb * L.ntiles * 2);
  L.items = take((size_t)nb * sizeof(int32_t));
  L.item_off = take((size_t)nb * sizeof(int32_t));
  L.work = take((size_t)L.wmax * 2 * sizeof(int32_t));
  L.nwork = take(sizeof(int32_t));
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

const char* infllmv2_strerror(int code) {
  switch (code) {
    case INFLLMV2_OK: return "ok";
    case INFLLMV2_EINVAL: return "invalid argument";
    case INFLLMV2_EUNSUPPORTED: return "unsupported configuration";
    case INFLLMV2_EWORKSPACE: return "workspace missing or too small";
    case INFLLMV2_EHIP: return "HIP launch failed";
    default: return "unknown error";
  }
}

const char* infllmv2_last_error(void) { return g_last_error.c_str(); }

const char* infllmv2_version(void) { return "infllmv2-gfx950 0.1.0"; }

int infllmv2_compress_k(const void* k, const int32_t* cu_seqlens_k, const int32_t* seqused_k,
                        int32_t batch, int32_t max_seqlen_k, int64_t rows_k, int32_t h_kv,
                        int32_t head_dim, int32_t kernel_size, int32_t stride,
                        const int32_t* cu_cmp, const int32_t* cmp_begin, int32_t max_new,
                        int64_t c_rows, void* k_cmp, void* stream) {
  REQUIRE(batch >= 0 && batch <= kMaxGrid, INFLLMV2_EINVAL, "batch %d out of range", batch);
  REQUIRE(max_seqlen_k >= 0 && rows_k >= 0 && c_rows >= 0, INFLLMV2_EINVAL, "negative size");
  REQUIRE(head_dim == kHeadDim, INFLLMV2_EUNSUPPORTED, "head_dim %d unsupported (128 only)", head_dim);
  REQUIRE(h_kv >= 1 && h_kv <= kMaxGrid, INFLLMV2_EINVAL, "h_kv %d out of range", h_kv);
  REQUIRE(kernel_size >= 1 && stride >= 1 && kernel_size <= 4096, INFLLMV2_EINVAL,
          "kernel_size %d / stride %d out of range", kernel_size, stride);
  REQUIRE(cmp_begin == nullptr || max_new >= 1, INFLLMV2_EINVAL, "max_new must be >= 1 with cmp_begin");
  const int64_t nw = max_seqlen_k >= kernel_size ? (max_seqlen_k - kernel_size) / stride + 1 : 0;
  const int64_t windows = cmp_begin ? std::min<int64_t>(max_new, nw) : nw;
  if (batch == 0 || windows == 0) return ok();
  REQUIRE(k && cu_seqlens_k && cu_cmp && k_cmp, INFLLMV2_EINVAL, "null pointer");
  const int64_t threads = windows * 16;
  REQUIRE(ceil_div(threads, 256) <= 0x7FFFFFFF, INFLLMV2_EUNSUPPORTED, "too many windows");
  CompressArgs a;
  a.k = reinterpret_cast<const uint16_t*>(k);
  a.cu_k = cu_seqlens_k;
  a.used_k = seqused_k;
  a.rows_k = rows_k;
  a.h_kv = h_kv;
  a.kernel = kernel_size;
  a.stride = stride;
  a.cu_cmp = cu_cmp;
  a.cmp_begin = cmp_begin;
  a.max_new = cmp_begin ? max_new : 0;
  a.c_rows = c_rows;
  a.k_cmp = reinterpret_cast<uint16_t*>(k_cmp);
  int rc = hip_status(launch_compress(a, batch, (int)windows, reinterpret_cast<hipStream_t>(stream)),
                      "compress_k launch");
  if (rc) return rc;
  return ok();
}

}  // extern "C"

namespace {

int select_common(const void* q, const void* k_c1, const void* k_c2,
                  const int32_t* cu_seqlens_q, const int32_t* seqused_q,
                  const int32_t* cu_seqlens_k, const int32_t* seqused_k,
                  const int32_t* cu_c1, const int32_t* cu_c2, int32_t batch,
                  int32_t max_seqlen_q, int32_t max_seqlen_k, int64_t rows_q,
                  int64_t c1_rows, int64_t c2_rows, int32_t h_q, int32_t h_kv,
                  int32_t head_dim, int32_t block_size, int32_t n_init, int32_t n_local,
                  int32_t n_topk, int32_t c1_kernel, int32_t c1_stride, int32_t c2_kernel,
                  int32_t c2_stride, int32_t pool_kernel, int32_t pool_stride,
                  int32_t pool_pad, float softmax_scale, void* workspace,
                  size_t* workspace_bytes, int32_t* block_idx, void* stream, bool unfused) {
  int rc = common_seq_checks(batch, max_seqlen_q, max_seqlen_k, rows_q, 0);
  if (rc) return rc;
  REQUIRE(c1_rows >= 0 && c2_rows >= 0, INFLLMV2_EINVAL, "negative compressed row count");
  REQUIRE(head_dim == kHeadDim, INFLLMV2_EUNSUPPORTED, "head_dim %d unsupported (128 only)", head_dim);
  REQUIRE(block_size == kBlock, INFLLMV2_EUNSUPPORTED, "block_size %d unsupported (64 only)", block_size);
  REQUIRE(h_kv >= 1 && h_q >= 1 && h_q % h_kv == 0, INFLLMV2_EINVAL, "h_q %d not a multiple of h_kv %d", h_q, h_kv);
  REQUIRE(h_kv <= kMaxGrid, INFLLMV2_EINVAL, "h_kv too large");
  REQUIRE(group_ok(h_q / h_kv), INFLLMV2_EUNSUPPORTED, "group size %d unsupported (1, 2, 4, 8, 16)", h_q / h_kv);
  REQUIRE(n_init >= 0 && n_local >= 0 && n_topk >= 0, INFLLMV2_EINVAL, "negative block count");
  REQUIRE(n_init + n_local + n_topk >= 1, INFLLMV2_EINVAL, "n_init + n_local + n_topk must be >= 1");
  REQUIRE(c1_kernel == 32 && c1_stride == 16, INFLLMV2_EUNSUPPORTED,
          "stage-1 compression (%d, %d) unsupported: (32, 16) = (B/2, B/4)", c1_kernel, c1_stride);
  REQUIRE(pool_kernel == 5 && pool_stride == 4 && pool_pad == 1, INFLLMV2_EUNSUPPORTED,
          "max pool (%d, %d, pad %d) unsupported: (5, 4, pad 1)", pool_kernel, pool_stride, pool_pad);
  const bool approx = k_c2 != nullptr;
  if (approx) {
    REQUIRE(c2_kernel == 128 && c2_stride == 64, INFLLMV2_EUNSUPPORTED,
            "coarse compression (%d, %d) unsupported: (128, 64) = 4x stage 1", c2_kernel, c2_stride);
    REQUIRE((n_init + n_local + n_topk) * block_size >= c2_kernel, INFLLMV2_EINVAL,
            "LSE approximation needs (n_init + n_local + n_topk) * 64 >= 128");
  }
  REQUIRE(std::isfinite(softmax_scale) && softmax_scale > 0.f, INFLLMV2_EINVAL, "softmax_scale must be finite and > 0");
  REQUIRE(ceil_div(max_seqlen_k, kBlock) <= kMaxBlocks, INFLLMV2_EUNSUPPORTED,
          "more than %d blocks per sequence", kMaxBlocks);
  const SelectLayout L = select_layout(rows_q, batch, max_seqlen_q, h_q, h_kv, max_seqlen_k, unfused, approx);
  bool query = false;
  rc = workspace_check(workspace, workspace_bytes, L.total, &query);
  if (rc || query) return rc;
  if (batch == 0 || max_seqlen_q == 0) return ok();
  REQUIRE(q && k_c1 && cu_seqlens_q && cu_seqlens_k && cu_c1 && block_idx, INFLLMV2_EINVAL, "null pointer");
  REQUIRE(!approx || cu_c2, INFLLMV2_EINVAL, "cu_c2 required with k_c2");
  REQUIRE(rows_q >= 1 && c1_rows >= 1 && (!approx || c2_rows >= 1), INFLLMV2_EINVAL,
          "rows_q and the compressed row counts must be >= 1");

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  ScoreArgs sa;
  sa.q = reinterpret_cast<const uint16_t*>(q);
  sa.cu_q = cu_seqlens_q;
  sa.used_q = seqused_q;
  sa.cu_k = cu_seqlens_k;
  sa.used_k = seqused_k;
  sa.rows_q = rows_q;
  sa.h_q = h_q;
  sa.h_kv = h_kv;
  sa.G = h_q / h_kv;
  sa.n_init = n_init;
  sa.n_local = n_local;
  sa.n_topk = n_topk;
  sa.scale = softmax_scale;
  sa.c = softmax_scale * 1.4426950408889634f;
  sa.lse = reinterpret_cast<float*>(ws);
  sa.bs = reinterpret_cast<float*>(ws + L.lse_bytes);
  sa.bs_ld = L.bs_ld;
  sa.batch = batch;
  sa.splits = L.splits;
  sa.part = L.splits > 0 ? reinterpret_cast<float*>(ws + L.lse_bytes + L.bs_bytes) : nullptr;
  sa.sc1 = unfused ? reinterpret_cast<float*>(ws + L.lse_bytes + L.bs_bytes + L.part_bytes) : nullptr;
  sa.sc1_ld = L.sc1_ld;
  sa.chunk0 = 0;
  sa.chunk_rows = L.chunk_rows;
  sa.zbuf = L.z_bytes > 0 ? reinterpret_cast<float*>(ws + L.lse_bytes + L.bs_bytes + L.part_bytes + L.sc1_bytes)
                          : nullptr;
  sa.z_ld = L.z_ld;

  // Pass 1: exact LSE over the stage-1 keys, or the approximation over the
  // coarse keys.
  ScoreArgs p1 = sa;
  p1.kc = reinterpret_cast<const uint16_t*>(approx ? k_c2 : k_c1);
  p1.cu_c = approx ? cu_c2 : cu_c1;
  p1.c_rows = approx ? c2_rows : c1_rows;
  p1.win_kernel = approx ? c2_kernel : c1_kernel;
  p1.win_stride = approx ? c2_stride : c1_stride;
  rc = hip_status(L.splits > 0 ? launch_score_lse_split(p1, st) : launch_score_lse(p1, batch, max_seqlen_q, st),
                  "score_lse launch");
  if (rc) return rc;

  // Pass 2: probabilities, group sum and max pool -> block scores, then the
  // top-k.
  TopkArgs ta;
  ta.bs = sa.bs;
  ta.bs_ld = L.bs_ld;
  ta.cu_q = cu_seqlens_q;
  ta.used_q = seqused_q;
  ta.cu_k = cu_seqlens_k;
  ta.used_k = seqused_k;
  ta.rows_q = rows_q;
  ta.n_init = n_init;
  ta.n_local = n_local;
  ta.n_topk = n_topk;
  ta.idx = block_idx;
  ta.batch = batch;
  const int max_blocks = (int)ceil_div(max_seqlen_k, kBlock);
  ScoreArgs p2 = sa;
  p2.kc = reinterpret_cast<const uint16_t*>(k_c1);
  p2.cu_c = cu_c1;
  p2.c_rows = c1_rows;
  p2.win_kernel = c1_kernel;
  p2.win_stride = c1_stride;
  rc = hip_status(unfused ? launch_score_unfused(p2, batch, max_seqlen_q, st)
                  : L.z_bytes > 0 ? launch_score_blocks_z_split(p2, st)
                  : L.splits > 0 ? launch_score_blocks_split(p2, st)
                                 : launch_score_blocks(p2, batch, max_seqlen_q, st),
                  "score_blocks launch");
  if (rc) return rc;
  rc = hip_status(L.splits > 0 ? launch_topk_rows(ta, h_kv, max_blocks, st)
                               : launch_topk(ta, batch, h_kv, max_seqlen_q, max_blocks, st),
                  "topk launch");
  if (rc) return rc;
  return ok();
}

}  // namespace

extern "C" {

int infllmv2_select_blocks(const void* q, const void* k_c1, const void* k_c2,
                           const int32_t* cu_seqlens_q, const int32_t* seqused_q,
                           const int32_t* cu_seqlens_k, const int32_t* seqused_k,
                           const int32_t* cu_c1, const int32_t* cu_c2, int32_t batch,
                           int32_t max_seqlen_q, int32_t max_seqlen_k, int64_t rows_q,
                           int64_t c1_rows, int64_t c2_rows, int32_t h_q, int32_t h_kv,
                           int32_t head_dim, int32_t block_size, int32_t n_init, int32_t n_local,
                           int32_t n_topk, int32_t c1_kernel, int32_t c1_stride, int32_t c2_kernel,
                           int32_t c2_stride, int32_t pool_kernel, int32_t pool_stride,
                           int32_t pool_pad, float softmax_scale, void* workspace,
                           size_t* workspace_bytes, int32_t* block_idx, void* stream) {
  return select_common(q, k_c1, k_c2, cu_seqlens_q, seqused_q, cu_seqlens_k, seqused_k, cu_c1, cu_c2,
                       batch, max_seqlen_q, max_seqlen_k, rows_q, c1_rows, c2_rows, h_q, h_kv,
                       head_dim, block_size, n_init, n_local, n_topk, c1_kernel, c1_stride,
                       c2_kernel, c2_stride, pool_kernel, pool_stride, pool_pad, softmax_scale,
                       workspace, workspace_bytes, block_idx, stream, false);
}

int infllmv2_select_blocks_unfused(const void* q, const void* k_c1, const void* k_c2,
                                   const int32_t* cu_seqlens_q, const int32_t* seqused_q,
                                   const int32_t* cu_seqlens_k, const int32_t* seqused_k,
                                   const int32_t* cu_c1, const int32_t* cu_c2, int32_t batch,
                                   int32_t max_seqlen_q, int32_t max_seqlen_k, int64_t rows_q,
                                   int64_t c1_rows, int64_t c2_rows, int32_t h_q, int32_t h_kv,
                                   int32_t head_dim, int32_t block_size, int32_t n_init,
                                   int32_t n_local, int32_t n_topk, int32_t c1_kernel,
                                   int32_t c1_stride, int32_t c2_kernel, int32_t c2_stride,
                                   int32_t pool_kernel, int32_t pool_stride, int32_t pool_pad,
                                   float softmax_scale, void* workspace, size_t* workspace_bytes,
                                   int32_t* block_idx, void* stream) {
  return select_common(q, k_c1, k_c2, cu_seqlens_q, seqused_q, cu_seqlens_k, seqused_k, cu_c1, cu_c2,
                       batch, max_seqlen_q, max_seqlen_k, rows_q, c1_rows, c2_rows, h_q, h_kv,
                       head_dim, block_size, n_init, n_local, n_topk, c1_kernel, c1_stride,
                       c2_kernel, c2_stride, pool_kernel, pool_stride, pool_pad, softmax_scale,
                       workspace, workspace_bytes, block_idx, stream, true);
}

int infllmv2_sparse_attn(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                         const int32_t* seqused_q, const int32_t* cu_seqlens_k,
                         const int32_t* seqused_k, int32_t batch, int32_t max_seqlen_q,
                         int32_t max_seqlen_k, int64_t rows_q, int64_t rows_k, int32_t h_q,
                         int32_t h_kv, int32_t head_dim, int32_t block_size,
                         const int32_t* block_idx, int32_t n_sel, int32_t n_init, int32_t n_local,
                         float softmax_scale, int64_t v_seq_stride, void* out, float* lse_out,
                         void* workspace, size_t* workspace_bytes, void* stream) {
  REQUIRE(block_size == kBlock, INFLLMV2_EUNSUPPORTED, "block_size %d unsupported (64 only)", block_size);
  return attn_common(q, k, v, cu_seqlens_q, seqused_q, cu_seqlens_k, seqused_k, batch, max_seqlen_q,
                     max_seqlen_k, rows_q, rows_k, h_q, h_kv, head_dim, block_idx, n_sel, n_init,
                     n_local, softmax_scale, v_seq_stride, out, lse_out, workspace, workspace_bytes,
                     stream, false);
}

int infllmv2_sparse_attn_noalloc(const void* q, const void* k, const void* v,
                                 const int32_t* cu_seqlens_q, const int32_t* seqused_q,
                                 const int32_t* cu_seqlens_k, const int32_t* seqused_k,
                                 int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                 int64_t rows_q, int64_t rows_k, int32_t h_q, int32_t h_kv,
                                 int32_t head_dim, int32_t block_size, const int32_t* block_idx,
                                 int32_t n_sel, int32_t n_init, int32_t n_local,
                                 float softmax_scale, int64_t v_seq_stride, void* out,
                                 float* lse_out, void* stream) {
  REQUIRE(block_size == kBlock, INFLLMV2_EUNSUPPORTED, "block_size %d unsupported (64 only)", block_size);
  return attn_common(q, k, v, cu_seqlens_q, seqused_q, cu_seqlens_k, seqused_k, batch, max_seqlen_q,
                     max_seqlen_k, rows_q, rows_k, h_q, h_kv, head_dim, block_idx, n_sel, n_init,
                     n_local, softmax_scale, v_seq_stride, out, lse_out, nullptr, nullptr, stream,
                     false, true);
}

int infllmv2_dense_attn(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                        const int32_t* seqused_q, const int32_t* cu_seqlens_k,
                        const int32_t* seqused_k, int32_t batch, int32_t max_seqlen_q,
                        int32_t max_seqlen_k, int64_t rows_q, int64_t rows_k, int32_t h_q,
                        int32_t h_kv, int32_t head_dim, float softmax_scale, int64_t v_seq_stride,
                        void* out, float* lse_out, void* workspace, size_t* workspace_bytes,
                        void* stream) {
  return attn_common(q, k, v, cu_seqlens_q, seqused_q, cu_seqlens_k, seqused_k, batch, max_seqlen_q,
                     max_seqlen_k, rows_q, rows_k, h_q, h_kv, head_dim, nullptr, 0, 0, 0,
                     softmax_scale, v_seq_stride, out, lse_out, workspace, workspace_bytes, stream,
                     true);
}

}  // extern "C"

extern "C" int infllmv2_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                                        const float* lse, const void* dout,
                                        const int32_t* cu_seqlens_q, const int32_t* seqused_q,
                                        const int32_t* cu_seqlens_k, const int32_t* seqused_k,
                                        int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                        int64_t rows_q, int64_t rows_k, int32_t h_q, int32_t h_kv,
                                        int32_t head_dim, int32_t block_size,
                                        const int32_t* block_idx, int32_t n_sel, int32_t n_init,
                                        int32_t n_local, float softmax_scale, void* dq, void* dk,
                                        void* dv, void* workspace, size_t* workspace_bytes,
                                        void* stream) {
  const bool dense = block_idx == nullptr;
  int rc = common_seq_checks(batch, max_seqlen_q, max_seqlen_k, rows_q, rows_k);
  if (rc) return rc;
  REQUIRE(head_dim == kHeadDim, INFLLMV2_EUNSUPPORTED, "head_dim %d unsupported (128 only)", head_dim);
  REQUIRE(block_size == kBlock, INFLLMV2_EUNSUPPORTED, "block_size %d unsupported (64 only)", block_size);
  REQUIRE(h_kv >= 1 && h_q >= 1 && h_q % h_kv == 0, INFLLMV2_EINVAL, "h_q %d not a multiple of h_kv %d", h_q, h_kv);
  REQUIRE(h_kv <= kMaxGrid, INFLLMV2_EINVAL, "h_kv too large");
  REQUIRE(group_ok(h_q / h_kv), INFLLMV2_EUNSUPPORTED, "group size %d unsupported (1, 2, 4, 8, 16)", h_q / h_kv);
  REQUIRE(std::isfinite(softmax_scale) && softmax_scale > 0.f, INFLLMV2_EINVAL, "softmax_scale must be finite and > 0");
  if (!dense) {
    REQUIRE(n_sel >= 1, INFLLMV2_EINVAL, "n_sel must be >= 1");
    REQUIRE(n_init >= 0 && n_local >= 0, INFLLMV2_EINVAL, "n_init and n_local must be >= 0");
  }
  REQUIRE(ceil_div(max_seqlen_k, kBlock) <= kBwdMaxBlocks, INFLLMV2_EUNSUPPORTED,
          "more than %d blocks per sequence", kBwdMaxBlocks);
  REQUIRE(ceil_div(max_seqlen_q, 16) <= kMaxGrid, INFLLMV2_EUNSUPPORTED, "too many query rows per sequence");
  REQUIRE((int64_t)h_kv * batch <= kMaxGrid, INFLLMV2_EUNSUPPORTED, "h_kv * batch above %d", kMaxGrid);
  REQUIRE((int64_t)h_kv * batch * ceil_div(std::max(1, max_seqlen_k), kBlock) <= 0x7FFFFFFF,
          INFLLMV2_EUNSUPPORTED, "too many blocks");
  REQUIRE(ceil_div(rows_q, 4) <= 0x7FFFFFFF, INFLLMV2_EUNSUPPORTED, "too many query rows");
  const BwdLayout L = bwd_layout(rows_q, rows_k, batch, max_seqlen_q, max_seqlen_k, h_kv, dense,
                                 n_sel, n_init, n_local);
  REQUIRE(L.wmax <= 0x7FFFFFFF, INFLLMV2_EUNSUPPORTED, "too many work items");
  bool query = false;
  rc = workspace_check(workspace, workspace_bytes, L.total, &query);
  if (rc || query) return rc;
  if (batch == 0 || max_seqlen_q == 0) return ok();
  REQUIRE(rows_q >= 1 && rows_k >= 1, INFLLMV2_EINVAL, "rows_q and rows_k must be >= 1");
  REQUIRE(q && k && v && out && lse && dout && dq && dk && dv && cu_seqlens_q && cu_seqlens_k,
          INFLLMV2_EINVAL, "null pointer");

  char* ws = reinterpret_cast<char*>(workspace);
  BwdArgs a;
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.k = reinterpret_cast<const uint16_t*>(k);
  a.v = reinterpret_cast<const uint16_t*>(v);
  a.out = reinterpret_cast<const uint16_t*>(out);
  a.lse = lse;
  a.dout = reinterpret_cast<const uint16_t*>(dout);
  a.cu_q = cu_seqlens_q;
  a.used_q = seqused_q;
  a.cu_k = cu_seqlens_k;
  a.used_k = seqused_k;
  a.rows_q = rows_q;
  a.rows_k = rows_k;
  a.batch = batch;
  a.h_q = h_q;
  a.h_kv = h_kv;
  a.G = h_q / h_kv;
  a.bidx = dense ? nullptr : block_idx;
  a.n_sel = dense ? 0 : n_sel;
  a.n_init = dense ? 0 : n_init;
  a.n_local = dense ? 0 : n_local;
  a.scale = softmax_scale;
  a.c = softmax_scale * 1.4426950408889634f;
  a.dq = reinterpret_cast<uint16_t*>(dq);
  a.dk = reinterpret_cast<uint16_t*>(dk);
  a.dv = reinterpret_cast<uint16_t*>(dv);
  a.lse2 = reinterpret_cast<float*>(ws + L.lse2);
  a.dd = reinterpret_cast<float*>(ws + L.dd);
  a.qt = reinterpret_cast<uint16_t*>(ws + L.qt);
  a.dot = reinterpret_cast<uint16_t*>(ws + L.dot);
  a.part = reinterpret_cast<float*>(ws + L.part);
  a.mask_t = reinterpret_cast<uint16_t*>(ws + L.mask_t);
  a.mask_b = reinterpret_cast<uint16_t*>(ws + L.mask_b);
  a.ntiles = (int)L.ntiles;
  a.nblk = (int)L.nblk;
  a.items = reinterpret_cast<int32_t*>(ws + L.items);
  a.item_off = reinterpret_cast<int32_t*>(ws + L.item_off);
  a.work = reinterpret_cast<int32_t*>(ws + L.work);
  a.nwork = reinterpret_cast<int32_t*>(ws + L.nwork);
  a.wmax = (int)L.wmax;
  rc = hip_status(launch_attention_bwd(a, max_seqlen_q, max_seqlen_k, reinterpret_cast<hipStream_t>(stream)),
                  "attention backward launch");
  if (rc) return rc;
  return ok();
}
