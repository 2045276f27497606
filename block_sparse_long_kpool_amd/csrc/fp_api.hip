// C ABI of the library: argument validation, size queries, workspace layout
// and kernel launches.  Nothing here allocates device memory or synchronises.
#include <math.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>

#include "fp_internal.hpp"

using namespace fp;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Validate the descriptor and fill the launch geometry.
int make_geometry(const fp_problem* p, Geometry* g) {
  if (!p) return fail(FP_ERR_INVALID, "problem descriptor is NULL");
  if (p->num_seqs < 1) return fail(FP_ERR_INVALID, "num_seqs must be >= 1 (got %d)", p->num_seqs);
  if (!p->cu_seqlens_host || !p->cu_seqlens_dev)
    return fail(FP_ERR_INVALID, "cu_seqlens_host and cu_seqlens_dev must be non-NULL");
  if (p->head_dim != kHeadDim) return fail(FP_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", p->head_dim);
  if (p->block_size != kBlock) return fail(FP_ERR_UNSUPPORTED, "block_size must be 128 (got %d)", p->block_size);
  if (p->num_kv_heads < 1 || p->num_q_heads < 1 || p->num_q_heads % p->num_kv_heads)
    return fail(FP_ERR_INVALID, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                p->num_q_heads, p->num_kv_heads);
  if (p->num_q_heads / p->num_kv_heads > 16)
    return fail(FP_ERR_UNSUPPORTED, "GQA group size %d > 16", p->num_q_heads / p->num_kv_heads);
  const int P = p->page_size;
  if (P < 1 || !((kBlock % P == 0) || (P % kBlock == 0)))
    return fail(FP_ERR_UNSUPPORTED, "page_size %d must divide 128 or be a multiple of 128", P);
  if (!p->page_table_dev) return fail(FP_ERR_INVALID, "page_table_dev is NULL");
  if (p->num_pages < 1) return fail(FP_ERR_INVALID, "num_pages must be >= 1");
  const int qk = p->qk_dtype, vd = p->v_dtype, od = p->out_dtype;
  const bool combo = (qk == FP_BF16 && vd == FP_BF16) || (qk == FP_E4M3 && vd == FP_BF16) ||
                     (qk == FP_F32 && vd == FP_F32);
  if (!combo) return fail(FP_ERR_UNSUPPORTED, "dtype combination qk=%d v=%d not supported", qk, vd);
  if (od != FP_F32 && od != FP_BF16) return fail(FP_ERR_UNSUPPORTED, "out_dtype %d not supported", od);
  if (qk == FP_E4M3 && (!p->q_scale_dev || !p->k_scale_dev))
    return fail(FP_ERR_INVALID, "e4m3 inputs need q_scale_dev and k_scale_dev");
  const int32_t* cu = p->cu_seqlens_host;
  if (cu[0] != 0) return fail(FP_ERR_INVALID, "cu_seqlens[0] must be 0");
  if ((p->ctx_lens_host == nullptr) != (p->ctx_lens_dev == nullptr))
    return fail(FP_ERR_INVALID, "ctx_lens_host and ctx_lens_dev must both be set or both be NULL");
  int64_t nblk = 0, nqblk = 0, causal = 0;
  int maxn = 0, maxlen = 0;
  for (int s = 0; s < p->num_seqs; ++s) {
    const int qlen = cu[s + 1] - cu[s];
    if (qlen < 0) return fail(FP_ERR_INVALID, "cu_seqlens must be nondecreasing (seq %d)", s);
    const int c = p->ctx_lens_host ? p->ctx_lens_host[s] : 0;
    if (c < 0 || c % kBlock)
      return fail(FP_ERR_INVALID, "ctx_lens[%d] = %d must be a nonnegative multiple of 128", s, c);
    if ((int64_t)c + qlen > (int64_t)kMaxBlocksPerSeq * kBlock)
      return fail(FP_ERR_UNSUPPORTED, "sequence %d of %lld tokens exceeds the %d-block limit", s,
                  (long long)c + qlen, kMaxBlocksPerSeq);
    const int len = c + qlen;
    const int n = (len + kBlock - 1) / kBlock;
    nblk += n;
    nqblk += n - c / kBlock;
    const int64_t i0 = c / kBlock;  // first query block
    causal += (int64_t)n * (n + 1) / 2 - i0 * (i0 + 1) / 2;
    maxn = std::max(maxn, n);
    maxlen = std::max(maxlen, len);
  }
  if (nqblk < 1) return fail(FP_ERR_INVALID, "batch has no query tokens");
  if (maxn > kMaxBlocksPerSeq)
    return fail(FP_ERR_UNSUPPORTED, "sequence of %d blocks exceeds the %d-block limit", maxn, kMaxBlocksPerSeq);
  if ((int64_t)p->max_pages_per_seq * P < maxlen)
    return fail(FP_ERR_INVALID, "max_pages_per_seq * page_size (%lld) < longest sequence (%d)",
                (long long)p->max_pages_per_seq * P, maxlen);
  g->num_seqs = p->num_seqs;
  g->hq = p->num_q_heads;
  g->hkv = p->num_kv_heads;
  g->group = p->num_q_heads / p->num_kv_heads;
  g->page_size = P;
  g->max_pages = p->max_pages_per_seq;
  g->num_blocks = nblk;
  g->num_qblocks = nqblk;
  g->max_blocks = maxn;
  if (p->head_lists != 0 && p->head_lists != 1)
    return fail(FP_ERR_INVALID, "head_lists must be 0 or 1 (got %d)", p->head_lists);
  g->lists = p->head_lists ? p->num_q_heads : p->num_kv_heads;
  g->lgroup = p->head_lists ? 1 : p->num_q_heads / p->num_kv_heads;
  g->kvdiv = p->head_lists ? p->num_q_heads / p->num_kv_heads : 1;
  g->num_rows = nqblk * g->lists;
  // row_ptr and col_idx offsets are int32: the list of every causal block
  // (the capacity col_idx must have) has to fit
  g->csr_capacity = causal * g->lists;
  if (g->csr_capacity > (int64_t)INT32_MAX)
    return fail(FP_ERR_UNSUPPORTED, "index lists of %lld entries (every causal block) exceed the "
                "int32 offsets of row_ptr", (long long)g->csr_capacity);
  g->total_tokens = cu[p->num_seqs];
  g->qk_dtype = qk;
  g->v_dtype = vd;
  g->out_dtype = od;
  g->softmax_scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / sqrtf((float)kHeadDim);
  g->softmax_scale_d = p->softmax_scale > 0.f ? (double)p->softmax_scale : 1.0 / sqrt((double)kHeadDim);
  if (p->attn_splits < 0) return fail(FP_ERR_INVALID, "attn_splits must be >= 0 (got %d)", p->attn_splits);
  g->attn_splits = p->attn_splits;
  return FP_OK;
}

// The dense baseline has no index lists: the g query heads of a KV head
// always share its tiles, whatever head_lists says.
void dense_geometry(Geometry* g) {
  g->lists = g->hkv;
  g->lgroup = g->group;
  g->kvdiv = 1;
  g->num_rows = g->num_qblocks * g->lists;
}

struct DiscoverWs { int32_t* kboff; int32_t* qboff; u16* km16; float* kres; float* bnorm; };
struct SelectWs { int32_t* kboff; int32_t* qboff; uint32_t* bits; int32_t* counts; };
struct AttnWs { int32_t* kboff; int32_t* qboff; u16* km16; u16* vm16; float* opart; float* lpart; int* queue; };

SeqMap seq_map(const fp_problem* p, int32_t* kboff, int32_t* qboff) {
  SeqMap m;
  m.cu = p->cu_seqlens_dev;
  m.ctx = p->ctx_lens_dev;
  m.kboff = kboff;
  m.qboff = qboff;
  m.num_seqs = p->num_seqs;
  return m;
}

size_t ws_layout(const Geometry& g, int which, void* base, void* out) {
  char* b = reinterpret_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    void* ptr = b ? b + off : nullptr;
    off = align_up(off + bytes);
    return ptr;
  };
  const size_t boff_bytes = sizeof(int32_t) * (size_t)(g.num_seqs + 1);
  const size_t pooled16 = sizeof(u16) * (size_t)g.hkv * (size_t)g.num_blocks * kHeadDim;
  if (which == FP_WS_DISCOVER) {
    DiscoverWs w;
    w.kboff = (int32_t*)take(boff_bytes);
    w.qboff = (int32_t*)take(boff_bytes);
    w.km16 = (u16*)take(pooled16);  // kbar rounded to bf16
    w.kres = (float*)take(sizeof(float) * (size_t)g.hkv * (size_t)g.num_blocks);
    w.bnorm = (float*)take(sizeof(float) * (size_t)g.hkv * (size_t)g.num_blocks);  // |bf16 kbar|
    if (out) *reinterpret_cast<DiscoverWs*>(out) = w;
  } else if (which == FP_WS_SELECT) {
    SelectWs w;
    const size_t words = (size_t)(g.max_blocks + 31) / 32;
    w.kboff = (int32_t*)take(boff_bytes);
    w.qboff = (int32_t*)take(boff_bytes);
    w.bits = (uint32_t*)take(sizeof(uint32_t) * words * (size_t)g.num_rows);
    w.counts = (int32_t*)take(sizeof(int32_t) * (size_t)g.num_rows);
    if (out) *reinterpret_cast<SelectWs*>(out) = w;
  } else if (which == FP_WS_ATTN) {
    AttnWs w;
    w.kboff = (int32_t*)take(boff_bytes);
    w.qboff = (int32_t*)take(boff_bytes);
    w.km16 = (u16*)take(pooled16);
    w.vm16 = (u16*)take(pooled16);
    w.queue = (int*)take(sizeof(int));  // item counter of the attention kernel
    w.opart = w.lpart = nullptr;
    const int splits = attn_splits(g);
    if (splits > 1) {  // partial outputs and lse of the KV-split parts
      const size_t rows = (size_t)splits * (size_t)g.total_tokens * (size_t)g.hq;
      w.opart = (float*)take(sizeof(float) * rows * kHeadDim);
      w.lpart = (float*)take(sizeof(float) * rows);
    }
    if (out) *reinterpret_cast<AttnWs*>(out) = w;
  } else {
    return 0;
  }
  return off;
}

int check_ws(const Geometry& g, int which, void* ws, size_t ws_bytes) {
  const size_t need = ws_layout(g, which, nullptr, nullptr);
  if (!ws) return fail(FP_ERR_INVALID, "workspace pointer is NULL");
  if (ws_bytes < need)
    return fail(FP_ERR_WORKSPACE, "workspace of %zu bytes < required %zu", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign)
    return fail(FP_ERR_INVALID, "workspace must be %zu-byte aligned", kAlign);
  return FP_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FP_OK;
  return fail(FP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int64_t fp_num_blocks(const fp_problem* p) {
  Geometry g;
  return make_geometry(p, &g) == FP_OK ? g.num_blocks : -1;
}

int64_t fp_num_query_blocks(const fp_problem* p) {
  Geometry g;
  return make_geometry(p, &g) == FP_OK ? g.num_qblocks : -1;
}

int32_t fp_max_blocks(const fp_problem* p) {
  Geometry g;
  return make_geometry(p, &g) == FP_OK ? g.max_blocks : -1;
}

int64_t fp_num_rows(const fp_problem* p) {
  Geometry g;
  return make_geometry(p, &g) == FP_OK ? g.num_rows : -1;
}

int64_t fp_scores_elems(const fp_problem* p) {
  Geometry g;
  // the scores, then one error bound per score row
  return make_geometry(p, &g) == FP_OK ? g.num_rows * ((int64_t)g.max_blocks + 1) : -1;
}

int64_t fp_csr_capacity(const fp_problem* p) {
  Geometry g;
  return make_geometry(p, &g) == FP_OK ? g.csr_capacity : -1;
}

size_t fp_workspace_bytes(const fp_problem* p, int32_t which) {
  Geometry g;
  if (make_geometry(p, &g) != FP_OK) return 0;
  if (which == FP_WS_DENSE) {
    dense_geometry(&g);
    which = FP_WS_ATTN;  // same layout (the pooled copies go unused)
  }
  return ws_layout(g, which, nullptr, nullptr);
}

const char* fp_status_string(int32_t status) {
  switch (status) {
    case FP_OK: return "ok";
    case FP_ERR_INVALID: return "invalid argument";
    case FP_ERR_UNSUPPORTED: return "unsupported configuration";
    case FP_ERR_WORKSPACE: return "workspace too small";
    case FP_ERR_CAPACITY: return "col_idx capacity too small";
    case FP_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* fp_last_error(void) { return g_err; }

int fp_discover(const fp_problem* p, const void* q, const void* k_cache, const void* v_cache,
                double* k_mean, double* v_mean, float* block_scores, void* ws, size_t ws_bytes,
                void* stream) {
  Geometry g;
  int st = make_geometry(p, &g);
  if (st) return st;
  if (!q || !k_cache || !v_cache || !k_mean || !v_mean || !block_scores)
    return fail(FP_ERR_INVALID, "fp_discover: a tensor pointer is NULL");
  if ((st = check_ws(g, FP_WS_DISCOVER, ws, ws_bytes))) return st;
  DiscoverWs w;
  ws_layout(g, FP_WS_DISCOVER, ws, &w);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const SeqMap m = seq_map(p, w.kboff, w.qboff);
  if ((st = hip_status(launch_plan(m, s), "plan"))) return st;
  // the discovery copy of the key means is pre-scaled to log2-domain logits
  const double lscale = g.softmax_scale_d * 1.4426950408889634074;  // log2(e)
  if ((st = hip_status(launch_pool(g, m, p->page_table_dev, k_cache, v_cache, p->k_scale_dev,
                                   lscale, k_mean, v_mean, w.km16, w.kres, w.bnorm, s), "pool")))
    return st;
  return hip_status(launch_scores(g, m, q, p->q_scale_dev, w.km16, w.kres, w.bnorm, block_scores, s),
                    "scores");
}

int fp_select(const fp_problem* p, const void* q, const double* k_mean, const float* block_scores,
              float alpha, int32_t sink_tokens, int32_t local_tokens, int32_t* row_ptr,
              int32_t* col_idx, int64_t col_capacity, void* ws, size_t ws_bytes, void* stream) {
  Geometry g;
  int st = make_geometry(p, &g);
  if (st) return st;
  if (!q || !k_mean || !block_scores || !row_ptr || !col_idx)
    return fail(FP_ERR_INVALID, "fp_select: a tensor pointer is NULL");
  if (sink_tokens < 0 || local_tokens < 0)
    return fail(FP_ERR_INVALID, "sink_tokens and local_tokens must be >= 0");
  if (isnan(alpha)) return fail(FP_ERR_INVALID, "alpha is NaN");
  const int64_t cap = g.csr_capacity;
  if (col_capacity < cap)
    return fail(FP_ERR_CAPACITY, "col_capacity %lld < %lld (every causal block kept)",
                (long long)col_capacity, (long long)cap);
  if ((st = check_ws(g, FP_WS_SELECT, ws, ws_bytes))) return st;
  SelectWs w;
  ws_layout(g, FP_WS_SELECT, ws, &w);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int n_sink = (sink_tokens + kBlock - 1) / kBlock;
  const int n_local = std::max(1, (local_tokens + kBlock - 1) / kBlock);
  const SeqMap m = seq_map(p, w.kboff, w.qboff);
  if ((st = hip_status(launch_plan(m, s), "plan"))) return st;
  return hip_status(launch_select(g, m, q, p->q_scale_dev, k_mean, block_scores, alpha, n_sink,
                                  n_local, w.bits, w.counts, row_ptr, col_idx, s),
                    "select");
}

// ---- fp_select_noalloc: fp_select with its workspace in a static device
// array, for callers that cannot allocate device memory -------------------

namespace {

// Scratch of fp_select_noalloc: one copy per device (the code object's
// device globals are instantiated on every device that loads the library)
// until the process ends.  Holds the select workspace: block offsets, the
// keep bitmask (4 bytes per 32 blocks per CSR row) and the row counts.
constexpr size_t kSelectScratchBytes = size_t(8) << 20;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kSelectScratchBytes];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; host code never uses the
// array's own name as an address (that is a host-side stand-in).
constexpr int kMaxDevices = 64;
std::atomic<uintptr_t> g_scratch_addr[kMaxDevices];

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FP_ERR_UNSUPPORTED, "fp_select_noalloc: device %d beyond the %d devices it tracks", dev,
                kMaxDevices);
  uintptr_t v = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!v) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(FP_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    v = reinterpret_cast<uintptr_t>(ptr);
    g_scratch_addr[dev].store(v, std::memory_order_release);  // racing threads store the same value
  }
  *out = reinterpret_cast<void*>(v);
  return FP_OK;
}

}  // namespace

int fp_select_noalloc(const fp_problem* p, const void* q, const double* k_mean,
                      const float* block_scores, float alpha, int32_t sink_tokens,
                      int32_t local_tokens, int32_t* row_ptr, int32_t* col_idx,
                      int64_t col_capacity, void* stream) {
  Geometry g;
  int st = make_geometry(p, &g);
  if (st) return st;
  const size_t need = ws_layout(g, FP_WS_SELECT, nullptr, nullptr);
  if (need > kSelectScratchBytes)
    return fail(FP_ERR_WORKSPACE,
                "fp_select_noalloc: this batch needs %zu bytes of select workspace, the static "
                "scratch holds %zu (call fp_select with a workspace instead)",
                need, kSelectScratchBytes);
  if (!q || !k_mean || !block_scores || !row_ptr || !col_idx)
    return fail(FP_ERR_INVALID, "fp_select_noalloc: a tensor pointer is NULL");
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  // the select kernels write every word of the workspace they read (block
  // offsets, each row's bitmask words and count), so nothing is cleared
  return fp_select(p, q, k_mean, block_scores, alpha, sink_tokens, local_tokens, row_ptr, col_idx,
                   col_capacity, ws, kSelectScratchBytes, stream);
}

namespace {
int select_ranked(const fp_problem* p, const float* block_scores, int mode, int32_t top_k, float top_p,
                  int32_t sink_tokens, int32_t local_tokens, int32_t* row_ptr, int32_t* col_idx,
                  int64_t col_capacity, void* ws, size_t ws_bytes, void* stream) {
  Geometry g;
  int st = make_geometry(p, &g);
  if (st) return st;
  if (!block_scores || !row_ptr || !col_idx) return fail(FP_ERR_INVALID, "fp_select_top%c: a tensor pointer is NULL", mode ? 'p' : 'k');
  if (sink_tokens < 0 || local_tokens < 0)
    return fail(FP_ERR_INVALID, "sink_tokens and local_tokens must be >= 0");
  if (mode == 0 && top_k < 0) return fail(FP_ERR_INVALID, "top_k must be >= 0 (got %d)", top_k);
  if (mode == 1 && !(top_p == top_p)) return fail(FP_ERR_INVALID, "top_p is NaN");
  const int64_t cap = g.csr_capacity;
  if (col_capacity < cap)
    return fail(FP_ERR_CAPACITY, "col_capacity %lld < %lld (every causal block kept)",
                (long long)col_capacity, (long long)cap);
  if ((st = check_ws(g, FP_WS_SELECT, ws, ws_bytes))) return st;
  SelectWs w;
  ws_layout(g, FP_WS_SELECT, ws, &w);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int n_sink = (sink_tokens + kBlock - 1) / kBlock;
  const int n_local = std::max(1, (local_tokens + kBlock - 1) / kBlock);
  const SeqMap m = seq_map(p, w.kboff, w.qboff);
  if ((st = hip_status(launch_plan(m, s), "plan"))) return st;
  return hip_status(launch_select_ranked(g, m, block_scores, mode, top_k, top_p, n_sink, n_local, w.bits,
                                         w.counts, row_ptr, col_idx, s),
                    "ranked select");
}
}  // namespace

int fp_select_topk(const fp_problem* p, const float* block_scores, int32_t top_k, int32_t sink_tokens,
                   int32_t local_tokens, int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                   void* ws, size_t ws_bytes, void* stream) {
  return select_ranked(p, block_scores, 0, top_k, 0.f, sink_tokens, local_tokens, row_ptr, col_idx,
                       col_capacity, ws, ws_bytes, stream);
}

int fp_select_topp(const fp_problem* p, const float* block_scores, float top_p, int32_t sink_tokens,
                   int32_t local_tokens, int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                   void* ws, size_t ws_bytes, void* stream) {
  return select_ranked(p, block_scores, 1, 0, top_p, sink_tokens, local_tokens, row_ptr, col_idx,
                       col_capacity, ws, ws_bytes, stream);
}

int fp_sparse_attn_paged(const fp_problem* p, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* row_ptr, const int32_t* col_idx, const double* k_mean,
                         const double* v_mean, int32_t mean_correction, void* out, float* lse, void* ws,
                         size_t ws_bytes, void* stream) {
  Geometry g;
  int st = make_geometry(p, &g);
  if (st) return st;
  if (!q || !k_cache || !v_cache || !row_ptr || !col_idx || !out)
    return fail(FP_ERR_INVALID, "fp_sparse_attn_paged: a tensor pointer is NULL");
  if (mean_correction && (!k_mean || !v_mean))
    return fail(FP_ERR_INVALID, "mean correction needs k_mean and v_mean");
  if ((st = check_ws(g, FP_WS_ATTN, ws, ws_bytes))) return st;
  AttnWs w;
  ws_layout(g, FP_WS_ATTN, ws, &w);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const SeqMap m = seq_map(p, w.kboff, w.qboff);
  if ((st = hip_status(launch_attn_prep(g, m, mean_correction ? k_mean : nullptr, v_mean, w.km16,
                                        w.vm16, w.queue, s), "attn prep")))
    return st;
  return hip_status(launch_attn(g, m, p->page_table_dev, q, k_cache, v_cache, p->q_scale_dev,
                                p->k_scale_dev, row_ptr, col_idx, w.km16, w.vm16,
                                mean_correction ? 1 : 0, out, lse, w.opart, w.lpart, w.queue, s, false),
                    "attn");
}

int fp_dense_attn_paged(const fp_problem* p, const void* q, const void* k_cache,
                        const void* v_cache, void* out, float* lse, void* ws, size_t ws_bytes,
                        void* stream) {
  Geometry g;
  int st = make_geometry(p, &g);
  if (st) return st;
  if (!q || !k_cache || !v_cache || !out)
    return fail(FP_ERR_INVALID, "fp_dense_attn_paged: a tensor pointer is NULL");
  dense_geometry(&g);
  if ((st = check_ws(g, FP_WS_ATTN, ws, ws_bytes))) return st;
  AttnWs w;
  ws_layout(g, FP_WS_ATTN, ws, &w);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const SeqMap m = seq_map(p, w.kboff, w.qboff);
  if ((st = hip_status(launch_attn_prep(g, m, nullptr, nullptr, w.km16, w.vm16, w.queue, s), "attn prep")))
    return st;
  return hip_status(launch_attn(g, m, p->page_table_dev, q, k_cache, v_cache, p->q_scale_dev,
                                p->k_scale_dev, nullptr, nullptr, w.km16, w.vm16, 0, out, lse, w.opart,
                                w.lpart, w.queue, s, true),
                    "dense attn");
}

}  // extern "C"
