// C ABI of libherald.so: argument validation (before any HIP call), workspace
// sizing and carving, kernel launches, error reporting and the host-pool gather.
// The operations and their definitions are documented in include/herald.h.
#include "herald.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

#include "kernels.hpp"

using namespace herald;

namespace {

thread_local std::string g_error;

constexpr int kNumKernels = 10;
struct KernelEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
thread_local KernelEvents g_events[kNumKernels];

herald_status fail(herald_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

herald_status ok() {
  g_error.clear();
  return HERALD_OK;
}

#define HERALD_HIP(call)                                                                    \
  do {                                                                                      \
    const hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess) return fail(HERALD_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

// Launch `call` (returns hipError_t) as kernel `id`, bracketed by its events if set.
// The events are recorded as external nodes when the stream is being captured into
// a graph, so they time the kernel on every replay.
// The events are recorded right before and after the kernel on its stream; while the
// stream is being captured into a graph they become external event nodes, so they time
// the kernel on every replay.
#define HERALD_LAUNCH(id, stream, call)                                                     \
  do {                                                                                      \
    (void)hipGetLastError(); /* the launcher reports hipGetLastError(): start clean */      \
    if (g_events[id].start) HERALD_HIP(record_event(g_events[id].start, stream));           \
    HERALD_HIP(call);                                                                       \
    if (g_events[id].stop) HERALD_HIP(record_event(g_events[id].stop, stream));             \
  } while (0)

hipError_t record_event(hipEvent_t ev, hipStream_t stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing(stream, &st);
  if (e != hipSuccess) return e;
  if (st == hipStreamCaptureStatusActive) return hipEventRecordWithFlags(ev, stream, hipEventRecordExternal);
  return hipEventRecord(ev, stream);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

herald_status check_ptr(const void* p, const char* name, bool nullable = false) {
  if (!p) return nullable ? HERALD_OK : fail(HERALD_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(HERALD_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return HERALD_OK;
}

#define HERALD_TRY(expr)                         \
  do {                                           \
    const herald_status st_ = (expr);            \
    if (st_ != HERALD_OK) return st_;            \
  } while (0)

// Validates the problem and fills the kernel-side shape. Host memory only.
herald_status make_shape(const herald_problem* p, Shape* s) {
  if (!p) return fail(HERALD_ERR_INVALID_ARG, "problem is NULL");
  if (p->reserved != 0) return fail(HERALD_ERR_INVALID_ARG, "reserved field must be 0");
  if (p->nseq < 0) return fail(HERALD_ERR_INVALID_ARG, "nseq = %d is negative", p->nseq);
  if (p->nseq > 65535) return fail(HERALD_ERR_UNSUPPORTED, "nseq = %d exceeds 65535", p->nseq);
  if (p->block_size < 1 || p->block_size > 64)
    return fail(p->block_size < 1 ? HERALD_ERR_INVALID_ARG : HERALD_ERR_UNSUPPORTED,
                "block_size = %d outside [1, 64]", p->block_size);
  if (p->num_kv_heads < 1) return fail(HERALD_ERR_INVALID_ARG, "num_kv_heads = %d < 1", p->num_kv_heads);
  if (p->num_kv_heads > 65535) return fail(HERALD_ERR_UNSUPPORTED, "num_kv_heads = %d exceeds 65535", p->num_kv_heads);
  if (p->num_q_heads < p->num_kv_heads || p->num_q_heads % p->num_kv_heads != 0)
    return fail(HERALD_ERR_INVALID_ARG, "num_q_heads = %d is not a positive multiple of num_kv_heads = %d",
                p->num_q_heads, p->num_kv_heads);
  if ((int64_t)p->nseq * p->num_kv_heads > 65535)
    return fail(HERALD_ERR_UNSUPPORTED, "nseq * num_kv_heads = %lld exceeds 65535", (long long)p->nseq * p->num_kv_heads);
  const int G = p->num_q_heads / p->num_kv_heads;
  if (G > 8) return fail(HERALD_ERR_UNSUPPORTED, "group size G = %d exceeds 8", G);
  if (p->block_size * G > 256)
    return fail(HERALD_ERR_UNSUPPORTED, "block_size * G = %d exceeds 256", p->block_size * G);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(HERALD_ERR_UNSUPPORTED, "head_dim = %d is not 64 or 128", p->head_dim);
  if (p->dtype != HERALD_F32 && p->dtype != HERALD_BF16) return fail(HERALD_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
  if (p->num_candidates < 1) return fail(HERALD_ERR_INVALID_ARG, "num_candidates = %d < 1", p->num_candidates);
  if (p->topk < 1 || p->topk > p->num_candidates)
    return fail(HERALD_ERR_INVALID_ARG, "topk = %d outside [1, num_candidates = %d]", p->topk, p->num_candidates);
  if (p->topk > kMaxTopk) return fail(HERALD_ERR_UNSUPPORTED, "topk = %d exceeds %d", p->topk, kMaxTopk);
  if (!std::isfinite(p->softmax_scale) || p->softmax_scale < 0.f)
    return fail(HERALD_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if (!p->seq_start_host) return fail(HERALD_ERR_INVALID_ARG, "seq_start_host is NULL");
  if (!p->seq_start_dev) return fail(HERALD_ERR_INVALID_ARG, "seq_start_dev is NULL");
  if (p->seq_start_host[0] != 0) return fail(HERALD_ERR_INVALID_ARG, "seq_start[0] must be 0");
  int64_t max_len = 0;
  for (int i = 0; i < p->nseq; ++i) {
    const int64_t L = p->seq_start_host[i + 1] - p->seq_start_host[i];
    if (L < p->num_candidates)
      return fail(HERALD_ERR_INVALID_ARG, "sequence %d has length %lld < num_candidates = %d", i, (long long)L,
                  p->num_candidates);
    if (L > (int64_t(1) << 30)) return fail(HERALD_ERR_UNSUPPORTED, "sequence %d is longer than 2^30", i);
    max_len = std::max(max_len, L);
  }
  s->nseq = p->nseq;
  s->B = p->block_size;
  s->Hq = p->num_q_heads;
  s->Hkv = p->num_kv_heads;
  s->D = p->head_dim;
  s->G = G;
  s->C = p->num_candidates;
  s->topk = p->topk;
  s->bf16 = p->dtype == HERALD_BF16;
  s->scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.f / std::sqrt((float)p->head_dim);
  s->total = p->seq_start_host[p->nseq];
  s->max_len = max_len;
  s->seq_start = p->seq_start_dev;
  return HERALD_OK;
}

size_t elem_bytes(const Shape& s) { return s.bf16 ? 2 : 4; }

// Carves consecutive 256-byte-aligned regions out of a workspace.
struct Carver {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t count) {
    T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
    off += align256(count * sizeof(T));
    return p;
  }
};

SelectWs carve_select(const Shape& s, void* ws, size_t* bytes) {
  Carver c{static_cast<char*>(ws)};
  SelectWs w;
  w.tpc = !s.bf16 && s.total * s.Hkv <= kScoreTokSmallUpTo ? kScanTokSmall : kScanTok;
  w.nchunk = (int)((s.max_len + w.tpc - 1) / w.tpc);
  w.nwords = (int)((s.max_len + 63) / 64);
  w.qbar = c.take<float>((size_t)s.nseq * s.Hq * s.D);
  w.logits = c.take<float>((size_t)s.Hkv * s.total * (s.G <= 4 ? 4 : 8));  // token-major, heads padded
  w.partials = c.take<float2>((size_t)s.nseq * s.Hq * w.nchunk);
  w.scores = c.take<float>((size_t)s.Hkv * s.total);
  w.hist = c.take<uint32_t>((size_t)s.nseq * s.Hkv * 3 * kRadixBins);
  w.bits = c.take<uint64_t>((size_t)s.nseq * s.Hkv * 2 * w.nwords);
  *bytes = c.off;
  return w;
}

// Compressed selection: the token-level buffers of the top-C (merged query, scores,
// histograms, bitmaps) and the compressed scan's own (logits, pairs, block scores,
// a scratch histogram, row offsets), for compressed sequences of ceil(L_s / stride) rows.
struct CompressedWs {
  SelectWs tok;    // qbar, scores [Hkv][total], hist, bits
  SelectWs blk;    // qbar (shared), logits, partials, scores = block scores [Hkv][ctotal], hist (scratch)
  int64_t* coff;   // [nseq + 1] compressed row offsets
  int64_t ctotal;  // compressed rows of the batch
  int64_t cmax;    // compressed rows of the longest sequence
};

int64_t compressed_total(const herald_problem* p, int stride, int64_t* cmax) {
  int64_t t = 0, mx = 0;
  for (int i = 0; i < p->nseq; ++i) {
    const int64_t m = (p->seq_start_host[i + 1] - p->seq_start_host[i] + stride - 1) / stride;
    t += m;
    mx = std::max(mx, m);
  }
  if (cmax) *cmax = mx;
  return t;
}

CompressedWs carve_compressed(const herald_problem* p, const Shape& s, int stride, void* ws, size_t* bytes) {
  Carver c{static_cast<char*>(ws)};
  CompressedWs w;
  w.ctotal = compressed_total(p, stride, &w.cmax);
  const int GP = s.G <= 4 ? 4 : 8;
  w.tok.tpc = w.blk.tpc = kScanTok;
  w.tok.nchunk = 0;
  w.blk.nchunk = (int)((w.cmax + kScanTok - 1) / kScanTok);
  w.tok.nwords = w.blk.nwords = (int)((s.max_len + 63) / 64);
  w.tok.qbar = w.blk.qbar = c.take<float>((size_t)s.nseq * s.Hq * s.D);
  w.tok.logits = nullptr;
  w.tok.partials = nullptr;
  w.tok.scores = c.take<float>((size_t)s.Hkv * s.total);
  w.tok.hist = c.take<uint32_t>((size_t)s.nseq * s.Hkv * 3 * kRadixBins);
  w.tok.bits = c.take<uint64_t>((size_t)s.nseq * s.Hkv * 2 * w.tok.nwords);
  w.blk.logits = c.take<float>((size_t)s.Hkv * w.ctotal * GP);
  w.blk.partials = c.take<float2>((size_t)s.nseq * s.Hq * std::max(w.blk.nchunk, 1));
  w.blk.scores = c.take<float>((size_t)s.Hkv * w.ctotal);
  w.blk.hist = c.take<uint32_t>((size_t)s.nseq * s.Hkv * 3 * kRadixBins);
  w.blk.bits = nullptr;
  w.coff = c.take<int64_t>((size_t)s.nseq + 1);
  *bytes = c.off;
  return w;
}

herald_status check_compression(int ksize, int stride) {
  if (stride < 2 || stride > 65536) return fail(HERALD_ERR_INVALID_ARG, "stride = %d outside [2, 65536]", stride);
  if (ksize < 1 || ksize > 65536) return fail(HERALD_ERR_INVALID_ARG, "ksize = %d outside [1, 65536]", ksize);
  return HERALD_OK;
}

RefineWs carve_refine(const Shape& s, void* ws, size_t* bytes) {
  Carver c{static_cast<char*>(ws)};
  RefineWs w;
  const int tile = refine_tile_of(s);
  w.ntile = (s.C + tile - 1) / tile;
  w.nsplit = refine_splits(s);
  w.row_stats = c.take<float2>((size_t)s.nseq * s.Hkv * ((w.ntile + 1) & ~1) * s.B * s.G);
  w.rscore = c.take<float>((size_t)w.nsplit * s.nseq * s.Hkv * s.C);
  *bytes = c.off;
  return w;
}

size_t gather_host_bytes(const Shape& s) { return align256(2 * (size_t)s.nseq * s.Hkv * s.topk * s.D * elem_bytes(s)); }

// The merged-query selection keeps its candidate set in LDS during emission.
herald_status check_select_shape(const Shape& s) {
  if (s.C > kMaxCandidates)
    return fail(HERALD_ERR_UNSUPPORTED, "num_candidates = %d exceeds %d for herald_select_merged", s.C, kMaxCandidates);
  return HERALD_OK;
}

herald_status check_attn_shape(const Shape& s) {
  if (!attn_fits(s))
    return fail(HERALD_ERR_UNSUPPORTED, "attention work split of %d sequences x %d KV heads x %d keys is too large",
                s.nseq, s.Hkv, s.topk + s.B);
  return HERALD_OK;
}

herald_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return HERALD_OK;
  if (!ws) return fail(HERALD_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if (!aligned16(ws)) return fail(HERALD_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (have < need) return fail(HERALD_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return HERALD_OK;
}

}  // namespace

// Scratch of herald_block_attn_static: one array per GPU the library runs on, held
// until the process ends. Host code never uses its name as an address (that would be
// the host-side shadow); static_scratch looks up the device address once per device.
static __device__ __align__(256) unsigned char scratch[HERALD_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on the first call on each
// device, with that device current).
herald_status static_scratch(void** out) {
  int dev = -1;
  HERALD_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(HERALD_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    HERALD_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) return fail(HERALD_ERR_HIP, "hipGetSymbolAddress returned NULL for the static scratch");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return HERALD_OK;
}

}  // namespace

extern "C" {

herald_status herald_workspace_size(const herald_problem* p, int op, size_t* bytes) {
  if (!bytes) return fail(HERALD_ERR_INVALID_ARG, "bytes is NULL");
  Shape s;
  HERALD_TRY(make_shape(p, &s));
  size_t n = 0;
  switch (op) {
    case HERALD_OP_SELECT:
      HERALD_TRY(check_select_shape(s));
      carve_select(s, nullptr, &n);
      break;
    case HERALD_OP_REFINE: carve_refine(s, nullptr, &n); break;
    case HERALD_OP_ATTN:
      HERALD_TRY(check_attn_shape(s));
      n = attn_ws_bytes(s);
      break;
    case HERALD_OP_SELECT_COMPRESSED:
      HERALD_TRY(check_select_shape(s));
      carve_compressed(p, s, 2, nullptr, &n);  // stride 2 has the most compressed rows
      break;
    case HERALD_OP_GATHER_HOST: n = gather_host_bytes(s); break;
    default: return fail(HERALD_ERR_INVALID_ARG, "unknown op %d", op);
  }
  if (s.nseq == 0) n = 0;
  *bytes = n;
  return ok();
}

size_t herald_workspace_bytes(const herald_problem* p, int op) {
  size_t n = 0;
  return herald_workspace_size(p, op, &n) == HERALD_OK ? n : SIZE_MAX;
}

int64_t herald_vsel_ld(int32_t topk) { return topk < 1 ? 0 : vsel_ld(topk); }

// Stage one with the query fed to the scan given as [nseq][nq][Hq][d]: the mean of
// nq rows per head (the block's B queries, or one given query when nq = 1).
static herald_status select_common(const herald_problem* p, const void* q, int nq, const void* k_cache,
                                   int32_t* cand_idx, float* cand_score, void* ws, size_t ws_bytes,
                                   hipStream_t stream, const char* qname) {
  Shape s;
  HERALD_TRY(make_shape(p, &s));
  HERALD_TRY(check_select_shape(s));
  if (s.nseq == 0) return ok();
  HERALD_TRY(check_ptr(q, qname));
  HERALD_TRY(check_ptr(k_cache, "k_cache"));
  HERALD_TRY(check_ptr(cand_idx, "cand_idx"));
  HERALD_TRY(check_ptr(cand_score, "cand_score", true));
  size_t need;
  carve_select(s, nullptr, &need);
  HERALD_TRY(check_ws(ws, ws_bytes, need));
  const SelectWs w = carve_select(s, ws, &need);
  Shape sq = s;
  sq.B = nq;
  if (scan_merges_query(s)) {
    HERALD_LAUNCH(0, stream, launch_scan(s, k_cache, w, stream, q, nq));
  } else {
    HERALD_HIP(launch_merge(sq, q, w, stream));
    HERALD_LAUNCH(0, stream, launch_scan(s, k_cache, w, stream));
  }
  HERALD_LAUNCH(1, stream, launch_score_hist(s, w, stream));
  if (topc_in_lds(s)) {
    HERALD_LAUNCH(3, stream, launch_topc_lds(s, w, cand_idx, cand_score, stream));
  } else {
    HERALD_LAUNCH(2, stream, launch_radix_pass(s, w, 2, stream));
    HERALD_LAUNCH(2, stream, launch_radix_pass(s, w, 3, stream));
    HERALD_LAUNCH(3, stream, launch_emit_candidates(s, w, cand_idx, cand_score, stream));
  }
  return ok();
}

herald_status herald_select_merged(const herald_problem* p, const void* q_merge, const void* k_cache,
                                   int32_t* cand_idx, float* cand_score, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  if (!p) return fail(HERALD_ERR_INVALID_ARG, "problem is NULL");
  return select_common(p, q_merge, p->block_size, k_cache, cand_idx, cand_score, ws, ws_bytes, stream, "q_merge");
}

herald_status herald_select_query(const herald_problem* p, const void* q_sel, const void* k_cache,
                                  int32_t* cand_idx, float* cand_score, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  return select_common(p, q_sel, 1, k_cache, cand_idx, cand_score, ws, ws_bytes, stream, "q_sel");
}

int64_t herald_compressed_rows(const herald_problem* p, int32_t stride) {
  Shape s;
  if (make_shape(p, &s) != HERALD_OK || check_compression(1, stride) != HERALD_OK) return -1;
  return compressed_total(p, stride, nullptr);
}

herald_status herald_compress_keys(const herald_problem* p, const void* k_cache, int32_t ksize, int32_t stride,
                                   float* k_comp, hipStream_t stream) {
  Shape s;
  HERALD_TRY(make_shape(p, &s));
  HERALD_TRY(check_compression(ksize, stride));
  if (s.nseq == 0) return ok();
  HERALD_TRY(check_ptr(k_cache, "k_cache"));
  HERALD_TRY(check_ptr(k_comp, "k_comp"));
  HERALD_HIP(launch_compress(s, k_cache, ksize, stride, k_comp, stream));
  return ok();
}

herald_status herald_select_compressed(const herald_problem* p, const void* q_merge, const float* k_comp,
                                       int32_t stride, int32_t* cand_idx, float* cand_score, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
  Shape s;
  HERALD_TRY(make_shape(p, &s));
  HERALD_TRY(check_select_shape(s));
  HERALD_TRY(check_compression(1, stride));
  if (s.nseq == 0) return ok();
  HERALD_TRY(check_ptr(q_merge, "q_merge"));
  HERALD_TRY(check_ptr(k_comp, "k_comp"));
  HERALD_TRY(check_ptr(cand_idx, "cand_idx"));
  HERALD_TRY(check_ptr(cand_score, "cand_score", true));
  size_t need;
  carve_compressed(p, s, 2, nullptr, &need);
  HERALD_TRY(check_ws(ws, ws_bytes, need));
  const CompressedWs w = carve_compressed(p, s, stride, ws, &need);
  // the compressed cache as a batch of its own: fp32 rows, offsets computed on the device
  Shape sc = s;
  sc.bf16 = 0;
  sc.seq_start = w.coff;
  sc.total = w.ctotal;
  sc.max_len = w.cmax;
  HERALD_HIP(launch_merge(s, q_merge, w.tok, stream));  // merged query; zeroes the token histograms
  HERALD_HIP(launch_coffsets(s, stride, w.coff, stream));
  HERALD_LAUNCH(0, stream, launch_scan(sc, k_comp, w.blk, stream));
  HERALD_LAUNCH(1, stream, launch_score_hist(sc, w.blk, stream));  // block scores (its histogram is not used)
  HERALD_LAUNCH(1, stream, launch_expand_hist(s, w.blk.scores, w.coff, w.ctotal, stride, w.tok, stream));
  if (topc_in_lds(s)) {
    HERALD_LAUNCH(3, stream, launch_topc_lds(s, w.tok, cand_idx, cand_score, stream));
  } else {
    HERALD_LAUNCH(2, stream, launch_radix_pass(s, w.tok, 2, stream));
    HERALD_LAUNCH(2, stream, launch_radix_pass(s, w.tok, 3, stream));
    HERALD_LAUNCH(3, stream, launch_emit_candidates(s, w.tok, cand_idx, cand_score, stream));
  }
  return ok();
}

herald_status herald_refine_topk(const herald_problem* p, const void* q_refine, const void* k_cache,
                                 const int32_t* cand_idx, int32_t* topk_idx, float* topk_score, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  Shape s;
  HERALD_TRY(make_shape(p, &s));
  if (s.nseq == 0) return ok();
  HERALD_TRY(check_ptr(q_refine, "q_refine"));
  HERALD_TRY(check_ptr(k_cache, "k_cache"));
  HERALD_TRY(check_ptr(cand_idx, "cand_idx"));
  HERALD_TRY(check_ptr(topk_idx, "topk_idx"));
  HERALD_TRY(check_ptr(topk_score, "topk_score", true));
  size_t need;
  carve_refine(s, nullptr, &need);
  HERALD_TRY(check_ws(ws, ws_bytes, need));
  const RefineWs w = carve_refine(s, ws, &need);
  HERALD_LAUNCH(4, stream, launch_refine_stats(s, q_refine, k_cache, cand_idx, w, stream));
  HERALD_LAUNCH(5, stream, launch_refine_scores(s, q_refine, k_cache, cand_idx, w, stream));
  HERALD_LAUNCH(6, stream, launch_refine_select(s, cand_idx, w, topk_idx, topk_score, stream));
  return ok();
}

herald_status herald_gather_kv(const herald_problem* p, const void* k_src, const void* v_src, int32_t src_is_host,
                               const int32_t* topk_idx, void* k_sel, void* v_sel, void* host_staging,
                               int32_t* host_idx, void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t done) {
  Shape s;
  HERALD_TRY(make_shape(p, &s));
  if (s.nseq == 0) return ok();
  HERALD_TRY(check_ptr(k_src, "k_src"));
  HERALD_TRY(check_ptr(v_src, "v_src"));
  HERALD_TRY(check_ptr(topk_idx, "topk_idx"));
  HERALD_TRY(check_ptr(k_sel, "k_sel"));
  HERALD_TRY(check_ptr(v_sel, "v_sel"));
  if (src_is_host < 0 || src_is_host > 2) return fail(HERALD_ERR_INVALID_ARG, "src_is_host must be 0, 1 or 2");
  // the device and GPU-read paths take an optional status word in ws
  int32_t* status = nullptr;
  if (src_is_host != 1 && ws) {
    if (ws_bytes < sizeof(int32_t)) return fail(HERALD_ERR_WORKSPACE, "status word needs 4 bytes, ws has %zu", ws_bytes);
    if ((reinterpret_cast<uintptr_t>(ws) & 3u) != 0) return fail(HERALD_ERR_INVALID_ARG, "status word is not 4-byte aligned");
    status = static_cast<int32_t*>(ws);
  }
  if (src_is_host == 0) {
    HERALD_LAUNCH(7, stream, launch_gather(s, k_src, v_src, topk_idx, k_sel, v_sel, status, stream));
    if (done) HERALD_HIP(hipEventRecord(done, stream));
    return ok();
  }
  if (src_is_host == 2) {
    // the kernel reads the pinned pool directly: device addresses of the host rows
    const void* src[2] = {k_src, v_src};
    const void* dev[2];
    for (int i = 0; i < 2; ++i) {
      hipPointerAttribute_t a{};
      if (hipPointerGetAttributes(&a, src[i]) != hipSuccess || a.type != hipMemoryTypeHost || !a.devicePointer) {
        (void)hipGetLastError();
        return fail(HERALD_ERR_INVALID_ARG, "%s is not pinned host memory (hipHostMalloc)", i ? "v_src" : "k_src");
      }
      dev[i] = a.devicePointer;
    }
    HERALD_LAUNCH(7, stream, launch_gather(s, dev[0], dev[1], topk_idx, k_sel, v_sel, status, stream));
    if (done) HERALD_HIP(hipEventRecord(done, stream));
    return ok();
  }
  HERALD_TRY(check_ptr(host_staging, "host_staging"));
  HERALD_TRY(check_ptr(host_idx, "host_idx"));
  if (!done) return fail(HERALD_ERR_INVALID_ARG, "done event is required on the host-pool path");
  const size_t need = gather_host_bytes(s);
  HERALD_TRY(check_ws(ws, ws_bytes, need));
  const size_t n = (size_t)s.nseq * s.Hkv * s.topk;
  const size_t row = (size_t)s.D * elem_bytes(s);
  HERALD_HIP(hipMemcpyAsync(host_idx, topk_idx, n * sizeof(int32_t), hipMemcpyDeviceToHost, stream));
  HERALD_HIP(hipStreamSynchronize(stream));
  const char* kh = static_cast<const char*>(k_src);
  const char* vh = static_cast<const char*>(v_src);
  char* kst = static_cast<char*>(host_staging);
  char* vst = kst + n * row;
  for (int sq = 0; sq < s.nseq; ++sq) {
    const int64_t j0 = p->seq_start_host[sq];
    const int64_t L = p->seq_start_host[sq + 1] - j0;
    for (int g = 0; g < s.Hkv; ++g) {
      const size_t unit = (size_t)sq * s.Hkv + g;
      for (int i = 0; i < s.topk; ++i) {
        const int32_t j = host_idx[unit * s.topk + i];
        if (j < 0 || j >= L)
          return fail(HERALD_ERR_INVALID_ARG, "topk_idx[%d][%d][%d] = %d outside [0, %lld)", sq, g, i, j, (long long)L);
        const size_t src = ((size_t)(j0 + j) * s.Hkv + g) * row;
        std::memcpy(kst + (unit * s.topk + i) * row, kh + src, row);
        std::memcpy(vst + (unit * s.topk + i) * row, vh + src, row);
      }
    }
  }
  HERALD_HIP(hipMemcpyAsync(ws, host_staging, 2 * n * row, hipMemcpyHostToDevice, stream));
  const char* wsc = static_cast<const char*>(ws);
  HERALD_LAUNCH(7, stream, launch_layout_packed(s, wsc, wsc + n * row, k_sel, v_sel, stream));
  HERALD_HIP(hipEventRecord(done, stream));
  return ok();
}

// Validation shared by both attention entry points (host memory only).
static herald_status attn_validate(const herald_problem* p, Shape* s, const void* q, const void* k_blk,
                                   const void* v_blk, const void* k_sel, const void* v_sel, const void* out) {
  HERALD_TRY(make_shape(p, s));
  if (s->nseq == 0) return HERALD_OK;
  HERALD_TRY(check_ptr(q, "q"));
  HERALD_TRY(check_ptr(k_blk, "k_blk"));
  HERALD_TRY(check_ptr(v_blk, "v_blk"));
  HERALD_TRY(check_ptr(k_sel, "k_sel"));
  HERALD_TRY(check_ptr(v_sel, "v_sel"));
  HERALD_TRY(check_ptr(out, "out"));
  return check_attn_shape(*s);
}

static herald_status attn_launch(const Shape& s, const void* q, const void* k_blk, const void* v_blk,
                                 const void* k_sel, const void* v_sel, void* out, void* ws, hipStream_t stream) {
  HERALD_LAUNCH(8, stream, launch_attn(s, q, k_blk, v_blk, k_sel, v_sel, out, ws, stream));
  if (attn_splits(s) > 1) HERALD_LAUNCH(9, stream, launch_attn_combine(s, ws, out, stream));
  return ok();
}

herald_status herald_block_attn(const herald_problem* p, const void* q, const void* k_blk, const void* v_blk,
                                const void* k_sel, const void* v_sel, void* out, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  Shape s;
  HERALD_TRY(attn_validate(p, &s, q, k_blk, v_blk, k_sel, v_sel, out));
  if (s.nseq == 0) return ok();
  HERALD_TRY(check_ws(ws, ws_bytes, attn_ws_bytes(s)));
  return attn_launch(s, q, k_blk, v_blk, k_sel, v_sel, out, ws, stream);
}

herald_status herald_block_attn_static(const herald_problem* p, const void* q, const void* k_blk, const void* v_blk,
                                       const void* k_sel, const void* v_sel, void* out, hipStream_t stream) {
  Shape s;
  HERALD_TRY(attn_validate(p, &s, q, k_blk, v_blk, k_sel, v_sel, out));
  if (s.nseq == 0) return ok();
  const size_t need = attn_ws_bytes(s);
  if (need > HERALD_STATIC_SCRATCH_BYTES)
    return fail(HERALD_ERR_UNSUPPORTED, "the split attention needs %zu bytes of scratch; the static buffer holds %zu",
                need, (size_t)HERALD_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) HERALD_TRY(static_scratch(&ws));
  return attn_launch(s, q, k_blk, v_blk, k_sel, v_sel, out, ws, stream);
}

const char* herald_last_error(void) { return g_error.c_str(); }

herald_status herald_set_kernel_events(int32_t kernel_id, hipEvent_t start, hipEvent_t stop) {
  if (kernel_id < 0 || kernel_id >= kNumKernels) return fail(HERALD_ERR_INVALID_ARG, "kernel id %d", kernel_id);
  if ((start == nullptr) != (stop == nullptr))
    return fail(HERALD_ERR_INVALID_ARG, "start and stop must both be set or both be NULL");
  g_events[kernel_id].start = start;
  g_events[kernel_id].stop = stop;
  return ok();
}

int32_t herald_attn_splits(const herald_problem* p) {
  Shape s;
  if (make_shape(p, &s) != HERALD_OK) return -1;
  return attn_splits(s);
}

}  // extern "C"
