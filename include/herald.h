/*
 * herald.h - C ABI of the HERALD-style once-per-block sparse KV selection and
 * sparse block attention library for MI355X (gfx950). Library: libherald.so.
 *
 * The method (HERALD, "High-Throughput Block Diffusion LLM Inference via CPU-GPU
 * Cooperative KV Cache Retrieval", arXiv 2606.21633 v3, abstract): a block dLLM
 * decodes a block of B tokens over T denoising steps. Once per block, a single
 * query merged from the block's B queries scans the full KV cache and keeps C
 * candidates; the B real queries then refine the candidates into the final
 * top-K subset; the denoising steps reuse that subset (HERALD abstract on the
 * mlsift "KV cache offloading" listing: selection scans the full cache once per
 * block, denoising reuses the small subset T times). The per-KV-head score is
 * the sum over the group's G query heads of softmax(q k^T / tau) (SparDA,
 * arXiv 2606.04511, hyper.ai summary, Method section, target-score equation).
 *
 * Definitions used by every entry point (one sequence s, KV head g, G = Hq/Hkv,
 * query head h belongs to KV head h / G, scale = softmax_scale or 1/sqrt(d)):
 *   merged query     qbar[h]   = (1/B) sum_b q_merge[s][b][h]
 *   selection score  S_g[j]    = sum_{h in g} softmax_j(scale <qbar[h], K[j][g]>),
 *                                softmax over all L_s keys of the sequence
 *   candidates       the C largest S_g[j], ties to the lower j
 *   refine score     R_g[c]    = sum_b sum_{h in g} softmax_c(scale <q_refine[s][b][h], K[cand_c][g]>),
 *                                softmax over the C candidates only
 *   final subset     the topk largest R_g[c], ties to the lower cache index
 *   block attention  out[b][h] = softmax(scale q[b][h] . keys^T) . values, keys = the
 *                                topk selected keys of g followed by the B in-block
 *                                keys of the step, no mask
 *
 * Conventions
 *   - The caller owns all memory. The library never allocates. Each op that needs
 *     scratch memory takes a device workspace of herald_workspace_size() bytes.
 *   - Tensors are row-major, head_dim fastest, in the problem's dtype (fp32 or
 *     bf16; Q, K, V and outputs share it). Every pointer is 16-byte aligned.
 *   - The KV cache is packed token-major: K[sumL][Hkv][d], sequence s owning the
 *     rows [seq_start[s], seq_start[s+1]).
 *   - Index outputs are int32, sequence-local, sorted ascending.
 *   - Every call validates all arguments before any HIP call, enqueues its
 *     kernels on `stream` and returns without waiting (except the host-pool
 *     gather, which waits on its own stream only). Kernel faults surface at the
 *     caller's next synchronisation.
 *   - Errors: a non-zero herald_status; herald_last_error() then describes it.
 *     No C++ exception crosses the ABI. Calls that use distinct workspaces and
 *     outputs may run concurrently on different streams.
 */
#ifndef HERALD_H
#define HERALD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum herald_status {
  HERALD_OK = 0,
  HERALD_ERR_INVALID_ARG = 1, /* a size, pointer, alignment or bound is wrong          */
  HERALD_ERR_UNSUPPORTED = 2, /* valid in principle, outside what the kernels support  */
  HERALD_ERR_WORKSPACE = 3,   /* workspace smaller than herald_workspace_size()        */
  HERALD_ERR_HIP = 4          /* a HIP runtime call failed; the message names it        */
} herald_status;

typedef enum herald_dtype { HERALD_F32 = 0, HERALD_BF16 = 1 } herald_dtype;

typedef enum herald_op {
  HERALD_OP_SELECT = 0,      /* herald_select_merged                                  */
  HERALD_OP_REFINE = 1,      /* herald_refine_topk                                    */
  HERALD_OP_ATTN = 2,        /* herald_block_attn                                     */
  HERALD_OP_GATHER_HOST = 3, /* herald_gather_kv with src_is_host = 1                 */
  HERALD_OP_SELECT_COMPRESSED = 4 /* herald_select_compressed, any stride >= 2       */
} herald_op;

/*
 * The shape of one batch. Limits (checked by every call):
 *   nseq >= 0 (0 makes every call a no-op); 1 <= block_size <= 64;
 *   num_kv_heads >= 1; num_q_heads = G * num_kv_heads with 1 <= G <= 8;
 *   block_size * G <= 256; head_dim in {64, 128};
 *   1 <= topk <= num_candidates <= L_s <= 2^30 for every s, topk <= 2^24
 *   (HERALD_ERR_UNSUPPORTED above); herald_select_merged (and
 *   its workspace query) also needs num_candidates <= 16384 (HERALD_ERR_UNSUPPORTED
 *   otherwise). The other calls take any candidate count and subset size up to the
 *   shortest sequence, which expresses the exact baselines: refine over every key of
 *   the sequence (num_candidates = L_s), or attention over the whole cache
 *   (topk = L_s).
 *   softmax_scale finite and >= 0 (0 selects 1/sqrt(head_dim)).
 * seq_start_host and seq_start_dev hold the same nseq+1 offsets (host copy for
 * validation and launch sizing, device copy for the kernels); seq_start[0] = 0.
 */
typedef struct herald_problem {
  int32_t nseq;
  int32_t block_size;     /* B: queries per block, and in-block keys per step   */
  int32_t num_q_heads;    /* Hq                                                 */
  int32_t num_kv_heads;   /* Hkv                                                */
  int32_t head_dim;       /* d                                                  */
  int32_t num_candidates; /* C: candidates kept by the merged-query scan        */
  int32_t topk;           /* final subset size per (sequence, KV head)          */
  int32_t dtype;          /* herald_dtype                                       */
  float softmax_scale;    /* 0 => 1/sqrt(head_dim)                              */
  int32_t reserved;       /* must be 0                                          */
  const int64_t* seq_start_host;
  const int64_t* seq_start_dev;
} herald_problem;

/* Bytes of device workspace `op` needs for problem `p` (written to *bytes). Errors
 * as the op itself reports them for the problem (HERALD_ERR_INVALID_ARG for an
 * invalid problem or op, HERALD_ERR_UNSUPPORTED for a shape the op does not take). */
herald_status herald_workspace_size(const herald_problem* p, int op, size_t* bytes);

/* The same size as a return value: the workspace query in the form the caller sizes
 * allocations with. Returns SIZE_MAX where herald_workspace_size returns an error
 * (herald_last_error() then names it); 0 is a valid size (no workspace needed). */
size_t herald_workspace_bytes(const herald_problem* p, int op);

/* Leading dimension (elements) of each d-row of v_sel: topk rounded up to 64. */
int64_t herald_vsel_ld(int32_t topk);

/*
 * Stage one: merged query, full-cache scan, top-C candidates (HERALD v3 abstract:
 * a single query merged from the block's B queries searches the full KV cache).
 *   q_merge    [nseq][B][Hq][d]   device, read
 *   k_cache    [sumL][Hkv][d]     device, read
 *   cand_idx   [nseq][Hkv][C]     device, written: int32, ascending, sequence-local
 *   cand_score [nseq][Hkv][C]     device, written (may be NULL): fp32 S_g of each candidate
 *   ws         workspace of herald_workspace_size(HERALD_OP_SELECT) bytes, device
 */
herald_status herald_select_merged(const herald_problem* p, const void* q_merge, const void* k_cache,
                                   int32_t* cand_idx, float* cand_score, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/*
 * Stage one from one given query per head instead of the block mean: the same scan,
 * scores and top-C as herald_select_merged, with q_sel taking the place of the merged
 * query (HERALD abstract on the mlsift listing: the selection cost is cut by searching
 * with a single [MASK] query; MAGE abstract: the All-[MASK] step's attention predicts
 * the important entries). Every other argument, the workspace and the errors are those
 * of herald_select_merged.
 *   q_sel      [nseq][Hq][d]      device, read
 */
herald_status herald_select_query(const herald_problem* p, const void* q_sel, const void* k_cache,
                                  int32_t* cand_idx, float* cand_score, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/*
 * Compressed keys (SparDA, hyper.ai summary, Method section: block-level relevance
 * against keys mean-pooled into overlapping compressed representations). Block m of
 * sequence s owns tokens [m*stride, (m+1)*stride) (the last block may be short); its
 * compressed key is the mean of the keys in [m*stride, m*stride + ksize), cut at the
 * end of the sequence (ksize > stride overlaps the windows).
 *   herald_compressed_rows: rows of the compressed cache, sum over s of
 *     ceil(L_s / stride); -1 for an invalid problem or stride.
 *   herald_compress_keys: k_comp [rows][Hkv][d] fp32, device, written (sequences
 *     concatenated in order); k_cache as for the other calls. 2 <= stride <= 65536,
 *     1 <= ksize <= 65536 (HERALD_ERR_INVALID_ARG otherwise). Reads each key
 *     ceil(ksize / stride) times; meant to be run when the cache grows, not per block.
 *   herald_select_compressed: stage one over the compressed cache: block score =
 *     sum over the group's heads of the merged query's softmax over the blocks of the
 *     sequence; every token takes its block's score, and the candidates are the exact
 *     top-C tokens of that (ties to the lower index: whole blocks in score order, the
 *     boundary block from its lowest token up). Outputs as herald_select_merged;
 *     workspace herald_workspace_size(HERALD_OP_SELECT_COMPRESSED) (valid for every
 *     stride >= 2). The scan reads the compressed cache instead of the token cache:
 *     4 * d bytes per block and KV head.
 */
int64_t herald_compressed_rows(const herald_problem* p, int32_t stride);
herald_status herald_compress_keys(const herald_problem* p, const void* k_cache, int32_t ksize, int32_t stride,
                                   float* k_comp, hipStream_t stream);
herald_status herald_select_compressed(const herald_problem* p, const void* q_merge, const float* k_comp,
                                       int32_t stride, int32_t* cand_idx, float* cand_score, void* ws,
                                       size_t ws_bytes, hipStream_t stream);

/*
 * Stage two: refine the candidates with the B real queries into the final subset
 * (HERALD v3 abstract: the GPU refines the candidates into the final top-K subset
 * with the block's real queries).
 *   q_refine   [nseq][B][Hq][d]   device, read
 *   k_cache    [sumL][Hkv][d]     device, read
 *   cand_idx   [nseq][Hkv][C]     device, read: ascending, sequence-local, each < L_s
 *                                 (C = L_s with cand_idx = 0..L_s-1 is the exact top-K
 *                                 of the real queries over the whole cache; candidate
 *                                 sets above 16384 are ranked from global memory)
 *   topk_idx   [nseq][Hkv][topk]  device, written: int32, ascending, sequence-local
 *   topk_score [nseq][Hkv][topk]  device, written (may be NULL): fp32 R_g of each pick
 *   ws         workspace of herald_workspace_size(HERALD_OP_REFINE) bytes, device
 */
herald_status herald_refine_topk(const herald_problem* p, const void* q_refine, const void* k_cache,
                                 const int32_t* cand_idx, int32_t* topk_idx, float* topk_score, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/*
 * Fetch the selected subset once per block into the sparse KV pool (HERALD
 * abstract on the mlsift listing: only a small critical subset is fetched, once
 * per block).
 *   k_src, v_src [sumL][Hkv][d]   the full cache: device memory (src_is_host = 0) or
 *                                 pinned host memory from hipHostMalloc (src_is_host = 1, 2)
 *   topk_idx  [nseq][Hkv][topk]   device, read
 *   k_sel     [nseq][Hkv][topk][d]               device, written
 *   v_sel     [nseq][Hkv][d][herald_vsel_ld(topk)] device, written: V stored d-major
 *             (entry [s][g][e][i] = V[row of pick i][g][e]); padding columns are zero
 * Device path (src_is_host = 0): one kernel on `stream`; host_staging and host_idx
 * may be NULL; `done`, when not NULL, is recorded after it. An index outside
 * [0, L_s) is never dereferenced: the kernel writes zero K and V rows for it. ws is
 * then an optional status word (NULL, or a device int32, ws_bytes >= 4, 4-byte
 * aligned) that the kernel sets to 1 when it met such an index; the caller clears it
 * beforehand and reads it after the stream has passed the call.
 * Host-pool path (src_is_host = 1): `stream` should be a side stream. The call
 * copies topk_idx to host_idx (pinned, nseq*Hkv*topk int32), waits for `stream`,
 * packs the picked rows of k_src and v_src into host_staging (pinned,
 * 2*nseq*Hkv*topk*d elements) on the calling thread, issues one hipMemcpyAsync
 * host-to-device of the packed rows into ws (herald_workspace_size(
 * HERALD_OP_GATHER_HOST) bytes), lays them out into k_sel / v_sel with a kernel and
 * records `done` (required). The main stream waits on `done` before attention.
 * Host-pool path read by the GPU (src_is_host = 2): the gather kernel itself reads the
 * picked rows from the pinned host pool over PCIe (each row 16-byte loads of one
 * contiguous row), with no host work and no synchronisation, so it can run on a side
 * stream while the other stream computes, and be captured into a graph. k_src and
 * v_src must be pinned host memory (HERALD_ERR_INVALID_ARG otherwise, checked with
 * hipPointerGetAttributes); host_staging and host_idx may be NULL; ws is the optional
 * status word of the device path (out-of-range indices read nothing, as there);
 * `done`, when not NULL, is recorded after the kernel.
 */
herald_status herald_gather_kv(const herald_problem* p, const void* k_src, const void* v_src,
                               int32_t src_is_host, const int32_t* topk_idx, void* k_sel, void* v_sel,
                               void* host_staging, int32_t* host_idx, void* ws, size_t ws_bytes,
                               hipStream_t stream, hipEvent_t done);

/*
 * One denoising step of B-query block attention over the selected subset plus the
 * step's in-block keys (HERALD abstract on the mlsift listing: the denoising phase
 * reuses the selected subset T times). Call once per step.
 *   q      [nseq][B][Hq][d]   device, read
 *   k_blk  [nseq][B][Hkv][d]  device, read: the step's in-block keys
 *   v_blk  [nseq][B][Hkv][d]  device, read
 *   k_sel, v_sel              device, read, as written by herald_gather_kv
 *   out    [nseq][B][Hq][d]   device, written (fp32 accumulation, rounded to the dtype)
 *   ws     workspace of herald_workspace_size(HERALD_OP_ATTN) bytes, device: partial
 *          results when the subset is long enough to be split into key ranges;
 *          NULL allowed when that size is 0
 * HERALD_ERR_UNSUPPORTED when the batch's work split exceeds the kernel's 32-bit
 * workgroup numbering (far beyond any realistic batch; checked on the host).
 */
herald_status herald_block_attn(const herald_problem* p, const void* q, const void* k_blk, const void* v_blk,
                                const void* k_sel, const void* v_sel, void* out, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/*
 * herald_block_attn without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, kernels, results and errors as herald_block_attn,
 * minus ws / ws_bytes: the split-range partial results go to a static device array of
 * HERALD_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs on until
 * the process ends. The call allocates nothing. A problem whose attention workspace
 * (herald_workspace_size(HERALD_OP_ATTN)) exceeds that size is refused with
 * HERALD_ERR_UNSUPPORTED before any HIP call. Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (concurrent streams, or threads) race and give
 * undefined results; calls ordered on one stream do not. The first call on a device
 * looks up the array's device address (hipGetSymbolAddress) with that device current.
 */
#define HERALD_STATIC_SCRATCH_BYTES (16u << 20)
herald_status herald_block_attn_static(const herald_problem* p, const void* q, const void* k_blk,
                                       const void* v_blk, const void* k_sel, const void* v_sel, void* out,
                                       hipStream_t stream);

/* Message for the last non-OK status on the calling thread ("" if none). Valid
 * until the next call on this thread. */
const char* herald_last_error(void);

/*
 * Instrumentation. Kernel ids: 0 merged-query scan, 1 selection scores + first
 * radix digit, 2 second and third radix digits (sequences longer than 36864 tokens
 * only), 3 candidate emission (with the second and third digits for sequences up to
 * 36864 tokens), 4 refine statistics, 5 refine scores, 6 final top-K, 7 gather,
 * 8 block attention, 9 merge of the attention key ranges (split subsets only). The
 * single-query and compressed selections use ids 0-3 the same way (for the compressed
 * one, 0 is the scan of the compressed cache and 1 the last of its two score kernels).
 * While set (non-NULL), every launch of that kernel on a call's stream is bracketed
 * by records of start and stop on the same stream (external event nodes when the
 * stream is being captured into a graph); the last launch wins; a kernel a call does
 * not launch records nothing. Pass NULL events to clear. Thread-local setting.
 */
herald_status herald_set_kernel_events(int32_t kernel_id, hipEvent_t start, hipEvent_t stop);

/* Number of key ranges herald_block_attn splits each (sequence, KV head)'s keys
 * into for problem p (for reporting; 1 means no merge kernel); -1 for an invalid
 * problem. */
int32_t herald_attn_splits(const herald_problem* p);

#ifdef __cplusplus
}
#endif

#endif /* HERALD_H */
