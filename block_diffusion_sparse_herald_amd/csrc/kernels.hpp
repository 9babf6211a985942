// Internal launch interface between the C ABI layer (abi.cpp) and the kernels.
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace herald {

// Every kernel launch of the library goes through here.
template <typename F, typename... Args>
inline void klaunch(F kernel, dim3 grid, dim3 block, size_t smem, hipStream_t st, Args... args) {
  hipLaunchKernelGGL(kernel, grid, block, smem, st, args...);
}

// Tokens one scan workgroup covers (one KV head), and tokens one score / radix
// workgroup covers.
constexpr int kScanTok = 256;
// fp32 caches of up to kScoreTokSmallUpTo (token, KV head) pairs scan in chunks of 64
// tokens, four times the workgroups of the full chunk on a cache that would fill few.
constexpr int kScanTokSmall = 64;
constexpr int kScoreTok = 1024;
// Score / radix workgroups of 2048 tokens once the cache holds this many tokens: fewer
// workgroups amortise the per-workgroup normaliser merge and histogram flush.
constexpr int kScoreTokLarge = 2048;
constexpr int64_t kScoreTokLargeFrom = 262144;
constexpr int kScoreTokSmall = 256;
constexpr int64_t kScoreTokSmallUpTo = 16384;  // (token, KV head) pairs in the batch
constexpr int kRadixBins = 2048;
// Longest sequence whose selection scores one 1024-thread workgroup keeps in registers
// (36 per thread) for the one-kernel top-C.
constexpr int kTopcLdsMaxLen = 36864;
// Candidates one refine workgroup covers (bf16 MFMA path: 64 per wave; fp32 path).
// Keys per attention block and the largest supported candidate count.
constexpr int kAttnKeyBlock = 64;
constexpr int kMaxCandidates = 16384;
// Largest subset size: every index arithmetic on a subset row offset (pick * head_dim,
// d-row offsets of the d-major V pool) stays inside int32.
constexpr int kMaxTopk = 1 << 24;

struct Shape {
  int nseq, B, Hq, Hkv, D, G, C, topk;
  int bf16;        // 1: bf16 tensors, 0: fp32
  float scale;     // softmax scale (already resolved)
  int64_t total;   // sum of the sequence lengths
  int64_t max_len; // longest sequence
  const int64_t* seq_start;  // device
};

struct SelectWs {
  float* qbar;       // [nseq][Hq][D] merged query * scale * log2(e)
  float* logits;     // [Hkv][total][4 or 8] base-2 logits of the merged query (heads of the group, padded)
  float2* partials;  // [nseq][Hq][nchunk] (max, sum 2^(x-max)) per scan chunk
  float* scores;     // [Hkv][total] selection score S
  uint32_t* hist;    // [nseq][Hkv][3][kRadixBins]
  uint64_t* bits;    // [nseq][Hkv][2][nwords] (above-prefix, equal-prefix) bitmaps
  int tpc;           // tokens per scan chunk
  int nchunk;        // scan chunks per sequence (max over sequences)
  int nwords;        // bitmap words per (sequence, KV head)
};


struct RefineWs {
  float2* row_stats;   // [nseq][Hkv][rows][ntile rounded up to even] (max, sum) per refine tile
  float* rscore;       // [nsplit][nseq][Hkv][C] partial refine scores of the row splits
  int ntile;
  int nsplit;          // row splits (refine_splits)
};
constexpr int kRefineMaxSplits = 4;
constexpr int kRefineSplitTarget = 256;  // split rows while the grid stays within one workgroup per compute unit

// Attention work split (see attn_geom): query tiles per workgroup, key ranges.
struct AttnGeom {
  int B, G, Hq, Hkv, topk;
  int64_t ldv;
  int nunits;  // nseq * Hkv
  int tpw;     // 16-row query tiles per workgroup (one per wave)
  int nrs;     // row splits: workgroups per key range
  int rpad;    // rows rounded up to whole tiles
  int nks;     // key ranges per unit
  int bps;     // 64-key blocks per key range
  int nst;     // LDS stages (blocks in flight) per workgroup
  int nitems;  // workgroups
  // multiply-high reciprocals of nrs, nks and Hkv (ceil(2^32 / d), 0 for d = 1): the
  // kernel decodes its workgroup with one s_mul_hi_u32 per division; exact because
  // every quotient taken is below nitems and nitems * d < 2^32 (checked by attn_geom)
  uint32_t rcp_nrs, rcp_nks, rcp_hkv;
  uint32_t rcp_g;   // ceil(2^32 / G), 0 for G = 1 (exact: query rows r < 2^16)
  uint32_t rcp_pu;  // ceil(2^32 / (B * G * D / 8)) for the range merge's thread index, 0 when that is
                    // not exact for every index (the merge then divides)
};
constexpr int kAttnBlocksPerRange = 32;
constexpr int kAttnTargetWorkgroups = 256;  // one per compute unit
constexpr int kAttnFewPairs = 96;  // below this (pairs x four-tile row groups x 5) the few-pairs geometry applies
constexpr int kAttnTargetWorkgroupsFew = 192;  // with two query tiles per workgroup
constexpr int kAttnMaxStages = 4;
constexpr int kAttnCombineThreads = 64;   // range-merge workgroup (8 output dims per thread); 256 once that
                                           // still gives >= 256 workgroups

// select
hipError_t launch_merge(const Shape& s, const void* q, const SelectWs& ws, hipStream_t st);
// q (with nq query rows per block): bf16 caches on the register scan form the merged
// query inside the scan and zero the histograms (scan_merges_query), in place of launch_merge
hipError_t launch_scan(const Shape& s, const void* k, const SelectWs& ws, hipStream_t st, const void* q = nullptr,
                       int nq = 0);
bool scan_merges_query(const Shape& s);
hipError_t launch_score_hist(const Shape& s, const SelectWs& ws, hipStream_t st);
hipError_t launch_radix_pass(const Shape& s, const SelectWs& ws, int pass, hipStream_t st);
hipError_t launch_emit_candidates(const Shape& s, const SelectWs& ws, int32_t* cand, float* cand_score,
                                  hipStream_t st);
// compressed keys (compress.hip)
hipError_t launch_compress(const Shape& s, const void* k, int ksize, int stride, float* k_comp, hipStream_t st);
hipError_t launch_coffsets(const Shape& s, int stride, int64_t* coff, hipStream_t st);
hipError_t launch_expand_hist(const Shape& s, const float* s_blk, const int64_t* coff, int64_t ctotal, int stride,
                              const SelectWs& ws, hipStream_t st);
bool topc_in_lds(const Shape& s);
hipError_t launch_topc_lds(const Shape& s, const SelectWs& ws, int32_t* cand, float* cand_score, hipStream_t st);
// refine
hipError_t launch_refine_stats(const Shape& s, const void* q, const void* k, const int32_t* cand,
                               const RefineWs& ws, hipStream_t st);
hipError_t launch_refine_scores(const Shape& s, const void* q, const void* k, const int32_t* cand,
                                const RefineWs& ws, hipStream_t st);
hipError_t launch_refine_select(const Shape& s, const int32_t* cand, const RefineWs& ws, int32_t* topk_idx,
                                float* topk_score, hipStream_t st);
// candidates per refine workgroup (256 for bf16, 64 for fp32)
int refine_tile_of(const Shape& s);
int refine_splits(const Shape& s);
// gather
hipError_t launch_gather(const Shape& s, const void* k, const void* v, const int32_t* idx, void* k_sel, void* v_sel,
                         int32_t* status, hipStream_t st);
hipError_t launch_layout_packed(const Shape& s, const void* packed_k, const void* packed_v, void* k_sel, void* v_sel,
                                hipStream_t st);
// attention
AttnGeom attn_geom(const Shape& s);
// False when the attention work split has too many workgroups for the kernel's 32-bit
// workgroup decode (checked on the host before any launch).
bool attn_fits(const Shape& s);
int attn_splits(const Shape& s);
size_t attn_ws_bytes(const Shape& s);
hipError_t launch_attn(const Shape& s, const void* q, const void* kb, const void* vb, const void* k_sel,
                       const void* v_sel, void* out, void* ws, hipStream_t st);
hipError_t launch_attn_combine(const Shape& s, void* ws, void* out, hipStream_t st);

inline size_t align256(size_t n) { return (n + 255) / 256 * 256; }
inline int64_t vsel_ld(int topk) { return ((int64_t)topk + 63) / 64 * 64; }

}  // namespace herald
