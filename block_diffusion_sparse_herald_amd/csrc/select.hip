// Stage one of the two-stage selection: merged query, full-cache scan, top-C.
//
// HERALD (arXiv 2606.21633 v3, abstract): a single query merged from the block's
// B queries searches the full KV cache and yields the candidates. The per-KV-head
// score is the sum over the group's G query heads of a softmax over the keys
// (SparDA, arXiv 2606.04511, hyper.ai summary, Method section, target-score
// equation), here taken over the whole cache of the sequence.
//
// Kernels, in launch order:
//   merge_kernel      qbar = mean_b q * scale * log2(e) (fp32); also zeroes the
//                     radix histograms.
//   scan_*_kernel     one pass over K: base-2 logits of every (query head, token),
//                     (scan_lds_kernel for large batches, else scan_mfma_kernel)
//                     stored token-major with the group's heads padded to 4 or 8,
//                     and per-chunk (max, sum 2^(x-max)) pairs. HBM-bound: on
//                     MFMA for bf16 caches, on the VALU for fp32 caches.
//   score_hist_kernel per-head normalisers from the pairs, S = sum_h 2^(x-M_h)/Z_h,
//                     first 11-bit radix histogram of the fp32 bit pattern of S.
//   radix_kernel<2>   second 11-bit digit among keys matching the first.
//   radix_kernel<3>   last 10-bit digit; bitmaps of keys above / equal to the
//                     22-bit prefix (wave ballots).
//   emit_kernel       one workgroup per (sequence, KV head): exact threshold from
//                     the three histograms, ties to the lowest indices, ascending
//                     indices from the bitmaps (block-wide prefix counts).
//   topc_lds_kernel   instead of the last three when every sequence's scores fit
//                     in the registers of one workgroup: digits two and three and
//                     the emission on the registers.
// S >= 0, so its IEEE bit pattern orders like its value and radix select is exact.
#include "common.hpp"
#include "kernels.hpp"

namespace herald {

// ------------------------------------------------------------------ merge

template <typename T>
__global__ __launch_bounds__(128) void merge_kernel(const T* __restrict__ q, int B, int Hq, int D, float mul,
                                                    float* __restrict__ qbar, int nmerge, uint32_t* __restrict__ zero,
                                                    int64_t zero_words) {
  const int blk = blockIdx.x;
  if (blk < nmerge) {
    const int s = blk / Hq, h = blk % Hq;
    const int e = threadIdx.x;
    if (e >= D) return;
    const T* p = q + ((int64_t)s * B * Hq + h) * D + e;
    const int64_t step = (int64_t)Hq * D;
    float acc = 0.f;
    int b = 0;
    for (; b + 8 <= B; b += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = to_f32(p[(b + u) * step]);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; b < B; ++b) acc += to_f32(p[b * step]);
    qbar[(int64_t)blk * D + e] = acc * mul;
  } else {
    const int64_t nz = (int64_t)(gridDim.x - nmerge) * blockDim.x;
    for (int64_t i = (int64_t)(blk - nmerge) * blockDim.x + threadIdx.x; i < zero_words; i += nz) zero[i] = 0u;
  }
}

// ------------------------------------------------------------------ scan

// bf16 caches: the merged-query logits as a skinny matrix product on MFMA, so the
// scan stays bound by HBM. Per 16 keys of one KV head and 32 dimensions, one
// v_mfma_f32_16x16x32_bf16 takes the group's query heads as A rows (the fp32
// merged query split into a bf16 high part and a bf16 residual, two MFMAs into
// one fp32 accumulator, relative error ~2^-18) and the keys as B columns, loaded
// straight from the token-major cache (each lane 16 bytes of one key row).
// A workgroup covers kScanTok tokens of one (sequence, KV head); each wave takes
// 64 of them, 16 per MFMA column block, all 16-byte loads issued up front.
// MERGE: the workgroup also forms the merged query of its G heads itself (the B query
// rows of the block summed in B / parts runs per thread while the key rows are in
// flight, the runs added in a fixed order, times mul), in place of merge_kernel, and
// zeroes its share of the radix histograms.
template <int D, bool MERGE>
__global__ __launch_bounds__(256) void scan_mfma_kernel(const bf16* __restrict__ k, const float* __restrict__ qbar,
                                                        const bf16* __restrict__ q, int B, float mul,
                                                        uint32_t* __restrict__ zero, int64_t zero_words,
                                                        const int64_t* __restrict__ seq_start, int Hq, int Hkv, int G,
                                                        int64_t total, int nchunk, float* __restrict__ logits,
                                                        float2* __restrict__ partials) {
  constexpr int KS = D / 32;                 // MFMA contraction steps per key row
  constexpr int NB = kScanTok / (4 * 16);    // 16-key column blocks per wave
  __shared__ float2 red[4][16];
  const int chunk = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  if (MERGE) {  // histograms of the candidate selection, zeroed before any workgroup leaves
    const int64_t wg = ((int64_t)s * gridDim.y + g) * gridDim.x + chunk;
    const int64_t nwg = (int64_t)gridDim.x * gridDim.y * gridDim.z;
    for (int64_t i = wg * 256 + threadIdx.x; i < zero_words; i += nwg * 256) zero[i] = 0u;
  }
  const int64_t j0 = seq_start[s];
  const int64_t L = seq_start[s + 1] - j0;
  const int64_t tok0 = (int64_t)chunk * kScanTok;
  if (tok0 >= L) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 15, kq = lane >> 4;  // MFMA column (key) and contraction quarter of this lane

  // MERGE: (head, 8-dim chunk) items of the merged query, G * D / 8 <= 128, each summed over
  // B / parts query rows by `parts` threads; a thread's first eight rows are in flight
  // together with the key rows (every load unconditional, from a clamped address)
  const int items = G * (D / 8), parts = 256 / items;
  const int qit = threadIdx.x % items, qpt = threadIdx.x / items;
  const int qper = (B + parts - 1) / parts, qb0 = qpt * qper, qb1 = min(B, qb0 + qper);
  const bool qthread = MERGE && qpt < parts;
  const bf16* qsrc = MERGE ? q + ((int64_t)s * B * Hq + g * G + qit / (D / 8)) * D + (qit % (D / 8)) * 8 : nullptr;
  uint4 qv[MERGE ? 8 : 1];
  if (MERGE) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      qv[u] = ld16_or_zero(qsrc + (int64_t)min(qb0 + u, B - 1) * Hq * D, qthread && qb0 + u < qb1);
  }

  // B operand: key rows, all loads of this wave in flight at once
  const int64_t row_stride = (int64_t)Hkv * D;
  const bf16* kbase = k + (j0 * Hkv + g) * D + kq * 8;
  const int64_t wtok0 = tok0 + w * (NB * 16);
  uint4 kb[NB][KS];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int64_t j = wtok0 + b * 16 + n;
    // keys past the sequence re-read its last row: their logits are computed and dropped
    const int64_t jc = j < L ? j : L - 1;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kb[b][ks] = ld16(kbase + jc * row_stride + ks * 32);
  }

  __shared__ __align__(16) float qm[MERGE ? 8 * D : 4];  // merged query of the group's heads (MERGE)
  if (MERGE) {
    __shared__ __align__(16) float part[256 * 8];
    if (qthread) {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
      for (int b = qb0; b < qb1; b += 8) {
        if (b > qb0) {  // rows past the first eight (B / parts > 8)
#pragma unroll
          for (int u = 0; u < 8; ++u) qv[u] = ld16_or_zero(qsrc + (int64_t)min(b + u, B - 1) * Hq * D, b + u < qb1);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t x[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += bf16_lo(x[e]);
            acc[2 * e + 1] += bf16_hi(x[e]);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) part[(qpt * items + qit) * 8 + e] = acc[e];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < G * D; i += 256) {
      const int it2 = i / 8, e = i % 8;
      float x = 0.f;
      for (int p2 = 0; p2 < parts; ++p2) x += part[(p2 * items + it2) * 8 + e];
      qm[i] = x * mul;  // [head][D]: item it2 = head * D/8 + chunk
    }
    __syncthreads();
  }

  // A operand: query head n of the group (rows >= G are zero), dims ks*32 + 8*kq .. +8, hi and lo parts
  uint4 ahi[KS], alo[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float x[8];
    if (n < G) {
      const float* qp = MERGE ? qm + n * D + ks * 32 + kq * 8 : qbar + ((int64_t)s * Hq + g * G + n) * D + ks * 32 + kq * 8;
      const float4 x0 = *reinterpret_cast<const float4*>(qp);
      const float4 x1 = *reinterpret_cast<const float4*>(qp + 4);
      x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w; x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    uint32_t h[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a0 = x[2 * e], a1 = x[2 * e + 1];
      h[e] = pack_bf16x2(a0, a1);
      const float r0 = a0 - __uint_as_float(h[e] << 16), r1 = a1 - __uint_as_float(h[e] & 0xffff0000u);
      lo[e] = pack_bf16x2(r0, r1);
    }
    ahi[ks] = make_uint4(h[0], h[1], h[2], h[3]);
    alo[ks] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }

  // lane holds logits of query heads 4*kq + i (i = 0..3) for key n of each column block;
  // stored token-major, the group's heads padded to 4 or 8 per token
  const int GP = G <= 4 ? 4 : 8;
  float xs[NB][4];  // the logits again, -inf past the sequence or the group's heads
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      acc = mfma16x16x32(ahi[ks], kb[b][ks], acc);
      acc = mfma16x16x32(alo[ks], kb[b][ks], acc);
    }
    const int64_t j = wtok0 + b * 16 + n;
    if (j < L && 4 * kq < GP)
      st16_stream(logits + ((int64_t)g * total + j0 + j) * GP + 4 * kq, make_float4(acc[0], acc[1], acc[2], acc[3]));
#pragma unroll
    for (int i = 0; i < 4; ++i) xs[b][i] = j < L && kq * 4 + i < G ? acc[i] : -INFINITY;
  }
  // (max, sum) per head over the wave's 64 keys: the max over the row of 16 lanes (every
  // lane gets it), each lane's sum of 2^(x - max), the sum over the row; then over the 4
  // waves in order
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float mx = xs[0][i];
#pragma unroll
    for (int b = 1; b < NB; ++b) mx = fmaxf(mx, xs[b][i]);
    mx = row_max16_all(mx);
    float zs = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int b = 0; b < NB; ++b) zs += fast_exp2(xs[b][i] - mx);
    }
    zs = row_sum16_all(zs);
    if (n == 0) red[w][kq * 4 + i] = make_float2(mx, zs);
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float M = -INFINITY, Z = 0.f;
    for (int ww = 0; ww < 4; ++ww) ms_merge(M, Z, red[ww][threadIdx.x].x, red[ww][threadIdx.x].y);
    partials[((int64_t)s * Hq + g * G + threadIdx.x) * nchunk + chunk] = make_float2(M, Z);
  }
}

// Chunk c of a row r of a scan stage is stored at chunk c ^ scan_swz(r): the 16 rows
// one MFMA operand read touches (16 consecutive tokens of one KV head) then fall in
// distinct banks. hshift = log2(Hkv); r >> hshift is the token within the stage.
template <int D>
__device__ __forceinline__ int scan_swz(int r, int hshift) {
  return (r >> hshift) & (D / 8 - 1);
}

// bf16 caches with Hkv in {1, 2, 4, 8}: the same logits (same MFMA sequence per key
// as scan_mfma_kernel), with the cache moved through LDS so that every load
// instruction reads 1 KiB of contiguous cache. A workgroup covers tpc tokens of one
// sequence, all KV heads, in steps of SR cache rows (SR / Hkv tokens x Hkv heads,
// contiguous in the token-major cache): direct-to-LDS loads of the step, one wait,
// every wave's fragments of the step into registers, then the next step's loads are
// issued before this step's products. The cache rows are loaded non-temporal: the
// gigabyte-scale stream then leaves the caches to what the next kernels read (16 x 32K
// and 4 x 128K steps -30 us). Several workgroups share a compute unit, so one's loads
// also overlap another's products. Wave w takes the step's 16-row blocks p = w, w + 4,
// ...; block p is 16 tokens (16 (p / Hkv) ..) of KV head p % Hkv. The logits of the tpc tokens
// collect in LDS and leave at the end as one contiguous run per KV head (small
// scattered stores between the loads cost several times their bytes).
template <int D, int SR>
__global__ __launch_bounds__(256) void scan_lds_kernel(const bf16* __restrict__ k, const float* __restrict__ qbar,
                                                       const int64_t* __restrict__ seq_start, int Hq, int Hkv, int G,
                                                       int64_t total, int tpc, int nchunk, float* __restrict__ logits,
                                                       float2* __restrict__ partials) {
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;      // rows per load instruction
  constexpr int NIS = SR / RPI / 4;  // load instructions per wave per step
  constexpr int NBW = SR / 64;       // 16-row blocks per wave per step
  constexpr int KS = D / 32;
  static_assert(NIS < 64 && NBW % 2 == 0, "step shape");
  __shared__ __align__(16) bf16 rows[SR * D];
  __shared__ float2 red[SR / 16][8];  // (max, sum) per block, per query head of the group
  extern __shared__ __align__(16) float lg[];  // [Hkv][tpc][GP] logits of this workgroup

  const int chunk = blockIdx.x, s = blockIdx.y;
  const int64_t j0 = seq_start[s];
  const int64_t L = seq_start[s + 1] - j0;
  const int64_t tok0 = (int64_t)chunk * tpc;
  if (tok0 >= L) return;
  const int hshift = 31 - __builtin_clz(Hkv);
  const int TS = SR >> hshift;  // tokens per step
  const int nstep = (int)((min((int64_t)tpc, L - tok0) + TS - 1) / TS);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, kq = lane >> 4;
  const int GP = G <= 4 ? 4 : 8;
  const uint32_t lds0 = (uint32_t)(uintptr_t)rows;

  // A operands: blocks w + 4q use KV head (w + 4q) % Hkv, which alternates between
  // two heads (q even / odd)
  uint4 ahi[2][KS], alo[2][KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int gg = (w + 4 * qb) & (Hkv - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8];
      if (n < G) {
        const float* qp = qbar + ((int64_t)s * Hq + gg * G + n) * D + ks * 32 + kq * 8;
        const float4 x0 = *reinterpret_cast<const float4*>(qp);
        const float4 x1 = *reinterpret_cast<const float4*>(qp + 4);
        x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w; x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
      uint32_t h[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a0 = x[2 * e], a1 = x[2 * e + 1];
        h[e] = pack_bf16x2(a0, a1);
        const float r0 = a0 - __uint_as_float(h[e] << 16), r1 = a1 - __uint_as_float(h[e] & 0xffff0000u);
        lo[e] = pack_bf16x2(r0, r1);
      }
      ahi[qb][ks] = make_uint4(h[0], h[1], h[2], h[3]);
      alo[qb][ks] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
  }
  float m[NBW][4], z[NBW][4];
#pragma unroll
  for (int q = 0; q < NBW; ++q)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      m[q][t] = -INFINITY;
      z[q][t] = 0.f;
    }

  const int rr = lane / CPR, pc = lane % CPR;
  // the step's rows into LDS: instruction u of wave w fills rows (4u + w) * RPI ..
  auto issue = [&](int i) {
    const int64_t t0 = tok0 + (int64_t)i * TS;
#pragma unroll
    for (int u = 0; u < NIS; ++u) {
      const int r = (4 * u + w) * RPI + rr;
      const int64_t tok = min(t0 + (r >> hshift), L - 1);
      const bf16* src = k + ((j0 + tok) * Hkv + (r & (Hkv - 1))) * D + ((pc ^ scan_swz<D>(r, hshift)) * 8);
      lds_dma16_nt(src, lds0 + (uint32_t)((4 * u + w) * RPI * D) * 2u);  // read once: not kept in the caches
    }
  };
  issue(0);
  for (int i = 0; i < nstep; ++i) {
    const int64_t t0 = tok0 + (int64_t)i * TS;
    wait_vm<0>();
    __syncthreads();  // step i's rows are in LDS
    // every fragment of the step into registers, then the rows are free for step i + 1,
    // whose loads run while this step's products and softmax do
    uint4 kb[NBW][KS];
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
      const int p = w + 4 * q;
      const int gg = p & (Hkv - 1);
      const int tl = (p >> hshift) * 16 + n;
      const int r = (tl << hshift) + gg;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kb[q][ks] = *reinterpret_cast<const uint4*>(rows + r * D + (((ks * 4 + kq) ^ scan_swz<D>(r, hshift)) * 8));
    }
    __syncthreads();  // every wave has its fragments
    if (i + 1 < nstep) issue(i + 1);
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
      const int p = w + 4 * q;
      const int gg = p & (Hkv - 1);
      const int tl = (p >> hshift) * 16 + n;  // token within the step
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        acc = mfma16x16x32(ahi[q & 1][ks], kb[q][ks], acc);
        acc = mfma16x16x32(alo[q & 1][ks], kb[q][ks], acc);
      }
      const int64_t j = t0 + tl;
      if (j < L) {
        if (4 * kq < GP)
          *reinterpret_cast<float4*>(lg + ((int64_t)gg * tpc + (j - tok0)) * GP + 4 * kq) =
              make_float4(acc[0], acc[1], acc[2], acc[3]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (kq * 4 + t < G) {
            const float x = acc[t];
            if (x > m[q][t]) {
              z[q][t] = z[q][t] * fast_exp2(m[q][t] - x) + 1.f;
              m[q][t] = x;
            } else {
              z[q][t] += fast_exp2(x - m[q][t]);
            }
          }
        }
      }
    }
  }
  // (max, sum) per block and head over the 16 tokens of the lane group: the row max (every
  // lane gets it), each lane's sum rescaled to it, the row sum (DPP, no LDS traffic)
#pragma unroll
  for (int q = 0; q < NBW; ++q)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float M = row_max16_all(m[q][t]);
      const float zz = row_sum16_all(M == -INFINITY ? 0.f : z[q][t] * fast_exp2(m[q][t] - M));
      if (n == 0 && kq * 4 + t < 8) red[w + 4 * q][kq * 4 + t] = make_float2(M, zz);
    }
  __syncthreads();
  // per query head: the blocks of its KV head (p = g, g + Hkv, ...) in order
  if (threadIdx.x < Hkv * G) {
    const int gg = threadIdx.x / G, hh = threadIdx.x % G;
    float M = -INFINITY, Z = 0.f;
    for (int p = gg; p < SR / 16; p += Hkv) ms_merge(M, Z, red[p][hh].x, red[p][hh].y);
    partials[((int64_t)s * Hq + gg * G + hh) * nchunk + chunk] = make_float2(M, Z);
  }
  // the logits, one contiguous run of ntok * GP floats per KV head
  const int n4 = (int)min((int64_t)tpc, L - tok0) * GP / 4;
  for (int gg = 0; gg < Hkv; ++gg) {
    float4* dst = reinterpret_cast<float4*>(logits + ((int64_t)gg * total + j0 + tok0) * GP);
    const float4* src = reinterpret_cast<const float4*>(lg + (int64_t)gg * tpc * GP);
    for (int i = threadIdx.x; i < n4; i += 256) st16_stream(dst + i, src[i]);
  }
}

// fp32 caches: VALU GEMV. 8 lanes share a key row (16-byte loads), the G query
// heads of the row's group are reduced with 3 xor steps. MERGE: as scan_mfma_kernel,
// the merged query of the group formed in the workgroup (16-byte chunks of the B query
// rows summed in runs per thread, the runs added in a fixed order, times mul), and the
// radix histograms zeroed.
template <int D, int MAXG, bool MERGE, int TOK>
__global__ __launch_bounds__(256) void scan_valu_kernel(const float* __restrict__ k, const float* __restrict__ qbar,
                                                        const float* __restrict__ q, int B, float mul,
                                                        uint32_t* __restrict__ zero, int64_t zero_words,
                                                        const int64_t* __restrict__ seq_start, int Hq, int Hkv, int G,
                                                        int64_t total, int nchunk, float* __restrict__ logits,
                                                        float2* __restrict__ partials) {
  constexpr int EPL = 4;             // fp32 elements per 16-byte load
  constexpr int NL = D / (8 * EPL);  // loads per lane per key row
  constexpr int PER = D / 8;         // elements per lane per key row
  constexpr int U = TOK >= 128 ? 4 : TOK / 32;  // key rows in flight per lane
  __shared__ float2 red[32][8];
  const int chunk = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  if (MERGE) {  // histograms of the candidate selection, zeroed before any workgroup leaves
    const int64_t wg = ((int64_t)s * gridDim.y + g) * gridDim.x + chunk;
    const int64_t nwg = (int64_t)gridDim.x * gridDim.y * gridDim.z;
    for (int64_t i = wg * 256 + threadIdx.x; i < zero_words; i += nwg * 256) zero[i] = 0u;
  }
  const int64_t j0 = seq_start[s];
  const int64_t L = seq_start[s + 1] - j0;
  const int64_t tok0 = (int64_t)chunk * TOK;
  if (tok0 >= L) return;
  const int sub = threadIdx.x & 7, slot = threadIdx.x >> 3;

  __shared__ __align__(16) float qm[MERGE ? MAXG * D : 4];  // merged query of the group's heads (MERGE)
  if (MERGE) {
    __shared__ float4 part[256];
    const int items = G * (D / 4), parts = 256 / items;  // (head, 4-dim chunk) items, G * D / 4 <= 256
    const int it = threadIdx.x % items, pt = threadIdx.x / items;
    const int per = (B + parts - 1) / parts, b0 = pt * per, b1 = min(B, b0 + per);
    if (pt < parts) {
      const float* src = q + ((int64_t)s * B * Hq + g * G + it / (D / 4)) * D + (it % (D / 4)) * 4;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int b = b0; b < b1; b += 8) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = b + u < b1 ? *reinterpret_cast<const float4*>(src + (int64_t)(b + u) * Hq * D) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          acc.x += v[u].x;
          acc.y += v[u].y;
          acc.z += v[u].z;
          acc.w += v[u].w;
        }
      }
      part[pt * items + it] = acc;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < G * D; i += 256) {
      float x = 0.f;
      for (int p2 = 0; p2 < parts; ++p2) {
        const float4 pv = part[p2 * items + i / 4];
        x += (i & 3) == 0 ? pv.x : (i & 3) == 1 ? pv.y : (i & 3) == 2 ? pv.z : pv.w;
      }
      qm[i] = x * mul;  // [head][D]
    }
    __syncthreads();
  }

  float qr[MAXG][PER];
#pragma unroll
  for (int hh = 0; hh < MAXG; ++hh)
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        qr[hh][i * EPL + e] = hh >= G ? 0.f
                              : MERGE ? qm[hh * D + (i * 8 + sub) * EPL + e]
                                      : qbar[((int64_t)s * Hq + g * G + hh) * D + (i * 8 + sub) * EPL + e];

  const int64_t row_stride = (int64_t)Hkv * D;
  const float* kbase = k + (j0 * Hkv + g) * D;
  float m = -INFINITY, ssum = 0.f;
  for (int it = 0; it < TOK / 32; it += U) {
    uint4 v[U][NL];
    int64_t jj[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      jj[u] = tok0 + (it + u) * 32 + slot;
#pragma unroll
      for (int i = 0; i < NL; ++i)
        v[u][i] = ld16(kbase + (jj[u] < L ? jj[u] : L - 1) * row_stride + (i * 8 + sub) * EPL);  // past L: dropped
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc[MAXG];
#pragma unroll
      for (int hh = 0; hh < MAXG; ++hh) acc[hh] = 0.f;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        float f[EPL];
        Vec16<float>::unpack(v[u][i], f);
#pragma unroll
        for (int e = 0; e < EPL; ++e)
#pragma unroll
          for (int hh = 0; hh < MAXG; ++hh) acc[hh] = fmaf(qr[hh][i * EPL + e], f[e], acc[hh]);
      }
      // sum over the 8 lanes sharing the row: quad swaps 1 and 2, then the half-row mirror
      // (DPP, no LDS traffic; every lane gets the same sum, paired as an xor butterfly)
#pragma unroll
      for (int hh = 0; hh < MAXG; ++hh) {
        float a = acc[hh];
        a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0xB1, 0xf, 0xf, false));  // quad_perm 1,0,3,2
        a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x4E, 0xf, 0xf, false));  // quad_perm 2,3,0,1
        a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x141, 0xf, 0xf, false));  // row_half_mirror
        acc[hh] = a;
      }
      float x = acc[0];
#pragma unroll
      for (int hh = 1; hh < MAXG; ++hh)
        if (sub == hh) x = acc[hh];
      if (sub < G && jj[u] < L) {
        logits[((int64_t)g * total + j0 + jj[u]) * (G <= 4 ? 4 : 8) + sub] = x;
        if (x > m) {
          ssum = ssum * fast_exp2(m - x) + 1.f;
          m = x;
        } else {
          ssum += fast_exp2(x - m);
        }
      }
    }
  }
  red[slot][sub] = make_float2(m, ssum);
  __syncthreads();
  if (threadIdx.x < G) {
    float M = -INFINITY, S = 0.f;
    for (int sl = 0; sl < 32; ++sl) ms_merge(M, S, red[sl][threadIdx.x].x, red[sl][threadIdx.x].y);
    partials[((int64_t)s * Hq + g * G + threadIdx.x) * nchunk + chunk] = make_float2(M, S);
  }
}

// ------------------------------------------------------------------ score + first radix digit

template <int GP, int TOK>
__global__ __launch_bounds__(256) void score_hist_kernel(const float* __restrict__ logits,
                                                         const float2* __restrict__ partials,
                                                         const int64_t* __restrict__ seq_start, int Hq, int Hkv,
                                                         int G, int64_t total, int nchunk, int tpc,
                                                         float* __restrict__ scores, uint32_t* __restrict__ hist) {
  const int chunk = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int64_t j0 = seq_start[s];
  const int64_t L = seq_start[s + 1] - j0;
  const int64_t tok0 = (int64_t)chunk * TOK;
  if (tok0 >= L) return;
  constexpr int IT = TOK / 256;
  __shared__ uint32_t h[kRadixBins];
  __shared__ float2 red[4][GP];
  __shared__ float Msh[GP], invZ[GP];

  // Loads first: this thread's first chunk statistics per head, then the workgroup's
  // logits (token-major, GP heads per token). The memory counter is in order, so with
  // the statistics issued first the normaliser merge below starts while the logits
  // are still in flight.
  const int nc = (int)((L + tpc - 1) / tpc);
  float2 p0[GP];
#pragma unroll
  for (int hh = 0; hh < GP; ++hh)
    p0[hh] = hh < G && (int)threadIdx.x < nc ? partials[((int64_t)s * Hq + g * G + hh) * nchunk + threadIdx.x]
                                              : make_float2(-INFINITY, 0.f);
  float4 lv[IT][GP / 4];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t j = min(tok0 + it * 256 + threadIdx.x, L - 1);
#pragma unroll
    for (int c = 0; c < GP / 4; ++c)
      lv[it][c] = *reinterpret_cast<const float4*>(logits + ((int64_t)g * total + j0 + j) * GP + 4 * c);
  }
  for (int i = threadIdx.x; i < kRadixBins; i += 256) h[i] = 0u;

  // per-head normalisers over the whole sequence, same order in every workgroup
  float m[GP], z[GP];
#pragma unroll
  for (int hh = 0; hh < GP; ++hh) {
    m[hh] = -INFINITY;
    z[hh] = 0.f;
    ms_merge(m[hh], z[hh], p0[hh].x, p0[hh].y);
  }
  for (int c = threadIdx.x + 256; c < nc; c += 256) {
    float2 p[GP];
#pragma unroll
    for (int hh = 0; hh < GP; ++hh)
      p[hh] = hh < G ? partials[((int64_t)s * Hq + g * G + hh) * nchunk + c] : make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int hh = 0; hh < GP; ++hh) ms_merge(m[hh], z[hh], p[hh].x, p[hh].y);
  }
#pragma unroll
  for (int hh = 0; hh < GP; ++hh) {
    ms_wave_merge(m[hh], z[hh]);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6][hh] = make_float2(m[hh], z[hh]);
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float M = -INFINITY, Z = 0.f;
    for (int w = 0; w < 4; ++w) ms_merge(M, Z, red[w][threadIdx.x].x, red[w][threadIdx.x].y);
    Msh[threadIdx.x] = M;
    invZ[threadIdx.x] = 1.f / Z;
  }
  __syncthreads();

#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t j = tok0 + it * 256 + threadIdx.x;
    if (j < L) {
      const float* x = reinterpret_cast<const float*>(&lv[it][0]);
      float S = 0.f;
#pragma unroll
      for (int hh = 0; hh < GP; ++hh)
        if (hh < G) S += fast_exp2(x[hh] - Msh[hh]) * invZ[hh];
      scores[(int64_t)g * total + j0 + j] = S;
      atomicAdd(&h[__float_as_uint(S) >> 21], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = hist + (int64_t)(s * Hkv + g) * 3 * kRadixBins;
  for (int i = threadIdx.x; i < kRadixBins; i += 256)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// ------------------------------------------------------------------ radix passes 2 and 3

template <int PASS, int TOK>
__global__ __launch_bounds__(256) void radix_kernel(const float* __restrict__ scores,
                                                    const int64_t* __restrict__ seq_start, int Hkv, int64_t total,
                                                    int C, int nwords, uint32_t* __restrict__ hist,
                                                    uint64_t* __restrict__ bits) {
  const int chunk = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int64_t j0 = seq_start[s];
  const int64_t L = seq_start[s + 1] - j0;
  const int64_t tok0 = (int64_t)chunk * TOK;
  if (tok0 >= L) return;
  __shared__ uint32_t h[kRadixBins];                // this pass
  __shared__ uint32_t prev[(PASS - 1) * kRadixBins];  // the finished histograms of the earlier passes
  __shared__ uint32_t dig[2];
  uint32_t* gh = hist + (int64_t)(s * Hkv + g) * 3 * kRadixBins;
  const float* sc = scores + (int64_t)g * total + j0;

  // issue the score loads first; they do not depend on the digits
  constexpr int IT = TOK / 256;
  uint32_t u[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t j = tok0 + it * 256 + threadIdx.x;
    u[it] = j < L ? __float_as_uint(sc[j]) : 0u;
  }
  for (int i = threadIdx.x; i < kRadixBins; i += 256) h[i] = 0u;
  for (int i = threadIdx.x; i < (PASS - 1) * kRadixBins / 4; i += 256)
    reinterpret_cast<uint4*>(prev)[i] = reinterpret_cast<const uint4*>(gh)[i];
  __syncthreads();
  if (threadIdx.x < 64) {
    int d1, d2 = 0;
    uint32_t a1, a2;
    wave_find_digit(prev, kRadixBins, (uint32_t)C, &d1, &a1);
    if (PASS == 3) wave_find_digit(prev + kRadixBins, kRadixBins, (uint32_t)C - a1, &d2, &a2);
    if (threadIdx.x == 0) {
      dig[0] = (uint32_t)d1;
      dig[1] = (uint32_t)d2;
    }
  }
  __syncthreads();
  const uint32_t d1 = dig[0];
  const uint32_t prefix = (dig[0] << 11) | dig[1];
  uint64_t* gt_bits = bits + (int64_t)(s * Hkv + g) * 2 * nwords;
  uint64_t* eq_bits = gt_bits + nwords;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;

#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t j = tok0 + it * 256 + threadIdx.x;
    const bool valid = j < L;
    if (PASS == 2) {
      if (valid && (u[it] >> 21) == d1) atomicAdd(&h[(u[it] >> 10) & 2047u], 1u);
    } else {
      const uint32_t top = u[it] >> 10;
      const bool eq = valid && top == prefix;
      const bool gt = valid && top > prefix;
      if (eq) atomicAdd(&h[u[it] & 1023u], 1u);
      const uint64_t bg = __ballot(gt), be = __ballot(eq);
      const int64_t w0 = tok0 + it * 256 + wid * 64;
      if (lane == 0 && w0 < L) {
        gt_bits[w0 >> 6] = bg;
        eq_bits[w0 >> 6] = be;
      }
    }
  }
  __syncthreads();
  uint32_t* out = gh + (PASS - 1) * kRadixBins;
  for (int i = threadIdx.x; i < kRadixBins; i += 256)
    if (h[i]) atomicAdd(&out[i], h[i]);
}

// ------------------------------------------------------------------ emit

// One workgroup per (sequence, KV head). Words of the prefix bitmaps are handled in
// rounds of 4 per thread; ties (keys equal to the threshold) are kept lowest index
// first, and the final indices come out in ascending order. The picks of a round are
// not written by the thread that owns their word (selected tokens cluster, so a few
// threads would own most of them): each word's mask and first output position go to
// LDS, with an anchor per 64 output slots (the word that holds the slot), and thread t
// fills slots t, t + 1024, ..., eight at a time: a branch-free binary search between
// the two anchors around the slot finds its word, a select of the set bits its token.
__global__ __launch_bounds__(1024) void emit_kernel(const float* __restrict__ scores,
                                                   const int64_t* __restrict__ seq_start, int Hkv, int64_t total,
                                                   int C, int nwords, const uint32_t* __restrict__ hist,
                                                   const uint64_t* __restrict__ bits, int32_t* __restrict__ cand,
                                                   float* __restrict__ cand_score) {
  constexpr int NT = 1024, WPT = 4;
  const int g = blockIdx.x, s = blockIdx.y;
  const int64_t j0 = seq_start[s];
  const int64_t L = seq_start[s + 1] - j0;
  __shared__ uint32_t hs[3 * kRadixBins];
  __shared__ uint32_t lds[NT / 64 + 4];
  extern __shared__ uint64_t wmask[];  // [NT * WPT] selected bits per word, then [NT * WPT] u32 first positions,
                                       // then [NT * WPT * 64 / 64 + 1] u32 anchors
  uint32_t* wpos = reinterpret_cast<uint32_t*>(wmask + NT * WPT);
  uint32_t* anchor = wpos + NT * WPT;
  const uint32_t* gh = hist + (int64_t)(s * Hkv + g) * 3 * kRadixBins;
  for (int i = threadIdx.x; i < 3 * kRadixBins / 4; i += NT)
    reinterpret_cast<uint4*>(hs)[i] = reinterpret_cast<const uint4*>(gh)[i];
  __syncthreads();
  if (threadIdx.x < 64) {
    uint32_t thr, ties;
    wave_threshold(hs, (uint32_t)C, &thr, &ties);
    if (threadIdx.x == 0) {
      lds[NT / 64 + 1] = thr & 1023u;
      lds[NT / 64 + 2] = ties;
    }
  }
  __syncthreads();
  const uint32_t d3 = lds[NT / 64 + 1];
  const uint32_t ties_wanted = lds[NT / 64 + 2];

  const uint64_t* gt_bits = bits + (int64_t)(s * Hkv + g) * 2 * nwords;
  const uint64_t* eq_bits = gt_bits + nwords;
  const float* sc = scores + (int64_t)g * total + j0;
  int32_t* out = cand + (int64_t)(s * Hkv + g) * C;
  float* outs = cand_score ? cand_score + (int64_t)(s * Hkv + g) * C : nullptr;
  const int64_t nw = (L + 63) >> 6;
  uint32_t tie_base = 0, pos_base = 0;
  for (int64_t r0 = 0; r0 < nw; r0 += (int64_t)NT * WPT) {
    const int64_t w0 = r0 + (int64_t)threadIdx.x * WPT;
    uint64_t gt[WPT], eq[WPT];
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      gt[i] = w0 + i < nw ? gt_bits[w0 + i] : 0ull;
      eq[i] = w0 + i < nw ? eq_bits[w0 + i] : 0ull;
    }
    // keys on the 22-bit prefix: above the threshold's last digit go in, equal ones are ties
    uint64_t tie[WPT];
    uint32_t my_ties = 0;
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      tie[i] = 0ull;
      uint64_t x = eq[i];
      while (x) {
        const int b = __builtin_ctzll(x);
        x &= x - 1;
        const uint32_t low = __float_as_uint(sc[((w0 + i) << 6) + b]) & 1023u;
        if (low > d3) gt[i] |= 1ull << b;
        else if (low == d3) tie[i] |= 1ull << b;
      }
      my_ties += (uint32_t)__builtin_popcountll(tie[i]);
    }
    uint32_t tot;
    uint32_t tie_rank = tie_base + block_exclusive_scan<NT>(my_ties, lds, &tot);
    tie_base += tot;
    uint32_t my_sel = 0;
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      uint64_t x = tie[i];
      while (x) {
        const int b = __builtin_ctzll(x);
        x &= x - 1;
        if (tie_rank < ties_wanted) gt[i] |= 1ull << b;
        ++tie_rank;
      }
      my_sel += (uint32_t)__builtin_popcountll(gt[i]);
    }
    uint32_t pos = pos_base + block_exclusive_scan<NT>(my_sel, lds, &tot);
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const uint32_t n = (uint32_t)__builtin_popcountll(gt[i]);
      wmask[threadIdx.x * WPT + i] = gt[i];
      wpos[threadIdx.x * WPT + i] = pos;
      // anchors: the word that holds every 64th slot of the round
      for (uint32_t a = (pos - pos_base + 63) & ~63u; a < pos - pos_base + n; a += 64)
        anchor[a >> 6] = threadIdx.x * WPT + i;
      pos += n;
    }
    __syncthreads();
    const int nwr = (int)min((int64_t)NT * WPT, nw - r0);  // words of this round
    const uint32_t qend = min(pos_base + tot, (uint32_t)C);
    constexpr int U = 8;
    for (uint32_t q0 = pos_base + threadIdx.x; q0 < qend; q0 += NT * U) {
      int lo[U], hi[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // slot q lies between the anchors of its 64-slot block and of the next one
        const uint32_t k = (q0 + u * NT - pos_base) >> 6;
        const bool in = q0 + u * NT < qend;
        lo[u] = in ? (int)anchor[k] : 0;
        hi[u] = in && pos_base + (k + 1) * 64 < pos_base + tot ? (int)anchor[k + 1] : nwr - 1;
        hi[u] = in ? hi[u] : 0;
      }
      // the last word whose first position is <= q holds slot q (it cannot be empty:
      // the next word's first position is above q)
#pragma unroll 1
      for (int step = 0; step < 13; ++step) {
        bool open = false;
#pragma unroll
        for (int u = 0; u < U; ++u) open |= lo[u] < hi[u];
        if (!__ballot(open)) break;
        uint32_t pm[U];
#pragma unroll
        for (int u = 0; u < U; ++u) pm[u] = wpos[(lo[u] + hi[u] + 1) >> 1];  // all reads of the step together
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int mid = (lo[u] + hi[u] + 1) >> 1;  // == lo once lo == hi: no change then
          const bool le = pm[u] <= q0 + u * NT;
          lo[u] = le ? mid : lo[u];
          hi[u] = le ? hi[u] : mid - 1;
        }
      }
      int32_t idx[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t m = wmask[lo[u]];
        uint32_t kk = q0 + u * NT - wpos[lo[u]];  // the slot's rank among the word's set bits
        // select the kk-th set bit: halve the word five times, then the last pair
        uint32_t x = (uint32_t)m, base = 0;
        uint32_t c = (uint32_t)__builtin_popcount(x);
        const bool up = kk >= c;
        kk = up ? kk - c : kk;
        x = up ? (uint32_t)(m >> 32) : x;
        base = up ? 32u : 0u;
#pragma unroll
        for (int sh = 16; sh >= 1; sh >>= 1) {
          c = (uint32_t)__builtin_popcount(x & ((1u << sh) - 1u));
          const bool hi2 = kk >= c;
          kk = hi2 ? kk - c : kk;
          x = hi2 ? x >> sh : x;
          base += hi2 ? (uint32_t)sh : 0u;
        }
        idx[u] = (int32_t)(((r0 + lo[u]) << 6) + base);
      }
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = (outs && q0 + u * NT < qend) ? sc[idx[u]] : 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t q = q0 + u * NT;
        if (q < qend) {
          out[q] = idx[u];
          if (outs) outs[q] = v[u];
        }
      }
    }
    pos_base += tot;
    __syncthreads();  // the next round rewrites the word masks
  }
}

// ------------------------------------------------------------------ top-C in registers

// One 1024-thread workgroup per (sequence, KV head) of up to kTopcLdsMaxLen tokens: the
// scores stay in registers (each wave a contiguous range of tokens, see topk_load),
// the first digit comes from the histogram score_hist_kernel built (read by wave 0
// while the score loads are in flight), digits two and three from LDS histograms of
// the keys that match the digits found so far, and the candidates are collected in
// ascending order in LDS through wave scans, then written out. Replaces radix_kernel<2>, radix_kernel<3> and emit_kernel.
__global__ __launch_bounds__(1024) void topc_lds_kernel(const float* __restrict__ scores,
                                                       const int64_t* __restrict__ seq_start, int Hkv,
                                                       int64_t total, int C, const uint32_t* __restrict__ hist,
                                                       int32_t* __restrict__ cand, float* __restrict__ cand_score) {
  constexpr int MAXIT = topk_chunks(kTopcLdsMaxLen);
  __shared__ uint32_t h2[kRadixBins], h3[kRadixBins / 2];
  __shared__ uint32_t wcnt[kTopkWaves][2];
  __shared__ uint32_t dig[4];
  extern __shared__ int32_t picks[];  // [C + kTopkSlack] candidates, then as many scores when they are wanted
  const int g = blockIdx.x, s = blockIdx.y;
  const int64_t j0 = seq_start[s];
  const int L = (int)(seq_start[s + 1] - j0);
  const int tid = threadIdx.x, w = tid >> 6;
  const int nit = topk_chunks(L);
  const float* sc = scores + (int64_t)g * total + j0;

  uint32_t v[MAXIT][4];
  topk_load<MAXIT>(sc, L, nit, v);
  for (int i = tid; i < kRadixBins; i += 1024) h2[i] = 0u;
  if (tid < kRadixBins / 2) h3[tid] = 0u;
  if (w == 0) {  // digit 1 (bits 31..21)
    int d;
    uint32_t above;
    wave_find_digit(hist + (int64_t)(s * Hkv + g) * 3 * kRadixBins, kRadixBins, (uint32_t)C, &d, &above);
    if (tid == 0) {
      dig[0] = (uint32_t)d;
      dig[1] = above;
    }
  }
  __syncthreads();
  const uint32_t d1 = dig[0];
  uint32_t want = (uint32_t)C - dig[1];
  topk_hist_sparse<MAXIT>(v, L, nit, 21, d1, 10, 2047u, h2);  // digit 2 (bits 20..10)
  __syncthreads();
  if (w == 0) {
    int d;
    uint32_t above;
    wave_find_digit(h2, kRadixBins, want, &d, &above);
    if (tid == 0) {
      dig[2] = (uint32_t)d;
      dig[3] = above;
    }
  }
  __syncthreads();
  want -= dig[3];
  const uint32_t prefix = (d1 << 11) | dig[2];
  topk_hist_sparse<MAXIT>(v, L, nit, 10, prefix, 0, 1023u, h3);  // digit 3 (bits 9..0)
  __syncthreads();
  if (w == 0) {
    int d;
    uint32_t above;
    wave_find_digit(h3, kRadixBins / 2, want, &d, &above);
    if (tid == 0) {
      dig[0] = (uint32_t)d;
      dig[1] = above;
    }
  }
  __syncthreads();
  const uint32_t thr = (prefix << 10) | dig[0];
  const uint32_t ties = want - dig[1];
  float* outs = cand_score ? cand_score + (int64_t)(s * Hkv + g) * C : nullptr;
  topk_emit<MAXIT>(v, [](int, int, int pos) { return (int32_t)pos; }, L, nit, thr, ties, h3[dig[0]] == ties,
                   (uint32_t)C, picks, outs ? reinterpret_cast<float*>(picks + C + kTopkSlack) : nullptr,
                   cand + (int64_t)(s * Hkv + g) * C, outs, wcnt);
}

// ------------------------------------------------------------------ launchers

hipError_t launch_merge(const Shape& s, const void* q, const SelectWs& ws, hipStream_t st) {
  const int nmerge = s.nseq * s.Hq;
  const int64_t zero_words = (int64_t)s.nseq * s.Hkv * 3 * kRadixBins;
  const int nz = (int)std::min<int64_t>(256, (zero_words + 127) / 128);
  const float mul = s.scale * kLog2e / (float)s.B;
  if (s.bf16)
    klaunch(merge_kernel<bf16>, nmerge + nz, 128, 0, st, (const bf16*)q, s.B, s.Hq, s.D, mul, ws.qbar, nmerge, ws.hist,
                                                    zero_words);
  else
    klaunch(merge_kernel<float>, nmerge + nz, 128, 0, st, (const float*)q, s.B, s.Hq, s.D, mul, ws.qbar, nmerge, ws.hist,
                                                     zero_words);
  return hipGetLastError();
}

static int maxg_of(int G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8; }

// The LDS-staged scan streams faster once there are enough workgroups to keep
// several on every compute unit; below that the register-load scan, with its 8x more
// workgroups (one KV head each), finishes sooner. Measured ahead with 8 KV heads and,
// since its cache rows are loaded non-temporal, with 4 (8 ragged sequences of
// 16K-64K tokens, 28/4 heads: step 880.9 -> 871.3 us); the kernel also takes 1 and 2
// KV heads, not measured, so those stay on the register scan.
static bool scan_in_lds(const Shape& s) {
  return s.bf16 && (s.Hkv == 8 || s.Hkv == 4) && s.G <= 8 && s.total >= (int64_t)4 * 256 * kScanTok;
}

// The merge inside the scan costs every scan workgroup a little; it pays only while
// there are few of them (measured: ahead at 1024 workgroups, behind at ~5200).
bool scan_merges_query(const Shape& s) {
  const int64_t nwg = (s.max_len + kScanTok - 1) / kScanTok * s.Hkv * s.nseq;
  return !scan_in_lds(s) && nwg <= 2048;
}

hipError_t launch_scan(const Shape& s, const void* k, const SelectWs& ws, hipStream_t st, const void* q, int nq) {
  dim3 grid(ws.nchunk, s.Hkv, s.nseq);
  if (scan_in_lds(s)) {
    const size_t smem = (size_t)s.Hkv * ws.tpc * (s.G <= 4 ? 4 : 8) * sizeof(float);
    const void* kern = s.D == 128 ? (const void*)scan_lds_kernel<128, 128> : (const void*)scan_lds_kernel<64, 128>;
    hipError_t e = allow_smem(kern, smem);
    if (e != hipSuccess) return e;
    if (s.D == 128)
      klaunch(scan_lds_kernel<128, 128>, dim3(ws.nchunk, s.nseq), 256, smem, st, (const bf16*)k, ws.qbar, s.seq_start,
              s.Hq, s.Hkv, s.G, s.total, ws.tpc, ws.nchunk, ws.logits, ws.partials);
    else
      klaunch(scan_lds_kernel<64, 128>, dim3(ws.nchunk, s.nseq), 256, smem, st, (const bf16*)k, ws.qbar, s.seq_start,
              s.Hq, s.Hkv, s.G, s.total, ws.tpc, ws.nchunk, ws.logits, ws.partials);
    return hipGetLastError();
  }
  // with q: the merged query formed inside the scan (scan_merges_query), no merge_kernel
  const bool merge = q != nullptr;
  const int nq1 = merge ? nq : 1;
  const float mul = s.scale * kLog2e / (float)nq1;
  const int64_t zero_words = merge ? (int64_t)s.nseq * s.Hkv * 3 * kRadixBins : 0;
  if (s.bf16) {
    auto kern = s.D == 128 ? (merge ? scan_mfma_kernel<128, true> : scan_mfma_kernel<128, false>)
                           : (merge ? scan_mfma_kernel<64, true> : scan_mfma_kernel<64, false>);
    klaunch(kern, grid, 256, 0, st, (const bf16*)k, ws.qbar, (const bf16*)q, nq1, mul, ws.hist, zero_words,
            s.seq_start, s.Hq, s.Hkv, s.G, s.total, ws.nchunk, ws.logits, ws.partials);
    return hipGetLastError();
  }
#define HERALD_SCAN_CASE(GG)                                                                                       \
  case GG:                                                                                                         \
    if (s.D == 128)                                                                                                \
      klaunch(small ? (merge ? scan_valu_kernel<128, GG, true, kScanTokSmall> : scan_valu_kernel<128, GG, false, kScanTokSmall>) \
                    : (merge ? scan_valu_kernel<128, GG, true, kScanTok> : scan_valu_kernel<128, GG, false, kScanTok>),      \
              grid, 256, 0, st, (const float*)k, ws.qbar, (const float*)q, nq1, mul, ws.hist, zero_words, s.seq_start,      \
              s.Hq, s.Hkv, s.G, s.total, ws.nchunk, ws.logits, ws.partials);                                              \
    else                                                                                                           \
      klaunch(small ? (merge ? scan_valu_kernel<64, GG, true, kScanTokSmall> : scan_valu_kernel<64, GG, false, kScanTokSmall>)   \
                    : (merge ? scan_valu_kernel<64, GG, true, kScanTok> : scan_valu_kernel<64, GG, false, kScanTok>),        \
              grid, 256, 0, st, (const float*)k, ws.qbar, (const float*)q, nq1, mul, ws.hist, zero_words, s.seq_start,      \
              s.Hq, s.Hkv, s.G, s.total, ws.nchunk, ws.logits, ws.partials);                                              \
    break;
  if (ws.tpc != kScanTok && ws.tpc != kScanTokSmall) return hipErrorInvalidValue;
  const bool small = ws.tpc == kScanTokSmall;
  switch (maxg_of(s.G)) {
    HERALD_SCAN_CASE(1)
    HERALD_SCAN_CASE(2)
    HERALD_SCAN_CASE(4)
    HERALD_SCAN_CASE(8)
  }
#undef HERALD_SCAN_CASE
  return hipGetLastError();
}

// Tokens per score workgroup: 2048 on large caches, 256 on small ones (a few thousand
// (token, KV head) pairs would otherwise make a handful of workgroups), else 1024. The
// small size never reaches the radix passes (sequences past the register top-C are longer).
static int score_tok(const Shape& s) {
  if (s.total >= kScoreTokLargeFrom) return kScoreTokLarge;
  return s.total * s.Hkv <= kScoreTokSmallUpTo ? kScoreTokSmall : kScoreTok;
}
static int score_chunks(const Shape& s) { return (int)((s.max_len + score_tok(s) - 1) / score_tok(s)); }

hipError_t launch_score_hist(const Shape& s, const SelectWs& ws, hipStream_t st) {
  dim3 grid(score_chunks(s), s.Hkv, s.nseq);
  const int tok = score_tok(s);
  auto kern = s.G <= 4 ? (tok == kScoreTokLarge ? score_hist_kernel<4, kScoreTokLarge>
                          : tok == kScoreTokSmall ? score_hist_kernel<4, kScoreTokSmall> : score_hist_kernel<4, kScoreTok>)
                       : (tok == kScoreTokLarge ? score_hist_kernel<8, kScoreTokLarge>
                          : tok == kScoreTokSmall ? score_hist_kernel<8, kScoreTokSmall> : score_hist_kernel<8, kScoreTok>);
  klaunch(kern, grid, 256, 0, st, ws.logits, ws.partials, s.seq_start, s.Hq, s.Hkv, s.G, s.total, ws.nchunk, ws.tpc,
          ws.scores, ws.hist);
  return hipGetLastError();
}

hipError_t launch_radix_pass(const Shape& s, const SelectWs& ws, int pass, hipStream_t st) {
  if (score_tok(s) == kScoreTokSmall) return hipErrorInvalidValue;  // small caches take the register top-C
  dim3 grid(score_chunks(s), s.Hkv, s.nseq);
  const bool large = score_tok(s) == kScoreTokLarge;
  auto kern = pass == 2 ? (large ? radix_kernel<2, kScoreTokLarge> : radix_kernel<2, kScoreTok>)
                        : (large ? radix_kernel<3, kScoreTokLarge> : radix_kernel<3, kScoreTok>);
  klaunch(kern, grid, 256, 0, st, ws.scores, s.seq_start, s.Hkv, s.total, s.C, ws.nwords, ws.hist, ws.bits);
  return hipGetLastError();
}

bool topc_in_lds(const Shape& s) { return s.max_len <= kTopcLdsMaxLen; }

hipError_t launch_topc_lds(const Shape& s, const SelectWs& ws, int32_t* cand, float* cand_score, hipStream_t st) {
  const size_t smem = (size_t)(s.C + kTopkSlack) * sizeof(int32_t) * (cand_score ? 2 : 1);
  hipError_t e = allow_smem((const void*)topc_lds_kernel, smem);
  if (e != hipSuccess) return e;
  klaunch(topc_lds_kernel, dim3(s.Hkv, s.nseq), 1024, smem, st, ws.scores, s.seq_start, s.Hkv, s.total, s.C, ws.hist,
          cand, cand_score);
  return hipGetLastError();
}

hipError_t launch_emit_candidates(const Shape& s, const SelectWs& ws, int32_t* cand, float* cand_score,
                                  hipStream_t st) {
  // word masks and positions, and one anchor per 64 slots (a round has at most 4096 * 64 slots)
  const size_t smem = (size_t)1024 * 4 * (sizeof(uint64_t) + sizeof(uint32_t)) + (size_t)(4096 + 1) * sizeof(uint32_t);
  hipError_t e = allow_smem((const void*)emit_kernel, smem);
  if (e != hipSuccess) return e;
  klaunch(emit_kernel, dim3(s.Hkv, s.nseq), 1024, smem, st, ws.scores, s.seq_start, s.Hkv, s.total, s.C, ws.nwords,
          ws.hist, ws.bits, cand, cand_score);
  return hipGetLastError();
}

}  // namespace herald
