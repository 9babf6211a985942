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
//   scan_kernel       one pass over K: base-2 logits of every (query head, token)
//                     and per-chunk (max, sum 2^(x-max)) pairs. HBM-bound GEMV:
//                     8 lanes share a 256-byte key row (two 128-byte coalesced
//                     loads), G query heads per row, 3-step xor reduction.
//   score_hist_kernel per-head normalisers from the pairs, S = sum_h 2^(x-M_h)/Z_h,
//                     first 11-bit radix histogram of the fp32 bit pattern of S.
//   radix_kernel<2>   second 11-bit digit among keys matching the first.
//   radix_kernel<3>   last 10-bit digit; bitmaps of keys above / equal to the
//                     22-bit prefix (wave ballots).
//   emit_kernel       exact threshold, ties to the lowest indices, ascending
//                     indices from the bitmaps (block-wide prefix counts).
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
    for (int e = threadIdx.x; e < D; e += blockDim.x) {
      float acc = 0.f;
      for (int b = 0; b < B; ++b) acc += to_f32(q[(((int64_t)s * B + b) * Hq + h) * D + e]);
      qbar[(int64_t)blk * D + e] = acc * mul;
    }
  } else {
    const int64_t nz = (int64_t)(gridDim.x - nmerge) * blockDim.x;
    for (int64_t i = (int64_t)(blk - nmerge) * blockDim.x + threadIdx.x; i < zero_words; i += nz) zero[i] = 0u;
  }
}

// ------------------------------------------------------------------ scan

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void scan_kernel(const T* __restrict__ k, const float* __restrict__ qbar,
                                                   const int64_t* __restrict__ seq_start, int Hq, int Hkv,
                                                   int64_t total, int nchunk, float* __restrict__ logits,
                                                   float2* __restrict__ partials) {
  constexpr int EPL = Vec16<T>::N;   // elements per 16-byte load
  constexpr int NL = D / (8 * EPL);  // loads per lane per key row
  constexpr int PER = D / 8;         // elements per lane per key row
  constexpr int U = 4;               // key rows in flight per lane
  static_assert(NL >= 1 && PER == NL * EPL, "row split");
  const int chunk = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int64_t j0 = seq_start[s];
  const int64_t L = seq_start[s + 1] - j0;
  const int64_t tok0 = (int64_t)chunk * kScanTok;
  if (tok0 >= L) return;
  const int sub = threadIdx.x & 7, slot = threadIdx.x >> 3;

  float qr[G][PER];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        qr[hh][i * EPL + e] = qbar[((int64_t)s * Hq + g * G + hh) * D + (i * 8 + sub) * EPL + e];

  const int64_t row_stride = (int64_t)Hkv * D;
  const T* kbase = k + (j0 * Hkv + g) * D;
  float m = -INFINITY, ssum = 0.f;

  for (int it = 0; it < kScanTok / 32; it += U) {
    uint4 v[U][NL];
    int64_t jj[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      jj[u] = tok0 + (it + u) * 32 + slot;
#pragma unroll
      for (int i = 0; i < NL; ++i)
        v[u][i] = jj[u] < L ? ld16(kbase + jj[u] * row_stride + (i * 8 + sub) * EPL) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) acc[hh] = 0.f;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        float f[EPL];
        Vec16<T>::unpack(v[u][i], f);
#pragma unroll
        for (int e = 0; e < EPL; ++e)
#pragma unroll
          for (int hh = 0; hh < G; ++hh) acc[hh] = fmaf(qr[hh][i * EPL + e], f[e], acc[hh]);
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) acc[hh] += __shfl_xor(acc[hh], o);
      float x = acc[0];
#pragma unroll
      for (int hh = 1; hh < G; ++hh)
        if (sub == hh) x = acc[hh];
      if (sub < G && jj[u] < L) {
        logits[(int64_t)(g * G + sub) * total + j0 + jj[u]] = x;
        if (x > m) {
          ssum = ssum * fast_exp2(m - x) + 1.f;
          m = x;
        } else {
          ssum += fast_exp2(x - m);
        }
      }
    }
  }

  __shared__ float2 red[32][8];
  red[slot][sub] = make_float2(m, ssum);
  __syncthreads();
  if (threadIdx.x < G) {
    float M = -INFINITY, S = 0.f;
    for (int sl = 0; sl < 32; ++sl) ms_merge(M, S, red[sl][threadIdx.x].x, red[sl][threadIdx.x].y);
    partials[((int64_t)s * Hq + g * G + threadIdx.x) * nchunk + chunk] = make_float2(M, S);
  }
}

// ------------------------------------------------------------------ score + first radix digit

template <int G>
__global__ __launch_bounds__(256) void score_hist_kernel(const float* __restrict__ logits,
                                                         const float2* __restrict__ partials,
                                                         const int64_t* __restrict__ seq_start, int Hq, int Hkv,
                                                         int64_t total, int nchunk, float* __restrict__ scores,
                                                         uint32_t* __restrict__ hist) {
  const int chunk = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int64_t j0 = seq_start[s];
  const int64_t L = seq_start[s + 1] - j0;
  const int64_t tok0 = (int64_t)chunk * kScoreTok;
  if (tok0 >= L) return;
  __shared__ uint32_t h[kRadixBins];
  __shared__ float2 red[4][G];
  __shared__ float Msh[G], invZ[G];
  for (int i = threadIdx.x; i < kRadixBins; i += 256) h[i] = 0u;

  // per-head normalisers over the whole sequence, same order in every workgroup
  const int nc = (int)((L + kScanTok - 1) / kScanTok);
  float m[G], z[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    z[hh] = 0.f;
  }
  for (int c = threadIdx.x; c < nc; c += 256)
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float2 p = partials[((int64_t)s * Hq + g * G + hh) * nchunk + c];
      ms_merge(m[hh], z[hh], p.x, p.y);
    }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
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

  for (int it = 0; it < kScoreTok / 256; ++it) {
    const int64_t j = tok0 + it * 256 + threadIdx.x;
    if (j < L) {
      float S = 0.f;
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
        S += fast_exp2(logits[(int64_t)(g * G + hh) * total + j0 + j] - Msh[hh]) * invZ[hh];
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

template <int PASS>
__global__ __launch_bounds__(256) void radix_kernel(const float* __restrict__ scores,
                                                    const int64_t* __restrict__ seq_start, int Hkv, int64_t total,
                                                    int C, int nwords, uint32_t* __restrict__ hist,
                                                    uint64_t* __restrict__ bits) {
  const int chunk = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int64_t j0 = seq_start[s];
  const int64_t L = seq_start[s + 1] - j0;
  const int64_t tok0 = (int64_t)chunk * kScoreTok;
  if (tok0 >= L) return;
  __shared__ uint32_t h[kRadixBins];
  __shared__ uint32_t lds[16];
  for (int i = threadIdx.x; i < kRadixBins; i += 256) h[i] = 0u;
  uint32_t* gh = hist + (int64_t)(s * Hkv + g) * 3 * kRadixBins;
  int d1, d2 = 0;
  uint32_t a1, a2;
  find_digit<256>(gh, kRadixBins, (uint32_t)C, lds, &d1, &a1);
  if (PASS == 3) find_digit<256>(gh + kRadixBins, kRadixBins, (uint32_t)C - a1, lds, &d2, &a2);
  const uint32_t prefix = ((uint32_t)d1 << 11) | (uint32_t)d2;
  uint64_t* gt_bits = bits + (int64_t)(s * Hkv + g) * 2 * nwords;
  uint64_t* eq_bits = gt_bits + nwords;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;

  for (int it = 0; it < kScoreTok / 256; ++it) {
    const int64_t j = tok0 + it * 256 + threadIdx.x;
    const bool valid = j < L;
    const uint32_t u = valid ? __float_as_uint(scores[(int64_t)g * total + j0 + j]) : 0u;
    if (PASS == 2) {
      if (valid && (u >> 21) == (uint32_t)d1) atomicAdd(&h[(u >> 10) & 2047u], 1u);
    } else {
      const uint32_t top = u >> 10;
      const bool eq = valid && top == prefix;
      const bool gt = valid && top > prefix;
      if (eq) atomicAdd(&h[u & 1023u], 1u);
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

__global__ __launch_bounds__(1024) void emit_kernel(const float* __restrict__ scores,
                                                   const int64_t* __restrict__ seq_start, int Hkv, int64_t total,
                                                   int C, int nwords, const uint32_t* __restrict__ hist,
                                                   uint64_t* __restrict__ bits, int32_t* __restrict__ cand,
                                                   float* __restrict__ cand_score) {
  const int g = blockIdx.x, s = blockIdx.y;
  const int64_t j0 = seq_start[s];
  const int64_t L = seq_start[s + 1] - j0;
  __shared__ uint32_t lds[32];
  const uint32_t* gh = hist + (int64_t)(s * Hkv + g) * 3 * kRadixBins;
  int d1, d2, d3;
  uint32_t a1, a2, a3;
  find_digit<1024>(gh, kRadixBins, (uint32_t)C, lds, &d1, &a1);
  const uint32_t k1 = (uint32_t)C - a1;
  find_digit<1024>(gh + kRadixBins, kRadixBins, k1, lds, &d2, &a2);
  const uint32_t k2 = k1 - a2;
  find_digit<1024>(gh + 2 * kRadixBins, 1024, k2, lds, &d3, &a3);
  const uint32_t ties_wanted = k2 - a3;  // keys equal to the threshold to keep, lowest indices first

  uint64_t* gt_bits = bits + (int64_t)(s * Hkv + g) * 2 * nwords;
  const uint64_t* eq_bits = gt_bits + nwords;
  const float* sc = scores + (int64_t)g * total + j0;
  const int64_t nw = (L + 63) >> 6;
  const int64_t wpt = (nw + 1023) / 1024;
  const int64_t w0 = (int64_t)threadIdx.x * wpt;
  const int64_t w1 = min(nw, w0 + wpt);

  // pass A: ties owned by this thread (keys on the 22-bit prefix whose last digit is d3)
  uint32_t my_ties = 0;
  for (int64_t w = w0; w < w1; ++w) {
    uint64_t x = eq_bits[w];
    while (x) {
      const int b = __builtin_ctzll(x);
      x &= x - 1;
      if ((__float_as_uint(sc[(w << 6) + b]) & 1023u) == (uint32_t)d3) ++my_ties;
    }
  }
  uint32_t tot;
  uint32_t tie_rank = block_exclusive_scan<1024>(my_ties, lds, &tot);

  // pass B: final membership word by word (written over the above-prefix bitmap)
  uint32_t my_sel = 0;
  for (int64_t w = w0; w < w1; ++w) {
    uint64_t sel = gt_bits[w];
    uint64_t x = eq_bits[w];
    while (x) {
      const int b = __builtin_ctzll(x);
      x &= x - 1;
      const uint32_t low = __float_as_uint(sc[(w << 6) + b]) & 1023u;
      if (low > (uint32_t)d3) {
        sel |= 1ull << b;
      } else if (low == (uint32_t)d3) {
        if (tie_rank < ties_wanted) sel |= 1ull << b;
        ++tie_rank;
      }
    }
    gt_bits[w] = sel;
    my_sel += (uint32_t)__builtin_popcountll(sel);
  }
  uint32_t pos = block_exclusive_scan<1024>(my_sel, lds, &tot);

  // pass C: ascending indices
  int32_t* out = cand + (int64_t)(s * Hkv + g) * C;
  float* outs = cand_score ? cand_score + (int64_t)(s * Hkv + g) * C : nullptr;
  for (int64_t w = w0; w < w1; ++w) {
    uint64_t x = gt_bits[w];
    while (x) {
      const int b = __builtin_ctzll(x);
      x &= x - 1;
      if (pos < (uint32_t)C) {
        const int64_t j = (w << 6) + b;
        out[pos] = (int32_t)j;
        if (outs) outs[pos] = sc[j];
      }
      ++pos;
    }
  }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_merge(const Shape& s, const void* q, const SelectWs& ws, hipStream_t st) {
  const int nmerge = s.nseq * s.Hq;
  const int64_t zero_words = (int64_t)s.nseq * s.Hkv * 3 * kRadixBins;
  const int nz = (int)std::min<int64_t>(256, (zero_words + 127) / 128);
  const float mul = s.scale * kLog2e / (float)s.B;
  if (s.bf16)
    merge_kernel<bf16><<<nmerge + nz, 128, 0, st>>>((const bf16*)q, s.B, s.Hq, s.D, mul, ws.qbar, nmerge, ws.hist,
                                                    zero_words);
  else
    merge_kernel<float><<<nmerge + nz, 128, 0, st>>>((const float*)q, s.B, s.Hq, s.D, mul, ws.qbar, nmerge, ws.hist,
                                                     zero_words);
  return hipGetLastError();
}

template <typename T, int D>
static void scan_dispatch_g(const Shape& s, const void* k, const SelectWs& ws, hipStream_t st) {
  dim3 grid(ws.nchunk, s.Hkv, s.nseq);
#define HERALD_SCAN_CASE(GG)                                                                                  \
  case GG:                                                                                                    \
    scan_kernel<T, D, GG><<<grid, 256, 0, st>>>((const T*)k, ws.qbar, s.seq_start, s.Hq, s.Hkv, s.total,      \
                                                ws.nchunk, ws.logits, ws.partials);                           \
    break;
  switch (s.G) {
    HERALD_SCAN_CASE(1)
    HERALD_SCAN_CASE(2)
    HERALD_SCAN_CASE(3)
    HERALD_SCAN_CASE(4)
    HERALD_SCAN_CASE(5)
    HERALD_SCAN_CASE(6)
    HERALD_SCAN_CASE(7)
    HERALD_SCAN_CASE(8)
  }
#undef HERALD_SCAN_CASE
}

hipError_t launch_scan(const Shape& s, const void* k, const SelectWs& ws, hipStream_t st) {
  if (s.bf16) {
    if (s.D == 128) scan_dispatch_g<bf16, 128>(s, k, ws, st);
    else scan_dispatch_g<bf16, 64>(s, k, ws, st);
  } else {
    if (s.D == 128) scan_dispatch_g<float, 128>(s, k, ws, st);
    else scan_dispatch_g<float, 64>(s, k, ws, st);
  }
  return hipGetLastError();
}

static int score_chunks(const Shape& s) { return (int)((s.max_len + kScoreTok - 1) / kScoreTok); }

hipError_t launch_score_hist(const Shape& s, const SelectWs& ws, hipStream_t st) {
  dim3 grid(score_chunks(s), s.Hkv, s.nseq);
#define HERALD_SCORE_CASE(GG)                                                                                    \
  case GG:                                                                                                       \
    score_hist_kernel<GG><<<grid, 256, 0, st>>>(ws.logits, ws.partials, s.seq_start, s.Hq, s.Hkv, s.total,      \
                                                ws.nchunk, ws.scores, ws.hist);                                  \
    break;
  switch (s.G) {
    HERALD_SCORE_CASE(1)
    HERALD_SCORE_CASE(2)
    HERALD_SCORE_CASE(3)
    HERALD_SCORE_CASE(4)
    HERALD_SCORE_CASE(5)
    HERALD_SCORE_CASE(6)
    HERALD_SCORE_CASE(7)
    HERALD_SCORE_CASE(8)
  }
#undef HERALD_SCORE_CASE
  return hipGetLastError();
}

hipError_t launch_radix_pass(const Shape& s, const SelectWs& ws, int pass, hipStream_t st) {
  dim3 grid(score_chunks(s), s.Hkv, s.nseq);
  if (pass == 2)
    radix_kernel<2><<<grid, 256, 0, st>>>(ws.scores, s.seq_start, s.Hkv, s.total, s.C, ws.nwords, ws.hist, ws.bits);
  else
    radix_kernel<3><<<grid, 256, 0, st>>>(ws.scores, s.seq_start, s.Hkv, s.total, s.C, ws.nwords, ws.hist, ws.bits);
  return hipGetLastError();
}

hipError_t launch_emit_candidates(const Shape& s, const SelectWs& ws, int32_t* cand, float* cand_score,
                                  hipStream_t st) {
  emit_kernel<<<dim3(s.Hkv, s.nseq), 1024, 0, st>>>(ws.scores, s.seq_start, s.Hkv, s.total, s.C, ws.nwords, ws.hist,
                                                    ws.bits, cand, cand_score);
  return hipGetLastError();
}

}  // namespace herald
