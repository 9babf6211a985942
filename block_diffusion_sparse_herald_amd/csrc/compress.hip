// Compressed keys and block-granular selection over them.
//
// SparDA (arXiv 2606.04511, hyper.ai summary, Method section): block-level relevance
// is computed against keys mean-pooled into overlapping compressed representations.
// Here block m of a sequence owns tokens [m*stride, (m+1)*stride) (the last block may
// be short); its compressed key is the mean of the keys in the window
// [m*stride, m*stride + ksize), cut at the end of the sequence. The compressed cache
// is fp32, [sum_s ceil(L_s / stride)][Hkv][d], sequences concatenated in order.
//
// Kernels:
//   compress_kernel     the compressed cache from the token cache (fp32 sums in token
//                       order, one division).
//   coffsets_kernel     compressed row offsets of the sequences (prefix over nseq).
//   expand_hist_kernel  token score = its block's score; first 11-bit radix histogram
//                       of the token scores, so the exact top-C of the selection path
//                       runs unchanged on them (whole blocks in score order, the
//                       boundary block from its lowest token up).
// The block scores themselves come from the selection path's scan and score kernels
// run over the compressed cache (scan_valu_kernel, score_hist_kernel).
#include "common.hpp"
#include "kernels.hpp"

namespace herald {

// First compressed row of sequence s: sum over t < s of ceil(L_t / stride), summed by
// the 256 threads of the workgroup (each a strided part, then through LDS).
__device__ __forceinline__ int64_t compressed_offset(const int64_t* __restrict__ seq_start, int s, int stride) {
  __shared__ int64_t part[256];
  int64_t off = 0;
  for (int t = threadIdx.x; t < s; t += 256) off += (seq_start[t + 1] - seq_start[t] + stride - 1) / stride;
  part[threadIdx.x] = off;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  return part[0];
}

// Four blocks per workgroup of one (sequence, KV head), 64 threads per block, each
// thread D/64 consecutive dimensions.
template <typename T, int D>
__global__ __launch_bounds__(256) void compress_kernel(const T* __restrict__ k, const int64_t* __restrict__ seq_start,
                                                       int Hkv, int ksize, int stride, float* __restrict__ k_comp) {
  constexpr int EPT = D / 64;
  const int g = blockIdx.y, s = blockIdx.z;
  const int64_t j0 = seq_start[s];
  const int64_t L = seq_start[s + 1] - j0;
  const int64_t M = (L + stride - 1) / stride;
  if ((int64_t)blockIdx.x * 4 >= M) return;  // whole workgroup past this sequence's blocks
  const int64_t cbase = compressed_offset(seq_start, s, stride);
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const int e0 = (threadIdx.x & 63) * EPT;
  const int64_t a = m * stride, b = min(a + (int64_t)ksize, L);
  float acc[EPT];
#pragma unroll
  for (int t = 0; t < EPT; ++t) acc[t] = 0.f;
  for (int64_t j = a; j < b; ++j) {
    const T* row = k + ((j0 + j) * Hkv + g) * D + e0;
#pragma unroll
    for (int t = 0; t < EPT; ++t) acc[t] += to_f32(row[t]);
  }
  const float n = (float)(b - a);
  float* out = k_comp + ((cbase + m) * Hkv + g) * D + e0;
#pragma unroll
  for (int t = 0; t < EPT; ++t) out[t] = acc[t] / n;
}

// One thread: coff[s] = sum over t < s of ceil(L_t / stride), s = 0..nseq.
__global__ void coffsets_kernel(const int64_t* __restrict__ seq_start, int nseq, int stride,
                                int64_t* __restrict__ coff) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  int64_t off = 0;
  for (int s = 0; s < nseq; ++s) {
    coff[s] = off;
    off += (seq_start[s + 1] - seq_start[s] + stride - 1) / stride;
  }
  coff[nseq] = off;
}

// kScoreTok tokens of one (sequence, KV head) per workgroup.
__global__ __launch_bounds__(256) void expand_hist_kernel(const float* __restrict__ s_blk,
                                                          const int64_t* __restrict__ seq_start,
                                                          const int64_t* __restrict__ coff, int Hkv, int64_t total,
                                                          int64_t ctotal, int stride, float* __restrict__ scores,
                                                          uint32_t* __restrict__ hist) {
  const int chunk = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int64_t j0 = seq_start[s];
  const int64_t L = seq_start[s + 1] - j0;
  const int64_t tok0 = (int64_t)chunk * kScoreTok;
  if (tok0 >= L) return;
  __shared__ uint32_t h[kRadixBins];
  for (int i = threadIdx.x; i < kRadixBins; i += 256) h[i] = 0u;
  __syncthreads();
  const float* sb = s_blk + (int64_t)g * ctotal + coff[s];
  for (int64_t j = tok0 + threadIdx.x; j < min(tok0 + kScoreTok, L); j += 256) {
    const float S = sb[j / stride];
    scores[(int64_t)g * total + j0 + j] = S;
    atomicAdd(&h[__float_as_uint(S) >> 21], 1u);
  }
  __syncthreads();
  uint32_t* gh = hist + (int64_t)(s * Hkv + g) * 3 * kRadixBins;
  for (int i = threadIdx.x; i < kRadixBins; i += 256)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// ------------------------------------------------------------------ launchers

hipError_t launch_compress(const Shape& s, const void* k, int ksize, int stride, float* k_comp, hipStream_t st) {
  const int64_t maxM = (s.max_len + stride - 1) / stride;
  const dim3 grid((unsigned)((maxM + 3) / 4), s.Hkv, s.nseq);
  if (s.bf16) {
    if (s.D == 128)
      klaunch(compress_kernel<bf16, 128>, grid, 256, 0, st, (const bf16*)k, s.seq_start, s.Hkv, ksize, stride, k_comp);
    else
      klaunch(compress_kernel<bf16, 64>, grid, 256, 0, st, (const bf16*)k, s.seq_start, s.Hkv, ksize, stride, k_comp);
  } else {
    if (s.D == 128)
      klaunch(compress_kernel<float, 128>, grid, 256, 0, st, (const float*)k, s.seq_start, s.Hkv, ksize, stride, k_comp);
    else
      klaunch(compress_kernel<float, 64>, grid, 256, 0, st, (const float*)k, s.seq_start, s.Hkv, ksize, stride, k_comp);
  }
  return hipGetLastError();
}

hipError_t launch_coffsets(const Shape& s, int stride, int64_t* coff, hipStream_t st) {
  klaunch(coffsets_kernel, 1, 64, 0, st, s.seq_start, s.nseq, stride, coff);
  return hipGetLastError();
}

hipError_t launch_expand_hist(const Shape& s, const float* s_blk, const int64_t* coff, int64_t ctotal, int stride,
                              const SelectWs& ws, hipStream_t st) {
  const dim3 grid((unsigned)((s.max_len + kScoreTok - 1) / kScoreTok), s.Hkv, s.nseq);
  klaunch(expand_hist_kernel, grid, 256, 0, st, s_blk, s.seq_start, coff, s.Hkv, s.total, ctotal, stride, ws.scores,
          ws.hist);
  return hipGetLastError();
}

}  // namespace herald
