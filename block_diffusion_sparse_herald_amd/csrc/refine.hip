// Stage two of the two-stage selection: refine the C candidates with the B real
// queries into the final top-K subset (HERALD, arXiv 2606.21633 v3, abstract).
//
// Refine score of candidate c of KV head g (the per-row softmax is over the C
// candidates only, summed over the B queries and the G heads of the group):
//   R_g[c] = sum_{b, h in g} 2^(x[b,h,c] - M[b,h]) / Z[b,h],
//   x = scale * log2(e) * <q[b][h], K[cand_c][g]>.
//
// bf16 path, two launches over the same (sequence, KV head, 256-candidate tile)
// grid; both compute x with identical MFMA code, so the logits agree bit for bit:
//   refine_stats_kernel   per row (b,h): (max, sum 2^(x-max)) over the tile
//                         (stored row-major: a row's tiles are contiguous).
//   refine_scores_kernel  per row: normalisers from all tiles; per candidate: the
//                         sum over rows, in a fixed order (each lane over its row's
//                         tiles, then over the 16 lanes of a row with DPP shifts).
// A workgroup covers kRefineTile candidates, each wave 64 of them (four 16-candidate
// MFMA tiles). The candidate key rows, gathered from the cache by index, go straight
// into registers as the A operand; the group's B*G query rows, shared by the waves,
// are streamed into LDS with direct-to-LDS loads and read as the B operand
// (v_mfma_f32_16x16x32_bf16, fp32 accumulate). Only the query rows take LDS (32 KiB
// at B*G = 128, d = 128), so several workgroups share a compute unit and one's loads
// overlap another's products.
// refine_select_kernel then takes, per (sequence, KV head), the exact top-K of R
// in LDS (three radix digits on the fp32 bit pattern, R >= 0), ties to the lower
// cache index, ascending output.
// fp32 path: the same stats / scores / select steps, with the logits on VALU.
#include "common.hpp"
#include "kernels.hpp"

namespace herald {

// 16-byte chunk c of an LDS row r (query row or candidate key row) is stored at chunk
// c ^ refine_swz(r): the 16 rows one MFMA fragment read touches hit distinct banks.
template <int D>
__device__ __forceinline__ int refine_swz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

template <int D>
__device__ __forceinline__ void refine_tile_logits(const uint4 (&a)[4][D / 32], const bf16* qs, int rt, int lane,
                                                   f32x4_t (&acc)[4]) {
  uint4 bq[D / 32];
  const int r = rt * 16 + (lane & 15);
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    bq[ks] = *reinterpret_cast<const uint4*>(qs + r * D + ((ks * 4 + (lane >> 4)) ^ refine_swz<D>(r)) * 8);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) acc[mt] = mfma16x16x32(a[mt][ks], bq[ks], acc[mt]);
  }
}

// Shared prologue of both refine kernels, in two parts. refine_issue_rows: the
// group's query rows go to LDS with coalesced direct-to-LDS loads (rows past R re-read
// query row 0, masked later), and each wave loads the MFMA fragments of its 64
// candidate key rows straight into registers, gathered from the cache by index
// (candidates past C re-read the last one, masked later); every lane reads 16 bytes of
// a row per load, a load covers 64 contiguous bytes of 16 rows. refine_wait_rows:
// once both have landed, the workgroup may read the query rows.
template <int D>
__device__ __forceinline__ void refine_issue_rows(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                  const int32_t* __restrict__ cand, int64_t j0, int s, int g, int B,
                                                  int Hq, int Hkv, int G, int C, int R, int RT, int ctile, bf16* qs,
                                                  uint4 (&a)[4][D / 32]) {
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int RPI = 64 / CPR; // rows per load instruction
  constexpr int NW = kRefineTile / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rr = lane / CPR, p = lane % CPR;
  // query rows: the waves take turns by instruction
  for (int r0 = w * RPI; r0 < RT * 16; r0 += NW * RPI) {
    const int r = r0 + rr;
    const int rq = r < R ? r : 0;
    const bf16* src = q + (((int64_t)s * B + rq / G) * Hq + g * G + rq % G) * D + (p ^ refine_swz<D>(r)) * 8;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(qs + r0 * D), 16, 0, 0);
  }
  // candidate key fragments of wave w: rows w*64 + mt*16 + (lane & 15) of the tile
  const int32_t* cd = cand + ((int64_t)s * Hkv + g) * C;
  const bf16* rows[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int c = min(ctile * kRefineTile + w * 64 + mt * 16 + (lane & 15), C - 1);
    rows[mt] = k + ((j0 + cd[c]) * Hkv + g) * D + (lane >> 4) * 8;
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) a[mt][ks] = *reinterpret_cast<const uint4*>(rows[mt] + ks * 32);
}

__device__ __forceinline__ void refine_wait_rows() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

template <int D>
__global__ __launch_bounds__(kRefineTile) void refine_stats_kernel(const bf16* __restrict__ q,
                                                                   const bf16* __restrict__ k,
                                                                   const int32_t* __restrict__ cand,
                                                                   const int64_t* __restrict__ seq_start, int B,
                                                                   int Hq, int Hkv, int G, int C, float scale2,
                                                                   int ntile, float2* __restrict__ row_stats) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NW = kRefineTile / 64;
  const int tile = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int R = B * G, RT = (R + 15) / 16;
  bf16* qs = reinterpret_cast<bf16*>(smem);                     // [RT*16][D]
  float2* wstat = reinterpret_cast<float2*>(qs + RT * 16 * D);  // [NW][RT*16]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cbase = tile * kRefineTile + w * 64;
  uint4 a[4][D / 32];
  refine_issue_rows<D>(q, k, cand, seq_start[s], s, g, B, Hq, Hkv, G, C, R, RT, tile, qs, a);
  refine_wait_rows();

  const bool full = cbase + 64 <= C;  // no candidate of this wave past C
  for (int rt = 0; rt < RT; ++rt) {
    f32x4_t acc[4];
    refine_tile_logits<D>(a, qs, rt, lane, acc);
    if (!full) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (cbase + mt * 16 + (lane >> 4) * 4 + i >= C) acc[mt][i] = -INFINITY;
    }
    // the row max on the raw products (scale2 > 0), the logits as one fma each
    float mr = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mr = fmaxf(mr, acc[mt][i]);
    mr = xmax4(mr);
    const float m = mr * scale2;
    float l = 0.f;
    if (mr != -INFINITY) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) l += fast_exp2(fmaf(acc[mt][i], scale2, -m));
    }
    l = xsum4(l);
    if (lane < 16) wstat[w * RT * 16 + rt * 16 + lane] = make_float2(m, l);
  }
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += kRefineTile) {
    float M = -INFINITY, Z = 0.f;
    for (int ww = 0; ww < NW; ++ww) {
      const float2 p = wstat[ww * RT * 16 + r];
      ms_merge(M, Z, p.x, p.y);
    }
    row_stats[(((int64_t)s * Hkv + g) * R + r) * ((ntile + 1) & ~1) + tile] = make_float2(M, Z);
  }
}

template <int D>
__global__ __launch_bounds__(kRefineTile) void refine_scores_kernel(const bf16* __restrict__ q,
                                                                    const bf16* __restrict__ k,
                                                                    const int32_t* __restrict__ cand,
                                                                    const int64_t* __restrict__ seq_start, int B,
                                                                    int Hq, int Hkv, int G, int C, float scale2,
                                                                    int ntile, const float2* __restrict__ row_stats,
                                                                    float* __restrict__ rscore) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tile = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int R = B * G, RT = (R + 15) / 16;
  bf16* qs = reinterpret_cast<bf16*>(smem);               // [RT*16][D]
  float* rowM = reinterpret_cast<float*>(qs + RT * 16 * D);  // [RT*16]
  float* rowIZ = rowM + RT * 16;                            // [RT*16]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cbase = tile * kRefineTile + w * 64;
  uint4 a[4][D / 32];
  refine_issue_rows<D>(q, k, cand, seq_start[s], s, g, B, Hq, Hkv, G, C, R, RT, tile, qs, a);
  // per-row normalisers over all tiles, merged in tile order while the rows stream in
  // (a row's tile statistics are contiguous; 16 tiles per batch of loads)
  for (int r = threadIdx.x; r < RT * 16; r += kRefineTile) {
    float M = -INFINITY, Z = 0.f;
    if (r < R) {
      const float2* rs = row_stats + (((int64_t)s * Hkv + g) * R + r) * ((ntile + 1) & ~1);  // 16-byte aligned rows
      for (int t0 = 0; t0 < ntile; t0 += 16) {
        float2 p[16];
#pragma unroll
        for (int u = 0; u < 16; u += 2) {
          if (t0 + u + 1 < ntile) {
            const float4 v = *reinterpret_cast<const float4*>(rs + t0 + u);
            p[u] = make_float2(v.x, v.y);
            p[u + 1] = make_float2(v.z, v.w);
          } else {
            p[u] = t0 + u < ntile ? rs[t0 + u] : make_float2(-INFINITY, 0.f);
            p[u + 1] = make_float2(-INFINITY, 0.f);
          }
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) ms_merge(M, Z, p[u].x, p[u].y);
      }
    }
    // rows past R: a reference far above any logit and a zero weight, so they add 0
    rowM[r] = r < R ? M : 3.0e38f;
    rowIZ[r] = r < R ? 1.f / Z : 0.f;
  }
  refine_wait_rows();

  float rs[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[mt][i] = 0.f;
  for (int rt = 0; rt < RT; ++rt) {
    f32x4_t acc[4];
    refine_tile_logits<D>(a, qs, rt, lane, acc);
    const int r = rt * 16 + (lane & 15);
    const float M = rowM[r], iz = rowIZ[r];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) rs[mt][i] = fmaf(fast_exp2(fmaf(acc[mt][i], scale2, -M)), iz, rs[mt][i]);
  }
  // each lane summed its query row over the row tiles; now sum the 16 rows of a lane row
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[mt][i] = row_sum16_last(rs[mt][i]);
  if ((lane & 15) == 15) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = cbase + mt * 16 + (lane >> 4) * 4 + i;
        if (c < C) rscore[((int64_t)s * Hkv + g) * C + c] = rs[mt][i];
      }
  }
}

// Exact top-K of the refine scores of one (sequence, KV head): three radix digits
// (11, 11, 10 bits of the fp32 pattern, R >= 0), ties to the lower position, ascending
// output. STAGED (C <= kMaxCandidates): scores and candidate indices stay in registers
// (topk_load's layout: each wave a contiguous range of positions), the histograms take
// LDS atomics and the picks are ordered by wave scans in LDS, then written out. Otherwise (candidate sets up to the
// whole sequence) the passes read them from global memory.
template <bool STAGED>
__global__ __launch_bounds__(1024) void refine_select_kernel(const int32_t* __restrict__ cand,
                                                            const float* __restrict__ rscore, int Hkv, int C,
                                                            int topk, int32_t* __restrict__ topk_idx,
                                                            float* __restrict__ topk_score) {
  constexpr int NT = 1024;
  const int g = blockIdx.x, s = blockIdx.y;
  __shared__ uint32_t h[kRadixBins];
  __shared__ uint32_t wcnt[NT / 64][2];
  __shared__ uint32_t dig[4];
  const int64_t base = ((int64_t)s * Hkv + g) * C;
  int32_t* out = topk_idx + ((int64_t)s * Hkv + g) * topk;
  float* outs = topk_score ? topk_score + ((int64_t)s * Hkv + g) * topk : nullptr;
  if constexpr (STAGED) {
    constexpr int MAXIT = topk_chunks(kMaxCandidates);
    __shared__ uint32_t h2[kRadixBins], h3[kRadixBins / 2];
    extern __shared__ int32_t picks[];  // [topk] picks, then [topk] scores when they are wanted
    const int tid = threadIdx.x, w = tid >> 6;
    const int nit = topk_chunks(C);
    uint32_t v[MAXIT][4], ix[MAXIT][4];
    topk_load<MAXIT>(rscore + base, C, nit, v);
    topk_load<MAXIT>(cand + base, C, nit, ix);
    for (int i = tid; i < kRadixBins; i += NT) h[i] = h2[i] = 0u;
    if (tid < kRadixBins / 2) h3[tid] = 0u;
    __syncthreads();
    topk_hist<MAXIT>(v, C, nit, 32, 0u, 21, 2047u, h);  // digit 1 (bits 31..21)
    __syncthreads();
    if (w == 0) {
      int d;
      uint32_t above;
      wave_find_digit(h, kRadixBins, (uint32_t)topk, &d, &above);
      if (tid == 0) {
        dig[0] = (uint32_t)d;
        dig[1] = above;
      }
    }
    __syncthreads();
    const uint32_t d1 = dig[0];
    uint32_t want = (uint32_t)topk - dig[1];
    topk_hist_sparse<MAXIT>(v, C, nit, 21, d1, 10, 2047u, h2);  // digit 2 (bits 20..10)
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
    topk_hist_sparse<MAXIT>(v, C, nit, 10, prefix, 0, 1023u, h3);  // digit 3 (bits 9..0)
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
    topk_emit<MAXIT>(v, [&](int it, int c, int) { return (int32_t)ix[it][c]; }, C, nit, thr, ties,
                     h3[dig[0]] == ties, (uint32_t)topk, picks, outs ? reinterpret_cast<float*>(picks + topk) : nullptr,
                     out, outs, wcnt);
  } else {
    const uint32_t* u = reinterpret_cast<const uint32_t*>(rscore + base);
    uint32_t ties;
    const uint32_t thr = lds_radix_threshold<NT>(u, C, (uint32_t)topk, h, dig, false, &ties);
    lds_emit<NT / 64>(u, C, thr, ties, cand + base, out, outs, wcnt);
  }
}

// fp32 path: candidate key rows of one TILE-candidate tile into LDS (row stride LD
// floats), NT threads: every candidate index is loaded first, then every row chunk,
// then the LDS stores, so the loads overlap instead of waiting one by one.
template <int D, int LD, int NT, int TILE>
__device__ __forceinline__ void stage_rows_f32(const float* __restrict__ k, const int32_t* __restrict__ cd,
                                               int64_t j0, int Hkv, int g, int C, int tile, float* dst) {
  constexpr int NI = TILE * D / 4 / NT;  // 16-byte chunks per thread
  static_assert(NI * NT == TILE * D / 4, "whole chunks per thread");
  int32_t idx[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int row = (threadIdx.x + u * NT) / (D / 4);
    idx[u] = cd[min(tile * TILE + row, C - 1)];
  }
  float4 v[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int ch = (threadIdx.x + u * NT) % (D / 4);
    v[u] = *reinterpret_cast<const float4*>(k + ((j0 + idx[u]) * Hkv + g) * D + 4 * ch);
  }
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int i = threadIdx.x + u * NT;
    *reinterpret_cast<float4*>(dst + (i / (D / 4)) * LD + 4 * (i % (D / 4))) = v[u];
  }
}

// fp32 path: the same three steps on VALU (stats over kRefineTileF32-candidate tiles,
// scores over kRefineScoreTileF32-candidate tiles, then refine_select_kernel). A logit is one fma chain over the head dimension
// in index order; fma is symmetric in its two factors, so the two kernels, which read
// the operands from different places, compute the same bits.
template <int D>
__device__ __forceinline__ void dot4_f32(const float (&reg)[D], const float* o0, const float* o1, const float* o2,
                                         const float* o3, float (&d)[4]) {
  d[0] = d[1] = d[2] = d[3] = 0.f;
#pragma unroll
  for (int e = 0; e < D; e += 4) {
    const float4 a = *reinterpret_cast<const float4*>(o0 + e);
    const float4 b = *reinterpret_cast<const float4*>(o1 + e);
    const float4 c = *reinterpret_cast<const float4*>(o2 + e);
    const float4 f = *reinterpret_cast<const float4*>(o3 + e);
    d[0] = fmaf(reg[e + 3], a.w, fmaf(reg[e + 2], a.z, fmaf(reg[e + 1], a.y, fmaf(reg[e], a.x, d[0]))));
    d[1] = fmaf(reg[e + 3], b.w, fmaf(reg[e + 2], b.z, fmaf(reg[e + 1], b.y, fmaf(reg[e], b.x, d[1]))));
    d[2] = fmaf(reg[e + 3], c.w, fmaf(reg[e + 2], c.z, fmaf(reg[e + 1], c.y, fmaf(reg[e], c.x, d[2]))));
    d[3] = fmaf(reg[e + 3], f.w, fmaf(reg[e + 2], f.z, fmaf(reg[e + 1], f.y, fmaf(reg[e], f.x, d[3]))));
  }
}

// The same chains with both operands in LDS: one row p (per lane) against four rows
// o0..o3 (broadcast).
template <int D>
__device__ __forceinline__ void dot4_lds_f32(const float* p, const float* o0, const float* o1, const float* o2,
                                             const float* o3, float (&d)[4]) {
  d[0] = d[1] = d[2] = d[3] = 0.f;
#pragma unroll 4
  for (int e = 0; e < D; e += 4) {
    const float4 r = *reinterpret_cast<const float4*>(p + e);
    const float4 a = *reinterpret_cast<const float4*>(o0 + e);
    const float4 b = *reinterpret_cast<const float4*>(o1 + e);
    const float4 c = *reinterpret_cast<const float4*>(o2 + e);
    const float4 f = *reinterpret_cast<const float4*>(o3 + e);
    d[0] = fmaf(r.w, a.w, fmaf(r.z, a.z, fmaf(r.y, a.y, fmaf(r.x, a.x, d[0]))));
    d[1] = fmaf(r.w, b.w, fmaf(r.z, b.z, fmaf(r.y, b.y, fmaf(r.x, b.x, d[1]))));
    d[2] = fmaf(r.w, c.w, fmaf(r.z, c.z, fmaf(r.y, c.y, fmaf(r.x, c.x, d[2]))));
    d[3] = fmaf(r.w, f.w, fmaf(r.z, f.z, fmaf(r.y, f.y, fmaf(r.x, f.x, d[3]))));
  }
}

template <int D>
__device__ __forceinline__ void load_row_f32(const float* __restrict__ src, float (&reg)[D]) {
#pragma unroll
  for (int e = 0; e < D; e += 4) {
    const float4 v = *reinterpret_cast<const float4*>(src + e);
    reg[e] = v.x;
    reg[e + 1] = v.y;
    reg[e + 2] = v.z;
    reg[e + 3] = v.w;
  }
}

// Per (query row, tile): (max, sum 2^(x-max)) over the tile's candidates. A workgroup
// takes one tile and 64 query rows (blockIdx.x = pass * ntile + tile); lanes are query
// rows (the row in registers); wave w of NW takes candidates w * CPW .. +CPW-1 of the
// tile from LDS (broadcast reads); the waves' pairs are merged in wave order. Eight
// waves at D = 64; four at D = 128, whose 128-float query row needs the register budget
// of one wave per SIMD.
template <int D>
__global__ __launch_bounds__(D == 128 ? 256 : 512) void refine_stats_f32_kernel(const float* __restrict__ q,
                                                               const float* __restrict__ k,
                                                               const int32_t* __restrict__ cand,
                                                               const int64_t* __restrict__ seq_start, int B, int Hq,
                                                               int Hkv, int G, int C, float scale2, int ntile,
                                                               float2* __restrict__ row_stats) {
  constexpr int NW = D == 128 ? 4 : 8, CPW = kRefineTileF32 / NW;
  static_assert(CPW % 4 == 0, "whole groups of four candidates per wave");
  extern __shared__ __align__(16) float ks[];  // [kRefineTileF32][D]
  __shared__ float2 wstat[NW][64];
  const int tile = blockIdx.x % ntile, r0 = blockIdx.x / ntile * 64, g = blockIdx.y, s = blockIdx.z;
  const int R = B * G;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t j0 = seq_start[s];
  const int32_t* cd = cand + ((int64_t)s * Hkv + g) * C;
  const int r = r0 + lane, rq = min(r, R - 1);
  float qr[D];
  load_row_f32<D>(q + (((int64_t)s * B + rq / G) * Hq + g * G + rq % G) * D, qr);
  stage_rows_f32<D, D, NW * 64, kRefineTileF32>(k, cd, j0, Hkv, g, C, tile, ks);
  __syncthreads();
  const int nvalid = min(kRefineTileF32, C - tile * kRefineTileF32);
  {
    float m = -INFINITY, l = 0.f;
#pragma unroll 1
    for (int c0 = w * CPW; c0 < w * CPW + CPW; c0 += 4) {
      float d[4];
      dot4_f32<D>(qr, ks + c0 * D, ks + (c0 + 1) * D, ks + (c0 + 2) * D, ks + (c0 + 3) * D, d);
      float x[4], mg = -INFINITY;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        x[u] = c0 + u < nvalid ? d[u] * scale2 : -INFINITY;
        mg = fmaxf(mg, x[u]);
      }
      if (mg == -INFINITY) continue;
      float lg = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) lg += fast_exp2(x[u] - mg);
      ms_merge(m, l, mg, lg);
    }
    wstat[w][lane] = make_float2(m, l);
  }
  __syncthreads();
  if (threadIdx.x < 64 && r < R) {
    float M = -INFINITY, Z = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) ms_merge(M, Z, wstat[ww][lane].x, wstat[ww][lane].y);
    row_stats[(((int64_t)s * Hkv + g) * R + r) * ((ntile + 1) & ~1) + tile] = make_float2(M, Z);
  }
}

// Per candidate: sum over query rows of 2^(x - M_row) / Z_row (M_row, Z_row merged over
// all statistics tiles). A workgroup takes kRefineScoreTileF32 = 64 candidates; lanes
// are candidates (key rows in LDS, padded by four words so that 16 lanes' 16-byte reads
// cover all banks); of the eight waves, wave w takes rows 8w .. 8w+7 of every 64-row
// pass; the eight waves' sums are added in wave order at the end.
template <int D>
__global__ __launch_bounds__(512) void refine_scores_f32_kernel(const float* __restrict__ q,
                                                                const float* __restrict__ k,
                                                                const int32_t* __restrict__ cand,
                                                                const int64_t* __restrict__ seq_start, int B,
                                                                int Hq, int Hkv, int G, int C, float scale2, int ntile,
                                                                const float2* __restrict__ row_stats,
                                                                float* __restrict__ rscore) {
  constexpr int KP = D + 4, TS = kRefineScoreTileF32;
  static_assert(TS == 64, "one candidate per lane");
  extern __shared__ __align__(16) float qs[];  // [64][D], [TS][KP], rowM[R], rowIZ[R]
  __shared__ float part[8][TS];
  const int tile = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int R = B * G;
  float* kt = qs + 64 * D;
  float* rowM = kt + TS * KP;
  float* rowIZ = rowM + R;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ci = lane;
  const int64_t j0 = seq_start[s];
  const int32_t* cd = cand + ((int64_t)s * Hkv + g) * C;
  stage_rows_f32<D, KP, 512, TS>(k, cd, j0, Hkv, g, C, tile, kt);
  for (int r = threadIdx.x; r < R; r += 512) {
    const float2* st = row_stats + (((int64_t)s * Hkv + g) * R + r) * ((ntile + 1) & ~1);
    float M = -INFINITY, Z = 0.f;
    for (int t0 = 0; t0 < ntile; t0 += 8) {  // eight tile statistics in flight, merged in tile order
      float2 p[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) p[u] = t0 + u < ntile ? st[t0 + u] : make_float2(-INFINITY, 0.f);
#pragma unroll
      for (int u = 0; u < 8; ++u) ms_merge(M, Z, p[u].x, p[u].y);
    }
    rowM[r] = M;
    rowIZ[r] = 1.f / Z;
  }
  float acc = 0.f;
  for (int r0 = 0; r0 < R; r0 += 64) {
    __syncthreads();
    {
      constexpr int NQ = 64 * D / 4 / 512;  // 16-byte chunks per thread, all loads first
      float4 qv[NQ];
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        const int i = threadIdx.x + u * 512, rr = i / (D / 4), ch = i % (D / 4);
        const int rq = min(r0 + rr, R - 1);
        qv[u] = *reinterpret_cast<const float4*>(q + (((int64_t)s * B + rq / G) * Hq + g * G + rq % G) * D + 4 * ch);
      }
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        const int i = threadIdx.x + u * 512;
        *reinterpret_cast<float4*>(qs + (i / (D / 4)) * D + 4 * (i % (D / 4))) = qv[u];
      }
    }
    __syncthreads();
    const int rb = w * 8;
#pragma unroll
    for (int j = rb; j < rb + 8; j += 4) {
      float d[4];
      dot4_lds_f32<D>(kt + ci * KP, qs + j * D, qs + (j + 1) * D, qs + (j + 2) * D, qs + (j + 3) * D, d);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = r0 + j + u;
        if (r < R) acc += fast_exp2(d[u] * scale2 - rowM[r]) * rowIZ[r];
      }
    }
  }
  part[w][ci] = acc;
  __syncthreads();
  if (threadIdx.x < TS) {
    const int cc = tile * TS + threadIdx.x;
    if (cc < C) {
      float sum = part[0][threadIdx.x];
#pragma unroll
      for (int ww = 1; ww < 8; ++ww) sum += part[ww][threadIdx.x];
      rscore[((int64_t)s * Hkv + g) * C + cc] = sum;
    }
  }
}

// ------------------------------------------------------------------ launchers

static size_t refine_smem(const Shape& s, bool stats) {
  const int RT = (s.B * s.G + 15) / 16;
  const size_t rows = (size_t)RT * 16 * s.D * sizeof(bf16);
  return rows + (stats ? (size_t)(kRefineTile / 64) * RT * 16 * sizeof(float2) : (size_t)2 * RT * 16 * sizeof(float));
}

hipError_t launch_refine_stats(const Shape& s, const void* q, const void* k, const int32_t* cand, const RefineWs& ws,
                               hipStream_t st) {
  dim3 grid(ws.ntile, s.Hkv, s.nseq);
  const float scale2 = s.scale * kLog2e;
  const size_t smem = refine_smem(s, true);
  const void* kern = s.D == 128 ? (const void*)refine_stats_kernel<128> : (const void*)refine_stats_kernel<64>;
  hipError_t e = allow_smem(kern, smem);
  if (e != hipSuccess) return e;
  if (s.D == 128)
    klaunch(refine_stats_kernel<128>, grid, kRefineTile, smem, st, (const bf16*)q, (const bf16*)k, cand, s.seq_start, s.B, s.Hq,
                                                      s.Hkv, s.G, s.C, scale2, ws.ntile, ws.row_stats);
  else
    klaunch(refine_stats_kernel<64>, grid, kRefineTile, smem, st, (const bf16*)q, (const bf16*)k, cand, s.seq_start, s.B, s.Hq,
                                                     s.Hkv, s.G, s.C, scale2, ws.ntile, ws.row_stats);
  return hipGetLastError();
}

hipError_t launch_refine_scores(const Shape& s, const void* q, const void* k, const int32_t* cand,
                                const RefineWs& ws, hipStream_t st) {
  dim3 grid(ws.ntile, s.Hkv, s.nseq);
  const float scale2 = s.scale * kLog2e;
  const size_t smem = refine_smem(s, false);
  const void* kern = s.D == 128 ? (const void*)refine_scores_kernel<128> : (const void*)refine_scores_kernel<64>;
  hipError_t e = allow_smem(kern, smem);
  if (e != hipSuccess) return e;
  if (s.D == 128)
    klaunch(refine_scores_kernel<128>, grid, kRefineTile, smem, st, (const bf16*)q, (const bf16*)k, cand, s.seq_start, s.B,
                                                       s.Hq, s.Hkv, s.G, s.C, scale2, ws.ntile, ws.row_stats,
                                                       ws.rscore);
  else
    klaunch(refine_scores_kernel<64>, grid, kRefineTile, smem, st, (const bf16*)q, (const bf16*)k, cand, s.seq_start, s.B,
                                                      s.Hq, s.Hkv, s.G, s.C, scale2, ws.ntile, ws.row_stats,
                                                      ws.rscore);
  return hipGetLastError();
}

hipError_t launch_refine_select(const Shape& s, const int32_t* cand, const RefineWs& ws, int32_t* topk_idx,
                                float* topk_score, hipStream_t st) {
  if (s.C > kMaxCandidates) {
    klaunch(refine_select_kernel<false>, dim3(s.Hkv, s.nseq), 1024, 0, st, cand, ws.rscore, s.Hkv, s.C, s.topk,
            topk_idx, topk_score);
    return hipGetLastError();
  }
  const size_t smem = (size_t)s.topk * sizeof(int32_t) * (topk_score ? 2 : 1);
  hipError_t e = allow_smem((const void*)refine_select_kernel<true>, smem);
  if (e != hipSuccess) return e;
  klaunch(refine_select_kernel<true>, dim3(s.Hkv, s.nseq), 1024, smem, st, cand, ws.rscore, s.Hkv, s.C, s.topk,
          topk_idx, topk_score);
  return hipGetLastError();
}

hipError_t launch_refine_f32(const Shape& s, const void* q, const void* k, const int32_t* cand, const RefineWs& ws,
                             bool stats, hipStream_t st) {
  // stats: one workgroup per (tile, 64-row pass); scores: one per 64-candidate tile, over all rows
  const int npass = (s.B * s.G + 63) / 64;
  const dim3 grid(stats ? ws.ntile * npass : (s.C + kRefineScoreTileF32 - 1) / kRefineScoreTileF32, s.Hkv, s.nseq);
  const float scale2 = s.scale * kLog2e;
  const size_t smem = stats ? (size_t)kRefineTileF32 * s.D * sizeof(float)
                            : ((size_t)64 * s.D + (size_t)kRefineScoreTileF32 * (s.D + 4) + 2 * (size_t)s.B * s.G) *
                                  sizeof(float);
  const void* kern = stats ? (s.D == 128 ? (const void*)refine_stats_f32_kernel<128>
                                         : (const void*)refine_stats_f32_kernel<64>)
                           : (s.D == 128 ? (const void*)refine_scores_f32_kernel<128>
                                         : (const void*)refine_scores_f32_kernel<64>);
  hipError_t e = allow_smem(kern, smem);
  if (e != hipSuccess) return e;
  const float* qf = (const float*)q;
  const float* kf = (const float*)k;
  if (stats) {
    if (s.D == 128)
      klaunch(refine_stats_f32_kernel<128>, grid, 256, smem, st, qf, kf, cand, s.seq_start, s.B, s.Hq, s.Hkv, s.G,
                                                             s.C, scale2, ws.ntile, ws.row_stats);
    else
      klaunch(refine_stats_f32_kernel<64>, grid, 512, smem, st, qf, kf, cand, s.seq_start, s.B, s.Hq, s.Hkv, s.G,
                                                            s.C, scale2, ws.ntile, ws.row_stats);
  } else {
    if (s.D == 128)
      klaunch(refine_scores_f32_kernel<128>, grid, 512, smem, st, qf, kf, cand, s.seq_start, s.B, s.Hq, s.Hkv, s.G,
                                                              s.C, scale2, ws.ntile, ws.row_stats, ws.rscore);
    else
      klaunch(refine_scores_f32_kernel<64>, grid, 512, smem, st, qf, kf, cand, s.seq_start, s.B, s.Hq, s.Hkv, s.G,
                                                             s.C, scale2, ws.ntile, ws.row_stats, ws.rscore);
  }
  return hipGetLastError();
}

}  // namespace herald
