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
// Each wave owns 64 candidates (four 16-candidate MFMA tiles). The candidate key
// rows (gathered from the cache by index) and the group's B*G query rows are
// streamed into LDS with coalesced direct-to-LDS loads; the key rows are the A
// operand (read once into registers), the query rows the B operand
// (v_mfma_f32_16x16x32_bf16, fp32 accumulate).
// refine_select_kernel then takes, per (sequence, KV head), the exact top-K of R
// in LDS (three radix digits on the fp32 bit pattern, R >= 0), ties to the lower
// cache index, ascending output.
// fp32 path: refine_f32_kernel, one workgroup per (sequence, KV head), same top-K.
#include "common.hpp"
#include "kernels.hpp"

namespace herald {

// Exact top-k of u[0..n) (fp32 bit patterns of non-negative scores, in LDS), ties
// to the lower position; writes cand[pos] (or pos when cand is NULL) and the score
// of each pick in ascending position order. h: kRadixBins LDS words; lds: NT/64+3.
template <int NT>
__device__ void lds_topk(const uint32_t* u, int n, int k, uint32_t* h, uint32_t* lds, const int32_t* cand,
                         int32_t* out, float* outs) {
  uint32_t want = (uint32_t)k;
  uint32_t prefix = 0;  // digits found so far
  const int shift[3] = {21, 10, 0};
  const int width[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    for (int i = threadIdx.x; i < kRadixBins; i += NT) h[i] = 0u;
    __syncthreads();
    const int hi_shift = shift[pass] + width[pass];
    const uint32_t mask = (1u << width[pass]) - 1u;
    for (int c = threadIdx.x; c < n; c += NT) {
      const uint32_t v = u[c];
      if (pass == 0 || (v >> hi_shift) == prefix) atomicAdd(&h[(v >> shift[pass]) & mask], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      int d;
      uint32_t above;
      wave_find_digit(h, width[pass] == 11 ? kRadixBins : 1024, want, &d, &above);
      if (threadIdx.x == 0) {
        lds[NT / 64 + 1] = (uint32_t)d;
        lds[NT / 64 + 2] = above;
      }
    }
    __syncthreads();
    want -= lds[NT / 64 + 2];
    prefix = (prefix << width[pass]) | lds[NT / 64 + 1];
    __syncthreads();
  }
  const uint32_t thr = prefix;  // bit pattern of the k-th largest score
  const uint32_t ties_wanted = want;

  const int cpt = (n + NT - 1) / NT;
  const int c0 = threadIdx.x * cpt, c1 = min(n, c0 + cpt);
  uint32_t my_ties = 0;
  for (int c = c0; c < c1; ++c) my_ties += u[c] == thr;
  uint32_t tot;
  const uint32_t tie_rank = block_exclusive_scan<NT>(my_ties, lds, &tot);
  uint32_t my_sel = 0;
  {
    uint32_t tr = tie_rank;
    for (int c = c0; c < c1; ++c) {
      if (u[c] > thr) ++my_sel;
      else if (u[c] == thr) {
        if (tr < ties_wanted) ++my_sel;
        ++tr;
      }
    }
  }
  uint32_t pos = block_exclusive_scan<NT>(my_sel, lds, &tot);
  uint32_t tr = tie_rank;
  for (int c = c0; c < c1; ++c) {
    bool take = false;
    if (u[c] > thr) take = true;
    else if (u[c] == thr) {
      take = tr < ties_wanted;
      ++tr;
    }
    if (take) {
      if (pos < (uint32_t)k) {
        out[pos] = cand ? cand[c] : c;
        if (outs) outs[pos] = __uint_as_float(u[c]);
      }
      ++pos;
    }
  }
}

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
// group's query rows and this workgroup's kRefineTile candidate key rows go to LDS
// with coalesced direct-to-LDS loads (rows past R re-read query row 0, candidates
// past C re-read the last one; both are masked later). refine_key_frags: once the
// loads have landed, each wave reads the key fragments of its 64 candidates into
// registers.
template <int D>
__device__ __forceinline__ void refine_issue_rows(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                  const int32_t* __restrict__ cand, int64_t j0, int s, int g, int B,
                                                  int Hq, int Hkv, int G, int C, int R, int RT, int ctile, bf16* qs,
                                                  bf16* kls) {
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
  // candidate key rows: wave w loads (and later uses) rows w*64 .. w*64+63 of the tile
  const int32_t* cd = cand + ((int64_t)s * Hkv + g) * C;
#pragma unroll
  for (int u = 0; u < 64 / RPI; ++u) {
    const int i = w * 64 + u * RPI + rr;
    const int c = min(ctile * kRefineTile + i, C - 1);
    const bf16* src = k + ((j0 + cd[c]) * Hkv + g) * D + (p ^ refine_swz<D>(i)) * 8;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(kls + (w * 64 + u * RPI) * D), 16, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void refine_key_frags(const bf16* kls, uint4 (&a)[4][D / 32]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int i = w * 64 + mt * 16 + (lane & 15);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      a[mt][ks] = *reinterpret_cast<const uint4*>(kls + i * D + ((ks * 4 + (lane >> 4)) ^ refine_swz<D>(i)) * 8);
  }
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
  bf16* kls = qs + RT * 16 * D;                                 // [kRefineTile][D]
  float2* wstat = reinterpret_cast<float2*>(kls + kRefineTile * D);  // [NW][RT*16]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cbase = tile * kRefineTile + w * 64;
  uint4 a[4][D / 32];
  refine_issue_rows<D>(q, k, cand, seq_start[s], s, g, B, Hq, Hkv, G, C, R, RT, tile, qs, kls);
  refine_key_frags<D>(kls, a);

  for (int rt = 0; rt < RT; ++rt) {
    f32x4_t acc[4];
    refine_tile_logits<D>(a, qs, rt, lane, acc);
    float x[4][4];
    float m = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = cbase + mt * 16 + (lane >> 4) * 4 + i;
        x[mt][i] = c < C ? acc[mt][i] * scale2 : -INFINITY;
        m = fmaxf(m, x[mt][i]);
      }
    m = xmax4(m);
    float l = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) l += fast_exp2(x[mt][i] - m);
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
  bf16* kls = qs + RT * 16 * D;                           // [kRefineTile][D]
  float* rowM = reinterpret_cast<float*>(kls + kRefineTile * D);  // [RT*16]
  float* rowIZ = rowM + RT * 16;                                 // [RT*16]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cbase = tile * kRefineTile + w * 64;
  refine_issue_rows<D>(q, k, cand, seq_start[s], s, g, B, Hq, Hkv, G, C, R, RT, tile, qs, kls);
  // per-row normalisers over all tiles, merged in tile order while the rows stream in
  // (a row's tile statistics are contiguous; 32 tiles per batch of loads)
  for (int r = threadIdx.x; r < RT * 16; r += kRefineTile) {
    float M = -INFINITY, Z = 0.f;
    if (r < R) {
      const float2* rs = row_stats + (((int64_t)s * Hkv + g) * R + r) * ((ntile + 1) & ~1);  // 16-byte aligned rows
      for (int t0 = 0; t0 < ntile; t0 += 32) {
        float2 p[32];
#pragma unroll
        for (int u = 0; u < 32; u += 2) {
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
        for (int u = 0; u < 32; ++u) ms_merge(M, Z, p[u].x, p[u].y);
      }
    }
    rowM[r] = M;
    rowIZ[r] = r < R ? 1.f / Z : 0.f;
  }
  uint4 a[4][D / 32];
  refine_key_frags<D>(kls, a);

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
      for (int i = 0; i < 4; ++i) rs[mt][i] += r < R ? fast_exp2(acc[mt][i] * scale2 - M) * iz : 0.f;
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

// Exact top-K of the refine scores of one (sequence, KV head), in LDS: scores and
// candidate indices staged with 16-byte loads, three radix digits, ballot emission.
__global__ __launch_bounds__(1024) void refine_select_kernel(const int32_t* __restrict__ cand,
                                                            const float* __restrict__ rscore, int Hkv, int C,
                                                            int topk, int32_t* __restrict__ topk_idx,
                                                            float* __restrict__ topk_score) {
  constexpr int NT = 1024;
  const int g = blockIdx.x, s = blockIdx.y;
  extern __shared__ uint32_t sm[];  // [C] scores, then [C] candidate indices
  uint32_t* u = sm;
  int32_t* ci = reinterpret_cast<int32_t*>(sm + C);
  __shared__ uint32_t h[kRadixBins];
  __shared__ uint32_t wcnt[NT / 64][2];
  __shared__ uint32_t dig[2];
  const int64_t base = ((int64_t)s * Hkv + g) * C;
  {
    constexpr int U = 4;
    const int n4 = C % 4 == 0 ? C / 4 : 0;  // 16-byte loads need 16-byte aligned rows
    for (int i0 = 0; i0 < n4; i0 += NT * U) {
      uint4 a[U], b[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int i = i0 + k * NT + threadIdx.x;
        a[k] = i < n4 ? *reinterpret_cast<const uint4*>(rscore + base + 4 * i) : make_uint4(0, 0, 0, 0);
        b[k] = i < n4 ? *reinterpret_cast<const uint4*>(cand + base + 4 * i) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int i = i0 + k * NT + threadIdx.x;
        if (i < n4) {
          reinterpret_cast<uint4*>(u)[i] = a[k];
          reinterpret_cast<uint4*>(ci)[i] = b[k];
        }
      }
    }
    for (int i = 4 * n4 + threadIdx.x; i < C; i += NT) {
      u[i] = __float_as_uint(rscore[base + i]);
      ci[i] = cand[base + i];
    }
  }
  __syncthreads();
  uint32_t ties;
  const uint32_t thr = lds_radix_threshold<NT>(u, C, (uint32_t)topk, h, dig, false, &ties);
  lds_emit<NT / 64>(u, C, thr, ties, ci, topk_idx + ((int64_t)s * Hkv + g) * topk,
                    topk_score ? topk_score + ((int64_t)s * Hkv + g) * topk : nullptr, wcnt);
}

// fp32 path: one workgroup per (sequence, KV head); rows first, then candidates.
template <int D>
__device__ __forceinline__ float dot_rows_f32(const float* __restrict__ a, const float* __restrict__ b) {
  float acc = 0.f;
#pragma unroll 8
  for (int e = 0; e < D; ++e) acc = fmaf(a[e], b[e], acc);
  return acc;
}

template <int D>
__global__ __launch_bounds__(256) void refine_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                         const int32_t* __restrict__ cand,
                                                         const int64_t* __restrict__ seq_start, int B, int Hq,
                                                         int Hkv, int G, int C, float scale2, int topk,
                                                         float* __restrict__ rscore, int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_score) {
  const int g = blockIdx.x, s = blockIdx.y;
  const int R = B * G;
  const int64_t j0 = seq_start[s];
  __shared__ float rowM[256], rowIZ[256];
  __shared__ uint32_t h[kRadixBins];
  __shared__ uint32_t lds[256 / 64 + 4];
  extern __shared__ uint32_t u[];  // [C]
  const int32_t* cd = cand + ((int64_t)s * Hkv + g) * C;
  auto qrow = [&](int r) { return q + (((int64_t)s * B + r / G) * Hq + g * G + r % G) * D; };
  auto krow = [&](int c) { return k + ((j0 + cd[c]) * Hkv + g) * D; };
  for (int r = threadIdx.x; r < R; r += 256) {
    float m = -INFINITY, z = 0.f;
    for (int c = 0; c < C; ++c) {
      const float x = dot_rows_f32<D>(qrow(r), krow(c)) * scale2;
      if (x > m) {
        z = z * fast_exp2(m - x) + 1.f;
        m = x;
      } else {
        z += fast_exp2(x - m);
      }
    }
    rowM[r] = m;
    rowIZ[r] = 1.f / z;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < C; c += 256) {
    float acc = 0.f;
    for (int r = 0; r < R; ++r) acc += fast_exp2(dot_rows_f32<D>(qrow(r), krow(c)) * scale2 - rowM[r]) * rowIZ[r];
    rscore[((int64_t)s * Hkv + g) * C + c] = acc;
    u[c] = __float_as_uint(acc);
  }
  __syncthreads();
  lds_topk<256>(u, C, topk, h, lds, cd, topk_idx + ((int64_t)s * Hkv + g) * topk,
                topk_score ? topk_score + ((int64_t)s * Hkv + g) * topk : nullptr);
}

// ------------------------------------------------------------------ launchers

static size_t refine_smem(const Shape& s, bool stats) {
  const int RT = (s.B * s.G + 15) / 16;
  const size_t rows = ((size_t)RT * 16 + kRefineTile) * s.D * sizeof(bf16);
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
  const size_t smem = 2 * (size_t)s.C * sizeof(uint32_t);
  hipError_t e = allow_smem((const void*)refine_select_kernel, smem);
  if (e != hipSuccess) return e;
  klaunch(refine_select_kernel, dim3(s.Hkv, s.nseq), 1024, smem, st, cand, ws.rscore, s.Hkv, s.C, s.topk, topk_idx,
                                                                topk_score);
  return hipGetLastError();
}

hipError_t launch_refine_f32(const Shape& s, const void* q, const void* k, const int32_t* cand, const RefineWs& ws,
                             int32_t* topk_idx, float* topk_score, hipStream_t st) {
  dim3 grid(s.Hkv, s.nseq);
  const float scale2 = s.scale * kLog2e;
  const size_t smem = (size_t)s.C * sizeof(uint32_t);
  const void* kern = s.D == 128 ? (const void*)refine_f32_kernel<128> : (const void*)refine_f32_kernel<64>;
  hipError_t e = allow_smem(kern, smem);
  if (e != hipSuccess) return e;
  if (s.D == 128)
    klaunch(refine_f32_kernel<128>, grid, 256, smem, st, (const float*)q, (const float*)k, cand, s.seq_start, s.B, s.Hq,
                                                    s.Hkv, s.G, s.C, scale2, s.topk, ws.rscore, topk_idx, topk_score);
  else
    klaunch(refine_f32_kernel<64>, grid, 256, smem, st, (const float*)q, (const float*)k, cand, s.seq_start, s.B, s.Hq,
                                                   s.Hkv, s.G, s.C, scale2, s.topk, ws.rscore, topk_idx, topk_score);
  return hipGetLastError();
}

}  // namespace herald
