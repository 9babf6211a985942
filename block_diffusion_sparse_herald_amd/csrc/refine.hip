// Stage two of the two-stage selection: refine the C candidates with the B real
// queries into the final top-K subset (HERALD, arXiv 2606.21633 v3, abstract).
//
// Refine score of candidate c of KV head g (the per-row softmax is over the C
// candidates only, summed over the B queries and the G heads of the group):
//   R_g[c] = sum_{b, h in g} 2^(x[b,h,c] - M[b,h]) / Z[b,h],
//   x = scale * log2(e) * <q[b][h], K[cand_c][g]>.
//
// Two launches over the same (sequence, KV head, candidate tile) grid; both compute x
// with identical MFMA code, so the logits agree bit for bit:
//   refine_stats_kernel   per row (b,h): (max, sum 2^(x-max)) over the tile
//                         (stored row-major: a row's tiles are contiguous).
//   refine_scores_kernel  per row: normalisers from all tiles; per candidate: the
//                         sum over rows, in a fixed order (each lane over its row's
//                         tiles, then over the 16 lanes of a row with DPP shifts).
// A workgroup of four waves covers 256 candidates (bf16: four 16-candidate MFMA tiles
// per wave) or 64 (fp32: one tile per wave); large bf16 candidate sets take eight waves
// and 512 candidates (refine_waves). The candidate key rows, gathered from the
// cache by index, go straight into registers as the A operand; the group's B*G query
// rows, shared by the waves, are streamed into LDS with direct-to-LDS loads and read as
// the B operand (v_mfma_f32_16x16x32_bf16 or v_mfma_f32_16x16x4_f32, fp32 accumulate).
// Only the query rows take LDS (32 KiB at B*G = 128, d = 128 in bf16), so several
// workgroups share a compute unit and one's loads overlap another's products.
// refine_select_kernel then takes, per (sequence, KV head), the exact top-K of R
// in LDS (three radix digits on the fp32 bit pattern, R >= 0), ties to the lower
// cache index, ascending output.
// fp32 path: the same kernels on v_mfma_f32_16x16x4_f32 (fp32 products and sums),
// 64-candidate tiles.
#include "common.hpp"
#include "kernels.hpp"

namespace herald {

// Candidate tiles (16 candidates each) per wave: 4 for bf16, 1 for fp32, whose MFMA
// does an eighth of the bf16 work per instruction (workgroups of 256 and 64
// candidates).
template <typename T>
constexpr int refine_mt() { return sizeof(T) == 2 ? 4 : 1; }
template <typename T, int NW>
constexpr int refine_tile() { return NW * 16 * refine_mt<T>(); }

// 16-byte chunk c of an LDS query row r is stored at chunk c ^ refine_swz(r): the 16
// rows one MFMA fragment read touches hit distinct banks.
template <typename T, int D>
__device__ __forceinline__ int refine_swz(int r) {
  return sizeof(T) == 4 || D == 128 ? (r & 15) : ((r >> 1) & 7);
}

// Operand layout of both products (v_mfma_f32_16x16x32_bf16, v_mfma_f32_16x16x4_f32):
// lane l supplies row l % 16 of A (a candidate key) and column l % 16 of B (a query row)
// at the contraction slots of lane group l / 16, and holds D[4 (l / 16) + i][l % 16].
// Each lane keeps D / 4 elements of its key row (D * sizeof(T) / 64 16-byte chunks per
// candidate tile). bf16: chunk ks of lane group j covers dimensions 32 ks + 8 j .. +8,
// one MFMA. fp32: lane group j covers dimensions j D/4 .. (j + 1) D/4 - 1, chunk c of it
// four MFMAs, one dimension each; the query side uses the same assignment, so the
// contraction runs over every dimension once.
template <typename T, int D>
struct RefineFrag {
  static constexpr int NC = D * (int)sizeof(T) / 64;  // 16-byte chunks per lane per candidate tile
  static constexpr int EPC = 16 / (int)sizeof(T);     // elements per chunk
  // element offset of chunk c of lane group j within a row
  __device__ static constexpr int off(int j, int c) { return sizeof(T) == 2 ? c * 32 + j * 8 : j * (D / 4) + c * 4; }
};

template <typename T, int D, int MT>
__device__ __forceinline__ void refine_tile_logits(const uint4 (&a)[MT][RefineFrag<T, D>::NC], const T* qs, int rt,
                                                   int lane, f32x4_t (&acc)[MT]) {
  using F = RefineFrag<T, D>;
  uint4 bq[F::NC];
  const int r = rt * 16 + (lane & 15);
#pragma unroll
  for (int c = 0; c < F::NC; ++c)
    bq[c] = *reinterpret_cast<const uint4*>(qs + r * D + ((F::off(lane >> 4, c) / F::EPC) ^ refine_swz<T, D>(r)) * F::EPC);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < F::NC; ++c) {
      if constexpr (sizeof(T) == 2) {
        acc[mt] = mfma16x16x32(a[mt][c], bq[c], acc[mt]);
      } else {
        const uint32_t av[4] = {a[mt][c].x, a[mt][c].y, a[mt][c].z, a[mt][c].w};
        const uint32_t bv[4] = {bq[c].x, bq[c].y, bq[c].z, bq[c].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(av[e]), __uint_as_float(bv[e]), acc[mt], 0,
                                                         0, 0);
      }
    }
  }
}

// Shared prologue of both refine kernels, in two parts. refine_issue_rows: the
// group's query rows go to LDS with coalesced direct-to-LDS loads (rows past R re-read
// query row 0, masked later), and each wave loads the MFMA fragments of its MT * 16
// candidate key rows straight into registers, gathered from the cache by index
// (candidates past C re-read the last one, masked later); every lane reads 16 bytes of
// a row per load. refine_wait_rows: once both have landed, the workgroup may read the
// query rows.
template <typename T, int D, int MT, int NW>
__device__ __forceinline__ void refine_issue_rows(const T* __restrict__ q, const T* __restrict__ k,
                                                  const int32_t* __restrict__ cand, int64_t j0, int s, int g, int B,
                                                  int Hq, int Hkv, int G, int C, int R, int row0, int RT, int ctile,
                                                  T* qs, uint4 (&a)[MT][RefineFrag<T, D>::NC]) {
  using F = RefineFrag<T, D>;
  constexpr int CPR = D / F::EPC;  // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;    // rows per load instruction
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rr = lane / CPR, p = lane % CPR;
  // query rows row0 .. row0 + 16 RT: the waves take turns by instruction
  for (int r0 = w * RPI; r0 < RT * 16; r0 += NW * RPI) {
    const int r = r0 + rr;
    const int rq = row0 + r < R ? row0 + r : 0;
    const T* src = q + (((int64_t)s * B + rq / G) * Hq + g * G + rq % G) * D + (p ^ refine_swz<T, D>(r)) * F::EPC;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(qs + r0 * D), 16, 0, 0);
  }
  // candidate key fragments of wave w: rows (w * MT + mt) * 16 + (lane & 15) of the tile
  const int32_t* cd = cand + ((int64_t)s * Hkv + g) * C;
  const T* rows[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int c = min(ctile * refine_tile<T, NW>() + (w * MT + mt) * 16 + (lane & 15), C - 1);
    rows[mt] = k + ((j0 + cd[c]) * Hkv + g) * D;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int c = 0; c < F::NC; ++c) a[mt][c] = *reinterpret_cast<const uint4*>(rows[mt] + F::off(lane >> 4, c));
}

__device__ __forceinline__ void refine_wait_rows() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

template <typename T, int D, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void refine_stats_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                           const int32_t* __restrict__ cand,
                                                           const int64_t* __restrict__ seq_start, int B, int Hq,
                                                           int Hkv, int G, int C, float scale2, int ntile,
                                                           int nsplit, float2* __restrict__ row_stats) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int MT = refine_mt<T>();
  // SPLIT: row split rsp of tile; otherwise the whole tile (nsplit = 1)
  const int tile = SPLIT ? blockIdx.x / nsplit : blockIdx.x, rsp = SPLIT ? blockIdx.x - tile * nsplit : 0;
  const int g = blockIdx.y, s = blockIdx.z;
  const int R = B * G, RTA = (R + 15) / 16, RTS = SPLIT ? (RTA + nsplit - 1) / nsplit : RTA;
  const int row0 = SPLIT ? rsp * RTS * 16 : 0, RT = SPLIT ? min(RTS, RTA - rsp * RTS) : RTA;  // its row tiles
  T* qs = reinterpret_cast<T*>(smem);                           // [RT*16][D]
  float2* wstat = reinterpret_cast<float2*>(qs + RT * 16 * D);  // [NW][RT*16]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cbase = tile * refine_tile<T, NW>() + w * MT * 16;
  uint4 a[MT][RefineFrag<T, D>::NC];
  refine_issue_rows<T, D, MT, NW>(q, k, cand, seq_start[s], s, g, B, Hq, Hkv, G, C, R, row0, RT, tile, qs, a);
  refine_wait_rows();

  const bool full = cbase + MT * 16 <= C;  // no candidate of this wave past C
  for (int rt = 0; rt < RT; ++rt) {
    f32x4_t acc[MT];
    refine_tile_logits<T, D, MT>(a, qs, rt, lane, acc);
    if (!full) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (cbase + mt * 16 + (lane >> 4) * 4 + i >= C) acc[mt][i] = -INFINITY;
    }
    // the row max on the raw products (scale2 > 0), the logits as one fma each
    float mr = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mr = fmaxf(mr, acc[mt][i]);
    mr = xmax4(mr);
    const float m = mr * scale2;
    float l = 0.f;
    if (mr != -INFINITY) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) l += fast_exp2(fmaf(acc[mt][i], scale2, -m));
    }
    l = xsum4(l);
    if (lane < 16) wstat[w * RT * 16 + rt * 16 + lane] = make_float2(m, l);
  }
  __syncthreads();
  for (int r = threadIdx.x; r < RT * 16 && row0 + r < R; r += NW * 64) {
    float M = -INFINITY, Z = 0.f;
    for (int ww = 0; ww < NW; ++ww) {
      const float2 p = wstat[ww * RT * 16 + r];
      ms_merge(M, Z, p.x, p.y);
    }
    row_stats[(((int64_t)s * Hkv + g) * R + row0 + r) * ((ntile + 1) & ~1) + tile] = make_float2(M, Z);
  }
}

template <typename T, int D, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void refine_scores_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                            const int32_t* __restrict__ cand,
                                                            const int64_t* __restrict__ seq_start, int B, int Hq,
                                                            int Hkv, int G, int C, float scale2, int ntile,
                                                            int nsplit, const float2* __restrict__ row_stats,
                                                            float* __restrict__ rscore) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int MT = refine_mt<T>();
  // SPLIT: row split rsp of tile; otherwise the whole tile (nsplit = 1)
  const int tile = SPLIT ? blockIdx.x / nsplit : blockIdx.x, rsp = SPLIT ? blockIdx.x - tile * nsplit : 0;
  const int g = blockIdx.y, s = blockIdx.z;
  const int R = B * G, RTA = (R + 15) / 16, RTS = SPLIT ? (RTA + nsplit - 1) / nsplit : RTA;
  const int row0 = SPLIT ? rsp * RTS * 16 : 0, RT = SPLIT ? min(RTS, RTA - rsp * RTS) : RTA;  // its row tiles
  T* qs = reinterpret_cast<T*>(smem);                        // [RT*16][D]
  float* rowM = reinterpret_cast<float*>(qs + RT * 16 * D);  // [RT*16]
  float* rowIZ = rowM + RT * 16;                             // [RT*16]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cbase = tile * refine_tile<T, NW>() + w * MT * 16;
  uint4 a[MT][RefineFrag<T, D>::NC];
  refine_issue_rows<T, D, MT, NW>(q, k, cand, seq_start[s], s, g, B, Hq, Hkv, G, C, R, row0, RT, tile, qs, a);
  // per-row normalisers over all tiles, merged in tile order while the rows stream in
  // (a row's tile statistics are contiguous; 16 tiles per batch of loads)
  for (int r = threadIdx.x; r < RT * 16; r += NW * 64) {
    float M = -INFINITY, Z = 0.f;
    if (row0 + r < R) {
      const float2* rs = row_stats + (((int64_t)s * Hkv + g) * R + row0 + r) * ((ntile + 1) & ~1);  // 16-byte aligned
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
    rowM[r] = row0 + r < R ? M : 3.0e38f;
    rowIZ[r] = row0 + r < R ? 1.f / Z : 0.f;
  }
  refine_wait_rows();

  float rs[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[mt][i] = 0.f;
  for (int rt = 0; rt < RT; ++rt) {
    f32x4_t acc[MT];
    refine_tile_logits<T, D, MT>(a, qs, rt, lane, acc);
    const int r = rt * 16 + (lane & 15);
    const float M = rowM[r], iz = rowIZ[r];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) rs[mt][i] = fmaf(fast_exp2(fmaf(acc[mt][i], scale2, -M)), iz, rs[mt][i]);
  }
  // each lane summed its query row over the row tiles; now sum the 16 rows of a lane row
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[mt][i] = row_sum16_last(rs[mt][i]);
  if ((lane & 15) == 15) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = cbase + mt * 16 + (lane >> 4) * 4 + i;
        // the row split's partial sum; the top-K kernel adds the splits in order
        if (c < C) rscore[(((int64_t)rsp * gridDim.z + s) * Hkv + g) * C + c] = rs[mt][i];
      }
  }
}

// Exact top-K of the refine scores of one (sequence, KV head): three radix digits
// (11, 11, 10 bits of the fp32 pattern, R >= 0), ties to the lower position, ascending
// output. STAGED (C <= kMaxCandidates): scores and candidate indices stay in registers
// (topk_load's layout: each wave a contiguous range of positions), the histograms take
// LDS atomics and the picks are ordered by wave scans in LDS, then written out. Otherwise (candidate sets up to the
// whole sequence) the passes read them from global memory.
template <bool STAGED, int ALIGN = 0>
__global__ __launch_bounds__(1024) void refine_select_kernel(const int32_t* __restrict__ cand,
                                                            const float* __restrict__ rscore, int nsplit, int Hkv,
                                                            int C, int topk, int32_t* __restrict__ topk_idx,
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
    extern __shared__ int32_t picks[];  // [topk + kTopkSlack] picks, then as many scores when they are wanted
    const int tid = threadIdx.x, w = tid >> 6;
    const int nit = topk_chunks(C);
    uint32_t v[MAXIT][4], ix[MAXIT][4];
    topk_load<MAXIT, float, ALIGN>(rscore + base, C, nit, v);
    topk_load<MAXIT, int32_t, ALIGN>(cand + base, C, nit, ix);
    // row splits: R is the sum of the splits' partial scores, added in split order. All
    // splits are loaded before the first sum (a split past nsplit re-reads the last one and
    // is not added), so their loads are in flight together
    if (nsplit > 1) {
      uint32_t u[kRefineMaxSplits - 1][MAXIT][4];
#pragma unroll
      for (int sp = 1; sp < kRefineMaxSplits; ++sp)
        topk_load<MAXIT, float, ALIGN>(rscore + (int64_t)min(sp, nsplit - 1) * gridDim.y * Hkv * C + base, C, nit,
                                       u[sp - 1]);
#pragma unroll
      for (int sp = 1; sp < kRefineMaxSplits; ++sp)
        if (sp < nsplit)
#pragma unroll
          for (int it = 0; it < MAXIT; ++it)
#pragma unroll
            for (int c = 0; c < 4; ++c)
              v[it][c] = __float_as_uint(__uint_as_float(v[it][c]) + __uint_as_float(u[sp - 1][it][c]));
    }
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
                     h3[dig[0]] == ties, (uint32_t)topk, picks, outs ? reinterpret_cast<float*>(picks + topk + kTopkSlack) : nullptr,
                     out, outs, wcnt);
  } else {
    const uint32_t* u = reinterpret_cast<const uint32_t*>(rscore + base);
    uint32_t ties;
    const uint32_t thr = lds_radix_threshold<NT>(u, C, (uint32_t)topk, h, dig, false, &ties);
    lds_emit<NT / 64>(u, C, thr, ties, cand + base, out, outs, wcnt);
  }
}

// ------------------------------------------------------------------ launchers

// Waves per refine workgroup: 4 (256 bf16 candidates), or 8 (512) when a (sequence,
// KV head) has more than 16 tiles of 256 and 512-candidate workgroups still number
// >= 256: the scores kernel then merges at most 16 tile statistics per row (one batch
// of loads), and the query rows in LDS serve twice the candidates. Measured at
// C = 8192 over 32 pairs: -6 us per step; at C = 4096 over 128 pairs 8 waves were
// not faster.
static int refine_waves(const Shape& s) {
  if (!s.bf16) return 4;
  const int t4 = (s.C + refine_tile<bf16, 4>() - 1) / refine_tile<bf16, 4>();
  const int64_t wg8 = (int64_t)((s.C + refine_tile<bf16, 8>() - 1) / refine_tile<bf16, 8>()) * s.Hkv * s.nseq;
  return t4 > 16 && wg8 >= 256 ? 8 : 4;
}

// Row splits of the refine: when the (sequence, KV head, candidate tile) grid leaves
// compute units idle, each tile's query rows are split over 2 or 4 workgroups (each
// with its rows' statistics and a partial score; the top-K kernel adds the partials).
// Only for candidate sets the top-K kernel stages in registers.
int refine_splits(const Shape& s) {
  const int tile = refine_tile_of(s);
  const int64_t nwg = (int64_t)((s.C + tile - 1) / tile) * s.Hkv * s.nseq;
  const int RT = (s.B * s.G + 15) / 16;
  int ns = 1;
  if (s.C <= kMaxCandidates)
    while (ns < kRefineMaxSplits && nwg * ns * 2 <= kRefineSplitTarget && RT % (ns * 2) == 0) ns *= 2;  // equal splits
  return ns;
}

static size_t refine_smem(const Shape& s, bool stats) {
  const int RT = (s.B * s.G + 15) / 16;
  const size_t rows = (size_t)RT * 16 * s.D * (s.bf16 ? 2 : 4);
  return rows + (stats ? (size_t)refine_waves(s) * RT * 16 * sizeof(float2) : (size_t)2 * RT * 16 * sizeof(float));
}

template <typename T, int D, int NW>
static hipError_t launch_refine_t(const Shape& s, const void* q, const void* k, const int32_t* cand,
                                  const RefineWs& ws, bool stats, hipStream_t st) {
  const dim3 grid(ws.ntile * ws.nsplit, s.Hkv, s.nseq);
  const float scale2 = s.scale * kLog2e;
  const size_t smem = refine_smem(s, stats);
  const bool split = ws.nsplit > 1;
  const void* kern = stats ? (split ? (const void*)refine_stats_kernel<T, D, NW, true>
                                    : (const void*)refine_stats_kernel<T, D, NW, false>)
                           : (split ? (const void*)refine_scores_kernel<T, D, NW, true>
                                    : (const void*)refine_scores_kernel<T, D, NW, false>);
  hipError_t e = allow_smem(kern, smem);
  if (e != hipSuccess) return e;
  if (stats) {
    auto kf = split ? refine_stats_kernel<T, D, NW, true> : refine_stats_kernel<T, D, NW, false>;
    klaunch(kf, grid, NW * 64, smem, st, (const T*)q, (const T*)k, cand, s.seq_start, s.B, s.Hq, s.Hkv, s.G, s.C,
            scale2, ws.ntile, ws.nsplit, ws.row_stats);
  } else {
    auto kf = split ? refine_scores_kernel<T, D, NW, true> : refine_scores_kernel<T, D, NW, false>;
    klaunch(kf, grid, NW * 64, smem, st, (const T*)q, (const T*)k, cand, s.seq_start, s.B, s.Hq, s.Hkv, s.G, s.C,
            scale2, ws.ntile, ws.nsplit, ws.row_stats, ws.rscore);
  }
  return hipGetLastError();
}

static hipError_t launch_refine(const Shape& s, const void* q, const void* k, const int32_t* cand,
                                const RefineWs& ws, bool stats, hipStream_t st) {
  if (s.bf16) {
    if (refine_waves(s) == 8)
      return s.D == 128 ? launch_refine_t<bf16, 128, 8>(s, q, k, cand, ws, stats, st)
                        : launch_refine_t<bf16, 64, 8>(s, q, k, cand, ws, stats, st);
    return s.D == 128 ? launch_refine_t<bf16, 128, 4>(s, q, k, cand, ws, stats, st)
                      : launch_refine_t<bf16, 64, 4>(s, q, k, cand, ws, stats, st);
  }
  return s.D == 128 ? launch_refine_t<float, 128, 4>(s, q, k, cand, ws, stats, st)
                    : launch_refine_t<float, 64, 4>(s, q, k, cand, ws, stats, st);
}

int refine_tile_of(const Shape& s) {
  if (!s.bf16) return refine_tile<float, 4>();
  return refine_waves(s) == 8 ? refine_tile<bf16, 8>() : refine_tile<bf16, 4>();
}

hipError_t launch_refine_stats(const Shape& s, const void* q, const void* k, const int32_t* cand, const RefineWs& ws,
                               hipStream_t st) {
  return launch_refine(s, q, k, cand, ws, true, st);
}

hipError_t launch_refine_scores(const Shape& s, const void* q, const void* k, const int32_t* cand,
                                const RefineWs& ws, hipStream_t st) {
  return launch_refine(s, q, k, cand, ws, false, st);
}

hipError_t launch_refine_select(const Shape& s, const int32_t* cand, const RefineWs& ws, int32_t* topk_idx,
                                float* topk_score, hipStream_t st) {
  if (s.C > kMaxCandidates) {
    klaunch(refine_select_kernel<false>, dim3(s.Hkv, s.nseq), 1024, 0, st, cand, ws.rscore, 1, s.Hkv, s.C, s.topk,
            topk_idx, topk_score);
    return hipGetLastError();
  }
  const size_t smem = (size_t)(s.topk + kTopkSlack) * sizeof(int32_t) * (topk_score ? 2 : 1);
  // the rows of C scores and candidates start 16-byte aligned when C % 4 == 0 and both
  // buffers do; then the kernel takes the 16-byte loads without a run-time check
  const bool aligned = s.C % 4 == 0 && ((uintptr_t)cand & 15) == 0 && ((uintptr_t)ws.rscore & 15) == 0;
  auto kern = aligned ? refine_select_kernel<true, 1> : refine_select_kernel<true, 0>;
  hipError_t e = allow_smem((const void*)kern, smem);
  if (e != hipSuccess) return e;
  klaunch(kern, dim3(s.Hkv, s.nseq), 1024, smem, st, cand, ws.rscore, ws.nsplit, s.Hkv, s.C,
          s.topk, topk_idx, topk_score);
  return hipGetLastError();
}

}  // namespace herald
