// B-query block attention over the selected subset plus the step's in-block keys,
// one denoising step per call (HERALD abstract on the mlsift "KV cache offloading"
// listing: the denoising phase reuses the selected subset T times; HERALD v3
// abstract: the final top-K subset). No mask.
//
// For KV head g the B*G query rows (b, h in g) share the keys
//   key i < topk:          k_sel[s][g][i]           (values: v_sel, stored d-major)
//   key topk + b':         k_blk[s][b'][g]           (values: v_blk[s][b'][g])
// The keys form 64-key blocks: ceil(topk/64) subset blocks (the last one masked past
// topk) and one block of the B <= 64 in-block keys.
//
// bf16 path. A compute unit pulls data from L2/HBM at a few tens of GB/s (the
// number of misses it can keep in flight bounds it), so the keys of one (sequence,
// KV head) are spread over many workgroups: attn_part_kernel gives each workgroup a
// contiguous range of key blocks and a set of 16-row query tiles (one per wave).
// Per block the workgroup stages K rows (XOR-swizzled 16-byte chunks, so that the
// 16 rows one MFMA reads fall in distinct LDS banks) and V^T (padded rows) in LDS,
// every wave reads its fragments from there: S^T = K.Q^T on v_mfma_f32_16x16x32_bf16
// (keys on M, the tile's query rows on N, Q fragments held in registers), an
// online softmax in base 2 per query row, then O^T += V^T.P^T with P^T taken from
// the S^T accumulators. The keys of a block are assigned to MFMA rows so that the
// 32-key contraction of the second product runs over consecutive keys (one 16-byte
// LDS read per V^T fragment). The next block is fetched into registers while the
// current one is used. With one key range the kernel writes the output; otherwise
// it writes partials (fp32 max and sum, the unnormalised output rounded to bf16)
// that attn_combine_kernel merges.
// fp32 path (attn_f32_kernel): one workgroup per query row, VALU.
#include "common.hpp"
#include "kernels.hpp"

namespace herald {

// Row m of key tile mt within a 64-key block -> key offset in the block. Tiles 2c and
// 2c+1 cover keys [32c, 32c+32); lane group j of the second product then contracts
// over keys 32c + 8j .. 32c + 8j + 7, which the accumulators of lane group j hold.
__device__ __forceinline__ int attn_key_of(int mt, int m) {
  return (mt >> 1) * 32 + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3);
}

// 16-byte chunk c of K row r lives at chunk c ^ swz(r): the rows one MFMA operand
// reads (attn_key_of(mt, 0..15)) map to 16 distinct values.
template <int D>
__device__ __forceinline__ int attn_swz(int r) {
  return ((r & 3) | ((r >> 1) & 12)) & (D / 8 - 1);
}

template <int D>
__global__ __launch_bounds__(512) void attn_part_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kb,
                                                        const bf16* __restrict__ vb, const bf16* __restrict__ k_sel,
                                                        const bf16* __restrict__ v_sel, AttnGeom a, float scale2,
                                                        bf16* __restrict__ out, bf16* __restrict__ o_part,
                                                        float2* __restrict__ ml_part) {
  constexpr int KB = kAttnKeyBlock;  // 64
  constexpr int KS = D / 32;         // contraction steps of S^T = K.Q^T
  constexpr int DT = D / 16;         // 16-dim output tiles
  constexpr int CPR = D / 8;         // 16-byte chunks per K row
  constexpr int LDV = KB + 8;        // V^T row stride in LDS (elements)
  constexpr int NCH = KB * CPR;      // 16-byte chunks of K (and of V) per block
  constexpr int PT = NCH / 256;      // chunks per thread at 256 threads
  __shared__ __align__(16) bf16 Ks[KB * D];
  __shared__ __align__(16) bf16 Vt[D * LDV];
  // 1-D grid, XCD-aware: workgroup x runs on XCD x % 8 and each XCD takes a contiguous
  // range of items; the row splits of one key range are adjacent and share an L2.
  const int per = gridDim.x >> 3;
  const int li = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (li >= a.nitems) return;
  const int rs = li % a.nrs, ksp = (li / a.nrs) % a.nks, unit = li / (a.nrs * a.nks);
  const int B = a.B, G = a.G, topk = a.topk;
  const int s = unit / a.Hkv, g = unit % a.Hkv;
  const int nthr = blockDim.x, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, qd = lane >> 4, lr = lane & 15;
  const int R = B * G, nA = (topk + KB - 1) / KB, nblk = nA + 1;
  const int b0 = ksp * a.bps, b1 = min(nblk, b0 + a.bps);
  const int tile = rs * a.tpw + w;
  const bool has_tile = w < a.tpw && tile * 16 < R;

  const bf16* ksrc = k_sel + (int64_t)unit * topk * D;
  const bf16* vsrc = v_sel + (int64_t)unit * D * a.ldv;
  const bf16* kbb = kb + ((int64_t)s * B * a.Hkv + g) * D;  // in-block key b at kbb + b * Hkv * D
  const bf16* vbb = vb + ((int64_t)s * B * a.Hkv + g) * D;
  const int64_t bstride = (int64_t)a.Hkv * D;

  uint4 qf[KS];
  {
    const int r = tile * 16 + lr;
    const bf16* qr =
        has_tile && r < R ? q + (((int64_t)s * B + r / G) * a.Hq + g * G + r % G) * D + qd * 8 : nullptr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = qr ? ld16(qr + ks * 32) : make_uint4(0, 0, 0, 0);
  }

  // ---- staging: chunk c of K is row c / CPR, chunk c % CPR; chunk c of V^T is, for the
  //      subset (d-major in memory), dim c / 8, keys 8*(c % 8) ..; for the in-block keys
  //      (key-major in memory), key c % 64, dims 8*(c / 64) .. (transposed into LDS).
  uint4 kreg[PT], vreg[PT];
  auto fetch = [&](int blk) {
    const bool sub = blk < nA;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = tid + i * nthr;
      kreg[i] = vreg[i] = make_uint4(0, 0, 0, 0);
      if (c < NCH) {
        const int r = c / CPR, ch = c % CPR;
        if (sub) {
          kreg[i] = ld16(ksrc + (int64_t)min(blk * KB + r, topk - 1) * D + ch * 8);
          vreg[i] = ld16(vsrc + (int64_t)(c >> 3) * a.ldv + blk * KB + (c & 7) * 8);
        } else {
          if (r < B) kreg[i] = ld16(kbb + r * bstride + ch * 8);
          if ((c & 63) < B) vreg[i] = ld16(vbb + (c & 63) * bstride + (c >> 6) * 8);
        }
      }
    }
  };
  auto stash = [&](int blk) {
    const bool sub = blk < nA;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = tid + i * nthr;
      if (c < NCH) {
        const int r = c / CPR, ch = c % CPR;
        *reinterpret_cast<uint4*>(&Ks[r * D + ((ch ^ attn_swz<D>(r)) * 8)]) = kreg[i];
        if (sub) {
          *reinterpret_cast<uint4*>(&Vt[(c >> 3) * LDV + (c & 7) * 8]) = vreg[i];
        } else {
          const int key = c & 63, e8 = (c >> 6) * 8;
          const uint32_t xs[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
          uint16_t* vt = reinterpret_cast<uint16_t*>(Vt);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            vt[(e8 + 2 * j) * LDV + key] = (uint16_t)(xs[j] & 0xffffu);
            vt[(e8 + 2 * j + 1) * LDV + key] = (uint16_t)(xs[j] >> 16);
          }
        }
      }
    }
  };

  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  fetch(b0);
  for (int blk = b0; blk < b1; ++blk) {
    if (blk > b0) __syncthreads();  // every wave is done with the previous block
    stash(blk);
    __syncthreads();
    if (blk + 1 < b1) fetch(blk + 1);
    if (!has_tile) continue;

    // ---- S^T = K Q^T: lane holds keys attn_key_of(mt, 4*qd + i) of query row lr
    f32x4_t sacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sacc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int r = attn_key_of(mt, lr);
        const uint4 kf = *reinterpret_cast<const uint4*>(&Ks[r * D + (((ks * 4 + qd) ^ attn_swz<D>(r)) * 8)]);
        sacc[mt] = mfma16x16x32(kf, qf[ks], sacc[mt]);
      }

    // ---- online softmax (base 2); the scale is folded into one FMA; the output is
    //      rescaled only when some row's running max grows (otherwise every factor is 1)
    const int valid = blk < nA ? topk - blk * KB : B;
    if (valid < KB) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (attn_key_of(mt, 4 * qd + i) >= valid) sacc[mt][i] = -INFINITY;
    }
    float bm = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) bm = fmaxf(bm, sacc[mt][i]);
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mn = fmaxf(m, bm * scale2);
    if (__ballot(mn > m)) {
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    m = mn;
    float p[4][4];
    float ps = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[mt][i] = fast_exp2(fmaf(sacc[mt][i], scale2, -mn));
        ps += p[mt][i];
      }
    l += ps;
    uint4 bp[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      bp[h2] = make_uint4(pack_bf16x2(p[2 * h2][0], p[2 * h2][1]), pack_bf16x2(p[2 * h2][2], p[2 * h2][3]),
                          pack_bf16x2(p[2 * h2 + 1][0], p[2 * h2 + 1][1]),
                          pack_bf16x2(p[2 * h2 + 1][2], p[2 * h2 + 1][3]));

    // ---- O^T += V^T P^T over the two 32-key halves of the block
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const uint4 vf = *reinterpret_cast<const uint4*>(&Vt[(dt * 16 + lr) * LDV + h2 * 32 + qd * 8]);
        o[dt] = mfma16x16x32(vf, bp[h2], o[dt]);
      }
  }
  if (!has_tile) return;

  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const int r = tile * 16 + lr;
  if (a.nks == 1) {
    if (r >= R) return;
    bf16* orow = out + (((int64_t)s * B + r / G) * a.Hq + g * G + r % G) * D + qd * 4;
    const float inv = 1.f / l;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<uint2*>(orow + dt * 16) =
          make_uint2(pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv), pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv));
  } else {
    const int64_t prow = ((int64_t)unit * a.nks + ksp) * a.rpad + r;
    bf16* orow = o_part + prow * D + qd * 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<uint2*>(orow + dt * 16) =
          make_uint2(pack_bf16x2(o[dt][0], o[dt][1]), pack_bf16x2(o[dt][2], o[dt][3]));
    if (qd == 0) ml_part[prow] = make_float2(m, l);
  }
}

// Merges the key ranges of one (sequence, KV head): 4 output dimensions per thread,
// the ranges taken 8 at a time (loads first) with a running (max, sum).
template <int D>
__global__ __launch_bounds__(64) void attn_combine_kernel(const bf16* __restrict__ o_part,
                                                           const float2* __restrict__ ml_part, AttnGeom a,
                                                           bf16* __restrict__ out) {
  constexpr int CH = 8;
  const int idx = blockIdx.x * 64 + threadIdx.x;
  const int R = a.B * a.G;
  const int per_unit = R * (D / 4);
  const int unit = idx / per_unit;
  if (unit >= a.nunits) return;
  const int r = (idx % per_unit) / (D / 4), e = (idx % (D / 4)) * 4;
  const int s = unit / a.Hkv, g = unit % a.Hkv;
  const int64_t base = (int64_t)unit * a.nks * a.rpad + r;
  float M = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < a.nks; k0 += CH) {
    float2 p[CH];
    uint2 vb[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      p[j] = make_float2(-INFINITY, 0.f);
      vb[j] = make_uint2(0, 0);
      if (k0 + j < a.nks) {
        const int64_t row = base + (int64_t)(k0 + j) * a.rpad;
        p[j] = ml_part[row];
        vb[j] = *reinterpret_cast<const uint2*>(o_part + row * D + e);
      }
    }
    float mc = M;
#pragma unroll
    for (int j = 0; j < CH; ++j) mc = fmaxf(mc, p[j].x);
    const float alpha = fast_exp2(M - mc);  // 0 on the first chunk (M = -inf)
    L *= alpha;
    acc.x *= alpha;
    acc.y *= alpha;
    acc.z *= alpha;
    acc.w *= alpha;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (p[j].x == -INFINITY) continue;
      const float wgt = fast_exp2(p[j].x - mc);
      L += wgt * p[j].y;
      acc.x += wgt * bf16_lo(vb[j].x);
      acc.y += wgt * bf16_hi(vb[j].x);
      acc.z += wgt * bf16_lo(vb[j].y);
      acc.w += wgt * bf16_hi(vb[j].y);
    }
    M = mc;
  }
  const float inv = 1.f / L;
  *reinterpret_cast<uint2*>(out + (((int64_t)s * a.B + r / a.G) * a.Hq + g * a.G + r % a.G) * D + e) =
      make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv));
}

// fp32 path: one workgroup per query row; keys in chunks of 1024 with an online softmax.
template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ kb,
                                                       const float* __restrict__ vb, const float* __restrict__ k_sel,
                                                       const float* __restrict__ v_sel, int B, int Hq, int Hkv,
                                                       int G, int topk, int64_t ldv, float scale2,
                                                       float* __restrict__ out) {
  constexpr int KC = 1024;
  __shared__ float qs[D];
  __shared__ float xs[KC];
  __shared__ float red[4];
  const int b = blockIdx.x / Hq, h = blockIdx.x % Hq, s = blockIdx.y;
  const int g = h / G;
  const int64_t unit = (int64_t)s * Hkv + g;
  const float* qrow = q + (((int64_t)s * B + b) * Hq + h) * D;
  for (int e = threadIdx.x; e < D; e += 256) qs[e] = qrow[e];
  __syncthreads();
  const int NK = topk + B;
  auto key = [&](int kk) -> const float* {
    return kk < topk ? k_sel + (unit * topk + kk) * D : kb + (((int64_t)s * B + (kk - topk)) * Hkv + g) * D;
  };
  auto val = [&](int kk, int e) -> float {
    return kk < topk ? v_sel[(unit * D + e) * ldv + kk] : vb[(((int64_t)s * B + (kk - topk)) * Hkv + g) * D + e];
  };
  float m = -INFINITY, l = 0.f, acc = 0.f;
  for (int k0 = 0; k0 < NK; k0 += KC) {
    const int n = min(KC, NK - k0);
    float lm = -INFINITY;
    for (int t = threadIdx.x; t < n; t += 256) {
      const float* kr = key(k0 + t);
      float d = 0.f;
      for (int e = 0; e < D; ++e) d = fmaf(qs[e], kr[e], d);
      xs[t] = d * scale2;
      lm = fmaxf(lm, xs[t]);
    }
    for (int o = 32; o > 0; o >>= 1) lm = fmaxf(lm, __shfl_xor(lm, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = lm;
    __syncthreads();
    const float mn = fmaxf(m, fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
    const float alpha = fast_exp2(m - mn);
    if (threadIdx.x < D) {
      float a = 0.f, ls = 0.f;
      for (int t = 0; t < n; ++t) {
        const float p = fast_exp2(xs[t] - mn);
        ls += p;
        a = fmaf(p, val(k0 + t, threadIdx.x), a);
      }
      acc = acc * alpha + a;
      l = l * alpha + ls;
    }
    m = mn;
    __syncthreads();
  }
  if (threadIdx.x < D) out[(((int64_t)s * B + b) * Hq + h) * D + threadIdx.x] = acc / l;
}

// ------------------------------------------------------------------ host side

// Work split: up to 8 query tiles (waves) per workgroup, then enough key ranges to
// give about kAttnTargetWorkgroups workgroups, at most kAttnMaxSplits ranges.
AttnGeom attn_geom(const Shape& s) {
  AttnGeom a{};
  a.B = s.B;
  a.G = s.G;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.topk = s.topk;
  a.ldv = vsel_ld(s.topk);
  a.nunits = s.nseq * s.Hkv;
  const int ntiles = (s.B * s.G + 15) / 16;
  a.tpw = ntiles <= 8 ? ntiles : (ntiles + 1) / 2;
  a.nrs = (ntiles + a.tpw - 1) / a.tpw;
  a.rpad = ntiles * 16;
  const int nblk = (s.topk + kAttnKeyBlock - 1) / kAttnKeyBlock + 1;
  const int64_t groups = (int64_t)a.nunits * a.nrs;
  int nks = (int)std::min<int64_t>(std::max<int64_t>(1, (kAttnTargetWorkgroups + groups - 1) / groups),
                                   std::min(nblk, kAttnMaxSplits));
  a.bps = (nblk + nks - 1) / nks;
  a.nks = (nblk + a.bps - 1) / a.bps;
  a.nitems = (int)(groups * a.nks);
  return a;
}

int attn_splits(const Shape& s) { return s.bf16 ? attn_geom(s).nks : 1; }

size_t attn_ws_bytes(const Shape& s) {
  if (!s.bf16) return 0;
  const AttnGeom a = attn_geom(s);
  if (a.nks == 1) return 0;
  const size_t rows = (size_t)a.nunits * a.nks * a.rpad;
  return align256(rows * s.D * sizeof(bf16)) + align256(rows * sizeof(float2));
}

hipError_t launch_attn(const Shape& s, const void* q, const void* kb, const void* vb, const void* k_sel,
                       const void* v_sel, void* out, void* ws, hipStream_t st) {
  const float scale2 = s.scale * kLog2e;
  if (!s.bf16) {
    const int64_t ldv = vsel_ld(s.topk);
    dim3 grid(s.B * s.Hq, s.nseq);
    if (s.D == 128)
      klaunch(attn_f32_kernel<128>, grid, 256, 0, st, (const float*)q, (const float*)kb, (const float*)vb,
                                                 (const float*)k_sel, (const float*)v_sel, s.B, s.Hq, s.Hkv, s.G,
                                                 s.topk, ldv, scale2, (float*)out);
    else
      klaunch(attn_f32_kernel<64>, grid, 256, 0, st, (const float*)q, (const float*)kb, (const float*)vb,
                                                (const float*)k_sel, (const float*)v_sel, s.B, s.Hq, s.Hkv, s.G,
                                                s.topk, ldv, scale2, (float*)out);
    return hipGetLastError();
  }
  const AttnGeom a = attn_geom(s);
  bf16* o_part = nullptr;
  float2* ml_part = nullptr;
  if (a.nks > 1) {
    const size_t rows = (size_t)a.nunits * a.nks * a.rpad;
    o_part = static_cast<bf16*>(ws);
    ml_part = reinterpret_cast<float2*>(static_cast<char*>(ws) + align256(rows * s.D * sizeof(bf16)));
  }
  const dim3 grid((unsigned)((a.nitems + 7) / 8 * 8));
  const int threads = 64 * std::max(4, a.tpw);
  if (s.D == 128)
    klaunch(attn_part_kernel<128>, grid, threads, 0, st, (const bf16*)q, (const bf16*)kb, (const bf16*)vb,
            (const bf16*)k_sel, (const bf16*)v_sel, a, scale2, (bf16*)out, o_part, ml_part);
  else
    klaunch(attn_part_kernel<64>, grid, threads, 0, st, (const bf16*)q, (const bf16*)kb, (const bf16*)vb,
            (const bf16*)k_sel, (const bf16*)v_sel, a, scale2, (bf16*)out, o_part, ml_part);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const Shape& s, void* ws, void* out, hipStream_t st) {
  const AttnGeom a = attn_geom(s);
  const size_t rows = (size_t)a.nunits * a.nks * a.rpad;
  const bf16* o_part = static_cast<const bf16*>(ws);
  const float2* ml_part = reinterpret_cast<const float2*>(static_cast<char*>(ws) + align256(rows * s.D * sizeof(bf16)));
  const int64_t n = (int64_t)a.nunits * s.B * s.G * (s.D / 4);
  const dim3 grid((unsigned)((n + 63) / 64));
  if (s.D == 128)
    klaunch(attn_combine_kernel<128>, grid, 64, 0, st, o_part, ml_part, a, (bf16*)out);
  else
    klaunch(attn_combine_kernel<64>, grid, 64, 0, st, o_part, ml_part, a, (bf16*)out);
  return hipGetLastError();
}

}  // namespace herald
