// B-query block attention over the selected subset plus the step's in-block keys,
// one denoising step per call (HERALD abstract on the mlsift "KV cache offloading"
// listing: the denoising phase reuses the selected subset T times; HERALD v3
// abstract: the final top-K subset). No mask.
//
// For KV head g the B*G query rows (b, h in g) share the keys
//   key i < topk:          k_sel[s][g][i]           (values: v_sel, stored d-major)
//   key topk + b':         k_blk[s][b'][g]           (values: v_blk[s][b'][g])
// bf16 path (attn_kernel): a workgroup takes up to 128 rows (4 waves x RT 16-row
// tiles) and a contiguous split of the keys, in 64-key blocks staged in LDS (K
// rows, and V^T). Per block: S^T = K.Q^T with v_mfma_f32_16x16x32_bf16 (keys on
// M, query rows on N, Q fragments held in registers), an online softmax in base 2
// per query row, then O^T += V^T.P^T, where P^T comes straight from the S^T
// accumulators (each lane already holds its query row's probabilities; the key
// order inside the 32-wide contraction is permuted the same way on the V^T side).
// With one key split the workgroup writes the output; with several it writes
// unnormalised fp32 partials that attn_combine_kernel merges.
// fp32 path (attn_f32_kernel): one workgroup per query row, VALU.
#include "common.hpp"
#include "kernels.hpp"

namespace herald {

template <int D, int RT>
__global__ __launch_bounds__(256) void attn_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kb,
                                                   const bf16* __restrict__ vb, const bf16* __restrict__ k_sel,
                                                   const bf16* __restrict__ v_sel, int B, int Hq, int Hkv, int G,
                                                   int topk, int64_t ldv, float scale2, int nsplit, int kps,
                                                   int rpad, int nunits, int nrg, bf16* __restrict__ out,
                                                   float* __restrict__ o_part, float2* __restrict__ ml) {
  constexpr int KB = kAttnKeyBlock;
  constexpr int LDK = D + 8;   // K tile row stride (elements)
  constexpr int LDV = KB + 8;  // V^T tile row stride (elements)
  __shared__ __align__(16) bf16 Ks[KB * LDK];
  __shared__ __align__(16) bf16 Vt[D * LDV];
  // 1-D grid, XCD-aware: workgroups are dispatched round-robin over the 8 XCDs, so
  // workgroup x runs on XCD x % 8. The row groups of one (unit, key split) item are
  // placed on the same XCD one after the other and share its L2 for the K/V blocks.
  const int x = blockIdx.x;
  const int kx = x >> 3;
  const int item = (kx / nrg) * 8 + (x & 7);
  const int rg = kx % nrg;
  if (item >= nunits * nsplit) return;
  const int sp = item % nsplit, unit = item / nsplit;
  const int s = unit / Hkv, g = unit % Hkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int R = B * G;
  const int NK = topk + B;
  const int kbeg = sp * kps, kend = min(NK, kbeg + kps);
  const int row0 = rg * (64 * RT) + w * (16 * RT);

  uint4 qf[RT][D / 32];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = row0 + rt * 16 + (lane & 15);
    const bf16* qr = nullptr;
    if (r < R) qr = q + (((int64_t)s * B + r / G) * Hq + g * G + r % G) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qf[rt][ks] = qr ? ld16(qr + ks * 32 + (lane >> 4) * 8) : make_uint4(0, 0, 0, 0);
  }

  f32x4_t o[D / 16][RT];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) o[dt][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[RT], l[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    l[rt] = 0.f;
  }

  const bf16* ksrc = k_sel + (int64_t)unit * topk * D;
  const bf16* vsrc = v_sel + (int64_t)unit * D * ldv;

  // Blocks that lie wholly inside the selected subset are prefetched into
  // registers one block ahead (16-byte loads of K rows and of V^T rows); the block
  // that reaches the in-block keys is staged element by element.
  constexpr int CPR = D / 8;                  // 16-byte chunks per K row
  constexpr int KCH = KB * CPR / 256;         // K chunks per thread
  constexpr int VCH = D * (KB / 8) / 256;     // V^T chunks per thread
  uint4 kreg[KCH], vreg[VCH];
  auto prefetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = threadIdx.x + i * 256;
      kreg[i] = ld16(ksrc + (int64_t)(k0 + c / CPR) * D + (c % CPR) * 8);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = threadIdx.x + i * 256;
      vreg[i] = ld16(vsrc + (int64_t)(c / (KB / 8)) * ldv + k0 + (c % (KB / 8)) * 8);
    }
  };
  if (kbeg + KB <= topk) prefetch(kbeg);

  for (int k0 = kbeg; k0 < kend; k0 += KB) {
    // ---- stage K rows and V^T for keys [k0, k0+KB)
    if (k0 + KB <= topk) {
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int c = threadIdx.x + i * 256;
        *reinterpret_cast<uint4*>(&Ks[(c / CPR) * LDK + (c % CPR) * 8]) = kreg[i];
      }
#pragma unroll
      for (int i = 0; i < VCH; ++i) {
        const int c = threadIdx.x + i * 256;
        *reinterpret_cast<uint4*>(&Vt[(c / (KB / 8)) * LDV + (c % (KB / 8)) * 8]) = vreg[i];
      }
    } else {
      for (int c = threadIdx.x; c < KB * CPR; c += 256) {
        const int r = c / CPR, ch = c % CPR;
        const int kk = k0 + r;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (kk < kend) {
          if (kk < topk) val = ld16(ksrc + (int64_t)kk * D + ch * 8);
          else val = ld16(kb + (((int64_t)s * B + (kk - topk)) * Hkv + g) * D + ch * 8);
        }
        *reinterpret_cast<uint4*>(&Ks[r * LDK + ch * 8]) = val;
      }
      for (int c = threadIdx.x; c < D * KB; c += 256) {
        const int e = c % D, r = c / D;
        const int kk = k0 + r;
        bf16 val = 0;
        if (kk < kend)
          val = kk < topk ? vsrc[(int64_t)e * ldv + kk] : vb[(((int64_t)s * B + (kk - topk)) * Hkv + g) * D + e];
        Vt[e * LDV + r] = val;
      }
    }
    __syncthreads();
    if (k0 + KB < kend && k0 + 2 * KB <= topk) prefetch(k0 + KB);

    // ---- S^T = K Q^T: lane holds keys mt*16 + 4*(lane/16) + i of query row lane%16
    f32x4_t sacc[4][RT];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) sacc[mt][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const uint4 a = *reinterpret_cast<const uint4*>(&Ks[(mt * 16 + (lane & 15)) * LDK + ks * 32 + (lane >> 4) * 8]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) sacc[mt][rt] = mfma16x16x32(a, qf[rt][ks], sacc[mt][rt]);
      }

    // ---- online softmax (base 2) and P^T fragments. The scale is folded into one FMA;
    //      the output is rescaled only when some row's running max grows (otherwise
    //      every factor is exactly 1); only the last block of a split can hold masked keys.
    const bool partial = k0 + KB > kend;
    uint4 bp[2][RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float bm = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (partial && k0 + mt * 16 + (lane >> 4) * 4 + i >= kend) sacc[mt][rt][i] = -INFINITY;
          bm = fmaxf(bm, sacc[mt][rt][i]);
        }
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float mn = fmaxf(m[rt], bm * scale2);
      if (__ballot(mn > m[rt])) {
        const float alpha = fast_exp2(m[rt] - mn);
        l[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt][rt] *= alpha;
      }
      m[rt] = mn;
      float p[4][4];
      float ps = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[mt][i] = fast_exp2(fmaf(sacc[mt][rt][i], scale2, -mn));
          ps += p[mt][i];
        }
      l[rt] += ps;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        bp[h2][rt] = make_uint4(pack_bf16x2(p[2 * h2][0], p[2 * h2][1]), pack_bf16x2(p[2 * h2][2], p[2 * h2][3]),
                                pack_bf16x2(p[2 * h2 + 1][0], p[2 * h2 + 1][1]),
                                pack_bf16x2(p[2 * h2 + 1][2], p[2 * h2 + 1][3]));
    }

    // ---- O^T += V^T P^T; contraction element j of lane l <-> key h2*32 + 4*(l/16) + j (j<4)
    //      or h2*32 + 16 + 4*(l/16) + j-4 (j>=4), matching the S^T accumulator layout
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const bf16* vr = &Vt[(dt * 16 + (lane & 15)) * LDV + h2 * 32 + (lane >> 4) * 4];
        const uint2 lo = *reinterpret_cast<const uint2*>(vr);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16);
        const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) o[dt][rt] = mfma16x16x32(a, bp[h2][rt], o[dt][rt]);
      }
    __syncthreads();
  }

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    l[rt] += __shfl_xor(l[rt], 16);
    l[rt] += __shfl_xor(l[rt], 32);
  }
  if (nsplit == 1) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = row0 + rt * 16 + (lane & 15);
      if (r >= R) continue;
      bf16* orow = out + (((int64_t)s * B + r / G) * Hq + g * G + r % G) * D;
      const float inv = 1.f / l[rt];
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const f32x4_t v = o[dt][rt];
        *reinterpret_cast<uint2*>(orow + dt * 16 + (lane >> 4) * 4) =
            make_uint2(pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv));
      }
    }
  } else {
    const int64_t pbase = ((int64_t)unit * nsplit + sp) * rpad;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = row0 + rt * 16 + (lane & 15);
      float* orow = o_part + (pbase + r) * D;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        *reinterpret_cast<float4*>(orow + dt * 16 + (lane >> 4) * 4) =
            make_float4(o[dt][rt][0], o[dt][rt][1], o[dt][rt][2], o[dt][rt][3]);
      if (lane < 16) ml[pbase + r] = make_float2(m[rt], l[rt]);
    }
  }
}

// Merges the key splits of one (sequence, KV head): 4 output dimensions per thread.
// All split partials are loaded before any is used (nsplit <= kAttnMaxSplits).
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ o_part,
                                                           const float2* __restrict__ ml, int B, int Hq, int Hkv,
                                                           int G, int D, int nsplit, int rpad,
                                                           bf16* __restrict__ out) {
  const int unit = blockIdx.y;
  const int s = unit / Hkv, g = unit % Hkv;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int r = idx / (D / 4), e = (idx % (D / 4)) * 4;
  if (r >= B * G) return;
  const int64_t base = (int64_t)unit * nsplit * rpad + r;
  float2 p[kAttnMaxSplits];
  float4 o[kAttnMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kAttnMaxSplits; ++sp) {
    if (sp < nsplit) {
      p[sp] = ml[base + (int64_t)sp * rpad];
      o[sp] = *reinterpret_cast<const float4*>(o_part + (base + (int64_t)sp * rpad) * D + e);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kAttnMaxSplits; ++sp)
    if (sp < nsplit) M = fmaxf(M, p[sp].x);
  float Lsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int sp = 0; sp < kAttnMaxSplits; ++sp) {
    if (sp < nsplit) {
      const float wgt = fast_exp2(p[sp].x - M);
      Lsum += wgt * p[sp].y;
      acc.x += wgt * o[sp].x;
      acc.y += wgt * o[sp].y;
      acc.z += wgt * o[sp].z;
      acc.w += wgt * o[sp].w;
    }
  }
  const float inv = 1.f / Lsum;
  *reinterpret_cast<uint2*>(out + (((int64_t)s * B + r / G) * Hq + g * G + r % G) * D + e) =
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

// 16-row MFMA tiles per wave: one, so that a workgroup takes 64 query rows and the
// grid holds more workgroups per CU to hide latency.
static int attn_rt(const Shape&) { return 1; }

static int attn_row_groups(const Shape& s) {
  const int rows = 64 * attn_rt(s);
  return (s.B * s.G + rows - 1) / rows;
}

int attn_splits(const Shape& s, int* keys_per_split) {
  const int NK = s.topk + s.B;
  const int nblk = (NK + kAttnKeyBlock - 1) / kAttnKeyBlock;
  if (!s.bf16) {
    *keys_per_split = nblk * kAttnKeyBlock;
    return 1;
  }
  const int64_t units = (int64_t)s.nseq * s.Hkv * attn_row_groups(s);
  const int64_t want = std::max<int64_t>(1, (kAttnTargetWorkgroups + units - 1) / units);
  int bps = (int)std::max<int64_t>(kAttnMinBlocksPerSplit, (nblk + want - 1) / want);
  bps = std::max(bps, (nblk + kAttnMaxSplits - 1) / kAttnMaxSplits);
  const int nsplit = (nblk + bps - 1) / bps;
  bps = (nblk + nsplit - 1) / nsplit;  // even out the splits
  *keys_per_split = bps * kAttnKeyBlock;
  return (NK + *keys_per_split - 1) / *keys_per_split;
}

int attn_rpad(const Shape& s) { return attn_row_groups(s) * 64 * attn_rt(s); }

hipError_t launch_attn(const Shape& s, const void* q, const void* kb, const void* vb, const void* k_sel,
                       const void* v_sel, void* out, const AttnWs& ws, hipStream_t st) {
  const float scale2 = s.scale * kLog2e;
  const int64_t ldv = vsel_ld(s.topk);
  if (!s.bf16) {
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
  const int nunits = s.nseq * s.Hkv, nrg = attn_row_groups(s);
  const int nitems = nunits * ws.nsplit;
  // items padded to a multiple of 8, times the row groups
  dim3 grid((unsigned)(((nitems + 7) / 8) * 8 * nrg), 1, 1);
  const int rpad = attn_rpad(s);
#define HERALD_ATTN(DD, RR)                                                                                         \
  klaunch(attn_kernel<DD, RR>, grid, 256, 0, st, (const bf16*)q, (const bf16*)kb, (const bf16*)vb, (const bf16*)k_sel,  \
                                            (const bf16*)v_sel, s.B, s.Hq, s.Hkv, s.G, s.topk, ldv, scale2,         \
                                            ws.nsplit, ws.keys_per_split, rpad, nunits, nrg, (bf16*)out, ws.o_part, ws.ml)
  if (s.D == 128) {
    if (attn_rt(s) == 1) HERALD_ATTN(128, 1);
    else HERALD_ATTN(128, 2);
  } else {
    if (attn_rt(s) == 1) HERALD_ATTN(64, 1);
    else HERALD_ATTN(64, 2);
  }
#undef HERALD_ATTN
  return hipGetLastError();
}

hipError_t launch_attn_combine(const Shape& s, const AttnWs& ws, void* out, hipStream_t st) {
  dim3 grid((s.B * s.G * (s.D / 4) + 255) / 256, s.nseq * s.Hkv);
  klaunch(attn_combine_kernel, grid, 256, 0, st, ws.o_part, ws.ml, s.B, s.Hq, s.Hkv, s.G, s.D, ws.nsplit, attn_rpad(s),
                                            (bf16*)out);
  return hipGetLastError();
}

}  // namespace herald
