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
// bf16 path (attn_kernel). A workgroup of 8 waves takes up to four 16-row query tiles
// of one (sequence, KV head) and a range of its key blocks (all of them unless the
// subset is long). Its two groups of 4 waves take alternate blocks, each wave one
// tile, and their partial results are merged through LDS at the end. Subset blocks
// stream into a ring of LDS stages with coalesced direct-to-LDS loads
// (global_load_lds_dwordx4, no registers held, up to four blocks in flight); K rows
// and V^T rows keep their 16-byte chunks XOR-permuted so that the 16 rows one MFMA
// fragment read touches fall in distinct banks. The in-block keys arrive key-major
// and are transposed into a stage through registers. Per block a wave computes
// S^T = K.Q^T on v_mfma_f32_16x16x32_bf16 (keys on M, its query rows on N, Q
// fragments held in registers), an online base-2 softmax per query row, then
// O^T += V^T.P^T with P^T taken from the S^T accumulators; the keys of a block are
// assigned to MFMA rows so that the 32-key contraction of the second product runs
// over consecutive keys. The running max is raised (and the output rescaled) only
// when a row's max grows by more than 8 (base 2): probabilities then stay below
// 2^8, exact in fp32 and bf16 range, and both sums use the same reference.
// With several key ranges each workgroup writes a partial (fp32 max and sum, the
// unnormalised output in fp32) that attn_combine_kernel merges; the output is rounded
// to bf16 once, at the end. The running sum adds the probabilities as rounded to bf16
// for the second product, so the applied weights are normalised up to fp32 rounding.
// Built with -fno-honor-nans (non-finite inputs are outside the contract): the max
// reductions then need no NaN-quieting operations.
// fp32 path (attn_f32_kernel): four query rows per workgroup, VALU, keys in chunks of 128.
#include "common.hpp"
#include "kernels.hpp"

namespace herald {

// Row m of key tile mt within a 64-key block -> key offset in the block. Tiles 2c and
// 2c+1 cover keys [32c, 32c+32); lane group j of the second product then contracts
// over keys 32c + 8j .. 32c + 8j + 7, which the accumulators of lane group j hold.
__device__ __forceinline__ int attn_key_of(int mt, int m) {
  return (mt >> 1) * 32 + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3);
}

// 16-byte chunk c of K row r is stored at chunk c ^ attn_kswz(r): the rows one MFMA
// operand reads (attn_key_of(mt, 0..15)) map to 16 distinct values.
template <int D>
__device__ __forceinline__ int attn_kswz(int r) {
  return ((r & 3) | ((r >> 1) & 12)) & (D / 8 - 1);
}
// 16-byte chunk c of V^T row e (64 keys, 128 bytes) is stored at chunk c ^ attn_vswz(e).
__device__ __forceinline__ int attn_vswz(int e) { return (e >> 1) & 7; }

template <int D>
__global__ __launch_bounds__(512) void attn_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kb,
                                                   const bf16* __restrict__ vb, const bf16* __restrict__ k_sel,
                                                   const bf16* __restrict__ v_sel, AttnGeom a, float scale2,
                                                   bf16* __restrict__ out, float* __restrict__ o_part,
                                                   float2* __restrict__ ml_part) {
  constexpr int NW = 8;              // waves: two groups of four
  constexpr int KB = kAttnKeyBlock;  // 64
  constexpr int KS = D / 32;         // contraction steps of S^T = K.Q^T
  constexpr int DT = D / 16;         // 16-dim output tiles
  constexpr int CPR = D / 8;         // 16-byte chunks per K row
  constexpr int RPI = 64 / CPR;      // K rows per load instruction
  constexpr int NT = NW * 64;
  constexpr int NCH = KB * CPR;      // 16-byte chunks of K (and of V^T) per block
  constexpr int NIK = NCH / NT;      // direct-to-LDS instructions per wave per block, K
  constexpr int NIV = NCH / NT;      //                                                V^T
  constexpr int NIPB = NIK + NIV;
  constexpr int STAGE = 2 * KB * D;  // elements per stage (K then V^T)
  constexpr float kRaise = 8.f;      // the running max moves only when exceeded by this
  static_assert(NIK >= 1 && 3 * NIPB < 64, "vmcnt budget");
  extern __shared__ __align__(16) bf16 stages[];

  // 1-D grid, XCD-aware: workgroup x runs on XCD x % 8 and each XCD takes a contiguous
  // range of items; the row splits of one key range are adjacent and share an L2.
  const int per = gridDim.x >> 3;
  const int li = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (li >= a.nitems) return;
  auto qdiv = [](uint32_t x, uint32_t rcp) { return rcp ? __umulhi(x, rcp) : x; };  // x / d, rcp as in AttnGeom
  const int q1 = (int)qdiv((uint32_t)li, a.rcp_nrs), q2 = (int)qdiv((uint32_t)q1, a.rcp_nks);
  const int rs = li - q1 * a.nrs, ksp = q1 - q2 * a.nks, unit = q2;
  const int B = a.B, G = a.G, topk = a.topk;
  const int s = (int)qdiv((uint32_t)unit, a.rcp_hkv), g = unit - s * a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, qd = lane >> 4, lr = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2, wl = w & 3;
  const int R = B * G, nA = (topk + KB - 1) / KB;
  const int b0 = ksp * a.bps, b1 = min(nA + 1, b0 + a.bps);
  const int has_ib = b1 == nA + 1 ? 1 : 0;  // the in-block keys belong to the last range
  const int nb = b1 - b0;                    // blocks of this workgroup: list index 0 is the
  const int nst = a.nst;                     // in-block block when it has one, then subset
  const int tile = rs * a.tpw + wl;
  const bool has_tile = wl < a.tpw && tile * 16 < R;

  const bf16* ksrc = k_sel + (int64_t)unit * topk * D;
  const bf16* vsrc = v_sel + (int64_t)unit * D * a.ldv;
  const bf16* kbb = kb + ((int64_t)s * B * a.Hkv + g) * D;  // in-block key b at kbb + b * Hkv * D
  const bf16* vbb = vb + ((int64_t)s * B * a.Hkv + g) * D;
  const int64_t bstride = (int64_t)a.Hkv * D;
  const uint32_t lds0 = (uint32_t)(uintptr_t)stages;

  // ---- per-lane parts of the direct-to-LDS addresses (the block only adds a base)
  int koff[NIK], voff[NIV], krow[NIK];
#pragma unroll
  for (int u = 0; u < NIK; ++u) {
    const int r = (u * NW + w) * RPI + lane / CPR;
    krow[u] = r;
    koff[u] = (lane % CPR ^ attn_kswz<D>(r)) * 8;
  }
#pragma unroll
  for (int u = 0; u < NIV; ++u) {
    const int e = (u * NW + w) * 8 + lane / 8;
    voff[u] = e * (int)a.ldv + ((lane % 8) ^ attn_vswz(e)) * 8;
  }
  // list index i >= has_ib is subset block b0 + i - has_ib, in stage i % nst
  auto issue = [&](int i) {
    const int blk = b0 + i - has_ib;
    const uint32_t sk = lds0 + (uint32_t)((i % nst) * STAGE) * 2u;
    const uint32_t sv = sk + KB * D * 2;
    const bool full = blk * KB + KB <= topk;
#pragma unroll
    for (int u = 0; u < NIK; ++u) {
      const int key = full ? blk * KB + krow[u] : min(blk * KB + krow[u], topk - 1);
      lds_dma16(ksrc + (int64_t)key * D + koff[u], sk + (uint32_t)((u * NW + w) * RPI * D) * 2u);
    }
#pragma unroll
    for (int u = 0; u < NIV; ++u)
      lds_dma16(vsrc + (int64_t)blk * KB + voff[u], sv + (uint32_t)((u * NW + w) * 8 * KB) * 2u);
  };
  int next = has_ib;  // next list index to fetch
  for (; next < min(nb, nst); ++next) issue(next);

  // ---- query fragments of this wave's tile
  uint4 qf[KS];
  {
    const int r = tile * 16 + lr, rb = (int)qdiv((uint32_t)r, a.rcp_g);  // block query of row r
    const bf16* qr =
        has_tile && r < R ? q + (((int64_t)s * B + rb) * a.Hq + g * G + (r - rb * G)) * D + qd * 8 : nullptr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = qr ? ld16(qr + ks * 32) : make_uint4(0, 0, 0, 0);
  }
  // ---- in-block keys (list index 0, stage 0): K rows and V^T (transposed) via registers
  if (has_ib) {
    constexpr int PT = NCH / NT;
    uint4 kst[PT], vst[PT];
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = tid + i * NT;
      const int r = c / CPR, ch = c % CPR;
      kst[i] = vst[i] = make_uint4(0, 0, 0, 0);
      if (r < B) {
        kst[i] = ld16(kbb + r * bstride + ch * 8);
        vst[i] = ld16(vbb + r * bstride + ch * 8);
      }
    }
    bf16* sk = stages;
    bf16* sv = stages + KB * D;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = tid + i * NT;
      const int r = c / CPR, ch = c % CPR;
      *reinterpret_cast<uint4*>(sk + r * D + ((ch ^ attn_kswz<D>(r)) * 8)) = kst[i];
      const uint32_t xs[4] = {vst[i].x, vst[i].y, vst[i].z, vst[i].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int e0 = ch * 8 + 2 * t;
        sv[e0 * KB + (((r >> 3) ^ attn_vswz(e0)) * 8) + (r & 7)] = (bf16)(xs[t] & 0xffffu);
        sv[(e0 + 1) * KB + (((r >> 3) ^ attn_vswz(e0 + 1)) * 8) + (r & 7)] = (bf16)(xs[t] >> 16);
      }
    }
  }

  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  // The query fragments (and in-block rows) are the only loads the compiler tracks.
  // Waiting for them here, once, on every path, keeps the compiler from placing that
  // wait inside the loop, where (the direct-to-LDS transfers being invisible to it) it
  // would be a full vmcnt(0) in every round, draining the blocks prefetched for the
  // next round before this one computes.
  wait_vm<0>();

  for (int j = 0; j < nb; j += 2) {
    // wait for this wave's loads of the subset blocks among j, j + 1
    const int need = min(j + 1, nb - 1);
    if (need >= has_ib) {
      const int later = next - 1 - need;  // subset blocks fetched after it
      if (later <= 0) wait_vm<0>();
      else if (later == 1) wait_vm<NIPB>();
      else if (later == 2) wait_vm<2 * NIPB>();
      else wait_vm<3 * NIPB>();
    }
    __syncthreads();  // blocks j, j + 1 are in LDS; every wave is done with j - 2, j - 1
    for (; next < nb && next < j + nst; ++next) issue(next);

    const int i = j + grp;  // this group's block
    if (i >= nb || !has_tile) continue;
    const bf16* sk = stages + (i % nst) * STAGE;
    const bf16* sv = sk + KB * D;
    const int valid = (i < has_ib) ? B : min(KB, topk - (b0 + i - has_ib) * KB);

    // ---- S^T = K Q^T: lane holds keys attn_key_of(mt, 4*qd + i) of query row lr. All
    //      fragment reads of a product are issued before its first MFMA; the V^T
    //      fragments are read while the softmax runs.
    uint4 kf[4][KS];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int r = attn_key_of(mt, lr);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[mt][ks] = *reinterpret_cast<const uint4*>(sk + r * D + (((ks * 4 + qd) ^ attn_kswz<D>(r)) * 8));
    }
    f32x4_t sacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sacc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) sacc[mt] = mfma16x16x32(kf[mt][ks], qf[ks], sacc[mt]);
    uint4 vf[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int e = dt * 16 + lr;
        vf[dt][h2] = *reinterpret_cast<const uint4*>(sv + e * KB + (((h2 * 4 + qd) ^ attn_vswz(e)) * 8));
      }

    // ---- online softmax (base 2) with the scale folded into one FMA
    if (valid < KB) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (attn_key_of(mt, 4 * qd + t) >= valid) sacc[mt][t] = -INFINITY;
    }
    float bm = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                     fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
    bm = fmaxf(bm, fmaxf(fmaxf(fmaxf(sacc[2][0], sacc[2][1]), fmaxf(sacc[2][2], sacc[2][3])),
                         fmaxf(fmaxf(sacc[3][0], sacc[3][1]), fmaxf(sacc[3][2], sacc[3][3]))));
    bm = xmax4(bm) * scale2;
    if (__ballot(bm > m + kRaise)) {
      const float mn = fmaxf(m, bm);
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      m = mn;
    }
    float p[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int t = 0; t < 4; ++t) p[mt][t] = fast_exp2(fmaf(sacc[mt][t], scale2, -m));
    uint4 bp[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      bp[h2] = make_uint4(pack_bf16x2(p[2 * h2][0], p[2 * h2][1]), pack_bf16x2(p[2 * h2][2], p[2 * h2][3]),
                          pack_bf16x2(p[2 * h2 + 1][0], p[2 * h2 + 1][1]),
                          pack_bf16x2(p[2 * h2 + 1][2], p[2 * h2 + 1][3]));
    // the normaliser sums the probabilities as the product below uses them (rounded to
    // bf16), so the weights applied to the values sum to one up to fp32 rounding: a query
    // whose attention falls on a few keys gets their values back without the weights'
    // bf16 rounding. Two dot2 chains of four pairs each.
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      ps0 = add_bf16x2(bp[h2].x, ps0);
      ps1 = add_bf16x2(bp[h2].y, ps1);
      ps0 = add_bf16x2(bp[h2].z, ps0);
      ps1 = add_bf16x2(bp[h2].w, ps1);
    }
    l += ps0 + ps1;

    // ---- O^T += V^T P^T over the two 32-key halves of the block
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) o[dt] = mfma16x16x32(vf[dt][h2], bp[h2], o[dt]);
  }
  l = xsum4(l);

  // ---- merge the two groups through LDS (the stages are free once all waves are here)
  constexpr int LDO = D + 4;
  float* xo = reinterpret_cast<float*>(stages);  // [4 tiles][16 rows][LDO]
  float2* xml = reinterpret_cast<float2*>(xo + 4 * 16 * LDO);
  __syncthreads();
  if (grp == 1 && has_tile) {
    float* orow = xo + (wl * 16 + lr) * LDO + qd * 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(orow + dt * 16) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (qd == 0) xml[wl * 16 + lr] = make_float2(m, l);
  }
  __syncthreads();
  if (grp == 1 || !has_tile) return;
  {
    const float2 mb = xml[wl * 16 + lr];
    const float M = fmaxf(m, mb.x);
    const float fa = fast_exp2(m - M), fb = mb.x == -INFINITY ? 0.f : fast_exp2(mb.x - M);
    l = l * fa + mb.y * fb;
    m = M;
    const float* orow = xo + (wl * 16 + lr) * LDO + qd * 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const float4 ob = *reinterpret_cast<const float4*>(orow + dt * 16);
      o[dt][0] = o[dt][0] * fa + ob.x * fb;
      o[dt][1] = o[dt][1] * fa + ob.y * fb;
      o[dt][2] = o[dt][2] * fa + ob.z * fb;
      o[dt][3] = o[dt][3] * fa + ob.w * fb;
    }
  }
  const int r = tile * 16 + lr;
  if (a.nks == 1) {
    if (r >= R) return;
    const int rb = (int)qdiv((uint32_t)r, a.rcp_g);
    bf16* orow = out + (((int64_t)s * B + rb) * a.Hq + g * G + (r - rb * G)) * D + qd * 4;
    const float inv = 1.f / l;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<uint2*>(orow + dt * 16) =
          make_uint2(pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv), pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv));
  } else {
    const int64_t prow = ((int64_t)unit * a.nks + ksp) * a.rpad + r;
    float* orow = o_part + prow * D + qd * 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(orow + dt * 16) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (qd == 0) ml_part[prow] = make_float2(m, l);
  }
}

// Merges the key ranges of one (sequence, KV head): 8 output dimensions per thread
// (two 16-byte fp32 loads per range, one 16-byte bf16 store), the ranges taken 8 at a
// time (loads first) with a running (max, sum).
template <int D>
__global__ __launch_bounds__(kAttnCombineThreads) void attn_combine_kernel(const float* __restrict__ o_part,
                                                                           const float2* __restrict__ ml_part,
                                                                           AttnGeom a, bf16* __restrict__ out) {
  constexpr int CH = 8, TPR = D / 8;  // threads per output row
  const int idx = blockIdx.x * kAttnCombineThreads + threadIdx.x;
  const int R = a.B * a.G;
  const int per_unit = R * TPR;
  const int unit = a.rcp_pu ? (int)__umulhi((uint32_t)idx, a.rcp_pu) : idx / per_unit;
  if (unit >= a.nunits) return;
  const int r = (idx - unit * per_unit) / TPR, e = (idx % TPR) * 8;
  const int s = a.rcp_hkv ? (int)__umulhi((uint32_t)unit, a.rcp_hkv) : unit, g = unit - s * a.Hkv;
  const int64_t base = (int64_t)unit * a.nks * a.rpad + r;
  float M = -INFINITY, L = 0.f;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int k0 = 0; k0 < a.nks; k0 += CH) {
    float2 p[CH];
    float4 va[CH], vc[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      p[j] = make_float2(-INFINITY, 0.f);
      va[j] = vc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (k0 + j < a.nks) {
        const int64_t row = base + (int64_t)(k0 + j) * a.rpad;
        p[j] = ml_part[row];
        va[j] = *reinterpret_cast<const float4*>(o_part + row * D + e);
        vc[j] = *reinterpret_cast<const float4*>(o_part + row * D + e + 4);
      }
    }
    float mc = M;
#pragma unroll
    for (int j = 0; j < CH; ++j) mc = fmaxf(mc, p[j].x);
    const float alpha = fast_exp2(M - mc);  // 0 on the first chunk (M = -inf)
    L *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= alpha;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (p[j].x == -INFINITY) continue;
      const float wgt = fast_exp2(p[j].x - mc);
      L += wgt * p[j].y;
      const float x8[8] = {va[j].x, va[j].y, va[j].z, va[j].w, vc[j].x, vc[j].y, vc[j].z, vc[j].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += wgt * x8[i];
    }
    M = mc;
  }
  const float inv = 1.f / L;
  const int rb = a.rcp_g ? (int)__umulhi((uint32_t)r, a.rcp_g) : r;  // block query of row r
  *reinterpret_cast<uint4*>(out + (((int64_t)s * a.B + rb) * a.Hq + g * a.G + (r - rb * a.G)) * D + e) =
      make_uint4(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                 pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv));
}

// fp32 path: a workgroup takes four query rows of one (sequence, KV head) and walks
// the keys in chunks of 128. Logits: one key per thread (its row read straight from
// memory), two of the four query rows per thread from LDS (broadcast reads). Online
// base-2 softmax: one wave per query row. Output: the chunk's values staged d-major in
// LDS (rows padded by one word, so the 64 lanes of a read hit 64 banks), each thread
// accumulating D/64 output elements of its wave's row.
template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ kb,
                                                       const float* __restrict__ vb, const float* __restrict__ k_sel,
                                                       const float* __restrict__ v_sel, int B, int Hq, int Hkv,
                                                       int G, int topk, int64_t ldv, float scale2,
                                                       float* __restrict__ out) {
  constexpr int KC = 128, RB = 4, EP = D / 64;
  __shared__ __align__(16) float qs[RB][D];
  __shared__ float xs[RB][KC];
  extern __shared__ float vs[];  // [D][KC + 1]
  const int g = blockIdx.y, s = blockIdx.z;
  const int R = B * G, r0 = blockIdx.x * RB;
  const int64_t unit = (int64_t)s * Hkv + g;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  auto qrow = [&](int r) { return q + (((int64_t)s * B + r / G) * Hq + g * G + r % G) * D; };
  for (int i = threadIdx.x; i < RB * D; i += 256) qs[i / D][i % D] = qrow(min(r0 + i / D, R - 1))[i % D];
  const int NK = topk + B;
  float m = -INFINITY, l = 0.f, acc[EP];
#pragma unroll
  for (int j = 0; j < EP; ++j) acc[j] = 0.f;
  for (int k0 = 0; k0 < NK; k0 += KC) {
    const int n = min(KC, NK - k0);
    __syncthreads();  // qs ready; the previous chunk's xs and vs consumed
    {
      const int kk = threadIdx.x % KC, rp = (threadIdx.x / KC) * 2;
      float x0 = -INFINITY, x1 = -INFINITY;
      if (kk < n) {
        const int key = k0 + kk;
        const float* kr = key < topk ? k_sel + (unit * topk + key) * D
                                     : kb + (((int64_t)s * B + (key - topk)) * Hkv + g) * D;
        float d0 = 0.f, d1 = 0.f;
#pragma unroll 8
        for (int e = 0; e < D; e += 4) {
          const float4 kv = *reinterpret_cast<const float4*>(kr + e);
          const float4 qa = *reinterpret_cast<const float4*>(&qs[rp][e]);
          const float4 qb = *reinterpret_cast<const float4*>(&qs[rp + 1][e]);
          d0 = fmaf(qa.w, kv.w, fmaf(qa.z, kv.z, fmaf(qa.y, kv.y, fmaf(qa.x, kv.x, d0))));
          d1 = fmaf(qb.w, kv.w, fmaf(qb.z, kv.z, fmaf(qb.y, kv.y, fmaf(qb.x, kv.x, d1))));
        }
        x0 = d0 * scale2;
        x1 = d1 * scale2;
      }
      xs[rp][kk] = x0;
      xs[rp + 1][kk] = x1;
    }
    {
      constexpr int NV = D * KC / 256;  // values per thread: all loads first, then the LDS stores
      float vv[NV];
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int i = threadIdx.x + u * 256, e = i / KC, kk = i % KC, key = k0 + kk;
        vv[u] = 0.f;
        if (kk < n)
          vv[u] = key < topk ? v_sel[(unit * D + e) * ldv + key]
                             : vb[(((int64_t)s * B + (key - topk)) * Hkv + g) * D + e];
      }
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int i = threadIdx.x + u * 256;
        vs[(i / KC) * (KC + 1) + i % KC] = vv[u];
      }
    }
    __syncthreads();
    const float x0 = xs[w][lane], x1 = xs[w][lane + 64];
    float cm = fmaxf(x0, x1);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) cm = fmaxf(cm, __shfl_xor(cm, o));
    const float mn = fmaxf(m, cm);  // finite: every chunk holds at least one key
    const float al = fast_exp2(m - mn);
    const float p0 = fast_exp2(x0 - mn), p1 = fast_exp2(x1 - mn);
    float ps = p0 + p1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) ps += __shfl_xor(ps, o);
    l = l * al + ps;
    m = mn;
    __syncthreads();  // every wave has read its logits before they become weights
    xs[w][lane] = p0;
    xs[w][lane + 64] = p1;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < EP; ++j) {
      const float* vr = vs + (lane + 64 * j) * (KC + 1);
      float a = acc[j] * al;
      for (int kk = 0; kk < n; ++kk) a = fmaf(xs[w][kk], vr[kk], a);
      acc[j] = a;
    }
  }
  if (r0 + w < R) {
    float* o = out + (((int64_t)s * B + (r0 + w) / G) * Hq + g * G + (r0 + w) % G) * D;
#pragma unroll
    for (int j = 0; j < EP; ++j) o[lane + 64 * j] = acc[j] / l;
  }
}

// ------------------------------------------------------------------ host side

// Work split: up to four 16-row query tiles per workgroup, and key ranges of at most
// kAttnBlocksPerRange blocks.
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
  const int nblk = (s.topk + kAttnKeyBlock - 1) / kAttnKeyBlock + 1;
  // Four query tiles per workgroup; two when few (sequence, KV head) pairs leave the
  // chip idle even with the keys split: twice the workgroups (each pulling the same
  // keys for fewer rows), a larger target for the key split and ranges of 3 blocks.
  // Long subsets (more than kAttnBlocksPerRange blocks, e.g. attention over a whole
  // cache) fill the chip through the key split alone and keep four tiles, so the keys
  // are streamed for half as many row groups.
  a.tpw = std::min(ntiles, 4);
  int target = kAttnTargetWorkgroups, minrange = kAttnMaxStages;
  if (a.nunits * ((ntiles + 3) / 4) * 5 < kAttnFewPairs && nblk <= kAttnBlocksPerRange) {
    a.tpw = std::min(ntiles, 2);
    target = kAttnTargetWorkgroupsFew;
    minrange = 3;
  }
  a.nrs = (ntiles + a.tpw - 1) / a.tpw;
  a.rpad = ntiles * 16;
  // A workgroup keeps at most kAttnMaxStages blocks in flight, so one pulling a long
  // range is bound by memory latency: with few (sequence, KV head) pairs the keys are
  // split into ranges of about kAttnMaxStages blocks, to spread them over enough
  // workgroups (the ranges are then merged by attn_combine_kernel).
  const int groups = std::max(1, a.nunits * a.nrs);  // an empty batch (nseq = 0) launches nothing
  const int spread = std::min((target + groups - 1) / groups, (nblk + minrange - 1) / minrange);
  const int nks = std::max((nblk + kAttnBlocksPerRange - 1) / kAttnBlocksPerRange, spread);
  a.bps = (nblk + nks - 1) / nks;
  a.nks = (nblk + a.bps - 1) / a.bps;
  // a range of at most kAttnMaxStages blocks is fetched at once; longer ranges cycle
  // through kAttnMaxStages stages (two blocks in use, the next two in flight)
  a.nst = std::min(a.bps, kAttnMaxStages);
  // workgroup count in 64 bits: attn_fits refuses the shape before it could overflow
  const int64_t nitems = (int64_t)a.nunits * a.nrs * a.nks;
  a.nitems = nitems < (int64_t(1) << 31) ? (int)nitems : -1;
  auto rcp = [&](int d) -> uint32_t {
    if (d <= 1) return 0u;
    if ((uint64_t)nitems * (uint64_t)d >= (1ull << 32)) return 0xffffffffu;  // flagged by attn_fits
    return (uint32_t)(((1ull << 32) + (uint64_t)d - 1) / (uint64_t)d);
  };
  a.rcp_nrs = rcp(a.nrs);
  a.rcp_nks = rcp(a.nks);
  a.rcp_hkv = rcp(a.Hkv);
  a.rcp_g = a.G <= 1 ? 0u : (uint32_t)(((1ull << 32) + (uint64_t)a.G - 1) / (uint64_t)a.G);
  const uint64_t pu = (uint64_t)s.B * s.G * (s.D / 8), nidx = (uint64_t)a.nunits * pu;
  a.rcp_pu = nidx * pu < (1ull << 32) ? (uint32_t)(((1ull << 32) + pu - 1) / pu) : 0u;
  return a;
}

bool attn_fits(const Shape& s) {
  if (!s.bf16 || s.nseq == 0) return true;
  const AttnGeom a = attn_geom(s);
  return a.nitems > 0 && a.rcp_nrs != 0xffffffffu && a.rcp_nks != 0xffffffffu && a.rcp_hkv != 0xffffffffu;
}

int attn_splits(const Shape& s) { return s.bf16 ? attn_geom(s).nks : 1; }

size_t attn_ws_bytes(const Shape& s) {
  if (!s.bf16) return 0;
  const AttnGeom a = attn_geom(s);
  if (a.nks == 1) return 0;
  const size_t rows = (size_t)a.nunits * a.nks * a.rpad;
  return align256(rows * s.D * sizeof(float)) + align256(rows * sizeof(float2));
}

template <int D>
static size_t attn_smem(const AttnGeom& a) {
  const size_t stages = (size_t)a.nst * 2 * kAttnKeyBlock * D * sizeof(bf16);
  const size_t merge = (size_t)4 * 16 * (D + 4) * sizeof(float) + 4 * 16 * sizeof(float2);
  return std::max(stages, merge);
}

template <int D>
static hipError_t launch_attn_bf16(const AttnGeom& a, const void* q, const void* kb, const void* vb,
                                   const void* k_sel, const void* v_sel, void* out, void* ws, float scale2,
                                   hipStream_t st) {
  float* o_part = nullptr;
  float2* ml_part = nullptr;
  if (a.nks > 1) {
    const size_t rows = (size_t)a.nunits * a.nks * a.rpad;
    o_part = static_cast<float*>(ws);
    ml_part = reinterpret_cast<float2*>(static_cast<char*>(ws) + align256(rows * D * sizeof(float)));
  }
  // more workgroups than the reciprocal decode covers exactly (refused by attn_fits on the host)
  if (a.nitems <= 0 || a.rcp_nrs == 0xffffffffu || a.rcp_nks == 0xffffffffu || a.rcp_hkv == 0xffffffffu)
    return hipErrorInvalidConfiguration;
  const size_t smem = attn_smem<D>(a);
  hipError_t e = allow_smem((const void*)attn_kernel<D>, smem);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((a.nitems + 7) / 8 * 8));
  klaunch(attn_kernel<D>, grid, 512, smem, st, (const bf16*)q, (const bf16*)kb, (const bf16*)vb, (const bf16*)k_sel,
          (const bf16*)v_sel, a, scale2, (bf16*)out, o_part, ml_part);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const Shape& s, void* ws, void* out, hipStream_t st) {
  const AttnGeom a = attn_geom(s);
  const size_t rows = (size_t)a.nunits * a.nks * a.rpad;
  const float* o_part = static_cast<const float*>(ws);
  const float2* ml_part = reinterpret_cast<const float2*>(static_cast<char*>(ws) + align256(rows * s.D * sizeof(float)));
  const int64_t n = (int64_t)a.nunits * a.B * a.G * (s.D / 8);
  const dim3 grid((unsigned)((n + kAttnCombineThreads - 1) / kAttnCombineThreads));
  if (s.D == 128)
    klaunch(attn_combine_kernel<128>, grid, kAttnCombineThreads, 0, st, o_part, ml_part, a, (bf16*)out);
  else
    klaunch(attn_combine_kernel<64>, grid, kAttnCombineThreads, 0, st, o_part, ml_part, a, (bf16*)out);
  return hipGetLastError();
}

hipError_t launch_attn(const Shape& s, const void* q, const void* kb, const void* vb, const void* k_sel,
                       const void* v_sel, void* out, void* ws, hipStream_t st) {
  const float scale2 = s.scale * kLog2e;
  if (!s.bf16) {
    const int64_t ldv = vsel_ld(s.topk);
    const dim3 grid((s.B * s.G + 3) / 4, s.Hkv, s.nseq);
    const size_t smem = (size_t)s.D * 129 * sizeof(float);
    const void* kern = s.D == 128 ? (const void*)attn_f32_kernel<128> : (const void*)attn_f32_kernel<64>;
    hipError_t e = allow_smem(kern, smem);
    if (e != hipSuccess) return e;
    if (s.D == 128)
      klaunch(attn_f32_kernel<128>, grid, 256, smem, st, (const float*)q, (const float*)kb, (const float*)vb,
                                                 (const float*)k_sel, (const float*)v_sel, s.B, s.Hq, s.Hkv, s.G,
                                                 s.topk, ldv, scale2, (float*)out);
    else
      klaunch(attn_f32_kernel<64>, grid, 256, smem, st, (const float*)q, (const float*)kb, (const float*)vb,
                                                (const float*)k_sel, (const float*)v_sel, s.B, s.Hq, s.Hkv, s.G,
                                                s.topk, ldv, scale2, (float*)out);
    return hipGetLastError();
  }
  const AttnGeom a = attn_geom(s);
  if (s.D == 128) return launch_attn_bf16<128>(a, q, kb, vb, k_sel, v_sel, out, ws, scale2, st);
  return launch_attn_bf16<64>(a, q, kb, vb, k_sel, v_sel, out, ws, scale2, st);
}

}  // namespace herald
