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
// fp32 path (attn_f32_kernel): one 16-row query tile per workgroup, eight waves over the
// key tiles, v_mfma_f32_16x16x4_f32, partial results merged through LDS.
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
    // wave priority up while a product's MFMAs issue: the SIMD's other wave, in its
    // softmax, then fills the VALU slots between them
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) sacc[mt] = mfma16x16x32(kf[mt][ks], qf[ks], sacc[mt]);
    __builtin_amdgcn_s_setprio(0);
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
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) o[dt] = mfma16x16x32(vf[dt][h2], bp[h2], o[dt]);
    __builtin_amdgcn_s_setprio(0);
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
// time (loads first) with a running (max, sum). NT threads per workgroup: 64 for small
// merges (more workgroups), 256 for large ones (fewer to dispatch).
// With three or more key ranges each workgroup takes rows of a unit whose ranges ran on
// its own XCD (attn_combine_home): 4 x 128K call 14.4 -> 13.1 us, 1 x 32K 9.14 -> 9.02;
// with two ranges (ragged 28/4 workload) the plain order was 0.25 us faster.
__host__ __device__ inline bool attn_combine_home(const AttnGeom& a) { return a.nks >= 3; }

template <int D, int NT, int CH, bool EXACT>
__global__ __launch_bounds__(NT) void attn_combine_kernel(const float* __restrict__ o_part,
                                                                           const float2* __restrict__ ml_part,
                                                                           AttnGeom a, bf16* __restrict__ out) {
  constexpr int TPR = D / 8;  // threads per output row
  const int R = a.B * a.G;
  const int per_unit = R * TPR;
  int unit, iu;
  if (attn_combine_home(a)) {
    // workgroup x of the grid runs on XCD x % 8 and takes a unit whose key ranges the
    // attention kernel ran on that XCD (it gives each XCD a contiguous range of
    // items), so the partials are read where they were written
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int ipu = a.nks * a.nrs, per = (a.nitems + 7) >> 3;
    const int u0 = (int)(((int64_t)x * per + ipu - 1) / ipu);
    const int u1 = min(a.nunits, (int)(((int64_t)(x + 1) * per + ipu - 1) / ipu));
    const int wpu = (per_unit + NT - 1) / NT;
    unit = u0 + j / wpu;
    iu = (j % wpu) * NT + threadIdx.x;
    if (unit >= u1 || iu >= per_unit) return;
  } else {
    const int idx = blockIdx.x * NT + threadIdx.x;
    unit = a.rcp_pu ? (int)__umulhi((uint32_t)idx, a.rcp_pu) : idx / per_unit;
    if (unit >= a.nunits) return;
    iu = idx - unit * per_unit;
  }
  const int r = iu / TPR, e = (iu % TPR) * 8;
  const int s = a.rcp_hkv ? (int)__umulhi((uint32_t)unit, a.rcp_hkv) : unit, g = unit - s * a.Hkv;
  const int64_t base = (int64_t)unit * a.nks * a.rpad + r;
  float M = -INFINITY, L = 0.f;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  const int nks = EXACT ? CH : a.nks;  // EXACT: a single, fully known chunk
  for (int k0 = 0; k0 < nks; k0 += CH) {
    float2 p[CH];
    float4 va[CH], vc[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      p[j] = make_float2(-INFINITY, 0.f);
      va[j] = vc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (EXACT || k0 + j < a.nks) {  // EXACT: CH == nks, one chunk, every load unconditional
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

// fp32 path (attn_f32_kernel): one workgroup per (sequence, KV head, 16-row query
// tile). Its 8 waves take the 16-key tiles t = w, w + 8, ... of the key list (subset
// tiles, then the in-block keys), with each tile's fragments loaded straight into
// registers (the next tile's loads in flight while one is computed), S^T = K.Q^T and
// O^T += V^T.P^T on v_mfma_f32_16x16x4_f32 (fp32 products and sums) and an online
// base-2 softmax per query row; the eight partial results are merged through LDS.
// v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16] and
// holds D[4 (l / 16) + i][l % 16]. First product: A = K (key l % 16 of the tile), B =
// Q^T (query row l % 16), contraction slot j = l / 16 of step c taking dimension
// j D/4 + c, so each lane reads a contiguous quarter of its rows. The product leaves
// lane l with keys 4 (l / 16) + i of row l % 16, which are the contraction slots of
// step i of the second product: A = V^T (dimension l % 16 of a 16-dimension tile, keys
// 4 (l / 16) + i), B = P^T, the lane's own probabilities.
template <int D>
struct AttnF32Frag {
  float4 k[D / 16];  // K row (key l % 16 of the tile), dimensions (l / 16) D/4 .. + D/4
  float4 v[D / 16];  // per 16-dimension tile dt: V^T row dt * 16 + l % 16, keys 4 (l / 16) .. + 4
};

template <int D>
__device__ __forceinline__ void attn_f32_load_tile(int t, int nts, const float* __restrict__ kb,
                                                   const float* __restrict__ vb, const float* __restrict__ k_sel,
                                                   const float* __restrict__ v_sel, int64_t unit, int s, int g, int B,
                                                   int Hkv, int topk, int64_t ldv, int lr, int j,
                                                   AttnF32Frag<D>& f) {
  constexpr int KQ = D / 4;
  if (t < nts) {  // subset keys t*16 .. (the tail past topk masked by the caller, its values zeroed here)
    const int key = min(t * 16 + lr, topk - 1);
    const float* kr = k_sel + (unit * topk + key) * D + j * KQ;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) f.k[c] = *reinterpret_cast<const float4*>(kr + 4 * c);
    const int k0 = t * 16 + 4 * j;  // < ldv: ldv is topk rounded up to 64
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      float4 v = *reinterpret_cast<const float4*>(v_sel + (unit * D + dt * 16 + lr) * ldv + k0);
      if (k0 + 4 > topk) {
        v.x = k0 < topk ? v.x : 0.f;
        v.y = k0 + 1 < topk ? v.y : 0.f;
        v.z = k0 + 2 < topk ? v.z : 0.f;
        v.w = 0.f;
      }
      f.v[dt] = v;
    }
  } else {  // in-block keys b = (t - nts)*16 .., key-major rows of k_blk / v_blk
    const int b0 = (t - nts) * 16;
    const int bk = min(b0 + lr, B - 1);
    const float* kr = kb + (((int64_t)s * B + bk) * Hkv + g) * D + j * KQ;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) f.k[c] = *reinterpret_cast<const float4*>(kr + 4 * c);
    float e[4][D / 16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = b0 + 4 * j + i;
      const float* vr = vb + (((int64_t)s * B + min(b, B - 1)) * Hkv + g) * D + lr;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) e[i][dt] = b < B ? vr[dt * 16] : 0.f;
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) f.v[dt] = make_float4(e[0][dt], e[1][dt], e[2][dt], e[3][dt]);
  }
}

template <int D>
__global__ __launch_bounds__(512) void attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ kb,
                                                       const float* __restrict__ vb, const float* __restrict__ k_sel,
                                                       const float* __restrict__ v_sel, int B, int Hq, int Hkv,
                                                       int G, int topk, int64_t ldv, float scale2,
                                                       float* __restrict__ out) {
  constexpr int NW = 8, NC = D / 16, DT = D / 16, LDO = D + 4;
  extern __shared__ __align__(16) float xo[];  // [NW][16][LDO] partial outputs, then [NW][16] (max, sum)
  float2* xml = reinterpret_cast<float2*>(xo + NW * 16 * LDO);
  const int rt = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int R = B * G;
  const int64_t unit = (int64_t)s * Hkv + g;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 15, j = lane >> 4;
  const int nts = (topk + 15) / 16, nt = nts + (B + 15) / 16;

  float4 qf[NC];  // query row rt*16 + lr (rows past R re-read the last row), dimensions j D/4 ..
  {
    const int r = min(rt * 16 + lr, R - 1);
    const float* qr = q + (((int64_t)s * B + r / G) * Hq + g * G + r % G) * D + j * (D / 4);
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = *reinterpret_cast<const float4*>(qr + 4 * c);
  }
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  AttnF32Frag<D> cur, nxt;
  int t = w;
  if (t < nt) attn_f32_load_tile<D>(t, nts, kb, vb, k_sel, v_sel, unit, s, g, B, Hkv, topk, ldv, lr, j, cur);
  for (; t < nt; t += NW) {
    if (t + NW < nt)
      attn_f32_load_tile<D>(t + NW, nts, kb, vb, k_sel, v_sel, unit, s, g, B, Hkv, topk, ldv, lr, j, nxt);
    f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float ka[4] = {cur.k[c].x, cur.k[c].y, cur.k[c].z, cur.k[c].w};
      const float qa[4] = {qf[c].x, qf[c].y, qf[c].z, qf[c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[e], qa[e], sacc, 0, 0, 0);
    }
    // keys 4j + i of the tile: past topk (subset) or past B (in-block) do not exist
    const int nvalid = t < nts ? topk - t * 16 : B - (t - nts) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * j + i >= nvalid) sacc[i] = -INFINITY;
    const float mx = xmax4(fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]))) * scale2;
    const float mn = fmaxf(m, mx);  // finite: every tile holds a key
    const float alpha = fast_exp2(m - mn);
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    m = mn;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(sacc[i], scale2, -m));
    l += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const float va[4] = {cur.v[dt].x, cur.v[dt].y, cur.v[dt].z, cur.v[dt].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va[i], p[i], o[dt], 0, 0, 0);
    }
    if (t + NW < nt) cur = nxt;
  }
  l = xsum4(l);
  // merge the eight waves' (max, sum, output) per row
  {
    float* orow = xo + (w * 16 + lr) * LDO + 4 * j;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(orow + dt * 16) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (j == 0) xml[w * 16 + lr] = make_float2(m, l);
  }
  __syncthreads();
  for (int it = threadIdx.x; it < 16 * (D / 4); it += NW * 64) {
    const int row = it / (D / 4), e = (it % (D / 4)) * 4, r = rt * 16 + row;
    if (r >= R) continue;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, xml[ww * 16 + row].x);
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float2 ml = xml[ww * 16 + row];
      if (ml.x == -INFINITY) continue;  // a wave without tiles
      const float f = fast_exp2(ml.x - M);
      L += f * ml.y;
      const float4 ov = *reinterpret_cast<const float4*>(xo + (ww * 16 + row) * LDO + e);
      acc.x += f * ov.x;
      acc.y += f * ov.y;
      acc.z += f * ov.z;
      acc.w += f * ov.w;
    }
    const float inv = 1.f / L;
    *reinterpret_cast<float4*>(out + (((int64_t)s * B + r / G) * Hq + g * G + r % G) * D + e) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
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
  const int nt = n >= (int64_t)256 * 256 ? 256 : kAttnCombineThreads;
  int64_t nwg = (n + nt - 1) / nt;
  if (attn_combine_home(a)) {  // units per XCD as the attention kernel placed them
    const int ipu = a.nks * a.nrs, per = (a.nitems + 7) / 8;
    const int64_t wpu = ((int64_t)a.B * a.G * (s.D / 8) + nt - 1) / nt;
    int64_t qmax = 0;
    for (int x = 0; x < 8; ++x) {
      const int64_t u0 = ((int64_t)x * per + ipu - 1) / ipu;
      const int64_t u1 = std::min<int64_t>(a.nunits, ((int64_t)(x + 1) * per + ipu - 1) / ipu);
      qmax = std::max<int64_t>(qmax, (u1 - u0) * wpu);
    }
    nwg = 8 * qmax;
  }
  if (nwg == 0) return hipSuccess;
  const dim3 grid((unsigned)nwg);
  // key-range counts with a kernel of their own take every load unconditionally
#define HERALD_COMBINE(NTT, CHH, EX)                                                                      \
  klaunch(s.D == 128 ? attn_combine_kernel<128, NTT, CHH, EX> : attn_combine_kernel<64, NTT, CHH, EX>, grid, NTT, 0, st, \
          o_part, ml_part, a, (bf16*)out)
#define HERALD_COMBINE_NKS(NTT)              \
  switch (a.nks) {                           \
    case 2: HERALD_COMBINE(NTT, 2, true); break; \
    case 3: HERALD_COMBINE(NTT, 3, true); break; \
    case 4: HERALD_COMBINE(NTT, 4, true); break; \
    case 6: HERALD_COMBINE(NTT, 6, true); break; \
    default: HERALD_COMBINE(NTT, 8, false);      \
  }
  if (nt == 256) {
    HERALD_COMBINE_NKS(256)
  } else {
    HERALD_COMBINE_NKS(kAttnCombineThreads)
  }
#undef HERALD_COMBINE_NKS
#undef HERALD_COMBINE
  return hipGetLastError();
}

hipError_t launch_attn(const Shape& s, const void* q, const void* kb, const void* vb, const void* k_sel,
                       const void* v_sel, void* out, void* ws, hipStream_t st) {
  const float scale2 = s.scale * kLog2e;
  if (!s.bf16) {
    const int64_t ldv = vsel_ld(s.topk);
    const dim3 grid((s.B * s.G + 15) / 16, s.Hkv, s.nseq);
    const size_t smem = ((size_t)8 * 16 * (s.D + 4) + 2 * 8 * 16) * sizeof(float);
    const void* kern = s.D == 128 ? (const void*)attn_f32_kernel<128> : (const void*)attn_f32_kernel<64>;
    hipError_t e = allow_smem(kern, smem);
    if (e != hipSuccess) return e;
    if (s.D == 128)
      klaunch(attn_f32_kernel<128>, grid, 512, smem, st, (const float*)q, (const float*)kb, (const float*)vb,
              (const float*)k_sel, (const float*)v_sel, s.B, s.Hq, s.Hkv, s.G, s.topk, ldv, scale2, (float*)out);
    else
      klaunch(attn_f32_kernel<64>, grid, 512, smem, st, (const float*)q, (const float*)kb, (const float*)vb,
              (const float*)k_sel, (const float*)v_sel, s.B, s.Hq, s.Hkv, s.G, s.topk, ldv, scale2, (float*)out);
    return hipGetLastError();
  }
  const AttnGeom a = attn_geom(s);
  if (s.D == 128) return launch_attn_bf16<128>(a, q, kb, vb, k_sel, v_sel, out, ws, scale2, st);
  return launch_attn_bf16<64>(a, q, kb, vb, k_sel, v_sel, out, ws, scale2, st);
}

}  // namespace herald
