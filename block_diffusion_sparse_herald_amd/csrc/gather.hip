// Fetch the selected subset into the sparse KV pool, once per block (HERALD
// abstract on the mlsift "KV cache offloading" listing: only a small critical
// subset is fetched; HERALD v3 abstract: the final top-K subset).
//
// Pool layout: K rows as they are in the cache ([nseq][Hkv][topk][d]); V stored
// d-major ([nseq][Hkv][d][ldv], ldv = topk rounded up to 64, padding zero) so the
// attention kernel can load V^T tiles, the left operand of its P.V product, with
// plain 16-byte loads. A bit-exact byte copy; HBM-bound.
#include "common.hpp"
#include "kernels.hpp"

namespace herald {

// One workgroup per 64 picks of one (sequence, KV head). PACKED selects where row i
// of the group comes from: the cache by index (device path) or packed
// [nseq][Hkv][topk][D] buffers (host-pool path, after their copy to the device).
// On the indexed path an index outside [0, L_s) is never dereferenced: its K and V
// rows are written as zeros and, when `status` is not NULL, *status is set to 1.
template <typename T, int D, bool PACKED>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                     const int32_t* __restrict__ idx,
                                                     const int64_t* __restrict__ seq_start, int Hkv, int topk,
                                                     int64_t ldv, T* __restrict__ k_sel, T* __restrict__ v_sel,
                                                     int32_t* __restrict__ status) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int CPR = D / EPL;  // 16-byte chunks per row
  constexpr int LDT = D + EPL;  // padded LDS row (elements)
  __shared__ __align__(16) T tile[64 * LDT];
  const int blk = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int i0 = blk * 64;
  const int64_t unit = (int64_t)s * Hkv + g;
  const int64_t j0 = PACKED ? 0 : seq_start[s];
  const int64_t L = PACKED ? 0 : seq_start[s + 1] - j0;

  // K rows (copied straight through) and V rows (staged in LDS): all loads first, the
  // indices of every chunk, then every row chunk. No load sits behind a branch (an
  // index outside the sequence reads its row 0, L >= 1, and the value is dropped), so
  // all of them are in flight together.
  constexpr int NPT = 64 * CPR / 256;  // 16-byte chunks per thread, each of K and V
  uint4 kv[NPT], vv[NPT];
  int32_t jj[NPT];
#pragma unroll
  for (int u = 0; u < NPT; ++u) {
    const int i = min(i0 + (int)(threadIdx.x + u * 256) / CPR, topk - 1);
    jj[u] = PACKED ? i : idx[unit * topk + i];
  }
  bool bad = false;
#pragma unroll
  for (int u = 0; u < NPT; ++u) {
    const int ch = (int)(threadIdx.x + u * 256) % CPR;
    const bool ok = PACKED || (jj[u] >= 0 && jj[u] < L);
    const int64_t row = PACKED ? unit * topk + jj[u] : (j0 + (ok ? jj[u] : 0)) * Hkv + g;
    bad |= !ok;
    kv[u] = ld16_or_zero(k + row * D + ch * EPL, ok);
    vv[u] = ld16_or_zero(v + row * D + ch * EPL, ok);
  }
  if (!PACKED && bad && status) *status = 1;
#pragma unroll
  for (int u = 0; u < NPT; ++u) {
    const int c = threadIdx.x + u * 256;
    const int r = c / CPR, ch = c % CPR;
    const int i = i0 + r;
    if (i < topk) st16(k_sel + (unit * topk + i) * D + ch * EPL, kv[u]);
    *reinterpret_cast<uint4*>(&tile[r * LDT + ch * EPL]) = i < topk ? vv[u] : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  // each 16-byte output chunk holds EPL consecutive picks of one dimension
  constexpr int KCH = 64 / EPL;  // chunks per dimension row within this block
  T* vout = v_sel + unit * D * ldv;
  for (int c = threadIdx.x; c < D * KCH; c += 256) {
    const int e = c / KCH, kc = c % KCH;
    union {
      T t[EPL];
      uint4 u;
    } pk;
#pragma unroll
    for (int t = 0; t < EPL; ++t) pk.t[t] = tile[(kc * EPL + t) * LDT + e];
    st16(vout + (int64_t)e * ldv + i0 + kc * EPL, pk.u);
  }
}

template <bool PACKED>
static hipError_t gather_dispatch(const Shape& s, const void* k, const void* v, const int32_t* idx, void* k_sel,
                                  void* v_sel, int32_t* status, hipStream_t st) {
  dim3 grid((s.topk + 63) / 64, s.Hkv, s.nseq);
  const int64_t ldv = vsel_ld(s.topk);
  if (s.bf16) {
    if (s.D == 128)
      klaunch(gather_kernel<bf16, 128, PACKED>, grid, 256, 0, st, (const bf16*)k, (const bf16*)v, idx, s.seq_start, s.Hkv,
                                                             s.topk, ldv, (bf16*)k_sel, (bf16*)v_sel, status);
    else
      klaunch(gather_kernel<bf16, 64, PACKED>, grid, 256, 0, st, (const bf16*)k, (const bf16*)v, idx, s.seq_start, s.Hkv,
                                                            s.topk, ldv, (bf16*)k_sel, (bf16*)v_sel, status);
  } else {
    if (s.D == 128)
      klaunch(gather_kernel<float, 128, PACKED>, grid, 256, 0, st, (const float*)k, (const float*)v, idx, s.seq_start,
                                                              s.Hkv, s.topk, ldv, (float*)k_sel, (float*)v_sel, status);
    else
      klaunch(gather_kernel<float, 64, PACKED>, grid, 256, 0, st, (const float*)k, (const float*)v, idx, s.seq_start,
                                                             s.Hkv, s.topk, ldv, (float*)k_sel, (float*)v_sel, status);
  }
  return hipGetLastError();
}

hipError_t launch_gather(const Shape& s, const void* k, const void* v, const int32_t* idx, void* k_sel, void* v_sel,
                         int32_t* status, hipStream_t st) {
  return gather_dispatch<false>(s, k, v, idx, k_sel, v_sel, status, st);
}

// Host-pool path: `packed_k` / `packed_v` hold the picked rows as [nseq][Hkv][topk][D].
hipError_t launch_layout_packed(const Shape& s, const void* packed_k, const void* packed_v, void* k_sel, void* v_sel,
                                hipStream_t st) {
  return gather_dispatch<true>(s, packed_k, packed_v, nullptr, k_sel, v_sel, nullptr, st);
}

}  // namespace herald
