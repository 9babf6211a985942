// Device helpers shared by the HERALD kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

namespace herald {

typedef uint16_t bf16;  // storage type of bf16 tensors (bit pattern)
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
// low / high bf16 of a packed pair, widened
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16, h);
}

// Two floats to a packed bf16 pair (lo in bits 0..15), round to nearest even: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 h = __builtin_convertvector((f2){lo, hi}, b2);
  return __builtin_bit_cast(uint32_t, h);
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<bf16>(bf16 v) { return bf16_to_f32(v); }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) { return f32_to_bf16(v); }

// 16-byte vector: elements per vector and unpacking to fp32.
template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static __forceinline__ void unpack(const uint4& v, float* o) {
    o[0] = __uint_as_float(v.x);
    o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z);
    o[3] = __uint_as_float(v.w);
  }
};
template <>
struct Vec16<bf16> {
  static constexpr int N = 8;
  __device__ static __forceinline__ void unpack(const uint4& v, float* o) {
    o[0] = __uint_as_float(v.x << 16);
    o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16);
    o[3] = __uint_as_float(v.y & 0xffff0000u);
    o[4] = __uint_as_float(v.z << 16);
    o[5] = __uint_as_float(v.z & 0xffff0000u);
    o[6] = __uint_as_float(v.w << 16);
    o[7] = __uint_as_float(v.w & 0xffff0000u);
  }
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// A 16-byte load whose value is replaced by zeros when `ok` is false. The load is always
// issued (p must be a valid address either way: callers clamp it) and the zeros are
// selected afterwards. Written as `ok ? ld16(p) : 0`, the load sits in a branch, and the
// register copy the compiler makes at the join needs the loaded value there: it waits for
// every load in flight at that point, which serialised the rest of a kernel's loads
// behind a full memory round trip.
__device__ __forceinline__ uint4 ld16_or_zero(const void* p, bool ok) {
  const uint4 v = ld16(p);
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }
// 16-byte store marked non-temporal (global_store_dwordx4 ... nt).
__device__ __forceinline__ void st16_stream(void* p, const float4& v) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store((v4f){v.x, v.y, v.z, v.w}, reinterpret_cast<v4f*>(p));
}

// acc + lo + hi of a packed bf16 pair, in fp32 (one v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float add_bf16x2(uint32_t pair, float acc) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair), __builtin_bit_cast(bf16x2_t, 0x3f803f80u),
                                         acc, false);
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- direct-to-LDS loads

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 * lane
// (global_load_lds_dwordx4; lds_base must be the same in every lane of the wave).
// Written as inline assembly so that the compiler does not wait for the transfer
// before every later LDS read: the kernel waits on vmcnt itself (wait_vm).
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base)
               : "memory", "m0");
}

// The same with the non-temporal hint (nt): for data read once in a long stream, so that
// it does not displace from the caches what the next kernels read (the full-cache scan:
// the candidate rows and logits that the score, refine and gather kernels read next).
__device__ __forceinline__ void lds_dma16_nt(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds_base)
               : "memory", "m0");
}

// s_waitcnt with vmcnt <= n (n < 64), the other counters not waited on.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// ---------------------------------------------------------------- (max, sum) pairs

// Merge two (max, sum-of-2^(x-max)) pairs. Commutative bit for bit, so butterfly
// reductions leave the same value in every lane. Empty pairs are (-inf, 0).
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  s = s * fast_exp2(m - M) + s2 * fast_exp2(m2 - M);
  m = M;
}

__device__ __forceinline__ void ms_wave_merge(float& m, float& s) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const float m2 = __shfl_xor(m, o);
    const float s2 = __shfl_xor(s, o);
    ms_merge(m, s, m2, s2);
  }
}

// max / sum of x over lanes l, l^16, l^32, l^48 (the four lane groups of one MFMA
// column), with the gfx950 row-swap permutes (no LDS traffic)
__device__ __forceinline__ float xmax4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xsum4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// sum of x over the 16 lanes of each row (lanes 16r .. 16r+15), complete in the last
// lane of the row (DPP row shifts, no LDS traffic)
__device__ __forceinline__ float row_sum16_last(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));  // row_shr:1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));  // row_shr:2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));  // row_shr:4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));  // row_shr:8
  return x;
}

// max / sum over the 16 lanes of each row, left in every lane of the row: rotations by
// 8, 4, 2, 1 within the row (DPP row_ror, no LDS traffic)
__device__ __forceinline__ float row_max16_all(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false)));
  return x;
}
__device__ __forceinline__ float row_sum16_all(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));
  return x;
}

// ---------------------------------------------------------------- block-wide scans

// Inclusive prefix sum over the 64 lanes of a wave with DPP (no LDS traffic): row
// shifts by 1, 2, 4, 8 within each row of 16 lanes (lanes shifted in from outside
// the row read 0), then the last lane of row 0 (and of row 2) is broadcast into the
// next row, and the last lane of row 1 into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Exclusive prefix sum of `v` over the NT threads of the block (NT multiple of 64).
// `lds` holds NT/64 + 1 ints. Every thread receives the block total in *total.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds, uint32_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const uint32_t x = wave_incl_scan(v);
  if (lane == kWave - 1) lds[wid] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t acc = 0;
    for (int w = 0; w < NT / kWave; ++w) {
      const uint32_t t = lds[w];
      lds[w] = acc;
      acc += t;
    }
    lds[NT / kWave] = acc;
  }
  __syncthreads();
  const uint32_t r = lds[wid] + x - v;
  *total = lds[NT / kWave];
  __syncthreads();
  return r;
}

// Radix-select step. hist[0..nbins) counts the keys of each digit value. Finds the
// largest digit b whose suffix count sum_{b' >= b} hist[b'] reaches k, and the
// count strictly above it. Result broadcast to every thread. Requires nbins % NT == 0.
template <int NT>
__device__ __forceinline__ void find_digit(const uint32_t* hist, int nbins, uint32_t k, uint32_t* lds,
                                           int* digit, uint32_t* above) {
  const int per = nbins / NT;
  // thread t owns the per bins [nbins-(t+1)*per, nbins-t*per): thread 0 the top ones
  const int hi = nbins - threadIdx.x * per;  // exclusive
  uint32_t sum = 0;
  for (int b = hi - 1; b >= hi - per; --b) sum += hist[b];
  uint32_t total;
  const uint32_t before = block_exclusive_scan<NT>(sum, lds, &total);
  if (threadIdx.x == 0) {
    lds[NT / kWave + 1] = 0;
    lds[NT / kWave + 2] = 0;
  }
  __syncthreads();
  if (before < k && before + sum >= k) {
    uint32_t acc = before;
    for (int b = hi - 1; b >= hi - per; --b) {
      const uint32_t c = hist[b];
      if (acc + c >= k) {
        lds[NT / kWave + 1] = (uint32_t)b;
        lds[NT / kWave + 2] = acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
  *digit = (int)lds[NT / kWave + 1];
  *above = lds[NT / kWave + 2];
  __syncthreads();
}

// Radix-select step run by one wave on a histogram (LDS or global memory): finds the
// largest digit b whose suffix count reaches k and the count strictly above it, with
// no branches. Lane l owns the PER = nbins/64 consecutive bins starting at
// (63 - l) * PER (lane 0 the top ones) and sums them (16-byte reads, rotated by lane so
// that the lanes of one read spread over the LDS banks); a wave scan of the sums names
// the lane whose bins reach k; its PER bins, one per lane from the top, are scanned
// again to name the bin. The result is returned in every lane.
template <int PER>
__device__ __forceinline__ void wave_find_digit_t(const uint32_t* hist, uint32_t k, int* digit, uint32_t* above) {
  constexpr int NQ = PER / 4;
  const int lane = threadIdx.x & (kWave - 1);
  const int lo = (kWave - 1 - lane) * PER;
  uint32_t sum = 0;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const uint4 t = *reinterpret_cast<const uint4*>(hist + lo + 4 * ((q + lane) & (NQ - 1)));
    sum += t.x + t.y + t.z + t.w;
  }
  const uint32_t incl = wave_incl_scan(sum);
  const uint32_t before = incl - sum;
  const uint64_t who = __ballot(before < k && incl >= k);
  const int src = who ? (int)__builtin_ctzll(who) : kWave - 1;
  const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)before, src);
  const int los = (kWave - 1 - src) * PER;
  const uint32_t c = lane < PER ? hist[los + PER - 1 - lane] : 0u;
  const uint32_t ci = wave_incl_scan(c);
  const uint64_t hit = __ballot(lane < PER && base + ci >= k);
  const int f = hit ? (int)__builtin_ctzll(hit) : PER - 1;
  *digit = los + PER - 1 - f;
  *above = base + (uint32_t)__builtin_amdgcn_readlane((int)(ci - c), f);
}

__device__ __forceinline__ void wave_find_digit(const uint32_t* hist, int nbins, uint32_t k, int* digit,
                                                uint32_t* above) {
  if (nbins == 2048) wave_find_digit_t<32>(hist, k, digit, above);
  else wave_find_digit_t<16>(hist, k, digit, above);
}

// The three radix digits (11, 11, 10 bits) of the k-th largest key from its three
// histograms hist[0..2048), hist[2048..4096), hist[4096..5120) in LDS. Wave 0 only.
// Returns the threshold bit pattern and how many keys equal to it are wanted.
__device__ __forceinline__ void wave_threshold(const uint32_t* hist, uint32_t k, uint32_t* thr, uint32_t* ties) {
  int d1, d2, d3;
  uint32_t a1, a2, a3;
  wave_find_digit(hist, 2048, k, &d1, &a1);
  const uint32_t k1 = k - a1;
  wave_find_digit(hist + 2048, 2048, k1, &d2, &a2);
  const uint32_t k2 = k1 - a2;
  wave_find_digit(hist + 4096, 1024, k2, &d3, &a3);
  *thr = ((uint32_t)d1 << 21) | ((uint32_t)d2 << 10) | (uint32_t)d3;
  *ties = k2 - a3;
}

// ---------------------------------------------------------------- radix threshold in LDS

// The k-th largest of the n keys u[0..n) (in LDS, or in global memory for sets too
// large for it; fp32 bit patterns of non-negative
// scores, so unsigned order is value order), digit by digit (11, 11, 10 bits) with
// histograms h[0..kRadixBins) in LDS. With have_first, h already holds the histogram
// of the first digit. Returns the key's bit pattern and, in *ties, how many keys
// equal to it belong to the top k. Every thread of the NT-thread workgroup calls it.
template <int NT>
__device__ __forceinline__ uint32_t lds_radix_threshold(const uint32_t* u, int n, uint32_t k, uint32_t* h,
                                                        uint32_t* dig, bool have_first, uint32_t* ties) {
  constexpr int kBins = 2048;
  const int tid = threadIdx.x;
  uint32_t want = k, prefix = 0;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    if (pass > 0 || !have_first) {
      const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
      const uint32_t mask = pass == 2 ? 1023u : 2047u;
      for (int i = tid; i < kBins; i += NT) h[i] = 0u;
      __syncthreads();
      // eight keys read before their atomics (the compiler cannot move reads of u
      // past atomics on h, which may alias)
      for (int i0 = tid; i0 < n; i0 += 8 * NT) {
        uint32_t x[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) x[q] = i0 + q * NT < n ? u[i0 + q * NT] : 0u;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (i0 + q * NT < n && (pass == 0 || (x[q] >> (shift + (pass == 2 ? 10 : 11))) == prefix))
            atomicAdd(&h[(x[q] >> shift) & mask], 1u);
      }
      __syncthreads();
    }
    if (tid < 64) {
      int d;
      uint32_t above;
      wave_find_digit(h, pass == 2 ? 1024 : kBins, want, &d, &above);
      if (tid == 0) {
        dig[0] = (uint32_t)d;
        dig[1] = above;
      }
    }
    __syncthreads();
    want -= dig[1];
    prefix = (prefix << (pass == 2 ? 10 : 11)) | dig[0];
    __syncthreads();
  }
  *ties = want;
  return prefix;
}

// ---------------------------------------------------------------- selection emission

// Writes, in ascending position order, every position i < n whose key u[i] (LDS or
// global memory) is
// above thr, plus the first ties_wanted positions whose key equals thr: out[p] gets
// the position (or idx[position] when idx is not NULL), outs[p] (if not NULL) the
// key as a float. Wave w of NW scans positions [w*span, (w+1)*span) with ballots,
// 64 positions per ballot and eight ballots per batch of LDS reads; one exchange of
// the per-wave counts (wcnt, NW pairs in LDS) fixes tie ranks and output offsets.
template <int NW>
__device__ __forceinline__ void lds_emit(const uint32_t* u, int n, uint32_t thr, uint32_t ties_wanted,
                                         const int32_t* __restrict__ idx, int32_t* __restrict__ out,
                                         float* __restrict__ outs, uint32_t (*wcnt)[2]) {
  constexpr int U = 8;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int span = ((n + NW - 1) / NW + 64 * U - 1) / (64 * U) * (64 * U);
  const int e0 = w * span;
  uint32_t ngt = 0, neq = 0;
  for (int it = 0; it < span; it += 64 * U) {
    uint32_t v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int e = e0 + it + k * 64 + lane;
      v[k] = e < n ? u[e] : 0u;
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int e = e0 + it + k * 64 + lane;
      ngt += (uint32_t)__builtin_popcountll(__ballot(e < n && v[k] > thr));
      neq += (uint32_t)__builtin_popcountll(__ballot(e < n && v[k] == thr));
    }
  }
  if (lane == 0) {
    wcnt[w][0] = ngt;
    wcnt[w][1] = neq;
  }
  __syncthreads();
  uint32_t tie = 0, pos = 0;
  for (int x = 0; x < w; ++x) {
    const uint32_t take = min(wcnt[x][1], ties_wanted - min(ties_wanted, tie));
    pos += wcnt[x][0] + take;
    tie += wcnt[x][1];
  }
  // set bits of m in the lanes below this one (v_mbcnt)
  auto below = [](uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  };
  for (int it = 0; it < span; it += 64 * U) {
    uint32_t v[U];
    int32_t ix[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int e = e0 + it + k * 64 + lane;
      v[k] = e < n ? u[e] : 0u;
      ix[k] = idx ? (e < n ? idx[e] : 0) : e;  // all reads of the batch issued together
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int e = e0 + it + k * 64 + lane;
      const bool gt = e < n && v[k] > thr, eq = e < n && v[k] == thr;
      const uint64_t beq = __ballot(eq);
      const uint32_t my_tie = tie + below(beq);
      const bool take = gt || (eq && my_tie < ties_wanted);
      const uint64_t btake = __ballot(take);
      if (take) {
        const uint32_t p = pos + below(btake);
        out[p] = ix[k];
        if (outs) outs[p] = __uint_as_float(v[k]);
      }
      pos += (uint32_t)__builtin_popcountll(btake);
      tie += (uint32_t)__builtin_popcountll(beq);
    }
  }
}

// ---------------------------------------------------------------- top-k in registers

// Exact top-k of n keys (fp32 bit patterns of non-negative scores, so unsigned order
// is value order; ties to the lower position) held in the registers of a 1024-thread
// workgroup: wave w holds positions [w * nit * 256, (w + 1) * nit * 256), in nit chunks
// of 256; lane l holds positions chunk * 256 + 4l + (0..3) of each chunk, so the order
// (wave, chunk, lane, element) is position order. No pass goes through LDS: the radix
// histograms take LDS atomics and the emission is ordered by wave scans.
constexpr int kTopkWaves = 16;

// 256-position chunks per wave for n keys.
__host__ __device__ constexpr int topk_chunks(int n) { return ((n + kTopkWaves - 1) / kTopkWaves + 255) / 256; }

// Loads this lane's keys src[0..n) (positions past n read as 0): 16-byte loads when src
// is 16-byte aligned and n a multiple of 4, else 4-byte loads. ALIGN = 1 or 2 fixes the
// choice at compile time (the caller knows it): with one path only, the compiler does not
// wait for the loads of an earlier call before issuing these.
template <int MAXIT, typename T, int ALIGN = 0>
__device__ __forceinline__ void topk_load(const T* __restrict__ src, int n, int nit, uint32_t (&v)[MAXIT][4]) {
  static_assert(sizeof(T) == 4, "32-bit keys");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t* s32 = reinterpret_cast<const uint32_t*>(src);
  if (ALIGN == 1 || (ALIGN == 0 && ((uintptr_t)src & 15) == 0 && (n & 3) == 0)) {
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
      const int e = (w * nit + it) * 256 + 4 * lane;
      uint4 t = make_uint4(0u, 0u, 0u, 0u);
      if (it < nit && e < n) t = *reinterpret_cast<const uint4*>(s32 + e);
      v[it][0] = t.x;
      v[it][1] = t.y;
      v[it][2] = t.z;
      v[it][3] = t.w;
    }
  } else {
#pragma unroll
    for (int it = 0; it < MAXIT; ++it)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = (w * nit + it) * 256 + 4 * lane + c;
        v[it][c] = it < nit && e < n ? s32[e] : 0u;
      }
  }
}

// Histogram of the digit (x >> shift) & mask over this lane's keys x inside n whose
// bits above hishift equal prefix (every key when hishift >= 32). Runs of equal digits
// among a lane's four consecutive keys take one atomic, which thins the same-address
// atomics of clustered scores.
template <int MAXIT>
__device__ __forceinline__ void topk_hist(const uint32_t (&v)[MAXIT][4], int n, int nit, int hishift,
                                          uint32_t prefix, int shift, uint32_t mask, uint32_t* h) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) {
    if (it >= nit) continue;
    const int e = (w * nit + it) * 256 + 4 * lane;
    uint32_t cur = 0xffffffffu, cnt = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t x = v[it][c];
      const bool in = e + c < n && (hishift >= 32 || (x >> hishift) == prefix);
      const uint32_t d = (x >> shift) & mask;
      if (in) {
        if (d == cur) {
          ++cnt;
        } else {
          if (cnt) atomicAdd(&h[cur], cnt);
          cur = d;
          cnt = 1;
        }
      }
    }
    if (cnt) atomicAdd(&h[cur], cnt);
  }
}

// Histogram of the digit (x >> shift) & mask over this lane's keys x inside n whose
// bits above hishift equal prefix: one atomic per matching key (the later digits,
// where few keys match and they spread over the bins).
template <int MAXIT, bool FULL>
__device__ __forceinline__ void topk_hist_sparse_t(const uint32_t (&v)[MAXIT][4], int n, int nit, int hishift,
                                                   uint32_t prefix, int shift, uint32_t mask, uint32_t* h) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) {
    if (it >= nit) continue;
    const int e = (w * nit + it) * 256 + 4 * lane;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t x = v[it][c];
      if ((FULL || e + c < n) && (x >> hishift) == prefix) atomicAdd(&h[(x >> shift) & mask], 1u);
    }
  }
}

// True when every position this wave holds is below n (no validity tests needed).
__device__ __forceinline__ bool topk_wave_full(int n, int nit) {
  return ((threadIdx.x >> 6) + 1) * nit * 256 <= n;
}

template <int MAXIT>
__device__ __forceinline__ void topk_hist_sparse(const uint32_t (&v)[MAXIT][4], int n, int nit, int hishift,
                                                 uint32_t prefix, int shift, uint32_t mask, uint32_t* h) {
  if (topk_wave_full(n, nit)) topk_hist_sparse_t<MAXIT, true>(v, n, nit, hishift, prefix, shift, mask, h);
  else topk_hist_sparse_t<MAXIT, false>(v, n, nit, hishift, prefix, shift, mask, h);
}

// Collects, in ascending position order, every key above thr plus the first ties_wanted
// keys equal to it (all_ties: every key equal to thr is wanted, so the test is x >= thr)
// into pick_idx[p] = index(chunk, element, position) and pick_val[p] (if not NULL) in
// LDS, then writes the k picks to out / outs (outs may be NULL) with coalesced stores.
// wcnt holds kTopkWaves pairs in LDS. Every thread of the workgroup calls it.
// Per-lane counts of the keys at or above lo (ngt) and equal to thr (neq, unless all_ties).
template <int MAXIT, bool FULL>
__device__ __forceinline__ uint2 topk_count_t(const uint32_t (&v)[MAXIT][4], int n, int nit, uint32_t lo, uint32_t thr,
                                              bool all_ties) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) {
    if (it >= nit) continue;
    const int e = (w * nit + it) * 256 + 4 * lane;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ngt += ((FULL || e + c < n) && v[it][c] >= lo) ? 1u : 0u;
      if (!all_ties) neq += ((FULL || e + c < n) && v[it][c] == thr) ? 1u : 0u;
    }
  }
  return make_uint2(ngt, neq);
}

// Collects this wave's picks: pos and tie are the wave's running output position and
// tie rank (uniform); teq says whether the wave holds keys equal to thr. Branch-free: a
// key that is not taken is written to this lane's discard slot k + lane (the pick arrays
// hold k + kTopkSlack entries), so no store needs an exec-mask branch.
constexpr int kTopkSlack = 64;
template <int MAXIT, bool FULL, bool VAL, typename IndexF>
__device__ __forceinline__ void topk_collect_t(const uint32_t (&v)[MAXIT][4], IndexF index, int n, int nit,
                                               uint32_t lo, uint32_t thr, uint32_t ties_wanted, uint32_t teq,
                                               uint32_t k, uint32_t pos, uint32_t tie, int32_t* pick_idx,
                                               float* pick_val) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t discard = k + (uint32_t)lane;
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) {
    if (it >= nit) continue;
    const int e = (w * nit + it) * 256 + 4 * lane;
    uint32_t take[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) take[c] = ((FULL || e + c < n) && v[it][c] >= lo) ? 1u : 0u;
    if (teq) {  // this wave holds keys equal to the threshold: rank them by position
      uint32_t eq[4], ne = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        eq[c] = ((FULL || e + c < n) && v[it][c] == thr) ? 1u : 0u;
        ne += eq[c];
      }
      const uint32_t incl = wave_incl_scan(ne);
      uint32_t r = tie + incl - ne;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (eq[c]) take[c] = r < ties_wanted ? 1u : 0u;
        r += eq[c];
      }
      tie += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    }
    const uint32_t nt = (take[0] + take[1]) + (take[2] + take[3]);
    const uint32_t incl = wave_incl_scan(nt);
    uint32_t p = pos + incl - nt;
    pos += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t dst = take[c] && p < k ? p : discard;
      pick_idx[dst] = index(it, c, e + c);
      if (VAL) pick_val[dst] = __uint_as_float(v[it][c]);
      p += take[c];
    }
  }
}

// Collects, in ascending position order, every key above thr plus the first ties_wanted
// keys equal to it (all_ties: every key equal to thr is wanted, so the test is x >= thr)
// into pick_idx[p] = index(chunk, element, position) and pick_val[p] (if not NULL) in
// LDS (each of k + kTopkSlack entries), then writes the k picks to out / outs (outs may
// be NULL) with coalesced stores.
// wcnt holds kTopkWaves pairs in LDS. Every thread of the workgroup calls it. Waves whose
// positions all lie below n skip the per-key validity tests.
template <int MAXIT, typename IndexF>
__device__ __forceinline__ void topk_emit(const uint32_t (&v)[MAXIT][4], IndexF index, int n, int nit,
                                          uint32_t thr, uint32_t ties_wanted, bool all_ties, uint32_t k,
                                          int32_t* pick_idx, float* pick_val, int32_t* __restrict__ out,
                                          float* __restrict__ outs, uint32_t (*wcnt)[2]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const bool full = topk_wave_full(n, nit);
  // with all_ties the keys equal to thr count as above it
  const uint32_t lo = all_ties ? thr : thr + 1u;
  const uint2 cnt = full ? topk_count_t<MAXIT, true>(v, n, nit, lo, thr, all_ties)
                         : topk_count_t<MAXIT, false>(v, n, nit, lo, thr, all_ties);
  const uint32_t tgt = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(cnt.x), 63);
  const uint32_t teq = all_ties ? 0u : (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(cnt.y), 63);
  if (lane == 0) {
    wcnt[w][0] = tgt;
    wcnt[w][1] = teq;
  }
  __syncthreads();
  uint32_t tie = 0, pos = 0;
  for (int x = 0; x < w; ++x) {
    const uint32_t take = min(wcnt[x][1], ties_wanted - min(ties_wanted, tie));
    pos += wcnt[x][0] + take;
    tie += wcnt[x][1];
  }
  if (pick_val) {
    if (full)
      topk_collect_t<MAXIT, true, true>(v, index, n, nit, lo, thr, ties_wanted, teq, k, pos, tie, pick_idx, pick_val);
    else
      topk_collect_t<MAXIT, false, true>(v, index, n, nit, lo, thr, ties_wanted, teq, k, pos, tie, pick_idx, pick_val);
  } else {
    if (full)
      topk_collect_t<MAXIT, true, false>(v, index, n, nit, lo, thr, ties_wanted, teq, k, pos, tie, pick_idx, pick_val);
    else
      topk_collect_t<MAXIT, false, false>(v, index, n, nit, lo, thr, ties_wanted, teq, k, pos, tie, pick_idx, pick_val);
  }
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < k; i += kTopkWaves * 64) {
    out[i] = pick_idx[i];
    if (outs) outs[i] = pick_val[i];
  }
}

// ---------------------------------------------------------------- MFMA

// D[16x16] += A[16x32] * B[32x16], bf16 inputs, fp32 accumulate (v_mfma_f32_16x16x32_bf16).
// Lane l supplies A[l%16][8*(l/16) .. +8) and B[8*(l/16) .. +8)[l%16], and holds
// D[4*(l/16) + i][l%16] for i = 0..3.
__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  c, 0, 0, 0);
}

// Lets `kernel` take up to the full 160 KiB of LDS of a gfx950 CU when a launch needs
// more than the default 64 KiB. Host side; the attribute is set once per kernel, so
// the call is cheap and safe to repeat (also while a stream is being captured).
// Lets `kernel` take `dynamic` bytes of dynamic LDS next to its static LDS (raises the
// per-kernel limit once, to what the 160 KiB of a compute unit leave).
inline hipError_t allow_smem(const void* kernel, size_t dynamic) {
  constexpr size_t kMaxLds = 160 * 1024;
  struct Entry {
    const void* kernel;
    size_t static_bytes;
    bool raised;
  };
  static std::mutex mu;
  static Entry seen[64];
  static int nseen = 0;
  std::lock_guard<std::mutex> lock(mu);
  Entry* e = nullptr;
  for (int i = 0; i < nseen; ++i)
    if (seen[i].kernel == kernel) e = &seen[i];
  if (!e) {
    hipFuncAttributes attr;
    const hipError_t st = hipFuncGetAttributes(&attr, kernel);
    if (st != hipSuccess) return st;
    if (nseen == 64) return hipErrorUnknown;
    seen[nseen] = Entry{kernel, attr.sharedSizeBytes, false};
    e = &seen[nseen++];
  }
  const size_t room = kMaxLds - std::min(kMaxLds, e->static_bytes);
  if (dynamic > room) return hipErrorInvalidValue;
  if (dynamic + e->static_bytes > 65536 && !e->raised) {
    const hipError_t st = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)room);
    if (st != hipSuccess) return st;
    e->raised = true;
  }
  return hipSuccess;
}

}  // namespace herald
