// mita_device.hpp — device-side building blocks shared by the MiTA kernels
// (gfx950 / CDNA4, wave64).
//
// MFMA operand layouts used throughout (16x16 output tiles):
//   v_mfma_f32_16x16x32_bf16  A[16][32], B[32][16]: lane l holds row (A) or
//     column (B) l%16 and the 8 consecutive K-elements 8*(l/16) .. +7.
//   v_mfma_f32_16x16x4_f32    A[16][4],  B[4][16]:  lane l holds row/column
//     l%16 and the single K-element l/16.
//   Output D[16][16] (both):  lane l holds column l%16 and rows
//     4*(l/16) + r in its 4 accumulator registers r = 0..3.
// All kernels put the "per-row statistic" dimension (landmark, query) on the
// output columns, so that softmax state, thresholds and rescaling for one
// landmark or query stay inside the 4 lanes l%16 == const.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mita {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// 2^x with the hardware v_exp_f32 (about 1 ulp; -inf gives 0, results below
// the fp32 normal range flush to 0, which softmax weights can ignore)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ __bf16 f32_to_bf16(float f) { return static_cast<__bf16>(f); }
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ float bf16_round(float f) { return static_cast<float>(f32_to_bf16(f)); }

// Round-to-nearest-even of an fp64 value straight into bf16 bits (no fp32
// step, so no double rounding).  Written from the IEEE-754 encodings: keep
// the top 8 significant bits (fewer below 2^-126, quantum 2^-133) and round
// on the discarded bits.
__device__ __forceinline__ uint16_t f64_to_bf16_bits_rne(double x) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t sign = static_cast<uint32_t>(u >> 63) << 15;
  const int e = static_cast<int>((u >> 52) & 0x7FF);
  const uint64_t frac = u & ((1ull << 52) - 1);
  if (e == 0x7FF) return static_cast<uint16_t>(sign | 0x7F80u | (frac ? 0x40u : 0u));
  if (e == 0) return static_cast<uint16_t>(sign);  // fp64 subnormals are < 2^-1022
  const int E = e - 1023;
  const uint64_t sig = (1ull << 52) | frac;        // 53 significant bits
  int shift = (E >= -126) ? 45 : (-81 - E);        // bits to drop
  if (shift >= 54) return static_cast<uint16_t>(sign);  // below half the smallest subnormal
  uint64_t keep = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (keep & 1))) ++keep;
  if (E >= -126) {
    int be = E + 127;
    if (keep == 256) {
      keep = 128;
      ++be;
    }
    if (be >= 255) return static_cast<uint16_t>(sign | 0x7F80u);
    return static_cast<uint16_t>(sign | (static_cast<uint32_t>(be) << 7) |
                                 static_cast<uint32_t>(keep & 0x7F));
  }
  // subnormal result: keep counts units of 2^-133; keep == 128 is the
  // smallest normal, which the same bit pattern encodes
  return static_cast<uint16_t>(sign | static_cast<uint32_t>(keep));
}

// ---------------------------------------------------------------------------
// ordered 64-bit selection keys: larger key = better (higher score, then
// lower index).  0 is below every real key and marks an empty slot.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t score_order_bits(float s) {
  uint32_t u = __float_as_uint(s + 0.0f);  // +0.0f turns -0 into +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t make_key(float s, uint32_t index) {
  return (static_cast<uint64_t>(score_order_bits(s)) << 32) | static_cast<uint32_t>(~index);
}
__device__ __forceinline__ float key_score(uint64_t key) {
  uint32_t o = static_cast<uint32_t>(key >> 32);
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint32_t key_index(uint64_t key) {
  return ~static_cast<uint32_t>(key);
}

// ---------------------------------------------------------------------------
// cross-lane helpers (ds_bpermute: any lane pattern, no bank conflicts)
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t lane_read(uint32_t v, int src_lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src_lane << 2, static_cast<int>(v)));
}
__device__ __forceinline__ float lane_read(float v, int src_lane) {
  return __uint_as_float(lane_read(__float_as_uint(v), src_lane));
}
__device__ __forceinline__ uint64_t lane_read(uint64_t v, int src_lane) {
  uint32_t lo = lane_read(static_cast<uint32_t>(v), src_lane);
  uint32_t hi = lane_read(static_cast<uint32_t>(v >> 32), src_lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
// Lanes l and l^16 (l^32) exchanged on the VALU with the gfx950 row/half
// swaps: v_permlane16_swap leaves each lane with its own value and that of
// lane l^16 (one in each result), v_permlane32_swap the same for l^32.  The
// max or sum of the pair is then the same number in both lanes.
__device__ __forceinline__ void xor_pair(float v, int mask, float& a, float& b) {
  const uint32_t u = __float_as_uint(v);
  if (mask == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else if (mask == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    const bool lower = (lane_id() & mask) == 0;
    const float o = lane_read(v, lane_id() ^ mask);
    a = lower ? v : o;
    b = lower ? o : v;
  }
}
// (value, index) of lanes l and l^mask combined: the larger value, on equal
// values the lower index.  Symmetric, so both lanes get the same pair.
__device__ __forceinline__ void xor_argmax(float& v, int& i, int mask) {
  float a, b;
  xor_pair(v, mask, a, b);
  const uint32_t u = static_cast<uint32_t>(i);
  uint32_t ia, ib;
  if (mask == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    ia = r[0];
    ib = r[1];
  } else if (mask == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    ia = r[0];
    ib = r[1];
  } else {
    const bool lower = (lane_id() & mask) == 0;
    const uint32_t o = lane_read(u, lane_id() ^ mask);
    ia = lower ? u : o;
    ib = lower ? o : u;
  }
  const bool take_b = b > a || (b == a && static_cast<int>(ib) < static_cast<int>(ia));
  v = take_b ? b : a;
  i = static_cast<int>(take_b ? ib : ia);
}

// max that propagates NaN (IEEE maximum): one v_maximum3 instruction, where
// fmaxf first has to quiet both operands; equal to fmaxf for non-NaN input
__device__ __forceinline__ float fmax_nc(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float xor_max(float v, int mask) {
  float a, b;
  xor_pair(v, mask, a, b);
  return fmax_nc(a, b);
}
__device__ __forceinline__ float xor_sum(float v, int mask) {
  float a, b;
  xor_pair(v, mask, a, b);
  return a + b;
}

// wave-uniform read of lane `l`'s value
__device__ __forceinline__ uint32_t uniform_read(uint32_t v, int l) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
}
__device__ __forceinline__ uint64_t uniform_read(uint64_t v, int l) {
  uint32_t lo = uniform_read(static_cast<uint32_t>(v), l);
  uint32_t hi = uniform_read(static_cast<uint32_t>(v >> 32), l);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// number of set bits of `mask` in lanes below the calling lane
__device__ __forceinline__ uint32_t count_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// ---------------------------------------------------------------------------
// wave-wide bitonic networks on one 64-bit key per lane (descending order)
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint64_t cmpx_desc(uint64_t v, int stride, bool desc_block) {
  const int l = lane_id();
  const uint64_t o = lane_read(v, l ^ stride);
  const bool lower = (l & stride) == 0;
  const bool take_max = (desc_block == lower);
  return take_max ? (v > o ? v : o) : (v < o ? v : o);
}

// sort 64 keys (one per lane) so that lane 0 holds the largest
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v) {
  const int l = lane_id();
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
    const bool desc_block = (l & size) == 0;
#pragma unroll
    for (int stride = size >> 1; stride >= 1; stride >>= 1) v = cmpx_desc(v, stride, desc_block);
  }
  return v;
}

// sort 64 keys of which only lanes 0..W-1 may be nonzero (W a power of two):
// the network's stages up to size W sort lanes 0..W-1 descending and leave
// the zero lanes zero, so the whole wave is then in descending order
template <int W>
__device__ __forceinline__ uint64_t wave_sort_desc_first(uint64_t v) {
  const int l = lane_id();
#pragma unroll
  for (int size = 2; size <= W; size <<= 1) {
    const bool desc_block = (l & size) == 0;
#pragma unroll
    for (int stride = size >> 1; stride >= 1; stride >>= 1) v = cmpx_desc(v, stride, desc_block);
  }
  return v;
}

// sort a bitonic sequence of 64 keys into descending order
__device__ __forceinline__ uint64_t wave_merge_desc(uint64_t v) {
#pragma unroll
  for (int stride = 32; stride >= 1; stride >>= 1) v = cmpx_desc(v, stride, true);
  return v;
}

// top (sorted descending, one key per lane) <- the 64 largest keys of
// top and cand (cand sorted descending).  max(top[i], cand[63-i]) keeps the
// 64 largest of the union as a bitonic sequence.
__device__ __forceinline__ uint64_t wave_merge_top(uint64_t top, uint64_t cand_sorted) {
  const uint64_t rev = lane_read(cand_sorted, 63 - lane_id());
  const uint64_t x = top > rev ? top : rev;
  return wave_merge_desc(x);
}

// ascending sort of one int32 per lane
__device__ __forceinline__ int32_t wave_sort_asc_i32(int32_t v) {
  const int l = lane_id();
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
    const bool asc_block = (l & size) == 0;
#pragma unroll
    for (int stride = size >> 1; stride >= 1; stride >>= 1) {
      const int32_t o = static_cast<int32_t>(lane_read(static_cast<uint32_t>(v), l ^ stride));
      const bool lower = (l & stride) == 0;
      const bool take_min = (asc_block == lower);
      v = take_min ? (v < o ? v : o) : (v > o ? v : o);
    }
  }
  return v;
}

// ---------------------------------------------------------------------------
// MFMA
// ---------------------------------------------------------------------------

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 join_f16x8(u32x2 lo, u32x2 hi) {
  u32x4 v = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(f16x8, v);
}
// two fp32 values -> one dword of two fp16 (round to nearest even)
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}
// 2^e as a float for -126 <= e <= 127
__device__ __forceinline__ float exp2i(int e) { return __uint_as_float(static_cast<uint32_t>(e + 127) << 23); }
__device__ __forceinline__ bf16x8 join_bf16x8(u32x2 lo, u32x2 hi) {
  u32x4 v = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8, v);
}

// split 8 fp32 values into bf16 hi + lo parts (hi = rne(p), lo = rne(p - hi))
// so that hi + lo carries ~16 significant bits into a bf16 MFMA
__device__ __forceinline__ void split_hi_lo(const float (&p)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = f32_to_bf16(p[i]);
    hi[i] = h;
    lo[i] = f32_to_bf16(p[i] - static_cast<float>(h));
  }
}

// the same split with pairwise conversions (one v_cvt_pk_bf16_f32 per two
// values); hi and lo are identical to split_hi_lo's
__device__ __forceinline__ void split_hi_lo_pk(const float (&p)[8], bf16x8& hi, bf16x8& lo) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const bf16x2 h = __builtin_convertvector(f32x2{p[i], p[i + 1]}, bf16x2);
    const f32x2 hf = __builtin_convertvector(h, f32x2);
    const bf16x2 r = __builtin_convertvector(f32x2{p[i] - hf[0], p[i + 1] - hf[1]}, bf16x2);
    hi[i] = h[0];
    hi[i + 1] = h[1];
    lo[i] = r[0];
    lo[i + 1] = r[1];
  }
}

// ---------------------------------------------------------------------------
// element types
// ---------------------------------------------------------------------------

struct BF16 {
  using elem = uint16_t;
  static constexpr int kBytes = 2;
  __device__ static float to_f32(elem v) { return bf16_to_f32(v); }
  __device__ static elem from_f64(double x) { return f64_to_bf16_bits_rne(x); }
};

struct F32 {
  using elem = float;
  static constexpr int kBytes = 4;
  __device__ static float to_f32(elem v) { return v; }
  __device__ static elem from_f64(double x) { return static_cast<float>(x); }  // RNE
};

}  // namespace mita
