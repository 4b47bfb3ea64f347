// kernels_backward.hip — the backward pass (training) of MiTA attention: the
// gradients dQ, dK, dV of sum(dout * out) with the experts idx and the routes
// held fixed (the selections carry no gradient) and the rounding of the
// landmark queries into the input type taken as the identity.  The pages'
// wall-clock results are training times ("NeurIPS'26：注意力也是FFN？…",
// section "长序列建模：训练时间从10.6小时降至2.4小时"; "Mixture-of-Top-k
// 注意力…", section "实验结果：接近完整注意力，长序列训练时间减少约 77%").
//
// The forward, per head (Ql[i] the mean of Q over window i, scale s):
//   A  = softmax_rows(s Ql K^T)           (m x N)    Vl = A V
//   out[q] = sum_p w_qp val_p,  w_q = softmax(s q . key_p) over the m + k
//   pairs p of q (keys [Ql; K[idx[route[q]]]], values [Vl; V[idx[...]]]).
// Its reverse, in launch order (all on the caller's stream):
//   zero      the expert step's per-(expert, key) sums = 0 (a fill kernel)
//   pool      Ql exactly as the forward computes it (the pooling kernel)
//   lmfwd     per key chunk: online-softmax partials of A V   (fp32 MFMA)
//   lmmerge   Vl and the log-sum-exp of each landmark row
//   count / prefix / scatter   the queries grouped by their given routes
//   attend    per expert work item (one expert, <= tpb * 64 queries):
//               g_qp = s w_qp (dout_q . val_p - dout_q . out_q)
//               dQ[q] = sum_p g_qp key_p          (stored: complete but for
//                                                   the pooling term)
//               sums per (expert, key) += g^T Q, w^T dout (atomics)
//               dQl/dVl partials of the item     (summed by reduce1)
//   reduce1   dVl, the expert step's dQl, and D_i = dVl_i . Vl_i
//   cross     per key chunk: h_it = s A_it (dVl_i . V_t - D_i);
//               dK[t] = sum_i h_it Ql_i,  dV[t] = sum_i A_it dVl_i
//               (stored: one block owns each key), and partials of
//               dQl += h K
//   keyadd    dK, dV at each expert key += the expert step's sums (atomics)
//   reduce2   dQl in full, divided by each window's size
//   poolbw    dQ[t] += sum over the windows i containing t of dQl_i / |W_i|
// With fp32 inputs every contraction runs on v_mfma_f32_16x16x4_f32 (fp32
// operands, fp32 accumulation).  With bf16 inputs the score products run on
// bf16 MFMA from the exact bf16 rows, and every other product of the
// landmark forward, the expert step and the cross step on bf16 MFMA too: operands exact in bf16 (Q, K, V rows) as they are, the
// computed ones (dout, Vl, g, the weights w) split into bf16 hi + lo parts
// (hi = rne(x), lo = rne(x - hi)), the lo x lo term dropped, so that each
// product is within about 2^-16 of the exact one, relative; fp32
// accumulation throughout.
//
// Roofline: per (token, head) the pass reads Q, K, V (3 d e bytes, e the
// input element size; K and V twice, in the landmark forward and the cross
// step) and dout (4d), and writes dQ, dK, dV (12d) plus dQ's
// read-modify-write in poolbw (8d): about 5de + 24d bytes.  The contractions cost about 2 d (5 (m + k) + 7 m)
// flops per (token, head) at fp32 MFMA rate, which exceeds the bytes' time
// at 157 TFLOP/s for m = k = 64: with fp32 operands the pass is MFMA-bound.
// On bf16 MFMA the expert step is bound by the latency of its dependent
// phases instead.
#include <type_traits>

#include "mita.h"
#include "mita_bucket.hpp"
#include "mita_device.hpp"
#include "mita_internal.hpp"

namespace mita {
namespace {

constexpr int kBwSt = 68;         // fp32 LDS row stride (64 + 4)
constexpr int kBwPairs = 128;     // m + k rounded up to 16 each, at most
constexpr int kBwGsSt = kBwPairs + 4;
constexpr int kBf16St = 72;       // bf16 LDS row stride (64 + 8: 144 B, 16-byte aligned)

// eight consecutive elements of a row, as fp32
__device__ __forceinline__ void load8(const uint16_t* __restrict__ p, float (&v)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* __restrict__ p, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}
// eight consecutive elements held in their storage type (a load in flight
// while the wave computes), converted to fp32 when stored to LDS
template <class T>
struct Raw8;
template <>
struct Raw8<BF16> {
  u32x4 w;
  __device__ void load(const uint16_t* __restrict__ p) { w = *reinterpret_cast<const u32x4*>(p); }
  __device__ void zero() { w = u32x4{0u, 0u, 0u, 0u}; }
  // the 8 bf16 values as they are (a bf16 LDS row)
  __device__ void store_raw(uint16_t* dst) const { *reinterpret_cast<u32x4*>(dst) = w; }
  __device__ void store(float* dst) const {
    *reinterpret_cast<f32x4*>(dst) = f32x4{__uint_as_float(w[0] << 16),
                                           __uint_as_float(w[0] & 0xFFFF0000u),
                                           __uint_as_float(w[1] << 16),
                                           __uint_as_float(w[1] & 0xFFFF0000u)};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{__uint_as_float(w[2] << 16),
                                               __uint_as_float(w[2] & 0xFFFF0000u),
                                               __uint_as_float(w[3] << 16),
                                               __uint_as_float(w[3] & 0xFFFF0000u)};
  }
};
template <>
struct Raw8<F32> {
  __device__ void store_raw(float* dst) const { store(dst); }
  f32x4 a, b;
  __device__ void load(const float* __restrict__ p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ void zero() { a = b = f32x4{0.f, 0.f, 0.f, 0.f}; }
  __device__ void store(float* dst) const {
    *reinterpret_cast<f32x4*>(dst) = a;
    *reinterpret_cast<f32x4*>(dst + 4) = b;
  }
};

// One 16 x 16 block of scores X Y^T over the 64 dims, X's row c16 held by
// the lane as the MFMA A operand (loaded once, used against several Y
// blocks), Y's rows from LDS.  bf16 inputs: two v_mfma_f32_16x16x32_bf16
// from bf16 rows (stride kBf16St elements), exact products; fp32 inputs:
// sixteen v_mfma_f32_16x16x4f32 from fp32 rows (stride kBwSt).  Output
// D[4g + r][c16], as every MFMA here.
template <class T>
struct ScoreA;
template <>
struct ScoreA<BF16> {
  bf16x8 a0, a1;
  __device__ void load(const float* base, int row, int g) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + row * kBf16St + 8 * g;
    a0 = as_bf16x8(*reinterpret_cast<const u32x4*>(p));
    a1 = as_bf16x8(*reinterpret_cast<const u32x4*>(p + 32));
  }
  __device__ f32x4 score(const float* ybase, int yrow, int g) const {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(ybase) + yrow * kBf16St + 8 * g;
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
    c = mfma_bf16(a0, as_bf16x8(*reinterpret_cast<const u32x4*>(p)), c);
    return mfma_bf16(a1, as_bf16x8(*reinterpret_cast<const u32x4*>(p + 32)), c);
  }
};
template <>
struct ScoreA<F32> {
  float a[16];
  __device__ void load(const float* base, int row, int g) {
#pragma unroll
    for (int s = 0; s < 16; ++s) a[s] = base[row * kBwSt + 4 * s + g];
  }
  __device__ f32x4 score(const float* ybase, int yrow, int g) const {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s) c = mfma_f32(a[s], ybase[yrow * kBwSt + 4 * s + g], c);
    return c;
  }
};

// Max and sum over the 16 lanes of a row (lanes 16j .. 16j + 15), every
// lane getting the result, on the VALU with DPP lane moves: two quad
// swaps, then the half-row mirror (quads 0 <-> 1, 2 <-> 3 of each 8) and
// the row mirror (the two halves), so that each step combines two partial
// results that cover disjoint lanes.
__device__ __forceinline__ float dpp_f(float v, int ctrl_sel) {
  const int x = __float_as_int(v);
  int y;
  switch (ctrl_sel) {  // the control must be a constant
    case 0: y = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false); break;   // quad_perm [1,0,3,2]
    case 1: y = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
    case 2: y = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    default: y = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false); break; // row_mirror
  }
  return __int_as_float(y);
}
__device__ __forceinline__ float row16_max(float v) {
#pragma unroll
  for (int c = 0; c < 4; ++c) v = fmaxf(v, dpp_f(v, c));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
  for (int c = 0; c < 4; ++c) v += dpp_f(v, c);
  return v;
}

// four consecutive elements, as fp32
__device__ __forceinline__ void load4(const uint16_t* __restrict__ p, float (&v)[4]) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  v[0] = __uint_as_float(w[0] << 16);
  v[1] = __uint_as_float(w[0] & 0xFFFF0000u);
  v[2] = __uint_as_float(w[1] << 16);
  v[3] = __uint_as_float(w[1] & 0xFFFF0000u);
}
__device__ __forceinline__ void load4(const float* __restrict__ p, float (&v)[4]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  v[0] = a[0];
  v[1] = a[1];
  v[2] = a[2];
  v[3] = a[3];
}
__device__ __forceinline__ void zero8(float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t n) {
  return v < 0 ? 0 : (v >= n ? n - 1 : v);
}

// Adaptive-pooling bin a of n bins over g cells: [floor(a g / n), ceil((a + 1) g / n)).
__device__ __forceinline__ void bin_range(int64_t a, int64_t g, int64_t n, int64_t& b0,
                                          int64_t& b1) {
  b0 = (a * g) / n;
  b1 = ((a + 1) * g + n - 1) / n;
}

// ---------------------------------------------------------------------------
// zero fill (the expert step's per-(expert, key) sums) — a kernel, not a
// memset, so the sequence stays capturable in a graph
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bw_zero(f32x4* __restrict__ a, f32x4* __restrict__ b,
                                                 int64_t n4) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    a[i] = z;
    b[i] = z;
  }
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x16_bf16: A[16][16], B[16][16], lane l holds row (A) or
// column (B) l % 16 and the 4 consecutive K-elements 4 (l / 16) .. + 3
__device__ __forceinline__ f32x4 mfma_bf16_k16(v4i16 a, v4i16 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// 4 fp32 values as bf16 hi = rne(x) and lo = rne(x - hi)
__device__ __forceinline__ void split4(const float (&x)[4], v4i16& hi, v4i16& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const __bf16 h = static_cast<__bf16>(x[i]);
    hi[i] = __builtin_bit_cast(short, h);
    lo[i] = __builtin_bit_cast(short, static_cast<__bf16>(x[i] - static_cast<float>(h)));
  }
}
__device__ __forceinline__ void split4(const f32x4& x, v4i16& hi, v4i16& lo) {
  const float v[4] = {x[0], x[1], x[2], x[3]};
  split4(v, hi, lo);
}

// ---------------------------------------------------------------------------
// landmark cross-attention, forward (Vl and its row log-sum-exp)
// ---------------------------------------------------------------------------

// Block (chunk, head): keys [chunk * csize, ...) in 16-key groups, wave w
// taking groups w, w + 4, ...  Per group: S^T = K_g Ql^T (keys on rows,
// landmarks on columns), the running column maximum and sum, and
// acc^T (dims x landmarks) += V_g^T P^T — the landmark on the output column
// keeps each landmark's rescale inside its own lanes.  The four waves'
// states are combined into the block's partial: stats [BH][P][64][2] (max
// in log2 units, sum), acc [BH][P][64][64], P = chunks.
template <class T, int MB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_bw_lmfwd(const typename T::elem* __restrict__ K,
                                                  const typename T::elem* __restrict__ V,
                                                  const typename T::elem* __restrict__ ql,
                                                  int64_t N, int m, int csize, float c2,
                                                  float* __restrict__ part_stats,
                                                  float* __restrict__ part_acc) {
  constexpr int MP = 16 * MB;
  constexpr bool kBf = std::is_same<T, BF16>::value;
  // bf16: the scores run on bf16 MFMA from bf16 copies of Ql and K (exact);
  // fp32: on fp32 MFMA from fp32 copies.  V is staged in fp32 for P.V.
  constexpr int kQlWords = kBf ? MP * kBf16St / 2 : MP * kBwSt;
  constexpr int kKWords = kBf ? 16 * kBf16St / 2 : 16 * kBwSt;
  constexpr int kStage = kQlWords + 4 * (kKWords + 16 * kBwSt);
  constexpr int kComb = 3 * MP * (kD + 2);  // waves 1..3's states at the end
  constexpr int kWords = kStage > kComb ? kStage : kComb;
  __shared__ __attribute__((aligned(16))) float smem[kWords];
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int64_t bh = blockIdx.y;
  const int P = static_cast<int>(gridDim.x);
  for (int u = threadIdx.x; u < MP * 8; u += 256) {
    const int row = u >> 3, j = u & 7;
    Raw8<T> v;
    if (row < m)
      v.load(ql + (bh * m + row) * kD + 8 * j);
    else
      v.zero();
    if constexpr (kBf)
      v.store_raw(reinterpret_cast<uint16_t*>(smem) + row * kBf16St + 8 * j);
    else
      v.store(smem + row * kBwSt + 8 * j);
  }
  __syncthreads();
  const int64_t k0 = static_cast<int64_t>(blockIdx.x) * csize;
  const int64_t k1 = k0 + csize < N ? k0 + csize : N;
  float M[MB], L[MB];
  f32x4 acc[MB][4];
#pragma unroll
  for (int lb = 0; lb < MB; ++lb) {
    M[lb] = -INFINITY;
    L[lb] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[lb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float* const sKw = smem + kQlWords + w * (kKWords + 16 * kBwSt);  // this wave's K rows
  float* const sV = sKw + kKWords;                                   // and V rows (fp32)
  // this wave's 16 keys, one group ahead: lane l holds chunks l and l + 64
  // (row u / 8, elements 8 (u % 8) ..) of K and V
  Raw8<T> rk[2], rv[2];
  auto fetch = [&](int64_t t0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int u = l + 64 * h;
      const int64_t t = t0 + (u >> 3);
      if (t < k1) {
        rk[h].load(K + (bh * N + t) * kD + 8 * (u & 7));
        rv[h].load(V + (bh * N + t) * kD + 8 * (u & 7));
      } else {
        rk[h].zero();
        rv[h].zero();
      }
    }
  };
  fetch(k0 + 16 * w);
  for (int64_t t0 = k0 + 16 * w; t0 < k1; t0 += 64) {
    // (the wave's LDS accesses complete in program order)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int u = l + 64 * h;
      if constexpr (kBf) {
        rk[h].store_raw(reinterpret_cast<uint16_t*>(sKw) + (u >> 3) * kBf16St + 8 * (u & 7));
        rv[h].store_raw(reinterpret_cast<uint16_t*>(sV) + (u >> 3) * kBf16St + 8 * (u & 7));
      } else {
        rk[h].store(sKw + (u >> 3) * kBwSt + 8 * (u & 7));
        rv[h].store(sV + (u >> 3) * kBwSt + 8 * (u & 7));
      }
    }
    fetch(t0 + 64);
    ScoreA<T> a;
    a.load(sKw, c16, g);
    // bf16: V^T (feature 16 db + c16, keys 4 g .. 4 g + 3; exact) as the A
    // operand of v_mfma_f32_16x16x16_bf16, P as hi + lo the B operand
    v4i16 vt[4];
    if constexpr (kBf) {
      const uint16_t* v16 = reinterpret_cast<const uint16_t*>(sV);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) vt[db][j] = static_cast<short>(v16[(4 * g + j) * kBf16St + 16 * db + c16]);
    }
#pragma unroll
    for (int lb = 0; lb < MB; ++lb) {
      const f32x4 S = a.score(smem, 16 * lb + c16, g);
      // S[r]: key t0 + 4g + r, landmark 16 lb + c16
      float x[4];
      float cm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = (t0 + 4 * g + r < k1) ? S[r] * c2 : -INFINITY;
        cm = fmaxf(cm, x[r]);
      }
      cm = xor_max(cm, 16);
      cm = xor_max(cm, 32);
      const float Mn = fmaxf(M[lb], cm);  // finite: key t0 is in range
      const float f = fast_exp2(M[lb] - Mn);
      float p[4], ps = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = fast_exp2(x[r] - Mn);
        ps += p[r];
      }
      ps = xor_sum(ps, 16);
      ps = xor_sum(ps, 32);
      L[lb] = L[lb] * f + ps;
      M[lb] = Mn;
      if constexpr (kBf) {
        v4i16 ph, pl;
        split4(p, ph, pl);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          acc[lb][db] *= f;
          acc[lb][db] = mfma_bf16_k16(vt[db], ph, acc[lb][db]);
          acc[lb][db] = mfma_bf16_k16(vt[db], pl, acc[lb][db]);
        }
      } else {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          acc[lb][db] *= f;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[lb][db] = mfma_f32(sV[(4 * g + r) * kBwSt + 16 * db + c16], p[r], acc[lb][db]);
        }
      }
    }
  }
  // the four waves' states combined by wave 0 (acc[lb][db][r]: dim
  // 16 db + 4 g + r of landmark 16 lb + c16)
  float* const xacc = smem;                // [3][MP][64]
  float* const xst = smem + 3 * MP * kD;   // [3][MP][2]
  __syncthreads();  // every wave done with its staging rows
  if (w > 0) {
#pragma unroll
    for (int lb = 0; lb < MB; ++lb) {
      const int row = (w - 1) * MP + 16 * lb + c16;
      if (g == 0) {
        xst[row * 2] = M[lb];
        xst[row * 2 + 1] = L[lb];
      }
#pragma unroll
      for (int db = 0; db < 4; ++db)
        *reinterpret_cast<f32x4*>(xacc + row * kD + 16 * db + 4 * g) = acc[lb][db];
    }
  }
  __syncthreads();
  if (w > 0) return;
  const int64_t pbase = (bh * P + blockIdx.x) * kMaxM;
#pragma unroll
  for (int lb = 0; lb < MB; ++lb) {
    const int i = 16 * lb + c16;
    // wave 0 had keys (the chunk's first group), so Mt is finite
    float Mt = M[lb];
#pragma unroll
    for (int v = 0; v < 3; ++v) Mt = fmaxf(Mt, xst[(v * MP + i) * 2]);
    const float f0 = fast_exp2(M[lb] - Mt);
    float Lt = L[lb] * f0;
    f32x4 at[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) at[db] = acc[lb][db] * f0;
#pragma unroll
    for (int v = 0; v < 3; ++v) {
      const float fv = fast_exp2(xst[(v * MP + i) * 2] - Mt);  // 0 for a wave without keys
      Lt += xst[(v * MP + i) * 2 + 1] * fv;
#pragma unroll
      for (int db = 0; db < 4; ++db)
        at[db] += *reinterpret_cast<const f32x4*>(xacc + (v * MP + i) * kD + 16 * db + 4 * g) * fv;
    }
    const int64_t row = pbase + i;
    if (g == 0) {
      part_stats[row * 2] = Mt;
      part_stats[row * 2 + 1] = Lt;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
      *reinterpret_cast<f32x4*>(part_acc + row * kD + 16 * db + 4 * g) = at[db];
  }
}

// Block (landmark, head), lane = dim: wave w merges partials w, w + 4, ...
// (online), then wave 0 the four results: Vl = acc / sum, lse2 = max +
// log2(sum) (log2 units of the scaled logits).  Every partial has keys.
__global__ __launch_bounds__(256) void k_bw_lmmerge(const float* __restrict__ part_stats,
                                                    const float* __restrict__ part_acc, int m,
                                                    int P, float* __restrict__ vl,
                                                    float* __restrict__ lse2) {
  __shared__ float sM[4], sL[4], sA[4][64];
  const int l = lane_id(), w = wave_id();
  const int64_t bh = blockIdx.y;
  const int i = blockIdx.x;
  float M = -INFINITY, L = 0.f, a = 0.f;
#pragma unroll 4
  for (int p = w; p < P; p += 4) {
    const int64_t row = (bh * P + p) * kMaxM + i;
    const float Mp = part_stats[row * 2];
    const float Lp = part_stats[row * 2 + 1];
    const float ap = part_acc[row * kD + l];
    const float Mn = fmaxf(M, Mp);
    const float f0 = fast_exp2(M - Mn), f1 = fast_exp2(Mp - Mn);
    L = L * f0 + Lp * f1;
    a = a * f0 + ap * f1;
    M = Mn;
  }
  if (l == 0) {
    sM[w] = M;
    sL[w] = L;
  }
  sA[w][l] = a;
  __syncthreads();
  if (w != 0) return;
  const float Mt = fmaxf(fmaxf(sM[0], sM[1]), fmaxf(sM[2], sM[3]));  // wave 0 had a partial
  float Lt = 0.f, at = 0.f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float f = fast_exp2(sM[v] - Mt);  // 0 for a wave without partials
    Lt += sL[v] * f;
    at += sA[v][l] * f;
  }
  vl[(bh * m + i) * kD + l] = at / Lt;
  if (l == 0) lse2[bh * m + i] = Mt + __log2f(Lt);
}

// ---------------------------------------------------------------------------
// grouping of the queries by their given routes (stable counting sort)
// ---------------------------------------------------------------------------

// Block (segment, head): per-expert counts of the segment's routes (routes
// outside [0, m) count as the nearest expert, as the scatter places them).
__global__ __launch_bounds__(256) void k_bw_count(const int32_t* __restrict__ route, int64_t N,
                                                  int m, int nseg, int32_t* __restrict__ counts) {
  __shared__ int cnt[kMaxM];
  if (threadIdx.x < kMaxM) cnt[threadIdx.x] = 0;
  __syncthreads();
  const int64_t bh = blockIdx.y;
  const int seg = blockIdx.x;
  const int64_t q0 = static_cast<int64_t>(seg) * kRouteSeg;
  for (int i = threadIdx.x; i < kRouteSeg; i += 256) {
    const int64_t q = q0 + i;
    if (q < N) {
      int r = route[bh * N + q];
      r = r < 0 ? 0 : (r >= m ? m - 1 : r);
      atomicAdd(&cnt[r], 1);
    }
  }
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < m) counts[(bh * m + threadIdx.x) * nseg + seg] = cnt[threadIdx.x];
}

__global__ __launch_bounds__(256) void k_bw_prefix(const int32_t* __restrict__ counts, int m,
                                                   int nseg, int32_t* __restrict__ colpre,
                                                   int32_t* __restrict__ totals) {
  __shared__ int wsum[4];
  bucket_prefix(counts, m, nseg, blockIdx.x, blockIdx.y, colpre, totals, wsum);
}

__global__ __launch_bounds__(256) void k_bw_scatter(const int32_t* __restrict__ route,
                                                    const int32_t* __restrict__ counts, int m,
                                                    int nseg, int64_t N, int tpb,
                                                    const int32_t* __restrict__ totals,
                                                    const int32_t* __restrict__ colpre,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ item_start,
                                                    int32_t* __restrict__ perm,
                                                    int32_t* __restrict__ item_order) {
  __shared__ ScatterLds L[4];
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  if (blockIdx.x == gridDim.x - 1) {  // trailing block: the expert step's dispatch order
    if (w == 0) write_item_order(totals, m, kAttendTile, tpb, blockIdx.y, item_order);
    return;
  }
  const int seg = static_cast<int>(blockIdx.x) * 4 + w;
  if (seg < nseg)
    scatter_segment(route, counts, m, nseg, N, kAttendTile, tpb, totals, colpre, offsets, nullptr,
                    item_start, perm, nullptr, seg, kRouteSeg, blockIdx.y, L[w]);
}

// ---------------------------------------------------------------------------
// the output softmax, per expert work item
// ---------------------------------------------------------------------------

// Block (work item, head), eight waves in two halves.  The item's expert
// is staged once as fp32 pair rows: keys [Ql; 0; K_e; 0] and values
// [Vl; 0; V_e; 0] with the landmarks padded to MP = 16 ceil(m / 16) rows and
// the raw keys to KP rows (PP = MP + KP <= 128, NB = PP / 16 column
// blocks).  Each half takes every other group of 16 queries (its next
// group's rows are loaded while it computes the current one); within a
// half, wave wl computes the logits and dout . value of column blocks wl
// and wl + 4 (queries on rows, pairs on columns), the row max and the sums
// over the pairs meet in LDS, and then
//   dKey[p] += sum_q g_qp q,  dVal[p] += sum_q w_qp dout_q
// run with the wave's own columns as the MFMA A operand straight from the
// accumulator layout (pairs on the output rows), while dQ = g [keys] takes
// g through LDS, wave wl producing dims 16 wl .. 16 wl + 15 of the 16
// queries.  At the end the second half's sums are added to the first's.
template <class T>
__global__ __launch_bounds__(512) void k_bw_attend(
    const typename T::elem* __restrict__ Q, const typename T::elem* __restrict__ K,
    const typename T::elem* __restrict__ V, const typename T::elem* __restrict__ ql,
    const float* __restrict__ vl, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ item_start, const int32_t* __restrict__ item_order, int tpb,
    int64_t N, int m, int k, float scale,
    const float* __restrict__ dout, float* __restrict__ dQ, float* __restrict__ dke,
    float* __restrict__ dve, float* __restrict__ part, int items) {
  __shared__ __attribute__((aligned(16))) float sPk[kBwPairs * kBwSt];
  __shared__ __attribute__((aligned(16))) float sPv[kBwPairs * kBwSt];
  __shared__ __attribute__((aligned(16))) float sQ[2][16 * kBwSt];
  __shared__ __attribute__((aligned(16))) float sG[2][16 * kBwSt];
  __shared__ __attribute__((aligned(16))) float sGs[2][16 * kBwGsSt];
  __shared__ float sRed[2][3][4][16];
  __shared__ int sQid[2][16];
  // bf16: the pair keys and the query rows also as bf16 rows (exact), for
  // the logits on bf16 MFMA
  constexpr bool kBf = std::is_same<T, BF16>::value;
  __shared__ __attribute__((aligned(16))) float sPk16[kBf ? kBwPairs * kBf16St / 2 : 1];
  __shared__ __attribute__((aligned(16))) float sQ16[2][kBf ? 16 * kBf16St / 2 : 1];
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int hf = w >> 2, wl = w & 3;
  const int tid = threadIdx.x;
  int64_t bh;
  int p;  // the block's position: its partial's slot
  TileInfo ti;
  if (!dispatch_item(item_start, item_order, offsets, m, tpb, bh, p, ti))
    return;  // whole block: past the head's last item
  const int MP = (m + 15) & ~15, KP = (k + 15) & ~15;
  const int PP = MP + KP, NB = PP / 16;
  const int32_t* ex = idx + (bh * m + ti.e) * k;
  for (int u = tid; u < PP * 8; u += 512) {
    const int row = u >> 3, j = u & 7;
    Raw8<T> kv;
    float vv[8];
    if (row < m) {
      kv.load(ql + (bh * m + row) * kD + 8 * j);
      load8(vl + (bh * m + row) * kD + 8 * j, vv);
    } else if (row >= MP && row < MP + k) {
      const int64_t t = clamp64(ex[row - MP], N);
      kv.load(K + (bh * N + t) * kD + 8 * j);
      load8(V + (bh * N + t) * kD + 8 * j, vv);
    } else {
      kv.zero();
      zero8(vv);
    }
    kv.store(sPk + row * kBwSt + 8 * j);
    if constexpr (kBf) kv.store_raw(reinterpret_cast<uint16_t*>(sPk16) + row * kBf16St + 8 * j);
    store8(sPv + row * kBwSt + 8 * j, vv);
  }
  const float* const sPks = kBf ? sPk16 : sPk;  // the rows the logits read
  const float c2 = scale * kLog2e;
  f32x4 aK[2][4], aV[2][4];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      aK[cb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      aV[cb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  // the half's query rows: thread (row, 4 dims), one group ahead
  const int srow = (tid & 255) >> 4, sc4 = tid & 15;
  float pq[4], pg[4];
  int pid = 0;
  auto fetch = [&](int q0h) {
    if (q0h + srow < ti.qe) {
      const int64_t q = clamp64(perm[bh * N + q0h + srow], N);
      load4(Q + (bh * N + q) * kD + 4 * sc4, pq);
      load4(dout + (bh * N + q) * kD + 4 * sc4, pg);
      pid = static_cast<int>(q);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) pq[i] = pg[i] = 0.f;
    }
  };
  fetch(ti.qb + 16 * hf);
  float* const hQ = sQ[hf];
  float* const hG = sG[hf];
  float* const hGs = sGs[hf];
  for (int qq = ti.qb; qq < ti.qe; qq += 32) {
    const int q0 = qq + 16 * hf;
    const int nv = ti.qe - q0 < 0 ? 0 : (ti.qe - q0 < 16 ? ti.qe - q0 : 16);
    __syncthreads();  // the expert staged; the previous groups' LDS reads done
    *reinterpret_cast<f32x4*>(hQ + srow * kBwSt + 4 * sc4) = f32x4{pq[0], pq[1], pq[2], pq[3]};
    if constexpr (kBf)  // the bf16 values, back from their exact fp32 form
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(sQ16[hf]) + srow * kBf16St + 4 * sc4) =
          u32x2{(__float_as_uint(pq[0]) >> 16) | (__float_as_uint(pq[1]) & 0xFFFF0000u),
                (__float_as_uint(pq[2]) >> 16) | (__float_as_uint(pq[3]) & 0xFFFF0000u)};
    *reinterpret_cast<f32x4*>(hG + srow * kBwSt + 4 * sc4) = f32x4{pg[0], pg[1], pg[2], pg[3]};
    if (sc4 == 0) sQid[hf][srow] = pid;
    fetch(q0 + 32);
    __syncthreads();
    ScoreA<T> aq;
    aq.load(kBf ? sQ16[hf] : hQ, c16, g);
    float ag[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) ag[s] = hG[c16 * kBwSt + 4 * s + g];
    f32x4 S[2], dW[2];
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int pb = wl + 4 * cb;
      S[cb] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      dW[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (pb < NB) {  // wave-uniform
        const f32x4 s4 = aq.score(sPks, 16 * pb + c16, g);
        f32x4 d4 = {0.f, 0.f, 0.f, 0.f}, d4b = d4;  // two chains of 8
#pragma unroll
        for (int s = 0; s < 16; s += 2) {
          d4 = mfma_f32(ag[s], sPv[(16 * pb + c16) * kBwSt + 4 * s + g], d4);
          d4b = mfma_f32(ag[s + 1], sPv[(16 * pb + c16) * kBwSt + 4 * (s + 1) + g], d4b);
        }
        d4 += d4b;
        const int p = 16 * pb + c16;
        const bool pv = p < m || (p >= MP && p < MP + k);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          S[cb][r] = pv ? s4[r] * c2 : -INFINITY;  // log2 units
          mx[r] = fmaxf(mx[r], S[cb][r]);
        }
        dW[cb] = d4;
      }
    }
    // row (query) statistics over all pairs in one exchange: each wave's max
    // and sums over its own columns (within 16 lanes), then rescaled to the
    // half's maximum.  A wave without columns (NB <= 3) reports -inf and 0.
    float E[2][4], z[4], y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      mx[r] = row16_max(mx[r]);
      z[r] = 0.f;
      y[r] = 0.f;
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        E[cb][r] = mx[r] == -INFINITY ? 0.f : fast_exp2(S[cb][r] - mx[r]);  // 0 when masked
        z[r] += E[cb][r];
        y[r] += E[cb][r] * dW[cb][r];
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = row16_sum(z[r]);
      y[r] = row16_sum(y[r]);
      if (c16 == 0) {
        sRed[hf][0][wl][4 * g + r] = mx[r];
        sRed[hf][1][wl][4 * g + r] = z[r];
        sRed[hf][2][wl][4 * g + r] = y[r];
      }
    }
    __syncthreads();
    float Wt[2][4], Gs[2][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * g + r;
      float mv[4], M = -INFINITY;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        mv[v] = sRed[hf][0][v][row];
        M = fmaxf(M, mv[v]);
      }
      float Z = 0.f, Y = 0.f;  // M is finite: some wave holds a valid pair
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float f = mv[v] == -INFINITY ? 0.f : fast_exp2(mv[v] - M);
        Z += sRed[hf][1][v][row] * f;
        Y += sRed[hf][2][v][row] * f;
      }
      const float own = mx[r] == -INFINITY ? 0.f : fast_exp2(mx[r] - M);
      const float inv = row < nv ? own / Z : 0.f;  // padding rows contribute nothing
      const float c = Y / Z;                       // dout . out of this query
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        Wt[cb][r] = E[cb][r] * inv;
        Gs[cb][r] = scale * Wt[cb][r] * (dW[cb][r] - c);
      }
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int pb = wl + 4 * cb;
      if (pb >= NB) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) hGs[(4 * g + r) * kBwGsSt + 16 * pb + c16] = Gs[cb][r];
      // pairs on the output rows: A = g^T (pair c16, query 4g + r), B = Q / dout rows
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          aK[cb][db] = mfma_f32(Gs[cb][r], hQ[(4 * g + r) * kBwSt + 16 * db + c16], aK[cb][db]);
          aV[cb][db] = mfma_f32(Wt[cb][r], hG[(4 * g + r) * kBwSt + 16 * db + c16], aV[cb][db]);
        }
    }
    __syncthreads();
    // dQ (16 queries x dims 16 wl .. 16 wl + 15) = g [keys]
    f32x4 dq[4];  // four independent chains over the pair steps
#pragma unroll
    for (int j = 0; j < 4; ++j) dq[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < 4 * NB; s += 4)  // 4 NB is a multiple of 4
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dq[j] = mfma_f32(hGs[c16 * kBwGsSt + 4 * (s + j) + g],
                         sPk[(4 * (s + j) + g) * kBwSt + 16 * wl + c16], dq[j]);
    dq[0] += dq[1] + dq[2] + dq[3];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * g + r;
      if (row < nv) dQ[(bh * N + sQid[hf][row]) * kD + 16 * wl + c16] = dq[0][r];
    }
  }
  // the second half's sums into the first's (through the staged expert's LDS)
  __syncthreads();
  if (hf == 1) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int pb = wl + 4 * cb;
      if (pb >= NB) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          sPk[(16 * pb + 4 * g + r) * kBwSt + 16 * db + c16] = aK[cb][db][r];
          sPv[(16 * pb + 4 * g + r) * kBwSt + 16 * db + c16] = aV[cb][db][r];
        }
    }
  }
  __syncthreads();
  if (hf == 1) return;
  // the item's sums: landmark rows to its partial, raw-key rows to the
  // expert's key sums
  float* pq_ = part + ((bh * items + p) * 2) * static_cast<int64_t>(m) * kD;
  float* pv_ = pq_ + static_cast<int64_t>(m) * kD;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int pb = wl + 4 * cb;
    if (pb >= NB) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = 16 * pb + 4 * g + r;
      float sk[4], sv[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        sk[db] = aK[cb][db][r] + sPk[p * kBwSt + 16 * db + c16];
        sv[db] = aV[cb][db][r] + sPv[p * kBwSt + 16 * db + c16];
      }
      if (p < m) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          pq_[p * kD + 16 * db + c16] = sk[db];
          pv_[p * kD + 16 * db + c16] = sv[db];
        }
      } else if (p >= MP && p < MP + k) {
        const int64_t row = (bh * m + ti.e) * k + (p - MP);  // expert e's j-th key
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          unsafeAtomicAdd(dke + row * kD + 16 * db + c16, sk[db]);
          unsafeAtomicAdd(dve + row * kD + 16 * db + c16, sv[db]);
        }
      }
    }
  }
}

// The same step for bf16 inputs in four-wave blocks whose LDS fits two
// blocks per CU (about 62 KiB), so that one block's barriers overlap the
// other's work: every operand that is exact in bf16 stays bf16 in LDS (the
// pair keys [Ql; K_e], the raw values V_e, the query rows), the landmark
// values as bf16 hi + lo, dout and g as fp32.  Every product runs on bf16
// MFMA: dout . [Vl; V_e]^T and g . [Ql; K_e] on v_mfma_f32_16x16x32_bf16,
// the pair-side sums g^T Q and w^T dout on v_mfma_f32_16x16x16_bf16 (its
// A operand is the lane's own four weights), computed operands as hi + lo
// (expert step at 2^20 tokens x 4 heads: 3.84 -> 2.45 ms against fp32
// MFMA).  One group of 16 queries at a time (the next group's rows in
// registers meanwhile); wave w owns column blocks w and w + 4 and dims
// 16 w .. 16 w + 15 of dQ, as in k_bw_attend.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_bw_attend_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ ql,
    const float* __restrict__ vl, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ item_start, const int32_t* __restrict__ item_order, int tpb,
    int64_t N, int m, int k, float scale,
    const float* __restrict__ dout, float* __restrict__ dQ, float* __restrict__ dke,
    float* __restrict__ dve, float* __restrict__ part, int items) {
  __shared__ __attribute__((aligned(16))) uint16_t sPk[kBwPairs * kBf16St];  // [Ql; 0; K_e; 0]
  __shared__ __attribute__((aligned(16))) uint16_t sVlh[kMaxM * kBf16St];   // Vl rows, bf16 hi
  __shared__ __attribute__((aligned(16))) uint16_t sVll[kMaxM * kBf16St];   // Vl rows, bf16 lo
  __shared__ __attribute__((aligned(16))) uint16_t sV[kMaxK * kBf16St];     // V_e rows
  __shared__ __attribute__((aligned(16))) uint16_t sQ[16 * kBf16St];
  __shared__ __attribute__((aligned(16))) float sG[16 * kBwSt];
  __shared__ __attribute__((aligned(16))) float sGs[16 * kBwGsSt];
  __shared__ float sRed[3][4][16];
  __shared__ int sQid[16];
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int tid = threadIdx.x;
  int64_t bh;
  int p;  // the block's position: its partial's slot
  TileInfo ti;
  if (!dispatch_item(item_start, item_order, offsets, m, tpb, bh, p, ti))
    return;  // whole block: past the head's last item
  const int MP = (m + 15) & ~15, KP = (k + 15) & ~15;
  const int PP = MP + KP, NB = PP / 16;
  const int32_t* ex = idx + (bh * m + ti.e) * k;
  for (int u = tid; u < PP * 8; u += 256) {
    const int row = u >> 3, j = u & 7;
    Raw8<BF16> kv;
    if (row < m) {
      kv.load(ql + (bh * m + row) * kD + 8 * j);
      float vv[8];
      load8(vl + (bh * m + row) * kD + 8 * j, vv);
      bf16x8 hi, lo;
      split_hi_lo_pk(vv, hi, lo);
      *reinterpret_cast<bf16x8*>(sVlh + row * kBf16St + 8 * j) = hi;
      *reinterpret_cast<bf16x8*>(sVll + row * kBf16St + 8 * j) = lo;
    } else if (row >= MP && row < MP + k) {
      const int64_t t = clamp64(ex[row - MP], N);
      kv.load(K + (bh * N + t) * kD + 8 * j);
      Raw8<BF16> v8;
      v8.load(V + (bh * N + t) * kD + 8 * j);
      v8.store_raw(sV + (row - MP) * kBf16St + 8 * j);
    } else {
      kv.zero();
      if (row < MP) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(sVlh + row * kBf16St + 8 * j) = z;
        *reinterpret_cast<u32x4*>(sVll + row * kBf16St + 8 * j) = z;
      } else {
        Raw8<BF16> z;
        z.zero();
        z.store_raw(sV + (row - MP) * kBf16St + 8 * j);
      }
    }
    kv.store_raw(sPk + row * kBf16St + 8 * j);
  }
  const float c2 = scale * kLog2e;
  f32x4 aK[2][4], aV[2][4];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      aK[cb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      aV[cb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  // one group ahead: thread (row, 4 dims) of Q (8 bytes) and of dout
  const int srow = tid >> 4, sc4 = tid & 15;
  u32x2 pq = {0u, 0u};
  f32x4 pg = {0.f, 0.f, 0.f, 0.f};
  int pid = 0;
  auto fetch = [&](int q0) {
    if (q0 + srow < ti.qe) {
      const int64_t q = clamp64(perm[bh * N + q0 + srow], N);
      pq = *reinterpret_cast<const u32x2*>(Q + (bh * N + q) * kD + 4 * sc4);
      pg = *reinterpret_cast<const f32x4*>(dout + (bh * N + q) * kD + 4 * sc4);
      pid = static_cast<int>(q);
    } else {
      pq = u32x2{0u, 0u};
      pg = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  // element (row, col) of a bf16 LDS array, widened
  auto bf = [](const uint16_t* a, int i) { return bf16_to_f32(a[i]); };
  fetch(ti.qb);
  for (int q0 = ti.qb; q0 < ti.qe; q0 += 16) {
    const int nv = ti.qe - q0 < 16 ? ti.qe - q0 : 16;
    __syncthreads();  // the expert staged; the previous group's LDS reads done
    *reinterpret_cast<u32x2*>(sQ + srow * kBf16St + 4 * sc4) = pq;
    *reinterpret_cast<f32x4*>(sG + srow * kBwSt + 4 * sc4) = pg;
    if (sc4 == 0) sQid[srow] = pid;
    fetch(q0 + 16);
    __syncthreads();
    ScoreA<BF16> aq;
    aq.load(reinterpret_cast<const float*>(sQ), c16, g);
    // dout of query c16, features 32 s + 8 g .. + 7, as bf16 hi + lo (the
    // A operand of dout . [Vl; V_e]^T)
    bf16x8 agh[2], agl[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(sG + c16 * kBwSt + 32 * s + 8 * g);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(sG + c16 * kBwSt + 32 * s + 8 * g + 4);
      const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      split_hi_lo_pk(x, agh[s], agl[s]);
    }
    // queries 4 g .. 4 g + 3 at feature 16 db + c16: Q (exact bf16) and dout
    // (hi + lo), the B operands of the key and value sums
    v4i16 bq[4], bgh[4], bgl[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bq[db][j] = static_cast<short>(sQ[(4 * g + j) * kBf16St + 16 * db + c16]);
        x[j] = sG[(4 * g + j) * kBwSt + 16 * db + c16];
      }
      split4(x, bgh[db], bgl[db]);
    }
    f32x4 S[2], dW[2];
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int pb = w + 4 * cb;
      S[cb] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      dW[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (pb < NB) {  // wave-uniform
        const f32x4 s4 = aq.score(reinterpret_cast<const float*>(sPk), 16 * pb + c16, g);
        f32x4 d4 = {0.f, 0.f, 0.f, 0.f}, d4b = d4;  // two chains of 8
        const int p = 16 * pb + c16;
        if (16 * pb < MP) {  // landmark values: hi + lo by hi + lo, lo x lo dropped
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const bf16x8 vh = as_bf16x8(*reinterpret_cast<const u32x4*>(sVlh + p * kBf16St + 32 * s + 8 * g));
            const bf16x8 vo = as_bf16x8(*reinterpret_cast<const u32x4*>(sVll + p * kBf16St + 32 * s + 8 * g));
            d4 = mfma_bf16(agh[s], vh, d4);
            d4b = mfma_bf16(agl[s], vh, d4b);
            d4 = mfma_bf16(agh[s], vo, d4);
          }
        } else {  // raw values (exact bf16)
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const bf16x8 vr = as_bf16x8(*reinterpret_cast<const u32x4*>(sV + (p - MP) * kBf16St + 32 * s + 8 * g));
            d4 = mfma_bf16(agh[s], vr, d4);
            d4b = mfma_bf16(agl[s], vr, d4b);
          }
        }
        d4 += d4b;
        const bool pv = p < m || (p >= MP && p < MP + k);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          S[cb][r] = pv ? s4[r] * c2 : -INFINITY;  // log2 units
          mx[r] = fmaxf(mx[r], S[cb][r]);
        }
        dW[cb] = d4;
      }
    }
    // row statistics in one exchange (each wave's own max and sums over its
    // columns, rescaled to the block's maximum; a wave without columns
    // reports -inf and 0)
    float E[2][4], z[4], y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      mx[r] = row16_max(mx[r]);
      z[r] = 0.f;
      y[r] = 0.f;
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        E[cb][r] = mx[r] == -INFINITY ? 0.f : fast_exp2(S[cb][r] - mx[r]);
        z[r] += E[cb][r];
        y[r] += E[cb][r] * dW[cb][r];
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = row16_sum(z[r]);
      y[r] = row16_sum(y[r]);
      if (c16 == 0) {
        sRed[0][w][4 * g + r] = mx[r];
        sRed[1][w][4 * g + r] = z[r];
        sRed[2][w][4 * g + r] = y[r];
      }
    }
    __syncthreads();
    float Wt[2][4], Gs[2][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * g + r;
      float mv[4], M = -INFINITY;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        mv[v] = sRed[0][v][row];
        M = fmaxf(M, mv[v]);
      }
      float Z = 0.f, Y = 0.f;  // M is finite: some wave holds a valid pair
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float f = mv[v] == -INFINITY ? 0.f : fast_exp2(mv[v] - M);
        Z += sRed[1][v][row] * f;
        Y += sRed[2][v][row] * f;
      }
      const float own = mx[r] == -INFINITY ? 0.f : fast_exp2(mx[r] - M);
      const float inv = row < nv ? own / Z : 0.f;  // padding rows contribute nothing
      const float c = Y / Z;                       // dout . out of this query
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        Wt[cb][r] = E[cb][r] * inv;
        Gs[cb][r] = scale * Wt[cb][r] * (dW[cb][r] - c);
      }
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int pb = w + 4 * cb;
      if (pb >= NB) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) sGs[(4 * g + r) * kBwGsSt + 16 * pb + c16] = Gs[cb][r];
      // sums over the 16 queries on v_mfma_f32_16x16x16_bf16: A = the lane's
      // own 4 weights (queries 4 g .. 4 g + 3 of pair column c16) as hi + lo
      v4i16 gh, gl, wh, wl;
      split4(Gs[cb], gh, gl);
      split4(Wt[cb], wh, wl);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        aK[cb][db] = mfma_bf16_k16(gh, bq[db], aK[cb][db]);
        aK[cb][db] = mfma_bf16_k16(gl, bq[db], aK[cb][db]);
        aV[cb][db] = mfma_bf16_k16(wh, bgh[db], aV[cb][db]);
        aV[cb][db] = mfma_bf16_k16(wl, bgh[db], aV[cb][db]);
        aV[cb][db] = mfma_bf16_k16(wh, bgl[db], aV[cb][db]);
      }
    }
    __syncthreads();
    // dQ (16 queries x dims 16 w .. 16 w + 15) = g [keys], four chains
    // bf16 MFMA over pairs in steps of 32 (g as hi + lo, the keys exact),
    // then 16 when NB is odd
    f32x4 dq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) dq[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kBwPairs / 32; ++t) {
      if (32 * t + 32 > 16 * NB) break;  // wave-uniform
      const float* gr = sGs + c16 * kBwGsSt + 32 * t + 8 * g;
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(gr);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(gr + 4);
      const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      bf16x8 ah, al;
      split_hi_lo_pk(x, ah, al);
      u32x4 kw;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        kw[j] = static_cast<uint32_t>(sPk[(32 * t + 8 * g + 2 * j) * kBf16St + 16 * w + c16]) |
                (static_cast<uint32_t>(sPk[(32 * t + 8 * g + 2 * j + 1) * kBf16St + 16 * w + c16]) << 16);
      dq[t & 1] = mfma_bf16(ah, as_bf16x8(kw), dq[t & 1]);
      dq[2 + (t & 1)] = mfma_bf16(al, as_bf16x8(kw), dq[2 + (t & 1)]);
    }
    if (NB & 1) {
      const int p0 = 16 * (NB - 1);
      float x[4];
      v4i16 kq;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = sGs[c16 * kBwGsSt + p0 + 4 * g + j];
        kq[j] = static_cast<short>(sPk[(p0 + 4 * g + j) * kBf16St + 16 * w + c16]);
      }
      v4i16 ah, al;
      split4(x, ah, al);
      dq[0] = mfma_bf16_k16(ah, kq, dq[0]);
      dq[1] = mfma_bf16_k16(al, kq, dq[1]);
    }
    dq[0] += dq[1] + dq[2] + dq[3];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * g + r;
      if (row < nv) dQ[(bh * N + sQid[row]) * kD + 16 * w + c16] = dq[0][r];
    }
  }
  // the item's sums: landmark rows to its partial, raw-key rows to the
  // expert's key sums
  float* pq_ = part + ((bh * items + p) * 2) * static_cast<int64_t>(m) * kD;
  float* pv_ = pq_ + static_cast<int64_t>(m) * kD;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int pb = w + 4 * cb;
    if (pb >= NB) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = 16 * pb + 4 * g + r;
      if (p < m) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          pq_[p * kD + 16 * db + c16] = aK[cb][db][r];
          pv_[p * kD + 16 * db + c16] = aV[cb][db][r];
        }
      } else if (p >= MP && p < MP + k) {
        const int64_t row = (bh * m + ti.e) * k + (p - MP);  // expert e's j-th key
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          unsafeAtomicAdd(dke + row * kD + 16 * db + c16, aK[cb][db][r]);
          unsafeAtomicAdd(dve + row * kD + 16 * db + c16, aV[cb][db][r]);
        }
      }
    }
  }
}

// Block (landmark, head), 16 waves, lane = dim: dVl and the expert step's
// dQl summed over the head's work items (wave w takes items w, w + 16, ...,
// four at a time), and D = dVl . Vl.
__global__ __launch_bounds__(1024) void k_bw_reduce1(const float* __restrict__ part,
                                                     const int32_t* __restrict__ item_start,
                                                     const float* __restrict__ vl, int m,
                                                     int items, float* __restrict__ dql,
                                                     float* __restrict__ dvl,
                                                     float* __restrict__ dd) {
  __shared__ float red[2][16][64];
  const int l = lane_id(), w = wave_id();
  const int64_t bh = blockIdx.y;
  const int i = blockIdx.x;
  const int n = item_start[bh * (m + 1) + m];
  const int64_t stride = static_cast<int64_t>(m) * kD;
  const float* base = part + bh * items * 2 * stride + i * kD + l;
  float sq = 0.f, sv = 0.f;
  int t = w;
  for (; t + 48 < n; t += 64) {
    float a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = base[(t + 16 * u) * 2 * stride];
      b[u] = base[(t + 16 * u) * 2 * stride + stride];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sq += a[u];
      sv += b[u];
    }
  }
  for (; t < n; t += 16) {
    sq += base[t * 2 * stride];
    sv += base[t * 2 * stride + stride];
  }
  red[0][w][l] = sq;
  red[1][w][l] = sv;
  __syncthreads();
  if (w != 0) return;
  sq = 0.f;
  sv = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    sq += red[0][v][l];
    sv += red[1][v][l];
  }
  const int64_t o = (bh * m + i) * kD + l;
  dql[o] = sq;
  dvl[o] = sv;
  float dv = sv * vl[o];
#pragma unroll
  for (int mk = 1; mk < 64; mk <<= 1) dv = xor_sum(dv, mk);
  if (l == 0) dd[bh * m + i] = dv;
}

// ---------------------------------------------------------------------------
// the landmark cross-attention, backward
// ---------------------------------------------------------------------------

// Block (chunk, head), wave w taking 16-key groups w, w + 4, ... of the chunk.
// Per group, keys on rows and landmarks on columns:
//   S^T = K_g Ql^T, dP^T = V_g dVl^T,  A = 2^(c2 S - lse2),  h = s A (dP - D)
//   dQl += h K_g            (A operand = h straight from the accumulators)
//   dK_g += h^T Ql, dV_g += A^T dVl   (h, A through the wave's LDS)
// The group's dK, dV rows are stored (each key belongs to one group); the
// wave's dQl sums go to partial 4 chunk + w.  bf16 inputs: every product on
// bf16 MFMA, V rows (exact) straight from global memory as the dP A
// operand, dVl as bf16 hi + lo in LDS, h and A as hi + lo (cross step at
// 2^20 tokens x 4 heads: 1.28 -> 0.72 ms against fp32 MFMA).
template <class T, int MB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_bw_cross(const typename T::elem* __restrict__ K,
                                                  const typename T::elem* __restrict__ V,
                                                  const typename T::elem* __restrict__ ql,
                                                  const float* __restrict__ dvl,
                                                  const float* __restrict__ lse2,
                                                  const float* __restrict__ dd, int64_t N, int m,
                                                  int csize, float scale,
                                                  float* __restrict__ dK, float* __restrict__ dV,
                                                  float* __restrict__ part2) {
  constexpr int MP = 16 * MB;
  constexpr bool kBf = std::is_same<T, BF16>::value;
  // bf16: Ql and each wave's K rows as bf16 rows (exact; the scores on bf16
  // MFMA, the fp32 operands read from them); fp32: fp32 rows
  __shared__ __attribute__((aligned(16))) float sQl[kBf ? MP * kBf16St / 2 : MP * kBwSt];
  __shared__ __attribute__((aligned(16))) float sdVl[kBf ? 1 : MP * kBwSt];
  // bf16: dVl rows as bf16 hi + lo (MFMA operands)
  __shared__ __attribute__((aligned(16))) uint16_t sdVlh[kBf ? MP * kBf16St : 1];
  __shared__ __attribute__((aligned(16))) uint16_t sdVll[kBf ? MP * kBf16St : 1];
  __shared__ float sLse[MP], sD[MP];
  __shared__ __attribute__((aligned(16))) float sKV[4][2][16 * kBwSt];
  __shared__ __attribute__((aligned(16))) float sK16[kBf ? 4 : 1][kBf ? 16 * kBf16St / 2 : 1];
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int64_t bh = blockIdx.y;
  const int P = static_cast<int>(gridDim.x) * 4;
  for (int u = threadIdx.x; u < MP * 8; u += 256) {
    const int row = u >> 3, j = u & 7;
    Raw8<T> a;
    float b[8];
    if (row < m) {
      a.load(ql + (bh * m + row) * kD + 8 * j);
      load8(dvl + (bh * m + row) * kD + 8 * j, b);
    } else {
      a.zero();
      zero8(b);
    }
    if constexpr (kBf) {
      a.store_raw(reinterpret_cast<uint16_t*>(sQl) + row * kBf16St + 8 * j);
      bf16x8 hi, lo;
      split_hi_lo_pk(b, hi, lo);
      *reinterpret_cast<bf16x8*>(sdVlh + row * kBf16St + 8 * j) = hi;
      *reinterpret_cast<bf16x8*>(sdVll + row * kBf16St + 8 * j) = lo;
    } else {
      a.store(sQl + row * kBwSt + 8 * j);
      store8(sdVl + row * kBwSt + 8 * j, b);
    }
  }
  if (threadIdx.x < MP) {
    const int i = threadIdx.x;
    sLse[i] = i < m ? lse2[bh * m + i] : INFINITY;  // padding landmarks: weight 0
    sD[i] = i < m ? dd[bh * m + i] : 0.f;
  }
  __syncthreads();
  const float c2 = scale * kLog2e;
  const int64_t k0 = static_cast<int64_t>(blockIdx.x) * csize;
  const int64_t k1 = k0 + csize < N ? k0 + csize : N;
  f32x4 aQ[MB][4];
#pragma unroll
  for (int lb = 0; lb < MB; ++lb)
#pragma unroll
    for (int db = 0; db < 4; ++db) aQ[lb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float* sK = sKV[w][0];  // fp32: K rows; then A^T (bf16: A^T only)
  float* sV = sKV[w][1];  // V rows; then h^T
  float* const sKs = kBf ? sK16[kBf ? w : 0] : sK;  // the rows the scores read
  // element (row, col) of K_g and of Ql as fp32
  auto kval = [&](int row, int col) -> float {
    if constexpr (kBf)
      return bf16_to_f32(reinterpret_cast<const uint16_t*>(sKs)[row * kBf16St + col]);
    else
      return sK[row * kBwSt + col];
  };
  auto qlval = [&](int row, int col) -> float {
    if constexpr (kBf)
      return bf16_to_f32(reinterpret_cast<const uint16_t*>(sQl)[row * kBf16St + col]);
    else
      return sQl[row * kBwSt + col];
  };
  Raw8<T> rk[2], rv[2];   // the next group's rows (as in k_bw_lmfwd)
  // bf16: the next group's V rows as the MFMA A operand (lane (c16, g): key
  // c16, features 32 s + 8 g .. + 7), straight from global memory
  u32x4 vq[2];
  auto fetch = [&](int64_t t0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int u = l + 64 * h;
      const int64_t t = t0 + (u >> 3);
      if (t < k1) {
        rk[h].load(K + (bh * N + t) * kD + 8 * (u & 7));
        if constexpr (!kBf) rv[h].load(V + (bh * N + t) * kD + 8 * (u & 7));
      } else {
        rk[h].zero();
        if constexpr (!kBf) rv[h].zero();
      }
    }
    if constexpr (kBf) {
      const int64_t t = t0 + c16;
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int s = 0; s < 2; ++s)
        vq[s] = t < k1 ? *reinterpret_cast<const u32x4*>(
                             reinterpret_cast<const uint16_t*>(V) + (bh * N + t) * kD + 32 * s + 8 * g)
                       : z;
    }
  };
  fetch(k0 + 16 * w);
  for (int64_t t0 = k0 + 16 * w; t0 < k1; t0 += 64) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int u = l + 64 * h;
      if constexpr (kBf) {
        rk[h].store_raw(reinterpret_cast<uint16_t*>(sKs) + (u >> 3) * kBf16St + 8 * (u & 7));
      } else {
        rk[h].store(sK + (u >> 3) * kBwSt + 8 * (u & 7));
        rv[h].store(sV + (u >> 3) * kBwSt + 8 * (u & 7));
      }
    }
    bf16x8 va[2];  // bf16: this group's V rows (exact)
    if constexpr (kBf) {
      va[0] = as_bf16x8(vq[0]);
      va[1] = as_bf16x8(vq[1]);
    }
    fetch(t0 + 64);
    ScoreA<T> ak;
    ak.load(sKs, c16, g);
    float av[16];
    if constexpr (!kBf) {
#pragma unroll
      for (int s = 0; s < 16; ++s) av[s] = sV[c16 * kBwSt + 4 * s + g];
    }
    float A[MB][4], Hh[MB][4];
#pragma unroll
    for (int lb = 0; lb < MB; ++lb) {
      const f32x4 S = ak.score(sQl, 16 * lb + c16, g);
      f32x4 dP = {0.f, 0.f, 0.f, 0.f};
      if constexpr (kBf) {  // V exact, dVl as hi + lo
        f32x4 dPb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int o = (16 * lb + c16) * kBf16St + 32 * s + 8 * g;
          dP = mfma_bf16(va[s], as_bf16x8(*reinterpret_cast<const u32x4*>(sdVlh + o)), dP);
          dPb = mfma_bf16(va[s], as_bf16x8(*reinterpret_cast<const u32x4*>(sdVll + o)), dPb);
        }
        dP += dPb;
      } else {
#pragma unroll
        for (int s = 0; s < 16; ++s)
          dP = mfma_f32(av[s], sdVl[(16 * lb + c16) * kBwSt + 4 * s + g], dP);
      }
      const int i = 16 * lb + c16;
      const float ls = sLse[i], Di = sD[i];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool kv = t0 + 4 * g + r < k1;
        A[lb][r] = kv ? fast_exp2(S[r] * c2 - ls) : 0.f;
        Hh[lb][r] = scale * A[lb][r] * (dP[r] - Di);
      }
    }
    // dQl += h K_g: landmarks on the output rows
    if constexpr (kBf) {  // v_mfma_f32_16x16x16_bf16: A = the lane's own h (hi + lo)
      v4i16 hh[MB], hl[MB];
#pragma unroll
      for (int lb = 0; lb < MB; ++lb) split4(Hh[lb], hh[lb], hl[lb]);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        v4i16 kq;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          kq[r] = static_cast<short>(
              reinterpret_cast<const uint16_t*>(sKs)[(4 * g + r) * kBf16St + 16 * db + c16]);
#pragma unroll
        for (int lb = 0; lb < MB; ++lb) {
          aQ[lb][db] = mfma_bf16_k16(hh[lb], kq, aQ[lb][db]);
          aQ[lb][db] = mfma_bf16_k16(hl[lb], kq, aQ[lb][db]);
        }
      }
    } else {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        float kb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) kb[r] = kval(4 * g + r, 16 * db + c16);
#pragma unroll
        for (int lb = 0; lb < MB; ++lb)
#pragma unroll
          for (int r = 0; r < 4; ++r) aQ[lb][db] = mfma_f32(Hh[lb][r], kb[r], aQ[lb][db]);
      }
    }
    // A and h transposed through the wave's LDS (after its reads of K and V)
#pragma unroll
    for (int lb = 0; lb < MB; ++lb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sK[(4 * g + r) * kBwSt + 16 * lb + c16] = A[lb][r];
        sV[(4 * g + r) * kBwSt + 16 * lb + c16] = Hh[lb][r];
      }
    // bf16: A operands h^T and A^T (key c16, landmarks 32 s + 8 g .. + 7)
    // as hi + lo, once for all four feature blocks; an odd landmark block
    // count ends with a 16-landmark step on v_mfma_f32_16x16x16_bf16
    constexpr int S32 = kBf ? MP / 32 : 1;
    constexpr int S32A = S32 > 0 ? S32 : 1;  // (array extent)
    bf16x8 hth[S32A], htl[S32A], ath[S32A], atl[S32A];
    v4i16 hth4, htl4, ath4, atl4;
    if constexpr (kBf) {
#pragma unroll
      for (int s = 0; s < S32; ++s) {
        float x[8], y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          x[j] = sV[c16 * kBwSt + 32 * s + 8 * g + j];
          y[j] = sK[c16 * kBwSt + 32 * s + 8 * g + j];
        }
        split_hi_lo_pk(x, hth[s], htl[s]);
        split_hi_lo_pk(y, ath[s], atl[s]);
      }
      if constexpr ((MB & 1) != 0) {
        float x[4], y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[j] = sV[c16 * kBwSt + 32 * S32 + 4 * g + j];
          y[j] = sK[c16 * kBwSt + 32 * S32 + 4 * g + j];
        }
        split4(x, hth4, htl4);
        split4(y, ath4, atl4);
      }
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      f32x4 dk = {0.f, 0.f, 0.f, 0.f}, dv = {0.f, 0.f, 0.f, 0.f};
      if constexpr (kBf) {
        const uint16_t* q16 = reinterpret_cast<const uint16_t*>(sQl);
        f32x4 dk2 = {0.f, 0.f, 0.f, 0.f}, dv2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < S32; ++s) {
          u32x4 bq, bh, bl;  // landmarks 32 s + 8 g + j at feature 16 db + c16
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r0 = (32 * s + 8 * g + 2 * j) * kBf16St + 16 * db + c16, r1 = r0 + kBf16St;
            bq[j] = static_cast<uint32_t>(q16[r0]) | (static_cast<uint32_t>(q16[r1]) << 16);
            bh[j] = static_cast<uint32_t>(sdVlh[r0]) | (static_cast<uint32_t>(sdVlh[r1]) << 16);
            bl[j] = static_cast<uint32_t>(sdVll[r0]) | (static_cast<uint32_t>(sdVll[r1]) << 16);
          }
          dk = mfma_bf16(hth[s], as_bf16x8(bq), dk);
          dk2 = mfma_bf16(htl[s], as_bf16x8(bq), dk2);
          dv = mfma_bf16(ath[s], as_bf16x8(bh), dv);
          dv2 = mfma_bf16(atl[s], as_bf16x8(bh), dv2);
          dv = mfma_bf16(ath[s], as_bf16x8(bl), dv);
        }
        if constexpr ((MB & 1) != 0) {
          v4i16 bq4, bh4, bl4;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = (32 * S32 + 4 * g + j) * kBf16St + 16 * db + c16;
            bq4[j] = static_cast<short>(q16[r]);
            bh4[j] = static_cast<short>(sdVlh[r]);
            bl4[j] = static_cast<short>(sdVll[r]);
          }
          dk = mfma_bf16_k16(hth4, bq4, dk);
          dk2 = mfma_bf16_k16(htl4, bq4, dk2);
          dv = mfma_bf16_k16(ath4, bh4, dv);
          dv2 = mfma_bf16_k16(atl4, bh4, dv2);
          dv = mfma_bf16_k16(ath4, bl4, dv);
        }
        dk += dk2;
        dv += dv2;
      } else {
#pragma unroll
        for (int s = 0; s < 4 * MB; ++s) {
          dk = mfma_f32(sV[c16 * kBwSt + 4 * s + g], qlval(4 * s + g, 16 * db + c16), dk);
          dv = mfma_f32(sK[c16 * kBwSt + 4 * s + g], sdVl[(4 * s + g) * kBwSt + 16 * db + c16], dv);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + 4 * g + r;
        if (t < k1) {  // the expert step's sums are added afterwards (k_bw_keyadd)
          dK[(bh * N + t) * kD + 16 * db + c16] = dk[r];
          dV[(bh * N + t) * kD + 16 * db + c16] = dv[r];
        }
      }
    }
  }
  const int64_t pbase = (bh * P + static_cast<int64_t>(blockIdx.x) * 4 + w) * kMaxM;
#pragma unroll
  for (int lb = 0; lb < MB; ++lb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * lb + 4 * g + r;
      if (i < m) {
#pragma unroll
        for (int db = 0; db < 4; ++db) part2[(pbase + i) * kD + 16 * db + c16] = aQ[lb][db][r];
      }
    }
}

// Block (expert, head), wave w taking the expert's keys j = w, w + 4, ...,
// lane = dim: the expert step's sums of each (expert, key) added into dK, dV
// at the key (atomically: a key may belong to several experts).
__global__ __launch_bounds__(256) void k_bw_keyadd(const float* __restrict__ dke,
                                                   const float* __restrict__ dve,
                                                   const int32_t* __restrict__ idx, int64_t N,
                                                   int m, int k, float* __restrict__ dK,
                                                   float* __restrict__ dV) {
  const int64_t bh = blockIdx.y;
  const int e = blockIdx.x;
  const int c = threadIdx.x & 63;
  for (int j = threadIdx.x >> 6; j < k; j += 4) {
    const int64_t row = (bh * m + e) * k + j;
    const int64_t t = clamp64(idx[row], N);
    unsafeAtomicAdd(dK + (bh * N + t) * kD + c, dke[row * kD + c]);
    unsafeAtomicAdd(dV + (bh * N + t) * kD + c, dve[row * kD + c]);
  }
}

// Block (landmark, head): dQl = the expert step's part + the cross partials,
// divided by the window's size.
__global__ __launch_bounds__(256) void k_bw_reduce2(const float* __restrict__ part2, int P,
                                                    const float* __restrict__ dql1, int m, int gh,
                                                    int gw, int mh, int mw,
                                                    float* __restrict__ dqlw) {
  __shared__ float red[4][64];
  const int l = lane_id(), w = wave_id();
  const int64_t bh = blockIdx.y;
  const int i = blockIdx.x;
  float s = 0.f;
  for (int p = w; p < P; p += 4) s += part2[((bh * P + p) * kMaxM + i) * kD + l];
  red[w][l] = s;
  __syncthreads();
  if (w != 0) return;
  s = red[0][l] + red[1][l] + red[2][l] + red[3][l] + dql1[(bh * m + i) * kD + l];
  int64_t r0, r1, c0, c1;
  bin_range(i / mw, gh, mh, r0, r1);
  bin_range(i % mw, gw, mw, c0, c1);
  dqlw[(bh * m + i) * kD + l] = s / static_cast<float>((r1 - r0) * (c1 - c0));
}

// Block (64 tokens, head), four threads per token with 16 dims each.  Grid
// cell r lies in bin a of n bins over g cells iff a g < (r + 1) n and
// r n < (a + 1) g (the bin rule [floor(a g / n), ceil((a + 1) g / n)) with
// the divisions multiplied out); only bins within two of floor(r n / g)
// qualify (n <= g), and that estimate comes from one fp64 division.
__global__ __launch_bounds__(256) void k_bw_poolbw(const float* __restrict__ dqlw, int64_t N,
                                                   int m, int gh, int gw, int mh, int mw,
                                                   float* __restrict__ dQ) {
  const int64_t bh = blockIdx.y;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 64 + (threadIdx.x >> 2);
  const int part = threadIdx.x & 3;
  if (t >= N) return;
  float* p = dQ + (bh * N + t) * kD + 16 * part;
  f32x4 cur[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cur[j] = *reinterpret_cast<const f32x4*>(p + 4 * j);
  const int row = static_cast<int>(t) / gw, col = static_cast<int>(t) - row * gw;
  const int a0 = static_cast<int>(static_cast<double>(row) * mh / gh);
  const int b0 = static_cast<int>(static_cast<double>(col) * mw / gw);
  const int a_lo = a0 - 2 > 0 ? a0 - 2 : 0, a_hi = a0 + 2 < mh - 1 ? a0 + 2 : mh - 1;
  const int b_lo = b0 - 2 > 0 ? b0 - 2 : 0, b_hi = b0 + 2 < mw - 1 ? b0 + 2 : mw - 1;
  for (int a = a_lo; a <= a_hi; ++a) {
    if (!(int64_t{a} * gh < (int64_t{row} + 1) * mh && int64_t{row} * mh < (int64_t{a} + 1) * gh))
      continue;
    for (int b = b_lo; b <= b_hi; ++b) {
      if (!(int64_t{b} * gw < (int64_t{col} + 1) * mw && int64_t{col} * mw < (int64_t{b} + 1) * gw))
        continue;
      const float* src = dqlw + (bh * m + a * mw + b) * kD + 16 * part;
#pragma unroll
      for (int j = 0; j < 4; ++j) cur[j] += *reinterpret_cast<const f32x4*>(src + 4 * j);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    __builtin_nontemporal_store(cur[j], reinterpret_cast<f32x4*>(p + 4 * j));
}

template <class T>
hipError_t launch_backward_t(const Shape& s, const BwPlan& bp, const BwWorkspace& ws,
                             const void* Qv, const void* Kv, const void* Vv, const int32_t* idx,
                             const int32_t* route, const float* dout, float* dQ, float* dK,
                             float* dV, hipStream_t st, int first, int last) {
  using E = typename T::elem;
  const E* Q = static_cast<const E*>(Qv);
  const E* K = static_cast<const E*>(Kv);
  const E* V = static_cast<const E*>(Vv);
  const E* ql = static_cast<const E*>(ws.fw.ql);
  const int BH = static_cast<int>(s.BH);
  const int mb = (s.m + 15) / 16;
  const float c2 = s.scale * kLog2e;
  hipError_t e = hipSuccess;
  auto step = [&](int i) { return e == hipSuccess && i >= first && i <= last; };
  if (step(kBwZero)) {
    const int64_t n4 = s.BH * s.m * s.k * kD / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_bw_zero, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                       reinterpret_cast<f32x4*>(ws.dke), reinterpret_cast<f32x4*>(ws.dve), n4);
    e = hipGetLastError();
  }
  if (step(kBwPool)) e = launch_pool(s, Qv, ws.fw, nullptr, 0, s.BH, st);
  if (step(kBwLandmarkFwd)) {
    const dim3 grid(bp.lm_chunks, BH);
    switch (mb) {
      case 1: hipLaunchKernelGGL((k_bw_lmfwd<T, 1>), grid, dim3(256), 0, st, K, V, ql, s.N, s.m, bp.lm_chunk, c2, ws.lm_stats, ws.lm_acc); break;
      case 2: hipLaunchKernelGGL((k_bw_lmfwd<T, 2>), grid, dim3(256), 0, st, K, V, ql, s.N, s.m, bp.lm_chunk, c2, ws.lm_stats, ws.lm_acc); break;
      case 3: hipLaunchKernelGGL((k_bw_lmfwd<T, 3>), grid, dim3(256), 0, st, K, V, ql, s.N, s.m, bp.lm_chunk, c2, ws.lm_stats, ws.lm_acc); break;
      default: hipLaunchKernelGGL((k_bw_lmfwd<T, 4>), grid, dim3(256), 0, st, K, V, ql, s.N, s.m, bp.lm_chunk, c2, ws.lm_stats, ws.lm_acc); break;
    }
    e = hipGetLastError();
    if (e == hipSuccess) {
      hipLaunchKernelGGL(k_bw_lmmerge, dim3(s.m, BH), dim3(256), 0, st, ws.lm_stats,
                         ws.lm_acc, s.m, bp.lm_chunks, ws.vl, ws.lse2);
      e = hipGetLastError();
    }
  }
  if (step(kBwBucket)) {
    hipLaunchKernelGGL(k_bw_count, dim3(bp.nseg, BH), dim3(256), 0, st, route, s.N, s.m, bp.nseg,
                       ws.counts);
    e = hipGetLastError();
    if (e == hipSuccess) {
      hipLaunchKernelGGL(k_bw_prefix, dim3(s.m, BH), dim3(256), 0, st, ws.counts, s.m, bp.nseg,
                         ws.colpre, ws.totals);
      e = hipGetLastError();
    }
    if (e == hipSuccess) {
      hipLaunchKernelGGL(k_bw_scatter, dim3((bp.nseg + 3) / 4 + 1, BH), dim3(256), 0, st, route,
                         ws.counts, s.m, bp.nseg, s.N, bp.tpb, ws.totals, ws.colpre, ws.offsets,
                         ws.item_start, ws.perm, ws.item_order);
      e = hipGetLastError();
    }
  }
  if (step(kBwAttend)) {
    if constexpr (std::is_same<T, BF16>::value)
      hipLaunchKernelGGL(k_bw_attend_bf16, dim3(bp.items, BH), dim3(256), 0, st, Q, K, V, ql,
                         ws.vl, idx, ws.perm, ws.offsets, ws.item_start, ws.item_order, bp.tpb,
                         s.N, s.m, s.k, s.scale, dout, dQ, ws.dke, ws.dve, ws.part1, bp.items);
    else
      hipLaunchKernelGGL(k_bw_attend<T>, dim3(bp.items, BH), dim3(512), 0, st, Q, K, V, ql,
                         ws.vl, idx, ws.perm, ws.offsets, ws.item_start, ws.item_order, bp.tpb,
                         s.N, s.m, s.k, s.scale, dout, dQ, ws.dke, ws.dve, ws.part1, bp.items);
    e = hipGetLastError();
    if (e == hipSuccess) {
      hipLaunchKernelGGL(k_bw_reduce1, dim3(s.m, BH), dim3(1024), 0, st, ws.part1, ws.item_start,
                         ws.vl, s.m, bp.items, ws.dql1, ws.dvl, ws.dd);
      e = hipGetLastError();
    }
  }
  if (step(kBwCross)) {
    const dim3 grid(bp.cross_chunks, BH);
    switch (mb) {
      case 1: hipLaunchKernelGGL((k_bw_cross<T, 1>), grid, dim3(256), 0, st, K, V, ql, ws.dvl, ws.lse2, ws.dd, s.N, s.m, bp.cross_chunk, s.scale, dK, dV, ws.part2); break;
      case 2: hipLaunchKernelGGL((k_bw_cross<T, 2>), grid, dim3(256), 0, st, K, V, ql, ws.dvl, ws.lse2, ws.dd, s.N, s.m, bp.cross_chunk, s.scale, dK, dV, ws.part2); break;
      case 3:
        if constexpr (std::is_same<T, BF16>::value)  // bf16: the three-block instance spills
          // registers; the four-block one gives the padding landmarks zero weight
          hipLaunchKernelGGL((k_bw_cross<T, 4>), grid, dim3(256), 0, st, K, V, ql, ws.dvl, ws.lse2, ws.dd, s.N, s.m, bp.cross_chunk, s.scale, dK, dV, ws.part2);
        else
          hipLaunchKernelGGL((k_bw_cross<T, 3>), grid, dim3(256), 0, st, K, V, ql, ws.dvl, ws.lse2, ws.dd, s.N, s.m, bp.cross_chunk, s.scale, dK, dV, ws.part2);
        break;
      default: hipLaunchKernelGGL((k_bw_cross<T, 4>), grid, dim3(256), 0, st, K, V, ql, ws.dvl, ws.lse2, ws.dd, s.N, s.m, bp.cross_chunk, s.scale, dK, dV, ws.part2); break;
    }
    e = hipGetLastError();
    if (e == hipSuccess) {
      hipLaunchKernelGGL(k_bw_keyadd, dim3(s.m, BH), dim3(256), 0, st, ws.dke, ws.dve, idx, s.N,
                         s.m, s.k, dK, dV);
      e = hipGetLastError();
    }
  }
  if (step(kBwPoolBw)) {
    hipLaunchKernelGGL(k_bw_reduce2, dim3(s.m, BH), dim3(256), 0, st, ws.part2,
                       4 * bp.cross_chunks, ws.dql1, s.m, s.gh, s.gw, s.mh, s.mw, ws.dqlw);
    e = hipGetLastError();
    if (e == hipSuccess) {
      hipLaunchKernelGGL(k_bw_poolbw, dim3(static_cast<unsigned>((s.N + 63) / 64), BH), dim3(256),
                         0, st, ws.dqlw, s.N, s.m, s.gh, s.gw, s.mh, s.mw, dQ);
      e = hipGetLastError();
    }
  }
  return e;
}

}  // namespace

BwPlan plan_backward(const Shape& s, int cus) {
  BwPlan p;
  // key chunks: about two blocks per CU over all heads, whole 64-key groups
  auto chunk_for = [&](int64_t min_keys) {
    int64_t c = (s.N * s.BH + 2 * cus - 1) / (2 * cus);
    c = (c + 63) / 64 * 64;
    if (c < min_keys) c = min_keys;
    const int64_t whole = (s.N + 63) / 64 * 64;
    if (c > whole) c = whole;
    return c;
  };
  const int64_t lc = chunk_for(256);
  p.lm_chunk = static_cast<int>(lc);
  p.lm_chunks = static_cast<int>((s.N + lc - 1) / lc);
  const int64_t cc = chunk_for(256);
  p.cross_chunk = static_cast<int>(cc);
  p.cross_chunks = static_cast<int>((s.N + cc - 1) / cc);
  p.nseg = static_cast<int>((s.N + kRouteSeg - 1) / kRouteSeg);
  // expert work items of up to tpb 64-query tiles, about two per CU
  const int64_t tiles = (s.N + kAttendTile - 1) / kAttendTile;
  int64_t tpb = (tiles * s.BH) / (2 * static_cast<int64_t>(cus));
  tpb = tpb < 1 ? 1 : (tpb > 16 ? 16 : tpb);
  p.tpb = static_cast<int>(tpb);
  p.items = static_cast<int>((tiles + tpb - 1) / tpb + s.m);
  return p;
}

size_t plan_bw_workspace(const Shape& s, const BwPlan& bp, BwWorkspace* ws, char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += (bytes + 255) / 256 * 256;
    return p;
  };
  const size_t BH = static_cast<size_t>(s.BH), es = s.dtype == MITA_BF16 ? 2 : 4;
  const size_t m = static_cast<size_t>(s.m);
  *ws = BwWorkspace{};
  ws->fw.pool_part = reinterpret_cast<double*>(take(BH * m * s.pool_splits * kD * sizeof(double)));
  ws->fw.ql = take(BH * m * kD * es);
  const size_t p1 = BH * bp.lm_chunks * kMaxM;
  ws->lm_stats = reinterpret_cast<float*>(take(p1 * 2 * sizeof(float)));
  ws->lm_acc = reinterpret_cast<float*>(take(p1 * kD * sizeof(float)));
  ws->vl = reinterpret_cast<float*>(take(BH * m * kD * sizeof(float)));
  ws->lse2 = reinterpret_cast<float*>(take(BH * m * sizeof(float)));
  ws->counts = reinterpret_cast<int32_t*>(take(BH * m * bp.nseg * 4));
  ws->colpre = reinterpret_cast<int32_t*>(take(BH * m * bp.nseg * 4));
  ws->totals = reinterpret_cast<int32_t*>(take(BH * m * 4));
  ws->offsets = reinterpret_cast<int32_t*>(take(BH * (m + 1) * 4));
  ws->item_start = reinterpret_cast<int32_t*>(take(BH * (m + 1) * 4));
  ws->item_order = reinterpret_cast<int32_t*>(take(BH * (2 * m + 1) * 4));
  ws->perm = reinterpret_cast<int32_t*>(take(BH * s.N * 4));
  ws->part1 = reinterpret_cast<float*>(take(BH * bp.items * 2 * m * kD * sizeof(float)));
  ws->dql1 = reinterpret_cast<float*>(take(BH * m * kD * sizeof(float)));
  ws->dvl = reinterpret_cast<float*>(take(BH * m * kD * sizeof(float)));
  ws->dd = reinterpret_cast<float*>(take(BH * m * sizeof(float)));
  ws->part2 = reinterpret_cast<float*>(take(BH * 4 * bp.cross_chunks * kMaxM * kD * sizeof(float)));
  ws->dqlw = reinterpret_cast<float*>(take(BH * m * kD * sizeof(float)));
  ws->dke = reinterpret_cast<float*>(take(BH * m * s.k * kD * sizeof(float)));
  ws->dve = reinterpret_cast<float*>(take(BH * m * s.k * kD * sizeof(float)));
  return off;
}

hipError_t launch_backward(const Shape& s, const BwPlan& bp, const BwWorkspace& ws,
                           const void* Q, const void* K, const void* V, const int32_t* idx,
                           const int32_t* route, const float* dout, float* dQ, float* dK,
                           float* dV, hipStream_t st, int first, int last) {
  return s.dtype == MITA_BF16
             ? launch_backward_t<BF16>(s, bp, ws, Q, K, V, idx, route, dout, dQ, dK, dV, st,
                                       first, last)
             : launch_backward_t<F32>(s, bp, ws, Q, K, V, idx, route, dout, dQ, dK, dV, st, first,
                                      last);
}

}  // namespace mita
