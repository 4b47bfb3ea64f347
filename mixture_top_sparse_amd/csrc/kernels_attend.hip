// kernels_attend.hip — step 5: each query attends over the concatenation of
// the m compressed pairs (keys Ql, values Vl) and its expert's k raw pairs
// (K[t], V[t] for t in the expert), with one softmax over all m + k logits
// ("NeurIPS'26：注意力也是FFN？…", section "用少量地标查询，同时构造全局概括与
// 细节专家"; "Mixture-of-Top-k 注意力…", section "MiTA：用少量地标查询，同时
// 完成压缩与专家构造"; "And attention is also FFN? …", Figure 3 and
// Algorithm 1 — the algorithm combines the two parts by online softmax, which
// equals the single softmax computed here).
//
// k_attend: one block per (expert tile of <= 64 queries, head).  The block
// stages the expert once in LDS — the m compressed keys and the k gathered
// raw key rows for the logits, and the values transposed for P.V — and all
// 64 queries reuse it.  Queries are gathered in expert order (perm) straight
// into MFMA operand registers; output rows are scattered back.
//   logits^T = [Ql; K_e] Q_tile^T   (pair rows x query columns, MFMA)
//   out^T    = [Vl; V_e]^T P^T       (MFMA; P and Vl as bf16 hi + lo parts)
// Every per-query quantity (max, sum, rescale) stays in the 4 lanes that hold
// that query's column.
//
// Roofline: HBM-bound per query: d*e bytes of Q gathered (one full row) and
// 4d bytes of fp32 output written; the staged expert (~40 KiB) comes from L2.
#include "mita_device.hpp"
#include "mita_internal.hpp"

namespace mita {

template <class T, int MPAD, int KPAD>
struct AttendLds;

template <int MPAD, int KPAD>
struct AttendLds<BF16, MPAD, KPAD> {
  static constexpr int PKST = 72;        // pair-key rows (elements)
  static constexpr int VCST = MPAD + 4;  // compressed Vl^T rows
  static constexpr int VRST = KPAD + 4;  // raw V^T rows
  uint16_t pk[(MPAD + KPAD) * PKST];
  uint16_t vch[kD * VCST];
  uint16_t vcl[kD * VCST];
  uint16_t vr[kD * VRST];
};

template <int MPAD, int KPAD>
struct AttendLds<F32, MPAD, KPAD> {
  static constexpr int PKST = 68;
  static constexpr int VST = 68;
  float pk[(MPAD + KPAD) * PKST];
  float val[(MPAD + KPAD) * VST];
};

struct TileInfo {
  int e;      // expert
  int qb;     // first perm slot of this work item
  int qe;     // one past its last perm slot
};

// Work item t of a head covers up to `tpb` consecutive 64-query tiles of one
// expert; item_start[e] is the first item of expert e (exclusive scan of
// ceil(tiles_e / tpb)).
__device__ __forceinline__ bool find_item(const int32_t* __restrict__ item_start,
                                          const int32_t* __restrict__ offsets, int m, int tpb,
                                          int t, TileInfo& ti) {
  if (t >= item_start[m]) return false;
  int e = 0;
  while (e < m - 1 && item_start[e + 1] <= t) ++e;
  const int j0 = (t - item_start[e]) * tpb;
  ti.e = e;
  ti.qb = offsets[e] + kAttendTile * j0;
  ti.qe = min(ti.qb + kAttendTile * tpb, static_cast<int>(offsets[e + 1]));
  return true;
}

__device__ __forceinline__ int64_t clamp_index(int64_t v, int64_t n) {
  return v < 0 ? 0 : (v >= n ? n - 1 : v);
}

// ---- bf16 ----------------------------------------------------------------

template <int MPAD, int KPAD>
__device__ void stage_bf16(AttendLds<BF16, MPAD, KPAD>& S, const uint16_t* __restrict__ K,
                           const uint16_t* __restrict__ V, const uint16_t* __restrict__ Ql,
                           const uint16_t* __restrict__ vlt_hi, const uint16_t* __restrict__ vlt_lo,
                           const int32_t* __restrict__ ex, int64_t N, int m, int k, int64_t bh) {
  using L = AttendLds<BF16, MPAD, KPAD>;
  constexpr int NP = MPAD + KPAD;
  const int tid = threadIdx.x;
  const u32x4 z = {0, 0, 0, 0};
  // pair keys: Ql rows then the expert's K rows (zero rows for padding)
  for (int c = tid; c < NP * 8; c += 256) {
    const int row = c >> 3, col = c & 7;
    u32x4 v = z;
    if (row < MPAD) {
      if (row < m) v = *reinterpret_cast<const u32x4*>(Ql + (bh * m + row) * kD + col * 8);
    } else if (row - MPAD < k) {
      const int64_t t = clamp_index(ex[row - MPAD], N);
      v = *reinterpret_cast<const u32x4*>(K + (bh * N + t) * kD + col * 8);
    }
    *reinterpret_cast<u32x4*>(S.pk + row * L::PKST + col * 8) = v;
  }
  // compressed values, already transposed and split (rows d, columns pairs)
  for (int c = tid; c < kD * (MPAD / 8); c += 256) {
    const int d = c / (MPAD / 8), col = c % (MPAD / 8);
    *reinterpret_cast<u32x4*>(S.vch + d * L::VCST + col * 8) =
        *reinterpret_cast<const u32x4*>(vlt_hi + (bh * kD + d) * MPAD + col * 8);
    *reinterpret_cast<u32x4*>(S.vcl + d * L::VCST + col * 8) =
        *reinterpret_cast<const u32x4*>(vlt_lo + (bh * kD + d) * MPAD + col * 8);
  }
  // raw values transposed: V^T[d][pair], two gathered rows per thread
  for (int c = tid; c < (KPAD / 2) * 8; c += 256) {
    const int rp = c >> 3, col = c & 7;
    u32x4 a = z, b = z;
    if (2 * rp < k)
      a = *reinterpret_cast<const u32x4*>(V + (bh * N + clamp_index(ex[2 * rp], N)) * kD + col * 8);
    if (2 * rp + 1 < k)
      b = *reinterpret_cast<const u32x4*>(V + (bh * N + clamp_index(ex[2 * rp + 1], N)) * kD +
                                          col * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t wa = a[i >> 1], wb = b[i >> 1];
      const uint32_t word =
          (i & 1) ? ((wa >> 16) | (wb & 0xFFFF0000u)) : ((wa & 0xFFFFu) | (wb << 16));
      *reinterpret_cast<uint32_t*>(S.vr + (col * 8 + i) * L::VRST + 2 * rp) = word;
    }
  }
}

// 16 queries of one wave (lane column c16 = query) against the staged expert
template <int MPAD, int KPAD>
__device__ __forceinline__ void attend_queries_bf16(const AttendLds<BF16, MPAD, KPAD>& S,
                                                    const bf16x8 (&qb)[2], bool qok, int64_t q,
                                                    int m, int k, float c2,
                                                    float* __restrict__ out_h) {
  using L = AttendLds<BF16, MPAD, KPAD>;
  constexpr int NPB = (MPAD + KPAD) / 16;
  const int l = lane_id(), g = l >> 4, c16 = l & 15;
  float x[NPB][4];
  float mx = -INFINITY;
#pragma unroll
  for (int pb = 0; pb < NPB; ++pb) {
    f32x4 a = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 kk = as_bf16x8(
          *reinterpret_cast<const u32x4*>(S.pk + (16 * pb + c16) * L::PKST + 32 * s + 8 * g));
      a = mfma_bf16(kk, qb[s], a);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = 16 * pb + 4 * g + r;
      const bool valid = (p < MPAD) ? (p < m) : (p - MPAD < k);
      x[pb][r] = valid ? a[r] : -INFINITY;
      mx = fmaxf(mx, x[pb][r]);
    }
  }
  mx = xor_max(mx, 16);
  mx = xor_max(mx, 32) * c2;
  float lsum = 0.f;
#pragma unroll
  for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[pb][r] = fast_exp2(fmaf(x[pb][r], c2, -mx));
      lsum += x[pb][r];
    }
  lsum = xor_sum(lsum, 16);
  lsum = xor_sum(lsum, 32);

  f32x4 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x4{0, 0, 0, 0};
  // compressed pairs: Vl (hi + lo) x P (hi + lo), dropping lo x lo
#pragma unroll
  for (int s2 = 0; s2 < MPAD / 32; ++s2) {
    float pp[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pp[r] = x[2 * s2][r];
      pp[4 + r] = x[2 * s2 + 1][r];
    }
    bf16x8 ph, pl;
    split_hi_lo(pp, ph, pl);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const uint16_t* rh = S.vch + (16 * dt + c16) * L::VCST + 32 * s2 + 4 * g;
      const uint16_t* rl = S.vcl + (16 * dt + c16) * L::VCST + 32 * s2 + 4 * g;
      const bf16x8 ah = join_bf16x8(*reinterpret_cast<const u32x2*>(rh),
                                    *reinterpret_cast<const u32x2*>(rh + 16));
      const bf16x8 al = join_bf16x8(*reinterpret_cast<const u32x2*>(rl),
                                    *reinterpret_cast<const u32x2*>(rl + 16));
      acc[dt] = mfma_bf16(ah, ph, acc[dt]);
      acc[dt] = mfma_bf16(ah, pl, acc[dt]);
      acc[dt] = mfma_bf16(al, ph, acc[dt]);
    }
  }
  // raw pairs: V (exact bf16) x P (hi + lo)
#pragma unroll
  for (int s2 = 0; s2 < KPAD / 32; ++s2) {
    float pp[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pp[r] = x[MPAD / 16 + 2 * s2][r];
      pp[4 + r] = x[MPAD / 16 + 2 * s2 + 1][r];
    }
    bf16x8 ph, pl;
    split_hi_lo(pp, ph, pl);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const uint16_t* rv = S.vr + (16 * dt + c16) * L::VRST + 32 * s2 + 4 * g;
      const bf16x8 a = join_bf16x8(*reinterpret_cast<const u32x2*>(rv),
                                   *reinterpret_cast<const u32x2*>(rv + 16));
      acc[dt] = mfma_bf16(a, ph, acc[dt]);
      acc[dt] = mfma_bf16(a, pl, acc[dt]);
    }
  }
  if (qok) {
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      *reinterpret_cast<f32x4*>(out_h + q * kD + 16 * dt + 4 * g) = acc[dt] * inv;
  }
}

template <int MPAD, int KPAD>
__device__ void attend_bf16(AttendLds<BF16, MPAD, KPAD>& S, const uint16_t* __restrict__ Q,
                            const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                            const uint16_t* __restrict__ Ql, const uint16_t* __restrict__ vlt_hi,
                            const uint16_t* __restrict__ vlt_lo, const int32_t* __restrict__ idx,
                            const int32_t* __restrict__ perm, int64_t N, int m, int k, float c2,
                            float* __restrict__ out, int64_t bh, const TileInfo& ti) {
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const uint16_t* Qh = Q + bh * N * kD;
  const int32_t* ph = perm + bh * N;
  float* out_h = out + bh * N * kD;
  const u32x4 z = {0, 0, 0, 0};

  // wave w handles the 16-query sub-tiles w, w+4, w+8, ... of the item;
  // the query index runs two sub-tiles ahead and the Q rows one ahead
  auto qpos = [&](int i) { return ti.qb + 16 * (w + 4 * i) + c16; };
  auto load_perm = [&](int i) -> int64_t {
    const int pos = qpos(i);
    return (pos < ti.qe && pos >= 0 && pos < N) ? clamp_index(ph[pos], N) : -1;
  };
  auto load_q = [&](int64_t q, bf16x8 (&qb)[2]) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
      qb[s] = as_bf16x8(q >= 0 ? *reinterpret_cast<const u32x4*>(Qh + q * kD + 32 * s + 8 * g) : z);
  };
  const int nsub = (ti.qe - ti.qb + 15) / 16;  // sub-tiles in this item
  int64_t q_cur = load_perm(0);
  int64_t q_nxt = load_perm(1);
  bf16x8 qb[2];
  load_q(q_cur, qb);

  stage_bf16<MPAD, KPAD>(S, K, V, Ql, vlt_hi, vlt_lo, idx + (bh * m + ti.e) * k, N, m, k, bh);
  __syncthreads();

  for (int i = 0; w + 4 * i < nsub; ++i) {
    bf16x8 qn[2];
    load_q(q_nxt, qn);  // next sub-tile's rows (q = -1 loads nothing)
    const int64_t q_nn = load_perm(i + 2);
    attend_queries_bf16<MPAD, KPAD>(S, qb, q_cur >= 0, q_cur, m, k, c2, out_h);
    q_cur = q_nxt;
    q_nxt = q_nn;
    qb[0] = qn[0];
    qb[1] = qn[1];
  }
}

// ---- fp32 ----------------------------------------------------------------

template <int MPAD, int KPAD>
__device__ void attend_f32(AttendLds<F32, MPAD, KPAD>& S, const float* __restrict__ Q,
                           const float* __restrict__ K, const float* __restrict__ V,
                           const float* __restrict__ Ql, const float* __restrict__ vl,
                           const int32_t* __restrict__ idx, const int32_t* __restrict__ perm,
                           int64_t N, int m, int k, float c2, float* __restrict__ out, int64_t bh,
                           const TileInfo& ti) {
  using L = AttendLds<F32, MPAD, KPAD>;
  constexpr int NP = MPAD + KPAD;
  constexpr int NPB = NP / 16;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int32_t* ex = idx + (bh * m + ti.e) * k;
  const f32x4 z = {0, 0, 0, 0};
  for (int c = tid; c < NP * 16; c += 256) {
    const int row = c >> 4, col = c & 15;
    f32x4 kv = z, vv = z;
    if (row < MPAD) {
      if (row < m) {
        kv = *reinterpret_cast<const f32x4*>(Ql + (bh * m + row) * kD + col * 4);
        vv = *reinterpret_cast<const f32x4*>(vl + (bh * m + row) * kD + col * 4);
      }
    } else if (row - MPAD < k) {
      const int64_t t = clamp_index(ex[row - MPAD], N);
      kv = *reinterpret_cast<const f32x4*>(K + (bh * N + t) * kD + col * 4);
      vv = *reinterpret_cast<const f32x4*>(V + (bh * N + t) * kD + col * 4);
    }
    *reinterpret_cast<f32x4*>(S.pk + row * L::PKST + col * 4) = kv;
    *reinterpret_cast<f32x4*>(S.val + row * L::VST + col * 4) = vv;
  }
  __syncthreads();

  const int nsub = (ti.qe - ti.qb + 15) / 16;
  for (int i = 0; w + 4 * i < nsub; ++i) {
    const int pos = ti.qb + 16 * (w + 4 * i) + c16;
    const bool qok = pos < ti.qe && pos >= 0 && pos < N;
    const int64_t q = qok ? clamp_index(perm[bh * N + pos], N) : 0;
    float qv[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) qv[s] = qok ? Q[(bh * N + q) * kD + 4 * s + g] : 0.f;
    float x[NPB][4];
    float mx = -INFINITY;
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
      f32x4 a = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 16; ++s)
        a = mfma_f32(S.pk[(16 * pb + c16) * L::PKST + 4 * s + g], qv[s], a);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = 16 * pb + 4 * g + r;
        const bool valid = (p < MPAD) ? (p < m) : (p - MPAD < k);
        x[pb][r] = valid ? a[r] * c2 : -INFINITY;
        mx = fmaxf(mx, x[pb][r]);
      }
    }
    mx = xor_max(mx, 16);
    mx = xor_max(mx, 32);
    float lsum = 0.f;
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[pb][r] = fast_exp2(x[pb][r] - mx);
        lsum += x[pb][r];
      }
    lsum = xor_sum(lsum, 16);
    lsum = xor_sum(lsum, 32);
    f32x4 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          acc[dt] =
              mfma_f32(S.val[(16 * pb + 4 * g + r) * L::VST + 16 * dt + c16], x[pb][r], acc[dt]);
    if (qok) {
      const float inv = 1.0f / lsum;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        *reinterpret_cast<f32x4*>(out + (bh * N + q) * kD + 16 * dt + 4 * g) = acc[dt] * inv;
    }
  }
}

// grid (work items, BH), 256 threads
template <class T, int MPAD, int KPAD>
__global__ __launch_bounds__(256) void k_attend(
    const typename T::elem* __restrict__ Q, const typename T::elem* __restrict__ K,
    const typename T::elem* __restrict__ V, const typename T::elem* __restrict__ Ql,
    const float* __restrict__ vl, const uint16_t* __restrict__ vlt_hi,
    const uint16_t* __restrict__ vlt_lo, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ item_start, int tpb, int64_t N, int m, int k, float c2,
    float* __restrict__ out) {
  __shared__ AttendLds<T, MPAD, KPAD> S;
  const int64_t bh = blockIdx.y;
  TileInfo ti;
  if (!find_item(item_start + bh * (m + 1), offsets + bh * (m + 1), m, tpb, blockIdx.x, ti))
    return;
  if constexpr (sizeof(typename T::elem) == 2)
    attend_bf16<MPAD, KPAD>(S, Q, K, V, Ql, vlt_hi, vlt_lo, idx, perm, N, m, k, c2, out, bh, ti);
  else
    attend_f32<MPAD, KPAD>(S, Q, K, V, Ql, vl, idx, perm, N, m, k, c2, out, bh, ti);
}

template <class T, int MPAD, int KPAD>
static hipError_t launch_attend_t(const Shape& s, const void* Q, const void* K, const void* V,
                                  const int32_t* idx, const Workspace& ws, float* out,
                                  hipStream_t st) {
  using E = typename T::elem;
  hipLaunchKernelGGL((k_attend<T, MPAD, KPAD>), dim3(s.attend_items, s.BH), dim3(256), 0, st,
                     static_cast<const E*>(Q), static_cast<const E*>(K), static_cast<const E*>(V),
                     static_cast<const E*>(ws.ql), ws.vl, ws.vlt_hi, ws.vlt_lo, idx, ws.perm,
                     ws.offsets, ws.item_start, s.attend_tpb, s.N, s.m, s.k, s.scale * kLog2e,
                     out);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_attend_d(const Shape& s, const void* Q, const void* K, const void* V,
                                  const int32_t* idx, const Workspace& ws, float* out,
                                  hipStream_t st) {
  if (s.mpad == 32 && s.kpad == 32) return launch_attend_t<T, 32, 32>(s, Q, K, V, idx, ws, out, st);
  if (s.mpad == 32) return launch_attend_t<T, 32, 64>(s, Q, K, V, idx, ws, out, st);
  if (s.kpad == 32) return launch_attend_t<T, 64, 32>(s, Q, K, V, idx, ws, out, st);
  return launch_attend_t<T, 64, 64>(s, Q, K, V, idx, ws, out, st);
}

hipError_t launch_attend(const Shape& s, const void* Q, const void* K, const void* V,
                         const int32_t* idx, const Workspace& ws, float* out, hipStream_t st) {
  return s.dtype == 1 ? launch_attend_d<BF16>(s, Q, K, V, idx, ws, out, st)
                      : launch_attend_d<F32>(s, Q, K, V, idx, ws, out, st);
}

}  // namespace mita
