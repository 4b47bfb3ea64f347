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
//   out^T    = [Vl; V_e]^T P^T       (bf16 MFMA; P and Vl as hi + lo pairs)
// Every per-query quantity (max, sum, rescale) stays in the 4 lanes that hold
// that query's column.
//
// Roofline: HBM-bound per query: d*e bytes of Q gathered (one full row) and
// 4d bytes of fp32 output written; the staged expert (~40 KiB) comes from L2.
#include "mita_bucket.hpp"
#include "mita_device.hpp"
#include "mita_internal.hpp"

namespace mita {

constexpr int kAttendWaves = 8;       // bf16 expert attention: waves per block

template <class T, int MPAD, int KPAD, int NW = kAttendWaves>
struct AttendLds;

// NW: waves per block (each stages its own output rows)
template <int MPAD, int KPAD, int NW>
struct AttendLds<BF16, MPAD, KPAD, NW> {
  static constexpr int PKST = 72;        // pair-key rows (bf16 elements)
  static constexpr int VCST = MPAD + 4;  // compressed Vl^T rows (bf16)
  static constexpr int VRST = KPAD + 4;  // raw V^T rows (bf16)
  alignas(16) uint16_t pk[(MPAD + KPAD) * PKST];
  alignas(16) uint16_t vch[kD * VCST];  // Vl^T, bf16 hi part
  alignas(16) uint16_t vcl[kD * VCST];  // Vl^T, bf16 lo part (Vl - hi, rounded)
  alignas(16) uint16_t vr[kD * VRST];   // V^T of the expert's rows (exact bf16)
  // 2-wave blocks (short items) keep each lane's query index in registers
  // and store output rows straight from them: without the index copy and the
  // output stage they need far less LDS, so several fit a CU and their
  // latency-bound items overlap more
  static constexpr bool kStageOut = NW > 2;
  alignas(16) int32_t perm[kStageOut ? kAttendTile * kAttendMaxTpb : 4];  // item's queries
  // per wave: 16 output rows of 64 floats, 16-byte chunks XOR-swizzled by row
  alignas(16) float ostage[kStageOut ? NW : 1][kStageOut ? 16 * kD : 4];
};

template <int MPAD, int KPAD, int NW>
struct AttendLds<F32, MPAD, KPAD, NW> {
  static constexpr int PKST = 68;
  static constexpr int VST = 68;
  alignas(16) float pk[(MPAD + KPAD) * PKST];
  alignas(16) float val[(MPAD + KPAD) * VST];
};

__device__ __forceinline__ int64_t clamp_index(int64_t v, int64_t n) {
  return v < 0 ? 0 : (v >= n ? n - 1 : v);
}

// ---- bf16 ----------------------------------------------------------------
//
// Logits run on bf16 MFMA (Q, Ql and K are exact bf16).  P.V runs on bf16
// MFMA too, with the computed operands split into hi + lo bf16 pairs
// (hi = rne(x), lo = rne(x - hi): about 16 significant bits): the softmax
// weights P always, the landmark values Vl for the compressed pairs.  Raw
// values are exact bf16.  Per 32 pairs: raw  acc += V^T P_hi + V^T P_lo;
// compressed  acc += Vl_hi^T P_hi + Vl_hi^T P_lo + Vl_lo^T P_hi (the
// dropped Vl_lo P_lo term is below 2^-16 of the product).  Each operand
// carries relative error <= 2^-16 (two roundings at unit 2^-8), so an output
// differs from the exact combination of its weights by at most about
// 3 * 2^-16 * max|value| plus fp32 accumulation, whatever the values' range.

// Stage the expert of this work item.  Every global load is issued before
// any LDS write (the expert's key indices first, then the rows they name,
// the landmark values and the landmark queries), so the item pays one
// index-then-row latency instead of one per operand.
template <int MPAD, int KPAD, int NW>
__device__ void stage_bf16(AttendLds<BF16, MPAD, KPAD, NW>& S, const uint16_t* __restrict__ K,
                          const uint16_t* __restrict__ V, const uint16_t* __restrict__ Ql,
                          const float* __restrict__ vl, const int32_t* __restrict__ ex, int64_t N,
                          int m, int k, int64_t bh) {
  using L = AttendLds<BF16, MPAD, KPAD, NW>;
  constexpr int NP = MPAD + KPAD;
  constexpr int NT = 64 * NW;
  const int tid = threadIdx.x;
  const u32x4 z = {0, 0, 0, 0};
  // raw values: unit u = rows 2rp, 2rp+1 of the expert, 8 features from
  // 8*col, stored transposed as bf16 pairs (row 2rp low, 2rp+1 high)
  constexpr int RU = (KPAD / 2) * 8, RPT = (RU + NT - 1) / NT;
  // landmark values: unit u = rows 2lp, 2lp+1, 8 features from 8*dc, split
  // into bf16 hi + lo and stored transposed
  constexpr int LP = MPAD / 2;
  constexpr int LU = LP * 8, LPT = (LU + NT - 1) / NT;
  // pair keys: Ql rows then the expert's K rows (zero rows for padding)
  constexpr int PU = NP * 8, PPT = (PU + NT - 1) / NT;

  int64_t rra[RPT], rrb[RPT];  // raw rows of each raw unit (-1: none)
  int64_t prow[PPT];           // source row of each pair-key chunk (-1: zero)
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int u = tid + NT * j, rp = u >> 3;
    rra[j] = (u < RU && 2 * rp < k) ? clamp_index(ex[2 * rp], N) : -1;
    rrb[j] = (u < RU && 2 * rp + 1 < k) ? clamp_index(ex[2 * rp + 1], N) : -1;
  }
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int c = tid + NT * j, row = c >> 3;
    prow[j] = (c >= PU || row >= NP) ? -1
              : row < MPAD           ? (row < m ? row : -1)
              : (row - MPAD < k ? clamp_index(ex[row - MPAD], N) : -1);
  }
  u32x4 va[RPT], vb[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int col = (tid + NT * j) & 7;
    va[j] = rra[j] >= 0 ? *reinterpret_cast<const u32x4*>(V + (bh * N + rra[j]) * kD + col * 8) : z;
    vb[j] = rrb[j] >= 0 ? *reinterpret_cast<const u32x4*>(V + (bh * N + rrb[j]) * kD + col * 8) : z;
  }
  f32x4 lv[LPT][2][2];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int u = tid + NT * j, lp = u % LP, dc = u / LP;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 2 * lp + h;
      const bool ok = u < LU && row < m;
#pragma unroll
      for (int q = 0; q < 2; ++q)
        lv[j][h][q] = ok ? *reinterpret_cast<const f32x4*>(vl + (bh * m + row) * kD + dc * 8 + 4 * q)
                         : f32x4{0, 0, 0, 0};
    }
  }
  u32x4 pv[PPT];
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int c = tid + NT * j, row = c >> 3, cc = c & 7;
    pv[j] = prow[j] < 0 ? z
            : row < MPAD ? *reinterpret_cast<const u32x4*>(Ql + (bh * m + prow[j]) * kD + cc * 8)
                         : *reinterpret_cast<const u32x4*>(K + (bh * N + prow[j]) * kD + cc * 8);
  }
  // LDS writes
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int u = tid + NT * j;
    if (u < RU) {
      const int rp = u >> 3, col = u & 7;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t a = (i & 1) ? (va[j][i >> 1] >> 16) : (va[j][i >> 1] & 0xFFFFu);
        const uint32_t b = (i & 1) ? (vb[j][i >> 1] >> 16) : (vb[j][i >> 1] & 0xFFFFu);
        *reinterpret_cast<uint32_t*>(S.vr + (col * 8 + i) * L::VRST + 2 * rp) = a | (b << 16);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int u = tid + NT * j;
    if (u < LU) {
      const int lp = u % LP, dc = u / LP;
      float la[8], lb[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        la[i] = lv[j][0][0][i];
        la[4 + i] = lv[j][0][1][i];
        lb[i] = lv[j][1][0][i];
        lb[4 + i] = lv[j][1][1][i];
      }
      bf16x8 ah, al, bh8, bl8;
      split_hi_lo_pk(la, ah, al);
      split_hi_lo_pk(lb, bh8, bl8);
      // the halves are taken from the raw bits (element i of a bf16x8 is
      // the low (even i) or high (odd i) half of dword i/2)
      const u32x4 wah = __builtin_bit_cast(u32x4, ah), wal = __builtin_bit_cast(u32x4, al);
      const u32x4 wbh = __builtin_bit_cast(u32x4, bh8), wbl = __builtin_bit_cast(u32x4, bl8);
      auto half = [](const u32x4& v, int i) {
        return (i & 1) ? (v[i >> 1] >> 16) : (v[i >> 1] & 0xFFFFu);
      };
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        *reinterpret_cast<uint32_t*>(S.vch + (dc * 8 + i) * L::VCST + 2 * lp) =
            half(wah, i) | (half(wbh, i) << 16);
        *reinterpret_cast<uint32_t*>(S.vcl + (dc * 8 + i) * L::VCST + 2 * lp) =
            half(wal, i) | (half(wbl, i) << 16);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int c = tid + NT * j;
    if (c < PU) {
      const int row = c >> 3, cc = c & 7;
      *reinterpret_cast<u32x4*>(S.pk + row * L::PKST + cc * 8) = pv[j];
    }
  }
}

// 16 queries of one wave (lane column c16 = query) against the staged expert
// `after_scores` runs once the logits have been formed (the Q operand is then
// free, so the caller can refill it while the rest of the sub-tile runs).
// qcol: the query row of this lane's column (used when rows are stored
// straight from registers).
template <int MPAD, int KPAD, int NW, bool FULL, class AfterScores>
__device__ __forceinline__ void attend_queries_bf16(AttendLds<BF16, MPAD, KPAD, NW>& S,
                                                    bf16x8 (&qb)[2], int sl0, int nq, int m,
                                                    int k, float c2, float* __restrict__ out_h,
                                                    int64_t qcol,
                                                    AfterScores&& after_scores) {
  using L = AttendLds<BF16, MPAD, KPAD, NW>;
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
      if constexpr (FULL) {
        x[pb][r] = a[r];
      } else {
        const int p = 16 * pb + 4 * g + r;
        const bool valid = (p < MPAD) ? (p < m) : (p - MPAD < k);
        x[pb][r] = valid ? a[r] : -INFINITY;
      }
      mx = fmaxf(mx, x[pb][r]);
    }
  }
  after_scores(qb);
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
  // 32 pairs per step: pair blocks 2*s2 and 2*s2+1 give this lane's 8 P
  // values, split into bf16 hi + lo
  auto p_split = [&](int pb0, bf16x8& hi, bf16x8& lo) {
    const float p[8] = {x[pb0][0],     x[pb0][1],     x[pb0][2],     x[pb0][3],
                        x[pb0 + 1][0], x[pb0 + 1][1], x[pb0 + 1][2], x[pb0 + 1][3]};
    split_hi_lo_pk(p, hi, lo);
  };
  auto vt = [&](const uint16_t* row) {
    return join_bf16x8(*reinterpret_cast<const u32x2*>(row),
                       *reinterpret_cast<const u32x2*>(row + 16));
  };
#pragma unroll
  for (int s2 = 0; s2 < MPAD / 32; ++s2) {
    bf16x8 ph, pl;
    p_split(2 * s2, ph, pl);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int off = (16 * dt + c16) * L::VCST + 32 * s2 + 4 * g;
      const bf16x8 vh = vt(S.vch + off), vlo = vt(S.vcl + off);
      acc[dt] = mfma_bf16(vlo, ph, acc[dt]);
      acc[dt] = mfma_bf16(vh, pl, acc[dt]);
      acc[dt] = mfma_bf16(vh, ph, acc[dt]);
    }
  }
#pragma unroll
  for (int s2 = 0; s2 < KPAD / 32; ++s2) {
    bf16x8 ph, pl;
    p_split(MPAD / 16 + 2 * s2, ph, pl);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const bf16x8 vv = vt(S.vr + (16 * dt + c16) * L::VRST + 32 * s2 + 4 * g);
      acc[dt] = mfma_bf16(vv, pl, acc[dt]);
      acc[dt] = mfma_bf16(vv, ph, acc[dt]);
    }
  }
  const float f = __builtin_amdgcn_rcpf(lsum);  // lsum >= 1
  if constexpr (!L::kStageOut) {
    // straight from registers: lane (query c16, g) holds features
    // 16dt + 4g .. +3, so the 4 lanes of a query store 64 contiguous bytes
    // per instruction.  Slots past the item repeat its last query (same
    // operands, identical bits).
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      *reinterpret_cast<f32x4*>(out_h + qcol * kD + 16 * dt + 4 * g) = acc[dt] * f;
    return;
  }
  // Output rows go through this wave's LDS stage: lane (query c16, g) holds
  // features 16dt + 4g .. +3 (16-byte chunk 4dt + g of row c16); read back,
  // 16 lanes cover one 256-byte row, so each store instruction writes four
  // complete rows.  Chunks are XOR-swizzled by row (no bank conflicts either
  // way).
  float* st = S.ostage[wave_id()];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    *reinterpret_cast<f32x4*>(st + c16 * kD + (((4 * dt + g) ^ c16) & 15) * 4) = acc[dt] * f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 4 * j + (l >> 4);
    // slots past the item repeat its last query: those lanes computed that
    // query's row from the same operands, so they store identical bits
    const int sl = min(sl0 + row, nq - 1);
    const f32x4 v = *reinterpret_cast<const f32x4*>(st + row * kD + (((l & 15) ^ row) & 15) * 4);
    const int64_t q = S.perm[sl];
    // non-temporal: the rows are not read again here, and written-through
    // lines do not leave dirty cache lines for the next kernel to flush
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(out_h + q * kD + 4 * (l & 15)));
  }
}

template <int MPAD, int KPAD, bool FULL, int NW>
__device__ void attend_bf16(AttendLds<BF16, MPAD, KPAD, NW>& S, const uint16_t* __restrict__ Q,
                            const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                            const uint16_t* __restrict__ Ql, const float* __restrict__ vl,
                            const int32_t* __restrict__ idx, const int32_t* __restrict__ perm,
                            int64_t N, int m, int k, float c2, float* __restrict__ out, int64_t bh,
                            const TileInfo& ti) {
  constexpr int D = 4;  // Q gathers in flight per wave (sub-tiles ahead)
  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const uint16_t* Qh = Q + bh * N * kD;
  const int32_t* ph = perm + bh * N;
  float* out_h = out + bh * N * kD;
  const int nq = ti.qe - ti.qb;  // queries in this item, 1 .. 64 * tpb
  if (nq <= 0) return;           // (items are never empty; uniform per block)
  const int nsub = (nq + 15) / 16;  // 16-query sub-tiles
  // wave w handles sub-tiles w, w+W, w+2W, ...; every slot index is clamped
  // to the item's last query, so each Q gather reads a valid row and needs no
  // branch (the wait counters then stay exact across the ring)
  constexpr int W = NW;
  auto slot = [&](int i) { return min(16 * (w + W * i) + c16, nq - 1); };
  auto load_q = [&](int64_t q, bf16x8 (&qb)[2]) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
      qb[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(Qh + q * kD + 32 * s + 8 * g));
  };
  // the first D sub-tiles' rows are requested before staging (perm from global)
  using L = AttendLds<BF16, MPAD, KPAD, NW>;
  int64_t pq[D];  // each ring slot's query row (this lane's column)
#pragma unroll
  for (int j = 0; j < D; ++j) pq[j] = clamp_index(ph[ti.qb + slot(j)], N);
  bf16x8 ring[D][2];
#pragma unroll
  for (int j = 0; j < D; ++j) load_q(pq[j], ring[j]);
  if constexpr (L::kStageOut)
    for (int c = tid; c < nq; c += 64 * NW)
      S.perm[c] = static_cast<int32_t>(clamp_index(ph[ti.qb + c], N));
  stage_bf16<MPAD, KPAD, NW>(S, K, V, Ql, vl, idx + (bh * m + ti.e) * k, N, m, k, bh);
  __syncthreads();

  const int nw = nsub > w ? (nsub - w + W - 1) / W : 0;  // this wave's sub-tiles
  if (nw >= D) {
    // whole ring rounds: the last round's extra sub-tiles repeat the item's
    // last query (same values stored again); refills past the end re-read it
    const int rounds = (nw + D - 1) / D;
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        const int i = r * D + j;
        // re-read the staged operands from LDS for every sub-tile instead of
        // pinning all of them in registers across the loop, and keep the
        // scheduler from interleaving sub-tiles (both keep occupancy)
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        attend_queries_bf16<MPAD, KPAD, NW, FULL>(
            S, ring[j], 16 * (w + W * i), nq, m, k, c2, out_h, pq[j],
            [&](bf16x8(&qb)[2]) {  // sub-tile i + D into this slot
              if constexpr (L::kStageOut) {
                load_q(S.perm[slot(i + D)], qb);
              } else {
                pq[j] = clamp_index(ph[ti.qb + slot(i + D)], N);
                load_q(pq[j], qb);
              }
            });
      }
    }
  } else {
    // fewer sub-tiles than ring slots: all were requested before staging
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (j < nw)
        attend_queries_bf16<MPAD, KPAD, NW, FULL>(S, ring[j], 16 * (w + W * j), nq, m, k, c2,
                                                  out_h, pq[j], [](bf16x8(&)[2]) {});
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

// grid (work items, BH).  bf16: 64 * NW threads.  NW = 8 for items of many
// sub-tiles: register budget for 4 waves per SIMD (LDS allows 2 blocks per
// CU).  NW = 2 for short items (a few queries per expert), whose smaller
// blocks fit several to a CU: budget for 2 waves per SIMD (LDS allows no
// more at m, k > 32; staging holds twice the values per thread).  fp32
// (small problems): 256 threads, default budget.
template <int MPAD, int KPAD, bool FULL, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW == 8 ? 4 : 2))) void k_attend_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ Ql, const float* __restrict__ vl, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ item_start, const int32_t* __restrict__ item_order, int tpb,
    int64_t N, int m, int k, float c2, float* __restrict__ out) {
  __shared__ AttendLds<BF16, MPAD, KPAD, NW> S;
  int64_t bh;
  TileInfo ti;
  int p;
  if (!dispatch_item(item_start, item_order, offsets, m, tpb, bh, p, ti)) return;
  attend_bf16<MPAD, KPAD, FULL, NW>(S, Q, K, V, Ql, vl, idx, perm, N, m, k, c2, out, bh, ti);
}

// ---- short items: several work items per block ---------------------------
//
// When experts hold few queries (the image-shaped workloads: 20-35 per
// expert), a block that stages one expert spends most of its life waiting on
// a chain of dependent loads: the work-item table, the expert's key list,
// the key and value rows it names.  Here each 2-wave block takes up to ipb
// work items of one head (consecutive ones, or, with at most 64 items per
// head, those that write_item_blocks assigned it by size): the compressed
// pairs (Ql rows, Vl as hi + lo) are staged once, the items' key lists are
// read once, and while the block computes one item the next item's key and
// value rows and its first query rows are already loading into registers
// (their positions in the bucket order were read one item earlier still).

template <int MPAD, int KPAD, int NT>
struct RawRows {  // one item's raw pairs in flight, NT threads
  static constexpr int RU = (KPAD / 2) * 8, RPT = (RU + NT - 1) / NT;  // value-row units
  static constexpr int KU = KPAD * 8, KPT = (KU + NT - 1) / NT;        // key-row chunks
  u32x4 va[RPT], vb[RPT], kv[KPT];
};

template <int MPAD, int KPAD, int NT>
__device__ __forceinline__ void raw_load(RawRows<MPAD, KPAD, NT>& R, const int32_t* ex,
                                         const uint16_t* __restrict__ K,
                                         const uint16_t* __restrict__ V, int64_t N, int k,
                                         int64_t bh) {
  using RR = RawRows<MPAD, KPAD, NT>;
  const int tid = threadIdx.x;
  const u32x4 z = {0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < RR::RPT; ++j) {
    const int u = tid + NT * j, rp = u >> 3, col = u & 7;
    const bool ok = u < RR::RU;
    R.va[j] = (ok && 2 * rp < k)
                  ? *reinterpret_cast<const u32x4*>(V + (bh * N + clamp_index(ex[2 * rp], N)) * kD + col * 8)
                  : z;
    R.vb[j] = (ok && 2 * rp + 1 < k)
                  ? *reinterpret_cast<const u32x4*>(V + (bh * N + clamp_index(ex[2 * rp + 1], N)) * kD + col * 8)
                  : z;
  }
#pragma unroll
  for (int j = 0; j < RR::KPT; ++j) {
    const int c = tid + NT * j, row = c >> 3, cc = c & 7;
    R.kv[j] = (c < RR::KU && row < k)
                  ? *reinterpret_cast<const u32x4*>(K + (bh * N + clamp_index(ex[row], N)) * kD + cc * 8)
                  : z;
  }
}

template <int MPAD, int KPAD, int NW>
__device__ __forceinline__ void raw_store(AttendLds<BF16, MPAD, KPAD, NW>& S,
                                          const RawRows<MPAD, KPAD, 64 * NW>& R) {
  constexpr int NT = 64 * NW;
  using L = AttendLds<BF16, MPAD, KPAD, NW>;
  using RR = RawRows<MPAD, KPAD, NT>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < RR::RPT; ++j) {
    const int u = tid + NT * j;
    if (u < RR::RU) {
      const int rp = u >> 3, col = u & 7;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t a = (i & 1) ? (R.va[j][i >> 1] >> 16) : (R.va[j][i >> 1] & 0xFFFFu);
        const uint32_t b = (i & 1) ? (R.vb[j][i >> 1] >> 16) : (R.vb[j][i >> 1] & 0xFFFFu);
        *reinterpret_cast<uint32_t*>(S.vr + (col * 8 + i) * L::VRST + 2 * rp) = a | (b << 16);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < RR::KPT; ++j) {
    const int c = tid + NT * j;
    if (c < RR::KU)
      *reinterpret_cast<u32x4*>(S.pk + (MPAD + (c >> 3)) * L::PKST + (c & 7) * 8) = R.kv[j];
  }
}

// the compressed pairs of head bh: Ql rows (pair-key rows 0 .. MPAD-1) and
// Vl^T as bf16 hi + lo, every load issued before any LDS write
template <int MPAD, int KPAD, int NW>
__device__ __forceinline__ void stage_compressed(AttendLds<BF16, MPAD, KPAD, NW>& S,
                                                 const uint16_t* __restrict__ Ql,
                                                 const float* __restrict__ vl, int m, int64_t bh) {
  constexpr int NT = 64 * NW;
  using L = AttendLds<BF16, MPAD, KPAD, NW>;
  constexpr int LP = MPAD / 2, LU = LP * 8, LPT = (LU + NT - 1) / NT;
  constexpr int QU = MPAD * 8, QPT = (QU + NT - 1) / NT;
  const int tid = threadIdx.x;
  const u32x4 z = {0, 0, 0, 0};
  f32x4 lv[LPT][2][2];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int u = tid + NT * j, lp = u % LP, dc = u / LP;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 2 * lp + h;
      const bool ok = u < LU && row < m;
#pragma unroll
      for (int q = 0; q < 2; ++q)
        lv[j][h][q] = ok ? *reinterpret_cast<const f32x4*>(vl + (bh * m + row) * kD + dc * 8 + 4 * q)
                         : f32x4{0, 0, 0, 0};
    }
  }
  u32x4 qv[QPT];
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int c = tid + NT * j, row = c >> 3;
    qv[j] = (c < QU && row < m) ? *reinterpret_cast<const u32x4*>(Ql + (bh * m + row) * kD + (c & 7) * 8) : z;
  }
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int u = tid + NT * j;
    if (u < LU) {
      const int lp = u % LP, dc = u / LP;
      float la[8], lb[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        la[i] = lv[j][0][0][i];
        la[4 + i] = lv[j][0][1][i];
        lb[i] = lv[j][1][0][i];
        lb[4 + i] = lv[j][1][1][i];
      }
      bf16x8 ah, al, bh8, bl8;
      split_hi_lo_pk(la, ah, al);
      split_hi_lo_pk(lb, bh8, bl8);
      const u32x4 wah = __builtin_bit_cast(u32x4, ah), wal = __builtin_bit_cast(u32x4, al);
      const u32x4 wbh = __builtin_bit_cast(u32x4, bh8), wbl = __builtin_bit_cast(u32x4, bl8);
      auto half = [](const u32x4& v, int i) {
        return (i & 1) ? (v[i >> 1] >> 16) : (v[i >> 1] & 0xFFFFu);
      };
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        *reinterpret_cast<uint32_t*>(S.vch + (dc * 8 + i) * L::VCST + 2 * lp) =
            half(wah, i) | (half(wbh, i) << 16);
        *reinterpret_cast<uint32_t*>(S.vcl + (dc * 8 + i) * L::VCST + 2 * lp) =
            half(wal, i) | (half(wbl, i) << 16);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int c = tid + NT * j;
    if (c < QU) *reinterpret_cast<u32x4*>(S.pk + (c >> 3) * L::PKST + (c & 7) * 8) = qv[j];
  }
}

// grid (ceil(items / kAttendIpb), BH), 128 threads
template <int MPAD, int KPAD, bool FULL>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void k_attend_items_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ Ql, const float* __restrict__ vl, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ item_start, const int32_t* __restrict__ item_blocks, int tpb,
    int64_t N, int m, int k, float c2, float* __restrict__ out, int ipb) {
  constexpr int NW = 2, D = 2;  // waves; query rows in flight per wave (sub-tiles)
  using L = AttendLds<BF16, MPAD, KPAD, NW>;
  __shared__ L S;
  __shared__ int32_t sex[kAttendIpbMax][KPAD];  // the items' key lists (clamped)
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int t0 = static_cast<int>(blockIdx.x) * ipb;
  const int32_t* IS = item_start + bh * (m + 1);
  const int32_t* OF = offsets + bh * (m + 1);
  // work items t0 .. t0 + nit - 1 (item t: expert e = the number of experts
  // e' < m - 1 whose successor starts at or before t; item_start is
  // non-decreasing); lane j keeps item j's expert and query range
  // the block's items: ipb consecutive ones, or its slots of item_blocks
  // (items assigned to blocks by size, empty slots last)
  int tl = 0, nit = 0;
  if (item_blocks != nullptr) {
    tl = l < ipb ? item_blocks[(bh * gridDim.x + blockIdx.x) * ipb + l] : -1;
    nit = __popcll(ballot(tl >= 0));
  } else {
    tl = t0 + l;
    nit = min(ipb, IS[m] - t0);
  }
  if (nit <= 0) return;  // whole block
  const int nextst = l < m - 1 ? IS[l + 1] : INT32_MAX;
  const int ist = l < m ? IS[l] : 0;
  const int ofl = l <= m && l < 64 ? OF[l] : 0;
  const int ofm = OF[m];
  int my_e = 0, my_qb = 0, my_qe = 0;
#pragma unroll
  for (int j = 0; j < kAttendIpbMax; ++j) {
    const int t = __builtin_amdgcn_readlane(tl, j);
    const int e = __popcll(ballot(nextst <= t));  // wave-uniform
    const int qb = __builtin_amdgcn_readlane(ofl, e) +
                   kAttendTile * tpb * (t - __builtin_amdgcn_readlane(ist, e));
    const int oe = e + 1 < 64 ? __builtin_amdgcn_readlane(ofl, e + 1) : ofm;  // offsets[e + 1]
    if (l == j) {
      my_e = e;
      my_qb = qb;
      my_qe = min(qb + kAttendTile * tpb, oe);
    }
  }
  // key lists of the block's items, then the compressed pairs
  for (int c = tid; c < kAttendIpbMax * KPAD; c += 128) {
    const int j = c / KPAD, r = c % KPAD;
    const int e = static_cast<int>(lane_read(static_cast<uint32_t>(my_e), j));
    sex[j][r] = (j < nit && r < k) ? static_cast<int32_t>(clamp_index(idx[(bh * m + e) * k + r], N)) : 0;
  }
  stage_compressed<MPAD, KPAD, NW>(S, Ql, vl, m, bh);
  __syncthreads();

  const uint16_t* Qh = Q + bh * N * kD;
  const int32_t* ph = perm + bh * N;
  float* out_h = out + bh * N * kD;
  auto load_q = [&](int64_t q, bf16x8 (&qb)[2]) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
      qb[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(Qh + q * kD + 32 * s + 8 * g));
  };
  // this wave's sub-tiles of item j: w, w + NW, ...; slots clamped to the
  // item's last query (every gather reads a valid row, so the ring needs no
  // branch and its waits stay exact)
  auto slot = [&](int nq, int i) { return min(16 * (w + NW * i) + c16, nq - 1); };
  RawRows<MPAD, KPAD, 64 * NW> R;
  // pq: this item's ring rows; pqn: the next item's first rows (read one
  // item ahead); pqnn: the item after that
  int64_t pq[D], pqn[D], pqnn[D];
  bf16x8 ring[D][2], ringn[D][2];
  auto first_rows = [&](int j, int64_t (&dst)[D]) {
    const int qbj = __builtin_amdgcn_readlane(my_qb, j);
    const int nqj = __builtin_amdgcn_readlane(my_qe, j) - qbj;
#pragma unroll
    for (int d = 0; d < D; ++d) dst[d] = clamp_index(ph[qbj + slot(nqj, d)], N);
  };
  {  // item 0: raw rows and first query rows; item 1's row positions
    first_rows(0, pq);
#pragma unroll
    for (int d = 0; d < D; ++d) load_q(pq[d], ring[d]);
    if (nit > 1) first_rows(1, pqn);
    raw_load<MPAD, KPAD, 64 * NW>(R, sex[0], K, V, N, k, bh);
    raw_store<MPAD, KPAD, NW>(S, R);
  }
  __syncthreads();
  for (int j = 0; j < nit; ++j) {  // nit is block-uniform
    const int qb = __builtin_amdgcn_readlane(my_qb, j), nq = __builtin_amdgcn_readlane(my_qe, j) - qb;
    const bool has_next = j + 1 < nit;
    if (has_next) {  // the next item's rows start loading now
#pragma unroll
      for (int d = 0; d < D; ++d) load_q(pqn[d], ringn[d]);
      raw_load<MPAD, KPAD, 64 * NW>(R, sex[j + 1], K, V, N, k, bh);
      if (j + 2 < nit) first_rows(j + 2, pqnn);
    }
    const int nsub = (nq + 15) / 16;
    const int nw = nsub > w ? (nsub - w + NW - 1) / NW : 0;  // this wave's sub-tiles
    if (nw >= D) {
      // whole ring rounds: the last round's extra slots repeat the item's
      // last query (same values stored again); refills past the end re-read it
      const int rounds = (nw + D - 1) / D;
      for (int r = 0; r < rounds; ++r) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const int i = r * D + d;
          __asm__ volatile("" ::: "memory");
          __builtin_amdgcn_sched_barrier(0);
          attend_queries_bf16<MPAD, KPAD, NW, FULL>(
              S, ring[d], 16 * (w + NW * i), nq, m, k, c2, out_h, pq[d],
              [&](bf16x8(&q)[2]) {
                pq[d] = clamp_index(ph[qb + slot(nq, i + D)], N);
                load_q(pq[d], q);
              });
        }
      }
    } else {
      // fewer sub-tiles than ring slots: all of them are in the ring already
#pragma unroll
      for (int d = 0; d < D; ++d)
        if (d < nw)
          attend_queries_bf16<MPAD, KPAD, NW, FULL>(S, ring[d], 16 * (w + NW * d), nq, m, k, c2,
                                                    out_h, pq[d], [](bf16x8(&)[2]) {});
    }
    __syncthreads();  // every wave is done with item j's raw pairs
    if (has_next) {
      raw_store<MPAD, KPAD, NW>(S, R);
#pragma unroll
      for (int d = 0; d < D; ++d) {
        pq[d] = pqn[d];
        pqn[d] = pqnn[d];
        ring[d][0] = ringn[d][0];
        ring[d][1] = ringn[d][1];
      }
      __syncthreads();
    }
  }
}

template <int MPAD, int KPAD, bool FULL>
__global__ __launch_bounds__(256) void k_attend_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ Ql, const float* __restrict__ vl, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ item_start, const int32_t* __restrict__ item_order, int tpb,
    int64_t N, int m, int k, float c2, float* __restrict__ out) {
  __shared__ AttendLds<F32, MPAD, KPAD> S;
  int64_t bh;
  TileInfo ti;
  int p;
  if (!dispatch_item(item_start, item_order, offsets, m, tpb, bh, p, ti)) return;
  attend_f32<MPAD, KPAD>(S, Q, K, V, Ql, vl, idx, perm, N, m, k, c2, out, bh, ti);
}

// ---- several experts per query (s > 1, bf16) -------------------------------
//
// The work items run over the N*s (query, expert) assignments grouped by
// expert (perm holds assignment indices a = q*s + j, j = the rank of the
// expert among the query's s).  Each assignment gets one softmax partial
// over its expert's k raw pairs, and over the m compressed pairs too when
// j = 0 (the query's best expert), so that every query sees the compressed
// pairs once and each of its experts' raw pairs once: m + s*k pairs in all,
// a key shared by two of its experts counted once per expert — the
// oracle's reading, which the Algorithm 1 caption of "And attention is also
// FFN? …" gives (each expert's query subset attended separately, the parts
// combined by online softmax).  Partials: the unnormalised P.V row, the
// maximum logit (times log2 e * scale) and the weight sum; k_combine_s
// merges a query's s partials.
template <int MPAD, int KPAD>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void k_attend_multi(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ Ql, const float* __restrict__ vl,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ item_start, int tpb,
    int64_t N, int s, int m, int k, float c2, float* __restrict__ pacc,
    float* __restrict__ pstat) {
  constexpr int NW = 2;
  using L = AttendLds<BF16, MPAD, KPAD, NW>;
  __shared__ L S;
  const int64_t bh = blockIdx.y;
  const int64_t NA = N * s;
  TileInfo ti;
  if (!find_item(item_start + bh * (m + 1), offsets + bh * (m + 1), m, tpb, blockIdx.x, ti))
    return;
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int nq = ti.qe - ti.qb;
  if (nq <= 0) return;
  stage_bf16<MPAD, KPAD, NW>(S, K, V, Ql, vl, idx + (bh * m + ti.e) * k, N, m, k, bh);
  __syncthreads();
  const uint16_t* Qh = Q + bh * N * kD;
  constexpr int NPB = (MPAD + KPAD) / 16;
  const int nsub = (nq + 15) / 16;
  for (int sub = w; sub < nsub; sub += NW) {
    const int slot = min(16 * sub + c16, nq - 1);  // slots past the item repeat its last
    const int64_t a = perm[bh * NA + ti.qb + slot];
    const int64_t q = a / s;
    const bool with_compressed = (a % s) == 0;
    bf16x8 qb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
      qb[t] = as_bf16x8(*reinterpret_cast<const u32x4*>(Qh + q * kD + 32 * t + 8 * g));
    float x[NPB][4];
    float mx = -INFINITY;
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 kk = as_bf16x8(
            *reinterpret_cast<const u32x4*>(S.pk + (16 * pb + c16) * L::PKST + 32 * t + 8 * g));
        acc = mfma_bf16(kk, qb[t], acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = 16 * pb + 4 * g + r;
        const bool valid = (p < MPAD) ? (p < m && with_compressed) : (p - MPAD < k);
        x[pb][r] = valid ? acc[r] : -INFINITY;
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
    f32x4 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x4{0, 0, 0, 0};
    auto p_split = [&](int pb0, bf16x8& hi, bf16x8& lo) {
      const float p8[8] = {x[pb0][0],     x[pb0][1],     x[pb0][2],     x[pb0][3],
                           x[pb0 + 1][0], x[pb0 + 1][1], x[pb0 + 1][2], x[pb0 + 1][3]};
      split_hi_lo_pk(p8, hi, lo);
    };
    auto vt = [&](const uint16_t* row) {
      return join_bf16x8(*reinterpret_cast<const u32x2*>(row),
                         *reinterpret_cast<const u32x2*>(row + 16));
    };
#pragma unroll
    for (int s2 = 0; s2 < MPAD / 32; ++s2) {
      bf16x8 ph, pl;
      p_split(2 * s2, ph, pl);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int off = (16 * dt + c16) * L::VCST + 32 * s2 + 4 * g;
        const bf16x8 vh = vt(S.vch + off), vlo = vt(S.vcl + off);
        o[dt] = mfma_bf16(vlo, ph, o[dt]);
        o[dt] = mfma_bf16(vh, pl, o[dt]);
        o[dt] = mfma_bf16(vh, ph, o[dt]);
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < KPAD / 32; ++s2) {
      bf16x8 ph, pl;
      p_split(MPAD / 16 + 2 * s2, ph, pl);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x8 vv = vt(S.vr + (16 * dt + c16) * L::VRST + 32 * s2 + 4 * g);
        o[dt] = mfma_bf16(vv, pl, o[dt]);
        o[dt] = mfma_bf16(vv, ph, o[dt]);
      }
    }
    if (16 * sub + c16 < nq) {  // the assignment's partial (unnormalised)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        *reinterpret_cast<f32x4*>(pacc + (bh * NA + a) * kD + 16 * dt + 4 * g) = o[dt];
      if (g == 0) {
        pstat[(bh * NA + a) * 2] = mx;
        pstat[(bh * NA + a) * 2 + 1] = lsum;
      }
    }
  }
}

// Merge each query's s partials: with M the largest partial maximum,
// out = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j.  Grid (ceil(N/16),
// BH), 256 threads: 16 lanes per query, four features each.
__global__ __launch_bounds__(256) void k_combine_s(const float* __restrict__ pacc,
                                                  const float* __restrict__ pstat, int64_t N,
                                                  int s, float* __restrict__ out) {
  const int64_t bh = blockIdx.y;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int f = (threadIdx.x & 15) * 4;
  if (q >= N) return;
  const int64_t NA = N * s;
  float M = -INFINITY;
  for (int j = 0; j < s; ++j) M = fmaxf(M, pstat[(bh * NA + q * s + j) * 2]);
  float z = 0.f;
  f32x4 acc = {0, 0, 0, 0};
  for (int j = 0; j < s; ++j) {
    const int64_t a = bh * NA + q * s + j;
    const float wj = fast_exp2(pstat[a * 2] - M);
    z += wj * pstat[a * 2 + 1];
    acc += wj * *reinterpret_cast<const f32x4*>(pacc + a * kD + f);
  }
  *reinterpret_cast<f32x4*>(out + (bh * N + q) * kD + f) = acc * (1.0f / z);
}

template <int MPAD, int KPAD>
static hipError_t launch_attend_multi_t(const Shape& s, const void* Q, const void* K,
                                        const void* V, const int32_t* idx, const Workspace& ws,
                                        float* out, hipStream_t st) {
  auto kern = k_attend_multi<MPAD, KPAD>;
  hipLaunchKernelGGL(kern, dim3(s.attend_items, s.BH), dim3(128), 0, st,
                     static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                     static_cast<const uint16_t*>(V), static_cast<const uint16_t*>(ws.ql), ws.vl,
                     idx, ws.perm, ws.offsets, ws.item_start, s.attend_tpb, s.N, s.s, s.m, s.k,
                     s.scale * kLog2e, ws.pacc, ws.pstat);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_combine_s, dim3((s.N + 15) / 16, s.BH), dim3(256), 0, st, ws.pacc,
                     ws.pstat, s.N, s.s, out);
  return hipGetLastError();
}

hipError_t launch_attend_multi(const Shape& s, const void* Q, const void* K, const void* V,
                               const int32_t* idx, const Workspace& ws, float* out,
                               hipStream_t st) {
  if (s.dtype != 1) return hipErrorInvalidValue;
  if (s.mpad == 32 && s.kpad == 32) return launch_attend_multi_t<32, 32>(s, Q, K, V, idx, ws, out, st);
  if (s.mpad == 32) return launch_attend_multi_t<32, 64>(s, Q, K, V, idx, ws, out, st);
  if (s.kpad == 32) return launch_attend_multi_t<64, 32>(s, Q, K, V, idx, ws, out, st);
  return launch_attend_multi_t<64, 64>(s, Q, K, V, idx, ws, out, st);
}

template <class T, int MPAD, int KPAD, bool FULL, int NW>
struct AttendKernel;
template <int MPAD, int KPAD, bool FULL, int NW>
struct AttendKernel<BF16, MPAD, KPAD, FULL, NW> {
  static constexpr auto fn = k_attend_bf16<MPAD, KPAD, FULL, NW>;
  static constexpr int threads = 64 * NW;
};
template <int MPAD, int KPAD, bool FULL, int NW>
struct AttendKernel<F32, MPAD, KPAD, FULL, NW> {
  static constexpr auto fn = k_attend_f32<MPAD, KPAD, FULL>;
  static constexpr int threads = 256;
};

template <class T, int MPAD, int KPAD, int NW>
static hipError_t launch_attend_w(const Shape& s, const void* Q, const void* K, const void* V,
                                  const int32_t* idx, const Workspace& ws, float* out,
                                  hipStream_t st) {
  if constexpr (std::is_same<T, BF16>::value && NW == 2) {
    auto kern = (s.m == MPAD && s.k == KPAD) ? k_attend_items_bf16<MPAD, KPAD, true>
                                             : k_attend_items_bf16<MPAD, KPAD, false>;
    // ipb items per block and nbx blocks per head, chosen when the call is
    // planned so that every block of the launch is resident at once (about
    // three 2-wave blocks per CU): no second round of blocks runs on a
    // half-empty GPU
    hipLaunchKernelGGL(kern, dim3(s.attend_nbx, s.BH), dim3(128), 0, st,
                       static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                       static_cast<const uint16_t*>(V), static_cast<const uint16_t*>(ws.ql),
                       ws.vl, idx, ws.perm, ws.offsets, ws.item_start, ws.item_blocks,
                       s.attend_tpb, s.N, s.m, s.k, s.scale * kLog2e, out, s.attend_ipb);
    return hipGetLastError();
  }
  using E = typename T::elem;
  auto kern = (s.m == MPAD && s.k == KPAD) ? AttendKernel<T, MPAD, KPAD, true, NW>::fn
                                           : AttendKernel<T, MPAD, KPAD, false, NW>::fn;
  hipLaunchKernelGGL(kern, dim3(s.attend_items, s.BH),
                     dim3(AttendKernel<T, MPAD, KPAD, true, NW>::threads), 0, st,
                     static_cast<const E*>(Q), static_cast<const E*>(K), static_cast<const E*>(V),
                     static_cast<const E*>(ws.ql), ws.vl, idx, ws.perm, ws.offsets, ws.item_start,
                     ws.item_order, s.attend_tpb, s.N, s.m, s.k, s.scale * kLog2e, out);
  return hipGetLastError();
}

// short work items (few queries per expert on average) take 2-wave blocks
template <class T, int MPAD, int KPAD>
static hipError_t launch_attend_t(const Shape& s, const void* Q, const void* K, const void* V,
                                  const int32_t* idx, const Workspace& ws, float* out,
                                  hipStream_t st) {
  if (std::is_same<T, BF16>::value && s.N < kAttendShortItems * static_cast<int64_t>(s.m))
    return launch_attend_w<T, MPAD, KPAD, 2>(s, Q, K, V, idx, ws, out, st);
  return launch_attend_w<T, MPAD, KPAD, kAttendWaves>(s, Q, K, V, idx, ws, out, st);
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
