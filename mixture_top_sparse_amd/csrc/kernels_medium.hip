// kernels_medium.hip — steps 2 to 4 of the MiTA forward pass in one launch
// for mid-length bf16 sequences (256 < N <= 1600 tokens per head): the
// segmentation-shaped workloads of the pages (32x32 and 40x40 token grids
// with m = k = 49: "Mixture-of-Top-k 注意力…", section "语义分割：在更长的视觉
// 序列上减少计算"), where the multi-launch path's pre-threshold, split scan
// and merge cost more than the work they organise.
//
// Two kinds of blocks (512 threads) share the launch; both need only the
// landmark queries Ql that the pooling launch before it wrote:
//
//   select blocks   (head, 32 landmarks): waves (lt, kq) = 2 landmark tiles
//                   of 16 x 4 key quarters.  Wave (lt, kq) takes the 16-key
//                   slice 16 kq .. 16 kq + 15 of every 64-key tile.
//     pass    one sweep over K and V: S^T = K Ql^T on bf16 MFMA (K rows
//             loaded straight into the operand registers); every score of
//             the wave stays in registers as its 32-bit order bits (a larger
//             key = a larger score); V_l = softmax(scale S) V by an online
//             softmax per wave, P as bf16 hi + lo against V rows staged
//             through LDS and read with the LDS transpose read
//             (v_mfma_f32_16x16x16_bf16, whose B operand is the scores' own
//             accumulator layout).  The four quarters' partial sums meet in
//             LDS at the end.
//     select  expert i = the k best keys, ties at the k-th score to the lower
//             keys (the reading the oracle follows).  theta = the k-th
//             largest 8-key group maximum is a lower bound of the k-th
//             score; the keys at or above it (about k to 2k) are collected
//             in LDS, and a bisection over their 32-bit order bits gives the
//             k-th score T.  The keys above T and the lowest-index ties
//             form the expert, written in ascending key order through a bit
//             mask.  A landmark with more than kMedCap candidates (heavy
//             ties) sends its block to an exact bisection over all keys
//             instead (counts summed over the key quarters through LDS).
//             Each wave searches for four landmarks at once, one 16-lane row
//             each.
//   route blocks    (one per head, after the select blocks): routing of all
//                   N queries (R^T = Ql Q^T on MFMA, argmax with ties to the
//                   lower landmark), then the stable counting sort by expert
//                   in LDS: perm, offsets and the attention's work items.
//
// ("Mixture-of-Top-k 注意力…", section "MiTA：用少量地标查询，同时完成压缩与
// 专家构造"; "NeurIPS'26：注意力也是FFN？…", section "用少量地标查询，同时构造
// 全局概括与细节专家".)  The scores are the same MFMA products as the
// multi-launch scan's (same operand layout), so the experts are the same.
//
// Roofline: per head, K and V are read once from HBM (the two select blocks
// of a head are dispatched to one XCD and share them through its L2) and Q
// once; idx, V_l, routes and the bucket order are written once.  At these
// sizes the launch is bound by issue: a select block's waves spend most of
// their time on the per-slice VALU work of the pass, the rest on the
// selection's dependent steps.
#include "mita.h"
#include "mita_bucket.hpp"
#include "mita_device.hpp"
#include "mita_internal.hpp"
#include "tile_dma.hpp"

namespace mita {

namespace {

constexpr int kMedThreads = 512;
constexpr int kMedPf = 4;    // K and V slices in flight per wave (register ring)
constexpr int kMedCap = 128; // candidate list per landmark (above it: the bisection)
constexpr int kMedQlSt = kD + 8;

template <int NTMAX>
struct MedSelectLds {
  alignas(16) uint8_t vslot[8][2][2048];  // per wave: two 16-row V slices (tile_dma layout)
  union {  // used one after the other
    uint32_t smax[32][NTMAX * 8 + 1];  // per landmark slot: order bits of each 8-key group's
                                       // maximum (rows padded against bank conflicts)
    uint64_t cand[32][kMedCap + 1];  // candidate keys: order bits << 32 | ~key index (rows
                                     // padded: the 16 lanes of a store hit 16 banks)
    struct {
      uint16_t gtm[32][NTMAX * 4];   // bisection path, per 16-key slice: keys above T
      uint16_t tiem[32][NTMAX * 4];  // ... and keys equal to T
    } bm;
  } u;
  uint32_t selm[32][kMediumMaxN / 32 + 14];  // selected keys as bits (64 words), per landmark slot
  uint32_t theta[32];                // candidate threshold per landmark slot
  int ccnt[32];                      // candidates per landmark slot
  alignas(16) int xcnt[2][32][4];    // bisection counts per [parity][landmark][quarter]
  alignas(16) int xflag[2][2];       // landmark tile finished, per [parity][tile]
  alignas(16) float xmax[32][4];     // largest score per [landmark][quarter]
  alignas(16) int xgt[32][4];        // keys above T per [landmark][quarter]
  alignas(16) float xsum[32][4];     // softmax weight sums per [landmark][quarter]
};

struct MedRouteLds {
  uint16_t qls[kMaxM * kMedQlSt];  // landmark queries, rows past m zero
  uint8_t route[kMediumMaxN];
  int cnt[kMaxM];
  int base[kMaxM];
  alignas(16) int wcnt[8][kMaxM];  // (also the block assignment's scratch, read as int4)
};

template <int NTMAX>
union MedLds {
  MedSelectLds<NTMAX> sel;
  MedRouteLds rt;
};

// LDS writes of this wave complete, then the block barrier (no wait on the
// vector-memory counter: V slices may stay in flight across it)
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// DPP row operations over the 16 lanes of a row (quad swaps, then the
// half-row and row mirrors): every lane ends with the row's total
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int row16_sum_i(int v) {
  v += dpp_i<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_i<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_i<0x141>(v);  // row_half_mirror
  v += dpp_i<0x140>(v);  // row_mirror
  return v;
}
__device__ __forceinline__ uint32_t row16_min_u(uint32_t v) {
  v = min(v, static_cast<uint32_t>(dpp_i<0xB1>(static_cast<int>(v))));
  v = min(v, static_cast<uint32_t>(dpp_i<0x4E>(static_cast<int>(v))));
  v = min(v, static_cast<uint32_t>(dpp_i<0x141>(static_cast<int>(v))));
  v = min(v, static_cast<uint32_t>(dpp_i<0x140>(static_cast<int>(v))));
  return v;
}
// inclusive prefix sum within each 16-lane row (row_shr 1, 2, 4, 8; lanes
// shifted in from outside the row read 0)
__device__ __forceinline__ int row16_incl_i(int v) {
  v += __builtin_amdgcn_mov_dpp(v, 0x111, 0xF, 0xF, true);
  v += __builtin_amdgcn_mov_dpp(v, 0x112, 0xF, 0xF, true);
  v += __builtin_amdgcn_mov_dpp(v, 0x114, 0xF, 0xF, true);
  v += __builtin_amdgcn_mov_dpp(v, 0x118, 0xF, 0xF, true);
  return v;
}
// lanes c16 + 16 g' (g' = 0..3) hold v: the exclusive prefix over g' < g and
// the total
__device__ __forceinline__ void prefix_over_g(int v, int c16, int g, int& before, int& total) {
  const int v0 = static_cast<int>(lane_read(static_cast<uint32_t>(v), c16));
  const int v1 = static_cast<int>(lane_read(static_cast<uint32_t>(v), c16 + 16));
  const int v2 = static_cast<int>(lane_read(static_cast<uint32_t>(v), c16 + 32));
  const int v3 = static_cast<int>(lane_read(static_cast<uint32_t>(v), c16 + 48));
  before = (g > 0 ? v0 : 0) + (g > 1 ? v1 : 0) + (g > 2 ? v2 : 0);
  total = v0 + v1 + v2 + v3;
}

__device__ __forceinline__ int xsum16_32(int v) {
  uint32_t u = static_cast<uint32_t>(v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  u = r[0] + r[1];
  r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return static_cast<int>(r[0] + r[1]);
}
__device__ __forceinline__ uint32_t xor16_32(uint32_t u) {
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  u = r[0] | r[1];
  r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return r[0] | r[1];
}

typedef unsigned short us16x2 __attribute__((ext_vector_type(2)));

// per 16-bit half: 1 where x < c, else 0 (saturating c - x, then min with
// 1: two packed instructions per two keys)
__device__ __forceinline__ uint32_t lt16x2(uint32_t c2x, uint32_t x) {
  uint32_t d, r;
  asm("v_pk_sub_u16 %0, %1, %2 clamp" : "=v"(d) : "v"(c2x), "v"(x));
  asm("v_pk_min_u16 %0, %1, %2" : "=v"(r) : "v"(d), "v"(0x00010001u));
  return r;
}

// the float whose order bits are o (inverse of score_order_bits)
__device__ __forceinline__ float order_bits_score(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ f32x4 mfma_bf16_k16(v4i16 a, v4i16 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// select block: landmarks 32 tb .. 32 tb + 31 of head bh
// ---------------------------------------------------------------------------
template <int NTMAX>
__device__ __forceinline__ void med_select(const uint16_t* __restrict__ K,
                                           const uint16_t* __restrict__ V,
                                           const uint16_t* __restrict__ Ql, int N, int m, int k,
                                           float c2, int64_t bh, int tb, float* __restrict__ vl,
                                           float* __restrict__ vl_copy,
                                           int32_t* __restrict__ idx_out,
                                           MedSelectLds<NTMAX>& S) {
  const int l = lane_id(), g = l >> 4, c16 = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const int lt = w >> 2, kq = w & 3;
  const int li = 16 * lt + c16;  // landmark slot of this lane's column (0 .. 31)
  const int i = 32 * tb + li;
  const bool iok = i < m;
  const int NT = (N + 63) >> 6;  // 64-key tiles
  const uint16_t* Kh = K + bh * N * kD;
  const uint16_t* Vh = V + bh * N * kD;
  const u32x4 z = {0, 0, 0, 0};

  bf16x8 qb[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
    qb[s] = as_bf16x8(iok ? *reinterpret_cast<const u32x4*>(Ql + (bh * m + i) * kD + 32 * s + 8 * g)
                          : z);
  if (threadIdx.x < 2) S.xflag[1][threadIdx.x] = 0;
  if (threadIdx.x < 32) S.ccnt[threadIdx.x] = 0;

  // ---- one pass over K and V: scores, V_l ------------------------------
  // Slice t of this wave: keys 64 t + 16 kq .. + 15.  K rows go straight
  // into the score MFMA's operand registers; V rows go through registers
  // into one of two LDS slots (the swizzled tile layout), from which the
  // LDS transpose read gives the P.V operand.  Both load unconditionally
  // (rows past N clamped to N - 1, their weights 0), kMedPf slices ahead.
  // V_l: online softmax per wave (running maximum in the scores' units,
  // P.V on v_mfma_f32_16x16x16_bf16 with P as bf16 hi + lo, V exact); the
  // four key quarters are combined at the end.  The scores are kept as
  // their order bits (0 for keys past N: below every real score), split
  // into 16-bit halves packed two keys to a register: H holds the high
  // halves of keys (t, 0), (t, 1) in H[2t] and of (t, 2), (t, 3) in H[2t+1],
  // L the low halves alike.
  uint32_t H[2 * NTMAX], L[2 * NTMAX];
  auto obits = [&](int t, int r) -> uint32_t {
    const uint32_t h = H[2 * t + (r >> 1)], lo = L[2 * t + (r >> 1)];
    return (r & 1) ? ((h & 0xFFFF0000u) | (lo >> 16)) : ((h << 16) | (lo & 0xFFFFu));
  };
  u32x4 kr[kMedPf][2], vr[kMedPf][2];
  auto load = [&](int t, u32x4 (&kd)[2], u32x4 (&vd)[2]) {
    const int row = min(64 * t + 16 * kq + c16, N - 1);
    kd[0] = *reinterpret_cast<const u32x4*>(Kh + static_cast<int64_t>(row) * kD + 8 * g);
    kd[1] = *reinterpret_cast<const u32x4*>(Kh + static_cast<int64_t>(row) * kD + 32 + 8 * g);
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // V chunk (row 8 j + l / 8, 16-byte column l % 8)
      const int vrow = min(64 * t + 16 * kq + 8 * j + (l >> 3), N - 1);
      vd[j] = *reinterpret_cast<const u32x4*>(Vh + static_cast<int64_t>(vrow) * kD + 8 * (l & 7));
    }
  };
  int vst[2], voff[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) vst[j] = tile_off(8 * j + (l >> 3), l & 7);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    voff[dt] = tile_off(4 * g + (c16 >> 2), 2 * dt + ((c16 & 3) >> 1)) + ((c16 & 1) << 3);
  float Mw = -INFINITY, lsum = 0.f;  // running maximum (unscaled score) and weight sum
  f32x4 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < kMedPf; ++j) load(j, kr[j], vr[j]);
#pragma unroll
  for (int t = 0; t < NTMAX; ++t) {
    const u32x4 a0 = kr[t % kMedPf][0], a1 = kr[t % kMedPf][1];
    const u32x4 v0 = vr[t % kMedPf][0], v1 = vr[t % kMedPf][1];
    if (t + kMedPf < NTMAX) load(t + kMedPf, kr[t % kMedPf], vr[t % kMedPf]);
    uint32_t o[4] = {0u, 0u, 0u, 0u};
    if (t < NT) {
      f32x4 a = {0, 0, 0, 0};
      a = mfma_bf16(as_bf16x8(a0), qb[0], a);
      a = mfma_bf16(as_bf16x8(a1), qb[1], a);
      float tm = -INFINITY;
      bool valid[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        valid[r] = 64 * t + 16 * kq + 4 * g + r < N;
        o[r] = valid[r] ? score_order_bits(a[r]) : 0u;
        tm = valid[r] ? fmax_nc(tm, a[r]) : tm;
      }
      // the largest score of each 8-key half of the slice for this lane's
      // landmark (order bits): keys 4g..4g+3 of lanes g = 0, 1 and of 2, 3
      uint32_t sm = max(max(o[0], o[1]), max(o[2], o[3]));
      auto r16 = __builtin_amdgcn_permlane16_swap(sm, sm, false, false);
      sm = max(r16[0], r16[1]);
      if ((g & 1) == 0) S.u.smax[li][8 * t + 2 * kq + (g >> 1)] = sm;
      // online softmax
      tm = xor_max(tm, 16);
      tm = xor_max(tm, 32);
      if (ballot(tm > Mw)) {  // wave-uniform
        const float Mn = fmax_nc(Mw, tm);
        const float alpha = fast_exp2((Mw - Mn) * c2);  // 0 on the first slice
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
        Mw = Mn;
      }
      const float mw2 = Mw * c2;
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = valid[r] ? fast_exp2(fmaf(a[r], c2, -mw2)) : 0.f;
        lsum += p[r];
      }
      v4i16 ph, pl;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint16_t h = f32_to_bf16_bits(p[r]);
        ph[r] = static_cast<short>(h);
        pl[r] = static_cast<short>(f32_to_bf16_bits(p[r] - bf16_to_f32(h)));
      }
      // this wave's LDS accesses complete in program order: slot t & 1 is
      // rewritten two slices later, after its transpose reads
      uint8_t* slot = &S.vslot[w][t & 1][0];
      *reinterpret_cast<u32x4*>(slot + vst[0]) = v0;
      *reinterpret_cast<u32x4*>(slot + vst[1]) = v1;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(slot + voff[dt]));
        acc[dt] = mfma_bf16_k16(x, ph, acc[dt]);
        acc[dt] = mfma_bf16_k16(x, pl, acc[dt]);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      H[2 * t + h] = (o[2 * h] >> 16) | (o[2 * h + 1] & 0xFFFF0000u);
      L[2 * t + h] = (o[2 * h] & 0xFFFFu) | (o[2 * h + 1] << 16);
      // opaque to the optimizer, which would otherwise see through obits()
      // and keep the unpacked bits alive beside the packed ones
      __asm__("" : "+v"(H[2 * t + h]), "+v"(L[2 * t + h]));
    }
  }
  lsum = xor_sum(lsum, 16);
  lsum = xor_sum(lsum, 32);
  if (g == 0) {
    S.xmax[li][kq] = Mw;
    S.xsum[li][kq] = lsum;
  }

  // ---- selection ------------------------------------------------------------
  // Candidates: theta = the k-th largest of the landmark's 8-key group
  // maxima (k distinct keys reach it, so the k-th best key does too; 0 when
  // there are fewer than k groups); the keys at or above theta (about k to
  // 2k of them for scores without many ties) go to a list in LDS.  With
  // 16-key groups the bound was loose at 1024 keys (the 49th of 64 maxima),
  // lists overflowed, and the exact bisection below ran for 18 us.  The
  // expert is then the first k of the list by (score, lower key).  A list
  // longer than kMedCap (heavy ties) sends the whole block to the exact
  // bisection over every key below instead.  Both searches handle a wave's
  // four landmark slots at once, one 16-lane row each (row sums on DPP).
  const int jj = l >> 4, p = l & 15;  // row = landmark slot 4 w + jj, lane p in it
  const int ls = 4 * w + jj;
  const bool lok = 32 * tb + ls < m;
  lds_barrier();  // slice maxima
  {
    constexpr int QN = (NTMAX * 8 + 15) / 16;  // group maxima per lane
    const int ns = 8 * NT;
    uint32_t v[QN];
#pragma unroll
    for (int q = 0; q < QN; ++q) v[q] = (lok && p + 16 * q < ns) ? S.u.smax[ls][p + 16 * q] : 0u;
    uint32_t th = 0;
    bool dn = !lok || ns < k;  // fewer groups than k: every key is a candidate
    for (int bit = 31; bit >= 0; --bit) {
      if (ballot(!dn) == 0ull) break;  // wave-uniform
      const uint32_t cand = th | (1u << bit);
      int c = 0;
#pragma unroll
      for (int q = 0; q < QN; ++q) c += v[q] >= cand ? 1 : 0;
      c = row16_sum_i(c);
      if (!dn && c >= k) {  // the largest th with >= k maxima at or above it
        th = cand;
        dn = c == k;  // the k maxima >= cand are the top k
      }
    }
    if (lok && p == 0) S.theta[ls] = th;
  }
  lds_barrier();  // theta (every wave is past its reads of the slice maxima)
  {
    // the lane's candidates, counted; one atomic per landmark and wave
    // reserves the wave's run of the list, split over the landmark's four
    // lanes in lane order (keys past N, order bits 0, never qualify)
    const uint32_t th = S.theta[li];
    int n = 0;
#pragma unroll
    for (int t = 0; t < NTMAX; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t ob = obits(t, r);
        n += (t < NT && ob != 0u && ob >= th) ? 1 : 0;
      }
    n = iok ? n : 0;
    int before, total;
    prefix_over_g(n, c16, g, before, total);
    int base = 0;
    if (g == 0 && total > 0) base = atomicAdd(&S.ccnt[li], total);
    int pos = static_cast<int>(lane_read(static_cast<uint32_t>(base), c16)) + before;
    // recompute the bits from an opaque copy rather than keep 4 NTMAX of
    // them alive from the count above
#pragma unroll
    for (int p2 = 0; p2 < 2 * NTMAX; ++p2) __asm__ volatile("" : "+v"(H[p2]), "+v"(L[p2]));
#pragma unroll
    for (int t = 0; t < NTMAX; ++t) {
      if (t < NT && n > 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t ob = obits(t, r);
          if (ob != 0u && ob >= th) {
            if (pos < kMedCap)
              S.u.cand[li][pos] = (static_cast<uint64_t>(ob) << 32) |
                                  static_cast<uint32_t>(~(64 * t + 16 * kq + 4 * g + r));
            ++pos;
          }
        }
      }
    }
  }
  lds_barrier();  // candidate lists
  const bool overflow = ballot(l < 32 && 32 * tb + l < m && S.ccnt[l] > kMedCap) != 0ull;
  if (!overflow) {  // block-uniform (every wave reads the same counts)
    // per landmark slot (one row): T = the k-th largest order bits among
    // the candidates (bisection); the keys above T, then those equal to T by
    // lower index, are the expert; their indices come out ascending through
    // a bit mask of the head's keys
    constexpr int QC = kMedCap / 16;
    const int c = lok ? S.ccnt[ls] : 0;  // >= k
    uint32_t oq[QC], kx[QC];
#pragma unroll
    for (int q = 0; q < QC; ++q) {
      const uint64_t e = p + 16 * q < c ? S.u.cand[ls][p + 16 * q] : 0ull;
      oq[q] = static_cast<uint32_t>(e >> 32);  // 0: empty
      kx[q] = ~static_cast<uint32_t>(e);       // key index
    }
    uint32_t T = 0;
    bool dn = !lok;
    for (int bit = 31; bit >= 0; --bit) {
      if (ballot(!dn) == 0ull) break;  // wave-uniform
      const uint32_t cand = T | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int q = 0; q < QC; ++q) cnt += oq[q] >= cand ? 1 : 0;
      cnt = row16_sum_i(cnt);
      if (!dn && cnt >= k) {
        T = cand;
        dn = cnt == k;  // exactly the k keys >= cand
      }
    }
    uint32_t selb = 0, tieb = 0;  // bit q: candidate q selected / tied at T
    int gt = 0;
#pragma unroll
    for (int q = 0; q < QC; ++q) {
      const bool sq = lok && oq[q] > T;  // T >= 1: empty slots never qualify
      selb |= sq ? 1u << q : 0u;
      tieb |= (lok && oq[q] == T) ? 1u << q : 0u;
      gt += sq ? 1 : 0;
    }
    int need = lok ? k - row16_sum_i(gt) : 0;  // ties taken, lowest key first
    while (ballot(need > 0) != 0ull) {  // wave-uniform; rare beyond one round
      uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
      for (int q = 0; q < QC; ++q) mn = ((tieb >> q) & 1u) ? min(mn, kx[q]) : mn;
      mn = row16_min_u(mn);
      if (need > 0) {
#pragma unroll
        for (int q = 0; q < QC; ++q)
          if (((tieb >> q) & 1u) && kx[q] == mn) {
            selb |= 1u << q;
            tieb &= ~(1u << q);
          }
        --need;
      }
    }
    uint32_t* sm = &S.selm[ls][0];
#pragma unroll
    for (int q = 0; q < 4; ++q) sm[4 * p + q] = 0u;  // this wave's LDS accesses stay in order
#pragma unroll
    for (int q = 0; q < QC; ++q)
      if ((selb >> q) & 1u) atomicOr(&sm[kx[q] >> 5], 1u << (kx[q] & 31u));
    uint32_t wd[4];
    int pc = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      wd[q] = sm[4 * p + q];
      pc += __popc(wd[q]);
    }
    int pos = row16_incl_i(pc) - pc;  // selected keys in the row's earlier words
    if (lok) {
      int32_t* dst = idx_out + (bh * m + 32 * tb + ls) * k;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t wq = wd[q];
        while (wq != 0u) {
          if (pos < k) dst[pos] = 32 * (4 * p + q) + __builtin_ctz(wq);
          ++pos;
          wq &= wq - 1u;
        }
      }
    }
  } else {
  // Exact bisection (the fallback).  The packed scores pass through an
  // opaque copy first, so that the compiler does not keep the candidate
  // step's unpacked bits alive across the bisection.
#pragma unroll
  for (int p2 = 0; p2 < 2 * NTMAX; ++p2) __asm__ volatile("" : "+v"(H[p2]), "+v"(L[p2]));
  // Packed 16-bit counting, two keys per register: while the candidate's low
  // half is zero (bits 31 .. 16) a key reaches it iff its high half does;
  // after that only keys whose high half equals T's can differ, compared on
  // their low halves (the others keep a fixed count).
  constexpr int NV = NTMAX * 4, NP = NV / 2;
  auto below16 = [&](const uint32_t (&v)[NP], uint32_t c) -> int {
    const uint32_t c2x = c * 0x10001u;
    us16x2 a0 = {0, 0}, a1 = {0, 0};
#pragma unroll
    for (int p2 = 0; p2 < NP; p2 += 2) {
      a0 += __builtin_bit_cast(us16x2, lt16x2(c2x, v[p2]));
      if (p2 + 1 < NP) a1 += __builtin_bit_cast(us16x2, lt16x2(c2x, v[p2 + 1]));
    }
    a0 += a1;
    return static_cast<int>(a0[0]) + static_cast<int>(a0[1]);
  };
  uint32_t T = 0;
  bool done = !iok;
  int par = 0;
  bool finished = false;  // block-uniform
  // One bisection step for candidate T | bit: this wave's count, the four
  // quarters' total through LDS, the decision (identical in the four waves
  // of a landmark tile), and the block-uniform stop one step after both
  // tiles have finished.
  auto step = [&](uint32_t cand, int c_local) {
    c_local = xsum16_32(c_local);
    if (g == 0) S.xcnt[par][li][kq] = c_local;
    lds_barrier();
    const int4 v = *reinterpret_cast<const int4*>(&S.xcnt[par][li][0]);
    const int total = v.x + v.y + v.z + v.w;
    finished = S.xflag[par ^ 1][0] != 0 && S.xflag[par ^ 1][1] != 0;
    if (!done && total >= k) {
      T = cand;
      done = total == k;
    }
    const bool tile_done = ballot(!done) == 0ull;
    if (kq == 0 && l == 0) S.xflag[par][lt] = tile_done ? 1 : 0;
    par ^= 1;
  };
  {
    for (int bit = 31; bit >= 16 && !finished; --bit) {
      const uint32_t cand = T | (1u << bit);
      step(cand, NV - below16(H, cand >> 16));
    }
    if (!finished) {
      const uint32_t hiT = T >> 16;
      const int above = hiT == 0xFFFFu ? 0 : NV - below16(H, hiT + 1);
      // the low halves of keys whose high half is T's, 0 for the others,
      // formed on the fly (this path is rare; a stored copy would cost
      // registers everywhere)
      auto below_lo = [&](uint32_t c) -> int {
        const uint32_t c2x = c * 0x10001u;
        us16x2 a0 = {0, 0}, a1 = {0, 0};
#pragma unroll
        for (int p2 = 0; p2 < NP; ++p2) {
          const uint32_t lp = ((H[p2] & 0xFFFFu) == hiT ? (L[p2] & 0xFFFFu) : 0u) |
                              ((H[p2] >> 16) == hiT ? (L[p2] & 0xFFFF0000u) : 0u);
          if (p2 & 1)
            a1 += __builtin_bit_cast(us16x2, lt16x2(c2x, lp));
          else
            a0 += __builtin_bit_cast(us16x2, lt16x2(c2x, lp));
        }
        a0 += a1;
        return static_cast<int>(a0[0]) + static_cast<int>(a0[1]);
      };
      for (int bit = 15; bit >= 0 && !finished; --bit) {
        const uint32_t cand = T | (1u << bit);
        step(cand, above + NV - below_lo(cand & 0xFFFFu));
      }
    }
  }
  // keys above T, keys equal to T (T >= 1: keys past N, order bits 0, are
  // neither), as 16-bit masks per 16-key slice
  {
    int gt = 0;
#pragma unroll
    for (int t = 0; t < NTMAX; ++t) {
      uint32_t gm = 0, tm = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t ob = obits(t, r);
        gm |= (ob > T ? 1u : 0u) << (4 * g + r);
        tm |= (ob == T ? 1u : 0u) << (4 * g + r);
      }
      gt += __popc(gm);
      if (t < NT) {
        gm = xor16_32(gm);
        tm = xor16_32(tm);
        if (g == 0) {
          S.u.bm.gtm[li][4 * t + kq] = static_cast<uint16_t>(gm);
          S.u.bm.tiem[li][4 * t + kq] = static_cast<uint16_t>(tm);
        }
      }
    }
    gt = xsum16_32(gt);
    if (g == 0) S.xgt[li][kq] = gt;
  }
  lds_barrier();
  // one wave per landmark slot 4w + j: expert list ascending, k entries
  {
    const int nw32 = 2 * NT;  // 32-key words
#pragma unroll 1
    for (int j = 0; j < 4; ++j) {
      const int ls = 4 * w + j, i2 = 32 * tb + ls;
      if (i2 >= m) break;  // wave-uniform
      const int4 gv = *reinterpret_cast<const int4*>(&S.xgt[ls][0]);
      const int need = k - (gv.x + gv.y + gv.z + gv.w);  // keys equal to T taken, lowest first
      const uint32_t gw = l < nw32 ? reinterpret_cast<const uint32_t*>(&S.u.bm.gtm[ls][0])[l] : 0u;
      uint32_t tw = l < nw32 ? reinterpret_cast<const uint32_t*>(&S.u.bm.tiem[ls][0])[l] : 0u;
      const int tc = __popc(tw);
      const int tbefore = wave_inclusive_sum(tc) - tc;
      int take = need - tbefore;
      take = take < 0 ? 0 : (take > tc ? tc : take);
      uint32_t sel = gw;
      for (; take > 0; --take) {
        sel |= tw & (0u - tw);  // lowest remaining tie
        tw &= tw - 1u;
      }
      const int sc = __popc(sel);
      int pos = wave_inclusive_sum(sc) - sc;
      int32_t* dst = idx_out + (bh * m + i2) * k;
      while (sel != 0u) {
        const int b = __builtin_ctz(sel);
        if (pos < k) dst[pos] = 32 * l + b;
        ++pos;
        sel &= sel - 1u;
      }
    }
  }

  }  // bisection fallback

  // ---- V_l: the four key quarters' partial softmax sums combined ---------
  lds_barrier();  // every wave is done with its V slots (and the selection)
  float* red = reinterpret_cast<float*>(&S.vslot[0][0][0]);  // [wave][dt][lane][4]
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    *reinterpret_cast<f32x4*>(red + ((w * 4 + dt) * 64 + l) * 4) = acc[dt];
  lds_barrier();
  {
    // wave (lt, kq) finishes feature block dt = kq of its 16 landmarks
    const int dt = kq;
    const float4 mv = *reinterpret_cast<const float4*>(&S.xmax[li][0]);
    const float4 sv = *reinterpret_cast<const float4*>(&S.xsum[li][0]);
    const float M = fmax_nc(fmax_nc(mv.x, mv.y), fmax_nc(mv.z, mv.w));
    const float f[4] = {fast_exp2((mv.x - M) * c2), fast_exp2((mv.y - M) * c2),
                        fast_exp2((mv.z - M) * c2), fast_exp2((mv.w - M) * c2)};
    f32x4 o = {0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o += *reinterpret_cast<const f32x4*>(red + (((4 * lt + q) * 4 + dt) * 64 + l) * 4) * f[q];
    const float inv = 1.0f / ((sv.x * f[0] + sv.y * f[1]) + (sv.z * f[2] + sv.w * f[3]));
    o *= inv;  // O^T[16 dt + 4 g + r][landmark c16]
    if (iok) {
      *reinterpret_cast<f32x4*>(vl + (bh * m + i) * kD + 16 * dt + 4 * g) = o;
      if (vl_copy) *reinterpret_cast<f32x4*>(vl_copy + (bh * m + i) * kD + 16 * dt + 4 * g) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// route block: routing and the stable counting sort of head bh
// ---------------------------------------------------------------------------
__device__ __forceinline__ void med_route_bucket(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Ql, int N, int m, int64_t bh,
    int tpb, int32_t* __restrict__ route_out, int32_t* __restrict__ offsets,
    int32_t* __restrict__ item_start, int32_t* __restrict__ perm, int32_t* __restrict__ off_copy,
    int32_t* __restrict__ perm_copy, int32_t* __restrict__ item_blocks, int ipb, int nbx,
    MedRouteLds& S) {
  const int tid = threadIdx.x, l = lane_id(), g = l >> 4, c16 = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const uint16_t* Qh = Q + bh * N * kD;
  const u32x4 z = {0, 0, 0, 0};
  // query groups of 16: G = w + 8 j; all of a wave's rows requested before
  // the landmark rows are staged (rows past N clamped, results unused)
  constexpr int NJ = (kMediumMaxN + 127) / 128;
  bf16x8 qr[NJ][2];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int q = min(16 * (w + 8 * j) + c16, N - 1);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      qr[j][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(Qh + static_cast<int64_t>(q) * kD +
                                                           32 * s + 8 * g));
  }
  for (int c = tid; c < kMaxM * 8; c += kMedThreads) {
    const int row = c >> 3, col = c & 7;
    *reinterpret_cast<u32x4*>(S.qls + row * kMedQlSt + col * 8) =
        row < m ? *reinterpret_cast<const u32x4*>(Ql + (bh * m + row) * kD + col * 8) : z;
  }
  if (tid < kMaxM) S.cnt[tid] = 0;
  __syncthreads();
  const int mtiles = (m + 15) >> 4;
  bf16x8 qlr[4][2];  // the landmark operands, read from LDS once
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int s = 0; s < 2; ++s)
      qlr[mt][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(
          S.qls + (16 * mt + c16) * kMedQlSt + 32 * s + 8 * g));
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int q0 = 16 * (w + 8 * j);
    if (q0 >= N) break;  // wave-uniform
    float best = -INFINITY;
    int bi = 0;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt < mtiles) {
        f32x4 a = {0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < 2; ++s) a = mfma_bf16(qlr[mt][s], qr[j][s], a);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lmi = 16 * mt + 4 * g + r;  // increasing within the lane
          const bool better = lmi < m && a[r] > best;
          best = better ? a[r] : best;
          bi = better ? lmi : bi;
        }
      }
    }
    xor_argmax(best, bi, 16);  // larger value, then lower landmark
    xor_argmax(best, bi, 32);
    const int q = q0 + c16;
    if (g == 0 && q < N) {
      route_out[bh * N + q] = bi;
      S.route[q] = static_cast<uint8_t>(bi);
      atomicAdd(&S.cnt[bi], 1);
    }
  }
  __syncthreads();
  if (w == 0) {  // offsets and work items (64-query tiles, tpb per item)
    const int c = l < m ? S.cnt[l] : 0;
    const int incl = wave_inclusive_sum(c);
    const int items = ((c + kAttendTile - 1) / kAttendTile + tpb - 1) / tpb;
    const int incl_items = wave_inclusive_sum(items);
    if (l < m) {
      S.base[l] = incl - c;
      offsets[bh * (m + 1) + l] = incl - c;
      item_start[bh * (m + 1) + l] = incl_items - items;
      if (off_copy) off_copy[bh * (m + 1) + l] = incl - c;
    }
    if (l == m - 1) {
      offsets[bh * (m + 1) + m] = incl;
      item_start[bh * (m + 1) + m] = incl_items;
      if (off_copy) off_copy[bh * (m + 1) + m] = incl;
    }
  }
  // stable scatter, 512 queries at a time: a query's slot = its expert's
  // running base + the same-expert queries of the earlier waves + its rank
  // among the same-expert lanes below it (six ballots over the route bits)
  const uint64_t below = l == 0 ? 0ull : (~0ull >> (64 - l));
  for (int q0 = 0; q0 < N; q0 += kMedThreads) {
    reinterpret_cast<int*>(&S.wcnt[0][0])[tid] = 0;  // 8 x 64 counters, one per thread
    __syncthreads();
    const int q = q0 + tid;
    const bool ok = q < N;
    const int r = ok ? S.route[q] : 0;
    uint64_t same = ballot(ok);
#pragma unroll
    for (int b = 0; b < 6; ++b) {
      const bool bit = (r >> b) & 1;
      const uint64_t bb = ballot(bit);
      same &= bit ? bb : ~bb;
    }
    const int rank = __popcll(same & below);
    if (ok && rank == __popcll(same) - 1) S.wcnt[w][r] = rank + 1;
    __syncthreads();
    if (ok) {
      int pos = S.base[r] + rank;
      for (int w2 = 0; w2 < w; ++w2) pos += S.wcnt[w2][r];
      perm[bh * N + pos] = q;
      if (perm_copy) perm_copy[bh * N + pos] = q;
    }
    __syncthreads();
    if (tid < m) {
      int add = 0;
#pragma unroll
      for (int w2 = 0; w2 < 8; ++w2) add += S.wcnt[w2][tid];
      S.base[tid] += add;
    }
    __syncthreads();  // bases read and counters summed before the next chunk
  }
  // the short-item attention's block assignment, after the scatter (the
  // scatter's waves need not wait for it)
  if (w == 0 && item_blocks != nullptr)  // (the counters' LDS is free now)
    write_item_blocks(l < m ? S.cnt[l] : 0, m, tpb, ipb, nbx, bh, item_blocks,
                      &S.wcnt[0][0]);
}

// grid: nsel select blocks, then BH route blocks.  Select block b: XCD
// b % 8 (blocks are handed to the XCDs in turn), so a head's select blocks
// get consecutive slots of one XCD and share its L2.
template <int NTMAX>
__global__ __launch_bounds__(kMedThreads) void k_medium_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ Ql, int N, int m, int k,
    float c2, int BH, int nblk, int nsel, int tpb, float* __restrict__ vl,
    float* __restrict__ vl_copy, int32_t* __restrict__ idx_out, int32_t* __restrict__ route_out,
    int32_t* __restrict__ offsets, int32_t* __restrict__ item_start, int32_t* __restrict__ perm,
    int32_t* __restrict__ off_copy, int32_t* __restrict__ perm_copy,
    int32_t* __restrict__ item_blocks, int ipb, int nbx) {
  __shared__ MedLds<NTMAX> S;
  const int b = static_cast<int>(blockIdx.x);
  if (b < nsel) {
    const int xcd = b & 7, slot = b >> 3;
    const int bh = (slot / nblk) * 8 + xcd, tb = slot % nblk;
    if (bh >= BH) return;  // whole block
    med_select<NTMAX>(K, V, Ql, N, m, k, c2, bh, tb, vl, vl_copy, idx_out, S.sel);
  } else {
    med_route_bucket(Q, Ql, N, m, b - nsel, tpb, route_out, offsets, item_start, perm, off_copy,
                     perm_copy, item_blocks, ipb, nbx, S.rt);
  }
}

template <int NTMAX>
hipError_t launch_medium_t(const Shape& s, const void* Q, const void* K, const void* V,
                           const Workspace& ws, int32_t* idx_out, int32_t* route_out,
                           float* vl_copy, int32_t* off_copy, int32_t* perm_copy,
                           hipStream_t st) {
  const int nblk = (s.m + 31) / 32;
  const int bh8 = static_cast<int>((s.BH + 7) / 8) * 8;
  const int nsel = bh8 * nblk;
  hipLaunchKernelGGL((k_medium_bf16<NTMAX>), dim3(nsel + static_cast<int>(s.BH)),
                     dim3(kMedThreads), 0, st, static_cast<const uint16_t*>(Q),
                     static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V),
                     static_cast<const uint16_t*>(ws.ql), static_cast<int>(s.N), s.m, s.k,
                     s.scale * kLog2e, static_cast<int>(s.BH), nblk, nsel, s.attend_tpb, ws.vl,
                     vl_copy, idx_out, route_out, ws.offsets, ws.item_start, ws.perm, off_copy,
                     perm_copy, ws.item_blocks, s.attend_ipb, s.attend_nbx);
  return hipGetLastError();
}

}  // namespace

bool medium_path_fits(const Shape& s) {
  return s.dtype == MITA_BF16 && s.s == 1 && s.N > kSmallMaxN && s.N <= kMediumMaxN &&
         s.m <= kMaxM && s.k <= kMaxK && s.BH <= (int64_t{1} << 24);
}

hipError_t launch_medium(const Shape& s, const void* Q, const void* K, const void* V,
                         const Workspace& ws, int32_t* idx_out, int32_t* route_out,
                         float* vl_copy, int32_t* off_copy, int32_t* perm_copy, hipStream_t st) {
  if (!medium_path_fits(s)) return hipErrorInvalidValue;
  // 64-key tiles held per wave: the fewest that cover N (25 at most: the
  // packed scores, the bisection's low halves and pass 2 then fit the 256
  // registers of two waves per SIMD without spilling)
  if (s.N <= 512)
    return launch_medium_t<8>(s, Q, K, V, ws, idx_out, route_out, vl_copy, off_copy, perm_copy,
                              st);
  if (s.N <= 1024)
    return launch_medium_t<16>(s, Q, K, V, ws, idx_out, route_out, vl_copy, off_copy, perm_copy,
                               st);
  return launch_medium_t<25>(s, Q, K, V, ws, idx_out, route_out, vl_copy, off_copy, perm_copy,
                             st);
}

}  // namespace mita
