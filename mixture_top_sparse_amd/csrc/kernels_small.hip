// kernels_small.hip — the whole MiTA forward pass of one (batch, head) in one
// workgroup, for short sequences (at most 256 tokens, bf16): the image-shaped
// workloads of the pages (14x14 patches with m = k = 25, 50 pairs per query:
// "NeurIPS'26：注意力也是FFN？…", section "用少量地标查询，同时构造全局概括与
// 细节专家"), where the multi-launch path spends its time in launch latency.
//
// One 256-thread block per head holds that head's K and V rows in LDS and
// runs the five steps back to back, separated by block barriers:
//   1. pool     landmark queries Ql: fp64 window sums, one fp64 divide, RNE
//               into bf16 (the same rule as the multi-launch pooling kernels)
//   2. scan     S^T = K Ql^T on bf16 MFMA, 16 landmarks per wave; expert
//               i = the k best keys (a bisection over the 32-bit score order
//               finds the k-th score, ties at it go to the lower keys);
//               Vl = softmax(scale*S) V on MFMA with P as bf16 hi + lo
//   3. route    R^T = Ql Q^T on MFMA, argmax per query (ties: lower landmark)
//   4. bucket   counting sort of the queries by expert (stable), in LDS
//   5. attend   per 16-query sub-tile of one expert (queries gathered in
//               bucket order): logits over [Ql; K rows of the expert] on
//               MFMA, one softmax over the m + k logits, P.V with P and Vl as
//               bf16 hi + lo (raw values exact), as the multi-launch expert
//               attention computes them
// ("Mixture-of-Top-k 注意力…", section "MiTA：用少量地标查询，同时完成压缩与
// 专家构造"; "And attention is also FFN? …", Figure 3 and Algorithm 1.)
//
// MFMA layouts as in mita_device.hpp: the per-row statistic (landmark in the
// scan, query in routing and attention) sits on the output columns, so its
// softmax state stays in the 4 lanes l % 16 == const.
//
// Roofline: per head, Q is read from global three times (pooling, routing,
// the attention's gather; the second and third hit L2), K and V once, the
// fp32 output and routes written once.  No work space.
#include "mita_bucket.hpp"
#include "mita_device.hpp"
#include "mita_internal.hpp"

namespace mita {

constexpr int kSmallThreads = 256;

template <int NMAX, int MPAD, int KPAD>
struct SmallLds {
  static constexpr int KST = 72;         // K and Ql rows (bf16 elements; 144 B, 16-byte aligned)
  static constexpr int VCST = MPAD + 4;  // Vl^T rows (bf16)
  alignas(16) uint16_t kr[NMAX * KST];   // K rows; rows past N are zero
  alignas(16) uint16_t vr[NMAX * kD];    // V rows; rows past N are zero
  alignas(16) uint16_t ql[MPAD * KST];   // landmark queries; rows past m are zero
  alignas(16) uint16_t vch[kD * VCST];   // Vl^T, bf16 hi part (columns past m zero)
  alignas(16) uint16_t vcl[kD * VCST];   // Vl^T, bf16 lo part
  int16_t idx[MPAD * KPAD];              // expert key lists, ascending
  int16_t route[NMAX];
  int16_t perm[NMAX];                    // queries in (expert, query) order
  int32_t cnt[MPAD + 1];                 // queries per expert
  int32_t off[MPAD + 1];                 // first bucket slot of each expert
  int32_t sub[MPAD + 1];                 // first 16-query sub-tile of each expert
  int32_t wcnt[4][MPAD];                 // routed queries per (wave, expert)
};

// round-to-nearest-even fp32 -> bf16 bits (finite input; NaN stays NaN)
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ int xor_sum_i(int v, int mask) {
  const uint32_t u = static_cast<uint32_t>(v);
  const auto r = mask == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                            : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return static_cast<int>(r[0] + r[1]);
}

// the values of lanes c16, c16 + 16, c16 + 32, c16 + 48 (g = 0..3): the
// exclusive prefix over g' < g and the total
__device__ __forceinline__ void prefix_over_g(int v, int c16, int g, int& before, int& total) {
  const int v0 = static_cast<int>(lane_read(static_cast<uint32_t>(v), c16));
  const int v1 = static_cast<int>(lane_read(static_cast<uint32_t>(v), c16 + 16));
  const int v2 = static_cast<int>(lane_read(static_cast<uint32_t>(v), c16 + 32));
  const int v3 = static_cast<int>(lane_read(static_cast<uint32_t>(v), c16 + 48));
  before = (g > 0 ? v0 : 0) + (g > 1 ? v1 : 0) + (g > 2 ? v2 : 0);
  total = v0 + v1 + v2 + v3;
}

typedef unsigned short us16x2 __attribute__((ext_vector_type(2)));

// per 16-bit half: 1 where x < c, else 0 (saturating c - x, then min with
// 1; written out so that the compiler keeps the two packed instructions
// instead of turning them into compares through VCC)
__device__ __forceinline__ uint32_t lt16x2(uint32_t c2x, uint32_t x) {
  uint32_t d, r;
  asm("v_pk_sub_u16 %0, %1, %2 clamp" : "=v"(d) : "v"(c2x), "v"(x));
  asm("v_pk_min_u16 %0, %1, %2" : "=v"(r) : "v"(d), "v"(0x00010001u));
  return r;
}

// 8 bf16 values (K-positions of a 16x16x32 MFMA operand) from lane-chosen
// rows of a row-major bf16 matrix: element j is row rows[j], column col
__device__ __forceinline__ bf16x8 gather_column8(const uint16_t* base, const int (&rows)[8],
                                                 int col) {
  u32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = static_cast<uint32_t>(base[rows[2 * j] * kD + col]) |
           (static_cast<uint32_t>(base[rows[2 * j + 1] * kD + col]) << 16);
  return as_bf16x8(w);
}

template <int NMAX, int MPAD, int KPAD>
__global__ __launch_bounds__(kSmallThreads) void k_small_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, int N, int gh, int gw, int mh, int mw, int k, float c2,
    float* __restrict__ out, int32_t* __restrict__ idx_out, int32_t* __restrict__ route_out,
    uint16_t* __restrict__ ql_copy, float* __restrict__ vl_copy, int32_t* __restrict__ perm_copy,
    int32_t* __restrict__ off_copy, int role_period) {
  using L = SmallLds<NMAX, MPAD, KPAD>;
  constexpr int NTMAX = NMAX / 16;  // key (and query) tiles of 16
  __shared__ L S;
  const int m = mh * mw;
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x, l = lane_id(), g = l >> 4, c16 = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  // the waves' roles in the middle phases (selection, landmark values,
  // routing): swapped between wave pairs (0, 2) and (1, 3) in every other
  // group of role_period blocks (the CU count), so that two blocks sharing
  // a CU - one from each group - run their selection waves on different
  // SIMDs
  const int rw = ((static_cast<int>(blockIdx.x) / role_period) & 1) ? (w ^ 2) : w;
  const int nt = (N + 15) / 16;
  const int ntp = (nt + 1) & ~1;  // whole 32-key MFMA steps
  const uint16_t* Qh = Q + bh * N * kD;
  const uint16_t* Kh = K + bh * N * kD;
  const uint16_t* Vh = V + bh * N * kD;
  const u32x4 z = {0, 0, 0, 0};

  // ---- 1. K and V rows into LDS; pooling --------------------------------
  // Every thread issues all of its K and V loads before storing any of them
  // (one memory latency, not one per row), and the pooling loads below go
  // out while these are in flight.
  constexpr int KVCH = NMAX * 8 / kSmallThreads;  // 16-byte chunks of K (and of V) per thread
  u32x4 kw[KVCH], vw[KVCH];
#pragma unroll
  for (int j = 0; j < KVCH; ++j) {
    const int c = tid + kSmallThreads * j, t = c >> 3, cc = c & 7;
    kw[j] = z;
    vw[j] = z;
    if (t < N) {
      kw[j] = *reinterpret_cast<const u32x4*>(Kh + t * kD + cc * 8);
      vw[j] = *reinterpret_cast<const u32x4*>(Vh + t * kD + cc * 8);
    }
  }
  // task (landmark i, 8 columns from 8*cg): fp64 sum over the window
  // rows [a*gh/mh, ceil((a+1)*gh/mh)) x columns [c*gw/mw, ceil((c+1)*gw/mw)),
  // sixteen tokens' loads in flight at a time
  for (int task = tid; task < MPAD * 8; task += kSmallThreads) {
    const int i = task >> 3, cg = task & 7;
    u32x4 word = z;
    if (i < m) {
      const int a = i / mw, cl = i % mw;
      const int r0 = (a * gh) / mh, r1 = ((a + 1) * gh + mh - 1) / mh;
      const int c0 = (cl * gw) / mw, c1 = ((cl + 1) * gw + mw - 1) / mw;
      const int wc = c1 - c0, W = (r1 - r0) * wc;
      double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int t0 = 0; t0 < W; t0 += 16) {
        u32x4 q[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int t = min(t0 + u, W - 1);
          q[u] = *reinterpret_cast<const u32x4*>(Qh + ((r0 + t / wc) * gw + c0 + t % wc) * kD +
                                                 cg * 8);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (t0 + u < W) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              acc[2 * j] += static_cast<double>(__uint_as_float(q[u][j] << 16));
              acc[2 * j + 1] += static_cast<double>(__uint_as_float(q[u][j] & 0xFFFF0000u));
            }
          }
      }
      const double cnt = static_cast<double>(W);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        word[j] = static_cast<uint32_t>(f64_to_bf16_bits_rne(acc[2 * j] / cnt)) |
                  (static_cast<uint32_t>(f64_to_bf16_bits_rne(acc[2 * j + 1] / cnt)) << 16);
      if (ql_copy)
        *reinterpret_cast<u32x4*>(ql_copy + (bh * m + i) * kD + cg * 8) = word;
    }
    *reinterpret_cast<u32x4*>(S.ql + i * L::KST + cg * 8) = word;
  }
#pragma unroll
  for (int j = 0; j < KVCH; ++j) {
    const int c = tid + kSmallThreads * j, t = c >> 3, cc = c & 7;
    *reinterpret_cast<u32x4*>(S.kr + t * L::KST + cc * 8) = kw[j];
    *reinterpret_cast<u32x4*>(S.vr + t * kD + cc * 8) = vw[j];
  }
  if (tid <= MPAD) S.cnt[tid] = 0;
  __syncthreads();

  // ---- 2. landmark scan ---------------------------------------------------
  // LT tiles of 16 landmarks.  Selection: wave w < LT scores tile w against
  // every key and picks the experts.  Landmark values: with LT = 2 the other
  // two waves score the same tiles again and compute Vl meanwhile; with
  // LT = 4 each wave does both, one after the other.
  constexpr int LT = MPAD / 16;
  auto tile_scores = [&](int lt, float (&sc)[NTMAX][4]) {
    const int i = 16 * lt + c16;
    bf16x8 qb[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
      qb[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(S.ql + i * L::KST + 32 * s + 8 * g));
#pragma unroll
    for (int kt = 0; kt < NTMAX; ++kt) {
      f32x4 a = {0, 0, 0, 0};
      if (kt < nt) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
          a = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(
                            S.kr + (16 * kt + c16) * L::KST + 32 * s + 8 * g)),
                        qb[s], a);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[kt][r] = (16 * kt + 4 * g + r < N) ? a[r] : -INFINITY;
    }
  };
  if (rw < LT) {
    const int i = 16 * rw + c16;  // this lane's landmark (>= m: nothing is kept)
    float sc[NTMAX][4];
    tile_scores(rw, sc);
    // 32-bit order bits of the scores of keys 16 kt + 4g + r (0, below
    // every real score, for the keys past N)
    uint32_t ob[NTMAX][4];
#pragma unroll
    for (int kt = 0; kt < NTMAX; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        ob[kt][r] = (16 * kt + 4 * g + r < N) ? score_order_bits(sc[kt][r]) : 0u;
    // expert: T = the k-th largest order bits (the largest t with at least
    // k keys >= t), found bit by bit; then ties at T by lower key.  A
    // landmark whose count reaches exactly k at some candidate stops there:
    // the keys >= that candidate are then exactly its top k (the tie step
    // below takes every key equal to it, if any), so the rest of the search
    // would not change the set.  The wave stops once all 16 have (lanes of
    // landmarks past m from the start).
    //   Counting runs on packed 16-bit halves, two keys per register: while
    // the candidate's low half is zero (bits 31 .. 16) a key reaches it iff
    // its high half does; after that only keys whose high half equals T's
    // can still differ, and they compare on their low halves (the others
    // keep a fixed count).  Keys past N have order bits 0 and never count.
    constexpr int NV = NTMAX * 4, NP = NV / 2;
    uint32_t hp[NP];
#pragma unroll
    for (int p2 = 0; p2 < NP; ++p2) {
      const uint32_t a = ob[(2 * p2) >> 2][(2 * p2) & 3], b = ob[(2 * p2 + 1) >> 2][(2 * p2 + 1) & 3];
      hp[p2] = (a >> 16) | (b & 0xFFFF0000u);
    }
    // keys below the candidate c (16 bits, >= 1) among the packed halves
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
    bool done = i >= m;
    for (int bit = 31; bit >= 16; --bit) {
      if (ballot(!done) == 0ull) break;  // wave-uniform
      const uint32_t cand = T | (1u << bit);
      int c = NV - below16(hp, cand >> 16);
      c = xor_sum_i(c, 16);
      c = xor_sum_i(c, 32);
      if (!done && c >= k) {
        T = cand;
        done = c == k;
      }
    }
    if (ballot(!done) != 0ull) {
      // low halves: keys whose high half is T's take their low half, the
      // others 0 (below every low candidate); those above T's high half
      // count for every low candidate
      const uint32_t hiT = T >> 16;
      const int above = hiT == 0xFFFFu ? 0 : NV - below16(hp, hiT + 1);
      uint32_t lp[NP];
#pragma unroll
      for (int p2 = 0; p2 < NP; ++p2) {
        const uint32_t a = ob[(2 * p2) >> 2][(2 * p2) & 3], b = ob[(2 * p2 + 1) >> 2][(2 * p2 + 1) & 3];
        lp[p2] = ((a >> 16) == hiT ? (a & 0xFFFFu) : 0u) | ((b >> 16) == hiT ? (b << 16) : 0u);
      }
      for (int bit = 15; bit >= 0; --bit) {
        if (ballot(!done) == 0ull) break;  // wave-uniform
        const uint32_t cand = T | (1u << bit);
        int c = above + NV - below16(lp, cand & 0xFFFFu);
        c = xor_sum_i(c, 16);
        c = xor_sum_i(c, 32);
        if (!done && c >= k) {
          T = cand;
          done = c == k;
        }
      }
    }
    int gt = 0;
#pragma unroll
    for (int kt = 0; kt < NTMAX; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) gt += ob[kt][r] > T ? 1 : 0;
    gt = xor_sum_i(gt, 16);
    gt = xor_sum_i(gt, 32);
    const int need = k - gt;  // keys scoring exactly T that are taken, lowest first
    // keys in index order are (kt, g, r): per key tile, the counts of the
    // landmark's 4 lanes are exchanged in one batch for all tiles
    int tb[NTMAX], tt[NTMAX];
#pragma unroll
    for (int kt = 0; kt < NTMAX; ++kt) {
      int nties = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) nties += ob[kt][r] == T ? 1 : 0;  // T > 0: keys past N never tie
      prefix_over_g(nties, c16, g, tb[kt], tt[kt]);
    }
    bool sel[NTMAX][4];
    int sb[NTMAX], st[NTMAX];
    int ties_before = 0;
#pragma unroll
    for (int kt = 0; kt < NTMAX; ++kt) {
      int rank = ties_before + tb[kt], nsel = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool tie = ob[kt][r] == T;
        sel[kt][r] = ob[kt][r] > T || (tie && rank < need);
        rank += tie ? 1 : 0;
        nsel += sel[kt][r] ? 1 : 0;
      }
      ties_before += tt[kt];
      prefix_over_g(nsel, c16, g, sb[kt], st[kt]);
    }
    int sel_before = 0;
#pragma unroll
    for (int kt = 0; kt < NTMAX; ++kt) {
      int pos = sel_before + sb[kt];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (sel[kt][r]) {
          if (i < m) {
            S.idx[i * KPAD + pos] = static_cast<int16_t>(16 * kt + 4 * g + r);
            idx_out[(bh * m + i) * k + pos] = 16 * kt + 4 * g + r;
          }
          ++pos;
        }
      sel_before += st[kt];
    }
  }
  // LT == 1, 2: wave LT computes every tile's landmark values in turn while
  // wave 3 routes and buckets; LT == 4: each wave its own tile
  for (int lt = LT == 4 ? w : 0; (LT == 4 || rw == LT) && lt < LT; lt += (LT == 4 ? LT : 1)) {
    const int i = 16 * lt + c16;
    float sc[NTMAX][4];
    tile_scores(lt, sc);
    // landmark values: softmax(scale * S) V; P as bf16 hi + lo, V exact
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < NTMAX; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[kt][r]);
    mx = xor_max(mx, 16);
    mx = xor_max(mx, 32) * c2;
    float lsum = 0.f;
#pragma unroll
    for (int kt = 0; kt < NTMAX; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[kt][r] = fast_exp2(fmaf(sc[kt][r], c2, -mx));  // keys past N: exp2(-inf) = 0
        lsum += sc[kt][r];
      }
    lsum = xor_sum(lsum, 16);
    lsum = xor_sum(lsum, 32);
    f32x4 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int s2 = 0; s2 < NTMAX / 2; ++s2) {
      if (2 * s2 < ntp) {
      const float p[8] = {sc[2 * s2][0],     sc[2 * s2][1],     sc[2 * s2][2],
                          sc[2 * s2][3],     sc[2 * s2 + 1][0], sc[2 * s2 + 1][1],
                          sc[2 * s2 + 1][2], sc[2 * s2 + 1][3]};
      bf16x8 ph, pl;
      split_hi_lo_pk(p, ph, pl);
      int rows[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) rows[j] = 32 * s2 + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x8 vt = gather_column8(S.vr, rows, 16 * dt + c16);
        acc[dt] = mfma_bf16(vt, pl, acc[dt]);
        acc[dt] = mfma_bf16(vt, ph, acc[dt]);
      }
      }
    }
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const f32x4 v = acc[dt] * inv;  // Vl[i][16 dt + 4g + r]
      if (i < m && vl_copy)
        *reinterpret_cast<f32x4*>(vl_copy + (bh * m + i) * kD + 16 * dt + 4 * g) = v;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = i < m ? v[r] : 0.f;
        const uint32_t hi = bf16_bits_rne(x);
        const uint32_t lo = bf16_bits_rne(x - __uint_as_float(hi << 16));
        S.vch[(16 * dt + 4 * g + r) * L::VCST + i] = static_cast<uint16_t>(hi);
        S.vcl[(16 * dt + 4 * g + r) * L::VCST + i] = static_cast<uint16_t>(lo);
      }
    }
  }

  // ---- 3. routing (and 4. bucketing) -------------------------------------
  // (needs only Ql, which step 1 left in LDS before the barrier).  A query's
  // route: the largest q . Ql[i] over the MFMA logits, ties to the lower
  // landmark.
  auto route_tile = [&](int qt, const bf16x8 (&qb)[2]) {
    const int q = min(16 * qt + c16, N - 1);
    float best = -INFINITY;
    int bi = 0;
#pragma unroll
    for (int lt = 0; lt < MPAD / 16; ++lt) {
      f32x4 a = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 2; ++s)
        a = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(
                          S.ql + (16 * lt + c16) * L::KST + 32 * s + 8 * g)),
                      qb[s], a);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int li = 16 * lt + 4 * g + r;
        const float v = li < m ? a[r] : -INFINITY;
        if (v > best) {  // strict: the first maximum in landmark order stays
          best = v;
          bi = li;
        }
      }
    }
    xor_argmax(best, bi, 16);
    xor_argmax(best, bi, 32);
    if (g == 0 && 16 * qt + c16 < N) {
      S.route[q] = static_cast<int16_t>(bi);
      route_out[bh * N + q] = bi;
      atomicAdd(&S.cnt[bi], 1);
    }
  };
  auto load_tile = [&](int qt, bf16x8 (&qb)[2]) {
    const int q = min(16 * qt + c16, N - 1);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      qb[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(Qh + q * kD + 32 * s + 8 * g));
  };
  if (LT < 4) {
    // One wave routes every query tile (two tiles' rows in flight) and then
    // sorts the queries by expert on its own, while waves 0 .. LT-1 select
    // the experts and wave LT computes the landmark values: routing and
    // bucketing leave the critical path.  A single wave's LDS accesses
    // complete in program order, so it needs no barrier of its own.
    if (rw == 3) {
      bf16x8 qa[2], qn[2];
      load_tile(0, qa);
      for (int qt = 0; qt < nt; ++qt) {
        if (qt + 1 < nt) load_tile(qt + 1, qn);
        route_tile(qt, qa);
        qa[0] = qn[0];
        qa[1] = qn[1];
      }
      // offsets and first sub-tile of each expert: lane e holds expert e
      const int c = l < m ? S.cnt[l] : 0;
      const int incl = wave_inclusive_sum(c);
      const int u = (c + 15) / 16;
      const int incl_u = wave_inclusive_sum(u);
      if (l < m) {
        S.off[l] = incl - c;
        S.sub[l] = incl_u - u;
      }
      if (l == m - 1) {
        S.off[m] = incl;
        S.sub[m] = incl_u;
      }
      if (off_copy && l < m) off_copy[bh * (m + 1) + l] = incl - c;
      if (off_copy && l == m - 1) off_copy[bh * (m + 1) + m] = incl;
      // stable ranks: queries 64 G + l in groups; lane e carries how many
      // queries of expert e the earlier groups placed
      int placed = 0;
      const int base = l < m ? incl - c : 0;
      for (int G = 0; 64 * G < N; ++G) {
        const int q = 64 * G + l;
        const int r = q < N ? S.route[q] : -1;
        int below = 0, mine = 0;
        for (int e = 0; e < m; ++e) {
          const uint64_t b = ballot(r == e);
          if (r == e) below = static_cast<int>(count_below(b));
          if (l == e) mine = static_cast<int>(__popcll(b));
        }
        const int start = static_cast<int>(lane_read(static_cast<uint32_t>(base + placed), r < 0 ? 0 : r));
        if (q < N) {
          const int pos = start + below;
          S.perm[pos] = static_cast<int16_t>(q);
          if (perm_copy) perm_copy[bh * N + pos] = q;
        }
        placed += mine;
      }
    }
    __syncthreads();
  } else {
    // LT == 4: every wave routes its own query tiles (all requested up
    // front), then the four sort together
    constexpr int RT = (NTMAX + 3) / 4;  // query tiles per wave, at most
    bf16x8 rq[RT][2];
#pragma unroll
    for (int j = 0; j < RT; ++j) load_tile(w + 4 * j, rq[j]);
#pragma unroll
    for (int j = 0; j < RT; ++j)
      if (w + 4 * j < nt) route_tile(w + 4 * j, rq[j]);
    __syncthreads();

  // ---- 4. bucketing: counting sort by expert, stable ---------------------
  if (tid == 0) {
    int s = 0, u = 0;
    for (int e = 0; e < m; ++e) {
      S.off[e] = s;
      S.sub[e] = u;
      s += S.cnt[e];
      u += (S.cnt[e] + 15) / 16;
    }
    S.off[m] = s;
    S.sub[m] = u;
  }
  __syncthreads();
  {
    // rank of query tid among the queries of its expert: the same-expert
    // lanes below it in its wave (one ballot per expert), plus the
    // same-expert queries of the waves before (per-wave counts in LDS)
    const int r = tid < N ? S.route[tid] : -1;
    int below = 0, mine = 0;
    for (int e = 0; e < m; ++e) {
      const uint64_t b = ballot(r == e);
      if (r == e) below = static_cast<int>(count_below(b));
      if (l == e) mine = static_cast<int>(__popcll(b));
    }
    if (l < m) S.wcnt[w][l] = mine;
    __syncthreads();
    if (tid < N) {
      int pos = S.off[r] + below;
      for (int w2 = 0; w2 < w; ++w2) pos += S.wcnt[w2][r];
      S.perm[pos] = static_cast<int16_t>(tid);
      if (perm_copy) perm_copy[bh * N + pos] = tid;
    }
  }
  if (off_copy && tid <= m) off_copy[bh * (m + 1) + tid] = S.off[tid];
  __syncthreads();
  }

  // ---- 5. expert attention: one 16-query sub-tile of one expert per wave --
  const int nsub = S.sub[m];
  const int next_start = l < m - 1 ? S.sub[l + 1] : 0x7FFFFFFF;
  // sub-tile u: its expert (the number of experts e < m - 1 whose successor
  // starts at or before u; sub is non-decreasing) and this lane's query
  // (slots past the group repeat its last query)
  auto locate = [&](int u, int& e, int& q, bool& qvalid) {
    e = __popcll(ballot(next_start <= u));
    const int j0 = (u - S.sub[e]) * 16, ne = S.cnt[e];
    qvalid = j0 + c16 < ne;
    q = S.perm[S.off[e] + min(j0 + c16, ne - 1)];
  };
  auto load_q = [&](int q, bf16x8 (&qb)[2]) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
      qb[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(Qh + q * kD + 32 * s + 8 * g));
  };
  // the next sub-tile's query rows are requested before this one is computed
  int e_n = 0, q_n = 0;
  bool v_n = false;
  bf16x8 qb_n[2];
  if (w < nsub) {
    locate(w, e_n, q_n, v_n);
    load_q(q_n, qb_n);
  }
  for (int u = w; u < nsub; u += kSmallThreads / 64) {
    const int e = e_n, q = q_n;
    const bool qvalid = v_n;
    bf16x8 qb[2] = {qb_n[0], qb_n[1]};
    if (u + kSmallThreads / 64 < nsub) {
      locate(u + kSmallThreads / 64, e_n, q_n, v_n);
      load_q(q_n, qb_n);
    }
    const int16_t* ex = S.idx + e * KPAD;
    constexpr int NPB = (MPAD + KPAD) / 16;
    float x[NPB][4];
    float mx = -INFINITY;
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
      const int p = 16 * pb + c16;  // this lane's pair row of the A operand
      const uint16_t* row = p < MPAD ? S.ql + p * L::KST
                                     : S.kr + (p - MPAD < k ? ex[p - MPAD] : 0) * L::KST;
      f32x4 a = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 2; ++s)
        a = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(row + 32 * s + 8 * g)), qb[s], a);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pp = 16 * pb + 4 * g + r;
        const bool valid = pp < MPAD ? pp < m : pp - MPAD < k;
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
    auto p_split = [&](int pb0, bf16x8& hi, bf16x8& lo) {
      const float p[8] = {x[pb0][0],     x[pb0][1],     x[pb0][2],     x[pb0][3],
                          x[pb0 + 1][0], x[pb0 + 1][1], x[pb0 + 1][2], x[pb0 + 1][3]};
      split_hi_lo_pk(p, hi, lo);
    };
#pragma unroll
    for (int s2 = 0; s2 < MPAD / 32; ++s2) {
      bf16x8 ph, pl;
      p_split(2 * s2, ph, pl);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int o = (16 * dt + c16) * L::VCST + 32 * s2 + 4 * g;
        const bf16x8 vh = join_bf16x8(*reinterpret_cast<const u32x2*>(S.vch + o),
                                      *reinterpret_cast<const u32x2*>(S.vch + o + 16));
        const bf16x8 vlo = join_bf16x8(*reinterpret_cast<const u32x2*>(S.vcl + o),
                                       *reinterpret_cast<const u32x2*>(S.vcl + o + 16));
        acc[dt] = mfma_bf16(vlo, ph, acc[dt]);
        acc[dt] = mfma_bf16(vh, pl, acc[dt]);
        acc[dt] = mfma_bf16(vh, ph, acc[dt]);
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < KPAD / 32; ++s2) {
      bf16x8 ph, pl;
      p_split(MPAD / 16 + 2 * s2, ph, pl);
      int rows[8];  // the expert's keys at this lane's 8 K-positions (pairs past k: key 0, weight 0)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 32 * s2 + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4);
        rows[j] = r < k ? ex[r] : 0;
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x8 vt = gather_column8(S.vr, rows, 16 * dt + c16);
        acc[dt] = mfma_bf16(vt, pl, acc[dt]);
        acc[dt] = mfma_bf16(vt, ph, acc[dt]);
      }
    }
    const float f = __builtin_amdgcn_rcpf(lsum);  // lsum >= 1
    if (qvalid) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        *reinterpret_cast<f32x4*>(out + (bh * N + q) * kD + 16 * dt + 4 * g) = acc[dt] * f;
    }
  }
}

template <int NMAX, int MPAD, int KPAD>
static hipError_t launch_small_t(const Shape& s, const void* Q, const void* K, const void* V,
                                 float* out, int32_t* idx_out, int32_t* route_out, void* ql_copy,
                                 float* vl_copy, int32_t* perm_copy, int32_t* off_copy,
                                 hipStream_t st) {
  auto kern = k_small_bf16<NMAX, MPAD, KPAD>;
  hipLaunchKernelGGL(kern, dim3(s.BH), dim3(kSmallThreads), 0, st,
                     static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                     static_cast<const uint16_t*>(V), static_cast<int>(s.N), s.gh, s.gw, s.mh,
                     s.mw, s.k, s.scale * kLog2e, out, idx_out, route_out,
                     static_cast<uint16_t*>(ql_copy), vl_copy, perm_copy, off_copy,
                     s.cus > 0 ? s.cus : 256);
  return hipGetLastError();
}

template <int NMAX>
static hipError_t launch_small_n(const Shape& s, const void* Q, const void* K, const void* V,
                                 float* out, int32_t* idx_out, int32_t* route_out, void* ql_copy,
                                 float* vl_copy, int32_t* perm_copy, int32_t* off_copy,
                                 hipStream_t st) {
  if (s.mpad == 32 && s.kpad == 32)
    return launch_small_t<NMAX, 32, 32>(s, Q, K, V, out, idx_out, route_out, ql_copy, vl_copy,
                                        perm_copy, off_copy, st);
  if (s.mpad == 32)
    return launch_small_t<NMAX, 32, 64>(s, Q, K, V, out, idx_out, route_out, ql_copy, vl_copy,
                                        perm_copy, off_copy, st);
  if (s.kpad == 32)
    return launch_small_t<NMAX, 64, 32>(s, Q, K, V, out, idx_out, route_out, ql_copy, vl_copy,
                                        perm_copy, off_copy, st);
  return launch_small_t<NMAX, 64, 64>(s, Q, K, V, out, idx_out, route_out, ql_copy, vl_copy,
                                      perm_copy, off_copy, st);
}

bool small_path_fits(const Shape& s) {
  return s.dtype == 1 && s.s == 1 && s.N <= kSmallMaxN && s.m <= kMaxM && s.k <= kMaxK;
}

hipError_t launch_small(const Shape& s, const void* Q, const void* K, const void* V, float* out,
                        int32_t* idx_out, int32_t* route_out, void* ql_copy, float* vl_copy,
                        int32_t* perm_copy, int32_t* off_copy, hipStream_t st) {
  if (s.N <= 224)
    return launch_small_n<224>(s, Q, K, V, out, idx_out, route_out, ql_copy, vl_copy, perm_copy,
                               off_copy, st);
  return launch_small_n<256>(s, Q, K, V, out, idx_out, route_out, ql_copy, vl_copy, perm_copy,
                             off_copy, st);
}

}  // namespace mita
