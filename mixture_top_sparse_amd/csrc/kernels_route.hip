// kernels_route.hip — steps 3 and 4: route every query to its best-matching
// landmark (one expert per query), then group queries by expert.
//
// Routing takes the landmark whose query-landmark dot product is largest;
// these dot products are the compressed-branch logits as well
// ("NeurIPS'26：注意力也是FFN？…", section "用少量地标查询，同时构造全局概括与
// 细节专家"; "Mixture-of-Top-k 注意力…", section "MiTA：用少量地标查询，同时
// 完成压缩与专家构造").  Queries are then processed grouped by expert (same
// sections and the implementation remark on the second page).
//
//   k_route          (segment, head): R^T = Ql Q^T on MFMA (landmark rows x
//                    query columns), argmax with ties to the lower landmark,
//                    route_out, and the segment's per-expert counts.
//   k_theta_groups   (tiles, head): the top-k pre-threshold's group maxima
//                    (its selection runs as k_route's leading blocks).
// The counting sort that groups queries by expert is finished by the block
// bodies in mita_bucket.hpp, inside the landmark-scan and merge launches.
//
// Roofline: k_route streams Q (N*d*e bytes per head) — HBM-bound.
#include "mita_device.hpp"
#include "mita_internal.hpp"

namespace mita {

// row stride (elements) of the block's LDS copy of the landmark queries
constexpr int kQlStride = kD + 8;

template <class T>
struct RouteTraits;

template <>
struct RouteTraits<BF16> {
  using E = uint16_t;
  struct QReg {
    bf16x8 v[2];
  };
  __device__ static void load_q(QReg& b, const E* row, bool ok, int g) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x4 z = {0, 0, 0, 0};
      b.v[s] = as_bf16x8(ok ? *reinterpret_cast<const u32x4*>(row + 32 * s + 8 * g) : z);
    }
  }
  // landmark rows 16mt.. from LDS straight into one MFMA: R^T block mt
  __device__ static f32x4 logits_lds(const E* qls, int mt, const QReg& b, int c16, int g) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 2; ++s)
      acc = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(
                          qls + (16 * mt + c16) * kQlStride + 32 * s + 8 * g)),
                      b.v[s], acc);
    return acc;
  }
};

template <>
struct RouteTraits<F32> {
  using E = float;
  struct QReg {
    float v[16];
  };
  __device__ static void load_q(QReg& b, const E* row, bool ok, int g) {
#pragma unroll
    for (int s = 0; s < 16; ++s) b.v[s] = ok ? row[4 * s + g] : 0.f;
  }
  __device__ static f32x4 logits_lds(const E* qls, int mt, const QReg& b, int c16, int g) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 16; ++s)
      acc = mfma_f32(qls[(16 * mt + c16) * kQlStride + 4 * s + g], b.v[s], acc);
    return acc;
  }
};

// The top-k pre-threshold's selection, one wave per landmark lm of head bh:
// theta[bh][lm] = the k-th largest group maximum's score, lowered by one ulp
// so that the scan's strict test (s > theta) keeps every score equal to it;
// -inf when fewer than k maxima exist.  The k-th largest score comes from a
// bisection over the scores' 32-bit order (the upper half of the keys): the
// largest T with at least k maxima at or above T.  Each step counts per lane
// and sums the counts with one ballot per count bit, so the search stays
// uniform across the wave.  KPL: maxima per lane (groups <= 64 * KPL).
template <int KPL>
__device__ __forceinline__ void theta_select_wave(const uint32_t* __restrict__ gmax, int m, int k,
                                                  int groups, int mrows, int lm, int64_t bh,
                                                  float* __restrict__ theta) {
  const int l = lane_id();
  const uint32_t* G = gmax + (bh * m + lm) * groups;
  uint32_t v[KPL];  // 0: no maximum (below every real key's order bits)
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int i = 64 * j + l;
    v[j] = i < groups ? G[i] : 0u;
  }
  // invariant: at least k values >= lo (lo = 0 holds: 64 * KPL >= groups >= k)
  uint32_t lo = 0u, hi = 0xFFFFFFFFu;
  while (lo < hi) {
    const uint32_t mid = lo + ((hi - lo) >> 1) + 1u;
    // per-lane count (vector registers), then the wave total bit by bit:
    // one ballot per bit of the count instead of one per register
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) c += v[j] >= mid ? 1u : 0u;
    int cnt = 0;
#pragma unroll
    for (int b = 0; (1 << b) <= KPL; ++b) cnt += __popcll(ballot((c >> b) & 1u)) << b;
    if (cnt >= k)
      lo = mid;
    else
      hi = mid - 1u;
  }
  if (l == 0)
    theta[bh * mrows + lm] =
        lo != 0u ? nextafterf(key_score(static_cast<uint64_t>(lo) << 32), -INFINITY) : -INFINITY;
}

// the landmark queries of head bh into LDS (row stride kQlStride), rows past
// m zeroed; the caller's barrier publishes them
template <class E>
__device__ __forceinline__ void stage_landmarks(const E* __restrict__ Ql, int m, int64_t bh,
                                                E* __restrict__ qls) {
  constexpr int CH = 16 / sizeof(E);  // elements per 16-byte chunk
  for (int c = threadIdx.x; c < kMaxM * (kD / CH); c += 256) {
    const int row = c / (kD / CH), col = c % (kD / CH);
    const u32x4 z = {0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(qls + row * kQlStride + col * CH) =
        row < m ? *reinterpret_cast<const u32x4*>(Ql + (bh * m + row) * kD + col * CH) : z;
  }
}

// One routing block (256 threads) routes queries seg*SEG + [0, SEG) of head
// bh (SEG = 1024 or 256) in groups of 16; wave w takes groups w, w + 4,
// w + 8, ... (so a short head keeps all four waves busy), four groups of Q
// rows in flight, and the block stores the segment's per-expert counts.
template <class T, int SEG>
__device__ __forceinline__ void route_segment(const typename T::elem* __restrict__ Q,
                                              const typename T::elem* __restrict__ Ql,
                                              int64_t N, int m, int nseg, int seg, int64_t bh,
                                              int32_t* __restrict__ route_out,
                                              int32_t* __restrict__ counts, int* cnt,
                                              typename T::elem* qls) {
  using TR = RouteTraits<T>;
  using E = typename T::elem;
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  if (threadIdx.x < kMaxM) cnt[threadIdx.x] = 0;
  stage_landmarks(Ql, m, bh, qls);
  const E* Qh = Q + bh * N * kD;
  // group G of this wave: queries qw + 64 G + [0, 16)
  const int64_t qw = static_cast<int64_t>(seg) * SEG + 16 * w;
  // a ring of D groups of 16 queries in flight
  constexpr int D = 4, NG = SEG / 64;
  // unconditional loads of a clamped row (results past N are never used):
  // branch-free, so the compiler's wait counts stay exact
  auto load_group = [&](int G, typename TR::QReg& dst) {
    const int64_t qq = qw + 64 * G + c16;
    TR::load_q(dst, Qh + (qq < N ? qq : N - 1) * kD, true, g);
  };
  typename TR::QReg ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) load_group(j, ring[j]);
  __syncthreads();  // landmark rows and counters staged
  const int mtiles = (m + 15) >> 4;
  // bf16: the landmark operands held in registers for the whole segment
  // (32 VGPRs, 5 waves per SIMD instead of 8; routing at 2^20 tokens x 4
  // heads 110.6 -> 108.7 us, 30.6 -> 29.7 us at 2^18, against re-reading
  // them from LDS for every group)
  bf16x8 la[4][2];
  if constexpr (sizeof(E) == 2) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        la[mt][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(
            reinterpret_cast<const uint16_t*>(qls) + (16 * mt + c16) * kQlStride + 32 * s + 8 * g));
  }
  // fully unrolled, so that each group's wait covers exactly its own rows
  // (a rolled ring loop makes the compiler wait for every group in flight)
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    if (qw + 64 * G >= N) break;
    {
      const int j = G % D;
      if constexpr (sizeof(E) != 2) __asm__ volatile("" ::: "memory");  // re-read the landmark operands
      float best = -INFINITY;
      int bi = 0;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt < mtiles) {
          f32x4 r4;
          if constexpr (sizeof(E) == 2) {
            r4 = mfma_bf16(la[mt][0], ring[j].v[0], f32x4{0, 0, 0, 0});
            r4 = mfma_bf16(la[mt][1], ring[j].v[1], r4);
          } else {
            r4 = TR::logits_lds(qls, mt, ring[j], c16, g);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int lmi = 16 * mt + 4 * g + r;  // increasing within the lane
            const bool better = lmi < m && r4[r] > best;
            best = better ? r4[r] : best;
            bi = better ? lmi : bi;
          }
        }
      }
      // combine the 4 lane groups holding this query: larger value, then
      // lower landmark index
      xor_argmax(best, bi, 16);
      xor_argmax(best, bi, 32);
      if (G + D < NG) load_group(G + D, ring[j]);
      const int64_t q = qw + 64 * G + c16;
      if (g == 0 && q < N) {
        route_out[bh * N + q] = bi;
        atomicAdd(&cnt[bi], 1);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < m) counts[(bh * m + threadIdx.x) * nseg + seg] = cnt[threadIdx.x];  // expert-major
}

// grid (nsel + nseg, BH), 256 threads (fp32 inputs, or no pre-threshold).
//  - blocks x < nsel (KPL > 0): the pre-threshold selection over the group
//    maxima of the separate group kernel, wave w of block x for landmark
//    4x + w (nsel = ceil(m / 4)).  They come first in the grid, so they are
//    dispatched before the routing blocks, and the scan, which follows on
//    the same stream, finds theta ready.
//  - the other blocks route, from the end of the heads' queries backwards:
//    pooling has just read Q front to back, so the first rows routed are
//    the ones most recently read (measured: about 1% faster than front to
//    back at 2^18 and 2^20 tokens; the last-level cache returns little of Q).
template <class T, int KPL, int SEG>
__global__ __launch_bounds__(256) void k_route(const typename T::elem* __restrict__ Q,
                                              const typename T::elem* __restrict__ Ql, int64_t N,
                                              int m, int nseg, int32_t* __restrict__ route_out,
                                              int32_t* __restrict__ counts, int nsel,
                                              const uint32_t* __restrict__ gmax, int k,
                                              int groups, int mrows,
                                              float* __restrict__ theta) {
  using E = typename T::elem;
  __shared__ int cnt[kMaxM];
  __shared__ __attribute__((aligned(16))) E qls[kMaxM * kQlStride];
  if constexpr (KPL > 0) {
    if (static_cast<int>(blockIdx.x) < nsel) {  // whole block
      const int lm = static_cast<int>(blockIdx.x) * 4 +
                     __builtin_amdgcn_readfirstlane(wave_id());
      if (lm < m) theta_select_wave<KPL>(gmax, m, k, groups, mrows, lm, blockIdx.y, theta);
      return;
    }
  }
  const int seg = nseg - 1 - (static_cast<int>(blockIdx.x) - (KPL > 0 ? nsel : 0));
  route_segment<T, SEG>(Q, Ql, N, m, nseg, seg, gridDim.y - 1 - blockIdx.y, route_out, counts,
                        cnt, qls);
}

// Several experts per query (s > 1, bf16): block (segment, head) covers
// assignments seg * kRouteSeg + [0, kRouteSeg) of the head's flattened
// [N][s] expert list, i.e. the queries whose assignments fall there.  A
// query's s experts are its s largest logits q . Ql[i], best first, ties to
// the lower landmark (s rounds of argmax, each dropping the landmark it took)
// — the reading of the pages' several-experts-per-query routing that the
// oracle's route_s follows ("Mixture-of-Top-k 注意力…", section "MiTA：用少量
// 地标查询，同时完成压缩与专家构造", s experts per query; the experiments use
// s = 1).  Only the assignments inside the segment are stored and counted
// (expert-major counts per segment, as k_route's), so the counting sort of
// step 4 runs over the N*s assignments unchanged.  Leading blocks: the
// pre-threshold selection, as in k_route.
template <int KPL>
__global__ __launch_bounds__(256) void k_route_s(const uint16_t* __restrict__ Q,
                                                const uint16_t* __restrict__ Ql, int64_t N, int m,
                                                int s, int nseg, int32_t* __restrict__ routes,
                                                int32_t* __restrict__ counts, int nsel,
                                                const uint32_t* __restrict__ gmax, int k,
                                                int groups, int mrows,
                                                float* __restrict__ theta) {
  using TR = RouteTraits<BF16>;
  __shared__ int cnt[kMaxM];
  __shared__ __attribute__((aligned(16))) uint16_t qls[kMaxM * kQlStride];
  if constexpr (KPL > 0) {
    if (static_cast<int>(blockIdx.x) < nsel) {  // whole block
      const int lm = static_cast<int>(blockIdx.x) * 4 +
                     __builtin_amdgcn_readfirstlane(wave_id());
      if (lm < m) theta_select_wave<KPL>(gmax, m, k, groups, mrows, lm, blockIdx.y, theta);
      return;
    }
  }
  const int seg = static_cast<int>(blockIdx.x) - (KPL > 0 ? nsel : 0);
  const int64_t bh = blockIdx.y;
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  if (threadIdx.x < kMaxM) cnt[threadIdx.x] = 0;
  stage_landmarks(Ql, m, bh, qls);
  __syncthreads();
  const int64_t NA = N * s;
  const int64_t a0 = static_cast<int64_t>(seg) * kRouteSeg;
  const int64_t a1 = a0 + kRouteSeg < NA ? a0 + kRouteSeg : NA;
  const int64_t q0 = a0 / s, q1 = (a1 - 1) / s + 1;  // queries with an assignment here
  const int mtiles = (m + 15) >> 4;
  const uint16_t* Qh = Q + bh * N * kD;
  for (int64_t qg = q0 + 16 * w; qg < q1; qg += 64) {  // 16 queries per wave and step
    const int64_t q = qg + c16;
    TR::QReg b;
    TR::load_q(b, Qh + (q < N ? q : N - 1) * kD, true, g);
    float v[4][4];  // logits of landmarks 16 mt + 4g + r
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 r4 = {0, 0, 0, 0};
      if (mt < mtiles) r4 = TR::logits_lds(qls, mt, b, c16, g);
#pragma unroll
      for (int r = 0; r < 4; ++r) v[mt][r] = (mt < mtiles && 16 * mt + 4 * g + r < m) ? r4[r] : -INFINITY;
    }
    for (int j = 0; j < s; ++j) {
      float best = -INFINITY;
      int bi = 0;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool better = v[mt][r] > best;  // increasing landmark order in the lane
          best = better ? v[mt][r] : best;
          bi = better ? 16 * mt + 4 * g + r : bi;
        }
      xor_argmax(best, bi, 16);
      xor_argmax(best, bi, 32);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * mt + 4 * g + r == bi) v[mt][r] = -INFINITY;  // taken
      const int64_t a = q * s + j;
      if (g == 0 && q < q1 && a >= a0 && a < a1) {
        routes[bh * NA + a] = bi;
        atomicAdd(&cnt[bi], 1);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < m) counts[(bh * m + threadIdx.x) * nseg + seg] = cnt[threadIdx.x];
}

// The pre-threshold's group maxima of one 64-key tile of head bh (bf16), one
// wave: the tile is scored against every landmark (operands from the LDS
// copy of the landmark queries), and the maximum key of each group of GS
// keys is stored.  SAMPLED: tile ti of `groups` evenly spaced sample tiles,
// one group per tile.  Else tile ti of the head in groups of GS keys (1:
// every key its own group; 16: 16-key blocks; 64: the tile).  Rows past N
// read row N - 1: every load is unconditional; those scores are dropped.
// The scores use the scan's operand layout and accumulation order, so they
// are bitwise the scores the scan computes.  The tile's key operands (ko)
// come from theta_tile_load, issued by the caller before it waits for the
// landmark staging.
template <bool SAMPLED>
__device__ __forceinline__ int64_t theta_tile_start(int64_t N, int groups, int ti) {
  const int64_t ntiles = (N + kTileKeys - 1) / kTileKeys;
  return SAMPLED ? ((static_cast<int64_t>(ti) * ntiles) / groups) * kTileKeys
                 : static_cast<int64_t>(ti) * kTileKeys;
}

template <bool SAMPLED>
__device__ __forceinline__ void theta_tile_load(const uint16_t* __restrict__ K, int64_t N,
                                                int groups, int ti, int64_t bh, u32x4 (&ko)[4][2]) {
  const int l = lane_id(), g = l >> 4, c16 = l & 15;
  const int64_t t0 = theta_tile_start<SAMPLED>(N, groups, ti);
  const uint16_t* Kh = K + bh * N * kD;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int64_t row = t0 + 16 * kb + c16;
    const int64_t rr = row < N ? row : N - 1;
#pragma unroll
    for (int s = 0; s < 2; ++s)
      ko[kb][s] = *reinterpret_cast<const u32x4*>(Kh + rr * kD + 32 * s + 8 * g);
  }
}

template <int GS, bool SAMPLED>
__device__ __forceinline__ void theta_tile_wave(const u32x4 (&ko)[4][2], const uint16_t* qls,
                                                int64_t N, int m, int groups, int ti, int64_t bh,
                                                uint32_t* __restrict__ gmax) {
  static_assert(GS == 1 || GS == 16 || GS == 64, "groups of 1, 16 or 64 keys");
  static_assert(!SAMPLED || GS == 64, "samples are whole tiles");
  const int l = lane_id(), g = l >> 4, c16 = l & 15;
  const int64_t t0 = theta_tile_start<SAMPLED>(N, groups, ti);
#pragma unroll
  for (int lb = 0; lb < 4; ++lb) {
    if (16 * lb >= m) break;  // uniform
    const uint16_t* qrow = qls + (16 * lb + c16) * kQlStride + 8 * g;
    const u32x4 q0 = *reinterpret_cast<const u32x4*>(qrow);
    const u32x4 q1 = *reinterpret_cast<const u32x4*>(qrow + 32);
    f32x4 sc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      sc[kb] = mfma_bf16(as_bf16x8(ko[kb][0]), as_bf16x8(q0), f32x4{0, 0, 0, 0});
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sc[kb] = mfma_bf16(as_bf16x8(ko[kb][1]), as_bf16x8(q1), sc[kb]);
    const int lm = 16 * lb + c16;
    uint32_t* G = gmax + (bh * m + (lm < m ? lm : 0)) * groups;
    uint64_t best = 0;  // running group maximum (GS = 16, 64)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + 16 * kb + 4 * g + r;
        const uint64_t key = t < N ? make_key(sc[kb][r], static_cast<uint32_t>(t)) : 0ull;
        if constexpr (GS == 1) {
          if (lm < m && t < N) G[t] = static_cast<uint32_t>(key >> 32);
        } else {
          best = key > best ? key : best;
        }
      }
      if constexpr (GS != 1) {
        if (GS == 16 || kb == 3) {  // end of a group: combine the 4 lane groups
#pragma unroll
          for (int mask = 16; mask <= 32; mask <<= 1) {
            const uint64_t o = lane_read(best, l ^ mask);
            best = o > best ? o : best;
          }
          const int64_t gi = GS == 16 ? (t0 >> 4) + kb : static_cast<int64_t>(ti);
          if (g == 0 && lm < m && gi < groups) G[gi] = static_cast<uint32_t>(best >> 32);
          best = 0;
        }
      }
    }
  }
}

// The pre-threshold's group maxima (bf16): grid (ceil(tiles / 4), BH), 256
// threads, wave w: tile 4x + w, scored against the block's LDS copy of the
// landmark queries.  Its own launch before routing: inside the routing
// launch, the selection would have to wait across blocks for every tile of
// the head, and the device-scope fences and polls that takes cost routing
// more than this launch does.  The key tile is requested before the
// landmark staging, so the two memory latencies overlap.  Rows are clamped,
// so a wave past the last tile loads in bounds and stores nothing.
template <int GS, bool SAMPLED>
__global__ __launch_bounds__(256) void k_theta_groups(const uint16_t* __restrict__ K,
                                                     const uint16_t* __restrict__ Ql, int64_t N,
                                                     int m, int groups,
                                                     uint32_t* __restrict__ gmax) {
  __shared__ __attribute__((aligned(16))) uint16_t qls[kMaxM * kQlStride];
  const int64_t bh = blockIdx.y;
  const int ti = static_cast<int>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(wave_id());
  const int64_t ntiles = (N + kTileKeys - 1) / kTileKeys;
  u32x4 ko[4][2];
  theta_tile_load<SAMPLED>(K, N, groups, ti, bh, ko);
  stage_landmarks(Ql, m, bh, qls);
  __syncthreads();
  if (ti < (SAMPLED ? groups : ntiles))
    theta_tile_wave<GS, SAMPLED>(ko, qls, N, m, groups, ti, bh, gmax);
}

template <class T, int SEG>
static hipError_t launch_route_seg(const Shape& s, const void* Q, const Workspace& ws,
                                 int32_t* route_out, hipStream_t st) {
  using E = typename T::elem;
  const E* Qp = static_cast<const E*>(Q);
  const E* Qlp = static_cast<const E*>(ws.ql);
  if (s.theta_groups > 64 * 64) return hipErrorInvalidValue;  // beyond the selection's registers
  const int nsel = s.theta_groups > 0 ? (s.m + 3) / 4 : 0;
  const dim3 grid(nsel + s.nseg, s.BH);
  // maxima per lane in the selection: the fewest that hold every group
  if (nsel == 0)
    hipLaunchKernelGGL((k_route<T, 0, SEG>), grid, dim3(256), 0, st, Qp, Qlp, s.N, s.m, s.nseg,
                       route_out, ws.counts, 0, nullptr, s.k, 0, s.mrows, nullptr);
  else if (s.theta_groups <= 64 * 4)
    hipLaunchKernelGGL((k_route<T, 4, SEG>), grid, dim3(256), 0, st, Qp, Qlp, s.N, s.m, s.nseg,
                       route_out, ws.counts, nsel, ws.gmax, s.k, s.theta_groups, s.mrows,
                       ws.theta);
  else if (s.theta_groups <= 64 * 16)
    hipLaunchKernelGGL((k_route<T, 16, SEG>), grid, dim3(256), 0, st, Qp, Qlp, s.N, s.m, s.nseg,
                       route_out, ws.counts, nsel, ws.gmax, s.k, s.theta_groups, s.mrows,
                       ws.theta);
  else if (s.theta_groups <= 64 * 32)
    hipLaunchKernelGGL((k_route<T, 32, SEG>), grid, dim3(256), 0, st, Qp, Qlp, s.N, s.m, s.nseg,
                       route_out, ws.counts, nsel, ws.gmax, s.k, s.theta_groups, s.mrows,
                       ws.theta);
  else
    hipLaunchKernelGGL((k_route<T, 64, SEG>), grid, dim3(256), 0, st, Qp, Qlp, s.N, s.m, s.nseg,
                       route_out, ws.counts, nsel, ws.gmax, s.k, s.theta_groups, s.mrows,
                       ws.theta);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_route_t(const Shape& s, const void* Q, const Workspace& ws,
                                 int32_t* route_out, hipStream_t st) {
  return s.rseg == kRouteSegSmall ? launch_route_seg<T, kRouteSegSmall>(s, Q, ws, route_out, st)
                                  : launch_route_seg<T, kRouteSeg>(s, Q, ws, route_out, st);
}

template <int GS, bool SAMPLED>
static void launch_groups_gs(const Shape& s, const void* K, const Workspace& ws, int nth,
                             hipStream_t st) {
  hipLaunchKernelGGL((k_theta_groups<GS, SAMPLED>), dim3(nth, s.BH), dim3(256), 0, st,
                     static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(ws.ql), s.N,
                     s.m, s.theta_groups, ws.gmax);
}

hipError_t launch_groups_bf16(const Shape& s, const void* K, const Workspace& ws, hipStream_t st) {
  const int64_t ktiles = (s.N + kTileKeys - 1) / kTileKeys;
  const int nth = static_cast<int>(((s.theta_sampled ? s.theta_groups : ktiles) + 3) / 4);
  if (s.theta_sampled)
    launch_groups_gs<64, true>(s, K, ws, nth, st);
  else if (s.theta_gs == 1)
    launch_groups_gs<1, false>(s, K, ws, nth, st);
  else if (s.theta_gs == 16)
    launch_groups_gs<16, false>(s, K, ws, nth, st);
  else
    launch_groups_gs<64, false>(s, K, ws, nth, st);
  return hipGetLastError();
}

hipError_t launch_route_s(const Shape& s, const void* Q, const Workspace& ws, int32_t* routes,
                          hipStream_t st) {
  const uint16_t* Qp = static_cast<const uint16_t*>(Q);
  const uint16_t* Qlp = static_cast<const uint16_t*>(ws.ql);
  if (s.dtype != 1 || s.theta_groups > 64 * 64) return hipErrorInvalidValue;
  const int nsel = s.theta_groups > 0 ? (s.m + 3) / 4 : 0;
  const dim3 grid(nsel + s.nseg, s.BH);
  if (nsel == 0)
    hipLaunchKernelGGL((k_route_s<0>), grid, dim3(256), 0, st, Qp, Qlp, s.N, s.m, s.s, s.nseg,
                       routes, ws.counts, 0, nullptr, s.k, 0, s.mrows, nullptr);
  else if (s.theta_groups <= 64 * 4)
    hipLaunchKernelGGL((k_route_s<4>), grid, dim3(256), 0, st, Qp, Qlp, s.N, s.m, s.s, s.nseg,
                       routes, ws.counts, nsel, ws.gmax, s.k, s.theta_groups, s.mrows, ws.theta);
  else if (s.theta_groups <= 64 * 16)
    hipLaunchKernelGGL((k_route_s<16>), grid, dim3(256), 0, st, Qp, Qlp, s.N, s.m, s.s, s.nseg,
                       routes, ws.counts, nsel, ws.gmax, s.k, s.theta_groups, s.mrows, ws.theta);
  else if (s.theta_groups <= 64 * 32)
    hipLaunchKernelGGL((k_route_s<32>), grid, dim3(256), 0, st, Qp, Qlp, s.N, s.m, s.s, s.nseg,
                       routes, ws.counts, nsel, ws.gmax, s.k, s.theta_groups, s.mrows, ws.theta);
  else
    hipLaunchKernelGGL((k_route_s<64>), grid, dim3(256), 0, st, Qp, Qlp, s.N, s.m, s.s, s.nseg,
                       routes, ws.counts, nsel, ws.gmax, s.k, s.theta_groups, s.mrows, ws.theta);
  return hipGetLastError();
}

hipError_t launch_route(const Shape& s, const void* Q, const Workspace& ws, int32_t* route_out,
                        hipStream_t st) {
  return s.dtype == 1 ? launch_route_t<BF16>(s, Q, ws, route_out, st)
                      : launch_route_t<F32>(s, Q, ws, route_out, st);
}

}  // namespace mita
