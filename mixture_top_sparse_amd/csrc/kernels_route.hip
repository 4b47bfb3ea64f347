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
//   k_bucket_scan    (expert, head): prefix of the expert's per-segment counts
//                    over the segments, and the expert's total.
//   k_bucket_scatter (segment, head), one wave: expert offsets from the
//                    totals, then a stable counting sort of the segment in
//                    LDS (a query's rank among equal routes inside a group
//                    of 64 comes from 6 ballots over the route bits), copied
//                    out one expert run at a time.  Segment 0 publishes the
//                    offsets and the first attention work item of each expert.
//
// Roofline: k_route streams Q (N*d*e bytes per head) — HBM-bound; the
// bucket kernels move ~16 bytes per query.
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

// grid (nseg, BH), 256 threads; wave w routes queries seg*1024 + 256w + [0, 256)
// in 16 groups of 16 queries, four groups of Q rows in flight
template <class T>
__global__ __launch_bounds__(256) void k_route(const typename T::elem* __restrict__ Q,
                                              const typename T::elem* __restrict__ Ql, int64_t N,
                                              int m, int nseg, int64_t bh0,
                                              int32_t* __restrict__ route_out,
                                              int32_t* __restrict__ counts) {
  using TR = RouteTraits<T>;
  using E = typename T::elem;
  __shared__ int cnt[kMaxM];
  __shared__ __attribute__((aligned(16))) E qls[kMaxM * kQlStride];
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  // blocks run from the end of the heads' queries backwards: pooling has just
  // read Q front to back, so the first rows routed are still in the last-level
  // cache
  const int seg = nseg - 1 - static_cast<int>(blockIdx.x);
  const int64_t bh = bh0 + (gridDim.y - 1 - blockIdx.y);
  if (threadIdx.x < kMaxM) cnt[threadIdx.x] = 0;
  {  // the landmark queries once per block, zero rows past m
    constexpr int CH = 16 / sizeof(E);  // elements per 16-byte chunk
    for (int c = threadIdx.x; c < kMaxM * (kD / CH); c += 256) {
      const int row = c / (kD / CH), col = c % (kD / CH);
      const u32x4 z = {0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(qls + row * kQlStride + col * CH) =
          row < m ? *reinterpret_cast<const u32x4*>(Ql + (bh * m + row) * kD + col * CH) : z;
    }
  }
  const E* Qh = Q + bh * N * kD;
  const int64_t qw = static_cast<int64_t>(seg) * kRouteSeg + 256 * w;
  // a ring of D groups of 16 queries in flight; the landmark operands are
  // read from LDS for every group (not pinned in registers: occupancy)
  constexpr int D = 4, NG = 16;
  // unconditional loads of a clamped row (results past N are never used):
  // branch-free, so the compiler's wait counts stay exact
  auto load_group = [&](int G, typename TR::QReg& dst) {
    const int64_t qq = qw + 16 * G + c16;
    TR::load_q(dst, Qh + (qq < N ? qq : N - 1) * kD, true, g);
  };
  typename TR::QReg ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) load_group(j, ring[j]);
  __syncthreads();  // landmark rows and counters staged
  const int mtiles = (m + 15) >> 4;
  // fully unrolled, so that each group's wait covers exactly its own rows
  // (a rolled ring loop makes the compiler wait for every group in flight)
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    if (qw + 16 * G >= N) break;
    {
      const int j = G % D;
      __asm__ volatile("" ::: "memory");  // re-read the landmark operands
      float best = -INFINITY;
      int bi = 0;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt < mtiles) {
          const f32x4 r4 = TR::logits_lds(qls, mt, ring[j], c16, g);
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
      const int64_t q = qw + 16 * G + c16;
      if (g == 0 && q < N) {
        route_out[bh * N + q] = bi;
        atomicAdd(&cnt[bi], 1);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < m) counts[(bh * m + threadIdx.x) * nseg + seg] = cnt[threadIdx.x];  // expert-major
}

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = static_cast<int>(lane_read(static_cast<uint32_t>(v), l >= d ? l - d : l));
    if (l >= d) v += o;
  }
  return v;
}

// grid (m, BH), 256 threads: for expert e, the exclusive prefix of its
// per-segment counts over the segments (colpre) and its total
__global__ __launch_bounds__(256) void k_bucket_scan(const int32_t* __restrict__ counts, int m,
                                                     int nseg, int32_t* __restrict__ colpre,
                                                     int32_t* __restrict__ totals) {
  __shared__ int wsum[4];
  const int e = blockIdx.x, t = threadIdx.x, l = lane_id(), w = wave_id();
  const int64_t bh = blockIdx.y;
  const int32_t* C = counts + (bh * m + e) * nseg;
  int32_t* P = colpre + (bh * m + e) * nseg;
  const int per = (nseg + 255) / 256;  // contiguous segments per thread
  const int s0 = t * per, s1 = min(s0 + per, nseg);
  int sum = 0;
  for (int s = s0; s < s1; ++s) sum += C[s];
  const int incl = wave_inclusive_sum(sum);
  if (l == 63) wsum[w] = incl;
  __syncthreads();
  int run = incl - sum;
  for (int v = 0; v < w; ++v) run += wsum[v];
  for (int s = s0; s < s1; ++s) {
    const int c = C[s];
    P[s] = run;
    run += c;
  }
  if (t == 255) totals[bh * m + e] = run;
}

// grid (nseg, BH), 64 threads: stable scatter of one segment's queries.
// Expert offsets come from the per-expert totals (exclusive scan over the m
// experts); segment 0 also publishes offsets and the attention work items.
// The segment is first sorted by route in LDS (ranks from ballots, bases
// from the routing kernel's per-segment counts); the sorted list is then
// copied out run by run, so consecutive lanes store consecutive positions of
// an expert's range instead of one lane per expert region.  Consecutive
// segments are taken by blocks on one XCD (groups of four), so the partial
// lines they leave at the ends of each run meet in one L2.
__global__ __launch_bounds__(64) void k_bucket_scatter(
    const int32_t* __restrict__ route, const int32_t* __restrict__ counts, int m, int nseg,
    int64_t N, int tile, int tpb, const int32_t* __restrict__ totals,
    const int32_t* __restrict__ colpre, int32_t* __restrict__ offsets,
    int32_t* __restrict__ offsets_copy, int32_t* __restrict__ item_start,
    int32_t* __restrict__ perm, int32_t* __restrict__ perm_copy) {
  constexpr int R = 4;  // consecutive segments per XCD
  __shared__ int lbase[kMaxM];   // next local slot of each expert
  __shared__ int gshift[kMaxM];  // global position minus local slot, per expert
  __shared__ int32_t sq[kRouteSeg];
  __shared__ uint8_t se[kRouteSeg];
  const int l = threadIdx.x;
  int seg = blockIdx.x;
  {  // blocks are dispatched to the XCDs round-robin: b -> XCD b % 8
    const int n = gridDim.x, full = n / (8 * R) * (8 * R), b = blockIdx.x;
    if (b < full) seg = ((b / 8 / R) * 8 + b % 8) * R + (b / 8) % R;
  }
  const int64_t bh = blockIdx.y;
  const int c = l < m ? totals[bh * m + l] : 0;
  const int incl = wave_inclusive_sum(c);
  if (seg == 0) {
    const int items = ((c + tile - 1) / tile + tpb - 1) / tpb;
    const int incl_items = wave_inclusive_sum(items);
    int32_t* O = offsets + bh * (m + 1);
    int32_t* I = item_start + bh * (m + 1);
    if (l < m) {
      O[l] = incl - c;
      I[l] = incl_items - items;
      if (offsets_copy) offsets_copy[bh * (m + 1) + l] = incl - c;
    }
    if (l == m - 1) {
      O[m] = incl;
      I[m] = incl_items;
      if (offsets_copy) offsets_copy[bh * (m + 1) + m] = incl;
    }
  }
  // all of the segment's routes in flight at once
  constexpr int NG = kRouteSeg / 64;
  const int64_t q0 = static_cast<int64_t>(seg) * kRouteSeg;
  const int nq = static_cast<int>(N - q0 < kRouteSeg ? N - q0 : kRouteSeg);
  int rr[NG];
#pragma unroll
  for (int it = 0; it < NG; ++it) {
    const int64_t q = q0 + 64 * it + l;
    rr[it] = q < N ? route[bh * N + q] : 0;
  }
  {
    const int cl = l < m ? counts[(bh * m + l) * nseg + seg] : 0;
    const int lex = wave_inclusive_sum(cl) - cl;  // local start of expert l
    if (l < m) {
      lbase[l] = lex;
      gshift[l] = (incl - c) + colpre[(bh * m + l) * nseg + seg] - lex;
    }
  }
  // one wave: its LDS accesses complete in program order, no barriers needed
  const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));
#pragma unroll
  for (int it = 0; it < NG; ++it) {
    if (64 * it >= nq) break;
    const bool ok = 64 * it + l < nq;
    int r = rr[it];
    r = r < 0 ? 0 : (r >= m ? m - 1 : r);  // routes come from k_route; clamp defensively
    uint64_t same = ballot(ok);
#pragma unroll
    for (int b = 0; b < 6; ++b) {  // m <= 64: routes fit in 6 bits
      const bool bit = (r >> b) & 1;
      const uint64_t bb = ballot(bit);
      same &= bit ? bb : ~bb;
    }
    const int rank = __popcll(same & below);
    const int total = __popcll(same);
    const int pos = ok ? lbase[r] + rank : -1;
    if (pos >= 0 && pos < kRouteSeg) {
      sq[pos] = static_cast<int32_t>(q0 + 64 * it + l);
      se[pos] = static_cast<uint8_t>(r);
    }
    if (ok && rank == total - 1) lbase[r] += total;  // after every lane's read of lbase[r]
  }
  // copy out in sorted order: lanes l, l+1 of one expert run store adjacent
  // positions
  for (int i = l; i < nq; i += 64) {
    const int e = se[i];
    const int pos = e < m ? gshift[e] + i : -1;
    if (pos >= 0 && pos < N) {
      perm[bh * N + pos] = sq[i];
      if (perm_copy) perm_copy[bh * N + pos] = sq[i];
    }
  }
}

template <class T>
static hipError_t launch_route_t(const Shape& s, const void* Q, const Workspace& ws,
                                 int32_t* route_out, int64_t bh0, int64_t nbh, hipStream_t st) {
  using E = typename T::elem;
  hipLaunchKernelGGL(k_route<T>, dim3(s.nseg, nbh), dim3(256), 0, st, static_cast<const E*>(Q),
                     static_cast<const E*>(ws.ql), s.N, s.m, s.nseg, bh0, route_out, ws.counts);
  return hipGetLastError();
}

hipError_t launch_route(const Shape& s, const void* Q, const Workspace& ws, int32_t* route_out,
                        int64_t bh0, int64_t nbh, hipStream_t st) {
  return s.dtype == 1 ? launch_route_t<BF16>(s, Q, ws, route_out, bh0, nbh, st)
                      : launch_route_t<F32>(s, Q, ws, route_out, bh0, nbh, st);
}

hipError_t launch_bucket(const Shape& s, const int32_t* route, const Workspace& ws,
                         int32_t* offsets_copy, int32_t* perm_copy, hipStream_t st) {
  hipLaunchKernelGGL(k_bucket_scan, dim3(s.m, s.BH), dim3(256), 0, st, ws.counts, s.m, s.nseg,
                     ws.colpre, ws.totals);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_bucket_scatter, dim3(s.nseg, s.BH), dim3(64), 0, st, route, ws.counts,
                     s.m, s.nseg, s.N, kAttendTile, s.attend_tpb, ws.totals, ws.colpre, ws.offsets,
                     offsets_copy, ws.item_start, ws.perm, perm_copy);
  return hipGetLastError();
}

}  // namespace mita
