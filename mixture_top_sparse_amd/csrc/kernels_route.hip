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
//   k_bucket_scan    (head): expert totals -> offsets, per-(segment, expert)
//                    bases, and the first attention work item of each expert.
//   k_bucket_scatter (segment, head), one wave: stable counting-sort scatter;
//                    a query's rank among equal routes inside a group of 64
//                    comes from 6 ballots over the route bits.
//
// Roofline: k_route streams Q (N*d*e bytes per head) — HBM-bound; the
// bucket kernels move ~16 bytes per query.
#include "mita_device.hpp"
#include "mita_internal.hpp"

namespace mita {

template <class T>
struct RouteTraits;

template <>
struct RouteTraits<BF16> {
  using E = uint16_t;
  struct QlReg {
    bf16x8 v[4][2];
  };
  struct QReg {
    bf16x8 v[2];
  };
  __device__ static void load_ql(QlReg& a, const E* Qlh, int m, int c16, int g) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int lm = 16 * mt + c16;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u32x4 z = {0, 0, 0, 0};
        a.v[mt][s] = as_bf16x8(
            lm < m ? *reinterpret_cast<const u32x4*>(Qlh + lm * kD + 32 * s + 8 * g) : z);
      }
    }
  }
  __device__ static void load_q(QReg& b, const E* row, bool ok, int g) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x4 z = {0, 0, 0, 0};
      b.v[s] = as_bf16x8(ok ? *reinterpret_cast<const u32x4*>(row + 32 * s + 8 * g) : z);
    }
  }
  __device__ static f32x4 logits(const QlReg& a, int mt, const QReg& b) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 2; ++s) acc = mfma_bf16(a.v[mt][s], b.v[s], acc);
    return acc;
  }
};

template <>
struct RouteTraits<F32> {
  using E = float;
  struct QlReg {
    float v[4][16];
  };
  struct QReg {
    float v[16];
  };
  __device__ static void load_ql(QlReg& a, const E* Qlh, int m, int c16, int g) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int lm = 16 * mt + c16;
#pragma unroll
      for (int s = 0; s < 16; ++s) a.v[mt][s] = lm < m ? Qlh[lm * kD + 4 * s + g] : 0.f;
    }
  }
  __device__ static void load_q(QReg& b, const E* row, bool ok, int g) {
#pragma unroll
    for (int s = 0; s < 16; ++s) b.v[s] = ok ? row[4 * s + g] : 0.f;
  }
  __device__ static f32x4 logits(const QlReg& a, int mt, const QReg& b) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 16; ++s) acc = mfma_f32(a.v[mt][s], b.v[s], acc);
    return acc;
  }
};

// grid (nseg, BH), 256 threads; wave w routes queries seg*1024 + 256w + [0, 256)
template <class T>
__global__ __launch_bounds__(256) void k_route(const typename T::elem* __restrict__ Q,
                                              const typename T::elem* __restrict__ Ql, int64_t N,
                                              int m, int nseg, int32_t* __restrict__ route_out,
                                              int32_t* __restrict__ counts) {
  using TR = RouteTraits<T>;
  __shared__ int cnt[kMaxM];
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int seg = blockIdx.x;
  const int64_t bh = blockIdx.y;
  if (threadIdx.x < kMaxM) cnt[threadIdx.x] = 0;
  typename TR::QlReg a;
  TR::load_ql(a, Ql + bh * m * kD, m, c16, g);
  const int mtiles = (m + 15) >> 4;
  __syncthreads();

  const typename T::elem* Qh = Q + bh * N * kD;
  for (int it = 0; it < 4; ++it) {
    const int64_t q0 = static_cast<int64_t>(seg) * kRouteSeg + 256 * w + 64 * it;
    if (q0 >= N) break;
    int rsel = 0;
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const int64_t qq = q0 + 16 * G + c16;
      typename TR::QReg b;
      TR::load_q(b, Qh + (qq < N ? qq : 0) * kD, qq < N, g);
      float best = -INFINITY;
      int bi = 0;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt < mtiles) {
          const f32x4 r4 = TR::logits(a, mt, b);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int lmi = 16 * mt + 4 * g + r;  // increasing within the lane
            if (lmi < m && r4[r] > best) {
              best = r4[r];
              bi = lmi;
            }
          }
        }
      }
      // combine the 4 lane groups holding this query: larger value, then
      // lower landmark index
#pragma unroll
      for (int mask = 16; mask <= 32; mask <<= 1) {
        const float ob = lane_read(best, l ^ mask);
        const int oi = static_cast<int>(lane_read(static_cast<uint32_t>(bi), l ^ mask));
        if (ob > best || (ob == best && oi < bi)) {
          best = ob;
          bi = oi;
        }
      }
      if (G == g) rsel = bi;  // lane l = 16G + c16 keeps query q0 + l
    }
    const int64_t q = q0 + l;
    if (q < N) {
      route_out[bh * N + q] = rsel;
      atomicAdd(&cnt[rsel], 1);
    }
  }
  __syncthreads();
  if (threadIdx.x < m) counts[(bh * nseg + seg) * m + threadIdx.x] = cnt[threadIdx.x];
}

// grid (BH), 1024 threads: thread (e = t % 64, part = t / 64) handles expert
// e over segments [part*nseg/16, (part+1)*nseg/16)
__global__ __launch_bounds__(1024) void k_bucket_scan(const int32_t* __restrict__ counts, int m,
                                                     int nseg, int64_t N, int tile, int tpb,
                                                     int32_t* __restrict__ seg_base,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ offsets_copy,
                                                     int32_t* __restrict__ item_start) {
  __shared__ int psum[16][kMaxM];
  __shared__ int off[kMaxM + 1];
  __shared__ int tst[kMaxM + 1];
  const int t = threadIdx.x, e = t & 63, part = t >> 6;
  const int64_t bh = blockIdx.x;
  const int s0 = static_cast<int>((static_cast<int64_t>(part) * nseg) / 16);
  const int s1 = static_cast<int>((static_cast<int64_t>(part + 1) * nseg) / 16);
  const int32_t* C = counts + bh * nseg * m;
  int sum = 0;
  if (e < m)
    for (int s = s0; s < s1; ++s) sum += C[s * m + e];
  psum[part][e] = sum;
  __syncthreads();
  if (t < 64) {
    int total = 0;
    if (e < m)
      for (int p = 0; p < 16; ++p) total += psum[p][e];
    // exclusive scans over experts of totals and of tile counts (one wave)
    const int tiles_e = (total + tile - 1) / tile;
    int ex = total, tl = (tiles_e + tpb - 1) / tpb;  // work items of expert e
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int a = static_cast<int>(lane_read(static_cast<uint32_t>(ex), t >= d ? t - d : t));
      const int b = static_cast<int>(lane_read(static_cast<uint32_t>(tl), t >= d ? t - d : t));
      if (t >= d) {
        ex += a;
        tl += b;
      }
    }
    // ex, tl are inclusive; shift to exclusive
    off[t + 1] = ex;
    tst[t + 1] = tl;
    if (t == 0) {
      off[0] = 0;
      tst[0] = 0;
    }
  }
  __syncthreads();
  if (t <= m) {
    offsets[bh * (m + 1) + t] = off[t];
    if (offsets_copy) offsets_copy[bh * (m + 1) + t] = off[t];
    item_start[bh * (m + 1) + t] = tst[t];
  }
  if (e < m) {
    int run = off[e];
    for (int p = 0; p < part; ++p) run += psum[p][e];
    int32_t* SB = seg_base + bh * nseg * m;
    for (int s = s0; s < s1; ++s) {
      SB[s * m + e] = run;
      run += C[s * m + e];
    }
  }
}

// grid (nseg, BH), 64 threads: stable scatter of one segment's queries
__global__ __launch_bounds__(64) void k_bucket_scatter(const int32_t* __restrict__ route, int m,
                                                      int nseg, int64_t N,
                                                      const int32_t* __restrict__ seg_base,
                                                      int32_t* __restrict__ perm,
                                                      int32_t* __restrict__ perm_copy) {
  __shared__ int base[kMaxM];
  const int l = threadIdx.x, seg = blockIdx.x;
  const int64_t bh = blockIdx.y;
  if (l < m) base[l] = seg_base[(bh * nseg + seg) * m + l];
  __syncthreads();
  const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));
  for (int it = 0; it < kRouteSeg / 64; ++it) {
    const int64_t q = static_cast<int64_t>(seg) * kRouteSeg + 64 * it + l;
    if (static_cast<int64_t>(seg) * kRouteSeg + 64 * it >= N) break;
    const bool ok = q < N;
    int r = ok ? route[bh * N + q] : 0;
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
    const int pos = ok ? base[r] + rank : 0;
    if (ok && pos >= 0 && pos < N) {
      perm[bh * N + pos] = static_cast<int32_t>(q);
      if (perm_copy) perm_copy[bh * N + pos] = static_cast<int32_t>(q);
    }
    __syncthreads();  // the reads of base[] above complete before the update
    if (ok && rank == total - 1) base[r] += total;
    __syncthreads();
  }
}

template <class T>
static hipError_t launch_route_t(const Shape& s, const void* Q, const Workspace& ws,
                                 int32_t* route_out, hipStream_t st) {
  using E = typename T::elem;
  hipLaunchKernelGGL(k_route<T>, dim3(s.nseg, s.BH), dim3(256), 0, st, static_cast<const E*>(Q),
                     static_cast<const E*>(ws.ql), s.N, s.m, s.nseg, route_out, ws.counts);
  return hipGetLastError();
}

hipError_t launch_route(const Shape& s, const void* Q, const Workspace& ws, int32_t* route_out,
                        hipStream_t st) {
  return s.dtype == 1 ? launch_route_t<BF16>(s, Q, ws, route_out, st)
                      : launch_route_t<F32>(s, Q, ws, route_out, st);
}

hipError_t launch_bucket(const Shape& s, const int32_t* route, const Workspace& ws,
                         int32_t* offsets_copy, int32_t* perm_copy, hipStream_t st) {
  hipLaunchKernelGGL(k_bucket_scan, dim3(s.BH), dim3(1024), 0, st, ws.counts, s.m, s.nseg, s.N,
                     kAttendTile, s.attend_tpb, ws.seg_base, ws.offsets, offsets_copy,
                     ws.item_start);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_bucket_scatter, dim3(s.nseg, s.BH), dim3(64), 0, st, route, s.m, s.nseg,
                     s.N, ws.seg_base, ws.perm, perm_copy);
  return hipGetLastError();
}

}  // namespace mita
