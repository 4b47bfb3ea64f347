// kernels_pool.hip — step 1: landmark queries by local average pooling of Q.
//
// Landmark i averages Q over its window of the token grid (the pages pool
// landmark queries locally from Q: "NeurIPS'26：注意力也是FFN？…", section
// "用少量地标查询，同时构造全局概括与细节专家"; "Mixture-of-Top-k 注意力…",
// section "MiTA：用少量地标查询，同时完成压缩与专家构造").  Windows are the
// adaptive-pooling bins rows [floor(a*gh/mh), ceil((a+1)*gh/mh)) x columns
// [floor(c*gw/mw), ceil((c+1)*gw/mw)).
//
// Precision: window sums are accumulated in fp64 and divided once in fp64,
// then rounded to the input type directly from fp64.  For bf16 inputs
// (8-bit significands) these fp64 sums are exact, hence independent of the
// order in which the partial sums below are combined.
//
// Roofline: HBM-bound streaming read of Q (N*d*e bytes per head), m*d*e
// bytes written.
#include "mita_device.hpp"
#include "mita_internal.hpp"

namespace mita {

__device__ __forceinline__ void window_bounds(int gh, int gw, int mh, int mw, int i, int64_t& r0,
                                              int64_t& r1, int64_t& c0, int64_t& c1) {
  const int64_t a = i / mw, c = i % mw;
  r0 = (a * gh) / mh;
  r1 = ((a + 1) * gh + mh - 1) / mh;
  c0 = (c * gw) / mw;
  c1 = ((c + 1) * gw + mw - 1) / mw;
}

// load 8 consecutive elements as float
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(w[j] << 16);
    v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = a[j];
    v[4 + j] = b[j];
  }
}

// grid (pool_splits, m, BH), 256 threads: 32 token rows x 8 column groups.
// With one split per window the block divides and rounds itself (ql, and
// ql_copy when non-null) and no final launch follows; otherwise it stores
// its fp64 partial sum.
template <class T>
__global__ __launch_bounds__(256) void k_pool_partial(const typename T::elem* __restrict__ Q,
                                                     int64_t N, int gh, int gw, int mh, int mw,
                                                     int splits, int64_t bh0,
                                                     double* __restrict__ part,
                                                     typename T::elem* __restrict__ ql,
                                                     typename T::elem* __restrict__ ql_copy) {
  __shared__ double red[32][kD + 1];
  const int split = blockIdx.x, i = blockIdx.y, m = mh * mw;
  const int64_t bh = bh0 + blockIdx.z;
  int64_t r0, r1, c0, c1;
  window_bounds(gh, gw, mh, mw, i, r0, r1, c0, c1);
  const int64_t wc = c1 - c0, W = (r1 - r0) * wc;
  const int64_t t_beg = static_cast<int64_t>(split) * kPoolChunk;
  const int64_t t_end = t_beg + kPoolChunk < W ? t_beg + kPoolChunk : W;
  const int col = threadIdx.x & 7, row = threadIdx.x >> 3;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const typename T::elem* Qh = Q + bh * N * kD;
  if (r1 - r0 == 1) {
    // one row segment (every 1D window): tokens are contiguous, 4 loads in
    // flight per thread
    const typename T::elem* p = Qh + (r0 * gw + c0 + t_beg + row) * kD + col * 8;
    const int n = t_beg + row < t_end ? static_cast<int>((t_end - t_beg - row + 31) / 32) : 0;
    int j = 0;
    for (; j + 4 <= n; j += 4) {
      float v[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) load8(p + static_cast<int64_t>(j + u) * 32 * kD, v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += static_cast<double>(v[u][e]);
    }
    for (; j < n; ++j) {
      float v[8];
      load8(p + static_cast<int64_t>(j) * 32 * kD, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += static_cast<double>(v[e]);
    }
  } else {
    // 2D window (few tokens): token position from the window-local index
    for (int64_t t = t_beg + row; t < t_end; t += 32) {
      const int64_t tok = (r0 + t / wc) * gw + (c0 + t % wc);
      float v[8];
      load8(Qh + tok * kD + col * 8, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += static_cast<double>(v[e]);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[row][col * 8 + j] = acc[j];
  __syncthreads();
  if (threadIdx.x < kD) {
    double s = 0.0;
    for (int r = 0; r < 32; ++r) s += red[r][threadIdx.x];
    if (splits == 1) {
      const typename T::elem v = T::from_f64(s / static_cast<double>(W));
      ql[(bh * m + i) * kD + threadIdx.x] = v;
      if (ql_copy) ql_copy[(bh * m + i) * kD + threadIdx.x] = v;
    } else {
      part[((bh * m + i) * splits + split) * kD + threadIdx.x] = s;
    }
  }
}

// grid (m, BH), 64 threads: combine partial sums, divide, round
template <class T>
__global__ __launch_bounds__(64) void k_pool_final(const double* __restrict__ part, int gh, int gw,
                                                  int mh, int mw, int splits, int64_t bh0,
                                                  typename T::elem* __restrict__ ql,
                                                  typename T::elem* __restrict__ ql_copy) {
  const int i = blockIdx.x, m = mh * mw, j = threadIdx.x;
  const int64_t bh = bh0 + blockIdx.y;
  int64_t r0, r1, c0, c1;
  window_bounds(gh, gw, mh, mw, i, r0, r1, c0, c1);
  const double W = static_cast<double>((r1 - r0) * (c1 - c0));
  double s = 0.0;
  for (int p = 0; p < splits; ++p) s += part[((bh * m + i) * splits + p) * kD + j];
  const typename T::elem v = T::from_f64(s / W);
  ql[(bh * m + i) * kD + j] = v;
  if (ql_copy) ql_copy[(bh * m + i) * kD + j] = v;
}

// Small windows (at most kPoolDirectMax tokens, the 2D image grids): grid
// (ceil(m / 8), BH), 256 threads; 32 lanes per landmark = 8 groups of 8
// columns x 4 token phases.  Each lane sums every fourth token of its
// landmark's window for its 8 columns in fp64, the four phases combine by
// lane swaps, and phase 0 divides once and rounds: one launch instead of a
// partial-sum and a final launch.  A lane's loads go out 16 at a time (rows
// past the window read the window's first token and are not added), and
// the tokens' window positions are stepped, not divided out per token
// (pooling at the 40x40 grid: 15.0 -> 13.7 us).  The fp64 sums are exact
// for bf16 inputs, so the order of the additions does not matter.
template <class T>
__global__ __launch_bounds__(256) void k_pool_direct(const typename T::elem* __restrict__ Q,
                                                    int64_t N, int gh, int gw, int mh, int mw,
                                                    typename T::elem* __restrict__ ql,
                                                    typename T::elem* __restrict__ ql_copy) {
  const int m = mh * mw;
  const int u = static_cast<int>(blockIdx.x) * 256 + threadIdx.x;
  const int i = u >> 5, col = (u >> 2) & 7, ph = u & 3;
  const int64_t bh = blockIdx.y;
  int64_t r0, r1, c0, c1;
  window_bounds(gh, gw, mh, mw, i < m ? i : m - 1, r0, r1, c0, c1);
  const int64_t wc = c1 - c0, W = (r1 - r0) * wc;
  const typename T::elem* Qh = Q + bh * N * kD + col * 8;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // the phase's tokens ph, ph + 4, ... as (row, column) in the window,
  // stepped without a division per token (wc <= W <= kPoolDirectMax)
  const int wc32 = static_cast<int>(wc), W32 = static_cast<int>(W);
  const int dr = 4 / wc32, dc = 4 % wc32;
  int rr = ph / wc32, cc = ph % wc32;
  constexpr int U = 16;  // tokens of this phase in flight
  for (int t0 = ph; t0 < W32; t0 += 4 * U) {
    float v[U][8];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      // past the window: any of its rows (the window's first), not added
      const int64_t tk = t0 + 4 * j < W32 ? (r0 + rr) * gw + (c0 + cc) : r0 * gw + c0;
      load8(Qh + tk * kD, v[j]);
      rr += dr;
      cc += dc;
      if (cc >= wc32) {
        cc -= wc32;
        ++rr;
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j)
      if (t0 + 4 * j < W32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += static_cast<double>(v[j][e]);
      }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc[e] += __shfl_xor(acc[e], 1);
    acc[e] += __shfl_xor(acc[e], 2);
  }
  if (ph == 0 && i < m) {
    const double Wd = static_cast<double>(W);
    typename T::elem* dst = ql + (bh * m + i) * kD + col * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const typename T::elem v = T::from_f64(acc[e] / Wd);
      dst[e] = v;
      if (ql_copy) ql_copy[(bh * m + i) * kD + col * 8 + e] = v;
    }
  }
}

template <class T>
static hipError_t launch_pool_t(const Shape& s, const void* Q, const Workspace& ws, void* ql_copy,
                                int64_t bh0, int64_t nbh, hipStream_t st) {
  using E = typename T::elem;
  if (s.pool_direct) {
    hipLaunchKernelGGL(k_pool_direct<T>, dim3((s.m + 7) / 8, nbh), dim3(256), 0, st,
                       static_cast<const E*>(Q) + bh0 * s.N * kD, s.N, s.gh, s.gw, s.mh, s.mw,
                       static_cast<E*>(ws.ql) + bh0 * s.m * kD,
                       ql_copy ? static_cast<E*>(ql_copy) + bh0 * s.m * kD : nullptr);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_pool_partial<T>, dim3(s.pool_splits, s.m, nbh), dim3(256), 0, st,
                     static_cast<const E*>(Q), s.N, s.gh, s.gw, s.mh, s.mw, s.pool_splits, bh0,
                     ws.pool_part, static_cast<E*>(ws.ql), static_cast<E*>(ql_copy));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || s.pool_splits == 1) return e;  // one split: already final
  hipLaunchKernelGGL(k_pool_final<T>, dim3(s.m, nbh), dim3(64), 0, st, ws.pool_part, s.gh, s.gw,
                     s.mh, s.mw, s.pool_splits, bh0, static_cast<E*>(ws.ql),
                     static_cast<E*>(ql_copy));
  return hipGetLastError();
}

hipError_t launch_pool(const Shape& s, const void* Q, const Workspace& ws, void* ql_copy,
                       int64_t bh0, int64_t nbh, hipStream_t st) {
  return s.dtype == 1 ? launch_pool_t<BF16>(s, Q, ws, ql_copy, bh0, nbh, st)
                      : launch_pool_t<F32>(s, Q, ws, ql_copy, bh0, nbh, st);
}

}  // namespace mita
