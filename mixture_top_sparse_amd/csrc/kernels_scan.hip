// kernels_scan.hip — step 2: one pass of the m landmark queries over all N
// keys feeds both the routed experts (top-k keys per landmark) and the
// landmark values (softmax cross-attention of the landmarks over K, V).
//
// The pages build both from the same landmark-key scores
// ("NeurIPS'26：注意力也是FFN？…", section "用少量地标查询，同时构造全局概括与
// 细节专家"; "Mixture-of-Top-k 注意力…", section "MiTA：用少量地标查询，同时
// 完成压缩与专家构造"), and note that the cross-attention can run as a
// FlashAttention-style pass (same page, implementation remark).  Here one
// kernel streams K and V once:
//
//   k_scan  (split, head) blocks; wave w owns landmarks 16w..16w+15.
//     per 64-key tile: S^T = K_tile Ql^T on MFMA (key rows x landmark
//     columns), online softmax of scale*S with P.V on MFMA (P split into
//     bf16 hi + lo parts), and an exact streaming top-k: scores above the
//     landmark's current k-th best are appended to an LDS candidate buffer;
//     a full buffer is sorted (wave bitonic network) and merged into the
//     landmark's top list, which lives in registers (lane i = i-th best).
//   k_merge (landmark, head) blocks: merges the per-split top lists and the
//     per-split softmax states (log-sum-exp) into idx_out and Vl.
//
// Selection keys are 64-bit (order-preserving score bits, inverted index),
// so "higher score, then lower index" is a plain unsigned comparison.
//
// Roofline: HBM-bound; K and V are read once (2*N*d*e bytes per head); the
// per-split partials add splits*mrows*(64*8 + 8 + 64*4) bytes per head.
#include "mita_device.hpp"
#include "mita_internal.hpp"

namespace mita {

// ---------------------------------------------------------------------------
// per-type tile staging and MFMA steps
// ---------------------------------------------------------------------------

template <class T>
struct ScanTraits;

// bf16: K rows in LDS (row stride 72 elements); V transposed in LDS
// (V^T[d][key], row stride 68) so that P.V's A operand (8 keys of one d)
// is two 8-byte reads.
template <>
struct ScanTraits<BF16> {
  using E = uint16_t;
  static constexpr int KST = 72;
  static constexpr int VST = 68;
  struct QReg {
    bf16x8 v[2];
  };
  template <int NT>
  struct Tile {
    static constexpr int CK = 512 / NT;  // 16-byte K chunks per thread
    static constexpr int CV = 256 / NT;  // V row pairs per thread
    u32x4 k[CK];
    u32x4 v[CV][2];
  };

  __device__ static void load_q(QReg& q, const E* ql_row, bool ok, int g) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 z = {0, 0, 0, 0};
      q.v[s] = as_bf16x8(ok ? *reinterpret_cast<const u32x4*>(ql_row + 32 * s + 8 * g) : z);
    }
  }

  template <int NT>
  __device__ static void load_tile(Tile<NT>& t, const E* Kh, const E* Vh, int64_t t0, int64_t kend,
                                   int tid) {
#pragma unroll
    for (int j = 0; j < Tile<NT>::CK; ++j) {
      const int c = tid + NT * j, row = c >> 3, col = c & 7;
      const u32x4 z = {0, 0, 0, 0};
      t.k[j] = (t0 + row < kend) ? *reinterpret_cast<const u32x4*>(Kh + (t0 + row) * kD + col * 8)
                                 : z;
    }
#pragma unroll
    for (int j = 0; j < Tile<NT>::CV; ++j) {
      const int p = tid + NT * j, rp = p >> 3, col = p & 7;
      const u32x4 z = {0, 0, 0, 0};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t row = t0 + 2 * rp + h;
        t.v[j][h] = (row < kend) ? *reinterpret_cast<const u32x4*>(Vh + row * kD + col * 8) : z;
      }
    }
  }

  template <int NT>
  __device__ static void store_tile(const Tile<NT>& t, E* klds, E* vlds, int tid) {
#pragma unroll
    for (int j = 0; j < Tile<NT>::CK; ++j) {
      const int c = tid + NT * j, row = c >> 3, col = c & 7;
      *reinterpret_cast<u32x4*>(klds + row * KST + col * 8) = t.k[j];
    }
#pragma unroll
    for (int j = 0; j < Tile<NT>::CV; ++j) {
      const int p = tid + NT * j, rp = p >> 3, col = p & 7;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t a = t.v[j][0][i >> 1], b = t.v[j][1][i >> 1];
        const uint32_t word = (i & 1) ? ((a >> 16) | (b & 0xFFFF0000u))
                                      : ((a & 0xFFFFu) | (b << 16));
        *reinterpret_cast<uint32_t*>(vlds + (col * 8 + i) * VST + 2 * rp) = word;
      }
    }
  }

  // S^T block: keys 16kb..16kb+15 (rows) x the wave's 16 landmarks (columns)
  __device__ static f32x4 score(const E* klds, int kb, const QReg& q, int c16, int g) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 a =
          as_bf16x8(*reinterpret_cast<const u32x4*>(klds + (16 * kb + c16) * KST + 32 * s + 8 * g));
      acc = mfma_bf16(a, q.v[s], acc);
    }
    return acc;
  }

  // the same block straight from global memory (key row `row` of this lane)
  __device__ static f32x4 score_global(const E* Kh, int64_t row, int64_t N, const QReg& q, int g) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x4 z = {0, 0, 0, 0};
      const bf16x8 a = as_bf16x8(
          row < N ? *reinterpret_cast<const u32x4*>(Kh + row * kD + 32 * s + 8 * g) : z);
      acc = mfma_bf16(a, q.v[s], acc);
    }
    return acc;
  }

  // O^T[d][lm] += V^T[d][keys] P^T[keys][lm] for the tile's 64 keys
  __device__ static void pv(f32x4 (&acc)[4], const E* vlds, const float (&p)[4][4], int c16, int g) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      float pp[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pp[r] = p[2 * s2][r];
        pp[4 + r] = p[2 * s2 + 1][r];
      }
      bf16x8 hi, lo;
      split_hi_lo(pp, hi, lo);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const E* row = vlds + (16 * dt + c16) * VST + 32 * s2 + 4 * g;
        const bf16x8 a = join_bf16x8(*reinterpret_cast<const u32x2*>(row),
                                     *reinterpret_cast<const u32x2*>(row + 16));
        acc[dt] = mfma_bf16(a, hi, acc[dt]);
        acc[dt] = mfma_bf16(a, lo, acc[dt]);
      }
    }
  }
};

// fp32: K and V rows in LDS (stride 68), fp32 MFMA 16x16x4.
template <>
struct ScanTraits<F32> {
  using E = float;
  static constexpr int KST = 68;
  static constexpr int VST = 68;
  struct QReg {
    float v[16];
  };
  template <int NT>
  struct Tile {
    static constexpr int C = 1024 / NT;  // 16-byte chunks per thread (K and V each)
    f32x4 k[C];
    f32x4 v[C];
  };

  __device__ static void load_q(QReg& q, const E* ql_row, bool ok, int g) {
#pragma unroll
    for (int s = 0; s < 16; ++s) q.v[s] = ok ? ql_row[4 * s + g] : 0.f;
  }

  template <int NT>
  __device__ static void load_tile(Tile<NT>& t, const E* Kh, const E* Vh, int64_t t0, int64_t kend,
                                   int tid) {
#pragma unroll
    for (int j = 0; j < Tile<NT>::C; ++j) {
      const int c = tid + NT * j, row = c >> 4, col = c & 15;
      const f32x4 z = {0, 0, 0, 0};
      const bool ok = t0 + row < kend;
      t.k[j] = ok ? *reinterpret_cast<const f32x4*>(Kh + (t0 + row) * kD + col * 4) : z;
      t.v[j] = ok ? *reinterpret_cast<const f32x4*>(Vh + (t0 + row) * kD + col * 4) : z;
    }
  }

  template <int NT>
  __device__ static void store_tile(const Tile<NT>& t, E* klds, E* vlds, int tid) {
#pragma unroll
    for (int j = 0; j < Tile<NT>::C; ++j) {
      const int c = tid + NT * j, row = c >> 4, col = c & 15;
      *reinterpret_cast<f32x4*>(klds + row * KST + col * 4) = t.k[j];
      *reinterpret_cast<f32x4*>(vlds + row * VST + col * 4) = t.v[j];
    }
  }

  __device__ static f32x4 score(const E* klds, int kb, const QReg& q, int c16, int g) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 16; ++s) acc = mfma_f32(klds[(16 * kb + c16) * KST + 4 * s + g], q.v[s], acc);
    return acc;
  }

  __device__ static f32x4 score_global(const E* Kh, int64_t row, int64_t N, const QReg& q, int g) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 16; ++s) acc = mfma_f32(row < N ? Kh[row * kD + 4 * s + g] : 0.f, q.v[s], acc);
    return acc;
  }

  __device__ static void pv(f32x4 (&acc)[4], const E* vlds, const float (&p)[4][4], int c16, int g) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          acc[dt] = mfma_f32(vlds[(16 * kb + 4 * g + r) * VST + 16 * dt + c16], p[kb][r], acc[dt]);
  }
};

// ---------------------------------------------------------------------------
// the scan kernel
// ---------------------------------------------------------------------------

// Block: 256 threads stage each 64-key tile (double-buffered LDS, two tiles
// of global loads in flight); waves 0..NW-1 each own 16 landmarks.
template <class T, int NW>
__global__ __launch_bounds__(256) void k_scan(
    const typename T::elem* __restrict__ K, const typename T::elem* __restrict__ V,
    const typename T::elem* __restrict__ Ql, const float* __restrict__ theta, int64_t N, int m,
    int k, int chunk, int splits, float c2, uint64_t* __restrict__ part_keys,
    float* __restrict__ part_stats, float* __restrict__ part_acc) {
  using TR = ScanTraits<T>;
  using E = typename T::elem;
  constexpr int NT = 256;
  constexpr int MROWS = NW * 16;
  __shared__ __attribute__((aligned(16))) E klds[2][64 * TR::KST];
  __shared__ __attribute__((aligned(16))) E vlds[2][64 * TR::VST];
  __shared__ uint64_t cand[MROWS][kTopCap];

  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const bool computes = w < NW;
  const int split = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int lm = w * 16 + c16;
  const bool lm_ok = computes && lm < m;
  const int64_t kbeg = static_cast<int64_t>(split) * chunk;
  const int64_t kend = (kbeg + chunk < N) ? kbeg + chunk : N;
  const int ntiles = static_cast<int>((kend - kbeg + kTileKeys - 1) / kTileKeys);
  const E* Kh = K + bh * N * kD;
  const E* Vh = V + bh * N * kD;

  typename TR::QReg q;
  TR::load_q(q, Ql + (bh * m + (lm_ok ? lm : 0)) * kD, lm_ok, g);

  float M = -INFINITY, Lsum = 0.f;
  f32x4 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x4{0, 0, 0, 0};
  uint64_t top[16];
#pragma unroll
  for (int L = 0; L < 16; ++L) top[L] = 0;
  float th = (theta != nullptr && lm_ok) ? theta[bh * MROWS + lm] : -INFINITY;
  int cnt = 0;

  // merge landmark slot L's candidate buffer into its top list (whole wave)
  auto merge_slot = [&](int L) __attribute__((always_inline)) {
    const int cL = static_cast<int>(uniform_read(static_cast<uint32_t>(cnt), L));
    uint64_t c = (l < cL) ? cand[w * 16 + L][l] : 0ull;
    c = wave_sort_desc(c);
    top[L] = wave_merge_top(top[L], c);
    const uint64_t kth = uniform_read(top[L], k - 1);
    if (c16 == L) {
      cnt = 0;
      if (kth != 0ull) th = fmaxf(th, key_score(kth));
    }
  };

  auto compute_tile = [&](const E* kl, const E* vl, int64_t t0) __attribute__((always_inline)) {
    float sc[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const f32x4 a = TR::score(kl, kb, q, c16, g);
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[kb][r] = a[r];
    }
    if (t0 + kTileKeys > kend) {  // ragged last tile: drop keys past the chunk
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t0 + 16 * kb + 4 * g + r >= kend) sc[kb][r] = -INFINITY;
    }
    float smax = sc[0][0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) smax = fmaxf(smax, sc[kb][r]);

    // ---- streaming top-k: only when some score beats its landmark's k-th best
    if (ballot(lm_ok && smax > th)) {
      uint32_t passbits = 0;
      int npass = 0;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = lm_ok && (sc[kb][r] > th);
          passbits |= static_cast<uint32_t>(ok) << (4 * kb + r);
          npass += ok;
        }
      const int n0 = static_cast<int>(lane_read(static_cast<uint32_t>(npass), c16));
      const int n1 = static_cast<int>(lane_read(static_cast<uint32_t>(npass), 16 + c16));
      const int n2 = static_cast<int>(lane_read(static_cast<uint32_t>(npass), 32 + c16));
      const int n3 = static_cast<int>(lane_read(static_cast<uint32_t>(npass), 48 + c16));
      const int tot = n0 + n1 + n2 + n3;
      const int pre = (g > 0 ? n0 : 0) + (g > 1 ? n1 : 0) + (g > 2 ? n2 : 0);
      const uint32_t need = static_cast<uint32_t>(ballot(cnt + tot > kTopCap)) & 0xFFFFu;
      if (need) {
#pragma unroll
        for (int L = 0; L < 16; ++L)
          if ((need >> L) & 1u) merge_slot(L);
      }
      if (passbits) {
        int pos = cnt + pre;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if ((passbits >> (4 * kb + r)) & 1u)
              cand[lm][pos++] =
                  make_key(sc[kb][r], static_cast<uint32_t>(t0 + 16 * kb + 4 * g + r));
      }
      cnt += tot;
    }

    // ---- online softmax (log2 domain, lazy rescale) and P.V ----
    float mx = xor_max(smax, 16);
    mx = xor_max(mx, 32) * c2;
    if (ballot(mx > M)) {
      const float Mn = fmaxf(M, mx);
      const float alpha = fast_exp2(M - Mn);
      Lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
      M = Mn;
    }
    float p[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kb][r] = fast_exp2(fmaf(sc[kb][r], c2, -M));
        Lsum += p[kb][r];
      }
    TR::pv(acc, vl, p, c16, g);
  };

  // prologue: tile 0 into LDS buffer 0, tiles 1 and 2 in flight
  typename TR::template Tile<NT> ra, rb;
  TR::template load_tile<NT>(ra, Kh, Vh, kbeg, kend, tid);
  TR::template store_tile<NT>(ra, klds[0], vlds[0], tid);
  if (ntiles > 1) TR::template load_tile<NT>(ra, Kh, Vh, kbeg + kTileKeys, kend, tid);
  if (ntiles > 2) TR::template load_tile<NT>(rb, Kh, Vh, kbeg + 2 * kTileKeys, kend, tid);
  __syncthreads();

  for (int it = 0; it < ntiles; it += 2) {
    const int64_t t0 = kbeg + static_cast<int64_t>(it) * kTileKeys;
    if (computes) compute_tile(klds[0], vlds[0], t0);
    if (it + 1 < ntiles) TR::template store_tile<NT>(ra, klds[1], vlds[1], tid);
    if (it + 3 < ntiles) TR::template load_tile<NT>(ra, Kh, Vh, t0 + 3 * kTileKeys, kend, tid);
    __syncthreads();
    if (it + 1 >= ntiles) break;
    if (computes) compute_tile(klds[1], vlds[1], t0 + kTileKeys);
    if (it + 2 < ntiles) TR::template store_tile<NT>(rb, klds[0], vlds[0], tid);
    if (it + 4 < ntiles) TR::template load_tile<NT>(rb, Kh, Vh, t0 + 4 * kTileKeys, kend, tid);
    __syncthreads();
  }
  if (!computes) return;

  // flush the candidate buffers
  const uint32_t need = static_cast<uint32_t>(ballot(cnt > 0)) & 0xFFFFu;
  if (need) {
#pragma unroll
    for (int L = 0; L < 16; ++L)
      if ((need >> L) & 1u) merge_slot(L);
  }

  const int64_t pbase = (bh * splits + split) * MROWS;
#pragma unroll
  for (int L = 0; L < 16; ++L) part_keys[(pbase + w * 16 + L) * kTopCap + l] = top[L];
  Lsum = xor_sum(Lsum, 16);
  Lsum = xor_sum(Lsum, 32);
  if (g == 0) {
    part_stats[(pbase + lm) * 2 + 0] = M;
    part_stats[(pbase + lm) * 2 + 1] = Lsum;
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    *reinterpret_cast<f32x4*>(part_acc + (pbase + lm) * kD + 16 * dt + 4 * g) = acc[dt];
}

// ---------------------------------------------------------------------------
// top-k pre-threshold from a key sample
// ---------------------------------------------------------------------------
//
// For each landmark, the k-th largest of G group maxima (G sample tiles of 64
// keys spread evenly over N) is the key of some real key t, and the k keys
// behind those maxima are distinct, so the global k-th best key is >= it.
// The scan may therefore drop every score below that sample key's score
// without changing the exact top-k.

// grid (G / kThetaTilesPerBlock, BH), 256 threads; wave w: landmarks 16w..16w+15
template <class T>
__global__ __launch_bounds__(256) void k_theta_sample(const typename T::elem* __restrict__ K,
                                                     const typename T::elem* __restrict__ Ql,
                                                     int64_t N, int m, int groups,
                                                     uint64_t* __restrict__ gmax) {
  using TR = ScanTraits<T>;
  using E = typename T::elem;
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int64_t bh = blockIdx.y;
  const int lm = w * 16 + c16;
  const bool lm_ok = lm < m;
  if (w * 16 >= m) return;  // whole wave beyond the landmarks
  typename TR::QReg q;
  TR::load_q(q, Ql + (bh * m + (lm_ok ? lm : 0)) * kD, lm_ok, g);
  const int64_t ntiles = (N + kTileKeys - 1) / kTileKeys;
  const E* Kh = K + bh * N * kD;
  for (int j = 0; j < kThetaTilesPerBlock; ++j) {
    const int gi = blockIdx.x * kThetaTilesPerBlock + j;
    const int64_t t0 = ((static_cast<int64_t>(gi) * ntiles) / groups) * kTileKeys;
    uint64_t best = 0;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const f32x4 a = TR::score_global(Kh, t0 + 16 * kb + c16, N, q, g);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + 16 * kb + 4 * g + r;
        if (t < N) {
          const uint64_t key = make_key(a[r], static_cast<uint32_t>(t));
          best = key > best ? key : best;
        }
      }
    }
#pragma unroll
    for (int mask = 16; mask <= 32; mask <<= 1) {
      const uint64_t o = lane_read(best, l ^ mask);
      best = o > best ? o : best;
    }
    if (g == 0 && lm_ok) gmax[(bh * m + lm) * groups + gi] = best;
  }
}

// grid (m, BH), 256 threads: theta[bh][lm] = score of the k-th largest group
// maximum, lowered by one ulp so that the scan's strict test (s > theta)
// keeps every score equal to it; -inf when fewer than k maxima exist.
__global__ __launch_bounds__(256) void k_theta_select(const uint64_t* __restrict__ gmax, int m,
                                                     int k, int groups, int mrows,
                                                     float* __restrict__ theta) {
  __shared__ uint64_t tops[4][64];
  const int l = lane_id(), w = wave_id(), lm = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const uint64_t* G = gmax + (bh * m + lm) * groups;
  uint64_t top = 0;
  for (int c = w; c * 64 < groups; c += 4) {
    const int i = c * 64 + l;
    uint64_t v = i < groups ? G[i] : 0ull;
    v = wave_sort_desc(v);
    top = wave_merge_top(top, v);
  }
  tops[w][l] = top;
  __syncthreads();
  if (w != 0) return;
  uint64_t t = tops[0][l];
#pragma unroll
  for (int v = 1; v < 4; ++v) t = wave_merge_top(t, tops[v][l]);
  const uint64_t kth = uniform_read(t, k - 1);
  if (l == 0)
    theta[bh * mrows + lm] = kth != 0ull ? nextafterf(key_score(kth), -INFINITY) : -INFINITY;
}

// ---------------------------------------------------------------------------
// merge of the per-split partials
// ---------------------------------------------------------------------------

// grid (m, BH), 256 threads
__global__ __launch_bounds__(256) void k_merge(
    const uint64_t* __restrict__ part_keys, const float* __restrict__ part_stats,
    const float* __restrict__ part_acc, int m, int k, int mrows, int splits,
    int32_t* __restrict__ idx_out, float* __restrict__ vl, float* __restrict__ vl_copy) {
  __shared__ uint64_t tops[4][64];
  __shared__ float sacc[4][64];
  __shared__ float sM[4], sL[4];
  const int l = lane_id(), w = wave_id(), lm = blockIdx.x;
  const int64_t bh = blockIdx.y;

  // top lists of splits w, w+4, ...
  uint64_t top = 0;
  auto list_at = [&](int s) { return part_keys[((bh * splits + s) * mrows + lm) * kTopCap + l]; };
  uint64_t nxt = (w < splits) ? list_at(w) : 0ull;
  for (int s = w; s < splits; s += 4) {
    const uint64_t cur = nxt;
    if (s + 4 < splits) nxt = list_at(s + 4);
    top = wave_merge_top(top, cur);
  }
  // softmax states of the same splits (lane = feature d)
  float Mw = -INFINITY, Lw = 0.f, aw = 0.f;
  for (int s = w; s < splits; s += 4) {
    const int64_t b = (bh * splits + s) * mrows + lm;
    const float Ms = part_stats[b * 2], Ls = part_stats[b * 2 + 1], as = part_acc[b * kD + l];
    const float Mn = fmaxf(Mw, Ms);
    const float f0 = fast_exp2(Mw - Mn), f1 = fast_exp2(Ms - Mn);
    Lw = Lw * f0 + Ls * f1;
    aw = aw * f0 + as * f1;
    Mw = Mn;
  }
  tops[w][l] = top;
  sacc[w][l] = aw;
  if (l == 0) {
    sM[w] = Mw;
    sL[w] = Lw;
  }
  __syncthreads();
  if (w != 0) return;

  uint64_t t = tops[0][l];
#pragma unroll
  for (int v = 1; v < 4; ++v) t = wave_merge_top(t, tops[v][l]);
  int32_t ix = (l < k) ? static_cast<int32_t>(key_index(t)) : INT32_MAX;
  ix = wave_sort_asc_i32(ix);
  if (l < k) idx_out[(bh * m + lm) * k + l] = ix;

  float Mt = sM[0];
#pragma unroll
  for (int v = 1; v < 4; ++v) Mt = fmaxf(Mt, sM[v]);
  float Lt = 0.f, at = 0.f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float f = fast_exp2(sM[v] - Mt);
    Lt += sL[v] * f;
    at += sacc[v][l] * f;
  }
  const float val = at / Lt;
  vl[(bh * m + lm) * kD + l] = val;
  if (vl_copy != nullptr) vl_copy[(bh * m + lm) * kD + l] = val;
}

// ---------------------------------------------------------------------------

template <class T, int NW>
static hipError_t launch_scan_t(const Shape& s, const void* K, const void* V, const Workspace& ws,
                                hipStream_t st) {
  using E = typename T::elem;
  const float c2 = s.scale * kLog2e;
  hipLaunchKernelGGL((k_scan<T, NW>), dim3(s.scan_splits, s.BH), dim3(256), 0, st,
                     static_cast<const E*>(K), static_cast<const E*>(V),
                     static_cast<const E*>(ws.ql), ws.theta, s.N, s.m, s.k, s.scan_chunk,
                     s.scan_splits, c2, ws.part_keys, ws.part_stats, ws.part_acc);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_scan_w(const Shape& s, const void* K, const void* V, const Workspace& ws,
                                hipStream_t st) {
  switch (s.scan_waves) {
    case 1: return launch_scan_t<T, 1>(s, K, V, ws, st);
    case 2: return launch_scan_t<T, 2>(s, K, V, ws, st);
    default: return launch_scan_t<T, 4>(s, K, V, ws, st);
  }
}

template <class T>
static hipError_t launch_theta_t(const Shape& s, const void* K, const Workspace& ws,
                                 hipStream_t st) {
  using E = typename T::elem;
  hipLaunchKernelGGL(k_theta_sample<T>, dim3(s.theta_groups / kThetaTilesPerBlock, s.BH), dim3(256),
                     0, st, static_cast<const E*>(K), static_cast<const E*>(ws.ql), s.N, s.m,
                     s.theta_groups, ws.gmax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_theta_select, dim3(s.m, s.BH), dim3(256), 0, st, ws.gmax, s.m, s.k,
                     s.theta_groups, s.mrows, ws.theta);
  return hipGetLastError();
}

hipError_t launch_threshold(const Shape& s, const void* K, const Workspace& ws,
                            hipStream_t st) {
  if (s.theta_groups == 0) return hipSuccess;
  return s.dtype == 1 ? launch_theta_t<BF16>(s, K, ws, st) : launch_theta_t<F32>(s, K, ws, st);
}

hipError_t launch_scan(const Shape& s, const void* K, const void* V, const Workspace& ws,
                       hipStream_t st) {
  return s.dtype == 1 ? launch_scan_w<BF16>(s, K, V, ws, st) : launch_scan_w<F32>(s, K, V, ws, st);
}

hipError_t launch_merge(const Shape& s, const Workspace& ws, int32_t* idx_out, float* vl_copy,
                        hipStream_t st) {
  hipLaunchKernelGGL(k_merge, dim3(s.m, s.BH), dim3(256), 0, st, ws.part_keys, ws.part_stats,
                     ws.part_acc, s.m, s.k, s.mrows, s.scan_splits, idx_out, ws.vl, vl_copy);
  return hipGetLastError();
}

}  // namespace mita
