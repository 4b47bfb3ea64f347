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
//   k_scan_bf16 / k_scan_f32  1D grid of (split, head) blocks, then the
//     blocks of step 4's prefix (mita_bucket.hpp); wave w owns landmarks
//     16w..16w+15.  Per 64-key tile: S^T = K_tile Ql^T on MFMA (key rows x
//     landmark columns), online softmax of scale*S with P.V on MFMA (bf16: P
//     split into bf16 hi + lo parts), and an exact streaming top-k: scores
//     above the landmark's current k-th best are appended to an LDS
//     candidate buffer; a full buffer is sorted (wave bitonic network) and
//     merged into the landmark's top list, which lives in registers (lane i
//     = i-th best).  The bf16 kernel stages K and V tiles straight into LDS
//     with the global-load-to-LDS DMA (no register staging, no transposing
//     stores) and reads V^T operands with the LDS transpose read.
//   k_merge (landmark, head) blocks, in one or two passes: merges the
//     per-split top lists and the per-split softmax states (log-sum-exp)
//     into idx_out and Vl; its first pass also carries step 4's scatter.
//   k_theta_fine / k_theta_sample: the top-k pre-threshold's group maxima
//     for fp32 inputs (the bf16 ones are in kernels_route.hip).
//
// Selection keys are 64-bit (order-preserving score bits, inverted index),
// so "higher score, then lower index" is a plain unsigned comparison.
//
// Roofline: HBM-bound; K and V are read once (2*N*d*e bytes per head); the
// per-split partials add about splits*mrows*(64*4 + 12) bytes per head plus
// the (few) surviving top-list entries.
#include "mita_bucket.hpp"
#include "mita_device.hpp"
#include "mita_internal.hpp"
#include "tile_dma.hpp"

namespace mita {

// ---------------------------------------------------------------------------
// per-type tile staging and MFMA steps
// ---------------------------------------------------------------------------

template <class T>
struct ScanTraits;

// bf16: the landmark query operand and the global-memory score (the
// pre-threshold sample); the scan's tile staging is in k_scan_bf16.
template <>
struct ScanTraits<BF16> {
  using E = uint16_t;
  struct QReg {
    bf16x8 v[2];
  };

  __device__ static void load_q(QReg& q, const E* ql_row, bool ok, int g) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 z = {0, 0, 0, 0};
      q.v[s] = as_bf16x8(ok ? *reinterpret_cast<const u32x4*>(ql_row + 32 * s + 8 * g) : z);
    }
  }

  // S^T blocks of the 64-key tile at t0 (block kb: key rows t0 + 16kb ..;
  // columns: the wave's landmarks).  Rows past N read row N - 1 (the caller
  // drops those scores): all eight loads are issued before the first product.
  __device__ static void score_tile_global(const E* Kh, int64_t t0, int64_t N, const QReg& q,
                                           int c16, int g, f32x4 (&sc)[4]) {
    u32x4 ko[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int64_t row = t0 + 16 * kb + c16;
      const int64_t rr = row < N ? row : N - 1;
#pragma unroll
      for (int s = 0; s < 2; ++s)
        ko[kb][s] = *reinterpret_cast<const u32x4*>(Kh + rr * kD + 32 * s + 8 * g);
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sc[kb] = mfma_bf16(as_bf16x8(ko[kb][0]), q.v[0], f32x4{0, 0, 0, 0});
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sc[kb] = mfma_bf16(as_bf16x8(ko[kb][1]), q.v[1], sc[kb]);
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

  __device__ static void score_tile_global(const E* Kh, int64_t t0, int64_t N, const QReg& q,
                                           int c16, int g, f32x4 (&sc)[4]) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int64_t row = t0 + 16 * kb + c16;
      const int64_t rr = row < N ? row : N - 1;
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 16; ++s) acc = mfma_f32(Kh[rr * kD + 4 * s + g], q.v[s], acc);
      sc[kb] = acc;
    }
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
// the scan kernels
// ---------------------------------------------------------------------------

// Per-split partial results of one wave (16 landmarks): the top lists
// (descending; only the nonzero entries are written, their number goes to
// part_cnt), the softmax state (max in log2 units, sum) and the unnormalised
// P.V accumulators O^T (lane: landmark column c16, rows d = 16dt + 4g + r).
template <int NW>
__device__ __forceinline__ void write_partials(const uint64_t (&top)[16], float M, float Lsum,
                                               const f32x4 (&acc)[4], int64_t pbase, int w, int l,
                                               int g, int lm, uint64_t* __restrict__ part_keys,
                                               int32_t* __restrict__ part_cnt,
                                               float* __restrict__ part_stats,
                                               float* __restrict__ part_acc) {
#pragma unroll
  for (int L = 0; L < 16; ++L) {
    const uint64_t nz = ballot(top[L] != 0ull);
    if (top[L] != 0ull) part_keys[(pbase + w * 16 + L) * kTopCap + l] = top[L];
    if (l == 0) part_cnt[pbase + w * 16 + L] = __popcll(nz);
  }
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

// fp32 scan.  Block: 256 threads stage each 64-key tile through registers
// (double-buffered LDS, two tiles of global loads in flight); waves
// 0..NW-1 each own 16 landmarks.
template <int NW>
__global__ __launch_bounds__(256) void k_scan_f32(
    const float* __restrict__ K, const float* __restrict__ V, const float* __restrict__ Ql,
    const float* __restrict__ theta, int64_t N, int m, int k, int chunk, int splits, float c2,
    uint64_t* __restrict__ part_keys, int32_t* __restrict__ part_cnt,
    float* __restrict__ part_stats, float* __restrict__ part_acc, int nbh, BucketArgs ba) {
  // 1D grid: splits * nbh scan blocks (split-fastest), then m * nbh blocks
  // for step 4's prefix (one per expert and head), which run in the scan's
  // tail
  if (static_cast<int>(blockIdx.x) >= splits * nbh) {  // whole block
    __shared__ int wsum[4];
    const int i = static_cast<int>(blockIdx.x) - splits * nbh;
    bucket_prefix(ba.counts, ba.m, ba.nseg, i % ba.m, i / ba.m, ba.colpre, ba.totals, wsum);
    return;
  }
  using T = F32;
  using TR = ScanTraits<T>;
  using E = typename T::elem;
  constexpr int NT = 256;
  constexpr int MROWS = NW * 16;
  __shared__ __attribute__((aligned(16))) E klds[2][64 * TR::KST];
  __shared__ __attribute__((aligned(16))) E vlds[2][64 * TR::VST];
  __shared__ uint64_t cand[MROWS][kTopCap];

  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const bool computes = w < NW;
  const int split = static_cast<int>(blockIdx.x) % splits;
  const int64_t bh = static_cast<int>(blockIdx.x) / splits;
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

  write_partials<NW>(top, M, Lsum, acc, (bh * splits + split) * MROWS, w, l, g, lm, part_keys,
                     part_cnt, part_stats, part_acc);
}

// Block: 4 waves; waves 0..NW-1 each own 16 landmarks, all 4 stage tiles.
// Two LDS tile buffers: while one tile is scored, the next is in flight.
// With three blocks per CU (at most 168 VGPRs) that keeps 48 KiB of tile
// requests in flight per CU; deeper rings (96 KiB per CU) measured slower,
// the DMA path losing bandwidth when that many requests queue up.
// CAP: candidate buffer entries per landmark.  8 in general; 64 (32 when
// k <= 32) where the pre-threshold is the exact k-th score (N <= 4096 keys):
// then about k keys per landmark pass it, and the buffer takes them all
// without a sort-and-merge per 8 candidates (the end-of-block flush sorts
// each once).  A full buffer is merged mid-scan, so any CAP is exact.
// NT: K and V tiles are loaded with the non-temporal cache policy (see
// launch_scan_nw for when).
template <int NW, int CAP, bool NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_scan_bf16(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ Ql, const float* __restrict__ theta, int64_t N, int m, int k,
    int splits, float c2, uint64_t* __restrict__ part_keys,
    int32_t* __restrict__ part_cnt, float* __restrict__ part_stats,
    float* __restrict__ part_acc, int nbh, BucketArgs ba) {
  // 1D grid: splits * nbh scan blocks (split-fastest), then m * nbh blocks
  // for step 4's prefix (one per expert and head), which run in the scan's
  // tail
  if (static_cast<int>(blockIdx.x) >= splits * nbh) {  // whole block
    __shared__ int wsum[4];
    const int i = static_cast<int>(blockIdx.x) - splits * nbh;
    bucket_prefix(ba.counts, ba.m, ba.nseg, i % ba.m, i / ba.m, ba.colpre, ba.totals, wsum);
    return;
  }
  using TR = ScanTraits<BF16>;
  constexpr int MROWS = NW * 16;
  // ring slots: K tile (8 KiB), then V tile (8 KiB)
  __shared__ __attribute__((aligned(16))) uint8_t b0[16384];
  __shared__ __attribute__((aligned(16))) uint8_t b1[16384];
  __shared__ uint64_t cand[MROWS][CAP];
  __shared__ int lcnt[MROWS];  // candidates buffered per landmark (may overshoot CAP)

  const int l = lane_id(), g = l >> 4, c16 = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const bool computes = w < NW;
  const int split = static_cast<int>(blockIdx.x) % splits;
  const int64_t bh = static_cast<int>(blockIdx.x) / splits;
  const int lm = w * 16 + c16;
  const bool lm_ok = computes && lm < m;
  // this block's tiles: split, split + splits, ... (all blocks of a head
  // sweep the keys together, which keeps the DRAM access streams adjacent)
  const int64_t ktiles = (N + kTileKeys - 1) / kTileKeys;
  const int ntiles = static_cast<int>((ktiles - split + splits - 1) / splits);
  const int64_t tstride = static_cast<int64_t>(splits) * kTileKeys;  // keys between my tiles
  const int64_t kbeg = static_cast<int64_t>(split) * kTileKeys;
  const uint16_t* Kh = K + bh * N * kD;
  const uint16_t* Vh = V + bh * N * kD;

  TR::QReg q;
  TR::load_q(q, Ql + (bh * m + (lm_ok ? lm : 0)) * kD, lm_ok, g);
  float th = (theta != nullptr && lm_ok) ? theta[bh * MROWS + lm] : -INFINITY;
  // these loads complete before the first tile request: inside the loop the
  // only outstanding requests are tiles, which the explicit waits below count
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __asm__ volatile("" ::: "memory");

  // prologue: tile 0 in flight
  const uint32_t soff0 = stage_src_off(w, 0, l), soff1 = stage_src_off(w, 1, l);
  const uint32_t a0 = lds_address(b0), a1 = lds_address(b1);
  stage_tile_bf16<NT>(Kh, Vh, kbeg, N, a0, a0 + 8192, w, soff0, soff1);
  if (threadIdx.x < MROWS) lcnt[threadIdx.x] = 0;  // visible after the first barrier

  float M = -INFINITY, Lsum = 0.f;
  f32x4 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x4{0, 0, 0, 0};
  uint64_t top[16];
#pragma unroll
  for (int L = 0; L < 16; ++L) top[L] = 0;
  const uint32_t lcnt_addr = lds_address(&lcnt[lm < MROWS ? lm : 0]);
  const uint32_t cand_addr = lds_address(&cand[lm < MROWS ? lm : 0][0]);

  // lane-constant LDS offsets of the MFMA operands (the swizzle term of the
  // rows an operand touches depends on the lane only)
  const int kq0 = tile_off(c16, g), kq1 = tile_off(c16, 4 + g);  // + 2048 kb
  int voff[4];  // + 4096 s2 + 2048 h
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    voff[dt] = tile_off(4 * g + (c16 >> 2), 2 * dt + ((c16 & 3) >> 1)) + ((c16 & 1) << 3);

  // merge landmark slot L's candidate buffer into its top list (whole wave)
  auto merge_slot = [&](int L) __attribute__((always_inline)) {
    const int n = min(lcnt[w * 16 + L], CAP);
    uint64_t c = (l < n) ? cand[w * 16 + L][l] : 0ull;
    c = wave_sort_desc_first<CAP>(c);
    top[L] = wave_merge_top(top[L], c);
    const uint64_t kth = uniform_read(top[L], k - 1);
    if (l == 0) lcnt[w * 16 + L] = 0;
    if (c16 == L && kth != 0ull) th = fmaxf(th, key_score(kth));
  };

  auto compute_tile = [&](const uint8_t* kl, const uint8_t* vl, int64_t t0)
      __attribute__((always_inline)) {
    float sc[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 a = {0, 0, 0, 0};
      a = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(kl + kq0 + 2048 * kb)), q.v[0], a);
      a = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(kl + kq1 + 2048 * kb)), q.v[1], a);
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[kb][r] = a[r];
    }
    if (t0 + kTileKeys > N) {  // ragged last tile of the head: drop keys past N
      __asm__ volatile("" ::: "memory");  // keep this a branch (no if-conversion)
      const int rel = static_cast<int>(N - t0) - 4 * g;  // key 16kb+4g+r valid iff 16kb+r < rel
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * kb + r >= rel) sc[kb][r] = -INFINITY;
    }
    float kbmax[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      kbmax[kb] = fmax_nc(fmax_nc(sc[kb][0], sc[kb][1]), fmax_nc(sc[kb][2], sc[kb][3]));
    const float smax = fmax_nc(fmax_nc(kbmax[0], kbmax[1]), fmax_nc(kbmax[2], kbmax[3]));

    // ---- streaming top-k: only when some score beats its landmark's k-th best.
    // One ballot per score position (uniform branches, rarely taken); lanes
    // with a passing score take a buffer slot with an LDS atomic.  Entries
    // that find their landmark's buffer full wait in `pend` for its merge.
    if (ballot(lm_ok && smax > th)) {
      uint32_t pend = 0;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if (ballot(lm_ok && kbmax[kb] > th)) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool pass = lm_ok && sc[kb][r] > th;
            if (ballot(pass)) {
              if (pass) {
                const int slot = lds_fetch_add1(lcnt_addr);
                if (slot < CAP)
                  lds_store_u64(cand_addr + 8 * slot,
                                make_key(sc[kb][r], static_cast<uint32_t>(t0 + 16 * kb + 4 * g + r)));
                else
                  pend |= 1u << (4 * kb + r);
              }
            }
          }
        }
      }
      while (true) {  // rare: merge the full buffers, then place the pending entries
        const uint64_t full = ballot(pend != 0u);
        if (full == 0ull) break;
        const uint32_t need =
            static_cast<uint32_t>((full | (full >> 16) | (full >> 32) | (full >> 48)) & 0xFFFFull);
#pragma unroll
        for (int L = 0; L < 16; ++L)
          if ((need >> L) & 1u) merge_slot(L);
        if (pend) {
          uint32_t left = 0;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const uint32_t bit = 1u << (4 * kb + r);
              if (pend & bit) {
                float v = sc[kb][r];
                __asm__ volatile("" : "+v"(v));  // keep the key work in this rare path
                const int slot = lds_fetch_add1(lcnt_addr);
                if (slot < CAP)
                  lds_store_u64(cand_addr + 8 * slot,
                                make_key(v, static_cast<uint32_t>(t0 + 16 * kb + 4 * g + r)));
                else
                  left |= bit;
              }
            }
          pend = left;
        }
      }
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
    // O^T[d][lm] += V^T[d][keys] P^T[keys][lm]; K-position 8g + j is key
    // 32 s2 + 4g + j (j < 4) or 32 s2 + 16 + 4g + (j - 4)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      float pp[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pp[r] = p[2 * s2][r];
        pp[4 + r] = p[2 * s2 + 1][r];
      }
      bf16x8 hi, lo;
      split_hi_lo_pk(pp, hi, lo);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(vl + voff[dt] + 4096 * s2));
        const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(vl + voff[dt] + 4096 * s2 + 2048));
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[dt] = mfma_bf16(a, hi, acc[dt]);
        acc[dt] = mfma_bf16(a, lo, acc[dt]);
      }
    }
  };

  // Tile `it` sits in buffer it % 2.  Before using it, wait for this wave's
  // requests (the only ones outstanding); the block barrier then makes every
  // wave's pieces visible and frees the other buffer, whose tile every wave
  // finished one step earlier, for tile it + 1.
  auto step = [&](int it, const uint8_t* cur, uint32_t nxt) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    // a plain barrier: __syncthreads() would add a workgroup release fence
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    const int64_t t0 = kbeg + static_cast<int64_t>(it) * tstride;
    if (it + 1 < ntiles)
      stage_tile_bf16<NT>(Kh, Vh, t0 + tstride, N, nxt, nxt + 8192, w, soff0, soff1);
    if (computes) compute_tile(cur, cur + 8192, t0);
  };
  for (int it = 0; it < ntiles; it += 2) {
    step(it, b0, a1);
    if (it + 1 >= ntiles) break;
    step(it + 1, b1, a0);
  }
  if (!computes) return;

  // flush the candidate buffers: all 16 slots at once, network stage by
  // network stage, so that the 16 independent cross-lane chains overlap
  {
    uint64_t c[16];
#pragma unroll
    for (int L = 0; L < 16; ++L) {
      const int n = min(lcnt[w * 16 + L], CAP);
      c[L] = (l < n) ? cand[w * 16 + L][l] : 0ull;
    }
#pragma unroll
    for (int size = 2; size <= CAP; size <<= 1) {
      const bool desc_block = (l & size) == 0;
#pragma unroll
      for (int stride = size >> 1; stride >= 1; stride >>= 1)
#pragma unroll
        for (int L = 0; L < 16; ++L) c[L] = cmpx_desc(c[L], stride, desc_block);
    }
#pragma unroll
    for (int L = 0; L < 16; ++L) {
      const uint64_t rev = lane_read(c[L], 63 - l);
      top[L] = top[L] > rev ? top[L] : rev;
    }
#pragma unroll
    for (int stride = 32; stride >= 1; stride >>= 1)
#pragma unroll
      for (int L = 0; L < 16; ++L) top[L] = cmpx_desc(top[L], stride, true);
  }
  write_partials<NW>(top, M, Lsum, acc, (bh * splits + split) * MROWS, w, l, g, lm, part_keys,
                     part_cnt, part_stats, part_acc);
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
                                                     uint32_t* __restrict__ gmax) {
  using TR = ScanTraits<T>;
  using E = typename T::elem;
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int64_t bh = blockIdx.y;
  const int lm = w * 16 + c16;
  const bool lm_ok = lm < m;
  if (w * 16 >= m) return;  // whole wave beyond the landmarks
  typename TR::QReg q;
  // lanes past m read landmark m - 1 (their maxima are not stored): the
  // loads stay unconditional, so the compiler's wait counts stay exact
  TR::load_q(q, Ql + (bh * m + (lm_ok ? lm : m - 1)) * kD, true, g);
  const int64_t ntiles = (N + kTileKeys - 1) / kTileKeys;
  const E* Kh = K + bh * N * kD;
  for (int j = 0; j < kThetaTilesPerBlock; ++j) {
    const int gi = blockIdx.x * kThetaTilesPerBlock + j;
    const int64_t t0 = ((static_cast<int64_t>(gi) * ntiles) / groups) * kTileKeys;
    uint64_t best = 0;
    f32x4 sc[4];
    TR::score_tile_global(Kh, t0, N, q, c16, g, sc);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const f32x4 a = sc[kb];
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
    if (g == 0 && lm_ok) gmax[(bh * m + lm) * groups + gi] = static_cast<uint32_t>(best >> 32);
  }
}

// Every key in groups of GS consecutive keys (GS = 1: each key is a group,
// so the threshold is the exact k-th largest score; GS = 16 or 64: the
// maximum of each 16-key block or 64-key tile).  grid (key tiles, BH), 256
// threads; wave w: landmarks 16w..16w+15.  Scores use the scan's operand
// layout and accumulation order, so they are bitwise the scores the scan
// computes.
template <class T, int GS>
__global__ __launch_bounds__(256) void k_theta_fine(const typename T::elem* __restrict__ K,
                                                   const typename T::elem* __restrict__ Ql,
                                                   int64_t N, int m, int groups,
                                                   uint32_t* __restrict__ gmax) {
  static_assert(GS == 1 || GS == 16 || GS == 64, "groups of 1, 16 or 64 keys");
  using TR = ScanTraits<T>;
  const int l = lane_id(), g = l >> 4, c16 = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  if (w * 16 >= m) return;  // whole wave beyond the landmarks
  const int64_t bh = blockIdx.y;
  const int lm = w * 16 + c16;
  const bool lm_ok = lm < m;
  typename TR::QReg q;
  TR::load_q(q, Ql + (bh * m + (lm_ok ? lm : m - 1)) * kD, true, g);
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTileKeys;
  f32x4 sc[4];
  TR::score_tile_global(K + bh * N * kD, t0, N, q, c16, g, sc);
  uint32_t* G = gmax + (bh * m + (lm_ok ? lm : 0)) * groups;
  uint64_t tbest = 0;  // running group maximum (GS = 16, 64)
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    uint64_t key[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = t0 + 16 * kb + 4 * g + r;
      key[r] = t < N ? make_key(sc[kb][r], static_cast<uint32_t>(t)) : 0ull;
    }
    if constexpr (GS == 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + 16 * kb + 4 * g + r;
        if (lm_ok && t < N) G[t] = static_cast<uint32_t>(key[r] >> 32);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) tbest = key[r] > tbest ? key[r] : tbest;
      if (GS == 16 || kb == 3) {  // end of a group: combine the 4 lane groups
#pragma unroll
        for (int mask = 16; mask <= 32; mask <<= 1) {
          const uint64_t o = lane_read(tbest, l ^ mask);
          tbest = o > tbest ? o : tbest;
        }
        const int64_t gi = GS == 16 ? (t0 >> 4) + kb : static_cast<int64_t>(blockIdx.x);
        if (g == 0 && lm_ok && gi < groups) G[gi] = static_cast<uint32_t>(tbest >> 32);
        tbest = 0;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// merge of the per-split partials
// ---------------------------------------------------------------------------

// 256 threads per block; a merge block handles landmark (block) lm of head
// bh for part p of P and combines the splits s = p, p + P, p + 2P, ...; wave
// w takes the w-th, (w+4)-th, ... of them in batches of 8 (loads first, then
// the arithmetic; only a split's stored entries are loaded).  A split's top list only
// enters the merge network when its best key beats the wave's current k-th
// best.  FINAL (P = 1): writes idx_out (ascending) and Vl.  Otherwise the
// block's combined top list and softmax state go to the out_* arrays in the
// layout of the scan's partials with P "splits", for a FINAL pass.
//
// Leading blocks (x < nsb) of the launch do step 4's scatter instead: wave w
// of block x sorts segment 4x + w (mita_bucket.hpp).  The merge blocks
// follow: block nsb + j is landmark block j % mx of part j / mx (P parts).
// The final pass has one trailing block per head that writes the expert
// attention's dispatch order (write_item_order) and its short-item blocks'
// items (write_item_blocks): both need only the experts' totals, which the
// scan launch's prefix blocks left.
template <bool FINAL, int NWM>
__global__ __launch_bounds__(256) void k_merge(
    const uint64_t* __restrict__ part_keys, const int32_t* __restrict__ part_cnt,
    const float* __restrict__ part_stats, const float* __restrict__ part_acc, int m, int k,
    int mrows, int splits, int32_t* __restrict__ idx_out, float* __restrict__ vl,
    float* __restrict__ vl_copy, uint64_t* __restrict__ out_keys, int32_t* __restrict__ out_cnt,
    float* __restrict__ out_stats, float* __restrict__ out_acc, int nsb, int mx, int P,
    BucketArgs ba) {
  static_assert(NWM == 1 || NWM == 4, "one or four waves per landmark");
  constexpr int kBatch = 8;
  // one LDS area: four scatter waves, or the merge's cross-wave exchange
  constexpr int kMergeLds = NWM * 64 * 12 + NWM * 8;
  constexpr int kLds = 4 * sizeof(ScatterLds) > kMergeLds ? 4 * sizeof(ScatterLds) : kMergeLds;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];
  const int l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const int64_t bh = blockIdx.y;
  if (FINAL && (ba.item_order != nullptr || ba.item_blocks != nullptr) &&
      blockIdx.x == gridDim.x - 1) {  // trailing block
    if (w == 0 && ba.item_order != nullptr)
      write_item_order(ba.totals, ba.m, ba.tile, ba.tpb, bh, ba.item_order);
    if (w == 1 && ba.item_blocks != nullptr)
      write_item_blocks(l < ba.m ? ba.totals[bh * ba.m + l] : 0, ba.m, ba.tpb, ba.ipb, ba.nbx, bh,
                        ba.item_blocks, reinterpret_cast<int*>(smem));
    return;
  }
  if (static_cast<int>(blockIdx.x) < nsb) {  // whole block: step 4's scatter
    const int seg = static_cast<int>(blockIdx.x) * 4 + w;
    if (seg < ba.nseg)
      scatter_segment(ba.route, ba.counts, ba.m, ba.nseg, ba.N, ba.tile, ba.tpb, ba.totals,
                      ba.colpre, ba.offsets, ba.offsets_copy, ba.item_start, ba.perm,
                      ba.perm_copy, seg, ba.seglen, bh, reinterpret_cast<ScatterLds*>(smem)[w]);
    return;
  }
  auto tops = reinterpret_cast<uint64_t(*)[64]>(smem);                   // [NWM][64]
  auto sacc = reinterpret_cast<float(*)[64]>(smem + NWM * 64 * 8);       // [NWM][64]
  float* sM = reinterpret_cast<float*>(smem + NWM * 64 * 12);            // [NWM]
  float* sL = sM + NWM;                                                  // [NWM]
  const int j = static_cast<int>(blockIdx.x) - nsb;
  const int bx = j % mx, p = j / mx;
  // NWM = 4: the block's four waves share landmark bx.  NWM = 1: each wave
  // takes a landmark of its own (4 * bx + w) and all of its splits.
  const int lm = NWM == 4 ? bx : bx * 4 + w;
  const int wi = NWM == 4 ? w : 0;  // the wave's index among its landmark's waves
  if (lm >= m) return;  // whole wave (NWM = 1 only)
  const int64_t row0 = bh * splits * mrows + lm;  // partial row of split s: row0 + s * mrows
  const int nmine = splits > p ? (splits - p + P - 1) / P : 0;  // splits of this block

  uint64_t top = 0;
  float Mw = -INFINITY, Lw = 0.f, aw = 0.f;
  for (int i0 = wi; i0 < nmine; i0 += NWM * kBatch) {
    int cnt[kBatch];
    float Ms[kBatch], Ls[kBatch], as[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + NWM * u;
      const int64_t r = row0 + static_cast<int64_t>(p + P * i) * mrows;
      const bool ok = i < nmine;
      cnt[u] = ok ? part_cnt[r] : 0;
      Ms[u] = ok ? part_stats[r * 2] : 0.f;
      Ls[u] = ok ? part_stats[r * 2 + 1] : 0.f;
      as[u] = ok ? part_acc[r * kD + l] : 0.f;
    }
    uint64_t lst[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {  // only the split's cnt stored entries
      const int i = i0 + NWM * u;
      const int64_t r = row0 + static_cast<int64_t>(i < nmine ? p + P * i : p) * mrows;
      lst[u] = l < cnt[u] ? part_keys[r * kTopCap + l] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (i0 + NWM * u >= nmine) break;
      const float Mn = fmaxf(Mw, Ms[u]);
      const float f0 = fast_exp2(Mw - Mn), f1 = fast_exp2(Ms[u] - Mn);
      Lw = Lw * f0 + Ls[u] * f1;
      aw = aw * f0 + as[u] * f1;
      Mw = Mn;
      if (cnt[u] > 0 && uniform_read(lst[u], 0) > uniform_read(top, k - 1))
        top = wave_merge_top(top, lst[u]);
    }
  }
  uint64_t t = top;
  float Mt = Mw, Lt = Lw, at = aw;
  if constexpr (NWM == 4) {
    tops[w][l] = top;
    sacc[w][l] = aw;
    if (l == 0) {
      sM[w] = Mw;
      sL[w] = Lw;
    }
    __syncthreads();
    if (w != 0) return;

    t = tops[0][l];
#pragma unroll
    for (int v = 1; v < 4; ++v) {
      const uint64_t o = tops[v][l];
      if (uniform_read(o, 0) > uniform_read(t, k - 1)) t = wave_merge_top(t, o);
    }
    Mt = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) Mt = fmaxf(Mt, sM[v]);
    Lt = 0.f;
    at = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (sM[v] == -INFINITY) continue;  // a wave that had no split
      const float f = fast_exp2(sM[v] - Mt);
      Lt += sL[v] * f;
      at += sacc[v][l] * f;
    }
  }
  if constexpr (FINAL) {
    int32_t ix = (l < k) ? static_cast<int32_t>(key_index(t)) : INT32_MAX;
    ix = wave_sort_asc_i32(ix);
    if (l < k) idx_out[(bh * m + lm) * k + l] = ix;
    const float val = at / Lt;
    vl[(bh * m + lm) * kD + l] = val;
    if (vl_copy != nullptr) vl_copy[(bh * m + lm) * kD + l] = val;
  } else {
    // this block's combination, as partial number p of P (every block of
    // the grid had at least one split, so Mt is finite)
    const int64_t r = (bh * P + p) * mrows + lm;
    const uint64_t nz = ballot(t != 0ull);
    if (t != 0ull) out_keys[r * kTopCap + l] = t;
    if (l == 0) {
      out_cnt[r] = __popcll(nz);
      out_stats[r * 2] = Mt;
      out_stats[r * 2 + 1] = Lt;
    }
    out_acc[r * kD + l] = at;
  }
}

// ---------------------------------------------------------------------------

// the bucket bodies' arguments for this call
static BucketArgs bucket_args(const Shape& s, const int32_t* route, const Workspace& ws,
                              int32_t* offsets_copy, int32_t* perm_copy) {
  BucketArgs a;
  a.route = route;
  a.counts = ws.counts;
  a.colpre = ws.colpre;
  a.totals = ws.totals;
  a.offsets = ws.offsets;
  a.offsets_copy = offsets_copy;
  a.item_start = ws.item_start;
  a.item_order = ws.item_order;
  a.item_blocks = ws.item_blocks;
  a.ipb = s.attend_ipb;
  a.nbx = s.attend_nbx;
  a.perm = ws.perm;
  a.perm_copy = perm_copy;
  a.m = s.m;
  a.nseg = s.nseg;
  a.seglen = s.rseg;
  a.tile = kAttendTile;
  a.tpb = s.attend_tpb;
  a.N = s.NA;  // the items sorted: queries, or (query, expert) assignments when s > 1
  return a;
}

// 1D grid: splits * BH scan blocks, then m * BH blocks for step 4's prefix
template <int NW>
static hipError_t launch_scan_nw(const Shape& s, const void* K, const void* V, const Workspace& ws,
                                 const BucketArgs& ba, hipStream_t st) {
  const float c2 = s.scale * kLog2e;
  const dim3 grid(static_cast<unsigned>((s.scan_splits + s.m) * s.BH));
  if (s.dtype == 1) {
    const bool exact = s.theta_groups > 0 && !s.theta_sampled && s.theta_gs == 1;
    // Non-temporal K/V loads when Q, K and V together overflow the
    // last-level cache: the scan's single pass over K and V then leaves the
    // Q rows that routing has just read in that cache for the expert
    // attention's gathers (256 MB per MI355X; measured: -6% per step at
    // 2^18 tokens x 4 heads, -2% at 2^20).  When everything fits, ordinary
    // loads keep K and V there as well, and the attention's staging of the
    // experts' rows hits it (+6% per step with non-temporal loads at 2^14
    // tokens x 32 heads).
    const bool nt = 3.0 * static_cast<double>(s.BH) * static_cast<double>(s.N) * kD * 2 >
                    static_cast<double>(kLastLevelCacheBytes);
    const uint16_t* Kp = static_cast<const uint16_t*>(K);
    const uint16_t* Vp = static_cast<const uint16_t*>(V);
    const uint16_t* Qlp = static_cast<const uint16_t*>(ws.ql);
    if (exact && s.k <= 32)  // about k candidates per landmark: a 32-entry buffer holds them
      hipLaunchKernelGGL((k_scan_bf16<NW, 32, false>), grid, dim3(256), 0, st, Kp, Vp, Qlp,
                         ws.theta, s.N, s.m, s.k, s.scan_splits, c2, ws.part_keys, ws.part_cnt,
                         ws.part_stats, ws.part_acc, static_cast<int>(s.BH), ba);
    else if (exact)
      hipLaunchKernelGGL((k_scan_bf16<NW, 64, false>), grid, dim3(256), 0, st, Kp, Vp, Qlp,
                         ws.theta, s.N, s.m, s.k, s.scan_splits, c2, ws.part_keys, ws.part_cnt,
                         ws.part_stats, ws.part_acc, static_cast<int>(s.BH), ba);
    else if (nt)
      hipLaunchKernelGGL((k_scan_bf16<NW, kCandCap, true>), grid, dim3(256), 0, st, Kp, Vp, Qlp,
                         ws.theta, s.N, s.m, s.k, s.scan_splits, c2, ws.part_keys, ws.part_cnt,
                         ws.part_stats, ws.part_acc, static_cast<int>(s.BH), ba);
    else
      hipLaunchKernelGGL((k_scan_bf16<NW, kCandCap, false>), grid, dim3(256), 0, st, Kp, Vp, Qlp,
                         ws.theta, s.N, s.m, s.k, s.scan_splits, c2, ws.part_keys, ws.part_cnt,
                         ws.part_stats, ws.part_acc, static_cast<int>(s.BH), ba);
  } else {
    hipLaunchKernelGGL((k_scan_f32<NW>), grid, dim3(256), 0, st,
                       static_cast<const float*>(K), static_cast<const float*>(V),
                       static_cast<const float*>(ws.ql), ws.theta, s.N, s.m, s.k, s.scan_chunk,
                       s.scan_splits, c2, ws.part_keys, ws.part_cnt, ws.part_stats, ws.part_acc,
                       static_cast<int>(s.BH), ba);
  }
  return hipGetLastError();
}

template <class T>
static hipError_t launch_theta_t(const Shape& s, const void* K, const Workspace& ws,
                                 hipStream_t st) {
  using E = typename T::elem;
  const int64_t ktiles = (s.N + kTileKeys - 1) / kTileKeys;
  if (!s.theta_sampled && s.theta_gs == 1) {
    hipLaunchKernelGGL((k_theta_fine<T, 1>), dim3(ktiles, s.BH), dim3(256), 0, st,
                       static_cast<const E*>(K), static_cast<const E*>(ws.ql), s.N, s.m,
                       s.theta_groups, ws.gmax);
  } else if (!s.theta_sampled && s.theta_gs == 16) {
    hipLaunchKernelGGL((k_theta_fine<T, 16>), dim3(ktiles, s.BH), dim3(256), 0, st,
                       static_cast<const E*>(K), static_cast<const E*>(ws.ql), s.N, s.m,
                       s.theta_groups, ws.gmax);
  } else if (!s.theta_sampled) {
    hipLaunchKernelGGL((k_theta_fine<T, 64>), dim3(ktiles, s.BH), dim3(256), 0, st,
                       static_cast<const E*>(K), static_cast<const E*>(ws.ql), s.N, s.m,
                       s.theta_groups, ws.gmax);
  } else {
    hipLaunchKernelGGL(k_theta_sample<T>, dim3(s.theta_groups / kThetaTilesPerBlock, s.BH),
                       dim3(256), 0, st, static_cast<const E*>(K), static_cast<const E*>(ws.ql),
                       s.N, s.m, s.theta_groups, ws.gmax);
  }
  return hipGetLastError();
}

hipError_t launch_threshold(const Shape& s, const void* K, const Workspace& ws,
                            hipStream_t st) {
  if (s.theta_groups == 0) return hipSuccess;
  return s.dtype == 1 ? launch_groups_bf16(s, K, ws, st) : launch_theta_t<F32>(s, K, ws, st);
}

hipError_t launch_scan(const Shape& s, const void* K, const void* V, const Workspace& ws,
                       const int32_t* route, hipStream_t st) {
  const BucketArgs ba = bucket_args(s, route, ws, nullptr, nullptr);
  switch (s.scan_waves) {
    case 1: return launch_scan_nw<1>(s, K, V, ws, ba, st);
    case 2: return launch_scan_nw<2>(s, K, V, ws, ba, st);
    default: return launch_scan_nw<4>(s, K, V, ws, ba, st);
  }
}

// one merge pass: nsb scatter blocks (step 4) ahead of the merge blocks
template <bool FINAL, int NWM>
static void merge_pass(const Shape& s, const uint64_t* keys, const int32_t* cnt,
                       const float* stats, const float* acc, int splits, int P, int nsb,
                       const BucketArgs& ba, int32_t* idx_out, float* vl, float* vl_copy,
                       uint64_t* out_keys, int32_t* out_cnt, float* out_stats, float* out_acc,
                       hipStream_t st) {
  const int mx = NWM == 4 ? s.m : (s.m + 3) / 4;
  // the final pass has one more block per head: the attention's dispatch order
  const int order = FINAL && (ba.item_order != nullptr || ba.item_blocks != nullptr) ? 1 : 0;
  hipLaunchKernelGGL((k_merge<FINAL, NWM>), dim3(nsb + mx * P + order, s.BH), dim3(256), 0, st, keys, cnt,
                     stats, acc, s.m, s.k, s.mrows, splits, idx_out, vl, vl_copy, out_keys,
                     out_cnt, out_stats, out_acc, nsb, mx, P, ba);
}

hipError_t launch_merge(const Shape& s, const Workspace& ws, int32_t* idx_out, float* vl_copy,
                        const int32_t* route, int32_t* offsets_copy, int32_t* perm_copy,
                        hipStream_t st) {
  // one wave per landmark (four landmarks per block) when a landmark has at
  // most 4 partials, else four waves per landmark (the one wave merges its
  // partials one after another: shorter only for a few).  The first pass
  // also carries step 4's scatter, a wave per route segment.
  const BucketArgs ba = bucket_args(s, route, ws, offsets_copy, perm_copy);
  const int nsb = (s.nseg + 3) / 4;
  if (s.merge_parts > 1) {  // first level: merge_parts partial combinations per landmark
    const int per = (s.scan_splits + s.merge_parts - 1) / s.merge_parts;
    if (per <= 4)
      merge_pass<false, 1>(s, ws.part_keys, ws.part_cnt, ws.part_stats, ws.part_acc,
                           s.scan_splits, s.merge_parts, nsb, ba, nullptr, nullptr, nullptr,
                           ws.part2_keys, ws.part2_cnt, ws.part2_stats, ws.part2_acc, st);
    else
      merge_pass<false, 4>(s, ws.part_keys, ws.part_cnt, ws.part_stats, ws.part_acc,
                           s.scan_splits, s.merge_parts, nsb, ba, nullptr, nullptr, nullptr,
                           ws.part2_keys, ws.part2_cnt, ws.part2_stats, ws.part2_acc, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (s.merge_parts <= 4)
      merge_pass<true, 1>(s, ws.part2_keys, ws.part2_cnt, ws.part2_stats, ws.part2_acc,
                          s.merge_parts, 1, 0, ba, idx_out, ws.vl, vl_copy, nullptr, nullptr,
                          nullptr, nullptr, st);
    else
      merge_pass<true, 4>(s, ws.part2_keys, ws.part2_cnt, ws.part2_stats, ws.part2_acc,
                          s.merge_parts, 1, 0, ba, idx_out, ws.vl, vl_copy, nullptr, nullptr,
                          nullptr, nullptr, st);
    return hipGetLastError();
  }
  if (s.scan_splits <= 4)
    merge_pass<true, 1>(s, ws.part_keys, ws.part_cnt, ws.part_stats, ws.part_acc, s.scan_splits,
                        1, nsb, ba, idx_out, ws.vl, vl_copy, nullptr, nullptr, nullptr, nullptr,
                        st);
  else
    merge_pass<true, 4>(s, ws.part_keys, ws.part_cnt, ws.part_stats, ws.part_acc, s.scan_splits,
                        1, nsb, ba, idx_out, ws.vl, vl_copy, nullptr, nullptr, nullptr, nullptr,
                        st);
  return hipGetLastError();
}

}  // namespace mita
