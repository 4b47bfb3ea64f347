// kernels_dense.hip — dense attention, the baseline MiTA is timed against.
//
// The pages report MiTA's throughput as a speedup over full attention, which
// every query computes over all N key/value pairs with one softmax
// ("NeurIPS 2026 | Mixture-of-Top-k 注意力…", section
// "长序列建模：实际运行时间也能明显缩短"; "NeurIPS'26：注意力也是FFN？…",
// section "长序列建模：训练时间从10.6小时降至2.4小时").  This kernel gives
// that ratio on the same GPU, with no library attention underneath.
//
// A flash-attention forward for bf16 inputs: grid (query tiles of 64 QB,
// B*H), 4 waves per block, wave w owning QB blocks of 16 queries.  Every
// 64-key tile of the head streams through a two-slot LDS ring by the same
// global-load-to-LDS staging as the landmark scan; each K and V operand
// read from it feeds QB MFMAs (with one 16-query block per wave, the LDS
// reads bounded the kernel).  Per tile and 16-query block:
// Sᵀ = K·Qᵀ on bf16 MFMA, an online softmax in the log2 domain (lazy rescale),
// and Oᵀ += Vᵀ·Pᵀ on bf16 MFMA with P rounded to bf16 once, as
// flash-attention kernels do; fp32 output.
//
// Roofline: 4·N²·d flops per (b, h) on bf16 MFMA (2.5 PFLOP/s dense peak);
// each block reads the head's K and V once, mostly from cache, since all
// resident blocks sweep the keys together.
#include "mita_device.hpp"
#include "mita_internal.hpp"
#include "tile_dma.hpp"

namespace mita {

// 16-query row blocks per wave.  Measured at 2^16 tokens x 8 heads: d = 64
// 821 (one block), 962 (two), 915 (three), 1000 TFLOP/s (four); d = 128 856
// (one), 1126 (two), 812 TFLOP/s (four, one wave per SIMD).
constexpr int kDenseQB64 = 4;
constexpr int kDenseQB128 = 2;

// QB: 16-query row blocks per wave (wave w owns rows 16 (QB w + j), j < QB,
// of the block's 64 QB queries).  Every K and V operand read from LDS feeds
// QB MFMAs, so QB = 2 halves the LDS traffic per flop.
template <int QB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(QB <= 2 ? 3 : 2))) void k_dense_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, int64_t N, float c2, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t b0[16384];  // K tile (8 KiB), then V tile
  __shared__ __attribute__((aligned(16))) uint8_t b1[16384];
  const int l = lane_id(), g = l >> 4, c16 = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const int64_t bh = blockIdx.y;
  int64_t q[QB];  // this lane's query in each row block
#pragma unroll
  for (int j = 0; j < QB; ++j)
    q[j] = static_cast<int64_t>(blockIdx.x) * (64 * QB) + 16 * (QB * w + j) + c16;
  const uint16_t* Kh = K + bh * N * kD;
  const uint16_t* Vh = V + bh * N * kD;
  const int ntiles = static_cast<int>((N + kTileKeys - 1) / kTileKeys);

  // the wave's queries as B operands (rows past N read row N - 1 and are not
  // stored); complete before the first tile request, so that inside the
  // loop the only outstanding requests are tiles
  bf16x8 qv[QB][2];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const uint16_t* qr = Q + (bh * N + (q[j] < N ? q[j] : N - 1)) * kD;
#pragma unroll
    for (int s = 0; s < 2; ++s)
      qv[j][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qr + 32 * s + 8 * g));
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __asm__ volatile("" ::: "memory");

  const uint32_t soff0 = stage_src_off(w, 0, l), soff1 = stage_src_off(w, 1, l);
  const uint32_t a0 = lds_address(b0), a1 = lds_address(b1);
  stage_tile_bf16<false>(Kh, Vh, 0, N, a0, a0 + 8192, w, soff0, soff1);

  float M[QB], Lsum[QB];
  f32x4 acc[QB][4];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    M[j] = -INFINITY;
    Lsum[j] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[j][dt] = f32x4{0, 0, 0, 0};
  }
  const int kq0 = tile_off(c16, g), kq1 = tile_off(c16, 4 + g);  // + 2048 kb
  int voff[4];  // + 4096 s2 + 2048 h
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    voff[dt] = tile_off(4 * g + (c16 >> 2), 2 * dt + ((c16 & 3) >> 1)) + ((c16 & 1) << 3);

  auto compute_tile = [&](const uint8_t* kl, const uint8_t* vl, int64_t t0)
      __attribute__((always_inline)) {
    float sc[QB][4][4];
    {
      u32x4 ko[4][2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        ko[kb][0] = *reinterpret_cast<const u32x4*>(kl + kq0 + 2048 * kb);
        ko[kb][1] = *reinterpret_cast<const u32x4*>(kl + kq1 + 2048 * kb);
      }
      f32x4 a[QB][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < QB; ++j)
          a[j][kb] = mfma_bf16(as_bf16x8(ko[kb][0]), qv[j][0], f32x4{0, 0, 0, 0});
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < QB; ++j) a[j][kb] = mfma_bf16(as_bf16x8(ko[kb][1]), qv[j][1], a[j][kb]);
#pragma unroll
      for (int j = 0; j < QB; ++j)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[j][kb][r] = a[j][kb][r];
    }
    if (t0 + kTileKeys > N) {  // ragged last tile: drop keys past N
      __asm__ volatile("" ::: "memory");  // keep this a branch
      const int rel = static_cast<int>(N - t0) - 4 * g;  // key 16kb+4g+r valid iff 16kb+r < rel
#pragma unroll
      for (int j = 0; j < QB; ++j)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kb + r >= rel) sc[j][kb][r] = -INFINITY;
    }
    float p[QB][4][4];
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        mx = fmax_nc(mx, fmax_nc(fmax_nc(sc[j][kb][0], sc[j][kb][1]),
                                 fmax_nc(sc[j][kb][2], sc[j][kb][3])));
      mx = xor_max(mx, 16);
      mx = xor_max(mx, 32) * c2;
      if (ballot(mx > M[j])) {
        const float Mn = fmaxf(M[j], mx);
        const float alpha = fast_exp2(M[j] - Mn);
        Lsum[j] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[j][dt] *= alpha;
        M[j] = Mn;
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[j][kb][r] = fast_exp2(fmaf(sc[j][kb][r], c2, -M[j]));
          Lsum[j] += p[j][kb][r];
        }
    }
    // Oᵀ[d][q] += Vᵀ[d][keys] Pᵀ[keys][q]; K-position 8g + j is key
    // 32 s2 + 4g + j (j < 4) or 32 s2 + 16 + 4g + (j - 4)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 va[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(vl + voff[dt] + 4096 * s2));
        const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(vl + voff[dt] + 4096 * s2 + 2048));
        va[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        float pp[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pp[r] = p[j][2 * s2][r];
          pp[4 + r] = p[j][2 * s2 + 1][r];
        }
        bf16x8 hi, lo;
        split_hi_lo_pk(pp, hi, lo);  // P in bf16 (the residual is not used)
        (void)lo;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[j][dt] = mfma_bf16(va[dt], hi, acc[j][dt]);
      }
    }
  };

  // Tile `it` sits in buffer it % 2: wait for this wave's requests, then the
  // block barrier makes every wave's pieces visible and frees the other
  // buffer (every wave finished its tile one step earlier) for tile it + 1.
  auto step = [&](int it, const uint8_t* cur, uint32_t nxt) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    // a plain barrier: __syncthreads() would add a workgroup release fence
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    const int64_t t0 = static_cast<int64_t>(it) * kTileKeys;
    if (it + 1 < ntiles) stage_tile_bf16<false>(Kh, Vh, t0 + kTileKeys, N, nxt, nxt + 8192, w, soff0, soff1);
    compute_tile(cur, cur + 8192, t0);
  };
  for (int it = 0; it < ntiles; it += 2) {
    step(it, b0, a1);
    if (it + 1 >= ntiles) break;
    step(it + 1, b1, a0);
  }

  // normalise: the query's weight sum is spread over its 4 lane groups
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    float ls = xor_sum(Lsum[j], 16);
    ls = xor_sum(ls, 32);
    if (q[j] < N) {
      const float f = 1.0f / ls;  // ls >= 1 (the maximum's weight)
      float* o = out + (bh * N + q[j]) * kD;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4*>(o + 16 * dt + 4 * g) = acc[j][dt] * f;
    }
  }
}

// ---- head dimension 128 ------------------------------------------------
//
// The same kernel for d = 128 (the embedding width of the pages' long-sequence
// throughput model, "Mixture-of-Top-k 注意力…", section "长序列建模：实际运行
// 时间也能明显缩短"): each 64-key tile is staged as two halves of 64 features
// (four 8 KiB pieces: K and V, features 0-63 and 64-127, each in the scan's
// swizzled 128-byte-row layout), scores take four 32-wide MFMA steps and
// P.V eight 16-feature output blocks.  Twice the MFMA work per exp of the
// d = 64 kernel.
constexpr int kD2 = 128;

// wave w's pieces of the K and V tile halves at key t0 (rows of 256 bytes in
// HBM; half h = features 64h..64h+63); rows past N re-read row N - 1
__device__ __forceinline__ void stage_tile_bf16_d128(const uint16_t* __restrict__ Kh,
                                                     const uint16_t* __restrict__ Vh, int64_t t0,
                                                     int64_t N, uint32_t buf, int w, int l) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int r = 16 * w + 8 * j + (l >> 3);
    const int c = (l & 7) ^ ((r >> 1) & 7);
    if (t0 + r >= N) r = static_cast<int>(N - 1 - t0);  // ragged last tile
    const uint32_t p = 2048u * static_cast<uint32_t>(w) + 1024u * j;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint16_t* src = Kh + (t0 + r) * kD2 + 64 * h + 8 * c;
      dma16_to_lds<false>(src, buf + 8192u * h + p);                 // K half h
      dma16_to_lds<false>(Vh + (t0 + r) * kD2 + 64 * h + 8 * c, buf + 16384u + 8192u * h + p);
    }
  }
}

// QB: 16-query row blocks per wave, as in k_dense_bf16.
template <int QB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_dense_bf16_d128(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, int64_t N, float c2, float* __restrict__ out) {
  // per stage: K half 0, K half 1, V half 0, V half 1 (8 KiB each)
  __shared__ __attribute__((aligned(16))) uint8_t b0[32768];
  __shared__ __attribute__((aligned(16))) uint8_t b1[32768];
  const int l = lane_id(), g = l >> 4, c16 = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const int64_t bh = blockIdx.y;
  int64_t q[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j)
    q[j] = static_cast<int64_t>(blockIdx.x) * (64 * QB) + 16 * (QB * w + j) + c16;
  const uint16_t* Kh = K + bh * N * kD2;
  const uint16_t* Vh = V + bh * N * kD2;
  const int ntiles = static_cast<int>((N + kTileKeys - 1) / kTileKeys);
  bf16x8 qv[QB][4];  // features 32s + 8g .. +7
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const uint16_t* qr = Q + (bh * N + (q[j] < N ? q[j] : N - 1)) * kD2;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qv[j][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qr + 32 * s + 8 * g));
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __asm__ volatile("" ::: "memory");
  const uint32_t a0 = lds_address(b0), a1 = lds_address(b1);
  stage_tile_bf16_d128(Kh, Vh, 0, N, a0, w, l);

  float M[QB], Lsum[QB];
  f32x4 acc[QB][8];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    M[j] = -INFINITY;
    Lsum[j] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[j][dt] = f32x4{0, 0, 0, 0};
  }
  const int kq0 = tile_off(c16, g), kq1 = tile_off(c16, 4 + g);
  int voff[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    voff[dt] = tile_off(4 * g + (c16 >> 2), 2 * dt + ((c16 & 3) >> 1)) + ((c16 & 1) << 3);

  auto compute_tile = [&](const uint8_t* buf, int64_t t0) __attribute__((always_inline)) {
    float sc[QB][4][4];
    {
      f32x4 a[QB][4];
#pragma unroll
      for (int j = 0; j < QB; ++j)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) a[j][kb] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint8_t* kl = buf + 8192 * h;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const bf16x8 k0 = as_bf16x8(*reinterpret_cast<const u32x4*>(kl + kq0 + 2048 * kb));
          const bf16x8 k1 = as_bf16x8(*reinterpret_cast<const u32x4*>(kl + kq1 + 2048 * kb));
#pragma unroll
          for (int j = 0; j < QB; ++j) {
            a[j][kb] = mfma_bf16(k0, qv[j][2 * h], a[j][kb]);
            a[j][kb] = mfma_bf16(k1, qv[j][2 * h + 1], a[j][kb]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < QB; ++j)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[j][kb][r] = a[j][kb][r];
    }
    if (t0 + kTileKeys > N) {
      __asm__ volatile("" ::: "memory");
      const int rel = static_cast<int>(N - t0) - 4 * g;
#pragma unroll
      for (int j = 0; j < QB; ++j)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kb + r >= rel) sc[j][kb][r] = -INFINITY;
    }
    float p[QB][4][4];
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        mx = fmax_nc(mx, fmax_nc(fmax_nc(sc[j][kb][0], sc[j][kb][1]),
                                 fmax_nc(sc[j][kb][2], sc[j][kb][3])));
      mx = xor_max(mx, 16);
      mx = xor_max(mx, 32) * c2;
      if (ballot(mx > M[j])) {
        const float Mn = fmaxf(M[j], mx);
        const float alpha = fast_exp2(M[j] - Mn);
        Lsum[j] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[j][dt] *= alpha;
        M[j] = Mn;
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[j][kb][r] = fast_exp2(fmaf(sc[j][kb][r], c2, -M[j]));
          Lsum[j] += p[j][kb][r];
        }
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 hi[QB];
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        float pp[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pp[r] = p[j][2 * s2][r];
          pp[4 + r] = p[j][2 * s2 + 1][r];
        }
        bf16x8 lo;
        split_hi_lo_pk(pp, hi[j], lo);  // P in bf16 (the residual is not used)
        (void)lo;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint8_t* vl = buf + 16384 + 8192 * h;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(vl + voff[dt] + 4096 * s2));
          const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(vl + voff[dt] + 4096 * s2 + 2048));
          const bf16x8 va =
              __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int j = 0; j < QB; ++j) acc[j][4 * h + dt] = mfma_bf16(va, hi[j], acc[j][4 * h + dt]);
        }
      }
    }
  };

  auto step = [&](int it, const uint8_t* cur, uint32_t nxt) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    const int64_t t0 = static_cast<int64_t>(it) * kTileKeys;
    if (it + 1 < ntiles) stage_tile_bf16_d128(Kh, Vh, t0 + kTileKeys, N, nxt, w, l);
    compute_tile(cur, t0);
  };
  for (int it = 0; it < ntiles; it += 2) {
    step(it, b0, a1);
    if (it + 1 >= ntiles) break;
    step(it + 1, b1, a0);
  }
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    float ls = xor_sum(Lsum[j], 16);
    ls = xor_sum(ls, 32);
    if (q[j] < N) {
      const float f = 1.0f / ls;
      float* o = out + (bh * N + q[j]) * kD2;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<f32x4*>(o + 16 * dt + 4 * g) = acc[j][dt] * f;
    }
  }
}

hipError_t launch_dense(int dtype, const void* Q, const void* K, const void* V, int64_t BH,
                        int64_t N, int64_t d, float scale, float* out, hipStream_t st) {
  if (dtype != 1) return hipErrorInvalidValue;  // bf16 only
  if (d == kD2) {
    constexpr int QB = kDenseQB128;
    hipLaunchKernelGGL(k_dense_bf16_d128<QB>, dim3((N + 64 * QB - 1) / (64 * QB), BH), dim3(256),
                       0, st, static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                       static_cast<const uint16_t*>(V), N, scale * kLog2e, out);
    return hipGetLastError();
  }
  constexpr int QB = kDenseQB64;
  hipLaunchKernelGGL(k_dense_bf16<QB>, dim3((N + 64 * QB - 1) / (64 * QB), BH), dim3(256), 0, st,
                     static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                     static_cast<const uint16_t*>(V), N, scale * kLog2e, out);
  return hipGetLastError();
}

}  // namespace mita
