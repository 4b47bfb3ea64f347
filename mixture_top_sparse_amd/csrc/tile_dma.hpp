// tile_dma.hpp — 64-key K/V tiles from HBM straight into LDS (global-load-to-
// LDS DMA), shared by the landmark scan and the dense-attention baseline.
//
// Each request moves 16 bytes per lane into a fixed lane*16 slot of a 1 KiB
// piece.  Tile layout: 64 key rows of 128 bytes, 16-byte chunk c of row r
// stored at chunk c ^ ((r >> 1) & 7), so that the 16 rows read by one MFMA
// operand fetch fall on distinct banks.  V stays row-major; the P.V operand
// (8 keys of one feature per lane) comes from the LDS transpose read, which
// hands lane i of each 16-lane group element i of four 8-byte row pieces.
#pragma once

#include "mita_device.hpp"
#include "mita_internal.hpp"

namespace mita {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// s_waitcnt immediates (gfx9 encoding): vmcnt <= n, expcnt and lgkmcnt not
// waited on.  Each staged tile is four requests per lane.
constexpr int kWaitVm0 = 0x0F70;

__device__ __forceinline__ int tile_off(int r, int c) {
  return (r << 7) | ((c ^ ((r >> 1) & 7)) << 4);
}

// Byte offset, inside a tile of 64 rows, of the global 16-byte chunk that
// lane l of wave w fetches for the wave's piece j (rows 16w + 8j .. +7):
// the chunk that lands at the lane's fixed LDS slot under the swizzle.
__device__ __forceinline__ uint32_t stage_src_off(int w, int j, int l) {
  const int r = 16 * w + 8 * j + (l >> 3);
  const int c = (l & 7) ^ ((r >> 1) & 7);
  return static_cast<uint32_t>(r * 128 + c * 16);
}

// LDS accesses of the candidate path, written as assembly: the compiler
// cannot tell these locations from the tile buffers that the in-flight DMA
// writes, and would otherwise wait for every outstanding tile first.  They
// complete before returning (explicit lgkmcnt wait).
template <class P>
__device__ __forceinline__ uint32_t lds_address(P* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)(p)));
}
__device__ __forceinline__ int lds_fetch_add1(uint32_t addr) {
  int old;
  const int one = 1;
  __asm__ volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)"
                   : "=v"(old)
                   : "v"(addr), "v"(one)
                   : "memory");
  return old;
}
__device__ __forceinline__ void lds_store_u64(uint32_t addr, uint64_t v) {
  __asm__ volatile("ds_write_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(addr), "v"(v) : "memory");
}

// One global-load-to-LDS request: each lane's 16 bytes at gaddr land at
// LDS address lds_base + 16 * lane (lds_base wave-uniform, in M0).  Written
// as assembly so that the compiler inserts no waits of its own for it: the
// scan orders every tile with explicit vmcnt waits and block barriers.
// NT: the non-temporal cache policy, for data read exactly once (the
// landmark scan's pass over K and V): the stream then does not displace
// what the last-level cache holds for later kernels.
template <bool NT>
__device__ __forceinline__ void dma16_to_lds(const void* gaddr, uint32_t lds_base) {
  if constexpr (NT)
    __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                     :
                     : "v"(gaddr), "s"(lds_base)
                     : "memory", "m0");
  else
    __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     :
                     : "v"(gaddr), "s"(lds_base)
                     : "memory", "m0");
}

// Wave `w` (wave-uniform) requests its two 1 KiB pieces (rows 16w..16w+15)
// of the K and V tiles starting at key t0 (LDS byte addresses kbuf, vbuf).
// Full tiles use the tile base plus the lane's 32-bit offset; a tile that
// runs past the head's last key re-reads key N-1 for the missing rows (their
// scores are masked and their probabilities are 0).
template <bool NT>
__device__ __forceinline__ void stage_tile_bf16(const uint16_t* __restrict__ Kh,
                                                const uint16_t* __restrict__ Vh, int64_t t0,
                                                int64_t N, uint32_t kbuf, uint32_t vbuf, int w,
                                                uint32_t off0, uint32_t off1) {
  const char* kt = reinterpret_cast<const char*>(Kh + t0 * kD);
  const char* vt = reinterpret_cast<const char*>(Vh + t0 * kD);
  uint32_t o0 = off0, o1 = off1;
  if (t0 + kTileKeys > N) {
    __asm__ volatile("" ::: "memory");  // keep this a branch
    const uint32_t last = static_cast<uint32_t>((N - 1 - t0) * 128);  // byte offset of key N-1
    if ((o0 & ~127u) > last) o0 = last + (o0 & 127u);
    if ((o1 & ~127u) > last) o1 = last + (o1 & 127u);
  }
  const uint32_t p0 = 2048u * static_cast<uint32_t>(w), p1 = p0 + 1024u;
  dma16_to_lds<NT>(kt + o0, kbuf + p0);
  dma16_to_lds<NT>(vt + o0, vbuf + p0);
  dma16_to_lds<NT>(kt + o1, kbuf + p1);
  dma16_to_lds<NT>(vt + o1, vbuf + p1);
}

}  // namespace mita
