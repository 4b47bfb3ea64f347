// mita_bucket.hpp — step 4's device work: group the queries by expert with a
// stable counting sort ("Mixture-of-Top-k 注意力…", section "MiTA：用少量地标
// 查询，同时完成压缩与专家构造", the implementation remark that queries are
// processed grouped by expert; "And attention is also FFN? …", Algorithm 1
// caption: each expert handles the subset of queries routed to it).
//
// The routing kernel leaves per-segment expert counts (segments of kRouteSeg
// queries, stored expert-major).  Two block bodies finish the sort; neither
// has a launch of its own:
//   bucket_prefix   (one 256-thread block per expert and head): exclusive
//                   prefix of the expert's counts over the segments, and the
//                   expert's total.  Trailing blocks of the landmark-scan
//                   launch, which follows routing on the same stream.
//   scatter_segment (one wave per segment): expert offsets from the totals,
//                   then a stable sort of the segment in LDS (a query's rank
//                   among equal routes inside a group of 64 comes from 6
//                   ballots over the route bits), copied out one expert run
//                   at a time.  Segment 0 publishes the offsets and the first
//                   attention work item of each expert.  Leading blocks of the
//                   first landmark-merge launch, four segments per block.
// Both depend only on the routes and the counts; the expert attention that
// reads their results is the next launch after the merge.
//
// Work items: an expert's queries in runs of up to tpb 64-query tiles
// (item_start[e] = its first item).  write_item_order gives the order in
// which the long-item attention dispatches them.
#pragma once

#include "mita_device.hpp"
#include "mita_internal.hpp"

namespace mita {

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

// Whole 256-thread block: for expert e of head bh, the exclusive prefix of
// its per-segment counts over the segments (colpre) and its total.  wsum:
// 4 ints of LDS.
__device__ __forceinline__ void bucket_prefix(const int32_t* __restrict__ counts, int m, int nseg,
                                              int e, int64_t bh, int32_t* __restrict__ colpre,
                                              int32_t* __restrict__ totals, int* wsum) {
  const int t = threadIdx.x, l = lane_id(), w = wave_id();
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

// LDS of one scatter wave
struct ScatterLds {
  int lbase[kMaxM];   // next local slot of each expert
  int gshift[kMaxM];  // global position minus local slot, per expert
  uint16_t sq[kRouteSeg];  // query index within the segment
  uint8_t se[kRouteSeg];
};

// One wave: stable scatter of segment seg of head bh.  Expert offsets come
// from the per-expert totals (exclusive scan over the m experts); segment 0
// also publishes offsets and the attention work items.  The segment is
// first sorted by route in LDS (ranks from ballots, bases from the routing
// kernel's per-segment counts); the sorted list is then copied out run by
// run, so consecutive lanes store consecutive positions of an expert's
// range instead of one lane per expert region.  The caller gives the four
// waves of a block four consecutive segments: one CU, one XCD, so the
// partial lines they leave at the ends of each run meet in one L2.
__device__ __forceinline__ void scatter_segment(
    const int32_t* __restrict__ route, const int32_t* __restrict__ counts, int m, int nseg,
    int64_t N, int tile, int tpb, const int32_t* __restrict__ totals,
    const int32_t* __restrict__ colpre, int32_t* __restrict__ offsets,
    int32_t* __restrict__ offsets_copy, int32_t* __restrict__ item_start,
    int32_t* __restrict__ perm, int32_t* __restrict__ perm_copy, int seg, int seglen, int64_t bh,
    ScatterLds& L) {
  const int l = lane_id();
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
  // all of the segment's routes in flight at once (seglen <= kRouteSeg)
  constexpr int NG = kRouteSeg / 64;
  const int64_t q0 = static_cast<int64_t>(seg) * seglen;
  const int nq = static_cast<int>(N - q0 < seglen ? N - q0 : seglen);
  int rr[NG];
#pragma unroll
  for (int it = 0; it < NG; ++it)
    rr[it] = 64 * it + l < nq ? route[bh * N + q0 + 64 * it + l] : 0;
  {
    const int cl = l < m ? counts[(bh * m + l) * nseg + seg] : 0;
    const int lex = wave_inclusive_sum(cl) - cl;  // local start of expert l
    if (l < m) {
      L.lbase[l] = lex;
      L.gshift[l] = (incl - c) + colpre[(bh * m + l) * nseg + seg] - lex;
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
    const int pos = ok ? L.lbase[r] + rank : -1;
    if (pos >= 0 && pos < kRouteSeg) {
      L.sq[pos] = static_cast<uint16_t>(64 * it + l);
      L.se[pos] = static_cast<uint8_t>(r);
    }
    if (ok && rank == total - 1) L.lbase[r] += total;  // after every lane's read of lbase[r]
  }
  // copy out in sorted order: lanes l, l+1 of one expert run store adjacent
  // positions
  for (int i = l; i < nq; i += 64) {
    const int e = L.se[i];
    const int pos = e < m ? L.gshift[e] + i : -1;
    if (pos >= 0 && pos < N) {
      const int32_t q = static_cast<int32_t>(q0 + L.sq[i]);
      perm[bh * N + pos] = q;
      if (perm_copy) perm_copy[bh * N + pos] = q;
    }
  }
}

// One wave: the long-item attention's dispatch order for head bh (item_order,
// [2m+1] per head): each expert's full items (tpb tiles) in expert order,
// then each expert's last, partly filled item, largest first (ties: lower
// expert), so that the short items fill the tail of the launch instead of a
// full item starting there (at 2^16 tokens x 4 heads the attention went 41
// -> 34 us).  Stored as the exclusive prefix of the experts' full items
// ([m+1]) and the experts by the size of their last item ([m]).  Needs only
// the experts' totals.
__device__ __forceinline__ void write_item_order(const int32_t* __restrict__ totals, int m,
                                                 int tile, int tpb, int64_t bh,
                                                 int32_t* __restrict__ item_order) {
  const int l = lane_id();
  const int c = l < m ? totals[bh * m + l] : 0;
  const int items = ((c + tile - 1) / tile + tpb - 1) / tpb;
  const int full = items > 0 ? items - 1 : 0;
  const int last = items > 0 ? c - full * tpb * tile : 0;  // queries in the last item
  const int full_incl = wave_inclusive_sum(full);
  int rank = 0;
  for (int j = 0; j < m; ++j) {
    const int lj = __builtin_amdgcn_readlane(last, j);
    rank += (lj > last || (lj == last && j < l)) ? 1 : 0;
  }
  int32_t* F = item_order + bh * (2 * m + 1);
  if (l < m) F[l] = full_incl - full;
  if (l == m - 1) F[m] = full_incl;
  if (items > 0) F[m + 1 + rank] = l;
}

// One wave: head bh's work items assigned to the short-item attention's nbx
// blocks of ipb slots (table [nbx * ipb] per head, -1 = empty slot).  A
// block of consecutive items costs what its items add up to, and at the
// segmentation shapes (20-70 queries per expert) the costliest block held
// twice the median's 16-query sub-tiles.  Here the items are ranked by cost
// (16-query sub-tiles plus two for the item's own staging, largest first)
// and dealt out in a snake: rank r goes to slot r / nbx of block r % nbx,
// or of block nbx - 1 - r % nbx on odd rounds.  Every lane places its own
// item; no block gets more than ceil(total / nbx) <= ipb items.  c: this
// lane's expert total (lanes < m); at most 64 items per head (one per
// lane).  lds: 128 ints of this wave's own (the comparisons read it as
// broadcasts, four values per read).
__device__ __forceinline__ void write_item_blocks(int c, int m, int tpb, int ipb, int nbx,
                                                  int64_t bh, int32_t* __restrict__ table,
                                                  int* lds) {
  const int l = lane_id();
  const int items = l < m ? ((c + kAttendTile - 1) / kAttendTile + tpb - 1) / tpb : 0;
  const int incl = wave_inclusive_sum(items);
  const int total = __builtin_amdgcn_readlane(incl, 63);
  int32_t* T = table + bh * (nbx * ipb);
  for (int i = l; i < nbx * ipb; i += 64) T[i] = -1;
  // lane t: work item t's expert (the experts whose items end at or before
  // t) and its queries
  lds[l] = incl;
  int e = 0;
#pragma unroll
  for (int j = 0; j < 64; j += 4) {
    const int4 v = *reinterpret_cast<const int4*>(lds + j);
    e += (j < m && v.x <= l) + (j + 1 < m && v.y <= l) + (j + 2 < m && v.z <= l) +
         (j + 3 < m && v.w <= l);
  }
  const int es = e < 64 ? e : 63;
  const int ce = static_cast<int>(lane_read(static_cast<uint32_t>(c), es));
  const int fe = static_cast<int>(lane_read(static_cast<uint32_t>(incl - items), es));
  const int q = l < total ? min(ce - (l - fe) * tpb * kAttendTile, tpb * kAttendTile) : 0;
  // sort key: cost (sub-tiles plus two), then the lower item first
  const int key = l < total ? (((q + 15) / 16 + 2) << 6) | (63 - l) : -1;
  lds[64 + l] = key;
  int rank = 0;
#pragma unroll
  for (int j = 0; j < 64; j += 4) {
    const int4 v = *reinterpret_cast<const int4*>(lds + 64 + j);
    rank += (v.x > key) + (v.y > key) + (v.z > key) + (v.w > key);
  }
  if (l < total) {
    const int round = rank / nbx, pos = rank % nbx;
    const int blk = (round & 1) ? nbx - 1 - pos : pos;
    if (round < ipb) T[blk * ipb + round] = l;  // (round < ipb: total <= nbx * ipb)
  }
}

// A work item of the expert-grouped attention kernels (forward and backward).
struct TileInfo {
  int e;      // expert
  int qb;     // first perm slot of this work item
  int qe;     // one past its last perm slot
};

// Work item t of a head covers up to `tpb` consecutive 64-query tiles of one
// expert; item_start[e] is the first item of expert e (exclusive scan of
// ceil(tiles_e / tpb)).  item_start is non-decreasing, so t's expert is the
// number of experts e < m - 1 whose successor starts at or before t.  Every
// lane loads its own expert's entries in one round (item_start[l],
// item_start[l + 1], offsets[l]; offsets[m]); the ballot then names the
// expert and the other values come from lane reads, so a work item costs
// one round of dependent loads instead of a chain of them.
__device__ __forceinline__ bool find_item(const int32_t* __restrict__ item_start,
                                          const int32_t* __restrict__ offsets, int m, int tpb,
                                          int t, TileInfo& ti) {
  const int l = lane_id();
  const int next = l < m - 1 ? item_start[l + 1] : INT32_MAX;
  const int ist = l < m ? item_start[l] : 0;
  const int ofl = l <= m && l < 64 ? offsets[l] : 0;
  const int total = item_start[m];
  const int ofm = offsets[m];
  if (t >= total) return false;
  const int e = __popcll(ballot(next <= t));  // wave-uniform
  const int j0 = (t - __builtin_amdgcn_readlane(ist, e)) * tpb;
  const int oe = e + 1 < 64 ? __builtin_amdgcn_readlane(ofl, e + 1) : ofm;  // offsets[e + 1]
  ti.e = e;
  ti.qb = __builtin_amdgcn_readlane(ofl, e) + kAttendTile * j0;
  ti.qe = min(ti.qb + kAttendTile * tpb, oe);
  return true;
}

// Work item t in the long-item dispatch order (item_order above, the head's
// slice): t < F (= the full items) is full item t - fs[e] of expert e, the
// number of experts whose successor's full items start at or before t; past
// them, t names the last item of expert last[t - F].  One round of loads
// (per lane: fs[l + 1], fs[l], offsets[l]) and one more for a last item.
__device__ __forceinline__ void find_item_ordered(const int32_t* __restrict__ order,
                                                  const int32_t* __restrict__ offsets, int m,
                                                  int tpb, int t, TileInfo& ti) {
  const int l = lane_id();
  const int next = l < m - 1 ? order[l + 1] : INT32_MAX;
  const int fsl = l <= m && l < 64 ? order[l] : 0;
  const int ofl = l <= m && l < 64 ? offsets[l] : 0;
  const int nfull = order[m];
  const int ofm = offsets[m];
  int e, j0;
  bool partial;
  if (t < nfull) {
    e = __popcll(ballot(next <= t));  // wave-uniform
    j0 = (t - __builtin_amdgcn_readlane(fsl, e)) * tpb;
    partial = false;
  } else {
    e = __builtin_amdgcn_readfirstlane(order[m + 1 + (t - nfull)]);
    const int full = (e + 1 < 64 ? __builtin_amdgcn_readlane(fsl, e + 1) : nfull) -
                     __builtin_amdgcn_readlane(fsl, e);
    j0 = full * tpb;
    partial = true;
  }
  const int oe = e + 1 < 64 ? __builtin_amdgcn_readlane(ofl, e + 1) : ofm;  // offsets[e + 1]
  ti.e = e;
  ti.qb = __builtin_amdgcn_readlane(ofl, e) + kAttendTile * j0;
  ti.qe = partial ? oe : min(ti.qb + kAttendTile * tpb, oe);
}

// One block per work item, grid (items per head, heads), the heads
// interleaved in dispatch order (linear block L: head L % heads, position p =
// L / heads).  With item_order the positions follow its order (full items,
// then the last items, largest first); without it (the mid-length path),
// item order.  False past the head's items.
__device__ __forceinline__ bool dispatch_item(const int32_t* __restrict__ item_start,
                                              const int32_t* __restrict__ item_order,
                                              const int32_t* __restrict__ offsets, int m, int tpb,
                                              int64_t& bh, int& p, TileInfo& ti) {
  const int64_t L = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
  bh = L % gridDim.y;
  p = static_cast<int>(L / gridDim.y);
  if (item_order == nullptr)
    return find_item(item_start + bh * (m + 1), offsets + bh * (m + 1), m, tpb, p, ti);
  if (p >= item_start[bh * (m + 1) + m]) return false;
  find_item_ordered(item_order + bh * (2 * m + 1), offsets + bh * (m + 1), m, tpb, p, ti);
  return true;
}

// Arguments of the bucket bodies, passed through the scan and merge launches.
struct BucketArgs {
  const int32_t* route;
  const int32_t* counts;
  int32_t* colpre;
  int32_t* totals;
  int32_t* offsets;
  int32_t* offsets_copy;
  int32_t* item_start;
  int32_t* item_order;
  int32_t* item_blocks;  // the short-item attention's table (or nullptr)
  int ipb, nbx;
  int32_t* perm;
  int32_t* perm_copy;
  int m, nseg, seglen, tile, tpb;
  int64_t N;
};

}  // namespace mita
