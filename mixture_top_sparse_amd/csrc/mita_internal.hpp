// mita_internal.hpp — shapes, work-space layout and kernel launchers of the
// MiTA forward pass (host side; no device code here).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mita {

constexpr int kD = 64;           // head dimension supported by this build
constexpr int kMaxM = 64;        // landmarks (= experts)
constexpr int kMaxK = 64;        // keys per expert
constexpr int kTopCap = 64;      // per-split top list length (one key per lane)
constexpr int kCandCap = 8;      // candidate buffer per landmark (bf16 landmark scan)
constexpr int kTileKeys = 64;    // keys per landmark-scan tile
constexpr int64_t kLastLevelCacheBytes = int64_t{256} << 20;  // MI355X Infinity Cache
constexpr int kRouteSeg = 1024;  // queries per routing/bucketing segment
constexpr int kRouteSegSmall = 256;  // the same for short heads (few segments)
constexpr int kAttendTile = 64;  // queries per expert-attention tile
constexpr int kAttendMaxTpb = 16;  // tiles per expert-attention work item, at most
constexpr int kAttendShortItems = 256;  // below this many queries per expert (mean): 2-wave blocks
constexpr int kAttendIpbMax = 8;        // 2-wave blocks: work items per block, at most
constexpr int kPoolChunk = 4096; // tokens per pooling partial sum (fewer, longer blocks stream faster)
constexpr int kPoolDirectMax = 128;  // windows up to this many tokens: one-launch pooling
constexpr int kThetaTilesPerBlock = 1;  // sample tiles per top-k pre-threshold block
constexpr int kThetaMaxGroups = 4096;  // group maxima the pre-threshold selection holds (64 per lane)
constexpr int kSmallMaxN = 256;  // bf16 heads up to this many tokens: one-launch path
constexpr int kMediumMaxN = 1600;  // bf16 heads up to this many tokens: steps 2-4 in one launch
constexpr int kMaxS = 8;         // experts per query, at most

struct Shape {
  int64_t B = 0, H = 0, BH = 0, N = 0;
  int m = 0, k = 0;
  int gh = 0, gw = 0, mh = 0, mw = 0;
  float scale = 0.f;
  int dtype = 0;  // mita_dtype
  // derived
  int mpad = 0;        // m rounded up to 32 (attention pair blocks)
  int kpad = 0;        // k rounded up to 32
  int scan_waves = 0;  // 1, 2 or 4 waves of 16 landmarks
  int mrows = 0;       // scan_waves * 16
  int scan_chunk = 0;  // keys per landmark-scan block (fp32; the bf16 scan interleaves tiles)
  int scan_splits = 0;
  int merge_parts = 0; // first-level merge partitions per landmark (1: single pass)
  int pool_splits = 0; // partial sums per landmark window
  bool pool_direct = false;  // small windows: one-launch pooling (k_pool_direct)
  int theta_groups = 0;// sample groups for the top-k pre-threshold (0: off)
  int theta_gs = 64;    // keys per pre-threshold group: 1, 16 or 64
  bool theta_sampled = false;  // groups are a sample of the 64-key tiles
  int rseg = kRouteSeg;  // queries (assignments) per routing/bucketing segment: 1024, or 256
  int nseg = 0;        // routing segments per head
  int attend_tpb = 0;   // 64-query tiles per expert-attention work item
  int attend_items = 0; // upper bound of work items per head
  bool attend_short = false;    // bf16 with few queries per expert: the 2-wave items kernel
  int attend_ipb = 1;           // its work items per block
  int attend_nbx = 1;           // its blocks per head
  bool attend_balanced = false; // its items assigned to blocks by size (at most 64 per head)
  bool small = false;   // one launch, one workgroup per head, no work space
  bool medium = false;  // scan, selection, routing and bucketing in one launch
  int s = 1;            // experts per query
  int64_t NA = 0;       // (query, expert) assignments per head: N * s
  int cus = 0;          // compute units of the device
};

// Work space carved from one stream-ordered allocation.
struct Workspace {
  double* pool_part = nullptr;   // [BH][m][pool_splits][64] fp64 partial window sums
  void* ql = nullptr;            // [BH][m][64] landmark queries (input type)
  uint32_t* gmax = nullptr;      // [BH][m][theta_groups] order bits of each group's maximum score
  float* theta = nullptr;        // [BH][mrows] top-k pre-threshold (nullptr: off)
  uint64_t* part_keys = nullptr; // [BH][splits][mrows][64] per-split top lists (first
                                 //   part_cnt entries valid, descending)
  int32_t* part_cnt = nullptr;   // [BH][splits][mrows] entries in each per-split top list
  float* part_stats = nullptr;   // [BH][splits][mrows][2] (max in log2 units, sum)
  float* part_acc = nullptr;     // [BH][splits][mrows][64] unnormalised P.V
  uint64_t* part2_keys = nullptr; // the same four arrays with merge_parts in place of splits
  int32_t* part2_cnt = nullptr;
  float* part2_stats = nullptr;
  float* part2_acc = nullptr;
  float* vl = nullptr;           // [BH][m][64] landmark values fp32
  int32_t* counts = nullptr;     // [BH][m][nseg] routed queries per expert and segment
  int32_t* colpre = nullptr;     // [BH][m][nseg] exclusive prefix of counts over segments
  int32_t* totals = nullptr;     // [BH][m] routed queries per expert
  int32_t* offsets = nullptr;    // [BH][m+1]
  int32_t* item_start = nullptr; // [BH][m+1] first attention work item of each expert
  int32_t* item_blocks = nullptr; // [BH][attend_nbx * attend_ipb] short-item blocks' items (-1:
                                  //   empty slot), when attend_balanced
  int32_t* item_order = nullptr; // [BH][2m+1] long-item dispatch order: each expert's first
                                 //   full item ([m+1], exclusive prefix), then the experts
                                 //   by the size of their last item ([m], largest first)
  int32_t* perm = nullptr;       // [BH][NA] queries (s > 1: assignments q*s + j) by expert
  float* pacc = nullptr;         // s > 1: [BH][NA][64] unnormalised P.V per assignment
  float* pstat = nullptr;        // s > 1: [BH][NA][2] (maximum logit in log2 units, weight sum)
};

size_t plan_workspace(const Shape& s, Workspace* ws, char* base);

// Kernel launchers; each returns the launch status.
hipError_t launch_pool(const Shape& s, const void* Q, const Workspace& ws, void* ql_copy,
                       int64_t bh0, int64_t nbh, hipStream_t st);
// the pre-threshold's group maxima (the selection runs in the routing
// launch); no-op when theta_groups == 0
hipError_t launch_threshold(const Shape& s, const void* K, const Workspace& ws,
                            hipStream_t st);
hipError_t launch_groups_bf16(const Shape& s, const void* K, const Workspace& ws, hipStream_t st);
// landmark scan, with step 4's prefix over the routing counts as trailing
// blocks (needs the routes' counts: after launch_route)
hipError_t launch_scan(const Shape& s, const void* K, const void* V, const Workspace& ws,
                       const int32_t* route, hipStream_t st);
// merge of the scan partials, with step 4's scatter as leading blocks of
// its first pass (perm, offsets and the attention work items)
hipError_t launch_merge(const Shape& s, const Workspace& ws, int32_t* idx_out, float* vl_copy,
                        const int32_t* route, int32_t* offsets_copy, int32_t* perm_copy,
                        hipStream_t st);
// routing, with the pre-threshold's selection as its leading blocks
hipError_t launch_route(const Shape& s, const void* Q, const Workspace& ws, int32_t* route_out,
                        hipStream_t st);
hipError_t launch_attend(const Shape& s, const void* Q, const void* K, const void* V,
                         const int32_t* idx, const Workspace& ws, float* out, hipStream_t st);
// several experts per query (s > 1, bf16): top-s routing over the flattened
// [N][s] assignments (with the pre-threshold's selection as leading blocks),
// and the attention's per-assignment partials merged per query
hipError_t launch_route_s(const Shape& s, const void* Q, const Workspace& ws, int32_t* routes,
                          hipStream_t st);
hipError_t launch_attend_multi(const Shape& s, const void* Q, const void* K, const void* V,
                               const int32_t* idx, const Workspace& ws, float* out,
                               hipStream_t st);
// the whole forward pass in one launch for short bf16 sequences (one
// workgroup per head, no work space); small_path_fits says when it applies
bool small_path_fits(const Shape& s);
hipError_t launch_small(const Shape& s, const void* Q, const void* K, const void* V, float* out,
                        int32_t* idx_out, int32_t* route_out, void* ql_copy, float* vl_copy,
                        int32_t* perm_copy, int32_t* off_copy, hipStream_t st);
// steps 2 to 4 in one launch for mid-length bf16 sequences (after pooling,
// before the expert attention): each landmark's exact top k and V_l from
// scores kept in registers, and per head the routes and the bucket order;
// medium_path_fits says when it applies
bool medium_path_fits(const Shape& s);
hipError_t launch_medium(const Shape& s, const void* Q, const void* K, const void* V,
                         const Workspace& ws, int32_t* idx_out, int32_t* route_out,
                         float* vl_copy, int32_t* off_copy, int32_t* perm_copy, hipStream_t st);
// dense attention over all N pairs (the baseline); bf16 only
hipError_t launch_dense(int dtype, const void* Q, const void* K, const void* V, int64_t BH,
                        int64_t N, int64_t d, float scale, float* out, hipStream_t st);

// ---------------------------------------------------------------------------
// backward pass (experts and routes given)
// ---------------------------------------------------------------------------

// its steps, in launch order (launch_backward runs steps first..last)
enum BwStep {
  kBwZero = 0,     // the expert step's per-(expert, key) sums = 0
  kBwPool,         // Ql, as the forward computes it
  kBwLandmarkFwd,  // Vl and the landmarks' log-sum-exp (partials, merge)
  kBwBucket,       // queries grouped by the given routes
  kBwAttend,       // the output softmax per expert item, then dVl, dQl part, D
  kBwCross,        // the landmark cross-attention's backward (stores dK, dV), then
                   // the expert step's key sums added in
  kBwPoolBw,       // dQl in full, spread back over the windows into dQ
  kBwStepCount
};

struct BwPlan {
  int lm_chunk = 0, lm_chunks = 0;        // keys per landmark-forward block, blocks per head
  int cross_chunk = 0, cross_chunks = 0;  // the same for the cross-attention backward
  int nseg = 0;                           // routing segments per head (kRouteSeg queries)
  int tpb = 1;                            // 64-query tiles per expert work item
  int items = 0;                          // upper bound of work items per head
};

struct BwWorkspace {
  Workspace fw;                 // pool_part and ql only
  float* lm_stats = nullptr;    // [BH][lm_chunks][64][2] (max in log2 units, sum)
  float* lm_acc = nullptr;      // [BH][lm_chunks][64][64] unnormalised A.V
  float* vl = nullptr;          // [BH][m][64]
  float* lse2 = nullptr;        // [BH][m] log2-sum-exp2 of the scaled logits (log2 units)
  int32_t* counts = nullptr;    // [BH][m][nseg]
  int32_t* colpre = nullptr;    // [BH][m][nseg]
  int32_t* totals = nullptr;    // [BH][m]
  int32_t* offsets = nullptr;   // [BH][m+1]
  int32_t* item_start = nullptr;// [BH][m+1]
  int32_t* item_order = nullptr;// [BH][2m+1] the expert step's dispatch order (write_item_order)
  int32_t* perm = nullptr;      // [BH][N]
  float* part1 = nullptr;       // [BH][items][2][m][64] per-item dQl, dVl
  float* dql1 = nullptr;        // [BH][m][64] the expert step's dQl
  float* dvl = nullptr;         // [BH][m][64]
  float* dd = nullptr;          // [BH][m] dVl . Vl
  float* part2 = nullptr;       // [BH][4 cross_chunks][64][64] the cross step's dQl
  float* dqlw = nullptr;        // [BH][m][64] dQl / |window|
  float* dke = nullptr;         // [BH][m][k][64] the expert step's dK sums per (expert, key)
  float* dve = nullptr;         // [BH][m][k][64] the same for dV
};

BwPlan plan_backward(const Shape& s, int cus);
size_t plan_bw_workspace(const Shape& s, const BwPlan& bp, BwWorkspace* ws, char* base);
hipError_t launch_backward(const Shape& s, const BwPlan& bp, const BwWorkspace& ws,
                           const void* Q, const void* K, const void* V, const int32_t* idx,
                           const int32_t* route, const float* dout, float* dQ, float* dK,
                           float* dV, hipStream_t st, int first, int last);

}  // namespace mita
