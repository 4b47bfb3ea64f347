/*
 * mita.h — C ABI of libmita.so: the Mixture-of-Top-k Attention (MiTA)
 * forward pass on one AMD Instinct MI355X (gfx950) GPU.
 *
 * What is computed (per batch b and head h; Q, K, V are [N][d]):
 *   1. m landmark queries Ql by local average pooling of Q, stored in the
 *      input type (fp64 sum and division, one round-to-nearest-even into the
 *      input type).
 *      [P1 "NeurIPS'26：注意力也是FFN？从快权重出发，重新理解高效注意力",
 *       section "用少量地标查询，同时构造全局概括与细节专家";
 *       P2 "NeurIPS 2026 | Mixture-of-Top-k 注意力：从快权重统一高效注意力，
 *       让 Top-k 专家灵活又可复用", section "MiTA：用少量地标查询，同时完成
 *       压缩与专家构造"]
 *   2. One pass over the keys scores S = Ql K^T and feeds two results:
 *      (a) expert i = the k keys with the largest S[i][t] (ties: lower key
 *          index), returned ascending in idx_out — the routed experts;
 *      (b) Vl = softmax(scale * S) V — the landmark values; (Ql, Vl) are the
 *          m compressed key/value pairs of the shared expert.  [P1, P2, same
 *          sections]
 *   3. Query q goes to expert argmax_i q . Ql[i] (ties: lower landmark
 *      index); these dot products are also the compressed-branch logits.
 *      [P1, P2, same sections]
 *   4. Queries are grouped by expert, stably (ascending query index within
 *      each group).  [P1 same section; P2 same section, implementation note]
 *   5. out[q] = softmax over the m + k logits scale*[q.Ql[0..m), q.K[t] for
 *      t in expert(q)] applied to the values [Vl[0..m), V[t] ...]; exactly
 *      m + k pairs, none merged or masked.  [P1, P2 same sections; P3 "And
 *      attention is also FFN? Starting with fast weighting, re-understanding
 *      efficient attention", Figure 3 and Algorithm 1]
 *
 * Memory: every tensor argument is a DEVICE pointer owned by the caller.
 * The library never frees them and keeps none after the call returns,
 * except inside the work it enqueued on `stream` (ordinary stream
 * semantics: keep buffers alive until the stream has passed the call).
 * Inputs are read-only; outputs are fully overwritten; inputs and outputs
 * must not overlap.  Layouts are dense, row-major, [B][H][...] with the
 * innermost dimension contiguous; every pointer must be 16-byte aligned.
 *
 * Work space: one device block per calling stream (up to 8 streams per
 * device), allocated stream-ordered on `stream` (hipMallocAsync) by the
 * first call that needs it and kept for later calls on that stream, which
 * are ordered after it by the stream itself.  A block that is too small for
 * a call is released with hipFreeAsync on its stream and replaced.  A new
 * stream beyond the eighth takes over the least recently used block: every
 * call records an event after its last kernel, and the new stream waits for
 * the old block's event on the GPU (hipStreamWaitEvent) before freeing it in
 * its own order, so the old stream's handle is never used again (it may have
 * been destroyed) and the host never waits.  mita_release_workspace(stream)
 * frees a stream's block early;
 * call it before destroying a stream that made calls, or after the last
 * call, to return the memory.  At 2^20 tokens x 4 heads the block is about
 * 54 MB.  bf16 calls with N <= 256 tokens take a one-launch path instead
 * (one workgroup per head holds the head's keys and values in LDS and runs
 * all five steps): they use no work space at all.  Every kernel of a call
 * runs on `stream`; there is no host synchronisation and no global state
 * besides the cached work-space blocks, the per-device attribute cache and
 * the optional stage profiler.  A per-device mutex serialises the enqueue
 * sequences of concurrent host calls; calls on different streams may run
 * concurrently on the GPU.
 *
 * Errors: every function returns a status.  Arguments are validated on the
 * host before any HIP call; nothing is enqueued when validation fails.  A
 * failed launch returns MITA_ERR_HIP.  Faults during kernel execution show
 * up at the caller's next synchronisation (HIP semantics).  NaN or infinite
 * inputs give unspecified values, not an error.  mita_last_error() returns a
 * human-readable reason for the calling thread's last failure.
 */
#ifndef MITA_H
#define MITA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MITA_VERSION 1

typedef enum {
  MITA_OK = 0,
  MITA_ERR_INVALID_ARG = -1, /* a pointer, size or value breaks the rules below */
  MITA_ERR_UNSUPPORTED = -2, /* valid MiTA, but outside this build's limits */
  MITA_ERR_OOM = -3,         /* work-space allocation failed */
  MITA_ERR_HIP = -4,         /* a HIP call or kernel launch failed */
  MITA_ERR_INTERNAL = -5     /* unexpected internal condition */
} mita_status;

typedef enum {
  MITA_F32 = 0, /* Q, K, V and Ql in fp32; fp32 MFMA and arithmetic */
  MITA_BF16 = 1 /* Q, K, V and Ql in bfloat16; bf16 MFMA, fp32 accumulation */
} mita_dtype;

/* Token grid gh x gw (tokens numbered row-major, gh*gw == N) and landmark
 * grid mh x mw (mh*mw == m).  Landmark i = a*mw + c pools rows
 * [floor(a*gh/mh), ceil((a+1)*gh/mh)) x columns [floor(c*gw/mw),
 * ceil((c+1)*gw/mw)).  A 1D sequence is {1, N, 1, m}: contiguous windows of
 * N/m tokens when m divides N. */
typedef struct {
  int32_t gh, gw, mh, mw;
} mita_grid;

/* Optional intermediate outputs (each pointer may be NULL): device buffers
 * owned by the caller.
 *   ql      [B][H][m][d]  landmark queries, input type
 *   vl      [B][H][m][d]  landmark values, fp32
 *   perm    [B][H][N]     queries ordered by (route, query index)
 *   offsets [B][H][m+1]   start of each expert's group in perm; offsets[m]=N */
typedef struct {
  void* ql;
  float* vl;
  int32_t* perm;
  int32_t* offsets;
} mita_intermediates;

/*
 * mita_forward — the whole forward pass, enqueued on `stream`.
 *
 *   Q, K, V    [B][H][N][d] in `dtype`
 *   dtype      a mita_dtype value
 *   B, H, N    >= 1, N < 2^31, B*H*N*d < 2^40
 *   d          head dimension; this build supports d == 64 only
 *              (others: MITA_ERR_UNSUPPORTED)
 *   grid       pooling geometry; NULL means the 1D grid {1, N, 1, m}
 *   m          number of landmarks/experts, 1 <= m <= N, m <= 64 in this build
 *   k          keys per expert, 1 <= k <= N, k <= 64 in this build
 *   scale      softmax temperature (usually 1/sqrt(d)); finite and > 0.
 *              Selection (step 2a) and routing (step 3) use unscaled dots.
 *   out        [B][H][N][d] fp32
 *   idx_out    [B][H][m][k] int32, ascending key indices of each expert
 *   route_out  [B][H][N] int32 in [0, m)
 *   stream     a hipStream_t (NULL = the default stream)
 *
 * Returns MITA_OK once the work is enqueued.
 */
int mita_forward(const void* Q, const void* K, const void* V, int dtype, int64_t B, int64_t H,
                 int64_t N, int64_t d, const mita_grid* grid, int64_t m, int64_t k, float scale,
                 float* out, int32_t* idx_out, int32_t* route_out, void* stream);

/* mita_forward_ex — mita_forward plus the intermediates of steps 1, 2b and 4
 * (dbg may be NULL, and so may each of its members). */
int mita_forward_ex(const void* Q, const void* K, const void* V, int dtype, int64_t B,
                    int64_t H, int64_t N, int64_t d, const mita_grid* grid, int64_t m,
                    int64_t k, float scale, float* out, int32_t* idx_out, int32_t* route_out,
                    void* stream, const mita_intermediates* dbg);

/*
 * mita_forward_s — MiTA with s experts per query.  The pages name the number
 * s of experts a query is routed to and run their experiments with s = 1
 * ["NeurIPS 2026 | Mixture-of-Top-k 注意力…", section "MiTA：用少量地标查询，
 * 同时完成压缩与专家构造"]; for s > 1 they leave open how the experts are
 * picked and combined.  Reading taken here: query q's experts are the s
 * landmarks with the largest q.Ql[i], best first (ties: lower landmark
 * index), and q attends with one softmax over the m compressed pairs and the
 * k raw pairs of each of its experts — m + s*k pairs, a key held by two of
 * its experts counted once per expert — which is what the Algorithm 1
 * caption of "And attention is also FFN? …" computes (each expert attends
 * its query subset, the parts combined by online softmax).
 *
 *   s          1 <= s <= m, s <= 8 in this build; s > 1 needs MITA_BF16
 *              inputs and N*s < 2^31 (else MITA_ERR_UNSUPPORTED)
 *   routes_out [B][H][N][s] int32: each query's experts, best first
 *   the other arguments, pointer rules and errors as in mita_forward.
 *
 * s = 1 computes exactly what mita_forward computes.  For s > 1 the work
 * space also holds one softmax partial per (query, expert): 264 bytes per
 * token, head and expert.
 */
int mita_forward_s(const void* Q, const void* K, const void* V, int dtype, int64_t B, int64_t H,
                   int64_t N, int64_t d, const mita_grid* grid, int64_t m, int64_t k, int64_t s,
                   float scale, float* out, int32_t* idx_out, int32_t* routes_out, void* stream);

/*
 * mita_forward_noalloc — mita_forward for callers that cannot allocate
 * device memory: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc.  It computes exactly what mita_forward
 * computes with the same kernels, but its work space is a static device
 * array of 64 MiB (one per device, allocated when the library's code object
 * loads and held until the process ends) instead of a cached
 * hipMallocAsync block: the call makes no hipMalloc, hipMallocAsync,
 * hipFree, hipFreeAsync or other allocating call, and records no event (the
 * stage profiler skips it).  Every call on a device shares that device's
 * array, so calls that overlap on one GPU race: issue them on one stream, or
 * order them.  Nothing in the array needs to start at zero; each call writes
 * every part it later reads.
 *
 * Same arguments, pointer rules and errors as mita_forward, plus
 * MITA_ERR_UNSUPPORTED (with the byte counts in mita_last_error()) when the
 * call's work space would exceed the 64 MiB array; nothing is enqueued then.
 * The 2^20-token 4-head workload (m = k = 64) needs about 60 MB.
 */
int mita_forward_noalloc(const void* Q, const void* K, const void* V, int dtype, int64_t B,
                         int64_t H, int64_t N, int64_t d, const mita_grid* grid, int64_t m,
                         int64_t k, float scale, float* out, int32_t* idx_out,
                         int32_t* route_out, void* stream);

/*
 * mita_dense_attention — dense (full) attention, the baseline the pages time
 * MiTA against ["NeurIPS 2026 | Mixture-of-Top-k 注意力…", section
 * "长序列建模：实际运行时间也能明显缩短"; P1, section "长序列建模：训练时间从
 * 10.6小时降至2.4小时"]: out[q] = softmax over all N logits scale*q.K[t],
 * applied to V.  A flash-attention kernel (one pass over K and V per tile of
 * 64 queries, online softmax, bf16 MFMA with fp32 accumulation; the softmax
 * weights are rounded to bf16 once before the P.V product, as flash-attention
 * kernels do).  Enqueued on `stream`; no work space.
 *
 *   Q, K, V    [B][H][N][d] bfloat16 (MITA_BF16 only in this build;
 *              MITA_F32 gives MITA_ERR_UNSUPPORTED)
 *   B, H, N    >= 1, N < 2^31, B*H <= 65535, B*H*N*d < 2^40
 *   d          64 or 128 in this build (others: MITA_ERR_UNSUPPORTED)
 *   scale      finite and > 0
 *   out        [B][H][N][d] fp32, fully overwritten
 *
 * Same pointer rules and error behaviour as mita_forward.
 */
int mita_dense_attention(const void* Q, const void* K, const void* V, int dtype, int64_t B,
                         int64_t H, int64_t N, int64_t d, float scale, float* out, void* stream);

/*
 * mita_backward — the gradients of MiTA attention for training.  The pages'
 * wall-clock results are training times ["NeurIPS'26：注意力也是FFN？…",
 * section "长序列建模：训练时间从10.6小时降至2.4小时"; "NeurIPS 2026 |
 * Mixture-of-Top-k 注意力…", section "实验结果：接近完整注意力，长序列训练时间
 * 减少约 77%"] but give no backward rule; reading taken here: the experts
 * idx and the routes are constants (selections carry no gradient), and the
 * rounding of the landmark queries into the input type passes gradients
 * unchanged.  Given dout = dL/d out, the call computes dQ, dK, dV of
 * L = sum(dout * out) through the output softmax (step 5), the landmark
 * cross-attention that gives Vl (step 2b) and the pooling (step 1): the
 * landmark queries and values are recomputed from Q, K, V, then every
 * contraction runs on fp32 MFMA with fp32 accumulation.
 *
 *   Q, K, V    [B][H][N][d] in `dtype`, the forward's inputs
 *   dtype, B, H, N, d, grid, m, k, scale   as in mita_forward (d == 64)
 *   idx        [B][H][m][k] int32, the experts (mita_forward's idx_out);
 *              entries outside [0, N) are clamped into it
 *   routes     [B][H][N] int32, one expert per query (mita_forward's
 *              route_out); entries outside [0, m) are clamped into it
 *   dout       [B][H][N][d] fp32
 *   dQ, dK, dV [B][H][N][d] fp32, fully overwritten; must not overlap the
 *              inputs or each other
 *   stream     a hipStream_t (NULL = the default stream)
 *
 * Work space: a cached stream-ordered block as in mita_forward (grown to
 * the larger call's need): the query grouping (4 bytes per token and head)
 * and fp32 partial sums of the landmark gradients (up to 32 KiB per expert
 * work item and 64 KiB per key block of a head).  dK and dV receive the expert
 * step's sums by fp32 atomic adds, so their last bits may differ between
 * runs; dQ is deterministic.  Same pointer rules (16-byte alignment) and
 * error behaviour as mita_forward.
 */
int mita_backward(const void* Q, const void* K, const void* V, int dtype, int64_t B, int64_t H,
                  int64_t N, int64_t d, const mita_grid* grid, int64_t m, int64_t k,
                  float scale, const int32_t* idx, const int32_t* routes, const float* dout,
                  float* dQ, float* dK, float* dV, void* stream);

/*
 * mita_release_workspace — free the work-space block cached for `stream` (a
 * hipStream_t; NULL = the default stream) on the current device.  For
 * callers that destroy streams or want the memory back; no step of the
 * method.  The block is freed in stream order (hipFreeAsync on `stream`),
 * after the calls already enqueued there, so `stream` must still exist.  A
 * stream with no cached block is not an error.  The next mita_forward call
 * on `stream` allocates a new block.  Returns MITA_OK, or MITA_ERR_HIP when
 * no device is current or the free fails.
 */
int mita_release_workspace(void* stream);

/* Static description of a status code (never NULL). */
const char* mita_status_string(int status);

/* Detail of the calling thread's last failed call ("" if none). */
const char* mita_last_error(void);

/* MITA_VERSION of the loaded library. */
int mita_version(void);

/*
 * Stage profiler (for measurement; off by default).  While enabled, each
 * forward call records a pair of HIP events around every stage on
 * `stream`.  Stages, in launch order (the array order of
 * mita_profile_read): pool, landmark_threshold (the top-k pre-threshold's
 * group maxima), route (with the pre-threshold's selection as leading
 * blocks), landmark_scan (with step 4's prefix over the routing counts as
 * trailing blocks), landmark_merge (its first pass carries step 4's
 * scatter), expert_attend, and single_launch (bf16 heads of at most 256
 * tokens run all five steps in one launch, one workgroup per head, with no
 * work space; the other stages then record nothing); each of route,
 * landmark_scan, expert_attend and single_launch is a single kernel launch.
 * Backward calls record bw_zero, bw_pool, bw_landmark_fwd (partials and
 * merge), bw_bucket (count, prefix, scatter), bw_attend (with its
 * reduction), bw_cross (one launch) and bw_pool_grad (reduction and spread);
 * a backward call counts as a call too.  mita_profile_read() waits for the recorded events and
 * returns, per stage, the summed milliseconds and the number of calls since
 * the last mita_profile_enable().  Not thread-safe: profile from one thread.
 *   mita_profile_enable(1) clears the sums and starts recording;
 *   mita_profile_enable(0) stops recording (the sums stay readable).
 */
int mita_profile_enable(int enabled);
int mita_profile_stage_count(void);
const char* mita_profile_stage_name(int stage);
int mita_profile_read(double* ms_per_stage, int64_t* calls, int n_stages);

#ifdef __cplusplus
}
#endif

#endif /* MITA_H */
