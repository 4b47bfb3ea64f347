/*
 * mita_oracle.h — plain fp64 CPU oracle for the Mixture-of-Top-k Attention
 * (MiTA) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, obviously correct
 * definition that the GPU path is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * source, header, table or helper with the GPU library, and the GPU library
 * never calls it.
 *
 * Sources (the method is described in prose only; every formula on the pages
 * is lost, so each step below is the plainest reading of the prose):
 *   [P1] "NeurIPS'26：注意力也是FFN？从快权重出发，重新理解高效注意力"
 *        section "用少量地标查询，同时构造全局概括与细节专家"
 *   [P2] "NeurIPS 2026 | Mixture-of-Top-k 注意力：从快权重统一高效注意力，
 *        让 Top-k 专家灵活又可复用", section "MiTA：用少量地标查询，同时完成
 *        压缩与专家构造"
 *   [P3] "And attention is also FFN? Starting with fast weighting,
 *        re-understanding efficient attention", Figure 3 and Algorithm 1
 *   [P4] "不止提速，还能兼容预训练模型：聊聊MiTA高效注意力", section
 *        "跳出选择困境：把压缩和路由真正结合起来"
 *
 * Conventions for every function:
 *   - one (batch, head) slice at a time; arrays are dense row-major;
 *   - Q, K, V are [N][d] fp64 arrays holding the input values exactly;
 *   - Ql (landmark queries) is [m][d], Vl (landmark values) is [m][d];
 *   - idx is [m][k] int32, ascending within each row; route is [N] int32;
 *   - scores used for selection and routing are plain (unscaled) dot
 *     products; `scale` multiplies logits only inside the two softmaxes;
 *   - return 0 on success, -1 on an invalid argument, -2 on allocation
 *     failure.  Nothing is printed.
 */
#ifndef MITA_ORACLE_H
#define MITA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Rounding applied to the pooled landmark queries (they are stored in the
 * input precision). */
enum {
  MITA_ORACLE_ROUND_NONE = 0, /* keep the fp64 mean */
  MITA_ORACLE_ROUND_F32 = 1,  /* round-to-nearest-even into fp32 */
  MITA_ORACLE_ROUND_BF16 = 2  /* round-to-nearest-even into bfloat16, directly
                                 from fp64 (no intermediate fp32 rounding) */
};

/* Round-to-nearest-even of an fp64 value into bfloat16 (8 significant bits,
 * fp32 exponent range, subnormals with quantum 2^-133), returned as the fp64
 * value of the bfloat16 result.  Overflow gives +-inf; NaN passes through. */
double mita_oracle_round_bf16(double x);

/* Pooling window of landmark i (0 <= i < mh*mw) on a gh x gw token grid
 * (tokens numbered row-major): rows [r0, r1) x columns [c0, c1) with
 *   r0 = floor(a*gh/mh), r1 = ceil((a+1)*gh/mh),
 *   c0 = floor(c*gw/mw), c1 = ceil((c+1)*gw/mw),  i = a*mw + c.
 * A 1D sequence is gh = mh = 1, gw = N, mw = m. */
int mita_oracle_window(int64_t gh, int64_t gw, int64_t mh, int64_t mw, int64_t i,
                       int64_t* r0, int64_t* r1, int64_t* c0, int64_t* c1);

/* Step 1 — landmark queries by local average pooling of Q [P1][P2][P4]:
 * Ql[i][j] = round( sum_{t in W_i} Q[t][j] / |W_i| ), sum and division in
 * fp64, `round_mode` one of MITA_ORACLE_ROUND_*. */
int mita_oracle_pool(const double* Q, int64_t N, int64_t d, int64_t gh, int64_t gw,
                     int64_t mh, int64_t mw, int round_mode, double* Ql);

/* Step 2a — routed experts [P1][P2]: landmark i scores every key with the
 * dot product S[i][t] = Ql[i] . K[t]; expert i is the k best keys, ordering
 * by larger score first and, on equal scores, lower key index first.  Each
 * row of idx is then written in ascending key order.
 * gap (nullable, [m][4]) receives, per landmark, the k-th and (k+1)-th
 * scores of that ordering and, for each of those two keys, the sum of
 * |Ql[i][j]*K[t][j]| over j (a bound for the rounding error of a
 * lower-precision dot product).  When k == N the (k+1)-th entries are
 * -inf and 0. */
int mita_oracle_topk(const double* Ql, const double* K, int64_t N, int64_t d, int64_t m,
                     int64_t k, int32_t* idx, double* gap);

/* Step 2b — landmark values by cross-attention of the landmarks over all N
 * keys [P1][P2]: Vl[i] = sum_t a_t V[t] / sum_t a_t with
 * a_t = exp(scale*S[i][t] - max_u scale*S[i][u]). */
int mita_oracle_landmark_values(const double* Ql, const double* K, const double* V,
                                int64_t N, int64_t d, int64_t m, double scale, double* Vl);

/* Step 3 — routing with one expert per query [P1][P2]: R[q][i] = Q[q] . Ql[i]
 * and route[q] = the lowest i reaching max_i R[q][i].
 * qsel (nullable) lists the nq queries to route; route and top2 are then
 * indexed by position in qsel.  When qsel is NULL, nq must equal N.
 * top2 (nullable, [nq][4]) receives the best and second-best logits (the
 * second over the other landmarks; -inf when m == 1) and their |.| sums. */
int mita_oracle_route(const double* Q, const double* Ql, int64_t N, int64_t d, int64_t m,
                      const int64_t* qsel, int64_t nq, int32_t* route, double* top2);

/* Step 4 — queries grouped by expert [P1][P2]: counts per expert, exclusive
 * offsets [m+1], and perm [N] = all queries ordered by (route, query index). */
int mita_oracle_bucket(const int32_t* route, int64_t N, int64_t m, int32_t* offsets,
                       int32_t* perm);

/* Step 5 — output [P1][P2][P3 Algorithm 1]: query q with expert e=route[q]
 * attends over exactly m + k key/value pairs — the m compressed pairs
 * (key Ql[i], value Vl[i]) followed by the k raw pairs (K[t], V[t]) for t in
 * idx[e] — with one softmax over the scaled logits.  No pair is merged or
 * masked.  qsel (nullable) selects nq queries; out is [nq][d] (or [N][d]).
 * route is indexed by query (length N) regardless of qsel. */
int mita_oracle_output(const double* Q, const double* K, const double* V, const double* Ql,
                       const double* Vl, const int32_t* idx, const int32_t* route, int64_t N,
                       int64_t d, int64_t m, int64_t k, double scale, const int64_t* qsel,
                       int64_t nq, double* out);

/* All five steps over B*H slices laid out [B][H][N][d].  Any output pointer
 * except out, idx and route may be NULL.  Per-slice arrays are stacked in
 * the same [B][H] order. */
int mita_oracle_forward(const double* Q, const double* K, const double* V, int64_t B,
                        int64_t H, int64_t N, int64_t d, int64_t gh, int64_t gw, int64_t mh,
                        int64_t mw, int64_t k, double scale, int round_mode, double* out,
                        int32_t* idx, int32_t* route, double* Ql, double* Vl,
                        int32_t* offsets, int32_t* perm);

/* ---- several experts per query (s >= 1) --------------------------------
 * The pages name the number s of experts a query is routed to and run only
 * s = 1 ([P2], the remark that each query goes to one expert in the
 * experiments; [P3], the configuration named before the concatenation).
 * For s > 1 they state neither how a query picks its experts nor how the
 * pairs of several experts meet.  Reading taken here:
 *   - a query's experts are the s landmarks with the largest logits
 *     Q[q] . Ql[i], ties to the lower landmark index, listed in that order
 *     (the s = 1 rule, repeated over the landmarks not yet taken);
 *   - the query attends over the m compressed pairs followed by the k raw
 *     pairs of each of its s experts, in list order, with one softmax over
 *     all m + s*k scaled logits.  Experts may share keys ([P2]: experts may
 *     pick overlapping pairs); a key held by two of the query's experts is
 *     counted once per expert.  This is what [P3] Algorithm 1 computes when
 *     each expert's query subset is attended separately and the partial
 *     results are combined by online softmax.
 * With s = 1 each function below equals its single-expert counterpart. */

/* Step 3 with s experts: routes is [nq][s] (positions in qsel when qsel is
 * non-NULL), each row the query's s experts in order; 1 <= s <= m. */
int mita_oracle_route_s(const double* Q, const double* Ql, int64_t N, int64_t d, int64_t m,
                        int64_t s, const int64_t* qsel, int64_t nq, int32_t* routes);

/* Step 4 with s experts: offsets [m+1] over all N*s (query, expert)
 * assignments; perm [N*s] = the query of each assignment, ordered by
 * (expert, query index).  The s experts of a query must be distinct. */
int mita_oracle_bucket_s(const int32_t* routes, int64_t N, int64_t m, int64_t s,
                         int32_t* offsets, int32_t* perm);

/* Step 5 with s experts: one softmax over the m compressed pairs and the k
 * raw pairs of each of the query's s experts (routes [N][s], indexed by
 * query regardless of qsel); out is [nq][d] (or [N][d]). */
int mita_oracle_output_s(const double* Q, const double* K, const double* V, const double* Ql,
                         const double* Vl, const int32_t* idx, const int32_t* routes, int64_t N,
                         int64_t d, int64_t m, int64_t k, int64_t s, double scale,
                         const int64_t* qsel, int64_t nq, double* out);

/* Dense attention, the baseline the pages time MiTA against (page 2,
 * section on wall-clock time in long-sequence modelling; page 1, section on
 * long-sequence training time): query q attends over all N key/value pairs
 * with one softmax, out[q] = sum_t softmax_t(scale * Q[q].K[t]) V[t].
 * qsel (nullable) selects nq queries; out is [nq][d] (or [N][d]). */
int mita_oracle_dense(const double* Q, const double* K, const double* V, int64_t N, int64_t d,
                      double scale, const int64_t* qsel, int64_t nq, double* out);

/* Backward pass (training; the pages' wall-clock results are training times:
 * [P1] section "长序列建模：训练时间从10.6小时降至2.4小时"): given dout [N][d],
 * the gradients dQ, dK, dV [N][d] of sum(dout * out) for one (batch, head),
 * out being the forward output with the experts idx [m][k] and routes [N]
 * held fixed (selections carry no gradient) and the rounding of the landmark
 * queries into the input type taken as the identity.  Three parts, in the
 * forward's reverse order: the output softmax of every query over its m + k
 * pairs (into dQ, dK, dV and the landmarks' dQl, dVl), the landmarks'
 * cross-attention over all N keys (into dQl, dK, dV), and the pooling (dQl
 * spread back over each window, divided by its size, into dQ).  Straight
 * loops, fp64. */
int mita_oracle_backward(const double* Q, const double* K, const double* V, int64_t N,
                         int64_t d, int64_t gh, int64_t gw, int64_t mh, int64_t mw, int64_t k,
                         double scale, int round_mode, const int32_t* idx, const int32_t* route,
                         const double* dout, double* dQ, double* dK, double* dV);

/* Number of OpenMP threads the oracle uses (for reporting). */
int mita_oracle_threads(void);

#ifdef __cplusplus
}
#endif

#endif /* MITA_ORACLE_H */
