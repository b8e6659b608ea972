/*
 * moe.h -- C ABI of a single-GPU MoE expert layer for AMD Instinct MI355X
 * (gfx950): softmax top-k routing, permute into per-expert groups, grouped
 * SwiGLU GEMM (forward, backward dX, backward dW), unpermute + gate-weighted
 * combine, and the backward of each step.
 *
 * Sources, cited by page title and section:
 *  [CANN-MoE]  "MoE算子优化：动态路由硬件加速与零拷贝通信实践" (gtnt.cn):
 *              s2.1 routing = Softmax -> Top-k -> mask; s2.2 experts are
 *              fully-connected layers computed tile by tile; s4.2 router FP32.
 *  [MoE-ops]   Huawei MoE training operator article (feedman.me): VectorSort
 *              section, Fig. 3 (reorder / anti-reorder of tokens); Host-Device
 *              section, Fig. 4 (token-dispatch preprocessing without a host wait).
 *  [Pangu-QA]  QbitAI article on the Pangu Ultra MoE report (rjtj.cn):
 *              dropless training; expert backward split into dW and dX;
 *              experimental results (output = weighted sum of shared and
 *              routed experts).
 *  [MindSpore-DSv3] "昇思MindSpore助力天翼云提供极致MoE大模型训练性能"
 *              (mindspore.cn): 01.1 tokens sorted inside a machine; 03.3
 *              GroupedMatmul over all experts.
 *
 * Conventions for every call
 *  - Pointers are DEVICE pointers unless stated; tensors are dense row-major
 *    and 16-byte aligned.  ``dt`` selects the storage type of token rows and
 *    expert weights: MOE_F32 (fp32) or MOE_BF16 (bf16 bits, fp32 arithmetic
 *    inside).  Router weights, logits, gates and their gradients are fp32.
 *  - Every call only enqueues work on ``stream`` (a hipStream_t; NULL is the
 *    null stream) and returns; none synchronises and none reads device data
 *    back to the host, so no output size depends on the routing: permuted
 *    buffers have R = T*k rows (dropless, [Pangu-QA]), or R = E*C in the
 *    drop-and-pad variant (moe_permute_capacity).
 *  - The caller owns every buffer, including workspaces.  The library keeps no
 *    device memory; its only global state is the per-device CU count and the
 *    thread-local text of the last error.
 *  - Arguments are validated on the host before any launch.  Errors:
 *    MOE_ERR_INVALID_ARG (null pointer, misalignment, negative or
 *    inconsistent size), MOE_ERR_UNSUPPORTED (outside the supported shapes:
 *    1 <= k <= E <= 1024, H and I multiples of 64, sizes below 2^31 elements
 *    per tensor), MOE_ERR_WORKSPACE (workspace too small), MOE_ERR_LAUNCH (the
 *    runtime rejected a launch).  T == 0 is a successful no-op.  Device data
 *    is not checked: logits must be finite; offsets and row maps must come
 *    from moe_permute / moe_permute_capacity.  A row index outside [0, R)
 *    stands for a dropped pair (reads as zeros, writes nothing); every other
 *    index is clamped to its buffer, so bad device data gives wrong numbers,
 *    never an out-of-bounds access.
 *  - Results are bitwise reproducible run to run (no floating-point atomics;
 *    every reduction has a fixed order).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* hipStream_t */

enum { MOE_F32 = 0, MOE_BF16 = 1 };
enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_LAUNCH = 4
};

/* Text for a status code; static storage. */
const char* moe_status_string(int status);
/* Detail of the last failing call on this host thread ("" if none). */
const char* moe_last_error(void);
/* ABI version of this header (bumped on any signature change). */
int moe_abi_version(void);

/* ---------------------------------------------------------------- router
 * Router projection, kept in fp32 ([CANN-MoE] s4.2):
 *   logits[T,E] = x[T,H] . Wg[H,E] + bias[E]     (bias nullable)
 * x has storage type dt and is widened to fp32; products accumulate in fp32.
 * For bf16 x with H and T multiples of 256 and E a multiple of 64 the
 * products run on the bf16 matrix cores: Wg is split into three bf16 parts
 * (together exact to fp32), K is cut into 8 slices summed in fp64, and the
 * result stays within a few fp32 ulps of the exact product.  That path needs
 * a workspace of moe_router_workspace_bytes(T,H,E,dt) bytes (256-byte
 * aligned, contents scratch); for other shapes the size is 0 and ws may be
 * NULL.
 */
size_t moe_router_workspace_bytes(int T, int H, int E, int dt);
int moe_router_logits(const void* x, int dt, const float* wg, const float* bias,
                      int T, int H, int E, float* logits, void* ws, size_t ws_bytes,
                      moe_stream_t stream);

/* Backward of moe_router_logits:
 *   dx[T,H]  = dlogits . Wg^T        (written, storage type dt)
 *   dwg[H,E] = x^T . dlogits         (written, fp32)
 *   dbias[E] = sum_t dlogits[t,:]    (written, fp32; nullable)
 * Same workspace as the forward.  On the matrix-core path dwg and dbias are
 * exact to fp32 like the logits; bf16 dx is formed from the high bf16 part
 * of each factor only (it is stored in bf16: its error stays within a few
 * bf16 roundings of the exact product).
 * flags: 0, or MOE_ROUTER_WG_SPLIT: ws still holds the split of this same
 * wg that moe_router_logits wrote (same T, H, E; workspace not used since),
 * so the backward skips splitting it again (bits unchanged).  Any other
 * bit gives MOE_ERR_INVALID_ARG.
 */
#define MOE_ROUTER_WG_SPLIT 1
int moe_router_logits_bwd(const float* dlogits, const void* x, int dt, const float* wg,
                          int T, int H, int E, void* dx, float* dwg, float* dbias, int flags,
                          void* ws, size_t ws_bytes, moe_stream_t stream);

/* ---------------------------------------------------------------- routing
 * Softmax -> top-k -> selection ([CANN-MoE] s2.1), one token per wavefront:
 *   idx[t,j]  = the j-th expert by descending fp32 logit; equal logits go
 *               to the lower expert index (int32, [T,k])
 *   gate[t,j] = softmax(logits[t,:])[idx[t,j]] (fp32, [T,k]; not
 *               renormalised over the k chosen experts)
 */
int moe_route(const float* logits, int T, int E, int k, int32_t* idx, float* gate,
              moe_stream_t stream);

/* Backward of the gate values (the selection has no gradient):
 *   dlogits[t,e] = p[t,e] * (dp[t,e] - sum_j gate[t,j] dgate[t,j])
 * with p = softmax(logits[t,:]) recomputed and dp = dgate at the chosen
 * experts, 0 elsewhere.  dlogits is [T,E] fp32, fully written.
 */
int moe_route_bwd(const float* logits, const int32_t* idx, const float* dgate,
                  int T, int E, int k, float* dlogits, moe_stream_t stream);

/* ---------------------------------------------------------------- permute
 * Reorder of tokens into contiguous per-expert groups ([MoE-ops] VectorSort,
 * Fig. 3; the counts stay on the device, [MoE-ops] Host-Device section, Fig. 4):
 *   counts[e]       number of (token, slot) pairs routed to e           [E]
 *   offsets[e]      exclusive scan of counts; offsets[E] = T*k           [E+1]
 *   row_id_map[t,j] row of pair (t,j): offsets[e] + number of tokens t' < t
 *                   that chose e (rows of a group keep token order)      [T,k]
 *   src_token[r]    token that row r came from                           [T*k]
 *   xp[r,:]         = x[src_token[r],:], a bit copy                      [T*k,H]
 * ws must hold moe_permute_workspace_bytes(T,E,k) bytes (contents scratch).
 * xp may be NULL: then only counts, offsets and the maps are written (no row
 * is copied, x may be NULL too) -- the recompute variant below reads token
 * rows from x through src_token instead.
 */
size_t moe_permute_workspace_bytes(int T, int E, int k);
int moe_permute(const void* x, int dt, const int32_t* idx, int T, int H, int E, int k,
                void* xp, int32_t* counts, int32_t* offsets, int32_t* row_id_map,
                int32_t* src_token, void* ws, size_t ws_bytes, moe_stream_t stream);

/* Load statistics of one routing step, from the per-expert counts (e.g.
 * moe_permute's), for the balance term of [CANN-MoE] s4.3 (0.01 times the
 * coefficient of variation of the experts' loads) and for an EP planner that
 * watches per-group loads ([Pangu-QA] MoE training analysis):
 *   load[e]          = counts[e] / N, N = sum of counts       fp32 [E], nullable
 *   group_counts[g]  = sum of counts[e], g*epg <= e < (g+1)*epg  int32 [E/epg], nullable
 *   cv[0]            = std(counts) / mean(counts)              fp32
 *   cv[1]            = std(group_counts) / mean(group_counts)  fp32 ([2], nullable)
 * std is the population standard deviation (divided by the number of
 * values).  When N == 0 every load and both cv are 0.  epg (experts per EP
 * group) must divide E; epg == E gives one group (cv[1] = 0).  One block,
 * fp64 inside, each output rounded once to its type.  counts must be >= 0
 * with N < 2^31 (true for moe_permute's; not checked on the device).
 */
int moe_load_stats(const int32_t* counts, int E, int experts_per_group, float* load, float* cv,
                   int32_t* group_counts, moe_stream_t stream);

/* moe_permute for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, outputs and bits as moe_permute, without the workspace
 * arguments.  Its rank workspace is a file-scope device array of
 * moe_permute_noalloc_max_scratch_bytes() bytes (4 MiB) that each GPU the
 * library runs on holds until the process ends; the call allocates nothing.
 * Limit: moe_permute_workspace_bytes(T, E, k) must not exceed that size
 * (T*k up to 2^24 pairs at E = 256, 2^22 at E = 1024); larger shapes get
 * MOE_ERR_UNSUPPORTED.  Every call on one GPU uses that GPU's one array, so
 * calls that overlap on one GPU (different streams, no ordering between them)
 * race and give wrong maps; calls ordered on one stream are safe.
 */
size_t moe_permute_noalloc_max_scratch_bytes(void);
int moe_permute_noalloc(const void* x, int dt, const int32_t* idx, int T, int H, int E, int k,
                        void* xp, int32_t* counts, int32_t* offsets, int32_t* row_id_map,
                        int32_t* src_token, moe_stream_t stream);

/* Drop-and-pad permute, the variant the pages compare dropless training with
 * ([CANN-MoE] s4.3 capacity factor 1.2; [Pangu-QA] MoE training analysis):
 * every expert owns C rows, R = E*C (C = ceil(factor * T*k / E) for a
 * capacity factor; any C >= 0 is accepted).
 *   counts[e]       pairs routed to e, dropped or not                    [E]
 *   offsets[e]      e*C                                                  [E+1]
 *   row_id_map[t,j] e*C + rank if the pair's rank among e's pairs in token
 *                   order is below C, else -1 (dropped)                  [T,k]
 *   src_token[r]    token of row r, -1 for a row no pair fills           [E*C]
 *   xp[r,:]         x[src_token[r],:], zeros for unfilled rows (nullable) [E*C,H]
 * The grouped GEMMs then run on whole padded groups (offsets as above),
 * combine and its backward skip dropped pairs, and the backward's dyp must
 * have its unfilled rows cleared (moe_clear_empty_rows) so that padded rows
 * stay exact zeros through dX and dW.  Same workspace as moe_permute.
 */
int moe_permute_capacity(const void* x, int dt, const int32_t* idx, int T, int H, int E, int k,
                         int C, void* xp, int32_t* counts, int32_t* offsets,
                         int32_t* row_id_map, int32_t* src_token, void* ws, size_t ws_bytes,
                         moe_stream_t stream);

/* buf[r,:] = 0 for every row r < R with src_token[r] < 0 (rows of a
 * drop-and-pad buffer that no pair fills); other rows are untouched.
 * buf is [R,H] of type dt. */
int moe_clear_empty_rows(const int32_t* src_token, int R, int dt, int H, void* buf,
                         moe_stream_t stream);

/* Backward of the permute (adjoint of the row copy), fp32 sums:
 *   dx[t,:] = sum_j dxp[row_id_map[t,j],:] + add0[t,:] + add1[t,:]
 * add0/add1 are optional [T,H] tensors of type dt (nullable), e.g. the shared
 * expert's and the router's input gradients.  dx is written.  dxp has R rows
 * (T*k dropless, E*C drop-and-pad); a dropped pair adds nothing.
 */
int moe_permute_bwd(const void* dxp, const int32_t* row_id_map, int dt, int T, int H, int k,
                    int R, const void* add0, const void* add1, void* dx, moe_stream_t stream);

/* Anti-reorder and gate-weighted combine ([MoE-ops] VectorSort; [Pangu-QA]
 * experimental results; the shared expert enters with weight 1):
 *   y[t,:] = y_shared[t,:] + sum_{j=0..k-1} gate[t,j] * yp[row_id_map[t,j],:]
 * summed in fp32 in ascending j; y_shared nullable.  yp has R rows; a
 * dropped pair (drop-and-pad) adds nothing.
 */
int moe_unpermute_combine(const void* yp, const int32_t* row_id_map, const float* gate,
                          const void* y_shared, int dt, int T, int H, int k, int R, void* y,
                          moe_stream_t stream);

/* Backward of moe_unpermute_combine:
 *   dyp[row_id_map[t,j],:] = gate[t,j] * dy[t,:]          (every pair's row written)
 *   dgate[t,j]             = <dy[t,:], yp[row_id_map[t,j],:]>   (fp32)
 * yp and dyp have R rows; a dropped pair writes no row and gets dgate 0.
 */
int moe_unpermute_combine_bwd(const void* dy, const void* yp, const int32_t* row_id_map,
                              const float* gate, int dt, int T, int H, int k, int R, void* dyp,
                              float* dgate, moe_stream_t stream);

/* ---------------------------------------------------------------- grouped GEMM
 * GroupedMatmul SwiGLU experts ([MindSpore-DSv3] 03.3; [CANN-MoE] s2.2) over
 * the groups g0 <= e < g0+G of a permuted buffer of R rows.  Group e owns
 * rows [offsets[e], offsets[e+1]) (read on the device).  Expert weights are
 * indexed e - g0 and stored whole per expert:
 *   w13 [G,2I,H]: rows 0..I-1 gate projection, rows I..2I-1 up projection
 *   w2  [G,H,I]
 * Row indices into xp/h13/act/yp/... are absolute; rows of other groups are
 * not touched (remote experts).  An optional shared expert runs on its own
 * T rows in the same launch (a dense group with its own weights).
 * Arithmetic: dt products, fp32 accumulation; outputs stored as dt.
 *
 * Workspace: ws (nullable) of moe_gmm_workspace_bytes() bytes (320 KiB plus
 * 256), 256-byte aligned, holding the tile scheduler's counters and the
 * forward's per-row-tile completion counters and per-tile start words.  It must be zero-filled before
 * its first use; every call returns it to zero when it completes.  With it,
 * the workgroups of each XCD take their tiles from a shared counter (a
 * workgroup that starts late, e.g. while another kernel still holds its CU,
 * just takes fewer tiles) and the forward runs as one launch (below); with
 * ws == NULL they take a fixed share.  Results are identical either way
 * (each tile is computed whole, in the same order, by one workgroup).  Calls
 * that run concurrently (on different streams) need separate workspaces.
 * The int at byte offset 44 is a sticky error word: a forward wait that
 * ran past one second (only possible when concurrent calls share a
 * workspace) gives up and sets it to 1; it is never cleared by the library.
 */
size_t moe_gmm_workspace_bytes(void);
typedef struct moe_shared_expert {
  int T;             /* rows of the shared expert (tokens) */
  const void* x;     /* [T,H]  input rows (forward, dW) */
  const void* w13;   /* [2I,H] */
  const void* w2;    /* [H,I]  */
  void* h13;         /* [T,2I] forward out; bwd_dx in */
  void* act;         /* [T,I]  forward out; bwd_dw in */
  void* y;           /* [T,H]  forward out */
  const void* dy;    /* [T,H]  bwd_dx / bwd_dw in */
  void* dh13;        /* [T,2I] bwd_dx out; bwd_dw in */
  void* dx;          /* [T,H]  bwd_dx out */
  void* dw13;        /* [2I,H] bwd_dw out */
  void* dw2;         /* [H,I]  bwd_dw out */
} moe_shared_expert;

/* Forward:  h13 = xp . w13[e]^T        (saved, [R,2I])
 *           act = silu(h13[:, :I]) * h13[:, I:]   (saved, [R,I]; silu(z) = z/(1+e^-z))
 *           yp  = act . w2[e]^T        ([R,H])
 * The activation is computed in fp32 from the gate and up values as h13
 * stores them (rounded to dt), so the backward, which reads h13, and
 * moe_grouped_gemm_bwd_dw_recompute see the same g and u.
 * With a workspace, both products run in one persistent launch: a row
 * tile's yp tiles start once every h13/act tile of that row tile is stored
 * (per-row-tile counters), so the second product fills the rounds the first
 * leaves partly idle.  Groups averaging half a tile or less, and windows of
 * more than 16384 row tiles, run as two launches. */
int moe_grouped_gemm_fwd(const void* xp, const int32_t* offsets, int g0, int G, int R,
                         int dt, int H, int I, const void* w13, const void* w2,
                         void* h13, void* act, void* yp, const moe_shared_expert* shared,
                         void* ws, size_t ws_bytes, moe_stream_t stream);

/* Backward dX ([Pangu-QA]: dX is computed apart from dW):
 *   dact = dyp . w2[e];  g = h13[:, :I], u = h13[:, I:], s = sigmoid(g)
 *   dh13[:, :I] = dact * u * s * (1 + g (1 - s));  dh13[:, I:] = dact * g * s
 *   dxp = dh13 . w13[e]                                   ([R,H])
 */
int moe_grouped_gemm_bwd_dx(const void* dyp, const int32_t* offsets, int g0, int G, int R,
                            int dt, int H, int I, const void* w13, const void* w2,
                            const void* h13, void* dh13, void* dxp,
                            const moe_shared_expert* shared, void* ws, size_t ws_bytes,
                            moe_stream_t stream);

/* Backward dW, contraction over each group's rows (K = its row count):
 *   dw2[e]  = dyp_e^T . act_e     ([G,H,I])
 *   dw13[e] = dh13_e^T . xp_e     ([G,2I,H])
 * A group with no rows gets exact zeros. */
int moe_grouped_gemm_bwd_dw(const void* xp, const void* act, const void* dyp, const void* dh13,
                            const int32_t* offsets, int g0, int G, int R, int dt, int H, int I,
                            void* dw13, void* dw2, const moe_shared_expert* shared,
                            void* ws, size_t ws_bytes, moe_stream_t stream);

/* dX and dW in one call: the outputs of moe_grouped_gemm_bwd_dx followed by
 * moe_grouped_gemm_bwd_dw (same arguments, same bits), computed in two
 * persistent launches that each pair one dX product with the weight-gradient
 * product that does not depend on it -- [dact + SwiGLU bwd | dw2], then
 * [dxp | dw13] -- so the weight-gradient tiles fill the rounds the dX
 * products leave partly idle (the first launch keeps whole rounds of its
 * long tiles; the dw2 tiles of the largest groups beyond that run at the
 * start of the second).  [Pangu-QA] keeps dW apart from dX so that dW
 * can overlap communication; on one GPU it overlaps the dX products instead.
 * Shapes the paired launches do not cover (a shared expert with no rows, no
 * routed rows, groups averaging half a tile or less) run the two calls'
 * launches.  Same workspace as the other grouped-GEMM calls.
 */
int moe_grouped_gemm_bwd(const void* xp, const void* act, const void* dyp,
                         const int32_t* offsets, int g0, int G, int R, int dt, int H, int I,
                         const void* w13, const void* w2, const void* h13, void* dh13,
                         void* dxp, void* dw13, void* dw2, const moe_shared_expert* shared,
                         void* ws, size_t ws_bytes, moe_stream_t stream);

/* ---------------------------------------------------------------- recompute variant
 * Fine-grained recompute in place of saved activations ([Pangu-QA], the
 * memory-saving part: modules such as the permute and the activation
 * function are recomputed instead of the whole layer): neither xp nor act has
 * to live from the forward to the backward.
 *  - moe_permute with xp == NULL builds the maps only;
 *  - moe_grouped_gemm_fwd_gather reads routed row r of the first product from
 *    x[src_token[r]] (x [T,H], src_token [R] from moe_permute); the rest is
 *    moe_grouped_gemm_fwd (act [R,I] is still written: the second product
 *    reads it, but nothing needs it afterwards);
 *  - moe_grouped_gemm_bwd_dw_recompute first recomputes act from h13 for the
 *    routed window (rows [offsets[g0], offsets[g0+G])) and for the shared
 *    expert (shared->act from shared->h13), writing it to act / shared->act
 *    (scratch of the call), then computes moe_grouped_gemm_bwd_dw with the
 *    routed xp rows read as x[src_token[r]].  The shared expert reads
 *    shared->x as before.
 * moe_grouped_gemm_bwd_dx needs neither xp nor act and is shared by both
 * variants.  Results are bitwise equal to the saving variant's (the same
 * products in the same order; act is recomputed from the same rounded h13).
 * bf16 only (MOE_ERR_UNSUPPORTED for MOE_F32); x must be below 2 GiB.
 * src_token entries outside [0, T) read zero rows (never out of bounds).
 */
int moe_grouped_gemm_fwd_gather(const void* x, const int32_t* src_token, int T,
                                const int32_t* offsets, int g0, int G, int R, int dt, int H,
                                int I, const void* w13, const void* w2, void* h13, void* act,
                                void* yp, const moe_shared_expert* shared, void* ws,
                                size_t ws_bytes, moe_stream_t stream);

int moe_grouped_gemm_bwd_dw_recompute(const void* x, const int32_t* src_token, int T,
                                      const void* h13, void* act, const void* dyp,
                                      const void* dh13, const int32_t* offsets, int g0, int G,
                                      int R, int dt, int H, int I, void* dw13, void* dw2,
                                      const moe_shared_expert* shared, void* ws, size_t ws_bytes,
                                      moe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
