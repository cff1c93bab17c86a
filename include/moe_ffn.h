/*
 * moe_ffn.h -- C ABI of the skew-aware MoE expert layer for AMD Instinct MI355X
 * (gfx950).
 *
 * The operations follow the MegaFlux summary (picx.dev/p/e4jAzZ):
 *   - routing statistics: per-expert counts c_e and the skew
 *     kappa = E * sum_e (c_e / sum_j c_j)^2  ("Routing Skew Problem");
 *   - token blocks of at most beta rows, b_e = ceil(c_e / beta), and the
 *     min-max block placement q (E x P) under a per-worker replica budget s
 *     ("Problem Formulation");
 *   - the bounded greedy planner with four searches and the
 *     reduction-aware backward variant C_lambda = max_r (l_r + lambda n_r)
 *     ("Bounded Greedy Search");
 *   - the SwiGLU expert computation and gated combine, and the gradients
 *     dA = D W2^T, dX = dZ W1^T, dW2 = A^T D, dW1 = X^T dZ, with replica
 *     partial weight gradients reduced into the owner in fp32 in a fixed
 *     order ("Forward" / "Backward" and their equations).
 *
 * The P workers of the pages are CU partitions of one GPU: worker r runs on
 * the XCDs {x : x * P / 8 == r} (P in {1, 2, 4, 8}).
 *
 * Conventions for every entry point:
 *   - pointers are DEVICE pointers unless marked (host);
 *   - every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *     default stream) and returns; it never synchronises the host, never
 *     allocates device memory and keeps no state between calls;
 *   - the caller owns every buffer; outputs are overwritten, never
 *     accumulated into;
 *   - the return value is a moe_status, decided on the host from the
 *     arguments alone (nothing is launched when it is not MOE_OK);
 *   - problems only visible on the device (an expert id >= E, a plan that
 *     breaks its constraints) are OR-ed into *status_dev as MOE_DEV_* bits;
 *     the caller zeroes it beforehand and reads it after its own sync;
 *   - `ws` is a caller-provided device workspace of at least
 *     moe_workspace_size(...) bytes, 256-byte aligned.  Calls that share a
 *     workspace must not overlap in time (use one stream per workspace).
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,          /* argument out of range, or a required pointer is NULL */
  MOE_ERR_UNSUPPORTED = -2,  /* valid in principle, not implemented (see each call) */
  MOE_ERR_WORKSPACE = -3,    /* ws is NULL, misaligned or smaller than required */
  MOE_ERR_HIP = -4           /* the HIP runtime refused a launch */
} moe_status;

/* bits OR-ed into *status_dev by device code */
#define MOE_DEV_BAD_EXPERT 1   /* a top-k id >= E (that row is skipped) */
#define MOE_DEV_BAD_PLAN   2   /* block_worker outside [0,P), a worker with more than s
                                  non-home experts, an (expert, worker) pair whose
                                  blocks are not one run (those blocks are skipped),
                                  or a plan that does not fit block_worker */
#define MOE_DEV_BAD_OWNER  4   /* owner[e] outside [0,P) */
#define MOE_DEV_WAIT_TIMEOUT 8 /* a two-phase launch waited over 2 s for rows of its
                                  first phase (its workgroups were not all resident);
                                  the results are not valid */

/* exec_flags of moe_forward and moe_backward */
#define MOE_EXEC_TWO_PHASE 1    /* run FC1 and FC2 (dA and dX) as one two-phase
                                   persistent launch with per-row-tile readiness
                                   counters instead of two launches; the results
                                   are the same bits */
/* With MOE_EXEC_TWO_PHASE, bits 8..15 of exec_flags split each worker's n
 * workgroups (n = G / P, G = the launch's workgroups, one per CU) into
 * producers and consumers: MOE_EXEC_SPLIT(n1), 1 <= n1 < n, lets the first n1
 * run only the first phase (FC1 or dA), publishing each finished row tile,
 * and the other n - n1 run only the second phase (FC2 or dX), each item
 * waiting for its row tile.  0 lets every workgroup run its first-phase items
 * and then its second-phase items.  moe_predict_split picks the mode from the
 * plan.  The results are the same bits in every mode. */
#define MOE_EXEC_SPLIT_SHIFT 8
#define MOE_EXEC_SPLIT(n1) (((n1) & 0xff) << MOE_EXEC_SPLIT_SHIFT)
/* e4m3 weights on the persistent stream kernels (d and d_ff multiples of
 * 256), two launches: every product except the weight gradients runs on the
 * fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4), its activation operand
 * quantized per row and 128 features with power-of-two scales
 * (moe_quantize_act_rows), the weights' codes used as stored and their fp32
 * block scales applied to the accumulators per 128-deep K block.
 *   moe_forward: x, and A = SiLU(G) * U as stored in bf16 (only the rows of
 *   the blocks in use), feed FC1 and FC2; the saved [G, U] come from the
 *   quantized x.
 *   moe_backward: dy feeds dA, and dZ, formed in bf16 from dA (stored in bf16)
 *   and the saved [G, U], feeds dX; the weight gradients are the default
 *   path's, with D and dZ requantized along the tokens.
 * The results differ from the default path by these quantizations (relative
 * error about 2^-5 per value).  MOE_ERR_ARG with the two-phase launch,
 * activations other than bf16, weights other than e4m3, or a layer off the
 * stream kernels. */
#define MOE_EXEC_FP8_ACT 2

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* Optional per-workgroup timeline of the persistent GEMM phases (moe_forward
 * and moe_backward's `timeline` argument): uint64 [MOE_TL_PHASES]
 * [MOE_TIMELINE_MAX_WG][2], entry [phase][g] = {start, end} of workgroup g of
 * that phase's launch on the GPU's constant 100 MHz real-time counter (end:
 * after the workgroup's last item and all its memory operations).  Workgroup g
 * belongs to worker (g % 8) * P / 8.  Written by the persistent 256 x 256
 * stream kernels (bf16 activations, d and d_ff multiples of 256, operands
 * below 2 GiB); other shapes and workgroups beyond the launch leave their
 * entries untouched.  Writing it changes no result. */
#define MOE_TIMELINE_MAX_WG 1024
enum { MOE_TL_FC1 = 0, MOE_TL_FC2 = 1, MOE_TL_DA = 2, MOE_TL_DX = 3, MOE_TL_DW = 4,
       MOE_TL_PHASES = 5 };
typedef enum { MOE_PLAN_FWD = 0, MOE_PLAN_BWD = 1, MOE_PLAN_QUOTA = 2 } moe_plan_mode;

/* One expert layer.  The weights are stored transposed with respect to the
 * pages' X W notation, so that both operands of every forward product are
 * contiguous along the reduction dimension:
 *   w1 [E][2*d_ff][d]: rows 0..d_ff-1 produce G, rows d_ff..2*d_ff-1 produce U;
 *   w2 [E][d][d_ff].
 * act_dtype (MOE_F32 or MOE_BF16) is the dtype of x, y, dy, dx and z_save.
 * w_dtype is MOE_F32 (with act MOE_F32), MOE_BF16 (with act MOE_BF16) or
 * MOE_FP8_E4M3 (OCP e4m3fn codes, act MOE_BF16; forward and backward); fp8 weights
 * carry one fp32 scale per 128x128 block:
 *   w1_scale [E][2*d_ff/128][d/128], w2_scale [E][d/128][d_ff/128].
 * Requires d % 128 == 0 and d_ff % 64 == 0 (fp8: d_ff % 128 == 0). */
typedef struct {
  int E, d, d_ff;
  int act_dtype;
  int w_dtype;
  const void* w1;
  const void* w2;
  const float* w1_scale;
  const float* w2_scale;
} moe_layer;

int moe_abi_version(void);
const char* moe_status_str(int status);

/* Upper bound of the padded slot count: T*k + E*(beta-1). */
size_t moe_max_slots(int T, int k, int E, int beta);
/* Upper bound of sum_e b_e: (T*k + E*(beta-1)) / beta. */
size_t moe_max_blocks(int T, int k, int E, int beta);

/* Workspace needed by moe_route_stats, moe_plan, moe_forward and (when
 * with_backward != 0) moe_backward for these sizes; one workspace serves all
 * of them.  `L` (host) must be valid; returns 0 for invalid arguments and for
 * sizes moe_forward rejects as too large (see there). */
size_t moe_workspace_size(const moe_layer* L, int T, int k, int beta, int P, int s,
                          int with_backward);

/* Routing statistics ("Routing Skew Problem" kappa equation; block
 * definition of "Problem Formulation").
 *   topk_ids [T][k] int32: expert of each (token, slot); id < 0 = no expert.
 *   counts [E]: c_e.  offsets [E+1]: exclusive prefix sum of c.
 *   block_counts [E]: b_e = ceil(c_e/beta).  block_offsets [E+1]: prefix sum of b.
 *   row_to_slot [T*k]: padded slot of routed row i = t*k + j, -1 when id < 0.
 *     Rows of expert e occupy slots beta*block_offsets[e] ... in increasing i.
 *   slot_to_row [moe_max_slots]: inverse map, -1 for padding slots.
 *   kappa [1] (double): E * sum c^2 / (sum c)^2 computed from exact integers
 *     with one IEEE division; 1.0 when nothing is routed.
 * Limits: 1 <= E <= 1024, 1 <= k, 1 <= beta, T >= 0, T*k < 2^31. */
int moe_route_stats(const int32_t* topk_ids, int T, int k, int E, int beta,
                    int32_t* counts, int32_t* offsets, int32_t* block_counts,
                    int32_t* block_offsets, int32_t* row_to_slot, int32_t* slot_to_row,
                    double* kappa, int32_t* status_dev, void* ws, size_t ws_bytes,
                    void* stream);

/* moe_route_stats for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and results without `ws`.  Its per-chunk counts live in
 * a scratch array inside the library, MOE_ROUTE_SCRATCH_BYTES on every GPU it
 * runs on, held until the process ends; the call allocates nothing.  Calls on
 * one GPU share that array: calls that overlap in time on one GPU (two
 * streams, two host threads) race, so serialise them.
 * Errors: as moe_route_stats, plus MOE_ERR_UNSUPPORTED when the counts need
 *   more than the array: ceil(T*k / 256) * E * 4 > MOE_ROUTE_SCRATCH_BYTES
 *   (e.g. T*k above 2,097,152 rows at E = 128); MOE_ERR_HIP when the array's
 *   device address cannot be obtained. */
#define MOE_ROUTE_SCRATCH_BYTES ((size_t)4 << 20)
int moe_route_stats_noalloc(const int32_t* topk_ids, int T, int k, int E, int beta,
                            int32_t* counts, int32_t* offsets, int32_t* block_counts,
                            int32_t* block_offsets, int32_t* row_to_slot,
                            int32_t* slot_to_row, double* kappa, int32_t* status_dev,
                            void* stream);

/* Replica placement and block assignment ("Problem Formulation", "Bounded
 * Greedy Search").  Runs entirely on the device (no host round trip), one
 * workgroup; integer-only, so the result is deterministic.
 *   block_counts [E], block_offsets [E+1]: from moe_route_stats.
 *   owner [E]: h(e) in [0, P), the home worker of each expert.
 *   mode MOE_PLAN_FWD minimises max_r l_r; MOE_PLAN_BWD minimises
 *   max_r (l_r + lambda * n_r), n_r = remote copies of r's experts.
 *   mode MOE_PLAN_QUOTA is the quota-driven solver of the UltraEP reading
 *   notes (section 4, Algorithm 1): a binary search for the smallest load
 *   threshold tau that a greedy quota pass meets; for this mode `lambda` is
 *   the quota floor u_min (>= 1 blocks): no replica is made for fewer blocks.
 *   s = 0 gives fixed placement (every mode).
 * Outputs: q [E][P] blocks of e on r; load [P] = l_r; block_worker
 *   [block_worker_cap entries, e.g. moe_max_blocks]: worker of each block
 *   (expert e's blocks go to its owner first, then to ascending workers;
 *   entries past sum b are untouched); plan_info [4] = {objective, chosen
 *   search 0..3 (4 for MOE_PLAN_QUOTA), replica count, tau (ceil(sum b / P),
 *   or the threshold found by MOE_PLAN_QUOTA)}.
 * Errors: MOE_ERR_ARG for a bad mode, s < 0, lambda < 0 (< 1 with
 *   MOE_PLAN_QUOTA), block_worker_cap < 0 or a null pointer;
 *   MOE_ERR_UNSUPPORTED for E > 512 or P outside {1,2,4,8}; an owner outside
 *   [0, P) sets MOE_DEV_BAD_OWNER in *status_dev; sum b = block_offsets[E]
 *   above block_worker_cap sets MOE_DEV_BAD_PLAN and leaves block_worker
 *   untouched (q, load and plan_info are still written).
 * Limits: 1 <= E <= 512, P in {1,2,4,8}, s >= 0, lambda >= 0. */
int moe_plan(const int32_t* block_counts, const int32_t* block_offsets,
             const int32_t* owner, int E, int P, int s, int mode, int lambda,
             int32_t* q, int32_t* load, int32_t* block_worker, int block_worker_cap,
             int32_t* plan_info, int32_t* status_dev, void* ws, size_t ws_bytes,
             void* stream);

/* Runtime replication gate (MegaFlux summary, "Limitations": enable
 * replication only when the predicted saving exceeds its cost; "Empirical
 * Validation": near-balanced routes gain nothing from replicas).  Applied on
 * the device to a plan made by moe_plan, in place, with no host round trip.
 * A plan's predicted cost is its objective max_r l_r (blocks on the busiest
 * worker) plus rho per replica; rho_milli is rho in thousandths of a block.
 * The plan is kept when
 *     1000 * (fixed-placement objective - plan objective) > rho_milli * replicas
 * or when it has no replica; otherwise q, load and block_worker are rewritten
 * as the fixed placement (every block on its owner) and plan_info becomes
 * {fixed objective, -1, 0, tau}.
 *   block_counts [E], block_offsets [E+1], owner [E]: as given to moe_plan.
 *   q [E][P], load [P], block_worker [block_worker_cap], plan_info [4]:
 *   moe_plan's outputs, read and (when gated off) overwritten.
 * Errors: MOE_ERR_ARG for E < 1, rho_milli < 0, block_worker_cap < 0 or a
 *   null pointer; MOE_ERR_UNSUPPORTED for E > 512 or P outside {1,2,4,8}; an
 *   owner outside [0, P) sets MOE_DEV_BAD_OWNER in *status_dev; a gated-off
 *   plan whose sum b exceeds block_worker_cap sets MOE_DEV_BAD_PLAN and
 *   leaves block_worker untouched. */
int moe_plan_gate(const int32_t* block_counts, const int32_t* block_offsets,
                  const int32_t* owner, int E, int P, int rho_milli, int32_t* q, int32_t* load,
                  int32_t* block_worker, int block_worker_cap, int32_t* plan_info,
                  int32_t* status_dev, void* stream);

/* Predicted time of one forward + backward pass under a pair of plans
 * ("Analytical Resource Management for Fine-grained MoE
 * Computation-Communication Overlap", abstract: a wave-quantized analytical
 * model picks the resource partition before each launch from routed-tile
 * counts and occupancy, with no candidate run).  The partition chosen here is
 * P, the number of CU partitions: call moe_plan for each candidate P (with
 * that P's owners), then this for each, and run with the smallest cost.
 *   counts [E], block_offsets [E+1]: from moe_route_stats.
 *   block_worker_fwd / block_worker_bwd [sum b]: the forward and backward
 *   plans' block workers; owner [E]: h(e) for this P.
 *   num_workgroups: workgroups of the persistent launches (one per CU);
 *   <= 0 takes the device's CU count.
 * Model: worker r owns n = num_workgroups / P workgroups and deals its items
 * round-robin, so each phase lasts as long as its busiest workgroup.  Items:
 * (row tile, N tile) pairs for FC1, FC2, dA and dX, a row tile being up to 256
 * slots of one (expert, worker) run; (segment, 256 x 256 tile) pairs for the
 * weight gradients, replica segments first.  An item costs its K steps of 64
 * plus its epilogue's bytes over 214,000 (what one CU stores in one step).
 * *cost_dev (int64): the sum over the five phases, thousandths of a step.
 * Errors: MOE_ERR_ARG for a non-positive size or a null pointer;
 *   MOE_ERR_UNSUPPORTED for E > 512, P outside {1,2,4,8}, d or d_ff not a
 *   multiple of 256, or num_workgroups not a multiple of P or above 256 P;
 *   a worker outside [0, P) in a plan sets MOE_DEV_BAD_PLAN, an owner outside
 *   [0, P) MOE_DEV_BAD_OWNER in *status_dev. */
int moe_predict_cost(const int32_t* counts, const int32_t* block_offsets,
                     const int32_t* block_worker_fwd, const int32_t* block_worker_bwd,
                     const int32_t* owner, int E, int beta, int P, int d, int d_ff,
                     int num_workgroups, int64_t* cost_dev, int32_t* status_dev, void* stream);

/* Producer/consumer split of the two-phase launches (same page, abstract:
 * the count of communication CTAs of a dependency-coupled overlap pipeline,
 * chosen before the launch from routed-tile counts, residency and split-level
 * readiness, with no candidate run).  On one GPU the pipeline is a
 * direction's pair of GEMM phases, FC1 -> FC2 (backward = 0) or dA -> dX
 * (backward = 1): the second phase's items of a row tile need all of that
 * row tile's first-phase items.  Predicts, for the plan block_worker, the
 * time of every mode and picks one:
 *   mode -1: two launches (exec_flags 0);
 *   mode 0: one two-phase launch, every workgroup runs its first-phase items
 *     and then its second-phase items (MOE_EXEC_TWO_PHASE);
 *   mode n1, 1 <= n1 < n = num_workgroups / P: one launch, n1 producer
 *     workgroups per worker run the first phase and n - n1 consumers the
 *     second (MOE_EXEC_TWO_PHASE | MOE_EXEC_SPLIT(n1)).
 * Model: worker r has T_r row tiles (as moe_predict_cost cuts them); items
 * are tile-major and dealt round-robin; an item costs its K steps of 64 plus
 * its epilogue bytes over 214,000; a first-phase item i dealt over m
 * workgroups ends at (i / m + 1) c1, a row tile is ready when its last
 * first-phase item ends, and a second-phase item starts when its workgroup is
 * free and its row tile is ready.  Integers throughout.
 *   counts [E], block_offsets [E+1]: from moe_route_stats; block_worker
 *   [sum b]: the direction's plan.  num_workgroups <= 0: the device's CUs.
 *   costs_dev (int64) [n + 1]: mode m's time at index m + 1, thousandths of a
 *   step.  choice_dev (int32): the mode of smallest time, ties to the lower
 *   mode.
 * Errors: as moe_predict_cost; a worker outside [0, P) sets MOE_DEV_BAD_PLAN
 *   in *status_dev. */
int moe_predict_split(const int32_t* counts, const int32_t* block_offsets,
                      const int32_t* block_worker, int E, int beta, int P, int d, int d_ff,
                      int num_workgroups, int backward, int64_t* costs_dev, int32_t* choice_dev,
                      int32_t* status_dev, void* stream);

/* Forward expert layer ("Backward" section, expert-computation equation):
 *   y_t = sum_{j: id_tj >= 0} p_tj * W2_e (SiLU(G) * U),  [G; U] = W1_e x_t,
 * executed over the planned blocks: worker r's CU partition runs the blocks
 * with block_worker == r.  The result does not depend on the plan: every
 * routed row is computed by the same code whatever worker runs it, and the k
 * contributions of a token are added in slot order in fp32.  Each
 * contribution p_tj * O is first stored in the activation dtype (for bf16 it
 * is rounded there, and the fp32 sum is rounded again to give y_t).
 *   x [T][d] act dtype; gates [T][k] fp32 (p_tj);
 *   counts/block_offsets/row_to_slot/slot_to_row from moe_route_stats;
 *   block_worker from moe_plan (or any assignment of blocks to [0,P)).
 *   y [T][d] act dtype.
 *   z_save (nullable) [moe_max_slots][2*d_ff] act dtype: receives [G, U] of
 *     every routed row, as needed by moe_backward.
 *   exec_flags: 0, or MOE_EXEC_TWO_PHASE (FC1 and FC2 in one launch), with
 *     an optional MOE_EXEC_SPLIT(n1) (FC1 producers and FC2 consumers); or
 *     MOE_EXEC_FP8_ACT (e4m3 weights: FC1 and FC2 on the fp8 MFMA).
 *   stage_events (host, nullable): 5 hipEvent_t recorded on `stream` at
 *     start / after scheduling / after FC1 / after FC2 / after combine (with
 *     MOE_EXEC_TWO_PHASE the FC1 and FC2 events follow the one launch).
 *   timeline (nullable): phases MOE_TL_FC1 and MOE_TL_FC2 (see above; in
 *     the two-phase launch a workgroup's FC1 ends where its FC2 starts).
 * Errors: MOE_ERR_ARG for an invalid layer, size or null pointer;
 *   MOE_ERR_UNSUPPORTED for E > 512, P outside {1,2,4,8}, d not a multiple
 *   of 128, d_ff not a multiple of 64 (128 with e4m3 weights), a dtype pair
 *   other than fp32/fp32, bf16/bf16 or bf16 activations with e4m3 weights,
 *   or an operand of 2 GiB or more (T*d, moe_max_slots*2*d_ff or
 *   moe_max_slots*d elements of the activation dtype, or 2*d_ff*d of the
 *   weight dtype): the kernels address operands with 32-bit byte offsets and
 *   read masked rows at offset 2^31;
 *   MOE_ERR_WORKSPACE for a missing, misaligned or short workspace.  A
 *   block_worker entry outside [0, P) sets MOE_DEV_BAD_PLAN in *status_dev. */
int moe_forward(const moe_layer* L, const void* x, const float* gates,
                const int32_t* topk_ids, int T, int k, int beta, int P,
                const int32_t* counts, const int32_t* block_offsets,
                const int32_t* row_to_slot, const int32_t* slot_to_row,
                const int32_t* block_worker, void* y, void* z_save,
                int32_t* status_dev, void* ws, size_t ws_bytes, int exec_flags,
                void* const* stage_events, uint64_t* timeline, void* stream);

/* Backward expert layer (gradient equations of the "Backward" section), with
 * D_t = p_tj * dy_t:
 *   dx_t = sum_j W1_e^T [dG; dU],  dG = dA * U * s(G)(1 + G(1 - s(G))),
 *   dU = dA * SiLU(G),  dA = W2_e^T D;
 *   dw2[e] = sum_rows D A^T,  dw1[e] = sum_rows [dG; dU] x^T   (fp32).
 * Worker r computes the weight-gradient partial of every expert it holds
 * blocks of; a non-owner's partial goes to one of its s replica slots in
 * `ws`, and each owner slot dw*[e] = owner partial + replica partials in
 * ascending worker order, in fp32 (early fixed-order owner reduction).
 *   dy [T][d], z_save from moe_forward on the same routing, owner [E] = h(e);
 *   dx [T][d] act dtype; dw1 [E][2*d_ff][d] fp32; dw2 [E][d][d_ff] fp32.
 *   exec_flags: 0, or MOE_EXEC_TWO_PHASE (dA and dX in one launch), with
 *     an optional MOE_EXEC_SPLIT(n1) (dA producers and dX consumers); or
 *     MOE_EXEC_FP8_ACT (e4m3 weights: dA and dX on the fp8 MFMA).
 *   stage_events (host, nullable): 7 events: start / after scheduling /
 *     after dA / after dX / after dx combine / after weight gradients /
 *     after replica reduction (with MOE_EXEC_TWO_PHASE the dA and dX events
 *     follow the one launch).
 *   timeline (nullable): phases MOE_TL_DA, MOE_TL_DX and MOE_TL_DW.
 * fp8 weights (MegaFlux summary, "Backward": overlapped token-axis
 * requantization of D_e and dZ_e): dA, dZ and dx use D and the weights as
 * the forward does (e4m3 codes times their 128 x 128 block scales); the
 * weight gradients take D and dZ requantized to e4m3 along the tokens, in
 * blocks of beta consecutive slots times one column (moe_quantize_token_blocks),
 * with x and A = SiLU(G) U unquantized: dw2 = Dq A^T, dw1 = dZq x^T.  The
 * requantized D and dZ live in `ws` (moe_workspace_size counts them): as
 * codes and scales, or, when d and d_ff are multiples of 256, widened back
 * to bf16 (code times scale), which is the value the products use.
 * Errors: as moe_forward, plus MOE_ERR_ARG for s < 0.  On the device, a
 *   plan whose blocks of one expert on one worker are not one contiguous run,
 *   or that gives a worker more than s replica experts, sets
 *   MOE_DEV_BAD_PLAN; an owner outside [0, P) sets MOE_DEV_BAD_OWNER. */
int moe_backward(const moe_layer* L, const void* x, const float* gates, const void* dy,
                 const void* z_save, const int32_t* topk_ids, int T, int k, int beta,
                 int P, int s, const int32_t* counts, const int32_t* block_offsets,
                 const int32_t* row_to_slot, const int32_t* slot_to_row,
                 const int32_t* owner, const int32_t* block_worker, void* dx, float* dw1,
                 float* dw2, int32_t* status_dev, void* ws, size_t ws_bytes, int exec_flags,
                 void* const* stage_events, uint64_t* timeline, void* stream);

/* Token-axis e4m3 requantization (MegaFlux summary, "Backward": D_e and dZ_e
 * are requantized along the tokens for the weight-gradient products).
 * Blocks of block_rows consecutive rows times one column: scale = amax / 448
 * over the block's column, code = e4m3(value / scale) rounded to nearest,
 * ties to even, magnitudes saturated at 448 (OCP e4m3fn), every step in fp32;
 * an all-zero block column gets scale 0 and codes 0.  Row r's values:
 *   row_map == NULL:  src[r * ld + c]
 *   row_map[r] < 0 or row_map[r] >= src_rows * row_div:   0
 *   otherwise:        src[(gather ? row_map[r] / row_div : r) * ld + c]
 *                     * (row_scale ? row_scale[row_map[r]] : 1)
 * (the backward uses slot_to_row as row_map: with gather, row_div = k and
 * row_scale = gates it forms D = p * dy per slot; without, it masks padding).
 *   src bf16 [src_rows][ld], device; row_map [rows] (nullable); row_scale
 *   (nullable) [src_rows * row_div] fp32; codes [rows][cols] uint8; scales
 *   [ceil(rows / block_rows)][cols] fp32; all device pointers, caller-owned.
 *   Every row read is below src_rows: in place (no map, or a map without
 *   gather) rows < src_rows is required; gathered map values past
 *   src_rows * row_div read as zero rows.
 * Errors: MOE_ERR_ARG for rows < 0, cols < 8, not a multiple of 8 or above
 *   8,388,480 (65535 tiles of 128 columns),
 *   ld < cols or not a multiple of 8, block_rows < 1, row_div < 1,
 *   src_rows < 0, src_rows < rows when rows are read in place, or a null
 *   src/codes/scales. */
int moe_quantize_token_blocks(const void* src, int ld, int src_rows, const int32_t* row_map,
                              int gather, int row_div, const float* row_scale, int rows,
                              int cols, int block_rows, uint8_t* codes, float* scales,
                              void* stream);

/* Activation rows for an fp8 x fp8 product: each row of src [rows][cols]
 * (bf16, cols a multiple of 128) is cut into blocks of 128 features; block b
 * of row r gets the power-of-two scale 2^e, e the smallest integer with
 * amax <= 448 * 2^e, clamped to [-127, 127] (-127 for a zero block), and
 * codes[r][c] = e4m3(src[r][c] * 2^-e), round to nearest even (the product
 * is exact).  This is how MOE_EXEC_FP8_ACT quantizes x, A and dy (dZ is
 * quantized the same way where it is formed).
 *   codes uint8 [rows][cols]; exps int32 [cols / 128][rows] (block-major:
 *   exps[b * rows + r] = e), all device memory owned by the caller.
 * Errors: MOE_ERR_ARG for rows < 0, cols not a positive multiple of 128, or
 *   a null pointer with rows > 0. */
int moe_quantize_act_rows(const void* src, int rows, int cols, uint8_t* codes, int32_t* exps,
                          void* stream);

/* Timing helpers so a caller without a HIP binding can time the stages:
 * create / destroy a hipEvent_t, and the milliseconds between two recorded
 * events (waits for `b`). */
int moe_event_create(void** ev);
int moe_event_destroy(void* ev);
int moe_event_record(void* ev, void* stream);
int moe_event_elapsed_ms(void* a, void* b, float* ms);

/* Number of CUs and XCDs of the current device (host; for reporting). */
int moe_device_info(int* num_cus, int* num_xcds, int* wg_per_cu_gemm);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
