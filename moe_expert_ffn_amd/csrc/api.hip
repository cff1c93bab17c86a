// C ABI of the MoE expert layer: argument checks on the host, workspace
// carving and kernel launches.  No allocation, no host synchronisation.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "moe_ffn.h"

using namespace moe;

namespace {

bool valid_P(int P) { return P == 1 || P == 2 || P == 4 || P == 8; }

bool ws_ok(const void* ws, size_t have, size_t need) {
  if (need == 0) return true;
  if (!ws) return false;
  if (((uintptr_t)ws) & 255u) return false;
  return have >= need;
}

// Shared validation of the layer description; returns MOE_OK or an error.
int check_layer(const moe_layer* L, bool backward) {
  if (!L) return MOE_ERR_ARG;
  if (L->E < 1 || L->d < 1 || L->d_ff < 1) return MOE_ERR_ARG;
  if (!L->w1 || !L->w2) return MOE_ERR_ARG;
  if (L->E > kMaxPlanExperts) return MOE_ERR_UNSUPPORTED;
  if (L->d % 128 != 0 || L->d_ff % 64 != 0) return MOE_ERR_UNSUPPORTED;
  const bool f32 = L->act_dtype == MOE_F32 && L->w_dtype == MOE_F32;
  const bool bf = L->act_dtype == MOE_BF16 && L->w_dtype == MOE_BF16;
  const bool f8 = L->act_dtype == MOE_BF16 && L->w_dtype == MOE_FP8_E4M3;
  if (!f32 && !bf && !f8) return L->act_dtype > MOE_BF16 || L->w_dtype > MOE_FP8_E4M3
                                     ? MOE_ERR_ARG : MOE_ERR_UNSUPPORTED;
  if (f8) {
    if (L->d_ff % 128 != 0) return MOE_ERR_UNSUPPORTED;
    if (!L->w1_scale || !L->w2_scale) return MOE_ERR_ARG;
  }
  return MOE_OK;
}

Sizes make_sizes(const moe_layer* L, int T, int k, int beta, int P, int s) {
  Sizes z{};
  z.T = T; z.k = k; z.E = L->E; z.d = L->d; z.dff = L->d_ff; z.beta = beta; z.P = P; z.s = s;
  z.act_bytes = L->act_dtype == MOE_F32 ? 4 : 2;
  z.fp8 = L->w_dtype == MOE_FP8_E4M3 ? 1 : 0;
  z.max_slots = moe_max_slots(T, k, L->E, beta);
  z.max_blocks = moe_max_blocks(T, k, L->E, beta);
  z.max_mt = max_tiles(z);
  return z;
}

bool sizes_ok(int T, int k, int E, int beta) {
  if (T < 0 || k < 1 || E < 1 || beta < 1) return false;
  const long long slots = (long long)T * k + (long long)E * (beta - 1);
  return slots < (1ll << 31);
}

// The GEMM kernels address every operand through buffer descriptors with
// 32-bit byte offsets, and send masked rows to offset 2^31, which reads as
// zeros only while the descriptor's size is below it.  Each such operand must
// therefore span less than 2 GiB: token rows (x, dy, y, dx), the
// slot-indexed buffers (A or dZ, O, P, z_save, the requantized D), all in the
// activation dtype, and one expert's weights.
bool extents_ok(const Sizes& z) {
  const unsigned long long lim = 1ull << 31, S = (unsigned long long)z.max_slots;
  const unsigned long long d = (unsigned long long)z.d, f = (unsigned long long)z.dff;
  const unsigned long long ab = (unsigned long long)z.act_bytes, wb = z.fp8 ? 1ull : ab;
  return (unsigned long long)z.T * d * ab < lim && S * 2 * f * ab < lim && S * d * ab < lim &&
         2 * f * d * wb < lim;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t moe_max_slots(int T, int k, int E, int beta) {
  if (!sizes_ok(T, k, E, beta)) return 0;
  return (size_t)T * k + (size_t)E * (beta - 1);
}

size_t moe_max_blocks(int T, int k, int E, int beta) {
  if (!sizes_ok(T, k, E, beta)) return 0;
  return ((size_t)T * k + (size_t)E * (beta - 1)) / beta;
}

size_t moe_workspace_size(const moe_layer* L, int T, int k, int beta, int P, int s,
                          int with_backward) {
  if (!L || !sizes_ok(T, k, L->E, beta) || !valid_P(P) || s < 0) return 0;
  if (L->E > kMaxExperts) return 0;
  size_t need = route_ws_bytes(T, k, L->E);
  if (L->E <= kMaxPlanExperts && L->d > 0 && L->d_ff > 0) {
    const Sizes z = make_sizes(L, T, k, beta, P, s);
    if (!extents_ok(z)) return 0;
    const size_t f = exec_layout(z, false).total;
    if (f > need) need = f;
    if (with_backward) {
      const size_t b = exec_layout(z, true).total;
      if (b > need) need = b;
    }
  }
  return need;
}

int moe_route_stats(const int32_t* topk_ids, int T, int k, int E, int beta, int32_t* counts,
                    int32_t* offsets, int32_t* block_counts, int32_t* block_offsets,
                    int32_t* row_to_slot, int32_t* slot_to_row, double* kappa,
                    int32_t* status_dev, void* ws, size_t ws_bytes, void* stream) {
  if (!sizes_ok(T, k, E, beta)) return MOE_ERR_ARG;
  if (E > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if ((T > 0 && (!topk_ids || !row_to_slot)) || !counts || !offsets || !block_counts ||
      !block_offsets || !slot_to_row || !kappa || !status_dev)
    return MOE_ERR_ARG;
  if (!ws_ok(ws, ws_bytes, route_ws_bytes(T, k, E))) return MOE_ERR_WORKSPACE;
  return launch_route_stats(topk_ids, T, k, E, beta, counts, offsets, block_counts,
                            block_offsets, row_to_slot, slot_to_row, kappa, status_dev, ws,
                            (hipStream_t)stream);
}

int moe_route_stats_noalloc(const int32_t* topk_ids, int T, int k, int E, int beta,
                            int32_t* counts, int32_t* offsets, int32_t* block_counts,
                            int32_t* block_offsets, int32_t* row_to_slot, int32_t* slot_to_row,
                            double* kappa, int32_t* status_dev, void* stream) {
  if (!sizes_ok(T, k, E, beta)) return MOE_ERR_ARG;
  if (E > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if ((T > 0 && (!topk_ids || !row_to_slot)) || !counts || !offsets || !block_counts ||
      !block_offsets || !slot_to_row || !kappa || !status_dev)
    return MOE_ERR_ARG;
  if (route_ws_bytes(T, k, E) > kRouteScratchBytes) return MOE_ERR_UNSUPPORTED;
  void* scr = nullptr;
  const int rc = route_scratch(&scr);
  if (rc != MOE_OK) return rc;
  return launch_route_stats(topk_ids, T, k, E, beta, counts, offsets, block_counts,
                            block_offsets, row_to_slot, slot_to_row, kappa, status_dev, scr,
                            (hipStream_t)stream);
}

int moe_plan(const int32_t* block_counts, const int32_t* block_offsets, const int32_t* owner,
             int E, int P, int s, int mode, int lambda, int32_t* q, int32_t* load,
             int32_t* block_worker, int block_worker_cap, int32_t* plan_info,
             int32_t* status_dev, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (E < 1 || s < 0 || lambda < 0 || block_worker_cap < 0 ||
      (mode != MOE_PLAN_FWD && mode != MOE_PLAN_BWD && mode != MOE_PLAN_QUOTA) ||
      (mode == MOE_PLAN_QUOTA && lambda < 1))
    return MOE_ERR_ARG;
  if (!valid_P(P) || E > kMaxPlanExperts) return MOE_ERR_UNSUPPORTED;
  if (!block_counts || !block_offsets || !owner || !q || !load || !block_worker ||
      !plan_info || !status_dev)
    return MOE_ERR_ARG;
  return launch_plan(block_counts, block_offsets, owner, E, P, s, mode, lambda, q, load,
                     block_worker, block_worker_cap, plan_info, status_dev, (hipStream_t)stream);
}

int moe_plan_gate(const int32_t* block_counts, const int32_t* block_offsets, const int32_t* owner,
                  int E, int P, int rho_milli, int32_t* q, int32_t* load, int32_t* block_worker,
                  int block_worker_cap, int32_t* plan_info, int32_t* status_dev, void* stream) {
  if (E < 1 || rho_milli < 0 || block_worker_cap < 0) return MOE_ERR_ARG;
  if (!valid_P(P) || E > kMaxPlanExperts) return MOE_ERR_UNSUPPORTED;
  if (!block_counts || !block_offsets || !owner || !q || !load || !block_worker || !plan_info ||
      !status_dev)
    return MOE_ERR_ARG;
  return launch_plan_gate(block_counts, block_offsets, owner, E, P, rho_milli, q, load,
                          block_worker, block_worker_cap, plan_info, status_dev,
                          (hipStream_t)stream);
}

int moe_quantize_token_blocks(const void* src, int ld, int src_rows, const int32_t* row_map,
                              int gather, int row_div, const float* row_scale, int rows, int cols,
                              int block_rows, uint8_t* codes, float* scales, void* stream) {
  if (rows < 0 || cols < 8 || cols % 8 || cols > kQtMaxCols || ld < cols || ld % 8 ||
      block_rows < 1 || row_div < 1 || src_rows < 0)
    return MOE_ERR_ARG;
  // rows read in place (no map, or a map without gather) need src_rows >= rows
  if ((!row_map || !gather) && src_rows < rows) return MOE_ERR_ARG;
  if (!src || !codes || !scales) return MOE_ERR_ARG;
  const long long lim = (long long)src_rows * row_div;
  return launch_quant_tok((const uint16_t*)src, ld, row_map, gather ? 1 : 0, row_div, row_scale,
                          lim < INT32_MAX ? (int)lim : INT32_MAX, rows, cols, block_rows, codes,
                          scales, (hipStream_t)stream);
}

int moe_quantize_act_rows(const void* src, int rows, int cols, uint8_t* codes, int32_t* exps,
                          void* stream) {
  if (rows < 0 || cols < 128 || cols % 128) return MOE_ERR_ARG;
  if (rows > 0 && (!src || !codes || !exps)) return MOE_ERR_ARG;
  if (rows == 0) return MOE_OK;
  return launch_quant_act((const uint16_t*)src, rows, cols, codes, exps, (hipStream_t)stream);
}

int moe_predict_cost(const int32_t* counts, const int32_t* block_offsets,
                     const int32_t* block_worker_fwd, const int32_t* block_worker_bwd,
                     const int32_t* owner, int E, int beta, int P, int d, int d_ff,
                     int num_workgroups, int64_t* cost_dev, int32_t* status_dev, void* stream) {
  if (E < 1 || beta < 1 || d < 1 || d_ff < 1) return MOE_ERR_ARG;
  if (!counts || !block_offsets || !block_worker_fwd || !block_worker_bwd || !owner || !cost_dev ||
      !status_dev)
    return MOE_ERR_ARG;
  if (!valid_P(P) || E > kMaxPlanExperts || d % 256 || d_ff % 256) return MOE_ERR_UNSUPPORTED;
  int G = num_workgroups;
  if (G <= 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&G, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return MOE_ERR_HIP;
  }
  if (G % P || G / P > 256) return MOE_ERR_UNSUPPORTED;
  return launch_predict_cost(counts, block_offsets, block_worker_fwd, block_worker_bwd, owner, E,
                             beta, P, d, d_ff, G, (long long*)cost_dev, status_dev,
                             (hipStream_t)stream);
}

int moe_predict_split(const int32_t* counts, const int32_t* block_offsets,
                      const int32_t* block_worker, int E, int beta, int P, int d, int d_ff,
                      int num_workgroups, int backward, int64_t* costs_dev, int32_t* choice_dev,
                      int32_t* status_dev, void* stream) {
  if (E < 1 || beta < 1 || d < 1 || d_ff < 1) return MOE_ERR_ARG;
  if (!counts || !block_offsets || !block_worker || !costs_dev || !choice_dev || !status_dev)
    return MOE_ERR_ARG;
  if (!valid_P(P) || E > kMaxPlanExperts || d % 256 || d_ff % 256) return MOE_ERR_UNSUPPORTED;
  int G = num_workgroups;
  if (G <= 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&G, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return MOE_ERR_HIP;
  }
  if (G % P || G / P > 256) return MOE_ERR_UNSUPPORTED;
  return launch_predict_split(counts, block_offsets, block_worker, E, beta, P, d, d_ff, G,
                              backward ? 1 : 0, (long long*)costs_dev, choice_dev, status_dev,
                              (hipStream_t)stream);
}

// known bits only; a producer/consumer split only with the two-phase launch
// (its upper bound, the workgroups of one worker, is checked at launch)
static bool exec_flags_ok(int f) {
  const int split = (f >> MOE_EXEC_SPLIT_SHIFT) & 0xff;
  const int known = MOE_EXEC_TWO_PHASE | MOE_EXEC_SPLIT(0xff) | MOE_EXEC_FP8_ACT;
  if (f & ~known) return false;
  return split == 0 || (f & MOE_EXEC_TWO_PHASE);
}

int moe_forward(const moe_layer* L, const void* x, const float* gates, const int32_t* topk_ids,
                int T, int k, int beta, int P, const int32_t* counts,
                const int32_t* block_offsets, const int32_t* row_to_slot,
                const int32_t* slot_to_row, const int32_t* block_worker, void* y, void* z_save,
                int32_t* status_dev, void* ws, size_t ws_bytes, int exec_flags,
                void* const* stage_events, uint64_t* timeline, void* stream) {
  (void)topk_ids;
  const int lc = check_layer(L, false);
  if (!exec_flags_ok(exec_flags)) return MOE_ERR_ARG;
  if (lc != MOE_OK) return lc;
  if (!sizes_ok(T, k, L->E, beta)) return MOE_ERR_ARG;
  if (!valid_P(P)) return MOE_ERR_UNSUPPORTED;
  if ((T > 0 && (!x || !gates || !row_to_slot || !y)) || !counts || !block_offsets ||
      !slot_to_row || !block_worker || !status_dev)
    return MOE_ERR_ARG;
  const Sizes z = make_sizes(L, T, k, beta, P, 0);
  if (!extents_ok(z)) return MOE_ERR_UNSUPPORTED;
  // the fp8 MFMA forward: bf16 x, e4m3 weights on the stream kernels, two launches
  if ((exec_flags & MOE_EXEC_FP8_ACT) &&
      (L->act_dtype != MOE_BF16 || L->w_dtype != MOE_FP8_E4M3 || !use_stream(z) ||
       (exec_flags & MOE_EXEC_TWO_PHASE)))
    return MOE_ERR_ARG;
  if (!ws_ok(ws, ws_bytes, exec_layout(z, false).total)) return MOE_ERR_WORKSPACE;
  LayerPtrs Lp{L->w1, L->w2, L->w1_scale, L->w2_scale, L->act_dtype, L->w_dtype};
  return launch_forward(z, Lp, x, gates, counts, block_offsets, row_to_slot, slot_to_row,
                        block_worker, y, z_save, status_dev, (char*)ws, exec_flags, stage_events,
                        timeline, (hipStream_t)stream);
}

int moe_backward(const moe_layer* L, const void* x, const float* gates, const void* dy,
                 const void* z_save, const int32_t* topk_ids, int T, int k, int beta, int P,
                 int s, const int32_t* counts, const int32_t* block_offsets,
                 const int32_t* row_to_slot, const int32_t* slot_to_row, const int32_t* owner,
                 const int32_t* block_worker, void* dx, float* dw1, float* dw2,
                 int32_t* status_dev, void* ws, size_t ws_bytes, int exec_flags,
                 void* const* stage_events, uint64_t* timeline, void* stream) {
  (void)topk_ids;
  const int lc = check_layer(L, true);
  if (!exec_flags_ok(exec_flags)) return MOE_ERR_ARG;
  if (lc != MOE_OK) return lc;
  if (!sizes_ok(T, k, L->E, beta) || s < 0) return MOE_ERR_ARG;
  if (!valid_P(P)) return MOE_ERR_UNSUPPORTED;
  if ((T > 0 && (!x || !gates || !dy || !z_save || !row_to_slot || !dx)) || !counts ||
      !block_offsets || !slot_to_row || !owner || !block_worker || !dw1 || !dw2 || !status_dev)
    return MOE_ERR_ARG;
  const Sizes z = make_sizes(L, T, k, beta, P, s);
  if (!extents_ok(z)) return MOE_ERR_UNSUPPORTED;
  // dA and dX on the fp8 MFMA: bf16 dy, e4m3 weights on the stream kernels, two launches
  if ((exec_flags & MOE_EXEC_FP8_ACT) &&
      (L->act_dtype != MOE_BF16 || L->w_dtype != MOE_FP8_E4M3 || !use_stream(z) ||
       (exec_flags & MOE_EXEC_TWO_PHASE)))
    return MOE_ERR_ARG;
  if (!ws_ok(ws, ws_bytes, exec_layout(z, true).total)) return MOE_ERR_WORKSPACE;
  LayerPtrs Lp{L->w1, L->w2, L->w1_scale, L->w2_scale, L->act_dtype, L->w_dtype};
  return launch_backward(z, Lp, x, gates, dy, z_save, counts, block_offsets, row_to_slot,
                         slot_to_row, owner, block_worker, dx, dw1, dw2, status_dev, (char*)ws,
                         exec_flags, stage_events, timeline, (hipStream_t)stream);
}

int moe_event_create(void** ev) {
  if (!ev) return MOE_ERR_ARG;
  return hipEventCreate((hipEvent_t*)ev) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
int moe_event_destroy(void* ev) {
  return hipEventDestroy((hipEvent_t)ev) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
int moe_event_record(void* ev, void* stream) {
  return hipEventRecord((hipEvent_t)ev, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
int moe_event_elapsed_ms(void* a, void* b, float* ms) {
  if (!ms) return MOE_ERR_ARG;
  if (hipEventSynchronize((hipEvent_t)b) != hipSuccess) return MOE_ERR_HIP;
  return hipEventElapsedTime(ms, (hipEvent_t)a, (hipEvent_t)b) == hipSuccess ? MOE_OK
                                                                              : MOE_ERR_HIP;
}

int moe_device_info(int* num_cus, int* num_xcds, int* wg_per_cu_gemm) {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MOE_ERR_HIP;
  if (num_cus) *num_cus = n;
  if (num_xcds) *num_xcds = 8;
  if (wg_per_cu_gemm) *wg_per_cu_gemm = gemm_wg_per_cu();
  return MOE_OK;
}

}  // extern "C"
