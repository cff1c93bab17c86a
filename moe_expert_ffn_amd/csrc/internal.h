// Library-internal declarations: limits, workspace layout and the launchers
// behind the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_ffn.h"

namespace moe {

constexpr int kMaxExperts = 1024;      // routing statistics
constexpr int kMaxPlanExperts = 512;   // planner and executors (LDS-resident tables)
constexpr int kNumCounters = 64;       // per-(phase, worker) work counters

inline size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

// Per-worker M-tile descriptor: expert, first slot, valid rows (<= tile rows).
// Per-worker weight-gradient segment: expert, first slot, valid rows,
// destination (-1 = the owner's slot dw*[e], else a replica slot index).
struct Sizes {
  int T, k, E, d, dff, beta, P, s;
  int act_bytes;
  int fp8;            // e4m3 weights: the backward requantizes D and dZ
  size_t max_slots, max_blocks, max_mt;
};

struct WsLayout {
  size_t ctr, mt_cnt, mt, seg_cnt, seg, rep_slot, owner_has, flags, bufA, bufO, rslots, bufP, sgate;
  size_t dq, dqs, zq, zqs;   // fp8 backward: token-axis e4m3 codes and scales of D and dZ
  size_t dhat;               // fp8 backward on the stream kernels: requantized D as bf16
  size_t xq, xe;             // fp8 MFMA forward: x as e4m3 codes and row exponents
  size_t hq, he;             // ... and A = SiLU(G) U as e4m3 codes and row exponents
  size_t total;
};

WsLayout exec_layout(const Sizes& z, bool backward);
bool use_big_tiles(const Sizes& z);
bool use_stream(const Sizes& z);
size_t max_tiles(const Sizes& z);
size_t route_ws_bytes(int T, int k, int E);
// the routing statistics' scratch array of moe_route_stats_noalloc
constexpr size_t kRouteScratchBytes = MOE_ROUTE_SCRATCH_BYTES;
int route_scratch(void** device_ptr);

int launch_route_stats(const int32_t* ids, int T, int k, int E, int beta, int32_t* counts,
                       int32_t* offsets, int32_t* block_counts, int32_t* block_offsets,
                       int32_t* row_to_slot, int32_t* slot_to_row, double* kappa,
                       int32_t* status, void* ws, hipStream_t st);
int launch_plan(const int32_t* bcnt, const int32_t* boff, const int32_t* owner, int E, int P,
                int s, int mode, int lam, int32_t* q, int32_t* load, int32_t* bw, int bw_cap,
                int32_t* info, int32_t* status, hipStream_t st);
constexpr int kQtMaxCols = 65535 * 128;   // column tiles of the quantizer grid
// map_lim: map values m >= map_lim read as zero rows (src rows * div)
int launch_quant_act(const uint16_t* x, int rows, int cols, uint8_t* codes, int32_t* exps,
                     hipStream_t st, const int32_t* blk_end = nullptr, int blk_rows = 0);
int launch_quant_tok(const uint16_t* src, int ld, const int32_t* map, int gather, int div,
                     const float* rscale, int map_lim, int rows, int cols, int brows,
                     uint8_t* codes, float* scales, hipStream_t st,
                     const int32_t* blk_end = nullptr);
int launch_predict_cost(const int32_t* counts, const int32_t* boff, const int32_t* bw_f,
                        const int32_t* bw_b, const int32_t* owner, int E, int beta, int P, int d,
                        int dff, int G, long long* cost, int32_t* status, hipStream_t st);
int launch_predict_split(const int32_t* counts, const int32_t* boff, const int32_t* bw, int E,
                         int beta, int P, int d, int dff, int G, int backward, long long* costs,
                         int32_t* choice, int32_t* status, hipStream_t st);
int launch_plan_gate(const int32_t* bcnt, const int32_t* boff, const int32_t* owner, int E, int P,
                     int rho_milli, int32_t* q, int32_t* load, int32_t* bw, int bw_cap,
                     int32_t* info, int32_t* status, hipStream_t st);

struct LayerPtrs {
  const void* w1;
  const void* w2;
  const float* w1s;
  const float* w2s;
  int act_dtype, w_dtype;
};

int launch_forward(const Sizes& z, const LayerPtrs& L, const void* x, const float* gates,
                   const int32_t* counts, const int32_t* boff, const int32_t* row_to_slot,
                   const int32_t* slot_to_row, const int32_t* block_worker, void* y,
                   void* z_save, int32_t* status, char* ws, int exec_flags, void* const* ev,
                   uint64_t* timeline, hipStream_t st);

int launch_backward(const Sizes& z, const LayerPtrs& L, const void* x, const float* gates,
                    const void* dy, const void* z_save, const int32_t* counts,
                    const int32_t* boff, const int32_t* row_to_slot,
                    const int32_t* slot_to_row, const int32_t* owner,
                    const int32_t* block_worker, void* dx, float* dw1, float* dw2,
                    int32_t* status, char* ws, int exec_flags, void* const* ev,
                    uint64_t* timeline, hipStream_t st);

int gemm_wg_per_cu();

}  // namespace moe
