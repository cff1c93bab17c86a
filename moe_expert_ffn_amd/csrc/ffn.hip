// Expert-layer executors on the planned blocks (MegaFlux summary,
// picx.dev/p/e4jAzZ: "Forward", "Backward" and their expert-computation and
// gradient equations).
//
// Worker r of the plan is a CU partition: the workgroups of a launch with
// blockIdx % 8 in r's XCDs.  Each phase is one persistent launch; a workgroup
// pulls tiles from its own worker's queue (an atomic counter), so a worker only
// ever runs the blocks the plan gave it, and a straggling worker shows up as a
// straggling set of XCDs exactly as a straggling GPU would.
//
// Forward:  schedule -> FC1 (gather x rows, SwiGLU epilogue) -> FC2 (gate
//           epilogue) -> combine (k contributions per token, fixed order).
// Backward: schedule -> dA (gather dy rows; SwiGLU-gradient epilogue writes
//           dZ = [dG, dU]) -> dX (combine over k) -> weight gradients per
//           (expert, worker) segment, replica segments first -> fixed-order
//           fp32 reduction of replica partials into the owner slot.
#include "common.h"
#include "gemm.h"
#include <cstdlib>
#include <cstring>
#include <utility>
#include "moe_ffn.h"

namespace moe {

struct SchedArgs {
  const int32_t* counts;
  const int32_t* boff;
  const int32_t* bw;
  const int32_t* owner;
  int E, P, s, beta, backward, bm, max_blocks;
  int32_t* ctr;
  int32_t* mt_cnt;
  int4* mt;
  int max_mt;
  int32_t* seg_cnt;
  int4* seg;
  int32_t* rep_slot;
  int32_t* owner_has;
  int32_t* flags;      // per (worker, row tile) readiness counters of the two-phase launches
  int32_t* status;
  // per-slot gates p (0 for padding slots), written by the workgroups past
  // the first: gate_out[i] = gate_src[gate_s2r[i]] for i < gate_n
  const int32_t* gate_s2r;
  const float* gate_src;
  float* gate_out;
  size_t gate_n;
};

MOE_DEV int expert_of(int g, const int* boff_s, int E) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (boff_s[mid] <= g) lo = mid; else hi = mid;
  }
  return lo;
}

// The scheduling workgroup.  M-tiles: a tile holds up to `bm` consecutive slots of one
// (expert, worker) run of blocks.  When bm is a multiple of beta, tiles start
// every bm/beta blocks from the start of each run; otherwise every block is cut
// into ceil(valid rows / bm) tiles of its own.  Tiles are listed per worker in
// block order (one exclusive scan per worker).  Segments (backward): the
// blocks of one (expert, worker) pair must form one contiguous run; its slot
// range and valid-row count become one weight-gradient segment, with a replica
// slot when the worker is not the owner (rank among that worker's non-home
// experts, in expert order).  A pair that breaks the plan's constraints (its
// blocks are not one run, or its worker already holds s replica experts) sets
// MOE_DEV_BAD_PLAN and gets no segment: its weight-gradient rows are dropped,
// and an owner without a segment receives only the replica partials (zeros
// when there are none).  A plan with more blocks than the slot space holds
// (block_offsets[E] > max_blocks) sets the bit and schedules nothing.
MOE_DEV int block_rows(int g, int e, int beta, const int* boff_s, const int* cnt_s) {
  return min(beta, beta * boff_s[e] + cnt_s[e] - beta * g);
}

// Workgroup 0 schedules, one wave per worker (P <= 8); the workgroups past it
// (if any) write the per-slot gates.  BWL: block_worker is first copied to LDS
// (when max_blocks entries fit), so each worker's pass over the blocks reads
// LDS instead of issuing a global load per 64 blocks.
constexpr int kSchedThreads = 512;
template <bool BWL>
__global__ __launch_bounds__(kSchedThreads) void k_sched(SchedArgs a) {
  extern __shared__ int sm[];
  if (blockIdx.x > 0) {          // the per-slot gates, beside the scheduling workgroup
    const size_t stride = (size_t)(gridDim.x - 1) * kSchedThreads;
    for (size_t i = (size_t)(blockIdx.x - 1) * kSchedThreads + threadIdx.x; i < a.gate_n; i += stride) {
      const int row = a.gate_s2r[i];
      a.gate_out[i] = row >= 0 ? a.gate_src[row] : 0.f;
    }
    return;
  }
  const int E = a.E, P = a.P;
  int* boff_s = sm;
  int* cnt_s = boff_s + E + 1;
  int* bw_s = cnt_s + E;                          // max_blocks entries when BWL
  int* s0_s = bw_s + (BWL ? a.max_blocks : 0);
  int* rows_s = s0_s + E * P;
  int* starts_s = rows_s + E * P;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  constexpr int NT = kSchedThreads, NW = kSchedThreads / 64;
  for (int i = tid; i <= E; i += NT) boff_s[i] = a.boff[i];
  for (int i = tid; i < E; i += NT) cnt_s[i] = a.counts[i];
  if (tid < kNumCounters) a.ctr[tid] = 0;
  for (int i = tid; i < P * a.max_mt; i += NT) a.flags[i] = 0;
  if (a.backward)
    for (int i = tid; i < E * P; i += NT) { s0_s[i] = INT_MAX; rows_s[i] = 0; starts_s[i] = 0; }
  __syncthreads();
  const int nb = boff_s[E];
  if (nb > a.max_blocks) {                        // more blocks than the slot space holds
    if (tid == 0) atomicOr(a.status, MOE_DEV_BAD_PLAN);
    if (tid < P) {
      a.mt_cnt[tid] = 0;
      if (a.backward) a.seg_cnt[tid] = 0;
    }
    if (a.backward) {                             // the replica reduction zeroes every owner slot
      for (int i = tid; i < E * P; i += NT) a.rep_slot[i] = -1;
      for (int e = tid; e < E; e += NT) a.owner_has[e] = 0;
    }
    return;
  }
  for (int g = tid; g < nb; g += NT) {
    const int w = a.bw[g];
    if (w < 0 || w >= P) atomicOr(a.status, MOE_DEV_BAD_PLAN);
    if constexpr (BWL) bw_s[g] = w;
  }
  if constexpr (BWL) __syncthreads();
  auto bw = [&](int g) { if constexpr (BWL) return bw_s[g]; else return a.bw[g]; };
  const bool grouped = (a.bm % a.beta) == 0;
  const int f = grouped ? a.bm / a.beta : 1;
  const uint64_t le_mask = (lane == 63) ? ~0ull : ((1ull << (lane + 1)) - 1);
  for (int r = wv; r < P; r += NW) {
    int run = 0, carry = 0;
    for (int base = 0; base < nb; base += 64) {
      const int g = base + lane;
      const bool mine = g < nb && bw(g) == r;
      int e = 0, bstart = 0, vrows = 0;
      bool start = false;
      if (mine) {
        e = expert_of(g, boff_s, E);
        bstart = a.beta * g;
        vrows = block_rows(g, e, a.beta, boff_s, cnt_s);
        start = (g == boff_s[e]) || bw(g - 1) != r;
      }
      const uint64_t sm_ = __ballot(start) & le_mask;
      const int rs = sm_ ? base + 63 - __clzll(sm_) : carry;
      carry = __shfl(rs, 63, 64);
      int nt = 0, trows = 0;
      if (mine) {
        if (grouped) {
          if ((g - rs) % f == 0) {
            nt = 1;
            for (int i = 0; i < f; ++i) {
              const int gi = g + i;
              if (gi >= boff_s[e + 1] || (i > 0 && bw(gi) != r)) break;
              trows += block_rows(gi, e, a.beta, boff_s, cnt_s);
            }
          }
        } else {
          nt = (vrows + a.bm - 1) / a.bm;
        }
      }
      const int inc = wave_incl_scan(nt);
      const int pos = run + inc - nt;
      for (int i = 0; i < nt; ++i) {
        const int rows = grouped ? trows : min(a.bm, vrows - i * a.bm);
        a.mt[(size_t)r * a.max_mt + pos + i] = make_int4(e, bstart + i * a.bm, rows, 0);
      }
      run += __shfl(inc, 63, 64);
    }
    if (lane == 0) a.mt_cnt[r] = run;
  }
  if (!a.backward) return;

  for (int g = tid; g < nb; g += NT) {
    const int w = bw(g);
    if (w < 0 || w >= P) continue;
    const int e = expert_of(g, boff_s, E);
    const int vrows = min(a.beta, a.beta * boff_s[e] + cnt_s[e] - a.beta * g);
    atomicMin(&s0_s[e * P + w], a.beta * g);
    atomicAdd(&rows_s[e * P + w], vrows);
    if (g == boff_s[e] || bw(g - 1) != w) atomicAdd(&starts_s[e * P + w], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += NT) {
    const int h = a.owner[e];
    const bool ok = h >= 0 && h < P;
    if (!ok) atomicOr(a.status, MOE_DEV_BAD_OWNER);
    a.owner_has[e] = (ok && rows_s[e * P + h] > 0 && starts_s[e * P + h] == 1) ? 1 : 0;
  }
  for (int r = wv; r < P; r += NW) {
    // pass 0: replica segments (non-home experts) first; pass 1: home segments
    int run = 0, rrun = 0;
    for (int pass = 0; pass < 2; ++pass) {
      for (int base = 0; base < E; base += 64) {
        const int e = base + lane;
        int cand = 0, dst = -1;
        bool bad = false;
        if (e < E) {
          const int h = a.owner[e];
          const int rows = rows_s[e * P + r];
          const bool home = (h == r);
          const bool mine = rows > 0 && home == (pass == 1) && h >= 0 && h < P;
          if (mine && starts_s[e * P + r] != 1) bad = true;   // not one run of blocks
          cand = (mine && !bad) ? 1 : 0;
          if (pass == 0) a.rep_slot[e * P + r] = -1;
        }
        // replica slots are ranked among the valid non-home segments
        const int nonhome = (pass == 0) ? cand : 0;
        const int rinc = wave_incl_scan(nonhome);
        const int rpos = rrun + rinc - nonhome;
        if (nonhome) {
          if (rpos >= a.s) { bad = true; cand = 0; }         // over the replica budget
          else dst = r * a.s + rpos;
        }
        if (bad) atomicOr(a.status, MOE_DEV_BAD_PLAN);
        const int inc = wave_incl_scan(cand);
        const int pos = run + inc - cand;
        if (cand) {
          a.seg[(size_t)r * E + pos] = make_int4(e, s0_s[e * P + r], rows_s[e * P + r], dst);
          if (nonhome) a.rep_slot[e * P + r] = dst;
        }
        run += __shfl(inc, 63, 64);
        rrun += __shfl(rinc, 63, 64);
      }
    }
    if (lane == 0) a.seg_cnt[r] = run;
  }
}

struct ExecArgs {
  const void* x;
  const float* gates;
  const void* w1;
  const void* w2;
  const float* w1s;
  const float* w2s;
  const int32_t* slot_to_row;
  const int32_t* row_to_slot;
  int T, k, E, d, dff, P, s, beta;
  const int4* mt;
  const int32_t* mt_cnt;
  int max_mt;
  const int4* seg;
  const int32_t* seg_cnt;
  const int32_t* rep_slot;
  const int32_t* owner_has;
  int32_t* ctr;
  void* bufA;     // forward: A = SiLU(G) * U   backward: dZ = [dG, dU]
  void* bufO;     // forward: p * O             backward: dX per routed row
  void* z_save;
  const void* dy;
  float* dw1;
  float* dw2;
  float* rslots;
  void* bufP;             // backward: P = p * SiLU(G) * U per routed row
  size_t slots;           // padded slot capacity (rows of bufA, bufO, bufP, z_save)
  const float* sgate;     // per-slot gate (0 for padding slots)
  uint32_t kmagic;        // ceil(2^32 / k): token = umulhi(row, kmagic)
  uint8_t* dq;            // fp8 backward: D = p * dy per slot, e4m3 [slots][d]
  float* dqs;             //   its scales [slots / beta][d]
  uint8_t* zq;            //   dZ, e4m3 [slots][2 d_ff]
  float* zqs;             //   its scales [slots / beta][2 d_ff]
  const void* xq;         // fp8 MFMA: x (dy in the backward) codes [T][d] and exponents
  const int32_t* xe;      // [d/128][T]; A (dZ) codes [slots][d_ff (2 d_ff)] and exponents
                          // [d_ff/128 (2 d_ff/128)][slots]
  void* hq;
  int32_t* he;
  void* dhat;             // fp8 backward on the stream kernels: D requantized and
                          //   widened back to bf16, [slots][d]
  const int32_t* boff;    // block offsets [E + 1]: boff[E] blocks of beta slots are in use
  uint64_t* timeline;     // nullable: per-workgroup start / end stamps of each stream phase
  int tl_phase;           //   this launch's phase row (a two-phase launch: its first phase)
  int32_t* flags;         // two-phase launches: finished first-phase items per (worker, row tile)
  int32_t* status;
};

enum { PH_FC1 = 0, PH_FC2 = 1, PH_DA = 2, PH_DX = 3, PH_DW = 4 };

// bf16 operands on the big tile go through the direct-to-LDS pipeline.
template <typename T, bool FP8, class C>
constexpr bool kUseDma = sizeof(T) == 2 && !FP8 && C::BM == 256 && C::BN == 256;

// Dynamic LDS of a GEMM kernel: operand staging or the largest epilogue tile
// (FC1 with [G, U] saved: two bf16 tiles of BM x (BN/2 + 8)).
template <typename T, class C> constexpr size_t gemm_lds_bytes() {
  const size_t reg = TileLds<T, C>::BYTES;
  const size_t dma = DmaCfg<C>::BYTES;
  const size_t epi = (size_t)2 * C::BM * (C::BN / 2 + 16 / sizeof(T)) * sizeof(T);
  size_t m = reg > dma ? reg : dma;
  return m > epi ? m : epi;
}

// ---- forward: FC1 + SwiGLU ------------------------------------------------
// N-tile nj covers A columns [nj*BN/2, (nj+1)*BN/2); its BN weight rows
// alternate 32 G rows and the matching 32 U rows, so a wave holds G and U of
// the same (row, column) in neighbouring accumulators and applies SwiGLU in
// registers.
template <typename T, bool FP8, class C>
__global__ __launch_bounds__(C::NT) void k_fc1(ExecArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int tslot;
  MOE_LDS T* smem = (MOE_LDS T*)smem_raw;
  constexpr int HALF = C::BN / 2;
  const int r = worker_of_block(a.P);
  const int nnt = a.dff / HALF;
  const int total = a.mt_cnt[r] * nnt;
  const int lane = threadIdx.x & 63;
  const int wn = wave_id() % C::WAVES_N;
  const T* X = (const T*)a.x;
  T* Ab = (T*)a.bufA;
  T* Z = (T*)a.z_save;
  while (true) {
    const int tile = next_tile(&a.ctr[PH_FC1 * kMaxP + r], &tslot);
    if (tile >= total) break;
    const int4 m = a.mt[(size_t)r * a.max_mt + tile / nnt];
    const int nj = tile % nnt;
    const int e = m.x, slot0 = m.y, nrows = m.z;
    RowLoad<T, C::BM, C::NT> la;
    if constexpr (!kUseDma<T, FP8, C>)
      la.init(X, [&](int row) { return row < nrows ? (a.slot_to_row[slot0 + row] / a.k) * a.d : -1; });
    auto w1row = [&](int rho) {
      const int q = rho >> 5;
      return (q & 1) * a.dff + nj * HALF + (q >> 1) * 32 + (rho & 31);
    };
    f32x16_t acc[C::MB][C::NB];
    const int nk = a.d / Elem<T>::BK;
    if constexpr (kUseDma<T, FP8, C>) {
      RowDma<C::BM, C::NT / 64> da;
      da.init(X, (uint32_t)((size_t)a.T * a.d * 2),
              [&](int row) { return row < nrows ? (a.slot_to_row[slot0 + row] / a.k) * a.d : -1; });
      RowDma<C::BN, C::NT / 64> db;
      db.init((const uint16_t*)a.w1 + (size_t)e * 2 * a.dff * a.d, (uint32_t)((size_t)4 * a.dff * a.d),
              [&](int rho) { return w1row(rho) * a.d; });
      gemm_tile_dma<C>(da, db, a.d / kDmaBK, smem, acc);
    } else if constexpr (FP8) {
      RowLoadFp8<C::BN, C::NT> lb;
      const uint8_t* W = (const uint8_t*)a.w1 + (size_t)e * 2 * a.dff * a.d;
      const float* S = a.w1s + (size_t)e * (2 * a.dff / 128) * (a.d / 128);
      lb.init([&](int rho) { return W + (size_t)w1row(rho) * a.d; },
              [&](int rho) { return S + (size_t)(w1row(rho) >> 7) * (a.d >> 7); });
      gemm_tile<T, C>(PlainLd<decltype(la)>{la}, PlainLd<decltype(lb)>{lb}, nk, smem, acc);
    } else {
      RowLoad<T, C::BN, C::NT> lb;
      lb.init((const T*)a.w1 + (size_t)e * 2 * a.dff * a.d, [&](int rho) { return w1row(rho) * a.d; });
      gemm_tile<T, C>(PlainLd<decltype(la)>{la}, PlainLd<decltype(lb)>{lb}, nk, smem, acc);
    }
    // SwiGLU in registers, then A (and [G, U] when saved) through LDS
    constexpr int LDA = HALF + 16 / (int)sizeof(T);
    const size_t abase = (size_t)slot0 * a.dff + nj * HALF;
    auto pairs = [&](auto&& put) {
#pragma unroll
      for (int p = 0; p < C::NB / 2; ++p) {
        const int lc = (wn * C::NB / 2 + p) * 32 + (lane & 31);
#pragma unroll
        for (int i = 0; i < C::MB; ++i)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            put(acc_row<C>(i, rr, lane), lc, acc[i][2 * p][rr], acc[i][2 * p + 1][rr]);
      }
    };
    MOE_LDS T* sa = smem;
    pairs([&](int row, int lc, float g, float u) {
      sa[row * LDA + lc] = to_act<T>(g / (1.f + expf(-g)) * u);
    });
    __syncthreads();
    lds_to_global<T, C::NT>(sa, C::BM, HALF, LDA, [&](int row, int col, const V16& v) {
      if (row < nrows) stg16(Ab + abase + (size_t)row * a.dff + col, v.u);
    });
    if (Z) {
      __syncthreads();
      MOE_LDS T* sg = smem;
      MOE_LDS T* su = smem + C::BM * LDA;
      pairs([&](int row, int lc, float g, float u) {
        sg[row * LDA + lc] = to_act<T>(g);
        su[row * LDA + lc] = to_act<T>(u);
      });
      __syncthreads();
      const size_t zbase = (size_t)slot0 * 2 * a.dff + nj * HALF;
      lds_to_global<T, C::NT>(sg, C::BM, HALF, LDA, [&](int row, int col, const V16& v) {
        if (row < nrows) stg16(Z + zbase + (size_t)row * 2 * a.dff + col, v.u);
      });
      lds_to_global<T, C::NT>(su, C::BM, HALF, LDA, [&](int row, int col, const V16& v) {
        if (row < nrows) stg16(Z + zbase + (size_t)row * 2 * a.dff + a.dff + col, v.u);
      });
    }
  }
}

// ---- forward: FC2 + gate ----------------------------------------------------
template <typename T, bool FP8, class C>
__global__ __launch_bounds__(C::NT) void k_fc2(ExecArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int tslot;
  __shared__ float pg[C::BM];
  MOE_LDS T* smem = (MOE_LDS T*)smem_raw;
  const int r = worker_of_block(a.P);
  const int nnt = a.d / C::BN;
  const int total = a.mt_cnt[r] * nnt;
  const int lane = threadIdx.x & 63;
  const T* Ab = (const T*)a.bufA;
  T* O = (T*)a.bufO;
  while (true) {
    const int tile = next_tile(&a.ctr[PH_FC2 * kMaxP + r], &tslot);
    if (tile >= total) break;
    const int4 m = a.mt[(size_t)r * a.max_mt + tile / nnt];
    const int nj = tile % nnt;
    const int e = m.x, slot0 = m.y, nrows = m.z;
    for (int i = threadIdx.x; i < C::BM; i += C::NT)
      pg[i] = i < nrows ? a.gates[a.slot_to_row[slot0 + i]] : 0.f;
    RowLoad<T, C::BM, C::NT> la;
    if constexpr (!kUseDma<T, FP8, C>)
      la.init(Ab + (size_t)slot0 * a.dff, [&](int row) { return row < nrows ? row * a.dff : -1; });
    f32x16_t acc[C::MB][C::NB];
    const int nk = a.dff / Elem<T>::BK;
    if constexpr (kUseDma<T, FP8, C>) {
      RowDma<C::BM, C::NT / 64> da;
      da.init((const uint16_t*)Ab, (uint32_t)(a.slots * a.dff * 2),
              [&](int row) { return row < nrows ? (slot0 + row) * a.dff : -1; });
      RowDma<C::BN, C::NT / 64> db;
      db.init((const uint16_t*)a.w2 + (size_t)e * a.d * a.dff, (uint32_t)((size_t)2 * a.d * a.dff),
              [&](int rho) { return (nj * C::BN + rho) * a.dff; });
      gemm_tile_dma<C>(da, db, a.dff / kDmaBK, smem, acc);
    } else if constexpr (FP8) {
      RowLoadFp8<C::BN, C::NT> lb;
      const uint8_t* W = (const uint8_t*)a.w2 + (size_t)e * a.d * a.dff;
      const float* S = a.w2s + (size_t)e * (a.d / 128) * (a.dff / 128);
      lb.init([&](int rho) { return W + (size_t)(nj * C::BN + rho) * a.dff; },
              [&](int rho) { return S + (size_t)((nj * C::BN + rho) >> 7) * (a.dff >> 7); });
      gemm_tile<T, C>(PlainLd<decltype(la)>{la}, PlainLd<decltype(lb)>{lb}, nk, smem, acc);
    } else {
      RowLoad<T, C::BN, C::NT> lb;
      lb.init((const T*)a.w2 + (size_t)e * a.d * a.dff + (size_t)nj * C::BN * a.dff,
              [&](int rho) { return rho * a.dff; });
      gemm_tile<T, C>(PlainLd<decltype(la)>{la}, PlainLd<decltype(lb)>{lb}, nk, smem, acc);
    }
    constexpr int LDO = C::BN + 16 / (int)sizeof(T);
    acc_to_lds<C>(acc, smem, LDO, 0, C::BM,
                  [&](float v, int row, int) { return to_act<T>(pg[row] * v); });
    __syncthreads();
    const size_t obase = (size_t)slot0 * a.d + nj * C::BN;
    lds_to_global<T, C::NT>(smem, C::BM, C::BN, LDO, [&](int row, int col, const V16& v) {
      if (row < nrows) stg16(O + obase + (size_t)row * a.d + col, v.u);
    });
  }
}

// ---- combine: out_t = sum_{j: slot(t,j) >= 0} src[slot(t,j)], fp32, j order ---
// One wave per (token, group of 64 16-byte chunks of the row): the token's
// slot indices are read (64 per load, lane j holding slot j) and taken out of
// their lanes as wave-uniform values; lane c covers chunk c of the group.  The
// values of up to 8 slots are loaded together and then added in slot order,
// starting from 0, in fp32, and the sum is rounded to the output dtype.  The
// slot rows themselves arrive in that dtype (FC2 and dX store them rounded),
// so a bf16 output is rounded twice in all.  Splitting a row into groups
// makes the units small (d = 2048 in bf16: four per token), so the last
// round of workgroups is short.
template <typename T>
__global__ __launch_bounds__(256) void k_combine(const T* __restrict__ src,
                                                 const int32_t* __restrict__ row_to_slot,
                                                 int T_, int k, int d, T* __restrict__ out) {
  constexpr int VE = Elem<T>::VE, G = 8;
  const int nch = d / VE, ngrp = (nch + 63) / 64;
  const size_t unit = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (unit >= (size_t)T_ * ngrp) return;                // the whole wave
  const int t = (int)(unit / ngrp), c = (int)(unit % ngrp) * 64 + lane;
  const bool live = c < nch;
  const int32_t* slots = row_to_slot + (size_t)t * k;
  float acc[VE];
#pragma unroll
  for (int v = 0; v < VE; ++v) acc[v] = 0.f;
  for (int j64 = 0; j64 < k; j64 += 64) {
    const int sl = j64 + lane < k ? slots[j64 + lane] : -1;
    const int nj = min(64, k - j64);
    for (int j0 = 0; j0 < nj; j0 += G) {
      V16 in[G];
      int sj[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        sj[g] = j0 + g < nj ? __builtin_amdgcn_readlane(sl, j0 + g) : -1;
        in[g].u = (sj[g] >= 0 && live) ? ldg16(src + (size_t)sj[g] * d + (size_t)c * VE) : zero4();
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (sj[g] < 0) continue;                        // wave-uniform
#pragma unroll
        for (int v = 0; v < VE; ++v) {
          if constexpr (sizeof(T) == 2) acc[v] += bf2f(in[g].h[v]);
          else acc[v] += in[g].f[v];
        }
      }
    }
  }
  if (!live) return;
  V16 o;
#pragma unroll
  for (int v = 0; v < VE; ++v) {
    if constexpr (sizeof(T) == 2) o.h[v] = f2bf(acc[v]);
    else o.f[v] = acc[v];
  }
  stg16(out + (size_t)t * d + (size_t)c * VE, o.u);
}

// grid of the combine: four waves (units) per workgroup
template <typename T> static dim3 combine_grid(int T_, int d) {
  const size_t units = (size_t)T_ * ((d / Elem<T>::VE + 63) / 64);
  return dim3((unsigned)((units + 3) / 4));
}

// ---- backward: dA -> dZ -------------------------------------------------------
// dA[slot, n] = p * sum_c dy[t, c] W2[c, n]; W2 is read as a K-major (c) by
// N-contiguous operand and transposed into LDS.
// ---- token-axis e4m3 requantization (fp8 backward) ----------------------------
// MegaFlux summary, "Backward": token-axis requantization of D_e and dZ_e.
// Blocks of `brows` consecutive rows (slots) times one column: scale =
// amax / 448, code = e4m3(value / scale) with round to nearest, ties to even,
// magnitudes saturated at 448; every step in fp32.  Row r's value is
//   map == nullptr: src[r * ld + c]
//   map[r] < 0 or map[r] >= map_lim:  0
//   otherwise:      src[(gather ? map[r] / div : r) * ld + c] * (rscale ? rscale[map[r]] : 1)
// (map_lim = rows of src times div, so a gathered row and its scale are in range).
// One workgroup per (block b, 128 columns): 16 threads cover a row's 128
// columns (8 each) and 16 rows are read at once.  Pass 1 takes each column's
// amax over the block's rows (exact in any order), reduced through LDS; pass
// 2 encodes.  A thread keeps its first kQtKeep rows (a 128-row block) in
// registers between the passes, as their bf16 source words and multiplier
// (the values are formed again, by the same product, in pass 2); rows beyond
// them are read again.  Row reads are branchless (a masked row loads row 0
// and keeps zero words), so a thread's rows are all in flight at once.
// DEQ: instead of codes and scales, write code * scale as bf16 to deq
// [rows][cols] (which may be src itself: pass 2 reads each value before the
// same thread overwrites it, and workgroups cover disjoint tiles).
// blk_end (nullable, device): only blocks b < *blk_end are processed; the
// layer passes the number of blocks in use, so the slot capacity beyond them
// costs one early exit per workgroup.
constexpr int kQtCols = 128, kQtRowLanes = 16, kQtKeep = 8;
template <bool DEQ>
__global__ __launch_bounds__(256) void k_quant_tok(const uint16_t* src, int ld,
                                                   const int32_t* __restrict__ map, int gather, int div,
                                                   const float* __restrict__ rscale, int map_lim,
                                                   int rows,
                                                   int cols, int brows, uint8_t* codes,
                                                   float* scales, uint16_t* deq,
                                                   const int32_t* __restrict__ blk_end) {
  __shared__ float part[kQtRowLanes][kQtCols];
  __shared__ float bsc[kQtCols];
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int b = blockIdx.x, c0 = blockIdx.y * kQtCols + tx * 8;
  if (blk_end && b >= *blk_end) return;                   // whole workgroup, before any barrier
  const bool colok = c0 < cols;
  const int r0 = b * brows, r1 = min(rows, r0 + brows);
  // a row's 8 bf16 source words and its multiplier; a masked row keeps zero
  // words (values +0) and multiplier 1
  auto raw8 = [&](int r, uint4& q, float& f) {
    int srow = r;
    bool ok = true;
    f = 1.f;
    if (map) {
      const int m = map[r];
      ok = m >= 0 && m < map_lim;
      if (gather) srow = ok ? m / div : 0;
      if (rscale) f = ok ? rscale[ok ? m : 0] : 1.f;
    }
    const uint4 l = *(const uint4*)(src + (size_t)srow * ld + c0);
    q = ok ? l : make_uint4(0, 0, 0, 0);
  };
  auto expand8 = [&](const uint4& q, float f, float* v) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16) * f;
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u) * f;
    }
  };
  auto value8 = [&](int r, float* v) {
    uint4 q;
    float f;
    raw8(r, q, f);
    expand8(q, f, v);
  };
  // v_cvt_pk_fp8_f32 rounds to nearest even on the OCP e4m3 grid: checked on
  // MI355X against a bit-level round-to-nearest-even encoder on every fp32
  // value of magnitude below 464, which covers every finite quotient here
  // (|v| <= amax, so |v / scale| <= 448 up to rounding)
  auto encode = [&](int r, const float* v, const float* sc) {
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = sc[i] > 0.f ? v[i] / sc[i] : 0.f;
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int p = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * h], q[4 * h + 1], 0, false);
      p = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * h + 2], q[4 * h + 3], p, true);
      w[h] = (uint32_t)p;
    }
    if constexpr (DEQ) {
      V16 o;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[h], false);
        const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[h], true);
        o.h[4 * h + 0] = f2bf(lo[0] * sc[4 * h + 0]);
        o.h[4 * h + 1] = f2bf(lo[1] * sc[4 * h + 1]);
        o.h[4 * h + 2] = f2bf(hi[0] * sc[4 * h + 2]);
        o.h[4 * h + 3] = f2bf(hi[1] * sc[4 * h + 3]);
      }
      *(uint4*)(deq + (size_t)r * cols + c0) = o.u;
    } else {
      *(uint2*)(codes + (size_t)r * cols + c0) = make_uint2(w[0], w[1]);
    }
  };
  // 5 registers a kept row instead of 8 values: more waves fit a SIMD
  uint4 kq[kQtKeep];
  float kf[kQtKeep];
  float amax[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (colok) {
#pragma unroll
    for (int u = 0; u < kQtKeep; ++u) {
      const int r = r0 + ty + kQtRowLanes * u;
      if (r < r1) {
        raw8(r, kq[u], kf[u]);
        float v[8];
        expand8(kq[u], kf[u], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax[i] = fmaxf(amax[i], fabsf(v[i]));
      }
    }
    for (int r = r0 + ty + kQtRowLanes * kQtKeep; r < r1; r += kQtRowLanes) {
      float v[8];
      value8(r, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax[i] = fmaxf(amax[i], fabsf(v[i]));
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[ty][tx * 8 + i] = amax[i];
  __syncthreads();
  if (ty == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float m = part[0][tx * 8 + i];
      for (int y = 1; y < kQtRowLanes; ++y) m = fmaxf(m, part[y][tx * 8 + i]);
      const float sc = m / 448.f;
      bsc[tx * 8 + i] = sc;
      if constexpr (!DEQ)
        if (colok) scales[(size_t)b * cols + c0 + i] = sc;
    }
  }
  __syncthreads();
  if (!colok) return;
  float sc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sc[i] = bsc[tx * 8 + i];
#pragma unroll
  for (int u = 0; u < kQtKeep; ++u) {
    const int r = r0 + ty + kQtRowLanes * u;
    if (r < r1) {
      float v[8];
      expand8(kq[u], kf[u], v);
      encode(r, v, sc);
    }
  }
  for (int r = r0 + ty + kQtRowLanes * kQtKeep; r < r1; r += kQtRowLanes) {
    float v[8];
    value8(r, v);
    encode(r, v, sc);
  }
}

// blocks on x (up to 2^31 - 1), 128-column tiles on y (cols <= kQtMaxCols)
static dim3 quant_grid(int rows, int cols, int brows) {
  return dim3((unsigned)((rows + brows - 1) / brows), (unsigned)((cols + kQtCols - 1) / kQtCols));
}

int launch_quant_tok(const uint16_t* src, int ld, const int32_t* map, int gather, int div,
                     const float* rscale, int map_lim, int rows, int cols, int brows,
                     uint8_t* codes, float* scales, hipStream_t st, const int32_t* blk_end) {
  if (rows > 0)
    hipLaunchKernelGGL(k_quant_tok<false>, quant_grid(rows, cols, brows), dim3(256), 0, st, src, ld,
                       map, gather, div, rscale, map_lim, rows, cols, brows, codes, scales, nullptr,
                       blk_end);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// ---- activation rows for the fp8 MFMA (power-of-two block scales) ------------
// Each row of x [rows][cols] (bf16) is cut into blocks of 128 features; block
// b of row r gets e = the smallest integer with amax <= 448 * 2^e (clamped to
// [-127, 127]; -127 for a zero block) and codes e4m3(x * 2^-e).  With amax =
// M * 2^E (M in [1, 2)) and 448 = 1.75 * 2^8 that is e = E - 8, or E - 7 when
// M > 1.75 (mantissa field above 0x600000).  One wave per row and group of 4
// blocks: 16 lanes per block, 8 values (16 bytes) per lane.  exps is
// block-major, exps[b * rows + r], so a GEMM step (one block) reads the
// exponents of its rows from one array row.
MOE_DEV int e8_exponent(float amax) {
  const uint32_t bits = __float_as_uint(amax);
  const int E = (int)((bits >> 23) & 0xFF) - 127;
  const int e = (bits & 0x7FFFFFFFu) == 0 ? -127 : E - 8 + ((bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// A task is one row and group of 4 blocks, one wave's work; waves walk the
// tasks grid-stride, two tasks in flight each.  With blk_end only the rows of
// the blocks in use (*blk_end blocks of blk_rows) are tasks.
__global__ __launch_bounds__(256) void k_quant_act(const uint16_t* __restrict__ x, int rows,
                                                   int cols, uint8_t* __restrict__ codes,
                                                   int32_t* __restrict__ exps,
                                                   const int32_t* __restrict__ blk_end, int blk_rows) {
  const int nb = cols / 128, ng = (nb + 3) / 4;
  long long rl = rows;
  if (blk_end) rl = min(rl, (long long)*blk_end * blk_rows);
  const long long ntask = rl * ng, nw = (long long)gridDim.x * 4;
  const int lane = threadIdx.x & 63;
  for (long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); t < ntask; t += 2 * nw) {
    uint4 q[2];
    size_t off[2];
    int r[2], b[2];
    bool on[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const long long tu = t + u * nw;
      r[u] = (int)(tu / ng);
      b[u] = (int)(tu % ng) * 4 + (lane >> 4);
      on[u] = tu < ntask && b[u] < nb;
      off[u] = on[u] ? (size_t)r[u] * cols + (size_t)b[u] * 128 + 8 * (lane & 15) : 0;
      q[u] = on[u] ? *(const uint4*)(x + off[u]) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && t + nw >= ntask) break;              // wave-uniform: no second task
      const uint32_t w[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
      float v[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
      for (int sh = 8; sh >= 1; sh >>= 1) m = fmaxf(m, __shfl_xor(m, sh, 64));  // within 16 lanes
      const int e = e8_exponent(m);
      uint32_t c[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int p = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * h], -e), ldexpf(v[4 * h + 1], -e), 0,
                                                false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * h + 2], -e), ldexpf(v[4 * h + 3], -e), p,
                                            true);
        c[h] = (uint32_t)p;
      }
      if (on[u]) {
        *(uint2*)(codes + off[u]) = make_uint2(c[0], c[1]);
        if ((lane & 15) == 0) exps[(size_t)b[u] * rows + r[u]] = e;
      }
    }
  }
}

// Every task its own wave when all rows are tasks; when the rows in use are
// known only on the device (blk_end), one resident round of workgroups (8 of
// 4 waves per CU) walks them, so the capacity past them costs nothing.
static constexpr long long kQuantActWG = 256 * 8;

int launch_quant_act(const uint16_t* x, int rows, int cols, uint8_t* codes, int32_t* exps,
                     hipStream_t st, const int32_t* blk_end, int blk_rows) {
  const long long tasks = (long long)rows * ((cols / 128 + 3) / 4);
  const long long all = (tasks + 3) / 4;
  const long long wg = (blk_end || all > (1LL << 30)) ? std::min(all, kQuantActWG) : all;
  if (tasks > 0)
    hipLaunchKernelGGL(k_quant_act, dim3((unsigned)wg), dim3(256), 0, st, x, rows, cols, codes,
                       exps, blk_end, blk_rows);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_DEV float sigm(float g) { return __builtin_amdgcn_rcpf(1.f + __expf(-g)); }

// SwiGLU gradient and dZ's e4m3 rows for dX on the fp8 MFMA: for each slot
// row s in use (s < *blk_end * beta, slot_to_row[s] >= 0) and feature f of
// d_ff, from dA (bf16 [slots][d_ff], gate applied) and [G, U] (z_save
// [slots][2 d_ff]): sg = sigmoid(G), dG = dA U sg (1 + G (1 - sg)),
// dU = dA G sg, P = SiLU(G) U.  dZ = [dG, dU] is stored bf16 into dz
// [slots][2 d_ff] and P into p [slots][d_ff]; dZ's bf16 values are
// quantized per row and 128 features as k_quant_act quantizes rows (codes
// [slots][2 d_ff], exps [2 d_ff / 128][slots]).  A task is one row and group
// of 4 blocks of 128 features, one wave, 16 lanes a block, 8 features a
// lane; waves walk the tasks grid-stride.  Padding slots are left alone.
__global__ __launch_bounds__(256) void k_swiglu_bwd_q(
    const uint16_t* __restrict__ dA, const uint16_t* __restrict__ Z,
    const int32_t* __restrict__ slot_to_row, int slots, int dff, uint16_t* __restrict__ dz,
    uint16_t* __restrict__ P, uint8_t* __restrict__ codes, int32_t* __restrict__ exps,
    const int32_t* __restrict__ blk_end, int beta) {
  const int nb = dff / 128, ng = (nb + 3) / 4;
  const long long rl = min((long long)slots, (long long)*blk_end * beta);
  const long long ntask = rl * ng, nw = (long long)gridDim.x * 4;
  const int lane = threadIdx.x & 63;
  for (long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); t < ntask; t += nw) {
    const int r = (int)(t / ng);
    if (slot_to_row[r] < 0) continue;                       // wave-uniform
    const int b = (int)(t % ng) * 4 + (lane >> 4);
    const bool on = b < nb;
    const int c = b * 128 + 8 * (lane & 15);
    uint4 qa = make_uint4(0, 0, 0, 0), qg = qa, qu = qa;
    if (on) {
      qa = *(const uint4*)(dA + (size_t)r * dff + c);
      qg = *(const uint4*)(Z + (size_t)r * 2 * dff + c);
      qu = *(const uint4*)(Z + (size_t)r * 2 * dff + dff + c);
    }
    const uint32_t wa[4] = {qa.x, qa.y, qa.z, qa.w}, wg[4] = {qg.x, qg.y, qg.z, qg.w},
                   wu[4] = {qu.x, qu.y, qu.z, qu.w};
    float vg[8], vu[8];
    uint32_t og[4], ou[4], op[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int sh = (i & 1) ? 16 : 0;
      const float da = bf2f((uint16_t)(wa[i >> 1] >> sh)), g = bf2f((uint16_t)(wg[i >> 1] >> sh)),
                  u = bf2f((uint16_t)(wu[i >> 1] >> sh));
      const float sg = sigm(g);
      const uint16_t hg = f2bf(da * u * sg * (1.f + g * (1.f - sg)));
      const uint16_t hu = f2bf(da * g * sg);
      const uint16_t hp = f2bf(g * sg * u);
      vg[i] = bf2f(hg);
      vu[i] = bf2f(hu);
      if (i & 1) {
        og[i >> 1] |= (uint32_t)hg << 16;
        ou[i >> 1] |= (uint32_t)hu << 16;
        op[i >> 1] |= (uint32_t)hp << 16;
      } else {
        og[i >> 1] = hg;
        ou[i >> 1] = hu;
        op[i >> 1] = hp;
      }
    }
    float mg = 0.f, mu = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mg = fmaxf(mg, fabsf(vg[i]));
      mu = fmaxf(mu, fabsf(vu[i]));
    }
#pragma unroll
    for (int sh = 8; sh >= 1; sh >>= 1) {                   // within 16 lanes
      mg = fmaxf(mg, __shfl_xor(mg, sh, 64));
      mu = fmaxf(mu, __shfl_xor(mu, sh, 64));
    }
    const int eg = e8_exponent(mg), eu = e8_exponent(mu);
    uint32_t cg[2], cu[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int p = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(vg[4 * h], -eg), ldexpf(vg[4 * h + 1], -eg), 0,
                                              false);
      cg[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(vg[4 * h + 2], -eg),
                                                        ldexpf(vg[4 * h + 3], -eg), p, true);
      p = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(vu[4 * h], -eu), ldexpf(vu[4 * h + 1], -eu), 0,
                                          false);
      cu[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(vu[4 * h + 2], -eu),
                                                        ldexpf(vu[4 * h + 3], -eu), p, true);
    }
    if (on) {
      const size_t rz = (size_t)r * 2 * dff;
      *(uint4*)(dz + rz + c) = make_uint4(og[0], og[1], og[2], og[3]);
      *(uint4*)(dz + rz + dff + c) = make_uint4(ou[0], ou[1], ou[2], ou[3]);
      *(uint4*)(P + (size_t)r * dff + c) = make_uint4(op[0], op[1], op[2], op[3]);
      *(uint2*)(codes + rz + c) = make_uint2(cg[0], cg[1]);
      *(uint2*)(codes + rz + dff + c) = make_uint2(cu[0], cu[1]);
      if ((lane & 15) == 0) {
        exps[(size_t)b * slots + r] = eg;
        exps[(size_t)(nb + b) * slots + r] = eu;
      }
    }
  }
}

static void launch_swiglu_bwd_q(const ExecArgs& a, int dff, const int32_t* blk_end, int beta,
                                hipStream_t st) {
  const long long tasks = (long long)a.slots * ((dff / 128 + 3) / 4);
  if (tasks > 0)
    hipLaunchKernelGGL(k_swiglu_bwd_q, dim3((unsigned)std::min((tasks + 3) / 4, kQuantActWG)),
                       dim3(256), 0, st, (const uint16_t*)a.bufO, (const uint16_t*)a.z_save,
                       a.slot_to_row, (int)a.slots, dff, (uint16_t*)a.bufA, (uint16_t*)a.bufP,
                       (uint8_t*)a.hq, a.he, blk_end, beta);
}

// The same blocks, written back as bf16 code * scale into deq [rows][cols].
static void launch_quant_dequant(const uint16_t* src, int ld, const int32_t* map, int gather,
                                 int div, const float* rscale, int map_lim, int rows, int cols,
                                 int brows, uint16_t* deq, const int32_t* blk_end, hipStream_t st) {
  if (rows > 0)
    hipLaunchKernelGGL(k_quant_tok<true>, quant_grid(rows, cols, brows), dim3(256), 0, st, src, ld,
                       map, gather, div, rscale, map_lim, rows, cols, brows, nullptr, nullptr, deq,
                       blk_end);
}

// fp8 weight rows read K-major: element (k, n) = code[k * ld + n] * scale[k / 128][n / 128],
// eight consecutive n widened to bf16 (n0 and every mn are multiples of 8)
struct SrcRowsMNFp8 {
  const uint8_t* base;
  const float* scale;
  int ld, n0, nlim, sld;
  MOE_DEV uint4 operator()(int kk, int mn) const {
    const int n = n0 + mn;
    if (n >= nlim) return zero4();
    const uint2 c = *(const uint2*)(base + (size_t)kk * ld + n);
    const float s = scale[(size_t)(kk >> 7) * sld + (n >> 7)];
    const uint32_t w[2] = {c.x, c.y};
    V16 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o.h[i] = f2bf(e4m3_to_f32((w[i >> 2] >> (8 * (i & 3))) & 0xFFu) * s);
    return o.u;
  }
};

// token-axis e4m3 slot rows: element (k, m) = code[(slot0 + k) * ld + m0 + m] *
// scale[(slot0 + k) / beta][m0 + m], widened to bf16
struct SrcSlotRowFp8 {
  const uint8_t* codes;
  const float* scales;
  int slot0, nrows, ld, m0, mlim, beta;
  MOE_DEV uint4 operator()(int kk, int mn) const {
    const int m = m0 + mn;
    if (kk >= nrows || m >= mlim) return zero4();
    const size_t slot = (size_t)slot0 + kk;
    const uint2 c = *(const uint2*)(codes + slot * ld + m);
    const float4 s0 = *(const float4*)(scales + (slot / beta) * ld + m);
    const float4 s1 = *(const float4*)(scales + (slot / beta) * ld + m + 4);
    const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    const uint32_t w[2] = {c.x, c.y};
    V16 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o.h[i] = f2bf(e4m3_to_f32((w[i >> 2] >> (8 * (i & 3))) & 0xFFu) * s[i]);
    return o.u;
  }
};

template <typename T> struct SrcRowsMN {       // element (k, n) = base[k * ld + n0 + n]
  const T* base;
  int ld, n0, nlim;
  MOE_DEV uint4 operator()(int kk, int mn) const {
    const int n = n0 + mn;
    return n < nlim ? ldg16(base + (size_t)kk * ld + n) : zero4();
  }
};

MOE_DEV void load4(const uint16_t* p, float* v) {
  const uint2 q = *(const uint2*)p;
  v[0] = bf2f((uint16_t)(q.x & 0xffff)); v[1] = bf2f((uint16_t)(q.x >> 16));
  v[2] = bf2f((uint16_t)(q.y & 0xffff)); v[3] = bf2f((uint16_t)(q.y >> 16));
}
MOE_DEV void load4(const float* p, float* v) {
  const float4 q = *(const float4*)p;
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
MOE_DEV void store4(uint16_t* p, const float* v) {
  uint2 q;
  q.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  q.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  *(uint2*)p = q;
}
MOE_DEV void store4(float* p, const float* v) { *(float4*)p = make_float4(v[0], v[1], v[2], v[3]); }

template <typename T, class C, bool FP8 = false>
__global__ __launch_bounds__(C::NT) void k_bwd_da(ExecArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int tslot;
  __shared__ float pg[C::BM];
  MOE_LDS T* smem = (MOE_LDS T*)smem_raw;
  const int r = worker_of_block(a.P);
  const int nnt = (a.dff + C::BN - 1) / C::BN;
  const int total = a.mt_cnt[r] * nnt;
  const int lane = threadIdx.x & 63;
  const T* DY = (const T*)a.dy;
  const T* Z = (const T*)a.z_save;
  T* dZ = (T*)a.bufA;
  T* PA = (T*)a.bufP;    // P = p * SiLU(G) * U, written when a consumer needs it
  while (true) {
    const int tile = next_tile(&a.ctr[PH_DA * kMaxP + r], &tslot);
    if (tile >= total) break;
    const int4 m = a.mt[(size_t)r * a.max_mt + tile / nnt];
    const int nj = tile % nnt;
    const int e = m.x, slot0 = m.y, nrows = m.z;
    for (int i = threadIdx.x; i < C::BM; i += C::NT)
      pg[i] = i < nrows ? a.gates[a.slot_to_row[slot0 + i]] : 0.f;
    RowLoad<T, C::BM, C::NT> la;
    la.init(DY, [&](int row) { return row < nrows ? (a.slot_to_row[slot0 + row] / a.k) * a.d : -1; });
    TransLoad<T, C::BN, C::NT> lb;
    lb.init();
    f32x16_t acc[C::MB][C::NB];
    if constexpr (FP8) {
      SrcRowsMNFp8 src{(const uint8_t*)a.w2 + (size_t)e * a.d * a.dff,
                       a.w2s + (size_t)e * (a.d / 128) * (a.dff / 128), a.dff, nj * C::BN, a.dff,
                       a.dff / 128};
      gemm_tile<T, C>(PlainLd<decltype(la)>{la}, TransLd<decltype(lb), SrcRowsMNFp8>{lb, src},
                      a.d / Elem<T>::BK, smem, acc);
    } else {
      SrcRowsMN<T> src{(const T*)a.w2 + (size_t)e * a.d * a.dff, a.dff, nj * C::BN, a.dff};
      gemm_tile<T, C>(PlainLd<decltype(la)>{la}, TransLd<decltype(lb), SrcRowsMN<T>>{lb, src},
                      a.d / Elem<T>::BK, smem, acc);
    }
    // p * dA in fp32 through LDS, 128 rows at a time; the SwiGLU gradient is
    // applied on the way out with 4-wide coalesced reads of the saved [G, U]
    constexpr int PASS = 128, LDD = C::BN + 4;
    MOE_LDS float* sd = (MOE_LDS float*)smem;
    for (int p0 = 0; p0 < C::BM; p0 += PASS) {
      if (p0) __syncthreads();
      acc_to_lds<C>(acc, sd, LDD, p0, PASS, [&](float v, int row, int) { return pg[row] * v; });
      __syncthreads();
      lds_to_global<float, C::NT>(sd, PASS, C::BN, LDD, [&](int rl, int col, const V16& v) {
        const int row = p0 + rl, n = nj * C::BN + col;
        if (row >= nrows || n >= a.dff) return;
        const size_t zb = ((size_t)slot0 + row) * 2 * a.dff + n;
        float g[4], u[4], dg[4], du[4], pa[4];
        load4(Z + zb, g);
        load4(Z + zb + a.dff, u);
        const float p = pg[row];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float sg = 1.f / (1.f + expf(-g[q]));
          dg[q] = v.f[q] * u[q] * sg * (1.f + g[q] * (1.f - sg));
          du[q] = v.f[q] * g[q] * sg;
          pa[q] = p * (g[q] * sg * u[q]);
        }
        store4(dZ + zb, dg);
        store4(dZ + zb + a.dff, du);
        if (PA) store4(PA + ((size_t)slot0 + row) * a.dff + n, pa);
      });
    }
  }
}

// ---- backward: dX per routed row ----------------------------------------------
template <typename T, class C, bool FP8 = false>
__global__ __launch_bounds__(C::NT) void k_bwd_dx(ExecArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int tslot;
  MOE_LDS T* smem = (MOE_LDS T*)smem_raw;
  const int r = worker_of_block(a.P);
  const int nnt = a.d / C::BN;
  const int total = a.mt_cnt[r] * nnt;
  const int lane = threadIdx.x & 63;
  const T* dZ = (const T*)a.bufA;
  T* dXp = (T*)a.bufO;
  while (true) {
    const int tile = next_tile(&a.ctr[PH_DX * kMaxP + r], &tslot);
    if (tile >= total) break;
    const int4 m = a.mt[(size_t)r * a.max_mt + tile / nnt];
    const int nj = tile % nnt;
    const int e = m.x, slot0 = m.y, nrows = m.z;
    RowLoad<T, C::BM, C::NT> la;
    la.init(dZ + (size_t)slot0 * 2 * a.dff, [&](int row) { return row < nrows ? row * 2 * a.dff : -1; });
    TransLoad<T, C::BN, C::NT> lb;
    lb.init();
    f32x16_t acc[C::MB][C::NB];
    if constexpr (FP8) {
      SrcRowsMNFp8 src{(const uint8_t*)a.w1 + (size_t)e * 2 * a.dff * a.d,
                       a.w1s + (size_t)e * (2 * a.dff / 128) * (a.d / 128), a.d, nj * C::BN, a.d,
                       a.d / 128};
      gemm_tile<T, C>(PlainLd<decltype(la)>{la}, TransLd<decltype(lb), SrcRowsMNFp8>{lb, src},
                      2 * a.dff / Elem<T>::BK, smem, acc);
    } else {
      SrcRowsMN<T> src{(const T*)a.w1 + (size_t)e * 2 * a.dff * a.d, a.d, nj * C::BN, a.d};
      gemm_tile<T, C>(PlainLd<decltype(la)>{la}, TransLd<decltype(lb), SrcRowsMN<T>>{lb, src},
                      2 * a.dff / Elem<T>::BK, smem, acc);
    }
    constexpr int LDO = C::BN + 16 / (int)sizeof(T);
    acc_to_lds<C>(acc, smem, LDO, 0, C::BM, [&](float v, int, int) { return to_act<T>(v); });
    __syncthreads();
    const size_t obase = (size_t)slot0 * a.d + nj * C::BN;
    lds_to_global<T, C::NT>(smem, C::BM, C::BN, LDO, [&](int row, int col, const V16& v) {
      if (row < nrows) stg16(dXp + obase + (size_t)row * a.d + col, v.u);
    });
  }
}

// ---- GEMM kernels on the persistent wide tile -----------------------------------
// 256 x 256 tiles, 8 waves, transposed accumulators: lane (lane & 31) of wave
// (wm, wn) owns rows wm*128 + 32 i + (lane & 31) and, per register quad g of
// block j, the four consecutive columns wn*64 + 32 j + 8 g + 4 (lane >> 5)
// .. +3, stored straight from registers.  Each workgroup walks its worker's
// items (M tile x N tile) in a static sequence through WideStream.  Fast exp
// and reciprocal in the SiLU terms: their error is far below the bf16
// rounding of every value they feed.

using WC = WideCfg;
constexpr int kWNW = WC::NT / 64;
// the row-tile kernels (FC1, FC2, dA, dX): K = 64 per stage, two stages
constexpr int kRowBK = 64;
using RowW = RowK<256, kWNW, kRowBK>;
using MnW = MnK<256, kWNW, kRowBK>;
constexpr int kItemSlots = 3;
constexpr size_t kItemBytes = 2048;           // 256 slot -> row entries, 256 slot gates
constexpr size_t kStageBytes = kWideLdsStages;
// vmcnt wait counts saturate at 63: a smaller count only waits for more
constexpr int vm_clamp(int n) { return n < 63 ? n : 63; }
constexpr size_t kEpiOff = kStageBytes + kItemSlots * kItemBytes;   // per-wave epilogue scratch
constexpr size_t kEpiWave = 2048;
constexpr size_t kStreamLds = kEpiOff + (WC::NT / 64) * kEpiWave;

// ---- row-contiguous epilogue stores ------------------------------------------
// A wave's transposed accumulators hold, per lane, 4-value pieces of one row;
// stored directly, every store instruction would touch 32 rows with 16 bytes
// each, which sustains well under a third of the HBM write rate of row
// segments.  So each 16-row half of a 32-row block goes through a 2 KB
// per-wave LDS scratch: the lanes holding those rows write their pieces, then
// all 64 lanes read back 16-byte chunks in row order and store them, each
// instruction covering whole row segments of SEG 32-column blocks
// (RB = 32 * SEG * sizeof(T) bytes, 64 or 128).  Chunk c of scratch row r
// sits at chunk c ^ swz(r), which keeps the 16-lane groups of both the writes
// and the reads on distinct banks.  A wave's LDS operations complete in
// order, so no barrier or wait is needed between the passes.
template <typename T, int SEG> struct RowStore {
  static constexpr int RB = 32 * SEG * (int)sizeof(T);
  static constexpr int CPR = RB / 16;
  static constexpr int NRD = 16 * CPR / 64;                 // read/store instructions per half block
  static constexpr int STORES = 2 * NRD;                    // emits per block
  static_assert(RB == 64 || RB == 128, "segment row bytes");
  // measured on gfx950 (bank-conflict counter): with these chunk swizzles the
  // row-block reads are conflict-free, the fp32 16-byte writes too, and the
  // bf16 8-byte writes of half the lanes take the 2 extra cycles that every
  // swizzle tried leaves them
  static MOE_DEV int swz(int r) { return RB == 128 ? r & 7 : (r >> 2) & 3; }
  // vals(jj, g, v): the 4 values of quad g of block j0 + jj of this lane's row;
  // emit(row, chunk, data): store 16 bytes at `row` (0..31 inside the block)
  // and 16-byte chunk `chunk` of the segment.
  // The values are computed and packed by every lane first; the two halves of
  // the block then take turns in the per-wave scratch.
  using Packed = typename std::conditional<sizeof(T) == 4, u32x4_t, u32x2_t>::type;
  template <class V>
  static MOE_DEV void pack(V vals, Packed (&p)[SEG][4]) {
#pragma unroll
    for (int jj = 0; jj < SEG; ++jj)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
        vals(jj, g, v);
        if constexpr (sizeof(T) == 4)
          p[jj][g] = u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                             __float_as_uint(v[3])};
        else
          p[jj][g] = u32x2_t{(uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16),
                             (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16)};
      }
  }
  template <class EM>
  static MOE_DEV void store(MOE_LDS char* scr, const Packed (&p)[SEG][4], EM emit) {
    const int lane = threadIdx.x & 63, lr = lane & 31, h = lane >> 5;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      wave_lds_sync();                     // the previous reads of the scratch are done
      if ((lr >> 4) == half) {
        const int r = lr & 15;
#pragma unroll
        for (int jj = 0; jj < SEG; ++jj)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            if constexpr (sizeof(T) == 4) {
              const int c = jj * 8 + 2 * g + h;
              *(MOE_LDS u32x4_t*)(scr + r * RB + ((c ^ swz(r)) << 4)) = p[jj][g];
            } else {
              const int c = jj * 4 + g;
              *(MOE_LDS u32x2_t*)(scr + r * RB + ((c ^ swz(r)) << 4) + 8 * h) = p[jj][g];
            }
          }
      }
      wave_lds_sync();                     // other lanes' writes are visible
      u32x4_t d[NRD];
#pragma unroll
      for (int sI = 0; sI < NRD; ++sI) {
        const int q = sI * 64 + lane, rr = q / CPR, c = q % CPR;
        d[sI] = *(const MOE_LDS u32x4_t*)(scr + rr * RB + ((c ^ swz(rr)) << 4));
      }
#pragma unroll
      for (int sI = 0; sI < NRD; ++sI) {
        const int q = sI * 64 + lane;
        emit(16 * half + q / CPR, q % CPR, d[sI]);
      }
    }
  }
  template <class V, class EM>
  static MOE_DEV void run(MOE_LDS char* scr, V vals, EM emit) {
    Packed p[SEG][4];
    pack(vals, p);
    store(scr, p, emit);
  }
};

MOE_DEV MOE_LDS char* epi_scratch(MOE_LDS uint16_t* smem) {
  return (MOE_LDS char*)smem + kEpiOff + (size_t)wave_id() * kEpiWave;
}
// Weight-gradient tiles are written once and not read again by this layer:
// non-temporal stores keep the 2.4 GB of fp32 tiles of a launch from evicting
// the operand panels the next tiles of the same segment read from L2 (6% off
// the kernel on the Qwen3-shaped workload, measured against plain stores).
MOE_DEV void stg4v(float* p, float v) { __builtin_nontemporal_store(v, (MOE_GLB float*)p); }
// 16 bytes at element column `col` of slot row `srow` of a [slots][ld] bf16
// buffer; a row past the tile's end is sent out of range and dropped, so an
// epilogue issues the same number of stores for every tile
template <int CP = kStoreLocal>
MOE_DEV void st_row16(const BufRsrc& r, int srow, int ld, int col, bool ok, const u32x4_t& d) {
  buf_store16c<CP>(r, ok ? ((uint32_t)srow * (uint32_t)ld + (uint32_t)col) * 2u : kOob, d);
}

MOE_DEV const MOE_LDS int* item_rows(const MOE_LDS uint16_t* smem, int slot) {
  return (const MOE_LDS int*)((const MOE_LDS char*)smem + kStageBytes + slot * kItemBytes);
}
MOE_DEV const MOE_LDS float* item_gates(const MOE_LDS uint16_t* smem, int slot) {
  return (const MOE_LDS float*)((const MOE_LDS char*)smem + kStageBytes + slot * kItemBytes + 1024);
}
// 256 consecutive 4-byte values from byte offset `off` of `rs` into LDS (one
// wave instruction; slots past the buffer read as zeros).
MOE_DEV void load_1k(BufRsrc rs, uint32_t off, MOE_LDS uint16_t* smem, size_t lds_off) {
  buf_load_lds16(rs, off + (uint32_t)(threadIdx.x & 63) * 16u,
                 (MOE_LDS void*)((MOE_LDS char*)smem + lds_off));
}
// token of routed row `row` = row / k, exact for the sizes the host admits
MOE_DEV uint32_t token_of(uint32_t row, uint32_t kmagic) { return __umulhi(row, kmagic); }

// M-tile item: tile idx / nnt of the worker's list, N tile idx % nnt.
struct MItem { int e, slot0, nrows, nj; };
struct MSrcBase {
  ExecArgs a;              // a copy: the fields stay in scalar registers
  MOE_LDS uint16_t* smem;
  int r, nnt, count, first, stride;
  MOE_DEV void init(const ExecArgs& args, MOE_LDS uint16_t* sm, int ntiles_n) {
    a = args;
    smem = sm;
    const WorkerSlot w = worker_slot(args.P);
    r = w.r;
    nnt = ntiles_n;
    count = args.mt_cnt[r] * nnt;
    first = w.j;
    stride = w.n;
  }
  // this wave's rows of the tile include routed rows
  MOE_DEV bool wave_active(const MItem& it) const {
    return (wave_id() / WC::WAVES_N) * WC::WM < it.nrows;
  }
  // scalar load: nothing waits on vector loads in flight
  MOE_DEV MItem load(int idx) const {
    const u32x4_t m = ((const MOE_CONST u32x4_t*)a.mt)[(size_t)r * a.max_mt + idx / nnt];
    return {(int)m.x, (int)m.y, (int)m.z, idx % nnt};
  }
  MOE_DEV void fill_rows(const MItem& it, int slot) const {     // slot -> row of the tile's rows
    if (wave_id() == 0)
      load_1k(make_rsrc(a.slot_to_row, (uint32_t)(a.slots * 4)), (uint32_t)it.slot0 * 4u, smem,
              kStageBytes + slot * kItemBytes);
  }
  MOE_DEV void fill_gates(const MItem& it, int slot) const {    // gate of the tile's rows
    if (wave_id() == 1)
      load_1k(make_rsrc(a.sgate, (uint32_t)(a.slots * 4)), (uint32_t)it.slot0 * 4u, smem,
              kStageBytes + slot * kItemBytes + 1024);
  }
  // A operand: gathered token rows of `base` ([T][ld]) for the tile's slots
  MOE_DEV RowW gathered(const MItem& it, int slot, const void* base, int ld) const {
    const MOE_LDS int* rows = item_rows(smem, slot);
    int o[RowW::NI];
#pragma unroll
    for (int i = 0; i < RowW::NI; ++i) {
      const int row = RowW::lane_row(i);
      o[i] = row < it.nrows ? (int)token_of((uint32_t)rows[row], a.kmagic) * ld : -1;
    }
    RowW x;
    x.init_offsets((const uint16_t*)base, (uint32_t)((size_t)a.T * ld * 2), o);
    return x;
  }
  // A operand: slot rows of `base` ([slots][ld])
  MOE_DEV RowW slotrows(const MItem& it, const void* base, int ld) const {
    RowW x;
    x.init((const uint16_t*)base, (uint32_t)(a.slots * ld * 2),
           [&](int row) { return row < it.nrows ? (it.slot0 + row) * ld : -1; });
    return x;
  }
};

// K-major weight operand: row k of a [K][ld] matrix from column col.
struct MnFixed {
  uint32_t ld2, col2;
  using Raw = uint32_t;
  MOE_DEV Raw pre(int, int k) const { return (uint32_t)k; }
  MOE_DEV uint32_t post(Raw raw, int) const { return raw * ld2 + col2; }
};
using MnFixedOp = MnKOperand<MnW, MnFixed>;
// e4m3 K-major weights (dA, dX)
using MnF8 = MnKFp8<256, kWNW, kRowBK>;
using MnF8Op = MnKOperand<MnF8, MnFixed>;

// e4m3 weight rows for the wide tile (the stream widens them to bf16)
using RowF8 = RowKFp8<256, kWNW, kRowBK>;

// FC1 + SwiGLU.  N tile nj covers A columns [128 nj, 128 nj + 128): weight
// rows alternate 32 G rows and the matching 32 U rows, so block j = 0 of a
// wave is G and block j = 1 is U of the same 32 columns.  With e4m3 weights
// the G rows of tile nj lie in scale block nj and the U rows in d_ff/128 + nj.
// COH: A is stored with device-scope completion, read by FC2 items of the
// same launch (the saved [G, U] is only read by later launches).
template <bool FP8, bool COH = false> struct SrcFc1T : MSrcBase {
  static constexpr bool kSkipIdle = true;
  using Item = MItem;
  using OB = typename std::conditional<FP8, RowF8, RowW>::type;
  MOE_DEV void fill(const Item& it, int slot) const { fill_rows(it, slot); }
  MOE_DEV RowW opA(const Item& it, int slot) const { return gathered(it, slot, a.x, a.d); }
  MOE_DEV OB opB(const Item& it, int) const {
    OB w;
    const int dff = a.dff, nj = it.nj;
    auto row = [&](int rho) {
      const int q = rho >> 5;
      return ((q & 1) * dff + nj * (WC::BN / 2) + (q >> 1) * 32 + (rho & 31)) * a.d;
    };
    if constexpr (FP8) {
      w.init((const uint8_t*)a.w1 + (size_t)it.e * 2 * dff * a.d, (uint32_t)((size_t)2 * dff * a.d),
             row);
      const int kb = a.d / 128;
      const MOE_CONST float* sc = (const MOE_CONST float*)a.w1s + (size_t)it.e * (2 * dff / 128) * kb;
      w.sp[0] = sc + (size_t)nj * kb;
      w.sp[1] = sc + (size_t)(dff / 128 + nj) * kb;
    } else {
      w.init((const uint16_t*)a.w1 + (size_t)it.e * 2 * dff * a.d, (uint32_t)((size_t)4 * dff * a.d),
             row);
    }
    return w;
  }
  MOE_DEV int steps(const Item&) const { return a.d / kRowBK; }
  static constexpr int kEpiVmA = WC::MB * RowStore<uint16_t, 1>::STORES;   // A only
  template <int B> MOE_DEV void relaxed_wait() const {
    if (a.z_save) wait_vm_lgkm0<vm_clamp(B + 3 * kEpiVmA)>();
    else wait_vm_lgkm0<vm_clamp(B + kEpiVmA)>();
  }
  MOE_DEV void epilogue(const Item& it, int, const f32x16_t (&acc)[WC::MB][WC::NB]) const {
    const int wm = wave_id() / WC::WAVES_N, wn = wave_id() % WC::WAVES_N;
    const int dff = a.dff, colb = it.nj * (WC::BN / 2) + wn * 32;
    const BufRsrc ra = make_rsrc(a.bufA, (uint32_t)(a.slots * dff * 2));
    const BufRsrc rz = make_rsrc(a.z_save, (uint32_t)(a.slots * dff * 4));
    MOE_LDS char* scr = epi_scratch(smem);
#pragma unroll
    for (int i = 0; i < WC::MB; ++i) {
      const int rb = wm * WC::WM + i * 32;
      auto emit_to = [&](const BufRsrc& r, int col0, int ld, auto cp) {
        return [&, col0, ld](int row, int c, const u32x4_t& d) {
          st_row16<decltype(cp)::value>(r, it.slot0 + rb + row, ld, col0 + colb + c * 8,
                                        rb + row < it.nrows, d);
        };
      };
      using CpA = std::integral_constant<int, COH ? kStoreDevice : kStoreLocal>;
      using CpZ = std::integral_constant<int, kStoreLocal>;
      RowStore<uint16_t, 1>::run(scr, [&](int, int g, float* v) {
        for (int q = 0; q < 4; ++q) {
          const float gv = acc[i][0][4 * g + q];
          v[q] = gv * sigm(gv) * acc[i][1][4 * g + q];
        }
      }, emit_to(ra, 0, dff, CpA{}));
      if (a.z_save) {
        RowStore<uint16_t, 1>::run(scr, [&](int, int g, float* v) {
          for (int q = 0; q < 4; ++q) v[q] = acc[i][0][4 * g + q];
        }, emit_to(rz, 0, 2 * dff, CpZ{}));
        RowStore<uint16_t, 1>::run(scr, [&](int, int g, float* v) {
          for (int q = 0; q < 4; ++q) v[q] = acc[i][1][4 * g + q];
        }, emit_to(rz, dff, 2 * dff, CpZ{}));
      }
    }
  }
};

// FC1 on the fp8 MFMA (MOE_EXEC_FP8_ACT, e4m3 weights): the A rows are x
// quantized per token row and 128 features with power-of-two scales
// (k_quant_act: codes in xq, exponents in xe), the B rows the weights' codes
// as stored; a K step is 128 codes (one weight scale block), the row
// exponents ride in the MFMA's scale operand and the weights' fp32 block
// scales are applied to the accumulators per step (WideStream's fp8 mode).
// The epilogue is FC1's.
constexpr size_t kScOff8 = kStreamLds;           // two 1 KB exponent regions after the scratch
constexpr size_t kStreamLds8 = kStreamLds + 2 * 1024;
using RowA8 = RowK8A<256, kWNW, kScOff8>;
using RowW8 = RowK8W<256, kWNW>;
// The tile's rows as quantized token rows: codes [T][d] (read as element
// offsets of code pairs, token * d / 2) and exponents [d / 128][T].
MOE_DEV RowA8 gathered8(const ExecArgs& a, const MItem& it, const MOE_LDS int* rows,
                        const void* codes, const int32_t* exps) {
  using RB = typename RowA8::Base;
  int o[RB::NI];
#pragma unroll
  for (int i = 0; i < RB::NI; ++i) {
    const int row = RB::lane_row(i);
    o[i] = row < it.nrows ? (int)token_of((uint32_t)rows[row], a.kmagic) * (a.d / 2) : -1;
  }
  RowA8 x;
  x.init_offsets((const uint16_t*)codes, (uint32_t)((size_t)a.T * a.d), o);
  const int w = wave_id(), row = w * 64 + (threadIdx.x & 63);
  x.rsc = make_rsrc(exps, (uint32_t)((size_t)(a.d / 128) * a.T * 4));
  x.scs = (uint32_t)a.T * 4u;
  x.sco = (w < 4 && row < it.nrows) ? token_of((uint32_t)rows[row], a.kmagic) * 4u : kOob;
  return x;
}
// The tile's slot rows of quantized codes [slots][ld] and exponents
// [ld / 128][slots].
MOE_DEV RowA8 slotrows8(const ExecArgs& a, const MItem& it, const void* codes,
                        const int32_t* exps, int ld) {
  RowA8 x;
  x.init((const uint16_t*)codes, (uint32_t)((size_t)a.slots * ld),
         [&](int row) { return row < it.nrows ? (it.slot0 + row) * (ld / 2) : -1; });
  const int w = wave_id(), row = w * 64 + (threadIdx.x & 63);
  x.rsc = make_rsrc(exps, (uint32_t)((size_t)(ld / 128) * a.slots * 4));
  x.scs = (uint32_t)a.slots * 4u;
  x.sco = (w < 4 && row < it.nrows) ? (uint32_t)(it.slot0 + row) * 4u : kOob;
  return x;
}

struct SrcFc1F8 : SrcFc1T<true> {
  using OB = RowW8;
  MOE_DEV RowA8 opA(const Item& it, int slot) const {
    return gathered8(a, it, item_rows(smem, slot), a.xq, a.xe);
  }
  MOE_DEV RowW8 opB(const Item& it, int) const {
    RowW8 w;
    const int dff = a.dff, nj = it.nj;
    auto row = [&](int rho) {           // element offsets of code pairs: row * d / 2
      const int q = rho >> 5;
      return ((q & 1) * dff + nj * (WC::BN / 2) + (q >> 1) * 32 + (rho & 31)) * (a.d / 2);
    };
    w.init((const uint16_t*)((const uint8_t*)a.w1 + (size_t)it.e * 2 * dff * a.d),
           (uint32_t)((size_t)2 * dff * a.d), row);
    const int kb = a.d / 128;
    const MOE_CONST float* sc = (const MOE_CONST float*)a.w1s + (size_t)it.e * (2 * dff / 128) * kb;
    w.sp[0] = sc + (size_t)nj * kb;
    w.sp[1] = sc + (size_t)(dff / 128 + nj) * kb;
    return w;
  }
  MOE_DEV int steps(const Item&) const { return a.d / 128; }
};

// FC2 with the gate: O[slot] = p * A W2^T.  With e4m3 weights a wave's 64
// rows nj * 256 + 64 wn .. +63 lie in scale block 2 nj + wn / 2.
template <bool FP8> struct SrcFc2T : MSrcBase {
  static constexpr bool kSkipIdle = true;
  using Item = MItem;
  using OB = typename std::conditional<FP8, RowF8, RowW>::type;
  MOE_DEV void fill(const Item& it, int slot) const { fill_gates(it, slot); }
  MOE_DEV RowW opA(const Item& it, int) const { return slotrows(it, a.bufA, a.dff); }
  MOE_DEV OB opB(const Item& it, int) const {
    OB w;
    const int nj = it.nj, dff = a.dff;
    auto row = [&](int rho) { return (nj * WC::BN + rho) * dff; };
    if constexpr (FP8) {
      w.init((const uint8_t*)a.w2 + (size_t)it.e * a.d * dff, (uint32_t)((size_t)a.d * dff), row);
      const int kb = dff / 128;
      const int wn = wave_id() % WC::WAVES_N;
      w.sp[0] = w.sp[1] = (const MOE_CONST float*)a.w2s + (size_t)it.e * (a.d / 128) * kb +
                          (size_t)(2 * nj + wn / 2) * kb;
    } else {
      w.init((const uint16_t*)a.w2 + (size_t)it.e * a.d * dff, (uint32_t)((size_t)2 * a.d * dff), row);
    }
    return w;
  }
  MOE_DEV int steps(const Item&) const { return a.dff / kRowBK; }
  static constexpr int kEpiVm = WC::MB * RowStore<uint16_t, 2>::STORES;
  template <int B> MOE_DEV void relaxed_wait() const { wait_vm_lgkm0<vm_clamp(B + kEpiVm)>(); }
  MOE_DEV void epilogue(const Item& it, int slot, const f32x16_t (&acc)[WC::MB][WC::NB]) const {
    const int lane = threadIdx.x & 63, wm = wave_id() / WC::WAVES_N, wn = wave_id() % WC::WAVES_N;
    const MOE_LDS float* gt = item_gates(smem, slot);
    const BufRsrc ro = make_rsrc(a.bufO, (uint32_t)(a.slots * a.d * 2));
    const int colb = it.nj * WC::BN + wn * WC::WN;
    MOE_LDS char* scr = epi_scratch(smem);
#pragma unroll
    for (int i = 0; i < WC::MB; ++i) {
      const int rb = wm * WC::WM + i * 32;
      const float pg = gt[rb + (lane & 31)];
      RowStore<uint16_t, 2>::run(scr, [&](int jj, int g, float* v) {
        for (int q = 0; q < 4; ++q) v[q] = pg * acc[i][jj][4 * g + q];
      }, [&](int row, int c, const u32x4_t& d) {
        st_row16(ro, it.slot0 + rb + row, a.d, colb + c * 8, rb + row < it.nrows, d);
      });
    }
  }
};

// FC2 on the fp8 MFMA: A rows are the e4m3 codes SrcFc1F8 wrote (slot rows of
// hq, exponents in he), B rows W2's codes; K steps of 128 over d_ff.  The
// epilogue (gate, O rows) is FC2's.
struct SrcFc2F8 : SrcFc2T<true> {
  using OB = RowW8;
  MOE_DEV RowA8 opA(const Item& it, int) const { return slotrows8(a, it, a.hq, a.he, a.dff); }
  MOE_DEV RowW8 opB(const Item& it, int) const {
    RowW8 w;
    const int nj = it.nj, dff = a.dff;
    w.init((const uint16_t*)((const uint8_t*)a.w2 + (size_t)it.e * a.d * dff),
           (uint32_t)((size_t)a.d * dff), [&](int rho) { return (nj * WC::BN + rho) * (dff / 2); });
    const int kb = dff / 128, wn = wave_id() % WC::WAVES_N;
    w.sp[0] = w.sp[1] = (const MOE_CONST float*)a.w2s + (size_t)it.e * (a.d / 128) * kb +
                        (size_t)(2 * nj + wn / 2) * kb;
    return w;
  }
  MOE_DEV int steps(const Item&) const { return a.dff / 128; }
};

// dA = p * dy W2 (W2 [d][d_ff] read K-major through transpose reads), then
// dZ = [dA U s (1 + G (1 - s)), dA G s] with s = sigmoid(G), and the gated
// activation P = p SiLU(G) U for the weight gradient of W2.  With e4m3
// weights the weight gradient of W2 takes the requantized D = p dy instead,
// so P is written without the gate.
// COH: dZ is stored with device-scope completion, read by dX items of the
// same launch.
template <bool FP8, bool COH = false> struct SrcDaT : MSrcBase {
  using Item = MItem;
  using OB = typename std::conditional<FP8, MnF8Op, MnFixedOp>::type;
  MOE_DEV void fill(const Item& it, int slot) const { fill_rows(it, slot); fill_gates(it, slot); }
  MOE_DEV RowW opA(const Item& it, int slot) const { return gathered(it, slot, a.dy, a.d); }
  MOE_DEV OB opB(const Item& it, int) const {
    if constexpr (FP8) {   // W2 [d][d_ff] codes; scale block (kt / 2, 2 nj + wn / 2)
      MnF8 m;
      m.rs = make_rsrc((const uint8_t*)a.w2 + (size_t)it.e * a.d * a.dff, (uint32_t)((size_t)a.d * a.dff));
      const int wn = wave_id() % WC::WAVES_N;
      m.sp = (const MOE_CONST float*)a.w2s + (size_t)it.e * (a.d / 128) * (a.dff / 128) +
             (2 * it.nj + wn / 2);
      m.sld = a.dff / 128;
      return {m, MnFixed{(uint32_t)a.dff, (uint32_t)it.nj * WC::BN}};
    } else {
      const MnW m{make_rsrc((const uint16_t*)a.w2 + (size_t)it.e * a.d * a.dff,
                            (uint32_t)((size_t)2 * a.d * a.dff))};
      return {m, MnFixed{(uint32_t)a.dff * 2u, (uint32_t)it.nj * WC::BN * 2u}};
    }
  }
  MOE_DEV int steps(const Item&) const { return a.d / kRowBK; }
  // per 32 x 32 block: 8 [G, U] loads and three row-store runs
  static constexpr int kEpiVm = WC::MB * WC::NB * (8 + 3 * RowStore<uint16_t, 1>::STORES);
  template <int B> MOE_DEV void relaxed_wait() const { wait_vm_lgkm0<vm_clamp(B + kEpiVm)>(); }
  MOE_DEV void epilogue(const Item& it, int slot, const f32x16_t (&acc)[WC::MB][WC::NB]) const {
    constexpr int NBLK = WC::MB * WC::NB;
    const int lane = threadIdx.x & 63, wm = wave_id() / WC::WAVES_N, wn = wave_id() % WC::WAVES_N;
    const MOE_LDS float* gt = item_gates(smem, slot);
    const uint16_t* Z = (const uint16_t*)a.z_save;
    const int dff = a.dff, colb = it.nj * WC::BN + wn * WC::WN;
    const BufRsrc rdz = make_rsrc(a.bufA, (uint32_t)(a.slots * dff * 4));
    const BufRsrc rp = make_rsrc(a.bufP, (uint32_t)(a.slots * dff * 2));
    MOE_LDS char* scr = epi_scratch(smem);
    // Block b = (i, j) of 32 x 32.  The lane's [G, U] of block b + 1 go into
    // the other register set while block b is formed, so their round trip runs
    // under block b's passes and stores: from block 1 on they are issued when
    // block b starts; block 1's wait until block 0's accumulators are spent
    // (after its second pass), which keeps the peak register count where a
    // single set puts it.  dG, dU and P leave through the per-wave scratch as
    // 64-byte row pieces.
    u32x2_t zg2[2][4], zu2[2][4];
    auto zload = [&](int b, u32x2_t (&g_)[4], u32x2_t (&u_)[4]) {
      const int i = b / WC::NB, j = b % WC::NB;
      const int myrow = wm * WC::WM + i * 32 + (lane & 31);
      const size_t sr = (size_t)it.slot0 + (myrow < it.nrows ? myrow : 0);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = colb + j * 32 + 8 * g + 4 * (lane >> 5);
        g_[g] = *(const MOE_GLB u32x2_t*)(Z + sr * 2 * dff + n);
        u_[g] = *(const MOE_GLB u32x2_t*)(Z + sr * 2 * dff + dff + n);
      }
    };
    zload(0, zg2[0], zu2[0]);
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const int i = b / WC::NB, j = b % WC::NB;
      if (b >= 1 && b + 1 < NBLK) zload(b + 1, zg2[(b + 1) & 1], zu2[(b + 1) & 1]);
      const u32x2_t(&zg)[4] = zg2[b & 1];
      const u32x2_t(&zu)[4] = zu2[b & 1];
      const int rb = wm * WC::WM + i * 32, cb = colb + j * 32;
      const float pg = gt[rb + (lane & 31)];
      using RS = RowStore<uint16_t, 1>;
      auto emit_to = [&](const BufRsrc& r, int col0, int ld, auto cp) {
        return [&, col0, ld](int row, int c, const u32x4_t& d) {
          st_row16<decltype(cp)::value>(r, it.slot0 + rb + row, ld, col0 + cb + c * 8,
                                        rb + row < it.nrows, d);
        };
      };
      using CpZ = std::integral_constant<int, COH ? kStoreDevice : kStoreLocal>;
      using CpP = std::integral_constant<int, kStoreLocal>;
      // one output per pass, 8 packed registers at a time; the sigmoid is
      // taken again in each pass (the empty asm keeps the passes apart, so
      // the compiler does not hold 32 sigmoids across them)
      auto pass = [&](int which, RS::Packed (&p)[1][4]) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t wg = q < 2 ? zg[g].x : zg[g].y, wu = q < 2 ? zu[g].x : zu[g].y;
            float gv = bf2f((uint16_t)((q & 1) ? wg >> 16 : wg & 0xffff));
            asm volatile("" : "+v"(gv));
            const float uv = bf2f((uint16_t)((q & 1) ? wu >> 16 : wu & 0xffff));
            const float sg = sigm(gv);
            if (which == 0) v[q] = pg * acc[i][j][4 * g + q] * uv * sg * (1.f + gv * (1.f - sg));
            else if (which == 1) v[q] = pg * acc[i][j][4 * g + q] * gv * sg;
            else v[q] = (FP8 ? 1.f : pg) * (gv * sg * uv);
          }
          p[0][g] = u32x2_t{(uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16),
                            (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16)};
        }
      };
      RS::Packed pk[1][4];
      pass(0, pk);
      RS::store(scr, pk, emit_to(rdz, 0, 2 * dff, CpZ{}));
      pass(1, pk);
      if (b == 0 && NBLK > 1) zload(1, zg2[1], zu2[1]);
      RS::store(scr, pk, emit_to(rdz, dff, 2 * dff, CpZ{}));
      pass(2, pk);
      RS::store(scr, pk, emit_to(rp, 0, dff, CpP{}));
    }
  }
};

// dX per routed row: dZ W1 (W1 [2 d_ff][d] read K-major through transpose reads).
template <bool FP8> struct SrcDxT : MSrcBase {
  static constexpr bool kSkipIdle = true;
  using Item = MItem;
  using OB = typename std::conditional<FP8, MnF8Op, MnFixedOp>::type;
  MOE_DEV void fill(const Item&, int) const {}
  MOE_DEV RowW opA(const Item& it, int) const { return slotrows(it, a.bufA, 2 * a.dff); }
  MOE_DEV OB opB(const Item& it, int) const {
    if constexpr (FP8) {   // W1 [2 d_ff][d] codes; scale block (kt / 2, 2 nj + wn / 2)
      MnF8 m;
      m.rs = make_rsrc((const uint8_t*)a.w1 + (size_t)it.e * 2 * a.dff * a.d,
                       (uint32_t)((size_t)2 * a.dff * a.d));
      const int wn = wave_id() % WC::WAVES_N;
      m.sp = (const MOE_CONST float*)a.w1s + (size_t)it.e * (2 * a.dff / 128) * (a.d / 128) +
             (2 * it.nj + wn / 2);
      m.sld = a.d / 128;
      return {m, MnFixed{(uint32_t)a.d, (uint32_t)it.nj * WC::BN}};
    } else {
      const MnW m{make_rsrc((const uint16_t*)a.w1 + (size_t)it.e * 2 * a.dff * a.d,
                            (uint32_t)((size_t)4 * a.dff * a.d))};
      return {m, MnFixed{(uint32_t)a.d * 2u, (uint32_t)it.nj * WC::BN * 2u}};
    }
  }
  MOE_DEV int steps(const Item&) const { return 2 * a.dff / kRowBK; }
  static constexpr int kEpiVm = WC::MB * RowStore<uint16_t, 2>::STORES;
  template <int B> MOE_DEV void relaxed_wait() const { wait_vm_lgkm0<vm_clamp(B + kEpiVm)>(); }
  MOE_DEV void epilogue(const Item& it, int, const f32x16_t (&acc)[WC::MB][WC::NB]) const {
    const int wm = wave_id() / WC::WAVES_N, wn = wave_id() % WC::WAVES_N;
    const BufRsrc ro = make_rsrc(a.bufO, (uint32_t)(a.slots * a.d * 2));
    const int colb = it.nj * WC::BN + wn * WC::WN;
    MOE_LDS char* scr = epi_scratch(smem);
#pragma unroll
    for (int i = 0; i < WC::MB; ++i) {
      const int rb = wm * WC::WM + i * 32;
      RowStore<uint16_t, 2>::run(scr, [&](int jj, int g, float* v) {
        for (int q = 0; q < 4; ++q) v[q] = acc[i][jj][4 * g + q];
      }, [&](int row, int c, const u32x4_t& d) {
        st_row16(ro, it.slot0 + rb + row, a.d, colb + c * 8, rb + row < it.nrows, d);
      });
    }
  }
};

// dA and dX on the fp8 MFMA (MOE_EXEC_FP8_ACT): the A rows are dy's token
// rows (dA) or the bf16 dZ slot rows (dX) quantized per row and 128 features
// with power-of-two scales (k_quant_act into xq / xe and hq / he), the B
// operand the weights' codes read K-major into the fp8 MFMA's layout, a K step
// of 128 codes; the epilogues are dA's and dX's.
using MnK8W = MnK8<256, kWNW>;
using MnK8Op = MnKOperand<MnK8W, MnFixed>;
struct SrcDaF8 : SrcDaT<true> {
  using OB = MnK8Op;
  MOE_DEV RowA8 opA(const Item& it, int slot) const {
    return gathered8(a, it, item_rows(smem, slot), a.xq, a.xe);
  }
  MOE_DEV MnK8Op opB(const Item& it, int) const {   // W2 [d][d_ff] codes; block (kt, 2 nj + wn / 2)
    MnK8W m;
    m.rs = make_rsrc((const uint8_t*)a.w2 + (size_t)it.e * a.d * a.dff, (uint32_t)((size_t)a.d * a.dff));
    const int wn = wave_id() % WC::WAVES_N;
    m.sp = (const MOE_CONST float*)a.w2s + (size_t)it.e * (a.d / 128) * (a.dff / 128) +
           (2 * it.nj + wn / 2);
    m.sld = a.dff / 128;
    return {m, MnFixed{(uint32_t)a.dff, (uint32_t)it.nj * WC::BN}};
  }
  MOE_DEV int steps(const Item&) const { return a.d / 128; }
  // p dA rows as bf16 into bufO [slots][d_ff]; dZ and P follow in
  // k_swiglu_bwd_q (forming them here, with the [G, U] loads, takes the
  // kernel past 256 VGPRs and spills inside its K loop)
  static constexpr int kEpiVm = WC::MB * RowStore<uint16_t, 2>::STORES;
  template <int B> MOE_DEV void relaxed_wait() const { wait_vm_lgkm0<vm_clamp(B + kEpiVm)>(); }
  MOE_DEV void epilogue(const Item& it, int slot, const f32x16_t (&acc)[WC::MB][WC::NB]) const {
    const int lane = threadIdx.x & 63, wm = wave_id() / WC::WAVES_N, wn = wave_id() % WC::WAVES_N;
    const MOE_LDS float* gt = item_gates(smem, slot);
    const BufRsrc ro = make_rsrc(a.bufO, (uint32_t)(a.slots * a.dff * 2));
    const int colb = it.nj * WC::BN + wn * WC::WN;
    MOE_LDS char* scr = epi_scratch(smem);
#pragma unroll
    for (int i = 0; i < WC::MB; ++i) {
      const int rb = wm * WC::WM + i * 32;
      const float pg = gt[rb + (lane & 31)];
      RowStore<uint16_t, 2>::run(scr, [&](int jj, int g, float* v) {
        for (int q = 0; q < 4; ++q) v[q] = pg * acc[i][jj][4 * g + q];
      }, [&](int row, int c, const u32x4_t& d) {
        st_row16(ro, it.slot0 + rb + row, a.dff, colb + c * 8, rb + row < it.nrows, d);
      });
    }
  }
};
struct SrcDxF8 : SrcDxT<true> {
  using OB = MnK8Op;
  MOE_DEV RowA8 opA(const Item& it, int) const { return slotrows8(a, it, a.hq, a.he, 2 * a.dff); }
  MOE_DEV MnK8Op opB(const Item& it, int) const {   // W1 [2 d_ff][d] codes; block (kt, 2 nj + wn / 2)
    MnK8W m;
    m.rs = make_rsrc((const uint8_t*)a.w1 + (size_t)it.e * 2 * a.dff * a.d,
                     (uint32_t)((size_t)2 * a.dff * a.d));
    const int wn = wave_id() % WC::WAVES_N;
    m.sp = (const MOE_CONST float*)a.w1s + (size_t)it.e * (2 * a.dff / 128) * (a.d / 128) +
           (2 * it.nj + wn / 2);
    m.sld = a.d / 128;
    return {m, MnFixed{(uint32_t)a.d, (uint32_t)it.nj * WC::BN}};
  }
  MOE_DEV int steps(const Item&) const { return 2 * a.dff / 128; }
};

// Two GEMM phases in one persistent launch (MegaFlux summary, Methodology
// section 2, "Executor: Pipelined Expert Replication — Forward": the second
// product of a block needs only the completed activation block of the first).
// P1 produces rows that P2 consumes: FC1 -> A -> FC2, or dA -> dZ -> dX.  Each
// workgroup first streams its share of the worker's P1 items (row tile m, N
// tile j), then its share of the P2 items, as two passes of the stream engine
// in one kernel.  Each finished P1 item adds one to flags[worker][m] once its
// stores are complete (at the next step's full wait, or at the end of the
// pass); a P2 item of row tile m issues its first loads only once that
// counter holds P1's N-tile count.  The rows P1 writes for P2 are stored with
// device-scope completion, and no workgroup reads them before their counter
// is complete, so no cache level holds an older copy when they are read (each
// launch starts with clean caches).  The workgroups of one launch are all
// resident (one per CU, grid = CU count) and a P2 wait depends only on P1
// items, which never wait.  A wait that outlasts kFlowWaitTicks (2 s) sets
// MOE_DEV_WAIT_TIMEOUT and goes on.
struct PItem : MItem { int m; };
constexpr uint64_t kFlowWaitTicks = 200000000ull;   // the 100 MHz real-time counter
template <class Src> struct FlowBase : Src {
  static constexpr bool kFlow = true;
  // the idle-wave branches push the merged kernels over the register file
  static constexpr bool kSkipIdle = false;
  using Item = PItem;
  MOE_DEV Item load(int idx) const {
    const int m = idx / this->nnt;
    const u32x4_t d = ((const MOE_CONST u32x4_t*)this->a.mt)[(size_t)this->r * this->a.max_mt + m];
    Item it;
    it.e = (int)d.x;
    it.slot0 = (int)d.y;
    it.nrows = (int)d.z;
    it.nj = idx - m * this->nnt;
    it.m = m;
    return it;
  }
  MOE_DEV int32_t* flag(int m) const {
    return this->a.flags + (size_t)this->r * this->a.max_mt + m;
  }
};
// first phase: publishes each finished row-tile item
template <class P1> struct FlowProducer : FlowBase<P1> {
  MOE_DEV int peek(const PItem&) const { return -1; }
  MOE_DEV void ready(const PItem&, int) const {}
  MOE_DEV int publish_key(const PItem& it) const { return it.m; }
  MOE_DEV void signal(int m) const {
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(this->flag(m), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
};
// second phase: waits for the n1 first-phase items of its row tile
template <class P2> struct FlowConsumer : FlowBase<P2> {
  int n1;
  MOE_DEV int publish_key(const PItem&) const { return -1; }
  MOE_DEV void signal(int) const {}
  MOE_DEV int peek(const PItem& it) const {
    return __hip_atomic_load(this->flag(it.m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the counter only grows: a complete value seen earlier stays complete
  MOE_DEV void ready(const PItem& it, int seen) const {
    if (__builtin_amdgcn_readfirstlane(seen) >= n1) return;
    int32_t* f = this->flag(it.m);
    auto done = [&]() {
      return __builtin_amdgcn_readfirstlane(
                 __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) >= n1;
    };
    if (done()) return;
    const uint64_t t_end = __builtin_amdgcn_s_memrealtime() + kFlowWaitTicks;
    while (true) {
      __builtin_amdgcn_s_sleep(8);
      if (done()) return;
      if (__builtin_amdgcn_s_memrealtime() > t_end) {
        if ((threadIdx.x & 63) == 0) atomicOr(this->a.status, MOE_DEV_WAIT_TIMEOUT);
        return;
      }
    }
  }
};

// One persistent workgroup per CU for the 256 x 256 tile (8 waves), two per
// CU for the 128 x 128 tile (4 waves): either way two waves per SIMD.
template <class Src, class C, class OA, class OB>
__global__ __launch_bounds__(C::NT, 512 / C::NT) void k_stream(ExecArgs a, int ntiles_n) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  MOE_LDS uint16_t* smem = (MOE_LDS uint16_t*)smem_raw;
  // optional timeline: the constant 100 MHz real-time counter when the
  // workgroup starts and once its last item is done (run() ends with a wait
  // for every memory operation and a barrier), written with vector stores
  const uint64_t t0 = a.timeline ? __builtin_amdgcn_s_memrealtime() : 0;
  Src src;
  src.init(a, smem, ntiles_n);
  f32x16_t acc[C::MB][C::NB];
  WideStream<C, OA, OB, src_rows_in_regs<Src>::value> p;
  p.run(src, smem, acc);
  if (a.timeline) {
    __syncthreads();
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0 && blockIdx.x < MOE_TIMELINE_MAX_WG) {
      MOE_GLB uint64_t* out =
          (MOE_GLB uint64_t*)a.timeline + ((size_t)a.tl_phase * MOE_TIMELINE_MAX_WG + blockIdx.x) * 2;
      out[0] = t0;
      out[1] = t1;
    }
  }
}

// The two-phase launch: the P1 pass, then the P2 pass (FlowProducer /
// FlowConsumer above).  ntiles: P1's N tiles in the low 16 bits, P2's above.
// split = 0: every workgroup runs both passes, its P1 items first.  split =
// n1 > 0 (a CTA split, "Analytical Resource Management for Fine-grained MoE
// Computation-Communication Overlap", abstract: the producer-CTA count of a
// dependency-coupled pipeline): workgroups j < n1 of each worker are
// producers and deal the worker's P1 items among themselves; the other n - n1
// are consumers and deal its P2 items.  Producers never wait, and every
// workgroup of the persistent grid is resident, so the consumers' waits end.
// The timeline gets both phases: P1 from the start to the end of the first
// pass, P2 from there to the end.
template <class S1, class S2, class C, class OA, class OB>
__global__ __launch_bounds__(C::NT, 512 / C::NT) void k_stream2(ExecArgs a, int ntiles, int split) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  MOE_LDS uint16_t* smem = (MOE_LDS uint16_t*)smem_raw;
  const uint64_t t0 = a.timeline ? __builtin_amdgcn_s_memrealtime() : 0;
  const int n1 = ntiles & 0xffff, n2 = ntiles >> 16;
  const WorkerSlot w = worker_slot(a.P);
  if (split >= w.n) split = 0;                   // the host admits 0 <= split < n only
  const bool producer = split == 0 || w.j < split;
  const bool consumer = split == 0 || w.j >= split;
  f32x16_t acc[C::MB][C::NB];
  WideStream<C, OA, OB> p;
  {
    S1 src;
    src.init(a, smem, n1);
    if (split > 0) src.stride = split;             // first = w.j < split
    if (producer) p.run(src, smem, acc);
  }
  const uint64_t tm = a.timeline ? __builtin_amdgcn_s_memrealtime() : 0;
  {
    S2 src;
    src.init(a, smem, n2);
    src.n1 = n1;
    if (split > 0) {
      src.first = w.j - split;
      src.stride = w.n - split;
    }
    if (consumer) p.run(src, smem, acc);
  }
  if (a.timeline) {
    __syncthreads();
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0 && blockIdx.x < MOE_TIMELINE_MAX_WG) {
      MOE_GLB uint64_t* out =
          (MOE_GLB uint64_t*)a.timeline + ((size_t)a.tl_phase * MOE_TIMELINE_MAX_WG + blockIdx.x) * 2;
      out[0] = t0;
      out[1] = tm;
      out[2 * MOE_TIMELINE_MAX_WG] = tm;
      out[2 * MOE_TIMELINE_MAX_WG + 1] = t1;
    }
  }
}
template <bool FP8> using FwdP1 = FlowProducer<SrcFc1T<FP8, true>>;
template <bool FP8> using FwdP2 = FlowConsumer<SrcFc2T<FP8>>;
template <bool FP8> using BwdP1 = FlowProducer<SrcDaT<FP8, true>>;
template <bool FP8> using BwdP2 = FlowConsumer<SrcDxT<FP8>>;

// ---- backward: weight gradients per (expert, worker) segment ------------------
// K runs over the segment's routed rows.  dW2[c, n] = sum D[c] * A[n] with
// D = dy_t (gathered) and the gate folded into A = p * SiLU(G) * U, rebuilt
// from the saved [G, U]; dW1[j, c] = sum dZ[j] * x_t[c].
template <typename T> struct SrcGatherRow {    // element (k, m) = base[t(slot0 + k) * ld + m0 + m]
  const T* base;
  const int32_t* slot_to_row;
  int slot0, nrows, topk, ld, m0, mlim;
  MOE_DEV uint4 operator()(int kk, int mn) const {
    const int m = m0 + mn;
    if (kk >= nrows || m >= mlim) return zero4();
    const int t = slot_to_row[slot0 + kk] / topk;
    return ldg16(base + (size_t)t * ld + m);
  }
};
template <typename T> struct SrcSlotRow {      // element (k, m) = base[(slot0 + k) * ld + m0 + m]
  const T* base;
  int slot0, nrows, ld, m0, mlim;
  MOE_DEV uint4 operator()(int kk, int mn) const {
    const int m = m0 + mn;
    if (kk >= nrows || m >= mlim) return zero4();
    return ldg16(base + ((size_t)slot0 + kk) * ld + m);
  }
};
template <typename T> struct SrcGatedAct {     // element (k, n) = p * SiLU(G) * U at slot0 + k
  const T* z;
  const float* gates;
  const int32_t* slot_to_row;
  int slot0, nrows, dff, n0;
  MOE_DEV uint4 operator()(int kk, int mn) const {
    constexpr int VE = Elem<T>::VE;
    const int n = n0 + mn;
    if (kk >= nrows || n >= dff) return zero4();
    const size_t zb = ((size_t)slot0 + kk) * 2 * dff;
    const float p = gates ? gates[slot_to_row[slot0 + kk]] : 1.f;   // no gates: A itself
    V16 g, u, o;
    g.u = ldg16(z + zb + n);
    u.u = ldg16(z + zb + dff + n);
#pragma unroll
    for (int v = 0; v < VE; ++v) {
      float gv, uv;
      if constexpr (sizeof(T) == 2) { gv = bf2f(g.h[v]); uv = bf2f(u.h[v]); }
      else { gv = g.f[v]; uv = u.f[v]; }
      const float av = p * (gv / (1.f + expf(-gv)) * uv);
      if constexpr (sizeof(T) == 2) o.h[v] = f2bf(av);
      else o.f[v] = av;
    }
    return o.u;
  }
};

template <typename T, class C, bool FP8 = false>
__global__ __launch_bounds__(C::NT) void k_bwd_dw(ExecArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int tslot;
  MOE_LDS T* smem = (MOE_LDS T*)smem_raw;
  const int r = worker_of_block(a.P);
  const int n2m = a.d / C::BM, n2n = (a.dff + C::BN - 1) / C::BN;   // dW2 [d][dff]
  const int n1m = 2 * a.dff / C::BM, n1n = a.d / C::BN;            // dW1 [2dff][d]
  const int per_seg = n2m * n2n + n1m * n1n;
  const int total = a.seg_cnt[r] * per_seg;
  const int lane = threadIdx.x & 63;
  const size_t w_elems = (size_t)3 * a.d * a.dff;
  while (true) {
    const int tile = next_tile(&a.ctr[PH_DW * kMaxP + r], &tslot);
    if (tile >= total) break;
    const int4 sg = a.seg[(size_t)r * a.E + tile / per_seg];
    const int e = sg.x, slot0 = sg.y, nrows = sg.z, dst = sg.w;
    if (e < 0) continue;
    int loc = tile % per_seg;
    const int nk = (nrows + Elem<T>::BK - 1) / Elem<T>::BK;
    f32x16_t acc[C::MB][C::NB];
    TransLoad<T, C::BM, C::NT> la;
    TransLoad<T, C::BN, C::NT> lb;
    la.init();
    lb.init();
    float* out;
    int ldo, mi, nj, nlim;
    if (loc < n2m * n2n) {
      mi = loc / n2n;
      nj = loc % n2n;
      if constexpr (FP8) {   // dW2 = Dq^T A: token-axis e4m3 D, ungated A
        SrcSlotRowFp8 sa{a.dq, a.dqs, slot0, nrows, a.d, mi * C::BM, a.d, a.beta};
        SrcGatedAct<T> sb{(const T*)a.z_save, nullptr, a.slot_to_row, slot0, nrows, a.dff,
                          nj * C::BN};
        gemm_tile<T, C>(TransLd<decltype(la), SrcSlotRowFp8>{la, sa},
                        TransLd<decltype(lb), SrcGatedAct<T>>{lb, sb}, nk, smem, acc);
      } else {
        SrcGatherRow<T> sa{(const T*)a.dy, a.slot_to_row, slot0, nrows, a.k, a.d, mi * C::BM, a.d};
        SrcGatedAct<T> sb{(const T*)a.z_save, a.gates, a.slot_to_row, slot0, nrows, a.dff,
                          nj * C::BN};
        gemm_tile<T, C>(TransLd<decltype(la), SrcGatherRow<T>>{la, sa},
                        TransLd<decltype(lb), SrcGatedAct<T>>{lb, sb}, nk, smem, acc);
      }
      out = (dst < 0 ? a.dw2 + (size_t)e * a.d * a.dff
                     : a.rslots + (size_t)dst * w_elems + (size_t)2 * a.dff * a.d);
      ldo = a.dff;
      nlim = a.dff;
    } else {
      loc -= n2m * n2n;
      mi = loc / n1n;
      nj = loc % n1n;
      SrcGatherRow<T> sb{(const T*)a.x, a.slot_to_row, slot0, nrows, a.k, a.d, nj * C::BN, a.d};
      if constexpr (FP8) {   // dW1 = dZq^T X: token-axis e4m3 dZ
        SrcSlotRowFp8 sa{a.zq, a.zqs, slot0, nrows, 2 * a.dff, mi * C::BM, 2 * a.dff, a.beta};
        gemm_tile<T, C>(TransLd<decltype(la), SrcSlotRowFp8>{la, sa},
                        TransLd<decltype(lb), SrcGatherRow<T>>{lb, sb}, nk, smem, acc);
      } else {
        SrcSlotRow<T> sa{(const T*)a.bufA, slot0, nrows, 2 * a.dff, mi * C::BM, 2 * a.dff};
        gemm_tile<T, C>(TransLd<decltype(la), SrcSlotRow<T>>{la, sa},
                        TransLd<decltype(lb), SrcGatherRow<T>>{lb, sb}, nk, smem, acc);
      }
      out = (dst < 0 ? a.dw1 + (size_t)e * 2 * a.dff * a.d : a.rslots + (size_t)dst * w_elems);
      ldo = a.d;
      nlim = a.d;
    }
    constexpr int PASS = 128, LDD = C::BN + 4;
    MOE_LDS float* sd = (MOE_LDS float*)smem;
    for (int p0 = 0; p0 < C::BM; p0 += PASS) {
      if (p0) __syncthreads();
      acc_to_lds<C>(acc, sd, LDD, p0, PASS, [](float v, int, int) { return v; });
      __syncthreads();
      lds_to_global<float, C::NT>(sd, PASS, C::BN, LDD, [&](int rl, int col, const V16& v) {
        const int n = nj * C::BN + col;
        if (n < nlim) stg16(out + ((size_t)mi * C::BM + p0 + rl) * ldo + n, v.u);
      });
    }
  }
}

// ---- weight gradients on the persistent wide tile --------------------------------
// Items are (segment, output tile): a segment is one (expert, worker) run of
// routed rows, K = its rows.  dW2[c, n] = sum dy_t[c] * P[n] (A: gathered dy
// rows, B: P rows); dW1[j, c] = sum dZ[j] * x_t[c] (A: dZ rows, B: gathered x
// rows).  Every operand is read in its natural [row][feature] layout through
// transpose reads; the token of a gathered row is read from the slot map
// early in the step before its loads are issued; rows past the segment read
// as zeros.  fp32 tiles go straight from registers to the owner slot or a
// replica slot.
struct MnSeg {
  const int32_t* slot_to_row;
  uint32_t kmagic, ld2, col2;
  int s0, nrows, gather;
  // The slot map is read for every row (no branch, so nothing waits on it
  // before the step-end wait) and used only for gathered operands.
  using Raw = uint32_t;
  MOE_DEV Raw pre(int, int k) const { return (uint32_t)slot_to_row[s0 + min(k, nrows - 1)]; }
  MOE_DEV uint32_t post(Raw raw, int k) const {
    const uint32_t row = gather ? token_of(raw, kmagic) : (uint32_t)(s0 + min(k, nrows - 1));
    return k < nrows ? row * ld2 + col2 : kOob;
  }
};
// Weight-gradient tiles: the 256 x 256 wide tile.
using DwCfg = WideCfg;
// K = 64 per stage, two stages.  The slot map of each K row is read with
// vector loads during the step, so a deeper pipeline would have to wait for
// them, and everything issued before them, ahead of the next step's loads.
constexpr int kDwBK = 64;
template <class C> using MnSegOpT = MnKOperand<MnK<C::BN, C::NT / 64, kDwBK>, MnSeg>;
using MnSegOp = MnSegOpT<DwCfg>;
constexpr size_t kDwLds = kStreamLds;

struct DwItem { int e, slot0, nrows, dst, is2, mi, nj; };
// With e4m3 weights (FP8) dW2's left operand is the requantized D, widened
// back to bf16 per slot (dhat), and P holds SiLU(G) U without the gate; dZ
// in bufA has been requantized in place.
template <class C, bool FP8 = false> struct SrcDwT {
  using Item = DwItem;
  static constexpr bool kRowsInRegs = true;      // the epilogue stores from the accumulators
  using MnC = MnK<C::BN, C::NT / 64, kDwBK>;
  static_assert(C::BM == C::BN, "one MN operand type for both sides");
  static_assert(MnC::RPI == 2, "a load instruction covers the K row pair kb, kb + 1");
  ExecArgs a;              // a copy: the fields stay in scalar registers
  MOE_LDS uint16_t* smem;
  int r, n2m, n2n, n1m, n1n, per_seg, count, first, stride;
  BufRsrc r_dy, r_x, r_dz, r_p, r_dh;
  MOE_DEV void init(const ExecArgs& args, MOE_LDS uint16_t* sm, int) {
    a = args;
    smem = sm;
    const WorkerSlot w = worker_slot(args.P);
    r = w.r;
    n2m = args.d / C::BM; n2n = args.dff / C::BN;           // dW2 [d][dff]
    n1m = 2 * args.dff / C::BM; n1n = args.d / C::BN;       // dW1 [2dff][d]
    per_seg = n2m * n2n + n1m * n1n;
    count = args.seg_cnt[r] * per_seg;
    first = w.j;
    stride = w.n;
    const uint32_t bx = (uint32_t)((size_t)args.T * args.d * 2);
    r_dy = make_rsrc(args.dy, bx);
    r_x = make_rsrc(args.x, bx);
    r_dz = make_rsrc(args.bufA, (uint32_t)(args.slots * 4 * args.dff));
    r_p = make_rsrc(args.bufP, (uint32_t)(args.slots * 2 * args.dff));
    if constexpr (FP8) r_dh = make_rsrc(args.dhat, (uint32_t)(args.slots * 2 * args.d));
  }
  MOE_DEV Item load(int idx) const {
    const u32x4_t sg = ((const MOE_CONST u32x4_t*)a.seg)[(size_t)r * a.E + idx / per_seg];
    const int loc = idx % per_seg;
    const int is2 = loc < n2m * n2n;
    const int l1 = loc - n2m * n2n;
    return {(int)sg.x, (int)sg.y, (int)sg.z, (int)sg.w, is2, is2 ? loc / n2n : l1 / n1n,
            is2 ? loc % n2n : l1 % n1n};
  }
  MOE_DEV void fill(const Item&, int) const {}
  MOE_DEV MnSegOpT<C> opA(const Item& it, int) const {
    const MnC m{it.is2 ? (FP8 ? r_dh : r_dy) : r_dz};
    const int ld = it.is2 ? a.d : 2 * a.dff;
    return {m, MnSeg{a.slot_to_row, a.kmagic, (uint32_t)ld * 2u, (uint32_t)it.mi * C::BM * 2u,
                     it.slot0, it.nrows, FP8 ? 0 : it.is2}};
  }
  MOE_DEV MnSegOpT<C> opB(const Item& it, int) const {
    const MnC m{it.is2 ? r_p : r_x};
    const int ld = it.is2 ? a.dff : a.d;
    return {m, MnSeg{a.slot_to_row, a.kmagic, (uint32_t)ld * 2u, (uint32_t)it.nj * C::BN * 2u,
                     it.slot0, it.nrows, !it.is2}};
  }
  MOE_DEV int steps(const Item& it) const {
    return max(wide_stages(kDwBK), (it.nrows + kDwBK - 1) / kDwBK);
  }
  // vector memory operations of one epilogue, per wave: one store per
  // accumulator register.  Above 63 the clamp makes the relaxed wait a no-op,
  // which is still exact: a wave cannot hold more than 63 operations in
  // flight (issue stalls), so by the time its last store issues, every load
  // issued before the epilogue has landed.
  static constexpr int kEpiVm = C::MB * C::NB * 16;
  template <int B> MOE_DEV void relaxed_wait() const { wait_vm_lgkm0<vm_clamp(B + kEpiVm)>(); }
  MOE_DEV void epilogue(const Item& it, int, const f32x16_t (&acc)[C::MB][C::NB]) const {
    const int lane = threadIdx.x & 63;
    const size_t w_elems = (size_t)3 * a.d * a.dff;
    float* out;
    int ldo;
    if (it.is2) {
      out = (it.dst < 0 ? a.dw2 + (size_t)it.e * a.d * a.dff
                        : a.rslots + (size_t)it.dst * w_elems + (size_t)2 * a.dff * a.d);
      ldo = a.dff;
    } else {
      out = (it.dst < 0 ? a.dw1 + (size_t)it.e * 2 * a.dff * a.d : a.rslots + (size_t)it.dst * w_elems);
      ldo = a.d;
    }
    out += (size_t)it.mi * C::BM * ldo + (size_t)it.nj * C::BN;
    const int wm = wave_id() / C::WAVES_N, wn = wave_id() % C::WAVES_N;
    // Straight from the accumulators (kRowsInRegs): register r of a 32 x 32
    // block holds row 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32, so
    // one store instruction writes two full 128-byte row pieces, with no LDS
    // staging.
#pragma unroll
    for (int i = 0; i < C::MB; ++i)
#pragma unroll
      for (int j = 0; j < C::NB; ++j) {
        float* ob = out + (size_t)(wm * C::WM + i * 32 + (lane >> 5) * 4) * ldo + wn * C::WN +
                    j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          stg4v(ob + (size_t)((r >> 2) * 8 + (r & 3)) * ldo, acc[i][j][r]);
      }
  }
};


// Owner slot <- (owner partial or 0) + replica partials in ascending worker
// order, fp32.  Experts with an owner partial and no replica are untouched.
// The per-expert table is staged in LDS once per workgroup.
__global__ __launch_bounds__(256) void k_bwd_reduce(const int32_t* __restrict__ rep_slot,
                                                    const int32_t* __restrict__ owner_has,
                                                    const float* __restrict__ rslots, int E,
                                                    int P, int d, int dff, float* dw1,
                                                    float* dw2) {
  __shared__ int tab[kMaxPlanExperts][kMaxP];
  __shared__ int own[kMaxPlanExperts];
  __shared__ int work[kMaxPlanExperts];
  __shared__ int nwork;
  if (threadIdx.x == 0) nwork = 0;
  for (int i = threadIdx.x; i < E * P; i += 256) tab[i / P][i % P] = rep_slot[i];
  for (int e = threadIdx.x; e < E; e += 256) own[e] = owner_has[e];
  __syncthreads();
  // experts with something to do: a replica partial, or no owner partial
  for (int e = threadIdx.x; e < E; e += 256) {
    bool rep = false;
    for (int w = 0; w < P; ++w) rep |= tab[e][w] >= 0;
    if (rep || !own[e]) work[atomicAdd(&nwork, 1)] = e;
  }
  __syncthreads();
  const size_t n1 = (size_t)2 * dff * d, n2 = (size_t)d * dff, w_elems = n1 + n2;
  const size_t nvec = w_elems / 4;
  for (int q0 = 0; q0 < nwork; ++q0) {
    const int e = work[q0];
    int slots[kMaxP];
    int nrep = 0;
#pragma unroll
    for (int w = 0; w < kMaxP; ++w)
      if (w < P && tab[e][w] >= 0) slots[nrep++] = tab[e][w];
    const bool ownp = own[e] != 0;
    for (size_t v = (size_t)blockIdx.x * 256 + threadIdx.x; v < nvec; v += (size_t)gridDim.x * 256) {
      const size_t i = v * 4;
      float* dst = (i < n1) ? dw1 + (size_t)e * n1 + i : dw2 + (size_t)e * n2 + (i - n1);
      float4 accv = ownp ? *(const float4*)dst : make_float4(0.f, 0.f, 0.f, 0.f);
      for (int q = 0; q < nrep; ++q) {
        const float4 p = *(const float4*)(rslots + (size_t)slots[q] * w_elems + i);
        accv.x += p.x; accv.y += p.y; accv.z += p.z; accv.w += p.w;
      }
      *(float4*)dst = accv;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
WsLayout exec_layout(const Sizes& z, bool backward) {
  WsLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align_up(bytes); return at; };
  L.ctr = take(sizeof(int32_t) * kNumCounters);
  L.mt_cnt = take(sizeof(int32_t) * kMaxP);
  L.mt = take(sizeof(int4) * (size_t)z.P * z.max_mt);
  L.seg_cnt = take(sizeof(int32_t) * kMaxP);
  L.seg = take(sizeof(int4) * (size_t)z.P * z.E);
  L.rep_slot = take(sizeof(int32_t) * (size_t)z.E * z.P);
  L.owner_has = take(sizeof(int32_t) * (size_t)z.E);
  L.flags = take(sizeof(int32_t) * (size_t)z.P * z.max_mt);
  L.bufA = take((size_t)z.act_bytes * z.max_slots * (backward ? 2 : 1) * z.dff);
  L.bufO = take((size_t)z.act_bytes * z.max_slots * z.d);
  L.rslots = backward ? take(sizeof(float) * (size_t)z.P * z.s * 3 * z.d * z.dff) : o;
  L.bufP = backward ? take((size_t)z.act_bytes * z.max_slots * z.dff) : o;
  L.sgate = take(sizeof(float) * z.max_slots);
  L.dq = L.dqs = L.zq = L.zqs = L.dhat = L.xq = L.xe = L.hq = L.he = o;
  if (z.fp8 && use_stream(z)) {      // MOE_EXEC_FP8_ACT: x (dy) and A (dZ) as e4m3 rows
    const size_t hc = (size_t)(backward ? 2 : 1) * z.dff;
    L.xq = take((size_t)z.T * z.d);
    L.xe = take(sizeof(int32_t) * (size_t)(z.d / 128) * z.T);
    L.hq = take(z.max_slots * hc);
    L.he = take(sizeof(int32_t) * (hc / 128) * z.max_slots);
  }
  if (backward && z.fp8 && use_stream(z)) {
    L.dhat = take((size_t)2 * z.max_slots * z.d);           // requantized D as bf16
  } else if (backward && z.fp8) {
    const size_t nblk = (z.max_slots + z.beta - 1) / z.beta;
    L.dq = take(z.max_slots * (size_t)z.d);
    L.dqs = take(sizeof(float) * nblk * z.d);
    L.zq = take(z.max_slots * (size_t)2 * z.dff);
    L.zqs = take(sizeof(float) * nblk * 2 * z.dff);
  }
  L.total = o;
  return L;
}

// The big tile needs every M/N extent it touches to be a multiple of 256.
bool use_big_tiles(const Sizes& z) {
  return z.act_bytes == 2 && z.d % 256 == 0 && z.dff % 128 == 0;
}

size_t max_tiles(const Sizes& z) {
  const int bm = use_big_tiles(z) ? BigCfg::BM : SmallCfg::BM;
  const size_t per_block = z.beta > bm ? (size_t)(z.beta + bm - 1) / bm : 1;
  return z.max_blocks * per_block;
}

static int num_cus() {
  static int n = 0;
  if (!n) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

template <typename K> static int persistent_grid(K kernel, int threads, size_t lds) {
  (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds);
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  int g = num_cus() * per_cu;
  g = (g / kXcds) * kXcds;
  return g < kXcds ? kXcds : g;
}

int gemm_wg_per_cu() {
  return persistent_grid(k_fc1<uint16_t, false, BigCfg>, BigCfg::NT,
                         TileLds<uint16_t, BigCfg>::BYTES) / num_cus();
}

static void rec(void* const* ev, int i, hipStream_t st) {
  if (ev && ev[i]) (void)hipEventRecord((hipEvent_t)ev[i], st);
}

static size_t sched_lds(const Sizes& z, bool bwd, bool bwl) {
  return sizeof(int) * ((size_t)2 * z.E + 1 + (bwl ? z.max_blocks : 0) +
                        (bwd ? (size_t)3 * z.E * z.P : 0));
}

// gates (optional, nullptr: none): the per-slot gates the stream kernels read
// (sgate) are written by extra workgroups of the same launch
static void launch_sched(const Sizes& z, const int32_t* counts, const int32_t* boff,
                         const int32_t* bw, const int32_t* owner, bool bwd, char* ws,
                         const WsLayout& L, int32_t* status, const int32_t* slot_to_row,
                         const float* gates, hipStream_t st) {
  SchedArgs s{};
  unsigned gate_wg = 0;
  if (gates && z.max_slots > 0) {
    s.gate_s2r = slot_to_row;
    s.gate_src = gates;
    s.gate_out = (float*)(ws + L.sgate);
    s.gate_n = z.max_slots;
    gate_wg = (unsigned)std::min<size_t>((z.max_slots + kSchedThreads - 1) / kSchedThreads, 2048);
  }
  s.counts = counts; s.boff = boff; s.bw = bw; s.owner = owner;
  s.E = z.E; s.P = z.P; s.s = z.s; s.beta = z.beta; s.backward = bwd ? 1 : 0;
  s.bm = use_big_tiles(z) ? BigCfg::BM : SmallCfg::BM;
  s.ctr = (int32_t*)(ws + L.ctr);
  s.mt_cnt = (int32_t*)(ws + L.mt_cnt);
  s.mt = (int4*)(ws + L.mt);
  s.max_mt = (int)z.max_mt;
  s.seg_cnt = (int32_t*)(ws + L.seg_cnt);
  s.seg = (int4*)(ws + L.seg);
  s.rep_slot = (int32_t*)(ws + L.rep_slot);
  s.owner_has = (int32_t*)(ws + L.owner_has);
  s.flags = (int32_t*)(ws + L.flags);
  s.status = status;
  s.max_blocks = (int)z.max_blocks;
  // block_worker goes through LDS when it fits next to the rest (64 KB)
  const bool bwl = sched_lds(z, true, true) <= 64 * 1024;
  const size_t lds = sched_lds(z, bwd, bwl);
  if (bwl) {
    (void)hipFuncSetAttribute((const void*)k_sched<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)sched_lds(z, true, true));
    hipLaunchKernelGGL(k_sched<true>, dim3(1 + gate_wg), dim3(kSchedThreads), lds, st, s);
  } else {
    (void)hipFuncSetAttribute((const void*)k_sched<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)sched_lds(z, true, false));
    hipLaunchKernelGGL(k_sched<false>, dim3(1 + gate_wg), dim3(kSchedThreads), lds, st, s);
  }
}

static ExecArgs make_exec(const Sizes& z, const LayerPtrs& Lp, char* ws, const WsLayout& L) {
  ExecArgs a{};
  a.w1 = Lp.w1; a.w2 = Lp.w2; a.w1s = Lp.w1s; a.w2s = Lp.w2s;
  a.T = z.T; a.k = z.k; a.E = z.E; a.d = z.d; a.dff = z.dff; a.P = z.P; a.s = z.s; a.beta = z.beta;
  a.mt = (const int4*)(ws + L.mt);
  a.mt_cnt = (const int32_t*)(ws + L.mt_cnt);
  a.max_mt = (int)z.max_mt;
  a.seg = (const int4*)(ws + L.seg);
  a.seg_cnt = (const int32_t*)(ws + L.seg_cnt);
  a.rep_slot = (const int32_t*)(ws + L.rep_slot);
  a.owner_has = (const int32_t*)(ws + L.owner_has);
  a.flags = (int32_t*)(ws + L.flags);
  a.ctr = (int32_t*)(ws + L.ctr);
  a.bufA = ws + L.bufA;
  a.bufO = ws + L.bufO;
  a.rslots = (float*)(ws + L.rslots);
  a.bufP = ws + L.bufP;
  a.slots = z.max_slots;
  a.sgate = (const float*)(ws + L.sgate);
  a.kmagic = (uint32_t)((((uint64_t)1 << 32) + (uint64_t)z.k - 1) / (uint64_t)z.k);
  if (z.fp8) {
    a.xq = ws + L.xq;
    a.xe = (const int32_t*)(ws + L.xe);
    a.hq = ws + L.hq;
    a.he = (int32_t*)(ws + L.he);
    a.dq = (uint8_t*)(ws + L.dq);
    a.dqs = (float*)(ws + L.dqs);
    a.zq = (uint8_t*)(ws + L.zq);
    a.zqs = (float*)(ws + L.zqs);
    a.dhat = ws + L.dhat;
  }
  return a;
}

template <typename T, bool FP8, class C>
static void run_forward(const Sizes& z, ExecArgs& a, const int32_t* row_to_slot, void* y,
                        void* const* ev, hipStream_t st) {
  const size_t lds = gemm_lds_bytes<T, C>();
  static int g1 = persistent_grid(k_fc1<T, FP8, C>, C::NT, lds);
  static int g2 = persistent_grid(k_fc2<T, FP8, C>, C::NT, lds);
  hipLaunchKernelGGL((k_fc1<T, FP8, C>), dim3(g1), dim3(C::NT), lds, st, a);
  rec(ev, 2, st);
  hipLaunchKernelGGL((k_fc2<T, FP8, C>), dim3(g2), dim3(C::NT), lds, st, a);
  rec(ev, 3, st);
  if (z.T > 0)
    hipLaunchKernelGGL(k_combine<T>, combine_grid<T>(z.T, z.d), dim3(256), 0, st,
                       (const T*)a.bufO, row_to_slot, z.T, z.k, z.d, (T*)y);
  rec(ev, 4, st);
}

// The persistent wide-tile kernels: bf16 activations and weights, 256 | d and
// 256 | d_ff (every M/N tile extent), every operand addressed through a
// buffer descriptor below 2 GiB, and token = umulhi(row, ceil(2^32/k)) exact
// for every routed row (row * (ceil(2^32/k) k - 2^32) < 2^32).
bool use_stream(const Sizes& z) {
  const size_t lim = (size_t)1 << 31;
  if (z.act_bytes != 2 || z.d % 256 || z.dff % 256 || z.k <= 0) return false;
  if ((size_t)z.T * z.d * 2 >= lim || z.max_slots * 4 * (size_t)z.dff >= lim ||
      z.max_slots * 2 * (size_t)z.d >= lim || (size_t)4 * z.dff * z.d >= lim || z.max_slots * 4 >= lim)
    return false;
  const uint64_t magic = (((uint64_t)1 << 32) + (uint64_t)z.k - 1) / (uint64_t)z.k;
  const uint64_t err = magic * (uint64_t)z.k - ((uint64_t)1 << 32);
  return (uint64_t)z.T * (uint64_t)z.k * err < ((uint64_t)1 << 32);
}

template <class Src, class C, class OA, class OB>
static void launch_stream(ExecArgs& a, int ntiles_n, size_t lds, hipStream_t st) {
  static int g = persistent_grid(k_stream<Src, C, OA, OB>, C::NT, lds);
  hipLaunchKernelGGL((k_stream<Src, C, OA, OB>), dim3(g), dim3(C::NT), lds, st, a, ntiles_n);
}
// the two-phase launch relies on every workgroup being resident: the grid is
// the persistent one (workgroups per CU that fit x CUs)
template <class S1, class S2, class C, class OA, class OB>
static void launch_stream2(ExecArgs& a, int ntiles, int split, size_t lds, hipStream_t st) {
  static_assert(std::is_same<typename S1::OB, OB>::value && std::is_same<typename S2::OB, OB>::value,
                "one B operand type");
  static int g = persistent_grid(k_stream2<S1, S2, C, OA, OB>, C::NT, lds);
  hipLaunchKernelGGL((k_stream2<S1, S2, C, OA, OB>), dim3(g), dim3(C::NT), lds, st, a, ntiles,
                     split);
}

// workgroups of one worker in the two-phase launches (one per CU)
static int wide_workers_wg(int P) {
  static int g = persistent_grid(k_stream2<FlowProducer<SrcFc1T<false, true>>,
                                           FlowConsumer<SrcFc2T<false>>, WC, RowW, RowW>,
                                 WC::NT, kStreamLds);
  return g / P;
}

// exec_flags: MOE_EXEC_TWO_PHASE and its producer count, checked against the
// workgroups of one worker (MOE_ERR_ARG when out of range)
static int exec_split(int exec_flags, int P, bool* two_launches) {
  const int n1 = (exec_flags >> MOE_EXEC_SPLIT_SHIFT) & 0xff;
  *two_launches = (exec_flags & MOE_EXEC_TWO_PHASE) == 0;
  return n1 < wide_workers_wg(P) ? n1 : -1;
}

template <bool FP8>
static void run_forward_stream(const Sizes& z, ExecArgs& a, const int32_t* row_to_slot, void* y,
                               bool split, int n1split, bool f8act, void* const* ev,
                               hipStream_t st) {
  const int n1 = z.dff / (WC::BN / 2), n2 = z.d / WC::BN;
  a.tl_phase = MOE_TL_FC1;
  if (FP8 && f8act) {                  // x quantized per row block, FC1 on the fp8 MFMA
    launch_quant_act((const uint16_t*)a.x, z.T, z.d, (uint8_t*)a.xq, (int32_t*)a.xe, st);
    launch_stream<SrcFc1F8, WC, RowA8, RowW8>(a, n1, kStreamLds8, st);
    // A's slot rows in use, quantized the same way for FC2
    launch_quant_act((const uint16_t*)a.bufA, (int)z.max_slots, z.dff, (uint8_t*)a.hq, a.he, st,
                     a.boff + z.E, z.beta);
    rec(ev, 2, st);
    a.tl_phase = MOE_TL_FC2;
    launch_stream<SrcFc2F8, WC, RowA8, RowW8>(a, n2, kStreamLds8, st);
  } else if (split) {
    launch_stream<SrcFc1T<FP8>, WC, RowW, typename SrcFc1T<FP8>::OB>(a, n1, kStreamLds, st);
    rec(ev, 2, st);
    a.tl_phase = MOE_TL_FC2;
    launch_stream<SrcFc2T<FP8>, WC, RowW, typename SrcFc2T<FP8>::OB>(a, n2, kStreamLds, st);
  } else {
    launch_stream2<FwdP1<FP8>, FwdP2<FP8>, WC, RowW, typename SrcFc1T<FP8>::OB>(
        a, n1 | (n2 << 16), n1split, kStreamLds, st);
    rec(ev, 2, st);
  }
  rec(ev, 3, st);
  if (z.T > 0)
    hipLaunchKernelGGL(k_combine<uint16_t>, combine_grid<uint16_t>(z.T, z.d), dim3(256), 0, st,
                       (const uint16_t*)a.bufO, row_to_slot, z.T, z.k, z.d, (uint16_t*)y);
  rec(ev, 4, st);
}

int launch_forward(const Sizes& z, const LayerPtrs& Lp, const void* x, const float* gates,
                   const int32_t* counts, const int32_t* boff, const int32_t* row_to_slot,
                   const int32_t* slot_to_row, const int32_t* block_worker, void* y,
                   void* z_save, int32_t* status, char* ws, int exec_flags, void* const* ev,
                   uint64_t* timeline, hipStream_t st) {
  bool split = true;
  const int n1split = exec_split(exec_flags, z.P, &split);
  if (n1split < 0) return MOE_ERR_ARG;
  // the fp8 MFMA forward: e4m3 weights on the stream kernels, two launches
  if ((exec_flags & MOE_EXEC_FP8_ACT) &&
      (Lp.act_dtype != MOE_BF16 || Lp.w_dtype != MOE_FP8_E4M3 || !use_stream(z) || !split))
    return MOE_ERR_ARG;
  const WsLayout L = exec_layout(z, false);
  rec(ev, 0, st);
  // the stream kernels read the per-slot gates, written beside the schedule
  const bool stream = Lp.act_dtype == MOE_BF16 &&
                      (Lp.w_dtype == MOE_BF16 || Lp.w_dtype == MOE_FP8_E4M3) && use_stream(z);
  launch_sched(z, counts, boff, block_worker, nullptr, false, ws, L, status,
               stream ? slot_to_row : nullptr, stream ? gates : nullptr, st);
  rec(ev, 1, st);
  ExecArgs a = make_exec(z, Lp, ws, L);
  a.x = x; a.gates = gates; a.slot_to_row = slot_to_row; a.row_to_slot = row_to_slot;
  a.z_save = z_save;
  a.boff = boff;
  a.timeline = timeline;
  a.status = status;
  const bool big = use_big_tiles(z);
  const bool f8act = (exec_flags & MOE_EXEC_FP8_ACT) != 0;
  if (Lp.act_dtype == MOE_BF16 && Lp.w_dtype == MOE_BF16 && use_stream(z))
    run_forward_stream<false>(z, a, row_to_slot, y, split, n1split, false, ev, st);
  else if (Lp.act_dtype == MOE_BF16 && Lp.w_dtype == MOE_FP8_E4M3 && use_stream(z))
    run_forward_stream<true>(z, a, row_to_slot, y, split, n1split, f8act, ev, st);
  else if (Lp.act_dtype == MOE_F32) run_forward<float, false, SmallCfg>(z, a, row_to_slot, y, ev, st);
  else if (Lp.w_dtype == MOE_FP8_E4M3) {
    if (big) run_forward<uint16_t, true, BigCfg>(z, a, row_to_slot, y, ev, st);
    else run_forward<uint16_t, true, SmallCfg>(z, a, row_to_slot, y, ev, st);
  } else {
    if (big) run_forward<uint16_t, false, BigCfg>(z, a, row_to_slot, y, ev, st);
    else run_forward<uint16_t, false, SmallCfg>(z, a, row_to_slot, y, ev, st);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// With e4m3 weights (FP8): D = p dy per slot is requantized along the tokens
// and widened back to bf16 (dhat) before dA; dZ is requantized in place in
// bufA once dX has used it; the weight gradients then read both as bf16.
// With f8act (FP8 only, MOE_EXEC_FP8_ACT) dA and dX run on the fp8 MFMA:
// dy's rows are quantized per 128 features before dA; dA leaves as bf16 rows
// (bufO), and k_swiglu_bwd_q forms dZ and P from them and quantizes dZ's rows
// for dX.
template <bool FP8>
static void run_backward_stream(const Sizes& z, ExecArgs& a, const int32_t* row_to_slot, void* dx,
                                float* dw1, float* dw2, bool split, int n1split, bool f8act,
                                void* const* ev, hipStream_t st) {
  const int rows = (int)z.max_slots;
  if constexpr (FP8)
    launch_quant_dequant((const uint16_t*)a.dy, z.d, a.slot_to_row, 1, z.k, a.gates, z.T * z.k,
                         rows, z.d, z.beta, (uint16_t*)a.dhat, a.boff + z.E, st);
  const int n1 = z.dff / WC::BN, n2 = z.d / WC::BN;
  a.tl_phase = MOE_TL_DA;
  if (FP8 && f8act) {
    launch_quant_act((const uint16_t*)a.dy, z.T, z.d, (uint8_t*)a.xq, (int32_t*)a.xe, st);
    launch_stream<SrcDaF8, WC, RowA8, MnK8Op>(a, n1, kStreamLds8, st);
    launch_swiglu_bwd_q(a, z.dff, a.boff + z.E, z.beta, st);
    rec(ev, 2, st);
    a.tl_phase = MOE_TL_DX;
    launch_stream<SrcDxF8, WC, RowA8, MnK8Op>(a, n2, kStreamLds8, st);
  } else if (split) {
    launch_stream<SrcDaT<FP8>, WC, RowW, typename SrcDaT<FP8>::OB>(a, n1, kStreamLds, st);
    rec(ev, 2, st);
    a.tl_phase = MOE_TL_DX;
    launch_stream<SrcDxT<FP8>, WC, RowW, typename SrcDxT<FP8>::OB>(a, n2, kStreamLds, st);
  } else {
    launch_stream2<BwdP1<FP8>, BwdP2<FP8>, WC, RowW, typename SrcDaT<FP8>::OB>(
        a, n1 | (n2 << 16), n1split, kStreamLds, st);
    rec(ev, 2, st);
  }
  rec(ev, 3, st);
  if (z.T > 0)
    hipLaunchKernelGGL(k_combine<uint16_t>, combine_grid<uint16_t>(z.T, z.d), dim3(256), 0, st,
                       (const uint16_t*)a.bufO, row_to_slot, z.T, z.k, z.d, (uint16_t*)dx);
  rec(ev, 4, st);
  if constexpr (FP8)
    launch_quant_dequant((const uint16_t*)a.bufA, 2 * z.dff, a.slot_to_row, 0, 1, nullptr,
                         z.T * z.k, rows, 2 * z.dff, z.beta, (uint16_t*)a.bufA, a.boff + z.E, st);
  a.tl_phase = MOE_TL_DW;
  launch_stream<SrcDwT<DwCfg, FP8>, DwCfg, MnSegOp, MnSegOp>(a, 0, kDwLds, st);
  rec(ev, 5, st);
  hipLaunchKernelGGL(k_bwd_reduce, dim3(num_cus() * 4), dim3(256), 0, st, a.rep_slot,
                     a.owner_has, (const float*)a.rslots, z.E, z.P, z.d, z.dff, dw1, dw2);
  rec(ev, 6, st);
}

template <typename T, class C, bool FP8 = false>
static void run_backward(const Sizes& z, ExecArgs& a, const int32_t* row_to_slot, void* dx,
                         float* dw1, float* dw2, void* const* ev, hipStream_t st) {
  a.bufP = nullptr;
  const size_t lds = gemm_lds_bytes<T, C>();
  static int ga = persistent_grid(k_bwd_da<T, C, FP8>, C::NT, lds);
  static int gx = persistent_grid(k_bwd_dx<T, C, FP8>, C::NT, lds);
  static int gw = persistent_grid(k_bwd_dw<T, C, FP8>, C::NT, lds);
  const int rows = (int)z.max_slots;
  if constexpr (FP8)   // D = p * dy per slot, e4m3 along tokens, for dW2
    launch_quant_tok((const uint16_t*)a.dy, z.d, a.slot_to_row, 1, z.k, a.gates, z.T * z.k, rows,
                     z.d, z.beta, a.dq, a.dqs, st, a.boff + z.E);
  hipLaunchKernelGGL((k_bwd_da<T, C, FP8>), dim3(ga), dim3(C::NT), lds, st, a);
  if constexpr (FP8)   // dZ per slot (padding slots read as zero), for dW1
    launch_quant_tok((const uint16_t*)a.bufA, 2 * z.dff, a.slot_to_row, 0, 1, nullptr, z.T * z.k,
                     rows, 2 * z.dff, z.beta, a.zq, a.zqs, st, a.boff + z.E);
  rec(ev, 2, st);
  hipLaunchKernelGGL((k_bwd_dx<T, C, FP8>), dim3(gx), dim3(C::NT), lds, st, a);
  rec(ev, 3, st);
  if (z.T > 0)
    hipLaunchKernelGGL(k_combine<T>, combine_grid<T>(z.T, z.d), dim3(256), 0, st,
                       (const T*)a.bufO, row_to_slot, z.T, z.k, z.d, (T*)dx);
  rec(ev, 4, st);
  hipLaunchKernelGGL((k_bwd_dw<T, C, FP8>), dim3(gw), dim3(C::NT), lds, st, a);
  rec(ev, 5, st);
  hipLaunchKernelGGL(k_bwd_reduce, dim3(num_cus() * 4), dim3(256), 0, st, a.rep_slot,
                     a.owner_has, (const float*)a.rslots, z.E, z.P, z.d, z.dff, dw1, dw2);
  rec(ev, 6, st);
}

int launch_backward(const Sizes& z, const LayerPtrs& Lp, const void* x, const float* gates,
                    const void* dy, const void* z_save, const int32_t* counts,
                    const int32_t* boff, const int32_t* row_to_slot,
                    const int32_t* slot_to_row, const int32_t* owner,
                    const int32_t* block_worker, void* dx, float* dw1, float* dw2,
                    int32_t* status, char* ws, int exec_flags, void* const* ev,
                    uint64_t* timeline, hipStream_t st) {
  bool split = true;
  const int n1split = exec_split(exec_flags, z.P, &split);
  if (n1split < 0) return MOE_ERR_ARG;
  if ((exec_flags & MOE_EXEC_FP8_ACT) &&
      (Lp.act_dtype != MOE_BF16 || Lp.w_dtype != MOE_FP8_E4M3 || !use_stream(z) || !split))
    return MOE_ERR_ARG;
  const WsLayout L = exec_layout(z, true);
  rec(ev, 0, st);
  const bool stream = Lp.act_dtype != MOE_F32 && use_stream(z);
  launch_sched(z, counts, boff, block_worker, owner, true, ws, L, status,
               stream ? slot_to_row : nullptr, stream ? gates : nullptr, st);
  rec(ev, 1, st);
  ExecArgs a = make_exec(z, Lp, ws, L);
  a.x = x; a.gates = gates; a.slot_to_row = slot_to_row; a.row_to_slot = row_to_slot;
  a.z_save = const_cast<void*>(z_save);
  a.dy = dy; a.dw1 = dw1; a.dw2 = dw2; a.boff = boff;
  a.timeline = timeline;
  a.status = status;
  if (Lp.act_dtype == MOE_F32) run_backward<float, SmallCfg>(z, a, row_to_slot, dx, dw1, dw2, ev, st);
  else if (Lp.w_dtype == MOE_FP8_E4M3) {
    if (use_stream(z))
      run_backward_stream<true>(z, a, row_to_slot, dx, dw1, dw2, split, n1split,
                                (exec_flags & MOE_EXEC_FP8_ACT) != 0, ev, st);
    else if (use_big_tiles(z)) run_backward<uint16_t, BigCfg, true>(z, a, row_to_slot, dx, dw1, dw2, ev, st);
    else run_backward<uint16_t, SmallCfg, true>(z, a, row_to_slot, dx, dw1, dw2, ev, st);
  } else if (use_stream(z))
    run_backward_stream<false>(z, a, row_to_slot, dx, dw1, dw2, split, n1split, false, ev, st);
  else if (use_big_tiles(z)) run_backward<uint16_t, BigCfg>(z, a, row_to_slot, dx, dw1, dw2, ev, st);
  else run_backward<uint16_t, SmallCfg>(z, a, row_to_slot, dx, dw1, dw2, ev, st);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
