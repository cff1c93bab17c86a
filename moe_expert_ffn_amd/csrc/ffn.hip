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
  int E, P, s, beta, backward, bm;
  int32_t* ctr;
  int32_t* mt_cnt;
  int4* mt;
  int max_mt;
  int32_t* seg_cnt;
  int4* seg;
  int32_t* rep_slot;
  int32_t* owner_has;
  int32_t* status;
};

MOE_DEV int expert_of(int g, const int* boff_s, int E) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (boff_s[mid] <= g) lo = mid; else hi = mid;
  }
  return lo;
}

// One workgroup.  M-tiles: a tile holds up to `bm` consecutive slots of one
// (expert, worker) run of blocks.  When bm is a multiple of beta, tiles start
// every bm/beta blocks from the start of each run; otherwise every block is cut
// into ceil(valid rows / bm) tiles of its own.  Tiles are listed per worker in
// block order (one exclusive scan per worker).  Segments (backward): the
// blocks of one (expert, worker) pair must form one contiguous run; its slot
// range and valid-row count become one weight-gradient segment, with a replica
// slot when the worker is not the owner (rank among that worker's non-home
// experts, in expert order).
MOE_DEV int block_rows(int g, int e, int beta, const int* boff_s, const int* cnt_s) {
  return min(beta, beta * boff_s[e] + cnt_s[e] - beta * g);
}

__global__ __launch_bounds__(256) void k_sched(SchedArgs a) {
  extern __shared__ int sm[];
  const int E = a.E, P = a.P;
  int* boff_s = sm;
  int* cnt_s = boff_s + E + 1;
  int* s0_s = cnt_s + E;
  int* rows_s = s0_s + E * P;
  int* starts_s = rows_s + E * P;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i <= E; i += 256) boff_s[i] = a.boff[i];
  for (int i = tid; i < E; i += 256) cnt_s[i] = a.counts[i];
  if (tid < kNumCounters) a.ctr[tid] = 0;
  if (a.backward)
    for (int i = tid; i < E * P; i += 256) { s0_s[i] = INT_MAX; rows_s[i] = 0; starts_s[i] = 0; }
  __syncthreads();
  const int nb = boff_s[E];
  for (int g = tid; g < nb; g += 256) {
    const int w = a.bw[g];
    if (w < 0 || w >= P) atomicOr(a.status, MOE_DEV_BAD_PLAN);
  }
  const bool grouped = (a.bm % a.beta) == 0;
  const int f = grouped ? a.bm / a.beta : 1;
  const uint64_t le_mask = (lane == 63) ? ~0ull : ((1ull << (lane + 1)) - 1);
  for (int r = wv; r < P; r += 4) {
    int run = 0, carry = 0;
    for (int base = 0; base < nb; base += 64) {
      const int g = base + lane;
      const bool mine = g < nb && a.bw[g] == r;
      int e = 0, bstart = 0, vrows = 0;
      bool start = false;
      if (mine) {
        e = expert_of(g, boff_s, E);
        bstart = a.beta * g;
        vrows = block_rows(g, e, a.beta, boff_s, cnt_s);
        start = (g == boff_s[e]) || a.bw[g - 1] != r;
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
              if (gi >= boff_s[e + 1] || (i > 0 && a.bw[gi] != r)) break;
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

  for (int g = tid; g < nb; g += 256) {
    const int w = a.bw[g];
    if (w < 0 || w >= P) continue;
    const int e = expert_of(g, boff_s, E);
    const int vrows = min(a.beta, a.beta * boff_s[e] + cnt_s[e] - a.beta * g);
    atomicMin(&s0_s[e * P + w], a.beta * g);
    atomicAdd(&rows_s[e * P + w], vrows);
    if (g == boff_s[e] || a.bw[g - 1] != w) atomicAdd(&starts_s[e * P + w], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    const int h = a.owner[e];
    const bool ok = h >= 0 && h < P;
    if (!ok) atomicOr(a.status, MOE_DEV_BAD_OWNER);
    a.owner_has[e] = (ok && rows_s[e * P + h] > 0 && starts_s[e * P + h] == 1) ? 1 : 0;
  }
  for (int r = wv; r < P; r += 4) {
    // pass 0: replica segments (non-home experts) first; pass 1: home segments
    int run = 0, rrun = 0;
    for (int pass = 0; pass < 2; ++pass) {
      for (int base = 0; base < E; base += 64) {
        const int e = base + lane;
        int take = 0, dst = -1;
        bool bad = false;
        if (e < E) {
          const int h = a.owner[e];
          const int rows = rows_s[e * P + r];
          const bool home = (h == r);
          if (rows > 0 && starts_s[e * P + r] != 1) bad = true;
          take = (rows > 0 && home == (pass == 1) && h >= 0 && h < P) ? 1 : 0;
          if (pass == 0) a.rep_slot[e * P + r] = -1;
        }
        const int nonhome = (pass == 0) ? take : 0;
        const int rinc = wave_incl_scan(nonhome);
        const int rpos = rrun + rinc - nonhome;
        if (nonhome) {
          if (rpos >= a.s) bad = true;
          else dst = r * a.s + rpos;
        }
        const int inc = wave_incl_scan(take);
        const int pos = run + inc - take;
        if (take) {
          if (bad) {
            atomicOr(a.status, MOE_DEV_BAD_PLAN);
            a.seg[(size_t)r * E + pos] = make_int4(-1, 0, 0, -1);
          } else {
            a.seg[(size_t)r * E + pos] = make_int4(e, s0_s[e * P + r], rows_s[e * P + r], dst);
            if (nonhome) a.rep_slot[e * P + r] = dst;
          }
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
  int T, k, E, d, dff, P, s;
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
template <typename T>
__global__ __launch_bounds__(256) void k_combine(const T* __restrict__ src,
                                                 const int32_t* __restrict__ row_to_slot,
                                                 int T_, int k, int d, T* __restrict__ out) {
  constexpr int VE = Elem<T>::VE;
  const int per_row = d / VE;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)T_ * per_row) return;
  const int t = (int)(idx / per_row), c = (int)(idx % per_row) * VE;
  float acc[VE];
#pragma unroll
  for (int v = 0; v < VE; ++v) acc[v] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int s = row_to_slot[(size_t)t * k + j];
    if (s < 0) continue;
    V16 in;
    in.u = ldg16(src + (size_t)s * d + c);
#pragma unroll
    for (int v = 0; v < VE; ++v) {
      if constexpr (sizeof(T) == 2) acc[v] += bf2f(in.h[v]);
      else acc[v] += in.f[v];
    }
  }
  V16 o;
#pragma unroll
  for (int v = 0; v < VE; ++v) {
    if constexpr (sizeof(T) == 2) o.h[v] = f2bf(acc[v]);
    else o.f[v] = acc[v];
  }
  stg16(out + (size_t)t * d + c, o.u);
}

// ---- backward: dA -> dZ -------------------------------------------------------
// dA[slot, n] = p * sum_c dy[t, c] W2[c, n]; W2 is read as a K-major (c) by
// N-contiguous operand and transposed into LDS.
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

template <typename T, class C>
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
    SrcRowsMN<T> src{(const T*)a.w2 + (size_t)e * a.d * a.dff, a.dff, nj * C::BN, a.dff};
    f32x16_t acc[C::MB][C::NB];
    gemm_tile<T, C>(PlainLd<decltype(la)>{la}, TransLd<decltype(lb), SrcRowsMN<T>>{lb, src},
                    a.d / Elem<T>::BK, smem, acc);
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
template <typename T, class C>
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
    SrcRowsMN<T> src{(const T*)a.w1 + (size_t)e * 2 * a.dff * a.d, a.d, nj * C::BN, a.d};
    f32x16_t acc[C::MB][C::NB];
    gemm_tile<T, C>(PlainLd<decltype(la)>{la}, TransLd<decltype(lb), SrcRowsMN<T>>{lb, src},
                    2 * a.dff / Elem<T>::BK, smem, acc);
    constexpr int LDO = C::BN + 16 / (int)sizeof(T);
    acc_to_lds<C>(acc, smem, LDO, 0, C::BM, [&](float v, int, int) { return to_act<T>(v); });
    __syncthreads();
    const size_t obase = (size_t)slot0 * a.d + nj * C::BN;
    lds_to_global<T, C::NT>(smem, C::BM, C::BN, LDO, [&](int row, int col, const V16& v) {
      if (row < nrows) stg16(dXp + obase + (size_t)row * a.d + col, v.u);
    });
  }
}

// ---- two workgroups per CU: FC1, FC2, dA, dX -----------------------------------
// 256-row M tiles of one (expert, worker) run, 128-wide N tiles, transposed
// accumulators: lane (lane & 31) of wave (wm, wn) owns rows wm*128 + 32 i +
// (lane & 31) and, per register quad g of block j, the four consecutive
// columns wn*64 + 32 j + 8 g + 4 (lane >> 5) .. +3, stored straight from
// registers.  Fast exp / reciprocal in the SiLU terms: their error is far
// below the bf16 rounding of every value they feed.
MOE_DEV float sigm(float g) { return __builtin_amdgcn_rcpf(1.f + __expf(-g)); }

template <class C> MOE_DEV int dual_row(int i, int lane) { return acc_row_t<C>(i, lane); }
template <class C> MOE_DEV int dual_col(int j, int g, int lane) { return acc_col_t<C>(j, g, lane); }

// Tile engines of the GEMM kernels below.  Both give every wave a 128 x 64
// piece of the tile (128 accumulator registers, two waves per SIMD) with
// transposed accumulators, so the epilogues are shared:
//   EngDual: 256 x 128 tiles, 4 waves, two workgroups per CU, K = 32 per
//            stage, three stages (72 KB);
//   EngWide: 256 x 256 tiles, 8 waves, one workgroup per CU, K = 64 per
//            stage (full 128-byte lines), two stages (128 KB).
struct EngDual {
  using C = DualCfg;
  static constexpr int BK = kDmaBK, MINB = 2;
  template <int R> using Row = RowDma<R, C::NT / 64>;
  template <int M> using Mn = MnDma<M, C::NT / 64>;
  template <class A, class B> using Pipe = DmaPipe<C, A, B, kDualStages, true>;
  template <class OP, class F> static MOE_DEV MnOperand<OP, F> mn(const OP& op, F f) { return {op, f}; }
  static constexpr size_t LDS = (size_t)kDualStages * (C::BM + C::BN) * kDmaBK * 2;
};
struct EngWide {
  using C = WideCfg;
  static constexpr int BK = kWideBK, MINB = 1;
  template <int R> using Row = Row64<R, C::NT / 64>;
  template <int M> using Mn = Mn64<M, C::NT / 64>;
  template <class A, class B> using Pipe = WidePipe<C, A, B>;
  template <class OP, class F> static MOE_DEV Mn64Operand<OP, F> mn(const OP& op, F f) { return {op, f}; }
  static constexpr size_t LDS = (size_t)kWideStages * (C::BM + C::BN) * kWideRowBytes;
};

// FC1 + SwiGLU.  N tile nj covers A columns [64 nj, 64 nj + 64): weight rows
// alternate 32 G rows and the matching 32 U rows, so block j = 0 of a wave is
// G and block j = 1 is U of the same 32 columns.
template <class E>
__global__ __launch_bounds__(E::C::NT, E::MINB) void k_fc1_t(ExecArgs a) {
  using C = typename E::C;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int tslot;
  MOE_LDS uint16_t* smem = (MOE_LDS uint16_t*)smem_raw;
  constexpr int NW = C::NT / 64, HALF = C::BN / 2;
  static_assert(C::NB == 2 && C::WN == 64, "one G block and one U block per wave");
  const int r = worker_of_block(a.P);
  const int nnt = a.dff / HALF;
  const int total = a.mt_cnt[r] * nnt;
  const int lane = threadIdx.x & 63;
  const int wn = wave_id() % C::WAVES_N;
  uint16_t* Ab = (uint16_t*)a.bufA;
  uint16_t* Z = (uint16_t*)a.z_save;
  const uint32_t bx = (uint32_t)((size_t)a.T * a.d * 2);
  while (true) {
    const int tile = next_tile(&a.ctr[PH_FC1 * kMaxP + r], &tslot);
    if (tile >= total) break;
    const int4 m = a.mt[(size_t)r * a.max_mt + tile / nnt];
    const int nj = tile % nnt;
    const int e = m.x, slot0 = m.y, nrows = m.z;
    typename E::template Row<C::BM> da;
    da.init((const uint16_t*)a.x, bx,
            [&](int row) { return row < nrows ? (a.slot_to_row[slot0 + row] / a.k) * a.d : -1; });
    typename E::template Row<C::BN> db;
    db.init((const uint16_t*)a.w1 + (size_t)e * 2 * a.dff * a.d, (uint32_t)((size_t)4 * a.dff * a.d),
            [&](int rho) {
              const int q = rho >> 5;
              return ((q & 1) * a.dff + nj * HALF + (q >> 1) * 32 + (rho & 31)) * a.d;
            });
    f32x16_t acc[C::MB][C::NB];
    typename E::template Pipe<typename E::template Row<C::BM>, typename E::template Row<C::BN>> p;
    p.run(da, db, a.d / E::BK, smem, acc);
    const int col0 = nj * HALF + wn * 32 + 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < C::MB; ++i) {
      const int row = dual_row<C>(i, lane);
      if (row >= nrows) continue;
      const size_t sr = (size_t)slot0 + row;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float gv[4], uv[4], av[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          gv[q] = acc[i][0][4 * g + q];
          uv[q] = acc[i][1][4 * g + q];
          av[q] = gv[q] * sigm(gv[q]) * uv[q];
        }
        const int c = col0 + 8 * g;
        store4(Ab + sr * a.dff + c, av);
        if (Z) {
          store4(Z + sr * 2 * a.dff + c, gv);
          store4(Z + sr * 2 * a.dff + a.dff + c, uv);
        }
      }
    }
  }
}

// FC2 with the gate: O[slot] = p * A W2^T.
template <class E>
__global__ __launch_bounds__(E::C::NT, E::MINB) void k_fc2_t(ExecArgs a) {
  using C = typename E::C;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int tslot;
  MOE_LDS uint16_t* smem = (MOE_LDS uint16_t*)smem_raw;
  constexpr int NW = C::NT / 64;
  const int r = worker_of_block(a.P);
  const int nnt = a.d / C::BN;
  const int total = a.mt_cnt[r] * nnt;
  const int lane = threadIdx.x & 63;
  uint16_t* O = (uint16_t*)a.bufO;
  while (true) {
    const int tile = next_tile(&a.ctr[PH_FC2 * kMaxP + r], &tslot);
    if (tile >= total) break;
    const int4 m = a.mt[(size_t)r * a.max_mt + tile / nnt];
    const int nj = tile % nnt;
    const int e = m.x, slot0 = m.y, nrows = m.z;
    typename E::template Row<C::BM> da;
    da.init((const uint16_t*)a.bufA, (uint32_t)(a.slots * a.dff * 2),
            [&](int row) { return row < nrows ? (slot0 + row) * a.dff : -1; });
    typename E::template Row<C::BN> db;
    db.init((const uint16_t*)a.w2 + (size_t)e * a.d * a.dff, (uint32_t)((size_t)2 * a.d * a.dff),
            [&](int rho) { return (nj * C::BN + rho) * a.dff; });
    f32x16_t acc[C::MB][C::NB];
    typename E::template Pipe<typename E::template Row<C::BM>, typename E::template Row<C::BN>> p;
    p.run(da, db, a.dff / E::BK, smem, acc);
#pragma unroll
    for (int i = 0; i < C::MB; ++i) {
      const int row = dual_row<C>(i, lane);
      if (row >= nrows) continue;
      const float pg = a.gates[a.slot_to_row[slot0 + row]];
      uint16_t* orow = O + ((size_t)slot0 + row) * a.d + nj * C::BN;
#pragma unroll
      for (int j = 0; j < C::NB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = pg * acc[i][j][4 * g + q];
          store4(orow + dual_col<C>(j, g, lane), v);
        }
    }
  }
}

// dA = p * dy W2 (W2 [d][d_ff] read K-major through transpose reads), then
// dZ = [dA U s (1 + G (1 - s)), dA G s] with s = sigmoid(G), and the gated
// activation P = p SiLU(G) U for the weight gradient of W2.
template <class E>
__global__ __launch_bounds__(E::C::NT, E::MINB) void k_bwd_da_t(ExecArgs a) {
  using C = typename E::C;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int tslot;
  MOE_LDS uint16_t* smem = (MOE_LDS uint16_t*)smem_raw;
  constexpr int NW = C::NT / 64;
  const int r = worker_of_block(a.P);
  const int nnt = a.dff / C::BN;
  const int total = a.mt_cnt[r] * nnt;
  const int lane = threadIdx.x & 63;
  const uint16_t* Z = (const uint16_t*)a.z_save;
  uint16_t* dZ = (uint16_t*)a.bufA;
  uint16_t* PA = (uint16_t*)a.bufP;
  const uint32_t bx = (uint32_t)((size_t)a.T * a.d * 2);
  while (true) {
    const int tile = next_tile(&a.ctr[PH_DA * kMaxP + r], &tslot);
    if (tile >= total) break;
    const int4 m = a.mt[(size_t)r * a.max_mt + tile / nnt];
    const int nj = tile % nnt;
    const int e = m.x, slot0 = m.y, nrows = m.z;
    typename E::template Row<C::BM> da;
    da.init((const uint16_t*)a.dy, bx,
            [&](int row) { return row < nrows ? (a.slot_to_row[slot0 + row] / a.k) * a.d : -1; });
    const typename E::template Mn<C::BN> mb{make_rsrc((const uint16_t*)a.w2 + (size_t)e * a.d * a.dff,
                                                      (uint32_t)((size_t)2 * a.d * a.dff))};
    const uint32_t bcol = (uint32_t)nj * C::BN * 2u, bld = (uint32_t)a.dff * 2u;
    auto ob = E::mn(mb, [=](int kk) -> uint32_t { return (uint32_t)kk * bld + bcol; });
    f32x16_t acc[C::MB][C::NB];
    typename E::template Pipe<typename E::template Row<C::BM>, decltype(ob)> p;
    p.run(da, ob, a.d / E::BK, smem, acc);
#pragma unroll
    for (int i = 0; i < C::MB; ++i) {
      const int row = dual_row<C>(i, lane);
      if (row >= nrows) continue;
      const size_t sr = (size_t)slot0 + row;
      const float pg = a.gates[a.slot_to_row[slot0 + row]];
#pragma unroll
      for (int j = 0; j < C::NB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = nj * C::BN + dual_col<C>(j, g, lane);
          float gv[4], uv[4], dg[4], du[4], pa[4];
          load4(Z + sr * 2 * a.dff + n, gv);
          load4(Z + sr * 2 * a.dff + a.dff + n, uv);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float v = pg * acc[i][j][4 * g + q];
            const float sg = sigm(gv[q]);
            dg[q] = v * uv[q] * sg * (1.f + gv[q] * (1.f - sg));
            du[q] = v * gv[q] * sg;
            pa[q] = pg * (gv[q] * sg * uv[q]);
          }
          store4(dZ + sr * 2 * a.dff + n, dg);
          store4(dZ + sr * 2 * a.dff + a.dff + n, du);
          store4(PA + sr * a.dff + n, pa);
        }
    }
  }
}

// dX per routed row: dZ W1 (W1 [2 d_ff][d] read K-major through transpose reads).
template <class E>
__global__ __launch_bounds__(E::C::NT, E::MINB) void k_bwd_dx_t(ExecArgs a) {
  using C = typename E::C;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int tslot;
  MOE_LDS uint16_t* smem = (MOE_LDS uint16_t*)smem_raw;
  constexpr int NW = C::NT / 64;
  const int r = worker_of_block(a.P);
  const int nnt = a.d / C::BN;
  const int total = a.mt_cnt[r] * nnt;
  const int lane = threadIdx.x & 63;
  uint16_t* dXp = (uint16_t*)a.bufO;
  while (true) {
    const int tile = next_tile(&a.ctr[PH_DX * kMaxP + r], &tslot);
    if (tile >= total) break;
    const int4 m = a.mt[(size_t)r * a.max_mt + tile / nnt];
    const int nj = tile % nnt;
    const int e = m.x, slot0 = m.y, nrows = m.z;
    typename E::template Row<C::BM> da;
    da.init((const uint16_t*)a.bufA, (uint32_t)(a.slots * 4 * a.dff),
            [&](int row) { return row < nrows ? (slot0 + row) * 2 * a.dff : -1; });
    const typename E::template Mn<C::BN> mb{make_rsrc((const uint16_t*)a.w1 + (size_t)e * 2 * a.dff * a.d,
                                                      (uint32_t)((size_t)4 * a.dff * a.d))};
    const uint32_t bcol = (uint32_t)nj * C::BN * 2u, bld = (uint32_t)a.d * 2u;
    auto ob = E::mn(mb, [=](int kk) -> uint32_t { return (uint32_t)kk * bld + bcol; });
    f32x16_t acc[C::MB][C::NB];
    typename E::template Pipe<typename E::template Row<C::BM>, decltype(ob)> p;
    p.run(da, ob, 2 * a.dff / E::BK, smem, acc);
#pragma unroll
    for (int i = 0; i < C::MB; ++i) {
      const int row = dual_row<C>(i, lane);
      if (row >= nrows) continue;
      uint16_t* orow = dXp + ((size_t)slot0 + row) * a.d + nj * C::BN;
#pragma unroll
      for (int j = 0; j < C::NB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = acc[i][j][4 * g + q];
          store4(orow + dual_col<C>(j, g, lane), v);
        }
    }
  }
}

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
    const float p = gates[slot_to_row[slot0 + kk]];
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

template <typename T, class C>
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
      SrcGatherRow<T> sa{(const T*)a.dy, a.slot_to_row, slot0, nrows, a.k, a.d, mi * C::BM, a.d};
      SrcGatedAct<T> sb{(const T*)a.z_save, a.gates, a.slot_to_row, slot0, nrows, a.dff,
                        nj * C::BN};
      gemm_tile<T, C>(TransLd<decltype(la), SrcGatherRow<T>>{la, sa},
                      TransLd<decltype(lb), SrcGatedAct<T>>{lb, sb}, nk, smem, acc);
      out = (dst < 0 ? a.dw2 + (size_t)e * a.d * a.dff
                     : a.rslots + (size_t)dst * w_elems + (size_t)2 * a.dff * a.d);
      ldo = a.dff;
      nlim = a.dff;
    } else {
      loc -= n2m * n2n;
      mi = loc / n1n;
      nj = loc % n1n;
      SrcSlotRow<T> sa{(const T*)a.bufA, slot0, nrows, 2 * a.dff, mi * C::BM, 2 * a.dff};
      SrcGatherRow<T> sb{(const T*)a.x, a.slot_to_row, slot0, nrows, a.k, a.d, nj * C::BN, a.d};
      gemm_tile<T, C>(TransLd<decltype(la), SrcSlotRow<T>>{la, sa},
                      TransLd<decltype(lb), SrcGatherRow<T>>{lb, sb}, nk, smem, acc);
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

// ---- weight gradients on the direct-to-LDS pipeline, two workgroups per CU ------
// Weight gradients per (expert, worker) segment; K = the segment's routed rows,
// in windows of up to kTokWin rows whose token indices sit in an LDS table.
// dW2[c, n] = sum dy_t[c] * P[n];  dW1[j, c] = sum dZ[j] * x_t[c].
// Every operand is read in its natural [row][feature] layout through transpose
// reads; rows past the segment read as zeros.  Tiles are 256 (M) x 128
// (N) with transposed accumulators: each lane stores 16-byte runs of one fp32
// output row directly, and the other workgroup on the CU computes meanwhile.
constexpr int kTokWin = 2048;
// Byte offset of (source row of K index k, col) in one operand: a gathered
// token row (token index from the LDS table) or a slot row; kOob past the
// window, which reads as zeros.
// The table is read unconditionally and the row picked arithmetically
// (g = 1: gathered, 0: slot row) so the reads of one step are all in flight
// together instead of each behind a branch.
struct DwRows {
  const MOE_LDS uint16_t* tok;
  int wrows, s0, ld, col;
  uint32_t g;
  MOE_DEV uint32_t operator()(int k) const {
    const int kk = min(k, wrows - 1);
    const uint32_t t = tok[kk];
    const uint32_t row = t * g + (uint32_t)(s0 + kk) * (1u - g);
    const uint32_t o = (row * (uint32_t)ld + (uint32_t)col) * 2u;
    return k < wrows ? o : kOob;
  }
};
template <class E> struct DwEng {
  using C = typename E::C;
  using OA = decltype(E::mn(std::declval<const typename E::template Mn<C::BM>&>(), std::declval<DwRows>()));
  using OB = decltype(E::mn(std::declval<const typename E::template Mn<C::BN>&>(), std::declval<DwRows>()));
  using Pipe = typename E::template Pipe<OA, OB>;
  static constexpr size_t STAGE_BYTES = Pipe::BYTES;
  static constexpr size_t LDS_BYTES = STAGE_BYTES + (size_t)kTokWin * 2;
};

template <class E>
__global__ __launch_bounds__(E::C::NT, E::MINB) void k_bwd_dw_t(ExecArgs a) {
  using C = typename E::C;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int tslot;
  MOE_LDS uint16_t* smem = (MOE_LDS uint16_t*)smem_raw;
  MOE_LDS uint16_t* tok = smem + DwEng<E>::STAGE_BYTES / 2;
  constexpr int NW = C::NT / 64;
  const int r = worker_of_block(a.P);
  const int n2m = a.d / C::BM, n2n = a.dff / C::BN;          // dW2 [d][dff]
  const int n1m = 2 * a.dff / C::BM, n1n = a.d / C::BN;      // dW1 [2dff][d]
  const int per_seg = n2m * n2n + n1m * n1n;
  const int total = a.seg_cnt[r] * per_seg;
  const size_t w_elems = (size_t)3 * a.d * a.dff;
  const uint32_t bx = (uint32_t)((size_t)a.T * a.d * 2);
  const BufRsrc r_dy = make_rsrc(a.dy, bx), r_x = make_rsrc(a.x, bx);
  const BufRsrc r_dz = make_rsrc(a.bufA, (uint32_t)(a.slots * 4 * a.dff));
  const BufRsrc r_p = make_rsrc(a.bufP, (uint32_t)(a.slots * 2 * a.dff));
  const int lane = threadIdx.x & 63;
  while (true) {
    const int tile = next_tile(&a.ctr[PH_DW * kMaxP + r], &tslot);
    if (tile >= total) break;
    const int4 sg = a.seg[(size_t)r * a.E + tile / per_seg];
    const int e = sg.x, slot0 = sg.y, nrows = sg.z, dst = sg.w;
    if (e < 0) continue;
    const int loc = tile % per_seg;
    const bool is2 = loc < n2m * n2n;
    const int mi = is2 ? loc / n2n : (loc - n2m * n2n) / n1n;
    const int nj = is2 ? loc % n2n : (loc - n2m * n2n) % n1n;
    // dW2 = dy^T P (A: gathered dy rows, B: P rows);  dW1 = dZ^T x (A: dZ rows, B: gathered x rows)
    const typename E::template Mn<C::BM> ma{is2 ? r_dy : r_dz};
    const typename E::template Mn<C::BN> mb{is2 ? r_p : r_x};
    f32x16_t acc[C::MB][C::NB];
    for (int w0 = 0; w0 < nrows; w0 += kTokWin) {
      const int wrows = min(kTokWin, nrows - w0);
      const int s0 = slot0 + w0;
      __syncthreads();                       // previous users of the table are done
      for (int i = threadIdx.x; i < wrows; i += C::NT) tok[i] = (uint16_t)(a.slot_to_row[s0 + i] / a.k);
      __syncthreads();
      uint32_t ga = __builtin_amdgcn_readfirstlane(is2 ? 1u : 0u);
      asm volatile("" : "+s"(ga));           // opaque: keeps the select arithmetic
      const DwRows ra{tok, wrows, s0, is2 ? a.d : 2 * a.dff, mi * C::BM, ga};
      const DwRows rb{tok, wrows, s0, is2 ? a.dff : a.d, nj * C::BN, 1u - ga};
      typename DwEng<E>::Pipe p;
      p.run(E::mn(ma, ra), E::mn(mb, rb), (wrows + E::BK - 1) / E::BK, smem, acc, w0 > 0);
    }
    float* out;
    int ldo;
    if (is2) {
      out = (dst < 0 ? a.dw2 + (size_t)e * a.d * a.dff
                     : a.rslots + (size_t)dst * w_elems + (size_t)2 * a.dff * a.d);
      ldo = a.dff;
    } else {
      out = (dst < 0 ? a.dw1 + (size_t)e * 2 * a.dff * a.d : a.rslots + (size_t)dst * w_elems);
      ldo = a.d;
    }
    out += (size_t)mi * C::BM * ldo + (size_t)nj * C::BN;
#pragma unroll
    for (int i = 0; i < C::MB; ++i) {
      float* orow = out + (size_t)acc_row_t<C>(i, lane) * ldo;
#pragma unroll
      for (int j = 0; j < C::NB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          stg16(orow + acc_col_t<C>(j, g, lane),
                make_uint4(__float_as_uint(acc[i][j][4 * g]), __float_as_uint(acc[i][j][4 * g + 1]),
                           __float_as_uint(acc[i][j][4 * g + 2]), __float_as_uint(acc[i][j][4 * g + 3])));
    }
  }
}

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
  L.bufA = take((size_t)z.act_bytes * z.max_slots * (backward ? 2 : 1) * z.dff);
  L.bufO = take((size_t)z.act_bytes * z.max_slots * z.d);
  L.rslots = backward ? take(sizeof(float) * (size_t)z.P * z.s * 3 * z.d * z.dff) : o;
  L.bufP = backward ? take((size_t)z.act_bytes * z.max_slots * z.dff) : o;
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

static size_t sched_lds(const Sizes& z, bool bwd) {
  return sizeof(int) * ((size_t)2 * z.E + 1 + (bwd ? (size_t)3 * z.E * z.P : 0));
}

static void launch_sched(const Sizes& z, const int32_t* counts, const int32_t* boff,
                         const int32_t* bw, const int32_t* owner, bool bwd, char* ws,
                         const WsLayout& L, int32_t* status, hipStream_t st) {
  SchedArgs s{};
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
  s.status = status;
  const size_t lds = sched_lds(z, bwd);
  (void)hipFuncSetAttribute((const void*)k_sched, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sched_lds(z, true));
  hipLaunchKernelGGL(k_sched, dim3(1), dim3(256), lds, st, s);
}

static ExecArgs make_exec(const Sizes& z, const LayerPtrs& Lp, char* ws, const WsLayout& L) {
  ExecArgs a{};
  a.w1 = Lp.w1; a.w2 = Lp.w2; a.w1s = Lp.w1s; a.w2s = Lp.w2s;
  a.T = z.T; a.k = z.k; a.E = z.E; a.d = z.d; a.dff = z.dff; a.P = z.P; a.s = z.s;
  a.mt = (const int4*)(ws + L.mt);
  a.mt_cnt = (const int32_t*)(ws + L.mt_cnt);
  a.max_mt = (int)z.max_mt;
  a.seg = (const int4*)(ws + L.seg);
  a.seg_cnt = (const int32_t*)(ws + L.seg_cnt);
  a.rep_slot = (const int32_t*)(ws + L.rep_slot);
  a.owner_has = (const int32_t*)(ws + L.owner_has);
  a.ctr = (int32_t*)(ws + L.ctr);
  a.bufA = ws + L.bufA;
  a.bufO = ws + L.bufO;
  a.rslots = (float*)(ws + L.rslots);
  a.bufP = ws + L.bufP;
  a.slots = z.max_slots;
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
  const long long nth = (long long)z.T * (z.d / Elem<T>::VE);
  if (nth > 0)
    hipLaunchKernelGGL(k_combine<T>, dim3((unsigned)((nth + 255) / 256)), dim3(256), 0, st,
                       (const T*)a.bufO, row_to_slot, z.T, z.k, z.d, (T*)y);
  rec(ev, 4, st);
}

// The two-workgroup kernels: bf16, 256 | d and 128 | d_ff (every M/N tile
// extent), and every operand addressed through a buffer descriptor below 2 GiB.
bool use_dual(const Sizes& z) {
  const size_t lim = (size_t)1 << 31;
  return z.act_bytes == 2 && z.d % 256 == 0 && z.dff % 128 == 0 &&
         (size_t)z.T * z.d * 2 < lim && z.max_slots * 4 * (size_t)z.dff < lim &&
         z.max_slots * 2 * (size_t)z.d < lim && (size_t)4 * z.dff * z.d < lim;
}

template <class E>
static void run_forward_eng(const Sizes& z, ExecArgs& a, const int32_t* row_to_slot, void* y,
                            void* const* ev, hipStream_t st) {
  using C = typename E::C;
  const size_t lds = E::LDS;
  static int g1 = persistent_grid(k_fc1_t<E>, C::NT, lds);
  static int g2 = persistent_grid(k_fc2_t<E>, C::NT, lds);
  hipLaunchKernelGGL(k_fc1_t<E>, dim3(g1), dim3(C::NT), lds, st, a);
  rec(ev, 2, st);
  hipLaunchKernelGGL(k_fc2_t<E>, dim3(g2), dim3(C::NT), lds, st, a);
  rec(ev, 3, st);
  const long long nth = (long long)z.T * (z.d / 8);
  if (nth > 0)
    hipLaunchKernelGGL(k_combine<uint16_t>, dim3((unsigned)((nth + 255) / 256)), dim3(256), 0, st,
                       (const uint16_t*)a.bufO, row_to_slot, z.T, z.k, z.d, (uint16_t*)y);
  rec(ev, 4, st);
}

// Engine choice: the wide tile wherever its extents divide the problem
// (256 | d_ff for the backward's d_ff-wide N tiles), else the two-workgroup
// tile.  MOE_FFN_ENGINE=dual|wide forces one (for measurement).
static int engine_override() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("MOE_FFN_ENGINE");
    v = (e && !strcmp(e, "dual")) ? 1 : (e && !strcmp(e, "wide")) ? 2 : 0;
  }
  return v;
}
static bool wide_fwd(const Sizes& z) { return engine_override() != 1; }
static bool wide_bwd(const Sizes& z) { return engine_override() != 1 && z.dff % 256 == 0; }

static void run_forward_sel(const Sizes& z, ExecArgs& a, const int32_t* row_to_slot, void* y,
                            void* const* ev, hipStream_t st) {
  if (wide_fwd(z)) run_forward_eng<EngWide>(z, a, row_to_slot, y, ev, st);
  else run_forward_eng<EngDual>(z, a, row_to_slot, y, ev, st);
}

int launch_forward(const Sizes& z, const LayerPtrs& Lp, const void* x, const float* gates,
                   const int32_t* counts, const int32_t* boff, const int32_t* row_to_slot,
                   const int32_t* slot_to_row, const int32_t* block_worker, void* y,
                   void* z_save, int32_t* status, char* ws, void* const* ev, hipStream_t st) {
  const WsLayout L = exec_layout(z, false);
  rec(ev, 0, st);
  launch_sched(z, counts, boff, block_worker, nullptr, false, ws, L, status, st);
  rec(ev, 1, st);
  ExecArgs a = make_exec(z, Lp, ws, L);
  a.x = x; a.gates = gates; a.slot_to_row = slot_to_row; a.row_to_slot = row_to_slot;
  a.z_save = z_save;
  const bool big = use_big_tiles(z);
  if (Lp.act_dtype == MOE_BF16 && Lp.w_dtype == MOE_BF16 && use_dual(z)) run_forward_sel(z, a, row_to_slot, y, ev, st);
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

// The two-workgroup backward also needs token indices that fit the 16-bit
// LDS table of the weight-gradient kernel.
bool use_dma_backward(const Sizes& z) { return use_dual(z) && z.T <= 65535; }

template <class E, class EW>
static void run_backward_eng(const Sizes& z, ExecArgs& a, const int32_t* row_to_slot, void* dx,
                             float* dw1, float* dw2, void* const* ev, hipStream_t st) {
  using C = typename E::C;
  const size_t glds = E::LDS;
  const size_t wlds = DwEng<EW>::LDS_BYTES;
  static int ga = persistent_grid(k_bwd_da_t<E>, C::NT, glds);
  static int gx = persistent_grid(k_bwd_dx_t<E>, C::NT, glds);
  static int gw = persistent_grid(k_bwd_dw_t<EW>, EW::C::NT, wlds);
  hipLaunchKernelGGL(k_bwd_da_t<E>, dim3(ga), dim3(C::NT), glds, st, a);
  rec(ev, 2, st);
  hipLaunchKernelGGL(k_bwd_dx_t<E>, dim3(gx), dim3(C::NT), glds, st, a);
  rec(ev, 3, st);
  const long long nth = (long long)z.T * (z.d / 8);
  if (nth > 0)
    hipLaunchKernelGGL(k_combine<uint16_t>, dim3((unsigned)((nth + 255) / 256)), dim3(256), 0, st,
                       (const uint16_t*)a.bufO, row_to_slot, z.T, z.k, z.d, (uint16_t*)dx);
  rec(ev, 4, st);
  hipLaunchKernelGGL(k_bwd_dw_t<EW>, dim3(gw), dim3(EW::C::NT), wlds, st, a);
  rec(ev, 5, st);
  hipLaunchKernelGGL(k_bwd_reduce, dim3(num_cus() * 4), dim3(256), 0, st, a.rep_slot,
                     a.owner_has, (const float*)a.rslots, z.E, z.P, z.d, z.dff, dw1, dw2);
  rec(ev, 6, st);
}

static void run_backward_sel(const Sizes& z, ExecArgs& a, const int32_t* row_to_slot, void* dx,
                             float* dw1, float* dw2, void* const* ev, hipStream_t st) {
  if (wide_bwd(z)) run_backward_eng<EngWide, EngWide>(z, a, row_to_slot, dx, dw1, dw2, ev, st);
  else run_backward_eng<EngDual, EngDual>(z, a, row_to_slot, dx, dw1, dw2, ev, st);
}

template <typename T, class C>
static void run_backward(const Sizes& z, ExecArgs& a, const int32_t* row_to_slot, void* dx,
                         float* dw1, float* dw2, void* const* ev, hipStream_t st) {
  a.bufP = nullptr;
  const size_t lds = gemm_lds_bytes<T, C>();
  static int ga = persistent_grid(k_bwd_da<T, C>, C::NT, lds);
  static int gx = persistent_grid(k_bwd_dx<T, C>, C::NT, lds);
  static int gw = persistent_grid(k_bwd_dw<T, C>, C::NT, lds);
  hipLaunchKernelGGL((k_bwd_da<T, C>), dim3(ga), dim3(C::NT), lds, st, a);
  rec(ev, 2, st);
  hipLaunchKernelGGL((k_bwd_dx<T, C>), dim3(gx), dim3(C::NT), lds, st, a);
  rec(ev, 3, st);
  const long long nth = (long long)z.T * (z.d / Elem<T>::VE);
  if (nth > 0)
    hipLaunchKernelGGL(k_combine<T>, dim3((unsigned)((nth + 255) / 256)), dim3(256), 0, st,
                       (const T*)a.bufO, row_to_slot, z.T, z.k, z.d, (T*)dx);
  rec(ev, 4, st);
  hipLaunchKernelGGL((k_bwd_dw<T, C>), dim3(gw), dim3(C::NT), lds, st, a);
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
                    int32_t* status, char* ws, void* const* ev, hipStream_t st) {
  const WsLayout L = exec_layout(z, true);
  rec(ev, 0, st);
  launch_sched(z, counts, boff, block_worker, owner, true, ws, L, status, st);
  rec(ev, 1, st);
  ExecArgs a = make_exec(z, Lp, ws, L);
  a.x = x; a.gates = gates; a.slot_to_row = slot_to_row; a.row_to_slot = row_to_slot;
  a.z_save = const_cast<void*>(z_save);
  a.dy = dy; a.dw1 = dw1; a.dw2 = dw2;
  if (Lp.act_dtype == MOE_F32) run_backward<float, SmallCfg>(z, a, row_to_slot, dx, dw1, dw2, ev, st);
  else if (use_dma_backward(z)) run_backward_sel(z, a, row_to_slot, dx, dw1, dw2, ev, st);
  else if (use_big_tiles(z)) run_backward<uint16_t, BigCfg>(z, a, row_to_slot, dx, dw1, dw2, ev, st);
  else run_backward<uint16_t, SmallCfg>(z, a, row_to_slot, dx, dw1, dw2, ev, st);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
