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
#include "moe_ffn.h"

namespace moe {

struct SchedArgs {
  const int32_t* counts;
  const int32_t* boff;
  const int32_t* bw;
  const int32_t* owner;
  int E, P, s, beta, backward;
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

// One workgroup.  M-tiles: every block of beta slots spawns ceil(valid/128)
// tiles on its worker, listed per worker in block order (one exclusive scan
// per worker).  Segments (backward): the blocks of one (expert, worker) pair
// must form one contiguous run; its slot range and valid-row count become one
// weight-gradient segment, with a replica slot when the worker is not the
// owner (rank among that worker's non-home experts, in expert order).
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
  for (int r = wv; r < P; r += 4) {
    int run = 0;
    for (int base = 0; base < nb; base += 64) {
      const int g = base + lane;
      int nt = 0, e = 0, bstart = 0, vrows = 0;
      if (g < nb && a.bw[g] == r) {
        e = expert_of(g, boff_s, E);
        bstart = a.beta * g;
        vrows = min(a.beta, a.beta * boff_s[e] + cnt_s[e] - bstart);
        nt = (vrows + kBM - 1) / kBM;
      }
      const int inc = wave_incl_scan(nt);
      const int pos = run + inc - nt;
      for (int i = 0; i < nt; ++i)
        a.mt[(size_t)r * a.max_mt + pos + i] =
            make_int4(e, bstart + i * kBM, min(kBM, vrows - i * kBM), 0);
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
};

enum { PH_FC1 = 0, PH_FC2 = 1, PH_DA = 2, PH_DX = 3, PH_DW = 4 };

// ---- forward: FC1 + SwiGLU ------------------------------------------------
// N-tile nj covers A columns [64 nj, 64 nj + 64); its 128 weight rows
// interleave 32 G rows and the matching 32 U rows, so each wave holds G and U
// of the same (row, column) in two accumulators and applies SwiGLU in
// registers.
template <typename T, bool FP8>
__global__ __launch_bounds__(256) void k_fc1(ExecArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int tslot;
  T* smem = (T*)smem_raw;
  const int r = worker_of_block(a.P);
  const int nnt = a.dff / 64;
  const int total = a.mt_cnt[r] * nnt;
  const int lane = threadIdx.x & 63;
  const T* X = (const T*)a.x;
  T* Ab = (T*)a.bufA;
  T* Z = (T*)a.z_save;
  while (true) {
    const int tile = next_tile(&a.ctr[PH_FC1 * kMaxP + r], &tslot);
    if (tile >= total) break;
    const int4 m = a.mt[(size_t)r * a.max_mt + tile / nnt];
    const int nj = tile % nnt;
    const int e = m.x, slot0 = m.y, nrows = m.z;
    RowLoad<T, kBM> la;
    la.init([&](int row) -> const T* {
      if (row >= nrows) return nullptr;
      return X + (size_t)(a.slot_to_row[slot0 + row] / a.k) * a.d;
    });
    auto w1row = [&](int rho) {
      const int q = rho >> 5;
      return (q & 1) * a.dff + nj * 64 + (q >> 1) * 32 + (rho & 31);
    };
    f32x16_t acc[2][2];
    const int nk = a.d / Elem<T>::BK;
    if constexpr (FP8) {
      RowLoadFp8<kBN> lb;
      const uint8_t* W = (const uint8_t*)a.w1 + (size_t)e * 2 * a.dff * a.d;
      const float* S = a.w1s + (size_t)e * (2 * a.dff / 128) * (a.d / 128);
      lb.init([&](int rho) { return W + (size_t)w1row(rho) * a.d; },
              [&](int rho) { return S + (size_t)(w1row(rho) >> 7) * (a.d >> 7); });
      gemm_tile<T>(PlainLd<RowLoad<T, kBM>>{la}, PlainLd<RowLoadFp8<kBN>>{lb}, nk, smem, acc);
    } else {
      RowLoad<T, kBN> lb;
      const T* W = (const T*)a.w1 + (size_t)e * 2 * a.dff * a.d;
      lb.init([&](int rho) -> const T* { return W + (size_t)w1row(rho) * a.d; });
      gemm_tile<T>(PlainLd<RowLoad<T, kBM>>{la}, PlainLd<RowLoad<T, kBN>>{lb}, nk, smem, acc);
    }
    const int c = nj * 64 + ((threadIdx.x >> 6) & 1) * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = acc_row(i, rr, lane);
        if (row < nrows) {
          const float g = acc[i][0][rr], u = acc[i][1][rr];
          const float av = g / (1.f + expf(-g)) * u;
          const size_t slot = (size_t)slot0 + row;
          Ab[slot * a.dff + c] = to_act<T>(av);
          if (Z) {
            Z[slot * 2 * a.dff + c] = to_act<T>(g);
            Z[slot * 2 * a.dff + a.dff + c] = to_act<T>(u);
          }
        }
      }
  }
}

// ---- forward: FC2 + gate ----------------------------------------------------
template <typename T, bool FP8>
__global__ __launch_bounds__(256) void k_fc2(ExecArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int tslot;
  __shared__ float pg[kBM];
  T* smem = (T*)smem_raw;
  const int r = worker_of_block(a.P);
  const int nnt = a.d / kBN;
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
    if (threadIdx.x < kBM)
      pg[threadIdx.x] = threadIdx.x < nrows ? a.gates[a.slot_to_row[slot0 + threadIdx.x]] : 0.f;
    RowLoad<T, kBM> la;
    la.init([&](int row) -> const T* {
      return row < nrows ? Ab + ((size_t)slot0 + row) * a.dff : nullptr;
    });
    f32x16_t acc[2][2];
    const int nk = a.dff / Elem<T>::BK;
    if constexpr (FP8) {
      RowLoadFp8<kBN> lb;
      const uint8_t* W = (const uint8_t*)a.w2 + (size_t)e * a.d * a.dff;
      const float* S = a.w2s + (size_t)e * (a.d / 128) * (a.dff / 128);
      lb.init([&](int rho) { return W + (size_t)(nj * kBN + rho) * a.dff; },
              [&](int rho) { return S + (size_t)((nj * kBN + rho) >> 7) * (a.dff >> 7); });
      gemm_tile<T>(PlainLd<RowLoad<T, kBM>>{la}, PlainLd<RowLoadFp8<kBN>>{lb}, nk, smem, acc);
    } else {
      RowLoad<T, kBN> lb;
      const T* W = (const T*)a.w2 + (size_t)e * a.d * a.dff;
      lb.init([&](int rho) -> const T* { return W + (size_t)(nj * kBN + rho) * a.dff; });
      gemm_tile<T>(PlainLd<RowLoad<T, kBM>>{la}, PlainLd<RowLoad<T, kBN>>{lb}, nk, smem, acc);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = acc_row(i, rr, lane);
        if (row < nrows) {
          const float p = pg[row];
          const size_t base = ((size_t)slot0 + row) * a.d + nj * kBN;
#pragma unroll
          for (int j = 0; j < 2; ++j) O[base + acc_col(j, lane)] = to_act<T>(p * acc[i][j][rr]);
        }
      }
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
    in.u = *(const uint4*)(src + (size_t)s * d + c);
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
  *(uint4*)(out + (size_t)t * d + c) = o.u;
}

// ---- backward: dA -> dZ -------------------------------------------------------
// dA[slot, n] = p * sum_c dy[t, c] W2[c, n]; W2 is read as a K-major (c) by
// N-contiguous operand and transposed into LDS.
template <typename T> struct SrcRowsMN {       // element (k, n) = base[k * ld + n0 + n]
  const T* base;
  int ld, n0, nlim;
  MOE_DEV uint4 operator()(int kk, int mn) const {
    const int n = n0 + mn;
    return n < nlim ? *(const uint4*)(base + (size_t)kk * ld + n) : zero4();
  }
};

template <typename T>
__global__ __launch_bounds__(256) void k_bwd_da(ExecArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int tslot;
  __shared__ float pg[kBM];
  T* smem = (T*)smem_raw;
  const int r = worker_of_block(a.P);
  const int nnt = (a.dff + kBN - 1) / kBN;
  const int total = a.mt_cnt[r] * nnt;
  const int lane = threadIdx.x & 63;
  const T* DY = (const T*)a.dy;
  const T* Z = (const T*)a.z_save;
  T* dZ = (T*)a.bufA;
  while (true) {
    const int tile = next_tile(&a.ctr[PH_DA * kMaxP + r], &tslot);
    if (tile >= total) break;
    const int4 m = a.mt[(size_t)r * a.max_mt + tile / nnt];
    const int nj = tile % nnt;
    const int e = m.x, slot0 = m.y, nrows = m.z;
    if (threadIdx.x < kBM)
      pg[threadIdx.x] = threadIdx.x < nrows ? a.gates[a.slot_to_row[slot0 + threadIdx.x]] : 0.f;
    RowLoad<T, kBM> la;
    la.init([&](int row) -> const T* {
      if (row >= nrows) return nullptr;
      return DY + (size_t)(a.slot_to_row[slot0 + row] / a.k) * a.d;
    });
    TransLoad<T, kBN> lb;
    lb.init();
    SrcRowsMN<T> src{(const T*)a.w2 + (size_t)e * a.d * a.dff, a.dff, nj * kBN, a.dff};
    f32x16_t acc[2][2];
    gemm_tile<T>(PlainLd<RowLoad<T, kBM>>{la}, TransLd<TransLoad<T, kBN>, SrcRowsMN<T>>{lb, src},
                 a.d / Elem<T>::BK, smem, acc);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = acc_row(i, rr, lane);
        if (row >= nrows) continue;
        const float p = pg[row];
        const size_t zb = ((size_t)slot0 + row) * 2 * a.dff;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = nj * kBN + acc_col(j, lane);
          if (n >= a.dff) continue;
          const float dA = p * acc[i][j][rr];
          const float g = from_act(Z[zb + n]), u = from_act(Z[zb + a.dff + n]);
          const float sg = 1.f / (1.f + expf(-g));
          dZ[zb + n] = to_act<T>(dA * u * sg * (1.f + g * (1.f - sg)));
          dZ[zb + a.dff + n] = to_act<T>(dA * g * sg);
        }
      }
  }
}

// ---- backward: dX per routed row ----------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_bwd_dx(ExecArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int tslot;
  T* smem = (T*)smem_raw;
  const int r = worker_of_block(a.P);
  const int nnt = a.d / kBN;
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
    RowLoad<T, kBM> la;
    la.init([&](int row) -> const T* {
      return row < nrows ? dZ + ((size_t)slot0 + row) * 2 * a.dff : nullptr;
    });
    TransLoad<T, kBN> lb;
    lb.init();
    SrcRowsMN<T> src{(const T*)a.w1 + (size_t)e * 2 * a.dff * a.d, a.d, nj * kBN, a.d};
    f32x16_t acc[2][2];
    gemm_tile<T>(PlainLd<RowLoad<T, kBM>>{la}, TransLd<TransLoad<T, kBN>, SrcRowsMN<T>>{lb, src},
                 2 * a.dff / Elem<T>::BK, smem, acc);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = acc_row(i, rr, lane);
        if (row >= nrows) continue;
        const size_t base = ((size_t)slot0 + row) * a.d + nj * kBN;
#pragma unroll
        for (int j = 0; j < 2; ++j) dXp[base + acc_col(j, lane)] = to_act<T>(acc[i][j][rr]);
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
    return *(const uint4*)(base + (size_t)t * ld + m);
  }
};
template <typename T> struct SrcSlotRow {      // element (k, m) = base[(slot0 + k) * ld + m0 + m]
  const T* base;
  int slot0, nrows, ld, m0, mlim;
  MOE_DEV uint4 operator()(int kk, int mn) const {
    const int m = m0 + mn;
    if (kk >= nrows || m >= mlim) return zero4();
    return *(const uint4*)(base + ((size_t)slot0 + kk) * ld + m);
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
    g.u = *(const uint4*)(z + zb + n);
    u.u = *(const uint4*)(z + zb + dff + n);
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

template <typename T>
__global__ __launch_bounds__(256) void k_bwd_dw(ExecArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int tslot;
  T* smem = (T*)smem_raw;
  const int r = worker_of_block(a.P);
  const int n2m = a.d / kBM, n2n = (a.dff + kBN - 1) / kBN;   // dW2 [d][dff]
  const int n1m = 2 * a.dff / kBM, n1n = a.d / kBN;          // dW1 [2dff][d]
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
    f32x16_t acc[2][2];
    TransLoad<T, kBM> la;
    TransLoad<T, kBN> lb;
    la.init();
    lb.init();
    float* out;
    int ldo, mi, nj, nlim;
    if (loc < n2m * n2n) {
      mi = loc / n2n;
      nj = loc % n2n;
      SrcGatherRow<T> sa{(const T*)a.dy, a.slot_to_row, slot0, nrows, a.k, a.d, mi * kBM, a.d};
      SrcGatedAct<T> sb{(const T*)a.z_save, a.gates, a.slot_to_row, slot0, nrows, a.dff, nj * kBN};
      gemm_tile<T>(TransLd<TransLoad<T, kBM>, SrcGatherRow<T>>{la, sa},
                   TransLd<TransLoad<T, kBN>, SrcGatedAct<T>>{lb, sb}, nk, smem, acc);
      out = (dst < 0 ? a.dw2 + (size_t)e * a.d * a.dff
                     : a.rslots + (size_t)dst * w_elems + (size_t)2 * a.dff * a.d);
      ldo = a.dff;
      nlim = a.dff;
    } else {
      loc -= n2m * n2n;
      mi = loc / n1n;
      nj = loc % n1n;
      SrcSlotRow<T> sa{(const T*)a.bufA, slot0, nrows, 2 * a.dff, mi * kBM, 2 * a.dff};
      SrcGatherRow<T> sb{(const T*)a.x, a.slot_to_row, slot0, nrows, a.k, a.d, nj * kBN, a.d};
      gemm_tile<T>(TransLd<TransLoad<T, kBM>, SrcSlotRow<T>>{la, sa},
                   TransLd<TransLoad<T, kBN>, SrcGatherRow<T>>{lb, sb}, nk, smem, acc);
      out = (dst < 0 ? a.dw1 + (size_t)e * 2 * a.dff * a.d : a.rslots + (size_t)dst * w_elems);
      ldo = a.d;
      nlim = a.d;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const size_t row = (size_t)mi * kBM + acc_row(i, rr, lane);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = nj * kBN + acc_col(j, lane);
          if (n < nlim) out[row * ldo + n] = acc[i][j][rr];
        }
      }
  }
}

// Owner slot <- (owner partial or 0) + replica partials in ascending worker
// order, fp32.  Experts with an owner partial and no replica are untouched.
__global__ __launch_bounds__(256) void k_bwd_reduce(const int32_t* __restrict__ rep_slot,
                                                    const int32_t* __restrict__ owner_has,
                                                    const float* __restrict__ rslots, int E,
                                                    int P, int d, int dff, float* dw1,
                                                    float* dw2) {
  const size_t n1 = (size_t)2 * dff * d, n2 = (size_t)d * dff, w_elems = n1 + n2;
  const size_t nvec = w_elems / 4;
  for (int e = 0; e < E; ++e) {
    int slots[kMaxP];
    int nrep = 0;
    for (int w = 0; w < P; ++w) {
      const int sl = rep_slot[e * P + w];
      if (sl >= 0) slots[nrep++] = sl;
    }
    const bool own = owner_has[e] != 0;
    if (own && nrep == 0) continue;
    for (size_t v = (size_t)blockIdx.x * 256 + threadIdx.x; v < nvec; v += (size_t)gridDim.x * 256) {
      const size_t i = v * 4;
      float* dst = (i < n1) ? dw1 + (size_t)e * n1 + i : dw2 + (size_t)e * n2 + (i - n1);
      float4 accv = own ? *(const float4*)dst : make_float4(0.f, 0.f, 0.f, 0.f);
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
  L.total = o;
  return L;
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

template <typename K> static int persistent_grid(K kernel, size_t lds) {
  static_assert(sizeof(K) > 0, "");
  (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds);
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, lds) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  int g = num_cus() * per_cu;
  g = (g / kXcds) * kXcds;
  return g < kXcds ? kXcds : g;
}

int gemm_wg_per_cu() {
  const size_t lds = TileCfg<uint16_t>::LDS_BYTES;
  return persistent_grid(k_fc1<uint16_t, false>, lds) / num_cus();
}

static void rec(void* const* ev, int i, hipStream_t st) {
  if (ev && ev[i]) (void)hipEventRecord((hipEvent_t)ev[i], st);
}

static size_t sched_lds(const Sizes& z, bool bwd) {
  return sizeof(int) * ((size_t)2 * z.E + 1 + (bwd ? (size_t)3 * z.E * z.P : 0));
}

static SchedArgs make_sched(const Sizes& z, const int32_t* counts, const int32_t* boff,
                            const int32_t* bw, const int32_t* owner, bool bwd, char* ws,
                            const WsLayout& L, int32_t* status) {
  SchedArgs s{};
  s.counts = counts; s.boff = boff; s.bw = bw; s.owner = owner;
  s.E = z.E; s.P = z.P; s.s = z.s; s.beta = z.beta; s.backward = bwd ? 1 : 0;
  s.ctr = (int32_t*)(ws + L.ctr);
  s.mt_cnt = (int32_t*)(ws + L.mt_cnt);
  s.mt = (int4*)(ws + L.mt);
  s.max_mt = (int)z.max_mt;
  s.seg_cnt = (int32_t*)(ws + L.seg_cnt);
  s.seg = (int4*)(ws + L.seg);
  s.rep_slot = (int32_t*)(ws + L.rep_slot);
  s.owner_has = (int32_t*)(ws + L.owner_has);
  s.status = status;
  return s;
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
  return a;
}

template <typename T, bool FP8>
static void run_forward(const Sizes& z, ExecArgs& a, const int32_t* row_to_slot, void* y,
                        void* const* ev, hipStream_t st) {
  const size_t lds = TileCfg<T>::LDS_BYTES;
  static int g1 = persistent_grid(k_fc1<T, FP8>, lds);
  static int g2 = persistent_grid(k_fc2<T, FP8>, lds);
  hipLaunchKernelGGL((k_fc1<T, FP8>), dim3(g1), dim3(256), lds, st, a);
  rec(ev, 2, st);
  hipLaunchKernelGGL((k_fc2<T, FP8>), dim3(g2), dim3(256), lds, st, a);
  rec(ev, 3, st);
  const long long nth = (long long)z.T * (z.d / Elem<T>::VE);
  if (nth > 0)
    hipLaunchKernelGGL(k_combine<T>, dim3((unsigned)((nth + 255) / 256)), dim3(256), 0, st,
                       (const T*)a.bufO, row_to_slot, z.T, z.k, z.d, (T*)y);
  rec(ev, 4, st);
}

int launch_forward(const Sizes& z, const LayerPtrs& Lp, const void* x, const float* gates,
                   const int32_t* counts, const int32_t* boff, const int32_t* row_to_slot,
                   const int32_t* slot_to_row, const int32_t* block_worker, void* y,
                   void* z_save, int32_t* status, char* ws, void* const* ev, hipStream_t st) {
  const WsLayout L = exec_layout(z, false);
  rec(ev, 0, st);
  SchedArgs sa = make_sched(z, counts, boff, block_worker, nullptr, false, ws, L, status);
  const size_t slds = sched_lds(z, false);
  (void)hipFuncSetAttribute((const void*)k_sched, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sched_lds(z, true));
  hipLaunchKernelGGL(k_sched, dim3(1), dim3(256), slds, st, sa);
  rec(ev, 1, st);
  ExecArgs a = make_exec(z, Lp, ws, L);
  a.x = x; a.gates = gates; a.slot_to_row = slot_to_row; a.row_to_slot = row_to_slot;
  a.z_save = z_save;
  if (Lp.act_dtype == MOE_F32) run_forward<float, false>(z, a, row_to_slot, y, ev, st);
  else if (Lp.w_dtype == MOE_FP8_E4M3) run_forward<uint16_t, true>(z, a, row_to_slot, y, ev, st);
  else run_forward<uint16_t, false>(z, a, row_to_slot, y, ev, st);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

template <typename T>
static void run_backward(const Sizes& z, ExecArgs& a, const int32_t* row_to_slot, void* dx,
                         float* dw1, float* dw2, void* const* ev, hipStream_t st) {
  const size_t lds = TileCfg<T>::LDS_BYTES;
  static int ga = persistent_grid(k_bwd_da<T>, lds);
  static int gx = persistent_grid(k_bwd_dx<T>, lds);
  static int gw = persistent_grid(k_bwd_dw<T>, lds);
  hipLaunchKernelGGL(k_bwd_da<T>, dim3(ga), dim3(256), lds, st, a);
  rec(ev, 2, st);
  hipLaunchKernelGGL(k_bwd_dx<T>, dim3(gx), dim3(256), lds, st, a);
  rec(ev, 3, st);
  const long long nth = (long long)z.T * (z.d / Elem<T>::VE);
  if (nth > 0)
    hipLaunchKernelGGL(k_combine<T>, dim3((unsigned)((nth + 255) / 256)), dim3(256), 0, st,
                       (const T*)a.bufO, row_to_slot, z.T, z.k, z.d, (T*)dx);
  rec(ev, 4, st);
  hipLaunchKernelGGL(k_bwd_dw<T>, dim3(gw), dim3(256), lds, st, a);
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
  SchedArgs sa = make_sched(z, counts, boff, block_worker, owner, true, ws, L, status);
  const size_t slds = sched_lds(z, true);
  (void)hipFuncSetAttribute((const void*)k_sched, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)slds);
  hipLaunchKernelGGL(k_sched, dim3(1), dim3(256), slds, st, sa);
  rec(ev, 1, st);
  ExecArgs a = make_exec(z, Lp, ws, L);
  a.x = x; a.gates = gates; a.slot_to_row = slot_to_row; a.row_to_slot = row_to_slot;
  a.z_save = const_cast<void*>(z_save);
  a.dy = dy; a.dw1 = dw1; a.dw2 = dw2;
  if (Lp.act_dtype == MOE_F32) run_backward<float>(z, a, row_to_slot, dx, dw1, dw2, ev, st);
  else run_backward<uint16_t>(z, a, row_to_slot, dx, dw1, dw2, ev, st);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
