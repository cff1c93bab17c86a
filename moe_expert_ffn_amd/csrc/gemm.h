// One 128x128 output tile of C = A * B on CDNA4 matrix cores.
//
// 256 threads = 4 waves in a 2x2 grid, each wave owning a 64x64 sub-tile as
// 2x2 blocks of 32x32 MFMA accumulators (16 fp32 per lane each).  Operands are
// staged through LDS in a K-contiguous layout, [row][BK + pad], double
// buffered: the global loads of K-tile kt+1 are in flight while the waves run
// the MFMAs of K-tile kt, and one barrier per K-tile separates the two
// buffers.  Row stride is BK*size + 16 bytes, so the 16-byte fragment reads of
// the 32 lanes of one half-wave land on distinct bank groups.
//
// Element types: bf16 (raw uint16_t) uses v_mfma_f32_32x32x16_bf16 (8 values
// per lane per operand, BK = 64); fp32 uses v_mfma_f32_32x32x2_f32 (BK = 32).
// Each lane of an MFMA operand holds a run of consecutive K values; both
// operands use the same K assignment, so the contraction is exact in order of
// the hardware's accumulation.
//
// Operand loaders come in two shapes:
//   RowLoad   -- the tile's rows are contiguous along K in memory (activation
//                rows, gathered through a row table, and weight rows);
//   TransLoad -- the source is contiguous along the tile's M/N axis and K
//                walks its rows (the transposed operands of the backward
//                pass); each thread reads a 4(K) x VE(MN) block with 16-byte
//                loads and writes it to LDS transposed.
#pragma once

#include "common.h"
#include "internal.h"

namespace moe {

template <typename T> struct Elem;
template <> struct Elem<uint16_t> { static constexpr int VE = 8, BK = 64; };
template <> struct Elem<float> { static constexpr int VE = 4, BK = 32; };

template <typename T> struct TileCfg {
  static constexpr int VE = Elem<T>::VE, BK = Elem<T>::BK;
  static constexpr int LDK = BK + VE;               // +16 bytes
  static constexpr int KC = 2 * VE;                 // K per MFMA chunk
  static constexpr int NKC = BK / KC;
  static constexpr int A_ELEMS = kBM * LDK, B_ELEMS = kBN * LDK;
  static constexpr size_t LDS_BYTES = 2 * (size_t)(A_ELEMS + B_ELEMS) * sizeof(T);
};

union V16 {
  uint4 u;
  uint16_t h[8];
  float f[4];
  uint8_t b[16];
};

MOE_DEV uint4 zero4() { return make_uint4(0, 0, 0, 0); }

// ---- MFMA on one K chunk of the staged tile -------------------------------
MOE_DEV void mma_chunk(f32x16_t (&acc)[2][2], const uint16_t* sA, const uint16_t* sB, int wm,
                       int wn, int kc, int lane) {
  constexpr int LDK = TileCfg<uint16_t>::LDK;
  const int ko = kc * 16 + (lane >> 5) * 8;
  bf16x8_t a[2], b[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    a[i] = *(const bf16x8_t*)(sA + (wm * 64 + i * 32 + (lane & 31)) * LDK + ko);
    b[i] = *(const bf16x8_t*)(sB + (wn * 64 + i * 32 + (lane & 31)) * LDK + ko);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

MOE_DEV void mma_chunk(f32x16_t (&acc)[2][2], const float* sA, const float* sB, int wm, int wn,
                       int kc, int lane) {
  constexpr int LDK = TileCfg<float>::LDK;
  const int ko = kc * 8 + (lane >> 5) * 4;
  f32x4_t a[2], b[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    a[i] = *(const f32x4_t*)(sA + (wm * 64 + i * 32 + (lane & 31)) * LDK + ko);
    b[i] = *(const f32x4_t*)(sB + (wn * 64 + i * 32 + (lane & 31)) * LDK + ko);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][v], b[j][v], acc[i][j], 0, 0, 0);
}

// ---- loaders ---------------------------------------------------------------
// K-contiguous rows.  rowptr(row) returns the row's first element (K index 0)
// or nullptr for a row that reads as zeros.
template <typename T, int ROWS> struct RowLoad {
  static constexpr int VE = Elem<T>::VE, BK = Elem<T>::BK, LDK = TileCfg<T>::LDK;
  static constexpr int CPR = BK / VE;               // 16-byte chunks per row
  static constexpr int NCH = ROWS * CPR / 256;
  const T* ptr[NCH];
  int soff[NCH];
  uint4 v[NCH];
  template <class F> MOE_DEV void init(F rowptr) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int row = c / CPR, col = (c % CPR) * VE;
      const T* p = rowptr(row);
      ptr[i] = p ? p + col : nullptr;
      soff[i] = row * LDK + col;
    }
  }
  MOE_DEV void load(int kt) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) v[i] = ptr[i] ? *(const uint4*)(ptr[i] + (size_t)kt * BK) : zero4();
  }
  MOE_DEV void store(T* s) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) *(uint4*)(s + soff[i]) = v[i];
  }
};

// e4m3 weight rows with one fp32 scale per 128x128 block, widened to bf16 on
// the way into LDS.  rowptr(row) gives the row's codes, rowscale(row) the
// scale row of its 128-row block (indexed by K/128).
template <int ROWS> struct RowLoadFp8 {
  static constexpr int BK = 64, LDK = TileCfg<uint16_t>::LDK;
  static constexpr int CPR = BK / 16;               // 16 codes per 16-byte chunk
  static constexpr int NCH = ROWS * CPR / 256;
  const uint8_t* ptr[NCH];
  const float* sc[NCH];
  int soff[NCH];
  uint4 v[NCH];
  float s[NCH];
  template <class F, class G> MOE_DEV void init(F rowptr, G rowscale) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int row = c / CPR, col = (c % CPR) * 16;
      const uint8_t* p = rowptr(row);
      ptr[i] = p ? p + col : nullptr;
      sc[i] = rowscale(row);
      soff[i] = row * LDK + col;
    }
  }
  MOE_DEV void load(int kt) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      v[i] = ptr[i] ? *(const uint4*)(ptr[i] + (size_t)kt * BK) : zero4();
      s[i] = ptr[i] ? sc[i][(kt * BK) >> 7] : 0.f;
    }
  }
  MOE_DEV void store(uint16_t* sm) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      V16 in, o0, o1;
      in.u = v[i];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        o0.h[j] = f2bf(e4m3_to_f32(in.b[j]) * s[i]);
        o1.h[j] = f2bf(e4m3_to_f32(in.b[8 + j]) * s[i]);
      }
      *(uint4*)(sm + soff[i]) = o0.u;
      *(uint4*)(sm + soff[i] + 8) = o1.u;
    }
  }
};

// Source contiguous along the tile's ROWS axis (M or N); K walks source rows.
// src(k, mn) returns 16 bytes = VE elements at (k, mn..mn+VE-1), zeros when
// out of range.  Thread t covers K rows k0..k0+3 and MN columns mn0..mn0+VE-1.
template <typename T, int ROWS> struct TransLoad {
  static constexpr int VE = Elem<T>::VE, BK = Elem<T>::BK, LDK = TileCfg<T>::LDK;
  static constexpr int MNG = ROWS / VE;
  static constexpr int KSUB = 4;
  static_assert(MNG * (BK / KSUB) == 256, "one 4 x VE block per thread");
  int mn0, k0;
  uint4 v[KSUB];
  MOE_DEV void init() {
    mn0 = (threadIdx.x % MNG) * VE;
    k0 = (threadIdx.x / MNG) * KSUB;
  }
  template <class S> MOE_DEV void load(int kt, S& src) {
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk) v[kk] = src(kt * BK + k0 + kk, mn0);
  }
  MOE_DEV void store(T* s) {
    if constexpr (sizeof(T) == 2) {
      V16 in[KSUB];
#pragma unroll
      for (int kk = 0; kk < KSUB; ++kk) in[kk].u = v[kk];
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        uint2 o;
        o.x = (uint32_t)in[0].h[e] | ((uint32_t)in[1].h[e] << 16);
        o.y = (uint32_t)in[2].h[e] | ((uint32_t)in[3].h[e] << 16);
        *(uint2*)(s + (mn0 + e) * LDK + k0) = o;
      }
    } else {
      V16 in[KSUB];
#pragma unroll
      for (int kk = 0; kk < KSUB; ++kk) in[kk].u = v[kk];
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        V16 o;
#pragma unroll
        for (int kk = 0; kk < KSUB; ++kk) o.f[kk] = in[kk].f[e];
        *(uint4*)(s + (mn0 + e) * LDK + k0) = o.u;
      }
    }
  }
};

// Loader adapters so the main loop can drive both kinds uniformly.
template <class L> struct PlainLd {
  L& l;
  MOE_DEV void load(int kt) { l.load(kt); }
  template <typename T> MOE_DEV void store(T* s) { l.store(s); }
};
template <class L, class S> struct TransLd {
  L& l;
  S& src;
  MOE_DEV void load(int kt) { l.load(kt, src); }
  template <typename T> MOE_DEV void store(T* s) { l.store(s); }
};

// ---- main loop ----------------------------------------------------------------
template <typename T, class LA, class LB>
MOE_DEV void gemm_tile(LA la, LB lb, int nk, T* smem, f32x16_t (&acc)[2][2]) {
  using C = TileCfg<T>;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = wv >> 1, wn = wv & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  if (nk <= 0) return;
  T* sA[2] = {smem, smem + C::A_ELEMS + C::B_ELEMS};
  T* sB[2] = {smem + C::A_ELEMS, smem + 2 * C::A_ELEMS + C::B_ELEMS};
  la.load(0);
  lb.load(0);
  la.store(sA[0]);
  lb.store(sB[0]);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(kt + 1);
      lb.load(kt + 1);
    }
#pragma unroll
    for (int kc = 0; kc < C::NKC; ++kc) mma_chunk(acc, sA[cur], sB[cur], wm, wn, kc, lane);
    if (more) {
      la.store(sA[cur ^ 1]);
      lb.store(sB[cur ^ 1]);
    }
    __syncthreads();
  }
}

// Coordinates of accumulator register r of block (i, j) for this lane.
MOE_DEV int acc_row(int i, int r, int lane) {
  const int wm = (threadIdx.x >> 6) >> 1;
  return wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}
MOE_DEV int acc_col(int j, int lane) {
  const int wn = (threadIdx.x >> 6) & 1;
  return wn * 64 + j * 32 + (lane & 31);
}

template <typename T> MOE_DEV T to_act(float f);
template <> MOE_DEV uint16_t to_act<uint16_t>(float f) { return f2bf(f); }
template <> MOE_DEV float to_act<float>(float f) { return f; }
MOE_DEV float from_act(uint16_t h) { return bf2f(h); }
MOE_DEV float from_act(float f) { return f; }

// Next tile of this worker's queue, shared with the whole workgroup.
MOE_DEV int next_tile(int32_t* ctr, int* slot) {
  if (threadIdx.x == 0) *slot = atomicAdd(ctr, 1);
  __syncthreads();
  const int t = *slot;
  __syncthreads();
  return t;
}

}  // namespace moe
