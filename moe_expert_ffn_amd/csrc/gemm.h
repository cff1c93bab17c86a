// One BM x BN output tile of C = A * B on CDNA4 matrix cores.
//
// Two shapes:
//   Big   -- 256 x 256, 4 waves (2 x 2, each a 128 x 128 sub-tile = 4 x 4
//            blocks of 32x32 MFMA accumulators, 256 accumulator registers per
//            lane); 256 threads, one workgroup per CU, one wave per SIMD with
//            the full 512-register file.  Each 64-wide K step loads 64 KB from
//            L2/HBM for 8.4 MFLOP, twice the reuse of a 128 x 128 tile, and
//            each wave reads 8 KB of LDS per 16 MFMAs.
//   Small -- 128 x 128, 4 waves (2 x 2, each 64 x 64); 256 threads; used when a
//            dimension is not a multiple of 256 or for fp32.
// Operands are staged through LDS in a K-contiguous layout, [row][BK + pad],
// double buffered: the global loads of K step kt+1 are in flight while the
// waves run the MFMAs of step kt; one barrier per step separates the buffers.
// The row stride is BK*size + 16 bytes, so the 16-byte fragment reads of the
// 32 lanes of one half-wave land on distinct bank groups.
//
// Element types: bf16 (raw uint16_t) uses v_mfma_f32_32x32x16_bf16 (8 values
// per lane per operand, BK = 64); fp32 uses v_mfma_f32_32x32x2_f32 (BK = 32).
// Each lane of an MFMA operand holds a run of consecutive K values; both
// operands use the same K assignment, so the contraction is exact up to the
// hardware's accumulation order.
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

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_> struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int MB = WM / 32, NB = WN / 32;
};
using BigCfg = GemmCfg<256, 256, 2, 2>;
using SmallCfg = GemmCfg<128, 128, 2, 2>;

template <typename T> struct Elem;
template <> struct Elem<uint16_t> { static constexpr int VE = 8, BK = 64; };
template <> struct Elem<float> { static constexpr int VE = 4, BK = 32; };

template <typename T, class C> struct TileLds {
  static constexpr int VE = Elem<T>::VE, BK = Elem<T>::BK;
  static constexpr int LDK = BK + VE;               // +16 bytes
  static constexpr int KC = 2 * VE;                 // K per MFMA chunk
  static constexpr int NKC = BK / KC;
  static constexpr int A_ELEMS = C::BM * LDK, B_ELEMS = C::BN * LDK;
  static constexpr size_t BYTES = 2 * (size_t)(A_ELEMS + B_ELEMS) * sizeof(T);
};

union V16 {
  uint4 u;
  uint16_t h[8];
  float f[4];
  uint8_t b[16];
};

MOE_DEV uint4 zero4() { return make_uint4(0, 0, 0, 0); }

// wave index within the workgroup, known to the compiler to be wave-uniform
MOE_DEV int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Lanes of one wave exchanging data through LDS.  The hardware keeps a wave's
// LDS accesses in order, so no wait is needed; the wavefront-scope fences tell
// the compiler that other lanes read and write the memory, so it neither
// reuses a value loaded before the exchange nor moves an access across it.
MOE_DEV void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- MFMA on one K chunk of the staged tile -------------------------------
template <class C>
MOE_DEV void mma_chunk(f32x16_t (&acc)[C::MB][C::NB], const MOE_LDS uint16_t* sA,
                       const MOE_LDS uint16_t* sB,
                       int kc, int lane) {
  constexpr int LDK = TileLds<uint16_t, C>::LDK;
  const int wm = wave_id() / C::WAVES_N, wn = wave_id() % C::WAVES_N;
  const int ko = kc * 16 + (lane >> 5) * 8;
  bf16x8_t a[C::MB], b[C::NB];
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
    a[i] = *(const MOE_LDS bf16x8_t*)(sA + (wm * C::WM + i * 32 + (lane & 31)) * LDK + ko);
#pragma unroll
  for (int j = 0; j < C::NB; ++j)
    b[j] = *(const MOE_LDS bf16x8_t*)(sB + (wn * C::WN + j * 32 + (lane & 31)) * LDK + ko);
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
#pragma unroll
    for (int j = 0; j < C::NB; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

template <class C>
MOE_DEV void mma_chunk(f32x16_t (&acc)[C::MB][C::NB], const MOE_LDS float* sA,
                       const MOE_LDS float* sB, int kc,
                       int lane) {
  constexpr int LDK = TileLds<float, C>::LDK;
  const int wm = wave_id() / C::WAVES_N, wn = wave_id() % C::WAVES_N;
  const int ko = kc * 8 + (lane >> 5) * 4;
  f32x4_t a[C::MB], b[C::NB];
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
    a[i] = *(const MOE_LDS f32x4_t*)(sA + (wm * C::WM + i * 32 + (lane & 31)) * LDK + ko);
#pragma unroll
  for (int j = 0; j < C::NB; ++j)
    b[j] = *(const MOE_LDS f32x4_t*)(sB + (wn * C::WN + j * 32 + (lane & 31)) * LDK + ko);
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int i = 0; i < C::MB; ++i)
#pragma unroll
      for (int j = 0; j < C::NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][v], b[j][v], acc[i][j], 0, 0, 0);
}

// ---- loaders ---------------------------------------------------------------
// K-contiguous rows.  rowoff(row) returns the element offset of the row's
// first element (K index 0) from `base`, or -1 for a row that reads as zeros.
// Offsets are 32-bit (every operand here is < 2^31 elements) and the LDS
// position of chunk i is a compile-time step from chunk 0, which keeps the
// loader at one register per chunk plus its data.
template <typename T, int ROWS, int NT> struct RowLoad {
  static constexpr int VE = Elem<T>::VE, BK = Elem<T>::BK, LDK = BK + VE;
  static constexpr int CPR = BK / VE;               // 16-byte chunks per row
  static constexpr int NCH = ROWS * CPR / NT;
  static_assert(NT % CPR == 0, "rows per pass");
  const T* base;
  int off[NCH];
  uint4 v[NCH];
  template <class F> MOE_DEV void init(const T* b, F rowoff) {
    base = b;
    const int col = (threadIdx.x % CPR) * VE;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int row = threadIdx.x / CPR + i * (NT / CPR);
      const int o = rowoff(row);
      off[i] = o < 0 ? -1 : o + col;
    }
  }
  MOE_DEV void load(int kt) {
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      v[i] = off[i] >= 0 ? ldg16(base + (size_t)(unsigned)off[i] + (size_t)kt * BK) : zero4();
  }
  MOE_DEV void store(MOE_LDS T* s) {
    MOE_LDS T* p = s + (threadIdx.x / CPR) * LDK + (threadIdx.x % CPR) * VE;
#pragma unroll
    for (int i = 0; i < NCH; ++i) lds_st16(p + i * (NT / CPR) * LDK, v[i]);
  }
};

// e4m3 weight rows with one fp32 scale per 128x128 block, widened to bf16 on
// the way into LDS.  rowptr(row) gives the row's codes, rowscale(row) the
// scale row of its 128-row block (indexed by K/128).
template <int ROWS, int NT> struct RowLoadFp8 {
  static constexpr int BK = 64, LDK = BK + 8;
  static constexpr int CPR = BK / 16;               // 16 codes per 16-byte chunk
  static constexpr int NCH = ROWS * CPR / NT;
  const uint8_t* ptr[NCH];
  const float* sc[NCH];
  int soff[NCH];
  uint4 v[NCH];
  float s[NCH];
  template <class F, class G> MOE_DEV void init(F rowptr, G rowscale) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + NT * i;
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
      v[i] = ptr[i] ? ldg16(ptr[i] + (size_t)kt * BK) : zero4();
      s[i] = ptr[i] ? *(const MOE_GLB float*)(sc[i] + ((kt * BK) >> 7)) : 0.f;
    }
  }
  MOE_DEV void store(MOE_LDS uint16_t* sm) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      V16 in, o0, o1;
      in.u = v[i];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        o0.h[j] = f2bf(e4m3_to_f32(in.b[j]) * s[i]);
        o1.h[j] = f2bf(e4m3_to_f32(in.b[8 + j]) * s[i]);
      }
      lds_st16(sm + soff[i], o0.u);
      lds_st16(sm + soff[i] + 8, o1.u);
    }
  }
};

// Source contiguous along the tile's ROWS axis (M or N); K walks source rows.
// src(k, mn) returns 16 bytes = VE elements at (k, mn..mn+VE-1), zeros when
// out of range.  Thread t covers K rows k0..k0+3 and MN columns mn0..mn0+VE-1.
template <typename T, int ROWS, int NT> struct TransLoad {
  static constexpr int VE = Elem<T>::VE, BK = Elem<T>::BK, LDK = BK + VE;
  static constexpr int MNG = ROWS / VE;
  static constexpr int KSUB = 4;
  static constexpr int NSUB = MNG * (BK / KSUB) / NT;   // 4 x VE blocks per thread
  static_assert(NSUB * NT == MNG * (BK / KSUB), "blocks must tile the threads");
  uint4 v[NSUB][KSUB];
  MOE_DEV void init() {}
  // K groups vary fastest across lanes: the 16 (bf16) lanes of one MN group
  // write one LDS row's K range as a contiguous run, and the next 16 lanes the
  // row VE further on, so a wave's transposed stores cover every bank once.
  static constexpr int KG = BK / KSUB;
  MOE_DEV int mn0(int i) const { return ((threadIdx.x + NT * i) / KG) * VE; }
  MOE_DEV int k0(int i) const { return ((threadIdx.x + NT * i) % KG) * KSUB; }
  template <class S> MOE_DEV void load(int kt, S& src) {
#pragma unroll
    for (int i = 0; i < NSUB; ++i)
#pragma unroll
      for (int kk = 0; kk < KSUB; ++kk) v[i][kk] = src(kt * BK + k0(i) + kk, mn0(i));
  }
  MOE_DEV void store(MOE_LDS T* s) {
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
      V16 in[KSUB];
#pragma unroll
      for (int kk = 0; kk < KSUB; ++kk) in[kk].u = v[i][kk];
      const int m0 = mn0(i), kb = k0(i);
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          uint2 o;
          o.x = (uint32_t)in[0].h[e] | ((uint32_t)in[1].h[e] << 16);
          o.y = (uint32_t)in[2].h[e] | ((uint32_t)in[3].h[e] << 16);
          lds_st8(s + (m0 + e) * LDK + kb, o);
        }
      } else {
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          V16 o;
#pragma unroll
          for (int kk = 0; kk < KSUB; ++kk) o.f[kk] = in[kk].f[e];
          lds_st16(s + (m0 + e) * LDK + kb, o.u);
        }
      }
    }
  }
};

// Loader adapters so the main loop can drive both kinds uniformly.
template <class L> struct PlainLd {
  L& l;
  MOE_DEV void load(int kt) { l.load(kt); }
  template <typename P> MOE_DEV void store(P s) { l.store(s); }
};
template <class L, class S> struct TransLd {
  L& l;
  S& src;
  MOE_DEV void load(int kt) { l.load(kt, src); }
  template <typename P> MOE_DEV void store(P s) { l.store(s); }
};

// ---- main loop ----------------------------------------------------------------
// Every wave runs every MFMA: a data-dependent skip would make the compiler
// copy the accumulators, which costs far more than the padding rows it saves.
template <typename T, class C, class LA, class LB>
MOE_DEV void gemm_tile(LA la, LB lb, int nk, MOE_LDS T* smem, f32x16_t (&acc)[C::MB][C::NB]) {
  using L = TileLds<T, C>;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
#pragma unroll
    for (int j = 0; j < C::NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  if (nk <= 0) return;
  constexpr int STAGE = L::A_ELEMS + L::B_ELEMS;
  la.load(0);
  lb.load(0);
  la.store(smem);
  lb.store(smem + L::A_ELEMS);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(kt + 1);
      lb.load(kt + 1);
    }
#pragma unroll
    for (int kc = 0; kc < L::NKC; ++kc)
      mma_chunk<C>(acc, smem + cur * STAGE, smem + cur * STAGE + L::A_ELEMS, kc, lane);
    if (more) {
      la.store(smem + (cur ^ 1) * STAGE);
      lb.store(smem + (cur ^ 1) * STAGE + L::A_ELEMS);
    }
    __syncthreads();
  }
}

// ---- direct-to-LDS pipeline (bf16, K-contiguous operands) ---------------------
// global_load_lds_dwordx4 moves 16 bytes per lane from global memory straight
// into LDS (lane i of a wave writes LDS bytes [16 i, 16 i + 16) after the
// wave-uniform base), so staging costs no registers and four stages fit:
// the loads of K step kt+3 are in flight while step kt computes.
// Stage layout: [rows][32 bf16 = 64 bytes], the four 16-byte chunks of a row
// XOR-swizzled by ((row >> 1) ^ (row >> 3)) & 3, so any 8 (or 16) lanes that
// read one chunk of 8 (16) consecutive rows hit distinct LDS bank groups.  A wave load instruction
// covers 16 rows; the 256 rows of a tile operand are 16 instructions, 4 per
// wave.  Completion is tracked with explicit vmcnt waits and a bare s_barrier
// (__syncthreads would wait for every load in flight).
constexpr int kDmaStages = 4, kDmaBK = 32, kDmaRowBytes = 64;

// Buffer resources: loads through a descriptor take a 32-bit byte offset per
// lane (one register instead of a 64-bit address), and an offset at or past
// the descriptor's size reads as zeros, which is how rows outside a segment
// are padded.  Every buffer addressed this way is below 2 GiB.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
constexpr uint32_t kOob = 0x80000000u;            // any offset >= this reads zeros
MOE_DEV BufRsrc make_rsrc(const void* base, uint32_t bytes) {
  // word 3 = 0x00020000: raw 32-bit data format, the untyped-buffer setting on CDNA
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
MOE_DEV void buf_load_lds16(BufRsrc r, uint32_t off, MOE_LDS void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, off, 0, 0, 0);
}
// 16-byte store through a buffer descriptor; an offset past the descriptor's
// size (kOob) is dropped by the buffer unit, so a masked store still counts as
// one vector memory operation
MOE_DEV void buf_store16(BufRsrc r, uint32_t off, const u32x4_t& d) {
  __builtin_amdgcn_raw_buffer_store_b128(d, r, off, 0, 0);
}
// the same with cache-policy bits CP (16 = sc1: the store completes once it is
// visible at device scope, so a workgroup on another XCD can read it)
template <int CP> MOE_DEV void buf_store16c(BufRsrc r, uint32_t off, const u32x4_t& d) {
  __builtin_amdgcn_raw_buffer_store_b128(d, r, off, 0, CP);
}
constexpr int kStoreLocal = 0, kStoreDevice = 16;

MOE_DEV int dma_swz(int row, int chunk) { return chunk ^ (((row >> 1) ^ (row >> 3)) & 3); }

template <int ROWS, int NWAVES> struct RowDma {
  static constexpr int NI = ROWS / 16 / NWAVES;     // load instructions per wave per step
  static constexpr int STAGE_ELEMS = ROWS * 32;
  // Fragment addresses.  Fragment i of a wave covers rows wave_base + 32 i ..
  // +31 (lane & 31) and K chunk kc; wave_base is a multiple of 32, so the
  // swizzle depends on the lane alone and the byte offset is
  // (lane part ^ 32 kc) + 2048 i: one register per lane, the rest immediates.
  struct Lane { uint32_t off; };
  static MOE_DEV Lane lane_info(int wave_base, int lane) {
    const int row = lane & 31;
    return {(uint32_t)((wave_base + row) * kDmaRowBytes + dma_swz(row, lane >> 5) * 16)};
  }
  template <int KC>
  static MOE_DEV bf16x8_t frag(const MOE_LDS uint16_t* st, const Lane& L, int i) {
    const MOE_LDS char* p = (const MOE_LDS char*)st + ((L.off ^ (32u * KC)) + 32u * kDmaRowBytes * i);
    return *(const MOE_LDS bf16x8_t*)p;
  }
  BufRsrc rs;
  uint32_t off[NI];                                 // byte offset of this lane's chunk at K step 0
  // rowoff(row) = element offset of the row's first element from b, or -1 for
  // a row that reads as zeros; `bytes` = extent of the buffer at b.
  template <class F> MOE_DEV void init(const uint16_t* b, uint32_t bytes, F rowoff) {
    rs = make_rsrc(b, bytes);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = (w + NWAVES * i) * 16 + (lane >> 2);
      const int o = rowoff(row);
      off[i] = o < 0 ? kOob : (uint32_t)o * 2u + dma_swz(row, lane & 3) * 16u;
    }
  }
  // Offsets of this wave's loads of K step kt, then their issue into the
  // stage at `st` (LDS).
  struct Offs { uint32_t o[NI]; };
  MOE_DEV Offs prep(int kt) const {
    Offs q;
#pragma unroll
    for (int i = 0; i < NI; ++i) q.o[i] = off[i] + (uint32_t)kt * kDmaRowBytes;
    return q;
  }
  MOE_DEV void issue(const Offs& q, MOE_LDS uint16_t* st) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      buf_load_lds16(rs, q.o[i], (MOE_LDS void*)(st + (w + NWAVES * i) * 16 * (kDmaRowBytes / 2)));
  }
};

template <class C> struct DmaCfg {
  static constexpr int STAGE_A = C::BM * 32, STAGE_B = C::BN * 32;   // elements
  static constexpr int STAGE = STAGE_A + STAGE_B;
  static constexpr size_t BYTES = (size_t)kDmaStages * STAGE * 2;
  static constexpr int LPS = C::BM / 16 / (C::NT / 64) + C::BN / 16 / (C::NT / 64);
};

template <int N> MOE_DEV void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));   // lgkmcnt(0)
}

// nk = K / 32 steps.  Schedule of step kt (stage kt % 4 holds its operands):
//   read chunk-1 fragments of kt | MFMAs of chunk 0
//   wait until this wave's loads of step kt+1 landed and its LDS reads are
//   done; barrier (now every wave's part of step kt+1 is in LDS and nobody
//   still reads stage kt % 4); issue the loads of step kt+4 into stage kt % 4;
//   read chunk-0 fragments of kt+1 | MFMAs of chunk 1 of kt.
// Loads past the last step re-read step nk-1 into stages nobody reads again,
// so every step has the same shape and the same wait counts.
// sched_barrier pins each fragment read ahead of the 16 MFMAs that hide it.
// OA / OB: operand objects with issue(step, stage) and a static
// frag(stage, row0, kc, lane) (RowDma, or an MnOperand).
template <class C, class OA, class OB, int STAGES = kDmaStages, bool SWAP = false>
struct DmaPipe {
  static_assert(STAGES >= 3, "at least three stages");
  static constexpr int STAGE_A = OA::STAGE_ELEMS, STAGE = OA::STAGE_ELEMS + OB::STAGE_ELEMS;
  static constexpr int LPS = OA::NI + OB::NI;
  static constexpr size_t BYTES = (size_t)STAGES * STAGE * 2;
  static_assert((STAGES - 1) * LPS < 64, "vmcnt range");
  bf16x8_t a0[C::MB], b0[C::NB], a1[C::MB], b1[C::NB];
  typename OA::Lane la;
  typename OB::Lane lb;
  template <int KC>
  MOE_DEV void read(bf16x8_t (&a)[C::MB], bf16x8_t (&b)[C::NB], const MOE_LDS uint16_t* st) {
#pragma unroll
    for (int i = 0; i < C::MB; ++i) a[i] = OA::template frag<KC>(st, la, i);
#pragma unroll
    for (int j = 0; j < C::NB; ++j) b[j] = OB::template frag<KC>(st + STAGE_A, lb, j);
  }
  // SWAP: the N fragment is the MFMA's first operand, so accumulator block
  // (i, j) holds the transposed 32 x 32 block: lane = row (M), registers = columns.
  static MOE_DEV void mma(f32x16_t (&acc)[C::MB][C::NB], const bf16x8_t (&a)[C::MB],
                          const bf16x8_t (&b)[C::NB]) {
#pragma unroll
    for (int i = 0; i < C::MB; ++i)
#pragma unroll
      for (int j = 0; j < C::NB; ++j)
        acc[i][j] = SWAP ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0)
                         : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  MOE_DEV void run(const OA& oa, const OB& ob, int nk, MOE_LDS uint16_t* smem,
                   f32x16_t (&acc)[C::MB][C::NB], bool accumulate = false) {
    const int lane = threadIdx.x & 63;
    if (!accumulate) {
#pragma unroll
      for (int i = 0; i < C::MB; ++i)
#pragma unroll
        for (int j = 0; j < C::NB; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    }
    if (nk <= 0) return;
    la = OA::lane_info((wave_id() / C::WAVES_N) * C::WM, lane);
    lb = OB::lane_info((wave_id() % C::WAVES_N) * C::WN, lane);
    __syncthreads();                      // the previous tile's users of the LDS are done
    // Load offsets of a step are computed (row tables read) well before the
    // loads are issued, so issuing never waits on them.
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
      const int kk = s < nk ? s : nk - 1;
      const auto pa = oa.prep(kk);
      const auto pb = ob.prep(kk);
      oa.issue(pa, smem + s * STAGE);
      ob.issue(pb, smem + s * STAGE + STAGE_A);
    }
    wait_vm_lgkm0<(STAGES - 1) * LPS>();
    __builtin_amdgcn_s_barrier();
    read<0>(a0, b0, smem);
    for (int kt = 0; kt + 1 < nk; ++kt) {
      const MOE_LDS uint16_t* sA = smem + (kt % STAGES) * STAGE;
      const MOE_LDS uint16_t* nA = smem + ((kt + 1) % STAGES) * STAGE;
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): chunk-0 fragments are in
      __builtin_amdgcn_sched_barrier(0);
      read<1>(a1, b1, sA);
      const int kn = kt + STAGES < nk ? kt + STAGES : nk - 1;
      const auto pa = oa.prep(kn);
      const auto pb = ob.prep(kn);
      __builtin_amdgcn_sched_barrier(0);
      mma(acc, a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      wait_vm_lgkm0<(STAGES - 2) * LPS>();
      __builtin_amdgcn_s_barrier();
      oa.issue(pa, smem + (kt % STAGES) * STAGE);
      ob.issue(pb, smem + (kt % STAGES) * STAGE + STAGE_A);
      read<0>(a0, b0, nA);
      __builtin_amdgcn_sched_barrier(0);
      mma(acc, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
    }
    {
      const MOE_LDS uint16_t* sA = smem + ((nk - 1) % STAGES) * STAGE;
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_sched_barrier(0);
      read<1>(a1, b1, sA);
      __builtin_amdgcn_sched_barrier(0);
      mma(acc, a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_sched_barrier(0);
      mma(acc, a1, b1);
    }
    wait_vm_lgkm0<0>();
    __syncthreads();                      // all loads landed, all waves done with the stages
  }
};

template <class C, class OA, class OB>
MOE_DEV void gemm_tile_dma(const OA& oa, const OB& ob, int nk, MOE_LDS uint16_t* smem,
                           f32x16_t (&acc)[C::MB][C::NB], bool accumulate = false) {
  DmaPipe<C, OA, OB> p;
  p.run(oa, ob, nk, smem, acc, accumulate);
}

// ---- wide tile: 256 x 256, 8 waves, direct-to-LDS stages -----------------------
// Eight waves (2 x 4, each 128 x 64 with 128 accumulator registers, two waves
// per SIMD) share one 256 x 256 tile.  The operands stream through 128 KB of
// LDS in stages loaded with direct-to-LDS buffer loads; the K per stage comes
// from the operand types and fixes the depth:
//   K = 64 per stage, two stages: every row segment is a full 128-byte line,
//     and a stage's loads have one step of MFMAs to land;
//   K = 32 per stage, four stages: three steps to land, half-line segments.
// Both are supported; every kernel here uses K = 64.  Measured on the FC1,
// FC2, dA and dX kernels, the four-stage form was 4-8% slower: the steps are
// bound by the throughput of the per-CU load path (about 18 bytes per clock
// per CU), not by its latency, and the shorter steps add barriers.
// Accumulators are transposed (the N fragment is the MFMA's first operand):
// each lane owns one output row and four consecutive columns per register quad.
//
// LDS swizzles, chosen from measured bank behaviour of gfx950:
//   ds_read_b128 serves 16 lanes per clock; on 128-byte rows XOR-ing the
//   16-byte chunk index with (row ^ row >> 3) & 7, on 64-byte rows with
//   (row >> 2) & 3, gives every group of 16 lanes distinct banks;
//   ds_read_b64_tr_b16 serves 32 lanes per clock (4 rows x 64 bytes); XOR-ing
//   the chunk index with 4 (row & 3) spreads those four rows over disjoint
//   64-byte bank ranges.
using WideCfg = GemmCfg<256, 256, 2, 4>;
constexpr size_t kWideLdsStages = 128 * 1024;     // LDS for the operand stages
// stages of a K-per-stage: as many as fit 128 KB for a 256 + 256 row tile
constexpr int wide_stages(int bk) { return (int)(kWideLdsStages / (512 * 2 * (size_t)bk)); }

MOE_DEV int swz_row128(int row) { return (row & 7) ^ ((row >> 3) & 3); }   // rows mod 32
MOE_DEV int swz_row64(int row) { return (row >> 2) & 3; }                   // rows mod 16
MOE_DEV int swz_tr(int row) { return (row & 3) << 2; }
typedef short s16x4_t __attribute__((ext_vector_type(4)));   // one transpose read

// K-contiguous bf16 operand: ROWS rows of K = BK per stage, [row][2 BK bytes].
// One wave instruction loads 1024 bytes: 8 rows of 128 bytes or 16 of 64.
template <int ROWS, int NWAVES, int BK_> struct RowK {
  static constexpr int BK = BK_;
  static constexpr int RB = 2 * BK;                 // row bytes per stage
  static constexpr int CPR = RB / 16;               // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;              // rows per wave instruction
  static constexpr int NI = ROWS / RPI / NWAVES;
  static constexpr int STAGE_BYTES = ROWS * RB;
  static_assert(NI * RPI * NWAVES == ROWS, "rows per stage");
  static_assert(RB == 64 || RB == 128, "stage row bytes");
  static MOE_DEV int swz(int row) { return RB == 128 ? swz_row128(row) : swz_row64(row); }
  BufRsrc rs;
  uint32_t off[NI];
  // Rows this lane loads: row(i) = (wave + NWAVES i) * RPI + lane / CPR.
  static MOE_DEV int lane_row(int i) {
    return ((threadIdx.x >> 6) + NWAVES * i) * RPI + ((threadIdx.x & 63) / CPR);
  }
  // rowoff(row) = element offset of the row's first K element from b, or -1 for
  // a row that reads as zeros; `bytes` = extent of the buffer at b.
  template <class F> MOE_DEV void init(const uint16_t* b, uint32_t bytes, F rowoff) {
    rs = make_rsrc(b, bytes);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = lane_row(i);
      const int o = rowoff(row);
      off[i] = o < 0 ? kOob : (uint32_t)o * 2u + (uint32_t)(((lane % CPR) ^ swz(row)) * 16);
    }
  }
  // From the element offsets of this lane's rows (-1 = zero row).
  MOE_DEV void init_offsets(const uint16_t* b, uint32_t bytes, const int (&o)[NI]) {
    rs = make_rsrc(b, bytes);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      off[i] = o[i] < 0 ? kOob : (uint32_t)o[i] * 2u + (uint32_t)(((lane % CPR) ^ swz(lane_row(i))) * 16);
  }
  struct Offs { uint32_t o[NI]; };
  MOE_DEV Offs prep(int kt) const {
    Offs q;
#pragma unroll
    for (int i = 0; i < NI; ++i) q.o[i] = off[i] + (uint32_t)kt * RB;
    return q;
  }
  MOE_DEV void issue(const Offs& q, MOE_LDS char* st) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      buf_load_lds16(rs, q.o[i], (MOE_LDS void*)(st + (w + NWAVES * i) * RPI * RB));
  }
  // Fragment i of a wave: rows wave_base + 32 i + (lane & 31), K chunk
  // 2 KC + (lane >> 5) of the stage; wave_base is a multiple of 32, so the
  // swizzle depends on the lane only and the offset is (lane part ^ 32 KC) +
  // 32 RB i.
  struct Lane { uint32_t off; };
  static MOE_DEV Lane lane_info(int wave_base, int lane) {
    const int lr = lane & 31, h = lane >> 5;
    return {(uint32_t)((wave_base + lr) * RB + ((h ^ swz(lr)) * 16))};
  }
  template <int KC> static MOE_DEV bf16x8_t frag(const MOE_LDS char* st, const Lane& L, int i) {
    return *(const MOE_LDS bf16x8_t*)(st + ((L.off ^ (32u * KC)) + 32u * RB * i));
  }
};

// K-contiguous e4m3 operand with 128 x 128 block scales: ROWS rows of BK codes
// per stage, [row][BK bytes]; one wave instruction loads 1024 / BK rows, and
// the 16-byte chunk c of row r sits at chunk c ^ swz(r).  An MFMA lane reads
// its 8 codes of a K chunk with one 8-byte LDS read; the stream widens them to
// bf16 (code times the block's scale, rounded to nearest even) just before
// the MFMAs that use them.  A wave's 32-row blocks j and a K step lie inside
// one 128 x 128 scale block each, so a step needs one scale per block j:
// sp[j][kt * BK / 128] (sp[j] = the scale row of block j's 128 rows).
template <int ROWS, int NWAVES, int BK_> struct RowKFp8 {
  static constexpr bool kFp8 = true;
  static constexpr int BK = BK_;
  static constexpr int RB = BK;                     // one code per K element
  static constexpr int CPR = RB / 16;
  static constexpr int RPI = 64 / CPR;
  static constexpr int NI = ROWS / RPI / NWAVES;
  static constexpr int STAGE_BYTES = ROWS * RB;
  static_assert(NI * RPI * NWAVES == ROWS, "rows per stage");
  static_assert(RB == 32 || RB == 64, "stage row bytes");
  BufRsrc rs;
  uint32_t off[NI];
  const MOE_CONST float* sp[2];
  static MOE_DEV int swz(int row) { return RB == 64 ? (row >> 2) & 3 : (row >> 3) & 1; }
  // rowoff(row) = byte offset of the row's first code from b, or -1 for a row
  // that reads as zeros; `bytes` = extent of the buffer at b.
  template <class F> MOE_DEV void init(const uint8_t* b, uint32_t bytes, F rowoff) {
    rs = make_rsrc(b, bytes);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = (w + NWAVES * i) * RPI + lane / CPR;
      const int o = rowoff(row);
      off[i] = o < 0 ? kOob : (uint32_t)o + (uint32_t)(((lane % CPR) ^ swz(row)) * 16);
    }
  }
  struct Offs { uint32_t o[NI]; };
  MOE_DEV Offs prep(int kt) const {
    Offs q;
#pragma unroll
    for (int i = 0; i < NI; ++i) q.o[i] = off[i] + (uint32_t)kt * RB;
    return q;
  }
  MOE_DEV void issue(const Offs& q, MOE_LDS char* st) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      buf_load_lds16(rs, q.o[i], (MOE_LDS void*)(st + (w + NWAVES * i) * RPI * RB));
  }
  // scale of block j for K step kt (wave-uniform: scalar loads)
  MOE_DEV float scale(int j, int kt) const { return sp[j & 1][kt / (128 / BK)]; }
  // Block j of a wave: rows wave_base + 32 j + (lane & 31), codes 16 KC + 8 (lane >> 5)
  // .. +7 of the stage; wave_base is a multiple of 32, so the swizzle depends on
  // the lane only and the offset is (lane part ^ 16 KC) + 32 RB j.
  struct Lane { uint32_t off; };
  static MOE_DEV Lane lane_info(int wave_base, int lane) {
    const int lr = lane & 31, h = lane >> 5;
    return {(uint32_t)((wave_base + lr) * RB + swz(lr) * 16 + 8 * h)};
  }
  template <int KC> static MOE_DEV u32x2_t codes(const MOE_LDS char* st, const Lane& L, int j) {
    return *(const MOE_LDS u32x2_t*)(st + ((L.off ^ (16u * KC)) + 32u * RB * j));
  }
};

// ---- e4m3 x e4m3 on the fp8 MFMA ------------------------------------------------
// v_mfma_scale_f32_32x32x64_f8f6f4 (probed on MI355X): lane l holds row l % 32
// of its operand; its bytes 0..15 are K 16 (l / 32) + 0..15 of the 64 and
// bytes 16..31 are K 32 + 16 (l / 32) + 0..15; the power-of-two scale of K
// block b (32 wide) of row i comes from lane i + 32 b, byte op_sel.
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// K-contiguous e4m3 rows for the fp8 MFMA: 128 codes (one K step of 128) per
// row and stage, loaded, laid out and swizzled exactly like a bf16 RowK row of
// 64 elements.  Fragment c (K 64 c .. 64 c + 63) of block i is the lane's
// 16-byte chunks 4c + h and 4c + 2 + h (h = lane / 32): RowK's fragments 2c
// and 2c + 1, which gives the MFMA's K order for A and B alike.
template <int ROWS, int NWAVES> struct RowK8 : RowK<ROWS, NWAVES, 64> {
  static constexpr bool kF8Mma = true;
  using Base = RowK<ROWS, NWAVES, 64>;
  template <int C> static MOE_DEV i32x8_t frag8(const MOE_LDS char* st, const typename Base::Lane& L, int i) {
    typedef int i32x4_t __attribute__((ext_vector_type(4)));
    const i32x4_t lo = __builtin_bit_cast(i32x4_t, Base::template frag<2 * C>(st, L, i));
    const i32x4_t hi = __builtin_bit_cast(i32x4_t, Base::template frag<2 * C + 1>(st, L, i));
    return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
};

// Weight rows (the MFMA's first operand) with 128 x 128 fp32 block scales: a
// wave's 32-row block j and a K step lie in one scale block, sp[j & 1][kt].
template <int ROWS, int NWAVES> struct RowK8W : RowK8<ROWS, NWAVES> {
  const MOE_CONST float* sp[2];
  MOE_DEV float scale(int j, int kt) const { return sp[j & 1][kt]; }
};

// Activation rows (the MFMA's second operand) with one power-of-two exponent
// per row and K step: exps [K steps][T] int32 (block-major), row r of the tile
// reading token t_r.  Waves 0 .. ROWS / 64 - 1 each move the exponents of 64
// rows into the stage's 1 KB exponent region (SC_OFF + stage * 1024 in LDS)
// with one dword direct load; a row past the item reads zero (scale 2^0,
// with zero codes).
template <int ROWS, int NWAVES, size_t SC_OFF> struct RowK8A : RowK8<ROWS, NWAVES> {
  static constexpr size_t kScOff = SC_OFF;
  static constexpr int kScRegion = 1024;
  static_assert(ROWS * 4 <= kScRegion, "exponent region");
  using Base = RowK<ROWS, NWAVES, 64>;
  BufRsrc rsc;
  uint32_t sco;          // this lane's exponent row: t_r * 4, or kOob
  uint32_t scs;          // bytes per K step: T * 4
  struct Offs { uint32_t o[Base::NI]; uint32_t s; };
  MOE_DEV Offs prep(int kt) const {
    Offs q;
#pragma unroll
    for (int i = 0; i < Base::NI; ++i) q.o[i] = this->off[i] + (uint32_t)kt * Base::RB;
    q.s = sco == kOob ? kOob : sco + (uint32_t)kt * scs;
    return q;
  }
  MOE_DEV void issue(const Offs& q, MOE_LDS char* st) const {
    typename Base::Offs b;
#pragma unroll
    for (int i = 0; i < Base::NI; ++i) b.o[i] = q.o[i];
    Base::issue(b, st);
  }
  MOE_DEV void issue_sc(const Offs& q, MOE_LDS char* region) const {
    const int w = wave_id();
    if (w < ROWS / 64)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, (MOE_LDS void*)(region + w * 256), 4, q.s, 0, 0, 0);
  }
  // the lane's four rows wave_base + 32 i + lane % 32 as E8M0 bytes (e + 127), byte i
  static MOE_DEV uint32_t scale_word(const MOE_LDS char* region, int wave_base, int lane) {
    const MOE_LDS int32_t* e = (const MOE_LDS int32_t*)region + wave_base + (lane & 31);
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w |= ((uint32_t)(e[32 * i] + 127) & 0xFFu) << (8 * i);
    return w;
  }
};
template <class T, class = void> struct op_f8mma { static constexpr bool value = false; };
template <class T> struct op_f8mma<T, decltype((void)T::kF8Mma)> { static constexpr bool value = T::kF8Mma; };

// 8 e4m3 codes (bytes of q, low first) times s, as bf16 rounded to nearest even.
MOE_DEV bf16x8_t dequant8(const u32x2_t& q, float s) {
  bf16x8_t o;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[w], false);   // bytes 0, 1
    const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[w], true);    // bytes 2, 3
    o[4 * w + 0] = (__bf16)(lo[0] * s);
    o[4 * w + 1] = (__bf16)(lo[1] * s);
    o[4 * w + 2] = (__bf16)(hi[0] * s);
    o[4 * w + 3] = (__bf16)(hi[1] * s);
  }
  return o;
}

template <class T, class = void> struct op_fp8 { static constexpr bool value = false; };
template <class T> struct op_fp8<T, decltype((void)T::kFp8)> { static constexpr bool value = T::kFp8; };
// A source that takes part in a two-phase launch (kFlow): peek(it) loads the
// readiness of the rows item `it` reads, ready(it, seen) returns once they are
// complete (seen: an earlier peek's value, or a negative number for none),
// publish_key(it) is what a finished item publishes (-1 for nothing), and
// signal(key) publishes it once the item's stores are complete.
template <class T, class = void> struct src_rows_in_regs { static constexpr bool value = false; };
template <class T> struct src_rows_in_regs<T, decltype((void)T::kRowsInRegs)> {
  static constexpr bool value = T::kRowsInRegs;
};
template <class T, class = void> struct src_flow { static constexpr bool value = false; };
template <class T> struct src_flow<T, decltype((void)T::kFlow)> { static constexpr bool value = T::kFlow; };
// A source whose items may leave whole waves without rows (kSkipIdle):
// wave_active(it) is false for a wave whose M range lies past the item's
// rows; that wave then skips its fragment reads and MFMAs (its accumulators
// stay zero, which is what those rows would hold) but still loads its share
// of each stage.
template <class T, class = void> struct src_skip_idle { static constexpr bool value = false; };
template <class T> struct src_skip_idle<T, decltype((void)T::kSkipIdle)> { static constexpr bool value = T::kSkipIdle; };

// MN-contiguous operand: BK K rows x MN elements per stage, [k][MN], fragments
// through ds_read_b64_tr_b16: inside each 16-lane group, lane j supplies the
// address of row k0 + j/4, columns m0 + 4 (j % 4) .. +3 and receives column
// m0 + j of rows k0 .. k0+3, i.e. four consecutive K values of one M/N index;
// two such reads give the eight K values an MFMA lane needs.  rowoff(k) = byte offset in the
// buffer of (source row of K index k, mn0), or kOob for a zero row.
template <int MN, int NWAVES, int BK_> struct MnK {
  static constexpr int BK = BK_;
  static constexpr int ROWB = MN * 2;
  static constexpr int RPI = 1024 / ROWB;           // K rows per wave instruction
  static constexpr int CPR = ROWB / 16;
  static constexpr int NI = BK / RPI / NWAVES;
  static constexpr int STAGE_BYTES = BK * ROWB;
  static_assert(NI * RPI * NWAVES == BK, "K rows per stage");
  BufRsrc rs;
  struct Offs { uint32_t o[NI]; };
  static MOE_DEV int chunk_swz(int row) { return swz_tr(row); }
  // stage row (K index within the step) loaded by this lane's instruction i
  static MOE_DEV int row_of(int i) { return ((threadIdx.x >> 6) + NWAVES * i) * RPI + (threadIdx.x & 63) / CPR; }
  // first of the RPI rows of instruction i (wave-uniform)
  static MOE_DEV int row_base(int i) { return (wave_id() + NWAVES * i) * RPI; }
  MOE_DEV void issue(const Offs& p, MOE_LDS char* st) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      buf_load_lds16(rs, p.o[i], (MOE_LDS void*)(st + (w + NWAVES * i) * RPI * ROWB));
  }
  // Lane j of 16-lane group G reads rows 16 KC + 8 (G >> 1) + j / 4 (+ 4) at
  // column wave_base + 32 i + 16 (G & 1) + 4 (j % 4); the swizzle touches
  // chunk bits 2..3 and fragment i adds 4 i chunks above the lane's bits 0..1,
  // so the offset is (lane part ^ 64 i) + KC * 16 * ROWB.
  struct Lane { uint32_t off[2]; };
  static MOE_DEV Lane lane_info(int wave_base, int lane) {
    const int G = lane >> 4, j = lane & 15;
    const int m = wave_base + 16 * (G & 1) + 4 * (j & 3);
    const int c = m >> 3, within = m & 7;
    Lane L;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * (G >> 1) + (j >> 2) + 4 * h;
      L.off[h] = (uint32_t)(row * ROWB + ((c ^ swz_tr(row)) << 4) + within * 2);
    }
    return L;
  }
  // Issued from inline asm: for a compiler-visible LDS read the compiler waits
  // for every direct-to-LDS load in flight first, which would serialise the
  // pipeline.  The caller consumes the result only after an explicit
  // lgkmcnt(0) wait.
  template <int KC> static MOE_DEV bf16x8_t frag(const MOE_LDS char* st, const Lane& L, int i) {
    s16x4_t lo, hi;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                 : "=v"(lo) : "v"(st + (L.off[0] ^ (64u * i))), "i"(KC * 16 * ROWB));
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                 : "=v"(hi) : "v"(st + (L.off[1] ^ (64u * i))), "i"(KC * 16 * ROWB));
    typedef short s16x8_t __attribute__((ext_vector_type(8)));
    const s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  }
};

// MN-contiguous e4m3 operand with 128 x 128 block scales: BK K rows x MN
// codes per stage, [k][MN bytes]; 16-byte chunk c of stage row r sits at chunk
// c ^ 2 (r & 7).  Fragments through ds_read_b64_tr_b8: inside each 16-lane
// group, lane j supplies the address of row k0 + j/2, codes m0 + 8 (j % 2) ..
// +7, and receives code m0 + j of rows k0 .. k0+7 (byte i from row k0 + i),
// i.e. the eight consecutive K values an MFMA lane needs, in one read.  The 8
// rows one 32-lane half of a read touches then cover all 16 chunk positions
// of a 256-byte bank window.  A wave's 64 columns and a K step lie inside one
// scale block: scale(j, kt) = sp[(kt * BK / 128) * sld] for both blocks j.
template <int MN, int NWAVES, int BK_> struct MnKFp8 {
  static constexpr bool kFp8 = true;
  static constexpr int BK = BK_;
  static constexpr int ROWB = MN;                   // one code per element
  static constexpr int RPI = 1024 / ROWB;
  static constexpr int CPR = ROWB / 16;
  static constexpr int NI = BK / RPI / NWAVES;
  static constexpr int STAGE_BYTES = BK * ROWB;
  static_assert(NI * RPI * NWAVES == BK, "K rows per stage");
  static_assert(CPR == 16, "chunk swizzle spans 16 chunks");
  BufRsrc rs;
  const MOE_CONST float* sp;
  int sld;
  struct Offs { uint32_t o[NI]; };
  static MOE_DEV int chunk_swz(int row) { return 2 * (row & 7); }
  static MOE_DEV int row_of(int i) { return ((threadIdx.x >> 6) + NWAVES * i) * RPI + (threadIdx.x & 63) / CPR; }
  static MOE_DEV int row_base(int i) { return (wave_id() + NWAVES * i) * RPI; }
  MOE_DEV void issue(const Offs& p, MOE_LDS char* st) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      buf_load_lds16(rs, p.o[i], (MOE_LDS void*)(st + (w + NWAVES * i) * RPI * ROWB));
  }
  MOE_DEV float scale(int, int kt) const { return sp[(kt / (128 / BK)) * sld]; }
  // Block j: lane j' of 16-lane group G covers column wave_base + 32 j +
  // 16 (G & 1) + j' and K rows 16 KC + 8 (G >> 1) .. +7; it addresses row
  // 16 KC + 8 (G >> 1) + j'/2, whose swizzle 2 (j'/2) depends on the lane only.
  struct Lane { uint32_t off[2]; };
  static MOE_DEV Lane lane_info(int wave_base, int lane) {
    const int G = lane >> 4, jl = lane & 15;
    const int row = 8 * (G >> 1) + (jl >> 1);
    Lane L;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = (wave_base + 32 * j) / 16 + (G & 1);
      L.off[j] = (uint32_t)(row * ROWB + ((c ^ chunk_swz(row)) << 4) + 8 * (jl & 1));
    }
    return L;
  }
  // Issued from inline asm, like MnK::frag: consumed after an explicit
  // lgkmcnt(0) wait.
  template <int KC> static MOE_DEV u32x2_t codes(const MOE_LDS char* st, const Lane& L, int j) {
    u32x2_t v;
    asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2"
                 : "=v"(v) : "v"(st + L.off[j & 1]), "i"(KC * 16 * ROWB));
    return v;
  }
};

// MN-contiguous e4m3 operand for the fp8 MFMA: 128 K rows x MN codes per
// stage (a K step of 128 codes is one 128 x 128 scale block deep), laid out
// and swizzled like MnKFp8.  BK = 64 in the stream's units (the bf16
// elements a RowK8 row of 128 codes stands for); KROWS = 128 K rows.  Block j
// of a wave, chunk C (K 64 C .. 64 C + 63): lane l holds column
// wave_base + 32 j + l % 32 and needs K 16 h + 0..15 and 32 + 16 h + 0..15 of
// the chunk (h = l / 32), four ds_read_b64_tr_b8 of 8 K rows each.  In
// 16-lane group G (columns 16 (G & 1) + 0..15, h = G >> 1) lane j' addresses
// row 64 C + 16 h + 8 (r & 1) + 32 (r >> 1) + j' / 2 for read r; the row
// offsets are multiples of 8, so the swizzle 2 (j' / 2) depends on the lane
// only and each read is the lane's base address plus an immediate.
template <int MN, int NWAVES> struct MnK8 {
  static constexpr bool kF8Mma = true;
  static constexpr int BK = 64;
  static constexpr int KROWS = 128;
  static constexpr int ROWB = MN;
  static constexpr int RPI = 1024 / ROWB;
  static constexpr int CPR = ROWB / 16;
  static constexpr int NI = KROWS / RPI / NWAVES;
  static constexpr int STAGE_BYTES = KROWS * ROWB;
  static_assert(NI * RPI * NWAVES == KROWS, "K rows per stage");
  static_assert(CPR == 16, "chunk swizzle spans 16 chunks");
  BufRsrc rs;
  const MOE_CONST float* sp;
  int sld;
  struct Offs { uint32_t o[NI]; };
  static MOE_DEV int chunk_swz(int row) { return 2 * (row & 7); }
  static MOE_DEV int row_of(int i) { return ((threadIdx.x >> 6) + NWAVES * i) * RPI + (threadIdx.x & 63) / CPR; }
  static MOE_DEV int row_base(int i) { return (wave_id() + NWAVES * i) * RPI; }
  MOE_DEV void issue(const Offs& p, MOE_LDS char* st) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      buf_load_lds16(rs, p.o[i], (MOE_LDS void*)(st + (w + NWAVES * i) * RPI * ROWB));
  }
  // a wave's 64 columns and a K step lie in one scale block
  MOE_DEV float scale(int, int kt) const { return sp[(size_t)kt * sld]; }
  struct Lane { uint32_t off[2]; };
  static MOE_DEV Lane lane_info(int wave_base, int lane) {
    const int G = lane >> 4, jl = lane & 15;
    const int row = 16 * (G >> 1) + (jl >> 1);
    Lane L;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = (wave_base + 32 * j) / 16 + (G & 1);
      L.off[j] = (uint32_t)(row * ROWB + ((c ^ chunk_swz(row)) << 4) + 8 * (jl & 1));
    }
    return L;
  }
  // Issued from inline asm, like MnK::frag: every output is consumed, after
  // an explicit lgkmcnt(0) wait.
  template <int C> static MOE_DEV i32x8_t frag8(const MOE_LDS char* st, const Lane& L, int j) {
    u32x2_t v0, v1, v2, v3;
    const MOE_LDS char* p = st + L.off[j & 1];
    asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(v0) : "v"(p), "i"((64 * C) * ROWB));
    asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(v1) : "v"(p), "i"((64 * C + 8) * ROWB));
    asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(v2) : "v"(p), "i"((64 * C + 32) * ROWB));
    asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(v3) : "v"(p), "i"((64 * C + 40) * ROWB));
    return i32x8_t{(int)v0[0], (int)v0[1], (int)v1[0], (int)v1[1],
                   (int)v2[0], (int)v2[1], (int)v3[0], (int)v3[1]};
  }
};

// MN-contiguous operand bound to its row function.  F::pre(k) gives a raw
// value for K index k (an index, or a value loaded from memory, not yet
// combined with anything, so no wait is needed until the loads are issued),
// F::post(raw, k) turns it into the byte offset of (row, mn0) in the buffer,
// or kOob for a zero row.  prep() runs early in a step, issue() after the
// step-end wait.
template <class OP, class F> struct MnKOperand {
  OP op;
  F f;
  static constexpr int BK = OP::BK, NI = OP::NI, STAGE_BYTES = OP::STAGE_BYTES;
  static constexpr int KR = OP::STAGE_BYTES / OP::ROWB;   // K rows per step
  static constexpr bool kFp8 = op_fp8<OP>::value;
  static constexpr bool kF8Mma = op_f8mma<OP>::value;
  using Lane = typename OP::Lane;
  // f.pre(kb, k): what post needs for the lane's K row k, where kb is the
  // wave-uniform first row of the same instruction
  struct Offs { typename F::Raw raw[NI]; int kt; };
  MOE_DEV Offs prep(int kt) const {
    Offs p;
    p.kt = kt;
#pragma unroll
    for (int i = 0; i < NI; ++i) p.raw[i] = f.pre(kt * KR + OP::row_base(i), kt * KR + OP::row_of(i));
    return p;
  }
  MOE_DEV void issue(const Offs& p, MOE_LDS char* st) const {
    typename OP::Offs q;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = OP::row_of(i);
      q.o[i] = f.post(p.raw[i], p.kt * KR + r) + (uint32_t)(((threadIdx.x & 63) % OP::CPR) ^ OP::chunk_swz(r)) * 16u;
    }
    op.issue(q, st);
  }
  static MOE_DEV Lane lane_info(int wave_base, int lane) { return OP::lane_info(wave_base, lane); }
  template <int KC> static MOE_DEV bf16x8_t frag(const MOE_LDS char* st, const Lane& L, int i) {
    return OP::template frag<KC>(st, L, i);
  }
  template <int KC> static MOE_DEV u32x2_t codes(const MOE_LDS char* st, const Lane& L, int j) {
    return OP::template codes<KC>(st, L, j);
  }
  template <int C> static MOE_DEV i32x8_t frag8(const MOE_LDS char* st, const Lane& L, int j) {
    return OP::template frag8<C>(st, L, j);
  }
  MOE_DEV float scale(int j, int kt) const { return op.scale(j, kt); }
};
// ---- wide tile, persistent across tiles -------------------------------------
// K runs in steps of BK (32 or 64) over S = wide_stages(BK) LDS stages; step
// g of the stream uses stage g % S.  A step is NCH = BK / 16 K chunks; the
// fragments of chunk c+1 are read while chunk c's 8 MFMAs per wave run, and
// the load offsets of step g+S are prepared early in the step.  After the
// second-to-last chunk's MFMAs: wait until this wave's loads of step g+1 have
// landed (the loads of the S-2 steps issued after them may stay in flight)
// and its LDS reads are done; barrier (every wave's part of step g+1 is in
// LDS and nobody reads stage g % S any more); issue step g+S into stage g % S;
// read chunk 0 of step g+1; then the last chunk's MFMAs.  Fragments read from
// asm (MnK) are consumed only after an explicit lgkmcnt(0) wait pinned by a
// scheduling barrier.
//
// The stream of K steps runs on from one work item to the next: the first S
// steps of the next item are issued during the last S steps of the current
// one, so a tile starts with its operands already in LDS, and the previous
// tile's stores drain while the next tile's first S-1 steps compute.  Items
// come from a static per-workgroup sequence (no queue atomics).  Because
// vector-memory completions are counted in order, nothing issued while loads
// are in flight may be waited for early: an item's descriptor is read three
// items ahead, its per-row data (moved into LDS by direct loads) two items
// ahead, and its operands are set up one item ahead; every one of those
// waits falls on a step-end wait that happens anyway.  Every item has at
// least S steps, and every step issues the same loads (past the stream's end
// they re-read the last step into stages nobody reads again), so the wait
// counts are fixed.
//
// Src provides:
//   Item load(int idx)                 descriptor of item idx (plain loads)
//   void fill(const Item&, int slot)   issue direct loads of per-row data into LDS
//                                      item slot `slot` (after a barrier: the
//                                      slot's previous item is finished)
//   OA opA(const Item&, int slot), OB opB(const Item&, int slot)
//   int steps(const Item&)             K steps, >= S
//   void epilogue(const Item&, int slot, acc)
//   template <int B> relaxed_wait()    the wait at the end of an item's first
//                                      S-1 steps: vmcnt(B + N) with N at most
//                                      the vector memory operations one
//                                      epilogue issues, then lgkmcnt(0)
//   int count, first, stride           items first, first + stride, ... < count
// An e4m3 B operand (kFp8) hands out raw codes and a scale per 32-row block
// and K step; the stream loads the next step's scales one step ahead and
// widens the codes to bf16 in mma().
// Accumulator layout of the 32 x 32 blocks.  By default the B fragment is the
// MFMA's first operand, so lane % 32 indexes the tile row (M) and register r
// with lane / 32 the column: 8 (r / 4) + 4 (lane / 32) + r % 4.  With
// ROWS_IN_REGS the A fragment goes first and the roles swap: register r with
// lane / 32 gives the row and lane % 32 the column, so one store instruction
// per register writes 32 consecutive elements of a row (two rows per wave).
template <class C, class OA, class OB, bool ROWS_IN_REGS = false> struct WideStream {
  static constexpr int BK = OA::BK;
  static_assert(OB::BK == BK, "one K step for both operands");
  // e4m3 rows on both sides (kF8Mma): the fp8 MFMA, a K step of 128 codes in
  // two 64-wide chunks
  static constexpr bool F8M = op_f8mma<OB>::value;
  static constexpr int S = wide_stages(BK), NCH = F8M ? 2 : BK / 16;
  static_assert(S >= 2 && (S & (S - 1)) == 0 && (NCH == 2 || NCH == 4), "stage shape");
  static constexpr int SA = OA::STAGE_BYTES, STAGE = OA::STAGE_BYTES + OB::STAGE_BYTES;
  static_assert((size_t)S * STAGE <= kWideLdsStages, "stages fit");
  static constexpr int LPS = OA::NI + OB::NI;
  static constexpr int VM_AHEAD = (S - 2) * LPS;  // loads younger than the next step's
  static_assert(VM_AHEAD < 64, "vmcnt range");
  // an e4m3 B operand keeps its raw codes in bq and is widened in mma()
  static constexpr bool BF8 = op_fp8<OB>::value;
  static_assert(!BF8 || C::NB == 2, "e4m3 operand: two 32-row blocks per wave");
  static_assert(!F8M || (op_f8mma<OA>::value && C::MB == 4 && C::NB == 2 && !ROWS_IN_REGS),
                "fp8 MFMA: e4m3 rows on both sides, the 8-wave tile");
  bf16x8_t a[2][C::MB], b[2][C::NB];
  u32x2_t bq[2][C::NB];
  float bs[C::NB];                                // B scales of the current step
  // fp8 MFMA: one fragment set (32 bytes a lane each), the E8M0 exponents of
  // the lane's four rows for the current step, and per block j the scale the
  // accumulators are counted in (seff: acc * seff is the running sum) with
  // this step's factor seff_old / scale and whether the block is nonzero
  i32x8_t a8[C::MB], b8[C::NB];
  uint32_t sa8;
  float seff[C::NB], rat[C::NB];
  bool live[C::NB];
  template <int CC> MOE_DEV void read8(const MOE_LDS char* st) {
#pragma unroll
    for (int i = 0; i < C::MB; ++i) a8[i] = OA::template frag8<CC>(st, la, i);
#pragma unroll
    for (int j = 0; j < C::NB; ++j) b8[j] = OB::template frag8<CC>(st + SA, lb, j);
  }
  template <int I>
  static MOE_DEV f32x16_t mfma8(const i32x8_t& w, const i32x8_t& x, const f32x16_t& c, uint32_t sx) {
    // first operand: weight rows, scale 2^0; second: activation rows, the
    // E8M0 byte I of sx (row block I of the lane)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, x, c, 0, 0, 0, 127, I, (int)sx);
  }
  // chunk CC of the step; chunk 0 first rescales the accumulators to the
  // step's weight scale (a block of zero scale adds nothing and keeps its scale)
  template <int CC> MOE_DEV void mma8(f32x16_t (&acc)[C::MB][C::NB]) const {
#pragma unroll
    for (int j = 0; j < C::NB; ++j) {
      if (!live[j]) continue;
#pragma unroll
      for (int i = 0; i < C::MB; ++i) {
        if constexpr (CC == 0) {
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[i][j][q] *= rat[j];
        }
        if (i == 0) acc[i][j] = mfma8<0>(b8[j], a8[i], acc[i][j], sa8);
        else if (i == 1) acc[i][j] = mfma8<1>(b8[j], a8[i], acc[i][j], sa8);
        else if (i == 2) acc[i][j] = mfma8<2>(b8[j], a8[i], acc[i][j], sa8);
        else acc[i][j] = mfma8<3>(b8[j], a8[i], acc[i][j], sa8);
      }
    }
  }
  // this step's weight scales bs: rescaling factors and live blocks
  MOE_DEV void step_scales() {
#pragma unroll
    for (int j = 0; j < C::NB; ++j) {
      const float sc = bs[j];
      live[j] = sc != 0.f;
      rat[j] = live[j] ? seff[j] / sc : 1.f;
      if (live[j]) seff[j] = sc;
    }
  }
  typename OA::Lane la;
  typename OB::Lane lb;
  template <int KC, int SB> MOE_DEV void read(const MOE_LDS char* st) {
#pragma unroll
    for (int i = 0; i < C::MB; ++i) a[SB][i] = OA::template frag<KC>(st, la, i);
#pragma unroll
    for (int j = 0; j < C::NB; ++j) {
      if constexpr (BF8) bq[SB][j] = OB::template codes<KC>(st + SA, lb, j);
      else b[SB][j] = OB::template frag<KC>(st + SA, lb, j);
    }
  }
  template <int SB> MOE_DEV void mma(f32x16_t (&acc)[C::MB][C::NB]) const {
    if constexpr (BF8) {
#pragma unroll
      for (int j = 0; j < C::NB; ++j) {
        const bf16x8_t bj = dequant8(bq[SB][j], bs[j]);
#pragma unroll
        for (int i = 0; i < C::MB; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bj, a[SB][i], acc[i][j], 0, 0, 0);
      }
    } else if constexpr (ROWS_IN_REGS) {
#pragma unroll
      for (int i = 0; i < C::MB; ++i)
#pragma unroll
        for (int j = 0; j < C::NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[SB][i], b[SB][j], acc[i][j], 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < C::MB; ++i)
#pragma unroll
        for (int j = 0; j < C::NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[SB][j], a[SB][i], acc[i][j], 0, 0, 0);
    }
  }
  static MOE_DEV void lgkm0() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_sched_barrier(0);
  }
  // LDS offset of a stage's row-exponent region (fp8 MFMA)
  static MOE_DEV size_t sc_region(int stage) {
    if constexpr (F8M) return OA::kScOff + (size_t)stage * OA::kScRegion;
    else return 0;
  }
  template <class Src>
  MOE_DEV void run(Src& src, MOE_LDS uint16_t* smem16, f32x16_t (&acc)[C::MB][C::NB]) {
    MOE_LDS char* smem = (MOE_LDS char*)smem16;
    const int lane = threadIdx.x & 63;
    const int s = src.stride;
    int idx = src.first;
    if (idx >= src.count) return;
    la = OA::lane_info((wave_id() / C::WAVES_N) * C::WM, lane);
    lb = OB::lane_info((wave_id() % C::WAVES_N) * C::WN, lane);
    using Item = typename Src::Item;
    // prologue: items 0 and 1 filled, item 2's descriptor read
    Item it0 = src.load(idx), it1 = it0, it2 = it0;
    bool h1 = idx + s < src.count, h2 = idx + 2 * s < src.count;
    if (h1) it1 = src.load(idx + s);
    if (h2) it2 = src.load(idx + 2 * s);
    src.fill(it0, 0);
    if (h1) src.fill(it1, 1);
    wait_vm_lgkm0<0>();
    __syncthreads();
    int slot = 0;                                // LDS item slot of it0 (items rotate over 3)
    OA a0 = src.opA(it0, slot);
    OB b0 = src.opB(it0, slot);
    int n0 = src.steps(it0);
    constexpr bool FLOW = src_flow<Src>::value;
    if constexpr (FLOW) src.ready(it0, -1);
#pragma unroll
    for (int st = 0; st < S; ++st) {
      const auto pa = a0.prep(st);
      const auto pb = b0.prep(st);
      a0.issue(pa, smem + st * STAGE);
      b0.issue(pb, smem + st * STAGE + SA);
      if constexpr (F8M) a0.issue_sc(pa, smem + sc_region(st));
    }
    // two-phase sources: the last finished item not yet published (its
    // epilogue stores are published at the next strict wait; -1: none)
    int pend = -1;
    // the next item's readiness, loaded one step before its first loads are
    // issued; the full wait ending that step covers the load
    int peeked = -1;
    float bsn[C::NB];                            // B scales of the next step
    if constexpr (BF8 || F8M) {
#pragma unroll
      for (int j = 0; j < C::NB; ++j) bsn[j] = b0.scale(j, 0);
    }
    if constexpr (F8M) {
#pragma unroll
      for (int j = 0; j < C::NB; ++j) seff[j] = 0.f;
    }
    const int wrow = (wave_id() / C::WAVES_N) * C::WM;
    wait_vm_lgkm0<(S - 1) * LPS>();
    __builtin_amdgcn_s_barrier();
    constexpr bool SKIP = src_skip_idle<Src>::value;
    bool act = true;                             // this wave has rows in item it0
    if constexpr (SKIP) act = src.wave_active(it0);
    if (act) {
      if constexpr (F8M) {
        read8<0>(smem);
        sa8 = OA::scale_word(smem + sc_region(0), wrow, lane);
      } else {
        read<0, 0>(smem);
      }
    }
    int g = 0;                                   // global step index: stage g % S
    while (true) {
      const int s1 = slot == 2 ? 0 : slot + 1, s2 = s1 == 2 ? 0 : s1 + 1;
      const bool h3 = idx + 3 * s < src.count;
      Item it3 = it2;
      if (h3) it3 = src.load(idx + 3 * s);
      OA a1 = a0;
      OB b1 = b0;
      int n1 = n0;
      if (h1) { a1 = src.opA(it1, s1); b1 = src.opB(it1, s1); n1 = src.steps(it1); }
#pragma unroll
      for (int i = 0; i < C::MB; ++i)
#pragma unroll
        for (int j = 0; j < C::NB; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
      // the item's first step landed before the previous item's last barrier
      if constexpr (SKIP) act = src.wave_active(it0);
      if (g > 0 && act) {
        if constexpr (F8M) {
          read8<0>(smem + (g & (S - 1)) * STAGE);
          sa8 = OA::scale_word(smem + sc_region(g & (S - 1)), wrow, lane);
        } else {
          read<0, 0>(smem + (g & (S - 1)) * STAGE);
        }
      }
      // During its first S-1 steps, the loads an item waits for were issued
      // before the previous item's epilogue, so the epilogue's stores (and
      // loads) may stay in flight: they drain under those steps.
      const bool relax = g > 0;
      for (int kt = 0; kt < n0; ++kt, ++g) {
        const MOE_LDS char* st = smem + (g & (S - 1)) * STAGE;
        if constexpr (BF8 || F8M) {
#pragma unroll
          for (int j = 0; j < C::NB; ++j) bs[j] = bsn[j];
        }
        if constexpr (F8M) {
          // single fragment set: chunk 0's MFMAs, then chunk 1's reads into
          // the same registers (landed by the step-end wait)
          step_scales();
          lgkm0();
          __builtin_amdgcn_sched_barrier(0);
          if (act) mma8<0>(acc);
          __builtin_amdgcn_sched_barrier(0);
          if (act) read8<1>(st);
        } else {
          lgkm0();
          if (act) read<1, 1>(st);
        }
        // step g + S of the stream: this item, the next one, or a harmless
        // re-read of this item's last step when the stream ends
        const bool own = kt + S < n0;
        const bool nxt = !own && h1;
        const int ks = own ? kt + S : nxt ? kt + S - n0 : n0 - 1;
        const auto pa = nxt ? a1.prep(ks) : a0.prep(ks);
        const auto pb = nxt ? b1.prep(ks) : b0.prep(ks);
        // B scales of the next step (or of the next item's first), scalar
        // loads that land by the next chunk's wait
        if constexpr (BF8 || F8M) {
#pragma unroll
          for (int j = 0; j < C::NB; ++j)
            bsn[j] = kt + 1 < n0 ? b0.scale(j, kt + 1) : h1 ? b1.scale(j, 0) : bs[j];
        }
        if constexpr (!F8M) {
          __builtin_amdgcn_sched_barrier(0);
          if (act) mma<0>(acc);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (NCH == 4) {
          lgkm0();
          if (act) read<2, 0>(st);
          __builtin_amdgcn_sched_barrier(0);
          if (act) mma<1>(acc);
          __builtin_amdgcn_sched_barrier(0);
          lgkm0();
          if (act) read<3, 1>(st);
          __builtin_amdgcn_sched_barrier(0);
          if (act) mma<0>(acc);
          __builtin_amdgcn_sched_barrier(0);
        }
        const bool strict = !(relax && kt < S - 1);
        if (!strict) src.template relaxed_wait<VM_AHEAD>();
        else wait_vm_lgkm0<VM_AHEAD>();
        __builtin_amdgcn_s_barrier();
        if constexpr (FLOW) {
          // every wave has waited for its stores of the previous item
          if (pend >= 0 && strict) { src.signal(pend); pend = -1; }
          if (nxt && ks == 0) {
            src.ready(it1, (S < n0 && strict) ? peeked : -1);
            peeked = -1;
          }
        }
        // every wave is past the previous item's epilogue: item slot s2 is free
        if (kt == 0 && h2) src.fill(it2, s2);
        if (nxt) {
          a1.issue(pa, smem + (g & (S - 1)) * STAGE);
          b1.issue(pb, smem + (g & (S - 1)) * STAGE + SA);
          if constexpr (F8M) a1.issue_sc(pa, smem + sc_region(g & (S - 1)));
        } else {
          a0.issue(pa, smem + (g & (S - 1)) * STAGE);
          b0.issue(pb, smem + (g & (S - 1)) * STAGE + SA);
          if constexpr (F8M) a0.issue_sc(pa, smem + sc_region(g & (S - 1)));
        }
        if constexpr (FLOW) {
          if (h1 && kt + S + 1 == n0) peeked = src.peek(it1);
        }
        if constexpr (F8M) {
          // chunk 1's MFMAs, then chunk 0 of the next step (and its row
          // exponents) into the registers they have read
          __builtin_amdgcn_sched_barrier(0);
          if (act) mma8<1>(acc);
          __builtin_amdgcn_sched_barrier(0);
          if (kt + 1 < n0 && act) {
            read8<0>(smem + ((g + 1) & (S - 1)) * STAGE);
            sa8 = OA::scale_word(smem + sc_region((g + 1) & (S - 1)), wrow, lane);
          }
        } else {
          // chunk 0 of the next step; for the next item it is read after the
          // epilogue, so its fragments are not live across it
          if (kt + 1 < n0 && act) read<0, 0>(smem + ((g + 1) & (S - 1)) * STAGE);
          __builtin_amdgcn_sched_barrier(0);
          if (act) mma<1>(acc);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (F8M) {
        // back from units of the last scale to values; the next item starts over
#pragma unroll
        for (int j = 0; j < C::NB; ++j) {
#pragma unroll
          for (int i = 0; i < C::MB; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] *= seff[j];
          seff[j] = 0.f;
        }
      }
      src.epilogue(it0, slot, acc);
      if constexpr (FLOW) pend = src.publish_key(it0);
      if (!h1) break;
      idx += s;
      slot = s1;
      it0 = it1;
      a0 = a1;
      b0 = b1;
      n0 = n1;
      it1 = it2;
      h1 = h2;
      it2 = it3;
      h2 = h3;
    }
    wait_vm_lgkm0<0>();
    __syncthreads();                      // all loads landed, all waves done with the stages
    if constexpr (FLOW) {
      if (pend >= 0) src.signal(pend);
    }
  }
};

// This workgroup's place among its worker's workgroups: worker r owns the
// XCDs x with x * P / 8 == r; the workgroups of a launch are dealt to XCDs
// round-robin (blockIdx % 8).
struct WorkerSlot { int r, j, n; };
MOE_DEV WorkerSlot worker_slot(int P) {
  const int x = (int)(blockIdx.x % kXcds), per = kXcds / P;
  const int r = x * P / kXcds;
  const int j = (int)(blockIdx.x / kXcds) * per + (x - r * per);
  const int n = (int)(gridDim.x / kXcds) * per;
  return {r, j, n};
}

// Coordinates of accumulator register r of block (i, j) for this lane, within
// the tile.
template <class C> MOE_DEV int acc_row(int i, int r, int lane) {
  const int wm = wave_id() / C::WAVES_N;
  return wm * C::WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}
template <class C> MOE_DEV int acc_col(int j, int lane) {
  const int wn = wave_id() % C::WAVES_N;
  return wn * C::WN + j * 32 + (lane & 31);
}

// ---- epilogue through LDS ----------------------------------------------------
// The accumulators are written unconditionally into an LDS tile (row-major,
// `ldn` elements per row), then the workgroup reads it back in 16-byte chunks
// along rows and calls emit(row, col, chunk) for global stores that are
// coalesced and can be masked by row.  Callers bracket the two phases with
// __syncthreads().
template <class C, typename LdsT, class XF>
MOE_DEV void acc_to_lds(const f32x16_t (&acc)[C::MB][C::NB], MOE_LDS LdsT* s, int ldn, int row0,
                        int rows, XF xf) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < C::MB; ++i) {
    const int rbase = (wave_id() / C::WAVES_N) * C::WM + i * 32;
    if (rbase < row0 || rbase >= row0 + rows) continue;   // whole 32-row block in or out
#pragma unroll
    for (int j = 0; j < C::NB; ++j)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = rbase + (rr >> 2) * 8 + (lane >> 5) * 4 + (rr & 3);
        const int col = (wave_id() % C::WAVES_N) * C::WN + j * 32 + (lane & 31);
        s[(row - row0) * ldn + col] = xf(acc[i][j][rr], row, col);
      }
  }
}

template <typename LdsT, int NT, class EMIT>
MOE_DEV void lds_to_global(const MOE_LDS LdsT* s, int rows, int cols, int ldn, EMIT emit) {
  constexpr int V = 16 / sizeof(LdsT);
  const int cpr = cols / V;
  for (int c = threadIdx.x; c < rows * cpr; c += NT) {
    const int row = c / cpr, col = (c % cpr) * V;
    V16 v;
    v.u = lds_ld16(s + row * ldn + col);
    emit(row, col, v);
  }
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
