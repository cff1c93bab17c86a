// Routing statistics and the on-device planner.
//
// Routing statistics (MegaFlux summary, "Routing Skew Problem" kappa equation
// and the block definition of "Problem Formulation"):
//   c_e, exclusive prefix sums, b_e = ceil(c_e / beta), kappa, and a stable
//   padded slotting in which expert e's rows occupy slots beta * sum_{e'<e} b_e'
//   onward in increasing flat index t*k + j.
// Three launches: per-chunk histograms (LDS atomics; order-free), one
// workgroup that scans them per expert and across experts, and a slotting pass
// in which each wave ranks equal ids with a ballot-based match, so the slot of
// a row depends only on the rows before it.
//
// Planner ("Problem Formulation", "Bounded Greedy Search"): one workgroup of
// four waves; wave w runs greedy search w (donor priority x fan-out), lane r of
// a wave holds worker r's load, replica count and remote-copy count, and the
// search state q lives in LDS.  Every quantity is an integer, so the plan is
// bit-identical on every run and to any other implementation of the same
// reading (owner-first contiguous expansion, smallest index on every tie).
#include <mutex>

#include "common.h"
#include "moe_ffn.h"
#include "internal.h"

namespace moe {

constexpr int kChunk = 256;

__global__ __launch_bounds__(256) void k_route_count(const int32_t* __restrict__ ids, int N,
                                                     int E, int32_t* __restrict__ chunk_cnt,
                                                     int32_t* __restrict__ slot_to_row, int cap,
                                                     int32_t* status) {
  __shared__ int cnt[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int i = blockIdx.x * kChunk + threadIdx.x;
  if (i < N) {
    const int v = ids[i];
    if (v >= E) atomicOr(status, MOE_DEV_BAD_EXPERT);
    else if (v >= 0) atomicAdd(&cnt[v], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) chunk_cnt[(size_t)blockIdx.x * E + e] = cnt[e];
  for (int sidx = blockIdx.x * kChunk + threadIdx.x; sidx < cap; sidx += gridDim.x * kChunk)
    slot_to_row[sidx] = -1;
}

// One workgroup of 1024 threads.  Thread (e, g), g < G = 1024 / E, owns expert
// e's chunks [g*nch/G, (g+1)*nch/G): it sums them, the partial sums meet in
// LDS, threads e < E scan across experts, and each (e, g) then rewrites its
// chunks as exclusive prefixes offset by beta * block_offset(e).
__global__ __launch_bounds__(1024) void k_route_scan(int32_t* __restrict__ chunk_cnt, int nchunks,
                                                     int E, int beta, int32_t* counts,
                                                     int32_t* offsets, int32_t* block_counts,
                                                     int32_t* block_offsets, double* kappa) {
  __shared__ int wtot_c[16], wtot_b[16];
  __shared__ long long red_s[16], red_s2[16];
  __shared__ int part[1024];           // [g][e] partial sums
  __shared__ int bbase[kMaxExperts];   // beta * block_offset(e)
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G = 1024 / E;
  const int e_own = tid % E, g = tid / E;
  const bool worker = g < G;
  const int c0 = worker ? (int)((long long)g * nchunks / G) : 0;
  const int c1 = worker ? (int)((long long)(g + 1) * nchunks / G) : 0;
  // The chunk counts were just written by every XCD, so each batch of loads is
  // a full memory round trip.  When a thread owns at most kKeep chunks (every
  // workload here: 32 at most), they are loaded once, all in flight together,
  // and kept in registers for the rewrite below.
  constexpr int kKeep = 32;
  const bool keep = c1 - c0 <= kKeep;
  int held[kKeep];
  int ps = 0;
  if (keep) {
#pragma unroll
    for (int u = 0; u < kKeep; ++u)
      held[u] = c0 + u < c1 ? chunk_cnt[(size_t)(c0 + u) * E + e_own] : 0;
#pragma unroll
    for (int u = 0; u < kKeep; ++u) ps += held[u];
  } else {
#pragma unroll 8
    for (int ch = c0; ch < c1; ++ch) ps += chunk_cnt[(size_t)ch * E + e_own];
  }
  if (worker) part[g * E + e_own] = ps;
  __syncthreads();
  const int e = tid;
  int c = 0;
  if (e < E)
    for (int q = 0; q < G; ++q) c += part[q * E + e];
  const int b = (c + beta - 1) / beta;
  const int ic = wave_incl_scan(c), ib = wave_incl_scan(b);
  if (lane == 63) { wtot_c[wv] = ic; wtot_b[wv] = ib; }
  long long s1 = wave_sum64((long long)c), s2 = wave_sum64((long long)c * c);
  if (lane == 0) { red_s[wv] = s1; red_s2[wv] = s2; }
  __syncthreads();
  int pc = 0, pb = 0;
  for (int w = 0; w < wv; ++w) { pc += wtot_c[w]; pb += wtot_b[w]; }
  const int exc_c = pc + ic - c, exc_b = pb + ib - b;
  if (e < E) {
    counts[e] = c;
    offsets[e] = exc_c;
    block_counts[e] = b;
    block_offsets[e] = exc_b;
    bbase[e] = beta * exc_b;
    if (e == E - 1) { offsets[E] = exc_c + c; block_offsets[E] = exc_b + b; }
  }
  if (e == 0) {
    long long S = 0, S2 = 0;
    for (int w = 0; w < 16; ++w) { S += red_s[w]; S2 += red_s2[w]; }
    // exact integers, then one correctly rounded IEEE division
    *kappa = (S == 0) ? 1.0 : (double)((long long)E * S2) / (double)(S * S);
  }
  __syncthreads();
  // Otherwise eight chunks' counts are loaded before any of them is
  // rewritten: loads and stores of one array do not pass each other, so a
  // load per store would wait out one memory round trip per chunk.
  if (worker && keep) {
    int run = bbase[e_own];
    for (int q = 0; q < g; ++q) run += part[q * E + e_own];
#pragma unroll
    for (int u = 0; u < kKeep; ++u)
      if (c0 + u < c1) {
        chunk_cnt[(size_t)(c0 + u) * E + e_own] = run;
        run += held[u];
      }
  } else if (worker) {
    int run = bbase[e_own];
    for (int q = 0; q < g; ++q) run += part[q * E + e_own];
    constexpr int U = 8;
    for (int ch0 = c0; ch0 < c1; ch0 += U) {
      int t[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        t[u] = ch0 + u < c1 ? chunk_cnt[(size_t)(ch0 + u) * E + e_own] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (ch0 + u < c1) {
          chunk_cnt[(size_t)(ch0 + u) * E + e_own] = run;
          run += t[u];
        }
    }
  }
}

__global__ __launch_bounds__(256) void k_route_slot(const int32_t* __restrict__ ids, int N, int E,
                                                    const int32_t* __restrict__ chunk_base,
                                                    int32_t* __restrict__ row_to_slot,
                                                    int32_t* __restrict__ slot_to_row) {
  __shared__ int wcnt[4][kMaxExperts];
  for (int i = threadIdx.x; i < 4 * E; i += blockDim.x) wcnt[i / E][i % E] = 0;
  __syncthreads();
  const int i = blockIdx.x * kChunk + threadIdx.x;
  const int wv = threadIdx.x >> 6;
  const int v = (i < N) ? ids[i] : -1;
  const bool act = (v >= 0) && (v < E);
  const uint64_t m = wave_match((uint32_t)(act ? v : 0), 10, act);
  const uint64_t below = m & lanemask_lt();
  const int rank = __popcll(below);
  if (act && below == 0) wcnt[wv][v] = __popcll(m);
  __syncthreads();
  if (i < N) {
    int slot = -1;
    if (act) {
      slot = chunk_base[(size_t)blockIdx.x * E + v] + rank;
      for (int w = 0; w < wv; ++w) slot += wcnt[w][v];
      slot_to_row[slot] = i;
    }
    row_to_slot[i] = slot;
  }
}

// ---------------------------------------------------------------------------
// Planner
// ---------------------------------------------------------------------------
MOE_DEV long long wave_max64(long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    long long o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}
// max over lanes 0..7 (the xor partners 4, 2, 1 stay inside each group of
// eight lanes), returned to every lane from lane 0
MOE_DEV long long lanes8_max64(long long v) {
#pragma unroll
  for (int off = 4; off > 0; off >>= 1) {
    long long o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return __shfl(v, 0, 64);
}
MOE_DEV int wave_max32(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    int o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

__global__ __launch_bounds__(256) void k_plan(const int32_t* __restrict__ bcnt,
                                              const int32_t* __restrict__ boff,
                                              const int32_t* __restrict__ owner, int E, int P,
                                              int s, int mode, int lam, int32_t* q_out,
                                              int32_t* load_out, int32_t* bw_out,
                                              int bw_cap, int32_t* info_out, int32_t* status) {
  extern __shared__ int sm[];
  int* b_s = sm;                     // [E]
  int* h_s = b_s + E;                // [E]
  int* boff_s = h_s + E;             // [E+1]
  int* qh_s = boff_s + E + 1;        // [4][E]   q[e][h(e)] per search
  int* qn_s = qh_s + 4 * E;          // [4][E][8] q[e][t], t != h(e)
  __shared__ int res_obj[4], res_rep[4], res_ell[4][kMaxP], best_w;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int e = tid; e < E; e += 256) {
    b_s[e] = bcnt[e];
    int h = owner[e];
    if (h < 0 || h >= P) { atomicOr(status, MOE_DEV_BAD_OWNER); h = 0; }
    h_s[e] = h;
  }
  for (int e = tid; e <= E; e += 256) boff_s[e] = boff[e];
  for (int i = tid; i < 4 * E * 8; i += 256) qn_s[i] = 0;
  __syncthreads();

  const bool bwd = (mode == MOE_PLAN_BWD);
  const bool homeload_key = (w >= 2);
  const bool fan_one = (w % 2) == 0;
  int* qh = qh_s + w * E;
  int* qn = qn_s + w * E * 8;

  long long Bp = 0;
  for (int e = lane; e < E; e += 64) Bp += b_s[e];
  const long long B = wave_sum64(Bp);
  const int tau = (int)((B + P - 1) / P);

  // worker state lives on lane r < P
  int ell = 0, rep = 0, nrem = 0;
  for (int e = lane; e < E; e += 64) qh[e] = b_s[e];
  for (int r = 0; r < P; ++r) {
    int part = 0;
    for (int e = lane; e < E; e += 64)
      if (h_s[e] == r) part += b_s[e];
    const int tot = wave_sum(part);
    if (lane == r) ell = tot;
  }

  for (int round = 0; round < P; ++round) {
    bool moved = false;
    const int myL0 = ell + (bwd ? lam * nrem : 0);
    int key = myL0 - tau;
    if (homeload_key) {
      key = 0;
      for (int r = 0; r < P; ++r) {
        int m = 0;
        for (int e = lane; e < E; e += 64)
          if (h_s[e] == r && qh[e] > m) m = qh[e];
        m = wave_max32(m);
        if (lane == r) key = m;
      }
    }
    const bool isdon = (lane < P) && (myL0 > tau);
    int rank = 0;
    for (int r2 = 0; r2 < P; ++r2) {
      const int k2 = __shfl(key, r2, 64);
      const int d2 = __shfl((int)isdon, r2, 64);
      if (d2 && (k2 > key || (k2 == key && r2 < lane))) ++rank;
    }
    const int ndon = __popcll(__ballot(isdon));
    for (int j = 0; j < ndon; ++j) {
      const int r = __ffsll((unsigned long long)__ballot(isdon && rank == j)) - 1;
      uint32_t done = 0;
      // Each pass marks one expert done, so E passes suffice; the cap only
      // guards against a logic error ever spinning forever on the device.
      for (int guard_e = 0; guard_e <= E; ++guard_e) {
        const int Lr0 = __shfl(ell, r, 64) + (bwd ? lam * __shfl(nrem, r, 64) : 0);
        if (Lr0 <= tau) break;
        // Backward mode: a home expert with at most lambda blocks and no copy
        // elsewhere has no candidate (a new copy must move more than lambda
        // blocks), and a failed search changes nothing, so it is skipped
        // here rather than searched.  No move of another expert can give it
        // a copy, so the experts that remain keep their snapshot order.
        long long bk = 0;
        for (int i = 0, e = lane; e < E; ++i, e += 64)
          if (h_s[e] == r && !((done >> i) & 1u) && qh[e] > 0) {
            bool can = !bwd || qh[e] > lam;
            if (!can) {
              int any = 0;
#pragma unroll
              for (int t = 0; t < 8; ++t) any |= qn[e * 8 + t];
              can = any != 0;                   // copy counts are never negative
            }
            if (!can) continue;
            const long long kk = ((long long)qh[e] << 32) | (long long)(0xFFFFFFFFu - (uint32_t)e);
            if (kk > bk) bk = kk;
          }
        bk = wave_max64(bk);
        if (bk == 0) break;
        const int e = (int)(0xFFFFFFFFu - (uint32_t)(bk & 0xFFFFFFFFll));
        int qer = (int)(bk >> 32);
        if (lane == (e & 63)) done |= 1u << (e >> 6);
        bool nc = false;
        // every move strictly lowers the donor's effective load (delta >= 1,
        // and a backward copy needs delta > lambda), so moves are bounded by it
        for (int guard_m = 0; guard_m <= Lr0 + 1; ++guard_m) {
          const int Lr = __shfl(ell, r, 64) + (bwd ? lam * __shfl(nrem, r, 64) : 0);
          if (Lr <= tau || qer <= 0) break;
          long long cand = -1;
          int dl = 0, isnew = 0;
          if (lane < P && lane != r) {
            const int Lt = ell + (bwd ? lam * nrem : 0);
            if (Lt < tau) {
              const int qet = qn[e * 8 + lane];
              bool ok = true;
              int delta = 0;
              if (qet > 0) {
                delta = min(min(Lr - tau, tau - Lt), qer);
              } else if (rep >= s || (fan_one && nc)) {
                ok = false;
              } else if (bwd) {
                delta = min(min(Lr - tau + lam, tau - Lt), qer);
                ok = delta > lam;
                isnew = 1;
              } else {
                delta = min(min(Lr - tau, tau - Lt), qer);
                isnew = 1;
              }
              if (ok) {
                cand = ((long long)(tau - Lt) << 8) | (long long)(255 - lane);
                dl = delta;
              }
            }
          }
          const long long bc = lanes8_max64(cand);     // candidates live on lanes t < P <= 8
          if (bc < 0) break;
          const int t = 255 - (int)(bc & 255);
          const int delta = __shfl(dl, t, 64);
          const int nw = __shfl(isnew, t, 64);
          if (lane == r) { ell -= delta; nrem += nw; }
          if (lane == t) { ell += delta; rep += nw; qn[e * 8 + t] += delta; }
          qer -= delta;
          if (nw) nc = true;
          moved = true;
        }
        if (lane == (e & 63)) qh[e] = qer;
      }
    }
    const int maxL = wave_max32(lane < P ? ell + (bwd ? lam * nrem : 0) : INT_MIN);
    if (!moved || maxL <= tau) break;
  }
  const int obj = wave_max32(lane < P ? ell + (bwd ? lam * nrem : 0) : INT_MIN);
  const int reps = wave_sum(lane < P ? rep : 0);
  if (lane == 0) { res_obj[w] = obj; res_rep[w] = reps; }
  if (lane < P) res_ell[w][lane] = ell;
  __syncthreads();
  if (tid == 0) {
    int bw = 0;
    for (int c = 1; c < 4; ++c)
      if (res_obj[c] < res_obj[bw] || (res_obj[c] == res_obj[bw] && res_rep[c] < res_rep[bw]))
        bw = c;
    best_w = bw;
    info_out[0] = res_obj[bw];
    info_out[1] = bw;
    info_out[2] = res_rep[bw];
    info_out[3] = tau;
  }
  __syncthreads();
  const int W = best_w;
  const int* qhb = qh_s + W * E;
  const int* qnb = qn_s + W * E * 8;
  if (tid < P) load_out[tid] = res_ell[W][tid];
  for (int i = tid; i < E * P; i += 256) {
    const int e = i / P, t = i % P;
    q_out[i] = (t == h_s[e]) ? qhb[e] : qnb[e * 8 + t];
  }
  const int nb = boff_s[E];
  if (nb > bw_cap) {                 // block_worker cannot hold the plan: nothing written
    if (tid == 0) atomicOr(status, MOE_DEV_BAD_PLAN);
    return;
  }
  for (int g = tid; g < nb; g += 256) {
    int lo = 0, hi = E;  // largest e with boff_s[e] <= g
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (boff_s[mid] <= g) lo = mid; else hi = mid;
    }
    const int e = lo, h = h_s[e];
    int i = g - boff_s[e];
    int wk = h;
    if (i >= qhb[e]) {
      i -= qhb[e];
      for (int t = 0; t < P; ++t) {
        if (t == h) continue;
        const int qt = qnb[e * 8 + t];
        if (i < qt) { wk = t; break; }
        i -= qt;
      }
    }
    bw_out[g] = wk;
  }
}

// ---------------------------------------------------------------------------
// Quota-driven planner (UltraEP reading notes, section 4 "The Quota-Driven
// Planning Solver", Algorithm 1), in block units: the smallest load threshold
// tau in [ceil(B/P), max fixed load] that one greedy pass meets, found by
// binary search.  A pass at tau starts from the fixed placement with
// exc_r = max(l_r - tau, 0), slk_r = max(tau - l_r, 0); overloaded workers by
// decreasing excess (ties: smaller r) hand their own experts (by decreasing
// b_e, ties: smaller e) to the worker with the most slack that does not host
// the expert yet and has a free replica slot (ties: smaller t), in amounts
// min(exc_r, slk_t, blocks left on r), but only when that is >= u_min.
//
// An expert's blocks and its set of hosts change only while that expert is
// being handed out, so a pass needs no per-expert state beyond the expert in
// hand: lane r of a wave holds worker r's load, excess, slack and replica
// count, and the expert order is a table built once.  Seven waves evaluate the
// next three levels of the binary search at once (the root's midpoint and
// the midpoints of every interval either answer can leave), which gives the
// same threshold as probing one midpoint at a time in a third of the rounds.
// The eighth wave then replays the pass at the chosen tau and records the
// moves for the outputs.
// ---------------------------------------------------------------------------
constexpr int kQuotaWaves = 8, kQuotaProbes = 7;

// One feasibility pass at tau on one wave.  With `moves` non-null the blocks
// each recipient takes are added to moves[e * 8 + t].  Lane r < P ends with
// worker r's load and replica count.
MOE_DEV bool quota_pass(int tau, int E, int P, int s, int umin, const int* b_s, const int* ord_s,
                        const int* goff_s, const int* ell0_s, int lane, int& ell, int& rep,
                        int* moves) {
  ell = lane < P ? ell0_s[lane] : 0;
  int exc = lane < P ? max(ell - tau, 0) : 0;
  int slk = lane < P ? max(tau - ell, 0) : 0;
  rep = 0;
  const bool isdon = exc > 0;
  int rank = 0;
  for (int r2 = 0; r2 < P; ++r2) {
    const int x2 = __shfl(exc, r2, 64);
    if (x2 > 0 && (x2 > exc || (x2 == exc && r2 < lane))) ++rank;
  }
  const int ndon = __popcll(__ballot(isdon));
  for (int j = 0; j < ndon; ++j) {
    const int r = __ffsll((unsigned long long)__ballot(isdon && rank == j)) - 1;
    for (int idx = goff_s[r]; idx < goff_s[r + 1]; ++idx) {
      if (__shfl(exc, r, 64) == 0) break;
      const int e = ord_s[idx];
      int left = b_s[e];                 // blocks of e still on r
      uint32_t hosts = 1u << r;          // workers holding a copy of e
      // each transfer gives e to a new worker, so at most P - 1 of them
      for (int guard = 0; guard < P && left > 0; ++guard) {
        const int er = __shfl(exc, r, 64);
        if (er == 0) break;
        long long cand = -1;
        if (lane < P && !((hosts >> lane) & 1u) && rep < s && slk > 0)
          cand = ((long long)slk << 8) | (long long)(255 - lane);
        const long long bc = wave_max64(cand);
        if (bc < 0) break;
        const int t = 255 - (int)(bc & 255);
        const int delta = min(min(er, (int)(bc >> 8)), left);
        if (delta < umin) break;
        if (lane == r) { exc -= delta; ell -= delta; }
        if (lane == t) { slk -= delta; ell += delta; rep += 1; }
        if (moves && lane == 0) moves[e * 8 + t] += delta;
        hosts |= 1u << t;
        left -= delta;
      }
    }
  }
  return __ballot(lane < P && exc > 0) == 0;
}

__global__ __launch_bounds__(512) void k_plan_quota(const int32_t* __restrict__ bcnt,
                                                    const int32_t* __restrict__ boff,
                                                    const int32_t* __restrict__ owner, int E,
                                                    int P, int s, int umin, int32_t* q_out,
                                                    int32_t* load_out, int32_t* bw_out,
                                                    int bw_cap, int32_t* info_out,
                                                    int32_t* status) {
  extern __shared__ int sm[];
  int* b_s = sm;                     // [E]
  int* h_s = b_s + E;                // [E]
  int* boff_s = h_s + E;             // [E+1]
  int* ord_s = boff_s + E + 1;       // [E] experts grouped by owner, by b desc, e asc
  int* mv_s = ord_s + E;             // [E][8] blocks moved from e's owner to t
  __shared__ int goff_s[kMaxP + 1], gcnt_s[kMaxP], ell0_s[kMaxP], feas_s[kQuotaProbes];
  __shared__ int lo_s, hi_s, fin_ell[kMaxP], fin_rep;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid < kMaxP) { gcnt_s[tid] = 0; ell0_s[tid] = 0; }
  __syncthreads();
  for (int e = tid; e < E; e += 512) {
    b_s[e] = bcnt[e];
    int h = owner[e];
    if (h < 0 || h >= P) { atomicOr(status, MOE_DEV_BAD_OWNER); h = 0; }
    h_s[e] = h;
    atomicAdd(&gcnt_s[h], 1);
    atomicAdd(&ell0_s[h], bcnt[e]);
  }
  for (int e = tid; e <= E; e += 512) boff_s[e] = boff[e];
  for (int i = tid; i < E * 8; i += 512) mv_s[i] = 0;
  __syncthreads();
  if (tid == 0) {
    goff_s[0] = 0;
    for (int r = 0; r < P; ++r) goff_s[r + 1] = goff_s[r] + gcnt_s[r];
    long long B = 0;
    int mx = 0;
    for (int r = 0; r < P; ++r) { B += ell0_s[r]; mx = max(mx, ell0_s[r]); }
    lo_s = (int)((B + P - 1) / P);
    hi_s = mx;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 512) {   // place e inside its owner's group
    const int h = h_s[e], be = b_s[e];
    int pos = goff_s[h];
    for (int e2 = 0; e2 < E; ++e2)
      if (h_s[e2] == h && (b_s[e2] > be || (b_s[e2] == be && e2 < e))) ++pos;
    ord_s[pos] = e;
  }
  __syncthreads();

  // binary search, three levels per round: probe wave i takes node i of the
  // next three levels (heap order) and the walk below follows the answers
  // exactly as a one-midpoint-at-a-time search would
  for (int round = 0; round < 32; ++round) {
    const int lo = lo_s, hi = hi_s;
    if (lo >= hi) break;
    if (w < kQuotaProbes) {
      int a = lo, bnd = hi;
      const int path = w + 1;                 // heap index + 1: bits below the top bit are the turns
      const int depth = 31 - __clz(path);
      for (int d = depth - 1; d >= 0; --d) {
        const int mid = (a + bnd) >> 1;
        if ((path >> d) & 1) a = mid + 1; else bnd = mid;   // right: infeasible at mid
      }
      int f = -1;
      if (a < bnd) {
        int ell, rep;
        f = quota_pass((a + bnd) >> 1, E, P, s, umin, b_s, ord_s, goff_s, ell0_s, lane, ell, rep,
                       nullptr) ? 1 : 0;
      }
      if (lane == 0) feas_s[w] = f;
    }
    __syncthreads();
    if (tid == 0) {
      int a = lo, bnd = hi, i = 0;
      for (int d = 0; d < 3 && a < bnd; ++d) {
        const int mid = (a + bnd) >> 1;
        if (feas_s[i] == 1) { bnd = mid; i = 2 * i + 1; } else { a = mid + 1; i = 2 * i + 2; }
      }
      lo_s = a;
      hi_s = bnd;
    }
    __syncthreads();
  }
  const int tau = lo_s;
  if (w == kQuotaWaves - 1) {
    int ell, rep;
    quota_pass(tau, E, P, s, umin, b_s, ord_s, goff_s, ell0_s, lane, ell, rep, mv_s);
    if (lane < P) fin_ell[lane] = ell;
    const int reps = wave_sum(lane < P ? rep : 0);
    if (lane == 0) fin_rep = reps;
  }
  __syncthreads();
  if (tid == 0) {
    int obj = 0;
    for (int r = 0; r < P; ++r) obj = max(obj, fin_ell[r]);
    info_out[0] = obj;
    info_out[1] = 4;
    info_out[2] = fin_rep;
    info_out[3] = tau;
  }
  if (tid < P) load_out[tid] = fin_ell[tid];
  for (int i = tid; i < E * P; i += 512) {
    const int e = i / P, t = i % P;
    int moved = 0;
    for (int u = 0; u < P; ++u) moved += mv_s[e * 8 + u];
    q_out[i] = (t == h_s[e]) ? b_s[e] - moved : mv_s[e * 8 + t];
  }
  const int nb = boff_s[E];
  if (nb > bw_cap) {                 // block_worker cannot hold the plan: nothing written
    if (tid == 0) atomicOr(status, MOE_DEV_BAD_PLAN);
    return;
  }
  for (int g = tid; g < nb; g += 512) {
    int lo = 0, hi = E;  // largest e with boff_s[e] <= g
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (boff_s[mid] <= g) lo = mid; else hi = mid;
    }
    const int e = lo, h = h_s[e];
    int moved = 0;
    for (int u = 0; u < P; ++u) moved += mv_s[e * 8 + u];
    int i = g - boff_s[e];
    int wk = h;
    if (i >= b_s[e] - moved) {
      i -= b_s[e] - moved;
      for (int t = 0; t < P; ++t) {
        if (t == h) continue;
        const int qt = mv_s[e * 8 + t];
        if (i < qt) { wk = t; break; }
        i -= qt;
      }
    }
    bw_out[g] = wk;
  }
}

// ---------------------------------------------------------------------------
// Runtime replication gate (MegaFlux summary, "Limitations": replication only
// when the predicted saving exceeds its cost; "Empirical Validation": balanced
// routes gain nothing).  Predicted cost of a plan, in blocks on the busiest
// worker: objective + rho per replica (rho in thousandths of a block).  The
// plan stays when 1000 (fixed objective - plan objective) > rho * replicas;
// otherwise it is rewritten in place as the fixed placement with plan_info =
// {fixed objective, -1, 0, tau}.  A plan without replicas is left as it is.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_plan_gate(const int32_t* __restrict__ bcnt,
                                                   const int32_t* __restrict__ boff,
                                                   const int32_t* __restrict__ owner, int E, int P,
                                                   int rho_milli, int32_t* q, int32_t* load,
                                                   int32_t* bw, int bw_cap, int32_t* info,
                                                   int32_t* status) {
  __shared__ int ellfix[kMaxP], keep_s;
  const int tid = threadIdx.x;
  if (tid < kMaxP) ellfix[tid] = 0;
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    int h = owner[e];
    if (h < 0 || h >= P) { atomicOr(status, MOE_DEV_BAD_OWNER); h = 0; }
    atomicAdd(&ellfix[h], bcnt[e]);
  }
  __syncthreads();
  if (tid == 0) {
    int objfix = 0, objplan = 0;
    for (int r = 0; r < P; ++r) { objfix = max(objfix, ellfix[r]); objplan = max(objplan, load[r]); }
    const int reps = info[2];
    const bool keep = reps == 0 ||
                      1000LL * (long long)(objfix - objplan) > (long long)rho_milli * (long long)reps;
    keep_s = keep;
    if (!keep) {
      info[0] = objfix;
      info[1] = -1;
      info[2] = 0;
    }
  }
  __syncthreads();
  if (keep_s) return;
  if (tid < P) load[tid] = ellfix[tid];
  for (int i = tid; i < E * P; i += 256) {
    const int e = i / P, t = i % P;
    int h = owner[e];
    if (h < 0 || h >= P) h = 0;
    q[i] = (t == h) ? bcnt[e] : 0;
  }
  const int nb = boff[E];
  if (nb > bw_cap) {                 // block_worker cannot hold the plan: nothing written
    if (tid == 0) atomicOr(status, MOE_DEV_BAD_PLAN);
    return;
  }
  for (int g = tid; g < nb; g += 256) {
    int lo = 0, hi = E;  // largest e with boff[e] <= g
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (boff[mid] <= g) lo = mid; else hi = mid;
    }
    int h = owner[lo];
    if (h < 0 || h >= P) h = 0;
    bw[g] = h;
  }
}

// ---------------------------------------------------------------------------
// Wave-quantized cost of a plan ("Analytical Resource Management for
// Fine-grained MoE Computation-Communication Overlap", abstract: choose the
// resource partition before the launch from routed-tile counts and occupancy,
// without candidate runs).  The resource partition here is P: a worker owns
// n = G / P workgroups and the persistent GEMM launches deal its items
// round-robin (workgroup j takes items j, j + n, ...), so a phase lasts as long
// as its busiest workgroup.  Items and their costs, in thousandths of a K step:
//   FC1, FC2, dA, dX: (row tile, N tile) pairs; a row tile is up to 256 slots
//   of one (expert, worker) run (beta | 256: ceil(blocks * beta / 256) per
//   run, else ceil(rows / 256) per block); cost = K / 64 steps plus the
//   epilogue's bytes over what one CU stores during a step (kEpiBytesPerStep);
//   weight gradients: (segment, 256 x 256 tile) pairs, replica segments first,
//   cost = max(2, ceil(rows / 64)) steps plus the fp32 tile's epilogue.
// One workgroup; every quantity is an integer.
// ---------------------------------------------------------------------------
constexpr long long kEpiBytesPerStep = 214000;
MOE_DEV long long epi_milli(long long bytes) { return bytes * 1000 / kEpiBytesPerStep; }
MOE_DEV long long ceil_div_ll(long long a, long long b) { return (a + b - 1) / b; }

__global__ __launch_bounds__(256) void k_predict_cost(const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ boff,
                                                      const int32_t* __restrict__ bw_f,
                                                      const int32_t* __restrict__ bw_b,
                                                      const int32_t* __restrict__ owner, int E,
                                                      int beta, int P, int d, int dff, int G,
                                                      long long* cost_out, int32_t* status) {
  extern __shared__ int sm[];
  int* cnt_s = sm;                    // [E]
  int* boff_s = cnt_s + E;            // [E+1]
  int* own_s = boff_s + E + 1;        // [E]
  int* nbf_s = own_s + E;             // [E][P] blocks of e on worker w, forward plan
  int* nbb_s = nbf_s + E * P;         // [E][P] same, backward plan
  int* rows_s = nbb_s + E * P;        // [E][P] valid rows of e on w, backward plan
  __shared__ int tiles_s[2][kMaxP];   // per-block tiles when beta does not divide 256
  __shared__ long long red_s[256];
  const int tid = threadIdx.x;
  constexpr int bm = 256;
  for (int e = tid; e < E; e += 256) {
    cnt_s[e] = counts[e];
    int h = owner[e];
    if (h < 0 || h >= P) { atomicOr(status, MOE_DEV_BAD_OWNER); h = 0; }
    own_s[e] = h;
  }
  for (int e = tid; e <= E; e += 256) boff_s[e] = boff[e];
  for (int i = tid; i < 3 * E * P; i += 256) nbf_s[i] = 0;
  if (tid < 2 * kMaxP) tiles_s[tid / kMaxP][tid % kMaxP] = 0;
  __syncthreads();
  const int nb = boff_s[E];
  for (int g = tid; g < nb; g += 256) {
    int lo = 0, hi = E;  // largest e with boff_s[e] <= g
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (boff_s[mid] <= g) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int vrows = min(beta, cnt_s[e] - beta * (g - boff_s[e]));
    int wf = bw_f[g], wb = bw_b[g];
    if (wf < 0 || wf >= P || wb < 0 || wb >= P) { atomicOr(status, MOE_DEV_BAD_PLAN); wf = wb = 0; }
    atomicAdd(&nbf_s[e * P + wf], 1);
    atomicAdd(&nbb_s[e * P + wb], 1);
    atomicAdd(&rows_s[e * P + wb], vrows);
    if (bm % beta != 0) {
      atomicAdd(&tiles_s[0][wf], (vrows + bm - 1) / bm);
      atomicAdd(&tiles_s[1][wb], (vrows + bm - 1) / bm);
    }
  }
  __syncthreads();
  const int n = G / P;
  // thread j < n is workgroup j of every worker in the weight-gradient phase
  long long dw = 0;
  if (tid < n) {
    const long long per_seg = (long long)(d / 256) * (dff / 256) + (long long)(2 * dff / 256) * (d / 256);
    const long long dwe = epi_milli(256LL * 256 * 4);
    for (int r = 0; r < P; ++r) {
      long long mine = 0, pos = 0;
      for (int pass = 0; pass < 2; ++pass)
        for (int e = 0; e < E; ++e) {
          const int rows = rows_s[e * P + r];
          if (rows <= 0 || (own_s[e] == r) != (pass == 1)) continue;
          const long long c = 1000LL * max(2, (rows + 63) / 64) + dwe;
          const long long base = pos * per_seg;
          const long long t0 = ((tid - base) % n + n) % n;     // first tile of this segment on j
          if (t0 < per_seg) mine += c * (1 + (per_seg - 1 - t0) / n);
          ++pos;
        }
      dw = max(dw, mine);
    }
  }
  red_s[tid] = dw;
  __syncthreads();
  if (tid == 0) {
    long long dwmax = 0;
    for (int j = 0; j < 256; ++j) dwmax = max(dwmax, red_s[j]);
    long long tf[kMaxP], tb[kMaxP];
    for (int r = 0; r < P; ++r) {
      if (bm % beta == 0) {
        const int f = bm / beta;
        long long a = 0, b = 0;
        for (int e = 0; e < E; ++e) {
          a += (nbf_s[e * P + r] + f - 1) / f;
          b += (nbb_s[e * P + r] + f - 1) / f;
        }
        tf[r] = a;
        tb[r] = b;
      } else {
        tf[r] = tiles_s[0][r];
        tb[r] = tiles_s[1][r];
      }
    }
    const long long fc1 = 1000LL * (d / 64) + epi_milli((long long)bm * (128 + 256) * 2);
    const long long fc2 = 1000LL * (dff / 64) + epi_milli((long long)bm * 256 * 2);
    const long long da = 1000LL * (d / 64) + epi_milli((long long)bm * 256 * 3 * 2 + (long long)bm * 512 * 2);
    const long long dx = 1000LL * (2 * dff / 64) + epi_milli((long long)bm * 256 * 2);
    long long p1 = 0, p2 = 0, p3 = 0, p4 = 0;
    for (int r = 0; r < P; ++r) {
      p1 = max(p1, ceil_div_ll(tf[r] * (2 * dff / 256), n) * fc1);
      p2 = max(p2, ceil_div_ll(tf[r] * (d / 256), n) * fc2);
      p3 = max(p3, ceil_div_ll(tb[r] * (dff / 256), n) * da);
      p4 = max(p4, ceil_div_ll(tb[r] * (d / 256), n) * dx);
    }
    *cost_out = p1 + p2 + p3 + p4 + dwmax;
  }
}

// ---------------------------------------------------------------------------
// Producer/consumer split of a two-phase launch (same page: the count of
// producer CTAs of a dependency-coupled pipeline, chosen before the launch
// from routed-tile counts and split-level readiness).  The pair is FC1 -> FC2
// (forward) or dA -> dX (backward); a second-phase item of row tile t needs
// every first-phase item of row tile t.  Worker r has T_r row tiles and
// n = G / P workgroups; items are tile-major (item i: row tile i / nnt) and
// all items of a phase cost the same (c1, c2: K steps plus the epilogue, as
// in the cost model above).  Modes:
//   -1  two launches: max_r ceil(T_r nnt1 / n) c1 + max_r ceil(T_r nnt2 / n) c2;
//    0  one launch, every workgroup j runs first-phase items j, j + n, ...,
//       then second-phase items j, j + n, ...;
//   n1  one launch, workgroups j < n1 deal the first-phase items, the other
//       n - n1 the second-phase items.
// A first-phase item i dealt over m workgroups ends at (i / m + 1) c1, so row
// tile t is ready at ((t nnt1 + nnt1 - 1) / m + 1) c1; a second-phase item
// starts when its workgroup is free and its row tile is ready.  A mode costs
// its latest workgroup over every worker.  One thread per mode.
// ---------------------------------------------------------------------------
MOE_DEV long long split_ready(long long t, int nnt1, int m, long long c1) {
  return ((t * nnt1 + nnt1 - 1) / m + 1) * c1;
}

__global__ __launch_bounds__(256) void k_predict_split(const int32_t* __restrict__ counts,
                                                       const int32_t* __restrict__ boff,
                                                       const int32_t* __restrict__ bw, int E,
                                                       int beta, int P, int d, int dff, int G,
                                                       int backward, long long* cost_out,
                                                       int32_t* choice_out, int32_t* status) {
  extern __shared__ int sm[];
  int* cnt_s = sm;                    // [E]
  int* boff_s = cnt_s + E;            // [E+1]
  int* nb_s = boff_s + E + 1;         // [E][P] blocks of e on worker w
  __shared__ int tiles_s[kMaxP];      // per-block tiles when beta does not divide 256
  __shared__ long long tr_s[kMaxP];   // row tiles of each worker
  __shared__ long long cost_s[257];
  const int tid = threadIdx.x;
  constexpr int bm = 256;
  for (int e = tid; e < E; e += 256) cnt_s[e] = counts[e];
  for (int e = tid; e <= E; e += 256) boff_s[e] = boff[e];
  for (int i = tid; i < E * P; i += 256) nb_s[i] = 0;
  if (tid < kMaxP) tiles_s[tid] = 0;
  __syncthreads();
  const int nb = boff_s[E];
  for (int g = tid; g < nb; g += 256) {
    int lo = 0, hi = E;  // largest e with boff_s[e] <= g
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (boff_s[mid] <= g) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int vrows = min(beta, cnt_s[e] - beta * (g - boff_s[e]));
    int w = bw[g];
    if (w < 0 || w >= P) { atomicOr(status, MOE_DEV_BAD_PLAN); w = 0; }
    atomicAdd(&nb_s[e * P + w], 1);
    if (bm % beta != 0) atomicAdd(&tiles_s[w], (vrows + bm - 1) / bm);
  }
  __syncthreads();
  if (tid < P) {
    long long t = 0;
    if (bm % beta == 0) {
      const int f = bm / beta;
      for (int e = 0; e < E; ++e) t += (nb_s[e * P + tid] + f - 1) / f;
    } else {
      t = tiles_s[tid];
    }
    tr_s[tid] = t;
  }
  __syncthreads();
  const int n = G / P;
  int nnt1, nnt2;
  long long c1, c2;
  if (backward) {
    nnt1 = dff / 256;
    nnt2 = d / 256;
    c1 = 1000LL * (d / 64) + epi_milli((long long)bm * 256 * 3 * 2 + (long long)bm * 512 * 2);
    c2 = 1000LL * (2 * dff / 64) + epi_milli((long long)bm * 256 * 2);
  } else {
    nnt1 = 2 * dff / 256;
    nnt2 = d / 256;
    c1 = 1000LL * (d / 64) + epi_milli((long long)bm * (128 + 256) * 2);
    c2 = 1000LL * (dff / 64) + epi_milli((long long)bm * 256 * 2);
  }
  for (int m = tid - 1; m < n; m += 256) {
    long long worst = 0;
    if (m == -1) {
      long long m1 = 0, m2 = 0;
      for (int r = 0; r < P; ++r) {
        m1 = max(m1, ceil_div_ll(tr_s[r] * nnt1, n));
        m2 = max(m2, ceil_div_ll(tr_s[r] * nnt2, n));
      }
      worst = m1 * c1 + m2 * c2;
    } else {
      for (int r = 0; r < P; ++r) {
        const long long N1 = tr_s[r] * nnt1, N2 = tr_s[r] * nnt2;
        if (m == 0) {
          for (int j = 0; j < n; ++j) {
            long long clock = (j < N1 ? (N1 - 1 - j) / n + 1 : 0) * c1;
            for (long long i2 = j; i2 < N2; i2 += n)
              clock = max(clock, split_ready(i2 / nnt2, nnt1, n, c1)) + c2;
            worst = max(worst, clock);
          }
        } else {
          const int n1 = m, n2 = n - m;
          worst = max(worst, ceil_div_ll(N1, n1) * c1);
          for (int j = 0; j < n2; ++j) {
            long long clock = 0;
            for (long long i2 = j; i2 < N2; i2 += n2)
              clock = max(clock, split_ready(i2 / nnt2, nnt1, n1, c1)) + c2;
            worst = max(worst, clock);
          }
        }
      }
    }
    cost_s[m + 1] = worst;
    cost_out[m + 1] = worst;
  }
  __syncthreads();
  if (tid == 0) {
    int best = 0;
    for (int i = 1; i <= n; ++i)
      if (cost_s[i] < cost_s[best]) best = i;
    *choice_out = best - 1;
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
size_t route_ws_bytes(int T, int k, int E) {
  const long long N = (long long)T * k;
  const long long nch = N > 0 ? (N + kChunk - 1) / kChunk : 1;
  return align_up((size_t)nch * E * sizeof(int32_t));
}

int launch_route_stats(const int32_t* ids, int T, int k, int E, int beta, int32_t* counts,
                       int32_t* offsets, int32_t* block_counts, int32_t* block_offsets,
                       int32_t* row_to_slot, int32_t* slot_to_row, double* kappa,
                       int32_t* status, void* ws, hipStream_t st) {
  const int N = T * k;
  const int nch = N > 0 ? (N + kChunk - 1) / kChunk : 1;
  const int cap = N + E * (beta - 1);
  int32_t* chunk = (int32_t*)ws;
  hipLaunchKernelGGL(k_route_count, dim3(nch), dim3(kChunk), 0, st, ids, N, E, chunk,
                     slot_to_row, cap, status);
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, st, chunk, nch, E, beta, counts,
                     offsets, block_counts, block_offsets, kappa);
  if (N > 0)
    hipLaunchKernelGGL(k_route_slot, dim3(nch), dim3(kChunk), 0, st, ids, N, E, chunk,
                       row_to_slot, slot_to_row);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// ---- routing statistics without a caller workspace -----------------------------
// For callers that cannot allocate: the per-chunk counts live in a file-scope
// device array, one copy per GPU, held until the process ends.  Host code
// never hands the array's name to a kernel (on the host it is only a stand-in
// for the symbol): its device address is looked up once per device, with that
// device current, and kept.  Every call writes the counts it reads before
// reading them, so nothing needs clearing between calls; calls that overlap in
// time on one GPU share the array and race.
static __device__ __align__(256) int32_t scratch[kRouteScratchBytes / sizeof(int32_t)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

int route_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

int launch_plan(const int32_t* bcnt, const int32_t* boff, const int32_t* owner, int E, int P,
                int s, int mode, int lam, int32_t* q, int32_t* load, int32_t* bw, int bw_cap,
                int32_t* info, int32_t* status, hipStream_t st) {
  if (mode == MOE_PLAN_QUOTA) {
    const size_t lds = sizeof(int) * (size_t)(4 * E + 1 + 8 * E);
    hipLaunchKernelGGL(k_plan_quota, dim3(1), dim3(512), lds, st, bcnt, boff, owner, E, P, s,
                       lam, q, load, bw, bw_cap, info, status);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
  const size_t lds = sizeof(int) * (size_t)(3 * E + 1 + 4 * E + 4 * E * 8);
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(256), lds, st, bcnt, boff, owner, E, P, s, mode,
                     lam, q, load, bw, bw_cap, info, status);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_plan_gate(const int32_t* bcnt, const int32_t* boff, const int32_t* owner, int E, int P,
                     int rho_milli, int32_t* q, int32_t* load, int32_t* bw, int bw_cap,
                     int32_t* info, int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(k_plan_gate, dim3(1), dim3(256), 0, st, bcnt, boff, owner, E, P, rho_milli,
                     q, load, bw, bw_cap, info, status);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_predict_cost(const int32_t* counts, const int32_t* boff, const int32_t* bw_f,
                        const int32_t* bw_b, const int32_t* owner, int E, int beta, int P, int d,
                        int dff, int G, long long* cost, int32_t* status, hipStream_t st) {
  const size_t lds = sizeof(int) * (size_t)(3 * E + 1 + 3 * E * P);
  hipLaunchKernelGGL(k_predict_cost, dim3(1), dim3(256), lds, st, counts, boff, bw_f, bw_b,
                     owner, E, beta, P, d, dff, G, cost, status);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_predict_split(const int32_t* counts, const int32_t* boff, const int32_t* bw, int E,
                         int beta, int P, int d, int dff, int G, int backward, long long* costs,
                         int32_t* choice, int32_t* status, hipStream_t st) {
  const size_t lds = sizeof(int) * (size_t)(2 * E + 1 + E * P);
  hipLaunchKernelGGL(k_predict_split, dim3(1), dim3(256), lds, st, counts, boff, bw, E, beta, P, d,
                     dff, G, backward, costs, choice, status);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
