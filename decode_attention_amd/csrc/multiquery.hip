// Paged attention of several queries per sequence (chunked prefill,
// speculative verification): the S queries of a sequence with L cached
// tokens sit at positions L - S .. L - 1 (their own keys are already in the
// cache) and each sees the keys l <= its position p; on sliding layers only
// those with p - w < l.
//
// Pages: Op Specs of google/gemma-4-12B, Attention.lean (causalGQA,
// slidingGQA); gemma-4-12b Model Spec, the attn.core rows of the sliding and
// global layers (head map h / G, scale 1, values = keys on global layers).
//
// Rows. A query row is one (query, head) pair of one KV head: on sliding
// layers its G = 2 heads, on global layers the 16 heads of the single KV head.
// A workgroup takes a block of 128 rows of one (sequence, KV head): on
// sliding layers 64 queries (mq_kernel, 8 waves of 16 rows x 256
// coordinates), on global layers 8 queries (mq_global_kernel, below), so that
// speculative verification of up to 8 draft tokens reads each sequence's
// keys once. Sliding calls with 128 or more queries in a sequence take
// 256-row blocks of 32-row tiles instead (mq_sliding_kernel, below).
//
// Sliding (mq_kernel). The workgroup walks the pages that some row of its block can see,
// two pages per step, staged in LDS (double-buffered), with the loads of the
// next two steps held in registers. Per step and wave:
//   S^T (16 tokens x 16 rows) = K Q^T: 8 mfma_f32_16x16x32_bf16 per page, K
//     read from LDS in the A-operand layout, Q^T kept in registers;
//   per-row masks (l <= p, and l > p - w on sliding layers), online softmax
//     in base 2 with lazy rescaling;
//   O^T (256 x 16) += V^T P^T: one mfma_f32_16x16x32_bf16 per 16-coordinate
//     tile, its 32-wide k dimension holding the 16 tokens of each page; V^T
//     read transposed from LDS with ds_read_b64_tr_b16.
// P enters the product rounded to bf16 and the denominator sums the same
// rounded values, so every output is a weighted average whose weights are
// exact to about 2^-9 relative.
//
// Split over keys. A unit (sequence, KV head, row block) may have its pages
// divided among several workgroups that write partial (acc, m, l) per row,
// and mq_merge_kernel combines them: M = max m_i,
// o = sum 2^(m_i - M) acc_i / sum 2^(m_i - M) l_i. By default:
//   sliding layers, when the units give too few workgroups for the chip: the
//     number of pieces of a unit follows its page count, so that long
//     sequences do not form the tail (mq_plan_kernel lays the pieces out and
//     gives every workgroup a descriptor (unit, piece, pieces, slot));
//   global layers, always: one workgroup per compute unit, each taking an
//     equal share of the steps of all units laid end to end
//     (mq_plan_contig_kernel), so that no workgroup runs longer than the
//     mean plus one step, whatever the mix of lengths.
// A caller-given number of splits divides every unit into that many pieces
// instead.
#include <algorithm>
#include <utility>

#include "common.hpp"
#include "launch.hpp"

namespace da {

constexpr int kMWaves = 8;
constexpr int kMThreads = kMWaves * kWave;
constexpr int kMSlice = 256;                 // coordinates per wave
constexpr int kMKSteps = kMSlice / 32;       // 16x16x32 k-steps per page and wave
constexpr int kMTiles = kMSlice / 16;        // 16-coordinate output tiles per wave
constexpr int kMRegion = 16384;              // LDS bytes per region of a step (2 pages of K, or of V)
constexpr float kMRescale = 32.f;            // lazy-rescale threshold, log2 units
constexpr int kMPlanThreads = 1024;          // one workgroup lays out a split
// Workgroups per compute unit of a split (measured on the 8-token
// verification workloads at B = 64: sliding 1, 2 and 6 slower than 3;
// global 2 and 3 slower than 1). A global workgroup takes all of a compute
// unit's LDS, so one per unit is a single round of workgroups and the fewest
// partial results to merge.
constexpr int kMPiecesPerCuSliding = 3;
constexpr int kMPiecesPerCuGlobal = 1;

struct MQArgs {
  const uint16_t* q;        // [T][Hq][D] bf16 bits; sequence b's rows from q_start[b]
  const uint16_t* k;        // sliding [P][Hkv][16][256]; global tiled [P][1][64][16][8]
  const uint16_t* v;        // sliding [P][Hkv][16][256]; global: the same as k
  const int32_t* bt;        // [B][P_max]
  const int32_t* seq_lens;  // [B]
  const int32_t* q_start;   // [B + 1]
  float* out;               // [T][Hq][D]
  float* ws;                // partial slots: [B*Hkv][nblk][nsplit][slot] (fixed split),
                            // [grid][slot] (balanced split) or [2 grid][slot] (contiguous)
  int* tab;                 // balanced split: [units + 1] first slot of each unit
  int4* desc;               // balanced split: [grid] (unit, piece, pieces, slot); unit -1: no work
  long long* hdr;           // contiguous split: {steps in all units, steps per workgroup}
  long long* off;           // contiguous split: [units + 1] first step of each unit
  int* wfirst;              // contiguous split: [grid] unit holding the workgroup's first step
  int B, Hkv, P_max, window, nblk, nsplit;
  int balanced;             // 1: pieces per unit follow its page count; 2: contiguous split
  int units, grid;          // balanced split: B*Hkv*nblk units over `grid` workgroups
};

template <int D, int G, int ROWS = 128>
struct MQShape {
  static_assert((D == 256 && G == 2) || (D == 512 && G == 16), "built shapes");
  static constexpr bool kSliding = D == 256;
  static constexpr int kRows = ROWS;                    // rows per workgroup
  static constexpr int kQueries = kRows / G;            // queries per workgroup
  static constexpr int kKPage = kSliding ? 8192 : 16384;  // LDS bytes per page of K (and of V)
  static constexpr int kVBase = kSliding ? kMRegion : 0;  // V region (global: V = K)
  static constexpr int kSlotFloats = kRows * D + 2 * kRows;
};

__device__ __forceinline__ int mq_rfl(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Element i of a layout array the plan kernel wrote, read as wave-uniform
// through the constant address space (a scalar load; the array is not
// written during the kernel).
template <typename T>
__device__ __forceinline__ T mq_sload(const T* p, long long i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

// Pages the rows of unit u = (sequence, KV head, row block) see, as the main
// kernel walks them (0 for a block without rows).
template <int D, int G, int ROWS = 128>
__device__ int mq_unit_pages(const MQArgs& a, int u) {
  using C = MQShape<D, G, ROWS>;
  const int blk = u % a.nblk, bc = u / a.nblk, b = bc / a.Hkv;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.P_max * kPage ? a.P_max * kPage : L);
  const int S = a.q_start[b + 1] - a.q_start[b];
  const int s0 = blk * C::kQueries;
  if (s0 >= S) return 0;
  const int p0 = L - S + s0, p1 = L - S + min(S, s0 + C::kQueries) - 1;
  const int klo = C::kSliding ? max(0, p0 - a.window + 1) : 0;
  const bool any = p1 >= 0 && (!C::kSliding || a.window > 0);
  return any ? p1 / kPage - klo / kPage + 1 : 0;
}

// Balanced split layout (one workgroup). A unit of n pages gets
// 1 + min(floor(n (grid - units) / total), n / 8) pieces, so the pieces of all
// units fit in the grid and hold about the same number of pages; unit u's
// pieces are slots tab[u] .. tab[u+1]-1, and workgroup w of the main kernel
// runs piece w - tab[u] of the unit with tab[u] <= w < tab[u+1].
template <int D, int G>
__global__ __launch_bounds__(kMPlanThreads) void mq_plan_kernel(MQArgs a) {
  __shared__ long long s_sum[kMPlanThreads];
  const int tid = threadIdx.x, U = a.units;
  const int per = (U + kMPlanThreads - 1) / kMPlanThreads, u0 = tid * per;
  long long loc = 0;
  for (int u = u0; u < u0 + per && u < U; ++u) loc += mq_unit_pages<D, G>(a, u);
  s_sum[tid] = loc;
  __syncthreads();
  for (int off = kMPlanThreads / 2; off > 0; off >>= 1) {
    if (tid < off) s_sum[tid] += s_sum[tid + off];
    __syncthreads();
  }
  const long long total = s_sum[0] > 0 ? s_sum[0] : 1;
  const long long spare = a.grid > U ? a.grid - U : 0;
  __syncthreads();
  int cnt = 0;
  for (int u = u0; u < u0 + per && u < U; ++u) {
    const int n = mq_unit_pages<D, G>(a, u);
    cnt += 1 + (int)min((long long)n * spare / total, (long long)(n / 8));
  }
  s_sum[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < kMPlanThreads; off <<= 1) {  // inclusive scan
    const long long v = tid >= off ? s_sum[tid - off] : 0;
    __syncthreads();
    s_sum[tid] += v;
    __syncthreads();
  }
  int run = (int)(s_sum[tid] - cnt);
  for (int u = u0; u < u0 + per && u < U; ++u) {
    const int n = mq_unit_pages<D, G>(a, u);
    const int k = 1 + (int)min((long long)n * spare / total, (long long)(n / 8));
    a.tab[u] = run;
    for (int i = 0; i < k; ++i) a.desc[run + i] = make_int4(u, i, k, run + i);
    run += k;
  }
  if (tid == kMPlanThreads - 1) a.tab[U] = run;  // the last thread's run is the total
  const int used = (int)s_sum[kMPlanThreads - 1];
  for (int w = used + tid; w < a.grid; w += kMPlanThreads) a.desc[w] = make_int4(-1, 0, 1, 0);
}

// Exclusive prefix sum over the plan workgroup (kMPlanThreads threads);
// `total` gets the sum of every thread's value.
template <typename T>
__device__ T mq_block_exscan(T v, T* s_w, T& total) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  T inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const T y = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += y;
  }
  if (lane == kWave - 1) s_w[wv] = inc;
  __syncthreads();
  T before = 0, all = 0;
  for (int i = 0; i < kMPlanThreads / kWave; ++i) {
    const T t = s_w[i];
    if (i < wv) before += t;
    all += t;
  }
  __syncthreads();
  total = all;
  return before + inc - v;
}

// Contiguous split layout (one workgroup), for the global layers. The steps
// (page pairs) of all units are laid end to end, unit after unit, and
// workgroup w of the main kernel runs steps [w per, (w + 1) per) of that list,
// per = ceil(steps / grid): every workgroup gets the same number of steps
// (one more at most), whatever the units' lengths, at the cost of a
// workgroup's range crossing unit boundaries. A unit that lies within one
// workgroup's range is finished by it (its rows written directly); a unit
// cut by a range boundary is run in pieces, one per workgroup it meets,
// which write partial slots tab[u] .. tab[u+1]-1 for the merge. Writes
// hdr = {steps, per}, off[u] (first step of unit u; off[units] = steps),
// tab, and wfirst[w] (the unit holding workgroup w's first step; -1: w has
// no steps).
template <int D, int G, int ROWS>
__global__ __launch_bounds__(kMPlanThreads) void mq_plan_contig_kernel(MQArgs a) {
  __shared__ long long s_w[kMPlanThreads / kWave];
  __shared__ int s_wi[kMPlanThreads / kWave];
  const int tid = threadIdx.x, U = a.units;
  const int per_t = (U + kMPlanThreads - 1) / kMPlanThreads;
  const int u0 = min(U, tid * per_t), u1 = min(U, u0 + per_t);
  auto unit_steps = [&](int u) -> long long { return (mq_unit_pages<D, G, ROWS>(a, u) + 1) / 2; };
  long long loc = 0;
  for (int u = u0; u < u1; ++u) loc += unit_steps(u);
  long long tot;
  const long long base = mq_block_exscan(loc, s_w, tot);
  long long run = base;
  const long long per = tot > 0 ? (tot + a.grid - 1) / a.grid : 1;
  int cnt = 0;
  for (int u = u0; u < u1; ++u) {
    const long long ns = unit_steps(u);
    a.off[u] = run;
    if (ns > 0) {
      const long long wf = run / per, wl = (run + ns - 1) / per;
      if (wl > wf) cnt += (int)(wl - wf + 1);
      for (long long w = (run + per - 1) / per; w <= wl; ++w) a.wfirst[w] = u;  // ranges starting in u
    }
    run += ns;
  }
  if (tid == kMPlanThreads - 1) a.off[U] = run;  // the last thread's run is the total
  int ctot;
  int crun = mq_block_exscan(cnt, s_wi, ctot);
  run = base;
  for (int u = u0; u < u1; ++u) {
    const long long ns = unit_steps(u);
    a.tab[u] = crun;
    if (ns > 0 && (run + ns - 1) / per > run / per) crun += (int)((run + ns - 1) / per - run / per + 1);
    run += ns;
  }
  if (tid == kMPlanThreads - 1) a.tab[U] = crun;
  const long long nwg = (tot + per - 1) / per;
  for (long long w = nwg + tid; w < a.grid; w += kMPlanThreads) a.wfirst[w] = -1;
  if (tid == 0) {
    a.hdr[0] = tot;
    a.hdr[1] = per;
  }
}

template <int D, int G>
__global__ __launch_bounds__(kMThreads) __attribute__((amdgpu_waves_per_eu(2))) void mq_kernel(MQArgs a) {
  using C = MQShape<D, G>;
  static_assert(C::kSliding, "global layers use mq_global_kernel");
  constexpr int kHalves = 1;  // one wave per 16 rows, all 256 coordinates
  __shared__ __attribute__((aligned(16))) uint8_t s_kv[2][2 * kMRegion];

  int blk = blockIdx.x, split = blockIdx.y, bc = blockIdx.z, nsplit = a.nsplit;
  size_t slot_idx = ((size_t)bc * a.nblk + blk) * a.nsplit + split;
  if (a.balanced) {
    const int4 dsc = a.desc[blockIdx.x];
    const int u = mq_rfl(dsc.x);
    if (u < 0) return;  // no piece for this workgroup
    blk = u % a.nblk;
    bc = u / a.nblk;
    split = mq_rfl(dsc.y);
    nsplit = mq_rfl(dsc.z);
    slot_idx = (size_t)mq_rfl(dsc.w);
  }
  const int b = bc / a.Hkv, c = bc - b * a.Hkv;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.P_max * kPage ? a.P_max * kPage : L);
  const int q0 = a.q_start[b];
  const int S = a.q_start[b + 1] - q0;
  const int s0 = blk * C::kQueries;
  if (s0 >= S) return;  // no rows in this block (the merge skips it too)
  const int s1 = min(S, s0 + C::kQueries) - 1;
  const int p0 = L - S + s0, p1 = L - S + s1;  // positions of the block's first and last query
  // Keys some row of the block sees: [klo, khi].
  const int klo = C::kSliding ? max(0, p0 - a.window + 1) : 0;
  const int khi = p1;
  const bool any = khi >= 0 && (!C::kSliding || a.window > 0);
  const int jlo = any ? klo / kPage : 0;
  const int np = any ? khi / kPage - jlo + 1 : 0;
  const int ja = jlo + (int)((long long)split * np / nsplit);
  const int jb = jlo + (int)((long long)(split + 1) * np / nsplit);
  const int nsteps = (jb - ja + 1) / 2;

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wv = mq_rfl(tid / kWave);
  const int rb = wv / kHalves, hf = wv % kHalves;
  const int n = lane & 15, g4 = lane >> 4;
  const int r_wg = rb * 16 + n;  // this lane's row within the workgroup
  const int s_r = s0 + r_wg / G;
  const int head = c * G + r_wg % G;
  const bool valid = s_r <= s1;
  const int pos_r = valid ? L - S + s_r : -1;  // -1: sees nothing
  const int lo_r = C::kSliding ? max(0, pos_r - a.window + 1) : 0;
  const int Hq = a.Hkv * G;

  // Q^T B operands: row n, coordinates 256 hf + 32 i + 8 g4 .. +8.
  uint4 qv[kMKSteps];
  {
    const uint16_t* qp = a.q + ((size_t)(q0 + s_r) * Hq + head) * D + hf * kMSlice + 8 * g4;
#pragma unroll
    for (int i = 0; i < kMKSteps; ++i) qv[i] = valid ? ld16(qp + 32 * i) : make_uint4(0u, 0u, 0u, 0u);
  }

  // Chunk u (0..3) of 16 bytes per step and thread. Sliding: u = 2 * (V) +
  // page; the row-major slab [16 tokens][256] is stored as [32 chunks][16
  // tokens][8], thread tid taking chunk tid >> 4 of token tid & 15. Global:
  // the tiled page [64 chunks][16 tokens][8] is read 16 bytes per thread,
  // chunk ((u & 1) * 512 + tid) >> 4 of page u >> 1, token tid & 15.
  // LDS layout of a page: chunks in pairs (2p, 2p+1) of 512 bytes, each pair
  // as [tokens 0-7 of 2p][tokens 0-7 of 2p+1][tokens 8-15 of 2p][tokens 8-15
  // of 2p+1], 16 bytes per token. The page stores (16 bytes per thread), the
  // K reads and the transposed V^T reads are then all free of bank conflicts
  // (the plain [chunk][token] order costs the transposed reads 2 extra cycles
  // each).
  const int c_tok = tid & 15;
  const int c_src = C::kSliding ? (tid & 15) * 256 + (tid >> 4) * 8 : tid * 8;  // + u-dependent part
  const int c_lds = (tid >> 5) * 512 + (((tid & 15) >> 3) * 2 + ((tid >> 4) & 1)) * 128 + (tid & 7) * 16;
  auto u_pg = [](int u) constexpr { return C::kSliding ? (u & 1) : (u >> 1); };
  auto u_src = [](int u) constexpr { return C::kSliding ? 0 : (u & 1) * kMThreads * 8; };
  auto u_lds = [](int u) constexpr {
    return C::kSliding ? (u >> 1) * kMRegion + (u & 1) * C::kKPage : (u >> 1) * C::kKPage + (u & 1) * kMThreads * 16;
  };
  const size_t slab = (size_t)kPage * D;
  // Every step issues the same loads: pages past the piece's end read the
  // zero page instead (selected, not branched around, so that the compiler
  // keeps counting the loads in flight and waits only for the step it needs).
  const uint16_t* zero = reinterpret_cast<const uint16_t*>(g_zero_page);
  auto load_step = [&](int k, uint4(&r)[4]) __attribute__((always_inline)) {
    const int j0 = ja + 2 * k;
    int ph[2];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) ph[pg] = a.bt[(size_t)b * a.P_max + min(j0 + pg, jb - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint16_t* src = (C::kSliding && u >= 2) ? a.v : a.k;
      const uint16_t* pgp = j0 + u_pg(u) < jb ? src + ((size_t)ph[u_pg(u)] * a.Hkv + c) * slab : zero;
      // plain loads: the row blocks of a sequence re-read its pages, which
      // the caches keep (the non-temporal hint made prefill chunks ~10% slower)
      r[u] = ld16(pgp + c_src + u_src(u));
    }
  };
  // Tokens no row of the block sees (and pages of other splits) are stored
  // as zeros, so that whatever that storage holds, NaN included, meets only
  // zero weights.
  auto store_step = [&](int k, const uint4(&r)[4], int buf) __attribute__((always_inline)) {
    const int j0 = ja + 2 * k;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u_pg(u), pos = j * kPage + c_tok;
      const bool keep = j < jb && pos >= klo && pos <= khi;
      *reinterpret_cast<uint4*>(&s_kv[buf][c_lds + u_lds(u)]) = keep ? r[u] : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  f32x4 acc[kMTiles];
#pragma unroll
  for (int t = 0; t < kMTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int s16 = lane & 15;
  // K (A operand): chunk lane >> 4 of a 4-chunk group, token lane & 15.
  const int k_off = (lane >> 5) * 512 + (((lane & 15) >> 3) * 2 + ((lane >> 4) & 1)) * 128 + (lane & 7) * 16;
  // V^T (transposed reads): chunk (s16 & 3) >> 1 of the tile's two, token
  // 4 g4 + (s16 >> 2), 8-byte half s16 & 1.
  const int tr_ch = (s16 & 3) >> 1;
  const int tr_tok = 4 * g4 + (s16 >> 2);
  const int tr_off = ((tr_tok >> 3) * 2 + tr_ch) * 128 + (tr_tok & 7) * 16 + (s16 & 1) * 8;

  // A wave whose 16 rows hold no query of the block (few queries per
  // sequence: speculative verification on sliding layers fills one wave of
  // eight) takes part in the loads and barriers only.
  const bool wact = s0 + (rb * 16) / G <= s1;

  auto compute = [&](int k, int buf) __attribute__((always_inline)) {
    const int j0 = ja + 2 * k;
    f32x4 sp[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      if (!wact) break;
      const uint8_t* kp = &s_kv[buf][pg * C::kKPage + hf * 8192 + k_off];
      f32x4 x[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      constexpr int kKB = 4;  // k-steps per batch of LDS reads
#pragma unroll
      for (int i0 = 0; i0 < kMKSteps; i0 += kKB) {
        uint4 kv4[kKB];
#pragma unroll
        for (int i = 0; i < kKB; ++i) kv4[i] = *reinterpret_cast<const uint4*>(kp + (i0 + i) * 1024);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kKB; ++i)
          x[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv4[i]),
                                                             __builtin_bit_cast(bf16x8, qv[i0 + i]), x[i & 1], 0, 0, 0);
      }
      sp[pg] = x[0] + x[1];
    }
    if (!wact) return;
    float sc[8];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + pg, pos = j * kPage + 4 * g4 + e;
        const bool vis = j < jb && pos >= lo_r && pos <= pos_r;
        sc[4 * pg + e] = vis ? sp[pg][e] * kLog2e : -INFINITY;
      }
    // Lazy rescaling (as in the decode kernels): the reference m_run moves
    // only when a score exceeds it by more than kMRescale.
    float lmax = sc[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) lmax = fmaxf(lmax, sc[e]);
    if (__any(lmax > m_run + kMRescale)) {
      float mp = fmaxf(lmax, xor16(lmax));
      mp = fmaxf(mp, xor32(mp));  // row max over the 4 lane groups of the row
      const float m_new = (mp > m_run + kMRescale) ? mp : m_run;
      const float alpha = (m_new == m_run) ? 1.f : exp2_fast(m_run - m_new);  // 0 from -inf
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < kMTiles; ++t) acc[t] *= alpha;
    }
    // P^T operand: k-slots 8 g4 + e hold page 0's token 4 g4 + e, slots
    // 8 g4 + 4 + e page 1's; the V^T operand is built the same way.
    bf16x8 pp;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pv = (sc[e] == -INFINITY) ? 0.f : exp2_fast(sc[e] - m_run);
      pp[e] = (__bf16)pv;
      l_run += (float)pp[e];
    }
    const uint8_t* vb = &s_kv[buf][C::kVBase + hf * 8192];
    constexpr int kVB = 2;  // tiles per batch of transposed reads (4 spills registers)
#pragma unroll
    for (int t0 = 0; t0 < kMTiles; t0 += kVB) {
      s16x4 v0[kVB], v1[kVB];
#pragma unroll
      for (int u = 0; u < kVB; ++u) {
        v0[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) uint8_t*)vb +
                                                       (t0 + u) * 512 + tr_off));
        v1[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) uint8_t*)vb +
                                                       C::kKPage + (t0 + u) * 512 + tr_off));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kVB; ++u) {
        const bf16x8 vt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0[u], v1[u], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[t0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pp, acc[t0 + u], 0, 0, 0);
      }
    }
  };

  if (nsteps > 0) {
    uint4 ra[4], rb2[4];
    load_step(0, ra);
    load_step(1, rb2);
    store_step(0, ra, 0);
    load_step(2, ra);
    __syncthreads();
    // Step k computes from buffer k % 2 while the registers hold steps k + 1
    // and k + 2. The loop runs an even number of steps: a step past the last
    // one holds zeros and no visible token, so it adds nothing (a loop exit
    // between the two halves made the compiler wait for every load in
    // flight in the first half).
    for (int k = 0; k < nsteps; k += 2) {
      compute(k, 0);
      store_step(k + 1, rb2, 1);
      load_step(k + 3, rb2);
      __syncthreads();
      compute(k + 1, 1);
      store_step(k + 2, ra, 0);
      load_step(k + 4, ra);
      __syncthreads();
    }
  }

  float lt = l_run + xor16(l_run);
  lt += xor32(lt);  // the row's denominator (its 4 lane groups)
  if (nsplit == 1) {
    if (valid) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;  // nothing visible: 0
      float* op = a.out + ((size_t)(q0 + s_r) * Hq + head) * D + hf * kMSlice + 4 * g4;
#pragma unroll
      for (int t = 0; t < kMTiles; ++t) *reinterpret_cast<f32x4*>(op + 16 * t) = acc[t] * inv;
    }
  } else {
    float* slot = a.ws + slot_idx * C::kSlotFloats;
    float* ap = slot + (size_t)r_wg * D + hf * kMSlice + 4 * g4;
#pragma unroll
    for (int t = 0; t < kMTiles; ++t) *reinterpret_cast<f32x4*>(ap + 16 * t) = acc[t];
    if (g4 == 0 && hf == 0) {
      slot[C::kRows * D + r_wg] = m_run;
      slot[C::kRows * D + C::kRows + r_wg] = lt;
    }
  }
}

// ---------------------------------------------------------------- global layers
// mq_global_kernel: 128 rows (8 queries x 16 heads of the single KV head) per
// workgroup, in 4 tiles of 32 rows; wave (rt, hf) = (wv / 2, wv % 2) owns row
// tile rt and coordinates [256 hf, 256 hf + 256). With 32x32 MFMA tiles each
// K and V element read from LDS serves 32 rows, half the LDS reads per row of
// 16-row tiles, and a sequence's keys are read once for up to 8 queries.
//
// Keys go HBM -> LDS directly (global_load_lds_dwordx4), two pages (32
// tokens) per step into a ring of 3 steps, loaded two steps ahead (64 KB
// in flight per workgroup; the ring and the score exchange take 128 KB of
// LDS; a ring of 4 steps loaded three ahead measured 1-2% slower and spills
// more registers); within each 1 KB of a page the 16-byte slots are
// swizzled so that both kinds of reads spread over all banks. A lane whose token no row of
// the block sees (past the last query's position, or a page past the piece)
// loads the zero page instead, so the LDS copy holds zeros there whatever
// the cache holds, NaN included. The waits for these loads are explicit
// (vmcnt) and the barriers are plain s_barrier (a __syncthreads would also
// wait for the loads still in flight); the reads of the ring are asm (see
// qg_read_k2), so the compiler adds no wait for the loads of its own.
//
// Per step and wave:
//   S^T (32 tokens x 32 rows) partial over the wave's 256 coordinates: 16 x
//     mfma_f32_32x32x16_bf16, K (A operand: lane l = token l % 32,
//     coordinates 256 hf + 16 i + 8 (l / 32) .. +8 of k-step i) read from
//     LDS, Q^T held in registers. Each wave adds its partner's partial from
//     LDS to its own; fp32 addition commutes, so both hold the same sums.
//   Accumulator element e = 4i + j of lane l holds token 8i + 4(l/32) + j
//     of row l % 32. The PV product takes P^T straight from it: k-step ks
//     (16 tokens) uses elements 8 ks .. 8 ks + 7, i.e. k-slot 8h + w is token
//     16 ks + 8 (w / 4) + 4 h + w % 4 (h = l / 32), and the V^T operand is
//     read in the same token order with two ds_read_b64_tr_b16 per tile.
//   O^T (256 coordinates x 32 rows) += V^T P^T: 8 tiles x 2 k-steps of
//     mfma_f32_32x32x16_bf16, the accumulators in lane order (coordinate
//     256 hf + 32 t + 8i + 4(l/32) + j of tile t, row l % 32).
// Registers are the limit (2 waves per SIMD, 256 each: 128 accumulators, 16
// for S, 64 of query rows), hence the small read batches; a step every row
// of a tile sees in full skips the mask.
constexpr int kQGStep = 2 * 16384;   // bytes of keys per step (two pages)
constexpr int kQGSlice = 256;        // coordinates per wave
constexpr int kQGDma = kQGStep / kMThreads / 16;  // 16-byte loads per thread and step (4)
typedef float f32x16 __attribute__((ext_vector_type(16)));

// s_waitcnt operands (gfx9): vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; the counters not named are left unconstrained.
#define DA_WAIT_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | 0x70 | 0xF00)
#define DA_WAIT_LGKM0 0xC07F

__device__ __forceinline__ void qg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t qg_lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

template <int... Is, class F>
__device__ __forceinline__ void qg_static_for(std::integer_sequence<int, Is...>, F&& f) {
  (f(std::integral_constant<int, Is>{}), ...);
}

// The reads of the key ring are written as asm, each batch with its own
// lgkmcnt(0): the compiler then adds no wait of its own for the loads into
// LDS in flight (its analysis of them has given a full vmcnt(0) before the
// first step of each pass over the ring), and the explicit vmcnt at the top
// of a step is the only wait for them.
template <int O0, int O1>
__device__ __forceinline__ void qg_read_k2(uint32_t a0, uint32_t a1, uint4& r0, uint4& r1) {
  asm volatile(
      "ds_read_b128 %0, %2 offset:%4\n\t"
      "ds_read_b128 %1, %3 offset:%5\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1)
      : "v"(a0), "v"(a1), "i"(O0), "i"(O1));
}
template <int O>
__device__ __forceinline__ void qg_read_v2(uint32_t a0, uint32_t a1, s16x4& r0, s16x4& r1, s16x4& r2, s16x4& r3) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %1, %5 offset:%6\n\t"
      "ds_read_b64_tr_b16 %2, %4 offset:%7\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a0), "v"(a1), "i"(O), "i"(O + 1024));
}

__global__ __launch_bounds__(kMThreads) __attribute__((amdgpu_waves_per_eu(2))) void mq_global_kernel(MQArgs a) {
  using C = MQShape<512, 16>;
  __shared__ __attribute__((aligned(16))) uint8_t s_k0[kQGStep];
  __shared__ __attribute__((aligned(16))) uint8_t s_k1[kQGStep];
  __shared__ __attribute__((aligned(16))) uint8_t s_k2[kQGStep];
  __shared__ f32x4 s_x[kMWaves][4][kWave];  // each wave's partial S^T, 4 pieces of 4 elements

  // The workgroup's pieces. Fixed split: one, (row block, piece, sequence)
  // = blockIdx. Contiguous split: steps [w per, (w + 1) per) of the units
  // laid end to end, one piece per unit met (the plan kernel's layout),
  // every value read here wave-uniform (scalar loads).
  const bool contig = a.balanced == 2;
  long long g0 = 0, g1 = 0, per = 1;
  int u = 0;
  if (contig) {
    const long long tot = mq_sload(a.hdr, 0);
    per = mq_sload(a.hdr, 1);
    g0 = (long long)blockIdx.x * per;
    g1 = min(g0 + per, tot);
    if (g0 >= g1) return;  // no steps for this workgroup
    u = mq_sload(a.wfirst, blockIdx.x);
  }
  for (bool first = true;; first = false) {
  int blk, bc, ja, jb, slot = -1;
  long long ls0 = 0, ls1 = 0;
  if (contig) {
    if (g0 >= g1) break;
    long long o0 = mq_sload(a.off, u), o1 = mq_sload(a.off, u + 1);
    while (o1 <= g0) {  // units without steps
      ++u;
      o0 = o1;
      o1 = mq_sload(a.off, u + 1);
    }
    const long long e = min(g1, o1);
    ls0 = g0 - o0;
    ls1 = e - o0;
    const int t0 = mq_sload(a.tab, u);
    if (mq_sload(a.tab, u + 1) > t0) slot = t0 + (int)((long long)blockIdx.x - o0 / per);
    blk = u % a.nblk;
    bc = u / a.nblk;
    g0 = e;
    ++u;
  } else {
    if (!first) break;
    // largest blocks first: a sequence's later row blocks see more keys, so
    // compute units that drew a short block take a long one next
    blk = a.nblk - 1 - (int)blockIdx.x;
    bc = blockIdx.z;
    if (a.nsplit > 1) slot = (bc * a.nblk + blk) * a.nsplit + (int)blockIdx.y;
  }
  if (!first) {
    // the previous piece's last step still reads the ring
    __builtin_amdgcn_s_waitcnt(DA_WAIT_LGKM0);
    qg_barrier();
  }
  const int b = bc;  // one KV head
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.P_max * kPage ? a.P_max * kPage : L);
  const int q0 = a.q_start[b];
  const int S = a.q_start[b + 1] - q0;
  const int s0 = blk * C::kQueries;
  if (s0 >= S) continue;  // no rows in this block (the merge skips it too)
  const int s1 = min(S, s0 + C::kQueries) - 1;
  const int khi = L - S + s1;  // position of the block's last query: the last key any row sees
  const int np = khi >= 0 ? khi / kPage + 1 : 0;
  if (contig) {
    ja = (int)(2 * ls0);
    jb = (int)min(2 * ls1, (long long)np);
  } else {
    ja = (int)((long long)blockIdx.y * np / a.nsplit);
    jb = (int)((long long)(blockIdx.y + 1) * np / a.nsplit);
  }
  const int nsteps = (jb - ja + 1) / 2;

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wv = mq_rfl(tid / kWave);
  const int rt = wv >> 1, hf = wv & 1;
  const int n = lane & 31, h = lane >> 5;
  const int r_wg = 32 * rt + n;   // this lane's row (column of its tiles)
  const int s_r = s0 + (r_wg >> 4);
  const int head = r_wg & 15;
  const bool valid = s_r <= s1;
  const int pos_r = valid ? L - S + s_r : -1;  // -1: sees nothing
  const bool wact = s0 + 2 * rt <= s1;        // a tile holds 2 queries: its first one exists

  // Q^T (B operand) for k-step i: row n, coordinates 256 hf + 16 i + 8 h .. +8
  uint4 qv[16];
  {
    const uint16_t* qp = a.q + ((size_t)(q0 + s_r) * 16 + head) * 512 + hf * kQGSlice + 8 * h;
#pragma unroll
    for (int i = 0; i < 16; ++i) qv[i] = valid ? ld16(qp + 16 * i) : make_uint4(0u, 0u, 0u, 0u);
  }

  // Loads of step k: wave w fills bytes [4w, 4w + 4) KB of the step's LDS
  // region, i.e. page w / 4 of the step's two, 1 KB (four chunks of 16
  // tokens) per load. Within each 1 KB the 16-byte slots are swizzled: slot p
  // of chunk c holds token p ^ 4 (c % 4), so that the transposing V reads
  // (two chunks x four tokens per 16 lanes) and the K reads (16 tokens of a
  // chunk per 16 lanes) both spread over all LDS banks. Lane l of load u thus
  // fetches chunk 16 (w % 4) + 4 u + l / 16, token (l % 16) ^ 4 (l / 16). The
  // wave's page id is loaded one step before its pages.
  const int pg_w = wv >> 2;
  const int tok_w = (lane & 15) ^ (4 * (lane >> 4));
  const int lane_src = ((wv & 3) * 16 + (lane >> 4)) * 128 + tok_w * 8;  // elements, + 512 u
  const uint16_t* zero = reinterpret_cast<const uint16_t*>(g_zero_page);
  auto load_id = [&](int k) __attribute__((always_inline)) -> int {
    // wave-uniform: a scalar load, counted by lgkmcnt, so that vmcnt counts
    // only the loads into LDS
    const int j = min(ja + 2 * k + pg_w, max(jb - 1, 0));
    // (the block table is read-only during the call: the constant address
    // space lets the compiler use s_load)
    const __attribute__((address_space(4))) int* bt = (const __attribute__((address_space(4))) int*)a.bt;
    return bt[(size_t)b * a.P_max + j];
  };
  auto issue = [&](int k, int id, uint8_t* buf) __attribute__((always_inline)) {
    const int j = ja + 2 * k + pg_w;
    const bool keep = j < jb && j * kPage + tok_w <= khi;
    const uint16_t* src = (keep ? a.k + (size_t)mq_rfl(id) * (kPage * 512) : zero) + lane_src;
    uint8_t* dst = buf + wv * (kQGDma * 1024);
#pragma unroll
    for (int u = 0; u < kQGDma; ++u)
      __builtin_amdgcn_global_load_lds(src + 512 * u, (__attribute__((address_space(3))) void*)(dst + u * 1024),
                                       16, 0, 0);
  };

  f32x16 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // K reads (A operand): token n (page n / 16), chunk C = 32 hf + 2 i + h of
  // k-step i, whose chunk index mod 4 is h + 2 (i % 2): two base offsets.
  const int k_base = (n >> 4) * 16384 + (32 * hf + h) * 256;
  const int k_off0 = k_base + (((n & 15) ^ (4 * h)) * 16);      // + 512 i, i even
  const int k_off1 = k_base + (((n & 15) ^ (4 * h + 8)) * 16);  // + 512 i, i odd
  // V^T reads: lane group g16 = lane / 16, position i16 = lane % 16 supplies
  // token T = 4 (g16 / 2) + i16 / 4 (+ 8 for the second read, + 16 ks: page
  // ks), coordinates 256 hf + 32 t + 16 (g16 % 2) + 4 (i16 % 4) .. +4, from
  // chunk C = 32 hf + 4 t + 2 (g16 % 2) + (i16 % 4) / 2; its slot is
  // T ^ 4 (C % 4), and the second read's token T + 8 flips bit 3 of it.
  const int g16 = lane >> 4, i16 = lane & 15;
  const int cl = 2 * (g16 & 1) + ((i16 & 3) >> 1);
  const int tr_off0 = (32 * hf + cl) * 256 + (((4 * (g16 >> 1) + (i16 >> 2)) ^ (4 * cl)) * 16) +
                      (i16 & 1) * 8;  // + 16384 ks + 1024 t
  const int tr_off1 = tr_off0 ^ 128;
  // The row tile's first row has the smallest position: a step every row of
  // the tile sees in full needs no mask.
  const int pos_tile = L - S + s0 + 2 * rt;

  auto compute = [&](int k, const uint8_t* kb) __attribute__((always_inline)) {
    f32x16 x = {};
    const uint32_t kb_addr = qg_lds_addr(kb);
    if (wact) {
      const uint32_t ka0 = kb_addr + k_off0, ka1 = kb_addr + k_off1;
      qg_static_for(std::make_integer_sequence<int, 8>{}, [&](auto bi) __attribute__((always_inline)) {
        constexpr int I = 2 * decltype(bi)::value;
        uint4 kv0, kv1;
        qg_read_k2<I * 512, (I + 1) * 512>(ka0, ka1, kv0, kv1);
        x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv0), __builtin_bit_cast(bf16x8, qv[I]),
                                                    x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv1),
                                                    __builtin_bit_cast(bf16x8, qv[I + 1]), x, 0, 0, 0);
      });
    }
    // the two coordinate halves of the row tile: half 0's partial plus half 1's
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) s_x[wv][c4][lane] = f32x4{x[4 * c4], x[4 * c4 + 1], x[4 * c4 + 2], x[4 * c4 + 3]};
    __builtin_amdgcn_s_waitcnt(DA_WAIT_LGKM0);
    qg_barrier();
    if (!wact) return;
    // own partial plus the partner's: the same sum in both waves (fp32
    // addition commutes)
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const f32x4 sx = s_x[wv ^ 1][c4][lane];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) x[4 * c4 + jj] += sx[jj];
    }
    const int j0 = ja + 2 * k;
    if (!(j0 + 2 <= jb && (j0 + 2) * kPage - 1 <= pos_tile)) {
      // element e = 4 c4 + jj holds token 8 c4 + 4 h + jj of the step (page of that / 16)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int tok = 8 * (e >> 2) + 4 * h + (e & 3);
        const int pos = (j0 + (tok >> 4)) * kPage + (tok & 15);
        if (!(j0 + (tok >> 4) < jb && pos <= pos_r)) x[e] = -INFINITY;
      }
    }
    float lmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) lmax = fmaxf(lmax, x[e]);
    lmax *= kLog2e;  // log2 units, as m_run
    // lazy rescaling (as in the decode kernels): the reference m_run moves
    // only when a score exceeds it by more than kMRescale
    if (__any(lmax > m_run + kMRescale)) {
      const float mp = fmaxf(lmax, xor32(lmax));  // the row's max: lanes l and l ^ 32 hold its tokens
      const float m_new = (mp > m_run + kMRescale) ? mp : m_run;
      const float alpha = (m_new == m_run) ? 1.f : exp2_fast(m_run - m_new);  // 0 from -inf
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] *= alpha;
    }
    // m_run is -inf only while every score so far, this step's included, is -inf
    const float mneg = m_run == -INFINITY ? 0.f : -m_run;
    bf16x8 pp[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) pp[e >> 3][e & 7] = (__bf16)exp2_fast(__builtin_fmaf(x[e], kLog2e, mneg));  // 0 from -inf
    // the denominator sums the weights as rounded for the PV product
    const uint4 p0 = __builtin_bit_cast(uint4, pp[0]), p1 = __builtin_bit_cast(uint4, pp[1]);
    constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 (1, 1)
    l_run = dot2_bf16(p0.x, kOnes, dot2_bf16(p0.y, kOnes, dot2_bf16(p0.z, kOnes, dot2_bf16(p0.w, kOnes, l_run))));
    l_run = dot2_bf16(p1.x, kOnes, dot2_bf16(p1.y, kOnes, dot2_bf16(p1.z, kOnes, dot2_bf16(p1.w, kOnes, l_run))));
    const uint32_t va0 = kb_addr + tr_off0, va1 = kb_addr + tr_off1;
    qg_static_for(std::make_integer_sequence<int, 8>{}, [&](auto bi) __attribute__((always_inline)) {
      constexpr int ks = decltype(bi)::value >> 2, t0 = 2 * (decltype(bi)::value & 3);
      s16x4 a0, a1, b0, b1;  // tiles t0 and t0 + 1, first and second read
      qg_read_v2<ks * 16384 + t0 * 1024>(va0, va1, a0, a1, b0, b1);
      acc[t0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7)), pp[ks], acc[t0], 0, 0, 0);
      acc[t0 + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7)), pp[ks], acc[t0 + 1], 0,
          0, 0);
    });
  };

  // One step. The pages of step k have landed once at most the pages of
  // step k + 1 (kQGDma loads) are in flight; past the barrier every wave's
  // part of step k is in LDS and every wave is done with step k - 1, whose
  // slot then takes step k + 2. The page ids come one step ahead through
  // scalar loads.
  int id_n = 0;  // id of step k + 2
  auto step = [&](int k, const uint8_t* cur, uint8_t* nxt2) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(DA_WAIT_VMCNT(kQGDma));
    qg_barrier();
    issue(k + 2, id_n, nxt2);
    id_n = load_id(k + 3);
    compute(k, cur);
  };
  if (nsteps > 0) {
    const int id0 = load_id(0), id1 = load_id(1);
    id_n = load_id(2);
    issue(0, id0, s_k0);
    issue(1, id1, s_k1);
    for (int k = 0; k < nsteps; k += 3) {
      step(k, s_k0, s_k2);
      if (k + 1 >= nsteps) break;
      step(k + 1, s_k1, s_k0);
      if (k + 2 >= nsteps) break;
      step(k + 2, s_k2, s_k1);
    }
  }
  __builtin_amdgcn_s_waitcnt(DA_WAIT_VMCNT(0));  // no load into LDS outlives the workgroup

  const float lt = l_run + xor32(l_run);  // the row's denominator (both lanes of the row)
  // coordinates 256 hf + 32 t + 8 i + 4 h .. +4 of row r_wg: elements 4i .. 4i + 3 of tile t
  if (slot < 0) {
    if (valid) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;  // nothing visible: 0
      float* op = a.out + ((size_t)(q0 + s_r) * 16 + head) * 512 + hf * kQGSlice + 4 * h;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<f32x4*>(op + 32 * t + 8 * i) =
              f32x4{acc[t][4 * i], acc[t][4 * i + 1], acc[t][4 * i + 2], acc[t][4 * i + 3]} * inv;
    }
  } else {
    float* sp = a.ws + (size_t)slot * C::kSlotFloats;
    float* ap = sp + (size_t)r_wg * 512 + hf * kQGSlice + 4 * h;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<f32x4*>(ap + 32 * t + 8 * i) =
            f32x4{acc[t][4 * i], acc[t][4 * i + 1], acc[t][4 * i + 2], acc[t][4 * i + 3]};
    if (h == 0 && hf == 0) {
      sp[C::kRows * 512 + r_wg] = m_run;
      sp[C::kRows * 512 + C::kRows + r_wg] = lt;
    }
  }
  }  // pieces
}

// ---------------------------------------------------------------- sliding layers, long chunks
// mq_sliding_kernel: the global kernel's 32-row tiles for the sliding layers,
// used when a call has 128 or more queries in a sequence (prefill chunks).
// 256 rows per workgroup: 128 queries x the 2 heads of one KV head, wave w
// owning row tile w (32 rows) and all 256 coordinates, so no partial scores
// are exchanged. K and V pages of the KV head go HBM -> LDS
// (global_load_lds_dwordx4) in the global kernel's order (16-byte chunks of
// 8 coordinates, chunk-major, slots XOR-swizzled by the chunk), the source
// addresses picking each chunk out of the row-major page: per step the two
// pages' K (2 x 8 KB) and V (2 x 8 KB), a ring of 4 steps (128 KB) loaded
// three steps ahead. A lane whose token no row of the block sees (outside
// [first query's position - window + 1, last query's position], or past the
// piece) loads the zero page. Per step and wave: S^T (32 tokens x 32 rows)
// with 16 x mfma_f32_32x32x16_bf16, masks (l <= p and l > p - window), the
// one-pass softmax, and O^T (256 x 32) += V^T P^T with 16 more, as in the
// global kernel. A step every row of a tile sees in full skips the mask.
constexpr int kQSRows = 256;                 // rows per workgroup
constexpr int kQSPage = 8192;                // bytes of one page of one KV head (16 x 256 bf16)
constexpr int kQSStep = 4 * kQSPage;         // K and V of two pages
constexpr int kQSVBase = 2 * kQSPage;        // the V pages' offset in a step
constexpr int kQSDma = kQSStep / kMThreads / 16;  // 16-byte loads per thread and step (4)
constexpr int kQSMinQueries = 128;           // calls with fewer queries per sequence use mq_kernel

__global__ __launch_bounds__(kMThreads) __attribute__((amdgpu_waves_per_eu(2))) void mq_sliding_kernel(MQArgs a) {
  using C = MQShape<256, 2, kQSRows>;
  __shared__ __attribute__((aligned(16))) uint8_t s_k0[kQSStep];
  __shared__ __attribute__((aligned(16))) uint8_t s_k1[kQSStep];
  __shared__ __attribute__((aligned(16))) uint8_t s_k2[kQSStep];
  __shared__ __attribute__((aligned(16))) uint8_t s_k3[kQSStep];

  // The workgroup's pieces, as in mq_global_kernel.
  const bool contig = a.balanced == 2;
  long long g0 = 0, g1 = 0, per = 1;
  int u = 0;
  if (contig) {
    const long long tot = mq_sload(a.hdr, 0);
    per = mq_sload(a.hdr, 1);
    g0 = (long long)blockIdx.x * per;
    g1 = min(g0 + per, tot);
    if (g0 >= g1) return;  // no steps for this workgroup
    u = mq_sload(a.wfirst, blockIdx.x);
  }
  for (bool first = true;; first = false) {
  int blk, bc, ja, jb, slot = -1;
  long long ls0 = 0, ls1 = 0;
  if (contig) {
    if (g0 >= g1) break;
    long long o0 = mq_sload(a.off, u), o1 = mq_sload(a.off, u + 1);
    while (o1 <= g0) {  // units without steps
      ++u;
      o0 = o1;
      o1 = mq_sload(a.off, u + 1);
    }
    const long long e = min(g1, o1);
    ls0 = g0 - o0;
    ls1 = e - o0;
    const int t0 = mq_sload(a.tab, u);
    if (mq_sload(a.tab, u + 1) > t0) slot = t0 + (int)((long long)blockIdx.x - o0 / per);
    blk = u % a.nblk;
    bc = u / a.nblk;
    g0 = e;
    ++u;
  } else {
    if (!first) break;
    blk = blockIdx.x;
    bc = blockIdx.z;
    if (a.nsplit > 1) slot = (bc * a.nblk + blk) * a.nsplit + (int)blockIdx.y;
  }
  if (!first) {
    // the previous piece's last step still reads the ring
    __builtin_amdgcn_s_waitcnt(DA_WAIT_LGKM0);
    qg_barrier();
  }
  const int b = bc / a.Hkv, c = bc - b * a.Hkv;
  const int Hq = 2 * a.Hkv;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.P_max * kPage ? a.P_max * kPage : L);
  const int q0 = a.q_start[b];
  const int S = a.q_start[b + 1] - q0;
  const int s0 = blk * C::kQueries;
  if (s0 >= S) continue;  // no rows in this block (the merge skips it too)
  const int s1 = min(S, s0 + C::kQueries) - 1;
  const int w = a.window;
  const int khi = L - S + s1;                   // the last key any row sees
  const int klo = max(0, L - S + s0 - w + 1);   // the first
  const int jlo = klo / kPage;
  const int np = (khi >= 0 && w > 0) ? khi / kPage - jlo + 1 : 0;  // pages of the block, from page jlo
  if (contig) {
    ja = (int)(2 * ls0);
    jb = (int)min(2 * ls1, (long long)np);
  } else {
    ja = (int)((long long)blockIdx.y * np / a.nsplit);
    jb = (int)((long long)(blockIdx.y + 1) * np / a.nsplit);
  }
  const int nsteps = (jb - ja + 1) / 2;

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wv = mq_rfl(tid / kWave);
  const int rt = wv;  // row tile
  const int n = lane & 31, h = lane >> 5;
  const int r_wg = 32 * rt + n;   // this lane's row (column of its tiles)
  const int s_r = s0 + (r_wg >> 1);
  const int gh = r_wg & 1;        // head within the KV head's group
  const bool valid = s_r <= s1;
  const int pos_r = valid ? L - S + s_r : -1;  // -1: sees nothing
  const bool wact = s0 + 16 * rt <= s1;        // a tile holds 16 queries: its first one exists

  // Q^T (B operand) for k-step i: row n, coordinates 16 i + 8 h .. +8
  uint4 qv[16];
  {
    const uint16_t* qp = a.q + ((size_t)(q0 + s_r) * Hq + 2 * c + gh) * 256 + 8 * h;
#pragma unroll
    for (int i = 0; i < 16; ++i) qv[i] = valid ? ld16(qp + 16 * i) : make_uint4(0u, 0u, 0u, 0u);
  }

  // Loads of step k: wave w fills bytes [4w, 4w + 4) KB of the step's LDS
  // region [K page 0][K page 1][V page 0][V page 1], i.e. half (w % 2) of
  // page (w / 2) % 2 of K (w < 4) or V, 1 KB (four chunks of 16 tokens) per
  // load. Slot p of chunk cc holds token p ^ 4 (cc % 4), so lane l of load u
  // fetches chunk 16 (w % 2) + 4 u + l / 16, token (l % 16) ^ 4 (l / 16),
  // from the row-major page (element 256 token + 8 chunk).
  const int pg_w = (wv >> 1) & 1;
  const int tok_w = (lane & 15) ^ (4 * (lane >> 4));
  const int lane_src = tok_w * 256 + 8 * (16 * (wv & 1) + (lane >> 4));  // elements, + 32 u
  const uint16_t* cache_w = wv < 4 ? a.k : a.v;
  const uint16_t* zero = reinterpret_cast<const uint16_t*>(g_zero_page);
  auto load_id = [&](int k) __attribute__((always_inline)) -> int {
    // wave-uniform: a scalar load, counted by lgkmcnt (the block table is
    // read-only during the call: the constant address space lets the
    // compiler use s_load)
    const int j = jlo + min(ja + 2 * k + pg_w, max(jb - 1, 0));
    const __attribute__((address_space(4))) int* bt = (const __attribute__((address_space(4))) int*)a.bt;
    return bt[(size_t)b * a.P_max + j];
  };
  auto issue = [&](int k, int id, uint8_t* buf) __attribute__((always_inline)) {
    const int jr = ja + 2 * k + pg_w;  // page within the block's range
    const int pos = (jlo + jr) * kPage + tok_w;
    const bool keep = jr < jb && pos >= klo && pos <= khi;
    // (lane_src + 32 u stays below 4096 elements: inside the page, and inside
    // the 16 KB zero page)
    const uint16_t* src = (keep ? cache_w + ((size_t)mq_rfl(id) * a.Hkv + c) * (kPage * 256) : zero) + lane_src;
    uint8_t* dst = buf + wv * (kQSDma * 1024);
#pragma unroll
    for (int uu = 0; uu < kQSDma; ++uu)
      __builtin_amdgcn_global_load_lds(src + 32 * uu, (__attribute__((address_space(3))) void*)(dst + uu * 1024), 16,
                                       0, 0);
  };

  f32x16 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // K reads (A operand): token n (page n / 16), chunk 2 i + h of k-step i,
  // whose index mod 4 is h + 2 (i % 2): two base offsets, + 512 i.
  const int k_base = (n >> 4) * kQSPage + h * 256;
  const int k_off0 = k_base + (((n & 15) ^ (4 * h)) * 16);      // + 512 i, i even
  const int k_off1 = k_base + (((n & 15) ^ (4 * h + 8)) * 16);  // + 512 i, i odd
  // V^T reads, as in the global kernel (chunk 4 t + cl of page ks):
  // + kQSVBase + kQSPage ks + 1024 t
  const int g16 = lane >> 4, i16 = lane & 15;
  const int cl = 2 * (g16 & 1) + ((i16 & 3) >> 1);
  const int tr_off0 = cl * 256 + (((4 * (g16 >> 1) + (i16 >> 2)) ^ (4 * cl)) * 16) + (i16 & 1) * 8;
  const int tr_off1 = tr_off0 ^ 128;
  // The tile's rows see positions [pos_first - w + 1, pos_last] at least and
  // at most [pos_last - w + 1, pos_first]: a step inside the latter needs no mask.
  const int pos_first = L - S + s0 + 16 * rt, pos_last = pos_first + 15;

  auto compute = [&](int k, const uint8_t* kb) __attribute__((always_inline)) {
    if (!wact) return;
    f32x16 x = {};
    const uint32_t kb_addr = qg_lds_addr(kb);
    const uint32_t ka0 = kb_addr + k_off0, ka1 = kb_addr + k_off1;
    qg_static_for(std::make_integer_sequence<int, 8>{}, [&](auto bi) __attribute__((always_inline)) {
      constexpr int I = 2 * decltype(bi)::value;
      uint4 kv0, kv1;
      qg_read_k2<I * 512, (I + 1) * 512>(ka0, ka1, kv0, kv1);
      x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv0), __builtin_bit_cast(bf16x8, qv[I]),
                                                  x, 0, 0, 0);
      x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv1),
                                                  __builtin_bit_cast(bf16x8, qv[I + 1]), x, 0, 0, 0);
    });
    const int jr0 = ja + 2 * k;
    const int T0 = (jlo + jr0) * kPage;  // position of the step's first token
    if (!(jr0 + 2 <= jb && T0 >= pos_last - w + 1 && T0 + 2 * kPage - 1 <= pos_first)) {
      // element e = 4 c4 + jj holds token 8 c4 + 4 h + jj of the step (page of that / 16)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int tok = 8 * (e >> 2) + 4 * h + (e & 3);
        const int pos = T0 + tok;
        if (!(jr0 + (tok >> 4) < jb && pos <= pos_r && pos > pos_r - w)) x[e] = -INFINITY;
      }
    }
    float lmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) lmax = fmaxf(lmax, x[e]);
    lmax *= kLog2e;  // log2 units, as m_run
    // lazy rescaling (as in the decode kernels)
    if (__any(lmax > m_run + kMRescale)) {
      const float mp = fmaxf(lmax, xor32(lmax));  // the row's max: lanes l and l ^ 32 hold its tokens
      const float m_new = (mp > m_run + kMRescale) ? mp : m_run;
      const float alpha = (m_new == m_run) ? 1.f : exp2_fast(m_run - m_new);  // 0 from -inf
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] *= alpha;
    }
    // m_run is -inf only while every score so far, this step's included, is -inf
    const float mneg = m_run == -INFINITY ? 0.f : -m_run;
    bf16x8 pp[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) pp[e >> 3][e & 7] = (__bf16)exp2_fast(__builtin_fmaf(x[e], kLog2e, mneg));  // 0 from -inf
    // the denominator sums the weights as rounded for the PV product
    const uint4 p0 = __builtin_bit_cast(uint4, pp[0]), p1 = __builtin_bit_cast(uint4, pp[1]);
    constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 (1, 1)
    l_run = dot2_bf16(p0.x, kOnes, dot2_bf16(p0.y, kOnes, dot2_bf16(p0.z, kOnes, dot2_bf16(p0.w, kOnes, l_run))));
    l_run = dot2_bf16(p1.x, kOnes, dot2_bf16(p1.y, kOnes, dot2_bf16(p1.z, kOnes, dot2_bf16(p1.w, kOnes, l_run))));
    const uint32_t va0 = kb_addr + tr_off0, va1 = kb_addr + tr_off1;
    qg_static_for(std::make_integer_sequence<int, 8>{}, [&](auto bi) __attribute__((always_inline)) {
      constexpr int ks = decltype(bi)::value >> 2, t0 = 2 * (decltype(bi)::value & 3);
      s16x4 a0, a1, b0, b1;  // tiles t0 and t0 + 1, first and second read
      qg_read_v2<kQSVBase + ks * kQSPage + t0 * 1024>(va0, va1, a0, a1, b0, b1);
      acc[t0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7)), pp[ks], acc[t0], 0, 0, 0);
      acc[t0 + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7)), pp[ks], acc[t0 + 1], 0,
          0, 0);
    });
  };

  // One step, as in mq_global_kernel but one step deeper: at most the pages
  // of steps k + 1 and k + 2 (2 kQSDma loads) are in flight past the wait; past the barrier
  // every wave's part of step k is in LDS and every wave is done with step
  // k - 1, whose slot then takes step k + 3.
  int id_n = 0;  // id of step k + 3
  auto step = [&](int k, const uint8_t* cur, uint8_t* nxt3) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(DA_WAIT_VMCNT(2 * kQSDma));
    qg_barrier();
    issue(k + 3, id_n, nxt3);
    id_n = load_id(k + 4);
    compute(k, cur);
  };
  if (nsteps > 0) {
    const int id0 = load_id(0), id1 = load_id(1), id2 = load_id(2);
    id_n = load_id(3);
    issue(0, id0, s_k0);
    issue(1, id1, s_k1);
    issue(2, id2, s_k2);
    for (int k = 0; k < nsteps; k += 4) {
      step(k, s_k0, s_k3);
      if (k + 1 >= nsteps) break;
      step(k + 1, s_k1, s_k0);
      if (k + 2 >= nsteps) break;
      step(k + 2, s_k2, s_k1);
      if (k + 3 >= nsteps) break;
      step(k + 3, s_k3, s_k2);
    }
  }
  __builtin_amdgcn_s_waitcnt(DA_WAIT_VMCNT(0));  // no load into LDS outlives the workgroup

  const float lt = l_run + xor32(l_run);  // the row's denominator (both lanes of the row)
  // coordinates 32 t + 8 i + 4 h .. +4 of row r_wg: elements 4i .. 4i + 3 of tile t
  if (slot < 0) {
    if (valid) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;  // nothing visible: 0
      float* op = a.out + ((size_t)(q0 + s_r) * Hq + 2 * c + gh) * 256 + 4 * h;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<f32x4*>(op + 32 * t + 8 * i) =
              f32x4{acc[t][4 * i], acc[t][4 * i + 1], acc[t][4 * i + 2], acc[t][4 * i + 3]} * inv;
    }
  } else {
    float* sp = a.ws + (size_t)slot * C::kSlotFloats;
    float* ap = sp + (size_t)r_wg * 256 + 4 * h;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<f32x4*>(ap + 32 * t + 8 * i) =
            f32x4{acc[t][4 * i], acc[t][4 * i + 1], acc[t][4 * i + 2], acc[t][4 * i + 3]};
    if (h == 0) {
      sp[C::kRows * 256 + r_wg] = m_run;
      sp[C::kRows * 256 + C::kRows + r_wg] = lt;
    }
  }
  }  // pieces
}

// Combines the nsplit partial slots of one row block. Thread item = (row, 4
// coordinates), one item per thread: the block's items are spread over
// kMergeChunks workgroups. The pieces are folded with a running max, 4 at a
// time with independent loads:
//   M = max m_i,  o = sum 2^(m_i - M) acc_i / sum 2^(m_i - M) l_i.
template <int D, int G, int ROWS = 128>
__global__ __launch_bounds__(256) void mq_merge_kernel(MQArgs a) {
  using C = MQShape<D, G, ROWS>;
  const int blk = blockIdx.x, bc = blockIdx.z;
  const int b = bc / a.Hkv, c = bc - b * a.Hkv;
  const int q0 = a.q_start[b];
  const int S = a.q_start[b + 1] - q0;
  const int s0 = blk * C::kQueries;
  if (s0 >= S) return;
  const int it = blockIdx.y * 256 + threadIdx.x;
  const int r = it / (D / 4), d = (it - r * (D / 4)) * 4;
  const int s_r = s0 + r / G;
  if (s_r >= S) return;
  const int unit = bc * a.nblk + blk;
  const int first = a.balanced ? a.tab[unit] : unit * a.nsplit;
  const int nsplit = a.balanced ? a.tab[unit + 1] - first : a.nsplit;
  float* op = a.out + ((size_t)(q0 + s_r) * (a.Hkv * G) + c * G + r % G) * D + d;
  if (nsplit <= 1) {
    // a single piece wrote its rows itself; in a contiguous split a unit
    // without a piece either lay within one workgroup's range or sees no key
    if (a.balanced == 2 && nsplit == 0 && mq_unit_pages<D, G, ROWS>(a, unit) == 0)
      *reinterpret_cast<f32x4*>(op) = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  const float* base = a.ws + (size_t)first * C::kSlotFloats;
  float m = -INFINITY, den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  constexpr int U = 4;
  for (int k0 = 0; k0 < nsplit; k0 += U) {
    float mi[U], li[U];
    f32x4 ai[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      mi[u] = -INFINITY;
      li[u] = 0.f;
      ai[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (k0 + u < nsplit) {
        const float* sl = base + (size_t)(k0 + u) * C::kSlotFloats;
        mi[u] = sl[C::kRows * D + r];
        li[u] = sl[C::kRows * D + C::kRows + r];
        ai[u] = *reinterpret_cast<const f32x4*>(sl + (size_t)r * D + d);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (mi[u] == -INFINITY) continue;  // no key in this piece
      const float mn = fmaxf(m, mi[u]);
      const float fo = exp2_fast(m - mn);  // 0 when m = -inf
      const float fi = exp2_fast(mi[u] - mn);
      num = num * fo + ai[u] * fi;
      den = den * fo + li[u] * fi;
      m = mn;
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  *reinterpret_cast<f32x4*>(op) = num * inv;
}

template <int D, int G>
static int mq_blocks(int max_queries) {
  return (max_queries + MQShape<D, G>::kQueries - 1) / MQShape<D, G>::kQueries;
}

static size_t mq_align(size_t x) { return (x + 255) & ~(size_t)255; }

// Byte offsets in the workspace of a contiguous split's layout arrays; the
// partial slots follow (at most 2 grid - 2 of them: a unit cut by k range
// boundaries has k + 1 pieces, and there are grid - 1 boundaries).
struct mq_contig_offsets {
  size_t hdr, wfirst, off, tab, total;
};
static mq_contig_offsets mq_contig_layout(int grid, int units) {
  mq_contig_offsets o;
  o.hdr = 0;
  o.wfirst = mq_align(2 * sizeof(long long));
  o.off = o.wfirst + mq_align((size_t)grid * sizeof(int));
  o.tab = o.off + mq_align(((size_t)units + 1) * sizeof(long long));
  o.total = o.tab + mq_align(((size_t)units + 1) * sizeof(int));
  return o;
}

mq_plan multiquery_plan(const da_shape& s, int max_queries, int window, int num_cus) {
  const bool sliding = s.head_dim == 256;
  mq_plan p{};
  if (sliding && max_queries >= kQSMinQueries) {
    // long chunks on sliding layers: mq_sliding_kernel, 256-row blocks. The
    // window bounds every block's keys, so blocks are alike: with two or
    // more per compute unit whole blocks are dispatched (no merge); with
    // fewer, the contiguous split; a caller-given number of pieces per block
    // otherwise.
    p.rows = kQSRows;
    p.nblk = (max_queries + MQShape<256, 2, kQSRows>::kQueries - 1) / MQShape<256, 2, kQSRows>::kQueries;
    p.units = (int)((long long)s.batch * s.num_kv_heads * p.nblk);
    const size_t slot = MQShape<256, 2, kQSRows>::kSlotFloats * sizeof(float);
    if (s.num_splits == 0 && p.units >= 2LL * num_cus) {
      p.nsplit = 1;
      p.grid = 0;
      p.ws_bytes = 0;
    } else if (s.num_splits == 0) {
      p.balanced = 2;
      p.nsplit = 0;
      p.grid = num_cus;
      p.ws_bytes = mq_contig_layout(p.grid, p.units).total + 2 * (size_t)p.grid * slot;
    } else {
      p.nsplit = s.num_splits;
      p.grid = 0;
      p.ws_bytes = p.nsplit > 1 ? (size_t)p.units * p.nsplit * slot : 0;
    }
    return p;
  }
  p.rows = MQShape<256, 2>::kRows;
  p.nblk = sliding ? mq_blocks<256, 2>(max_queries) : mq_blocks<512, 16>(max_queries);
  const long long units = (long long)s.batch * s.num_kv_heads * p.nblk;
  const size_t slot = (sliding ? MQShape<256, 2>::kSlotFloats : MQShape<512, 16>::kSlotFloats) * sizeof(float);
  // One workgroup runs on a compute unit at a time (8 waves of ~190-250
  // VGPRs; the global kernel's 128 KB of LDS). With fewer than two units per
  // compute unit the keys are split, into kMPiecesPerCu pieces' worth per
  // compute unit: the dispatcher hands the later pieces to the compute units
  // that finish first, and every piece writes one partial slot.
  const long long target = (long long)(sliding ? kMPiecesPerCuSliding : kMPiecesPerCuGlobal) * num_cus;
  if (!sliding && s.num_splits == 0 && units >= 2LL * num_cus) {
    // many blocks: whole blocks, largest first (the kernel reverses the
    // block index), no plan and no merge
    p.nsplit = 1;
    p.units = (int)units;
    p.grid = 0;
    p.ws_bytes = 0;
    return p;
  }
  if (!sliding && s.num_splits == 0) {
    // fewer: the contiguous split
    p.balanced = 2;
    p.nsplit = 0;
    p.units = (int)units;
    p.grid = (int)target;
    p.ws_bytes = mq_contig_layout(p.grid, p.units).total + 2 * (size_t)p.grid * slot;
    return p;
  }
  if (s.num_splits == 0 && units < 2LL * num_cus) {
    // pieces per unit follow its page count, laid out on the device
    p.balanced = 1;
    p.nsplit = 0;
    p.units = (int)units;
    p.grid = (int)target;
    const size_t desc = (size_t)p.grid * sizeof(int4), tab = (size_t)(p.units + 1) * sizeof(int);
    p.ws_bytes = mq_align(desc) + mq_align(tab) + (size_t)p.grid * slot;
    return p;
  }
  int nsplit = s.num_splits;
  if (nsplit <= 0) nsplit = 1;  // units >= two per compute unit: no split
  p.nsplit = nsplit;
  p.units = (int)units;
  p.grid = 0;
  p.ws_bytes = nsplit > 1 ? (size_t)units * nsplit * slot : 0;
  return p;
}

da_status launch_multiquery(const void* q, const int32_t* q_start, int max_queries, const void* k_cache,
                            const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                            int window, void* out, const da_shape& s, const mq_plan& p, void* workspace,
                            hipStream_t stream) {
  MQArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k_cache;
  a.v = (const uint16_t*)v_cache;
  a.bt = block_table;
  a.seq_lens = seq_lens;
  a.q_start = q_start;
  a.out = (float*)out;
  a.B = s.batch;
  a.Hkv = s.num_kv_heads;
  a.P_max = s.max_pages_per_seq;
  a.window = window;
  a.nblk = p.nblk;
  a.nsplit = p.nsplit;
  a.balanced = p.balanced;
  a.units = p.units;
  a.grid = p.grid;
  a.ws = nullptr;
  a.tab = nullptr;
  a.desc = nullptr;
  a.hdr = nullptr;
  a.off = nullptr;
  a.wfirst = nullptr;
  const bool sliding = s.head_dim == 256;
  dim3 grid((unsigned)a.nblk, (unsigned)a.nsplit, (unsigned)(s.batch * s.num_kv_heads));
  const bool long_sliding = p.rows == kQSRows;
  if (p.balanced == 2) {
    uint8_t* w = (uint8_t*)workspace;
    const mq_contig_offsets o = mq_contig_layout(p.grid, p.units);
    a.hdr = (long long*)(w + o.hdr);
    a.wfirst = (int*)(w + o.wfirst);
    a.off = (long long*)(w + o.off);
    a.tab = (int*)(w + o.tab);
    a.ws = (float*)(w + o.total);
    grid = dim3((unsigned)p.grid, 1, 1);
    if (long_sliding)
      hipLaunchKernelGGL((mq_plan_contig_kernel<256, 2, kQSRows>), dim3(1), dim3(kMPlanThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((mq_plan_contig_kernel<512, 16, 128>), dim3(1), dim3(kMPlanThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return DA_ERR_LAUNCH;
  } else if (p.balanced) {
    uint8_t* w = (uint8_t*)workspace;
    a.desc = (int4*)w;
    a.tab = (int*)(w + mq_align((size_t)p.grid * sizeof(int4)));
    a.ws = (float*)(w + mq_align((size_t)p.grid * sizeof(int4)) + mq_align((size_t)(p.units + 1) * sizeof(int)));
    grid = dim3((unsigned)p.grid, 1, 1);
    if (sliding)
      hipLaunchKernelGGL((mq_plan_kernel<256, 2>), dim3(1), dim3(kMPlanThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((mq_plan_kernel<512, 16>), dim3(1), dim3(kMPlanThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return DA_ERR_LAUNCH;
  } else if (p.nsplit > 1) {
    a.ws = (float*)workspace;
  }
  if (long_sliding)
    hipLaunchKernelGGL(mq_sliding_kernel, grid, dim3(kMThreads), 0, stream, a);
  else if (sliding)
    hipLaunchKernelGGL((mq_kernel<256, 2>), grid, dim3(kMThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(mq_global_kernel, grid, dim3(kMThreads), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return DA_ERR_LAUNCH;
  if (!p.balanced && p.nsplit <= 1) return DA_OK;
  constexpr int kChunksSliding = MQShape<256, 2>::kRows * 256 / 4 / 256;
  constexpr int kChunksLongSliding = MQShape<256, 2, kQSRows>::kRows * 256 / 4 / 256;
  constexpr int kChunksGlobal = MQShape<512, 16>::kRows * 512 / 4 / 256;
  const dim3 mgrid((unsigned)a.nblk,
                   (unsigned)(long_sliding ? kChunksLongSliding : (sliding ? kChunksSliding : kChunksGlobal)),
                   (unsigned)(s.batch * s.num_kv_heads));
  if (long_sliding)
    hipLaunchKernelGGL((mq_merge_kernel<256, 2, kQSRows>), mgrid, dim3(256), 0, stream, a);
  else if (sliding)
    hipLaunchKernelGGL((mq_merge_kernel<256, 2>), mgrid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((mq_merge_kernel<512, 16>), mgrid, dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

}  // namespace da
