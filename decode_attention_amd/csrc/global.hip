// decodeGQA over a paged K=V cache, tiled layout [pages][1][D/8][16][8] bf16.
//
// Pages: Op Specs of google/gemma-4-12B (Attention.lean: softmax, causalGQA,
// decodeGQA) and the gemma-4-12b Model Spec attn.core row for the global
// layers (scale 1, 16 query heads on 1 KV head, D = 512, values = keys).
//
// Work split. The cached pages of the whole batch form one list (sequence by
// sequence); workgroup w of G takes pages [w*N/G, (w+1)*N/G). A sequence
// that lies inside one workgroup's range is finished there; a sequence cut
// by range boundaries leaves one partial result (unnormalised output, running
// max m and sum l per head) per piece, and lse_merge_kernel combines them:
//   M = max_i m_i,  o = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i
// (scores are kept in the log2 domain). This is exact over the reals because
// the softmax over a union of disjoint key sets factorises that way.
//
// Inside a workgroup the 4 waves share every page: wave w owns coordinates
// [128w, 128w+128), i.e. 4 KB of the 16 KB page, loaded with lane-linear
// 16-byte loads that land directly in the MFMA A-operand layout of K.
//   S^T (16 tokens x 16 heads) = K Q^T : 4 x mfma_f32_16x16x32_bf16 per wave
//     on its 128 coordinates; the 4 partial tiles are summed through LDS in a
//     fixed order, so every wave holds the same scores.
//   The S^T accumulator layout (lane: head l%16, tokens 4(l/16)..+3) is the
//     B operand of mfma_f32_16x16x16_bf16 for P^T, so the probabilities never
//     move between lanes.
//   O^T (512 x 16) += V^T P^T: V = K, the wave's 4 KB is written to LDS once
//     and read back transposed with ds_read_b64_tr_b16 (each instruction
//     covers 512 contiguous bytes, no bank conflicts).
#include "common.hpp"
#include "launch.hpp"

namespace da {

constexpr int kGD = 512;          // head dim
constexpr int kGH = 16;           // query heads (KV head count 1)
constexpr int kGWaves = 4;        // waves per workgroup
constexpr int kGThreads = kGWaves * kWave;
constexpr int kGSlice = kGD / kGWaves;        // coordinates per wave (128)
constexpr int kGKSteps = kGSlice / 32;        // 16x16x32 k-steps per wave (4)
constexpr int kGMTiles = kGSlice / 16;        // 16-row output tiles per wave (8)
constexpr int kGPageElems = kPage * kGD;      // bf16 elements per page (8192)
constexpr int kGSlotFloats = kGH * kGD + 2 * kGH;  // acc[16][512], m[16], l[16]
constexpr int kGMaxBatch = 1024;
constexpr float kGRescale = 32.f;  // lazy-rescale threshold, log2 units
constexpr int kGIdChunk = 4 * kWave;  // page ids gathered per refill (4 per lane); even
// Workspace: a header with the page prefix table (written by workgroup 0 of
// the decode kernel, read by the merge), then 2*G partial-result slots.
constexpr size_t kGHeaderBytes = 16384;  // >= (2*kGMaxBatch + 1) ints
static_assert((2 * kGMaxBatch + 1) * sizeof(int) <= kGHeaderBytes, "header too small");
#ifndef DA_GLOBAL_RING
#define DA_GLOBAL_RING 3
#endif
constexpr int kGBuf = DA_GLOBAL_RING;  // two-page steps held per wave (ring; kGBuf-1 ahead)

struct GlobalArgs {
  const uint16_t* q;         // [B][16][512] bf16 bits
  const uint16_t* kv;        // [P][1][64][16][8] bf16 bits
  const int32_t* bt;         // [B][P_max]
  const int32_t* seq_lens;   // [B]
  float* out;                // [B][16][512]
  int* ws_hdr;               // [B+1] page prefix, then [B] clamped lengths
  float* ws;                 // [2*G][kGSlotFloats]
  int B, P_max, G;
};

// Shared by both kernels: per-sequence page counts and their prefix sums.
// L is clamped to 16*P_max so no block-table read can leave the row.
__device__ __forceinline__ void build_prefix(const GlobalArgs& a, int* s_pre, int* s_len, int* s_tmp) {
  const int tid = threadIdx.x;
  const int per = (a.B + blockDim.x - 1) / blockDim.x;
  const int i0 = tid * per;
  int local = 0;
  for (int i = i0; i < i0 + per && i < a.B; ++i) {
    int L = a.seq_lens[i];
    L = L < 0 ? 0 : (L > a.P_max * kPage ? a.P_max * kPage : L);
    s_len[i] = L;
    local += (L + kPage - 1) / kPage;
  }
  s_tmp[tid] = local;
  __syncthreads();
  for (int off = 1; off < (int)blockDim.x; off <<= 1) {  // inclusive scan
    const int v = tid >= off ? s_tmp[tid - off] : 0;
    __syncthreads();
    s_tmp[tid] += v;
    __syncthreads();
  }
  int run = s_tmp[tid] - local;
  if (tid == 0) s_pre[0] = 0;
  for (int i = i0; i < i0 + per && i < a.B; ++i) {
    run += (s_len[i] + kPage - 1) / kPage;
    s_pre[i + 1] = run;
  }
  __syncthreads();
}

__device__ __forceinline__ int range_start(int w, int N, int G) {
  return (int)(((long long)w * N) / G);
}

// Sequence holding global page p (skips sequences without pages).
__device__ __forceinline__ int seq_of_page(const int* s_pre, int B, int p) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s_pre[mid + 1] <= p) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kGThreads) void global_decode_kernel(GlobalArgs a) {
  __shared__ int s_pre[kGMaxBatch + 1];
  __shared__ int s_len[kGMaxBatch];
  __shared__ int s_tmp[kGThreads];
  __shared__ f32x4 s_part[2][kGWaves][2][kWave];  // partial S^T tiles, 2 pages
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kGWaves][2][kGSlice * kPage];  // V slices

  build_prefix(a, s_pre, s_len, s_tmp);
  const int N = s_pre[a.B];
  const int w = blockIdx.x;
  if (w == 0 && a.ws_hdr != nullptr) {  // publish the table for the merge kernel
    for (int i = threadIdx.x; i <= a.B; i += blockDim.x) a.ws_hdr[i] = s_pre[i];
    for (int i = threadIdx.x; i < a.B; i += blockDim.x) a.ws_hdr[a.B + 1 + i] = s_len[i];
  }
  const int r0 = range_start(w, N, a.G);
  const int r1 = range_start(w + 1, N, a.G);
  if (r0 >= r1) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int hq = lane & 15;        // head of this lane's S^T / O^T column
  const int g = lane >> 4;         // token quad of this lane (S^T rows 4g..4g+3)

  // ---- physical page ids of the range, 256 at a time: lane i of ids[q]
  // holds the id of page c0 + 64q + i, so no block-table read sits on the
  // path of a page load.
  int ids[4] = {0, 0, 0, 0};
  // ring of kGBuf steps; a step is 2 consecutive pages of the range
  uint4 buf[kGBuf][2][kGKSteps];
  const size_t lane_off = (size_t)wv * kGKSteps * 512 + (size_t)lane * 8;
  auto page_id = [&](int kk) {  // kk: page index inside the current chunk
    const int r = kk & (kWave - 1), q = kk >> 6;
    const int i0 = __builtin_amdgcn_readlane(ids[0], r), i1 = __builtin_amdgcn_readlane(ids[1], r);
    const int i2 = __builtin_amdgcn_readlane(ids[2], r), i3 = __builtin_amdgcn_readlane(ids[3], r);
    return q == 0 ? i0 : q == 1 ? i1 : q == 2 ? i2 : i3;
  };
  auto issue = [&](int slot, int kk, int cn) {  // pages kk, kk+1 (clamped to the chunk)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const size_t base = (size_t)page_id(min(kk + h, cn - 1)) * kGPageElems + lane_off;
#pragma unroll
      for (int i = 0; i < kGKSteps; ++i) buf[slot][h][i] = ld16(a.kv + base + (size_t)i * 512);
    }
  };

  // ---- compute state; b_beg/b_end/b_len cache s_pre[b], s_pre[b+1] and
  // s_len[b] of the current sequence, so steps read no LDS for them.
  int b_cur = -1, b_beg = 0, b_end = 0, b_len = 0;
  int seg_start = r0;
  uint4 qreg[kGKSteps];
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[kGMTiles];
#pragma unroll
  for (int t = 0; t < kGMTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // transposed-read byte offset inside a V slice (m-tile t adds 512 t)
  const int s16 = lane & 15;
  const int tr_tok = 4 * g + (s16 >> 2);
  const int tr_off = ((s16 & 3) >> 1) * 256 + tr_tok * 16 + (s16 & 1) * 8;

  auto load_q = [&](int b) {
    const uint16_t* qb = a.q + ((size_t)b * kGH + hq) * kGD + wv * kGSlice + 8 * g;
#pragma unroll
    for (int i = 0; i < kGKSteps; ++i) qreg[i] = ld16(qb + 32 * i);
    wait_vmem_all();
  };

  auto finish_segment = [&](int b, int seg_end) {
    float lt = l_run + xor16(l_run);
    lt += xor32(lt);
    const bool whole = (seg_start == b_beg) && (seg_end == b_end);
    float* dst;
    float scale;
    if (whole) {
      dst = a.out + (size_t)b * kGH * kGD;
      scale = 1.f / lt;
    } else {
      const int slot = 2 * w + (seg_start == r0 ? 0 : 1);
      float* ws = a.ws + (size_t)slot * kGSlotFloats;
      dst = ws;
      scale = 1.f;
      if (wv == 0 && g == 0) {
        ws[kGH * kGD + hq] = m_run;
        ws[kGH * kGD + kGH + hq] = lt;
      }
    }
#pragma unroll
    for (int t = 0; t < kGMTiles; ++t) {
      const int d = wv * kGSlice + t * 16 + 4 * g;
      f32x4 v = acc[t] * scale;
      *reinterpret_cast<f32x4*>(dst + (size_t)hq * kGD + d) = v;
      acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    m_run = -INFINITY;
    l_run = 0.f;
    seg_start = seg_end;
  };

  // One step over the two pages of ring slot `slot` for sequence b. Page h
  // (0 or 1) takes part iff use[h]; j[h] is its page index in the sequence.
  // Tokens past the end of the sequence, and pages that do not take part,
  // get weight 0 and a zeroed V (0 * NaN would poison the MFMA sums).
  // s_part is double-buffered by exchange: consecutive steps must alternate
  // buffers (one barrier separates a buffer's reads from its next writes).
  int xb = 0;
  auto step = [&](int slot, int jA, bool useA, int jB, bool useB) {
    const int L = b_len;
    const int it = xb;
    xb ^= 1;
    const int jj[2] = {jA, jB};
    const bool use[2] = {useA, useB};
    f32x4 sp[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sp[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < kGKSteps; ++i)
        sp[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, buf[slot][h][i]),
                                                        __builtin_bit_cast(bf16x8, qreg[i]), sp[h], 0, 0, 0);
      s_part[it & 1][wv][h][lane] = sp[h];
    }
    // Edge step: a page left out, or tokens past the sequence end. Rare, so
    // the common path carries no masking work.
    const bool edge = !useA || !useB || (jB + 1) * kPage > L;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint16_t* vs = s_v[wv][h];
#pragma unroll
      for (int i = 0; i < kGKSteps; ++i)
        *reinterpret_cast<uint4*>(vs + i * 512 + lane * 8) = buf[slot][h][i];
    }
    if (edge) {  // zero the V rows of tokens with weight 0 (this lane's token)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (!(use[h] && jj[h] * kPage + (lane & 15) < L)) {
          uint16_t* vs = s_v[wv][h];
#pragma unroll
          for (int i = 0; i < kGKSteps; ++i)
            *reinterpret_cast<uint4*>(vs + i * 512 + lane * 8) = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
    __syncthreads();
    float sc[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 s = s_part[it & 1][0][h][lane];
#pragma unroll
      for (int ww = 1; ww < kGWaves; ++ww) s += s_part[it & 1][ww][h][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[4 * h + e] = s[e] * kLog2e;
    }
    if (edge) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (!(use[h] && jj[h] * kPage + 4 * g + e < L)) sc[4 * h + e] = -INFINITY;
    }
    // Lazy rescaling: m_run is a reference, not the exact running max. It
    // moves (and the state is rescaled) only when a score exceeds it by more
    // than kGRescale (log2 units), so p = 2^(s - m_run) stays below
    // 2^kGRescale and no fp32 quantity can overflow; any reference gives the
    // same softmax since numerator and denominator share it. The common case
    // needs no cross-lane max at all. Always taken on a segment's first step
    // (m_run = -inf).
    float lmax = sc[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) lmax = fmaxf(lmax, sc[e]);
    if (__any(lmax > m_run + kGRescale)) {
      float mp = fmaxf(lmax, xor16(lmax));
      mp = fmaxf(mp, xor32(mp));                                   // head max
      const float m_new = (mp > m_run + kGRescale) ? mp : m_run;  // mp finite
      const float alpha = exp2_fast(m_run - m_new);                // 0 from -inf
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < kGMTiles; ++t) acc[t] *= alpha;
    }
    // p = p_hi + p_lo with both parts in bf16: the two MFMAs below carry p
    // to about 2^-17 relative, so the result does not depend on where the
    // reference (and hence the bf16 rounding of p) happened to be.
    bf16x8 ph, pl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pv = exp2_fast(sc[e] - m_run);
      ph[e] = (__bf16)pv;
      pl[e] = (__bf16)(pv - (float)ph[e]);
      l_run += pv;
    }
    // O^T (d x heads) += V^T P^T over the 32 tokens of the step:
    // k-slots 8g..8g+3 are page A's tokens 4g..4g+3, 8g+4..8g+7 page B's.
#pragma unroll
    for (int t = 0; t < kGMTiles; ++t) {
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) char*)s_v[wv][0] +
                                                     t * 512 + tr_off));
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) char*)s_v[wv][1] +
                                                     t * 512 + tr_off));
      const bf16x8 vt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, ph, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pl, acc[t], 0, 0, 0);
    }
  };

  // Sequence of page p (uniform); reloads q when the sequence changes.
  auto enter = [&](int p) {
    if (p >= b_end) {  // also true before the first page (b_end = 0)
      b_cur = (b_cur < 0) ? seq_of_page(s_pre, a.B, p) : b_cur;
      while (s_pre[b_cur + 1] <= p) ++b_cur;
      b_beg = __builtin_amdgcn_readfirstlane(s_pre[b_cur]);
      b_end = __builtin_amdgcn_readfirstlane(s_pre[b_cur + 1]);
      b_len = __builtin_amdgcn_readfirstlane(s_len[b_cur]);
      load_q(b_cur);
    }
    return b_cur;
  };

  // Steps of two pages in range order. A step whose second page starts a new
  // sequence is done twice, once per page, with the other page left out.
  auto run_step = [&](int slot, int c0, int kk, int cn) {
    const int pA = c0 + kk, pB = pA + 1;
    const bool hasB = pB < r1 && kk + 1 < cn;
    // pass 0: page A (and B if it is in A's segment); pass 1: page B alone
    for (int pass = 0; pass < 2; ++pass) {
      const int pf = pass == 0 ? pA : pB;     // first page of this pass
      const int b = enter(pf);
      const int end = min(r1, b_end);  // end of the segment
      const bool useA = pass == 0;
      const bool useB = hasB && (pass == 1 || pB < end);
      step(slot, pA - b_beg, useA, pB - b_beg, useB);
      const int last = useB ? pB : pA;
      if (last + 1 == end) finish_segment(b, end);
      if (useB || !hasB) break;  // nothing left for a second pass
    }
  };

  // Ring of kGBuf steps, kGBuf-1 steps ahead. Loads past the chunk's end are
  // clamped to its last page (redundant, cache-resident) so that every pass
  // issues the same loads and the compiler waits only for the slot in use.
  for (int c0 = r0; c0 < r1; c0 += kGIdChunk) {
    const int cn = min(r1 - c0, kGIdChunk);   // even except at the range's end
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = c0 + q * kWave + lane;
      int id = 0;
      if (p < r1) {
        const int bb = seq_of_page(s_pre, a.B, p);
        id = a.bt[(size_t)bb * a.P_max + (p - s_pre[bb])];
      }
      ids[q] = id;
    }
    wait_vmem_all();
#pragma unroll
    for (int u = 0; u < kGBuf - 1; ++u) issue(u, min(2 * u, cn - 1), cn);
    for (int base = 0; base < cn; base += 2 * kGBuf) {
#pragma unroll
      for (int u = 0; u < kGBuf; ++u) {
        const int kk = base + 2 * u;
        issue((u + kGBuf - 1) % kGBuf, min(kk + 2 * (kGBuf - 1), cn - 1), cn);
        if (kk < cn) run_step(u, c0, kk, cn);
      }
    }
  }
}

// Log-sum-exp merge of the partial results of split sequences. Workgroup:
// (sequence b, head h, coordinate chunk of 4*TPS); its 256 threads form
// 256/TPS slot groups of TPS threads, each thread one float4 of the chunk, so
// the partials of a long sequence (hundreds of them) are read in parallel.
// Each group folds its slots with a running max; the groups are then combined
// the same way. The page prefix table comes from the workspace header.
template <int TPS>
__global__ __launch_bounds__(256) void lse_merge_kernel(GlobalArgs a) {
  constexpr int NG = 256 / TPS;   // slot groups
  constexpr int DCH = 4 * TPS;    // coordinates per workgroup
  constexpr int NDC = kGD / DCH;  // chunks per head
  __shared__ f32x4 s_num[NG][TPS];
  __shared__ float s_m[NG], s_den[NG];
  const int b = blockIdx.x / (kGH * NDC);
  const int rem = blockIdx.x - b * (kGH * NDC);
  const int h = rem / NDC;
  const int tid = threadIdx.x;
  const int grp = tid / TPS;
  const int d0 = (rem - h * NDC) * DCH + (tid % TPS) * 4;
  float* ob = a.out + ((size_t)b * kGH + h) * kGD + d0;
  const int* pre = a.ws_hdr;
  const int L = pre[a.B + 1 + b];
  if (L == 0) {
    if (grp == 0) *reinterpret_cast<f32x4*>(ob) = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  const int N = pre[a.B];
  const int pb = pre[b], pe = pre[b + 1];
  // workgroup whose range holds page p: largest w with range_start(w) <= p
  auto wg_of = [&](int p) { return (int)((((long long)p + 1) * a.G - 1) / N); };
  const int w0 = wg_of(pb), w1 = wg_of(pe - 1);
  if (w0 == w1) return;  // finished inside one workgroup
  float m = -INFINITY, den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  constexpr int U = 4;  // pieces gathered per step, loads independent
  for (int w = w0 + grp; w <= w1; w += U * NG) {
    float mi[U], li[U];
    f32x4 ai[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ww = w + u * NG;
      mi[u] = -INFINITY;
      li[u] = 0.f;
      ai[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (ww > w1) continue;
      const int rs = range_start(ww, N, a.G);
      if (rs == range_start(ww + 1, N, a.G)) continue;  // empty range: no piece
      const int sl = 2 * ww + ((ww == w0 && rs != pb) ? 1 : 0);
      const float* ws = a.ws + (size_t)sl * kGSlotFloats;
      mi[u] = ws[kGH * kGD + h];
      li[u] = ws[kGH * kGD + kGH + h];
      ai[u] = *reinterpret_cast<const f32x4*>(ws + (size_t)h * kGD + d0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (mi[u] == -INFINITY) continue;
      const float mn = fmaxf(m, mi[u]);
      const float fo = exp2_fast(m - mn);  // 0 when m = -inf
      const float fi = exp2_fast(mi[u] - mn);
      num = num * fo + ai[u] * fi;
      den = den * fo + li[u] * fi;
      m = mn;
    }
  }
  s_num[grp][tid % TPS] = num;
  if (tid % TPS == 0) {
    s_m[grp] = m;
    s_den[grp] = den;
  }
  __syncthreads();
  if (grp == 0) {
    float M = s_m[0];
#pragma unroll
    for (int gq = 1; gq < NG; ++gq) M = fmaxf(M, s_m[gq]);
    f32x4 n = {0.f, 0.f, 0.f, 0.f};
    float dd = 0.f;
#pragma unroll
    for (int gq = 0; gq < NG; ++gq) {
      const float f = (s_m[gq] == -INFINITY) ? 0.f : exp2_fast(s_m[gq] - M);
      n += f * s_num[gq][tid];
      dd += f * s_den[gq];
    }
    *reinterpret_cast<f32x4*>(ob) = n * (1.f / dd);
  }
}

int global_num_splits(const da_shape& s, int num_cus) {
  if (s.num_splits > 0) return s.num_splits;
  return 2 * num_cus;
}

size_t global_workspace_bytes(const da_shape& s, int num_splits) {
  (void)s;
  if (num_splits <= 1) return 0;  // one workgroup finishes every sequence itself
  return kGHeaderBytes + (size_t)2 * (size_t)num_splits * kGSlotFloats * sizeof(float);
}

da_status launch_global(const void* q, const void* kv_cache, const int32_t* block_table,
                        const int32_t* seq_lens, void* out, const da_shape& s, int num_splits,
                        void* workspace, hipStream_t stream) {
  GlobalArgs a;
  a.q = (const uint16_t*)q;
  a.kv = (const uint16_t*)kv_cache;
  a.bt = block_table;
  a.seq_lens = seq_lens;
  a.out = (float*)out;
  a.ws_hdr = num_splits > 1 ? (int*)workspace : nullptr;
  a.ws = num_splits > 1 ? (float*)((char*)workspace + kGHeaderBytes) : nullptr;
  a.B = s.batch;
  a.P_max = s.max_pages_per_seq;
  a.G = num_splits;
  hipLaunchKernelGGL(global_decode_kernel, dim3((unsigned)num_splits), dim3(kGThreads), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return DA_ERR_LAUNCH;
  if (num_splits <= 1) return DA_OK;  // nothing was split: no merge
  // Expected pieces per sequence ~ G/B + 2: more pieces, more slot groups.
  const int est = num_splits / s.batch + 2;
  const unsigned nb = (unsigned)s.batch * kGH;
  if (est <= 16)
    hipLaunchKernelGGL(lse_merge_kernel<128>, dim3(nb * 1), dim3(256), 0, stream, a);
  else if (est <= 32)
    hipLaunchKernelGGL(lse_merge_kernel<64>, dim3(nb * 2), dim3(256), 0, stream, a);
  else if (est <= 64)
    hipLaunchKernelGGL(lse_merge_kernel<32>, dim3(nb * 4), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(lse_merge_kernel<16>, dim3(nb * 8), dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

}  // namespace da
