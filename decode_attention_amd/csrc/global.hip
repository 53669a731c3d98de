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
// A workgroup (one per compute unit) has 8 waves in 4 pairs. The pairs take
// the pages of a segment round-robin, 4 pages per step, and all 8 waves meet
// at one barrier per step, so no wave on the compute unit runs ahead of the
// others; the 4 pair states are merged through LDS when the segment ends.
// Inside a pair the 2 waves share a page: wave half h owns coordinates
// [256h, 256h+256), i.e. 8 KB of the 16 KB page, loaded with lane-linear
// 16-byte loads that land directly in the MFMA A-operand layout of K.
//   S^T (16 tokens x 16 heads) = K Q^T : 8 x mfma_f32_16x16x32_bf16 per wave
//     on its 256 coordinates; the 2 partial tiles are added through LDS in a
//     fixed order, so both waves hold the same scores.
//   The S^T accumulator layout (lane: head l%16, tokens 4(l/16)..+3) is the
//     B operand layout of the PV product, so probabilities never move
//     between lanes.
//   O^T (256 x 16 per wave) += V^T P^T: V = K, the wave's 8 KB is written to
//     LDS once and read back transposed with ds_read_b64_tr_b16 (512
//     contiguous bytes per instruction). One mfma_f32_16x16x32_bf16 per
//     16-row tile: its 32-wide k dimension holds the page's 16 tokens twice,
//     against bf16(p) and against bf16(p - bf16(p)), so p enters the product
//     to about 2^-17 relative.
#include "common.hpp"
#include "launch.hpp"

namespace da {

constexpr int kGD = 512;          // head dim
constexpr int kGH = 16;           // query heads (KV head count 1)
constexpr int kGPair = 2;         // waves sharing a page (coordinate halves)
constexpr int kGPairs = 4;        // pairs per workgroup (4 pages per step)
constexpr int kGWaves = kGPair * kGPairs;
constexpr int kGThreads = kGWaves * kWave;
constexpr int kGSlice = kGD / kGPair;         // coordinates per wave (256)
constexpr int kGKSteps = kGSlice / 32;        // 16x16x32 k-steps per wave (8)
constexpr int kGMTiles = kGSlice / 16;        // 16-row output tiles per wave (16)
constexpr int kGPageElems = kPage * kGD;      // bf16 elements per page (8192)
// Partial slot: the unnormalised output in lane order, [2 halves][16 tiles]
// [64 lanes][4] floats (element (h, d) with d = 256f + 16t + 4g + e sits at
// lane h + 16g, tile t, half f), then m[16] and l[16].
constexpr int kGSlotFloats = kGH * kGD + 2 * kGH;
constexpr int kGMaxBatch = 256;   // the model's batch domain is [1, 256]
constexpr float kGRescale = 32.f;  // lazy-rescale threshold, log2 units
constexpr int kGIdChunk = 4 * kWave;  // page ids gathered per refill (4 per lane); even
// Workspace: a header with the page prefix table (written by workgroup 0 of
// the decode kernel, read by the merge), then 2*G partial-result slots.
constexpr size_t kGHeaderBytes = 16384;  // >= (2*kGMaxBatch + 1) ints
static_assert((2 * kGMaxBatch + 1) * sizeof(int) <= kGHeaderBytes, "header too small");
#ifndef DA_GLOBAL_RING
#define DA_GLOBAL_RING 3
#endif
constexpr int kGBuf = DA_GLOBAL_RING;  // pages held per wave (ring; kGBuf-1 ahead)

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

__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(2))) void global_decode_kernel(GlobalArgs a) {
  __shared__ int s_pre[kGMaxBatch + 1];
  __shared__ int s_len[kGMaxBatch];
  __shared__ int s_tmp[kGThreads];
  __shared__ f32x4 s_part[2][kGWaves][kWave];  // partial S^T tiles (double-buffered)
  // V slices, one per wave; also the merge area at the end of a segment
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kGWaves][kGSlice * kPage];
  __shared__ float s_ml[4][2][kWave];           // m, l of the wave states being merged

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
  const int pr = wv >> 1;          // pair
  const int hf = wv & 1;           // coordinate half of this wave
  const int hq = lane & 15;        // head of this lane's S^T / O^T column
  const int g = lane >> 4;         // token quad of this lane (S^T rows 4g..4g+3)

  int ids[4] = {0, 0, 0, 0};       // physical ids of this pair's pages, 256 at a time
  uint4 buf[kGBuf][kGKSteps];      // ring of this wave's page slices
  uint4 qreg[kGKSteps];            // Q^T B operands: head hq, d = 256hf + 32i + 8g .. +8
  f32x4 acc[kGMTiles];             // O^T: head hq, d = 256hf + 16t + 4g + e
  float m_run = -INFINITY, l_run = 0.f;
  const size_t lane_off = (size_t)hf * kGKSteps * 512 + (size_t)lane * 8;
  uint16_t* vs = s_v[wv];
  const int s16 = lane & 15;
  const int tr_tok = 4 * g + (s16 >> 2);
  const int tr_off = ((s16 & 3) >> 1) * 256 + tr_tok * 16 + (s16 & 1) * 8;  // + 512 t

  auto issue = [&](int slot, int kk) {  // kk: step index inside the current id chunk
    const int r = kk & (kWave - 1), q = kk >> 6;
    const int i0 = __builtin_amdgcn_readlane(ids[0], r), i1 = __builtin_amdgcn_readlane(ids[1], r);
    const int i2 = __builtin_amdgcn_readlane(ids[2], r), i3 = __builtin_amdgcn_readlane(ids[3], r);
    const int phys = q == 0 ? i0 : q == 1 ? i1 : q == 2 ? i2 : i3;
    const size_t base = (size_t)phys * kGPageElems + lane_off;
#pragma unroll
    for (int i = 0; i < kGKSteps; ++i) buf[slot][i] = ld16(a.kv + base + (size_t)i * 512);
  };

  // s_part is double-buffered by step: consecutive steps alternate buffers
  // (one barrier separates a buffer's reads from its next writes).
  int xb = 0;
  // One step for this pair: page j of the current sequence (L cached tokens)
  // from ring slot `slot`; `valid` false when the pair has no page this step.
  auto compute = [&](int slot, int j, bool valid, int L) {
    f32x4 s2[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int i = 0; i < kGKSteps; ++i)
      s2[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, buf[slot][i]),
                                                          __builtin_bit_cast(bf16x8, qreg[i]), s2[i & 1],
                                                          0, 0, 0);
    s_part[xb][wv][lane] = s2[0] + s2[1];
#pragma unroll
    for (int i = 0; i < kGKSteps; ++i) *reinterpret_cast<uint4*>(vs + i * 512 + lane * 8) = buf[slot][i];
    const bool edge = !valid || (j + 1) * kPage > L;  // rare
    if (edge && (!valid || j * kPage + (lane & 15) >= L)) {
      // zero the V row of this lane's token (weight 0; 0 * NaN would poison)
#pragma unroll
      for (int i = 0; i < kGKSteps; ++i)
        *reinterpret_cast<uint4*>(vs + i * 512 + lane * 8) = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();
    const f32x4 s = s_part[xb][wv & ~1][lane] + s_part[xb][wv | 1][lane];
    xb ^= 1;
    if (!valid) return;  // uniform per pair; no barrier follows in this step
    float sc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) sc[e] = s[e] * kLog2e;
    if (edge) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j * kPage + 4 * g + e >= L) sc[e] = -INFINITY;
    }
    // Lazy rescaling: m_run is a reference, not the exact running max. It
    // moves (and the state is rescaled) only when a score exceeds it by more
    // than kGRescale (log2 units), so p = 2^(s - m_run) stays below
    // 2^kGRescale and no fp32 quantity can overflow; any reference gives the
    // same softmax since numerator and denominator share it. The common case
    // needs no cross-lane max. Always taken on a pair's first page.
    const float lmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
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
    // P^T operand: k-slots 8g..8g+3 hold bf16(p) of tokens 4g..4g+3 and
    // 8g+4..8g+7 the remainder bf16(p - bf16(p)); the V^T operand repeats the
    // same 4 tokens in both halves.
    bf16x8 pp;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float pv = exp2_fast(sc[e] - m_run);
      pp[e] = (__bf16)pv;
      pp[4 + e] = (__bf16)(pv - (float)pp[e]);
      l_run += pv;
    }
#pragma unroll
    for (int t = 0; t < kGMTiles; ++t) {
      const s16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) char*)vs +
                                                     t * 512 + tr_off));
      const bf16x8 vt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v4, v4, 0, 1, 2, 3, 0, 1, 2, 3));
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pp, acc[t], 0, 0, 0);
    }
  };

  // End-of-segment merge through LDS (the V regions are free by then): a
  // wave state is m (per head), l (lane partial) and its 16 accumulator tiles.
  f32x4* st = reinterpret_cast<f32x4*>(&s_v[0][0]);  // 4 states of [16][64] f32x4
  auto put_state = [&](int k) {
#pragma unroll
    for (int t = 0; t < kGMTiles; ++t) st[(k * kGMTiles + t) * kWave + lane] = acc[t];
    s_ml[k][0][lane] = m_run;
    s_ml[k][1][lane] = l_run;
  };
  auto take_state = [&](int k) {  // fold stored state k into this one
    const float m_o = s_ml[k][0][lane], l_o = s_ml[k][1][lane];
    const float M = fmaxf(m_run, m_o);
    const float fs = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - M);
    const float fo = (m_o == -INFINITY) ? 0.f : exp2_fast(m_o - M);
#pragma unroll
    for (int t = 0; t < kGMTiles; ++t) acc[t] = acc[t] * fs + st[(k * kGMTiles + t) * kWave + lane] * fo;
    l_run = l_run * fs + l_o * fo;
    m_run = M;
  };

  int b = seq_of_page(s_pre, a.B, r0);
  for (int s0 = r0; s0 < r1;) {
    while (s_pre[b + 1] <= s0) ++b;  // uniform; skips empty sequences
    const int pb = __builtin_amdgcn_readfirstlane(s_pre[b]);
    const int pe = __builtin_amdgcn_readfirstlane(s_pre[b + 1]);
    const int L = __builtin_amdgcn_readfirstlane(s_len[b]);
    const int s1 = min(r1, pe);                            // segment [s0, s1) of sequence b
    const int nsteps = (s1 - s0 + kGPairs - 1) / kGPairs;  // this pair's page of step k: s0 + 4k + pr
    {
      const uint16_t* qb = a.q + ((size_t)b * kGH + hq) * kGD + hf * kGSlice + 8 * g;
#pragma unroll
      for (int i = 0; i < kGKSteps; ++i) qreg[i] = ld16(qb + 32 * i);
    }
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int t = 0; t < kGMTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nsteps; c0 += kGIdChunk) {
      const int cn = min(nsteps - c0, kGIdChunk);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = c0 + q * kWave + lane;
        const int pg = s0 + kGPairs * k + pr;  // a step past the end loads the first page again
        ids[q] = a.bt[(size_t)b * a.P_max + (k < nsteps && pg < s1 ? pg : s0) - pb];
      }
      wait_vmem_all();
      // Ring of kGBuf steps, kGBuf-1 ahead; loads past the chunk's end are
      // clamped to its last step (redundant, cache-resident) so that every
      // pass issues the same loads and the compiler waits only for the slot
      // in use.
#pragma unroll
      for (int u = 0; u < kGBuf - 1; ++u) issue(u, min(u, cn - 1));
      for (int base = 0; base < cn; base += kGBuf) {
#pragma unroll
        for (int u = 0; u < kGBuf; ++u) {
          const int kk = base + u;
          issue((u + kGBuf - 1) % kGBuf, min(kk + kGBuf - 1, cn - 1));
          if (kk < cn) {
            const int pg = s0 + kGPairs * (c0 + kk) + pr;
            compute(u, pg - pb, pg < s1, L);
          }
        }
      }
    }
    // Merge the 4 pair states (same coordinate half): 2 -> 0 and 3 -> 1, then 1 -> 0.
    __syncthreads();  // every wave is done with its V region
    if (pr >= 2) put_state((pr - 2) * kGPair + hf);
    __syncthreads();
    if (pr < 2) take_state(pr * kGPair + hf);
    __syncthreads();
    if (pr == 1) put_state(hf);
    __syncthreads();
    if (pr == 0) {
      take_state(hf);
      float lt = l_run + xor16(l_run);
      lt += xor32(lt);
      if (s0 == pb && s1 == pe) {  // whole sequence in this workgroup: o[b][h][d]
        float* dst = a.out + ((size_t)b * kGH + hq) * kGD + hf * kGSlice + 4 * g;
        const float inv = 1.f / lt;
#pragma unroll
        for (int t = 0; t < kGMTiles; ++t) *reinterpret_cast<f32x4*>(dst + t * 16) = acc[t] * inv;
      } else {                     // partial slot, lane order: 1 KB contiguous per store
        float* ws = a.ws + (size_t)(2 * w + (s0 == r0 ? 0 : 1)) * kGSlotFloats;
        if (hf == 0 && g == 0) {
          ws[kGH * kGD + hq] = m_run;
          ws[kGH * kGD + kGH + hq] = lt;
        }
#pragma unroll
        for (int t = 0; t < kGMTiles; ++t)
          *reinterpret_cast<f32x4*>(ws + ((size_t)(hf * kGMTiles + t) * kWave + lane) * 4) = acc[t];
      }
    }
    __syncthreads();  // the merge area is page space again
    s0 = s1;
  }
}

// Log-sum-exp merge of the partial results of split sequences. Workgroup:
// (sequence b, output tile T = 16 coordinates of all 16 heads, i.e. one
// lane-order tile of a partial slot); its NG groups of 64 threads fold the
// sequence's pieces w0+grp, w0+grp+NG, ... with a running max, reading 1 KB
// contiguous per piece, and are then combined the same way. The page prefix
// table comes from the workspace header.
template <int NG>
__global__ __launch_bounds__(64 * NG) void lse_merge_kernel(GlobalArgs a) {
  constexpr int kTiles = kGPair * kGMTiles;   // 32 tiles of 16 coordinates
  __shared__ f32x4 s_num[NG][kWave];
  __shared__ float s_m[NG][kWave], s_den[NG][kWave];
  const int b = blockIdx.x / kTiles;
  const int T = blockIdx.x - b * kTiles;
  const int lane = threadIdx.x & (kWave - 1);
  const int grp = threadIdx.x / kWave;
  const int h = lane & 15, g = lane >> 4;
  const int d0 = (T / kGMTiles) * kGSlice + (T % kGMTiles) * 16 + 4 * g;
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
  const size_t off = ((size_t)T * kWave + lane) * 4;
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
      ai[u] = *reinterpret_cast<const f32x4*>(ws + off);
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
  s_num[grp][lane] = num;
  s_m[grp][lane] = m;
  s_den[grp][lane] = den;
  __syncthreads();
  if (grp == 0) {
    float M = s_m[0][lane];
#pragma unroll
    for (int gq = 1; gq < NG; ++gq) M = fmaxf(M, s_m[gq][lane]);
    f32x4 n = {0.f, 0.f, 0.f, 0.f};
    float dd = 0.f;
#pragma unroll
    for (int gq = 0; gq < NG; ++gq) {
      const float f = (s_m[gq][lane] == -INFINITY) ? 0.f : exp2_fast(s_m[gq][lane] - M);
      n += f * s_num[gq][lane];
      dd += f * s_den[gq][lane];
    }
    *reinterpret_cast<f32x4*>(ob) = n * (1.f / dd);
  }
}

int global_num_splits(const da_shape& s, int num_cus) {
  if (s.num_splits > 0) return s.num_splits;
  return num_cus;  // one workgroup per compute unit
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
  const unsigned nb = (unsigned)s.batch * (kGPair * kGMTiles);
  if (est <= 24)
    hipLaunchKernelGGL(lse_merge_kernel<4>, dim3(nb), dim3(4 * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL(lse_merge_kernel<16>, dim3(nb), dim3(16 * kWave), 0, stream, a);
  return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

}  // namespace da
