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
constexpr int kGIdChunk = 4 * kWave;  // page ids gathered per refill (4 per lane)
// Workspace: a header with the page prefix table (written by workgroup 0 of
// the decode kernel, read by the merge), then 2*G partial-result slots.
constexpr size_t kGHeaderBytes = 16384;  // >= (2*kGMaxBatch + 1) ints
static_assert((2 * kGMaxBatch + 1) * sizeof(int) <= kGHeaderBytes, "header too small");
#ifndef DA_GLOBAL_RING
#define DA_GLOBAL_RING 4
#endif
constexpr int kGBuf = DA_GLOBAL_RING;  // page slices held per wave (ring; kGBuf-1 in flight ahead)

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
  __shared__ f32x4 s_part[2][kGWaves][kWave];            // partial S^T tiles
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kGWaves][kGSlice * kPage];  // V slices

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
  uint4 buf[kGBuf][kGKSteps];
  const size_t lane_off = (size_t)wv * kGKSteps * 512 + (size_t)lane * 8;
  auto issue = [&](int slot, int kk) {  // kk: page index inside the current chunk
    const int r = kk & (kWave - 1), q = kk >> 6;
    const int i0 = __builtin_amdgcn_readlane(ids[0], r), i1 = __builtin_amdgcn_readlane(ids[1], r);
    const int i2 = __builtin_amdgcn_readlane(ids[2], r), i3 = __builtin_amdgcn_readlane(ids[3], r);
    const int phys = q == 0 ? i0 : q == 1 ? i1 : q == 2 ? i2 : i3;
    const size_t base = (size_t)phys * kGPageElems + lane_off;
#pragma unroll
    for (int i = 0; i < kGKSteps; ++i) buf[slot][i] = ld16(a.kv + base + (size_t)i * 512);
  };

  // ---- compute state
  int b_cur = -1;
  int seg_start = r0;
  uint4 qreg[kGKSteps];
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[kGMTiles];
#pragma unroll
  for (int t = 0; t < kGMTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // transposed-read byte offsets inside this wave's V slice, per m-tile
  const int s16 = lane & 15;
  const int tr_tok = 4 * g + (s16 >> 2);
  const int tr_off = ((s16 & 3) >> 1) * 256 + tr_tok * 16 + (s16 & 1) * 8;
  uint16_t* vs = s_v[wv];

  auto finish_segment = [&](int b, int seg_end) {
    float lt = l_run + xor16(l_run);
    lt += xor32(lt);
    const bool whole = (seg_start == s_pre[b]) && (seg_end == s_pre[b + 1]);
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

  auto compute = [&](int slot, int p, int it) {
    // sequence of page p (uniform); reload q at a sequence change
    if (b_cur < 0 || s_pre[b_cur + 1] <= p) {
      b_cur = (b_cur < 0) ? seq_of_page(s_pre, a.B, p) : b_cur;
      while (s_pre[b_cur + 1] <= p) ++b_cur;
      const uint16_t* qb = a.q + ((size_t)b_cur * kGH + hq) * kGD + wv * kGSlice + 8 * g;
#pragma unroll
      for (int i = 0; i < kGKSteps; ++i) qreg[i] = ld16(qb + 32 * i);
      wait_vmem_all();
    }
    const int b = b_cur;
    const int j = p - s_pre[b];
    const int L = s_len[b];
    const bool last_page = (j + 1) * kPage > L;

    // partial S^T over this wave's 128 coordinates
    f32x4 sp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kGKSteps; ++i)
      sp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, buf[slot][i]),
                                                   __builtin_bit_cast(bf16x8, qreg[i]), sp, 0, 0, 0);
    s_part[it & 1][wv][lane] = sp;
    // V slice: zero tokens past the end of the sequence (0 * NaN = NaN)
    if (last_page && j * kPage + (lane & 15) >= L) {
#pragma unroll
      for (int i = 0; i < kGKSteps; ++i) buf[slot][i] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < kGKSteps; ++i)
      *reinterpret_cast<uint4*>(vs + i * 512 + lane * 8) = buf[slot][i];
    __syncthreads();
    f32x4 s = s_part[it & 1][0][lane];
#pragma unroll
    for (int ww = 1; ww < kGWaves; ++ww) s += s_part[it & 1][ww][lane];

    float sc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sc[e] = s[e] * kLog2e;
      if (last_page && j * kPage + 4 * g + e >= L) sc[e] = -INFINITY;
    }
    float mp = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mp = fmaxf(mp, xor16(mp));
    mp = fmaxf(mp, xor32(mp));
    // Lazy rescaling: m_run is a reference, not the exact running max. It
    // moves (and the state is rescaled) only when a head's page max exceeds
    // it by more than kGRescale (log2 units), so p = 2^(s - m_run) stays
    // below 2^kGRescale and no fp32 quantity can overflow; any reference
    // gives the same softmax since numerator and denominator share it.
    // Always taken on a segment's first page (m_run = -inf).
    if (__any(mp > m_run + kGRescale)) {
      const float m_new = (mp > m_run + kGRescale) ? mp : m_run;  // mp finite
      const float alpha = exp2_fast(m_run - m_new);                // 0 from -inf
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < kGMTiles; ++t) acc[t] *= alpha;
    }
    const float m_new = m_run;
    // p = p_hi + p_lo with both parts in bf16: the two MFMAs below carry p
    // to about 2^-17 relative, so the result does not depend on where the
    // reference (and hence the bf16 rounding of p) happened to be.
    bf16x4 ph, pl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = exp2_fast(sc[e] - m_new);
      ph[e] = (__bf16)p;
      pl[e] = (__bf16)(p - (float)ph[e]);
      l_run += p;
    }
#pragma unroll
    for (int t = 0; t < kGMTiles; ++t) {
      const bf16x4 vt = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) char*)vs +
                                                     t * 512 + tr_off)));
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, ph, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pl, acc[t], 0, 0, 0);
    }
    const int seg_end = min(r1, s_pre[b + 1]);
    if (p + 1 == seg_end) finish_segment(b, seg_end);
  };

  // Ring of kGBuf page slices, kGBuf-1 pages ahead. Prefetches past the
  // chunk's end are clamped to its last page (redundant, cache-resident
  // loads) so that every pass issues the same loads.
  int it = 0;
  for (int c0 = r0; c0 < r1; c0 += kGIdChunk) {
    const int cn = min(r1 - c0, kGIdChunk);
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
    for (int u = 0; u < kGBuf - 1; ++u) issue(u, min(u, cn - 1));
    for (int base = 0; base < cn; base += kGBuf) {
      // No early exit: every step issues one page, so the compiler sees the
      // same number of loads in flight on every path and waits only for the
      // slot being computed.
#pragma unroll
      for (int u = 0; u < kGBuf; ++u) {
        const int kk = base + u;
        issue((u + kGBuf - 1) % kGBuf, min(kk + kGBuf - 1, cn - 1));
        if (kk < cn) {
          compute(u, c0 + kk, it);
          ++it;
        }
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
