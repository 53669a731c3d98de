// decodeGQA over a paged K=V cache, tiled layout [pages][1][D/8][16][8] bf16.
//
// Pages: Op Specs of google/gemma-4-12B (Attention.lean: softmax, causalGQA,
// decodeGQA) and the gemma-4-12b Model Spec attn.core row for the global
// layers (scale 1, 16 query heads on 1 KV head, D = 512, values = keys).
//
// Work split. The cached pages of the whole batch form one list (sequence by
// sequence); workgroup w of G takes the range of pages [w*N/G, (w+1)*N/G)
// and walks it in steps of up to 4 pages of one sequence. A sequence that lies inside one range is finished there; a
// sequence cut by range boundaries leaves one partial result (unnormalised
// output, running max m and sum l per head) per piece, and lse_merge_kernel
// combines them:
//   M = max_i m_i,  o = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i
// (scores are kept in the log2 domain). This is exact over the reals because
// the softmax over a union of disjoint key sets factorises that way.
//
// The split is static: equal page counts per workgroup, one workgroup per
// compute unit by default, and the result is reproducible bit for bit.
//
// A workgroup (one per compute unit) has 8 waves in 4 pairs. The pairs take
// the pages of a step (pair p: page P + p), and all 8 waves meet at one
// barrier per step, so no wave on the compute unit runs ahead of the others;
// the 4 pair states are merged through LDS when a segment (the part of one
// sequence inside a range) ends. Inside a pair the 2 waves share a page:
// wave half h owns coordinates [256h, 256h+256), i.e. 8 KB of the 16 KB page,
// loaded with lane-linear 16-byte loads that land directly in the MFMA
// A-operand layout of K.
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
// Loads run ahead of the compute across segment and sequence boundaries:
// page ids 4 steps, page slices 2 steps; a segment change costs a q reload
// and an LDS merge, not a pipeline restart.
//
// Pre-norm variant (PRE): the cache holds the shared pre-norm projection x
// of every token (Model Spec compute-graph nodes attn.qk_norm, attn.v_norm,
// attn.rope on global layers: k = rope(rmsnorm(x, w_k)), v = rmsnormUnit(x);
// Op Specs Norm.lean and Rope.lean, theta 1e6, rot = denom = 512, the first
// 64 frequencies active). With r = 1/sqrt(mean(x^2) + eps) per token,
//   q . k = r * (q . R(x * w_k))   and   v = r * x,
// so the page is still read once: r scales the score and the weight p of
// the PV product (the denominator keeps p), w_k moves onto q for the 384
// coordinates RoPE leaves alone (q * w_k as bf16 hi + lo, two MFMAs), and the
// 128 rotated coordinates are rotated in fp32 in registers and enter the
// MFMA as bf16 hi + lo. The cache layout puts the 32-coordinate block B in
// half B % 2, k-step B / 2, so a rotation pair (d, d + 256), d < 64, sits in
// one lane: k-steps 0 and 4 of each half. Angles: pos * theta^(-d/256) in
// revolutions, in fp64, wrapped to [-1/2, 1/2] before the fp32 sin/cos.
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace da {

constexpr int kGD = 512;          // head dim
constexpr int kGH = 16;           // query heads (KV head count 1)
constexpr int kGPair = 2;         // waves sharing a page (coordinate halves)
constexpr int kGPairs = 4;        // pairs per workgroup (up to 4 pages per step)
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
constexpr int kGBuf = 3;          // page slices per wave in flight (ring, 2 ahead)
constexpr int kGDesc = 6;         // step descriptors kept (ids are loaded 4 ahead)
#ifndef DA_GLOBAL_VT_BATCH
#define DA_GLOBAL_VT_BATCH 8
#endif


// Workspace: a header with the page prefix table (written by workgroup 0 of
// the decode kernel, read by the merge), then 2*G partial-result slots.
constexpr size_t kGHeaderBytes = 16384;  // >= (3*kGMaxBatch + 2) ints
static_assert((3 * kGMaxBatch + 2) * sizeof(int) <= kGHeaderBytes, "header too small");
// The split weighs a sequence start as this many pages: a workgroup whose
// range opens another segment merges and writes the previous one and stages
// the next q rows (~4 us at B = 64, about 8 pages of its page walk), so it
// takes that many pages less.
constexpr int kGSegPages = 8;

struct GlobalArgs {
  const float* w_k;          // pre-norm variant: k-norm weight [512]; else null
  const uint16_t* q;         // [B][16][512] bf16 bits
  const uint16_t* kv;        // [P][1][64][16][8] bf16 bits
  const int32_t* bt;         // [B][P_max]
  const int32_t* seq_lens;   // [B]
  void* out;                 // [B][16][512], fp32 or (out_bf16) bf16
  const float* gate;         // [B][16][512] sigmoidGate epilogue, or null
  int* ws_hdr;               // [B+1] page prefix, [B] clamped lengths, [B+1] weighted prefix
  float* ws;                 // [2*G][kGSlotFloats] partial slots
  unsigned long long* trace; // [G][4] per-workgroup timeline (TRACE instance only)
  int B, P_max, G;
  int out_bf16;              // the output is bf16 (rounded to nearest even), else fp32
};

// Shared by both kernels: per-sequence page counts and their prefix sums.
// L is clamped to 16*P_max so no block-table read can leave the row.
// s_vpre is the same prefix in weighted pages: kGSegPages more before each
// sequence that has pages, s_vpre[b] = s_pre[b] + kGSegPages * (sequences
// with pages among 0 .. b-1).
// One wave builds both (lane l takes sequences 4l .. 4l + 3, one scan
// across the wave, no barrier inside); the other waves wait at the single
// barrier at the end.
static_assert(kGMaxBatch <= 4 * kWave, "one wave scans the batch");
__device__ __forceinline__ void build_prefix(const GlobalArgs& a, int* s_pre, int* s_len, int* s_vpre) {
  if (threadIdx.x < kWave) {
    const int l = threadIdx.x;
    // pages in the low word (at most batch * P_max <= 2^30, checked by the
    // host), sequences with pages in the high word: one scan for both
    constexpr unsigned long long kSeq = 1ull << 32;
    int L[4];
    unsigned long long local = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = 4 * l + k;
      int v = i < a.B ? a.seq_lens[i] : 0;
      v = v < 0 ? 0 : (v > a.P_max * kPage ? a.P_max * kPage : v);
      L[k] = v;
      local += (unsigned long long)((v + kPage - 1) / kPage) + (v > 0 ? kSeq : 0ull);
    }
    unsigned long long incl = local;  // inclusive scan across the wave
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const unsigned long long y = __shfl_up(incl, d, kWave);
      if (l >= d) incl += y;
    }
    unsigned long long run = incl - local;
    if (l == 0) {
      s_pre[0] = 0;
      s_vpre[0] = 0;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = 4 * l + k;
      if (i < a.B) {
        s_len[i] = L[k];
        run += (unsigned long long)((L[k] + kPage - 1) / kPage) + (L[k] > 0 ? kSeq : 0ull);
        const int pages = (int)(run & (kSeq - 1)), seqs = (int)(run >> 32);
        s_pre[i + 1] = pages;
        s_vpre[i + 1] = pages + kGSegPages * seqs;
      }
    }
  }
  __syncthreads();
}

// First page of workgroup w's range: the split is even in weighted pages,
// workgroup w starting at weighted position v = floor(w V / G); a position in
// the kGSegPages before a sequence's first page maps to that page.
__device__ __forceinline__ int range_real(int w, int G, const int* s_pre, const int* s_vpre, int B) {
  const int V = s_vpre[B];
  const int v = (int)(((long long)w * V) / G);
  if (v >= V) return s_pre[B];
  // the sequence b with s_vpre[b] <= v < s_vpre[b + 1] (it has pages)
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s_vpre[mid + 1] <= v) lo = mid + 1; else hi = mid;
  }
  return s_pre[lo] + max(0, v - s_vpre[lo] - kGSegPages);
}

__device__ __forceinline__ int range_start(int w, int N, int G) {
  return (int)(((long long)w * N) / G);
}

// floor(x / d) for 0 <= x < 2^52 and 0 < d < 2^31, through a double quotient
// (within one of the exact one) and one correction step: a few instructions
// where a 64-bit integer division takes dozens.
__device__ __forceinline__ int div_floor_small(long long x, int d) {
  long long q = (long long)((double)x / (double)d);
  if (q * d > x) --q;
  else if ((q + 1) * d <= x) ++q;
  return (int)q;
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

__device__ __forceinline__ int rfl(int x) { return __builtin_amdgcn_readfirstlane(x); }


// x, opaque to the optimiser: addresses derived from it inside a rarely taken
// branch are computed there, not hoisted out of the loop into registers that
// would stay live across every step.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// s_getreg operands: hwreg(HW_REG_XCC_ID, 0, 16) and hwreg(HW_REG_HW_ID, 0, 32)
constexpr int kHwRegXccId = 20 | (15 << 11);
constexpr int kHwRegHwId = 4 | (31 << 11);

constexpr double kPreTheta = 1000000.0;  // RoPE base of the global layers
constexpr int kPreActive = 64;           // active frequencies (pairs d, d + 256 with d < 64)
constexpr float kPreEps = 1e-6f;

// Dword e (compile-time after unrolling) of a uint4 held in registers;
// taking the address of a register array would move it to scratch.
__device__ __forceinline__ uint32_t u4_get(const uint4& v, int e) {
  return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}
__device__ __forceinline__ uint32_t pack_bf16(__bf16 lo, __bf16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// (a, b) rounded to bf16, packed (a in the low half): one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// hi = bf16(a, b), lo = bf16 of the remainders: a ~ hi + lo to about 2^-17
__device__ __forceinline__ void split_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = cvt_pk_bf16(a, b);
  lo = cvt_pk_bf16(a - bf16_lo(hi), b - bf16_hi(hi));
}
// Four consecutive output elements from element e on, in the output's type.
__device__ __forceinline__ void store_out4(const GlobalArgs& a, size_t e, f32x4 v) {
  if (a.out_bf16)
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + e) =
        make_uint2(cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3]));
  else
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + e) = v;
}

// Logical coordinate of element e of k-step i of half hf, lane group g, in
// the pre-norm layout (block 2i + hf), or in the K=V layout.
template <bool PRE>
__device__ __forceinline__ int coord_of(int hf, int i, int g) {
  return PRE ? 64 * i + 32 * hf + 8 * g : kGSlice * hf + 32 * i + 8 * g;
}
// First coordinate of output tile t (16 coordinates) of half hf.
template <bool PRE>
__device__ __forceinline__ int tile_coord(int hf, int t) {
  return PRE ? 64 * (t >> 1) + 32 * hf + 16 * (t & 1) : kGSlice * hf + 16 * t;
}

// TRACE: the instance behind attn_decode_global_traced, which also writes a
// per-workgroup timeline entry; the production instances carry none of it.
template <bool PRE, bool TRACE = false>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(2))) void global_decode_kernel(GlobalArgs a) {
  __shared__ int s_pre[kGMaxBatch + 1];
  __shared__ int s_len[kGMaxBatch];
  __shared__ int s_vpre[kGMaxBatch + 1];
  __shared__ f32x4 s_part[2][kGWaves][kWave];  // partial S^T tiles (double-buffered)
  // V slices, one per wave; also the merge area at the end of a segment
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kGWaves][kGSlice * kPage];
  __shared__ float s_ml[4][2][kWave];           // m, l of the wave states being merged
  // Q^T B operands of the current segment: [half][k-step][lane], lane h + 16g
  // holding head h, coordinates 256*half + 32*kstep + 8g .. +8
  // (PRE: [half][k-step][hi, lo][lane]: q * w_k split into bf16 hi and lo on
  // unrotated k-steps, q twice on the rotated ones)
  constexpr int kQParts = PRE ? 2 : 1;
  __shared__ uint4 s_q[kGPair][kGKSteps][kQParts][kWave];
  __shared__ double s_g[PRE ? kPreActive : 1];      // theta^(-d/256) / (2 pi): revolutions per position
  __shared__ float s_ss[PRE ? 2 : 1][kGWaves][16];  // per-token sums of squares of each wave's half
  // The rotation by pos * omega_d, pos = 16 j + t, is the rotation by the
  // page's angle 16 j omega_d after the one by t omega_d. The second, with
  // w_k folded in, is a table over the 16 token offsets of a page: entry
  // [t][d] = (w0 c, w1 s, w1 c, w0 s), c = cos(2 pi t g_d), s = sin(..),
  // (w0, w1) = (w_k[d], w_k[d + 256]); rows padded by 16 bytes so that the
  // 16 tokens' reads of one d fall in different banks.
  __shared__ f32x4 s_rt[PRE ? kPage : 1][PRE ? kPreActive + 1 : 1];
  // cos and sin of the page angle of the wave's 32 frequencies
  __shared__ float s_base[PRE ? kGWaves : 1][PRE ? 64 : 1];

  if constexpr (PRE) {
    for (int i = threadIdx.x; i < kPage * kPreActive; i += blockDim.x) {
      const int t = i / kPreActive, d = i % kPreActive;
      const double g = pow(kPreTheta, -(double)d / 256.0) * 0.15915494309189535;  // 1 / (2 pi)
      if (t == 0) s_g[d] = g;
      double rev = (double)t * g;
      rev -= rint(rev);
      double sn, cs;
      sincos(rev * 6.283185307179586, &sn, &cs);
      const double w0 = a.w_k[d], w1 = a.w_k[d + 256];
      s_rt[t][d] = f32x4{(float)(w0 * cs), (float)(w1 * sn), (float)(w1 * cs), (float)(w0 * sn)};
    }
  }

  // timeline of this workgroup (start time, segments flushed), kept in LDS so
  // that no register stays live across the page walk for it
  __shared__ unsigned long long s_trace[TRACE ? 2 : 1];
  if (TRACE && threadIdx.x == 0) {
    s_trace[0] = __builtin_amdgcn_s_memrealtime();
    s_trace[1] = 0;
  }
  build_prefix(a, s_pre, s_len, s_vpre);
  const int N = rfl(s_pre[a.B]);
  const int w = blockIdx.x;
  if (w == 0 && a.ws_hdr != nullptr) {  // publish the table for the merge kernel
    for (int i = threadIdx.x; i <= a.B; i += blockDim.x) a.ws_hdr[i] = s_pre[i];
    for (int i = threadIdx.x; i < a.B; i += blockDim.x) a.ws_hdr[a.B + 1 + i] = s_len[i];
    for (int i = threadIdx.x; i <= a.B; i += blockDim.x) a.ws_hdr[2 * a.B + 1 + i] = s_vpre[i];
  }
  if (w == 0 && a.ws_hdr == nullptr) {  // no merge follows: rows of empty sequences are 0 here
    for (int i = threadIdx.x; i < a.B * (kGH * kGD / 4); i += blockDim.x)
      if (s_len[i / (kGH * kGD / 4)] == 0) store_out4(a, (size_t)4 * i, f32x4{0.f, 0.f, 0.f, 0.f});
  }

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = rfl(threadIdx.x / kWave);
  const int pr = wv >> 1;          // pair
  const int hf = wv & 1;           // coordinate half of this wave
  const int hq = lane & 15;        // head of this lane's S^T / O^T column
  const int g = lane >> 4;         // token quad of this lane (S^T rows 4g..4g+3)

  uint4 buf[kGBuf][kGKSteps];      // ring of this wave's page slices
  int idv[kGBuf];                  // physical page ids, 2 steps before their pages
  int iduse[kGBuf];                // the pair has a page in that step (else: zero page)
  f32x4 acc[kGMTiles];             // O^T: head hq, d = 256hf + 16t + 4g + e
  float m_run = -INFINITY, l_run = 0.f;
  const size_t lane_off = (size_t)hf * kGKSteps * 512 + (size_t)lane * 8;
  uint16_t* vs = s_v[wv];
  const int s16 = lane & 15;
  const int tr_tok = 4 * g + (s16 >> 2);
  const int tr_off = ((s16 & 3) >> 1) * 256 + tr_tok * 16 + (s16 & 1) * 8;  // + 512 t

  // Step descriptors (uniform): first page, pages (0: no step), sequence,
  // whether the step opens a segment, page index of the first page within its
  // sequence, and the sequence's length.
  int dP[kGDesc], dN[kGDesc], dB[kGDesc], dS[kGDesc], dJ[kGDesc], dL[kGDesc];

  // This workgroup's range [R0, R1); segment state.
  const int R0 = range_real(w, a.G, s_pre, s_vpre, a.B), R1 = range_real(w + 1, a.G, s_pre, s_vpre, a.B);
  int xb = 0;                      // s_part buffer of the next step
  bool seg_active = false;         // the pair states hold pages of segment seg_b
  int seg_b = 0, seg_first = 0, seg_end = 0;

  auto reset_state = [&]() __attribute__((always_inline)) {
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int t = 0; t < kGMTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // Stage the query rows of sequence b in s_q (after the last use of the
  // previous ones). Rare: waits for every outstanding load.
  auto load_q = [&](int b) __attribute__((always_inline)) {
    const int tid = opaque(threadIdx.x);
    uint4 t[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int u = 2 * tid + r;  // half, k-step, lane
      const int f = u / (kGKSteps * kWave), i = (u / kWave) % kGKSteps, l = u % kWave;
      t[r] = ld16(a.q + ((size_t)b * kGH + (l & 15)) * kGD + coord_of<PRE>(f, i, l >> 4));
    }
    wait_vmem_all();
    if constexpr (!PRE) {
#pragma unroll
      for (int r = 0; r < 2; ++r) (&s_q[0][0][0][0])[2 * tid + r] = t[r];
    } else {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int u = 2 * tid + r;
        const int f = u / (kGKSteps * kWave), i = (u / kWave) % kGKSteps, l = u % kWave;
        uint4 hi = t[r], lo = t[r];
        if (i % 4 != 0) {  // unrotated: q * w_k as hi + lo
          const int d0 = coord_of<true>(f, i, l >> 4);
          uint32_t ph[4], pl[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t qw = u4_get(t[r], e);
            const float v0 = bf16_lo(qw) * a.w_k[d0 + 2 * e], v1 = bf16_hi(qw) * a.w_k[d0 + 2 * e + 1];
            const __bf16 h0 = (__bf16)v0, h1 = (__bf16)v1;
            ph[e] = pack_bf16(h0, h1);
            pl[e] = pack_bf16((__bf16)(v0 - (float)h0), (__bf16)(v1 - (float)h1));
          }
          hi = make_uint4(ph[0], ph[1], ph[2], ph[3]);
          lo = make_uint4(pl[0], pl[1], pl[2], pl[3]);
        }
        s_q[f][i][0][l] = hi;
        s_q[f][i][1][l] = lo;
      }
    }
    __syncthreads();
  };

  // End-of-segment merge through LDS (the V regions are free by then): a
  // wave state is m (per head), l (lane partial) and its 16 accumulator tiles.
  f32x4* st = reinterpret_cast<f32x4*>(&s_v[0][0]);  // 4 states of [16][64] f32x4
  auto put_state = [&](int k, int ln) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kGMTiles; ++t) st[(k * kGMTiles + t) * kWave + ln] = acc[t];
    s_ml[k][0][ln] = m_run;
    s_ml[k][1][ln] = l_run;
  };
  auto take_state = [&](int k, int ln) __attribute__((always_inline)) {  // fold stored state k into this one
    const float m_o = s_ml[k][0][ln], l_o = s_ml[k][1][ln];
    const float M = fmaxf(m_run, m_o);
    const float fs = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - M);
    const float fo = (m_o == -INFINITY) ? 0.f : exp2_fast(m_o - M);
#pragma unroll
    for (int t = 0; t < kGMTiles; ++t) acc[t] = acc[t] * fs + st[(k * kGMTiles + t) * kWave + ln] * fo;
    l_run = l_run * fs + l_o * fo;
    m_run = M;
  };
  // Merge the 4 pair states (2 -> 0 and 3 -> 1, then 1 -> 0) and write the
  // segment [seg_first, seg_end) of sequence seg_b: the output row if it is
  // the whole sequence, else a partial slot of this workgroup (the first
  // segment of the range in slot 2w, the last in slot 2w + 1).
  auto flush = [&]() __attribute__((always_inline)) {
    const int ln = opaque(lane), lh = ln & 15, lg = ln >> 4;
    __syncthreads();  // every wave is done with its V region
    if (pr >= 2) put_state((pr - 2) * kGPair + hf, ln);
    __syncthreads();
    if (pr < 2) take_state(pr * kGPair + hf, ln);
    __syncthreads();
    if (pr == 1) put_state(hf, ln);
    __syncthreads();
    if (pr == 0) {
      take_state(hf, ln);
      float lt = l_run + xor16(l_run);
      lt += xor32(lt);
      const int pb = rfl(s_pre[seg_b]), pe = rfl(s_pre[seg_b + 1]);
      if (seg_first == pb && seg_end == pe) {  // whole sequence: o[b][h][d]
        const size_t row = ((size_t)seg_b * kGH + lh) * kGD + 4 * lg;
        const float inv = 1.f / lt;
#pragma unroll
        for (int t = 0; t < kGMTiles; ++t) {
          f32x4 o = acc[t] * inv;
          const int dt = tile_coord<PRE>(hf, t);
          if (a.gate) {  // sigmoidGate epilogue (set when no merge follows, or for bf16 output)
            const f32x4 gt = *reinterpret_cast<const f32x4*>(a.gate + row + dt);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] *= sigmoidf(gt[e]);
          }
          store_out4(a, row + dt, o);
        }
      } else {  // partial slot, lane order: 1 KB contiguous per store
        const int slot = 2 * w + (seg_first == R0 ? 0 : 1);
        float* ws = a.ws + (size_t)slot * kGSlotFloats;
        if (hf == 0 && lg == 0) {
          ws[kGH * kGD + lh] = m_run;
          ws[kGH * kGD + kGH + lh] = lt;
        }
#pragma unroll
        for (int t = 0; t < kGMTiles; ++t)
          *reinterpret_cast<f32x4*>(ws + ((size_t)(hf * kGMTiles + t) * kWave + ln) * 4) = acc[t];
      }
    }
    // (no wait for the stores or the page loads in flight: the loads land in
    // registers, and draining them here cost every segment change a pipeline
    // restart, 1.3% of the B = 64 call)
    __syncthreads();  // the merge area is page space again
    reset_state();
    seg_active = false;
    if (TRACE && threadIdx.x == 0) ++s_trace[1];
  };

  if (R0 < R1) {
    const int t_end = R1;
    int gp = R0, gb = seq_of_page(s_pre, a.B, R0);
    // first page, end page and length of sequence gb (read again only when
    // the generator moves to another sequence)
    int gpb = rfl(s_pre[gb]), gpe = rfl(s_pre[gb + 1]), gL = rfl(s_len[gb]);
    size_t last_idx = 0;

    // Next step descriptor into slot d: up to 4 pages of one sequence from
    // page gp on, or no step (0 pages) past the range's end.
    auto gen = [&](int d) __attribute__((always_inline)) {
      int n = 0, nw = 0;
      if (gp < t_end) {
        while (gpe <= gp) {  // next sequence with pages
          ++gb;
          gpb = gpe;
          gpe = rfl(s_pre[gb + 1]);
          gL = rfl(s_len[gb]);
        }
        n = min(kGPairs, min(gpe, t_end) - gp);
        nw = (gp == gpb || gp == R0) ? 1 : 0;
      }
      dP[d] = gp;
      dN[d] = n;
      dB[d] = gb;
      dS[d] = nw;
      dJ[d] = gp - gpb;
      dL[d] = gL;
      gp += n;
    };
    // This pair's page id of step d (a past-the-end step repeats the last id;
    // a pair without a page in the step then loads the zero page).
    auto load_id = [&](int is, int d) __attribute__((always_inline)) {
      if (dN[d] > 0) last_idx = (size_t)dB[d] * a.P_max + (size_t)(dJ[d] + min(pr, dN[d] - 1));
      iduse[is] = PRE || pr < dN[d];  // (the pre-norm kernel, short of registers, reloads instead)
      size_t idx = last_idx;
      // a vector load: a scalar one would be waited for by every LDS wait
      asm volatile("" : "+v"(idx));
      idv[is] = a.bt[idx];
    };
    auto issue = [&](int bs, int is) __attribute__((always_inline)) {
      const int phys = rfl(idv[is]);
      const uint16_t* src = (iduse[is] ? a.kv + (size_t)phys * kGPageElems
                                       : reinterpret_cast<const uint16_t*>(g_zero_page)) + lane_off;
#pragma unroll
      for (int i = 0; i < kGKSteps; ++i) buf[bs][i] = ld16_stream(src + (size_t)i * 512);
    };
    // One step from ring slot bs and descriptor d. Returns false for a step
    // past the range's end; the open segment is then flushed outside the
    // ring loop, where the ring's registers are free.
    auto compute = [&](int bs, int d) __attribute__((always_inline)) -> bool {
      const int P = dP[d], n = dN[d], b = dB[d];
      const int L = dL[d];
      const int j = dJ[d] + pr;  // this pair's page within sequence b
      f32x4 s2[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      if constexpr (!PRE) {
        // all LDS reads first, then the MFMAs (the scheduler would otherwise
        // pay the LDS latency once per MFMA)
        uint4 qv[kGKSteps];
#pragma unroll
        for (int i = 0; i < kGKSteps; ++i) qv[i] = s_q[hf][i][0][lane];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kGKSteps; ++i)
          s2[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, buf[bs][i]),
                                                              __builtin_bit_cast(bf16x8, qv[i]), s2[i & 1],
                                                              0, 0, 0);
      } else {
        // sum of squares of this wave's 256 coordinates of each token: the
        // diagonal of K K^T, on the MFMA units (a K row's A-operand registers
        // are also its B-operand layout as a column of K^T); element (t, t)
        // sits at lane t + 16 (t / 4), element t % 4
        f32x4 gram = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kGKSteps; ++i)
          gram = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, buf[bs][i]),
                                                         __builtin_bit_cast(bf16x8, buf[bs][i]), gram, 0, 0, 0);
        if (((lane & 15) >> 2) == g) {
          const int e = lane & 3;
          s_ss[xb][wv][lane & 15] = e == 0 ? gram[0] : (e == 1 ? gram[1] : (e == 2 ? gram[2] : gram[3]));
        }
        // RoPE of the pairs (d, d + 256), d = 32 hf + 8 g + e: elements e of
        // k-steps 0 and 4, at position 16 j + (lane & 15); rotated k as hi + lo.
        // The page angle of the wave's 32 frequencies: lane l gives the cos
        // (l < 32) or sin of frequency 32 hf + l % 32, in revolutions (fp64,
        // wrapped to [-1/2, 1/2]; v_sin/v_cos take revolutions).
        {
          double rev = (double)(j * kPage) * s_g[32 * hf + (lane & 31)];
          rev -= rint(rev);
          const float rf = (float)rev;
          s_base[wv][lane] = lane < 32 ? __builtin_amdgcn_cosf(rf) : __builtin_amdgcn_sinf(rf);
        }
        uint4 kr[2][2];  // [k-step 0 / 4][hi / lo]
        {
          const float* cb = &s_base[wv][8 * g];
          const float* sb = &s_base[wv][32 + 8 * g];
          const f32x4* tab = &s_rt[lane & 15][32 * hf + 8 * g];
          uint32_t k0h[4], k0l[4], k4h[4], k4l[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            float k0[2], k4[2];
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
              const int e = 2 * e2 + hb;
              const f32x4 r = tab[e];
              const uint32_t u0 = u4_get(buf[bs][0], e2), u4 = u4_get(buf[bs][4], e2);
              const float x0 = hb ? bf16_hi(u0) : bf16_lo(u0);
              const float x1 = hb ? bf16_hi(u4) : bf16_lo(u4);
              const float y0 = r.x * x0 - r.y * x1;  // R(t omega) (w (.) x)
              const float y1 = r.z * x1 + r.w * x0;
              k0[hb] = cb[e] * y0 - sb[e] * y1;       // then R(16 j omega)
              k4[hb] = cb[e] * y1 + sb[e] * y0;
            }
            split_bf16(k0[0], k0[1], k0h[e2], k0l[e2]);
            split_bf16(k4[0], k4[1], k4h[e2], k4l[e2]);
          }
          kr[0][0] = make_uint4(k0h[0], k0h[1], k0h[2], k0h[3]);
          kr[0][1] = make_uint4(k0l[0], k0l[1], k0l[2], k0l[3]);
          kr[1][0] = make_uint4(k4h[0], k4h[1], k4h[2], k4h[3]);
          kr[1][1] = make_uint4(k4l[0], k4l[1], k4l[2], k4l[3]);
        }
        // k-steps 0, 4: (k hi, q) + (k lo, q); others: (x, q w hi) + (x, q w lo)
#pragma unroll
        for (int i0 = 0; i0 < kGKSteps; i0 += 4) {
          uint4 qh[4], ql[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            qh[u] = s_q[hf][i0 + u][0][lane];
            ql[u] = s_q[hf][i0 + u][1][lane];
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint4 a1 = u == 0 ? kr[i0 / 4][0] : buf[bs][i0 + u];
            const uint4 a2 = u == 0 ? kr[i0 / 4][1] : buf[bs][i0 + u];
            s2[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1),
                                                            __builtin_bit_cast(bf16x8, qh[u]), s2[0], 0, 0, 0);
            s2[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a2),
                                                            __builtin_bit_cast(bf16x8, ql[u]), s2[1], 0, 0, 0);
          }
        }
      }
      s_part[xb][wv][lane] = s2[0] + s2[1];
#pragma unroll
      for (int i = 0; i < kGKSteps; ++i) *reinterpret_cast<uint4*>(vs + i * 512 + lane * 8) = buf[bs][i];
      const bool edge = pr < n && (j + 1) * kPage > L;  // rare: the sequence's last page
      if (edge && j * kPage + (lane & 15) >= L) {
        // zero the V row of this lane's token (weight 0; 0 * NaN would poison)
#pragma unroll
        for (int i = 0; i < kGKSteps; ++i)
          *reinterpret_cast<uint4*>(vs + i * 512 + lane * 8) = make_uint4(0u, 0u, 0u, 0u);
      }
      __syncthreads();
      const f32x4 s = s_part[xb][wv & ~1][lane] + s_part[xb][wv | 1][lane];
      float rr[4] = {1.f, 1.f, 1.f, 1.f};  // PRE: 1 / rms of tokens 4g .. 4g+3
      if constexpr (PRE) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sst = s_ss[xb][wv & ~1][4 * g + e] + s_ss[xb][wv | 1][4 * g + e];
          rr[e] = __builtin_amdgcn_rsqf(sst * (1.f / kGD) + kPreEps);
        }
      }
      xb ^= 1;
      if (n == 0) return false;  // past the end: the open segment is flushed after the loop
      if (!seg_active) {
        seg_active = true;
        seg_b = b;
        seg_first = P;
      }
      seg_end = P + n;
      if (pr < n) {
        float sc[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[e] = (PRE ? s[e] * rr[e] : s[e]) * kLog2e;
        if (edge) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j * kPage + 4 * g + e >= L) sc[e] = -INFINITY;
        }
        // Lazy rescaling: m_run is a reference, not the exact running max.
        // It moves (and the state is rescaled) only when a score exceeds it
        // by more than kGRescale (log2 units), so p = 2^(s - m_run) stays
        // below 2^kGRescale and no fp32 quantity can overflow; any reference
        // gives the same softmax since numerator and denominator share it.
        // The common case needs no cross-lane max. Always taken on a pair's
        // first page of a segment.
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
        // 8g+4..8g+7 the remainder bf16(p - bf16(p)); the V^T operand
        // repeats the same 4 tokens in both halves.
        // (PRE: the PV weight is p * r, since v = r * x; a masked token's r
        // may be NaN, so its weight is set, not multiplied)
        bf16x8 pp;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = exp2_fast(sc[e] - m_run);
          const float pw = PRE ? (sc[e] == -INFINITY ? 0.f : pv * rr[e]) : pv;
          pp[e] = (__bf16)pw;
          pp[4 + e] = (__bf16)(pw - (float)pp[e]);
          l_run += pv;
        }
        constexpr int kVB = DA_GLOBAL_VT_BATCH;  // transposed reads in flight per batch
#pragma unroll
        for (int t0 = 0; t0 < kGMTiles; t0 += kVB) {
          s16x4 v4[kVB];
#pragma unroll
          for (int u = 0; u < kVB; ++u)
            v4[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) char*)vs +
                                                           (t0 + u) * 512 + tr_off));
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < kVB; ++u) {
            const bf16x8 vt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v4[u], v4[u], 0, 1, 2, 3, 0, 1, 2, 3));
            acc[t0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pp, acc[t0 + u], 0, 0, 0);
          }
        }
      }
      const int dn = (d + 1) % kGDesc;
      if (dS[dn]) {  // the next step opens another segment: finish this one
        flush();
        load_q(dB[dn]);
      }
      return true;
    };

    // Prologue: descriptors 0..3, ids 0..3, pages of steps 0, 1.
#pragma unroll
    for (int d = 0; d < 4; ++d) gen(d);
    reset_state();
    load_q(dB[0]);
    load_id(0, 0);
    load_id(1, 1);
    load_id(2, 2);
    issue(0, 0);
    issue(1, 1);
    load_id(0, 3);
    // Step k = k0 + u: ring slot k % 3, descriptor k % 6. Every pass issues
    // the same loads; steps past the range's end reload its last page.
    for (;;) {
#pragma unroll
      for (int u = 0; u < kGDesc; ++u) {
        gen((u + 4) % kGDesc);
        load_id((u + 4) % kGBuf, (u + 4) % kGDesc);
        issue((u + 2) % kGBuf, (u + 2) % kGBuf);
        if (!compute(u % kGBuf, u)) goto range_done;
      }
    }
  range_done:
    wait_vmem_all();
    if (seg_active) flush();
  }
  if (TRACE && threadIdx.x == 0) {
    // timeline entry: start and end (100 MHz real-time counter), XCC id and
    // segments, pages and the hardware id of the first wave
    unsigned long long* t = a.trace + 4 * (size_t)w;
    t[0] = s_trace[0];
    t[1] = __builtin_amdgcn_s_memrealtime();
    t[2] = (unsigned long long)(__builtin_amdgcn_s_getreg(kHwRegXccId) & 0xF) | (s_trace[1] << 8);
    t[3] = (unsigned long long)(unsigned)(R1 - R0) | ((unsigned long long)__builtin_amdgcn_s_getreg(kHwRegHwId) << 32);
  }
}

// ---------------------------------------------------------------- fp32 cache
// decodeGQA over an fp32 K=V cache, tiled [pages][1][128][16][4]: chunk c
// (coordinates 4c .. 4c+3) of token t at floats (16 c + t) * 4 of the page.
// Same work split, workspace header, partial slots and merge as the bf16
// kernel; every product is fp32 (mfma_f32_16x16x4f32, fp32 weights), so the
// result is the exact softmax average up to fp32 rounding.
//
// 8 waves: a step takes up to 2 pages of one sequence, page slot pr = wv / 4,
// and the 4 waves of a page split its 512 coordinates, quarter qd = wv % 4
// owning [128 qd, 128 qd + 128): 8 KB of the 32 KB page, 8 lane-linear 1 KB
// loads. Load i puts chunk 32 qd + 4 i + l / 16 of token l % 16 in lane l.
//   S^T (16 tokens x 16 heads) partial over the wave's 128 coordinates, in
//     fp64: 32 x mfma_f64_16x16x4f64 on the fp32 values (exact products and
//     fp64 sums: at D = 512 the scores reach ~100, where fp32 spacing alone
//     moves a weight by several 1e-6). A = the loaded K (lane t + 16 j,
//     element e of load i: coordinate 128 qd + 16 i + 4 j + e, i.e. the k
//     index j of MFMA (i, e) stands for that coordinate), B = Q^T in the same
//     coordinate order from LDS. The 4 partials of a page are added through
//     LDS in a fixed order, in fp64.
//   The fp64 accumulator holds tokens g + 4e of head l % 16 (g = l / 16):
//     k-step s of the PV product takes tokens 4s .. 4s+3, token 4s + j in k
//     slot j, so its B operand P^T is element s of the lane's own weights,
//     unmoved.
//   O^T += V^T P^T in fp32: the wave's 8 KB of V go to LDS ([token][128
//     coordinates], 16-byte columns XOR-swizzled by the token) and come back
//     16 bytes per lane: token 4s + l / 16, coordinates 4 m .. 4 m + 3 with
//     m = 16 q + l % 16, the A operands of tiles 4q .. 4q+3 (tile 4q + e, row
//     r = coordinate 128 qd + 4 (16 q + r) + e). 8 tiles x 4 k-steps of
//     mfma_f32_16x16x4f32, whose accumulator rows are 4 (l / 16) + i.
// Steps, descriptors and loads run as in the bf16 kernel (page slices of
// steps k + 1 and k + 2 in flight).
constexpr int kFPages = 2;              // pages per step
constexpr int kFQuads = 4;              // waves per page (coordinate quarters)
constexpr int kFWaves = kFPages * kFQuads;
constexpr int kFThreads = kFWaves * kWave;
constexpr int kFSlice = kGD / kFQuads;  // coordinates per wave (128)
constexpr int kFLoads = kFSlice / 16;   // 1 KB loads per wave and page (8)
constexpr int kFTiles = kFSlice / 16;   // 16-coordinate output tiles per wave (8)
constexpr int kFPageFloats = kPage * kGD;
constexpr float kFRescale = 8.f;        // lazy-rescale threshold, log2 units
constexpr double kLog2e64 = 1.4426950408889634074;
typedef double f64x4 __attribute__((ext_vector_type(4)));
static_assert(kFThreads == kGThreads, "the prefix table is built by the same block size");

__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(2))) void global_decode_f32_kernel(
    GlobalArgs a) {
  __shared__ int s_pre[kGMaxBatch + 1];
  __shared__ int s_len[kGMaxBatch];
  __shared__ int s_vpre[kGMaxBatch + 1];
  __shared__ f64x4 s_part[2][kFWaves][kWave];  // partial S^T tiles, fp64 (double-buffered)
  // V of each wave's slice ([16 tokens][128 coordinates]); also the merge
  // area at the end of a segment
  __shared__ __attribute__((aligned(16))) float s_v[kFWaves][kPage * kFSlice];
  __shared__ float s_ml[kFQuads][2][kWave];  // m, l of the wave states being merged
  // Q^T B operands of the current segment: [quarter][load][lane], lane h + 16j
  // holding head h, coordinates 128 qd + 16 i + 4 j .. +4
  __shared__ uint4 s_q[kFQuads][kFLoads][kWave];

  const float* qf = reinterpret_cast<const float*>(a.q);
  const float* kvf = reinterpret_cast<const float*>(a.kv);

  build_prefix(a, s_pre, s_len, s_vpre);
  const int N = rfl(s_pre[a.B]);
  const int w = blockIdx.x;
  if (w == 0 && a.ws_hdr != nullptr) {  // publish the table for the merge kernel
    for (int i = threadIdx.x; i <= a.B; i += blockDim.x) a.ws_hdr[i] = s_pre[i];
    for (int i = threadIdx.x; i < a.B; i += blockDim.x) a.ws_hdr[a.B + 1 + i] = s_len[i];
    for (int i = threadIdx.x; i <= a.B; i += blockDim.x) a.ws_hdr[2 * a.B + 1 + i] = s_vpre[i];
  }
  if (w == 0 && a.ws_hdr == nullptr) {  // no merge follows: rows of empty sequences are 0 here
    for (int i = threadIdx.x; i < a.B * (kGH * kGD / 4); i += blockDim.x)
      if (s_len[i / (kGH * kGD / 4)] == 0) store_out4(a, (size_t)4 * i, f32x4{0.f, 0.f, 0.f, 0.f});
  }

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = rfl(threadIdx.x / kWave);
  const int pr = wv >> 2;    // page slot of a step
  const int qd = wv & 3;     // coordinate quarter of this wave
  const int g = lane >> 4;   // this lane's S^T rows: tokens g + 4e
  const int tk = lane & 15;  // token of this lane's loads; head of its S^T / O^T column

  uint4 buf[kGBuf][kFLoads];  // ring of this wave's page slices
  int idv[kGBuf];             // physical page ids, 2 steps before their pages
  int iduse[kGBuf];           // the page slot has a page in that step (else: zero page)
  f32x4 acc[kFTiles];         // O^T: head tk, coordinate 128 qd + 4 (16 (t / 4) + 4 g + e) + t % 4
  float m_run = -INFINITY, l_run = 0.f;
  const size_t qd_off = (size_t)qd * kFSlice * kPage;  // floats: the quarter's chunks
  float* vs = s_v[wv];
  // V staging: load i of lane l goes to row tk, 16-byte column (4 i + g) ^ tk
  // (the XOR keeps each column group of 16 and spreads a write's 16 lanes of
  // one column over all banks, as it does the reads' 16 columns of one row)
  const int vw_row = tk * kFSlice;

  int dP[kGDesc], dN[kGDesc], dB[kGDesc], dS[kGDesc], dJ[kGDesc], dL[kGDesc];
  const int R0 = range_real(w, a.G, s_pre, s_vpre, a.B), R1 = range_real(w + 1, a.G, s_pre, s_vpre, a.B);
  int xb = 0;
  bool seg_active = false;
  int seg_b = 0, seg_first = 0, seg_end = 0;

  auto reset_state = [&]() __attribute__((always_inline)) {
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int t = 0; t < kFTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // Stage the query rows of sequence b in s_q (after the last use of the
  // previous ones). Rare: waits for every outstanding load.
  auto load_q = [&](int b) __attribute__((always_inline)) {
    const int tid = opaque(threadIdx.x);
    uint4 t[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int u = 4 * tid + r;  // quarter, load, lane
      const int f = u / (kFLoads * kWave), i = (u / kWave) % kFLoads, l = u % kWave;
      t[r] = ld16(qf + ((size_t)b * kGH + (l & 15)) * kGD + kFSlice * f + 16 * i + 4 * (l >> 4));
    }
    wait_vmem_all();
#pragma unroll
    for (int r = 0; r < 4; ++r) (&s_q[0][0][0])[4 * tid + r] = t[r];
    __syncthreads();
  };

  f32x4* st = reinterpret_cast<f32x4*>(&s_v[0][0]);  // 4 states of [8][64] f32x4
  auto put_state = [&](int k, int ln) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kFTiles; ++t) st[(k * kFTiles + t) * kWave + ln] = acc[t];
    s_ml[k][0][ln] = m_run;
    s_ml[k][1][ln] = l_run;
  };
  auto take_state = [&](int k, int ln) __attribute__((always_inline)) {
    const float m_o = s_ml[k][0][ln], l_o = s_ml[k][1][ln];
    const float M = fmaxf(m_run, m_o);
    const float fs = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - M);
    const float fo = (m_o == -INFINITY) ? 0.f : exp2_fast(m_o - M);
#pragma unroll
    for (int t = 0; t < kFTiles; ++t) acc[t] = acc[t] * fs + st[(k * kFTiles + t) * kWave + ln] * fo;
    l_run = l_run * fs + l_o * fo;
    m_run = M;
  };
  // Merge the 2 page-slot states (1 -> 0) and write the segment: the output
  // row if it is the whole sequence, else a partial slot (the first segment of
  // the range in slot 2w, the last in slot 2w + 1), in the bf16 kernel's lane
  // order: coordinate d = 256 f + 16 T + 4 g' + e of head h at lane h + 16 g',
  // tile T, half f.
  auto flush = [&]() __attribute__((always_inline)) {
    const int ln = opaque(lane), lh = ln & 15, lg = ln >> 4;
    __syncthreads();  // every wave is done with its V region
    if (pr == 1) put_state(qd, ln);
    __syncthreads();
    if (pr == 0) {
      take_state(qd, ln);
      float lt = l_run + xor16(l_run);
      lt += xor32(lt);
      const int pb = rfl(s_pre[seg_b]), pe = rfl(s_pre[seg_b + 1]);
      if (seg_first == pb && seg_end == pe) {  // whole sequence: o[b][h][d]
        const size_t row = ((size_t)seg_b * kGH + lh) * kGD;
        const float inv = 1.f / lt;
#pragma unroll
        for (int q4 = 0; q4 < kFTiles / 4; ++q4)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int d = kFSlice * qd + 64 * q4 + 16 * lg + 4 * i;
            f32x4 o = f32x4{acc[4 * q4][i], acc[4 * q4 + 1][i], acc[4 * q4 + 2][i], acc[4 * q4 + 3][i]} * inv;
            if (a.gate) {  // sigmoidGate epilogue (set when no merge follows, or for bf16 output)
              const f32x4 gt = *reinterpret_cast<const f32x4*>(a.gate + row + d);
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] *= sigmoidf(gt[e]);
            }
            store_out4(a, row + d, o);
          }
      } else {
        const int slot = 2 * w + (seg_first == R0 ? 0 : 1);
        float* ws = a.ws + (size_t)slot * kGSlotFloats;
        if (qd == 0 && lg == 0) {
          ws[kGH * kGD + lh] = m_run;
          ws[kGH * kGD + kGH + lh] = lt;
        }
#pragma unroll
        for (int q4 = 0; q4 < kFTiles / 4; ++q4)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int T = 8 * (qd & 1) + 4 * q4 + lg;
            *reinterpret_cast<f32x4*>(ws + ((size_t)((qd >> 1) * kGMTiles + T) * kWave + lh + 16 * i) * 4) =
                f32x4{acc[4 * q4][i], acc[4 * q4 + 1][i], acc[4 * q4 + 2][i], acc[4 * q4 + 3][i]};
          }
      }
    }
    __syncthreads();  // the merge area is page space again (the page loads in flight stay so)
    reset_state();
    seg_active = false;
  };

  if (R0 < R1) {
    const int t_end = R1;
    int gp = R0, gb = seq_of_page(s_pre, a.B, R0);
    int gpb = rfl(s_pre[gb]), gpe = rfl(s_pre[gb + 1]), gL = rfl(s_len[gb]);
    size_t last_idx = 0;

    auto gen = [&](int d) __attribute__((always_inline)) {
      int n = 0, nw = 0;
      if (gp < t_end) {
        while (gpe <= gp) {  // next sequence with pages
          ++gb;
          gpb = gpe;
          gpe = rfl(s_pre[gb + 1]);
          gL = rfl(s_len[gb]);
        }
        n = min(kFPages, min(gpe, t_end) - gp);
        nw = (gp == gpb || gp == R0) ? 1 : 0;
      }
      dP[d] = gp;
      dN[d] = n;
      dB[d] = gb;
      dS[d] = nw;
      dJ[d] = gp - gpb;
      dL[d] = gL;
      gp += n;
    };
    auto load_id = [&](int is, int d) __attribute__((always_inline)) {
      if (dN[d] > 0) last_idx = (size_t)dB[d] * a.P_max + (size_t)(dJ[d] + min(pr, dN[d] - 1));
      iduse[is] = pr < dN[d];
      size_t idx = last_idx;
      asm volatile("" : "+v"(idx));  // a vector load (a scalar one would be waited for by every LDS wait)
      idv[is] = a.bt[idx];
    };
    auto issue = [&](int bs, int is) __attribute__((always_inline)) {
      const int phys = rfl(idv[is]);
      const float* src = (iduse[is] ? kvf + (size_t)phys * kFPageFloats + qd_off
                                    : reinterpret_cast<const float*>(g_zero_page)) + (size_t)lane * 4;
#pragma unroll
      for (int i = 0; i < kFLoads; ++i) buf[bs][i] = ld16_stream(src + (size_t)i * 256);
    };
    auto compute = [&](int bs, int d) __attribute__((always_inline)) -> bool {
      const int P = dP[d], n = dN[d], b = dB[d];
      const int L = dL[d];
      const int j = dJ[d] + pr;  // this page slot's page within sequence b
      f64x4 s2[2] = {f64x4{0.0, 0.0, 0.0, 0.0}, f64x4{0.0, 0.0, 0.0, 0.0}};
      {
        uint4 qv[kFLoads];
#pragma unroll
        for (int i = 0; i < kFLoads; ++i) qv[i] = s_q[qd][i][lane];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kFLoads; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s2[e & 1] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)__uint_as_float(u4_get(buf[bs][i], e)),
                                                             (double)__uint_as_float(u4_get(qv[i], e)), s2[e & 1],
                                                             0, 0, 0);
      }
      s_part[xb][wv][lane] = s2[0] + s2[1];
      const bool edge = pr < n && (j + 1) * kPage > L;  // rare: the sequence's last page
      const bool zero_row = edge && j * kPage + tk >= L;  // this lane's token is not visible
#pragma unroll
      for (int i = 0; i < kFLoads; ++i)
        *reinterpret_cast<uint4*>(vs + vw_row + (((4 * i + g) ^ tk) << 2)) =
            zero_row ? make_uint4(0u, 0u, 0u, 0u) : buf[bs][i];  // 0 * NaN would poison the sum
      __syncthreads();
      const f64x4 s = ((s_part[xb][4 * pr][lane] + s_part[xb][4 * pr + 1][lane]) + s_part[xb][4 * pr + 2][lane]) +
                      s_part[xb][4 * pr + 3][lane];
      xb ^= 1;
      if (n == 0) return false;  // past the end: the open segment is flushed after the loop
      if (!seg_active) {
        seg_active = true;
        seg_b = b;
        seg_first = P;
      }
      seg_end = P + n;
      if (pr < n) {
        double sn[4];  // scores of tokens g + 4e (natural units), -inf where not visible
#pragma unroll
        for (int e = 0; e < 4; ++e) sn[e] = s[e];
        if (edge) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j * kPage + g + 4 * e >= L) sn[e] = -INFINITY;
        }
        // Lazy rescaling as in the bf16 kernel, with a reference m_run (log2
        // units, an fp32 value) at most kFRescale below the scores; the
        // exponent s log2 e - m_run of a weight is formed in fp64 and rounded
        // once, to a number below kFRescale.
        const float lmax = (float)(fmax(fmax(sn[0], sn[1]), fmax(sn[2], sn[3])) * kLog2e64);
        if (__any(lmax > m_run + kFRescale)) {
          float mp = fmaxf(lmax, xor16(lmax));
          mp = fmaxf(mp, xor32(mp));
          const float m_new = (mp > m_run + kFRescale) ? mp : m_run;
          const float alpha = exp2_fast(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int t = 0; t < kFTiles; ++t) acc[t] *= alpha;
        }
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = exp2_fast((float)__builtin_fma(sn[e], kLog2e64, -(double)m_run));  // 0 where sn = -inf
          l_run += p[e];
        }
#pragma unroll
        for (int q4 = 0; q4 < kFTiles / 4; ++q4) {
          f32x4 v[4];
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) {
            const int T = 4 * s4 + g;
            v[s4] = *reinterpret_cast<const f32x4*>(vs + T * kFSlice + (((16 * q4 + tk) ^ T) << 2));
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[4 * q4 + e] = __builtin_amdgcn_mfma_f32_16x16x4f32(v[s4][e], p[s4], acc[4 * q4 + e], 0, 0, 0);
        }
      }
      const int dn = (d + 1) % kGDesc;
      if (dS[dn]) {  // the next step opens another segment: finish this one
        flush();
        load_q(dB[dn]);
      }
      return true;
    };

#pragma unroll
    for (int d = 0; d < 4; ++d) gen(d);
    reset_state();
    load_q(dB[0]);
    load_id(0, 0);
    load_id(1, 1);
    load_id(2, 2);
    issue(0, 0);
    issue(1, 1);
    load_id(0, 3);
    for (;;) {
#pragma unroll
      for (int u = 0; u < kGDesc; ++u) {
        gen((u + 4) % kGDesc);
        load_id((u + 4) % kGBuf, (u + 4) % kGDesc);
        issue((u + 2) % kGBuf, (u + 2) % kGBuf);
        if (!compute(u % kGBuf, u)) goto range_done;
      }
    }
  range_done:
    wait_vmem_all();
    if (seg_active) flush();
  }
}

// Log-sum-exp merge of the partial results of split sequences. Workgroup:
// (sequence b, output tile T = 16 coordinates of all 16 heads, i.e. one
// lane-order tile of a partial slot, or with LW = 16 a quarter of it: 4
// coordinates of the 16 heads, so that a few long sequences still spread
// over many workgroups); its NG groups of LW threads fold the sequence's
// pieces grp, grp+NG, ... with a running max, U pieces' loads in flight at a
// time, and are then combined the same way. The pieces are found from the
// page prefix table in the workspace header.
template <int NG, int U, int LW = kWave>
__global__ __launch_bounds__(LW * NG) void lse_merge_kernel(GlobalArgs a) {
  constexpr int kTiles = kGPair * kGMTiles;   // 32 tiles of 16 coordinates
  constexpr int kQ = kWave / LW;              // workgroups per tile
  __shared__ f32x4 s_num[NG][LW];
  __shared__ float s_m[NG][LW], s_den[NG][LW];
  const int bt = blockIdx.x / kQ;
  const int b = bt / kTiles;
  const int T = bt - b * kTiles;
  const int ln = threadIdx.x % LW;
  const int lane = (kQ == 1 ? 0 : (blockIdx.x % kQ) * LW) + ln;  // lane of the slot's tile
  const int grp = threadIdx.x / LW;
  const int h = lane & 15, g = lane >> 4;
  const int Tt = T % kGMTiles, Th = T / kGMTiles;  // tile, half
  const int d0 = (a.w_k ? 64 * (Tt >> 1) + 32 * Th + 16 * (Tt & 1) : kGSlice * Th + 16 * Tt) + 4 * g;
  const size_t ob = ((size_t)b * kGH + h) * kGD + d0;  // output element
  // sigmoidGate epilogue operands, loaded first so that their latency hides
  // behind the header reads: the gate, and (fp32 output) the row as the
  // decode kernel wrote it, used only if the sequence was not split (with
  // bf16 output the decode kernel gates such rows itself)
  f32x4 gt = {0.f, 0.f, 0.f, 0.f}, o1 = gt;
  if (a.gate && grp == 0) {
    gt = *reinterpret_cast<const f32x4*>(a.gate + ob);
    if (!a.out_bf16) o1 = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.out) + ob);
  }
  const int* pre = a.ws_hdr;
  const int L = pre[a.B + 1 + b];
  if (L == 0) {
    if (grp == 0) store_out4(a, ob, f32x4{0.f, 0.f, 0.f, 0.f});
    return;
  }
  const int* vpre = pre + 2 * a.B + 1;
  const int V = vpre[a.B];
  const int pb = pre[b], pe = pre[b + 1];
  const int vb = vpre[b];  // the sequence's weighted start; its first page at vb + kGSegPages
  // workgroup whose range holds weighted position v: the largest w with
  // floor(w V / G) <= v
  auto wg_of = [&](int v) __attribute__((always_inline)) {
    return div_floor_small(((long long)v + 1) * a.G - 1, V);
  };
  const int w0 = wg_of(vb + kGSegPages);
  const int np = wg_of(vb + kGSegPages + (pe - 1 - pb)) - w0 + 1;  // pieces
  if (np == 1) {  // finished inside one workgroup: the row is written
    if (a.gate && !a.out_bf16 && grp == 0) {  // in place: the decode kernel left the row ungated
#pragma unroll
      for (int e = 0; e < 4; ++e) o1[e] *= sigmoidf(gt[e]);
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + ob) = o1;
    }
    return;
  }
  // slot of piece i, or -1 for an empty range. With at least as many
  // weighted pages as workgroups every range is at least one weighted page
  // long, and a piece's range then holds pages of the sequence (the ranges
  // after w0 start past its first page); only the first piece needs its
  // range start: its workgroup began in the previous sequence unless its
  // weighted start lies at or after vb.
  const bool dense = V >= a.G;
  const int first_slot = 2 * w0 + (div_floor_small((long long)w0 * V, a.G) < vb ? 1 : 0);
  auto slot_of = [&](int i) __attribute__((always_inline)) -> int {
    const int ww = w0 + i;
    if (!dense && range_start(ww, V, a.G) == range_start(ww + 1, V, a.G)) return -1;  // empty range
    return i == 0 ? first_slot : 2 * ww;
  };
  const size_t off = ((size_t)T * kWave + lane) * 4;
  float m = -INFINITY, den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  for (int i = grp; i < np; i += U * NG) {
    float mi[U], li[U];
    f32x4 ai[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ii = i + u * NG;
      mi[u] = -INFINITY;
      li[u] = 0.f;
      ai[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (ii >= np) continue;
      const int sl = slot_of(ii);
      if (sl < 0) continue;
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
  s_num[grp][ln] = num;
  s_m[grp][ln] = m;
  s_den[grp][ln] = den;
  __syncthreads();
  if (grp == 0) {
    float M = s_m[0][ln];
#pragma unroll
    for (int gq = 1; gq < NG; ++gq) M = fmaxf(M, s_m[gq][ln]);
    f32x4 n = {0.f, 0.f, 0.f, 0.f};
    float dd = 0.f;
#pragma unroll
    for (int gq = 0; gq < NG; ++gq) {
      const float f = (s_m[gq][ln] == -INFINITY) ? 0.f : exp2_fast(s_m[gq][ln] - M);
      n += f * s_num[gq][ln];
      dd += f * s_den[gq][ln];
    }
    f32x4 o = n * (1.f / dd);
    if (a.gate) {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] *= sigmoidf(gt[e]);
    }
    store_out4(a, ob, o);
  }
}

// Device memory of the allocation-free global call: the header and the
// partial slots of at most kGScratchSplits workgroups (16.9 MB). Every device
// the library runs on holds its own copy until the process ends. In host code
// `scratch` names a host-side stand-in, never the device array: its device
// address comes from hipGetSymbolAddress, once per device, and only that
// address is passed to kernels.
constexpr int kGScratchSplits = 256;
constexpr size_t kGScratchBytes = kGHeaderBytes + (size_t)2 * kGScratchSplits * kGSlotFloats * sizeof(float);
static __device__ __align__(256) unsigned char scratch[kGScratchBytes];

namespace {
constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kScratchMaxDevices];
}  // namespace

da_status global_scratch(int dev, void** ptr, size_t* bytes, int* max_splits) {
  if (dev < 0 || dev >= kScratchMaxDevices) return DA_ERR_NO_DEVICE;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {  // first call on this device (it is current)
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return DA_ERR_LAUNCH;
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  *bytes = kGScratchBytes;
  *max_splits = kGScratchSplits;
  return DA_OK;
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
                        const int32_t* seq_lens, const float* gate, const float* w_k, void* out,
                        const da_shape& s, int num_splits, void* workspace, hipStream_t stream,
                        unsigned long long* trace) {
  GlobalArgs a;
  a.trace = trace;
  a.w_k = w_k;
  a.q = (const uint16_t*)q;
  a.kv = (const uint16_t*)kv_cache;
  a.bt = block_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.out_bf16 = s.out_dtype == DA_DTYPE_BF16 ? 1 : 0;
  // With a merge to follow, the merge applies the gate to every row: a gate
  // load in the decode kernel's flush would wait (in-order vmcnt) for all the
  // page loads it has in flight. With bf16 output the decode kernel gates
  // the rows it finishes itself (the merge would round them twice).
  a.gate = (num_splits > 1 && !a.out_bf16) ? nullptr : gate;
  a.ws_hdr = num_splits > 1 ? (int*)workspace : nullptr;
  a.ws = num_splits > 1 ? (float*)((char*)workspace + kGHeaderBytes) : nullptr;
  a.B = s.batch;
  a.P_max = s.max_pages_per_seq;
  a.G = num_splits;
  if (s.kv_dtype == DA_DTYPE_F32)
    hipLaunchKernelGGL(global_decode_f32_kernel, dim3((unsigned)num_splits), dim3(kFThreads), 0, stream, a);
  else if (w_k)
    hipLaunchKernelGGL(global_decode_kernel<true>, dim3((unsigned)num_splits), dim3(kGThreads), 0, stream, a);
  else if (trace)
    hipLaunchKernelGGL((global_decode_kernel<false, true>), dim3((unsigned)num_splits), dim3(kGThreads), 0, stream,
                       a);
  else
    hipLaunchKernelGGL(global_decode_kernel<false>, dim3((unsigned)num_splits), dim3(kGThreads), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return DA_ERR_LAUNCH;
  if (num_splits <= 1) return DA_OK;  // nothing was split: no merge
  a.gate = gate;
  // Expected pieces per sequence ~ G/B + 2: more pieces, more slot groups
  // and more loads in flight per thread, so that few rounds of dependent
  // loads remain (one for up to 16, 64 and 192 pieces).
  const int est = num_splits / s.batch + 2;
  const unsigned nb = (unsigned)s.batch * (kGPair * kGMTiles);
  // Beyond 16 pieces (few sequences, so few tiles) a workgroup takes a
  // quarter tile, four times as many workgroups sharing the reads. Up to 8,
  // two groups of 4 loads: at B = 64 (~6 pieces) 5.9-6.7 us against 7.4-7.9
  // for four groups (kernel trace).
  if (est <= 8)
    hipLaunchKernelGGL((lse_merge_kernel<2, 4>), dim3(nb), dim3(2 * kWave), 0, stream, a);
  else if (est <= 16)
    hipLaunchKernelGGL((lse_merge_kernel<4, 4>), dim3(nb), dim3(4 * kWave), 0, stream, a);
  else if (est <= 64)
    hipLaunchKernelGGL((lse_merge_kernel<16, 4, 16>), dim3(4 * nb), dim3(16 * 16), 0, stream, a);
  else
    hipLaunchKernelGGL((lse_merge_kernel<16, 12, 16>), dim3(4 * nb), dim3(16 * 16), 0, stream, a);
  return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

}  // namespace da
