// slidingDecodeGQA over row-major paged k/v caches ([pages][Hkv][16][D]).
//
// Pages: Op Specs of google/gemma-4-12B (Attention.lean: softmax, slidingGQA,
// decodeGQA) and the op-specs NOTE that names the sliding decode node; the
// gemma-4-12b Model Spec attn.core row for the sliding layers (scale 1,
// window 1024, 16 query heads on 8 KV heads, D = 256).
//
// One workgroup per (sequence b, KV head c); its NW waves take the window's
// pages round-robin, each with its own online-softmax state, and merge in LDS
// at the end. Group size G = 2, so QK^T is a 2 x D by D x 16 product per page:
// too thin for MFMA, done on the VALU with bf16 dot2.
//
// Lane mapping (per page slab of 16 tokens x D for one KV head, contiguous):
//   load instruction i, lane l reads 16-byte chunk 64*i + l of the slab, i.e.
//   token i*TPI + l/CPR, coordinates [E*(l%CPR), E*(l%CPR)+E), where E is the
//   number of elements per chunk (8 bf16 or 4 fp32), CPR = D/E chunks per row
//   and TPI = 64/CPR tokens per instruction. Each wave instruction covers 1 KB
//   of contiguous memory, and the loaded registers are already in the layout
//   the dot products need: no LDS staging.
//   QK partial sums are reduced over the lanes of one token: a permlane16
//   swap folds lane bit 4 while splitting the two heads between even and odd
//   16-lane rows, then a 4-step xor butterfly folds lane bits 0..3 (and a
//   permlane32 swap folds bit 5 when a token spans the whole wave, fp32).
#include "common.hpp"
#include "launch.hpp"

namespace da {

template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {  // bf16 bit patterns
  static constexpr int E = 8;
};
template <>
struct Elem<float> {
  static constexpr int E = 4;
};

// fp32 values of the 16-byte chunk `u` (E elements).
template <typename T>
__device__ __forceinline__ void chunk_to_f32(const uint4& u, float* f);
template <>
__device__ __forceinline__ void chunk_to_f32<uint16_t>(const uint4& u, float* f) {
  f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
  f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z);
  f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}
template <>
__device__ __forceinline__ void chunk_to_f32<float>(const uint4& u, float* f) {
  f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
  f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
}

// <q chunk, k chunk> partial dot product, fp32 accumulate.
template <typename T>
__device__ __forceinline__ float chunk_dot(const uint4& qv, const uint4& kv);
template <>
__device__ __forceinline__ float chunk_dot<uint16_t>(const uint4& qv, const uint4& kv) {
  float s = dot2_bf16(qv.x, kv.x, 0.f);
  s = dot2_bf16(qv.y, kv.y, s);
  s = dot2_bf16(qv.z, kv.z, s);
  return dot2_bf16(qv.w, kv.w, s);
}
template <>
__device__ __forceinline__ float chunk_dot<float>(const uint4& qv, const uint4& kv) {
  float s = __uint_as_float(qv.x) * __uint_as_float(kv.x);
  s = fmaf(__uint_as_float(qv.y), __uint_as_float(kv.y), s);
  s = fmaf(__uint_as_float(qv.z), __uint_as_float(kv.z), s);
  return fmaf(__uint_as_float(qv.w), __uint_as_float(kv.w), s);
}

// fp32 caches: the same dot product in fp64 (exact products of the fp32
// values, fp64 sums), so that the scores carry no fp32 rounding into the
// weights (see the kernel).
__device__ __forceinline__ double chunk_dot_f64(const uint4& qv, const uint4& kv) {
  double s = (double)__uint_as_float(qv.x) * (double)__uint_as_float(kv.x);
  s = __builtin_fma((double)__uint_as_float(qv.y), (double)__uint_as_float(kv.y), s);
  s = __builtin_fma((double)__uint_as_float(qv.z), (double)__uint_as_float(kv.z), s);
  return __builtin_fma((double)__uint_as_float(qv.w), (double)__uint_as_float(kv.w), s);
}
constexpr double kSlLog2e64 = 1.4426950408889634074;

template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * kWave) void sliding_decode_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int window,
    const float* __restrict__ gate, void* __restrict__ out, int out_bf16, int Hkv, int P_max) {
  constexpr int G = 2;
  constexpr int E = Elem<T>::E;
  constexpr int CPR = D / E;
  constexpr int TPI = kWave / CPR;
  constexpr int NI = kPage / TPI;
  static_assert(CPR == 32 || CPR == 64, "one token row must span half or all of the wave");

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int b = blockIdx.x / Hkv;
  const int c = blockIdx.x - b * Hkv;
  const int dc = lane % CPR;   // coordinate chunk of this lane
  const int tt = lane / CPR;   // token offset inside a load instruction

  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];
  __shared__ float s_acc[NW][G][D];

  // Lengths beyond the block-table row are clamped so no read leaves it.
  const int L = min(seq_lens[b], P_max * kPage);
  // output rows of (b, c), fp32 or (out_bf16) bf16 rounded to nearest even
  const size_t ob = ((size_t)b * Hkv * G + (size_t)c * G) * D;
  auto store = [&](int i, float v) __attribute__((always_inline)) {
    if (out_bf16)
      reinterpret_cast<__bf16*>(out)[ob + i] = (__bf16)v;
    else
      reinterpret_cast<float*>(out)[ob + i] = v;
  };
  const float* gb = gate ? gate + ((size_t)b * Hkv * G + (size_t)c * G) * D : nullptr;
  if (L <= 0 || window <= 0) {  // no visible key: the output rows are 0
    for (int i = threadIdx.x; i < G * D; i += NW * kWave) store(i, 0.f);
    return;
  }
  const int lo = L > window ? L - window : 0;  // first visible position
  const int j_lo = lo / kPage;
  const int npages = (L - 1) / kPage - j_lo + 1;
  const int nmine = npages > wv ? (npages - wv + NW - 1) / NW : 0;

  const T* qb = q + ((size_t)b * Hkv * G + (size_t)c * G) * D + dc * E;
  const uint4 q0 = ld16(qb), q1 = ld16(qb + D);

  float m_run = -INFINITY;  // running max (log2 domain) of head hl
  float l_run = 0.f;        // running sum of head hl over this lane's tokens
  float acc0[E], acc1[E];   // unnormalised output, heads 0 and 1
#pragma unroll
  for (int e = 0; e < E; ++e) acc0[e] = acc1[e] = 0.f;

  const int32_t* btb = block_table + (size_t)b * P_max;
  const size_t slab = (size_t)kPage * D;
  const size_t lane_off = (size_t)lane * E;

  // Physical ids of this wave's pages, 64 at a time: lane i holds the id of
  // page k0 + i, so no block-table load sits on the path of a page load.
  int ids = 0;
  uint4 kb[2][NI], vb[2][NI];
  // kk: page index inside the current chunk; a slot the loop will not
  // compute (use = false) loads the zero page instead.
  auto load = [&](int buf, int kk, bool use) {
    const int phys = __builtin_amdgcn_readlane(ids, kk);
    const size_t base = ((size_t)phys * Hkv + c) * slab;
    const T* kp = (use ? kc + base : reinterpret_cast<const T*>(g_zero_page)) + lane_off;
    const T* vp = (use ? vc + base : reinterpret_cast<const T*>(g_zero_page)) + lane_off;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      kb[buf][i] = ld16_stream(kp + (size_t)i * kWave * E);
      vb[buf][i] = ld16_stream(vp + (size_t)i * kWave * E);
    }
  };

  auto compute = [&](int buf, int k) {
    const int t0 = (j_lo + wv + NW * k) * kPage;
    const bool edge = (t0 < lo) || (t0 + kPage > L);
    // scores of this lane's head (even 16-lane rows: head 0, odd: head 1):
    // bf16, fp32 in log2 units; fp32 caches, fp64 in natural units (at
    // D = 256 fp32 sums alone move the scores by up to ~1e-5 relative to
    // the weights' tolerance)
    constexpr bool kF64 = sizeof(T) == 4;
    float s[kF64 ? 1 : NI];
    double sd[kF64 ? NI : 1];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (kF64) {
        // a token spans the wave: fixed xor butterfly over all 64 lanes, in
        // fp64 (commutative steps: every lane ends with the same sums)
        double t0 = chunk_dot_f64(q0, kb[buf][i]), t1 = chunk_dot_f64(q1, kb[buf][i]);
#pragma unroll
        for (int off = kWave / 2; off >= 1; off >>= 1) {
          t0 += __shfl_xor(t0, off);
          t1 += __shfl_xor(t1, off);
        }
        sd[i] = ((lane >> 4) & 1) ? t1 : t0;
      } else {
        const float p0 = chunk_dot<T>(q0, kb[buf][i]);
        const float p1 = chunk_dot<T>(q1, kb[buf][i]);
        const f2 r = swap16(p0, p1);  // even rows: head 0, odd rows: head 1
        float u = row_sum16(r.a + r.b);
        if constexpr (TPI == 1) {
          const f2 h = swap32(u, u);
          u = h.a + h.b;
        }
        s[i] = u * kLog2e;
      }
    }
    if (edge) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int pos = t0 + i * TPI + tt;
        if (pos < lo || pos >= L) {
          if constexpr (kF64)
            sd[i] = -INFINITY;
          else
            s[i] = -INFINITY;
          vb[buf][i] = make_uint4(0u, 0u, 0u, 0u);  // 0 * NaN would poison the sum
        }
      }
    }
    float mp;
    if constexpr (kF64) {
      double md = sd[0];
#pragma unroll
      for (int i = 1; i < NI; ++i) md = fmax(md, sd[i]);
      mp = (float)(md * kSlLog2e64);
    } else {
      mp = s[0];
#pragma unroll
      for (int i = 1; i < NI; ++i) mp = fmaxf(mp, s[i]);
    }
    if constexpr (TPI == 2) mp = fmaxf(mp, xor32(mp));
    const float m_new = fmaxf(m_run, mp);  // finite: every page has a visible key
    const float alpha = exp2_fast(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
    const f2 al = swap16(alpha, alpha);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      acc0[e] *= al.a;
      acc1[e] *= al.b;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      // (fp32 caches: the exponent s log2 e - m formed in fp64, rounded once)
      const float p = kF64 ? exp2_fast((float)__builtin_fma(sd[kF64 ? i : 0], kSlLog2e64, -(double)m_new))
                           : exp2_fast(s[kF64 ? 0 : i] - m_new);
      l_run += p;
      const f2 pp = swap16(p, p);  // .a head 0, .b head 1, same token
      float v[E];
      chunk_to_f32<T>(vb[buf][i], v);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        acc0[e] = fmaf(pp.a, v[e], acc0[e]);
        acc1[e] = fmaf(pp.b, v[e], acc1[e]);
      }
    }
  };

  // Software pipeline: the next page's 16 loads are always issued before the
  // current page is computed (past the chunk's end from the zero page, so
  // every pass issues the same loads and the compiler can count them).
  for (int k0 = 0; k0 < nmine; k0 += kWave) {
    const int kn = min(nmine - k0, kWave);
    ids = (k0 + lane < nmine) ? btb[j_lo + wv + NW * (k0 + lane)] : 0;
    wait_vmem_all();
    load(0, 0, true);
    for (int k = 0; k < kn; k += 2) {
      load(1, min(k + 1, kn - 1), k + 1 < kn);
      compute(0, k0 + k);
      if (k + 1 >= kn) break;
      load(0, min(k + 2, kn - 1), k + 2 < kn);
      compute(1, k0 + k + 1);
    }
  }

  // Fold the token halves (bf16: lanes l and l^32 saw different tokens).
  float l_tot = l_run;
  if constexpr (TPI == 2) {
    l_tot += xor32(l_run);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      acc0[e] += xor32(acc0[e]);
      acc1[e] += xor32(acc1[e]);
    }
  }
  const f2 mm = swap16(m_run, m_run);
  const f2 ll = swap16(l_tot, l_tot);
  if (lane == 0) {
    s_m[wv][0] = mm.a; s_m[wv][1] = mm.b;
    s_l[wv][0] = ll.a; s_l[wv][1] = ll.b;
  }
  if (tt == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      s_acc[wv][0][dc * E + e] = acc0[e];
      s_acc[wv][1][dc * E + e] = acc1[e];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += NW * kWave) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = s_m[w][h];
      const float f = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
      num = fmaf(f, s_acc[w][h][d], num);
      den = fmaf(f, s_l[w][h], den);
    }
    const float o = num / den;
    store(idx, gb ? o * sigmoidf(gb[idx]) : o);  // sigmoidGate epilogue
  }
}

constexpr int kSlidingWaves = 4;  // default waves per (sequence, KV head)

template <typename T, int NW>
static void launch_sliding_nw(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, int32_t window, const float* gate, void* out, int out_bf16,
                              const da_shape& s, hipStream_t stream) {
  hipLaunchKernelGGL((sliding_decode_kernel<T, 256, NW>), dim3((unsigned)s.batch * (unsigned)s.num_kv_heads),
                     dim3(NW * kWave), 0, stream, (const T*)q, (const T*)k_cache, (const T*)v_cache, block_table,
                     seq_lens, window, gate, out, out_bf16, s.num_kv_heads, s.max_pages_per_seq);
}

template <typename T>
static void launch_sliding_t(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                             const int32_t* seq_lens, int32_t window, const float* gate, void* out, int out_bf16,
                             const da_shape& s, hipStream_t stream) {
  // s.num_splits: waves a unit's window is divided among (0: the default);
  // the API has admitted only 0, 1, 2, 4 and 8 (8 with bf16 caches only)
  switch (s.num_splits == 0 ? kSlidingWaves : s.num_splits) {
    case 1: launch_sliding_nw<T, 1>(q, k_cache, v_cache, block_table, seq_lens, window, gate, out, out_bf16, s,
                                    stream); break;
    case 2: launch_sliding_nw<T, 2>(q, k_cache, v_cache, block_table, seq_lens, window, gate, out, out_bf16, s,
                                    stream); break;
    case 8:  // bf16 only: the fp32 kernel's registers exceed 2 waves per SIMD
      if constexpr (sizeof(T) == 2)
        launch_sliding_nw<T, 8>(q, k_cache, v_cache, block_table, seq_lens, window, gate, out, out_bf16, s, stream);
      break;
    default: launch_sliding_nw<T, 4>(q, k_cache, v_cache, block_table, seq_lens, window, gate, out, out_bf16, s,
                                     stream); break;
  }
}

da_status launch_sliding(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, const int32_t* seq_lens, int32_t window, const float* gate,
                         void* out, const da_shape& s, hipStream_t stream) {
  const int out_bf16 = s.out_dtype == DA_DTYPE_BF16 ? 1 : 0;
  if (s.kv_dtype == DA_DTYPE_BF16)
    launch_sliding_t<uint16_t>(q, k_cache, v_cache, block_table, seq_lens, window, gate, out, out_bf16, s, stream);
  else
    launch_sliding_t<float>(q, k_cache, v_cache, block_table, seq_lens, window, gate, out, out_bf16, s, stream);
  return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

}  // namespace da
