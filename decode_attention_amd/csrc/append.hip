// Decode-step preparation of each sequence's new token: per-head RMSNorm
// (with the q or k weight; without weight for v), rotary embedding of q and
// k at the token's position, q written out and k (and v) stored in the
// token's slot of the paged caches.
//
// Pages: Op Specs of google/gemma-4-12B (Norm.lean: rmsnorm, rmsnormUnit;
// Rope.lean: invFreq, rope) and the gemma-4-12b Model Spec attn.qk_norm,
// attn.v_norm and attn.rope rows: eps 1e-6; sliding layers theta 10^4,
// rot = denom = 256, active 128; global layers theta 10^6, rot = denom = 512,
// active 64 (one 512-wide projection is both k and v there; the cache keeps
// k, which the decode reads as v as well).
//
// One wave per (sequence, row); the rows of a sequence are its Hq query
// heads, then its Hkv key heads, then (separate caches) its Hkv value heads.
// Lane l holds coordinates l + 64j, so a rotation pair (i, i + D/2) sits in
// one lane (j and j + D/128). Norms and rotations run in fp32; the angles
// pos * theta^(-2i/denom) are formed in fp64, since at positions near 2^18 an
// fp32 product would be off by up to ~0.02 rad.
#include "common.hpp"
#include "launch.hpp"

namespace da {

constexpr float kAppendEps = 1e-6f;
constexpr int kAppendWaves = 4;

struct AppendArgs {
  const float* q_raw;   // [B][Hq][D]
  const float* k_raw;   // [B][Hkv][D]
  const float* v_raw;   // [B][Hkv][D] (separate caches only)
  const float* w_q;     // [D]
  const float* w_k;     // [D]
  const int32_t* bt;    // [B][P_max]
  const int32_t* pos;   // [B]
  void* k_cache;        // sliding: [P][Hkv][16][D]; global: [P][Hkv][D/x][16][x]
  void* v_cache;        // sliding: [P][Hkv][16][D]
  void* q_out;          // [B][Hq][D], cache dtype
  int B, Hkv, G, P_max;
  double theta;
  int denom, active;
};

template <typename T>
__device__ __forceinline__ T store_cast(float x);
template <>
__device__ __forceinline__ float store_cast<float>(float x) { return x; }
template <>
__device__ __forceinline__ uint16_t store_cast<uint16_t>(float x) {  // round to nearest even
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Sum over the 64 lanes, the same total in every lane.
__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum16(x);
  x += xor16(x);
  x += xor32(x);
  return x;
}

// T: cache and q_out element type; D: head dim; SEP: separate k and v caches
// (row-major pages) rather than one K=V cache (tiled pages). PRE (global
// layers, bf16): the cache keeps the pre-norm projection x of each token,
// which the pre-norm decode normalises and rotates itself, so the k row is
// stored as it comes, in that cache's layout: coordinate d of block
// B = d / 32 goes to chunk 32 (B % 2) + 4 (B / 2) + (d / 8) % 4, element d % 8
// ([P][Hkv][64][16][8]).
template <typename T, int D, bool SEP, bool PRE = false>
__global__ __launch_bounds__(kAppendWaves * kWave) void kv_append_kernel(AppendArgs a) {
  static_assert(!PRE || (D == 512 && !SEP), "pre-norm cache: global layers");
  constexpr int J = D / kWave;       // coordinates per lane
  constexpr int JH = J / 2;          // pairs per lane
  constexpr int X = 16 / sizeof(T);  // elements per 16-byte chunk of a tiled page
  const int lane = threadIdx.x & (kWave - 1);
  const int Hq = a.Hkv * a.G;
  const int rows = Hq + (SEP ? 2 : 1) * a.Hkv;
  const long long task = (long long)blockIdx.x * kAppendWaves + threadIdx.x / kWave;
  if (task >= (long long)a.B * rows) return;  // no barrier in this kernel
  const int b = (int)(task / rows);
  const int r = (int)(task - (long long)b * rows);
  const int pos = a.pos[b];
  if (pos < 0 || pos >= a.P_max * kPage) return;  // documented: the row is left untouched

  const bool is_q = r < Hq, is_k = !is_q && r < Hq + a.Hkv;
  const int c = is_q ? r : (is_k ? r - Hq : r - Hq - a.Hkv);
  const float* src = is_q ? a.q_raw + ((size_t)b * Hq + c) * D
                          : (is_k ? a.k_raw : a.v_raw) + ((size_t)b * a.Hkv + c) * D;
  float y[J];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    y[j] = src[lane + kWave * j];
    ss = fmaf(y[j], y[j], ss);
  }
  const float inv = 1.f / sqrtf(wave_sum(ss) / (float)D + kAppendEps);
  const bool raw = PRE && is_k;  // stored as the pre-norm projection
  const float* w = is_q ? a.w_q : (is_k ? a.w_k : nullptr);
  if (!raw) {
#pragma unroll
    for (int j = 0; j < J; ++j) y[j] = y[j] * inv * (w ? w[lane + kWave * j] : 1.f);
  }

  if (is_q || (is_k && !raw)) {  // rotate pairs (i, i + D/2), i = lane + 64j
#pragma unroll
    for (int j = 0; j < JH; ++j) {
      const int i = lane + kWave * j;
      double s = 0.0, co = 1.0;
      if (i < a.active) sincos((double)pos * pow(a.theta, -2.0 * (double)i / (double)a.denom), &s, &co);
      const float cf = (float)co, sf = (float)s;
      const float lo = y[j], hi = y[j + JH];
      y[j] = lo * cf - hi * sf;
      y[j + JH] = hi * cf + lo * sf;
    }
  }

  if (is_q) {
    T* dst = reinterpret_cast<T*>(a.q_out) + ((size_t)b * Hq + c) * D;
#pragma unroll
    for (int j = 0; j < J; ++j) dst[lane + kWave * j] = store_cast<T>(y[j]);
    return;
  }
  const size_t page = (size_t)a.bt[(size_t)b * a.P_max + pos / kPage];
  const int slot = pos % kPage;
  T* cache = reinterpret_cast<T*>(is_k ? a.k_cache : a.v_cache);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int d = lane + kWave * j;
    size_t off;
    if constexpr (SEP)
      off = ((page * a.Hkv + c) * kPage + slot) * D + d;  // [P][Hkv][16][D]
    else if constexpr (PRE)
      off = (((page * a.Hkv + c) * (D / X) + 32 * ((d >> 5) & 1) + 4 * (d >> 6) + ((d >> 3) & 3)) * kPage + slot) * X +
            (d & 7);  // [P][Hkv][64][16][8], pre-norm chunk order
    else
      off = (((page * a.Hkv + c) * (D / X) + d / X) * kPage + slot) * X + d % X;  // [P][Hkv][D/X][16][X]
    cache[off] = store_cast<T>(y[j]);
  }
}

static da_status run_append(const AppendArgs& a, int D, bool sep, int kv_dtype, hipStream_t stream) {
  const int rows = a.Hkv * a.G + (sep ? 2 : 1) * a.Hkv;
  const long long tasks = (long long)a.B * rows;
  const dim3 grid((unsigned)((tasks + kAppendWaves - 1) / kAppendWaves)), block(kAppendWaves * kWave);
  if (D == 256 && sep) {
    if (kv_dtype == DA_DTYPE_BF16)
      hipLaunchKernelGGL((kv_append_kernel<uint16_t, 256, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((kv_append_kernel<float, 256, true>), grid, block, 0, stream, a);
  } else if (D == 512 && !sep) {
    if (kv_dtype == DA_DTYPE_BF16)
      hipLaunchKernelGGL((kv_append_kernel<uint16_t, 512, false>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((kv_append_kernel<float, 512, false>), grid, block, 0, stream, a);
  } else {
    return DA_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

da_status launch_append_sliding(const float* q_raw, const float* k_raw, const float* v_raw, const float* w_q,
                                const float* w_k, const int32_t* block_table, const int32_t* positions,
                                void* k_cache, void* v_cache, void* q_out, const da_shape& s, hipStream_t stream) {
  AppendArgs a = {q_raw, k_raw, v_raw, w_q, w_k, block_table, positions, k_cache, v_cache, q_out,
                  s.batch, s.num_kv_heads, s.group, s.max_pages_per_seq, 10000.0, 256, 128};
  return run_append(a, s.head_dim, true, s.kv_dtype, stream);
}

da_status launch_append_global_prenorm(const float* q_raw, const float* x_raw, const float* w_q,
                                       const int32_t* block_table, const int32_t* positions, void* x_cache,
                                       void* q_out, const da_shape& s, hipStream_t stream) {
  if (s.head_dim != 512 || s.kv_dtype != DA_DTYPE_BF16) return DA_ERR_UNSUPPORTED;
  const AppendArgs a = {q_raw, x_raw, nullptr, w_q, nullptr, block_table, positions, x_cache, nullptr, q_out,
                        s.batch, s.num_kv_heads, s.group, s.max_pages_per_seq, 1000000.0, 512, 64};
  const long long tasks = (long long)a.B * (a.Hkv * a.G + a.Hkv);
  const dim3 grid((unsigned)((tasks + kAppendWaves - 1) / kAppendWaves)), block(kAppendWaves * kWave);
  hipLaunchKernelGGL((kv_append_kernel<uint16_t, 512, false, true>), grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

da_status launch_append_global(const float* q_raw, const float* kv_raw, const float* w_q, const float* w_k,
                               const int32_t* block_table, const int32_t* positions, void* kv_cache, void* q_out,
                               const da_shape& s, hipStream_t stream) {
  AppendArgs a = {q_raw, kv_raw, nullptr, w_q, w_k, block_table, positions, kv_cache, nullptr, q_out,
                  s.batch, s.num_kv_heads, s.group, s.max_pages_per_seq, 1000000.0, 512, 64};
  return run_append(a, s.head_dim, false, s.kv_dtype, stream);
}

}  // namespace da
