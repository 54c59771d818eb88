// Memory-bound kernels of the hot path: modulated RMSNorm (optionally fused with the per-row
// int8 quantisation of its output), per-row int8 quantisation of activations, token merge /
// unmerge, the Euler update, assembly of the DiT input, weight packing (bf16 / f32 permutation
// and int8 quantisation), the 3D RoPE table and a plain copy. All read 16 bytes per lane per
// access.
#include <math.h>

#include "launch.h"

namespace h3x {
namespace {

constexpr int kThreads = 256;

template <class E> struct Vec;
template <> struct Vec<F32> { static constexpr int n = 4; };
template <> struct Vec<BF16> { static constexpr int n = 8; };

// Load / store n consecutive elements (16 bytes) as floats; unpack16 is load16 on a chunk
// already in registers.
template <class E>
__device__ __forceinline__ void unpack16(const uint4 raw, float* out) {
  if constexpr (sizeof(typename E::T) == 4) {
    out[0] = __uint_as_float(raw.x); out[1] = __uint_as_float(raw.y);
    out[2] = __uint_as_float(raw.z); out[3] = __uint_as_float(raw.w);
  } else {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}
template <class E>
__device__ __forceinline__ void load16(const typename E::T* p, float* out) {
  unpack16<E>(*reinterpret_cast<const uint4*>(p), out);
}
template <class E>
__device__ __forceinline__ void store16(typename E::T* p, const float* v) {
  uint4 raw;
  if constexpr (sizeof(typename E::T) == 4) {
    raw.x = __float_as_uint(v[0]); raw.y = __float_as_uint(v[1]);
    raw.z = __float_as_uint(v[2]); raw.w = __float_as_uint(v[3]);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16_bits(v[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16_bits(v[2 * i + 1])) << 16);
    raw = make_uint4(w[0], w[1], w[2], w[3]);
  }
  *reinterpret_cast<uint4*>(p) = raw;
}

// ---------------------------------------------------------------- modulated RMSNorm
// One workgroup per row: sum of squares in float32 (wave reduction, then across the four
// waves through LDS), then y = x * rsqrt(ms + eps) * (1 + scale) + shift.
template <class E>
__global__ __launch_bounds__(kThreads) void norm_mod_kernel(const typename E::T* __restrict__ x,
                                                            const float* __restrict__ shift,
                                                            const float* __restrict__ scale,
                                                            typename E::T* __restrict__ y,
                                                            int d, float eps, int out_tiled) {
  constexpr int V = Vec<E>::n;
  __shared__ float part[kThreads / 64];
  const int64_t row = blockIdx.x;
  const typename E::T* xr = x + row * d;
  typename E::T* yr = y + row * d;
  float ss = 0.f;
  for (int i = threadIdx.x * V; i < d; i += kThreads * V) {
    float v[V];
    load16<E>(xr + i, v);
#pragma unroll
    for (int j = 0; j < V; ++j) ss = fmaf(v[j], v[j], ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) tot += part[w];
  const float r = 1.0f / sqrtf(tot / static_cast<float>(d) + eps);
  for (int i = threadIdx.x * V; i < d; i += kThreads * V) {
    float v[V];
    load16<E>(xr + i, v);
    const float4* sc4 = reinterpret_cast<const float4*>(scale + i);
    const float4* sh4 = reinterpret_cast<const float4*>(shift + i);
#pragma unroll
    for (int j = 0; j < V / 4; ++j) {
      const float4 sc = sc4[j], sh = sh4[j];
      v[4 * j + 0] = fmaf(v[4 * j + 0] * r, 1.f + sc.x, sh.x);
      v[4 * j + 1] = fmaf(v[4 * j + 1] * r, 1.f + sc.y, sh.y);
      v[4 * j + 2] = fmaf(v[4 * j + 2] * r, 1.f + sc.z, sh.z);
      v[4 * j + 3] = fmaf(v[4 * j + 3] * r, 1.f + sc.w, sh.w);
    }
    if (out_tiled)  // bf16 only: 256-row x 32-column slabs (see slab_offset)
      store16<E>(reinterpret_cast<typename E::T*>(reinterpret_cast<uint8_t*>(y) + slab_offset(row, i, d)), v);
    else
      store16<E>(yr + i, v);
  }
}

// kRows rows per workgroup with the rows held in registers as loaded (each row read once; 16
// bytes per chunk, so bfloat16 rows take half the registers of float32 values and more
// workgroups stay resident) and shift / scale loaded once for all kRows rows; kChunks 16-byte
// chunks per thread and row cover d <= kChunks * 256 * V. Same arithmetic, in the same order,
// as norm_mod_kernel.
template <class E, int kChunks, int kRows>
__global__ __launch_bounds__(kThreads) void norm_rows_kernel(const typename E::T* __restrict__ x,
                                                             const float* __restrict__ shift,
                                                             const float* __restrict__ scale,
                                                             typename E::T* __restrict__ y,
                                                             int64_t n_rows, int d, float eps,
                                                             int out_tiled) {
  constexpr int V = Vec<E>::n;
  __shared__ float part[kRows][kThreads / 64];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kRows;
  uint4 raw[kRows][kChunks];
  float ss[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    ss[r] = 0.f;
    const int64_t row = r0 + r;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int i = (c * kThreads + threadIdx.x) * V;
      raw[r][c] = make_uint4(0u, 0u, 0u, 0u);
      if (row < n_rows && i < d) {
        raw[r][c] = *reinterpret_cast<const uint4*>(x + row * d + i);
        float v[V];
        unpack16<E>(raw[r][c], v);
#pragma unroll
        for (int j = 0; j < V; ++j) ss[r] = fmaf(v[j], v[j], ss[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    ss[r] = wave_sum(ss[r]);
    if ((threadIdx.x & 63) == 0) part[r][threadIdx.x >> 6] = ss[r];
  }
  __syncthreads();
  float rs[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) tot += part[r][w];
    rs[r] = 1.0f / sqrtf(tot / static_cast<float>(d) + eps);
  }
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int i = (c * kThreads + threadIdx.x) * V;
    if (i >= d) continue;
    float sc[V], sh[V];
#pragma unroll
    for (int j = 0; j < V / 4; ++j) {
      const float4 a = reinterpret_cast<const float4*>(scale + i)[j];
      const float4 b = reinterpret_cast<const float4*>(shift + i)[j];
      sc[4 * j] = 1.f + a.x; sc[4 * j + 1] = 1.f + a.y; sc[4 * j + 2] = 1.f + a.z; sc[4 * j + 3] = 1.f + a.w;
      sh[4 * j] = b.x; sh[4 * j + 1] = b.y; sh[4 * j + 2] = b.z; sh[4 * j + 3] = b.w;
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int64_t row = r0 + r;
      if (row >= n_rows) continue;
      float v[V], o[V];
      unpack16<E>(raw[r][c], v);
#pragma unroll
      for (int j = 0; j < V; ++j) o[j] = fmaf(v[j] * rs[r], sc[j], sh[j]);
      if (out_tiled)  // bf16 only: 256-row x 32-column slabs (see slab_offset)
        store16<E>(reinterpret_cast<typename E::T*>(reinterpret_cast<uint8_t*>(y) + slab_offset(row, i, d)), o);
      else
        store16<E>(y + row * d + i, o);
    }
  }
}

// ---------------------------------------------------------------- per-row int8 activations
// Quantisation parameters of a row whose largest magnitude is a: inv = 127 / a and s = a / 127
// (IEEE float32 divisions); a == 0 or an inverse that overflows gives s = 0 and zero codes.
__device__ __forceinline__ void quant_params(float a, float& inv, float& s) {
  inv = 127.0f / a;
  s = a / 127.0f;
  if (!(inv <= 3.402823466e38f)) {  // a == 0, or a so small that 127 / a is infinite
    inv = 0.f;
    s = 0.f;
  }
}
// Eight values -> eight codes clamp(rint(v * inv), -127, 127) packed little-endian.
__device__ __forceinline__ uint2 quant8(const float* v, float inv) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int qi = static_cast<int>(fminf(fmaxf(rintf(v[j] * inv), -127.f), 127.f));
    const uint32_t b = static_cast<uint32_t>(qi) & 0xffu;
    if (j < 4) lo |= b << (8 * j); else hi |= b << (8 * (j - 4));
  }
  return make_uint2(lo, hi);
}

// Largest value over the workgroup for each of kRows rows (part: kRows x 4 floats of LDS).
template <int kRows>
__device__ __forceinline__ void block_max_rows(float* m, float (*part)[kThreads / 64]) {
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    m[r] = wave_max(m[r]);
    if ((threadIdx.x & 63) == 0) part[r][threadIdx.x >> 6] = m[r];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    float a = part[r][0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) a = fmaxf(a, part[r][w]);
    m[r] = a;
  }
}

// Modulated RMSNorm of kRows bfloat16 rows (the arithmetic of norm_rows_kernel), rounded to
// bfloat16, then quantised per row: codes in slab_offset_q8 order, float32 scales.
template <int kChunks, int kRows>
__global__ __launch_bounds__(kThreads) void norm_quant_kernel(const uint16_t* __restrict__ x,
                                                              const float* __restrict__ shift,
                                                              const float* __restrict__ scale,
                                                              int8_t* __restrict__ q,
                                                              float* __restrict__ qscale,
                                                              int64_t n_rows, int d, float eps) {
  constexpr int V = 8;
  __shared__ float part[kRows][kThreads / 64];
  __shared__ float pmax[kRows][kThreads / 64];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kRows;
  // Each chunk stays in registers as its 8 bfloat16 values: first the input, then the
  // normalised values rounded to bfloat16 (exactly what the codes are formed from).
  uint4 raw[kRows][kChunks];
  float ss[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    ss[r] = 0.f;
    const int64_t row = r0 + r;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int i = (c * kThreads + threadIdx.x) * V;
      raw[r][c] = make_uint4(0u, 0u, 0u, 0u);
      if (row < n_rows && i < d) {
        raw[r][c] = *reinterpret_cast<const uint4*>(x + row * d + i);
        float v[V];
        unpack16<BF16>(raw[r][c], v);
#pragma unroll
        for (int j = 0; j < V; ++j) ss[r] = fmaf(v[j], v[j], ss[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    ss[r] = wave_sum(ss[r]);
    if ((threadIdx.x & 63) == 0) part[r][threadIdx.x >> 6] = ss[r];
  }
  __syncthreads();
  float rs[kRows], amax[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) tot += part[r][w];
    rs[r] = 1.0f / sqrtf(tot / static_cast<float>(d) + eps);
    amax[r] = 0.f;
  }
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int i = (c * kThreads + threadIdx.x) * V;
    if (i >= d) continue;
    float sc[V], sh[V];
#pragma unroll
    for (int j = 0; j < V / 4; ++j) {
      const float4 a = reinterpret_cast<const float4*>(scale + i)[j];
      const float4 b = reinterpret_cast<const float4*>(shift + i)[j];
      sc[4 * j] = 1.f + a.x; sc[4 * j + 1] = 1.f + a.y; sc[4 * j + 2] = 1.f + a.z; sc[4 * j + 3] = 1.f + a.w;
      sh[4 * j] = b.x; sh[4 * j + 1] = b.y; sh[4 * j + 2] = b.z; sh[4 * j + 3] = b.w;
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      float v[V];
      unpack16<BF16>(raw[r][c], v);
      uint32_t bits[V];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        bits[j] = f32_to_bf16_bits(fmaf(v[j] * rs[r], sc[j], sh[j]));
        amax[r] = fmaxf(amax[r], fabsf(bf16_bits_to_f32(bits[j])));
      }
      raw[r][c] = make_uint4(bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16),
                             bits[4] | (bits[5] << 16), bits[6] | (bits[7] << 16));
    }
  }
  block_max_rows<kRows>(amax, pmax);
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int64_t row = r0 + r;
    if (row >= n_rows) continue;
    float inv, s;
    quant_params(amax[r], inv, s);
    if (threadIdx.x == 0) qscale[row] = s;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int i = (c * kThreads + threadIdx.x) * V;
      float v[V];
      unpack16<BF16>(raw[r][c], v);
      if (i < d) *reinterpret_cast<uint2*>(q + slab_offset_q8(row, i, d)) = quant8(v, inv);
    }
  }
}

// One workgroup per bfloat16 row [cols]: the row stays in registers (kChunks 16-byte chunks per
// thread, cols <= kChunks * 2048), amax over the workgroup, then codes and scale as above.
template <int kChunks>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(const uint16_t* __restrict__ a,
                                                              int8_t* __restrict__ q,
                                                              float* __restrict__ qscale,
                                                              int64_t cols) {
  __shared__ float pmax[1][kThreads / 64];
  const int64_t row = blockIdx.x;
  const uint16_t* ar = a + row * cols;
  u32x4 raw[kChunks];
  float amax[1] = {0.f};
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int64_t i = (c * kThreads + threadIdx.x) * 8;
    raw[c] = u32x4{0u, 0u, 0u, 0u};
    if (i < cols) raw[c] = *reinterpret_cast<const u32x4*>(ar + i);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      amax[0] = fmaxf(amax[0], fmaxf(fabsf(__uint_as_float(raw[c][j] << 16)),
                                     fabsf(__uint_as_float(raw[c][j] & 0xffff0000u))));
  }
  block_max_rows<1>(amax, pmax);
  float inv, s;
  quant_params(amax[0], inv, s);
  if (threadIdx.x == 0) qscale[row] = s;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int64_t i = (c * kThreads + threadIdx.x) * 8;
    if (i >= cols) continue;
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(raw[c][j] << 16);
      v[2 * j + 1] = __uint_as_float(raw[c][j] & 0xffff0000u);
    }
    *reinterpret_cast<uint2*>(q + slab_offset_q8(row, i, cols)) = quant8(v, inv);
  }
}

// ---------------------------------------------------------------- token merge / unmerge
// Merged row p < n_video/2 is the mean of unmerged rows 2p and 2p+1: their float32 sum is
// exact (or, when it is not, too small a change to move the bfloat16 result), halving is exact,
// so a single rounding to the storage type gives the correctly rounded mean.
template <class E>
__global__ __launch_bounds__(kThreads) void merge_kernel(const typename E::T* __restrict__ x,
                                                         typename E::T* __restrict__ xm,
                                                         int64_t nv_half, int64_t n_out,
                                                         int d) {
  constexpr int V = Vec<E>::n;
  const int64_t cpr = d / V;
  const int64_t total = n_out * cpr;
  for (int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * kThreads) {
    const int64_t row = idx / cpr, c = (idx % cpr) * V;
    float out[V];
    if (row < nv_half) {
      float a[V], b[V];
      load16<E>(x + (2 * row) * d + c, a);
      load16<E>(x + (2 * row + 1) * d + c, b);
#pragma unroll
      for (int j = 0; j < V; ++j) out[j] = (a[j] + b[j]) * 0.5f;
    } else {
      load16<E>(x + (row + nv_half) * d + c, out);
    }
    store16<E>(xm + row * d + c, out);
  }
}

template <class E>
__global__ __launch_bounds__(kThreads) void unmerge_kernel(const typename E::T* __restrict__ xm,
                                                           typename E::T* __restrict__ x,
                                                           int64_t n_video, int64_t n_out,
                                                           int d) {
  // One lane per 16-byte chunk of a merged row, read once: a video pair's chunk is written to
  // both rows of the pair.
  constexpr int V = Vec<E>::n;
  const int64_t cpr = d / V;
  const int64_t nv_half = n_video / 2;
  const int64_t total = (n_out - nv_half) * cpr;  // merged rows
  for (int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * kThreads) {
    const int64_t p = idx / cpr, c = (idx % cpr) * V;
    const uint4 raw = *reinterpret_cast<const uint4*>(xm + p * d + c);
    if (p < nv_half) {
      *reinterpret_cast<uint4*>(x + (2 * p) * d + c) = raw;
      *reinterpret_cast<uint4*>(x + (2 * p + 1) * d + c) = raw;
    } else {
      *reinterpret_cast<uint4*>(x + (p + nv_half) * d + c) = raw;
    }
  }
}

// ---------------------------------------------------------------- Euler update
// z <- fma(delta, v, z): one rounding of the exact z + delta * v.
// Fixed condition rows of the Euler update: video rows [0, lo) and [hi, n_video) of z.
struct CondRows {
  int64_t lo, hi, n_video;
};

// z += delta * v, one float32 rounding (fmaf), 4 elements per lane, except on fixed condition
// rows. v is the fresh velocity (copied to v_copy when given) or, on reused steps with
// v_prev, the extrapolation fmaf(w, float32(v - v_prev), v).
template <class E>
__global__ __launch_bounds__(kThreads) void euler_kernel(float* __restrict__ z,
                                                         const typename E::T* __restrict__ v,
                                                         const typename E::T* __restrict__ v_prev,
                                                         float w, float delta,
                                                         typename E::T* __restrict__ v_copy,
                                                         int64_t n4, int d, CondRows cond) {
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t row = (4 * i) / d;
    float vv[4], pv[4];
    if constexpr (sizeof(typename E::T) == 4) {
      const float4 t = reinterpret_cast<const float4*>(v)[i];
      vv[0] = t.x; vv[1] = t.y; vv[2] = t.z; vv[3] = t.w;
      if (v_copy) reinterpret_cast<float4*>(v_copy)[i] = t;
      if (v_prev) {
        const float4 u = reinterpret_cast<const float4*>(v_prev)[i];
        pv[0] = u.x; pv[1] = u.y; pv[2] = u.z; pv[3] = u.w;
      }
    } else {
      const uint2 t = reinterpret_cast<const uint2*>(v)[i];
      vv[0] = __uint_as_float(t.x << 16); vv[1] = __uint_as_float(t.x & 0xffff0000u);
      vv[2] = __uint_as_float(t.y << 16); vv[3] = __uint_as_float(t.y & 0xffff0000u);
      if (v_copy) reinterpret_cast<uint2*>(v_copy)[i] = t;
      if (v_prev) {
        const uint2 u = reinterpret_cast<const uint2*>(v_prev)[i];
        pv[0] = __uint_as_float(u.x << 16); pv[1] = __uint_as_float(u.x & 0xffff0000u);
        pv[2] = __uint_as_float(u.y << 16); pv[3] = __uint_as_float(u.y & 0xffff0000u);
      }
    }
    if (row < cond.lo || (row >= cond.hi && row < cond.n_video)) continue;  // held condition row
    if (v_prev) {
#pragma unroll
      for (int j = 0; j < 4; ++j) vv[j] = fmaf(w, vv[j] - pv[j], vv[j]);
    }
    float4 zz = reinterpret_cast<float4*>(z)[i];
    zz.x = fmaf(delta, vv[0], zz.x);
    zz.y = fmaf(delta, vv[1], zz.y);
    zz.z = fmaf(delta, vv[2], zz.z);
    zz.w = fmaf(delta, vv[3], zz.w);
    reinterpret_cast<float4*>(z)[i] = zz;
  }
}

// Core reuse: save (delta = x), diff (delta = x - delta) and apply (x = act(x + delta)) over
// n4 groups of 4 elements; delta is float32.
template <class E, int kOp>
__global__ __launch_bounds__(kThreads) void core_kernel(typename E::T* __restrict__ x,
                                                        float* __restrict__ delta, int64_t n4) {
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * kThreads) {
    float xv[4];
    if constexpr (sizeof(typename E::T) == 4) {
      const float4 t = reinterpret_cast<const float4*>(x)[i];
      xv[0] = t.x; xv[1] = t.y; xv[2] = t.z; xv[3] = t.w;
    } else {
      const uint2 t = reinterpret_cast<const uint2*>(x)[i];
      xv[0] = __uint_as_float(t.x << 16); xv[1] = __uint_as_float(t.x & 0xffff0000u);
      xv[2] = __uint_as_float(t.y << 16); xv[3] = __uint_as_float(t.y & 0xffff0000u);
    }
    float4* dp = reinterpret_cast<float4*>(delta) + i;
    if constexpr (kOp == 0) {
      *dp = make_float4(xv[0], xv[1], xv[2], xv[3]);
    } else if constexpr (kOp == 1) {
      const float4 dd = *dp;
      *dp = make_float4(xv[0] - dd.x, xv[1] - dd.y, xv[2] - dd.z, xv[3] - dd.w);
    } else {
      const float4 dd = *dp;
      const float y[4] = {xv[0] + dd.x, xv[1] + dd.y, xv[2] + dd.z, xv[3] + dd.w};
      if constexpr (sizeof(typename E::T) == 4) {
        reinterpret_cast<float4*>(x)[i] = make_float4(y[0], y[1], y[2], y[3]);
      } else {
        reinterpret_cast<uint2*>(x)[i] =
            make_uint2(static_cast<uint32_t>(f32_to_bf16_bits(y[0])) | (static_cast<uint32_t>(f32_to_bf16_bits(y[1])) << 16),
                       static_cast<uint32_t>(f32_to_bf16_bits(y[2])) | (static_cast<uint32_t>(f32_to_bf16_bits(y[3])) << 16));
      }
    }
  }
}

// ---------------------------------------------------------------- DiT input [act(z); text]
template <class E>
__global__ __launch_bounds__(kThreads) void assemble_kernel(const float* __restrict__ z,
                                                            const typename E::T* __restrict__ text,
                                                            typename E::T* __restrict__ x,
                                                            int64_t n_state, int64_t n_rows,
                                                            int d) {
  const int64_t cpr = d / 4;
  const int64_t total = n_rows * cpr;
  for (int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * kThreads) {
    const int64_t row = idx / cpr, c = (idx % cpr) * 4;
    if (row < n_state) {
      const float4 t = *reinterpret_cast<const float4*>(z + row * d + c);
      E::store(x, row * d + c + 0, t.x);
      E::store(x, row * d + c + 1, t.y);
      E::store(x, row * d + c + 2, t.z);
      E::store(x, row * d + c + 3, t.w);
    } else {
      const int64_t tr = row - n_state;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[row * d + c + j] = text[tr * d + c + j];
    }
  }
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const uint4* __restrict__ src,
                                                        uint4* __restrict__ dst, int64_t n16) {
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kThreads)
    dst[i] = src[i];
}

// ---------------------------------------------------------------- 3D RoPE table
// Entry (axis, position, pair k) = (cos, sin) of position * theta^(-2k / D), D the chunk size,
// evaluated in double precision and rounded to float32. The x axis is tabulated at half-unit
// positions so that merged tokens (x = 2m + 0.5) index it directly.
__global__ void rope_table_kernel(float2* __restrict__ table, int frames, int grid_h,
                                  int grid_w, int kt, int ky, double log2_theta) {
  const int n_t = frames * kt, n_y = grid_h * ky, n_x = 2 * grid_w * ky;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_t + n_y + n_x) return;
  double pos;
  int k, pairs;
  if (i < n_t) {
    pos = i / kt; k = i % kt; pairs = kt;
  } else if (i < n_t + n_y) {
    pos = (i - n_t) / ky; k = (i - n_t) % ky; pairs = ky;
  } else {
    pos = 0.5 * ((i - n_t - n_y) / ky); k = (i - n_t - n_y) % ky; pairs = ky;
  }
  const double omega = exp2(-2.0 * k / (2.0 * pairs) * log2_theta);
  const double phi = pos * omega;
  table[i] = make_float2(static_cast<float>(cos(phi)), static_cast<float>(sin(phi)));
}

// Per video row, the entry offsets of its t, y and x positions in the table above.
__global__ void rope_rowbase_kernel(int4* __restrict__ rowbase, GeomDev g, int kt, int ky) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= g.n_video) return;
  const int per_frame = g.grid_h * g.cols;
  const int t = r / per_frame;
  const int y = (r % per_frame) / g.cols;
  const int c = r % g.cols;
  const int x2 = g.merged ? 4 * c + 1 : 2 * c;
  const int off_y = g.frames * kt, off_x = off_y + g.grid_h * ky;
  rowbase[r] = make_int4(t * kt, off_y + y * ky, off_x + x2 * ky, 0);
}

// ---------------------------------------------------------------- weight packing
// float32 weights: packed rows stay row-major. bfloat16 weights: packed rows are stored as
// 256-row x 32-column slabs (slab_offset), the operand order of the MFMA GEMM.
template <class T>
__global__ __launch_bounds__(kThreads) void pack_kernel(const T* __restrict__ w,
                                                        T* __restrict__ packed, int kind,
                                                        int64_t rows, int64_t cols) {
  constexpr int V = 16 / sizeof(T);
  const int64_t cpr = cols / V;
  const int64_t total = rows * cpr;
  for (int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * kThreads) {
    const int64_t p = idx / cpr, c = (idx % cpr) * V;
    const int64_t src = packed_source_row(kind, p, rows);
    T* dst = sizeof(T) == 2 ? reinterpret_cast<T*>(reinterpret_cast<uint8_t*>(packed) + slab_offset(p, c, cols))
                            : packed + p * cols + c;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(w + src * cols + c);
  }
}

// One workgroup per packed row: amax, scale = bf16(amax / 127), codes = clamp(rint(w / s)).
// Codes are stored as 256-row x 32-byte slabs (slab_offset_i8), or as 256-row x 64-byte slabs
// (slab_offset_q8) for the W8A8 GEMM; scales in packed row order.
__global__ __launch_bounds__(kThreads) void pack_int8_kernel(const uint16_t* __restrict__ w,
                                                             int8_t* __restrict__ q,
                                                             uint16_t* __restrict__ scale,
                                                             int kind, int64_t rows,
                                                             int64_t cols, int slab64) {
  __shared__ float part[kThreads / 64];
  const int64_t p = blockIdx.x;
  const int64_t src = packed_source_row(kind, p, rows);
  const uint16_t* wr = w + src * cols;
  float amax = 0.f;
  for (int64_t c = threadIdx.x * 8; c < cols; c += kThreads * 8) {
    float v[8];
    load16<BF16>(wr + c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
  __syncthreads();
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) a = fmaxf(a, part[i]);
  const uint16_t sbits = a == 0.f ? 0 : f32_to_bf16_bits(a / 127.0f);
  const float s = bf16_bits_to_f32(sbits);
  if (threadIdx.x == 0) scale[p] = sbits;
  for (int64_t c = threadIdx.x * 8; c < cols; c += kThreads * 8) {
    float v[8];
    load16<BF16>(wr + c, v);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int qi = 0;
      if (s != 0.f) qi = static_cast<int>(fminf(fmaxf(rintf(v[j] / s), -127.f), 127.f));
      const uint32_t b = static_cast<uint32_t>(qi) & 0xffu;
      if (j < 4) lo |= b << (8 * j); else hi |= b << (8 * (j - 4));
    }
    const int64_t off = slab64 ? slab_offset_q8(p, c, cols) : slab_offset_i8(p, c, cols);
    *reinterpret_cast<uint2*>(q + off) = make_uint2(lo, hi);
  }
}

// int8 codes in slab_offset_i8 order -> the same values as bfloat16 in slab_offset order (exact:
// |q| <= 127). One lane per 16-byte output chunk, in output order: a 16 KB bf16 slab is written
// linearly while its 8 KB int8 slab is read once.
__global__ __launch_bounds__(kThreads) void widen_int8_kernel(const int8_t* __restrict__ q,
                                                              uint16_t* __restrict__ w,
                                                              int64_t rows, int64_t cols) {
  const int64_t total = rows * cols / 8;  // 16-byte output chunks
  const int64_t kslabs = cols / 32;
  for (int64_t o = blockIdx.x * (int64_t)kThreads + threadIdx.x; o < total; o += (int64_t)gridDim.x * kThreads) {
    const int64_t slab = o >> 10;                  // 1024 chunks per 16 KB slab
    const int rr = static_cast<int>((o >> 2) & 255), pc = static_cast<int>(o & 3);
    const int lc = pc ^ ((rr >> 2) & 3);           // logical 8-column chunk of the row
    const int64_t r = (slab / kslabs) * 256 + rr;
    const int64_t c = (slab % kslabs) * 32 + lc * 8;
    const uint2 raw = *reinterpret_cast<const uint2*>(q + slab_offset_i8(r, c, cols));
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t word = j < 4 ? raw.x : raw.y;
      v[j] = static_cast<float>(static_cast<int8_t>((word >> (8 * (j & 3))) & 0xffu));
    }
    store16<BF16>(w + o * 8, v);
  }
}

int grid_for(int64_t work_items) {
  int64_t g = (work_items + kThreads - 1) / kThreads;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

}  // namespace

hipError_t launch_norm_mod(int act, int64_t n_rows, int d, float eps, const void* x,
                           const float* shift, const float* scale, void* y, int out_tiled,
                           hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  constexpr int kRows = 4;
  const unsigned grid = static_cast<unsigned>((n_rows + kRows - 1) / kRows);
  if (act == H3X_BF16) {
    const uint16_t* xx = static_cast<const uint16_t*>(x);
    uint16_t* yy = static_cast<uint16_t*>(y);
    switch ((d + kThreads * 8 - 1) / (kThreads * 8)) {
      case 1: norm_rows_kernel<BF16, 1, kRows><<<grid, kThreads, 0, s>>>(xx, shift, scale, yy, n_rows, d, eps, out_tiled); break;
      case 2: norm_rows_kernel<BF16, 2, kRows><<<grid, kThreads, 0, s>>>(xx, shift, scale, yy, n_rows, d, eps, out_tiled); break;
      case 3: norm_rows_kernel<BF16, 3, kRows><<<grid, kThreads, 0, s>>>(xx, shift, scale, yy, n_rows, d, eps, out_tiled); break;
      case 4: norm_rows_kernel<BF16, 4, kRows><<<grid, kThreads, 0, s>>>(xx, shift, scale, yy, n_rows, d, eps, out_tiled); break;
      default: norm_mod_kernel<BF16><<<dim3(n_rows), kThreads, 0, s>>>(xx, shift, scale, yy, d, eps, out_tiled);
    }
  } else {
    const float* xx = static_cast<const float*>(x);
    float* yy = static_cast<float*>(y);
    switch ((d + kThreads * 4 - 1) / (kThreads * 4)) {
      case 1: norm_rows_kernel<F32, 1, kRows><<<grid, kThreads, 0, s>>>(xx, shift, scale, yy, n_rows, d, eps, 0); break;
      case 2: norm_rows_kernel<F32, 2, kRows><<<grid, kThreads, 0, s>>>(xx, shift, scale, yy, n_rows, d, eps, 0); break;
      default: norm_mod_kernel<F32><<<dim3(n_rows), kThreads, 0, s>>>(xx, shift, scale, yy, d, eps, 0);
    }
  }
  return hipGetLastError();
}

hipError_t launch_token_merge(int act, const GeomDev& g, int d, const void* x, void* xm,
                              hipStream_t s) {
  const int64_t nv_half = g.n_video / 2;
  const int64_t n_out = nv_half + g.n_audio + g.n_text;
  const int V = act == H3X_BF16 ? 8 : 4;
  const int grid = grid_for(n_out * (d / V));
  if (act == H3X_BF16)
    merge_kernel<BF16><<<grid, kThreads, 0, s>>>(static_cast<const uint16_t*>(x),
                                                 static_cast<uint16_t*>(xm), nv_half, n_out, d);
  else
    merge_kernel<F32><<<grid, kThreads, 0, s>>>(static_cast<const float*>(x),
                                                static_cast<float*>(xm), nv_half, n_out, d);
  return hipGetLastError();
}

hipError_t launch_token_unmerge(int act, const GeomDev& g, int d, const void* xm, void* x,
                                hipStream_t s) {
  const int64_t n_out = g.n_video + g.n_audio + g.n_text;
  const int V = act == H3X_BF16 ? 8 : 4;
  const int grid = grid_for((n_out - g.n_video / 2) * (d / V));
  if (act == H3X_BF16)
    unmerge_kernel<BF16><<<grid, kThreads, 0, s>>>(static_cast<const uint16_t*>(xm),
                                                   static_cast<uint16_t*>(x), g.n_video, n_out, d);
  else
    unmerge_kernel<F32><<<grid, kThreads, 0, s>>>(static_cast<const float*>(xm),
                                                  static_cast<float*>(x), g.n_video, n_out, d);
  return hipGetLastError();
}

hipError_t launch_euler(int act, int64_t n_elems, int d, float* z, const void* v,
                        const void* v_prev, float w, float delta, void* v_copy, int64_t cond_lo,
                        int64_t cond_hi, int64_t n_video, hipStream_t s) {
  const int64_t n4 = n_elems / 4;
  if (n4 == 0) return hipSuccess;
  const int grid = grid_for(n4);
  const CondRows cond{cond_lo, cond_hi, n_video};
  if (act == H3X_BF16)
    euler_kernel<BF16><<<grid, kThreads, 0, s>>>(z, static_cast<const uint16_t*>(v),
                                                 static_cast<const uint16_t*>(v_prev), w, delta,
                                                 static_cast<uint16_t*>(v_copy), n4, d, cond);
  else
    euler_kernel<F32><<<grid, kThreads, 0, s>>>(z, static_cast<const float*>(v),
                                                static_cast<const float*>(v_prev), w, delta,
                                                static_cast<float*>(v_copy), n4, d, cond);
  return hipGetLastError();
}

hipError_t launch_core(int act, int op, int64_t n_elems, void* x, float* delta, hipStream_t s) {
  const int64_t n4 = n_elems / 4;
  if (n4 == 0) return hipSuccess;
  const int grid = grid_for(n4);
  if (act == H3X_BF16) {
    uint16_t* xx = static_cast<uint16_t*>(x);
    if (op == 0) core_kernel<BF16, 0><<<grid, kThreads, 0, s>>>(xx, delta, n4);
    else if (op == 1) core_kernel<BF16, 1><<<grid, kThreads, 0, s>>>(xx, delta, n4);
    else core_kernel<BF16, 2><<<grid, kThreads, 0, s>>>(xx, delta, n4);
  } else {
    float* xx = static_cast<float*>(x);
    if (op == 0) core_kernel<F32, 0><<<grid, kThreads, 0, s>>>(xx, delta, n4);
    else if (op == 1) core_kernel<F32, 1><<<grid, kThreads, 0, s>>>(xx, delta, n4);
    else core_kernel<F32, 2><<<grid, kThreads, 0, s>>>(xx, delta, n4);
  }
  return hipGetLastError();
}

hipError_t launch_assemble(int act, int64_t n_state, int64_t n_text, int d, const float* z,
                           const void* text, void* x, hipStream_t s) {
  const int64_t n_rows = n_state + n_text;
  const int grid = grid_for(n_rows * (d / 4));
  if (act == H3X_BF16)
    assemble_kernel<BF16><<<grid, kThreads, 0, s>>>(z, static_cast<const uint16_t*>(text),
                                                    static_cast<uint16_t*>(x), n_state, n_rows, d);
  else
    assemble_kernel<F32><<<grid, kThreads, 0, s>>>(z, static_cast<const float*>(text),
                                                   static_cast<float*>(x), n_state, n_rows, d);
  return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  if (n16 == 0) return hipSuccess;
  copy_kernel<<<grid_for(n16), kThreads, 0, s>>>(static_cast<const uint4*>(src),
                                                 static_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_rope_table(const GeomDev& g, int head_dim, float theta, float2* table,
                             int4* rowbase, hipStream_t s) {
  const int kt = head_dim / 8, ky = 3 * head_dim / 16;
  const int n = g.frames * kt + g.grid_h * ky + 2 * g.grid_w * ky;
  if (n == 0) return hipSuccess;  // no video axis at all (audio / text only)
  rope_table_kernel<<<(n + 255) / 256, 256, 0, s>>>(table, g.frames, g.grid_h, g.grid_w, kt, ky,
                                                    log2(static_cast<double>(theta)));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.n_video == 0) return e;
  rope_rowbase_kernel<<<(g.n_video + 255) / 256, 256, 0, s>>>(rowbase, g, kt, ky);
  return hipGetLastError();
}

hipError_t launch_pack(int wdtype, int kind, int64_t rows, int64_t cols, const void* w,
                       void* packed, hipStream_t s) {
  if (wdtype == H3X_BF16) {
    pack_kernel<uint16_t><<<grid_for(rows * cols / 8), kThreads, 0, s>>>(
        static_cast<const uint16_t*>(w), static_cast<uint16_t*>(packed), kind, rows, cols);
  } else {
    pack_kernel<float><<<grid_for(rows * cols / 4), kThreads, 0, s>>>(
        static_cast<const float*>(w), static_cast<float*>(packed), kind, rows, cols);
  }
  return hipGetLastError();
}

hipError_t launch_pack_int8(int kind, int64_t rows, int64_t cols, const void* w_bf16,
                            int8_t* q, uint16_t* scale, int slab64, hipStream_t s) {
  pack_int8_kernel<<<dim3(rows), kThreads, 0, s>>>(static_cast<const uint16_t*>(w_bf16), q,
                                                  scale, kind, rows, cols, slab64);
  return hipGetLastError();
}

hipError_t launch_quant_rows(int64_t n_rows, int64_t cols, const void* a, int8_t* q, float* qscale,
                             hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  if (cols % 64 || cols > 16 * kThreads * 8) return hipErrorInvalidValue;
  const uint16_t* aa = static_cast<const uint16_t*>(a);
  const dim3 grid(static_cast<unsigned>(n_rows));
  const int64_t chunks = (cols + kThreads * 8 - 1) / (kThreads * 8);
  if (chunks <= 1) quant_rows_kernel<1><<<grid, kThreads, 0, s>>>(aa, q, qscale, cols);
  else if (chunks <= 2) quant_rows_kernel<2><<<grid, kThreads, 0, s>>>(aa, q, qscale, cols);
  else if (chunks <= 3) quant_rows_kernel<3><<<grid, kThreads, 0, s>>>(aa, q, qscale, cols);
  else if (chunks <= 4) quant_rows_kernel<4><<<grid, kThreads, 0, s>>>(aa, q, qscale, cols);
  else if (chunks <= 6) quant_rows_kernel<6><<<grid, kThreads, 0, s>>>(aa, q, qscale, cols);
  else if (chunks <= 8) quant_rows_kernel<8><<<grid, kThreads, 0, s>>>(aa, q, qscale, cols);
  else if (chunks <= 12) quant_rows_kernel<12><<<grid, kThreads, 0, s>>>(aa, q, qscale, cols);
  else quant_rows_kernel<16><<<grid, kThreads, 0, s>>>(aa, q, qscale, cols);
  return hipGetLastError();
}

hipError_t launch_norm_mod_quant(int64_t n_rows, int d, float eps, const void* x, const float* shift,
                                 const float* scale, int8_t* q, float* qscale, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  if (d % 64 || d > 4 * kThreads * 8) return hipErrorInvalidValue;
  constexpr int kRows = 4;
  const unsigned grid = static_cast<unsigned>((n_rows + kRows - 1) / kRows);
  const uint16_t* xx = static_cast<const uint16_t*>(x);
  switch ((d + kThreads * 8 - 1) / (kThreads * 8)) {
    case 1: norm_quant_kernel<1, kRows><<<grid, kThreads, 0, s>>>(xx, shift, scale, q, qscale, n_rows, d, eps); break;
    case 2: norm_quant_kernel<2, kRows><<<grid, kThreads, 0, s>>>(xx, shift, scale, q, qscale, n_rows, d, eps); break;
    case 3: norm_quant_kernel<3, kRows><<<grid, kThreads, 0, s>>>(xx, shift, scale, q, qscale, n_rows, d, eps); break;
    default: norm_quant_kernel<4, kRows><<<grid, kThreads, 0, s>>>(xx, shift, scale, q, qscale, n_rows, d, eps); break;
  }
  return hipGetLastError();
}

hipError_t launch_widen_int8(int64_t rows, int64_t cols, const int8_t* q, void* w, hipStream_t s) {
  widen_int8_kernel<<<grid_for(rows * cols / 8), kThreads, 0, s>>>(q, static_cast<uint16_t*>(w), rows, cols);
  return hipGetLastError();
}

}  // namespace h3x
