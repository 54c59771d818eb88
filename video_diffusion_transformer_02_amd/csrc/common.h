// Shared device helpers and launch-side declarations of the h3x kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3x.h"

namespace h3x {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Plain 16- and 8-byte vectors (ext_vector types stay in registers, unlike HIP's uint4 struct).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- element conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest even (gfx950 has a native conversion instruction for this).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// Element type tags: float storage or bfloat16 storage (uint16_t bits).
struct F32 {
  using T = float;
  static __device__ __forceinline__ float load(const T* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(T* p, int64_t i, float v) { p[i] = v; }
  static constexpr int kBytes = 4;
};
struct BF16 {
  using T = uint16_t;
  static __device__ __forceinline__ float load(const T* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
  static __device__ __forceinline__ void store(T* p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }
  static constexpr int kBytes = 2;
};

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------- geometry on the device
// Positions of video row r: latent (t, y) and twice the x position (x2 = 2x, or 4m + 1 for a
// merged pair m, i.e. x = 2m + 0.5). Audio and text rows (r >= n_video) are not rotated.
struct GeomDev {
  int32_t frames, grid_h, grid_w, n_audio, n_text, merged;
  int32_t cols;     // video columns per latent row: grid_w, or grid_w / 2 when merged
  int32_t n_video;  // frames * grid_h * cols
  int32_t n_tokens;
};

inline GeomDev geom_dev(const h3x_geom& g) {
  GeomDev d;
  d.frames = g.frames; d.grid_h = g.grid_h; d.grid_w = g.grid_w;
  d.n_audio = g.n_audio; d.n_text = g.n_text; d.merged = g.merged;
  d.cols = g.merged ? g.grid_w / 2 : g.grid_w;
  d.n_video = g.frames * g.grid_h * d.cols;
  d.n_tokens = d.n_video + g.n_audio + g.n_text;
  return d;
}

// RoPE table: float2 (cos, sin) entries for axis t [frames x kt], axis y [grid_h x ky],
// axis x [2*grid_w half-unit positions x kx], kt = Dh/8, ky = kx = 3Dh/16 pairs.
struct RopeDev {
  const float2* table;   // (cos, sin) entries
  const int4* rowbase;   // per video row: entry offsets of its t, y and x positions
  int32_t head_dim;
  int32_t kt, ky;        // pairs per chunk: t chunk, y chunk (x chunk has ky pairs too)
  int32_t off_y, off_x;  // table offsets (entries) of the y and x sections
};

}  // namespace h3x
