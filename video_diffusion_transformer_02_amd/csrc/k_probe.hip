// Matrix-core throughput probe: the MFMA rate the chip sustains with operands that change from
// one instruction to the next (as in a GEMM's K loop) but without any memory traffic, so that
// the projection GEMMs can be compared with what their instruction mix can reach at the clock
// the chip holds under that load, next to the nominal peak.
//
// Every wave keeps 8 A and 8 B fragments of pseudo-random values (bf16 with |x| in [0.5, 2)
// and random signs, or int8 codes in [-127, 127]) and 4 accumulators, and per iteration issues
// 64 MFMAs over the 64 (A, B) pairs, four independent accumulation chains in turn. One
// workgroup of eight waves per compute unit (two waves per SIMD, as in the GEMMs).
#include <type_traits>

#include "launch.h"

namespace h3x {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeMfmas = 64;  // per wave and iteration

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  // Integer hash (xorshift-multiply): only a source of varied bit patterns.
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// bf16 bits with a random sign and mantissa and exponent 126 or 127: |x| in [0.5, 2).
__device__ __forceinline__ uint32_t bf16_pair(uint32_t r) {
  const uint32_t lo = (r & 0x807fu) | (0x3f00u + ((r >> 7) & 0x80u));
  const uint32_t hi = ((r >> 16) & 0x807fu) | (0x3f00u + ((r >> 23) & 0x80u));
  return lo | (hi << 16);
}

// int8 codes in [-127, 127] (the byte 0x80 is replaced by 0x81).
__device__ __forceinline__ uint32_t i8_quad(uint32_t r) {
  uint32_t out = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint32_t v = (r >> (8 * b)) & 0xffu;
    v = v == 0x80u ? 0x81u : v;
    out |= v << (8 * b);
  }
  return out;
}

template <bool kI8>
__global__ __launch_bounds__(kProbeThreads, 1) void mfma_probe_kernel(int64_t iters, float* __restrict__ out) {
  const uint32_t seed = (blockIdx.x * kProbeThreads + threadIdx.x) * 0x9e3779b9u;
  u32x4 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t ra = mix32(seed + 8 * i + e), rb = mix32(seed + 64 + 8 * i + e);
      a[i][e] = kI8 ? i8_quad(ra) : bf16_pair(ra);
      b[i][e] = kI8 ? i8_quad(rb) : bf16_pair(rb);
    }
  using Acc = std::conditional_t<kI8, i32x16, f32x16>;
  Acc acc[4] = {};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = (8 * r + i) & 3;
        if constexpr (kI8)
          acc[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a[i]),
                                                        __builtin_bit_cast(i32x4, b[(i + r) & 7]), acc[k], 0, 0, 0);
        else
          acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                          __builtin_bit_cast(bf16x8, b[(i + r) & 7]), acc[k], 0, 0, 0);
      }
  }
  // Keep the products: a lane stores only if its total hits one exact value.
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) t += static_cast<float>(acc[k][e]);
  if (t == 1234.5f) out[0] = t;
}

}  // namespace

static int64_t mfma_probe_workgroups() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

double mfma_probe_ops(int i8, int64_t iters) {
  const double per_mfma = i8 ? 2.0 * 32 * 32 * 32 : 2.0 * 32 * 32 * 16;
  return per_mfma * kProbeMfmas * static_cast<double>(iters) * (kProbeThreads / 64) *
         static_cast<double>(mfma_probe_workgroups());
}

hipError_t launch_mfma_probe(int i8, int64_t iters, float* out, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(mfma_probe_workgroups());
  if (i8)
    mfma_probe_kernel<true><<<grid, kProbeThreads, 0, s>>>(iters, out);
  else
    mfma_probe_kernel<false><<<grid, kProbeThreads, 0, s>>>(iters, out);
  return hipGetLastError();
}

}  // namespace h3x
