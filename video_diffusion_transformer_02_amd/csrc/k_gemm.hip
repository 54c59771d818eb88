// Projection GEMMs of the block: C = A * W^T with fused epilogues.
//
//  * gemm_mfma_kernel: bfloat16 activations, bfloat16 or int8 weights, float32 accumulation on
//    the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16). 256 x 256 output tile per workgroup of
//    eight waves (2 x 4, each 128 x 64), K step 32 in a five-stage LDS pipeline filled by
//    buffer loads that write LDS directly (operands stored as 256 x 32 slabs in LDS order, so a
//    K step is one contiguous copy). The two halves of the workgroup (one wave of each per
//    SIMD) run ping-pong: while one issues its MFMAs the other reads its next fragments and
//    streams the next K step, offset by one barrier interval. int8 weights are
//    widened to bfloat16 in registers (exact: |q| <= 127) and their per-row scale is applied in
//    the epilogue. W8A8 (int8 weights and per-row int8 activations): the same pipeline over
//    64-code K steps (a 256 x 64-byte slab per operand, the byte layout of a bfloat16 step) on
//    v_mfma_i32_32x32x32_i8 with int32 accumulation; the epilogue converts the exact integer
//    sums to float32 and applies the activation row scale and the weight column scale.
//    Workgroups are remapped so that each XCD (own L2) walks a contiguous run of
//    a grouped tile order: consecutive tiles share weight panels and activation panels.
//  * gemm_f32_kernel: float32 activations and weights (small configurations): 64 x 64 tiles,
//    plain FMA, same epilogues.
//
// Epilogues: QKV (3D RoPE on video rows of q and k, v written transposed, pad rows zeroed),
// gated residual (x += gate * acc), SwiGLU over the 32-row gate/up interleave, float32 store.
#include <math.h>
#include <type_traits>

#include "launch.h"

namespace h3x {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 256, BK = 32;
constexpr int kStages = 5;  // LDS stages of the K pipeline (32 KB each for bf16)

// ---------------------------------------------------------------- shared epilogue math
__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }
// The same with the hardware reciprocal (1 ulp) in place of the IEEE division: the bfloat16 h
// it feeds rounds far more coarsely, and the division's refinement steps were a visible part of
// the SwiGLU epilogue.
__device__ __forceinline__ float silu_rcp(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// Table index of the (cos, sin) entry turning pair `dh/2` of video row `row`.
__device__ __forceinline__ int rope_index(const RopeDev& r, int64_t row, int dh) {
  const int ct = r.head_dim / 4, cy = 3 * r.head_dim / 8;
  const int4 base = r.rowbase[row];
  if (dh < ct) return base.x + dh / 2;
  if (dh < ct + cy) return base.y + (dh - ct) / 2;
  return base.z + (dh - ct - cy) / 2;
}

// Rotated value of a pair member: v is this element, p its partner; even = first of the pair.
__device__ __forceinline__ float rope_apply(float v, float p, float2 cs, bool even) {
  return even ? fmaf(v, cs.x, -p * cs.y) : fmaf(p, cs.y, v * cs.x);
}

// ---------------------------------------------------------------- MFMA kernel
template <bool kInt8>
struct Smem {
  static constexpr int kA = BM * BK * 2;                 // bytes of one A stage (16 KB)
  static constexpr int kB = BN * BK * (kInt8 ? 1 : 2);   // bytes of one B stage (16 / 8 KB)
  static constexpr int kStage = kA + kB;
  static constexpr int kTotal = kStages * kStage;
};

// LDS byte offset of 16-byte chunk c (0..3) of a 64-byte bf16 row (32 values). Rows r and r+4
// share banks, so the chunk index is flipped by bits 2..3 of the row: any 8 consecutive rows
// read at one chunk hit 8 distinct 16-byte bank groups.
__device__ __forceinline__ int swz16(int row, int c) { return row * 64 + ((c ^ ((row >> 2) & 3)) << 4); }
// LDS byte offset of 16-byte chunk c (0..1) of a 32-byte int8 row (32 codes); rows r and r+8
// share banks, so bit 3 of the row flips the chunk.
__device__ __forceinline__ int swz8(int row, int c) { return row * 32 + ((c ^ ((row >> 3) & 1)) << 4); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// 8 int8 codes (two dwords) -> 8 bfloat16 values, exact.
__device__ __forceinline__ bf16x8 widen_i8(u32x2 v) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = i < 2 ? v.x : v.y;
    const int sh = (i & 1) * 16;
    const float lo = static_cast<float>(static_cast<int8_t>((w >> sh) & 0xff));
    const float hi = static_cast<float>(static_cast<int8_t>((w >> (sh + 8)) & 0xff));
    o[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
  }
  return as_bf16x8(u32x4{o[0], o[1], o[2], o[3]});
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for the LDS pipeline: this wave's LDS reads are complete (so no stage it
// read can be overwritten under it) and at most N of its global->LDS loads are in flight; the
// loads that remain in flight target stages nobody reads before a later barrier. (A plain
// __syncthreads would also drain every outstanding global->LDS load.)
template <int N>
__device__ __forceinline__ void pipeline_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Waves of a workgroup: 2 along M, kWN along N. kWN = 4: eight waves, each 128 x 64 (128
// accumulator registers, two waves per SIMD, so one wave's MFMAs can run while the other waits).
template <int kWN>
struct Layout {
  static constexpr int kWaves = 2 * kWN;
  static constexpr int kThreadsT = 64 * kWaves;
  static constexpr int SN = BN / kWN;  // columns per wave
  static constexpr int NB = SN / 32;   // 32-wide MFMA blocks per wave along N
};

template <bool kInt8, int kEpi, int kWN, bool kATiled, bool kA8>
__global__ __launch_bounds__(Layout<kWN>::kThreadsT, 1) void gemm_mfma_kernel(GemmArgs p, int tiles_m,
                                                                                int tiles_n, int group_m) {
  static_assert(!kA8 || (kATiled && !kInt8), "W8A8 takes tiled int8 activations and 64-byte weight slabs");
  using L = Layout<kWN>;
  constexpr int NB = L::NB, SN = L::SN, kWaves = L::kWaves;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Smem<kInt8>::kTotal];

  // ---- tile selection: XCD-contiguous runs of a grouped (m-group, n) order
  const int total = tiles_m * tiles_n;
  const int per_xcd = gridDim.x / 8;
  const int logical = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (logical >= total) return;
  const int group_size = group_m * tiles_n;
  const int first_m = (logical / group_size) * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int in_group = logical % group_size;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;
  const int64_t m0 = static_cast<int64_t>(tm) * BM;
  const int64_t n0 = static_cast<int64_t>(tn) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kWN, wn = wave % kWN;
  const int li = lane & 31, hi = lane >> 5;
  const int64_t K = p.k;
  constexpr int kKStep = kA8 ? 64 : BK;  // K elements per pipeline step: 64 bytes of a row
  const int ktiles = static_cast<int>(K / kKStep);

  // ---- global -> LDS without registers: buffer_load_dwordx4 ... lds writes lane l's 16 bytes
  // at (wave-uniform base) + 16 l, so one wave instruction fills 1 KB of a stage.
  //  * Packed weights and tiled activations are stored as 256-row x 32-column slabs already in
  //    the LDS order (see slab_offset), so a K step of an operand is one contiguous 16 KB (bf16)
  //    or 8 KB (int8) run that the lanes copy linearly.
  //  * Row-major A (the kernel-level entry points): each lane fetches the 16-byte chunk that the
  //    swizzle places at its LDS position; rows past the end of A lie outside the buffer's range
  //    and read as zeros.
  constexpr int kSlabA = BM * BK * 2, kSlabB = BN * BK * (kInt8 ? 1 : 2);
  const uint8_t* Ab = static_cast<const uint8_t*>(p.a) + (kATiled ? tm * (K / kKStep) * kSlabA : m0 * K * 2);
  const uint8_t* Wb = static_cast<const uint8_t*>(p.w) + tn * (K / kKStep) * kSlabB;
  const int64_t a_rows = p.m - m0 < BM ? p.m - m0 : BM;
  const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Ab), 0, static_cast<int>(kATiled ? (K / kKStep) * kSlabA : a_rows * K * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Wb), 0, static_cast<int>((K / kKStep) * kSlabB), 0x00020000);
  const uint32_t lin_voff = static_cast<uint32_t>(wave * 1024 + lane * 16);
  const uint32_t lin_step = static_cast<uint32_t>(kWaves * 1024);
  const int a_row = lane >> 2, a_chunk = (lane & 3) ^ ((lane >> 4) & 3);
  const uint32_t a_voff = kATiled ? lin_voff : static_cast<uint32_t>((wave * 16 + a_row) * K * 2 + a_chunk * 16);
  const uint32_t a_step = kATiled ? lin_step : static_cast<uint32_t>(16 * kWaves * K * 2);
  const uint32_t b_voff = lin_voff, b_step = lin_step;
  constexpr int kLoadsA = Smem<kInt8>::kA / 1024 / kWaves;  // per thread per stage
  constexpr int kLoadsB = Smem<kInt8>::kB / 1024 / kWaves;
  constexpr int kLoads = kLoadsA + kLoadsB;

  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto issue_loads = [&](int kt) {
    uint8_t* sa = smem + (kt % kStages) * Smem<kInt8>::kStage;
    uint8_t* sb = sa + Smem<kInt8>::kA;
    const uint32_t ka = static_cast<uint32_t>(kt) * (kATiled ? kSlabA : BK * 2);
    const uint32_t kb = static_cast<uint32_t>(kt) * kSlabB;
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, (lds_ptr)(sa + (kWaves * i + wave) * 1024), 16,
                                               a_voff + i * a_step, ka, 0, 0);
#pragma unroll
    for (int i = 0; i < kLoadsB; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_b, (lds_ptr)(sb + (kWaves * i + wave) * 1024), 16,
                                               b_voff + i * b_step, kb, 0, 0);
  };

  using Acc = std::conditional_t<kA8, i32x16, f32x16>;
  Acc acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  // Operand fragments of one K slice (16 bfloat16 values, or 32 codes for W8A8: 32 bytes of a
  // row either way): A rows of the four m-blocks, B rows of the n-blocks (int8 weights of the
  // bfloat16 path stay packed until just before the multiply).
  struct Frags {
    u32x4 a[4];   // bf16: 8 values; W8A8: 16 codes
    u32x4 b[NB];  // bf16: 8 values; int8: 8 codes in .xy; W8A8: 16 codes
  };
  auto read_frags = [&](int kt, int slice, Frags& f) {
    const uint8_t* sa = smem + (kt % kStages) * Smem<kInt8>::kStage;
    const uint8_t* sb = sa + Smem<kInt8>::kA;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      f.a[mb] = *reinterpret_cast<const u32x4*>(sa + swz16(wm * 128 + mb * 32 + li, 2 * slice + hi));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int row = wn * SN + nb * 32 + li;
      if constexpr (kInt8) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(sb + swz8(row, slice) + 8 * hi);
        f.b[nb] = u32x4{v.x, v.y, 0u, 0u};
      } else {
        f.b[nb] = *reinterpret_cast<const u32x4*>(sb + swz16(row, 2 * slice + hi));
      }
    }
  };
  // The MFMAs of a slice walk the (m-block, n-block) grid in snake order, so that each one
  // changes only one of its two operands from the one before (the matrix cores draw less power
  // when fewer operand bits toggle; measured 0.3-1 % faster on the bf16 GEMMs).
  auto mma = [&](const Frags& f) {
    if constexpr (kA8) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int nb = (mb & 1) ? NB - 1 - j : j;
          acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, f.a[mb]),
                                                             __builtin_bit_cast(i32x4, f.b[nb]), acc[mb][nb], 0, 0, 0);
        }
      return;
    }
    bf16x8 bv[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (kInt8) bv[nb] = widen_i8(u32x2{f.b[nb].x, f.b[nb].y});
      else bv[nb] = as_bf16x8(f.b[nb]);
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int nb = (mb & 1) ? NB - 1 - j : j;
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(f.a[mb]), bv[nb], acc[mb][nb], 0, 0, 0);
      }
  };
  // Ping-pong schedule (eight waves, two per SIMD): waves 0-3 and 4-7 alternate between a
  // memory phase (stream a future K step into LDS, read this K step's fragments) and a
  // compute phase (its 16 MFMAs), offset by one barrier interval, so that on every SIMD one
  // wave feeds the matrix core while the other one loads. Every interval ends with a
  // workgroup barrier at which each wave has at most kStages-2 of its K-step loads in
  // flight: the step read next has landed, and the stage written next has been read by both
  // groups in earlier intervals.
  Frags fa, fb;
  const int group = wave / kWN;
  auto barrier_main = [&]() { pipeline_barrier<(kStages - 2) * kLoads>(); };
  auto barrier_drain = [&]() { pipeline_barrier<0>(); };
  auto compute = [&]() {
    __builtin_amdgcn_s_setprio(1);
    mma(fa);
    mma(fb);
    __builtin_amdgcn_s_setprio(0);
  };
  const int pre = ktiles < kStages - 1 ? ktiles : kStages - 1;
  for (int t = 0; t < pre; ++t) issue_loads(t);
  if (pre == kStages - 1) barrier_main(); else barrier_drain();
  if (group == 1) barrier_main();  // group 1 runs one interval behind
  int kt = 0;
  for (; kt + kStages - 1 < ktiles; ++kt) {
    read_frags(kt, 0, fa);
    read_frags(kt, 1, fb);
    issue_loads(kt + kStages - 1);
    barrier_main();
    compute();
    barrier_main();
  }
  for (; kt < ktiles; ++kt) {
    read_frags(kt, 0, fa);
    read_frags(kt, 1, fb);
    barrier_drain();
    compute();
    barrier_drain();
  }
  if (group == 0) barrier_drain();  // same number of barriers in both groups

  // ---- epilogue through LDS. Each wave stages its 128 x SN float32 result 32 rows at a time
  // (row stride SN + 8 floats: the two half-waves of an MFMA block store to disjoint banks),
  // then reads it back row-wise (8 consecutive columns per lane: RoPE pairs and 16-byte
  // stores) or, for the transposed v, column-wise. Element (mb, nb, 4b + r) of a lane sits at
  // row 8b + 4hi + r of slice mb and column nb*32 + li of the wave's sub-tile.
  constexpr int kStride = SN + 8;
  constexpr int kLanesRow = SN / 8;          // lanes covering one row in row-wise passes
  constexpr int kRowsPass = 64 / kLanesRow;  // rows per row-wise instruction
  float* st = reinterpret_cast<float*>(smem) + wave * 32 * kStride;
  const int64_t row_base = m0 + wm * 128;
  const int64_t col_base = n0 + wn * SN;
  const int lc = (lane % kLanesRow) * 8;  // first of this lane's 8 columns in row-wise passes
  const int lr = lane / kLanesRow;
  float csc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) csc[j] = 1.0f;
  // Weight row scales: int8 codes, or int8 codes widened to bfloat16 ahead of a bf16 launch.
  const bool wscaled = kInt8 || kA8 || p.wscale != nullptr;
  if (kEpi != EPI_SWIGLU && wscaled) {
    const u32x4 sraw = *reinterpret_cast<const u32x4*>(p.wscale + col_base + lc);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      csc[2 * j] = __uint_as_float(sraw[j] << 16);
      csc[2 * j + 1] = __uint_as_float(sraw[j] & 0xffff0000u);
    }
  }
  // Global operands of the row-wise epilogues are fetched one 32-row slice ahead, so that their
  // latency is paid once per tile rather than once per slice: the residual rows of x and the
  // activation row scales (W8A8). The gated residual's column factors gate * scale are formed
  // once.
  constexpr int kIt = 32 / kRowsPass;
  [[maybe_unused]] u32x4 xbuf[2][kIt];
  [[maybe_unused]] float rsl[4];  // W8A8 row scales of each slice: lane l holds row l % 32's
  [[maybe_unused]] float gsc[8];
  auto fetch_rows = [&](int mb) {
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int64_t row = row_base + mb * 32 + it * kRowsPass + lr;
      if constexpr (kEpi == EPI_RESID) {  // rows past m read row m-1 (never stored): no branch
        const int64_t rl = row < p.m ? row : p.m - 1;
        xbuf[mb & 1][it] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.x) + rl * p.n + col_base + lc);
      }
    }
  };
  if constexpr (kA8 && kEpi != EPI_SWIGLU) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) rsl[mb] = p.ascale[row_base + mb * 32 + li];
  }
  // The row scale of row r of slice mb, for this lane.
  auto row_scale = [&](int mb, int r) { return __shfl(rsl[mb], r, 64); };
  if constexpr (kEpi == EPI_RESID) {
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(p.gate + col_base + lc);
    const f32x4 g1 = *reinterpret_cast<const f32x4*>(p.gate + col_base + lc + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      gsc[j] = g0[j] * csc[j];
      gsc[4 + j] = g1[j] * csc[4 + j];
    }
  }
  if constexpr (kEpi == EPI_RESID) fetch_rows(0);
  // QKV, q and k columns: a lane's 8 features lie in one RoPE chunk (axis, first pair k0); the
  // table offsets of its rows are read once, the (cos, sin) entries of a slice while it is staged.
  const int region = kEpi == EPI_QKV ? static_cast<int>(n0 / p.d_model) : 0;  // 0 q, 1 k, 2 v
  const int64_t fq = col_base + lc - static_cast<int64_t>(region) * p.d_model;  // first of 8 features
  [[maybe_unused]] int rbase[4][kIt];
  [[maybe_unused]] f32x4 csb[kIt][2];
  // Rows past the video rows read the entries of the last video row and do not use them, so
  // that no load sits behind a branch (a branch makes the compiler wait for every load).
  const bool has_rope = kEpi == EPI_QKV && region < 2 && p.geom.n_video > 0;
  auto fetch_rope = [&](int mb) {
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      csb[it][0] = *reinterpret_cast<const f32x4*>(p.rope.table + rbase[mb][it]);
      csb[it][1] = *reinterpret_cast<const f32x4*>(p.rope.table + rbase[mb][it] + 2);
    }
  };
  if constexpr (kEpi == EPI_QKV) {
    if (has_rope) {
      const int dh = static_cast<int>(fq % p.rope.head_dim);
      const int ct = p.rope.head_dim / 4, cy = 3 * p.rope.head_dim / 8;
      const int axis = dh < ct ? 0 : (dh < ct + cy ? 1 : 2);
      const int k0 = axis == 0 ? dh / 2 : (axis == 1 ? (dh - ct) / 2 : (dh - ct - cy) / 2);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
          const int64_t row = row_base + mb * 32 + it * kRowsPass + lr;
          const int64_t rl = row < p.geom.n_video ? row : p.geom.n_video - 1;
          rbase[mb][it] = reinterpret_cast<const int*>(p.rope.rowbase + rl)[axis] + k0;
        }
    }
  }
  // SwiGLU: SN packed columns = SN/64 groups of [32 gate | 32 up] -> SN/2 h features per row;
  // a lane owns 8 consecutive features (their gate and up columns) on kItH rows per slice.
  constexpr int kLanesH = SN / 16, kRowsH = 64 / kLanesH, kItH = 32 / kRowsH;
  const int hc = (lane % kLanesH) * 8;  // this lane's first h feature within the wave's SN/2
  const int gcol = (hc / 32) * 64 + hc % 32, ucol = gcol + 32;
  [[maybe_unused]] float sg[8], su[8], rsh[4][kItH];
  if constexpr (kEpi == EPI_SWIGLU) {
#pragma unroll
    for (int j = 0; j < 8; ++j) { sg[j] = 1.0f; su[j] = 1.0f; }
    if (wscaled) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(p.wscale + col_base + gcol);
      const u32x4 b = *reinterpret_cast<const u32x4*>(p.wscale + col_base + ucol);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sg[2 * j] = __uint_as_float(a[j] << 16); sg[2 * j + 1] = __uint_as_float(a[j] & 0xffff0000u);
        su[2 * j] = __uint_as_float(b[j] << 16); su[2 * j + 1] = __uint_as_float(b[j] & 0xffff0000u);
      }
    }
    if constexpr (kA8) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int it = 0; it < kItH; ++it) rsh[mb][it] = p.ascale[row_base + mb * 32 + it * kRowsH + lane / kLanesH];
    }
  }

  // Tiles that lie wholly inside the m rows (all but the last row of tiles) run without per-row
  // checks.
  auto epilogue = [&]<bool kRagged>() {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if constexpr (kEpi == EPI_RESID)
      if (mb + 1 < 4) fetch_rows(mb + 1);
    if constexpr (kEpi == EPI_QKV)  // this slice's entries, loaded while the slice is staged
      if (has_rope) fetch_rope(mb);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        st[(8 * (e >> 2) + 4 * hi + (e & 3)) * kStride + nb * 32 + li] = static_cast<float>(acc[mb][nb][e]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int64_t r0 = row_base + mb * 32;

    if constexpr (kEpi == EPI_F32 || kEpi == EPI_RESID) {
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        const int r = it * kRowsPass + lr;
        const int64_t row = r0 + r;
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(st + r * kStride + lc);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(st + r * kStride + lc + 4);
        float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        if constexpr (kA8) {
          const float rs = row_scale(mb, r);
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] *= rs;
        }
        if (!kRagged || row < p.m) {
          if constexpr (kEpi == EPI_F32) {
            float* o = p.out + row * p.n + col_base + lc;
            *reinterpret_cast<f32x4*>(o) = f32x4{v[0] * csc[0], v[1] * csc[1], v[2] * csc[2], v[3] * csc[3]};
            *reinterpret_cast<f32x4*>(o + 4) = f32x4{v[4] * csc[4], v[5] * csc[5], v[6] * csc[6], v[7] * csc[7]};
          } else {
            uint16_t* xp = static_cast<uint16_t*>(p.x) + row * p.n + col_base + lc;
            const u32x4 xr = xbuf[mb & 1][it];
            u32x4 out;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float x0 = __uint_as_float(xr[j] << 16), x1 = __uint_as_float(xr[j] & 0xffff0000u);
              const float y0 = fmaf(gsc[2 * j], v[2 * j], x0);
              const float y1 = fmaf(gsc[2 * j + 1], v[2 * j + 1], x1);
              out[j] = static_cast<uint32_t>(f32_to_bf16_bits(y0)) |
                       (static_cast<uint32_t>(f32_to_bf16_bits(y1)) << 16);
            }
            *reinterpret_cast<u32x4*>(xp) = out;
          }
        }
      }
    } else if constexpr (kEpi == EPI_SWIGLU) {
      const int64_t F = p.n / 2;
      const int64_t f0 = col_base / 2 + hc;
#pragma unroll
      for (int it = 0; it < kItH; ++it) {
        const int r = it * kRowsH + lane / kLanesH;
        const int64_t row = r0 + r;
        const f32x4 ga = *reinterpret_cast<const f32x4*>(st + r * kStride + gcol);
        const f32x4 gb = *reinterpret_cast<const f32x4*>(st + r * kStride + gcol + 4);
        const f32x4 ua = *reinterpret_cast<const f32x4*>(st + r * kStride + ucol);
        const f32x4 ub = *reinterpret_cast<const f32x4*>(st + r * kStride + ucol + 4);
        float gv[8] = {ga[0], ga[1], ga[2], ga[3], gb[0], gb[1], gb[2], gb[3]};
        float uv[8] = {ua[0], ua[1], ua[2], ua[3], ub[0], ub[1], ub[2], ub[3]};
        if constexpr (kA8) {
          const float rs = rsh[mb][it];
#pragma unroll
          for (int j = 0; j < 8; ++j) { gv[j] *= rs; uv[j] *= rs; }
        }
        if (!kRagged || row < p.m) {
          u32x4 out;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float h0 = silu_rcp(gv[2 * j] * sg[2 * j]) * (uv[2 * j] * su[2 * j]);
            const float h1 = silu_rcp(gv[2 * j + 1] * sg[2 * j + 1]) * (uv[2 * j + 1] * su[2 * j + 1]);
            out[j] = static_cast<uint32_t>(f32_to_bf16_bits(h0)) |
                     (static_cast<uint32_t>(f32_to_bf16_bits(h1)) << 16);
          }
          if (p.out_tiled)
            *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(p.h) + slab_offset(row, f0, F)) = out;
          else
            *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.h) + row * F + f0) = out;
        }
      }
    } else {  // EPI_QKV
      const int64_t d = p.d_model;
      if (region < 2) {
        uint16_t* dst = static_cast<uint16_t*>(region == 0 ? p.q : p.kk);
        const int64_t f = fq;
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
          const int r = it * kRowsPass + lr;
          const int64_t row = r0 + r;
          const f32x4 v0 = *reinterpret_cast<const f32x4*>(st + r * kStride + lc);
          const f32x4 v1 = *reinterpret_cast<const f32x4*>(st + r * kStride + lc + 4);
          float v[8] = {v0[0] * csc[0], v0[1] * csc[1], v0[2] * csc[2], v0[3] * csc[3],
                        v1[0] * csc[4], v1[1] * csc[5], v1[2] * csc[6], v1[3] * csc[7]};
          if constexpr (kA8) {
            const float rs = row_scale(mb, r);
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] *= rs;
          }
          if (has_rope) {
            const bool rot = row < p.geom.n_video;  // selected, not branched on
            const f32x4 cs01 = csb[it][0];
            const f32x4 cs23 = csb[it][1];
            const float c[4] = {cs01[0], cs01[2], cs23[0], cs23[2]};
            const float sn[4] = {cs01[1], cs01[3], cs23[1], cs23[3]};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float a = v[2 * j], b = v[2 * j + 1];
              const float ra = fmaf(a, c[j], -b * sn[j]);
              const float rb = fmaf(a, sn[j], b * c[j]);
              v[2 * j] = rot ? ra : a;
              v[2 * j + 1] = rot ? rb : b;
            }
          }
          // Every row of the tile is below m_pad (a multiple of 256); rows past m get zeros.
          u32x4 out;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool live = !kRagged || row < p.m;
            const float y0 = live ? v[2 * j] : 0.f, y1 = live ? v[2 * j + 1] : 0.f;
            out[j] = static_cast<uint32_t>(f32_to_bf16_bits(y0)) |
                     (static_cast<uint32_t>(f32_to_bf16_bits(y1)) << 16);
          }
          *reinterpret_cast<u32x4*>(dst + row * d + f) = out;
        }
      } else {
        // v transposed: each lane walks one column (feature) down the 32 staged rows and writes
        // them as 64 contiguous bytes of v^T.
        uint16_t* vt = static_cast<uint16_t*>(p.vt);
#pragma unroll
        for (int half = 0; half < SN / 64; ++half) {
          const int c = lane + 64 * half;
          const int64_t f = col_base + c - 2 * d;
          float sc = 1.0f;
          if (wscaled) sc = bf16_bits_to_f32(p.wscale[col_base + c]);
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            u32x4 out;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int r = q4 * 8 + 2 * j;
              float s0 = sc, s1 = sc;
              if constexpr (kA8) {
                s0 *= __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rsl[mb]), r));
                s1 *= __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rsl[mb]), r + 1));
              }
              const float a0 = st[r * kStride + c], a1 = st[(r + 1) * kStride + c];
              const float y0 = (!kRagged || r0 + r < p.m) ? a0 * s0 : 0.f;
              const float y1 = (!kRagged || r0 + r + 1 < p.m) ? a1 * s1 : 0.f;
              out[j] = static_cast<uint32_t>(f32_to_bf16_bits(y0)) |
                       (static_cast<uint32_t>(f32_to_bf16_bits(y1)) << 16);
            }
            *reinterpret_cast<u32x4*>(vt + f * p.m_pad + r0 + q4 * 8) = out;
          }
        }
      }
    }
  }
  };
  if (m0 + BM <= p.m) epilogue.template operator()<false>();
  else epilogue.template operator()<true>();
}

// ---------------------------------------------------------------- float32 kernel
// Thread (tx, ty) of 16 x 16 owns rows ty + 16i (i < 4) and columns {2tx, 2tx+1, 2tx+32,
// 2tx+33} of the 64 x 64 tile: RoPE pairs (2tx, 2tx+1) and gate/up partners (c, c+32) are in
// the same thread.
template <int kEpi>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmArgs p) {
  constexpr int T = 64, TK = 16;
  __shared__ float As[TK][T + 1];
  __shared__ float Bs[TK][T + 1];
  const float* A = static_cast<const float*>(p.a);
  const float* W = static_cast<const float*>(p.w);
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * T;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * T;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  int cols[4] = {2 * tx, 2 * tx + 1, 2 * tx + 32, 2 * tx + 33};
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < p.k; k0 += TK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = threadIdx.x + kThreads * i;  // 0..1023 over [64 rows x 16 k]
      const int r = e / TK, kk = e % TK;
      int64_t gr = m0 + r;
      if (gr >= p.m) gr = p.m - 1;
      As[kk][r] = A[gr * p.k + k0 + kk];
      Bs[kk][r] = W[(n0 + r) * p.k + k0 + kk];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][cols[j]];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + ty + 16 * i;
    if constexpr (kEpi == EPI_F32) {
      if (row < p.m)
        for (int j = 0; j < 4; ++j) p.out[row * p.n + n0 + cols[j]] = acc[i][j];
    } else if constexpr (kEpi == EPI_RESID) {
      float* x = static_cast<float*>(p.x);
      if (row < p.m)
        for (int j = 0; j < 4; ++j) {
          const int64_t c = n0 + cols[j];
          x[row * p.n + c] = fmaf(p.gate[c], acc[i][j], x[row * p.n + c]);
        }
    } else if constexpr (kEpi == EPI_SWIGLU) {
      float* h = static_cast<float*>(p.h);
      const int64_t F = p.n / 2;
      if (row < p.m)
        for (int j = 0; j < 2; ++j) {
          const int64_t f = (n0 / 64) * 32 + cols[j];
          h[row * F + f] = silu(acc[i][j]) * acc[i][j + 2];
        }
    } else {  // EPI_QKV
      const int64_t d = p.d_model;
      const int region = static_cast<int>(n0 / d);
      if (row >= p.m_pad) continue;
      for (int j = 0; j < 4; ++j) {
        const int64_t f = n0 + cols[j] - region * d;
        float out = acc[i][j];
        if (region < 2 && row < p.geom.n_video) {
          const int dh = static_cast<int>(f % p.rope.head_dim);
          const float2 cs = p.rope.table[rope_index(p.rope, row, dh)];
          out = rope_apply(acc[i][j], acc[i][j ^ 1], cs, (j & 1) == 0);
        }
        if (row >= p.m) out = 0.f;
        if (region == 0) static_cast<float*>(p.q)[row * d + f] = out;
        else if (region == 1) static_cast<float*>(p.kk)[row * d + f] = out;
        else static_cast<float*>(p.vt)[f * p.m_pad + row] = out;
      }
    }
  }
}

template <bool kInt8, int kWN, bool kATiled, bool kA8 = false>
hipError_t launch_mfma(int epi, const GemmArgs& a, hipStream_t s) {
  const int tiles_m = static_cast<int>((a.m + BM - 1) / BM);
  const int tiles_n = static_cast<int>(a.n / BN);
  const int total = tiles_m * tiles_n;
  const int grid = (total + 7) / 8 * 8;
  const int group_m = 8;
  constexpr int T = Layout<kWN>::kThreadsT;
  switch (epi) {
    case EPI_QKV:
      gemm_mfma_kernel<kInt8, EPI_QKV, kWN, kATiled, kA8><<<grid, T, 0, s>>>(a, tiles_m, tiles_n, group_m);
      break;
    case EPI_RESID:
      gemm_mfma_kernel<kInt8, EPI_RESID, kWN, kATiled, kA8><<<grid, T, 0, s>>>(a, tiles_m, tiles_n, group_m);
      break;
    case EPI_SWIGLU:
      gemm_mfma_kernel<kInt8, EPI_SWIGLU, kWN, kATiled, kA8><<<grid, T, 0, s>>>(a, tiles_m, tiles_n, group_m);
      break;
    default:
      gemm_mfma_kernel<kInt8, EPI_F32, kWN, kATiled, kA8><<<grid, T, 0, s>>>(a, tiles_m, tiles_n, group_m);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int act, int wdtype, int epi, const GemmArgs& a, hipStream_t s) {
  if (a.m == 0) return hipSuccess;
  if (act == H3X_F32) {
    // EPI_QKV also writes the zero pad rows m .. m_pad-1 of q, k and v^T.
    const int64_t rows = epi == EPI_QKV ? a.m_pad : a.m;
    dim3 grid(static_cast<unsigned>(a.n / 64), static_cast<unsigned>((rows + 63) / 64));
    switch (epi) {
      case EPI_QKV: gemm_f32_kernel<EPI_QKV><<<grid, kThreads, 0, s>>>(a); break;
      case EPI_RESID: gemm_f32_kernel<EPI_RESID><<<grid, kThreads, 0, s>>>(a); break;
      case EPI_SWIGLU: gemm_f32_kernel<EPI_SWIGLU><<<grid, kThreads, 0, s>>>(a); break;
      default: gemm_f32_kernel<EPI_F32><<<grid, kThreads, 0, s>>>(a); break;
    }
    return hipGetLastError();
  }
  if (wdtype == H3X_I8A8) return launch_mfma<false, 4, true, true>(epi, a, s);
  const bool i8 = wdtype == H3X_I8;
  if (a.a_tiled) return i8 ? launch_mfma<true, 4, true>(epi, a, s) : launch_mfma<false, 4, true>(epi, a, s);
  return i8 ? launch_mfma<true, 4, false>(epi, a, s) : launch_mfma<false, 4, false>(epi, a, s);
}

}  // namespace h3x
