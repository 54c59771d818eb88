// Full bidirectional attention over the joint token sequence, softmax(q k^T / sqrt(Dh)) v per
// head, with no mask (every token attends to every token).
//
//  * attn_mfma8_kernel (bfloat16, Dh = 128): flash attention with online softmax. A workgroup
//    of eight waves (one per CU, two per SIMD) owns 256 queries of one head (32 per wave) and
//    walks the keys in tiles of 64, double-buffered in LDS and fetched by buffer loads that
//    write LDS directly; each tile is shared by all 256 queries. Each wave
//    computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so that a lane holds 32 scores of a
//    single query: a max needs one cross-lane exchange (lane ^ 32), the running sum none until
//    the end. The probabilities are already in the B-operand layout of O^T += V^T P^T, so they
//    never leave registers. Scores are scaled into base-2 exponent units inside the exponent's
//    FMA and exponentiated with the hardware exp2. The running max is lazy: each tile's
//    probabilities are first taken against the max as it stands, and only when a query's tile
//    sum would exceed 2^16 (or is not finite: the first tile) is the tile max formed and the
//    tile redone, so nearly every tile skips both the max reduction and the O rescale.
//    The queries of a last, partly filled round of workgroups are split over key ranges; the
//    pieces' partial results (unnormalised O, lazy max, sum) are merged by attn_combine_kernel.
//  * attn_f32_kernel: float32, one thread per (query, head), online softmax over keys; the
//    k and v reads of a wave are broadcasts (all its lanes read the same key).
#include <mutex>
#include <math.h>

#include "launch.h"

namespace h3x {
namespace {

constexpr int kDh = 128;
constexpr int kBK = 64;   // keys per tile
constexpr int kTile = kBK * kDh * 2;  // bytes of one K tile or one V^T tile
constexpr int kVBase = 2 * kTile;     // LDS: K stage 0 | K stage 1 | V^T stage 0 | V^T stage 1
// The running max only moves when some query's tile sum of probabilities, taken against the
// max as it stands, exceeds kSpecMax (so every probability stays <= 2^16); the final
// normalisation divides the same factor out of the numerator and the denominator.
constexpr float kSpecMax = 65536.0f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// K tile in LDS: [64 rows][128 dims], 256-byte rows of 16 chunks of 16 bytes, chunk index
// ^ (row & 15), so the 16 rows read by 16 lanes at one chunk fall on distinct banks. LDS row p
// holds key sigma(p) of the tile, sigma swapping bits 2 and 3: the S^T accumulator rows then
// come out in the order in which the P^T operand of O^T += V^T P^T wants its keys, and each
// lane's V^T operand is 8 consecutive keys, one 16-byte read.
__device__ __forceinline__ int key_of_row(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }
// V^T tile in LDS: [128 dims][64 keys], 128-byte rows of 8 chunks, chunk index ^ f(row) with
// f(r) = (r ^ (r >> 3 & 1)) & 7: rows 0..7 get distinct f, and so do the even and the odd rows
// of 0..15, so 16-byte reads of 16 consecutive rows at one chunk are conflict-free whether the
// LDS serves 128 or 256 bytes per cycle.
__device__ __forceinline__ int v_swz(int r) { return (r ^ ((r >> 3) & 1)) & 7; }

typedef __attribute__((address_space(3))) void* lds_ptr;

template <int kWaves>
__device__ __forceinline__ void attn_body(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                          const uint16_t* __restrict__ vt, uint16_t* __restrict__ o,
                                          int n, int n_pad, int n_heads, AttnPlan plan, int full_grid,
                                          int o_tiled, float* __restrict__ part) {
  constexpr int kBQ = 32 * kWaves;       // queries per workgroup
  constexpr int kPieces = 16 / kWaves;   // 1 KB pieces of each tile per wave
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * kTile];

  // Whole items first (blocks 0 .. full_grid-1, each XCD a contiguous run of items so that the
  // workgroups of one head share its K/V tiles in that XCD's L2), then the key pieces of the
  // last round's items (tiles t0 .. t1-1 of one item each).
  int item, t0, t1, slot = -1;
  if (static_cast<int>(blockIdx.x) < full_grid) {
    const int per_xcd = full_grid / 8;
    const int logical = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (logical >= plan.full_items) return;
    item = logical;
    t0 = 0;
    t1 = plan.ktiles;
  } else {
    slot = blockIdx.x - full_grid;
    item = plan.full_items + slot / plan.pieces;
    t0 = (slot % plan.pieces) * plan.tiles;
    t1 = min(plan.ktiles, t0 + plan.tiles);
  }
  const int head = item / plan.qblocks;
  const int qb = item % plan.qblocks;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, hi = lane >> 5;
  const int64_t d = static_cast<int64_t>(n_heads) * kDh;
  const int64_t qrow = static_cast<int64_t>(qb) * kBQ + wave * 32 + li;

  // Q fragments (B operand): dims 16s + 8hi .. +8 of this lane's query.
  bf16x8 qf[8];
  {
    const uint16_t* qp = q + qrow * d + head * kDh + 8 * hi;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * s));
  }

  // K and V^T tiles stream straight into LDS (buffer_load_dwordx4 ... lds: lane l's 16 bytes
  // land at the wave's 1 KB piece + 16 l); each lane fetches the chunk that the row order and
  // the swizzle place at its LDS position.
  const __amdgpu_buffer_rsrc_t rsrc_k = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(k), 0, static_cast<int>(static_cast<int64_t>(n_pad) * d * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_v = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vt), 0, static_cast<int>(static_cast<int64_t>(n_pad) * d * 2), 0x00020000);
  uint32_t k_voff[kPieces], v_voff[kPieces];
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int kr = 4 * (kWaves * i + wave) + (lane >> 4);     // LDS row of the K tile
    const int kc = (lane & 15) ^ (kr & 15);
    k_voff[i] = static_cast<uint32_t>((key_of_row(kr) * d + head * kDh + kc * 8) * 2);
    const int vr = 8 * (kWaves * i + wave) + (lane >> 3);     // dim row of the V^T tile
    const int vc = (lane & 7) ^ v_swz(vr);
    v_voff[i] = static_cast<uint32_t>(((static_cast<int64_t>(head) * kDh + vr) * n_pad + vc * 8) * 2);
  }
  auto issue_tile = [&](int kb, int stage) {
    uint8_t* sk = smem + stage * kTile;
    uint8_t* sv = smem + kVBase + stage * kTile;
    const uint32_t ko = static_cast<uint32_t>(kb) * kBK * static_cast<uint32_t>(d) * 2;
    const uint32_t vo = static_cast<uint32_t>(kb) * kBK * 2;
#pragma unroll
    for (int i = 0; i < kPieces; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_k, (lds_ptr)(sk + (kWaves * i + wave) * 1024), 16, k_voff[i], ko, 0, 0);
#pragma unroll
    for (int i = 0; i < kPieces; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_v, (lds_ptr)(sv + (kWaves * i + wave) * 1024), 16, v_voff[i], vo, 0, 0);
  };

  // Per-lane LDS read offsets, fixed for the whole key loop (stage and block offsets are
  // immediates): K rows li (+32) at chunk 2s + hi, V^T rows li (+32 db) at chunk 2j + hi.
  int k_rd[8], v_rd[4];
#pragma unroll
  for (int s = 0; s < 8; ++s) k_rd[s] = li * 256 + (((2 * s + hi) ^ (li & 15)) << 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) v_rd[j] = li * 128 + (((2 * j + hi) ^ v_swz(li)) << 4);

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // running max in base-2 exponent units, partial sum
  const float c = 1.4426950408889634f / sqrtf(static_cast<float>(kDh));
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};


  auto tile = [&]<int kStage, bool kTail>(int kb) {
    if (kb + 1 < t1) issue_tile(kb + 1, kStage ^ 1);
    const uint8_t* sk = smem + kStage * kTile;
    const uint8_t* sv = smem + kVBase + kStage * kTile;

    // S^T: sacc[kh] element 4b + r holds key 32kh + 16(b >> 1) + 8hi + 4(b & 1) + r of the tile.
    // The two 32-key halves alternate, so no MFMA waits on the one just issued.
    const f32x16 zero = {};
    f32x16 sacc[2] = {zero, zero};
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(sk + kh * 8192 + k_rd[s]));
        sacc[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kh], 0, 0, 0);
      }
    if constexpr (kTail) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int b = e >> 2;
          const int key = kb * kBK + 32 * kh + 16 * (b >> 1) + 8 * hi + 4 * (b & 1) + (e & 3);
          if (key >= n) sacc[kh][e] = -INFINITY;
        }
    }

    // Online softmax in base-2 units with the score scale folded into the exponent's FMA. The
    // probabilities are first taken against the running max as it stands; only when some
    // query's tile sum leaves (0, 2^16] (the first tile, where the max is -inf, or scores that
    // outgrew the max) is the tile max formed, O and the sum rescaled and the tile redone.
    bf16x8 pf[4];
    auto probs = [&](float& lt) {
      // pf[j] element e is key 16j + 8hi + e, built from bfloat16 pairs; the sum is taken over
      // the same bfloat16 values that enter the product.
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x2 pp[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int b = 2 * (j & 1) + (t >> 1);
          const int e0 = 4 * b + 2 * (t & 1);
          pp[t] = bf16x2{static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sacc[j >> 1][e0], c, -m_run))),
                         static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sacc[j >> 1][e0 + 1], c, -m_run)))};
          lt = __builtin_amdgcn_fdot2_f32_bf16(pp[t], ones, lt, false);
        }
        pf[j] = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                        __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    float lt = 0.f;
    probs(lt);
    if (__ballot(!(lt <= kSpecMax))) {  // also true for inf and NaN sums
      float mx = -INFINITY;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kh][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
      lt = 0.f;
      probs(lt);
    }
    l_run += lt;

    // O^T[dim][query] += V^T P^T.
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(sv + db * 4096 + v_rd[j]));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[j], oacc[db], 0, 0, 0);
      }

    // Tile kb+1 has landed (own loads) and every wave is done with tile kb's stage.
    if (kb + 1 < t1) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  // Tiles t0 .. t1-1; only the sequence's last tile can be ragged.
  const int tail = (t1 == plan.ktiles && n % kBK != 0) ? 1 : 0;
  const int nfull = t1 - t0 - tail;
  issue_tile(t0, 0);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  int i = 0;
  for (; i + 2 <= nfull; i += 2) {
    tile.template operator()<0, false>(t0 + i);
    tile.template operator()<1, false>(t0 + i + 1);
  }
  if (i < nfull) {
    tile.template operator()<0, false>(t0 + i);
    if (tail) tile.template operator()<1, true>(t0 + i + 1);
  } else if (tail) {
    tile.template operator()<0, true>(t0 + i);
  }

  const float l = l_run + __shfl_xor(l_run, 32, 64);
  if (slot >= 0) {
    // Partial result of a key piece: unnormalised O (fp32, [query][dim]), lazy max, row sum.
    float* rec = part + static_cast<size_t>(slot) * (attn_part_bytes(kBQ) / 4);
    const int ql = wave * 32 + li;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        *reinterpret_cast<f32x4*>(rec + ql * kDh + 32 * db + 8 * b + 4 * hi) =
            f32x4{oacc[db][4 * b + 0], oacc[db][4 * b + 1], oacc[db][4 * b + 2], oacc[db][4 * b + 3]};
    if (hi == 0) {
      rec[kBQ * kDh + ql] = m_run;
      rec[kBQ * kDh + kBQ + ql] = l;
    }
    return;
  }
  const float inv = 1.0f / l;
  if (qrow < n) {
    uint16_t* op = o + qrow * d + head * kDh;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int dim = 32 * db + 8 * b + 4 * hi;
        const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16_bits(oacc[db][4 * b + 0] * inv)) |
                            (static_cast<uint32_t>(f32_to_bf16_bits(oacc[db][4 * b + 1] * inv)) << 16);
        const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16_bits(oacc[db][4 * b + 2] * inv)) |
                            (static_cast<uint32_t>(f32_to_bf16_bits(oacc[db][4 * b + 3] * inv)) << 16);
        if (o_tiled)  // 256-row x 32-column slabs (slab_offset); 4 dims stay inside one chunk
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(o) + slab_offset(qrow, head * kDh + dim, d)) = u32x2{w0, w1};
        else
          *reinterpret_cast<u32x2*>(op + dim) = u32x2{w0, w1};
      }
  }
}

__global__ __launch_bounds__(512, 1) void attn_mfma8_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ vt,
                                                            uint16_t* __restrict__ o, int n, int n_pad,
                                                            int n_heads, AttnPlan plan, int full_grid,
                                                            int o_tiled, float* __restrict__ part) {
  attn_body<8>(q, k, vt, o, n, n_pad, n_heads, plan, full_grid, o_tiled, part);
}

// Merges the key pieces of the last round's items: with M the largest piece max, O = sum_p O_p
// 2^(m_p - M) divided by sum_p l_p 2^(m_p - M). One thread per (query, 8 dims); a workgroup
// covers 16 queries of one item.
template <int kBQ>
__global__ __launch_bounds__(256) void attn_combine_kernel(uint16_t* __restrict__ o,
                                                           const float* __restrict__ part, int n,
                                                           int n_heads, AttnPlan plan, int o_tiled) {
  constexpr size_t kRec = attn_part_bytes(kBQ) / 4;
  const int r = blockIdx.x / (kBQ / 16);
  const int item = plan.full_items + r;
  const int head = item / plan.qblocks, qb = item % plan.qblocks;
  const int ql = (blockIdx.x % (kBQ / 16)) * 16 + (threadIdx.x >> 4);
  const int dim = 8 * (threadIdx.x & 15);
  const int64_t qrow = static_cast<int64_t>(qb) * kBQ + ql;
  if (qrow >= n) return;
  const int64_t d = static_cast<int64_t>(n_heads) * kDh;
  const float* rec0 = part + static_cast<size_t>(r) * plan.pieces * kRec;
  float mmax = -INFINITY;
  for (int p = 0; p < plan.pieces; ++p) mmax = fmaxf(mmax, rec0[p * kRec + kBQ * kDh + ql]);
  float lsum = 0.f;
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < plan.pieces; ++p) {
    const float* rec = rec0 + p * kRec;
    const float w = __builtin_amdgcn_exp2f(rec[kBQ * kDh + ql] - mmax);
    lsum = fmaf(rec[kBQ * kDh + kBQ + ql], w, lsum);
    a0 += *reinterpret_cast<const f32x4*>(rec + ql * kDh + dim) * w;
    a1 += *reinterpret_cast<const f32x4*>(rec + ql * kDh + dim + 4) * w;
  }
  const float inv = 1.0f / lsum;
  u32x4 packed;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    packed[t] = static_cast<uint32_t>(f32_to_bf16_bits(a0[2 * t] * inv)) |
                (static_cast<uint32_t>(f32_to_bf16_bits(a0[2 * t + 1] * inv)) << 16);
    packed[2 + t] = static_cast<uint32_t>(f32_to_bf16_bits(a1[2 * t] * inv)) |
                    (static_cast<uint32_t>(f32_to_bf16_bits(a1[2 * t + 1] * inv)) << 16);
  }
  const int64_t col = static_cast<int64_t>(head) * kDh + dim;
  if (o_tiled)  // 8 dims = one 16-byte chunk of a slab row
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(o) + slab_offset(qrow, col, d)) = packed;
  else
    *reinterpret_cast<u32x4*>(o + qrow * d + col) = packed;
}

template <int DH>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ q,
                                                      const float* __restrict__ k,
                                                      const float* __restrict__ vt,
                                                      float* __restrict__ o, int n, int n_pad,
                                                      int n_heads) {
  const int head = blockIdx.y;
  const int64_t qi = static_cast<int64_t>(blockIdx.x) * 64 + threadIdx.x;
  const int64_t d = static_cast<int64_t>(n_heads) * DH;
  const int64_t qr = qi < n ? qi : n - 1;
  float qv[DH], acc[DH];
  const float scale = 1.0f / sqrtf(static_cast<float>(DH));
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    qv[c] = q[qr * d + head * DH + c] * scale;
    acc[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j < n; ++j) {
    const float* kj = k + static_cast<int64_t>(j) * d + head * DH;
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < DH; ++c) s = fmaf(qv[c], kj[c], s);
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);
    const float pj = expf(s - m_new);
    l = fmaf(l, alpha, pj);
    m = m_new;
    const float* vj = vt + static_cast<int64_t>(head) * DH * n_pad + j;
#pragma unroll
    for (int c = 0; c < DH; ++c) acc[c] = fmaf(pj, vj[static_cast<int64_t>(c) * n_pad], acc[c] * alpha);
  }
  if (qi < n) {
#pragma unroll
    for (int c = 0; c < DH; ++c) o[qi * d + head * DH + c] = acc[c] / l;
  }
}

}  // namespace

int device_cu_count() {
  // The compute-unit count of each device, queried once per device (thread-safe).
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static int cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  });
  return cus[dev];
}

int attention_slots(int requested) {
  const int cap = kAttnMaxPieceQueries / kAttnQueries;
  if (requested > 0) return requested < cap ? requested : cap;
  // One eight-wave workgroup per CU (two waves per SIMD).
  const int cus = device_cu_count();
  return cus < cap ? cus : cap;
}

AttnPlan attention_plan(int64_t n_tokens, int n_heads, int slots) {
  AttnPlan p;
  const int n = static_cast<int>(n_tokens);
  p.bq = kAttnQueries;
  p.qblocks = (n + p.bq - 1) / p.bq;
  p.items = p.qblocks * n_heads;
  p.ktiles = (n + kBK - 1) / kBK;
  p.full_items = p.items;
  p.rem = 0;
  p.pieces = 1;
  p.tiles = p.ktiles;
  const int rounds = p.items / slots, rem = p.items - rounds * slots;
  int pieces = rem > 0 ? slots / rem : 1;
  if (pieces > p.ktiles) pieces = p.ktiles;
  if (pieces >= 2) {
    p.tiles = (p.ktiles + pieces - 1) / pieces;
    p.pieces = (p.ktiles + p.tiles - 1) / p.tiles;
    p.rem = rem;
    p.full_items = rounds * slots;
  }
  return p;
}

size_t attention_ws_bytes(int act, int64_t n_tokens, int n_heads, int slots) {
  if (act != H3X_BF16 || n_tokens < 1) return 0;
  const AttnPlan p = attention_plan(n_tokens, n_heads, slots);
  return static_cast<size_t>(p.rem) * p.pieces * attn_part_bytes(p.bq);
}

hipError_t launch_attention(int act, int64_t n_tokens, int64_t n_pad, int n_heads, int head_dim,
                            const void* q, const void* k, const void* vt, void* o, int o_tiled,
                            int slots, void* ws, hipStream_t s) {
  if (n_tokens == 0) return hipSuccess;
  const int n = static_cast<int>(n_tokens), np = static_cast<int>(n_pad);
  if (act == H3X_BF16) {
    const AttnPlan plan = attention_plan(n_tokens, n_heads, slots);
    const int full_grid = (plan.full_items + 7) / 8 * 8;
    const int grid = full_grid + plan.rem * plan.pieces;
    const uint16_t *qq = static_cast<const uint16_t*>(q), *kk = static_cast<const uint16_t*>(k);
    const uint16_t* vv = static_cast<const uint16_t*>(vt);
    uint16_t* oo = static_cast<uint16_t*>(o);
    float* pp = static_cast<float*>(ws);
    attn_mfma8_kernel<<<grid, 512, 0, s>>>(qq, kk, vv, oo, n, np, n_heads, plan, full_grid, o_tiled, pp);
    if (plan.rem > 0) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      attn_combine_kernel<kAttnQueries><<<plan.rem * (kAttnQueries / 16), 256, 0, s>>>(oo, pp, n, n_heads, plan, o_tiled);
    }
  } else {
    dim3 grid(static_cast<unsigned>((n + 63) / 64), static_cast<unsigned>(n_heads));
    if (head_dim == 64)
      attn_f32_kernel<64><<<grid, 64, 0, s>>>(static_cast<const float*>(q),
                                              static_cast<const float*>(k),
                                              static_cast<const float*>(vt),
                                              static_cast<float*>(o), n, np, n_heads);
    else
      attn_f32_kernel<128><<<grid, 64, 0, s>>>(static_cast<const float*>(q),
                                               static_cast<const float*>(k),
                                               static_cast<const float*>(vt),
                                               static_cast<float*>(o), n, np, n_heads);
  }
  return hipGetLastError();
}

}  // namespace h3x
