// Host-side launchers of the h3x kernels. Each enqueues exactly one kernel on `stream` and
// returns hipGetLastError() of that launch. Arguments are validated by the caller (api.cpp).
#pragma once

#include "common.h"

namespace h3x {

// Elementwise and memory-bound kernels (k_elementwise.hip).
hipError_t launch_norm_mod(int act, int64_t n_rows, int d, float eps, const void* x,
                           const float* shift, const float* scale, void* y, int out_tiled,
                           hipStream_t s);
hipError_t launch_token_merge(int act, const GeomDev& g, int d, const void* x, void* xm,
                              hipStream_t s);
hipError_t launch_token_unmerge(int act, const GeomDev& g, int d, const void* xm, void* x,
                                hipStream_t s);
// z += delta * v on every row except the fixed condition rows [0, cond_lo) and
// [cond_hi, n_video); v_prev != nullptr: v is extrapolated as fmaf(w, v - v_prev, v).
hipError_t launch_euler(int act, int64_t n_elems, int d, float* z, const void* v,
                        const void* v_prev, float w, float delta, void* v_copy, int64_t cond_lo,
                        int64_t cond_hi, int64_t n_video, hipStream_t s);
// Core reuse: op 0 delta = x, op 1 delta = x - delta, op 2 x = act(x + delta).
hipError_t launch_core(int act, int op, int64_t n_elems, void* x, float* delta, hipStream_t s);
hipError_t launch_assemble(int act, int64_t n_state, int64_t n_text, int d, const float* z,
                           const void* text, void* x, hipStream_t s);
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
// Matrix-core throughput probe (k_probe.hip): i8 selects v_mfma_i32_32x32x32_i8, else
// v_mfma_f32_32x32x16_bf16; mfma_probe_ops = operations (2 per multiply-add) of one launch.
hipError_t launch_mfma_probe(int i8, int64_t iters, float* out, hipStream_t s);
double mfma_probe_ops(int i8, int64_t iters);
hipError_t launch_rope_table(const GeomDev& g, int head_dim, float theta, float2* table,
                             int4* rowbase, hipStream_t s);
hipError_t launch_pack(int wdtype, int kind, int64_t rows, int64_t cols, const void* w,
                       void* packed, hipStream_t s);
// slab64 = 0: codes in slab_offset_i8 order (int8 weights, bfloat16 activations); 1: in
// slab_offset_q8 order (int8 weights and int8 activations).
hipError_t launch_pack_int8(int kind, int64_t rows, int64_t cols, const void* w_bf16,
                            int8_t* q, uint16_t* scale, int slab64, hipStream_t s);
// int8 weight codes (slab_offset_i8 order) widened to bfloat16 in slab_offset order, exact; the
// bf16 GEMM then multiplies them and applies the row scales given in GemmArgs.wscale.
hipError_t launch_widen_int8(int64_t rows, int64_t cols, const int8_t* q, void* w, hipStream_t s);
// Per-row int8 quantisation of bfloat16 rows (row-major [n_rows x cols]): codes q in
// slab_offset_q8 order, float32 scales qscale[n_rows]. cols % 64 == 0, cols <= 32768.
hipError_t launch_quant_rows(int64_t n_rows, int64_t cols, const void* a, int8_t* q, float* qscale,
                             hipStream_t s);
// Modulated RMSNorm (bfloat16) followed by the per-row quantisation of its bfloat16-rounded
// output: codes and scales as launch_quant_rows. d <= 8192.
hipError_t launch_norm_mod_quant(int64_t n_rows, int d, float eps, const void* x, const float* shift,
                                 const float* scale, int8_t* q, float* qscale, hipStream_t s);

// Byte offset of bf16 element (r, c) of a [rows x k] matrix stored as 256-row x 32-column slabs:
// slab (r / 256, c / 32) at ((r / 256) * (k / 32) + c / 32) * 16 KB; inside it, row rr = r % 256
// holds 64 bytes whose four 16-byte chunks are permuted by chunk ^ ((rr >> 2) & 3). This is the
// order in which the MFMA GEMM keeps an operand K step in LDS, so one K step of one 256-row tile
// is a contiguous copy. k must be a multiple of 32.
__host__ __device__ inline int64_t slab_offset(int64_t r, int64_t c, int64_t k) {
  const int64_t rr = r & 255, cc = c & 31;
  return (((r >> 8) * (k >> 5) + (c >> 5)) << 14) + rr * 64 + ((((cc >> 3) ^ ((rr >> 2) & 3))) << 4) +
         (cc & 7) * 2;
}
// Same for int8 codes: 256 x 32-byte slabs of 8 KB, two 16-byte chunks per row permuted by
// chunk ^ ((rr >> 3) & 1).
__host__ __device__ inline int64_t slab_offset_i8(int64_t r, int64_t c, int64_t k) {
  const int64_t rr = r & 255, cc = c & 31;
  return (((r >> 8) * (k >> 5) + (c >> 5)) << 13) + rr * 32 + ((((cc >> 4) ^ ((rr >> 3) & 1))) << 4) +
         (cc & 15);
}

// Same for int8 codes of the W8A8 GEMM: 256 x 64-byte slabs of 16 KB, the byte layout of the
// bfloat16 slabs (four 16-byte chunks per row permuted by chunk ^ ((rr >> 2) & 3)), so that one
// K step covers 64 codes. k must be a multiple of 64.
__host__ __device__ inline int64_t slab_offset_q8(int64_t r, int64_t c, int64_t k) {
  const int64_t rr = r & 255, cc = c & 63;
  return (((r >> 8) * (k >> 6) + (c >> 6)) << 14) + rr * 64 + ((((cc >> 4) ^ ((rr >> 2) & 3))) << 4) +
         (cc & 15);
}

// Source row of packed row p (the gate/up interleave; identity for the other kinds).
__host__ __device__ inline int64_t packed_source_row(int kind, int64_t p, int64_t rows) {
  if (kind != H3X_W_GATE_UP) return p;
  const int64_t f = rows / 2;
  const int64_t j = p / 64, i = p % 64;
  return i < 32 ? 32 * j + i : f + 32 * j + (i - 32);
}

// Contractions. Epilogue kinds of the GEMM kernels.
enum Epi : int {
  EPI_QKV = 0,    // RoPE on q, k of video rows; q, k row-major, v transposed; zero pad rows
  EPI_RESID = 1,  // x += gate * acc
  EPI_SWIGLU = 2, // h[f] = silu(acc_gate) * acc_up over the 32-row interleave
  EPI_F32 = 3     // out = acc (float32)
};

struct GemmArgs {
  const void* a;        // [m x k] act type: row-major, or slabs (a_tiled) as slab_offset();
                        // int8 codes as slab_offset_q8() for W8A8 weights
  const float* ascale;  // W8A8: float32 scale per row of a (m rounded up to 256 entries)
  int a_tiled;          // bf16 MFMA path only (always set for W8A8)
  int out_tiled;        // EPI_SWIGLU: h written as slabs instead of row-major
  const void* w;        // packed weight [n x k] (bf16, f32 or int8 codes)
  const uint16_t* wscale;  // int8 scales [n] (bfloat16) or nullptr
  int64_t m, n, k;
  int64_t m_pad;        // rows written by EPI_QKV (multiple of 256, >= m)
  // EPI_QKV
  void* q; void* kk; void* vt;
  int32_t d_model;
  GeomDev geom;
  RopeDev rope;
  // EPI_RESID
  void* x; const float* gate;
  // EPI_SWIGLU
  void* h;
  // EPI_F32
  float* out;
};

hipError_t launch_gemm(int act, int wdtype, int epi, const GemmArgs& args, hipStream_t s);
// Work split of the bfloat16 attention over `slots` concurrently resident workgroups. An item
// is bq queries of one head; items 0 .. full_items-1 run whole, in full rounds of `slots`; the
// rem items left for a last, partly empty round are cut into `pieces` key ranges of `tiles`
// 64-key tiles each, whose partial results a second kernel merges.
struct AttnPlan {
  int bq, qblocks, items, ktiles;
  int full_items, rem, pieces, tiles;
};
// Partial results of at most 2^17 queries (pieces x bq) are kept: O (fp32, 128 dims), max, sum.
constexpr int kAttnMaxPieceQueries = 1 << 17;
constexpr int kAttnQueries = 256;  // queries per workgroup of the bfloat16 attention (8 waves x 32)
constexpr size_t attn_part_bytes(int bq) { return static_cast<size_t>(bq) * (128 * 4 + 2 * 4); }
int attention_slots(int requested);  // 0 = what the current device runs at once
int device_cu_count();               // compute units of the current device (queried once per device)
AttnPlan attention_plan(int64_t n_tokens, int n_heads, int slots);
size_t attention_ws_bytes(int act, int64_t n_tokens, int n_heads, int slots);
hipError_t launch_attention(int act, int64_t n_tokens, int64_t n_pad, int n_heads, int head_dim,
                            const void* q, const void* k, const void* vt, void* o, int o_tiled,
                            int slots, void* ws, hipStream_t s);

}  // namespace h3x
