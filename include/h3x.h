/*
 * h3x.h -- C ABI of the h3x DiT denoiser hot path for AMD Instinct MI355X (gfx950).
 *
 * The library computes, on one GPU, the denoiser forward pass of a dense single-stream omni
 * transformer over one joint video + audio + text token sequence, the horizontal token-pair
 * reduction of the middle blocks, and the flow-matching Euler step with whole-velocity reuse.
 * The method is that of the h3.c engine for MiniMax H3 as described on the pages about it:
 *   - mobbang.com, section "MiniMax H3：视频与音轨一起生成的开源模型": dense single-stream
 *     omni transformer, video and audio generated together;
 *   - siami.tw, section "技術亮點 › 1. 完整的 Metal 原生堆疊": a DiT forward module and a
 *     separate denoising-schedule module;
 *   - siami.tw, section "速度與品質的可調旋鈕", control table: --steps, --reuse (20 / 11 / 8
 *     fresh DiT evaluations at 20 steps), --layers, --token-reduction;
 *   - jdon.com, section "330亿参数是什么概念": fused kernels, activation-buffer reuse, token
 *     reduction by pairing adjacent video tokens;
 *   - 21cto.com, section "M5 Max 生产环境实测数据", item 4, and siami.tw, "2. 數據會說話":
 *     int8 weights for the MLP, QKV and attention-output projections.
 * The pages print no formula; the readings this library implements are stated per function.
 *
 * Conventions (all entry points):
 *   - Pointers named "dev" are device (HBM) pointers on the current HIP device; all others are
 *     host pointers read only during the call. The caller owns every buffer. The library never
 *     allocates device memory and never synchronises the stream.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued asynchronously.
 *   - Every argument is validated before the first launch: a call that returns an error has
 *     enqueued nothing. Launch failures return H3X_EHIP. Faults inside kernels surface at the
 *     caller's next synchronisation. Nothing is thrown and nothing aborts across the ABI.
 *   - h3x_last_error() returns a thread-local message for the last failed call on the thread.
 *   - Matrices are row-major; "[r x c]" means r rows of c contiguous elements.
 *   - Token rows are ordered video, audio, text. Video row (t*H + y)*W + x is latent frame t,
 *     row y, column x. In a merged geometry, video row (t*H + y)*(W/2) + m stands for the
 *     horizontal pair x = 2m, 2m+1.
 */
#ifndef H3X_H
#define H3X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define H3X_ABI_VERSION 4

typedef enum {
  H3X_OK = 0,
  H3X_EINVAL = 1,     /* an argument is out of range or inconsistent */
  H3X_ENOTSUP = 2,    /* valid, but a shape/dtype combination the library has no kernel for */
  H3X_EWORKSPACE = 3, /* workspace smaller than the matching *_workspace_bytes() */
  H3X_EHIP = 4        /* a HIP launch or runtime call failed */
} h3x_status;

/* H3X_I8A8 (weights only): the int8 weights of H3X_I8 (same codes and scales, another packed
 * layout) multiplied by int8 activations: every projection input (the normalised rows, the
 * attention output and the SwiGLU product), as stored in bfloat16, is quantised per row with a
 * float32 scale (a = max |x|; inv = 127 / a and s = a / 127 as IEEE float32 divisions;
 * q = clamp(rint(x * inv), -127, 127); a == 0 or an infinite inv gives s = 0 and zero codes),
 * the products are summed exactly in int32 and scaled by s_row * s_col in float32. Pages:
 * jdon.com "选配还是选速" (an experimental int8 FC2 with one activation scale per row) and the
 * W8A8 remark on arex-research.com, "一个 MiniMax 工程师的 Redis 启蒙"; here applied to all four
 * projections. */
typedef enum { H3X_F32 = 0, H3X_BF16 = 1, H3X_I8 = 2, H3X_I8A8 = 3 } h3x_dtype;

typedef enum {
  H3X_W_QKV = 0,     /* [3d x d]: rows Q | K | V, each head-major */
  H3X_W_OUT = 1,     /* [d x d] attention-output projection */
  H3X_W_GATE_UP = 2, /* [2F x d]: rows 0..F-1 = W_gate, rows F..2F-1 = W_up */
  H3X_W_DOWN = 3     /* [d x F] MLP down projection ("FC2") */
} h3x_wkind;

/* Shape and numeric types of one block. Supported combinations:
 *   act F32  + weight F32  : head_dim 64 or 128, d_model % 64 == 0, ffn_inner % 64 == 0;
 *   act BF16 + weight BF16 or I8 : head_dim 128, d_model % 256 == 0, ffn_inner % 128 == 0;
 *   act BF16 + weight I8A8       : as BF16, and d_model <= 8192, ffn_inner <= 32768.
 * d_model must equal n_heads * head_dim, d_model <= 65536 and ffn_inner <= 262144 (one GEMM
 * operand panel of 256 rows is addressed with 32-bit offsets). norm_eps > 0 (1e-6),
 * rope_theta > 1 (10000). Row and token counts of every call are at most 2^26. */
typedef struct {
  int32_t d_model, n_heads, head_dim, ffn_inner;
  int32_t act;    /* h3x_dtype of activations: H3X_F32 or H3X_BF16 */
  int32_t weight; /* h3x_dtype of weights: H3X_F32, H3X_BF16, H3X_I8 or H3X_I8A8 */
  float norm_eps;
  float rope_theta;
} h3x_block_cfg;

/* Latent geometry of the joint sequence. frames x grid_h x grid_w video tokens (halved when
 * merged == 1; grid_w must then be even), then n_audio, then n_text tokens. Sizes are
 * non-negative, each grid extent at most 2^20 and the sequence at most 2^26 tokens (else
 * H3X_EINVAL). With bfloat16
 * activations the entry points that run attention return H3X_ENOTSUP when
 * round_up(N, 256) * d_model * 2 reaches 2^31 bytes (the K and V^T matrices are addressed with
 * 32-bit offsets): about 174k tokens at d_model 6144. */
typedef struct {
  int32_t frames, grid_h, grid_w, n_audio, n_text;
  int32_t merged;
} h3x_geom;

/* Packed weights of one block (device pointers, produced by h3x_pack_weights_bf16 /
 * h3x_pack_weights_f32 or h3x_pack_int8_weights). For H3X_I8 and H3X_I8A8 the s_* pointers hold
 * one bfloat16 scale per packed row; for F32 / BF16 weights they must be NULL. */
typedef struct {
  const void *qkv, *out, *gate_up, *down;
  const void *s_qkv, *s_out, *s_gate_up, *s_down;
} h3x_block_weights;

/* One sampler step (host struct). Zero-initialised variant fields give the plain step. */
typedef struct {
  int32_t step, n_steps, reuse;     /* 0 <= step < n_steps, reuse >= 1 */
  float sigma, sigma_next;          /* finite; the update uses float32(sigma_next - sigma) */
  int32_t n_blocks;                 /* active blocks, >= 1 */
  const h3x_block_weights *blocks;  /* host array [n_blocks] of device weight pointers */
  const float *mod;                 /* dev [n_blocks x 6 x d] float32 modulation of this step */
  int32_t tr_first, tr_last;        /* token reduction over blocks tr_first..tr_last (0-based,
                                       inclusive); -1, -1 = off */
  /* ---- variants (ABI 2) */
  int32_t cond_first, cond_last;    /* fixed condition rows: the video rows of the first
                                       cond_first and last cond_last latent frames are left
                                       unchanged by the update (the DiT sees them as usual);
                                       cond_first + cond_last <= frames. Pages: siami.tw
                                       "專業音訊" (fixed condition rows in the DiT). */
  void *v_prev;                     /* dev [(Nv + Na) x d] act type, or NULL: on fresh steps it
                                       receives the previous content of v_cache */
  float extrap;                     /* reused steps: v = fmaf(extrap, float32(v_cache - v_prev),
                                       v_cache) (linear extrapolation in sigma; 0 = hold the last
                                       fresh velocity; nonzero needs v_prev). Pages: mobbang.com
                                       / jdon.com list of tested schedules. */
  int32_t core_reuse;               /* 0 or 1 = off; k >= 2: blocks core_first..core_last run
                                       only on steps fresh for period k (h3x_step_is_fresh); on
                                       the others they are replaced by x + core_delta. Needs
                                       reuse == 1 (the two are exclusive: siami.tw control
                                       table, row "核心復用"). With token reduction the core
                                       must lie wholly inside tr_first..tr_last or wholly
                                       outside it (else H3X_EINVAL). */
  int32_t core_first, core_last;    /* 0 <= core_first <= core_last < n_blocks */
  float *core_delta;                /* dev [(Nv + Na + Nt) x d] float32: written on core-fresh
                                       steps (x after the core - x before), read on the others;
                                       a core inside the reduced blocks uses only the first
                                       (Nv / 2 + Na + Nt) x d values (merged rows) */
} h3x_step;

int32_t h3x_abi_version(void);
const char *h3x_status_string(h3x_status s);
const char *h3x_last_error(void);

/* Number of tokens of a geometry (video rows halved when merged); -1 if invalid. */
int64_t h3x_geom_tokens(const h3x_geom *geom);

/* ------------------------------------------------------------------ weight packing
 * Packed row order (all weight types): rows of the source are kept whole and in order, except
 * for H3X_W_GATE_UP, whose packed row 64j + i is W_gate row 32j + i and packed row 64j + 32 + i
 * is W_up row 32j + i (i < 32), so that one 64-column output group holds the gate and up values
 * of the same 32 inner features.
 * Packed storage: F32 weights are row-major [rows x cols]. BF16 weights and I8 codes are stored
 * as slabs of 256 packed rows x 32 columns, slab (r / 256, c / 32) at byte offset
 * ((r / 256) * (cols / 32) + c / 32) * S with S = 16384 (BF16) or 8192 (I8); inside a slab,
 * packed row rr = r % 256 holds 64 (BF16) or 32 (I8) bytes made of 16-byte chunks, chunk q of
 * the row stored at position q ^ ((rr >> 2) & 3) (BF16) or q ^ ((rr >> 3) & 1) (I8). This is
 * the order in which the matrix-core GEMM keeps one 32-wide K step of a 256-row tile in LDS.
 * I8A8 codes use the BF16 byte layout with 64 codes per slab row: slab (r / 256, c / 64) at
 * ((r / 256) * (cols / 64) + c / 64) * 16384, row rr holding 64 bytes in four 16-byte chunks
 * placed at q ^ ((rr >> 2) & 3) (one 64-wide K step of the int8 GEMM).
 * `rows` x `cols` is the shape of the master (source) weight and must be the shape `kind` has
 * for cfg: H3X_W_QKV 3d x d, H3X_W_OUT d x d, H3X_W_GATE_UP 2F x d, H3X_W_DOWN d x F (the
 * redundant pair is a check on the caller's tensor: a mismatch is H3X_EINVAL, and 0 bytes here).
 * Packed size in bytes for the cfg's weight type (I8, I8A8: the codes; scales are
 * h3x_packed_scale_count() bfloat16 values in packed row order). */
size_t h3x_packed_weight_bytes(const h3x_block_cfg *cfg, int32_t kind, int64_t rows, int64_t cols);
int64_t h3x_packed_rows(const h3x_block_cfg *cfg, int32_t kind);
int64_t h3x_packed_scale_count(const h3x_block_cfg *cfg, int32_t kind);

/* Pack one bfloat16 master weight w (dev [rows x cols] bfloat16, cfg->weight H3X_BF16) into
 * `packed` (dev, h3x_packed_weight_bytes bytes, not overlapping w) in the slab order above: a
 * pure permutation, bit-exact. The weights are laid out once, ahead of every run, in the order
 * the matrix cores read them, so that the block never re-arranges them (the pages' engine keeps
 * its weights where they are loaded instead of copying them: jdon.com,
 * "330亿参数是什么概念"). h3x_pack_weights_f32 is the same for the float32 configuration
 * (cfg->weight H3X_F32, row-major packed rows). */
h3x_status h3x_pack_weights_bf16(const h3x_block_cfg *cfg, int32_t kind, const void *w,
                                 int64_t rows, int64_t cols, void *packed, void *stream);
h3x_status h3x_pack_weights_f32(const h3x_block_cfg *cfg, int32_t kind, const void *w,
                                int64_t rows, int64_t cols, void *packed, void *stream);

/* Per-output-channel symmetric int8 quantisation of a bfloat16 master weight (dev [rows x cols])
 * into int8 codes `q_packed` (dev, packed row order, h3x_packed_weight_bytes bytes) and
 * bfloat16 scales `scale_bf16` (dev, one per packed row). Per source row r: a = max|W[r,:]|;
 * a == 0 gives scale 0 and zero codes; otherwise s = bf16(a / 127) (IEEE float32 division,
 * round to nearest even, then round to bfloat16); s == 0 (underflow) gives zero codes; else
 * q = clamp(rint(W / s), -127, 127) with an IEEE float32 division by the stored s. Bit-exact
 * (no choice is left to the kernel). Pages: 21cto.com "M5 Max 生产环境实测数据" item 4;
 * siami.tw "2. 數據會說話". cfg->weight must be H3X_I8 or H3X_I8A8 (cfg->act H3X_BF16); the two
 * differ only in the order in which the codes are stored. */
h3x_status h3x_pack_int8_weights(const h3x_block_cfg *cfg, int32_t kind, const void *w_bf16,
                                 int64_t rows, int64_t cols, void *q_packed, void *scale_bf16,
                                 void *stream);

/* ------------------------------------------------------------------ one block
 * x (dev [N x d], act type, in place): x1 = x + gate1 * (attn(rope(qkv(y))) @ W_out^T) with
 * y = x / sqrt(mean(x^2) + eps) * (1 + scale1) + shift1; x2 = x1 + gate2 * (silu(y2 @ W_g^T) *
 * (y2 @ W_u^T)) @ W_down^T with y2 the same modulated RMSNorm of x1 (shift2, scale2).
 * Attention is softmax(q k^T / sqrt(Dh)) v per head over all N tokens (no mask). 3D RoPE turns
 * q and k of video rows: head dims split into (t | y | x) chunks of Dh/4, 3Dh/8, 3Dh/8; pair
 * (2k, 2k+1) of a chunk of size D turns by pos * theta^(-2k/D); merged tokens sit at x = 2m+0.5;
 * audio and text rows are not turned. mod (dev [6 x d] float32): shift1, scale1, gate1,
 * shift2, scale2, gate2. ws (dev) must hold h3x_block_workspace_bytes(cfg, geom) bytes; its
 * contents on entry are ignored and on return undefined. (With H3X_I8 weights the workspace
 * also receives each weight matrix widened to bfloat16 just before its product: the codes are
 * small integers, so the widening is exact and the scales are applied afterwards.) */
size_t h3x_block_workspace_bytes(const h3x_block_cfg *cfg, const h3x_geom *geom);
h3x_status h3x_dit_block_forward(const h3x_block_cfg *cfg, const h3x_geom *geom,
                                 const h3x_block_weights *w, const float *mod, void *x,
                                 void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): h3x_dit_block_forward with the workspace taken from a
 * device array inside the library, H3X_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held from the
 * library's load until the process ends. The caller still owns x, mod and the weights. Nothing
 * is allocated and no part of the array needs to start at zero (every region is written before
 * it is read). A block whose h3x_block_workspace_bytes exceeds the array returns
 * H3X_EWORKSPACE before anything is enqueued. All calls on one GPU share its array: calls that
 * overlap in time on that GPU (different streams, or several threads) race and give undefined
 * results; calls ordered on one stream are safe. */
#define H3X_NOALLOC_SCRATCH_BYTES (64ull << 20)
h3x_status h3x_dit_block_forward_noalloc(const h3x_block_cfg *cfg, const h3x_geom *geom,
                                         const h3x_block_weights *w, const float *mod, void *x,
                                         void *stream);

/* ------------------------------------------------------------------ one sampler step
 * 1 if step i of n runs the DiT (i % reuse == 0 or i == n - 1), 0 if it reuses the cached
 * velocity, -1 on invalid arguments. Pages: siami.tw control table, row "整體 denoiser 復用". */
int32_t h3x_step_is_fresh(int32_t step, int32_t n_steps, int32_t reuse);

/* Sigma grids (host): sigma_out[0..n_steps] (host float array), each value computed in double
 * and rounded once to float. H3X_SCHED_LINEAR: 1 - i/n. H3X_SCHED_POWER: (1 - i/n)^param
 * (2, 3: the quadratic and cubic warps). H3X_SCHED_LINEAR_TERMINAL: 1 - i/param for i < n
 * (param = a base step count >= n), then 0: a few-step run on a longer linear base grid with
 * one terminal step. Pages: mobbang.com / jdon.com (tested schedules), siami.tw control-table
 * section (the few-step runs' linear base grid with a single terminal endpoint). */
typedef enum { H3X_SCHED_LINEAR = 0, H3X_SCHED_POWER = 1, H3X_SCHED_LINEAR_TERMINAL = 2 } h3x_schedule;
h3x_status h3x_sigma_schedule(int32_t kind, int32_t n_steps, double param, float *sigma_out);

/* Extrapolation weight for h3x_step.extrap: float((s - s_a) / (s_a - s_b)) in double from the
 * float sigmas of this step (s) and of the last two fresh steps (s_a after s_b). NaN if
 * s_a == s_b. */
float h3x_extrapolation_weight(float sigma, float sigma_a, float sigma_b);

/* Workspace of h3x_denoise_step: the block workspace of the unmerged geometry plus two token
 * buffers (unmerged and merged). geom must be unmerged. */
size_t h3x_step_workspace_bytes(const h3x_block_cfg *cfg, const h3x_geom *geom);

/* z (dev [(Nv + Na) x d] float32, in place): the sampler state of the video and audio rows.
 * text (dev [Nt x d], act type): fixed conditioning rows. v_cache (dev [(Nv + Na) x d], act
 * type): on fresh steps the DiT output of the video and audio rows is written here, on other
 * steps it is read. A fresh step feeds [act(z); text] through blocks 0..n_blocks-1, merging
 * video pairs by their mean before block tr_first and duplicating them back before block
 * tr_last + 1 (or after the last block). Then z <- float32(z + (sigma_next - sigma) * v),
 * rounded once, except on the fixed condition rows. The variant fields of h3x_step add
 * linear velocity extrapolation on reused steps and core reuse. geom must be unmerged; token
 * reduction needs an even grid_w. */
h3x_status h3x_denoise_step(const h3x_block_cfg *cfg, const h3x_geom *geom, const h3x_step *st,
                            float *z, const void *text, void *v_cache, void *ws,
                            size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* H3X_H */
