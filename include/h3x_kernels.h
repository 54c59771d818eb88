/*
 * h3x_kernels.h -- kernel-level entry points of libh3x: one step of the block or the sampler
 * per call, for per-kernel parity tests and per-kernel timing. Same conventions as h3x.h
 * (device pointers named "dev", caller-owned buffers, asynchronous on `stream`, validation
 * before any launch, status codes, no allocation). Row and token counts (n_rows, m, n_tokens)
 * are at most 2^26 (else H3X_EINVAL). A call with zero rows (n_rows, m) is valid, enqueues
 * nothing and does not look at its data pointers (they may be NULL).
 *
 * Internal attention layouts used by these entry points, for a sequence of N tokens and
 * Npad = N rounded up to a multiple of 256:
 *   q, k : dev [Npad x d] act type, head-major columns (head h = columns h*Dh .. h*Dh+Dh-1);
 *   vt   : dev [d x Npad] act type, the value matrix transposed (row h*Dh + j, column token).
 * Rows (columns of vt) N .. Npad-1 are written as zeros by h3x_qkv_project.
 */
#ifndef H3X_KERNELS_H
#define H3X_KERNELS_H

#include "h3x.h"

#ifdef __cplusplus
extern "C" {
#endif

/* y = x / sqrt(mean(x^2) + eps) * (1 + scale) + shift, per row of x (dev [n_rows x d], act
 * type) into y (dev, same shape and type). shift, scale: dev [d] float32. Modulated RMSNorm is a
 * reading: the pages only speak of a normalised MLP input (siami.tw, "3. 記憶體策略…"). */
h3x_status h3x_norm_mod(const h3x_block_cfg *cfg, int64_t n_rows, const void *x,
                        const float *shift, const float *scale, void *y, void *stream);

/* The per-geometry 3D RoPE cos/sin table that h3x_qkv_project reads (dev float32 pairs,
 * h3x_rope_table_bytes bytes). Built once per geometry and reused by every block. */
size_t h3x_rope_table_bytes(const h3x_block_cfg *cfg, const h3x_geom *geom);
h3x_status h3x_rope_table(const h3x_block_cfg *cfg, const h3x_geom *geom, void *table,
                          void *stream);

/* QKV projection of y (dev [N x d]) with packed W_qkv (and int8 scales for I8 configs, else
 * NULL), 3D RoPE on the q and k of video rows, written to q, k, vt in the layouts above. */
h3x_status h3x_qkv_project(const h3x_block_cfg *cfg, const h3x_geom *geom, const void *y,
                           const void *w_qkv, const void *s_qkv, const void *rope_table,
                           void *q, void *k, void *vt, void *stream);

/* o (dev [N x d] act type) = per-head softmax(q k^T / sqrt(Dh)) v over all N keys.
 * bfloat16: the work (256 queries of one head per workgroup) is planned for `slots` workgroups
 * running at once (0 = one per compute unit of the current device, at most 512); the queries
 * of a last, partly filled round are split over key ranges whose partial results go to ws (dev,
 * h3x_attention_workspace_bytes for the same arguments, 0 when nothing is split) and are merged
 * by a second kernel. float32 needs no workspace. */
size_t h3x_attention_workspace_bytes(const h3x_block_cfg *cfg, int64_t n_tokens, int32_t slots);
h3x_status h3x_attention(const h3x_block_cfg *cfg, int64_t n_tokens, const void *q,
                         const void *k, const void *vt, void *o, int32_t slots, void *ws,
                         size_t ws_bytes, void *stream);

/* x (dev [M x d] act type, in place) += gate (dev [d] float32) * (a @ W^T), for kind H3X_W_OUT
 * (a: [M x d]) or H3X_W_DOWN (a: [M x F]); w packed, s its int8 scales or NULL. */
h3x_status h3x_linear_residual(const h3x_block_cfg *cfg, int32_t kind, int64_t m, const void *a,
                               const void *w, const void *s, const float *gate, void *x,
                               void *stream);

/* h (dev [M x F] act type) = silu(y2 @ W_gate^T) * (y2 @ W_up^T) with the packed gate/up
 * weight (and int8 scales or NULL). */
h3x_status h3x_linear_swiglu(const h3x_block_cfg *cfg, int64_t m, const void *y2,
                             const void *w_gate_up, const void *s_gate_up, void *h,
                             void *stream);

/* out (dev [M x packed_rows] float32) = a @ W_packed^T (times the int8 scales): the plain
 * product, in packed column order, for checking the contraction alone. */
h3x_status h3x_linear_f32out(const h3x_block_cfg *cfg, int32_t kind, int64_t m, const void *a,
                             const void *w, const void *s, float *out, void *stream);

/* W8A8 activations (the per-row rule documented with H3X_I8A8 in h3x.h). Codes are stored as
 * slabs of 256 rows x 64 codes in the I8A8 weight layout (slab (r / 256, c / 64) at
 * ((r / 256) * (cols / 64) + c / 64) * 16384, row rr = r % 256 holding four 16-byte chunks at
 * q ^ ((rr >> 2) & 3)); rows m .. round_up(m, 256) - 1 of a slab are left as they were.
 * quant_rows: a (dev [m x cols] bfloat16, row-major) -> q (dev, round_up(m, 256) * cols bytes),
 * s (dev float32 [m]); 0 < cols <= 32768, cols % 64 == 0.
 * norm_mod_quant: the modulated RMSNorm of h3x_norm_mod (bfloat16, cfg->weight I8A8), rounded to
 * bfloat16, then quantised as above (cols = d_model). */
h3x_status h3x_quant_rows(int64_t m, int64_t cols, const void *a, void *q, float *s, void *stream);
h3x_status h3x_norm_mod_quant(const h3x_block_cfg *cfg, int64_t n_rows, const void *x,
                              const float *shift, const float *scale, void *q, float *s,
                              void *stream);

/* out (dev [m x packed_rows] float32)[r][c] = float(sum_k qa[r][k] w[c][k]) * sa[r] * sw[c]
 * for an I8A8 cfg: qa, sa as written by h3x_quant_rows (qa holding round_up(m, 256) rows, sa
 * round_up(m, 256) entries: the GEMM reads whole 256-row tiles; the values of rows past m
 * only reach discarded outputs), w and sw from h3x_pack_int8_weights. The integer sums are
 * exact. The other kernel-level projections return H3X_ENOTSUP for I8A8 configs. */
h3x_status h3x_linear_a8_f32out(const h3x_block_cfg *cfg, int32_t kind, int64_t m,
                                const void *qa, const float *sa, const void *w, const void *sw,
                                float *out, void *stream);

/* Token reduction (jdon.com, "330亿参数是什么概念"; siami.tw control table, row
 * "Token 縮減"). geom is the unmerged geometry. merge: x [N x d] -> xm [N' x d], video pair
 * (2p, 2p+1) -> row p = their mean rounded once to the act type; audio and text rows copied.
 * unmerge: xm [N' x d] -> x [N x d], merged row p written to rows 2p and 2p+1. */
h3x_status h3x_token_merge(const h3x_block_cfg *cfg, const h3x_geom *geom, const void *x,
                           void *xm, void *stream);
h3x_status h3x_token_unmerge(const h3x_block_cfg *cfg, const h3x_geom *geom, const void *xm,
                             void *x, void *stream);

/* Euler step on n_rows x d elements: z (dev float32, in place) <- float32(z + (sigma_next -
 * sigma) * v), rounded once; v dev act type. If v_copy is not NULL, v is also copied there
 * (the fresh-step velocity cache write). */
h3x_status h3x_euler(const h3x_block_cfg *cfg, int64_t n_rows, float *z, const void *v,
                     float sigma, float sigma_next, void *v_copy, void *stream);

/* Plain device copy of `bytes` bytes (multiple of 16, 16-byte aligned pointers); used to
 * calibrate hardware byte counters against a transfer of known size. */
h3x_status h3x_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Matrix-core throughput probe: one workgroup per compute unit runs `iters` (1 .. 2^32)
 * iterations of 64 MFMAs per wave (v_mfma_f32_32x32x16_bf16 for H3X_BF16,
 * v_mfma_i32_32x32x32_i8 for H3X_I8) on register operands of pseudo-random values that change
 * from one instruction to the next, with no memory traffic. *ops (host) receives the launch's
 * operation count (2 per multiply-add); out (dev, one float) is written only to keep the
 * products alive. Timing the call gives the rate the chip sustains for dense MFMA work at the
 * clock it holds under that load. */
h3x_status h3x_mfma_probe(int32_t dtype, int64_t iters, float *out, double *ops, void *stream);

/* Per-kernel timing. While enabled, every launch made by the library is bracketed by HIP
 * events on its stream. h3x_profile_end waits for the recorded events, writes at most
 * max_entries per-kernel totals and returns the number written (or -1 on error). */
typedef struct {
  char name[48];
  int32_t launches;
  double total_ms;
} h3x_kernel_time;
h3x_status h3x_profile_begin(void);
int32_t h3x_profile_end(h3x_kernel_time *out, int32_t max_entries);

#ifdef __cplusplus
}
#endif
#endif /* H3X_KERNELS_H */
