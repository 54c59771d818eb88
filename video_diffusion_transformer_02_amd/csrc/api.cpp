// C ABI of libh3x: argument validation, workspace layout, dispatch of the kernel launchers,
// error reporting and optional per-kernel event timing. No device memory is allocated here.
#include <cmath>
#include <math.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "h3x.h"
#include "h3x_kernels.h"
#include "launch.h"

using namespace h3x;

namespace {

thread_local std::string g_last_error;

h3x_status fail(h3x_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

// ---------------------------------------------------------------- per-kernel event timing
struct Rec {
  const char* name;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<Rec> g_prof_recs;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one launch with events when timing is on.
class Timed {
 public:
  Timed(const char* name, hipStream_t s) : name_(name), s_(s) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on) return;
    start_ = take_event();
    stop_ = take_event();
    if (start_ && stop_ && hipEventRecord(start_, s_) == hipSuccess) return;
    give_back();  // no timing for this launch
  }
  ~Timed() {
    if (!start_ || !stop_) return;
    const bool ok = hipEventRecord(stop_, s_) == hipSuccess;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (ok) g_prof_recs.push_back({name_, start_, stop_});
    else give_back();
  }

 private:
  // Returns the events to the pool (g_prof_mu held).
  void give_back() {
    if (start_) g_event_pool.push_back(start_);
    if (stop_) g_event_pool.push_back(stop_);
    start_ = stop_ = nullptr;
  }
  const char* name_;
  hipStream_t s_;
  hipEvent_t start_ = nullptr, stop_ = nullptr;
};

h3x_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return H3X_OK;
  return fail(H3X_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define H3X_LAUNCH(name, stream, call)                 \
  do {                                                 \
    Timed _t(name, stream);                            \
    h3x_status _st = hip_check((call), name);          \
    if (_st != H3X_OK) return _st;                     \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }
int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
int elem_bytes(int act) { return act == H3X_BF16 ? 2 : 4; }
// Weight types stored as int8 codes with one bfloat16 scale per packed row.
bool int8_weights(const h3x_block_cfg* c) { return c->weight == H3X_I8 || c->weight == H3X_I8A8; }

// ---------------------------------------------------------------- validation
h3x_status check_cfg(const h3x_block_cfg* c) {
  if (!c) return fail(H3X_EINVAL, "cfg is NULL");
  if (c->d_model <= 0 || c->n_heads <= 0 || c->head_dim <= 0 || c->ffn_inner <= 0)
    return fail(H3X_EINVAL, "cfg: sizes must be positive");
  if (static_cast<int64_t>(c->n_heads) * c->head_dim != c->d_model)
    return fail(H3X_EINVAL, "cfg: d_model != n_heads * head_dim");
  // The GEMMs address one operand panel (256 rows x K) with 32-bit buffer offsets.
  if (c->d_model > 65536 || c->ffn_inner > 262144)
    return fail(H3X_ENOTSUP, "cfg: d_model <= 65536 and ffn_inner <= 262144 supported");
  if (!(c->norm_eps > 0.f) || !isfinite(c->norm_eps)) return fail(H3X_EINVAL, "cfg: norm_eps must be > 0");
  if (!(c->rope_theta > 1.f) || !isfinite(c->rope_theta)) return fail(H3X_EINVAL, "cfg: rope_theta must be > 1");
  if (c->act != H3X_F32 && c->act != H3X_BF16) return fail(H3X_EINVAL, "cfg: act must be F32 or BF16");
  if (c->weight != H3X_F32 && c->weight != H3X_BF16 && c->weight != H3X_I8 && c->weight != H3X_I8A8)
    return fail(H3X_EINVAL, "cfg: weight must be F32, BF16, I8 or I8A8");
  if (c->act == H3X_F32) {
    if (c->weight != H3X_F32) return fail(H3X_ENOTSUP, "cfg: F32 activations need F32 weights");
    if (c->head_dim != 64 && c->head_dim != 128) return fail(H3X_ENOTSUP, "cfg: F32 path supports head_dim 64 or 128");
    if (c->d_model % 64 || c->ffn_inner % 64) return fail(H3X_ENOTSUP, "cfg: F32 path needs d_model, ffn_inner % 64 == 0");
  } else {
    if (c->weight == H3X_F32) return fail(H3X_ENOTSUP, "cfg: BF16 activations need BF16 or I8 weights");
    if (c->head_dim != 128) return fail(H3X_ENOTSUP, "cfg: BF16 path supports head_dim 128");
    if (c->d_model % 256 || c->ffn_inner % 128)
      return fail(H3X_ENOTSUP, "cfg: BF16 path needs d_model % 256 == 0 and ffn_inner % 128 == 0");
    // W8A8: the fused norm-quantise kernel holds a row of <= 8192 values in registers, the
    // quantise kernel one of <= 32768.
    if (c->weight == H3X_I8A8 && (c->d_model > 8192 || c->ffn_inner > 32768))
      return fail(H3X_ENOTSUP, "cfg: I8A8 needs d_model <= 8192 and ffn_inner <= 32768");
  }
  return H3X_OK;
}

h3x_status check_geom(const h3x_geom* g) {
  if (!g) return fail(H3X_EINVAL, "geom is NULL");
  if (g->frames < 0 || g->grid_h < 0 || g->grid_w < 0 || g->n_audio < 0 || g->n_text < 0)
    return fail(H3X_EINVAL, "geom: negative size");
  if (g->merged != 0 && g->merged != 1) return fail(H3X_EINVAL, "geom: merged must be 0 or 1");
  if (g->merged && (g->grid_w % 2)) return fail(H3X_EINVAL, "geom: merged geometry needs an even grid_w");
  // Each grid extent is at most 2^20 (which keeps the RoPE table's int32 entry indices in
  // range), so their product stays below 2^60 and is formed without overflow.
  const int64_t lim = int64_t(1) << 26, grid_lim = int64_t(1) << 20;
  if (g->frames > grid_lim || g->grid_h > grid_lim || g->grid_w > grid_lim)
    return fail(H3X_EINVAL, "geom: a grid extent above 2^20");
  if (g->n_audio > lim || g->n_text > lim) return fail(H3X_EINVAL, "geom: too many tokens");
  const int64_t nv = static_cast<int64_t>(g->frames) * g->grid_h * g->grid_w;
  const int64_t n = (g->merged ? nv / 2 : nv) + g->n_audio + g->n_text;
  if (n <= 0) return fail(H3X_EINVAL, "geom: no tokens");
  if (n > lim) return fail(H3X_EINVAL, "geom: too many tokens");
  return H3X_OK;
}

// The bfloat16 attention addresses K and V^T of a sequence through 32-bit buffer offsets: one
// head-major K or V^T matrix of Npad x d bfloat16 must stay below 2^31 bytes.
h3x_status check_seq(const h3x_block_cfg* c, int64_t n) {
  if (c->act == H3X_BF16 && ((n + 255) / 256 * 256) * static_cast<int64_t>(c->d_model) * 2 > INT32_MAX)
    return fail(H3X_ENOTSUP, "sequence too long: Npad * d_model * 2 must stay below 2^31 bytes");
  return H3X_OK;
}

int64_t geom_tokens(const h3x_geom* g) {
  const int64_t nv = static_cast<int64_t>(g->frames) * g->grid_h * g->grid_w;
  return (g->merged ? nv / 2 : nv) + g->n_audio + g->n_text;
}

void weight_shape(const h3x_block_cfg* c, int kind, int64_t* rows, int64_t* cols) {
  const int64_t d = c->d_model, f = c->ffn_inner;
  switch (kind) {
    case H3X_W_QKV: *rows = 3 * d; *cols = d; break;
    case H3X_W_OUT: *rows = d; *cols = d; break;
    case H3X_W_GATE_UP: *rows = 2 * f; *cols = d; break;
    case H3X_W_DOWN: *rows = d; *cols = f; break;
    default: *rows = -1; *cols = -1;
  }
}

// ---------------------------------------------------------------- workspace layout
size_t rope_entries(const h3x_block_cfg* c, const h3x_geom* g) {
  const int64_t kt = c->head_dim / 8, ky = 3 * c->head_dim / 16;
  return static_cast<size_t>(g->frames * kt + g->grid_h * ky + 2 * g->grid_w * ky);
}
size_t rope_bytes(const h3x_block_cfg* c, const h3x_geom* g) {
  const int64_t nv = static_cast<int64_t>(g->frames) * g->grid_h * g->grid_w / (g->merged ? 2 : 1);
  return align256(rope_entries(c, g) * 8) + align256(static_cast<size_t>(nv) * 16);
}

struct BlockWs {
  int64_t n, n_pad;
  uint8_t* y;      // [n_pad x d]
  uint8_t* q;      // [n_pad x d]
  uint8_t* k;      // [n_pad x d]
  uint8_t* vt;     // [d x n_pad]
  uint8_t* o;      // [n_pad x d]
  uint8_t* h;      // [n_pad x F], aliases q, k, vt, o (dead once h is produced)
  uint8_t* rope;   // rope table of the geometry
  uint8_t* attn;   // partial results of key-split attention workgroups
  uint8_t* a8;     // W8A8: int8 codes of the current projection input, [n_pad x max(d, F)] slabs
  float* a8s;      // W8A8: their float32 row scales [n_pad]
  uint8_t* w16;    // int8 weights: one weight matrix widened to bfloat16 ahead of its GEMM
  size_t bytes;
};

// Upper bound of attention_ws_bytes over every device and bfloat16 attention kernel: at most
// kAttnMaxPieceQueries queries in pieces, and never more than one 256-query piece per
// (128-query block, key tile).
size_t attn_region_bytes(const h3x_block_cfg* c, int64_t n) {
  if (c->act != H3X_BF16) return 0;
  const size_t cap = static_cast<size_t>(kAttnMaxPieceQueries / 128) * attn_part_bytes(128);
  const size_t per_tile = static_cast<size_t>((n + 127) / 128) * c->n_heads * ((n + 63) / 64) * attn_part_bytes(256);
  return per_tile < cap ? per_tile : cap;
}

// Address `off` bytes into a workspace. Integer arithmetic, so that a layout can also be
// computed for base == nullptr (the size queries) without pointer arithmetic on a null pointer.
uint8_t* at(uint8_t* base, size_t off) {
  return reinterpret_cast<uint8_t*>(reinterpret_cast<uintptr_t>(base) + off);
}

// Activation arenas by lifetime: R2 holds y (norm before attention), then y2 (norm before the
// MLP); R1 holds q, k, v^T and the attention output o, then the SwiGLU hidden h.
BlockWs block_layout(const h3x_block_cfg* c, const h3x_geom* g, uint8_t* base) {
  BlockWs w;
  w.n = geom_tokens(g);
  w.n_pad = round_up(w.n, 256);
  const size_t es = elem_bytes(c->act);
  const size_t nd = static_cast<size_t>(w.n_pad) * c->d_model * es;
  const size_t r1 = static_cast<size_t>(w.n_pad) * es *
                    static_cast<size_t>(c->ffn_inner > 4 * c->d_model ? c->ffn_inner : 4 * c->d_model);
  size_t off = 0;
  w.y = at(base, off); off = align256(off + nd);
  w.q = at(base, off); w.k = at(base, off + nd); w.vt = at(base, off + 2 * nd); w.o = at(base, off + 3 * nd);
  w.h = w.q;
  off = align256(off + r1);
  w.rope = at(base, off); off = align256(off + rope_bytes(c, g));
  w.attn = at(base, off); off = align256(off + attn_region_bytes(c, w.n));
  w.a8 = nullptr;
  w.a8s = nullptr;
  w.w16 = nullptr;
  if (c->weight == H3X_I8A8) {
    const size_t cols = static_cast<size_t>(c->ffn_inner > c->d_model ? c->ffn_inner : c->d_model);
    w.a8 = at(base, off); off = align256(off + static_cast<size_t>(w.n_pad) * cols);
    w.a8s = reinterpret_cast<float*>(at(base, off)); off = align256(off + static_cast<size_t>(w.n_pad) * 4);
  }
  if (c->weight == H3X_I8) {
    const size_t d = c->d_model, f = c->ffn_inner;
    const size_t most = 3 * d * d > 2 * f * d ? 3 * d * d : 2 * f * d;  // the largest matrix
    w.w16 = at(base, off); off = align256(off + most * 2);
  }
  w.bytes = off;
  return w;
}

RopeDev rope_dev(const h3x_block_cfg* c, const h3x_geom* g, const uint8_t* rope) {
  RopeDev r;
  r.table = reinterpret_cast<const float2*>(rope);
  r.rowbase = reinterpret_cast<const int4*>(rope + align256(rope_entries(c, g) * 8));
  r.head_dim = c->head_dim;
  r.kt = c->head_dim / 8;
  r.ky = 3 * c->head_dim / 16;
  r.off_y = g->frames * r.kt;
  r.off_x = r.off_y + g->grid_h * r.ky;
  return r;
}

h3x_status build_rope(const h3x_block_cfg* c, const h3x_geom* g, uint8_t* rope, hipStream_t s) {
  const RopeDev r = rope_dev(c, g, rope);
  H3X_LAUNCH("rope_table", s,
             launch_rope_table(geom_dev(*g), c->head_dim, c->rope_theta,
                               reinterpret_cast<float2*>(rope), const_cast<int4*>(r.rowbase), s));
  return H3X_OK;
}

h3x_status check_weights(const h3x_block_cfg* c, const h3x_block_weights* w) {
  if (!w) return fail(H3X_EINVAL, "weights is NULL");
  const void* p[4] = {w->qkv, w->out, w->gate_up, w->down};
  const void* sc[4] = {w->s_qkv, w->s_out, w->s_gate_up, w->s_down};
  for (int i = 0; i < 4; ++i) {
    if (!p[i] || !aligned16(p[i])) return fail(H3X_EINVAL, "weights: NULL or misaligned weight pointer");
    if (int8_weights(c) && !sc[i]) return fail(H3X_EINVAL, "weights: int8 weights need scales");
    if (!int8_weights(c) && sc[i]) return fail(H3X_EINVAL, "weights: scales given for non-int8 weights");
  }
  return H3X_OK;
}

const char* gemm_name(int epi) {
  switch (epi) {
    case EPI_QKV: return "gemm_qkv_rope";
    case EPI_RESID: return "gemm_resid";
    case EPI_SWIGLU: return "gemm_gate_up_swiglu";
    default: return "gemm_f32out";
  }
}

GemmArgs gemm_args(const h3x_block_cfg* c, int kind, int64_t m, const void* a, const void* w,
                   const void* s) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  int64_t rows, cols;
  weight_shape(c, kind, &rows, &cols);
  g.a = a; g.w = w; g.wscale = static_cast<const uint16_t*>(s);
  g.ascale = nullptr;
  g.m = m; g.n = rows; g.k = cols;
  g.m_pad = round_up(m, 256);
  g.d_model = c->d_model;
  return g;
}

// W8A8 block: every projection input is quantised per row (the normalised rows by the norm
// kernel itself, the attention output and the SwiGLU product by a pass of their own) into the
// a8 region, and the GEMMs multiply int8 by int8.
h3x_status block_forward_a8(const h3x_block_cfg* c, const h3x_geom* g, const h3x_block_weights* w,
                            const float* mod, void* x, const BlockWs& ws, hipStream_t s) {
  const int64_t n = ws.n, d = c->d_model;
  const float *shift1 = mod, *scale1 = mod + d, *gate1 = mod + 2 * d;
  const float *shift2 = mod + 3 * d, *scale2 = mod + 4 * d, *gate2 = mod + 5 * d;
  int8_t* qa = reinterpret_cast<int8_t*>(ws.a8);
  float* sa = ws.a8s;
  auto args = [&](int kind, const void* wt, const void* sc) {
    GemmArgs a = gemm_args(c, kind, n, qa, wt, sc);
    a.ascale = sa;
    a.a_tiled = 1;
    return a;
  };
  H3X_LAUNCH("norm_mod_quant", s, launch_norm_mod_quant(n, c->d_model, c->norm_eps, x, shift1, scale1, qa, sa, s));
  GemmArgs qg = args(H3X_W_QKV, w->qkv, w->s_qkv);
  qg.m_pad = ws.n_pad;
  qg.q = ws.q; qg.kk = ws.k; qg.vt = ws.vt; qg.geom = geom_dev(*g); qg.rope = rope_dev(c, g, ws.rope);
  H3X_LAUNCH(gemm_name(EPI_QKV), s, launch_gemm(c->act, c->weight, EPI_QKV, qg, s));
  H3X_LAUNCH("attention", s, launch_attention(c->act, n, ws.n_pad, c->n_heads, c->head_dim, ws.q, ws.k, ws.vt, ws.o, 0,
                                              attention_slots(0), ws.attn, s));
  H3X_LAUNCH("quant_rows", s, launch_quant_rows(n, d, ws.o, qa, sa, s));
  GemmArgs og = args(H3X_W_OUT, w->out, w->s_out);
  og.x = x; og.gate = gate1;
  H3X_LAUNCH("gemm_out_resid", s, launch_gemm(c->act, c->weight, EPI_RESID, og, s));
  H3X_LAUNCH("norm_mod_quant", s, launch_norm_mod_quant(n, c->d_model, c->norm_eps, x, shift2, scale2, qa, sa, s));
  GemmArgs gg = args(H3X_W_GATE_UP, w->gate_up, w->s_gate_up);
  gg.h = ws.h;  // row-major bfloat16, quantised next
  H3X_LAUNCH(gemm_name(EPI_SWIGLU), s, launch_gemm(c->act, c->weight, EPI_SWIGLU, gg, s));
  H3X_LAUNCH("quant_rows", s, launch_quant_rows(n, c->ffn_inner, ws.h, qa, sa, s));
  GemmArgs dg = args(H3X_W_DOWN, w->down, w->s_down);
  dg.x = x; dg.gate = gate2;
  H3X_LAUNCH("gemm_down_resid", s, launch_gemm(c->act, c->weight, EPI_RESID, dg, s));
  return H3X_OK;
}

// One block on prepared workspace and rope table (no validation).
h3x_status block_forward_impl(const h3x_block_cfg* c, const h3x_geom* g, const h3x_block_weights* w,
                              const float* mod, void* x, const BlockWs& ws, hipStream_t s) {
  const int64_t n = ws.n, d = c->d_model;
  const GeomDev gd = geom_dev(*g);
  const RopeDev rd = rope_dev(c, g, ws.rope);
  const float *shift1 = mod, *scale1 = mod + d, *gate1 = mod + 2 * d;
  const float *shift2 = mod + 3 * d, *scale2 = mod + 4 * d, *gate2 = mod + 5 * d;
  if (c->weight == H3X_I8A8) return block_forward_a8(c, g, w, mod, x, ws, s);

  // bf16: the GEMM A operands (y, o, y2, h) live in the slab layout of the MFMA GEMM.
  const int tiled = c->act == H3X_BF16 ? 1 : 0;
  // int8 weights: each matrix is widened to bfloat16 (exact) just before its GEMM, which then runs
  // the bf16 kernel with the row scales in its epilogue. Widening inside the GEMM's K loop costs
  // VALU work that the SIMDs cannot overlap with their MFMAs; this costs one pass over the codes.
  const int wd = c->weight == H3X_I8 ? H3X_BF16 : c->weight;
  hipError_t widen_err = hipSuccess;
  auto widened = [&](int kind, const void* wq) -> const void* {
    if (c->weight != H3X_I8) return wq;
    int64_t rows, cols;
    weight_shape(c, kind, &rows, &cols);
    Timed _t("widen_int8", s);
    widen_err = launch_widen_int8(rows, cols, static_cast<const int8_t*>(wq), ws.w16, s);
    return widen_err == hipSuccess ? ws.w16 : nullptr;
  };
  auto widen_failed = [&]() { return hip_check(widen_err, "widen_int8"); };
  H3X_LAUNCH("norm_mod", s, launch_norm_mod(c->act, n, c->d_model, c->norm_eps, x, shift1, scale1, ws.y, tiled, s));

  const void* wqkv = widened(H3X_W_QKV, w->qkv);
  if (!wqkv) return widen_failed();
  GemmArgs qa = gemm_args(c, H3X_W_QKV, n, ws.y, wqkv, w->s_qkv);
  qa.a_tiled = tiled;
  qa.m_pad = ws.n_pad;
  qa.q = ws.q; qa.kk = ws.k; qa.vt = ws.vt; qa.geom = gd; qa.rope = rd;
  H3X_LAUNCH(gemm_name(EPI_QKV), s, launch_gemm(c->act, wd, EPI_QKV, qa, s));

  H3X_LAUNCH("attention", s, launch_attention(c->act, n, ws.n_pad, c->n_heads, c->head_dim, ws.q, ws.k, ws.vt, ws.o, tiled,
                                              attention_slots(0), ws.attn, s));

  const void* wout = widened(H3X_W_OUT, w->out);
  if (!wout) return widen_failed();
  GemmArgs oa = gemm_args(c, H3X_W_OUT, n, ws.o, wout, w->s_out);
  oa.a_tiled = tiled;
  oa.x = x; oa.gate = gate1;
  H3X_LAUNCH("gemm_out_resid", s, launch_gemm(c->act, wd, EPI_RESID, oa, s));

  H3X_LAUNCH("norm_mod", s, launch_norm_mod(c->act, n, c->d_model, c->norm_eps, x, shift2, scale2, ws.y, tiled, s));

  const void* wgu = widened(H3X_W_GATE_UP, w->gate_up);
  if (!wgu) return widen_failed();
  GemmArgs ga = gemm_args(c, H3X_W_GATE_UP, n, ws.y, wgu, w->s_gate_up);
  ga.a_tiled = tiled;
  ga.out_tiled = tiled;
  ga.h = ws.h;
  H3X_LAUNCH(gemm_name(EPI_SWIGLU), s, launch_gemm(c->act, wd, EPI_SWIGLU, ga, s));

  const void* wdn = widened(H3X_W_DOWN, w->down);
  if (!wdn) return widen_failed();
  GemmArgs da = gemm_args(c, H3X_W_DOWN, n, ws.h, wdn, w->s_down);
  da.a_tiled = tiled;
  da.x = x; da.gate = gate2;
  H3X_LAUNCH("gemm_down_resid", s, launch_gemm(c->act, wd, EPI_RESID, da, s));
  return H3X_OK;
}

struct StepWs {
  BlockWs blk;       // sized for the unmerged geometry
  uint8_t* x;        // [N x d] DiT activations
  uint8_t* xm;       // [N' x d] merged activations
  uint8_t* rope_m;   // rope table of the merged geometry
  size_t bytes;
};

StepWs step_layout(const h3x_block_cfg* c, const h3x_geom* g, uint8_t* base) {
  StepWs w;
  w.blk = block_layout(c, g, base);
  size_t off = align256(w.blk.bytes);
  const size_t es = elem_bytes(c->act);
  const int64_t n = geom_tokens(g);
  w.x = at(base, off); off = align256(off + static_cast<size_t>(n) * c->d_model * es);
  h3x_geom gm = *g;
  gm.merged = 1;
  const int64_t nv = static_cast<int64_t>(g->frames) * g->grid_h * g->grid_w;
  const int64_t nm = nv / 2 + g->n_audio + g->n_text;
  w.xm = at(base, off); off = align256(off + static_cast<size_t>(nm) * c->d_model * es);
  w.rope_m = at(base, off); off += rope_bytes(c, &gm);
  w.bytes = off;
  return w;
}

}  // namespace

// ---------------------------------------------------------------- allocation-free scratch
// Device-resident workspace of h3x_dit_block_forward_noalloc: one copy per GPU, held from the
// library's load until the process ends. Host code never passes `scratch` itself (its name is a
// host-side stand-in, not a device address): the address is looked up per device with
// hipGetSymbolAddress and kept.
static __device__ __align__(256) uint8_t scratch[H3X_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::once_flag g_scratch_once[kScratchDevices];
uint8_t* g_scratch_ptr[kScratchDevices];
hipError_t g_scratch_err[kScratchDevices];

// The current device's copy of `scratch` (looked up once per device, with that device current).
h3x_status scratch_ptr(uint8_t** out) {
  int dev = 0;
  h3x_status st = hip_check(hipGetDevice(&dev), "noalloc: hipGetDevice");
  if (st != H3X_OK) return st;
  if (dev < 0 || dev >= kScratchDevices) return fail(H3X_ENOTSUP, "noalloc: device index beyond 63");
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  });
  if ((st = hip_check(g_scratch_err[dev], "noalloc: hipGetSymbolAddress(scratch)")) != H3X_OK) return st;
  if (!g_scratch_ptr[dev]) return fail(H3X_EHIP, "noalloc: no device address for the scratch array");
  *out = g_scratch_ptr[dev];
  return H3X_OK;
}
}  // namespace

// ====================================================================== exported entry points
extern "C" {

int32_t h3x_abi_version(void) { return H3X_ABI_VERSION; }

const char* h3x_status_string(h3x_status s) {
  switch (s) {
    case H3X_OK: return "ok";
    case H3X_EINVAL: return "invalid argument";
    case H3X_ENOTSUP: return "unsupported shape or type";
    case H3X_EWORKSPACE: return "workspace too small";
    case H3X_EHIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* h3x_last_error(void) { return g_last_error.c_str(); }

int64_t h3x_geom_tokens(const h3x_geom* g) {
  if (check_geom(g) != H3X_OK) return -1;
  return geom_tokens(g);
}

int64_t h3x_packed_rows(const h3x_block_cfg* c, int32_t kind) {
  if (check_cfg(c) != H3X_OK) return -1;
  int64_t r, cc;
  weight_shape(c, kind, &r, &cc);
  return r;
}

size_t h3x_packed_weight_bytes(const h3x_block_cfg* c, int32_t kind, int64_t rows, int64_t cols) {
  if (check_cfg(c) != H3X_OK) return 0;
  int64_t r, cc;
  weight_shape(c, kind, &r, &cc);
  if (r < 0 || rows != r || cols != cc) return 0;
  const size_t es = int8_weights(c) ? 1 : (c->weight == H3X_BF16 ? 2 : 4);
  return static_cast<size_t>(r) * cc * es;
}

int64_t h3x_packed_scale_count(const h3x_block_cfg* c, int32_t kind) {
  if (check_cfg(c) != H3X_OK) return -1;
  int64_t r, cc;
  weight_shape(c, kind, &r, &cc);
  if (r < 0) return -1;
  return int8_weights(c) ? r : 0;
}

}  // extern "C"

namespace {
// Shared checks of the packing calls: kind, the caller's source shape, pointers.
h3x_status check_pack(const h3x_block_cfg* c, int32_t kind, int64_t rows, int64_t cols, const void* w,
                      const void* out, const char* who) {
  int64_t r, cc;
  weight_shape(c, kind, &r, &cc);
  if (r < 0) return fail(H3X_EINVAL, std::string(who) + ": bad kind");
  if (rows != r || cols != cc)
    return fail(H3X_EINVAL, std::string(who) + ": source is " + std::to_string(rows) + " x " + std::to_string(cols) +
                                ", the kind needs " + std::to_string(r) + " x " + std::to_string(cc));
  if (!w || !out || !aligned16(w) || !aligned16(out)) return fail(H3X_EINVAL, std::string(who) + ": NULL or misaligned pointer");
  if (w == out) return fail(H3X_EINVAL, std::string(who) + ": in-place packing is not supported");
  return H3X_OK;
}

h3x_status pack_plain(const h3x_block_cfg* c, int32_t kind, const void* w, int64_t rows, int64_t cols,
                      void* packed, void* stream, int want, const char* who) {
  h3x_status st = check_cfg(c);
  if (st != H3X_OK) return st;
  if (c->weight != want)
    return fail(H3X_EINVAL, std::string(who) + (want == H3X_BF16 ? ": cfg->weight must be BF16" : ": cfg->weight must be F32"));
  if ((st = check_pack(c, kind, rows, cols, w, packed, who)) != H3X_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  H3X_LAUNCH("pack", s, launch_pack(c->weight, kind, rows, cols, w, packed, s));
  return H3X_OK;
}
}  // namespace

extern "C" {

h3x_status h3x_pack_weights_bf16(const h3x_block_cfg* c, int32_t kind, const void* w, int64_t rows,
                                 int64_t cols, void* packed, void* stream) {
  return pack_plain(c, kind, w, rows, cols, packed, stream, H3X_BF16, "pack_weights_bf16");
}

h3x_status h3x_pack_weights_f32(const h3x_block_cfg* c, int32_t kind, const void* w, int64_t rows,
                                int64_t cols, void* packed, void* stream) {
  return pack_plain(c, kind, w, rows, cols, packed, stream, H3X_F32, "pack_weights_f32");
}

h3x_status h3x_pack_int8_weights(const h3x_block_cfg* c, int32_t kind, const void* w_bf16, int64_t rows,
                                 int64_t cols, void* q_packed, void* scale_bf16, void* stream) {
  h3x_status st = check_cfg(c);
  if (st != H3X_OK) return st;
  if (!int8_weights(c)) return fail(H3X_EINVAL, "pack_int8_weights: cfg->weight must be I8 or I8A8");
  if ((st = check_pack(c, kind, rows, cols, w_bf16, q_packed, "pack_int8_weights")) != H3X_OK) return st;
  if (!scale_bf16) return fail(H3X_EINVAL, "pack_int8_weights: NULL scale pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  H3X_LAUNCH("pack_int8", s, launch_pack_int8(kind, rows, cols, w_bf16, static_cast<int8_t*>(q_packed),
                                              static_cast<uint16_t*>(scale_bf16), c->weight == H3X_I8A8, s));
  return H3X_OK;
}

size_t h3x_block_workspace_bytes(const h3x_block_cfg* c, const h3x_geom* g) {
  if (check_cfg(c) != H3X_OK || check_geom(g) != H3X_OK) return 0;
  return block_layout(c, g, nullptr).bytes;
}

h3x_status h3x_dit_block_forward(const h3x_block_cfg* c, const h3x_geom* g, const h3x_block_weights* w,
                                 const float* mod, void* x, void* ws, size_t ws_bytes, void* stream) {
  h3x_status st = check_cfg(c);
  if (st != H3X_OK) return st;
  if ((st = check_geom(g)) != H3X_OK) return st;
  if ((st = check_seq(c, geom_tokens(g))) != H3X_OK) return st;
  if ((st = check_weights(c, w)) != H3X_OK) return st;
  if (!mod || !x || !ws || !aligned16(mod) || !aligned16(x) || !aligned16(ws))
    return fail(H3X_EINVAL, "block_forward: NULL or misaligned mod / x / ws");
  const BlockWs lay = block_layout(c, g, static_cast<uint8_t*>(ws));
  if (ws_bytes < lay.bytes)
    return fail(H3X_EWORKSPACE, "block_forward: workspace needs " + std::to_string(lay.bytes) + " bytes");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = build_rope(c, g, lay.rope, s)) != H3X_OK) return st;
  return block_forward_impl(c, g, w, mod, x, lay, s);
}

h3x_status h3x_dit_block_forward_noalloc(const h3x_block_cfg* c, const h3x_geom* g, const h3x_block_weights* w,
                                         const float* mod, void* x, void* stream) {
  h3x_status st = check_cfg(c);
  if (st != H3X_OK) return st;
  if ((st = check_geom(g)) != H3X_OK) return st;
  if ((st = check_seq(c, geom_tokens(g))) != H3X_OK) return st;
  if ((st = check_weights(c, w)) != H3X_OK) return st;
  if (!mod || !x || !aligned16(mod) || !aligned16(x)) return fail(H3X_EINVAL, "block_forward_noalloc: NULL or misaligned mod / x");
  const size_t need = block_layout(c, g, nullptr).bytes;
  if (need > H3X_NOALLOC_SCRATCH_BYTES)
    return fail(H3X_EWORKSPACE, "block_forward_noalloc: this block needs " + std::to_string(need) +
                                    " bytes of workspace, beyond the " + std::to_string(H3X_NOALLOC_SCRATCH_BYTES) +
                                    "-byte device scratch; use h3x_dit_block_forward with a workspace");
  uint8_t* base = nullptr;
  if ((st = scratch_ptr(&base)) != H3X_OK) return st;
  const BlockWs lay = block_layout(c, g, base);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = build_rope(c, g, lay.rope, s)) != H3X_OK) return st;
  return block_forward_impl(c, g, w, mod, x, lay, s);
}

int32_t h3x_step_is_fresh(int32_t step, int32_t n_steps, int32_t reuse) {
  if (n_steps < 1 || reuse < 1 || step < 0 || step >= n_steps) return -1;
  return (step % reuse == 0 || step == n_steps - 1) ? 1 : 0;
}

h3x_status h3x_sigma_schedule(int32_t kind, int32_t n_steps, double param, float* out) {
  if (n_steps < 1 || !out) return fail(H3X_EINVAL, "sigma_schedule: need n_steps >= 1 and an output");
  if (!std::isfinite(param)) return fail(H3X_EINVAL, "sigma_schedule: non-finite param");
  if (kind == H3X_SCHED_POWER && !(param > 0)) return fail(H3X_EINVAL, "sigma_schedule: power needs param > 0");
  if (kind == H3X_SCHED_LINEAR_TERMINAL && param < n_steps)
    return fail(H3X_EINVAL, "sigma_schedule: the base step count must be >= n_steps");
  if (kind < H3X_SCHED_LINEAR || kind > H3X_SCHED_LINEAR_TERMINAL) return fail(H3X_EINVAL, "sigma_schedule: bad kind");
  for (int32_t i = 0; i <= n_steps; ++i) {
    const double t = static_cast<double>(i);
    double v;
    if (kind == H3X_SCHED_LINEAR) v = 1.0 - t / n_steps;
    else if (kind == H3X_SCHED_POWER) v = std::pow(1.0 - t / n_steps, param);
    else v = i == n_steps ? 0.0 : 1.0 - t / param;
    out[i] = static_cast<float>(v);
  }
  return H3X_OK;
}

float h3x_extrapolation_weight(float sigma, float sigma_a, float sigma_b) {
  const double sa = sigma_a, sb = sigma_b;
  if (sa == sb) return NAN;
  return static_cast<float>((static_cast<double>(sigma) - sa) / (sa - sb));
}

size_t h3x_step_workspace_bytes(const h3x_block_cfg* c, const h3x_geom* g) {
  if (check_cfg(c) != H3X_OK || check_geom(g) != H3X_OK || g->merged) return 0;
  return step_layout(c, g, nullptr).bytes;
}

h3x_status h3x_denoise_step(const h3x_block_cfg* c, const h3x_geom* g, const h3x_step* st_,
                            float* z, const void* text, void* v_cache, void* ws, size_t ws_bytes,
                            void* stream) {
  h3x_status st = check_cfg(c);
  if (st != H3X_OK) return st;
  if ((st = check_geom(g)) != H3X_OK) return st;
  if (g->merged) return fail(H3X_EINVAL, "denoise_step: geom must be unmerged");
  if ((st = check_seq(c, geom_tokens(g))) != H3X_OK) return st;
  if (!st_) return fail(H3X_EINVAL, "denoise_step: step is NULL");
  const int fresh = h3x_step_is_fresh(st_->step, st_->n_steps, st_->reuse);
  if (fresh < 0) return fail(H3X_EINVAL, "denoise_step: need 0 <= step < n_steps and reuse >= 1");
  if (!isfinite(st_->sigma) || !isfinite(st_->sigma_next)) return fail(H3X_EINVAL, "denoise_step: non-finite sigma");
  const int64_t nv = static_cast<int64_t>(g->frames) * g->grid_h * g->grid_w;
  const int64_t n_state = nv + g->n_audio;
  if (!z || !v_cache || !aligned16(z) || !aligned16(v_cache)) return fail(H3X_EINVAL, "denoise_step: NULL or misaligned z / v_cache");
  if (st_->cond_first < 0 || st_->cond_last < 0 || st_->cond_first + st_->cond_last > g->frames)
    return fail(H3X_EINVAL, "denoise_step: need cond_first, cond_last >= 0 and their sum <= frames");
  if (!std::isfinite(st_->extrap)) return fail(H3X_EINVAL, "denoise_step: non-finite extrap");
  if (st_->v_prev && !aligned16(st_->v_prev)) return fail(H3X_EINVAL, "denoise_step: misaligned v_prev");
  if (!fresh && st_->extrap != 0.0f && !st_->v_prev)
    return fail(H3X_EINVAL, "denoise_step: extrapolation needs v_prev");
  const bool core_on = st_->core_reuse >= 2;
  if (st_->core_reuse < 0) return fail(H3X_EINVAL, "denoise_step: negative core_reuse");
  if (core_on) {
    if (st_->reuse != 1) return fail(H3X_EINVAL, "denoise_step: core reuse and whole-velocity reuse are exclusive");
    if (st_->core_first < 0 || st_->core_first > st_->core_last || st_->core_last >= st_->n_blocks)
      return fail(H3X_EINVAL, "denoise_step: need 0 <= core_first <= core_last < n_blocks");
    // With token reduction the core runs wholly in one geometry: inside the reduced blocks (its
    // kept change then has the merged row count) or wholly before or after them.
    if (st_->tr_first >= 0) {
      const bool inside = st_->tr_first <= st_->core_first && st_->core_last <= st_->tr_last;
      const bool outside = st_->core_last < st_->tr_first || st_->core_first > st_->tr_last;
      if (!inside && !outside)
        return fail(H3X_EINVAL, "denoise_step: the core blocks straddle a token-reduction boundary");
    }
    if (!st_->core_delta || !aligned16(st_->core_delta)) return fail(H3X_EINVAL, "denoise_step: NULL or misaligned core_delta");
  }
  if (fresh) {
    if (st_->n_blocks < 1 || !st_->blocks || !st_->mod || !aligned16(st_->mod))
      return fail(H3X_EINVAL, "denoise_step: fresh step needs n_blocks >= 1, blocks and mod");
    for (int b = 0; b < st_->n_blocks; ++b)
      if ((st = check_weights(c, &st_->blocks[b])) != H3X_OK) return st;
    const bool tr_off = st_->tr_first == -1 && st_->tr_last == -1;
    if (!tr_off) {
      if (st_->tr_first < 0 || st_->tr_first > st_->tr_last || st_->tr_last >= st_->n_blocks)
        return fail(H3X_EINVAL, "denoise_step: need 0 <= tr_first <= tr_last < n_blocks (or -1, -1)");
      if (g->grid_w % 2) return fail(H3X_EINVAL, "denoise_step: token reduction needs an even grid_w");
    }
    if (g->n_text > 0 && (!text || !aligned16(text))) return fail(H3X_EINVAL, "denoise_step: NULL or misaligned text");
    if (!ws || !aligned16(ws)) return fail(H3X_EINVAL, "denoise_step: NULL or misaligned workspace");
    const size_t need = step_layout(c, g, nullptr).bytes;
    if (ws_bytes < need)
      return fail(H3X_EWORKSPACE, "denoise_step: workspace needs " + std::to_string(need) + " bytes");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float delta = st_->sigma_next - st_->sigma;  // float32 subtraction
  const int64_t n_elems = n_state * c->d_model;
  // Fixed condition rows: video rows of the first cond_first and last cond_last frames.
  const int64_t per_frame = static_cast<int64_t>(g->grid_h) * g->grid_w;
  const int64_t cond_lo = st_->cond_first * per_frame;
  const int64_t cond_hi = (static_cast<int64_t>(g->frames) - st_->cond_last) * per_frame;
  if (!fresh) {
    const void* vp = st_->extrap != 0.0f ? st_->v_prev : nullptr;
    H3X_LAUNCH("euler", s, launch_euler(c->act, n_elems, c->d_model, z, v_cache, vp, st_->extrap, delta, nullptr,
                                        cond_lo, cond_hi, nv, s));
    return H3X_OK;
  }
  // The velocity about to be replaced becomes the previous one.
  if (st_->v_prev)
    H3X_LAUNCH("copy", s, launch_copy(v_cache, st_->v_prev, static_cast<size_t>(n_elems) * elem_bytes(c->act), s));
  const StepWs lay = step_layout(c, g, static_cast<uint8_t*>(ws));
  h3x_geom gm = *g;
  gm.merged = 1;
  if ((st = build_rope(c, g, lay.blk.rope, s)) != H3X_OK) return st;
  const bool use_tr = st_->tr_first >= 0;
  if (use_tr && (st = build_rope(c, &gm, lay.rope_m, s)) != H3X_OK) return st;

  H3X_LAUNCH("assemble", s, launch_assemble(c->act, n_state, g->n_text, c->d_model, z, text, lay.x, s));
  const size_t mod_stride = 6 * static_cast<size_t>(c->d_model);
  const bool core_fresh = core_on && h3x_step_is_fresh(st_->step, st_->n_steps, st_->core_reuse) == 1;
  bool merged = false;
  for (int b = 0; b < st_->n_blocks; ++b) {
    if (use_tr && b == st_->tr_first) {
      H3X_LAUNCH("token_merge", s, launch_token_merge(c->act, geom_dev(*g), c->d_model, lay.x, lay.xm, s));
      merged = true;
    }
    if (merged && b == st_->tr_last + 1) {
      H3X_LAUNCH("token_unmerge", s, launch_token_unmerge(c->act, geom_dev(*g), c->d_model, lay.xm, lay.x, s));
      merged = false;
    }
    const h3x_geom* gb = merged ? &gm : g;
    void* xb = merged ? lay.xm : lay.x;
    // The core's change lives in the geometry its blocks run in (validated above: one geometry).
    const int64_t n_cur = geom_tokens(gb) * c->d_model;
    if (core_on && b == st_->core_first) {
      if (core_fresh) {
        H3X_LAUNCH("core_save", s, launch_core(c->act, 0, n_cur, xb, st_->core_delta, s));
      } else {  // the kept change of the core replaces its blocks
        H3X_LAUNCH("core_apply", s, launch_core(c->act, 2, n_cur, xb, st_->core_delta, s));
        b = st_->core_last;
        continue;
      }
    }
    BlockWs bw = lay.blk;
    bw.n = geom_tokens(gb);
    bw.n_pad = round_up(bw.n, 256);
    // Re-derive the y and R1 arenas for the (smaller) merged sequence inside the unmerged ones.
    // Only those two are re-laid: past them lies the unmerged rope table, which the blocks after
    // the reduced range still read, so the merged rope table, the attention pieces and the W8A8
    // codes keep regions of their own (each unmerged region bounds the merged one).
    if (merged) {
      BlockWs m = block_layout(c, gb, lay.blk.y);
      m.rope = lay.rope_m;
      m.attn = lay.blk.attn;
      m.a8 = lay.blk.a8;
      m.a8s = lay.blk.a8s;
      m.w16 = lay.blk.w16;
      bw = m;
    }
    if ((st = block_forward_impl(c, gb, &st_->blocks[b], st_->mod + b * mod_stride, xb, bw, s)) != H3X_OK)
      return st;
    if (core_fresh && b == st_->core_last)
      H3X_LAUNCH("core_diff", s, launch_core(c->act, 1, n_cur, xb, st_->core_delta, s));
  }
  if (merged)
    H3X_LAUNCH("token_unmerge", s, launch_token_unmerge(c->act, geom_dev(*g), c->d_model, lay.xm, lay.x, s));
  H3X_LAUNCH("euler", s, launch_euler(c->act, n_elems, c->d_model, z, lay.x, nullptr, 0.0f, delta, v_cache,
                                      cond_lo, cond_hi, nv, s));
  return H3X_OK;
}

// ---------------------------------------------------------------- kernel-level entry points
h3x_status h3x_norm_mod(const h3x_block_cfg* c, int64_t n_rows, const void* x, const float* shift,
                        const float* scale, void* y, void* stream) {
  h3x_status st = check_cfg(c);
  if (st != H3X_OK) return st;
  if (n_rows < 0 || n_rows > (int64_t(1) << 26)) return fail(H3X_EINVAL, "norm_mod: bad n_rows");
  if (n_rows == 0) return H3X_OK;
  if (!x || !shift || !scale || !y || !aligned16(x) || !aligned16(y) || !aligned16(shift) || !aligned16(scale))
    return fail(H3X_EINVAL, "norm_mod: NULL or misaligned pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  H3X_LAUNCH("norm_mod", s, launch_norm_mod(c->act, n_rows, c->d_model, c->norm_eps, x, shift, scale, y, 0, s));
  return H3X_OK;
}

size_t h3x_rope_table_bytes(const h3x_block_cfg* c, const h3x_geom* g) {
  if (check_cfg(c) != H3X_OK || check_geom(g) != H3X_OK) return 0;
  return rope_bytes(c, g);
}

h3x_status h3x_rope_table(const h3x_block_cfg* c, const h3x_geom* g, void* table, void* stream) {
  h3x_status st = check_cfg(c);
  if (st != H3X_OK) return st;
  if ((st = check_geom(g)) != H3X_OK) return st;
  if (!table || !aligned16(table)) return fail(H3X_EINVAL, "rope_table: NULL or misaligned table");
  return build_rope(c, g, static_cast<uint8_t*>(table), static_cast<hipStream_t>(stream));
}

h3x_status h3x_qkv_project(const h3x_block_cfg* c, const h3x_geom* g, const void* y, const void* w_qkv,
                           const void* s_qkv, const void* rope_table, void* q, void* k, void* vt,
                           void* stream) {
  h3x_status st = check_cfg(c);
  if (st != H3X_OK) return st;
  if ((st = check_geom(g)) != H3X_OK) return st;
  if (!y || !w_qkv || !rope_table || !q || !k || !vt) return fail(H3X_EINVAL, "qkv_project: NULL pointer");
  if (!aligned16(y) || !aligned16(w_qkv) || !aligned16(rope_table) || !aligned16(q) || !aligned16(k) || !aligned16(vt))
    return fail(H3X_EINVAL, "qkv_project: misaligned pointer");
  if (c->weight == H3X_I8A8) return fail(H3X_ENOTSUP, "qkv_project: I8A8 projections run inside the block");
  if ((c->weight == H3X_I8) != (s_qkv != nullptr)) return fail(H3X_EINVAL, "qkv_project: scales iff int8 weights");
  const int64_t n = geom_tokens(g);
  GemmArgs a = gemm_args(c, H3X_W_QKV, n, y, w_qkv, s_qkv);
  a.q = q; a.kk = k; a.vt = vt; a.geom = geom_dev(*g);
  a.rope = rope_dev(c, g, static_cast<const uint8_t*>(rope_table));
  hipStream_t s = static_cast<hipStream_t>(stream);
  H3X_LAUNCH(gemm_name(EPI_QKV), s, launch_gemm(c->act, c->weight, EPI_QKV, a, s));
  return H3X_OK;
}

size_t h3x_attention_workspace_bytes(const h3x_block_cfg* c, int64_t n_tokens, int32_t slots) {
  if (check_cfg(c) != H3X_OK || n_tokens < 1 || n_tokens > (int64_t(1) << 26) || slots < 0) return 0;
  return attention_ws_bytes(c->act, n_tokens, c->n_heads, attention_slots(slots));
}

h3x_status h3x_attention(const h3x_block_cfg* c, int64_t n_tokens, const void* q, const void* k,
                         const void* vt, void* o, int32_t slots, void* ws, size_t ws_bytes, void* stream) {
  h3x_status st = check_cfg(c);
  if (st != H3X_OK) return st;
  if (n_tokens < 1 || n_tokens > (int64_t(1) << 26)) return fail(H3X_EINVAL, "attention: bad n_tokens");
  if ((st = check_seq(c, n_tokens)) != H3X_OK) return st;
  if (slots < 0) return fail(H3X_EINVAL, "attention: negative slots");
  if (!q || !k || !vt || !o || !aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(o))
    return fail(H3X_EINVAL, "attention: NULL or misaligned pointer");
  const int sl = attention_slots(slots);
  const size_t need = attention_ws_bytes(c->act, n_tokens, c->n_heads, sl);
  if (need > 0 && (!ws || !aligned16(ws))) return fail(H3X_EINVAL, "attention: NULL or misaligned workspace");
  if (ws_bytes < need) return fail(H3X_EWORKSPACE, "attention: workspace too small");
  hipStream_t s = static_cast<hipStream_t>(stream);
  H3X_LAUNCH("attention", s, launch_attention(c->act, n_tokens, round_up(n_tokens, 256), c->n_heads, c->head_dim, q, k, vt, o, 0,
                                              sl, ws, s));
  return H3X_OK;
}

static h3x_status linear_common(const h3x_block_cfg* c, int32_t kind, int64_t m, const void* a,
                                const void* w, const void* sc) {
  h3x_status st = check_cfg(c);
  if (st != H3X_OK) return st;
  if (kind < H3X_W_QKV || kind > H3X_W_DOWN) return fail(H3X_EINVAL, "linear: bad kind");
  if (m < 0 || m > (int64_t(1) << 26)) return fail(H3X_EINVAL, "linear: bad m");
  if (c->weight == H3X_I8A8) return fail(H3X_ENOTSUP, "linear: I8A8 takes quantised activations (h3x_linear_a8_f32out)");
  if (m == 0) return H3X_OK;  // nothing to do; the callers return before looking at pointers
  if (!a || !w || !aligned16(a) || !aligned16(w)) return fail(H3X_EINVAL, "linear: NULL or misaligned pointer");
  if ((c->weight == H3X_I8) != (sc != nullptr)) return fail(H3X_EINVAL, "linear: scales iff int8 weights");
  return H3X_OK;
}

h3x_status h3x_quant_rows(int64_t m, int64_t cols, const void* a, void* q, float* sc, void* stream) {
  if (m < 0 || m > (int64_t(1) << 26)) return fail(H3X_EINVAL, "quant_rows: bad m");
  if (cols <= 0 || cols % 64 || cols > 32768) return fail(H3X_EINVAL, "quant_rows: need 0 < cols <= 32768, cols % 64 == 0");
  if (m == 0) return H3X_OK;
  if (!a || !q || !sc || !aligned16(a) || !aligned16(q) || !aligned16(sc))
    return fail(H3X_EINVAL, "quant_rows: NULL or misaligned pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  H3X_LAUNCH("quant_rows", s, launch_quant_rows(m, cols, a, static_cast<int8_t*>(q), sc, s));
  return H3X_OK;
}

h3x_status h3x_norm_mod_quant(const h3x_block_cfg* c, int64_t n_rows, const void* x, const float* shift,
                              const float* scale, void* q, float* sc, void* stream) {
  h3x_status st = check_cfg(c);
  if (st != H3X_OK) return st;
  if (c->weight != H3X_I8A8) return fail(H3X_EINVAL, "norm_mod_quant: cfg->weight must be I8A8");
  if (n_rows < 0 || n_rows > (int64_t(1) << 26)) return fail(H3X_EINVAL, "norm_mod_quant: bad n_rows");
  if (n_rows == 0) return H3X_OK;
  if (!x || !shift || !scale || !q || !sc || !aligned16(x) || !aligned16(shift) || !aligned16(scale) ||
      !aligned16(q) || !aligned16(sc))
    return fail(H3X_EINVAL, "norm_mod_quant: NULL or misaligned pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  H3X_LAUNCH("norm_mod_quant", s, launch_norm_mod_quant(n_rows, c->d_model, c->norm_eps, x, shift, scale,
                                                        static_cast<int8_t*>(q), sc, s));
  return H3X_OK;
}

h3x_status h3x_linear_a8_f32out(const h3x_block_cfg* c, int32_t kind, int64_t m, const void* qa, const float* sa,
                                const void* w, const void* sw, float* out, void* stream) {
  h3x_status st = check_cfg(c);
  if (st != H3X_OK) return st;
  if (c->weight != H3X_I8A8) return fail(H3X_EINVAL, "linear_a8_f32out: cfg->weight must be I8A8");
  if (kind < H3X_W_QKV || kind > H3X_W_DOWN) return fail(H3X_EINVAL, "linear_a8_f32out: bad kind");
  if (m < 0 || m > (int64_t(1) << 26)) return fail(H3X_EINVAL, "linear_a8_f32out: bad m");
  if (m == 0) return H3X_OK;
  if (!qa || !sa || !w || !sw || !out || !aligned16(qa) || !aligned16(sa) || !aligned16(w) || !aligned16(out))
    return fail(H3X_EINVAL, "linear_a8_f32out: NULL or misaligned pointer");
  GemmArgs g = gemm_args(c, kind, m, qa, w, sw);
  g.ascale = sa;
  g.a_tiled = 1;
  g.out = out;
  hipStream_t s = static_cast<hipStream_t>(stream);
  H3X_LAUNCH(gemm_name(EPI_F32), s, launch_gemm(c->act, c->weight, EPI_F32, g, s));
  return H3X_OK;
}

h3x_status h3x_linear_residual(const h3x_block_cfg* c, int32_t kind, int64_t m, const void* a, const void* w,
                               const void* sc, const float* gate, void* x, void* stream) {
  h3x_status st = linear_common(c, kind, m, a, w, sc);
  if (st != H3X_OK || m == 0) return st;
  if (kind != H3X_W_OUT && kind != H3X_W_DOWN) return fail(H3X_EINVAL, "linear_residual: kind must be OUT or DOWN");
  if (!gate || !x || !aligned16(x)) return fail(H3X_EINVAL, "linear_residual: NULL or misaligned gate / x");
  GemmArgs g = gemm_args(c, kind, m, a, w, sc);
  g.x = x; g.gate = gate;
  hipStream_t s = static_cast<hipStream_t>(stream);
  H3X_LAUNCH(kind == H3X_W_OUT ? "gemm_out_resid" : "gemm_down_resid", s, launch_gemm(c->act, c->weight, EPI_RESID, g, s));
  return H3X_OK;
}

h3x_status h3x_linear_swiglu(const h3x_block_cfg* c, int64_t m, const void* y2, const void* w, const void* sc,
                             void* h, void* stream) {
  h3x_status st = linear_common(c, H3X_W_GATE_UP, m, y2, w, sc);
  if (st != H3X_OK || m == 0) return st;
  if (!h || !aligned16(h)) return fail(H3X_EINVAL, "linear_swiglu: NULL or misaligned h");
  GemmArgs g = gemm_args(c, H3X_W_GATE_UP, m, y2, w, sc);
  g.h = h;
  hipStream_t s = static_cast<hipStream_t>(stream);
  H3X_LAUNCH(gemm_name(EPI_SWIGLU), s, launch_gemm(c->act, c->weight, EPI_SWIGLU, g, s));
  return H3X_OK;
}

h3x_status h3x_linear_f32out(const h3x_block_cfg* c, int32_t kind, int64_t m, const void* a, const void* w,
                             const void* sc, float* out, void* stream) {
  h3x_status st = linear_common(c, kind, m, a, w, sc);
  if (st != H3X_OK || m == 0) return st;
  if (!out || !aligned16(out)) return fail(H3X_EINVAL, "linear_f32out: NULL or misaligned out");
  GemmArgs g = gemm_args(c, kind, m, a, w, sc);
  g.out = out;
  hipStream_t s = static_cast<hipStream_t>(stream);
  H3X_LAUNCH(gemm_name(EPI_F32), s, launch_gemm(c->act, c->weight, EPI_F32, g, s));
  return H3X_OK;
}

h3x_status h3x_token_merge(const h3x_block_cfg* c, const h3x_geom* g, const void* x, void* xm, void* stream) {
  h3x_status st = check_cfg(c);
  if (st != H3X_OK) return st;
  if ((st = check_geom(g)) != H3X_OK) return st;
  if (g->merged || g->grid_w % 2) return fail(H3X_EINVAL, "token_merge: need an unmerged geometry with even grid_w");
  if (!x || !xm || !aligned16(x) || !aligned16(xm) || x == xm) return fail(H3X_EINVAL, "token_merge: bad pointers");
  hipStream_t s = static_cast<hipStream_t>(stream);
  H3X_LAUNCH("token_merge", s, launch_token_merge(c->act, geom_dev(*g), c->d_model, x, xm, s));
  return H3X_OK;
}

h3x_status h3x_token_unmerge(const h3x_block_cfg* c, const h3x_geom* g, const void* xm, void* x, void* stream) {
  h3x_status st = check_cfg(c);
  if (st != H3X_OK) return st;
  if ((st = check_geom(g)) != H3X_OK) return st;
  if (g->merged || g->grid_w % 2) return fail(H3X_EINVAL, "token_unmerge: need an unmerged geometry with even grid_w");
  if (!x || !xm || !aligned16(x) || !aligned16(xm) || x == xm) return fail(H3X_EINVAL, "token_unmerge: bad pointers");
  hipStream_t s = static_cast<hipStream_t>(stream);
  H3X_LAUNCH("token_unmerge", s, launch_token_unmerge(c->act, geom_dev(*g), c->d_model, xm, x, s));
  return H3X_OK;
}

h3x_status h3x_euler(const h3x_block_cfg* c, int64_t n_rows, float* z, const void* v, float sigma,
                     float sigma_next, void* v_copy, void* stream) {
  h3x_status st = check_cfg(c);
  if (st != H3X_OK) return st;
  if (n_rows < 0 || n_rows > (int64_t(1) << 26)) return fail(H3X_EINVAL, "euler: bad n_rows");
  if (n_rows == 0) return H3X_OK;
  if (!isfinite(sigma) || !isfinite(sigma_next)) return fail(H3X_EINVAL, "euler: non-finite sigma");
  if (!z || !v || !aligned16(z) || !aligned16(v) || (v_copy && !aligned16(v_copy)))
    return fail(H3X_EINVAL, "euler: NULL or misaligned pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  H3X_LAUNCH("euler", s, launch_euler(c->act, n_rows * c->d_model, c->d_model, z, v, nullptr, 0.0f, sigma_next - sigma,
                                      v_copy, 0, 0, 0, s));
  return H3X_OK;
}

h3x_status h3x_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || !aligned16(src) || !aligned16(dst) || (bytes & 15))
    return fail(H3X_EINVAL, "copy: NULL / misaligned pointer or size not a multiple of 16");
  hipStream_t s = static_cast<hipStream_t>(stream);
  H3X_LAUNCH("copy", s, launch_copy(src, dst, bytes, s));
  return H3X_OK;
}

h3x_status h3x_mfma_probe(int32_t dtype, int64_t iters, float* out, double* ops, void* stream) {
  if (dtype != H3X_BF16 && dtype != H3X_I8) return fail(H3X_EINVAL, "mfma_probe: dtype must be H3X_BF16 or H3X_I8");
  if (iters < 1 || iters > (int64_t(1) << 32)) return fail(H3X_EINVAL, "mfma_probe: iters out of range");
  if (!out || !ops) return fail(H3X_EINVAL, "mfma_probe: NULL pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  *ops = mfma_probe_ops(dtype == H3X_I8, iters);
  H3X_LAUNCH("mfma_probe", s, launch_mfma_probe(dtype == H3X_I8, iters, out, s));
  return H3X_OK;
}

h3x_status h3x_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = true;
  return H3X_OK;
}

int32_t h3x_profile_end(h3x_kernel_time* out, int32_t max_entries) {
  std::vector<Rec> recs;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = false;
    recs.swap(g_prof_recs);
  }
  std::vector<h3x_kernel_time> agg;
  int32_t status = 0;
  for (const Rec& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      status = -1;
      continue;
    }
    bool found = false;
    for (auto& a : agg)
      if (strncmp(a.name, r.name, sizeof(a.name)) == 0) {
        a.launches += 1;
        a.total_ms += ms;
        found = true;
      }
    if (!found) {
      h3x_kernel_time t;
      memset(&t, 0, sizeof(t));
      strncpy(t.name, r.name, sizeof(t.name) - 1);
      t.launches = 1;
      t.total_ms = ms;
      agg.push_back(t);
    }
  }
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (const Rec& r : recs) {
      g_event_pool.push_back(r.start);
      g_event_pool.push_back(r.stop);
    }
  }
  if (status < 0) {
    g_last_error = "profile_end: event query failed";
    return -1;
  }
  const int32_t n = static_cast<int32_t>(agg.size()) < max_entries ? static_cast<int32_t>(agg.size()) : max_entries;
  for (int32_t i = 0; i < n && out; ++i) out[i] = agg[i];
  return n;
}

}  // extern "C"
