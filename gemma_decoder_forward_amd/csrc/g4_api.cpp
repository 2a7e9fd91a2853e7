// The g4 C ABI: host-side validation of every argument, then asynchronous launches on the caller's
// stream. The library owns no device memory; scratch comes from the caller's workspace.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "g4_internal.h"

namespace g4 {

static thread_local std::string g_last_error;

g4_status fail(g4_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

g4_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(G4_EHIP, "%s: %s", what, hipGetErrorString(e));
  return G4_OK;
}

// ---- launch timer (g4_timer_enable / g4_timer_read) ----------------------------------------------
struct Timer {
  int32_t cls = 0;
  int32_t cap = 0, n = 0;
  hipEvent_t* ev = nullptr;
};
static Timer g_timer;

struct TimedScope {  // records an event pair around the launches of one class
  bool on;
  hipStream_t s;
  TimedScope(int32_t cls, hipStream_t st) : on(g_timer.cls == cls && g_timer.n < g_timer.cap), s(st) {
    if (on) (void)hipEventRecord(g_timer.ev[2 * g_timer.n], s);
  }
  ~TimedScope() {
    if (on) {
      (void)hipEventRecord(g_timer.ev[2 * g_timer.n + 1], s);
      ++g_timer.n;
    }
  }
};

static bool dt_ok(int32_t dt) { return dt == G4_F32 || dt == G4_BF16; }

#define G4_REQ(cond, st, ...)                 \
  do {                                        \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

static g4_status check_model(const g4_model_desc* m) {
  G4_REQ(m, G4_EINVAL, "model descriptor is NULL");
  G4_REQ(dt_ok(m->dtype), G4_EINVAL, "model dtype %d is not G4_F32 or G4_BF16", m->dtype);
  G4_REQ(m->hidden > 0 && m->n_heads > 0 && m->n_kv_heads > 0 && m->head_dim_swa > 0 && m->head_dim_full > 0 &&
             m->ffn > 0 && m->ple_dim > 0 && m->n_layers > 0,
         G4_EINVAL, "model sizes must be positive");
  G4_REQ(m->n_heads % m->n_kv_heads == 0, G4_EGEOM, "n_heads %lld is not a multiple of n_kv_heads %lld",
         (long long)m->n_heads, (long long)m->n_kv_heads);
  G4_REQ(m->n_kv_heads_full >= 0 && (m->n_kv_heads_full == 0 || m->n_heads % m->n_kv_heads_full == 0), G4_EGEOM,
         "n_heads %lld is not a multiple of n_kv_heads_full %lld", (long long)m->n_heads,
         (long long)m->n_kv_heads_full);
  G4_REQ(m->k_eq_v == 0 || m->k_eq_v == 1, G4_EINVAL, "k_eq_v must be 0 or 1");
  G4_REQ(m->head_dim_swa % 2 == 0 && m->head_dim_full % 2 == 0, G4_EGEOM, "head dims must be even");
  G4_REQ(m->head_dim_swa <= 512 && m->head_dim_full <= 512, G4_ERANGE, "head dims above 512 are not supported");
  G4_REQ(m->window >= 1, G4_ERANGE, "window %lld < 1", (long long)m->window);
  G4_REQ(m->partial_rotary >= 0.f && m->partial_rotary <= 1.f, G4_EINVAL, "partial_rotary %g outside [0,1]",
         (double)m->partial_rotary);
  G4_REQ(m->eps >= 0.f, G4_EINVAL, "eps < 0");
  G4_REQ(m->theta_swa > 0.f && m->theta_full > 0.f, G4_EINVAL, "RoPE bases must be positive");
  G4_REQ(m->hidden <= 16384, G4_ERANGE, "hidden %lld > 16384", (long long)m->hidden);
  G4_REQ(m->ple_dim <= 512, G4_ERANGE, "ple_dim %lld > 512", (long long)m->ple_dim);
  return G4_OK;
}

// KV heads of a layer type: full layers may carry their own count.
static int64_t kv_heads(const g4_model_desc* m, int sliding) {
  return (!sliding && m->n_kv_heads_full > 0) ? m->n_kv_heads_full : m->n_kv_heads;
}

static int64_t max_kv_heads(const g4_model_desc* m) {
  return m->n_kv_heads_full > m->n_kv_heads ? m->n_kv_heads_full : m->n_kv_heads;
}

// FFN width of a layer (0 in the descriptor: the model's).
static int64_t ffn_of(const g4_model_desc* m, const g4_layer_desc* l) { return l->ffn > 0 ? l->ffn : m->ffn; }

// A full layer of a K=V model takes V from the K projection's output.
static bool v_from_k(const g4_model_desc* m, const g4_layer_desc* l) { return m->k_eq_v && !l->sliding; }

static int64_t rot_pairs(const g4_model_desc* m, int sliding) {
  if (sliding) return m->head_dim_swa / 2;
  return (int64_t)((double)m->head_dim_full * (double)m->partial_rotary / 2.0);
}

// Routing and cache checks shared by the attention entry points and the layer forward.
static g4_status check_kv(const g4_kv_entry* kv, int32_t n_kv, int32_t layer, int32_t kv_src, int32_t sliding,
                          int64_t hd, int64_t T, int32_t mode, int64_t window) {
  G4_REQ(kv, G4_EINVAL, "kv table is NULL");
  G4_REQ(n_kv > 0, G4_EINVAL, "n_kv %d <= 0", n_kv);
  G4_REQ(layer >= 0 && layer < n_kv, G4_EINVAL, "layer %d outside the kv table [0,%d)", layer, n_kv);
  G4_REQ(kv_src >= 0 && kv_src <= layer, G4_EGEOM, "kv_src %d must be in [0, layer %d]", kv_src, layer);
  const g4_kv_entry& e = kv[kv_src];
  G4_REQ(e.k && e.v, G4_EGEOM, "kv_src %d has no cache (a shared layer cannot be a source)", kv_src);
  G4_REQ(e.hd == hd, G4_EGEOM, "layer %d head_dim %lld != kv_src %d cache head_dim %lld", layer, (long long)hd,
         kv_src, (long long)e.hd);
  G4_REQ(e.sliding == sliding, G4_EGEOM, "layer %d attention type differs from kv_src %d", layer, kv_src);
  G4_REQ(e.cap > 0, G4_ERANGE, "cache capacity %lld <= 0", (long long)e.cap);
  G4_REQ(e.ring == 0 || e.ring == 1, G4_EINVAL, "kv entry %d: ring must be 0 or 1", kv_src);
  if (e.ring) {
    G4_REQ(e.sliding, G4_EGEOM, "kv entry %d: only a sliding-window cache can be a ring", kv_src);
    G4_REQ(e.cap >= window, G4_ERANGE, "ring of %lld rows is shorter than the window %lld", (long long)e.cap,
           (long long)window);
    G4_REQ(T <= e.cap - window + 1, G4_ERANGE,
           "T %lld > ring rows %lld - window %lld + 1 (prefill longer prompts in chunks)", (long long)T,
           (long long)e.cap, (long long)window);
  } else {
    G4_REQ(T <= e.cap, G4_ERANGE, "T %lld exceeds cache capacity %lld", (long long)T, (long long)e.cap);
  }
  G4_REQ(mode != G4_DECODE || T == 1, G4_EINVAL, "decode takes T == 1");
  G4_REQ(mode != G4_ENCODE || !e.ring, G4_EINVAL, "kv entry %d: the encoder's attention needs a linear cache",
         kv_src);
  return G4_OK;
}

// ---- workspace plan of the layer forward -----------------------------------------------------
struct Plan {
  size_t xn, qkv, ao, f32buf, act, hb, gm, dec, aws, aws_bytes, gws, gws_bytes, fx, fx_bytes, fy, fy_bytes, emb_e, emb_p,
      total;
  int64_t qkv_ld, splits;
};

static size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

static Plan plan(const g4_model_desc* m, int64_t B, int64_t T, int64_t cap, int32_t mode) {
  Plan p{};
  const size_t E = dsize(m->dtype);
  const int64_t M = B * T;
  const int64_t hdm = m->head_dim_swa > m->head_dim_full ? m->head_dim_swa : m->head_dim_full;
  p.qkv_ld = (m->n_heads + 2 * max_kv_heads(m)) * hdm;
  p.splits = 4;
  size_t o = 0;
  p.xn = o; o += al(M * m->hidden * E);
  p.qkv = o; o += al(M * p.qkv_ld * E);
  p.ao = o; o += al(M * m->n_heads * hdm * E);
  p.f32buf = o; o += al((size_t)p.splits * M * m->hidden * 4);
  p.act = o; o += al(M * m->ffn * E);
  p.hb = o; o += al(M * m->hidden * E);
  p.gm = o; o += al(M * m->ple_dim * E);
  p.dec = o;
  if (mode == G4_DECODE) o += al(attn_decode_ws(B, m->n_heads, hdm, cap > 0 ? cap : 1));
  p.aws = o;  // key-split partials of a short prefill's attention
  p.aws_bytes = 0;
  if (mode != G4_DECODE) {
    const size_t s0 = attn_prefill_ws(B, T, m->n_heads, kv_heads(m, 1), m->head_dim_swa);
    const size_t s1 = attn_prefill_ws(B, T, m->n_heads, kv_heads(m, 0), m->head_dim_full);
    p.aws_bytes = s0 > s1 ? s0 : s1;
    o += al(p.aws_bytes);
  }
  p.gws = o;
  p.gws_bytes = 0;
  if (M <= 64 && m->dtype == G4_BF16) {  // partial sums of the few-row GEMM
    const int64_t H = m->hidden, nh = m->n_heads, hs = m->head_dim_swa, hf = m->head_dim_full;
    const int64_t ns = kv_heads(m, 1), nf = kv_heads(m, 0);
    auto ws_x = [&](int64_t rows) { return gemm_skinny_ws(M, (rows + 63) / 64 * 64, (H + 127) / 128 * 128); };
    auto ws_y = [&](int64_t k) { return gemm_skinny_ws(M, (H + 63) / 64 * 64, (k + 127) / 128 * 128); };
    // the FFN's two GEMMs at every width a layer may have (the split count depends on the width, so the
    // scratch is not largest at the largest width); the few-row kernels take multiples of 64 only
    size_t ffn_x = 0, ffn_y = 0;
    for (int64_t f = 64;; f += 64) {
      if (f > m->ffn) f = m->ffn;
      ffn_x = std::max(ffn_x, ws_x(2 * f));
      ffn_y = std::max(ffn_y, ws_y(f));
      if (f == m->ffn) break;
    }
    p.gws_bytes = std::max(ffn_x, ffn_y);
    for (const int64_t rows : {nh * hs, (nh + 2 * ns) * hs, nh * hf, (nh + nf) * hf, (nh + 2 * nf) * hf, m->ple_dim})
      p.gws_bytes = std::max(p.gws_bytes, ws_x(rows));
    for (const int64_t k : {nh * hs, nh * hf, m->ple_dim}) p.gws_bytes = std::max(p.gws_bytes, ws_y(k));
    o += al(p.gws_bytes);
    // the few-row layer path: split-K partials of q/k/v, gate/up and the PLE gate (fx) and of the
    // projections back to H (fy); a GEMM reading one region writes the other
    p.fx_bytes = ffn_x;  // q only (shared layers), q/k (K=V full layers) or q/k/v
    for (const int64_t rows : {nh * hs, (nh + 2 * ns) * hs, nh * hf, (nh + nf) * hf, (nh + 2 * nf) * hf, m->ple_dim})
      p.fx_bytes = std::max(p.fx_bytes, ws_x(rows));
    p.fy_bytes = ffn_y;
    for (const int64_t k : {nh * hs, nh * hf, m->ple_dim}) p.fy_bytes = std::max(p.fy_bytes, ws_y(k));
    p.fx = o; o += al(p.fx_bytes);
    p.fy = o; o += al(p.fy_bytes);
  }
  p.total = o;
  // the entry (embedding + PLE) reuses the start of the workspace
  p.emb_e = 0;
  p.emb_p = al(M * m->hidden * E);
  const size_t emb_total = p.emb_p + al(M * m->n_layers * m->ple_dim * 4);
  if (emb_total > p.total) p.total = emb_total;
  return p;
}

// GEMM with validation of the shapes it must see.
static thread_local void* g_gws = nullptr;  // scratch of the current layer call for the few-row GEMM
static thread_local size_t g_gws_bytes = 0;

static g4_status run_gemm(const void* A, int64_t lda, const void* B, const void* B2, int64_t ldb, void* C,
                          int64_t ldc, int32_t c_dtype, int64_t M, int64_t N, int64_t K, int32_t epi,
                          const float* aux, int64_t aux_ld, int32_t splits, int64_t split_stride, int32_t dt,
                          hipStream_t s) {
  GemmArgs a{};
  a.ws = g_gws; a.ws_bytes = g_gws_bytes;
  a.A = A; a.lda = lda; a.B = B; a.B2 = B2; a.ldb = ldb; a.C = C; a.ldc = ldc; a.c_dtype = c_dtype;
  a.aux = aux; a.aux_ld = aux_ld; a.M = M; a.N = N; a.K = K; a.epi = epi;
  a.splits = splits < 1 ? 1 : splits; a.split_stride = split_stride;
  return gemm(a, dt, s);
}

// gelu_tanh(A W^T) * aux into C (dtype). The PLE gate has few output columns (the PLE width), so at
// prefill sizes it has too few output tiles to fill the device: K is then split over float32 slices in
// `part` ([splits][M][N]) and a finisher sums them in a fixed order and applies the epilogue.
static g4_status run_gelu_mul(const void* A, int64_t lda, const void* W, int64_t ldb, void* C, int64_t ldc,
                              const float* aux, int64_t aux_ld, int64_t M, int64_t N, int64_t K, int32_t dt,
                              float* part, size_t part_bytes, hipStream_t s) {
  int32_t splits = 1;
  if (dt == G4_BF16 && M > 64 && ((M + 127) / 128) * ((N + 127) / 128) < 256) {
    GemmArgs ga{};
    ga.A = A; ga.lda = lda; ga.B = W; ga.ldb = ldb; ga.C = C; ga.ldc = ldc; ga.c_dtype = dt; ga.aux = aux;
    ga.aux_ld = aux_ld; ga.M = M; ga.N = N; ga.K = K; ga.epi = EPI_GELU_MUL; ga.splits = 1;
    g4_status st = G4_OK;
    if (gemm_mfma_tiles64(ga, s, &st)) return st;
  }
  if (dt == G4_BF16 && M > 64 && part) {
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    while (splits < 8 && tiles * splits * 2 <= 256 && K / (splits * 2) >= 256 &&
           (size_t)(splits * 2) * M * N * 4 <= part_bytes)
      splits *= 2;
  }
  if (splits == 1) return run_gemm(A, lda, W, nullptr, ldb, C, ldc, dt, M, N, K, EPI_GELU_MUL, aux, aux_ld, 1, 0, dt, s);
  g4_status st = run_gemm(A, lda, W, nullptr, ldb, part, N, G4_F32, M, N, K, EPI_STORE, nullptr, 0, splits, M * N, dt, s);
  if (st != G4_OK) return st;
  GemmArgs ga{};
  ga.M = M; ga.N = N; ga.C = C; ga.ldc = ldc; ga.c_dtype = dt; ga.epi = EPI_GELU_MUL; ga.aux = aux; ga.aux_ld = aux_ld;
  return gemm_skinny_finish(ga, part, splits, N, s);
}

struct LayerCtx {
  const g4_model_desc* m;
  const g4_layer_desc* l;
  int32_t layer;
  float* h;
  const float* ple_in;
  const g4_kv_entry* kv;
  int32_t n_kv;
  const int32_t* pos;
  int64_t B, T;
  int32_t mode;
  char* ws;
  const Plan* p;
  hipStream_t s;
  bool xn_ready;                 // xn already holds rms(h) * input_norm (fused by the previous layer)
  const void* next_input_norm;   // if set, the last tail also writes the next layer's xn
};

static g4_status check_layer(const g4_model_desc* m, const g4_layer_desc* l, int32_t layer, const g4_kv_entry* kv,
                             int32_t n_kv, int64_t T, int32_t mode) {
  G4_REQ(l, G4_EINVAL, "layer descriptor is NULL");
  G4_REQ(layer >= 0 && layer < m->n_layers, G4_EINVAL, "layer %d outside [0, %lld)", layer, (long long)m->n_layers);
  G4_REQ(n_kv == m->n_layers, G4_EINVAL, "n_kv %d != n_layers %lld", n_kv, (long long)m->n_layers);
  G4_REQ(l->sliding == 0 || l->sliding == 1, G4_EINVAL, "layer %d: sliding must be 0 or 1", layer);
  G4_REQ(l->ffn >= 0 && l->ffn <= m->ffn, G4_ERANGE, "layer %d: ffn %d outside [0, model ffn %lld]", layer, l->ffn,
         (long long)m->ffn);
  G4_REQ(l->input_norm && l->wq && l->wo && l->q_norm && l->post_attn_norm && l->pre_ffn_norm && l->w_gate &&
             l->w_up && l->w_down && l->post_ffn_norm && l->ple_gate && l->ple_proj && l->post_ple_norm,
         G4_EINVAL, "layer %d: a weight pointer is NULL", layer);
  if (l->kv_src == layer)
    G4_REQ(l->wk && (l->wv || v_from_k(m, l)) && l->k_norm, G4_EINVAL,
           "layer %d owns its cache but wk/wv/k_norm is NULL", layer);
  else G4_REQ(l->kv_src < layer, G4_EGEOM, "layer %d: kv_src %d is not an earlier layer", layer, l->kv_src);
  const int64_t hd = l->sliding ? m->head_dim_swa : m->head_dim_full;
  // decode attention groups at most 8 query heads per kv head (checked here, before anything launches)
  G4_REQ(mode != G4_DECODE || m->n_heads / kv_heads(m, l->sliding) <= 8, G4_EUNSUP,
         "layer %d: decode attention takes at most 8 query heads per kv head (%lld)", layer,
         (long long)(m->n_heads / kv_heads(m, l->sliding)));
  return check_kv(kv, n_kv, layer, l->kv_src, l->sliding, hd, T, mode, m->window);
}

// The layer for few token rows (decode batches, M <= 64, bf16): every projection streams its weights
// once through the few-row GEMM and leaves float32 split-K partials, and the next step sums them as it
// reads them -- the per-head norm/RoPE kernel for q/k/v, the row tails for the projections back to H,
// and the staging of the next GEMM's A operand for the gelu-tanh products (gate * up, PLE gate * input).
// Same arithmetic as the general path; fewer launches and no intermediate finishing passes.
static bool few_row_ok(const LayerCtx& c) {
  const g4_model_desc* m = c.m;
  const g4_layer_desc* l = c.l;
  const int64_t M = c.B * c.T, H = m->hidden, nh = m->n_heads, nkv = kv_heads(m, l->sliding), F = ffn_of(m, l);
  const int64_t hd = l->sliding ? m->head_dim_swa : m->head_dim_full;
  if (m->dtype != G4_BF16 || M > 64 || c.p->fx_bytes == 0) return false;
  const void* q3[3] = {l->wq, l->wk, l->wv};
  const int64_t r3[3] = {nh * hd, nkv * hd, nkv * hd};
  const int nseg = l->kv_src != c.layer ? 1 : (v_from_k(m, l) ? 2 : 3);
  const void* gu[2] = {l->w_gate, l->w_up};
  const int64_t rgu[2] = {F, F};
  const void* wo[1] = {l->wo};
  const void* wd[1] = {l->w_down};
  const void* pg[1] = {l->ple_gate};
  const void* pp[1] = {l->ple_proj};
  const int64_t rH[1] = {H}, rd[1] = {m->ple_dim};
  return skinny_ok(M, H, q3, r3, nseg, H) && skinny_ok(M, nh * hd, wo, rH, 1, nh * hd) &&
         skinny_ok(M, H, gu, rgu, 2, H) && skinny_ok(M, F, wd, rH, 1, F) &&
         skinny_ok(M, H, pg, rd, 1, H) && skinny_ok(M, m->ple_dim, pp, rH, 1, m->ple_dim) &&
         (F % 4) == 0 && (m->ple_dim % 4) == 0 && ((uintptr_t)c.ple_in & 15) == 0;
}

// Whether the consumer GEMM (K x Nc weights) should form its A operand from `parts` float32 slices while
// staging it (each of its blocks re-reads its slice of the partials from L2), rather than after a
// separate finishing pass writes A once in bf16: fused while the re-reads stay within a few MB.
static bool stage_from_parts(int64_t M, int64_t Kc, int64_t Nc, int parts, int reads_per_value) {
  int rows = 0, kc = 0, sp = 0;
  skinny_plan(M, Kc, Nc, &rows, &kc, &sp);
  const double bytes = (double)(Nc / rows) * sp * M * kc * parts * 4.0 * reads_per_value;
  return bytes <= 16e6;
}

// Where the few-row layer leaves the few-row kernels (42-layer decode steps, tokens/s, against 16 rows
// for the projections and 12 for the one-pass gate/up): q/k/v, o and down take the tiled kernel above
// kTiledRows token rows (B = 4 944 -> 983, B = 8 1705 -> 1838, B = 12 2224 -> 2586, B = 16 2944 ->
// 3288; tiling one or two rows was 8% slower), gate/up the one-pass few-row kernel up to kGatedRows
// (the tiled gated product ties at 8 rows and wins from 12), and the PLE pair the tiled kernel above
// kTiledPleRows (equal at 32 rows, ahead at 64).
constexpr int64_t kTiledRows = 2, kGatedRows = 8, kTiledPleRows = 16;

// A few-row product on the tiled kernel (one 64-row tile over the token rows), K split into float32
// slices [slice][M][N] of the stacked matrices' rows: about 256 (tile, K slice) pairs, slices of at
// least 256 k, none empty, and no more slices than `out` holds. The few-row kernel re-stages the
// activations for every 16 or 64 weight rows, as many bytes as it streams at 64 rows. Returns false,
// with nothing launched, when the tiled kernel does not take the shape.
static bool tiled_slices(const void* A, int64_t lda, const void* const* segs, const int64_t* rows, int nseg,
                         int64_t ldb, int64_t M, int64_t K, float* out, size_t out_bytes, int* slices,
                         hipStream_t s, g4_status* st) {
  int64_t N = 0;
  for (int i = 0; i < nseg; ++i) N += rows[i];
  GemmArgs ga{};
  ga.A = A; ga.lda = lda; ga.B = segs[0]; ga.ldb = ldb; ga.C = out; ga.ldc = N; ga.c_dtype = G4_F32;
  ga.M = M; ga.N = N; ga.K = K; ga.epi = EPI_STORE; ga.splits = 1; ga.split_stride = M * N;
  if (nseg > 1) {
    ga.nseg = nseg;
    for (int i = 0; i < nseg; ++i) { ga.segB[i] = segs[i]; ga.seg_rows[i] = rows[i]; }
  }
  const int cols = gemm_rows64_cols(ga);
  if (cols == 0) return false;
  const int64_t tiles = N / cols;
  int64_t sd = 256 / tiles < K / 256 ? 256 / tiles : K / 256;
  if (sd < 1) sd = 1;
  const int64_t kper = ((K + sd - 1) / sd + 63) / 64 * 64;  // the kernel's slice length
  sd = (K + kper - 1) / kper;                               // so that no slice is empty
  while (sd > 1 && (size_t)sd * M * N * 4 > out_bytes) --sd;
  if ((size_t)sd * M * N * 4 > out_bytes) return false;
  ga.splits = (int32_t)sd;
  if (!gemm_mfma(ga, s, st)) return false;
  *slices = (int)sd;
  return true;
}

static g4_status few_row_layer(const LayerCtx& c) {
  const g4_model_desc* m = c.m;
  const g4_layer_desc* l = c.l;
  const int32_t dt = m->dtype;
  const size_t E = dsize(dt);
  const int64_t M = c.B * c.T, H = m->hidden, nh = m->n_heads, d = m->ple_dim;
  const int sliding = l->sliding;
  const int64_t nkv = kv_heads(m, sliding), F = ffn_of(m, l);
  const int64_t hd = sliding ? m->head_dim_swa : m->head_dim_full;
  const bool own = l->kv_src == c.layer;
  const bool vk = v_from_k(m, l);
  char* xn = c.ws + c.p->xn;
  char* qkv = c.ws + c.p->qkv;
  char* ao = c.ws + c.p->ao;
  char* hb = c.ws + c.p->hb;
  char* act = c.ws + c.p->act;
  char* gm = c.ws + c.p->gm;
  float* X = (float*)(c.ws + c.p->fx);
  float* Y = (float*)(c.ws + c.p->fy);
  const size_t XB = c.p->fx_bytes, YB = c.p->fy_bytes;
  const int64_t qld = c.p->qkv_ld;
  g4_status st;
#define G4_TRY(x)                 \
  do {                            \
    if ((st = (x)) != G4_OK) return st; \
  } while (0)
  if (!c.xn_ready)
    G4_TRY(rownorm(c.h, G4_F32, 1, 0, l->input_norm, xn, nullptr, 1.f, nullptr, nullptr, M, H, m->eps, dt, c.s));
  // q, k, v partials, then per-head norms + RoPE from their sums; k and v land in the cache (with K=V
  // there is no v projection: the v heads are formed from the k partials, without scale and rotation)
  const int nseg = own ? (vk ? 2 : 3) : 1;
  const int64_t Nq = nh * hd + (nseg - 1) * nkv * hd;
  int s1 = 0;
  {
    TimedScope ts(G4_KC_QKV_GEMM, c.s);
    const void* segs[3] = {l->wq, l->wk, l->wv};
    const int64_t rows[3] = {nh * hd, nkv * hd, nkv * hd};
    g4_status mst = G4_OK;
    if (M > kTiledRows && tiled_slices(xn, H, segs, rows, nseg, H, M, H, X, XB, &s1, c.s, &mst)) {
      G4_TRY(mst);
    } else {
      SkA sa{};
      sa.a = xn; sa.lda = H; sa.kind = SKA_BF16;
      G4_TRY(gemm_skinny_part(sa, M, H, segs, rows, nseg, H, X, XB, &s1, c.s));
    }
  }
  const g4_kv_entry& src = c.kv[l->kv_src];
  AttnArgs aa{};
  aa.q = qkv; aa.q_ld = qld; aa.k = src.k; aa.v = src.v; aa.cap = src.cap; aa.pos0 = c.pos;
  aa.B = c.B; aa.T = c.T; aa.nh = nh; aa.nkv = nkv; aa.hd = hd; aa.sliding = sliding; aa.window = m->window;
  aa.scale = 1.f; aa.out = ao; aa.out_ld = nh * hd; aa.ring = src.ring; aa.bidir = c.mode == G4_ENCODE;
  const float theta = sliding ? m->theta_swa : m->theta_full;
  // decode: the attention launch forms q, and on a layer that owns its cache the new key's k and v, from
  // the partials itself (one launch fewer per layer); otherwise the head-norm kernel writes q and the
  // cache rows first
  bool fused = false;
  if (c.mode == G4_DECODE && dt == G4_BF16) {
    DecFuse f{};
    f.x = X; f.x_ld = Nq; f.part_stride = M * Nq; f.parts = s1;
    f.q_off = 0;
    f.k_off = own ? nh * hd : -1;
    f.v_off = own ? (vk ? nh : nh + nkv) * hd : -1;
    f.qw = (const bf16*)l->q_norm; f.kw = (const bf16*)l->k_norm;
    f.n_rot = (int32_t)rot_pairs(m, sliding); f.eps = m->eps;
    rope_table(f.tab, theta, hd, f.n_rot);
    TimedScope ts(G4_KC_ATTENTION, c.s);
    g4_status mst = G4_OK;
    fused = attn_decode_fused(aa, f, c.ws + c.p->dec, c.p->fx - c.p->dec, c.s, &mst);
    if (fused) G4_TRY(mst);
  }
  if (!fused) {
    {
      TimedScope ts(G4_KC_QK_NORM_ROPE, c.s);
      HeadSeg segs[3];
      int ns = 0;
      segs[ns++] = HeadSeg{X, Nq, l->q_norm, qkv, qld, 0, (int32_t)nh, 1};
      if (own) {
        const g4_kv_entry& e = c.kv[c.layer];
        segs[ns++] = HeadSeg{X + nh * hd, Nq, l->k_norm, e.k, 0, e.cap, (int32_t)nkv, 1, e.ring};
        segs[ns++] = HeadSeg{X + (vk ? nh : nh + nkv) * hd, Nq, nullptr, e.v, 0, e.cap, (int32_t)nkv, 0, e.ring};
      }
      G4_TRY(qk_norm_rope_parts(segs, ns, s1, M * Nq, c.pos, c.B, c.T, hd, theta, rot_pairs(m, sliding), m->eps, dt,
                                c.s));
    }
    TimedScope ts(G4_KC_ATTENTION, c.s);
    if (c.mode == G4_DECODE) G4_TRY(attn_decode(aa, c.ws + c.p->dec, c.p->fx - c.p->dec, dt, c.s));
    else G4_TRY(attn_prefill(aa, dt, c.s));
  }
  const void* wo[1] = {l->wo};
  const void* wd[1] = {l->w_down};
  const void* wpg[1] = {l->ple_gate};
  const void* wpp[1] = {l->ple_proj};
  const int64_t rH[1] = {H}, rd[1] = {d};
  // o projection; h += rms(a) * w_pa; xn2 = rms(h) * w_pf
  int s2 = 0;
  {
    TimedScope ts(G4_KC_O_GEMM, c.s);
    g4_status mst = G4_OK;
    if (M > kTiledRows && tiled_slices(ao, nh * hd, wo, rH, 1, nh * hd, M, nh * hd, Y, YB, &s2, c.s, &mst)) {
      G4_TRY(mst);
    } else {
      SkA sa{};
      sa.a = ao; sa.lda = nh * hd; sa.kind = SKA_BF16;
      G4_TRY(gemm_skinny_part(sa, M, nh * hd, wo, rH, 1, nh * hd, Y, YB, &s2, c.s));
    }
  }
  {
    TimedScope ts(G4_KC_ROW_TAIL, c.s);
    G4_TRY(rownorm(Y, G4_F32, s2, M * H, l->post_attn_norm, nullptr, c.h, 1.f, l->pre_ffn_norm, xn, M, H, m->eps,
                   dt, c.s));
  }
  // gate/up: up to kGatedRows one weight-streaming pass writes the bf16 product; above that the tiled
  // gated-product kernel does. Decode steps, 42 layers (gate/up ms per step, one pass / 64-row tiles):
  // 1.22 / 1.23 at 8 rows, 1.51 / 1.24 at 12; at 64 rows the split-K few-row form took 2.83 against
  // 1.77 on 128-row tiles and 1.52 on 64-row ones (each few-row block re-stages as many activation
  // bytes as it streams weights). Failing both, partials, whose gelu_tanh(gate) * up the down
  // projection forms in its A.
  int s3 = 0, s4 = 0;
  bool gated = false;  // act holds the bf16 product
  {
    TimedScope ts(G4_KC_GATE_UP_GEMM, c.s);
    SkA sa{};
    sa.a = xn; sa.lda = H; sa.kind = SKA_BF16;
    if (M <= kGatedRows && skinny_gated_ok(M, H, F)) {
      G4_TRY(gemm_skinny_gated(sa, M, H, l->w_gate, l->w_up, F, H, act, F, c.s));
      gated = true;
    } else {
      GemmArgs ga{};
      ga.A = xn; ga.lda = H; ga.B = l->w_gate; ga.B2 = l->w_up; ga.ldb = H; ga.C = act; ga.ldc = F; ga.c_dtype = dt;
      ga.M = M; ga.N = F; ga.K = H; ga.epi = EPI_GEGLU; ga.splits = 1;
      g4_status mst = G4_OK;
      if (gemm_mfma(ga, c.s, &mst)) {
        G4_TRY(mst);
        gated = true;
      } else if (skinny_gated_ok(M, H, F)) {
        G4_TRY(gemm_skinny_gated(sa, M, H, l->w_gate, l->w_up, F, H, act, F, c.s));
        gated = true;
      }
    }
    if (!gated) {
      const void* segs[2] = {l->w_gate, l->w_up};
      const int64_t rows[2] = {F, F};
      G4_TRY(gemm_skinny_part(sa, M, H, segs, rows, 2, H, X, XB, &s3, c.s));
    }
  }
  {
    TimedScope ts(G4_KC_DOWN_GEMM, c.s);
    // with the product in act: the tiled kernel, K split into slices the row tail sums
    bool down_done = false;
    if (gated && M > kTiledRows) {
      g4_status mst = G4_OK;
      down_done = tiled_slices(act, F, wd, rH, 1, F, M, F, Y, YB, &s4, c.s, &mst);
      if (down_done) G4_TRY(mst);
    }
    if (!down_done) {
      SkA sa{};
      if (gated) {
        sa.a = act; sa.lda = F; sa.kind = SKA_BF16;
      } else if (stage_from_parts(M, F, H, s3, 2)) {
        sa.a = X; sa.lda = 2 * F; sa.kind = SKA_GEGLU; sa.parts = s3; sa.part_stride = M * 2 * F; sa.up_off = F;
      } else {
        GemmArgs ga{};
        ga.M = M; ga.N = F; ga.C = act; ga.ldc = F; ga.c_dtype = dt; ga.epi = EPI_GEGLU;
        G4_TRY(gemm_skinny_finish(ga, X, s3, 2 * F, c.s));
        sa.a = act; sa.lda = F; sa.kind = SKA_BF16;
      }
      G4_TRY(gemm_skinny_part(sa, M, F, wd, rH, 1, F, Y, YB, &s4, c.s));
    }
  }
  {
    TimedScope ts(G4_KC_ROW_TAIL, c.s);
    G4_TRY(rownorm(Y, G4_F32, s4, M * H, l->post_ffn_norm, nullptr, c.h, 1.f, nullptr, hb, M, H, m->eps, dt, c.s));
  }
  // PLE: gate partials from the raw residual; up to kTiledPleRows the projection forms
  // gelu_tanh(gate) * ple_in while staging. Above, both products run on the tiled kernel with a
  // finishing pass between them: each few-row projection block would re-form 64 x 256 activations from
  // every gate slice, ten times its own weight bytes (64 rows, 42 layers: 0.82 against 1.11 ms per step;
  // no change at 32).
  int s5 = 0, s6 = 0;
  {
    TimedScope ts(G4_KC_PLE_GEMM, c.s);
    bool gate_tiled = false;
    if (M > kTiledPleRows) {
      g4_status mst = G4_OK;
      gate_tiled = tiled_slices(hb, H, wpg, rd, 1, H, M, H, X, XB, &s5, c.s, &mst);
      if (gate_tiled) G4_TRY(mst);
    }
    if (!gate_tiled) {
      SkA sa{};
      sa.a = hb; sa.lda = H; sa.kind = SKA_BF16;
      G4_TRY(gemm_skinny_part(sa, M, H, wpg, rd, 1, H, X, XB, &s5, c.s));
    }
    const float* ple_l = c.ple_in + (int64_t)c.layer * d;
    SkA sb{};
    if (M <= kTiledPleRows && stage_from_parts(M, d, H, s5, 1)) {
      sb.a = X; sb.lda = d; sb.kind = SKA_GELU_MUL; sb.parts = s5; sb.part_stride = M * d;
      sb.aux = ple_l; sb.aux_ld = m->n_layers * d;
    } else {
      GemmArgs ga{};
      ga.M = M; ga.N = d; ga.C = gm; ga.ldc = d; ga.c_dtype = dt; ga.epi = EPI_GELU_MUL;
      ga.aux = ple_l; ga.aux_ld = m->n_layers * d;
      G4_TRY(gemm_skinny_finish(ga, X, s5, d, c.s));
      sb.a = gm; sb.lda = d; sb.kind = SKA_BF16;
    }
    bool proj_tiled = false;
    if (M > kTiledPleRows) {
      g4_status mst = G4_OK;
      proj_tiled = tiled_slices(gm, d, wpp, rH, 1, d, M, d, Y, YB, &s6, c.s, &mst);
      if (proj_tiled) G4_TRY(mst);
    }
    if (!proj_tiled) G4_TRY(gemm_skinny_part(sb, M, d, wpp, rH, 1, d, Y, YB, &s6, c.s));
  }
  {
    TimedScope ts(G4_KC_ROW_TAIL, c.s);
    G4_TRY(rownorm(Y, G4_F32, s6, M * H, l->post_ple_norm, nullptr, c.h, l->layer_scalar, c.next_input_norm,
                   c.next_input_norm ? xn : nullptr, M, H, m->eps, dt, c.s));
  }
#undef G4_TRY
  (void)E;
  return G4_OK;
}

static g4_status layer_impl(const LayerCtx& c) {
  if (c.B * c.T > 0 && few_row_ok(c)) return few_row_layer(c);
  const g4_model_desc* m = c.m;
  const g4_layer_desc* l = c.l;
  const int32_t dt = m->dtype;
  const size_t E = dsize(dt);
  const int64_t M = c.B * c.T, H = m->hidden, nh = m->n_heads, d = m->ple_dim;
  const int sliding = l->sliding;
  const int64_t nkv = kv_heads(m, sliding), F = ffn_of(m, l);
  const int64_t hd = sliding ? m->head_dim_swa : m->head_dim_full;
  const bool vk = v_from_k(m, l);
  const float theta = sliding ? m->theta_swa : m->theta_full;
  const int64_t nrot = rot_pairs(m, sliding);
  const bool own = l->kv_src == c.layer;
  char* xn = c.ws + c.p->xn;
  char* qkv = c.ws + c.p->qkv;
  char* ao = c.ws + c.p->ao;
  float* fb = (float*)(c.ws + c.p->f32buf);
  char* act = c.ws + c.p->act;
  char* hb = c.ws + c.p->hb;
  char* gm = c.ws + c.p->gm;
  const int64_t qld = c.p->qkv_ld;
  g4_status st;
#define G4_TRY(x)                 \
  do {                            \
    if ((st = (x)) != G4_OK) return st; \
  } while (0)
  if (M == 0) return G4_OK;
  g_gws = c.ws + c.p->gws;
  g_gws_bytes = c.p->gws_bytes;
  struct ClearGws { ~ClearGws() { g_gws = nullptr; g_gws_bytes = 0; } } clear_gws;
  // 1. pre-attention norm
  if (!c.xn_ready)
    G4_TRY(rownorm(c.h, G4_F32, 1, 0, l->input_norm, xn, nullptr, 1.f, nullptr, nullptr, M, H, m->eps, dt, c.s));
  // 2. projections: q, and k, v when the layer owns its cache (k only with K=V: v is formed from it)
  {
    TimedScope ts(G4_KC_QKV_GEMM, c.s);
    GemmArgs ga{};
    ga.A = xn; ga.lda = H; ga.ldb = H; ga.C = qkv; ga.ldc = qld; ga.c_dtype = dt; ga.M = M; ga.K = H;
    ga.epi = EPI_STORE; ga.splits = 1; ga.ws = g_gws; ga.ws_bytes = g_gws_bytes;
    ga.nseg = own ? (vk ? 2 : 3) : 1;
    ga.segB[0] = l->wq; ga.seg_rows[0] = nh * hd;
    ga.segB[1] = l->wk; ga.seg_rows[1] = nkv * hd;
    ga.segB[2] = l->wv; ga.seg_rows[2] = nkv * hd;
    ga.N = nh * hd + (ga.nseg - 1) * nkv * hd;
    ga.B = l->wq;
    G4_TRY(gemm(ga, dt, c.s));
  }
  // 3. per-head norms + RoPE; k and v go straight into this layer's cache rows
  HeadSeg segs[3];
  int ns = 0;
  segs[ns++] = HeadSeg{qkv, qld, l->q_norm, qkv, qld, 0, (int32_t)nh, 1};
  if (own) {
    const g4_kv_entry& e = c.kv[c.layer];
    segs[ns++] = HeadSeg{qkv + nh * hd * E, qld, l->k_norm, e.k, 0, e.cap, (int32_t)nkv, 1, e.ring};
    segs[ns++] = HeadSeg{qkv + (vk ? nh : nh + nkv) * hd * E, qld, nullptr, e.v, 0, e.cap, (int32_t)nkv, 0, e.ring};
  }
  {
    TimedScope ts(G4_KC_QK_NORM_ROPE, c.s);
    G4_TRY(qk_norm_rope(segs, ns, c.pos, c.B, c.T, hd, theta, nrot, m->eps, dt, c.s));
  }
  // 4. attention over the source layer's cache (no copy)
  const g4_kv_entry& src = c.kv[l->kv_src];
  AttnArgs aa{};
  aa.q = qkv; aa.q_ld = qld; aa.k = src.k; aa.v = src.v; aa.cap = src.cap; aa.pos0 = c.pos;
  aa.B = c.B; aa.T = c.T; aa.nh = nh; aa.nkv = nkv; aa.hd = hd; aa.sliding = sliding; aa.window = m->window;
  aa.scale = 1.f; aa.out = ao; aa.out_ld = nh * hd; aa.ring = src.ring; aa.bidir = c.mode == G4_ENCODE;
  aa.ws = (float*)(c.ws + c.p->aws); aa.ws_bytes = c.p->aws_bytes;
  {
    TimedScope ts(G4_KC_ATTENTION, c.s);
    if (c.mode == G4_DECODE) G4_TRY(attn_decode(aa, c.ws + c.p->dec, c.p->total - c.p->dec, dt, c.s));
    else G4_TRY(attn_prefill(aa, dt, c.s));
  }
  // 5-6. o projection, then h += rms(a) * w_pa and xn2 = rms(h) * w_pf
  const int32_t so = gemm_pick_splits(M, H, nh * hd, (int32_t)c.p->splits);
  {
  TimedScope ts(G4_KC_O_GEMM, c.s);
  G4_TRY(run_gemm(ao, nh * hd, l->wo, nullptr, nh * hd, fb, H, G4_F32, M, H, nh * hd, EPI_STORE, nullptr, 0, so,
                  M * H, dt, c.s));
  }
  {
  TimedScope ts(G4_KC_ROW_TAIL, c.s);
  G4_TRY(rownorm(fb, G4_F32, so, M * H, l->post_attn_norm, nullptr, c.h, 1.f, l->pre_ffn_norm, xn, M, H, m->eps, dt,
                 c.s));
  // 7. gate/up GEMM with the gelu-tanh product in its epilogue
  }
  {
    TimedScope ts(G4_KC_GATE_UP_GEMM, c.s);
    G4_TRY(run_gemm(xn, H, l->w_gate, l->w_up, H, act, F, dt, M, F, H, EPI_GEGLU, nullptr, 0, 1, 0, dt, c.s));
  }
  // 8-9. down projection, then h += rms(ffn) * w_pff; hb = h in dtype for the PLE gate
  const int32_t sd = gemm_pick_splits(M, H, F, (int32_t)c.p->splits);
  {
  TimedScope ts(G4_KC_DOWN_GEMM, c.s);
  G4_TRY(run_gemm(act, F, l->w_down, nullptr, F, fb, H, G4_F32, M, H, F, EPI_STORE, nullptr, 0, sd, M * H, dt, c.s));
  }
  {
  TimedScope ts(G4_KC_ROW_TAIL, c.s);
  G4_TRY(rownorm(fb, G4_F32, sd, M * H, l->post_ffn_norm, nullptr, c.h, 1.f, nullptr, hb, M, H, m->eps, dt, c.s));
  }
  // 10. PLE gate: gelu_tanh(h W_pg^T) * ple_in[:, layer]
  const int64_t Ld = m->n_layers * d;
  {
  TimedScope ts(G4_KC_PLE_GEMM, c.s);
  G4_TRY(run_gelu_mul(hb, H, l->ple_gate, H, gm, d, c.ple_in + (int64_t)c.layer * d, Ld, M, d, H, dt, fb,
                      (size_t)c.p->splits * M * H * 4, c.s));
  // 11-12. PLE projection, h = (h + rms(p) * w_post_ple) * layer_scalar (+ next layer's xn)
  G4_TRY(run_gemm(gm, d, l->ple_proj, nullptr, d, fb, H, G4_F32, M, H, d, EPI_STORE, nullptr, 0, 1, M * H, dt, c.s));
  }
  {
  TimedScope ts(G4_KC_ROW_TAIL, c.s);
  G4_TRY(rownorm(fb, G4_F32, 1, M * H, l->post_ple_norm, nullptr, c.h, l->layer_scalar, c.next_input_norm,
                 c.next_input_norm ? xn : nullptr, M, H, m->eps, dt, c.s));
  }
#undef G4_TRY
  return G4_OK;
}

}  // namespace g4

using namespace g4;

extern "C" {

const char* g4_status_str(int status) {
  switch (status) {
    case G4_OK: return "G4_OK";
    case G4_EINVAL: return "G4_EINVAL";
    case G4_EGEOM: return "G4_EGEOM";
    case G4_ERANGE: return "G4_ERANGE";
    case G4_EHIP: return "G4_EHIP";
    case G4_EUNSUP: return "G4_EUNSUP";
    default: return "G4_UNKNOWN";
  }
}

const char* g4_last_error(void) { return g_last_error.c_str(); }

int g4_version(void) { return 300; }

g4_status g4_kv_sources(const int32_t* sliding, int32_t n_layers, int32_t n_shared, int32_t* kv_src) {
  G4_REQ(sliding && kv_src, G4_EINVAL, "sliding or kv_src is NULL");
  G4_REQ(n_layers > 0 && n_shared >= 0 && n_shared <= n_layers, G4_EINVAL, "n_layers %d, n_shared %d", n_layers,
         n_shared);
  const int32_t first_shared = n_layers - n_shared;
  for (int32_t l = 0; l < n_layers; ++l) {
    G4_REQ(sliding[l] == 0 || sliding[l] == 1, G4_EINVAL, "sliding[%d] must be 0 or 1", l);
    kv_src[l] = l;
    if (l < first_shared) continue;
    for (int32_t j = first_shared - 1; j >= 0; --j)
      if (sliding[j] == sliding[l]) {
        kv_src[l] = j;
        break;
      }
  }
  return G4_OK;
}

g4_status g4_rmsnorm(const void* x, int32_t x_dtype, int32_t x_parts, const void* w, void* y, float* res,
                     float res_scale, const void* w_next, void* y_next, int64_t rows, int64_t dim, float eps,
                     int32_t dtype, void* stream) {
  G4_REQ(dt_ok(dtype), G4_EINVAL, "dtype %d", dtype);
  G4_REQ(x_dtype == G4_F32 || x_dtype == dtype, G4_EINVAL, "x_dtype must be G4_F32 or dtype");
  G4_REQ(rows >= 0 && dim > 0, G4_EINVAL, "rows %lld / dim %lld", (long long)rows, (long long)dim);
  if (rows == 0) return G4_OK;
  G4_REQ(x, G4_EINVAL, "x is NULL");
  G4_REQ(dim <= 16384, G4_ERANGE, "dim %lld > 16384", (long long)dim);
  G4_REQ(x_parts >= 1, G4_EINVAL, "x_parts %d < 1", x_parts);
  G4_REQ(!y_next || res, G4_EINVAL, "y_next requires res");
  G4_REQ(y || res, G4_EINVAL, "nothing to write: y and res are NULL");
  G4_REQ(eps >= 0.f, G4_EINVAL, "eps < 0");
  return rownorm(x, x_dtype, x_parts, rows * dim, w, y, res, res_scale, w_next, y_next, rows, dim, eps, dtype,
                 (hipStream_t)stream);
}

g4_status g4_qk_norm_rope(const void* x, int64_t x_ld, const void* w, void* y, int64_t y_ld, int64_t y_cap,
                          const int32_t* pos, int64_t B, int64_t T, int64_t heads, int64_t hd, float theta,
                          int64_t rotated_pairs, float eps, int32_t dtype, void* stream) {
  G4_REQ(dt_ok(dtype), G4_EINVAL, "dtype %d", dtype);
  G4_REQ(B >= 0 && T >= 0 && heads > 0 && hd > 0, G4_EINVAL, "sizes must be positive");
  if (B * T == 0) return G4_OK;
  G4_REQ(x && y, G4_EINVAL, "x or y is NULL");
  G4_REQ(hd % 2 == 0, G4_EGEOM, "head_dim %lld is odd", (long long)hd);
  G4_REQ(hd <= 512, G4_ERANGE, "head_dim %lld > 512", (long long)hd);
  G4_REQ(x_ld >= heads * hd, G4_EINVAL, "x_ld %lld < heads*hd", (long long)x_ld);
  G4_REQ(y_cap > 0 || y_ld >= heads * hd, G4_EINVAL, "y_ld %lld < heads*hd", (long long)y_ld);
  G4_REQ(y_cap >= 0, G4_EINVAL, "y_cap < 0");
  G4_REQ(y_cap == 0 || T <= y_cap, G4_ERANGE, "T %lld > cache capacity %lld", (long long)T, (long long)y_cap);
  G4_REQ(rotated_pairs >= 0 && rotated_pairs <= hd / 2, G4_ERANGE, "rotated_pairs %lld outside [0, hd/2]",
         (long long)rotated_pairs);
  G4_REQ(pos || (rotated_pairs == 0 && y_cap == 0), G4_EINVAL, "pos is NULL");
  G4_REQ(rotated_pairs == 0 || theta > 0.f, G4_EINVAL, "theta <= 0");
  HeadSeg sg{x, x_ld, w, y, y_ld, y_cap, (int32_t)heads, rotated_pairs > 0 ? 1 : 0};
  return qk_norm_rope(&sg, 1, pos, B, T, hd, theta, rotated_pairs, eps, dtype, (hipStream_t)stream);
}

static g4_status check_attn(const void* q, int64_t q_ld, const g4_kv_entry* kv, int32_t n_kv, int32_t layer,
                            int32_t kv_src, int32_t sliding, int64_t window, const int32_t* pos, int64_t B,
                            int64_t T, int64_t nh, int64_t nkv, int64_t hd, void* out, int64_t out_ld,
                            int32_t dtype, int32_t mode) {
  G4_REQ(dt_ok(dtype), G4_EINVAL, "dtype %d", dtype);
  G4_REQ(B >= 0 && T >= 0 && nh > 0 && nkv > 0 && hd > 0, G4_EINVAL, "sizes must be positive");
  G4_REQ(B * T == 0 || (q && out && pos), G4_EINVAL, "q, out or pos is NULL");
  G4_REQ(nh % nkv == 0, G4_EGEOM, "nh %lld is not a multiple of nkv %lld", (long long)nh, (long long)nkv);
  G4_REQ(hd <= 512, G4_ERANGE, "head_dim %lld > 512", (long long)hd);
  G4_REQ(q_ld >= nh * hd && out_ld >= nh * hd, G4_EINVAL, "q_ld/out_ld smaller than nh*hd");
  G4_REQ(sliding == 0 || sliding == 1, G4_EINVAL, "sliding must be 0 or 1");
  G4_REQ(!sliding || window >= 1, G4_ERANGE, "window %lld < 1", (long long)window);
  return check_kv(kv, n_kv, layer, kv_src, sliding, hd, T, mode, window);
}

size_t g4_attn_prefill_ws(int64_t B, int64_t T, int64_t nh, int64_t nkv, int64_t hd) {
  if (B <= 0 || T <= 0 || nh <= 0 || nkv <= 0 || hd <= 0 || nh % nkv) return 0;
  return attn_prefill_ws(B, T, nh, nkv, hd);
}

static g4_status attn_prefill_entry(const void* q, int64_t q_ld, const g4_kv_entry* kv, int32_t n_kv, int32_t layer,
                                    int32_t kv_src, int32_t sliding, int64_t window, const int32_t* pos0, int64_t B,
                                    int64_t T, int64_t nh, int64_t nkv, int64_t hd, float scale, void* out,
                                    int64_t out_ld, void* ws, size_t ws_bytes, int32_t dtype, void* stream,
                                    int32_t mode) {
  g4_status st = check_attn(q, q_ld, kv, n_kv, layer, kv_src, sliding, window, pos0, B, T, nh, nkv, hd, out,
                            out_ld, dtype, mode);
  if (st != G4_OK) return st;
  if (ws) {
    const size_t need = g4_attn_prefill_ws(B, T, nh, nkv, hd);
    G4_REQ(ws_bytes >= need, G4_EINVAL, "attention workspace too small (%zu < %zu)", ws_bytes, need);
    G4_REQ(((uintptr_t)ws & 15) == 0, G4_EINVAL, "attention workspace is not 16-byte aligned");
  }
  AttnArgs a{};
  a.ws = (float*)ws; a.ws_bytes = ws ? ws_bytes : 0;
  a.q = q; a.q_ld = q_ld; a.k = kv[kv_src].k; a.v = kv[kv_src].v; a.cap = kv[kv_src].cap; a.pos0 = pos0;
  a.B = B; a.T = T; a.nh = nh; a.nkv = nkv; a.hd = hd; a.sliding = sliding; a.window = window; a.scale = scale;
  a.out = out; a.out_ld = out_ld; a.ring = kv[kv_src].ring; a.bidir = mode == G4_ENCODE;
  if (B * T == 0) return G4_OK;
  return attn_prefill(a, dtype, (hipStream_t)stream);
}

g4_status g4_attn_prefill(const void* q, int64_t q_ld, const g4_kv_entry* kv, int32_t n_kv, int32_t layer,
                          int32_t kv_src, int32_t sliding, int64_t window, const int32_t* pos0, int64_t B,
                          int64_t T, int64_t nh, int64_t nkv, int64_t hd, float scale, void* out, int64_t out_ld,
                          void* ws, size_t ws_bytes, int32_t dtype, void* stream) {
  return attn_prefill_entry(q, q_ld, kv, n_kv, layer, kv_src, sliding, window, pos0, B, T, nh, nkv, hd, scale, out,
                            out_ld, ws, ws_bytes, dtype, stream, G4_PREFILL);
}

g4_status g4_attn_encode(const void* q, int64_t q_ld, const g4_kv_entry* kv, int32_t n_kv, int32_t layer,
                         int32_t kv_src, int32_t sliding, int64_t window, const int32_t* pos0, int64_t B,
                         int64_t T, int64_t nh, int64_t nkv, int64_t hd, float scale, void* out, int64_t out_ld,
                         void* ws, size_t ws_bytes, int32_t dtype, void* stream) {
  return attn_prefill_entry(q, q_ld, kv, n_kv, layer, kv_src, sliding, window, pos0, B, T, nh, nkv, hd, scale, out,
                            out_ld, ws, ws_bytes, dtype, stream, G4_ENCODE);
}

size_t g4_attn_decode_ws(int64_t B, int64_t nh, int64_t hd, int64_t cap) { return attn_decode_ws(B, nh, hd, cap); }

g4_status g4_attn_decode(const void* q, int64_t q_ld, const g4_kv_entry* kv, int32_t n_kv, int32_t layer,
                         int32_t kv_src, int32_t sliding, int64_t window, const int32_t* pos, int64_t B, int64_t nh,
                         int64_t nkv, int64_t hd, float scale, void* out, int64_t out_ld, void* ws, size_t ws_bytes,
                         int32_t dtype, void* stream) {
  g4_status st = check_attn(q, q_ld, kv, n_kv, layer, kv_src, sliding, window, pos, B, 1, nh, nkv, hd, out, out_ld,
                            dtype, G4_DECODE);
  if (st != G4_OK) return st;
  if (B == 0) return G4_OK;
  G4_REQ(ws, G4_EINVAL, "workspace is NULL");
  AttnArgs a{};
  a.q = q; a.q_ld = q_ld; a.k = kv[kv_src].k; a.v = kv[kv_src].v; a.cap = kv[kv_src].cap; a.pos0 = pos;
  a.B = B; a.T = 1; a.nh = nh; a.nkv = nkv; a.hd = hd; a.sliding = sliding; a.window = window; a.scale = scale;
  a.out = out; a.out_ld = out_ld; a.ring = kv[kv_src].ring;
  return attn_decode(a, ws, ws_bytes, dtype, (hipStream_t)stream);
}

g4_status g4_linear(const void* A, const void* W, void* C, int64_t M, int64_t N, int64_t K, int32_t c_dtype,
                    int32_t dtype, void* ws, size_t ws_bytes, void* stream) {
  (void)ws; (void)ws_bytes;
  G4_REQ(dt_ok(dtype), G4_EINVAL, "dtype %d", dtype);
  G4_REQ(c_dtype == G4_F32 || c_dtype == dtype, G4_EINVAL, "c_dtype must be G4_F32 or dtype");
  G4_REQ(M >= 0 && N > 0 && K > 0, G4_EINVAL, "M %lld N %lld K %lld", (long long)M, (long long)N, (long long)K);
  if (M == 0) return G4_OK;
  G4_REQ(A && W && C, G4_EINVAL, "A, W or C is NULL");
  g_gws = ws;  // optional scratch for the few-row kernel
  g_gws_bytes = ws ? ws_bytes : 0;
  const g4_status st =
      run_gemm(A, K, W, nullptr, K, C, N, c_dtype, M, N, K, EPI_STORE, nullptr, 0, 1, 0, dtype, (hipStream_t)stream);
  g_gws = nullptr;
  g_gws_bytes = 0;
  return st;
}

size_t g4_logits_ws(int64_t M, int64_t H, int64_t vocab, int32_t dtype) {
  if (M <= 0 || H <= 0 || vocab <= 0) return 0;
  size_t sk = 0;
  if (M <= 64 && dtype == G4_BF16) sk = gemm_skinny_ws(M, (vocab + 63) / 64 * 64, (H + 127) / 128 * 128);
  return al((size_t)M * H * dsize(dtype)) + al(sk);
}

g4_status g4_logits(const float* h, int64_t M, int64_t H, const void* out_norm, const void* w_out, int64_t vocab,
                    float eps, float softcap, float* logits, void* ws, size_t ws_bytes, int32_t dtype, void* stream) {
  G4_REQ(dt_ok(dtype), G4_EINVAL, "dtype %d", dtype);
  G4_REQ(M >= 0 && H > 0 && vocab > 0, G4_EINVAL, "M %lld H %lld vocab %lld", (long long)M, (long long)H,
         (long long)vocab);
  G4_REQ(softcap >= 0.f, G4_EINVAL, "softcap %g < 0", (double)softcap);
  if (M == 0) return G4_OK;
  G4_REQ(h && out_norm && w_out && logits, G4_EINVAL, "h, out_norm, w_out or logits is NULL");
  const size_t need = g4_logits_ws(M, H, vocab, dtype);
  G4_REQ(ws && ws_bytes >= need, G4_EINVAL, "workspace too small (%zu < %zu)", ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  char* xn = (char*)ws;
  g_gws = (char*)ws + al((size_t)M * H * dsize(dtype));
  g_gws_bytes = ws_bytes - al((size_t)M * H * dsize(dtype));
  struct ClearGws { ~ClearGws() { g_gws = nullptr; g_gws_bytes = 0; } } clear_gws;
  g4_status st = rownorm(h, G4_F32, 1, 0, out_norm, xn, nullptr, 1.f, nullptr, nullptr, M, H, eps, dtype, s);
  if (st != G4_OK) return st;
  // up to 64 rows, the softcap in the product's last pass: the finisher of the few-row split-K product
  // (up to 16 rows) or the store of the 64-row tiles (17 to 64 rows, where wide products take them)
  if (dtype == G4_BF16 && softcap > 0.f && M <= 64) {
    GemmArgs ga{};
    ga.A = xn; ga.lda = H; ga.B = w_out; ga.ldb = H; ga.C = logits; ga.ldc = vocab; ga.c_dtype = G4_F32;
    ga.M = M; ga.N = vocab; ga.K = H; ga.epi = EPI_SOFTCAP; ga.cap = softcap; ga.splits = 1;
    ga.split_stride = M * vocab;
    if (M > 16) {
      if (gemm_mfma(ga, s, &st)) return st;
    } else {
      const void* segs[1] = {w_out};
      const int64_t rows[1] = {vocab};
      if (gemm_skinny(ga, segs, rows, 1, g_gws, g_gws_bytes, s, &st)) return st;
    }
  }
  st = run_gemm(xn, H, w_out, nullptr, H, logits, vocab, G4_F32, M, vocab, H, EPI_STORE, nullptr, 0, 1, 0, dtype, s);
  if (st != G4_OK) return st;
  return softcap_inplace(logits, M * vocab, softcap, s);
}

size_t g4_ffn_geglu_ws(int64_t M, int64_t H, int64_t F, int32_t dtype) {
  size_t sk = 0;
  if (M <= 64 && dtype == G4_BF16) {
    const size_t a = gemm_skinny_ws(M, (2 * F + 63) / 64 * 64, (H + 127) / 128 * 128);
    const size_t b = gemm_skinny_ws(M, (H + 63) / 64 * 64, (F + 127) / 128 * 128);
    sk = a > b ? a : b;
  }
  return al((size_t)M * F * dsize(dtype)) + al(sk);
}

g4_status g4_ffn_geglu(const void* x, const void* w_gate, const void* w_up, const void* w_down, float* out, int64_t M,
                       int64_t H, int64_t F, void* ws, size_t ws_bytes, int32_t dtype, void* stream) {
  G4_REQ(dt_ok(dtype), G4_EINVAL, "dtype %d", dtype);
  G4_REQ(M >= 0 && H > 0 && F > 0, G4_EINVAL, "sizes");
  if (M == 0) return G4_OK;
  G4_REQ(x && w_gate && w_up && w_down && out, G4_EINVAL, "a pointer is NULL");
  G4_REQ(ws && ws_bytes >= g4_ffn_geglu_ws(M, H, F, dtype), G4_EINVAL, "workspace too small (%zu < %zu)", ws_bytes,
         g4_ffn_geglu_ws(M, H, F, dtype));
  if (M == 0) return G4_OK;
  hipStream_t s = (hipStream_t)stream;
  g_gws = (char*)ws + al((size_t)M * F * dsize(dtype));
  g_gws_bytes = ws_bytes - al((size_t)M * F * dsize(dtype));
  g4_status st = run_gemm(x, H, w_gate, w_up, H, ws, F, dtype, M, F, H, EPI_GEGLU, nullptr, 0, 1, 0, dtype, s);
  if (st == G4_OK) st = run_gemm(ws, F, w_down, nullptr, F, out, H, G4_F32, M, H, F, EPI_STORE, nullptr, 0, 1, 0, dtype, s);
  g_gws = nullptr;
  g_gws_bytes = 0;
  return st;
}

size_t g4_ple_inject_ws(int64_t M, int64_t H, int64_t d, int32_t dtype) {
  return al((size_t)M * H * dsize(dtype)) + al((size_t)M * d * dsize(dtype)) + al((size_t)M * H * 4);
}

g4_status g4_ple_inject(float* h, const void* w_gate, const float* ple, int64_t ple_ld, const void* w_proj,
                        const void* w_post, float layer_scalar, int64_t M, int64_t H, int64_t d, float eps, void* ws,
                        size_t ws_bytes, int32_t dtype, void* stream) {
  G4_REQ(dt_ok(dtype), G4_EINVAL, "dtype %d", dtype);
  G4_REQ(M >= 0 && H > 0 && d > 0 && ple_ld >= d, G4_EINVAL, "sizes");
  if (M == 0) return G4_OK;
  G4_REQ(h && w_gate && ple && w_proj && w_post, G4_EINVAL, "a pointer is NULL");
  G4_REQ(H <= 16384, G4_ERANGE, "H > 16384");
  G4_REQ(ws && ws_bytes >= g4_ple_inject_ws(M, H, d, dtype), G4_EINVAL, "workspace too small");
  if (M == 0) return G4_OK;
  hipStream_t s = (hipStream_t)stream;
  char* hb = (char*)ws;
  char* gmb = hb + al((size_t)M * H * dsize(dtype));
  float* pb = (float*)(gmb + al((size_t)M * d * dsize(dtype)));
  g4_status st;
  if ((st = cast_rows(h, hb, M * H, dtype, s)) != G4_OK) return st;
  if ((st = run_gelu_mul(hb, H, w_gate, H, gmb, d, ple, ple_ld, M, d, H, dtype, pb, (size_t)M * H * 4, s)) != G4_OK)
    return st;
  if ((st = run_gemm(gmb, d, w_proj, nullptr, d, pb, H, G4_F32, M, H, d, EPI_STORE, nullptr, 0, 1, 0, dtype, s)) != G4_OK)
    return st;
  return rownorm(pb, G4_F32, 1, M * H, w_post, nullptr, h, layer_scalar, nullptr, nullptr, M, H, eps, dtype, s);
}

g4_status g4_embed_ple(const int32_t* ids, int64_t M, const void* E, const void* Tab, const void* W_pm,
                       const void* ple_norm, const g4_model_desc* model, float* h_out, float* ple_out, void* ws,
                       size_t ws_bytes, void* stream) {
  g4_status st = check_model(model);
  if (st != G4_OK) return st;
  G4_REQ(M >= 0, G4_EINVAL, "M < 0");
  if (M == 0) return G4_OK;
  G4_REQ(ids && E && Tab && W_pm && ple_norm && h_out && ple_out, G4_EINVAL, "a pointer is NULL");
  G4_REQ(model->vocab > 0 && model->ple_vocab > 0, G4_EINVAL, "vocab sizes must be positive");
  Plan p = plan(model, M, 1, 0, G4_PREFILL);
  G4_REQ(ws && ws_bytes >= p.total, G4_EINVAL, "workspace too small (%zu < %zu)", ws_bytes, p.total);
  if (M == 0) return G4_OK;
  hipStream_t s = (hipStream_t)stream;
  const int32_t dt = model->dtype;
  char* ecast = (char*)ws + p.emb_e;
  float* P = (float*)((char*)ws + p.emb_p);
  const int64_t Ld = model->n_layers * model->ple_dim;
  if ((st = embed_rows(ids, M, E, model->vocab, model->hidden, h_out, ecast, dt, s)) != G4_OK) return st;
  if ((st = run_gemm(ecast, model->hidden, W_pm, nullptr, model->hidden, P, Ld, G4_F32, M, Ld, model->hidden,
                     EPI_STORE, nullptr, 0, 1, 0, dt, s)) != G4_OK)
    return st;
  return ple_combine(ids, M, P, Tab, model->ple_vocab, ple_norm, model->hidden, model->n_layers, model->ple_dim,
                     model->eps, ple_out, dt, s);
}

g4_status g4_timer_enable(int32_t cls, int32_t max_launches) {
  G4_REQ(cls >= G4_KC_QKV_GEMM && cls <= G4_KC_ROW_TAIL, G4_EINVAL, "kernel class %d", cls);
  G4_REQ(max_launches > 0 && max_launches <= 1 << 20, G4_EINVAL, "max_launches %d", max_launches);
  if (g_timer.cap < max_launches) {
    hipEvent_t* ev = new hipEvent_t[2 * (size_t)max_launches];
    for (int32_t i = 0; i < 2 * max_launches; ++i) {
      if (hipEventCreate(&ev[i]) != hipSuccess) {
        for (int32_t j = 0; j < i; ++j) (void)hipEventDestroy(ev[j]);
        delete[] ev;
        return fail(G4_EHIP, "hipEventCreate failed");
      }
    }
    for (int32_t i = 0; i < 2 * g_timer.cap; ++i) (void)hipEventDestroy(g_timer.ev[i]);
    delete[] g_timer.ev;
    g_timer.ev = ev;
    g_timer.cap = max_launches;
  }
  g_timer.cls = cls;
  g_timer.n = 0;
  return G4_OK;
}

g4_status g4_timer_read(double* total_ms, int32_t* launches) {
  G4_REQ(total_ms && launches, G4_EINVAL, "NULL output");
  g_timer.cls = 0;
  double t = 0;
  for (int32_t i = 0; i < g_timer.n; ++i) {
    float ms = 0;
    if (hipEventSynchronize(g_timer.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_timer.ev[2 * i], g_timer.ev[2 * i + 1]) != hipSuccess)
      return fail(G4_EHIP, "event timing failed");
    t += ms;
  }
  *total_ms = t;
  *launches = g_timer.n;
  return G4_OK;
}

size_t g4_workspace_size(const g4_model_desc* model, int64_t B, int64_t T, int64_t cap, int32_t mode) {
  if (check_model(model) != G4_OK || B < 0 || T < 0) return 0;
  return plan(model, B, T, cap, mode).total;
}

// Plan of a layer-forward call over the caches its layers read: decode partials are sized by the largest
// capacity among them, so one plan (and one workspace check) covers every layer of the call.
static Plan call_plan(const g4_model_desc* model, const g4_layer_desc* layers, int32_t n_layers, const g4_kv_entry* kv,
                      int64_t B, int64_t T, int32_t mode) {
  int64_t cap = 1;
  for (int32_t i = 0; i < n_layers; ++i) cap = std::max(cap, kv[layers[i].kv_src].cap);
  return plan(model, B, T, cap, mode);
}

static g4_status check_ws(const Plan& p, const void* ws, size_t ws_bytes) {
  G4_REQ(ws && ws_bytes >= p.total, G4_EINVAL, "workspace too small (%zu < %zu)", ws_bytes, p.total);
  G4_REQ(((uintptr_t)ws & 255) == 0, G4_EINVAL, "workspace is not 256-byte aligned");
  return G4_OK;
}

static g4_status layer_entry(const g4_model_desc* model, const g4_layer_desc* ld, int32_t layer, float* h,
                             const float* ple_in, const g4_kv_entry* kv, int32_t n_kv, const int32_t* pos, int64_t B,
                             int64_t T, int32_t mode, void* ws, const Plan& p, void* stream, bool xn_ready,
                             const void* next_norm) {
  LayerCtx c{model, ld, layer, h, ple_in, kv, n_kv, pos, B, T, mode, (char*)ws, &p, (hipStream_t)stream, xn_ready,
             next_norm};
  return layer_impl(c);
}

static g4_status check_call(const g4_model_desc* model, const float* h, const float* ple_in, const int32_t* pos,
                            int64_t B, int64_t T, int32_t mode) {
  g4_status st = check_model(model);
  if (st != G4_OK) return st;
  G4_REQ(mode == G4_PREFILL || mode == G4_DECODE || mode == G4_ENCODE, G4_EINVAL, "mode %d", mode);
  G4_REQ(h && ple_in && pos, G4_EINVAL, "h, ple_in or pos is NULL");
  G4_REQ(B >= 0 && T >= 0, G4_EINVAL, "B, T");
  return G4_OK;
}

g4_status g4_layer_forward(const g4_model_desc* model, const g4_layer_desc* ld, int32_t layer, float* h,
                           const float* ple_in, const g4_kv_entry* kv, int32_t n_kv, const int32_t* pos, int64_t B,
                           int64_t T, int32_t mode, void* ws, size_t ws_bytes, void* stream) {
  g4_status st = check_call(model, h, ple_in, pos, B, T, mode);
  if (st != G4_OK) return st;
  if ((st = check_layer(model, ld, layer, kv, n_kv, T, mode)) != G4_OK) return st;
  const Plan p = call_plan(model, ld, 1, kv, B, T, mode);
  if ((st = check_ws(p, ws, ws_bytes)) != G4_OK) return st;
  return layer_entry(model, ld, layer, h, ple_in, kv, n_kv, pos, B, T, mode, ws, p, stream, false, nullptr);
}

// Every check of a stack call (model, each layer, workspace) happens before the first launch.
static g4_status stack_run(const g4_model_desc* model, const g4_layer_desc* layers, float* h, const float* ple_in,
                           const g4_kv_entry* kv, int32_t n_kv, const int32_t* pos, int64_t B, int64_t T, int32_t mode,
                           void* ws, const Plan& p, void* stream) {
  for (int32_t l = 0; l < model->n_layers; ++l) {
    const void* nn = l + 1 < model->n_layers ? layers[l + 1].input_norm : nullptr;
    const g4_status st = layer_entry(model, &layers[l], l, h, ple_in, kv, n_kv, pos, B, T, mode, ws, p, stream, l > 0, nn);
    if (st != G4_OK) return st;
  }
  return G4_OK;
}

static g4_status check_stack(const g4_model_desc* model, const g4_layer_desc* layers, const float* h,
                             const float* ple_in, const g4_kv_entry* kv, int32_t n_kv, const int32_t* pos, int64_t B,
                             int64_t T, int32_t mode) {
  g4_status st = check_call(model, h, ple_in, pos, B, T, mode);
  if (st != G4_OK) return st;
  G4_REQ(layers, G4_EINVAL, "layers is NULL");
  for (int32_t l = 0; l < model->n_layers; ++l)
    if ((st = check_layer(model, &layers[l], l, kv, n_kv, T, mode)) != G4_OK) return st;
  return G4_OK;
}

// ---- the stack forward without a caller workspace --------------------------------------------------
// Scratch of g4_stack_forward_noalloc: one static array per GPU the library runs on, held until the
// process ends. Host code never passes `scratch` itself to a kernel (on the host that name is only a
// stand-in): its device address is resolved once per device with hipGetSymbolAddress, with that device
// current, and kept in g_scratch_dev.
static __device__ __align__(256) unsigned char scratch[G4_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_dev[kMaxDevices];

static g4_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(G4_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  G4_REQ(dev >= 0 && dev < kMaxDevices, G4_EUNSUP, "device ordinal %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(G4_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return G4_OK;
}

g4_status g4_stack_forward_noalloc(const g4_model_desc* model, const g4_layer_desc* layers, float* h,
                                   const float* ple_in, const g4_kv_entry* kv, int32_t n_kv, const int32_t* pos,
                                   int64_t B, int64_t T, int32_t mode, void* stream) {
  g4_status st = check_stack(model, layers, h, ple_in, kv, n_kv, pos, B, T, mode);
  if (st != G4_OK) return st;
  const Plan p = call_plan(model, layers, (int32_t)model->n_layers, kv, B, T, mode);
  G4_REQ(p.total <= G4_NOALLOC_SCRATCH_BYTES, G4_ERANGE,
         "this call needs %zu bytes of scratch; the static buffer holds %zu (use g4_stack_forward with a workspace)",
         p.total, (size_t)G4_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != G4_OK) return st;
  return stack_run(model, layers, h, ple_in, kv, n_kv, pos, B, T, mode, ws, p, stream);
}

g4_status g4_stack_forward(const g4_model_desc* model, const g4_layer_desc* layers, float* h, const float* ple_in,
                           const g4_kv_entry* kv, int32_t n_kv, const int32_t* pos, int64_t B, int64_t T, int32_t mode,
                           void* ws, size_t ws_bytes, void* stream) {
  g4_status st = check_stack(model, layers, h, ple_in, kv, n_kv, pos, B, T, mode);
  if (st != G4_OK) return st;
  const Plan p = call_plan(model, layers, (int32_t)model->n_layers, kv, B, T, mode);
  if ((st = check_ws(p, ws, ws_bytes)) != G4_OK) return st;
  return stack_run(model, layers, h, ple_in, kv, n_kv, pos, B, T, mode, ws, p, stream);
}

}  // extern "C"
