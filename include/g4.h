/*
 * g4 -- Gemma-4 E-series decoder-layer forward on AMD MI355X (gfx950), C ABI.
 *
 * Conventions shared by every entry point:
 *  - Tensor arguments are DEVICE pointers to row-major arrays owned by the caller; the library
 *    allocates no device memory. Scratch space comes from a caller workspace (`ws`, `ws_bytes`).
 *  - `dtype` selects the element type of weights and activations: G4_F32 or G4_BF16. The residual
 *    stream `h` and per-layer inputs are always float32. Accumulation is always float32.
 *  - Weight matrices use the [out, in] layout: y = x W^T, rows of W are contiguous in `in`.
 *  - Token-major activations: row m = b*T + t holds token t of sequence b.
 *  - KV caches are [B, nkv, cap, head_dim], nkv the kv head count of the owning layer's type; token t of
 *    sequence b sits at row pos[b] + t.
 *  - `pos` is a DEVICE int32 array [B] with the position of each sequence's first token in the call.
 *    Positions are not visible to the host: kernels skip cache writes and clip key ranges that fall
 *    outside [0, cap), so a bad position yields wrong values but never an out-of-bounds access.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is queued asynchronously.
 *  - Every argument is validated on the host before anything is launched. On failure nothing is
 *    launched and the status says why; g4_last_error() gives a message (per thread).
 *
 * The operations follow five public source pages: cortiq-engine `g4e.rs` (the E-series stack),
 * ferrox-models `gemma4_engine.rs`, memra-engine `forward.rs`, taconite-embeddinggemma2 `model.rs` and
 * turbospark-runtime `gemma4/attn.rs`. Each declaration below names the passage it implements.
 */
#ifndef G4_H
#define G4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum g4_status {
  G4_OK = 0,
  G4_EINVAL = 1, /* null pointer, non-positive size, unknown dtype/mode, workspace too small */
  G4_EGEOM = 2,  /* inconsistent geometry: kv_src routing, head-dim or attention-type mismatch */
  G4_ERANGE = 3, /* a size beyond a capacity: T > cap, window < 1, dims beyond kernel limits */
  G4_EHIP = 4,   /* a HIP runtime call or kernel launch failed (see g4_last_error) */
  G4_EUNSUP = 5  /* a combination the library does not implement */
} g4_status;

typedef enum g4_dtype { G4_F32 = 0, G4_BF16 = 1 } g4_dtype;

/* G4_ENCODE: a prefill whose attention is the encoder's non-causal mask (taconite-embeddinggemma2
 * model.rs, `text_attention`); see g4_attn_encode. */
typedef enum g4_mode { G4_PREFILL = 0, G4_DECODE = 1, G4_ENCODE = 2 } g4_mode;

/* Model hyper-parameters (cortiq-engine `G4eGlobals`; ferrox-models `Gemma4Hparams`). */
typedef struct g4_model_desc {
  int64_t hidden;        /* H */
  int64_t n_heads;       /* query heads nh */
  int64_t n_kv_heads;    /* kv heads nkv of sliding layers (and of full layers when n_kv_heads_full == 0);
                            nh % nkv == 0, head h reads kv head h / (nh/nkv) */
  int64_t head_dim_swa;  /* head width of sliding layers */
  int64_t head_dim_full; /* head width of full layers (global_head_dim) */
  int64_t ffn;           /* gated FFN width F of every layer whose descriptor gives none; the workspace is
                            sized for it, so it must be the largest width of the model */
  int64_t ple_dim;       /* per-layer input width d */
  int64_t n_layers;      /* L */
  int64_t window;        /* sliding window W: a query at i sees keys i-W < j <= i */
  int64_t vocab;         /* rows of the embedding table */
  int64_t ple_vocab;     /* rows of the per-layer embedding table */
  float eps;             /* RMSNorm epsilon (inside the mean) */
  float theta_swa;       /* RoPE base of sliding layers */
  float theta_full;      /* RoPE base of full layers */
  float partial_rotary;  /* full layers rotate floor(head_dim_full * partial_rotary / 2) pairs */
  int32_t dtype;         /* g4_dtype of weights and activations */
  int32_t k_eq_v;        /* 1: full layers have no V projection; V is the K projection's output, normed
                            without scale and not rotated (turbospark-runtime families/gemma4/attn.rs,
                            forward_layer, `attention_k_eq_v`); 0: every layer projects V with wv */
  int64_t n_kv_heads_full; /* kv heads of full layers (turbospark-runtime forward_layer, `num_full_kv_heads`);
                              0: the same as n_kv_heads */
} g4_model_desc;

/* One layer's weights (cortiq-engine `G4eLayer`). Norm weights are [H] or [head_dim]; all in dtype. */
typedef struct g4_layer_desc {
  int32_t sliding;       /* 1: sliding-window layer (head_dim_swa, theta_swa); 0: full layer */
  int32_t kv_src;        /* layer whose cache this layer attends over; == its own index if it owns one */
  float layer_scalar;    /* h *= layer_scalar after the block (1.0 when the model has none) */
  int32_t ffn;           /* this layer's FFN width, 1 .. model ffn (ferrox-models gemma4_engine.rs,
                            Gemma4Hparams::ffn_dim); 0: the model's ffn */
  const void* input_norm;     /* [H] */
  const void* wq;             /* [nh*hd, H] */
  const void* wk;             /* [nkv*hd, H]; read only when the layer owns its cache */
  const void* wv;             /* [nkv*hd, H]; idem; not read (may be NULL) on a full layer of a k_eq_v model */
  const void* wo;             /* [H, nh*hd] */
  const void* q_norm;         /* [hd] */
  const void* k_norm;         /* [hd]; idem */
  const void* post_attn_norm; /* [H] */
  const void* pre_ffn_norm;   /* [H] */
  const void* w_gate;         /* [F, H], F the layer's FFN width */
  const void* w_up;           /* [F, H] */
  const void* w_down;         /* [H, F] */
  const void* post_ffn_norm;  /* [H] */
  const void* ple_gate;       /* [d, H] */
  const void* ple_proj;       /* [H, d] */
  const void* post_ple_norm;  /* [H] */
} g4_layer_desc;

/* One entry of the per-layer KV table (ferrox-models `Gemma4DecodeState`: one cache per owning layer,
 * holes for shared layers). A hole has k == v == NULL. */
typedef struct g4_kv_entry {
  void* k;         /* [B, nkv, cap, hd] in dtype */
  void* v;         /* [B, nkv, cap, hd] in dtype */
  int64_t cap;     /* rows per (sequence, kv head) */
  int64_t hd;      /* head width of the rows */
  int32_t sliding; /* attention type of the layer that owns the cache */
  int32_t ring;    /* 0: position p lives in row p (p < cap). 1 (sliding layers only): a ring of cap >= window
                      rows, position p lives in row p mod cap (the ring capacity of a sliding layer's cache in turbospark-runtime,
                      families/gemma4/attn.rs, encode_gemma4_layer_attn_and_router); a call of T tokens
                      per sequence then needs T <= cap - window + 1, so that no key a query of the call can
                      see is overwritten by the call's own writes (longer prompts are prefilled in chunks) */
} g4_kv_entry;

/* ---- helpers ---------------------------------------------------------------------------------- */
const char* g4_status_str(int status);
/* Message of the last failure on the calling thread ("" if none). */
const char* g4_last_error(void);
/* Library version, major*10000 + minor*100 + patch. */
int g4_version(void);

/* Shared-KV routing (cortiq-engine module doc: the last n_shared layers carry no K/V projections and
 * attend over the cache of the last non-shared layer of the same attention type; ferrox
 * `n_layer_kv_from_start`). Host arrays: sliding[l] is 1 for sliding layers; kv_src[l] receives the
 * layer whose cache layer l reads (l itself for the first n_layers - n_shared layers). A shared layer
 * with no earlier owner of its type keeps its own cache (kv_src[l] == l). Runs on the host only. */
g4_status g4_kv_sources(const int32_t* sliding, int32_t n_layers, int32_t n_shared, int32_t* kv_src);

/* ---- row operations --------------------------------------------------------------------------- */

/* Plain RMSNorm with fused residual tail (cortiq-engine `rms` and `rms_plain`; the sandwich
 * residuals of `g4e_forward`; taconite `add_normed`):
 *   s      = sum over p < x_parts of x[p]            x: x_parts slices [rows, dim] in x_dtype
 *   n      = s * (mean(s^2) + eps)^-1/2 * w          w: [dim] in dtype, or NULL for no weight
 *   y      = n                                        if y != NULL        ([rows, dim] in dtype)
 *   res    = (res + n) * res_scale                    if res != NULL      (float32 [rows, dim])
 *   y_next = rms(res) * w_next  (or res itself when w_next == NULL)   if y_next != NULL (dtype)
 * y_next requires res. x_dtype is G4_F32 or dtype. */
g4_status g4_rmsnorm(const void* x, int32_t x_dtype, int32_t x_parts, const void* w, void* y,
                     float* res, float res_scale, const void* w_next, void* y_next, int64_t rows,
                     int64_t dim, float eps, int32_t dtype, void* stream);

/* Per-head RMSNorm then NeoX RoPE of head vectors (cortiq-engine `g4e_forward` q/k/v head loops;
 * turbospark `encode_rms_norm_bf16w_perhead`, `encode_rms_norm_no_scale_perhead`,
 * `encode_rope_proportional_neox`; taconite `rope_half`).
 *   x: rows m = b*T + t, head h at x + m*x_ld + h*hd (elements, dtype).
 *   v = x_head * (mean(x_head^2) + eps)^-1/2 * w      (w NULL: no weight, the V norm)
 *   pairs j < rotated_pairs: (v_j, v_{j+hd/2}) rotated by (pos[b]+t) * theta^(-2j/hd); other pairs
 *   unchanged (rotated_pairs == 0: no RoPE).
 *   y_cap == 0: y row m head h at y + m*y_ld + h*hd (may alias x exactly).
 *   y_cap  > 0: y is a cache [B, heads, y_cap, hd]; the vector goes to row pos[b]+t (skipped if
 *               outside [0, y_cap)).
 * pos may be NULL only when rotated_pairs == 0 and y_cap == 0. */
g4_status g4_qk_norm_rope(const void* x, int64_t x_ld, const void* w, void* y, int64_t y_ld,
                          int64_t y_cap, const int32_t* pos, int64_t B, int64_t T, int64_t heads,
                          int64_t hd, float theta, int64_t rotated_pairs, float eps, int32_t dtype,
                          void* stream);

/* ---- attention -------------------------------------------------------------------------------- */

/* Causal GQA attention of a prefill chunk over a layer's cache (cortiq-engine `attend_all_heads`
 * called with scale 1.0 and the window; ferrox `causal_gqa_attention(_windowed)`; taconite
 * `text_attention` head map kh = hh / group).
 *   q: [B*T, nh*hd] rows with leading dimension q_ld; query t of sequence b is at position pos0[b]+t.
 *   Keys/values come from kv[kv_src] (no copy): query i sees cache rows j with lo <= j <= i,
 *   lo = 0 (sliding == 0) or i - window + 1 (sliding == 1). Those rows must already hold this call's
 *   K/V (written by g4_qk_norm_rope) and earlier tokens.
 *   out[b*T+t, h*hd:(h+1)*hd] = softmax_j(scale * q.k_j) v_j, leading dimension out_ld.
 *   ws, ws_bytes: optional scratch (16-byte aligned) for the key split of a short prefill, whose few query
 *   blocks would leave most compute units idle: the blocks then split their key ranges and a merge pass
 *   combines the partial softmax sums. ws == NULL: no split (same result, fewer blocks in flight);
 *   otherwise ws_bytes >= g4_attn_prefill_ws(B, T, nh, nkv, hd), else G4_EINVAL.
 * Validation: kv_src <= layer, kv[kv_src] present with hd and attention type equal to this call's. */
size_t g4_attn_prefill_ws(int64_t B, int64_t T, int64_t nh, int64_t nkv, int64_t hd);
g4_status g4_attn_prefill(const void* q, int64_t q_ld, const g4_kv_entry* kv, int32_t n_kv,
                          int32_t layer, int32_t kv_src, int32_t sliding, int64_t window,
                          const int32_t* pos0, int64_t B, int64_t T, int64_t nh, int64_t nkv,
                          int64_t hd, float scale, void* out, int64_t out_ld, void* ws,
                          size_t ws_bytes, int32_t dtype, void* stream);

/* The encoder's non-causal attention (taconite-embeddinggemma2 model.rs, `text_attention`: every key
 * of the sequence, a sliding layer's keys within |i - j| <= window). Arguments as g4_attn_prefill; the
 * sequence is this call: query i = pos0[b]+t sees the cache rows j of the call's own tokens,
 * pos0[b] <= j <= pos0[b]+T-1, all of them (sliding == 0) or those with |i - j| <= window
 * (sliding == 1), so rows before pos0[b] are never read. The call's K/V rows must already be in the
 * cache. The cache must be linear (ring == 0), else G4_EINVAL. The workspace is g4_attn_prefill's
 * (same size query, NULL allowed). */
g4_status g4_attn_encode(const void* q, int64_t q_ld, const g4_kv_entry* kv, int32_t n_kv,
                         int32_t layer, int32_t kv_src, int32_t sliding, int64_t window,
                         const int32_t* pos0, int64_t B, int64_t T, int64_t nh, int64_t nkv,
                         int64_t hd, float scale, void* out, int64_t out_ld, void* ws,
                         size_t ws_bytes, int32_t dtype, void* stream);

/* Decode attention: one query per sequence at position pos[b] (turbospark `encode_attention_any`
 * over [kv_start, seq_len)). Same semantics as g4_attn_prefill with T = 1. Split over key chunks;
 * the workspace holds per-chunk partial results (size from g4_attn_decode_ws). */
g4_status g4_attn_decode(const void* q, int64_t q_ld, const g4_kv_entry* kv, int32_t n_kv,
                         int32_t layer, int32_t kv_src, int32_t sliding, int64_t window,
                         const int32_t* pos, int64_t B, int64_t nh, int64_t nkv, int64_t hd,
                         float scale, void* out, int64_t out_ld, void* ws, size_t ws_bytes,
                         int32_t dtype, void* stream);
size_t g4_attn_decode_ws(int64_t B, int64_t nh, int64_t hd, int64_t cap);

/* ---- projections ------------------------------------------------------------------------------ */

/* C = A W^T (memra `e.matmul` with m = T token rows). A [M, K], W [N, K] in dtype; C [M, N] in
 * c_dtype (G4_F32 or dtype). Float32 accumulation. */
g4_status g4_linear(const void* A, const void* W, void* C, int64_t M, int64_t N, int64_t K,
                    int32_t c_dtype, int32_t dtype, void* ws, size_t ws_bytes, void* stream);

/* Gelu-tanh gated FFN branch (cortiq-engine `gelu_tanh` and the FFN block of `g4e_forward`; taconite
 * `mlp`): out = (gelu_tanh(x W_gate^T) * (x W_up^T)) W_down^T.
 *   x [M, H] dtype; w_gate, w_up [F, H]; w_down [H, F]; out float32 [M, H]. */
size_t g4_ffn_geglu_ws(int64_t M, int64_t H, int64_t F, int32_t dtype);
g4_status g4_ffn_geglu(const void* x, const void* w_gate, const void* w_up, const void* w_down,
                       float* out, int64_t M, int64_t H, int64_t F, void* ws, size_t ws_bytes,
                       int32_t dtype, void* stream);

/* Per-layer-input injection (cortiq-engine PLE block of `g4e_forward`; ferrox `per_layer_inp_gate`):
 *   h = (h + rms(W_proj (gelu_tanh(W_gate h) * ple)) * w_post) * layer_scalar
 *   h float32 [M, H] in place; the gate reads the raw residual h. ple float32 rows [M, d] with
 *   leading dimension ple_ld. w_gate [d, H], w_proj [H, d], w_post [H] in dtype. */
size_t g4_ple_inject_ws(int64_t M, int64_t H, int64_t d, int32_t dtype);
g4_status g4_ple_inject(float* h, const void* w_gate, const float* ple, int64_t ple_ld,
                        const void* w_proj, const void* w_post, float layer_scalar, int64_t M,
                        int64_t H, int64_t d, float eps, void* ws, size_t ws_bytes, int32_t dtype,
                        void* stream);

/* Output head after the stack (ferrox-models `forward_token_on_worker` tail; cortiq-engine module doc:
 * final norm + lm_head + final-logit softcap):
 *   logits[m, :] = cap * tanh((W_out * (rms(h[m]) * out_norm)) / cap)      (no tanh when softcap == 0)
 * h float32 [M, H] (contiguous rows: pass the rows whose logits are wanted, e.g. each sequence's last
 * token); out_norm [H] and W_out [vocab, H] in dtype (W_out may be the token embedding table);
 * logits float32 [M, vocab]. Workspace: g4_logits_ws bytes. softcap < 0 is G4_EINVAL. */
size_t g4_logits_ws(int64_t M, int64_t H, int64_t vocab, int32_t dtype);
g4_status g4_logits(const float* h, int64_t M, int64_t H, const void* out_norm, const void* w_out, int64_t vocab,
                    float eps, float softcap, float* logits, void* ws, size_t ws_bytes, int32_t dtype,
                    void* stream);

/* Token embedding and per-layer inputs (cortiq-engine `extend_embedding`; ferrox
 * `project_per_layer_inputs` and the embedding scale of `forward_token_on_worker`):
 *   h_out[m]        = E[id] * sqrt(H)                              (zero row if id outside [0,vocab))
 *   ple_out[m, l, :] = (rms(P_l * H^-1/2) * ple_norm + sqrt(d) * Tab[id, l*d:(l+1)*d]) / sqrt(2)
 *   with P = W_pm h_out[m]; the table term is zero if id outside [0, ple_vocab).
 * ids int32 [M]; E [vocab, H]; Tab [ple_vocab, L*d]; W_pm [L*d, H]; ple_norm [d] (dtype).
 * h_out float32 [M, H]; ple_out float32 [M, L*d]. */
g4_status g4_embed_ple(const int32_t* ids, int64_t M, const void* E, const void* Tab,
                       const void* W_pm, const void* ple_norm, const g4_model_desc* model,
                       float* h_out, float* ple_out, void* ws, size_t ws_bytes, void* stream);

/* ---- layer and stack -------------------------------------------------------------------------- */

/* One decoder layer over M = B*T token rows (cortiq-engine `g4e_forward` layer body):
 *   h float32 [M, H] residual, updated in place; ple_in float32 [M, L*d] (this layer reads its
 *   d-wide slice); kv the per-layer cache table (n_kv == model->n_layers); pos int32 [B].
 *   mode G4_PREFILL: T tokens per sequence at pos[b] .. pos[b]+T-1.
 *   mode G4_DECODE:  T must be 1.
 *   mode G4_ENCODE:  as G4_PREFILL, with the encoder's attention (g4_attn_encode) over the call's
 *                    tokens; linear caches only.
 * A layer that owns its cache (kv_src == layer) writes its K/V rows before attending.
 * ws: 256-byte aligned device scratch of at least g4_workspace_size(model, B, T, cap, mode) bytes, cap the
 * capacity of the cache this layer reads. */
g4_status g4_layer_forward(const g4_model_desc* model, const g4_layer_desc* layer_desc,
                           int32_t layer, float* h, const float* ple_in, const g4_kv_entry* kv,
                           int32_t n_kv, const int32_t* pos, int64_t B, int64_t T, int32_t mode,
                           void* ws, size_t ws_bytes, void* stream);

/* All n_layers layers in order; layers is an array of n_layers descriptors. Returns the hidden state
 * before the final norm, in h. ws as for g4_layer_forward, with cap the largest capacity among the caches
 * the layers read. Every layer and the workspace are validated before the first launch, so a failing
 * call leaves h and the caches untouched. */
g4_status g4_stack_forward(const g4_model_desc* model, const g4_layer_desc* layers, float* h,
                           const float* ple_in, const g4_kv_entry* kv, int32_t n_kv,
                           const int32_t* pos, int64_t B, int64_t T, int32_t mode, void* ws,
                           size_t ws_bytes, void* stream);

/* g4_stack_forward for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. Same arguments and results as g4_stack_forward, without
 * the workspace: scratch is a static device array of G4_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends. No call allocates or frees device memory; the first call
 * on a device resolves the array's address there (hipGetSymbolAddress, with the stream's device current).
 * A call needing more scratch than that (g4_workspace_size with cap the largest cache capacity the layers
 * read: e.g. decode of up to 64 sequences over caches of 8192 rows fits, a prefill of 2048 tokens does
 * not) returns G4_ERANGE with nothing launched. Every call on one GPU shares that GPU's array, which keeps
 * the last call's contents (no kernel reads scratch it has not written in the same call); calls that
 * overlap on one GPU, on different streams or threads, race on it and must be serialized by the caller. */
#define G4_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
g4_status g4_stack_forward_noalloc(const g4_model_desc* model, const g4_layer_desc* layers, float* h,
                                   const float* ple_in, const g4_kv_entry* kv, int32_t n_kv,
                                   const int32_t* pos, int64_t B, int64_t T, int32_t mode, void* stream);

/* ---- timing instrumentation ------------------------------------------------------------------ */

/* Kernel classes of the layer forward, for g4_timer_enable. */
typedef enum g4_kernel_class {
  G4_KC_QKV_GEMM = 1,   /* q/k/v projections */
  G4_KC_QK_NORM_ROPE = 2,
  G4_KC_ATTENTION = 3,
  G4_KC_O_GEMM = 4,
  G4_KC_GATE_UP_GEMM = 5, /* gate/up projection with the gelu-tanh product epilogue */
  G4_KC_DOWN_GEMM = 6,
  G4_KC_PLE_GEMM = 7,
  G4_KC_ROW_TAIL = 8    /* fused RMSNorm residual tails */
} g4_kernel_class;

/* While enabled, every launch of kernel class `cls` made by g4_layer_forward / g4_stack_forward is
 * bracketed by two HIP events recorded on the caller's stream (at most max_launches launches; later
 * ones are not timed). Enabling creates the events (no device memory). Not thread-safe: one timer
 * per process. */
g4_status g4_timer_enable(int32_t cls, int32_t max_launches);
/* Stops recording and returns the summed device time (ms) and the number of timed launches; waits for
 * the recorded events to complete. */
g4_status g4_timer_read(double* total_ms, int32_t* launches);

/* Workspace bytes g4_layer_forward / g4_stack_forward / g4_embed_ple need for M = B*T rows over
 * caches of capacity `cap` (decode splits attention over key chunks of the cache). 0 if the model
 * descriptor is invalid. */
size_t g4_workspace_size(const g4_model_desc* model, int64_t B, int64_t T, int64_t cap, int32_t mode);

#ifdef __cplusplus
}
#endif
#endif /* G4_H */
