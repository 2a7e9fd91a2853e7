// Internal declarations of the g4 library: element types, wave/block reductions, launch helpers.
// Every kernel of the library is written for gfx950 (CDNA4): 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/g4.h"

namespace g4 {

// bf16 stored as raw bits; arithmetic is always float32.
typedef uint16_t bf16;

__device__ __forceinline__ float bf2f(bf16 v) { return __uint_as_float((uint32_t)v << 16); }

// Round to nearest even (NaN stays NaN): the hardware conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16 f2bf(float f) { return __builtin_bit_cast(bf16, (__bf16)f); }

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_hw;
// Four floats rounded to bf16 and packed for one 8-byte store.
__device__ __forceinline__ uint2 pack_bf16x4(const float* v) {
  bf16x2_hw lo, hi;
  lo[0] = (__bf16)v[0]; lo[1] = (__bf16)v[1];
  hi[0] = (__bf16)v[2]; hi[1] = (__bf16)v[3];
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

template <typename T> struct io;
template <> struct io<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <> struct io<bf16> {
  static __device__ __forceinline__ float ld(const bf16* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(bf16* p, float v) { *p = f2bf(v); }
};
template <typename T> __device__ __forceinline__ float ldf(const T* p) { return io<T>::ld(p); }
template <typename T> __device__ __forceinline__ void stf(T* p, float v) { io<T>::st(p, v); }

// Lane 0's value of a float, broadcast (the builtin is int -> int: pass the bits, not the value).
__device__ __forceinline__ float first_lane_f(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// Sum over the 64 lanes of a wave, the same value in every lane. Within each row of 16 lanes the partial
// sums move by DPP (swap neighbours, swap pairs, mirror each half row, mirror the row), so every lane
// of a row ends with the row's sum; the four row sums are then read out and added in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Sum over a block of NT threads (NT multiple of 64, <= 1024). `sh` holds >= 17 floats.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) sh[w] = v;
  __syncthreads();
  if (w == 0) {
    float t = (l < NT / 64) ? sh[l] : 0.f;
    t = wave_sum(t);
    if (l == 0) sh[16] = t;
  }
  __syncthreads();
  float r = sh[16];
  __syncthreads();
  return r;
}

// gelu, tanh form: 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3). Evaluated as the equal
// x / (1 + exp(-2u)), with exp(-2u) = 2^t, t = -2 log2(e) u, through the hardware base-2 exponential
// and reciprocal (about 1 ulp each): large |u| saturate to x or to 0 without overflow trouble.
__device__ __forceinline__ float gelu_tanh(float x) {
  const float t = x * (-2.302208198144325f - 0.1029432395800235f * x * x);
  return x * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(t));
}

inline size_t dsize(int32_t dt) { return dt == G4_BF16 ? 2 : 4; }

// ---- error state (g4_api.cpp) ------------------------------------------------------------------
g4_status fail(g4_status st, const char* fmt, ...);
g4_status check_launch(const char* what);

// ---- GEMM epilogues --------------------------------------------------------------------------
enum Epi : int {
  EPI_STORE = 0,     // C = acc (C in c_dtype)
  EPI_GEGLU = 1,     // dual B (gate, up): C = gelu_tanh(acc_gate) * acc_up, C in dtype
  EPI_GELU_MUL = 2,  // C = gelu_tanh(acc) * aux[m*aux_ld + n], aux float32, C in dtype
  EPI_SOFTCAP = 3,   // C = cap * tanh(acc / cap), C float32, no K split (64-row tiles only)
};

struct GemmArgs {
  const void* A; int64_t lda;
  const void* B; const void* B2; int64_t ldb;  // B2: the `up` matrix of EPI_GEGLU
  void* C; int64_t ldc; int32_t c_dtype;
  const float* aux; int64_t aux_ld;
  int64_t M, N, K;
  int32_t epi;
  int32_t splits;        // split-K slices (EPI_STORE with f32 C only): slice s at C + s*split_stride
  int64_t split_stride;  // elements between slices
  // EPI_STORE only: B rows (= C columns) are the concatenation of nseg (1..3) matrices segB[i] with
  // seg_rows[i] rows each (nseg == 0 means one matrix, B, of N rows)
  int32_t nseg;
  const void* segB[3];
  int64_t seg_rows[3];
  void* ws; size_t ws_bytes;  // scratch for the few-row kernel's partial sums (may be null)
  float cap;                  // EPI_SOFTCAP: the cap (> 0)
};

// Launchers (return G4_OK or a failure with the message set).
g4_status gemm(const GemmArgs& a, int32_t dtype, hipStream_t s);
// Smallest ws bytes gemm() might use for these sizes (0 today: no internal scratch).
size_t gemm_ws(int64_t M, int64_t N, int64_t K, int32_t dtype);

struct HeadSeg {
  const void* x; int64_t x_ld;
  const void* w;           // per-head norm weight or nullptr
  void* y; int64_t y_ld; int64_t y_cap;  // y_cap > 0: y is a cache [B, heads, y_cap, hd]
  int32_t heads; int32_t rope;
  int32_t ring;            // the cache is a ring: position p lives in row p mod y_cap
};
g4_status qk_norm_rope(const HeadSeg* segs, int nseg, const int32_t* pos, int64_t B, int64_t T,
                       int64_t hd, float theta, int64_t n_rot, float eps, int32_t dtype,
                       hipStream_t s);
// The same with every input segment read as the sum of `parts` float32 slices part_stride apart (the
// split-K partials of the projection); outputs in dtype.
g4_status qk_norm_rope_parts(const HeadSeg* segs, int nseg, int parts, int64_t part_stride, const int32_t* pos,
                             int64_t B, int64_t T, int64_t hd, float theta, int64_t n_rot, float eps, int32_t dtype,
                             hipStream_t s);

g4_status rownorm(const void* x, int32_t x_dtype, int32_t x_parts, int64_t part_stride,
                  const void* w, void* y, float* res, float res_scale, const void* w_next,
                  void* y_next, int64_t rows, int64_t dim, float eps, int32_t dtype,
                  hipStream_t s);

struct AttnArgs {
  const void* q; int64_t q_ld;
  const void* k; const void* v; int64_t cap;
  const int32_t* pos0;
  int64_t B, T, nh, nkv, hd;
  int32_t sliding; int64_t window;
  float scale;
  void* out; int64_t out_ld;
  int32_t ring;  // the cache is a ring of cap rows: key j lives in row j mod cap
  int32_t bidir; // prefill only: the encoder's non-causal mask over the call's own keys
  // Prefill only, optional: float32 scratch of attn_prefill_ws() bytes for key-split partial results
  // (used when a short prefill gives too few query blocks to fill the device); null = no key split.
  float* ws; size_t ws_bytes;
};

// Cache row of key position j, and the last key a query at position i can see in the cache.
__device__ __forceinline__ int64_t kv_row(int64_t j, int64_t cap, int32_t ring) {
  if (!ring) return j;
  // positions and capacities below 2^32 (every real cache) take the much shorter 32-bit remainder
  if (((uint64_t)j | (uint64_t)cap) >> 32) return (int64_t)((uint64_t)j % (uint64_t)cap);
  return (int64_t)((uint32_t)j % (uint32_t)cap);
}
__device__ __forceinline__ int64_t kv_last(int64_t i, int64_t cap, int32_t ring) {
  return ring || i < cap - 1 ? i : cap - 1;
}

// Keys a query at position i sees, as [max(i - back, kmin), min(i + fwd, kmax)].
//   causal (decoder): back = W - 1 on sliding layers (W keys, itself included), unbounded on full
//     layers; fwd = 0; kmin = 0; kmax = the last row of a linear cache.
//   bidir (encoder, taconite-embeddinggemma2 `text_attention`): the call's keys p0 .. p0 + T - 1 only,
//     with back = fwd = W on sliding layers (|i - j| <= W) and unbounded on full layers.
struct KeySpan {
  int64_t back, fwd, kmin, kmax;
};
__device__ __forceinline__ KeySpan key_span(int32_t bidir, int32_t sliding, int64_t window, int64_t cap,
                                            int32_t ring, int64_t p0, int64_t T) {
  const int64_t big = (int64_t)1 << 48;  // "unbounded": i +- big cannot overflow for any real position
  const int64_t w = window < big ? window : big;
  KeySpan s;
  if (bidir) {
    s.back = sliding ? w : big;
    s.fwd = s.back;
    s.kmin = p0 > 0 ? p0 : 0;  // rows below 0 do not exist, whatever pos0 holds
    s.kmax = p0 + T - 1 < cap - 1 ? p0 + T - 1 : cap - 1;
  } else {
    s.back = sliding ? w - 1 : big;
    s.fwd = 0;
    s.kmin = 0;
    s.kmax = ring ? big : cap - 1;
  }
  return s;
}
g4_status attn_prefill(const AttnArgs& a, int32_t dtype, hipStream_t s);
g4_status attn_decode(const AttnArgs& a, void* ws, size_t ws_bytes, int32_t dtype, hipStream_t s);
size_t attn_decode_ws(int64_t B, int64_t nh, int64_t hd, int64_t cap);
// Compute units of the current device (256 when no device is visible).
int device_cus();
// Scratch bytes the prefill attention may use to split key ranges (0 when it would not split).
size_t attn_prefill_ws(int64_t B, int64_t T, int64_t nh, int64_t nkv, int64_t hd);
bool attn_decode_mfma(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t s, g4_status* st);
size_t attn_decode_mfma_ws(int64_t B, int64_t nh, int64_t hd, int64_t cap);

// Rotation frequencies of a launch in revolutions per position, inv_j / (2 pi), from the host in f64;
// zero past the rotated pairs.
struct RopeTab { double rev[256]; };
void rope_table(RopeTab& t, float theta, int64_t hd, int64_t n_rot);

// Decode attention that forms its own inputs from the q/k/v projection's split-K partial sums: the
// per-head RMS norm and RoPE of qk_norm_rope_parts folded into the attention launch (one token per
// sequence). x holds `parts` float32 slices [B][x_ld], part_stride apart; the q heads start at element
// q_off of a row, the k and v heads of a layer that owns its cache at k_off and v_off (v: scale-less
// norm, no rotation). k_off < 0: the layer reads another layer's cache and writes no key.
struct DecFuse {
  const float* x; int64_t x_ld; int64_t part_stride; int32_t parts;
  int64_t q_off, k_off, v_off;
  const bf16* qw; const bf16* kw;
  int32_t n_rot; float eps;
  RopeTab tab;
};
// false (nothing launched) when the shape or alignment does not suit the fused kernel.
bool attn_decode_fused(const AttnArgs& a, const DecFuse& f, void* ws, size_t ws_bytes, hipStream_t s,
                       g4_status* st);

g4_status cast_rows(const float* x, void* y, int64_t n, int32_t dtype, hipStream_t s);
g4_status softcap_inplace(float* x, int64_t n, float cap, hipStream_t s);
g4_status gemm_simt(const GemmArgs& a, int32_t dtype, hipStream_t s);
bool gemm_mfma(const GemmArgs& a, hipStream_t s, g4_status* st);
bool gemm_mfma_tiles64(const GemmArgs& a, hipStream_t s, g4_status* st);
int gemm_rows64_cols(const GemmArgs& a);  // output columns per 64-row tile (M <= 64), 0 if none fits
// Split-K slices (1..max_splits) for a float32-output product whose consumer sums the slices: the
// count whose MFMA tiling (tile width and slices together) takes the fewest tile-passes.
int32_t gemm_pick_splits(int64_t M, int64_t N, int64_t K, int32_t max_splits);
bool gemm_skinny(const GemmArgs& a, const void* const* segs, const int64_t* seg_rows, int nseg, void* ws,
                 size_t ws_bytes, hipStream_t s, g4_status* st);
size_t gemm_skinny_ws(int64_t M, int64_t Nt, int64_t K);

// Few-row GEMM writing float32 split-K partials [splits][M][Nt] (Nt = sum of the segment rows), for a
// consumer that sums the slices itself. The A operand is bf16 rows, or is formed while it is staged from
// float32 partial slices of an earlier few-row GEMM:
enum SkAKind : int {
  SKA_BF16 = 0,      // A[m][k] = a[m*lda + k] (bf16)
  SKA_GEGLU = 1,     // A[m][k] = bf16(gelu_tanh(sum_p P[m*lda + k]) * sum_p P[m*lda + up_off + k])
  SKA_GELU_MUL = 2,  // A[m][k] = bf16(gelu_tanh(sum_p P[m*lda + k]) * aux[m*aux_ld + k])
};
struct SkA {
  const void* a; int64_t lda;
  int32_t kind; int32_t parts; int64_t part_stride;  // partial slices: `parts` slices part_stride floats apart
  int64_t up_off;
  const float* aux; int64_t aux_ld;
};
// True if the few-row kernel takes these shapes (M <= 64, K % 128 == 0, segments of 64-row multiples,
// 16-byte aligned rows).
bool skinny_ok(int64_t M, int64_t K, const void* const* segs, const int64_t* seg_rows, int nseg, int64_t ldb);
void skinny_plan(int64_t M, int64_t K, int64_t Nt, int* rows_per_block, int* kc, int* splits);
// C[M, F] (bf16, row stride ldc) = bf16(gelu_tanh(A w_gate^T) * (A w_up^T)) in one pass, for M <= 16.
bool skinny_gated_ok(int64_t M, int64_t K, int64_t F);
g4_status gemm_skinny_gated(const SkA& sa, int64_t M, int64_t K, const void* w_gate, const void* w_up, int64_t F,
                            int64_t ldb, void* C, int64_t ldc, hipStream_t s);
// Sums `splits` partial slices [splits][M][Nt] and applies a's epilogue into a.C (a.M, a.N, a.ldc, ...).
g4_status gemm_skinny_finish(const GemmArgs& a, const float* part, int splits, int64_t Nt, hipStream_t s);
g4_status gemm_skinny_part(const SkA& sa, int64_t M, int64_t K, const void* const* segs, const int64_t* seg_rows,
                           int nseg, int64_t ldb, float* part, size_t part_bytes, int* splits, hipStream_t s);
g4_status attn_rowwise(const AttnArgs& a, int32_t dtype, hipStream_t s);
bool attn_mfma(const AttnArgs& a, hipStream_t s, g4_status* st);
g4_status embed_rows(const int32_t* ids, int64_t M, const void* E, int64_t vocab, int64_t H,
                     float* h_out, void* e_cast, int32_t dtype, hipStream_t s);
g4_status ple_combine(const int32_t* ids, int64_t M, const float* P, const void* Tab,
                      int64_t ple_vocab, const void* ple_norm, int64_t H, int64_t L, int64_t d,
                      float eps, float* ple_out, int32_t dtype, hipStream_t s);

}  // namespace g4
