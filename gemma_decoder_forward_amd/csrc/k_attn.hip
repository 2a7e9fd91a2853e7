// Causal GQA attention over a layer's KV cache (cortiq-engine `attend_all_heads` with scale 1.0 and the
// sliding window; ferrox `causal_gqa_attention(_windowed)`; turbospark `encode_attention_any` over
// [kv_start, seq_len)). Query at absolute position i sees cache rows lo <= j <= i with lo = 0 on full
// layers and i - W + 1 on sliding layers. Head h reads kv head h / (nh / nkv). A prefill may instead
// take the encoder's mask (taconite-embeddinggemma2 `text_attention`): the call's own keys, within
// |i - j| <= W on sliding layers (key_span).
//
// This file holds the vector-ALU kernels:
//   * k_attn_rowwise: one wave per (query, head), online softmax; any head width <= 512, any dtype.
//   * k_attn_dec_part + k_attn_dec_merge: decode (one query per sequence), split over key chunks so
//     B * nkv * chunks blocks stream the cache; the G = nh/nkv heads of a group share every K/V read.
#include "g4_internal.h"

namespace g4 {

// [lo, hi]: the keys query position i sees (causal, or the encoder's mask; see key_span). Keys beyond
// a linear cache do not exist.
__device__ __forceinline__ void key_range(const AttnArgs& a, int64_t p0, int64_t i, int64_t& lo, int64_t& hi) {
  const KeySpan ks = key_span(a.bidir, a.sliding, a.window, a.cap, a.ring, p0, a.T);
  lo = i - ks.back;
  if (lo < ks.kmin) lo = ks.kmin;
  hi = i + ks.fwd;
  if (hi > ks.kmax) hi = ks.kmax;
}

// --------------------------------------------------------------------------------------------
template <typename T, int EPL>  // EPL: elements of the head per lane (hd <= 64 * EPL)
__global__ __launch_bounds__(256) void k_attn_rowwise(AttnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  const int64_t h = blockIdx.y, b = blockIdx.z;
  if (t >= a.T) return;
  const int64_t grp = a.nh / a.nkv, g = h / grp;
  const int hd = (int)a.hd;
  const int64_t p0 = a.pos0[b], i = p0 + t;
  int64_t lo, hi;
  key_range(a, p0, i, lo, hi);
  const T* qr = (const T*)a.q + (b * a.T + t) * a.q_ld + h * hd;
  const T* Kb = (const T*)a.k + (b * a.nkv + g) * a.cap * hd;
  const T* Vb = (const T*)a.v + (b * a.nkv + g) * a.cap * hd;
  float q[EPL], acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int d = lane + 64 * e;
    q[e] = d < hd ? ldf(qr + d) * a.scale : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int64_t j = lo; j <= hi; ++j) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int d = lane + 64 * e;
      if (d < hd) s += q[e] * ldf(Kb + kv_row(j, a.cap, a.ring) * hd + d);
    }
    s = wave_sum(s);
    const float mn = fmaxf(m, s);
    const float c = __expf(m - mn), p = __expf(s - mn);
    l = l * c + p;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int d = lane + 64 * e;
      acc[e] = acc[e] * c + (d < hd ? p * ldf(Vb + kv_row(j, a.cap, a.ring) * hd + d) : 0.f);
    }
    m = mn;
  }
  T* orow = (T*)a.out + (b * a.T + t) * a.out_ld + h * hd;
  const float il = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int d = lane + 64 * e;
    if (d < hd) stf(orow + d, acc[e] * il);
  }
}

g4_status attn_rowwise(const AttnArgs& a, int32_t dtype, hipStream_t s) {
  dim3 g((unsigned)((a.T + 3) / 4), (unsigned)a.nh, (unsigned)a.B);
  const int epl = (int)((a.hd + 63) / 64);
#define G4_AR(TT, E) hipLaunchKernelGGL((k_attn_rowwise<TT, E>), g, dim3(256), 0, s, a)
  if (dtype == G4_BF16) {
    if (epl <= 1) G4_AR(bf16, 1); else if (epl <= 2) G4_AR(bf16, 2); else if (epl <= 4) G4_AR(bf16, 4); else G4_AR(bf16, 8);
  } else {
    if (epl <= 1) G4_AR(float, 1); else if (epl <= 2) G4_AR(float, 2); else if (epl <= 4) G4_AR(float, 4); else G4_AR(float, 8);
  }
#undef G4_AR
  return check_launch("attn_rowwise");
}

// --------------------------------------------------------------------------------------------
// Decode. Partial pass: block (chunk c, kv head g, sequence b) scores the chunk's keys for all G
// heads of the group, then accumulates the unnormalised P V. Partials go to the workspace as
// [B, nh, nchunk, hd + 2] floats: (acc[hd], m, l).
// --------------------------------------------------------------------------------------------
constexpr int DEC_GMAX = 8;
constexpr int DEC_CHMAX = 256;

template <typename T, int EPL>
__global__ __launch_bounds__(256) void k_attn_dec_part(AttnArgs a, int chunk, int nchunk, float* __restrict__ ws) {
  __shared__ float qs[DEC_GMAX * 512];
  __shared__ float sc[DEC_GMAX * DEC_CHMAX];
  __shared__ float red[4 * 512];
  __shared__ float ml[DEC_GMAX * 2];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x;
  const int64_t g = blockIdx.y, b = blockIdx.z;
  const int G = (int)(a.nh / a.nkv);
  const int hd = (int)a.hd;
  const int64_t i = a.pos0[b];
  int64_t lo, hi;
  key_range(a, i, i, lo, hi);  // decode is always causal
  const int64_t k0 = lo + (int64_t)c * chunk;
  int64_t k1 = k0 + chunk - 1;
  if (k1 > hi) k1 = hi;
  const int nk = k1 >= k0 ? (int)(k1 - k0 + 1) : 0;
  // q of the group's heads, pre-scaled
  for (int x = threadIdx.x; x < G * hd; x += 256) {
    const int hh = x / hd, d = x % hd;
    qs[x] = ldf((const T*)a.q + b * a.q_ld + (g * G + hh) * hd + d) * a.scale;
  }
  __syncthreads();
  const T* Kb = (const T*)a.k + (b * a.nkv + g) * a.cap * hd;
  const T* Vb = (const T*)a.v + (b * a.nkv + g) * a.cap * hd;
  // scores: wave per key, lane per EPL elements
  for (int kk = wave; kk < nk; kk += 4) {
    float kv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int d = lane * EPL + e;
      kv[e] = d < hd ? ldf(Kb + kv_row(k0 + kk, a.cap, a.ring) * hd + d) : 0.f;
    }
    for (int hh = 0; hh < G; ++hh) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int d = lane * EPL + e;
        if (d < hd) s += kv[e] * qs[hh * hd + d];
      }
      s = wave_sum(s);
      if (lane == 0) sc[hh * DEC_CHMAX + kk] = s;
    }
  }
  __syncthreads();
  // per-head chunk max and sum of exponentials (wave hh handles heads hh, hh+4)
  for (int hh = wave; hh < G; hh += 4) {
    float mx = -INFINITY;
    for (int kk = lane; kk < nk; kk += 64) mx = fmaxf(mx, sc[hh * DEC_CHMAX + kk]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int kk = lane; kk < nk; kk += 64) {
      const float p = __expf(sc[hh * DEC_CHMAX + kk] - mx);
      sc[hh * DEC_CHMAX + kk] = p;
      sum += p;
    }
    sum = wave_sum(sum);
    if (lane == 0) { ml[hh * 2] = mx; ml[hh * 2 + 1] = sum; }
  }
  __syncthreads();
  // P V: waves split the keys, lanes the head elements
  for (int hh = 0; hh < G; ++hh) {
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    for (int kk = wave; kk < nk; kk += 4) {
      const float p = sc[hh * DEC_CHMAX + kk];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int d = lane * EPL + e;
        if (d < hd) acc[e] += p * ldf(Vb + kv_row(k0 + kk, a.cap, a.ring) * hd + d);
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int d = lane * EPL + e;
      if (d < hd) red[wave * 512 + d] = acc[e];
    }
    __syncthreads();
    float* dst = ws + (((b * a.nh + g * G + hh) * nchunk) + c) * (int64_t)(hd + 2);
    for (int d = threadIdx.x; d < hd; d += 256)
      dst[d] = red[d] + red[512 + d] + red[1024 + d] + red[1536 + d];
    if (threadIdx.x == 0) {
      dst[hd] = nk > 0 ? ml[hh * 2] : -INFINITY;
      dst[hd + 1] = nk > 0 ? ml[hh * 2 + 1] : 0.f;
    }
    __syncthreads();
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_attn_dec_merge(AttnArgs a, int nchunk, const float* __restrict__ ws) {
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / a.nh, h = bh % a.nh;
  const int hd = (int)a.hd;
  const float* src = ws + bh * nchunk * (int64_t)(hd + 2);
  float M = -INFINITY;
  for (int c = 0; c < nchunk; ++c) M = fmaxf(M, src[c * (hd + 2) + hd]);
  float L = 0.f;
  for (int c = 0; c < nchunk; ++c) {
    const float mc = src[c * (hd + 2) + hd];
    if (mc > -INFINITY) L += src[c * (hd + 2) + hd + 1] * __expf(mc - M);
  }
  const float il = L > 0.f ? 1.f / L : 0.f;
  for (int d = threadIdx.x; d < hd; d += 256) {
    float o = 0.f;
    for (int c = 0; c < nchunk; ++c) {
      const float mc = src[c * (hd + 2) + hd];
      if (mc > -INFINITY) o += src[c * (hd + 2) + d] * __expf(mc - M);
    }
    stf((T*)a.out + b * a.out_ld + h * hd + d, o * il);
  }
}

static void dec_plan(int64_t B, int64_t nkv, int64_t max_keys, int& chunk, int& nchunk) {
  chunk = DEC_CHMAX;
  // smaller chunks until there are enough blocks to cover the chip
  while (chunk > 64 && B * nkv * ((max_keys + chunk - 1) / chunk) < 1024) chunk >>= 1;
  nchunk = (int)((max_keys + chunk - 1) / chunk);
  if (nchunk < 1) nchunk = 1;
}

size_t attn_decode_ws(int64_t B, int64_t nh, int64_t hd, int64_t cap) {
  int chunk, nchunk;
  dec_plan(B, 1, cap, chunk, nchunk);  // nkv = 1 gives the largest chunk count
  const size_t a = (size_t)B * nh * nchunk * (hd + 2) * sizeof(float);
  const size_t b = attn_decode_mfma_ws(B, nh, hd, cap);
  return a > b ? a : b;
}

g4_status attn_decode(const AttnArgs& a, void* ws, size_t ws_bytes, int32_t dtype, hipStream_t s) {
  if (a.B == 0) return G4_OK;
  g4_status mst = G4_OK;
  if (dtype == G4_BF16 && attn_decode_mfma(a, ws, ws_bytes, s, &mst)) return mst;
  const int64_t G = a.nh / a.nkv;
  if (G > DEC_GMAX) return fail(G4_EUNSUP, "attn_decode: %lld query heads per kv head (max %d)", (long long)G, DEC_GMAX);
  if (a.hd > 512) return fail(G4_ERANGE, "attn_decode: head_dim %lld > 512", (long long)a.hd);
  const int64_t max_keys = a.sliding ? (a.window < a.cap ? a.window : a.cap) : a.cap;
  int chunk, nchunk;
  dec_plan(a.B, a.nkv, max_keys, chunk, nchunk);
  const size_t need = (size_t)a.B * a.nh * nchunk * (a.hd + 2) * sizeof(float);
  if (ws_bytes < need) return fail(G4_EINVAL, "attn_decode: workspace %zu < %zu bytes", ws_bytes, need);
  dim3 g((unsigned)nchunk, (unsigned)a.nkv, (unsigned)a.B);
  const int epl = (int)((a.hd + 63) / 64);
#define G4_AD(TT, E) hipLaunchKernelGGL((k_attn_dec_part<TT, E>), g, dim3(256), 0, s, a, chunk, nchunk, (float*)ws)
  if (dtype == G4_BF16) {
    if (epl <= 1) G4_AD(bf16, 1); else if (epl <= 2) G4_AD(bf16, 2); else if (epl <= 4) G4_AD(bf16, 4); else G4_AD(bf16, 8);
  } else {
    if (epl <= 1) G4_AD(float, 1); else if (epl <= 2) G4_AD(float, 2); else if (epl <= 4) G4_AD(float, 4); else G4_AD(float, 8);
  }
#undef G4_AD
  g4_status st = check_launch("attn_decode_part");
  if (st != G4_OK) return st;
  dim3 gm((unsigned)(a.B * a.nh));
  if (dtype == G4_BF16) hipLaunchKernelGGL(k_attn_dec_merge<bf16>, gm, dim3(256), 0, s, a, nchunk, (const float*)ws);
  else hipLaunchKernelGGL(k_attn_dec_merge<float>, gm, dim3(256), 0, s, a, nchunk, (const float*)ws);
  return check_launch("attn_decode_merge");
}

}  // namespace g4
