// Decode attention (one query per sequence) for bf16 caches: split over key chunks so that
// B x nkv x chunks blocks stream the cache, every K/V row read once per kv group (the G query heads of
// the group share it).
//
// Scores: v_mfma_f32_16x16x32_bf16 with the group's query heads as rows (padded to 16) and 16 keys as
// columns. Lane l supplies key (l % 16) and head elements 128c + 32t + 8*(l/16) .. +7 for MFMA t of
// 128-element chunk c, straight from memory: the four lanes of a key read 64 contiguous bytes per load.
// The queries sit in registers in the same element order. Lanes 0..15 then hold the scores of heads
// 0..3 for key (l % 16).
// P V: each lane owns HD/64 consecutive head elements for all heads of the group; V rows are read
// coalesced and each probability is broadcast from the lane that holds it (readlane), so the
// accumulation is plain FMAs. Online softmax in the exp2 domain.
// The 4 waves of a block split its chunk, combine through LDS, and write one partial (unnormalised o,
// m, l) per head; k_attn_dec_merge2 combines the chunks.
// Fused form (k_attn_dec_mfmaf): the block forms its inputs from the q/k/v projection's split-K
// partials instead of reading a finished q: waves 0 .. G-1 each form one query head (RMS norm with its
// weight, RoPE at the sequence's position, bf16) in LDS; in the block whose chunk holds the new key,
// wave 2 forms that key's k head and wave 3 its v head (scale-less norm), write them to the cache row
// for the steps that follow, and leave them in LDS, from where the wave that owns the key takes its
// K and V operands (its own load of that cache row races the write and is discarded).
#include "g4_internal.h"

namespace g4 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr int DM_G = 4;  // query heads per kv head handled (rows of the score MFMA in use)

// EP consecutive floats (EP = 1, 2 or 4; p aligned to EP floats), and EP bf16 values (aligned to EP).
template <int EP> __device__ __forceinline__ void dl_f32(const float* p, float* v) {
  if (EP == 4) { const float4 t = *(const float4*)p; v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w; }
  else if (EP == 2) { const float2 t = *(const float2*)p; v[0] = t.x; v[1] = t.y; }
  else v[0] = *p;
}
template <int EP> __device__ __forceinline__ void dl_bf16(const bf16* p, float* v) {
  if (EP == 4) {
    const uint2 u = *(const uint2*)p;
    v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
  } else if (EP == 2) {
    const uint32_t u = *(const uint32_t*)p;
    v[0] = __uint_as_float(u << 16); v[1] = __uint_as_float(u & 0xffff0000u);
  } else {
    v[0] = bf2f(*p);
  }
}
template <int EP> __device__ __forceinline__ void ds_bf16(bf16* p, const float* v) {
  if (EP == 4) *(uint2*)p = pack_bf16x4(v);
  else if (EP == 2) *(uint32_t*)p = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  else *p = f2bf(v[0]);
}

// One head of the token at position p from the split-K partials (slice 0 at xh, the others part_stride
// apart): RMS norm over the head (times w when given), RoPE on pairs j < n_rot (pair j: elements j and
// j + HD/2) when rope, rounded to bf16 into lds[HD] (and glob[HD] when given). One wave; lane l takes
// pairs EP l .. EP l + EP - 1. The arithmetic is that of the separate head-norm kernel.
template <int HD>
__device__ __forceinline__ void dec_form_head(const DecFuse& f, const float* xh, const bf16* w, bool rope, int64_t p,
                                              bf16* lds, bf16* glob) {
  constexpr int EP = HD / 128, half = HD / 2;
  const int lane = threadIdx.x & 63;
  const int j0 = EP * lane;
  float av[EP], cv[EP], wa[EP], wc[EP];
  dl_f32<EP>(xh + j0, av);
  dl_f32<EP>(xh + j0 + half, cv);
#pragma unroll
  for (int e = 0; e < EP; ++e) wa[e] = wc[e] = 1.f;
  if (w) {
    dl_bf16<EP>(w + j0, wa);
    dl_bf16<EP>(w + j0 + half, wc);
  }
  float co[EP], sn[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    double r = (double)p * f.tab.rev[j0 + e];
    r -= rint(r);
    co[e] = __builtin_amdgcn_cosf((float)r);
    sn[e] = __builtin_amdgcn_sinf((float)r);
  }
  for (int p0 = 1; p0 < f.parts; p0 += 4) {  // further slices, summed in order, four per round trip
    float ta[4][EP], tc[4][EP];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t off = (int64_t)min(p0 + q, f.parts - 1) * f.part_stride;  // past the last: re-read it
      dl_f32<EP>(xh + off + j0, ta[q]);
      dl_f32<EP>(xh + off + j0 + half, tc[q]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (p0 + q < f.parts)
#pragma unroll
        for (int e = 0; e < EP; ++e) { av[e] += ta[q][e]; cv[e] += tc[q][e]; }
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EP; ++e) ss += av[e] * av[e] + cv[e] * cv[e];
  ss = wave_sum(ss);
  const float inv = 1.f / sqrtf(ss / (float)HD + f.eps);
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    float u = av[e] * inv * wa[e], v = cv[e] * inv * wc[e];
    if (rope && j0 + e < f.n_rot) {
      const float u2 = u * co[e] - v * sn[e];
      const float v2 = v * co[e] + u * sn[e];
      u = u2; v = v2;
    }
    av[e] = u; cv[e] = v;
  }
  ds_bf16<EP>(lds + j0, av);
  ds_bf16<EP>(lds + j0 + half, cv);
  if (glob) {
    ds_bf16<EP>(glob + j0, av);
    ds_bf16<EP>(glob + j0 + half, cv);
  }
}

template <int HD, bool FQ>
__device__ __forceinline__ void dec_body(const AttnArgs& a, int chunk, int nchunk, float sl2, float* __restrict__ ws,
                                         const DecFuse* f) {
  constexpr int NC = HD / 128;  // 128-element chunks of a head
  constexpr int EPL = HD / 64;  // head elements per lane in P V
  __shared__ float red_o[4][DM_G][HD];
  __shared__ float red_ml[4][DM_G][2];
  __shared__ __attribute__((aligned(16))) bf16 q_lds[FQ ? DM_G : 1][FQ ? HD : 8];  // fused: the formed q heads
  __shared__ __attribute__((aligned(16))) bf16 kv_lds[FQ ? 2 : 1][FQ ? HD : 8];    // fused: the new key's k, v
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, q4 = lane >> 4;
  const int c = blockIdx.x;
  const int64_t g = blockIdx.y, b = blockIdx.z;
  const int G = (int)(a.nh / a.nkv);
  const int64_t i = a.pos0[b];
  int64_t lo = a.sliding ? i - a.window + 1 : 0;
  if (lo < 0) lo = 0;
  const int64_t hi = kv_last(i, a.cap, a.ring);
  // this wave's keys: [k0, k1)
  const int64_t cb = lo + (int64_t)c * chunk;
  const int wch = chunk / 4;
  int64_t k0 = cb + (int64_t)wave * wch, k1 = k0 + wch;
  if (k1 > hi + 1) k1 = hi + 1;
  const bf16* Kb = (const bf16*)a.k + (b * a.nkv + g) * a.cap * HD;
  const bf16* Vb = (const bf16*)a.v + (b * a.nkv + g) * a.cap * HD;

  // The K rows of the scores and the 16 V rows of P V of the step at key kt (a key past the range reads
  // the range's last row; its probability is exactly 0).
  typedef __attribute__((ext_vector_type(EPL / 2))) uint32_t vraw_t;
  uint4 kw[NC][4];
  vraw_t vw[16];
  auto load_kv = [&](int64_t kt) {
    const int64_t key = kt + col;
    const bf16* kr = Kb + kv_row(key < k1 ? key : kt, a.cap, a.ring) * HD + 8 * q4;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
      for (int t = 0; t < 4; ++t) kw[cc][t] = *(const uint4*)(kr + 128 * cc + 32 * t);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t kj = kt + j < k1 ? kt + j : k1 - 1;
      vw[j] = *(const vraw_t*)(Vb + kv_row(kj, a.cap, a.ring) * HD + lane * EPL);
    }
  };
  // fused, head dims up to 256: the first step's loads go out before q is formed, so the partials' round
  // trip overlaps them (at 512 the registers do not allow it)
  constexpr bool HOIST = FQ && HD <= 256;
  if (HOIST && k0 < k1) load_kv(k0);

  // queries of the group (rows = heads), element order matching the K operand
  bf16x8_t qf[NC][4];
  bool own_i = false;  // fused: this block's chunk holds the new key (a cache row this launch writes)
  if constexpr (FQ) {
    own_i = f->k_off >= 0 && i >= 0 && hi == i && i >= cb && i < cb + chunk;
    const float* xrow = f->x + b * f->x_ld;
    if (wave < G) dec_form_head<HD>(*f, xrow + f->q_off + (g * G + wave) * HD, f->qw, true, i, q_lds[wave], nullptr);
    if (own_i && wave >= 2) {
      const bool isk = wave == 2;
      bf16* crow = (bf16*)(isk ? a.k : a.v) + ((b * a.nkv + g) * a.cap + kv_row(i, a.cap, a.ring)) * HD;
      dec_form_head<HD>(*f, xrow + (isk ? f->k_off : f->v_off) + g * HD, isk ? f->kw : nullptr, isk, i,
                        kv_lds[wave - 2], crow);
    }
    __syncthreads();
    const bool real = col < G;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint4 v = real ? *(const uint4*)&q_lds[real ? col : 0][128 * cc + 32 * t + 8 * q4] : make_uint4(0, 0, 0, 0);
        qf[cc][t] = *(bf16x8_t*)&v;
      }
  } else {
    const bool real = col < G;
    const bf16* qr = (const bf16*)a.q + b * a.q_ld + (g * G + (real ? col : 0)) * HD + 8 * q4;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint4 v = real ? *(const uint4*)(qr + 128 * cc + 32 * t) : make_uint4(0, 0, 0, 0);
        qf[cc][t] = *(bf16x8_t*)&v;
      }
  }
  float acc[DM_G][EPL];
#pragma unroll
  for (int h = 0; h < DM_G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  float m_run[DM_G], l_run[DM_G];
#pragma unroll
  for (int h = 0; h < DM_G; ++h) { m_run[h] = -INFINITY; l_run[h] = 0.f; }

  for (int64_t kt = k0; kt < k1; kt += 16) {
    const bool kv = kt + col < k1;
    // every load of the step is issued before its first use
    if (!HOIST || kt != k0) load_kv(kt);
    if constexpr (FQ) {
      if (own_i && i >= kt && i < kt + 16) {  // wave-uniform: the new key's K and V from LDS
        const int jn = (int)(i - kt);
        if (col == jn)
#pragma unroll
          for (int cc = 0; cc < NC; ++cc)
#pragma unroll
            for (int t = 0; t < 4; ++t) kw[cc][t] = *(const uint4*)&kv_lds[0][128 * cc + 32 * t + 8 * q4];
        const vraw_t vn = *(const vraw_t*)&kv_lds[1][lane * EPL];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (j == jn) vw[j] = vn;
      }
    }
    // scores S[head][key] for 16 keys
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[cc][t], *(bf16x8_t*)&kw[cc][t], s, 0, 0, 0);
    // lanes 0..15: s[h] = score of head h for key kt + col
    float p[DM_G];
#pragma unroll
    for (int h = 0; h < DM_G; ++h) {
      const float v = (kv && q4 == 0) ? s[h] * sl2 : -INFINITY;
      float mt = v;
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) mt = fmaxf(mt, __shfl_xor(mt, off, 64));
      mt = first_lane_f(mt);  // lanes 0..15 agree; broadcast lane 0's value
      const float m_new = fmaxf(m_run[h], mt);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_use);
      p[h] = __builtin_amdgcn_exp2f(v - m_use);
      l_run[h] = l_run[h] * alpha + p[h];  // per-lane partial sum (lanes 0..15 carry the keys)
      m_run[h] = m_new;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
    }
    // P V over the 16 keys
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float vv[EPL];
#pragma unroll
      for (int e = 0; e < EPL / 2; ++e) {
        vv[2 * e] = __uint_as_float(vw[j][e] << 16);
        vv[2 * e + 1] = __uint_as_float(vw[j][e] & 0xffff0000u);
      }
#pragma unroll
      for (int h = 0; h < DM_G; ++h) {
        const float pf = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(p[h]), j));
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pf, vv[e], acc[h][e]);
      }
    }
  }
  // per-wave totals, then combine the 4 waves of the block
#pragma unroll
  for (int h = 0; h < DM_G; ++h) {
    float l = l_run[h];
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) l += __shfl_xor(l, off, 64);
    l_run[h] = first_lane_f(l);
  }
#pragma unroll
  for (int h = 0; h < DM_G; ++h) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) red_o[wave][h][lane * EPL + e] = acc[h][e];
    if (lane == 0) { red_ml[wave][h][0] = m_run[h]; red_ml[wave][h][1] = l_run[h]; }
  }
  __syncthreads();
  for (int x = tid; x < G * HD; x += 256) {
    const int h = x / HD, d = x - h * HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_ml[w][h][0]);
    float L = 0.f, o = 0.f;
    if (M > -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float sc = __builtin_amdgcn_exp2f(red_ml[w][h][0] - M);
        L += red_ml[w][h][1] * sc;
        o += red_o[w][h][d] * sc;
      }
    }
    float* dst = ws + (((b * a.nh + g * G + h) * nchunk) + c) * (int64_t)(HD + 2);
    dst[d] = o;
    if (d == 0) { dst[HD] = M; dst[HD + 1] = L; }
  }
}

template <int HD>
__global__ __launch_bounds__(256) void k_attn_dec_mfma(AttnArgs a, int chunk, int nchunk, float sl2,
                                                       float* __restrict__ ws) {
  dec_body<HD, false>(a, chunk, nchunk, sl2, ws, nullptr);
}

template <int HD>
__global__ __launch_bounds__(256) void k_attn_dec_mfmaf(AttnArgs a, int chunk, int nchunk, float sl2,
                                                        float* __restrict__ ws, DecFuse f) {
  dec_body<HD, true>(a, chunk, nchunk, sl2, ws, &f);
}

// Combines the key-chunk partials (m in the exp2 domain) of one (sequence, head) and 256 head elements
// (grid.y covers the head). The chunk weights exp2(m_c - M) are formed once in LDS; every thread then
// adds its element over the chunks with independent loads.
constexpr int DM_MAX_CHUNKS = 2048;

__global__ __launch_bounds__(256) void k_attn_dec_merge2(AttnArgs a, int nchunk, const float* __restrict__ ws) {
  __shared__ float wgt[DM_MAX_CHUNKS];
  __shared__ float sh[32];
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / a.nh, h = bh % a.nh;
  const int hd = (int)a.hd;
  const int tid = threadIdx.x;
  const float* src = ws + bh * nchunk * (int64_t)(hd + 2);
  float mloc = -INFINITY;
  for (int c = tid; c < nchunk; c += 256) mloc = fmaxf(mloc, src[c * (hd + 2) + hd]);
  mloc = wave_max(mloc);
  if ((tid & 63) == 0) sh[tid >> 6] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
  float lloc = 0.f;
  for (int c = tid; c < nchunk; c += 256) {
    const float w = M > -INFINITY ? __builtin_amdgcn_exp2f(src[c * (hd + 2) + hd] - M) : 0.f;
    wgt[c] = w;
    lloc += src[c * (hd + 2) + hd + 1] * w;
  }
  lloc = wave_sum(lloc);
  __syncthreads();
  if ((tid & 63) == 0) sh[4 + (tid >> 6)] = lloc;
  __syncthreads();
  const float L = sh[4] + sh[5] + sh[6] + sh[7];
  const float il = L > 0.f ? 1.f / L : 0.f;
  const int d = blockIdx.y * 256 + tid;
  if (d >= hd) return;
  float o = 0.f;
#pragma unroll 8
  for (int c = 0; c < nchunk; ++c) o += wgt[c] * src[c * (hd + 2) + d];
  stf((bf16*)a.out + b * a.out_ld + h * hd + d, o * il);
}

static void dm_plan(int64_t B, int64_t nkv, int64_t max_keys, int& chunk, int& nchunk) {
  chunk = 1024;
  while (chunk > 64 && B * nkv * ((max_keys + chunk - 1) / chunk) < 512) chunk >>= 1;
  nchunk = (int)((max_keys + chunk - 1) / chunk);
  while (nchunk > DM_MAX_CHUNKS) {  // the merge keeps one weight per chunk in LDS
    chunk *= 2;
    nchunk = (int)((max_keys + chunk - 1) / chunk);
  }
  if (nchunk < 1) nchunk = 1;
}

size_t attn_decode_mfma_ws(int64_t B, int64_t nh, int64_t hd, int64_t cap) {
  int chunk, nchunk;
  dm_plan(B, 1, cap, chunk, nchunk);
  return (size_t)B * nh * nchunk * (hd + 2) * sizeof(float);
}

// bf16, head_dim 128/256/512, at most 4 query heads per kv head, 16-byte aligned rows.
bool attn_decode_mfma(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t s, g4_status* st) {
  const int64_t G = a.nh / a.nkv;
  if (G > DM_G || !(a.hd == 128 || a.hd == 256 || a.hd == 512)) return false;
  if ((a.q_ld | a.out_ld) & 7) return false;
  if (((uintptr_t)a.q | (uintptr_t)a.k | (uintptr_t)a.v) & 15) return false;
  const int64_t max_keys = a.sliding ? (a.window < a.cap ? a.window : a.cap) : a.cap;
  int chunk, nchunk;
  dm_plan(a.B, a.nkv, max_keys, chunk, nchunk);
  const size_t need = (size_t)a.B * a.nh * nchunk * (a.hd + 2) * sizeof(float);
  if (!ws || ws_bytes < need) return false;
  dim3 g((unsigned)nchunk, (unsigned)a.nkv, (unsigned)a.B);
  const float sl2 = a.scale * 1.4426950408889634f;
  if (a.hd == 128) hipLaunchKernelGGL(k_attn_dec_mfma<128>, g, dim3(256), 0, s, a, chunk, nchunk, sl2, (float*)ws);
  else if (a.hd == 256) hipLaunchKernelGGL(k_attn_dec_mfma<256>, g, dim3(256), 0, s, a, chunk, nchunk, sl2, (float*)ws);
  else hipLaunchKernelGGL(k_attn_dec_mfma<512>, g, dim3(256), 0, s, a, chunk, nchunk, sl2, (float*)ws);
  if ((*st = check_launch("attn_decode_mfma")) != G4_OK) return true;
  hipLaunchKernelGGL(k_attn_dec_merge2, dim3((unsigned)(a.B * a.nh), (unsigned)((a.hd + 255) / 256)), dim3(256), 0, s, a,
                     nchunk, (const float*)ws);
  *st = check_launch("attn_decode_merge");
  return true;
}

// The fused form: one token per sequence, the shapes of attn_decode_mfma, the partials 16-byte aligned with
// every stride and offset a multiple of 4 elements, the norm weights 8-byte aligned.
bool attn_decode_fused(const AttnArgs& a, const DecFuse& f, void* ws, size_t ws_bytes, hipStream_t s, g4_status* st) {
  const int64_t G = a.nh / a.nkv;
  if (a.T != 1 || G > DM_G || !(a.hd == 128 || a.hd == 256 || a.hd == 512)) return false;
  if ((a.out_ld & 7) || (((uintptr_t)a.k | (uintptr_t)a.v) & 15)) return false;
  if (!f.x || !f.qw || f.parts < 1 || ((uintptr_t)f.x & 15) || ((f.x_ld | f.part_stride | f.q_off) & 3)) return false;
  if (f.k_off >= 0 && (!f.kw || f.v_off < 0 || ((f.k_off | f.v_off) & 3) || ((uintptr_t)f.kw & 7))) return false;
  if ((uintptr_t)f.qw & 7) return false;
  const int64_t max_keys = a.sliding ? (a.window < a.cap ? a.window : a.cap) : a.cap;
  int chunk, nchunk;
  dm_plan(a.B, a.nkv, max_keys, chunk, nchunk);
  const size_t need = (size_t)a.B * a.nh * nchunk * (a.hd + 2) * sizeof(float);
  if (!ws || ws_bytes < need) return false;
  dim3 g((unsigned)nchunk, (unsigned)a.nkv, (unsigned)a.B);
  const float sl2 = a.scale * 1.4426950408889634f;
  if (a.hd == 128) hipLaunchKernelGGL(k_attn_dec_mfmaf<128>, g, dim3(256), 0, s, a, chunk, nchunk, sl2, (float*)ws, f);
  else if (a.hd == 256) hipLaunchKernelGGL(k_attn_dec_mfmaf<256>, g, dim3(256), 0, s, a, chunk, nchunk, sl2, (float*)ws, f);
  else hipLaunchKernelGGL(k_attn_dec_mfmaf<512>, g, dim3(256), 0, s, a, chunk, nchunk, sl2, (float*)ws, f);
  if ((*st = check_launch("attn_decode_fused")) != G4_OK) return true;
  hipLaunchKernelGGL(k_attn_dec_merge2, dim3((unsigned)(a.B * a.nh), (unsigned)((a.hd + 255) / 256)), dim3(256), 0, s, a,
                     nchunk, (const float*)ws);
  *st = check_launch("attn_decode_merge");
  return true;
}

}  // namespace g4
