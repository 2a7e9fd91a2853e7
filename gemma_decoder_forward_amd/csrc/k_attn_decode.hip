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
#include "g4_internal.h"

namespace g4 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr int DM_G = 4;  // query heads per kv head handled (rows of the score MFMA in use)

template <int HD>
__global__ __launch_bounds__(256) void k_attn_dec_mfma(AttnArgs a, int chunk, int nchunk, float sl2,
                                                       float* __restrict__ ws) {
  constexpr int NC = HD / 128;  // 128-element chunks of a head
  constexpr int EPL = HD / 64;  // head elements per lane in P V
  __shared__ float red_o[4][DM_G][HD];
  __shared__ float red_ml[4][DM_G][2];
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

  // queries of the group (rows = heads), element order matching the K operand
  bf16x8_t qf[NC][4];
  {
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
  const bf16* Kb = (const bf16*)a.k + (b * a.nkv + g) * a.cap * HD;
  const bf16* Vb = (const bf16*)a.v + (b * a.nkv + g) * a.cap * HD;

  float acc[DM_G][EPL];
#pragma unroll
  for (int h = 0; h < DM_G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  float m_run[DM_G], l_run[DM_G];
#pragma unroll
  for (int h = 0; h < DM_G; ++h) { m_run[h] = -INFINITY; l_run[h] = 0.f; }

  for (int64_t kt = k0; kt < k1; kt += 16) {
    const int64_t key = kt + col;
    const bool kv = key < k1;
    // Every load of the step is issued before its first use: the K rows of the scores and the 16 V
    // rows of P V (a key past the range reads the range's last row; its probability is exactly 0).
    const bf16* kr = Kb + kv_row(kv ? key : kt, a.cap, a.ring) * HD + 8 * q4;
    uint4 kw[NC][4];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
      for (int t = 0; t < 4; ++t) kw[cc][t] = *(const uint4*)(kr + 128 * cc + 32 * t);
    typedef __attribute__((ext_vector_type(EPL / 2))) uint32_t vraw_t;
    vraw_t vw[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t kj = kt + j < k1 ? kt + j : k1 - 1;
      vw[j] = *(const vraw_t*)(Vb + kv_row(kj, a.cap, a.ring) * HD + lane * EPL);
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

}  // namespace g4
