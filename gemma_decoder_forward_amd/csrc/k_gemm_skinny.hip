// Weight-streaming GEMM for few token rows (decode: M = batch <= 64): C = A B^T with B the weights.
//
// HBM-bound: every weight byte is read once. A block owns 64 weight rows (one 16-row MFMA block per wave)
// or 16 rows (see RW below) and a K range of kc; the activation slice A[0:M, k-range] is staged once in
// LDS. Per 128-k step a lane reads four 16-byte pieces of its weight row; load t of a step covers
// k = 32t .. 32t+31 of 16 rows, the four lanes of a row reading 64 contiguous bytes, and
// v_mfma_f32_16x16x32_bf16 t takes exactly those: lane l supplies row (l % 16) and k = 32t + 8(l/16)
// .. +7, for the activations and the weights alike.
// Blocks over K write float32 partials [split][M][rows]; k_gemm_finish sums them and applies the
// epilogue (store, gelu-tanh gate*up, gelu*aux).
//
// B may be the concatenation of up to three matrices (q/k/v projections, or gate then up) so that one
// launch covers them; the output columns follow the concatenation.
//
// For at most 4 token rows (k_gemv) the products are formed on the vector ALUs instead: a wave reads
// its weight rows as contiguous 1 KB runs (64 lanes x 16 bytes), the pattern that keeps HBM streaming
// (the MFMA operand layout makes each load instruction touch 64 bytes of 16 different rows, which caps
// a pure read of the gate/up weights near 4.4 TB/s against 5.6 TB/s row by row on the same device).
// Each lane takes 8 consecutive k of a row per 512-k chunk, the 16-byte A pieces at the same k from LDS,
// and accumulates with v_dot2c_f32_bf16; a wave sum per (row, token row) finishes. Same partial-slice
// output and epilogues as k_gemm_skinny.
#include "g4_internal.h"

namespace g4 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

struct SkSeg {
  const bf16* b[3];
  int64_t end[3];  // row ranges [end[i-1], end[i]) of the concatenated B
  int64_t ldb;
};

__device__ __forceinline__ const bf16* sk_row(const SkSeg& s, int64_t r) {
  if (r < s.end[0]) return s.b[0] + r * s.ldb;
  if (r < s.end[1]) return s.b[1] + (r - s.end[0]) * s.ldb;
  return s.b[2] + (r - s.end[1]) * s.ldb;
}

constexpr int SK_D = 4;  // 128-k steps per batch of weight loads

// LDS rows of the staged A slice: the M token rows, plus a zero row when the MFMA blocks have more rows.
__host__ __device__ inline int sk_lds_rows(int mb, int64_t M) { return M < 16 * mb ? (int)M + 1 : 16 * mb; }

// 8 consecutive A values formed from float32 partial slices (see SkAKind), rounded to bf16. The slices'
// loads go out four at a time (one memory round trip per four slices), and are added in slice order.
template <int AK>
__device__ __forceinline__ uint4 sk_a_from_parts(const SkA& sa, int64_t m, int64_t k) {
  const float* pr = (const float*)sa.a + m * sa.lda + k;
  constexpr int PB = 4;
  float g[8], u[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) g[e] = u[e] = 0.f;
  for (int p0 = 0; p0 < sa.parts; p0 += PB) {
    float4 x0[PB], x1[PB], y0[PB], y1[PB];
#pragma unroll
    for (int q = 0; q < PB; ++q) {
      const int p = p0 + q < sa.parts ? p0 + q : sa.parts - 1;  // past the last slice: re-read it (unused)
      const float* ps = pr + p * sa.part_stride;
      x0[q] = *(const float4*)ps;
      x1[q] = *(const float4*)(ps + 4);
      if (AK == SKA_GEGLU) {
        y0[q] = *(const float4*)(ps + sa.up_off);
        y1[q] = *(const float4*)(ps + sa.up_off + 4);
      }
    }
#pragma unroll
    for (int q = 0; q < PB; ++q) {
      if (p0 + q >= sa.parts) break;
      g[0] += x0[q].x; g[1] += x0[q].y; g[2] += x0[q].z; g[3] += x0[q].w;
      g[4] += x1[q].x; g[5] += x1[q].y; g[6] += x1[q].z; g[7] += x1[q].w;
      if (AK == SKA_GEGLU) {
        u[0] += y0[q].x; u[1] += y0[q].y; u[2] += y0[q].z; u[3] += y0[q].w;
        u[4] += y1[q].x; u[5] += y1[q].y; u[6] += y1[q].z; u[7] += y1[q].w;
      }
    }
  }
  if (AK == SKA_GELU_MUL) {
    const float* ar = sa.aux + m * sa.aux_ld + k;
    const float4 y0 = *(const float4*)ar, y1 = *(const float4*)(ar + 4);
    u[0] = y0.x; u[1] = y0.y; u[2] = y0.z; u[3] = y0.w; u[4] = y1.x; u[5] = y1.y; u[6] = y1.z; u[7] = y1.w;
  }
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = (uint32_t)f2bf(gelu_tanh(g[2 * e]) * u[2 * e]) | ((uint32_t)f2bf(gelu_tanh(g[2 * e + 1]) * u[2 * e + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// RW = 4: each wave owns 16 weight rows over the block's whole K range (64 rows per block, A shared by
// the four waves). RW = 1: the four waves share 16 rows and split the block's K range between them,
// adding their sums through LDS at the end -- for matrices with few rows, so that the grid fills the
// chip with fewer K splits (fewer partial slices for the consumer to add).
// GATED: the gelu-tanh gated product of two matrices in one pass (one K split): block b owns output
// columns 16b .. 16b+15; waves 0, 1 take those gate rows and waves 2, 3 the same up rows, each pair
// splitting K in halves. The four sums meet in LDS and wave 0 stores bf16(gelu_tanh(gate) * up) to
// C[m][16b + ...] (ldc = Nt).
// Stages A[0:M, k0:k0+kn] in LDS as bf16 rows of stride ald, plus zero rows up to nrow.
template <int AK>
__device__ __forceinline__ void sk_stage_a(const SkA& sa, int64_t M, int64_t k0, int kn, int nrow, int ald, bf16* As) {
  const int cpr = kn / 8;
  for (int idx = threadIdx.x; idx < nrow * cpr; idx += 256) {
    const int m = idx / cpr, c = idx - m * cpr;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (m < M) {
      if (AK == SKA_BF16) v = *(const uint4*)((const bf16*)sa.a + m * sa.lda + k0 + 8 * c);
      else v = sk_a_from_parts<AK>(sa, m, k0 + 8 * c);
    }
    *(uint4*)(As + m * ald + 8 * c) = v;
  }
}

template <int MB, int AK, int RW, bool GATED = false>
__global__ __launch_bounds__(256) void k_gemm_skinny(SkA sa, int64_t M, SkSeg sg, int64_t K, int kc,
                                                     float* __restrict__ part, int64_t Nt) {
  extern __shared__ __attribute__((aligned(16))) bf16 As[];
  constexpr int BR = 16 * RW;  // weight rows per block
  const int ald = kc + 8;  // LDS row stride (bf16); (kc + 8) * 2 bytes = 4 (mod 64) words -> conflict-free rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t k0 = (int64_t)blockIdx.y * kc;
  const int kn = (int)((K - k0) < kc ? (K - k0) : kc);
  const int nst = kn >> 7;  // 128-k steps of this block
  const int q = lane >> 4;
  const int wrow0 = RW == 4 && !GATED ? wave * 16 : 0;
  // steps of each wave: [sbeg, send)
  const int spw = GATED ? (nst + 1) / 2 : (RW == 4 ? nst : (nst + 3) / 4);
  const int sbeg = GATED ? (wave & 1) * spw : (RW == 4 ? 0 : wave * spw);
  const int send = sbeg + spw < nst ? sbeg + spw : nst;
  const int nmine = send > sbeg ? send - sbeg : 0;

  // Weights through a buffer descriptor that starts at the block's first row (a block never straddles
  // two matrices of the concatenation): a step past this wave's K range gets an offset beyond the
  // descriptor's size, reads as zero and costs no memory traffic. So every load below is issued
  // unconditionally, the compiler's wait counts stay exact, and batches are double-buffered in
  // registers: the loads of batch i+1 are in flight while batch i is multiplied.
  const bf16* wblk = GATED ? sg.b[__builtin_amdgcn_readfirstlane(wave) >> 1] + (int64_t)blockIdx.x * 16 * sg.ldb + k0
                           : sk_row(sg, (int64_t)blockIdx.x * BR) + k0;
  const int64_t wbytes = ((GATED ? 15 : BR - 1) * sg.ldb + kn) * 2;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)wblk, (short)0, (int)wbytes, 0x00020000);
  const uint32_t lrow = (uint32_t)(((GATED ? 0 : wrow0) + (lane & 15)) * sg.ldb + 8 * q) * 2;
  auto load_batch = [&](uint4 (&w)[SK_D][4], int s0) {
#pragma unroll
    for (int s = 0; s < SK_D; ++s) {
      const int st = sbeg + s0 + s;
      const uint32_t off = st < send ? lrow + (uint32_t)st * 256 : 0x80000000u;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(off + 64 * t), 0, 0);
        w[s][t] = *(const uint4*)&v;
      }
    }
  };
  uint4 wa[SK_D][4], wb[SK_D][4];
  load_batch(wa, 0);

  // stage A[0:M, k0:k0+kn] while the first weights arrive, plus one zero row that stands in for every
  // MFMA row >= M (so the LDS slice and its staging scale with M, not with the 16-row MFMA blocks)
  const int nrow = sk_lds_rows(MB, M);
  sk_stage_a<AK>(sa, M, k0, kn, nrow, ald, As);
  __syncthreads();

  int aoff[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = mb * 16 + (lane & 15);
    aoff[mb] = (m < M ? m : nrow - 1) * ald + 8 * q;
  }
  f32x4_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  auto mul_batch = [&](const uint4 (&w)[SK_D][4], int s0) {
#pragma unroll
    for (int s = 0; s < SK_D; ++s)
      if (s0 + s < nmine) {  // uniform; the LDS slice of A ends at this block's K range
        const int kk = (sbeg + s0 + s) * 128;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x8_t bw = *(const bf16x8_t*)&w[s][t];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const bf16x8_t af = *(const bf16x8_t*)(As + aoff[mb] + kk + 32 * t);
            acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bw, acc[mb], 0, 0, 0);
          }
        }
      }
  };
  // two register batches alternate roles (no copies between them, so no waits for data in flight)
  for (int s0 = 0; s0 < nmine; s0 += 2 * SK_D) {
    load_batch(wb, s0 + SK_D);
    mul_batch(wa, s0);
    load_batch(wa, s0 + 2 * SK_D);
    mul_batch(wb, s0 + SK_D);
  }
  if (GATED) {
    __shared__ f32x4_t xs[3][MB][64];
    if (wave > 0)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) xs[wave - 1][mb][lane] = acc[mb];
    __syncthreads();
    if (wave > 0) return;
    bf16* C = (bf16*)part;
    const int64_t n = (int64_t)blockIdx.x * 16 + (lane & 15);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const f32x4_t g = acc[mb] + xs[0][mb][lane], u = xs[1][mb][lane] + xs[2][mb][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = mb * 16 + 4 * q + i;
        if (m < M) C[m * Nt + n] = f2bf(gelu_tanh(g[i]) * u[i]);
      }
    }
    return;
  }
  if (RW == 1) {  // add the four waves' sums
    __shared__ f32x4_t red[3][MB][64];
    if (wave > 0)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) red[wave - 1][mb][lane] = acc[mb];
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int w = 0; w < 3; ++w) acc[mb] += red[w][mb][lane];
  }
  // C[m][r]: lane holds column (lane % 16) and rows 4*(lane/16) + i of each 16-row block
  const int64_t r = (int64_t)blockIdx.x * BR + wrow0 + (lane & 15);
  float* pb = part + (int64_t)blockIdx.y * M * Nt;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = mb * 16 + 4 * q + i;
      if (m < M) pb[m * Nt + r] = acc[mb][i];
    }
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v;
// Token rows taken by k_gemv, from timings of both kernels on the decode shapes (gate+up 20480 x 2560,
// down 2560 x 10240, q/k/v 3072 x 2560, o 2560 x 2048): the vector-ALU path is faster on every shape
// up to 2 rows (by 1.6-4.2 us), on all but gate+up at 3-4 rows, and slower from 6 rows on, where each
// 16-row block re-staging M x K activations costs more than the better weight stream saves.
constexpr int GV_MAX = 4;        // split-K products
constexpr int GV_MAX_GATED = 2;  // the one-pass gate/up product
constexpr int GV_CH = 5;   // 512-k chunks of each weight row loaded per round trip

// 16 bytes of a weight row dotted with 16 bytes of an A row: four bf16 pairs, float32 accumulation.
__device__ __forceinline__ float gv_dot8(const uint4& w, const uint4& a, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, w.x), __builtin_bit_cast(bf16x2_v, a.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, w.y), __builtin_bit_cast(bf16x2_v, a.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, w.z), __builtin_bit_cast(bf16x2_v, a.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, w.w), __builtin_bit_cast(bf16x2_v, a.w), acc, false);
  return acc;
}

// MM: compile-time bound on the token rows (M <= MM). Block = 4 waves, each wave four weight rows over
// the block's K range [k0, k0 + kc): rows 16 b + 4 w .. +3 of the concatenation (partial slices out), or
// (GATED, one K range) the gate and up rows of output columns 8 b + 2 w and 8 b + 2 w + 1, written as
// bf16(gelu_tanh(gate) * up) to C[m][col] (row stride Nt).
template <int MM, int AK, bool GATED>
__global__ __launch_bounds__(256) void k_gemv(SkA sa, int64_t M, SkSeg sg, int64_t K, int kc,
                                              float* __restrict__ part, int64_t Nt) {
  extern __shared__ __attribute__((aligned(16))) bf16 As[];
  const int ald = kc + 8;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t k0 = (int64_t)blockIdx.y * kc;
  const int kn = (int)((K - k0) < kc ? (K - k0) : kc);
  const int nch = (kn + 511) >> 9;

  // The wave's four rows, each through a buffer descriptor of exactly its kn elements: a chunk's lanes
  // past the row's end read zero and cost no traffic. (Segments are multiples of 64 rows, so the four
  // rows of a wave lie in one matrix.)
  const bf16* wr[4];
  if (GATED) {
    const int64_t c0 = (int64_t)blockIdx.x * 8 + 2 * wave;
    wr[0] = sg.b[0] + c0 * sg.ldb + k0;
    wr[2] = sg.b[1] + c0 * sg.ldb + k0;
    wr[1] = wr[0] + sg.ldb;
    wr[3] = wr[2] + sg.ldb;
  } else {
    wr[0] = sk_row(sg, (int64_t)blockIdx.x * 16 + 4 * wave) + k0;
    wr[1] = wr[0] + sg.ldb;
    wr[2] = wr[1] + sg.ldb;
    wr[3] = wr[2] + sg.ldb;
  }
  __amdgpu_buffer_rsrc_t rs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) rs[j] = __builtin_amdgcn_make_buffer_rsrc((void*)wr[j], (short)0, kn * 2, 0x00020000);

  // first round trip of weights in flight while A is staged
  uint4 w[4][GV_CH];
  auto load = [&](int cg) {
#pragma unroll
    for (int c = 0; c < GV_CH; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs[j], 16 * lane + 1024 * (cg + c), 0, 0);
        w[j][c] = *(const uint4*)&v;
      }
  };
  load(0);
  const int nrow = sk_lds_rows(1, M);
  sk_stage_a<AK>(sa, M, k0, kn, nrow, ald, As);
  __syncthreads();

  float acc[4][MM];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int m = 0; m < MM; ++m) acc[j][m] = 0.f;
  for (int cg = 0; cg < nch; cg += GV_CH) {
    if (cg > 0) load(cg);
#pragma unroll
    for (int c = 0; c < GV_CH; ++c) {
      const int kk = 8 * lane + 512 * (cg + c);
      if (cg + c < nch) {  // uniform
#pragma unroll
        for (int m = 0; m < MM; ++m) {
          const uint4 a = (m < M && kk < kn) ? *(const uint4*)(As + m * ald + kk) : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j][m] = gv_dot8(w[j][c], a, acc[j][m]);
        }
      }
    }
  }
  if (GATED) {
    bf16* C = (bf16*)part;
    const int64_t c0 = (int64_t)blockIdx.x * 8 + 2 * wave;
#pragma unroll
    for (int m = 0; m < MM; ++m)
      if (m < M) {
        const float g0 = wave_sum(acc[0][m]), g1 = wave_sum(acc[1][m]);
        const float u0 = wave_sum(acc[2][m]), u1 = wave_sum(acc[3][m]);
        if (lane < 2) C[m * Nt + c0 + lane] = f2bf(lane == 0 ? gelu_tanh(g0) * u0 : gelu_tanh(g1) * u1);
      }
    return;
  }
  float* pb = part + (int64_t)blockIdx.y * M * Nt + (int64_t)blockIdx.x * 16 + 4 * wave;
#pragma unroll
  for (int m = 0; m < MM; ++m)
    if (m < M) {
      const float s0 = wave_sum(acc[0][m]), s1 = wave_sum(acc[1][m]);
      const float s2 = wave_sum(acc[2][m]), s3 = wave_sum(acc[3][m]);
      if (lane < 4) pb[m * Nt + lane] = lane == 0 ? s0 : (lane == 1 ? s1 : (lane == 2 ? s2 : s3));
    }
}

// Sums the split partials and applies the epilogue. GEGLU: part columns [0, N) are gate, [N, 2N) up.
// SOFTCAP: float32 C = cap * tanh(sum / cap).
template <int EPI, bool CF32>
__global__ __launch_bounds__(256) void k_gemm_finish(GemmArgs a, const float* __restrict__ part, int splits,
                                                     int64_t Nt) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.M * a.N) return;
  const int64_t m = idx / a.N, n = idx - m * a.N;
  float v = 0.f, u = 0.f;
  for (int s = 0; s < splits; ++s) {
    v += part[((int64_t)s * a.M + m) * Nt + n];
    if (EPI == EPI_GEGLU) u += part[((int64_t)s * a.M + m) * Nt + a.N + n];
  }
  if (EPI == EPI_GEGLU) {
    ((bf16*)a.C)[m * a.ldc + n] = f2bf(gelu_tanh(v) * u);
  } else if (EPI == EPI_GELU_MUL) {
    ((bf16*)a.C)[m * a.ldc + n] = f2bf(gelu_tanh(v) * a.aux[m * a.aux_ld + n]);
  } else if (EPI == EPI_SOFTCAP) {
    ((float*)a.C)[m * a.ldc + n] = a.cap * tanhf(v * (1.f / a.cap));
  } else if (CF32) {
    ((float*)a.C)[m * a.ldc + n] = v;
  } else {
    ((bf16*)a.C)[m * a.ldc + n] = f2bf(v);
  }
}

// Rows per block: 64 (four waves on separate rows) when the matrix has enough rows, else 16 (four waves
// splitting K). With more than 16 token rows every block stages a large A slice, so 64-row blocks
// (which share it four ways) are preferred down to 2048-row matrices. Then the K range per block (kc, a multiple of 128) and the number of K splits: about
// three blocks per CU, each wave with at least one 128-k step, and the LDS slice of A, 16*mb rows x
// (kc + 8) bf16, within 66 KB (mb 1, 2) or 132 KB (mb 4, one block per CU with deep weight loads).
static void sk_plan(int mb, int64_t K, int64_t Nt, int& rw, int& kc, int& splits) {
  rw = Nt / 64 >= (mb == 1 ? 192 : 32) ? 4 : 1;  // with more token rows, A staging favours 64-row blocks
  const int64_t rowblocks = Nt / (16 * rw);
  const int64_t steps = K / 128;
  const int64_t max_steps = mb == 1 ? 16 : 8;
  int64_t s = (768 + rowblocks - 1) / rowblocks;
  if (rw == 1 && s > steps / 4) s = steps / 4;  // at least one step per wave
  const int64_t smin = (steps + max_steps - 1) / max_steps;
  if (s < smin) s = smin;
  if (s > steps) s = steps;
  if (s < 1) s = 1;
  const int64_t per = (steps + s - 1) / s;
  kc = (int)(per * 128);
  splits = (int)((steps + per - 1) / per);
}

// k_gemv: 16-row blocks, K split so that about four blocks per CU stream (blocks of one K range each), the
// K range a multiple of 128 and its A slice within 64 KB of LDS. At most 4 K ranges for up to two token
// rows (8 above): every consumer adds the slices, four per memory round trip, on the step's critical path
// (the PLE gate, 256 outputs, would otherwise split 20 ways: 3.69 -> 3.45 ms per 42-layer step at one
// token row, 4.44 -> 4.25 at four).
static void gv_plan(int64_t M, int64_t K, int64_t Nt, int& kc, int& splits) {
  const int64_t rowblocks = Nt / 16;
  const int64_t steps = K / 128;
  const int64_t max_steps = ((65536 / (2 * sk_lds_rows(1, M))) - 8) / 128;
  int64_t s = (1024 + rowblocks - 1) / rowblocks;
  const int64_t cap = M <= 2 ? 4 : 8;
  if (s > cap) s = cap;
  const int64_t smin = (steps + max_steps - 1) / max_steps;
  if (s < smin) s = smin;
  if (s > steps) s = steps;
  if (s < 1) s = 1;
  const int64_t per = (steps + s - 1) / s;
  kc = (int)(per * 128);
  splits = (int)((steps + per - 1) / per);
}

size_t gemm_skinny_ws(int64_t M, int64_t Nt, int64_t K) {
  int rw, kc, splits;
  if (M <= GV_MAX) {
    gv_plan(M, K, Nt, kc, splits);
  } else {
    sk_plan(M <= 16 ? 1 : (M <= 32 ? 2 : 4), K, Nt, rw, kc, splits);
  }
  return (size_t)splits * M * Nt * sizeof(float);
}

bool skinny_ok(int64_t M, int64_t K, const void* const* segs, const int64_t* seg_rows, int nseg, int64_t ldb) {
  if (M > 64 || M <= 0 || K % 128 || ldb % 8 || nseg < 1 || nseg > 3) return false;
  for (int i = 0; i < nseg; ++i)
    if (seg_rows[i] % 64 || ((uintptr_t)segs[i] & 15)) return false;
  return true;
}

template <int MB, int RW>
static void sk_launch(const SkA& sa, dim3 g, size_t lds, hipStream_t s, int64_t M, const SkSeg& sg, int64_t K,
                      int kc, float* part, int64_t Nt) {
  static bool lds_set = false;  // allow > 64 KB of dynamic LDS (gfx950 has 160 KB per CU)
  if (!lds_set) {
    (void)hipFuncSetAttribute((const void*)k_gemm_skinny<MB, SKA_BF16, RW>, hipFuncAttributeMaxDynamicSharedMemorySize, 140 * 1024);
    (void)hipFuncSetAttribute((const void*)k_gemm_skinny<MB, SKA_GEGLU, RW>, hipFuncAttributeMaxDynamicSharedMemorySize, 140 * 1024);
    (void)hipFuncSetAttribute((const void*)k_gemm_skinny<MB, SKA_GELU_MUL, RW>, hipFuncAttributeMaxDynamicSharedMemorySize, 140 * 1024);
    lds_set = true;
  }
  if (sa.kind == SKA_GEGLU)
    hipLaunchKernelGGL((k_gemm_skinny<MB, SKA_GEGLU, RW>), g, dim3(256), lds, s, sa, M, sg, K, kc, part, Nt);
  else if (sa.kind == SKA_GELU_MUL)
    hipLaunchKernelGGL((k_gemm_skinny<MB, SKA_GELU_MUL, RW>), g, dim3(256), lds, s, sa, M, sg, K, kc, part, Nt);
  else
    hipLaunchKernelGGL((k_gemm_skinny<MB, SKA_BF16, RW>), g, dim3(256), lds, s, sa, M, sg, K, kc, part, Nt);
}

template <bool GATED>
static void gv_launch(const SkA& sa, dim3 g, hipStream_t s, int64_t M, const SkSeg& sg, int64_t K, int kc, float* part,
                      int64_t Nt) {
  const size_t lds = (size_t)sk_lds_rows(1, M) * (kc + 8) * sizeof(bf16);  // <= 64 KB (gv_plan)
#define G4_GV(MM, AKV) hipLaunchKernelGGL((k_gemv<MM, AKV, GATED>), g, dim3(256), lds, s, sa, M, sg, K, kc, part, Nt)
#define G4_GV_M(AKV) \
  do { if (M <= 1) G4_GV(1, AKV); else if (M <= 2) G4_GV(2, AKV); else G4_GV(4, AKV); } while (0)
  if constexpr (GATED) {
    G4_GV_M(SKA_BF16);
  } else {
    if (sa.kind == SKA_BF16) G4_GV_M(SKA_BF16);
    else if (sa.kind == SKA_GEGLU) G4_GV_M(SKA_GEGLU);
    else G4_GV_M(SKA_GELU_MUL);
  }
#undef G4_GV_M
#undef G4_GV
}

g4_status gemm_skinny_part(const SkA& sa, int64_t M, int64_t K, const void* const* segs, const int64_t* seg_rows,
                           int nseg, int64_t ldb, float* part, size_t part_bytes, int* splits_out, hipStream_t s) {
  if (!skinny_ok(M, K, segs, seg_rows, nseg, ldb))
    return fail(G4_EUNSUP, "few-row GEMM: unsupported shape M=%lld K=%lld", (long long)M, (long long)K);
  if (sa.kind == SKA_BF16 ? (sa.lda % 8 || ((uintptr_t)sa.a & 15))
                          : (sa.lda % 4 || sa.part_stride % 4 || sa.up_off % 4 || sa.parts < 1 || ((uintptr_t)sa.a & 15) ||
                             (sa.kind == SKA_GELU_MUL && (sa.aux_ld % 4 || ((uintptr_t)sa.aux & 15)))))
    return fail(G4_EUNSUP, "few-row GEMM: A operand rows not 16-byte aligned");
  SkSeg sg{};
  int64_t Nt = 0;
  for (int i = 0; i < 3; ++i) {
    if (i < nseg) {
      Nt += seg_rows[i];
      sg.b[i] = (const bf16*)segs[i];
    } else {
      sg.b[i] = sg.b[nseg - 1];
    }
    sg.end[i] = Nt;
  }
  sg.ldb = ldb;
  if (M <= GV_MAX) {
    int kc, splits;
    gv_plan(M, K, Nt, kc, splits);
    if ((size_t)splits * M * Nt * sizeof(float) > part_bytes)
      return fail(G4_EINVAL, "few-row GEMM: partial buffer too small");
    gv_launch<false>(sa, dim3((unsigned)(Nt / 16), (unsigned)splits), s, M, sg, K, kc, part, Nt);
    *splits_out = splits;
    return check_launch("gemv");
  }
  const int mb = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  int rw, kc, splits;
  sk_plan(mb, K, Nt, rw, kc, splits);
  if ((size_t)splits * M * Nt * sizeof(float) > part_bytes)
    return fail(G4_EINVAL, "few-row GEMM: partial buffer too small");
  dim3 g((unsigned)(Nt / (16 * rw)), (unsigned)splits);
  const size_t lds = (size_t)sk_lds_rows(mb, M) * (kc + 8) * sizeof(bf16);
  if (rw == 4) {
    if (mb == 1) sk_launch<1, 4>(sa, g, lds, s, M, sg, K, kc, part, Nt);
    else if (mb == 2) sk_launch<2, 4>(sa, g, lds, s, M, sg, K, kc, part, Nt);
    else sk_launch<4, 4>(sa, g, lds, s, M, sg, K, kc, part, Nt);
  } else {
    if (mb == 1) sk_launch<1, 1>(sa, g, lds, s, M, sg, K, kc, part, Nt);
    else if (mb == 2) sk_launch<2, 1>(sa, g, lds, s, M, sg, K, kc, part, Nt);
    else sk_launch<4, 1>(sa, g, lds, s, M, sg, K, kc, part, Nt);
  }
  *splits_out = splits;
  return check_launch("gemm_skinny");
}

void skinny_plan(int64_t M, int64_t K, int64_t Nt, int* rows_per_block, int* kc, int* splits) {
  if (M <= GV_MAX) {
    gv_plan(M, K, Nt, *kc, *splits);
    *rows_per_block = 16;
    return;
  }
  int rw = 0;
  sk_plan(M <= 16 ? 1 : (M <= 32 ? 2 : 4), K, Nt, rw, *kc, *splits);
  *rows_per_block = 16 * rw;
}

g4_status gemm_skinny_finish(const GemmArgs& a, const float* part, int splits, int64_t Nt, hipStream_t s) {
  if (a.M * a.N == 0) return G4_OK;
  dim3 gf((unsigned)((a.M * a.N + 255) / 256));
  if (a.epi == EPI_GEGLU) hipLaunchKernelGGL((k_gemm_finish<EPI_GEGLU, false>), gf, dim3(256), 0, s, a, part, splits, Nt);
  else if (a.epi == EPI_GELU_MUL) hipLaunchKernelGGL((k_gemm_finish<EPI_GELU_MUL, false>), gf, dim3(256), 0, s, a, part, splits, Nt);
  else if (a.epi == EPI_SOFTCAP) {
    if (a.c_dtype != G4_F32 || !(a.cap > 0.f)) return fail(G4_EUNSUP, "gemm_finish: softcap needs a float32 C and cap > 0");
    hipLaunchKernelGGL((k_gemm_finish<EPI_SOFTCAP, true>), gf, dim3(256), 0, s, a, part, splits, Nt);
  } else if (a.c_dtype == G4_F32) hipLaunchKernelGGL((k_gemm_finish<EPI_STORE, true>), gf, dim3(256), 0, s, a, part, splits, Nt);
  else hipLaunchKernelGGL((k_gemm_finish<EPI_STORE, false>), gf, dim3(256), 0, s, a, part, splits, Nt);
  return check_launch("gemm_finish");
}

bool skinny_gated_ok(int64_t M, int64_t K, int64_t F) {
  return M >= 1 && M <= 16 && K % 256 == 0 && F % 16 == 0 && (size_t)sk_lds_rows(1, M) * (K + 8) * sizeof(bf16) <= 96 * 1024;
}

g4_status gemm_skinny_gated(const SkA& sa, int64_t M, int64_t K, const void* w_gate, const void* w_up, int64_t F,
                            int64_t ldb, void* C, int64_t ldc, hipStream_t s) {
  if (!skinny_gated_ok(M, K, F) || sa.kind != SKA_BF16 || ldb % 8 || ((uintptr_t)w_gate & 15) || ((uintptr_t)w_up & 15) ||
      sa.lda % 8 || ((uintptr_t)sa.a & 15))
    return fail(G4_EUNSUP, "gated few-row GEMM: unsupported shape M=%lld K=%lld F=%lld", (long long)M, (long long)K,
                (long long)F);
  SkSeg sg{};
  sg.b[0] = (const bf16*)w_gate;
  sg.b[1] = (const bf16*)w_up;
  sg.b[2] = (const bf16*)w_up;
  sg.end[0] = F; sg.end[1] = 2 * F; sg.end[2] = 2 * F;
  sg.ldb = ldb;
  const int kc = (int)K;
  const size_t lds = (size_t)sk_lds_rows(1, M) * (kc + 8) * sizeof(bf16);
  if (M <= GV_MAX_GATED && lds <= 65536) {
    gv_launch<true>(sa, dim3((unsigned)(F / 8), 1), s, M, sg, K, kc, (float*)C, ldc);
    return check_launch("gemv_gated");
  }
  static bool lds_set = false;
  if (!lds_set) {
    (void)hipFuncSetAttribute((const void*)k_gemm_skinny<1, SKA_BF16, 4, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              96 * 1024);
    lds_set = true;
  }
  hipLaunchKernelGGL((k_gemm_skinny<1, SKA_BF16, 4, true>), dim3((unsigned)(F / 16), 1), dim3(256), lds, s, sa, M, sg, K,
                     kc, (float*)C, ldc);
  return check_launch("gemm_skinny_gated");
}

// M <= 64 rows, bf16, K % 128 == 0, every B segment a multiple of 64 rows. Returns false if not taken.
bool gemm_skinny(const GemmArgs& a, const void* const* segs, const int64_t* seg_rows, int nseg, void* ws,
                 size_t ws_bytes, hipStream_t s, g4_status* st) {
  if (!skinny_ok(a.M, a.K, segs, seg_rows, nseg, a.ldb) || a.lda % 8 || ((uintptr_t)a.A & 15)) return false;
  int64_t Nt = 0;
  for (int i = 0; i < nseg; ++i) Nt += seg_rows[i];
  if (!ws || ws_bytes < gemm_skinny_ws(a.M, Nt, a.K)) return false;
  SkA sa{};
  sa.a = a.A; sa.lda = a.lda; sa.kind = SKA_BF16;
  float* part = (float*)ws;
  int splits = 0;
  if ((*st = gemm_skinny_part(sa, a.M, a.K, segs, seg_rows, nseg, a.ldb, part, ws_bytes, &splits, s)) != G4_OK)
    return true;
  *st = gemm_skinny_finish(a, part, splits, Nt, s);
  return true;
}

}  // namespace g4
