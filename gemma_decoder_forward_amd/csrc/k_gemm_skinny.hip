// Weight-streaming GEMM for few token rows (decode: M = batch <= 64): C = A B^T with B the weights.
//
// HBM-bound: every weight byte is read once. A block owns 64 weight rows (one 16-row MFMA block per wave)
// and a K range of kc; the activation slice A[0:M, k-range] is staged once in LDS and shared by the four
// waves. Per 128-k step a lane reads 64 contiguous bytes of its weight row (4 lanes cover 256 bytes of
// a row), the next step's weights are prefetched into registers, and v_mfma_f32_16x16x32_bf16 forms
// the products: lane l supplies row (l % 16) and k values 32*(l/16) + 8t .. +7 for MFMA t of the step,
// for the activations and the weights alike, so both operands see the same k order.
// Blocks over K write float32 partials [split][M][rows]; k_gemm_finish sums them and applies the
// epilogue (store, gelu-tanh gate*up, gelu*aux).
//
// B may be the concatenation of up to three matrices (q/k/v projections, or gate then up) so that one
// launch covers them; the output columns follow the concatenation.
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

template <int MB>
__global__ __launch_bounds__(256) void k_gemm_skinny(const bf16* __restrict__ A, int64_t lda, int64_t M, SkSeg sg,
                                                     int64_t K, int kc, float* __restrict__ part, int64_t Nt) {
  extern __shared__ __attribute__((aligned(16))) bf16 As[];
  const int ald = kc + 8;  // LDS row stride (bf16); (kc + 8) * 2 bytes = 4 (mod 64) words -> conflict-free rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t k0 = (int64_t)blockIdx.y * kc;
  const int kn = (int)((K - k0) < kc ? (K - k0) : kc);
  // stage A[0:16*MB, k0:k0+kn] (rows >= M are zero)
  const int cpr = kn / 8;
  for (int idx = tid; idx < 16 * MB * cpr; idx += 256) {
    const int m = idx / cpr, c = idx - m * cpr;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (m < M) v = *(const uint4*)(A + m * lda + k0 + 8 * c);
    *(uint4*)(As + m * ald + 8 * c) = v;
  }
  __syncthreads();

  const int64_t r = (int64_t)blockIdx.x * 64 + wave * 16 + (lane & 15);
  const int q = lane >> 4;
  const bf16* wrow = sk_row(sg, r) + k0 + 32 * q;
  const bf16* arow = As + (lane & 15) * ald + 32 * q;
  f32x4_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  uint4 wcur[4], wnxt[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) wcur[t] = *(const uint4*)(wrow + 8 * t);
  for (int kk = 0; kk < kn; kk += 128) {
    const bool more = kk + 128 < kn;
#pragma unroll
    for (int t = 0; t < 4; ++t) wnxt[t] = more ? *(const uint4*)(wrow + kk + 128 + 8 * t) : wcur[t];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x8_t bw = *(const bf16x8_t*)&wcur[t];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8_t af = *(const bf16x8_t*)(arow + mb * 16 * ald + kk + 8 * t);
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bw, acc[mb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) wcur[t] = wnxt[t];
  }
  // C[m][r]: lane holds column (lane % 16) and rows 4*(lane/16) + i of each 16-row block
  float* pb = part + (int64_t)blockIdx.y * M * Nt;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = mb * 16 + 4 * q + i;
      if (m < M) pb[m * Nt + r] = acc[mb][i];
    }
}

// Sums the split partials and applies the epilogue. GEGLU: part columns [0, N) are gate, [N, 2N) up.
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
  } else if (CF32) {
    ((float*)a.C)[m * a.ldc + n] = v;
  } else {
    ((bf16*)a.C)[m * a.ldc + n] = f2bf(v);
  }
}

static int sk_kc(int mb, int64_t K, int64_t rowblocks) {
  int kc = mb >= 4 ? 1024 : 2048;                    // LDS: 16*mb rows x (kc + 8) bf16 <= ~132 KB
  while (kc > 128 && rowblocks * ((K + kc - 1) / kc) < 512) kc >>= 1;  // enough blocks for 256 CUs
  if (kc > K) kc = (int)((K + 127) / 128 * 128);
  return kc;
}

size_t gemm_skinny_ws(int64_t M, int64_t Nt, int64_t K) {
  const int mb = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  const int kc = sk_kc(mb, K, Nt / 64);
  return (size_t)((K + kc - 1) / kc) * M * Nt * sizeof(float);
}

// M <= 64 rows, bf16, K % 128 == 0, every B segment a multiple of 64 rows. Returns false if not taken.
bool gemm_skinny(const GemmArgs& a, const void* const* segs, const int64_t* seg_rows, int nseg, void* ws,
                 size_t ws_bytes, hipStream_t s, g4_status* st) {
  if (a.M > 64 || a.M <= 0 || a.K % 128 || a.lda % 8 || a.ldb % 8) return false;
  SkSeg sg{};
  int64_t Nt = 0;
  for (int i = 0; i < 3; ++i) {
    if (i < nseg) {
      if (seg_rows[i] % 64 || ((uintptr_t)segs[i] & 15)) return false;
      Nt += seg_rows[i];
      sg.b[i] = (const bf16*)segs[i];
    } else {
      sg.b[i] = sg.b[nseg - 1];
    }
    sg.end[i] = Nt;
  }
  sg.ldb = a.ldb;
  if (((uintptr_t)a.A & 15)) return false;
  const int mb = a.M <= 16 ? 1 : (a.M <= 32 ? 2 : 4);
  const int kc = sk_kc(mb, a.K, Nt / 64);
  const int splits = (int)((a.K + kc - 1) / kc);
  const size_t need = (size_t)splits * a.M * Nt * sizeof(float);
  if (!ws || ws_bytes < need) return false;
  dim3 g((unsigned)(Nt / 64), (unsigned)splits);
  const size_t lds = (size_t)16 * mb * (kc + 8) * sizeof(bf16);
  static bool lds_set = false;  // allow > 64 KB of dynamic LDS (gfx950 has 160 KB per CU)
  if (!lds_set) {
    (void)hipFuncSetAttribute((const void*)k_gemm_skinny<1>, hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024);
    (void)hipFuncSetAttribute((const void*)k_gemm_skinny<2>, hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024);
    (void)hipFuncSetAttribute((const void*)k_gemm_skinny<4>, hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024);
    lds_set = true;
  }
  float* part = (float*)ws;
  if (mb == 1) hipLaunchKernelGGL(k_gemm_skinny<1>, g, dim3(256), lds, s, (const bf16*)a.A, a.lda, a.M, sg, a.K, kc, part, Nt);
  else if (mb == 2) hipLaunchKernelGGL(k_gemm_skinny<2>, g, dim3(256), lds, s, (const bf16*)a.A, a.lda, a.M, sg, a.K, kc, part, Nt);
  else hipLaunchKernelGGL(k_gemm_skinny<4>, g, dim3(256), lds, s, (const bf16*)a.A, a.lda, a.M, sg, a.K, kc, part, Nt);
  if ((*st = check_launch("gemm_skinny")) != G4_OK) return true;
  dim3 gf((unsigned)((a.M * a.N + 255) / 256));
  if (a.epi == EPI_GEGLU) hipLaunchKernelGGL((k_gemm_finish<EPI_GEGLU, false>), gf, dim3(256), 0, s, a, part, splits, Nt);
  else if (a.epi == EPI_GELU_MUL) hipLaunchKernelGGL((k_gemm_finish<EPI_GELU_MUL, false>), gf, dim3(256), 0, s, a, part, splits, Nt);
  else if (a.c_dtype == G4_F32) hipLaunchKernelGGL((k_gemm_finish<EPI_STORE, true>), gf, dim3(256), 0, s, a, part, splits, Nt);
  else hipLaunchKernelGGL((k_gemm_finish<EPI_STORE, false>), gf, dim3(256), 0, s, a, part, splits, Nt);
  *st = check_launch("gemm_finish");
  return true;
}

}  // namespace g4
