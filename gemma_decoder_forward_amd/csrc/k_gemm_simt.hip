// Generic tiled GEMM, C = A B^T (A [M,K], B [N,K] row-major), float32 FMA on the vector ALUs.
// Used for float32 models and for shapes the bf16 MFMA kernels do not tile (any M, N, K).
// 64x64 output tile per 256-thread block, 4x4 outputs per thread, K staged through LDS in steps of 16.
#include "g4_internal.h"

namespace g4 {

template <typename T, int EPI>
__global__ __launch_bounds__(256) void k_gemm_simt(GemmArgs a) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  __shared__ float B2s[EPI == EPI_GEGLU ? BK : 1][BN + 4];
  const T* A = (const T*)a.A;
  const T* B = (const T*)a.B;
  const T* B2 = (const T*)a.B2;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  // split-K: slice z handles K range [kb, ke)
  const int64_t kper = ((a.K + a.splits - 1) / a.splits + BK - 1) / BK * BK;
  const int64_t kb = (int64_t)blockIdx.z * kper;
  const int64_t ke = kb + kper < a.K ? kb + kper : a.K;
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {}, acc2[4][4] = {};
  const int lr = tid >> 2, lc = (tid & 3) * 4;  // loader: row 0..63, k offset 0,4,8,12
  for (int64_t k0 = kb; k0 < ke; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t k = k0 + lc + i;
      const int64_t am = m0 + lr, bn = n0 + lr;
      As[lc + i][lr] = (am < a.M && k < ke) ? ldf(A + am * a.lda + k) : 0.f;
      Bs[lc + i][lr] = (bn < a.N && k < ke) ? ldf(B + bn * a.ldb + k) : 0.f;
      if (EPI == EPI_GEGLU) B2s[lc + i][lr] = (bn < a.N && k < ke) ? ldf(B2 + bn * a.ldb + k) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float av[4], bv[4], b2v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = As[kk][ty * 4 + i];
        bv[i] = Bs[kk][tx * 4 + i];
        if (EPI == EPI_GEGLU) b2v[i] = B2s[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
          if (EPI == EPI_GEGLU) acc2[i][j] = fmaf(av[i], b2v[j], acc2[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx * 4 + j;
      if (n >= a.N) continue;
      const float v = acc[i][j];
      if (EPI == EPI_STORE) {
        if (a.c_dtype == G4_F32)
          ((float*)a.C)[(int64_t)blockIdx.z * a.split_stride + m * a.ldc + n] = v;
        else
          stf((T*)a.C + m * a.ldc + n, v);
      } else if (EPI == EPI_GEGLU) {
        stf((T*)a.C + m * a.ldc + n, gelu_tanh(v) * acc2[i][j]);
      } else {
        stf((T*)a.C + m * a.ldc + n, gelu_tanh(v) * a.aux[m * a.aux_ld + n]);
      }
    }
  }
}

g4_status gemm_simt(const GemmArgs& a, int32_t dtype, hipStream_t s) {
  dim3 g((unsigned)((a.N + 63) / 64), (unsigned)((a.M + 63) / 64), (unsigned)a.splits);
#define G4_GS(TT)                                                                          \
  do {                                                                                     \
    if (a.epi == EPI_STORE) hipLaunchKernelGGL((k_gemm_simt<TT, EPI_STORE>), g, dim3(256), 0, s, a); \
    else if (a.epi == EPI_GEGLU) hipLaunchKernelGGL((k_gemm_simt<TT, EPI_GEGLU>), g, dim3(256), 0, s, a); \
    else hipLaunchKernelGGL((k_gemm_simt<TT, EPI_GELU_MUL>), g, dim3(256), 0, s, a);        \
  } while (0)
  if (dtype == G4_BF16) G4_GS(bf16);
  else G4_GS(float);
#undef G4_GS
  return check_launch("gemm_simt");
}

}  // namespace g4
