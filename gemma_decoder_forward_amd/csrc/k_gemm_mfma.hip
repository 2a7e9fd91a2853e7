// bf16 GEMM on the CDNA4 matrix cores: C = A B^T, A [M,K] and B [N,K] row-major (K contiguous),
// float32 accumulation with v_mfma_f32_32x32x16_bf16.
//
// Block: 256 threads = 4 waves in a 2x2 grid; a wave owns a (BM/2) x (BN/2) sub-tile made of 32x32
// MFMA blocks. K advances in steps of 64. Both operand tiles live in LDS as rows of 64 bf16 padded to
// 72 (144-byte stride: the 16-byte fragment reads of consecutive rows land on distinct banks), double
// buffered; the next K step is fetched into registers while the current one is multiplied.
//
// MFMA operand layout (32x32x16 bf16): lane l supplies row (l % 32) and the 8 consecutive k values
// starting at 8 * (l / 32), for A and for B alike (B is stored [N, K], so its rows are the output
// columns). Accumulator register j of lane l holds C[8*(j/4) + 4*(l/32) + j%4][l % 32].
//
// Epilogues: float32 or bf16 store, split-K float32 slices, the gelu-tanh gated product of two weight
// matrices (gate and up rows interleaved in 32-row blocks of the B tile, so a lane holds matching gate
// and up accumulators), and gelu_tanh(acc) * aux.
#include "g4_internal.h"

namespace g4 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int MF_BK = 64;
constexpr int MF_LDK = MF_BK + 8;  // padded LDS row, in bf16 elements

// Linear block id -> (tile_m, tile_n). Blocks are dispatched round-robin over the 8 XCDs; renumber so
// each XCD walks a contiguous range, then walk that range in groups of 8 tile rows so neighbouring
// blocks on one XCD share A rows and B rows in its L2.
__device__ __forceinline__ void tile_of(int bid, int tm, int tn, int& im, int& in_) {
  const int total = tm * tn;
  int id = bid;
  if ((total & 7) == 0) id = (bid & 7) * (total >> 3) + (bid >> 3);
  constexpr int G = 8;
  const int group = id / (G * tn);
  const int first = group * G;
  const int gm = (tm - first) < G ? (tm - first) : G;
  const int r = id - group * G * tn;
  im = first + r % gm;
  in_ = r / gm;
}

template <int BM, int BN, int EPI, bool CF32>
__global__ __launch_bounds__(256, 1) void k_gemm_mfma(GemmArgs a, int tiles_m, int tiles_n) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int ACH = BM * 8 / 256;  // 16-byte chunks of the A tile per thread
  constexpr int BCH = BN * 8 / 256;
  static_assert(EPI != EPI_GEGLU || (FN % 2) == 0, "gate/up pairs must sit in one wave");
  __shared__ __attribute__((aligned(16))) bf16 lds[2][(BM + BN) * MF_LDK];

  int im, in_;
  tile_of(blockIdx.x, tiles_m, tiles_n, im, in_);
  const int64_t m0 = (int64_t)im * BM;
  // output columns of this tile (GEGLU: BN B rows make BN/2 output columns)
  const int64_t n0 = (int64_t)in_ * (EPI == EPI_GEGLU ? BN / 2 : BN);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // split-K range
  const int64_t kper = ((a.K + a.splits - 1) / a.splits + MF_BK - 1) / MF_BK * MF_BK;
  const int64_t kb = (int64_t)blockIdx.z * kper;
  int64_t ke = kb + kper;
  if (ke > a.K) ke = a.K;
  const int nk = ke > kb ? (int)((ke - kb) / MF_BK) : 0;

  // Loader: thread t moves 16-byte chunk (t % 8) of tile rows t/8 + 32j, j = 0, 1, ... For the gated
  // product, B tile rows 32j..32j+31 come from the gate matrix (j even) or the up matrix (j odd).
  const int lrow = tid >> 3, lc8 = (tid & 7) * 8;
  const bf16* abase = (const bf16*)a.A + (m0 + lrow) * a.lda + kb + lc8;
  uint32_t amask = 0;
#pragma unroll
  for (int j = 0; j < ACH; ++j) amask |= (m0 + lrow + 32 * j < a.M ? 1u : 0u) << j;
  const int64_t astep = 32 * a.lda;
  const bf16* bbase;
  const bf16* bbase2;
  if (EPI == EPI_GEGLU) {
    bbase = (const bf16*)a.B + (n0 + lrow) * a.ldb + kb + lc8;
    bbase2 = (const bf16*)a.B2 + (n0 + lrow) * a.ldb + kb + lc8;
  } else {
    bbase = (const bf16*)a.B + (n0 + lrow) * a.ldb + kb + lc8;
    bbase2 = bbase;
  }
  const int64_t bstep = 32 * a.ldb;
  const int ldst = lrow * MF_LDK + lc8;
  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra[ACH], rb[BCH];
  auto gload = [&](int kt) {
    const int64_t off = (int64_t)kt * MF_BK;
#pragma unroll
    for (int j = 0; j < ACH; ++j)
      ra[j] = ((amask >> j) & 1) ? *(const uint4*)(abase + j * astep + off) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < BCH; ++j) {
      if (EPI == EPI_GEGLU) rb[j] = *(const uint4*)(((j & 1) ? bbase2 : bbase) + (j >> 1) * bstep + off);
      else rb[j] = *(const uint4*)(bbase + j * bstep + off);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < ACH; ++j) *(uint4*)&lds[buf][ldst + j * 32 * MF_LDK] = ra[j];
#pragma unroll
    for (int j = 0; j < BCH; ++j) *(uint4*)&lds[buf][ldst + (BM + j * 32) * MF_LDK] = rb[j];
  };

  const int frow = lane & 31, fk = (lane >> 5) * 8;
  if (nk > 0) {
    gload(0);
    lstore(0);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const bf16* la = &lds[cur][(wm * WM + frow) * MF_LDK + fk];
    const bf16* lb = &lds[cur][(BM + wn * WN + frow) * MF_LDK + fk];
#pragma unroll
    for (int ks = 0; ks < MF_BK / 16; ++ks) {
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *(const bf16x8_t*)(la + i * 32 * MF_LDK + ks * 16);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = *(const bf16x8_t*)(lb + j * 32 * MF_LDK + ks * 16);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue
  const int ecol = lane & 31, erow = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = m0 + wm * WM + i * 32 + (r >> 2) * 8 + erow + (r & 3);
      if (m >= a.M) continue;
      if (EPI == EPI_GEGLU) {
#pragma unroll
        for (int p = 0; p < FN / 2; ++p) {
          const int64_t n = n0 + (wn * (FN / 2) + p) * 32 + ecol;
          const float g = acc[i][2 * p][r], u = acc[i][2 * p + 1][r];
          ((bf16*)a.C)[m * a.ldc + n] = f2bf(gelu_tanh(g) * u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t n = n0 + wn * WN + j * 32 + ecol;
          const float v = acc[i][j][r];
          if (EPI == EPI_GELU_MUL) {
            ((bf16*)a.C)[m * a.ldc + n] = f2bf(gelu_tanh(v) * a.aux[m * a.aux_ld + n]);
          } else if (CF32) {
            ((float*)a.C)[(int64_t)blockIdx.z * a.split_stride + m * a.ldc + n] = v;
          } else {
            ((bf16*)a.C)[m * a.ldc + n] = f2bf(v);
          }
        }
      }
    }
  }
}

// Shapes the MFMA kernel takes: bf16, K a multiple of 64, output columns a multiple of the tile,
// 16-byte aligned rows.
static bool mfma_ok(const GemmArgs& a, int BN) {
  const int ncols = a.epi == EPI_GEGLU ? BN / 2 : BN;
  if (a.K % MF_BK || a.N % ncols) return false;
  if ((a.lda | a.ldb) & 7) return false;
  if (((uintptr_t)a.A | (uintptr_t)a.B | (uintptr_t)(a.B2 ? a.B2 : a.B)) & 15) return false;
  return true;
}

template <int BM, int BN>
static g4_status launch_mfma(const GemmArgs& a, hipStream_t s) {
  const int ncols = a.epi == EPI_GEGLU ? BN / 2 : BN;
  const int tm = (int)((a.M + BM - 1) / BM), tn = (int)(a.N / ncols);
  dim3 g((unsigned)(tm * tn), 1, (unsigned)a.splits);
  if (a.epi == EPI_GEGLU) hipLaunchKernelGGL((k_gemm_mfma<BM, BN, EPI_GEGLU, false>), g, dim3(256), 0, s, a, tm, tn);
  else if (a.epi == EPI_GELU_MUL) hipLaunchKernelGGL((k_gemm_mfma<BM, BN, EPI_GELU_MUL, false>), g, dim3(256), 0, s, a, tm, tn);
  else if (a.c_dtype == G4_F32) hipLaunchKernelGGL((k_gemm_mfma<BM, BN, EPI_STORE, true>), g, dim3(256), 0, s, a, tm, tn);
  else hipLaunchKernelGGL((k_gemm_mfma<BM, BN, EPI_STORE, false>), g, dim3(256), 0, s, a, tm, tn);
  return check_launch("gemm_mfma");
}

// Picks a tile that gives enough blocks for 256 CUs; false if the shape does not suit the MFMA path.
bool gemm_mfma(const GemmArgs& a, hipStream_t s, g4_status* st) {
  const int64_t tiles256 = ((a.M + 255) / 256) * (a.N / (a.epi == EPI_GEGLU ? 128 : 256)) * a.splits;
  if (mfma_ok(a, 256) && tiles256 >= 256) {
    *st = launch_mfma<256, 256>(a, s);
    return true;
  }
  if (mfma_ok(a, 128)) {
    *st = launch_mfma<128, 128>(a, s);
    return true;
  }
  return false;
}

}  // namespace g4
