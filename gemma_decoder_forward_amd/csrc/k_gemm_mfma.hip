// bf16 GEMM on the CDNA4 matrix cores: C = A B^T, A [M,K] and B [N,K] row-major (K contiguous),
// float32 accumulation with v_mfma_f32_32x32x16_bf16.
//
// Block: 256 threads = 4 waves in a 2x2 grid; a wave owns a (BM/2) x (BN/2) sub-tile made of 32x32
// MFMA blocks. K advances in steps of 64 (one 128-byte row segment per tile row).
//
// Operand staging: buffer loads write straight into LDS (buffer_load_dwordx4 ... lds), so no registers
// hold staged data and the accumulators keep the whole accumulation-register file. One wave load
// instruction fills 1 KB = 8 tile rows; inside a row the 8 16-byte chunks are XOR-permuted with
// (row ^ row >> 3) & 7, which puts the 16-byte fragment reads of 8 (or 16) consecutive rows on distinct
// LDS banks. Two stages: the loads of step k+1 are in flight while step k is multiplied. Buffer
// descriptors start at the tile's first row, so rows past the matrix read as zero (ragged M) and every
// per-row offset fits 32 bits; the per-load row step and the K step ride in the scalar offset.
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
typedef __attribute__((address_space(3))) void lds_void;

constexpr int MF_BK = 64;

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

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

typedef __attribute__((ext_vector_type(4))) uint32_t rsrc_t;

// Raw buffer descriptor (gfx9 layout): base address, stride 0, num_records bytes, data format.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint64_t p = (uint64_t)base;
  const uint32_t n = bytes > 0x7fffffff ? 0x7fffffffu : (bytes < 0 ? 0u : (uint32_t)bytes);
  rsrc_t r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)p);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xffffu);
  r.z = __builtin_amdgcn_readfirstlane(n);
  r.w = 0x00020000u;
  return r;
}

// 16 bytes per lane from buffer offset voff + soff straight into LDS at m0 + 16 * lane. Issued through
// inline assembly so the compiler's wait insertion does not treat every later LDS read as dependent
// on it; completion is awaited explicitly with vmcnt before the barrier that precedes the reads.
__device__ __forceinline__ void lds_dma16(const rsrc_t& r, uint32_t voff, uint32_t soff, uint32_t m0) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" : : "v"(voff), "s"(r), "s"(soff), "{m0}"(m0) : "memory");
}

// vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt[3:0] and [15:14]).
#define G4_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

template <int BM, int BN, int EPI, bool CF32>
__global__ __launch_bounds__(256, 1) void k_gemm_mfma(GemmArgs a, int tiles_m, int tiles_n) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int AJ = BM / 32, BJ = BN / 32;  // 1 KB load instructions per wave per K step
  constexpr int ASZ = BM * MF_BK, STAGE = (BM + BN) * MF_BK;  // in bf16 elements
  static_assert(EPI != EPI_GEGLU || (FN % 2) == 0, "gate/up pairs must sit in one wave");
  __shared__ __attribute__((aligned(1024))) bf16 lds[2 * STAGE];

  int im, in_;
  tile_of(blockIdx.x, tiles_m, tiles_n, im, in_);
  im = __builtin_amdgcn_readfirstlane(im);  // block-uniform: keeps the buffer descriptors in SGPRs
  in_ = __builtin_amdgcn_readfirstlane(in_);
  const int64_t m0 = (int64_t)im * BM;
  // output columns of this tile (GEGLU: BN B rows make BN/2 output columns)
  const int64_t n0 = (int64_t)in_ * (EPI == EPI_GEGLU ? BN / 2 : BN);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (feeds the LDS base in M0)
  const int wm = wave >> 1, wn = wave & 1;

  // split-K range
  const int64_t kper = ((a.K + a.splits - 1) / a.splits + MF_BK - 1) / MF_BK * MF_BK;
  const int64_t kb = (int64_t)blockIdx.z * kper;
  int64_t ke = kb + kper;
  if (ke > a.K) ke = a.K;
  const int nk = ke > kb ? (int)((ke - kb) / MF_BK) : 0;

  // Loader geometry. Instruction j of wave w fills LDS rows 8(w + 4j) .. +7; lane i loads row
  // 8(w + 4j) + i/8 into LDS chunk i%8, which holds global chunk (i%8) ^ swz(row). swz depends on j
  // only through its parity (row >> 3 = w + 4j).
  const int lr = lane >> 3, lp = lane & 7;
  const rsrc_t ra =
      make_rsrc((const bf16*)a.A + m0 * a.lda + kb, (a.M - m0) * a.lda * 2 - kb * 2);
  const rsrc_t rb =
      make_rsrc((const bf16*)a.B + n0 * a.ldb + kb, (a.N - n0) * a.ldb * 2 - kb * 2);
  const rsrc_t rb2 =
      EPI == EPI_GEGLU ? make_rsrc((const bf16*)a.B2 + n0 * a.ldb + kb, (a.N - n0) * a.ldb * 2 - kb * 2) : rb;
  uint32_t avoff[2], bvoff[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int row = 8 * (wave + 4 * par) + lr;
    const int c = lp ^ swz(row);
    avoff[par] = (uint32_t)(((int64_t)(8 * wave + lr) * a.lda + 8 * c) * 2);
    bvoff[par] = (uint32_t)(((int64_t)(8 * wave + lr) * a.ldb + 8 * c) * 2);
  }
  const uint32_t arow32 = (uint32_t)(32 * a.lda * 2), brow32 = (uint32_t)(32 * a.ldb * 2);
  auto issue = [&](int kt, bf16* base) {
    const uint32_t koff = (uint32_t)kt * MF_BK * 2;
    const uint32_t lbase = (uint32_t)(uintptr_t)(lds_void*)base;
#pragma unroll
    for (int j = 0; j < AJ; ++j) lds_dma16(ra, avoff[j & 1], j * arow32 + koff, lbase + (wave + 4 * j) * 1024);
#pragma unroll
    for (int j = 0; j < BJ; ++j) {
      const uint32_t dst = lbase + ASZ * 2 + (wave + 4 * j) * 1024;
      if (EPI == EPI_GEGLU)  // B tile rows 32j..32j+31: gate (j even) or up (j odd) rows 32(j/2) + ...
        lds_dma16((j & 1) ? rb2 : rb, bvoff[j & 1], (j >> 1) * brow32 + koff, dst);
      else
        lds_dma16(rb, bvoff[j & 1], j * brow32 + koff, dst);
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment addresses (elements within a stage): row r, k chunk 2ks + h at chunk (2ks + h) ^ swz(r)
  const int frow = lane & 31, fh = lane >> 5;
  int arow[FM], asw[FM], brow[FN], bsw[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = wm * WM + 32 * i + frow;
    arow[i] = row * MF_BK;
    asw[i] = swz(row);
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int row = wn * WN + 32 * j + frow;
    brow[j] = ASZ + row * MF_BK;
    bsw[j] = swz(row);
  }

  auto compute = [&](const bf16* st) {
#pragma unroll
    for (int ks = 0; ks < MF_BK / 16; ++ks) {
      const int c = 2 * ks + fh;
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *(const bf16x8_t*)(st + arow[i] + ((c ^ asw[i]) << 3));
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = *(const bf16x8_t*)(st + brow[j] + ((c ^ bsw[j]) << 3));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };
  // step kt reads stage kt % 2 while the loads of step kt + 1 fill the other stage
  if (nk > 0) issue(0, lds);
  for (int kt = 0; kt < nk - 1; ++kt) {
    issue(kt + 1, lds + ((kt + 1) & 1) * STAGE);
    G4_WAIT_VMCNT(AJ + BJ);
    __syncthreads();
    compute(lds + (kt & 1) * STAGE);
    __syncthreads();
  }
  if (nk > 0) {
    G4_WAIT_VMCNT(0);
    __syncthreads();
    compute(lds + ((nk - 1) & 1) * STAGE);
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
// 16-byte aligned rows, and operands small enough for 32-bit buffer offsets.
static bool mfma_ok(const GemmArgs& a, int BN) {
  const int ncols = a.epi == EPI_GEGLU ? BN / 2 : BN;
  if (a.K % MF_BK || a.N % ncols) return false;
  if ((a.lda | a.ldb) & 7) return false;
  if (((uintptr_t)a.A | (uintptr_t)a.B | (uintptr_t)(a.B2 ? a.B2 : a.B)) & 15) return false;
  if (a.M * a.lda * 2 > 0x7fffffffLL || a.N * a.ldb * 2 > 0x7fffffffLL) return false;
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
  if (mfma_ok(a, 256) && tiles256 >= 192) {
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
