// bf16 GEMM on the CDNA4 matrix cores: C = A B^T, A [M,K] and B [N,K] row-major (K contiguous),
// float32 accumulation with v_mfma_f32_32x32x16_bf16.
//
// Block: 256 threads = 4 waves in a 2x2 grid; a wave owns a (BM/2) x (BN/2) sub-tile made of 32x32
// MFMA blocks. K advances in steps of 32 (one 64-byte row segment per tile row, two MFMA k-slices).
//
// Operand staging: buffer loads write straight into LDS (buffer_load_dwordx4 ... lds), so no registers
// hold staged data and the accumulators keep the whole accumulation-register file. One wave load
// instruction fills 1 KB = 16 tile rows; inside a row the 4 16-byte chunks are XOR-permuted with
// ((row >> 1) ^ (row >> 2)) & 3, which keeps the 16-byte fragment reads free of bank conflicts. NS stages in a ring: the loads of step k + NS are issued as soon as every wave has finished
// reading step k's stage, so global loads have NS - 1 steps of MFMA work to land in.
//
// Latency hiding without a second wave per SIMD (a 128x128 wave tile needs the whole accumulation
// file): the operand fragments of the next k-slice are read from LDS while the MFMAs of the current
// one run (two register sets, A/B ping-pong), and the block meets once per step, between the two
// k-slices, where the waits for the next stage and for the freed stage coincide.
//
// Buffer descriptors start at the tile's first row, so rows past the matrix read as zero (ragged M)
// and every per-row offset fits 32 bits; the per-load row step and the K step ride in the scalar offset.
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

constexpr int MF_BK = 32;  // K per step
constexpr int MF_NS = 4;   // LDS stages

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

// chunk permutation of a 64-byte LDS row: the fragment reads of any 8 consecutive rows (one 128-byte
// bank line per cycle) and of any 16 consecutive rows land on distinct 16-byte bank groups
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

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
  constexpr int NMF = FM * FN;                // MFMAs per wave per k-slice
  constexpr int NRD = FM + FN;                // fragment reads per wave per k-slice
  constexpr int AJ = BM / 64, BJ = BN / 64;  // 1 KB load instructions per wave per K step
  constexpr int LG = AJ + BJ;                 // load instructions per wave per stage
  constexpr int ASZ = BM * MF_BK, STAGE = (BM + BN) * MF_BK;  // in bf16 elements
  static_assert(EPI != EPI_GEGLU || (FN % 2) == 0, "gate/up pairs must sit in one wave");
  static_assert(NRD <= NMF && LG <= NMF, "every read and load rides behind an MFMA");
  static_assert((MF_NS - 1) * LG <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) bf16 lds[MF_NS * STAGE];

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

  // Loader geometry. Instruction j of wave w fills LDS rows 16(w + 4j) .. +15; lane i loads row
  // 16(w + 4j) + i/4 into LDS chunk i%4, which holds global chunk (i%4) ^ swz(row); swz(row) depends
  // on the lane only. GEGLU: B tile row block b (32 rows) holds gate rows (b even) or up rows (b odd)
  // 32(b/2) .. +31, so wave w's instructions all read gate (w < 2) or up (w >= 2) rows 32j + 16(w&1) + i/4.
  const int lr = lane >> 2, lc = (lane & 3) ^ swz(lane >> 2);
  const rsrc_t ra = make_rsrc((const bf16*)a.A + m0 * a.lda + kb, (a.M - m0) * a.lda * 2 - kb * 2);
  const bf16* bsrc = (EPI == EPI_GEGLU && (wave >> 1)) ? (const bf16*)a.B2 : (const bf16*)a.B;
  const rsrc_t rb = make_rsrc(bsrc + n0 * a.ldb + kb, (a.N - n0) * a.ldb * 2 - kb * 2);
  const uint32_t avoff = (uint32_t)(((int64_t)(16 * wave + lr) * a.lda + 8 * lc) * 2);
  const int brow0 = EPI == EPI_GEGLU ? 16 * (wave & 1) : 16 * wave;
  const uint32_t bvoff = (uint32_t)(((int64_t)(brow0 + lr) * a.ldb + 8 * lc) * 2);
  const uint32_t astep = (uint32_t)(64 * a.lda * 2);
  const uint32_t bstep = (uint32_t)((EPI == EPI_GEGLU ? 32 : 64) * a.ldb * 2);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)lds;
  // Load instruction q (A rows first, then B rows) of step kt. A step past the range (the ring keeps
  // issuing one stage per step) gets a scalar offset beyond the buffer, which the range check turns
  // into zeros without moving data, so every step keeps the same number of loads in flight.
  auto dma = [&](int kt, int q) {
    const uint32_t koff = kt < nk ? (uint32_t)kt * MF_BK * 2 : 0x80000000u;
    const uint32_t lbase = lds0 + (uint32_t)(kt % MF_NS) * STAGE * 2;
    if (q < AJ) lds_dma16(ra, avoff, q * astep + koff, lbase + (wave + 4 * q) * 1024);
    else lds_dma16(rb, bvoff, (q - AJ) * bstep + koff, lbase + ASZ * 2 + (wave + 4 * (q - AJ)) * 1024);
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
  int aoff[2][FM], boff[2][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = wm * WM + 32 * i + frow;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) aoff[ks][i] = row * MF_BK + (((2 * ks + fh) ^ swz(row)) << 3);
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int row = wn * WN + 32 * j + frow;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) boff[ks][j] = ASZ + row * MF_BK + (((2 * ks + fh) ^ swz(row)) << 3);
  }

  // Two fragment sets. Read q of a k-slice comes in the order the MFMAs consume them: A0, B0..B(FN-1),
  // A1..A(FM-1); MFMA q multiplies A fragment q / FN with B fragment q % FN. Operands are swapped
  // (B first) so that a lane's accumulator registers run along output columns.
  bf16x8_t fa[2][FM], fb[2][FN];
  auto rd = [&](int set, int ks, const bf16* st, int q) {
    if (q == 0) fa[set][0] = *(const bf16x8_t*)(st + aoff[ks][0]);
    else if (q <= FN) fb[set][q - 1] = *(const bf16x8_t*)(st + boff[ks][q - 1]);
    else fa[set][q - FN] = *(const bf16x8_t*)(st + aoff[ks][q - FN]);
  };
  auto mf = [&](int set, int q) {
    const int i = q / FN, j = q % FN;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0);
  };

  if (nk > 0) {
#pragma unroll
    for (int kt = 0; kt < MF_NS; ++kt)
#pragma unroll
      for (int q = 0; q < LG; ++q) dma(kt, q);
    G4_WAIT_VMCNT((MF_NS - 1) * LG);  // step 0 landed
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NRD; ++q) rd(0, 0, lds, q);
    for (int kt = 0; kt < nk; ++kt) {
      const bf16* st = lds + (kt % MF_NS) * STAGE;
      const bf16* st1 = lds + ((kt + 1) % MF_NS) * STAGE;
      // k-slice 0: MFMAs on set 0, with the reads of slice 1 into set 1 riding behind them
#pragma unroll
      for (int q = 0; q < NMF; ++q) {
        mf(0, q);
        if (q < NRD) rd(1, 1, st, q);
        __builtin_amdgcn_sched_barrier(0);
      }
      // step kt + 1 landed in every wave, and every wave is done reading step kt's stage
      G4_WAIT_VMCNT((MF_NS - 2) * LG);
      __syncthreads();
      // k-slice 1: MFMAs on set 1; behind them the reads of the next step's slice 0, then the loads
      // that refill the stage just consumed with step kt + NS
#pragma unroll
      for (int q = 0; q < NMF; ++q) {
        mf(1, q);
        if (q < NRD) rd(0, 0, st1, q);
        if (q >= NMF - LG) dma(kt + MF_NS, q - (NMF - LG));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    G4_WAIT_VMCNT(0);  // the zero-filling loads past the range land before the block's LDS is released
  }

  // epilogue: lane l holds, for 32x32 block (i, j) and register group g, C[m][n .. n+3] with
  // m = 32 i + l % 32 and n = 32 j + 8 g + 4 (l / 32) (wave-relative)
  const int em = lane & 31, en = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + wm * WM + i * 32 + em;
    if (m >= a.M) continue;
    if (EPI == EPI_GEGLU) {
#pragma unroll
      for (int p = 0; p < FN / 2; ++p) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = n0 + (wn * (FN / 2) + p) * 32 + 8 * g + en;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = gelu_tanh(acc[i][2 * p][4 * g + e]) * acc[i][2 * p + 1][4 * g + e];
          *(uint2*)((bf16*)a.C + m * a.ldc + n) = pack_bf16x4(v);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = n0 + wn * WN + j * 32 + 8 * g + en;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
          if (EPI == EPI_GELU_MUL) {
            const float4 x = *(const float4*)(a.aux + m * a.aux_ld + n);
            v[0] = gelu_tanh(v[0]) * x.x; v[1] = gelu_tanh(v[1]) * x.y;
            v[2] = gelu_tanh(v[2]) * x.z; v[3] = gelu_tanh(v[3]) * x.w;
            *(uint2*)((bf16*)a.C + m * a.ldc + n) = pack_bf16x4(v);
          } else if (CF32) {
            *(float4*)((float*)a.C + (int64_t)blockIdx.z * a.split_stride + m * a.ldc + n) =
                make_float4(v[0], v[1], v[2], v[3]);
          } else {
            *(uint2*)((bf16*)a.C + m * a.ldc + n) = pack_bf16x4(v);
          }
        }
      }
    }
  }
}

// Shapes the MFMA kernel takes: bf16, K a multiple of 32, output columns a multiple of the tile,
// 16-byte aligned rows, operands small enough for 32-bit buffer offsets, and outputs (and the
// GELU_MUL factor) whose rows take 4-column vector stores.
static bool mfma_ok(const GemmArgs& a, int BN) {
  const int ncols = a.epi == EPI_GEGLU ? BN / 2 : BN;
  if (a.K % MF_BK || a.N % ncols) return false;
  if ((a.lda | a.ldb) & 7) return false;
  if (((uintptr_t)a.A | (uintptr_t)a.B | (uintptr_t)(a.B2 ? a.B2 : a.B)) & 15) return false;
  if (a.M * a.lda * 2 > 0x7fffffffLL || a.N * a.ldb * 2 > 0x7fffffffLL) return false;
  const bool f32 = a.epi == EPI_STORE && a.c_dtype == G4_F32;
  if ((a.ldc & 3) || ((uintptr_t)a.C & (f32 ? 15 : 7))) return false;
  if (f32 && a.splits > 1 && (a.split_stride & 3)) return false;
  if (a.epi == EPI_GELU_MUL && ((a.aux_ld & 3) || ((uintptr_t)a.aux & 15))) return false;
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
