// bf16 GEMM on the CDNA4 matrix cores: C = A B^T, A [M,K] and B [N,K] row-major (K contiguous),
// float32 accumulation with v_mfma_f32_32x32x16_bf16.
//
// Block: NW waves in a WGM x (NW/WGM) grid (by default (NW/2) x 2); a wave owns a (BM/WGM) x
// (BN/(NW/WGM)) sub-tile made of 32x32 MFMA blocks. The 256x256 tile runs 8 waves (two per SIMD,
// 64x128 each), so one wave's MFMAs cover the other's waits; the 128x128 tile runs 4. The 64-row tiles
// serve 17 to 64 token rows (batched decode), where the weight stream, not the MFMAs, sets the pace.
// K advances in steps of BK (one BK*2-byte row segment per tile row, BK/16 MFMA k-slices).
//
// Operand staging: buffer loads write straight into LDS (buffer_load_dwordx4 ... lds), so no registers
// hold staged data. One wave load instruction fills 1 KB of a stage: 1024 / (2 BK) tile rows. Global
// reads move through the vector L1, which can keep only a bounded number of line requests in flight
// per CU; BK = 64 makes every request a whole 128-byte line, twice the bytes per request of BK = 32,
// and that doubles what the L1 can pull from L2 per unit of latency. Inside a row the 16-byte chunks
// are XOR-permuted so that the fragment reads of any 8 (and any 16) consecutive rows fall on distinct
// bank groups. NS stages form a ring: the loads for step k + NS are issued as soon as every wave has
// finished reading step k's stage.
//
// Schedule: two fragment register sets alternate between k-slices; the reads of the next slice and
// the global loads ride between the MFMAs of the current one. The block meets once per step, before
// the last k-slice, where the wait for the next stage and the release of the current one coincide.
// Loads of steps past the K range use a scalar offset beyond the buffer; the range check turns them
// into zeros without memory traffic, so every step keeps the same loads in flight.
//
// Buffer descriptors start at the tile's first row, so rows past the matrix read as zero (ragged M)
// and every per-row offset fits 32 bits.
//
// MFMA operand layout (32x32x16 bf16): lane l supplies row (l % 32) and the 8 consecutive k values
// starting at 8 * (l / 32), for A and for B alike (B is stored [N, K], so its rows are the output
// columns). B goes in as the first operand, so register r of lane l holds C[m][n] with m = l % 32 and
// n = 8 (r / 4) + 4 (l / 32) + r % 4: four consecutive output columns per register group.
//
// Epilogues: float32 or bf16 store, split-K float32 slices, the gelu-tanh gated product of two weight
// matrices, and gelu_tanh(acc) * aux. Gated product: gate and up rows alternate in blocks of RPI rows
// (one load instruction's rows: 8 for BK = 64, 16 for BK = 32) down the B tile. A 32-column MFMA block
// then holds 16 gate and 16 up columns, and by the register layout above the up partner of gate
// register r is register r + RPI/2 of the same lane, so every block finishes its own 16 outputs.
#include "g4_internal.h"

namespace g4 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((address_space(3))) void lds_void;

#ifndef G4_GEMM_BK
#define G4_GEMM_BK 64
#endif
#ifndef G4_GEMM_NS
#define G4_GEMM_NS 2
#endif
#ifndef G4_GEMM_NW
#define G4_GEMM_NW 8
#endif
constexpr int MF_KMIN = 64;  // K granularity the MFMA path accepts (every configuration's BK divides it)

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

// Chunk permutation of an LDS row of BK bf16 (BK/8 chunks of 16 bytes). 128-byte rows: row ^ (row >> 3)
// permutes the 8 chunks of 8 consecutive rows, and pairs of 8-row groups differ in row parity.
// 64-byte rows: ((row >> 1) ^ (row >> 2)) covers the 4 chunks twice over 8 rows, once per row parity.
template <int BK>
__device__ __forceinline__ int swz(int row) {
  return BK == 64 ? (row ^ (row >> 3)) & 7 : ((row >> 1) ^ (row >> 2)) & 3;
}

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
// The descriptor, scalar offset and LDS base are wave-uniform by construction; readfirstlane states it
// to the compiler (free for values already in scalar registers).
__device__ __forceinline__ void lds_dma16(const rsrc_t& r, uint32_t voff, uint32_t soff, uint32_t m0) {
  rsrc_t u;
  u.x = __builtin_amdgcn_readfirstlane(r.x);
  u.y = __builtin_amdgcn_readfirstlane(r.y);
  u.z = __builtin_amdgcn_readfirstlane(r.z);
  u.w = __builtin_amdgcn_readfirstlane(r.w);
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(u), "s"(__builtin_amdgcn_readfirstlane(soff)), "{m0}"(__builtin_amdgcn_readfirstlane(m0))
               : "memory");
}

// vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt[3:0] and [15:14]).
#define G4_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

// SEGB: every B load group (RPI rows) gets its own descriptor at its first row, so a tile may straddle
// the boundary between two stacked B matrices (segments a multiple of RPI rows long).
template <int BM, int BN, int NW, int BK, int NS, int EPI, bool CF32, bool SEGB = false, int WGM = NW / 2>
__global__ __launch_bounds__(NW * 64, 1) void k_gemm_mfma(GemmArgs a, int tiles_m, int tiles_n) {
  constexpr int WGN = NW / WGM;                  // waves in a WGM x WGN grid
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int NMF = FM * FN;                  // MFMAs per wave per k-slice
  constexpr int NRD = FM + FN;                  // fragment reads per wave per k-slice
  constexpr int NQ = NMF > NRD ? NMF : NRD;     // issue slots per k-slice (reads past the MFMAs follow them)
  constexpr int KS = BK / 16;                   // k-slices per step
  constexpr int CPR = BK / 8, RPI = 64 / CPR;   // 16-byte chunks per LDS row, rows per load instruction
  constexpr int AJ = BM / (RPI * NW), BJ = BN / (RPI * NW);  // load instructions per wave per step
  constexpr int LG = AJ + BJ;
  constexpr int ASZ = BM * BK, STAGE = (BM + BN) * BK;  // in bf16 elements
  static_assert(EPI != EPI_GEGLU || RPI == 8 || RPI == 16, "gate/up blocks of one load instruction's rows");
  static_assert((NW == 4 || NW == 8) && AJ * RPI * NW == BM && BJ * RPI * NW == BN, "loader covers the tile");
  static_assert(KS % 2 == 0 && MF_KMIN % BK == 0, "k-slices alternate two register sets");
  static_assert(WGM * WGN == NW && FM >= 1 && FN >= 1 && WM == 32 * FM && WN == 32 * FN, "wave grid");
  static_assert(!SEGB || EPI == EPI_STORE, "segmented B rows: plain store epilogue");
  static_assert((NS - 1) * LG <= 63 && NS >= 2, "vmcnt range");
  static_assert(NS * STAGE * 2 <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) bf16 lds[NS * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (feeds the LDS base in M0)
  const int wm = wave / WGN, wn = wave % WGN;
  const int per_split = tiles_m * tiles_n, total = per_split * a.splits;
  const int64_t kper = ((a.K + a.splits - 1) / a.splits + BK - 1) / BK * BK;  // split-K range length

  // A tile's place and operands. Tile t: split z = t / (tiles_m tiles_n), then tile_of within the split.
  struct Tile {
    int64_t m0, n0;
    int z, nk;
    rsrc_t ra, rg, ru;
    rsrc_t rq[SEGB ? BJ : 1];  // SEGB: B load group q's rows
  };
  auto tile_at = [&](int t) {
    Tile c;
    c.nk = 0;
    c.m0 = c.n0 = 0;
    c.z = 0;
    if (t < total) {
      c.z = t / per_split;
      int im, in_;
      tile_of(t - c.z * per_split, tiles_m, tiles_n, im, in_);
      c.m0 = (int64_t)im * BM;
      c.n0 = (int64_t)in_ * (EPI == EPI_GEGLU ? BN / 2 : BN);  // GEGLU: BN B rows make BN/2 outputs
      const int64_t kb = (int64_t)c.z * kper;
      int64_t ke = kb + kper;
      if (ke > a.K) ke = a.K;
      c.nk = ke > kb ? (int)((ke - kb) / BK) : 0;
    }
    const int64_t kb = (int64_t)c.z * kper;
    c.ra = make_rsrc((const bf16*)a.A + c.m0 * a.lda + kb, (a.M - c.m0) * a.lda * 2 - kb * 2);
    // B rows: one matrix, or (EPI_STORE) up to three stacked matrices; a tile never straddles two
    const bf16* bbase = (const bf16*)a.B;
    int64_t nloc = c.n0, nrows = a.N;
    if (EPI == EPI_STORE && a.nseg > 1) {
      const int64_t r0 = a.seg_rows[0], r1 = a.seg_rows[1];
      const int sg = c.n0 < r0 ? 0 : (c.n0 < r0 + r1 ? 1 : 2);
      bbase = (const bf16*)(sg == 0 ? a.segB[0] : (sg == 1 ? a.segB[1] : a.segB[2]));
      nloc = c.n0 - (sg == 0 ? 0 : (sg == 1 ? r0 : r0 + r1));
      nrows = sg == 0 ? r0 : (sg == 1 ? r1 : a.seg_rows[2]);
    }
    c.rg = make_rsrc(bbase + nloc * a.ldb + kb, (nrows - nloc) * a.ldb * 2 - kb * 2);
    c.ru = EPI == EPI_GEGLU ? make_rsrc((const bf16*)a.B2 + c.n0 * a.ldb + kb, (a.N - c.n0) * a.ldb * 2 - kb * 2) : c.rg;
    if (SEGB) {
#pragma unroll
      for (int q = 0; q < (SEGB ? BJ : 1); ++q) {
        const int64_t r = c.n0 + RPI * (wave + NW * q);  // the group's first B row (wave-uniform)
        const bf16* base = (const bf16*)a.B;
        int64_t loc = r, len = a.N;
        if (a.nseg > 1) {
          const int64_t r0 = a.seg_rows[0], r1 = a.seg_rows[1];
          const int sg = r < r0 ? 0 : (r < r0 + r1 ? 1 : 2);
          base = (const bf16*)(sg == 0 ? a.segB[0] : (sg == 1 ? a.segB[1] : a.segB[2]));
          loc = r - (sg == 0 ? 0 : (sg == 1 ? r0 : r0 + r1));
          len = sg == 0 ? r0 : (sg == 1 ? r1 : a.seg_rows[2]);
        }
        c.rq[q] = make_rsrc(base + loc * a.ldb + kb, (len - loc) * a.ldb * 2 - kb * 2);
      }
    }
    return c;
  };

  // Loader geometry. Load instruction q covers the RPI LDS rows of group g = wave + NW q (A rows for
  // q < AJ, B rows after): lane i fills LDS row RPI g + i / CPR, chunk i % CPR, from global chunk
  // (i % CPR) ^ swz(row). GEGLU: B group g holds gate rows (g even) or up rows (g odd)
  // RPI (g / 2) + i / CPR of the tile's output columns.
  const int lr = lane / CPR, lcp = lane % CPR;
  uint32_t voff[LG];
  bool use_up[LG];
#pragma unroll
  for (int q = 0; q < LG; ++q) {
    const bool isa = q < AJ;
    const int g = wave + NW * (isa ? q : q - AJ);
    const int row = RPI * g + lr;  // LDS row within the A or B part of the stage
    const int chunk = lcp ^ swz<BK>(row);
    int src = row;
    use_up[q] = false;
    if (!isa && EPI == EPI_GEGLU) {
      use_up[q] = g & 1;
      src = RPI * (g >> 1) + lr;
    }
    if (!isa && SEGB) src = lr;  // relative to the group's own descriptor
    voff[q] = (uint32_t)(((int64_t)src * (isa ? a.lda : a.ldb) + 8 * chunk) * 2);
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)lds;

  // The ring of NS stages runs across this block's tiles: global step G + s is step s of the current
  // tile (s < cur.nk) or step s - cur.nk of the next one, and lives in stage (G + s) % NS. A step that
  // belongs to no tile gets an offset beyond the buffer (zeros, no traffic), so every step keeps the
  // same number of loads in flight. The host runs one tile per block when a tile has fewer than NS
  // steps, so a step never belongs to the tile after next.
  Tile cur = tile_at(blockIdx.x), nxt = tile_at(blockIdx.x + gridDim.x);
  int G = 0;
  auto dma = [&](int s, int q) {
    const bool in_cur = s < cur.nk, in_nxt = !in_cur && s - cur.nk < nxt.nk;
    const int ss = in_cur ? s : s - cur.nk;
    const uint32_t koff = (in_cur || in_nxt) ? (uint32_t)ss * BK * 2 : 0x80000000u;
    const uint32_t lbase = lds0 + (uint32_t)((G + s) % NS) * STAGE * 2;
    // value selects (a reference to one of the two tiles would put them in scratch memory)
    if (q < AJ) {
      lds_dma16(in_nxt ? nxt.ra : cur.ra, voff[q], koff, lbase + (wave + NW * q) * 1024);
    } else if (SEGB) {
      const int qb = SEGB ? q - AJ : 0;
      lds_dma16(in_nxt ? nxt.rq[qb] : cur.rq[qb], voff[q], koff, lbase + ASZ * 2 + (wave + NW * (q - AJ)) * 1024);
    } else {
      const rsrc_t rc = use_up[q] ? (in_nxt ? nxt.ru : cur.ru) : (in_nxt ? nxt.rg : cur.rg);
      lds_dma16(rc, voff[q], koff, lbase + ASZ * 2 + (wave + NW * (q - AJ)) * 1024);
    }
  };

  // fragment addresses (elements within a stage): row r, k chunk 2ks + h at chunk (2ks + h) ^ swz(r).
  // Row r + 64 has the swizzle of row r (BK = 64 reads row bits 0-5, and bits 3-5 move by 8 mod 8;
  // BK = 32 reads bits 1-3 only), so fragment j sits a constant 32 (j - j % 2) rows after fragment
  // j % 2: two offsets per k-slice stay in registers and the rest fold into the read's immediate.
  const int frow = lane & 31, fh = lane >> 5;
  int aoff[KS][2], boff[KS][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = wm * WM + 32 * i + frow;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) aoff[ks][i] = row * BK + (((2 * ks + fh) ^ swz<BK>(row)) << 3);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = wn * WN + 32 * j + frow;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) boff[ks][j] = ASZ + row * BK + (((2 * ks + fh) ^ swz<BK>(row)) << 3);
  }
  auto aof = [&](int ks, int i) { return aoff[ks][i & 1] + 32 * (i & ~1) * BK; };
  auto bof = [&](int ks, int j) { return boff[ks][j & 1] + 32 * (j & ~1) * BK; };

  // Two fragment sets. Read q of a k-slice comes in the order the MFMAs consume them: A0, B0..B(FN-1),
  // A1..A(FM-1); MFMA q multiplies A fragment q / FN with B fragment q % FN.
  f32x16_t acc[FM][FN];
  bf16x8_t fa[2][FM], fb[2][FN];
  auto rd = [&](int set, int ks, const bf16* st, int q) {
    if (q == 0) fa[set][0] = *(const bf16x8_t*)(st + aof(ks, 0));
    else if (q <= FN) fb[set][q - 1] = *(const bf16x8_t*)(st + bof(ks, q - 1));
    else fa[set][q - FN] = *(const bf16x8_t*)(st + aof(ks, q - FN));
  };
  auto mf = [&](int set, int q) {
    const int i = q / FN, j = q % FN;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0);
  };

  // Epilogue: lane l holds, for 32x32 block (i, j) and register group g, C[m][n .. n+3] with
  // m = 32 i + l % 32 and n = 32 j + 8 g + 4 (l / 32) (wave-relative).
  auto store_tile = [&](int64_t m0, int64_t n0, int z) {
    const int em = lane & 31, en = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t m = m0 + wm * WM + i * 32 + em;
      if (m >= a.M) continue;
      if (EPI == EPI_GEGLU) {
        // block j: columns c = 8 g + en of register group g are gate when (c / RPI) is even; the up
        // partner is group g + RPI / 8; output column n0 + 16 (wn FN + j) + the gate column's rank
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            if (((8 * g) / RPI) & 1) continue;  // an up group
            const int c = 8 * g + en;
            const int64_t n = n0 + 16 * (wn * FN + j) + RPI * (c / (2 * RPI)) + c % RPI;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = gelu_tanh(acc[i][j][4 * g + e]) * acc[i][j][4 * (g + RPI / 8) + e];
            *(uint2*)((bf16*)a.C + m * a.ldc + n) = pack_bf16x4(v);
          }
        }
      } else {
        // GELU_MUL factors, JC column blocks at a time, loaded before the first store of those blocks
        // (which could alias them as far as the compiler knows, and would otherwise hold each load back
        // behind the store before it)
        constexpr int JC = FN <= 2 ? FN : 2;
        float4 xs[EPI == EPI_GELU_MUL ? JC : 1][4];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if (EPI == EPI_GELU_MUL && j % JC == 0)
#pragma unroll
            for (int jj = 0; jj < JC; ++jj)
#pragma unroll
              for (int g = 0; g < 4; ++g)
                xs[EPI == EPI_GELU_MUL ? jj : 0][g] =
                    *(const float4*)(a.aux + m * a.aux_ld + n0 + wn * WN + (j + jj) * 32 + 8 * g + en);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int64_t n = n0 + wn * WN + j * 32 + 8 * g + en;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
            if (EPI == EPI_GELU_MUL) {
              const float4 x = xs[EPI == EPI_GELU_MUL ? j % JC : 0][g];
              v[0] = gelu_tanh(v[0]) * x.x; v[1] = gelu_tanh(v[1]) * x.y;
              v[2] = gelu_tanh(v[2]) * x.z; v[3] = gelu_tanh(v[3]) * x.w;
              *(uint2*)((bf16*)a.C + m * a.ldc + n) = pack_bf16x4(v);
            } else if (CF32) {
              if (EPI == EPI_SOFTCAP) {
                const float inv = 1.f / a.cap;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = a.cap * tanhf(v[e] * inv);
              }
              *(float4*)((float*)a.C + (int64_t)z * a.split_stride + m * a.ldc + n) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
              *(uint2*)((bf16*)a.C + m * a.ldc + n) = pack_bf16x4(v);
            }
          }
        }
      }
    }
  };

  if (blockIdx.x >= total) return;
  // first tile: fill the ring, then the first fragments
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int q = 0; q < LG; ++q) dma(s, q);
  G4_WAIT_VMCNT((NS - 1) * LG);  // step 0 landed
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NRD; ++q) rd(0, 0, lds, q);

  for (int t = blockIdx.x; t < total; t += gridDim.x) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    for (int kt = 0; kt < cur.nk; ++kt) {
      const bf16* st = lds + ((G + kt) % NS) * STAGE;
      const bf16* st1 = lds + ((G + kt + 1) % NS) * STAGE;
      // k-slices 0 .. KS-2: MFMAs on one set while the next slice's fragments load into the other
#pragma unroll
      for (int ks = 0; ks < KS - 1; ++ks) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          if (q < NMF) mf(ks & 1, q);
          if (q < NRD) rd((ks + 1) & 1, ks + 1, st, q);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // step kt + 1 landed in every wave, and every wave has read all of step kt's stage
      G4_WAIT_VMCNT((NS - 2) * LG);
      __syncthreads();
      // last k-slice; behind its MFMAs the next step's first fragments (the next tile's, after the last
      // step), then the loads that refill the stage just released with step kt + NS (behind the last
      // LG MFMAs, or spread over all of them when there are more loads than MFMAs)
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (q < NMF) mf(1, q);
        if (q < NRD) rd(0, 0, st1, q);
        if (q < NMF) {
          if (LG <= NMF) {
            if (q >= NMF - LG) dma(kt + NS, q - (NMF - LG));
          } else {
#pragma unroll
            for (int l = q * LG / NMF; l < (q + 1) * LG / NMF; ++l) dma(kt + NS, l);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // epilogue, while the next tile's first steps are in flight
    store_tile(cur.m0, cur.n0, cur.z);
    G += cur.nk;
    cur = nxt;
    nxt = tile_at(t + 2 * gridDim.x);
  }
  G4_WAIT_VMCNT(0);  // loads issued past the last tile land before the block's LDS is released
}

// Shapes the MFMA kernel takes: bf16, K a multiple of 64, output columns a multiple of the tile,
// 16-byte aligned rows, operands small enough for 32-bit buffer offsets, and outputs (and the
// GELU_MUL factor) whose rows take 4-column vector stores. Stacked B matrices must each be a whole
// number of tiles, or (seg, the segmented loader) a whole number of 8-row load groups.
static bool mfma_ok(const GemmArgs& a, int BN, bool seg = false) {
  const int ncols = a.epi == EPI_GEGLU ? BN / 2 : BN;
  if (a.K % MF_KMIN || a.N % ncols) return false;
  if ((a.lda | a.ldb) & 7) return false;
  if (((uintptr_t)a.A | (uintptr_t)a.B | (uintptr_t)(a.B2 ? a.B2 : a.B)) & 15) return false;
  if (a.M * a.lda * 2 > 0x7fffffffLL || a.N * a.ldb * 2 > 0x7fffffffLL) return false;
  if (a.epi == EPI_SOFTCAP && (a.c_dtype != G4_F32 || a.splits > 1 || !(a.cap > 0.f) || a.nseg > 1)) return false;
  const bool f32 = (a.epi == EPI_STORE || a.epi == EPI_SOFTCAP) && a.c_dtype == G4_F32;
  if ((a.ldc & 3) || ((uintptr_t)a.C & (f32 ? 15 : 7))) return false;
  if (f32 && a.splits > 1 && (a.split_stride & 3)) return false;
  if (a.epi == EPI_GELU_MUL && ((a.aux_ld & 3) || ((uintptr_t)a.aux & 15))) return false;
  if (seg && a.epi != EPI_STORE) return false;
  if (a.nseg > 1) {  // stacked B matrices: aligned, 32-bit offsets, whole tiles (or load groups)
    if (a.epi != EPI_STORE || a.nseg > 3) return false;
    int64_t rows = 0;
    for (int i = 0; i < a.nseg; ++i) {
      if (a.seg_rows[i] % (seg ? 8 : ncols) || ((uintptr_t)a.segB[i] & 15) || a.seg_rows[i] * a.ldb * 2 > 0x7fffffffLL)
        return false;
      rows += a.seg_rows[i];
    }
    if (rows != a.N) return false;
  }
  return true;
}

// Blocks of kernel `k` that fit on the device at once (resident blocks per CU times CUs).
static int resident_blocks(const void* k, int threads) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, threads, 0) != hipSuccess) return 0;
  return cus * per_cu;
}

template <int BM, int BN, int NW, int BK, int NS, int EPI, bool CF32, bool SEGB = false, int WGM = NW / 2>
static void launch_one(const GemmArgs& a, int tm, int tn, int total, bool persist, hipStream_t s) {
  const void* k = (const void*)k_gemm_mfma<BM, BN, NW, BK, NS, EPI, CF32, SEGB, WGM>;
  int grid = total;
  if (persist) {
    const int res = resident_blocks(k, NW * 64);
    if (res > 0 && res < total) grid = res;
  }
  hipLaunchKernelGGL((k_gemm_mfma<BM, BN, NW, BK, NS, EPI, CF32, SEGB, WGM>), dim3((unsigned)grid), dim3(NW * 64), 0,
                     s, a, tm, tn);
}

// One launch walks every (split, tile) pair. When every split spans at least NS K-steps, the grid is
// what fits on the device at once and each block walks several tiles, prefetching the next tile's
// first steps under the current tile's last ones; otherwise each block takes one tile.
template <int BM, int BN, int NW, int BK, int NS, bool SEGB = false, int WGM = NW / 2>
static g4_status launch_mfma(const GemmArgs& a, hipStream_t s) {
  const int ncols = a.epi == EPI_GEGLU ? BN / 2 : BN;
  const int tm = (int)((a.M + BM - 1) / BM), tn = (int)(a.N / ncols);
  const int total = tm * tn * a.splits;
  const int64_t kper = ((a.K + a.splits - 1) / a.splits + BK - 1) / BK * BK;
  const int64_t last = a.K - (int64_t)(a.splits - 1) * kper;
  const bool persist = (last < kper ? last : kper) >= (int64_t)NS * BK;
  if constexpr (SEGB) {
    if (a.c_dtype == G4_F32) launch_one<BM, BN, NW, BK, NS, EPI_STORE, true, true, WGM>(a, tm, tn, total, persist, s);
    else launch_one<BM, BN, NW, BK, NS, EPI_STORE, false, true, WGM>(a, tm, tn, total, persist, s);
  } else {
    if (a.epi == EPI_GEGLU) launch_one<BM, BN, NW, BK, NS, EPI_GEGLU, false, false, WGM>(a, tm, tn, total, persist, s);
    else if (a.epi == EPI_GELU_MUL) launch_one<BM, BN, NW, BK, NS, EPI_GELU_MUL, false, false, WGM>(a, tm, tn, total, persist, s);
    else if (a.epi == EPI_SOFTCAP) {
      if constexpr (BM == 64) launch_one<BM, BN, NW, BK, NS, EPI_SOFTCAP, true, false, WGM>(a, tm, tn, total, persist, s);
      else return fail(G4_EUNSUP, "gemm_mfma: the softcap epilogue is built for 64-row tiles only");
    }
    else if (a.c_dtype == G4_F32) launch_one<BM, BN, NW, BK, NS, EPI_STORE, true, false, WGM>(a, tm, tn, total, persist, s);
    else launch_one<BM, BN, NW, BK, NS, EPI_STORE, false, false, WGM>(a, tm, tn, total, persist, s);
  }
  return check_launch("gemm_mfma");
}

// Up to 64 token rows (batched decode): one 64-row tile covers every token row, and the weights stream
// once in whole 128-byte lines (K steps of 64) through four stages. Plain stores take 64 x 64 tiles
// (2 x 2 waves of 32 x 32): the most tiles, so the most CUs pulling weights (at 64 rows, 42 decode
// layers: q/k/v, o and down 1.71 ms per step against 1.77 with 64 x 128 tiles, 2.02 with 64 x 256 and
// 2.13 with the 256-row tiles). The gated product takes 64 x 128 tiles (64 outputs, 2 x 2 waves of
// 32 x 64): 1.52 ms against 1.69 with 64 x 64 (twice the activation re-reads) and 1.76 with 128 x 128
// tiles in K steps of 32. Deeper rings (five to eight stages) measured slower. A plain product so wide
// that 128-wide tiles still number four per CU (an output head over a vocabulary) takes 64 x 128 tiles:
// half the activation re-reads of 64-wide ones, which at 64 rows are as many bytes as the weights.
// Returns the output columns per tile, 0 when the shape does not fit.
int gemm_rows64_cols(const GemmArgs& a) {
  if (a.M > 64) return 0;
  if (a.epi == EPI_GEGLU && mfma_ok(a, 128)) return 64;
  const bool plain = a.epi == EPI_STORE || a.epi == EPI_SOFTCAP;
  if (plain && a.nseg <= 1 && a.N / 256 >= 4 * (int64_t)device_cus() && mfma_ok(a, 256)) return 256;
  if (plain && a.nseg <= 1 && a.N / 128 >= 4 * (int64_t)device_cus() && mfma_ok(a, 128)) return 128;
  if (mfma_ok(a, 64)) return a.epi == EPI_GEGLU ? 32 : 64;
  return 0;
}

static bool gemm_mfma_rows64(const GemmArgs& a, hipStream_t s, g4_status* st) {
  const int cols = gemm_rows64_cols(a);
  if (cols == 0) return false;
  if (cols == 256) *st = launch_mfma<64, 256, 4, 64, 3, false, 2>(a, s);
  else if (cols == 128 || (a.epi == EPI_GEGLU && cols == 64)) *st = launch_mfma<64, 128, 4, 64, 4, false, 2>(a, s);
  else *st = launch_mfma<64, 64, 4, 64, 4, false, 2>(a, s);
  return true;
}

// 64 x 64 tiles at any row count, K whole (plain stores and the gelu-times-factor epilogue): for
// products with few output columns, where 128-row tiles would need a K split and a finishing pass to
// fill the CUs.
bool gemm_mfma_tiles64(const GemmArgs& a, hipStream_t s, g4_status* st) {
  if (a.splits > 1 || (a.epi != EPI_STORE && a.epi != EPI_GELU_MUL) || a.nseg > 1 || !mfma_ok(a, 64)) return false;
  *st = launch_mfma<64, 64, 4, 64, 4, false, 2>(a, s);
  return true;
}

// Cost of a 256-row tiling in tile-passes over the CUs, weighted by the tile's width and its split's
// K length (each extra split-K slice also costs its float32 traffic, counted as 3%). 0 when the
// tiling leaves more than a quarter of the CUs idle in its only pass (the 128 x 128 kernel then does
// better).
static double tiling_cost(int64_t M, int64_t N, int64_t K, int bn, int splits, int64_t cus) {
  const int64_t items = ((M + 255) / 256) * (N / bn) * splits;
  if (items * 4 < cus * 3) return 0.0;
  const int64_t kper = ((K + splits - 1) / splits + 63) / 64 * 64;
  const int64_t passes = (items + cus - 1) / cus;
  return (double)passes * bn / 256.0 * (double)kper * (1.0 + 0.03 * (splits - 1));
}

// The plain-store widths: 256, 320 (five 32-column blocks per wave), 192 through the segmented loader
// (stacked B matrices need not be whole tiles), and 128 when its tiles fit in one pass (with a second
// pass the 128 x 128 kernel, two blocks per CU, does better: 4096 x 2560 outputs at K = 256 take 23.8 us
// in 256 x 128 tiles, 18.7 us in 128 x 128 ones). Ties go to the wider tile.
static int pick_width(const GemmArgs& a, int64_t cus, double* cost) {
  int best = 0;
  double bc = 0.0;
  const int widths[4] = {256, 320, 192, 128};
  for (int w : widths) {
    if (!mfma_ok(a, w, w == 192)) continue;
    if (w == 128 && ((a.M + 255) / 256) * (a.N / 128) * a.splits > cus) continue;
    const double c = tiling_cost(a.M, a.N, a.K, w, a.splits, cus);
    if (c > 0.0 && (best == 0 || c < bc - 1e-9)) { best = w; bc = c; }
  }
  if (cost) *cost = bc;
  return best;
}

int32_t gemm_pick_splits(int64_t M, int64_t N, int64_t K, int32_t max_splits) {
  if (M < 128 || K % 256) return 1;
  const int64_t cus = device_cus();
  GemmArgs a{};
  a.M = M; a.N = N; a.K = K; a.lda = a.ldb = K; a.ldc = N; a.c_dtype = G4_F32; a.epi = EPI_STORE;
  a.split_stride = M * N;
  int32_t best = 1;
  double bc = 0.0;
  for (int32_t s = 1; s <= max_splits; ++s) {
    if (K / s < 512) break;
    a.splits = s;
    double c = 0.0;
    if (pick_width(a, cus, &c) == 0) continue;
    if (bc == 0.0 || c < bc - 1e-9) { bc = c; best = s; }
  }
  return best;
}

// Picks a tile that gives enough blocks for 256 CUs (up to 64 token rows, the 64-row tiles above); false
// if the shape does not suit the MFMA path.
// The gated product may take 256 x 320 tiles (160 outputs each) where they need fewer passes over the
// CUs, counting a 320-wide tile as 1.25 of a 256-wide one: at 2048 token rows and 10240 outputs, 640
// tiles of 256 x 256 take three passes of 256 CUs (the last half empty), 512 of 256 x 320 take two.
// Plain stores choose among 256, 320, 192 and 128 wide tiles by the same count (tiling_cost).
bool gemm_mfma(const GemmArgs& a, hipStream_t s, g4_status* st) {
  const int64_t cus = device_cus();
  if (a.M <= 64 && gemm_mfma_rows64(a, s, st)) return true;
  if (a.epi == EPI_SOFTCAP) return false;  // built for the 64-row tiles only
  if (a.epi == EPI_GEGLU) {
    const int64_t tiles256 = ((a.M + 255) / 256) * (a.N / 128) * a.splits;
    if (a.splits == 1 && mfma_ok(a, 320) && tiles256 >= 192) {
      const int64_t tiles320 = ((a.M + 255) / 256) * (a.N / 160);
      const double p256 = (double)((tiles256 + cus - 1) / cus), p320 = 1.25 * (double)((tiles320 + cus - 1) / cus);
      if (p320 < p256 - 1e-9) {
        const int tm = (int)((a.M + 255) / 256), tn = (int)(a.N / 160);
        const bool persist = a.K >= 2 * 64;
        launch_one<256, 320, 8, 64, 2, EPI_GEGLU, false>(a, tm, tn, tm * tn, persist, s);
        *st = check_launch("gemm_mfma_320");
        return true;
      }
    }
    if (mfma_ok(a, 256) && tiles256 >= 192) {
      *st = launch_mfma<256, 256, G4_GEMM_NW, G4_GEMM_BK, G4_GEMM_NS>(a, s);
      return true;
    }
  } else if (a.epi == EPI_STORE) {
    const int w = pick_width(a, cus, nullptr);
    if (w == 256) { *st = launch_mfma<256, 256, G4_GEMM_NW, G4_GEMM_BK, G4_GEMM_NS>(a, s); return true; }
    if (w == 320) { *st = launch_mfma<256, 320, 8, 64, 2>(a, s); return true; }
    if (w == 192) { *st = launch_mfma<256, 192, 8, 64, 2, true>(a, s); return true; }
    if (w == 128) { *st = launch_mfma<256, 128, 8, 64, 2>(a, s); return true; }
  } else if (mfma_ok(a, 256) && ((a.M + 255) / 256) * (a.N / 256) * a.splits >= 192) {
    *st = launch_mfma<256, 256, G4_GEMM_NW, G4_GEMM_BK, G4_GEMM_NS>(a, s);
    return true;
  }
  if (mfma_ok(a, 128)) {
    *st = launch_mfma<128, 128, 4, 32, 4>(a, s);
    return true;
  }
  return false;
}

}  // namespace g4
