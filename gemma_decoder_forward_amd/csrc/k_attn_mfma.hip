// Flash-style prefill attention on the CDNA4 matrix cores (bf16 operands, float32 softmax and
// accumulation), causal with an optional sliding window or with the encoder's non-causal mask (key_span),
// GQA groups sharing every K/V tile.
// Three kernels: k_attn_w16 (16-query waves, head dim 256) and k_attn_w16p (its head-dim-512 form
// with the two waves of a query group sharing P), each described before it, and k_attn_mfma (32-query
// waves, head dim 128), described here.
//
// Block = 4 waves. A "query group" is one head x 32 consecutive tokens; each wave owns one, and the
// block's four groups (the heads of one kv group for G = 4) share every K/V tile. For head dim 512 a
// wave holds Q (32 x 512, 128 registers) and O (256 accumulation registers). Keys advance in tiles of
// 32 staged in an LDS ring of two or four stages: later tiles' rows are loaded straight into LDS
// (buffer_load ... lds, one instruction per row) while the current tile is multiplied.
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: A = K rows from LDS,
//     B = the wave's Q held in registers for the whole key loop;
//   * lane l then holds query (l % 32) and 16 of the tile's keys: 8*(j/4) + 4*(l/32) + j%4 for
//     register j. The online softmax (exp2 form, max over the two lanes of a query) runs in place;
//   * O^T = V^T P^T uses those probabilities directly as the B operand: for the 16-key MFMA step s,
//     the lane's registers j = 8s..8s+7 are keys {16s + 4h + 0..3, 16s + 8 + 4h + 0..3} (h = l/32), and
//     the A operand reads V^T at exactly those keys, so P never moves between lanes;
//   * V stays row-major in LDS and the V^T operand comes from the LDS transpose read; K and V rows are
//     padded (strides of 16 and 32 bytes mod 256) so both operand reads are free of bank conflicts.
// The O accumulator (HD/32 32x32 blocks per wave) lives in the accumulation registers.
#include <functional>
#include <queue>
#include <type_traits>
#include <utility>
#include <vector>

#include "g4_internal.h"

namespace g4 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int AT_KB = 32;        // keys per tile
constexpr int AT_PS = 4;         // most key parts one query block is split into

// Key split of a launch's query blocks: block b takes 1 + (b >= th1) + (b >= th2) + (b >= th3) parts
// (th1 <= th2 <= th3 <= nblk), each part a contiguous share of the block's key tiles. Work items run
// heaviest first: the 4-part blocks from the last one down, then the 3-part, 2-part and whole ones.
struct AtSplit {
  int th1, th2, th3;
};
__device__ __forceinline__ void at_item(int v, int nblk, const AtSplit& sp, int& blk, int& part, int& nparts) {
  const int c4 = nblk - sp.th3, c3 = sp.th3 - sp.th2, c2 = sp.th2 - sp.th1;
  if (v < 4 * c4) { blk = nblk - 1 - v / 4; part = v % 4; nparts = 4; return; }
  v -= 4 * c4;
  if (v < 3 * c3) { blk = sp.th3 - 1 - v / 3; part = v % 3; nparts = 3; return; }
  v -= 3 * c3;
  if (v < 2 * c2) { blk = sp.th2 - 1 - v / 2; part = v & 1; nparts = 2; return; }
  v -= 2 * c2;
  blk = sp.th1 - 1 - v; part = 0; nparts = 1;
}

typedef __attribute__((address_space(3))) void at_lds_void;
typedef short at_v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) at_v4s at_lds_v4s;
typedef __attribute__((ext_vector_type(4))) uint32_t at_rsrc;

// K and V are staged by direct buffer-to-LDS loads (one instruction per row: 64, 32 or 16 lanes of
// 16 bytes for head dim 512, 256, 128) and V stays row-major; the V^T operand then comes from the LDS
// transpose read.
template <int HD>
struct AttnLds {
  static constexpr int KLD = HD + 8;   // K row stride in bf16 (16-lane chunk reads hit every bank once)
  static constexpr int VROW = HD + 16; // row-major V stride (a transpose read's four row pieces on distinct banks)
  static constexpr int KSZ = AT_KB * KLD;
  static constexpr int VSZ = AT_KB * VROW;
  static constexpr int STAGE = KSZ + VSZ;
};

__device__ __forceinline__ at_rsrc at_make_rsrc(const void* base, int64_t bytes) {
  const uint64_t p = (uint64_t)base;
  const uint32_t n = bytes > 0x7fffffff ? 0x7fffffffu : (bytes < 0 ? 0u : (uint32_t)bytes);
  at_rsrc r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)p);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xffffu);
  r.z = __builtin_amdgcn_readfirstlane(n);
  r.w = 0x00020000u;
  return r;
}

// 16 bytes per lane from voff + soff straight into LDS at m0 + 16 * lane (inline assembly: the
// completion is awaited with an explicit vmcnt before the barrier that precedes the reads).
__device__ __forceinline__ void at_dma16(const at_rsrc& r, uint32_t voff, uint32_t soff, uint32_t m0) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" : : "v"(voff), "s"(r), "s"(soff), "{m0}"(m0) : "memory");
}

// K/V stages in the LDS ring: the loads of a tile are issued NS - 1 tiles ahead of its use. A tile of
// 32 keys at head dim 256 or less is a short stretch of matrix work, shorter than a trip to memory, so
// those dims keep four stages in flight (137 KB of LDS at 256); head dim 512 fits two (134 KB).
// The 16-query kernel's staging: K rows padded by 32 bytes (see k_attn_w16), V rows as above; tiles
// of KB keys. Head dim 256 takes 64-key tiles, so the per-tile costs that do not scale with the
// tile's matrix work (block barrier, stage wait, load addressing, softmax bookkeeping) are paid once
// per 64 keys; a 64-key stage is 70 KB, two fit. Head dim 512 keeps 32-key tiles (two 68 KB stages).
template <int HD> struct AttnTileW {
  static constexpr int KB = HD == 256 ? 64 : 32;
  static constexpr int NS = 2;
};
template <int HD>
struct AttnLdsW {
  static constexpr int KB = AttnTileW<HD>::KB;
  static constexpr int KLD = HD + 16;
  static constexpr int VROW = HD + 16;
  static constexpr int KSZ = KB * KLD;
  static constexpr int VSZ = KB * VROW;
  static constexpr int STAGE = KSZ + VSZ;
};

template <int HD> struct AttnStages { static constexpr int NS = HD == 512 ? 2 : 4; };

#define G4_ATT_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

template <int HD>
__global__ __launch_bounds__(256, 1) void k_attn_mfma(AttnArgs a, int G, float sl2, AtSplit sp) {
  using L = AttnLds<HD>;
  constexpr int NB = HD / 32;      // O blocks per wave
  constexpr int KS = HD / 16;      // MFMA k-steps for S
  constexpr int QG = 4;            // query groups per block
  constexpr int NS = AttnStages<HD>::NS;
  constexpr int LPT = 2 * (AT_KB / 4);  // direct-to-LDS load instructions per wave per tile (K and V rows)
  static_assert((NS - 2) * LPT <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) bf16 lds[NS * L::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  // query groups are numbered run * G + head_in_group; a block takes QG consecutive ones
  const int nruns = (int)((a.T + 31) / 32);
  const int ngroups = nruns * G;
  const int nblk = (ngroups + QG - 1) / QG;
  // Work items, heaviest first (AtSplit): a split block comes as one item per share of its key tiles;
  // consecutive blocks of the grid take the same item of each kv head and sequence.
  int blk, part, nparts;
  const int64_t g = (int64_t)blockIdx.x % a.nkv, b = ((int64_t)blockIdx.x / a.nkv) % a.B;
  at_item((int)((int64_t)blockIdx.x / (a.nkv * a.B)), nblk, sp, blk, part, nparts);
  const int gi = blk * QG + wave;
  const int run = gi / G;
  const int64_t head = g * G + gi % G;
  const int64_t tq = (int64_t)run * 32 + col;  // this lane's query token
  const int64_t p0 = a.pos0[b];
  const bool qvalid = gi < ngroups && tq < a.T;
  const int64_t qi = p0 + tq;                  // absolute position of the query

  // block key range (union over its groups)
  const int g_first = blk * QG, g_last = (blk * QG + QG - 1) < ngroups - 1 ? blk * QG + QG - 1 : ngroups - 1;
  int64_t tlast = (int64_t)(g_last / G) * 32 + 31;
  if (tlast > a.T - 1) tlast = a.T - 1;
  const int64_t imin = p0 + (int64_t)(g_first / G) * 32, imax = p0 + tlast;
  const KeySpan ksp = key_span(a.bidir, a.sliding, a.window, a.cap, a.ring, p0, a.T);
  int64_t lob = imin - ksp.back;
  if (lob < ksp.kmin) lob = ksp.kmin;
  int64_t hib = imax + ksp.fwd;
  if (hib > ksp.kmax) hib = ksp.kmax;
  const int64_t kstart = lob & ~(int64_t)(AT_KB - 1);
  const int ntiles = hib >= lob ? (int)((hib - kstart) / AT_KB + 1) : 0;
  const int it0 = part * ntiles / nparts, it1 = (part + 1) * ntiles / nparts;
  int64_t qlo = qi - ksp.back;
  if (qlo < ksp.kmin) qlo = ksp.kmin;
  const int64_t qhi = qi + ksp.fwd < hib ? qi + ksp.fwd : hib;  // this query's last visible key
  // keys visible to every query of the wave: [wlo_all, whi_all] (empty for a wave with invalid queries)
  int64_t wlo_all, whi_all;
  {
    const int64_t first = p0 + (int64_t)run * 32, last = p0 + (int64_t)run * 32 + 31;
    wlo_all = last - ksp.back;
    if (wlo_all < lob) wlo_all = lob;
    whi_all = first + ksp.fwd < hib ? first + ksp.fwd : hib;
    if (!(gi < ngroups && (int64_t)run * 32 + 31 < a.T)) { wlo_all = 1; whi_all = 0; }
  }

  // Q fragments (B operand of S^T): query col, hd 16s + 8h .. +7
  bf16x8_t qf[KS];
  {
    const bf16* qrow = (const bf16*)a.q + (b * a.T + (qvalid ? tq : 0)) * a.q_ld + (qvalid ? head : 0) * HD +
                       8 * h;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 v = qvalid ? *(const uint4*)(qrow + 16 * s) : make_uint4(0, 0, 0, 0);
      qf[s] = *(bf16x8_t*)&v;
    }
  }
  // Q has landed before the first tile load is issued. The compiler does not see the direct-to-LDS
  // loads (inline assembly); left to itself it would wait for Q at its first use inside the key loop
  // with a full memory wait, which also waits out the tiles in flight, on every step.
#pragma unroll
  for (int s = 0; s < KS; ++s) asm volatile("" : : "v"(qf[s]));

  const bf16* Kb = (const bf16*)a.k + (b * a.nkv + g) * a.cap * HD;
  const bf16* Vb = (const bf16*)a.v + (b * a.nkv + g) * a.cap * HD;
  // Staging: rows 8w .. 8w+7 of the tile from wave w, K and V. Keys past the cache
  // clamp to its last row (they are masked); V rows whose keys lie outside [lob, hib] are zeroed after
  // they land (a masked probability times a stale value must stay zero, not NaN).
  const at_rsrc rks = at_make_rsrc(Kb, a.cap * HD * 2), rvs = at_make_rsrc(Vb, a.cap * HD * 2);
  // Tile it into ring slot it % NS. A tile past the block's range (the ring keeps issuing one tile per
  // step) gets a scalar offset beyond the buffer, which the range check turns into zeros without moving
  // data, so every step keeps the same number of loads in flight and the waits below stay exact.
  auto dma = [&](int it) {
    const int64_t k0 = kstart + (int64_t)it * AT_KB;
    const bool live = it < it1;
    const uint32_t kb0 = (uint32_t)(uintptr_t)(at_lds_void*)(lds + (it % NS) * L::STAGE);
    const uint32_t vb0 = kb0 + L::KSZ * 2;
    const int wv = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform: offsets and M0 live in SGPRs
    // cache row of this wave's first key (one remainder per tile); the next rows follow it, wrapping once
    const int64_t kb = k0 + (AT_KB / 4) * wv;
    const int64_t rb = kv_row(kb, a.cap, a.ring);
#pragma unroll
    for (int r = 0; r < AT_KB / 4; ++r) {
      const int row = (AT_KB / 4) * wv + r;
      int64_t cr;
      if (!a.ring) cr = kb + r > a.cap - 1 ? a.cap - 1 : kb + r;  // keys past the cache clamp to its last row
      else if (a.cap >= AT_KB / 4) cr = rb + r >= a.cap ? rb + r - a.cap : rb + r;
      else cr = kv_row(kb + r, a.cap, a.ring);
      // the row's byte offset in the per-lane offset: no scalar register written by a vector
      // instruction feeds the load (the compiler's hazard checks do not see into the assembly)
      const uint32_t voff = (uint32_t)(cr * HD * 2) + (uint32_t)lane * 16;
      const uint32_t oob = live ? 0u : 0x80000000u;
      if (lane < HD / 8) {  // a row is HD / 8 lanes of 16 bytes
        at_dma16(rks, voff, oob, kb0 + (uint32_t)(row * L::KLD * 2));
        at_dma16(rvs, voff, oob, vb0 + (uint32_t)(row * L::VROW * 2));
      }
    }
  };
  auto edge_tile = [&](int it) {
    const int64_t k0 = kstart + (int64_t)it * AT_KB;
    return !(k0 >= lob && k0 + AT_KB - 1 <= hib);
  };
  auto vclean = [&](int it, int buf) {
    const int64_t k0 = kstart + (int64_t)it * AT_KB;
    bf16* vs = lds + buf * L::STAGE + L::KSZ;
    for (int u = tid; u < AT_KB * (HD / 8); u += 256) {
      const int row = u / (HD / 8);
      const int64_t key = k0 + row;
      if (key < lob || key > hib) *(uint4*)(vs + row * L::VROW + 8 * (u % (HD / 8))) = make_uint4(0, 0, 0, 0);
    }
  };

  f32x16_t o[NB];
#pragma unroll
  for (int d = 0; d < NB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  if (it1 > it0) {
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) dma(it0 + j);
    G4_ATT_WAIT_VMCNT((NS - 2) * LPT);  // tile it0 landed
    __syncthreads();
    if (edge_tile(it0)) {
      vclean(it0, it0 % NS);
      __syncthreads();
    }
  }
  for (int it = it0; it < it1; ++it) {
    const int cur = it % NS;
    dma(it + NS - 1);  // into the slot read in the previous step, which every wave has left
    const bf16* ks = lds + cur * L::STAGE;
    const bf16* vs = ks + L::KSZ;
    const int64_t k0 = kstart + (int64_t)it * AT_KB;
    // S^T = K Q^T
    f32x16_t s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    const bf16* kf = ks + col * L::KLD + 8 * h;
#pragma unroll
    for (int st = 0; st < KS; ++st)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_t*)(kf + 16 * st), qf[st], s, 0, 0, 0);
    // mask (only on tiles that cut the causal edge, the window start or the block's key range), scale
    // to the exp2 domain, online softmax
    float mt = -INFINITY;
    if (k0 >= wlo_all && k0 + AT_KB - 1 <= whi_all) {  // every key of the tile visible to every query
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] *= sl2;
        mt = fmaxf(mt, s[r]);
      }
    } else {
      const int rel = (int)(k0 - qlo), lim = (int)(qhi - k0);  // visible keys: rel + key' >= 0, key' <= lim
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 8 * (r >> 2) + 4 * h + (r & 3);
        const bool vis = qvalid && kk + rel >= 0 && kk <= lim;
        const float v = vis ? s[r] * sl2 : -INFINITY;
        s[r] = v;
        mt = fmaxf(mt, v);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    // The reference maximum is raised only when the tile's maximum exceeds it by more than 32 (log2
    // domain). Probabilities then stay below 2^32: bf16 P keeps its 8-bit relative precision at any
    // magnitude, and the float32 sums stay far from overflow (below 2^32 x keys x max|v|). The
    // accumulator rescale -- a multiply of every O register -- then runs only when the maximum has
    // grown by 2^32, a few times per query row at most. The result is the same softmax: every term and
    // the normaliser use one reference.
    const bool raise = mt > m_run + 32.f;
    const float m_new = raise ? mt : m_run;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    float psum = 0.f;
    bf16x8_t pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(s[r] - m_use);
      psum += p;
      pb[r >> 3][r & 7] = (__bf16)p;
    }
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // some query of the wave moved its reference
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
      // The rescale touches the accumulators through their accumulation registers (read, multiply,
      // write back one register at a time). Written as plain float code, the compiler keeps every
      // accumulator in an ordinary register across the key loop instead, which for head dim 512 needs
      // more registers than a wave has.
#pragma unroll
      for (int d = 0; d < NB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float tmp;
          asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                       : "+a"(o[d][r]), "=&v"(tmp)
                       : "v"(alpha));
        }
    }
    l_run += psum;
    m_run = m_new;
    // O^T += V^T P^T. MFMA step st takes keys 16st + 4h + (0..3) and 16st + 8 + 4h + (0..3) for lane half
    // h (the order of the score registers).
    {
      // LDS transpose read (ds_read_b64_tr_b16): within a 16-lane group lane i receives element i % 4 of
      // the 8 bytes addressed by lane 4j + i/4, j = 0..3. Lane a of group q addresses key row
      // kb + a/4 at head elements 32d + 16(q % 2) + 4(a % 4), so lane i gets keys kb .. kb+3 of head
      // element 32d + 16(q % 2) + i: the A operand row of lane 16(q % 2) + i.
      const int a16 = lane & 15, grp = lane >> 4;
      const bf16* vb = vs + (4 * (grp >> 1) + (a16 >> 2)) * L::VROW + 16 * (grp & 1) + 4 * (a16 & 3);
#pragma unroll
      for (int d = 0; d < NB; ++d) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          bf16x4_t part[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const bf16* addr = vb + (16 * st + 8 * e) * L::VROW + 32 * d;
            part[e] = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((at_lds_v4s*)(at_lds_void*)addr));
          }
          const bf16x8_t va = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[st], o[d], 0, 0, 0);
        }
      }
      G4_ATT_WAIT_VMCNT((NS - 2) * LPT);  // tile it + 1 landed; later tiles may still be in flight
      __syncthreads();
      if (it + 1 < it1 && edge_tile(it + 1)) {
        vclean(it + 1, (it + 1) % NS);
        __syncthreads();
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!qvalid) return;
  if (nparts > 1) {  // unnormalised partial O with its reference and normaliser, merged afterwards
    const int64_t row = ((part * a.B + b) * a.T + tq) * a.nh + head;
    float* po = a.ws + row * HD;
#pragma unroll
    for (int d = 0; d < NB; ++d)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *(float4*)(po + 32 * d + 8 * r4 + 4 * h) =
            make_float4(o[d][4 * r4], o[d][4 * r4 + 1], o[d][4 * r4 + 2], o[d][4 * r4 + 3]);
    if (h == 0) {
      float* ml = a.ws + AT_PS * a.B * a.T * a.nh * HD + 2 * row;
      ml[0] = m_run;
      ml[1] = l_tot;
    }
    return;
  }
  const float il = l_tot > 0.f ? 1.f / l_tot : 0.f;
  bf16* orow = (bf16*)a.out + (b * a.T + tq) * a.out_ld + head * HD;
#pragma unroll
  for (int d = 0; d < NB; ++d)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int hd0 = 32 * d + 8 * r4 + 4 * h;
      uint2 pk;
      pk.x = (uint32_t)f2bf(o[d][4 * r4] * il) | ((uint32_t)f2bf(o[d][4 * r4 + 1] * il) << 16);
      pk.y = (uint32_t)f2bf(o[d][4 * r4 + 2] * il) | ((uint32_t)f2bf(o[d][4 * r4 + 3] * il) << 16);
      *(uint2*)(orow + hd0) = pk;
    }
}

// Maximum of x over lanes l and l ^ 16 (l ^ 32): the permlane swaps exchange 16-lane rows (32-lane
// halves) between two registers in the vector unit, so the pair meets in every lane without an LDS
// round trip.
__device__ __forceinline__ float at_max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float at_max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// --------------------------------------------------------------------------------------------
// The same attention with 16-query waves on v_mfma_f32_16x16x32_bf16, eight waves per block.
//
// A query group (head x 32 tokens) is split between two waves of 16 queries each, so a wave holds Q
// (16 x HD: HD / 8 registers) and O (HD / 4 accumulation registers) -- for head dim 512, 64 and 128
// instead of 128 and 256 -- and two waves fit on each SIMD: one wave's LDS reads, softmax and tile
// bookkeeping run while the other's matrix instructions execute. The block covers the same four
// query groups, key tiles and work items as k_attn_mfma (same grid and scratch layout), so every K/V
// tile staged in LDS still feeds 128 query rows.
//   * S^T = K Q^T in 16x16 blocks: A = 16 keys x 32 head elements of K from LDS, B = the wave's Q in
//     registers. K rows are padded by 32 bytes: the operand read (16 rows x four 16-byte chunks) is
//     then free of bank conflicts (measured; a 16-byte pad made every such read a two-way conflict). Lane l holds query l % 16 and, per key block kb, keys 16 kb + 4 (l / 16) + 0..3.
//   * O^T += V^T P^T: the B operand's 32 k-slots of lane group q = l / 16 are keys {4q + 0..3,
//     16 + 4q + 0..3}, exactly the lane's eight probabilities; the A operand reads V^T at those keys
//     with two LDS transpose reads (four consecutive key rows of 16 head elements each).
//   * A query's scores of a tile sit in the four lanes l % 16 + 16j: its maximum takes two
//     cross-lane steps; the normaliser is summed per lane and across the four lanes at the end.
//   * Tiles of KB keys (64 at head dim 256, 32 at 512; the P V operand above repeats per 32 keys).
//     Software pipeline: while a wave takes the softmax of tile t, the S MFMAs of tile t + 1 issue
//     between its vector instructions (the matrix unit and the vector unit work side by side), then
//     come the P V MFMAs of tile t. Two LDS stages hold K of tiles t + 1 and t + 2 and V of tiles t and
//     t + 1: the K rows of t + 2 and the V rows of t + 1 load during tile t into the halves whose
//     previous contents every wave finished before the last barrier.
// --------------------------------------------------------------------------------------------
template <int HD, bool RING>
__global__ __launch_bounds__(512, 1) void k_attn_w16(AttnArgs a, int G, float sl2, AtSplit sp) {
  using L = AttnLdsW<HD>;
  typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
  constexpr int KB = L::KB;        // keys per tile
  constexpr int NKB = KB / 16;     // 16-key blocks of S per tile
  constexpr int NPV = KB / 32;     // 32-key steps of P V per tile
  constexpr int NO = HD / 16;      // O blocks (16 head elements each) per wave
  constexpr int KS = HD / 32;      // k-steps of S (32 head elements each)
  constexpr int QG = 4;            // query groups per block, two waves each
  constexpr int NS = AttnTileW<HD>::NS;
  constexpr int NE = 4 * NKB;      // scores per lane per tile
  constexpr int RPW = KB / 8;      // tile rows staged by each wave
  static_assert(NS == 2, "K and V tiles alternate between two stages");
  static_assert(KS >= 8, "the softmax steps ride behind the S steps");
  __shared__ __attribute__((aligned(16))) bf16 lds[NS * L::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 15, qq = lane >> 4;  // query of the lane within the wave; lane group
  const int nruns = (int)((a.T + 31) / 32);
  const int ngroups = nruns * G;
  const int nblk = (ngroups + QG - 1) / QG;
  int blk, part, nparts;
  const int64_t g = (int64_t)blockIdx.x % a.nkv, b = ((int64_t)blockIdx.x / a.nkv) % a.B;
  at_item((int)((int64_t)blockIdx.x / (a.nkv * a.B)), nblk, sp, blk, part, nparts);
  const int gi = blk * QG + (wave >> 1);
  const int run = gi / G;
  const int64_t head = g * G + gi % G;
  const int64_t tq0 = (int64_t)run * 32 + 16 * (wave & 1);  // the wave's first query token
  const int64_t tq = tq0 + ql;                                // this lane's query token
  const int64_t p0 = a.pos0[b];
  const bool qvalid = gi < ngroups && tq < a.T;
  const int64_t qi = p0 + tq;

  // block key range (union over its groups), as in k_attn_mfma
  const int g_first = blk * QG, g_last = (blk * QG + QG - 1) < ngroups - 1 ? blk * QG + QG - 1 : ngroups - 1;
  int64_t tlast = (int64_t)(g_last / G) * 32 + 31;
  if (tlast > a.T - 1) tlast = a.T - 1;
  const int64_t imin = p0 + (int64_t)(g_first / G) * 32, imax = p0 + tlast;
  const KeySpan ksp = key_span(a.bidir, a.sliding, a.window, a.cap, RING ? 1 : 0, p0, a.T);
  int64_t lob = imin - ksp.back;
  if (lob < ksp.kmin) lob = ksp.kmin;
  const int64_t hib = imax + ksp.fwd < ksp.kmax ? imax + ksp.fwd : ksp.kmax;
  const int64_t kstart = lob & ~(int64_t)(KB - 1);
  const int ntiles = hib >= lob ? (int)((hib - kstart) / KB + 1) : 0;
  const int it0 = part * ntiles / nparts, it1 = (part + 1) * ntiles / nparts;
  int64_t qlo = qi - ksp.back;
  if (qlo < ksp.kmin) qlo = ksp.kmin;
  const int64_t qhi = qi + ksp.fwd < hib ? qi + ksp.fwd : hib;
  // the lane's visible keys relative to the first tile, in 32 bits (none for an invalid query)
  const int vlo = qvalid ? (int)(qlo - kstart) : 0x7fffffff, vhi = qvalid ? (int)(qhi - kstart) : -1;
  // keys visible to every query of the wave (empty when some query of the wave is invalid)
  int64_t wlo_all, whi_all;
  {
    const int64_t first = p0 + tq0, last = p0 + tq0 + 15;
    wlo_all = last - ksp.back;
    if (wlo_all < lob) wlo_all = lob;
    whi_all = first + ksp.fwd < hib ? first + ksp.fwd : hib;
    if (!(gi < ngroups && tq0 + 15 < a.T)) { wlo_all = 1; whi_all = 0; }
  }
  // per-tile range tests in 32 bits, relative to the first tile's first key
  const int lob_r = (int)(lob - kstart), hib_r = (int)(hib - kstart);
  const int wlo_r = (int)(wlo_all - kstart), whi_r = wlo_all > whi_all ? -1 : (int)(whi_all - kstart);

  // Q fragments (B operand of S^T): query ql, head elements 32 s + 8 qq .. +7
  bf16x8_t qf[KS];
  {
    const bf16* qrow = (const bf16*)a.q + (b * a.T + (qvalid ? tq : 0)) * a.q_ld + (qvalid ? head : 0) * HD + 8 * qq;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 u = qvalid ? *(const uint4*)(qrow + 32 * s) : make_uint4(0, 0, 0, 0);
      qf[s] = *(bf16x8_t*)&u;
    }
  }
  // Q is in flight together with the first tiles: the prologue waits for both at once, before the key
  // loop (see k_attn_mfma for why the wait must not be left to the compiler)

  const bf16* Kb = (const bf16*)a.k + (b * a.nkv + g) * a.cap * HD;
  const bf16* Vb = (const bf16*)a.v + (b * a.nkv + g) * a.cap * HD;
  const at_rsrc rks = at_make_rsrc(Kb, a.cap * HD * 2), rvs = at_make_rsrc(Vb, a.cap * HD * 2);
  // Tile it into ring slot it % NS; rows RPW w .. RPW w + RPW - 1 from wave w (see k_attn_mfma for the
  // out-of-range tiles and the clamped rows).
  // Cache rows in 32 bits: the byte offsets of a cache fit the 31-bit buffer range (the descriptor's
  // size saturates there), so every row index that reaches a load does too.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int cap32 = (int)a.cap;
  const uint32_t lds_k = (uint32_t)(uintptr_t)(at_lds_void*)lds + (uint32_t)(RPW * wv * L::KLD * 2);
  const uint32_t lds_v = (uint32_t)(uintptr_t)(at_lds_void*)lds + L::KSZ * 2 + (uint32_t)(RPW * wv * L::VROW * 2);
  // K (isv false) or V rows of tile it into stage it % 2: rows RPW w .. RPW w + RPW - 1 from wave w
  // (see k_attn_mfma for the out-of-range tiles and the clamped rows).
  auto dma = [&](int it, bool isv) {
    const bool live = it < it1;
    const uint32_t so = (uint32_t)(it % NS) * L::STAGE * 2;
    const int64_t kb = kstart + (int64_t)it * KB + RPW * wv;  // the wave's first key of the tile
    const int rb = RING ? (int)kv_row(kb, a.cap, 1) : (int)(kb < a.cap ? kb : a.cap - 1);
    // The row's byte offset rides in the per-lane offset, so no scalar register written by a vector
    // instruction feeds the load (the compiler's hazard checks do not see into the assembly); the
    // scalar offset only marks a tile past the range.
    const uint32_t oob = live ? 0u : 0x80000000u;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      int cr;
      if (!RING) cr = rb + r < cap32 - 1 ? rb + r : cap32 - 1;  // keys past the cache clamp to its last row
      else if (cap32 >= RPW) cr = rb + r >= cap32 ? rb + r - cap32 : rb + r;
      else cr = (int)kv_row(kb + r, a.cap, 1);
      const uint32_t voff = (uint32_t)cr * (HD * 2) + (uint32_t)lane * 16;
      if (lane < HD / 8) {
        if (isv) at_dma16(rvs, voff, oob, lds_v + so + (uint32_t)(r * L::VROW * 2));
        else at_dma16(rks, voff, oob, lds_k + so + (uint32_t)(r * L::KLD * 2));
      }
    }
  };
  auto edge_tile = [&](int it) {
    const int kt = it * KB;
    return !(kt >= lob_r && kt + KB - 1 <= hib_r);
  };
  auto vclean = [&](int it, int buf) {
    const int kt = it * KB;
    bf16* vs = lds + buf * L::STAGE + L::KSZ;
    for (int u = tid; u < KB * (HD / 8); u += 512) {
      const int row = u / (HD / 8);
      const int key = kt + row;
      if (key < lob_r || key > hib_r) *(uint4*)(vs + row * L::VROW + 8 * (u % (HD / 8))) = make_uint4(0, 0, 0, 0);
    }
  };

  f32x4_t o[NO];
#pragma unroll
  for (int d = 0; d < NO; ++d) o[d] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  // operand addresses within a stage (bf16 elements)
  const int kfo = ql * L::KLD + 8 * qq;                                   // K: key row ql, chunk qq
  const int vfo = (4 * qq + (ql >> 2)) * L::VROW + 4 * (ql & 3);          // V^T: rows 4qq + ql/4

  // S^T of one tile for the tile's NKB key blocks (independent accumulation chains). K fragments are
  // read PK steps ahead in a rolling window, pinned by scheduling barriers (at head dim 512 the two
  // waves per SIMD leave registers for two steps only). step(st) runs after the MFMAs of k-step st,
  // inside the same scheduling region, so its vector work issues between them.
  constexpr int PK = HD == 256 ? 3 : 2;
  auto s_tile = [&](const bf16* ks, f32x4_t (&acc)[NKB], auto&& step) {
    bf16x8_t kw[NKB][PK];
#pragma unroll
    for (int k = 0; k < NKB; ++k) {
      acc[k] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < PK; ++j) kw[k][j] = *(const bf16x8_t*)(ks + kfo + 16 * k * L::KLD + 32 * j);
    }
#pragma unroll
    for (int st = 0; st < KS; ++st) {
#pragma unroll
      for (int k = 0; k < NKB; ++k) {
        acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kw[k][st % PK], qf[st], acc[k], 0, 0, 0);
        if (st + PK < KS) kw[k][st % PK] = *(const bf16x8_t*)(ks + kfo + 16 * k * L::KLD + 32 * (st + PK));
      }
      step(st);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The online softmax of one tile, cut into KS steps that ride behind the next tile's S MFMAs:
  // step 0 scales (and on edge tiles masks) the lane's NE scores and takes their maximum, steps 1 and
  // 2 complete the maximum over the four lanes of each query (permlane swaps: no LDS round trip),
  // step 2 also sets the reference, and steps 3 .. KS-1 take the exponentials. The lane holds keys
  // 16 k + 4 qq + (r & 3) of key block k = r / 4 in sc[r]; the P operand of the 32-key step h is the
  // lane's keys {32 h + 4 qq + 0..3, 32 h + 16 + 4 qq + 0..3}, sc[8 h .. 8 h + 7].
  float sc[NE];
  float mt = -INFINITY, m_new = -INFINITY, m_use = 0.f, psum = 0.f;
  bool raise = false, full = false;
  int kt = 0;
  bf16x8_t pb[NPV];
  auto smax_step = [&](int st) {
    if (st == 0) {
      // the maximum of the unscaled scores (sl2 > 0: the host takes only positive scales here); the
      // scale rides in the exponential's fused multiply-add
      mt = -INFINITY;
      if (full) {
#pragma unroll
        for (int r = 0; r < NE; ++r) mt = fmaxf(mt, sc[r]);
      } else {
#pragma unroll
        for (int r = 0; r < NE; ++r) {
          const int kk = kt + 16 * (r >> 2) + 4 * qq + (r & 3);
          const bool vis = kk >= vlo && kk <= vhi;
          const float x = vis ? sc[r] : -INFINITY;
          sc[r] = x;
          mt = fmaxf(mt, x);
        }
      }
    } else if (st == 1) {
      mt = at_max_xor16(mt);
    } else if (st == 2) {
      mt = at_max_xor32(mt) * sl2;
      // lazy reference, as in k_attn_mfma: raised only when the tile exceeds it by more than 32 (log2)
      raise = mt > m_run + 32.f;
      m_new = raise ? mt : m_run;
      m_use = m_new == -INFINITY ? 0.f : m_new;
      psum = 0.f;
    } else {
#pragma unroll
      for (int r = 0; r < NE; ++r)
        if (3 + r * (KS - 3) / NE == st) {
          const float pr = __builtin_amdgcn_exp2f(fmaf(sc[r], sl2, -m_use));
          psum += pr;
          pb[r / 8][r % 8] = (__bf16)pr;
        }
    }
  };

  // One tile: the softmax of tile it (S already in sacc) behind the S MFMAs of tile it + 1 (MORE),
  // then O^T += V^T P^T. Tile it + 2's K rows and tile it + 1's V rows load meanwhile: each into the
  // half of the stage whose previous tile every wave finished before the last barrier.
  f32x4_t sacc[NKB], snext[NKB];
  auto iter = [&](int it, auto more_t) {
    constexpr bool MORE = decltype(more_t)::value;
    const int cur = it % NS, nx = (it + 1) % NS;
    if (MORE) {
      dma(it + 2, false);
      dma(it + 1, true);
    }
    kt = it * KB;  // the tile's first key relative to kstart
    full = kt >= wlo_r && kt + KB - 1 <= whi_r;
#pragma unroll
    for (int k = 0; k < NKB; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * k + i] = sacc[k][i];
    if constexpr (MORE) {
      // the wave in this phase issues first: its matrix and vector work overlap each other, and the
      // SIMD's other wave, whose P V MFMAs have no vector work beside them, fills the gaps
      __builtin_amdgcn_s_setprio(1);
      s_tile(lds + nx * L::STAGE, snext, smax_step);
      __builtin_amdgcn_s_setprio(0);
    } else {
#pragma unroll
      for (int st = 0; st < KS; ++st) smax_step(st);
    }
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < NO; ++d) o[d] *= alpha;
    }
    l_run += psum;
    m_run = m_new;
    // O^T += V^T P^T, 16 head elements per MFMA, for each 32-key step h; V^T fragments read PV MFMAs
    // ahead
    const bf16* vs = lds + cur * L::STAGE + L::KSZ;
    constexpr int PV = HD == 256 ? 8 : 4;
    constexpr int NM = NPV * NO;
    auto vread = [&](int j) {
      const int h = j / NO, d = j % NO;
      const bf16* va = vs + vfo + 32 * h * L::VROW + 16 * d;
      const bf16x4_t lo = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((at_lds_v4s*)(at_lds_void*)va));
      const bf16x4_t hi = __builtin_bit_cast(
          bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((at_lds_v4s*)(at_lds_void*)(va + 16 * L::VROW)));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8_t vw[PV];
#pragma unroll
    for (int j = 0; j < PV; ++j) vw[j] = vread(j);
#pragma unroll
    for (int j = 0; j < NM; ++j) {
      o[j % NO] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vw[j % PV], pb[j / NO], o[j % NO], 0, 0, 0);
      if (j + PV < NM) vw[j % PV] = vread(j + PV);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (MORE) {
      G4_ATT_WAIT_VMCNT(0);  // tile it + 2's K and tile it + 1's V landed
      __syncthreads();
      if (edge_tile(it + 1)) {
        vclean(it + 1, nx);
        __syncthreads();
      }
#pragma unroll
      for (int k = 0; k < NKB; ++k) sacc[k] = snext[k];
    }
  };

  if (it1 > it0) {
    dma(it0, false);
    dma(it0, true);
    dma(it0 + 1, false);
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" : : "v"(qf[s]));
    G4_ATT_WAIT_VMCNT(0);
    __syncthreads();
    if (edge_tile(it0)) vclean(it0, it0 % NS);
    s_tile(lds + (it0 % NS) * L::STAGE, sacc, [](int) {});
    __syncthreads();  // every wave is done with tile it0's K rows (refilled by the first iteration)
    int it = it0;
    for (; it + 1 < it1; ++it) iter(it, std::true_type{});
    iter(it, std::false_type{});
  }

  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (!qvalid) return;
  // lane holds head elements 16 d + 4 qq + 0..3 of query tq
  if (nparts > 1) {
    const int64_t row = ((part * a.B + b) * a.T + tq) * a.nh + head;
    float* po = a.ws + row * HD;
#pragma unroll
    for (int d = 0; d < NO; ++d) *(float4*)(po + 16 * d + 4 * qq) = make_float4(o[d][0], o[d][1], o[d][2], o[d][3]);
    if (qq == 0) {
      float* ml = a.ws + AT_PS * a.B * a.T * a.nh * HD + 2 * row;
      ml[0] = m_run;
      ml[1] = l_tot;
    }
    return;
  }
  const float il = l_tot > 0.f ? 1.f / l_tot : 0.f;
  bf16* orow = (bf16*)a.out + (b * a.T + tq) * a.out_ld + head * HD;
#pragma unroll
  for (int d = 0; d < NO; ++d) {
    uint2 pk;
    pk.x = (uint32_t)f2bf(o[d][0] * il) | ((uint32_t)f2bf(o[d][1] * il) << 16);
    pk.y = (uint32_t)f2bf(o[d][2] * il) | ((uint32_t)f2bf(o[d][3] * il) << 16);
    *(uint2*)(orow + 16 * d + 4 * qq) = pk;
  }
}

// --------------------------------------------------------------------------------------------
// k_attn_w16p: k_attn_w16's blocks, tiles and pipeline at head dim 512, with the two waves of a query
// group (32 tokens x one head, 16 queries each) splitting the head elements of O instead of the
// queries. Each wave computes S and the softmax of its own 16 queries as in k_attn_w16, publishes its
// P (bf16), its per-query rescale factors and whether it raised its maximum to a double-buffered
// exchange in LDS, and after the block barrier reads its partner's. Its O accumulators hold head
// elements hf HD/2 .. hf HD/2 + HD/2 - 1 (hf = wave & 1) for both waves' queries (HD/32 + HD/32
// blocks, the same 128 registers as O of 16 queries over the whole head), so every V^T fragment read
// from LDS feeds two MFMAs (own P, partner's P): half the V reads of k_attn_w16 per MFMA. The partner's
// O half is rescaled only when the partner raised its maximum. At the end the normalisers are swapped
// through LDS and each wave writes its half of both queries' rows (the m and l of a split part come
// from the query's own wave).
template <int HD, bool RING>
__global__ __launch_bounds__(512, 1) void k_attn_w16p(AttnArgs a, int G, float sl2, AtSplit sp) {
  using L = AttnLdsW<HD>;
  typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
  constexpr int KB = L::KB;        // keys per tile
  constexpr int NKB = KB / 16;     // 16-key blocks of S per tile
  constexpr int NPV = KB / 32;     // 32-key steps of P V per tile
  constexpr int NOH = HD / 32;     // O blocks (16 head elements each) per query block in the wave's half
  constexpr int KS = HD / 32;      // k-steps of S (32 head elements each)
  constexpr int QG = 4;            // query groups per block, two waves each
  constexpr int NS = AttnTileW<HD>::NS;
  constexpr int NE = 4 * NKB;      // scores per lane per tile
  constexpr int RPW = KB / 8;      // tile rows staged by each wave
  static_assert(NS == 2, "K and V tiles alternate between two stages");
  static_assert(KS >= 8, "the softmax steps ride behind the S steps");
  __shared__ __attribute__((aligned(16))) bf16 lds[NS * L::STAGE];
  // the pair's exchange: P of each wave (two buffers), its queries' rescale factors and whether any
  // was raised, and at the end their normalisers
  __shared__ bf16x8_t px[2][8][NPV][64];
  __shared__ float ax[2][8][64];
  __shared__ int fx[2][8];
  __shared__ float lx[8][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 15, qq = lane >> 4;  // query of the lane within the wave; lane group
  const int nruns = (int)((a.T + 31) / 32);
  const int ngroups = nruns * G;
  const int nblk = (ngroups + QG - 1) / QG;
  int blk, part, nparts;
  const int64_t g = (int64_t)blockIdx.x % a.nkv, b = ((int64_t)blockIdx.x / a.nkv) % a.B;
  at_item((int)((int64_t)blockIdx.x / (a.nkv * a.B)), nblk, sp, blk, part, nparts);
  const int gi = blk * QG + (wave >> 1);
  const int run = gi / G;
  const int64_t head = g * G + gi % G;
  const int hf = wave & 1;                                    // which 16 queries; which half of O
  const int64_t tq0 = (int64_t)run * 32 + 16 * hf;            // the wave's first query token
  const int64_t tq = tq0 + ql;                                // this lane's query token
  const int64_t ptq = (int64_t)run * 32 + 16 * (1 - hf) + ql; // the partner wave's query in this lane
  const int64_t p0 = a.pos0[b];
  const bool qvalid = gi < ngroups && tq < a.T;
  const bool pvalid = gi < ngroups && ptq < a.T;
  const int64_t qi = p0 + tq;

  // block key range (union over its groups), as in k_attn_mfma
  const int g_first = blk * QG, g_last = (blk * QG + QG - 1) < ngroups - 1 ? blk * QG + QG - 1 : ngroups - 1;
  int64_t tlast = (int64_t)(g_last / G) * 32 + 31;
  if (tlast > a.T - 1) tlast = a.T - 1;
  const int64_t imin = p0 + (int64_t)(g_first / G) * 32, imax = p0 + tlast;
  const KeySpan ksp = key_span(a.bidir, a.sliding, a.window, a.cap, RING ? 1 : 0, p0, a.T);
  int64_t lob = imin - ksp.back;
  if (lob < ksp.kmin) lob = ksp.kmin;
  const int64_t hib = imax + ksp.fwd < ksp.kmax ? imax + ksp.fwd : ksp.kmax;
  const int64_t kstart = lob & ~(int64_t)(KB - 1);
  const int ntiles = hib >= lob ? (int)((hib - kstart) / KB + 1) : 0;
  const int it0 = part * ntiles / nparts, it1 = (part + 1) * ntiles / nparts;
  int64_t qlo = qi - ksp.back;
  if (qlo < ksp.kmin) qlo = ksp.kmin;
  const int64_t qhi = qi + ksp.fwd < hib ? qi + ksp.fwd : hib;
  // the lane's visible keys relative to the first tile, in 32 bits (none for an invalid query)
  const int vlo = qvalid ? (int)(qlo - kstart) : 0x7fffffff, vhi = qvalid ? (int)(qhi - kstart) : -1;
  // keys visible to every query of the wave (empty when some query of the wave is invalid)
  int64_t wlo_all, whi_all;
  {
    const int64_t first = p0 + tq0, last = p0 + tq0 + 15;
    wlo_all = last - ksp.back;
    if (wlo_all < lob) wlo_all = lob;
    whi_all = first + ksp.fwd < hib ? first + ksp.fwd : hib;
    if (!(gi < ngroups && tq0 + 15 < a.T)) { wlo_all = 1; whi_all = 0; }
  }
  // per-tile range tests in 32 bits, relative to the first tile's first key
  const int lob_r = (int)(lob - kstart), hib_r = (int)(hib - kstart);
  const int wlo_r = (int)(wlo_all - kstart), whi_r = wlo_all > whi_all ? -1 : (int)(whi_all - kstart);

  // Q fragments (B operand of S^T): query ql, head elements 32 s + 8 qq .. +7
  bf16x8_t qf[KS];
  {
    const bf16* qrow = (const bf16*)a.q + (b * a.T + (qvalid ? tq : 0)) * a.q_ld + (qvalid ? head : 0) * HD + 8 * qq;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 u = qvalid ? *(const uint4*)(qrow + 32 * s) : make_uint4(0, 0, 0, 0);
      qf[s] = *(bf16x8_t*)&u;
    }
  }
  // Q is in flight together with the first tiles: the prologue waits for both at once, before the key
  // loop (see k_attn_mfma for why the wait must not be left to the compiler)

  const bf16* Kb = (const bf16*)a.k + (b * a.nkv + g) * a.cap * HD;
  const bf16* Vb = (const bf16*)a.v + (b * a.nkv + g) * a.cap * HD;
  const at_rsrc rks = at_make_rsrc(Kb, a.cap * HD * 2), rvs = at_make_rsrc(Vb, a.cap * HD * 2);
  // Tile it into ring slot it % NS; rows RPW w .. RPW w + RPW - 1 from wave w (see k_attn_mfma for the
  // out-of-range tiles and the clamped rows).
  // Cache rows in 32 bits: the byte offsets of a cache fit the 31-bit buffer range (the descriptor's
  // size saturates there), so every row index that reaches a load does too.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int cap32 = (int)a.cap;
  const uint32_t lds_k = (uint32_t)(uintptr_t)(at_lds_void*)lds + (uint32_t)(RPW * wv * L::KLD * 2);
  const uint32_t lds_v = (uint32_t)(uintptr_t)(at_lds_void*)lds + L::KSZ * 2 + (uint32_t)(RPW * wv * L::VROW * 2);
  // K (isv false) or V rows of tile it into stage it % 2: rows RPW w .. RPW w + RPW - 1 from wave w
  // (see k_attn_mfma for the out-of-range tiles and the clamped rows).
  auto dma = [&](int it, bool isv) {
    const bool live = it < it1;
    const uint32_t so = (uint32_t)(it % NS) * L::STAGE * 2;
    const int64_t kb = kstart + (int64_t)it * KB + RPW * wv;  // the wave's first key of the tile
    const int rb = RING ? (int)kv_row(kb, a.cap, 1) : (int)(kb < a.cap ? kb : a.cap - 1);
    // The row's byte offset rides in the per-lane offset, so no scalar register written by a vector
    // instruction feeds the load (the compiler's hazard checks do not see into the assembly); the
    // scalar offset only marks a tile past the range.
    const uint32_t oob = live ? 0u : 0x80000000u;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      int cr;
      if (!RING) cr = rb + r < cap32 - 1 ? rb + r : cap32 - 1;  // keys past the cache clamp to its last row
      else if (cap32 >= RPW) cr = rb + r >= cap32 ? rb + r - cap32 : rb + r;
      else cr = (int)kv_row(kb + r, a.cap, 1);
      const uint32_t voff = (uint32_t)cr * (HD * 2) + (uint32_t)lane * 16;
      if (lane < HD / 8) {
        if (isv) at_dma16(rvs, voff, oob, lds_v + so + (uint32_t)(r * L::VROW * 2));
        else at_dma16(rks, voff, oob, lds_k + so + (uint32_t)(r * L::KLD * 2));
      }
    }
  };
  auto edge_tile = [&](int it) {
    const int kt = it * KB;
    return !(kt >= lob_r && kt + KB - 1 <= hib_r);
  };
  auto vclean = [&](int it, int buf) {
    const int kt = it * KB;
    bf16* vs = lds + buf * L::STAGE + L::KSZ;
    for (int u = tid; u < KB * (HD / 8); u += 512) {
      const int row = u / (HD / 8);
      const int key = kt + row;
      if (key < lob_r || key > hib_r) *(uint4*)(vs + row * L::VROW + 8 * (u % (HD / 8))) = make_uint4(0, 0, 0, 0);
    }
  };

  // O^T of the wave's half of the head elements (hf HD/2 + 16 d + 4 qq + 0..3 in lane (ql, qq)) for its
  // own 16 queries and for the partner wave's 16
  f32x4_t oo[NOH], op[NOH];
#pragma unroll
  for (int d = 0; d < NOH; ++d) oo[d] = op[d] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int kfo = ql * L::KLD + 8 * qq;                                   // K: key row ql, chunk qq
  const int vfo = (4 * qq + (ql >> 2)) * L::VROW + 4 * (ql & 3) + hf * (HD / 2);  // V^T: rows 4qq + ql/4

  constexpr int PK = 2;
  auto s_tile = [&](const bf16* ks, f32x4_t (&acc)[NKB], auto&& step) {
    bf16x8_t kw[NKB][PK];
#pragma unroll
    for (int k = 0; k < NKB; ++k) {
      acc[k] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < PK; ++j) kw[k][j] = *(const bf16x8_t*)(ks + kfo + 16 * k * L::KLD + 32 * j);
    }
#pragma unroll
    for (int st = 0; st < KS; ++st) {
#pragma unroll
      for (int k = 0; k < NKB; ++k) {
        acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kw[k][st % PK], qf[st], acc[k], 0, 0, 0);
        if (st + PK < KS) kw[k][st % PK] = *(const bf16x8_t*)(ks + kfo + 16 * k * L::KLD + 32 * (st + PK));
      }
      step(st);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  float sc[NE];
  float mt = -INFINITY, m_new = -INFINITY, m_use = 0.f, psum = 0.f;
  bool raise = false, full = false;
  int kt = 0;
  bf16x8_t pb[NPV];
  auto smax_step = [&](int st) {
    if (st == 0) {
      // the maximum of the unscaled scores (sl2 > 0: the host takes only positive scales here); the
      // scale rides in the exponential's fused multiply-add
      mt = -INFINITY;
      if (full) {
#pragma unroll
        for (int r = 0; r < NE; ++r) mt = fmaxf(mt, sc[r]);
      } else {
#pragma unroll
        for (int r = 0; r < NE; ++r) {
          const int kk = kt + 16 * (r >> 2) + 4 * qq + (r & 3);
          const bool vis = kk >= vlo && kk <= vhi;
          const float x = vis ? sc[r] : -INFINITY;
          sc[r] = x;
          mt = fmaxf(mt, x);
        }
      }
    } else if (st == 1) {
      mt = at_max_xor16(mt);
    } else if (st == 2) {
      mt = at_max_xor32(mt) * sl2;
      raise = mt > m_run + 32.f;
      m_new = raise ? mt : m_run;
      m_use = m_new == -INFINITY ? 0.f : m_new;
      psum = 0.f;
    } else {
#pragma unroll
      for (int r = 0; r < NE; ++r)
        if (3 + r * (KS - 3) / NE == st) {
          const float pr = __builtin_amdgcn_exp2f(fmaf(sc[r], sl2, -m_use));
          psum += pr;
          pb[r / 8][r % 8] = (__bf16)pr;
        }
    }
  };

  // Tile it, in this order: the softmax of tile it behind the S MFMAs of tile it + 1 (MORE); P and the
  // rescale factors to the pair's exchange; the block barrier (tile it's V, tile it + 2's K and the
  // partner's P all in place; every wave past the last tile's reads); the loads of tile it + 3's K and
  // tile it + 1's V into the halves those reads freed; then O^T += V^T P^T for both waves' queries,
  // each V^T fragment feeding two MFMAs.
  f32x4_t sacc[NKB], snext[NKB];
  auto iter = [&](int it, auto more_t) {
    constexpr bool MORE = decltype(more_t)::value;
    const int cur = it % NS, nx = (it + 1) % NS;
    kt = it * KB;
    full = kt >= wlo_r && kt + KB - 1 <= whi_r;
#pragma unroll
    for (int k = 0; k < NKB; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * k + i] = sacc[k][i];
    if constexpr (MORE) {
      __builtin_amdgcn_s_setprio(1);
      s_tile(lds + nx * L::STAGE, snext, smax_step);
      __builtin_amdgcn_s_setprio(0);
    } else {
#pragma unroll
      for (int st = 0; st < KS; ++st) smax_step(st);
    }
    const bool rs = __builtin_amdgcn_ballot_w64(raise) != 0;
    float alpha = 1.f;
    if (rs) {
      alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < NOH; ++d) oo[d] *= alpha;
    }
    l_run += psum;
    m_run = m_new;
    const int xb = it & 1;
#pragma unroll
    for (int h = 0; h < NPV; ++h) px[xb][wave][h][lane] = pb[h];
    ax[xb][wave][lane] = alpha;
    if (lane == 0) fx[xb][wave] = rs ? 1 : 0;
    G4_ATT_WAIT_VMCNT(0);
    __syncthreads();
    if (MORE) {
      dma(it + 3, false);
      dma(it + 1, true);
    }
    if (it > it0 && edge_tile(it)) {
      vclean(it, cur);
      __syncthreads();
    }
    if (MORE) {
#pragma unroll
      for (int k = 0; k < NKB; ++k) sacc[k] = snext[k];
    }
    bf16x8_t pp[NPV];
#pragma unroll
    for (int h = 0; h < NPV; ++h) pp[h] = px[xb][wave ^ 1][h][lane];
    if (fx[xb][wave ^ 1]) {
      const float pa = ax[xb][wave ^ 1][lane];
#pragma unroll
      for (int d = 0; d < NOH; ++d) op[d] *= pa;
    }
    const bf16* vs = lds + cur * L::STAGE + L::KSZ;
    constexpr int PV = 4;
    constexpr int NM = NPV * NOH;
    auto vread = [&](int j) {
      const int h = j / NOH, d = j % NOH;
      const bf16* va = vs + vfo + 32 * h * L::VROW + 16 * d;
      const bf16x4_t lo = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((at_lds_v4s*)(at_lds_void*)va));
      const bf16x4_t hi = __builtin_bit_cast(
          bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((at_lds_v4s*)(at_lds_void*)(va + 16 * L::VROW)));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8_t vw[PV];
#pragma unroll
    for (int j = 0; j < PV; ++j) vw[j] = vread(j);
#pragma unroll
    for (int j = 0; j < NM; ++j) {
      oo[j % NOH] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vw[j % PV], pb[j / NOH], oo[j % NOH], 0, 0, 0);
      op[j % NOH] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vw[j % PV], pp[j / NOH], op[j % NOH], 0, 0, 0);
      if (j + PV < NM) vw[j % PV] = vread(j + PV);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (it1 > it0) {
    dma(it0, false);
    dma(it0, true);
    dma(it0 + 1, false);
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" : : "v"(qf[s]));
    G4_ATT_WAIT_VMCNT(0);
    __syncthreads();
    if (edge_tile(it0)) vclean(it0, it0 % NS);
    s_tile(lds + (it0 % NS) * L::STAGE, sacc, [](int) {});
    __syncthreads();  // tile it0's K rows are read: its half takes tile it0 + 2's
    dma(it0 + 2, false);
    int it = it0;
    for (; it + 1 < it1; ++it) iter(it, std::true_type{});
    iter(it, std::false_type{});
  }

  // normalisers of the pair's queries (lane (ql, qq) holds its query's sum after the two steps)
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  lx[wave][lane] = l_tot;
  __syncthreads();
  const float l_par = lx[wave ^ 1][lane];
  // lane holds head elements hf HD/2 + 16 d + 4 qq + 0..3 of queries tq (own) and ptq (partner)
  auto emit = [&](const f32x4_t (&o)[NOH], int64_t q, float lt, float m, bool owner) {
    if (nparts > 1) {
      const int64_t row = ((part * a.B + b) * a.T + q) * a.nh + head;
      float* po = a.ws + row * HD + hf * (HD / 2);
#pragma unroll
      for (int d = 0; d < NOH; ++d) *(float4*)(po + 16 * d + 4 * qq) = make_float4(o[d][0], o[d][1], o[d][2], o[d][3]);
      if (owner && qq == 0) {
        float* ml = a.ws + AT_PS * a.B * a.T * a.nh * HD + 2 * row;
        ml[0] = m;
        ml[1] = lt;
      }
      return;
    }
    const float il = lt > 0.f ? 1.f / lt : 0.f;
    bf16* orow = (bf16*)a.out + (b * a.T + q) * a.out_ld + head * HD + hf * (HD / 2);
#pragma unroll
    for (int d = 0; d < NOH; ++d) {
      uint2 pk;
      pk.x = (uint32_t)f2bf(o[d][0] * il) | ((uint32_t)f2bf(o[d][1] * il) << 16);
      pk.y = (uint32_t)f2bf(o[d][2] * il) | ((uint32_t)f2bf(o[d][3] * il) << 16);
      *(uint2*)(orow + 16 * d + 4 * qq) = pk;
    }
  };
  if (qvalid) emit(oo, tq, l_tot, m_run, true);
  if (pvalid) emit(op, ptq, l_par, 0.f, false);
}

// Merges the key-share partials of each split query row: O = sum_p O_p 2^(m_p - m) / sum_p l_p 2^(m_p - m)
// with m = max_p m_p (exp2 domain), parts in order; a row that saw no key stays zero. One wave per
// (sequence, query token >= tq_lo, head); the row's part count comes from its query block (AtSplit).
template <int HD>
__global__ __launch_bounds__(64) void k_attn_merge_split(AttnArgs a, int64_t tq_lo, int G, int QG, AtSplit sp) {
  constexpr int EPL = HD / 64;
  const int64_t tq = tq_lo + blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int blk = (int)(((tq / 32) * G + head % G) / QG);
  const int np = 1 + (blk >= sp.th1) + (blk >= sp.th2) + (blk >= sp.th3);
  if (np == 1) return;  // an unsplit block wrote this row itself (with 8 heads per kv head a run's heads
                        // may straddle the first split block)
  const float* ml = a.ws + AT_PS * a.B * a.T * a.nh * HD;
  float mp[AT_PS], lp[AT_PS], m = -INFINITY;
#pragma unroll
  for (int p = 0; p < AT_PS; ++p) {
    const int64_t row = ((p * a.B + b) * a.T + tq) * a.nh + head;
    mp[p] = p < np ? ml[2 * row] : -INFINITY;
    lp[p] = p < np ? ml[2 * row + 1] : 0.f;
    m = fmaxf(m, mp[p]);
  }
  float w[AT_PS], den = 0.f;
#pragma unroll
  for (int p = 0; p < AT_PS; ++p) {
    w[p] = (p < np && m != -INFINITY) ? __builtin_amdgcn_exp2f(mp[p] - m) : 0.f;
    den += lp[p] * w[p];
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll
  for (int p = 0; p < AT_PS; ++p)
    if (p < np) {
      const float* pp = a.ws + (((p * a.B + b) * a.T + tq) * a.nh + head) * HD + lane * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += pp[e] * w[p];
    }
  bf16* out = (bf16*)a.out + (b * a.T + tq) * a.out_ld + head * HD + lane * EPL;
#pragma unroll
  for (int e = 0; e < EPL; e += 2)
    *(uint32_t*)(out + e) = (uint32_t)f2bf(acc[e] * inv) | ((uint32_t)f2bf(acc[e + 1] * inv) << 16);
}

// Query blocks of one launch and their key split (AtSplit). Only a launch with fewer blocks than the
// device keeps busy splits (twice the CUs for causal full layers, whose blocks differ in length; the
// CUs otherwise). Candidate splits give block b min(AT_PS, ceil(tiles_b / t)) parts for a tile target
// t, made non-decreasing in the block index (the latest causal queries have the longest key ranges),
// so three thresholds describe each. The plan keeps the candidate (or no split) whose items, dispatched
// in the kernels' order onto the earliest free CU, finish first, counting each part of a split block
// HD/512 of a tile more for its partial and the merge. Tile counts assume the call starts at position
// 0 (positions live on the device): any split gives the same result, this one balances the usual
// case. Plans are cached per shape. Returns false if the shape is not the MFMA path's.
struct AtPlanKey {
  int64_t B, T, nh, nkv, hd, window, cus;
  int32_t sliding, bidir;
  bool operator==(const AtPlanKey& o) const {
    return B == o.B && T == o.T && nh == o.nh && nkv == o.nkv && hd == o.hd && window == o.window && cus == o.cus &&
           sliding == o.sliding && bidir == o.bidir;
  }
};

static AtSplit at_choose_split(const AtPlanKey& k, int nblk, int64_t G, int64_t ngroups, int QG) {
  // the kernel's tile: 32 keys, 64 for the 16-query kernel at head dim 256
  const int64_t kb = k.hd == 256 ? AttnTileW<256>::KB : AT_KB;
  std::vector<int64_t> tl(nblk);
  int64_t maxt = 1;
  for (int b = 0; b < nblk; ++b) {  // key tiles of block b for a call from position 0
    const int64_t g0 = (int64_t)b * QG, g1 = (g0 + QG < ngroups ? g0 + QG : ngroups) - 1;
    const int64_t imin = (g0 / G) * 32, imax = (g1 / G) * 32 + 31 < k.T - 1 ? (g1 / G) * 32 + 31 : k.T - 1;
    int64_t lo = 0, hi = imax;
    if (k.bidir) {
      if (k.sliding) { lo = imin - k.window; hi = imax + k.window < k.T - 1 ? imax + k.window : k.T - 1; }
      else hi = k.T - 1;
    } else if (k.sliding) {
      lo = imin - k.window + 1;
    }
    if (lo < 0) lo = 0;
    tl[b] = (hi - (lo & ~(int64_t)(kb - 1))) / kb + 1;
    if (tl[b] > maxt) maxt = tl[b];
  }
  const int64_t copies = k.nkv * k.B;
  const double part_cost = (double)k.hd / 512.0 * (double)AT_KB / (double)kb;
  auto split_for = [&](int64_t t) {
    AtSplit sp{nblk, nblk, nblk};
    int prev = 1;
    for (int b = 0; b < nblk; ++b) {
      int64_t p = (tl[b] + t - 1) / t;
      if (p > AT_PS) p = AT_PS;
      if (p < prev) p = prev;
      prev = (int)p;
      if (p >= 2 && sp.th1 == nblk) sp.th1 = b;
      if (p >= 3 && sp.th2 == nblk) sp.th2 = b;
      if (p >= 4 && sp.th3 == nblk) sp.th3 = b;
    }
    return sp;
  };
  auto makespan = [&](const AtSplit& sp) {
    std::priority_queue<double, std::vector<double>, std::greater<double>> cu;
    for (int64_t c = 0; c < k.cus; ++c) cu.push(0.0);
    const int th[5] = {0, sp.th1, sp.th2, sp.th3, nblk};
    double end = 0.0;
    for (int np = AT_PS; np >= 1; --np)  // the kernels' item order: 4-part blocks from the last down, ...
      for (int b = th[np] - 1; b >= th[np - 1]; --b)
        for (int p = 0; p < np; ++p) {
          const double dur = (double)((p + 1) * tl[b] / np - p * tl[b] / np) + (np > 1 ? part_cost : 0.0);
          for (int64_t c = 0; c < copies; ++c) {
            const double t0 = cu.top();
            cu.pop();
            cu.push(t0 + dur);
            if (t0 + dur > end) end = t0 + dur;
          }
        }
    return end;
  };
  AtSplit best{nblk, nblk, nblk};
  double best_ms = makespan(best);
  const int64_t tmin = (maxt + AT_PS - 1) / AT_PS, stride = (maxt - tmin) / 48 + 1;
  for (int64_t t = tmin; t < maxt; t += stride) {
    const AtSplit sp = split_for(t);
    const double ms = makespan(sp);
    if (ms < best_ms - 1e-9) { best_ms = ms; best = sp; }
  }
  return best;
}

static bool attn_plan(int64_t B, int64_t T, int64_t nh, int64_t nkv, int64_t hd, int32_t sliding, int32_t bidir,
                      int64_t window, int* nblk, AtSplit* sp, int64_t* tq_lo) {
  if (nkv <= 0 || nh % nkv) return false;
  const int64_t G = nh / nkv;
  if (!(G == 1 || G == 2 || G == 4 || G == 8) || !(hd == 128 || hd == 256 || hd == 512)) return false;
  const int64_t runs = (T + 31) / 32, cus = device_cus();
  const int QG = 4;  // query groups (head x 32 tokens) per block
  const int64_t ngroups = runs * G;
  *nblk = (int)((ngroups + QG - 1) / QG);
  *sp = AtSplit{*nblk, *nblk, *nblk};
  const int64_t blocks = (int64_t)*nblk * nkv * B;
  if ((sliding || bidir) ? blocks < cus : blocks < 2 * cus) {
    static thread_local std::vector<std::pair<AtPlanKey, AtSplit>> cache;
    const AtPlanKey key{B, T, nh, nkv, hd, (sliding || bidir) ? window : 0, cus, sliding, bidir};
    bool hit = false;
    for (const auto& e : cache)
      if (e.first == key) { *sp = e.second; hit = true; break; }
    if (!hit) {
      *sp = at_choose_split(key, *nblk, G, ngroups, QG);
      if (cache.size() >= 64) cache.erase(cache.begin());
      cache.emplace_back(key, *sp);
    }
  }
  *tq_lo = ((int64_t)sp->th1 * QG / G) * 32;
  return true;
}

static size_t attn_split_bytes(int64_t B, int64_t T, int64_t nh, int64_t hd) {
  return (size_t)AT_PS * B * T * nh * (hd + 2) * 4;
}

// Scratch for the key-split partials of any launch attn_mfma may make for these shapes (the largest
// split trigger is the causal full layer's).
size_t attn_prefill_ws(int64_t B, int64_t T, int64_t nh, int64_t nkv, int64_t hd) {
  if (nkv <= 0 || nh % nkv) return 0;
  const int64_t nblk = ((T + 31) / 32 * (nh / nkv) + 3) / 4;
  return nblk * nkv * B < 2 * device_cus() ? attn_split_bytes(B, T, nh, hd) : 0;
}

// bf16, head_dim 128/256/512, groups of 1, 2, 4 or 8 query heads per kv head, 16-byte aligned rows.
bool attn_mfma(const AttnArgs& a, hipStream_t s, g4_status* st) {
  if ((a.q_ld | a.out_ld) & 7) return false;
  // the 16-query kernels take the maximum of the unscaled scores: positive, finite scales only
  if (a.hd != 128 && !(a.scale > 0.f && a.scale < INFINITY)) return false;
  if (((uintptr_t)a.q | (uintptr_t)a.k | (uintptr_t)a.v | (uintptr_t)a.out) & 15) return false;
  int nblk = 0;
  AtSplit sp{};
  int64_t tq_lo = 0;
  if (!attn_plan(a.B, a.T, a.nh, a.nkv, a.hd, a.sliding, a.bidir, a.window, &nblk, &sp, &tq_lo)) return false;
  if (!a.ws || a.ws_bytes < attn_split_bytes(a.B, a.T, a.nh, a.hd) || ((uintptr_t)a.ws & 15)) {
    sp.th1 = sp.th2 = sp.th3 = nblk;  // no scratch: no split
    tq_lo = a.T;
  }
  const int64_t G = a.nh / a.nkv;
  const int items = nblk + (nblk - sp.th1) + (nblk - sp.th2) + (nblk - sp.th3);
  dim3 grid((unsigned)((int64_t)items * a.nkv * a.B));
  const float sl2 = a.scale * 1.4426950408889634f;
  if (a.hd == 128) hipLaunchKernelGGL((k_attn_mfma<128>), grid, dim3(256), 0, s, a, (int)G, sl2, sp);
  else if (a.hd == 256 && a.ring) hipLaunchKernelGGL((k_attn_w16<256, true>), grid, dim3(512), 0, s, a, (int)G, sl2, sp);
  else if (a.hd == 256) hipLaunchKernelGGL((k_attn_w16<256, false>), grid, dim3(512), 0, s, a, (int)G, sl2, sp);
  else if (a.ring) hipLaunchKernelGGL((k_attn_w16p<512, true>), grid, dim3(512), 0, s, a, (int)G, sl2, sp);
  else hipLaunchKernelGGL((k_attn_w16p<512, false>), grid, dim3(512), 0, s, a, (int)G, sl2, sp);
  if ((*st = check_launch("attn_mfma")) != G4_OK || sp.th1 == nblk || tq_lo >= a.T) return true;
  dim3 gm((unsigned)(a.T - tq_lo), (unsigned)a.nh, (unsigned)a.B);
  if (a.hd == 128) hipLaunchKernelGGL((k_attn_merge_split<128>), gm, dim3(64), 0, s, a, tq_lo, (int)G, 4, sp);
  else if (a.hd == 256) hipLaunchKernelGGL((k_attn_merge_split<256>), gm, dim3(64), 0, s, a, tq_lo, (int)G, 4, sp);
  else hipLaunchKernelGGL((k_attn_merge_split<512>), gm, dim3(64), 0, s, a, tq_lo, (int)G, 4, sp);
  *st = check_launch("attn_merge_split");
  return true;
}

}  // namespace g4
