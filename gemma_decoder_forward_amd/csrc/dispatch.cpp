// Kernel selection: which of the library's kernels runs a given GEMM / attention call.
#include "g4_internal.h"

namespace g4 {

static g4_status gemm_one(const GemmArgs& a, int32_t dtype, hipStream_t s) {
  g4_status st = G4_OK;
  if (dtype == G4_BF16 && gemm_mfma(a, s, &st)) return st;
  return gemm_simt(a, dtype, s);
}

g4_status gemm(const GemmArgs& a, int32_t dtype, hipStream_t s) {
  if (a.M == 0) return G4_OK;
  if (a.epi == EPI_SOFTCAP) return fail(G4_EUNSUP, "gemm: the softcap epilogue is reached through its own routes only");
  g4_status st = G4_OK;
  const int nseg = a.nseg > 0 ? a.nseg : 1;
  // few token rows (decode): stream the weights once, all segments in one launch -- except wide, short
  // products above 16 rows, where the tiled kernel has enough tiles and the few-row blocks would
  // re-stage as many activation bytes as weight bytes (20480 x 2560 weights at 32 rows: 23.5 vs 32.4 us)
  const int64_t n_all = a.epi == EPI_GEGLU ? 2 * a.N : a.N;
  const bool wide = a.M > 16 && n_all >= 16384 && a.K <= 4096;
  if (dtype == G4_BF16 && a.M <= 64 && a.splits <= 1 && !wide) {
    const void* segs[3];
    int64_t rows[3];
    int n;
    if (a.epi == EPI_GEGLU) {
      segs[0] = a.B; segs[1] = a.B2; rows[0] = rows[1] = a.N; n = 2;
    } else if (a.nseg > 0) {
      for (int i = 0; i < nseg; ++i) { segs[i] = a.segB[i]; rows[i] = a.seg_rows[i]; }
      n = nseg;
    } else {
      segs[0] = a.B; rows[0] = a.N; n = 1;
    }
    if (gemm_skinny(a, segs, rows, n, a.ws, a.ws_bytes, s, &st)) return st;
  }
  if (a.nseg <= 1) {
    GemmArgs b = a;
    if (a.nseg == 1) b.B = a.segB[0];
    return gemm_one(b, dtype, s);
  }
  // several B matrices: one MFMA launch over all of them when each is a whole number of tiles ...
  if (dtype == G4_BF16) {
    GemmArgs b = a;
    b.B = a.segB[0];
    if (gemm_mfma(b, s, &st)) return st;
  }
  // ... else one launch per segment, each writing its own column range of C
  int64_t col = 0;
  for (int i = 0; i < nseg; ++i) {
    GemmArgs b = a;
    b.nseg = 0;
    b.B = a.segB[i];
    b.N = a.seg_rows[i];
    b.C = (char*)a.C + col * (a.c_dtype == G4_F32 ? 4 : 2);
    if ((st = gemm_one(b, dtype, s)) != G4_OK) return st;
    col += a.seg_rows[i];
  }
  return G4_OK;
}

size_t gemm_ws(int64_t, int64_t, int64_t, int32_t) { return 0; }

int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      return 256;  // no device visible (host-only sizing): the MI355X count
    cus = n;
  }
  return cus;
}

g4_status attn_prefill(const AttnArgs& a, int32_t dtype, hipStream_t s) {
  if (a.B * a.T == 0) return G4_OK;
  g4_status st = G4_OK;
  if (dtype == G4_BF16 && attn_mfma(a, s, &st)) return st;
  return attn_rowwise(a, dtype, s);
}

}  // namespace g4
