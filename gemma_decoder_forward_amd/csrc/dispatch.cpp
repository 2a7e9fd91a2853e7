// Kernel selection: which of the library's kernels runs a given GEMM / attention call.
#include "g4_internal.h"

namespace g4 {

g4_status gemm(const GemmArgs& a, int32_t dtype, hipStream_t s) {
  if (a.M == 0) return G4_OK;
  g4_status st = G4_OK;
  if (dtype == G4_BF16 && gemm_mfma(a, s, &st)) return st;
  return gemm_simt(a, dtype, s);
}

size_t gemm_ws(int64_t, int64_t, int64_t, int32_t) { return 0; }

g4_status attn_prefill(const AttnArgs& a, int32_t dtype, hipStream_t s) {
  if (a.B * a.T == 0) return G4_OK;
  g4_status st = G4_OK;
  if (dtype == G4_BF16 && attn_mfma(a, s, &st)) return st;
  return attn_rowwise(a, dtype, s);
}

}  // namespace g4
