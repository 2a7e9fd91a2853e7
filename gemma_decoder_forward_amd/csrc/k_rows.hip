// Row kernels: the fused RMSNorm residual tail, per-head norm + NeoX RoPE (into a cache slot or in
// place), the scaled embedding gather and the per-layer-input combination.
//
// Every one is HBM-bound: one pass over its rows, 16-byte-friendly contiguous access along the row,
// float32 arithmetic, block or wave reductions with cross-lane shuffles.
#include "g4_internal.h"

namespace g4 {

// --------------------------------------------------------------------------------------------
// Fused RMSNorm tail (cortiq-engine `rms`/`rms_plain` and the sandwich residual adds of `g4e_forward`).
// One 256-thread block per row; values stay in registers between the two reductions.
// --------------------------------------------------------------------------------------------
template <typename TX, typename T, int VPT>
__global__ __launch_bounds__(256) void k_rownorm(const TX* __restrict__ x, int parts, int64_t part_stride,
                                                 const T* __restrict__ w, T* __restrict__ y,
                                                 float* __restrict__ res, float res_scale,
                                                 const T* __restrict__ w_next, T* __restrict__ y_next,
                                                 int64_t dim, float eps) {
  __shared__ float sh[32];
  const int64_t row = blockIdx.x;
  const TX* xr = x + row * dim;
  // Every operand of the row is loaded up front, so the row costs one memory round trip, not three.
  float v[VPT], rv[VPT], wv[VPT], wn[VPT];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int64_t c = threadIdx.x + (int64_t)i * 256;
    float s = 0.f;
    rv[i] = 0.f;
    wv[i] = wn[i] = 1.f;
    if (c < dim) {
      for (int p = 0; p < parts; ++p) s += ldf(xr + p * part_stride + c);
      if (res) rv[i] = res[row * dim + c];
      if (w) wv[i] = ldf(w + c);
      if (w_next) wn[i] = ldf(w_next + c);
    }
    v[i] = s;
    ss += s * s;
  }
  ss = block_sum<256>(ss, sh);
  const float inv = 1.f / sqrtf(ss / (float)dim + eps);
  float ss2 = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int64_t c = threadIdx.x + (int64_t)i * 256;
    if (c < dim) {
      const float n = v[i] * inv * wv[i];
      if (y) stf(y + row * dim + c, n);
      if (res) {
        const float r = (rv[i] + n) * res_scale;
        res[row * dim + c] = r;
        v[i] = r;
        ss2 += r * r;
      }
    }
  }
  if (y_next) {
    float inv2 = 1.f;
    if (w_next) {
      ss2 = block_sum<256>(ss2, sh);
      inv2 = 1.f / sqrtf(ss2 / (float)dim + eps);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t c = threadIdx.x + (int64_t)i * 256;
      if (c < dim) stf(y_next + row * dim + c, w_next ? v[i] * inv2 * wn[i] : v[i]);
    }
  }
}

// 4 consecutive values as float (16-byte float or 8-byte bf16 loads) and back.
__device__ __forceinline__ float4 ld4(const float* p) { return *(const float4*)p; }
__device__ __forceinline__ float4 ld4(const bf16* p) {
  const uint2 u = *(const uint2*)p;
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ void st4(float* p, float4 v) { *(float4*)p = v; }
__device__ __forceinline__ void st4(bf16* p, float4 v) {
  *(uint2*)p = make_uint2((uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16), (uint32_t)f2bf(v.z) | ((uint32_t)f2bf(v.w) << 16));
}
__device__ __forceinline__ float4 operator+(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }
__device__ __forceinline__ float4 operator*(float4 a, float4 b) { return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w); }
__device__ __forceinline__ float4 operator*(float4 a, float s) { return make_float4(a.x * s, a.y * s, a.z * s, a.w * s); }
__device__ __forceinline__ float dot4(float4 a) { return a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w; }

// A row of `bytes` bytes as a buffer: a load past its end, or from a NULL row, reads zero and moves no
// data. Loads through it need no branch around them, so the compiler keeps them all in flight together
// (a branch per optional operand would put a wait for memory at every join).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, p ? (int)bytes : 0, 0x00020000);
}
// values c .. c+3 of a buffer row of floats / bf16s
__device__ __forceinline__ float4 bld4(__amdgpu_buffer_rsrc_t r, const float*, int64_t c) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(c * 4), 0, 0);
  const uint4 u = *(const uint4*)&v;
  return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}
__device__ __forceinline__ float4 bld4(__amdgpu_buffer_rsrc_t r, const bf16*, int64_t c) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)(c * 2), 0, 0);
  const uint2 u = *(const uint2*)&v;
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}

// The same tail for dim % 4 == 0 with 4-wide loads, for launches with few rows (decode), where the row's
// latency is the cost: every load goes through a row buffer (above), the residual and both weights in
// one batch and the split-K slices eight at a time, so a row costs one memory round trip per eight
// slices. Slices are added in slice order.
template <typename TX, typename T, int V4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4))) void k_rownorm4(const TX* __restrict__ x, int parts, int64_t part_stride,
                                                  const T* __restrict__ w, T* __restrict__ y,
                                                  float* __restrict__ res, float res_scale,
                                                  const T* __restrict__ w_next, T* __restrict__ y_next,
                                                  int64_t dim, float eps) {
  __shared__ float sh[32];
  const int64_t row = blockIdx.x;
  const TX* xr = x + row * dim;
  const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
  const auto rr = row_rsrc(res ? res + row * dim : nullptr, dim * 4);
  const auto rw = row_rsrc(w, dim * (int64_t)sizeof(T)), rn = row_rsrc(w_next, dim * (int64_t)sizeof(T));
  float4 v[V4], rv[V4], wv[V4], wn[V4];
#pragma unroll
  for (int i = 0; i < V4; ++i) v[i] = zero;
  for (int p = 0; p < parts; p += 8) {
    __amdgpu_buffer_rsrc_t rx[8];  // slices past the last read zero
#pragma unroll
    for (int j = 0; j < 8; ++j)
      rx[j] = row_rsrc(p + j < parts ? xr + (int64_t)(p + j) * part_stride : nullptr, dim * (int64_t)sizeof(TX));
    float4 t[V4][8];
#pragma unroll
    for (int i = 0; i < V4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) t[i][j] = bld4(rx[j], x, 4 * (threadIdx.x + (int64_t)i * 256));
    if (p == 0)  // the other operands ride behind the first slices
#pragma unroll
      for (int i = 0; i < V4; ++i) {
        const int64_t c = 4 * (threadIdx.x + (int64_t)i * 256);
        rv[i] = bld4(rr, (const float*)nullptr, c);
        wv[i] = bld4(rw, w, c);
        wn[i] = bld4(rn, w_next, c);
      }
#pragma unroll
    for (int i = 0; i < V4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i] = v[i] + t[i][j];
  }
  // a missing weight read as zero and stands for ones
  const float w1 = w ? 0.f : 1.f, n1 = w_next ? 0.f : 1.f;
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    wv[i] = wv[i] + make_float4(w1, w1, w1, w1);
    wn[i] = wn[i] + make_float4(n1, n1, n1, n1);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < V4; ++i) ss += dot4(v[i]);
  ss = block_sum<256>(ss, sh);
  const float inv = 1.f / sqrtf(ss / (float)dim + eps);
  float ss2 = 0.f;
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    const int64_t c = 4 * (threadIdx.x + (int64_t)i * 256);
    if (c < dim) {
      const float4 n = v[i] * inv * wv[i];
      if (y) st4(y + row * dim + c, n);
      if (res) {
        const float4 r = (rv[i] + n) * res_scale;
        st4(res + row * dim + c, r);
        v[i] = r;
        ss2 += dot4(r);
      }
    }
  }
  if (y_next) {
    float inv2 = 1.f;
    if (w_next) {
      ss2 = block_sum<256>(ss2, sh);
      inv2 = 1.f / sqrtf(ss2 / (float)dim + eps);
    }
#pragma unroll
    for (int i = 0; i < V4; ++i) {
      const int64_t c = 4 * (threadIdx.x + (int64_t)i * 256);
      if (c < dim) st4(y_next + row * dim + c, w_next ? v[i] * inv2 * wn[i] : v[i]);
    }
  }
}

// Four consecutive values of a buffer row as loaded (8 bytes of bf16, 16 of float), converted at use.
template <typename T> struct Raw4;
template <> struct Raw4<float> { uint4 u; };
template <> struct Raw4<bf16> { uint2 u; };
__device__ __forceinline__ Raw4<float> braw4(__amdgpu_buffer_rsrc_t r, const float*, int64_t c) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(c * 4), 0, 0);
  return Raw4<float>{*(const uint4*)&v};
}
__device__ __forceinline__ Raw4<bf16> braw4(__amdgpu_buffer_rsrc_t r, const bf16*, int64_t c) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)(c * 2), 0, 0);
  return Raw4<bf16>{*(const uint2*)&v};
}
__device__ __forceinline__ float4 cvt4(Raw4<float> r) {
  return make_float4(__uint_as_float(r.u.x), __uint_as_float(r.u.y), __uint_as_float(r.u.z), __uint_as_float(r.u.w));
}
__device__ __forceinline__ float4 cvt4(Raw4<bf16> r) {
  return make_float4(__uint_as_float(r.u.x << 16), __uint_as_float(r.u.x & 0xffff0000u), __uint_as_float(r.u.y << 16),
                     __uint_as_float(r.u.y & 0xffff0000u));
}

// The same tail with one wave per row (four rows per block) for launches with many rows: the two
// reductions are wave reductions with no block barrier, and the row's loads (the first split-K slice
// and the residual) are all issued before the first wait, through row buffers. Further slices come
// one per round trip, added in slice order: a batch of slices held registers enough to cost a wave
// per SIMD, and three waves per SIMD keep more rows in flight than the saved round trips.
template <typename TX, typename T, int V>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(V <= 10 ? 3 : 1))) void k_rownorm_w(const TX* __restrict__ x, int parts, int64_t part_stride,
                                                   const T* __restrict__ w, T* __restrict__ y, float* __restrict__ res,
                                                   float res_scale, const T* __restrict__ w_next, T* __restrict__ y_next,
                                                   int64_t rows, int64_t dim, float eps) {
  const int lane = threadIdx.x & 63;
  // wave-uniform row (rows < 2^31): the row buffers' descriptors stay in scalar registers
  const int64_t row = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
  if (row >= rows) return;
  const TX* xr = x + row * dim;
  const int64_t xbytes = dim * (int64_t)sizeof(TX), wbytes = dim * (int64_t)sizeof(T);
  const auto rx = row_rsrc(xr, xbytes), rr = row_rsrc(res ? res + row * dim : nullptr, dim * 4);
  Raw4<TX> xa[V];
  Raw4<float> ra[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int64_t c = 4 * (lane + 64 * i);
    xa[i] = braw4(rx, x, c);
    ra[i] = braw4(rr, (const float*)nullptr, c);
  }
  float4 v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = cvt4(xa[i]);
  for (int p = 1; p < parts; ++p) {
    const auto rp = row_rsrc(xr + (int64_t)p * part_stride, xbytes);
    Raw4<TX> t[V];
#pragma unroll
    for (int i = 0; i < V; ++i) t[i] = braw4(rp, x, 4 * (lane + 64 * i));
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = v[i] + cvt4(t[i]);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) ss += dot4(v[i]);
  // the weights (shared by every row, so mostly cache hits) after the first reduction
  const auto rw = row_rsrc(w, wbytes), rn = row_rsrc(w_next, wbytes);
  Raw4<T> wa[V], na[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    wa[i] = braw4(rw, w, 4 * (lane + 64 * i));
    na[i] = braw4(rn, w_next, 4 * (lane + 64 * i));
  }
  const float inv = 1.f / sqrtf(wave_sum(ss) / (float)dim + eps);
  // a missing weight read as zero and stands for ones
  const float w1 = w ? 0.f : 1.f, n1 = w_next ? 0.f : 1.f;
  const float4 w1v = make_float4(w1, w1, w1, w1), n1v = make_float4(n1, n1, n1, n1);
  float ss2 = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int64_t c = 4 * (lane + 64 * i);
    const float4 n = v[i] * inv * (cvt4(wa[i]) + w1v);
    if (res) {
      const float4 r = (cvt4(ra[i]) + n) * res_scale;
      v[i] = r;
      ss2 += dot4(r);  // zero past the row's end
      if (c < dim) st4(res + row * dim + c, r);
    }
    if (y && c < dim) st4(y + row * dim + c, n);
  }
  if (y_next) {
    const float inv2 = w_next ? 1.f / sqrtf(wave_sum(ss2) / (float)dim + eps) : 1.f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int64_t c = 4 * (lane + 64 * i);
      if (c < dim) st4(y_next + row * dim + c, w_next ? v[i] * inv2 * (cvt4(na[i]) + n1v) : v[i]);
    }
  }
}

template <typename TX, typename T>
static void launch_rownorm(int vpt, dim3 g, hipStream_t s, const TX* x, int parts, int64_t ps,
                           const T* w, T* y, float* res, float rs, const T* wn, T* yn, int64_t dim,
                           float eps) {
  const bool vec = (dim % 4) == 0 && (ps % 4) == 0 && dim <= 4096 &&
                   (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y | (uintptr_t)res | (uintptr_t)wn | (uintptr_t)yn) &
                    15) == 0;
  if (vec && g.x >= 1024 && parts >= 1) {  // many rows: one wave per row
    const int64_t rows = g.x;
    const int vw = (int)((dim / 4 + 63) / 64);
    const dim3 gw((unsigned)((rows + 3) / 4));
#define G4_RNW(V)                                                                                             \
  hipLaunchKernelGGL((k_rownorm_w<TX, T, V>), gw, dim3(256), 0, s, x, parts, ps, w, y, res, rs, wn, yn, rows, dim, \
                     eps)
    if (vw <= 2) G4_RNW(2);
    else if (vw <= 4) G4_RNW(4);
    else if (vw <= 8) G4_RNW(8);
    else if (vw <= 10) G4_RNW(10);
    else G4_RNW(16);
#undef G4_RNW
    return;
  }
  if (vec) {
    const int v4 = (int)((dim / 4 + 255) / 256);
#define G4_RN4(V) \
  hipLaunchKernelGGL((k_rownorm4<TX, T, V>), g, dim3(256), 0, s, x, parts, ps, w, y, res, rs, wn, yn, dim, eps)
    if (v4 <= 1) G4_RN4(1);
    else if (v4 <= 2) G4_RN4(2);
    else if (v4 <= 3) G4_RN4(3);
    else G4_RN4(4);
#undef G4_RN4
    return;
  }
#define G4_RN(V) \
  hipLaunchKernelGGL((k_rownorm<TX, T, V>), g, dim3(256), 0, s, x, parts, ps, w, y, res, rs, wn, yn, dim, eps)
  if (vpt <= 1) G4_RN(1);
  else if (vpt <= 2) G4_RN(2);
  else if (vpt <= 4) G4_RN(4);
  else if (vpt <= 8) G4_RN(8);
  else if (vpt <= 12) G4_RN(12);
  else if (vpt <= 16) G4_RN(16);
  else if (vpt <= 32) G4_RN(32);
  else G4_RN(64);
#undef G4_RN
}

g4_status rownorm(const void* x, int32_t x_dtype, int32_t x_parts, int64_t part_stride,
                  const void* w, void* y, float* res, float res_scale, const void* w_next,
                  void* y_next, int64_t rows, int64_t dim, float eps, int32_t dtype, hipStream_t s) {
  if (rows == 0) return G4_OK;
  if (dim > 64 * 256) return fail(G4_ERANGE, "rmsnorm: dim %lld exceeds 16384", (long long)dim);
  const int vpt = (int)((dim + 255) / 256);
  dim3 g((unsigned)rows);
  if (dtype == G4_BF16) {
    if (x_dtype == G4_F32)
      launch_rownorm<float, bf16>(vpt, g, s, (const float*)x, x_parts, part_stride, (const bf16*)w, (bf16*)y,
                                  res, res_scale, (const bf16*)w_next, (bf16*)y_next, dim, eps);
    else
      launch_rownorm<bf16, bf16>(vpt, g, s, (const bf16*)x, x_parts, part_stride, (const bf16*)w, (bf16*)y,
                                 res, res_scale, (const bf16*)w_next, (bf16*)y_next, dim, eps);
  } else {
    launch_rownorm<float, float>(vpt, g, s, (const float*)x, x_parts, part_stride, (const float*)w, (float*)y,
                                 res, res_scale, (const float*)w_next, (float*)y_next, dim, eps);
  }
  return check_launch("rmsnorm");
}

// --------------------------------------------------------------------------------------------
// Per-head RMSNorm + NeoX RoPE (cortiq-engine q/k/v head loops; turbospark per-head norms and
// `encode_rope_proportional_neox`; taconite `rope_half`). One block per (token row, four heads), one
// wave per head.
// Pair j of a head pairs elements j and j + hd/2; pairs j >= n_rot are left untouched (zero frequency).
// --------------------------------------------------------------------------------------------
struct SegDev {
  const void* x; int64_t x_ld;
  const void* w;
  void* y; int64_t y_ld; int64_t y_cap;
  int32_t heads; int32_t rope; int32_t ring;
};
struct SegPack { SegDev s[3]; int n; int total_heads; int parts; int64_t part_stride; };


// EPL consecutive values of one row (EPL in {1, 2, 4}) as floats, and back: one vector access when VEC,
// else element by element, the first n of them.
template <int EPL, bool VEC> __device__ __forceinline__ void ldv(const float* p, float* v, int n) {
  if (!VEC) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) v[e] = e < n ? p[e] : 0.f;
  } else if (EPL == 4) {
    const float4 t = *(const float4*)p; v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else if (EPL == 2) {
    const float2 t = *(const float2*)p; v[0] = t.x; v[1] = t.y;
  } else {
    v[0] = *p;
  }
}
template <int EPL, bool VEC> __device__ __forceinline__ void ldv(const bf16* p, float* v, int n) {
  if (!VEC) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) v[e] = e < n ? bf2f(p[e]) : 0.f;
  } else if (EPL == 4) {
    const uint2 u = *(const uint2*)p;
    v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
  } else if (EPL == 2) {
    const uint32_t u = *(const uint32_t*)p;
    v[0] = __uint_as_float(u << 16); v[1] = __uint_as_float(u & 0xffff0000u);
  } else {
    v[0] = bf2f(*p);
  }
}
template <int EPL, bool VEC> __device__ __forceinline__ void stv(float* p, const float* v, int n) {
  if (!VEC) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) if (e < n) p[e] = v[e];
  } else if (EPL == 4) {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
  } else if (EPL == 2) {
    *(float2*)p = make_float2(v[0], v[1]);
  } else {
    *p = v[0];
  }
}
template <int EPL, bool VEC> __device__ __forceinline__ void stv(bf16* p, const float* v, int n) {
  if (!VEC) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) if (e < n) p[e] = f2bf(v[e]);
  } else if (EPL == 4) {
    *(uint2*)p = pack_bf16x4(v);
  } else if (EPL == 2) {
    *(uint32_t*)p = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  } else {
    *p = f2bf(v[0]);
  }
}

// TI: input element type (float for summed split-K slices); T: output type. One wave per head; lane l
// owns pairs EPL l .. EPL l + EPL - 1 of the head (hd / 2 <= 64 EPL), i.e. elements j and j + hd/2 of
// each. VEC: rows aligned for EPL-wide accesses and hd / 2 a multiple of EPL. The lane's angles come
// while its loads are in flight: angle of pair j in revolutions, p * rev_j, reduced to [-1/2, 1/2] in
// float64, then the hardware sine and cosine of one revolution-scaled float32 (v_sin_f32 / v_cos_f32).
template <typename TI, typename T, int EPL, bool VEC>
__global__ __launch_bounds__(256) void k_qknr(SegPack pk, RopeTab tab, const int32_t* __restrict__ pos, int64_t T_,
                                              int hd, int n_rot, float eps) {
  const int gh = __builtin_amdgcn_readfirstlane(blockIdx.y * 4 + (threadIdx.x >> 6));  // wave-uniform
  if (gh >= pk.total_heads) return;
  const int lane = threadIdx.x & 63;
  const int64_t m = blockIdx.x;
  const uint32_t b = (uint32_t)blockIdx.x / (uint32_t)T_, t = (uint32_t)blockIdx.x % (uint32_t)T_;  // B T < 2^32
  const int64_t p = pos ? (int64_t)pos[b] + t : 0;
  const int half = hd >> 1;
  const int j0 = EPL * lane;
  const bool on = j0 < half;
  const int nv = half - j0;  // pairs of this lane inside the head (at least EPL when VEC)
  // the head's segment, picked with constant indexes so its fields come in scalar loads
  int h = gh;
  SegDev sg = pk.s[0];
  if (pk.n > 1 && h >= pk.s[0].heads) {
    h -= pk.s[0].heads;
    sg = pk.s[1];
    if (pk.n > 2 && h >= pk.s[1].heads) {
      h -= pk.s[1].heads;
      sg = pk.s[2];
    }
  }
  const bool rope = sg.rope != 0;
  double rv[EPL];  // j0 + e <= 255: inside the table, zero past the rotated pairs
#pragma unroll
  for (int e = 0; e < EPL; ++e) rv[e] = tab.rev[j0 + e];
  const TI* xh = (const TI*)sg.x + m * sg.x_ld + (int64_t)h * hd;
  float a[EPL], c[EPL], wa[EPL], wc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) a[e] = c[e] = 0.f, wa[e] = wc[e] = 1.f;
  // without a weight the loads read the head's own input (in range for either type) and the weight is 1
  const T* wp = sg.w ? (const T*)sg.w : (const T*)(const void*)xh;
  if (on) {
    ldv<EPL, VEC>(xh + j0, a, nv);
    ldv<EPL, VEC>(xh + j0 + half, c, nv);
    ldv<EPL, VEC>(wp + j0, wa, nv);
    ldv<EPL, VEC>(wp + j0 + half, wc, nv);
  }
  if (!sg.w)
#pragma unroll
    for (int e = 0; e < EPL; ++e) wa[e] = wc[e] = 1.f;
  float co[EPL], sn[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    double r = (double)p * rv[e];
    r -= rint(r);
    co[e] = __builtin_amdgcn_cosf((float)r);
    sn[e] = __builtin_amdgcn_sinf((float)r);
  }
  if (on)  // further split-K slices, summed in order after the first, four per round trip
    for (int p0 = 1; p0 < pk.parts; p0 += 4) {
      float ta[4][EPL], tc[4][EPL];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t off = (int64_t)min(p0 + q, pk.parts - 1) * pk.part_stride;  // past the last: re-read it
        ldv<EPL, VEC>(xh + off + j0, ta[q], nv);
        ldv<EPL, VEC>(xh + off + j0 + half, tc[q], nv);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (p0 + q < pk.parts)
#pragma unroll
          for (int e = 0; e < EPL; ++e) { a[e] += ta[q][e]; c[e] += tc[q][e]; }
    }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) ss += a[e] * a[e] + c[e] * c[e];
  ss = wave_sum(ss);
  const float inv = 1.f / sqrtf(ss / (float)hd + eps);
  T* yh;
  if (sg.y_cap > 0) {
    if (p < 0 || (!sg.ring && p >= sg.y_cap)) return;  // out-of-range position: no write
    const int64_t row = sg.ring ? p % sg.y_cap : p;
    yh = (T*)sg.y + ((((int64_t)b * sg.heads + h) * sg.y_cap) + row) * hd;
  } else {
    yh = (T*)sg.y + m * sg.y_ld + (int64_t)h * hd;
  }
  if (!on) return;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    float u = a[e] * inv * wa[e], v = c[e] * inv * wc[e];
    if (rope && j0 + e < n_rot) {
      const float u2 = u * co[e] - v * sn[e];
      const float v2 = v * co[e] + u * sn[e];
      u = u2; v = v2;
    }
    a[e] = u; c[e] = v;
  }
  stv<EPL, VEC>(yh + j0, a, nv);
  stv<EPL, VEC>(yh + j0 + half, c, nv);
}

void rope_table(RopeTab& t, float theta, int64_t hd, int64_t n_rot) {
  for (int j = 0; j < 256; ++j)
    t.rev[j] = j < n_rot ? pow((double)theta, -2.0 * j / (double)hd) / 6.283185307179586 : 0.0;
}

static g4_status qknr_launch(const HeadSeg* segs, int nseg, int parts, int64_t part_stride, bool f32_in,
                             const int32_t* pos, int64_t B, int64_t T, int64_t hd, float theta, int64_t n_rot,
                             float eps, int32_t dtype, hipStream_t s) {
  if (B * T == 0) return G4_OK;
  if (hd > 512 || hd < 2 || (hd & 1)) return fail(G4_ERANGE, "qk_norm_rope: head_dim %lld not in [2, 512]", (long long)hd);
  SegPack pk{};
  pk.n = nseg;
  pk.total_heads = 0;
  pk.parts = parts;
  pk.part_stride = part_stride;
  int any_rope = 0;
  for (int i = 0; i < nseg; ++i) {
    pk.s[i] = SegDev{segs[i].x, segs[i].x_ld, segs[i].w, segs[i].y, segs[i].y_ld, segs[i].y_cap,
                     segs[i].heads, segs[i].rope, segs[i].ring};
    pk.total_heads += segs[i].heads;
    any_rope |= segs[i].rope;
  }
  const int nr = any_rope ? (int)n_rot : 0;
  RopeTab tab;
  rope_table(tab, theta, hd, nr);
  // pairs per lane: vector accesses when every row start is aligned to them, else per element
  const int64_t half = hd / 2;
  const size_t isz = f32_in ? 4 : (dtype == G4_BF16 ? 2 : 4), osz = dtype == G4_BF16 ? 2 : 4;
  auto aligned = [&](int e) {
    if ((half % e) || (part_stride % e)) return false;
    for (int i = 0; i < nseg; ++i) {
      if ((segs[i].x_ld % e) || ((uintptr_t)segs[i].x % (isz * e)) || ((uintptr_t)segs[i].y % (osz * e))) return false;
      if (segs[i].y_cap == 0 && (segs[i].y_ld % e)) return false;
      if (segs[i].w && ((uintptr_t)segs[i].w % (osz * e))) return false;
    }
    return true;
  };
  const int need = half <= 64 ? 1 : (half <= 128 ? 2 : 4);  // fewest pairs per lane that cover the head
  const bool vec = need == 1 || aligned(need);
  // one wave per head: blocks of four heads, so a token's heads run in parallel
  dim3 g((unsigned)(B * T), (unsigned)((pk.total_heads + 3) / 4));
#define G4_QK(TI, TT, P, V) \
  hipLaunchKernelGGL((k_qknr<TI, TT, P, V>), g, dim3(256), 0, s, pk, tab, pos, T, (int)hd, nr, eps)
#define G4_QKE(TI, TT)                                                      \
  do {                                                                      \
    if (need == 1) G4_QK(TI, TT, 1, true);                                  \
    else if (need == 2) { if (vec) G4_QK(TI, TT, 2, true); else G4_QK(TI, TT, 2, false); } \
    else { if (vec) G4_QK(TI, TT, 4, true); else G4_QK(TI, TT, 4, false); } \
  } while (0)
  if (dtype == G4_BF16 && f32_in) G4_QKE(float, bf16);
  else if (dtype == G4_BF16) G4_QKE(bf16, bf16);
  else G4_QKE(float, float);
#undef G4_QKE
#undef G4_QK
  return check_launch("qk_norm_rope");
}

g4_status qk_norm_rope(const HeadSeg* segs, int nseg, const int32_t* pos, int64_t B, int64_t T,
                       int64_t hd, float theta, int64_t n_rot, float eps, int32_t dtype, hipStream_t s) {
  return qknr_launch(segs, nseg, 1, 0, false, pos, B, T, hd, theta, n_rot, eps, dtype, s);
}

g4_status qk_norm_rope_parts(const HeadSeg* segs, int nseg, int parts, int64_t part_stride, const int32_t* pos,
                             int64_t B, int64_t T, int64_t hd, float theta, int64_t n_rot, float eps, int32_t dtype,
                             hipStream_t s) {
  return qknr_launch(segs, nseg, parts, part_stride, true, pos, B, T, hd, theta, n_rot, eps, dtype, s);
}

// --------------------------------------------------------------------------------------------
// Scaled embedding gather (ferrox `forward_token_on_worker`: row times sqrt(H)); ids outside
// [0, vocab) give a zero row. Also writes the row in the model dtype for the PLE projection GEMM.
// --------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_embed(const int32_t* __restrict__ ids, const T* __restrict__ E,
                                               int64_t vocab, int64_t H, float scale, float* __restrict__ h,
                                               T* __restrict__ ecast) {
  const int64_t m = blockIdx.x;
  const int64_t id = ids[m];
  const bool ok = id >= 0 && id < vocab;
  for (int64_t c = threadIdx.x; c < H; c += 256) {
    const float v = ok ? ldf(E + id * H + c) * scale : 0.f;
    h[m * H + c] = v;
    if (ecast) stf(ecast + m * H + c, v);
  }
}

g4_status embed_rows(const int32_t* ids, int64_t M, const void* E, int64_t vocab, int64_t H,
                     float* h_out, void* e_cast, int32_t dtype, hipStream_t s) {
  if (M == 0) return G4_OK;
  const float scale = sqrtf((float)H);
  if (dtype == G4_BF16)
    hipLaunchKernelGGL(k_embed<bf16>, dim3((unsigned)M), dim3(256), 0, s, ids, (const bf16*)E, vocab, H, scale,
                       h_out, (bf16*)e_cast);
  else
    hipLaunchKernelGGL(k_embed<float>, dim3((unsigned)M), dim3(256), 0, s, ids, (const float*)E, vocab, H, scale,
                       h_out, (float*)e_cast);
  return check_launch("embed");
}

// --------------------------------------------------------------------------------------------
// Per-layer inputs from the projected embedding (cortiq-engine `extend_embedding`, ferrox
// `project_per_layer_inputs`): per (token, layer) chunk of d values,
//   (rms(P * H^-1/2) * ple_norm + sqrt(d) * Tab[id, chunk]) / sqrt(2).
// One wave per chunk, d <= 512.
// --------------------------------------------------------------------------------------------
template <typename T, int PER>
__global__ __launch_bounds__(256) void k_ple_combine(const int32_t* __restrict__ ids, const float* __restrict__ P,
                                                     const T* __restrict__ Tab, int64_t ple_vocab,
                                                     const T* __restrict__ norm, int64_t L, int d,
                                                     float pscale, float eps, float* __restrict__ out) {
  const int64_t m = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t id = ids[m];
  const bool ok = id >= 0 && id < ple_vocab;
  const float tscale = sqrtf((float)d);
  const float half = 0.70710678118654752f;
  for (int64_t l = blockIdx.y * 4 + wave; l < L; l += (int64_t)gridDim.y * 4) {
    const float* pr = P + (m * L + l) * d;
    float v[PER];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = lane + 64 * i;
      v[i] = j < d ? pr[j] * pscale : 0.f;
      ss += v[i] * v[i];
    }
    ss = wave_sum(ss);
    const float inv = 1.f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = lane + 64 * i;
      if (j >= d) continue;
      float r = v[i] * inv * ldf(norm + j);
      if (ok) r += ldf(Tab + id * (L * d) + l * d + j) * tscale;
      out[(m * L + l) * d + j] = r * half;
    }
  }
}

// The same with four consecutive values per lane (d a multiple of 4, 16-byte aligned rows): every load
// of the chunk (projection, table row, norm weight) is issued before the reduction, in 16-byte pieces.
template <typename T, int PER4>
__global__ __launch_bounds__(256) void k_ple_combine4(const int32_t* __restrict__ ids, const float* __restrict__ P,
                                                      const T* __restrict__ Tab, int64_t ple_vocab,
                                                      const T* __restrict__ norm, int64_t L, int d,
                                                      float pscale, float eps, float* __restrict__ out) {
  const int64_t m = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t l = blockIdx.y * 4 + wave;
  if (l >= L) return;
  const int64_t id = ids[m];
  const bool ok = id >= 0 && id < ple_vocab;
  const float tscale = sqrtf((float)d);
  const float half = 0.70710678118654752f;
  const float* pr = P + (m * L + l) * d;
  const T* tr = Tab + (ok ? id : 0) * (L * d) + l * d;
  float4 v[PER4], tv[PER4], nw[PER4];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < PER4; ++i) {
    const int j = 4 * lane + 256 * i;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    v[i] = j < d ? *(const float4*)(pr + j) : z;
    tv[i] = (ok && j < d) ? ld4(tr + j) : z;
    nw[i] = j < d ? ld4(norm + j) : z;
  }
#pragma unroll
  for (int i = 0; i < PER4; ++i) {
    v[i] = v[i] * pscale;
    ss += dot4(v[i]);
  }
  ss = wave_sum(ss);
  const float inv = 1.f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int i = 0; i < PER4; ++i) {
    const int j = 4 * lane + 256 * i;
    if (j >= d) continue;
    const float4 r = (v[i] * inv * nw[i] + tv[i] * tscale) * half;
    *(float4*)(out + (m * L + l) * d + j) = r;
  }
}

g4_status ple_combine(const int32_t* ids, int64_t M, const float* P, const void* Tab, int64_t ple_vocab,
                      const void* ple_norm, int64_t H, int64_t L, int64_t d, float eps, float* ple_out,
                      int32_t dtype, hipStream_t s) {
  if (M == 0) return G4_OK;
  if (d > 512) return fail(G4_ERANGE, "ple_dim %lld exceeds 512", (long long)d);
  const float pscale = 1.f / sqrtf((float)H);
  dim3 g((unsigned)M, (unsigned)((L + 3) / 4));
  const int per = (int)((d + 63) / 64);
  const size_t tsz = dtype == G4_BF16 ? 2 : 4;
  if (d % 4 == 0 && ((uintptr_t)P & 15) == 0 && ((uintptr_t)ple_out & 15) == 0 && ((uintptr_t)Tab % (4 * tsz)) == 0 &&
      ((uintptr_t)ple_norm % (4 * tsz)) == 0) {
    const int per4 = (int)((d + 255) / 256);
#define G4_PC4(TT, P4)                                                                                     \
  hipLaunchKernelGGL((k_ple_combine4<TT, P4>), g, dim3(256), 0, s, ids, P, (const TT*)Tab, ple_vocab, \
                     (const TT*)ple_norm, L, (int)d, pscale, eps, ple_out)
    if (dtype == G4_BF16) {
      if (per4 <= 1) G4_PC4(bf16, 1); else G4_PC4(bf16, 2);
    } else {
      if (per4 <= 1) G4_PC4(float, 1); else G4_PC4(float, 2);
    }
#undef G4_PC4
    return check_launch("ple_combine");
  }
#define G4_PC(TT, P) hipLaunchKernelGGL((k_ple_combine<TT, P>), g, dim3(256), 0, s, ids, P_, (const TT*)Tab, ple_vocab, (const TT*)ple_norm, L, (int)d, pscale, eps, ple_out)
  const float* P_ = P;
  if (dtype == G4_BF16) {
    if (per <= 1) G4_PC(bf16, 1); else if (per <= 4) G4_PC(bf16, 4); else G4_PC(bf16, 8);
  } else {
    if (per <= 1) G4_PC(float, 1); else if (per <= 4) G4_PC(float, 4); else G4_PC(float, 8);
  }
#undef G4_PC
  return check_launch("ple_combine");
}

}  // namespace g4

namespace g4 {
template <typename T>
__global__ __launch_bounds__(256) void k_cast(const float* __restrict__ x, T* __restrict__ y, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) stf(y + i, x[i]);
}
g4_status cast_rows(const float* x, void* y, int64_t n, int32_t dtype, hipStream_t s) {
  if (n == 0) return G4_OK;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (dtype == G4_BF16) hipLaunchKernelGGL(k_cast<bf16>, dim3((unsigned)blocks), dim3(256), 0, s, x, (bf16*)y, n);
  else hipLaunchKernelGGL(k_cast<float>, dim3((unsigned)blocks), dim3(256), 0, s, x, (float*)y, n);
  return check_launch("cast");
}
// --------------------------------------------------------------------------------------------
// Final-logit softcap in place (ferrox-models `forward_token_on_worker`: softcap after the output
// head): x <- cap * tanh(x / cap).
// --------------------------------------------------------------------------------------------
// Four consecutive floats per thread (x 16-byte aligned, n a multiple of 4) when V4, else one.
template <bool V4>
__global__ __launch_bounds__(256) void k_softcap(float* __restrict__ x, int64_t n, float cap) {
  const float inv = 1.f / cap;
  if constexpr (V4) {
    for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += (int64_t)gridDim.x * 1024) {
      float4 v = *(const float4*)(x + i);
      v.x = cap * tanhf(v.x * inv); v.y = cap * tanhf(v.y * inv);
      v.z = cap * tanhf(v.z * inv); v.w = cap * tanhf(v.w * inv);
      *(float4*)(x + i) = v;
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
      x[i] = cap * tanhf(x[i] * inv);
  }
}

g4_status softcap_inplace(float* x, int64_t n, float cap, hipStream_t s) {
  if (n == 0 || cap <= 0.f) return G4_OK;
  const bool v4 = n % 4 == 0 && ((uintptr_t)x & 15) == 0;
  int64_t blocks = (v4 ? n / 4 + 255 : n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (v4) hipLaunchKernelGGL(k_softcap<true>, dim3((unsigned)blocks), dim3(256), 0, s, x, n, cap);
  else hipLaunchKernelGGL(k_softcap<false>, dim3((unsigned)blocks), dim3(256), 0, s, x, n, cap);
  return check_launch("softcap");
}

}  // namespace g4
