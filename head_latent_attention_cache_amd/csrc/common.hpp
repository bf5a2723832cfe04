// Shared device/host helpers of the MLA library (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/mla.h"

namespace mla {

// ---------------------------------------------------------------------------
// element types: float or bfloat16 stored as its 16-bit pattern
// ---------------------------------------------------------------------------
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}

// round to nearest even with gfx950's v_cvt_pk_bf16_f32 (pairs of adjacent
// conversions share one instruction); NaN stays NaN
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(bf16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// value stored in the cache / output format, read back as float
template <typename T> __device__ __forceinline__ float round_to(float v);
template <> __device__ __forceinline__ float round_to<float>(float v) { return v; }
template <> __device__ __forceinline__ float round_to<bf16_t>(float v) { return bf16_to_f32(f32_to_bf16(v)); }

// ---------------------------------------------------------------------------
// cache geometry (ring of `window` frames of P tokens per sequence)
// ---------------------------------------------------------------------------
struct Geo {
  int P;          // tokens per frame
  int grid_w;
  int window;     // frames in the ring
  int fpb;        // frames per block (block-causal)
  int capacity;   // window * P
};

// slot of token tok of frame f (f may be any integer; the ring index is taken mod window)
__device__ __forceinline__ int ring_slot(const Geo& g, int f, int tok) {
  int r = f % g.window;
  if (r < 0) r += g.window;
  return r * g.P + tok;
}

// frame held by ring position rp (0 <= rp < window) when `newest` is the newest
// frame written; negative when the slot was never written.  nm = newest mod window.
__device__ __forceinline__ int ring_frame(int rp, int newest, int nm, int window) {
  int t = nm - rp;
  if (t < 0) t += window;
  return newest - t;
}

__device__ __forceinline__ int floor_div(int a, int b) {
  int q = a / b;
  return (a % b != 0 && ((a < 0) != (b < 0))) ? q - 1 : q;
}

__device__ __forceinline__ bool key_visible(int fq, int fk, int window, int fpb) {
  return fk >= 0 && floor_div(fk, fpb) <= floor_div(fq, fpb) && (fq - fk) < window;
}

// rotary coordinates of token tok of frame f
__device__ __forceinline__ void token_coords(int rope_dims, int P, int grid_w, int f, int tok,
                                             double* c) {
  if (rope_dims == 3) {
    c[0] = (double)f;
    c[1] = (double)(tok / grid_w);
    c[2] = (double)(tok % grid_w);
  } else {
    c[0] = (double)f * (double)P + (double)tok;
  }
}

// ---------------------------------------------------------------------------
// kernel-side copy of the model dimensions
// ---------------------------------------------------------------------------
struct Dims {
  int H, d_model, d_nope, d_v, d_c, d_r, d_qk;
  int rope_dims, band0, band1, band2;
  float theta, scale;
  int dtype, cache_fmt;
  int qk_norm;    // 1: QK-normalised attention (per-slot key inverse RMS in the aux buffer)
  float qk_eps;
};

// low-bit caches (INT4, INT2): bits per content code, code bytes per cache
// row (content codes, then the INT4 rotary codes)
__host__ __device__ __forceinline__ bool lowbit_cache(const Dims& d) { return d.cache_fmt != MLA_CACHE_DENSE; }
__host__ __device__ __forceinline__ int content_bits(const Dims& d) { return d.cache_fmt == MLA_CACHE_INT2 ? 2 : 4; }
__host__ __device__ __forceinline__ int code_row_bytes(const Dims& d) { return d.d_c * content_bits(d) / 8 + d.d_r / 2; }

// byte offset of the per-slot key inverse RMS (QK normalisation) in the aux
// buffer of `rows` slots: after the fp16 scales of a low-bit cache, 16-byte aligned
__host__ __device__ __forceinline__ size_t key_scale_offset(const Dims& d, size_t rows) {
  return lowbit_cache(d) ? (rows * (d.d_c / 32 + 1) * 2 + 15) / 16 * 16 : 0;
}

// integer code of element j of a low-bit cache row (two's complement, the
// lowest bits first: INT4 element 2i in the low nibble of byte i, INT2
// element 4i + k in bits 2k .. 2k+1; the rotary part is INT4 after the content)
__device__ __forceinline__ int lowbit_code(const uint8_t* row, const Dims& d, int j) {
  if (j < d.d_c && d.cache_fmt == MLA_CACHE_INT2) {
    const int q = (row[j >> 2] >> (2 * (j & 3))) & 3;
    return (q ^ 2) - 2;
  }
  const int off = j < d.d_c ? 0 : d.d_c * content_bits(d) / 8;
  const int jj = j < d.d_c ? j : j - d.d_c;
  const uint8_t byte = row[off + (jj >> 1)];
  const int q = (jj & 1) ? (byte >> 4) : (byte & 0xF);
  return (q ^ 8) - 8;
}

}  // namespace mla
