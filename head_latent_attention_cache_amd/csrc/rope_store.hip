// Rotary embedding, cache-row storage (dense, INT4 or INT2) and the absorbed query's
// rotary half.
//
// Rotary embedding: "Multi-Head Latent Attention" concept page, The RoPE
// problem, and the decoupled fix (a position-dependent rotation whose query/key
// product depends on the offset only); VideoMLA review, Key Concepts (3D-RoPE
// over time, height and width).  Pair i of a band of width b at coordinate p
// rotates by p * theta^(-2i/b); bands are ordered (t, h, w).
//
// Low-bit storage: "Multi-Head Latent Attention" topic page, QuantMLA abstract
// (both cache paths in INT4, dequantised inside attention; a deeper variant
// with the content latent in INT2 and the rotary key in INT4).  For b bits:
// scale = fp16(amax / (2^(b-1) - 1)), code = round-half-even(x / scale)
// clamped to [-2^(b-1), 2^(b-1) - 1] in IEEE fp32, the lowest bits first.
#include "skinny_gemm.hpp"

namespace mla {

// cosine and sine of rotary pair i of one token: angle in fp64, reduced to
// [-pi, pi] in fp64, then an fp32 sine/cosine
__device__ __forceinline__ void rope_pair(const Dims& d, const double* coord, int i, float* c, float* s) {
  int axis = 0, ii = i, band = d.band0;
  if (d.rope_dims == 3) {
    if (ii >= d.band0 / 2) {
      ii -= d.band0 / 2;
      axis = 1;
      band = d.band1;
      if (ii >= d.band1 / 2) {
        ii -= d.band1 / 2;
        axis = 2;
        band = d.band2;
      }
    }
  }
  const double freq = exp2(-2.0 * (double)ii / (double)band * log2((double)d.theta));
  const double ang = coord[axis] * freq;
  const double two_pi = 6.283185307179586476925286766559;
  const float r = (float)(ang - two_pi * rint(ang / two_pi));
  sincosf(r, s, c);
}

// angles of all d_r/2 rotary pairs of one token
__device__ void rope_table(const Dims& d, const double* coord, float* cosv, float* sinv) {
  for (int i = threadIdx.x; i < d.d_r / 2; i += blockDim.x) rope_pair(d, coord, i, &cosv[i], &sinv[i]);
}

// quantise n values (n a multiple of 8 / bits) of an LDS row to `bits`-bit
// codes (4 or 2) + one fp16 scale
__device__ __forceinline__ void quant_lowbit(const float* v, int n, int bits, uint8_t* codes, __half* scale) {
  const int qmax = (1 << (bits - 1)) - 1, per_byte = 8 / bits, mask = (1 << bits) - 1;
  float amax = 0.f;
  for (int j = 0; j < n; ++j) amax = fmaxf(amax, fabsf(v[j]));
  __half s16 = __float2half_rn(amax / (float)qmax);
  float s = __half2float(s16);
  *scale = s16;
  for (int j = 0; j < n; j += per_byte) {
    int byte = 0;
    for (int k = 0; k < per_byte; ++k) {
      int q = 0;
      if (s != 0.f) q = (int)fminf(fmaxf(rintf(v[j + k] / s), (float)(-qmax - 1)), (float)qmax);
      byte |= (q & mask) << (bits * k);
    }
    codes[j / per_byte] = (uint8_t)byte;
  }
}

// ---------------------------------------------------------------------------
// finish the append: sum the K-split partials of the projected row, rotate its
// k_rope columns, round to the storage type and store it at its ring slot.
// grid (n_tokens, B); y: [nsplit][B, n_tokens, d_qk] fp32 partials of
// x . w_dkr^T.  One work item per thread: a content element, or a rotary pair
// (whose angle the same thread computes); every partial of an item is loaded
// before the sum (fixed split order), so the work-group waits for one round
// of loads.
// ---------------------------------------------------------------------------
template <typename T, bool LOWBIT>
__global__ void append_store_kernel(Dims d, Geo g, const float* __restrict__ y, int n_tokens,
                                    const int* __restrict__ frame, void* __restrict__ cache,
                                    __half* __restrict__ aux, int batch, int nsplit) {
  extern __shared__ float row[];           // d_qk (low-bit: the rounded row, quantised at the end)
  constexpr int PG = 16;                   // partials loaded together
  const int i = blockIdx.x, b = blockIdx.y;
  const int f = frame[b] + i / g.P, tok = i % g.P;
  const float* src = y + ((size_t)b * n_tokens + i) * d.d_qk;
  const size_t split_stride = (size_t)batch * n_tokens * d.d_qk;
  auto proj = [&](int j) {
    if (nsplit == 1) return src[j];
    float v = 0.f;
    for (int sp0 = 0; sp0 < nsplit; sp0 += PG) {
      float t[PG];
#pragma unroll
      for (int u = 0; u < PG; ++u) t[u] = src[(size_t)min(sp0 + u, nsplit - 1) * split_stride + j];
#pragma unroll
      for (int u = 0; u < PG; ++u)
        if (sp0 + u < nsplit) v = sp0 + u == 0 ? t[u] : v + t[u];
    }
    return v;
  };
  const int slot = ring_slot(g, f, tok);
  const size_t srow = (size_t)b * g.capacity + slot;
  T* out = (T*)cache + srow * d.d_qk;
  const int n_items = d.d_c + d.d_r / 2;
  for (int it = threadIdx.x; it < n_items; it += blockDim.x) {
    if (it < d.d_c) {
      const float v = round_to<T>(proj(it));
      if (LOWBIT) row[it] = v;
      else Elem<T>::store(out, it, v);
    } else {
      const int p = it - d.d_c;
      const float x0 = proj(d.d_c + 2 * p), x1 = proj(d.d_c + 2 * p + 1);
      double coord[3];
      token_coords(d.rope_dims, g.P, g.grid_w, f, tok, coord);
      float c, s;
      rope_pair(d, coord, p, &c, &s);
      const float r0 = round_to<T>(x0 * c - x1 * s), r1 = round_to<T>(x0 * s + x1 * c);
      if (LOWBIT) {
        row[d.d_c + 2 * p] = r0;
        row[d.d_c + 2 * p + 1] = r1;
      } else {
        Elem<T>::store(out, d.d_c + 2 * p, r0);
        Elem<T>::store(out, d.d_c + 2 * p + 1, r1);
      }
    }
  }
  if (LOWBIT) {
    __syncthreads();
    const int cb = content_bits(d);
    uint8_t* codes = (uint8_t*)cache + srow * code_row_bytes(d);
    const int ng = d.d_c / 32;
    __half* cscale = aux + srow * ng;
    __half* rscale = aux + (size_t)batch * g.capacity * ng + srow;
    for (int grp = threadIdx.x; grp <= ng; grp += blockDim.x) {
      if (grp < ng) quant_lowbit(row + grp * 32, 32, cb, codes + grp * 32 * cb / 8, cscale + grp);
      else quant_lowbit(row + d.d_c, d.d_r, 4, codes + d.d_c * cb / 8, rscale);
    }
  }
}

// ---------------------------------------------------------------------------
// rotary half of the absorbed query: q_abs[b,t,h,d_c:] = RoPE(q_rope[b,t,h])
// grid (n_q, B, ceil(H / 16)).  QK normalisation ("Multi-Head Latent
// Attention" topic page, QK-Norm abstract): the work-group also scales its
// heads' content part by inv_q = 1 / sqrt(mean(q_nope[b, t]^2) + eps), the
// mean over every head of the token (each work-group of the token computes
// the same sum in the same order).
// ---------------------------------------------------------------------------
// work-group (t, b, hz): query token t of sequence b, heads 16 hz .. 16 hz + 15
template <typename T>
__device__ __forceinline__ void q_rope_body(const Dims& d, const Geo& g, const T* __restrict__ q_rope, int n_q,
                                            const int* __restrict__ q_first, const T* __restrict__ q_nope,
                                            T* __restrict__ q_abs, int t, int b, int hz) {
  extern __shared__ float smem[];
  float* cosv = smem;
  float* sinv = smem + d.d_r / 2;
  __shared__ float red[4];
  const int f = q_first[b] + t / g.P, tok = t % g.P;
  double coord[3];
  token_coords(d.rope_dims, g.P, g.grid_w, f, tok, coord);
  rope_table(d, coord, cosv, sinv);
  __syncthreads();
  const int npair = d.d_r / 2;
  const size_t tok_index = (size_t)b * n_q + t;
  const int h0 = hz * 16, h1 = min(d.H, h0 + 16);
  for (int e = threadIdx.x; e < (h1 - h0) * npair; e += blockDim.x) {
    const int h = h0 + e / npair, p = e % npair;
    const T* src = q_rope + (tok_index * d.H + h) * d.d_r;
    T* dst = q_abs + (tok_index * d.H + h) * d.d_qk + d.d_c;
    float x0 = Elem<T>::load(src, 2 * p), x1 = Elem<T>::load(src, 2 * p + 1);
    float c = cosv[p], s = sinv[p];
    Elem<T>::store(dst, 2 * p, x0 * c - x1 * s);
    Elem<T>::store(dst, 2 * p + 1, x0 * s + x1 * c);
  }
  if (d.qk_norm) {
    const int n = d.H * d.d_nope;
    const T* qn = q_nope + tok_index * n;
    float acc = 0.f;
    if constexpr (sizeof(T) == 2) {
      // bf16: eight values per 16-byte load (n and d_c are multiples of 8)
      for (int e = threadIdx.x * 8; e < n; e += blockDim.x * 8) {
        const uint4 v = *(const uint4*)(qn + e);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float lo = __uint_as_float(w[k] << 16), hi = __uint_as_float(w[k] & 0xFFFF0000u);
          acc = fmaf(lo, lo, acc);
          acc = fmaf(hi, hi, acc);
        }
      }
    } else {
      for (int e = threadIdx.x; e < n; e += blockDim.x) {
        const float v = Elem<T>::load(qn, e);
        acc = fmaf(v, v, acc);
      }
    }
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    const float ms = (red[0] + red[1] + red[2] + red[3]) / (float)n + d.qk_eps;
    const float inv = ms > 0.f ? 1.f / sqrtf(ms) : 0.f;
    if constexpr (sizeof(T) == 2) {
      for (int e = threadIdx.x * 8; e < (h1 - h0) * d.d_c; e += blockDim.x * 8) {
        T* dst = q_abs + (tok_index * d.H + h0 + e / d.d_c) * d.d_qk + e % d.d_c;
        uint4 v = *(const uint4*)dst;
        uint32_t* w = (uint32_t*)&v;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float lo = __uint_as_float(w[k] << 16) * inv, hi = __uint_as_float(w[k] & 0xFFFF0000u) * inv;
          w[k] = (uint32_t)__builtin_bit_cast(uint16_t, f32_to_bf16(lo)) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, f32_to_bf16(hi)) << 16);
        }
        *(uint4*)dst = v;
      }
    } else {
      for (int e = threadIdx.x; e < (h1 - h0) * d.d_c; e += blockDim.x) {
        T* dst = q_abs + (tok_index * d.H + h0 + e / d.d_c) * d.d_qk;
        const int j = e % d.d_c;
        Elem<T>::store(dst, j, Elem<T>::load(dst, j) * inv);
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void q_rope_kernel(Dims d, Geo g, const T* __restrict__ q_rope, int n_q,
                                                     const int* __restrict__ q_first, const T* __restrict__ q_nope,
                                                     T* __restrict__ q_abs) {
  q_rope_body<T>(d, g, q_rope, n_q, q_first, q_nope, q_abs, blockIdx.x, blockIdx.y, blockIdx.z);
}

// ---------------------------------------------------------------------------
// the decode-time absorbed query in one launch (bf16, no QK normalisation,
// at most 32 query rows, d_nope <= 128): work-groups [0, n_gemm) form the
// content half, the skinny product q_nope[:, h] . w_uk[h]^T (column block,
// head), the others the rotary half (query token, sequence, group of 16
// heads), the work of q_rope_kernel.  The halves are disjoint columns of
// q_abs, so they run side by side instead of one launch after the other,
// each with the same code and results as its own kernel.
// ---------------------------------------------------------------------------
constexpr int ABSORB_BN = 128, ABSORB_SEG = 128;
__global__ __launch_bounds__(256) void absorb_rope_kernel(GemmArgs ga, int gemm_bx, Dims d, Geo g, int batch,
                                                          const bf16_t* __restrict__ q_rope, int n_q,
                                                          const int* __restrict__ q_first, bf16_t* __restrict__ q_abs) {
  const int id = blockIdx.x, n_gemm = gemm_bx * ga.batch;
  if (id < n_gemm) {
    skinny_gemm_body<1, ABSORB_BN, ABSORB_SEG>(ga, id % gemm_bx, 0, id / gemm_bx);
    return;
  }
  const int r = id - n_gemm;
  q_rope_body<bf16_t>(d, g, q_rope, n_q, q_first, nullptr, q_abs, r % n_q, (r / n_q) % batch, r / (n_q * batch));
}

bool absorb_rope_fusable(const Dims& d, const GemmArgs& ga) {
  return d.dtype == MLA_BF16 && !d.qk_norm && ga.M <= 32 && ga.K <= ABSORB_SEG && ga.ksplit == 1;
}

hipError_t launch_absorb_rope(const Dims& d, const Geo& g, const GemmArgs& ga, int batch, const void* q_rope, int n_q,
                              const int* q_first, void* q_abs, hipStream_t st) {
  if (!absorb_rope_fusable(d, ga)) return hipErrorInvalidValue;
  const int gemm_bx = (ga.N + ABSORB_BN - 1) / ABSORB_BN;
  const long long blocks = (long long)gemm_bx * ga.batch + (long long)n_q * batch * ((d.H + 15) / 16);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const size_t shm = (size_t)d.d_r * sizeof(float);   // the rotary work-groups' cosine and sine table
  absorb_rope_kernel<<<(unsigned)blocks, 256, shm, st>>>(ga, gemm_bx, d, g, batch, (const bf16_t*)q_rope, n_q, q_first,
                                                          (bf16_t*)q_abs);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// cache rows as float (inspection utility)
// ---------------------------------------------------------------------------
template <typename T, bool LOWBIT>
__global__ void dequant_kernel(Dims d, Geo g, int batch, const void* __restrict__ cache,
                               const __half* __restrict__ aux, float* __restrict__ out) {
  const size_t total = (size_t)batch * g.capacity * d.d_qk;
  const int ng = d.d_c / 32;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const size_t srow = e / d.d_qk;
    const int j = (int)(e % d.d_qk);
    float v;
    if (!LOWBIT) {
      v = Elem<T>::load((const T*)cache, e);
    } else {
      const int q = lowbit_code((const uint8_t*)cache + srow * code_row_bytes(d), d, j);
      const float s = j < d.d_c ? __half2float(aux[srow * ng + j / 32])
                                : __half2float(aux[(size_t)batch * g.capacity * ng + srow]);
      v = (float)q * s;
    }
    out[e] = v;
  }
}

// ---------------------------------------------------------------------------
// re-rotation of stored rotary keys by a coordinate shift ("Multi-Head Latent
// Attention" topic page, Irminsul abstract: the rotary part of a row is
// corrected in closed form when its token moves, the content latent is
// position-free).  Rotations by angles proportional to the coordinate
// compose, R(p + delta) = R(delta) R(p), so every row of a sequence turns by
// the same table.  grid (ceil(n_slots / rows_per_block), B): one rotary pair
// per thread and row; low-bit rows are dequantised, rotated, rounded to bf16
// and re-quantised (new per-token scale) once the work-group holds them.  A
// shift that is zero in the coordinates the embedding uses returns at once.
// ---------------------------------------------------------------------------
template <typename T, bool LOWBIT>
__global__ void rope_shift_kernel(Dims d, Geo g, int batch, const int* __restrict__ delta, int slot_begin,
                                  int n_slots, int rows_per_block, void* __restrict__ cache,
                                  __half* __restrict__ aux) {
  extern __shared__ float smem[];
  float* cosv = smem;                 // [d_r / 2]
  float* sinv = smem + d.d_r / 2;     // [d_r / 2]
  float* rows = smem + d.d_r;         // low-bit: [rows_per_block][d_r] rotated keys, then row maxima
  int* amax = (int*)(rows + rows_per_block * d.d_r);
  const int b = blockIdx.y;
  const int dt = delta[3 * b], dh = delta[3 * b + 1], dw = delta[3 * b + 2];
  if (dt == 0 && (d.rope_dims == 1 || (dh == 0 && dw == 0))) return;
  const double coord[3] = {(double)dt, (double)dh, (double)dw};
  rope_table(d, coord, cosv, sinv);
  const int s0 = slot_begin + blockIdx.x * rows_per_block;
  const int nrow = min(rows_per_block, slot_begin + n_slots - s0);
  if (LOWBIT)
    for (int r = threadIdx.x; r < nrow; r += blockDim.x) amax[r] = 0;
  __syncthreads();
  const int npair = d.d_r / 2;
  const size_t rs_base = (size_t)batch * g.capacity * (d.d_c / 32);   // per-token rotary scales
  const size_t rot_off = (size_t)d.d_c * content_bits(d) / 8;        // low-bit: rotary codes in a row
  for (int e = threadIdx.x; e < nrow * npair; e += blockDim.x) {
    const int r = e / npair, p = e % npair;
    const size_t srow = (size_t)b * g.capacity + s0 + r;
    float x0, x1;
    if (!LOWBIT) {
      const T* k = (const T*)cache + srow * d.d_qk + d.d_c;
      x0 = Elem<T>::load(k, 2 * p);
      x1 = Elem<T>::load(k, 2 * p + 1);
    } else {
      // INT4 rotary codes: element 2p in the low nibble of byte p
      const int byte = ((const uint8_t*)cache)[srow * code_row_bytes(d) + rot_off + p];
      const float s = __half2float(aux[rs_base + srow]);
      x0 = (float)(((byte & 15) ^ 8) - 8) * s;
      x1 = (float)(((byte >> 4) ^ 8) - 8) * s;
    }
    const float c = cosv[p], sn = sinv[p];
    const float r0 = round_to<T>(x0 * c - x1 * sn), r1 = round_to<T>(x0 * sn + x1 * c);
    if (!LOWBIT) {
      T* k = (T*)cache + srow * d.d_qk + d.d_c;
      Elem<T>::store(k, 2 * p, r0);
      Elem<T>::store(k, 2 * p + 1, r1);
    } else {
      rows[r * d.d_r + 2 * p] = r0;
      rows[r * d.d_r + 2 * p + 1] = r1;
      // row maximum of |x| (non-negative floats order as their bit patterns)
      atomicMax(&amax[r], __float_as_int(fmaxf(fabsf(r0), fabsf(r1))));
    }
  }
  if (LOWBIT) {
    // every code of these rows is read before any is rewritten; then the
    // quantiser of the append, one byte (two codes) per thread
    __syncthreads();
    for (int e = threadIdx.x; e < nrow * npair; e += blockDim.x) {
      const int r = e / npair, p = e % npair;
      const size_t srow = (size_t)b * g.capacity + s0 + r;
      const __half s16 = __float2half_rn(__int_as_float(amax[r]) / 7.f);
      const float s = __half2float(s16);
      int byte = 0;
      for (int k = 0; k < 2; ++k) {
        int q = 0;
        if (s != 0.f) q = (int)fminf(fmaxf(rintf(rows[r * d.d_r + 2 * p + k] / s), -8.f), 7.f);
        byte |= (q & 15) << (4 * k);
      }
      ((uint8_t*)cache)[srow * code_row_bytes(d) + rot_off + p] = (uint8_t)byte;
      if (p == 0) aux[rs_base + srow] = s16;
    }
  }
}

// rows per work-group of the shift: 64 dense; low-bit rows are held in LDS
inline int rope_shift_rows(const Dims& d) { return lowbit_cache(d) ? max(1, min(64, 4096 / d.d_r)) : 64; }

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
hipError_t launch_append_store(const Dims& d, const Geo& g, int batch, const float* y, int n_tokens,
                               const int* frame, void* cache, void* aux, int nsplit, hipStream_t st) {
  dim3 grid(n_tokens, batch);
  const size_t shm = lowbit_cache(d) ? (size_t)d.d_qk * sizeof(float) : 0;
  // one thread per work item (content element or rotary pair), at most 1024
  const int items = d.d_c + d.d_r / 2;
  const int threads = min(1024, (items + 63) / 64 * 64);
  if (lowbit_cache(d))
    append_store_kernel<bf16_t, true><<<grid, threads, shm, st>>>(d, g, y, n_tokens, frame, cache, (__half*)aux, batch, nsplit);
  else if (d.dtype == MLA_BF16)
    append_store_kernel<bf16_t, false><<<grid, threads, shm, st>>>(d, g, y, n_tokens, frame, cache, nullptr, batch, nsplit);
  else
    append_store_kernel<float, false><<<grid, threads, shm, st>>>(d, g, y, n_tokens, frame, cache, nullptr, batch, nsplit);
  return hipGetLastError();
}

hipError_t launch_q_rope(const Dims& d, const Geo& g, int batch, const void* q_rope, int n_q,
                         const int* q_first, const void* q_nope, void* q_abs, hipStream_t st) {
  dim3 grid(n_q, batch, (d.H + 15) / 16);
  size_t shm = (size_t)d.d_r * sizeof(float);
  if (d.dtype == MLA_BF16)
    q_rope_kernel<bf16_t><<<grid, 256, shm, st>>>(d, g, (const bf16_t*)q_rope, n_q, q_first, (const bf16_t*)q_nope,
                                                  (bf16_t*)q_abs);
  else
    q_rope_kernel<float><<<grid, 256, shm, st>>>(d, g, (const float*)q_rope, n_q, q_first, (const float*)q_nope,
                                                 (float*)q_abs);
  return hipGetLastError();
}

hipError_t launch_dequant(const Dims& d, const Geo& g, int batch, const void* cache, const void* aux,
                          float* out, hipStream_t st) {
  const size_t total = (size_t)batch * g.capacity * d.d_qk;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 65536) blocks = 65536;
  if (lowbit_cache(d))
    dequant_kernel<bf16_t, true><<<blocks, 256, 0, st>>>(d, g, batch, cache, (const __half*)aux, out);
  else if (d.dtype == MLA_BF16)
    dequant_kernel<bf16_t, false><<<blocks, 256, 0, st>>>(d, g, batch, cache, nullptr, out);
  else
    dequant_kernel<float, false><<<blocks, 256, 0, st>>>(d, g, batch, cache, nullptr, out);
  return hipGetLastError();
}

hipError_t launch_rope_shift(const Dims& d, const Geo& g, int batch, const int* delta, int slot_begin,
                             int n_slots, void* cache, void* aux, hipStream_t st) {
  const int rpb = rope_shift_rows(d);
  dim3 grid((n_slots + rpb - 1) / rpb, batch);
  const size_t shm = (size_t)d.d_r * sizeof(float) + (lowbit_cache(d) ? (size_t)rpb * (d.d_r + 1) * sizeof(float) : 0);
  if (lowbit_cache(d))
    rope_shift_kernel<bf16_t, true><<<grid, 256, shm, st>>>(d, g, batch, delta, slot_begin, n_slots, rpb, cache,
                                                             (__half*)aux);
  else if (d.dtype == MLA_BF16)
    rope_shift_kernel<bf16_t, false><<<grid, 256, shm, st>>>(d, g, batch, delta, slot_begin, n_slots, rpb, cache,
                                                              nullptr);
  else
    rope_shift_kernel<float, false><<<grid, 256, shm, st>>>(d, g, batch, delta, slot_begin, n_slots, rpb, cache,
                                                             nullptr);
  return hipGetLastError();
}

}  // namespace mla
