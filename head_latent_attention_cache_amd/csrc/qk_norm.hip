// QK-normalised MLA: the static weights folded into the key up-projection,
// the Gram matrix of the key up-projection, the per-slot key inverse RMS and
// the query's inverse RMS.
//
// "Multi-Head Latent Attention" topic page, QK-Norm abstract: post-projection
// RMSNorm of query and key splits into a static per-dimension weight (folded
// into the query-side projection) and a dynamic RMS statistic, which for the
// key is one scalar per token because every head's key is projected from the
// one cached latent.  The norm covers the content query / key of all heads
// of a token together (H * d_nope values), with eps inside the root:
//   key:   ||W^UK c||^2 = sum_h ||w_uk[h]^T c||^2 = c^T G c,  G = sum_h w_uk[h] w_uk[h]^T
//   inv_k = 1 / sqrt(c^T G c / (H d_nope) + eps),  inv_q = 1 / sqrt(mean(q_nope^2) + eps)
#include "launch.hpp"

namespace mla {

// ---------------------------------------------------------------------------
// w_uk_folded[h][a][i] = w_uk[h][a][i] * g_q[h][i] * g_k[h][i] (fp32 product,
// one rounding to the storage type)
// ---------------------------------------------------------------------------
template <typename T>
__global__ void qkn_fold_kernel(Dims d, const T* __restrict__ w_uk, const T* __restrict__ g_q,
                                const T* __restrict__ g_k, T* __restrict__ out) {
  const size_t n = (size_t)d.H * d.d_c * d.d_nope;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
    const int i = (int)(e % d.d_nope);
    const int h = (int)(e / ((size_t)d.d_c * d.d_nope));
    const size_t gi = (size_t)h * d.d_nope + i;
    Elem<T>::store(out, e, Elem<T>::load(w_uk, e) * (Elem<T>::load(g_q, gi) * Elem<T>::load(g_k, gi)));
  }
}

// ---------------------------------------------------------------------------
// G[a][b] = sum over (h, i) of w_uk[h][a][i] * w_uk[h][b][i], fp32.  32 x 32
// output tile per work-group, the (h, i) range in chunks of 32 through LDS.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void qkn_gram_kernel(Dims d, const T* __restrict__ w_uk, float* __restrict__ gram) {
  __shared__ float As[32][33];
  __shared__ float Bs[32][33];
  const int a0 = blockIdx.y * 32, b0 = blockIdx.x * 32;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  const int K = d.H * d.d_nope;
  for (int k0 = 0; k0 < K; k0 += 32) {
    for (int e = threadIdx.x; e < 1024; e += 256) {
      const int r = e / 32, c = e % 32, k = k0 + c;
      const int h = k / d.d_nope, i = k % d.d_nope;
      const size_t base = (size_t)h * d.d_c * d.d_nope + i;
      As[r][c] = (a0 + r < d.d_c && k < K) ? Elem<T>::load(w_uk, base + (size_t)(a0 + r) * d.d_nope) : 0.f;
      Bs[r][c] = (b0 + r < d.d_c && k < K) ? Elem<T>::load(w_uk, base + (size_t)(b0 + r) * d.d_nope) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < 32; ++c)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v) acc[u][v] = fmaf(As[ty + 16 * u][c], Bs[tx + 16 * v][c], acc[u][v]);
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int a = a0 + ty + 16 * u, bb = b0 + tx + 16 * v;
      if (a < d.d_c && bb < d.d_c) gram[(size_t)a * d.d_c + bb] = acc[u][v];
    }
}

// ---------------------------------------------------------------------------
// inv_k of the rows of appended tokens: token i of sequence b (frame
// frame[b] + i / P, tok i % P) -> slot; c = the stored latent (low-bit:
// dequantised); t = G c (G symmetric: column j read as row j, coalesced),
// inv_k = 1 / sqrt(c . t / (H d_nope) + eps).  grid (ceil(n_tokens / tpb),
// B), tpb <= KN_TOK tokens per work-group (their latents in LDS); thread
// owns columns j = tid + 256 u.
// ---------------------------------------------------------------------------
constexpr int KN_TOK = 16;
constexpr int KN_MAXU = 4;   // d_c <= 1024

template <typename T, bool LOWBIT>
__global__ __launch_bounds__(256) void key_norm_kernel(Dims d, Geo g, int batch, int n_tokens, int tpb,
                                                       const int* __restrict__ frame, const float* __restrict__ gram,
                                                       const void* __restrict__ cache, const __half* __restrict__ aux,
                                                       float* __restrict__ kscale) {
  extern __shared__ float cs[];                 // [KN_TOK][d_c]
  __shared__ float red[4][KN_TOK];
  const int b = blockIdx.y, i0 = blockIdx.x * tpb;
  const int nt = min(tpb, n_tokens - i0);
  const int ng = d.d_c / 32;
  auto slot_of = [&](int i) { return ring_slot(g, frame[b] + i / g.P, i % g.P); };
  for (int e = threadIdx.x; e < nt * d.d_c; e += blockDim.x) {
    const int t = e / d.d_c, j = e % d.d_c;
    const size_t srow = (size_t)b * g.capacity + slot_of(i0 + t);
    float v;
    if (!LOWBIT) {
      v = Elem<T>::load((const T*)cache, srow * d.d_qk + j);
    } else {
      const int q = lowbit_code((const uint8_t*)cache + srow * code_row_bytes(d), d, j);
      v = (float)q * __half2float(aux[srow * ng + j / 32]);
    }
    cs[t * d.d_c + j] = v;
  }
  __syncthreads();
  float acc[KN_TOK][KN_MAXU];
#pragma unroll
  for (int t = 0; t < KN_TOK; ++t)
#pragma unroll
    for (int u = 0; u < KN_MAXU; ++u) acc[t][u] = 0.f;
  for (int k = 0; k < d.d_c; ++k) {
    float gk[KN_MAXU];
#pragma unroll
    for (int u = 0; u < KN_MAXU; ++u) {
      const int j = threadIdx.x + 256 * u;
      gk[u] = j < d.d_c ? gram[(size_t)k * d.d_c + j] : 0.f;
    }
#pragma unroll
    for (int t = 0; t < KN_TOK; ++t) {
      const float c = t < nt ? cs[t * d.d_c + k] : 0.f;
#pragma unroll
      for (int u = 0; u < KN_MAXU; ++u) acc[t][u] = fmaf(gk[u], c, acc[t][u]);
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int t = 0; t < KN_TOK; ++t) {
    float p = 0.f;
#pragma unroll
    for (int u = 0; u < KN_MAXU; ++u) {
      const int j = threadIdx.x + 256 * u;
      if (j < d.d_c && t < nt) p = fmaf(cs[t * d.d_c + j], acc[t][u], p);
    }
    for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
    if (lane == 0) red[wave][t] = p;
  }
  __syncthreads();
  if (threadIdx.x < nt) {
    const int t = threadIdx.x;
    const float q = red[0][t] + red[1][t] + red[2][t] + red[3][t];
    const float ms = q / (float)(d.H * d.d_nope) + d.qk_eps;
    kscale[(size_t)b * g.capacity + slot_of(i0 + t)] = ms > 0.f ? 1.f / sqrtf(ms) : 0.f;
  }
}

// ---------------------------------------------------------------------------
// query side: q_abs[b, t, :, 0:d_c] *= inv_q, inv_q = 1 / sqrt(mean over all
// heads of q_nope[b, t]^2 + eps).  grid (n_q, B).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void q_norm_kernel(Dims d, int n_q, const T* __restrict__ q_nope,
                                                     T* __restrict__ q_abs) {
  __shared__ float red[4];
  const int t = blockIdx.x, b = blockIdx.y;
  const size_t tok = (size_t)b * n_q + t;
  const int n = d.H * d.d_nope;
  const T* q = q_nope + tok * n;
  float p = 0.f;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const float v = Elem<T>::load(q, e);
    p = fmaf(v, v, p);
  }
  for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = p;
  __syncthreads();
  const float ms = (red[0] + red[1] + red[2] + red[3]) / (float)n + d.qk_eps;
  const float inv = ms > 0.f ? 1.f / sqrtf(ms) : 0.f;
  T* out = q_abs + tok * d.H * d.d_qk;
  for (int e = threadIdx.x; e < d.H * d.d_c; e += blockDim.x) {
    const size_t off = (size_t)(e / d.d_c) * d.d_qk + e % d.d_c;
    Elem<T>::store(out, off, Elem<T>::load(out, off) * inv);
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
hipError_t launch_qkn_prepare(const Dims& d, const void* w_uk, const void* g_q, const void* g_k, void* w_uk_folded,
                              float* gram, hipStream_t st) {
  const size_t n = (size_t)d.H * d.d_c * d.d_nope;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 65536);
  dim3 grid_g((d.d_c + 31) / 32, (d.d_c + 31) / 32);
  if (d.dtype == MLA_BF16) {
    qkn_fold_kernel<bf16_t><<<blocks, 256, 0, st>>>(d, (const bf16_t*)w_uk, (const bf16_t*)g_q, (const bf16_t*)g_k,
                                                    (bf16_t*)w_uk_folded);
    qkn_gram_kernel<bf16_t><<<grid_g, 256, 0, st>>>(d, (const bf16_t*)w_uk, gram);
  } else {
    qkn_fold_kernel<float><<<blocks, 256, 0, st>>>(d, (const float*)w_uk, (const float*)g_q, (const float*)g_k,
                                                   (float*)w_uk_folded);
    qkn_gram_kernel<float><<<grid_g, 256, 0, st>>>(d, (const float*)w_uk, gram);
  }
  return hipGetLastError();
}

hipError_t launch_key_norm(const Dims& d, const Geo& g, int batch, int n_tokens, const int* frame, const float* gram,
                           const void* cache, void* aux, hipStream_t st) {
  const int tpb = d.d_c <= 512 ? KN_TOK : KN_TOK / 2;   // latents staged in at most 32 KB
  dim3 grid((n_tokens + tpb - 1) / tpb, batch);
  const size_t shm = (size_t)tpb * d.d_c * sizeof(float);
  float* kscale = (float*)((char*)aux + key_scale_offset(d, (size_t)batch * g.capacity));
  if (lowbit_cache(d))
    key_norm_kernel<bf16_t, true><<<grid, 256, shm, st>>>(d, g, batch, n_tokens, tpb, frame, gram, cache,
                                                          (const __half*)aux, kscale);
  else if (d.dtype == MLA_BF16)
    key_norm_kernel<bf16_t, false><<<grid, 256, shm, st>>>(d, g, batch, n_tokens, tpb, frame, gram, cache, nullptr,
                                                           kscale);
  else
    key_norm_kernel<float, false><<<grid, 256, shm, st>>>(d, g, batch, n_tokens, tpb, frame, gram, cache, nullptr, kscale);
  return hipGetLastError();
}

hipError_t launch_q_norm(const Dims& d, int batch, int n_q, const void* q_nope, void* q_abs, hipStream_t st) {
  dim3 grid(n_q, batch);
  if (d.dtype == MLA_BF16)
    q_norm_kernel<bf16_t><<<grid, 256, 0, st>>>(d, n_q, (const bf16_t*)q_nope, (bf16_t*)q_abs);
  else
    q_norm_kernel<float><<<grid, 256, 0, st>>>(d, n_q, (const float*)q_nope, (float*)q_abs);
  return hipGetLastError();
}

}  // namespace mla
