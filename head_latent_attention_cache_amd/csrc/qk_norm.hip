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
// dequantised); inv_k = 1 / sqrt(c^T G c / (H d_nope) + eps).  grid
// (ceil(n_tokens / TPB), B, slices): the work-group's TPB latents sit in LDS
// (read as broadcasts); it takes the rows [z rows_per_slice, ...) of G, thread
// tid the rows k = tid + 256 u of those (16-byte loads along the row, each
// used for all TPB tokens; G stays resident in L2), accumulates c_k (G_k . c)
// per token, and the partial sums are added by a fixed tree.  With one slice
// the work-group writes inv_k; with several (few tokens: the rows of G spread
// over more work-groups) it writes its partial sum to `partial`
// [slices][B][n_tokens] and key_norm_finish adds them in slice order.  The
// result does not depend on scheduling.
// ---------------------------------------------------------------------------
template <typename T, bool LOWBIT, int TPB>
__global__ __launch_bounds__(256) void key_norm_kernel(Dims d, Geo g, int batch, int n_tokens, int rows_per_slice,
                                                       const int* __restrict__ frame, const float* __restrict__ gram,
                                                       const void* __restrict__ cache, const __half* __restrict__ aux,
                                                       float* __restrict__ kscale, float* __restrict__ partial) {
  extern __shared__ __attribute__((aligned(16))) float cs[];   // [TPB][d_c]
  __shared__ float red[4][TPB];
  const int b = blockIdx.y, i0 = blockIdx.x * TPB;
  const int nt = min(TPB, n_tokens - i0);
  const int ng = d.d_c / 32;
  auto srow_of = [&](int t) {
    return (size_t)b * g.capacity + ring_slot(g, frame[b] + (i0 + t) / g.P, (i0 + t) % g.P);
  };
  for (int e = threadIdx.x; e < TPB * d.d_c; e += blockDim.x) {
    const int t = e / d.d_c, j = e % d.d_c;
    float v = 0.f;
    if (t < nt) {
      const size_t srow = srow_of(t);
      if (!LOWBIT) {
        v = Elem<T>::load((const T*)cache, srow * d.d_qk + j);
      } else {
        const int q = lowbit_code((const uint8_t*)cache + srow * code_row_bytes(d), d, j);
        v = (float)q * __half2float(aux[srow * ng + j / 32]);
      }
    }
    cs[e] = v;
  }
  __syncthreads();
  float p[TPB];
#pragma unroll
  for (int t = 0; t < TPB; ++t) p[t] = 0.f;
  const int k_end = min(d.d_c, (int)(blockIdx.z + 1) * rows_per_slice);
  for (int k = blockIdx.z * rows_per_slice + threadIdx.x; k < k_end; k += blockDim.x) {
    const float4* gk = (const float4*)(gram + (size_t)k * d.d_c);
    float dot[TPB];
#pragma unroll
    for (int t = 0; t < TPB; ++t) dot[t] = 0.f;
#pragma unroll 16
    for (int j4 = 0; j4 < d.d_c / 4; ++j4) {
      const float4 gv = gk[j4];
#pragma unroll
      for (int t = 0; t < TPB; ++t) {
        const float4 cv = *(const float4*)(cs + t * d.d_c + 4 * j4);
        dot[t] = fmaf(gv.x, cv.x, dot[t]);
        dot[t] = fmaf(gv.y, cv.y, dot[t]);
        dot[t] = fmaf(gv.z, cv.z, dot[t]);
        dot[t] = fmaf(gv.w, cv.w, dot[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < TPB; ++t) p[t] = fmaf(cs[t * d.d_c + k], dot[t], p[t]);
  }
#pragma unroll
  for (int t = 0; t < TPB; ++t) {
    float v = p[t];
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6][t] = v;
  }
  __syncthreads();
  if (threadIdx.x < nt) {
    const int t = threadIdx.x;
    const float q = (red[0][t] + red[1][t]) + (red[2][t] + red[3][t]);
    if (partial) {
      partial[((size_t)blockIdx.z * batch + b) * n_tokens + i0 + t] = q;
    } else {
      const float ms = q / (float)(d.H * d.d_nope) + d.qk_eps;
      kscale[srow_of(t)] = ms > 0.f ? 1.f / sqrtf(ms) : 0.f;
    }
  }
}

__global__ void key_norm_finish(Dims d, Geo g, int batch, int n_tokens, int slices, const int* __restrict__ frame,
                                const float* __restrict__ partial, float* __restrict__ kscale) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= batch * n_tokens) return;
  const int b = e / n_tokens, i = e % n_tokens;
  float q = 0.f;
  for (int z = 0; z < slices; ++z) q += partial[((size_t)z * batch + b) * n_tokens + i];
  const float ms = q / (float)(d.H * d.d_nope) + d.qk_eps;
  kscale[(size_t)b * g.capacity + ring_slot(g, frame[b] + i / g.P, i % g.P)] = ms > 0.f ? 1.f / sqrtf(ms) : 0.f;
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

// row slices of G per token for a call: enough work-groups to spread the
// reads of G when there are few tokens (decode)
int key_norm_slices(const Dims& d, int batch, int n_tokens) {
  const long long groups = (long long)batch * n_tokens;
  if (groups >= 256) return 1;
  int z = 1;
  while (z < 8 && groups * z * 2 <= 512 && d.d_c / (z * 2) >= 64) z *= 2;
  return z;
}

hipError_t launch_key_norm(const Dims& d, const Geo& g, int batch, int n_tokens, const int* frame, const float* gram,
                           const void* cache, void* aux, float* partial, hipStream_t st) {
  // one token per work-group for short appends (decode: parallelism), eight
  // when there are many (each row of G read once per eight tokens)
  const bool many = n_tokens >= 64;
  const int tpb = many ? 8 : 1;
  const int slices = key_norm_slices(d, batch, n_tokens);
  const int rps = (d.d_c + slices - 1) / slices;
  if (slices == 1) partial = nullptr;
  dim3 grid((n_tokens + tpb - 1) / tpb, batch, slices);
  const size_t shm = (size_t)tpb * d.d_c * sizeof(float);
  float* kscale = (float*)((char*)aux + key_scale_offset(d, (size_t)batch * g.capacity));
#define KN_LAUNCH(T, LB, TPB)                                                                              \
  key_norm_kernel<T, LB, TPB><<<grid, 256, shm, st>>>(d, g, batch, n_tokens, rps, frame, gram, cache,      \
                                                      (const __half*)aux, kscale, partial)
  if (lowbit_cache(d)) {
    if (many) KN_LAUNCH(bf16_t, true, 8); else KN_LAUNCH(bf16_t, true, 1);
  } else if (d.dtype == MLA_BF16) {
    if (many) KN_LAUNCH(bf16_t, false, 8); else KN_LAUNCH(bf16_t, false, 1);
  } else {
    if (many) KN_LAUNCH(float, false, 8); else KN_LAUNCH(float, false, 1);
  }
#undef KN_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !partial) return e;
  const int n = batch * n_tokens;
  key_norm_finish<<<(n + 255) / 256, 256, 0, st>>>(d, g, batch, n_tokens, slices, frame, partial, kscale);
  return hipGetLastError();
}

}  // namespace mla
