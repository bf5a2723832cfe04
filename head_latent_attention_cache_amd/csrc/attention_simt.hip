// Latent attention, generic SIMT kernel (any width, fp32 / bf16 / INT4 / INT2 cache).
//
// "Multi-Head Latent Attention" concept page, Low-rank joint compression:
// with W^UK absorbed into the query every head scores the shared cache row
// directly, in latent space, and The RoPE problem, and the
// decoupled fix: the score is the content term plus the rotary term, i.e. one
// dot product with the concatenated row [c_kv | k_rope].  The value of a key is
// its content latent c_kv (W^UV is applied after attention).
//
// This kernel is the full-precision path (fp32 storage) and serves any shape
// the MFMA kernel does not cover.  A block owns RB consecutive (token, head)
// rows of one sequence, stages the query rows and a tile of KT cache rows (as
// fp32) in LDS, and keeps an online softmax per row.
#include "launch.hpp"

namespace mla {

constexpr int SIMT_RB = 8;        // rows per block
constexpr int SIMT_MAXU = 32;     // d_c <= 32 * 32


template <typename T, bool LOWBIT>
__global__ __launch_bounds__(256) void attn_simt_kernel(AttnArgs a, int KT) {
  extern __shared__ float smem[];
  const Dims& d = a.d;
  const int dqk = d.d_qk;
  float* qs = smem;                          // [RB][dqk]
  float* ks = qs + SIMT_RB * dqk;            // [KT][dqk]
  float* sc = ks + KT * dqk;                 // [RB][KT]
  float* row_m = sc + SIMT_RB * KT;          // [RB]
  float* row_l = row_m + SIMT_RB;            // [RB]
  float* row_a = row_l + SIMT_RB;            // [RB] rescale factor of this tile
  int* row_fq = (int*)(row_a + SIMT_RB);     // [RB]

  const int b = blockIdx.y;
  const int r0 = blockIdx.x * SIMT_RB;
  const int tid = threadIdx.x;
  const int newest = a.newest[b];
  int nm = newest % a.g.window;
  if (nm < 0) nm += a.g.window;
  const T* q = (const T*)a.q_abs + (size_t)b * a.n_rows * dqk;

  for (int e = tid; e < SIMT_RB * dqk; e += blockDim.x) {
    const int r = e / dqk, j = e % dqk;
    qs[e] = (r0 + r < a.n_rows) ? Elem<T>::load(q, (size_t)(r0 + r) * dqk + j) : 0.f;
  }
  if (tid < SIMT_RB) {
    row_m[tid] = -INFINITY;
    row_l[tid] = 0.f;
    const int t = (r0 + tid) / d.H;
    row_fq[tid] = a.q_first[b] + t / a.g.P;
  }
  const int my_r = tid / 32;                 // output row of this thread
  const int my_j0 = tid % 32;                // dims my_j0 + 32 u
  const int nu = d.d_c / 32;
  float acc[SIMT_MAXU];
#pragma unroll
  for (int u = 0; u < SIMT_MAXU; ++u) acc[u] = 0.f;
  const float scale_log2 = d.scale * 1.4426950408889634f;
  const int ng = d.d_c / 32;
  __syncthreads();

  for (int s0 = 0; s0 < a.g.capacity; s0 += KT) {
    // stage KT cache rows as fp32; never-written slots (whose bytes are
    // whatever the allocation held) are staged as zeros so that a masked
    // probability of 0 never meets a NaN
    for (int e = tid; e < KT * dqk; e += blockDim.x) {
      const int k = e / dqk, j = e % dqk, s = s0 + k;
      float v = 0.f;
      if (s < a.g.capacity && ring_frame(s / a.g.P, newest, nm, a.g.window) >= 0) {
        const size_t srow = (size_t)b * a.g.capacity + s;
        if (!LOWBIT) {
          v = Elem<T>::load((const T*)a.cache, srow * dqk + j);
        } else {
          const int qv = lowbit_code((const uint8_t*)a.cache + srow * code_row_bytes(d), d, j);
          const float sc16 = j < d.d_c ? __half2float(a.aux[srow * ng + j / 32])
                                       : __half2float(a.aux[(size_t)a.batch * a.g.capacity * ng + srow]);
          v = (float)qv * sc16;
        }
      }
      ks[e] = v;
    }
    __syncthreads();
    // scores (log2 domain), masked
    for (int e = tid; e < SIMT_RB * KT; e += blockDim.x) {
      const int r = e / KT, k = e % KT, s = s0 + k;
      float v = -INFINITY;
      if (s < a.g.capacity && r0 + r < a.n_rows) {
        const int fk = ring_frame(s / a.g.P, newest, nm, a.g.window);
        if (key_visible(row_fq[r], fk, a.g.window, a.g.fpb)) {
          float dot = 0.f;
          const float* qr = qs + r * dqk;
          const float* kr = ks + k * dqk;
          if (!a.kscale) {
            for (int j = 0; j < dqk; ++j) dot = fmaf(qr[j], kr[j], dot);
          } else {
            // QK normalisation: the content term times the key's inverse RMS
            for (int j = 0; j < d.d_c; ++j) dot = fmaf(qr[j], kr[j], dot);
            dot *= a.kscale[(size_t)b * a.g.capacity + s];
            for (int j = d.d_c; j < dqk; ++j) dot = fmaf(qr[j], kr[j], dot);
          }
          v = dot * scale_log2;
        }
      }
      sc[e] = v;
    }
    __syncthreads();
    // online softmax bookkeeping, one thread per row
    if (tid < SIMT_RB) {
      float mx = row_m[tid];
      for (int k = 0; k < KT; ++k) mx = fmaxf(mx, sc[tid * KT + k]);
      const float m_use = (mx == -INFINITY) ? 0.f : mx;
      const float alpha = (row_m[tid] == -INFINITY) ? 0.f : exp2f(row_m[tid] - m_use);
      float sum = 0.f;
      for (int k = 0; k < KT; ++k) {
        const float p = exp2f(sc[tid * KT + k] - m_use);
        sc[tid * KT + k] = p;
        sum += p;
      }
      row_l[tid] = row_l[tid] * alpha + sum;
      row_m[tid] = mx;
      row_a[tid] = alpha;
    }
    __syncthreads();
    {
      const float alpha = row_a[my_r];
#pragma unroll
      for (int u = 0; u < SIMT_MAXU; ++u) {
        if (u < nu) {
          float o = acc[u] * alpha;
          const int j = my_j0 + 32 * u;
          for (int k = 0; k < KT; ++k) o = fmaf(sc[my_r * KT + k], ks[k * dqk + j], o);
          acc[u] = o;
        }
      }
    }
    __syncthreads();
  }

  const int R = r0 + my_r;
  if (R < a.n_rows) {
    const float l = row_l[my_r];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    T* out = (T*)a.o_lat + ((size_t)b * a.n_rows + R) * d.d_c;
#pragma unroll
    for (int u = 0; u < SIMT_MAXU; ++u)
      if (u < nu) Elem<T>::store(out, my_j0 + 32 * u, acc[u] * inv);
    if (a.lse && my_j0 == 0)
      a.lse[(size_t)b * a.n_rows + R] = l > 0.f ? (row_m[my_r] + log2f(l)) * 0.6931471805599453f : -INFINITY;
  }
}

size_t simt_lds_bytes(int dqk, int KT) {
  return (size_t)(SIMT_RB * dqk + KT * dqk + SIMT_RB * KT + 4 * SIMT_RB) * sizeof(float);
}

int simt_key_tile(int dqk) {
  int kt = 24576 / dqk;   // staged key tile + query rows stay below 160 KB of LDS
  if (kt > 32) kt = 32;
  if (kt < 1) kt = 1;
  return kt;
}

hipError_t launch_attn_simt(const AttnArgs& a, hipStream_t st) {
  const int KT = simt_key_tile(a.d.d_qk);
  const size_t shm = simt_lds_bytes(a.d.d_qk, KT);
  dim3 grid((a.n_rows + SIMT_RB - 1) / SIMT_RB, a.batch);
  const void* fn = lowbit_cache(a.d) ? (const void*)attn_simt_kernel<bf16_t, true>
                   : a.d.dtype == MLA_BF16         ? (const void*)attn_simt_kernel<bf16_t, false>
                                                   : (const void*)attn_simt_kernel<float, false>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  if (lowbit_cache(a.d))
    attn_simt_kernel<bf16_t, true><<<grid, 256, shm, st>>>(a, KT);
  else if (a.d.dtype == MLA_BF16)
    attn_simt_kernel<bf16_t, false><<<grid, 256, shm, st>>>(a, KT);
  else
    attn_simt_kernel<float, false><<<grid, 256, shm, st>>>(a, KT);
  return hipGetLastError();
}

}  // namespace mla
