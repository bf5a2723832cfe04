// Strided-batched "NT" products C[z] = A[z] . B[z]^T with fp32 accumulation.
//
// Every matrix product of the path has this form because every weight is
// stored output-feature major (row n of B is output feature n):
//   append    y      = x . w_dkr^T                       (one batch)
//   absorb    q_lat  = q_nope[:, h] . w_uk[h]^T           (batched over heads)
//   un-absorb o_h    = o_lat[:, h] . w_uv[h]^T            (batched over heads)
//             y      = o_heads . w_o^T                    (one batch)
//
// Two kernels: a bf16 MFMA kernel (v_mfma_f32_32x32x16_bf16, LDS double
// buffered) for bfloat16 storage, and a plain fp32 SIMT kernel for fp32
// storage (the small full-precision workloads).
#include "skinny_gemm.hpp"

namespace mla {


// ---------------------------------------------------------------------------
// fp32 SIMT kernel: 32 x 32 tile per 256 threads, 2 x 2 outputs per thread
// ---------------------------------------------------------------------------
template <typename TO>
__global__ __launch_bounds__(256) void gemm_nt_f32_kernel(GemmArgs a) {
  __shared__ float As[32][33];
  __shared__ float Bs[32][33];
  const int z = blockIdx.z;
  const float* A = (const float*)a.A + (size_t)z * a.sA;
  const float* B = (const float*)a.B + (size_t)z * a.sB;
  TO* C = (TO*)a.C + (size_t)z * a.sC;
  const int m0 = blockIdx.y * 32, n0 = blockIdx.x * 32;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  for (int k0 = 0; k0 < a.K; k0 += 32) {
    for (int e = threadIdx.x; e < 1024; e += 256) {
      const int r = e / 32, c = e % 32;
      const int m = m0 + r, n = n0 + r, k = k0 + c;
      As[r][c] = (m < a.M && k < a.K) ? A[(size_t)m * a.lda + k] : 0.f;
      Bs[r][c] = (n < a.N && k < a.K) ? B[(size_t)n * a.ldb + k] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < 32; ++k) {
      const float a0 = As[ty * 2][k], a1 = As[ty * 2 + 1][k];
      const float b0 = Bs[tx * 2][k], b1 = Bs[tx * 2 + 1][k];
      acc[0][0] = fmaf(a0, b0, acc[0][0]);
      acc[0][1] = fmaf(a0, b1, acc[0][1]);
      acc[1][0] = fmaf(a1, b0, acc[1][0]);
      acc[1][1] = fmaf(a1, b1, acc[1][1]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) {
      const int m = m0 + ty * 2 + i, n = n0 + tx * 2 + j;
      if (m < a.M && n < a.N) C[(size_t)m * a.ldc + n] = acc[i][j];
    }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
//   block tile BM x BN, K step 32, 4 waves in a 2 x 2 grid, each wave owns a
//   (BM/2) x (BN/2) sub-tile of 32 x 32 MFMA blocks.
//   LDS holds A and B K-slices as [row][32] bf16 with 16-byte chunks swizzled
//   by row so that the 16-byte fragment reads of 16 consecutive rows hit
//   distinct banks.  Global loads are 16 bytes per lane, prefetched into
//   registers one K step ahead.
//   Requirements (checked by the host): K % 8 == 0, lda/ldb % 8 == 0, 16-byte
//   aligned operands.  Ragged M, N and K tails are zero-filled.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int BM, int BN>
__global__ __launch_bounds__(256) void gemm_nt_bf16_kernel(GemmArgs a) {
  constexpr int BK = 32;                    // bf16 elements per K step = 4 chunks of 16 B
  constexpr int WM = BM / 2, WN = BN / 2;   // wave sub-tile
  constexpr int TM = WM / 32, TN = WN / 32; // MFMA blocks per wave
  constexpr int A_CHUNKS = BM * 4, B_CHUNKS = BN * 4;
  constexpr int A_PER_T = (A_CHUNKS + 255) / 256, B_PER_T = (B_CHUNKS + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * 64];

  const int z = blockIdx.z;
  const bf16_t* A = (const bf16_t*)a.A + (size_t)z * a.sA;
  const bf16_t* B = (const bf16_t*)a.B + (size_t)z * a.sB;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int wm = (wave / 2) * WM, wn = (wave % 2) * WN;

  u32x4_t ra[A_PER_T], rb[B_PER_T];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int c = tid + i * 256;
      const int r = c / 4, kc = c % 4;
      const int m = m0 + r, k = k0 + kc * 8;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (c < A_CHUNKS && m < a.M && k < a.K) v = *(const u32x4_t*)(A + (size_t)m * a.lda + k);
      ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int c = tid + i * 256;
      const int r = c / 4, kc = c % 4;
      const int n = n0 + r, k = k0 + kc * 8;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (c < B_CHUNKS && n < a.N && k < a.K) v = *(const u32x4_t*)(B + (size_t)n * a.ldb + k);
      rb[i] = v;
    }
  };
  // chunk kc of row r lives at byte r*64 + ((kc ^ ((r >> 2) & 3)) * 16)
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int c = tid + i * 256;
      if (c < A_CHUNKS) {
        const int r = c / 4, kc = c % 4;
        *(u32x4_t*)(&lds[buf][r * 64 + ((kc ^ ((r >> 2) & 3)) * 16)]) = ra[i];
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int c = tid + i * 256;
      if (c < B_CHUNKS) {
        const int r = c / 4, kc = c % 4;
        *(u32x4_t*)(&lds[buf][BM * 64 + r * 64 + ((kc ^ ((r >> 2) & 3)) * 16)]) = rb[i];
      }
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = (a.K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {           // two 16-wide MFMA K steps per BK
      const int kc = ks * 2 + lane / 32;       // 16-byte chunk holding this lane's 8 k values
      bf16x8_t fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm + i * 32 + lane % 32;
        fa[i] = *(const bf16x8_t*)(&lds[buf][r * 64 + ((kc ^ ((r >> 2) & 3)) * 16)]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn + j * 32 + lane % 32;
        fb[j] = *(const bf16x8_t*)(&lds[buf][BM * 64 + r * 64 + ((kc ^ ((r >> 2) & 3)) * 16)]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      lstore(buf ^ 1);
    }
    __syncthreads();
  }

  // C layout of a 32x32 block: lane l, value e -> row 8(e/4) + 4(l/32) + e%4, column l%32
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm + i * 32 + 8 * (e / 4) + 4 * (lane / 32) + (e % 4);
        const int n = n0 + wn + j * 32 + lane % 32;
        if (m < a.M && n < a.N) {
          if (a.out_f32)
            ((float*)a.C)[(size_t)z * a.sC + (size_t)m * a.ldc + n] = acc[i][j][e];
          else
            ((bf16_t*)a.C)[(size_t)z * a.sC + (size_t)m * a.ldc + n] = f32_to_bf16(acc[i][j][e]);
        }
      }
}

// the skinny product as a kernel of its own (grid: column blocks, K splits, batch)
template <int SK_NST, int BN, int SEG>
__global__ __launch_bounds__(256) void gemm_skinny_bf16_kernel(GemmArgs a) {
  skinny_gemm_body<SK_NST, BN, SEG>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

int gemm_skinny_ksplit(int dtype, int M, int N, int K, int batch) {
  if (dtype != MLA_BF16 || M > 32 || M <= 0) return 1;
  const int wgs = ((N + SK_BN - 1) / SK_BN) * batch;
  const int kst = (K + SK_SEG - 1) / SK_SEG;
  int ks = 1;
  // aim at >= 512 work-groups, keeping >= 4 K stages per work-group
  while (wgs * ks < 512 && kst / (ks * 2) >= 4) ks *= 2;
  return ks;
}

// ---------------------------------------------------------------------------
// load-time fold of the query and key up-projections ("Multi-Head Latent
// Attention" concept page, Low-rank joint compression: the product
// W^UQ^T W^UK can be formed once):
//   w_fold[h][a][j] = sum_i w_uk[h][a][i] * w_uq[h d_nope + i][j]
// fp32 accumulation in the order i = 0 .. d_nope - 1, rounded once to the
// storage type.  grid (ceil(d_cq / 256), ceil(d_c / FOLD_ROWS), H): a thread
// owns one column j of FOLD_ROWS rows a; the w_uq row segment is read once
// per work-group step (coalesced along j), the w_uk values are broadcasts.
// ---------------------------------------------------------------------------
constexpr int FOLD_ROWS = 8;

template <typename T>
__global__ __launch_bounds__(256) void fold_query_kernel(int d_nope, int d_c, int d_cq, const T* __restrict__ w_uq,
                                                         const T* __restrict__ w_uk, T* __restrict__ w_fold) {
  const int h = blockIdx.z, j = blockIdx.x * 256 + threadIdx.x, a0 = blockIdx.y * FOLD_ROWS;
  if (j >= d_cq) return;
  float acc[FOLD_ROWS];
#pragma unroll
  for (int r = 0; r < FOLD_ROWS; ++r) acc[r] = 0.f;
  const T* uk = w_uk + (size_t)h * d_c * d_nope;
  const T* uq = w_uq + (size_t)h * d_nope * d_cq + j;
  for (int i = 0; i < d_nope; ++i) {
    const float q = Elem<T>::load(uq, (size_t)i * d_cq);
#pragma unroll
    for (int r = 0; r < FOLD_ROWS; ++r)
      if (a0 + r < d_c) acc[r] = fmaf(Elem<T>::load(uk, (size_t)(a0 + r) * d_nope + i), q, acc[r]);
  }
  T* out = w_fold + (size_t)h * d_c * d_cq + j;
#pragma unroll
  for (int r = 0; r < FOLD_ROWS; ++r)
    if (a0 + r < d_c) Elem<T>::store(out, (size_t)(a0 + r) * d_cq, acc[r]);
}

hipError_t launch_fold_query(const Dims& d, int d_cq, const void* w_uq, const void* w_uk, void* w_fold,
                             hipStream_t st) {
  dim3 grid((d_cq + 255) / 256, (d.d_c + FOLD_ROWS - 1) / FOLD_ROWS, d.H);
  if (d.dtype == MLA_BF16)
    fold_query_kernel<bf16_t><<<grid, 256, 0, st>>>(d.d_nope, d.d_c, d_cq, (const bf16_t*)w_uq, (const bf16_t*)w_uk,
                                                    (bf16_t*)w_fold);
  else
    fold_query_kernel<float><<<grid, 256, 0, st>>>(d.d_nope, d.d_c, d_cq, (const float*)w_uq, (const float*)w_uk,
                                                   (float*)w_fold);
  return hipGetLastError();
}

hipError_t launch_gemm_nt(int dtype, const GemmArgs& a, hipStream_t st) {
  if (a.M == 0 || a.N == 0 || a.batch == 0) return hipSuccess;
  if (dtype == MLA_F32) {
    dim3 grid((a.N + 31) / 32, (a.M + 31) / 32, a.batch);
    if (a.out_f32) gemm_nt_f32_kernel<float><<<grid, 256, 0, st>>>(a);
    else gemm_nt_f32_kernel<float><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  if (a.M <= 32 && a.K <= 128 && a.ksplit == 1) {
    // one short K stage per work-group (absorbed query): 128 columns each
    dim3 grid((a.N + 127) / 128, 1, a.batch);
    gemm_skinny_bf16_kernel<1, 128, 128><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  if (a.M <= 32) {
    dim3 grid((a.N + SK_BN - 1) / SK_BN, a.ksplit, a.batch);
    // two K stages in flight (measured best for the 64-column tile: deeper
    // pipelines cost occupancy), one when the work-group has a single stage
    const int kst = (a.K + SK_SEG - 1) / SK_SEG;
    const int wg_st = (kst + a.ksplit - 1) / a.ksplit;
    if (wg_st >= 2) gemm_skinny_bf16_kernel<2, SK_BN, SK_SEG><<<grid, 256, 0, st>>>(a);
    else gemm_skinny_bf16_kernel<1, SK_BN, SK_SEG><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  // bf16: small-M products use 64-row tiles, wide ones 128 x 128
  if (a.M <= 64) {
    dim3 grid((a.N + 63) / 64, (a.M + 63) / 64, a.batch);
    gemm_nt_bf16_kernel<64, 64><<<grid, 256, 0, st>>>(a);
  } else {
    dim3 grid((a.N + 127) / 128, (a.M + 127) / 128, a.batch);
    gemm_nt_bf16_kernel<128, 128><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mla
