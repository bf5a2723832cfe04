// Internal launch interface between the C-ABI layer and the kernels.
#pragma once
#include "common.hpp"

namespace mla {

// C[z] = A[z] . B[z]^T, strides in elements
struct GemmArgs {
  int M, N, K, batch;
  const void* A; long long lda, sA;
  const void* B; long long ldb, sB;
  void* C; long long ldc, sC;
  int out_f32;  // 1: C is float, 0: C has the storage type
  // split of the K range over work-groups (skinny products only): partial
  // products go to C + s * sSplit (float) and the caller sums them
  int ksplit = 1;
  long long sSplit = 0;
};

// K splits the skinny product would use for an M x N x K problem (1 if not skinny)
int gemm_skinny_ksplit(int dtype, int M, int N, int K, int batch);

struct AttnArgs {
  Dims d;
  Geo g;
  int n_q, n_rows;         // rows per sequence = n_q * H, heads fastest
  const void* q_abs;
  const int* q_first;
  const int* newest;
  const void* cache;
  const __half* aux;
  const float* kscale = nullptr;   // QK normalisation: per-slot key inverse RMS [B, capacity], else null
  int batch;
  void* o_lat;
  float* lse;
};

hipError_t launch_gemm_nt(int dtype, const GemmArgs& a, hipStream_t st);
hipError_t launch_qkn_prepare(const Dims& d, const void* w_uk, const void* g_q, const void* g_k, void* w_uk_folded,
                              float* gram, hipStream_t st);
int key_norm_slices(const Dims& d, int batch, int n_tokens);
hipError_t launch_key_norm(const Dims& d, const Geo& g, int batch, int n_tokens, const int* frame, const float* gram,
                           const void* cache, void* aux, float* partial, hipStream_t st);
hipError_t launch_fold_query(const Dims& d, int d_cq, const void* w_uq, const void* w_uk, void* w_fold,
                             hipStream_t st);
hipError_t launch_append_store(const Dims& d, const Geo& g, int batch, const float* y, int n_tokens,
                               const int* frame, void* cache, void* aux, int nsplit, hipStream_t st);
// q_abs in one launch (content product and rotary half side by side) where
// absorb_rope_fusable(d, ga) holds; ga as for the content product
bool absorb_rope_fusable(const Dims& d, const GemmArgs& ga);
hipError_t launch_absorb_rope(const Dims& d, const Geo& g, const GemmArgs& ga, int batch, const void* q_rope, int n_q,
                              const int* q_first, void* q_abs, hipStream_t st);
hipError_t launch_q_rope(const Dims& d, const Geo& g, int batch, const void* q_rope, int n_q,
                         const int* q_first, const void* q_nope, void* q_abs, hipStream_t st);
hipError_t launch_dequant(const Dims& d, const Geo& g, int batch, const void* cache, const void* aux,
                          float* out, hipStream_t st);
hipError_t launch_rope_shift(const Dims& d, const Geo& g, int batch, const int* delta, int slot_begin,
                             int n_slots, void* cache, void* aux, hipStream_t st);
hipError_t launch_attn_simt(const AttnArgs& a, hipStream_t st);
bool attn_mfma_supported(const Dims& d, const Geo& g);
size_t attn_mfma_workspace(const Dims& d, const Geo& g, int batch, int n_rows);
hipError_t launch_attn_mfma(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t st);
bool attn_dsplit_supported(const Dims& d);
size_t attn_dsplit_workspace(const Dims& d, const Geo& g, int batch, int n_rows);
hipError_t launch_attn_dsplit(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t st);

}  // namespace mla
