// Roofline references measured on the device that runs the MLA kernels: a
// stream of independent bf16 MFMAs (the matrix-core rate the attention
// kernels are compared with) and a coalesced streaming read (the HBM rate of
// the decode cache read).  Measurement only: no MLA arithmetic here.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/mla_probe.h"

namespace mla {

namespace {

typedef __bf16 probe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float probe_f32x16 __attribute__((ext_vector_type(16)));

constexpr int PROBE_CHAINS = 4;      // independent accumulators per wave
constexpr int PROBE_ROUNDS = 4;      // MFMAs per chain per loop iteration

// a bf16 in [-1, 1) from 16 pseudo-random bits (the "lowbias32" 32-bit
// integer hash published by C. Wellons)
__device__ __forceinline__ __bf16 probe_rand_bf16(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
  return (__bf16)((float)(int)(x & 0xffffu) * (1.0f / 32768.0f) - 1.0f);
}

// each wave: iters * PROBE_ROUNDS * PROBE_CHAINS 32x32x16 bf16 MFMAs
// (2 * 32 * 32 * 16 flop each); one float per thread keeps the result live.
// toggle = 0: one fixed, small-integer operand pair; toggle = 1: two pairs of
// pseudo-random operands used in turn, so the multiplier inputs change on
// every instruction as they do with real data (more switching power)
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, int toggle, float* out) {
  probe_bf16x8 a, b, a1, b1;
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = toggle ? probe_rand_bf16(t * 32u + e) : (__bf16)((float)((threadIdx.x + e) & 7) * 0.0625f);
    b[e] = toggle ? probe_rand_bf16(t * 32u + 8 + e) : (__bf16)((float)((threadIdx.x * 3 + e) & 7) * 0.0625f);
    a1[e] = toggle ? probe_rand_bf16(t * 32u + 16 + e) : a[e];
    b1[e] = toggle ? probe_rand_bf16(t * 32u + 24 + e) : b[e];
  }
  probe_f32x16 acc[PROBE_CHAINS];
#pragma unroll
  for (int k = 0; k < PROBE_CHAINS; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < PROBE_ROUNDS; ++r)
#pragma unroll
      for (int k = 0; k < PROBE_CHAINS; ++k)
        acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((r + k) & 1 ? a1 : a, (r + k) & 1 ? b1 : b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < PROBE_CHAINS; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// grid-stride read of n16 16-byte words, four loads in flight per thread;
// the XOR of everything read is written per thread so no load is dead
__global__ __launch_bounds__(256) void probe_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
    x ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
    x ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

}  // namespace

double probe_mfma_flops(int n_workgroups, int iters) {
  return (double)n_workgroups * (256 / 64) * iters * PROBE_ROUNDS * PROBE_CHAINS * (2.0 * 32 * 32 * 16);
}

hipError_t launch_probe_mfma(int n_workgroups, int iters, int toggle, float* out, hipStream_t st) {
  probe_mfma_kernel<<<n_workgroups, 256, 0, st>>>(iters, toggle, out);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, size_t n_bytes, int n_workgroups, uint32_t* out, hipStream_t st) {
  probe_read_kernel<<<n_workgroups, 256, 0, st>>>((const uint4*)src, n_bytes / 16, out);
  return hipGetLastError();
}

}  // namespace mla

namespace {

thread_local std::string g_probe_error;

mla_status probe_fail(mla_status st, const char* msg) {
  g_probe_error = msg;
  return st;
}

mla_status probe_launched(hipError_t e, const char* what) {
  if (e == hipSuccess) return MLA_OK;
  g_probe_error = std::string(what) + ": " + hipGetErrorString(e);
  return MLA_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

const char* mla_probe_last_error(void) { return g_probe_error.c_str(); }

mla_status mla_probe_mfma(void* stream, int32_t n_workgroups, int32_t iters, int32_t toggle, float* out,
                          double* flops) {
  g_probe_error.clear();
  if (n_workgroups <= 0 || n_workgroups > (1 << 20) || iters <= 0 || iters > (1 << 24))
    return probe_fail(MLA_ERR_INVALID_ARG, "n_workgroups must be in [1, 2^20] and iters in [1, 2^24]");
  if (toggle != 0 && toggle != 1) return probe_fail(MLA_ERR_INVALID_ARG, "toggle must be 0 or 1");
  if (!out || !aligned16(out)) return probe_fail(MLA_ERR_INVALID_ARG, "out is NULL or not 16-byte aligned");
  if (flops) *flops = mla::probe_mfma_flops(n_workgroups, iters);
  return probe_launched(mla::launch_probe_mfma(n_workgroups, iters, toggle, out, (hipStream_t)stream), "MFMA probe");
}

mla_status mla_probe_hbm_read(void* stream, const void* src, int64_t n_bytes, int32_t n_workgroups,
                              uint32_t* out) {
  g_probe_error.clear();
  if (n_bytes <= 0 || n_bytes % 16) return probe_fail(MLA_ERR_INVALID_ARG, "n_bytes must be a positive multiple of 16");
  if (n_workgroups <= 0 || n_workgroups > (1 << 20))
    return probe_fail(MLA_ERR_INVALID_ARG, "n_workgroups must be in [1, 2^20]");
  if (!src || !aligned16(src)) return probe_fail(MLA_ERR_INVALID_ARG, "src is NULL or not 16-byte aligned");
  if (!out || !aligned16(out)) return probe_fail(MLA_ERR_INVALID_ARG, "out is NULL or not 16-byte aligned");
  return probe_launched(mla::launch_probe_read(src, (size_t)n_bytes, n_workgroups, out, (hipStream_t)stream),
                        "HBM read probe");
}

}  // extern "C"
