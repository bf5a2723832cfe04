// The skinny bf16 product (M <= 32 rows: decode-time projections, bound by
// the weight stream) as a device function of its work-group coordinates, so
// that it can share a launch with independent work.
#pragma once
#include "launch.hpp"

namespace mla {
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// skinny bf16 kernel for M <= 32 (decode-time products, weight-bandwidth bound)
//   work-group (bx, by, bz): all M rows x BN output columns (column block bx,
//   K split by, batch entry bz).  The weight block of a K
//   stage (BN weight rows x SEG elements) is read with fully coalesced 16-byte
//   loads (each wave instruction covers 1 KB of consecutive row bytes),
//   staged through registers into LDS, and read back as MFMA B fragments; the
//   SEG / 16 MFMA steps of a stage are split over the 4 waves, each step
//   serving BN / 32 column blocks with one activation fragment.  The
//   activation (A) is re-read once per work-group, so wider tiles cut that
//   traffic.  SK_NST stages are in flight per wave; every load is
//   unconditional (addresses clamped into the operand, values zeroed by
//   mask), so the compiler's load counting keeps the later stages in flight
//   while one is consumed.  The activation fragments come straight from
//   global memory (cache-resident).  The four wave partials are summed in
//   LDS at the end (fixed order).
//   Optional split of the K range over work-groups (coordinate by) writes float
//   partials at C + split * sSplit for the caller to sum.
// ---------------------------------------------------------------------------
constexpr int SK_BN = 64, SK_SEG = 256;
template <int SK_NST, int BN, int SEG>
__device__ __forceinline__ void skinny_gemm_body(const GemmArgs& a, int bx, int by, int bz) {
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  constexpr int CPR = SEG / 8;                 // 16-byte chunks per weight row and stage
  static_assert(CPR % 16 == 0, "the row swizzle permutes chunks in groups of 16");
  constexpr int WLOADS = BN * CPR / 256;       // 16-byte weight loads per lane and stage
  constexpr int NB = BN / 32;                  // 32-column MFMA blocks
  constexpr int TSTEPS = SEG / 64;             // 16-wide MFMA steps per wave and stage
  static_assert(BN % 32 == 0 && SEG % 64 == 0 && (BN * CPR) % 256 == 0, "skinny tile");
  // two weight stages; the wave-partial reduction at the end reuses the space
  constexpr int WB_BYTES = BN * SEG * 2, RED_BYTES = 4 * NB * 64 * 17 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t wsm[2 * WB_BYTES > RED_BYTES ? 2 * WB_BYTES : RED_BYTES];
  uint8_t (*wbuf)[WB_BYTES] = (uint8_t (*)[WB_BYTES])wsm;
  const int z = bz;
  const bf16_t* A = (const bf16_t*)a.A + (size_t)z * a.sA;
  const bf16_t* B = (const bf16_t*)a.B + (size_t)z * a.sB;
  const int n0 = bx * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  // K stages of this work-group
  const int kst = (a.K + SEG - 1) / SEG;
  const int wg_st = (kst + a.ksplit - 1) / a.ksplit;
  const int s_begin = by * wg_st;
  const int s_end = min(s_begin + wg_st, kst);
  const int k_last = a.K - 8;   // K % 8 == 0: a clamped 8-element load stays inside the row

  // weight loads: load q of this lane takes linear chunk (q * 4 + wave) * 64 + lane
  // of the stage block (row-major [BN][CPR]), so each wave instruction reads
  // 1 KB of consecutive row bytes; LDS keeps a row's chunk c at position
  // c ^ (row & 15): a row is a multiple of 256 bytes, so every row starts at
  // the same bank, and the fragment reads take 16 consecutive rows (one chunk
  // each) per 16-lane phase of the 64-bank LDS: the 16 rows land on 16
  // distinct 16-byte bank groups, and the row-major stores stay a
  // permutation of each row's chunks
  const bf16_t* wrow[WLOADS];
  int wcol[WLOADS], wlds[WLOADS];
#pragma unroll
  for (int q = 0; q < WLOADS; ++q) {
    const int L = (q * 4 + wave) * 64 + lane;
    const int r = L / CPR, c = L % CPR;
    wrow[q] = B + (size_t)min(n0 + r, a.N - 1) * a.ldb;
    wcol[q] = c * 8;
    wlds[q] = r * (SEG * 2) + ((c ^ (r & 15)) << 4);
  }
  // fragments: lane (l32, g) of MFMA step t of this wave reads chunk
  // c = 2 * (TSTEPS * wave + t) + g of weight row 32 * j + l32 (B, block j)
  // and of activation row l32 (A)
  const bool m_ok = l32 < a.M;
  const bf16_t* arow = A + (size_t)(m_ok ? l32 : 0) * a.lda;

  struct Stage { u32x4v w[WLOADS], x[TSTEPS]; int s; };
  auto load_stage = [&](Stage& st, int sidx) {
    st.s = min(sidx, s_end);
    const int sc = min(sidx, s_end - 1);
#pragma unroll
    for (int q = 0; q < WLOADS; ++q)
      st.w[q] = *(const u32x4v*)(wrow[q] + min(sc * SEG + wcol[q], k_last));
#pragma unroll
    for (int t = 0; t < TSTEPS; ++t)
      st.x[t] = *(const u32x4v*)(arow + min(sc * SEG + (2 * (TSTEPS * wave + t) + g) * 8, k_last));
  };
  f32x16_t acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  int buf = 0;
  auto use_stage = [&](const Stage& st) {
    if (st.s >= s_end) return;   // empty stage (wave-uniform)
    lds_u8* wb = (lds_u8*)wbuf[buf];
#pragma unroll
    for (int q = 0; q < WLOADS; ++q) *(__attribute__((address_space(3))) u32x4v*)(wb + wlds[q]) = st.w[q];
    // barrier without __syncthreads()'s fence, which would also wait for the
    // global loads of the later stages: only this stage's LDS writes must land
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int t = 0; t < TSTEPS; ++t) {
      const int c = 2 * (TSTEPS * wave + t) + g;
      const int k = st.s * SEG + c * 8;
      // zeroing by mask (a select would be folded into the load's address)
      const uint32_t ma = (k < a.K && m_ok) ? ~0u : 0u;
      const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, st.x[t] & ma);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int r = 32 * j + l32;
        const u32x4v wv = *(const __attribute__((address_space(3))) u32x4v*)(wb + r * (SEG * 2) + ((c ^ (r & 15)) << 4));
        const uint32_t mb = (k < a.K && n0 + r < a.N) ? ~0u : 0u;
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, __builtin_bit_cast(bf16x8_t, wv & mb), acc[j], 0, 0, 0);
      }
    }
    buf ^= 1;
  };
  if (s_begin < s_end) {
    // every load is issued inside the loop (the first pass consumes empty
    // stages), so the outstanding-load count at the loop head is the same on
    // entry and on the back edge
    Stage st[SK_NST];
    const u32x4v zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < SK_NST; ++i) {
      st[i].s = s_end;
#pragma unroll
      for (int q = 0; q < WLOADS; ++q) st[i].w[q] = zero;
#pragma unroll
      for (int t = 0; t < TSTEPS; ++t) st[i].x[t] = zero;
    }
    for (int c = s_begin - SK_NST; c < s_end; c += SK_NST) {
#pragma unroll
      for (int i = 0; i < SK_NST; ++i) {
        use_stage(st[i]);
        load_stage(st[i], c + i + SK_NST);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // sum the four wave partials (fixed order) and store
  __syncthreads();
  float* red = (float*)wsm;   // [4 waves][NB][64 lanes][17]
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) red[((wave * NB + j) * 64 + lane) * 17 + e] = acc[j][e];
  __syncthreads();
  for (int o = tid; o < NB * 64 * 16; o += 256) {
    const int e = o & 15, l = (o >> 4) & 63, j = o >> 10;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) v += red[((w * NB + j) * 64 + l) * 17 + e];
    const int mm = 8 * (e / 4) + 4 * (l / 32) + (e % 4);
    const int nn = n0 + 32 * j + (l & 31);
    if (mm < a.M && nn < a.N) {
      if (a.ksplit > 1)
        ((float*)a.C)[(size_t)by * a.sSplit + (size_t)z * a.sC + (size_t)mm * a.ldc + nn] = v;
      else if (a.out_f32)
        ((float*)a.C)[(size_t)z * a.sC + (size_t)mm * a.ldc + nn] = v;
      else
        ((bf16_t*)a.C)[(size_t)z * a.sC + (size_t)mm * a.ldc + nn] = f32_to_bf16(v);
    }
  }
}

}  // namespace mla
