// Pieces shared by the MFMA latent-attention kernels (gfx950): LDS DMA and
// barrier helpers, the key-tile layout, tile classification and the key-split
// bookkeeping.
#pragma once
#include <cstdlib>
#include <cstring>

#include "launch.hpp"

namespace mla {
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))

constexpr int MF_WAVES = 4;
constexpr int MF_ROWS = 32 * MF_WAVES;   // rows per work-group
constexpr int MF_BN = 32;                // keys per tile
constexpr int MF_MAX_TPS = 2048;         // tiles per split (size of a class table)

// work-group barrier without the memory fence of __syncthreads(): the fence
// would wait for every outstanding global->LDS load (vmcnt(0)), including the
// tiles prefetched ahead.  Callers wait explicitly for what they need
// (vmcnt for the tile being consumed, lgkmcnt for their own LDS writes).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 * lane
// (global_load_lds_dwordx4).  Issued through asm so that the compiler does not
// track it: it has no result register, and the kernel orders it explicitly
// with s_waitcnt vmcnt before the barrier that publishes the tile (the
// compiler's own tracking would add vmcnt(0) waits in front of later
// transposed LDS reads, draining the prefetch pipeline).
// The compiler inserts no wait states in front of inline assembly, so each
// block carries its own: one after the scalar write of M0 that an LDS-DMA load
// reads, and five for a scalar base address, which the register allocator may
// restore with v_readlane (a VALU write of the SGPR) right before the block:
// a vector-memory read of an SGPR needs five wait states after a VALU write
// of it, or it sees the old value (a wrong address).
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(lds_base) : "memory");
}
// same, with a wave-uniform 64-bit base and a 32-bit per-lane byte offset
__device__ __forceinline__ void dma16_sv(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_base) : "memory");
}
// one dword per lane (same conventions as dma16)
__device__ __forceinline__ void dma4(const void* gsrc, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gsrc), "{m0}"(lds_base) : "memory");
}

// acc += A . B with v_mfma_f32_32x32x16_bf16, the accumulator in VGPRs (the
// builtin lets the register allocator pick AGPRs).  A chain of these on one
// accumulator needs no waits between steps (same-shape source-C forwarding,
// also with an independent MFMA between two steps); the chain's last step is
// mfma_vgpr_last(), which carries the wait states a later read needs.
__device__ __forceinline__ void mfma_vgpr(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// first step of a chain: acc = A . B (the accumulator operand is the inline
// constant 0, so acc needs no zeroing; early-clobber keeps it off A and B)
__device__ __forceinline__ void mfma_vgpr_zero(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
// the last step of a chain with its wait states (the 8-pass 32x32x16 MFMA
// needs about a dozen before a VALU or memory instruction reads its result;
// 20 are given) in the same asm statement: the compiler takes an asm's
// outputs as ready when the statement ends, so wait states in a statement of
// their own would not stop it from copying the accumulator to other
// registers between the MFMA and the waits
__device__ __forceinline__ void mfma_vgpr_last(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 15\n\ts_nop 3" : "+v"(acc) : "v"(a), "v"(b));
}

// wait states between a VALU write of the accumulator and an MFMA reading it
// (as the accumulator operand of the chain's next step)
__device__ __forceinline__ void mfma_vgpr_after_valu(f32x16_t& acc) {
  asm volatile("s_nop 4" : "+v"(acc));
}

// max / sum of a value over the two 32-lane halves of a wave (lane l and
// lane l ^ 32), with v_permlane32_swap (a VALU op; no LDS round trip): the
// swap of x with itself yields, per lane, the pair {own, other} in some order
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// four floats to four bf16 (round to nearest even, v_cvt_pk_bf16_f32; the
// same bits as the bit-level rounding for every finite value), packed
__device__ __forceinline__ u32x2_t pack4_bf16(float x0, float x1, float x2, float x3) {
  bf16x4_t v;
  v[0] = (__bf16)x0; v[1] = (__bf16)x1; v[2] = (__bf16)x2; v[3] = (__bf16)x3;
  return __builtin_bit_cast(u32x2_t, v);
}

// two floats to two bf16 in one word (round to nearest even, one
// v_cvt_pk_bf16_f32): lo in bits 0..15, hi in bits 16..31
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Eight cache values bf16(q * s) from their packed codes (the low-bit
// cache: INT4 or INT2 content codes, INT4 rotary codes) and their fp16 scale
// s (already converted, 0 for never-written slots).  Each value is rounded
// once to nearest even from the exact product (q * s is exact in fp32: at
// most 4 x 11 significant bits).  4-bit codes (`codes`: 8 nibbles, element
// 2i in the low nibble of byte i): offset binary (code ^ 8 = q + 8) in single
// bytes, byte to float, then q s = (q + 8) s - 8 s in one exact FMA.  2-bit
// codes (`codes`: bits 2k .. 2k + 1 of byte j hold element 4j + k): the four
// values bf16(q s), q = 0, 1, -2, -1 (two's complement), form an 8-byte table
// that v_perm_b32 indexes.
__device__ __forceinline__ u32x4_t dequant8_bf16(uint32_t codes, float sc, bool two_bit) {
  u32x4_t out;
  if (two_bit) {
    const uint32_t lut_lo = pack2_bf16(0.f, sc), lut_hi = pack2_bf16(-2.f * sc, -sc);
    const uint32_t w = codes | (codes << 14);   // code 2p + 1 copied to bit 4p + 16
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // codes 2p, 2p + 1 at bits 0 and 16, then byte selectors (2c, 2c + 1) per half
      const uint32_t t = (w >> (4 * p)) & 0x00030003u;
      out[p] = __builtin_amdgcn_perm(lut_hi, lut_lo, t * 0x202u + 0x01000100u);
    }
  } else {
    const uint32_t ev = (codes & 0x0F0F0F0Fu) ^ 0x08080808u;          // elements 0, 2, 4, 6
    const uint32_t od = ((codes >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;   // elements 1, 3, 5, 7
    const float off = -8.f * sc;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      out[p] = pack2_bf16(fmaf((float)((ev >> (8 * p)) & 0xFFu), sc, off),
                          fmaf((float)((od >> (8 * p)) & 0xFFu), sc, off));
  }
  return out;
}

// 16-byte chunk swizzle of a key row: chunk c of key k sits at position
// c ^ key_swizzle(k) of the row's 128 bytes (a key row spans half of the
// 256-byte, 64-bank LDS period).  Requirements:
//  * the 16-byte key reads of the scores are served 16 lanes (16 consecutive
//    keys, one chunk each, 256 bytes) per phase: keys of equal row parity
//    among any 16 aligned consecutive keys need distinct swizzles, and any 8
//    aligned consecutive keys need 8 distinct swizzles;
//  * the transposed 8-byte value reads (4 consecutive keys x 2 adjacent
//    chunks {2i, 2i+1} per 16-lane phase) need distinct chunk pairs over any
//    4 aligned consecutive keys, i.e. distinct key_swizzle(k) >> 1.
// (k & 3) << 1 | (k >> 2 & 1) meets the 8-key and 4-key conditions; bit 3 of
// the key flipping bit 1 of the swizzle separates keys k and k + 8 (a
// constant XOR inside each aligned group of 8 keeps the other two).  The
// bank-conflict counter of the video-chunk attention kernel reads 0.5 % of
// LDS-active cycles with it, 36 % without the bit-3 term.
__device__ __forceinline__ int key_swizzle(int key) {
  return (((key & 3) << 1) | ((key >> 2) & 1)) ^ ((key >> 2) & 2);
}

// Launch plan of an attention kernel: work-group (b, split, row block)
// attends the split's key tiles; where a row block has more than one split it
// writes a normalised partial output (bf16, the output precision) and an fp32
// LSE per row, merged afterwards in a fixed split order with fp32 weights.
// Two groups of row blocks may use different split counts: rows blocks
// [0, n_a) of every sequence with ns_a splits (the large pieces, dispatched
// first on every XCD), [n_a, n_rb) with ns_b (the small pieces that fill the
// last round).  ns_a == ns_b is the uniform plan.
// (Measured on the chunk workloads: a schedule of whole row blocks with a
// stream-K tail ran slower than key splits, because work-groups at staggered
// key offsets no longer share L2 lines.)
struct MfmaArgs {
  AttnArgs a;
  int n_rb;          // row blocks per sequence
  int rows_wg;       // rows per row block (work-group)
  int tiles;         // key tiles per sequence
  int n_a;           // row blocks per sequence in the first group
  int ns_a, tps_a;   // splits and tiles per split of the first group
  int ns_b, tps_b;   // of the second group
  int nsplit;        // max(ns_a, ns_b): split slots of the partial buffers
  bf16_t* ws_o;      // [nsplit][B][n_rows][d_c] partial outputs (normalised, bf16)
  float* ws_lse;     // [nsplit][B][n_rows]
  // softmax: a row reruns the key loop once its maximum exceeds the fixed
  // reference by more than this many log2 units (64; smaller values make the
  // rerun fire on ordinary inputs, for testing)
  float rerun_log2;
};

// split count of row block rb (of any sequence)
__host__ __device__ __forceinline__ int plan_splits(const MfmaArgs& ma, int rb) {
  return rb < ma.n_a ? ma.ns_a : ma.ns_b;
}

// one contiguous key range of one row block handled by a work-group; the
// partial pointers address the row block's first row (null: final output)
struct Piece {
  int rbg;           // global row block: b * n_rb + rb
  int t0, t1;        // key tiles [t0, t1)
  bf16_t* part_o;
  float* part_lse;
};

// the piece of this work-group.  Work-group id runs on XCD id % 8 as number
// id / 8 of that XCD; every XCD takes its share of the first group's pieces
// first, then of the second group's, each group in (b, split, rb) order
// (consecutive work-groups of an XCD attend the same key range).  With
// `chip_order` and a one-group plan the pieces go in work-group id order
// instead: the 256 work-groups running at once (32 per XCD) attend one key
// range, so a key range too large for the L2s is streamed from HBM once into
// the last-level cache that all XCDs share, not once per pair of XCDs with
// four ranges competing for that cache.
__device__ __forceinline__ Piece wg_piece(const MfmaArgs& ma, bool chip_order = false) {
  const int B = ma.a.batch, n_rows = ma.a.n_rows, DC = ma.a.d.d_c;
  const int N = gridDim.x, id = blockIdx.x;
  const int x = id & 7, j = id >> 3;
  const int NB = B * ma.n_a * ma.ns_a;
  const int big_x = NB / 8 + (x < NB % 8 ? 1 : 0);
  const int big_before = x * (NB / 8) + min(x, NB % 8);
  int b, split, rb, tps;
  if (j < big_x) {
    const int k = chip_order && NB == N ? id : big_before + j;
    const int per_b = ma.ns_a * ma.n_a;
    b = k / per_b;
    split = (k % per_b) / ma.n_a;
    rb = k % ma.n_a;
    tps = ma.tps_a;
  } else {
    const int n_b = ma.n_rb - ma.n_a;
    const int k = (x * (N / 8) + min(x, N % 8)) - big_before + (j - big_x);
    const int per_b = ma.ns_b * n_b;
    b = k / per_b;
    split = (k % per_b) / n_b;
    rb = ma.n_a + k % n_b;
    tps = ma.tps_b;
  }
  Piece pc;
  pc.rbg = b * ma.n_rb + rb;
  pc.t0 = split * tps;
  pc.t1 = min(pc.t0 + tps, ma.tiles);
  pc.part_o = nullptr;
  pc.part_lse = nullptr;
  if (plan_splits(ma, rb) > 1) {
    const size_t row0 = ((size_t)split * B + b) * n_rows + (size_t)rb * ma.rows_wg;
    pc.part_o = ma.ws_o + row0 * DC;
    pc.part_lse = ma.ws_lse + row0;
  }
  return pc;
}

// frame range [f_min, f_max] held by the slots of a tile (ring positions rp0..rp1)
__device__ __forceinline__ void tile_frames(int rp0, int rp1, int newest, int nm, int W, int* fmin,
                                            int* fmax) {
  const int f0 = ring_frame(rp0, newest, nm, W), f1 = ring_frame(rp1, newest, nm, W);
  int lo = f0 < f1 ? f0 : f1, hi = f0 > f1 ? f0 : f1;
  const int wrap = nm + 1;                // first ring position after the newest frame
  if (wrap > rp0 && wrap <= rp1) {        // the tile crosses from newest back to oldest
    const int fa = ring_frame(wrap, newest, nm, W), fb = ring_frame(wrap - 1, newest, nm, W);
    lo = min(lo, min(fa, fb));
    hi = max(hi, max(fa, fb));
  }
  *fmin = lo;
  *fmax = hi;
}

// tile classes
enum : uint8_t { TILE_SKIP = 0, TILE_FULL = 1, TILE_MASKED = 2, TILE_MASKED_ZERO = 3 };

// class of key tile [k0, k0 + MF_BN) for the query frames [gfq_min, gfq_max]
// of a work-group: skipped (no visible key), fully visible, masked, or masked
// with never-written / past-the-end slots (their LDS bytes must be zeroed)
__device__ __forceinline__ uint8_t classify_tile(int k0, int cap, int P, int newest, int nm, int W, int fpb,
                                                 int gfq_min, int gfq_max) {
  const int k1 = min(k0 + MF_BN, cap) - 1;
  int fmin, fmax;
  tile_frames(k0 / P, k1 / P, newest, nm, W, &fmin, &fmax);
  const int fminw = fmin < 0 ? 0 : fmin;
  if (fmax < 0 || floor_div(fminw, fpb) > floor_div(gfq_max, fpb) || gfq_min - fmax >= W) return TILE_SKIP;
  if (fmin < 0 || k0 + MF_BN > cap) return TILE_MASKED_ZERO;
  if (floor_div(fmax, fpb) <= floor_div(gfq_min, fpb) && gfq_max - fmin < W) return TILE_FULL;
  return TILE_MASKED;
}

// the rerun threshold of the fixed-reference softmax: 64 log2 units, or
// MLA_SOFTMAX_RERUN_SLACK=<x> (>= 0; testing: 0 reruns every row whose maximum
// is not in its first visible tile)
float softmax_rerun_slack();

// launch plan (key-split fields of MfmaArgs) for row blocks of `rows_per_wg`
// and MF_BN-key tiles; returns the number of work-groups (the grid must be
// exactly that: wg_piece derives each work-group's piece from it)
// max_piece > 0: at most that many key tiles per piece (more splits)
int attn_plan(const Dims& d, const Geo& g, int batch, int n_rows, int rows_per_wg, MfmaArgs* ma, int max_piece = 0);
// workspace bytes of a plan
size_t attn_plan_workspace(const MfmaArgs& ma);
// point the plan's partial buffers into the workspace
void attn_plan_bind(MfmaArgs* ma, void* ws);
// deterministic log-sum-exp merge of the splits' partial outputs
hipError_t launch_attn_merge(const MfmaArgs& ma, hipStream_t st);

}  // namespace mla
