// Latent attention on bf16 MFMA (gfx950): the dense cache path.
//
// "Multi-Head Latent Attention" concept page, Low-rank joint compression: with
// W^UK absorbed into the query, every head attends directly in latent space,
// so all H heads of all query tokens score the same shared cache rows; and The
// RoPE problem, and the decoupled fix: the score is one dot product with the
// concatenated row [c_kv | k_rope].  The value of a key is its content latent.
// Because every (token, head) row shares the keys, the whole chunk is one dense
// contraction: rows x keys x (d_c + d_r) for the scores, rows x d_c x keys for
// the output.
//
// Work-group: 4 waves, 128 rows (32 per wave), 32-key tiles.
//  * Scores are formed transposed, S^T = K . Q^T, with v_mfma_f32_32x32x16_bf16
//    (A = 32 keys x 16 dims from LDS, B = 16 dims x 32 rows from registers).
//    Each lane then owns one query row: the row max and sum are in-lane
//    reductions plus one exchange between the two 32-lane halves.
//  * The queries of a wave stay in registers for the whole key loop, except
//    the last 8 of the 16-dim steps, which sit in LDS (8 KB per wave).
//  * O^T (d_c x 32 rows) accumulates in 16 blocks of 32 x 32.  The
//    probabilities feed the MFMA B operand straight from the score
//    accumulators: their key order is a fixed permutation, and the value
//    fragments (A operand) are read in the same permuted order with
//    ds_read_b64_tr_b16 from the very LDS tile that served as the keys.
//  * Key tiles stream into LDS with global_load_lds_dwordx4 (no register
//    staging) into three buffers: the tile being scored, the previous tile
//    (its output product runs during this tile's score chain) and the next
//    tile, whose copy is issued between this tile's score MFMAs; one barrier
//    per tile.  Every tile of the work-group's key range is classified once
//    up front (skipped / fully visible / masked / masked with never-written
//    keys).  Tile layout: [64-dim group][key][8 x 16 B], chunk c of key k
//    stored at c ^ key_swizzle(k) (attention_common.hpp), so that the 16-byte
//    key reads and the transposed value reads hit distinct banks.
//  * Softmax in the log2 domain against a fixed reference per row: the
//    maximum of the row's first visible tile.  Probabilities are
//    exp2(score - reference), so later scores above the reference only grow
//    them (bf16/fp32 hold 2^64 with full relative precision) and the O
//    accumulators are never rescaled - no VALU instruction ever reads them,
//    so they live in the MFMA accumulation registers for the whole loop.  If
//    a row's maximum exceeds its reference by more than 64 (log2 units), the
//    work-group discards its accumulators and runs the key loop once more
//    with the final maxima as references, which cannot overflow.
//  * Never-written slots are zeroed in LDS (their bytes are whatever the
//    allocation held, and 0 * NaN would poison the output).
//  * Optional split of the key range over work-groups with a deterministic
//    log-sum-exp merge (decode and load balance); the block order is
//    XCD-aware so that the work-groups sharing a key range share an L2.
#include <algorithm>
#include <cstdio>
#include <mutex>
#include <vector>

#include "attention_common.hpp"

namespace mla {

constexpr int MF_NBUF = 3;               // LDS tile buffers: scored, previous (output product), next (copy)
constexpr int MF_QLDS_STEPS = 8;         // query 16-dim steps kept in LDS (per wave 8 KB)
constexpr int PREAD_AHEAD = 3;           // score steps between the probability reads and the chain's end

// LDS bytes of one packed INT4 tile (staging): codes [key][DQK / 2 B], then
// the content scales [key][DC / 32] fp16, then the rotary scales [key] fp16
template <int DC, int DR, int CB>
constexpr int q4_stage_bytes() { return MF_BN * (DC * CB / 8 + DR / 2) + MF_BN * (DC / 32) * 2 + MF_BN * 2; }

template <int DC, int DR, bool Q4, int CB = 4, bool QKN = false>
constexpr size_t attn_mfma_lds_bytes() {
  return (size_t)(Q4 ? 2 : MF_NBUF) * ((DC + DR) / 64) * MF_BN * 128 +
         (Q4 ? 2 * (size_t)q4_stage_bytes<DC, DR, CB>() : 0) + (size_t)MF_WAVES * MF_QLDS_STEPS * 1024 +
         2 * MF_WAVES * 2 * 1024 + MF_ROWS * sizeof(float) + (QKN ? 3 * MF_BN * sizeof(float) : 0) + MF_MAX_TPS;
}

template <int DC, int DR, bool Q4, int CB = 4, bool QKN = false>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_mfma_kernel(MfmaArgs ma) {
  constexpr int DQK = DC + DR;
  constexpr int NTB = Q4 ? 2 : MF_NBUF;      // bf16 tile buffers
  constexpr int NKS = DQK / 16;              // 16-dim MFMA steps of the score product
  constexpr int NCG = DQK / 64;              // 64-dim groups per row (128 B)
  constexpr int TILE_BYTES = NCG * MF_BN * 128;
  constexpr int LOADS = TILE_BYTES / (256 * 16);
  constexpr int NKS_LDS = MF_QLDS_STEPS;      // score steps whose query fragments sit in LDS
  constexpr int NKS_REG = NKS - NKS_LDS;     // the others stay in VGPRs
  constexpr int WDIMS = DC / MF_WAVES;       // output dims owned by one wave
  constexpr int NDB = WDIMS / 32;            // its 32-dim output blocks
  static_assert(DQK % 64 == 0 && WDIMS % 32 == 0, "widths");
  static_assert(TILE_BYTES % (256 * 16) == 0, "tile");

  constexpr int STG_BYTES = Q4 ? q4_stage_bytes<DC, DR, CB>() : 0;
  static_assert(STG_BYTES % 16 == 0, "staging");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* stg = smem + NTB * TILE_BYTES;                   // INT4: [2] packed tiles
  uint8_t* qlds = stg + 2 * STG_BYTES;                      // [wave][NKS_LDS][64][16 B]
  uint8_t* plds = qlds + MF_WAVES * NKS_LDS * 1024;         // [2][wave][2 steps][64][16 B]
  float* lrow = (float*)(plds + 2 * MF_WAVES * 2 * 1024);   // [128] row sums
  float* ksl = lrow + MF_ROWS;                              // QK norm: [3][MF_BN] key inverse RMS per tile
  uint8_t* cls = (uint8_t*)(ksl + (QKN ? 3 * MF_BN : 0));
  const AttnArgs& a = ma.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int g = lane >> 5;                   // half of the wave
  const int P = a.g.P, W = a.g.window, cap = a.g.capacity, fpb = a.g.fpb;

  const Piece pc = wg_piece(ma);
  const int b = pc.rbg / ma.n_rb;
  const int rb = pc.rbg % ma.n_rb;

  const int newest = a.newest[b];
  int nm = newest % W;
  if (nm < 0) nm += W;
  const int qf0 = a.q_first[b];
  const int n_rows = a.n_rows, H = a.d.H;

  // rows scored by this lane / work-group
  const int row = rb * MF_ROWS + wave * 32 + (lane & 31);
  const bool row_ok = row < n_rows;
  const int fq = qf0 + (min(row, n_rows - 1) / H) / P;
  const int gfq_min = qf0 + ((rb * MF_ROWS) / H) / P;
  const int gfq_max = qf0 + (min(rb * MF_ROWS + MF_ROWS - 1, n_rows - 1) / H) / P;

  const int t_begin = pc.t0;
  const int ntl = pc.t1 - pc.t0;   // tiles of this piece

  // ---- classify every tile of the split once ----
  bool not_full = false;
  for (int i = tid; i < ntl; i += 256) {
    const uint8_t c = classify_tile((t_begin + i) * MF_BN, cap, P, newest, nm, W, fpb, gfq_min, gfq_max);
    cls[i] = c;
    not_full |= c != TILE_FULL;
  }
  // the first tile with a visible key (every thread finds the same one)
  int first = 0;
  while (first < ntl &&
         classify_tile((t_begin + first) * MF_BN, cap, P, newest, nm, W, fpb, gfq_min, gfq_max) == TILE_SKIP)
    ++first;


  // O^T blocks: [output-dim block of this wave][row block of the work-group]
  f32x16_t o[NDB * MF_WAVES];
  float m_run = -INFINITY, l_run = 0.f;    // reference maximum and row sum (lane partial)
  float m_seen = -INFINITY;                // true running maximum of the row
  const float c_l2 = a.d.scale * 1.4426950408889634f;
  const bf16_t* cache_b = (const bf16_t*)a.cache + (size_t)b * cap * DQK;
  const int gg = lane >> 4, li = lane & 15;

  auto next_tile = [&](int i) -> int {
    while (i < ntl && cls[i] == TILE_SKIP) ++i;
    return i;
  };
  // lane part of the DMA source offset: load q of wave w fills 1 KB block
  // (q * 4 + w) = 64-dim group q, keys 8w .. 8w+7, 8 swizzled chunks per key
  const int dma_key = (wave << 3) + (lane >> 3);
  const uint32_t dma_off = (uint32_t)(dma_key * DQK * 2 + (((lane & 7) ^ key_swizzle(dma_key)) << 4));
  // Copy of key tile i into LDS buffer `buf`, described as a scalar source
  // base, a per-lane byte offset and the LDS base; piece q (0..LOADS-1) moves
  // one 64-dim group.  Past-the-end keys of the last tile read the last slot
  // (zeroed later).  The pieces are issued between the score MFMAs of the
  // current tile: each LDS-DMA instruction takes the wave a while to issue,
  // and there it overlaps the matrix work.
  struct DmaPlan { const uint8_t* tb; uint32_t voff, lds0; int tile, kslot; };
  auto dma_plan = [&](int i, int buf) -> DmaPlan {
    const int k0 = (t_begin + i) * MF_BN;
    DmaPlan d;
    d.tile = i;
    d.kslot = buf;
    d.tb = (const uint8_t*)(cache_b + (size_t)k0 * DQK);
    d.lds0 = (uint32_t)(uintptr_t)(LDS_AS uint8_t*)(smem + buf * TILE_BYTES) + wave * 1024;
    d.voff = dma_off;
    if (k0 + MF_BN > cap) {
      const int key = min(dma_key, cap - 1 - k0);
      d.voff = (uint32_t)(key * DQK * 2 + (((lane & 7) ^ key_swizzle(dma_key)) << 4));
    }
    return d;
  };
  auto dma_piece = [&](const DmaPlan& d, int q) { dma16_sv(d.tb + q * 128, d.voff, d.lds0 + q * 4096); };
  // QK normalisation: the tile's 32 key inverse RMS values into LDS slot
  // `slot` (one dword per lane of the first half-wave; past-the-end keys read
  // the last slot)
  const float* ksc_row = QKN ? a.kscale + (size_t)b * cap : nullptr;
  auto ksl_dma = [&](int i, int slot) {
    if constexpr (QKN) {
      if (wave == 0 && lane < MF_BN) {
        const float* src = ksc_row + min((t_begin + i) * MF_BN + lane, cap - 1);
        const uint32_t dst = (uint32_t)(uintptr_t)(LDS_AS float*)(ksl + slot * MF_BN);
        dma4(src, dst);
      }
    }
  };
  auto issue_loads = [&](int i, int buf) {
    const DmaPlan d = dma_plan(i, buf);
#pragma unroll
    for (int q = 0; q < LOADS; ++q) dma_piece(d, q);
    ksl_dma(i, buf);
  };
  // the first tile's copy is in flight while the queries load
  if (!Q4 && first < ntl) issue_loads(first, 0);

  // ---- queries of this lane's row: B fragments of the score steps ----
  const bf16_t* qrow = (const bf16_t*)a.q_abs + ((size_t)b * n_rows + (row_ok ? row : 0)) * DQK;
  bf16x8_t qf[NKS_REG];
  LDS_AS uint8_t* qw = (LDS_AS uint8_t*)(qlds + wave * NKS_LDS * 1024);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    bf16x8_t v = *(const bf16x8_t*)(qrow + ks * 16 + g * 8);
    if (!row_ok) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (__bf16)0.0f;
    }
    if (ks < NKS_REG) qf[ks] = v;
    else *(LDS_AS bf16x8_t*)(qw + ((ks - NKS_REG) * 64 + lane) * 16) = v;
  }
  // every work-group tile is fully visible: no per-tile class lookups
  const bool all_full = !__syncthreads_or(not_full);
  // per-lane parts of the transposed value-read addresses.  For value dim
  // block d (0..3) and key step j (0..1) the read of keys key0 (key1 = key0 + 8)
  // lands at: group (2 * wave + d / 2), key j * 16 + kq, 16-byte chunk
  // ((d & 1) * 4 + cpart) ^ swizzle(key), byte half; the swizzle of key0 and
  // key1 does not depend on j.
  const int kq = 4 * g + (li >> 2);
  const int cpart = 2 * (gg & 1) + ((li >> 1) & 1);
  const int vhalf = (li & 1) * 8;
  const int vsw0 = key_swizzle(kq), vsw1 = key_swizzle(kq + 8);
  // O^T[wave's dims][all rows] += V^T . P^T for the tile in `vbuf` whose
  // probabilities sit in P buffer `pb`: fragments are read first (pv_read),
  // the MFMAs issued later (pv_mfma), so that the softmax of the current tile
  // can run between them
  struct PVFrag {
    bf16x8_t pfr[2][MF_WAVES];
    i16x4_t v0[2][NDB], v1[2][NDB];
  };
  // value fragments of key step j, output-dim block d
  auto pv_read_v1 = [&](int vbuf, PVFrag& f, int j, int d) {
    const LDS_AS uint8_t* vt = (const LDS_AS uint8_t*)(smem + vbuf * TILE_BYTES) + (2 * wave) * MF_BN * 128;
    const LDS_AS uint8_t* gbase = vt + (d >> 1) * MF_BN * 128 + (j * 16 + kq) * 128 + vhalf;
    f.v0[j][d] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (LDS_AS i16x4_t*)(gbase + ((((d & 1) * 4 + cpart) ^ vsw0) << 4)));
    f.v1[j][d] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (LDS_AS i16x4_t*)(gbase + 8 * 128 + ((((d & 1) * 4 + cpart) ^ vsw1) << 4)));
  };
  auto pv_read_v = [&](int vbuf, PVFrag& f) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int d = 0; d < NDB; ++d) pv_read_v1(vbuf, f, j, d);
  };
  auto pv_read_p = [&](int pb, PVFrag& f) {
    const LDS_AS uint8_t* pbase = (const LDS_AS uint8_t*)(plds + pb * MF_WAVES * 2 * 1024) + lane * 16;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < MF_WAVES; ++r)
        f.pfr[j][r] = *(const LDS_AS bf16x8_t*)(pbase + (r * 2 + j) * 1024);
  };
  auto pv_read = [&](int vbuf, int pb, PVFrag& f) {
    pv_read_v(vbuf, f);
    pv_read_p(pb, f);
  };
  auto pv_mfma = [&](const PVFrag& f) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        const bf16x4_t h0 = __builtin_bit_cast(bf16x4_t, f.v0[j][d]), h1 = __builtin_bit_cast(bf16x4_t, f.v1[j][d]);
        bf16x8_t vf;
        vf[0] = h0[0]; vf[1] = h0[1]; vf[2] = h0[2]; vf[3] = h0[3];
        vf[4] = h1[0]; vf[5] = h1[1]; vf[6] = h1[2]; vf[7] = h1[3];
#pragma unroll
        for (int r = 0; r < MF_WAVES; ++r)
          o[d * MF_WAVES + r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, f.pfr[j][r], o[d * MF_WAVES + r], 0, 0, 0);
      }
  };
  auto output_product = [&](int vbuf, int pb) {
    PVFrag f;
    pv_read(vbuf, pb, f);
    pv_mfma(f);
  };

  // ---- packed INT4 tiles: the packed bytes and scales of a tile are copied
  // into a staging buffer (global_load_lds), then dequantised into the bf16
  // tile layout.  Requires capacity % 8 == 0 (16-byte aligned scale rows).
  constexpr int CODE_ROW = DC * CB / 8 + DR / 2;        // code bytes per key (content, rotary)
  constexpr int Q4_CODE_CH = MF_BN * CODE_ROW / 16;     // 16-byte chunks of codes
  constexpr int Q4_CS_CH = MF_BN * DC / 256;            // of content scales
  constexpr int Q4_RS_CH = MF_BN * 2 / 16;              // of rotary scales
  constexpr int Q4_CH = Q4_CODE_CH + Q4_CS_CH + Q4_RS_CH;
  constexpr int Q4_CODE_BYTES = MF_BN * CODE_ROW, Q4_CS_BYTES = MF_BN * DC / 16;
  static_assert(CB == 4 || CB == 2, "content code bits");
  const uint8_t* q4_codes = (const uint8_t*)a.cache + (size_t)b * cap * CODE_ROW;
  const uint8_t* q4_cs = (const uint8_t*)a.aux + (size_t)b * cap * (DC / 16);
  const uint8_t* q4_rs = (const uint8_t*)a.aux + (size_t)a.batch * cap * (DC / 16) + (size_t)b * cap * 2;
  static_assert(Q4_CODE_CH % 64 == 0 && Q4_CS_CH == 64 && Q4_RS_CH == 4, "staging chunk counts");
  constexpr int CODE_BLK = Q4_CODE_CH / 64;             // 1 KB blocks of codes
  auto stage_dma = [&](int t, int sidx) {
    const int k0 = (t_begin + t) * MF_BN;
    const uint32_t lds_stage = (uint32_t)(uintptr_t)(LDS_AS uint8_t*)(stg + sidx * STG_BYTES);
    if (k0 + MF_BN <= cap) {
      // whole tile: each plane is one contiguous run; chunk j lands at 16 j;
      // 1 KB block n goes to wave n % 4 (codes, then the content scales, then
      // the rotary scales)
      const uint8_t* cb = q4_codes + (size_t)k0 * CODE_ROW;
#pragma unroll
      for (int i = 0; i < (CODE_BLK + 2 + 3) / 4; ++i) {
        const int blk = wave + 4 * i;   // wave-uniform
        if (blk < CODE_BLK)
          dma16_sv(cb, (uint32_t)(blk * 64 + lane) * 16, lds_stage + blk * 1024);
        else if (blk == CODE_BLK)
          dma16_sv(q4_cs + (size_t)k0 * (DC / 16), (uint32_t)lane * 16, lds_stage + CODE_BLK * 1024);
        else if (blk == CODE_BLK + 1 && lane < Q4_RS_CH)
          dma16_sv(q4_rs + (size_t)k0 * 2, (uint32_t)lane * 16, lds_stage + (CODE_BLK + 1) * 1024);
      }
      return;
    }
#pragma unroll
    for (int r = 0; r < (Q4_CH + 255) / 256; ++r) {
      if (r * 256 + wave * 64 >= Q4_CH) break;   // wave-uniform
      const int j = r * 256 + wave * 64 + lane;
      const uint8_t* src;
      if (j < Q4_CODE_CH) {
        const int key = j / (CODE_ROW / 16), off = j % (CODE_ROW / 16);
        src = q4_codes + (size_t)min(k0 + key, cap - 1) * CODE_ROW + off * 16;
      } else if (j < Q4_CODE_CH + Q4_CS_CH) {
        const int jj = j - Q4_CODE_CH, key = jj / (DC / 256);
        src = q4_cs + (size_t)min(k0 + key, cap - 1) * (DC / 16) + (jj % (DC / 256)) * 16;
      } else {
        // 8 keys per chunk; past-the-end chunks re-read the last 8 keys
        const int jj = min(j - Q4_CODE_CH - Q4_CS_CH, Q4_RS_CH - 1);
        src = q4_rs + (size_t)min(k0 + 8 * jj, cap - 8) * 2;
      }
      if (j < Q4_CH) dma16(src, lds_stage + (r * 256 + wave * 64) * 16);
    }
  };
  // dequantisation of a staged tile into the bf16 tile layout: thread tid
  // converts key tid / 8, 16-byte output chunks c = tid % 8 + 8 i (i = 0 .. 8,
  // i.e. 64-dim group i), so every LDS address is a per-thread base plus a
  // constant offset; the rotary group (last) uses the per-token scale
  static_assert(MF_BN * 8 == 256 && DQK == 8 * 72 && DC == 512, "one key per 8 threads, 9 groups");
  const int dq_key = tid >> 3, dq_cb = tid & 7;
  // split of a tile's dequantisation: DQ_QK groups during the score chain
  // (one every DQ_GAP steps), the others one every DQ_PV_GAP output MFMAs
  constexpr int DQ_QK = 5, DQ_GAP = 5, DQ_PV_GAP = 6, DQ_LEAD = 2;
  static_assert(DQ_LEAD <= 3 && DQ_LEAD < DQ_GAP, "reads of a group's packed word run ahead of its conversion");
  struct DqPlan { const LDS_AS uint8_t *sp, *cp, *rp, *scp; LDS_AS uint8_t* tp; float keep; };
  auto dequant_plan = [&](int t, int sidx, int tbuf) -> DqPlan {
    DqPlan d;
    d.sp = (const LDS_AS uint8_t*)(stg + sidx * STG_BYTES);
    d.cp = d.sp + dq_key * CODE_ROW + dq_cb * CB;                        // + 8 CB i (content)
    d.rp = d.sp + dq_key * CODE_ROW + DC * CB / 8 + dq_cb * 4;            // rotary codes
    d.scp = d.sp + Q4_CODE_BYTES + dq_key * (DC / 16) + (dq_cb >> 2) * 2;  // + 4 i
    d.tp = (LDS_AS uint8_t*)(smem + tbuf * TILE_BYTES) + dq_key * 128 +
           ((dq_cb ^ key_swizzle(dq_key)) << 4);                             // + 4096 i
    d.keep = 1.f;
    if (cls[t] == TILE_MASKED_ZERO) {
      // never-written slots hold arbitrary bytes: a zero scale gives zeros
      const int sl = (t_begin + t) * MF_BN + dq_key;
      d.keep = sl < cap && ring_frame(sl / P, newest, nm, W) >= 0 ? 1.f : 0.f;
    }
    return d;
  };
  // 64-dim group i of this thread's key: the packed word and the scale are
  // read from the staging buffer (dq_load) apart from the conversion
  // (dq_store), so the reads can be issued a few MFMAs before their use
  struct DqRaw { uint32_t codes, sbits; };
  auto dq_load = [&](const DqPlan& d, int i) -> DqRaw {
    const bool content = i < DC / 64;
    DqRaw r;
    r.codes = !content ? *(const LDS_AS uint32_t*)d.rp
              : CB == 4 ? *(const LDS_AS uint32_t*)(d.cp + 8 * CB * i)
                        : (uint32_t)*(const LDS_AS uint16_t*)(d.cp + 8 * CB * i);
    r.sbits = content ? *(const LDS_AS uint16_t*)(d.scp + 4 * i)
                      : *(const LDS_AS uint16_t*)(d.sp + Q4_CODE_BYTES + Q4_CS_BYTES + dq_key * 2);
    return r;
  };
  // every value is bf16(q * s), rounded once (dequant8_bf16)
  auto dq_store = [&](const DqPlan& d, int i, DqRaw r) {
    const bool content = i < DC / 64;
    // the conversion starts here, not next to the reads (no early wait for them)
    asm volatile("" : "+v"(r.codes), "+v"(r.sbits));
    // a zero scale for never-written slots (their bytes are arbitrary)
    const float s16 = __half2float(__ushort_as_half((unsigned short)r.sbits));
    const float sc = d.keep != 0.f ? s16 : 0.f;
    *(LDS_AS u32x4_t*)(d.tp + i * MF_BN * 128) = dequant8_bf16(r.codes, sc, content && CB == 2);
  };
  auto dequant_chunk = [&](const DqPlan& d, int i) { dq_store(d, i, dq_load(d, i)); };
  auto dequant = [&](int t, int sidx, int tbuf) {
    const DqPlan d = dequant_plan(t, sidx, tbuf);
#pragma unroll 3
    for (int i = 0; i < NCG; ++i) dequant_chunk(d, i);
  };

  // ---- scores of one tile, S^T = K . Q^T (one 32-key block, LDS reads KPF
  // steps ahead).  The previous tile's value fragments (buffer vprev) are
  // read two per step over the first steps, its probabilities (P buffer
  // pprev) PREAD_AHEAD steps before the end: both land while the chain runs
  // and neither holds up the first MFMA that needs them ----
  // INT4: with do_dq, the next tile is dequantised into buffer vprev during
  // the chain: once every wave holds its value fragments of vprev (a barrier
  // after their reads), one 64-dim group every third step.
  // QK normalisation: the content part of a key's score (the first DC / 16
  // steps of the chain) is multiplied by the key's inverse RMS (LDS slot
  // kslot) before the rotary steps accumulate onto it.  The values are read
  // QKN_LEAD steps ahead: 0 measured best (registers held across steps cost
  // spills that outweigh the exposed LDS latency)
  constexpr int NKS_C = DC / 16, QKN_LEAD = 0;
  auto qk_scores = [&](const uint8_t* tile, int kslot, const DmaPlan& dp, bool dma, PVFrag& f, int vprev, int pprev,
                       bool do_dq, const DqPlan& dqp) -> f32x16_t {
    // the score accumulator lives in VGPRs (mfma_vgpr): the 256 AGPRs hold
    // the output accumulators, and an AGPR score block would be swapped with
    // one of them every tile (copies that wait for the MFMA pipe to drain)
    f32x16_t s;
    const int key = lane & 31;
    const int sw = key_swizzle(key) ^ g;
    const LDS_AS uint8_t* krow = (const LDS_AS uint8_t*)(tile + key * 128);
    auto kaddr = [&](int ks) -> const LDS_AS bf16x8_t* {
      return (const LDS_AS bf16x8_t*)(krow + (ks >> 2) * MF_BN * 128 + ((((ks & 3) << 1) ^ sw) << 4));
    };
    auto qaddr = [&](int ks) -> const LDS_AS bf16x8_t* {
      return (const LDS_AS bf16x8_t*)(qw + ((ks - NKS_REG) * 64 + lane) * 16);
    };
    constexpr int KPF = 4;
    bf16x8_t kb[KPF], qb[KPF];
    float ksc[QKN ? 16 : 1];
    DqRaw raw[DQ_QK];
#pragma unroll
    for (int i = 0; i < KPF; ++i) kb[i] = *kaddr(i);
    // scheduling barriers keep every read KPF MFMAs ahead of its use
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8_t cur_k = kb[ks % KPF];
      const bf16x8_t cur_q = ks < NKS_REG ? qf[ks < NKS_REG ? ks : 0] : qb[ks % KPF];
      if (ks + KPF < NKS) {
        kb[ks % KPF] = *kaddr(ks + KPF);
        if (ks + KPF >= NKS_REG) qb[ks % KPF] = *qaddr(ks + KPF);
      }
      // (the chain's last step, and its last content step under QK
      // normalisation, carry their wait states: their result is read next)
      if (ks == 0) mfma_vgpr_zero(s, cur_k, cur_q);
      else if (ks == NKS - 1 || (QKN && ks == NKS_C - 1)) mfma_vgpr_last(s, cur_k, cur_q);
      else mfma_vgpr(s, cur_k, cur_q);
      if constexpr (QKN) {
        if (dma && ks == 0) ksl_dma(dp.tile, dp.kslot);   // the next tile's values, with its copy
        if (ks == NKS_C - 1 - QKN_LEAD) {
          // score element e is key 8 (e / 4) + 4 g + e % 4 of the tile
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            typedef float f32x4_v __attribute__((ext_vector_type(4)));
            const f32x4_v v = *(const LDS_AS f32x4_v*)(LDS_AS float*)(ksl + kslot * MF_BN + 8 * j + 4 * g);
            ksc[4 * j] = v[0]; ksc[4 * j + 1] = v[1]; ksc[4 * j + 2] = v[2]; ksc[4 * j + 3] = v[3];
          }
        }
        if (ks == NKS_C - 1) {
#pragma unroll
          for (int e = 0; e < 16; ++e) s[e] *= ksc[e];
          mfma_vgpr_after_valu(s);
        }
      }
      // one piece of the next tile's copy every NKS / LOADS steps, two steps
      // into each group (measured: decode 2.70 -> 2.27 us per tile step,
      // chunk 2.48 -> 2.35, against the first step of each group)
      if (ks % (NKS / LOADS) == 2 && ks / (NKS / LOADS) < LOADS && dma) dma_piece(dp, ks / (NKS / LOADS));
      if (ks >= 1 && ks <= 2 * NDB) pv_read_v1(vprev, f, (ks - 1) / NDB, (ks - 1) % NDB);
      if (!Q4 && ks == NKS - PREAD_AHEAD) pv_read_p(pprev, f);   // (INT4: registers are short)
      if constexpr (Q4) {
        static_assert(2 * NDB + DQ_GAP * DQ_QK <= NKS, "dequantisation steps");
        if (do_dq) {
          if (ks == 2 * NDB) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            lds_barrier();
          }
          // groups 0 .. DQ_QK - 1 here, one every DQ_GAP steps (its packed
          // word read DQ_LEAD steps earlier); the rest with the output MFMAs
          const int rel = ks + DQ_LEAD - 2 * NDB - 1;
          if (rel >= 0 && rel % DQ_GAP == 0 && rel / DQ_GAP < DQ_QK) raw[rel / DQ_GAP] = dq_load(dqp, rel / DQ_GAP);
          if (ks > 2 * NDB && (ks - 2 * NDB - 1) % DQ_GAP == 0 && (ks - 2 * NDB - 1) / DQ_GAP < DQ_QK)
            dq_store(dqp, (ks - 2 * NDB - 1) / DQ_GAP, raw[(ks - 2 * NDB - 1) / DQ_GAP]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return s;
  };
  // branch-free (selects only), so the score registers stay put
  auto mask_scores = [&](f32x16_t& s, int k0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int sl = k0 + 8 * (e >> 2) + 4 * g + (e & 3);
      const int slc = min(sl, cap - 1);
      const bool vis = (sl < cap) & key_visible(fq, ring_frame(slc / P, newest, nm, W), W, fpb);
      s[e] = vis ? s[e] : -INFINITY;
    }
  };
  // ---- probabilities against the row's reference maximum (log2 domain),
  // published to P buffer `pbuf` in the B-fragment layout of the output
  // product ----
  bool overflow = false;
  // row maximum of the tile (log2 units), reference update; returns -reference
  auto softmax_max = [&](const f32x16_t& s) -> float {
    float mloc = s[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mloc = fmaxf(mloc, s[e]);
    mloc = halves_max(mloc) * c_l2;
    m_seen = fmaxf(m_seen, mloc);
    if (m_run == -INFINITY) m_run = mloc;          // first visible tile of the row
    else if (mloc > m_run + ma.rerun_log2) overflow = true; // rerun with the final maxima
    return m_run == -INFINITY ? 0.f : -m_run;
  };
  auto softmax_publish = [&](const f32x16_t& s, float neg_m, int pbuf) {
    float lsum = 0.f;
    LDS_AS uint8_t* pw = (LDS_AS uint8_t*)(plds + (pbuf * MF_WAVES + wave) * 2 * 1024);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bf16x8_t pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[j * 8 + e], c_l2, neg_m));
        lsum += p;
        pf[e] = (__bf16)p;
      }
      *(LDS_AS bf16x8_t*)(pw + (j * 64 + lane) * 16) = pf;
    }
    l_run += lsum;
  };
  // one tile: scores, mask and row maximum, then the output product of the
  // previous tile issued together with this tile's exponentials (independent
  // work: the VALU runs while the MFMAs execute).  Before the first tile of a
  // pass the "previous" probabilities are zeros (any finite tile serves as
  // values).
  auto tile_step = [&](const uint8_t* tile, int k0, int kslot, int cl, int pbuf, int vprev, int pprev, const DmaPlan& dp,
                       bool dma, bool do_dq, const DqPlan& dqp) {
    PVFrag f;
    f32x16_t s = qk_scores(tile, kslot, dp, dma, f, vprev, pprev, do_dq, dqp);
    if (cl != TILE_FULL) mask_scores(s, k0);
    if constexpr (Q4) pv_read_p(pprev, f);
    const float neg_m = softmax_max(s);
    __builtin_amdgcn_sched_barrier(0);
    // output MFMAs with one exponential after every other one: the VALU work
    // runs while the matrix core is busy (scheduling barriers pin the order)
    float p[16];
    float lsum = 0.f;
    DqRaw praw{0u, 0u};
#pragma unroll
    for (int i = 0; i < 2 * NDB * MF_WAVES; ++i) {
      const int j = i / (NDB * MF_WAVES), d = (i / MF_WAVES) % NDB, r = i % MF_WAVES;
      const bf16x4_t h0 = __builtin_bit_cast(bf16x4_t, f.v0[j][d]), h1 = __builtin_bit_cast(bf16x4_t, f.v1[j][d]);
      bf16x8_t vf;
      vf[0] = h0[0]; vf[1] = h0[1]; vf[2] = h0[2]; vf[3] = h0[3];
      vf[4] = h1[0]; vf[5] = h1[1]; vf[6] = h1[2]; vf[7] = h1[3];
      o[d * MF_WAVES + r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, f.pfr[j][r], o[d * MF_WAVES + r], 0, 0, 0);
      if constexpr (Q4) {
        static_assert(DQ_PV_GAP * (NCG - DQ_QK) <= 2 * NDB * MF_WAVES, "dequantisation steps");
        if (do_dq && i % DQ_PV_GAP == 3 - DQ_LEAD && DQ_QK + i / DQ_PV_GAP < NCG)
          praw = dq_load(dqp, DQ_QK + i / DQ_PV_GAP);
        if (do_dq && i % DQ_PV_GAP == 3 && DQ_QK + i / DQ_PV_GAP < NCG) dq_store(dqp, DQ_QK + i / DQ_PV_GAP, praw);
      }
      if ((i & 1) == 0 && i / 2 < 16) {
        const int e = i / 2;
        p[e] = __builtin_amdgcn_exp2f(fmaf(s[e], c_l2, neg_m));
        lsum += p[e];
        asm volatile("" ::"v"(p[e]), "v"(lsum));   // computed here, not sunk to its use
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    LDS_AS uint8_t* pw = (LDS_AS uint8_t*)(plds + (pbuf * MF_WAVES + wave) * 2 * 1024);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bf16x8_t pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = (__bf16)p[j * 8 + e];
      *(LDS_AS bf16x8_t*)(pw + (j * 64 + lane) * 16) = pf;
    }
    l_run += lsum;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  // zero probabilities for the output product issued with a pass's first tile
  auto zero_p = [&](int pbuf) {
    for (int i = tid; i < MF_WAVES * 2 * 64; i += 256)
      *(uint4*)(plds + pbuf * MF_WAVES * 2 * 1024 + i * 16) = make_uint4(0, 0, 0, 0);
  };

  for (int pass = 0;; ++pass) {
#pragma unroll
  for (int d = 0; d < NDB * MF_WAVES; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  l_run = 0.f;
  m_run = pass == 0 ? -INFINITY : m_seen;
  overflow = false;

  if constexpr (!Q4) {
    int cur = first;
    int bcur = 0, bprev = -1, pb = 0;
    zero_p(1);
    if (pass > 0 && cur < ntl) issue_loads(cur, 0);
    while (cur < ntl) {
      const int nxt = all_full ? cur + 1 : next_tile(cur + 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      // one barrier per tile: this tile is in LDS, the previous tile's
      // probabilities are published, and the buffer two tiles back is free
      lds_barrier();
      // buffer of the next tile: the one holding neither this tile nor the previous one
      const int bnext = bprev < 0 ? (bcur + 1) % MF_NBUF : 3 - bcur - bprev;
      const DmaPlan dp = dma_plan(nxt < ntl ? nxt : cur, bnext);
      uint8_t* tile = smem + bcur * TILE_BYTES;
      const int k0 = (t_begin + cur) * MF_BN;
      const int cl = all_full ? (int)TILE_FULL : (int)cls[cur];
      if (cl == TILE_MASKED_ZERO) {
        // zero never-written (or past-the-end) keys of this tile
        for (int e = tid; e < MF_BN * NCG * 8; e += 256) {
          const int key = e / (NCG * 8), rest = e % (NCG * 8);
          const int s = k0 + key;
          const bool ok = s < cap && ring_frame(s / P, newest, nm, W) >= 0;
          if (!ok) {
            const int cg = rest >> 3, pos = rest & 7;
            *(uint4*)(tile + (cg * MF_BN + key) * 128 + pos * 16) = make_uint4(0, 0, 0, 0);
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
      }
      // the previous tile's probabilities were published before this barrier
      // (the copy is issued every step: after the last tile it copies this
      // tile again into the free buffer, which costs less than a branch per piece)
      tile_step(tile, k0, bcur, cl, pb, bprev >= 0 ? bprev : bcur, pb ^ 1, dp, true, false, DqPlan{});
      bprev = bcur;
      bcur = bnext;
      pb ^= 1;
      cur = nxt;
    }
    if (bprev >= 0) {
      lds_barrier();
      output_product(bprev, pb ^ 1);
    }
  } else {
    // tile sequence number `it` uses bf16 buffer it & 1 and staging it & 1;
    // the copy of tile it + 2 is issued at the top of step it, tile it + 1 is
    // dequantised during the score chain of step it
    int cur = next_tile(0), it = 0, pb = 0;
    zero_p(1);
    if (cur < ntl) {
      stage_dma(cur, 0);
      ksl_dma(cur, 0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
      dequant(cur, 0, 0);
    }
    int nxt = next_tile(cur + 1);
    if (nxt < ntl) {
      stage_dma(nxt, 1);
      ksl_dma(nxt, 1);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    while (cur < ntl) {
      const int bc = it & 1;
      const int nn = nxt < ntl ? next_tile(nxt + 1) : ntl;
      // this tile is dequantised, the next tile's packed bytes have landed,
      // the previous probabilities are published, staging it & 1 is free
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
      if (nn < ntl) {
        stage_dma(nn, bc);
        ksl_dma(nn, (it + 2) % 3);   // key inverse RMS slots follow the tile sequence mod 3
      }
      const bool do_dq = nxt < ntl;
      const DqPlan dqp = do_dq ? dequant_plan(nxt, bc ^ 1, bc ^ 1) : DqPlan{};
      tile_step(smem + bc * TILE_BYTES, (t_begin + cur) * MF_BN, it % 3, cls[cur], pb, it > 0 ? (bc ^ 1) : bc, pb ^ 1,
                DmaPlan{nullptr, 0u, 0u}, false, do_dq, dqp);
      ++it;
      pb ^= 1;
      cur = nxt;
      nxt = nn;
    }
    if (it > 0) {
      lds_barrier();
      output_product((it - 1) & 1, pb ^ 1);
    }
  }
  __syncthreads();
  if (!__syncthreads_or(overflow)) break;
  }

  // ---- epilogue: row sums to every wave, then O / l ----
  const float l_tot = halves_sum(l_run);
  const float lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
  if (g == 0) lrow[wave * 32 + lane] = l_tot;
  __syncthreads();
  if (row_ok && g == 0) {
    if (!pc.part_o) {
      if (a.lse) a.lse[(size_t)b * n_rows + row] = lse;
    } else {
      pc.part_lse[row - rb * MF_ROWS] = lse;
    }
  }
  // normalised bf16 rows staged in LDS ([row][DC], 16-byte chunks XOR-swizzled
  // by row & 7; the tile buffers are free now), then each wave writes 32 rows,
  // one 1 KB row per instruction (the final output or this split's partial)
  LDS_AS uint8_t* ost = (LDS_AS uint8_t*)smem;
  static_assert(DC == 512, "one 16-byte chunk per lane per row");
  static_assert((size_t)NTB * TILE_BYTES + 2 * STG_BYTES + MF_WAVES * NKS_LDS * 1024 + 2 * MF_WAVES * 2 * 1024 >=
                    (size_t)MF_ROWS * DC * 2,
                "the staged output stays below the row sums");
#pragma unroll
  for (int r = 0; r < MF_WAVES; ++r) {
    const int lr = r * 32 + (lane & 31);
    const float lt = lrow[lr];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int dim = wave * WDIMS + d * 32 + 8 * q + 4 * g;
        const f32x16_t& ob = o[d * MF_WAVES + r];
        const u32x2_t pk = pack4_bf16(ob[4 * q] * inv, ob[4 * q + 1] * inv, ob[4 * q + 2] * inv, ob[4 * q + 3] * inv);
        *(LDS_AS u32x2_t*)(ost + lr * (DC * 2) + (((dim >> 3) ^ (lr & 7)) << 4) + (dim & 7) * 2) = pk;
      }
  }
  __syncthreads();
  // eight staged rows read, then their eight stores issued
  constexpr int WROWS = 32;
  const int nvalid = min(WROWS, max(0, n_rows - (rb * MF_ROWS + wave * WROWS)));
#pragma unroll
  for (int i0 = 0; i0 < WROWS; i0 += 8) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int lr = wave * WROWS + i0 + u;
      v[u] = *(const LDS_AS u32x4_t*)(ost + lr * (DC * 2) + ((lane ^ (lr & 7)) << 4));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int lr = wave * WROWS + i0 + u;
      if (i0 + u < nvalid) {
        bf16_t* out = pc.part_o ? pc.part_o + (size_t)lr * DC
                                : (bf16_t*)a.o_lat + ((size_t)b * n_rows + rb * MF_ROWS + lr) * DC;
        *(u32x4_t*)(out + lane * 8) = v[u];
      }
    }
  }
}

// A low-bit cache attended by a chunk of queries (four or more row blocks per
// sequence) is dequantised once per call into a bf16 copy in the workspace
// ([B][capacity][d_c + d_r], the dense cache layout), which the dense kernel
// then reads: the fused path dequantises every tile once per row block that
// reads it, on the VALU, while the copy costs one pass over the packed bytes
// and the bf16 rows.  The values are those the fused path forms
// (dequant8_bf16); never-written slots hold whatever their codes give, and
// the dense kernel zeroes them in LDS as it does for a dense cache.  Thread:
// one 16-byte chunk (8 values) of one row; INT4 or INT2 content codes, INT4
// rotary codes.
template <int CB>
__global__ __launch_bounds__(256) void predequant_kernel(size_t rows, const uint8_t* __restrict__ codes,
                                                         const __half* __restrict__ cscale,
                                                         const __half* __restrict__ rscale, bf16_t* __restrict__ out) {
  constexpr int DC = 512, DR = 64, DQK = DC + DR, CH = DQK / 8;
  constexpr int CODE_ROW = DC * CB / 8 + DR / 2;
  const size_t total = rows * CH;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    const size_t r = e / CH;
    const int c = (int)(e % CH);
    const uint8_t* row = codes + r * CODE_ROW;
    uint32_t w;
    float sc;
    if (c < DC / 8) {
      w = CB == 4 ? *(const uint32_t*)(row + 4 * c) : (uint32_t)*(const uint16_t*)(row + 2 * c);
      sc = __half2float(cscale[r * (DC / 32) + c / 4]);
    } else {
      w = *(const uint32_t*)(row + DC * CB / 8 + 4 * (c - DC / 8));
      sc = __half2float(rscale[r]);
    }
    *(u32x4_t*)(out + r * DQK + c * 8) = dequant8_bf16(w, sc, CB == 2 && c < DC / 8);
  }
}

// merge of the key splits: o = sum_i w_i o_i / sum_i w_i, w_i = exp(lse_i - max)
// one wave per row, 8 consecutive dims per lane; fixed split order
// (deterministic).  The LSEs and partial rows of MG splits are loaded
// together, before any is used, so their latencies overlap.
template <int DC>
__global__ __launch_bounds__(256) void attn_merge_kernel(MfmaArgs ma) {
  static_assert(DC == 64 * 8, "8 dims per lane");
  constexpr int MG = 8;
  const AttnArgs& a = ma.a;
  const int lane = threadIdx.x & 63;
  const size_t rows = (size_t)a.batch * a.n_rows;
  const size_t r = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int ns = plan_splits(ma, (int)(r % a.n_rows) / ma.rows_wg);
  if (ns <= 1) return;   // a single split wrote the final row itself
  float mx = -INFINITY;
  float acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.f;
  float wsum = 0.f;
  for (int sp0 = 0; sp0 < ns; sp0 += MG) {
    uint4 v[MG];
    float l[MG];
#pragma unroll
    for (int u = 0; u < MG; ++u) {
      const int sp = min(sp0 + u, ns - 1);
      l[u] = ma.ws_lse[(size_t)sp * rows + r];
      v[u] = *(const uint4*)(ma.ws_o + ((size_t)sp * rows + r) * DC + lane * 8);
    }
    if (sp0 == 0) {
      // the maximum over every split (the first group's are in registers)
#pragma unroll
      for (int u = 0; u < MG; ++u) mx = fmaxf(mx, l[u]);
      for (int sp = MG; sp < ns; ++sp) mx = fmaxf(mx, ma.ws_lse[(size_t)sp * rows + r]);
      if (mx == -INFINITY) break;   // no visible key in any split
    }
#pragma unroll
    for (int u = 0; u < MG; ++u) {
      // a split with no visible key has w = 0 and a zero partial row
      const float w = sp0 + u < ns ? expf(l[u] - mx) : 0.f;
      wsum += w;
      const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(w, bf16_to_f32((bf16_t)(wd[e] & 0xffffu)), acc[2 * e]);
        acc[2 * e + 1] = fmaf(w, bf16_to_f32((bf16_t)(wd[e] >> 16)), acc[2 * e + 1]);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const u32x2_t lo = pack4_bf16(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  const u32x2_t hi = pack4_bf16(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  *(uint4*)((bf16_t*)a.o_lat + r * DC + lane * 8) = make_uint4(lo[0], lo[1], hi[0], hi[1]);
  if (a.lse && lane == 0) a.lse[r] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Shapes with an MFMA kernel: bf16, d_c = 512, d_r = 64; the packed INT4 and
// INT2 caches also need capacity % 8 == 0 (16-byte aligned scale rows).
bool attn_mfma_supported(const Dims& d, const Geo& g) {
  // MLA_ATTN_KERNEL=generic or =dsplit routes these shapes to another kernel (testing)
  static const bool other = [] {
    const char* e = getenv("MLA_ATTN_KERNEL");
    return e && (strcmp(e, "generic") == 0 || strcmp(e, "dsplit") == 0);
  }();
  if (other || d.dtype != MLA_BF16 || d.d_c != 512 || d.d_r != 64) return false;
  return d.cache_fmt == MLA_CACHE_DENSE || (lowbit_cache(d) && g.capacity % 8 == 0);
}

// cost model of a plan (seconds): the busiest CU's queue under greedy
// dispatch (each XCD's 32 CUs take its work-groups in order, large pieces
// first), at a fitted time per 32-key tile (+1 tile per piece for the query
// load and the epilogue), plus the bf16 partial outputs written and merged
static double plan_cost(int B, int n_rb, int rows_wg, int n_rows, int tiles, int d_c, int n_a, int ns_a,
                        int ns_b) {
  constexpr int XCDS = 8, CUS = 32;
  constexpr double T_TILE = 2.5e-6;
  const int tps_a = (tiles + ns_a - 1) / ns_a, tps_b = (tiles + ns_b - 1) / ns_b;
  const long long NB = (long long)B * n_a * ns_a, NS = (long long)B * (n_rb - n_a) * ns_b, N = NB + NS;
  double worst = 0.0;
  for (int x = 0; x < XCDS; x += XCDS - 1) {   // the XCDs with the most and the fewest large pieces
    const long long cnt = N / XCDS + (x < N % XCDS ? 1 : 0);
    const long long big = NB / XCDS + (x < NB % XCDS ? 1 : 0);
    const long long small = cnt - big;
    if (small < 0) return 1e30;
    double load[CUS] = {0.0};
    auto put = [&](double w) {
      int m = 0;
      for (int c = 1; c < CUS; ++c)
        if (load[c] < load[m]) m = c;
      load[m] += w;
    };
    for (long long i = 0; i < big; ++i) put(tps_a + 1.0);
    for (long long i = 0; i < small; ++i) put(tps_b + 1.0);
    for (int c = 0; c < CUS; ++c) worst = load[c] > worst ? load[c] : worst;
  }
  const double rows_a = (double)B * std::min(n_a * rows_wg, n_rows);
  const double rows_b = (double)B * n_rows - rows_a;
  double part = 0.0;
  if (ns_a > 1) part += rows_a * ns_a;
  if (ns_b > 1) part += rows_b * ns_b;
  return worst * T_TILE + part * d_c * 4.0 / 4.0e12;   // bf16 partial written and read
}

// MLA_ATTN_SPLITS=<n> fixes a uniform plan with n splits (testing: results
// must not depend on it beyond rounding)
static int forced_splits() {
  static int v = [] {
    const char* e = getenv("MLA_ATTN_SPLITS");
    return e ? atoi(e) : 0;
  }();
  return v;
}

// the plan of a shape: the best uniform split count, then two-group plans
// with 1 or 2 more splits for the last row blocks of every sequence; chosen
// once per shape (the search runs a small dispatch simulation) and cached
struct PlanKey { int B, n_rb, rows_wg, n_rows, tiles, d_c, max_piece; };
struct PlanVal { int n_a, ns_a, ns_b; };
static PlanVal search_plan(const PlanKey& k) {
  // a class table holds MF_MAX_TPS tiles; max_piece > 0 caps a piece's tiles
  const int min_ns = std::max((k.tiles + MF_MAX_TPS - 1) / MF_MAX_TPS,
                              k.max_piece > 0 ? (k.tiles + k.max_piece - 1) / k.max_piece : 1);
  auto cost = [&](int n_a, int ns_a, int ns_b) {
    return plan_cost(k.B, k.n_rb, k.rows_wg, k.n_rows, k.tiles, k.d_c, n_a, ns_a, ns_b);
  };
  PlanVal best{k.n_rb, min_ns, min_ns};
  double best_cost = cost(k.n_rb, min_ns, min_ns);
  for (int ns = min_ns + 1; ns <= 64 && ns <= k.tiles; ++ns) {
    const double c = cost(k.n_rb, ns, ns);
    if (c < best_cost * 0.98) {
      best_cost = c;
      best = PlanVal{k.n_rb, ns, ns};
    }
  }
  // the cheapest two-group plan, taken if it beats the uniform one by 2 %
  const int ns0 = best.ns_a;
  PlanVal mixed = best;
  double mixed_cost = 1e30;
  for (int extra = 1; extra <= 2; ++extra) {
    const int ns_b = ns0 + extra;
    if (ns_b > k.tiles) break;
    for (int n_a = 0; n_a < k.n_rb; ++n_a) {
      const double c = cost(n_a, ns0, ns_b);
      if (c < mixed_cost) {
        mixed_cost = c;
        mixed = PlanVal{n_a, ns0, ns_b};
      }
    }
  }
  return mixed_cost < best_cost * 0.98 ? mixed : best;
}

// (a fixed table: choosing a plan allocates nothing, so the call can run
// where the caller forbids allocation)
static PlanVal cached_plan(const PlanKey& k) {
  constexpr int CAP = 256;
  static std::mutex mu;
  static PlanKey keys[CAP];
  static PlanVal vals[CAP];
  static int n = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n; ++i)
    if (memcmp(&keys[i], &k, sizeof(PlanKey)) == 0) return vals[i];
  const PlanVal v = search_plan(k);
  if (n < CAP) {
    keys[n] = k;
    vals[n] = v;
    ++n;
  }
  return v;
}

float softmax_rerun_slack() {
  static const float v = [] {
    const char* e = getenv("MLA_SOFTMAX_RERUN_SLACK");
    const float x = e ? (float)atof(e) : 64.f;
    return x >= 0.f && x <= 64.f ? x : 64.f;
  }();
  return v;
}

int attn_plan(const Dims& d, const Geo& g, int batch, int n_rows, int rows_per_wg, MfmaArgs* ma, int max_piece) {
  ma->rerun_log2 = softmax_rerun_slack();
  ma->n_rb = (n_rows + rows_per_wg - 1) / rows_per_wg;
  ma->rows_wg = rows_per_wg;
  ma->tiles = (g.capacity + MF_BN - 1) / MF_BN;
  PlanVal v;
  static const char* forced_plan = getenv("MLA_ATTN_PLAN");   // "n_a:ns_a:ns_b" (testing)
  int fa = 0, fsa = 0, fsb = 0;
  if (forced_plan && sscanf(forced_plan, "%d:%d:%d", &fa, &fsa, &fsb) == 3 && fsa > 0 && fsb > 0) {
    const int min_ns = (ma->tiles + MF_MAX_TPS - 1) / MF_MAX_TPS;
    v = PlanVal{std::max(0, std::min(fa, ma->n_rb)), std::max(min_ns, std::min(fsa, ma->tiles)),
                std::max(min_ns, std::min(fsb, ma->tiles))};
  } else if (forced_splits() > 0) {
    const int min_ns = (ma->tiles + MF_MAX_TPS - 1) / MF_MAX_TPS;
    const int ns = std::max(min_ns, std::min(forced_splits(), ma->tiles));
    v = PlanVal{ma->n_rb, ns, ns};
  } else {
    PlanKey k;
    memset(&k, 0, sizeof(k));
    k.B = batch; k.n_rb = ma->n_rb; k.rows_wg = rows_per_wg; k.n_rows = n_rows; k.tiles = ma->tiles; k.d_c = d.d_c;
    k.max_piece = max_piece;
    v = cached_plan(k);
  }
  ma->n_a = v.n_a;
  ma->tps_a = (ma->tiles + v.ns_a - 1) / v.ns_a;
  ma->ns_a = (ma->tiles + ma->tps_a - 1) / ma->tps_a;   // splits that hold tiles
  ma->tps_b = (ma->tiles + v.ns_b - 1) / v.ns_b;
  ma->ns_b = (ma->tiles + ma->tps_b - 1) / ma->tps_b;
  if (ma->n_a == ma->n_rb) ma->ns_b = ma->ns_a, ma->tps_b = ma->tps_a;   // uniform
  ma->nsplit = std::max(ma->ns_a, ma->ns_b);
  return batch * (ma->n_a * ma->ns_a + (ma->n_rb - ma->n_a) * ma->ns_b);
}

size_t attn_plan_workspace(const MfmaArgs& ma) {
  const int d_c = ma.a.d.d_c;
  if (ma.nsplit > 1) return (size_t)ma.nsplit * ma.a.batch * ma.a.n_rows * (d_c * sizeof(bf16_t) + sizeof(float));
  return 0;
}

void attn_plan_bind(MfmaArgs* ma, void* ws) {
  ma->ws_o = nullptr;
  ma->ws_lse = nullptr;
  const int d_c = ma->a.d.d_c;
  if (ma->nsplit > 1) {
    ma->ws_o = (bf16_t*)ws;
    ma->ws_lse = (float*)(ma->ws_o + (size_t)ma->nsplit * ma->a.batch * ma->a.n_rows * d_c);
  }
}

// the low-bit cache dequantised once per call (see predequant_kernel): when
// each cache row is read by four or more row blocks (with fewer, e.g. a few
// decode tokens over a long cache, writing and re-reading the bf16 copy can
// cost more than dequantising each tile a few times); MLA_LOWBIT_PREDEQUANT=0
// or =1 forces either path (testing)
static bool use_predequant(const Dims& d, int n_rows) {
  static const int forced = [] {
    const char* e = getenv("MLA_LOWBIT_PREDEQUANT");
    return e && (e[0] == '0' || e[0] == '1') ? e[0] - '0' : -1;
  }();
  if (!lowbit_cache(d)) return false;
  if (forced >= 0) return forced == 1;
  return (n_rows + MF_ROWS - 1) / MF_ROWS >= 4;
}

// workspace: the plan's partials, then (dequantised path) the bf16 rows at a 256-byte boundary
static size_t predequant_offset(size_t plan_bytes) { return (plan_bytes + 255) & ~(size_t)255; }
static size_t predequant_bytes(const Dims& d, const Geo& g, int batch) {
  return (size_t)batch * g.capacity * (d.d_c + d.d_r) * sizeof(bf16_t);
}

size_t attn_mfma_workspace(const Dims& d, const Geo& g, int batch, int n_rows) {
  MfmaArgs ma;
  ma.a.d = d;
  ma.a.batch = batch;
  ma.a.n_rows = n_rows;
  attn_plan(d, g, batch, n_rows, MF_ROWS, &ma);
  const size_t plan = attn_plan_workspace(ma);
  return use_predequant(d, n_rows) ? predequant_offset(plan) + predequant_bytes(d, g, batch) : plan;
}

hipError_t launch_attn_mfma(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t st) {
  MfmaArgs ma;
  ma.a = a;
  const int blocks = attn_plan(a.d, a.g, a.batch, a.n_rows, MF_ROWS, &ma);
  const size_t plan = attn_plan_workspace(ma);
  if (use_predequant(a.d, a.n_rows)) {
    // the packed rows once into bf16, then the dense kernel over them
    const size_t off = predequant_offset(plan), rows = (size_t)a.batch * a.g.capacity;
    if (ws_bytes < off + predequant_bytes(a.d, a.g, a.batch)) return hipErrorInvalidValue;
    bf16_t* dq = (bf16_t*)((uint8_t*)ws + off);
    const __half* cs = (const __half*)a.aux;
    const __half* rs = cs + rows * (a.d.d_c / 32);
    const size_t chunks = rows * ((a.d.d_c + a.d.d_r) / 8);
    const unsigned grid = (unsigned)std::min<size_t>((chunks + 255) / 256, 65536);
    if (a.d.cache_fmt == MLA_CACHE_INT2)
      predequant_kernel<2><<<grid, 256, 0, st>>>(rows, (const uint8_t*)a.cache, cs, rs, dq);
    else
      predequant_kernel<4><<<grid, 256, 0, st>>>(rows, (const uint8_t*)a.cache, cs, rs, dq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ma.a.cache = dq;
    ma.a.d.cache_fmt = MLA_CACHE_DENSE;
  } else if (ws_bytes < plan) {
    return hipErrorInvalidValue;
  }
  attn_plan_bind(&ma, ws);
  constexpr int DC = 512, DR = 64;
  const int fmt = ma.a.d.cache_fmt;
  const bool qkn = a.kscale != nullptr;
  const size_t shm = fmt == MLA_CACHE_INT4   ? (qkn ? attn_mfma_lds_bytes<DC, DR, true, 4, true>()
                                                    : attn_mfma_lds_bytes<DC, DR, true, 4>())
                     : fmt == MLA_CACHE_INT2 ? (qkn ? attn_mfma_lds_bytes<DC, DR, true, 2, true>()
                                                    : attn_mfma_lds_bytes<DC, DR, true, 2>())
                                             : (qkn ? attn_mfma_lds_bytes<DC, DR, false, 4, true>()
                                                    : attn_mfma_lds_bytes<DC, DR, false>());
  auto kern = qkn ? (fmt == MLA_CACHE_INT4   ? attn_mfma_kernel<DC, DR, true, 4, true>
                         : fmt == MLA_CACHE_INT2 ? attn_mfma_kernel<DC, DR, true, 2, true>
                                                 : attn_mfma_kernel<DC, DR, false, 4, true>)
                       : (fmt == MLA_CACHE_INT4   ? attn_mfma_kernel<DC, DR, true, 4>
                         : fmt == MLA_CACHE_INT2 ? attn_mfma_kernel<DC, DR, true, 2>
                                                 : attn_mfma_kernel<DC, DR, false>);
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  kern<<<blocks, 256, shm, st>>>(ma);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attn_merge(ma, st);
}

hipError_t launch_attn_merge(const MfmaArgs& ma, hipStream_t st) {
  if (ma.a.d.d_c != 512) return hipErrorInvalidValue;
  if (ma.nsplit <= 1) return hipSuccess;
  const size_t rows = (size_t)ma.a.batch * ma.a.n_rows;
  attn_merge_kernel<512><<<(unsigned)((rows + 3) / 4), 256, 0, st>>>(ma);
  return hipGetLastError();
}

}  // namespace mla
