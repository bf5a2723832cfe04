// Latent attention on bf16 MFMA for wide cache rows: the score contraction
// split over the waves of a work-group.
//
// "VideoMLA: Compressing Video Diffusion Memory by 92.7% with Low-Rank Latent
// Attention" (review), Core Mechanism: the long-horizon cache row is a
// 512-wide content latent plus a 512-wide shared positional key, so the score
// of a query against a cache row is a 1024-long dot product ("Multi-Head
// Latent Attention" concept page, The RoPE problem, and the decoupled fix: one
// dot product with the concatenated row), while the output still sums only
// the 512-wide content latents.  A wave cannot keep a 1024-wide query block in
// registers next to its output accumulators, so here the row is cut in four:
//
// Work-group: 4 waves, 64 rows (2 blocks of 32), 32-key tiles, two LDS tile
// buffers.  One tile step:
//  * The tile has landed (barrier); the next tile's copy into the other
//    buffer is issued right away, one 1 KB piece per wave after each score
//    MFMA, so it has a whole step to arrive.
//  * Wave w holds the queries of both row blocks for dims [w, w + 1) * DQK / 4
//    in registers and forms partial scores S^T_w = K_w . Q_w^T for both
//    blocks with v_mfma_f32_32x32x16_bf16 (each key fragment read from LDS
//    feeds two MFMAs, two independent accumulation chains).  The four waves'
//    fp32 partials go to LDS (barrier).
//  * The softmax is shared by all four waves: wave w takes rows 16 w .. 16 w
//    + 15 of the work-group, four lanes per row and eight keys per lane.  A
//    lane adds its eight scores over the four quarters in a fixed order
//    (deterministic), masks, takes the row maximum over the row's four lanes
//    (two lane swaps) and exponentiates against the row's fixed reference
//    (the maximum of its first visible tile; no rescaling of the output
//    accumulators, and a rerun of the key loop if a row's maximum outgrows
//    its reference by 2^64, as in the narrow kernel).  The bf16
//    probabilities go back to LDS, into partial-score entries this wave has
//    already read (barrier).
//  * O^T (d_c x 64 rows): wave w owns d_c / 4 output dims of both row blocks
//    and adds this tile's product, value fragments read with
//    ds_read_b64_tr_b16 from the same LDS tile (issued during the softmax).
//  * Key splits over work-groups with the deterministic log-sum-exp merge,
//    XCD-aware block order, as in the narrow kernel.
#include "attention_common.hpp"

namespace mla {

constexpr int DS_ROWS = 64;   // rows per work-group (2 blocks of 32)

template <int DC, int DR>
constexpr size_t attn_dsplit_lds_bytes() {
  return 2 * (size_t)((DC + DR) / 64) * MF_BN * 128   // two key tiles
         + 2 * 4 * 64 * 64;                             // partial scores [block][quarter][lane][16 floats]
}

template <int DC, int DR, bool QKN = false>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_dsplit_kernel(MfmaArgs ma) {
  constexpr int DQK = DC + DR;
  constexpr int NCG = DQK / 64;             // 64-dim groups per row (128 B)
  constexpr int TILE_BYTES = NCG * MF_BN * 128;
  constexpr int LOADS = TILE_BYTES / (256 * 16);
  constexpr int NKSW = DQK / 64;            // 16-dim score steps of one wave (a quarter row)
  constexpr int WDIMS = DC / 4;             // output dims owned by one wave
  constexpr int NDB = WDIMS / 32;           // its 32-dim output blocks
  static_assert(DQK % 64 == 0 && WDIMS % 64 == 0 && TILE_BYTES % (256 * 16) == 0, "widths");
  static_assert(LOADS <= NKSW, "one copy piece per score step");
  // QK normalisation: waves 0 and 1 hold the content quarters, 2 and 3 the
  // rotary ones, so the content part of a score is the sum of the first two
  static_assert(!QKN || 2 * (DQK / 4) == DC, "content and rotary quarters");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* sx = smem + 2 * TILE_BYTES;      // partial scores, then probabilities; row sums at the end
  float* lrow = (float*)sx;                 // [64] row sums (epilogue)
  const AttnArgs& a = ma.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int P = a.g.P, W = a.g.window, cap = a.g.capacity, fpb = a.g.fpb;

  const Piece pc = wg_piece(ma);
  const int b = pc.rbg / ma.n_rb;
  const int rb = pc.rbg % ma.n_rb;

  const int newest = a.newest[b];
  int nm = newest % W;
  if (nm < 0) nm += W;
  const int qf0 = a.q_first[b];
  const int n_rows = a.n_rows, H = a.d.H;
  const int row0 = rb * DS_ROWS;
  const int gfq_min = qf0 + (row0 / H) / P;
  const int gfq_max = qf0 + (min(row0 + DS_ROWS - 1, n_rows - 1) / H) / P;

  const int t_begin = pc.t0;
  const int ntl = pc.t1 - pc.t0;
  // work-group OR through four flags in the partial-score area (free where
  // this is called); HIP's __syncthreads_or would add static LDS beyond 160 KB
  auto block_any = [&](bool v) -> bool {
    const bool wv = __builtin_amdgcn_ballot_w64(v) != 0;
    __syncthreads();
    if (lane == 0) ((int*)sx)[wave] = wv ? 1 : 0;
    __syncthreads();
    const bool r = (((int*)sx)[0] | ((int*)sx)[1] | ((int*)sx)[2] | ((int*)sx)[3]) != 0;
    __syncthreads();
    return r;
  };
  auto tile_class = [&](int i) -> int {
    return classify_tile((t_begin + i) * MF_BN, cap, P, newest, nm, W, fpb, gfq_min, gfq_max);
  };
  bool not_full = false;
  for (int i = tid; i < ntl; i += 256) not_full |= tile_class(i) != TILE_FULL;

  // softmax lane: row 16 wave + ri of the work-group (row block sb, row r32
  // of the block), keys of score elements 8 sj .. 8 sj + 7 of MFMA lane sl
  // (keys 16 sj + 4 sg + i and 16 sj + 8 + 4 sg + i, i = 0 .. 3)
  const int ri = lane & 15, sc = lane >> 4, sj = sc >> 1, sg = sc & 1;
  const int sb = wave >> 1, r32 = 16 * (wave & 1) + ri;
  const int sl = r32 + 32 * sg;
  const int srow = row0 + 32 * sb + r32;
  const int fq = qf0 + (min(srow, n_rows - 1) / H) / P;
  // partial scores in LDS: chunk k (score elements 4k .. 4k + 3) of MFMA
  // lane ml, block blk, quarter q at [blk][q][k][ml] (16 bytes each): every
  // MFMA-layout write and probability read is one contiguous 1 KB, every
  // softmax read four contiguous 256-byte runs.  (Entries of 64 bytes per
  // lane, even with their chunks rotated, made the 1 KB writes bank-conflict:
  // a third of the LDS cycles.)
  auto sx_chunk = [&](int blk, int q, int ml, int k) -> LDS_AS uint8_t* {
    return (LDS_AS uint8_t*)(sx + (((blk * 4 + q) * 4 + k) * 64 + ml) * 16);
  };


  // queries of both row blocks, this wave's quarter of the row
  bf16x8_t qf[2][NKSW];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = row0 + r * 32 + (lane & 31);
    const bool ok = row < n_rows;
    const bf16_t* qrow = (const bf16_t*)a.q_abs + ((size_t)b * n_rows + (ok ? row : 0)) * DQK + wave * (DQK / 4);
#pragma unroll
    for (int ks = 0; ks < NKSW; ++ks) {
      bf16x8_t v = *(const bf16x8_t*)(qrow + ks * 16 + g * 8);
      if (!ok) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)0.0f;
      }
      qf[r][ks] = v;
    }
  }
  // every tile fully visible: no class computation in the loop
  const bool all_full = !block_any(not_full);

  f32x16_t o[NDB * 2];                      // O^T blocks [output-dim block][row block]
  float m_run = -INFINITY, l_run = 0.f, m_seen = -INFINITY;
  const float c_l2 = a.d.scale * 1.4426950408889634f;
  const bf16_t* cache_b = (const bf16_t*)a.cache + (size_t)b * cap * DQK;
  const int gg = lane >> 4, li = lane & 15;

  auto next_tile = [&](int i) -> int {
    if (all_full) return i;
    while (i < ntl && tile_class(i) == TILE_SKIP) ++i;
    return i;
  };
  // DMA of a key tile: piece q of wave w fills 1 KB block (q * 4 + w) =
  // 64-dim group q, keys 8w .. 8w+7, 8 swizzled chunks per key; past-the-end
  // keys of the last tile read the last slot (zeroed later)
  const int dma_key = (wave << 3) + (lane >> 3);
  const uint32_t dma_off = (uint32_t)(dma_key * DQK * 2 + (((lane & 7) ^ key_swizzle(dma_key)) << 4));
  struct DmaPlan { const uint8_t* tb; uint32_t voff, lds0; };
  auto dma_plan = [&](int i, int buf) -> DmaPlan {
    const int k0 = (t_begin + i) * MF_BN;
    DmaPlan d;
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
  // value fragments of the tile in `vbuf` for this wave's output dims; the
  // probabilities' key order is the score accumulators' (a fixed
  // permutation), and the value fragments are read in the same order
  const int kq = 4 * g + (li >> 2);
  const int cpart = 2 * (gg & 1) + ((li >> 1) & 1);
  const int vhalf = (li & 1) * 8;
  const int vsw0 = key_swizzle(kq), vsw1 = key_swizzle(kq + 8);
  struct VFrag { i16x4_t v0[NDB], v1[NDB]; };
  auto read_values = [&](int vbuf, int j, VFrag& f) {
    const LDS_AS uint8_t* vt =
        (const LDS_AS uint8_t*)(smem + vbuf * TILE_BYTES) + (WDIMS / 64) * wave * MF_BN * 128;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const LDS_AS uint8_t* gbase = vt + (d >> 1) * MF_BN * 128 + (j * 16 + kq) * 128 + vhalf;
      f.v0[d] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS i16x4_t*)(gbase + ((((d & 1) * 4 + cpart) ^ vsw0) << 4)));
      f.v1[d] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS i16x4_t*)(gbase + 8 * 128 + ((((d & 1) * 4 + cpart) ^ vsw1) << 4)));
    }
  };
  // O^T[wave's dims][both row blocks] += V^T . P^T for key step j; the
  // probabilities of block r, step j sit in chunk 0 of partial-score entry
  // (r, j, lane)
  auto output_mfma = [&](const VFrag& f, int j) {
    bf16x8_t pfr[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) pfr[r] = *(const LDS_AS bf16x8_t*)sx_chunk(r, j, lane, 0);
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const bf16x4_t h0 = __builtin_bit_cast(bf16x4_t, f.v0[d]), h1 = __builtin_bit_cast(bf16x4_t, f.v1[d]);
      bf16x8_t vf;
      vf[0] = h0[0]; vf[1] = h0[1]; vf[2] = h0[2]; vf[3] = h0[3];
      vf[4] = h1[0]; vf[5] = h1[1]; vf[6] = h1[2]; vf[7] = h1[3];
#pragma unroll
      for (int r = 0; r < 2; ++r)
        o[d * 2 + r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pfr[r], o[d * 2 + r], 0, 0, 0);
    }
  };
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  // the softmax lane's eight key positions in the tile (score elements 8 sj + i)
  auto skey = [&](int i) -> int { return 16 * sj + 8 * (i >> 2) + 4 * sg + (i & 3); };

  for (int pass = 0;; ++pass) {
#pragma unroll
  for (int d = 0; d < NDB * 2; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  l_run = 0.f;
  m_run = pass == 0 ? -INFINITY : m_seen;
  bool overflow = false;

  // QK normalisation: the key inverse RMS of this lane's eight keys of tile
  // t, loaded one step before the tile is scored (into ksc_next), ahead of
  // that step's tile copy; the wait at the top of the next step (a
  // compiler-visible s_waitcnt) covers them, so neither the copy into ksc nor
  // the use waits for a tile copy in flight.  (ksc_next is not loaded before
  // the loop: a value from outside the loop would be merged with the loop's
  // by a register copy, which waits for the load.)
  float ksc[QKN ? 8 : 1], ksc_next[QKN ? 8 : 1];
  auto load_ksc = [&](int t, float* dst) {
    if constexpr (QKN) {
      const float* kr = a.kscale + (size_t)b * cap;
      const int kt = (t_begin + t) * MF_BN;
      if ((cap & 3) == 0 && kt + MF_BN <= cap) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4_t v = *(const f32x4_t*)(kr + kt + skey(4 * h));
          dst[4 * h] = v[0]; dst[4 * h + 1] = v[1]; dst[4 * h + 2] = v[2]; dst[4 * h + 3] = v[3];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[i] = kr[min(kt + skey(i), cap - 1)];
      }
    }
  };
  int cur = next_tile(0), bc = 0;
  bool first_step = true;
  if (cur < ntl) {
    const DmaPlan d0 = dma_plan(cur, 0);
#pragma unroll
    for (int q = 0; q < LOADS; ++q) dma_piece(d0, q);
  }
  while (cur < ntl) {
    const int nxt = next_tile(cur + 1);
    // vmcnt(0) lgkmcnt(0), as the builtin: the compiler counts it as done
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070);
    asm volatile("" ::: "memory");
    // barrier 1: this tile is in LDS; every wave is done with the previous
    // tile (its buffer takes the next one; the probability area is free)
    lds_barrier();
    uint8_t* tile = smem + bc * TILE_BYTES;
    const int k0 = (t_begin + cur) * MF_BN;
    const int cl = all_full ? (int)TILE_FULL : tile_class(cur);
    const bool do_dma = nxt < ntl;
    const DmaPlan dp = dma_plan(do_dma ? nxt : cur, bc ^ 1);
    if constexpr (QKN) {
      // (this tile's values arrived before the wait above; the first tile of
      // a pass loads its own here, and its use waits for this step's copy)
      if (first_step) {
        load_ksc(cur, ksc);
        // wait for them here, before this step's tile copy is issued
#pragma unroll
        for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(ksc[i]));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) ksc[i] = ksc_next[i];
      }
      load_ksc(do_dma ? nxt : cur, ksc_next);   // (unconditional: no merge copy that would wait for it)
    }
    first_step = false;
    if (cl == TILE_MASKED_ZERO) {
      // zero never-written (or past-the-end) keys of this tile
      for (int e = tid; e < MF_BN * NCG * 8; e += 256) {
        const int key = e / (NCG * 8), rest = e % (NCG * 8);
        const int sl = k0 + key;
        const bool ok = sl < cap && ring_frame(sl / P, newest, nm, W) >= 0;
        if (!ok) {
          const int cg = rest >> 3, pos = rest & 7;
          *(uint4*)(tile + (cg * MF_BN + key) * 128 + pos * 16) = make_uint4(0, 0, 0, 0);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      lds_barrier();
    }

    // ---- partial scores of both row blocks over this wave's quarter; the
    // next tile's copy issued between the MFMAs ----
    f32x16_t s0, s1;
#pragma unroll
    for (int e = 0; e < 16; ++e) s0[e] = s1[e] = 0.f;
    {
      const int key = lane & 31;
      const int sw = key_swizzle(key) ^ g;
      const LDS_AS uint8_t* krow = (const LDS_AS uint8_t*)(tile + key * 128);
      auto kaddr = [&](int ks) -> const LDS_AS bf16x8_t* {
        const int gks = wave * NKSW + ks;
        return (const LDS_AS bf16x8_t*)(krow + (gks >> 2) * MF_BN * 128 + ((((gks & 3) << 1) ^ sw) << 4));
      };
      constexpr int KPF = 4;
      bf16x8_t kb[KPF];
#pragma unroll
      for (int i = 0; i < KPF; ++i) kb[i] = *kaddr(i < NKSW ? i : 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < NKSW; ++ks) {
        const bf16x8_t cur_k = kb[ks % KPF];
        if (ks + KPF < NKSW) kb[ks % KPF] = *kaddr(ks + KPF);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur_k, qf[0][ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur_k, qf[1][ks], s1, 0, 0, 0);
        if (ks < LOADS && do_dma) dma_piece(dp, ks);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      *(LDS_AS f32x4_t*)sx_chunk(0, wave, lane, k) = f32x4_t{s0[4 * k], s0[4 * k + 1], s0[4 * k + 2], s0[4 * k + 3]};
      *(LDS_AS f32x4_t*)sx_chunk(1, wave, lane, k) = f32x4_t{s1[4 * k], s1[4 * k + 1], s1[4 * k + 2], s1[4 * k + 3]};
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // barrier 2: every quarter's partial scores are in LDS
    lds_barrier();

    // ---- softmax of this lane's row and eight keys ----
    float sv[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4_t lo = *(const LDS_AS f32x4_t*)sx_chunk(sb, q, sl, 2 * sj);
      const f32x4_t hi = *(const LDS_AS f32x4_t*)sx_chunk(sb, q, sl, 2 * sj + 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = q == 0 ? lo[i] : sv[i] + lo[i];
        sv[4 + i] = q == 0 ? hi[i] : sv[4 + i] + hi[i];
      }
      if constexpr (QKN) {
        if (q == 1)
#pragma unroll
          for (int i = 0; i < 8; ++i) sv[i] *= ksc[i];
      }
    }
    // the value fragments of this tile's first key step, read while the
    // softmax runs
    VFrag vf0;
    read_values(bc, 0, vf0);
    if (cl != TILE_FULL) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int sl2 = k0 + skey(i);
        bool vis = sl2 < cap;
        if (vis) vis = key_visible(fq, ring_frame(sl2 / P, newest, nm, W), W, fpb);
        if (!vis) sv[i] = -INFINITY;
      }
    }
    float mloc = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mloc = fmaxf(mloc, sv[i]);
    {
      // over the row's four lanes (lane ^ 16, lane ^ 32)
      const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mloc), __float_as_uint(mloc), false, false);
      mloc = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
      mloc = halves_max(mloc) * c_l2;
    }
    m_seen = fmaxf(m_seen, mloc);
    if (m_run == -INFINITY) m_run = mloc;                   // first visible tile of the row
    else if (mloc > m_run + ma.rerun_log2) overflow = true; // rerun with the final maxima
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
    bf16x8_t pf;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sv[i], c_l2, neg_m));
      l_run += p;
      pf[i] = (__bf16)p;
    }
    // (chunk 0 of entry (sb, sj, sl): this wave read it above; every lane
    // that reads this entry's chunks belongs to this wave and has read them)
    *(LDS_AS bf16x8_t*)sx_chunk(sb, sj, sl, 0) = pf;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // barrier 3: every row's probabilities of this tile are published
    lds_barrier();

    // ---- this tile's output product ----
    VFrag vf1;
    read_values(bc, 1, vf1);
    output_mfma(vf0, 0);
    output_mfma(vf1, 1);
    bc ^= 1;
    cur = nxt;
  }
  if (!block_any(overflow)) break;
  }

  // ---- epilogue: row sums to every wave, then O / l ----
  {
    // the row's sum over its four lanes
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    const float l2 = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const float l_tot = halves_sum(l2);
    const float lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
    if (sc == 0) lrow[32 * sb + r32] = l_tot;
    if (sc == 0 && srow < n_rows) {
      if (!pc.part_o) {
        if (a.lse) a.lse[(size_t)b * n_rows + srow] = lse;
      } else {
        pc.part_lse[srow - row0] = lse;
      }
    }
  }
  __syncthreads();
  // normalised bf16 rows staged in LDS ([row][DC], 16-byte chunks XOR-swizzled
  // by row & 7, in the free tile buffers), then each wave writes 16 rows, one
  // 1 KB row per instruction (the final output or this split's partial)
  static_assert(DC == 512 && 2 * TILE_BYTES >= DS_ROWS * DC * 2, "output staging");
  LDS_AS uint8_t* ost = (LDS_AS uint8_t*)smem;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int lr = r * 32 + (lane & 31);
    const float lt = lrow[lr];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int dim = wave * WDIMS + d * 32 + 8 * q + 4 * g;
        const f32x16_t& ob = o[d * 2 + r];
        const u32x2_t pk = pack4_bf16(ob[4 * q] * inv, ob[4 * q + 1] * inv, ob[4 * q + 2] * inv, ob[4 * q + 3] * inv);
        *(LDS_AS u32x2_t*)(ost + lr * (DC * 2) + (((dim >> 3) ^ (lr & 7)) << 4) + (dim & 7) * 2) = pk;
      }
  }
  __syncthreads();
  // eight staged rows read, then their eight stores issued
  constexpr int WROWS = (DS_ROWS / 4);
  const int nvalid = min(WROWS, max(0, n_rows - (row0 + wave * WROWS)));
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
                                : (bf16_t*)a.o_lat + ((size_t)b * n_rows + row0 + lr) * DC;
        *(u32x4_t*)(out + lane * 8) = v[u];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Shapes with this kernel: bf16 dense cache, d_c = 512, d_r = 512 (the
// long-horizon row); MLA_ATTN_KERNEL=dsplit also routes d_r = 64 here (testing)
static bool dsplit_forced() {
  static const bool v = [] {
    const char* e = getenv("MLA_ATTN_KERNEL");
    return e && strcmp(e, "dsplit") == 0;
  }();
  return v;
}

bool attn_dsplit_supported(const Dims& d) {
  static const bool generic = [] {
    const char* e = getenv("MLA_ATTN_KERNEL");
    return e && strcmp(e, "generic") == 0;
  }();
  // (QK normalisation: content and rotary quarters must be whole waves, d_r = 512)
  if (generic || d.dtype != MLA_BF16 || d.cache_fmt != MLA_CACHE_DENSE || d.d_c != 512) return false;
  if (d.qk_norm && d.d_r != 512) return false;
  return d.d_r == 512 || (d.d_r == 64 && dsplit_forced());
}

size_t attn_dsplit_workspace(const Dims& d, const Geo& g, int batch, int n_rows) {
  MfmaArgs ma;
  ma.a.d = d;
  ma.a.batch = batch;
  ma.a.n_rows = n_rows;
  attn_plan(d, g, batch, n_rows, DS_ROWS, &ma);
  return attn_plan_workspace(ma);
}

template <int DC, int DR, bool QKN>
static hipError_t launch_dsplit_shape(const MfmaArgs& ma, int blocks, hipStream_t st) {
  const size_t shm = attn_dsplit_lds_bytes<DC, DR>();
  auto kern = attn_dsplit_kernel<DC, DR, QKN>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  kern<<<blocks, 256, shm, st>>>(ma);
  return hipGetLastError();
}

hipError_t launch_attn_dsplit(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t st) {
  MfmaArgs ma;
  ma.a = a;
  const int blocks = attn_plan(a.d, a.g, a.batch, a.n_rows, DS_ROWS, &ma);
  if (ws_bytes < attn_plan_workspace(ma)) return hipErrorInvalidValue;
  attn_plan_bind(&ma, ws);
  hipError_t e = a.d.d_r != 512 ? launch_dsplit_shape<512, 64, false>(ma, blocks, st)
                 : a.kscale     ? launch_dsplit_shape<512, 512, true>(ma, blocks, st)
                                : launch_dsplit_shape<512, 512, false>(ma, blocks, st);
  if (e != hipSuccess) return e;
  return launch_attn_merge(ma, st);
}

}  // namespace mla
