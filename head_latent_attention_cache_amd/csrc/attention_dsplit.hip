// Latent attention on bf16 MFMA for wide cache rows: the score contraction
// split over the waves of a work-group, the softmax of one key tile hidden
// under the score products of the next.
//
// "VideoMLA: Compressing Video Diffusion Memory by 92.7% with Low-Rank Latent
// Attention" (review), Core Mechanism: the long-horizon cache row is a
// 512-wide content latent plus a 512-wide shared positional key, so the score
// of a query against a cache row is a 1024-long dot product ("Multi-Head
// Latent Attention" concept page, The RoPE problem, and the decoupled fix: one
// dot product with the concatenated row), while the output still sums only
// the 512-wide content latents.  A wave cannot keep a 1024-wide query block in
// registers next to its output accumulators, so here the row is cut in four:
// wave w takes content dims [w, w + 1) * d_c / 4 and rotary dims
// [w, w + 1) * d_r / 4 of both 32-row blocks of the work-group (64 rows).
//
// Only the content part of a key tile goes through LDS (it is read twice:
// as keys by the scores and, transposed, as values by the output product);
// each wave loads its rotary quarter of the tile's keys straight into the
// registers the score MFMAs take (no LDS bytes for it), one tile ahead.  The
// content is copied into its LDS buffer one step ahead as well, by
// global-to-LDS loads.  Three content buffers (96 KB), the partial scores
// (32 KB), the probabilities (4 KB), the L2 prefetch's landing area (1 KB)
// and the key-scale slots of three tiles (768 B) take 133.75 KB of LDS.  Step s of the
// key loop, with tiles t_s (attended now), t_s+1 (scored now) and t_s+2
// (loaded now):
//  * top: every load of the previous step has landed; barrier A (the partial
//    scores of t_s and t_s+1's content are in LDS).  Wave 0 starts the L2
//    prefetch of a slice of the tile eight steps ahead.
//  * phase 1: the partial scores of t_s+1 for both row blocks,
//    S^T_w = K_w . Q_w^T with v_mfma_f32_32x32x16_bf16 (each key fragment
//    feeds two MFMAs: two independent accumulation chains), rotary steps from
//    registers (each register set reloaded with t_s+2 right after its
//    MFMAs) alternating with content steps from LDS, and half of t_s+2's
//    content copy between them; and, spread between the same MFMAs, the softmax of
//    t_s: wave w takes rows 16 w .. 16 w + 15, four lanes per row and eight
//    keys per lane, adds the four quarters' partials in a fixed order
//    (deterministic), masks, takes the row maximum over the row's four lanes
//    (two lane swaps) and exponentiates against the row's fixed reference
//    (the maximum of its first visible tile; no rescaling of the output
//    accumulators, and a rerun of the key loop if a row's maximum outgrows
//    its reference by 2^64, as in the narrow kernel); the bf16 probabilities
//    go to LDS.  Barrier B.
//  * phase 2: O^T (d_c x 64 rows) += V^T . P^T for t_s (wave w owns d_c / 4
//    output dims of both row blocks, value fragments read with
//    ds_read_b64_tr_b16 from t_s's content buffer during phase 1), with the
//    other half of t_s+2's content copy between its MFMAs and the partial
//    scores of t_s+1 written to LDS between its two key steps.
// QK normalisation ("Multi-Head Latent Attention" topic page, QK-Norm
// abstract; the key's inverse RMS scales the content part of its score):
// the contraction is split by kind instead of by quarter, waves 0 and 1 on
// the content dims, waves 2 and 3 on the rotary dims, so that the softmax
// scales the content partials of each key and the chain keeps one
// accumulator per row block.
// What bounds it: the vector-memory side.  64 KB of cache rows per 64 rows
// and 32 keys is 2.5 times the bytes per MFMA of the narrow kernel (128
// rows per 1152-byte row); a step with every load removed runs in 60 % of
// the time.  Key splits over work-groups with the deterministic log-sum-exp
// merge, as in the narrow kernel; pieces in work-group id order.
#include "attention_common.hpp"

namespace mla {

constexpr int DS_ROWS = 64;   // rows per work-group (2 blocks of 32)

constexpr int DS_PF_AHEAD = 8;  // L2 prefetch distance (tiles)
// at most this many key tiles per work-group piece: the long video (2340
// tiles per row block) measured 69.3 ms with 6 or 8 splits against 72.1 ms
// with the 2 the plan's cost model picks (4: 70.9, 10: 70.4, 16: 71.4; one
// box); the model counts the partials' traffic but not what shorter pieces
// gain, whose concurrently running work-groups attend a narrower key range
constexpr int DS_MAX_PIECE_TILES = 400;

template <int DC, int DR>
constexpr size_t attn_dsplit_lds_bytes() {
  return 3 * (size_t)(DC / 64) * MF_BN * 128   // three content tiles
         + 2 * 4 * 64 * 64                       // partial scores [block][quarter][chunk][lane] (16 B)
         + 2 * 2 * 64 * 16                       // probabilities [block][key step][lane] (16 B)
         + 1024                                  // landing area of the L2 prefetch (never read)
         + 3 * 256;                              // key scales of QK normalisation, three tiles
}

template <int DC, int DR, bool QKN = false>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_dsplit_kernel(MfmaArgs ma) {
  constexpr int DQK = DC + DR;
  constexpr int CT_BYTES = (DC / 64) * MF_BN * 128;   // content part of a key tile
  constexpr int LOADS = CT_BYTES / (256 * 16);        // its 1 KB copy pieces per wave
  constexpr int NKC = DC / 64;              // 16-dim content score steps of one wave (d_c / 4 dims)
  constexpr int NKR = DR / 64;              // rotary score steps of one wave (d_r / 4 dims)
  constexpr int NKS = NKC + NKR;
  // QK normalisation with d_r = d_c: the score contraction split by kind
  // instead of by quarter: waves 0 and 1 take content dims [256 w, 256 w +
  // 256), waves 2 and 3 rotary dims [256 (w - 2), ...), so that a wave's
  // partial score is all content or all rotary and the softmax applies each
  // key's inverse RMS to the content partials alone (no second accumulator)
  constexpr bool RS = QKN && DR == DC;
  constexpr int NKR_W = RS ? NKS : NKR;     // rotary key fragments a wave holds
  constexpr int WDIMS = DC / 4;             // output dims owned by one wave
  constexpr int NDB = WDIMS / 32;           // its 32-dim output blocks
  static_assert(DC == 512 && DR % 64 == 0 && CT_BYTES % 4096 == 0, "widths");
  static_assert(LOADS <= NKS, "one copy piece per score step");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* sx = smem + 3 * CT_BYTES;        // partial scores; row sums at the end
  uint8_t* pbuf = sx + 2 * 4 * 64 * 64;     // probabilities
  uint8_t* pf_sink = pbuf + 2 * 2 * 64 * 16;  // L2 prefetch landing area
  uint8_t* ksl = pf_sink + 1024;             // key scales, two 256-byte slots
  float* lrow = (float*)sx;                 // [64] row sums (epilogue)
  const AttnArgs& a = ma.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int P = a.g.P, W = a.g.window, cap = a.g.capacity, fpb = a.g.fpb;

  // (pieces in work-group id order: the long key ranges of this kernel's
  // workloads exceed the L2s, and a key range shared by every XCD at once
  // stays in the last-level cache; measured 15 % faster on the long video)
  const Piece pc = wg_piece(ma, true);
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
  // this is called); HIP's __syncthreads_or would add static LDS
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
  // MFMA-layout write is one contiguous 1 KB, every softmax read four
  // contiguous 256-byte runs.  (Entries of 64 bytes per lane, even with their
  // chunks rotated, made the 1 KB writes bank-conflict: a third of the LDS
  // cycles.)
  auto sx_chunk = [&](int blk, int q, int ml, int k) -> LDS_AS uint8_t* {
    return (LDS_AS uint8_t*)(sx + (((blk * 4 + q) * 4 + k) * 64 + ml) * 16);
  };
  // probabilities of block blk, key step j (16 keys) in the MFMA B-operand
  // layout of lane ml: 16 bytes at [blk][j][ml]
  auto p_entry = [&](int blk, int j, int ml) -> LDS_AS uint8_t* {
    return (LDS_AS uint8_t*)(pbuf + ((blk * 2 + j) * 64 + ml) * 16);
  };

  // queries of both row blocks, this wave's content and rotary quarters:
  // steps 0 .. NKC - 1 content dims wave * d_c / 4 + 16 ks, then rotary dims
  // d_c + wave * d_r / 4 + 16 (ks - NKC); split by kind, step ks of content
  // wave w (0, 1) is dim 256 w + 16 ks, of rotary wave w (2, 3) dim
  // d_c + 256 (w - 2) + 16 ks
  bf16x8_t qf[2][NKS];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = row0 + r * 32 + (lane & 31);
    const bool ok = row < n_rows;
    const bf16_t* qrow = (const bf16_t*)a.q_abs + ((size_t)b * n_rows + (ok ? row : 0)) * DQK + g * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int dim = RS ? (wave < 2 ? wave * (DC / 2) + ks * 16 : DC + (wave - 2) * (DR / 2) + ks * 16)
                         : ks < NKC ? wave * (DC / 4) + ks * 16 : DC + wave * (DR / 4) + (ks - NKC) * 16;
      bf16x8_t v = *(const bf16x8_t*)(qrow + dim);
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
  auto class_of = [&](int i) -> int { return all_full ? (int)TILE_FULL : tile_class(i); };
  // Copy of a tile's content into LDS: piece q of wave w is 1 KB block
  // (q * 4 + w) of the LDS tile (64-dim group q, keys 8w .. 8w + 7, 16 bytes
  // per lane, chunk c of a key read from c ^ its swizzle), one
  // global_load_lds_dwordx4 per piece; past-the-end keys of the last tile
  // read the last slot (zeroed later).  (Staged through registers and
  // written at the top of the step instead, the copy's LDS writes sat in
  // front of the step's barrier: 4 % slower.)
  const int cp_key = (wave << 3) + (lane >> 3);
  auto content_src = [&](int t) -> const uint8_t* {
    const int k0 = (t_begin + t) * MF_BN;
    const int key = min(cp_key, cap - 1 - k0);
    return (const uint8_t*)(cache_b + ((size_t)k0 + key) * DQK) + (((lane & 7) ^ key_swizzle(cp_key)) << 4);
  };
  // piece q of the content at `cs` (content_src) into buffer buf
  auto copy_load = [&](const uint8_t* cs, int q, int buf) {
    dma16(cs + q * 128, (uint32_t)(uintptr_t)(LDS_AS uint8_t*)(smem + buf * CT_BYTES) + wave * 1024 + q * 4096);
  };
  // the score steps that load a copy piece: every other step where the chain
  // is long enough, else the first LOADS steps
  auto copy_step = [](int i) -> bool { return NKS >= 2 * LOADS ? i % 2 == 1 && i / 2 < LOADS : i < LOADS; };
  auto copy_piece = [](int i) -> int { return NKS >= 2 * LOADS ? i / 2 : i; };
  // in the key loop the first LP1 pieces go between the score MFMAs (one
  // every four steps) and the rest between the output MFMAs, so that the
  // vector-memory instructions spread over the whole step
  constexpr int LP1 = NKS >= 2 * LOADS ? LOADS / 2 : LOADS;
  auto loop_copy_step = [](int i) -> bool { return LP1 < LOADS ? i % 4 == 1 && i / 4 < LP1 : i < LOADS; };
  auto loop_copy_piece = [](int i) -> int { return LP1 < LOADS ? i / 4 : i; };
  // zero the content of never-written (or past-the-end) keys of tile t in
  // buffer buf (their rotary scores are masked; their values must be 0)
  auto zero_content = [&](int buf, int t) {
    uint8_t* tile = smem + buf * CT_BYTES;
    const int k0 = (t_begin + t) * MF_BN;
    for (int e = tid; e < MF_BN * (DC / 64) * 8; e += 256) {
      const int key = e / ((DC / 64) * 8), rest = e % ((DC / 64) * 8);
      const int sl2 = k0 + key;
      const bool ok = sl2 < cap && ring_frame(sl2 / P, newest, nm, W) >= 0;
      if (!ok) {
        const int cg = rest >> 3, pos = rest & 7;
        *(uint4*)(tile + (cg * MF_BN + key) * 128 + pos * 16) = make_uint4(0, 0, 0, 0);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    lds_barrier();
  };
  // this wave's rotary key fragments of tile t (key lane & 31, 16 dims per
  // score step), straight from the cache into registers; past-the-end keys
  // read the last slot (their scores are masked)
  bf16x8_t kr[NKR_W];
  auto rope_src = [&](int t) -> const bf16_t* {
    const int key = min((t_begin + t) * MF_BN + (lane & 31), cap - 1);
    return cache_b + (size_t)key * DQK + DC + (RS ? (wave & 1) * (DR / 2) : wave * (DR / 4)) + g * 8;
  };
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
        (const LDS_AS uint8_t*)(smem + vbuf * CT_BYTES) + (WDIMS / 64) * wave * MF_BN * 128;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const LDS_AS uint8_t* gbase = vt + (d >> 1) * MF_BN * 128 + (j * 16 + kq) * 128 + vhalf;
      f.v0[d] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS i16x4_t*)(gbase + ((((d & 1) * 4 + cpart) ^ vsw0) << 4)));
      f.v1[d] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS i16x4_t*)(gbase + 8 * 128 + ((((d & 1) * 4 + cpart) ^ vsw1) << 4)));
    }
  };
  // O^T[wave's dims][both row blocks] += V^T . P^T, one MFMA: output-dim
  // block d, row block r of one key step
  auto output_one = [&](const VFrag& f, const bf16x8_t* pfr, int d, int r) {
    const bf16x4_t h0 = __builtin_bit_cast(bf16x4_t, f.v0[d]), h1 = __builtin_bit_cast(bf16x4_t, f.v1[d]);
    bf16x8_t vf;
    vf[0] = h0[0]; vf[1] = h0[1]; vf[2] = h0[2]; vf[3] = h0[3];
    vf[4] = h1[0]; vf[5] = h1[1]; vf[6] = h1[2]; vf[7] = h1[3];
    o[d * 2 + r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pfr[r], o[d * 2 + r], 0, 0, 0);
  };
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  // the softmax lane's eight key positions in the tile (score elements 8 sj + i)
  auto skey = [&](int i) -> int { return 16 * sj + 8 * (i >> 2) + 4 * sg + (i & 3); };

  // QK normalisation: the content part of a score is scaled by its key's
  // inverse RMS.  The contraction is split by kind (RS): the content
  // partials of waves 0 and 1 are scaled in the softmax, which reads the
  // scales of its eight keys of the tile.  A tile's 32 scales reach LDS two
  // steps before that softmax, one 4-byte global-to-LDS load per lane of
  // wave 1 (lanes 32 .. 63 repeat lanes 0 .. 31), into one of three slots
  // (the tiles being softmaxed, scored and loaded).
  auto ksc_copy = [&](int t, int slot) {
    if (QKN && wave == 1) {
      const int kt = (t_begin + t) * MF_BN;
      dma4(a.kscale + (size_t)b * cap + min(kt + (lane & 31), cap - 1),
           (uint32_t)(uintptr_t)(LDS_AS uint8_t*)(ksl + slot * 256));
    }
  };
  // Partial scores of both row blocks over this wave's dims for the tile
  // whose content sits in buffer kbuf and whose rotary fragments are in kr;
  // kr is reloaded from `rnext` as it is consumed.  Quarters: rotary and
  // content steps alternate (the register loads spread over the chain);
  // split by kind: all of a wave's steps are of its kind (measured on the
  // long video: the split by kind costs the plain kernel 9 %, and saves the
  // QK-normalised one the second pair of accumulators, +11.5 % -> +5.3 %
  // over the plain kernel).
  // stage(i) runs after score step i (copy pieces, softmax work).
  f32x16_t s0, s1;
  constexpr int NALT = NKR < NKC ? NKR : NKC;   // alternating pairs
  static_assert(!QKN || RS, "QK normalisation: the split by kind (d_r = d_c)");
  auto score_chain = [&](int kbuf, const bf16_t* rnext, auto&& stage) {
    const int key = lane & 31;
    const int sw = key_swizzle(key) ^ g;
    const LDS_AS uint8_t* krow = (const LDS_AS uint8_t*)(smem + kbuf * CT_BYTES + key * 128);
    auto kaddr = [&](int ks) -> const LDS_AS bf16x8_t* {
      const int gks = (RS ? (wave & 1) * NKS : wave * NKC) + ks;
      return (const LDS_AS bf16x8_t*)(krow + (gks >> 2) * MF_BN * 128 + ((((gks & 3) << 1) ^ sw) << 4));
    };
    constexpr int KPF = 4;
    bf16x8_t kb[KPF];
    if constexpr (RS) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s0[e] = s1[e] = 0.f;
      if (wave >= 2) {
        // rotary waves: every step from the registers, each reloaded with the
        // next tile right after its MFMAs
#pragma unroll
        for (int i = 0; i < NKS; ++i) {
          const bf16x8_t k = kr[i];
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, qf[0][i], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, qf[1][i], s1, 0, 0, 0);
          kr[i] = *(const bf16x8_t*)(rnext + i * 16);
          stage(i);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        // content waves: every step from LDS, read KPF steps ahead
#pragma unroll
        for (int i = 0; i < KPF; ++i) kb[i] = *kaddr(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NKS; ++i) {
          const bf16x8_t k = kb[i % KPF];
          if (i + KPF < NKS) kb[i % KPF] = *kaddr(i + KPF);
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, qf[0][i], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, qf[1][i], s1, 0, 0, 0);
          stage(i);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < KPF; ++i) kb[i] = *kaddr(i);
#pragma unroll
    for (int e = 0; e < 16; ++e) s0[e] = s1[e] = 0.f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NKS; ++i) {
      const bool rot = i < 2 * NALT ? i % 2 == 0 : NKR > NKC;
      if (rot) {
        const int kj = i < 2 * NALT ? i / 2 : i - NALT;
        const bf16x8_t k = kr[kj];
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, qf[0][NKC + kj], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, qf[1][NKC + kj], s1, 0, 0, 0);
        kr[kj] = *(const bf16x8_t*)(rnext + kj * 16);
      } else {
        const int ks = i < 2 * NALT ? i / 2 : i - NALT;
        const bf16x8_t k = kb[ks % KPF];
        if (ks + KPF < NKC) kb[ks % KPF] = *kaddr(ks + KPF);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, qf[0][ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, qf[1][ks], s1, 0, 0, 0);
      }
      stage(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto write_partials = [&]() {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      *(LDS_AS f32x4_t*)sx_chunk(0, wave, lane, k) = f32x4_t{s0[4 * k], s0[4 * k + 1], s0[4 * k + 2], s0[4 * k + 3]};
      *(LDS_AS f32x4_t*)sx_chunk(1, wave, lane, k) = f32x4_t{s1[4 * k], s1[4 * k + 1], s1[4 * k + 2], s1[4 * k + 3]};
    }
  };

  for (int pass = 0;; ++pass) {
#pragma unroll
  for (int d = 0; d < NDB * 2; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  l_run = 0.f;
  m_run = pass == 0 ? -INFINITY : m_seen;
  bool overflow = false;

  int ta = next_tile(0);
  if (ta < ntl) {
    // ---- prologue: the first tile's content, rotary fragments and scores;
    // the second tile's copy issued between its MFMAs ----
    int tb = next_tile(ta + 1);
    int ba = 0, bb = 1, bn = 2;   // content buffers of t_s, t_s+1 and t_s+2
    int ksa = 0, ksb = 1;         // key-scale slots of t_s and t_s+1 (of three)
    {
      const uint8_t* cs = content_src(ta);
#pragma unroll
      for (int q = 0; q < LOADS; ++q) copy_load(cs, q, ba);
      const bf16_t* rs = rope_src(ta);
      if (!RS || wave >= 2) {
#pragma unroll
        for (int i = 0; i < NKR_W; ++i) kr[i] = *(const bf16x8_t*)(rs + i * 16);
      }
      ksc_copy(ta, 0);
    }
    // vmcnt(0) lgkmcnt(0), as the builtin: the compiler counts it as done
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070);
    asm volatile("" ::: "memory");
    lds_barrier();
    int cla = class_of(ta);
    if (cla == TILE_MASKED_ZERO) zero_content(ba, ta);
    {
      const bool have_b = tb < ntl;
      ksc_copy(have_b ? tb : ta, 1);
      const uint8_t* cs = content_src(have_b ? tb : ta);
      score_chain(ba, rope_src(have_b ? tb : ta), [&](int i) {
        if (copy_step(i)) copy_load(cs, copy_piece(i), bb);
      });
      write_partials();
    }

    for (;;) {
      // ---- top of step: t_s+1's content (in LDS) and rotary fragments (in
      // registers) have landed, this wave's partial scores of t_s are
      // written ----
      const bool have_b = tb < ntl;
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0x0070);
      asm volatile("" ::: "memory");
      // barrier A: every partial score of t_s and t_s+1's content are in
      // LDS; every wave is done with the probabilities
      lds_barrier();
      const int tc = have_b ? next_tile(tb + 1) : ntl;
      const bool have_c = tc < ntl;
      const int ksn = 3 - ksa - ksb;   // the third slot: t_s+2's
      ksc_copy(have_c ? tc : ta, ksn);
      // L2 prefetch of the tile DS_PF_AHEAD steps ahead: wave 0 loads one
      // 16-byte piece of each of 64 of its 128-byte lines (a global-to-LDS
      // load into a landing area nothing reads), slice (work-group / 8) of
      // the tile's lines, so that the work-groups of an XCD, which walk the
      // same tiles together, bring each tile into L2 before any of them
      // needs it (one step's loads would otherwise wait on the fetch from
      // beyond L2 together).  The wait at the top of the next step covers it.
      if (wave == 0) {
        constexpr int LPK = DQK / 64, TL = MF_BN * LPK, NSL = (TL + 63) / 64;   // lines per key, per tile
        const int kp0 = (t_begin + min(ta + DS_PF_AHEAD, ntl - 1)) * MF_BN;
        const int ln = min(64 * (int)((blockIdx.x >> 3) % NSL) + lane, TL - 1);
        const int kk = min(ln / LPK, cap - 1 - kp0);
        dma16((const uint8_t*)(cache_b + (size_t)(kp0 + kk) * DQK) + (ln % LPK) * 128,
              (uint32_t)(uintptr_t)(LDS_AS uint8_t*)pf_sink);
      }
      const int clb = have_b ? class_of(tb) : (int)TILE_FULL;
      if (clb == TILE_MASKED_ZERO) zero_content(bb, tb);
      const int k0a = (t_begin + ta) * MF_BN;
      const uint8_t* cs = content_src(have_c ? tc : ta);

      // ---- phase 1: scores of t_s+1 (a discarded repeat of t_s's content
      // when there is none), the softmax of t_s between them ----
      f32x4_t pr[8];
      f32x4_t kin[QKN ? 2 : 1];   // inverse RMS of the lane's eight keys of t_s
      float sv[8];
      float mloc = 0.f, neg_m = 0.f;
      bf16x8_t pf;
      VFrag vf0, vf1;
      score_chain(have_b ? bb : ba, rope_src(have_c ? tc : ta), [&](int i) {
        if (loop_copy_step(i) && have_c) copy_load(cs, loop_copy_piece(i), bn);
        if (i == 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            pr[2 * q] = *(const LDS_AS f32x4_t*)sx_chunk(sb, q, sl, 2 * sj);
            pr[2 * q + 1] = *(const LDS_AS f32x4_t*)sx_chunk(sb, q, sl, 2 * sj + 1);
          }
          if constexpr (QKN) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
              kin[h] = *(const LDS_AS f32x4_t*)(LDS_AS float*)(ksl + ksa * 256 + (16 * sj + 8 * h + 4 * sg) * 4);
          }
        } else if (i == 2) {
          if constexpr (QKN) {
            // content quarters (waves 0, 1) scaled by the key's inverse RMS,
            // then the rotary quarters (waves 2, 3), in a fixed order
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sv[e] = (fmaf(pr[0][e] + pr[2][e], kin[0][e], pr[4][e])) + pr[6][e];
              sv[4 + e] = (fmaf(pr[1][e] + pr[3][e], kin[1][e], pr[5][e])) + pr[7][e];
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sv[e] = ((pr[0][e] + pr[2][e]) + pr[4][e]) + pr[6][e];
              sv[4 + e] = ((pr[1][e] + pr[3][e]) + pr[5][e]) + pr[7][e];
            }
          }
          if (cla != TILE_FULL) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int sl2 = k0a + skey(e);
              bool vis = sl2 < cap;
              if (vis) vis = key_visible(fq, ring_frame(sl2 / P, newest, nm, W), W, fpb);
              if (!vis) sv[e] = -INFINITY;
            }
          }
          mloc = sv[0];
#pragma unroll
          for (int e = 1; e < 8; ++e) mloc = fmaxf(mloc, sv[e]);
        } else if (i == 3) {
          // over the row's four lanes (lane ^ 16, lane ^ 32)
          const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mloc), __float_as_uint(mloc), false, false);
          mloc = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
          mloc = halves_max(mloc) * c_l2;
        } else if (i == 4) {
          m_seen = fmaxf(m_seen, mloc);
          if (m_run == -INFINITY) m_run = mloc;                   // first visible tile of the row
          else if (mloc > m_run + ma.rerun_log2) overflow = true; // rerun with the final maxima
          neg_m = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sv[e], c_l2, neg_m));
            l_run += p;
            pf[e] = (__bf16)p;
          }
        } else if (i == 5) {
#pragma unroll
          for (int e = 4; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sv[e], c_l2, neg_m));
            l_run += p;
            pf[e] = (__bf16)p;
          }
          *(LDS_AS bf16x8_t*)p_entry(sb, sj, sl) = pf;
        }
        // t_s's value fragments, read while the last score steps run
        if (i == (NKS - 6 > 6 ? NKS - 6 : 6)) read_values(ba, 0, vf0);
        if (i == (NKS - 3 > 7 ? NKS - 3 : 7)) read_values(ba, 1, vf1);
      });
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // barrier B: every row's probabilities of t_s are published; every
      // partial score of t_s has been read
      lds_barrier();

      // ---- phase 2: t_s+1's partial scores to LDS, t_s's output product ----
      bf16x8_t pfr0[2], pfr1[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) pfr0[r] = *(const LDS_AS bf16x8_t*)p_entry(r, 0, lane);
#pragma unroll
      for (int r = 0; r < 2; ++r) pfr1[r] = *(const LDS_AS bf16x8_t*)p_entry(r, 1, lane);
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        output_one(m < 8 ? vf0 : vf1, m < 8 ? pfr0 : pfr1, (m & 7) >> 1, m & 1);
        if (LP1 < LOADS && m % 4 == 1 && have_c) copy_load(cs, LP1 + m / 4, bn);
        // (after the first key step's MFMAs: its probability reads are not
        // queued behind these writes; unconditional in the plain instance, so
        // the compiler can count them: a branch around them turned the wait
        // for the second key step's probabilities into lgkmcnt(0), behind all
        // eight writes.  After the last tile they write a discarded repeat
        // nobody reads.  With QK normalisation they follow the last MFMA,
        // where no read waits behind them: measured 2 % faster there.)
        if (QKN ? m == 15 && have_b : m == 7) write_partials();
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!have_b) break;
      ta = tb;
      tb = tc;
      cla = clb;
      const int bt = ba;
      ba = bb;
      bb = bn;
      bn = bt;
      ksa = ksb;
      ksb = ksn;
    }
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
  static_assert(DC == 512 && 3 * CT_BYTES >= DS_ROWS * DC * 2, "output staging");
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
  attn_plan(d, g, batch, n_rows, DS_ROWS, &ma, DS_MAX_PIECE_TILES);
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
  const int blocks = attn_plan(a.d, a.g, a.batch, a.n_rows, DS_ROWS, &ma, DS_MAX_PIECE_TILES);
  if (ws_bytes < attn_plan_workspace(ma)) return hipErrorInvalidValue;
  attn_plan_bind(&ma, ws);
  hipError_t e = a.d.d_r != 512 ? launch_dsplit_shape<512, 64, false>(ma, blocks, st)
                 : a.kscale     ? launch_dsplit_shape<512, 512, true>(ma, blocks, st)
                                : launch_dsplit_shape<512, 512, false>(ma, blocks, st);
  if (e != hipSuccess) return e;
  return launch_attn_merge(ma, st);
}

}  // namespace mla
