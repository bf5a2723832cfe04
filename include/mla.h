/*
 * mla.h - C-ABI of the MI355X (gfx950) multi-head latent attention library.
 *
 * Multi-head latent attention (MLA) caches, per token, one low-rank content
 * latent c_kv (d_c values) and one decoupled rotary key k_rope (d_r values),
 * shared by every head.  The key up-projection W^UK is absorbed into the query
 * and the value up-projection W^UV into the output, so per-head keys and values
 * are never materialised.
 *
 * Pages this interface follows (cited by title and section):
 *   [MLA concept]   "Multi-Head Latent Attention" (praveentn.live concept page):
 *                   Low-rank joint compression; The RoPE problem, and the
 *                   decoupled fix; When it breaks.
 *   [MLA explainer] "Understanding Multi-Head Latent Attention and KV
 *                   Compression": Low-Rank Joint Compression; On-the-Fly
 *                   Reconstruction and Matrix Absorption; Decoupling RoPE.
 *   [VideoMLA review] "VideoMLA: Compressing Video Diffusion Memory by 92.7%
 *                   with Low-Rank Latent Attention": The Gap; Core Mechanism;
 *                   Key Concepts.
 *   [MLA topics]    "Multi-Head Latent Attention" (thelatestinai.com topic
 *                   page): VideoMLA abstract; QuantMLA abstract.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer, owned by the caller, row-major
 *   and contiguous with the last dimension fastest, 16-byte aligned.  The
 *   library never allocates, frees or retains device memory.
 * - Floating-point tensors use dims->dtype (MLA_F32: float, MLA_BF16:
 *   bfloat16) for storage; all arithmetic accumulates in fp32.  `lse` is float.
 * - `stream` is a hipStream_t passed as void* (NULL = default stream).  Every
 *   call validates its arguments on the host, enqueues kernels on `stream` and
 *   returns without synchronising.
 * - Per-sequence frame counters (`frame`, `q_first`, `newest`) are DEVICE
 *   int32 arrays of length geom->batch, so a captured or repeated launch can
 *   advance them without a host round trip.
 * - Errors: an invalid argument returns MLA_ERR_INVALID_ARG (or
 *   MLA_ERR_UNSUPPORTED for a valid shape with no kernel) before anything is
 *   launched, leaving every output untouched; a failed launch returns
 *   MLA_ERR_HIP.  mla_last_error() gives a thread-local message for the last
 *   non-OK return.  Faults inside kernels surface at the caller's next
 *   synchronisation.  No C++ exception crosses this interface.
 * - Sizes of zero (batch, n_tokens, n_q) are valid and launch nothing.
 *
 * Cache geometry ([VideoMLA review, The Gap]; [MLA topics, VideoMLA abstract]:
 * a fixed-size sliding window of recent frames)
 * ---------------------------------------------------------------------------
 * A frame is grid_h x grid_w tokens, P = grid_h * grid_w, ordered row-major.
 * Each sequence owns a ring of `window` frames, capacity = window * P slots;
 * token `tok` of frame f lives in slot (f mod window) * P + tok.  A language
 * model is the same geometry with grid 1 x 1 (one token per frame, frame index
 * = token position) and window = the maximum context.
 * With `newest` the newest frame written, slot s holds frame
 *     f_k = newest - ((newest - s / P) mod window),   written iff f_k >= 0,
 * and a query of frame f_q sees that key iff it is written, is not in a later
 * block (f_k / frames_per_block <= f_q / frames_per_block: block-causal by
 * frame when frames_per_block = 1) and f_q - f_k < window.
 *
 * Rotary embedding ([MLA concept, The RoPE problem, and the decoupled fix];
 * [VideoMLA review, Key Concepts]: 3D-RoPE over time, height and width)
 * ---------------------------------------------------------------------------
 * rope_dims = 3: the d_r values split into bands of widths band[0..2] for
 * the coordinates (t, h, w) = (frame, row, column); rope_dims = 1: one band of
 * width d_r over the position frame * P + tok.  In a band of width b at
 * coordinate p, pair i = (u[2i], u[2i+1]) rotates by the angle p * theta^(-2i/b).
 */
#ifndef MLA_AMD_H
#define MLA_AMD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 1

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,
  MLA_ERR_UNSUPPORTED = -2,
  MLA_ERR_WORKSPACE = -3,
  MLA_ERR_HIP = -4
} mla_status;

enum { MLA_F32 = 0, MLA_BF16 = 1 };
enum { MLA_CACHE_DENSE = 0, MLA_CACHE_INT4 = 1, MLA_CACHE_INT2 = 2 };

/* Model dimensions, identical for every call on one cache. */
typedef struct {
  int32_t n_heads;     /* H */
  int32_t d_model;     /* hidden width */
  int32_t d_nope;      /* per-head content query/key width */
  int32_t d_v;         /* per-head value width */
  int32_t d_c;         /* shared content latent width (multiple of 32 for INT4 / INT2) */
  int32_t d_r;         /* shared rotary key width (even) */
  int32_t rope_dims;   /* 1 or 3 */
  int32_t band[3];     /* rotary band widths; 3D: (t, h, w), each even, sum d_r; 1D: band[0] = d_r */
  float rope_theta;    /* frequency base, e.g. 10000 */
  float softmax_scale; /* <= 0 selects 1/sqrt(d_nope + d_r) */
  int32_t dtype;       /* MLA_F32 or MLA_BF16 */
  int32_t cache_fmt;   /* MLA_CACHE_DENSE, MLA_CACHE_INT4 or MLA_CACHE_INT2 (low-bit: MLA_BF16 only) */
  int32_t qk_norm;     /* 1: QK-normalised attention (see "QK normalisation"), 0: off */
  float qk_norm_eps;   /* >= 0, added to the mean square inside the root (qk_norm = 1; d_c % 32 == 0) */
} mla_dims;

/* Cache geometry shared by every sequence of a batch. */
typedef struct {
  int32_t batch;            /* B sequences */
  int32_t grid_h, grid_w;   /* tokens per frame P = grid_h * grid_w */
  int32_t window;           /* frames per ring; capacity = window * P slots */
  int32_t frames_per_block; /* block-causal granularity (>= 1) */
} mla_geom;

/*
 * Cache storage.
 *   DENSE: cache = [B, capacity, d_c + d_r] in dims->dtype; cache_aux unused.
 *   INT4 ([MLA topics, QuantMLA abstract]: both cache paths in INT4, unpacked
 *   and dequantised inside attention):
 *     cache     = [B, capacity, (d_c + d_r) / 2] bytes; content codes then
 *                 rotary codes, element 2j in the low nibble of byte j, 2j+1 in
 *                 the high nibble, two's complement in [-8, 7];
 *     cache_aux = fp16 scales: [B, capacity, d_c / 32] per 32-element content
 *                 group, followed by [B, capacity] per-token rotary scales.
 *     value = code * scale; scale = fp16(amax / 7), code = round-half-even of
 *     x / scale clamped to [-8, 7] (IEEE fp32), a zero scale gives zero codes.
 *   INT2 (the same abstract's deeper variant: the content latent in INT2, the
 *   rotary key in INT4):
 *     cache     = [B, capacity, d_c / 4 + d_r / 2] bytes; content codes (element
 *                 4j + k in bits 2k .. 2k+1 of byte j, two's complement in
 *                 [-2, 1]) then the rotary codes as for INT4;
 *     cache_aux = as for INT4.  Content: scale = fp16(amax / 1), code =
 *     round-half-even of x / scale clamped to [-2, 1] (so -1, 0 or 1);
 *     rotary key as for INT4.
 *   QK normalisation on (dims->qk_norm = 1), any format: cache_aux also holds
 *     one float per slot, the key's inverse RMS [B, capacity], at byte offset
 *     0 (DENSE) or after the fp16 scales rounded up to 16 bytes (INT4, INT2);
 *     written by mla_cache_key_norm.
 * Both functions return 0 when the arguments are invalid.
 */
size_t mla_cache_bytes(const mla_dims* dims, const mla_geom* geom);
size_t mla_cache_aux_bytes(const mla_dims* dims, const mla_geom* geom);

/*
 * mla_cache_append: [MLA concept, Low-rank joint compression] and
 * [MLA explainer, Low-Rank Joint Compression; Decoupling RoPE].
 * For every sequence b and token i < n_tokens of x[b], with frame
 * f = frame[b] + i / P and tok = i % P:
 *     c      = w_dkr[0 : d_c] . x[b, i]        (content latent)
 *     k_rope = RoPE(w_dkr[d_c : d_c + d_r] . x[b, i], coordinates of (f, tok))
 *     cache row at slot (f mod window) * P + tok  <-  [c | k_rope] in the cache format.
 *   x       [B, n_tokens, d_model]   dims->dtype
 *   frame   [B] int32 (device)        first frame written per sequence (>= 0)
 *   w_dkr   [d_c + d_r, d_model]      dims->dtype (output-feature major)
 *   cache, cache_aux                  see "Cache storage"
 *   workspace: >= mla_append_workspace_size() bytes of device scratch.
 * n_tokens must be a multiple of P and n_tokens / P <= window.  The caller
 * tracks the newest frame (frame[b] + n_tokens / P - 1).
 */
size_t mla_append_workspace_size(const mla_dims* dims, const mla_geom* geom, int32_t n_tokens);
mla_status mla_cache_append(const mla_dims* dims, const mla_geom* geom, void* stream,
                            const void* x, int32_t n_tokens, const int32_t* frame,
                            const void* w_dkr, void* cache, void* cache_aux,
                            void* workspace, size_t workspace_bytes);

/*
 * mla_absorb_q: [MLA concept, Low-rank joint compression]: since
 * q . (W^UK c) = ((W^UK)^T q) . c, the key up-projection folds into the query.
 * For query token t of sequence b (frame q_first[b] + t / P, tok t % P) and head h:
 *     q_abs[b, t, h, 0 : d_c]        = w_uk[h] . q_nope[b, t, h]
 *     q_abs[b, t, h, d_c : d_c + d_r] = RoPE(q_rope[b, t, h], coordinates of the token)
 *   q_nope  [B, n_q, H, d_nope]; q_rope [B, n_q, H, d_r] (unrotated)
 *   q_first [B] int32 (device)
 *   w_uk    [H, d_c, d_nope]   w_uk[h] = (W^UK_h)^T, W^UK_h mapping c to the head's content key
 *   q_abs   [B, n_q, H, d_c + d_r]
 * With dims->qk_norm = 1 the content part is multiplied by inv_q of the token
 * (see "QK normalisation"; w_uk is then the folded weight).
 */
mla_status mla_absorb_q(const mla_dims* dims, const mla_geom* geom, void* stream, int32_t n_q,
                        const void* q_nope, const void* q_rope, const int32_t* q_first,
                        const void* w_uk, void* q_abs);

/*
 * QK normalisation ([MLA topics, QK-Norm abstract]: post-projection RMSNorm of
 * query and key splits into a static per-dimension weight, which folds into
 * the query side, and a dynamic RMS statistic, which for the key is one
 * scalar per token because every head's key comes from the one cached latent).
 * With g_q, g_k [H, d_nope] the norm weights and rms(v) = sqrt(mean(v^2) + eps)
 * over the H * d_nope content values of one token (all heads together), the
 * score of head h is
 *     scale * ( (g_q . q_h / rms(q)) . (g_k . W^UK_h c / rms(W^UK c)) + q_rope . k_rope )
 *   = scale * ( inv_q * inv_k * (w_uk'[h] q_h) . c + q_rope . k_rope )
 * with w_uk'[h][a][i] = w_uk[h][a][i] g_q[h][i] g_k[h][i] (folded at load
 * time), inv_q = 1 / rms(q_nope) (applied by mla_absorb_q) and
 * inv_k = 1 / sqrt(c^T G c / (H d_nope) + eps), G = sum_h w_uk[h] w_uk[h]^T
 * (stored per slot by mla_cache_key_norm, applied to the content score by
 * mla_attention).  The rotary parts are not normalised.
 * mla_qk_norm_prepare (load time):
 *   w_uk [H, d_c, d_nope] (unweighted), g_q, g_k [H, d_nope] (dims->dtype)
 *   -> w_uk_folded [H, d_c, d_nope] (dims->dtype; pass it to mla_absorb_q)
 *      gram [d_c, d_c] float (pass it to mla_cache_key_norm)
 * mla_cache_key_norm: after mla_cache_append with the same n_tokens and
 *   frame (or after rows were written otherwise), stores inv_k of those rows,
 *   computed from the stored latent (what attention reads); workspace: >=
 *   mla_key_norm_workspace_size() bytes (0 when the call has many tokens;
 *   partial sums otherwise, added in a fixed order).
 * With qk_norm = 1, mla_absorb_q_folded returns MLA_ERR_UNSUPPORTED.
 */
mla_status mla_qk_norm_prepare(const mla_dims* dims, void* stream, const void* w_uk, const void* g_q,
                               const void* g_k, void* w_uk_folded, float* gram);
size_t mla_key_norm_workspace_size(const mla_dims* dims, const mla_geom* geom, int32_t n_tokens);
mla_status mla_cache_key_norm(const mla_dims* dims, const mla_geom* geom, void* stream, int32_t n_tokens,
                              const int32_t* frame, const float* gram, const void* cache, void* cache_aux,
                              void* workspace, size_t workspace_bytes);

/*
 * Low-rank query with the key up-projection folded in when the weights are
 * loaded: [MLA concept, Low-rank joint compression] (q . k = c^Q^T (W^UQ^T
 * W^UK) c^KV, so the product of the two up-projections is formed once).
 * mla_fold_query_weights (load time):
 *     w_fold[h] = w_uk[h] . W^UQ_h        (fp32 accumulation, one rounding)
 *   w_uq   [H * d_nope, d_cq]  the query up-projection, output-feature major:
 *          q_nope[.., h, i] = sum_j w_uq[h * d_nope + i, j] c_q[.., j]
 *   w_uk   [H, d_c, d_nope]    as for mla_absorb_q
 *   w_fold [H, d_c, d_cq]
 * mla_absorb_q_folded (instead of mla_absorb_q when the model has a query latent):
 *     q_abs[b, t, h, 0 : d_c]        = w_fold[h] . c_q[b, t]
 *     q_abs[b, t, h, d_c : d_c + d_r] = RoPE(q_rope[b, t, h], coordinates of the token)
 *   c_q [B, n_q, d_cq]; q_rope, q_first, q_abs as for mla_absorb_q.
 * d_cq must be positive (bf16: a multiple of 8, else MLA_ERR_UNSUPPORTED).
 * The fold trades the per-head product over d_nope (plus the query
 * up-projection, outside this library) for one product over d_cq with a
 * weight d_c / d_nope times the size of W^UQ.
 */
mla_status mla_fold_query_weights(const mla_dims* dims, void* stream, int32_t d_cq, const void* w_uq,
                                  const void* w_uk, void* w_fold);
mla_status mla_absorb_q_folded(const mla_dims* dims, const mla_geom* geom, void* stream, int32_t n_q,
                               int32_t d_cq, const void* c_q, const void* q_rope, const int32_t* q_first,
                               const void* w_fold, void* q_abs);

/*
 * mla_attention: [MLA concept, Low-rank joint compression] (with both
 * up-projections absorbed, decode-time attention runs on the latents
 * themselves) and [The RoPE problem, and the decoupled fix] (score = content
 * term + rotary term); [MLA explainer, Decoupling RoPE] (concatenated rows).
 * For every (b, t, h), over the slots s visible to frame q_first[b] + t / P:
 *     a_s = scale * q_abs[b, t, h] . cache_row[b, s]          (width d_c + d_r)
 *     o_lat[b, t, h] = sum_s softmax(a)_s * cache_row[b, s, 0 : d_c]
 *     lse[b, t, h]   = log sum_s exp(a_s)
 * A row with no visible key gives o_lat = 0 and lse = -inf.
 * With dims->qk_norm = 1 the content part of a_s (the first d_c terms) is
 * multiplied by the slot's stored inv_k (see "QK normalisation").
 *   q_abs   [B, n_q, H, d_c + d_r]; q_first [B], newest [B] int32 (device)
 *   o_lat   [B, n_q, H, d_c]; lse [B, n_q, H] float, or NULL
 *   workspace: >= mla_attention_workspace_size() bytes (split-key partials).
 */
size_t mla_attention_workspace_size(const mla_dims* dims, const mla_geom* geom, int32_t n_q);
mla_status mla_attention(const mla_dims* dims, const mla_geom* geom, void* stream, int32_t n_q,
                         const void* q_abs, const int32_t* q_first, const int32_t* newest,
                         const void* cache, const void* cache_aux,
                         void* o_lat, float* lse, void* workspace, size_t workspace_bytes);

/*
 * mla_attention_noalloc: mla_attention for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments and results as mla_attention minus
 * the workspace: the split-key partials go to a static device array of
 * MLA_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, held until the
 * process ends, its address looked up on the first call on each device).
 * Nothing is allocated, freed or cleared by the call.
 *   - A call whose partials need more than MLA_NOALLOC_SCRATCH_BYTES (see
 *     mla_attention_workspace_size) returns MLA_ERR_WORKSPACE before anything
 *     is launched; decode at batch 32 x 128 heads needs about 32 MiB, a
 *     1560-token video chunk about 245 MiB (use mla_attention there).
 *   - Every call on one GPU shares that GPU's array: calls that overlap on one
 *     GPU (concurrent streams, or host threads) race and give wrong results.
 *     Serialise them, or use mla_attention with a workspace per stream.
 *   - The stream must belong to the calling thread's current device.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)
mla_status mla_attention_noalloc(const mla_dims* dims, const mla_geom* geom, void* stream, int32_t n_q,
                                 const void* q_abs, const int32_t* q_first, const int32_t* newest,
                                 const void* cache, const void* cache_aux, void* o_lat, float* lse);

/*
 * mla_unabsorb_out: [MLA concept, Low-rank joint compression] (W^UV is absorbed
 * on the output side, as W^UK is on the query side); [MLA explainer, On-the-Fly
 * Reconstruction and Matrix Absorption].
 *     o_heads[b, t, h*d_v : (h+1)*d_v] = w_uv[h] . o_lat[b, t, h]
 *     y[b, t] = w_o . o_heads[b, t]
 *   o_lat [B, n_q, H, d_c]; w_uv [H, d_v, d_c]; w_o [d_model, H * d_v]
 *   o_heads [B, n_q, H * d_v] (written, also usable as scratch); y [B, n_q, d_model]
 */
mla_status mla_unabsorb_out(const mla_dims* dims, const mla_geom* geom, void* stream, int32_t n_q,
                            const void* o_lat, const void* w_uv, const void* w_o,
                            void* o_heads, void* y);

/*
 * mla_cache_rope_shift: [MLA topics, Irminsul abstract] (the rotary key of a
 * cached row is corrected in closed form when its token moves; the content
 * latent carries no position) and [MLA topics, the RedKnot head-aware reuse
 * abstract] (content computed at one position is relocated to another).
 * Rotations by angles proportional to the coordinate compose,
 * R(p + delta) = R(delta) R(p), so for every sequence b and slot s in
 * [slot_begin, slot_begin + n_slots):
 *     cache_row[b, s, d_c : d_c + d_r]  <-  R(delta[b]) cache_row[b, s, d_c : d_c + d_r]
 * i.e. the key as if the token had been appended delta[b] further along
 * (pair i of a band of width w turns by delta_axis * theta^(-2i/w)).
 *   delta  [B, 3] int32 (device): the shift of (t, h, w); rope_dims = 1 uses
 *          delta[b, 0] (a position shift) and ignores the rest
 *   cache, cache_aux: see "Cache storage"; the content latent and every other
 *          slot are left untouched.  Dense: rotated in fp32, rounded to
 *          dims->dtype.  Low-bit: the INT4 rotary codes are dequantised,
 *          rotated, rounded to bf16 and re-quantised with a new per-token
 *          scale.  A shift that is zero in the coordinates used leaves the
 *          rows unchanged bit for bit.
 * Errors: the slot range must lie inside [0, capacity) (MLA_ERR_INVALID_ARG).
 * The caller owns the positions: queries that should see the moved keys at
 * their new offsets are absorbed at positions shifted by the same delta.
 */
mla_status mla_cache_rope_shift(const mla_dims* dims, const mla_geom* geom, void* stream,
                                const int32_t* delta, int32_t slot_begin, int32_t n_slots,
                                void* cache, void* cache_aux);

/* Inspection utility (not on the hot path): cache rows as float [B, capacity, d_c + d_r]. */
mla_status mla_cache_dequant(const mla_dims* dims, const mla_geom* geom, void* stream,
                             const void* cache, const void* cache_aux, float* out);

const char* mla_status_string(int status);
const char* mla_last_error(void);
int mla_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_AMD_H */
