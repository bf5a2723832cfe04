// C-ABI entry points: host-side validation and dispatch to the HIP kernels.
// Every check runs before anything is enqueued, so an invalid call leaves all
// outputs untouched.  No exception crosses the interface; the last error
// message is kept per thread.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "launch.hpp"


using namespace mla;

namespace {

thread_local std::string g_last_error;

mla_status fail(mla_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool sync_check_enabled() {
  static int v = [] {
    const char* e = getenv("MLA_SYNC_CHECK");
    return (e && e[0] == '1') ? 1 : 0;
  }();
  return v != 0;
}

mla_status hip_status(hipError_t e, hipStream_t st, const char* what) {
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  if (sync_check_enabled()) {
    e = hipStreamSynchronize(st);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s (synchronised check): %s", what, hipGetErrorString(e));
  }
  return MLA_OK;
}

// validate dims; fill the kernel-side copy
mla_status check_dims(const mla_dims* dm, Dims* d) {
  if (!dm) return fail(MLA_ERR_INVALID_ARG, "dims is NULL");
  if (dm->n_heads <= 0 || dm->d_model <= 0 || dm->d_nope <= 0 || dm->d_v <= 0 || dm->d_c <= 0 ||
      dm->d_r <= 0)
    return fail(MLA_ERR_INVALID_ARG, "n_heads, d_model, d_nope, d_v, d_c and d_r must be positive");
  if (dm->d_r % 2) return fail(MLA_ERR_INVALID_ARG, "d_r must be even (rotary pairs), got %d", dm->d_r);
  if (dm->rope_dims == 1) {
    if (dm->band[0] != dm->d_r)
      return fail(MLA_ERR_INVALID_ARG, "1D rotary: band[0] must equal d_r");
  } else if (dm->rope_dims == 3) {
    for (int i = 0; i < 3; ++i)
      if (dm->band[i] < 0 || dm->band[i] % 2)
        return fail(MLA_ERR_INVALID_ARG, "3D rotary: band widths must be even and >= 0");
    if (dm->band[0] + dm->band[1] + dm->band[2] != dm->d_r)
      return fail(MLA_ERR_INVALID_ARG, "3D rotary: band widths sum to %d, d_r is %d",
                  dm->band[0] + dm->band[1] + dm->band[2], dm->d_r);
  } else {
    return fail(MLA_ERR_INVALID_ARG, "rope_dims must be 1 or 3, got %d", dm->rope_dims);
  }
  if (!(dm->rope_theta > 0.f)) return fail(MLA_ERR_INVALID_ARG, "rope_theta must be positive");
  if (dm->dtype != MLA_F32 && dm->dtype != MLA_BF16)
    return fail(MLA_ERR_INVALID_ARG, "dtype must be MLA_F32 or MLA_BF16");
  if (dm->cache_fmt != MLA_CACHE_DENSE && dm->cache_fmt != MLA_CACHE_INT4 && dm->cache_fmt != MLA_CACHE_INT2)
    return fail(MLA_ERR_INVALID_ARG, "cache_fmt must be MLA_CACHE_DENSE, MLA_CACHE_INT4 or MLA_CACHE_INT2");
  if (dm->cache_fmt != MLA_CACHE_DENSE) {
    if (dm->dtype != MLA_BF16) return fail(MLA_ERR_INVALID_ARG, "a low-bit cache requires MLA_BF16");
    if (dm->d_c % 32) return fail(MLA_ERR_INVALID_ARG, "a low-bit cache requires d_c %% 32 == 0");
  }
  if (dm->qk_norm != 0 && dm->qk_norm != 1) return fail(MLA_ERR_INVALID_ARG, "qk_norm must be 0 or 1");
  if (dm->qk_norm && !(dm->qk_norm_eps >= 0.f && dm->qk_norm_eps < 1e30f))
    return fail(MLA_ERR_INVALID_ARG, "qk_norm_eps must be finite and >= 0");
  if (dm->qk_norm && dm->d_c % 32)
    return fail(MLA_ERR_UNSUPPORTED, "QK normalisation needs d_c divisible by 32, got %d", dm->d_c);
  const int dqk = dm->d_c + dm->d_r;
  if (dm->d_c > 1024 || dqk > 1536)
    return fail(MLA_ERR_UNSUPPORTED, "d_c <= 1024 and d_c + d_r <= 1536 are supported");
  if (dm->dtype == MLA_BF16) {
    // 16-byte vector loads in the bf16 kernels
    if (dm->d_model % 8 || dm->d_nope % 8 || dm->d_c % 8 || dm->d_v % 8 || dm->d_r % 8)
      return fail(MLA_ERR_UNSUPPORTED, "bf16 kernels need d_model, d_nope, d_v, d_c, d_r divisible by 8");
  }
  d->H = dm->n_heads;
  d->d_model = dm->d_model;
  d->d_nope = dm->d_nope;
  d->d_v = dm->d_v;
  d->d_c = dm->d_c;
  d->d_r = dm->d_r;
  d->d_qk = dqk;
  d->rope_dims = dm->rope_dims;
  d->band0 = dm->band[0];
  d->band1 = dm->rope_dims == 3 ? dm->band[1] : 0;
  d->band2 = dm->rope_dims == 3 ? dm->band[2] : 0;
  d->theta = dm->rope_theta;
  d->scale = dm->softmax_scale > 0.f ? dm->softmax_scale : 1.0f / sqrtf((float)(dm->d_nope + dm->d_r));
  d->dtype = dm->dtype;
  d->cache_fmt = dm->cache_fmt;
  d->qk_norm = dm->qk_norm;
  d->qk_eps = dm->qk_norm ? dm->qk_norm_eps : 0.f;
  return MLA_OK;
}

mla_status check_geom(const mla_geom* gm, const Dims& d, Geo* g) {
  if (!gm) return fail(MLA_ERR_INVALID_ARG, "geom is NULL");
  if (gm->batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 0");
  if (gm->grid_h <= 0 || gm->grid_w <= 0 || gm->window <= 0 || gm->frames_per_block <= 0)
    return fail(MLA_ERR_INVALID_ARG, "grid_h, grid_w, window and frames_per_block must be positive");
  const long long P = (long long)gm->grid_h * gm->grid_w;
  const long long cap = P * gm->window;
  if (cap >= (1ll << 30)) return fail(MLA_ERR_INVALID_ARG, "capacity window * P too large");
  if ((long long)gm->batch * cap * d.d_qk >= (1ll << 40))
    return fail(MLA_ERR_INVALID_ARG, "cache too large");
  g->P = (int)P;
  g->grid_w = gm->grid_w;
  g->window = gm->window;
  g->fpb = gm->frames_per_block;
  g->capacity = (int)cap;
  return MLA_OK;
}

size_t elem_size(const Dims& d) { return d.dtype == MLA_BF16 ? 2 : 4; }

#define CHECK(expr)            \
  do {                         \
    mla_status _s = (expr);    \
    if (_s != MLA_OK) return _s; \
  } while (0)

#define NEED_PTR(p)                                                                   \
  do {                                                                                \
    if (!(p)) return fail(MLA_ERR_INVALID_ARG, "%s is NULL", #p);                     \
    if (!aligned16(p)) return fail(MLA_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
  } while (0)

}  // namespace

extern "C" {

int mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_last_error(void) { return g_last_error.c_str(); }

const char* mla_status_string(int s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    default: return "unknown mla_status";
  }
}

size_t mla_cache_bytes(const mla_dims* dims, const mla_geom* geom) {
  Dims d;
  Geo g;
  if (check_dims(dims, &d) != MLA_OK || check_geom(geom, d, &g) != MLA_OK) return 0;
  const size_t rows = (size_t)geom->batch * g.capacity;
  if (lowbit_cache(d)) return rows * code_row_bytes(d);
  return rows * d.d_qk * elem_size(d);
}

size_t mla_cache_aux_bytes(const mla_dims* dims, const mla_geom* geom) {
  Dims d;
  Geo g;
  if (check_dims(dims, &d) != MLA_OK || check_geom(geom, d, &g) != MLA_OK) return 0;
  const size_t rows = (size_t)geom->batch * g.capacity;
  if (d.qk_norm) return key_scale_offset(d, rows) + rows * sizeof(float);
  if (!lowbit_cache(d)) return 0;
  return rows * (d.d_c / 32 + 1) * sizeof(__half);
}

// fp32 projection rows of the appended tokens, one copy per K split
static size_t append_ws_bytes(const Dims& d, int batch, int n_tokens) {
  const int M = batch * n_tokens;
  const int ks = gemm_skinny_ksplit(d.dtype, M, d.d_qk, d.d_model, 1);
  return (size_t)ks * M * d.d_qk * sizeof(float);
}

size_t mla_append_workspace_size(const mla_dims* dims, const mla_geom* geom, int32_t n_tokens) {
  Dims d;
  Geo g;
  if (check_dims(dims, &d) != MLA_OK || check_geom(geom, d, &g) != MLA_OK || n_tokens < 0) return 0;
  return append_ws_bytes(d, geom->batch, n_tokens);
}

mla_status mla_cache_append(const mla_dims* dims, const mla_geom* geom, void* stream, const void* x,
                            int32_t n_tokens, const int32_t* frame, const void* w_dkr, void* cache,
                            void* cache_aux, void* workspace, size_t workspace_bytes) {
  Dims d;
  Geo g;
  CHECK(check_dims(dims, &d));
  CHECK(check_geom(geom, d, &g));
  if (n_tokens < 0) return fail(MLA_ERR_INVALID_ARG, "n_tokens must be >= 0");
  if (n_tokens % g.P) return fail(MLA_ERR_INVALID_ARG, "n_tokens (%d) must be a multiple of P (%d)", n_tokens, g.P);
  if (n_tokens / g.P > g.window)
    return fail(MLA_ERR_INVALID_ARG, "one append may not write more frames (%d) than the window (%d)",
                n_tokens / g.P, g.window);
  const int B = geom->batch;
  if (B == 0 || n_tokens == 0) return MLA_OK;
  NEED_PTR(x);
  NEED_PTR(frame);
  NEED_PTR(w_dkr);
  NEED_PTR(cache);
  NEED_PTR(workspace);
  if (lowbit_cache(d)) NEED_PTR(cache_aux);
  const size_t need = append_ws_bytes(d, B, n_tokens);
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "append workspace needs %zu bytes, got %zu", need, workspace_bytes);
  hipStream_t st = (hipStream_t)stream;
  GemmArgs ga;
  ga.M = B * n_tokens;
  ga.N = d.d_qk;
  ga.K = d.d_model;
  ga.batch = 1;
  ga.A = x; ga.lda = d.d_model; ga.sA = 0;
  ga.B = w_dkr; ga.ldb = d.d_model; ga.sB = 0;
  ga.C = workspace; ga.ldc = d.d_qk; ga.sC = 0;
  ga.out_f32 = 1;
  ga.ksplit = gemm_skinny_ksplit(d.dtype, ga.M, ga.N, ga.K, 1);
  ga.sSplit = (long long)ga.M * d.d_qk;
  hipError_t e = launch_gemm_nt(d.dtype, ga, st);
  if (e != hipSuccess) return hip_status(e, st, "append projection");
  e = launch_append_store(d, g, B, (const float*)workspace, n_tokens, frame, cache, cache_aux, ga.ksplit, st);
  return hip_status(e, st, "append store");
}

mla_status mla_absorb_q(const mla_dims* dims, const mla_geom* geom, void* stream, int32_t n_q,
                        const void* q_nope, const void* q_rope, const int32_t* q_first,
                        const void* w_uk, void* q_abs) {
  Dims d;
  Geo g;
  CHECK(check_dims(dims, &d));
  CHECK(check_geom(geom, d, &g));
  if (n_q < 0) return fail(MLA_ERR_INVALID_ARG, "n_q must be >= 0");
  const int B = geom->batch;
  if (B == 0 || n_q == 0) return MLA_OK;
  NEED_PTR(q_nope);
  NEED_PTR(q_rope);
  NEED_PTR(q_first);
  NEED_PTR(w_uk);
  NEED_PTR(q_abs);
  hipStream_t st = (hipStream_t)stream;
  // per head h: q_abs[:, h, 0:d_c] = q_nope[:, h, :] . w_uk[h]^T
  GemmArgs ga;
  ga.M = B * n_q;
  ga.N = d.d_c;
  ga.K = d.d_nope;
  ga.batch = d.H;
  ga.A = q_nope; ga.lda = (long long)d.H * d.d_nope; ga.sA = d.d_nope;
  ga.B = w_uk; ga.ldb = d.d_nope; ga.sB = (long long)d.d_c * d.d_nope;
  ga.C = q_abs; ga.ldc = (long long)d.H * d.d_qk; ga.sC = d.d_qk;
  ga.out_f32 = 0;
  if (absorb_rope_fusable(d, ga))
    return hip_status(launch_absorb_rope(d, g, ga, B, q_rope, n_q, q_first, q_abs, st), st,
                      "absorbed query");
  hipError_t e = launch_gemm_nt(d.dtype, ga, st);
  if (e != hipSuccess) return hip_status(e, st, "absorb projection");
  e = launch_q_rope(d, g, B, q_rope, n_q, q_first, q_nope, q_abs, st);
  return hip_status(e, st, "query rotary");
}

static mla_status check_d_cq(const Dims& d, int32_t d_cq) {
  if (d_cq <= 0) return fail(MLA_ERR_INVALID_ARG, "d_cq must be positive, got %d", d_cq);
  if (d.dtype == MLA_BF16 && d_cq % 8)
    return fail(MLA_ERR_UNSUPPORTED, "bf16 kernels need d_cq divisible by 8, got %d", d_cq);
  return MLA_OK;
}

mla_status mla_fold_query_weights(const mla_dims* dims, void* stream, int32_t d_cq, const void* w_uq,
                                  const void* w_uk, void* w_fold) {
  Dims d;
  CHECK(check_dims(dims, &d));
  CHECK(check_d_cq(d, d_cq));
  NEED_PTR(w_uq);
  NEED_PTR(w_uk);
  NEED_PTR(w_fold);
  hipStream_t st = (hipStream_t)stream;
  return hip_status(launch_fold_query(d, d_cq, w_uq, w_uk, w_fold, st), st, "query weight fold");
}

mla_status mla_absorb_q_folded(const mla_dims* dims, const mla_geom* geom, void* stream, int32_t n_q,
                               int32_t d_cq, const void* c_q, const void* q_rope, const int32_t* q_first,
                               const void* w_fold, void* q_abs) {
  Dims d;
  Geo g;
  CHECK(check_dims(dims, &d));
  CHECK(check_geom(geom, d, &g));
  CHECK(check_d_cq(d, d_cq));
  if (d.qk_norm)
    return fail(MLA_ERR_UNSUPPORTED, "QK normalisation needs the query's content values (use mla_absorb_q)");
  if (n_q < 0) return fail(MLA_ERR_INVALID_ARG, "n_q must be >= 0");
  const int B = geom->batch;
  if (B == 0 || n_q == 0) return MLA_OK;
  NEED_PTR(c_q);
  NEED_PTR(q_rope);
  NEED_PTR(q_first);
  NEED_PTR(w_fold);
  NEED_PTR(q_abs);
  hipStream_t st = (hipStream_t)stream;
  // per head h: q_abs[:, h, 0:d_c] = c_q . w_fold[h]^T (every head reads the same query latents)
  GemmArgs ga;
  ga.M = B * n_q;
  ga.N = d.d_c;
  ga.K = d_cq;
  ga.batch = d.H;
  ga.A = c_q; ga.lda = d_cq; ga.sA = 0;
  ga.B = w_fold; ga.ldb = d_cq; ga.sB = (long long)d.d_c * d_cq;
  ga.C = q_abs; ga.ldc = (long long)d.H * d.d_qk; ga.sC = d.d_qk;
  ga.out_f32 = 0;
  hipError_t e = launch_gemm_nt(d.dtype, ga, st);
  if (e != hipSuccess) return hip_status(e, st, "folded absorb projection");
  e = launch_q_rope(d, g, B, q_rope, n_q, q_first, nullptr, q_abs, st);
  return hip_status(e, st, "query rotary");
}

size_t mla_attention_workspace_size(const mla_dims* dims, const mla_geom* geom, int32_t n_q) {
  Dims d;
  Geo g;
  if (check_dims(dims, &d) != MLA_OK || check_geom(geom, d, &g) != MLA_OK || n_q < 0) return 0;
  if (attn_mfma_supported(d, g)) return attn_mfma_workspace(d, g, geom->batch, n_q * d.H);
  if (attn_dsplit_supported(d)) return attn_dsplit_workspace(d, g, geom->batch, n_q * d.H);
  return 0;
}

}  // extern "C"

namespace {

// Scratch of the allocation-free attention call: a file-scope device array
// (each GPU the library runs on holds its own copy until the process ends).
// Host code never passes the array's name to a kernel: it stands for a host
// shadow there; the device address comes from hipGetSymbolAddress, looked up
// once per device with that device current.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)MLA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];   // device address of `scratch` per device (null: not looked up yet)

mla_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES)
    return fail(MLA_ERR_UNSUPPORTED, "device %d: the static scratch is kept for devices 0 .. %d", dev,
                MAX_DEVICES - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

// mla_attention and mla_attention_noalloc: validation, then the kernels with
// the caller's workspace (noalloc = false) or the static scratch
mla_status attention_impl(const mla_dims* dims, const mla_geom* geom, void* stream, int32_t n_q,
                          const void* q_abs, const int32_t* q_first, const int32_t* newest,
                          const void* cache, const void* cache_aux, void* o_lat, float* lse,
                          void* workspace, size_t workspace_bytes, bool noalloc) {
  Dims d;
  Geo g;
  CHECK(check_dims(dims, &d));
  CHECK(check_geom(geom, d, &g));
  if (n_q < 0) return fail(MLA_ERR_INVALID_ARG, "n_q must be >= 0");
  const int B = geom->batch;
  if (B == 0 || n_q == 0) return MLA_OK;
  if ((long long)n_q * d.H >= (1ll << 30)) return fail(MLA_ERR_INVALID_ARG, "n_q * n_heads too large");
  NEED_PTR(q_abs);
  NEED_PTR(q_first);
  NEED_PTR(newest);
  NEED_PTR(cache);
  NEED_PTR(o_lat);
  if (lse && ((uintptr_t)lse & 3u)) return fail(MLA_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  if (lowbit_cache(d) || d.qk_norm) NEED_PTR(cache_aux);
  AttnArgs a;
  a.d = d;
  a.g = g;
  a.n_q = n_q;
  a.n_rows = n_q * d.H;
  a.q_abs = q_abs;
  a.q_first = q_first;
  a.newest = newest;
  a.cache = cache;
  a.aux = (const __half*)cache_aux;
  a.kscale = d.qk_norm ? (const float*)((const char*)cache_aux + key_scale_offset(d, (size_t)B * g.capacity))
                       : nullptr;
  a.batch = B;
  a.o_lat = o_lat;
  a.lse = lse;
  hipStream_t st = (hipStream_t)stream;
  const bool narrow = attn_mfma_supported(d, g), wide = !narrow && attn_dsplit_supported(d);
  if (narrow || wide) {
    const size_t need = narrow ? attn_mfma_workspace(d, g, B, a.n_rows) : attn_dsplit_workspace(d, g, B, a.n_rows);
    if (noalloc) {
      if (need > NOALLOC_SCRATCH_BYTES)
        return fail(MLA_ERR_WORKSPACE,
                    "this call needs %zu bytes of scratch; the library's static scratch holds %zu "
                    "(use mla_attention with a workspace)", need, NOALLOC_SCRATCH_BYTES);
      workspace = nullptr;
      workspace_bytes = NOALLOC_SCRATCH_BYTES;
      if (need) CHECK(scratch_of_current_device(&workspace));
    } else {
      if (need && (workspace_bytes < need || !workspace))
        return fail(MLA_ERR_WORKSPACE, "attention workspace needs %zu bytes, got %zu", need, workspace_bytes);
      if (need && !aligned16(workspace)) return fail(MLA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    }
    if (narrow) return hip_status(launch_attn_mfma(a, workspace, workspace_bytes, st), st, "latent attention (MFMA)");
    return hip_status(launch_attn_dsplit(a, workspace, workspace_bytes, st), st, "latent attention (MFMA, split rows)");
  }
  return hip_status(launch_attn_simt(a, st), st, "latent attention");
}

}  // namespace

extern "C" {

mla_status mla_attention(const mla_dims* dims, const mla_geom* geom, void* stream, int32_t n_q,
                         const void* q_abs, const int32_t* q_first, const int32_t* newest,
                         const void* cache, const void* cache_aux, void* o_lat, float* lse,
                         void* workspace, size_t workspace_bytes) {
  return attention_impl(dims, geom, stream, n_q, q_abs, q_first, newest, cache, cache_aux, o_lat, lse, workspace,
                        workspace_bytes, false);
}

mla_status mla_attention_noalloc(const mla_dims* dims, const mla_geom* geom, void* stream, int32_t n_q,
                                 const void* q_abs, const int32_t* q_first, const int32_t* newest,
                                 const void* cache, const void* cache_aux, void* o_lat, float* lse) {
  return attention_impl(dims, geom, stream, n_q, q_abs, q_first, newest, cache, cache_aux, o_lat, lse, nullptr, 0,
                        true);
}

mla_status mla_unabsorb_out(const mla_dims* dims, const mla_geom* geom, void* stream, int32_t n_q,
                            const void* o_lat, const void* w_uv, const void* w_o, void* o_heads,
                            void* y) {
  Dims d;
  Geo g;
  CHECK(check_dims(dims, &d));
  CHECK(check_geom(geom, d, &g));
  if (n_q < 0) return fail(MLA_ERR_INVALID_ARG, "n_q must be >= 0");
  const int B = geom->batch;
  if (B == 0 || n_q == 0) return MLA_OK;
  NEED_PTR(o_lat);
  NEED_PTR(w_uv);
  NEED_PTR(w_o);
  NEED_PTR(o_heads);
  NEED_PTR(y);
  hipStream_t st = (hipStream_t)stream;
  GemmArgs ga;
  ga.M = B * n_q;
  ga.N = d.d_v;
  ga.K = d.d_c;
  ga.batch = d.H;
  ga.A = o_lat; ga.lda = (long long)d.H * d.d_c; ga.sA = d.d_c;
  ga.B = w_uv; ga.ldb = d.d_c; ga.sB = (long long)d.d_v * d.d_c;
  ga.C = o_heads; ga.ldc = (long long)d.H * d.d_v; ga.sC = d.d_v;
  ga.out_f32 = 0;
  hipError_t e = launch_gemm_nt(d.dtype, ga, st);
  if (e != hipSuccess) return hip_status(e, st, "value up-projection");
  GemmArgs gb;
  gb.M = B * n_q;
  gb.N = d.d_model;
  gb.K = d.H * d.d_v;
  gb.batch = 1;
  gb.A = o_heads; gb.lda = (long long)d.H * d.d_v; gb.sA = 0;
  gb.B = w_o; gb.ldb = (long long)d.H * d.d_v; gb.sB = 0;
  gb.C = y; gb.ldc = d.d_model; gb.sC = 0;
  gb.out_f32 = 0;
  e = launch_gemm_nt(d.dtype, gb, st);
  return hip_status(e, st, "output projection");
}

mla_status mla_cache_dequant(const mla_dims* dims, const mla_geom* geom, void* stream,
                             const void* cache, const void* cache_aux, float* out) {
  Dims d;
  Geo g;
  CHECK(check_dims(dims, &d));
  CHECK(check_geom(geom, d, &g));
  if (geom->batch == 0) return MLA_OK;
  NEED_PTR(cache);
  NEED_PTR(out);
  if (lowbit_cache(d)) NEED_PTR(cache_aux);
  hipStream_t st = (hipStream_t)stream;
  return hip_status(launch_dequant(d, g, geom->batch, cache, cache_aux, out, st), st, "cache dequant");
}

mla_status mla_qk_norm_prepare(const mla_dims* dims, void* stream, const void* w_uk, const void* g_q,
                               const void* g_k, void* w_uk_folded, float* gram) {
  Dims d;
  CHECK(check_dims(dims, &d));
  NEED_PTR(w_uk);
  NEED_PTR(g_q);
  NEED_PTR(g_k);
  NEED_PTR(w_uk_folded);
  NEED_PTR(gram);
  hipStream_t st = (hipStream_t)stream;
  return hip_status(launch_qkn_prepare(d, w_uk, g_q, g_k, w_uk_folded, gram, st), st, "QK-norm weight preparation");
}

static size_t key_norm_ws_bytes(const Dims& d, int batch, int n_tokens) {
  const int z = key_norm_slices(d, batch, n_tokens);
  return z > 1 ? (size_t)z * batch * n_tokens * sizeof(float) : 0;
}

size_t mla_key_norm_workspace_size(const mla_dims* dims, const mla_geom* geom, int32_t n_tokens) {
  Dims d;
  Geo g;
  if (check_dims(dims, &d) != MLA_OK || check_geom(geom, d, &g) != MLA_OK || n_tokens < 0) return 0;
  return key_norm_ws_bytes(d, geom->batch, n_tokens);
}

mla_status mla_cache_key_norm(const mla_dims* dims, const mla_geom* geom, void* stream, int32_t n_tokens,
                              const int32_t* frame, const float* gram, const void* cache, void* cache_aux,
                              void* workspace, size_t workspace_bytes) {
  Dims d;
  Geo g;
  CHECK(check_dims(dims, &d));
  CHECK(check_geom(geom, d, &g));
  if (!d.qk_norm) return fail(MLA_ERR_INVALID_ARG, "mla_cache_key_norm needs dims->qk_norm = 1");
  if (n_tokens < 0) return fail(MLA_ERR_INVALID_ARG, "n_tokens must be >= 0");
  if (n_tokens % g.P) return fail(MLA_ERR_INVALID_ARG, "n_tokens (%d) must be a multiple of P (%d)", n_tokens, g.P);
  if (n_tokens / g.P > g.window)
    return fail(MLA_ERR_INVALID_ARG, "more frames (%d) than the window (%d)", n_tokens / g.P, g.window);
  if (geom->batch == 0 || n_tokens == 0) return MLA_OK;
  NEED_PTR(frame);
  NEED_PTR(gram);
  NEED_PTR(cache);
  NEED_PTR(cache_aux);
  const size_t need = key_norm_ws_bytes(d, geom->batch, n_tokens);
  if (need && (!workspace || workspace_bytes < need))
    return fail(MLA_ERR_WORKSPACE, "key norm workspace needs %zu bytes, got %zu", need, workspace_bytes);
  hipStream_t st = (hipStream_t)stream;
  return hip_status(launch_key_norm(d, g, geom->batch, n_tokens, frame, gram, cache, cache_aux, (float*)workspace, st),
                    st, "key inverse RMS");
}

mla_status mla_cache_rope_shift(const mla_dims* dims, const mla_geom* geom, void* stream, const int32_t* delta,
                                int32_t slot_begin, int32_t n_slots, void* cache, void* cache_aux) {
  Dims d;
  Geo g;
  CHECK(check_dims(dims, &d));
  CHECK(check_geom(geom, d, &g));
  if (slot_begin < 0 || n_slots < 0 || (int64_t)slot_begin + n_slots > g.capacity)
    return fail(MLA_ERR_INVALID_ARG, "slots [%d, %d + %d) must lie inside [0, capacity = %d)", slot_begin,
                slot_begin, n_slots, g.capacity);
  if (geom->batch == 0 || n_slots == 0) return MLA_OK;
  NEED_PTR(delta);
  NEED_PTR(cache);
  if (lowbit_cache(d)) NEED_PTR(cache_aux);
  hipStream_t st = (hipStream_t)stream;
  return hip_status(launch_rope_shift(d, g, geom->batch, delta, slot_begin, n_slots, cache, cache_aux, st), st,
                    "rotary key shift");
}

}  // extern "C"
