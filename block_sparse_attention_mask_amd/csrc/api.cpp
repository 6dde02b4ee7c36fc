// C-ABI entry points of libbsa (see include/bsa.h for the contract of each call).
// Host-side only: argument validation, workspace carving and kernel launches.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "bsa.h"
#include "launch.h"

namespace {

thread_local std::string g_err;

bsa_status fail(bsa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

bsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return BSA_OK;
  return fail(BSA_EHIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// compute units of the current device (cached per device)
int device_cus() {
  static thread_local int dev_cached = -1, cus_cached = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != dev_cached) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    dev_cached = dev;
    cus_cached = cus;
  }
  return cus_cached;
}

size_t dtype_size(bsa_dtype t) { return t == BSA_F32 ? 4 : (t == BSA_BF16 ? 2 : 1); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

bsa_status check_shape(const bsa_shape* s, bool need_valid_d = true) {
  if (!s) return fail(BSA_EINVAL, "shape is NULL");
  if (s->N != 64) return fail(BSA_EUNSUPPORTED, "block size N=%d (only 64 is supported)", s->N);
  if (s->B < 1 || s->H < 1) return fail(BSA_EINVAL, "B=%d, H=%d must be >= 1", s->B, s->H);
  if ((int64_t)s->B * s->H > 65535) return fail(BSA_EUNSUPPORTED, "B*H=%lld exceeds 65535", (long long)s->B * s->H);
  if (s->S < 64 || s->S % 64) return fail(BSA_EINVAL, "S=%d must be a positive multiple of 64", s->S);
  if (s->S_valid < 1 || s->S_valid > s->S) return fail(BSA_EINVAL, "S_valid=%d must be in [1, S=%d]", s->S_valid, s->S);
  if (need_valid_d && s->D != 64 && s->D != 128) return fail(BSA_EUNSUPPORTED, "head dim D=%d (64 or 128 supported)", s->D);
  return BSA_OK;
}

bsa_status check_tensor(const char* name, const bsa_tensor* t, const bsa_shape* s) {
  if (!t) return fail(BSA_EINVAL, "%s is NULL", name);
  if (!t->ptr) return fail(BSA_EINVAL, "%s->ptr is NULL", name);
  if (t->dtype != BSA_F32 && t->dtype != BSA_BF16 && t->dtype != BSA_FP8_E4M3FN)
    return fail(BSA_EINVAL, "%s has an unknown dtype %d", name, (int)t->dtype);
  if (!aligned16(t->ptr)) return fail(BSA_EINVAL, "%s->ptr is not 16-byte aligned", name);
  const int64_t es = (int64_t)dtype_size(t->dtype);
  if (t->sb < 0 || t->sh < 0 || t->ss < s->D)
    return fail(BSA_EINVAL, "%s strides (sb=%lld, sh=%lld, ss=%lld) invalid for D=%d", name, (long long)t->sb,
                (long long)t->sh, (long long)t->ss, s->D);
  if ((t->ss * es) % 16 || (t->sh * es) % 16 || (t->sb * es) % 16)
    return fail(BSA_EINVAL, "%s strides must be multiples of 16 bytes", name);
  return BSA_OK;
}

}  // namespace

extern "C" {

const char* bsa_last_error(void) { return g_err.c_str(); }
int bsa_abi_version(void) { return 13; }

int bsa_checked_build(void) {
#ifdef BSA_CHECKED
  return 1;
#else
  return 0;
#endif
}

unsigned bsa_check_flags(int clear) {
  const unsigned w[3] = {bsa::check_flags_attn(clear), bsa::check_flags_mask_ops(clear), bsa::check_flags_bwd(clear)};
  unsigned v = 0;
  for (unsigned x : w) {
    if (x == ~0u) return ~0u;
    v |= x;
  }
  return v;
}

// ---------------------------------------------------------------------------
size_t nabla_workspace_size(const bsa_shape* s) {
  if (!s || s->S <= 0 || s->D <= 0) return 0;
  const size_t nbp = ((size_t)s->S / 64 + 15) / 16 * 16, bh = (size_t)s->B * s->H;   // 16-block tiles
  return 2 * align256(bh * nbp * (size_t)s->D * sizeof(double));
}

// Near-threshold band of the cumulative-mass rule: flagged entries have an exclusive
// mass E with |E - (1 - thr)| <= NEAR_BAND, evaluated on the fixed-point mass E 2^60:
// floor((1 - thr - band) 2^60) <= E 2^60 <= floor((1 - thr + band) 2^60).
constexpr double NEAR_BAND = 1e-6;

static bsa::SelNear near_targets(uint8_t* flags, double thr) {
  bsa::SelNear n = {flags, 0, 0};
  if (!flags) return n;
  const double lo = 1.0 - thr - NEAR_BAND, hi = 1.0 - thr + NEAR_BAND;
  n.t_lo = lo > 0.0 ? (uint64_t)std::floor(std::ldexp(lo, 60)) : 0;
  n.t_hi = (uint64_t)std::floor(std::ldexp(hi, 60)) + 1;
  return n;
}

static bsa_status nabla_common(const bsa_tensor* q, const bsa_tensor* k, const bsa_shape* shape, double thr,
                               double scale, const uint8_t* or_mask, int64_t or_sb, int64_t or_sh,
                               uint8_t* mask_out, const bsa::Fp8Out* f8, void* ws, size_t ws_bytes,
                               bsa_stream_t stream, int topk = 0, bsa::StaRule sta = {0, 0, 0, 0, 0, 0},
                               const bsa::StaGeom* plane_geom = nullptr, uint8_t* plane = nullptr,
                               void* sta_ws = nullptr, const bsa::SelLists* lists = nullptr,
                               uint8_t* near_out = nullptr) {
  bsa_status st;
  if ((st = check_shape(shape)) != BSA_OK) return st;
  if ((st = check_tensor("q", q, shape)) != BSA_OK) return st;
  if ((st = check_tensor("k", k, shape)) != BSA_OK) return st;
  if (q->dtype != k->dtype || (q->dtype != BSA_BF16 && q->dtype != BSA_F32))
    return fail(BSA_EUNSUPPORTED, "nabla_build_mask needs q and k both bf16 or both f32");
  if (!(thr >= 0.0 && thr < 1.0)) return fail(BSA_EINVAL, "thr=%g must satisfy 0 <= thr < 1", thr);
  if (!std::isfinite(scale)) return fail(BSA_EINVAL, "scale is not finite");
  const int nb = shape->S / 64;
  if (nb > 2048) return fail(BSA_EUNSUPPORTED, "nb=%d exceeds 2048 blocks per sequence", nb);
  if (!mask_out) return fail(BSA_EINVAL, "mask_out is NULL");
  if (near_out && near_out == mask_out) return fail(BSA_EINVAL, "near_thr_out must not alias mask_out");
  if (or_mask && (or_sb < 0 || or_sh < 0)) return fail(BSA_EINVAL, "or_mask strides must be >= 0");
  const size_t need = nabla_workspace_size(shape);
  if (!ws || ws_bytes < need) return fail(BSA_EWORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  if ((uintptr_t)ws & 255) return fail(BSA_EINVAL, "workspace must be 256-byte aligned");
  if (scale <= 0.0) scale = 1.0 / std::sqrt((double)shape->D);

  const size_t bh = (size_t)shape->B * shape->H, nbp = ((size_t)nb + 15) / 16 * 16;
  double* qbar = (double*)ws;
  double* kbarT = (double*)((char*)ws + align256(bh * nbp * (size_t)shape->D * sizeof(double)));
  const int64_t qs[3] = {q->sb, q->sh, q->ss}, ks[3] = {k->sb, k->sh, k->ss};
  hipStream_t hs = (hipStream_t)stream;
  if (plane_geom) {   // a sliding-tile plane to build (after validation) and OR in
    hipError_t e = bsa::launch_sta(*plane_geom, (int32_t*)sta_ws, plane, hs);
    if (e != hipSuccess) return hip_status(e, "sta launch");
    or_mask = plane;
    or_sb = or_sh = 0;
  }
  const bsa::SelLists sl = lists ? *lists : bsa::SelLists{};
  hipError_t e = bsa::launch_pool(q->dtype == BSA_F32, shape->D, q->ptr, qs, k->ptr, ks, shape->B, shape->H, nb,
                                  qbar, kbarT, f8, hs);
  if (e != hipSuccess) return hip_status(e, "pool launch");
  const uint64_t T_fixed = (uint64_t)std::ldexp(1.0 - thr, 60);
  e = bsa::launch_select(qbar, kbarT, shape->B, shape->H, nb, shape->D, scale, T_fixed, topk, or_mask, or_sb,
                         or_sh, sta, mask_out, hs, sl, near_targets(topk ? nullptr : near_out, thr));
  return hip_status(e, "select launch");
}

bsa_status nabla_build_mask(const bsa_tensor* q, const bsa_tensor* k, const bsa_shape* shape, double thr,
                            double scale, const uint8_t* or_mask, int64_t or_sb, int64_t or_sh, uint8_t* mask_out,
                            uint8_t* near_thr_out, void* ws, size_t ws_bytes, bsa_stream_t stream) {
  g_err.clear();
  return nabla_common(q, k, shape, thr, scale, or_mask, or_sb, or_sh, mask_out, nullptr, ws, ws_bytes, stream, 0,
                      bsa::StaRule{0, 0, 0, 0, 0, 0}, nullptr, nullptr, nullptr, nullptr, near_thr_out);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The workspace of nabla_build_mask_noalloc: a static device array, one copy per GPU
// (held until the process ends). In host code `scratch` names a host-side stand-in, not
// device memory: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is handed to kernels.
static __device__ __align__(256) char scratch[BSA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// device address of the current device's scratch (looked up on the first call per device)
bsa_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(BSA_EUNSUPPORTED, "device %d: at most %d devices", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p || ((uintptr_t)p & 255)) return fail(BSA_EHIP, "scratch has no 256-byte aligned device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BSA_OK;
}
}  // namespace

extern "C" {

bsa_status nabla_build_mask_noalloc(const bsa_tensor* q, const bsa_tensor* k, const bsa_shape* shape, double thr,
                                    double scale, const uint8_t* or_mask, int64_t or_sb, int64_t or_sh,
                                    uint8_t* mask_out, uint8_t* near_thr_out, bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_shape(shape)) != BSA_OK) return st;
  const size_t need = nabla_workspace_size(shape);
  if (need > (size_t)BSA_NOALLOC_SCRATCH_BYTES)
    return fail(BSA_EUNSUPPORTED, "nabla_build_mask_noalloc: this shape needs %zu bytes of scratch, more than the %zu "
                "the library holds (split the heads over several calls, or use nabla_build_mask)",
                need, (size_t)BSA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != BSA_OK) return st;
  return nabla_common(q, k, shape, thr, scale, or_mask, or_sb, or_sh, mask_out, nullptr, ws,
                      (size_t)BSA_NOALLOC_SCRATCH_BYTES, stream, 0, bsa::StaRule{0, 0, 0, 0, 0, 0}, nullptr, nullptr,
                      nullptr, nullptr, near_thr_out);
}

static bsa_status check_fp8_out(const char* name, const bsa_tensor* c, const float* sc, const bsa_shape* shape) {
  bsa_status st;
  if ((st = check_tensor(name, c, shape)) != BSA_OK) return st;
  if (c->dtype != BSA_FP8_E4M3FN) return fail(BSA_EINVAL, "%s must have dtype fp8 e4m3fn", name);
  if (!sc || ((uintptr_t)sc & 3)) return fail(BSA_EINVAL, "%s scales are NULL or not 4-byte aligned", name);
  return BSA_OK;
}

static bsa::Fp8Out fp8_out(const bsa_tensor* c0, float* s0, const bsa_tensor* c1, float* s1) {
  bsa::Fp8Out f = {};
  const bsa_tensor* c[2] = {c0, c1};
  float* sc[2] = {s0, s1};
  for (int x = 0; x < 2; ++x) {
    if (!c[x]) continue;
    f.codes[x] = (uint8_t*)c[x]->ptr;
    f.sb[x] = c[x]->sb; f.sh[x] = c[x]->sh; f.ss[x] = c[x]->ss;
    f.scale[x] = sc[x];
  }
  return f;
}

bsa_status nabla_build_mask_topk(const bsa_tensor* q, const bsa_tensor* k, const bsa_shape* shape, int topk,
                                 double scale, const uint8_t* or_mask, int64_t or_sb, int64_t or_sh,
                                 uint8_t* mask_out, void* ws, size_t ws_bytes, bsa_stream_t stream) {
  g_err.clear();
  if (topk < 1) return fail(BSA_EINVAL, "topk=%d must be >= 1", topk);
  return nabla_common(q, k, shape, 0.0, scale, or_mask, or_sb, or_sh, mask_out, nullptr, ws, ws_bytes, stream, topk);
}

bsa_status nabla_build_mask_fp8(const bsa_tensor* q, const bsa_tensor* k, const bsa_shape* shape, double thr,
                                double scale, const uint8_t* or_mask, int64_t or_sb, int64_t or_sh,
                                uint8_t* mask_out, uint8_t* near_thr_out, const bsa_tensor* q8, float* q_scale,
                                const bsa_tensor* k8, float* k_scale, void* ws, size_t ws_bytes,
                                bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_shape(shape)) != BSA_OK) return st;
  if ((st = check_fp8_out("q8", q8, q_scale, shape)) != BSA_OK) return st;
  if ((st = check_fp8_out("k8", k8, k_scale, shape)) != BSA_OK) return st;
  const bsa::Fp8Out f8 = fp8_out(q8, q_scale, k8, k_scale);
  return nabla_common(q, k, shape, thr, scale, or_mask, or_sb, or_sh, mask_out, &f8, ws, ws_bytes, stream, 0,
                      bsa::StaRule{0, 0, 0, 0, 0, 0}, nullptr, nullptr, nullptr, nullptr, near_thr_out);
}

bsa_status quantize_fp8_blocks(const bsa_tensor* x, const bsa_shape* shape, const bsa_tensor* codes, float* scales,
                               bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_shape(shape)) != BSA_OK) return st;
  if ((st = check_tensor("x", x, shape)) != BSA_OK) return st;
  if (x->dtype != BSA_BF16 && x->dtype != BSA_F32) return fail(BSA_EUNSUPPORTED, "x must be bf16 or f32");
  if ((st = check_fp8_out("codes", codes, scales, shape)) != BSA_OK) return st;
  const bsa::Fp8Out f8 = fp8_out(codes, scales, nullptr, nullptr);
  const int64_t xs[3] = {x->sb, x->sh, x->ss};
  return hip_status(bsa::launch_pool(x->dtype == BSA_F32, shape->D, x->ptr, xs, x->ptr, xs, shape->B, shape->H,
                                     shape->S / 64, nullptr, nullptr, &f8, (hipStream_t)stream),
                    "quantize launch");
}

// incoherent processing: the signs (host bit words) and the key side's 1/D
static bsa_status fp8_rotation(bsa::Fp8Out* f, const uint64_t* sign_bits, const bsa_shape* shape, bool key0,
                               bool key1) {
  if (!sign_bits) return fail(BSA_EINVAL, "sign_bits is NULL");
  f->rot = 1;
  f->sbits[0] = sign_bits[0];
  f->sbits[1] = shape->D > 64 ? sign_bits[1] : 0ull;
  const float inv_d = 1.f / (float)shape->D;   // a power of two: exact
  f->smul[0] = key0 ? inv_d : 1.f;
  f->smul[1] = key1 ? inv_d : 1.f;
  return BSA_OK;
}

bsa_status quantize_fp8_blocks_rotated(const bsa_tensor* x, const bsa_shape* shape, const uint64_t* sign_bits,
                                       int key_side, const bsa_tensor* codes, float* scales, bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_shape(shape)) != BSA_OK) return st;
  if ((st = check_tensor("x", x, shape)) != BSA_OK) return st;
  if (x->dtype != BSA_BF16 && x->dtype != BSA_F32) return fail(BSA_EUNSUPPORTED, "x must be bf16 or f32");
  if ((st = check_fp8_out("codes", codes, scales, shape)) != BSA_OK) return st;
  if (key_side != 0 && key_side != 1) return fail(BSA_EINVAL, "key_side=%d (0 query side, 1 key side)", key_side);
  bsa::Fp8Out f8 = fp8_out(codes, scales, nullptr, nullptr);
  if ((st = fp8_rotation(&f8, sign_bits, shape, key_side == 1, false)) != BSA_OK) return st;
  const int64_t xs[3] = {x->sb, x->sh, x->ss};
  return hip_status(bsa::launch_pool(x->dtype == BSA_F32, shape->D, x->ptr, xs, x->ptr, xs, shape->B, shape->H,
                                     shape->S / 64, nullptr, nullptr, &f8, (hipStream_t)stream),
                    "quantize launch");
}

bsa_status nabla_build_mask_fp8_rotated(const bsa_tensor* q, const bsa_tensor* k, const bsa_shape* shape,
                                        double thr, double scale, const uint8_t* or_mask, int64_t or_sb,
                                        int64_t or_sh, uint8_t* mask_out, uint8_t* near_thr_out,
                                        const uint64_t* sign_bits, const bsa_tensor* q8, float* q_scale,
                                        const bsa_tensor* k8, float* k_scale, void* ws, size_t ws_bytes,
                                        bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_shape(shape)) != BSA_OK) return st;
  if ((st = check_fp8_out("q8", q8, q_scale, shape)) != BSA_OK) return st;
  if ((st = check_fp8_out("k8", k8, k_scale, shape)) != BSA_OK) return st;
  bsa::Fp8Out f8 = fp8_out(q8, q_scale, k8, k_scale);
  if ((st = fp8_rotation(&f8, sign_bits, shape, false, true)) != BSA_OK) return st;
  return nabla_common(q, k, shape, thr, scale, or_mask, or_sb, or_sh, mask_out, &f8, ws, ws_bytes, stream, 0,
                      bsa::StaRule{0, 0, 0, 0, 0, 0}, nullptr, nullptr, nullptr, nullptr, near_thr_out);
}

// ---------------------------------------------------------------------------
size_t sta_workspace_size(const bsa_shape* s) {
  if (!s || s->S <= 0) return 0;
  return align256((size_t)(s->S / 64) * (bsa::STA_MAX_TILES + 1) * sizeof(int32_t));
}

// sliding-tile arguments -> geometry (shape already checked)
static bsa_status sta_geom_from(const bsa_shape* shape, const int grid_thw[3], const int tile_thw[3],
                                const int win_thw[3], int token_order, const int order_tile_thw[3], bsa::StaGeom* g) {
  if (!grid_thw || !tile_thw || !win_thw) return fail(BSA_EINVAL, "grid/tile/window arrays must not be NULL");
  if (token_order != 0 && token_order != 1) return fail(BSA_EINVAL, "token_order=%d (0 row-major, 1 tile-major)", token_order);
  if (token_order == 1 && !order_tile_thw) return fail(BSA_EINVAL, "order_tile_thw is NULL for tile-major order");
  for (int x = 0; x < 3; ++x) {
    if (grid_thw[x] < 1 || tile_thw[x] < 1 || win_thw[x] < 1)
      return fail(BSA_EINVAL, "grid, tile and window sizes must be >= 1");
    if (win_thw[x] % 2 == 0) return fail(BSA_EINVAL, "window sizes must be odd (centred window), got %d", win_thw[x]);
    if ((grid_thw[x] + tile_thw[x] - 1) / tile_thw[x] > 1023)
      return fail(BSA_EUNSUPPORTED, "more than 1023 tiles along one axis");
    if (token_order == 1 && order_tile_thw[x] < 1) return fail(BSA_EINVAL, "order tile sizes must be >= 1");
  }
  const int64_t cells = (int64_t)grid_thw[0] * grid_thw[1] * grid_thw[2];
  if (cells != shape->S_valid)
    return fail(BSA_EINVAL, "T*H*W=%lld must equal S_valid=%d", (long long)cells, shape->S_valid);
  g->T = grid_thw[0]; g->H = grid_thw[1]; g->W = grid_thw[2];
  g->tt = tile_thw[0]; g->th = tile_thw[1]; g->tw = tile_thw[2];
  g->rt = win_thw[0] / 2; g->rh = win_thw[1] / 2; g->rw = win_thw[2] / 2;
  g->order = token_order;
  g->ot = token_order ? order_tile_thw[0] : 1;
  g->oh = token_order ? order_tile_thw[1] : 1;
  g->ow = token_order ? order_tile_thw[2] : 1;
  g->S_valid = shape->S_valid;
  g->nb = shape->S / 64;
  return BSA_OK;
}

bsa_status sta_build_mask(const bsa_shape* shape, const int grid_thw[3], const int tile_thw[3], const int win_thw[3],
                          int token_order, const int order_tile_thw[3], uint8_t* mask_out, void* ws, size_t ws_bytes,
                          bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_shape(shape, false)) != BSA_OK) return st;
  bsa::StaGeom g;
  if ((st = sta_geom_from(shape, grid_thw, tile_thw, win_thw, token_order, order_tile_thw, &g)) != BSA_OK) return st;
  if (!mask_out) return fail(BSA_EINVAL, "mask_out is NULL");
  const size_t need = sta_workspace_size(shape);
  if (!ws || ws_bytes < need) return fail(BSA_EWORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  return hip_status(bsa::launch_sta(g, (int32_t*)ws, mask_out, (hipStream_t)stream), "sta launch");
}

size_t nabla_sta_workspace_size(const bsa_shape* s) {
  if (!s || s->S <= 0 || s->D <= 0) return 0;
  const size_t nb = (size_t)s->S / 64;
  return nabla_workspace_size(s) + align256(nb * nb) + sta_workspace_size(s);
}

bsa_status nabla_build_mask_sta(const bsa_tensor* q, const bsa_tensor* k, const bsa_shape* shape, double thr,
                                double scale, const int grid_thw[3], const int tile_thw[3], const int win_thw[3],
                                int token_order, const int order_tile_thw[3], uint8_t* mask_out,
                                uint8_t* near_thr_out, void* ws, size_t ws_bytes, bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_shape(shape)) != BSA_OK) return st;
  bsa::StaGeom g;
  if ((st = sta_geom_from(shape, grid_thw, tile_thw, win_thw, token_order, order_tile_thw, &g)) != BSA_OK) return st;
  const size_t need = nabla_sta_workspace_size(shape);
  if (!ws || ws_bytes < need) return fail(BSA_EWORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  if ((uintptr_t)ws & 255) return fail(BSA_EINVAL, "workspace must be 256-byte aligned");
  const bsa::StaRule rule = bsa::sta_rule_of(g);
  const size_t nws = nabla_workspace_size(shape);
  if (rule.bpt)   // aligned layout: the rule is applied inside the select
    return nabla_common(q, k, shape, thr, scale, nullptr, 0, 0, mask_out, nullptr, ws, nws, stream, 0, rule, nullptr,
                        nullptr, nullptr, nullptr, near_thr_out);
  // otherwise the sliding-tile plane is built in the workspace and OR'd like any mask
  const size_t nb = (size_t)shape->S / 64;
  return nabla_common(q, k, shape, thr, scale, nullptr, 0, 0, mask_out, nullptr, ws, nws, stream, 0, rule, &g,
                      (uint8_t*)ws + nws, (char*)ws + nws + align256(nb * nb), nullptr, near_thr_out);
}

static int work_order_slots(const bsa_shape* s);

size_t nabla_lists_workspace_size(const bsa_shape* s) { return nabla_sta_workspace_size(s); }

bsa_status nabla_build_mask_lists(const bsa_tensor* q, const bsa_tensor* k, const bsa_shape* shape, double thr,
                                  double scale, const int grid_thw[3], const int tile_thw[3], const int win_thw[3],
                                  int token_order, const int order_tile_thw[3], uint8_t* mask_out,
                                  uint8_t* near_thr_out, int32_t* kv_len, int32_t* kv_idx, int32_t* work_order,
                                  void* ws, size_t ws_bytes, bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_shape(shape)) != BSA_OK) return st;
  const int nb = shape->S / 64;
  if (nb > bsa::SELR_MAX_NB)
    return fail(BSA_EUNSUPPORTED, "nb=%d: kv lists from the mask build need nb <= %d (use bsa_mask_to_csr)", nb,
                bsa::SELR_MAX_NB);
  if (!kv_len || !kv_idx) return fail(BSA_EINVAL, "kv_len / kv_idx is NULL");
  if ((int64_t)shape->B * shape->H * nb * nb >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "too many list entries");
  if (work_order && !work_order_slots(shape))
    return fail(BSA_EUNSUPPORTED, "this shape runs in the default order (attn_work_order_slots is 0)");
  const size_t need = nabla_lists_workspace_size(shape);
  if (!ws || ws_bytes < need) return fail(BSA_EWORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  if ((uintptr_t)ws & 255) return fail(BSA_EINVAL, "workspace must be 256-byte aligned");
  const size_t nws = nabla_workspace_size(shape);
  const bsa::SelLists lists = {kv_len, kv_idx};
  if (!grid_thw) {
    st = nabla_common(q, k, shape, thr, scale, nullptr, 0, 0, mask_out, nullptr, ws, nws, stream, 0,
                      bsa::StaRule{0, 0, 0, 0, 0, 0}, nullptr, nullptr, nullptr, &lists, near_thr_out);
  } else {
    bsa::StaGeom g;
    if ((st = sta_geom_from(shape, grid_thw, tile_thw, win_thw, token_order, order_tile_thw, &g)) != BSA_OK) return st;
    const bsa::StaRule rule = bsa::sta_rule_of(g);
    if (rule.bpt)   // aligned layout: the rule inside the selection
      st = nabla_common(q, k, shape, thr, scale, nullptr, 0, 0, mask_out, nullptr, ws, nws, stream, 0, rule, nullptr,
                        nullptr, nullptr, &lists, near_thr_out);
    else            // the sliding-tile plane built in the workspace first
      st = nabla_common(q, k, shape, thr, scale, nullptr, 0, 0, mask_out, nullptr, ws, nws, stream, 0, rule, &g,
                        (uint8_t*)ws + nws, (char*)ws + nws + align256((size_t)nb * nb), &lists, near_thr_out);
  }
  if (st != BSA_OK || !work_order) return st;
  // the work order from the list lengths: one small launch (a single workgroup)
  return hip_status(bsa::launch_pair_schedule_len(kv_len, shape->B * shape->H, nb, work_order, (hipStream_t)stream),
                    "work order launch");
}

// ---------------------------------------------------------------------------
bsa_status token_reorder(const bsa_tensor* x, const bsa_shape* shape, const int grid_thw[3], int order,
                         const int tile_thw[3], int inverse, const bsa_tensor* out, bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_shape(shape)) != BSA_OK) return st;
  if ((st = check_tensor("x", x, shape)) != BSA_OK) return st;
  if ((st = check_tensor("out", out, shape)) != BSA_OK) return st;
  if (x->dtype != out->dtype) return fail(BSA_EINVAL, "x and out must have the same dtype");
  if (x->ptr == out->ptr) return fail(BSA_EINVAL, "token_reorder does not work in place");
  if (!grid_thw) return fail(BSA_EINVAL, "grid_thw is NULL");
  if (order != BSA_ORDER_ROW && order != BSA_ORDER_TILE && order != BSA_ORDER_SPATIAL)
    return fail(BSA_EINVAL, "order=%d (0 row-major, 1 tile-major, 2 spatial-major)", order);
  if (order == BSA_ORDER_TILE && !tile_thw) return fail(BSA_EINVAL, "tile_thw is NULL for the tile-major order");
  for (int d = 0; d < 3; ++d) {
    if (grid_thw[d] < 1) return fail(BSA_EINVAL, "grid sizes must be >= 1");
    if (order == BSA_ORDER_TILE && tile_thw[d] < 1) return fail(BSA_EINVAL, "tile sizes must be >= 1");
  }
  if ((int64_t)grid_thw[0] * grid_thw[1] * grid_thw[2] != shape->S_valid)
    return fail(BSA_EINVAL, "T*H*W must equal S_valid=%d", shape->S_valid);
  bsa::ReorderGeom g;
  g.T = grid_thw[0]; g.H = grid_thw[1]; g.W = grid_thw[2];
  g.tt = order == BSA_ORDER_TILE ? tile_thw[0] : 1;
  g.th = order == BSA_ORDER_TILE ? tile_thw[1] : 1;
  g.tw = order == BSA_ORDER_TILE ? tile_thw[2] : 1;
  g.order = order;
  const int64_t es = (int64_t)dtype_size(x->dtype);
  const int64_t xs[3] = {x->sb * es, x->sh * es, x->ss * es}, os[3] = {out->sb * es, out->sh * es, out->ss * es};
  return hip_status(bsa::launch_token_reorder(x->ptr, xs, (void*)out->ptr, os, shape->B, shape->H, shape->S,
                                              (int)(shape->D * es), g, inverse != 0, (hipStream_t)stream),
                    "reorder launch");
}

// ---------------------------------------------------------------------------
bsa_status mask_or(uint8_t* dst, const uint8_t* a, int64_t n, const uint8_t* b, int64_t b_n, bsa_stream_t stream) {
  g_err.clear();
  if (!dst || !a || !b) return fail(BSA_EINVAL, "mask_or: NULL pointer");
  if (n < 0 || b_n < 1 || n % b_n) return fail(BSA_EINVAL, "mask_or: b_n=%lld must divide n=%lld", (long long)b_n, (long long)n);
  if (n == 0) return BSA_OK;
  return hip_status(bsa::launch_mask_or(dst, a, n, b, b_n, (hipStream_t)stream), "mask_or launch");
}

// ---------------------------------------------------------------------------
size_t csr_workspace_size(int B, int H, int nb) {
  if (B < 1 || H < 1 || nb < 1) return 0;
  const size_t rows = (size_t)B * H * nb;
  return align256((rows + rows / 1024 + 1) * sizeof(int32_t)) +   // counts + segment sums
         align256(bsa::lpt_rows_ws_ints((int)rows, nb + 1) * sizeof(int32_t));   // order
}

static bsa_status check_mask_args(const uint8_t* mask, int64_t sb, int64_t sh, int B, int H, int nb) {
  if (!mask) return fail(BSA_EINVAL, "mask is NULL");
  if (sb < 0 || sh < 0) return fail(BSA_EINVAL, "mask strides must be >= 0");
  if (B < 1 || H < 1 || nb < 1) return fail(BSA_EINVAL, "B, H, nb must be >= 1");
  if ((int64_t)B * H * nb >= (1ll << 31) / 2) return fail(BSA_EUNSUPPORTED, "too many rows");
  if ((int64_t)B * H * nb * nb >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "B*H*nb*nb must be < 2^31");
  return BSA_OK;
}

bsa_status bsa_mask_to_csr(const uint8_t* mask, int64_t mask_sb, int64_t mask_sh, int B, int H, int nb,
                           int32_t* row_ptr, int32_t* col_idx, int32_t* order, void* ws, size_t ws_bytes,
                           bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_mask_args(mask, mask_sb, mask_sh, B, H, nb)) != BSA_OK) return st;
  if (!row_ptr || !col_idx) return fail(BSA_EINVAL, "row_ptr / col_idx is NULL");
  const int rows = B * H * nb;
  if (order && bsa::lpt_rows_ws_ints(rows, nb + 1) == 0)
    return fail(BSA_EUNSUPPORTED, "order: nb=%d too large for the count sort (at most 16382)", nb);
  const size_t need = csr_workspace_size(B, H, nb);
  if (!ws || ws_bytes < need) return fail(BSA_EWORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  hipError_t e = bsa::launch_csr(mask, mask_sb, mask_sh, B, H, nb, row_ptr, col_idx, (int32_t*)ws, (hipStream_t)stream);
  if (e != hipSuccess || !order) return hip_status(e, "csr launch");
  int32_t* sort_ws = (int32_t*)((char*)ws + align256(((size_t)rows + rows / 1024 + 1) * sizeof(int32_t)));
  return hip_status(bsa::launch_lpt_rows(row_ptr, rows, nb, sort_ws, order, (hipStream_t)stream), "order launch");
}


bsa_status bsa_mask_to_csr_ordered(const uint8_t* mask, int64_t mask_sb, int64_t mask_sh, int B, int H, int nb,
                                   int32_t* row_ptr, int32_t* col_idx, int32_t* work_order, void* ws,
                                   size_t ws_bytes, bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_mask_args(mask, mask_sb, mask_sh, B, H, nb)) != BSA_OK) return st;
  if (!row_ptr || !col_idx || !work_order) return fail(BSA_EINVAL, "row_ptr / col_idx / work_order is NULL");
  const bsa_shape shape = {B, H, nb * 64, nb * 64, 128, 64};
  if (!work_order_slots(&shape)) return fail(BSA_EUNSUPPORTED, "this shape runs in the default order (0 slots)");
  const size_t need = csr_workspace_size(B, H, nb);
  if (!ws || ws_bytes < need) return fail(BSA_EWORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  return hip_status(bsa::launch_csr(mask, mask_sb, mask_sh, B, H, nb, row_ptr, col_idx, (int32_t*)ws,
                                    (hipStream_t)stream, work_order),
                    "csr launch");
}

// ---------------------------------------------------------------------------
static size_t split_bytes(const bsa_shape* s) {
  return align256((size_t)s->B * s->H * s->S * s->D * 2);
}

// Work order of the attention kernel. The longest-first order pays off when the work
// items make only a few rounds over the workgroup slots (3 per compute unit), where
// the tail is a large part of the run. With many rounds the default order does as well
// without the extra launch.
static int work_order_slots(const bsa_shape* s) {
  const int nb = s->S / 64, BH = s->B * s->H;
  if (!bsa::pair_schedule_fits(BH, nb)) return 0;
  const int64_t items = (int64_t)BH * ((nb + 1) / 2);
  if (items > 4 * 3 * (int64_t)device_cus()) return 0;
  return bsa::pair_schedule_slots(BH, nb);
}
// Shapes with more work items than the work order takes run in per-XCD ranges of the
// natural item order; from this many key blocks on, the attention kernel orders each
// head's items longest first (at the 14B shape 46.5 ms against 49.7 ms per launch; the
// order costs each workgroup a few microseconds, noise against items of ~2 ms).
constexpr int HEAD_ORDER_MIN_NB = 512;

// Width of the kv-chunked attention walk (0: rows walked whole), set by bsa_set_attn_kv_chunk.
// Whole rows are the default: at the 14B shape the chunked walk cuts the attention kernel's
// L2 misses twelvefold without changing its time, and its combine then adds ~12%.
static std::atomic<int> g_kv_chunk{0};
static int kv_chunk_of(const bsa_shape*) { return g_kv_chunk.load(); }

int bsa_set_attn_kv_chunk(int kv_chunk) { return g_kv_chunk.exchange(kv_chunk > 0 ? kv_chunk : 0); }

// Shapes run with each head's pairing offset (pairs of query blocks chosen for alike kv
// lists) from this many key blocks on, when they have no work order: at the 14B shape the
// offset one frame apart cuts the union steps by ~7%, at a cost of three small launches.
constexpr int PAIR_OFFSET_MIN_NB = 512;
static bool pairing_of(const bsa_shape* s) {
  return s->S / 64 >= PAIR_OFFSET_MIN_NB && work_order_slots(s) == 0;
}
static size_t pairing_bytes(const bsa_shape* s) {
  if (!pairing_of(s)) return 0;
  const int64_t BH = (int64_t)s->B * s->H;
  return align256((size_t)BH * 4) + bsa::pair_bits_ws(BH * (s->S / 64), s->S / 64);
}

size_t attn_csr_workspace_size(const bsa_shape* s, bsa_dtype qk_dtype) {
  if (!s || s->S <= 0 || s->D <= 0 || s->B < 1 || s->H < 1) return 0;
  const size_t split = qk_dtype == BSA_F32 ? 6 * split_bytes(s) : 0;   // hi/lo bf16 copies of f32 q, k, v
  return split + bsa::chunk_ws_bytes((int64_t)s->B * s->H * (s->S / 64), s->S / 64, s->D, kv_chunk_of(s)) +
         pairing_bytes(s);
}

size_t attn_workspace_size(const bsa_shape* s, bsa_dtype qk_dtype) {
  if (!s || s->S <= 0 || s->D <= 0) return 0;
  const size_t rows = (size_t)s->B * s->H * (s->S / 64), nb = s->S / 64;
  return align256((rows + 1) * 4) + align256(rows * nb * 4) + csr_workspace_size(s->B, s->H, (int)nb) +
         attn_csr_workspace_size(s, qk_dtype);
}

static bsa_status attn_common(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v, const bsa_shape* shape,
                              const int32_t* row_ptr, const int32_t* col_idx, const int32_t* work_order,
                              const float* q_scale, const float* k_scale, double scale, const bsa_tensor* o,
                              float* lse, void* ws, hipStream_t hs, const int32_t* row_len = nullptr) {
  bsa::AttnArgs a = {};
  bsa::AttnMode mode;
  if (q->dtype == BSA_BF16) mode = bsa::ATTN_BF16;
  else if (q->dtype == BSA_F32) mode = bsa::ATTN_SPLIT_F32;
  else mode = bsa::ATTN_FP8;
  if (scale <= 0.0) scale = 1.0 / std::sqrt((double)shape->D);
  a.q = q->ptr; a.q_sb = q->sb; a.q_sh = q->sh; a.q_ss = q->ss;
  a.k = k->ptr; a.k_sb = k->sb; a.k_sh = k->sh; a.k_ss = k->ss;
  a.v = v->ptr; a.v_sb = v->sb; a.v_sh = v->sh; a.v_ss = v->ss;
  a.o = (void*)o->ptr; a.o_sb = o->sb; a.o_sh = o->sh; a.o_ss = o->ss;
  a.lse = lse;
  a.row_ptr = row_ptr; a.col_idx = col_idx;
  a.row_len = row_len; a.row_stride = shape->S / 64;
  a.q_scale = q_scale; a.k_scale = k_scale;
  a.B = shape->B; a.H = shape->H; a.nb = shape->S / 64; a.S = shape->S; a.S_valid = shape->S_valid; a.D = shape->D;
  a.scale_log2 = (float)(scale * 1.4426950408889634);
  const int slots = work_order_slots(shape);
  if (slots) {
    if (!work_order) a.derive_order = 1;   // each workgroup derives its item from the list lengths
    a.pair_order = work_order;
    a.n_slots = slots;
  } else if (shape->S / 64 >= HEAD_ORDER_MIN_NB) {
    a.derive_order = 2;       // many rounds of long rows: longest first inside each head
  }
  void* split_ws = ws;
  char* wnext = (char*)ws + (mode == bsa::ATTN_SPLIT_F32 ? 6 * split_bytes(shape) : 0);
  if ((a.kv_chunk = kv_chunk_of(shape)) > 0) {
    a.pair_order = nullptr;
    a.derive_order = 0;
    bsa::chunk_ws_carve(a, wnext);
    wnext += bsa::chunk_ws_bytes((int64_t)a.B * a.H * a.nb, a.nb, a.D, a.kv_chunk);
  }
  if (pairing_of(shape)) {
    int32_t* pair_d = (int32_t*)wnext;
    uint64_t* bits = (uint64_t*)(wnext + align256((size_t)a.B * a.H * 4));
    hipError_t e = bsa::launch_pair_offsets(row_ptr, col_idx, row_len, a.row_stride, a.B * a.H, a.nb, bits, pair_d, hs);
    if (e != hipSuccess) return hip_status(e, "pairing offsets launch");
    a.pair_d = pair_d;
    a.row_bits = bits;
    a.nw = (a.nb + 63) / 64;
  }
  if (mode == bsa::ATTN_SPLIT_F32) {
    const size_t sb = split_bytes(shape);
    uint16_t* p[6];
    for (int x = 0; x < 6; ++x) p[x] = (uint16_t*)((char*)split_ws + x * sb);
    const bsa_tensor* src[3] = {q, k, v};
    for (int x = 0; x < 3; ++x) {
      hipError_t e = bsa::launch_split_f32((const float*)src[x]->ptr, src[x]->sb, src[x]->sh, src[x]->ss, shape->B,
                                           shape->H, shape->S, shape->D, p[2 * x], p[2 * x + 1], hs);
      if (e != hipSuccess) return hip_status(e, "split launch");
    }
    a.q = p[0]; a.q_lo = p[1]; a.k = p[2]; a.k_lo = p[3]; a.v = p[4]; a.v_lo = p[5];
  }
  return hip_status(bsa::launch_attn(a, mode, hs), "attention launch");
}

static bsa_status check_attn(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v, const bsa_shape* shape,
                             const float* q_scale, const float* k_scale, const bsa_tensor* o) {
  bsa_status st;
  if ((st = check_shape(shape)) != BSA_OK) return st;
  if ((st = check_tensor("q", q, shape)) != BSA_OK) return st;
  if ((st = check_tensor("k", k, shape)) != BSA_OK) return st;
  if ((st = check_tensor("v", v, shape)) != BSA_OK) return st;
  if ((st = check_tensor("o", o, shape)) != BSA_OK) return st;
  if (q->dtype != k->dtype) return fail(BSA_EINVAL, "q and k must have the same dtype");
  if (q->dtype == BSA_F32) {
    if (v->dtype != BSA_F32 || o->dtype != BSA_F32) return fail(BSA_EINVAL, "f32 q/k need f32 v and f32 o");
  } else {
    if (v->dtype != BSA_BF16 || o->dtype != BSA_BF16)
      return fail(BSA_EINVAL, "bf16/fp8 q/k need bf16 v and bf16 o");
  }
  if (q->dtype == BSA_FP8_E4M3FN) {
    if (!q_scale || !k_scale) return fail(BSA_EINVAL, "fp8 q/k need q_scale and k_scale");
  }
  if ((int64_t)shape->B * shape->H * (shape->S / 64) >= (1ll << 30)) return fail(BSA_EUNSUPPORTED, "too many rows");
  return BSA_OK;
}

bsa_status block_sparse_attn_fwd(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                 const bsa_shape* shape, const uint8_t* mask, int64_t mask_sb, int64_t mask_sh,
                                 const float* q_scale, const float* k_scale, double scale, const bsa_tensor* o,
                                 float* lse, void* ws, size_t ws_bytes, bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_attn(q, k, v, shape, q_scale, k_scale, o)) != BSA_OK) return st;
  if (!std::isfinite(scale)) return fail(BSA_EINVAL, "scale is not finite");
  const int nb = shape->S / 64;
  if ((st = check_mask_args(mask, mask_sb, mask_sh, shape->B, shape->H, nb)) != BSA_OK) return st;
  const size_t need = attn_workspace_size(shape, q->dtype);
  if (!ws || ws_bytes < need) return fail(BSA_EWORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  if ((uintptr_t)ws & 255) return fail(BSA_EINVAL, "workspace must be 256-byte aligned");
  const size_t rows = (size_t)shape->B * shape->H * nb;
  char* w = (char*)ws;
  int32_t* row_ptr = (int32_t*)w;
  w += align256((rows + 1) * 4);
  int32_t* col_idx = (int32_t*)w;
  w += align256(rows * nb * 4);
  int32_t* counts = (int32_t*)w;
  w += csr_workspace_size(shape->B, shape->H, nb);
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = bsa::launch_csr(mask, mask_sb, mask_sh, shape->B, shape->H, nb, row_ptr, col_idx, counts, hs);
  if (e != hipSuccess) return hip_status(e, "csr launch");
  return attn_common(q, k, v, shape, row_ptr, col_idx, nullptr, q_scale, k_scale, scale, o, lse, w, hs);
}

size_t attn_pair_workspace_size(const bsa_shape* s) {
  if (!s || s->S <= 0 || s->B < 1 || s->H < 1) return 0;
  const int64_t BH = (int64_t)s->B * s->H;
  return bsa::pair_bits_ws(BH * (s->S / 64), s->S / 64);
}

bsa_status attn_pair_offsets(const bsa_shape* shape, const int32_t* row_ptr, const int32_t* col_idx,
                             const int32_t* kv_len, int32_t* pair_d, void* ws, size_t ws_bytes, bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_shape(shape, false)) != BSA_OK) return st;
  if (!col_idx || !pair_d || (!row_ptr && !kv_len)) return fail(BSA_EINVAL, "col_idx / pair_d / lists are NULL");
  const int nb = shape->S / 64;
  if ((int64_t)shape->B * shape->H * nb * nb >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "too many list entries");
  const size_t need = attn_pair_workspace_size(shape);
  if (!ws || ws_bytes < need) return fail(BSA_EWORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  if ((uintptr_t)ws & 255) return fail(BSA_EINVAL, "workspace must be 256-byte aligned");
  return hip_status(bsa::launch_pair_offsets(row_ptr, col_idx, row_ptr ? nullptr : kv_len, nb, shape->B * shape->H, nb,
                                             (uint64_t*)ws, pair_d, (hipStream_t)stream),
                    "pairing offsets launch");
}

int attn_work_order_slots(const bsa_shape* shape) {
  g_err.clear();
  if (check_shape(shape, false) != BSA_OK) return -1;
  return work_order_slots(shape);
}

bsa_status attn_work_order(const bsa_shape* shape, const int32_t* row_ptr, int32_t* order, bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_shape(shape, false)) != BSA_OK) return st;
  if (!row_ptr || !order) return fail(BSA_EINVAL, "row_ptr / order is NULL");
  if (!work_order_slots(shape)) return fail(BSA_EUNSUPPORTED, "this shape runs in the default order (0 slots)");
  return hip_status(bsa::launch_pair_schedule(row_ptr, shape->B * shape->H, shape->S / 64, order, (hipStream_t)stream),
                    "work order launch");
}

bsa_status block_sparse_attn_fwd_csr(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                     const bsa_shape* shape, const int32_t* row_ptr, const int32_t* col_idx,
                                     const int32_t* work_order, const float* q_scale, const float* k_scale,
                                     double scale, const bsa_tensor* o, float* lse, void* ws, size_t ws_bytes,
                                     bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_attn(q, k, v, shape, q_scale, k_scale, o)) != BSA_OK) return st;
  if (!std::isfinite(scale)) return fail(BSA_EINVAL, "scale is not finite");
  if (!row_ptr || !col_idx) return fail(BSA_EINVAL, "row_ptr / col_idx is NULL");
  const size_t need = attn_csr_workspace_size(shape, q->dtype);
  if (need && (!ws || ws_bytes < need)) return fail(BSA_EWORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  if ((uintptr_t)ws & 255) return fail(BSA_EINVAL, "workspace must be 256-byte aligned");
  return attn_common(q, k, v, shape, row_ptr, col_idx, work_order, q_scale, k_scale, scale, o, lse, ws,
                     (hipStream_t)stream);
}

bsa_status block_sparse_attn_fwd_lists(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                       const bsa_shape* shape, const int32_t* kv_len, const int32_t* kv_idx,
                                       const int32_t* work_order, const float* q_scale, const float* k_scale,
                                       double scale, const bsa_tensor* o, float* lse, void* ws, size_t ws_bytes,
                                       bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_attn(q, k, v, shape, q_scale, k_scale, o)) != BSA_OK) return st;
  if (!std::isfinite(scale)) return fail(BSA_EINVAL, "scale is not finite");
  if (!kv_len || !kv_idx) return fail(BSA_EINVAL, "kv_len / kv_idx is NULL");
  const int64_t nb = shape->S / 64;
  if ((int64_t)shape->B * shape->H * nb * nb >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "too many list entries");
  const size_t need = attn_csr_workspace_size(shape, q->dtype);
  if (need && (!ws || ws_bytes < need)) return fail(BSA_EWORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  if ((uintptr_t)ws & 255) return fail(BSA_EINVAL, "workspace must be 256-byte aligned");
  return attn_common(q, k, v, shape, nullptr, kv_idx, work_order, q_scale, k_scale, scale, o, lse, ws,
                     (hipStream_t)stream, kv_len);
}

// ---------------------------------------------------------------------------
static size_t bwd_ld_bytes(const bsa_shape* s) { return align256(((size_t)s->B * s->H * s->S + 64) * 8); }

// The backward pairs blocks at each head's offset, for its key-block pairs (dK, dV) and its
// query-block pairs (dQ), from the same size on as the forward.
static size_t bwd_pairing_bytes(const bsa_shape* s) {
  const int nb = s->S / 64;
  if (nb < PAIR_OFFSET_MIN_NB) return 0;
  const int64_t BH = (int64_t)s->B * s->H;
  return 2 * (align256((size_t)BH * 4) + bsa::pair_bits_ws(BH * nb, nb));
}

size_t attn_bwd_workspace_size(const bsa_shape* s) {
  if (!s || s->S <= 0 || s->B < 1 || s->H < 1) return 0;
  const size_t nb = s->S / 64, rows = (size_t)s->B * s->H * nb;
  return bwd_ld_bytes(s) + align256(rows * nb) + 2 * (align256((rows + 1) * 4) + align256(rows * nb * 4)) +
         csr_workspace_size(s->B, s->H, (int)nb) + bwd_pairing_bytes(s);
}

bsa_status block_sparse_attn_bwd(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                 const bsa_tensor* o, const bsa_tensor* d_o, const float* lse,
                                 const bsa_shape* shape, const uint8_t* mask, int64_t mask_sb, int64_t mask_sh,
                                 double scale, const bsa_tensor* dq, const bsa_tensor* dk, const bsa_tensor* dv,
                                 void* ws, size_t ws_bytes, bsa_stream_t stream) {
  g_err.clear();
  bsa_status st;
  if ((st = check_shape(shape)) != BSA_OK) return st;
  const bsa_tensor* in[5] = {q, k, v, o, d_o};
  const char* in_name[5] = {"q", "k", "v", "o", "d_o"};
  for (int x = 0; x < 5; ++x) {
    if ((st = check_tensor(in_name[x], in[x], shape)) != BSA_OK) return st;
    if (in[x]->dtype != BSA_BF16) return fail(BSA_EUNSUPPORTED, "backward: %s must be bf16", in_name[x]);
  }
  const bsa_tensor* out[3] = {dq, dk, dv};
  const char* out_name[3] = {"dq", "dk", "dv"};
  for (int x = 0; x < 3; ++x) {
    if ((st = check_tensor(out_name[x], out[x], shape)) != BSA_OK) return st;
    if (out[x]->dtype != dq->dtype || (dq->dtype != BSA_BF16 && dq->dtype != BSA_F32))
      return fail(BSA_EINVAL, "backward: dq, dk, dv must all be bf16 or all f32");
  }
  if (!lse || ((uintptr_t)lse & 3)) return fail(BSA_EINVAL, "lse is NULL or not 4-byte aligned");
  if (!std::isfinite(scale)) return fail(BSA_EINVAL, "scale is not finite");
  const int nb = shape->S / 64;
  if ((st = check_mask_args(mask, mask_sb, mask_sh, shape->B, shape->H, nb)) != BSA_OK) return st;
  const size_t need = attn_bwd_workspace_size(shape);
  if (!ws || ws_bytes < need) return fail(BSA_EWORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  if ((uintptr_t)ws & 255) return fail(BSA_EINVAL, "workspace must be 256-byte aligned");
  if (scale <= 0.0) scale = 1.0 / std::sqrt((double)shape->D);

  bsa::BwdArgs a = {};
  a.derive_order = shape->S / 64 >= HEAD_ORDER_MIN_NB ? 1 : 0;   // as the forward, for long rows
  a.q = q->ptr; a.q_sb = q->sb; a.q_sh = q->sh; a.q_ss = q->ss;
  a.k = k->ptr; a.k_sb = k->sb; a.k_sh = k->sh; a.k_ss = k->ss;
  a.v = v->ptr; a.v_sb = v->sb; a.v_sh = v->sh; a.v_ss = v->ss;
  a.o = o->ptr; a.o_sb = o->sb; a.o_sh = o->sh; a.o_ss = o->ss;
  a.d_o = d_o->ptr; a.do_sb = d_o->sb; a.do_sh = d_o->sh; a.do_ss = d_o->ss;
  a.lse = lse;
  a.dq = (void*)dq->ptr; a.dq_sb = dq->sb; a.dq_sh = dq->sh; a.dq_ss = dq->ss;
  a.dk = (void*)dk->ptr; a.dk_sb = dk->sb; a.dk_sh = dk->sh; a.dk_ss = dk->ss;
  a.dv = (void*)dv->ptr; a.dv_sb = dv->sb; a.dv_sh = dv->sh; a.dv_ss = dv->ss;
  a.B = shape->B; a.H = shape->H; a.nb = nb; a.S = shape->S; a.S_valid = shape->S_valid; a.D = shape->D;
  a.scale = (float)scale;
  a.scale_log2 = (float)(scale * 1.4426950408889634);

  const size_t rows = (size_t)shape->B * shape->H * nb;
  char* w = (char*)ws;
  float2* ld = (float2*)w;
  w += bwd_ld_bytes(shape);
  uint8_t* mt = (uint8_t*)w;
  w += align256(rows * nb);
  int32_t* row_ptr = (int32_t*)w;
  w += align256((rows + 1) * 4);
  int32_t* col_idx = (int32_t*)w;
  w += align256(rows * nb * 4);
  int32_t* col_ptr = (int32_t*)w;
  w += align256((rows + 1) * 4);
  int32_t* row_idx = (int32_t*)w;
  w += align256(rows * nb * 4);
  int32_t* counts = (int32_t*)w;
  w += csr_workspace_size(shape->B, shape->H, nb);

  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = bsa::launch_bwd_prep(a, ld, hs);
  if (e != hipSuccess) return hip_status(e, "backward prep launch");
  e = bsa::launch_csr(mask, mask_sb, mask_sh, shape->B, shape->H, nb, row_ptr, col_idx, counts, hs);
  if (e != hipSuccess) return hip_status(e, "csr launch");
  e = bsa::launch_mask_transpose(mask, mask_sb, mask_sh, shape->B, shape->H, nb, mt, hs);
  if (e != hipSuccess) return hip_status(e, "mask transpose launch");
  e = bsa::launch_csr(mt, (int64_t)shape->H * nb * nb, (int64_t)nb * nb, shape->B, shape->H, nb, col_ptr, row_idx,
                      counts, hs);
  if (e != hipSuccess) return hip_status(e, "csr launch (transposed)");
  if (bwd_pairing_bytes(shape)) {
    const int BH = shape->B * shape->H;
    const size_t one = align256((size_t)BH * 4) + bsa::pair_bits_ws((int64_t)BH * nb, nb);
    int32_t* pk = (int32_t*)w;
    uint64_t* bk = (uint64_t*)(w + align256((size_t)BH * 4));
    int32_t* pq = (int32_t*)(w + one);
    uint64_t* bq = (uint64_t*)(w + one + align256((size_t)BH * 4));
    e = bsa::launch_pair_offsets(col_ptr, row_idx, nullptr, nb, BH, nb, bk, pk, hs);
    if (e != hipSuccess) return hip_status(e, "pairing offsets launch (key blocks)");
    e = bsa::launch_pair_offsets(row_ptr, col_idx, nullptr, nb, BH, nb, bq, pq, hs);
    if (e != hipSuccess) return hip_status(e, "pairing offsets launch (query blocks)");
    a.pair_dk = pk; a.bits_k = bk;
    a.pair_dq = pq; a.bits_q = bq;
    a.nw = (nb + 63) / 64;
  }
  return hip_status(bsa::launch_bwd(a, dq->dtype == BSA_F32, row_ptr, col_idx, col_ptr, row_idx, ld, hs),
                    "backward launch");
}

}  // extern "C"
