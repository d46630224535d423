// capi.hip — the extern "C" boundary of libbsa.so (declared in bsa.h).
//
// Every entry point validates its arguments on the host before any launch,
// leaves outputs untouched on failure, records a message in a thread-local
// string, and returns a bsa_status.  No exception crosses the boundary.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/bsa.h"
#include "bsa_internal.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return BSA_OK;
  return fail(BSA_EHIP, "%s: HIP error %d (%s)", what, static_cast<int>(e), hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool block_ok(int b) { return b == 64 || b == 128; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// runs f, turning any C++ exception into BSA_EHIP; the return type is f's
// (int for the calls, int64_t for the size queries)
template <typename F>
auto guarded(F&& f) -> decltype(f()) {
  try {
    return f();
  } catch (...) {
    return fail(BSA_EHIP, "internal error");
  }
}

// Shared validation of bsa_mask_params; fills the geometry.
int mask_geom(int32_t G, int32_t F, int32_t H, int32_t W, int32_t d, const bsa_mask_params* p,
              bsa::MaskGeom& m) {
  if (!p) return fail(BSA_EINVAL, "mask params pointer is NULL");
  if (G <= 0 || F <= 0 || H <= 0 || W <= 0) return fail(BSA_EINVAL, "G, F, H, W must be positive");
  const int64_t N = static_cast<int64_t>(F) * H * W;
  if (N >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "N = F*H*W must be < 2^31");
  if (!block_ok(p->Bq) || !block_ok(p->Bk)) return fail(BSA_EUNSUPPORTED, "Bq, Bk must be 64 or 128");
  if (p->score != 0 && p->score != 1) return fail(BSA_EINVAL, "score must be 0 (DOT) or 1 (COSINE)");
  if (p->rho_den <= 0 || p->rho_num < 0) return fail(BSA_EINVAL, "rho_num >= 0 and rho_den > 0 required");
  if (p->win_T >= 31) return fail(BSA_EINVAL, "win_T must be < 31");
  if (p->win_T >= 0 && p->win_r0 < 0) return fail(BSA_EINVAL, "win_r0 must be >= 0");
  m.G = G; m.F = F; m.H = H; m.W = W; m.d = d; m.N = N;
  m.Bq = p->Bq; m.Bk = p->Bk;
  m.nq = static_cast<int>((N + p->Bq - 1) / p->Bq);
  m.nk = static_cast<int>((N + p->Bk - 1) / p->Bk);
  if (m.nk > 8192) return fail(BSA_EUNSUPPORTED, "Nkv = %d exceeds 8192", m.nk);
  m.words = (m.nk + 63) / 64;
  m.score = p->score;
  int64_t k = (2ll * p->rho_num * m.nk + p->rho_den) / (2ll * p->rho_den);
  if (k > m.nk) k = m.nk;
  if (k < 1) k = 1;
  m.k = static_cast<int>(k);
  m.force_diag = p->force_diag != 0;
  m.win_T = p->win_T < 0 ? -1 : p->win_T;
  m.win_r0 = p->win_r0;
  if (static_cast<int64_t>(G) * m.nq >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "too many rows");
  return BSA_OK;
}

int64_t capacity_of(const bsa::MaskGeom& m) {
  int64_t per = m.k;
  if (m.force_diag) per += (m.Bq + m.Bk - 1) / m.Bk + 1;
  if (m.win_T >= 0) per = m.nk;
  if (per > m.nk) per = m.nk;
  return per * m.G * static_cast<int64_t>(m.nq);
}

// Validation of a natural-order output (the inverse reorder fused into the
// forward's epilogue); fills the output map.
int natural_out(const uint8_t* axis_order, int32_t F, int32_t H, int32_t W, int32_t G, int32_t d,
                int64_t sg, int64_t sn, bsa::OutMap& om, int32_t& N) {
  if (!axis_order) return fail(BSA_EINVAL, "axis_order is NULL");
  if (F <= 0 || H <= 0 || W <= 0) return fail(BSA_EINVAL, "F, H, W must be positive");
  const int64_t n64 = static_cast<int64_t>(F) * H * W;
  if (n64 >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "N = F*H*W must be < 2^31");
  if (sg < 0 || sn < 0 || sg % 8 || sn % 8)
    return fail(BSA_EINVAL, "natural strides must be non-negative multiples of 8");
  // rows (n, g) of d elements must not overlap: [N][G][d]-like or [G][N][d]-like strides
  const bool ng = sg >= d && sn >= static_cast<int64_t>(G) * sg;
  const bool gn = sn >= d && sg >= n64 * sn;
  if (!ng && !gn) return fail(BSA_EINVAL, "natural strides make output rows overlap");
  om.orders = axis_order;
  om.F = F; om.H = H; om.W = W;
  om.sg = sg; om.sn = sn;
  N = static_cast<int32_t>(n64);
  return BSA_OK;
}

// elem: bytes per K / V element (2 bf16, 1 int8).  The kernels address one
// head's K and V through 32-bit buffer resources, so N*d*elem must stay
// below 2^31.
int attn_common(const void* Q, const void* K, const void* V, const int32_t* row_ptr,
                const int32_t* col_idx, int64_t col_len, int32_t mask_G, void* Op, int32_t G,
                int32_t N, int32_t d, int32_t Bq, int32_t Bk, int elem) {
  if (!Q || !K || !V || !row_ptr || !Op) return fail(BSA_EINVAL, "NULL tensor pointer");
  if (col_len < 0 || (col_len > 0 && !col_idx)) return fail(BSA_EINVAL, "bad col_idx / col_len");
  if (G <= 0 || N <= 0) return fail(BSA_EINVAL, "G and N must be positive");
  if (d != 64 && d != 128) return fail(BSA_EUNSUPPORTED, "d must be 64 or 128 (got %d)", d);
  if (!block_ok(Bq) || !block_ok(Bk)) return fail(BSA_EUNSUPPORTED, "Bq, Bk must be 64 or 128");
  if (mask_G <= 0 || mask_G > G) return fail(BSA_EINVAL, "mask_G must be in [1, G]");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(Op, 16))
    return fail(BSA_EINVAL, "tensor pointers must be 16-byte aligned");
  const int64_t nq = (static_cast<int64_t>(N) + Bq - 1) / Bq;
  if (static_cast<int64_t>(G) * nq >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "grid too large");
  if (static_cast<int64_t>(G) * N * d >= (1ll << 40)) return fail(BSA_EUNSUPPORTED, "tensor too large");
  if (static_cast<int64_t>(N) * d * elem >= (1ll << 31))
    return fail(BSA_EUNSUPPORTED, "one head's K/V must be < 2^31 bytes (N*d*%d = %lld)", elem,
                static_cast<long long>(N) * d * elem);
  return BSA_OK;
}

}  // namespace

extern "C" {

int32_t bsa_abi_version(void) { return BSA_ABI_VERSION; }

const char* bsa_last_error(void) { return g_err.c_str(); }

int bsa_permute(int32_t direction, const void* src, int32_t src_dt, void* dst, int32_t dst_dt,
                int64_t nat_stride_g, int64_t nat_stride_n, int32_t G, int32_t F, int32_t H,
                int32_t W, int32_t d, const uint8_t* axis_order, void* stream) {
  return guarded([&]() -> int {
    if (direction != 0 && direction != 1) return fail(BSA_EINVAL, "direction must be 0 or 1");
    if (!src || !dst || !axis_order) return fail(BSA_EINVAL, "NULL pointer");
    if ((src_dt != BSA_F32 && src_dt != BSA_BF16) || (dst_dt != BSA_F32 && dst_dt != BSA_BF16))
      return fail(BSA_EUNSUPPORTED, "permute dtypes must be F32 or BF16");
    if (G <= 0 || F <= 0 || H <= 0 || W <= 0 || d <= 0) return fail(BSA_EINVAL, "sizes must be positive");
    if (d % 8 != 0) return fail(BSA_EINVAL, "d must be a multiple of 8");
    if (G > 65535) return fail(BSA_EUNSUPPORTED, "G must be <= 65535");
    if (nat_stride_g < 0 || nat_stride_n < 0 || nat_stride_g % 8 || nat_stride_n % 8)
      return fail(BSA_EINVAL, "natural strides must be non-negative multiples of 8");
    const int64_t N = static_cast<int64_t>(F) * H * W;
    if (N >= (1ll << 31) || N * (d / 8) >= (1ll << 31))
      return fail(BSA_EUNSUPPORTED, "N*d/8 must be < 2^31");
    if (N * G * d >= (1ll << 40)) return fail(BSA_EUNSUPPORTED, "tensor too large");
    if (!aligned(src, 16) || !aligned(dst, 16)) return fail(BSA_EINVAL, "pointers must be 16-byte aligned");
    return hip_status(bsa::launch_permute(direction, src, src_dt, dst, dst_dt, nat_stride_g,
                                          nat_stride_n, G, F, H, W, d, axis_order, as_stream(stream)),
                      "bsa_permute");
  });
}

int64_t bsa_mask_capacity(int32_t G, int32_t F, int32_t H, int32_t W, const bsa_mask_params* p_host) {
  return guarded([&]() -> int64_t {
    bsa::MaskGeom m{};
    const int rc = mask_geom(G, F, H, W, 64, p_host, m);
    if (rc != BSA_OK) return rc;
    return capacity_of(m);
  });
}

int64_t bsa_mask_workspace(int32_t G, int32_t F, int32_t H, int32_t W, int32_t d,
                           const bsa_mask_params* p_host) {
  return guarded([&]() -> int64_t {
    if (d != 64 && d != 128) return fail(BSA_EUNSUPPORTED, "d must be 64 or 128");
    bsa::MaskGeom m{};
    const int rc = mask_geom(G, F, H, W, d, p_host, m);
    if (rc != BSA_OK) return rc;
    return static_cast<int64_t>(bsa::mask_workspace_layout(m).total);
  });
}

int bsa_build_mask(const void* Qp, const void* Kp, int32_t dt, int32_t G, int32_t F, int32_t H,
                   int32_t W, int32_t d, const uint8_t* axis_order, const bsa_mask_params* p_host,
                   int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, int32_t* nnz,
                   void* workspace, int64_t ws_bytes, void* stream) {
  return guarded([&]() -> int {
    if (!Qp || !Kp || !axis_order || !row_ptr || !col_idx || !nnz || !workspace)
      return fail(BSA_EINVAL, "NULL pointer");
    if (dt != BSA_BF16) return fail(BSA_EUNSUPPORTED, "build_mask takes bf16 Qp/Kp");
    if (d != 64 && d != 128) return fail(BSA_EUNSUPPORTED, "d must be 64 or 128");
    bsa::MaskGeom m{};
    const int rc = mask_geom(G, F, H, W, d, p_host, m);
    if (rc != BSA_OK) return rc;
    const int64_t cap = capacity_of(m);
    if (cap >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "mask capacity %lld exceeds int32", (long long)cap);
    if (col_capacity < cap)
      return fail(BSA_ECAPACITY, "col_capacity %lld < required bound %lld", (long long)col_capacity,
                  (long long)cap);
    const int64_t need = static_cast<int64_t>(bsa::mask_workspace_layout(m).total);
    if (ws_bytes < need)
      return fail(BSA_ECAPACITY, "workspace %lld bytes < required %lld", (long long)ws_bytes, (long long)need);
    if (!aligned(workspace, 256)) return fail(BSA_EINVAL, "workspace must be 256-byte aligned");
    if (!aligned(Qp, 16) || !aligned(Kp, 16)) return fail(BSA_EINVAL, "Qp/Kp must be 16-byte aligned");
    return hip_status(bsa::launch_build_mask(m, static_cast<const uint16_t*>(Qp),
                                             static_cast<const uint16_t*>(Kp), axis_order, row_ptr,
                                             col_idx, col_capacity, nnz, static_cast<char*>(workspace),
                                             as_stream(stream)),
                      "bsa_build_mask");
  });
}

int bsa_permute_pool(const void* src, int32_t src_dt, void* dst, int64_t nat_stride_g,
                     int64_t nat_stride_n, int32_t G, int32_t F, int32_t H, int32_t W, int32_t d,
                     const uint8_t* axis_order, int32_t B, float* sums, int8_t* xq, float* scale,
                     void* stream) {
  return guarded([&]() -> int {
    if (!src || !axis_order) return fail(BSA_EINVAL, "NULL pointer");
    if (!dst && !sums && !xq) return fail(BSA_EINVAL, "no output requested");
    if ((xq == nullptr) != (scale == nullptr))
      return fail(BSA_EINVAL, "xq and scale are given together or not at all");
    if (src_dt != BSA_F32 && src_dt != BSA_BF16) return fail(BSA_EUNSUPPORTED, "src must be F32 or BF16");
    if (G <= 0 || F <= 0 || H <= 0 || W <= 0) return fail(BSA_EINVAL, "sizes must be positive");
    if (d != 64 && d != 128) return fail(BSA_EUNSUPPORTED, "d must be 64 or 128");
    if (!block_ok(B)) return fail(BSA_EUNSUPPORTED, "B must be 64 or 128");
    if (G > 65535) return fail(BSA_EUNSUPPORTED, "G must be <= 65535");
    if (nat_stride_g < 0 || nat_stride_n < 0 || nat_stride_g % 8 || nat_stride_n % 8)
      return fail(BSA_EINVAL, "natural strides must be non-negative multiples of 8");
    const int64_t N = static_cast<int64_t>(F) * H * W;
    if (N >= (1ll << 31) || N * d >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "N*d must be < 2^31");
    if ((N + B - 1) / B > 65535 * 64) return fail(BSA_EUNSUPPORTED, "too many blocks");
    if (!aligned(src, 16) || (dst && !aligned(dst, 16)))
      return fail(BSA_EINVAL, "src/dst must be 16-byte aligned");
    if (sums && !aligned(sums, 4)) return fail(BSA_EINVAL, "sums must be 4-byte aligned");
    if (xq && !aligned(xq, 8)) return fail(BSA_EINVAL, "xq must be 8-byte aligned");
    return hip_status(bsa::launch_permute_pool(src, src_dt, static_cast<uint16_t*>(dst), nat_stride_g,
                                               nat_stride_n, G, F, H, W, d, axis_order, B, sums, xq,
                                               scale, as_stream(stream)),
                      "bsa_permute_pool");
  });
}

int bsa_build_mask_pooled(const float* sums_q, const float* sums_k, int32_t G, int32_t F, int32_t H,
                          int32_t W, int32_t d, const uint8_t* axis_order,
                          const bsa_mask_params* p_host, int32_t* row_ptr, int32_t* col_idx,
                          int64_t col_capacity, int32_t* nnz, void* workspace, int64_t ws_bytes,
                          void* stream) {
  return guarded([&]() -> int {
    if (!sums_q || !sums_k || !axis_order || !row_ptr || !col_idx || !nnz || !workspace)
      return fail(BSA_EINVAL, "NULL pointer");
    if (d != 64 && d != 128) return fail(BSA_EUNSUPPORTED, "d must be 64 or 128");
    bsa::MaskGeom m{};
    const int rc = mask_geom(G, F, H, W, d, p_host, m);
    if (rc != BSA_OK) return rc;
    const int64_t cap = capacity_of(m);
    if (cap >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "mask capacity %lld exceeds int32", (long long)cap);
    if (col_capacity < cap)
      return fail(BSA_ECAPACITY, "col_capacity %lld < required bound %lld", (long long)col_capacity,
                  (long long)cap);
    const int64_t need = static_cast<int64_t>(bsa::mask_workspace_layout(m).total);
    if (ws_bytes < need)
      return fail(BSA_ECAPACITY, "workspace %lld bytes < required %lld", (long long)ws_bytes, (long long)need);
    if (!aligned(workspace, 256)) return fail(BSA_EINVAL, "workspace must be 256-byte aligned");
    return hip_status(bsa::launch_build_mask_pooled(m, sums_q, sums_k, axis_order, row_ptr, col_idx,
                                                    col_capacity, nnz, static_cast<char*>(workspace),
                                                    as_stream(stream)),
                      "bsa_build_mask_pooled");
  });
}

int bsa_build_mask_pooled_noalloc(const float* sums_q, const float* sums_k, int32_t G, int32_t F,
                                  int32_t H, int32_t W, int32_t d, const uint8_t* axis_order,
                                  const bsa_mask_params* p_host, int32_t* row_ptr, int32_t* col_idx,
                                  int64_t col_capacity, int32_t* nnz, void* stream) {
  return guarded([&]() -> int {
    if (!sums_q || !sums_k || !axis_order || !row_ptr || !col_idx || !nnz)
      return fail(BSA_EINVAL, "NULL pointer");
    if (d != 64 && d != 128) return fail(BSA_EUNSUPPORTED, "d must be 64 or 128");
    bsa::MaskGeom m{};
    const int rc = mask_geom(G, F, H, W, d, p_host, m);
    if (rc != BSA_OK) return rc;
    const int64_t cap = capacity_of(m);
    if (cap >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "mask capacity %lld exceeds int32", (long long)cap);
    if (col_capacity < cap)
      return fail(BSA_ECAPACITY, "col_capacity %lld < required bound %lld", (long long)col_capacity,
                  (long long)cap);
    const size_t need = bsa::mask_workspace_layout(m).total;
    if (need > bsa::mask_scratch_bytes())
      return fail(BSA_ECAPACITY,
                  "this mask build needs %zu bytes of scratch; the fixed scratch holds %zu "
                  "(use bsa_build_mask_pooled with a caller workspace)",
                  need, bsa::mask_scratch_bytes());
    void* ws = nullptr;
    const int st = hip_status(bsa::mask_scratch_ptr(&ws), "bsa_build_mask_pooled_noalloc: scratch address");
    if (st != BSA_OK) return st;
    return hip_status(bsa::launch_build_mask_pooled(m, sums_q, sums_k, axis_order, row_ptr, col_idx,
                                                    col_capacity, nnz, static_cast<char*>(ws),
                                                    as_stream(stream)),
                      "bsa_build_mask_pooled_noalloc");
  });
}

int64_t bsa_order_workspace(int32_t G, int32_t F, int32_t H, int32_t W, int32_t B) {
  if (G <= 0 || F <= 0 || H <= 0 || W <= 0 || !block_ok(B)) return -1;
  const int64_t N = static_cast<int64_t>(F) * H * W;
  if (N >= (1ll << 31)) return -1;
  return static_cast<int64_t>(bsa::order_workspace_bytes(G, static_cast<int>(N), B));
}

int bsa_order_scores(const void* src, int32_t src_dt, int64_t nat_stride_g, int64_t nat_stride_n,
                     int32_t G, int32_t F, int32_t H, int32_t W, int32_t d, int32_t B, float* scores,
                     void* workspace, int64_t ws_bytes, void* stream) {
  return guarded([&]() -> int {
    if (!src || !scores || !workspace) return fail(BSA_EINVAL, "NULL pointer");
    if (src_dt != BSA_F32 && src_dt != BSA_BF16) return fail(BSA_EUNSUPPORTED, "src must be F32 or BF16");
    if (G <= 0 || F <= 0 || H <= 0 || W <= 0) return fail(BSA_EINVAL, "sizes must be positive");
    if (d != 64 && d != 128) return fail(BSA_EUNSUPPORTED, "d must be 64 or 128");
    if (!block_ok(B)) return fail(BSA_EUNSUPPORTED, "B must be 64 or 128");
    if (G > 65535) return fail(BSA_EUNSUPPORTED, "G must be <= 65535");
    if (nat_stride_g < 0 || nat_stride_n < 0 || nat_stride_g % 8 || nat_stride_n % 8)
      return fail(BSA_EINVAL, "natural strides must be non-negative multiples of 8");
    const int64_t N = static_cast<int64_t>(F) * H * W;
    if (N >= (1ll << 31) || N * d >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "N*d must be < 2^31");
    if (!aligned(src, 16)) return fail(BSA_EINVAL, "src must be 16-byte aligned");
    if (!aligned(workspace, 4)) return fail(BSA_EINVAL, "workspace must be 4-byte aligned");
    const int64_t need = static_cast<int64_t>(bsa::order_workspace_bytes(G, static_cast<int>(N), B));
    if (ws_bytes < need)
      return fail(BSA_ECAPACITY, "workspace %lld bytes < required %lld", (long long)ws_bytes, (long long)need);
    return hip_status(bsa::launch_order_scores(src, src_dt, nat_stride_g, nat_stride_n, G, F, H, W, d,
                                               B, scores, workspace, as_stream(stream)),
                      "bsa_order_scores");
  });
}

int bsa_select_orders(const float* scores_a, const float* scores_b, int32_t G, uint8_t* axis_order,
                      void* stream) {
  return guarded([&]() -> int {
    if (!scores_a || !axis_order) return fail(BSA_EINVAL, "NULL pointer");
    if (G <= 0) return fail(BSA_EINVAL, "G must be positive");
    return hip_status(bsa::launch_select_orders(scores_a, scores_b, G, axis_order, as_stream(stream)),
                      "bsa_select_orders");
  });
}

int bsa_quantize_int8(const void* Xp, int8_t* Xq, float* scale, int32_t G, int32_t N, int32_t d,
                      int32_t B, void* stream) {
  return guarded([&]() -> int {
    if (!Xp || !Xq || !scale) return fail(BSA_EINVAL, "NULL pointer");
    if (G <= 0 || N <= 0 || d <= 0) return fail(BSA_EINVAL, "sizes must be positive");
    if (!block_ok(B)) return fail(BSA_EUNSUPPORTED, "B must be 64 or 128");
    if (d % 8 != 0 || d > 128) return fail(BSA_EUNSUPPORTED, "d must be a multiple of 8, <= 128");
    if (G > 65535) return fail(BSA_EUNSUPPORTED, "G must be <= 65535");
    if (!aligned(Xp, 16) || !aligned(Xq, 8)) return fail(BSA_EINVAL, "Xp 16-byte, Xq 8-byte alignment required");
    return hip_status(bsa::launch_quantize_int8(static_cast<const uint16_t*>(Xp), Xq, scale, G, N, d,
                                                B, as_stream(stream)),
                      "bsa_quantize_int8");
  });
}

int bsa_forward(const void* Qp, const void* Kp, const void* Vp, const int32_t* row_ptr,
                const int32_t* col_idx, int64_t col_len, int32_t mask_G, void* Op, float* lse,
                int32_t G, int32_t N, int32_t d, int32_t Bq, int32_t Bk, float sm_scale,
                void* stream) {
  return guarded([&]() -> int {
    const int rc = attn_common(Qp, Kp, Vp, row_ptr, col_idx, col_len, mask_G, Op, G, N, d, Bq, Bk, 2);
    if (rc != BSA_OK) return rc;
    if (!std::isfinite(sm_scale)) return fail(BSA_EINVAL, "sm_scale must be finite");
    bsa::AttnArgs a{};
    a.Q = Qp; a.K = Kp; a.V = Vp;
    a.row_ptr = row_ptr; a.col_idx = col_idx; a.col_len = col_len; a.mask_G = mask_G;
    a.O = static_cast<uint16_t*>(Op); a.lse = lse;
    a.G = G; a.N = N; a.d = d; a.Bq = Bq; a.Bk = Bk; a.sm_scale = sm_scale;
    return hip_status(bsa::launch_forward_bf16(a, as_stream(stream)), "bsa_forward");
  });
}

int bsa_forward_int8(const int8_t* Qq, const float* sQ, const int8_t* Kq, const float* sK,
                     const int8_t* Vq, const float* sV, const int32_t* row_ptr,
                     const int32_t* col_idx, int64_t col_len, int32_t mask_G, void* Op, float* lse,
                     int32_t G, int32_t N, int32_t d, int32_t Bq, int32_t Bk, float sm_scale,
                     void* stream) {
  return guarded([&]() -> int {
    const int rc = attn_common(Qq, Kq, Vq, row_ptr, col_idx, col_len, mask_G, Op, G, N, d, Bq, Bk, 1);
    if (rc != BSA_OK) return rc;
    if (!sQ || !sK || !sV) return fail(BSA_EINVAL, "NULL scale pointer");
    if (!std::isfinite(sm_scale)) return fail(BSA_EINVAL, "sm_scale must be finite");
    bsa::AttnArgs a{};
    a.Q = Qq; a.K = Kq; a.V = Vq; a.sQ = sQ; a.sK = sK; a.sV = sV;
    a.row_ptr = row_ptr; a.col_idx = col_idx; a.col_len = col_len; a.mask_G = mask_G;
    a.O = static_cast<uint16_t*>(Op); a.lse = lse;
    a.G = G; a.N = N; a.d = d; a.Bq = Bq; a.Bk = Bk; a.sm_scale = sm_scale;
    return hip_status(bsa::launch_forward_int8(a, as_stream(stream)), "bsa_forward_int8");
  });
}

int bsa_debug_int8_qk(const int8_t* Qq, const int8_t* Kq, int32_t G, int32_t N, int32_t d,
                      int32_t Bq, int32_t Bk, const int32_t* gij, int32_t n, int32_t* S,
                      void* stream) {
  return guarded([&]() -> int {
    if (!Qq || !Kq || !gij || !S) return fail(BSA_EINVAL, "NULL pointer");
    if (G <= 0 || N <= 0 || n <= 0) return fail(BSA_EINVAL, "G, N, n must be positive");
    if (d != 64 && d != 128) return fail(BSA_EUNSUPPORTED, "d must be 64 or 128");
    if (!block_ok(Bq) || !block_ok(Bk)) return fail(BSA_EUNSUPPORTED, "Bq, Bk must be 64 or 128");
    if (!aligned(Qq, 16) || !aligned(Kq, 16)) return fail(BSA_EINVAL, "16-byte alignment required");
    return hip_status(bsa::launch_debug_int8_qk(Qq, Kq, G, N, d, Bq, Bk, gij, n, S, as_stream(stream)),
                      "bsa_debug_int8_qk");
  });
}

int bsa_debug_int8_pv(const int8_t* P8, const int8_t* Vq, int32_t G, int32_t N, int32_t d,
                      int32_t Bq, int32_t Bk, const int32_t* gj, int32_t n, int32_t* OV,
                      void* stream) {
  return guarded([&]() -> int {
    if (!P8 || !Vq || !gj || !OV) return fail(BSA_EINVAL, "NULL pointer");
    if (G <= 0 || N <= 0 || n <= 0) return fail(BSA_EINVAL, "G, N, n must be positive");
    if (d != 64 && d != 128) return fail(BSA_EUNSUPPORTED, "d must be 64 or 128");
    if (!block_ok(Bq) || !block_ok(Bk)) return fail(BSA_EUNSUPPORTED, "Bq, Bk must be 64 or 128");
    if (!aligned(Vq, 16)) return fail(BSA_EINVAL, "16-byte alignment required");
    return hip_status(bsa::launch_debug_int8_pv(P8, Vq, G, N, d, Bq, Bk, gj, n, OV, as_stream(stream)),
                      "bsa_debug_int8_pv");
  });
}


// ---- offline calibration and static masks ---------------------------------

int bsa_attn_block_stats(const void* Qp, const void* Kp, int32_t G, int32_t N, int32_t d, int32_t B,
                         float sm_scale, float eps, int32_t* cnt, float* bsum, float* bmax,
                         void* stream) {
  return guarded([&]() -> int {
    if (!Qp || !Kp || !cnt || !bsum || !bmax) return fail(BSA_EINVAL, "NULL pointer");
    if (G <= 0 || N <= 0) return fail(BSA_EINVAL, "G and N must be positive");
    if (d != 64 && d != 128) return fail(BSA_EUNSUPPORTED, "d must be 64 or 128");
    if (!block_ok(B)) return fail(BSA_EUNSUPPORTED, "B must be 64 or 128");
    if (G > 65535) return fail(BSA_EUNSUPPORTED, "G must be <= 65535");
    if (static_cast<int64_t>(N) * d >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "N*d must be < 2^31");
    if (!std::isfinite(sm_scale)) return fail(BSA_EINVAL, "sm_scale must be finite");
    if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(BSA_EINVAL, "eps must be positive and finite");
    if (!aligned(Qp, 16) || !aligned(Kp, 16)) return fail(BSA_EINVAL, "Qp and Kp must be 16-byte aligned");
    if (!aligned(cnt, 4) || !aligned(bsum, 4) || !aligned(bmax, 4))
      return fail(BSA_EINVAL, "outputs must be 4-byte aligned");
    const float sc = sm_scale > 0.0f ? sm_scale : 1.0f / std::sqrt(static_cast<float>(d));
    return hip_status(bsa::launch_block_stats(static_cast<const uint16_t*>(Qp),
                                              static_cast<const uint16_t*>(Kp), G, N, d, B, sc, eps,
                                              cnt, bsum, bmax, as_stream(stream)),
                      "bsa_attn_block_stats");
  });
}

int bsa_paro_metric(const int32_t* cnt, const float* bsum, const float* bmax, int32_t G, int32_t N,
                    int32_t B, int32_t sigma_num, int32_t sigma_den, float alpha, int32_t order,
                    float* stats, void* stream) {
  return guarded([&]() -> int {
    if (!cnt || !bsum || !bmax || !stats) return fail(BSA_EINVAL, "NULL pointer");
    if (G <= 0 || N <= 0) return fail(BSA_EINVAL, "G and N must be positive");
    if (!block_ok(B)) return fail(BSA_EUNSUPPORTED, "B must be 64 or 128");
    if (sigma_den <= 0 || sigma_num < 0 || sigma_num > sigma_den)
      return fail(BSA_EINVAL, "0 <= sigma_num <= sigma_den, sigma_den > 0 required");
    if (!(alpha >= 0.0f) || !std::isfinite(alpha)) return fail(BSA_EINVAL, "alpha must be >= 0 and finite");
    if (order < 0 || order > 5) return fail(BSA_EINVAL, "order must be 0..5");
    if (G > 65535) return fail(BSA_EUNSUPPORTED, "G must be <= 65535");
    return hip_status(bsa::launch_paro_metric(cnt, bsum, bmax, G, N, B, sigma_num, sigma_den, alpha,
                                              order, stats, as_stream(stream)),
                      "bsa_paro_metric");
  });
}

int bsa_paro_select(const float* stats, int32_t G, uint8_t* axis_order, void* stream) {
  return guarded([&]() -> int {
    if (!stats || !axis_order) return fail(BSA_EINVAL, "NULL pointer");
    if (G <= 0) return fail(BSA_EINVAL, "G must be positive");
    return hip_status(bsa::launch_paro_select(stats, G, axis_order, as_stream(stream)),
                      "bsa_paro_select");
  });
}

int64_t bsa_mask_sums_workspace(int32_t G, int32_t N, int32_t Bq, int32_t Bk) {
  if (G <= 0 || N <= 0 || !block_ok(Bq) || !block_ok(Bk)) return -1;
  const int nq = (N + Bq - 1) / Bq, nk = (N + Bk - 1) / Bk;
  if (nk > 8192 || static_cast<int64_t>(G) * nq >= (1ll << 31)) return -1;
  return static_cast<int64_t>(bsa::sorted_select_workspace_bytes(G, nq, nk));
}

int bsa_mask_from_block_sums(const float* keys, int32_t G, int32_t N, int32_t Bq, int32_t Bk,
                             float mass, int32_t force_diag, int32_t* row_ptr, int32_t* col_idx,
                             int64_t col_capacity, int32_t* nnz, void* workspace, int64_t ws_bytes,
                             void* stream) {
  return guarded([&]() -> int {
    if (!keys || !row_ptr || !col_idx || !nnz || !workspace) return fail(BSA_EINVAL, "NULL pointer");
    if (G <= 0 || N <= 0) return fail(BSA_EINVAL, "G and N must be positive");
    if (!block_ok(Bq) || !block_ok(Bk)) return fail(BSA_EUNSUPPORTED, "Bq, Bk must be 64 or 128");
    if (!(mass > 0.0f && mass <= 1.0f)) return fail(BSA_EINVAL, "mass must be in (0, 1]");
    const int64_t nq = (N + Bq - 1) / Bq, nk = (N + Bk - 1) / Bk;
    if (nk > 8192) return fail(BSA_EUNSUPPORTED, "Nkv = %lld exceeds 8192", (long long)nk);
    if (G * nq >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "too many rows");
    const int64_t need_cols = G * nq * nk;
    if (col_capacity < need_cols)
      return fail(BSA_ECAPACITY, "col_capacity %lld < G*Nq*Nkv = %lld", (long long)col_capacity,
                  (long long)need_cols);
    const int64_t need = bsa_mask_sums_workspace(G, N, Bq, Bk);
    if (!aligned(workspace, 256)) return fail(BSA_EINVAL, "workspace must be 256-byte aligned");
    if (ws_bytes < need)
      return fail(BSA_ECAPACITY, "workspace %lld bytes < required %lld", (long long)ws_bytes, (long long)need);
    // the block-sum mass mode of the sorted selection (no window: the
    // token grid only matters for it, so the sequence is passed as 1 x 1 x N)
    return hip_status(bsa::launch_sorted_select(2, keys, nullptr, 0.0f, nullptr, G, 1, 1, N, Bq, Bk,
                                                0, mass, 0.0f, force_diag != 0, -1, 0, row_ptr,
                                                col_idx, col_capacity, nnz, workspace,
                                                as_stream(stream)),
                      "bsa_mask_from_block_sums");
  });
}

int64_t bsa_mask_bits_workspace(int32_t rows) {
  if (rows <= 0) return -1;
  return (static_cast<int64_t>(rows) * 4 + 255) & ~static_cast<int64_t>(255);
}

int bsa_mask_from_bits(const uint64_t* bits, int32_t rows, int32_t nk, int32_t* row_ptr,
                       int32_t* col_idx, int64_t col_capacity, int32_t* nnz, void* workspace,
                       int64_t ws_bytes, void* stream) {
  return guarded([&]() -> int {
    if (!bits || !row_ptr || !col_idx || !nnz || !workspace) return fail(BSA_EINVAL, "NULL pointer");
    if (rows <= 0 || nk <= 0) return fail(BSA_EINVAL, "rows and nk must be positive");
    if (!aligned(bits, 8) || !aligned(workspace, 4)) return fail(BSA_EINVAL, "bits 8-byte, workspace 4-byte alignment required");
    const int64_t need_cols = static_cast<int64_t>(rows) * nk;
    if (need_cols >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "rows*nk must be < 2^31");
    if (col_capacity < need_cols)
      return fail(BSA_ECAPACITY, "col_capacity %lld < rows*nk = %lld", (long long)col_capacity,
                  (long long)need_cols);
    if (ws_bytes < bsa_mask_bits_workspace(rows))
      return fail(BSA_ECAPACITY, "workspace %lld bytes < required %lld", (long long)ws_bytes,
                  (long long)bsa_mask_bits_workspace(rows));
    return hip_status(bsa::launch_bits_to_csr(reinterpret_cast<const unsigned long long*>(bits), rows,
                                              nk, static_cast<int32_t*>(workspace), row_ptr, col_idx,
                                              col_capacity, nnz, as_stream(stream)),
                      "bsa_mask_from_bits");
  });
}

int bsa_block_scores(const float* sums_q, const float* sums_k, int32_t G, int32_t F, int32_t H,
                     int32_t W, int32_t d, const bsa_mask_params* p_host, float* scores,
                     void* workspace, int64_t ws_bytes, void* stream) {
  return guarded([&]() -> int {
    bsa::MaskGeom m{};
    const int rc = mask_geom(G, F, H, W, d, p_host, m);
    if (rc != BSA_OK) return rc;
    if (!sums_q || !sums_k || !scores || !workspace) return fail(BSA_EINVAL, "NULL pointer");
    if (d != 64 && d != 128) return fail(BSA_EUNSUPPORTED, "d must be 64 or 128");
    if (!aligned(sums_k, 16) || !aligned(workspace, 256))
      return fail(BSA_EINVAL, "sums_k 16-byte, workspace 256-byte alignment required");
    const int64_t need = static_cast<int64_t>(bsa::mask_workspace_layout(m).total);
    if (ws_bytes < need)
      return fail(BSA_ECAPACITY, "workspace %lld bytes < required %lld", (long long)ws_bytes, (long long)need);
    return hip_status(bsa::launch_block_scores(m, sums_q, sums_k, scores, static_cast<char*>(workspace),
                                               as_stream(stream)),
                      "bsa_block_scores");
  });
}

int64_t bsa_scores_select_workspace(int32_t G, int32_t F, int32_t H, int32_t W, int32_t Bq,
                                    int32_t Bk) {
  if (G <= 0 || F <= 0 || H <= 0 || W <= 0 || !block_ok(Bq) || !block_ok(Bk)) return -1;
  const int64_t N = static_cast<int64_t>(F) * H * W;
  if (N >= (1ll << 31)) return -1;
  const int64_t nq = (N + Bq - 1) / Bq, nk = (N + Bk - 1) / Bk;
  if (nk > 8192 || G * nq >= (1ll << 31)) return -1;
  return static_cast<int64_t>(bsa::sorted_select_workspace_bytes(G, static_cast<int>(nq),
                                                                 static_cast<int>(nk)));
}

int bsa_mask_from_scores(const float* scores, const float* noise, float noise_scale, int32_t G,
                         int32_t F, int32_t H, int32_t W, const uint8_t* axis_order,
                         const bsa_mask_params* p_host, int32_t mode, float top_p, float temp,
                         int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, int32_t* nnz,
                         void* workspace, int64_t ws_bytes, void* stream) {
  return guarded([&]() -> int {
    bsa::MaskGeom m{};
    const int rc = mask_geom(G, F, H, W, 64, p_host, m);
    if (rc != BSA_OK) return rc;
    if (!scores || !row_ptr || !col_idx || !nnz || !workspace) return fail(BSA_EINVAL, "NULL pointer");
    if (m.win_T >= 0 && !axis_order) return fail(BSA_EINVAL, "axis_order is required with a window");
    if (mode != 0 && mode != 1) return fail(BSA_EINVAL, "mode must be 0 (top-k) or 1 (top-p)");
    if (mode == 1 && !(top_p > 0.0f && top_p <= 1.0f)) return fail(BSA_EINVAL, "top_p must be in (0, 1]");
    if (mode == 1 && !(temp >= 0.0f && std::isfinite(temp))) return fail(BSA_EINVAL, "temp must be >= 0 and finite");
    if (noise && !std::isfinite(noise_scale)) return fail(BSA_EINVAL, "noise_scale must be finite");
    const int64_t need_cols = mode == 0 ? capacity_of(m) : static_cast<int64_t>(G) * m.nq * m.nk;
    if (col_capacity < need_cols)
      return fail(BSA_ECAPACITY, "col_capacity %lld < %lld", (long long)col_capacity, (long long)need_cols);
    const int64_t need = bsa_scores_select_workspace(G, F, H, W, m.Bq, m.Bk);
    if (!aligned(workspace, 256)) return fail(BSA_EINVAL, "workspace must be 256-byte aligned");
    if (ws_bytes < need)
      return fail(BSA_ECAPACITY, "workspace %lld bytes < required %lld", (long long)ws_bytes, (long long)need);
    return hip_status(bsa::launch_sorted_select(mode, scores, noise, noise_scale, axis_order, G, F, H, W,
                                                m.Bq, m.Bk, m.k, top_p, temp, m.force_diag, m.win_T,
                                                m.win_r0, row_ptr, col_idx, col_capacity, nnz,
                                                workspace, as_stream(stream)),
                      "bsa_mask_from_scores");
  });
}

int64_t bsa_fo_workspace(int32_t G, int32_t N, int32_t d, int32_t Bq, int32_t Bk) {
  return guarded([&]() -> int64_t {
    if (G <= 0 || N <= 0) return fail(BSA_EINVAL, "G and N must be positive");
    if (d != 64 && d != 128) return fail(BSA_EUNSUPPORTED, "d must be 64 or 128");
    if (!block_ok(Bq) || !block_ok(Bk)) return fail(BSA_EUNSUPPORTED, "Bq, Bk must be 64 or 128");
    const int64_t nk = (static_cast<int64_t>(N) + Bk - 1) / Bk;
    if (nk > 32768) return fail(BSA_EUNSUPPORTED, "Nkv = %lld exceeds 32768", (long long)nk);
    const int64_t nq = (static_cast<int64_t>(N) + Bq - 1) / Bq;
    if (nq > 32768) return fail(BSA_EUNSUPPORTED, "Nq = %lld exceeds 32768", (long long)nq);
    return static_cast<int64_t>(bsa::fo_layout(G, N, d, Bq, Bk).total);
  });
}

int bsa_fo_compensate(const void* Qp, const void* Kp, const void* Vp, const int32_t* row_ptr,
                      const int32_t* col_idx, int64_t col_len, int32_t mask_G,
                      const uint8_t* axis_order, int32_t F, int32_t H, int32_t W, void* O,
                      int64_t nat_stride_g, int64_t nat_stride_n, float* lse, int32_t G, int32_t d,
                      int32_t Bq, int32_t Bk, float sm_scale, void* workspace, int64_t ws_bytes,
                      void* stream) {
  return guarded([&]() -> int {
    bsa::OutMap om{};
    int32_t N = 0;
    if (axis_order != nullptr) {
      const int rc = natural_out(axis_order, F, H, W, G, d, nat_stride_g, nat_stride_n, om, N);
      if (rc != BSA_OK) return rc;
    } else {
      if (F <= 0 || H <= 0 || W <= 0) return fail(BSA_EINVAL, "F, H, W must be positive");
      const int64_t n64 = static_cast<int64_t>(F) * H * W;
      if (n64 >= (1ll << 31)) return fail(BSA_EUNSUPPORTED, "N = F*H*W must be < 2^31");
      N = static_cast<int32_t>(n64);
    }
    int rc = attn_common(Qp, Kp, Vp, row_ptr, col_idx, col_len, mask_G, O, G, N, d, Bq, Bk, 2);
    if (rc != BSA_OK) return rc;
    if (!lse) return fail(BSA_EINVAL, "lse is required (the forward's log-sum-exp is updated)");
    if (!aligned(lse, 4)) return fail(BSA_EINVAL, "lse must be 4-byte aligned");
    if (!std::isfinite(sm_scale)) return fail(BSA_EINVAL, "sm_scale must be finite");
    const int64_t need = bsa_fo_workspace(G, N, d, Bq, Bk);
    if (need < 0) return static_cast<int>(need);
    if (!workspace) return fail(BSA_EINVAL, "NULL workspace");
    if (!aligned(workspace, 256)) return fail(BSA_EINVAL, "workspace must be 256-byte aligned");
    if (ws_bytes < need)
      return fail(BSA_ECAPACITY, "workspace %lld bytes < required %lld", (long long)ws_bytes, (long long)need);
    const bsa::FoLayout L = bsa::fo_layout(G, N, d, Bq, Bk);
    if (L.gemm_tiles >= (1ll << 31) || static_cast<int64_t>(G) * L.nkp >= (1ll << 31) ||
        static_cast<int64_t>(G) * L.nqp >= (1ll << 31))
      return fail(BSA_EUNSUPPORTED, "grid too large");
    return hip_status(bsa::launch_fo_compensate(static_cast<const uint16_t*>(Qp),
                                                static_cast<const uint16_t*>(Kp),
                                                static_cast<const uint16_t*>(Vp), row_ptr, col_idx,
                                                col_len, mask_G, G, N, d, Bq, Bk, sm_scale,
                                                static_cast<uint16_t*>(O), lse, om,
                                                static_cast<char*>(workspace), as_stream(stream)),
                      "bsa_fo_compensate");
  });
}

int bsa_forward_natural(const void* Qp, const void* Kp, const void* Vp, const int32_t* row_ptr,
                        const int32_t* col_idx, int64_t col_len, int32_t mask_G,
                        const uint8_t* axis_order, int32_t F, int32_t H, int32_t W, void* O,
                        int64_t nat_stride_g, int64_t nat_stride_n, float* lse, int32_t G, int32_t d,
                        int32_t Bq, int32_t Bk, float sm_scale, void* stream) {
  return guarded([&]() -> int {
    bsa::AttnArgs a{};
    int32_t N = 0;
    int rc = natural_out(axis_order, F, H, W, G, d, nat_stride_g, nat_stride_n, a.out, N);
    if (rc != BSA_OK) return rc;
    rc = attn_common(Qp, Kp, Vp, row_ptr, col_idx, col_len, mask_G, O, G, N, d, Bq, Bk, 2);
    if (rc != BSA_OK) return rc;
    if (!std::isfinite(sm_scale)) return fail(BSA_EINVAL, "sm_scale must be finite");
    a.Q = Qp; a.K = Kp; a.V = Vp;
    a.row_ptr = row_ptr; a.col_idx = col_idx; a.col_len = col_len; a.mask_G = mask_G;
    a.O = static_cast<uint16_t*>(O); a.lse = lse;
    a.G = G; a.N = N; a.d = d; a.Bq = Bq; a.Bk = Bk; a.sm_scale = sm_scale;
    return hip_status(bsa::launch_forward_bf16(a, as_stream(stream)), "bsa_forward_natural");
  });
}

int bsa_forward_int8_natural(const int8_t* Qq, const float* sQ, const int8_t* Kq, const float* sK,
                             const int8_t* Vq, const float* sV, const int32_t* row_ptr,
                             const int32_t* col_idx, int64_t col_len, int32_t mask_G,
                             const uint8_t* axis_order, int32_t F, int32_t H, int32_t W, void* O,
                             int64_t nat_stride_g, int64_t nat_stride_n, float* lse, int32_t G,
                             int32_t d, int32_t Bq, int32_t Bk, float sm_scale, void* stream) {
  return guarded([&]() -> int {
    bsa::AttnArgs a{};
    int32_t N = 0;
    int rc = natural_out(axis_order, F, H, W, G, d, nat_stride_g, nat_stride_n, a.out, N);
    if (rc != BSA_OK) return rc;
    rc = attn_common(Qq, Kq, Vq, row_ptr, col_idx, col_len, mask_G, O, G, N, d, Bq, Bk, 1);
    if (rc != BSA_OK) return rc;
    if (!sQ || !sK || !sV) return fail(BSA_EINVAL, "NULL scale pointer");
    if (!std::isfinite(sm_scale)) return fail(BSA_EINVAL, "sm_scale must be finite");
    a.Q = Qq; a.K = Kq; a.V = Vq; a.sQ = sQ; a.sK = sK; a.sV = sV;
    a.row_ptr = row_ptr; a.col_idx = col_idx; a.col_len = col_len; a.mask_G = mask_G;
    a.O = static_cast<uint16_t*>(O); a.lse = lse;
    a.G = G; a.N = N; a.d = d; a.Bq = Bq; a.Bk = Bk; a.sm_scale = sm_scale;
    return hip_status(bsa::launch_forward_int8(a, as_stream(stream)), "bsa_forward_int8_natural");
  });
}

}  // extern "C"
