// bsa_internal.hpp — declarations shared between the C-ABI front end
// (capi.hip) and the kernel translation units.  Launchers assume their
// arguments were validated by the front end; they only launch and return
// the HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

// ---- permute.hip -----------------------------------------------------------
hipError_t launch_permute(int direction, const void* src, int src_dt, void* dst, int dst_dt,
                          int64_t stride_g, int64_t stride_n, int G, int F, int H, int W, int d,
                          const uint8_t* orders, hipStream_t s);

// ---- mask.hip --------------------------------------------------------------
struct MaskGeom {
  int G, F, H, W, d;
  int64_t N;
  int Bq, Bk;
  int nq, nk;      // ceil(N/Bq), ceil(N/Bk)
  int words;       // 64-bit words per bitmask row = ceil(nk/64)
  int score;
  int k;           // per-row top-k budget
  int force_diag;
  int win_T, win_r0;
};
// Workspace carve-up (byte offsets, 256-aligned).
struct MaskWs {
  size_t sum_q, sum_k, norm_q, norm_k, counts, bits, total;
};
MaskWs mask_workspace_layout(const MaskGeom& m);
hipError_t launch_build_mask(const MaskGeom& m, const uint16_t* Qp, const uint16_t* Kp,
                             const uint8_t* orders, int32_t* row_ptr, int32_t* col_idx,
                             int64_t col_capacity, int32_t* nnz, char* ws, hipStream_t s);
// as launch_build_mask from per-block channel sums (Bq blocks of Q, Bk of K)
hipError_t launch_build_mask_pooled(const MaskGeom& m, const float* sums_q, const float* sums_k,
                                    const uint8_t* orders, int32_t* row_ptr, int32_t* col_idx,
                                    int64_t col_capacity, int32_t* nnz, char* ws, hipStream_t s);

// the fixed device scratch of the mask build (file-scope array in mask.hip):
// its size, and its device address on the current device (looked up once
// per device with hipGetSymbolAddress)
size_t mask_scratch_bytes();
hipError_t mask_scratch_ptr(void** out);

// bitmask rows [R][ceil(nk/64)] -> counts (scratch, R ints) -> CSR; bits at
// kv-block >= nk are ignored
hipError_t launch_bits_to_csr(const unsigned long long* bits, int R, int nk, int32_t* counts,
                              int32_t* row_ptr, int32_t* col_idx, int64_t cap, int32_t* nnz,
                              hipStream_t s);

// score matrix [G][nq][nk] of every (q-block, kv-block) pair from per-block
// channel sums (same fp32 sequence as the select step)
hipError_t launch_block_scores(const MaskGeom& m, const float* sums_q, const float* sums_k,
                               float* scores, char* ws, hipStream_t s);
// selection from a score matrix by sorting each row: mode 0 top-k (k),
// 1 top-p (frac, temp), 2 block-sum mass (frac); optional noise (key' =
// fmaf(noise, nscale, key)); forced diagonal / window; CSR.  orders may be
// null when win_T < 0.  Workspace: sorted_select_workspace_bytes.
size_t sorted_select_workspace_bytes(int G, int nq, int nk);
hipError_t launch_sorted_select(int mode, const float* keys, const float* noise, float nscale,
                                const uint8_t* orders, int G, int F, int H, int W, int Bq, int Bk,
                                int k, float frac, float temp, int force_diag, int win_T,
                                int win_r0, int32_t* row_ptr, int32_t* col_idx, int64_t cap,
                                int32_t* nnz, void* ws, hipStream_t s);

// ---- calib.hip -------------------------------------------------------------
hipError_t launch_block_stats(const uint16_t* Qp, const uint16_t* Kp, int G, int N, int d, int B,
                              float sm_scale, float eps, int32_t* cnt, float* bsum, float* bmax,
                              hipStream_t s);
hipError_t launch_paro_metric(const int32_t* cnt, const float* bsum, const float* bmax, int G,
                              int N, int B, int sigma_num, int sigma_den, float alpha, int order,
                              float* stats, hipStream_t s);
hipError_t launch_paro_select(const float* stats, int G, uint8_t* orders, hipStream_t s);

// ---- fused.hip -------------------------------------------------------------
hipError_t launch_permute_pool(const void* src, int src_dt, uint16_t* dst, int64_t stride_g,
                               int64_t stride_n, int G, int F, int H, int W, int d,
                               const uint8_t* orders, int B, float* sums, int8_t* xq, float* scale,
                               hipStream_t s);

// ---- order.hip -------------------------------------------------------------
size_t order_workspace_bytes(int G, int N, int B);
hipError_t launch_order_scores(const void* src, int src_dt, int64_t stride_g, int64_t stride_n,
                               int G, int F, int H, int W, int d, int B, float* scores, void* ws,
                               hipStream_t s);
hipError_t launch_select_orders(const float* a, const float* b, int G, uint8_t* orders,
                                hipStream_t s);

// ---- quant.hip -------------------------------------------------------------
hipError_t launch_quantize_int8(const uint16_t* X, int8_t* Xq, float* scale, int G, int N, int d,
                                int B, hipStream_t s);

// ---- attn.hip --------------------------------------------------------------
// Where a forward writes O (and lse): orders == nullptr -> reordered
// [G][N][d] (lse [G][N]); else the natural token order, row (n, g) at
// n*sn + g*sg elements (lse[g*N + n]), n = the natural index of reordered
// position r under orders[g] on an F x H x W grid.
struct OutMap {
  const uint8_t* orders;
  int F, H, W;
  int64_t sg, sn;
};
struct AttnArgs {
  const void* Q;  // bf16 or int8 [G][N][d]
  const void* K;
  const void* V;
  const float* sQ;  // int8 path only
  const float* sK;
  const float* sV;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int64_t col_len;
  int mask_G;
  uint16_t* O;  // bf16 [G][N][d]
  float* lse;   // [G][N] or nullptr
  int G, N, d, Bq, Bk;
  float sm_scale;
  OutMap out;   // out.orders == nullptr: reordered output
};
hipError_t launch_forward_bf16(const AttnArgs& a, hipStream_t s);

// ---- comp.hip --------------------------------------------------------------
// Workspace of the first-order compensation: per-kv-block moments X (bf16
// [G][nkp][Lp]), skip mask S (bf16 [G][nqp][nkp]), sums over the skipped set
// C (fp32 [G][nqp][Lp]); byte offsets 256-aligned.
struct FoLayout {
  int nq, nk, nqp, nkp, Lp;
  int Lt;              // columns of C past the d x d block (sums of k and v, count, padding)
  int64_t gemm_tiles;  // skip-mask GEMM workgroups over all heads
  size_t x, s, ckv, ct, total;  // moments, skip mask, C's d x d block (bf16), C's tail (fp32)
};
FoLayout fo_layout(int G, int N, int d, int Bq, int Bk);
// O (bf16) and lse (fp32) as a forward wrote them (reordered, or natural
// through om) are updated in place.
hipError_t launch_fo_compensate(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                const int32_t* row_ptr, const int32_t* col_idx, int64_t col_len,
                                int mask_G, int G, int N, int d, int Bq, int Bk, float sm_scale,
                                uint16_t* O, float* lse, const OutMap& om, char* ws,
                                hipStream_t s);
hipError_t launch_forward_int8(const AttnArgs& a, hipStream_t s);
hipError_t launch_debug_int8_qk(const int8_t* Qq, const int8_t* Kq, int G, int N, int d, int Bq,
                                int Bk, const int32_t* gij, int n, int32_t* S, hipStream_t s);
hipError_t launch_debug_int8_pv(const int8_t* P8, const int8_t* Vq, int G, int N, int d, int Bq,
                                int Bk, const int32_t* gj, int n, int32_t* OV, hipStream_t s);

}  // namespace bsa
