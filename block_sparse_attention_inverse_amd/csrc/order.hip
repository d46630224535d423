// order.hip — online choice of each head's axis order by the sum of
// intra-block cosine similarities (SICS).
//
// SPADE machine verdict (pith.science, arXiv 2608.03335), key machinery and
// core discovery: every candidate blocking of a head's Q/K token grid is
// scored by the sum of all pairwise cosine similarities inside its blocks,
// computed online in O(block * d) from partial sums, and the blocking with
// the highest score is chosen (referee summary and desk-editor letter: the
// online recurrence).  The candidates here are the six axis orders of the
// reordering (PAROAttention verdict, key machinery), cut into blocks of B
// consecutive reordered tokens.  For a block, the sum over ordered pairs
// (a, b) of cos(x_a, x_b) equals |sum_a x_a/|x_a||^2, so one pass per block
// suffices; counting unordered pairs or leaving out a == b changes every
// order's score by the same affine map and not the argmax.
//
// Fixed fp32 sequence (exactly reproducible, the argmax is an integer
// outcome decided by it): for head g, order o, block b of len rows (rows in
// increasing reordered position):
//   n_r   = fmaf chain over c of x[r][c]^2 from +0;   inv_r = 1 / sqrt(n_r)
//           (correctly rounded sqrt, then divide; inv_r = 0 if n_r == 0)
//   u[c]  = fmaf chain over r of x[r][c] * inv_r from +0
//   q_b   = fmaf chain over c of u[c]^2 from +0
//   score[g][o] = running sum of q_b over b in increasing order from +0.
// Selection: the order maximising score_a[g][o] + score_b[g][o] (fp32 add;
// ties go to the lower order code).
#pragma clang fp contract(off)

#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// inv[g][n] = 1 / sqrt(fmaf chain over channels of x^2) for every token n
// of head g (0 for an all-zero token); a token's norm does not depend on
// the order, so it is computed once for all six.  One thread per token
// (used for fp32 input; bf16 input takes the staged variant below).
template <bool F32, int D>
__global__ __launch_bounds__(256) void sics_inv_kernel(const void* __restrict__ src,
                                                       int64_t stride_g, int64_t stride_n,
                                                       uint32_t N, int G, float* __restrict__ inv) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // g * N + n
  if (idx >= static_cast<int64_t>(G) * N) return;
  const int64_t g = idx / N, n = idx % N;
  const int64_t off = n * stride_n + g * stride_g;
  float nr = 0.0f;
  if constexpr (F32) {
    const u32x4* xr = reinterpret_cast<const u32x4*>(static_cast<const float*>(src) + off);
#pragma unroll
    for (int c4 = 0; c4 < D / 4; c4++) {
      const u32x4 v = xr[c4];
#pragma unroll
      for (int q = 0; q < 4; q++) nr = __builtin_fmaf(__uint_as_float(v[q]), __uint_as_float(v[q]), nr);
    }
  } else {
    const u32x4* xr = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + off);
#pragma unroll
    for (int c8 = 0; c8 < D / 8; c8++) {
      const u32x4 v = xr[c8];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const float lo = bf16_bits_to_f32(v[q] & 0xffffu), hi = bf16_bits_to_f32(v[q] >> 16);
        nr = __builtin_fmaf(lo, lo, nr);
        nr = __builtin_fmaf(hi, hi, nr);
      }
    }
  }
  inv[idx] = nr > 0.0f ? 1.0f / __builtin_sqrtf(nr) : 0.0f;
}

// bf16 variant of the same table: a workgroup stages 128 consecutive
// tokens of one head through LDS (each token's row read by 16 lanes as one
// coalesced 256-byte access at d = 128), chunk c of token r stored at
// c ^ (r mod 16) within the row, then thread r runs token r's chain over the
// channels in order.
constexpr int kInvRows = 128;
template <int D>
__global__ __launch_bounds__(256) void sics_inv_bf16_kernel(const uint16_t* __restrict__ src,
                                                            int64_t stride_g, int64_t stride_n,
                                                            uint32_t N, float* __restrict__ inv) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  constexpr int SW = CPR - 1 < 15 ? CPR - 1 : 15;
  constexpr int PER = kInvRows * CPR / 256;
  __shared__ u32x4 xs[kInvRows * CPR];
  const int g = blockIdx.y, t = threadIdx.x;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kInvRows;
  const int len = static_cast<int>(min(static_cast<int64_t>(kInvRows), static_cast<int64_t>(N) - n0));
  const int nc = len * CPR;
  u32x4 v[PER];
#pragma unroll
  for (int m = 0; m < PER; m++) {
    const int c = min(t + 256 * m, nc - 1);  // past the last token: reload it, unused
    const int r = c / CPR, ch = c % CPR;
    v[m] = *reinterpret_cast<const u32x4*>(src + (n0 + r) * stride_n + g * stride_g + ch * 8);
  }
#pragma unroll
  for (int m = 0; m < PER; m++) {
    const int c = t + 256 * m;
    if (c < nc) {
      const int r = c / CPR, ch = c % CPR;
      xs[r * CPR + (ch ^ (r & SW))] = v[m];
    }
  }
  __syncthreads();
  if (t < len) {
    float nr = 0.0f;
#pragma unroll
    for (int ch = 0; ch < CPR; ch++) {
      const u32x4 w = xs[t * CPR + (ch ^ (t & SW))];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const float lo = bf16_bits_to_f32(w[q] & 0xffffu), hi = bf16_bits_to_f32(w[q] >> 16);
        nr = __builtin_fmaf(lo, lo, nr);
        nr = __builtin_fmaf(hi, hi, nr);
      }
    }
    inv[static_cast<int64_t>(g) * N + n0 + t] = nr > 0.0f ? 1.0f / __builtin_sqrtf(nr) : 0.0f;
  }
}

// One wave per (block b, order o, head g): q_b into part[g][o][b].  Lane l
// owns channels l*CPL .. l*CPL+CPL-1 and runs their chains over the block's
// rows in order, reading each row straight from global memory (one
// coalesced access per row); row r's natural index comes from the lane
// that computed it, its inverse norm from the per-token table.
template <bool F32, int D>
__global__ __launch_bounds__(kWave) void sics_block_kernel(
    const void* __restrict__ src, int64_t stride_g, int64_t stride_n, uint32_t N, uint32_t F,
    uint32_t H, uint32_t W, int B, int nb, const float* __restrict__ inv, float* __restrict__ part) {
  constexpr int CPL = D / kWave;  // channels per lane
  __shared__ __align__(16) float u[D];
  const int b = blockIdx.x, o = blockIdx.y, g = blockIdx.z;
  const int lane = threadIdx.x;
  const int r0 = b * B;
  const int len = min(B, static_cast<int>(N) - r0);  // B <= 2 * kWave
  const uint32_t n_lo = lane < len ? natural_index(o, static_cast<uint32_t>(r0 + lane), F, H, W) : 0u;
  const uint32_t n_hi =
      lane + kWave < len ? natural_index(o, static_cast<uint32_t>(r0 + kWave + lane), F, H, W) : 0u;
  const float* invg = inv + static_cast<int64_t>(g) * N;
  const int64_t gofs = static_cast<int64_t>(g) * stride_g + lane * CPL;
  float a[CPL];
#pragma unroll
  for (int k = 0; k < CPL; k++) a[k] = 0.0f;
  // row r: its natural index from the lane that computed it, its inverse
  // norm, and this lane's channels of it
  auto fetch = [&](int r, float& ir, float (&x)[CPL]) {
    const uint32_t n = __builtin_amdgcn_readlane(r < kWave ? n_lo : n_hi, r & (kWave - 1));
    ir = invg[n];
    const int64_t off = static_cast<int64_t>(n) * stride_n + gofs;
    if constexpr (F32) {
      const float* xp = static_cast<const float*>(src) + off;
#pragma unroll
      for (int k = 0; k < CPL; k++) x[k] = xp[k];
    } else if constexpr (CPL == 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(src) + off);
      x[0] = bf16_bits_to_f32(w & 0xffffu);
      x[1] = bf16_bits_to_f32(w >> 16);
    } else {
      x[0] = bf16_bits_to_f32(static_cast<const uint16_t*>(src)[off]);
    }
  };
  constexpr int kRun = 16;  // rows whose loads are in flight together
  int r = 0;
  for (; r + kRun <= len; r += kRun) {
    float ir[kRun], x[kRun][CPL];
#pragma unroll
    for (int e = 0; e < kRun; e++) fetch(r + e, ir[e], x[e]);
#pragma unroll
    for (int e = 0; e < kRun; e++)
#pragma unroll
      for (int k = 0; k < CPL; k++) a[k] = __builtin_fmaf(x[e][k], ir[e], a[k]);
  }
  for (; r < len; r++) {
    float ir, x[CPL];
    fetch(r, ir, x);
#pragma unroll
    for (int k = 0; k < CPL; k++) a[k] = __builtin_fmaf(x[k], ir, a[k]);
  }
#pragma unroll
  for (int k = 0; k < CPL; k++) u[lane * CPL + k] = a[k];
  __syncthreads();
  if (lane == 0) {
    float q = 0.0f;
    const float4* u4 = reinterpret_cast<const float4*>(u);
#pragma unroll 8
    for (int c4 = 0; c4 < D / 4; c4++) {
      const float4 v = u4[c4];
      q = __builtin_fmaf(v.x, v.x, q);
      q = __builtin_fmaf(v.y, v.y, q);
      q = __builtin_fmaf(v.z, v.z, q);
      q = __builtin_fmaf(v.w, v.w, q);
    }
    part[(static_cast<int64_t>(g) * 6 + o) * nb + b] = q;
  }
}

// score[g][o] = sum of part[g][o][0..nb) in order: one workgroup per
// (g, o) stages the terms through LDS in coalesced runs, one lane adds them
constexpr int kSumThreads = 256;
constexpr int kSumRun = 4096;
__global__ __launch_bounds__(kSumThreads) void sics_sum_kernel(const float* __restrict__ part,
                                                               int nb, float* __restrict__ scores) {
  __shared__ __align__(16) float run[kSumRun];
  const int i = blockIdx.x, t = threadIdx.x;
  const float* p = part + static_cast<int64_t>(i) * nb;
  float s = 0.0f;
  for (int b0 = 0; b0 < nb; b0 += kSumRun) {
    const int n = min(kSumRun, nb - b0);
    for (int e = t; e < n; e += kSumThreads) run[e] = p[b0 + e];
    __syncthreads();
    if (t == 0) {
      int e = 0;
      for (; e + 4 <= n; e += 4) {
        const float4 v = *reinterpret_cast<const float4*>(run + e);
        s = s + v.x;
        s = s + v.y;
        s = s + v.z;
        s = s + v.w;
      }
      for (; e < n; e++) s = s + run[e];
    }
    __syncthreads();
  }
  if (t == 0) scores[i] = s;
}

__global__ void select_orders_kernel(const float* __restrict__ a, const float* __restrict__ b,
                                     int G, uint8_t* __restrict__ orders) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= G) return;
  int best = 0;
  float bv = 0.0f;
  for (int o = 0; o < 6; o++) {
    float v = a[g * 6 + o];
    if (b != nullptr) v = v + b[g * 6 + o];
    if (o == 0 || v > bv) { best = o; bv = v; }
  }
  orders[g] = static_cast<uint8_t>(best);
}

}  // namespace

// workspace: part [G][6][nb] fp32, then (256-byte aligned) inv [G][N] fp32
static size_t part_bytes(int G, int N, int B) {
  const size_t nb = static_cast<size_t>((N + B - 1) / B);
  return (sizeof(float) * static_cast<size_t>(G) * 6 * nb + 255) & ~static_cast<size_t>(255);
}

size_t order_workspace_bytes(int G, int N, int B) {
  return part_bytes(G, N, B) + sizeof(float) * static_cast<size_t>(G) * static_cast<size_t>(N);
}

hipError_t launch_order_scores(const void* src, int src_dt, int64_t stride_g, int64_t stride_n,
                               int G, int F, int H, int W, int d, int B, float* scores, void* ws,
                               hipStream_t s) {
  const uint32_t N = static_cast<uint32_t>(F) * H * W;
  const int nb = static_cast<int>((N + B - 1) / B);
  float* part = static_cast<float*>(ws);
  float* inv = reinterpret_cast<float*>(static_cast<char*>(ws) + part_bytes(G, static_cast<int>(N), B));
  const uint32_t inv_grid = static_cast<uint32_t>((static_cast<int64_t>(G) * N + 255) / 256);
  const dim3 grid(nb, 6, G);
  const dim3 inv16_grid((N + kInvRows - 1) / kInvRows, G);
  const uint16_t* s16 = static_cast<const uint16_t*>(src);
  const bool f32 = src_dt == 0;
  if (d == 128) {
    if (f32) sics_inv_kernel<true, 128><<<inv_grid, 256, 0, s>>>(src, stride_g, stride_n, N, G, inv);
    else sics_inv_bf16_kernel<128><<<inv16_grid, 256, 0, s>>>(s16, stride_g, stride_n, N, inv);
    if (f32) sics_block_kernel<true, 128><<<grid, kWave, 0, s>>>(src, stride_g, stride_n, N, F, H, W, B, nb, inv, part);
    else sics_block_kernel<false, 128><<<grid, kWave, 0, s>>>(src, stride_g, stride_n, N, F, H, W, B, nb, inv, part);
  } else {
    if (f32) sics_inv_kernel<true, 64><<<inv_grid, 256, 0, s>>>(src, stride_g, stride_n, N, G, inv);
    else sics_inv_bf16_kernel<64><<<inv16_grid, 256, 0, s>>>(s16, stride_g, stride_n, N, inv);
    if (f32) sics_block_kernel<true, 64><<<grid, kWave, 0, s>>>(src, stride_g, stride_n, N, F, H, W, B, nb, inv, part);
    else sics_block_kernel<false, 64><<<grid, kWave, 0, s>>>(src, stride_g, stride_n, N, F, H, W, B, nb, inv, part);
  }
  const int n = G * 6;
  sics_sum_kernel<<<n, kSumThreads, 0, s>>>(part, nb, scores);
  return hipGetLastError();
}

hipError_t launch_select_orders(const float* a, const float* b, int G, uint8_t* orders,
                                hipStream_t s) {
  select_orders_kernel<<<(G + 255) / 256, 256, 0, s>>>(a, b, G, orders);
  return hipGetLastError();
}

}  // namespace bsa
