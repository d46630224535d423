// bsa_device.hpp — small device-side helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, round-robin dispatch

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even; NaN stays quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Natural token index of reordered position p for axis-order code `order`
// (outermost -> innermost: 0 FHW, 1 FWH, 2 HFW, 3 HWF, 4 WFH, 5 WHF).
// The innermost coordinate is p mod (its extent), the middle one the next
// digit, the outermost what remains; natural index = (f*H + h)*W + w.
__device__ __forceinline__ uint32_t natural_index(int order, uint32_t p, uint32_t F, uint32_t H,
                                                  uint32_t W) {
  uint32_t f, h, w;
  switch (order) {
    default:
    case 0: w = p % W; p /= W; h = p % H; f = p / H; break;  // F H W
    case 1: h = p % H; p /= H; w = p % W; f = p / W; break;  // F W H
    case 2: w = p % W; p /= W; f = p % F; h = p / F; break;  // H F W
    case 3: f = p % F; p /= F; w = p % W; h = p / W; break;  // H W F
    case 4: h = p % H; p /= H; f = p % F; w = p / F; break;  // W F H
    case 5: f = p % F; p /= F; h = p % H; w = p / H; break;  // W H F
  }
  return (f * H + h) * W + w;
}

// The same map as natural_index, split into the order's extents and the
// natural strides of its axes (outermost, middle, innermost), so that a
// kernel mapping many positions resolves the order once:
//   n = (p / (d1*d2)) * s0 + ((p / d2) % d1) * s1 + (p % d2) * s2.
struct OrderMap {
  uint32_t d1, d2, s0, s1, s2;
  __device__ __forceinline__ uint32_t operator()(uint32_t p) const {
    const uint32_t q = p / d2;
    return (q / d1) * s0 + (q % d1) * s1 + (p % d2) * s2;
  }
};

__device__ __forceinline__ OrderMap order_map(int order, uint32_t F, uint32_t H, uint32_t W) {
  const uint32_t sf = H * W, sh = W, sw = 1;
  switch (order) {
    default:
    case 0: return {H, W, sf, sh, sw};  // F H W
    case 1: return {W, H, sf, sw, sh};  // F W H
    case 2: return {F, W, sh, sf, sw};  // H F W
    case 3: return {W, F, sh, sw, sf};  // H W F
    case 4: return {F, H, sw, sf, sh};  // W F H
    case 5: return {H, F, sw, sh, sf};  // W H F
  }
}

// XCD-contiguous tile order for (head, row-block) grids: the G*nq tiles in
// head-major order are cut into 8 contiguous ranges of T = ceil(G*nq/8), and
// XCD x (which receives workgroups bid with bid % 8 == x) runs range x in
// order.  The workgroups resident on one XCD then belong to one head almost
// all the time, so its L2 serves a single head's K/V instead of two.  Grid
// size must be 8 * T; returns false for the padding slots.
__device__ __forceinline__ bool xcd_range_tile(uint32_t bid, int nq, int G, int& g, int& i) {
  const int64_t total = static_cast<int64_t>(G) * nq;
  const int64_t T = (total + kNumXcd - 1) / kNumXcd;
  const int64_t item = (bid % kNumXcd) * T + bid / kNumXcd;
  if (item >= total) return false;
  g = static_cast<int>(item / nq);
  i = static_cast<int>(item % nq);
  return true;
}

// Grouped tile order for (head, row-block) grids: the 8 XCDs form groups of
// kXcdGroup; group p takes heads [p*hpg, (p+1)*hpg) in order, and within a
// head XCD member m of the group takes the contiguous rows [m*per,
// (m+1)*per).  Two heads are in flight at a time (their K/V stay resident in
// the last-level cache) and each XCD's concurrent workgroups are neighbouring
// rows of one head (which share K/V in its L2).  Grid size:
// xcd_group_grid(nq, G); returns false for the padding slots.
constexpr int kXcdGroup = 4;
inline uint32_t xcd_group_grid(int nq, int G) {
  constexpr int groups = kNumXcd / kXcdGroup;
  const int64_t hpg = (G + groups - 1) / groups, per = (nq + kXcdGroup - 1) / kXcdGroup;
  return static_cast<uint32_t>(kNumXcd * hpg * per);
}
__device__ __forceinline__ bool xcd_group_tile(uint32_t bid, int nq, int G, int& g, int& i) {
  constexpr int groups = kNumXcd / kXcdGroup;
  const int x = static_cast<int>(bid % kNumXcd), k = static_cast<int>(bid / kNumXcd);
  const int hpg = (G + groups - 1) / groups, per = (nq + kXcdGroup - 1) / kXcdGroup;
  const int hl = k / per;
  g = (x / kXcdGroup) * hpg + hl;
  i = (x % kXcdGroup) * per + k % per;
  return hl < hpg && g < G && i < nq;
}

// Output row of reordered position r of head g under an OutMap-like
// description: reordered [G][N][D] when orders is null, else the natural
// token n = perm_g(r) at n*sn + g*sg; lse_idx receives the matching
// [G][N] index (g*N + r, or g*N + n).
template <int D>
__device__ __forceinline__ uint16_t* out_row(uint16_t* O, const uint8_t* orders, int F, int H, int W,
                                             int64_t sg, int64_t sn, int g, int N, int r,
                                             int64_t& lse_idx) {
  if (orders == nullptr) {
    lse_idx = static_cast<int64_t>(g) * N + r;
    return O + lse_idx * D;
  }
  const uint32_t n = natural_index(orders[g], static_cast<uint32_t>(r), F, H, W);
  lse_idx = static_cast<int64_t>(g) * N + n;
  return O + static_cast<int64_t>(n) * sn + static_cast<int64_t>(g) * sg;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    T u = __shfl_xor(v, o);
    v = v > u ? v : u;
  }
  return v;
}

}  // namespace bsa
