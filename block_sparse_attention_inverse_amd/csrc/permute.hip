// permute.hip — per-head token reordering and its inverse.
//
// PAROAttention machine verdict (pith.science, arXiv 2506.16054), key
// machinery: every head reorders its flattened F x H x W sequence by one of
// the six axis orders, so that the axis it aggregates along becomes
// contiguous.  The permutation is never stored: each thread derives the
// natural index of its reordered row from the order code by div/mod.
//
// HBM-bound gather/scatter.  A chunk is 8 channels (16 B of bf16 or 32 B of
// fp32); d/8 consecutive threads cover one row, so every wave reads and
// writes whole rows contiguously on both sides.
#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {
namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 8 consecutive channels: two 16-byte words for fp32, one for bf16 (lo only).
template <bool F32>
__device__ __forceinline__ void load8(const void* base, int64_t off, u32x4& lo, u32x4& hi) {
  if constexpr (F32) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(base) + off);
    lo = __builtin_nontemporal_load(p);
    hi = __builtin_nontemporal_load(p + 1);
  } else {
    lo = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off));
  }
}

template <bool SRC_F32, bool DST_F32>
__device__ __forceinline__ void store8(void* base, int64_t off, const u32x4& lo, const u32x4& hi) {
  if constexpr (DST_F32) {
    u32x4 a, b;
    if constexpr (SRC_F32) {
      a = lo;
      b = hi;
    } else {  // bf16 -> fp32 is exact: the bf16 bits are the upper half
      a = u32x4{lo.x << 16, lo.x & 0xffff0000u, lo.y << 16, lo.y & 0xffff0000u};
      b = u32x4{lo.z << 16, lo.z & 0xffff0000u, lo.w << 16, lo.w & 0xffff0000u};
    }
    u32x4* p = reinterpret_cast<u32x4*>(static_cast<float*>(base) + off);
    __builtin_nontemporal_store(a, p);
    __builtin_nontemporal_store(b, p + 1);
  } else {
    u32x4 o;
    if constexpr (SRC_F32) {
      auto cv = [](uint32_t x, uint32_t y) {
        return f32_to_bf16_bits(__uint_as_float(x)) | (f32_to_bf16_bits(__uint_as_float(y)) << 16);
      };
      o = u32x4{cv(lo.x, lo.y), cv(lo.z, lo.w), cv(hi.x, hi.y), cv(hi.z, hi.w)};
    } else {
      o = lo;
    }
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + off));
  }
}

// grid: (ceil(N*d/8 / (kThreads*kChunks)), G).  direction 0 gathers
// natural -> reordered, direction 1 scatters reordered -> natural.  Each
// thread moves kChunks 8-channel chunks, kThreads apart, with all of its
// loads issued before its first store; the order is resolved once.
constexpr int kChunks = 4;
template <bool SRC_F32, bool DST_F32, bool GATHER>
__global__ __launch_bounds__(kThreads) void permute_kernel(
    const void* __restrict__ src, void* __restrict__ dst, int64_t stride_g, int64_t stride_n,
    uint32_t N, uint32_t F, uint32_t H, uint32_t W, uint32_t chunks_per_row,
    const uint8_t* __restrict__ orders) {
  const uint32_t g = blockIdx.y;
  const OrderMap nat_of = order_map(orders[g], F, H, W);
  const uint64_t total = static_cast<uint64_t>(N) * chunks_per_row;
  const int d = static_cast<int>(chunks_per_row * 8);
  const uint64_t c0 = static_cast<uint64_t>(blockIdx.x) * kThreads * kChunks + threadIdx.x;
  u32x4 lo[kChunks], hi[kChunks];
  int64_t to[kChunks];
#pragma unroll
  for (int m = 0; m < kChunks; m++) {
    // chunks past the end reload the last one (no branch around the load)
    const uint64_t c = c0 + static_cast<uint64_t>(m) * kThreads;
    const uint64_t cc = c < total ? c : total - 1;
    const uint32_t p = static_cast<uint32_t>(cc / chunks_per_row);
    const uint32_t c8 = static_cast<uint32_t>(cc - static_cast<uint64_t>(p) * chunks_per_row) * 8;
    const int64_t nat = static_cast<int64_t>(nat_of(p)) * stride_n + static_cast<int64_t>(g) * stride_g + c8;
    const int64_t red = (static_cast<int64_t>(g) * N + p) * d + c8;
    load8<SRC_F32>(src, GATHER ? nat : red, lo[m], hi[m]);
    to[m] = GATHER ? red : nat;
  }
#pragma unroll
  for (int m = 0; m < kChunks; m++)
    if (c0 + static_cast<uint64_t>(m) * kThreads < total) store8<SRC_F32, DST_F32>(dst, to[m], lo[m], hi[m]);
}

template <bool S32, bool D32>
hipError_t launch_typed(int direction, const void* src, void* dst, int64_t stride_g,
                        int64_t stride_n, int G, int F, int H, int W, int d, const uint8_t* orders,
                        hipStream_t s) {
  const uint32_t N = static_cast<uint32_t>(F) * H * W;
  const uint32_t cpr = static_cast<uint32_t>(d / 8);
  const uint64_t threads = static_cast<uint64_t>(N) * cpr;
  dim3 grid(static_cast<uint32_t>((threads + kThreads * kChunks - 1) / (kThreads * kChunks)), G);
  if (direction == 0)
    permute_kernel<S32, D32, true><<<grid, kThreads, 0, s>>>(src, dst, stride_g, stride_n, N, F,
                                                             H, W, cpr, orders);
  else
    permute_kernel<S32, D32, false><<<grid, kThreads, 0, s>>>(src, dst, stride_g, stride_n, N, F,
                                                              H, W, cpr, orders);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_permute(int direction, const void* src, int src_dt, void* dst, int dst_dt,
                          int64_t stride_g, int64_t stride_n, int G, int F, int H, int W, int d,
                          const uint8_t* orders, hipStream_t s) {
  const bool s32 = src_dt == 0, d32 = dst_dt == 0;
  if (s32 && d32)
    return launch_typed<true, true>(direction, src, dst, stride_g, stride_n, G, F, H, W, d, orders, s);
  if (s32)
    return launch_typed<true, false>(direction, src, dst, stride_g, stride_n, G, F, H, W, d, orders, s);
  if (d32)
    return launch_typed<false, true>(direction, src, dst, stride_g, stride_n, G, F, H, W, d, orders, s);
  return launch_typed<false, false>(direction, src, dst, stride_g, stride_n, G, F, H, W, d, orders, s);
}

}  // namespace bsa
