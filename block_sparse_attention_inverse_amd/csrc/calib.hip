// calib.hip — offline calibration of the static path: statistics of the dense
// post-softmax map per block, the order metric built from them, and the
// argmin over the six axis orders (the static mask by block-sum
// thresholding is the mass mode of the sorted selection in mask.hip).
//
// PAROAttention machine verdict (pith.science, arXiv 2506.16054), key
// machinery: each head's axis order is picked offline from its post-softmax
// attention map by a metric that weighs block sparsifiability (the share of
// blocks whose entries are mostly below a small threshold) against the
// blocks' quantisation incoherence (largest over mean |A| inside a block);
// the static mask keeps blocks chosen by thresholding block sums.  Referee
// minor comment on Eq. (1): n^{<eps}_{ij} counts block (i, j)'s entries
// below eps; referee major comment on Sec. 4.1 Eq. (3): the weight alpha is
// not given.
//
// Block statistics kernel (dense, two passes over every key):
//   S^T = K . Q^T with v_mfma_f32_32x32x16_bf16: A = 32 key rows read from
//   LDS (64-key tiles staged once per workgroup, double-buffered), B = 32
//   query rows held in registers (every lane holds one query column and 16
//   keys of it).
//   Pass 1 keeps a per-lane running maximum and sum in log2 units and
//   merges the two lane halves: lse2 = m + log2(l) per query row.
//   Pass 2 recomputes S, forms A = exp2(S*c - lse2) and accumulates count
//   below eps, sum and maximum per (q-block, kv-block), reduced over the
//   wave (and, for 128-row blocks, over the two waves of the q-block through
//   LDS).  Each wave owns 64 query rows as two 32-row halves, so each K
//   operand feeds two MFMAs; a workgroup of four waves covers 256 rows.
#include <algorithm>

#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kStatRows = 256;  // query rows per workgroup (4 waves x 64)

__device__ __forceinline__ bf16x8 load8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// K staging: 64-key tiles move global -> LDS once per workgroup (four waves
// share them) with 16-byte buffer loads that write LDS directly; rows past N
// read as zero (their keys are masked).  16-byte chunk c of tile row r sits
// at chunk position c ^ (r mod CH), so that the operand reads (32 rows, one
// chunk each per half-wave) hit distinct banks; the swizzle is realised by
// the chunk each lane fetches.
template <int D>
struct KStage {
  static constexpr int CH = D / 8;                 // 16-byte chunks per row
  static constexpr int ROWB = D * 2;               // bytes per row
  static constexpr int TILEB = 64 * ROWB;          // bytes per 64-key tile
  static constexpr int RPL = 1024 / ROWB;          // rows per 1 KB wave-load
  static constexpr int NL = TILEB / 1024 / 4;      // loads per wave per tile
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff;  // load q of wave w fills rows RPL*(4q + w) + lane/CH; the swizzle is q-independent
  uint32_t wb;
  __device__ __forceinline__ void init(const uint16_t* K, int N, int t) {
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(K), 0, N * ROWB, 0x00020000);
    const int lane = t & 63, w = t >> 6;
    const int r = RPL * w + lane / CH, p = lane % CH;
    voff = static_cast<uint32_t>(r * ROWB + ((p ^ (r % CH)) << 4));
    wb = static_cast<uint32_t>(w) * 1024u;
  }
  __device__ __forceinline__ void load(uint8_t* lds, int key0) const {
#pragma unroll
    for (int q = 0; q < NL; q++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(lds + q * 4096 + wb), 16, voff,
          static_cast<uint32_t>((key0 + 4 * RPL * q) * ROWB), 0, 0);
  }
};

// S^T of sub-tile u (keys 32u .. 32u+31 of the LDS tile) against the
// wave's 2 x 32 queries.  A operand of k-step ks: lane L takes tile row
// 32u + L%32, channels 16ks + 8(L/32) .. +7; each operand is read right
// before the two MFMAs that use it, which keeps few K registers live.
template <int D>
__device__ __forceinline__ void s_tile_lds(const uint8_t* lds, int u, int lane,
                                           const bf16x8 (&qop)[2][D / 16], f32x16 (&acc)[2]) {
  constexpr int CH = D / 8, ROWB = D * 2;
  const int row = 32 * u + lane % 32;
  const uint8_t* base = lds + row * ROWB;
  acc[0] = f32x16{};
  acc[1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ks++) {
    const int ch = 2 * ks + lane / 32;
    const bf16x8 kop =
        __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(base + ((ch ^ (row % CH)) * 16)));
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[0][ks], acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[1][ks], acc[1], 0, 0, 0);
  }
}

__device__ __forceinline__ int key_of(int slot, int lane) {
  return 8 * (slot / 4) + 4 * (lane / 32) + slot % 4;
}

// three waves per SIMD (168 VGPRs): the kernel is latency-bound, and more
// resident waves hide the MFMA-to-VALU and LDS latencies
template <int D, int B>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void block_stats_kernel(
    const uint16_t* __restrict__ Qp, const uint16_t* __restrict__ Kp, int N, float c, float eps,
    int32_t* __restrict__ cnt, float* __restrict__ bsum, float* __restrict__ bmax) {
  constexpr int KS = D / 16;
  constexpr int SUBS = B / 32;  // 32-key sub-tiles per kv-block
  __shared__ float part[2][4][3];
  const int g = blockIdx.y;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int r0 = blockIdx.x * kStatRows + 64 * w;  // this wave's first query row
  const int nb = (N + B - 1) / B;
  const uint16_t* Q = Qp + static_cast<int64_t>(g) * N * D;
  const uint16_t* K = Kp + static_cast<int64_t>(g) * N * D;

  bf16x8 qop[2][KS];
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    const int row = min(r0 + 32 * qb + lane % 32, N - 1);
    const uint16_t* p = Q + static_cast<int64_t>(row) * D + 8 * (lane / 32);
#pragma unroll
    for (int ks = 0; ks < KS; ks++) qop[qb][ks] = load8(p + 16 * ks);
  }

  // ---- pass 1: row log-sum-exp (log2 units), per lane over its keys
  __shared__ __attribute__((aligned(16))) uint8_t kt[2][KStage<D>::TILEB];
  const int tid = threadIdx.x;
  const int nt = (N + 31) / 32;       // 32-key sub-tiles
  const int ntile = (N + 63) / 64;    // 64-key LDS tiles
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.0f, 0.0f};
  KStage<D> st;
  st.init(K, N, tid);
  auto lse_sub = [&](int t, const uint8_t* lds, int u) {
    f32x16 acc[2];
    s_tile_lds<D>(lds, u, lane, qop, acc);
    if (32 * t + 32 > N) {
      // keys past N take no weight
#pragma unroll
      for (int qb = 0; qb < 2; qb++)
#pragma unroll
        for (int e = 0; e < 16; e++)
          if (32 * t + key_of(e, lane) >= N) acc[qb][e] = -INFINITY;
    }
#pragma unroll
    for (int qb = 0; qb < 2; qb++) {
      float tm = acc[qb][0];
#pragma unroll
      for (int e = 1; e < 16; e++) tm = fmaxf(tm, acc[qb][e]);
      // c > 0, so the scaled maximum is the maximum of the scaled scores;
      // mn is finite: every sub-tile holds at least one real key
      const float mn = fmaxf(m[qb], tm * c);
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; e++) s += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[qb][e], c, -mn));
      l[qb] = l[qb] * __builtin_amdgcn_exp2f(m[qb] - mn) + s;
      m[qb] = mn;
    }
  };
  // one barrier per tile: in step T the waves read buffer T&1, then write
  // tile T+1 into the other buffer, which every wave finished reading in
  // step T-1 (before the barrier that ended it)
  st.load(kt[0], 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int T = 0; T < ntile; T++) {
    // the other buffer was last read in tile T-1, before the barrier that ended it
    if (T + 1 < ntile) st.load(kt[(T + 1) & 1], 64 * (T + 1));
    lse_sub(2 * T, kt[T & 1], 0);
    if (2 * T + 1 < nt) lse_sub(2 * T + 1, kt[T & 1], 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  float lse2[2];
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    const float mo = __shfl_xor(m[qb], 32), lo = __shfl_xor(l[qb], 32);
    const float mm = fmaxf(m[qb], mo);
    const float lt = l[qb] * __builtin_amdgcn_exp2f(m[qb] - mm) + lo * __builtin_amdgcn_exp2f(mo - mm);
    lse2[qb] = mm + __log2f(lt);
  }

  // ---- pass 2: statistics per (q-block, kv-block); a 64-key tile never
  // straddles two kv-blocks
  const bool rv[2] = {r0 + lane % 32 < N, r0 + 32 + lane % 32 < N};
  const bool rows_full = r0 + 64 <= N;
  const int qblk = r0 / B;  // the wave's 64 rows lie in one q-block
  int ccount = 0;  // wave-uniform: each element's test is counted once per wave via a ballot
  float csum = 0.0f, xmax = -INFINITY;  // maximum exponent; the block maximum is exp2(xmax)
  auto stat_sub = [&](int t, const uint8_t* lds, int u) {
    f32x16 acc[2];
    s_tile_lds<D>(lds, u, lane, qop, acc);
    if (rows_full && 32 * t + 32 <= N) {
#pragma unroll
      for (int qb = 0; qb < 2; qb++) {
#pragma unroll
        for (int e = 0; e < 16; e++) {
          const float x = __builtin_fmaf(acc[qb][e], c, -lse2[qb]);
          const float a = __builtin_amdgcn_exp2f(x);
          ccount += __popcll(__ballot(a < eps));
          csum += a;
          xmax = fmaxf(xmax, x);
        }
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < 2; qb++) {
#pragma unroll
        for (int e = 0; e < 16; e++) {
          const bool real = rv[qb] && 32 * t + key_of(e, lane) < N;
          const float x = real ? __builtin_fmaf(acc[qb][e], c, -lse2[qb]) : -INFINITY;
          const float a = __builtin_amdgcn_exp2f(x);
          ccount += __popcll(__ballot(real && a < eps));
          csum += a;
          xmax = fmaxf(xmax, x);
        }
      }
    }
  };
  auto flush = [&](int j) {
    float cmax = __builtin_amdgcn_exp2f(xmax);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      csum += __shfl_xor(csum, o);
      cmax = fmaxf(cmax, __shfl_xor(cmax, o));
    }
    const int64_t o = (static_cast<int64_t>(g) * nb + qblk) * nb + j;
    if constexpr (B == 64) {
      if (lane == 0 && r0 < N) {
        cnt[o] = ccount;
        bsum[o] = csum;
        bmax[o] = cmax;
      }
    } else {
      // the two waves of a 128-row q-block meet in LDS (double-buffered by j)
      float* slot = part[j & 1][w];
      if (lane == 0) {
        slot[0] = __int_as_float(ccount);
        slot[1] = csum;
        slot[2] = cmax;
      }
      __syncthreads();
      if ((w & 1) == 0 && lane == 0 && r0 < N) {
        const float* other = part[j & 1][w + 1];
        cnt[o] = ccount + __float_as_int(other[0]);
        bsum[o] = csum + other[1];
        bmax[o] = fmaxf(cmax, other[2]);
      }
    }
    ccount = 0;
    csum = 0.0f;
    xmax = -INFINITY;
  };
  st.load(kt[0], 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int T = 0; T < ntile; T++) {
    if (T + 1 < ntile) st.load(kt[(T + 1) & 1], 64 * (T + 1));
    stat_sub(2 * T, kt[T & 1], 0);
    if (2 * T + 1 < nt) stat_sub(2 * T + 1, kt[T & 1], 1);
    // the tile ends kv-block T*64/B when it is the block's last tile or the
    // last tile of all
    if ((64 * (T + 1)) % B == 0 || T + 1 == ntile) flush((64 * T) / B);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
}

// ---- order metric: one workgroup per head
constexpr int kMetThreads = 1024;

__global__ __launch_bounds__(kMetThreads) void paro_metric_kernel(
    const int32_t* __restrict__ cnt, const float* __restrict__ bsum, const float* __restrict__ bmax,
    int N, int B, int sigma_num, int sigma_den, float alpha, int order, float* __restrict__ stats) {
  __shared__ int s_n[kMetThreads / kWave];
  __shared__ float s_i[kMetThreads / kWave];
  const int g = blockIdx.x, t = threadIdx.x;
  const int nb = (N + B - 1) / B;
  const int64_t nblk = static_cast<int64_t>(nb) * nb;
  const int64_t base = static_cast<int64_t>(g) * nblk;
  int nsp = 0;
  float isum = 0.0f;
  // every thread strides over the flattened nb x nb blocks (independent
  // loads, all threads busy); (i, j) follow the flat index incrementally
  const int di = kMetThreads / nb, dj = kMetThreads % nb;
  int i = t / nb, j = t % nb;
#pragma unroll 4
  for (int64_t e = t; e < nblk; e += kMetThreads) {
    const int64_t area = static_cast<int64_t>(min(B, N - i * B)) * min(B, N - j * B);
    nsp += static_cast<int64_t>(cnt[base + e]) * sigma_den >= static_cast<int64_t>(sigma_num) * area;
    const float s = bsum[base + e];
    isum += s > 0.0f ? bmax[base + e] * static_cast<float>(area) / s : 1.0f;
    i += di;
    j += dj;
    if (j >= nb) { j -= nb; i++; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    nsp += __shfl_xor(nsp, o);
    isum += __shfl_xor(isum, o);
  }
  if (t % kWave == 0) { s_n[t / kWave] = nsp; s_i[t / kWave] = isum; }
  __syncthreads();
  if (t == 0) {
    int ns = 0;
    float is = 0.0f;
    for (int w = 0; w < kMetThreads / kWave; w++) { ns += s_n[w]; is += s_i[w]; }
    const float nf = static_cast<float>(nblk);
    const float r = static_cast<float>(ns) / nf, ib = is / nf;
    float* out = stats + (static_cast<int64_t>(g) * 6 + order) * 3;
    out[0] = (1.0f - r) + alpha * ib;
    out[1] = r;
    out[2] = ib;
  }
}

__global__ void paro_select_kernel(const float* __restrict__ stats, int G, uint8_t* __restrict__ orders) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= G) return;
  int best = 0;
  float bv = stats[static_cast<int64_t>(g) * 18];
  for (int o = 1; o < 6; o++) {
    const float v = stats[(static_cast<int64_t>(g) * 6 + o) * 3];
    if (v < bv || (bv != bv && v == v)) { bv = v; best = o; }  // a NaN never wins
  }
  orders[g] = static_cast<uint8_t>(best);
}

}  // namespace

hipError_t launch_block_stats(const uint16_t* Qp, const uint16_t* Kp, int G, int N, int d, int B,
                              float sm_scale, float eps, int32_t* cnt, float* bsum, float* bmax,
                              hipStream_t s) {
  const dim3 grid((N + kStatRows - 1) / kStatRows, G);
  const float c = sm_scale * kLog2e;
  if (d == 128 && B == 64)
    block_stats_kernel<128, 64><<<grid, 256, 0, s>>>(Qp, Kp, N, c, eps, cnt, bsum, bmax);
  else if (d == 128)
    block_stats_kernel<128, 128><<<grid, 256, 0, s>>>(Qp, Kp, N, c, eps, cnt, bsum, bmax);
  else if (B == 64)
    block_stats_kernel<64, 64><<<grid, 256, 0, s>>>(Qp, Kp, N, c, eps, cnt, bsum, bmax);
  else
    block_stats_kernel<64, 128><<<grid, 256, 0, s>>>(Qp, Kp, N, c, eps, cnt, bsum, bmax);
  return hipGetLastError();
}

hipError_t launch_paro_metric(const int32_t* cnt, const float* bsum, const float* bmax, int G,
                              int N, int B, int sigma_num, int sigma_den, float alpha, int order,
                              float* stats, hipStream_t s) {
  paro_metric_kernel<<<G, kMetThreads, 0, s>>>(cnt, bsum, bmax, N, B, sigma_num, sigma_den, alpha,
                                               order, stats);
  return hipGetLastError();
}

hipError_t launch_paro_select(const float* stats, int G, uint8_t* orders, hipStream_t s) {
  paro_select_kernel<<<(G + 63) / 64, 64, 0, s>>>(stats, G, orders);
  return hipGetLastError();
}

}  // namespace bsa
