// comp.hip — first-order compensation of the skipped keys, applied to the
// output of a block-sparse forward.
//
// PASA review (pith.science, arXiv 2604.12219), Figure 2 caption: grouped
// first-order compensation for the blocks outside the selected set; the
// keys outside a query's selected set are skipped with coarse
// approximations.  The pages give neither the groups nor the expansion
// point; here the group is everything a q-block row skips.  For q-block i
// of head g, U = the real tokens of the kv-blocks not in its CSR row,
// n = |U|, kbar = sum_U k / n, Vhat = sum_U v, M = sum_U (k - kbar) v^T.  The
// first-order expansion of exp(s q.k) around kbar adds, for every real row
// r of the q-block, exp(s q_r.kbar) (Vhat + s M^T q_r) to the numerator and
// exp(s q_r.kbar) n to the denominator of its softmax (the first-order term
// of the denominator vanishes).  The forward already wrote O = num/den and
// lse = ln den of the kept blocks; the update reads them back:
//   mu  = max(lse, a + ln n),  a = s q_r.kbar
//   den = exp(lse - mu) + n exp(a - mu)
//   O'  = (O exp(lse - mu) + exp(a - mu) (Vhat + s M^T q_r)) / den,
//   lse' = mu + ln den.
//
// Four steps:
//   1. kv_moments_kernel: per kv-block j, X_j = [sum k v^T (d x d, row-major)
//      | sum k | sum v | rows | 0...], bf16, one row of length Lp;
//   2. skip_mask_kernel: S[i][j] = 1 for the kv-blocks row i skips, else 0
//      (bits, one 64-bit word per row and 64 kv-blocks; rows padded to a
//      multiple of 128, columns to one of 64, with zeros);
//   3. skip_gemm_kernel: C = S . X per head (bf16 MFMA, fp32 accumulation):
//      row i of C holds the sums over U_i, so M_i = C_kv - kbar Vhat^T (the
//      d x d block C_kv stored as bf16, the sums and the count as fp32);
//   4. apply_kernel: one workgroup per q-block, the update above.
// Step 3 is the only heavy one: 2 * nq * nk * Lp flops per head.
#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {
namespace {

#define LDS_AS __attribute__((address_space(3)))

constexpr int kCompThreads = 256;
constexpr int kTileI = 128;  // C rows (q-blocks) per GEMM workgroup
constexpr int kTileC = 128;  // C columns per GEMM workgroup
constexpr int kStageJ = 64;  // kv-block padding (the GEMM's stage)

__device__ __forceinline__ uint16_t bf16_bits(float x) { return static_cast<uint16_t>(f32_to_bf16_bits(x)); }

// 1. per kv-block moments on v_mfma_f32_32x32x16_bf16, one workgroup per
// (head, kv-block).  K and V move global -> LDS in 64-row sub-tiles with
// 16-byte buffer loads that write LDS directly (rows past N read as zero),
// chunk p of row r at p ^ (2r mod CH); both operands of
// sum_r k_r v_r^T = K^T V come out of ds_read_b64_tr_b16 (A = K^T: a lane
// holds one channel a of K over 8 rows; B = V: one channel b over the same
// 8 rows).  sum k and sum v are the same products against a bf16 ones
// operand.  Wave w takes the KV tiles w*TPW .. w*TPW+TPW-1 (32 x 32 each)
// and SPW of the 2*D/32 sum blocks (k blocks first, then v blocks).  LDS
// holds exactly the block's SUB = Bk/64 sub-tiles of K and V (32 KB at
// d = 128, Bk = 64, three workgroups per CU), and the d x d block leaves
// through the same area.
template <int D, int SUB>
__global__ __launch_bounds__(kCompThreads) void kv_moments_kernel(const uint16_t* __restrict__ K,
                                                                  const uint16_t* __restrict__ V,
                                                                  int N, int Bk, int nk, int nkp,
                                                                  int Lp, uint16_t* __restrict__ X) {
  constexpr int ROWB = 2 * D, CH = ROWB / 16, RPI = 1024 / ROWB;
  constexpr int TB = 64 * ROWB;              // bytes of a 64-row sub-tile
  constexpr int NI = TB / 1024 / 4;          // staging loads per wave per sub-tile
  constexpr int DB = D / 32;
  constexpr int TPW = DB * DB / 4, SPW = 2 * DB / 4;
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef short s8 __attribute__((ext_vector_type(8)));
  // K sub-tiles u at u * TB, V sub-tiles at (SUB + u) * TB (SUB = Bk / 64)
  __shared__ __attribute__((aligned(1024))) uint8_t kvs[2 * SUB * TB];
  auto kt = [&](int u) { return kvs + u * TB; };
  auto vt = [&](int u) { return kvs + (SUB + u) * TB; };
  const int g = blockIdx.x / nkp, j = blockIdx.x % nkp;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  uint16_t* xr = X + (static_cast<int64_t>(g) * nkp + j) * Lp;
  if (j >= nk) {
    for (int c = t; c < Lp; c += kCompThreads) xr[c] = 0;
    return;
  }
  const int r0 = j * Bk, r1 = min(N, r0 + Bk);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(K + static_cast<int64_t>(g) * N * D), 0, N * ROWB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(V + static_cast<int64_t>(g) * N * D), 0, N * ROWB, 0x00020000);
  // load q of wave w fills rows RPI*(4q + w) + lane/CH; the swizzle does not depend on q
  const int rl = RPI * w + lane / CH;
  const uint32_t voff = static_cast<uint32_t>(rl * ROWB + (((lane % CH) ^ ((2 * rl) & (CH - 1))) << 4));
  for (int u = 0; u < SUB; u++)
#pragma unroll
    for (int q = 0; q < NI; q++) {
      const uint32_t so = static_cast<uint32_t>((r0 + 64 * u + 4 * RPI * q) * ROWB);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (LDS_AS void*)(kt(u) + (4 * q + w) * 1024), 16, voff, so, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (LDS_AS void*)(vt(u) + (4 * q + w) * 1024), 16, voff, so, 0, 0);
    }
  // transposed-read offsets (channel block x: xor x << 6)
  const int rsub = (lane & 15) >> 2;
  const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int sv = (2 * (4 * h + rsub)) & (CH - 1);
  const uint32_t vread = static_cast<uint32_t>((4 * h + rsub) * ROWB + ((cl ^ sv) << 4) + (lane & 1) * 8);
  auto tr = [&](const uint8_t* base, int ks, int blk) {
    const uint32_t o = vread ^ static_cast<uint32_t>(blk << 6);
    const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s4*)(base + 16 * ks * ROWB + o));
    const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s4*)(base + (16 * ks + 8) * ROWB + o));
    return __builtin_bit_cast(bf16x8, (s8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  };
  const bf16x8 ones = __builtin_bit_cast(bf16x8, (s8){0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80});
  f32x16 kv[TPW], sm[SPW];
#pragma unroll
  for (int x = 0; x < TPW; x++) kv[x] = f32x16{};
#pragma unroll
  for (int y = 0; y < SPW; y++) sm[y] = f32x16{};
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int u = 0; u < SUB; u++)
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
#pragma unroll
      for (int x = 0; x < TPW; x++) {
        const int k = w * TPW + x, ab = k / DB, bb = k % DB;
        kv[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr(kt(u), ks, ab), tr(vt(u), ks, bb), kv[x], 0, 0, 0);
      }
#pragma unroll
      for (int y = 0; y < SPW; y++) {
        const int sb = w * SPW + y;
        if (sb < DB) sm[y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr(kt(u), ks, sb), ones, sm[y], 0, 0, 0);
        else sm[y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, tr(vt(u), ks, sb - DB), sm[y], 0, 0, 0);
      }
    }
  // KV tile: lane holds channel b = 32bb + l32 of rows a = 32ab + 8(r/4) + 4h + r%4.
  // The tiles go through LDS (over the staged K, which every wave has
  // finished reading) so that the row is written with 16-byte stores.
  static_assert(2 * SUB * TB >= D * D * 2, "the staging area holds the d x d block");
  __syncthreads();
  uint16_t* ot = reinterpret_cast<uint16_t*>(kvs);
#pragma unroll
  for (int x = 0; x < TPW; x++) {
    const int k = w * TPW + x, ab = k / DB, bb = k % DB;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int a = 32 * ab + 8 * (r / 4) + 4 * h + (r % 4);
      ot[a * D + 32 * bb + l32] = bf16_bits(kv[x][r]);
    }
  }
  // sum k (rows of the product, every column alike: column 0 writes) and
  // sum v (columns, every row alike: row slot 0 of lane half 0 writes)
#pragma unroll
  for (int y = 0; y < SPW; y++) {
    const int sb = w * SPW + y;
    if (sb < DB) {
      if (l32 == 0)
#pragma unroll
        for (int r = 0; r < 16; r++) xr[D * D + 32 * sb + 8 * (r / 4) + 4 * h + (r % 4)] = bf16_bits(sm[y][r]);
    } else if (h == 0) {
      xr[D * D + D + 32 * (sb - DB) + l32] = bf16_bits(sm[y][0]);
    }
  }
  if (t == 0) xr[D * D + 2 * D] = bf16_bits(static_cast<float>(r1 - r0));
  for (int c = D * D + 2 * D + 1 + t; c < Lp; c += kCompThreads) xr[c] = 0;
  __syncthreads();
#pragma unroll
  for (int c = t; c < D * D / 8; c += kCompThreads)
    *reinterpret_cast<uint4*>(xr + 8 * c) = *reinterpret_cast<const uint4*>(ot + 8 * c);
}

// 2. the skip mask as bits: S[g][i][j] = 1 for the kv-blocks q-block row i
// skips (padding: 0).  Word w of a row covers kv-blocks 64w .. 64w+63; its
// byte 2ks + h holds in bits 0..3 the kv-blocks 16ks + 4h + 0..3 and in
// bits 4..7 the kv-blocks 16ks + 8 + 4h + 0..3 of the word: the order in
// which the GEMM's transposing reads of X hand lane half h its k values.
__global__ __launch_bounds__(kCompThreads) void skip_mask_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t col_len,
    int mask_G, int nq, int nk, int nqp, int nkp, uint64_t* __restrict__ S) {
  extern __shared__ uint8_t srow[];  // [nkp]
  const int g = blockIdx.x / nqp, i = blockIdx.x % nqp;
  const int t = threadIdx.x;
  for (int j = t; j < nkp; j += kCompThreads) srow[j] = (i < nq && j < nk) ? 1 : 0;
  __syncthreads();
  if (i < nq) {
    const int64_t r = static_cast<int64_t>(g % mask_G) * nq + i;
    int64_t e0 = row_ptr[r], e1 = row_ptr[r + 1];
    e0 = e0 < 0 ? 0 : (e0 > col_len ? col_len : e0);
    e1 = e1 < e0 ? e0 : (e1 > col_len ? col_len : e1);
    for (int64_t e = e0 + t; e < e1; e += kCompThreads) {
      const int j = col_idx[e];
      if (static_cast<unsigned>(j) < static_cast<unsigned>(nk)) srow[j] = 0;
    }
  }
  __syncthreads();
  const int nw = nkp / 64;
  uint64_t* out = S + (static_cast<int64_t>(g) * nqp + i) * nw;
  for (int wd = t; wd < nw; wd += kCompThreads) {
    uint64_t v = 0;
#pragma unroll
    for (int by = 0; by < 8; by++) {
      const int base = 64 * wd + 16 * (by >> 1) + 4 * (by & 1);
#pragma unroll
      for (int bt = 0; bt < 8; bt++)
        v |= static_cast<uint64_t>(srow[base + (bt & 3) + 8 * (bt >> 2)]) << (8 * by + bt);
    }
    out[wd] = v;
  }
}

// 3. C[g][i][c] = sum_j S[g][i][j] X[g][j][c].  Products C^T = X^T . S^T on
// v_mfma_f32_32x32x16_bf16: A = X^T (32 columns x 16 kv-blocks), B = S^T
// (16 kv-blocks x 32 rows).  A workgroup owns 128 rows i and 128 columns c;
// each stage of 64 kv-blocks of X moves global -> LDS with 16-byte buffer
// loads that write LDS directly (double-buffered, the next stage in flight
// under the current one's products, one barrier per stage):
//   X stage: 64 x 128 (256-byte rows), chunk p of row r at
//            p ^ (2r mod 16); A operands come out of ds_read_b64_tr_b16, two
//            reads per operand, which give a lane half h the kv-blocks
//            16ks + 4h + (0..3) and 16ks + 8 + 4h + (0..3) of k-step ks;
//   S:       each lane reads its row's 64-bit word of the stage straight from
//            memory one stage ahead; the byte of its k-step and lane half
//            indexes a 256-entry LDS table of the eight bf16 0/1 values.
// Eight waves: wave w owns rows [32(w/2), +32) and columns [64(w%2), +64)
// (channel blocks 2(w%2), 2(w%2)+1): two accumulators; lane l of an
// accumulator holds row 32(w/2) + l%32 and columns cb + 8(r/4) + 4(l/32) + r%4.
// Tiles go to XCDs in contiguous ranges ordered (head, column tile, row
// tile), so the row tiles that share an X stage run together on one L2.
constexpr int kGemmJ = 64;       // kv-blocks per stage
constexpr int kXSub = 64 * 256;   // bytes of one X stage (64 rows x 128 columns)

__global__ __launch_bounds__(512, 2) void skip_gemm_kernel(const uint64_t* __restrict__ S,
                                                                    const uint16_t* __restrict__ X,
                                                                    int G, int nqp, int nkp, int Lp,
                                                                    int dd, int tiles_i, int tiles_c,
                                                                    uint16_t* __restrict__ Ckv,
                                                                    float* __restrict__ Ct) {
  __shared__ __attribute__((aligned(1024))) uint8_t xs[2][kXSub];
  __shared__ __attribute__((aligned(16))) uint4 tbl[256];  // byte v -> eight bf16 (bit e ? 1 : 0)
  int g, item;
  if (!xcd_range_tile(blockIdx.x, tiles_i * tiles_c, G, g, item)) return;
  const int tc = item / tiles_i, ti = item % tiles_i;
  const int i0 = ti * kTileI, c0 = tc * kTileC;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wr = w >> 1, wc = w & 1;  // 32-row quarter, 64-column half
  const int l32 = lane & 31, h = lane >> 5;
  if (t < 256) {
    uint32_t q[4];
#pragma unroll
    for (int e = 0; e < 4; e++)
      q[e] = ((t >> (2 * e)) & 1 ? 0x3F80u : 0u) | ((t >> (2 * e + 1)) & 1 ? 0x3F800000u : 0u);
    tbl[t] = make_uint4(q[0], q[1], q[2], q[3]);
  }
  const uint16_t* Xg = X + static_cast<int64_t>(g) * nkp * Lp;
  const int nw = nkp / kGemmJ;
  const uint64_t* Srow = S + (static_cast<int64_t>(g) * nqp + i0 + 32 * wr + l32) * nw;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Xg), 0, static_cast<int>(static_cast<int64_t>(nkp) * Lp * 2), 0x00020000);
  // staging lane offsets: X load q of wave w fills rows 32q + 4w + lane/16
  // (the swizzle depends on lane and w only)
  const uint32_t vx_ld = static_cast<uint32_t>((4 * w + (lane >> 4)) * (Lp * 2) +
                                               (((lane & 15) ^ ((8 * w + 2 * (lane >> 4)) & 15)) << 4));
  const uint32_t wb = static_cast<uint32_t>(w) * 1024u;
  auto stage = [&](int j0, int buf) {
#pragma unroll
    for (int q = 0; q < 2; q++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (LDS_AS void*)(&xs[buf][q * 8192 + wb]), 16, vx_ld,
          static_cast<uint32_t>((j0 + 32 * q) * Lp * 2 + c0 * 2), 0, 0);
  };
  // operand read offsets
  const int rsub = (lane & 15) >> 2;
  const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int sv = (2 * (4 * h + rsub)) & 15;
  const uint32_t vread = static_cast<uint32_t>((4 * h + rsub) * 256 + ((cl ^ sv) << 4) + (lane & 1) * 8);
  uint32_t ax[2];
#pragma unroll
  for (int cbk = 0; cbk < 2; cbk++) ax[cbk] = vread ^ static_cast<uint32_t>((2 * wc + cbk) << 6);
  f32x16 acc[2][1];
#pragma unroll
  for (int a = 0; a < 2; a++) acc[a][0] = f32x16{};
  const int nst = nkp / kGemmJ;
  stage(0, 0);
  uint64_t sw = Srow[0];
  for (int st = 0; st < nst; st++) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const uint64_t cur = sw;
    if (st + 1 < nst) {
      stage((st + 1) * kGemmJ, (st + 1) & 1);
      sw = Srow[st + 1];
    }
    const uint8_t* xt = xs[st & 1];
#pragma unroll
    for (int ks = 0; ks < kGemmJ / 16; ks++) {
      bf16x8 a[2];
#pragma unroll
      for (int cbk = 0; cbk < 2; cbk++) {
        typedef short s4 __attribute__((ext_vector_type(4)));
        const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s4*)(xt + 16 * ks * 256 + ax[cbk]));
        const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s4*)(xt + (16 * ks + 8) * 256 + ax[cbk]));
        a[cbk] = __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){
                                                lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
      const uint32_t half = ks < 2 ? static_cast<uint32_t>(cur) : static_cast<uint32_t>(cur >> 32);
      const uint32_t idx = (half >> (8 * ((2 * ks + h) & 3))) & 0xFFu;
      const bf16x8 b = __builtin_bit_cast(bf16x8, tbl[idx]);
#pragma unroll
      for (int cbk = 0; cbk < 2; cbk++)
        acc[cbk][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cbk], b, acc[cbk][0], 0, 0, 0);
    }
  }
  // C's d x d block is stored as bf16 (it becomes the bf16 M^T operand of the
  // update), the sums and the count as fp32; a tile lies wholly on one side
  const int i = i0 + 32 * wr + l32;
  const int64_t row = static_cast<int64_t>(g) * nqp + i;
  const int Lt = Lp - dd;
#pragma unroll
  for (int cbk = 0; cbk < 2; cbk++)
#pragma unroll
    for (int r4 = 0; r4 < 4; r4++) {
      const int c = c0 + 64 * wc + 32 * cbk + 8 * r4 + 4 * h;
      const float v[4] = {acc[cbk][0][4 * r4], acc[cbk][0][4 * r4 + 1], acc[cbk][0][4 * r4 + 2],
                          acc[cbk][0][4 * r4 + 3]};
      if (c0 < dd) {
        uint2 pk;
        pk.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
        pk.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
        *reinterpret_cast<uint2*>(Ckv + row * dd + c) = pk;
      } else {
        *reinterpret_cast<float4*>(Ct + row * Lt + (c - dd)) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
}

// 4. the update of O and lse, one workgroup per (head, q-block); wave w
// owns rows 32w..32w+31 (lane l and l+32 share row 32w + l%32).
//   a. every read of C first (the d x d block: thread t takes the 8 x 1
//      column pieces e = t + 256k; the sums of k and v; the skipped count),
//      and the wave's Q fragments (the A operand of step d);
//   b. M^T (bf16, [b][a]) into LDS: M[a][b] = C_kv[a][b] - kbar_a Vhat_b;
//   c. per row, from the Q fragments: a = s q.kbar, the old and new terms'
//      weights divided by the new denominator, the new lse;
//   d. Y^T = M^T Q_i^T on v_mfma_f32_32x32x16_bf16 (A = M^T rows from LDS,
//      B = the Q fragments); lane l of accumulator bb holds row 32w + l%32
//      and channels 32bb + 8(r/4) + 4(l/32) + r%4;
//   e. O' = O w_old + w_new (Vhat + s y), written where the forward wrote O,
//      four consecutive channels of the lane's own row per 8-byte access
//      (every old value is read before the first store).
template <int D>
__global__ __launch_bounds__(kCompThreads, 3) void apply_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Ckv, const float* __restrict__ Ct,
    int N, int Bq, int nq, int nqp, int Lt, float sm, uint16_t* __restrict__ O, float* __restrict__ lse,
    OutMap om) {
  constexpr int NB = D / 32;      // 32-channel blocks of the output
  constexpr int KS = D / 16;      // k-steps of Y = Q M
  constexpr int PM = D + 8;       // bf16 per LDS row of M^T
  __shared__ __attribute__((aligned(16))) float kbar[D];
  __shared__ __attribute__((aligned(16))) float vhat[D];
  __shared__ __attribute__((aligned(16))) uint16_t mt[D][PM];
  __shared__ float w_old[128], w_new[128];
  __shared__ int64_t row_off[128];  // element offset of each row's output
  const int g = blockIdx.x / nq, i = blockIdx.x % nq;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const uint16_t* Ci = Ckv + (static_cast<int64_t>(g) * nqp + i) * D * D;  // sums over U of k v^T
  const float* Cs = Ct + (static_cast<int64_t>(g) * nqp + i) * Lt;          // sum k, sum v, count
  const int r0 = i * Bq, nr = min(Bq, N - r0);
  const uint16_t* Qi = Q + (static_cast<int64_t>(g) * N + r0) * D;
  const int rb = 32 * w, qrow = rb + l32;
  // a. reads
  constexpr int KM = D * (D / 8) / kCompThreads;
  uint16_t cm[KM][8];
#pragma unroll
  for (int k = 0; k < KM; k++) {
    const int e = t + kCompThreads * k, b = e % D, a0 = 8 * (e / D);
#pragma unroll
    for (int q = 0; q < 8; q++) cm[k][q] = Ci[(a0 + q) * D + b];
  }
  const float sums = t < 2 * D ? Cs[t] : 0.0f;
  const float n = Cs[2 * D];
  uint4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ks++) {
    qf[ks] = make_uint4(0u, 0u, 0u, 0u);
    if (qrow < nr) qf[ks] = *reinterpret_cast<const uint4*>(Qi + static_cast<int64_t>(qrow) * D + 16 * ks + 8 * h);
  }
  if (!(n > 0.5f)) return;  // nothing skipped (the same for the whole workgroup): O and lse stay
  if (t < D) kbar[t] = sums / n;
  else if (t < 2 * D) vhat[t - D] = sums;
  __syncthreads();
  // b. M^T into LDS, 8 consecutive a per 16-byte write
#pragma unroll
  for (int k = 0; k < KM; k++) {
    const int e = t + kCompThreads * k, b = e % D, a0 = 8 * (e / D);
    const float vb = vhat[b];
    uint32_t pk[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const float m0 = bf16_bits_to_f32(cm[k][2 * q]) - kbar[a0 + 2 * q] * vb;
      const float m1 = bf16_bits_to_f32(cm[k][2 * q + 1]) - kbar[a0 + 2 * q + 1] * vb;
      pk[q] = f32_to_bf16_bits(m0) | (f32_to_bf16_bits(m1) << 16);
    }
    *reinterpret_cast<uint4*>(&mt[b][a0]) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
  // c. per-row weights and the new lse: this lane's half of q.kbar (channels
  // 16ks + 8h .. +7), the halves added across the wave
  if (rb < nr) {
    float part = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      const uint32_t wv[4] = {qf[ks].x, qf[ks].y, qf[ks].z, qf[ks].w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        part = __builtin_fmaf(bf16_bits_to_f32(wv[e] & 0xFFFFu), kbar[16 * ks + 8 * h + 2 * e], part);
        part = __builtin_fmaf(bf16_bits_to_f32(wv[e] >> 16), kbar[16 * ks + 8 * h + 2 * e + 1], part);
      }
    }
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    const float a = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * sm;
    if (h == 0 && qrow < nr) {
      int64_t li;
      row_off[qrow] = out_row<D>(O, om.orders, om.F, om.H, om.W, om.sg, om.sn, g, N, r0 + qrow, li) - O;
      const float lo = lse[li];
      const float mu = fmaxf(lo, a + logf(n));
      const float wo = lo > -INFINITY ? expf(lo - mu) : 0.0f;
      const float wc = expf(a - mu);
      const float den = wo + wc * n;
      w_old[qrow] = wo / den;
      w_new[qrow] = wc / den;
      lse[li] = mu + logf(den);  // only this lane touches lse[li]
    }
  }
  __syncthreads();
  if (rb >= nr) return;  // no later barrier
  // d. Y^T = M^T Q_i^T for the wave's 32 rows: lane l of accumulator bb holds
  // query row rb + l%32 and channels 32bb + 8(r/4) + 4(l/32) + r%4, so each
  // lane updates four consecutive channels of its own row per (bb, r/4)
  f32x16 acc[NB];
#pragma unroll
  for (int bb = 0; bb < NB; bb++) acc[bb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ks++) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, qf[ks]);
#pragma unroll
    for (int bb = 0; bb < NB; bb++) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&mt[32 * bb + l32][16 * ks + 8 * h]);
      acc[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[bb], 0, 0, 0);
    }
  }
  // e. the update, 8-byte reads and writes of this lane's row
  if (qrow < nr) {
    const float wo = w_old[qrow], wn = w_new[qrow];
    uint16_t* op = O + row_off[qrow];
    uint2 old[NB][4];  // every old value first (the stores below could alias them as far as the compiler knows)
#pragma unroll
    for (int bb = 0; bb < NB; bb++)
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) old[bb][r4] = *reinterpret_cast<const uint2*>(op + 32 * bb + 8 * r4 + 4 * h);
#pragma unroll
    for (int bb = 0; bb < NB; bb++)
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) {
        const int b0 = 32 * bb + 8 * r4 + 4 * h;
        const uint2 ov = old[bb][r4];
        const float4 vh = *reinterpret_cast<const float4*>(&vhat[b0]);
        const float y0 = __builtin_fmaf(sm, acc[bb][4 * r4 + 0], vh.x);
        const float y1 = __builtin_fmaf(sm, acc[bb][4 * r4 + 1], vh.y);
        const float y2 = __builtin_fmaf(sm, acc[bb][4 * r4 + 2], vh.z);
        const float y3 = __builtin_fmaf(sm, acc[bb][4 * r4 + 3], vh.w);
        uint2 nv;
        nv.x = f32_to_bf16_bits(__builtin_fmaf(bf16_bits_to_f32(ov.x & 0xFFFFu), wo, wn * y0)) |
               (f32_to_bf16_bits(__builtin_fmaf(bf16_bits_to_f32(ov.x >> 16), wo, wn * y1)) << 16);
        nv.y = f32_to_bf16_bits(__builtin_fmaf(bf16_bits_to_f32(ov.y & 0xFFFFu), wo, wn * y2)) |
               (f32_to_bf16_bits(__builtin_fmaf(bf16_bits_to_f32(ov.y >> 16), wo, wn * y3)) << 16);
        *reinterpret_cast<uint2*>(op + b0) = nv;
      }
  }
}

int round_up(int x, int m) { return (x + m - 1) / m * m; }

}  // namespace

FoLayout fo_layout(int G, int N, int d, int Bq, int Bk) {
  FoLayout L{};
  L.nq = (N + Bq - 1) / Bq;
  L.nk = (N + Bk - 1) / Bk;
  L.nqp = round_up(L.nq, kTileI);
  L.nkp = round_up(L.nk, kStageJ);
  L.Lp = round_up(d * d + 2 * d + 1, kTileC);
  L.gemm_tiles = static_cast<int64_t>(G) * (L.nqp / kTileI) * (L.Lp / kTileC);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) & ~static_cast<size_t>(255);
    return o;
  };
  L.x = take(sizeof(uint16_t) * static_cast<size_t>(G) * L.nkp * L.Lp);
  L.s = take(static_cast<size_t>(G) * L.nqp * (L.nkp / 64) * sizeof(uint64_t));
  L.Lt = L.Lp - d * d;
  L.ckv = take(sizeof(uint16_t) * static_cast<size_t>(G) * L.nqp * d * d);
  L.ct = take(sizeof(float) * static_cast<size_t>(G) * L.nqp * L.Lt);
  L.total = off;
  return L;
}

hipError_t launch_fo_compensate(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                const int32_t* row_ptr, const int32_t* col_idx, int64_t col_len,
                                int mask_G, int G, int N, int d, int Bq, int Bk, float sm_scale,
                                uint16_t* O, float* lse, const OutMap& om, char* ws,
                                hipStream_t s) {
  const FoLayout L = fo_layout(G, N, d, Bq, Bk);
  auto* X = reinterpret_cast<uint16_t*>(ws + L.x);
  auto* S = reinterpret_cast<uint64_t*>(ws + L.s);
  auto* Ckv = reinterpret_cast<uint16_t*>(ws + L.ckv);
  auto* Ct = reinterpret_cast<float*>(ws + L.ct);
  const float sm = sm_scale > 0.0f ? sm_scale : 1.0f / sqrtf(static_cast<float>(d));
  const uint32_t gm = static_cast<uint32_t>(G) * L.nkp;
  if (d == 128 && Bk == 64) kv_moments_kernel<128, 1><<<gm, kCompThreads, 0, s>>>(K, V, N, Bk, L.nk, L.nkp, L.Lp, X);
  else if (d == 128) kv_moments_kernel<128, 2><<<gm, kCompThreads, 0, s>>>(K, V, N, Bk, L.nk, L.nkp, L.Lp, X);
  else if (Bk == 64) kv_moments_kernel<64, 1><<<gm, kCompThreads, 0, s>>>(K, V, N, Bk, L.nk, L.nkp, L.Lp, X);
  else kv_moments_kernel<64, 2><<<gm, kCompThreads, 0, s>>>(K, V, N, Bk, L.nk, L.nkp, L.Lp, X);
  skip_mask_kernel<<<static_cast<uint32_t>(G) * L.nqp, kCompThreads, L.nkp, s>>>(
      row_ptr, col_idx, col_len, mask_G, L.nq, L.nk, L.nqp, L.nkp, S);
  const int ti = L.nqp / kTileI, tc = L.Lp / kTileC;
  const uint32_t ng = kNumXcd * static_cast<uint32_t>((L.gemm_tiles + kNumXcd - 1) / kNumXcd);
  skip_gemm_kernel<<<ng, 512, 0, s>>>(S, X, G, L.nqp, L.nkp, L.Lp, d * d, ti, tc, Ckv, Ct);
  const uint32_t ga = static_cast<uint32_t>(G) * L.nq;
  if (d == 128)
    apply_kernel<128><<<ga, kCompThreads, 0, s>>>(Q, Ckv, Ct, N, Bq, L.nq, L.nqp, L.Lt, sm, O, lse, om);
  else
    apply_kernel<64><<<ga, kCompThreads, 0, s>>>(Q, Ckv, Ct, N, Bq, L.nq, L.nqp, L.Lt, sm, O, lse, om);
  return hipGetLastError();
}

}  // namespace bsa
