// attn.hip — INT8 block-sparse flash attention forward for gfx950, and the
// debug entry points exposing its integer tile routines.
//
// SPADE machine verdict (pith.science, arXiv 2608.03335), key machinery: a
// flash-style block-sparse kernel with online softmax computes only the
// kept blocks; referee minor comment on §2.2 Eq. (2): the block mask is
// additive (0 kept, -inf pruned).  PAROAttention machine verdict
// (pith.science, arXiv 2506.16054), key machinery and core discovery: the
// INT8 variant runs Q.K^T in INT8 and quantises the post-softmax map to
// INT8, with quantisation blocks equal to the attention blocks.
//
// Per kept tile (q-block i, kv-block j), in CSR order, for every row r:
//   I   = q8 . k8 (exact int32),  x = I * sQ_i * sK_j * sm_scale * log2(e)
//   m'  = max(m, max_c x),  Pt = 2^(x - m'),  l = l * 2^(m - m') + sum_c Pt
//   mP  = max of Pt over the tile's real rows and columns (whole workgroup)
//   P8  = rint(Pt * 127 / mP) in [0, 127]
//   acc = acc * 2^(m - m') + (mP / 127) * sV_j * (P8 . v8) (exact int32)
// and O = acc / l, LSE = (m + log2 l) * ln 2.  The integer tile product
// reaches acc through a biased fp32 read (see kPBias).
//
// Work split: one workgroup per (head g, q-block i); Bq/32 waves of 32 query
// rows; XCD x runs a contiguous range of the head-major (head, q-block) tiles
// (its L2 serves one head's INT8 K/V at a time).  Two workgroups per CU put two waves on every SIMD, so one wave's
// v_mfma_i32_32x32x32_i8 products run under the other's softmax, quantising
// and rescaling work (each wave needs at most 256 registers).  A tile is one
// kv-block (the quantisation unit of P).
//   S^T = K . Q^T     A = K rows from LDS (ds_read_b128), B = Q fragments in
//                     registers; the accumulator gives every lane one query
//                     row (the two wave halves share a row): lane half h, slot
//                     s of a 32-column group holds kv 8(s/4) + 4h + s%4.
//   O^T += V^T . P8^T A = V^T read by ds_read_b64_tr_b8 (a 16-lane group
//                     reads an 8-row x 16-column byte block and hands every
//                     lane its column's 8 rows), B = P8 packed in registers.
//                     V rows are permuted within each 32-row block on their
//                     way into LDS so that the two transposed reads of a lane
//                     half return exactly the kv indices its P8 slots carry.
// K and V move global -> LDS with 16-byte buffer loads that write LDS
// directly; chunk c of LDS row r sits at c ^ ((r / (16/CH)) mod CH) (CH
// chunks per row), which keeps the K and V operand reads conflict-free.  Rows
// past N read as zero through the buffer range check; their columns are
// masked.  K is triple- and V double-buffered so one barrier per tile covers
// both the staging hand-off and the workgroup-wide maximum of Pt.
#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {
namespace {

typedef int i32x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2_127 = 6.988684686772166f;
// Score bias: the forward's Q.K^T accumulators start at the bit pattern of
// 1.5 * 2^23.  Every |q8.k8| <= 127^2 * 128 < 2^22, so the int32 result,
// read as an fp32, is exactly 1.5 * 2^23 + q8.k8: the scores reach the
// VALU as floats without a conversion, and the offset folds into the
// exponent's fma.
constexpr int kSBias = 0x4B400000;
constexpr float kSBiasF = 12582912.0f;
constexpr float kRefInit = -1.0e30f;  // running maximum before any score: finite, below all
// Largest score scale f (log2 units per integer score unit) for the biased
// exponent: bias*f < 1.5*2^12, so the folded offset is rounded by at most
// 2^-12 (log2 units) and y = Pt*127/mP stays below 127.02 (code <= 127).
constexpr float kNarrowF = 0x1p-11f;
// O and l follow the running row maximum lazily: their reference moves only
// when the maximum has risen more than this (log2 units) above it, so the
// per-tile contributions carry a factor of at most 2^kLazy
constexpr float kLazy = 8.0f;
// Product bias: each tile's P8.V8 products start from the bit pattern of
// 2^23 + 2^20 (Bk = 64) or 2^23 + 2^21 (Bk = 128); every |p8.v8| over the
// tile is below 2^20 (2^21), so the int32 result read as an fp32 is exactly
// that bias plus the integer product and enters O's fma without a
// conversion.  O then carries bias * (the tile's scale) per tile, the same
// for every element of a row; a per-row scalar keeps that offset and is
// taken out of O every kFold tiles, so the offset never exceeds kFold tiles'
// worth (each fma rounds at most ulp(|O| + kFold * bias * scale) / 2).
template <int BK>
constexpr int kPBias = BK == 64 ? 0x4B100000 : 0x4B200000;
template <int BK>
constexpr float kPBiasF = BK == 64 ? 9437184.0f : 10485760.0f;
static_assert(64 * 127 * 127 < (1 << 20) && 128 * 127 * 127 < (1 << 21), "product range of a tile");
constexpr int kFold = 4;
// 32-row halves per wave: one, so a 128-row q-block is four waves and two
// workgroups give every SIMD two waves whose products and softmax interleave
constexpr int kQB = 1;
constexpr int kRowsPerWave = 32 * kQB;

// accumulator row of element r for lane half h (32x32 MFMA tiles)
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <int D, int BK, int NW>
struct L8 {
  static constexpr int ROWB = D;                 // bytes per K / V row
  static constexpr int CH = D / 16;              // 16-byte chunks per row
  static constexpr int SROW = 16 / CH;           // rows per 256-byte bank line
  static constexpr int TB = BK * D;              // bytes per tile
  static constexpr int NI = TB / 1024 / NW;      // 1 KB staging loads per wave per tile
  // staging lane offsets repeat every P loads (32 rows: the V row permutation)
  static constexpr int P0 = 32 * ROWB / (NW * 1024);
  static constexpr int P = P0 < 1 ? 1 : (P0 > NI ? NI : P0);
  static_assert(NI >= 1, "tile too small for the staging loads");
  // stage one tile (kv rows kv0 .. kv0+BK) of K or V (one head: base, nrec
  // bytes; rows past the end read as zero) into LDS; offs: the matching lane
  // offsets (Stage8::k or Stage8::v)
  static __device__ __forceinline__ void stage(const int8_t* base, int nrec, const uint32_t* offs,
                                               int kv0, uint8_t* tile) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(base), 0, nrec, 0x00020000);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int q = 0; q < NI; q++) {
      const uint32_t soff = static_cast<uint32_t>(kv0 * ROWB + (q / P) * P * NW * 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(tile + (q * NW + w) * 1024),
                                               16, offs[q % P], soff, 0, 0);
    }
  }
};

// chunk swizzle of LDS row r
template <int D>
__device__ __forceinline__ int swz(int r) {
  return (r / (16 / (D / 16))) % (D / 16);
}

// LDS row p of a V tile holds kv row sigma(p): within each 32-row block,
// LDS rows 8q..8q+7 hold kv {0-3, 8-11} + 16(q%2) + 4(q/2).
__device__ __forceinline__ int sigma(int p) {
  const int q = (p >> 3) & 3, e = p & 7;
  return (p & ~31) | (16 * (q & 1) + 4 * (q >> 1) + 8 * (e >> 2) + (e & 3));
}

// Lane offsets of the staging loads: load q of wave w writes LDS bytes
// [(q*NW + w)*1024, +1024), lane l the 16 bytes at +16l: LDS row p, physical
// chunk x, which hold logical chunk x ^ swz(p) of source row p (K) or
// sigma(p) (V).  Offsets repeat every P loads up to a shift of P*NW*1024.
template <int D, int BK, int NW>
struct Stage8 {
  using L = L8<D, BK, NW>;
  uint32_t k[L::P], v[L::P];
  __device__ __forceinline__ void init() {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < L::P; q++) {
      const int o = (q * NW + w) * 1024 + 16 * lane;
      const int p = o / L::ROWB, x = (o % L::ROWB) / 16;
      const int c = x ^ swz<D>(p);
      k[q] = static_cast<uint32_t>(p * L::ROWB + 16 * c);
      v[q] = static_cast<uint32_t>(sigma(p) * L::ROWB + 16 * c);
    }
  }
};

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// LDS read offsets of this lane's operands
template <int D>
__device__ __forceinline__ void k_offsets(uint32_t (&kx)[D / 32]) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
  const uint32_t base = static_cast<uint32_t>(l32 * D + ((h ^ swz<D>(l32)) << 4));
#pragma unroll
  for (int ks = 0; ks < D / 32; ks++) kx[ks] = base ^ (ks << 5);
}
template <int D>
__device__ __forceinline__ uint32_t v_read_off() {
  const int lane = threadIdx.x & 63, li = lane & 15, grp = lane >> 4, h = lane >> 5;
  const int row = 16 * h + (li >> 1);
  return static_cast<uint32_t>(row * D + (((grp & 1) ^ swz<D>(row)) << 4) + (li & 1) * 8);
}

// S^T = K . Q^T for the wave's two row halves: s[qb][b] covers kv 32b..32b+31
template <int D, int BK, int BIAS = 0>
__device__ __forceinline__ void qk_i8(const uint8_t* kt, const uint32_t (&kx)[D / 32],
                                      const i32x4 (&qf)[kQB][D / 32], i32x16 (&s)[kQB][BK / 32]) {
#pragma unroll
  for (int b = 0; b < BK / 32; b++)
#pragma unroll
    for (int qb = 0; qb < kQB; qb++) s[qb][b] = BIAS;
#pragma unroll
  for (int ks = 0; ks < D / 32; ks++)
#pragma unroll
    for (int b = 0; b < BK / 32; b++) {
      const i32x4 a = *reinterpret_cast<const i32x4*>(kt + b * 32 * D + kx[ks]);
#pragma unroll
      for (int qb = 0; qb < kQB; qb++)
        s[qb][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[qb][ks], s[qb][b], 0, 0, 0);
    }
}

// One channel block of O^T (int32, this tile only) = V^T . P8^T for the
// wave's row halves: ov[qb] covers channels 32db..32db+31 of half qb.  The
// first product takes its accumulator from acc0, a register block that holds
// its start value for the whole kernel (zeros, or the forward's product
// bias; the product writes ov, not acc0), so no per-tile clearing of ov is
// issued.
template <int D, int BK>
__device__ __forceinline__ void pv_block(const uint8_t* vt, uint32_t vread, const i32x4 (&pf)[kQB][BK / 32],
                                         int db, const i32x16& acc0, i32x16 (&ov)[kQB]) {
  const uint32_t vhi = (vread ^ ((D / 32) << 4)) + 8 * D;  // rows +8: the swizzle flips CH/2
#pragma unroll
  for (int b = 0; b < BK / 32; b++) {
    const i32x2 lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (LDS_AS i32x2*)(vt + b * 32 * D + (vread ^ (db << 5))));
    const i32x2 hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (LDS_AS i32x2*)(vt + b * 32 * D + (vhi ^ (db << 5))));
    const i32x4 a = (i32x4){lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
    for (int qb = 0; qb < kQB; qb++)
      ov[qb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, pf[qb][b], b == 0 ? acc0 : ov[qb], 0, 0, 0);
  }
}

// Q fragments of the wave's rows qbase + 32qb + l32: k-step ks holds channels
// 32ks + 16h .. +15 (rows past N read as zero)
template <int D>
__device__ __forceinline__ void load_q(const int8_t* __restrict__ Q, int g, int qbase, int N,
                                       i32x4 (&qf)[kQB][D / 32]) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int qb = 0; qb < kQB; qb++) {
    const int row = qbase + 32 * qb + l32;
    const bool ok = row < N;
    const int8_t* p = Q + (static_cast<int64_t>(g) * N + (ok ? row : 0)) * D + 16 * h;
#pragma unroll
    for (int ks = 0; ks < D / 32; ks++) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (ok) v = *reinterpret_cast<const uint4*>(p + 32 * ks);
      qf[qb][ks] = __builtin_bit_cast(i32x4, v);
    }
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  // every lane has a source under the controls used here; bound_ctrl lets
  // the move fold into the consuming v_max_f32 as its DPP operand
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
// max over the 32 rows of a wave (lanes l and l + 32 carry the same row), in
// VALU cross-lane moves only: within quads, 8-lane and 16-lane rows by DPP,
// then the two 16-lane rows of each half by permlane16_swap
__device__ __forceinline__ float rows_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(x));  // row_mirror
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// P8 = rint(Pt * 127 / mP) for the wave's rows (mP = 2^dm, the tile maximum
// of Pt), l += lsc * sum y (lsc = mP/127 times the row's frame factor: l
// sums Pt).  The exponential argument folds the quantisation scale in:
// y = Pt * 127 / mP = 2^(x - m - dm + log2 127).
// MASK: columns outside the tile and a tile without real rows give zero.
// WIDE: a score scale f above kNarrowF, where the biased fp32 score would
// lose too many bits of the offset bias*f (an exponent error of ulp(bias*f)/2
// could lift the tile maximum's y past 127.5 and its code to 128, which the
// signed MFMA reads as -128); the integer score is converted exactly instead,
// and y is clamped to 127 so the code stays in [0, 127] for any input.
template <bool MASK, bool WIDE, int NB>
__device__ __forceinline__ void quantize_tile(const i32x16 (&s)[kQB][NB], float f, const float (&m)[kQB],
                                              float dm, bool any, int kv0, bool jvalid, int N,
                                              const float (&lsc)[kQB], float (&l)[kQB],
                                              i32x4 (&pf)[kQB][NB]) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int qb = 0; qb < kQB; qb++) {
    // exponent (q8.k8) * f - off.  Narrow: the score read as biased fp32,
    // fma(score, f, -(off + bias * f)), one rounding of the folded offset.
    // Wide: fma(float(q8.k8), f, -off), the integer converted exactly.
    const float off0 = any ? m[qb] + dm - kLog2_127 : 0.0f;
    const float off = WIDE ? off0 : __builtin_fmaf(kSBiasF, f, off0);
    float ys = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; b++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const int r = 4 * q4 + e;
          float y;
          if constexpr (WIDE) {
            y = __builtin_amdgcn_exp2f(
                __builtin_fmaf(static_cast<float>(s[qb][b][r] - kSBias), f, -off));
            y = fminf(y, 127.0f);
          } else {
            y = __builtin_amdgcn_exp2f(__builtin_fmaf(__int_as_float(s[qb][b][r]), f, -off));
          }
          if constexpr (MASK) {
            const int kv = kv0 + 32 * b + acc_row(r, h);
            if (!any || !jvalid || kv >= N) y = 0.0f;
          }
          ys = b == 0 && r == 0 ? y : ys + y;
          // v_cvt_pk_u8_f32 rounds half to even (checked against rintf on
          // every quarter step of 0..255 and next to every .5)
          word = __builtin_amdgcn_cvt_pk_u8_f32(y, e, word);
        }
        pf[qb][b][q4] = static_cast<int>(word);
      }
    l[qb] = __builtin_fmaf(ys, lsc[qb], l[qb]);
  }
}

template <int D, int BQ, int BK>
__global__ __launch_bounds__(BQ / kRowsPerWave * kWave) void fwd_i8_kernel(
    const int8_t* __restrict__ Q, const float* __restrict__ sQ, const int8_t* __restrict__ K,
    const float* __restrict__ sK, const int8_t* __restrict__ V, const float* __restrict__ sV,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t col_len,
    int mask_G, uint16_t* __restrict__ O, float* __restrict__ lse, int G, int N, int nq, int nk,
    float scale_log2, OutMap om) {
  constexpr int NW = BQ / kRowsPerWave;
  constexpr int NB = BK / 32;
  using L = L8<D, BK, NW>;
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf[3][L::TB];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf[2][L::TB];
  __shared__ float tile_max[2][NW];

  int g, i;
  if (!xcd_range_tile(blockIdx.x, nq, G, g, i)) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int qbase = i * BQ + w * kRowsPerWave;

  Stage8<D, BK, NW> sg;
  sg.init();
  const uint32_t vread = v_read_off<D>();
  uint32_t kx[D / 32];  // this lane's K operand offsets, one per k-step
  k_offsets<D>(kx);

  i32x4 qf[kQB][D / 32];
  load_q<D>(Q, g, qbase, N, qf);
  const float sq = sQ[static_cast<int64_t>(g) * nq + i] * scale_log2;

  int64_t e0 = row_ptr[static_cast<int64_t>(g % mask_G) * nq + i];
  int64_t e1 = row_ptr[static_cast<int64_t>(g % mask_G) * nq + i + 1];
  e0 = e0 < 0 ? 0 : (e0 > col_len ? col_len : e0);
  e1 = e1 < e0 ? e0 : (e1 > col_len ? col_len : e1);
  const int nt = static_cast<int>(e1 - e0);

  const int head_bytes = N * L::ROWB;
  const int8_t* kh = K + static_cast<int64_t>(g) * N * D;
  const int8_t* vh = V + static_cast<int64_t>(g) * N * D;
  // kv-block index of tile t (0 past the list), its first row (0 when out of range)
  auto col_of = [&](int t) { return t < nt ? col_idx[e0 + t] : 0; };
  auto kv0_of = [&](int j) { return static_cast<unsigned>(j) < static_cast<unsigned>(nk) ? j * BK : 0; };

  // m: the exact running row maximum (the P quantisation is relative to
  // it); O and l are kept relative to an older reference mf <= m and only
  // moved to the running maximum when it has risen more than kLazy above mf
  float m[kQB], mf[kQB], l[kQB], pend[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; qb++) { m[qb] = kRefInit; mf[qb] = kRefInit; l[qb] = 0.0f; pend[qb] = 0.0f; }
  i32x16 pacc;
#pragma unroll
  for (int r = 0; r < 16; r++) pacc[r] = kPBias<BK>;
  asm volatile("" : "+v"(pacc));  // the product bias kept in registers (see pv_block)
  f32x16 o[kQB][D / 32];
#pragma unroll
  for (int qb = 0; qb < kQB; qb++)
#pragma unroll
    for (int db = 0; db < D / 32; db++) o[qb][db] = f32x16{};

  if (nt > 0) {
    // prologue: K(0), K(1), V(0)
    // indices of tiles t, t+1, t+2 and the scales of tile t, each read one
    // tile before its use so no scalar load is waited on inside a tile
    int j0 = col_of(0), j1 = col_of(1), j2 = col_of(2);
    auto sk_of = [&](int j) {
      return static_cast<unsigned>(j) < static_cast<unsigned>(nk) ? sK[static_cast<int64_t>(g) * nk + j] : 0.0f;
    };
    auto sv_of = [&](int j) {
      return static_cast<unsigned>(j) < static_cast<unsigned>(nk) ? sV[static_cast<int64_t>(g) * nk + j] : 0.0f;
    };
    float sk0 = sk_of(j0), sv0 = sv_of(j0);
    L::stage(kh, head_bytes, sg.k, kv0_of(j0), kbuf[0]);
    if (nt > 1) L::stage(kh, head_bytes, sg.k, kv0_of(j1), kbuf[1]);
    L::stage(vh, head_bytes, sg.v, kv0_of(j0), vbuf[0]);
    wait_loads();
    __syncthreads();
    int kb = 0;  // K buffer of tile t (t mod 3)
    for (int t = 0; t < nt; t++) {
      const int j = j0;
      const bool jvalid = static_cast<unsigned>(j) < static_cast<unsigned>(nk);
      const int kv0 = jvalid ? j * BK : 0;
      const bool masked = !jvalid || kv0 + BK > N;
      const float f = sq * sk0, svj = sv0;
      // next tile's scales and the index of tile t+3, consumed one tile later
      const int j3 = col_of(t + 3);
      const float sk1 = sk_of(j1), sv1 = sv_of(j1);

      // ---- scores and the exact running maximum of every row
      i32x16 s[kQB][NB];
      qk_i8<D, BK, kSBias>(kbuf[kb], kx, qf, s);
      float x_max[kQB];
      if (!masked) {
#pragma unroll
        for (int qb = 0; qb < kQB; qb++) {
          int im = s[qb][0][0];
#pragma unroll
          for (int b = 0; b < NB; b++)
#pragma unroll
            for (int r = 0; r < 16; r++) im = im > s[qb][b][r] ? im : s[qb][b][r];
          const auto sw = __builtin_amdgcn_permlane32_swap(im, im, false, false);
          im = static_cast<int>(sw[0]) > static_cast<int>(sw[1]) ? static_cast<int>(sw[0])
                                                                 : static_cast<int>(sw[1]);
          x_max[qb] = static_cast<float>(im - kSBias) * f;
        }
      } else {
#pragma unroll
        for (int qb = 0; qb < kQB; qb++) {
          float xm = -INFINITY;
#pragma unroll
          for (int b = 0; b < NB; b++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
              const int kv = kv0 + 32 * b + acc_row(r, h);
              if (jvalid && kv < N) xm = fmaxf(xm, static_cast<float>(s[qb][b][r] - kSBias) * f);
            }
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(xm), __float_as_uint(xm),
                                                           false, false);
          x_max[qb] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
      }
      float dmax = -INFINITY;
      bool resc = false;
#pragma unroll
      for (int qb = 0; qb < kQB; qb++) {
        const float mn = fmaxf(m[qb], x_max[qb]);
        m[qb] = mn;
        resc = resc || mn - mf[qb] > kLazy;
        // largest log2 Pt of this row in the tile (real rows only)
        if (qbase + 32 * qb + l32 < N) dmax = fmaxf(dmax, x_max[qb] - mn);
      }
      // the running maximum rose far above the reference of O and l: move
      // them to it (rows that did not rise keep factor 1)
      if (__ballot(resc) != 0ull) {
#pragma unroll
        for (int qb = 0; qb < kQB; qb++) {
          const bool up = m[qb] - mf[qb] > kLazy;
          const float alpha = up ? __builtin_amdgcn_exp2f(mf[qb] - m[qb]) : 1.0f;
          mf[qb] = up ? m[qb] : mf[qb];
          l[qb] *= alpha;
          pend[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; db++)
#pragma unroll
            for (int r = 0; r < 16; r++) o[qb][db][r] *= alpha;
        }
      }
      dmax = rows_max(dmax);
      if (lane == 0) tile_max[t & 1][w] = dmax;

      // ---- hand-off: this tile's V and the next K are in LDS, the tile
      // maximum of every wave is visible
      wait_loads();
      __syncthreads();
      if (t + 2 < nt) L::stage(kh, head_bytes, sg.k, kv0_of(j2), kbuf[kb == 0 ? 2 : kb - 1]);
      if (t + 1 < nt) L::stage(vh, head_bytes, sg.v, kv0_of(j1), vbuf[(t + 1) & 1]);
      float dm = tile_max[t & 1][0];
#pragma unroll
      for (int ww = 1; ww < NW; ww++) dm = fmaxf(dm, tile_max[t & 1][ww]);

      // ---- P8 = rint(Pt * 127 / mP), mP = 2^dm; l sums Pt = y * mP / 127,
      // expressed relative to mf: times the row's frame factor 2^(m - mf)
      const bool any = dm > -INFINITY;
      const float mp127 = any ? __builtin_amdgcn_exp2f(dm - kLog2_127) : 0.0f;  // mP / 127
      float lsc[kQB], cv[kQB];
#pragma unroll
      for (int qb = 0; qb < kQB; qb++) {
        lsc[qb] = mp127 * __builtin_amdgcn_exp2f(m[qb] - mf[qb]);
        cv[qb] = lsc[qb] * svj;
      }
      i32x4 pf[kQB][NB];
      // masked columns (ragged tail, invalid block) and a tile without real
      // rows take the checked variant
      if (f > kNarrowF)
        quantize_tile<true, true>(s, f, m, dm, any, kv0, jvalid, N, lsc, l, pf);
      else if (masked || !any)
        quantize_tile<true, false>(s, f, m, dm, any, kv0, jvalid, N, lsc, l, pf);
      else
        quantize_tile<false, false>(s, f, m, dm, any, kv0, jvalid, N, lsc, l, pf);

      // ---- O += (mP/127) sV_j 2^(m - mf) (P8 . V8), one channel block at a time
#pragma unroll
      for (int db = 0; db < D / 32; db++) {
        i32x16 ov[kQB];
        pv_block<D, BK>(vbuf[t & 1], vread, pf, db, pacc, ov);
#pragma unroll
        for (int qb = 0; qb < kQB; qb++)
#pragma unroll
          for (int r = 0; r < 16; r++)
            o[qb][db][r] = __builtin_fmaf(__int_as_float(ov[qb][r]), cv[qb], o[qb][db][r]);
      }
#pragma unroll
      for (int qb = 0; qb < kQB; qb++) pend[qb] = __builtin_fmaf(cv[qb], kPBiasF<BK>, pend[qb]);
      if (t % kFold == kFold - 1) {
#pragma unroll
        for (int qb = 0; qb < kQB; qb++) {
#pragma unroll
          for (int db = 0; db < D / 32; db++)
#pragma unroll
            for (int r = 0; r < 16; r++) o[qb][db][r] -= pend[qb];
          pend[qb] = 0.0f;
        }
      }
      j0 = j1; j1 = j2; j2 = j3;
      kb = kb == 2 ? 0 : kb + 1;
      sk0 = sk1; sv0 = sv1;
    }
  }

#pragma unroll
  for (int qb = 0; qb < kQB; qb++) {
    // the offset of the last tiles since the previous fold
#pragma unroll
    for (int db = 0; db < D / 32; db++)
#pragma unroll
      for (int r = 0; r < 16; r++) o[qb][db][r] -= pend[qb];
    const float lt = l[qb] + __shfl_xor(l[qb], 32);
    const int row = qbase + 32 * qb + l32;
    if (row < N) {
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
      int64_t li;
      uint16_t* op = out_row<D>(O, om.orders, om.F, om.H, om.W, om.sg, om.sn, g, N, row, li);
#pragma unroll
      for (int db = 0; db < D / 32; db++)
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++) {
          const int d0 = 32 * db + 8 * r4 + 4 * h;
          uint2 pk;
          pk.x = f32_to_bf16_bits(o[qb][db][4 * r4 + 0] * inv) |
                 (f32_to_bf16_bits(o[qb][db][4 * r4 + 1] * inv) << 16);
          pk.y = f32_to_bf16_bits(o[qb][db][4 * r4 + 2] * inv) |
                 (f32_to_bf16_bits(o[qb][db][4 * r4 + 3] * inv) << 16);
          *reinterpret_cast<uint2*>(op + d0) = pk;
        }
      if (lse != nullptr && h == 0)
        lse[li] = lt > 0.0f ? mf[qb] * kLn2 + logf(lt) : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// Debug entry points: the forward kernel's own staging and int8 tile
// routines on chosen tiles, writing exact int32 products.
template <int D, int BQ, int BK>
__global__ __launch_bounds__(BQ / kRowsPerWave * kWave) void dbg_qk_kernel(const int8_t* __restrict__ Q,
                                                    const int8_t* __restrict__ K, int G, int N,
                                                    int nq, int nk, const int32_t* __restrict__ gij,
                                                    int32_t* __restrict__ S) {
  constexpr int NW = BQ / kRowsPerWave;
  using L = L8<D, BK, NW>;
  __shared__ __attribute__((aligned(1024))) uint8_t kt[1][L::TB];
  const int t = blockIdx.x;
  int g = gij[3 * t], i = gij[3 * t + 1];
  const int j = gij[3 * t + 2];
  // an out-of-range head or q-block yields an all-zero tile; an out-of-range
  // kv-block reads as zero
  const bool ok = g >= 0 && g < G && i >= 0 && i < nq;
  if (!ok) { g = 0; i = nq; }
  const bool jvalid = static_cast<unsigned>(j) < static_cast<unsigned>(nk);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  Stage8<D, BK, NW> sg;
  sg.init();
  const int nrec = jvalid ? N * D : 0;
  L::stage(K + static_cast<int64_t>(g) * N * D, nrec, sg.k, jvalid ? j * BK : 0, kt[0]);
  i32x4 qf[kQB][D / 32];
  load_q<D>(Q, g, i * BQ + w * kRowsPerWave, N, qf);
  wait_loads();
  __syncthreads();
  i32x16 s[kQB][BK / 32];
  uint32_t kx[D / 32];
  k_offsets<D>(kx);
  qk_i8<D, BK>(kt[0], kx, qf, s);
  int32_t* out = S + static_cast<int64_t>(t) * BQ * BK;
#pragma unroll
  for (int qb = 0; qb < kQB; qb++) {
    const int qr = w * kRowsPerWave + 32 * qb + l32;
#pragma unroll
    for (int b = 0; b < BK / 32; b++)
#pragma unroll
      for (int r = 0; r < 16; r++) out[qr * BK + 32 * b + acc_row(r, h)] = s[qb][b][r];
  }
}

template <int D, int BQ, int BK>
__global__ __launch_bounds__(BQ / kRowsPerWave * kWave) void dbg_pv_kernel(const int8_t* __restrict__ P8,
                                                    const int8_t* __restrict__ V, int G, int N,
                                                    int nk, const int32_t* __restrict__ gj,
                                                    int32_t* __restrict__ OV) {
  constexpr int NW = BQ / kRowsPerWave;
  using L = L8<D, BK, NW>;
  __shared__ __attribute__((aligned(1024))) uint8_t vt[1][L::TB];
  const int t = blockIdx.x;
  int g = gj[2 * t], j = gj[2 * t + 1];
  // an out-of-range head or kv-block reads as an all-zero V tile
  if (g < 0 || g >= G) { g = 0; j = -1; }
  const bool jvalid = static_cast<unsigned>(j) < static_cast<unsigned>(nk);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  Stage8<D, BK, NW> sg;
  sg.init();
  const int nrec = jvalid ? N * D : 0;
  L::stage(V + static_cast<int64_t>(g) * N * D, nrec, sg.v, jvalid ? j * BK : 0, vt[0]);
  // P8 operand: slot s of lane half h carries kv 8(s/4) + 4h + s%4
  i32x4 pf[kQB][BK / 32];
#pragma unroll
  for (int qb = 0; qb < kQB; qb++) {
    const int8_t* prow = P8 + (static_cast<int64_t>(t) * BQ + w * kRowsPerWave + 32 * qb + l32) * BK;
#pragma unroll
    for (int b = 0; b < BK / 32; b++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 4; e++)
          word |= static_cast<uint32_t>(static_cast<uint8_t>(prow[32 * b + acc_row(4 * q4 + e, h)]))
                  << (8 * e);
        pf[qb][b][q4] = static_cast<int>(word);
      }
  }
  wait_loads();
  __syncthreads();
  int32_t* out = OV + static_cast<int64_t>(t) * BQ * D;
  const uint32_t vread = v_read_off<D>();
  i32x16 zacc = {};
  asm volatile("" : "+v"(zacc));
#pragma unroll
  for (int db = 0; db < D / 32; db++) {
    i32x16 ov[kQB];
    pv_block<D, BK>(vt[0], vread, pf, db, zacc, ov);
#pragma unroll
    for (int qb = 0; qb < kQB; qb++) {
      const int qr = w * kRowsPerWave + 32 * qb + l32;
#pragma unroll
      for (int r = 0; r < 16; r++) out[qr * D + 32 * db + acc_row(r, h)] = ov[qb][r];
    }
  }
}

// ---------------------------------------------------------------------------
template <template <int, int, int> class Launch, typename... Args>
hipError_t dispatch(int d, int Bq, int Bk, Args&&... args) {
  if (d == 128) {
    if (Bq == 128 && Bk == 64) return Launch<128, 128, 64>::run(args...);
    if (Bq == 128 && Bk == 128) return Launch<128, 128, 128>::run(args...);
    if (Bq == 64 && Bk == 64) return Launch<128, 64, 64>::run(args...);
    if (Bq == 64 && Bk == 128) return Launch<128, 64, 128>::run(args...);
  } else {
    if (Bq == 128 && Bk == 64) return Launch<64, 128, 64>::run(args...);
    if (Bq == 128 && Bk == 128) return Launch<64, 128, 128>::run(args...);
    if (Bq == 64 && Bk == 64) return Launch<64, 64, 64>::run(args...);
    if (Bq == 64 && Bk == 128) return Launch<64, 64, 128>::run(args...);
  }
  return hipErrorInvalidValue;
}

float scale_log2_of(const AttnArgs& a) {
  const float sm = a.sm_scale > 0.0f ? a.sm_scale : 1.0f / sqrtf(static_cast<float>(a.d));
  return sm * kLog2e;
}

template <int D, int BQ, int BK>
struct LaunchI8 {
  static hipError_t run(const AttnArgs& a, hipStream_t s) {
    const int nq = (a.N + BQ - 1) / BQ, nk = (a.N + BK - 1) / BK;
    const uint32_t nwg = kNumXcd * static_cast<uint32_t>((static_cast<int64_t>(a.G) * nq + kNumXcd - 1) / kNumXcd);
    fwd_i8_kernel<D, BQ, BK><<<nwg, BQ / kRowsPerWave * kWave, 0, s>>>(
        static_cast<const int8_t*>(a.Q), a.sQ, static_cast<const int8_t*>(a.K), a.sK,
        static_cast<const int8_t*>(a.V), a.sV, a.row_ptr, a.col_idx, a.col_len, a.mask_G, a.O,
        a.lse, a.G, a.N, nq, nk, scale_log2_of(a), a.out);
    return hipGetLastError();
  }
};

template <int D, int BQ, int BK>
struct LaunchDbgQk {
  static hipError_t run(const int8_t* Q, const int8_t* K, int G, int N, const int32_t* gij, int n,
                        int32_t* S, hipStream_t s) {
    const int nq = (N + BQ - 1) / BQ, nk = (N + BK - 1) / BK;
    dbg_qk_kernel<D, BQ, BK><<<n, BQ / kRowsPerWave * kWave, 0, s>>>(Q, K, G, N, nq, nk, gij, S);
    return hipGetLastError();
  }
};

template <int D, int BQ, int BK>
struct LaunchDbgPv {
  static hipError_t run(const int8_t* P8, const int8_t* V, int G, int N, const int32_t* gj, int n,
                        int32_t* OV, hipStream_t s) {
    const int nk = (N + BK - 1) / BK;
    dbg_pv_kernel<D, BQ, BK><<<n, BQ / kRowsPerWave * kWave, 0, s>>>(P8, V, G, N, nk, gj, OV);
    return hipGetLastError();
  }
};

}  // namespace

hipError_t launch_forward_int8(const AttnArgs& a, hipStream_t s) {
  return dispatch<LaunchI8>(a.d, a.Bq, a.Bk, a, s);
}
hipError_t launch_debug_int8_qk(const int8_t* Qq, const int8_t* Kq, int G, int N, int d, int Bq,
                                int Bk, const int32_t* gij, int n, int32_t* S, hipStream_t s) {
  return dispatch<LaunchDbgQk>(d, Bq, Bk, Qq, Kq, G, N, gij, n, S, s);
}
hipError_t launch_debug_int8_pv(const int8_t* P8, const int8_t* Vq, int G, int N, int d, int Bq,
                                int Bk, const int32_t* gj, int n, int32_t* OV, hipStream_t s) {
  return dispatch<LaunchDbgPv>(d, Bq, Bk, P8, Vq, G, N, gj, n, OV, s);
}

}  // namespace bsa
