// attn_bf16.hip — bf16 block-sparse flash attention forward for gfx950.
//
// SPADE machine verdict (pith.science, arXiv 2608.03335), key machinery: a
// flash-style block-sparse kernel with online softmax computes only the
// kept blocks; referee minor comment on §2.2 Eq. (2): the block mask is
// additive (0 on kept, -inf on pruned block pairs).
//
// Work split: one workgroup per (head g, q-block i); Bq/64 waves, each wave
// owns 64 query rows as two 32-row halves, so every K and V operand read
// from LDS feeds two MFMAs.  One wave per SIMD (two workgroups per CU): the
// 64-row waves keep LDS read traffic at half of what 32-row waves need.
//
// Per 64-row kv sub-tile (a 128-wide kv-block is two sub-tiles):
//   S^T = K . Q^T     v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = Q
//                     fragments in registers; the accumulator holds one query
//                     row per lane (the two wave halves share a row).
//   online softmax    in registers: one cross-half exchange per row max; row
//                     sums stay per lane until the end (bf16 dot2 with 1s);
//                     the reference max is raised only when a tile exceeds
//                     it by 2^8, so the O rescale is rare and O = acc/l stays
//                     exact.
//   O^T += V^T . P^T  A = V^T read with ds_read_b64_tr_b16 from row-major V
//                     (a 16-lane group reads a 4x16 block and receives it
//                     transposed), B = P converted to bf16 in registers.
// Both operands of an MFMA map the reduction index to slots the same way, so
// the kv order inside a k-step only has to agree between P and V^T: P slot j
// of lane half h carries kv 16s + 8(j/4) + 4h + j%4, which is what two
// transposed reads at rows 16s + 4h and 16s + 8 + 4h return.
//
// Pipeline (one barrier per sub-tile): iteration t issues the global->LDS
// loads of K(t+2) and V(t+1), computes S(t+1) = K(t+1).Q^T, its softmax, and
// O += P(t).V(t), so the MFMA stream of both products covers the softmax.
// K and V move global -> LDS directly (16-byte global_load_lds).  LDS chunk
// c of row r sits at c ^ (r mod 16) for K and c ^ (2r mod 16) for V, which
// makes the MFMA operand reads conflict-free; the swizzle is realised by
// choosing which global chunk each lane fetches.  A ragged last sub-tile is
// loaded as the 64-row window that ends at row N (all rows real) and its
// columns outside the sub-tile are masked.
#include <utility>

#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int KT = 64;          // kv rows per sub-tile
constexpr float kTau = 8.0f;    // lazy-rescale threshold of the first tile, log2 units
constexpr float kRefInit = -1.0e30f;    // reference before any score: finite, below every score
constexpr float kSumBound = 65536.0f;   // tile row-half sum that raises the reference
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
#ifndef BSA_PF_A
#define BSA_PF_A 2
#endif
#ifndef BSA_PF_B
#define BSA_PF_B 2
#endif
constexpr int kPfA = BSA_PF_A;  // LDS operand prefetch distance (MFMA steps), S = K.Q^T
constexpr int kPfB = BSA_PF_B;  // same for O += P.V
#ifndef BSA_LOAD_STEPS
#define BSA_LOAD_STEPS 0
#endif

template <int D, int NW>
struct Ly {
  static constexpr int ROWB = D * 2;           // bytes per K/V row
  static constexpr int CH = ROWB / 16;         // 16-byte chunks per row
  static constexpr int TB = KT * ROWB;         // bytes per sub-tile
  static constexpr int RPI = 1024 / ROWB;      // rows per wave-wide 1 KB load
  static constexpr int NI = TB / 1024 / NW;    // loads per wave per sub-tile
  static constexpr int RW = NW * RPI;          // rows covered by one load of all waves
};

// Where a sub-tile's rows come from: window start (all rows real when
// N >= 64), the logical start of the sub-tile, and validity.
struct Tile {
  int win;    // first row loaded
  int kv0;    // first row that belongs to the sub-tile
  bool valid; // kv-block index in range
  bool mask;  // some column of the window must be masked
};

template <int BK>
__device__ __forceinline__ Tile tile_of(const int32_t* __restrict__ col_idx, int64_t e0, int t,
                                        int N, int nk) {
  constexpr int SUB = BK / KT;
  const int j = col_idx[e0 + t / SUB];
  Tile T;
  T.valid = static_cast<unsigned>(j) < static_cast<unsigned>(nk);
  T.kv0 = T.valid ? j * BK + (t % SUB) * KT : 0;
  T.win = T.kv0 + KT <= N ? T.kv0 : (N >= KT ? N - KT : 0);
  T.mask = !T.valid || T.win != T.kv0 || T.kv0 + KT > N;
  return T;
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int D, int NW>
__device__ __forceinline__ void qk(const uint8_t* kt, uint32_t kread, const bf16x8 (&qf)[2][D / 16],
                                   f32x16 (&s)[2][2]) {
  using L = Ly<D, NW>;
#pragma unroll
  for (int b = 0; b < 2; b++) {
    s[0][b] = f32x16{};
    s[1][b] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ks++) {
      const bf16x8 a =
          *reinterpret_cast<const bf16x8*>(kt + b * 32 * L::ROWB + (kread ^ (ks << 5)));
      s[0][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[0][ks], s[0][b], 0, 0, 0);
      s[1][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[1][ks], s[1][b], 0, 0, 0);
    }
  }
}

template <int D, int NW>
__device__ __forceinline__ void pv(const uint8_t* vt, uint32_t vread, const bf16x8 (&p)[2][4],
                                   f32x16 (&o)[2][D / 32]) {
  using L = Ly<D, NW>;
#pragma unroll
  for (int db = 0; db < D / 32; db++) {
    const uint32_t cb = vread ^ (db << 6);
#pragma unroll
    for (int st = 0; st < 4; st++) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS i16x4*)(vt + (16 * st) * L::ROWB + cb));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS i16x4*)(vt + (16 * st + 8) * L::ROWB + cb));
      const bf16x8 a = __builtin_bit_cast(
          bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      o[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[0][st], o[0][db], 0, 0, 0);
      o[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[1][st], o[1][db], 0, 0, 0);
    }
  }
}

// Online softmax of one sub-tile.  Raw scores s; c = sm_scale*log2(e).
// Updates the reference max m (log2 units) and per-lane partial row sums l,
// writes P (bf16) and the O rescale factors; returns whether any row of
// this lane raised its reference.
template <bool MASK>
__device__ __forceinline__ bool softmax(f32x16 (&s)[2][2], const Tile& T, int N, float c,
                                        float (&m)[2], float (&l)[2], bf16x8 (&p)[2][4],
                                        float (&alpha)[2]) {
  const int h = (threadIdx.x & 63) >> 5;
  bool upd_any = false;
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    if constexpr (MASK) {
#pragma unroll
      for (int b = 0; b < 2; b++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int kv = T.win + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
          if (!T.valid || kv < T.kv0 || kv >= N) s[qb][b][r] = -INFINITY;
        }
    }
    float mt = s[qb][0][0];
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int r = 0; r < 16; r++) mt = fmaxf(mt, s[qb][b][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mt2 = mt * c;
    const bool upd = mt2 > m[qb] + kTau;
    alpha[qb] = upd ? __builtin_amdgcn_exp2f(m[qb] - mt2) : 1.0f;
    m[qb] = upd ? mt2 : m[qb];
    upd_any |= upd;
    const float ref = m[qb];
    float sum = 0.0f;
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][b][r], c, -ref));
        const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][b][r + 1], c, -ref));
        const bf16x2 pr = (bf16x2){static_cast<__bf16>(x0), static_cast<__bf16>(x1)};
        p[qb][2 * b + (r >> 3)][r & 7] = pr[0];
        p[qb][2 * b + (r >> 3)][(r & 7) + 1] = pr[1];
        sum = __builtin_amdgcn_fdot2_f32_bf16(pr, (bf16x2){static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)}, sum, false);
      }
    l[qb] = l[qb] * alpha[qb] + sum;
  }
  return upd_any;
}

template <int D>
__device__ __forceinline__ void rescale(f32x16 (&o)[2][D / 32], const float (&alpha)[2]) {
#pragma unroll
  for (int qb = 0; qb < 2; qb++)
#pragma unroll
    for (int db = 0; db < D / 32; db++)
#pragma unroll
      for (int r = 0; r < 16; r++) o[qb][db][r] *= alpha[qb];
}

// max of x over the two 32-lane halves (a row is split across them)
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int D, int NW>
__device__ __forceinline__ bf16x8 k_operand(const uint8_t* kt, uint32_t kread, int b, int ks) {
  return *reinterpret_cast<const bf16x8*>(kt + b * 32 * Ly<D, NW>::ROWB + (kread ^ (ks << 5)));
}

template <int D, int NW>
__device__ __forceinline__ bf16x8 v_operand(const uint8_t* vt, uint32_t vread, int st, int db) {
  using L = Ly<D, NW>;
  const uint32_t cb = vread ^ (db << 6);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vt + (16 * st) * L::ROWB + cb));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vt + (16 * st + 8) * L::ROWB + cb));
  return __builtin_bit_cast(bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// Lane offsets of the global->LDS loads.  Load q of wave w writes LDS bytes
// [(q*NW + w)*1024, +1024); lane l's 16 bytes land in row
// r = q*RW + w*RPI + l/CH, physical chunk l%CH, and must hold logical
// chunk (l%CH) ^ swz(r).  The q-dependence of the swizzle repeats with a
// short period, so a few lane constants plus a per-load scalar offset
// q*NW*1024 cover all loads.
template <int D, int NW>
struct Stage {
  using L = Ly<D, NW>;
  static constexpr int NVK = L::RW >= L::CH ? 1 : L::CH / L::RW;
  static constexpr int NVV = 2 * L::RW >= L::CH ? 1 : L::CH / (2 * L::RW);
  uint32_t k[NVK], v[NVV];
  __device__ __forceinline__ void init() {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int rw = w * L::RPI + lane / L::CH, p = lane % L::CH;
#pragma unroll
    for (int a = 0; a < NVK; a++) {
      const int r = a * L::RW + rw;
      k[a] = static_cast<uint32_t>(rw * L::ROWB + ((p ^ (r & (L::CH - 1))) << 4));
    }
#pragma unroll
    for (int a = 0; a < NVV; a++) {
      const int r = a * L::RW + rw;
      v[a] = static_cast<uint32_t>(rw * L::ROWB + ((p ^ ((2 * r) & (L::CH - 1))) << 4));
    }
  }
  // byte offset (inside the window) of load q, SMALLN: rows past N clamped
  template <bool ISV, bool SMALLN>
  __device__ __forceinline__ uint32_t lane_off(int q, int N) const {
    const uint32_t o = ISV ? v[q % NVV] : k[q % NVK];
    if constexpr (!SMALLN) return o;
    const int r = (q * L::RW * L::ROWB + static_cast<int>(o)) / L::ROWB;
    return r < N ? o : o - static_cast<uint32_t>((r - (N - 1)) * L::ROWB);
  }
};

template <int D, int NW, bool ISV, bool SMALLN>
__device__ __forceinline__ void load_one(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, int win, int q,
                                         uint8_t* tile) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const uint32_t soff = static_cast<uint32_t>(win * Ly<D, NW>::ROWB + q * NW * 1024);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)(tile + (q * NW + w) * 1024), 16,
                                           voff, soff, 0, 0);
}

template <int D, int NW, bool SMALLN>
__device__ __forceinline__ void stage_all(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                          const Stage<D, NW>& sg, const Tile& T, int N, uint8_t* kt,
                                          uint8_t* vt) {
#pragma unroll
  for (int q = 0; q < Ly<D, NW>::NI; q++) {
    if (kt) load_one<D, NW, false, SMALLN>(kr, sg.template lane_off<false, SMALLN>(q, N), T.win, q, kt);
    if (vt) load_one<D, NW, true, SMALLN>(vr, sg.template lane_off<true, SMALLN>(q, N), T.win, q, vt);
  }
}

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }
// Pins a value's computation to this point of the instruction stream (an
// empty volatile asm that reads and rewrites it).
__device__ __forceinline__ void anchor(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void anchor(uint32_t& x) { asm volatile("" : "+v"(x)); }

// One steady-state iteration, in an explicit instruction order:
//   phase A: S(t+1) = K(t+1).Q^T — 2*(D/16) steps of 2 MFMAs (alternating kv
//            halves so that four accumulation chains are in flight); step x
//            reads the K operand of step x+2 and issues a share of the
//            global->LDS loads of K(t+2) and V(t+1);
//   phase B: O += P(t).V(t) — 4*(D/32) steps of 2 MFMAs with the V operands
//            read two steps ahead; the softmax of S(t+1) is cut into as many
//            slices, one per step (row maxima in the first two, then the
//            exponentials, bf16 packing and row sums).
// A scheduling fence closes every step and each slice's results are pinned
// inside it, so the compiler cannot regroup the stream.
// exponentials of score pair pp (of 32: row half pp/16, kv half (pp/8)%2,
// accumulator slots 2(pp%8), +1) against reference m, their sum, and their
// bf16 pair as word pp%4 of P[pp/16][(pp%16)/4]
__device__ __forceinline__ void exp_pair(const f32x16 (&s)[2][2], float c, const float (&m)[2],
                                         int pp, float (&sum)[2], u32x4 (&pw)[2][4]) {
  const int qb = pp >> 4, b = (pp >> 3) & 1, r = 2 * (pp & 7);
  const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][b][r], c, -m[qb]));
  const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][b][r + 1], c, -m[qb]));
#ifdef BSA_SUM_DOT2
  const bf16x2 pr = (bf16x2){static_cast<__bf16>(x0), static_cast<__bf16>(x1)};
  sum[qb] = __builtin_amdgcn_fdot2_f32_bf16(
      pr, (bf16x2){static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)}, sum[qb], false);
  pw[qb][(pp & 15) >> 2][pp & 3] = __builtin_bit_cast(uint32_t, pr);
#else
  sum[qb] = (sum[qb] + x0) + x1;
  pw[qb][(pp & 15) >> 2][pp & 3] =
      __builtin_bit_cast(uint32_t, (bf16x2){static_cast<__bf16>(x0), static_cast<__bf16>(x1)});
#endif
  if ((pp & 3) == 3) asm volatile("" : "+v"(pw[qb][(pp & 15) >> 2]));
}

template <int D, int NW, bool SMALLN>
__device__ __forceinline__ uint64_t step(int N, float c, __amdgpu_buffer_rsrc_t krs,
                                     __amdgpu_buffer_rsrc_t vrs, const Stage<D, NW>& sg,
                                     uint32_t kread, uint32_t vread, uint8_t* __restrict__ kb_next,
                                     uint8_t* __restrict__ kb_free, uint8_t* __restrict__ vb_cur,
                                     uint8_t* __restrict__ vb_free,
                                     const Tile& Tn, const Tile& Tk,
                                     const bf16x8 (&qf)[2][D / 16], f32x16 (&o)[2][D / 32],
                                     const bf16x8 (&p)[2][4], bf16x8 (&p_nxt)[2][4],
                                     float (&m)[2], float (&l)[2], float (&alpha)[2]) {
  using L = Ly<D, NW>;
  constexpr int NA = 2 * (D / 16);   // phase A steps
  constexpr int NB = 4 * (D / 32);   // phase B steps
  constexpr int NG = 2 * L::NI;      // global loads per wave
  // the global loads go out over the first NL steps of phase A
  constexpr int NL = BSA_LOAD_STEPS > 0 && BSA_LOAD_STEPS < NA ? BSA_LOAD_STEPS : NA;
  constexpr int DB = D / 32;
  const int h = (threadIdx.x & 63) >> 5;

  // ---- phase A
  f32x16 s[2][2];
#pragma unroll
  for (int b = 0; b < 2; b++) { s[0][b] = f32x16{}; s[1][b] = f32x16{}; }
  bf16x8 ka[kPfA + 1];
#pragma unroll
  for (int x = 0; x < kPfA; x++) ka[x] = k_operand<D, NW>(kb_next, kread, x & 1, x >> 1);
#pragma unroll
  for (int x = 0; x < NA; x++) {
    const int b = x & 1, ks = x >> 1;
    if (x + kPfA < NA)
      ka[(x + kPfA) % (kPfA + 1)] = k_operand<D, NW>(kb_next, kread, (x + kPfA) & 1, (x + kPfA) >> 1);
#pragma unroll
    for (int gq = x * NG / NL; gq < (x + 1) * NG / NL && gq < NG; gq++) {
      if (gq < L::NI)
        load_one<D, NW, false, SMALLN>(krs, sg.template lane_off<false, SMALLN>(gq, N), Tk.win, gq, kb_free);
      else
        load_one<D, NW, true, SMALLN>(vrs, sg.template lane_off<true, SMALLN>(gq - L::NI, N), Tn.win,
                                      gq - L::NI, vb_free);
    }
    s[0][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[x % (kPfA + 1)], qf[0][ks], s[0][b], 0, 0, 0);
    s[1][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[x % (kPfA + 1)], qf[1][ks], s[1][b], 0, 0, 0);
    fence();
  }

  // columns outside the sub-tile (ragged tail, invalid block index): -inf.
  // Only the scores pass through this branch.
  if (Tn.mask) {
#pragma unroll
    for (int qb = 0; qb < 2; qb++)
#pragma unroll
      for (int b = 0; b < 2; b++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int kv = Tn.win + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
          if (!Tn.valid || kv < Tn.kv0 || kv >= N) s[qb][b][r] = -INFINITY;
        }
  }

  // ---- phase B
  u32x4 pw[2][4];  // P as packed bf16 pairs: pw[qb][st][w] = words of P[qb][st]
  float sum[2] = {0.0f, 0.0f};
  bf16x8 va[kPfB + 1];
#pragma unroll
  for (int k = 0; k < kPfB; k++) va[k] = v_operand<D, NW>(vb_cur, vread, k / DB, k % DB);
#pragma unroll
  for (int k = 0; k < NB; k++) {
    if (k + kPfB < NB)
      va[(k + kPfB) % (kPfB + 1)] = v_operand<D, NW>(vb_cur, vread, (k + kPfB) / DB, (k + kPfB) % DB);
    const int st = k / DB, db = k % DB;
    o[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[k % (kPfB + 1)], p[0][st], o[0][db], 0, 0, 0);
    o[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[k % (kPfB + 1)], p[1][st], o[1][db], 0, 0, 0);
    // exponentials of score pairs [lo, hi) out of 32 against the running reference
#pragma unroll
    for (int pp = k * 32 / NB; pp < (k + 1) * 32 / NB; pp++) exp_pair(s, c, m, pp, sum, pw);
    fence();
  }
  // A tile row-half sum past the bound means scores rose well above the
  // reference: redo this tile's exponentials against its exact row maximum
  // (and rescale O before the next product).  Rare after the first tiles.
  const uint64_t upd = __ballot(!(sum[0] <= kSumBound && sum[1] <= kSumBound));
  if (upd != 0ull) {
#pragma unroll
    for (int qb = 0; qb < 2; qb++) {
      float x = s[qb][0][0];
#pragma unroll
      for (int b = 0; b < 2; b++)
#pragma unroll
        for (int r = 0; r < 16; r++) x = fmaxf(x, s[qb][b][r]);
      const float mn = fmaxf(m[qb], halves_max(x) * c);
      alpha[qb] = __builtin_amdgcn_exp2f(m[qb] - mn);
      m[qb] = mn;
      sum[qb] = 0.0f;
#pragma unroll
      for (int pp = 16 * qb; pp < 16 * qb + 16; pp++) exp_pair(s, c, m, pp, sum, pw);
      l[qb] = l[qb] * alpha[qb] + sum[qb];
    }
  } else {
    l[0] += sum[0];
    l[1] += sum[1];
  }
#pragma unroll
  for (int qb = 0; qb < 2; qb++)
#pragma unroll
    for (int st = 0; st < 4; st++) p_nxt[qb][st] = __builtin_bit_cast(bf16x8, pw[qb][st]);
  wait_loads();
  return upd;
}

template <int D, int BQ, int BK, bool SMALLN>
__global__ __launch_bounds__(BQ) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t col_len,
    int mask_G, uint16_t* __restrict__ O, float* __restrict__ lse, int N, int nq, int nk,
    float c) {
  constexpr int NW = BQ / 64;
  constexpr int SUB = BK / KT;
  using L = Ly<D, NW>;
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[L::TB];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[L::TB];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[L::TB];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[L::TB];

  int g, i;
  if (!head_sync_tile(blockIdx.x, nq, g, i)) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int qbase = i * BQ + w * 64;

  // lane constants: staging offsets and the LDS read offsets of the MFMA operands
  Stage<D, NW> sg;
  sg.init();
  const uint32_t kread = static_cast<uint32_t>(l32 * L::ROWB + ((h ^ (l32 & (L::CH - 1))) << 4));
  uint32_t vread;
  {
    const int rsub = (lane & 15) >> 2;
    const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int sv = (2 * (4 * h + rsub)) & (L::CH - 1);
    vread = static_cast<uint32_t>((4 * h + rsub) * L::ROWB + ((cl ^ sv) << 4) + (lane & 1) * 8);
  }

  bf16x8 qf[2][D / 16];
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    const int row = qbase + 32 * qb + l32;
    const bool ok = row < N;
    const uint16_t* qp = Q + (static_cast<int64_t>(g) * N + (ok ? row : 0)) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < D / 16; ks++) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (ok) v = *reinterpret_cast<const uint4*>(qp + 16 * ks);
      qf[qb][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  int64_t e0 = row_ptr[static_cast<int64_t>(g % mask_G) * nq + i];
  int64_t e1 = row_ptr[static_cast<int64_t>(g % mask_G) * nq + i + 1];
  e0 = e0 < 0 ? 0 : (e0 > col_len ? col_len : e0);
  e1 = e1 < e0 ? e0 : (e1 > col_len ? col_len : e1);
  const int nt = static_cast<int>(e1 - e0) * SUB;

  const int head_bytes = N * L::ROWB;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(K + static_cast<int64_t>(g) * N * D), 0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(V + static_cast<int64_t>(g) * N * D), 0, head_bytes, 0x00020000);

  float m[2] = {kRefInit, kRefInit}, l[2] = {0.0f, 0.0f}, alpha[2] = {1.0f, 1.0f};
  f32x16 o[2][D / 32];
#pragma unroll
  for (int qb = 0; qb < 2; qb++)
#pragma unroll
    for (int db = 0; db < D / 32; db++) o[qb][db] = f32x16{};

  if (nt > 0) {
    bf16x8 p[2][4];
    {
      const Tile T0 = tile_of<BK>(col_idx, e0, 0, N, nk);
      stage_all<D, NW, SMALLN>(krs, vrs, sg, T0, N, kb0, vb0);
      if (nt > 1) stage_all<D, NW, SMALLN>(krs, vrs, sg, tile_of<BK>(col_idx, e0, 1, N, nk), N, kb1, nullptr);
      wait_loads();
      __syncthreads();
      f32x16 s[2][2];
      qk<D, NW>(kb0, kread, qf, s);
      if (T0.mask) softmax<true>(s, T0, N, c, m, l, p, alpha);
      else softmax<false>(s, T0, N, c, m, l, p, alpha);
      __syncthreads();
    }
    uint64_t upd = 0;  // O is still zero: nothing to rescale yet
    // tiles t+1 and t+2 are fetched one iteration ahead; pinning them at the
    // end of the iteration retires the scalar loads outside the LDS phases.
    // K(t+2) is always loaded (at t+2 == nt the last tile is reloaded into a
    // buffer that is not read again), which keeps the iteration branch-free.
    Tile Tn = tile_of<BK>(col_idx, e0, nt > 1 ? 1 : 0, N, nk);
    Tile Tk = tile_of<BK>(col_idx, e0, nt > 2 ? 2 : nt - 1, N, nk);
    int t = 0;
    for (; t + 1 < nt; t++) {
      if (upd != 0ull) rescale<D>(o, alpha);
      const bool odd = t & 1;
      bf16x8 pn[2][4];
      upd = step<D, NW, SMALLN>(N, c, krs, vrs, sg, kread, vread, odd ? kb0 : kb1, odd ? kb1 : kb0,
                                odd ? vb1 : vb0, odd ? vb0 : vb1, Tn, Tk, qf, o, p, pn, m, l, alpha);
#pragma unroll
      for (int qb = 0; qb < 2; qb++)
#pragma unroll
        for (int st = 0; st < 4; st++) p[qb][st] = pn[qb][st];
      Tn = Tk;
      Tk = tile_of<BK>(col_idx, e0, t + 3 < nt ? t + 3 : nt - 1, N, nk);
      asm volatile("" ::"s"(Tk.win), "s"(Tk.kv0), "s"(static_cast<int>(Tk.valid)));
      __syncthreads();
    }
    if (upd != 0ull) rescale<D>(o, alpha);
    pv<D, NW>((t & 1) ? vb1 : vb0, vread, p, o);
  }

#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    const float lt = l[qb] + __shfl_xor(l[qb], 32);
    const int row = qbase + 32 * qb + l32;
    if (row < N) {
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
      uint16_t* op = O + (static_cast<int64_t>(g) * N + row) * D;
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
        lse[static_cast<int64_t>(g) * N + row] = lt > 0.0f ? m[qb] * kLn2 + logf(lt) : -INFINITY;
    }
  }
}

template <int D, int BQ, int BK>
hipError_t launch(const AttnArgs& a, hipStream_t s) {
  const int nq = (a.N + BQ - 1) / BQ, nk = (a.N + BK - 1) / BK;
  const uint32_t nwg = static_cast<uint32_t>(a.G) * kNumXcd * ((nq + kNumXcd - 1) / kNumXcd);
  const float sm = a.sm_scale > 0.0f ? a.sm_scale : 1.0f / sqrtf(static_cast<float>(a.d));
  auto kern = a.N >= KT ? fwd_bf16_kernel<D, BQ, BK, false> : fwd_bf16_kernel<D, BQ, BK, true>;
  kern<<<nwg, BQ, 0, s>>>(static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                          static_cast<const uint16_t*>(a.V), a.row_ptr, a.col_idx, a.col_len,
                          a.mask_G, a.O, a.lse, a.N, nq, nk, sm * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.d == 128) {
    if (a.Bq == 128 && a.Bk == 64) return launch<128, 128, 64>(a, s);
    if (a.Bq == 128 && a.Bk == 128) return launch<128, 128, 128>(a, s);
    if (a.Bq == 64 && a.Bk == 64) return launch<128, 64, 64>(a, s);
    if (a.Bq == 64 && a.Bk == 128) return launch<128, 64, 128>(a, s);
  } else if (a.d == 64) {
    if (a.Bq == 128 && a.Bk == 64) return launch<64, 128, 64>(a, s);
    if (a.Bq == 128 && a.Bk == 128) return launch<64, 128, 128>(a, s);
    if (a.Bq == 64 && a.Bk == 64) return launch<64, 64, 64>(a, s);
    if (a.Bq == 64 && a.Bk == 128) return launch<64, 64, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace bsa
