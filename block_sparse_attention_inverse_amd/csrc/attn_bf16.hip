// attn_bf16.hip — bf16 block-sparse flash attention forward for gfx950.
//
// SPADE machine verdict (pith.science, arXiv 2608.03335), key machinery: a
// flash-style block-sparse kernel with online softmax computes only the
// kept blocks; referee minor comment on §2.2 Eq. (2): the block mask is
// additive (0 on kept, -inf on pruned block pairs).
//
// Work split: one workgroup per (head g, q-block i); Bq/64 waves, each wave
// owns 64 query rows as two 32-row halves (qb), so every K and V operand
// read from LDS feeds two MFMAs.  One wave per SIMD (two workgroups per CU).
//
// Products (v_mfma_f32_32x32x16_bf16), per 32-row kv half-tile u:
//   S_u^T = K_u . Q^T - m    A = K rows from LDS, B = Q fragments held in
//                            AGPRs; the accumulator starts at -m (the row's
//                            reference), so each probability is one multiply
//                            by c = sm_scale*log2(e) and one exp2.  Every
//                            lane holds one query row; lane half h, slot r
//                            carries kv 8(r/4) + 4h + r%4 of the half.
//   O^T += V_u^T . P_u^T     A = V^T read with ds_read_b64_tr_b16 (the
//                            transposing LDS read) from row-major V, B = P
//                            converted to bf16 in registers: slots 8s..8s+7
//                            of a lane are exactly the kv indices that the two
//                            transposed reads at rows 16s + 4h and 16s + 8 + 4h
//                            return, so P never moves between lanes.
//
// Software pipeline, one step per half-tile u: the MFMA stream alternates
// S_{u+1} = K_{u+1}.Qc^T and O += P_{u-1}.V_{u-1}, and under it the VALU
// computes P_u = exp2(S_u), its bf16 pairs and row sums, one score per MFMA,
// so the exponentials are spread over both products.  Two S and two P
// register sets alternate between steps.
//
// Reference m: the first half-tile of a row sets it to that half-tile's
// exact row maximum and it never moves afterwards.  O = acc / l does not
// depend on m, so the only requirement is that no exponential overflows: a
// half-tile row sum above 2^96 (later scores far above m), or a row that ends
// with no weight, raises a flag, and a workgroup with the flag set recomputes
// its rows on an exact two-pass path (row maxima over every kept column
// first, then O and l against them).  The first half-tile of a row whose
// columns are all masked leaves m at 0.
//
// K and V move HBM -> LDS in 64-row sub-tiles with 16-byte buffer loads that
// write LDS directly, double-buffered (64 KB per workgroup).  LDS chunk c of
// row r sits at c ^ (r mod 16) for K and c ^ (2r mod 16) for V, which makes
// the operand reads conflict-free; the swizzle is realised by choosing which
// global chunk each lane fetches.  The second step of a sub-tile issues the
// loads of K two sub-tiles ahead and V one ahead; one barrier per sub-tile.
// The kv-block index of each sub-tile reaches the scalar unit through a
// vector load issued a sub-tile ahead (so no scalar memory load is pending
// while LDS operand reads are waited on).  A ragged last sub-tile is loaded
// as the 64-row window that ends at row N (all rows real) and its columns
// outside the sub-tile are masked.
//
// Grid order: workgroup b runs on XCD b mod 8; the XCDs work in two groups
// of four, each group on one head at a time with every XCD of the group on
// a contiguous quarter of that head's q-blocks, so the workgroups resident
// on an XCD are neighbouring q-blocks of one head (its 4 MB L2 serves a
// single head's K/V) and only two heads' K/V (78 MB at 720p) are in flight
// in the last-level cache.
#include <utility>

#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int KT = 64;                  // kv rows per staged sub-tile
constexpr float kSumBound = 0x1p96f;    // half-tile row sum that flags overflow
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kPf = 4;                  // LDS operand prefetch distance (operands)

template <int D, int NW>
struct Ly {
  static constexpr int ROWB = D * 2;           // bytes per K/V row
  static constexpr int CH = ROWB / 16;         // 16-byte chunks per row
  static constexpr int TB = KT * ROWB;         // bytes per sub-tile
  static constexpr int RPI = 1024 / ROWB;      // rows per wave-wide 1 KB load
  static constexpr int NI = TB / 1024 / NW;    // loads per wave per sub-tile
  static constexpr int RW = NW * RPI;          // rows covered by one load of all waves
  static constexpr int KS = D / 16;            // k-steps of S (and K operands per half)
  static constexpr int DB = D / 32;            // 32-channel blocks of O
  static constexpr int NV = 2 * DB;            // V operands per half
  static constexpr int NS = D / 4;             // MFMA slots per step (KS*2 + NV*2)
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
__device__ __forceinline__ Tile make_tile(int j, int t, int N, int nk) {
  constexpr int SUB = BK / KT;
  Tile T;
  T.valid = static_cast<unsigned>(j) < static_cast<unsigned>(nk);
  T.kv0 = T.valid ? j * BK + (t % SUB) * KT : 0;
  T.win = T.kv0 + KT <= N ? T.kv0 : (N >= KT ? N - KT : 0);
  T.mask = !T.valid || T.win != T.kv0 || T.kv0 + KT > N;
  return T;
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }
template <typename T>
__device__ __forceinline__ void opaque(T& x) { asm volatile("" : "+v"(x)); }

// S accumulation as VGPR-form MFMAs written out explicitly, so that the
// scores land in VGPRs (where the exponentials read them) while O stays in
// AGPRs and the Q fragments are read from AGPRs.  The compiler does not see
// these as MFMAs: every VALU access to a score register within 24 wait
// states of its MFMA is preceded by mfma_drain().
__device__ __forceinline__ void mfma_s_init(f32x16& d, const bf16x8& a, const bf16x8& b,
                                            const f32x16& c) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c));
}
__device__ __forceinline__ void mfma_s_acc(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// max of x over the two 32-lane halves (a row is split across them)
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
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
  uint32_t wb;  // this wave's byte offset inside a staged tile (wave-uniform, kept in an SGPR)
  __device__ __forceinline__ void init() {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    wb = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(w) * 1024u);
    asm volatile("" : "+s"(wb));  // computed once, not re-derived from the thread id per load
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

template <int D, int NW>
__device__ __forceinline__ void load_raw(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, int win, int q,
                                         uint8_t* tile, uint32_t wb) {
  const uint32_t soff = static_cast<uint32_t>(win * Ly<D, NW>::ROWB + q * NW * 1024);
  // opaque per load, so the LDS address is one add here instead of a
  // register per (buffer, q) held across the loop
  asm volatile("" : "+s"(wb));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)(tile + q * NW * 1024 + wb), 16, voff,
                                           soff, 0, 0);
}
// load q of the staging of a K (ISV false) or V sub-tile whose window starts at row win
template <int D, int NW, bool ISV, bool SMALLN>
__device__ __forceinline__ void load_one(__amdgpu_buffer_rsrc_t rsrc, const Stage<D, NW>& sg, int N,
                                         int win, int q, uint8_t* tile) {
  load_raw<D, NW>(rsrc, sg.template lane_off<ISV, SMALLN>(q, N), win, q, tile, sg.wb);
}

template <int D, int NW, bool SMALLN>
__device__ __forceinline__ void stage_tile(__amdgpu_buffer_rsrc_t rs, const Stage<D, NW>& sg, int N,
                                           int win, uint8_t* tile, bool isv) {
#pragma unroll
  for (int q = 0; q < Ly<D, NW>::NI; q++) {
    if (isv) load_one<D, NW, true, SMALLN>(rs, sg, N, win, q, tile);
    else load_one<D, NW, false, SMALLN>(rs, sg, N, win, q, tile);
  }
}

// Per-lane LDS read offsets of the MFMA operands: kx[ks] for the K operand of
// k-step ks (row l32 of a 32-row half, chunk 2ks + h, swizzled), vx[db] for
// the transposed V reads of channel block db.  Kept in registers so every
// operand read is one ds_read with an immediate offset.
template <int D, int NW>
struct Addr {
  using L = Ly<D, NW>;
  uint32_t kx[L::KS], vx[L::DB];
  __device__ __forceinline__ void init() {
    const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
    const uint32_t kread = static_cast<uint32_t>(l32 * L::ROWB + ((h ^ (l32 & (L::CH - 1))) << 4));
    const int rsub = (lane & 15) >> 2;
    const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int sv = (2 * (4 * h + rsub)) & (L::CH - 1);
    const uint32_t vread =
        static_cast<uint32_t>((4 * h + rsub) * L::ROWB + ((cl ^ sv) << 4) + (lane & 1) * 8);
#pragma unroll
    for (int ks = 0; ks < L::KS; ks++) {
      kx[ks] = kread ^ static_cast<uint32_t>(ks << 5);
      opaque(kx[ks]);
    }
#pragma unroll
    for (int db = 0; db < L::DB; db++) {
      vx[db] = vread ^ static_cast<uint32_t>(db << 6);
      opaque(vx[db]);
    }
  }
};

// K operand of k-step ks for kv half hb of the sub-tile at kt
template <int D, int NW>
__device__ __forceinline__ bf16x8 k_operand(const uint8_t* kt, const Addr<D, NW>& ad, int hb, int ks) {
  return *reinterpret_cast<const bf16x8*>(kt + hb * 32 * Ly<D, NW>::ROWB + ad.kx[ks]);
}

// V^T operand of PV k-step st (16 kv rows 16st..16st+15 of the sub-tile,
// transposed), channel block db
template <int D, int NW>
__device__ __forceinline__ bf16x8 v_operand(const uint8_t* vt, const Addr<D, NW>& ad, int st, int db) {
  constexpr int R = Ly<D, NW>::ROWB;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vt + 16 * st * R + ad.vx[db]));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vt + (16 * st + 8) * R + ad.vx[db]));
  return __builtin_bit_cast(bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// operand index -> (k-step / channel block) for the prefetch rings:
// K operand x: ks = x.  V operand x: s2 = x / DB, db = x % DB.
template <int D, int NW>
__device__ __forceinline__ bf16x8 v_operand_x(const uint8_t* vt, const Addr<D, NW>& ad, int hb, int x) {
  constexpr int DB = Ly<D, NW>::DB;
  return v_operand<D, NW>(vt, ad, 2 * hb + x / DB, x % DB);
}

// columns of kv half hb of tile T outside the sub-tile (ragged tail,
// invalid block index): -inf
__device__ __forceinline__ void mask_half(f32x16 (&s)[2], const Tile& T, int hb, int N) {
  mfma_drain();
  int base = T.win + 32 * hb + 4 * ((threadIdx.x & 63) >> 5);
  opaque(base);  // per-slot offsets stay immediates
#pragma unroll
  for (int qb = 0; qb < 2; qb++)
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int kv = base + 8 * (r >> 2) + (r & 3);
      if (!T.valid || kv < T.kv0 || kv >= N) s[qb][r] = -INFINITY;
    }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Softmax of one half-tile, one score at a time: exp_issue(e) computes
// y_e = 2^(c * S_e) for score e (0..31: row half e/16, slot e%16); its
// consumers run one score later (exp_retire), so the exponential's latency
// passes under the next MFMA: y_e joins the row-half sum, and every second
// one completes a bf16 pair, word (e%8)/2 of P operand (e%16)/8.  The
// exponential is written out (and each result pinned) so that the work stays
// in its slot between the scheduling fences.
struct Ex {
  float y[4];  // y_e in y[e & 3]: a pair is packed while the next score is in flight
};
__device__ __forceinline__ void exp_issue(const f32x16 (&s)[2], int e, Ex& ex, float cs) {
  const int qb = e >> 4, r = e & 15;
  float x;
  asm volatile("v_mul_f32 %0, %2, %1\n\tv_exp_f32 %0, %0" : "=&v"(x) : "v"(s[qb][r]), "s"(cs));
  ex.y[e & 3] = x;
}
__device__ __forceinline__ void exp_retire(int e, Ex& ex, float (&sum)[2], u32x4 (&p)[2][2]) {
  const int qb = e >> 4, r = e & 15;
  sum[qb] += ex.y[e & 3];
  opaque(sum[qb]);
  if (r & 1) {
    uint32_t wd = __builtin_bit_cast(
        uint32_t, (bf16x2){static_cast<__bf16>(ex.y[(e - 1) & 3]), static_cast<__bf16>(ex.y[e & 3])});
    opaque(wd);
    p[qb][r >> 3][(r & 7) >> 1] = wd;
  }
}

// One pipeline step (kv half-tile u): the MFMA stream alternates
// S_{u+1} = K.Qc^T - m (K of half u+1: half H of sub-tile kt) and
// O += P_{u-1}.V (V of half u-1: half H of sub-tile vt); under it the
// exponentials of S_u give P_u and their row sums.  A half-tile row sum past
// kSumBound (scores far above the reference) raises the overflow flag.  The
// K / V operand rings ka / va arrive with their first kPf entries read.
// LM (staging issued under the step): 0 none; 1 the V sub-tile at row vwin
// into vl, then the K sub-tile at row kwin into kl.
template <int D, int NW, bool SMALLN, int H, bool PV, int LM>
__device__ __forceinline__ void step(const Addr<D, NW>& ad, const Stage<D, NW>& sg, int N,
                                     const uint8_t* __restrict__ kt, const uint8_t* __restrict__ vt,
                                     const bf16x8 (&qf)[2][D / 16], const f32x16 (&negm)[2],
                                     f32x16 (&o)[2][D / 32], const f32x16 (&s_cur)[2],
                                     f32x16 (&s_nxt)[2], u32x4 (&p_cur)[2][2],
                                     const u32x4 (&p_prv)[2][2], float (&l)[2], bool& ovf,
                                     bf16x8 (&ka)[kPf + 1], bf16x8 (&va)[kPf + 1],
                                     __amdgpu_buffer_rsrc_t krs, int kwin, uint8_t* __restrict__ kl,
                                     __amdgpu_buffer_rsrc_t vrs, int vwin, uint8_t* __restrict__ vl,
                                     float cs) {
  using L = Ly<D, NW>;
  constexpr int NS = L::NS;
  // staging loads of this step per wave: V first, then K
  constexpr int NG = LM == 1 ? 2 * L::NI : 0;
  float sum[2] = {0.0f, 0.0f};
  Ex ex;
#pragma unroll
  for (int x = 0; x < NS; x++) {
    const int i = x >> 1;
    if ((x & 1) == 0) {
      // S_{u+1}: MFMA i = k-step i/2, row half i%2
      const int ks = i >> 1, qb = i & 1;
      if (qb == 0 && ks + kPf < L::KS) ka[(ks + kPf) % (kPf + 1)] = k_operand<D, NW>(kt, ad, H, ks + kPf);
      if (ks == 0) mfma_s_init(s_nxt[qb], ka[ks % (kPf + 1)], qf[qb][ks], negm[qb]);
      else mfma_s_acc(s_nxt[qb], ka[ks % (kPf + 1)], qf[qb][ks]);
    } else if constexpr (PV) {
      // O += P_{u-1} . V_{u-1}: MFMA i = V operand i/2, row half i%2
      const int vi = i >> 1, qb = i & 1;
      if (qb == 0 && vi + kPf < L::NV) va[(vi + kPf) % (kPf + 1)] = v_operand_x<D, NW>(vt, ad, H, vi + kPf);
      const int s2 = vi / L::DB, db = vi % L::DB;
      o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          va[vi % (kPf + 1)], __builtin_bit_cast(bf16x8, p_prv[qb][s2]), o[qb][db], 0, 0, 0);
      asm volatile("" : "+a"(o[qb][db]));  // keeps the product in its slot
    }
    fence();  // the MFMA goes first in its slot
    // softmax of S_u: scores [x*32/NS, (x+1)*32/NS), each retired one score later
#pragma unroll
    for (int e = x * 32 / NS; e < (x + 1) * 32 / NS; e++) {
      exp_issue(s_cur, e, ex, cs);
      if (e > 0) exp_retire(e - 1, ex, sum, p_cur);
    }
    if constexpr (LM != 0) {
#pragma unroll
      for (int gq = x * NG / NS; gq < (x + 1) * NG / NS; gq++) {
        if (gq < L::NI) load_one<D, NW, true, SMALLN>(vrs, sg, N, vwin, gq, vl);
        else load_one<D, NW, false, SMALLN>(krs, sg, N, kwin, gq - L::NI, kl);
      }
    }
    fence();
  }
  exp_retire(31, ex, sum, p_cur);
  l[0] += sum[0];
  l[1] += sum[1];
  ovf = ovf || !(sum[0] <= kSumBound && sum[1] <= kSumBound);
}

template <int D, int NW>
__device__ __forceinline__ void prefetch(const Addr<D, NW>& ad, const uint8_t* kt, const uint8_t* vt,
                                         int hb, bf16x8 (&ka)[kPf + 1], bf16x8 (&va)[kPf + 1]) {
#pragma unroll
  for (int x = 0; x < kPf; x++) {
    ka[x] = k_operand<D, NW>(kt, ad, hb, x);
    va[x] = v_operand_x<D, NW>(vt, ad, hb, x);
  }
}

// O += P . V of one half (no S product alongside): the last half of a row
template <int D, int NW>
__device__ __forceinline__ void pv_only(const Addr<D, NW>& ad, const uint8_t* vt, int hb,
                                        const u32x4 (&p)[2][2], f32x16 (&o)[2][D / 32]) {
  using L = Ly<D, NW>;
#pragma unroll
  for (int vi = 0; vi < L::NV; vi++) {
    const bf16x8 a = v_operand_x<D, NW>(vt, ad, hb, vi);
    const int s2 = vi / L::DB, db = vi % L::DB;
    o[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, p[0][s2]), o[0][db], 0, 0, 0);
    o[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, p[1][s2]), o[1][db], 0, 0, 0);
  }
}

// S of half hb of the sub-tile at kt (accumulator start negm), drained
template <int D, int NW>
__device__ __forceinline__ void s_half(const Addr<D, NW>& ad, const uint8_t* kt, int hb,
                                       const bf16x8 (&qf)[2][D / 16], const f32x16 (&negm)[2],
                                       f32x16 (&s)[2]) {
#pragma unroll
  for (int ks = 0; ks < Ly<D, NW>::KS; ks++) {
    const bf16x8 a = k_operand<D, NW>(kt, ad, hb, ks);
#pragma unroll
    for (int qb = 0; qb < 2; qb++) {
      if (ks == 0) mfma_s_init(s[qb], a, qf[qb][ks], negm[qb]);
      else mfma_s_acc(s[qb], a, qf[qb][ks]);
    }
  }
  mfma_drain();
}

// row maximum of S over both lane halves (-inf if every column is masked)
__device__ __forceinline__ void row_max(const f32x16 (&s)[2], float (&mx)[2]) {
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    float x = s[qb][0];
#pragma unroll
    for (int r = 1; r < 16; r++) x = fmaxf(x, s[qb][r]);
    mx[qb] = fmaxf(mx[qb], halves_max(x));
  }
}

// Q fragments of the wave's rows qbase + 32qb + l32 (rows past N read as
// zero); k-step ks holds channels 16ks + 8h .. +7.
template <int D>
__device__ __forceinline__ void load_q(const uint16_t* __restrict__ Q, int g, int N, int qbase,
                                       bf16x8 (&qf)[2][D / 16]) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
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
      asm volatile("" : "+a"(qf[qb][ks]));  // held in AGPRs: only MFMAs read it
    }
  }
}

template <int D, int BQ, int BK, bool SMALLN>
__global__ __launch_bounds__(BQ) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t col_len,
    int mask_G, uint16_t* __restrict__ O, float* __restrict__ lse, int G, int N, int nq, int nk,
    float c, OutMap om) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int NW = BQ / 64;
  constexpr int SUB = BK / KT;
  using L = Ly<D, NW>;
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[L::TB];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[L::TB];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[L::TB];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[L::TB];

  int g, i;
  if (!xcd_group_tile(blockIdx.x, nq, G, g, i)) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int qbase = i * BQ + w * 64;

  Stage<D, NW> sg;
  sg.init();
  Addr<D, NW> ad;
  ad.init();

  bf16x8 qf[2][D / 16];
  load_q<D>(Q, g, N, qbase, qf);

  const int64_t rbase = static_cast<int64_t>(g % mask_G) * nq + i;
  int64_t e0 = row_ptr[rbase], e1 = row_ptr[rbase + 1];
  e0 = e0 < 0 ? 0 : (e0 > col_len ? col_len : e0);
  e1 = e1 < e0 ? e0 : (e1 > col_len ? col_len : e1);
  const int nt = static_cast<int>(e1 - e0) * SUB;

  const int head_bytes = N * L::ROWB;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(K + static_cast<int64_t>(g) * N * D), 0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(V + static_cast<int64_t>(g) * N * D), 0, head_bytes, 0x00020000);
  // a resource with no records: staging through it fetches nothing
  const __amdgpu_buffer_rsrc_t nrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(K), 0, 0, 0x00020000);

  float m[2] = {0.0f, 0.0f}, l[2] = {0.0f, 0.0f};
  f32x16 o[2][D / 32];
  f32x16 negm[2];
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    negm[qb] = f32x16{};
#pragma unroll
    for (int db = 0; db < D / 32; db++) o[qb][db] = f32x16{};
  }

  auto tile = [&](int j, int t) { return make_tile<BK>(j, t, N, nk); };
  // kv-block index of sub-tile t through a vector load (a VGPR offset the
  // compiler cannot see through keeps it off the scalar unit); indices past
  // the row repeat its last entry
  int vzero = 0;
  opaque(vzero);
  auto col_load = [&](int t) {
    const int64_t e = e0 + t / SUB;
    return col_idx[(e < e1 ? e : e1 - 1) + vzero];
  };

  // The reference comes from the first half-tile.  If a half-tile row sum
  // then overflows the bound, or a row ends with no weight, the workgroup
  // recomputes its rows on the exact path below (exact row maxima first).
  bool ovf = false;
  if (nt > 0) {
    f32x16 sA[2], sB[2];
    u32x4 pA[2][2], pB[2][2];
    bf16x8 ka[kPf + 1], va[kPf + 1];
#pragma unroll
    for (int qb = 0; qb < 2; qb++)
#pragma unroll
      for (int s2 = 0; s2 < 2; s2++) { pA[qb][s2] = u32x4{}; pB[qb][s2] = u32x4{}; }

    // prologue: K(0), K(1), V(0) resident
    Tile Tt = tile(col_idx[e0], 0);
    Tile Tn = tile(nt > 1 ? col_idx[e0 + 1 / SUB] : -1, 1);
    stage_tile<D, NW, SMALLN>(krs, sg, N, Tt.win, kb0, false);
    stage_tile<D, NW, SMALLN>(nt > 1 ? krs : nrs, sg, N, Tn.win, kb1, false);
    stage_tile<D, NW, SMALLN>(vrs, sg, N, Tt.win, vb0, true);
    int jv = col_load(2);  // sub-tile 3, read at the first odd step
    wait_loads();
    __syncthreads();

    // S_0 = K(0) half 0; pass 0 sets the reference to its row maxima
    s_half<D, NW>(ad, kb0, 0, qf, negm, sA);
    if (Tt.mask) mask_half(sA, Tt, 0, N);
    {
      float mx[2] = {-INFINITY, -INFINITY};
      row_max(sA, mx);
#pragma unroll
      for (int qb = 0; qb < 2; qb++) {
        m[qb] = mx[qb] > -INFINITY ? mx[qb] : 0.0f;
        sA[qb] -= m[qb];
        negm[qb] -= m[qb];
      }
      asm volatile("s_nop 4" ::: "memory");  // VALU-written negm before an MFMA reads it
    }
    prefetch<D, NW>(ad, kb0, vb0, 1, ka, va);
    // step 0: P_0; S_1 = K(0) half 1; no PV yet
    step<D, NW, SMALLN, 1, false, 0>(ad, sg, N, kb0, vb0, qf, negm, o, sA, sB, pA, pB, l, ovf, ka, va,
                                     nrs, 0, kb1, nrs, 0, vb1, c);
    __syncthreads();  // K(0) free for K(2)
    prefetch<D, NW>(ad, kb1, vb0, 0, ka, va);

    // Steady state.  Iteration t (sub-tile t, with K(t+1) and V(t) resident):
    //   odd step 2t+1:  P_{2t+1}; S_{2t+2} = K(t+1) half 0; O += P_{2t}.V(t)
    //                   half 0; stage V(t+1) and K(t+2)
    //   even step 2t+2: P_{2t+2}; S_{2t+3} = K(t+1) half 1; O += P_{2t+1}.V(t)
    //                   half 1; wait for the staging, barrier.
    // K(t) and V(t) live in buffer t % 2; two sub-tiles per loop trip keep
    // every buffer choice static.  Tt, Tn: tiles t, t+1.
    int t = 0;
#define BSA_ITER(KC, VC, KL, VL, KF)                                                                 \
  {                                                                                                  \
    const Tile Tk = tile(__builtin_amdgcn_readfirstlane(jv), t + 2);                                 \
    jv = col_load(t + 3);                                                                            \
    if (Tt.mask) mask_half(sB, Tt, 1, N);                                                            \
    step<D, NW, SMALLN, 0, true, 1>(ad, sg, N, KC, VC, qf, negm, o, sB, sA, pB, pA, l, ovf, ka, va,  \
                                    t + 2 < nt ? krs : nrs, Tk.win, KL, t + 1 < nt ? vrs : nrs,      \
                                    Tn.win, VL, c);                                                  \
    if (t + 1 >= nt) break;                                                                          \
    prefetch<D, NW>(ad, KC, VC, 1, ka, va);                                                          \
    if (Tn.mask) mask_half(sA, Tn, 0, N);                                                            \
    step<D, NW, SMALLN, 1, true, 0>(ad, sg, N, KC, VC, qf, negm, o, sA, sB, pA, pB, l, ovf, ka, va,  \
                                    nrs, 0, KL, nrs, 0, VL, c);                                      \
    wait_loads();                                                                                    \
    __syncthreads();                                                                                 \
    prefetch<D, NW>(ad, KF, VL, 0, ka, va);                                                          \
    Tt = Tn;                                                                                         \
    Tn = Tk;                                                                                         \
    t++;                                                                                             \
  }
    while (true) {
      BSA_ITER(kb1, vb0, kb0, vb1, kb0)  // t even
      BSA_ITER(kb0, vb1, kb1, vb0, kb1)  // t odd
    }
#undef BSA_ITER
    // last half (2nt-1): O += P_{2nt-1}.V(nt-1) half 1
    if (t & 1) pv_only<D, NW>(ad, vb1, 1, pB, o);
    else pv_only<D, NW>(ad, vb0, 1, pB, o);
    // no staging may still be landing in LDS when the buffers are reused or
    // the workgroup ends
    wait_loads();

    // a row with no weight left (every exponential underflowed) also takes
    // the exact path
#pragma unroll
    for (int qb = 0; qb < 2; qb++) ovf = ovf || !(l[qb] + __shfl_xor(l[qb], 32) > 0.0f);
    // workgroup-wide OR of the flag through the (now idle) staging buffer
    __syncthreads();
    if (lane == 0) reinterpret_cast<volatile int*>(kb0)[w] = __ballot(ovf) != 0ull;
    __syncthreads();
    ovf = false;
#pragma unroll
    for (int ww = 0; ww < NW; ww++) ovf = ovf || reinterpret_cast<volatile int*>(kb0)[ww] != 0;
    __syncthreads();
  }

  if (ovf) {
    // Exact path, one sub-tile at a time: the row maxima over every kept
    // column, then O and l against them (every score <= 0).
    load_q<D>(Q, g, N, qbase, qf);
    f32x16 sA[2];
    u32x4 pA[2][2];
    float mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int qb = 0; qb < 2; qb++) negm[qb] = f32x16{};
    asm volatile("s_nop 4" ::: "memory");
    for (int t = 0; t < nt; t++) {
      const Tile T = tile(col_idx[e0 + t / SUB], t);
      stage_tile<D, NW, SMALLN>(krs, sg, N, T.win, kb0, false);
      wait_loads();
      __syncthreads();
#pragma unroll
      for (int hb = 0; hb < 2; hb++) {
        s_half<D, NW>(ad, kb0, hb, qf, negm, sA);
        if (T.mask) mask_half(sA, T, hb, N);
        row_max(sA, mx);
      }
      __syncthreads();
    }
#pragma unroll
    for (int qb = 0; qb < 2; qb++) {
      m[qb] = mx[qb] > -INFINITY ? mx[qb] : 0.0f;
      l[qb] = 0.0f;
      negm[qb] = -m[qb];
#pragma unroll
      for (int db = 0; db < D / 32; db++) o[qb][db] = f32x16{};
    }
    asm volatile("s_nop 4" ::: "memory");
    for (int t = 0; t < nt; t++) {
      const Tile T = tile(col_idx[e0 + t / SUB], t);
      stage_tile<D, NW, SMALLN>(krs, sg, N, T.win, kb0, false);
      stage_tile<D, NW, SMALLN>(vrs, sg, N, T.win, vb0, true);
      wait_loads();
      __syncthreads();
#pragma unroll
      for (int hb = 0; hb < 2; hb++) {
        s_half<D, NW>(ad, kb0, hb, qf, negm, sA);
        if (T.mask) mask_half(sA, T, hb, N);
        float sum[2] = {0.0f, 0.0f};
        Ex ex;
#pragma unroll
        for (int e = 0; e < 32; e++) {
          exp_issue(sA, e, ex, c);
          asm volatile("s_nop 0");
          exp_retire(e, ex, sum, pA);
        }
        l[0] += sum[0];
        l[1] += sum[1];
        pv_only<D, NW>(ad, vb0, hb, pA, o);
      }
      __syncthreads();
    }
  }

#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
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
        lse[li] = lt > 0.0f ? m[qb] * c * kLn2 + logf(lt) : -INFINITY;
    }
  }
}

template <int D, int BQ, int BK>
hipError_t launch(const AttnArgs& a, hipStream_t s) {
  const int nq = (a.N + BQ - 1) / BQ, nk = (a.N + BK - 1) / BK;
  const uint32_t nwg = xcd_group_grid(nq, a.G);
  const float sm = a.sm_scale > 0.0f ? a.sm_scale : 1.0f / sqrtf(static_cast<float>(a.d));
  auto kern = a.N >= KT ? fwd_bf16_kernel<D, BQ, BK, false> : fwd_bf16_kernel<D, BQ, BK, true>;
  kern<<<nwg, BQ, 0, s>>>(static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                          static_cast<const uint16_t*>(a.V), a.row_ptr, a.col_idx, a.col_len,
                          a.mask_G, a.O, a.lse, a.G, a.N, nq, nk, sm * kLog2e, a.out);
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
