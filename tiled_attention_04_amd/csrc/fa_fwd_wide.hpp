// fa_fwd_wide.hpp -- the 16-bit attention forward for head_dim 129..256
// (gfx950): one pass over the keys with a hand-ordered, software-pipelined
// step, one wave per SIMD.
//
// Method: as in fa_fwd_kernels.hpp -- the FlashAttention-2 forward of
// "[CS336] Assignment 2: Systems", section "FlashAttention V2 / Forward
// Pass", and of "Understanding Triton Tutorials Part 2", section "Fused
// Attention 2": Q resident, K/V tiles streamed, running max and sum, exp2
// with log2(e) folded into the scale, O divided by the row sum once at the
// end, logsumexp emitted, causal tiles above the diagonal skipped.
//
// What differs from the 32-row kernel of fa_fwd_kernels.hpp (MI355X design,
// not from the pages):
//  * at D = 256 the O^T accumulator alone takes 128 registers and Q another
//    64: with compiler-placed MFMAs the scores, weights and operand
//    fragments no longer fit beside them.  Here the MFMAs are inline
//    assembly with fixed register classes, so Q and the accumulator live in
//    AGPRs (only the matrix core reads them) and everything else in VGPRs:
//    one wave per SIMD (NW = 4), no spills, one pass over the keys;
//  * the step is software-pipelined over three tiles so that all of a wave's
//    matrix work of one step overlaps all of its softmax work: step t issues
//      P(t) V(t)                (MFMAs, V^T by transposing reads)
//      softmax(t + 1)           (row max, lazy rescale decision, exp2, packing, sum)
//      S(t + 2) = K(t + 2) Q^T  (MFMAs, K by 128-bit reads)
//    with no dependence between the three parts, in an instruction order
//    fixed by hand: one MFMA per slot, each followed by a short unit of the
//    softmax.  With one wave per SIMD the VALU work has to sit in the shadows
//    of the wave's own MFMAs; above head_dim 128 each step carries enough
//    MFMAs for it.  The rescale of the accumulator that softmax(t + 1) may
//    ask for is applied at the start of step t + 1, after P(t) V(t) is in;
//  * K and V have two LDS stages each, filled direct-to-LDS: K(t + 3) and
//    V(t + 1) are loaded during step t.  The stage of every access is a
//    compile-time parity, so the compiler can tell the stages apart and
//    never makes a read wait for the loads into the other stage;
//  * every step is a full one: near the end of the workgroup's key range the
//    softmax of tile t + 1 >= t1 and the scores of tile t + 2 >= t1 run on
//    tiles that are not part of it; the mask hides all of their keys from
//    every row, so they change neither m, l nor the accumulator (one step
//    body, one register allocation).
//
// The body also compiles for head_dim <= 128 with eight waves (two per
// SIMD); there it is slower than the compiler-scheduled 32-row kernel, whose
// softmax VALU work per MFMA is the larger share, so only the wide
// instantiations are used.
#pragma once
#include "fa_fwd_kernels.hpp"
#include "fa_mfma_asm.hpp"

namespace fa {

template <typename T, int D, int NW_>
struct TileWide {
  static constexpr int NW = NW_;          // waves per workgroup
  static constexpr int NT = 64 * NW;      // threads per workgroup
  static constexpr int BM = 32 * NW;      // query rows per workgroup
  static constexpr int BN = 64;           // keys per tile
  static constexpr int KSTEPS = D / 16;   // k-steps of S^T (16 dims each)
  static constexpr int DBLK = (D + 31) / 32;  // 32-dim blocks of O^T
  static constexpr int KROW = D * 2 + 16;                  // bytes, = 16 mod 256
  static constexpr int VROW = tr_row_stride(DBLK * 64);    // bytes, 64 or 192 mod 256
  static constexpr int KSLOTS = KROW / 16, VSLOTS = VROW / 16;
  static constexpr int KINSTR = BN * KSLOTS / 64, VINSTR = BN * VSLOTS / 64;
  static constexpr int KPER = (KINSTR + NW - 1) / NW, VPER = (VINSTR + NW - 1) / NW;
  static constexpr int KBYTES = BN * KROW, VBYTES = BN * VROW;
  static_assert(D % 16 == 0 && D <= 256, "head_dim padding of the wide kernel");
  static_assert((BN * KSLOTS) % 64 == 0 && (BN * VSLOTS) % 64 == 0, "whole wave loads");
};

template <typename T, int D, int NW_>
__device__ __forceinline__ void fa_fwd_wide_body(const FwdArgs& a) {
  using G = TileWide<T, D, NW_>;
  using M = Mfma<T>;
  using X = MfmaPin<T>;
  typedef typename M::frag frag;
  constexpr int BN = G::BN, KSTEPS = G::KSTEPS, DBLK = G::DBLK, NW = G::NW;
  constexpr int KROW = G::KROW, VROW = G::VROW;
  constexpr int NPV = 4 * DBLK;     // P.V MFMAs per step (four 16-key steps per 32-dim block)
  constexpr int NS = 2 * KSTEPS;    // S MFMAs per step (two 32-key blocks)

  // separate objects per stage: the compiler then sees that a step's operand
  // reads never touch the stages its direct-to-LDS loads are filling
  __shared__ __attribute__((aligned(1024))) char k_st0[G::KBYTES];
  __shared__ __attribute__((aligned(1024))) char k_st1[G::KBYTES];
  __shared__ __attribute__((aligned(1024))) char v_st0[G::VBYTES];
  __shared__ __attribute__((aligned(1024))) char v_st1[G::VBYTES];
  // K(j) and V(j) live in stage (j - t0) % 2.  Stages are picked by
  // compile-time parities only: the compiler then knows which object a read
  // touches and does not wait for the direct-to-LDS loads into the other.
  auto kstage = [&](auto pc) -> FA_LDS char* {
    if constexpr (decltype(pc)::value % 2 == 0) return (FA_LDS char*)k_st0;
    else return (FA_LDS char*)k_st1;
  };
  auto vstage = [&](auto pc) -> FA_LDS char* {
    if constexpr (decltype(pc)::value % 2 == 0) return (FA_LDS char*)v_st0;
    else return (FA_LDS char*)v_st1;
  };
  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;   // query column owned by this lane
  const int hi = lane >> 5;    // which half of the 32x32 result rows

  int bh, qt, split;
  map_workgroup(a, blockIdx.x, bh, qt, split);
  const int b = bh / a.heads, h = bh - b * a.heads;
  const T* qg = (const T*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
  const T* kg = (const T*)a.k + (int64_t)b * a.k_sb + (int64_t)h * a.k_sh;
  const T* vg = (const T*)a.v + (int64_t)b * a.v_sb + (int64_t)h * a.v_sh;
  T* og = (T*)a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh;

  const int q0 = qt * G::BM;
  const int qw = q0 + wave * 32;  // first query row of this wave
  const bool wave_live = qw < a.seq_q;
  const int wave_rows = wave_live ? min(32, a.seq_q - qw) : 0;

  // keys this workgroup must visit (causal: up to its last real query), and
  // with key splitting its share [t0, t1) of those 64-key tiles; keys at or
  // past key_end belong to no tile of the share
  const int kv_end = a.causal ? min(a.seq_k, min(a.seq_q, q0 + G::BM)) : a.seq_k;
  const int n_all = (kv_end + BN - 1) / BN;
  const int chunk = (n_all + a.n_splits - 1) / a.n_splits;
  const int t0 = min(n_all, split * chunk);
  const int t1 = min(n_all, t0 + chunk);
  const int key_end = min(a.seq_k, t1 * BN);
  // last key this lane's row may see
  const int key_lim = a.causal ? min(key_end - 1, qw + l32) : key_end - 1;

  // ---- resident Q fragment (B operand of S^T), moved to AGPRs once
  frag qf[KSTEPS];
  {
    const int32_t nrec = wave_rows > 0 ? (wave_rows - 1) * (int32_t)a.q_ss * 2 + a.head_dim * 2 : 0;
    const auto rq = make_rsrc(qg + (int64_t)(wave_live ? qw : 0) * a.q_ss, nrec);
    const uint32_t sign = a.neg_scale ? 0x80008000u : 0u;
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
      const int col = st * 16 + hi * 8;
      const uint32_t off = col < a.head_dim ? (uint32_t)(l32 * (int32_t)a.q_ss * 2 + col * 2)
                                            : kOutOfRange;
      u32x4_t raw = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
      raw ^= (u32x4_t){sign, sign, sign, sign};
      qf[st] = __builtin_bit_cast(frag, raw);
    }
  }
  pin_agpr<KSTEPS>(qf);

  // ---- direct-to-LDS tile loads (per-lane offsets are tile independent);
  // rows >= seq_k and dims >= head_dim land as zeros
  uint32_t koff[G::KPER], voff[G::VPER];
#pragma unroll
  for (int n = 0; n < G::KPER; ++n) {
    const int slot = (wave + NW * n) * 64 + lane;
    const int row = slot / G::KSLOTS, ch = slot - (slot / G::KSLOTS) * G::KSLOTS;
    koff[n] = ch * 8 < a.head_dim ? (uint32_t)(row * (int32_t)a.k_ss * 2 + ch * 16) : kOutOfRange;
  }
#pragma unroll
  for (int n = 0; n < G::VPER; ++n) {
    const int slot = (wave + NW * n) * 64 + lane;
    const int row = slot / G::VSLOTS, ch = slot - (slot / G::VSLOTS) * G::VSLOTS;
    voff[n] = ch * 8 < a.head_dim ? (uint32_t)(row * (int32_t)a.v_ss * 2 + ch * 16) : kOutOfRange;
  }
  // (called for tiles j < t1 only, so a tile holds at least one key row)
  auto issue_k = [&](int j, FA_LDS char* dst) {
    const int key0 = j * BN;
    const int rows = min(BN, a.seq_k - key0);
    const auto rk = make_rsrc(kg + (int64_t)key0 * a.k_ss, (rows - 1) * (int32_t)a.k_ss * 2 + a.head_dim * 2);
#pragma unroll
    for (int n = 0; n < G::KPER; ++n)
      if (wave + NW * n < G::KINSTR)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (FA_LDS void*)(dst + (wave + NW * n) * 1024), 16,
                                                 koff[n], 0, 0, 0);
  };
  auto issue_v = [&](int j, FA_LDS char* dst) {
    const int key0 = j * BN;
    const int rows = min(BN, a.seq_k - key0);
    const auto rv = make_rsrc(vg + (int64_t)key0 * a.v_ss, (rows - 1) * (int32_t)a.v_ss * 2 + a.head_dim * 2);
#pragma unroll
    for (int n = 0; n < G::VPER; ++n)
      if (wave + NW * n < G::VINSTR)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (FA_LDS void*)(dst + (wave + NW * n) * 1024), 16,
                                                 voff[n], 0, 0, 0);
  };

  // ---- online-softmax state (per lane: query l32 of the wave)
  f32x16_t acc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) acc[db] = (f32x16_t){};
  float m = -INFINITY;   // reference max (base-2 scaled units)
  float l = 0.f;         // partial row sum of the rounded weights
  float alpha = 1.f;     // rescale of the accumulator pending for the next step
  const float c = a.c;

  const int k_lane = l32 * KROW + hi * 16;
  const int s16 = lane & 15;
  const int v_lane = (4 * hi + (s16 >> 2)) * VROW + (16 * ((lane >> 4) & 1) + 4 * (s16 & 3)) * 2;

  // V^T fragment j of the tile in vb (16-key step j / DBLK, 32-dim block j % DBLK)
  auto v_frag = [&](FA_LDS char* vb, int j) {
    FA_LDS char* p0 = vb + v_lane + (16 * (j / DBLK)) * VROW + (j % DBLK) * 64;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)p0);
    const i16x4_t up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)(p0 + 8 * VROW));
    const u32x4_t vraw = {__builtin_bit_cast(u32x2_t, lo)[0], __builtin_bit_cast(u32x2_t, lo)[1],
                          __builtin_bit_cast(u32x2_t, up)[0], __builtin_bit_cast(u32x2_t, up)[1]};
    return __builtin_bit_cast(frag, vraw);
  };
  // K fragment j of the tile in kb (32-key block j / KSTEPS, 16-dim step j % KSTEPS)
  auto k_frag = [&](FA_LDS char* kb, int j) {
    return __builtin_bit_cast(
        frag, *(FA_LDS u32x4_t*)(kb + k_lane + (j / KSTEPS) * 32 * KROW + (j % KSTEPS) * 32));
  };
  // packed P of 16-key step u: the B operand of O^T += V^T P^T
  auto p_frag = [&](const uint32_t (&pk)[2][8], int u) {
    const u32x4_t r = {pk[u >> 1][4 * (u & 1) + 0], pk[u >> 1][4 * (u & 1) + 1],
                       pk[u >> 1][4 * (u & 1) + 2], pk[u >> 1][4 * (u & 1) + 3]};
    return __builtin_bit_cast(frag, r);
  };
  // S^T = K Q^T for the K tile in kb, MFMAs in order (prologue only)
  auto scores = [&](FA_LDS char* kb, f32x16_t (&s)[2]) {
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const frag kf = k_frag(kb, kb2 * KSTEPS + st);
        if (st == 0) X::first(s[kb2], kf, qf[st]);
        else X::next(s[kb2], kf, qf[st]);
      }
  };
  // masks of tile t (end of the share's keys, causal diagonal) as one
  // uniform branch; a tile at or past t1 is masked whole
  auto mask = [&](int t, f32x16_t (&s)[2]) {
    const int key0 = t * BN;
    if ((key0 + BN > key_end) || (a.causal && key0 + BN - 1 > qw)) {
      // key key0 + cr + 4 hi (cr = kb2 32 + 8 (r / 4) + r % 4, a constant)
      // is visible iff cr <= dl
      const int dl = key_lim - key0 - 4 * hi;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cr = kb2 * 32 + 8 * (r >> 2) + (r & 3);
          s[kb2][r] = cr <= dl ? s[kb2][r] : -INFINITY;
        }
    }
  };

  // operand fragments in flight ahead of their MFMAs (slots)
  constexpr int PDV = 3, PDK = 3;

  // One step t (stage parity P = (t - t0) & 1 known at compile time).  On
  // entry: P(t) in pk_c, S(t + 1) in s_c; on exit P(t + 1) in pk_n and
  // S(t + 2) in s_n.
  //
  // Slots: the NPV MFMAs of P(t) V(t), then the NS of S(t + 2), each slot one
  // MFMA followed by a unit of the softmax of tile t + 1 (scheduling barriers
  // between slots keep the order).  Units: the row max and rescale decision
  // in three parts, then two half units per pair of scores -- "scale,
  // subtract, exp2 of the first" and "exp2 of the second, then round, pack
  // and sum the previous pair" -- and a last unit that packs pair 15.
  // Operand fragments are read from LDS PDV / PDK slots ahead of their MFMAs.
  auto step = [&](int t, auto parity, f32x16_t (&s_c)[2], f32x16_t (&s_n)[2],
                  uint32_t (&pk_c)[2][8], uint32_t (&pk_n)[2][8]) {
    constexpr int P = decltype(parity)::value;
    using Cur = std::integral_constant<int, P>;
    using Nxt = std::integral_constant<int, 1 - P>;
    // S(t + 1) was last written by MFMAs: drain them before the VALU reads below
    mfma_drain_v(s_c[0], s_c[1]);
    // the rescale that softmax(t) asked for, now that P(t - 1) V(t - 1) is in
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
      mfma_drain_a<DBLK>(acc);
      // one 16-register block at a time (each block's reads are ordered after
      // the previous block's writes), so at most 16 values sit in VGPRs
      static_for<0, DBLK>([&](auto ic) {
        constexpr int db = decltype(ic)::value;
        acc[db] *= alpha;
        if constexpr (db + 1 < DBLK) asm volatile("" : "+a"(acc[db]), "+a"(acc[db + 1]));
      });
      alpha = 1.f;
      mfma_drain_a<DBLK>(acc);  // VALU writes before the next MFMA reads them
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's K(t + 2) and V(t) loads have landed
    __syncthreads();                // ... everyone's; and K(t + 1), V(t - 1) are free
#ifdef FA_LDS_POISON
    lds_poison<G::NT>(kstage(Nxt{}), G::KBYTES);
    lds_poison<G::NT>(vstage(Nxt{}), G::VBYTES);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#endif
    if (t + 3 < t1) issue_k(t + 3, kstage(Nxt{}));
    if (t + 1 < t1) issue_v(t + 1, vstage(Nxt{}));
    mask(t + 1, s_c);
    FA_LDS char* const vb = vstage(Cur{});
    FA_LDS char* const kb = kstage(Cur{});

    float mt[11];                  // partial maxima of the tree
    float msub = 0.f;
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    float ex[2][16];               // exp2 results waiting to be packed
    auto stat_part = [&](auto kc) {
      constexpr int K = decltype(kc)::value;
      if constexpr (K == 0) {
        static_for<0, 5>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          mt[i] = __builtin_elementwise_maximum(
              s_c[0][3 * i], __builtin_elementwise_maximum(s_c[0][3 * i + 1], s_c[0][3 * i + 2]));
          pin(mt[i]);
        });
      } else if constexpr (K == 1) {
        static_for<0, 5>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          mt[5 + i] = __builtin_elementwise_maximum(
              s_c[1][3 * i], __builtin_elementwise_maximum(s_c[1][3 * i + 1], s_c[1][3 * i + 2]));
          pin(mt[5 + i]);
        });
        mt[10] = __builtin_elementwise_maximum(s_c[0][15], s_c[1][15]);
        pin(mt[10]);
      } else {
        const float u0 = __builtin_elementwise_maximum(mt[0], __builtin_elementwise_maximum(mt[1], mt[2]));
        const float u1 = __builtin_elementwise_maximum(mt[3], __builtin_elementwise_maximum(mt[4], mt[5]));
        const float u2 = __builtin_elementwise_maximum(mt[6], __builtin_elementwise_maximum(mt[7], mt[8]));
        const float u3 = __builtin_elementwise_maximum(mt[9], mt[10]);
        const float mx = xlane_max(__builtin_elementwise_maximum(__builtin_elementwise_maximum(u0, u1),
                                                                 __builtin_elementwise_maximum(u2, u3)));
        const float m_new = __builtin_elementwise_maximum(m, mx * c);
        const bool upd = m_new > m + kRescaleLog2;
        alpha = upd ? fast_exp2(m - m_new) : 1.f;  // exp2(-inf) = 0 on the first visible tile
        l = upd ? l * alpha : l;
        m = upd ? m_new : m;
        msub = (m == -INFINITY) ? 0.f : m;
        pin(msub);
        pin(l);
      }
    };
    // pair q = 0..15: key block q / 8, scores 2 (q % 8) and 2 (q % 8) + 1
    auto half0 = [&](auto qc) {
      constexpr int q = decltype(qc)::value, kb2 = q / 8, r = 2 * (q % 8);
      ex[kb2][r] = fast_exp2(__builtin_fmaf(s_c[kb2][r], c, -msub));
      ex[kb2][r + 1] = __builtin_fmaf(s_c[kb2][r + 1], c, -msub);
      pin(ex[kb2][r]);
      pin(ex[kb2][r + 1]);
    };
    auto pack = [&](auto qc) {
      constexpr int q = decltype(qc)::value, kb2 = q / 8, r = 2 * (q % 8);
      pk_n[kb2][r >> 1] = M::pack2(ex[kb2][r], ex[kb2][r + 1]);
      part[(r >> 1) & 3] = M::sum2(pk_n[kb2][r >> 1], part[(r >> 1) & 3]);
      pin(pk_n[kb2][r >> 1]);
      pin(part[(r >> 1) & 3]);
    };
    auto half1 = [&](auto qc) {
      constexpr int q = decltype(qc)::value, kb2 = q / 8, r = 2 * (q % 8);
      ex[kb2][r + 1] = fast_exp2(ex[kb2][r + 1]);
      pin(ex[kb2][r + 1]);
      if constexpr (q > 0) pack(std::integral_constant<int, q - 1>{});
    };
    constexpr int NU = 3 + 32 + 1;  // units of the step
    auto unit = [&](auto nc) {
      constexpr int n = decltype(nc)::value;
      if constexpr (n < 3) {
        stat_part(std::integral_constant<int, n>{});
      } else if constexpr (n < NU - 1) {
        constexpr int q = (n - 3) / 2;
        if constexpr (((n - 3) & 1) == 0) half0(std::integral_constant<int, q>{});
        else half1(std::integral_constant<int, q>{});
      } else {
        pack(std::integral_constant<int, 15>{});
      }
    };
    // placement: units 0..18 (row max and pairs 0..7, all of key block 0)
    // over the P(t) V(t) slots, units 19..35 over the S(t + 2) slots; key
    // block 0 of S(t + 2) then reuses the registers of key block 0 of S(t + 1)
    constexpr int NU0 = 19;
    auto units_at = [&](auto slotc, auto segc) {
      constexpr int slot = decltype(slotc)::value;
      if constexpr (decltype(segc)::value == 0) {
        static_for<0, NU0>([&](auto nc) {
          if constexpr ((decltype(nc)::value * NPV) / NU0 == slot) unit(nc);
        });
      } else {
        static_for<NU0, NU>([&](auto nc) {
          if constexpr (((decltype(nc)::value - NU0) * NS) / (NU - NU0) == slot) unit(nc);
        });
      }
    };
    using Seg0 = std::integral_constant<int, 0>;
    using Seg1 = std::integral_constant<int, 1>;

    // ---- P(t) V(t): slot j = V^T fragment j
    frag vq[NPV], kq[NS];
    static_for<0, PDV>([&](auto mc) { vq[decltype(mc)::value] = v_frag(vb, decltype(mc)::value); });
    static_for<0, NPV>([&](auto jc) {
      constexpr int j = decltype(jc)::value, u = j / DBLK, db = j % DBLK;
      if constexpr (j + PDV < NPV) vq[j + PDV] = v_frag(vb, j + PDV);
      // the first K fragments of S(t + 2) during the last slots
      if constexpr (j >= NPV - PDK) kq[j - (NPV - PDK)] = k_frag(kb, j - (NPV - PDK));
      X::acc(acc[db], vq[j], p_frag(pk_c, u));
      units_at(jc, Seg0{});
      __builtin_amdgcn_sched_barrier(0);
    });
    // ---- S(t + 2) = K(t + 2) Q^T: slot j = K fragment j (key block j / KSTEPS)
    static_for<0, NS>([&](auto jc) {
      constexpr int j = decltype(jc)::value, kb2 = j / KSTEPS, st = j % KSTEPS;
      if constexpr (j + PDK < NS) kq[j + PDK] = k_frag(kb, j + PDK);
      if constexpr (st == 0) X::first(s_n[kb2], kq[j], qf[st]);
      else X::next(s_n[kb2], kq[j], qf[st]);
      units_at(jc, Seg1{});
      __builtin_amdgcn_sched_barrier(0);
    });
    l += (part[0] + part[1]) + (part[2] + part[3]);
  };

  if (t1 > t0) {
    // ---- prologue: S(t0) -> P(t0), and S(t0 + 1)
    f32x16_t s0[2], s1[2];
    uint32_t p0[2][8], p1[2][8];
    issue_k(t0, kstage(Even{}));
    issue_v(t0, vstage(Even{}));
    if (t0 + 1 < t1) issue_k(t0 + 1, kstage(Odd{}));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    scores(kstage(Even{}), s0);
    mfma_drain_v(s0[0], s0[1]);
    mask(t0, s0);
    {
      const float mx = xlane_max(row_max32(s0[0], s0[1]));
      m = mx * c;  // the first tile: the reference starts at its max (-inf if none visible)
      const float msub = (m == -INFINITY) ? 0.f : m;
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float e0 = fast_exp2(__builtin_fmaf(s0[kb2][r], c, -msub));
          const float e1 = fast_exp2(__builtin_fmaf(s0[kb2][r + 1], c, -msub));
          p0[kb2][r >> 1] = M::pack2(e0, e1);
          part[(r >> 1) & 3] = M::sum2(p0[kb2][r >> 1], part[(r >> 1) & 3]);
        }
      l = (part[0] + part[1]) + (part[2] + part[3]);
    }
    scores(kstage(Odd{}), s1);  // S(t0 + 1), masked whole later if t0 + 1 >= t1
    __syncthreads();            // K(t0) consumed by all waves before K(t0 + 2) is loaded over it
#ifdef FA_LDS_POISON
    lds_poison<G::NT>(kstage(Even{}), G::KBYTES);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#endif
    if (t0 + 2 < t1) issue_k(t0 + 2, kstage(Even{}));

    // ---- every step a full one; even steps read S from set 1 and write set 0
    for (int t = t0;; t += 2) {
      step(t, Even{}, s1, s0, p0, p1);
      if (t + 1 >= t1) break;
      step(t + 1, Odd{}, s0, s1, p1, p0);
      if (t + 2 >= t1) break;
    }
    mfma_drain_a<DBLK>(acc);
    __syncthreads();  // every wave's last reads of the K stages are done
  }

  // ---- epilogue: O = acc / l, lse = ln2 * (m + log2 l)
  if (!wave_live) return;
  const float l_tot = xlane_sum(l);
  if (a.n_splits > 1) {
    // fp32 partials of this key share; a row that saw none of its keys has
    // l = 0 and gets O_r = 0, lse_r = -inf (weight 0 in the merge)
    const bool seen = l_tot > 0.f;
    const float inv = seen ? 1.0f / l_tot : 0.f;
    const int64_t row0 = ((int64_t)split * a.n_bh + bh) * a.seq_q + qw;
    const auto rp = make_rsrc(a.part_o + row0 * a.head_dim, wave_rows * a.head_dim * 4);
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * hi;
        const uint32_t off = (d0 < a.head_dim && l32 < wave_rows)
                                 ? (uint32_t)((l32 * a.head_dim + d0) * 4) : kOutOfRange;
        const u32x4_t w = {__float_as_uint(acc[db][4 * g + 0] * inv),
                           __float_as_uint(acc[db][4 * g + 1] * inv),
                           __float_as_uint(acc[db][4 * g + 2] * inv),
                           __float_as_uint(acc[db][4 * g + 3] * inv)};
        __builtin_amdgcn_raw_buffer_store_b128(w, rp, off, 0, 0);
      }
    if (hi == 0 && l32 < wave_rows)
      a.part_lse[row0 + l32] = seen ? (m + __log2f(l_tot)) * kLn2 : -INFINITY;
    return;
  }
  const float inv = 1.0f / l_tot;
  const int32_t onrec = (wave_rows - 1) * (int32_t)a.o_ss * 2 + a.head_dim * 2;
  const auto ro = make_rsrc(og + (int64_t)qw * a.o_ss, onrec);
  // O through LDS: the barrier after the key loop has freed the K stages,
  // each of which holds two waves' 32 output rows at the K row stride; then every
  // lane stores whole 16-byte pieces of rows, consecutive lanes on
  // consecutive bytes
  static_assert(G::KBYTES == 2 * 32 * KROW, "two waves' rows per K stage");
  FA_LDS char* const ob = (wave < 2 ? (FA_LDS char*)k_st0 : (FA_LDS char*)k_st1) + (wave & 1) * 32 * KROW;
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = db * 32 + 8 * g + 4 * hi;
      const u32x2_t w = {M::pack2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv),
                         M::pack2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
      *(FA_LDS u32x2_t*)(ob + l32 * KROW + d0 * 2) = w;
    }
  constexpr int CPR = D / 8;  // 16-byte pieces per row
#pragma unroll
  for (int c0 = 0; c0 < 32 * CPR; c0 += 64) {
    const int c = c0 + lane;
    const int row = c / CPR, col = c - (c / CPR) * CPR;
    const u32x4_t w = *(FA_LDS u32x4_t*)(ob + row * KROW + col * 16);
    const uint32_t off = (row < wave_rows && col * 8 < a.head_dim)
                             ? (uint32_t)(row * (int32_t)a.o_ss * 2 + col * 16) : kOutOfRange;
    __builtin_amdgcn_raw_buffer_store_b128(w, ro, off, 0, 0);
  }
  if (hi == 0 && a.lse != nullptr && l32 < wave_rows)
    a.lse[(int64_t)bh * a.seq_q + qw + l32] = (m + __log2f(l_tot)) * kLn2;
}

}  // namespace fa
