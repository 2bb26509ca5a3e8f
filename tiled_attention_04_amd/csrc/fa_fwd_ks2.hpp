// fa_fwd_ks2.hpp -- the 16-bit attention forward for small grids, with each
// query tile's keys split between two wave groups of one workgroup.
//
// Method: as in fa_fwd_kernels.hpp -- the FlashAttention-2 forward of
// "[CS336] Assignment 2: Systems", section "FlashAttention V2 / Forward
// Pass", and of "Understanding Triton Tutorials Part 2", section "Fused
// Attention 2" -- run twice over disjoint key sets, then the two running
// states (m, l, O) are merged exactly as the online softmax rescales one
// state by another: with M = max(m0, m1), O = O0 2^(m0 - M) + O1 2^(m1 - M)
// and l likewise.
//
// MI355X design (not from the pages): a grid of a few hundred 4-wave
// workgroups leaves each wave alone on its SIMD for a long chain of key
// tiles (fp16, 16 heads, 1000 queries x 1537 keys, head_dim 64: 128
// workgroups of 25 key tiles each; bf16 [4, 12, 2048] causal: a tail of 32
// tiles).
// Here a workgroup of 8 waves serves the same 128 query rows: waves 0-3
// (group 0) walk the even key tiles of the query tile, waves 4-7 (group 1)
// the odd ones, two waves per SIMD, half the chain each, with no workspace
// and no second launch; at the end group 1 hands its state to group 0
// through LDS and group 0 writes O and lse.  Each group runs the two-stage
// step of the 4-wave kernel; the K tiles of both groups in one stage parity
// form one LDS object, the V tiles another (four objects, picked by
// compile-time parities, so that no read waits for a load into another
// object).
#pragma once
#include "fa_fwd_kernels.hpp"

namespace fa {

template <typename T, int D, bool XB>
__device__ __forceinline__ void fa_fwd_ks2_body(const FwdArgs& a) {
  using G = Tile16<T, D, 4, XB>;  // one key group: 4 waves x 32 query rows
  using M = Mfma<T>;
  typedef typename M::frag frag;
  constexpr int BN = G::BN, KSTEPS = G::KSTEPS, DBLK = G::DBLK, NWG = 4;
  constexpr int KROW = G::KROW, VROW = G::VROW;
  constexpr bool kOnesCol = (D % 32) != 0 || XB;  // row sum on the matrix core
  constexpr int E = 16 * DBLK + 2;                // floats per lane handed over
  static_assert(64 * E * 4 <= 2 * G::KBYTES && 64 * E * 4 <= 2 * G::VBYTES &&
                    G::OBYTES <= 2 * G::KBYTES && G::OBYTES <= 2 * G::VBYTES,
                "one wave pair's hand-over and one wave's output rows fit any of the four objects");

  struct Tag;
  // stage parity p: group g's K tile at g * KBYTES of kstage(p), its V tile
  // at g * VBYTES of vstage(p)
  auto kstage = [&](auto pc) -> FA_LDS char* {
    return lds_object<Tag, decltype(pc)::value % 2, 2 * G::KBYTES>();
  };
  auto vstage = [&](auto pc) -> FA_LDS char* {
    return lds_object<Tag, 2 + decltype(pc)::value % 2, 2 * G::VBYTES>();
  };
  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  // object i of the four (K even, K odd, V even, V odd), for the hand-over
  // and the output staging after the key loop
  auto object = [&](int i) -> FA_LDS char* {
    return i == 0 ? kstage(Even{}) : i == 1 ? kstage(Odd{}) : i == 2 ? vstage(Even{}) : vstage(Odd{});
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;   // key group
  const int wg = wave & 3;     // row block (and wave within the group)
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bh, qt, split;
  map_workgroup(a, blockIdx.x, bh, qt, split);
  const int b = bh / a.heads, h = bh - b * a.heads;

  const T* qg = (const T*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
  const T* kg = (const T*)a.k + (int64_t)b * a.k_sb + (int64_t)h * a.k_sh;
  const T* vg = (const T*)a.v + (int64_t)b * a.v_sb + (int64_t)h * a.v_sh;
  T* og = (T*)a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh;

  const int q0 = qt * G::BM;
  const int qw = q0 + wg * 32;
  const int my_q = qw + l32;
  const int key_lim = a.causal ? min(a.seq_k - 1, my_q) : a.seq_k - 1;
  const bool wave_live = qw < a.seq_q;
  const int wave_rows = wave_live ? min(32, a.seq_q - qw) : 0;

  // key tiles of the query tile (no key splitting across workgroups here);
  // group g takes tiles t0 + 2 j + g, j < Jg; both groups run J0 steps
  const int kv_end = a.causal ? min(a.seq_k, min(a.seq_q, q0 + G::BM)) : a.seq_k;
  const int t0 = 0, t1 = (kv_end + BN - 1) / BN;
  const int Jg = max(0, (t1 - t0 - grp + 1) / 2);
  const int J0 = (t1 - t0 + 1) / 2;
  auto tile = [&](int j) { return t0 + 2 * j + grp; };

  // ---- resident Q fragment (both groups load their rows)
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

  // ---- direct-to-LDS tile loads: each group's 4 waves load its tiles
  uint32_t koff[G::KPER], voff[G::VPER];
  bool vlive[G::VPER];
#pragma unroll
  for (int n = 0; n < G::KPER; ++n) {
    const int slot = (wg + NWG * n) * 64 + lane;
    const int row = slot / G::KSLOTS, ch = slot - (slot / G::KSLOTS) * G::KSLOTS;
    koff[n] = ch * 8 < a.head_dim ? (uint32_t)(row * (int32_t)a.k_ss * 2 + ch * 16) : kOutOfRange;
  }
#pragma unroll
  for (int n = 0; n < G::VPER; ++n) {
    const int slot = (wg + NWG * n) * 64 + lane;
    const int row = slot / G::VSLOTS, ch = slot - (slot / G::VSLOTS) * G::VSLOTS;
    voff[n] = ch * 8 < a.head_dim ? (uint32_t)(row * (int32_t)a.v_ss * 2 + ch * 16) : kOutOfRange;
    vlive[n] = ch * 8 < D;
  }
  auto issue_k = [&](int j, auto pc) {
    const int key0 = tile(j) * BN;
    const int rows = min(BN, a.seq_k - key0);
    const auto rk = make_rsrc(kg + (int64_t)key0 * a.k_ss, (rows - 1) * (int32_t)a.k_ss * 2 + a.head_dim * 2);
    FA_LDS char* kb = kstage(pc) + grp * G::KBYTES;
#pragma unroll
    for (int n = 0; n < G::KPER; ++n)
      if (wg + NWG * n < G::KINSTR)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (FA_LDS void*)(kb + (wg + NWG * n) * 1024), 16,
                                                 koff[n], 0, 0, 0);
  };
  auto issue_v = [&](int j, auto pc) {
    const int key0 = tile(j) * BN;
    const int rows = min(BN, a.seq_k - key0);
    const auto rv = make_rsrc(vg + (int64_t)key0 * a.v_ss, (rows - 1) * (int32_t)a.v_ss * 2 + a.head_dim * 2);
    FA_LDS char* vb = vstage(pc) + grp * G::VBYTES;
#pragma unroll
    for (int n = 0; n < G::VPER; ++n)
      if (wg + NWG * n < G::VINSTR && (!kOnesCol || vlive[n]))
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (FA_LDS void*)(vb + (wg + NWG * n) * 1024), 16,
                                                 voff[n], 0, 0, 0);
  };
  // (row-sum column) V columns D..32 DBLK - 1 of both groups' stages: 1.0 in
  // column D, zeros after it; written once, never loaded over
  auto pad_cols = [&](auto pc) {
    if constexpr (kOnesCol) {
      constexpr int C0 = D / 8, NC = 4 * DBLK - D / 8;
      for (int i = tid; i < 2 * BN * NC; i += 2 * G::NT) {
        const int g2 = i / (BN * NC), r = i - g2 * (BN * NC);
        const int row = r / NC, chk = C0 + r % NC;
        const u32x4_t val = {chk == C0 ? M::kOneBits : 0u, 0u, 0u, 0u};
        *(FA_LDS u32x4_t*)(vstage(pc) + g2 * G::VBYTES + row * VROW + chk * 16) = val;
      }
    }
  };
  if constexpr (kOnesCol) {
    pad_cols(Even{});
    pad_cols(Odd{});
  }

  // ---- online-softmax state
  f32x16_t acc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) acc[db] = (f32x16_t){};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c = a.c;

  const int k_lane = l32 * KROW + hi * 16;
  const int s16 = lane & 15;
  const int v_lane = (4 * hi + (s16 >> 2)) * VROW + (16 * ((lane >> 4) & 1) + 4 * (s16 & 3)) * 2;

  auto scores = [&](auto pc, f32x16_t (&s)[2]) {
    FA_LDS char* kb = kstage(pc) + grp * G::KBYTES;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) s[kb2] = (f32x16_t){};
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const frag kf = __builtin_bit_cast(
            frag, *(FA_LDS u32x4_t*)(kb + k_lane + kb2 * 32 * KROW + st * 32));
        s[kb2] = M::mma(kf, qf[st], s[kb2]);
      }
  };

  // masks, row max and the lazy rescale for key tile kt (as in the 4-wave kernel)
  auto stats = [&](int kt, f32x16_t (&s)[2]) {
    const int key0 = kt * BN;
    const bool need_mask = (key0 + BN > a.seq_k) || (a.causal && key0 + BN - 1 > qw);
    if (need_mask) {
      const int dl = key_lim - key0 - 4 * hi;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cr = kb2 * 32 + 8 * (r >> 2) + (r & 3);
          s[kb2][r] = cr <= dl ? s[kb2][r] : -INFINITY;
        }
    }
    float mx = row_max32(s[0], s[1]);
    mx = xlane_max(mx);
    const float m_tile = mx * c;
    const float m_new = __builtin_elementwise_maximum(m_run, m_tile);
    const bool upd = m_new > m_run + kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(upd)) {
      const float alpha = upd ? fast_exp2(m_run - m_new) : 1.f;
      if constexpr (!kOnesCol) l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) acc[db] *= alpha;
      m_run = upd ? m_new : m_run;
    }
  };

  auto probs = [&](const f32x16_t (&s)[2], uint32_t (&pk)[2][8]) {
    const float msub = (m_run == -INFINITY) ? 0.f : m_run;
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s[kb2][r], c, -msub));
        const float p1 = fast_exp2(__builtin_fmaf(s[kb2][r + 1], c, -msub));
        pk[kb2][r >> 1] = M::pack2(p0, p1);
        if constexpr (!kOnesCol) part[(r >> 1) & 3] = M::sum2(pk[kb2][r >> 1], part[(r >> 1) & 3]);
      }
    if constexpr (!kOnesCol) l_run += (part[0] + part[1]) + (part[2] + part[3]);
  };

  auto pv = [&](auto pc, const uint32_t (&pk)[2][8]) {
    FA_LDS char* vb = vstage(pc) + grp * G::VBYTES;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4_t praw = {pk[u >> 1][4 * (u & 1) + 0], pk[u >> 1][4 * (u & 1) + 1],
                            pk[u >> 1][4 * (u & 1) + 2], pk[u >> 1][4 * (u & 1) + 3]};
      const frag pf = __builtin_bit_cast(frag, praw);
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        FA_LDS char* p0 = vb + v_lane + (16 * u) * VROW + db * 64;
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)p0);
        const i16x4_t up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)(p0 + 8 * VROW));
        const u32x4_t vraw = {__builtin_bit_cast(u32x2_t, lo)[0], __builtin_bit_cast(u32x2_t, lo)[1],
                              __builtin_bit_cast(u32x2_t, up)[0], __builtin_bit_cast(u32x2_t, up)[1]};
        acc[db] = M::mma(__builtin_bit_cast(frag, vraw), pf, acc[db]);
      }
    }
  };

  // Group step j (stage parity of j known at compile time): its tile
  // tile(j) when j < Jg (the group whose tiles ran out idles through the
  // last step); S of its next tile is formed alongside (from a stale stage
  // when there is none, and then never used).  K runs one tile ahead of V:
  // K(j + 2) and V(j + 1) of the group load meanwhile.
  auto step = [&](int j, auto parity, f32x16_t (&cur)[2], f32x16_t (&nxt)[2]) {
    using Cur = decltype(parity);
    using Nxt = std::integral_constant<int, 1 - Cur::value>;
#ifdef FA_LDS_POISON
    // the group's K area of stage Cur (read by S(j) in the previous step)
    // and V area of stage Nxt (read by P V in the previous step) are free;
    // K(j + 2) and V(j + 1) refill them
    {
      const int gt = tid & (G::NT - 1);
      FA_LDS char* const kz = kstage(Cur{}) + grp * G::KBYTES;
      FA_LDS char* const vz = vstage(Nxt{}) + grp * G::VBYTES;
      if (j < Jg) {
        for (int off = gt * 16; off < G::KBYTES; off += G::NT * 16)
          *(FA_LDS u32x4_t*)(kz + off) = (u32x4_t){0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
        for (int off = gt * 16; off < G::VBYTES; off += G::NT * 16)
          *(FA_LDS u32x4_t*)(vz + off) = (u32x4_t){0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
      }
      if constexpr (kOnesCol) {  // the padding columns are never reloaded: restore them
        constexpr int C0 = D / 8, NC = 4 * DBLK - D / 8;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (j < Jg)
          for (int i = gt; i < BN * NC; i += G::NT) {
            const int row = i / NC, chk = C0 + i % NC;
            *(FA_LDS u32x4_t*)(vz + row * VROW + chk * 16) = (u32x4_t){chk == C0 ? M::kOneBits : 0u, 0u, 0u, 0u};
          }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#endif
    if (j < Jg) {
      // a wave without query rows only loads its share of the tiles
      if (wave_live) stats(tile(j), cur);
      if (j + 2 < Jg) issue_k(j + 2, Cur{});
      if (j + 1 < Jg) issue_v(j + 1, Nxt{});
      if (wave_live) {
        uint32_t pk[2][8];
        scores(Nxt{}, nxt);
        probs(cur, pk);
        pv(Cur{}, pk);
      } else {
        nxt[0] = nxt[1] = (f32x16_t){};  // (defined on both paths)
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads have landed
    __syncthreads();                // ... and everyone's; the areas read in step j are free
  };

  f32x16_t sa[2], sb[2];
  if (Jg > 0) {
    issue_k(0, Even{});
    issue_v(0, Even{});
    if (Jg > 1) issue_k(1, Odd{});
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (Jg > 0) scores(Even{}, sa);
  __syncthreads();  // K of step 0 consumed before step 0 loads K of step 2 over it
  for (int j = 0;; j += 2) {
    step(j, Even{}, sa, sb);
    if (j + 1 >= J0) break;
    step(j + 1, Odd{}, sb, sa);
    if (j + 2 >= J0) break;
  }

  // ---- hand-over: group 1 publishes its state per lane, group 0 merges it.
  // Wave pair wg uses object wg, element e of lane l at float (e * 64 + l).
  FA_LDS float* const hb = (FA_LDS float*)object(wg);
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) hb[(16 * db + r) * 64 + lane] = acc[db][r];
    hb[(16 * DBLK) * 64 + lane] = m_run;
    hb[(16 * DBLK + 1) * 64 + lane] = l_run;
  }
  __syncthreads();
  if (grp == 0) {
    const float m1 = hb[(16 * DBLK) * 64 + lane];
    const float l1 = hb[(16 * DBLK + 1) * 64 + lane];
    const float mm = __builtin_elementwise_maximum(m_run, m1);
    // a state that saw no key has m = -inf and weight 0 (group 0 always
    // sees key 0 of its rows, so mm is finite)
    const float a0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - mm);
    const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mm);
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = acc[db][r] * a0 + hb[(16 * db + r) * 64 + lane] * a1;
    l_run = l_run * a0 + l1 * a1;
    m_run = mm;
  }
  __syncthreads();  // every hand-over read is done before the output staging below
  if (grp == 1 || !wave_live) return;

  // ---- epilogue (group 0): O = acc / l, lse = ln2 * (m + log2 l)
  float l_tot;
  if constexpr (kOnesCol) {
    constexpr int ld = D - 32 * (DBLK - 1), r1 = 4 * (ld / 8) + ld % 4, h1 = (ld % 8) / 4;
    l_tot = xlane_sum(hi == h1 ? acc[DBLK - 1][r1] : 0.f);
  } else {
    l_tot = xlane_sum(l_run);
  }
  const float inv = 1.0f / l_tot;
  const int32_t onrec = (wave_rows - 1) * (int32_t)a.o_ss * 2 + a.head_dim * 2;
  const auto ro = make_rsrc(og + (int64_t)qw * a.o_ss, onrec);
  // O through LDS: this wave's 32 rows at stride OROW in object wg, then
  // whole 16-byte pieces of rows
  FA_LDS char* const ob = object(wg);
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (db * 32 + 8 * g >= D) continue;  // the row-sum block (XB) is not output
      const int d0 = db * 32 + 8 * g + 4 * hi;
      const u32x2_t w = {M::pack2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv),
                         M::pack2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
      *(FA_LDS u32x2_t*)(ob + l32 * G::OROW + d0 * 2) = w;
    }
  constexpr int CPR = D / 8;
#pragma unroll
  for (int c0 = 0; c0 < 32 * CPR; c0 += 64) {
    const int cc = c0 + lane;
    const int row = cc / CPR, col = cc - (cc / CPR) * CPR;
    if (32 * CPR % 64 == 0 || cc < 32 * CPR) {
      const u32x4_t w = *(FA_LDS u32x4_t*)(ob + row * G::OROW + col * 16);
      const uint32_t off = (row < wave_rows && col * 8 < a.head_dim)
                               ? (uint32_t)(row * (int32_t)a.o_ss * 2 + col * 16) : kOutOfRange;
      __builtin_amdgcn_raw_buffer_store_b128(w, ro, off, 0, 0);
    }
  }
  if (hi == 0 && a.lse != nullptr && my_q < a.seq_q)
    a.lse[(int64_t)bh * a.seq_q + my_q] = (m_run + __log2f(l_tot)) * kLn2;
}

}  // namespace fa
