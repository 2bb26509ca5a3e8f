// fa_bwd_kernels.hpp -- gfx950 (MI355X) kernels of the attention backward.
//
// Method: the recomputation form of the FlashAttention-2 backward in
// "[CS336] Assignment 2: Systems", section "FlashAttention V2": with the
// forward's logsumexp L and D = rowsum(dO o O),
//     P = exp(S - L),  dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),
//     dQ = scale dS K,  dK = scale dS^T Q,
// split, as that page's "Backward Pass" section does, into a phase that
// fixes a query block and walks the keys (dQ) and a phase that fixes a key
// block and walks the queries (dK, dV), each recomputing P.
//
// MI355X design (not taken from the pages):
//  * three launches: fa_bwd_delta (D, one 8-lane group per row), the dQ
//    kernel and the dK/dV kernel; every launch writes disjoint outputs, so
//    there are no atomics and the result is deterministic;
//  * dQ kernel: the forward's structure.  S^T = K Q^T and dP^T = V dO^T with
//    v_mfma_f32_32x32x16_{bf16,f16} (K, V from LDS as A operands, the wave's
//    Q and dO fragments resident in registers as B operands), so lane l owns
//    query l % 32 and L, D are one register each; dS^T is rounded to the
//    input type and used straight from registers as the B operand of
//    dQ^T += K^T dS^T, whose K^T fragments come from LDS with transposing
//    reads (ds_read_b64_tr_b16);
//  * dK/dV kernel: 8 waves x 32 keys, each wave's K and V fragments
//    resident (V in the wave's own LDS rows at head_dim 128); Q and dO
//    tiles of 32 queries stream through LDS with the tile's lse and delta.
//    S = Q K^T and dP = dO V^T (K, V as B operands), so lane l owns key
//    l % 32 and register r holds query row 8 (r / 4) + 4 (l / 32) + r % 4 --
//    the row order in which transposing reads deliver the k index of an A
//    operand.  P and dS (input type) are therefore the B operands of
//    dV^T += dO^T P and dK^T += Q^T dS straight from registers, with the
//    dO^T / Q^T fragments read transposed from the streamed tiles;
//  * tiles read both row-wise (ds_read_b128) and transposed use a row stride
//    s with s/16 odd and s, 2s, 3s (mod 256) at least 32 bytes from a
//    multiple of 256, so neither access pattern has bank conflicts;
//  * K/V (dQ kernel) and Q/dO (dK/dV kernel) tiles are double-buffered with
//    direct-to-LDS buffer loads; rows past the sequence end and dims past
//    head_dim arrive as zeros, and P is forced to 0 wherever a key is masked
//    (causal, key tail) or a query does not exist.
#pragma once
#include "fa_fwd_kernels.hpp"
#include "fa_mfma_asm.hpp"

namespace fa {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;  // [n_bh, seq_q], natural log
  float* delta;      // [n_bh, seq_q], written by fa_bwd_delta
  void* dq;
  void* dk;
  void* dv;
  int64_t q_sb, q_sh, q_ss;  // element strides: batch, head, seq (dim stride is 1)
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t do_sb, do_sh, do_ss;
  int64_t dq_sb, dq_sh, dq_ss;
  int64_t dk_sb, dk_sh, dk_ss;
  int64_t dv_sb, dv_sh, dv_ss;
  int32_t heads, seq_q, seq_k, head_dim;
  int32_t n_tiles;    // workgroups per (batch, head) of the launch
  int32_t n_bh;       // batch * heads
  float scale;        // sm_scale (signed)
  float c;            // |sm_scale| * log2(e), at least 1e-30
  int32_t neg_scale;  // sm_scale < 0: one score operand is negated in registers
  int32_t causal;
  int32_t xcd_remap;  // n_bh % 8 == 0: keep one (batch, head) on one XCD
};

// Workgroup id -> (batch*head, tile), grouping the tiles of one (batch, head)
// on one XCD; `reverse` hands out the last tiles first.
__device__ inline void map_bwd_workgroup(const BwdArgs& a, int wg, bool reverse, int& bh,
                                         int& tile) {
  int rank;
  if (a.xcd_remap) {
    const int per = a.n_bh >> 3;
    const int xcd = wg & 7, slot = wg >> 3;
    bh = xcd * per + slot % per;
    rank = slot / per;
  } else {
    bh = wg % a.n_bh;
    rank = wg / a.n_bh;
  }
  tile = reverse ? a.n_tiles - 1 - rank : rank;
}

// Rows of the tiles that are read both row-wise (16-byte MFMA operand reads,
// 16 lanes = 16 consecutive rows at one 16-byte chunk per LDS cycle) and
// transposed (ds_read_b64_tr_b16, 32 lanes = 4 consecutive rows x 64 bytes per
// cycle).  The row stride is 64 or 192 mod 256 bytes, which puts the 4 rows of
// a transposing read into the four 64-byte bank windows; inside each 64-byte
// group the four 16-byte chunks of row r are stored XOR-permuted by
// (r / 4) % 4, so the 16 rows of a row-wise read, which share each window four
// at a time, use its four different 16-byte slots.  Slot p of row r holds
// chunk swz_chunk(p, r) of the row (and chunk p sits in that same slot).
__device__ constexpr int swz_chunk(int p, int row) { return (p & ~3) | ((p & 3) ^ ((row >> 2) & 3)); }

// ---------------------------------------------------------------------------
// D_i = sum_t dO_it O_it  (fp32), 8 lanes per row.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void fa_bwd_delta(BwdArgs a) {
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * 32 + (tid >> 3);
  const int sub = tid & 7;
  const int64_t rows = (int64_t)a.n_bh * a.seq_q;
  float part = 0.f;
  if (row < rows) {
    const int bh = (int)(row / a.seq_q), i = (int)(row - (int64_t)bh * a.seq_q);
    const int b = bh / a.heads, h = bh - b * a.heads;
    const T* orow = (const T*)a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)i * a.o_ss;
    const T* drow =
        (const T*)a.dout + (int64_t)b * a.do_sb + (int64_t)h * a.do_sh + (int64_t)i * a.do_ss;
    if constexpr (sizeof(T) == 4) {
      // fp32 rows are only 4-byte aligned: element loads, lane sub takes dims sub + 8 i
      for (int d = sub; d < a.head_dim; d += 8)
        part = __builtin_fmaf((float)drow[d], (float)orow[d], part);
    } else {
      // 8-element chunks: lane sub takes chunks sub, sub + 8, ... (dims 8 sub + 64 i ..)
      for (int d0 = 8 * sub; d0 < a.head_dim; d0 += 64) {
        typedef T t8 __attribute__((ext_vector_type(8)));
        const t8 ov = *(const t8*)(orow + d0);
        const t8 dv = *(const t8*)(drow + d0);
#pragma unroll
        for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)dv[e], (float)ov[e], part);
      }
    }
  }
  // sum over the 8 lanes of the row
  part += __shfl_xor(part, 1, 8);
  part += __shfl_xor(part, 2, 8);
  part += __shfl_xor(part, 4, 8);
  if (row < rows && sub == 0) a.delta[row] = part;
}

// Per-lane byte offsets for direct-to-LDS loads of a tile of `rows` rows of
// `slots` 16-byte LDS slots each (slot s of the tile is filled by lane s % 64
// of instruction s / 64); slots past the tile or past head_dim read nothing.
__device__ inline uint32_t tile_slot_offset(int slot, int rows, int slots, int64_t seq_stride,
                                            int head_dim) {
  const int row = slot / slots, ch = slot - (slot / slots) * slots;
  return (row < rows && ch * 8 < head_dim) ? (uint32_t)(row * (int32_t)seq_stride * 2 + ch * 16)
                                           : kOutOfRange;
}

// The same for the swizzled dual-read tiles: slot p < data_slots of a row
// receives chunk swz_chunk(p, row); the padding slots read nothing.
__device__ inline uint32_t swz_slot_offset(int slot, int rows, int slots, int data_slots,
                                           int64_t seq_stride, int head_dim) {
  const int row = slot / slots, p = slot - (slot / slots) * slots;
  const int ch = swz_chunk(p, row);
  return (row < rows && p < data_slots && ch * 8 < head_dim)
             ? (uint32_t)(row * (int32_t)seq_stride * 2 + ch * 16)
             : kOutOfRange;
}

// ---------------------------------------------------------------------------
// dQ kernel: one workgroup per (batch*head, block of 32*NW queries).
// ---------------------------------------------------------------------------
template <typename T, int D, int NW>
struct BwdQTile {
  static constexpr int BM = 32 * NW;             // query rows per workgroup
  static constexpr int BN = 64;                  // keys per K/V tile
  static constexpr int KSTEPS = D / 16;
  static constexpr int DBLK = (D + 31) / 32;
  static constexpr int KR = tr_row_stride(DBLK * 64);  // K rows: b128 + transposed, swizzled
  static constexpr int VR = D * 2 + 16;          // V rows: b128 only (16 mod 256)
  static constexpr int KSLOTS = KR / 16, VSLOTS = VR / 16;
  static constexpr int KINSTR = BN * KSLOTS / 64, VINSTR = BN * VSLOTS / 64;
  static constexpr int KPER = (KINSTR + NW - 1) / NW, VPER = (VINSTR + NW - 1) / NW;
  static constexpr int KBYTES = BN * KR, VBYTES = BN * VR;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int LDS_BYTES = 2 * STAGE;  // two LDS objects of STAGE bytes
  static_assert(D % 16 == 0 && D <= 256, "head_dim padding");
  static_assert(KR >= DBLK * 64, "transposed reads of the K tile stay inside a row");
};

template <typename T, int D, int NW>
__device__ __forceinline__ void fa_bwd_dq_body(const BwdArgs& a) {
  using G = BwdQTile<T, D, NW>;
  using M = Mfma<T>;
  using X = MfmaPin<T>;
  typedef typename M::frag frag;
  constexpr int BN = G::BN, KSTEPS = G::KSTEPS, DBLK = G::DBLK, KR = G::KR, VR = G::VR;
  // Above head_dim 128 the MFMAs are inline assembly that keeps the Q
  // fragments and the dQ^T accumulator in AGPRs (4 DBLK + KSTEPS * 4
  // registers, 192 at D = 256), where the register allocator would move them
  // between AGPRs and VGPRs inside the key loop.
  constexpr bool kPinAcc = D > 128;
  // S before dP (measured: +2-4% at head_dim 64 and 80, -2% at 128)
  constexpr bool kSFirst = D == 64 || D == 80;

  // the two tile stages as separate LDS objects, so that the compiler can
  // tell reads of one stage from the asynchronous loads into the other
  __shared__ __attribute__((aligned(1024))) char stage0[G::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[G::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  int bh, qt;
  map_bwd_workgroup(a, blockIdx.x, a.causal != 0, bh, qt);
  const int b = bh / a.heads, h = bh - b * a.heads;
  const T* qg = (const T*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
  const T* dog = (const T*)a.dout + (int64_t)b * a.do_sb + (int64_t)h * a.do_sh;
  const T* kg = (const T*)a.k + (int64_t)b * a.k_sb + (int64_t)h * a.k_sh;
  const T* vg = (const T*)a.v + (int64_t)b * a.v_sb + (int64_t)h * a.v_sh;
  T* dqg = (T*)a.dq + (int64_t)b * a.dq_sb + (int64_t)h * a.dq_sh;

  const int q0 = qt * G::BM;
  const int qw = q0 + wave * 32;
  const int my_q = qw + l32;
  const int wave_rows = max(0, min(32, a.seq_q - qw));
  // last key this lane's query sees (the key tail, and causal: its own row)
  const int key_lim = a.causal ? min(a.seq_k - 1, my_q) : a.seq_k - 1;
  const int kv_end = a.causal ? min(a.seq_k, min(a.seq_q, q0 + G::BM)) : a.seq_k;
  const int n_tiles = (kv_end + BN - 1) / BN;

  // resident fragments (B operands): lane = (query l32, dims 8*hi..+7 of each k-step)
  frag qf[KSTEPS], dof[KSTEPS];
  {
    const int32_t nq = wave_rows > 0 ? (wave_rows - 1) * (int32_t)a.q_ss * 2 + a.head_dim * 2 : 0;
    const int32_t nd = wave_rows > 0 ? (wave_rows - 1) * (int32_t)a.do_ss * 2 + a.head_dim * 2 : 0;
    const auto rq = make_rsrc(qg + (int64_t)(wave_rows > 0 ? qw : 0) * a.q_ss, nq);
    const auto rd = make_rsrc(dog + (int64_t)(wave_rows > 0 ? qw : 0) * a.do_ss, nd);
    const uint32_t sign = a.neg_scale ? 0x80008000u : 0u;
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
      const int col = st * 16 + hi * 8;
      const bool in = col < a.head_dim;
      u32x4_t rawq = __builtin_amdgcn_raw_buffer_load_b128(
          rq, in ? (uint32_t)(l32 * (int32_t)a.q_ss * 2 + col * 2) : kOutOfRange, 0, 0);
      const u32x4_t rawd = __builtin_amdgcn_raw_buffer_load_b128(
          rd, in ? (uint32_t)(l32 * (int32_t)a.do_ss * 2 + col * 2) : kOutOfRange, 0, 0);
      rawq ^= (u32x4_t){sign, sign, sign, sign};
      qf[st] = __builtin_bit_cast(frag, rawq);
      dof[st] = __builtin_bit_cast(frag, rawd);
    }
  }
  if constexpr (kPinAcc) pin_agpr<KSTEPS>(qf);
  const bool q_ok = my_q < a.seq_q;
  const float L2 = q_ok ? a.lse[(int64_t)bh * a.seq_q + my_q] * kLog2e : 0.f;
  const float Dl = q_ok ? a.delta[(int64_t)bh * a.seq_q + my_q] : 0.f;
  const float c = a.c;

  // direct-to-LDS tile loads, all NW waves
  uint32_t koff[G::KPER], voff[G::VPER];
#pragma unroll
  for (int n = 0; n < G::KPER; ++n)
    koff[n] = swz_slot_offset((wave + NW * n) * 64 + lane, BN, G::KSLOTS, 4 * DBLK, a.k_ss,
                              a.head_dim);
#pragma unroll
  for (int n = 0; n < G::VPER; ++n)
    voff[n] = tile_slot_offset((wave + NW * n) * 64 + lane, BN, G::VSLOTS, a.v_ss, a.head_dim);
  auto issue = [&](int j, FA_LDS char* kb) {
    const int key0 = j * BN;
    const int rows = min(BN, a.seq_k - key0);
    const auto rk = make_rsrc(kg + (int64_t)key0 * a.k_ss, (rows - 1) * (int32_t)a.k_ss * 2 + a.head_dim * 2);
    const auto rv = make_rsrc(vg + (int64_t)key0 * a.v_ss, (rows - 1) * (int32_t)a.v_ss * 2 + a.head_dim * 2);
    FA_LDS char* vb = kb + G::KBYTES;
#pragma unroll
    for (int n = 0; n < G::KPER; ++n)
      if (wave + NW * n < G::KINSTR)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (FA_LDS void*)(kb + (wave + NW * n) * 1024), 16,
                                                 koff[n], 0, 0, 0);
#pragma unroll
    for (int n = 0; n < G::VPER; ++n)
      if (wave + NW * n < G::VINSTR)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (FA_LDS void*)(vb + (wave + NW * n) * 1024), 16,
                                                 voff[n], 0, 0, 0);
  };

  f32x16_t acc[DBLK];  // dQ^T: rows = dims of block db, column = query l32
#pragma unroll
  for (int db = 0; db < DBLK; ++db) acc[db] = (f32x16_t){};

  // b128 row reads of K (row l32 of a 32-row block, chunk 2 st + hi; even
  // and odd k-steps differ in bit 1 of the swizzled chunk) and of V
  const int sw = (l32 >> 2) & 3;
  const int k_even = l32 * KR + 16 * (hi ^ sw), k_odd = l32 * KR + 16 * (hi ^ sw ^ 2);
  const int v_lane = l32 * VR + hi * 16;
  // transposing reads of K: rows 16 u + 4 hi + s16 / 4 (swizzle hi) and 8
  // rows further (swizzle hi ^ 2), chunk 4 db + 2 ((lane / 16) % 2) + (s16 % 4) / 2
  const int s16 = lane & 15;
  const int t_row = 4 * hi + (s16 >> 2);
  const int t_ch = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1), t_half = 8 * (s16 & 1);
  const int t_lo = t_row * KR + 16 * (t_ch ^ hi) + t_half;
  const int t_up = (t_row + 8) * KR + 16 * (t_ch ^ hi ^ 2) + t_half;

  // one key tile; its K / V are in stage kb, the next tile loads into nb
  auto step = [&](int t, FA_LDS char* kb, FA_LDS char* nb) {
#ifdef FA_LDS_POISON
    lds_poison<64 * NW>(nb, G::STAGE);  // tile t - 1 (read in the previous step) is free
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#endif
    if (t + 1 < n_tiles) issue(t + 1, nb);
    FA_LDS char* vb = kb + G::KBYTES;

    // S^T = K Q^T and dP^T = V dO^T for the two 32-key blocks of the tile
    f32x16_t s[2], dp[2];
    if constexpr (kPinAcc) {
      // fragments read PD k-steps ahead of their MFMAs, scheduling barriers
      // between the k-steps (bounded registers in flight)
      constexpr int PD = 2;
      frag kfr[KSTEPS][2], vfr[KSTEPS][2];
      auto rd = [&](auto ic) {
        constexpr int st = decltype(ic)::value;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          kfr[st][kb2] = __builtin_bit_cast(
              frag, *(FA_LDS u32x4_t*)(kb + ((st & 1) ? k_odd : k_even) + kb2 * 32 * KR + 64 * (st >> 1)));
          vfr[st][kb2] = __builtin_bit_cast(frag, *(FA_LDS u32x4_t*)(vb + v_lane + kb2 * 32 * VR + st * 32));
        }
      };
      static_for<0, PD>(rd);
      static_for<0, KSTEPS>([&](auto ic) {
        constexpr int st = decltype(ic)::value;
        if constexpr (st + PD < KSTEPS) rd(std::integral_constant<int, st + PD>{});
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          if constexpr (st == 0) {
            X::first(s[kb2], kfr[st][kb2], qf[st]);
            X::vfirst(dp[kb2], vfr[st][kb2], dof[st]);
          } else {
            X::next(s[kb2], kfr[st][kb2], qf[st]);
            X::vnext(dp[kb2], vfr[st][kb2], dof[st]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      mfma_drain_v(s[0], s[1]);  // before the VALU reads of S and dP
      mfma_drain_v(dp[0], dp[1]);
    } else {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        s[kb2] = (f32x16_t){};
        dp[kb2] = (f32x16_t){};
      }
      auto kfrag = [&](int st, int kb2) {
        return __builtin_bit_cast(
            frag, *(FA_LDS u32x4_t*)(kb + ((st & 1) ? k_odd : k_even) + kb2 * 32 * KR + 64 * (st >> 1)));
      };
      auto vfrag = [&](int st, int kb2) {
        return __builtin_bit_cast(frag, *(FA_LDS u32x4_t*)(vb + v_lane + kb2 * 32 * VR + st * 32));
      };
      if constexpr (kSFirst) {
        // all of S first, a scheduling barrier, then dP: the exponentials of
        // S can run beside the dP MFMAs
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2) s[kb2] = M::mma(kfrag(st, kb2), qf[st], s[kb2]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2) dp[kb2] = M::mma(vfrag(st, kb2), dof[st], dp[kb2]);
      } else {
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2) {
            s[kb2] = M::mma(kfrag(st, kb2), qf[st], s[kb2]);
            dp[kb2] = M::mma(vfrag(st, kb2), dof[st], dp[kb2]);
          }
      }
    }

    // P = exp2(s c - L2) (0 where masked), dS = P (dP - D), rounded pairwise
    const int key0 = t * BN;
    const bool need_mask = (key0 + BN > a.seq_k) || (a.causal && key0 + BN - 1 > qw);
    uint32_t pk[2][8];
    // key key0 + cr + 4 hi (cr = kb2 32 + 8 (r / 4) + r % 4, a constant) is
    // visible to this lane's query iff cr <= dl
    const int dl = key_lim - key0 - 4 * hi;
    // the masks in one branch after all the exponentials, so that the
    // exponentials form one block of straight-line code with the MFMAs
    // (head_dim 128: dS too before the branch, which measured faster there;
    // the other widths keep the products after it)
    constexpr bool kEarlyDs = D == 128;
    float pe[2][16];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pe[kb2][r] = fast_exp2(__builtin_fmaf(s[kb2][r], c, -L2));
        if constexpr (kEarlyDs) pe[kb2][r] *= dp[kb2][r] - Dl;
      }
    if (need_mask) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cr = kb2 * 32 + 8 * (r >> 2) + (r & 3);
          pe[kb2][r] = cr <= dl ? pe[kb2][r] : 0.f;
        }
    }
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        if constexpr (kEarlyDs)
          pk[kb2][r >> 1] = M::pack2(pe[kb2][r], pe[kb2][r + 1]);
        else
          pk[kb2][r >> 1] = M::pack2(pe[kb2][r] * (dp[kb2][r] - Dl), pe[kb2][r + 1] * (dp[kb2][r + 1] - Dl));
      }

    // dQ^T += K^T dS^T: four 16-key steps per 32-dim block
    auto ktr = [&](int u, int db) {
      FA_LDS char* p0 = kb + (16 * u) * KR + db * 64;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)(p0 + t_lo));
      const i16x4_t up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)(p0 + t_up));
      const u32x4_t kraw = {__builtin_bit_cast(u32x2_t, lo)[0], __builtin_bit_cast(u32x2_t, lo)[1],
                            __builtin_bit_cast(u32x2_t, up)[0], __builtin_bit_cast(u32x2_t, up)[1]};
      return __builtin_bit_cast(frag, kraw);
    };
    auto s_frag = [&](int u) {
      const u32x4_t sraw = {pk[u >> 1][4 * (u & 1) + 0], pk[u >> 1][4 * (u & 1) + 1],
                            pk[u >> 1][4 * (u & 1) + 2], pk[u >> 1][4 * (u & 1) + 3]};
      return __builtin_bit_cast(frag, sraw);
    };
    if constexpr (kPinAcc) {
      // the transposing reads PD blocks ahead of their MFMAs
      constexpr int PD = 2, NB = 4 * DBLK;
      frag kt[NB];
      static_for<0, PD>([&](auto ic) { kt[decltype(ic)::value] = ktr(decltype(ic)::value / DBLK, decltype(ic)::value % DBLK); });
      static_for<0, NB>([&](auto ic) {
        constexpr int j = decltype(ic)::value, u = j / DBLK, db = j % DBLK;
        if constexpr (j + PD < NB) kt[j + PD] = ktr((j + PD) / DBLK, (j + PD) % DBLK);
        X::acc_fresh(acc[db], kt[j], s_frag(u));
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const frag sf = s_frag(u);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) acc[db] = M::mma(ktr(u, db), sf, acc[db]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of tile t+1 have landed
    __syncthreads();                // ... and everyone's; stage t is free
  };

  if (n_tiles > 0) {
    issue(0, (FA_LDS char*)stage0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int t = 0;
    for (; t + 1 < n_tiles; t += 2) {
      step(t, (FA_LDS char*)stage0, (FA_LDS char*)stage1);
      step(t + 1, (FA_LDS char*)stage1, (FA_LDS char*)stage0);
    }
    if (t < n_tiles) step(t, (FA_LDS char*)stage0, (FA_LDS char*)stage1);
  }

  // dQ = scale * (K^T dS^T)^T, rounded to the input type
  if constexpr (kPinAcc) mfma_drain_a<DBLK>(acc);  // the last MFMAs before the VALU reads
  if (wave_rows == 0) return;
  const int32_t onrec = (wave_rows - 1) * (int32_t)a.dq_ss * 2 + a.head_dim * 2;
  const auto ro = make_rsrc(dqg + (int64_t)qw * a.dq_ss, onrec);
  const uint32_t orow = (uint32_t)(l32 * (int32_t)a.dq_ss * 2);
  const float sc = a.scale;
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = db * 32 + 8 * g + 4 * hi;
      const uint32_t off = (d0 < a.head_dim && l32 < wave_rows) ? orow + d0 * 2 : kOutOfRange;
      const u32x2_t w = {M::pack2(acc[db][4 * g + 0] * sc, acc[db][4 * g + 1] * sc),
                         M::pack2(acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc)};
      __builtin_amdgcn_raw_buffer_store_b64(w, ro, off, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// dK/dV kernel: one workgroup per (batch*head, block of 32*NW keys).
// ---------------------------------------------------------------------------
template <typename T, int D, int NW>
struct BwdKVTile {
  static constexpr int BK = 32 * NW;             // keys per workgroup
  static constexpr int BQ = 32;                  // queries per streamed tile
  static constexpr int KSTEPS = D / 16;
  static constexpr int DBLK = (D + 31) / 32;
  static constexpr int QR = tr_row_stride(DBLK * 64);  // Q / dO rows: b128 + transposed, swizzled
  static constexpr int QSLOTS = QR / 16;
  static constexpr int QINSTR = (BQ * QSLOTS + 63) / 64;  // wave-wide loads per tile
  static constexpr int QPER = (QINSTR + NW - 1) / NW;
  static constexpr int TBYTES = QINSTR * 1024;   // one tile, rounded to whole loads
  static constexpr int LD_OFF = 2 * TBYTES;      // then the tile's lse*log2e and delta (fp32)
  static constexpr int STAGE = 2 * TBYTES + 2 * BQ * 4;
  // at d = 128 each wave keeps its 32 V rows in LDS rather than in KSTEPS
  // registers (16 mod 256 byte rows: conflict-free 16-byte row reads)
  static constexpr bool V_IN_LDS = (D >= 128);
  static constexpr int VR = D * 2 + 16;
  static constexpr int VWBYTES = V_IN_LDS ? 32 * VR : 0;
  static constexpr int LDS_BYTES = 2 * STAGE + NW * VWBYTES;  // over three objects
  static_assert(D % 16 == 0 && D <= 256, "head_dim padding");
  static_assert(QR >= DBLK * 64, "transposed reads stay inside a row");
};

typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T, int D, int NW>
__device__ __forceinline__ void fa_bwd_dkv_body(const BwdArgs& a) {
  using G = BwdKVTile<T, D, NW>;
  using M = Mfma<T>;
  using X = MfmaPin<T>;
  typedef typename M::frag frag;
  constexpr int BQ = G::BQ, KSTEPS = G::KSTEPS, DBLK = G::DBLK, QR = G::QR;
  // Above head_dim 128 the two accumulators take 2 x 4 DBLK registers (256
  // at D = 256): their MFMAs are then written as inline assembly that keeps
  // them in AGPRs, where the register allocator would shuttle them between
  // AGPRs and VGPRs and spill.
  constexpr bool kPinAcc = D > 128;
  // S before dP (measured: +2-4% at head_dim 64 and 80, -2% at 128)
  constexpr bool kSFirst = D == 64 || D == 80;

  // three LDS objects -- the two tile stages and the V rows -- so that the
  // compiler knows which accesses the asynchronous tile loads into one stage
  // can touch, and does not make reads of the other stage wait for them
  __shared__ __attribute__((aligned(1024))) char stage0[G::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[G::STAGE];
  __shared__ __attribute__((aligned(1024))) char v_mem[G::V_IN_LDS ? NW * G::VWBYTES : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  int bh, kt;
  map_bwd_workgroup(a, blockIdx.x, false, bh, kt);
  const int b = bh / a.heads, h = bh - b * a.heads;
  const T* qg = (const T*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
  const T* dog = (const T*)a.dout + (int64_t)b * a.do_sb + (int64_t)h * a.do_sh;
  const T* kg = (const T*)a.k + (int64_t)b * a.k_sb + (int64_t)h * a.k_sh;
  const T* vg = (const T*)a.v + (int64_t)b * a.v_sb + (int64_t)h * a.v_sh;
  T* dkg = (T*)a.dk + (int64_t)b * a.dk_sb + (int64_t)h * a.dk_sh;
  T* dvg = (T*)a.dv + (int64_t)b * a.dv_sb + (int64_t)h * a.dv_sh;
  const float* lseg = a.lse + (int64_t)bh * a.seq_q;
  const float* delg = a.delta + (int64_t)bh * a.seq_q;

  const int k0 = kt * G::BK;
  const int kw = k0 + wave * 32;        // first key of this wave
  const int wave_keys = max(0, min(32, a.seq_k - kw));
  // query tiles that see any key of the workgroup (causal: queries >= k0)
  const int qt0 = a.causal ? min(k0, a.seq_q) / BQ : 0;
  const int qt_end = (a.seq_q + BQ - 1) / BQ;

  // resident B operands: lane = (key l32, dims 8*hi..+7 of each k-step); K negated for scale < 0
  FA_LDS char* v_lds = (FA_LDS char*)v_mem + wave * G::VWBYTES;
  const int v_lane = l32 * G::VR + hi * 16;
  frag kf[KSTEPS], vf[G::V_IN_LDS ? 1 : KSTEPS];
  {
    const int32_t nk = wave_keys > 0 ? (wave_keys - 1) * (int32_t)a.k_ss * 2 + a.head_dim * 2 : 0;
    const int32_t nv = wave_keys > 0 ? (wave_keys - 1) * (int32_t)a.v_ss * 2 + a.head_dim * 2 : 0;
    const auto rk = make_rsrc(kg + (int64_t)(wave_keys > 0 ? kw : 0) * a.k_ss, nk);
    const auto rv = make_rsrc(vg + (int64_t)(wave_keys > 0 ? kw : 0) * a.v_ss, nv);
    const uint32_t sign = a.neg_scale ? 0x80008000u : 0u;
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
      const int col = st * 16 + hi * 8;
      const bool in = col < a.head_dim;
      u32x4_t rawk = __builtin_amdgcn_raw_buffer_load_b128(
          rk, in ? (uint32_t)(l32 * (int32_t)a.k_ss * 2 + col * 2) : kOutOfRange, 0, 0);
      const u32x4_t rawv = __builtin_amdgcn_raw_buffer_load_b128(
          rv, in ? (uint32_t)(l32 * (int32_t)a.v_ss * 2 + col * 2) : kOutOfRange, 0, 0);
      rawk ^= (u32x4_t){sign, sign, sign, sign};
      kf[st] = __builtin_bit_cast(frag, rawk);
      if constexpr (G::V_IN_LDS)
        *(FA_LDS u32x4_t*)(v_lds + v_lane + st * 32) = rawv;
      else
        vf[st] = __builtin_bit_cast(frag, rawv);
    }
  }
  const float c = a.c;

  // direct-to-LDS loads of the Q and dO tiles, all NW waves
  uint32_t qoff[G::QPER], doff[G::QPER];
#pragma unroll
  for (int n = 0; n < G::QPER; ++n) {
    const int slot = (wave + NW * n) * 64 + lane;
    qoff[n] = swz_slot_offset(slot, BQ, G::QSLOTS, 4 * DBLK, a.q_ss, a.head_dim);
    doff[n] = swz_slot_offset(slot, BQ, G::QSLOTS, 4 * DBLK, a.do_ss, a.head_dim);
  }
  auto issue = [&](int j, FA_LDS char* qb) {
    const int qa = j * BQ;
    const int rows = min(BQ, a.seq_q - qa);
    const auto rq = make_rsrc(qg + (int64_t)qa * a.q_ss, (rows - 1) * (int32_t)a.q_ss * 2 + a.head_dim * 2);
    const auto rd = make_rsrc(dog + (int64_t)qa * a.do_ss, (rows - 1) * (int32_t)a.do_ss * 2 + a.head_dim * 2);
    FA_LDS char* db_ = qb + G::TBYTES;
#pragma unroll
    for (int n = 0; n < G::QPER; ++n)
      if (wave + NW * n < G::QINSTR) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (FA_LDS void*)(qb + (wave + NW * n) * 1024), 16,
                                                 qoff[n], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (FA_LDS void*)(db_ + (wave + NW * n) * 1024), 16,
                                                 doff[n], 0, 0, 0);
      }
  };

  // dV^T and dK^T: rows = dims of block db, column = key l32
  f32x16_t dvacc[DBLK], dkacc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
    dvacc[db] = (f32x16_t){};
    dkacc[db] = (f32x16_t){};
  }

  // b128 row reads of Q / dO (row l32, chunk 2 st + hi, swizzled) and
  // transposing reads (rows 16 u + 4 hi + s16 / 4 and 8 rows further)
  const int sw = (l32 >> 2) & 3;
  const int q_even = l32 * QR + 16 * (hi ^ sw), q_odd = l32 * QR + 16 * (hi ^ sw ^ 2);
  const int s16 = lane & 15;
  const int t_row = 4 * hi + (s16 >> 2);
  const int t_ch = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1), t_half = 8 * (s16 & 1);
  const int t_lo = t_row * QR + 16 * (t_ch ^ hi) + t_half;
  const int t_up = (t_row + 8) * QR + 16 * (t_ch ^ hi ^ 2) + t_half;

  // lse and delta of query tile j: wave 0 loads them (lane = row, index
  // clamped) while the tile before it is processed, and stores lse * log2e
  // and delta next to the tile's Q and dO.  The loads go out before the
  // tile's Q / dO loads and nothing uses them until the store at the end of
  // the step: loads complete in order, so a use right after them would wait
  // for the whole next tile as well.
  float ld_l = 0.f, ld_d = 0.f;
  auto stats_load = [&](int j) {
    if (wave == 0) {
      const int qi = min(j * BQ + l32, a.seq_q - 1);
      ld_l = lseg[qi];
      ld_d = delg[qi];
    }
  };
  auto stats_store = [&](FA_LDS char* qb) {
    if (wave == 0 && hi == 0) {
      *(FA_LDS float*)(qb + G::LD_OFF + l32 * 4) = ld_l * kLog2e;
      *(FA_LDS float*)(qb + G::LD_OFF + BQ * 4 + l32 * 4) = ld_d;
    }
  };

  // one query tile; its Q / dO tile is in stage qb, the next tile loads
  // into the other stage nb meanwhile
  auto step = [&](int t, FA_LDS char* qb, FA_LDS char* nb) {
#ifdef FA_LDS_POISON
    lds_poison<64 * NW>(nb, G::STAGE);  // tile t - 1 (read in the previous step) is free
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#endif
    if (t + 1 < qt_end) {
      stats_load(t + 1);
      issue(t + 1, nb);
    }
    FA_LDS char* dob = qb + G::TBYTES;

    // S = Q K^T, dP = dO V^T: rows = the tile's 32 queries, column = key l32;
    // register r of lane half hi holds query row 8 (r / 4) + 4 hi + r % 4,
    // the row order of the transposing reads below, so P and dS serve as the
    // B operands of the dV and dK products straight from registers
    f32x16_t s = (f32x16_t){}, dp = (f32x16_t){};
    if constexpr (kPinAcc) {
      // fragments read PD k-steps ahead of their MFMAs, scheduling barriers
      // between the k-steps: the reads of all k-steps hoisted to the top
      // would hold 12 registers per k-step
      constexpr int PD = 2;
      frag qfr[KSTEPS], dfr[KSTEPS], vfr[KSTEPS];
      auto rd = [&](auto ic) {
        constexpr int st = decltype(ic)::value;
        const int qo = ((st & 1) ? q_odd : q_even) + 64 * (st >> 1);
        qfr[st] = __builtin_bit_cast(frag, *(FA_LDS u32x4_t*)(qb + qo));
        dfr[st] = __builtin_bit_cast(frag, *(FA_LDS u32x4_t*)(dob + qo));
        vfr[st] = __builtin_bit_cast(frag, *(FA_LDS u32x4_t*)(v_lds + v_lane + st * 32));
      };
      static_for<0, PD>(rd);
      static_for<0, KSTEPS>([&](auto ic) {
        constexpr int st = decltype(ic)::value;
        if constexpr (st + PD < KSTEPS) rd(std::integral_constant<int, st + PD>{});
        // (as inline assembly too: with AGPR operands in the kernel the
        // compiler would give these results AGPRs and copy them out)
        if constexpr (st == 0) {
          X::vfirst(s, qfr[st], kf[st]);
          X::vfirst(dp, dfr[st], vfr[st]);
        } else {
          X::vnext(s, qfr[st], kf[st]);
          X::vnext(dp, dfr[st], vfr[st]);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      mfma_drain_v(s, dp);  // before the VALU reads of S and dP
    } else {
      auto s_k = [&](int st) {
        const int qo = ((st & 1) ? q_odd : q_even) + 64 * (st >> 1);
        s = M::mma(__builtin_bit_cast(frag, *(FA_LDS u32x4_t*)(qb + qo)), kf[st], s);
      };
      auto dp_k = [&](int st) {
        const int qo = ((st & 1) ? q_odd : q_even) + 64 * (st >> 1);
        const frag dfr = __builtin_bit_cast(frag, *(FA_LDS u32x4_t*)(dob + qo));
        if constexpr (G::V_IN_LDS) {
          const frag vfr = __builtin_bit_cast(frag, *(FA_LDS u32x4_t*)(v_lds + v_lane + st * 32));
          dp = M::mma(dfr, vfr, dp);
        } else {
          dp = M::mma(dfr, vf[st], dp);
        }
      };
      if constexpr (kSFirst) {
        // all of S first, a scheduling barrier, then dP: the exponentials of
        // S can run beside the dP MFMAs
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) s_k(st);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) dp_k(st);
      } else {
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) {
          s_k(st);
          dp_k(st);
        }
      }
    }

    const int qa = t * BQ;
    const int my_k = kw + l32;
    const bool need_mask = (qa + BQ > a.seq_q) || (kw + 32 > a.seq_k) || (a.causal && kw + 31 > qa);
    // query qa + 4 hi + cq (cq = 8 j + i, a constant) sees this lane's key
    // iff dlo <= cq <= dhi (a key past seq_k: dhi < 0, seen by nobody)
    const int dlo = (a.causal ? my_k : 0) - qa - 4 * hi;
    const int dhi = (my_k < a.seq_k ? a.seq_q - 1 : -1 - 64) - qa - 4 * hi;
    // P = exp2(s c - L2) and dS = P (dP - D) in the input type, paired along queries
    // (the masks in one branch after all the exponentials, so that the
    // exponentials form one block of straight-line code with the MFMAs)
    // (head_dim 128: dS too before the branch, which measured faster there;
    // the other widths keep the products after it)
    constexpr bool kEarlyDs = D == 128;
    uint32_t pp[8], ps[8];
    float pe[16], ds[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4_t L4 = *(FA_LDS f32x4_t*)(qb + G::LD_OFF + (8 * j + 4 * hi) * 4);
      const f32x4_t D4 = *(FA_LDS f32x4_t*)(qb + G::LD_OFF + BQ * 4 + (8 * j + 4 * hi) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pe[4 * j + i] = fast_exp2(__builtin_fmaf(s[4 * j + i], c, -L4[i]));
        if constexpr (kEarlyDs) ds[4 * j + i] = pe[4 * j + i] * (dp[4 * j + i] - D4[i]);
      }
    }
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int cq = 8 * (r >> 2) + (r & 3);
        const bool vis = cq >= dlo && cq <= dhi;
        pe[r] = vis ? pe[r] : 0.f;
        if constexpr (kEarlyDs) ds[r] = vis ? ds[r] : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4_t D4 = *(FA_LDS f32x4_t*)(qb + G::LD_OFF + BQ * 4 + (8 * j + 4 * hi) * 4);
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const int r = 4 * j + i;
        if constexpr (!kEarlyDs) {
          ds[r] = pe[r] * (dp[r] - D4[i]);
          ds[r + 1] = pe[r + 1] * (dp[r + 1] - D4[i + 1]);
        }
        pp[r >> 1] = M::pack2(pe[r], pe[r + 1]);
        ps[r >> 1] = M::pack2(ds[r], ds[r + 1]);
      }
    }

    // dV^T += dO^T P and dK^T += Q^T dS: two 16-query steps per 32-dim block
    if constexpr (kPinAcc) {
      // the same with the transposing reads PD blocks ahead of their MFMAs
      constexpr int PD = 2, NB = 2 * DBLK;
      frag dtr[NB], qtr[NB];
      auto rd = [&](auto ic) {
        constexpr int j = decltype(ic)::value, u = j / DBLK, db = j % DBLK;
        FA_LDS char* d0 = dob + (16 * u) * QR + db * 64;
        FA_LDS char* q0p = qb + (16 * u) * QR + db * 64;
        const i16x4_t dlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)(d0 + t_lo));
        const i16x4_t dup = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)(d0 + t_up));
        const i16x4_t qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)(q0p + t_lo));
        const i16x4_t qup = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)(q0p + t_up));
        dtr[j] = __builtin_bit_cast(frag, (u32x4_t){__builtin_bit_cast(u32x2_t, dlo)[0], __builtin_bit_cast(u32x2_t, dlo)[1],
                                                    __builtin_bit_cast(u32x2_t, dup)[0], __builtin_bit_cast(u32x2_t, dup)[1]});
        qtr[j] = __builtin_bit_cast(frag, (u32x4_t){__builtin_bit_cast(u32x2_t, qlo)[0], __builtin_bit_cast(u32x2_t, qlo)[1],
                                                    __builtin_bit_cast(u32x2_t, qup)[0], __builtin_bit_cast(u32x2_t, qup)[1]});
      };
      static_for<0, PD>(rd);
      static_for<0, NB>([&](auto ic) {
        constexpr int j = decltype(ic)::value, u = j / DBLK, db = j % DBLK;
        if constexpr (j + PD < NB) rd(std::integral_constant<int, j + PD>{});
        const frag pfr = __builtin_bit_cast(frag, (u32x4_t){pp[4 * u], pp[4 * u + 1], pp[4 * u + 2], pp[4 * u + 3]});
        const frag sfr = __builtin_bit_cast(frag, (u32x4_t){ps[4 * u], ps[4 * u + 1], ps[4 * u + 2], ps[4 * u + 3]});
        X::acc_fresh(dvacc[db], dtr[j], pfr);
        X::acc_fresh(dkacc[db], qtr[j], sfr);
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const frag pfr = __builtin_bit_cast(frag, (u32x4_t){pp[4 * u], pp[4 * u + 1], pp[4 * u + 2], pp[4 * u + 3]});
      const frag sfr = __builtin_bit_cast(frag, (u32x4_t){ps[4 * u], ps[4 * u + 1], ps[4 * u + 2], ps[4 * u + 3]});
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        FA_LDS char* d0 = dob + (16 * u) * QR + db * 64;
        FA_LDS char* q0p = qb + (16 * u) * QR + db * 64;
        const i16x4_t dlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)(d0 + t_lo));
        const i16x4_t dup = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)(d0 + t_up));
        const i16x4_t qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)(q0p + t_lo));
        const i16x4_t qup = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)(q0p + t_up));
        const u32x4_t draw = {__builtin_bit_cast(u32x2_t, dlo)[0], __builtin_bit_cast(u32x2_t, dlo)[1],
                              __builtin_bit_cast(u32x2_t, dup)[0], __builtin_bit_cast(u32x2_t, dup)[1]};
        const u32x4_t qraw = {__builtin_bit_cast(u32x2_t, qlo)[0], __builtin_bit_cast(u32x2_t, qlo)[1],
                              __builtin_bit_cast(u32x2_t, qup)[0], __builtin_bit_cast(u32x2_t, qup)[1]};
        dvacc[db] = M::mma(__builtin_bit_cast(frag, draw), pfr, dvacc[db]);
        dkacc[db] = M::mma(__builtin_bit_cast(frag, qraw), sfr, dkacc[db]);
      }
    }
    }
    if (t + 1 < qt_end) stats_store(nb);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of tile t+1 have landed
    __syncthreads();                // ... and everyone's; stage t is free
  };

  if (qt0 < qt_end) {
    issue(qt0, (FA_LDS char*)stage0);
    stats_load(qt0);
    stats_store((FA_LDS char*)stage0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int t = qt0;
    for (; t + 1 < qt_end; t += 2) {
      step(t, (FA_LDS char*)stage0, (FA_LDS char*)stage1);
      step(t + 1, (FA_LDS char*)stage1, (FA_LDS char*)stage0);
    }
    if (t < qt_end) step(t, (FA_LDS char*)stage0, (FA_LDS char*)stage1);
  }

  // dK = scale * dK^T^T, dV = dV^T^T, rounded to the input type
  if constexpr (kPinAcc) {  // the last accumulator MFMAs before the VALU reads
    mfma_drain_a<DBLK>(dvacc);
    mfma_drain_a<DBLK>(dkacc);
  }
  if (wave_keys == 0) return;
  const auto rdk = make_rsrc(dkg + (int64_t)kw * a.dk_ss, (wave_keys - 1) * (int32_t)a.dk_ss * 2 + a.head_dim * 2);
  const auto rdv = make_rsrc(dvg + (int64_t)kw * a.dv_ss, (wave_keys - 1) * (int32_t)a.dv_ss * 2 + a.head_dim * 2);
  const uint32_t krow = (uint32_t)(l32 * (int32_t)a.dk_ss * 2);
  const uint32_t vrow = (uint32_t)(l32 * (int32_t)a.dv_ss * 2);
  const float sc = a.scale;
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = db * 32 + 8 * g + 4 * hi;
      const bool ok = d0 < a.head_dim && l32 < wave_keys;
      const u32x2_t wk = {M::pack2(dkacc[db][4 * g + 0] * sc, dkacc[db][4 * g + 1] * sc),
                          M::pack2(dkacc[db][4 * g + 2] * sc, dkacc[db][4 * g + 3] * sc)};
      const u32x2_t wv = {M::pack2(dvacc[db][4 * g + 0], dvacc[db][4 * g + 1]),
                          M::pack2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3])};
      __builtin_amdgcn_raw_buffer_store_b64(wk, rdk, ok ? krow + d0 * 2 : kOutOfRange, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b64(wv, rdv, ok ? vrow + d0 * 2 : kOutOfRange, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// fp32 inputs: a small-problem path in the style of the fp32 forward -- the
// same two phases with v_mfma_f32_32x32x2f32, single-buffered LDS tiles
// filled with plain loads, P and dS kept in fp32.  D = head_dim rounded up to
// 32.  An MFMA of this shape contracts 2 elements: lane half hi supplies
// k-slot hi, and every operand below addresses its element by the same
// (register, hi) -> key or query map, so each product sees matching k.
// ---------------------------------------------------------------------------
template <int D>
struct BwdF32 {
  static constexpr int NW = 4;
  static constexpr int KSTEPS = D / 2;
  static constexpr int DBLK = D / 32;
  static constexpr int ROW = D + 1;  // floats; odd stride spreads rows over banks
  static_assert(D % 32 == 0 && D <= 128, "head_dim padding");
};

__device__ inline f32x16_t mma_f32(float a, float b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// dQ: 4 waves x 32 queries; 64-key K/V tiles.  S^T = K Q^T, dP^T = V dO^T
// (lane = query), dQ^T += K^T dS^T.
template <int D>
__device__ __forceinline__ void fa_bwd_dq_f32_body(const BwdArgs& a) {
  using G = BwdF32<D>;
  constexpr int BN = 64, NW = G::NW, KSTEPS = G::KSTEPS, DBLK = G::DBLK, ROW = G::ROW;
  __shared__ float kt_lds[BN * ROW];
  __shared__ float vt_lds[BN * ROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  int bh, qt;
  map_bwd_workgroup(a, blockIdx.x, a.causal != 0, bh, qt);
  const int b = bh / a.heads, h = bh - b * a.heads;
  const float* qg = (const float*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
  const float* dog = (const float*)a.dout + (int64_t)b * a.do_sb + (int64_t)h * a.do_sh;
  const float* kg = (const float*)a.k + (int64_t)b * a.k_sb + (int64_t)h * a.k_sh;
  const float* vg = (const float*)a.v + (int64_t)b * a.v_sb + (int64_t)h * a.v_sh;
  float* dqg = (float*)a.dq + (int64_t)b * a.dq_sb + (int64_t)h * a.dq_sh;

  const int q0 = qt * 32 * NW;
  const int qw = q0 + wave * 32, my_q = qw + l32;
  const bool q_ok = my_q < a.seq_q;
  const int wave_last = min(qw + 31, a.seq_q - 1);
  const int kv_end = a.causal ? min(a.seq_k, min(a.seq_q, q0 + 32 * NW)) : a.seq_k;
  const int n_tiles = (kv_end + BN - 1) / BN;

  float qf[KSTEPS], dof[KSTEPS];
  const float qsign = a.neg_scale ? -1.f : 1.f;
#pragma unroll
  for (int st = 0; st < KSTEPS; ++st) {
    const int col = 2 * st + hi;
    const bool in = q_ok && col < a.head_dim;
    qf[st] = in ? qsign * qg[(int64_t)my_q * a.q_ss + col] : 0.f;
    dof[st] = in ? dog[(int64_t)my_q * a.do_ss + col] : 0.f;
  }
  const float L2 = q_ok ? a.lse[(int64_t)bh * a.seq_q + my_q] * kLog2e : 0.f;
  const float Dl = q_ok ? a.delta[(int64_t)bh * a.seq_q + my_q] : 0.f;
  const float c = a.c;

  f32x16_t acc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) acc[db] = (f32x16_t){};

  for (int t = 0; t < n_tiles; ++t) {
    __syncthreads();  // previous tile consumed
    const int key0 = t * BN;
    for (int e = tid; e < BN * D; e += 64 * NW) {
      const int row = e / D, col = e - (e / D) * D;
      const bool ok = key0 + row < a.seq_k && col < a.head_dim;
      kt_lds[row * ROW + col] = ok ? kg[(int64_t)(key0 + row) * a.k_ss + col] : 0.f;
      vt_lds[row * ROW + col] = ok ? vg[(int64_t)(key0 + row) * a.v_ss + col] : 0.f;
    }
    __syncthreads();
    if (qw >= a.seq_q || (a.causal && key0 > wave_last)) continue;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      f32x16_t s = (f32x16_t){}, dp = (f32x16_t){};
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st) {
        s = mma_f32(kt_lds[(kb2 * 32 + l32) * ROW + 2 * st + hi], qf[st], s);
        dp = mma_f32(vt_lds[(kb2 * 32 + l32) * ROW + 2 * st + hi], dof[st], dp);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = kb2 * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);  // key of register r
        const int key = key0 + kl;
        const bool vis = q_ok && key < a.seq_k && (!a.causal || key <= my_q);
        const float p = vis ? fast_exp2(__builtin_fmaf(s[r], c, -L2)) : 0.f;
        const float ds = p * (dp[r] - Dl);
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
          acc[db] = mma_f32(kt_lds[kl * ROW + db * 32 + l32], ds, acc[db]);
      }
    }
  }
  if (!q_ok) return;
  const float sc = a.scale;
  float* row = dqg + (int64_t)my_q * a.dq_ss;
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = db * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (d < a.head_dim) row[d] = acc[db][r] * sc;
    }
}

// dK/dV: 4 waves x 32 keys; 32-query Q/dO tiles with their lse and delta.
// S = Q K^T, dP = dO V^T (rows = queries, lane = key), then
// dV^T += dO^T P and dK^T += Q^T dS.
template <int D>
__device__ __forceinline__ void fa_bwd_dkv_f32_body(const BwdArgs& a) {
  using G = BwdF32<D>;
  constexpr int BQ = 32, NW = G::NW, KSTEPS = G::KSTEPS, DBLK = G::DBLK, ROW = G::ROW;
  __shared__ float q_lds[BQ * ROW];
  __shared__ float do_lds[BQ * ROW];
  __shared__ float l_lds[BQ];
  __shared__ float d_lds[BQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  int bh, kt;
  map_bwd_workgroup(a, blockIdx.x, false, bh, kt);
  const int b = bh / a.heads, h = bh - b * a.heads;
  const float* qg = (const float*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
  const float* dog = (const float*)a.dout + (int64_t)b * a.do_sb + (int64_t)h * a.do_sh;
  const float* kg = (const float*)a.k + (int64_t)b * a.k_sb + (int64_t)h * a.k_sh;
  const float* vg = (const float*)a.v + (int64_t)b * a.v_sb + (int64_t)h * a.v_sh;
  float* dkg = (float*)a.dk + (int64_t)b * a.dk_sb + (int64_t)h * a.dk_sh;
  float* dvg = (float*)a.dv + (int64_t)b * a.dv_sb + (int64_t)h * a.dv_sh;
  const float* lseg = a.lse + (int64_t)bh * a.seq_q;
  const float* delg = a.delta + (int64_t)bh * a.seq_q;

  const int k0 = kt * 32 * NW;
  const int kw = k0 + wave * 32, my_k = kw + l32;
  const bool k_ok = my_k < a.seq_k;
  const int qt0 = a.causal ? min(k0, a.seq_q) / BQ : 0;
  const int qt_end = (a.seq_q + BQ - 1) / BQ;

  float kf[KSTEPS], vf[KSTEPS];
  const float ksign = a.neg_scale ? -1.f : 1.f;
#pragma unroll
  for (int st = 0; st < KSTEPS; ++st) {
    const int col = 2 * st + hi;
    const bool in = k_ok && col < a.head_dim;
    kf[st] = in ? ksign * kg[(int64_t)my_k * a.k_ss + col] : 0.f;
    vf[st] = in ? vg[(int64_t)my_k * a.v_ss + col] : 0.f;
  }
  const float c = a.c;
  f32x16_t dvacc[DBLK], dkacc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
    dvacc[db] = (f32x16_t){};
    dkacc[db] = (f32x16_t){};
  }

  for (int t = qt0; t < qt_end; ++t) {
    __syncthreads();  // previous tile consumed
    const int qa = t * BQ;
    for (int e = tid; e < BQ * D; e += 64 * NW) {
      const int row = e / D, col = e - (e / D) * D;
      const bool ok = qa + row < a.seq_q && col < a.head_dim;
      q_lds[row * ROW + col] = ok ? qg[(int64_t)(qa + row) * a.q_ss + col] : 0.f;
      do_lds[row * ROW + col] = ok ? dog[(int64_t)(qa + row) * a.do_ss + col] : 0.f;
    }
    if (tid < BQ) {
      const bool ok = qa + tid < a.seq_q;
      l_lds[tid] = ok ? lseg[qa + tid] * kLog2e : 0.f;
      d_lds[tid] = ok ? delg[qa + tid] : 0.f;
    }
    __syncthreads();
    if (kw >= a.seq_k || (a.causal && kw > qa + BQ - 1)) continue;
    f32x16_t s = (f32x16_t){}, dp = (f32x16_t){};
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
      s = mma_f32(q_lds[l32 * ROW + 2 * st + hi], kf[st], s);
      dp = mma_f32(do_lds[l32 * ROW + 2 * st + hi], vf[st], dp);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ql = 8 * (r >> 2) + 4 * hi + (r & 3);  // query of register r
      const int q = qa + ql;
      const bool vis = k_ok && q < a.seq_q && (!a.causal || my_k <= q);
      const float p = vis ? fast_exp2(__builtin_fmaf(s[r], c, -l_lds[ql])) : 0.f;
      const float ds = p * (dp[r] - d_lds[ql]);
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        dvacc[db] = mma_f32(do_lds[ql * ROW + db * 32 + l32], p, dvacc[db]);
        dkacc[db] = mma_f32(q_lds[ql * ROW + db * 32 + l32], ds, dkacc[db]);
      }
    }
  }
  if (!k_ok) return;
  const float sc = a.scale;
  float* krow = dkg + (int64_t)my_k * a.dk_ss;
  float* vrow = dvg + (int64_t)my_k * a.dv_ss;
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = db * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (d < a.head_dim) {
        krow[d] = dkacc[db][r] * sc;
        vrow[d] = dvacc[db][r];
      }
    }
}

}  // namespace fa
