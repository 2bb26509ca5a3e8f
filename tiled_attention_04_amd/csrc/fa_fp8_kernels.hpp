// fa_fp8_kernels.hpp -- gfx950 forward for float8 e5m2 inputs.
//
// The fp8 variant of "Understanding Triton Tutorials Part 2", section "Fused
// Attention 2": Q, K and V in float8 e5m2, V stored transposed (key index
// contiguous), P cast to e5m2 before P V, O written in e5m2, the softmax
// itself in fp32 (the same online algorithm as the 16-bit kernel).
//
// MI355X design (not taken from the pages):
//  * v_mfma_f32_32x32x64_f8f6f4 (e5m2 x e5m2, twice the bf16 rate): each MFMA
//    contracts 64 bytes; A and B pair their bytes through the same (lane
//    half, byte) -> k map, so any k order used identically on both operands
//    is exact;
//  * S^T = K Q^T: K from LDS (A), the wave's Q resident in registers (B);
//  * the K tile is loaded with its rows permuted inside every 32-row block
//    (LDS row 8j + 4h + i holds key 16h + 4j + i), so the 16 score registers
//    of lane half h belong to 16 consecutive keys;
//  * P (e5m2) is then directly the B operand of O^T += V^T P^T with k = the 64
//    keys of the tile, and the V^T fragments are two 16-byte reads of the
//    key-major V tile (no transposing read needed);
//  * rows are padded to 16 (mod 256) bytes: conflict-free 16-row reads.
#pragma once
#include "fa_fwd_kernels.hpp"

namespace fa {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

__device__ inline f32x16_t mma_e5m2(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c) {
  // format codes 1 = bf8 (e5m2) for A and B; no block scaling
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 1, 1, 0, 0, 0, 0);
}

// four floats -> four e5m2 bytes (round to nearest even), x0 in the low byte
__device__ inline uint32_t pack4_e5m2(float x0, float x1, float x2, float x3) {
  // the first conversion writes bytes 0-1 and keeps bytes 2-3 of its old
  // value, which the second overwrites: start from an unspecified register
  // instead of materialising a zero
  int w;
  asm volatile("" : "=v"(w));
  w = __builtin_amdgcn_cvt_pk_bf8_f32(x0, x1, w, false);
  w = __builtin_amdgcn_cvt_pk_bf8_f32(x2, x3, w, true);
  return (uint32_t)w;
}

template <int D, int NW>
struct TileF8 {
  static constexpr int BM = 32 * NW;      // query rows per workgroup
  static constexpr int BN = 64;           // keys per K/V tile
  static constexpr int KSTEPS = D / 64;   // 64-byte k-steps of S^T
  static constexpr int DBLK = D / 32;     // 32-dim blocks of O^T
  static constexpr int KROW = D + 16;     // K rows: head_dim bytes + pad (16 mod 256 for d <= 128)
  static constexpr int VROW = BN + 16;    // V^T rows (one per dim): 64 key bytes + pad
  static constexpr int KSLOTS = KROW / 16, VSLOTS = VROW / 16;
  static constexpr int KINSTR = BN * KSLOTS / 64;            // wave-wide 1 KiB loads per K tile
  static constexpr int VINSTR = (D * VSLOTS + 63) / 64;      // ... per V^T tile
  static constexpr int KPER = (KINSTR + NW - 1) / NW, VPER = (VINSTR + NW - 1) / NW;
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VBYTES = VINSTR * 1024;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static_assert(D == 64 || D == 128 || D == 256, "fp8 head_dim padding");
  static_assert((BN * KSLOTS) % 64 == 0, "whole wave loads of K");
};

// key held in LDS row m (0..63) of a K tile
__device__ inline int f8_key_of_row(int m) {
  const int blk = m & ~31, r = m & 31;
  return blk + 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

template <int D, int NW>
__device__ __forceinline__ void fa_fwd_e5m2_body(const FwdArgs& a) {
  using G = TileF8<D, NW>;
  constexpr int BN = G::BN, KSTEPS = G::KSTEPS, DBLK = G::DBLK, KROW = G::KROW, VROW = G::VROW;

  __shared__ __attribute__((aligned(1024))) char smem[G::LDS_BYTES];
  FA_LDS char* lds = (FA_LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  int bh, qt, split;
  map_workgroup(a, blockIdx.x, bh, qt, split);
  const int b = bh / a.heads, h = bh - b * a.heads;
  const uint8_t* qg = (const uint8_t*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
  const uint8_t* kg = (const uint8_t*)a.k + (int64_t)b * a.k_sb + (int64_t)h * a.k_sh;
  const uint8_t* vg = (const uint8_t*)a.v + (int64_t)b * a.v_sb + (int64_t)h * a.v_sh;  // [dim][key]
  uint8_t* og = (uint8_t*)a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh;

  const int q0 = qt * G::BM;
  const int qw = q0 + wave * 32;
  const int my_q = qw + l32;
  // last key this lane's row may see (the key tail, and causal: its own row)
  const int key_lim = a.causal ? min(a.seq_k - 1, my_q) : a.seq_k - 1;
  const bool wave_live = qw < a.seq_q;
  const int wave_rows = wave_live ? min(32, a.seq_q - qw) : 0;
  const int kv_end = a.causal ? min(a.seq_k, min(a.seq_q, q0 + G::BM)) : a.seq_k;
  const int n_tiles = (kv_end + BN - 1) / BN;

  // resident Q (B operand): lane = (query l32, bytes 64*st + 32*hi .. +31)
  i32x8_t qf[KSTEPS];
  {
    const int32_t nrec = wave_rows > 0 ? (wave_rows - 1) * (int32_t)a.q_ss + a.head_dim : 0;
    const auto rq = make_rsrc(qg + (int64_t)(wave_live ? qw : 0) * a.q_ss, nrec);
    const uint32_t sign = a.neg_scale ? 0x80808080u : 0u;
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int col = st * 64 + hi * 32 + half * 16;
        const uint32_t off = col < a.head_dim ? (uint32_t)(l32 * (int32_t)a.q_ss + col) : kOutOfRange;
        u32x4_t raw = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
        raw ^= (u32x4_t){sign, sign, sign, sign};
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[st][4 * half + e] = (int32_t)raw[e];
      }
  }

  // direct-to-LDS loads: K rows permuted (see f8_key_of_row), V^T rows = dims
  uint32_t koff[G::KPER];
#pragma unroll
  for (int n = 0; n < G::KPER; ++n) {
    const int slot = (wave + NW * n) * 64 + lane;
    const int row = slot / G::KSLOTS, ch = slot - (slot / G::KSLOTS) * G::KSLOTS;
    koff[n] = ch * 16 < a.head_dim ? (uint32_t)(f8_key_of_row(row) * (int32_t)a.k_ss + ch * 16)
                                   : kOutOfRange;
  }
  int vrow_of[G::VPER], vch_of[G::VPER];
#pragma unroll
  for (int n = 0; n < G::VPER; ++n) {
    const int slot = (wave + NW * n) * 64 + lane;
    vrow_of[n] = slot / G::VSLOTS;
    vch_of[n] = slot - (slot / G::VSLOTS) * G::VSLOTS;
  }
  // tile j: K into the K area, V^T into the V area of LDS stage j & 1
  auto issue_k = [&](int j) {
    const int key0 = j * BN;
    const int rows = min(BN, a.seq_k - key0);
    const auto rk = make_rsrc(kg + (int64_t)key0 * a.k_ss, (rows - 1) * (int32_t)a.k_ss + a.head_dim);
    FA_LDS char* kb = lds + (j & 1) * G::STAGE;
#pragma unroll
    for (int n = 0; n < G::KPER; ++n)
      if (wave + NW * n < G::KINSTR)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (FA_LDS void*)(kb + (wave + NW * n) * 1024), 16,
                                                 koff[n], 0, 0, 0);
  };
  // V^T rows are dims with the keys contiguous; 16-key chunks starting at or
  // past seq_k read nothing, and a chunk that straddles seq_k reads the row
  // up to the next multiple of 16 keys (those bytes meet P = 0)
  auto issue_v = [&](int j) {
    const int key0 = j * BN;
    const int rows = min(BN, a.seq_k - key0);
    const auto rv = make_rsrc(vg + key0, (a.head_dim - 1) * (int32_t)a.v_sd + ((rows + 15) & ~15));
    FA_LDS char* vb = lds + (j & 1) * G::STAGE + G::KBYTES;
#pragma unroll
    for (int n = 0; n < G::VPER; ++n)
      if (wave + NW * n < G::VINSTR) {
        const bool ok = vrow_of[n] < a.head_dim && vch_of[n] < 4 && vch_of[n] * 16 < rows;
        const uint32_t off = ok ? (uint32_t)(vrow_of[n] * (int32_t)a.v_sd + vch_of[n] * 16) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (FA_LDS void*)(vb + (wave + NW * n) * 1024), 16,
                                                 off, 0, 0, 0);
      }
  };

  f32x16_t acc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) acc[db] = (f32x16_t){};
  // reference max starts at the lowest finite value rather than -inf: the first
  // tile with any visible key replaces it (alpha = 0), and exp2(s c - m_run)
  // needs no guard against -inf - (-inf)
  float m_run = -__FLT_MAX__, l_run = 0.f;
  const float c = a.c;
  const int k_lane = l32 * KROW + hi * 32;  // A operand of S^T: LDS row l32 (+32 kb2), 32 bytes
  const int v_lane = l32 * VROW + hi * 16;  // A operand of O^T: dim row l32 (+32 db), keys 16h.., 32+16h..

  auto scores = [&](int stage, f32x16_t (&s)[2]) {
    FA_LDS char* kb = lds + stage * G::STAGE;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) s[kb2] = (f32x16_t){};
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        FA_LDS char* p = kb + k_lane + kb2 * 32 * KROW + st * 64;
        const u32x4_t lo = *(FA_LDS u32x4_t*)p;
        const u32x4_t up = *(FA_LDS u32x4_t*)(p + 16);
        const i32x8_t kf = {(int32_t)lo[0], (int32_t)lo[1], (int32_t)lo[2], (int32_t)lo[3],
                            (int32_t)up[0], (int32_t)up[1], (int32_t)up[2], (int32_t)up[3]};
        s[kb2] = mma_e5m2(kf, qf[st], s[kb2]);
      }
  };

  // masks, row max and the lazy rescale; score register r of block kb2 in
  // lane half hi belongs to key 32 kb2 + 16 hi + r
  auto stats = [&](int t, f32x16_t (&s)[2]) {
    const int key0 = t * BN;
    if ((key0 + BN > a.seq_k) || (a.causal && key0 + BN - 1 > qw)) {
      // key 32 kb2 + 16 hi + r is visible iff its offset 32 kb2 + r (a
      // constant) is at most dl: one compare and one select per score
      const int dl = key_lim - key0 - 16 * hi;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb2][r] = kb2 * 32 + r <= dl ? s[kb2][r] : -INFINITY;
    }
    const float m_tile = xlane_max(row_max32(s[0], s[1])) * c;
    const float m_new = __builtin_elementwise_maximum(m_run, m_tile);
    const bool upd = m_new > m_run + kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(upd)) {
      const float alpha = upd ? fast_exp2(m_run - m_new) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) acc[db] *= alpha;
      m_run = upd ? m_new : m_run;
    }
  };

  // P = exp2(s c - m) in e5m2: bytes 0..15 keys 16 hi + r (block 0), 16..31 block 1
  auto probs = [&](const f32x16_t (&s)[2], i32x8_t& pf) {
    const float msub = m_run;
    float part[4];  // four partial sums, each started by its first term
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const float p0 = fast_exp2(__builtin_fmaf(s[kb2][r], c, -msub));
        const float p1 = fast_exp2(__builtin_fmaf(s[kb2][r + 1], c, -msub));
        const float p2 = fast_exp2(__builtin_fmaf(s[kb2][r + 2], c, -msub));
        const float p3 = fast_exp2(__builtin_fmaf(s[kb2][r + 3], c, -msub));
        if (kb2 == 0)
          part[r >> 2] = (p0 + p1) + (p2 + p3);
        else
          part[r >> 2] += (p0 + p1) + (p2 + p3);
        pf[4 * kb2 + (r >> 2)] = (int32_t)pack4_e5m2(p0, p1, p2, p3);
      }
    l_run += (part[0] + part[1]) + (part[2] + part[3]);
  };

  auto pv = [&](int stage, const i32x8_t& pf) {
    FA_LDS char* vb = lds + stage * G::STAGE + G::KBYTES;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      FA_LDS char* p = vb + v_lane + db * 32 * VROW;
      const u32x4_t lo = *(FA_LDS u32x4_t*)p;           // keys 16 hi .. +15
      const u32x4_t up = *(FA_LDS u32x4_t*)(p + 32);    // keys 32 + 16 hi .. +15
      const i32x8_t vf = {(int32_t)lo[0], (int32_t)lo[1], (int32_t)lo[2], (int32_t)lo[3],
                          (int32_t)up[0], (int32_t)up[1], (int32_t)up[2], (int32_t)up[3]};
      acc[db] = mma_e5m2(vf, pf, acc[db]);
    }
  };

  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  // One pipelined step for tile t (parity P = t & 1): S(t+1) alongside the
  // softmax of tile t, then P(t) V(t); K runs one tile ahead of V, so K(t+2)
  // and V(t+1) load during step t.
  auto step = [&](int t, auto parity, auto has_next, f32x16_t (&cur)[2], f32x16_t (&nxt)[2]) {
    constexpr int P = decltype(parity)::value;
    stats(t, cur);
    if (t + 2 < n_tiles) issue_k(t + 2);
    if (t + 1 < n_tiles) issue_v(t + 1);
    i32x8_t pf;
    if constexpr (decltype(has_next)::value) scores(1 - P, nxt);
    probs(cur, pf);
    pv(P, pf);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  f32x16_t sa[2], sb[2];
  if (n_tiles > 0) {
    issue_k(0);
    issue_v(0);
    if (n_tiles > 1) issue_k(1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    scores(0, sa);
    __syncthreads();  // K(0) consumed before step 0 loads K(2) over it
    int t = 0;
    for (; t + 2 < n_tiles; t += 2) {
      step(t, Even{}, Yes{}, sa, sb);
      step(t + 1, Odd{}, Yes{}, sb, sa);
    }
    if (t + 1 < n_tiles) {
      step(t, Even{}, Yes{}, sa, sb);
      step(t + 1, Odd{}, No{}, sb, sa);
    } else {
      step(t, Even{}, No{}, sa, sb);
    }
  }

  // epilogue: O = acc / l in e5m2, lse = ln2 * (m + log2 l)
  if (!wave_live) return;
  const float l_tot = xlane_sum(l_run);
  const float inv = 1.0f / l_tot;
  const int32_t onrec = (wave_rows - 1) * (int32_t)a.o_ss + a.head_dim;
  const auto ro = make_rsrc(og + (int64_t)qw * a.o_ss, onrec);
  const uint32_t orow = (uint32_t)(l32 * (int32_t)a.o_ss);
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = db * 32 + 8 * g + 4 * hi;
      const uint32_t off = (d0 < a.head_dim && l32 < wave_rows) ? orow + d0 : kOutOfRange;
      const uint32_t w = pack4_e5m2(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv,
                                    acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
      __builtin_amdgcn_raw_buffer_store_b32(w, ro, off, 0, 0);
    }
  if (hi == 0 && a.lse != nullptr && my_q < a.seq_q)
    a.lse[(int64_t)bh * a.seq_q + my_q] = (m_run + __log2f(l_tot)) * kLn2;
}

}  // namespace fa
