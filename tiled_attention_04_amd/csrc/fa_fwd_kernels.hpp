// fa_fwd_kernels.hpp -- gfx950 (MI355X) kernels of the fused attention forward.
//
// Method: the FlashAttention-2 forward of "[CS336] Assignment 2: Systems",
// section "FlashAttention V2 / Forward Pass", and of "Understanding Triton
// Tutorials Part 2", section "Fused Attention 2": a tile of queries stays
// resident, K/V tiles stream past it, a running row max m and row sum l keep
// the softmax online (with exp2 and log2(e) folded into the scale), the
// un-normalised output accumulates in fp32 and is divided by l once at the
// end, and the per-row logsumexp is emitted.  Causal tiles above the
// diagonal are never visited.
//
// MI355X design (not taken from the pages):
//  * one workgroup of NW waves per (batch*head, query tile of 32*NW rows);
//    each wave owns 32 query rows for the whole key loop;
//  * scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_{bf16,f16}: K (from LDS) is the A operand and the
//    wave's Q fragment (registers, loaded once) is the B operand.  In the
//    32x32 result layout lane l holds 16 keys of query (l % 32), so row max
//    and row sum are in-lane except for one exchange with lane l ^ 32;
//  * P stays in registers: the result layout of S^T, rounded to bf16/f16, is
//    directly the B operand of O^T += V^T P^T (keys permuted consistently on
//    both operands); V^T fragments come from LDS with ds_read_b64_tr_b16,
//    which transposes 4 keys x 16 dims per 16-lane group on the fly;
//  * K/V tiles are double-buffered in LDS, loaded one tile ahead by buffer
//    loads that write LDS directly, rows padded so the MFMA operand reads of
//    one wave spread over the banks (8-wave workgroups at head_dim 64 and
//    128: four stages each, loads two tiles ahead);
//  * keys >= seq_k and (causal) keys > query are masked to -inf; key rows
//    beyond seq_k and dims beyond head_dim are zero-filled;
//  * the running max is refreshed lazily: O and l are rescaled only when the
//    row max grows by more than RESCALE_LOG2 (base 2), so P <= 2^RESCALE_LOG2.
//    Any reference value at or below the true running max gives the same
//    O = acc / l and lse = m + log l in exact arithmetic; the pages rescale on
//    every tile;
//  * workgroup ids are remapped so all query tiles of one (batch, head) run
//    on the same XCD (shared L2 for its K/V stream), heaviest causal tiles
//    first;
//  * head_dim 129..256 runs the same method in fa_fwd_wide.hpp.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (P <= 256)




struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_sb, q_sh, q_ss;  // element strides: batch, head, seq (dim stride is 1)
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t v_sd;      // dim stride of V (the e5m2 path takes V key-major: seq stride 1)
  int32_t heads, seq_q, seq_k, head_dim;
  int32_t n_qtiles;  // ceil(seq_q / BM)
  int32_t n_bh;      // batch * heads
  float c;           // |sm_scale| * log2(e), at least 1e-30
  int32_t neg_scale;  // sm_scale < 0: Q is negated in registers
  int32_t causal;
  int32_t xcd_remap;  // n_bh % 8 == 0: keep one (batch, head) on one XCD
  // key splitting: n_splits workgroups share each query tile's key tiles and
  // write fp32 partials (O_r normalised by its own row sum, lse_r; -inf and 0
  // for rows that see no key of the share) that fa_fwd_combine merges
  int32_t n_splits;   // 1: no splitting, O and lse written directly
  float* part_o;      // [n_splits, n_bh, seq_q, head_dim]
  float* part_lse;    // [n_splits, n_bh, seq_q]
};

// Map the linear workgroup id to (batch*head, query tile, key split).
// Workgroups are handed to the 8 XCDs round-robin, so ids with the same
// residue mod 8 share an XCD and its L2; all tiles of one (batch, head) get
// the same residue.  Causal: heaviest (last) query tiles are dispatched first.
__device__ inline void map_workgroup(const FwdArgs& a, int wg, int& bh, int& qt, int& split) {
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
  split = rank % a.n_splits;
  rank /= a.n_splits;
  qt = a.causal ? a.n_qtiles - 1 - rank : rank;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
  typedef bf16x8_t frag;
  __device__ static inline f32x16_t mma(const frag& a, const frag& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // round-to-nearest-even pair conversion (v_cvt_pk_bf16_f32)
  __device__ static inline uint32_t pack2(float x, float y) {
    f32x2_t v = {x, y};
    bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, r);
  }
  static constexpr uint32_t kOneBits = 0x3F80u;  // 1.0
  // acc + both halves of a packed pair, in fp32 (v_dot2_f32_bf16 against (1, 1))
  __device__ static inline float sum2(uint32_t packed, float acc) {
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, packed), one, acc, false);
  }
};

template <>
struct Mfma<_Float16> {
  typedef f16x8_t frag;
  __device__ static inline f32x16_t mma(const frag& a, const frag& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float x, float y) {
    f32x2_t v = {x, y};
    f16x2_t r = __builtin_convertvector(v, f16x2_t);
    return __builtin_bit_cast(uint32_t, r);
  }
  static constexpr uint32_t kOneBits = 0x3C00u;  // 1.0
  __device__ static inline float sum2(uint32_t packed, float acc) {  // v_dot2_f32_f16
    const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, packed), one, acc, false);
  }
};

#ifdef FA_LDS_POISON
// Race check (a debug build only): the kernels fill an LDS area with NaN
// (all-ones 16-bit words) once the barrier that ends its last read has
// passed, just before its next tile is loaded; a wave that read a stage
// outside its window would then see NaN, which the parity tests catch.
template <int NT>
__device__ inline void lds_poison(FA_LDS char* base, int bytes) {
  for (int off = (int)threadIdx.x * 16; off < bytes; off += NT * 16)
    *(FA_LDS u32x4_t*)(base + off) = (u32x4_t){0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
}
#endif

// Smallest row stride (bytes, multiple of 16, >= min_bytes) congruent to 64
// or 192 modulo 256: then the 4 rows x 64 bytes that 32 lanes of a
// transposing read gather fall into disjoint bank windows.
constexpr int tr_row_stride(int min_bytes) {
  int st = (min_bytes + 15) / 16 * 16;
  while (st % 256 != 64 && st % 256 != 192) st += 16;
  return st;
}

// Slot permutation of the 16-byte chunks of an unpadded row r of ROWB bytes.
// 256-byte rows: the high two bits of the chunk index are XORed with r % 4,
// the low two with (r / 4) % 4.  128-byte rows (two per 256-byte bank
// window): bit 2 with (r / 2) % 2, the low two with (r / 4) % 4.  Either
// way 16 consecutive rows read at one chunk land on 16 distinct bank groups
// (row reads of 16 lanes per cycle), and the four rows of a transposing
// read's 32 lanes cover all 64 banks.
template <int ROWB>
__device__ __host__ constexpr int lds_swizzle(int r) {
  static_assert(ROWB == 256 || ROWB == 128, "swizzled row widths");
  return ROWB == 256 ? ((r & 3) << 2) | ((r >> 2) & 3) : (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// ---------------------------------------------------------------------------
// Buffer-resource helpers.  A raw buffer load whose byte offset lies at or
// beyond num_records returns zeros without touching memory, which gives
// branch-free zero padding of ragged tiles; a store there is dropped.
// ---------------------------------------------------------------------------
constexpr int kBufferFlags = 0x00020000;  // raw 32-bit dword access, no swizzle
constexpr uint32_t kOutOfRange = 0xFFFFFF00u;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_bytes,
                                           kBufferFlags);
}

__device__ inline float xlane_max(float x) {  // max with lane l ^ 32
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

__device__ inline float xlane_sum(float x) {  // sum with lane l ^ 32
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Maximum of the 32 values of two 16-register score blocks as a depth-4 tree
// of v_maximum3_f32 (a linear chain would be 16 dependent instructions).
__device__ inline float row_max32(const f32x16_t& a, const f32x16_t& b) {
  float t[11];
#pragma unroll
  for (int i = 0; i < 5; ++i)
    t[i] = __builtin_elementwise_maximum(a[3 * i], __builtin_elementwise_maximum(a[3 * i + 1], a[3 * i + 2]));
#pragma unroll
  for (int i = 0; i < 5; ++i)
    t[5 + i] = __builtin_elementwise_maximum(b[3 * i], __builtin_elementwise_maximum(b[3 * i + 1], b[3 * i + 2]));
  t[10] = __builtin_elementwise_maximum(a[15], b[15]);
  const float u0 = __builtin_elementwise_maximum(t[0], __builtin_elementwise_maximum(t[1], t[2]));
  const float u1 = __builtin_elementwise_maximum(t[3], __builtin_elementwise_maximum(t[4], t[5]));
  const float u2 = __builtin_elementwise_maximum(t[6], __builtin_elementwise_maximum(t[7], t[8]));
  const float u3 = __builtin_elementwise_maximum(t[9], t[10]);
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(u0, u1),
                                       __builtin_elementwise_maximum(u2, u3));
}

// ---------------------------------------------------------------------------
// 16-bit inputs (bf16 / f16).  D = head_dim rounded up to 16, NW waves per
// workgroup, OCC waves per SIMD targeted by the register allocator.
// ---------------------------------------------------------------------------
template <typename T, int D, int NW, bool XB = false, bool SWZ = false>
struct Tile16 {
  static constexpr int BM = 32 * NW;           // query rows per workgroup
  static constexpr int BN = 64;                // keys per K/V tile
  static constexpr int NT = 64 * NW;           // threads per workgroup
  static constexpr int KSTEPS = D / 16;        // k-steps of the S^T MFMA (16 dims each)
  // 32-dim blocks of the O^T accumulator (XB: one more, for the row-sum column)
  static constexpr int DBLK = (D + 31) / 32 + (XB ? 1 : 0);
  // K rows: stride = 16 (mod 256) bytes, so the 32 lanes reading one 16-byte
  // chunk of 32 consecutive rows fall on distinct bank groups.
  // V rows: stride = 64 or 192 (mod 256) bytes, so the rows gathered by a
  // transposing read fall on distinct banks.
  // SWZ (head_dim 64 and 128): unpadded rows of 128 or 256 bytes, 16-byte
  // chunk c of row r at slot c ^ lds_swizzle(r) instead: 8 or 16 loads of
  // 1 KiB per tile, which eight waves issue one or two each.
  static constexpr int KROW = SWZ ? D * 2 : D * 2 + 16;
  static constexpr int VROW = SWZ ? DBLK * 64 : tr_row_stride(DBLK * 64);
  static_assert(!SWZ || (KROW == VROW && (KROW == 256 || KROW == 128)), "swizzled row widths");
  static constexpr int KSLOTS = KROW / 16;     // 16-byte LDS slots per K row (incl. padding)
  static constexpr int VSLOTS = VROW / 16;
  static constexpr int KINSTR = BN * KSLOTS / 64;  // wave-wide 1 KiB loads per K tile
  static constexpr int VINSTR = BN * VSLOTS / 64;
  static constexpr int KPER = (KINSTR + NW - 1) / NW;  // per wave
  static constexpr int VPER = (VINSTR + NW - 1) / NW;
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VBYTES = BN * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
  // the epilogue stages each wave's 32 x D output rows in LDS (row stride
  // D * 2 + 16 bytes) to store them as whole 16-byte pieces of rows
  static constexpr int OROW = D * 2 + 16;
  static constexpr int OBYTES = 32 * OROW;
  static constexpr int LDS_BYTES = 2 * STAGE > NW * OBYTES ? 2 * STAGE : NW * OBYTES;
  static_assert(D % 16 == 0 && D <= 128, "head_dim padding (wider ones: fa_fwd_wide.hpp)");
  static_assert(KROW % 16 == 0 && VROW % 16 == 0, "16-byte aligned rows");
  static_assert((BN * KSLOTS) % 64 == 0 && (BN * VSLOTS) % 64 == 0, "whole wave loads");
};

// One LDS object per (Tag, ID): a distinct __shared__ variable, so that the
// compiler can tell a direct-to-LDS load into one object from reads of
// another and does not wait for the load before those reads.
template <typename Tag, int ID, int BYTES>
__device__ __forceinline__ FA_LDS char* lds_object() {
  __shared__ __attribute__((aligned(1024))) char buf[BYTES];
  return (FA_LDS char*)buf;
}

// Body of the 16-bit kernel; the __global__ entry points that instantiate it
// (with their occupancy attributes) are defined next to the launcher.
//
// DEEP: the K/V loads run two tiles ahead instead of one.  Four LDS stages
// each for K and V, the stage of every access a compile-time constant of a
// four-step unrolled loop; the barrier at the end of step t waits only for
// the loads issued in step t - 1 (K(t + 2), V(t + 1)), so each load has two
// steps to land.
template <typename T, int D, int NW, bool XB = false, bool DEEP = false>
__device__ __forceinline__ void fa_fwd_16bit_body(const FwdArgs& a) {
  constexpr bool SWZ = DEEP;  // (head_dim 64 and 128) unpadded swizzled rows: no surplus loads
  using G = Tile16<T, D, NW, XB, SWZ>;
  using M = Mfma<T>;
  typedef typename M::frag frag;
  constexpr int BN = G::BN, KSTEPS = G::KSTEPS, DBLK = G::DBLK;
  constexpr int KROW = G::KROW, VROW = G::VROW;
  // Row sum by the matrix core where the P.V product pads the head dims (D
  // not a multiple of 32, or XB: one 32-dim block added for it): V's column
  // D is 1.0 in both LDS stages, so row D of O^T accumulates the sum of the
  // rounded weights of each query along with the output, and the VALU row
  // sum (16 dot products per tile and wave) and its rescale drop out.  The
  // padding columns are written once and never loaded over.
  constexpr bool kOnesCol = (D % 32) != 0 || XB;

  // LDS areas: without DEEP one object of two stages (K then V each); with
  // DEEP four K and four V objects.  kbuf / vbuf take a compile-time stage.
  struct Tag;
  auto kbuf = [&](auto pc) -> FA_LDS char* {
    constexpr int P = decltype(pc)::value;
    if constexpr (DEEP) return lds_object<Tag, P % 4, G::KBYTES>();
    else return lds_object<Tag, 8, G::LDS_BYTES>() + (P % 2) * G::STAGE;
  };
  auto vbuf = [&](auto pc) -> FA_LDS char* {
    constexpr int P = decltype(pc)::value;
    if constexpr (DEEP) return lds_object<Tag, 4 + P % 4, G::VBYTES>();
    else return lds_object<Tag, 8, G::LDS_BYTES>() + (P % 2) * G::STAGE + G::KBYTES;
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
  const int qw = q0 + wave * 32;        // first query row of this wave
  const int my_q = qw + l32;            // query row of this lane
  // last key this lane's row may see (the key tail, and causal: its own row)
  const int key_lim = a.causal ? min(a.seq_k - 1, my_q) : a.seq_k - 1;
  const bool wave_live = qw < a.seq_q;
  const int wave_rows = wave_live ? min(32, a.seq_q - qw) : 0;

  // keys this workgroup must visit (causal: up to its last real query), and
  // with key splitting its share [t0, t1) of those 64-key tiles
  const int kv_end = a.causal ? min(a.seq_k, min(a.seq_q, q0 + G::BM)) : a.seq_k;
  const int n_all = (kv_end + BN - 1) / BN;
  const int chunk = (n_all + a.n_splits - 1) / a.n_splits;
  const int t0 = min(n_all, split * chunk);
  const int t1 = min(n_all, t0 + chunk);

  // ---- resident Q fragment: B operand of S^T, lane = (query l32, dims 8*hi..+7 of each step)
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

  // ---- per-lane byte offsets of the direct-to-LDS tile loads (tile independent)
  uint32_t koff[G::KPER], voff[G::VPER];
  bool vlive[G::VPER];  // (ones-column layout) this lane's V chunk lies below dim D
  // DEEP: every wave issues KPER K and VPER V loads, so that the count per
  // wave is a compile-time constant; a share beyond the tile's instructions
  // repeats a valid one (the same bytes to the same place).  (Reading out of
  // range into a dump area instead measured slower.)
  auto kinstr = [&](int n) { const int i = wave + NW * n; return DEEP && i >= G::KINSTR ? i % G::KINSTR : i; };
  auto vinstr = [&](int n) { const int i = wave + NW * n; return DEEP && i >= G::VINSTR ? i % G::VINSTR : i; };
#pragma unroll
  for (int n = 0; n < G::KPER; ++n) {
    const int slot = kinstr(n) * 64 + lane;
    const int row = slot / G::KSLOTS;
    int ch = slot - row * G::KSLOTS;
    if constexpr (SWZ) ch ^= lds_swizzle<KROW>(row);  // the chunk this slot holds
    koff[n] = ch * 8 < a.head_dim ? (uint32_t)(row * (int32_t)a.k_ss * 2 + ch * 16) : kOutOfRange;
  }
#pragma unroll
  for (int n = 0; n < G::VPER; ++n) {
    const int slot = vinstr(n) * 64 + lane;
    const int row = slot / G::VSLOTS;
    int ch = slot - row * G::VSLOTS;
    if constexpr (SWZ) ch ^= lds_swizzle<VROW>(row);
    voff[n] = ch * 8 < a.head_dim ? (uint32_t)(row * (int32_t)a.v_ss * 2 + ch * 16) : kOutOfRange;
    vlive[n] = ch * 8 < D;
  }
  // Tile j's K goes to the K area and its V to the V area of LDS stage
  // (j - t0) & 1 (DEEP: stage (j - t0) % 4, passed as the compile-time pc);
  // rows >= seq_k and dims >= head_dim land as zeros.  DEEP issues the same
  // loads every step: a tile j >= t1 gets an empty range (zeros, no memory
  // access).
  auto issue_k = [&](int j, auto pc) {
    const int key0 = j * BN;
    const int rows = min(BN, a.seq_k - key0);
    const int32_t nrec = (rows - 1) * (int32_t)a.k_ss * 2 + a.head_dim * 2;
    const auto rk = make_rsrc(kg + (int64_t)key0 * a.k_ss, (!DEEP || j < t1) ? nrec : 0);
    FA_LDS char* kb;
    if constexpr (DEEP) kb = kbuf(pc);
    else kb = lds_object<Tag, 8, G::LDS_BYTES>() + ((j - t0) & 1) * G::STAGE;
#pragma unroll
    for (int n = 0; n < G::KPER; ++n)
      if (DEEP || wave + NW * n < G::KINSTR)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (FA_LDS void*)(kb + kinstr(n) * 1024), 16,
                                                 koff[n], 0, 0, 0);
  };
  auto issue_v = [&](int j, auto pc) {
    const int key0 = j * BN;
    const int rows = min(BN, a.seq_k - key0);
    const int32_t nrec = (rows - 1) * (int32_t)a.v_ss * 2 + a.head_dim * 2;
    const auto rv = make_rsrc(vg + (int64_t)key0 * a.v_ss, (!DEEP || j < t1) ? nrec : 0);
    FA_LDS char* vb;
    if constexpr (DEEP) vb = vbuf(pc);
    else vb = lds_object<Tag, 8, G::LDS_BYTES>() + ((j - t0) & 1) * G::STAGE + G::KBYTES;
#pragma unroll
    for (int n = 0; n < G::VPER; ++n)
      if ((DEEP || wave + NW * n < G::VINSTR) && (!kOnesCol || vlive[n]))
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (FA_LDS void*)(vb + vinstr(n) * 1024), 16,
                                                 voff[n], 0, 0, 0);
  };
  // (ones-column layout) V columns D..32 DBLK - 1 of every stage: 1.0 in
  // column D, zeros after it; written once, never loaded over
  auto pad_cols = [&](auto pc) {
    if constexpr (kOnesCol) {
      constexpr int C0 = D / 8, NC = 4 * DBLK - D / 8;  // first padding chunk, padding chunks per row
      for (int i = tid; i < BN * NC; i += G::NT) {
        const int row = i / NC, chk = C0 + i % NC;
        const u32x4_t val = {chk == C0 ? M::kOneBits : 0u, 0u, 0u, 0u};
        *(FA_LDS u32x4_t*)(vbuf(pc) + row * VROW + chk * 16) = val;
      }
    }
  };
  if constexpr (kOnesCol) {
    pad_cols(Even{});
    pad_cols(Odd{});
    if constexpr (DEEP) {
      pad_cols(std::integral_constant<int, 2>{});
      pad_cols(std::integral_constant<int, 3>{});
    }
  }

  // ---- online-softmax state (per lane: query l32; both halves agree on m)
  f32x16_t acc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) acc[db] = (f32x16_t){};
  float m_run = -INFINITY;  // reference max, base-2 scaled units
  float l_run = 0.f;        // partial row sum over this lane's keys (not with the ones column)
  const float c = a.c;

  // lane-constant LDS offsets of the MFMA operand reads
  const int k_lane = l32 * KROW + hi * 16;
  // SWZ: the byte offset of chunk 2 st + hi of row l32 (and of row 32 + l32)
  int k_swz[SWZ ? KSTEPS : 1];
  if constexpr (SWZ) {
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) k_swz[st] = l32 * KROW + 16 * ((2 * st + hi) ^ lds_swizzle<KROW>(l32));
  }
  const int s16 = lane & 15;
  const int v_lane = (4 * hi + (s16 >> 2)) * VROW + (16 * ((lane >> 4) & 1) + 4 * (s16 & 3)) * 2;
  // SWZ: the byte offsets of this lane's 8-byte pieces of 32-dim block db in
  // rows 4 hi + s16 / 4 and 8 further (the same in every 16-row group)
  int v_swz[SWZ ? 2 * DBLK : 1];
  if constexpr (SWZ) {
    const int r = 4 * hi + (s16 >> 2);
    const int byte = 32 * ((lane >> 4) & 1) + 8 * (s16 & 3);
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const int c = (byte >> 4) + 4 * db;
      v_swz[2 * db] = r * VROW + 16 * (c ^ lds_swizzle<VROW>(r)) + (byte & 15);
      v_swz[2 * db + 1] = (r + 8) * VROW + 16 * (c ^ lds_swizzle<VROW>(r + 8)) + (byte & 15);
    }
  }

  // S^T = K Q^T for the two 32-key blocks of the K tile in stage pc
  auto scores = [&](auto pc, f32x16_t (&s)[2]) {
    FA_LDS char* kb = kbuf(pc);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) s[kb2] = (f32x16_t){};
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const frag kf = __builtin_bit_cast(
            frag, *(FA_LDS u32x4_t*)(kb + (SWZ ? k_swz[SWZ ? st : 0] : k_lane + st * 32) + kb2 * 32 * KROW));
        s[kb2] = M::mma(kf, qf[st], s[kb2]);
      }
  };

  // masks (key tail, causal diagonal), row max and the lazy rescale for tile t
  auto stats = [&](int t, f32x16_t (&s)[2]) {
    const int key0 = t * BN;
    const bool need_mask = (key0 + BN > a.seq_k) || (a.causal && key0 + BN - 1 > qw);
    if (need_mask) {
      // key kb2 32 + 8 (r / 4) + 4 hi + r % 4 of the tile is visible iff its
      // offset cr = kb2 32 + 8 (r / 4) + r % 4 (a constant, 0..63) is at most
      // dl: one compare against an inline constant and one select per score
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
    const float m_tile = mx * c;  // c > 0, so max(s) * c = max(s * c)
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

  // P = exp2(s*c - m) rounded to the input type, and its partial row sum.
  // The sum is taken over the rounded weights, exactly the ones the P.V
  // product consumes, so O = acc / l is a convex combination of V rows: with
  // the unrounded sum, a row dominated by one key whose weight rounds off by
  // 2^-9 carries that relative error into O (up to 0.01 at |O| ~ 6, on top of
  // O's own bf16 rounding).
  auto probs = [&](const f32x16_t (&s)[2], uint32_t (&pk)[2][8]) {
    const float msub = (m_run == -INFINITY) ? 0.f : m_run;
    float part[4] = {0.f, 0.f, 0.f, 0.f};  // four short add chains instead of one long one
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

  // O^T += V^T P^T with the V tile in stage P: four 16-key steps per 32-dim block
  auto pv = [&](auto pc, const uint32_t (&pk)[2][8]) {
    FA_LDS char* vb = vbuf(pc);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4_t praw = {pk[u >> 1][4 * (u & 1) + 0], pk[u >> 1][4 * (u & 1) + 1],
                            pk[u >> 1][4 * (u & 1) + 2], pk[u >> 1][4 * (u & 1) + 3]};
      const frag pf = __builtin_bit_cast(frag, praw);
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        FA_LDS char* p0 = SWZ ? vb + v_swz[SWZ ? 2 * db : 0] + (16 * u) * VROW
                              : vb + v_lane + (16 * u) * VROW + db * 64;
        FA_LDS char* p1 = SWZ ? vb + v_swz[SWZ ? 2 * db + 1 : 0] + (16 * u) * VROW : p0 + 8 * VROW;
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)p0);
        const i16x4_t up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)p1);
        const u32x4_t vraw = {__builtin_bit_cast(u32x2_t, lo)[0], __builtin_bit_cast(u32x2_t, lo)[1],
                              __builtin_bit_cast(u32x2_t, up)[0], __builtin_bit_cast(u32x2_t, up)[1]};
        acc[db] = M::mma(__builtin_bit_cast(frag, vraw), pf, acc[db]);
      }
    }
  };

  // One pipelined step for tile t (parity = (t - t0) & 1, known at compile time):
  // the MFMAs of S(t+1) are issued in the same basic block as the softmax
  // VALU work of tile t, so the matrix pipe stays busy while P(t) is formed;
  // then P(t) V(t).  K runs one tile ahead of V in LDS: during step t the
  // loads of K(t+2) and V(t+1) are in flight.
  auto step = [&](int t, auto parity, auto has_next, f32x16_t (&cur)[2], f32x16_t (&nxt)[2]) {
    using Cur = decltype(parity);
    using Nxt = std::integral_constant<int, 1 - Cur::value>;
#ifdef FA_LDS_POISON
    // K(t) (read by S(t) in the previous step) and V(t - 1) (read by P V in
    // the previous step) are free now; K(t + 2) and V(t + 1) refill them
    lds_poison<G::NT>(kbuf(Cur{}), G::KBYTES);
    lds_poison<G::NT>(vbuf(Nxt{}), G::VBYTES);
    if constexpr (kOnesCol) {  // the padding columns are never reloaded: restore them
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      pad_cols(Nxt{});
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#endif
    // 4-wave workgroups (the small grids of short sequences): a wave without
    // query rows only loads its share of the tiles; its matrix and softmax
    // work would take LDS reads and SIMD time from the waves that have rows.
    // (The 8-wave kernel, whose grids are large, and head_dim 128, whose
    // registers are nearly all taken, keep one path: the branch measured
    // 2-3% slower there.)
    const bool work = NW != 4 || D == 128 || wave_live;
    if (work) stats(t, cur);
    if (t + 2 < t1) issue_k(t + 2, Cur{});
    if (t + 1 < t1) issue_v(t + 1, Nxt{});
    if (work) {
      uint32_t pk[2][8];
      if constexpr (decltype(has_next)::value) scores(Nxt{}, nxt);
      probs(cur, pk);
      pv(Cur{}, pk);
    } else {
      // (defined on both paths, so that the registers of the tile before
      // are not kept alive for the merge)
      nxt[0] = nxt[1] = (f32x16_t){};
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's K(t+2) / V(t+1) loads have landed
    __syncthreads();                // ... and everyone's; the areas read in step t are free
  };
  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;

  f32x16_t sa[2], sb[2];

  // DEEP: every wave issues LMIN = KPER + VPER loads in every step, so
  // vmcnt <= LMIN at the end of step t leaves only step t's own loads in
  // flight.
  constexpr int LMIN = G::KPER + G::VPER;
  static_assert(!DEEP || LMIN <= 15, "vmcnt immediate");
  // A barrier that leaves step t's loads in flight: this wave's LDS reads
  // and stores done (lgkmcnt 0), its loads older than the last LMIN landed,
  // then s_barrier.  __syncthreads() would add a workgroup release fence,
  // which waits for every LDS write in flight, the direct-to-LDS loads
  // included; the empty asm statements keep the compiler from moving LDS
  // accesses across the barrier instead.
  auto deep_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0070 | LMIN);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // step I (0..3) of the unrolled loop handles tile t = t0 + 4 m + I (its K
  // and V in stage I); it loads K(t + 3) over K(t - 1) (read by S(t - 1) two
  // steps earlier) and V(t + 2) over V(t - 2).  S(t + 1) is always formed
  // (for the last tile from a stage of zeros, never used) so that every step
  // has one shape.
  auto deep_step = [&](int t, auto ic, f32x16_t (&cur)[2], f32x16_t (&nxt)[2]) {
    constexpr int I = decltype(ic)::value;
    using K1 = std::integral_constant<int, (I + 1) % 4>;
    using K3 = std::integral_constant<int, (I + 3) % 4>;
    using V0 = std::integral_constant<int, I>;
    using V2 = std::integral_constant<int, (I + 2) % 4>;
#ifdef FA_LDS_POISON
    lds_poison<G::NT>(kbuf(K3{}), G::KBYTES);
    lds_poison<G::NT>(vbuf(V2{}), G::VBYTES);
    if constexpr (kOnesCol) {  // the padding columns are never reloaded: restore them
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      pad_cols(V2{});
    }
    deep_barrier();  // the poison stores done; step t - 1's loads may fly
#endif
    stats(t, cur);
    issue_k(t + 3, K3{});
    issue_v(t + 2, V2{});
    uint32_t pk[2][8];
    scores(K1{}, nxt);
    probs(cur, pk);
    pv(V0{}, pk);
    deep_barrier();  // this wave's loads of step t - 1 (K(t + 2), V(t + 1)) have landed, and everyone's
  };
  auto deep_loop = [&]() {
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    for (int t = t0;; t += 4) {
      deep_step(t, I0{}, sa, sb);
      if (t + 1 >= t1) break;
      deep_step(t + 1, I1{}, sb, sa);
      if (t + 2 >= t1) break;
      deep_step(t + 2, I2{}, sa, sb);
      if (t + 3 >= t1) break;
      deep_step(t + 3, I3{}, sb, sa);
      if (t + 4 >= t1) break;
    }
  };

  if (t1 > t0) {
    issue_k(t0, Even{});
    issue_v(t0, Even{});
    if constexpr (DEEP) {
      issue_k(t0 + 1, Odd{});
      issue_k(t0 + 2, std::integral_constant<int, 2>{});
      issue_v(t0 + 1, Odd{});
    } else {
      if (t0 + 1 < t1) issue_k(t0 + 1, Odd{});
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    scores(Even{}, sa);
    // K(t0) consumed by all waves before the first step loads K(t0+2) over
    // it (DEEP: the first step loads into stages not yet used)
    if constexpr (!DEEP) __syncthreads();
    if constexpr (DEEP) {
      deep_loop();
      __builtin_amdgcn_s_waitcnt(0);  // the last steps' loads (zeros) have landed
      __syncthreads();                // ... before the epilogue reuses the V stages
    } else {
      int t = t0;
      for (; t + 2 < t1; t += 2) {
        step(t, Even{}, Yes{}, sa, sb);
        step(t + 1, Odd{}, Yes{}, sb, sa);
      }
      if (t + 1 < t1) {
        step(t, Even{}, Yes{}, sa, sb);
        step(t + 1, Odd{}, No{}, sb, sa);
      } else {
        step(t, Even{}, No{}, sa, sb);
      }
    }
  }

  // ---- epilogue: O = acc / l, lse = ln2 * (m + log2 l)
  if (!wave_live) return;
  float l_tot;
  if constexpr (kOnesCol) {
    // row D of O^T: local dim ld of the last block, held by the lanes of half h1
    constexpr int ld = D - 32 * (DBLK - 1), r1 = 4 * (ld / 8) + ld % 4, h1 = (ld % 8) / 4;
    l_tot = xlane_sum(hi == h1 ? acc[DBLK - 1][r1] : 0.f);
  } else {
    l_tot = xlane_sum(l_run);
  }
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
      a.part_lse[row0 + l32] = seen ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    return;
  }
  const float inv = 1.0f / l_tot;
  const int32_t onrec = (wave_rows - 1) * (int32_t)a.o_ss * 2 + a.head_dim * 2;
  const auto ro = make_rsrc(og + (int64_t)qw * a.o_ss, onrec);
  // O through LDS (every wave is past the last barrier of the key loop, so
  // the tile stages are free): this lane's 4-dim pieces of query row l32
  // go to the wave's own 32-row area, then each lane stores whole 16-byte
  // pieces of rows, consecutive lanes covering consecutive bytes of a row
  FA_LDS char* ob;
  int orow = G::OROW;
  if constexpr (DEEP) {
    // waves 2 i and 2 i + 1 share V stage i: 64 rows at the K row stride
    // where it fits, else at the V row stride (>= 2 D bytes)
    constexpr int OR = G::KROW <= G::VROW ? G::KROW : G::VROW;
    static_assert(OR >= 2 * D, "two waves' output rows per V stage");
    orow = OR;
    const int vi = wave >> 1;
    ob = (vi == 0 ? vbuf(Even{}) : vi == 1 ? vbuf(Odd{})
          : vi == 2 ? vbuf(std::integral_constant<int, 2>{}) : vbuf(std::integral_constant<int, 3>{})) +
         (wave & 1) * 32 * OR;
  } else {
    ob = lds_object<Tag, 8, G::LDS_BYTES>() + wave * G::OBYTES;
  }
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (db * 32 + 8 * g >= D) continue;  // the row-sum block (XB) is not output
      const int d0 = db * 32 + 8 * g + 4 * hi;
      const u32x2_t w = {M::pack2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv),
                         M::pack2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
      *(FA_LDS u32x2_t*)(ob + l32 * orow + d0 * 2) = w;
    }
  constexpr int CPR = D / 8;  // 16-byte pieces per row
#pragma unroll
  for (int c0 = 0; c0 < 32 * CPR; c0 += 64) {
    const int c = c0 + lane;
    const int row = c / CPR, col = c - (c / CPR) * CPR;
    if (32 * CPR % 64 == 0 || c < 32 * CPR) {
      const u32x4_t w = *(FA_LDS u32x4_t*)(ob + row * orow + col * 16);
      const uint32_t off = (row < wave_rows && col * 8 < a.head_dim)
                               ? (uint32_t)(row * (int32_t)a.o_ss * 2 + col * 16) : kOutOfRange;
      __builtin_amdgcn_raw_buffer_store_b128(w, ro, off, 0, 0);
    }
  }
  if (hi == 0 && a.lse != nullptr && my_q < a.seq_q)
    a.lse[(int64_t)bh * a.seq_q + my_q] = (m_run + __log2f(l_tot)) * kLn2;
}

// ---------------------------------------------------------------------------
// fp32 inputs: same schedule with v_mfma_f32_32x32x2f32; scores, P and the
// accumulator stay fp32 end to end.  D = head_dim rounded up to 32.
// ---------------------------------------------------------------------------
template <int D>
struct Tile32 {
  static constexpr int NW = 4;
  static constexpr int BM = 32 * NW;
  static constexpr int BN = 64;
  static constexpr int NT = 64 * NW;
  static constexpr int KSTEPS = D / 2;
  static constexpr int DBLK = D / 32;
  static constexpr int KROW = D + 1;  // floats; odd stride spreads rows over banks
  static constexpr int VROW = D;      // floats; lanes read consecutive columns
  static constexpr int STAGE = BN * (KROW + VROW);  // floats
  static constexpr int LDS_BYTES = STAGE * 4;  // single stage: fp32 is a small-problem path
  static_assert(D % 32 == 0 && D <= 256, "head_dim padding");
};

template <int D>
__global__ __launch_bounds__(256) void fa_fwd_f32(FwdArgs a) {
  using G = Tile32<D>;
  constexpr int BN = G::BN, NT = G::NT, KSTEPS = G::KSTEPS, DBLK = G::DBLK;
  constexpr int KROW = G::KROW, VROW = G::VROW;

  __shared__ __attribute__((aligned(16))) float smem[G::LDS_BYTES / 4];
  FA_LDS float* lds = (FA_LDS float*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bh, qt, split;
  map_workgroup(a, blockIdx.x, bh, qt, split);
  const int b = bh / a.heads, h = bh - b * a.heads;
  const float* qg = (const float*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
  const float* kg = (const float*)a.k + (int64_t)b * a.k_sb + (int64_t)h * a.k_sh;
  const float* vg = (const float*)a.v + (int64_t)b * a.v_sb + (int64_t)h * a.v_sh;
  float* og = (float*)a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh;

  const int q0 = qt * G::BM;
  const int qw = q0 + wave * 32;
  const int my_q = qw + l32;
  const int wave_last = min(qw + 31, a.seq_q - 1);
  const bool wave_live = qw < a.seq_q;
  const int kv_end = a.causal ? min(a.seq_k, min(a.seq_q, q0 + G::BM)) : a.seq_k;
  const int n_tiles = (kv_end + BN - 1) / BN;

  float qf[KSTEPS];
  const float qsign = a.neg_scale ? -1.f : 1.f;
#pragma unroll
  for (int st = 0; st < KSTEPS; ++st) {
    const int col = 2 * st + hi;
    qf[st] = (my_q < a.seq_q && col < a.head_dim) ? qsign * qg[(int64_t)my_q * a.q_ss + col] : 0.f;
  }

  auto fill_tile = [&](int t, int stage) {
    FA_LDS float* kb = lds + stage * G::STAGE;
    FA_LDS float* vb = kb + BN * KROW;
    const int key0 = t * BN;
    for (int e = tid; e < BN * D; e += NT) {
      const int row = e / D, col = e - (e / D) * D;
      const bool ok = key0 + row < a.seq_k && col < a.head_dim;
      kb[row * KROW + col] = ok ? kg[(int64_t)(key0 + row) * a.k_ss + col] : 0.f;
      vb[row * VROW + col] = ok ? vg[(int64_t)(key0 + row) * a.v_ss + col] : 0.f;
    }
  };

  f32x16_t acc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) acc[db] = (f32x16_t){};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.c;

  for (int t = 0; t < n_tiles; ++t) {
    __syncthreads();  // previous tile fully consumed
    fill_tile(t, 0);
    __syncthreads();
    const int key0 = t * BN;
    if (!wave_live || (a.causal && key0 > wave_last)) continue;
    FA_LDS float* kb = lds;
    FA_LDS float* vb = kb + BN * KROW;

    f32x16_t s[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      f32x16_t sc = (f32x16_t){};
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st)
        sc = __builtin_amdgcn_mfma_f32_32x32x2f32(kb[(kb2 * 32 + l32) * KROW + 2 * st + hi],
                                                  qf[st], sc, 0, 0, 0);
      s[kb2] = sc;
    }
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + kb2 * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        const bool vis = key < a.seq_k && (!a.causal || key <= my_q);
        s[kb2][r] = vis ? s[kb2][r] : -INFINITY;
      }
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c);
    const bool upd = m_new > m_run + kRescaleLog2;
    if (__ballot(upd)) {
      const float alpha = upd ? fast_exp2(m_run - m_new) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) acc[db] *= alpha;
      m_run = upd ? m_new : m_run;
    }
    const float msub = (m_run == -INFINITY) ? 0.f : m_run;
    float lsum = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[kb2][r] = fast_exp2(__builtin_fmaf(s[kb2][r], c, -msub));
        lsum += s[kb2][r];
      }
    l_run += lsum;
    // O^T += V^T P^T, one MFMA per result register r: k index = lane half
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb2 * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vb[key * VROW + db * 32 + l32], s[kb2][r],
                                                         acc[db], 0, 0, 0);
      }
  }

  if (!wave_live) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (my_q < a.seq_q) {
    const float inv = 1.0f / l_tot;
    float* orow = og + (int64_t)my_q * a.o_ss;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = db * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (d < a.head_dim) orow[d] = acc[db][r] * inv;
      }
    if (hi == 0 && a.lse != nullptr)
      a.lse[(int64_t)bh * a.seq_q + my_q] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Merge of the key-split partials:  lse = log sum_r exp(lse_r),
// O = sum_r exp(lse_r - lse) O_r  (the lse-weighted combination that also
// merges two online-softmax states), rounded once into the output type.
// 8 lanes per row, each covering dims 8*sub + 64*c .. +7.
// ---------------------------------------------------------------------------
constexpr int kMaxSplits = 16;

// SMAX: a compile-time bound on the split count (2, 4, 8 or 16), so every
// partial of a row is loaded with straight-line, independent loads.
template <typename T, int SMAX>
__global__ __launch_bounds__(256) void fa_fwd_combine(FwdArgs a) {
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * 32 + (tid >> 3);
  const int sub = tid & 7;
  const int64_t rows = (int64_t)a.n_bh * a.seq_q;
  if (row >= rows) return;
  const int S = a.n_splits;
  // all partial lse values at once (independent loads in flight together)
  float l[SMAX];
#pragma unroll
  for (int r = 0; r < SMAX; ++r)
    l[r] = r < S ? a.part_lse[(int64_t)r * rows + row] : -INFINITY;
  float m = l[0];
#pragma unroll
  for (int r = 1; r < SMAX; ++r) m = fmaxf(m, l[r]);
  float den = 0.f;
#pragma unroll
  for (int r = 0; r < SMAX; ++r) {
    l[r] = __expf(l[r] - m);  // weight before normalisation (0 for absent splits)
    den += l[r];
  }
  const float inv = 1.0f / den;
  const float lse = m + __logf(den);
  const int bh = (int)(row / a.seq_q), i = (int)(row - (int64_t)bh * a.seq_q);
  const int b = bh / a.heads, h = bh - b * a.heads;
  T* orow = (T*)a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)i * a.o_ss;
  typedef T t8 __attribute__((ext_vector_type(8)));
  typedef float f8 __attribute__((ext_vector_type(8)));
  for (int d0 = sub * 8; d0 < a.head_dim; d0 += 64) {
    f8 part[SMAX];
#pragma unroll
    for (int r = 0; r < SMAX; ++r)
      part[r] = r < S ? *(const f8*)(a.part_o + ((int64_t)r * rows + row) * a.head_dim + d0)
                      : (f8){};
    f8 acc = {};
#pragma unroll
    for (int r = 0; r < SMAX; ++r) acc += (l[r] * inv) * part[r];
    t8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (T)acc[e];
    *(t8*)(orow + d0) = out;
  }
  if (sub == 0 && a.lse != nullptr) a.lse[row] = lse;
}

}  // namespace fa
