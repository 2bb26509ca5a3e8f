// fa_mfma_asm.hpp -- gfx950 MFMAs written as inline assembly, for kernels
// whose accumulators must stay in AGPRs (the register allocator would
// otherwise keep them in VGPRs and copy or spill them), and the helpers that
// go with them: hand-placed wait states, ordering pins, compile-time loops.
#pragma once
#include "fa_fwd_kernels.hpp"

namespace fa {

// MFMAs as inline assembly with fixed register classes.  The compiler does
// not know these are MFMAs, so the wait states the ISA requires between an
// MFMA and a VALU access of its result (and between a VALU write of an
// accumulator and the MFMA that reads it) are inserted by hand with the
// drain statements below, at the few places where such accesses happen.
// Chains that accumulate into the same registers need none (the matrix core
// forwards them).
template <typename T>
struct MfmaPin;

template <>
struct MfmaPin<__bf16> {
  typedef bf16x8_t frag;
  // s = k q (no accumulator input); s must not overlap the sources.  The two
  // wait states keep a VALU write of a register of s just before apart from
  // the MFMA's write of it.
  __device__ static inline void first(f32x16_t& s, const frag& k, const frag& q) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(k), "a"(q));
  }
  __device__ static inline void next(f32x16_t& s, const frag& k, const frag& q) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(k), "a"(q));
  }
  __device__ static inline void acc(f32x16_t& o, const frag& v, const frag& p) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
  }
  // the same after two wait states, for operands a VALU may have written
  // just before
  __device__ static inline void acc_fresh(f32x16_t& o, const frag& v, const frag& p) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
  }
  // VGPR result and operands: d = a b (d must not overlap the sources), d += a b;
  // both after two wait states (the operands may come straight from a VALU)
  __device__ static inline void vfirst(f32x16_t& d, const frag& a, const frag& b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  }
  __device__ static inline void vnext(f32x16_t& d, const frag& a, const frag& b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
  }
};

template <>
struct MfmaPin<_Float16> {
  typedef f16x8_t frag;
  __device__ static inline void first(f32x16_t& s, const frag& k, const frag& q) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(s) : "v"(k), "a"(q));
  }
  __device__ static inline void next(f32x16_t& s, const frag& k, const frag& q) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(s) : "v"(k), "a"(q));
  }
  __device__ static inline void acc(f32x16_t& o, const frag& v, const frag& p) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
  }
  __device__ static inline void acc_fresh(f32x16_t& o, const frag& v, const frag& p) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
  }
  // VGPR result and operands: d = a b (d must not overlap the sources), d += a b;
  // both after two wait states (the operands may come straight from a VALU)
  __device__ static inline void vfirst(f32x16_t& d, const frag& a, const frag& b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  }
  __device__ static inline void vnext(f32x16_t& d, const frag& a, const frag& b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
  }
};

// 24 wait states (more than the 8-pass 32x32 MFMA needs before a VALU access
// of its result), ordered after every producer and before every consumer of
// the registers passed: each operand is "modified" by the statement.
#define FA_DRAIN "s_nop 7\n\ts_nop 7\n\ts_nop 7"
__device__ inline void mfma_drain_v(f32x16_t& a0, f32x16_t& a1) {
  asm volatile(FA_DRAIN : "+v"(a0), "+v"(a1));
}
// (the wait states sit in the first statement; the following empty ones are
// ordered after it, and each orders the accesses of its own block)
template <int DBLK>
__device__ inline void mfma_drain_a(f32x16_t (&x)[DBLK]) {
  asm volatile(FA_DRAIN : "+a"(x[0]));
#pragma unroll
  for (int i = 1; i < DBLK; ++i) asm volatile("" : "+a"(x[i]));
}
// An empty statement that "redefines" x in place: a value computed before it
// cannot sink below it (the instruction order of a slot is kept).
template <typename V>
__device__ inline void pin(V& x) {
  asm volatile("" : "+v"(x));
}
// Moves the Q fragments to AGPRs (the two wait states cover a VALU write of
// a register followed by its move).
template <int N, typename F>
__device__ inline void pin_agpr(F (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("s_nop 1" : "+a"(x[i]));
}

// Compile-time loop: f(integral_constant<int, I>) for I = B..E-1, so every
// index inside is a constant (register arrays stay in registers).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(static_cast<F&&>(f));
  }
}

}  // namespace fa
