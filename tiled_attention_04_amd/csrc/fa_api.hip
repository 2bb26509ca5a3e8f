// fa_api.hip -- host side of libfa_mi355x.so: argument validation, kernel
// selection and launch for the C ABI declared in include/fa.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <string>

#include "../../include/fa.h"
#include "fa_fwd_kernels.hpp"

namespace {

thread_local std::string g_last_error;

fa_status_t fail(fa_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

constexpr int64_t kInt32Max = 2147483647;

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Tiles are addressed with 32-bit byte offsets from a per-tile base, so one
// tile's rows must span less than 2 GiB: seq stride < 2^24 elements.
constexpr int64_t kMaxSeqStride = (int64_t)1 << 24;

fa_status_t check_strides(const char* name, const fa_strides_t& st, int64_t mult) {
  if (st.dim != 1) return fail(FA_ERR_LAYOUT, "%s: dim stride must be 1 (got %lld)", name, (long long)st.dim);
  if (st.seq >= kMaxSeqStride)
    return fail(FA_ERR_LAYOUT, "%s: seq stride %lld must be below 2^24 elements", name, (long long)st.seq);
  const int64_t s[3] = {st.batch, st.head, st.seq};
  const char* n[3] = {"batch", "head", "seq"};
  for (int i = 0; i < 3; ++i) {
    if (s[i] < 0) return fail(FA_ERR_LAYOUT, "%s: negative %s stride", name, n[i]);
    if (s[i] % mult != 0)
      return fail(FA_ERR_LAYOUT, "%s: %s stride %lld is not a multiple of %lld elements", name, n[i],
                  (long long)s[i], (long long)mult);
  }
  return FA_OK;
}

template <typename Kernel>
fa_status_t launch(Kernel kernel, int64_t grid, int threads, const fa::FwdArgs& args, void* stream) {
  fa::FwdArgs a = args;
  void* params[] = {&a};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)grid),
                                 dim3((unsigned)threads), params, 0, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

// Instantiated head-dim paddings: the smallest one >= head_dim is used.
#ifndef FA_OCC16
#define FA_OCC16 2  // waves per SIMD the register budget is sized for
#endif

template <typename T, int D, int NW, int OCC>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void fa_fwd_16bit(fa::FwdArgs a) {
  fa::fa_fwd_16bit_body<T, D, NW>(a);
}

// Workgroups of 8 waves (256 query rows) halve the K/V traffic per query and
// run two waves per SIMD from one workgroup; 4-wave workgroups (128 rows) are
// used when the 8-wave grid would be too small to fill the 256 CUs well.
template <typename T, int NW>
fa_status_t launch_16bit_nw(fa::FwdArgs& a, int64_t head_dim, void* stream) {
  constexpr int OCC = FA_OCC16;
  a.n_qtiles = (int32_t)((a.seq_q + 32 * NW - 1) / (32 * NW));
  const int64_t grid = (int64_t)a.n_bh * a.n_qtiles;
  if (grid > kInt32Max) return fail(FA_ERR_SHAPE, "grid of %lld workgroups is too large", (long long)grid);
  a.xcd_remap = (a.n_bh % 8 == 0) ? 1 : 0;
#define FA_CASE(DP)                                                            \
  if (head_dim <= DP) return launch(fa_fwd_16bit<T, DP, NW, OCC>, grid, 64 * NW, a, stream);
  FA_CASE(32) FA_CASE(64) FA_CASE(80) FA_CASE(96) FA_CASE(128)
#undef FA_CASE
  // head_dim > 128 does not fit two waves per SIMD: 4-wave workgroups, one wave per SIMD
#define FA_CASE(DP)                                                            \
  if (head_dim <= DP) return launch(fa_fwd_16bit<T, DP, 4, 1>, grid4, 256, a4, stream);
  fa::FwdArgs a4 = a;
  a4.n_qtiles = (int32_t)((a.seq_q + 127) / 128);
  const int64_t grid4 = (int64_t)a.n_bh * a4.n_qtiles;
  if (grid4 > kInt32Max) return fail(FA_ERR_SHAPE, "grid of %lld workgroups is too large", (long long)grid4);
  FA_CASE(160) FA_CASE(192) FA_CASE(256)
#undef FA_CASE
  return fail(FA_ERR_HEAD_DIM, "head_dim %lld unsupported", (long long)head_dim);
}

template <typename T>
fa_status_t launch_16bit(fa::FwdArgs& a, int64_t head_dim, void* stream) {
#ifdef FA_FORCE_NW16
  return launch_16bit_nw<T, FA_FORCE_NW16>(a, head_dim, stream);
#else
  const int64_t wg8 = (int64_t)a.n_bh * ((a.seq_q + 255) / 256);
  if (wg8 >= 1024) return launch_16bit_nw<T, 8>(a, head_dim, stream);
  return launch_16bit_nw<T, 4>(a, head_dim, stream);
#endif
}

fa_status_t launch_f32(fa::FwdArgs& a, int64_t head_dim, void* stream) {
  a.n_qtiles = (int32_t)((a.seq_q + 127) / 128);
  const int64_t grid = (int64_t)a.n_bh * a.n_qtiles;
  if (grid > kInt32Max) return fail(FA_ERR_SHAPE, "grid of %lld workgroups is too large", (long long)grid);
  a.xcd_remap = (a.n_bh % 8 == 0) ? 1 : 0;
#define FA_CASE(DP) \
  if (head_dim <= DP) return launch(fa::fa_fwd_f32<DP>, grid, 256, a, stream);
  FA_CASE(32) FA_CASE(64) FA_CASE(128) FA_CASE(256)
#undef FA_CASE
  return fail(FA_ERR_HEAD_DIM, "head_dim %lld unsupported", (long long)head_dim);
}

}  // namespace

extern "C" {

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k, int64_t head_dim,
                   fa_strides_t q_st, fa_strides_t k_st, fa_strides_t v_st, fa_strides_t o_st,
                   float sm_scale, int causal, fa_dtype_t dtype, void* stream) {
  g_last_error.clear();
  if (batch < 0 || heads < 0 || seq_q < 0)
    return fail(FA_ERR_SHAPE, "batch, heads and seq_q must be >= 0");
  if (seq_k < 1) return fail(FA_ERR_SHAPE, "seq_k must be >= 1 (softmax over no keys)");
  if (seq_q > kInt32Max - 256 || seq_k > kInt32Max - 256 || batch > kInt32Max || heads > kInt32Max ||
      batch * heads > kInt32Max || batch * heads * seq_q > INT64_MAX / 2)
    return fail(FA_ERR_SHAPE, "a size exceeds the 32-bit index range");
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
    return fail(FA_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  const bool f32 = dtype == FA_DTYPE_F32;
  const int64_t hd_mult = f32 ? 4 : 8;
  if (head_dim < 1 || head_dim > 256 || head_dim % hd_mult != 0)
    return fail(FA_ERR_HEAD_DIM, "head_dim %lld must be in 1..256 and a multiple of %lld",
                (long long)head_dim, (long long)hd_mult);
  const int64_t mult = f32 ? 1 : 8;
  fa_status_t s;
  if ((s = check_strides("q", q_st, mult)) != FA_OK) return s;
  if ((s = check_strides("k", k_st, mult)) != FA_OK) return s;
  if ((s = check_strides("v", v_st, mult)) != FA_OK) return s;
  if ((s = check_strides("o", o_st, mult)) != FA_OK) return s;
  if (!std::isfinite(sm_scale)) return fail(FA_ERR_SCALE, "sm_scale must be finite");
  // an empty problem touches no memory, so its pointers may be NULL
  if (batch == 0 || heads == 0 || seq_q == 0) return FA_OK;
  if (!q || !k || !v || !o) return fail(FA_ERR_NULL, "q, k, v and o must be non-NULL");
  const uintptr_t align = f32 ? 4 : 16;
  if (!aligned(q, align) || !aligned(k, align) || !aligned(v, align) || !aligned(o, align))
    return fail(FA_ERR_LAYOUT, "q, k, v and o must be %d-byte aligned", (int)align);
  if (lse && !aligned(lse, 4)) return fail(FA_ERR_LAYOUT, "lse must be 4-byte aligned");

  fa::FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.q_sb = q_st.batch; a.q_sh = q_st.head; a.q_ss = q_st.seq;
  a.k_sb = k_st.batch; a.k_sh = k_st.head; a.k_ss = k_st.seq;
  a.v_sb = v_st.batch; a.v_sh = v_st.head; a.v_ss = v_st.seq;
  a.o_sb = o_st.batch; a.o_sh = o_st.head; a.o_ss = o_st.seq;
  a.heads = (int32_t)heads;
  a.seq_q = (int32_t)seq_q;
  a.seq_k = (int32_t)seq_k;
  a.head_dim = (int32_t)head_dim;
  a.n_bh = (int32_t)(batch * heads);
  a.c = std::fmax(std::fabs(sm_scale) * fa::kLog2e, 1e-30f);
  a.neg_scale = sm_scale < 0.f ? 1 : 0;
  a.causal = causal ? 1 : 0;
  switch (dtype) {
    case FA_DTYPE_BF16: return launch_16bit<__bf16>(a, head_dim, stream);
    case FA_DTYPE_F16: return launch_16bit<_Float16>(a, head_dim, stream);
    default: return launch_f32(a, head_dim, stream);
  }
}

const char* fa_status_string(fa_status_t s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE";
    case FA_ERR_HEAD_DIM: return "FA_ERR_HEAD_DIM";
    case FA_ERR_LAYOUT: return "FA_ERR_LAYOUT";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    case FA_ERR_SCALE: return "FA_ERR_SCALE";
  }
  return "FA_ERR_UNKNOWN";
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

int fa_version(void) { return 100; }

}  // extern "C"
