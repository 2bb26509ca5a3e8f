// fa_api.hip -- host side of libfa_mi355x.so: argument validation, kernel
// selection and launch for the C ABI declared in include/fa.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <mutex>
#include <string>

#include "../../include/fa.h"
#include "fa_fwd_kernels.hpp"
#include "fa_fwd_ks2.hpp"
#include "fa_fwd_wide.hpp"
#include "fa_bwd_kernels.hpp"
#include "fa_fp8_kernels.hpp"

// Split partials of fa_fwd_splitk_static, for callers that cannot allocate:
// a fixed device array per GPU (each GPU the library runs on holds its own
// copy for the life of the process).  Host code never uses this name as an
// address: the device address comes from hipGetSymbolAddress, per device.
constexpr size_t kStaticScratchBytes = FA_SPLITK_STATIC_MAX_BYTES;
__device__ __attribute__((aligned(256))) char scratch[kStaticScratchBytes];

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

// One dispatch covers at most 2^32 - 1 work-items (the packet's grid size
// is a 32-bit count of work-items, not of workgroups).
constexpr int64_t kMaxWorkItems = 0xFFFFFFFFll;

fa_status_t check_dispatch(int64_t grid, int threads) {
  if (grid > kInt32Max || grid * threads > kMaxWorkItems)
    return fail(FA_ERR_SHAPE, "a launch of %lld workgroups x %d threads exceeds the 2^32 work-items of one dispatch",
                (long long)grid, threads);
  return FA_OK;
}

template <typename Kernel>
fa_status_t launch(Kernel kernel, int64_t grid, int threads, const fa::FwdArgs& args, void* stream) {
  if (fa_status_t s = check_dispatch(grid, threads)) return s;
  fa::FwdArgs a = args;
  void* params[] = {&a};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)grid),
                                 dim3((unsigned)threads), params, 0, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

// Instantiated head-dim paddings: the smallest one >= head_dim is used.
template <typename T, int D, int NW, int OCC, bool XB = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void fa_fwd_16bit(fa::FwdArgs a) {
  // 8-wave workgroups at head_dim 64 and 128 load two tiles ahead (measured
  // 3% faster there; slower at 32 and with the row-sum column at 80 and 96)
  fa::fa_fwd_16bit_body<T, D, NW, XB, NW == 8 && (D == 64 || D == 128)>(a);
}

// small grids: 8 waves over 128 query rows, the key tiles split between two
// groups of 4 waves that merge their states at the end
template <typename T, int D, bool XB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_ks2(fa::FwdArgs a) {
  fa::fa_fwd_ks2_body<T, D, XB>(a);
}

// head_dim 129..256 in one pass: 4 waves of 32 query rows, one per SIMD, Q
// and the O^T accumulator in AGPRs
template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_fwd_wide(fa::FwdArgs a) {
  fa::fa_fwd_wide_body<T, D, 4>(a);
}


// Workgroups of 8 waves (256 query rows) halve the K/V traffic per query and
// run two waves per SIMD from one workgroup; 4-wave workgroups (128 rows) are
// used when the 8-wave grid would be too small to fill the 256 CUs well.
template <typename T, int NW>
fa_status_t launch_16bit_nw(fa::FwdArgs& a, int64_t head_dim, void* stream) {
  constexpr int OCC = 2;  // waves per SIMD the register budget is sized for
  a.n_qtiles = (int32_t)((a.seq_q + 32 * NW - 1) / (32 * NW));
  const int64_t grid = (int64_t)a.n_bh * a.n_qtiles * a.n_splits;
  if (grid > kInt32Max) return fail(FA_ERR_SHAPE, "grid of %lld workgroups is too large", (long long)grid);
  a.xcd_remap = (a.n_bh % 8 == 0) ? 1 : 0;
#define FA_CASE(DP)                                                            \
  if (head_dim <= DP) return launch(fa_fwd_16bit<T, DP, NW, OCC>, grid, 64 * NW, a, stream);
  FA_CASE(32)
  // head_dim 33..64 in 4-wave workgroups (small grids): P.V over 96 dims so
  // that dim 64 carries the row sum (the VALU-bound shape trades 4 MFMAs per
  // tile for 16 dot products; in 8-wave workgroups it does not pay)
  if (head_dim <= 64) {
    if constexpr (NW == 4) return launch(fa_fwd_16bit<T, 64, NW, OCC, true>, grid, 64 * NW, a, stream);
    else return launch(fa_fwd_16bit<T, 64, NW, OCC>, grid, 64 * NW, a, stream);
  }
  FA_CASE(80) FA_CASE(96) FA_CASE(128)
#undef FA_CASE
  // head_dim > 128: the wide kernel, 4-wave workgroups (128 query rows)
  fa::FwdArgs a4 = a;
  a4.n_qtiles = (int32_t)((a.seq_q + 127) / 128);
  const int64_t grid4 = (int64_t)a.n_bh * a4.n_qtiles * a.n_splits;
  if (grid4 > kInt32Max) return fail(FA_ERR_SHAPE, "grid of %lld workgroups is too large", (long long)grid4);
  if (head_dim <= 160) return launch(fa_fwd_wide<T, 160>, grid4, 256, a4, stream);
  if (head_dim <= 192) return launch(fa_fwd_wide<T, 192>, grid4, 256, a4, stream);
  if (head_dim <= 256) return launch(fa_fwd_wide<T, 256>, grid4, 256, a4, stream);
  return fail(FA_ERR_HEAD_DIM, "head_dim %lld unsupported", (long long)head_dim);
}

// Waves per workgroup of the 16-bit forward (8 when the grid stays large).
int waves_16bit(int64_t n_bh, int64_t seq_q, int64_t head_dim) {
  if (head_dim > 128) return 4;
  return n_bh * ((seq_q + 255) / 256) >= 1024 ? 8 : 4;
}

// Grids of at most 256 query tiles of 128 rows (one 8-wave workgroup per
// CU), without key splitting across workgroups: the in-workgroup key split
// (two key groups over 128 query rows) halves each workgroup's chain of key
// tiles.  Larger grids keep 4-wave workgroups, two per CU: there the split
// costs a second round of workgroups (bf16 [4, 12, 2048] causal, head_dim
// 64, 768 tiles: 22% slower).
template <typename T>
fa_status_t launch_ks2(fa::FwdArgs& a, int64_t head_dim, void* stream) {
  a.n_qtiles = (int32_t)((a.seq_q + 127) / 128);
  const int64_t grid = (int64_t)a.n_bh * a.n_qtiles;
  a.xcd_remap = (a.n_bh % 8 == 0) ? 1 : 0;
  if (head_dim <= 32) return launch(fa_fwd_ks2<T, 32, false>, grid, 512, a, stream);
  if (head_dim <= 64) return launch(fa_fwd_ks2<T, 64, true>, grid, 512, a, stream);
  if (head_dim <= 80) return launch(fa_fwd_ks2<T, 80, false>, grid, 512, a, stream);
  if (head_dim <= 96) return launch(fa_fwd_ks2<T, 96, false>, grid, 512, a, stream);
  return launch(fa_fwd_ks2<T, 128, false>, grid, 512, a, stream);
}

template <typename T>
fa_status_t launch_16bit(fa::FwdArgs& a, int64_t head_dim, void* stream) {
  if (waves_16bit(a.n_bh, a.seq_q, head_dim) == 8) return launch_16bit_nw<T, 8>(a, head_dim, stream);
  if (a.n_splits == 1 && head_dim <= 128 && a.seq_k > 64 &&
      (int64_t)a.n_bh * ((a.seq_q + 127) / 128) <= 256)
    return launch_ks2<T>(a, head_dim, stream);
  return launch_16bit_nw<T, 4>(a, head_dim, stream);
}

// Key splitting: about one workgroup per CU, each split keeping at least
// eight 64-key tiles (a workgroup's prologue and epilogue cost several
// microseconds, so short shares do not pay), at most 16 splits.
int choose_splits(int64_t n_bh, int64_t seq_q, int64_t seq_k, int64_t head_dim, int causal) {
  const int64_t rows = 32 * waves_16bit(n_bh, seq_q, head_dim);
  const int64_t grid = n_bh * ((seq_q + rows - 1) / rows);
  if (grid <= 0 || grid >= 256) return 1;
  const int64_t keys = causal ? std::min(seq_k, seq_q) : seq_k;  // longest key range of a tile
  const int64_t tiles = (keys + 63) / 64;
  int64_t s = (256 + grid - 1) / grid;
  s = std::min<int64_t>(s, std::max<int64_t>(1, tiles / 8));
  // two splits are what the unsplit small-grid kernel does inside each
  // workgroup (two key groups, merged in LDS), without the partials and the
  // second launch: fp16, 16 heads, 1000 queries x 1537 keys, head_dim 64,
  // runs in 21 us unsplit against 25.6 us with two splits
  if (s == 2 && head_dim <= 128) s = 1;
  return (int)std::min<int64_t>(s, 16);
}

size_t splitk_workspace_bytes(int64_t n_bh, int64_t seq_q, int64_t head_dim, int splits) {
  if (splits <= 1) return 0;
  return (size_t)splits * (size_t)n_bh * (size_t)seq_q * (size_t)(head_dim + 1) * sizeof(float);
}

template <typename T>
fa_status_t launch_combine(const fa::FwdArgs& a, void* stream) {
  const int64_t rows = (int64_t)a.n_bh * a.seq_q;
  if (fa_status_t s = check_dispatch((rows + 31) / 32, 256)) return s;
  fa::FwdArgs c = a;
  void* params[] = {&c};
  const void* kernel = a.n_splits <= 2   ? reinterpret_cast<const void*>(fa::fa_fwd_combine<T, 2>)
                       : a.n_splits <= 4 ? reinterpret_cast<const void*>(fa::fa_fwd_combine<T, 4>)
                       : a.n_splits <= 8 ? reinterpret_cast<const void*>(fa::fa_fwd_combine<T, 8>)
                                         : reinterpret_cast<const void*>(fa::fa_fwd_combine<T, 16>);
  hipError_t e = hipLaunchKernel(kernel,
                                 dim3((unsigned)((rows + 31) / 32)), dim3(256), params, 0,
                                 (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_e5m2(fa::FwdArgs a) {
  fa::fa_fwd_e5m2_body<D, NW>(a);
}

// head_dim 129..256: one wave per SIMD (the O^T accumulator alone takes 128 VGPRs)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_fwd_e5m2_d256(fa::FwdArgs a) {
  fa::fa_fwd_e5m2_body<256, 4>(a);
}

template <int NW>
fa_status_t launch_e5m2_nw(fa::FwdArgs& a, int64_t head_dim, void* stream) {
  a.n_qtiles = (int32_t)((a.seq_q + 32 * NW - 1) / (32 * NW));
  const int64_t grid = (int64_t)a.n_bh * a.n_qtiles;
  if (grid > kInt32Max) return fail(FA_ERR_SHAPE, "grid of %lld workgroups is too large", (long long)grid);
  a.xcd_remap = (a.n_bh % 8 == 0) ? 1 : 0;
  if (head_dim <= 64) return launch(fa_fwd_e5m2<64, NW>, grid, 64 * NW, a, stream);
  return launch(fa_fwd_e5m2<128, NW>, grid, 64 * NW, a, stream);
}

fa_status_t launch_e5m2(fa::FwdArgs& a, int64_t head_dim, void* stream) {
  if (head_dim > 128) {
    a.n_qtiles = (int32_t)((a.seq_q + 127) / 128);
    const int64_t grid = (int64_t)a.n_bh * a.n_qtiles;
    if (grid > kInt32Max) return fail(FA_ERR_SHAPE, "grid of %lld workgroups is too large", (long long)grid);
    a.xcd_remap = (a.n_bh % 8 == 0) ? 1 : 0;
    return launch(fa_fwd_e5m2_d256, grid, 256, a, stream);
  }
  if (waves_16bit(a.n_bh, a.seq_q, head_dim) == 8) return launch_e5m2_nw<8>(a, head_dim, stream);
  return launch_e5m2_nw<4>(a, head_dim, stream);
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

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq(fa::BwdArgs a) {
  fa::fa_bwd_dq_body<T, D, 4>(a);
}

template <typename T, int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkv(fa::BwdArgs a) {
  fa::fa_bwd_dkv_body<T, D, 8>(a);
}

// head_dim 129..256: one wave per SIMD (the dK/dV accumulators alone take 256 VGPRs);
// dK/dV workgroups of 4 waves (128 keys), so two tile stages and the V rows fit in LDS
template <typename T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_bwd_dq_d256(fa::BwdArgs a) {
  fa::fa_bwd_dq_body<T, 256, 4>(a);
}

template <typename T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_bwd_dkv_d256(fa::BwdArgs a) {
  fa::fa_bwd_dkv_body<T, 256, 4>(a);
}

// fp32 backward (one wave per SIMD: the fp32 fragments take twice the registers)
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_bwd_dq_f32(fa::BwdArgs a) {
  fa::fa_bwd_dq_f32_body<D>(a);
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_bwd_dkv_f32(fa::BwdArgs a) {
  fa::fa_bwd_dkv_f32_body<D>(a);
}

template <typename Kernel>
fa_status_t launch_bwd(Kernel kernel, int64_t grid, int threads, const fa::BwdArgs& args,
                       void* stream) {
  if (fa_status_t s = check_dispatch(grid, threads)) return s;
  fa::BwdArgs a = args;
  void* params[] = {&a};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)grid),
                                 dim3((unsigned)threads), params, 0, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

// D (delta), then dQ (query blocks of 128, heaviest causal blocks first), then
// dK/dV (key blocks of 256), all on `stream`.
template <typename T, int DP>
fa_status_t launch_bwd_dp(fa::BwdArgs a, void* stream) {
  fa_status_t s;
  const int64_t rows = (int64_t)a.n_bh * a.seq_q;
  if (rows > 0) {
    if ((s = launch_bwd(fa::fa_bwd_delta<T>, (rows + 31) / 32, 256, a, stream)) != FA_OK) return s;
    a.n_tiles = (int32_t)((a.seq_q + 127) / 128);
    if ((s = launch_bwd(fa_bwd_dq<T, DP>, (int64_t)a.n_bh * a.n_tiles, 256, a, stream)) != FA_OK)
      return s;
  }
  a.n_tiles = (int32_t)((a.seq_k + 255) / 256);
  return launch_bwd(fa_bwd_dkv<T, DP>, (int64_t)a.n_bh * a.n_tiles, 512, a, stream);
}

// fp32: D, then dQ (query blocks of 128), then dK/dV (key blocks of 128)
template <int D>
fa_status_t launch_bwd_f32_d(fa::BwdArgs a, void* stream) {
  fa_status_t s;
  const int64_t rows = (int64_t)a.n_bh * a.seq_q;
  if (rows > 0) {
    if ((s = launch_bwd(fa::fa_bwd_delta<float>, (rows + 31) / 32, 256, a, stream)) != FA_OK) return s;
    a.n_tiles = (int32_t)((a.seq_q + 127) / 128);
    if ((s = launch_bwd(fa_bwd_dq_f32<D>, (int64_t)a.n_bh * a.n_tiles, 256, a, stream)) != FA_OK)
      return s;
  }
  a.n_tiles = (int32_t)((a.seq_k + 127) / 128);
  return launch_bwd(fa_bwd_dkv_f32<D>, (int64_t)a.n_bh * a.n_tiles, 256, a, stream);
}

fa_status_t launch_bwd_f32(const fa::BwdArgs& a, int64_t head_dim, void* stream) {
  if (head_dim <= 32) return launch_bwd_f32_d<32>(a, stream);
  if (head_dim <= 64) return launch_bwd_f32_d<64>(a, stream);
  if (head_dim <= 96) return launch_bwd_f32_d<96>(a, stream);
  return launch_bwd_f32_d<128>(a, stream);
}

template <typename T>
fa_status_t launch_bwd_16bit_d256(fa::BwdArgs a, void* stream) {
  fa_status_t s;
  const int64_t rows = (int64_t)a.n_bh * a.seq_q;
  if (rows > 0) {
    if ((s = launch_bwd(fa::fa_bwd_delta<T>, (rows + 31) / 32, 256, a, stream)) != FA_OK) return s;
    a.n_tiles = (int32_t)((a.seq_q + 127) / 128);
    if ((s = launch_bwd(fa_bwd_dq_d256<T>, (int64_t)a.n_bh * a.n_tiles, 256, a, stream)) != FA_OK)
      return s;
  }
  a.n_tiles = (int32_t)((a.seq_k + 127) / 128);
  return launch_bwd(fa_bwd_dkv_d256<T>, (int64_t)a.n_bh * a.n_tiles, 256, a, stream);
}

template <typename T>
fa_status_t launch_bwd_16bit(const fa::BwdArgs& a, int64_t head_dim, void* stream) {
  if (head_dim > 128) return launch_bwd_16bit_d256<T>(a, stream);
  if (head_dim <= 32) return launch_bwd_dp<T, 32>(a, stream);
  if (head_dim <= 64) return launch_bwd_dp<T, 64>(a, stream);
  if (head_dim <= 80) return launch_bwd_dp<T, 80>(a, stream);
  if (head_dim <= 96) return launch_bwd_dp<T, 96>(a, stream);
  return launch_bwd_dp<T, 128>(a, stream);
}



// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

fa_status_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FA_ERR_HIP, "device %d beyond the %d devices the static scratch serves", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(FA_ERR_HIP, "hipGetSymbolAddress of the static scratch failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

// Shared by fa_fwd (splits == 1, no workspace), fa_fwd_splitk and
// fa_fwd_splitk_static (use_static: the partials go to `scratch`).
fa_status_t fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k, int64_t head_dim,
                     fa_strides_t q_st, fa_strides_t k_st, fa_strides_t v_st, fa_strides_t o_st,
                     float sm_scale, int causal, fa_dtype_t dtype, int splits, void* workspace,
                     size_t workspace_bytes, bool split_api, void* stream, bool use_static = false) {
  if (batch < 0 || heads < 0 || seq_q < 0)
    return fail(FA_ERR_SHAPE, "batch, heads and seq_q must be >= 0");
  if (seq_k < 1) return fail(FA_ERR_SHAPE, "seq_k must be >= 1 (softmax over no keys)");
  if (seq_q > kInt32Max - 256 || seq_k > kInt32Max - 256 || batch > kInt32Max || heads > kInt32Max ||
      batch * heads > kInt32Max || batch * heads * seq_q > INT64_MAX / 2)
    return fail(FA_ERR_SHAPE, "a size exceeds the 32-bit index range");
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16 &&
      dtype != FA_DTYPE_E5M2)
    return fail(FA_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  const bool f32 = dtype == FA_DTYPE_F32;
  const bool e5m2 = dtype == FA_DTYPE_E5M2;
  if (split_api) {
    if (splits < 0 || splits > fa::kMaxSplits)
      return fail(FA_ERR_WORKSPACE, "num_splits %d outside 0..%d", splits, fa::kMaxSplits);
    if (splits == 0)
      splits = (f32 || e5m2) ? 1 : choose_splits(batch * heads, seq_q, seq_k, head_dim, causal);
    if ((f32 || e5m2) && splits > 1)
      return fail(FA_ERR_DTYPE, "key splitting needs bf16 or fp16 inputs");
  }
  const int64_t hd_mult = f32 ? 4 : e5m2 ? 16 : 8;
  const int64_t hd_max = 256;
  if (head_dim < 1 || head_dim > hd_max || head_dim % hd_mult != 0)
    return fail(FA_ERR_HEAD_DIM, "head_dim %lld must be in 1..%lld and a multiple of %lld",
                (long long)head_dim, (long long)hd_max, (long long)hd_mult);
  const int64_t mult = f32 ? 1 : e5m2 ? 16 : 8;  // 16-byte rows
  fa_status_t s;
  if ((s = check_strides("q", q_st, mult)) != FA_OK) return s;
  if ((s = check_strides("k", k_st, mult)) != FA_OK) return s;
  if (e5m2) {
    // V key-major: seq stride 1, one row of >= seq_k keys per dim
    if (v_st.seq != 1) return fail(FA_ERR_LAYOUT, "v: e5m2 takes V key-major (seq stride 1)");
    if (v_st.dim < seq_k || v_st.dim % 16 != 0 || v_st.dim >= kMaxSeqStride)
      return fail(FA_ERR_LAYOUT, "v: dim stride %lld must be a multiple of 16, >= seq_k and < 2^24",
                  (long long)v_st.dim);
    // a V tile is addressed by 32-bit byte offsets spanning head_dim key rows
    if ((head_dim - 1) * v_st.dim + 64 > kInt32Max)
      return fail(FA_ERR_LAYOUT, "v: (head_dim - 1) * dim stride exceeds the 32-bit tile range");
    if (v_st.batch < 0 || v_st.head < 0 || v_st.batch % 16 != 0 || v_st.head % 16 != 0)
      return fail(FA_ERR_LAYOUT, "v: batch/head strides must be non-negative multiples of 16");
  } else if ((s = check_strides("v", v_st, mult)) != FA_OK) {
    return s;
  }
  if ((s = check_strides("o", o_st, mult)) != FA_OK) return s;
  if (!std::isfinite(sm_scale)) return fail(FA_ERR_SCALE, "sm_scale must be finite");
  // an empty problem touches no memory, so its pointers may be NULL
  if (batch == 0 || heads == 0 || seq_q == 0) return FA_OK;
  if (!q || !k || !v || !o) return fail(FA_ERR_NULL, "q, k, v and o must be non-NULL");
  const uintptr_t align = f32 ? 4 : 16;
  if (!aligned(q, align) || !aligned(k, align) || !aligned(v, align) || !aligned(o, align))
    return fail(FA_ERR_LAYOUT, "q, k, v and o must be %d-byte aligned", (int)align);
  if (lse && !aligned(lse, 4)) return fail(FA_ERR_LAYOUT, "lse must be 4-byte aligned");
  const size_t need = splitk_workspace_bytes(batch * heads, seq_q, head_dim, splits);
  if (need > 0 && use_static) {
    if (need > kStaticScratchBytes)
      return fail(FA_ERR_WORKSPACE, "%zu bytes of split partials exceed the %zu-byte static scratch "
                  "(fewer splits or fa_fwd_splitk with a workspace)", need, kStaticScratchBytes);
  } else if (need > 0) {
    if (!workspace) return fail(FA_ERR_WORKSPACE, "a workspace of %zu bytes is needed", need);
    if (!aligned(workspace, 256)) return fail(FA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu needed", workspace_bytes, need);
  }

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
  a.n_splits = splits;
  a.v_sd = v_st.dim;
  if (splits > 1 && !use_static) {
    a.part_o = (float*)workspace;
    a.part_lse = a.part_o + (size_t)splits * (size_t)(batch * heads) * (size_t)seq_q * (size_t)head_dim;
  }
  // the merge runs after the split shares: bound its dispatch before any launch
  if (splits > 1) {
    if (fa_status_t s2 = check_dispatch((batch * heads * seq_q + 31) / 32, 256)) return s2;
  }
  if (need > 0 && use_static) {
    if (fa_status_t s2 = static_scratch(&workspace)) return s2;
    a.part_o = (float*)workspace;
    a.part_lse = a.part_o + (size_t)splits * (size_t)(batch * heads) * (size_t)seq_q * (size_t)head_dim;
  }
  fa_status_t st;
  switch (dtype) {
    case FA_DTYPE_BF16:
      st = launch_16bit<__bf16>(a, head_dim, stream);
      if (st == FA_OK && splits > 1) st = launch_combine<__bf16>(a, stream);
      return st;
    case FA_DTYPE_F16:
      st = launch_16bit<_Float16>(a, head_dim, stream);
      if (st == FA_OK && splits > 1) st = launch_combine<_Float16>(a, stream);
      return st;
    case FA_DTYPE_E5M2: return launch_e5m2(a, head_dim, stream);
    default: return launch_f32(a, head_dim, stream);
  }
}

}  // namespace

extern "C" {

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k, int64_t head_dim,
                   fa_strides_t q_st, fa_strides_t k_st, fa_strides_t v_st, fa_strides_t o_st,
                   float sm_scale, int causal, fa_dtype_t dtype, void* stream) {
  g_last_error.clear();
  return fwd_impl(q, k, v, o, lse, batch, heads, seq_q, seq_k, head_dim, q_st, k_st, v_st, o_st,
                  sm_scale, causal, dtype, 1, nullptr, 0, false, stream);
}

int fa_fwd_splitk_choose(int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k,
                         int64_t head_dim, int causal) {
  if (batch <= 0 || heads <= 0 || seq_q <= 0 || seq_k <= 0 || head_dim <= 0) return 1;
  return choose_splits(batch * heads, seq_q, seq_k, head_dim, causal);
}

size_t fa_fwd_splitk_workspace(int64_t batch, int64_t heads, int64_t seq_q, int64_t head_dim,
                               int num_splits) {
  if (batch <= 0 || heads <= 0 || seq_q <= 0 || head_dim <= 0) return 0;
  return splitk_workspace_bytes(batch * heads, seq_q, head_dim, num_splits);
}

fa_status_t fa_fwd_splitk(const void* q, const void* k, const void* v, void* o, float* lse,
                          int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k,
                          int64_t head_dim, fa_strides_t q_st, fa_strides_t k_st,
                          fa_strides_t v_st, fa_strides_t o_st, float sm_scale, int causal,
                          fa_dtype_t dtype, int num_splits, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return fwd_impl(q, k, v, o, lse, batch, heads, seq_q, seq_k, head_dim, q_st, k_st, v_st, o_st,
                  sm_scale, causal, dtype, num_splits, workspace, workspace_bytes, true, stream);
}

fa_status_t fa_fwd_splitk_static(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k,
                                 int64_t head_dim, fa_strides_t q_st, fa_strides_t k_st,
                                 fa_strides_t v_st, fa_strides_t o_st, float sm_scale, int causal,
                                 fa_dtype_t dtype, int num_splits, void* stream) {
  g_last_error.clear();
  return fwd_impl(q, k, v, o, lse, batch, heads, seq_q, seq_k, head_dim, q_st, k_st, v_st, o_st,
                  sm_scale, causal, dtype, num_splits, nullptr, 0, true, stream, true);
}

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, float* delta, void* dq, void* dk, void* dv,
                   int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k, int64_t head_dim,
                   fa_strides_t q_st, fa_strides_t k_st, fa_strides_t v_st, fa_strides_t o_st,
                   fa_strides_t do_st, fa_strides_t dq_st, fa_strides_t dk_st, fa_strides_t dv_st,
                   float sm_scale, int causal, fa_dtype_t dtype, void* stream) {
  g_last_error.clear();
  if (batch < 0 || heads < 0 || seq_q < 0)
    return fail(FA_ERR_SHAPE, "batch, heads and seq_q must be >= 0");
  if (seq_k < 1) return fail(FA_ERR_SHAPE, "seq_k must be >= 1 (softmax over no keys)");
  if (seq_q > kInt32Max - 256 || seq_k > kInt32Max - 256 || batch > kInt32Max || heads > kInt32Max ||
      batch * heads > kInt32Max || batch * heads * seq_q > INT64_MAX / 2)
    return fail(FA_ERR_SHAPE, "a size exceeds the 32-bit index range");
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16 &&
      dtype != FA_DTYPE_E5M2)
    return fail(FA_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  if (dtype == FA_DTYPE_E5M2)
    return fail(FA_ERR_DTYPE, "the backward supports fp32, bf16 and fp16");
  const bool f32 = dtype == FA_DTYPE_F32;
  const int64_t hd_mult = f32 ? 4 : 8;
  const int64_t hd_max = f32 ? 128 : 256;
  if (head_dim < 1 || head_dim > hd_max || head_dim % hd_mult != 0)
    return fail(FA_ERR_HEAD_DIM, "backward: head_dim %lld must be in 1..%lld and a multiple of %lld",
                (long long)head_dim, (long long)hd_max, (long long)hd_mult);
  fa_status_t s;
  const fa_strides_t* sts[8] = {&q_st, &k_st, &v_st, &o_st, &do_st, &dq_st, &dk_st, &dv_st};
  const char* names[8] = {"q", "k", "v", "o", "dout", "dq", "dk", "dv"};
  for (int i = 0; i < 8; ++i)
    if ((s = check_strides(names[i], *sts[i], f32 ? 1 : 8)) != FA_OK) return s;
  if (!std::isfinite(sm_scale)) return fail(FA_ERR_SCALE, "sm_scale must be finite");
  if (batch == 0 || heads == 0) return FA_OK;  // nothing to read or write
  if (!k || !v || !dk || !dv) return fail(FA_ERR_NULL, "k, v, dk and dv must be non-NULL");
  if (seq_q > 0 && (!q || !o || !dout || !lse || !delta || !dq))
    return fail(FA_ERR_NULL, "q, o, dout, lse, delta and dq must be non-NULL");
  const void* ptrs[8] = {q, k, v, o, dout, dq, dk, dv};
  const uintptr_t align = f32 ? 4 : 16;
  for (int i = 0; i < 8; ++i)
    if (ptrs[i] && !aligned(ptrs[i], align))
      return fail(FA_ERR_LAYOUT, "%s must be %d-byte aligned", names[i], (int)align);
  if ((lse && !aligned(lse, 4)) || (delta && !aligned(delta, 4)))
    return fail(FA_ERR_LAYOUT, "lse and delta must be 4-byte aligned");

  // bound all three dispatches before the first is enqueued: delta (8 lanes
  // per query row), dQ (128-query blocks of 256 threads), dK/dV (at most 2
  // threads per key: 256-key blocks of 512 or 128-key blocks of 256)
  {
    const int64_t bh = batch * heads;
    if (seq_q > 0) {
      if (fa_status_t s2 = check_dispatch((bh * seq_q + 31) / 32, 256)) return s2;
      if (fa_status_t s2 = check_dispatch(bh * ((seq_q + 127) / 128), 256)) return s2;
    }
    if (fa_status_t s2 = check_dispatch(bh * ((seq_k + 255) / 256), 512)) return s2;
    if (fa_status_t s2 = check_dispatch(bh * ((seq_k + 127) / 128), 256)) return s2;
  }

  fa::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse; a.delta = delta;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.q_sb = q_st.batch; a.q_sh = q_st.head; a.q_ss = q_st.seq;
  a.k_sb = k_st.batch; a.k_sh = k_st.head; a.k_ss = k_st.seq;
  a.v_sb = v_st.batch; a.v_sh = v_st.head; a.v_ss = v_st.seq;
  a.o_sb = o_st.batch; a.o_sh = o_st.head; a.o_ss = o_st.seq;
  a.do_sb = do_st.batch; a.do_sh = do_st.head; a.do_ss = do_st.seq;
  a.dq_sb = dq_st.batch; a.dq_sh = dq_st.head; a.dq_ss = dq_st.seq;
  a.dk_sb = dk_st.batch; a.dk_sh = dk_st.head; a.dk_ss = dk_st.seq;
  a.dv_sb = dv_st.batch; a.dv_sh = dv_st.head; a.dv_ss = dv_st.seq;
  a.heads = (int32_t)heads;
  a.seq_q = (int32_t)seq_q;
  a.seq_k = (int32_t)seq_k;
  a.head_dim = (int32_t)head_dim;
  a.n_bh = (int32_t)(batch * heads);
  a.scale = sm_scale;
  a.c = std::fmax(std::fabs(sm_scale) * fa::kLog2e, 1e-30f);
  a.neg_scale = sm_scale < 0.f ? 1 : 0;
  a.causal = causal ? 1 : 0;
  a.xcd_remap = (a.n_bh % 8 == 0) ? 1 : 0;
  if (f32) return launch_bwd_f32(a, head_dim, stream);
  if (dtype == FA_DTYPE_BF16) return launch_bwd_16bit<__bf16>(a, head_dim, stream);
  return launch_bwd_16bit<_Float16>(a, head_dim, stream);
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
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
  }
  return "FA_ERR_UNKNOWN";
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

int fa_version(void) { return 300; }

}  // extern "C"
