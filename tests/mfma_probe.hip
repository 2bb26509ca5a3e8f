// mfma_probe.hip -- TEST INFRASTRUCTURE: runs single float8 e5m2 matrix
// instructions (v_mfma_f32_32x32x64_f8f6f4, the instruction of the e5m2
// attention forward) on operands the test chooses, so the test can check the
// instruction's arithmetic (how its 64 products are grouped, truncated and
// summed) and the error bound G that the e5m2 parity tests rely on.
//
// One wave per instance.  Instance n reads, for every lane l, 32 bytes of A
// at a + (64 n + l) * 32 and 32 bytes of B at b + (64 n + l) * 32 (lane l's
// A register operand: row l % 32 of A, lane half l / 32; B: column l % 32),
// and writes its 16 accumulator floats to d + (64 n + l) * 16 (column l % 32,
// rows 8 (r / 4) + 4 (l / 32) + r % 4 for r = 0..15).  The accumulator input
// is zero.  The caller sizes a and b to n * 2048 bytes and d to n * 4096 bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(64) void e5m2_mfma_probe(const i32x8_t* a, const i32x8_t* b,
                                                      f32x16_t* d) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  const f32x16_t zero = {};
  // format codes 1 = bf8 (e5m2) for both operands, no block scaling
  d[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[i], zero, 1, 1, 0, 0, 0, 0);
}

extern "C" int e5m2_mfma_probe_run(const void* a, const void* b, void* d, int n, void* stream) {
  if (n <= 0 || n > 65535 || !a || !b || !d) return -1;
  hipLaunchKernelGGL(e5m2_mfma_probe, dim3(n), dim3(64), 0, (hipStream_t)stream,
                     (const i32x8_t*)a, (const i32x8_t*)b, (f32x16_t*)d);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
