// Test-only probe: runs single MFMA instructions on caller-provided per-lane
// register contents so a test can compare them with a CPU model of the gfx950
// operand and result layouts (which lane holds which row, column and k index).
// The attention kernels rely on exactly these layouts: operand rows/columns in
// lane % 16, the k index split by lane / 16 (identically for A and B), and
// result rows 4 * (lane / 16) + r in register r.
//
// Every entry point launches one wave64 (one workgroup of 64 threads) that reads
// 64 lanes' worth of operands and writes 64 lanes' worth of results; buffers are
// device pointers sized exactly as documented below.

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

namespace {

__global__ __launch_bounds__(64) void probe_bf16(const bf16x8* a, const bf16x8* b, f32x4* d) {
  const int t = threadIdx.x;
  d[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t], b[t], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}

__global__ __launch_bounds__(64) void probe_i8(const i32x4* a, const i32x4* b, i32x4* d) {
  const int t = threadIdx.x;
  d[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], b[t], i32x4{0, 0, 0, 0}, 0, 0, 0);
}

}  // namespace

extern "C" {

// a, b: bf16 [64 lanes][8]; d: float32 [64 lanes][4]. Returns 0 or a hipError_t.
int gqa_probe_mfma_f32_16x16x32_bf16(const void* a, const void* b, void* d, void* stream) {
  if (!a || !b || !d) return -1;
  hipLaunchKernelGGL(probe_bf16, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     static_cast<const bf16x8*>(a), static_cast<const bf16x8*>(b),
                     static_cast<f32x4*>(d));
  return (int)hipGetLastError();
}

// a, b: int8 [64 lanes][16]; d: int32 [64 lanes][4]. Returns 0 or a hipError_t.
int gqa_probe_mfma_i32_16x16x64_i8(const void* a, const void* b, void* d, void* stream) {
  if (!a || !b || !d) return -1;
  hipLaunchKernelGGL(probe_i8, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     static_cast<const i32x4*>(a), static_cast<const i32x4*>(b),
                     static_cast<i32x4*>(d));
  return (int)hipGetLastError();
}

}  // extern "C"
