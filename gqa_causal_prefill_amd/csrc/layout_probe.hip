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
typedef short i16x4 __attribute__((ext_vector_type(4)));

namespace {

__global__ __launch_bounds__(64) void probe_bf16(const bf16x8* a, const bf16x8* b, f32x4* d) {
  const int t = threadIdx.x;
  d[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t], b[t], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}

__global__ __launch_bounds__(64) void probe_i8(const i32x4* a, const i32x4* b, i32x4* d) {
  const int t = threadIdx.x;
  d[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], b[t], i32x4{0, 0, 0, 0}, 0, 0, 0);
}

// ds_read_b64_tr_b16: an 8 KiB LDS image (4096 x 16-bit) is loaded, then each lane
// issues one transposing read at its own byte offset (multiple of 8, < 8192).
__global__ __launch_bounds__(64) void probe_tr16(const short* image, const int* offs, i16x4* out) {
  __shared__ __attribute__((aligned(16))) short lds[4096];
  const int t = threadIdx.x;
  for (int i = t; i < 4096; i += 64) lds[i] = image[i];
  __syncthreads();
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  out[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((char*)lds + offs[t]));
}

// global_load_lds_dwordx4: every lane loads 16 bytes from src + 16 * lane into LDS
// whose wave-uniform base is 256 bytes into a 4 KiB array; the array (pre-filled
// with -1) is then copied out.
__global__ __launch_bounds__(64) void probe_load_lds(const int* src, int* out) {
  __shared__ __attribute__((aligned(16))) int lds[1024];
  const int t = threadIdx.x;
  for (int i = t; i < 1024; i += 64) lds[i] = -1;
  __syncthreads();
  __builtin_amdgcn_global_load_lds(src + 4 * t, lds + 64, 16, 0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int i = t; i < 1024; i += 64) out[i] = lds[i];
}

// v_permlane16_swap / v_permlane32_swap on (old = 1000 + lane, src = 2000 + lane).
__global__ __launch_bounds__(64) void probe_permlane(int* out) {
  const int t = threadIdx.x;
  const unsigned a = 1000u + t, b = 2000u + t;
  const auto r16 = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  const auto r32 = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  out[4 * t + 0] = (int)r16[0];
  out[4 * t + 1] = (int)r16[1];
  out[4 * t + 2] = (int)r32[0];
  out[4 * t + 3] = (int)r32[1];
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

// image: int16 [4096]; offs: int32 [64] byte offsets (multiples of 8 below 8192,
// checked here on the host copy the caller passes in host_offs); out: int16 [64][4].
int gqa_probe_ds_read_tr16_b64(const void* image, const void* offs, const int* host_offs,
                               void* out, void* stream) {
  if (!image || !offs || !host_offs || !out) return -1;
  for (int i = 0; i < 64; ++i)
    if (host_offs[i] < 0 || host_offs[i] > 8192 - 8 || (host_offs[i] & 7)) return -2;
  hipLaunchKernelGGL(probe_tr16, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     static_cast<const short*>(image), static_cast<const int*>(offs),
                     static_cast<i16x4*>(out));
  return (int)hipGetLastError();
}

// src: int32 [256]; out: int32 [1024].
int gqa_probe_global_load_lds_dwordx4(const void* src, void* out, void* stream) {
  if (!src || !out) return -1;
  hipLaunchKernelGGL(probe_load_lds, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     static_cast<const int*>(src), static_cast<int*>(out));
  return (int)hipGetLastError();
}

// out: int32 [64][4] = (permlane16_swap old', src', permlane32_swap old', src').
int gqa_probe_permlane_swaps(void* out, void* stream) {
  if (!out) return -1;
  hipLaunchKernelGGL(probe_permlane, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     static_cast<int*>(out));
  return (int)hipGetLastError();
}

}  // extern "C"
