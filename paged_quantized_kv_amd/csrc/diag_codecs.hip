// Diagnostic kernels: the exact device codec paths the store kernels use,
// applied elementwise so a test can sweep them over binary32 inputs.
#include "device_common.h"
#include "launch.h"

namespace pkv {

namespace {

constexpr int kDiagThreads = 256;

// 16 inputs per lane: E4M3 codes as one 16-byte store.
__global__ __launch_bounds__(kDiagThreads) void diag_e4m3_kernel(const float* __restrict__ y,
                                                                  uint8_t* __restrict__ out,
                                                                  int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kDiagThreads;
  for (int64_t i = (int64_t)blockIdx.x * kDiagThreads + threadIdx.x; i < n16; i += stride) {
    const u32x4* p = reinterpret_cast<const u32x4*>(y + i * 16);
    u32x4 v[4] = {p[0], p[1], p[2], p[3]};
    u32x4 c;
    c.x = e4m3_pack4(__uint_as_float(v[0].x), __uint_as_float(v[0].y), __uint_as_float(v[0].z), __uint_as_float(v[0].w));
    c.y = e4m3_pack4(__uint_as_float(v[1].x), __uint_as_float(v[1].y), __uint_as_float(v[1].z), __uint_as_float(v[1].w));
    c.z = e4m3_pack4(__uint_as_float(v[2].x), __uint_as_float(v[2].y), __uint_as_float(v[2].z), __uint_as_float(v[2].w));
    c.w = e4m3_pack4(__uint_as_float(v[3].x), __uint_as_float(v[3].y), __uint_as_float(v[3].z), __uint_as_float(v[3].w));
    *reinterpret_cast<u32x4*>(out + i * 16) = c;
  }
}

// 16 inputs per lane: E2M1 codes, one per output byte (low nibble).
__global__ __launch_bounds__(kDiagThreads) void diag_e2m1_kernel(const float* __restrict__ y,
                                                                  uint8_t* __restrict__ out,
                                                                  int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kDiagThreads;
  for (int64_t i = (int64_t)blockIdx.x * kDiagThreads + threadIdx.x; i < n16; i += stride) {
    const u32x4* p = reinterpret_cast<const u32x4*>(y + i * 16);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 v = p[q];
      // two packed bytes hold four nibbles; spread them to one nibble per byte
      uint32_t pk = e2m1_pack2<0>(__uint_as_float(v.x), __uint_as_float(v.y), 0u);
      pk = e2m1_pack2<1>(__uint_as_float(v.z), __uint_as_float(v.w), pk);
      w[q] = (pk & 0xfu) | ((pk >> 4) & 0xfu) << 8 | ((pk >> 8) & 0xfu) << 16 |
             ((pk >> 12) & 0xfu) << 24;
    }
    u32x4 c = {w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4*>(out + i * 16) = c;
  }
}

int64_t diag_blocks(int64_t n16) {
  int64_t b = (n16 + kDiagThreads - 1) / kDiagThreads;
  if (b > 65536) b = 65536;
  return b < 1 ? 1 : b;
}

}  // namespace

int launch_diag_e4m3(const float* y, uint8_t* out, int64_t n, hipStream_t stream) {
  const int64_t n16 = n / 16;
  hipLaunchKernelGGL(diag_e4m3_kernel, dim3((unsigned)diag_blocks(n16)), dim3(kDiagThreads), 0,
                     stream, y, out, n16);
  return (int)hipGetLastError();
}

int launch_diag_e2m1(const float* y, uint8_t* out, int64_t n, hipStream_t stream) {
  const int64_t n16 = n / 16;
  hipLaunchKernelGGL(diag_e2m1_kernel, dim3((unsigned)diag_blocks(n16)), dim3(kDiagThreads), 0,
                     stream, y, out, n16);
  return (int)hipGetLastError();
}

}  // namespace pkv
