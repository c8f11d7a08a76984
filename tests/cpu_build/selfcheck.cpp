// Two kernels with planted mistakes, to show that the CPU build reports them:
//   oob   -- lane 255 reads one element past the end of its buffer
//             (AddressSanitizer stops the run);
//   skip  -- half of each wave takes part in a cross-lane exchange while the
//             other half waits at the workgroup barrier (neither wait can
//             complete: the CPU build reports a deadlock).
// Usage: selfcheck oob|skip
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <vector>

__global__ void read_past_the_end(const float* a, float* out) {
  const int i = threadIdx.x;
  out[i] = a[i + (i == 255 ? 1 : 0)];
}

__global__ void half_wave_exchange(float* out) {
  const int lane = threadIdx.x & 63;
  float x = (float)lane;
  if (lane < 32)
    x = __shfl_xor(x, 1);
  else
    __syncthreads();
  out[threadIdx.x] = x;
}

int main(int argc, char** argv) {
  if (argc != 2) return 2;
  std::vector<float> a(256, 1.0f), out(256);
  if (!std::strcmp(argv[1], "oob"))
    hipLaunchKernelGGL(read_past_the_end, dim3(1), dim3(256), 0, nullptr, a.data(), out.data());
  else
    hipLaunchKernelGGL(half_wave_exchange, dim3(1), dim3(256), 0, nullptr, out.data());
  std::printf("finished\n");
  return 0;
}
