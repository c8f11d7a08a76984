// Host stand-in for the HIP runtime API types used by the launch interface.
#pragma once
#include <stdint.h>
typedef void* hipStream_t;
typedef int hipError_t;
enum { hipSuccess = 0 };
struct dim3 {
  unsigned x, y, z;
  dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};
