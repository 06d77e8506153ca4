// Host-only stand-in for <hip/hip_runtime.h>, used only to build the C-ABI
// validation layer (api.cpp) with the host compiler's address and
// undefined-behaviour sanitizers. It declares just what that layer uses; the
// definitions live in the sanitizer driver, which also replaces the kernel
// launchers with recorders. No GPU code is ever built with this header.
#pragma once
#include <stddef.h>
#include <stdint.h>

#define __host__
#define __device__
#define __forceinline__ inline

typedef enum hipError_t {
    hipSuccess = 0,
    hipErrorInvalidValue = 1,
    hipErrorInvalidDevice = 101,
    hipErrorInvalidSymbol = 13,
} hipError_t;

typedef struct ihipStream_t* hipStream_t;

typedef struct hipDeviceProp_t {
    char gcnArchName[256];
    int multiProcessorCount;
} hipDeviceProp_t;

hipError_t hipGetDevice(int* dev);
hipError_t hipGetDeviceProperties(hipDeviceProp_t* prop, int dev);
