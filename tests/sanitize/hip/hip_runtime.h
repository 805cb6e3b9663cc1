/* Host-only stand-in for <hip/hip_runtime.h>, used to build the C-ABI
 * layer (fa2_api.cpp) with the host compiler and its sanitizers, without
 * any GPU code.  Only the names that layer and fa2_internal.h use. */
#pragma once
#include <stddef.h>
#include <stdint.h>
typedef int hipError_t;
enum {
  hipSuccess = 0,
  hipErrorInvalidValue = 1,
  hipErrorInvalidSymbol = 13,
  hipErrorInvalidDevice = 101,
  hipErrorLaunchFailure = 719
};
typedef struct ihipStream_t *hipStream_t;
typedef int hipDevice_t;
#define hipStreamLegacy ((hipStream_t)1)
#define hipStreamPerThread ((hipStream_t)2)
/* defined by the sanitizer test program, which decides what they report */
hipError_t hipGetDevice(int *device);
hipError_t hipStreamGetDevice(hipStream_t stream, hipDevice_t *device);
