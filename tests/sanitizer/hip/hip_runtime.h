// Stand-in for <hip/hip_runtime.h> in the CPU-only sanitizer build of the
// library's host code (attn_api.cpp, attn_host.cpp). Declares only what that
// code uses; hip_stub.cpp defines it. Test infrastructure: never part of the
// shipped library.
#pragma once

#include <stddef.h>

#define __host__
#define __device__
#define __forceinline__ inline

typedef enum hipError_t {
    hipSuccess = 0,
    hipErrorInvalidValue = 1,
    hipErrorOutOfMemory = 2,
    hipErrorNoDevice = 100,
} hipError_t;

typedef struct ihipStream_t *hipStream_t;
typedef struct ihipEvent_t *hipEvent_t;

typedef enum hipMemcpyKind {
    hipMemcpyHostToHost = 0,
    hipMemcpyHostToDevice = 1,
    hipMemcpyDeviceToHost = 2,
    hipMemcpyDeviceToDevice = 3,
    hipMemcpyDefault = 4,
} hipMemcpyKind;

#define hipEventDisableTiming 0x2

typedef struct hipDeviceProp_t {
    char name[256];
    char gcnArchName[256];
    size_t totalGlobalMem;
    int multiProcessorCount;
} hipDeviceProp_t;

hipError_t hipGetDevice(int *dev);
hipError_t hipGetDeviceProperties(hipDeviceProp_t *prop, int dev);
const char *hipGetErrorString(hipError_t e);
hipError_t hipMalloc(void **ptr, size_t bytes);
hipError_t hipFree(void *ptr);
hipError_t hipMemcpy(void *dst, const void *src, size_t bytes, hipMemcpyKind kind);
hipError_t hipEventCreateWithFlags(hipEvent_t *ev, unsigned flags);
hipError_t hipEventRecord(hipEvent_t ev, hipStream_t stream);
hipError_t hipEventSynchronize(hipEvent_t ev);
hipError_t hipStreamWaitEvent(hipStream_t stream, hipEvent_t ev, unsigned flags);
