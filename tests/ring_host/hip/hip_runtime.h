// Host-only stand-in for the few HIP runtime calls the ring's bookkeeping makes, for building
// that bookkeeping with g++ under AddressSanitizer / UndefinedBehaviorSanitizer on the CPU.
// Streams and events are simulated with vector clocks (see sim.h); nothing touches a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

typedef enum {
  hipSuccess = 0,
  hipErrorOutOfMemory = 2,
  hipErrorInvalidValue = 1,
} hipError_t;

typedef struct SimStream* hipStream_t;
typedef struct SimEvent* hipEvent_t;

enum { hipStreamNonBlocking = 1, hipEventDisableTiming = 2 };
typedef enum { hipMemcpyHostToDevice = 1, hipMemcpyDeviceToHost = 2 } hipMemcpyKind;

const char* hipGetErrorString(hipError_t e);
hipError_t hipGetLastError(void);
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned flags);
hipError_t hipStreamDestroy(hipStream_t s);
hipError_t hipStreamSynchronize(hipStream_t s);
hipError_t hipStreamWaitEvent(hipStream_t s, hipEvent_t e, unsigned flags);
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned flags);
hipError_t hipEventDestroy(hipEvent_t e);
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s);
hipError_t hipEventSynchronize(hipEvent_t e);
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind kind,
                          hipStream_t s);
hipError_t hipHostGetDevicePointer(void** dev, void* host, unsigned flags);
