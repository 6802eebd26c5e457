// A host-memory test double of the few HIP runtime calls the library's host
// code makes, so that code (ring metadata, capsules, staging fences,
// argument validation, launch planning) can run on a machine without a GPU
// under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Every "device" pointer the driver passes is host memory. Copies are done
// with memcpy; kernel launches are recorded (grid, block and the first
// integer arguments) but not run; events are heap objects, so a leaked or
// doubly destroyed event shows up as an ASan report. Test-only: nothing in
// the library links this file.

#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <string.h>

#include "hip_host_double.h"
#include "internal.h"       // the ring's run-copy kernel, which the double performs

namespace dbl {
HostDouble g;
}

using dbl::g;

extern "C" {

void** __hipRegisterFatBinary(const void*) {
    static void* handle = nullptr;
    return &handle;
}
void __hipUnregisterFatBinary(void**) {}
void __hipRegisterFunction(void**, const void*, char*, const char*, unsigned int, void*, void*, void*, void*, int*) {}
void __hipRegisterVar(void**, void*, char*, char*, int, size_t, int, int) {}
char hip_double_fatbin[16] = {0};

// the configuration a kernel stub pushes and pops before its launch
static dim3 cfg_grid, cfg_block;
static size_t cfg_shmem;
static hipStream_t cfg_stream;

hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t shmem, hipStream_t stream) {
    cfg_grid = grid;
    cfg_block = block;
    cfg_shmem = shmem;
    cfg_stream = stream;
    return hipSuccess;
}
hipError_t __hipPopCallConfiguration(dim3* grid, dim3* block, size_t* shmem, hipStream_t* stream) {
    *grid = cfg_grid;
    *block = cfg_block;
    *shmem = cfg_shmem;
    *stream = cfg_stream;
    return hipSuccess;
}

hipError_t hipLaunchKernel(const void* fn, dim3 grid, dim3 block, void** args, size_t shmem, hipStream_t) {
    g.launches += 1;
    g.last_grid = grid.x * (long long)grid.y * grid.z;
    g.last_block = block.x * (long long)block.y * block.z;
    if (grid.x == 0 || grid.y == 0 || grid.z == 0 || g.last_block <= 0 || g.last_block > 1024 ||
        grid.y > 65535 || grid.z > 65535 || shmem > 160 * 1024)
        g.bad_launches += 1;
    // A one-thread launch is the ring's state-word write (int4*, int, int, int):
    // record its arguments; other kernels' arguments are not read.
    if (g.last_grid == 1 && g.last_block == 1 && args) {
        g.last_ptr = *static_cast<void**>(args[0]);
        for (int i = 0; i < 3; ++i) g.last_int[i] = *static_cast<int*>(args[i + 1]);
        g.state_writes += 1;
    }
    // The ring's frame and prefix copies move bytes the driver checks: the
    // double performs them, one run per (tensor, layer) the grid covers.
    if (fn == reinterpret_cast<const void*>(&pa::copy_kv_runs) && args) {
        const pa::RunCopy& c = *static_cast<const pa::RunCopy*>(args[0]);
        for (unsigned y = 0; y < grid.y; ++y) {
            const int t = y & 1, l = y >> 1;
            memcpy(c.dst[t] + (long long)l * c.dst_stride, c.src[t] + (long long)l * c.run, (size_t)c.run * 16);
        }
        g.copies += 1;
    }
    return hipSuccess;
}

hipError_t hipMemcpy2DAsync(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t height,
                            hipMemcpyKind, hipStream_t) {
    g.copies += 1;
    if (width > dpitch || width > spitch) return hipErrorInvalidValue;
    for (size_t r = 0; r < height; ++r)
        memcpy(static_cast<char*>(dst) + r * dpitch, static_cast<const char*>(src) + r * spitch, width);
    return hipSuccess;
}

hipError_t hipEventCreateWithFlags(hipEvent_t* ev, unsigned) {
    *ev = reinterpret_cast<hipEvent_t>(new int(0));
    g.live_events += 1;
    return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t ev) {
    delete reinterpret_cast<int*>(ev);
    g.live_events -= 1;
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t ev, hipStream_t) {
    *reinterpret_cast<int*>(ev) += 1;
    g.records += 1;
    return hipSuccess;
}
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t ev, unsigned) {
    g.waits += 1;
    g.last_wait_count = *reinterpret_cast<int*>(ev);
    return hipSuccess;
}
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* st) {
    *st = g.capturing ? hipStreamCaptureStatusActive : hipStreamCaptureStatusNone;
    return hipSuccess;
}
hipError_t hipGetDevice(int* d) {
    *d = 0;
    return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** p, const void* symbol) {
    *p = const_cast<void*>(symbol);     // the host shadow of a __device__ array
    return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "host double"; }

}  // extern "C"
