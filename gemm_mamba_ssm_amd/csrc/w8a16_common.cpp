// Status strings and the per-device compute-unit count used to size grids.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "w8a16_host.h"

namespace w8a16 {

int device_cu_count() {
    constexpr int kMaxDevices = 64;
    static int cached[kMaxDevices] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

bool allow_large_lds(const void* kernel, size_t bytes) {
    struct Raised {
        int dev;
        const void* kernel;
        size_t bytes;
    };
    static std::mutex mu;
    static std::vector<Raised> done;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    std::lock_guard<std::mutex> lock(mu);
    Raised* entry = nullptr;
    for (auto& d : done)
        if (d.dev == dev && d.kernel == kernel) entry = &d;
    if (entry && entry->bytes >= bytes) return true;
    if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes)) != hipSuccess)
        return false;
    if (entry)
        entry->bytes = bytes;
    else
        done.push_back(Raised{dev, kernel, bytes});
    return true;
}

}  // namespace w8a16

extern "C" const char* w8a16_strerror(int status) {
    switch (status) {
        case W8A16_OK: return "ok";
        case W8A16_ERR_NULL: return "a required pointer is NULL";
        case W8A16_ERR_SHAPE: return "M, N or K out of range (K must be >= 16 and a multiple of 16)";
        case W8A16_ERR_ALIGN: return "A, Wq (and dequant out) must be 16-byte aligned; scale and out 2-byte aligned";
        case W8A16_ERR_LAUNCH: return "HIP kernel launch failed";
        case W8A16_ERR_ALIAS: return "out overlaps an input buffer";
        case W8A16_ERR_ARG: return "invalid argument";
        case W8A16_ERR_WORKSPACE: return "the GEMM workspace is smaller than w8a16_gemm_workspace_size";
        case W8A16_ERR_SCRATCH:
            return "the shape needs more scratch than w8a16_gemm_noalloc holds (w8a16_gemm_noalloc_scratch_bytes)";
        default: return "unknown w8a16 status";
    }
}
