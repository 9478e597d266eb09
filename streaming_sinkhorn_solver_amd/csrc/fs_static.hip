// fs_static.hip -- the allocation-free form of set-up + solve.
//
// fs_sinkhorn_solve_static runs fs_potentials_init and fs_sinkhorn_solve with
// their workspace in a file-scope device array instead of caller memory, for
// callers that cannot allocate device memory.  Each GPU the library runs on
// holds its own copy of the array (kStaticScratchBytes) from the moment the
// library's code is loaded on it until the process ends.  In host code the
// array's name is only a stand-in: its device address on the current GPU is
// looked up once per device with hipGetSymbolAddress and that address is what
// the kernels receive.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "fs_internal.h"
#include "fs_sinkhorn.h"

namespace {

constexpr size_t kStaticScratchBytes = FS_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_lock;
void* g_ptr[kMaxDevices] = {};

thread_local char g_msg[256];

// The device address of `scratch` on the current device (looked up on the
// first call there), or nullptr with a message in g_msg.
void* scratch_on_current_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        std::snprintf(g_msg, sizeof(g_msg), "hipGetDevice: %s (device %d)",
                      hipGetErrorString(e), dev);
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_lock);
    if (!g_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            std::snprintf(g_msg, sizeof(g_msg), "hipGetSymbolAddress(scratch) on device %d: %s",
                          dev, hipGetErrorString(e));
            return nullptr;
        }
        g_ptr[dev] = ptr;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" {

size_t fs_static_scratch_bytes(void) { return kStaticScratchBytes; }

fs_status fs_sinkhorn_solve_static(const float* X, const float* Y, const float* a,
                                   const float* b, int64_t n, int64_t m, int32_t d,
                                   fs_score_prec prec, const fs_solve_opts* opts, float* f,
                                   float* g, fs_solve_info* info, void* stream) {
    const size_t need = fs_workspace_bytes(n, m, d, 0, prec);
    if (need == 0)  // invalid sizes or precision: the set-up's checks name the problem
        return fs::solve_in_workspace(X, Y, a, b, n, m, d, prec, opts, nullptr, 0, f, g, info,
                                      stream);
    if (need > kStaticScratchBytes) {
        std::snprintf(g_msg, sizeof(g_msg),
                      "problem needs %zu bytes of workspace; the static scratch holds %zu "
                      "(use fs_potentials_init with a caller workspace)",
                      need, kStaticScratchBytes);
        return fs::report(FS_ERR_WORKSPACE, g_msg);
    }
    void* ptr = scratch_on_current_device();
    if (!ptr) return fs::report(FS_ERR_DEVICE, g_msg);
    return fs::solve_in_workspace(X, Y, a, b, n, m, d, prec, opts, ptr, kStaticScratchBytes, f, g,
                                  info, stream);
}

}  // extern "C"
