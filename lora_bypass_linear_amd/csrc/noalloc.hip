// noalloc.hip -- the LoRA-bypass forward for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc): lyc_lora_linear_fwd_noalloc.
//
// It runs exactly the kernels of lyc_lora_linear_fwd.  Their scratch memory
// (h_r, the compute-dtype copies of the factors and of fp32 operands, down's
// hi/lo split and norms, the guard counter, split-K partial sums) lives in one
// file-scope device array instead of a caller workspace.  Each GPU the
// library runs on holds its own copy of the array (LYC_NOALLOC_SCRATCH_BYTES)
// from the first call on that GPU until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and only that address is ever passed to a kernel.
#include "../../include/lyc.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

static __device__ __align__(256) unsigned char scratch[LYC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
std::atomic<void*> g_scratch[MAX_DEVICES];

// The device that owns `stream` (the current device for the NULL stream).
int stream_device(hipStream_t s, int* dev) {
    if (s == nullptr) return hipGetDevice(dev) == hipSuccess ? LYC_OK : LYC_ERR_HIP;
    return hipStreamGetDevice(s, dev) == hipSuccess ? LYC_OK : LYC_ERR_HIP;
}

// The device address of `scratch` on device `dev`, looked up on the first call
// for that device with the device current (and the caller's device restored).
int scratch_on(int dev, void** out) {
    if (dev < 0 || dev >= MAX_DEVICES) return LYC_ERR_UNSUPPORTED;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lk(g_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            int prev = -1;
            if (hipGetDevice(&prev) != hipSuccess) return LYC_ERR_HIP;
            if (prev != dev && hipSetDevice(dev) != hipSuccess) return LYC_ERR_HIP;
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (prev != dev && hipSetDevice(prev) != hipSuccess) return LYC_ERR_HIP;
            if (e != hipSuccess || p == nullptr) return LYC_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return LYC_OK;
}

}  // namespace

extern "C" int lyc_lora_linear_fwd_noalloc(const void* x, int x_dt, const void* w, int w_dt, const void* bias,
                                           int bias_dt, const void* down, int down_dt, const void* up, int up_dt,
                                           int64_t rank, double scale, void* y, int y_dt, int64_t M, int64_t N,
                                           int64_t K, void* stream) {
    // the problem's scratch need, with every shape and dtype check of the
    // forward (no HIP call yet)
    size_t need = 0;
    int st = lyc_lora_linear_workspace_size(M, N, K, rank, x_dt, w_dt, bias_dt, down_dt, up_dt, &need);
    if (st != LYC_OK) return st;
    if (need > (size_t)LYC_NOALLOC_SCRATCH_BYTES) return LYC_ERR_SCRATCH;
    int dev = 0;
    if ((st = stream_device((hipStream_t)stream, &dev)) != LYC_OK) return st;
    void* ws = nullptr;
    if ((st = scratch_on(dev, &ws)) != LYC_OK) return st;
    // the forward checks the remaining arguments before its first launch and
    // clears the guard counter with a kernel of its own
    return lyc_lora_linear_fwd(x, x_dt, w, w_dt, bias, bias_dt, down, down_dt, up, up_dt, rank, scale, y, y_dt, M, N,
                               K, ws, (size_t)LYC_NOALLOC_SCRATCH_BYTES, stream);
}
