// fdl_block_score_topc_noalloc: block scoring for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops, harnesses that forbid it).
//
// The workspace of fdl_block_score_topc (each KV head's part of R, R, and the block means
// when they are computed from the keys) lives in a file-scope device array, `scratch`, of
// kScratchBytes.  Each GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends.  Host code never passes the array's name to a kernel
// (in host code that name is a host-side stand-in, not a device address): on its first call
// on a device, with that device current, the entry point looks the array's device address
// up with hipGetSymbolAddress and keeps it per device.
//
// Every call on one GPU shares that GPU's array and leaves its contents behind; the
// kernels of this entry point write every workspace element they read, so nothing has to
// start at zero.  Calls that overlap on one GPU (on different streams, or from different
// host threads without ordering) race on the array.

#include <mutex>

#include "ops.cuh"

namespace {
constexpr size_t kScratchBytes = size_t(8) << 20;   // 8 MiB (the 32K-context shapes need at most 4.2 MB)
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device (looked up once per device).
fdl_status scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FDL_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FDL_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return FDL_OK;
}

}  // namespace

extern "C" {

size_t fdl_block_score_topc_noalloc_max_bytes(void) { return kScratchBytes; }

fdl_status fdl_block_score_topc_noalloc(fdl_dtype dt, int B, int Hq, int Hkv, int L, int P, int d, const void* q,
                                        fdl_strides qs, const int32_t* q_idx, const int32_t* n_q, int nq_max,
                                        const void* k, fdl_strides ks, float scale, int bs, int C,
                                        int32_t* block_idx, double* R, float* kbar, hipStream_t stream) {
    const size_t need = fdl_block_score_topc_workspace_bytes(dt, B, Hq, Hkv, P, d, bs, nq_max);
    if (need > kScratchBytes) return FDL_ERR_WORKSPACE;
    void* ws = nullptr;
    const fdl_status st = scratch_on_current_device(&ws);
    if (st != FDL_OK) return st;
    return fdl_block_score_topc(dt, B, Hq, Hkv, L, P, d, q, qs, q_idx, n_q, nq_max, k, ks, scale, bs, C, block_idx, R,
                                kbar, ws, kScratchBytes, stream);
}

}  // extern "C"
