// qk_launch.h -- internal launch entry points (C++ linkage) behind the C ABI.
// Arguments are validated by the callers in qk_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace qk {

// Host state kept per device and safe under concurrent calls from several
// threads (the C ABI's calls are thread-safe).  Devices are numbered below
// MAX_DEVICES.
constexpr int MAX_DEVICES = 64;

inline int current_device() {
    int d = 0;
    return hipGetDevice(&d) == hipSuccess && d >= 0 && d < MAX_DEVICES ? d : 0;
}

// Compute units of the current device, read once per device.
inline int device_cus() {
    static std::atomic<int> cache[MAX_DEVICES];
    const int dev = current_device();
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

// Kernel F's opt-in to `bytes` of dynamic LDS (above the default 64 KB) on
// the current device, made once per device and kernel (a racing thread may
// repeat it: harmless).
template <auto F>
inline hipError_t lds_opt_in(int bytes) {
    static std::atomic<uint64_t> done{0};
    const uint64_t bit = uint64_t(1) << current_device();
    if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(F),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
    return e;
}

// Layout flag carried in the type argument (QK_PLANAR of the C ABI).
constexpr int PLANAR_FLAG = 0x100;

// What happens at the store of y (a by-value kernel argument; all-zero = the
// plain GEMV): act = W x, or silu(W x) * (W2 x) when W2 is set (the up tensor,
// same type, layout and shape as W); then y = act + res when res is set (fp32
// [N][ncols], may be y itself); y is fp16 (round to nearest even) when f16.
struct Epilogue {
    const void *W2;
    const float *res;
    int f16;
};

// ncols == 1: the streaming GEMV.
hipError_t launch_gemv1(int type, const void *W, const void *x, void *y, int64_t N, int64_t K,
                        const Epilogue &ep, hipStream_t stream);

// Independent one-column GEMVs in one launch (at most MAX_BATCH).
constexpr int MAX_BATCH = 16;
struct BatchEntry {
    int type;
    const void *W;
    const void *x;
    void *y;
    int64_t N, K;
};
hipError_t launch_gemv_batch(const BatchEntry *entries, int count, hipStream_t stream);

// ncols in 2..8: the few-column verify form (matrix cores).
hipError_t launch_gemv_multi(int type, const void *W, const void *x, void *y, int64_t N, int64_t K,
                             int ncols, const Epilogue &ep, hipStream_t stream);

// Chain of one-column steps in one persistent launch (see qk_kernels.hip).
struct ChainEntryIn {
    int type, f16;
    const void *W, *W2, *x;
    void *y;
    const void *res;
    int64_t N, K, row_bytes;
};
int64_t chain_plan_bytes(int nsteps, int nentries);
hipError_t chain_plan(const ChainEntryIn *entries, int nentries, const int *step_sizes, int nsteps, void *plan,
                      int64_t bytes);
int chain_steps(const void *plan_host);  // steps of a plan, or -1 if it is not one
hipError_t launch_chain(const void *plan_host, const void *plan_dev, uint32_t *sync, int64_t sync_words,
                        int64_t timeout_us, hipStream_t stream);
const char *chain_stage();  // the step of the calling thread's last failed launch_chain
// launch_chain with the counters in the library's own per-device array of
// CHAIN_SCRATCH_WORDS words (nsteps + 2 must fit); status: NULL or a device
// word that receives the run's flag word after the chain.
constexpr int CHAIN_SCRATCH_WORDS = 4096;
hipError_t launch_chain_noalloc(const void *plan_host, const void *plan_dev, void *status, int64_t timeout_us,
                                hipStream_t stream);

// fp32 dequantisation of the whole tensor (either layout).
hipError_t launch_dequant(int type, const void *W, void *out, int64_t N, int64_t K, hipStream_t stream);

// GGUF rows -> PLANAR rows (type without the flag).
hipError_t launch_repack(int type, const void *W, void *Wp, int64_t N, int64_t K, hipStream_t stream);

}  // namespace qk
