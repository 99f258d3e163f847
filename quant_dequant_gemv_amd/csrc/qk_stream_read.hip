// qk_stream_read.hip -- the achievable-bandwidth reference of the benchmark
// (libqkcalib.so, not part of the GEMV library): every 16-byte chunk of a
// buffer read once in a grid-stride loop and XOR-folded, so that no load is
// dead.  On one MI355X the non-temporal form of this plain read is the
// fastest of the launch shapes tried for a few tens of MB per launch; the
// GEMV's HBM rate is compared with it as well as with the 8 TB/s peak.  The
// form with ordinary loads serves, beside a device copy, as a second known
// read for scaling the HBM byte counters.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__global__ void __launch_bounds__(1024) stream_read_kernel(const u32x4 *__restrict__ p, size_t n16,
                                                           uint32_t *__restrict__ out) {
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        u32x4 v;
        if constexpr (NT) v = __builtin_nontemporal_load(p + i);
        else v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

template <bool NT>
static int stream_read(const void *p, size_t bytes, void *out, int blocks, int threads, void *stream) {
    if (!p || !out || ((uintptr_t)p & 15) || (bytes & 15) || blocks < 1 || threads < 64 || threads > 1024 ||
        (threads & 63))
        return -1;
    hipLaunchKernelGGL(stream_read_kernel<NT>, dim3((unsigned)blocks), dim3((unsigned)threads), 0,
                       (hipStream_t)stream, (const u32x4 *)p, bytes / 16, (uint32_t *)out);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Reads `bytes` (a multiple of 16) at p (16-byte aligned) with `blocks` x
// `threads` threads (threads a multiple of 64, at most 1024); out receives
// blocks * threads uint32 words.  Returns 0, -1 for bad arguments, -2 if the
// launch fails.  qk_stream_read: non-temporal loads; qk_stream_read_plain:
// ordinary loads.
extern "C" int qk_stream_read(const void *p, size_t bytes, void *out, int blocks, int threads, void *stream) {
    return stream_read<true>(p, bytes, out, blocks, threads, stream);
}

extern "C" int qk_stream_read_plain(const void *p, size_t bytes, void *out, int blocks, int threads, void *stream) {
    return stream_read<false>(p, bytes, out, blocks, threads, stream);
}
