// Streaming-read reference for the roofline (gfx950): how fast this chip's
// HBM delivers a plain sequential read, measured in the same run as the
// decode, so the decode's bandwidth can be quoted against what a read-only
// kernel reaches as well as against the nominal 8 TB/s.
//
// Not part of the decode library: bench.py loads it (libmla_hbm_probe.so)
// for its reference figure only.
//
// Each thread reads 16 bytes per load with eight non-temporal loads in
// flight, grid-striding over the buffer; the XOR of everything read decides
// a store that never happens in practice, so no load can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ void __launch_bounds__(kThreads) stream_read_kernel(const i32x4* p, int64_t n16, int32_t* sink) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    i32x4 acc = {0, 0, 0, 0};
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        i32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= p[i];
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x7a3b9c1d) sink[0] = 1;
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16, 16-byte aligned) from device buffer `buf`
// once on `stream` with `grid` workgroups of 256 threads.  `sink` is a
// device int32 the kernel may write.  Returns 0, or 1 on a bad argument or
// launch failure.
int32_t mla_hbm_read_probe(const void* buf, int64_t bytes, int32_t grid, int32_t* sink, void* stream) {
    if (!buf || !sink || bytes <= 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15) || grid < 1)
        return 1;
    hipLaunchKernelGGL(stream_read_kernel, dim3(uint32_t(grid)), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), static_cast<const i32x4*>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
