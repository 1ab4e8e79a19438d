// bench_copy.hip -- a plain device copy of known size, used by bench.py only:
// (1) as the copy ceiling the norm kernels are compared with, and (2) to
// calibrate rocprofv3's FETCH_SIZE / WRITE_SIZE counters (bytes counted per
// byte actually moved).  One 16-byte vector per lane, one workgroup of 256
// lanes per 4 KiB, cached loads and stores: the simplest streaming kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void plain_copy16(const u32x4* __restrict__ src,
                                                    u32x4* __restrict__ dst, uint64_t n16) {
    const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) dst[i] = src[i];
}

// bytes must be a multiple of 16 and both pointers 16-byte aligned.
// Returns 0 on success, 1 on a bad argument, 2 if the launch failed.
extern "C" int bench_plain_copy(const void* src, void* dst, uint64_t bytes, void* stream) {
    if (!src || !dst || bytes % 16 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return 1;
    const uint64_t n16 = bytes / 16;
    if (n16 == 0) return 0;
    const uint64_t blocks = (n16 + 255) / 256;
    if (blocks > 0xffffffffull) return 1;
    hipLaunchKernelGGL(plain_copy16, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
