// bench_copy.hip -- plain device streams of known size, used by bench.py only:
// (1) as the ceilings the norm kernels are compared with (a copy of x's bytes
// into y, read-only / write-only streams of the same bytes, and copies with
// a kernel's own mix of streams: two in and two out for the residual add,
// two in and one out for the backward), and (2) to
// calibrate rocprofv3's FETCH_SIZE / WRITE_SIZE counters (bytes counted per
// byte actually moved).  One 16-byte vector per lane, one workgroup of 256
// lanes per 4 KiB: the simplest streaming kernels, with ordinary (cached) or
// nontemporal accesses.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void plain_copy16(const u32x4* __restrict__ src,
                                                    u32x4* __restrict__ dst, uint64_t n16) {
    const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void nt_copy16(const u32x4* __restrict__ src,
                                                 u32x4* __restrict__ dst, uint64_t n16) {
    const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// reads every vector; writes one only if its four words XOR to a value the
// caller's data never holds (the store keeps the loads from being removed)
__global__ __launch_bounds__(256) void nt_read16(const u32x4* __restrict__ src,
                                                 u32x4* __restrict__ dst, uint64_t n16) {
    const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        if ((v.x ^ v.y ^ v.z ^ v.w) == 0x9e3779b9u && v.x == 0x7f800001u) dst[i] = v;
    }
}

__global__ __launch_bounds__(256) void nt_write16(const u32x4* __restrict__ src,
                                                  u32x4* __restrict__ dst, uint64_t n16) {
    const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) __builtin_nontemporal_store(u32x4{(unsigned)i, 0u, 0u, 0u}, dst + i);
}

// kind: 0 cached copy, 1 nontemporal copy, 2 nontemporal read of src (dst is
// only written where the impossible value above occurs), 3 nontemporal write
// of dst (src unused).  bytes must be a multiple of 16 and both pointers
// 16-byte aligned.  Returns 0 on success, 1 on a bad argument, 2 if the
// launch failed.
extern "C" int bench_stream(int kind, const void* src, void* dst, uint64_t bytes, void* stream) {
    if (kind < 0 || kind > 3 || !src || !dst || bytes % 16 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15))
        return 1;
    const uint64_t n16 = bytes / 16;
    if (n16 == 0) return 0;
    const uint64_t blocks = (n16 + 255) / 256;
    if (blocks > 0xffffffffull) return 1;
    void (*k)(const u32x4*, u32x4*, uint64_t) =
        kind == 0 ? plain_copy16 : kind == 1 ? nt_copy16 : kind == 2 ? nt_read16 : nt_write16;
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// the cached copy (kind 0), the counter calibration reference
extern "C" int bench_plain_copy(const void* src, void* dst, uint64_t bytes, void* stream) {
    return bench_stream(0, src, dst, bytes, stream);
}

// Two sources of n16 vectors each: kind 0 copies src0 to dst0 and src1 to
// dst1 (two streams in, two out); kind 1 writes src0 ^ src1 to dst0 (two in,
// one out; dst1 unused).  All nontemporal.
__global__ __launch_bounds__(256) void nt_copy22(const u32x4* __restrict__ s0, const u32x4* __restrict__ s1,
                                                 u32x4* __restrict__ d0, u32x4* __restrict__ d1, uint64_t n16) {
    const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) {
        const u32x4 a = __builtin_nontemporal_load(s0 + i), b = __builtin_nontemporal_load(s1 + i);
        __builtin_nontemporal_store(a, d0 + i);
        __builtin_nontemporal_store(b, d1 + i);
    }
}

__global__ __launch_bounds__(256) void nt_copy21(const u32x4* __restrict__ s0, const u32x4* __restrict__ s1,
                                                 u32x4* __restrict__ d0, u32x4* __restrict__ d1, uint64_t n16) {
    (void)d1;
    const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(s0 + i) ^ __builtin_nontemporal_load(s1 + i), d0 + i);
}

// kind 0: two streams in, two out; 1: two in, one out (dst1 may be NULL).
// Same argument rules and return codes as bench_stream.
extern "C" int bench_stream2(int kind, const void* src0, const void* src1, void* dst0, void* dst1, uint64_t bytes,
                             void* stream) {
    auto al = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    if (kind < 0 || kind > 1 || !src0 || !src1 || !dst0 || (kind == 0 && !dst1) || bytes % 16 || !al(src0) ||
        !al(src1) || !al(dst0) || !al(dst1))
        return 1;
    const uint64_t n16 = bytes / 16;
    if (n16 == 0) return 0;
    const uint64_t blocks = (n16 + 255) / 256;
    if (blocks > 0xffffffffull) return 1;
    hipLaunchKernelGGL(kind == 0 ? nt_copy22 : nt_copy21, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const u32x4*>(src0), static_cast<const u32x4*>(src1), static_cast<u32x4*>(dst0),
                       static_cast<u32x4*>(dst1), n16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
