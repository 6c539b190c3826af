// Test infrastructure: a CPU stand-in for the subset of HIP the library uses,
// so the library's own kernel and host sources compile as plain C++ and run on
// the host under AddressSanitizer.  Kernels run one thread at a time; barriers,
// waits and scheduling hints are no-ops and MFMA returns its accumulator
// unchanged, so results are meaningless: what is checked is that every global
// address a kernel forms stays inside its buffer.  Direct-to-LDS loads copy the
// lane's bytes into the (static) LDS array.
#pragma once
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

// plain pointers for the kernels' global accesses: AddressSanitizer does not
// instrument accesses through address-space-qualified pointers on the host
#define GMEM
#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ static
#define LDS_AS
#define __align__(n) __attribute__((aligned(n)))
#define HIP_SYMBOL(x) (&(x))

struct dim3 {
    unsigned x, y, z;
    dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};
struct emu_idx { unsigned x, y, z; };
extern emu_idx threadIdx, blockIdx;
extern dim3 gridDim, blockDim;

typedef int hipError_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1 };
typedef void* hipStream_t;
typedef void* hipEvent_t;
enum hipMemcpyKind { hipMemcpyHostToDevice = 1, hipMemcpyDeviceToHost = 2, hipMemcpyDeviceToDevice = 3 };
#define hipHostMallocDefault 0
#define hipEventDisableTiming 2

inline hipError_t hipGetDeviceCount(int* n) { *n = 1; return hipSuccess; }
inline hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
inline hipError_t hipSetDevice(int) { return hipSuccess; }
inline hipError_t hipMalloc(void** p, size_t n) { *p = std::malloc(n); return *p ? hipSuccess : 2; }
template <class T> inline hipError_t hipMalloc(T** p, size_t n) { return hipMalloc(reinterpret_cast<void**>(p), n); }
inline hipError_t hipFree(void* p) { std::free(p); return hipSuccess; }
inline hipError_t hipHostMalloc(void** p, size_t n, unsigned) { *p = std::malloc(n); return *p ? hipSuccess : 2; }
inline hipError_t hipHostFree(void* p) { std::free(p); return hipSuccess; }
inline hipError_t hipMemcpyAsync(void* d, const void* s, size_t n, hipMemcpyKind, hipStream_t) { std::memcpy(d, s, n); return hipSuccess; }
inline hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
inline hipError_t hipDeviceSynchronize() { return hipSuccess; }
inline hipError_t hipEventCreate(hipEvent_t* e) { *e = (void*)1; return hipSuccess; }
inline hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) { *e = (void*)1; return hipSuccess; }
inline hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
inline hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
inline hipError_t hipEventDestroy(hipEvent_t) { return hipSuccess; }
inline hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) { *ms = 0; return hipSuccess; }
inline hipError_t hipGetLastError() { return hipSuccess; }
enum { hipErrorInvalidDevice = 101 };
template <class T> inline hipError_t hipGetSymbolAddress(void** p, T sym) {
    *p = (void*)sym;
    return hipSuccess;
}
enum hipStreamCaptureStatus { hipStreamCaptureStatusNone = 0, hipStreamCaptureStatusActive = 1 };
inline hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* s) {
    *s = hipStreamCaptureStatusNone;
    return hipSuccess;
}
inline const char* hipGetErrorString(hipError_t) { return "emulated"; }

inline float __uint_as_float(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
template <class T> inline T __shfl_xor(T v, int, int) { return v; }
inline void __syncthreads() {}
inline unsigned atomicAdd(unsigned* p, unsigned v) { const unsigned o = *p; *p = o + v; return o; }

#define __builtin_amdgcn_readfirstlane(x) (x)
#define __builtin_amdgcn_s_waitcnt(x) ((void)0)

// direct-to-LDS: lane L writes its `size` bytes at lds + L * size
inline void emu_global_load_lds(const void* src, void* lds, int size) {
    const unsigned lane = threadIdx.x & 63;
    std::memcpy(static_cast<char*>(lds) + lane * size, src, size);
}
#define __builtin_amdgcn_global_load_lds(src, lds, size, off, aux) emu_global_load_lds((src), (lds), (size))
inline void emu_lds_dma16s(const char* sbase, uint32_t voff, char* lds) { emu_global_load_lds(sbase + voff, lds, 16); }
#define MUON_LDS_DMA16S emu_lds_dma16s
#define __builtin_amdgcn_sched_group_barrier(a, b, c) ((void)0)

template <class P> inline auto emu_tr16(P p) { return *p; }
#define __builtin_amdgcn_ds_read_tr16_b64_v4i16(p) emu_tr16(p)

template <class A, class B, class C> inline C emu_mfma(A, B, C c) { return c; }
#define __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, x, y, z) emu_mfma((a), (b), (c))
#define __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, x, y, z) emu_mfma((a), (b), (c))

extern long emu_launches;
extern int emu_verbose;
template <class F, class... A>
inline void emu_launch(const char* name, F f, dim3 g, dim3 b, A... a) {
    ++emu_launches;
    if (emu_verbose) std::fprintf(stderr, "launch %s grid %u block %u\n", name, g.x, b.x);
    gridDim = g;
    blockDim = b;
    for (unsigned bx = 0; bx < g.x; ++bx)
        for (unsigned tx = 0; tx < b.x; ++tx) {
            blockIdx = {bx, 0, 0};
            threadIdx = {tx, 0, 0};
            f(a...);
        }
}
#define hipLaunchKernelGGL(K, G, B, SH, ST, ...) emu_launch(#K, K, G, B, __VA_ARGS__)
