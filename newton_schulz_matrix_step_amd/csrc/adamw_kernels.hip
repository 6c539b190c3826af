// gfx950 kernel of the AdamW step the hybrid Muon setup runs on the
// parameters Muon does not take (embeddings, output head, norm gains, biases):
// "14 -- modded-nanogpt: the Speedrun Community", section 3, and the Muon
// page's list of where Muon does not apply.  The pages give no formula; this
// is the standard AdamW (decoupled weight decay, bias-corrected moments):
//
//   m' = beta1 m + (1 - beta1) g ;  v' = beta2 v + (1 - beta2) g^2
//   p' = p (1 - lr wd) - (lr / (1 - beta1^t)) m' / (sqrt(v') / sqrt(1 - beta2^t) + eps)
//
// Pure streaming work (22 bytes an element with bf16 parameters, 28 with
// fp32, no reuse): HBM bound.  One launch covers every tensor of the call; a
// workgroup owns one 4096-element chunk of one tensor, each lane four runs of
// four consecutive elements, all loads of a lane issued before any use.

#include <hip/hip_ext.h>

#include "muon_internal.hpp"

namespace muon {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kAdamThreads = 256;
constexpr int kRuns = kAdamChunk / (4 * kAdamThreads);   // runs of 4 elements per lane
static_assert(kRuns * 4 * kAdamThreads == kAdamChunk, "chunk = lanes x runs x 4");

#ifndef GMEM   // a host build for bounds checking defines it empty
#define GMEM __attribute__((address_space(1)))
#endif
template <class T>
__device__ __forceinline__ GMEM T* gm(T* p) { return (GMEM T*)p; }

// Nothing here is read twice: the 16-byte accesses (moments, float32
// parameters) are streaming (nontemporal) loads and stores, 20 % faster than
// plain ones on the GPT-2 124M set; on the 8-byte bf16 accesses the same hint
// measured slower, so those stay plain.
template <class T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load(gm(p)); }
template <class T>
__device__ __forceinline__ void st_nt(T* p, T v) { __builtin_nontemporal_store(v, gm(p)); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {   // round to nearest even
    __bf16 h = (__bf16)f;
    return uint32_t(__builtin_bit_cast(uint16_t, h));
}

struct Elem {
    float p, m, v;
};

__device__ __forceinline__ Elem adamw_elem(float p, float g, float m, float v, const AdamArgs& a) {
    Elem e;
    e.m = fmaf(a.beta1, m, a.one_minus_beta1 * g);
    e.v = fmaf(a.beta2, v, a.one_minus_beta2 * g * g);
    const float denom = fmaf(__builtin_sqrtf(e.v), a.inv_sqrt_bc2, a.eps);
    e.p = fmaf(-a.step_size, e.m / denom, p * a.decay);
    return e;
}

template <int DT>   // 0: bf16 param/grad, 1: f32
__device__ __forceinline__ void adamw_vec(const AdamDesc& d, int64_t begin, const AdamArgs& a) {
    const int lane = threadIdx.x;
    f32x4_t p[kRuns], g[kRuns], m[kRuns], v[kRuns];
#pragma unroll
    for (int u = 0; u < kRuns; ++u) {
        const int64_t i = begin + int64_t(u * kAdamThreads + lane) * 4;
        if constexpr (DT == 0) {
            const u32x2_t pw = *gm(reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(d.param) + i));
            const u32x2_t gw = *gm(reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(d.grad) + i));
            p[u] = f32x4_t{bf16_bits_to_f32(pw[0] & 0xFFFFu), bf16_bits_to_f32(pw[0] >> 16),
                           bf16_bits_to_f32(pw[1] & 0xFFFFu), bf16_bits_to_f32(pw[1] >> 16)};
            g[u] = f32x4_t{bf16_bits_to_f32(gw[0] & 0xFFFFu), bf16_bits_to_f32(gw[0] >> 16),
                           bf16_bits_to_f32(gw[1] & 0xFFFFu), bf16_bits_to_f32(gw[1] >> 16)};
        } else {
            p[u] = ld_nt(reinterpret_cast<const f32x4_t*>(static_cast<const float*>(d.param) + i));
            g[u] = ld_nt(reinterpret_cast<const f32x4_t*>(static_cast<const float*>(d.grad) + i));
        }
        m[u] = ld_nt(reinterpret_cast<const f32x4_t*>(d.m + i));
        v[u] = ld_nt(reinterpret_cast<const f32x4_t*>(d.v + i));
    }
#pragma unroll
    for (int u = 0; u < kRuns; ++u) {
        const int64_t i = begin + int64_t(u * kAdamThreads + lane) * 4;
        f32x4_t pn, mn, vn;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const Elem e = adamw_elem(p[u][k], g[u][k], m[u][k], v[u][k], a);
            pn[k] = e.p;
            mn[k] = e.m;
            vn[k] = e.v;
        }
        st_nt(reinterpret_cast<f32x4_t*>(d.m + i), mn);
        st_nt(reinterpret_cast<f32x4_t*>(d.v + i), vn);
        if constexpr (DT == 0) {
            *gm(reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(d.param) + i)) =
                u32x2_t{f32_to_bf16_bits(pn[0]) | (f32_to_bf16_bits(pn[1]) << 16),
                        f32_to_bf16_bits(pn[2]) | (f32_to_bf16_bits(pn[3]) << 16)};
        } else {
            st_nt(reinterpret_cast<f32x4_t*>(static_cast<float*>(d.param) + i), pn);
        }
    }
}

__device__ __forceinline__ void adamw_scalar(const AdamDesc& d, int64_t begin, int64_t end, const AdamArgs& a) {
    for (int64_t i = begin + threadIdx.x; i < end; i += kAdamThreads) {
        float p, g;
        if (d.dtype == 0) {
            p = bf16_bits_to_f32(gm(static_cast<const uint16_t*>(d.param))[i]);
            g = bf16_bits_to_f32(gm(static_cast<const uint16_t*>(d.grad))[i]);
        } else {
            p = gm(static_cast<const float*>(d.param))[i];
            g = gm(static_cast<const float*>(d.grad))[i];
        }
        const Elem e = adamw_elem(p, g, gm(d.m)[i], gm(d.v)[i], a);
        gm(d.m)[i] = e.m;
        gm(d.v)[i] = e.v;
        if (d.dtype == 0)
            gm(static_cast<uint16_t*>(d.param))[i] = uint16_t(f32_to_bf16_bits(e.p));
        else
            gm(static_cast<float*>(d.param))[i] = e.p;
    }
}

__global__ __launch_bounds__(kAdamThreads) void adamw_kernel(const AdamChunk* __restrict__ chunks,
                                                             const AdamDesc* __restrict__ tensors, AdamArgs a) {
    const AdamChunk ch = chunks[blockIdx.x];
    const AdamDesc d = tensors[ch.t];
    const int64_t end = ch.begin + kAdamChunk < d.numel ? ch.begin + kAdamChunk : d.numel;
    if (d.vec && end - ch.begin == kAdamChunk) {
        if (d.dtype == 0) adamw_vec<0>(d, ch.begin, a);
        else adamw_vec<1>(d, ch.begin, a);
    } else {
        adamw_scalar(d, ch.begin, end, a);
    }
}

}  // namespace

hipError_t launch_adamw(const AdamChunk* chunks, int n_chunks, const AdamDesc* tensors, AdamArgs a, hipStream_t s,
                        hipEvent_t ev0, hipEvent_t ev1) {
    if (n_chunks <= 0) return hipSuccess;
    hipExtLaunchKernelGGL(adamw_kernel, dim3(n_chunks), dim3(kAdamThreads), 0, s, ev0, ev1, 0, chunks, tensors, a);
    return hipGetLastError();
}

}  // namespace muon
