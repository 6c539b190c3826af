// gfx950 kernels of the Muon step.
//
//  momentum_kernel      m' = beta m + g, u = g + beta m' (Nesterov) or m',
//                       operand copy of u, per-unit sum of u^2      (HBM bound)
//  finalize_norm        1 / (||u||_F + eps) per matrix, fixed-order sum
//  ns_gemm_bf16<KIND>   the three products of one quintic Newton-Schulz
//                       iteration, grouped over every matrix of the call:
//                         GRAM  A = X X^T           (upper tiles, mirrored store)
//                         POLY  B = b A + c A A     (A symmetric: A A = A A^T)
//                         AXPY  X' = a X + B X      (master X: bf16 hi + 8-bit lo)
//                         AXPY_LAST  same, then W' = W (1 - lr wd) - lr s O
//  ns_gemm_kernel<KIND> the same phases in fp32 (validation mode)
//  direct_update        the update when ns_steps == 0
//
// The iteration follows the Newton-Schulz routine of the "NanoGPT Speedrun"
// page (modded-nanogpt README mirror), Muon section; the momentum and update
// follow "14 -- modded-nanogpt", section 3 pseudocode.
//
// MFMA products: v_mfma_f32_16x16x32_bf16 (bf16 mode) or v_mfma_f32_16x16x4_f32
// (fp32 validation mode), fp32 accumulation.

#include <hip/hip_ext.h>

#include <type_traits>

#include "muon_internal.hpp"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

// Every buffer the kernels read or write outside LDS (caller tensors, workspace)
// is global memory.  Pointers loaded from a descriptor are generic, and generic
// accesses become flat instructions, which count against the LDS wait counter as
// well: an epilogue that mixes them with LDS staging waits for its global loads
// at every LDS wait.  gm() restates the address space.
#ifndef GMEM   // a host build for bounds checking defines it empty
#define GMEM __attribute__((address_space(1)))
#endif
template <class T>
__device__ __forceinline__ GMEM T* gm(T* p) { return (GMEM T*)p; }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Streaming (nontemporal) 16-byte accesses for data a kernel touches once.
template <class T>
__device__ __forceinline__ T ld_nt(const GMEM T* p) { return __builtin_nontemporal_load(p); }
template <class T>
__device__ __forceinline__ void st_nt(GMEM T* p, T v) { __builtin_nontemporal_store(v, p); }

// Round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

// Low part of the master X in one byte: the remainder x - bf16(x) counted in
// units of 1/256 of the bf16 spacing at hi (spacing 2^(E-134) for biased
// exponent E >= 1, the denormal spacing for E = 0), rounded to nearest and
// stored offset by 128.  The remainder of a round-to-nearest is at most half
// a spacing, 128 units (clamped to 127); hi + lo then holds x to half a unit,
// one unit at such ties: 2^-15 relative at worst.
__device__ __forceinline__ int lo8_unit_exp(uint32_t hbits) {
    const int e = int((hbits >> 7) & 0xFFu);
    return (e < 1 ? 1 : e) - 142;
}
__device__ __forceinline__ uint32_t enc_lo8(float rem, uint32_t hbits) {
    float q = __builtin_rintf(ldexpf(rem, -lo8_unit_exp(hbits)));
    q = fminf(fmaxf(q, -127.f), 127.f);
    return uint32_t(int(q) + 128);
}
__device__ __forceinline__ float dec_lo8(uint32_t byte, uint32_t hbits) {
    return ldexpf(float(byte) - 128.f, lo8_unit_exp(hbits));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// dtype 0 = bf16, 1 = f32
__device__ __forceinline__ float load_elem(const void* p, int64_t i, int dt) {
    return dt == 0 ? bf16_to_f32(gm(static_cast<const uint16_t*>(p))[i]) : gm(static_cast<const float*>(p))[i];
}

__device__ __forceinline__ void store_elem(void* p, int64_t i, int dt, float v) {
    if (dt == 0)
        gm(static_cast<uint16_t*>(p))[i] = f32_to_bf16(v);
    else
        gm(static_cast<float*>(p))[i] = v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Sum over the 256 threads of a block in a fixed order; result valid in thread 0.
__device__ __forceinline__ double block_sum(double v, double* red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0) t = ((red[0] + red[1]) + red[2]) + red[3];
    return t;
}

// The orthogonalised input u at stored element (r, c), computed from the updated
// momentum m' and the gradient exactly as the momentum pass computed it.
__device__ __forceinline__ float u_at(const MatDesc& md, int64_t r, int64_t c, float beta, bool nest) {
    const float g = load_elem(md.grad, r * md.ld_grad + c, md.io_dtype);
    if (!md.has_mom) return g;
    const float mn = gm(md.mom)[r * md.ld_mom + c];
    return nest ? fmaf(beta, mn, g) : mn;
}

// ---------------------------------------------------------------------------
// workspace zero fill
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void fill_zero_kernel(u32x4_t* p, size_t n16) {
    const u32x4_t z = {0u, 0u, 0u, 0u};
    for (size_t i = blockIdx.x * size_t(kThreads) + threadIdx.x; i < n16; i += size_t(gridDim.x) * kThreads) p[i] = z;
}

// ---------------------------------------------------------------------------
// debug guard bands: write the pattern, or count the words that lost it
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void guard_kernel(char* ws, const int64_t* __restrict__ offsets, int n_guards,
                                                         uint32_t* bad) {
    constexpr int kWords = kGuardBytes / 4;
    for (int g = blockIdx.x; g < n_guards; g += gridDim.x) {
        GMEM uint32_t* p = gm(reinterpret_cast<uint32_t*>(ws + offsets[g]));
        for (int i = threadIdx.x; i < kWords; i += kThreads) {
            if (!bad) p[i] = kGuardPattern;
            else if (p[i] != kGuardPattern) atomicAdd(bad, 1u);
        }
    }
}

// ---------------------------------------------------------------------------
// momentum + operand copy + partial sums of squares
// ---------------------------------------------------------------------------
// The sum of squares runs in double: u^2 of any finite float is finite there,
// and the sum of 2^31 of them neither overflows nor loses the small terms, so
// the norm is right at every gradient scale.  g and m are read once and m' is
// written once (streaming accesses, MUON_MOM_NT); the operand copy of u is
// read again by the first iteration's products (plain stores: a streaming
// store of it measured 7 % slower on the GPT-2 124M set).
#ifndef MUON_MOM_NT
#define MUON_MOM_NT 1
#endif
#ifndef MUON_MOM_FLAT
#define MUON_MOM_FLAT 1
#endif
template <class T>
__device__ __forceinline__ T mom_ld(const GMEM T* p) {
    if (MUON_MOM_NT) return ld_nt(p);
    return *p;
}
template <class T>
__device__ __forceinline__ void mom_st(GMEM T* p, T v) {
    if (MUON_MOM_NT) st_nt(p, v);
    else *p = v;
}
// KU: runs of 4 elements in flight per lane and pass of the flat path.  Four
// suit calls of up to about 200 M elements (GPT-2 124M set: 79 % of HBM with
// four, 73 % with eight), eight larger ones (large layer share: 75 % with
// eight, 70 % with four).
template <int KU>
__global__ __launch_bounds__(kThreads) void momentum_kernel(const Unit* __restrict__ units,
                                                            const MatDesc* __restrict__ mats, MomentumArgs ka) {
    __shared__ double red[4];
    const Unit un = units[blockIdx.x];
    const MatDesc& md = mats[un.mat];
    const bool F32C = md.f32 != 0;   // this entry's iteration runs in float32
    const int C = md.C;
    const int rows = un.r1 - un.r0;
    const float beta = ka.beta;
    const bool nest = ka.nesterov != 0;
    const bool has_mom = md.has_mom != 0;
    char* ub = ka.ws + md.off_u;
    const int64_t ldu = md.Cp;
    double ss = 0.0;

    // Contiguous rows (grad, momentum and the operand copy all with leading
    // dimension C): the unit is one flat range of elements, taken in runs of 4
    // per lane with no row arithmetic, so each load and store instruction of a
    // wave covers one contiguous span (1 KB of m and m', 512 B of bf16 g and
    // u).  Runs of 8 per lane (two 16-byte halves of m 32 bytes apart) left
    // every m instruction half-coalesced: 69 % of HBM on the large layer
    // share against 75 % now.  KU runs per lane are in flight per pass.
    const bool flat = MUON_MOM_FLAT && md.vec_ok && md.ld_grad == C && (!has_mom || md.ld_mom == C) && ldu == C;
    if (flat) {
        const int64_t e0 = int64_t(un.r0) * C;
        const int n4 = (rows * C) >> 2;   // runs of 4 in the unit (C % 8 == 0)
        const bool bf = md.io_dtype == 0;
        const GMEM char* gbase = gm(static_cast<const char*>(md.grad));
        GMEM float* mbase = gm(md.mom) + e0;
        for (int base = threadIdx.x; base < n4; base += kThreads * KU) {
            u32x4_t graw[KU];
            f32x4_t mv[KU];
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                const int q = base + u * kThreads;
                if (q < n4) {
                    const int64_t e = e0 + (int64_t(q) << 2);
                    if (bf) {
                        const u32x2_t w = mom_ld(reinterpret_cast<const GMEM u32x2_t*>(gbase + e * 2));
                        graw[u] = u32x4_t{w[0], w[1], 0u, 0u};
                    } else {
                        graw[u] = mom_ld(reinterpret_cast<const GMEM u32x4_t*>(gbase + e * 4));
                    }
                    if (has_mom) mv[u] = mom_ld(reinterpret_cast<const GMEM f32x4_t*>(mbase + (int64_t(q) << 2)));
                }
            }
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                const int q = base + u * kThreads;
                if (q >= n4) continue;
                float g[4];
                if (bf) {
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        g[2 * k] = __uint_as_float(graw[u][k] << 16);
                        g[2 * k + 1] = __uint_as_float(graw[u][k] & 0xFFFF0000u);
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) g[k] = __uint_as_float(graw[u][k]);
                }
                float uu[4];
                if (has_mom) {
                    f32x4_t m0 = mv[u];
#pragma unroll
                    for (int k = 0; k < 4; ++k) m0[k] = fmaf(beta, m0[k], g[k]);
                    mom_st(reinterpret_cast<GMEM f32x4_t*>(mbase + (int64_t(q) << 2)), m0);
#pragma unroll
                    for (int k = 0; k < 4; ++k) uu[k] = nest ? fmaf(beta, m0[k], g[k]) : m0[k];
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) uu[k] = g[k];
                }
                // squares summed as a tree, one dependent add into ss per run
                double sq[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) sq[k] = double(uu[k]) * double(uu[k]);
                ss += (sq[0] + sq[1]) + (sq[2] + sq[3]);
                const int64_t e = e0 + (int64_t(q) << 2);
                if (F32C) {
                    *gm(reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(ub) + e)) =
                        f32x4_t{uu[0], uu[1], uu[2], uu[3]};
                } else {
                    *gm(reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(ub) + e)) =
                        u32x2_t{pack_bf16x2(uu[0], uu[1]), pack_bf16x2(uu[2], uu[3])};
                }
            }
        }
    } else if (md.vec_ok) {
        // kU groups of 8 columns per thread per pass: every load of the pass is
        // issued before the first use, so each thread keeps kU x 48 bytes in
        // flight, as many as the flat path (this path's registers set the
        // kernel's register count, hence its occupancy, on both paths)
        constexpr int kU = KU / 2;
        const int gpr = C >> 3;  // groups of 8 columns per row
        const int total = rows * gpr;
        const bool bf = md.io_dtype == 0;
        const GMEM char* gbase = gm(static_cast<const char*>(md.grad));
        GMEM float* mbase = gm(md.mom);
        for (int base = threadIdx.x; base < total; base += kThreads * kU) {
            u32x4_t graw[kU][2];
            f32x4_t mv[kU][2];
            int64_t row[kU];
            int col[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int idx = base + u * kThreads;
                const int rr = idx < total ? idx / gpr : 0;
                row[u] = un.r0 + rr;
                col[u] = (idx - rr * gpr) << 3;
                if (idx < total) {
                    if (bf) {
                        graw[u][0] = mom_ld(reinterpret_cast<const GMEM u32x4_t*>(gbase + (row[u] * md.ld_grad + col[u]) * 2));
                    } else {
                        const GMEM u32x4_t* gp = reinterpret_cast<const GMEM u32x4_t*>(gbase + (row[u] * md.ld_grad + col[u]) * 4);
                        graw[u][0] = mom_ld(gp);
                        graw[u][1] = mom_ld(gp + 1);
                    }
                    if (has_mom) {
                        const GMEM f32x4_t* mp = reinterpret_cast<const GMEM f32x4_t*>(mbase + row[u] * md.ld_mom + col[u]);
                        mv[u][0] = mom_ld(mp);
                        mv[u][1] = mom_ld(mp + 1);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int idx = base + u * kThreads;
                if (idx >= total) continue;
                float g[8];
                if (bf) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        g[2 * q] = __uint_as_float(graw[u][0][q] << 16);
                        g[2 * q + 1] = __uint_as_float(graw[u][0][q] & 0xFFFF0000u);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        g[q] = __uint_as_float(graw[u][0][q]);
                        g[4 + q] = __uint_as_float(graw[u][1][q]);
                    }
                }
                float uu[8];
                if (has_mom) {
                    f32x4_t m0 = mv[u][0], m1 = mv[u][1];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        m0[q] = fmaf(beta, m0[q], g[q]);
                        m1[q] = fmaf(beta, m1[q], g[4 + q]);
                    }
                    GMEM f32x4_t* mp = reinterpret_cast<GMEM f32x4_t*>(mbase + row[u] * md.ld_mom + col[u]);
                    mom_st(mp, m0);
                    mom_st(mp + 1, m1);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        uu[q] = nest ? fmaf(beta, m0[q], g[q]) : m0[q];
                        uu[4 + q] = nest ? fmaf(beta, m1[q], g[4 + q]) : m1[q];
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 8; ++q) uu[q] = g[q];
                }
                double sq[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) sq[q] = double(uu[q]) * double(uu[q]);
                ss += ((sq[0] + sq[1]) + (sq[2] + sq[3])) + ((sq[4] + sq[5]) + (sq[6] + sq[7]));
                if (F32C) {
                    GMEM f32x4_t* up = gm(reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(ub) + row[u] * ldu + col[u]));
                    up[0] = f32x4_t{uu[0], uu[1], uu[2], uu[3]};
                    up[1] = f32x4_t{uu[4], uu[5], uu[6], uu[7]};
                } else {
                    u32x4_t w;
#pragma unroll
                    for (int q = 0; q < 4; ++q) w[q] = pack_bf16x2(uu[2 * q], uu[2 * q + 1]);
                    *gm(reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(ub) + row[u] * ldu + col[u])) = w;
                }
            }
        }
    } else {
        const int total = rows * C;
        for (int idx = threadIdx.x; idx < total; idx += kThreads) {
            const int rr = idx / C;
            const int c = idx - rr * C;
            const int64_t r = un.r0 + rr;
            const float g = load_elem(md.grad, r * md.ld_grad + c, md.io_dtype);
            float u = g;
            if (has_mom) {
                GMEM float* mp = gm(md.mom + r * md.ld_mom + c);
                const float mn = fmaf(beta, *mp, g);
                *mp = mn;
                u = nest ? fmaf(beta, mn, g) : mn;
            }
            ss = fma(double(u), double(u), ss);
            if (F32C)
                gm(reinterpret_cast<float*>(ub))[r * ldu + c] = u;
            else
                gm(reinterpret_cast<uint16_t*>(ub))[r * ldu + c] = f32_to_bf16(u);
        }
    }
    const double tot = block_sum(ss, red);
    if (threadIdx.x == 0) ka.partials[blockIdx.x] = tot;
}

// ---------------------------------------------------------------------------
// per-matrix norm: fixed-order double sum of the unit partials, and the
// power-of-two range of the operand copy (NormScale)
// ---------------------------------------------------------------------------
constexpr int kSafeExp = 30;   // nu in [2^-30, 2^30]: operand copy kept as u

__global__ __launch_bounds__(kThreads) void finalize_norm_kernel(const MatDesc* __restrict__ mats,
                                                                 const double* __restrict__ partials,
                                                                 NormScale* __restrict__ norm, float eps) {
    __shared__ double red[kThreads];
    const MatDesc& md = mats[blockIdx.x];
    double s = 0.0;
    for (int i = threadIdx.x; i < md.nunits; i += kThreads) s += partials[md.unit0 + i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
        if (int(threadIdx.x) < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double nu = sqrt(red[0]);
        int k = 0;
        if (nu > 0.0 && nu < __builtin_inf() && (nu < ldexp(1.0, -kSafeExp) || nu > ldexp(1.0, kSafeExp)))
            k = ilogb(nu);
        const double inv = 1.0 / (nu + double(eps));
        NormScale ns;
        ns.inv = float(inv);
        ns.first = float(ldexp(inv, k));
        ns.k = k;
        ns.nu = float(nu);
        norm[blockIdx.x] = ns;
    }
}

// Operand copy of u -> u 2^-k for the entries whose norm lies outside the
// safe range (exact: a power-of-two scaling of values far from the ends of
// the exponent range).  Workgroups stride over the momentum-pass units; in
// the common case every unit's k is 0 and each workgroup only reads them.
__global__ __launch_bounds__(kThreads) void rescale_kernel(const Unit* __restrict__ units, int n_units,
                                                           const MatDesc* __restrict__ mats,
                                                           const NormScale* __restrict__ norm, char* ws) {
    for (int ui = blockIdx.x; ui < n_units; ui += gridDim.x) {
        const Unit un = units[ui];
        const int k = norm[un.mat].k;
        if (k == 0) continue;
        const MatDesc& md = mats[un.mat];
        const bool F32C = md.f32 != 0;
        const int C = md.C;
        const int total = (un.r1 - un.r0) * C;
        for (int idx = threadIdx.x; idx < total; idx += kThreads) {
            const int rr = idx / C;
            const int64_t i = int64_t(un.r0 + rr) * md.Cp + (idx - rr * C);
            if (F32C) {
                GMEM float* p = gm(reinterpret_cast<float*>(ws + md.off_u)) + i;
                *p = ldexpf(*p, -k);
            } else {
                GMEM uint16_t* p = gm(reinterpret_cast<uint16_t*>(ws + md.off_u)) + i;
                *p = f32_to_bf16(ldexpf(bf16_to_f32(*p), -k));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Newton-Schulz products
// ---------------------------------------------------------------------------

// Physical 16-byte chunk of logical chunk `ch` in LDS row `r` (8 chunks per row).
// Conflict-free for the fragment reads (8 consecutive rows, same chunk), the
// row-contiguous stores (one row, 8 chunks) and the transposed stores (rows
// 8 apart, same chunk).
__device__ __forceinline__ int swz(int r, int ch) { return ch ^ ((r ^ (r >> 3)) & 7); }

template <bool F32>
struct GemmCfg {
    static constexpr int BM = kTileF32;            // square output tiles
    static constexpr int EPC = F32 ? 4 : 8;        // elements per 16-byte chunk
    static constexpr int ES = F32 ? 4 : 2;         // element bytes
    static constexpr int BK = EPC * 8;             // k per block: 8 chunks per LDS row
    static constexpr int WM = BM / 2;              // 2 x 2 waves
    static constexpr int TI = WM / 16;             // 16 x 16 MFMA tiles per wave edge
    static constexpr int KC_PER_T = BM * 8 / kThreads;       // row-contiguous loader chunks per thread
    static constexpr int KS_BLK = 8 * (BM / EPC);            // EPC x EPC blocks, k-strided loader
    static constexpr int KS_PER_T = (KS_BLK + kThreads - 1) / kThreads;
    static constexpr int NREG = (KC_PER_T > KS_PER_T * EPC) ? KC_PER_T : KS_PER_T * EPC;
};

// Load one BM x BK operand slab (rows [row0, row0 + BM), k [k0, k0 + BK)) into registers.
// kc: element (row, k) at base[row * ld + k]; otherwise at base[k * ld + row].
template <bool F32>
__device__ __forceinline__ void gload(const char* __restrict__ base, int64_t ld, bool kc, int row0, int k0,
                                      u32x4_t* reg) {
    using G = GemmCfg<F32>;
    if (kc) {
#pragma unroll
        for (int p = 0; p < G::KC_PER_T; ++p) {
            const int q = threadIdx.x + kThreads * p;
            const int r = q >> 3, ch = q & 7;
            reg[p] = *reinterpret_cast<const u32x4_t*>(base + (int64_t(row0 + r) * ld + k0 + ch * G::EPC) * G::ES);
        }
    } else {
#pragma unroll
        for (int p = 0; p < G::KS_PER_T; ++p) {
            const int q = threadIdx.x + kThreads * p;
            if (q < G::KS_BLK) {
                const int kb = q / (G::BM / G::EPC), rb = q % (G::BM / G::EPC);
#pragma unroll
                for (int i = 0; i < G::EPC; ++i)
                    reg[p * G::EPC + i] = *reinterpret_cast<const u32x4_t*>(
                        base + (int64_t(k0 + kb * G::EPC + i) * ld + row0 + rb * G::EPC) * G::ES);
            }
        }
    }
}

// Store the registers of gload into an LDS slab laid out [row][chunk].
template <bool F32>
__device__ __forceinline__ void sstore(u32x4_t* __restrict__ s, bool kc, const u32x4_t* reg) {
    using G = GemmCfg<F32>;
    if (kc) {
#pragma unroll
        for (int p = 0; p < G::KC_PER_T; ++p) {
            const int q = threadIdx.x + kThreads * p;
            const int r = q >> 3, ch = q & 7;
            s[r * 8 + swz(r, ch)] = reg[p];
        }
    } else {
#pragma unroll
        for (int p = 0; p < G::KS_PER_T; ++p) {
            const int q = threadIdx.x + kThreads * p;
            if (q < G::KS_BLK) {
                const int kb = q / (G::BM / G::EPC), rb = q % (G::BM / G::EPC);
                const u32x4_t* v = reg + p * G::EPC;
                if (F32) {
                    // 4 x 4 floats: w[e][i] = v[i][e]
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = rb * 4 + e;
                        s[r * 8 + swz(r, kb)] = u32x4_t{v[0][e], v[1][e], v[2][e], v[3][e]};
                    }
                } else {
                    // 8 x 8 bf16: column e of the block gathers the 8 k values
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int qd = e >> 1;
                        u32x4_t w;
#pragma unroll
                        for (int pp = 0; pp < 4; ++pp) {
                            const uint32_t lo = v[2 * pp][qd], hi = v[2 * pp + 1][qd];
                            w[pp] = (e & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
                        }
                        const int r = rb * 8 + e;
                        s[r * 8 + swz(r, kb)] = w;
                    }
                }
            }
        }
    }
}

// Operands of one Newton-Schulz product for one matrix.  "kc": element (row, k)
// at ptr[row * ld + k]; otherwise at ptr[k * ld + row].
struct Operands {
    const char* a;
    const char* b;
    int64_t lda, ldb;
    bool a_kc, b_kc;
    int K;
    int64_t off_cur;   // workspace offset of the current X operand copy
};

// X lives in the caller's stored orientation throughout (R x C, leading
// dimension Cp): for a transposed matrix (R > C) the iteration variable
// X = U^T is kept as X^T.  Then
//   GRAM  A = X X^T      : rows of X along k (kc), or columns of X^T (ks)
//   POLY  A A = A A^T    : rows of A (A symmetric)
//   AXPY  X' = a X + B X : rows of B with columns of X (ks); transposed
//                          X'^T = a X^T + X^T B: rows of X^T with rows of B
//                          (B symmetric), output tile in the stored orientation.
template <int KIND>
__device__ __forceinline__ Operands resolve_operands(const MatDesc& md, const PhaseArgs& pa) {
    Operands o;
    const char* ws = pa.ws;
    const int it = pa.iter;
    // current X: the momentum pass's copy of u on the first iteration,
    // afterwards the operand copy written by the previous iteration
    o.off_cur = (it == 1) ? md.off_u : (((it - 2) & 1) ? md.off_xb1 : md.off_xb0);
    const bool trans = md.trans != 0;
    if (KIND == PH_GRAM) {
        o.K = md.n;
        o.a = o.b = ws + o.off_cur;
        o.lda = o.ldb = md.Cp;
        o.a_kc = o.b_kc = !trans;
    } else if (KIND == PH_POLY) {
        o.K = md.m;
        o.a = o.b = ws + md.off_a;
        o.lda = o.ldb = md.mp;
        o.a_kc = o.b_kc = true;
    } else {
        o.K = md.m;
        if (!trans) {
            o.a = ws + md.off_b;
            o.lda = md.mp;
            o.a_kc = true;
            o.b = ws + o.off_cur;
            o.ldb = md.Cp;
            o.b_kc = false;
        } else {
            o.a = ws + o.off_cur;
            o.lda = md.Cp;
            o.a_kc = true;
            o.b = ws + md.off_b;
            o.ldb = md.mp;
            o.b_kc = true;
        }
    }
    return o;
}

// Epilogue of one output tile.  acc[i][j][e] is element
// (gr0 + 16 i + e, gc0 + 16 j) of the NS-orientation product (MFMA 16x16
// output layout: lane holds column lane & 15 and rows 4 (lane >> 4) + e).
template <int KIND, bool F32, int TI>
__device__ __forceinline__ void epilogue(const MatDesc& md, const Tile& t, const PhaseArgs& pa,
                                         const f32x4_t (&acc)[TI][TI], int gr0, int gc0, int64_t off_cur) {
    char* const ws = pa.ws;
    const int it = pa.iter;
    constexpr int ODT = F32 ? 1 : 0;  // workspace element type
    if (KIND == PH_GRAM || KIND == PH_POLY) {
        const int m = md.m;
        const int64_t ld = md.mp;
        char* outp = ws + (KIND == PH_GRAM ? md.off_a : md.off_b);
        const char* ain = ws + md.off_a;
        float scl = 1.f;
        if (KIND == PH_GRAM && it == 1) {
            const float s = pa.norm[t.mat].first;
            scl = s * s;
        }
        const bool diag = t.ti == t.tj;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TI; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = gr0 + 16 * i + e, c = gc0 + 16 * j;
                    // upper triangle (r <= c on diagonal tiles) written twice: (r, c) and (c, r)
                    if (r < m && c < m && (!diag || r <= c)) {
                        float v = acc[i][j][e];
                        if (KIND == PH_GRAM)
                            v *= scl;
                        else
                            v = pa.b * load_elem(ain, int64_t(r) * ld + c, ODT) + pa.c * v;
                        store_elem(outp, int64_t(r) * ld + c, ODT, v);
                        if (r != c) store_elem(outp, int64_t(c) * ld + r, ODT, v);
                    }
                }
    } else {
        // AXPY output tiles cover the stored R x C shape (see resolve_operands)
        const int R = md.R, C = md.C;
        const int64_t ldx = md.Cp;
        const float alpha = (it == 1) ? pa.norm[t.mat].first : 1.f;
        const int k0 = (it == 1) ? pa.norm[t.mat].k : 0;   // the master term is u: scale it like the copy
        const bool nest = pa.nesterov != 0;
        const float* xm = reinterpret_cast<const float*>(ws + off_cur);   // fp32 mode: X itself
        char* xb_next = ws + (((it - 1) & 1) ? md.off_xb1 : md.off_xb0);
        const float wdec = 1.f - pa.lr * pa.wd;
        const float step = pa.lr * md.shape_scale;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TI; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = gr0 + 16 * i + e, c = gc0 + 16 * j;
                    if (r < R && c < C) {
                        const float master =
                            (it == 1) ? ldexpf(u_at(md, r, c, pa.beta, nest), -k0) : xm[int64_t(r) * ldx + c];
                        const float v = alpha * fmaf(pa.a, master, acc[i][j][e]);
                        if (KIND == PH_AXPY) {
                            store_elem(xb_next, int64_t(r) * ldx + c, ODT, v);
                        } else {
                            if (md.has_param) {
                                const int64_t pi = int64_t(r) * md.ld_param + c;
                                const float w = load_elem(md.param, pi, md.io_dtype);
                                store_elem(md.param, pi, md.io_dtype, fmaf(-step, v, w * wdec));
                            }
                            if (md.upd) gm(md.upd)[int64_t(r) * md.ld_upd + c] = v;
                        }
                    }
                }
    }
}

// Workgroup b runs on XCD b % 8.  Tile lists hold 8 equal chunks, chunk x
// being the tiles XCD x runs in dispatch order; padding entries have mat < 0.
__device__ __forceinline__ int xcd_tile(int bid, int n_tiles) { return (bid & 7) * (n_tiles >> 3) + (bid >> 3); }

// ---------------------------------------------------------------------------
// fp32 validation-mode GEMM: 128 x 128 tiles, register-staged loads
// ---------------------------------------------------------------------------
template <int KIND, bool F32>
__global__ __launch_bounds__(kThreads) void ns_gemm_kernel(const Tile* __restrict__ tiles,
                                                           const MatDesc* __restrict__ mats, PhaseArgs pa) {
    using G = GemmCfg<F32>;
    constexpr int BM = G::BM, BK = G::BK, TI = G::TI, WM = G::WM;
    __shared__ u32x4_t sA[2][BM * 8];
    __shared__ u32x4_t sB[2][BM * 8];

    const Tile t = tiles[xcd_tile(blockIdx.x, gridDim.x)];
    if (t.mat < 0) return;
    const MatDesc& md = mats[t.mat];
    const Operands op = resolve_operands<KIND>(md, pa);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wr = (wave >> 1) * WM, wc = (wave & 1) * WM;
    const int row_a0 = t.ti * BM, row_b0 = t.tj * BM;

    f32x4_t acc[TI][TI];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TI; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t ra[G::NREG], rb[G::NREG];
    const int nk = (op.K + BK - 1) / BK;
    gload<F32>(op.a, op.lda, op.a_kc, row_a0, 0, ra);
    gload<F32>(op.b, op.ldb, op.b_kc, row_b0, 0, rb);
    sstore<F32>(sA[0], op.a_kc, ra);
    sstore<F32>(sB[0], op.b_kc, rb);
    __syncthreads();

    for (int kb = 0; kb < nk; ++kb) {
        const int cur = kb & 1;
        const bool more = kb + 1 < nk;
        if (more) {
            gload<F32>(op.a, op.lda, op.a_kc, row_a0, (kb + 1) * BK, ra);
            gload<F32>(op.b, op.ldb, op.b_kc, row_b0, (kb + 1) * BK, rb);
        }
        const u32x4_t* __restrict__ cA = sA[cur];
        const u32x4_t* __restrict__ cB = sB[cur];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int ch = 4 * s + (lane >> 4);
            u32x4_t fa[TI], fb[TI];
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                const int r = wr + 16 * i + (lane & 15);
                fa[i] = cA[r * 8 + swz(r, ch)];
                const int c = wc + 16 * i + (lane & 15);
                fb[i] = cB[c * 8 + swz(c, ch)];
            }
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TI; ++j) {
                    if (F32) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(fa[i][e]),
                                                                             __uint_as_float(fb[j][e]), acc[i][j], 0, 0, 0);
                    } else {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fa[i]),
                                                                            __builtin_bit_cast(bf16x8_t, fb[j]),
                                                                            acc[i][j], 0, 0, 0);
                    }
                }
        }
        if (more) {
            sstore<F32>(sA[cur ^ 1], op.a_kc, ra);
            sstore<F32>(sB[cur ^ 1], op.b_kc, rb);
        }
        __syncthreads();
    }
    epilogue<KIND, F32, TI>(md, t, pa, acc, row_a0 + wr + 4 * (lane >> 4), row_b0 + wc + (lane & 15), op.off_cur);
}

// ---------------------------------------------------------------------------
// bf16 GEMM: BM x BM tiles (BM = 128), 4 waves of (BM/2)^2 outputs each, k
// blocks of 64 through a ring of two LDS stages (64 KB: two workgroups per CU).
//
// Global -> LDS uses direct-to-LDS 16-byte loads (no staging registers),
// issued from inline asm with explicit vmcnt waits, so each stage is waited
// for exactly when it is consumed.  Row-contiguous operands sit in LDS as
// [row][8 chunks of 8 k] (chunk XOR row & 7) and feed the MFMA with
// ds_read_b128; k-strided operands sit as [k][BM] (chunks swizzled by kswz) and
// feed it with ds_read_b64_tr_b16, which hands lane j of each 16-lane group
// column j of a 4 x 16 block.  Operand layouts are template parameters so the
// k loop is straight-line code.
// ---------------------------------------------------------------------------
typedef short i16x4_t __attribute__((ext_vector_type(4)));
#ifndef LDS_AS
#define LDS_AS __attribute__((address_space(3)))
#endif

template <int BM, int BK_ = 64>
struct BfCfg {
    static constexpr int BK = BK_;                // k per LDS stage (32 or 64)
    // LDS stages (ring; the epilogue reuses them), within 64 KB so two
    // workgroups share a CU
    static constexpr int LDS_BUDGET = 64 * 1024;
    static constexpr int NST = LDS_BUDGET / (2 * BM * BK * 2) > 8 ? 8 : LDS_BUDGET / (2 * BM * BK * 2);
    static constexpr int CPK = BK / 8;            // 16-byte chunks per [row][BK] row
    static constexpr int WT = BM / 2;             // wave tile edge
    static constexpr int TI = WT / 16;            // MFMA tiles per wave edge
    static constexpr int OPB = BM * BK * 2;       // LDS bytes of one operand stage
    static constexpr int STB = 2 * OPB;           // LDS bytes of one stage (A then B)
    static constexpr int LPW = OPB / 1024 / 4;    // 1 KB loads per wave per operand per stage
    static constexpr int LPS = 2 * LPW;           // loads per wave per stage
    static constexpr int CPR = BM / 8;            // 16-byte chunks per [k][BM] row
    static constexpr int RPK = 64 / CPR;          // [k][BM] rows per 1 KB
};
constexpr int kBK = 64;

// Swizzle of the 16-byte chunks of a [k][BM] LDS row.  A ds_read_b64_tr_b16
// group of 16 lanes reads rows k0..k0+3 (4 rows x 32 bytes): bits 1-2 spread
// those rows over one 128-byte window; bit 3 puts the neighbouring 16-lane
// group (rows 8 further on) in the other 128-byte half of the bank space.
__device__ __forceinline__ int kswz(int k) { return ((2 * k) & 6) | ((((k >> 3) ^ (k >> 2)) & 1) << 3); }

// Swizzle of the 16-byte chunks of a [row][CPK chunks] LDS row: the 8 rows a
// ds_read_b128 phase touches land on 8 distinct 16-byte bank groups.
template <int CPK>
__device__ __forceinline__ int kcswz(int r) { return CPK == 8 ? (r & 7) : ((r >> 1) & 3); }

#ifndef MUON_LDS_DMA16S
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from global memory straight into LDS, from address
// sbase + voff (sbase wave-uniform, in SGPRs; voff per lane): lane L's bytes
// land at lds + 16 L (lds must be wave-uniform).  Nothing is returned in
// registers; completion is tracked by vmcnt and waited for with vm_wait().
__device__ __forceinline__ void lds_dma16s(const char* sbase, uint32_t voff, char* lds) {
    const uint32_t a = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS char*)lds)));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(a), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
#pragma clang diagnostic pop
#else
#define lds_dma16s MUON_LDS_DMA16S
#endif

// s_waitcnt vmcnt(N), no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Issue the loads of one operand of one stage.  Row-contiguous (KC) operand:
// 1 KB block blk holds rows blk * 64/CPK ..; a lane's row within the block and
// its swizzled chunk do not depend on blk (the swizzle's period divides the
// block), so one per-lane offset serves every block and only the SGPR base
// moves.  k-strided operand: 1 KB block blk holds k rows blk * RPK ..; the
// chunk swizzle depends on k, so the per-lane offset is recomputed per block.
template <int BM, int BK, bool KC>
__device__ __forceinline__ void issue_operand(char* __restrict__ lds, const char* __restrict__ g, int64_t ld, int row0,
                                              int k0, int wave, int lane) {
    using C = BfCfg<BM, BK>;
    if (KC) {
        constexpr int RB = 64 / C::CPK;
        const int rl = lane / C::CPK;
        const int c = (lane % C::CPK) ^ kcswz<C::CPK>(rl);
        const uint32_t voff = uint32_t(rl * ld * 2 + c * 16);
#pragma unroll
        for (int q = 0; q < C::LPW; ++q) {
            const int blk = wave * C::LPW + q;
            lds_dma16s(g + (int64_t(row0 + blk * RB) * ld + k0) * 2, voff, lds + blk * 1024);
        }
    } else {
        const int kl = lane / C::CPR;
#pragma unroll
        for (int q = 0; q < C::LPW; ++q) {
            const int blk = wave * C::LPW + q;
            const int c = (lane % C::CPR) ^ kswz(blk * C::RPK + kl);
            const uint32_t voff = uint32_t(kl * ld * 2 + c * 16);
            lds_dma16s(g + (int64_t(k0 + blk * C::RPK) * ld + row0) * 2, voff, lds + blk * 1024);
        }
    }
}

// One MFMA operand fragment (8 k values k = 32 s + 8 (lane >> 4) + e of
// row/column rc16 + (lane & 15)) from one operand stage.
template <int BM, int BK, bool KC>
__device__ __forceinline__ bf16x8_t frag(const char* __restrict__ lds, int rc16, int s, int lane) {
    using C = BfCfg<BM, BK>;
    if (KC) {
        const int r = rc16 + (lane & 15);
        const int c = (4 * s + (lane >> 4)) ^ kcswz<C::CPK>(r);
        return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(lds + r * (C::CPK * 16) + c * 16));
    }
    const int i = lane & 15;
    const int n = rc16 + 4 * (i & 3);
    i16x4_t h[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int k = 32 * s + 8 * (lane >> 4) + 4 * hh + (i >> 2);
        const int c = (n >> 3) ^ kswz(k);
        const char* p = lds + k * (BM * 2) + c * 16 + (n & 7) * 2;
        h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(p));
    }
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int BM, int BK, bool AKC, bool BKC>
__device__ __forceinline__ void issue_stage(char* __restrict__ st, const Operands& op, int row_a0, int row_b0, int k0,
                                            int wave, int lane) {
    issue_operand<BM, BK, AKC>(st, op.a, op.lda, row_a0, k0, wave, lane);
    issue_operand<BM, BK, BKC>(st + BfCfg<BM, BK>::OPB, op.b, op.ldb, row_b0, k0, wave, lane);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1, so
// array indices derived from I stay constant whatever the unroller decides.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <int TI>
struct EpiGeom {
    static constexpr int WT = TI * 16;    // wave tile edge
    static constexpr int LDW = WT + 4;    // padded LDS row (floats)
    static constexpr int NQ = WT / 16;    // 4-element runs per lane per band
};

template <int TI>
__device__ __forceinline__ void stage_band(float* __restrict__ stg, const f32x4_t (&acc)[TI][TI], int i, int lane) {
    constexpr int LDW = EpiGeom<TI>::LDW;
    const int g = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int j = 0; j < TI; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) stg[(4 * g + e) * LDW + 16 * j + c16] = acc[i][j][e];
}

// Row-major pass geometry: run q of a lane covers band row lr, columns lc..lc+3.
template <int TI>
__device__ __forceinline__ void row_run(int q, int lane, int& lr, int& lc) {
    constexpr int WT = EpiGeom<TI>::WT;
    const int idx = q * 256 + lane * 4;
    lr = idx / WT;
    lc = idx % WT;
}

// The bf16 copy of the master X that an AXPY output tile needs passes through
// LDS as operand data during one k block (128-wide tiles: a wave's 64 x 64
// quadrant is exactly one 64-deep block).  HiCap keeps it, in the epilogue's
// run order (band i, run q: row 16 i + lr, columns lc..lc+3), so the epilogue
// does not read it again from HBM.  CAP 1: X is the k-strided B operand
// ([k][BM], quadrant rows = k); CAP 2: X is the row-contiguous A operand
// ([row][k], quadrant columns = k).  CAP 3: the same for POLY's own A operand
// (A (r, c) for its b A term), in the swapped accumulator layout.
template <int TI>
struct HiCap {
    static constexpr int N = TI * 16 == 64 ? TI : 1;   // only quadrants of one 64-deep k block capture
    u32x2_t v[N][N];
    int kb;   // k block holding the quadrant
};

template <int BM, int BK, int CAP, int TI>
__device__ __forceinline__ void capture_hi(const char* __restrict__ st, HiCap<TI>& cap, int wr, int wc, int lane) {
    using C = BfCfg<BM, BK>;
    static_for<0, TI>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
#pragma unroll
        for (int q = 0; q < TI; ++q) {
            int lr, lc;
            row_run<TI>(q, lane, lr, lc);
            int off;
            if constexpr (CAP == 1) {
                const int k = 16 * i + lr, n = wc + lc;
                off = C::OPB + k * (BM * 2) + (((n >> 3) ^ kswz(k)) << 4) + (n & 7) * 2;
            } else if constexpr (CAP == 2) {
                const int r = wr + 16 * i + lr, k = lc;
                off = r * (C::CPK * 16) + (((k >> 3) ^ kcswz<C::CPK>(r)) << 4) + (k & 7) * 2;
            } else {   // CAP 3: swapped accumulator layout (row 16 i + (lane & 15), columns 16 q + 4 (lane >> 4) ..)
                const int r = wr + 16 * i + (lane & 15), k = 16 * q + 4 * (lane >> 4);
                off = r * (C::CPK * 16) + (((k >> 3) ^ kcswz<C::CPK>(r)) << 4) + (k & 7) * 2;
            }
            cap.v[i][q] = *reinterpret_cast<const u32x2_t*>(st + off);
        }
    });
}

// SWAP: feed the MFMA (B fragment, A fragment), so each lane accumulates 4
// consecutive output columns of one row instead of 4 rows of one column.
struct NoPre {
    __device__ __forceinline__ void operator()() const {}
};

// pre(): called once, at the start of the last k block (after its operands
// landed), so an epilogue can issue its first global loads behind the last MFMAs.
template <int BM, int BK, bool AKC, bool BKC, bool SWAP, int CAP = 0, class Pre = NoPre>
__device__ __forceinline__ void mainloop(char* __restrict__ smem, const Operands& op, int row_a0, int row_b0, int wave,
                                         int lane, f32x4_t (&acc)[BfCfg<BM, BK>::TI][BfCfg<BM, BK>::TI],
                                         HiCap<BfCfg<BM, BK>::TI>* cap = nullptr, const Pre& pre = Pre()) {
    using C = BfCfg<BM, BK>;
    constexpr int TI = C::TI;
    const int wr = (wave >> 1) * C::WT, wc = (wave & 1) * C::WT;
    const int nk = (op.K + C::BK - 1) / C::BK;
    // prologue: stages 0 .. NST-2
#pragma unroll
    for (int s = 0; s < C::NST - 1; ++s)
        if (s < nk) issue_stage<BM, BK, AKC, BKC>(smem + s * C::STB, op, row_a0, row_b0, s * C::BK, wave, lane);
    for (int kb = 0; kb < nk; ++kb) {
        // stage kb has landed once at most (stages issued after it) x LPS loads are pending
        const int ahead = nk - 1 - kb;
        const int pend = ahead < C::NST - 2 ? ahead : C::NST - 2;
        static_for<0, C::NST - 1>([&](auto pc) {
            constexpr int p = decltype(pc)::value;
            if (pend == p) vm_wait<p * C::LPS>();
        });
        __syncthreads();   // every wave's share of stage kb is in LDS; stage kb-1 is free
        if (kb + C::NST - 1 < nk)
            issue_stage<BM, BK, AKC, BKC>(smem + ((kb + C::NST - 1) % C::NST) * C::STB, op, row_a0, row_b0,
                                          (kb + C::NST - 1) * C::BK, wave, lane);
        const char* sa = smem + (kb % C::NST) * C::STB;
        const char* sb = sa + C::OPB;
        if constexpr (CAP != 0)
            if (kb == cap->kb) capture_hi<BM, BK, CAP, TI>(sa, *cap, wr, wc, lane);
        if constexpr (!std::is_same_v<Pre, NoPre>)
            if (kb == nk - 1) pre();
        // the block's two 32-deep steps: step 1's fragments are read from
        // LDS while step 0's MFMAs run (two fragment buffers; 1-2 % faster
        // than reading each step's fragments right before its MFMAs)
        static_assert(BK == 64, "two 32-deep steps per k block");
        constexpr int kReads = TI * ((AKC ? 1 : 2) + (BKC ? 1 : 2));
        bf16x8_t fa0[TI], fb0[TI], fa1[TI], fb1[TI];
#pragma unroll
        for (int i = 0; i < TI; ++i) fa0[i] = frag<BM, BK, AKC>(sa, wr + 16 * i, 0, lane);
#pragma unroll
        for (int j = 0; j < TI; ++j) fb0[j] = frag<BM, BK, BKC>(sb, wc + 16 * j, 0, lane);
        __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
#pragma unroll
        for (int i = 0; i < TI; ++i) fa1[i] = frag<BM, BK, AKC>(sa, wr + 16 * i, 1, lane);
#pragma unroll
        for (int j = 0; j < TI; ++j) fb1[j] = frag<BM, BK, BKC>(sb, wc + 16 * j, 1, lane);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TI; ++j)
                acc[i][j] = SWAP ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb0[j], fa0[i], acc[i][j], 0, 0, 0)
                                 : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa0[i], fb0[j], acc[i][j], 0, 0, 0);
        static_for<0, kReads>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                   // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, TI * TI / kReads > 0 ? TI * TI / kReads : 1, 0);  // MFMAs
        });
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TI; ++j)
                acc[i][j] = SWAP ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb1[j], fa1[i], acc[i][j], 0, 0, 0)
                                 : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa1[i], fb1[j], acc[i][j], 0, 0, 0);
    }
}


__device__ __forceinline__ void st4_bf16(void* p, f32x4_t v) {
    *gm(reinterpret_cast<u32x2_t*>(p)) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ void st4_io(void* p, int64_t i, int dt, bool vec, int nvalid, f32x4_t v) {
    if (vec) {
        if (dt == 0)
            st4_bf16(static_cast<uint16_t*>(p) + i, v);
        else
            *gm(reinterpret_cast<f32x4_t*>(static_cast<float*>(p) + i)) = v;
        return;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (q < nvalid) store_elem(p, i + q, dt, v[q]);
}

// The caller-buffer fields of one descriptor, copied into registers once per
// epilogue: read through the descriptor after the epilogue's own global stores,
// they would be reloaded (the compiler cannot rule out that a store hit the
// descriptor table), each reload costing a full wait on outstanding memory.
struct IoView {
    const void* grad;
    const float* mom;
    void* param;
    float* upd;
    int64_t ld_grad, ld_mom, ld_param, ld_upd;
    int dt;                     // storage dtype of param / grad
    bool has_mom, has_param, nest, vio;
};

__device__ __forceinline__ IoView io_view(const MatDesc& md, bool nest) {
    IoView v;
    v.grad = md.grad;
    v.mom = md.mom;
    v.param = md.param;
    v.upd = md.upd;
    v.ld_grad = md.ld_grad;
    v.ld_mom = md.ld_mom;
    v.ld_param = md.ld_param;
    v.ld_upd = md.ld_upd;
    v.dt = md.io_dtype;
    v.has_mom = md.has_mom != 0;
    v.has_param = md.has_param != 0;
    v.nest = nest;
    v.vio = md.vec_io != 0;
    return v;
}

// Epilogue through LDS.  Each wave stages its (16 x WT) row bands in fp32 in its
// own LDS region and reads them back as 4-element runs along rows (row-major
// pass) or down columns (column-major pass), so global traffic moves in 8- and
// 16-byte vectors along contiguous rows of the destination.  Every global value
// a band needs is loaded before the band is staged, and the next band's loads
// are issued before the current band is stored, so each lane keeps a band's
// worth of loads in flight.

// ---- AXPY: X' = alpha (a X + B X) on the stored R x C tile grid (see
// resolve_operands): fp32 master and bf16 operand copy, or on the last
// iteration O = X' applied to the weight: W = W (1 - lr wd) - lr s O and the
// optional fp32 copy of O.  Runs are 4 consecutive stored columns of one row.
struct AxpyCtx {
    const uint16_t* xhi;       // current X, bf16 (the operand copy this GEMM reads)
    uint8_t* xlo;              // X - hi in 8 bits (enc_lo8): with hi, the master copy of X
    uint16_t* xb_next;
    int64_t ldq;
    int R, C;
    bool vio;
    int k0;                    // first iteration: the operand copy holds u 2^-k0 (NormScale)
    float alpha, a, beta, wdec, step;
    IoView io;
};

// 4 consecutive elements of a caller buffer exactly as loaded (f32: 4 words;
// bf16: 2 words in [0], [1]).  Decoding happens where the values are used, so
// the wait for a load falls at its use, a band later, not right after issue.
__device__ __forceinline__ u32x4_t ld4_raw(const void* p, int64_t i, int dt, bool vec, int nvalid) {
    u32x4_t r = {0u, 0u, 0u, 0u};
    if (vec) {
        if (dt == 0) {
            const u32x2_t w = *gm(reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(p) + i));
            r[0] = w[0];
            r[1] = w[1];
        } else {
            r = *gm(reinterpret_cast<const u32x4_t*>(static_cast<const float*>(p) + i));
        }
        return r;
    }
    if (dt == 0) {
        const GMEM uint16_t* q = gm(static_cast<const uint16_t*>(p)) + i;
        uint32_t h[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (k < nvalid) h[k] = q[k];
        r[0] = h[0] | (h[1] << 16);
        r[1] = h[2] | (h[3] << 16);
    } else {
        const GMEM uint32_t* q = gm(static_cast<const uint32_t*>(p)) + i;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (k < nvalid) r[k] = q[k];
    }
    return r;
}

__device__ __forceinline__ f32x4_t dec4(u32x4_t r, int dt) {
    if (dt == 0)
        return f32x4_t{__uint_as_float(r[0] << 16), __uint_as_float(r[0] & 0xFFFF0000u),
                       __uint_as_float(r[1] << 16), __uint_as_float(r[1] & 0xFFFF0000u)};
    return f32x4_t{__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[2]), __uint_as_float(r[3])};
}

// Caller-buffer configuration of an AXPY epilogue: read from the descriptor at
// run time (IoRuntime), or fixed at compile time (IoFixed) for the interior
// fast path, where it removes every per-run branch on dtype and buffer presence.
struct IoRuntime {
    static constexpr bool fixed = false;
};
template <int DT, bool MOM, bool NEST, bool PARAM, bool UPD>
struct IoFixed {
    static constexpr bool fixed = true;
    static constexpr int dt = DT;
    static constexpr bool mom = MOM, nest = NEST, param = PARAM, upd = UPD;
};
template <class M>
__device__ __forceinline__ int io_dt(const IoView& v) { if constexpr (M::fixed) return M::dt; else return v.dt; }
template <class M>
__device__ __forceinline__ bool io_mom(const IoView& v) { if constexpr (M::fixed) return M::mom; else return v.has_mom; }
template <class M>
__device__ __forceinline__ bool io_nest(const IoView& v) { if constexpr (M::fixed) return M::nest; else return v.nest; }
template <class M>
__device__ __forceinline__ bool io_param(const IoView& v) { if constexpr (M::fixed) return M::param; else return v.has_param; }
template <class M>
__device__ __forceinline__ bool io_upd(const IoView& v) { if constexpr (M::fixed) return M::upd; else return v.upd != nullptr; }

// Raw operands of one band of the AXPY epilogue, per 4-element run:
//   ra: the master, hi words in [0..1] and lo words in [2..3] or, on the first
//       iteration, m' (g without a momentum buffer);  rb: g on the first
//       iteration with Nesterov;  rc: W on the last iteration.
template <int TI>
struct AxpyRaw {
    u32x4_t ra[EpiGeom<TI>::NQ], rb[EpiGeom<TI>::NQ], rc[EpiGeom<TI>::NQ];
};

// EDGE = false: the wave's whole tile lies inside R x C and every caller buffer
// allows 4-element vectors, so no access needs a bounds check or a scalar tail.
template <int TI, bool FIRST, bool LAST, bool EDGE, class M, bool CAPHI>
__device__ __forceinline__ void axpy_load(const AxpyCtx& x, const HiCap<TI>& cap, int row0, int col0, int lane,
                                          int band, AxpyRaw<TI>& w) {
#pragma unroll
    for (int q = 0; q < EpiGeom<TI>::NQ; ++q) {
        int lr, lc;
        row_run<TI>(q, lane, lr, lc);
        const int r = row0 + 16 * band + lr, c = col0 + lc;
        int nv = x.C - c;
        nv = nv > 4 ? 4 : nv;
        const bool in = !EDGE || (r < x.R && c < x.C);
        const bool vec = !EDGE || (x.vio && nv == 4);
        if (!FIRST) {   // padded buffers: in bounds
            const int64_t off = int64_t(r) * x.ldq + c;
            u32x2_t hi;
            if constexpr (CAPHI) hi = cap.v[band][q];
            else hi = *gm(reinterpret_cast<const u32x2_t*>(x.xhi + off));
            const uint32_t lo = *gm(reinterpret_cast<const uint32_t*>(x.xlo + off));
            w.ra[q] = u32x4_t{hi[0], hi[1], lo, 0u};
        } else {
            w.ra[q] = u32x4_t{0u, 0u, 0u, 0u};
            w.rb[q] = u32x4_t{0u, 0u, 0u, 0u};
            if (in) {
                if (io_mom<M>(x.io)) {
                    w.ra[q] = ld4_raw(x.io.mom, int64_t(r) * x.io.ld_mom + c, 1, vec, nv);
                    if (io_nest<M>(x.io))
                        w.rb[q] = ld4_raw(x.io.grad, int64_t(r) * x.io.ld_grad + c, io_dt<M>(x.io), vec, nv);
                } else {
                    w.ra[q] = ld4_raw(x.io.grad, int64_t(r) * x.io.ld_grad + c, io_dt<M>(x.io), vec, nv);
                }
            }
        }
        if (LAST) {
            w.rc[q] = u32x4_t{0u, 0u, 0u, 0u};
            if (io_param<M>(x.io) && in)
                w.rc[q] = ld4_raw(x.io.param, int64_t(r) * x.io.ld_param + c, io_dt<M>(x.io), vec, nv);
        }
    }
}

template <int TI, bool FIRST, bool LAST, bool EDGE, class M>
__device__ __forceinline__ void axpy_store(const AxpyCtx& x, const float* __restrict__ stg, int row0, int col0,
                                           int lane, int band, const AxpyRaw<TI>& w) {
    using E = EpiGeom<TI>;
#pragma unroll
    for (int q = 0; q < E::NQ; ++q) {
        int lr, lc;
        row_run<TI>(q, lane, lr, lc);
        const int r = row0 + 16 * band + lr, c = col0 + lc;
        if (EDGE && (r >= x.R || c >= x.C)) continue;
        int nv = x.C - c;
        nv = nv > 4 ? 4 : nv;
        f32x4_t mst;
        if (!FIRST) {
            mst = dec4(w.ra[q], 0);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                mst[k] += dec_lo8((w.ra[q][2] >> (8 * k)) & 0xFFu, w.ra[q][k >> 1] >> (16 * (k & 1)));
        } else if (io_mom<M>(x.io)) {
            mst = dec4(w.ra[q], 1);
            if (io_nest<M>(x.io)) {
                const f32x4_t g = dec4(w.rb[q], io_dt<M>(x.io));
#pragma unroll
                for (int k = 0; k < 4; ++k) mst[k] = fmaf(x.beta, mst[k], g[k]);
            }
        } else {
            mst = dec4(w.ra[q], io_dt<M>(x.io));
        }
        if (FIRST) {   // u on the operand copy's scale
#pragma unroll
            for (int k = 0; k < 4; ++k) mst[k] = ldexpf(mst[k], -x.k0);
        }
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stg + lr * E::LDW + lc);
        const f32x4_t o = x.alpha * (x.a * (mst + v));   // acc holds (B / a) X
        if (!LAST) {
            // X' = hi + lo: hi its bf16 rounding, lo the 8-bit code of the
            // (exact) remainder
            const int64_t off = int64_t(r) * x.ldq + c;
            uint16_t h[4];
            uint32_t l = 0u;
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
                h[q2] = f32_to_bf16(o[q2]);
                l |= enc_lo8(o[q2] - bf16_to_f32(h[q2]), h[q2]) << (8 * q2);
            }
            if (!EDGE || nv == 4) {
                // streaming stores: the next phase reads them once per tile
                // that needs them (2 % faster on the 124M set)
                __builtin_nontemporal_store(
                    u32x2_t{uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16)},
                    gm(reinterpret_cast<u32x2_t*>(x.xb_next + off)));
                __builtin_nontemporal_store(l, gm(reinterpret_cast<uint32_t*>(x.xlo + off)));
            } else {
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2)
                    if (q2 < nv) {
                        gm(x.xb_next)[off + q2] = h[q2];
                        gm(x.xlo)[off + q2] = uint8_t(l >> (8 * q2));
                    }
            }
        } else {
            const bool vec = !EDGE || (x.vio && nv == 4);
            if (io_param<M>(x.io)) {
                const f32x4_t wold = dec4(w.rc[q], io_dt<M>(x.io));
                f32x4_t wn;
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2) wn[q2] = fmaf(-x.step, o[q2], wold[q2] * x.wdec);
                st4_io(x.io.param, int64_t(r) * x.io.ld_param + c, io_dt<M>(x.io), vec, nv, wn);
            }
            if (io_upd<M>(x.io)) st4_io(x.io.upd, int64_t(r) * x.io.ld_upd + c, 1, vec, nv, o);
        }
    }
}

// PRE bands' raw operands arrive in wp (loaded during the last k block); with
// PRE = TI the epilogue issues no load at all.
template <int TI, bool FIRST, bool LAST, bool EDGE, class M, bool CAPHI, int PRE>
__device__ __forceinline__ void epi_axpy_body(const AxpyCtx& x, const HiCap<TI>& cap, const AxpyRaw<TI> (&wp)[PRE ? PRE : 1],
                                              const f32x4_t (&acc)[TI][TI], int row0, int col0, int lane,
                                              float* __restrict__ stg) {
    if constexpr (PRE == TI) {
        static_for<0, TI>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            stage_band<TI>(stg, acc, i, lane);
            axpy_store<TI, FIRST, LAST, EDGE, M>(x, stg, row0, col0, lane, i, wp[i]);
        });
        return;
    }
    AxpyRaw<TI> w[2];
    if constexpr (PRE > 0) w[0] = wp[0];
    else axpy_load<TI, FIRST, LAST, EDGE, M, CAPHI>(x, cap, row0, col0, lane, 0, w[0]);
    static_for<0, TI>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i + 1 < TI)   // one band ahead
            axpy_load<TI, FIRST, LAST, EDGE, M, CAPHI>(x, cap, row0, col0, lane, i + 1, w[(i + 1) & 1]);
        stage_band<TI>(stg, acc, i, lane);
        axpy_store<TI, FIRST, LAST, EDGE, M>(x, stg, row0, col0, lane, i, w[i & 1]);
    });
}

template <bool FIRST>
__device__ __forceinline__ AxpyCtx axpy_ctx(const MatDesc& md, const Tile& t, const PhaseArgs& pa) {
    AxpyCtx x;
    const int it = pa.iter;
    x.xhi = reinterpret_cast<const uint16_t*>(pa.ws + (((it - 2) & 1) ? md.off_xb1 : md.off_xb0));   // it >= 2
    x.xlo = reinterpret_cast<uint8_t*>(pa.ws + md.off_xlo);
    x.xb_next = reinterpret_cast<uint16_t*>(pa.ws + (((it - 1) & 1) ? md.off_xb1 : md.off_xb0));
    x.ldq = md.Cp;
    x.R = md.R;
    x.C = md.C;
    x.vio = md.vec_io != 0;
    x.alpha = FIRST ? pa.norm[t.mat].first : 1.f;
    x.k0 = FIRST ? pa.norm[t.mat].k : 0;
    x.a = pa.a;
    x.beta = pa.beta;
    x.wdec = 1.f - pa.lr * pa.wd;
    x.step = pa.lr * md.shape_scale;
    x.io = io_view(md, pa.nesterov != 0);
    return x;
}

// PRE: the first PRE bands' raw operands were loaded during the last k block (w0).
template <int TI, bool FIRST, bool LAST, bool CAPHI, int PRE>
__device__ __forceinline__ void epi_axpy(const AxpyCtx& x, const f32x4_t (&acc)[TI][TI], const HiCap<TI>& cap,
                                         const AxpyRaw<TI> (&w0)[PRE ? PRE : 1], int row0, int col0, int lane,
                                         float* __restrict__ stg) {
    constexpr int WT = EpiGeom<TI>::WT;
    if (!(x.vio && row0 + WT <= x.R && col0 + WT <= x.C)) {
        epi_axpy_body<TI, FIRST, LAST, true, IoRuntime, CAPHI, PRE>(x, cap, w0, acc, row0, col0, lane, stg);
        return;
    }
    // interior: pick the caller-buffer configuration at compile time
    const IoView& v = x.io;
    if constexpr (FIRST == LAST) {   // middle iterations read no caller buffer; both at once (one iteration) stays generic
        epi_axpy_body<TI, FIRST, LAST, false, IoRuntime, CAPHI, PRE>(x, cap, w0, acc, row0, col0, lane, stg);
    } else if constexpr (FIRST) {
        auto go = [&](auto dtc) __attribute__((always_inline)) {
            constexpr int D = decltype(dtc)::value;
            if (v.has_mom && !v.nest)
                epi_axpy_body<TI, true, false, false, IoFixed<D, true, false, false, false>, CAPHI, PRE>(x, cap, w0, acc, row0, col0, lane, stg);
            else if (v.has_mom)
                epi_axpy_body<TI, true, false, false, IoFixed<D, true, true, false, false>, CAPHI, PRE>(x, cap, w0, acc, row0, col0, lane, stg);
            else
                epi_axpy_body<TI, true, false, false, IoFixed<D, false, false, false, false>, CAPHI, PRE>(x, cap, w0, acc, row0, col0, lane, stg);
        };
        if (v.dt == 0) go(std::integral_constant<int, 0>{});
        else go(std::integral_constant<int, 1>{});
    } else {
        auto go = [&](auto dtc) __attribute__((always_inline)) {
            constexpr int D = decltype(dtc)::value;
            if (v.has_param && !v.upd)
                epi_axpy_body<TI, false, true, false, IoFixed<D, false, false, true, false>, CAPHI, PRE>(x, cap, w0, acc, row0, col0, lane, stg);
            else if (v.has_param)
                epi_axpy_body<TI, false, true, false, IoFixed<D, false, false, true, true>, CAPHI, PRE>(x, cap, w0, acc, row0, col0, lane, stg);
            else if (v.upd)
                epi_axpy_body<TI, false, true, false, IoFixed<D, false, false, false, true>, CAPHI, PRE>(x, cap, w0, acc, row0, col0, lane, stg);
            else
                epi_axpy_body<TI, false, true, false, IoRuntime, CAPHI, PRE>(x, cap, w0, acc, row0, col0, lane, stg);
        };
        if (v.dt == 0) go(std::integral_constant<int, 0>{});
        else go(std::integral_constant<int, 1>{});
    }
}

// ---- GRAM (A = s^2 X X^T) and POLY (B / a = (b A + c A A) / a): the upper
// triangle is written by a row pass and mirrored by a second pass, so both the
// stored matrix and its padding are exactly symmetric.
//
// The main loop runs with swapped MFMA operands, so each lane holds 4
// consecutive columns of one row: acc[i][j][e] = C[16 i + (lane & 15)]
// [16 j + 4 (lane >> 4) + e].  Row pass, straight from registers: combine
// (POLY: b A + c acc, A read in the same layout), round once, store 8 bytes
// along the row, and write the 4 values into the wave's transposed bf16 copy of
// its tile in LDS, T[c][r] (8-element blocks of r XOR-swizzled by c).  Mirror
// pass: rows of T are stored as 16-byte runs along the destination rows.
// Padding rows and columns hold zeros on both sides (the operands' padding is
// zero), so no access needs a bounds check; diagonal tiles write r <= c in the
// row pass and r < c in the mirror pass.
struct SymCtx {
    uint16_t* out;
    const uint16_t* ain;
    int64_t ldq;
    bool diag;
    float scl, b, c;
};

template <int TI>
struct SymGeom {
    static constexpr int WT = TI * 16;
    static constexpr int BPR = WT / 8;              // 8-element blocks per row of T
    static constexpr int NM = WT * BPR / 64;        // mirror runs per lane
    static constexpr int HM = BPR < 16 ? BPR - 1 : 15;
    static constexpr int T_BYTES = WT * WT * 2;     // transposed tile per wave
};

// T[c][r]: block r / 8 of row c stored at block (r / 8) ^ h(c)
template <int TI>
__device__ __forceinline__ int t_index(int c, int r) {
    const int h = (c >> 2) & SymGeom<TI>::HM;
    return c * SymGeom<TI>::WT + ((((r >> 3) ^ h) << 3) | (r & 7));
}

template <int TI>
__device__ __forceinline__ void sym_mirror(const SymCtx& x, const uint16_t* __restrict__ tt, int row0, int col0,
                                           int lane) {
    using G = SymGeom<TI>;
#pragma unroll
    for (int q = 0; q < G::NM; ++q) {
        const int u = q * 64 + lane;
        const int cl = u / G::BPR, blk = u % G::BPR;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(tt + t_index<TI>(cl, 8 * blk));
        const int r = row0 + 8 * blk, c = col0 + cl;   // destination (c, r..r+7)
        GMEM uint16_t* o = gm(x.out + int64_t(c) * x.ldq + r);
        if (!x.diag || r + 7 < c) {
            *reinterpret_cast<GMEM u32x4_t*>(o) = v;
        } else if (r < c) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (r + k < c) o[k] = uint16_t(v[k >> 1] >> (16 * (k & 1)));
        }
    }
}

template <int KIND, int TI, bool CAPA>
__device__ __forceinline__ void epi_sym(const MatDesc& md, const Tile& t, const PhaseArgs& pa,
                                        const f32x4_t (&acc)[TI][TI], const HiCap<TI>& cap, int row0, int col0,
                                        int lane, char* __restrict__ wlds) {
    constexpr bool POLY = KIND == PH_POLY;
    uint16_t* tt = reinterpret_cast<uint16_t*>(wlds);
    SymCtx x;
    x.out = reinterpret_cast<uint16_t*>(pa.ws + (KIND == PH_GRAM ? md.off_a : md.off_b));
    x.ain = reinterpret_cast<const uint16_t*>(pa.ws + md.off_a);
    x.ldq = md.mp;
    x.diag = t.ti == t.tj;
    x.scl = 1.f;
    if (KIND == PH_GRAM && pa.iter == 1) {
        const float sn = pa.norm[t.mat].first;
        x.scl = sn * sn;
    }
    // the bf16 AXPY accumulates on top of the unscaled master X, so POLY
    // stores B / a and AXPY scales the sum by a: X' = a (X + (B / a) X)
    x.b = pa.b / pa.a;
    x.c = pa.c / pa.a;
    const int l16 = lane & 15, g4 = 4 * (lane >> 4);
    u32x2_t av[TI][TI];
    if constexpr (POLY) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TI; ++j) {
                if constexpr (CAPA) av[i][j] = cap.v[i][j];   // kept from the operand stream
                else
                    av[i][j] = *gm(reinterpret_cast<const u32x2_t*>(x.ain + int64_t(row0 + 16 * i + l16) * x.ldq +
                                                                    col0 + 16 * j + g4));
            }
    }
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
        for (int j = 0; j < TI; ++j) {
            const int rl = 16 * i + l16, cl = 16 * j + g4;
            const u32x2_t& ava = av[i][j];
            f32x4_t w;
            if constexpr (POLY) {
                const f32x4_t a = dec4(u32x4_t{ava[0], ava[1], 0u, 0u}, 0);
                w = x.b * a + x.c * acc[i][j];
            } else {
                w = acc[i][j] * x.scl;
            }
            uint16_t h[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                h[k] = f32_to_bf16(w[k]);
                tt[t_index<TI>(cl + k, rl)] = h[k];
            }
            const int r = row0 + rl, c = col0 + cl;
            GMEM uint16_t* o = gm(x.out + int64_t(r) * x.ldq + c);
            if (!x.diag || r <= c) {
                *reinterpret_cast<GMEM u32x2_t*>(o) = u32x2_t{uint32_t(h[0]) | (uint32_t(h[1]) << 16),
                                                              uint32_t(h[2]) | (uint32_t(h[3]) << 16)};
            } else {
#pragma unroll
                for (int k = 1; k < 4; ++k)
                    if (r <= c + k) o[k] = h[k];
            }
        }
    }
    sym_mirror<TI>(x, tt, row0, col0, lane);   // same wave wrote tt: program order suffices
}

// ---------------------------------------------------------------------------
// Wide tiles for large matrices: 256 x 256 output tiles, one workgroup of 8
// waves per CU (two per SIMD), each wave a 128 x 64 block (8 x 4 MFMA tiles)
// instead of 64 x 64.  Per flop it reads a quarter fewer fragment bytes from
// LDS and streams half the operand bytes from L2 into LDS (the 128-wide
// kernel's two workgroups of four 64 x 64 waves need about 190 B/clk of LDS
// traffic per CU at the MFMA rate, more than the LDS delivers).  k blocks of
// 64 through two 64 KB LDS stages.  Every output element sums k in the same
// order as in the 128-wide kernel, so the two give bitwise equal results.
// The epilogues are the 128-wide kernel's, run on the wave's two 64 x 64
// halves, reading from memory what that kernel keeps from the operand stream
// (AXPY: the bf16 X; POLY: A), whose registers do not fit beside the 128
// accumulators.  The symmetric phases take the upper triangle in 256-wide
// tiles; in a diagonal tile the waves whose block lies wholly below the
// diagonal skip their MFMAs and epilogue.  (The planner gives wide tiles to
// the GRAM and the AXPY; POLY keeps its 128-wide kernel, which takes A from
// the operand stream.)
//
// WideCfg<TM, TN, BK, NST>: TM x TN tile, (TM / 128) x (TN / 64) waves, LDS
// stages of BK k (a ring of NST).  Measured alternative: 256 x 128 tiles of
// four waves, two workgroups per CU, three 32-deep stages each: slower than
// the 128-wide kernel.
// ---------------------------------------------------------------------------
template <int TM_, int TN_, int BK_, int NST_>
struct WideCfg {
    static constexpr int TM = TM_, TN = TN_, BK = BK_, NST = NST_;
    static constexpr int WR = TM / 128, WC = TN / 64;   // waves along rows and columns
    static constexpr int NW = WR * WC;
    static constexpr int THREADS = 64 * NW;
    static constexpr int OPA = TM * BK * 2, OPB = TN * BK * 2;   // LDS bytes of each operand stage
    static constexpr int STB = OPA + OPB;
    static constexpr int LPA = OPA / 1024 / NW, LPB = OPB / 1024 / NW;   // 1 KB loads per wave
    static constexpr int LPS = LPA + LPB;
    static_assert(LPA * 1024 * NW == OPA && LPB * 1024 * NW == OPB, "whole 1 KB loads per wave");
    static_assert(LPS <= 8, "the next stage's loads go out between the 8 MFMA rows of a step");
};
using WCfg = WideCfg<kTileWide, kTileWide, 64, 2>;

// One 1 KB load (block q of this wave's share) of a ROWS x BK operand stage,
// with the layouts and swizzles of issue_operand (a [k][ROWS] row of 512
// bytes maps to the banks exactly as a 256-byte one).
template <int ROWS, int BK, int NW, bool KC>
__device__ __forceinline__ void issue_operand_wide(char* __restrict__ lds, const char* __restrict__ g, int64_t ld,
                                                   int row0, int k0, int wave, int lane, int q) {
    constexpr int LPW = ROWS * BK * 2 / 1024 / NW;
    const int blk = wave * LPW + q;
    if (KC) {
        constexpr int CPK = BK / 8;
        constexpr int RB = 64 / CPK;
        const int rl = lane / CPK;
        const int c = (lane % CPK) ^ kcswz<CPK>(rl);
        const uint32_t voff = uint32_t(rl * ld * 2 + c * 16);
        lds_dma16s(g + (int64_t(row0 + blk * RB) * ld + k0) * 2, voff, lds + blk * 1024);
    } else {
        constexpr int CPR = ROWS / 8;
        constexpr int RPK = 64 / CPR;
        const int kl = lane / CPR;
        const int c = (lane % CPR) ^ kswz(blk * RPK + kl);
        const uint32_t voff = uint32_t(kl * ld * 2 + c * 16);
        lds_dma16s(g + (int64_t(k0 + blk * RPK) * ld + row0) * 2, voff, lds + blk * 1024);
    }
}

// Load q (operand A first, then operand B) of this wave's share of one stage.
template <class C, bool AKC, bool BKC>
__device__ __forceinline__ void issue_wide_load(char* __restrict__ st, const Operands& op, int row_a0, int row_b0,
                                                int k0, int wave, int lane, int q) {
    if (q < C::LPA) issue_operand_wide<C::TM, C::BK, C::NW, AKC>(st, op.a, op.lda, row_a0, k0, wave, lane, q);
    else issue_operand_wide<C::TN, C::BK, C::NW, BKC>(st + C::OPA, op.b, op.ldb, row_b0, k0, wave, lane, q - C::LPA);
}

// SWAP: feed the MFMA (B fragment, A fragment), the GRAM/POLY accumulator
// layout; idle: this wave's block needs no output (its loads still go out).
template <class C, bool AKC, bool BKC, bool SWAP>
__device__ __forceinline__ void mainloop_wide(char* __restrict__ smem, const Operands& op, int row_a0, int row_b0,
                                              int wave, int lane, f32x4_t (&acc)[8][4], bool idle = false) {
    const int wr = (wave / C::WC) * 128, wc = (wave % C::WC) * 64;
    const int nk = (op.K + C::BK - 1) / C::BK;
    // prologue: stages 0 .. NST-2
#pragma unroll
    for (int s = 0; s < C::NST - 1; ++s)
        if (s < nk) {
#pragma unroll
            for (int q = 0; q < C::LPS; ++q)
                issue_wide_load<C, AKC, BKC>(smem + s * C::STB, op, row_a0, row_b0, s * C::BK, wave, lane, q);
        }
    for (int kb = 0; kb < nk; ++kb) {
        // stage kb has landed once at most (stages issued after it) x LPS loads are pending
        const int ahead = nk - 1 - kb;
        const int pend = ahead < C::NST - 2 ? ahead : C::NST - 2;
        static_for<0, C::NST - 1>([&](auto pc) {
            constexpr int p = decltype(pc)::value;
            if (pend == p) vm_wait<p * C::LPS>();
        });
        __syncthreads();   // every wave's share of stage kb is in LDS; stage kb-1 is free
        const bool more = kb + C::NST - 1 < nk;
        char* nxt = smem + ((kb + C::NST - 1) % C::NST) * C::STB;
        const int k_nxt = (kb + C::NST - 1) * C::BK;
        const char* sa = smem + (kb % C::NST) * C::STB;
        const char* sb = sa + C::OPA;
#pragma unroll
        for (int s = 0; s < C::BK / 32; ++s) {
            bf16x8_t fa[8], fb[4];
#pragma unroll
            for (int i = 0; i < 8; ++i) fa[i] = frag<C::TM, C::BK, AKC>(sa, wr + 16 * i, s, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) fb[j] = frag<C::TN, C::BK, BKC>(sb, wc + 16 * j, s, lane);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // the next stage's loads go out one between each row of the
                // first step's MFMAs, not all at once after the barrier (about
                // 1 % faster)
                if (s == 0 && i < C::LPS && more)
                    issue_wide_load<C, AKC, BKC>(nxt, op, row_a0, row_b0, k_nxt, wave, lane, i);
                if (idle) continue;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = SWAP ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0)
                                     : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
            }
        }
    }
}

template <int KIND, bool FIRST>
__global__ __launch_bounds__(WCfg::THREADS, 8 / WCfg::NW) void ns_gemm_wide(const Tile* __restrict__ tiles,
                                                                            const MatDesc* __restrict__ mats,
                                                                            PhaseArgs pa, int n_tiles) {
    using C = WCfg;
    constexpr int TI = 4;   // epilogue quadrant of 4 x 4 MFMA tiles
    constexpr bool AXPY = KIND == PH_AXPY || KIND == PH_AXPY_LAST;
    constexpr int EPI_BYTES = AXPY ? 16 * (16 * TI + 4) * 4 : SymGeom<TI>::T_BYTES;   // per wave
    constexpr int LDS_BYTES = C::NST * C::STB;
    static_assert(C::NW * EPI_BYTES <= LDS_BYTES, "epilogue staging fits the operand stages");
    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const Tile t = tiles[xcd_tile(blockIdx.x, n_tiles)];
    if (t.mat < 0) return;
    const MatDesc& md = mats[t.mat];
    const Operands op = resolve_operands<KIND>(md, pa);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row_a0 = t.ti * C::TM, row_b0 = t.tj * C::TN;
    const int wr = (wave / C::WC) * 128, wc = (wave % C::WC) * 64;
    const int er0 = row_a0 + wr, ec0 = row_b0 + wc;

    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (AXPY) {
        if (op.a_kc && op.b_kc)   // transposed matrix: X^T B
            mainloop_wide<C, true, true, false>(smem, op, row_a0, row_b0, wave, lane, acc);
        else                      // B X
            mainloop_wide<C, true, false, false>(smem, op, row_a0, row_b0, wave, lane, acc);
        __syncthreads();   // operand stages are dead: reuse LDS for the epilogue
        constexpr bool LAST = KIND == PH_AXPY_LAST;
        const AxpyCtx x = axpy_ctx<FIRST>(md, t, pa);
        const HiCap<TI> cap{};   // not used: the epilogue reads the bf16 X from memory
        const AxpyRaw<TI> w0[1]{};
        float* stg = reinterpret_cast<float*>(smem + wave * EPI_BYTES);
        epi_axpy<TI, FIRST, LAST, false, 0>(x, reinterpret_cast<const f32x4_t(&)[TI][TI]>(acc[0]), cap, w0, er0, ec0,
                                            lane, stg);
        epi_axpy<TI, FIRST, LAST, false, 0>(x, reinterpret_cast<const f32x4_t(&)[TI][TI]>(acc[4]), cap, w0, er0 + 64,
                                            ec0, lane, stg);
    } else {
        // GRAM (kc, kc) or, for transposed matrices, (ks, ks); POLY (kc, kc)
        const bool idle = ec0 + 63 < er0;   // wholly below the diagonal (diagonal tiles only)
        if (op.a_kc && op.b_kc)
            mainloop_wide<C, true, true, true>(smem, op, row_a0, row_b0, wave, lane, acc, idle);
        else
            mainloop_wide<C, false, false, true>(smem, op, row_a0, row_b0, wave, lane, acc, idle);
        __syncthreads();   // operand stages are dead: reuse LDS for the epilogue
        const HiCap<TI> cap{};   // not used: POLY reads A from memory
        char* tt = smem + wave * EPI_BYTES;
        // each 64 x 64 half: skipped when wholly below the diagonal; the
        // epilogue's own element checks handle the halves that cross it
        if (ec0 + 63 >= er0)
            epi_sym<KIND, TI, false>(md, t, pa, reinterpret_cast<const f32x4_t(&)[TI][TI]>(acc[0]), cap, er0, ec0,
                                     lane, tt);
        if (ec0 + 63 >= er0 + 64)
            epi_sym<KIND, TI, false>(md, t, pa, reinterpret_cast<const f32x4_t(&)[TI][TI]>(acc[4]), cap, er0 + 64,
                                     ec0, lane, tt);
    }
}

// FIRST: iteration 1 (X0 read from the momentum pass's copy of u; the master
// term recomputed from the caller's momentum and gradient).
template <int KIND, int BM, bool FIRST>
__global__ __launch_bounds__(kThreads, 2) void ns_gemm_bf16(const Tile* __restrict__ tiles,
                                                            const MatDesc* __restrict__ mats, PhaseArgs pa,
                                                            int n_tiles) {
    constexpr int BK = kBK;
    using C = BfCfg<BM, BK>;
    constexpr int TI = C::TI, WT = C::WT;
    // operand stages; afterwards the epilogue's per-wave regions
    constexpr int EPI_AXPY_BYTES = 16 * (WT + 4) * 4;
    constexpr int EPI_SYM_BYTES = SymGeom<TI>::T_BYTES;
    constexpr int EPI_BYTES = 4 * (KIND == PH_AXPY || KIND == PH_AXPY_LAST ? EPI_AXPY_BYTES : EPI_SYM_BYTES);
    constexpr int LDS_BYTES = C::NST * C::STB > EPI_BYTES ? C::NST * C::STB : EPI_BYTES;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const Tile t = tiles[xcd_tile(blockIdx.x, n_tiles)];
    if (t.mat < 0) return;
    const MatDesc& md = mats[t.mat];
    const Operands op = resolve_operands<KIND>(md, pa);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = (wave >> 1) * WT, wc = (wave & 1) * WT;
    const int row_a0 = t.ti * BM, row_b0 = t.tj * BM;

    f32x4_t acc[TI][TI];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TI; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    HiCap<TI> cap;
    if constexpr (KIND == PH_AXPY || KIND == PH_AXPY_LAST) {
        constexpr bool LAST = KIND == PH_AXPY_LAST;
        // 128-wide tiles after the first iteration keep the bf16 X of their own
        // quadrant from the operand stream (see HiCap).  The first iteration
        // issues the epilogue's first band of loads during the last k block;
        // the middle ones, which load only the low part of the master, issue
        // every band's loads there (4 words a lane), so the epilogue never
        // waits on memory band by band.
        constexpr bool CAPHI = !FIRST && BM == 128 && WT == kBK;
        constexpr int PRE = BM != 128 || LAST ? 0 : (CAPHI ? TI : 1);   // (measured slower on the last iteration)
        const AxpyCtx x = axpy_ctx<FIRST>(md, t, pa);
        AxpyRaw<TI> w0[PRE ? PRE : 1];
        const int er0 = row_a0 + wr, ec0 = row_b0 + wc;
        auto pre = [&]() __attribute__((always_inline)) {
            static_for<0, PRE>([&](auto bc) {
                axpy_load<TI, FIRST, LAST, true, IoRuntime, CAPHI>(x, cap, er0, ec0, lane, decltype(bc)::value,
                                                                   w0[decltype(bc)::value]);
            });
        };
        auto run = [&](auto capc, auto akc) __attribute__((always_inline)) {
            constexpr int CAPV = decltype(capc)::value;
            constexpr bool AKC_ALL = decltype(akc)::value;
            if constexpr (PRE > 0)
                mainloop<BM, BK, true, AKC_ALL, false, CAPV>(smem, op, row_a0, row_b0, wave, lane, acc, &cap, pre);
            else
                mainloop<BM, BK, true, AKC_ALL, false, CAPV>(smem, op, row_a0, row_b0, wave, lane, acc, &cap);
        };
        if (op.a_kc && op.b_kc) {   // transposed matrix: X^T B, X is the A operand
            cap.kb = (row_b0 + wc) / kBK;
            run(std::integral_constant<int, CAPHI ? 2 : 0>{}, std::true_type{});
        } else {                    // B X, X is the B operand
            cap.kb = (row_a0 + wr) / kBK;
            run(std::integral_constant<int, CAPHI ? 1 : 0>{}, std::false_type{});
        }
        __syncthreads();   // operand stages are dead: reuse LDS for the epilogue
        epi_axpy<TI, FIRST, LAST, CAPHI, PRE>(x, acc, cap, w0, er0, ec0, lane,
                                              reinterpret_cast<float*>(smem + wave * EPI_AXPY_BYTES));
    } else {
        // GRAM (kc, kc) or, for transposed matrices, (ks, ks); POLY (kc, kc),
        // keeping A (r, c) of its quadrant for the b A term (see HiCap)
        constexpr bool CAPA = KIND == PH_POLY && WT == BK;
        if constexpr (KIND == PH_POLY) {
            cap.kb = (row_b0 + wc) / BK;
            mainloop<BM, BK, true, true, true, CAPA ? 3 : 0>(smem, op, row_a0, row_b0, wave, lane, acc, &cap);
        } else if (op.a_kc && op.b_kc) {
            mainloop<BM, BK, true, true, true>(smem, op, row_a0, row_b0, wave, lane, acc);
        } else {
            mainloop<BM, BK, false, false, true>(smem, op, row_a0, row_b0, wave, lane, acc);
        }
        __syncthreads();   // operand stages are dead: reuse LDS for the epilogue
        epi_sym<KIND, TI, CAPA>(md, t, pa, acc, cap, row_a0 + wr, row_b0 + wc, lane, smem + wave * EPI_SYM_BYTES);
    }
}

// ---------------------------------------------------------------------------
// ns_steps == 0: O = u / (||u||_F + eps) in the stored orientation
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void direct_update_kernel(const Unit* __restrict__ units,
                                                                 const MatDesc* __restrict__ mats, PhaseArgs pa) {
    const Unit un = units[blockIdx.x];
    const MatDesc& md = mats[un.mat];
    const int C = md.C;
    const int total = (un.r1 - un.r0) * C;
    const float s = pa.norm[un.mat].inv;
    const float wdec = 1.f - pa.lr * pa.wd;
    const float step = pa.lr * md.shape_scale;
    const bool nest = pa.nesterov != 0;
    for (int idx = threadIdx.x; idx < total; idx += kThreads) {
        const int rr = idx / C;
        const int64_t r = un.r0 + rr, c = idx - rr * C;
        const float o = s * u_at(md, r, c, pa.beta, nest);
        if (md.has_param) {
            const int64_t pi = r * md.ld_param + c;
            const float w = load_elem(md.param, pi, md.io_dtype);
            store_elem(md.param, pi, md.io_dtype, fmaf(-step, o, w * wdec));
        }
        if (md.upd) gm(md.upd)[r * md.ld_upd + c] = o;
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// launch wrappers
// ---------------------------------------------------------------------------
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    size_t blocks = (n16 + kThreads - 1) / kThreads;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, s, static_cast<u32x4_t*>(p), n16);
    return hipGetLastError();
}

hipError_t launch_guards(char* ws, const int64_t* offsets, int n_guards, uint32_t* bad, hipStream_t s) {
    if (n_guards <= 0) return hipSuccess;
    const int grid = n_guards < 1024 ? n_guards : 1024;
    hipLaunchKernelGGL(guard_kernel, dim3(grid), dim3(kThreads), 0, s, ws, offsets, n_guards, bad);
    return hipGetLastError();
}

hipError_t launch_momentum(const Unit* units, int n_units, const MatDesc* mats, MomentumArgs a, hipStream_t s,
                           hipEvent_t ev0, hipEvent_t ev1) {
    if (n_units <= 0) return hipSuccess;
    // units hold about 8 K elements each: up to 24 K units is up to ~200 M elements
    if (n_units <= 24576)
        hipExtLaunchKernelGGL(momentum_kernel<4>, dim3(n_units), dim3(kThreads), 0, s, ev0, ev1, 0, units, mats, a);
    else
        hipExtLaunchKernelGGL(momentum_kernel<8>, dim3(n_units), dim3(kThreads), 0, s, ev0, ev1, 0, units, mats, a);
    return hipGetLastError();
}

hipError_t launch_finalize_norm(const MatDesc* mats, int n_mats, const double* partials, NormScale* norm, float eps,
                                hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (n_mats <= 0) return hipSuccess;
    hipExtLaunchKernelGGL(finalize_norm_kernel, dim3(n_mats), dim3(kThreads), 0, s, ev0, ev1, 0, mats, partials, norm,
                          eps);
    return hipGetLastError();
}

hipError_t launch_rescale(const Unit* units, int n_units, const MatDesc* mats, const NormScale* norm, char* ws,
                          hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (n_units <= 0) return hipSuccess;
    const int grid = n_units < 1024 ? n_units : 1024;
    hipExtLaunchKernelGGL(rescale_kernel, dim3(grid), dim3(kThreads), 0, s, ev0, ev1, 0, units, n_units, mats, norm,
                          ws);
    return hipGetLastError();
}

template <int KIND, int BM>
static void launch_bf16(bool first, const Tile* tiles, int n_tiles, const MatDesc* mats, PhaseArgs a, hipStream_t s,
                        hipEvent_t ev0, hipEvent_t ev1) {
    // only AXPY epilogues differ on the first iteration
    if constexpr (KIND == PH_AXPY || KIND == PH_AXPY_LAST) {
        if (first) {
            hipExtLaunchKernelGGL((ns_gemm_bf16<KIND, BM, true>), dim3(n_tiles), dim3(kThreads), 0, s, ev0, ev1, 0,
                                  tiles, mats, a, n_tiles);
            return;
        }
    }
    hipExtLaunchKernelGGL((ns_gemm_bf16<KIND, BM, false>), dim3(n_tiles), dim3(kThreads), 0, s, ev0, ev1, 0, tiles,
                          mats, a, n_tiles);
}

template <int KIND>
static void launch_kind(bool f32c, int tile, const Tile* tiles, int n_tiles, const MatDesc* mats, PhaseArgs a,
                        hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (f32c) {
        hipExtLaunchKernelGGL((ns_gemm_kernel<KIND, true>), dim3(n_tiles), dim3(kThreads), 0, s, ev0, ev1, 0, tiles,
                              mats, a);
        return;
    }
    if (tile == kTileWide) {
        // only AXPY epilogues differ on the first iteration
        if constexpr (KIND == PH_AXPY || KIND == PH_AXPY_LAST) {
            if (a.iter == 1) {
                hipExtLaunchKernelGGL((ns_gemm_wide<KIND, true>), dim3(n_tiles), dim3(WCfg::THREADS), 0, s, ev0, ev1,
                                      0, tiles, mats, a, n_tiles);
                return;
            }
        }
        hipExtLaunchKernelGGL((ns_gemm_wide<KIND, false>), dim3(n_tiles), dim3(WCfg::THREADS), 0, s, ev0, ev1, 0,
                              tiles, mats, a, n_tiles);
        return;
    }
    launch_bf16<KIND, 128>(a.iter == 1, tiles, n_tiles, mats, a, s, ev0, ev1);
}

hipError_t launch_ns_phase(int kind, bool f32c, int tile, const Tile* tiles, int n_tiles, const MatDesc* mats,
                           PhaseArgs a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (n_tiles <= 0) return hipSuccess;
    // 256-wide tiles: bf16 iterations only
    const bool wide_ok = tile == kTileWide && !f32c;
    if (tile != kTileBf16 && !wide_ok) return hipErrorInvalidValue;
    switch (kind) {
        case PH_GRAM: launch_kind<PH_GRAM>(f32c, tile, tiles, n_tiles, mats, a, s, ev0, ev1); break;
        case PH_POLY: launch_kind<PH_POLY>(f32c, tile, tiles, n_tiles, mats, a, s, ev0, ev1); break;
        case PH_AXPY: launch_kind<PH_AXPY>(f32c, tile, tiles, n_tiles, mats, a, s, ev0, ev1); break;
        case PH_AXPY_LAST: launch_kind<PH_AXPY_LAST>(f32c, tile, tiles, n_tiles, mats, a, s, ev0, ev1); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_direct_update(const Unit* units, int n_units, const MatDesc* mats, PhaseArgs a, hipStream_t s,
                                hipEvent_t ev0, hipEvent_t ev1) {
    if (n_units <= 0) return hipSuccess;
    hipExtLaunchKernelGGL(direct_update_kernel, dim3(n_units), dim3(kThreads), 0, s, ev0, ev1, 0, units, mats, a);
    return hipGetLastError();
}

}  // namespace muon

