// gfx950 kernels of the Muon step.
//
//  momentum_kernel      m' = beta m + g, u = g + beta m' (Nesterov) or m',
//                       operand copy of u, per-unit sum of u^2      (HBM bound)
//  finalize_norm        1 / (||u||_F + eps) per matrix, fixed-order sum
//  ns_gemm_kernel<KIND> the three products of one quintic Newton-Schulz
//                       iteration, grouped over every matrix of the call:
//                         GRAM  A = X X^T           (upper tiles, mirrored store)
//                         POLY  B = b A + c A A     (A symmetric: A A = A A^T)
//                         AXPY  X' = a X + B X      (fp32 master + operand copy)
//                         AXPY_LAST  same, then W' = W (1 - lr wd) - lr s O
//  direct_update        the update when ns_steps == 0
//
// The iteration follows the Newton-Schulz routine of the "NanoGPT Speedrun"
// page (modded-nanogpt README mirror), Muon section; the momentum and update
// follow "14 -- modded-nanogpt", section 3 pseudocode.
//
// MFMA products: v_mfma_f32_16x16x32_bf16 (bf16 mode) or v_mfma_f32_16x16x4_f32
// (fp32 validation mode), fp32 accumulation.  Both operands are staged in LDS
// as [row][k] in 16-byte chunks, XOR-swizzled; an operand whose k index is the
// row index in memory is transposed in registers on its way to LDS.

#include "muon_internal.hpp"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// dtype 0 = bf16, 1 = f32
__device__ __forceinline__ float load_elem(const void* p, int64_t i, int dt) {
    return dt == 0 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

__device__ __forceinline__ void store_elem(void* p, int64_t i, int dt, float v) {
    if (dt == 0)
        static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
    else
        static_cast<float*>(p)[i] = v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Sum over the 256 threads of a block in a fixed order; result valid in thread 0.
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float t = 0.f;
    if (threadIdx.x == 0) t = ((red[0] + red[1]) + red[2]) + red[3];
    return t;
}

// The orthogonalised input u at stored element (r, c), computed from the updated
// momentum m' and the gradient exactly as the momentum pass computed it.
__device__ __forceinline__ float u_at(const MatDesc& md, int64_t r, int64_t c, float beta, bool nest) {
    const float g = load_elem(md.grad, r * md.ld_grad + c, md.io_dtype);
    if (!md.has_mom) return g;
    const float mn = md.mom[r * md.ld_mom + c];
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
// momentum + operand copy + partial sums of squares
// ---------------------------------------------------------------------------
template <bool F32C>
__global__ __launch_bounds__(kThreads) void momentum_kernel(const Unit* __restrict__ units,
                                                            const MatDesc* __restrict__ mats, MomentumArgs ka) {
    __shared__ float red[4];
    const Unit un = units[blockIdx.x];
    const MatDesc& md = mats[un.mat];
    const int C = md.C;
    const int rows = un.r1 - un.r0;
    const float beta = ka.beta;
    const bool nest = ka.nesterov != 0;
    const bool has_mom = md.has_mom != 0;
    char* ub = ka.ws + md.off_u;
    const int64_t ldu = md.Cp;
    float ss = 0.f;

    if (md.vec_ok) {
        const int gpr = C >> 3;  // groups of 8 columns per row
        const int total = rows * gpr;
        for (int idx = threadIdx.x; idx < total; idx += kThreads) {
            const int rr = idx / gpr;
            const int c = (idx - rr * gpr) << 3;
            const int64_t r = un.r0 + rr;
            float g[8];
            if (md.io_dtype == 0) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(md.grad) + r * md.ld_grad + c);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    g[2 * q] = __uint_as_float(v[q] << 16);
                    g[2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
                }
            } else {
                const f32x4_t* gp = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(md.grad) + r * md.ld_grad + c);
                const f32x4_t v0 = gp[0], v1 = gp[1];
#pragma unroll
                for (int q = 0; q < 4; ++q) { g[q] = v0[q]; g[4 + q] = v1[q]; }
            }
            float u[8];
            if (has_mom) {
                f32x4_t* mp = reinterpret_cast<f32x4_t*>(md.mom + r * md.ld_mom + c);
                f32x4_t m0 = mp[0], m1 = mp[1];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    m0[q] = fmaf(beta, m0[q], g[q]);
                    m1[q] = fmaf(beta, m1[q], g[4 + q]);
                }
                mp[0] = m0;
                mp[1] = m1;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    u[q] = nest ? fmaf(beta, m0[q], g[q]) : m0[q];
                    u[4 + q] = nest ? fmaf(beta, m1[q], g[4 + q]) : m1[q];
                }
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) u[q] = g[q];
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) ss = fmaf(u[q], u[q], ss);
            if (F32C) {
                f32x4_t* up = reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(ub) + r * ldu + c);
                up[0] = f32x4_t{u[0], u[1], u[2], u[3]};
                up[1] = f32x4_t{u[4], u[5], u[6], u[7]};
            } else {
                u32x4_t w;
#pragma unroll
                for (int q = 0; q < 4; ++q) w[q] = pack_bf16x2(u[2 * q], u[2 * q + 1]);
                *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(ub) + r * ldu + c) = w;
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
                float* mp = md.mom + r * md.ld_mom + c;
                const float mn = fmaf(beta, *mp, g);
                *mp = mn;
                u = nest ? fmaf(beta, mn, g) : mn;
            }
            ss = fmaf(u, u, ss);
            if (F32C)
                reinterpret_cast<float*>(ub)[r * ldu + c] = u;
            else
                reinterpret_cast<uint16_t*>(ub)[r * ldu + c] = f32_to_bf16(u);
        }
    }
    const float tot = block_sum(ss, red);
    if (threadIdx.x == 0) ka.partials[blockIdx.x] = tot;
}

// ---------------------------------------------------------------------------
// per-matrix norm: fixed-order double sum of the unit partials
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void finalize_norm_kernel(const MatDesc* __restrict__ mats,
                                                                 const float* __restrict__ partials,
                                                                 float* __restrict__ inv_norm,
                                                                 float* __restrict__ nu_out, float eps) {
    __shared__ double red[kThreads];
    const MatDesc& md = mats[blockIdx.x];
    double s = 0.0;
    for (int i = threadIdx.x; i < md.nunits; i += kThreads) s += double(partials[md.unit0 + i]);
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double nu = sqrt(red[0]);
        inv_norm[blockIdx.x] = float(1.0 / (nu + double(eps)));
        nu_out[blockIdx.x] = float(nu);
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

template <int KIND>
__device__ __forceinline__ Operands resolve_operands(const MatDesc& md, const PhaseArgs& pa) {
    Operands o;
    const char* ws = pa.ws;
    const int it = pa.iter;
    // current X: the momentum pass's copy of u (stored orientation) on the first
    // iteration, afterwards the operand copy written by the previous iteration
    o.off_cur = (it == 1) ? md.off_u : (((it - 2) & 1) ? md.off_xb1 : md.off_xb0);
    if (KIND == PH_GRAM) {
        // A = X X^T: both operands are rows of X
        o.K = md.n;
        o.a = o.b = ws + o.off_cur;
        if (it == 1) {
            o.lda = o.ldb = md.Cp;
            o.a_kc = o.b_kc = !md.trans;   // X0 = U^T when transposed
        } else {
            o.lda = o.ldb = md.np;
            o.a_kc = o.b_kc = true;
        }
    } else if (KIND == PH_POLY) {
        // A A = A A^T (A symmetric): both operands are rows of A
        o.K = md.m;
        o.a = o.b = ws + md.off_a;
        o.lda = o.ldb = md.mp;
        o.a_kc = o.b_kc = true;
    } else {
        // B X: rows of B, columns of X (X^T rows when X0 = U^T)
        o.K = md.m;
        o.a = ws + md.off_b;
        o.lda = md.mp;
        o.a_kc = true;
        o.b = ws + o.off_cur;
        if (it == 1) {
            o.ldb = md.Cp;
            o.b_kc = md.trans != 0;
        } else {
            o.ldb = md.np;
            o.b_kc = false;
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
            const float s = pa.inv_norm[t.mat];
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
        const int m = md.m, n = md.n;
        const int64_t ldx = md.np;
        const float alpha = (it == 1) ? pa.inv_norm[t.mat] : 1.f;
        const bool nest = pa.nesterov != 0;
        const bool trans = md.trans != 0;
        const float* xm = reinterpret_cast<const float*>(ws + (F32 ? off_cur : md.off_xm));
        float* xm_out = reinterpret_cast<float*>(ws + md.off_xm);
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
                    if (r < m && c < n) {
                        const int64_t sr = trans ? c : r, sc = trans ? r : c;  // stored coordinates
                        const float master = (it == 1) ? u_at(md, sr, sc, pa.beta, nest) : xm[int64_t(r) * ldx + c];
                        const float v = alpha * fmaf(pa.a, master, acc[i][j][e]);
                        if (KIND == PH_AXPY) {
                            if (!F32) xm_out[int64_t(r) * ldx + c] = v;
                            store_elem(xb_next, int64_t(r) * ldx + c, ODT, v);
                        } else {
                            if (md.has_param) {
                                const int64_t pi = sr * md.ld_param + sc;
                                const float w = load_elem(md.param, pi, md.io_dtype);
                                store_elem(md.param, pi, md.io_dtype, fmaf(-step, v, w * wdec));
                            }
                            if (md.upd) md.upd[sr * md.ld_upd + sc] = v;
                        }
                    }
                }
    }
}

// Workgroups are handed to the 8 XCDs round-robin; give each XCD a contiguous
// range of the tile list so neighbouring tiles share that XCD's L2.
__device__ __forceinline__ int xcd_tile(int bid, int n) {
    const int q = n >> 3, r = n & 7;
    const int x = bid & 7, idx = bid >> 3;
    return (x < r) ? x * (q + 1) + idx : r * (q + 1) + (x - r) * q + idx;
}

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

    const Tile t = tiles[blockIdx.x];
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
// bf16 GEMM: BM x BM tiles (BM = 256 or 128), 4 waves of (BM/2)^2, BK = 64.
//
// Global -> LDS with direct-to-LDS 16-byte loads (no staging registers), two
// LDS stages, one barrier per k-block.  Row-contiguous operands sit in LDS as
// [row][8 chunks of 8 k] (chunk XOR-swizzled by row & 7) and feed the MFMA with
// ds_read_b128; k-strided operands sit as [k][BM] (chunk XOR-swizzled by
// 2 (k & 7)) and feed it with ds_read_b64_tr_b16, which hands lane j of each
// 16-lane group column j of a 4 x 16 block.
// ---------------------------------------------------------------------------
typedef short i16x4_t __attribute__((ext_vector_type(4)));
#ifndef LDS_AS
#define LDS_AS __attribute__((address_space(3)))
#endif

template <int BM>
struct BfCfg {
    static constexpr int BK = 64;
    static constexpr int WT = BM / 2;             // wave tile edge
    static constexpr int TI = WT / 16;            // MFMA tiles per wave edge
    static constexpr int OPB = BM * BK * 2;       // LDS bytes of one operand stage
    static constexpr int LPW = OPB / 1024 / 4;    // 1 KB direct loads per wave per operand
    static constexpr int CPR = BM / 8;            // 16-byte chunks per [k][BM] row
    static constexpr int RPK = 64 / CPR;          // [k][BM] rows per 1 KB
};

__device__ __forceinline__ int kswz(int k) { return (2 * k) & 14; }

// Issue the direct-to-LDS loads of one operand stage.
template <int BM>
__device__ __forceinline__ void lds_fill(char* __restrict__ lds, const char* __restrict__ g, int64_t ld, bool kc,
                                         int row0, int k0, int wave, int lane) {
    using C = BfCfg<BM>;
#pragma unroll
    for (int q = 0; q < C::LPW; ++q) {
        const int blk = wave * C::LPW + q;
        const char* src;
        if (kc) {
            const int r = blk * 8 + (lane >> 3);
            const int c = (lane & 7) ^ (r & 7);
            src = g + (int64_t(row0 + r) * ld + k0 + c * 8) * 2;
        } else {
            const int k = blk * C::RPK + lane / C::CPR;
            const int c = (lane % C::CPR) ^ kswz(k);
            src = g + (int64_t(k0 + k) * ld + row0 + c * 8) * 2;
        }
        __builtin_amdgcn_global_load_lds(src, (LDS_AS void*)(lds + blk * 1024), 16, 0, 0);
    }
}

// One MFMA operand fragment: 8 k values (k = 32 s + 8 (lane >> 4) + e) of
// row/column `rc` of the stage.
template <int BM>
__device__ __forceinline__ bf16x8_t frag(const char* __restrict__ lds, bool kc, int rc16, int s, int lane) {
    if (kc) {
        const int r = rc16 + (lane & 15);
        const int c = (4 * s + (lane >> 4)) ^ (r & 7);
        return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(lds + r * 128 + c * 16));
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
    const i16x4_t lo = h[0], hi = h[1];
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_t ld4_bf16(const void* p) {
    const u32x2_t w = *reinterpret_cast<const u32x2_t*>(p);
    return f32x4_t{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u), __uint_as_float(w[1] << 16),
                   __uint_as_float(w[1] & 0xFFFF0000u)};
}
__device__ __forceinline__ void st4_bf16(void* p, f32x4_t v) {
    *reinterpret_cast<u32x2_t*>(p) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
// 4 consecutive elements of a caller buffer (dtype 0 bf16 / 1 f32); `vec`: aligned and in range
__device__ __forceinline__ f32x4_t ld4_io(const void* p, int64_t i, int dt, bool vec, int nvalid) {
    if (vec) {
        if (dt == 0) return ld4_bf16(static_cast<const uint16_t*>(p) + i);
        return *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p) + i);
    }
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (q < nvalid) v[q] = load_elem(p, i + q, dt);
    return v;
}
__device__ __forceinline__ void st4_io(void* p, int64_t i, int dt, bool vec, int nvalid, f32x4_t v) {
    if (vec) {
        if (dt == 0)
            st4_bf16(static_cast<uint16_t*>(p) + i, v);
        else
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(p) + i) = v;
        return;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (q < nvalid) store_elem(p, i + q, dt, v[q]);
}

// u at 4 consecutive stored elements (r, c..c+3)
__device__ __forceinline__ f32x4_t u4_at(const MatDesc& md, int64_t r, int64_t c, float beta, bool nest, bool vec,
                                         int nvalid) {
    const f32x4_t g = ld4_io(md.grad, r * md.ld_grad + c, md.io_dtype, vec, nvalid);
    if (!md.has_mom) return g;
    const f32x4_t mn = ld4_io(md.mom, r * md.ld_mom + c, 1, vec, nvalid);
    if (!nest) return mn;
    f32x4_t u;
#pragma unroll
    for (int q = 0; q < 4; ++q) u[q] = fmaf(beta, mn[q], g[q]);
    return u;
}

// Epilogue through LDS.  Each wave stages its (16 x WT) row bands in fp32 in its
// own LDS region and reads them back as 4-element runs along rows (row-major
// pass) or down columns (column-major pass), so global traffic moves in 8- and
// 16-byte vectors along contiguous rows of the destination.
template <int KIND, int TI>
__device__ __forceinline__ void epilogue_staged(const MatDesc& md, const Tile& t, const PhaseArgs& pa,
                                                const f32x4_t (&acc)[TI][TI], int row0, int col0, int lane,
                                                float* __restrict__ stg) {
    constexpr int WT = TI * 16, LDW = WT + 4;
    char* const ws = pa.ws;
    const int it = pa.iter;
    const int m = md.m, n = md.n;
    const bool trans = md.trans != 0;
    const bool nest = pa.nesterov != 0;
    const bool vio = md.vec_io != 0;
    const bool gp = (KIND == PH_GRAM || KIND == PH_POLY);
    const bool diag = gp && t.ti == t.tj;
    // GRAM/POLY: out (and A for POLY); AXPY: X master / operand copies
    const int64_t ldq = gp ? md.mp : md.np;
    uint16_t* out = reinterpret_cast<uint16_t*>(ws + (KIND == PH_GRAM ? md.off_a : md.off_b));
    const uint16_t* ain = reinterpret_cast<const uint16_t*>(ws + md.off_a);
    float scl = 1.f;
    if (KIND == PH_GRAM && it == 1) {
        const float s = pa.inv_norm[t.mat];
        scl = s * s;
    }
    const float alpha = (it == 1) ? pa.inv_norm[t.mat] : 1.f;
    float* xm = reinterpret_cast<float*>(ws + md.off_xm);
    uint16_t* xb_next = reinterpret_cast<uint16_t*>(ws + (((it - 1) & 1) ? md.off_xb1 : md.off_xb0));
    const float wdec = 1.f - pa.lr * pa.wd;
    const float step = pa.lr * md.shape_scale;
    const bool row_pass = gp || KIND == PH_AXPY || !trans;
    const bool col_pass = gp || (KIND == PH_AXPY_LAST && trans);
    const int g = lane >> 4, c16 = lane & 15;

#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
        for (int j = 0; j < TI; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) stg[(4 * g + e) * LDW + 16 * j + c16] = acc[i][j][e];
        const int rb = row0 + 16 * i;
        if (row_pass) {
#pragma unroll 2
            for (int q = 0; q < WT / 16; ++q) {
                const int idx = q * 256 + lane * 4;
                const int lr = idx / WT, lc = idx % WT;
                const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stg + lr * LDW + lc);
                const int r = rb + lr, c = col0 + lc;
                if (gp) {
                    if (r >= m) continue;
                    int nv = m - c;                 // columns inside the matrix
                    nv = nv > 4 ? 4 : nv;
                    int first = 0;                  // diagonal tiles keep r <= c
                    if (diag && r > c) first = r - c;
                    if (nv <= first) continue;
                    const int64_t o = int64_t(r) * ldq + c;
                    f32x4_t w;
                    if (KIND == PH_GRAM) {
                        w = v * scl;
                    } else {
                        const f32x4_t a4 = (nv == 4) ? ld4_bf16(ain + o) : ld4_io(ain, o, 0, false, nv);
                        w = pa.b * a4 + pa.c * v;
                    }
                    if (nv == 4 && first == 0)
                        st4_bf16(out + o, w);
                    else
#pragma unroll
                        for (int q2 = 0; q2 < 4; ++q2)
                            if (q2 >= first && q2 < nv) out[o + q2] = f32_to_bf16(w[q2]);
                } else {
                    if (r >= m || c >= n) continue;
                    int nv = n - c;
                    nv = nv > 4 ? 4 : nv;
                    f32x4_t master;
                    if (it == 1)
                        master = trans ? f32x4_t{u_at(md, c, r, pa.beta, nest),
                                                 nv > 1 ? u_at(md, c + 1, r, pa.beta, nest) : 0.f,
                                                 nv > 2 ? u_at(md, c + 2, r, pa.beta, nest) : 0.f,
                                                 nv > 3 ? u_at(md, c + 3, r, pa.beta, nest) : 0.f}
                                       : u4_at(md, r, c, pa.beta, nest, vio && nv == 4, nv);
                    else
                        master = *reinterpret_cast<const f32x4_t*>(xm + int64_t(r) * ldq + c);  // padded: in bounds
                    f32x4_t x = alpha * (pa.a * master + v);
                    if (KIND == PH_AXPY) {
                        const int64_t o = int64_t(r) * ldq + c;
                        if (nv == 4) {
                            *reinterpret_cast<f32x4_t*>(xm + o) = x;
                            st4_bf16(xb_next + o, x);
                        } else {
#pragma unroll
                            for (int q2 = 0; q2 < 4; ++q2)
                                if (q2 < nv) {
                                    xm[o + q2] = x[q2];
                                    xb_next[o + q2] = f32_to_bf16(x[q2]);
                                }
                        }
                    } else {  // last iteration, stored orientation = NS orientation
                        const bool vec = vio && nv == 4;
                        if (md.has_param) {
                            const int64_t pi = int64_t(r) * md.ld_param + c;
                            const f32x4_t w = ld4_io(md.param, pi, md.io_dtype, vec, nv);
                            f32x4_t wn;
#pragma unroll
                            for (int q2 = 0; q2 < 4; ++q2) wn[q2] = fmaf(-step, x[q2], w[q2] * wdec);
                            st4_io(md.param, pi, md.io_dtype, vec, nv, wn);
                        }
                        if (md.upd) st4_io(md.upd, int64_t(r) * md.ld_upd + c, 1, vec, nv, x);
                    }
                }
            }
        }
        if (col_pass) {
#pragma unroll 2
            for (int q = 0; q < WT / 16; ++q) {
                const int task = q * 64 + lane;
                const int lc = task % WT, quad = task / WT;
                const int r = rb + 4 * quad, c = col0 + lc;   // elements (r..r+3, c)
                f32x4_t v;
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2) v[q2] = stg[(4 * quad + q2) * LDW + lc];
                if (gp) {
                    // mirror: (r + q2, c) -> (c, r + q2); diagonal tiles mirror only r + q2 < c
                    if (c >= m) continue;
                    int nv = m - r;
                    nv = nv > 4 ? 4 : nv;
                    if (diag) {
                        const int lim = c - r;        // q2 < lim  <=>  r + q2 < c
                        nv = nv < lim ? nv : lim;
                    }
                    if (nv <= 0) continue;
                    const int64_t o = int64_t(c) * ldq + r;
                    f32x4_t w;
                    if (KIND == PH_GRAM) {
                        w = v * scl;
                    } else {
                        const f32x4_t a4 = (nv == 4) ? ld4_bf16(ain + o) : ld4_io(ain, o, 0, false, nv);  // A symmetric
                        w = pa.b * a4 + pa.c * v;
                    }
                    if (nv == 4)
                        st4_bf16(out + o, w);
                    else
#pragma unroll
                        for (int q2 = 0; q2 < 4; ++q2)
                            if (q2 < nv) out[o + q2] = f32_to_bf16(w[q2]);
                } else {
                    // last iteration of a transposed matrix: NS (r + q2, c) is stored (c, r + q2)
                    if (c >= n || r >= m) continue;
                    int nv = m - r;
                    nv = nv > 4 ? 4 : nv;
                    const bool vec = vio && nv == 4;
                    f32x4_t master;
                    if (it == 1) {
                        master = u4_at(md, c, r, pa.beta, nest, vec, nv);
                    } else {
#pragma unroll
                        for (int q2 = 0; q2 < 4; ++q2) master[q2] = xm[int64_t(r + q2) * ldq + c];  // padded rows
                    }
                    const f32x4_t x = alpha * (pa.a * master + v);
                    if (md.has_param) {
                        const int64_t pi = int64_t(c) * md.ld_param + r;
                        const f32x4_t w = ld4_io(md.param, pi, md.io_dtype, vec, nv);
                        f32x4_t wn;
#pragma unroll
                        for (int q2 = 0; q2 < 4; ++q2) wn[q2] = fmaf(-step, x[q2], w[q2] * wdec);
                        st4_io(md.param, pi, md.io_dtype, vec, nv, wn);
                    }
                    if (md.upd) st4_io(md.upd, int64_t(c) * md.ld_upd + r, 1, vec, nv, x);
                }
            }
        }
    }
}

template <int KIND, int BM>
__global__ __launch_bounds__(kThreads, 1) void ns_gemm_bf16(const Tile* __restrict__ tiles,
                                                            const MatDesc* __restrict__ mats, PhaseArgs pa,
                                                            int n_tiles) {
    using C = BfCfg<BM>;
    constexpr int TI = C::TI, WT = C::WT;
    __shared__ __attribute__((aligned(1024))) char smem[4 * C::OPB];   // [stage][A | B]

    const Tile t = tiles[xcd_tile(blockIdx.x, n_tiles)];
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

    const int nk = (op.K + C::BK - 1) / C::BK;
    lds_fill<BM>(smem, op.a, op.lda, op.a_kc, row_a0, 0, wave, lane);
    lds_fill<BM>(smem + C::OPB, op.b, op.ldb, op.b_kc, row_b0, 0, wave, lane);

    for (int kb = 0; kb < nk; ++kb) {
        char* cur = smem + (kb & 1) * 2 * C::OPB;
        __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of stage kb have landed
        __syncthreads();                 // ... and every wave's; stage kb-1 is free
        if (kb + 1 < nk) {
            char* nxt = smem + ((kb + 1) & 1) * 2 * C::OPB;
            lds_fill<BM>(nxt, op.a, op.lda, op.a_kc, row_a0, (kb + 1) * C::BK, wave, lane);
            lds_fill<BM>(nxt + C::OPB, op.b, op.ldb, op.b_kc, row_b0, (kb + 1) * C::BK, wave, lane);
        }
        const char* sa = cur;
        const char* sb = cur + C::OPB;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8_t fa[TI], fb[TI];
#pragma unroll
            for (int i = 0; i < TI; ++i) fa[i] = frag<BM>(sa, op.a_kc, wr + 16 * i, s, lane);
#pragma unroll
            for (int j = 0; j < TI; ++j) fb[j] = frag<BM>(sb, op.b_kc, wc + 16 * j, s, lane);
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TI; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    }
    __syncthreads();   // operand stages are dead: reuse LDS for the epilogue
    epilogue_staged<KIND, TI>(md, t, pa, acc, row_a0 + wr, row_b0 + wc, lane,
                              reinterpret_cast<float*>(smem) + wave * 16 * (WT + 4));
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
    const float s = pa.inv_norm[un.mat];
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
        if (md.upd) md.upd[r * md.ld_upd + c] = o;
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

hipError_t launch_momentum(const Unit* units, int n_units, const MatDesc* mats, MomentumArgs a, bool f32c,
                           hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    if (f32c)
        hipLaunchKernelGGL(momentum_kernel<true>, dim3(n_units), dim3(kThreads), 0, s, units, mats, a);
    else
        hipLaunchKernelGGL(momentum_kernel<false>, dim3(n_units), dim3(kThreads), 0, s, units, mats, a);
    return hipGetLastError();
}

hipError_t launch_finalize_norm(const MatDesc* mats, int n_mats, const float* partials, float* inv_norm, float* nu,
                                float eps, hipStream_t s) {
    if (n_mats <= 0) return hipSuccess;
    hipLaunchKernelGGL(finalize_norm_kernel, dim3(n_mats), dim3(kThreads), 0, s, mats, partials, inv_norm, nu, eps);
    return hipGetLastError();
}

template <int KIND>
static void launch_kind(bool f32c, int tile, const Tile* tiles, int n_tiles, const MatDesc* mats, PhaseArgs a,
                        hipStream_t s) {
    if (f32c)
        hipLaunchKernelGGL((ns_gemm_kernel<KIND, true>), dim3(n_tiles), dim3(kThreads), 0, s, tiles, mats, a);
    else if (tile == 256)
        hipLaunchKernelGGL((ns_gemm_bf16<KIND, 256>), dim3(n_tiles), dim3(kThreads), 0, s, tiles, mats, a, n_tiles);
    else
        hipLaunchKernelGGL((ns_gemm_bf16<KIND, 128>), dim3(n_tiles), dim3(kThreads), 0, s, tiles, mats, a, n_tiles);
}

hipError_t launch_ns_phase(int kind, bool f32c, int tile, const Tile* tiles, int n_tiles, const MatDesc* mats,
                           PhaseArgs a, hipStream_t s) {
    if (n_tiles <= 0) return hipSuccess;
    if (f32c ? tile != 128 : (tile != 128 && tile != 256)) return hipErrorInvalidValue;
    switch (kind) {
        case PH_GRAM: launch_kind<PH_GRAM>(f32c, tile, tiles, n_tiles, mats, a, s); break;
        case PH_POLY: launch_kind<PH_POLY>(f32c, tile, tiles, n_tiles, mats, a, s); break;
        case PH_AXPY: launch_kind<PH_AXPY>(f32c, tile, tiles, n_tiles, mats, a, s); break;
        case PH_AXPY_LAST: launch_kind<PH_AXPY_LAST>(f32c, tile, tiles, n_tiles, mats, a, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_direct_update(const Unit* units, int n_units, const MatDesc* mats, PhaseArgs a, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    hipLaunchKernelGGL(direct_update_kernel, dim3(n_units), dim3(kThreads), 0, s, units, mats, a);
    return hipGetLastError();
}

}  // namespace muon
