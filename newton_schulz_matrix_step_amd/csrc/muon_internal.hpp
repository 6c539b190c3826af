// Internal descriptors shared by the host planner (muon_api.cpp) and the
// gfx950 kernels (muon_kernels.hip).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

// All workspace matrices are padded to multiples of this many rows/columns and
// zero-filled once, so tile loads never leave the allocation and padding reads
// contribute zeros to every contraction.
constexpr int kPad = 128;

// Entries with min(R, C) at most this run the iteration in float32 in either
// compute mode: their products cost next to nothing, and with few singular
// values bf16 operands cost them the most accuracy.
constexpr int kSmallM = 64;

// Per-matrix descriptor, one entry per matrix of the call, in device memory.
// "Stored" = the caller's orientation (R x C); "NS" = the m x n orientation the
// iteration works in (m = min(R, C) rows, transposed when R > C).
struct MatDesc {
    int32_t R, C;              // stored shape
    int32_t m, n;              // NS shape, m <= n
    int32_t Rp, Cp;            // padded stored shape (U buffer)
    int32_t mp, np;            // padded NS shape
    int32_t trans;             // R > C
    int32_t io_dtype;          // storage dtype of param / grad / input (0 bf16, 1 f32)
    int32_t has_param;         // 0 for the orthogonalise-only entry point
    int32_t has_mom;           // 0: u = g (no momentum buffer)
    int32_t unit0, nunits;     // momentum-pass units owned by this matrix
    int32_t vec_ok;            // momentum pass: 8-element vectors legal for grad/mom
    int32_t vec_io;            // epilogues: 4-element vectors legal for param/grad/mom/upd
    float shape_scale;         // sqrt(max(1, R / C))
    int32_t f32;               // the iteration runs in float32 (workspace buffers float32)
    int64_t off_u;             // workspace byte offsets
    int64_t off_xlo;           // bf16 mode: X - bf16(X) in one byte per element; with the operand copy, the master X
    int64_t off_xb0, off_xb1;  // operand copies of X, ping-pong
    int64_t off_a, off_b;      // A = X X^T and B = b A + c A^2 (mp x mp)
    void* param;
    const void* grad;
    float* mom;
    float* upd;
    int64_t ld_param, ld_grad, ld_mom, ld_upd;
};

// One work unit of the momentum pass: rows [r0, r1) of matrix `mat`.
struct Unit {
    int32_t mat, r0, r1, pad;
};

// One output tile of a Newton-Schulz product.
struct Tile {
    int32_t mat, ti, tj, pad;
};

enum PhaseKind : int { PH_GRAM = 0, PH_POLY = 1, PH_AXPY = 2, PH_AXPY_LAST = 3 };

// Norm of one plan entry's input and the scales derived from it (norm
// finalize kernel).  The operand copy of u is kept as u 2^-k: k = 0 while
// nu lies in [2^-30, 2^30], where the products of the first iteration can
// neither overflow nor lose their terms to underflow in float32; outside it the
// rescale pass multiplies the copy by 2^-k (exact) with k the exponent of nu,
// and the first iteration applies first = 2^k / (nu + eps) to it.
struct NormScale {
    float inv;                 // 1 / (nu + eps)
    float first;               // 2^k / (nu + eps): scale of X0 relative to the operand copy
    int32_t k;                 // the operand copy holds u 2^-k
    float nu;                  // ||u||_F
};

struct PhaseArgs {
    char* ws;
    const NormScale* norm;     // per matrix
    float a, b, c;
    float lr, wd, beta;
    int32_t iter;              // 1-based iteration index
    int32_t nesterov;
};

struct MomentumArgs {
    char* ws;
    double* partials;          // one sum of squares per unit
    float beta;
    int32_t nesterov;
};

// Launch wrappers (muon_kernels.hip).  All return the launch status.  ev0 / ev1,
// when not null, are recorded by the dispatch itself at the kernel's start and
// end (hipExtLaunchKernelGGL), which adds no packets to the stream.
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_momentum(const Unit* units, int n_units, const MatDesc* mats, MomentumArgs a, hipStream_t s,
                           hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_finalize_norm(const MatDesc* mats, int n_mats, const double* partials,
                                NormScale* norm, float eps, hipStream_t s,
                                hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
// Multiplies the operand copy of every entry with k != 0 by 2^-k (one
// workgroup per momentum-pass unit; the others return at once).
hipError_t launch_rescale(const Unit* units, int n_units, const MatDesc* mats, const NormScale* norm, char* ws,
                          hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
// Debug guard bands after every workspace buffer: kGuardBytes of a fixed
// pattern.  bad == nullptr: write the pattern; otherwise add to *bad the
// number of 4-byte words that differ from it.
constexpr int kGuardBytes = 256;
constexpr uint32_t kGuardPattern = 0xA5C3F00Du;
hipError_t launch_guards(char* ws, const int64_t* offsets, int n_guards, uint32_t* bad, hipStream_t s);
hipError_t launch_ns_phase(int kind, bool f32_compute, int tile, const Tile* tiles, int n_tiles,
                           const MatDesc* mats, PhaseArgs a, hipStream_t s,
                           hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_direct_update(const Unit* units, int n_units, const MatDesc* mats,
                                PhaseArgs a, hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// ---- AdamW step (adamw_kernels.hip) ----
// Elements per workgroup: a tensor of the call is cut into chunks of this many
// elements (the last one ragged); one chunk table entry per chunk.
constexpr int kAdamChunk = 4096;

struct AdamDesc {
    void* param;
    const void* grad;
    float* m;
    float* v;
    int64_t numel;
    int32_t dtype;             // 0 bf16, 1 f32 (param and grad)
    int32_t vec;               // bases allow 4-element vectors
};

struct AdamChunk {
    int32_t t;                 // tensor index
    int32_t pad;
    int64_t begin;             // first element; the chunk ends at min(begin + kAdamChunk, numel)
};

struct AdamArgs {
    float beta1, one_minus_beta1, beta2, one_minus_beta2;
    float decay;               // 1 - lr * weight_decay
    float step_size;           // lr / (1 - beta1^t)
    float inv_sqrt_bc2;        // 1 / sqrt(1 - beta2^t)
    float eps;
};

hipError_t launch_adamw(const AdamChunk* chunks, int n_chunks, const AdamDesc* tensors, AdamArgs a, hipStream_t s,
                        hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// ---- static scratch of the no-allocation entry point (muon_static.hip) ----
// A file-scope device array of this many bytes per GPU, held until the
// process ends; its device address is looked up once per device.
constexpr size_t kStaticScratchBytes = size_t(256) << 20;
constexpr int kMaxStaticDevices = 64;
// Device address of the scratch on `device` (which must be current).
hipError_t static_scratch_base(int device, char** base);

// Tile edge of the Newton-Schulz GEMMs (both modes use 128 x 128 tiles; the
// bf16 AXPY of large matrices may use 256 x 256 tiles).
constexpr int kTileF32 = 128;
constexpr int kTileBf16 = 128;
constexpr int kTileWide = 256;

}  // namespace muon
