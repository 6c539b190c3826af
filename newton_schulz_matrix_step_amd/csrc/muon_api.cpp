// Host side of the Muon C ABI: argument validation, the grouping planner
// (workspace layout, momentum units, tile lists), descriptor upload and the
// launch sequence of one step.
//
// One step = momentum pass + norm finalize + ns_steps x (GRAM, POLY, AXPY)
// launches, each launch covering every matrix of the call.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

// the library is built with hidden visibility: only the C ABI is exported
#pragma GCC visibility push(default)
#include "../../include/muon.h"
#pragma GCC visibility pop
#include "muon_internal.hpp"

using namespace muon;

namespace {

// the order is the ABI's muon_role
enum KernelRole {
    K_MOMENTUM = 0,
    K_FINALIZE,
    K_GRAM,
    K_POLY,
    K_AXPY,
    K_AXPY_LAST,
    K_DIRECT,
    K_FILL,
    K_ADAMW,
    K_RESCALE,
    K_NROLES
};
static_assert(int(K_MOMENTUM) == int(MUON_ROLE_MOMENTUM) && int(K_GRAM) == int(MUON_ROLE_GRAM) &&
                  int(K_AXPY) == int(MUON_ROLE_AXPY) && int(K_AXPY_LAST) == int(MUON_ROLE_AXPY_UPDATE) &&
                  int(K_ADAMW) == int(MUON_ROLE_ADAMW) && int(K_RESCALE) == int(MUON_ROLE_RESCALE) &&
                  K_NROLES == 10,
              "kernel roles follow muon_role");
const char* const kRoleNames[K_NROLES] = {"momentum_norm", "norm_finalize", "ns_gram", "ns_poly",
                                          "ns_axpy", "ns_axpy_update", "direct_update", "fill_zero",
                                          "adamw", "norm_rescale"};
constexpr uint32_t kRoleBits = (1u << K_NROLES) - 1u;

constexpr int kStageSlots = 4;
constexpr int kMaxTables = 16;     // descriptor tables per plan that a new pointer set may overwrite
constexpr int kMaxNsSteps = 64;
constexpr int64_t kMaxDim = int64_t(1) << 20;
constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxEntries = 65536;   // plan entries (matrices or blocks) per muon_step call
#ifndef MUON_UNIT_ELEMS
#define MUON_UNIT_ELEMS 8192
#endif
constexpr int kUnitElems = MUON_UNIT_ELEMS;  // momentum-pass elements per workgroup (target)

// Tile rows per item of the tile lists (see build_list): GRAM / POLY items of
// 8 rows (4 rows of 256-wide tiles: 5 % faster than 8 or 16 on the large
// layer share's GRAM); an AXPY output of at most 8 tile rows is one item,
// taller ones go in items of 4 rows (8 measured slower there, also for
// 256-wide tiles).
constexpr int kItemRowsSym = 8;
constexpr int kItemRowsWideSym = 4;
constexpr int kItemRowsAxpyWhole = 8;
constexpr int kItemRowsAxpy = 4;

// Tile lists per phase, one per kernel: [0] bf16 iterations on 128-wide
// tiles, [1] float32 iterations, [2] bf16 iterations of large matrices on
// 256-wide tiles.  A matrix may take wide tiles when its padded shape is a
// multiple of 256 and both sides are at least kWideMinDim (smaller ones have
// too few wide tiles to fill the CUs: 768-wide matrices measured 3 % slower
// on them, 1024 x 4096 ones 7 % faster).  A phase uses its wide list only
// when such matrices hold at least half of its flops: a phase split over two
// launches waits for the first one's tail (the MoE stack's four 2048 x 2048
// matrices beside 128 experts of 2048 x 1408 measured 4 % slower split).
constexpr int kListKinds = 3;
#ifndef MUON_WIDE_MIN
#define MUON_WIDE_MIN 1024
#endif
constexpr int kWideMinDim = MUON_WIDE_MIN;

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Pinned host slots for descriptor uploads: a slot is reused once the copy out
// of it has completed (its event).
struct Staging {
    void* h[kStageSlots] = {};
    hipEvent_t ev[kStageSlots] = {};
    bool used[kStageSlots] = {};
    int slot = 0;
    size_t bytes = 0;
};

// One descriptor table on the device: the pointers (and geometry) of one call.
// A table read by a step captured into a HIP graph is frozen: it is never
// rewritten, so the graph's replays keep reading exactly what was captured.
template <class D>
struct DescTable {
    D* d = nullptr;
    std::vector<D> host;       // what the device copy holds
    bool frozen = false;
    uint64_t last_use = 0;
};

template <class D>
struct TableSet {
    std::vector<DescTable<D>> tables;
    Staging stage;
    uint64_t clock = 0;
};

struct TileList {
    Tile* d = nullptr;
    int n = 0;                 // 8 per-XCD chunks of equal length, padded with mat = -1
};

// Everything one call signature (list of shapes, dtypes, buffer presence and
// compute mode) needs, built on first sight and kept until muon_destroy.
struct Plan {
    std::vector<int64_t> key;
    int n = 0;
    std::vector<MatDesc> geom;     // static part of every descriptor
    // per phase, one list per kernel: [0] bf16-iteration entries, [1] float32 entries
    TileList gram[kListKinds], poly[kListKinds], axpy[kListKinds];
    Unit* d_units = nullptr;
    int n_units = 0;
    double* d_partials = nullptr;
    NormScale* d_norm = nullptr;
    char* ws = nullptr;
    size_t ws_bytes = 0;
    int64_t* d_guards = nullptr;   // debug handles: guard band offsets and the check's counter
    int n_guards = 0;
    uint32_t* d_guard_bad = nullptr;
    TableSet<MatDesc> tabs;
};

// AdamW: chunk table (static per list of sizes and dtypes) and its descriptor tables.
struct AdamPlan {
    std::vector<int64_t> key;
    int n = 0;
    AdamChunk* d_chunks = nullptr;
    int n_chunks = 0;
    TableSet<AdamDesc> tabs;
};

struct Pending {
    int role;
    hipEvent_t a, b;
};

}  // namespace

struct muon_handle {
    int device = 0;
    uint32_t flags = 0;
    std::string err;
    std::map<std::vector<int64_t>, std::unique_ptr<Plan>> plans;
    std::map<std::vector<int64_t>, std::unique_ptr<AdamPlan>> adam_plans;
    Plan* last_step = nullptr;   // plan of the latest muon_step (norm readback)
    int last_step_n = 0;
    bool profile = false;
    uint32_t role_mask = 0;   // roles timed on a profiling handle
    std::vector<Pending> pending;
    std::vector<hipEvent_t> ev_pool;
    int64_t launches[K_NROLES] = {};
    double total_ms[K_NROLES] = {};
};

namespace {

muon_status fail(muon_handle* h, muon_status st, const char* fmt, ...) {
    if (h) {
        char buf[512];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof buf, fmt, ap);
        va_end(ap);
        h->err = buf;
    }
    return st;
}

muon_status hip_fail(muon_handle* h, hipError_t e, const char* what) {
    return fail(h, MUON_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Restores the caller's current device on scope exit.
struct DeviceGuard {
    int old = -1;
    bool ok = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&old) != hipSuccess) old = -1;
        ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard() {
        if (old >= 0) (void)hipSetDevice(old);
    }
};

void free_staging(Staging& st) {
    for (int i = 0; i < kStageSlots; ++i) {
        if (st.ev[i]) (void)hipEventDestroy(st.ev[i]);
        if (st.h[i]) (void)hipHostFree(st.h[i]);
    }
    st = Staging();
}

template <class D>
void free_tables(TableSet<D>& ts) {
    for (DescTable<D>& t : ts.tables) (void)hipFree(t.d);
    ts.tables.clear();
    free_staging(ts.stage);
}

void free_plan(Plan& p) {
    for (int m = 0; m < kListKinds; ++m) {
        (void)hipFree(p.gram[m].d);
        (void)hipFree(p.poly[m].d);
        (void)hipFree(p.axpy[m].d);
    }
    (void)hipFree(p.d_units);
    (void)hipFree(p.d_partials);
    (void)hipFree(p.d_norm);
    (void)hipFree(p.ws);
    (void)hipFree(p.d_guards);
    (void)hipFree(p.d_guard_bad);
    free_tables(p.tabs);
    p = Plan();
}

void free_adam_plan(AdamPlan& p) {
    (void)hipFree(p.d_chunks);
    free_tables(p.tabs);
    p = AdamPlan();
}

muon_status alloc_staging(muon_handle* h, Staging& st, size_t bytes) {
    st.bytes = std::max<size_t>(bytes, 16);
    for (int i = 0; i < kStageSlots; ++i)
        if (hipHostMalloc(&st.h[i], st.bytes, hipHostMallocDefault) != hipSuccess ||
            hipEventCreateWithFlags(&st.ev[i], hipEventDisableTiming) != hipSuccess) {
            (void)hipGetLastError();
            return fail(h, MUON_ERR_OOM, "descriptor staging allocation failed");
        }
    return MUON_OK;
}

// Is `stream` being captured into a graph?  A capturing call may only enqueue
// kernels that read state already on the device.
muon_status capture_state(muon_handle* h, hipStream_t stream, bool* capturing) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return hip_fail(h, e, "hipStreamIsCapturing");
    }
    *capturing = cs != hipStreamCaptureStatusNone;
    return MUON_OK;
}

// The device descriptor table holding exactly `desc`: an existing table when
// one matches (no upload), else an upload into the least recently used table
// that no captured graph reads (a new table while fewer than kMaxTables are
// in use).  Under capture only an existing table may serve, and it is frozen.
template <class D>
muon_status select_table(muon_handle* h, TableSet<D>& ts, const std::vector<D>& desc, bool capturing,
                         hipStream_t stream, const D** out) {
    const size_t bytes = sizeof(D) * desc.size();
    ++ts.clock;
    for (DescTable<D>& t : ts.tables)
        if (t.host.size() == desc.size() && std::memcmp(t.host.data(), desc.data(), bytes) == 0) {
            if (capturing) t.frozen = true;
            t.last_use = ts.clock;
            *out = t.d;
            return MUON_OK;
        }
    if (capturing)
        return fail(h, MUON_ERR_INVALID_ARG,
                    "a call captured into a HIP graph must first run once outside capture with the same shapes "
                    "and pointers (its plan and descriptor table are then resident)");
    DescTable<D>* slot = nullptr;
    int free_tables_n = 0;
    for (DescTable<D>& t : ts.tables)
        if (!t.frozen) {
            ++free_tables_n;
            if (!slot || t.last_use < slot->last_use) slot = &t;
        }
    if (!slot || free_tables_n < kMaxTables) {
        if (h->flags & MUON_INIT_FAIL_ALLOC)
            return fail(h, MUON_ERR_OOM, "descriptor table allocation failed (forced by MUON_INIT_FAIL_ALLOC)");
        DescTable<D> t;
        if (hipMalloc(reinterpret_cast<void**>(&t.d), std::max<size_t>(bytes, 16)) != hipSuccess) {
            (void)hipGetLastError();
            return fail(h, MUON_ERR_OOM, "descriptor table allocation failed");
        }
        ts.tables.push_back(std::move(t));
        slot = &ts.tables.back();
    }
    Staging& st = ts.stage;
    const int s = st.slot;
    hipError_t e;
    if (st.used[s]) {
        e = hipEventSynchronize(st.ev[s]);
        if (e != hipSuccess) return hip_fail(h, e, "descriptor staging wait");
    }
    std::memcpy(st.h[s], desc.data(), bytes);
    e = hipMemcpyAsync(slot->d, st.h[s], bytes, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipEventRecord(st.ev[s], stream);
    if (e != hipSuccess) return hip_fail(h, e, "descriptor upload");
    st.used[s] = true;
    st.slot = (s + 1) % kStageSlots;
    slot->host = desc;
    slot->last_use = ts.clock;
    *out = slot->d;
    return MUON_OK;
}

// Everything a caller passes for one matrix, before validation.
struct MatIn {
    void* param;
    const void* grad;
    float* mom;
    float* upd;
    int64_t R, C, ld_param, ld_grad, ld_mom, ld_upd;
    int32_t dtype;
    bool has_param, has_mom;
};

muon_status validate_hp(muon_handle* h, const muon_hparams* hp) {
    if (!hp) return fail(h, MUON_ERR_INVALID_ARG, "hparams is NULL");
    if (hp->compute != MUON_COMPUTE_BF16 && hp->compute != MUON_COMPUTE_FP32)
        return fail(h, MUON_ERR_DTYPE, "unknown compute mode %d", hp->compute);
    if (hp->ns_steps < 0 || hp->ns_steps > kMaxNsSteps)
        return fail(h, MUON_ERR_INVALID_ARG, "ns_steps %d outside 0..%d", hp->ns_steps, kMaxNsSteps);
    if (!(std::fabs(hp->a) > 0.f) || !std::isfinite(hp->a) || !std::isfinite(hp->b) || !std::isfinite(hp->c))
        return fail(h, MUON_ERR_INVALID_ARG, "coefficients must be finite with a != 0");
    if (hp->coeffs)
        for (int k = 0; k < hp->ns_steps; ++k) {
            const float* t = hp->coeffs + 3 * k;
            if (!(std::fabs(t[0]) > 0.f) || !std::isfinite(t[0]) || !std::isfinite(t[1]) || !std::isfinite(t[2]))
                return fail(h, MUON_ERR_INVALID_ARG, "coefficient triple %d must be finite with a != 0", k + 1);
        }
    if (hp->nesterov != 0 && hp->nesterov != 1)
        return fail(h, MUON_ERR_INVALID_ARG, "nesterov must be 0 or 1, got %d", hp->nesterov);
    return MUON_OK;
}

muon_status validate_mat(muon_handle* h, const MatIn& m, int idx) {
    if (m.dtype != MUON_BF16 && m.dtype != MUON_F32) return fail(h, MUON_ERR_DTYPE, "matrix %d: unknown dtype %d", idx, m.dtype);
    if (!m.grad) return fail(h, MUON_ERR_INVALID_ARG, "matrix %d: grad/input is NULL", idx);
    if (m.has_param && !m.param) return fail(h, MUON_ERR_INVALID_ARG, "matrix %d: param is NULL", idx);
    if (m.has_mom && !m.mom) return fail(h, MUON_ERR_INVALID_ARG, "matrix %d: momentum is NULL", idx);
    if (!m.has_param && !m.upd) return fail(h, MUON_ERR_INVALID_ARG, "matrix %d: output is NULL", idx);
    if (m.R < 1 || m.C < 1 || m.R > kMaxDim || m.C > kMaxDim || m.R * m.C > kMaxElems)
        return fail(h, MUON_ERR_INVALID_ARG, "matrix %d: bad shape %lld x %lld", idx, (long long)m.R, (long long)m.C);
    if (m.ld_grad < m.C || (m.has_param && m.ld_param < m.C) || (m.has_mom && m.ld_mom < m.C) ||
        (m.upd && m.ld_upd < m.C))
        return fail(h, MUON_ERR_INVALID_ARG, "matrix %d: leading dimension smaller than cols", idx);
    if (m.ld_grad > kMaxElems || m.ld_param > kMaxElems || m.ld_mom > kMaxElems || m.ld_upd > kMaxElems)
        return fail(h, MUON_ERR_INVALID_ARG, "matrix %d: leading dimension too large", idx);
    const void* g = m.grad;
    if (m.has_param && m.param == g) return fail(h, MUON_ERR_INVALID_ARG, "matrix %d: param aliases grad", idx);
    if (m.has_mom && (static_cast<const void*>(m.mom) == g || static_cast<void*>(m.mom) == m.param))
        return fail(h, MUON_ERR_INVALID_ARG, "matrix %d: momentum aliases param or grad", idx);
    if (m.upd && (static_cast<const void*>(m.upd) == g || static_cast<void*>(m.upd) == m.param ||
                  (m.has_mom && m.upd == m.mom)))
        return fail(h, MUON_ERR_INVALID_ARG, "matrix %d: update_out aliases another buffer", idx);
    return MUON_OK;
}

// Sub-block orthogonalisation: a validated matrix cut into bh x bw blocks
// enters the plan as one entry per block (row-major), each a strided view of
// the caller's buffers with the whole matrix's leading dimensions.
muon_status append_blocks(muon_handle* h, const MatIn& m, int32_t block_rows, int32_t block_cols, int idx,
                          std::vector<MatIn>& out) {
    if (block_rows < 0 || block_cols < 0)
        return fail(h, MUON_ERR_INVALID_ARG, "matrix %d: negative block size %d x %d", idx, block_rows, block_cols);
    const int64_t bh = block_rows ? block_rows : m.R;
    const int64_t bw = block_cols ? block_cols : m.C;
    if (m.R % bh != 0 || m.C % bw != 0)
        return fail(h, MUON_ERR_INVALID_ARG, "matrix %d: block %lld x %lld does not tile %lld x %lld", idx,
                    (long long)bh, (long long)bw, (long long)m.R, (long long)m.C);
    const int64_t nb = (m.R / bh) * (m.C / bw);
    if (int64_t(out.size()) + nb > kMaxEntries)
        return fail(h, MUON_ERR_INVALID_ARG, "matrix %d: more than %lld plan entries in one call", idx,
                    (long long)kMaxEntries);
    const int64_t es = m.dtype == MUON_BF16 ? 2 : 4;
    for (int64_t r0 = 0; r0 < m.R; r0 += bh)
        for (int64_t c0 = 0; c0 < m.C; c0 += bw) {
            MatIn b = m;
            b.R = bh;
            b.C = bw;
            b.grad = static_cast<const char*>(m.grad) + (r0 * m.ld_grad + c0) * es;
            if (m.param) b.param = static_cast<char*>(m.param) + (r0 * m.ld_param + c0) * es;
            if (m.mom) b.mom = m.mom + (r0 * m.ld_mom + c0);
            if (m.upd) b.upd = m.upd + (r0 * m.ld_upd + c0);
            out.push_back(b);
        }
    return MUON_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Host side of a plan: static geometry, workspace layout, units and tile
// lists of one call signature (no device memory).
struct PlanLayout {
    std::vector<MatDesc> geom;
    std::vector<Unit> units;
    std::vector<Tile> lists[3][kListKinds];   // [phase: GRAM, POLY, AXPY][list kind]
    std::vector<int64_t> guards;     // debug handles: workspace offsets of the guard bands
    size_t ws_bytes = 0;
};

muon_status layout_plan(muon_handle* h, const std::vector<MatIn>& mats, bool f32c, PlanLayout& L,
                        bool guard_bands = false) {
    const int n = int(mats.size());
    std::vector<MatDesc> geom(n);
    std::vector<Unit> units;
    size_t off = 0;
    // each workspace buffer 256-byte aligned; on a debug handle followed by a
    // guard band that no kernel may write
    auto take = [&](int64_t bytes) {
        const size_t o = off;
        off += size_t(round_up(bytes, 256));
        if (guard_bands) {
            L.guards.push_back(int64_t(off));
            off += kGuardBytes;
        }
        return int64_t(o);
    };
    for (int i = 0; i < n; ++i) {
        const MatIn& m = mats[i];
        MatDesc d;
        std::memset(&d, 0, sizeof d);
        d.R = int32_t(m.R);
        d.C = int32_t(m.C);
        d.trans = m.R > m.C;
        d.m = int32_t(std::min(m.R, m.C));
        d.n = int32_t(std::max(m.R, m.C));
        d.f32 = f32c || d.m <= kSmallM;
        d.Rp = int32_t(round_up(m.R, kPad));
        d.Cp = int32_t(round_up(m.C, kPad));
        d.mp = int32_t(round_up(d.m, kPad));
        d.np = int32_t(round_up(d.n, kPad));
        d.io_dtype = m.dtype;
        d.has_param = m.has_param;
        d.has_mom = m.has_mom;
        d.shape_scale = float(std::sqrt(std::max(1.0, double(m.R) / double(m.C))));
        const int64_t es = d.f32 ? 4 : 2;
        const int64_t xe = int64_t(d.mp) * d.np;
        d.off_u = take(int64_t(d.Rp) * d.Cp * es);
        d.off_xlo = d.f32 ? 0 : take(xe);
        d.off_xb0 = take(xe * es);
        d.off_xb1 = take(xe * es);
        d.off_a = take(int64_t(d.mp) * d.mp * es);
        d.off_b = take(int64_t(d.mp) * d.mp * es);
        // momentum-pass units: whole rows, about kUnitElems elements each
        const int rows_per_unit = int(std::max<int64_t>(1, kUnitElems / m.C));
        d.unit0 = int32_t(units.size());
        for (int64_t r = 0; r < m.R; r += rows_per_unit)
            units.push_back(Unit{i, int32_t(r), int32_t(std::min<int64_t>(m.R, r + rows_per_unit)), 0});
        d.nunits = int32_t(units.size()) - d.unit0;
        geom[i] = d;
    }
    // Newton-Schulz tile edge: 128 x 128 for every phase and both modes, and
    // 256 x 256 for the bf16 iterations of large matrices (kListKinds).  Two 128-wide
    // workgroups share a CU, so one tile's epilogue overlaps another's main
    // loop; AXPY tiles of this size also keep their quadrant of X from the
    // operand stream.  256-wide tiles of four 128 x 128 waves (one per SIMD)
    // measured no faster on any workload; wide tiles of eight 128 x 64 waves
    // (two per SIMD) are faster on large matrices.
    static_assert(kTileBf16 == kTileF32, "one tile edge for both modes");
    auto tile_of = [](int lk) { return lk == 2 ? kTileWide : kTileBf16; };
    // (every wide-eligible matrix has m >= 1024, so mp = Rp or Cp is a multiple of 256 too)
    auto wide_ok = [&](const MatDesc& d) {
        return !d.f32 && d.Rp % kTileWide == 0 && d.Cp % kTileWide == 0 && std::min(d.R, d.C) >= kWideMinDim;
    };
    // Per phase kind: GRAM, POLY, AXPY.  POLY stays on 128-wide tiles, which
    // keep A's quadrant from the operand stream for the b A term (wide POLY
    // measured 1 % faster on the large share, 3 % slower on the 350M-style set).
    bool use_wide[3] = {};
    for (int kind : {PH_GRAM, PH_AXPY}) {
        double all = 0.0, wide = 0.0;
        for (int i = 0; i < n; ++i) {
            const MatDesc& d = geom[i];
            if (d.f32) continue;
            const double f = double(d.m) * d.m * d.n;   // GRAM and AXPY flops up to a common factor
            all += f;
            if (wide_ok(d)) wide += f;
        }
        use_wide[kind] = wide > 0.0 && wide >= 0.5 * all;
    }
    // list of entry i in a phase (see kListKinds)
    auto list_kind = [&](int kind, int i) {
        const MatDesc& d = geom[i];
        if (d.f32) return 1;
        return use_wide[kind] && wide_ok(d) ? 2 : 0;
    };
    // Tile lists, one per phase and per iteration precision (bf16 and float32
    // entries run different kernels).  Workgroup b runs on XCD b % 8, and each
    // XCD has its own L2, so every list is 8 chunks, one per XCD: chunk x
    // holds the tiles XCD x runs, in dispatch order.  Tiles come in items (one
    // matrix's group of up to 4 or 8 tile rows across all tile columns, which
    // share operand panels; within an item the rows of one column are
    // consecutive); items are dealt to the XCDs largest first, each to the
    // least-loaded one (load = tiles x k blocks), so every XCD gets about the
    // same work however mixed the matrix shapes (keeping a matrix on one XCD
    // for L2 reuse measured slower: it costs balance); within a chunk, the
    // longest-k tiles go first.  GRAM (k = n) and POLY (k = m) weigh the same
    // tiles differently, so each gets its own list.
    auto build_list = [&](int kind, int lk, std::vector<Tile>& out) {
        const bool sym = kind != PH_AXPY;
        const int T = tile_of(lk);
        struct Item {
            int mat, a0;
            int64_t w;
        };
        std::vector<Item> items;
        auto ksteps = [&](const MatDesc& d) -> int64_t {
            const int64_t K = kind == PH_GRAM ? d.n : d.m;
            return (K + 63) / 64;
        };
        auto dims = [&](const MatDesc& d, int& tm, int& tn) {
            // GRAM/POLY outputs are m x m (upper triangle); AXPY outputs are R x C
            tm = sym ? (d.m + T - 1) / T : (d.R + T - 1) / T;
            tn = sym ? tm : (d.C + T - 1) / T;
        };
        auto item_rows = [&](int tm) {
            if (sym) return lk == 2 ? kItemRowsWideSym : kItemRowsSym;
            return tm <= kItemRowsAxpyWhole ? tm : kItemRowsAxpy;
        };
        for (int i = 0; i < n; ++i) {
            if (list_kind(kind, i) != lk) continue;
            int tm, tn;
            dims(geom[i], tm, tn);
            const int IR = item_rows(tm);
            for (int a0 = 0; a0 < tm; a0 += IR) {
                int64_t cnt = 0;
                for (int a = a0; a < std::min(tm, a0 + IR); ++a) cnt += sym ? tn - a : tn;
                items.push_back(Item{i, a0, cnt * ksteps(geom[i])});
            }
        }
        out.clear();
        if (items.empty()) return;
        std::stable_sort(items.begin(), items.end(), [](const Item& x, const Item& y) { return x.w > y.w; });
        std::vector<Tile> bins[8];
        int64_t load[8] = {};
        for (const Item& it : items) {
            int x = 0;
            for (int c = 1; c < 8; ++c)
                if (load[c] < load[x]) x = c;
            load[x] += it.w;
            int tm, tn;
            dims(geom[it.mat], tm, tn);
            const int IR = item_rows(tm);
            for (int b = 0; b < tn; ++b)
                for (int a = it.a0; a < std::min(tm, it.a0 + IR); ++a)
                    if (!sym || b >= a) bins[x].push_back(Tile{it.mat, a, b, 0});
        }
        size_t chunk = 0;
        for (auto& bin : bins) {
            std::stable_sort(bin.begin(), bin.end(), [&](const Tile& x, const Tile& y) {
                return ksteps(geom[x.mat]) > ksteps(geom[y.mat]);
            });
            chunk = std::max(chunk, bin.size());
        }
        out.assign(8 * chunk, Tile{-1, 0, 0, 0});
        for (int x = 0; x < 8; ++x) std::copy(bins[x].begin(), bins[x].end(), out.begin() + x * chunk);
    };
    std::vector<Tile> lists[3][kListKinds];
    for (int lk = 0; lk < kListKinds; ++lk) {
        build_list(PH_GRAM, lk, lists[0][lk]);
        build_list(PH_POLY, lk, lists[1][lk]);
        build_list(PH_AXPY, lk, lists[2][lk]);
    }
    // every tile's operand panels must lie inside the padded workspace buffers
    for (int lk = 0; lk < kListKinds; ++lk) {
        const int T = tile_of(lk);
        for (int l = 0; l < 2; ++l)
            for (const Tile& t : lists[l][lk]) {
                if (t.mat < 0) continue;
                const MatDesc& d = geom[t.mat];
                if ((t.ti + 1) * T > d.mp || (t.tj + 1) * T > d.mp || t.tj < t.ti)
                    return fail(h, MUON_ERR_HIP, "internal: gram tile (%d, %d) outside matrix %d", t.ti, t.tj, t.mat);
            }
        for (const Tile& t : lists[2][lk]) {
            if (t.mat < 0) continue;
            const MatDesc& d = geom[t.mat];
            if ((t.ti + 1) * T > d.Rp || (t.tj + 1) * T > d.Cp)
                return fail(h, MUON_ERR_HIP, "internal: axpy tile (%d, %d) outside matrix %d", t.ti, t.tj, t.mat);
        }
    }

    L.geom = std::move(geom);
    L.units = std::move(units);
    for (int l = 0; l < 3; ++l)
        for (int lk = 0; lk < kListKinds; ++lk) L.lists[l][lk] = std::move(lists[l][lk]);
    L.ws_bytes = off;
    return MUON_OK;
}

// A plan of its own for a new signature: device tables and a zero-filled
// workspace, uploaded and waited for once.
muon_status build_plan(muon_handle* h, const std::vector<MatIn>& mats, bool f32c, const std::vector<int64_t>& key,
                       hipStream_t stream, Plan** out) {
    const int n = int(mats.size());
    PlanLayout L;
    const bool debug = (h->flags & MUON_INIT_DEBUG) != 0;
    muon_status st = layout_plan(h, mats, f32c, L, debug);
    if (st != MUON_OK) return st;
    const size_t off = L.ws_bytes;
    if (h->flags & MUON_INIT_FAIL_ALLOC) return fail(h, MUON_ERR_OOM, "workspace allocation failed (forced by MUON_INIT_FAIL_ALLOC)");

    std::unique_ptr<Plan> q(new (std::nothrow) Plan());
    if (!q) return fail(h, MUON_ERR_OOM, "plan allocation failed");
    auto dmalloc = [&](void** ptr, size_t bytes) -> bool {
        return hipMalloc(ptr, std::max<size_t>(bytes, 16)) == hipSuccess;
    };
    TileList* tl[3] = {q->gram, q->poly, q->axpy};
    bool ok = true;
    for (int l = 0; ok && l < 3; ++l)
        for (int lk = 0; ok && lk < kListKinds; ++lk)
            if (!L.lists[l][lk].empty())
                ok = dmalloc(reinterpret_cast<void**>(&tl[l][lk].d), sizeof(Tile) * L.lists[l][lk].size());
    ok = ok && dmalloc(reinterpret_cast<void**>(&q->d_units), sizeof(Unit) * L.units.size()) &&
         dmalloc(reinterpret_cast<void**>(&q->d_partials), sizeof(double) * L.units.size()) &&
         dmalloc(reinterpret_cast<void**>(&q->d_norm), sizeof(NormScale) * n) &&
         dmalloc(reinterpret_cast<void**>(&q->ws), off) &&
         (!debug || (dmalloc(reinterpret_cast<void**>(&q->d_guards), sizeof(int64_t) * L.guards.size()) &&
                     dmalloc(reinterpret_cast<void**>(&q->d_guard_bad), 16)));
    if (!ok) {
        (void)hipGetLastError();
        free_plan(*q);
        return fail(h, MUON_ERR_OOM, "workspace allocation of %.3f GB failed", double(off) / 1e9);
    }
    st = alloc_staging(h, q->tabs.stage, sizeof(MatDesc) * n);
    if (st != MUON_OK) {
        free_plan(*q);
        return st;
    }
    q->ws_bytes = off;
    hipError_t e = launch_fill_zero(q->ws, off, stream);
    for (int l = 0; e == hipSuccess && l < 3; ++l)
        for (int lk = 0; e == hipSuccess && lk < kListKinds; ++lk)
            if (!L.lists[l][lk].empty()) {
                e = hipMemcpyAsync(tl[l][lk].d, L.lists[l][lk].data(), sizeof(Tile) * L.lists[l][lk].size(),
                                   hipMemcpyHostToDevice, stream);
                tl[l][lk].n = int(L.lists[l][lk].size());
            }
    if (e == hipSuccess)
        e = hipMemcpyAsync(q->d_units, L.units.data(), sizeof(Unit) * L.units.size(), hipMemcpyHostToDevice, stream);
    if (debug && e == hipSuccess && !L.guards.empty()) {
        e = hipMemcpyAsync(q->d_guards, L.guards.data(), sizeof(int64_t) * L.guards.size(), hipMemcpyHostToDevice,
                           stream);
        q->n_guards = int(L.guards.size());
        if (e == hipSuccess) e = launch_guards(q->ws, q->d_guards, q->n_guards, nullptr, stream);
    }
    // the host vectors die with this call: wait for the copies
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
        free_plan(*q);
        return hip_fail(h, e, "plan upload");
    }
    q->n = n;
    q->geom = std::move(L.geom);
    q->n_units = int(L.units.size());
    q->key = key;
    Plan* raw = q.get();
    h->plans[key] = std::move(q);
    *out = raw;
    return MUON_OK;
}

hipEvent_t get_event(muon_handle* h) {
    if (!h->ev_pool.empty()) {
        hipEvent_t e = h->ev_pool.back();
        h->ev_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// `launch(ev0, ev1)` enqueues one kernel; on a profiling handle the dispatch
// records ev0 / ev1 at its start and end (unless `events` is false: the
// no-allocation entry point creates no events).
template <class F>
hipError_t timed(muon_handle* h, int role, F&& launch, bool events = true) {
    if (!events || !h->profile || !((h->role_mask >> role) & 1u)) return launch(nullptr, nullptr);
    hipEvent_t a = get_event(h), b = get_event(h);
    if (!a || !b) return launch(nullptr, nullptr);
    const hipError_t e = launch(a, b);
    if (e == hipSuccess) h->pending.push_back(Pending{role, a, b});
    return e;
}

// One phase over its tile lists (wide bf16 tiles first, then 128-wide bf16,
// then float32); on a profiling handle the phase is timed as one, from the
// first launch's start to the last one's end.
hipError_t launch_phase_lists(int kind, const TileList (&l)[kListKinds], const MatDesc* desc, const PhaseArgs& pa,
                              hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
    static constexpr int kOrder[kListKinds] = {2, 0, 1};
    int first = -1, last = -1;
    for (int lk : kOrder)
        if (l[lk].n) {
            if (first < 0) first = lk;
            last = lk;
        }
    for (int lk : kOrder) {
        if (!l[lk].n) continue;
        const hipError_t e = launch_ns_phase(kind, lk == 1, lk == 2 ? kTileWide : kTileBf16, l[lk].d, l[lk].n, desc,
                                             pa, stream, lk == first ? e0 : nullptr, lk == last ? e1 : nullptr);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

std::vector<int64_t> signature(const std::vector<MatIn>& mats, bool f32c) {
    std::vector<int64_t> key;
    key.reserve(2 + 5 * mats.size());
    key.push_back(int64_t(mats.size()));
    key.push_back(f32c);
    for (const MatIn& m : mats) {
        key.push_back(m.R);
        key.push_back(m.C);
        key.push_back(m.dtype);
        key.push_back(m.has_param);
        key.push_back(m.has_mom);
    }
    return key;
}

// Descriptor table of one call: the plan's static geometry + the call's pointers.
std::vector<MatDesc> call_descriptors(const std::vector<MatDesc>& geom, const std::vector<MatIn>& mats) {
    std::vector<MatDesc> desc(geom);
    for (size_t i = 0; i < mats.size(); ++i) {
        const MatIn& m = mats[i];
        MatDesc& d = desc[i];
        d.param = m.param;
        d.grad = m.grad;
        d.mom = m.mom;
        d.upd = m.upd;
        d.ld_param = m.ld_param;
        d.ld_grad = m.ld_grad;
        d.ld_mom = m.ld_mom;
        d.ld_upd = m.ld_upd;
        d.vec_ok = (m.C % 8 == 0) && (m.ld_grad % 8 == 0) && aligned16(m.grad) &&
                   (!m.has_mom || ((m.ld_mom % 8 == 0) && aligned16(m.mom)));
        const int64_t pe = m.dtype == MUON_BF16 ? 8 : 16;   // bytes of 4 param/grad elements
        auto al = [](const void* q, int64_t b) { return (reinterpret_cast<uintptr_t>(q) % uintptr_t(b)) == 0; };
        d.vec_io = (m.C % 4 == 0) && (m.ld_grad % 4 == 0) && al(m.grad, pe) &&
                   (!m.has_param || ((m.ld_param % 4 == 0) && al(m.param, pe))) &&
                   (!m.has_mom || ((m.ld_mom % 4 == 0) && al(m.mom, 16))) &&
                   (!m.upd || ((m.ld_upd % 4 == 0) && al(m.upd, 16)));
    }
    return desc;
}

// The launches of one step over a plan's device tables and workspace.
muon_status enqueue_step(muon_handle* h, const Plan& plan, const MatDesc* d_desc, int n, const muon_hparams* hp,
                         hipStream_t stream, bool events = true) {
    MomentumArgs ma;
    ma.ws = plan.ws;
    ma.partials = plan.d_partials;
    ma.beta = hp->beta;
    ma.nesterov = hp->nesterov;
    hipError_t e = timed(h, K_MOMENTUM, [&](hipEvent_t e0, hipEvent_t e1) {
        return launch_momentum(plan.d_units, plan.n_units, d_desc, ma, stream, e0, e1);
    }, events);
    if (e != hipSuccess) return hip_fail(h, e, "momentum launch");
    e = timed(h, K_FINALIZE, [&](hipEvent_t e0, hipEvent_t e1) {
        return launch_finalize_norm(d_desc, n, plan.d_partials, plan.d_norm, hp->eps, stream, e0, e1);
    }, events);
    if (e != hipSuccess) return hip_fail(h, e, "norm launch");

    PhaseArgs pa;
    pa.ws = plan.ws;
    pa.norm = plan.d_norm;
    pa.a = hp->a;
    pa.b = hp->b;
    pa.c = hp->c;
    pa.lr = hp->lr;
    pa.wd = hp->weight_decay;
    pa.beta = hp->beta;
    pa.nesterov = hp->nesterov;
    pa.iter = 0;
    if (hp->ns_steps == 0) {
        e = timed(h, K_DIRECT, [&](hipEvent_t e0, hipEvent_t e1) {
            return launch_direct_update(plan.d_units, plan.n_units, d_desc, pa, stream, e0, e1);
        }, events);
        if (e != hipSuccess) return hip_fail(h, e, "update launch");
        return MUON_OK;
    }
    e = timed(h, K_RESCALE, [&](hipEvent_t e0, hipEvent_t e1) {
        return launch_rescale(plan.d_units, plan.n_units, d_desc, plan.d_norm, plan.ws, stream, e0, e1);
    }, events);
    if (e != hipSuccess) return hip_fail(h, e, "rescale launch");
    for (int it = 1; it <= hp->ns_steps; ++it) {
        pa.iter = it;
        if (hp->coeffs) {   // this iteration's triple
            pa.a = hp->coeffs[3 * (it - 1)];
            pa.b = hp->coeffs[3 * (it - 1) + 1];
            pa.c = hp->coeffs[3 * (it - 1) + 2];
        }
        e = timed(h, K_GRAM, [&](hipEvent_t e0, hipEvent_t e1) {
            return launch_phase_lists(PH_GRAM, plan.gram, d_desc, pa, stream, e0, e1);
        }, events);
        if (e != hipSuccess) return hip_fail(h, e, "gram launch");
        e = timed(h, K_POLY, [&](hipEvent_t e0, hipEvent_t e1) {
            return launch_phase_lists(PH_POLY, plan.poly, d_desc, pa, stream, e0, e1);
        }, events);
        if (e != hipSuccess) return hip_fail(h, e, "poly launch");
        const bool last = it == hp->ns_steps;
        e = timed(h, last ? K_AXPY_LAST : K_AXPY, [&](hipEvent_t e0, hipEvent_t e1) {
            return launch_phase_lists(last ? PH_AXPY_LAST : PH_AXPY, plan.axpy, d_desc, pa, stream, e0, e1);
        }, events);
        if (e != hipSuccess) return hip_fail(h, e, "axpy launch");
    }
    return MUON_OK;
}

// Debug handles: after the step, count the guard-band words that no longer
// hold the pattern (the stream is waited for).
muon_status check_guards(muon_handle* h, const Plan& plan, hipStream_t stream) {
    uint32_t bad = 0;
    hipError_t e = launch_fill_zero(plan.d_guard_bad, 16, stream);
    if (e == hipSuccess) e = launch_guards(plan.ws, plan.d_guards, plan.n_guards, plan.d_guard_bad, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(&bad, plan.d_guard_bad, sizeof bad, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(h, e, "guard band check");
    if (bad != 0)
        return fail(h, MUON_ERR_HIP, "debug check: %u words of the workspace guard bands were overwritten", bad);
    return MUON_OK;
}

muon_status run(muon_handle* h, const std::vector<MatIn>& mats, const muon_hparams* hp, hipStream_t stream,
                 Plan** used) {
    const int n = int(mats.size());
    const bool f32c = hp->compute == MUON_COMPUTE_FP32;
    bool capturing = false;
    muon_status st = capture_state(h, stream, &capturing);
    if (st != MUON_OK) return st;
    const std::vector<int64_t> key = signature(mats, f32c);
    Plan* pp = nullptr;
    auto it = h->plans.find(key);
    if (it != h->plans.end()) {
        pp = it->second.get();
    } else {
        if (capturing)
            return fail(h, MUON_ERR_INVALID_ARG,
                        "a call captured into a HIP graph must first run once outside capture with the same shapes "
                        "and pointers (its plan and descriptor table are then resident)");
        st = build_plan(h, mats, f32c, key, stream, &pp);
        if (st != MUON_OK) return st;
    }
    Plan& plan = *pp;
    const std::vector<MatDesc> desc = call_descriptors(plan.geom, mats);
    const MatDesc* d_desc = nullptr;
    st = select_table(h, plan.tabs, desc, capturing, stream, &d_desc);
    if (st != MUON_OK) return st;
    if (used) *used = pp;
    st = enqueue_step(h, plan, d_desc, n, hp, stream);
    if (st == MUON_OK && plan.n_guards > 0 && !capturing) st = check_guards(h, plan, stream);
    return st;
}

// ---- the no-allocation variant: everything in the device's static scratch ----

// What one device's scratch holds: the signature whose layout (zero-filled
// workspace, tile lists, units) was written last and the descriptor table
// written last.  Guarded by `mu`; the scratch itself is shared by every call
// on the device, so calls that overlap on one GPU race.
struct StaticDevice {
    std::mutex mu;
    std::vector<int64_t> key;
    std::vector<MatDesc> desc;
    bool layout_valid = false, desc_valid = false;
};
StaticDevice g_static[kMaxStaticDevices];

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

muon_status run_static(muon_handle* h, const std::vector<MatIn>& mats, const muon_hparams* hp, hipStream_t stream) {
    const int n = int(mats.size());
    const bool f32c = hp->compute == MUON_COMPUTE_FP32;
    if (h->device < 0 || h->device >= kMaxStaticDevices)
        return fail(h, MUON_ERR_INVALID_ARG, "device %d: the static scratch serves devices 0..%d", h->device,
                    kMaxStaticDevices - 1);
    const std::vector<int64_t> key = signature(mats, f32c);
    PlanLayout L;
    muon_status st = layout_plan(h, mats, f32c, L);
    if (st != MUON_OK) return st;
    // scratch layout: workspace | 6 tile lists | units | partials | norms | descriptors
    size_t off = align256(L.ws_bytes);
    size_t list_off[3][kListKinds];
    for (int l = 0; l < 3; ++l)
        for (int lk = 0; lk < kListKinds; ++lk) {
            list_off[l][lk] = off;
            off = align256(off + sizeof(Tile) * L.lists[l][lk].size());
        }
    const size_t units_off = off;
    off = align256(off + sizeof(Unit) * L.units.size());
    const size_t partials_off = off;
    off = align256(off + sizeof(double) * L.units.size());
    const size_t norm_off = off;
    off = align256(off + sizeof(NormScale) * size_t(n));
    const size_t desc_off = off;
    off = align256(off + sizeof(MatDesc) * size_t(n));
    if (off > kStaticScratchBytes)
        return fail(h, MUON_ERR_INVALID_ARG,
                    "this call needs %.1f MiB of scratch (workspace %.1f MiB); the static scratch holds %.0f MiB",
                    double(off) / (1 << 20), double(L.ws_bytes) / (1 << 20), double(kStaticScratchBytes) / (1 << 20));
    char* base = nullptr;
    hipError_t e = static_scratch_base(h->device, &base);
    if (e != hipSuccess) return hip_fail(h, e, "static scratch address");

    Plan plan;   // views into the scratch: owns no device memory
    TileList* tl[3] = {plan.gram, plan.poly, plan.axpy};
    for (int l = 0; l < 3; ++l)
        for (int lk = 0; lk < kListKinds; ++lk) {
            tl[l][lk].d = reinterpret_cast<Tile*>(base + list_off[l][lk]);
            tl[l][lk].n = int(L.lists[l][lk].size());
        }
    plan.d_units = reinterpret_cast<Unit*>(base + units_off);
    plan.n_units = int(L.units.size());
    plan.d_partials = reinterpret_cast<double*>(base + partials_off);
    plan.d_norm = reinterpret_cast<NormScale*>(base + norm_off);
    plan.ws = base;
    plan.ws_bytes = L.ws_bytes;
    MatDesc* d_desc = reinterpret_cast<MatDesc*>(base + desc_off);
    const std::vector<MatDesc> desc = call_descriptors(L.geom, mats);

    StaticDevice& sd = g_static[h->device];
    std::lock_guard<std::mutex> lock(sd.mu);
    // The scratch keeps the last call's contents.  A new signature moves the
    // layout: clear the workspace (its padding must read as zeros) and write
    // the tile lists and units; a new descriptor table is written too.  Each
    // copy reads host memory that dies with this call, so the stream is waited
    // for before returning from such a call.
    bool wait = false;
    if (!sd.layout_valid || sd.key != key) {
        sd.layout_valid = false;
        sd.desc_valid = false;
        e = launch_fill_zero(base, L.ws_bytes, stream);
        for (int l = 0; e == hipSuccess && l < 3; ++l)
            for (int lk = 0; e == hipSuccess && lk < kListKinds; ++lk)
                if (!L.lists[l][lk].empty())
                    e = hipMemcpyAsync(tl[l][lk].d, L.lists[l][lk].data(), sizeof(Tile) * L.lists[l][lk].size(),
                                       hipMemcpyHostToDevice, stream);
        if (e == hipSuccess)
            e = hipMemcpyAsync(plan.d_units, L.units.data(), sizeof(Unit) * L.units.size(), hipMemcpyHostToDevice,
                               stream);
        if (e != hipSuccess) return hip_fail(h, e, "static scratch layout upload");
        wait = true;
    }
    if (!sd.desc_valid || sd.desc.size() != desc.size() ||
        std::memcmp(sd.desc.data(), desc.data(), sizeof(MatDesc) * desc.size()) != 0) {
        sd.desc_valid = false;
        e = hipMemcpyAsync(d_desc, desc.data(), sizeof(MatDesc) * desc.size(), hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) return hip_fail(h, e, "static scratch descriptor upload");
        wait = true;
    }
    if (wait) {
        e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_fail(h, e, "static scratch upload wait");
        sd.key = key;
        sd.layout_valid = true;
        sd.desc = desc;
        sd.desc_valid = true;
    }
    return enqueue_step(h, plan, d_desc, n, hp, stream, false);
}

}  // namespace

extern "C" {

int muon_abi_version(void) { return MUON_ABI_VERSION; }

muon_status muon_init(muon_handle** out, int device, uint32_t flags) {
    if (!out) return MUON_ERR_INVALID_ARG;
    *out = nullptr;
    if (flags & ~(MUON_INIT_PROFILE | MUON_INIT_FAIL_ALLOC | MUON_INIT_DEBUG | MUON_INIT_PROFILE_ROLES(kRoleBits)))
        return MUON_ERR_INVALID_ARG;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return MUON_ERR_NO_DEVICE;
    }
    if (device < 0 || device >= count) return MUON_ERR_INVALID_ARG;
    muon_handle* h = new (std::nothrow) muon_handle();
    if (!h) return MUON_ERR_OOM;
    h->device = device;
    h->flags = flags;
    h->profile = (flags & MUON_INIT_PROFILE) != 0;
    h->role_mask = (flags >> 16) & kRoleBits;
    if (h->role_mask == 0) h->role_mask = kRoleBits;
    *out = h;
    return MUON_OK;
}

muon_status muon_step(muon_handle* h, const muon_matrix* mats, int32_t n_mats, const muon_hparams* hp, void* stream) {
    if (!h) return MUON_ERR_INVALID_ARG;
    h->err.clear();
    if (n_mats < 0) return fail(h, MUON_ERR_INVALID_ARG, "n_mats %d < 0", n_mats);
    if (n_mats == 0) return MUON_OK;
    if (!mats) return fail(h, MUON_ERR_INVALID_ARG, "mats is NULL");
    muon_status st = validate_hp(h, hp);
    if (st != MUON_OK) return st;
    std::vector<MatIn> in;
    in.reserve(size_t(n_mats));
    for (int i = 0; i < n_mats; ++i) {
        const muon_matrix& m = mats[i];
        if (m.reserved != 0) return fail(h, MUON_ERR_INVALID_ARG, "matrix %d: reserved field must be 0", i);
        const MatIn whole{m.param, m.grad, m.momentum, m.update_out, m.rows, m.cols, m.ld_param,
                          m.ld_grad, m.ld_mom, m.update_out ? m.ld_update : 0, m.dtype, true, true};
        st = validate_mat(h, whole, i);
        if (st != MUON_OK) return st;
        st = append_blocks(h, whole, m.block_rows, m.block_cols, i, in);
        if (st != MUON_OK) return st;
    }
    DeviceGuard g(h->device);
    if (!g.ok) return fail(h, MUON_ERR_NO_DEVICE, "cannot select device %d", h->device);
    Plan* used = nullptr;
    st = run(h, in, hp, static_cast<hipStream_t>(stream), &used);
    if (used) {
        h->last_step = used;
        h->last_step_n = int(in.size());
    }
    return st;
}

muon_status muon_step_noalloc(muon_handle* h, const muon_matrix* mats, int32_t n_mats, const muon_hparams* hp,
                              void* stream) {
    if (!h) return MUON_ERR_INVALID_ARG;
    h->err.clear();
    if (n_mats < 0) return fail(h, MUON_ERR_INVALID_ARG, "n_mats %d < 0", n_mats);
    if (n_mats == 0) return MUON_OK;
    if (!mats) return fail(h, MUON_ERR_INVALID_ARG, "mats is NULL");
    muon_status st = validate_hp(h, hp);
    if (st != MUON_OK) return st;
    std::vector<MatIn> in;
    in.reserve(size_t(n_mats));
    for (int i = 0; i < n_mats; ++i) {
        const muon_matrix& m = mats[i];
        if (m.reserved != 0) return fail(h, MUON_ERR_INVALID_ARG, "matrix %d: reserved field must be 0", i);
        const MatIn whole{m.param, m.grad, m.momentum, m.update_out, m.rows, m.cols, m.ld_param,
                          m.ld_grad, m.ld_mom, m.update_out ? m.ld_update : 0, m.dtype, true, true};
        st = validate_mat(h, whole, i);
        if (st != MUON_OK) return st;
        st = append_blocks(h, whole, m.block_rows, m.block_cols, i, in);
        if (st != MUON_OK) return st;
    }
    DeviceGuard g(h->device);
    if (!g.ok) return fail(h, MUON_ERR_NO_DEVICE, "cannot select device %d", h->device);
    return run_static(h, in, hp, static_cast<hipStream_t>(stream));
}

muon_status muon_orthogonalize(muon_handle* h, const void* in, float* out, int64_t rows, int64_t cols, int64_t ld_in,
                               int64_t ld_out, int32_t in_dtype, const muon_hparams* hp, void* stream) {
    if (!h) return MUON_ERR_INVALID_ARG;
    h->err.clear();
    muon_status st = validate_hp(h, hp);
    if (st != MUON_OK) return st;
    if (!out) return fail(h, MUON_ERR_INVALID_ARG, "out is NULL");
    if (in == static_cast<const void*>(out)) return fail(h, MUON_ERR_INVALID_ARG, "in aliases out");
    std::vector<MatIn> m(1);
    m[0] = MatIn{nullptr, in, nullptr, out, rows, cols, 0, ld_in, 0, ld_out, in_dtype, false, false};
    st = validate_mat(h, m[0], 0);
    if (st != MUON_OK) return st;
    DeviceGuard g(h->device);
    if (!g.ok) return fail(h, MUON_ERR_NO_DEVICE, "cannot select device %d", h->device);
    return run(h, m, hp, static_cast<hipStream_t>(stream), nullptr);
}

namespace {

muon_status build_adam_plan(muon_handle* h, const muon_adamw_tensor* ts, int n, const std::vector<int64_t>& key,
                            hipStream_t stream, AdamPlan** out) {
    std::vector<AdamChunk> chunks;
    for (int t = 0; t < n; ++t)
        for (int64_t b = 0; b < ts[t].numel; b += kAdamChunk) chunks.push_back(AdamChunk{t, 0, b});
    if (h->flags & MUON_INIT_FAIL_ALLOC) return fail(h, MUON_ERR_OOM, "allocation failed (forced by MUON_INIT_FAIL_ALLOC)");
    std::unique_ptr<AdamPlan> q(new (std::nothrow) AdamPlan());
    if (!q) return fail(h, MUON_ERR_OOM, "AdamW plan allocation failed");
    if (hipMalloc(reinterpret_cast<void**>(&q->d_chunks), sizeof(AdamChunk) * std::max<size_t>(chunks.size(), 1)) !=
        hipSuccess) {
        (void)hipGetLastError();
        free_adam_plan(*q);
        return fail(h, MUON_ERR_OOM, "AdamW plan allocation failed");
    }
    muon_status st = alloc_staging(h, q->tabs.stage, sizeof(AdamDesc) * size_t(n));
    if (st != MUON_OK) {
        free_adam_plan(*q);
        return st;
    }
    hipError_t e = hipSuccess;
    if (!chunks.empty()) {
        e = hipMemcpyAsync(q->d_chunks, chunks.data(), sizeof(AdamChunk) * chunks.size(), hipMemcpyHostToDevice, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);   // the host vector dies with this call
    }
    if (e != hipSuccess) {
        free_adam_plan(*q);
        return hip_fail(h, e, "AdamW plan upload");
    }
    q->n = n;
    q->n_chunks = int(chunks.size());
    q->key = key;
    AdamPlan* raw = q.get();
    h->adam_plans[key] = std::move(q);
    *out = raw;
    return MUON_OK;
}

}  // namespace

muon_status muon_adamw_step(muon_handle* h, const muon_adamw_tensor* ts, int32_t n, const muon_adamw_hparams* hp,
                            void* stream) {
    if (!h) return MUON_ERR_INVALID_ARG;
    h->err.clear();
    if (n < 0) return fail(h, MUON_ERR_INVALID_ARG, "n %d < 0", n);
    if (n == 0) return MUON_OK;
    if (!ts) return fail(h, MUON_ERR_INVALID_ARG, "tensors is NULL");
    if (!hp) return fail(h, MUON_ERR_INVALID_ARG, "hparams is NULL");
    if (!std::isfinite(hp->lr) || !std::isfinite(hp->weight_decay) || !std::isfinite(hp->eps) || !(hp->eps > 0.f))
        return fail(h, MUON_ERR_INVALID_ARG, "lr, weight_decay must be finite and eps finite and > 0");
    if (!(hp->beta1 >= 0.f && hp->beta1 < 1.f) || !(hp->beta2 >= 0.f && hp->beta2 < 1.f))
        return fail(h, MUON_ERR_INVALID_ARG, "beta1, beta2 must lie in [0, 1)");
    if (hp->step < 1) return fail(h, MUON_ERR_INVALID_ARG, "step %d < 1", hp->step);
    int64_t chunks = 0;
    for (int i = 0; i < n; ++i) {
        const muon_adamw_tensor& t = ts[i];
        if (t.reserved != 0) return fail(h, MUON_ERR_INVALID_ARG, "tensor %d: reserved field must be 0", i);
        if (t.dtype != MUON_BF16 && t.dtype != MUON_F32) return fail(h, MUON_ERR_DTYPE, "tensor %d: unknown dtype %d", i, t.dtype);
        if (t.numel < 0) return fail(h, MUON_ERR_INVALID_ARG, "tensor %d: numel %lld < 0", i, (long long)t.numel);
        if (t.numel == 0) continue;
        if (!t.param || !t.grad || !t.exp_avg || !t.exp_avg_sq)
            return fail(h, MUON_ERR_INVALID_ARG, "tensor %d: a buffer is NULL", i);
        const void* b[4] = {t.param, t.grad, t.exp_avg, t.exp_avg_sq};
        for (int x = 0; x < 4; ++x)
            for (int y = x + 1; y < 4; ++y)
                if (b[x] == b[y]) return fail(h, MUON_ERR_INVALID_ARG, "tensor %d: two buffers alias", i);
        chunks += (t.numel + kAdamChunk - 1) / kAdamChunk;
        if (chunks > int64_t(INT32_MAX)) return fail(h, MUON_ERR_INVALID_ARG, "more than 2^31 - 1 chunks of %d elements", kAdamChunk);
    }
    DeviceGuard g(h->device);
    if (!g.ok) return fail(h, MUON_ERR_NO_DEVICE, "cannot select device %d", h->device);
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::vector<int64_t> key;
    key.reserve(1 + 2 * size_t(n));
    key.push_back(n);
    for (int i = 0; i < n; ++i) {
        key.push_back(ts[i].numel);
        key.push_back(ts[i].dtype);
    }
    bool capturing = false;
    muon_status cst = capture_state(h, s, &capturing);
    if (cst != MUON_OK) return cst;
    AdamPlan* pp = nullptr;
    auto pit = h->adam_plans.find(key);
    if (pit != h->adam_plans.end()) {
        pp = pit->second.get();
    } else {
        if (capturing)
            return fail(h, MUON_ERR_INVALID_ARG,
                        "a call captured into a HIP graph must first run once outside capture with the same sizes "
                        "and pointers (its plan and descriptor table are then resident)");
        cst = build_adam_plan(h, ts, n, key, s, &pp);
        if (cst != MUON_OK) return cst;
    }
    AdamPlan& plan = *pp;
    std::vector<AdamDesc> desc(static_cast<size_t>(n));
    for (int i = 0; i < n; ++i) {
        const muon_adamw_tensor& t = ts[i];
        AdamDesc& d = desc[size_t(i)];
        std::memset(&d, 0, sizeof d);
        d.param = t.param;
        d.grad = t.grad;
        d.m = t.exp_avg;
        d.v = t.exp_avg_sq;
        d.numel = t.numel;
        d.dtype = t.dtype;
        const uintptr_t pa = t.dtype == MUON_BF16 ? 8 : 16;   // bytes of 4 param/grad elements
        auto al = [](const void* q, uintptr_t b) { return (reinterpret_cast<uintptr_t>(q) % b) == 0; };
        d.vec = al(t.param, pa) && al(t.grad, pa) && al(t.exp_avg, 16) && al(t.exp_avg_sq, 16);
    }
    const AdamDesc* d_desc = nullptr;
    cst = select_table(h, plan.tabs, desc, capturing, s, &d_desc);
    if (cst != MUON_OK) return cst;
    hipError_t e;
    // bias corrections in double, then the per-call constants in float
    const double bc1 = 1.0 - std::pow(double(hp->beta1), double(hp->step));
    const double bc2 = 1.0 - std::pow(double(hp->beta2), double(hp->step));
    AdamArgs a;
    a.beta1 = hp->beta1;
    a.one_minus_beta1 = float(1.0 - double(hp->beta1));
    a.beta2 = hp->beta2;
    a.one_minus_beta2 = float(1.0 - double(hp->beta2));
    a.decay = float(1.0 - double(hp->lr) * double(hp->weight_decay));
    a.step_size = float(double(hp->lr) / bc1);
    a.inv_sqrt_bc2 = float(1.0 / std::sqrt(bc2));
    a.eps = hp->eps;
    e = timed(h, K_ADAMW, [&](hipEvent_t e0, hipEvent_t e1) {
        return launch_adamw(plan.d_chunks, plan.n_chunks, d_desc, a, s, e0, e1);
    });
    if (e != hipSuccess) return hip_fail(h, e, "adamw launch");
    return MUON_OK;
}

muon_status muon_read_norms(muon_handle* h, float* out, int32_t n, void* stream) {
    if (!h || !out || n < 0) return MUON_ERR_INVALID_ARG;
    if (!h->last_step || n > h->last_step_n) return fail(h, MUON_ERR_INVALID_ARG, "no step with %d matrices yet", n);
    if (n == 0) return MUON_OK;
    DeviceGuard g(h->device);
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::vector<NormScale> buf(static_cast<size_t>(n));
    hipError_t e = hipMemcpyAsync(buf.data(), h->last_step->d_norm, sizeof(NormScale) * n, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(h, e, "norm readback");
    for (int i = 0; i < n; ++i) out[i] = buf[size_t(i)].nu;
    return MUON_OK;
}

int32_t muon_kernel_stats_read(muon_handle* h, muon_kernel_stats* out, int32_t max) {
    if (!h) return 0;
    DeviceGuard g(h->device);
    for (const Pending& p : h->pending) {
        float ms = 0.f;
        if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
            h->launches[p.role] += 1;
            h->total_ms[p.role] += ms;
        }
        h->ev_pool.push_back(p.a);
        h->ev_pool.push_back(p.b);
    }
    h->pending.clear();
    int32_t k = 0;
    for (int r = 0; r < K_NROLES && out && k < max; ++r) {
        if (h->launches[r] == 0) continue;
        std::memset(&out[k], 0, sizeof(muon_kernel_stats));
        std::snprintf(out[k].name, sizeof out[k].name, "%s", kRoleNames[r]);
        out[k].launches = h->launches[r];
        out[k].total_ms = h->total_ms[r];
        ++k;
    }
    return k;
}

void muon_kernel_stats_reset(muon_handle* h) {
    if (!h) return;
    (void)muon_kernel_stats_read(h, nullptr, 0);
    for (int r = 0; r < K_NROLES; ++r) {
        h->launches[r] = 0;
        h->total_ms[r] = 0.0;
    }
}

int64_t muon_workspace_bytes(const muon_handle* h) {
    if (!h) return 0;
    int64_t b = 0;
    for (const auto& kv : h->plans) b += int64_t(kv.second->ws_bytes);
    return b;
}

muon_status muon_destroy(muon_handle* h) {
    if (!h) return MUON_OK;
    {
        DeviceGuard g(h->device);
        (void)hipDeviceSynchronize();
        for (auto& kv : h->plans) free_plan(*kv.second);
        for (auto& kv : h->adam_plans) free_adam_plan(*kv.second);
        for (const Pending& p : h->pending) {
            (void)hipEventDestroy(p.a);
            (void)hipEventDestroy(p.b);
        }
        for (hipEvent_t e : h->ev_pool) (void)hipEventDestroy(e);
    }
    delete h;
    return MUON_OK;
}

const char* muon_status_str(muon_status s) {
    switch (s) {
        case MUON_OK: return "MUON_OK";
        case MUON_ERR_INVALID_ARG: return "MUON_ERR_INVALID_ARG";
        case MUON_ERR_DTYPE: return "MUON_ERR_DTYPE";
        case MUON_ERR_NO_DEVICE: return "MUON_ERR_NO_DEVICE";
        case MUON_ERR_OOM: return "MUON_ERR_OOM";
        case MUON_ERR_HIP: return "MUON_ERR_HIP";
    }
    return "MUON_ERR_UNKNOWN";
}

const char* muon_last_error(const muon_handle* h) { return h ? h->err.c_str() : ""; }

}  // extern "C"
