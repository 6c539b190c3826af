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
    K_NROLES
};
static_assert(K_MOMENTUM == MUON_ROLE_MOMENTUM && K_GRAM == MUON_ROLE_GRAM && K_AXPY == MUON_ROLE_AXPY &&
                  K_AXPY_LAST == MUON_ROLE_AXPY_UPDATE && K_ADAMW == MUON_ROLE_ADAMW && K_NROLES == 9,
              "kernel roles follow muon_role");
const char* const kRoleNames[K_NROLES] = {"momentum_norm", "norm_finalize", "ns_gram", "ns_poly",
                                          "ns_axpy", "ns_axpy_update", "direct_update", "fill_zero",
                                          "adamw"};

constexpr int kStageSlots = 4;
constexpr int kMaxNsSteps = 64;
constexpr int64_t kMaxDim = int64_t(1) << 20;
constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxEntries = 65536;   // plan entries (matrices or blocks) per muon_step call
constexpr int kUnitElems = 16384;  // momentum-pass elements per workgroup (target)
// Tile rows per item of the tile lists (see build_list): GRAM / POLY items of
// 8 rows; an AXPY output of at most 8 tile rows is one item, taller ones go in
// items of 4 rows (8 measured slower there).
constexpr int kItemRowsSym = 8;
constexpr int kItemRowsAxpyWhole = 8;
constexpr int kItemRowsAxpy = 4;



int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct Plan {
    bool valid = false;
    std::vector<int64_t> key;
    int n = 0;
    bool f32c = false;
    std::vector<MatDesc> geom;     // static part of every descriptor
    std::vector<MatDesc> uploaded; // last descriptor table sent to the device
    bool have_uploaded = false;
    MatDesc* d_desc = nullptr;
    // tile lists: 8 per-XCD chunks of equal length (n_* = 8 x chunk), padded
    // with skip entries (mat = -1)
    Tile* d_gram = nullptr;
    int n_gram = 0;
    int gram_tile = 0;
    Tile* d_poly = nullptr;
    int n_poly = 0;
    Tile* d_axpy = nullptr;
    int n_axpy = 0;
    int axpy_tile = 0;
    Unit* d_units = nullptr;
    int n_units = 0;
    float* d_partials = nullptr;
    float* d_inv = nullptr;
    float* d_nu = nullptr;
    char* ws = nullptr;
    size_t ws_bytes = 0;
    MatDesc* h_stage[kStageSlots] = {};
    hipEvent_t stage_ev[kStageSlots] = {};
    bool stage_used[kStageSlots] = {};
    int slot = 0;
};

// AdamW: chunk table (static per list of sizes and dtypes) and the last
// descriptor table sent to the device.
struct AdamPlan {
    bool valid = false;
    std::vector<int64_t> key;
    int n = 0;
    AdamDesc* d_desc = nullptr;
    AdamChunk* d_chunks = nullptr;
    int n_chunks = 0;
    std::vector<AdamDesc> uploaded;
    bool have_uploaded = false;
    AdamDesc* h_stage[kStageSlots] = {};
    hipEvent_t stage_ev[kStageSlots] = {};
    bool stage_used[kStageSlots] = {};
    int slot = 0;
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
    Plan step_plan, ortho_plan;
    AdamPlan adam_plan;
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

void free_adam_plan(AdamPlan& p) {
    (void)hipFree(p.d_desc);
    (void)hipFree(p.d_chunks);
    for (int i = 0; i < kStageSlots; ++i) {
        if (p.stage_ev[i]) (void)hipEventDestroy(p.stage_ev[i]);
        if (p.h_stage[i]) (void)hipHostFree(p.h_stage[i]);
    }
    p = AdamPlan();
}

void free_plan(Plan& p) {
    (void)hipFree(p.d_desc);
    (void)hipFree(p.d_gram);
    (void)hipFree(p.d_poly);
    (void)hipFree(p.d_axpy);
    (void)hipFree(p.d_units);
    (void)hipFree(p.d_partials);
    (void)hipFree(p.d_inv);
    (void)hipFree(p.d_nu);
    (void)hipFree(p.ws);
    for (int i = 0; i < kStageSlots; ++i) {
        if (p.stage_ev[i]) (void)hipEventDestroy(p.stage_ev[i]);
        if (p.h_stage[i]) (void)hipHostFree(p.h_stage[i]);
    }
    p = Plan();
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

// Static geometry, workspace layout, units and tiles for one call signature.
muon_status build_plan(muon_handle* h, Plan& p, const std::vector<MatIn>& mats, bool f32c,
                       const std::vector<int64_t>& key, hipStream_t stream) {
    if (p.valid || p.ws) {
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return hip_fail(h, e, "hipDeviceSynchronize before re-plan");
        free_plan(p);
    }
    const int n = int(mats.size());
    const int64_t es = f32c ? 4 : 2;
    std::vector<MatDesc> geom(n);
    std::vector<Unit> units;
    std::vector<Tile> gram, axpy;
    size_t off = 0;
    auto take = [&](int64_t bytes) {
        const size_t o = off;
        off += size_t(round_up(bytes, 256));
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
        d.Rp = int32_t(round_up(m.R, kPad));
        d.Cp = int32_t(round_up(m.C, kPad));
        d.mp = int32_t(round_up(d.m, kPad));
        d.np = int32_t(round_up(d.n, kPad));
        d.io_dtype = m.dtype;
        d.has_param = m.has_param;
        d.has_mom = m.has_mom;
        d.shape_scale = float(std::sqrt(std::max(1.0, double(m.R) / double(m.C))));
        const int64_t xe = int64_t(d.mp) * d.np;
        d.off_u = take(int64_t(d.Rp) * d.Cp * es);
        d.off_xlo = f32c ? 0 : take(xe);
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

    // Newton-Schulz tile edge: 128 x 128 in bf16 mode for every phase.  Two
    // workgroups share a CU, so one tile's epilogue overlaps another's main
    // loop; AXPY tiles of this size also keep their quadrant of X from the
    // operand stream.  256-wide tiles (one workgroup per CU, half the operand
    // traffic per flop) measured slower on every workload once those
    // epilogue savings were in.
    const int gram_tile = f32c ? kTileF32 : kTileBf16;
    const int axpy_tile = gram_tile;
    // Tile lists.  Workgroup b runs on XCD b % 8, and each XCD has its own L2,
    // so every list is 8 chunks, one per XCD: chunk x holds the tiles XCD x
    // runs, in dispatch order.  Tiles come in items (one matrix's group of up
    // to 4 or 8 tile rows across all tile columns, which share operand panels;
    // within an item the rows of one column are consecutive);
    // items are dealt to the XCDs largest first, each to the least-loaded one
    // (load = tiles x k blocks), so every XCD gets about the same work however
    // mixed the matrix shapes (keeping a matrix on one XCD for L2 reuse
    // measured slower: it costs balance); within a chunk, the longest-k tiles
    // go first.
    // GRAM (k = n) and POLY (k = m) weigh the same tiles differently, so each
    // gets its own list.
    auto build_list = [&](int T, int kind, std::vector<Tile>& out) {
        const bool sym = kind != PH_AXPY;
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
        auto item_rows = [&](int tm) { return sym ? kItemRowsSym : (tm <= kItemRowsAxpyWhole ? tm : kItemRowsAxpy); };
        for (int i = 0; i < n; ++i) {
            int tm, tn;
            dims(geom[i], tm, tn);
            const int IR = item_rows(tm);
            for (int a0 = 0; a0 < tm; a0 += IR) {
                int64_t cnt = 0;
                for (int a = a0; a < std::min(tm, a0 + IR); ++a) cnt += sym ? tn - a : tn;
                items.push_back(Item{i, a0, cnt * ksteps(geom[i])});
            }
        }
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
    std::vector<Tile> poly;
    build_list(gram_tile, PH_GRAM, gram);
    build_list(gram_tile, PH_POLY, poly);
    build_list(axpy_tile, PH_AXPY, axpy);
    // every tile's operand panels must lie inside the padded workspace buffers
    for (const std::vector<Tile>* lst : {&gram, &poly})
        for (const Tile& t : *lst) {
            if (t.mat < 0) continue;
            const MatDesc& d = geom[t.mat];
            if ((t.ti + 1) * gram_tile > d.mp || (t.tj + 1) * gram_tile > d.mp || t.tj < t.ti)
                return fail(h, MUON_ERR_HIP, "internal: gram tile (%d, %d) outside matrix %d", t.ti, t.tj, t.mat);
        }
    for (const Tile& t : axpy) {
        if (t.mat < 0) continue;
        const MatDesc& d = geom[t.mat];
        if ((t.ti + 1) * axpy_tile > d.Rp || (t.tj + 1) * axpy_tile > d.Cp)
            return fail(h, MUON_ERR_HIP, "internal: axpy tile (%d, %d) outside matrix %d", t.ti, t.tj, t.mat);
    }

    if (h->flags & MUON_INIT_FAIL_ALLOC) return fail(h, MUON_ERR_OOM, "workspace allocation failed (forced by MUON_INIT_FAIL_ALLOC)");

    Plan q;
    auto dmalloc = [&](void** ptr, size_t bytes) -> bool {
        return hipMalloc(ptr, std::max<size_t>(bytes, 16)) == hipSuccess;
    };
    bool ok = dmalloc(reinterpret_cast<void**>(&q.d_desc), sizeof(MatDesc) * n) &&
              dmalloc(reinterpret_cast<void**>(&q.d_gram), sizeof(Tile) * gram.size()) &&
              dmalloc(reinterpret_cast<void**>(&q.d_poly), sizeof(Tile) * poly.size()) &&
              dmalloc(reinterpret_cast<void**>(&q.d_axpy), sizeof(Tile) * axpy.size()) &&
              dmalloc(reinterpret_cast<void**>(&q.d_units), sizeof(Unit) * units.size()) &&
              dmalloc(reinterpret_cast<void**>(&q.d_partials), sizeof(float) * units.size()) &&
              dmalloc(reinterpret_cast<void**>(&q.d_inv), sizeof(float) * n) &&
              dmalloc(reinterpret_cast<void**>(&q.d_nu), sizeof(float) * n) &&
              dmalloc(reinterpret_cast<void**>(&q.ws), off);
    for (int i = 0; ok && i < kStageSlots; ++i) {
        ok = hipHostMalloc(reinterpret_cast<void**>(&q.h_stage[i]), sizeof(MatDesc) * std::max(n, 1), hipHostMallocDefault) == hipSuccess &&
             hipEventCreateWithFlags(&q.stage_ev[i], hipEventDisableTiming) == hipSuccess;
    }
    if (!ok) {
        (void)hipGetLastError();
        free_plan(q);
        return fail(h, MUON_ERR_OOM, "workspace allocation of %.3f GB failed", double(off) / 1e9);
    }
    q.ws_bytes = off;
    hipError_t e = launch_fill_zero(q.ws, off, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(q.d_gram, gram.data(), sizeof(Tile) * gram.size(), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(q.d_poly, poly.data(), sizeof(Tile) * poly.size(), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(q.d_axpy, axpy.data(), sizeof(Tile) * axpy.size(), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(q.d_units, units.data(), sizeof(Unit) * units.size(), hipMemcpyHostToDevice, stream);
    // the host vectors die with this call: wait for the copies
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
        free_plan(q);
        return hip_fail(h, e, "plan upload");
    }
    q.n = n;
    q.f32c = f32c;
    q.geom = std::move(geom);
    q.n_gram = int(gram.size());
    q.n_poly = int(poly.size());
    q.n_axpy = int(axpy.size());
    q.gram_tile = gram_tile;
    q.axpy_tile = axpy_tile;
    q.n_units = int(units.size());
    q.key = key;
    q.valid = true;
    p = std::move(q);
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
// records ev0 / ev1 at its start and end.
template <class F>
hipError_t timed(muon_handle* h, int role, F&& launch) {
    if (!h->profile || !((h->role_mask >> role) & 1u)) return launch(nullptr, nullptr);
    hipEvent_t a = get_event(h), b = get_event(h);
    if (!a || !b) return launch(nullptr, nullptr);
    const hipError_t e = launch(a, b);
    if (e == hipSuccess) h->pending.push_back(Pending{role, a, b});
    return e;
}

muon_status run(muon_handle* h, Plan& plan, const std::vector<MatIn>& mats, const muon_hparams* hp, hipStream_t stream) {
    const int n = int(mats.size());
    const bool f32c = hp->compute == MUON_COMPUTE_FP32;
    std::vector<int64_t> key;
    key.reserve(2 + 5 * size_t(n));
    key.push_back(n);
    key.push_back(f32c);
    for (const MatIn& m : mats) {
        key.push_back(m.R);
        key.push_back(m.C);
        key.push_back(m.dtype);
        key.push_back(m.has_param);
        key.push_back(m.has_mom);
    }
    if (!plan.valid || plan.key != key) {
        muon_status st = build_plan(h, plan, mats, f32c, key, stream);
        if (st != MUON_OK) return st;
    }

    // descriptor table: static geometry + this call's pointers
    std::vector<MatDesc> desc(plan.geom);
    for (int i = 0; i < n; ++i) {
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
        {
            const int64_t pe = m.dtype == MUON_BF16 ? 8 : 16;   // bytes of 4 param/grad elements
            auto al = [](const void* q, int64_t b) { return (reinterpret_cast<uintptr_t>(q) % uintptr_t(b)) == 0; };
            d.vec_io = (m.C % 4 == 0) && (m.ld_grad % 4 == 0) && al(m.grad, pe) &&
                       (!m.has_param || ((m.ld_param % 4 == 0) && al(m.param, pe))) &&
                       (!m.has_mom || ((m.ld_mom % 4 == 0) && al(m.mom, 16))) &&
                       (!m.upd || ((m.ld_upd % 4 == 0) && al(m.upd, 16)));
        }
    }
    hipError_t e;
    if (!plan.have_uploaded || std::memcmp(desc.data(), plan.uploaded.data(), sizeof(MatDesc) * n) != 0) {
        const int s = plan.slot;
        if (plan.stage_used[s]) {
            e = hipEventSynchronize(plan.stage_ev[s]);
            if (e != hipSuccess) return hip_fail(h, e, "descriptor staging wait");
        }
        std::memcpy(plan.h_stage[s], desc.data(), sizeof(MatDesc) * n);
        e = hipMemcpyAsync(plan.d_desc, plan.h_stage[s], sizeof(MatDesc) * n, hipMemcpyHostToDevice, stream);
        if (e == hipSuccess) e = hipEventRecord(plan.stage_ev[s], stream);
        if (e != hipSuccess) return hip_fail(h, e, "descriptor upload");
        plan.stage_used[s] = true;
        plan.slot = (s + 1) % kStageSlots;
        plan.uploaded = desc;
        plan.have_uploaded = true;
    }

    MomentumArgs ma;
    ma.ws = plan.ws;
    ma.partials = plan.d_partials;
    ma.beta = hp->beta;
    ma.nesterov = hp->nesterov;
    e = timed(h, K_MOMENTUM, [&](hipEvent_t e0, hipEvent_t e1) {
        return launch_momentum(plan.d_units, plan.n_units, plan.d_desc, ma, f32c, stream, e0, e1);
    });
    if (e != hipSuccess) return hip_fail(h, e, "momentum launch");
    e = timed(h, K_FINALIZE, [&](hipEvent_t e0, hipEvent_t e1) {
        return launch_finalize_norm(plan.d_desc, n, plan.d_partials, plan.d_inv, plan.d_nu, hp->eps, stream, e0, e1);
    });
    if (e != hipSuccess) return hip_fail(h, e, "norm launch");

    PhaseArgs pa;
    pa.ws = plan.ws;
    pa.inv_norm = plan.d_inv;
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
            return launch_direct_update(plan.d_units, plan.n_units, plan.d_desc, pa, stream, e0, e1);
        });
        if (e != hipSuccess) return hip_fail(h, e, "update launch");
        return MUON_OK;
    }
    for (int it = 1; it <= hp->ns_steps; ++it) {
        pa.iter = it;
        if (hp->coeffs) {   // this iteration's triple
            pa.a = hp->coeffs[3 * (it - 1)];
            pa.b = hp->coeffs[3 * (it - 1) + 1];
            pa.c = hp->coeffs[3 * (it - 1) + 2];
        }
        e = timed(h, K_GRAM, [&](hipEvent_t e0, hipEvent_t e1) {
            return launch_ns_phase(PH_GRAM, f32c, plan.gram_tile, plan.d_gram, plan.n_gram, plan.d_desc, pa, stream, e0, e1);
        });
        if (e != hipSuccess) return hip_fail(h, e, "gram launch");
        e = timed(h, K_POLY, [&](hipEvent_t e0, hipEvent_t e1) {
            return launch_ns_phase(PH_POLY, f32c, plan.gram_tile, plan.d_poly, plan.n_poly, plan.d_desc, pa, stream, e0, e1);
        });
        if (e != hipSuccess) return hip_fail(h, e, "poly launch");
        const bool last = it == hp->ns_steps;
        e = timed(h, last ? K_AXPY_LAST : K_AXPY, [&](hipEvent_t e0, hipEvent_t e1) {
            return launch_ns_phase(last ? PH_AXPY_LAST : PH_AXPY, f32c, plan.axpy_tile, plan.d_axpy, plan.n_axpy,
                                   plan.d_desc, pa, stream, e0, e1);
        });
        if (e != hipSuccess) return hip_fail(h, e, "axpy launch");
    }
    return MUON_OK;
}

}  // namespace

extern "C" {

int muon_abi_version(void) { return MUON_ABI_VERSION; }

muon_status muon_init(muon_handle** out, int device, uint32_t flags) {
    if (!out) return MUON_ERR_INVALID_ARG;
    *out = nullptr;
    if (flags & ~(MUON_INIT_PROFILE | MUON_INIT_FAIL_ALLOC | MUON_INIT_PROFILE_ROLES(0x1FFu))) return MUON_ERR_INVALID_ARG;
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
    h->role_mask = (flags >> 16) & 0x1FFu;
    if (h->role_mask == 0) h->role_mask = (1u << K_NROLES) - 1u;
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
    return run(h, h->step_plan, in, hp, static_cast<hipStream_t>(stream));
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
    return run(h, h->ortho_plan, m, hp, static_cast<hipStream_t>(stream));
}

namespace {

muon_status build_adam_plan(muon_handle* h, AdamPlan& p, const muon_adamw_tensor* ts, int n,
                            const std::vector<int64_t>& key, hipStream_t stream) {
    if (p.valid || p.d_desc) {
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return hip_fail(h, e, "hipDeviceSynchronize before re-plan");
        free_adam_plan(p);
    }
    std::vector<AdamChunk> chunks;
    for (int t = 0; t < n; ++t)
        for (int64_t b = 0; b < ts[t].numel; b += kAdamChunk) chunks.push_back(AdamChunk{t, 0, b});
    if (h->flags & MUON_INIT_FAIL_ALLOC) return fail(h, MUON_ERR_OOM, "allocation failed (forced by MUON_INIT_FAIL_ALLOC)");
    AdamPlan q;
    bool ok = hipMalloc(reinterpret_cast<void**>(&q.d_desc), sizeof(AdamDesc) * size_t(n)) == hipSuccess &&
              hipMalloc(reinterpret_cast<void**>(&q.d_chunks), sizeof(AdamChunk) * std::max<size_t>(chunks.size(), 1)) ==
                  hipSuccess;
    for (int i = 0; ok && i < kStageSlots; ++i)
        ok = hipHostMalloc(reinterpret_cast<void**>(&q.h_stage[i]), sizeof(AdamDesc) * size_t(n), hipHostMallocDefault) ==
                 hipSuccess &&
             hipEventCreateWithFlags(&q.stage_ev[i], hipEventDisableTiming) == hipSuccess;
    if (!ok) {
        (void)hipGetLastError();
        free_adam_plan(q);
        return fail(h, MUON_ERR_OOM, "AdamW plan allocation failed");
    }
    hipError_t e = hipSuccess;
    if (!chunks.empty()) {
        e = hipMemcpyAsync(q.d_chunks, chunks.data(), sizeof(AdamChunk) * chunks.size(), hipMemcpyHostToDevice, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);   // the host vector dies with this call
    }
    if (e != hipSuccess) {
        free_adam_plan(q);
        return hip_fail(h, e, "AdamW plan upload");
    }
    q.n = n;
    q.n_chunks = int(chunks.size());
    q.key = key;
    q.valid = true;
    p = std::move(q);
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
    AdamPlan& plan = h->adam_plan;
    if (!plan.valid || plan.key != key) {
        muon_status st = build_adam_plan(h, plan, ts, n, key, s);
        if (st != MUON_OK) return st;
    }
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
    hipError_t e;
    if (!plan.have_uploaded || std::memcmp(desc.data(), plan.uploaded.data(), sizeof(AdamDesc) * size_t(n)) != 0) {
        const int sl = plan.slot;
        if (plan.stage_used[sl]) {
            e = hipEventSynchronize(plan.stage_ev[sl]);
            if (e != hipSuccess) return hip_fail(h, e, "AdamW descriptor staging wait");
        }
        std::memcpy(plan.h_stage[sl], desc.data(), sizeof(AdamDesc) * size_t(n));
        e = hipMemcpyAsync(plan.d_desc, plan.h_stage[sl], sizeof(AdamDesc) * size_t(n), hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipEventRecord(plan.stage_ev[sl], s);
        if (e != hipSuccess) return hip_fail(h, e, "AdamW descriptor upload");
        plan.stage_used[sl] = true;
        plan.slot = (sl + 1) % kStageSlots;
        plan.uploaded = desc;
        plan.have_uploaded = true;
    }
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
        return launch_adamw(plan.d_chunks, plan.n_chunks, plan.d_desc, a, s, e0, e1);
    });
    if (e != hipSuccess) return hip_fail(h, e, "adamw launch");
    return MUON_OK;
}

muon_status muon_read_norms(muon_handle* h, float* out, int32_t n, void* stream) {
    if (!h || !out || n < 0) return MUON_ERR_INVALID_ARG;
    if (!h->step_plan.valid || n > h->step_plan.n) return fail(h, MUON_ERR_INVALID_ARG, "no step with %d matrices yet", n);
    if (n == 0) return MUON_OK;
    DeviceGuard g(h->device);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(out, h->step_plan.d_nu, sizeof(float) * n, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(h, e, "norm readback");
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
    return int64_t(h->step_plan.ws_bytes + h->ortho_plan.ws_bytes);
}

muon_status muon_destroy(muon_handle* h) {
    if (!h) return MUON_OK;
    {
        DeviceGuard g(h->device);
        (void)hipDeviceSynchronize();
        free_plan(h->step_plan);
        free_plan(h->ortho_plan);
        free_adam_plan(h->adam_plan);
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
