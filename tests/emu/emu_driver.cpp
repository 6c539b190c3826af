// Test infrastructure: runs muon_step and muon_adamw_step of the library, built
// against the CPU stand-in of HIP (tests/emu/hip), on exactly sized host
// buffers, so AddressSanitizer reports any access outside a caller buffer or
// the workspace.  The stand-in runs the momentum pass's element arithmetic for
// real, so every new momentum element is also checked against beta m + g
// (position-dependent values, so a wrong index shows) and the padding between
// rows against its old value.  Usage: emu_driver SHAPES NS_STEPS DTYPE [BLOCK_ROWS [LD_PAD [SHIFT [GRAD [NOALLOC [DEBUG]]]]]]
//   SHAPES "RxC,RxC,...", DTYPE 0 = bf16, 1 = f32 (also selects fp32 compute),
//   BLOCK_ROWS > 0 cuts every matrix whose rows it divides into row blocks,
//   LD_PAD extra elements per row (views into wider buffers), SHIFT elements
//   by which every buffer starts past its allocation (unaligned bases).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "muon.h"

emu_idx threadIdx, blockIdx;
dim3 gridDim, blockDim;
long emu_launches = 0;
int emu_verbose = 0;

// position-dependent values, exact in bf16 (multiples of 1/16 up to 14/16)
static float grad_at(long i, long j) { return float((i * 37 + j * 11) % 29 - 14) * 0.0625f; }
static float mom_at(long q) { return float((q * 13) % 23 - 11) * 0.125f; }

int main(int argc, char** argv) {
    if (argc < 4) return 2;
    emu_verbose = std::getenv("EMU_VERBOSE") != nullptr;   // list every launch on stderr
    const std::string spec = argv[1];
    const int ns = std::atoi(argv[2]);
    const int dtype = std::atoi(argv[3]);
    const int block_rows = argc > 4 ? std::atoi(argv[4]) : 0;
    const long pad = argc > 5 ? std::atol(argv[5]) : 0;
    const long shift = argc > 6 ? std::atol(argv[6]) : 0;
    const double gval = argc > 7 ? std::atof(argv[7]) : 0.0;
    const bool noalloc = argc > 8 && std::atoi(argv[8]) != 0;
    const bool debug = argc > 9 && std::atoi(argv[9]) != 0;
    std::vector<std::pair<long, long>> shapes;
    for (size_t p = 0; p < spec.size();) {
        size_t q = spec.find(',', p);
        const std::string t = spec.substr(p, q == std::string::npos ? std::string::npos : q - p);
        shapes.push_back({std::atol(t.c_str()), std::atol(t.c_str() + t.find('x') + 1)});
        if (q == std::string::npos) break;
        p = q + 1;
    }
    const int es = dtype == 0 ? 2 : 4;
    std::vector<muon_matrix> mats;
    std::vector<void*> blocks_to_free;
    auto buf = [&](long r, long ld, long c, int bytes) {
        // exactly sized: the last row ends at its last element
        char* p = static_cast<char*>(std::calloc((r - 1) * ld + c + shift, bytes));
        blocks_to_free.push_back(p);
        return static_cast<void*>(p + shift * bytes);
    };
    for (auto [r, c] : shapes) {
        muon_matrix m{};
        const long ld = c + pad;
        m.param = buf(r, ld, c, es);
        void* g = buf(r, ld, c, es);
        for (long i = 0; i < r; ++i)
            for (long j = 0; j < c; ++j) {
                const float v = gval != 0.0 ? float(gval) : grad_at(i, j);
                if (es == 4) {
                    static_cast<float*>(g)[i * ld + j] = v;
                } else {
                    uint32_t u;
                    std::memcpy(&u, &v, 4);
                    static_cast<uint16_t*>(g)[i * ld + j] = uint16_t(u >> 16);
                }
            }
        m.grad = g;
        m.momentum = static_cast<float*>(buf(r, ld, c, 4));
        for (long q = 0; q < (r - 1) * ld + c; ++q) m.momentum[q] = mom_at(q);
        m.update_out = static_cast<float*>(buf(r, ld, c, 4));
        m.rows = r;
        m.cols = c;
        m.ld_param = m.ld_grad = m.ld_mom = m.ld_update = ld;
        m.dtype = dtype;
        if (block_rows > 0 && r % block_rows == 0) m.block_rows = block_rows;
        mats.push_back(m);
    }
    muon_handle* h = nullptr;
    if (muon_init(&h, 0, debug ? MUON_INIT_DEBUG : 0u) != MUON_OK) return 3;
    const float sched[6] = {3.4445f, -4.7750f, 2.0315f, 1.5f, -0.5f, 0.0f};
    muon_hparams hp{0.02f, 0.95f, 0.01f, 1e-7f, 3.4445f, -4.775f, 2.0315f, 1, ns,
                    dtype == 0 ? MUON_COMPUTE_BF16 : MUON_COMPUTE_FP32, ns == 2 ? sched : nullptr};
    int st;
    if (noalloc) {
        st = muon_step_noalloc(h, mats.data(), static_cast<int>(mats.size()), &hp, nullptr);
        if (st == MUON_OK) st = muon_step_noalloc(h, mats.data(), 1, &hp, nullptr);
    } else {
        st = muon_step(h, mats.data(), static_cast<int>(mats.size()), &hp, nullptr);
    }
    std::printf("step %d (%s) launches %ld\n", st, muon_last_error(h), emu_launches);
    // momentum: matrix k went through `calls` steps (the no-allocation run
    // repeats the first matrix alone); padding keeps its value
    long bad = 0;
    for (size_t k = 0; k < mats.size() && st == MUON_OK; ++k) {
        const muon_matrix& m = mats[k];
        const int calls = noalloc && k == 0 ? 2 : 1;
        for (long q = 0; q < (m.rows - 1) * m.ld_mom + m.cols; ++q) {
            const long i = q / m.ld_mom, j = q % m.ld_mom;
            float want = mom_at(q);
            if (j < m.cols) {
                float gv;
                if (gval != 0.0) gv = float(gval);
                else gv = grad_at(i, j);
                if (es == 2) {   // the stored bf16 gradient
                    uint32_t u;
                    std::memcpy(&u, &gv, 4);
                    u &= 0xFFFF0000u;
                    std::memcpy(&gv, &u, 4);
                }
                for (int t = 0; t < calls; ++t) want = std::fmaf(hp.beta, want, gv);
            }
            if (m.momentum[q] != want && bad++ < 5)
                std::printf("momentum of matrix %zu at (%ld, %ld): %g, want %g\n", k, i, j, m.momentum[q], want);
        }
    }
    std::printf("momentum mismatches %ld\n", bad);
    if (bad) st = -1;
    // AdamW over ragged sizes: vector path, ragged tail and scalar path
    const long sizes[5] = {1, 4095, 4096, 4097, 10001};
    std::vector<muon_adamw_tensor> ts;
    for (long n : sizes) {
        muon_adamw_tensor t{};
        t.param = buf(1, n, n, es);
        t.grad = buf(1, n, n, es);
        t.exp_avg = static_cast<float*>(buf(1, n, n, 4));
        t.exp_avg_sq = static_cast<float*>(buf(1, n, n, 4));
        t.numel = n;
        t.dtype = dtype;
        ts.push_back(t);
    }
    muon_adamw_hparams ah{1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, 1};
    const int st2 = muon_adamw_step(h, ts.data(), static_cast<int>(ts.size()), &ah, nullptr);
    std::printf("adamw %d (%s)\n", st2, muon_last_error(h));
    muon_destroy(h);
    for (void* p : blocks_to_free) std::free(p);
    return st != MUON_OK ? 4 : (st2 != MUON_OK ? 5 : 0);
}
