// Host-side checks of the C ABI's argument validation and workspace sizing,
// built with AddressSanitizer and UndefinedBehaviorSanitizer on the host
// code (tests/test_sanitizers.py).  Every call here returns before any
// launch, so no GPU is needed; device pointers are stand-in addresses that
// are never dereferenced.  Exit status 0 when every status code matches.
#include <climits>
#include <cstdint>
#include <cstdio>

#include "gdn2.h"

namespace {

int failures = 0;

void expect(int got, int want, const char* what) {
    if (got != want) {
        std::printf("FAIL %s: got %d, want %d\n", what, got, want);
        ++failures;
    }
}

void* P(uintptr_t x) { return reinterpret_cast<void*>(x << 12); }
float* F(uintptr_t x) { return static_cast<float*>(P(x)); }
const int32_t* CU(uintptr_t x) { return static_cast<const int32_t*>(P(x)); }

struct Fwd {
    const void *q = P(1), *k = P(2), *v = P(3), *alpha = P(4), *b = P(5), *w = P(6);
    int32_t gates = GDN2_GATES_FULL, erase = GDN2_ERASE_READ, in_dtype = GDN2_BF16;
    const float* S0 = nullptr;
    void* o = P(7);
    int32_t out_dtype = GDN2_BF16;
    float* S_T = nullptr;
    const int32_t* cu = nullptr;
    int32_t num_seqs = 0, B = 1, T = 64, H = 1, dk = 128, dv = 128;
    void* ws = nullptr;
    size_t wsb = 0;
    int fwd() const {
        return gdn2_fwd(q, k, v, alpha, b, w, in_dtype, S0, o, out_dtype, S_T, cu, num_seqs, B, T,
                        H, dk, dv, ws, wsb, nullptr);
    }
    int gated() const {
        return gdn2_fwd_gates(q, k, v, alpha, b, w, gates, in_dtype, S0, o, out_dtype, S_T, cu,
                              num_seqs, B, T, H, dk, dv, ws, wsb, nullptr);
    }
    int ex() const {
        return gdn2_fwd_ex(q, k, v, alpha, b, w, gates, erase, in_dtype, S0, o, out_dtype, S_T,
                           cu, num_seqs, B, T, H, dk, dv, ws, wsb, nullptr);
    }
    int noalloc() const {
        return gdn2_fwd_noalloc(q, k, v, alpha, b, w, gates, in_dtype, S0, o, out_dtype, S_T, cu,
                                num_seqs, B, T, H, dk, dv, nullptr);
    }
};

struct Dec {
    const void *q = P(1), *k = P(2), *v = P(3), *alpha = P(4), *b = P(5), *w = P(6);
    int32_t gates = GDN2_GATES_FULL, erase = GDN2_ERASE_READ, in_dtype = GDN2_BF16;
    float* S = F(8);
    void* o = P(7);
    int32_t out_dtype = GDN2_BF16, N = 4, H = 2, dk = 128, dv = 128;
    int run() const {
        return gdn2_decode_ex(q, k, v, alpha, b, w, gates, erase, in_dtype, S, o, out_dtype, N, H,
                              dk, dv, nullptr);
    }
};

struct Bwd {
    const void *q = P(1), *k = P(2), *v = P(3), *alpha = P(4), *b = P(5), *w = P(6);
    int32_t in_dtype = GDN2_BF16;
    const float* S0 = nullptr;
    const void* dout = P(9);
    const float* dS_T = nullptr;
    void *dq = P(10), *dk = P(11), *dv = P(12), *dalpha = P(13), *db = P(14), *dw = P(15);
    int32_t grad_dtype = GDN2_BF16;
    float* dS0 = nullptr;
    const int32_t* cu = nullptr;
    int32_t num_seqs = 0, B = 1, T = 64, H = 1, dkd = 128, dvd = 128;
    void* ws = nullptr;
    size_t wsb = 0;
    int run() const {
        return gdn2_bwd(q, k, v, alpha, b, w, in_dtype, S0, dout, dS_T, dq, dk, dv, dalpha, db,
                        dw, grad_dtype, dS0, cu, num_seqs, B, T, H, dkd, dvd, ws, wsb, nullptr);
    }
};

struct Pro {
    const void *xq = P(1), *xk = P(2), *xv = P(3), *ga = P(4), *gb = P(5), *gw = P(6);
    const float *Wq = F(20), *Wk = F(21), *Wv = F(22);
    int32_t K = 4;
    float eps = 1e-6f;
    void *q = P(30), *k = P(31), *v = P(32), *alpha = P(33), *b = P(34), *w = P(35);
    const int32_t* cu = nullptr;
    int32_t num_seqs = 0, B = 1, T = 64, H = 2, dk = 128, dv = 128, dtype = GDN2_BF16;
    int run() const {
        return gdn2_prologue(xq, xk, xv, ga, gb, gw, Wq, Wk, Wv, K, eps, q, k, v, alpha, b, w, cu,
                             num_seqs, B, T, H, dk, dv, dtype, nullptr);
    }
};

}  // namespace

int main() {
    // status strings and version
    for (int s = -6; s <= 2; ++s)
        if (!gdn2_status_string(s)) expect(0, 1, "status string is never null");
    expect(gdn2_version() >= 1, 1, "version");

    // ---- forward ----
    { Fwd a; a.q = nullptr; expect(a.fwd(), GDN2_ERR_INVALID_ARG, "fwd q null"); }
    { Fwd a; a.o = nullptr; expect(a.fwd(), GDN2_ERR_INVALID_ARG, "fwd o null"); }
    { Fwd a; a.B = 0; expect(a.fwd(), GDN2_ERR_INVALID_ARG, "fwd B = 0"); }
    { Fwd a; a.T = -1; expect(a.fwd(), GDN2_ERR_INVALID_ARG, "fwd T < 0"); }
    { Fwd a; a.H = 0; expect(a.fwd(), GDN2_ERR_INVALID_ARG, "fwd H = 0"); }
    { Fwd a; a.cu = CU(40); a.B = 2; a.num_seqs = 2; expect(a.fwd(), GDN2_ERR_INVALID_ARG, "fwd packed B != 1"); }
    { Fwd a; a.cu = CU(40); a.num_seqs = -1; expect(a.fwd(), GDN2_ERR_INVALID_ARG, "fwd num_seqs < 0"); }
    { Fwd a; a.dk = 96; expect(a.fwd(), GDN2_ERR_UNSUPPORTED, "fwd dk = 96"); }
    { Fwd a; a.dv = 32; expect(a.fwd(), GDN2_ERR_UNSUPPORTED, "fwd dv = 32"); }
    { Fwd a; a.in_dtype = 7; expect(a.fwd(), GDN2_ERR_UNSUPPORTED, "fwd in_dtype"); }
    { Fwd a; a.in_dtype = GDN2_F32; a.dk = 64; expect(a.fwd(), GDN2_ERR_UNSUPPORTED, "fwd fp32 in, bf16 out"); }
    { Fwd a; a.o = const_cast<void*>(a.q); expect(a.fwd(), GDN2_ERR_INVALID_ARG, "fwd o aliases q"); }
    { Fwd a; a.S_T = F(50); a.o = a.S_T; expect(a.fwd(), GDN2_ERR_INVALID_ARG, "fwd o aliases S_T"); }
    { Fwd a; a.H = 1 << 17; expect(a.fwd(), GDN2_ERR_INVALID_ARG, "fwd H d >= 2^24"); }
    { Fwd a; a.H = INT_MAX; a.dk = a.dv = 64; expect(a.fwd(), GDN2_ERR_INVALID_ARG, "fwd H = INT_MAX"); }
    { Fwd a; a.B = INT_MAX; a.H = 1 << 16; a.dk = a.dv = 64; expect(a.fwd(), GDN2_ERR_INVALID_ARG, "fwd N H too large"); }
    { Fwd a; a.q = a.k = a.v = a.alpha = a.b = a.w = nullptr; a.o = nullptr; a.T = 0; expect(a.fwd(), GDN2_OK, "fwd empty batch"); }
    { Fwd a; a.T = 65536; a.H = 16; expect(a.fwd(), GDN2_ERR_WORKSPACE, "fwd long context without workspace"); }
    { Fwd a; a.T = 65536; a.H = 16; a.ws = P(60); a.wsb = 1024; expect(a.fwd(), GDN2_ERR_WORKSPACE, "fwd workspace too small"); }
    // gate forms and erase readings
    { Fwd a; a.gates = 3; expect(a.gated(), GDN2_ERR_INVALID_ARG, "gates = 3"); }
    { Fwd a; a.gates = -1; expect(a.gated(), GDN2_ERR_INVALID_ARG, "gates = -1"); }
    { Fwd a; a.gates = GDN2_GATES_KDA; a.dk = 96; expect(a.gated(), GDN2_ERR_UNSUPPORTED, "KDA form dk = 96"); }
    { Fwd a; a.erase = 2; expect(a.ex(), GDN2_ERR_INVALID_ARG, "erase = 2"); }
    { Fwd a; a.erase = GDN2_ERASE_ROWS; a.q = nullptr; expect(a.ex(), GDN2_ERR_INVALID_ARG, "erase rows q null"); }
    { Fwd a; a.erase = GDN2_ERASE_ROWS; a.q = a.k = a.v = a.alpha = a.b = a.w = nullptr; a.o = nullptr; a.T = 0; expect(a.ex(), GDN2_OK, "erase rows empty batch"); }
    // the forward that allocates nothing
    { Fwd a; a.q = nullptr; expect(a.noalloc(), GDN2_ERR_INVALID_ARG, "noalloc q null"); }
    { Fwd a; a.dk = 96; expect(a.noalloc(), GDN2_ERR_UNSUPPORTED, "noalloc dk = 96"); }
    { Fwd a; a.cu = CU(40); a.num_seqs = 100; a.T = 200000; expect(a.noalloc(), GDN2_ERR_WORKSPACE, "noalloc plan beyond the scratch"); }

    // ---- decode ----
    { Dec a; a.q = nullptr; expect(a.run(), GDN2_ERR_INVALID_ARG, "decode q null"); }
    { Dec a; a.S = nullptr; expect(a.run(), GDN2_ERR_INVALID_ARG, "decode S null"); }
    { Dec a; a.N = -1; expect(a.run(), GDN2_ERR_INVALID_ARG, "decode N < 0"); }
    { Dec a; a.H = 0; expect(a.run(), GDN2_ERR_INVALID_ARG, "decode H = 0"); }
    { Dec a; a.dk = 32; expect(a.run(), GDN2_ERR_UNSUPPORTED, "decode dk = 32"); }
    { Dec a; a.in_dtype = GDN2_F32; expect(a.run(), GDN2_ERR_UNSUPPORTED, "decode fp32 in, bf16 out"); }
    { Dec a; a.o = a.S; expect(a.run(), GDN2_ERR_INVALID_ARG, "decode o aliases S"); }
    { Dec a; a.gates = 9; expect(a.run(), GDN2_ERR_INVALID_ARG, "decode gates = 9"); }
    { Dec a; a.erase = -3; expect(a.run(), GDN2_ERR_INVALID_ARG, "decode erase = -3"); }
    { Dec a; a.N = INT_MAX; a.H = INT_MAX; expect(a.run(), GDN2_ERR_INVALID_ARG, "decode grid too large"); }
    { Dec a; a.N = 0; a.q = nullptr; a.S = nullptr; expect(a.run(), GDN2_OK, "decode N = 0"); }

    // ---- backward ----
    { Bwd a; a.dout = nullptr; expect(a.run(), GDN2_ERR_INVALID_ARG, "bwd dout null"); }
    { Bwd a; a.dw = nullptr; expect(a.run(), GDN2_ERR_INVALID_ARG, "bwd dw null"); }
    { Bwd a; a.dq = const_cast<void*>(a.q); expect(a.run(), GDN2_ERR_INVALID_ARG, "bwd dq aliases q"); }
    { Bwd a; a.db = const_cast<void*>(a.dout); expect(a.run(), GDN2_ERR_INVALID_ARG, "bwd db aliases dout"); }
    { Bwd a; a.dv = a.dk; expect(a.run(), GDN2_ERR_INVALID_ARG, "bwd dv aliases dk"); }
    { Bwd a; a.dkd = 96; expect(a.run(), GDN2_ERR_UNSUPPORTED, "bwd dk = 96"); }
    { Bwd a; a.in_dtype = GDN2_F32; expect(a.run(), GDN2_ERR_UNSUPPORTED, "bwd fp32 in, bf16 grads"); }
    { Bwd a; expect(a.run(), GDN2_ERR_WORKSPACE, "bwd without workspace"); }

    // ---- mixer ----
    { Pro a; a.K = 0; expect(a.run(), GDN2_ERR_INVALID_ARG, "prologue width 0"); }
    { Pro a; a.K = 5; expect(a.run(), GDN2_ERR_INVALID_ARG, "prologue width 5"); }
    { Pro a; a.eps = -1.f; expect(a.run(), GDN2_ERR_INVALID_ARG, "prologue eps < 0"); }
    { Pro a; a.Wv = nullptr; expect(a.run(), GDN2_ERR_INVALID_ARG, "prologue conv_v null"); }
    { Pro a; a.k = const_cast<void*>(a.xk); expect(a.run(), GDN2_ERR_INVALID_ARG, "prologue k aliases xk"); }
    { Pro a; a.w = a.b; expect(a.run(), GDN2_ERR_INVALID_ARG, "prologue w aliases b"); }
    { Pro a; a.dtype = 3; expect(a.run(), GDN2_ERR_UNSUPPORTED, "prologue dtype"); }
    { Pro a; a.dv = 96; expect(a.run(), GDN2_ERR_UNSUPPORTED, "prologue dv = 96"); }
    { Pro a; a.cu = CU(40); a.B = 2; a.num_seqs = 2; expect(a.run(), GDN2_ERR_INVALID_ARG, "prologue packed B != 1"); }
    { Pro a; a.T = 0; expect(a.run(), GDN2_OK, "prologue empty"); }
    expect(gdn2_epilogue(P(1), P(2), nullptr, 1e-6f, P(3), -1, 2, 128, GDN2_BF16, GDN2_BF16, nullptr),
           GDN2_ERR_INVALID_ARG, "epilogue rows < 0");
    expect(gdn2_epilogue(P(1), P(2), nullptr, -1.f, P(3), 8, 2, 128, GDN2_BF16, GDN2_BF16, nullptr),
           GDN2_ERR_INVALID_ARG, "epilogue eps < 0");
    expect(gdn2_epilogue(P(1), P(2), nullptr, 1e-6f, P(1), 8, 2, 128, GDN2_BF16, GDN2_BF16, nullptr),
           GDN2_ERR_INVALID_ARG, "epilogue y aliases o");
    expect(gdn2_epilogue(P(1), P(2), nullptr, 1e-6f, P(3), 8, 2, 96, GDN2_BF16, GDN2_BF16, nullptr),
           GDN2_ERR_UNSUPPORTED, "epilogue dv = 96");
    expect(gdn2_epilogue(P(1), P(2), nullptr, 1e-6f, P(3), 8, 2, 128, GDN2_F32, GDN2_BF16, nullptr),
           GDN2_ERR_UNSUPPORTED, "epilogue fp32 in, bf16 out");
    expect(gdn2_epilogue(nullptr, nullptr, nullptr, 1e-6f, nullptr, 0, 2, 128, GDN2_BF16, GDN2_BF16, nullptr),
           GDN2_OK, "epilogue empty");

    // ---- workspace sizes over a grid that includes the extremes ----
    const int32_t Bs[] = {-1, 0, 1, 8, 1000, INT_MAX};
    const int32_t Ts[] = {-1, 0, 1, 64, 65536, INT_MAX};
    const int32_t Hs[] = {0, 1, 16, 1 << 20, INT_MAX};
    const int32_t Ns[] = {0, 1, 32, 100000, INT_MAX};
    const int32_t ds[] = {64, 96, 128};
    size_t sum = 0;
    for (int32_t B : Bs)
        for (int32_t T : Ts)
            for (int32_t H : Hs)
                for (int32_t N : Ns)
                    for (int32_t dk : ds)
                        for (int32_t dv : ds)
                            for (int32_t dt = 0; dt < 3; ++dt) {
                                sum += gdn2_fwd_workspace_size(B, T, H, dk, dv, N, dt);
                                sum += gdn2_bwd_workspace_size(B, T, H, dk, dv, N, dt);
                            }
    std::printf("workspace grid checksum %zu\n", sum);
    if (failures == 0) std::printf("OK\n");
    return failures == 0 ? 0 : 1;
}
