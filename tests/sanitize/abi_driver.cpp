// Exercises the host side of the C ABI (include/dn.h) -- size and layout
// queries over many shapes, and every rejection path of the entry points with
// pointers that are never dereferenced -- with the ABI layer (dn_api.cpp)
// built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py, which fails on any report.  No call here reaches a
// kernel launch, so no GPU is needed.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "dn.h"

static int bad = 0;
#define EXPECT(cond)                                                     \
    do {                                                                 \
        if (!(cond)) {                                                   \
            std::printf("abi driver: expectation failed: %s\n", #cond);  \
            bad = 1;                                                     \
        }                                                                \
    } while (0)

static dn_shape shape(int B, int H, int T, int d, int C, int dtype, int gate, unsigned flags = 0, float eps = 0.f) {
    dn_shape s;
    std::memset(&s, 0, sizeof(s));
    s.B = B; s.H = H; s.T = T; s.dk = d; s.dv = d; s.C = C; s.dtype = dtype; s.gate = gate; s.flags = flags; s.eps = eps;
    return s;
}

static void* P(uintptr_t i) { return reinterpret_cast<void*>(i << 30); }   // distinct, aligned, never read
static float* F(uintptr_t i) { return reinterpret_cast<float*>(P(i)); }

int main() {
    const int ds[] = {16, 32, 64, 128}, Cs[] = {16, 32, 64}, Ts[] = {0, 1, 63, 64, 65, 4096, 32768 + 7};
    for (int dtype = 0; dtype <= 1; ++dtype)
        for (int gate = 0; gate <= 2; ++gate)
            for (int d : ds)
                for (int C : Cs)
                    for (int T : Ts)
                        for (unsigned flags = 0; flags <= 3; ++flags) {
                            const dn_shape s = shape(2, 3, T, d, C, dtype, gate, flags, 1e-6f);
                            size_t so[7], wo[10];
                            const size_t sb = dn_states_bytes(&s);
                            if (dn_states_layout(&s, so) == DN_OK) EXPECT(so[6] == sb);
                            for (int pass = 0; pass <= 2; ++pass) {
                                const size_t wb = dn_workspace_bytes(&s, pass);
                                if (dn_workspace_layout(&s, pass, wo) == DN_OK) EXPECT(wo[9] == wb);
                            }
                        }
    // rejections
    dn_shape s = shape(1, 2, 100, 64, 64, 1, 1);
    const size_t ws = dn_workspace_bytes(&s, DN_PASS_FWD);
    EXPECT(ws > 0);
    EXPECT(dn_chunk_fwd(nullptr, P(1), P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, nullptr, P(7), ws, nullptr) == DN_ERR_INVALID);
    EXPECT(dn_chunk_fwd(&s, nullptr, P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, nullptr, P(7), ws, nullptr) == DN_ERR_INVALID);
    EXPECT(dn_chunk_fwd(&s, P(1), P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, nullptr, P(7), ws - 1, nullptr) == DN_ERR_WORKSPACE);
    EXPECT(dn_chunk_fwd(&s, P(1), P(2), P(3), F(4), F(5), nullptr, P(3), nullptr, nullptr, P(7), ws, nullptr) == DN_ERR_INVALID);
    EXPECT(std::strstr(dn_last_error(), "overlaps") != nullptr);
    EXPECT(dn_chunk_fwd(&s, reinterpret_cast<char*>(P(1)) + 4, P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, nullptr, P(7), ws, nullptr) == DN_ERR_INVALID);
    dn_shape bad_s = s;
    bad_s.C = 48;
    EXPECT(dn_chunk_fwd(&bad_s, P(1), P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, nullptr, P(7), ws, nullptr) == DN_ERR_UNSUPPORTED);
    bad_s = s;
    bad_s.flags = 8;
    EXPECT(dn_chunk_fwd(&bad_s, P(1), P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, nullptr, P(7), ws, nullptr) == DN_ERR_INVALID);
    bad_s = s;
    bad_s.flags = DN_FLAG_KACZMARZ;
    bad_s.eps = -1.f;
    EXPECT(dn_chunk_fwd(&bad_s, P(1), P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, nullptr, P(7), ws, nullptr) == DN_ERR_INVALID);
    bad_s = s;
    bad_s.dtype = 9;
    EXPECT(dn_chunk_fwd(&bad_s, P(1), P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, nullptr, P(7), ws, nullptr) == DN_ERR_DTYPE);
    const size_t wb = dn_workspace_bytes(&s, DN_PASS_BWD_RECOMPUTE);
    EXPECT(dn_chunk_bwd(&s, P(1), P(2), P(3), F(4), F(5), nullptr, P(8), nullptr, nullptr, P(9), P(10), P(11), F(12),
                        nullptr, nullptr, P(14), wb, nullptr) == DN_ERR_INVALID);   // dg missing with a gate
    EXPECT(dn_chunk_bwd(&s, P(1), P(2), P(3), F(4), F(5), nullptr, P(8), nullptr, nullptr, P(9), P(10), P(11), F(12),
                        F(13), nullptr, P(14), wb - 256, nullptr) == DN_ERR_WORKSPACE);
    EXPECT(dn_chunk_bwd(&s, P(1), P(2), P(3), F(4), F(5), nullptr, P(8), nullptr, nullptr, P(9), P(9), P(11), F(12),
                        F(13), nullptr, P(14), wb, nullptr) == DN_ERR_INVALID);   // dq and dk alias
    dn_shape big = shape(8, 16, 4096, 128, 64, 1, 1);
    EXPECT(dn_chunk_fwd_noalloc(&big, P(1), P(2), P(3), F(4), F(5), nullptr, P(6), nullptr, nullptr) == DN_ERR_WORKSPACE);
    dn_shape r = shape(2, 2, 3, 64, 64, 1, 2);
    r.dv = 40;
    EXPECT(dn_recurrent_fwd(&r, P(1), P(2), P(3), F(4), F(5), F(6), P(7), nullptr) == DN_ERR_UNSUPPORTED);
    r.dv = 64;
    EXPECT(dn_recurrent_fwd(&r, P(1), P(2), P(3), F(4), nullptr, F(6), P(7), nullptr) == DN_ERR_INVALID);
    EXPECT(dn_recurrent_phase_fwd(&r, P(1), P(2), P(3), F(4), F(5), nullptr, F(6), F(8), P(7), nullptr) == DN_ERR_INVALID);
    EXPECT(dn_recurrent_phase_fwd(&r, P(1), P(2), P(3), F(4), F(5), F(9), F(6), F(6), P(7), nullptr) == DN_ERR_INVALID);
    for (int st = 0; st >= -7; --st) EXPECT(dn_status_string(static_cast<dn_status>(st)) != nullptr);
    size_t offs[10];
    EXPECT(dn_workspace_layout(&s, 5, offs) == DN_ERR_INVALID);
    EXPECT(dn_workspace_layout(&s, 0, nullptr) == DN_ERR_INVALID);
    EXPECT(dn_states_layout(nullptr, offs) == DN_ERR_INVALID);
    std::printf(bad ? "abi driver: FAILED\n" : "abi driver: ok\n");
    return bad;
}
