// Host-side checks of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer: every
// sizing function over ordinary and extreme shapes, and every entry point with arguments that its
// validation rejects (those calls return before any HIP call, so no GPU is needed).  Exit status 0
// when every rejected call returned an error code; the sanitizers report any out-of-bounds access,
// overflow or other undefined behaviour on the way.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "glowq.h"

namespace {

int failures = 0;
volatile size_t sink = 0;  // keeps the sizing results alive

// A rejected call must return the status its validation names, before any HIP call (a HIP error
// here would mean the call got past its checks).
void check_status(int code, int expected, const char* what) {
    if (getenv("ABI_DRIVER_VERBOSE")) std::printf("%-16s %d\n", what, code);
    if (code != expected) {
        std::printf("FAIL: %s returned %d, expected %d\n", what, code, expected);
        ++failures;
    }
}

void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>((uintptr_t)0x10000 + off); }

}  // namespace

int main() {
    // sizing functions: ordinary, boundary and out-of-range shapes (must not overflow or crash)
    const int64_t Ts[] = {-1, 0, 1, 15, 16, 17, 64, 65, 2048, (int64_t)1 << 20, ((int64_t)1 << 20) + 1,
                          (int64_t)1 << 40};
    const int64_t ds[] = {-128, 0, 100, 128, 4096, 14336, (int64_t)1 << 20, ((int64_t)1 << 20) + 128,
                          (int64_t)1 << 40};
    const int32_t rs[] = {-8, 0, 8, 12, 64, 256, 264, 1 << 30};
    for (int64_t T : Ts)
        for (int32_t r : rs)
            for (int32_t p : {0, 1, 8, 9}) sink += glowq_workspace_bytes(T, r, p);
    for (int64_t T : Ts)
        for (int64_t d : ds)
            for (int32_t r : rs) {
                sink += glowq_w4a8_workspace_bytes(T, d, r);
                sink += glowq_mx8_workspace_bytes(T, d, r);
                sink += glowq_second_moment_workspace_bytes(T, d);
                for (int32_t share : {-1, 0, 1, 2}) sink += glowq_moe_workspace_bytes(T, d, r, share);
            }
    const int64_t ns[] = {-1, 0, 1, 16, 17, 4096, (int64_t)1 << 24, ((int64_t)1 << 24) + 1, (int64_t)1 << 40};
    for (int64_t n : ns) {
        sink += glowq_ner_workspace_bytes(n);
        for (int64_t k : ds) {
            sink += glowq_q_bytes(n, k) + glowq_sz_bytes(n, k);
            for (int32_t f : {-1, 0, 1, 2, 3, 4}) sink += glowq_mx_q_bytes(f, n, k);
            for (int32_t kk : {0, 8, 72, 1 << 20})
                for (int32_t r : rs) sink += glowq_solve_workspace_bytes(n, k, kk, r);
        }
    }
    sink += glowq_static_scratch_bytes();
    for (int s = -12; s <= 2; ++s) sink += (size_t)glowq_status_string(s)[0];
    sink += (size_t)glowq_version();

    // forward entry points with rejected arguments
    glowq_qweight w{};
    w.q = fake();
    w.sz = fake();
    w.n_out = 32;
    w.k_in = 256;
    glowq_qweight w_bad = w;
    w_bad.k_in = 384;
    glowq_qweight w_fmt = w;
    w_fmt.format = 7;
    const void* a1[1] = {fake()};
    void* y1[1] = {fake()};
    const void* a_null[1] = {nullptr};
    void* y_mis[1] = {fake(2)};
    const size_t big = (size_t)1 << 24;
    check_status(glowq_group_forward(nullptr, 4, 256, 1, &w, fake(), a1, 8, 1, fake(), big, y1, nullptr), GLOWQ_ERR_INVALID_ARG, "null x");
    check_status(glowq_group_forward(fake(), 4, 100, 1, &w, fake(), a1, 8, 1, fake(), big, y1, nullptr), GLOWQ_ERR_SHAPE, "d % 128");
    check_status(glowq_group_forward(fake(), -1, 256, 1, &w, fake(), a1, 8, 1, fake(), big, y1, nullptr), GLOWQ_ERR_SHAPE, "T < 0");
    check_status(glowq_group_forward(fake(), 4, 256, 0, &w, fake(), a1, 8, 1, fake(), big, y1, nullptr), GLOWQ_ERR_SHAPE, "m = 0");
    check_status(glowq_group_forward(fake(), 4, 256, 9, &w, fake(), a1, 8, 1, fake(), big, y1, nullptr), GLOWQ_ERR_UNSUPPORTED, "m = 9");
    check_status(glowq_group_forward(fake(), 4, 256, 1, &w, fake(), a1, 264, 1, fake(), big, y1, nullptr), GLOWQ_ERR_UNSUPPORTED, "r = 264");
    check_status(glowq_group_forward(fake(), 4, 256, 1, &w, fake(), a1, 12, 1, fake(), big, y1, nullptr), GLOWQ_ERR_UNSUPPORTED, "r % 8");
    check_status(glowq_group_forward(fake(), 4, 256, 1, &w_bad, fake(), a1, 8, 1, fake(), big, y1, nullptr), GLOWQ_ERR_SHAPE, "k_in");
    check_status(glowq_group_forward(fake(), 4, 256, 1, &w_fmt, fake(), a1, 8, 1, fake(), big, y1, nullptr), GLOWQ_ERR_INVALID_ARG, "format");
    check_status(glowq_group_forward(fake(), 4, 256, 1, &w, fake(), a_null, 8, 1, fake(), big, y1, nullptr), GLOWQ_ERR_INVALID_ARG, "a null");
    check_status(glowq_group_forward(fake(), 4, 256, 1, &w, fake(), a1, 8, 1, fake(), big, y_mis, nullptr), GLOWQ_ERR_ALIGN, "y align");
    check_status(glowq_group_forward(fake(), 4, 256, 1, &w, fake(), a1, 8, 1, nullptr, big, y1, nullptr), GLOWQ_ERR_WORKSPACE, "no ws");
    check_status(glowq_group_forward(fake(), 4, 256, 1, &w, fake(), a1, 8, 1, fake(), 100, y1, nullptr), GLOWQ_ERR_WORKSPACE, "small ws");
    check_status(glowq_group_forward(fake(), (int64_t)1 << 19, 4096, 1, &w, fake(), a1, 8, 1, fake(), big, y1, nullptr), GLOWQ_ERR_UNSUPPORTED, "T d over 2^30");
    check_status(glowq_group_forward(fake(), (int64_t)1 << 40, 4096, 1, &w, fake(), a1, 8, 1, fake(), big, y1, nullptr), GLOWQ_ERR_UNSUPPORTED, "T 2^40");
    check_status(glowq_solo_forward(fake(), 4, 256, nullptr, fake(), fake(), 8, 1, fake(), big, fake(), nullptr), GLOWQ_ERR_INVALID_ARG, "solo w");
    check_status(glowq_solo_forward(fake(), 4, 256, &w, nullptr, fake(), 8, 1, fake(), big, fake(), nullptr), GLOWQ_ERR_INVALID_ARG, "solo b");
    const void* b2[2] = {fake(), nullptr};
    const void* a2[2] = {fake(), fake()};
    void* y2[2] = {fake(), fake()};
    glowq_qweight w2[2] = {w, w};
    check_status(glowq_layerwise_forward(fake(), 4, 256, 2, w2, b2, a2, 8, 1, fake(), big, y2, nullptr), GLOWQ_ERR_INVALID_ARG, "layerwise b");
    check_status(glowq_group_forward_static(fake(), 1 << 16, 256, 1, &w, fake(), a1, 256, 1, y1, nullptr), GLOWQ_ERR_WORKSPACE, "static scratch");
    check_status(glowq_group_forward_w4a8(fake(), 4, 32768, 1, &w, fake(), a1, 8, 1, fake(), big, y1, nullptr), GLOWQ_ERR_SHAPE, "w4a8 d");
    glowq_qweight w_mx = w;
    w_mx.format = GLOWQ_FMT_MXFP4;
    check_status(glowq_group_forward_w4a8(fake(), 4, 256, 1, &w_mx, fake(), a1, 8, 1, fake(), big, y1, nullptr), GLOWQ_ERR_UNSUPPORTED, "w4a8 mx");
    check_status(glowq_group_forward_mx8(fake(), 4, 256, 1, &w, fake(), a1, 8, 1, fake(), big, y1, nullptr), GLOWQ_ERR_UNSUPPORTED, "mx8 int4");
    glowq_qweight wm2[2] = {w_mx, w_mx};
    wm2[1].format = GLOWQ_FMT_MXFP6_E2M3;
    check_status(glowq_group_forward_mx8(fake(), 4, 256, 2, wm2, fake(), a2, 8, 1, fake(), big, y2, nullptr), GLOWQ_ERR_UNSUPPORTED, "mx8 mixed");
    check_status(glowq_workspace_init(nullptr, 1 << 20, nullptr), GLOWQ_ERR_INVALID_ARG, "ws init null");
    check_status(glowq_workspace_status(fake(16), 1 << 20, nullptr), GLOWQ_ERR_ALIGN, "ws status align");
    check_status(glowq_repack(fake(), fake(), fake(), 16, 100, fake(), fake(), (int32_t*)fake(), nullptr), GLOWQ_ERR_SHAPE, "repack k");
    check_status(glowq_repack_mx(9, fake(), fake(), 16, 128, fake(), fake(), nullptr, nullptr), GLOWQ_ERR_INVALID_ARG, "repack_mx fmt");
    check_status(glowq_dequant(&w, fake(), 7, nullptr), GLOWQ_ERR_INVALID_ARG, "dequant dtype");

    // mixture of experts
    glowq_moe_module mm{};
    mm.q = fake();
    mm.sz = fake();
    mm.a = fake();
    mm.y = fake();
    mm.n_out = 64;
    mm.k_in = 256;
    check_status(glowq_moe_forward(fake(), 4, 256, 0, 1, &mm, fake(), 0, 8, 1, nullptr, (const int32_t*)fake(), 8, fake(),
                                   big, nullptr), GLOWQ_ERR_UNSUPPORTED, "moe n_exp 0");
    check_status(glowq_moe_forward(fake(), 4, 256, 257, 1, &mm, fake(), 0, 8, 1, nullptr, (const int32_t*)fake(), 8,
                                   fake(), big, nullptr), GLOWQ_ERR_UNSUPPORTED, "moe n_exp 257");
    check_status(glowq_moe_forward(fake(), 4, 256, 8, 5, &mm, fake(), 0, 8, 1, nullptr, (const int32_t*)fake(), 8, fake(),
                                   big, nullptr), GLOWQ_ERR_UNSUPPORTED, "moe m 5");
    check_status(glowq_moe_forward(fake(), 4, 256, 8, 1, &mm, fake(), 2, 8, 1, nullptr, (const int32_t*)fake(), 8, fake(),
                                   big, nullptr), GLOWQ_ERR_INVALID_ARG, "moe share");
    check_status(glowq_moe_forward(fake(), 4, 256, 8, 1, &mm, fake(), 0, 8, 1, nullptr, nullptr, 8, fake(), big, nullptr), GLOWQ_ERR_INVALID_ARG, "moe offsets");

    // decoder-layer schedule
    glowq_unit u{};
    u.kind = 3;
    u.m = 1;
    u.x = fake();
    u.T = 4;
    u.d = 256;
    u.w = &w;
    u.b = fake();
    u.a = a1;
    u.r = 8;
    u.restore = 1;
    u.y = y1;
    check_status(glowq_path_forward(&u, 1, fake(), big, nullptr), GLOWQ_ERR_INVALID_ARG, "path kind");
    check_status(glowq_path_forward(nullptr, 1, fake(), big, nullptr), GLOWQ_ERR_INVALID_ARG, "path null");

    // restore selection, second moment, factor solve
    check_status(glowq_restore_topk(nullptr, 32, 7, 16, (double*)fake(), (int32_t*)fake(), nullptr), GLOWQ_ERR_INVALID_ARG, "topk null");
    check_status(glowq_restore_topk((const double*)fake(), 0, 7, 0, (double*)fake(), (int32_t*)fake(), nullptr), GLOWQ_ERR_SHAPE, "topk units 0");
    check_status(glowq_restore_topk((const double*)fake(), 32, 7, 33, (double*)fake(), (int32_t*)fake(), nullptr), GLOWQ_ERR_SHAPE, "topk k");
    check_status(glowq_restore_select((const double*)fake(), 32, 7, 16, -1.0, (double*)fake(), (int32_t*)fake(),
                                      nullptr), GLOWQ_ERR_INVALID_ARG, "select tol");
    check_status(glowq_restore_select((const double*)fake(), 32, 7, 16, 2.0, (double*)fake(), (int32_t*)fake(),
                                      nullptr), GLOWQ_ERR_INVALID_ARG, "select tol 2");
    std::vector<int64_t> extremes = {-1, 0, (int64_t)1 << 40};
    for (int64_t N : extremes)
        check_status(glowq_second_moment(fake(), N, 4096, (float*)fake(), fake(), big, nullptr),
                     N == ((int64_t)1 << 40) ? GLOWQ_ERR_UNSUPPORTED : GLOWQ_ERR_SHAPE, "moment N");
    check_status(glowq_second_moment(fake(), 64, 100, (float*)fake(), fake(), big, nullptr), GLOWQ_ERR_SHAPE, "moment d");
    const double* dp = (const double*)fake();
    double* dq = (double*)fake(64);
    check_status(glowq_solve_factors(nullptr, 64, 256, dp, dp, 8, 8, 1, dq, dq, dq, fake(), big, nullptr), GLOWQ_ERR_INVALID_ARG, "solve e");
    check_status(glowq_solve_factors(dp, 64, 256, dp, dp, 8, 4, 1, dq, dq, dq, fake(), big, nullptr), GLOWQ_ERR_SHAPE, "solve k < r");
    check_status(glowq_solve_factors(dp, 64, 256, dp, dp, 8, 8, 17, dq, dq, dq, fake(), big, nullptr), GLOWQ_ERR_SHAPE, "solve q");
    check_status(glowq_solve_factors(dp, 64, 256, dp, dp, 8, 8, 1, dq, dq, dq, fake(), 64, nullptr), GLOWQ_ERR_WORKSPACE, "solve ws");
    check_status(glowq_ec_score(dp, 64, 256, dp, dp, 65, dq, fake(), big, nullptr), GLOWQ_ERR_SHAPE, "ec r");
    for (int64_t m : extremes)
        for (int64_t d : ds) sink += glowq_ec_score_workspace_bytes(m, d);

    std::printf("%s (%d failures, sink %zu)\n", failures ? "FAILED" : "OK", failures, (size_t)sink);
    return failures ? 1 : 0;
}
