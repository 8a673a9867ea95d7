// Drives every entry point of libwkv7's C ABI layer, built for the host only with
// the stub launchers, under AddressSanitizer and UndefinedBehaviorSanitizer.
// Pointers are fake, far-apart device addresses that the host layer only compares
// and never dereferences.  Every call's status (and, for accepted calls, which
// launcher ran with which sizes) is checked; the program exits non-zero on the
// first mismatch, and the sanitizers abort it on any memory or arithmetic fault
// in the validation code (sizes up to INT_MAX included).
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/wkv7.h"
#include "stub_log.h"

static int g_fail = 0;

static void expect(bool ok, const char *what, int line)
{
    if (!ok) {
        std::fprintf(stderr, "host_driver: line %d: %s\n", line, what);
        g_fail = 1;
    }
}
#define EXPECT(x) expect((x), #x, __LINE__)

static void *fake(int i, long long off = 0)
{
    return reinterpret_cast<void *>((1ull << 40) + (static_cast<unsigned long long>(i) << 34) + off);
}
static float *ffake(int i, long long off = 0) { return static_cast<float *>(fake(i, off)); }

static void reset_log() { g_log = StubLog{}; }

static int fwd(int B, int T, int H, int N = 64, int in_dt = WKV7_BF16, int o_dt = WKV7_F32, void *sout = nullptr,
               void *sin = fake(7))
{
    reset_log();
    return wkv7_forward(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), in_dt, static_cast<float *>(sin),
                        fake(6), o_dt, sout ? static_cast<float *>(sout) : ffake(8), B, T, H, N, nullptr);
}

static int step(int B, int T, int H, void *pos = fake(9), void *sout = fake(8))
{
    reset_log();
    return wkv7_step(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), WKV7_BF16, ffake(7), fake(6), WKV7_F32,
                     static_cast<float *>(sout), static_cast<float *>(pos), B, T, H, 64, nullptr);
}

int main()
{
    // ---- accepted calls reach the right launcher with the caller's sizes
    EXPECT(fwd(2, 40, 3) == WKV7_OK && g_log.calls == 1 && !std::strcmp(g_log.kind, "chunk"));
    EXPECT(g_log.B == 2 && g_log.T == 40 && g_log.H == 3 && g_log.seq.in_bf16 == 1 && g_log.seq.o_bf16 == 0);
    EXPECT(fwd(2, 8, 3) == WKV7_OK && !std::strcmp(g_log.kind, "step"));
    EXPECT(fwd(2, 9, 3) == WKV7_OK && !std::strcmp(g_log.kind, "chunk"));
    EXPECT(fwd(2, 0, 3) == WKV7_OK && !std::strcmp(g_log.kind, "copy") && g_log.n == 2LL * 3 * 64 * 64);
    EXPECT(fwd(2, 0, 3, 64, WKV7_BF16, WKV7_F32, fake(7)) == WKV7_OK && g_log.calls == 0);  // in place, T = 0
    EXPECT(fwd(2, 40, 3, 64, WKV7_F32, WKV7_BF16, fake(7)) == WKV7_OK && g_log.seq.state_out == ffake(7));
    EXPECT(step(4, 5, 6) == WKV7_OK && !std::strcmp(g_log.kind, "step") && g_log.seq.state_pos == ffake(9));
    EXPECT(step(4, 5, 6, fake(9), nullptr) == WKV7_OK && g_log.seq.state_out == nullptr);

    // ---- argument errors, before any launch
    EXPECT(fwd(2, 40, 3, 32) == WKV7_ERR_UNSUPPORTED && g_log.calls == 0);
    EXPECT(fwd(2, 40, 3, 64, 7) == WKV7_ERR_UNSUPPORTED && g_log.calls == 0);
    EXPECT(fwd(0, 40, 3) == WKV7_ERR_SHAPE && fwd(2, -1, 3) == WKV7_ERR_SHAPE && fwd(2, 40, 0) == WKV7_ERR_SHAPE);
    EXPECT(fwd(INT_MAX, INT_MAX, INT_MAX) == WKV7_ERR_SHAPE && g_log.calls == 0);
    EXPECT(fwd(1, INT_MAX, 1) == WKV7_ERR_ALIAS);  // fits int64; o then spans the next fake buffers
    EXPECT(fwd(1, 80, WKV7_MAX_H_CHUNK + 1) == WKV7_ERR_SHAPE);
    EXPECT(fwd(WKV7_MAX_HEADS_CHUNK + 1, 16, 1) == WKV7_ERR_SHAPE);
    EXPECT(step(WKV7_MAX_HEADS_STEP + 1, 5, 1) == WKV7_ERR_SHAPE && step(INT_MAX, 1, INT_MAX) == WKV7_ERR_SHAPE);
    EXPECT(fwd(2, 40, 3, 64, WKV7_BF16, WKV7_F32, fake(0)) == WKV7_ERR_ALIAS);     // state_out on r
    EXPECT(fwd(2, 40, 3, 64, WKV7_BF16, WKV7_F32, fake(7, 256)) == WKV7_ERR_ALIAS); // partly on state_in
    EXPECT(fwd(2, 40, 3, 64, WKV7_BF16, WKV7_F32, fake(8, 4)) == WKV7_ERR_ALIGN);
    EXPECT(step(4, 5, 6, fake(6, 1024)) == WKV7_ERR_ALIAS);  // state_pos inside o
    EXPECT(step(4, 5, 6, nullptr, nullptr) == WKV7_ERR_NULL);
    reset_log();
    EXPECT(wkv7_forward(nullptr, fake(1), fake(2), fake(3), fake(4), fake(5), WKV7_BF16, nullptr, fake(6), WKV7_F32,
                        ffake(8), 2, 5, 3, 64, nullptr) == WKV7_ERR_NULL);

    // ---- variable-length rows
    int *len = static_cast<int *>(fake(10));
    reset_log();
    EXPECT(wkv7_forward_varlen(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), WKV7_BF16, ffake(7), fake(6),
                               WKV7_F32, ffake(8), len, 3, 50, 2, 64, nullptr) == WKV7_OK &&
           g_log.seq.lengths == len && !std::strcmp(g_log.kind, "chunk"));
    reset_log();
    EXPECT(wkv7_forward_varlen(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), WKV7_BF16, ffake(7), fake(6),
                               WKV7_F32, ffake(8), static_cast<int *>(fake(8, 64)), 3, 50, 2, 64,
                               nullptr) == WKV7_ERR_ALIAS);
    EXPECT(wkv7_forward_varlen(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), WKV7_BF16, ffake(7), fake(6),
                               WKV7_F32, ffake(8), static_cast<int *>(fake(10, 2)), 3, 50, 2, 64,
                               nullptr) == WKV7_ERR_ALIGN);

    // ---- reset, commit
    reset_log();
    EXPECT(wkv7_state_reset(ffake(7), 5, 4, 64, nullptr, nullptr) == WKV7_OK && !std::strcmp(g_log.kind, "reset"));
    EXPECT(wkv7_state_reset(ffake(7), 5, 4, 64, static_cast<unsigned char *>(fake(7, 100)), nullptr) == WKV7_ERR_ALIAS);
    EXPECT(wkv7_state_reset(ffake(7, 8), 5, 4, 64, nullptr, nullptr) == WKV7_ERR_ALIGN);
    EXPECT(wkv7_state_reset(ffake(7), INT_MAX, INT_MAX, 64, nullptr, nullptr) == WKV7_ERR_SHAPE);
    reset_log();
    EXPECT(wkv7_state_commit(ffake(9), static_cast<int *>(fake(10)), ffake(7), ffake(7), 16, 5, 64, 64, nullptr) ==
               WKV7_OK && !std::strcmp(g_log.kind, "commit") && g_log.T == 5);
    EXPECT(wkv7_state_commit(ffake(9), static_cast<int *>(fake(10)), ffake(7), ffake(9, 4096), 16, 5, 64, 64,
                             nullptr) == WKV7_ERR_ALIAS);
    EXPECT(wkv7_state_commit(nullptr, static_cast<int *>(fake(10)), nullptr, ffake(8), 16, 5, 64, 64, nullptr) ==
           WKV7_ERR_NULL);

    // ---- the time-mix tail, fused and as a pass
    reset_log();
    EXPECT(wkv7_step_tail(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), WKV7_BF16, ffake(7), fake(11),
                          ffake(12), ffake(13), ffake(14), 1e-3f, fake(6), WKV7_F32, ffake(8), nullptr, 32, 1, 40, 64,
                          nullptr) == WKV7_OK &&
           g_log.seq.gate == fake(11) && g_log.seq.ln_w == ffake(13));
    EXPECT(wkv7_step_tail(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), WKV7_BF16, ffake(7), fake(6, 64),
                          ffake(12), ffake(13), ffake(14), 1e-3f, fake(6), WKV7_F32, ffake(8), nullptr, 32, 1, 40, 64,
                          nullptr) == WKV7_ERR_ALIAS);
    reset_log();
    EXPECT(wkv7_tmix_tail(fake(6), WKV7_F32, fake(0), fake(2), fake(3), fake(11), WKV7_BF16, ffake(12), ffake(13),
                          ffake(14), 1e-3f, fake(6), WKV7_F32, 4, 100, 64, 64, nullptr) == WKV7_OK &&
           g_log.n == 4LL * 100 * 64);
    EXPECT(wkv7_tmix_tail(fake(6), WKV7_F32, fake(0), fake(2), fake(3), fake(11), WKV7_BF16, ffake(12), ffake(13),
                          ffake(14), 1e-3f, fake(6), WKV7_BF16, 4, 100, 64, 64, nullptr) == WKV7_ERR_ALIAS);
    EXPECT(wkv7_tmix_tail(fake(6), WKV7_F32, fake(0), fake(2), fake(3), fake(11), WKV7_BF16, ffake(12), ffake(13),
                          ffake(14), 1e-3f, fake(15), WKV7_F32, INT_MAX, INT_MAX, INT_MAX, 64,
                          nullptr) == WKV7_ERR_SHAPE);

    // ---- the prefill with the fused tail: which kernels run
    auto ftail = [&](int in_dt, int x_dt, int T) {
        reset_log();
        return wkv7_forward_tail(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), in_dt, ffake(7), fake(11),
                                 ffake(12), ffake(13), ffake(14), 1e-3f, fake(6), x_dt, ffake(8), 4, T, 64, 64,
                                 nullptr);
    };
    EXPECT(ftail(WKV7_BF16, WKV7_F32, 100) == WKV7_OK && g_log.calls == 1 && !std::strcmp(g_log.kind, "chunk") &&
           g_log.seq.gate == fake(11));
    EXPECT(ftail(WKV7_BF16, WKV7_BF16, 8) == WKV7_OK && !std::strcmp(g_log.kind, "step") && g_log.seq.gate);
    EXPECT(ftail(WKV7_F32, WKV7_F32, 100) == WKV7_OK && g_log.calls == 2 && !std::strcmp(g_log.kind, "tail"));
    EXPECT(ftail(WKV7_F32, WKV7_BF16, 100) == WKV7_OK && g_log.calls == 1 && !std::strcmp(g_log.kind, "step") &&
           g_log.seq.gate == fake(11));
    EXPECT(ftail(WKV7_BF16, 3, 100) == WKV7_ERR_UNSUPPORTED && g_log.calls == 0);

    // ---- backward
    auto bwd = [&](void *dso, void *dsi, float *g0) {
        reset_log();
        return wkv7_backward(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), WKV7_BF16, ffake(7), ffake(9),
                             ffake(10), static_cast<float *>(dso), g0, ffake(12), ffake(13), ffake(14), ffake(15),
                             ffake(16), static_cast<float *>(dsi), 2, 30, 3, 64, nullptr);
    };
    EXPECT(bwd(fake(17), fake(18), ffake(11)) == WKV7_OK && !std::strcmp(g_log.kind, "backward"));
    EXPECT(bwd(fake(17), fake(17), ffake(11)) == WKV7_OK);                  // in place over d_state_out
    EXPECT(bwd(fake(17), fake(18), ffake(17, 1024)) == WKV7_ERR_ALIAS);     // a gradient inside d_state_out
    EXPECT(bwd(fake(17), fake(17, 256), ffake(11)) == WKV7_ERR_ALIAS);
    EXPECT(bwd(nullptr, nullptr, ffake(11)) == WKV7_ERR_NULL);
    EXPECT(bwd(fake(17), fake(18), ffake(11)) == WKV7_OK && g_log.bwd.state_pos == ffake(9) && !g_log.bwd.ckpt);

    // ---- the training pair: chunk checkpoints
    auto fck = [&](int T, void *sin, void *ck) {
        reset_log();
        return wkv7_forward_ckpt(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), WKV7_BF16,
                                 static_cast<float *>(sin), ffake(6), ffake(8), static_cast<float *>(ck), 2, T, 3,
                                 64, nullptr);
    };
    EXPECT(fck(40, fake(7), fake(9)) == WKV7_OK && g_log.calls == 1 && !std::strcmp(g_log.kind, "chunk") &&
           g_log.seq.ckpt == ffake(9) && !g_log.seq.state_pos && !g_log.seq.o_bf16);
    EXPECT(fck(8, fake(7), fake(9)) == WKV7_OK && g_log.calls == 2 && !std::strcmp(g_log.kind, "step") &&
           g_log.n == 2LL * 3 * 64 * 64 && !g_log.seq.ckpt);       // state_in in tile order, then the step kernel
    EXPECT(fck(1, nullptr, fake(9)) == WKV7_OK && g_log.calls == 2 && !std::strcmp(g_log.kind, "step"));
    EXPECT(fck(0, fake(7), nullptr) == WKV7_OK && !std::strcmp(g_log.kind, "copy"));
    EXPECT(fck(40, fake(7), nullptr) == WKV7_ERR_NULL && g_log.calls == 0);
    EXPECT(fck(40, fake(7), fake(9, 8)) == WKV7_ERR_ALIGN);
    EXPECT(fck(40, fake(7), fake(6, 1024)) == WKV7_ERR_ALIAS);    // inside o
    EXPECT(fck(40, fake(7), fake(7, 4096)) == WKV7_ERR_ALIAS);    // inside state_in
    // three chunks of 2 x 3 heads: o just below the checkpoints' end overlaps, at their end it does not
    const long long ck3 = 2LL * 3 * 3 * 64 * 64 * 4;
    reset_log();
    EXPECT(wkv7_forward_ckpt(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), WKV7_BF16, ffake(7),
                             ffake(9, ck3 - 16), ffake(8), ffake(9), 2, 40, 3, 64, nullptr) == WKV7_ERR_ALIAS);
    EXPECT(wkv7_forward_ckpt(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), WKV7_BF16, ffake(7),
                             ffake(9, ck3), ffake(8), ffake(9), 2, 40, 3, 64, nullptr) == WKV7_OK);
    auto bck = [&](void *ck, float *g0, void *dsi) {
        reset_log();
        return wkv7_backward_ckpt(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), WKV7_BF16, static_cast<float *>(ck),
                                  ffake(10), ffake(17), g0, ffake(12), ffake(13), ffake(14), ffake(15), ffake(16),
                                  static_cast<float *>(dsi), 2, 30, 3, 64, nullptr);
    };
    EXPECT(bck(fake(9), ffake(11), fake(18)) == WKV7_OK && !std::strcmp(g_log.kind, "backward_ckpt") &&
           g_log.bwd.ckpt == ffake(9) && !g_log.bwd.state_pos && !g_log.bwd.state_in && g_log.T == 30);
    // T = 30: two chunks; a gradient inside the second one's checkpoints overlaps
    const long long ck2 = 2LL * 2 * 3 * 64 * 64 * 4;
    EXPECT(bck(fake(9), ffake(9, ck2 - 16), fake(18)) == WKV7_ERR_ALIAS);
    EXPECT(bck(fake(9), ffake(9, ck2), fake(18)) == WKV7_OK);
    EXPECT(bck(nullptr, ffake(11), fake(18)) == WKV7_ERR_NULL && g_log.calls == 0);
    EXPECT(bck(fake(9, 4), ffake(11), fake(18)) == WKV7_ERR_ALIGN);
    EXPECT(bck(fake(9), ffake(11), fake(9)) == WKV7_ERR_ALIAS);

    // The checkpoints' tile order: a permutation of one state's N*N offsets, equal to the
    // formula the header documents, and the order the chunked kernel's stores and the
    // backward's loads assume (a wave's row tile is one contiguous kilobyte, a lane's four
    // rows of a column one 16-byte unit).
    {
        static bool seen[64 * 64];
        bool perm = true, documented = true, kernel = true;
        for (int i = 0; i < 64; ++i)
            for (int j = 0; j < 64; ++j) {
                const int off = wkv7::ckpt_offset(i, j);
                perm = perm && off >= 0 && off < 64 * 64 && !seen[off];
                if (off >= 0 && off < 64 * 64)
                    seen[off] = true;
                documented = documented && off == (j / 16) * 1024 + (i / 16) * 256 + (i / 4 % 4) * 64 + (j % 16) * 4 + i % 4;
            }
        for (int jb = 0; jb < 4; ++jb)
            for (int pt = 0; pt < 4; ++pt)
                for (int lane = 0; lane < 64; ++lane)
                    for (int e = 0; e < 4; ++e)
                        kernel = kernel && wkv7::ckpt_offset(16 * pt + 4 * (lane / 16) + e, 16 * jb + lane % 16) ==
                                               jb * 1024 + pt * 256 + lane * 4 + e;
        EXPECT(perm);
        EXPECT(documented);
        EXPECT(kernel);
    }

    for (int st = -8; st <= 2; ++st)
        EXPECT(wkv7_status_string(st) != nullptr && std::strlen(wkv7_status_string(st)) > 0);
    EXPECT(wkv7_abi_version() == WKV7_ABI_VERSION);

    if (g_fail)
        return 1;
    std::printf("host_driver: all checks passed\n");
    return 0;
}
