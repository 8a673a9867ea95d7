// Stand-ins for the kernel launchers of libwkv7, for a host-only build of its C ABI
// layer (wkv7_api.hip) under AddressSanitizer and UndefinedBehaviorSanitizer.  Each
// records the call it received; nothing touches a device.
#include <cstring>

#include "../../rwkv_linear_attention_amd/csrc/wkv7_launch.h"
#include "stub_log.h"

StubLog g_log;

static hipError_t note(const char *kind, int B, int T, int H)
{
    g_log.calls += 1;
    std::strncpy(g_log.kind, kind, sizeof(g_log.kind) - 1);
    g_log.B = B;
    g_log.T = T;
    g_log.H = H;
    return hipSuccess;
}

namespace wkv7 {

hipError_t launch_step(const SeqArgs &a, hipStream_t)
{
    g_log.seq = a;
    return note("step", a.B, a.T, a.H);
}
hipError_t launch_chunk(const SeqArgs &a, hipStream_t)
{
    g_log.seq = a;
    return note("chunk", a.B, a.T, a.H);
}
hipError_t launch_state_copy(const float *, float *, long long n, hipStream_t)
{
    g_log.n = n;
    return note("copy", 0, 0, 0);
}
hipError_t launch_state_reset(float *, int B, int H, const unsigned char *, hipStream_t)
{
    return note("reset", B, 0, H);
}
hipError_t launch_ckpt_from_state(const float *, float *, int B, int H, hipStream_t)
{
    g_log.n = static_cast<long long>(B) * H * 64 * 64;
    return note("ckpt_from_state", B, 0, H);
}
hipError_t launch_tail(const TailArgs &a, hipStream_t)
{
    g_log.n = a.rows;
    return note("tail", 0, 0, a.H);
}
hipError_t launch_backward(const BwdArgs &a, hipStream_t)
{
    g_log.bwd = a;
    return note("backward", a.B, a.T, a.H);
}
hipError_t launch_backward_chunked(const BwdArgs &a, hipStream_t)
{
    g_log.bwd = a;
    return note("backward_ckpt", a.B, a.T, a.H);
}
hipError_t launch_state_commit(const float *, const int *, const float *, float *, int B, int T, int H,
                               hipStream_t)
{
    return note("commit", B, T, H);
}

}  // namespace wkv7
