// Host-only stand-ins for the kernel launchers, so that the C ABI's host code (api.cpp) can be built with
// the host sanitizers and driven through every entry point without a GPU: each launcher only checks
// that the argument block it receives is self-consistent and returns success.
#include <cstdio>
#include <cstdlib>

#include "launch.h"

namespace attn {

static void need(bool ok, const char *what)
{
    if (!ok) {
        std::fprintf(stderr, "stub launcher: %s\n", what);
        std::abort();
    }
}

hipError_t launch_decode_split(const SplitArgs &a, int B, uint16_t *o, float *, hipStream_t)
{
    need(B > 0 && a.num_splits > 1 && a.G * a.Hkv == a.Hq && o && a.ws_o && a.ws_lse > a.ws_o, "split args");
    return hipSuccess;
}
hipError_t launch_decode_seq(const SeqArgs &a, int B, hipStream_t)
{
    need(B > 0 && a.G * a.Hkv == a.Hq && a.o, "sequential args");
    return hipSuccess;
}
hipError_t launch_decode_multi(const MultiArgs &a, int B, int total_q, uint16_t *o, float *, hipStream_t)
{
    need(B > 0 && total_q > 0 && a.ncb >= 1 && o && a.ws_lse > a.ws_o, "multi args");
    return hipSuccess;
}
hipError_t launch_smallseq(const SmallArgs &a, hipStream_t)
{
    need(a.B > 0 && a.max_s >= 0 && a.max_s <= 16 && a.o, "small-seq args");
    return hipSuccess;
}
hipError_t launch_prefill(const PrefillArgs &a, bool, int D, hipStream_t)
{
    need(a.B > 0 && (D == 64 || D == 128) && a.o, "prefill args");
    return hipSuccess;
}
hipError_t launch_prefill_d128(const PrefillArgs &a, hipStream_t)
{
    need(a.B > 0 && a.o && a.bt && a.seq_lens, "paged prefill args");
    return hipSuccess;
}
hipError_t launch_prefill_bwd(const BwdArgs &a, hipStream_t)
{
    need(a.B > 0 && a.dsum && a.lse2 > a.dsum && a.dq && a.dk && a.dv, "backward args");
    return hipSuccess;
}
hipError_t launch_smallseq_bwd(const SmallBwdArgs &a, hipStream_t)
{
    need(a.B > 0 && a.dq && a.dk && a.dv, "small-seq backward args");
    return hipSuccess;
}
hipError_t check_indices(const CheckSpec &, hipStream_t, CheckResult *out)
{
    out->code = 0;
    out->row = 0;
    return hipSuccess;
}

} // namespace attn
