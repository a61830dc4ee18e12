// Host-only stand-ins for the kernel launchers, so that the C ABI layer
// (attn_api.cpp) can be built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU.  Each stand-in
// checks the launch parameters it receives the way the real launcher relies
// on them, records the call, and launches nothing.
#include "attn_fwd.h"
#include "attn_launch.h"
#include "abi_stubs.h"

#include <cmath>
#include <cstdio>
#include <cstdlib>

namespace stub {
int calls = 0;
int last = 0;  // which launcher ran last (LAUNCH_*)
attn_detail::LaunchArgs args;
attn_detail::DecodeArgs dargs;
void* k_out = nullptr;
}  // namespace stub

namespace {
void fail(const char* what) {
    std::fprintf(stderr, "launch parameters violate the launcher's assumptions: %s\n", what);
    std::abort();
}

void check(const attn_detail::LaunchArgs& a) {
    if (!a.q || !a.k || !a.v || !a.o) fail("null tensor");
    if (a.B <= 0 || a.S <= 0 || a.Hq <= 0 || a.Hkv <= 0 || a.Hq % a.Hkv) fail("sizes");
    if (!(a.scale > 0.0f) || !std::isfinite(a.scale)) fail("scale");
    if (a.causal != 0 && a.causal != 1) fail("causal");
    if (a.padded && !a.pad_lens) fail("padding without lengths");
    if (a.D % 16 || a.D < 16 || a.D > 256) fail("head dim");
    if (a.dtype != ATTN_F32 && a.dtype != ATTN_F16 && a.dtype != ATTN_BF16) fail("dtype");
}
}  // namespace

namespace attn_detail {

int launch(const LaunchArgs& a) {
    check(a);
    if (!attn_detail::tuned_head_dim(a.dtype, a.D)) fail("tuned kernel head dim");
    if (a.cu_seqlens && (a.total < a.S || a.total <= 0)) fail("packed rows");
    stub::args = a;
    stub::last = stub::LAUNCH_FWD;
    ++stub::calls;
    return ATTN_OK;
}

int launch_masked(const LaunchArgs& a) {
    check(a);
    if (!a.mask || a.dtype == ATTN_F32) fail("mask");
    stub::args = a;
    stub::last = stub::LAUNCH_MASKED;
    ++stub::calls;
    return ATTN_OK;
}

int launch_masked_tuned(const LaunchArgs& a) {
    check(a);
    if (!a.mask || a.dtype == ATTN_F32 || (a.D != 64 && a.D != 128)) fail("tuned mask kernel");
    if ((a.S * (a.mask_bool ? 1 : 2)) % 16 != 0) fail("mask rows of 16-byte multiples");
    stub::args = a;
    stub::last = stub::LAUNCH_MASKED_TUNED;
    ++stub::calls;
    return ATTN_OK;
}

int launch_general(const LaunchArgs& a) {
    check(a);
    if (a.dtype == ATTN_F32 || a.B > 65535) fail("general kernel");
    stub::args = a;
    stub::last = stub::LAUNCH_GENERAL;
    ++stub::calls;
    return ATTN_OK;
}

int launch_rope_k(const LaunchArgs& a, void* k_out) {
    check(a);
    if (!k_out || !a.rope) fail("rope");
    for (int i = 0; i < a.D / 2; ++i)
        if (!(a.rope_f[i] > 0.0) || !std::isfinite(a.rope_f[i])) fail("rope frequencies");
    stub::k_out = k_out;
    stub::last = stub::LAUNCH_ROPE_K;
    ++stub::calls;
    return ATTN_OK;
}

int64_t decode_splits(int64_t Sk) { return Sk > 256 ? Sk / 256 + (Sk % 256 != 0) : 1; }

int decode_scratch(void** ws) {
    static float fake[16];  // an address only; nothing is written through it
    *ws = fake;
    return ATTN_OK;
}

int launch_decode(const DecodeArgs& a) {
    if (!a.q || !a.o || !a.workspace) fail("decode tensors");
    if (a.Sk > 0 && (!a.k || !a.v)) fail("decode cache");
    if (a.B <= 0 || a.Sq <= 0 || a.Hq <= 0 || a.Hkv <= 0 || a.Hq % a.Hkv) fail("decode sizes");
    if (a.n_split != decode_splits(a.Sk)) fail("decode splits");
    if (!(a.scale > 0.0f)) fail("decode scale");
    stub::dargs = a;
    stub::last = stub::LAUNCH_DECODE;
    ++stub::calls;
    return ATTN_OK;
}

}  // namespace attn_detail
