// Drives every entry point of the C ABI through its checks and its launch
// parameters, host side only (the launchers are the stand-ins of
// abi_stubs.cpp).  Built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_abi_sanitize.py: any overflow,
// out-of-bounds access or other undefined behaviour in the validation and
// packing code aborts the run; a wrong return code or launch parameter
// prints the case and exits non-zero.
#include "attn_fwd.h"
#include "abi_stubs.h"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include <limits>

namespace {

int n_cases = 0, n_bad = 0;

void expect(const char* name, int got, int want) {
    ++n_cases;
    if (got != want) {
        ++n_bad;
        std::printf("FAIL %s: returned %d (%s), expected %d\n", name, got, attn_strerror(got), want);
    }
}

void expect_true(const char* name, bool ok) {
    ++n_cases;
    if (!ok) {
        ++n_bad;
        std::printf("FAIL %s\n", name);
    }
}

// Distinct, 16-byte aligned fake device addresses (never dereferenced on
// the host), far enough apart that no two tensors of the cases overlap.
void* dev(int i) { return reinterpret_cast<void*>(uintptr_t(0x100000000ull) * uintptr_t(i + 1)); }

attn_tensor_t T(int i, int dt, int64_t B, int64_t S, int64_t H, int64_t D) {
    return attn_tensor_t{dev(i), dt, B, S, H, D};
}

struct Fwd {
    attn_tensor_t q, k, v, o;
    int mask_kind = ATTN_MASK_NONE;
    const int32_t* pad = nullptr;
    float scale = 0.0f;
    int causal = 1;
    int hq, hkv;
    float* lse = nullptr;
    Fwd(int dt, int64_t B, int64_t S, int hq_, int hkv_, int64_t D)
        : q(T(0, dt, B, S, hq_, D)), k(T(1, dt, B, S, hkv_, D)), v(T(2, dt, B, S, hkv_, D)),
          o(T(3, dt, B, S, hq_, D)), hq(hq_), hkv(hkv_) {}
    int run() { return attn_fwd(&q, &k, &v, mask_kind, pad, scale, causal, hq, hkv, &o, lse, nullptr); }
};

void fwd_cases() {
    const int64_t big = std::numeric_limits<int64_t>::max();
    {
        Fwd f(ATTN_BF16, 1, 2048, 32, 32, 128);
        stub::calls = 0;
        expect("fwd valid", f.run(), ATTN_OK);
        expect_true("fwd launched the tuned kernel", stub::calls == 1 && stub::last == stub::LAUNCH_FWD);
        expect_true("fwd default scale", std::fabs(stub::args.scale - 1.0f / std::sqrt(128.0f)) < 1e-7f);
        expect_true("fwd packed sizes", stub::args.B == 1 && stub::args.S == 2048 && stub::args.Hq == 32 &&
                                            stub::args.Hkv == 32 && stub::args.D == 128 && stub::args.causal == 1);
        for (float s : {-1.0f, std::nanf(""), std::numeric_limits<float>::infinity(), -0.0f}) {
            f.scale = s;
            expect("fwd scale fallback", f.run(), ATTN_OK);
            expect_true("fwd scale fallback value", std::fabs(stub::args.scale - 1.0f / std::sqrt(128.0f)) < 1e-7f);
        }
        f.scale = 0.25f;
        expect("fwd explicit scale", f.run(), ATTN_OK);
        expect_true("fwd explicit scale value", stub::args.scale == 0.25f);
    }
    {
        Fwd f(ATTN_F16, 2, 300, 8, 2, 176);
        stub::calls = 0;
        expect("fwd general head dim", f.run(), ATTN_OK);
        expect_true("fwd general kernel", stub::last == stub::LAUNCH_GENERAL && stub::calls == 1);
        for (int64_t d : {int64_t(80), int64_t(96), int64_t(112), int64_t(144), int64_t(160), int64_t(192),
                          int64_t(256)}) {
            Fwd t(ATTN_BF16, 1, 300, 8, 2, d);
            expect("fwd padded head dim", t.run(), ATTN_OK);
            expect_true("fwd padded head dim: tuned kernel", stub::last == stub::LAUNCH_FWD && stub::args.D == d);
        }
        Fwd g(ATTN_F32, 2, 300, 8, 2, 96);
        expect("fwd fp32 general head dim", g.run(), ATTN_ERR_UNSUPPORTED);
        Fwd h(ATTN_F32, 2, 300, 8, 2, 64);
        expect("fwd fp32 D64", h.run(), ATTN_OK);
        for (int64_t d : {int64_t(8), int64_t(72), int64_t(264), int64_t(0), big}) {
            Fwd x(ATTN_BF16, 1, 64, 4, 4, d);
            expect("fwd bad head dim", x.run(), ATTN_ERR_UNSUPPORTED);
        }
    }
    {
        Fwd f(ATTN_BF16, 1, 128, 4, 4, 64);
        stub::calls = 0;
        f.q.B = f.k.B = f.v.B = f.o.B = 0;
        expect("fwd B=0", f.run(), ATTN_OK);
        f.q.B = f.k.B = f.v.B = f.o.B = 1;
        f.q.S = f.k.S = f.v.S = f.o.S = 0;
        expect("fwd S=0", f.run(), ATTN_OK);
        expect_true("empty inputs launch nothing", stub::calls == 0);
    }
    // pointers, dtypes, shapes, heads
    {
        Fwd f(ATTN_BF16, 1, 128, 4, 4, 64);
        expect("fwd null q", attn_fwd(nullptr, &f.k, &f.v, 0, nullptr, 0.f, 0, 4, 4, &f.o, nullptr, nullptr),
               ATTN_ERR_NULL);
        expect("fwd null out", attn_fwd(&f.q, &f.k, &f.v, 0, nullptr, 0.f, 0, 4, 4, nullptr, nullptr, nullptr),
               ATTN_ERR_NULL);
        Fwd g = f;
        g.q.data = nullptr;
        expect("fwd null q data", g.run(), ATTN_ERR_NULL);
        g = f;
        g.v.dtype = 9;
        expect("fwd unknown dtype", g.run(), ATTN_ERR_DTYPE);
        g = f;
        g.k.dtype = ATTN_F16;
        expect("fwd mixed dtype", g.run(), ATTN_ERR_DTYPE);
        g = f;
        g.q.B = -1;
        expect("fwd negative B", g.run(), ATTN_ERR_SHAPE);
        g = f;
        g.v.S = 127;
        expect("fwd S mismatch", g.run(), ATTN_ERR_SHAPE);
        g = f;
        g.o.D = 128;
        expect("fwd D mismatch", g.run(), ATTN_ERR_SHAPE);
        g = f;
        g.hq = 0;
        expect("fwd zero heads", g.run(), ATTN_ERR_HEADS);
        g = f;
        g.hkv = 3;
        g.k.H = g.v.H = 3;
        expect("fwd Hq % Hkv", g.run(), ATTN_ERR_HEADS);
        g = f;
        g.q.H = 8;
        expect("fwd q heads vs n_q_heads", g.run(), ATTN_ERR_HEADS);
        Fwd h(ATTN_BF16, 1, 128, 70000, 70000, 64);
        expect("fwd too many heads", h.run(), ATTN_ERR_UNSUPPORTED);
    }
    // masks and alignment
    {
        Fwd f(ATTN_BF16, 2, 256, 4, 4, 128);
        f.causal = 2;
        expect("fwd causal 2", f.run(), ATTN_ERR_MASK);
        f.causal = 0;
        f.mask_kind = 7;
        expect("fwd unknown mask kind", f.run(), ATTN_ERR_MASK);
        f.mask_kind = ATTN_MASK_KEY_PADDING;
        expect("fwd padding without lengths", f.run(), ATTN_ERR_MASK);
        f.pad = reinterpret_cast<const int32_t*>(uintptr_t(dev(5)) + 2);
        expect("fwd misaligned lengths", f.run(), ATTN_ERR_ALIGN);
        f.pad = static_cast<const int32_t*>(dev(5));
        expect("fwd padding", f.run(), ATTN_OK);
        expect_true("fwd padding packed", stub::args.padded == 1 && stub::args.pad_lens == f.pad);
        f.mask_kind = ATTN_MASK_NONE;
        expect("fwd lengths without padding", f.run(), ATTN_ERR_MASK);
        f.pad = nullptr;
        f.q.data = reinterpret_cast<void*>(uintptr_t(dev(0)) + 8);
        expect("fwd misaligned q", f.run(), ATTN_ERR_ALIGN);
        f.q.data = dev(0);
        f.lse = reinterpret_cast<float*>(uintptr_t(dev(6)) + 2);
        expect("fwd misaligned lse", f.run(), ATTN_ERR_ALIGN);
    }
    // sizes at and past the limits: no overflow on the way to the error
    {
        for (int64_t s : {int64_t(1) << 29, big, big / 2 + 1}) {
            Fwd f(ATTN_BF16, 1, s, 4, 4, 128);
            expect("fwd S at the limit", f.run(), ATTN_ERR_UNSUPPORTED);
        }
        for (int64_t b : {big, big / 3, int64_t(1) << 40}) {
            Fwd f(ATTN_F32, b, 1 << 20, 65535, 65535, 128);
            expect("fwd huge batch", f.run(), ATTN_ERR_UNSUPPORTED);
        }
        Fwd f(ATTN_F32, 1, (int64_t(1) << 29) - 1, 64, 64, 128);
        expect("fwd K/V beyond 32-bit offsets", f.run(), ATTN_ERR_UNSUPPORTED);
    }
}

void varlen_cases() {
    attn_tensor_t q = T(0, ATTN_BF16, 1, 4096, 8, 64), k = T(1, ATTN_BF16, 1, 4096, 2, 64),
                  v = T(2, ATTN_BF16, 1, 4096, 2, 64), o = T(3, ATTN_BF16, 1, 4096, 8, 64);
    const int32_t* cu = static_cast<const int32_t*>(dev(4));
    stub::calls = 0;
    expect("varlen valid", attn_fwd_varlen(&q, &k, &v, cu, 5, 1500, 0.f, 1, 8, 2, &o, nullptr, nullptr), ATTN_OK);
    expect_true("varlen packed", stub::calls == 1 && stub::args.B == 5 && stub::args.S == 1500 &&
                                     stub::args.total == 4096 && stub::args.cu_seqlens == cu);
    expect("varlen null offsets", attn_fwd_varlen(&q, &k, &v, nullptr, 5, 1500, 0.f, 1, 8, 2, &o, nullptr, nullptr),
           ATTN_ERR_NULL);
    expect("varlen misaligned offsets",
           attn_fwd_varlen(&q, &k, &v, reinterpret_cast<const int32_t*>(uintptr_t(dev(4)) + 1), 5, 1500, 0.f, 1, 8,
                           2, &o, nullptr, nullptr),
           ATTN_ERR_ALIGN);
    expect("varlen negative count", attn_fwd_varlen(&q, &k, &v, cu, -1, 1500, 0.f, 1, 8, 2, &o, nullptr, nullptr),
           ATTN_ERR_SHAPE);
    expect("varlen max beyond T", attn_fwd_varlen(&q, &k, &v, cu, 5, 4097, 0.f, 1, 8, 2, &o, nullptr, nullptr),
           ATTN_ERR_SHAPE);
    expect("varlen zero sequences", attn_fwd_varlen(&q, &k, &v, cu, 0, 1500, 0.f, 1, 8, 2, &o, nullptr, nullptr),
           ATTN_OK);
    attn_tensor_t q2 = q, k2 = k, v2 = v, o2 = o;
    q2.B = k2.B = v2.B = o2.B = 2;
    expect("varlen batch of two", attn_fwd_varlen(&q2, &k2, &v2, cu, 5, 1500, 0.f, 1, 8, 2, &o2, nullptr, nullptr),
           ATTN_ERR_SHAPE);
    attn_tensor_t qh = T(0, ATTN_BF16, 1, 4096, 65535, 64), oh = T(3, ATTN_BF16, 1, 4096, 65535, 64),
                  kh = T(1, ATTN_BF16, 1, 4096, 65535, 64), vh = T(2, ATTN_BF16, 1, 4096, 65535, 64);
    expect("varlen too much work",
           attn_fwd_varlen(&qh, &kh, &vh, cu, 2147483647, 4096, 0.f, 1, 65535, 65535, &oh, nullptr, nullptr),
           ATTN_ERR_UNSUPPORTED);
}

void masked_cases() {
    attn_tensor_t q = T(0, ATTN_BF16, 2, 512, 8, 128), k = T(1, ATTN_BF16, 2, 512, 8, 128),
                  v = T(2, ATTN_BF16, 2, 512, 8, 128), o = T(3, ATTN_BF16, 2, 512, 8, 128);
    const void* m = dev(4);
    stub::calls = 0;
    expect("masked valid", attn_fwd_masked(&q, &k, &v, m, ATTN_MASK_ADDITIVE, 2, 1, 0.f, 0, 8, 8, &o, nullptr, nullptr),
           ATTN_OK);
    expect_true("masked packed", stub::last == stub::LAUNCH_MASKED_TUNED && stub::args.mask == m &&
                                     stub::args.mask_b == 1 && stub::args.mask_h == 0 && stub::args.mask_bool == 0);
    {
        // rows that are not 16-byte multiples, or other head dims: the general kernel
        attn_tensor_t q5 = q, k5 = k, v5 = v, o5 = o;
        q5.S = k5.S = v5.S = o5.S = 500;
        expect("masked unaligned rows",
               attn_fwd_masked(&q5, &k5, &v5, m, ATTN_MASK_ADDITIVE, 1, 1, 0.f, 1, 8, 8, &o5, nullptr, nullptr), ATTN_OK);
        expect_true("masked unaligned rows: general kernel", stub::last == stub::LAUNCH_MASKED);
        q5.S = k5.S = v5.S = o5.S = 520;
        expect("masked bool rows of 520 bytes",
               attn_fwd_masked(&q5, &k5, &v5, m, ATTN_MASK_BOOL, 1, 1, 0.f, 1, 8, 8, &o5, nullptr, nullptr), ATTN_OK);
        expect_true("masked bool 520: general kernel", stub::last == stub::LAUNCH_MASKED);
        expect("masked additive rows of 1040 bytes",
               attn_fwd_masked(&q5, &k5, &v5, m, ATTN_MASK_ADDITIVE, 1, 1, 0.f, 1, 8, 8, &o5, nullptr, nullptr), ATTN_OK);
        expect_true("masked additive 520: tuned kernel", stub::last == stub::LAUNCH_MASKED_TUNED);
        attn_tensor_t q9 = T(0, ATTN_BF16, 1, 256, 2, 96), k9 = T(1, ATTN_BF16, 1, 256, 2, 96),
                      v9 = T(2, ATTN_BF16, 1, 256, 2, 96), o9 = T(3, ATTN_BF16, 1, 256, 2, 96);
        expect("masked D96", attn_fwd_masked(&q9, &k9, &v9, m, 0, 1, 1, 0.f, 1, 2, 2, &o9, nullptr, nullptr), ATTN_OK);
        expect_true("masked D96: general kernel", stub::last == stub::LAUNCH_MASKED);
        attn_tensor_t qb = T(0, ATTN_BF16, 1, 40000, 1, 64), kb = T(1, ATTN_BF16, 1, 40000, 1, 64),
                      vb = T(2, ATTN_BF16, 1, 40000, 1, 64), ob = T(3, ATTN_BF16, 1, 40000, 1, 64);
        expect("masked plane of 3.2 GB", attn_fwd_masked(&qb, &kb, &vb, m, 0, 1, 1, 0.f, 1, 1, 1, &ob, nullptr, nullptr),
               ATTN_OK);
        expect_true("masked plane beyond 2^31 bytes: general kernel", stub::last == stub::LAUNCH_MASKED);
    }
    expect("masked bool", attn_fwd_masked(&q, &k, &v, m, ATTN_MASK_BOOL, 1, 8, 0.f, 1, 8, 8, &o, nullptr, nullptr),
           ATTN_OK);
    expect_true("masked bool packed", stub::args.mask_bool == 1 && stub::args.mask_b == 0 && stub::args.mask_h == 1 &&
                                          stub::last == stub::LAUNCH_MASKED_TUNED);
    expect("masked bad type", attn_fwd_masked(&q, &k, &v, m, 5, 1, 1, 0.f, 0, 8, 8, &o, nullptr, nullptr),
           ATTN_ERR_MASK);
    expect("masked bad batch dim", attn_fwd_masked(&q, &k, &v, m, 0, 3, 1, 0.f, 0, 8, 8, &o, nullptr, nullptr),
           ATTN_ERR_MASK);
    expect("masked bad head dim", attn_fwd_masked(&q, &k, &v, m, 0, 1, 4, 0.f, 0, 8, 8, &o, nullptr, nullptr),
           ATTN_ERR_MASK);
    expect("masked null mask", attn_fwd_masked(&q, &k, &v, nullptr, 0, 1, 1, 0.f, 0, 8, 8, &o, nullptr, nullptr),
           ATTN_ERR_NULL);
    expect("masked misaligned mask",
           attn_fwd_masked(&q, &k, &v, reinterpret_cast<const void*>(uintptr_t(dev(4)) + 4), 0, 1, 1, 0.f, 0, 8, 8,
                           &o, nullptr, nullptr),
           ATTN_ERR_ALIGN);
    attn_tensor_t q32 = q, k32 = k, v32 = v, o32 = o;
    q32.dtype = k32.dtype = v32.dtype = o32.dtype = ATTN_F32;
    expect("masked fp32", attn_fwd_masked(&q32, &k32, &v32, m, 0, 1, 1, 0.f, 0, 8, 8, &o32, nullptr, nullptr),
           ATTN_ERR_UNSUPPORTED);
    attn_tensor_t qb = T(0, ATTN_BF16, 70000, 16, 1, 64), kb = T(1, ATTN_BF16, 70000, 16, 1, 64),
                  vb = T(2, ATTN_BF16, 70000, 16, 1, 64), ob = T(3, ATTN_BF16, 70000, 16, 1, 64);
    expect("masked batch beyond the grid",
           attn_fwd_masked(&qb, &kb, &vb, m, 0, 1, 1, 0.f, 0, 1, 1, &ob, nullptr, nullptr), ATTN_ERR_UNSUPPORTED);
}

void rope_cases() {
    attn_tensor_t q = T(0, ATTN_BF16, 1, 1024, 8, 128), k = T(1, ATTN_BF16, 1, 1024, 8, 128),
                  v = T(2, ATTN_BF16, 1, 1024, 8, 128), o = T(3, ATTN_BF16, 1, 1024, 8, 128),
                  kr = T(4, ATTN_BF16, 1, 1024, 8, 128);
    stub::calls = 0;
    expect("rope valid", attn_fwd_rope(&q, &k, &v, 0, nullptr, 0.f, 1, 8, 8, nullptr, 0.f, &kr, &o, nullptr, nullptr),
           ATTN_OK);
    expect_true("rope two launches", stub::calls == 2 && stub::last == stub::LAUNCH_FWD && stub::k_out == kr.data &&
                                         stub::args.k == kr.data && stub::args.rope == 1);
    expect_true("rope default base", std::fabs(stub::args.rope_lb - std::log2(10000.0)) < 1e-12);
    for (float base : {-3.0f, std::nanf(""), std::numeric_limits<float>::infinity()}) {
        expect("rope base fallback",
               attn_fwd_rope(&q, &k, &v, 0, nullptr, 0.f, 1, 8, 8, nullptr, base, &kr, &o, nullptr, nullptr), ATTN_OK);
        expect_true("rope base fallback value", std::fabs(stub::args.rope_lb - std::log2(10000.0)) < 1e-12);
    }
    expect("rope in place", attn_fwd_rope(&q, &k, &v, 0, nullptr, 0.f, 1, 8, 8, nullptr, 500000.f, &k, &o, nullptr,
                                          nullptr),
           ATTN_OK);
    expect("rope null k_rot", attn_fwd_rope(&q, &k, &v, 0, nullptr, 0.f, 1, 8, 8, nullptr, 0.f, nullptr, &o, nullptr,
                                            nullptr),
           ATTN_ERR_NULL);
    attn_tensor_t bad = kr;
    bad.dtype = ATTN_F16;
    expect("rope k_rot dtype", attn_fwd_rope(&q, &k, &v, 0, nullptr, 0.f, 1, 8, 8, nullptr, 0.f, &bad, &o, nullptr,
                                             nullptr),
           ATTN_ERR_DTYPE);
    bad = kr;
    bad.S = 1023;
    expect("rope k_rot shape", attn_fwd_rope(&q, &k, &v, 0, nullptr, 0.f, 1, 8, 8, nullptr, 0.f, &bad, &o, nullptr,
                                             nullptr),
           ATTN_ERR_SHAPE);
    bad = kr;
    bad.data = reinterpret_cast<void*>(uintptr_t(k.data) + 4096);
    expect("rope k_rot inside k", attn_fwd_rope(&q, &k, &v, 0, nullptr, 0.f, 1, 8, 8, nullptr, 0.f, &bad, &o, nullptr,
                                                nullptr),
           ATTN_ERR_ALIAS);
    bad.data = o.data;
    expect("rope k_rot on out", attn_fwd_rope(&q, &k, &v, 0, nullptr, 0.f, 1, 8, 8, nullptr, 0.f, &bad, &o, nullptr,
                                              nullptr),
           ATTN_ERR_ALIAS);
    float* lse = static_cast<float*>(dev(4));
    expect("rope k_rot on lse", attn_fwd_rope(&q, &k, &v, 0, nullptr, 0.f, 1, 8, 8, nullptr, 0.f, &kr, &o, lse, nullptr),
           ATTN_ERR_ALIAS);
    expect("rope misaligned positions",
           attn_fwd_rope(&q, &k, &v, 0, nullptr, 0.f, 1, 8, 8, reinterpret_cast<const int32_t*>(uintptr_t(dev(7)) + 2),
                         0.f, &kr, &o, nullptr, nullptr),
           ATTN_ERR_ALIGN);
    attn_tensor_t q96 = T(0, ATTN_BF16, 1, 64, 2, 96), k96 = T(1, ATTN_BF16, 1, 64, 2, 96),
                  v96 = T(2, ATTN_BF16, 1, 64, 2, 96), o96 = T(3, ATTN_BF16, 1, 64, 2, 96),
                  r96 = T(4, ATTN_BF16, 1, 64, 2, 96);
    expect("rope general head dim", attn_fwd_rope(&q96, &k96, &v96, 0, nullptr, 0.f, 1, 2, 2, nullptr, 0.f, &r96, &o96,
                                                  nullptr, nullptr),
           ATTN_ERR_UNSUPPORTED);
}

void decode_cases() {
    const int64_t big = std::numeric_limits<int64_t>::max();
    expect("workspace negative", int(attn_decode_workspace_bytes(-1, 1, 8, 128, 10)), -1);
    expect_true("workspace value", attn_decode_workspace_bytes(2, 3, 8, 128, 1000) == 1024 + 4 * 2 * 8 * 3 * 131 * 4);
    expect_true("workspace empty cache", attn_decode_workspace_bytes(1, 1, 1, 64, 0) == 1024 + 67 * 4);
    expect_true("workspace overflow", attn_decode_workspace_bytes(big, big, 65535, 128, big) == -1);
    expect_true("workspace overflow D", attn_decode_workspace_bytes(1, 1, 1, big, 10) == -1);
    // partials fit int64 (4 * (big / 4) = big - 3), the counter header does not
    expect_true("workspace overflow by the counters", attn_decode_workspace_bytes(1, 1, 1, big / 4 - 3, 0) == -1);
    expect_true("workspace overflow near the edge",
                attn_decode_workspace_bytes(int64_t(1) << 30, int64_t(1) << 19, 65535, 256, (int64_t(1) << 29) - 1) ==
                    -1);

    attn_tensor_t q = T(0, ATTN_BF16, 8, 1, 64, 128), kc = T(1, ATTN_BF16, 8, 4096, 8, 128),
                  vc = T(2, ATTN_BF16, 8, 4096, 8, 128), o = T(3, ATTN_BF16, 8, 1, 64, 128);
    const int32_t* lens = static_cast<const int32_t*>(dev(5));
    const int64_t need = attn_decode_workspace_bytes(8, 1, 64, 128, 4096);
    stub::calls = 0;
    expect("decode valid", attn_fwd_decode(&q, &kc, &vc, lens, 0.f, 1, 64, 8, &o, nullptr, dev(6), need, nullptr),
           ATTN_OK);
    expect_true("decode packed", stub::last == stub::LAUNCH_DECODE && stub::dargs.Sk == 4096 &&
                                     stub::dargs.workspace == dev(6) && stub::dargs.cache_lens == lens);
    expect("decode small workspace",
           attn_fwd_decode(&q, &kc, &vc, lens, 0.f, 1, 64, 8, &o, nullptr, dev(6), need - 1, nullptr),
           ATTN_ERR_WORKSPACE);
    expect("decode null workspace",
           attn_fwd_decode(&q, &kc, &vc, lens, 0.f, 1, 64, 8, &o, nullptr, nullptr, need, nullptr), ATTN_ERR_NULL);
    expect("decode misaligned workspace",
           attn_fwd_decode(&q, &kc, &vc, lens, 0.f, 1, 64, 8, &o, nullptr,
                           reinterpret_cast<void*>(uintptr_t(dev(6)) + 4), need, nullptr),
           ATTN_ERR_ALIGN);
    expect("decode misaligned lengths",
           attn_fwd_decode(&q, &kc, &vc, reinterpret_cast<const int32_t*>(uintptr_t(dev(5)) + 1), 0.f, 1, 64, 8, &o,
                           nullptr, dev(6), need, nullptr),
           ATTN_ERR_ALIGN);
    expect("noalloc valid", attn_fwd_decode_noalloc(&q, &kc, &vc, lens, 0.f, 1, 64, 8, &o, nullptr, nullptr), ATTN_OK);
    attn_tensor_t qb = T(0, ATTN_BF16, 64, 16, 64, 128), kb = T(1, ATTN_BF16, 64, 32768, 8, 128),
                  vb = T(2, ATTN_BF16, 64, 32768, 8, 128), ob = T(3, ATTN_BF16, 64, 16, 64, 128);
    expect("noalloc beyond its workspace",
           attn_fwd_decode_noalloc(&qb, &kb, &vb, nullptr, 0.f, 1, 64, 8, &ob, nullptr, nullptr), ATTN_ERR_SCRATCH);
    attn_tensor_t kd = kc;
    kd.D = 64;
    expect("decode D mismatch", attn_fwd_decode(&q, &kd, &vc, lens, 0.f, 1, 64, 8, &o, nullptr, dev(6), need, nullptr),
           ATTN_ERR_SHAPE);
    attn_tensor_t q0 = q, o0 = o;
    q0.B = o0.B = kc.B = vc.B = 0;
    stub::calls = 0;
    expect("decode empty batch", attn_fwd_decode(&q0, &kc, &vc, lens, 0.f, 1, 64, 8, &o0, nullptr, nullptr, 0, nullptr),
           ATTN_OK);
    expect_true("decode empty launches nothing", stub::calls == 0);
    kc.B = vc.B = 8;
    // sizes near every limit: no overflow on the way to the error
    attn_tensor_t qx = T(0, ATTN_F32, 65535, (int64_t(1) << 20) - 1, 65535, 128),
                  ox = T(3, ATTN_F32, 65535, (int64_t(1) << 20) - 1, 65535, 128),
                  kx = T(1, ATTN_F32, 65535, (int64_t(1) << 29) - 1, 1, 128),
                  vx = T(2, ATTN_F32, 65535, (int64_t(1) << 29) - 1, 1, 128);
    expect("decode huge", attn_fwd_decode(&qx, &kx, &vx, nullptr, 0.f, 0, 65535, 1, &ox, nullptr, dev(6), big, nullptr),
           ATTN_ERR_UNSUPPORTED);
    qx.S = ox.S = big;
    kx.S = vx.S = big;
    expect("decode int64 sizes",
           attn_fwd_decode(&qx, &kx, &vx, nullptr, 0.f, 0, 65535, 1, &ox, nullptr, dev(6), big, nullptr),
           ATTN_ERR_UNSUPPORTED);
}

void misc_cases() {
    for (int c = -20; c <= 5; ++c) expect_true("strerror never null", attn_strerror(c) != nullptr);
    expect_true("version", attn_version() != nullptr);
}

}  // namespace

int main() {
    fwd_cases();
    varlen_cases();
    masked_cases();
    rope_cases();
    decode_cases();
    misc_cases();
    std::printf("%d cases, %d failed\n", n_cases, n_bad);
    return n_bad == 0 ? 0 : 1;
}
