// Exercises the argument checks of the C ABI (include/evo_attn.h) with
// adversarial sizes, strides and pointers: sizes and strides drawn from the
// edges of the int64 range and of the 2^31 / 2^32 / 2^62 limits the checks
// enforce, pointers that are null, misaligned or overlapping.  Pointers are
// fake addresses: the checks only compare them, and the launchers are stubs
// (launch_stubs.cpp).  Built with -fsanitize=address,undefined, any overflow
// or out-of-bounds access in the checks stops the run with an error.  A few
// cases with a known answer are asserted as well.  Test infrastructure only.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "evo_attn.h"

namespace evo_stub {
extern long launches;
}

namespace {

uint64_t rng = 0x9E3779B97F4A7C15ull;
uint64_t next() {  // xorshift64*
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return rng * 0x2545F4914F6CDD1Dull;
}

const int64_t kEdges[] = {0,
                          1,
                          2,
                          3,
                          7,
                          8,
                          16,
                          31,
                          32,
                          64,
                          65,
                          383,
                          384,
                          1024,
                          32767,
                          32768,
                          (int64_t(1) << 31) - 1,
                          int64_t(1) << 31,
                          int64_t(1) << 32,
                          (int64_t(1) << 61) + 1,
                          (int64_t(1) << 62) - 1,
                          int64_t(1) << 62,
                          INT64_MAX - 3,
                          INT64_MAX,
                          -1,
                          INT64_MIN};
constexpr int kNumEdges = sizeof(kEdges) / sizeof(kEdges[0]);

int64_t pick_size() {
    const uint64_t r = next();
    if (r % 4 == 0) return kEdges[next() % kNumEdges];
    return 1 + (int64_t)(next() % 70);  // mostly small, valid sizes
}
int64_t pick_stride(int64_t dense) {
    const uint64_t r = next() % 6;
    if (r < 3) return dense;
    if (r == 3) return dense < (int64_t(1) << 62) ? dense + 8 * (int64_t)(next() % 4) : dense;
    return kEdges[next() % kNumEdges];
}
const void* pick_ptr(int i) {
    const uint64_t r = next() % 10;
    if (r == 0) return nullptr;
    const uintptr_t base = (uintptr_t(1) << 40) + uintptr_t(i) * (uintptr_t(1) << 34);
    if (r == 1) return reinterpret_cast<const void*>(base + 2);                   // misaligned
    if (r == 2) return reinterpret_cast<const void*>((uintptr_t(1) << 40) + 64);  // overlaps others
    if (r == 3) return reinterpret_cast<const void*>(~uintptr_t(0) << 4);          // at the top of the space
    return reinterpret_cast<const void*>(base);
}
evo_dtype_t pick_dtype() {
    const uint64_t r = next() % 8;
    return r < 7 ? static_cast<evo_dtype_t>(r % 3) : static_cast<evo_dtype_t>(7);
}

int failures = 0;
void expect(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "unexpected result: %s\n", what);
        ++failures;
    }
}

void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }

void known_cases() {
    const uintptr_t G = uintptr_t(1) << 36;  // tensors 64 GiB apart
    evo_shape_t s{1, 4, 64, 2, 32};
    expect(evo_attn_check(P(G), P(2 * G), P(3 * G), P(4 * G), P(5 * G), P(6 * G), (float*)P(7 * G), &s,
                          EVO_DTYPE_BF16) == EVO_OK, "valid bf16 forward");
    expect(evo_attn_check(P(G), P(2 * G), P(3 * G), nullptr, nullptr, P(G), nullptr, &s, EVO_DTYPE_BF16) ==
               EVO_ERR_ALIASING, "out over q");
    expect(evo_attn_check(P(G + 2), P(2 * G), P(3 * G), nullptr, nullptr, P(6 * G), nullptr, &s, EVO_DTYPE_F16) ==
               EVO_ERR_MISALIGNED, "misaligned q");
    evo_shape_t huge{1, 1, int64_t(1) << 40, 1, 32};
    expect(evo_attn_check(P(G), P(2 * G), P(3 * G), nullptr, nullptr, P(6 * G), nullptr, &huge, EVO_DTYPE_BF16) ==
               EVO_ERR_BAD_SHAPE, "tensor past 2^62 bytes");
    // a size-1 axis may carry any non-negative stride
    evo_layout_t lay;
    evo_attn_dense_layout(&s, &lay);
    lay.q[0] = INT64_MAX;
    expect(evo_attn_check_strided(P(G), P(2 * G), P(3 * G), nullptr, nullptr, P(6 * G), nullptr, &lay, &s,
                                  EVO_DTYPE_BF16) == EVO_ERR_MISALIGNED, "stride of 2^63 - 1 on a size-1 axis");
    evo_shape_t wide{1, 1, INT64_MAX, 1, 32};
    expect(evo_attn_bwd_workspace_size(&wide, EVO_DTYPE_BF16) == 0, "workspace of an impossible shape");
    evo_trimul_shape_t ts{1, 128, 384};
    expect(evo_trimul_check(P(G), P(2 * G), P(3 * G), &ts, EVO_TRIMUL_OUTGOING, EVO_DTYPE_BF16) == EVO_OK,
           "valid trimul");
}

}  // namespace

int main(int argc, char** argv) {
    const long iters = argc > 1 ? std::atol(argv[1]) : 200000;
    if (argc > 2) rng ^= std::strtoull(argv[2], nullptr, 10) * 0xD1B54A32D192ED03ull;
    known_cases();
    long calls = 0, ok = 0;
    for (long it = 0; it < iters; ++it) {
        evo_shape_t s{pick_size(), pick_size(), pick_size(), pick_size(), pick_size()};
        if (next() % 3 == 0) s.D = (int64_t)8 << (next() % 4);
        evo_layout_t lay;
        evo_attn_dense_layout(&s, &lay);
        int64_t* fields[] = {&lay.q[0],   &lay.q[1],   &lay.q[2],   &lay.q[3],   &lay.k[0],   &lay.k[1],
                             &lay.k[2],   &lay.k[3],   &lay.v[0],   &lay.v[1],   &lay.v[2],   &lay.v[3],
                             &lay.out[0], &lay.out[1], &lay.out[2], &lay.out[3], &lay.mask_b, &lay.mask_n,
                             &lay.pair_b, &lay.pair_h, &lay.pair_i, &lay.lse_row};
        const int nmut = (int)(next() % 4);
        for (int m = 0; m < nmut; ++m) {
            int64_t* f = fields[next() % (sizeof(fields) / sizeof(fields[0]))];
            *f = pick_stride(*f);
        }
        const evo_dtype_t dt = pick_dtype();
        const void* p[16];
        for (int i = 0; i < 16; ++i) p[i] = pick_ptr(i);
        const size_t ws_bytes = (size_t)kEdges[next() % kNumEdges];
        evo_status_t r;
        switch (it % 9) {
        case 0: r = evo_attn_check(p[0], p[1], p[2], p[3], p[4], p[5], (const float*)p[6], &s, dt); break;
        case 1:
            r = evo_attn_check_strided(p[0], p[1], p[2], p[3], p[4], p[5], (const float*)p[6], &lay, &s, dt);
            break;
        case 2:
            r = evo_attn_fwd_strided(p[0], p[1], p[2], p[3], p[4], (void*)p[5], (float*)p[6], &lay, &s, dt, nullptr);
            break;
        case 3: r = evo_attn_fwd(p[0], p[1], p[2], p[3], p[4], (void*)p[5], (float*)p[6], &s, dt, nullptr); break;
        case 4:
            r = evo_attn_bwd_check_strided(p[0], p[1], p[2], p[3], p[4], p[5], (const float*)p[6], p[7], p[8], p[9],
                                           p[10], p[11], p[12], (const float*)p[13], p[14], ws_bytes, &lay, &s, dt);
            break;
        case 5:
            r = evo_attn_bwd_strided(p[0], p[1], p[2], p[3], p[4], p[5], (const float*)p[6], p[7], (void*)p[8],
                                     (void*)p[9], (void*)p[10], (void*)p[11], (void*)p[12], (float*)p[13],
                                     (void*)p[14], ws_bytes, &lay, &s, dt, nullptr);
            break;
        case 6:
            r = evo_attn_bwd(p[0], p[1], p[2], p[3], p[4], p[5], (const float*)p[6], p[7], (void*)p[8], (void*)p[9],
                             (void*)p[10], (void*)p[11], (void*)p[12], (float*)p[13], (void*)p[14], ws_bytes, &s, dt,
                             nullptr);
            break;
        case 7: {
            const size_t w = evo_attn_bwd_workspace_size(&s, dt);
            r = (w % 4 == 0) ? EVO_OK : EVO_ERR_BAD_SHAPE;
            expect(w % 4 == 0, "workspace size a multiple of 4");
            break;
        }
        default: {
            evo_trimul_shape_t ts{s.B, s.N, s.L};
            r = evo_trimul(p[0], p[1], (void*)p[2], &ts, static_cast<evo_trimul_direction_t>(next() % 3), dt,
                           nullptr);
            break;
        }
        }
        ++calls;
        ok += r == EVO_OK;
        expect((int)r >= 0 && (int)r <= 9, "status in range");
        (void)evo_status_string(r);
    }
    std::printf("abi_fuzz: %ld calls, %ld accepted, %ld launches reached, %d failures\n", calls, ok,
                evo_stub::launches, failures);
    return failures ? 1 : 0;
}
