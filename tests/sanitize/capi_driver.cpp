// capi_driver.cpp -- calls every entry point of the C ABI (include/fp4q.h)
// with valid and invalid arguments against stubbed launchers: each rejected
// call must return its status without launching, each valid one must launch.
// Built with -fsanitize=address,undefined; exits 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "fp4q.h"

namespace fp4q {
extern int stub_launches;
}

static int failures = 0;
#define CHECK(cond)                                                               \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

// fake device addresses, aligned as the ABI requires; the stubs never use them
static void* dev(uintptr_t k) { return reinterpret_cast<void*>(k << 16); }

static fp4q_spec spec(int fmt = FP4Q_NVFP4, int rule = FP4Q_SCALE_SWEEP, int obj = FP4Q_OBJ_MSE,
                      int rot = 0)
{
    fp4q_spec s{};
    s.format = fmt;
    s.block = fmt == FP4Q_MXFP4 ? 32 : 16;
    s.scale_rule = rule;
    s.objective = obj;
    s.sweep_lo = obj == FP4Q_OBJ_WMSE ? -8 : -3;
    s.sweep_hi = 7;
    s.rotate = rot;
    s.global_scale_given = 0;
    return s;
}

// expect status `want`, and a launch exactly when it is FP4Q_OK
#define EXPECT(call, want)                                                        \
    do {                                                                          \
        const int before = fp4q::stub_launches;                                   \
        const fp4q_status got = (call);                                           \
        CHECK(got == (want));                                                     \
        CHECK((fp4q::stub_launches > before) == ((want) == FP4Q_OK));             \
    } while (0)

int main()
{
    auto* x = dev(1);
    auto* codes = static_cast<uint8_t*>(dev(2));
    auto* scales = static_cast<uint8_t*>(dev(3));
    auto* gs = static_cast<float*>(dev(4));
    auto* ws = dev(5);
    auto* imp = static_cast<const float*>(dev(6));
    const size_t wsb = fp4q_workspace_bytes(nullptr, 4, 64);
    CHECK(wsb == 0);
    fp4q_spec s = spec();
    const size_t need = fp4q_workspace_bytes(&s, 4, 64);
    CHECK(need >= 256 && need <= FP4Q_NOALLOC_SCRATCH_BYTES);

    // quantize: valid, then one defect at a time
    EXPECT(fp4q_quantize(&s, x, FP4Q_BF16, 4, 64, nullptr, codes, scales, gs, ws, need, nullptr), FP4Q_OK);
    EXPECT(fp4q_quantize(nullptr, x, FP4Q_BF16, 4, 64, nullptr, codes, scales, gs, ws, need, nullptr), FP4Q_E_NULL);
    EXPECT(fp4q_quantize(&s, x, 7, 4, 64, nullptr, codes, scales, gs, ws, need, nullptr), FP4Q_E_ARG);
    EXPECT(fp4q_quantize(&s, x, FP4Q_BF16, -1, 64, nullptr, codes, scales, gs, ws, need, nullptr), FP4Q_E_SHAPE);
    EXPECT(fp4q_quantize(&s, x, FP4Q_BF16, 4, 60, nullptr, codes, scales, gs, ws, need, nullptr), FP4Q_E_SHAPE);
    EXPECT(fp4q_quantize(&s, x, FP4Q_BF16, INT64_MAX, 64, nullptr, codes, scales, gs, ws, need, nullptr), FP4Q_E_SHAPE);
    EXPECT(fp4q_quantize(&s, x, FP4Q_BF16, 4, 64, nullptr, codes, scales, gs, ws, need - 1, nullptr), FP4Q_E_ARG);
    EXPECT(fp4q_quantize(&s, x, FP4Q_BF16, 4, 64, nullptr, codes, scales, gs, nullptr, need, nullptr), FP4Q_E_NULL);
    EXPECT(fp4q_quantize(&s, static_cast<char*>(x) + 8, FP4Q_BF16, 4, 64, nullptr, codes, scales, gs, ws, need, nullptr), FP4Q_E_ALIGN);
    EXPECT(fp4q_quantize(&s, nullptr, FP4Q_BF16, 0, 64, nullptr, nullptr, nullptr, gs, ws, need, nullptr), FP4Q_OK);
    fp4q_spec w = spec(FP4Q_NVFP4, FP4Q_SCALE_SWEEP, FP4Q_OBJ_WMSE);
    EXPECT(fp4q_quantize(&w, x, FP4Q_F32, 4, 64, nullptr, codes, scales, gs, ws, need, nullptr), FP4Q_E_NULL);
    EXPECT(fp4q_quantize(&w, x, FP4Q_F32, 4, 64, imp, codes, scales, gs, ws, need, nullptr), FP4Q_OK);
    EXPECT(fp4q_quantize(&w, x, FP4Q_F32, 4, 64, imp + 1, codes, scales, gs, ws, need, nullptr), FP4Q_E_ALIGN);
    fp4q_spec bad = s;
    bad.sweep_lo = 9;
    EXPECT(fp4q_quantize(&bad, x, FP4Q_BF16, 4, 64, nullptr, codes, scales, gs, ws, need, nullptr), FP4Q_E_ARG);
    bad = spec(FP4Q_MXFP4, FP4Q_SCALE_FOUR_OVER_SIX);
    EXPECT(fp4q_quantize(&bad, x, FP4Q_BF16, 4, 64, nullptr, codes, scales, nullptr, ws, need, nullptr), FP4Q_E_UNSUPPORTED);
    bad = s;
    bad.block = 32;
    EXPECT(fp4q_quantize(&bad, x, FP4Q_BF16, 4, 64, nullptr, codes, scales, gs, ws, need, nullptr), FP4Q_E_UNSUPPORTED);
    bad = s;
    bad.rotate = 8;
    EXPECT(fp4q_quantize(&bad, x, FP4Q_BF16, 4, 64, nullptr, codes, scales, gs, ws, need, nullptr), FP4Q_E_ARG);

    // IF3 / IF6: their own code alignment (2 and 4 bytes), no Four Over Six
    for (int fmt : {FP4Q_IF3, FP4Q_IF6}) {
        fp4q_spec a = spec(fmt);
        EXPECT(fp4q_quantize(&a, x, FP4Q_BF16, 4, 64, nullptr, codes, scales, gs, ws, need, nullptr), FP4Q_OK);
        EXPECT(fp4q_quantize(&a, x, FP4Q_BF16, 4, 64, nullptr, codes + (fmt == FP4Q_IF3 ? 1 : 2), scales, gs,
                             ws, need, nullptr), FP4Q_E_ALIGN);
        EXPECT(fp4q_dequantize(&a, codes + (fmt == FP4Q_IF3 ? 2 : 4), scales, gs, 4, 64, 0, dev(8), FP4Q_F32,
                               nullptr), FP4Q_OK);
        fp4q_spec f = spec(fmt, FP4Q_SCALE_FOUR_OVER_SIX);
        EXPECT(fp4q_quantize(&f, x, FP4Q_BF16, 4, 64, nullptr, codes, scales, gs, ws, need, nullptr),
               FP4Q_E_UNSUPPORTED);
        fp4q_spec wq = spec(fmt, FP4Q_SCALE_ABSMAX, FP4Q_OBJ_WMSE);
        EXPECT(fp4q_quantize(&wq, x, FP4Q_BF16, 4, 64, nullptr, codes, scales, gs, ws, need, nullptr), FP4Q_E_NULL);
    }

    // the entry point without a workspace
    EXPECT(fp4q_quantize_noalloc(&s, x, FP4Q_BF16, 4, 64, nullptr, codes, scales, gs, nullptr), FP4Q_OK);
    EXPECT(fp4q_quantize_noalloc(&s, x, FP4Q_BF16, 4, 64, nullptr, codes, scales, nullptr, nullptr), FP4Q_E_NULL);
    EXPECT(fp4q_quantize_noalloc(&w, x, FP4Q_BF16, 4, 64, nullptr, codes, scales, gs, nullptr), FP4Q_E_NULL);

    // FOCUS deploy encode
    auto* coef = static_cast<const float*>(dev(7));
    EXPECT(fp4q_quantize_relaxed(&s, x, FP4Q_BF16, 4, 64, coef, 8, 0, codes, scales, gs, ws, need, nullptr), FP4Q_OK);
    EXPECT(fp4q_quantize_relaxed(&s, x, FP4Q_BF16, 4, 64, coef, 4, 0, codes, scales, gs, ws, need, nullptr), FP4Q_E_ARG);
    EXPECT(fp4q_quantize_relaxed(&s, x, FP4Q_BF16, 4, 64, nullptr, 8, 0, codes, scales, gs, ws, need, nullptr), FP4Q_E_NULL);
    fp4q_spec i4 = spec(FP4Q_IF4);
    EXPECT(fp4q_quantize_relaxed(&i4, x, FP4Q_BF16, 4, 64, coef, 8, 0, codes, scales, gs, ws, need, nullptr), FP4Q_E_UNSUPPORTED);

    // dequantize
    void* y = dev(8);
    EXPECT(fp4q_dequantize(&s, codes, scales, gs, 4, 64, 0, y, FP4Q_BF16, nullptr), FP4Q_OK);
    EXPECT(fp4q_dequantize(&s, codes, scales, gs, 4, 64, 16, y, FP4Q_F32, nullptr), FP4Q_OK);
    EXPECT(fp4q_dequantize(&s, codes, scales, gs, 4, 64, 32, y, FP4Q_F32, nullptr), FP4Q_E_ARG);
    EXPECT(fp4q_dequantize(&s, codes, scales, nullptr, 4, 64, 0, y, FP4Q_F32, nullptr), FP4Q_E_NULL);
    EXPECT(fp4q_dequantize(&s, codes + 1, scales, gs, 4, 64, 0, y, FP4Q_F32, nullptr), FP4Q_E_ALIGN);

    // error report (the stubbed copy writes zeros to out_host)
    double out[2] = {1.0, 1.0};
    EXPECT(fp4q_error(&s, x, FP4Q_BF16, 4, 64, imp, codes, scales, gs, ws, need, out, nullptr), FP4Q_OK);
    CHECK(out[0] == 0.0 && out[1] == 0.0);
    EXPECT(fp4q_error(&s, x, FP4Q_BF16, 4, 64, imp, codes, scales, gs, ws, need, nullptr, nullptr), FP4Q_E_NULL);
    EXPECT(fp4q_error(&s, x, FP4Q_BF16, 4, 64, imp, codes, scales, gs, ws, 16, out, nullptr), FP4Q_E_ARG);

    // every status has a string
    for (int st = 0; st >= -7; --st)
        CHECK(fp4q_status_string(static_cast<fp4q_status>(st)) != nullptr);
    CHECK(fp4q_abi_version() == FP4Q_ABI_VERSION);

    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("C ABI driver: every argument check ran clean\n");
    return 0;
}
