// Host-only exercise of the library's C++ (argument checks, the workspace
// layout planning, the randomized SVD) built with AddressSanitizer and
// UndefinedBehaviorSanitizer, without a GPU: the device launchers are stubs
// that never run, and every device-touching path returns an error status
// before reaching them.  Exit status 0 when every expectation holds.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "dq.h"
#include "dq_internal.h"

namespace dq {
static hipError_t stub() { return hipErrorNoDevice; }
hipError_t launch_residual(const void*, int, const uint16_t*, const uint16_t*, int64_t, int64_t, int, float*, hipStream_t) { return stub(); }
hipError_t launch_encode_fp4_rows(const float*, int64_t, int64_t, int64_t, int64_t, uint8_t*, uint8_t*, hipStream_t) { return stub(); }
hipError_t launch_quantize(const dq_weights*, const void*, int, dq_qact*, hipStream_t) { return stub(); }
hipError_t launch_slot_tokens(const Geom&, int64_t, int*, int64_t, hipStream_t) { return stub(); }
hipError_t launch_decode_fp4_bf16(const uint8_t*, const uint8_t*, int64_t, int64_t, uint16_t*, hipStream_t) { return stub(); }
hipError_t launch_forward(const dq_weights*, dq_qact*, float*, int, hipStream_t) { return stub(); }
hipError_t launch_forward_fused(const dq_weights*, dq_qact*, float*, hipStream_t) { return stub(); }
hipError_t launch_forward6(const dq_weights*, dq_act6*, float*, hipStream_t) { return stub(); }
hipError_t launch_encode_fp6(const void*, int, int64_t, int64_t, int64_t, int64_t, uint8_t*, uint8_t*, int, hipStream_t) { return stub(); }
hipError_t launch_text_lowrank(const void*, int, int64_t, int64_t, int, int, const uint16_t*, int, float*, uint16_t*, hipStream_t) { return stub(); }
int text_lowrank_splits(int Ci) { return (Ci + 255) / 256; }
}  // namespace dq

static int failures = 0;
#define EXPECT(cond)                                                              \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::printf("FAILED line %d: %s (%s)\n", __LINE__, #cond, dq_last_error()); \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

int main() {
    std::mt19937 rng(7);
    std::normal_distribution<float> nd(0.0f, 1.0f);
    // ---- the host SVD on several shapes, fp32 and bf16 weights
    const int shapes[][3] = {{64, 48, 8}, {96, 200, 32}, {256, 128, 128}, {32, 1, 1}, {160, 33, 16}};
    for (auto& sh : shapes) {
        const int Ci = sh[0], Co = sh[1], r = sh[2];
        std::vector<float> w((size_t)Ci * Co);
        for (auto& v : w) v = nd(rng) / std::sqrt((float)Ci);
        std::vector<uint16_t> wb(w.size());
        for (size_t i = 0; i < w.size(); ++i) {
            uint32_t u;
            std::memcpy(&u, &w[i], 4);
            wb[i] = (uint16_t)(u >> 16);
        }
        std::vector<uint16_t> l1((size_t)Ci * r), l2((size_t)r * Co);
        EXPECT(dq_lowrank_factors(w.data(), DQ_F32, Ci, Co, r, 3, l1.data(), l2.data()) == DQ_OK);
        for (uint16_t b : l1) EXPECT(std::isfinite(bf16_to_f32(b)));
        EXPECT(dq_lowrank_factors(wb.data(), DQ_BF16, Ci, Co, r, 4, l1.data(), l2.data()) == DQ_OK);
        for (uint16_t b : l2) EXPECT(std::isfinite(bf16_to_f32(b)));
    }
    // ---- argument rejections (no device is reached)
    std::vector<float> w(96 * 64, 0.5f);
    std::vector<uint16_t> l1(96 * 8), l2(8 * 64);
    dq_weights* hw = nullptr;
    dq_act6* ha = nullptr;
    EXPECT(dq_lowrank_factors(nullptr, DQ_F32, 96, 64, 8, 0, l1.data(), l2.data()) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_lowrank_factors(w.data(), DQ_F32, 96, 64, 65, 0, l1.data(), l2.data()) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_lowrank_factors(w.data(), DQ_F32, 0, 64, 0, 0, nullptr, nullptr) == DQ_ERR_SHAPE);
    EXPECT(dq_lowrank_factors(w.data(), (dq_dtype)9, 96, 64, 8, 0, l1.data(), l2.data()) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_lowrank_factors(w.data(), DQ_F32, 96, 64, 0, 0, nullptr, nullptr) == DQ_OK);
    EXPECT(dq_prepare_weights_lowrank(w.data(), DQ_F32, 48, 64, 8, l1.data(), l2.data(), 0, &hw) == DQ_ERR_SHAPE);
    EXPECT(dq_prepare_weights_lowrank(w.data(), DQ_F32, 96, 64, 129, l1.data(), l2.data(), 0, &hw) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_prepare_weights_lowrank(w.data(), DQ_F32, 96, 64, 8, nullptr, l2.data(), 0, &hw) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_prepare_weights_lowrank(w.data(), DQ_F32, 96, 64, 8, l1.data(), l2.data(), 0, nullptr) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_prepare_weights_w6(w.data(), DQ_F32, 96, 64, 8, l1.data(), l2.data(), 5, 0, &hw) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_prepare_weights(w.data(), DQ_F32, 96, 64, 65, 0, 0, &hw) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_prepare_weights(w.data(), DQ_F32, int64_t(1) << 62, 64, 8, 0, 0, &hw) == DQ_ERR_SHAPE);
    EXPECT(dq_lowrank_factors(w.data(), DQ_F32, int64_t(1) << 62, int64_t(1) << 62, 8, 0, l1.data(), l2.data()) == DQ_ERR_SHAPE);
    EXPECT(dq_act6_create(nullptr, -1, &ha) == DQ_ERR_INVALID_ARG);
    {   // without a GPU the device check fails cleanly
        dq_status st = dq_prepare_weights_lowrank(w.data(), DQ_F32, 96, 64, 8, l1.data(), l2.data(), 0, &hw);
        EXPECT(st == DQ_ERR_DEVICE || st == DQ_ERR_UNSUPPORTED || st == DQ_ERR_INVALID_ARG);
        EXPECT(hw == nullptr);
    }
    dq_qact* hq = nullptr;
    dq_geom g0{2, 4, 4, 1, 2, 2};
    EXPECT(dq_qact_create(nullptr, g0, &hq) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_qact_create_ex(nullptr, g0, 32, 8, &hq) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_act6_create(nullptr, 16, &ha) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_quantize_act(nullptr, w.data(), DQ_F32, nullptr, nullptr) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_linear_forward(nullptr, nullptr, nullptr, nullptr) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_core_term(nullptr, nullptr, nullptr) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_delta_term(nullptr, nullptr, nullptr, nullptr) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_linear(nullptr, nullptr, DQ_F32, nullptr, nullptr, nullptr) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_quantize_act6(nullptr, nullptr, DQ_F32, nullptr, nullptr) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_linear6_forward(nullptr, nullptr, nullptr, nullptr) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_linear6(nullptr, nullptr, DQ_F32, nullptr, nullptr, nullptr) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_qact_export(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_act6_export(nullptr, nullptr, nullptr, nullptr, nullptr) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_weights_info(nullptr, nullptr, nullptr, nullptr, nullptr) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_weights_export(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == DQ_ERR_INVALID_ARG);
    EXPECT(dq_qact_info(nullptr, nullptr, nullptr, nullptr) == DQ_ERR_INVALID_ARG);
    for (int s = 0; s < 7; ++s) EXPECT(dq_status_str((dq_status)s)[0] != 0);
    dq_weights_destroy(nullptr);
    dq_qact_destroy(nullptr);
    dq_act6_destroy(nullptr);
    // ---- workspace layout planning over many geometries, with a weight that
    // exists only on the host (sizes only)
    dq_weights fw;
    fw.Ci = 160;
    fw.Co = 200;
    fw.Kp = 256;
    fw.Cop = 256;
    fw.rank = 16;
    fw.rp = 32;
    long long planned = 0;
    for (int T = 1; T <= 9; ++T)
        for (int H = 1; H <= 7; H += 2)
            for (int W = 1; W <= 11; W += 3)
                for (int t = 1; t <= T; ++t)
                    for (int h = 1; h <= H; ++h)
                        for (int ww = 1; ww <= W; ++ww) {
                            dq_qact q{};
                            int64_t mp = 0;
                            dq_geom g{T, H, W, t, h, ww};
                            if (dq::plan_qact(&fw, g, 32, 8, &q, &mp) != DQ_OK) { ++failures; continue; }
                            // the segments tile the grid: tokens and cubes add up, rows are 256-aligned
                            int64_t tok = 0, cubes = 0;
                            for (int i = 0; i < q.nseg; ++i) {
                                EXPECT(q.seg[i].row0 % 256 == 0 && q.seg[i].krow0 % 256 == 0);
                                EXPECT(q.seg[i].tok0 == tok && q.seg[i].k0 == cubes);
                                tok += q.seg[i].g.N;
                                cubes += q.seg[i].g.K;
                            }
                            EXPECT(tok == (int64_t)T * H * W && cubes == q.g.K);
                            EXPECT(q.Nslot_pad % 256 == 0 && q.K_pad % 256 == 0);
                            ++planned;
                        }
    {   // invalid and huge geometries are refused
        dq_qact q{};
        int64_t mp = 0;
        EXPECT(dq::plan_qact(&fw, dq_geom{2, 2, 2, 3, 1, 1}, 32, 8, &q, &mp) == DQ_ERR_SHAPE);
        EXPECT(dq::plan_qact(&fw, dq_geom{0, 2, 2, 1, 1, 1}, 32, 8, &q, &mp) == DQ_ERR_SHAPE);
        EXPECT(dq::plan_qact(&fw, dq_geom{2, 2, 2, 1, 1, 1}, 48, 8, &q, &mp) == DQ_ERR_INVALID_ARG);
        EXPECT(dq::plan_qact(&fw, dq_geom{2, 2, 2, 1, 1, 1}, 32, 6, &q, &mp) == DQ_ERR_INVALID_ARG);
        EXPECT(dq::plan_qact(&fw, dq_geom{2, 2, 2, 1, 1, 1}, 64, 8, &q, &mp) == DQ_ERR_SHAPE);   // 64 does not divide 160
        EXPECT(dq::plan_qact(&fw, dq_geom{1 << 20, 1 << 20, 1 << 20, 1, 1, 1}, 32, 8, &q, &mp) == DQ_ERR_SHAPE);
        EXPECT(dq::plan_qact(&fw, dq_geom{2147483647, 2147483647, 2147483647, 2, 2, 2}, 32, 8, &q, &mp) == DQ_ERR_SHAPE);
        fw.wfmt = 2;
        EXPECT(dq::plan_qact(&fw, dq_geom{2, 2, 2, 1, 1, 1}, 32, 8, &q, &mp) == DQ_ERR_INVALID_ARG);
    }
    // ---- the core GEMM's last-round K split: structure over many shapes, and
    // the decisions on the 720p and 14B layers' core GEMMs (FP8 x FP4, 256 CUs)
    for (int mt = 1; mt <= 60; mt += 7)
        for (int nt = 1; nt <= 90; nt += 11)
            for (int nks : {1, 3, 8, 40, 108, 160})
                for (int ns : {3, 4}) {
                    const dq::KSplit k = dq::plan_ksplit(mt, nt, nks, ns, 256, 1.6);
                    if (k.rm == 0) continue;
                    EXPECT(k.main_tiles + k.rm == mt * nt && k.main_tiles % 256 == 0 && k.rm < 256);
                    EXPECT(k.p >= 2 && k.rm * k.p <= 256 && nks / k.p >= ns);
                }
    {
        const dq::KSplit up = dq::plan_ksplit(54, 76, 40, 3, 256, 1.6);        // FFN up, 1x2x2: one launch
        EXPECT(up.rm == 0);
        const dq::KSplit d222 = dq::plan_ksplit(20, 40, 108, 3, 256, 1.6);     // FFN down, 2x2x2
        EXPECT(d222.main_tiles == 768 && d222.rm == 32 && d222.p == 8);
        const dq::KSplit glob = dq::plan_ksplit(20, 1, 108, 3, 256, 1.6);      // FFN down, global cube
        EXPECT(glob.main_tiles == 0 && glob.rm == 20 && glob.p == 11);
        const dq::KSplit attn = dq::plan_ksplit(20, 16, 40, 3, 256, 1.6);      // 14B attention, 2x2x2
        EXPECT(attn.main_tiles == 256 && attn.rm == 64 && attn.p == 4);
        const dq::KSplit u428 = dq::plan_ksplit(54, 6, 40, 3, 256, 1.6);       // FFN up, 4x2x8
        EXPECT(u428.main_tiles == 256 && u428.rm == 68 && u428.p == 3);
        EXPECT(dq::plan_ksplit(6, 32, 12, 3, 256, 1.6).rm == 0);             // Wan 1.3B: one round of 192 tiles, short K
    }
    // ---- the activation pass's channel split: the part count divides the
    // chunks, leaves at least 4 per part and fits the CUs; the decisions on
    // the 21-frame layers' last-frame segments and their main segments
    for (long long nb = 1; nb <= 300; nb += 13)
        for (int nch = 1; nch <= 120; nch += 7) {
            const int p = dq::quant_kparts(nb, nch, 256);
            EXPECT(p >= 1 && p <= dq::QMAXPARTS && nch % p == 0);
            EXPECT(p == 1 || (nch / p >= 4 && nb * p <= 256 && nb * 2 <= 256));
        }
    EXPECT(dq::quant_kparts(57, 40, 256) == 4);      // 4x2x8 / 4x1x4, last frame (5120 bf16 channels)
    EXPECT(dq::quant_kparts(58, 108, 256) == 4);     // FFN down 2x2x2, last frame (13824 channels)
    EXPECT(dq::quant_kparts(1125, 40, 256) == 1);    // 4x2x8, the other 20 frames
    EXPECT(dq::quant_kparts(2, 17, 256) == 1);       // 17 chunks: no divisor
    {   // a clipped last frame group: its small segment gets U partials
        dq_weights fu;
        fu.Ci = 5120;
        fu.Co = 512;
        fu.Kp = 5120;
        fu.Cop = 512;
        fu.rank = 32;
        fu.rp = 32;
        dq_qact q{};
        int64_t mp = 0;
        EXPECT(dq::plan_qact(&fu, dq_geom{21, 45, 80, 4, 2, 8}, 32, 8, &q, &mp) == DQ_OK);
        EXPECT(q.nseg == 2 && q.upart_rows == q.seg[1].g.Nslot && q.seg[1].g.Nslot == 23 * 10 * 16);
    }
    {   // the forward's form: one kernel for 4-token cubes with FP8 cores on
        // layers of at most 16 rounds of 256 x 256 tiles per CU of the
        // workspace's device (256 here: without a device the count falls back
        // to it), two kernels otherwise
        auto layer = [](int64_t Ci, int64_t Co) {
            dq_weights f;
            f.Ci = Ci;
            f.Co = Co;
            f.Kp = (Ci + 255) / 256 * 256;
            f.Cop = (Co + 255) / 256 * 256;
            f.rank = 32;
            f.rp = 32;
            return f;
        };
        alignas(16) static float yy[4];
        auto form = [&](const dq_weights& f, dq_geom g, int bits, const float* y, int cus, bool* applies) {
            dq_qact q{};
            int64_t mp = 0;
            if (dq::plan_qact(&f, g, 32, bits, &q, &mp) != DQ_OK) { ++failures; return false; }
            EXPECT(q.cus == 256);
            if (cus) q.cus = cus;
            *applies = dq::fused_applies(&f, &q, y);
            return dq::fused_preferred(&f, &q, y);
        };
        const dq_weights wan = layer(1536, 1536), attn = layer(5120, 5120), up = layer(5120, 13824), down = layer(13824, 5120);
        bool ap = false;
        EXPECT(form(wan, dq_geom{21, 30, 52, 1, 2, 2}, 8, yy, 0, &ap) && ap);            //   768 tiles
        EXPECT(form(attn, dq_geom{20, 30, 52, 1, 2, 2}, 8, yy, 0, &ap) && ap);           //  2440 tiles
        EXPECT(!form(up, dq_geom{21, 45, 80, 1, 2, 2}, 8, yy, 0, &ap) && ap);            // 16308 tiles
        EXPECT(!form(down, dq_geom{21, 45, 80, 1, 2, 2}, 8, yy, 0, &ap) && ap);          //  6040 tiles
        EXPECT(!form(attn, dq_geom{20, 30, 52, 1, 2, 2}, 8, yy, 64, &ap) && ap);         // a 64-CU device: 1024 at most
        EXPECT(form(wan, dq_geom{21, 30, 52, 1, 2, 2}, 8, yy, 64, &ap) && ap);
        EXPECT(!form(attn, dq_geom{20, 30, 52, 2, 2, 2}, 8, yy, 0, &ap) && !ap);         // 8-token cubes
        EXPECT(!form(attn, dq_geom{20, 30, 52, 1, 2, 2}, 4, yy, 0, &ap) && !ap);         // FP4 cores
        EXPECT(!form(attn, dq_geom{20, 30, 52, 1, 2, 2}, 8, yy + 1, 0, &ap) && !ap);     // y not 16-byte aligned
        EXPECT(!form(layer(256, 5120), dq_geom{20, 30, 52, 1, 2, 2}, 8, yy, 0, &ap) && !ap);   // 2 K steps
        EXPECT(form(layer(384, 5120), dq_geom{20, 30, 52, 1, 2, 2}, 8, yy, 0, &ap) && ap);     // 4 (Kp 512)
    }
    std::printf("host sanitize driver: %lld geometries planned, %d failures\n", planned, failures);
    return failures ? 1 : 0;
}
