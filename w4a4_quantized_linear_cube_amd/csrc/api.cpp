// C ABI of the delta-W4A4 layer: argument checks, handle ownership, device
// buffers, launches.  Every arithmetic step of the layer runs in the HIP
// kernels of quant.hip and gemm.hip; the host SVD of svd.cpp only produces
// the low-rank factors.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <limits>
#include <memory>
#include <new>
#include <string>
#include <vector>

#include "dq.h"
#include "dq_internal.h"

namespace dq {

void lowrank_svd(const float* wt, int64_t Ci, int64_t Co, int rank, uint64_t seed, uint16_t* l1, uint16_t* l2);

namespace {
thread_local std::string g_last_error;
}  // namespace

dq_status fail(dq_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

dq_status hip_fail(hipError_t e, const char* what) {
    if (e == hipErrorOutOfMemory) return fail(DQ_ERR_OUT_OF_MEMORY, std::string(what) + ": out of device memory");
    return fail(DQ_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

namespace {

dq_status check_device(int device) {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return fail(DQ_ERR_DEVICE, "no HIP device available");
    if (device < 0 || device >= n) return fail(DQ_ERR_INVALID_ARG, "device index out of range");
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return fail(DQ_ERR_DEVICE, "hipGetDeviceProperties failed");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(DQ_ERR_UNSUPPORTED, std::string("device is ") + prop.gcnArchName + ", gfx950 required");
    return DQ_OK;
}

// Zero-filled device allocation.
template <class T>
hipError_t dalloc(T** p, size_t count, size_t* total) {
    *p = nullptr;
    if (count == 0) return hipSuccess;
    size_t bytes = count * sizeof(T);
    hipError_t e = hipMalloc((void**)p, bytes);
    if (e != hipSuccess) {
        *p = nullptr;
        return e;
    }
    *total += bytes;
    return hipMemset(*p, 0, bytes);
}

bool mul_ok(int64_t a, int64_t b, int64_t limit) { return a >= 0 && b >= 0 && (a == 0 || b <= limit / a); }

void free_weights(dq_weights* w) {
    if (!w) return;
    DeviceGuard dg(w->device);
    (void)hipFree(w->rq);
    (void)hipFree(w->rs);
    (void)hipFree(w->r);
    (void)hipFree(w->l1t);
    (void)hipFree(w->l2t);
    delete w;
}

void free_qact(dq_qact* q) {
    if (!q) return;
    DeviceGuard dg(q->device);
    (void)hipFree(q->dq);
    (void)hipFree(q->ds);
    (void)hipFree(q->cq);
    (void)hipFree(q->cs);
    (void)hipFree(q->stok);
    (void)hipFree(q->zero);
    (void)hipFree(q->sink);
    (void)hipFree(q->u);
    (void)hipFree(q->bias);
    (void)hipFree(q->coref);
    (void)hipFree(q->part);
    (void)hipFree(q->kpart);
    (void)hipFree(q->upart);
    (void)hipFree(q->cbf);
    (void)hipFree(q->rbf);
    delete q;
}

long long host_slot_token(const Geom& g, long long slot) {
    long long k = slot / g.S;
    int s = (int)(slot - k * g.S);
    int dw = s % g.w, dh = (s / g.w) % g.h, dt = s / (g.w * g.h);
    long long kw = k % g.Wc, kh = (k / g.Wc) % g.Hc, kt = k / ((long long)g.Wc * g.Hc);
    long long ti = kt * g.t + dt, hi = kh * g.h + dh, wi = kw * g.w + dw;
    if (k >= g.K || ti >= g.T || hi >= g.H || wi >= g.W) return -1;
    return (ti * g.H + hi) * g.W + wi;
}

}  // namespace

void set_error(const std::string& msg) { g_last_error = msg; }

// Host copies of the step-major operand layout back to plain rows (exports).
hipError_t fetch_all(const void* src, size_t bytes, std::vector<uint8_t>& dst) {
    dst.resize(bytes);
    return hipMemcpy(dst.data(), src, bytes, hipMemcpyDeviceToHost);
}
void unstep_fp4(const std::vector<uint8_t>& buf, long long row, int64_t Ci, int64_t Kp, uint8_t* out) {
    for (long long G = 0; G < Ci / 32; ++G) std::memcpy(out + 16 * G, &buf[off_fp4(row, G, Kp / 128)], 16);
}
void unstep_fp8(const std::vector<uint8_t>& buf, long long row, int64_t Ci, int64_t Kp, uint8_t* out) {
    for (long long c = 0; c < Ci / 16; ++c) std::memcpy(out + 16 * c, &buf[off_fp8(row, c >> 3, (int)(c & 7), Kp / 128)], 16);
}
void unstep_fp6(const std::vector<uint8_t>& buf, long long row, int64_t Ci, int64_t Kp, uint8_t* out) {
    for (long long G = 0; G < Ci / 32; ++G)
        for (int i = 0; i < 3; ++i) std::memcpy(out + 24 * G + 8 * i, &buf[off_fp6(row, G, i, Kp / 128)], 8);
}
void unstep_scales(const std::vector<uint8_t>& buf, long long row, int64_t Ci, int64_t Kp, uint8_t* out) {
    for (long long G = 0; G < Ci / 32; ++G) out[G] = buf[off_scale(row, G, Kp / 128)];
}

}  // namespace dq

using namespace dq;

namespace dq {
// The shapes the one-kernel forward takes: cubes of exactly 4 slots with FP8
// cores in one frame segment (a 256-slot tile's cubes are then the 64 rows
// 64 tn .. of the core codes, inside one 256-row core tile), rank 32, Co a
// multiple of 256, y rows 16-byte aligned with 32-bit element offsets, and K
// loops of 4 or more 128-channel steps.
bool fused_applies(const dq_weights* w, const dq_qact* q, const float* y) {
    return q->core_bits == 8 && q->g.S == 4 && q->nseg == 1 && w->Kp / 128 >= 4 && w->rp == 32 && w->Co % 256 == 0 &&
           (uintptr_t)y % 16 == 0 && q->g.N * w->Co < (1ll << 31) && q->Nslot_pad / 4 <= q->K_pad;
}

// The form the whole forward takes: the one-kernel form where it applies and
// the layer has at most 16 rounds of 256 x 256 tiles per CU, else the two
// kernels.  Measured with 4-token cubes on MI355X (one-kernel time over
// two-kernel time): Wan 1.3B projection, 3 rounds, 0.72-0.77; 14B attention
// projection, 9.5 rounds, 0.95; 720p FFN down, 23.6 rounds, 1.02; 720p FFN up,
// 63.7 rounds, 1.03.  The two-kernel form's fixed costs (the core GEMM's
// launch and partly filled last round, the per-cube term's round trip) weigh
// most on small layers; on large ones the fused K loop's extra operand bytes
// cost more than they save.
bool fused_preferred(const dq_weights* w, const dq_qact* q, const float* y) {
    if (!fused_applies(w, q, y)) return false;
    const long long tiles = (w->Cop / 256) * (q->Nslot_pad / 256);
    return tiles <= 16ll * q->cus;
}
}  // namespace dq

extern "C" {

const char* dq_last_error(void) { return g_last_error.c_str(); }

const char* dq_status_str(dq_status s) {
    switch (s) {
        case DQ_OK: return "ok";
        case DQ_ERR_INVALID_ARG: return "invalid argument";
        case DQ_ERR_SHAPE: return "invalid shape";
        case DQ_ERR_UNSUPPORTED: return "unsupported device";
        case DQ_ERR_OUT_OF_MEMORY: return "out of memory";
        case DQ_ERR_DEVICE: return "device error";
    }
    return "unknown status";
}

dq_status dq_lowrank_factors(const void* w_host, dq_dtype dt, int64_t Ci, int64_t Co, int32_t rank, uint64_t seed,
                             uint16_t* l1_host, uint16_t* l2_host) {
    g_last_error.clear();
    if (Ci < 1 || Co < 1) return fail(DQ_ERR_SHAPE, "Ci and Co must be >= 1");
    if (!mul_ok(Ci, Co, std::numeric_limits<int64_t>::max() / 8)) return fail(DQ_ERR_SHAPE, "Ci * Co overflows");
    if (!w_host) return fail(DQ_ERR_INVALID_ARG, "w_host is NULL");
    if (dt != DQ_F32 && dt != DQ_BF16) return fail(DQ_ERR_INVALID_ARG, "unknown dtype");
    if (rank < 0 || rank > std::min(Ci, Co)) return fail(DQ_ERR_INVALID_ARG, "rank must be in [0, min(Ci, Co)]");
    if (rank == 0) return DQ_OK;
    if (!l1_host || !l2_host) return fail(DQ_ERR_INVALID_ARG, "factor output is NULL");
    std::vector<float> wf;
    const float* wt = (const float*)w_host;
    try {
        if (dt == DQ_BF16) {
            wf.resize((size_t)(Ci * Co));
            const uint16_t* b = (const uint16_t*)w_host;
            for (size_t i = 0; i < wf.size(); ++i) {
                uint32_t u = (uint32_t)b[i] << 16;
                std::memcpy(&wf[i], &u, 4);
            }
            wt = wf.data();
        }
        lowrank_svd(wt, Ci, Co, rank, seed, l1_host, l2_host);
    } catch (const std::bad_alloc&) {
        return fail(DQ_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    return DQ_OK;
}

}  // extern "C"

// Weight preparation for a given code format of R (FMT_FP4, or the 6-bit
// FMT_FP6 / FMT_BF6).
static dq_status prepare_weights(const void* w_host, dq_dtype dt, int64_t Ci, int64_t Co, int32_t rank,
                                 const uint16_t* l1_host, const uint16_t* l2_host, int32_t device, int wfmt,
                                 dq_weights** out) {
    g_last_error.clear();
    if (!out) return fail(DQ_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!w_host) return fail(DQ_ERR_INVALID_ARG, "w_host is NULL");
    if (dt != DQ_F32 && dt != DQ_BF16) return fail(DQ_ERR_INVALID_ARG, "unknown dtype");
    if (Ci < 32 || Ci % 32 != 0) return fail(DQ_ERR_SHAPE, "Ci must be a positive multiple of 32");
    if (Co < 1) return fail(DQ_ERR_SHAPE, "Co must be >= 1");
    if (Ci > (1 << 24) || Co > (1 << 24)) return fail(DQ_ERR_SHAPE, "Ci and Co must be <= 2^24");
    if (rank < 0 || rank > std::min(Ci, Co)) return fail(DQ_ERR_INVALID_ARG, "rank must be in [0, min(Ci, Co)]");
    if (rank > 128) return fail(DQ_ERR_INVALID_ARG, "rank must be <= 128");
    if (rank > 0 && (!l1_host || !l2_host)) return fail(DQ_ERR_INVALID_ARG, "factors are NULL");
    dq_status st = check_device(device);
    if (st != DQ_OK) return st;
    DeviceGuard dg(device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");

    auto* w = new (std::nothrow) dq_weights();
    if (!w) return fail(DQ_ERR_OUT_OF_MEMORY, "host allocation failed");
    std::unique_ptr<dq_weights, void (*)(dq_weights*)> guard(w, free_weights);
    w->device = device;
    w->Ci = Ci;
    w->Co = Co;
    w->rank = rank;
    w->rp = (int)round_up(rank, RPAD);
    w->Kp = round_up(Ci, KPAD);
    w->Cop = round_up(Co, NPAD);
    w->wfmt = wfmt;
    const bool six = wfmt != 4;
    const size_t esz = dt == DQ_BF16 ? 2 : 4;

    void* wdev = nullptr;
    uint16_t *l1d = nullptr, *l2d = nullptr;
    size_t scratch = 0;
    hipError_t e = hipSuccess;
    auto cleanup = [&]() {
        (void)hipFree(wdev);
        (void)hipFree(l1d);
        (void)hipFree(l2d);
    };
    try {
        w->l1.assign(l1_host ? l1_host : (const uint16_t*)nullptr, l1_host ? l1_host + Ci * rank : nullptr);
        w->l2.assign(l2_host ? l2_host : (const uint16_t*)nullptr, l2_host ? l2_host + (int64_t)rank * Co : nullptr);
    } catch (const std::bad_alloc&) {
        return fail(DQ_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    if ((e = hipMalloc(&wdev, (size_t)(Ci * Co) * esz)) != hipSuccess) { cleanup(); return hip_fail(e, "hipMalloc W"); }
    if ((e = hipMemcpy(wdev, w_host, (size_t)(Ci * Co) * esz, hipMemcpyHostToDevice)) != hipSuccess) { cleanup(); return hip_fail(e, "copy W"); }
    if (rank > 0) {
        if ((e = dalloc(&l1d, (size_t)(Ci * rank), &scratch)) != hipSuccess ||
            (e = dalloc(&l2d, (size_t)(rank * Co), &scratch)) != hipSuccess) { cleanup(); return hip_fail(e, "hipMalloc factors"); }
        if ((e = hipMemcpy(l1d, l1_host, (size_t)(Ci * rank) * 2, hipMemcpyHostToDevice)) != hipSuccess ||
            (e = hipMemcpy(l2d, l2_host, (size_t)(rank * Co) * 2, hipMemcpyHostToDevice)) != hipSuccess) { cleanup(); return hip_fail(e, "copy factors"); }
    }
    if ((e = dalloc(&w->r, (size_t)(Ci * Co), &w->bytes)) != hipSuccess ||
        (e = dalloc(&w->rq, (size_t)(w->Cop * w->Kp / 2 * (six ? 3 : 2) / 2), &w->bytes)) != hipSuccess ||
        (e = dalloc(&w->rs, (size_t)(w->Cop * w->Kp / 32), &w->bytes)) != hipSuccess) { cleanup(); return hip_fail(e, "hipMalloc weight"); }
    if ((e = launch_residual(wdev, dt == DQ_BF16, l1d, l2d, Ci, Co, rank, w->r, nullptr)) != hipSuccess) { cleanup(); return hip_fail(e, "residual kernel"); }
    e = six ? launch_encode_fp6(w->r, 0, Co, Ci, Ci, w->Kp, w->rq, w->rs, wfmt == 3, nullptr)
            : launch_encode_fp4_rows(w->r, Co, Ci, Ci, w->Kp, w->rq, w->rs, nullptr);
    if (e != hipSuccess) { cleanup(); return hip_fail(e, "encode kernel"); }
    if (w->rp > 0) {
        std::vector<uint16_t> l1t((size_t)(w->rp * w->Kp), 0), l2t((size_t)(w->Cop * w->rp), 0);
        for (int64_t c = 0; c < Ci; ++c)
            for (int q = 0; q < rank; ++q) l1t[(size_t)(q * w->Kp + c)] = l1_host[c * rank + q];
        for (int q = 0; q < rank; ++q)
            for (int64_t j = 0; j < Co; ++j) l2t[(size_t)(j * w->rp + q)] = l2_host[(int64_t)q * Co + j];
        if ((e = dalloc(&w->l1t, l1t.size(), &w->bytes)) != hipSuccess ||
            (e = dalloc(&w->l2t, l2t.size(), &w->bytes)) != hipSuccess) { cleanup(); return hip_fail(e, "hipMalloc factors"); }
        if ((e = hipMemcpy(w->l1t, l1t.data(), l1t.size() * 2, hipMemcpyHostToDevice)) != hipSuccess ||
            (e = hipMemcpy(w->l2t, l2t.data(), l2t.size() * 2, hipMemcpyHostToDevice)) != hipSuccess) { cleanup(); return hip_fail(e, "copy factors"); }
    }
    if ((e = hipDeviceSynchronize()) != hipSuccess) { cleanup(); return hip_fail(e, "weight preparation"); }
    cleanup();
    *out = guard.release();
    return DQ_OK;
}

extern "C" {

dq_status dq_prepare_weights_lowrank(const void* w_host, dq_dtype dt, int64_t Ci, int64_t Co, int32_t rank,
                                     const uint16_t* l1_host, const uint16_t* l2_host, int32_t device,
                                     dq_weights** out) {
    return prepare_weights(w_host, dt, Ci, Co, rank, l1_host, l2_host, device, 4, out);
}

dq_status dq_prepare_weights_w6(const void* w_host, dq_dtype dt, int64_t Ci, int64_t Co, int32_t rank,
                                const uint16_t* l1_host, const uint16_t* l2_host, int32_t fp6_format, int32_t device,
                                dq_weights** out) {
    if (out) *out = nullptr;
    if (fp6_format != DQ_FP6_E2M3 && fp6_format != DQ_FP6_E3M2) {
        g_last_error.clear();
        return fail(DQ_ERR_INVALID_ARG, "fp6_format must be DQ_FP6_E2M3 or DQ_FP6_E3M2");
    }
    return prepare_weights(w_host, dt, Ci, Co, rank, l1_host, l2_host, device, (int)fp6_format, out);
}

dq_status dq_prepare_weights(const void* w_host, dq_dtype dt, int64_t Ci, int64_t Co, int32_t rank, uint64_t seed,
                             int32_t device, dq_weights** out) {
    if (!out) return fail(DQ_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (Ci < 1 || Co < 1) return fail(DQ_ERR_SHAPE, "Ci and Co must be >= 1");
    if (Ci > (1 << 24) || Co > (1 << 24)) return fail(DQ_ERR_SHAPE, "Ci and Co must be <= 2^24");
    if (rank < 0 || rank > std::min(Ci, Co)) return fail(DQ_ERR_INVALID_ARG, "rank must be in [0, min(Ci, Co)]");
    std::vector<uint16_t> l1, l2;
    try {
        l1.resize((size_t)(Ci * rank));
        l2.resize((size_t)(rank * Co));
    } catch (const std::bad_alloc&) {
        return fail(DQ_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    dq_status st = dq_lowrank_factors(w_host, dt, Ci, Co, rank, seed, l1.data(), l2.data());
    if (st != DQ_OK) return st;
    return dq_prepare_weights_lowrank(w_host, dt, Ci, Co, rank, l1.data(), l2.data(), device, out);
}

void dq_weights_destroy(dq_weights* w) { free_weights(w); }

dq_status dq_weights_info(const dq_weights* w, int64_t* Ci, int64_t* Co, int32_t* rank, int32_t* device) {
    if (!w) return fail(DQ_ERR_INVALID_ARG, "weights handle is NULL");
    if (Ci) *Ci = w->Ci;
    if (Co) *Co = w->Co;
    if (rank) *rank = w->rank;
    if (device) *device = w->device;
    return DQ_OK;
}

dq_status dq_weights_export(const dq_weights* w, uint16_t* l1_host, uint16_t* l2_host, float* r_host,
                            uint8_t* rcodes_host, uint8_t* rscales_host) {
    g_last_error.clear();
    if (!w) return fail(DQ_ERR_INVALID_ARG, "weights handle is NULL");
    DeviceGuard dg(w->device);
    if (l1_host && w->rank) std::memcpy(l1_host, w->l1.data(), w->l1.size() * 2);
    if (l2_host && w->rank) std::memcpy(l2_host, w->l2.data(), w->l2.size() * 2);
    hipError_t e;
    if (r_host && (e = hipMemcpy(r_host, w->r, (size_t)(w->Ci * w->Co) * 4, hipMemcpyDeviceToHost)) != hipSuccess)
        return hip_fail(e, "copy R");
    try {
        std::vector<uint8_t> buf;
        if (rcodes_host && w->wfmt != 4) {
            if ((e = fetch_all(w->rq, (size_t)(w->Cop * w->Kp / 4 * 3), buf)) != hipSuccess) return hip_fail(e, "copy R codes");
            for (int64_t j = 0; j < w->Co; ++j) unstep_fp6(buf, j, w->Ci, w->Kp, rcodes_host + j * (w->Ci / 4 * 3));
        } else if (rcodes_host) {
            if ((e = fetch_all(w->rq, (size_t)(w->Cop * w->Kp / 2), buf)) != hipSuccess) return hip_fail(e, "copy R codes");
            for (int64_t j = 0; j < w->Co; ++j) unstep_fp4(buf, j, w->Ci, w->Kp, rcodes_host + j * (w->Ci / 2));
        }
        if (rscales_host) {
            if ((e = fetch_all(w->rs, (size_t)(w->Cop * w->Kp / 32), buf)) != hipSuccess) return hip_fail(e, "copy R scales");
            for (int64_t j = 0; j < w->Co; ++j) unstep_scales(buf, j, w->Ci, w->Kp, rscales_host + j * (w->Ci / 32));
        }
    } catch (const std::bad_alloc&) {
        return fail(DQ_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    return DQ_OK;
}

dq_status dq_qact_create(const dq_weights* w, dq_geom geom, dq_qact** out) {
    return dq_qact_create_ex(w, geom, 32, 8, out);
}

}  // extern "C"

namespace dq {
// Checks a geometry and the core options against a weight and fills the
// workspace's sizes and frame segments (no allocation, no device work).
KSplit plan_ksplit(int mt, int nt, int nks, int ns, int cus, double step_us) {
    KSplit k;
    const int G = std::max(8, cus / 8 * 8);                         // the persistent grid of a full round
    const int T = mt * nt, full = T / G * G, rm = T - full;
    if (rm == 0) return k;
    // time saved against one more round of whole tiles: the chunks' share of
    // the tile, less the partials' round trip (0.07 us per 256 KB unit,
    // written and read back), about 10 us for the two extra launches, and
    // the part of the last round that hides in the spread of the full
    // rounds' finishing times (the workgroups of a persistent launch end
    // about 4 % of its length apart, and each starts its last-round tile as
    // it finishes).  Same-box core-term times, split against one launch:
    //   FP8 x FP4, 720p FFN down, 2x2x2 cubes (3 rounds + 32 tiles of 108
    //     steps): 0.642 -> 0.55 ms; global cube (20 tiles): 0.149 -> 0.043;
    //   FP8 x FP4, 14B attention projection (1 round + 64 tiles of 40 steps):
    //     0.140 -> 0.124; 720p FFN up, 4x2x8 cubes (1 round + 68): 0.147 -> 0.128;
    //   bf16, the same two layers (160 steps of 32 channels): 0.259 -> 0.199
    //     and 0.268 -> 0.212;
    //   FP8 x FP4, 720p FFN up, 1x2x2 cubes (16 rounds + 8 tiles of 40 steps):
    //     1.094 -> 1.112, so that one (drift 41 us against a 38 us saving)
    //     keeps one launch.
    const double tile = nks * step_us, drift = 0.04 * (full / G) * tile;
    double best = 0;
    for (int q = 2; q * rm <= G && nks / q >= ns; ++q) {
        const double gain = tile * (1.0 - 1.0 / q) - 0.07 * rm * q - 10.0 - drift;
        if (gain > best) {
            best = gain;
            k.p = q;
        }
    }
    if (best < std::max(5.0, 0.15 * tile)) return KSplit{};         // (within the model's error: keep one launch)
    k.main_tiles = full;
    k.rm = rm;
    return k;
}

dq_status plan_qact(const dq_weights* w, const dq_geom& geom, int core_group, int core_bits, dq_qact* q,
                    int64_t* max_partials_out) {
    if (w->wfmt != 4) return fail(DQ_ERR_INVALID_ARG, "a 6-bit weight takes the 6-bit entry points");
    if (core_group != 32 && core_group != 64) return fail(DQ_ERR_INVALID_ARG, "core_group must be 32 or 64");
    if (core_bits != 8 && core_bits != 4 && core_bits != 16) return fail(DQ_ERR_INVALID_ARG, "core_bits must be 8, 4 or 16");
    if (w->Ci % core_group != 0) return fail(DQ_ERR_SHAPE, "core_group must divide Ci");
    const dq_geom& G = geom;
    if (G.T < 1 || G.H < 1 || G.W < 1) return fail(DQ_ERR_SHAPE, "T, H, W must be >= 1");
    if (G.t < 1 || G.t > G.T || G.h < 1 || G.h > G.H || G.w < 1 || G.w > G.W)
        return fail(DQ_ERR_SHAPE, "cube extents must satisfy 1 <= t <= T, 1 <= h <= H, 1 <= w <= W");
    const int64_t lim = int64_t(1) << 40;
    // (products checked before they are formed: T, H, W reach 2^31 - 1)
    if (!mul_ok(G.T, G.H, lim) || !mul_ok((int64_t)G.T * G.H, G.W, lim)) return fail(DQ_ERR_SHAPE, "token grid too large");
    int64_t N = (int64_t)G.T * G.H * G.W;
    int Tc = (int)(((int64_t)G.T + G.t - 1) / G.t), Hc = (int)(((int64_t)G.H + G.h - 1) / G.h),
        Wc = (int)(((int64_t)G.W + G.w - 1) / G.w);
    int64_t K = (int64_t)Tc * Hc * Wc;
    int64_t S = (int64_t)G.t * G.h * G.w;
    if (N > (int64_t(1) << 31) || !mul_ok(K, S, lim)) return fail(DQ_ERR_SHAPE, "token grid too large");
    int64_t Nslot = K * S;
    if (Nslot > (int64_t(1) << 31) - MPAD) return fail(DQ_ERR_SHAPE, "slot count too large");
    q->device = w->device;
    q->Ci = w->Ci;
    q->Co = w->Co;
    q->Kp = w->Kp;
    q->Cop = w->Cop;
    q->rp = w->rp;
    q->rank = w->rank;
    q->g = Geom{G.T, G.H, G.W, G.t, G.h, G.w, Tc, Hc, Wc, (int)S, (long long)N, (long long)K, (long long)Nslot};
    q->core_group = core_group;
    q->core_bits = core_bits;
    // frame segments: whole frame groups, then the clipped last group (if any)
    const int T0 = G.T - G.T % G.t;                  // >= t, since t <= T
    const int segT[2] = {T0, G.T - T0}, segt[2] = {G.t, G.T - T0};
    q->nseg = T0 < G.T ? 2 : 1;
    int64_t row = 0, krow = 0, tok = 0, kk = 0, max_partials = 0;
    for (int i = 0; i < q->nseg; ++i) {
        dq_segment& sg = q->seg[i];
        const int tc = (segT[i] + segt[i] - 1) / segt[i];
        const int64_t Ks = (int64_t)tc * Hc * Wc, Ss = (int64_t)segt[i] * G.h * G.w;
        const int64_t Ns = (int64_t)segT[i] * G.H * G.W;
        sg.g = Geom{segT[i], G.H, G.W, segt[i], G.h, G.w, tc, Hc, Wc, (int)Ss, (long long)Ns, (long long)Ks,
                    (long long)(Ks * Ss)};
        sg.tok0 = tok;
        sg.k0 = kk;
        sg.row0 = row;
        sg.krow0 = krow;
        sg.core_mode = Ss <= 64 ? 0 : 1;
        sg.nblk = (Ss + CORE_BLOCK - 1) / CORE_BLOCK;
        if (sg.core_mode == 1) max_partials = std::max(max_partials, Ks * sg.nblk);
        tok += Ns;
        kk += Ks;
        row += round_up(Ks * Ss, MPAD);
        krow += round_up(Ks, MPAD);
    }
    q->Nslot_pad = row;
    q->K_pad = krow;
    if (!mul_ok(q->Nslot_pad, q->Kp, lim) || !mul_ok(q->K_pad, q->Cop, lim) || !mul_ok(max_partials, q->Kp, lim))
        return fail(DQ_ERR_SHAPE, "workspace too large");
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, w->device) != hipSuccess || cus <= 0) cus = 256;
    q->cus = cus;
    // the activation pass's channel split: the U partials of the largest
    // segment it may split (blocks of 64 slots, or of whole cubes up to 64
    // tokens)
    q->upart_rows = 0;
    for (int i = 0; i < q->nseg; ++i) {
        const dq_segment& sg = q->seg[i];
        const int64_t nblocks = sg.core_mode == 0 ? (sg.g.K + 64 / sg.g.S - 1) / (64 / sg.g.S) : (sg.g.Nslot + 63) / 64;
        if (nblocks * 2 <= cus) q->upart_rows = std::max<int64_t>(q->upart_rows, sg.g.Nslot);
    }
    // the core GEMM's K split (one-token cubes with FP8 or FP4 cores run no
    // core GEMM).  Per-step times of a tile with every CU busy: FP8 x FP4
    // steps of 128 channels 1.6 us, FP4 x FP4 1.0 us, bf16 steps of 32
    // channels 0.8 us (720p FFN up-projection).
    q->ks = KSplit{};
    if (!(S == 1 && core_bits != 16)) {
        const int nks = (int)(core_bits == 16 ? q->Kp / 32 : q->Kp / 128);
        q->ks = plan_ksplit((int)(q->Cop / 256), (int)(q->K_pad / 256), nks, core_bits == 8 ? 3 : 4, cus,
                            core_bits == 8 ? 1.6 : (core_bits == 4 ? 1.0 : 0.8));
    }
    *max_partials_out = max_partials;
    return DQ_OK;
}
}  // namespace dq

extern "C" {

dq_status dq_qact_create_ex(const dq_weights* w, dq_geom geom, int32_t core_group, int32_t core_bits,
                            dq_qact** out) {
    g_last_error.clear();
    if (!out) return fail(DQ_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!w) return fail(DQ_ERR_INVALID_ARG, "weights handle is NULL");
    auto* q = new (std::nothrow) dq_qact();
    if (!q) return fail(DQ_ERR_OUT_OF_MEMORY, "host allocation failed");
    std::unique_ptr<dq_qact, void (*)(dq_qact*)> guard(q, free_qact);
    int64_t max_partials = 0;
    dq_status st = plan_qact(w, geom, core_group, core_bits, q, &max_partials);
    if (st != DQ_OK) return st;
    DeviceGuard dg(w->device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");
    hipError_t e;
    if ((e = dalloc(&q->dq, (size_t)(q->Nslot_pad * q->Kp / 2), &q->bytes)) != hipSuccess ||
        (e = dalloc(&q->ds, (size_t)(q->Nslot_pad * q->Kp / 32), &q->bytes)) != hipSuccess ||
        (e = dalloc(&q->cq, (size_t)(q->K_pad * q->Kp), &q->bytes)) != hipSuccess ||
        (e = dalloc(&q->cs, (size_t)(q->K_pad * q->Kp / 32), &q->bytes)) != hipSuccess ||
        (e = dalloc(&q->u, (size_t)(q->Nslot_pad * q->rp), &q->bytes)) != hipSuccess ||
        (e = dalloc(&q->bias, (size_t)(q->K_pad * q->Cop), &q->bytes)) != hipSuccess ||
        (e = dalloc(&q->stok, (size_t)q->Nslot_pad, &q->bytes)) != hipSuccess ||
        (e = dalloc(&q->zero, (size_t)512, &q->bytes)) != hipSuccess ||
        (e = dalloc(&q->sink, (size_t)512, &q->bytes)) != hipSuccess)
        return hip_fail(e, "hipMalloc workspace");
    for (int i = 0; i < q->nseg; ++i) {
        const dq_segment& sg = q->seg[i];
        const int64_t rows = (i + 1 < q->nseg ? q->seg[i + 1].row0 : q->Nslot_pad) - sg.row0;
        if ((e = launch_slot_tokens(sg.g, sg.tok0, q->stok + sg.row0, rows, nullptr)) != hipSuccess)
            return hip_fail(e, "slot table");
    }
    if (max_partials > 0) {
        if ((e = dalloc(&q->coref, (size_t)(q->K_pad * q->Kp), &q->bytes)) != hipSuccess ||
            (e = dalloc(&q->part, (size_t)(max_partials * q->Kp), &q->bytes)) != hipSuccess)
            return hip_fail(e, "hipMalloc workspace");
    }
    if (q->ks.rm > 0 && (e = dalloc(&q->kpart, q->ks.part_bytes() / 4, &q->bytes)) != hipSuccess)
        return hip_fail(e, "hipMalloc workspace");
    if (q->upart_rows > 0 && q->rp > 0 &&
        (e = dalloc(&q->upart, (size_t)(QMAXPARTS * q->upart_rows * q->rp), &q->bytes)) != hipSuccess)
        return hip_fail(e, "hipMalloc workspace");
    if (core_bits == 16) {                          // bf16 cores: Q4(R) as bf16 for the bf16 GEMM
        if ((e = dalloc(&q->cbf, (size_t)(q->K_pad * q->Kp), &q->bytes)) != hipSuccess ||
            (e = dalloc(&q->rbf, (size_t)(q->Cop * q->Kp), &q->bytes)) != hipSuccess)
            return hip_fail(e, "hipMalloc workspace");
        if ((e = launch_decode_fp4_bf16(w->rq, w->rs, q->Cop, q->Kp, q->rbf, nullptr)) != hipSuccess)
            return hip_fail(e, "decode Q4(R)");
    }
    if ((e = hipDeviceSynchronize()) != hipSuccess) return hip_fail(e, "workspace init");
    *out = guard.release();
    return DQ_OK;
}

void dq_qact_destroy(dq_qact* q) { free_qact(q); }

dq_status dq_qact_info(const dq_qact* q, int64_t* N, int64_t* K, int64_t* device_bytes) {
    if (!q) return fail(DQ_ERR_INVALID_ARG, "workspace handle is NULL");
    if (N) *N = q->g.N;
    if (K) *K = q->g.K;
    if (device_bytes) *device_bytes = (int64_t)q->bytes;
    return DQ_OK;
}

static dq_status check_pair(const dq_weights* w, const dq_qact* q) {
    if (!w) return fail(DQ_ERR_INVALID_ARG, "weights handle is NULL");
    if (!q) return fail(DQ_ERR_INVALID_ARG, "workspace handle is NULL");
    if (w->wfmt != 4) return fail(DQ_ERR_INVALID_ARG, "a 6-bit weight takes the 6-bit entry points");
    if (q->Ci != w->Ci || q->Co != w->Co || q->rp != w->rp || q->device != w->device)
        return fail(DQ_ERR_INVALID_ARG, "workspace was created for a different weight");
    return DQ_OK;
}

dq_status dq_quantize_act(const dq_weights* w, const void* x_dev, dq_dtype dt, dq_qact* q, void* stream) {
    g_last_error.clear();
    dq_status st = check_pair(w, q);
    if (st != DQ_OK) return st;
    if (!x_dev) return fail(DQ_ERR_INVALID_ARG, "x_dev is NULL");
    if (((uintptr_t)x_dev) % 16 != 0) return fail(DQ_ERR_INVALID_ARG, "x_dev must be 16-byte aligned");
    if (dt != DQ_F32 && dt != DQ_BF16) return fail(DQ_ERR_INVALID_ARG, "unknown dtype");
    DeviceGuard dg(q->device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");
    hipError_t e = launch_quantize(w, x_dev, dt == DQ_BF16, q, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "activation pass launch");
    return DQ_OK;
}

static dq_status forward_parts(const dq_weights* w, dq_qact* q, float* y_dev, int parts, void* stream) {
    g_last_error.clear();
    dq_status st = check_pair(w, q);
    if (st != DQ_OK) return st;
    if ((parts & dq::FWD_DELTA) && !y_dev) return fail(DQ_ERR_INVALID_ARG, "y_dev is NULL");
    if (((uintptr_t)y_dev) % 4 != 0) return fail(DQ_ERR_INVALID_ARG, "y_dev must be 4-byte aligned");
    DeviceGuard dg(q->device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");
    hipError_t e = launch_forward(w, q, y_dev, parts, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "forward launch");
    return DQ_OK;
}

dq_status dq_linear_forward(const dq_weights* w, dq_qact* q, float* y_dev, void* stream) {
    return forward_parts(w, q, y_dev, dq::FWD_CORE | dq::FWD_DELTA, stream);
}

dq_status dq_forward_form(const dq_weights* w, const dq_qact* q, int* one_kernel) {
    g_last_error.clear();
    dq_status st = check_pair(w, q);
    if (st != DQ_OK) return st;
    if (!one_kernel) return fail(DQ_ERR_INVALID_ARG, "one_kernel is NULL");
    DeviceGuard dg(q->device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");
    alignas(16) static const float aligned_y = 0.0f;           // stands for a 16-byte aligned y_dev
    *one_kernel = dq::fused_preferred(w, q, &aligned_y) ? 1 : 0;
    return DQ_OK;
}

dq_status dq_linear_forward_fused(const dq_weights* w, dq_qact* q, float* y_dev, void* stream) {
    g_last_error.clear();
    dq_status st = check_pair(w, q);
    if (st != DQ_OK) return st;
    if (!y_dev) return fail(DQ_ERR_INVALID_ARG, "y_dev is NULL");
    if (!dq::fused_applies(w, q, y_dev))
        return fail(DQ_ERR_INVALID_ARG, "the fused forward takes cubes of 4 tokens with FP8 cores in one frame segment, "
                                        "rank 32, Co a multiple of 256, Ci of 512 or more and a 16-byte aligned y_dev");
    DeviceGuard dg(q->device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");
    hipError_t e = dq::launch_forward_fused(w, q, y_dev, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "fused forward launch");
    return DQ_OK;
}

dq_status dq_core_term(const dq_weights* w, dq_qact* q, void* stream) {
    return forward_parts(w, q, nullptr, dq::FWD_CORE, stream);
}

dq_status dq_delta_term(const dq_weights* w, dq_qact* q, float* y_dev, void* stream) {
    return forward_parts(w, q, y_dev, dq::FWD_DELTA, stream);
}

dq_status dq_linear(const dq_weights* w, const void* x_dev, dq_dtype dt, dq_qact* q, float* y_dev, void* stream) {
    dq_status st = dq_quantize_act(w, x_dev, dt, q, stream);
    if (st != DQ_OK) return st;
    return dq_linear_forward(w, q, y_dev, stream);
}

dq_status dq_qact_export(const dq_qact* q, uint8_t* dcodes_host, uint8_t* dscales_host, uint8_t* ccodes_host,
                         uint8_t* cscales_host, uint16_t* u_host, void* stream) {
    g_last_error.clear();
    if (!q) return fail(DQ_ERR_INVALID_ARG, "workspace handle is NULL");
    DeviceGuard dg(q->device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "stream synchronize");
    const Geom& g = q->g;
    const int64_t Ci = q->Ci, Kp = q->Kp;
    // (slot row, token) of every token, and the row of every cube
    auto each_slot = [&](auto&& fn) {
        for (int i = 0; i < q->nseg; ++i) {
            const dq_segment& sg = q->seg[i];
            for (long long s = 0; s < sg.g.Nslot; ++s) {
                const long long t = host_slot_token(sg.g, s);
                if (t >= 0) fn(sg.row0 + s, sg.tok0 + t);
            }
        }
    };
    auto cube_row = [&](long long k) {
        const dq_segment& sg = q->seg[q->nseg > 1 && k >= q->seg[1].k0 ? 1 : 0];
        return sg.krow0 + (k - sg.k0);
    };
    try {
        std::vector<uint8_t> buf;
        // One-token cubes: every delta is x - x = +0 exactly, coded 0 with
        // scale code 0 (2^-127); the activation pass does not store them.
        const bool zero_deltas = g.S == 1;
        if (dcodes_host && zero_deltas) {
            std::memset(dcodes_host, 0, (size_t)(g.N * (Ci / 2)));
        } else if (dcodes_host) {
            if ((e = fetch_all(q->dq, (size_t)(q->Nslot_pad * Kp / 2), buf)) != hipSuccess) return hip_fail(e, "copy delta codes");
            each_slot([&](long long s, long long t) { unstep_fp4(buf, s, Ci, Kp, dcodes_host + t * (Ci / 2)); });
        }
        if (dscales_host && zero_deltas) {
            std::memset(dscales_host, 0, (size_t)(g.N * (Ci / 32)));
        } else if (dscales_host) {
            if ((e = fetch_all(q->ds, (size_t)(q->Nslot_pad * Kp / 32), buf)) != hipSuccess) return hip_fail(e, "copy delta scales");
            each_slot([&](long long s, long long t) { unstep_scales(buf, s, Ci, Kp, dscales_host + t * (Ci / 32)); });
        }
        if (ccodes_host && q->core_bits == 16) {            // bf16 bits, two bytes per value
            if ((e = fetch_all(q->cbf, (size_t)(q->K_pad * Kp * 2), buf)) != hipSuccess) return hip_fail(e, "copy cores");
            for (long long k = 0; k < g.K; ++k)
                for (int64_t c = 0; c < Ci; c += 8)
                    std::memcpy(ccodes_host + (k * Ci + c) * 2, &buf[off_bf16(cube_row(k), c, Kp / 32)], 16);
        } else if (ccodes_host) {
            if ((e = fetch_all(q->cq, (size_t)(q->K_pad * Kp), buf)) != hipSuccess) return hip_fail(e, "copy core codes");
            if (q->core_bits == 4) {                      // packed nibbles -> one code per byte
                std::vector<uint8_t> row((size_t)(Ci / 2));
                for (long long k = 0; k < g.K; ++k) {
                    unstep_fp4(buf, cube_row(k), Ci, Kp, row.data());
                    for (int64_t c = 0; c < Ci; ++c) ccodes_host[k * Ci + c] = (uint8_t)((row[c / 2] >> (4 * (c & 1))) & 15);
                }
            } else {
                for (long long k = 0; k < g.K; ++k) unstep_fp8(buf, cube_row(k), Ci, Kp, ccodes_host + k * Ci);
            }
        }
        if (cscales_host && q->core_bits != 16) {
            if ((e = fetch_all(q->cs, (size_t)(q->K_pad * Kp / 32), buf)) != hipSuccess) return hip_fail(e, "copy core scales");
            for (long long k = 0; k < g.K; ++k) unstep_scales(buf, cube_row(k), Ci, Kp, cscales_host + k * (Ci / 32));
        }
        if (u_host && q->rank > 0) {
            if ((e = fetch_all(q->u, (size_t)(q->Nslot_pad * q->rp * 2), buf)) != hipSuccess) return hip_fail(e, "copy U");
            const uint16_t* ub = (const uint16_t*)buf.data();
            each_slot([&](long long s, long long t) { std::memcpy(u_host + t * q->rank, ub + s * q->rp, (size_t)q->rank * 2); });
        }
    } catch (const std::bad_alloc&) {
        return fail(DQ_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    return DQ_OK;
}


// ---------------------------------------------------------------- 6-bit layers ----
static void free_act6(dq_act6* a) {
    if (!a) return;
    DeviceGuard dg(a->device);
    (void)hipFree(a->xq);
    (void)hipFree(a->xs);
    (void)hipFree(a->u);
    (void)hipFree(a->upart);
    (void)hipFree(a->stok);
    (void)hipFree(a->sink);
    delete a;
}

dq_status dq_act6_create(const dq_weights* w, int64_t N, dq_act6** out) {
    g_last_error.clear();
    if (!out) return fail(DQ_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!w) return fail(DQ_ERR_INVALID_ARG, "weights handle is NULL");
    if (w->wfmt == 4) return fail(DQ_ERR_INVALID_ARG, "a 4-bit weight takes dq_qact_create");
    if (N < 1 || N > (int64_t(1) << 31) - MPAD) return fail(DQ_ERR_SHAPE, "N must be in [1, 2^31 - 256]");
    if (!mul_ok(round_up(N, MPAD), w->Kp, int64_t(1) << 40) || !mul_ok(N, w->Co, int64_t(1) << 40))
        return fail(DQ_ERR_SHAPE, "workspace too large");
    DeviceGuard dg(w->device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");
    auto* a = new (std::nothrow) dq_act6();
    if (!a) return fail(DQ_ERR_OUT_OF_MEMORY, "host allocation failed");
    std::unique_ptr<dq_act6, void (*)(dq_act6*)> guard(a, free_act6);
    a->device = w->device;
    a->N = N;
    a->N_pad = round_up(N, MPAD);
    a->Ci = w->Ci;
    a->Co = w->Co;
    a->Kp = w->Kp;
    a->Cop = w->Cop;
    a->rp = w->rp;
    a->rank = w->rank;
    a->wfmt = w->wfmt;
    hipError_t e;
    if ((e = dalloc(&a->xq, (size_t)(a->N_pad * a->Kp / 4 * 3), &a->bytes)) != hipSuccess ||
        (e = dalloc(&a->xs, (size_t)(a->N_pad * a->Kp / 32), &a->bytes)) != hipSuccess ||
        (e = dalloc(&a->u, (size_t)(a->N_pad * a->rp), &a->bytes)) != hipSuccess ||
        (e = dalloc(&a->upart, (size_t)(text_lowrank_splits((int)a->Ci) * a->N_pad * a->rp), &a->bytes)) != hipSuccess ||
        (e = dalloc(&a->stok, (size_t)a->N_pad, &a->bytes)) != hipSuccess ||
        (e = dalloc(&a->sink, (size_t)512, &a->bytes)) != hipSuccess)
        return hip_fail(e, "hipMalloc workspace");
    // rows are tokens: the identity map (one-token "cubes" of a 1 x 1 x N grid), -1 past N
    const Geom g{1, 1, (int)N, 1, 1, 1, 1, 1, (int)N, 1, (long long)N, (long long)N, (long long)N};
    if ((e = launch_slot_tokens(g, 0, a->stok, a->N_pad, nullptr)) != hipSuccess) return hip_fail(e, "row table");
    if ((e = hipDeviceSynchronize()) != hipSuccess) return hip_fail(e, "workspace init");
    *out = guard.release();
    return DQ_OK;
}

void dq_act6_destroy(dq_act6* a) { free_act6(a); }

static dq_status check_pair6(const dq_weights* w, const dq_act6* a) {
    if (!w) return fail(DQ_ERR_INVALID_ARG, "weights handle is NULL");
    if (!a) return fail(DQ_ERR_INVALID_ARG, "workspace handle is NULL");
    if (w->wfmt == 4) return fail(DQ_ERR_INVALID_ARG, "a 4-bit weight takes the 4-bit entry points");
    if (a->Ci != w->Ci || a->Co != w->Co || a->rp != w->rp || a->device != w->device || a->wfmt != w->wfmt)
        return fail(DQ_ERR_INVALID_ARG, "workspace was created for a different weight");
    return DQ_OK;
}

dq_status dq_quantize_act6(const dq_weights* w, const void* x_dev, dq_dtype dt, dq_act6* a, void* stream) {
    g_last_error.clear();
    dq_status st = check_pair6(w, a);
    if (st != DQ_OK) return st;
    if (!x_dev) return fail(DQ_ERR_INVALID_ARG, "x_dev is NULL");
    if (((uintptr_t)x_dev) % 16 != 0) return fail(DQ_ERR_INVALID_ARG, "x_dev must be 16-byte aligned");
    if (dt != DQ_F32 && dt != DQ_BF16) return fail(DQ_ERR_INVALID_ARG, "unknown dtype");
    DeviceGuard dg(a->device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_encode_fp6(x_dev, dt == DQ_BF16, a->N, a->Ci, a->Ci, a->Kp, a->xq, a->xs, a->wfmt == 3, s);
    if (e != hipSuccess) return hip_fail(e, "6-bit activation launch");
    e = launch_text_lowrank(x_dev, dt == DQ_BF16, a->N, a->N_pad, (int)a->Ci, (int)a->Kp, w->l1t, a->rp, a->upart, a->u, s);
    if (e != hipSuccess) return hip_fail(e, "low-rank launch");
    return DQ_OK;
}

dq_status dq_linear6_forward(const dq_weights* w, dq_act6* a, float* y_dev, void* stream) {
    g_last_error.clear();
    dq_status st = check_pair6(w, a);
    if (st != DQ_OK) return st;
    if (!y_dev) return fail(DQ_ERR_INVALID_ARG, "y_dev is NULL");
    if (((uintptr_t)y_dev) % 4 != 0) return fail(DQ_ERR_INVALID_ARG, "y_dev must be 4-byte aligned");
    DeviceGuard dg(a->device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");
    hipError_t e = launch_forward6(w, a, y_dev, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "6-bit forward launch");
    return DQ_OK;
}

dq_status dq_linear6(const dq_weights* w, const void* x_dev, dq_dtype dt, dq_act6* a, float* y_dev, void* stream) {
    dq_status st = dq_quantize_act6(w, x_dev, dt, a, stream);
    if (st != DQ_OK) return st;
    return dq_linear6_forward(w, a, y_dev, stream);
}

dq_status dq_act6_export(const dq_act6* a, uint8_t* codes_host, uint8_t* scales_host, uint16_t* u_host, void* stream) {
    g_last_error.clear();
    if (!a) return fail(DQ_ERR_INVALID_ARG, "workspace handle is NULL");
    DeviceGuard dg(a->device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "stream synchronize");
    try {
        std::vector<uint8_t> buf;
        if (codes_host) {
            if ((e = fetch_all(a->xq, (size_t)(a->N_pad * a->Kp / 4 * 3), buf)) != hipSuccess) return hip_fail(e, "copy codes");
            for (int64_t n = 0; n < a->N; ++n) unstep_fp6(buf, n, a->Ci, a->Kp, codes_host + n * (a->Ci / 4 * 3));
        }
        if (scales_host) {
            if ((e = fetch_all(a->xs, (size_t)(a->N_pad * a->Kp / 32), buf)) != hipSuccess) return hip_fail(e, "copy scales");
            for (int64_t n = 0; n < a->N; ++n) unstep_scales(buf, n, a->Ci, a->Kp, scales_host + n * (a->Ci / 32));
        }
        if (u_host && a->rank > 0) {
            if ((e = fetch_all(a->u, (size_t)(a->N_pad * a->rp * 2), buf)) != hipSuccess) return hip_fail(e, "copy U");
            const uint16_t* ub = (const uint16_t*)buf.data();
            for (int64_t n = 0; n < a->N; ++n) std::memcpy(u_host + n * a->rank, ub + n * a->rp, (size_t)a->rank * 2);
        }
    } catch (const std::bad_alloc&) {
        return fail(DQ_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    return DQ_OK;
}

}  // extern "C"
