// Rotated-basis W4A4 layers in the manner of the OrbitQuant notes (方法:
// 核心思路, 离线的权重量化, 在线的激活量化): a random permuted block Hadamard
// rotation (RPBH) maps every row onto a normalized basis in which its
// coordinates are close to N(0, 1); each coordinate is coded as its nearest
// level of one fixed Lloyd-Max codebook of N(0, 1).  Weights are rotated and
// coded offline, row by row; activations per call, token by token; the
// rotation cancels in the product, y = x W^T.
//
// Conventions of this implementation (the notes fix none of them):
//   * rotation: x' = blockdiag(H_256 / 16) x[perm], the permutation given by
//     the caller; the Walsh-Hadamard transform as the radix-2 butterfly
//     network in fp32 (stages h = 1, 2, .., 128), then the exact 1/16;
//   * normalization: s = sqrt(sum x'^2 / Ci) in fp32 (squares summed per
//     256-channel block in channel order, then over blocks in order); the
//     coordinates coded are fl32(x' / s) (0 when s = 0);
//   * codebook: the Lloyd-Max quantizer of N(0, 1) with 2^bits levels, each
//     level rounded to bf16 (the operand type of the matrix cores, since a
//     Lloyd-Max level set is no float format); nearest level, exact ties to
//     the even index;
//   * y[n][j] = fl32(fl32(acc s_x[n]) s_w[j]), acc the bf16 MFMA contraction
//     of the decoded levels (fp32 accumulation).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <memory>
#include <new>
#include <string>
#include <vector>

#include "dq.h"
#include "dq_device.h"
#include "dq_internal.h"

struct dq_orbit {
    int device = 0;
    int64_t Ci = 0, Co = 0, Kp = 0, Cop = 0;
    int wbits = 4, abits = 4;
    uint16_t wlev[16] = {}, alev[16] = {};   // bf16 codebooks (ascending)
    int* perm = nullptr;       // [Ci] device
    uint16_t* wdec = nullptr;  // Cop x Kp bf16 decoded weight levels, off_bf16 layout
    uint8_t* wcodes = nullptr; // [Cop][Kp/2] level indices, two per byte
    float* wscale = nullptr;   // [Cop] row scales (0 past Co)
    size_t bytes = 0;
};

struct dq_orbit_act {
    int device = 0;
    int64_t N = 0, N_pad = 0, Ci = 0, Kp = 0;
    uint16_t* xdec = nullptr;  // N_pad x Kp bf16 decoded activation levels, off_bf16 layout
    uint8_t* xcodes = nullptr; // [N_pad][Kp/2]
    float* xscale = nullptr;   // [N_pad]
    int* rows = nullptr;       // [N_pad] identity, -1 past N
    float* sink = nullptr;     // [512]
    size_t bytes = 0;
};

namespace dq {
namespace {

constexpr int OBLOCK = 256;       // Hadamard block
constexpr int MAX_CI = 15360;     // the rotation pass holds a row twice in LDS (at most 120 KB of the 160 KB)

// Lloyd-Max quantizer of N(0, 1) with L levels, ascending: the fixed point of
// boundaries at the midpoints of neighbouring levels and levels at the
// conditional means of their cells, E[X | a < X <= b] =
// (pdf(a) - pdf(b)) / (cdf(b) - cdf(a)), iterated from evenly spaced points.
void lloyd_max(int L, double* y) {
    const double rt2pi = std::sqrt(2.0 * M_PI);
    auto pdf = [&](double t) { return std::isinf(t) ? 0.0 : std::exp(-0.5 * t * t) / rt2pi; };
    auto cdf = [&](double t) { return std::isinf(t) ? (t > 0 ? 1.0 : 0.0) : 0.5 * std::erfc(-t / std::sqrt(2.0)); };
    for (int i = 0; i < L; ++i) y[i] = -2.5 + 5.0 * (i + 0.5) / L;
    std::vector<double> t(L + 1);
    for (int it = 0; it < 100000; ++it) {
        t[0] = -INFINITY;
        t[L] = INFINITY;
        for (int i = 1; i < L; ++i) t[i] = 0.5 * (y[i - 1] + y[i]);
        double moved = 0.0;
        for (int i = 0; i < L; ++i) {
            const double v = (pdf(t[i]) - pdf(t[i + 1])) / (cdf(t[i + 1]) - cdf(t[i]));
            moved = std::max(moved, std::fabs(v - y[i]));
            y[i] = v;
        }
        if (moved <= 1e-15) break;
    }
}

// double -> bf16 bits, round to nearest even (one rounding to 8 significant bits)
uint16_t bf16_of(double v) {
    int k;
    const double m = std::frexp(v, &k);
    const double r = std::ldexp(std::rint(std::ldexp(m, 8)), k - 8);
    const float f = (float)r;
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

void codebook(int bits, uint16_t* lev) {
    double y[16];
    lloyd_max(1 << bits, y);
    for (int i = 0; i < (1 << bits); ++i) lev[i] = bf16_of(y[i]);
}

float bf16_value(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

struct RowsArgs {
    const void* x;
    int Ci, Kp;
    const int* perm;
    float mids[16];          // midpoints of neighbouring levels (exact in fp32), +inf past the last
    uint16_t lev[16];        // bf16 levels
    uint8_t* codes;          // [rows_pad][Kp/2]
    float* scale;            // [rows_pad]
    uint16_t* dec;           // off_bf16 layout
};

// Four radix-2 butterfly stages over 16 values (index bits 0-3, h = 1, 2, 4,
// 8 in that order): (v[i], v[i + h]) -> (v[i] + v[i + h], v[i] - v[i + h]).
__device__ __forceinline__ void butterfly16(float* v) {
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if ((i & h) == 0) {
                const float u = v[i], w = v[i + h];
                v[i] = u + w;
                v[i + h] = u - w;
            }
}

// One workgroup (4 waves) per row.
//  1. The row is copied into LDS (16 bytes per lane).
//  2. Rotation, per 256-channel block b: element i = 16 a + g.  Pair (b, g)
//     (16 lanes of one wave per block) gathers channels 16 g .. 16 g + 15 by
//     the permutation and runs the stages on index bits 0-3 (h = 1 .. 8) in
//     registers; the same 16 lanes then take the columns (element 16 a + g,
//     a = 0 .. 15: bits 4-7, h = 16 .. 128) through LDS.  The block never
//     leaves its wave, whose LDS operations complete in order: no barrier.
//     The stages run in the order h = 1, 2, .., 128, then the exact 1/16.
//  3. The squares are summed per block in channel order (one lane per
//     block), then over the blocks in order; s = sqrt(sum / Ci), IEEE
//     division and correctly rounded square root.
//  4. Codes: v = fl32(x' / s) (IEEE division; 0 when s = 0), the count of
//     midpoints strictly below v by a branch-free binary search over the
//     16-entry table (+inf past the last midpoint), an exact tie to the even
//     index; 8 channels per thread and pass (one 4-byte code store, one
//     16-byte store of the decoded bf16 levels).
template <bool BF16X>
__global__ __launch_bounds__(256) void k_orbit_rows(RowsArgs a) {
    constexpr int ESZ = BF16X ? 2 : 4;
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
    __shared__ float tbl[16];
    __shared__ uint16_t lvl[16];
    __shared__ float part[MAX_CI / OBLOCK];
    __shared__ float srow;
    const int Ci = a.Ci, nb = Ci / OBLOCK;
    float* const rot = (float*)dyn;                    // [Ci] fp32
    uint8_t* const raw = dyn + 4 * (size_t)Ci;         // [Ci] input elements
    const long long r = blockIdx.x;
    const int t = threadIdx.x;
    if (t < 16) {
        tbl[t] = a.mids[t];
        lvl[t] = a.lev[t];
    }
    const uint8_t* xr = (const uint8_t*)a.x + r * (long long)Ci * ESZ;
    for (int o = 16 * t; o < Ci * ESZ; o += 4096) *(uint4*)(raw + o) = *(const uint4*)(xr + o);
    __syncthreads();

    for (int p = t; p < nb * 16; p += 256) {           // a block's 16 pairs: 16 lanes of one wave
        const int b = p >> 4, g = p & 15;
        float v[16];
        const int4* pp = (const int4*)(a.perm + 256 * b + 16 * g);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int4 c = pp[q];
            const int cs[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (BF16X) v[4 * q + e] = __uint_as_float((uint32_t)((const uint16_t*)raw)[cs[e]] << 16);
                else v[4 * q + e] = ((const float*)raw)[cs[e]];
            }
        }
        butterfly16(v);
        float4* rg = (float4*)(rot + 256 * b + 16 * g);
#pragma unroll
        for (int q = 0; q < 4; ++q) rg[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float* col = rot + 256 * b + g;
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = col[16 * i];
        butterfly16(v);
#pragma unroll
        for (int i = 0; i < 16; ++i) col[16 * i] = v[i] * 0.0625f;
    }
    __syncthreads();

    if (t < nb) {                                      // wave 0 (nb <= 60)
        // the block's 256 squares added in channel order (from +0, which
        // leaves the first square unchanged), 32 at a time, the next 32
        // channels' reads in flight meanwhile (one read at a time left each
        // read's latency in the chain)
        const float4* rb = (const float4*)(rot + 256 * t);
        float4 q[8], n[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = rb[i];
        float s2 = 0.0f;
#pragma unroll
        for (int b8 = 0; b8 < 8; ++b8) {
            if (b8 + 1 < 8) {
#pragma unroll
                for (int i = 0; i < 8; ++i) n[i] = rb[8 * (b8 + 1) + i];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                s2 = s2 + q[i].x * q[i].x;
                s2 = s2 + q[i].y * q[i].y;
                s2 = s2 + q[i].z * q[i].z;
                s2 = s2 + q[i].w * q[i].w;
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = n[i];
        }
        part[t] = s2;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (t == 0) {
        float tot = part[0];
        for (int j = 1; j < nb; ++j) tot = tot + part[j];
        const float sr = sqrtf(__fdiv_rn(tot, (float)Ci));   // correctly rounded (llvm.sqrt.f32), unlike __fsqrt_rn here
        srow = sr;
        a.scale[r] = sr;
    }
    __syncthreads();
    const float sr = srow;
    for (int c0 = 8 * t; c0 < Ci; c0 += 2048) {
        const float4 x0 = *(const float4*)(rot + c0), x1 = *(const float4*)(rot + c0 + 4);
        const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        uint32_t nib = 0;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = sr > 0.0f ? __fdiv_rn(xs[e], sr) : 0.0f;
            int idx = v > tbl[7] ? 8 : 0;
            idx += v > tbl[idx + 3] ? 4 : 0;
            idx += v > tbl[idx + 1] ? 2 : 0;
            idx += v > tbl[idx] ? 1 : 0;
            idx += (v == tbl[idx] && (idx & 1)) ? 1 : 0;          // exact tie: the even index
            nib |= (uint32_t)idx << (4 * e);
            const uint32_t l = lvl[idx];
            if (e & 1) w[e >> 1] |= l << 16;
            else w[e >> 1] = l;
        }
        *(uint32_t*)(a.codes + r * (a.Kp / 2) + c0 / 2) = nib;
        *(uint4*)((uint8_t*)a.dec + off_bf16(r, c0, a.Kp / 32)) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

hipError_t launch_rows(const void* x, int x_bf16, int64_t rows, int Ci, int Kp, const int* perm, const uint16_t* lev,
                       int nlev, uint8_t* codes, float* scale, uint16_t* dec, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    RowsArgs a{};
    a.x = x;
    a.Ci = Ci;
    a.Kp = Kp;
    a.perm = perm;
    for (int i = 0; i < 16; ++i) a.mids[i] = INFINITY;
    for (int i = 0; i < nlev; ++i) a.lev[i] = lev[i];
    for (int i = 0; i + 1 < nlev; ++i) a.mids[i] = 0.5f * (bf16_value(lev[i]) + bf16_value(lev[i + 1]));
    a.codes = codes;
    a.scale = scale;
    a.dec = dec;
    const size_t lds = (size_t)Ci * (4 + (x_bf16 ? 2 : 4));   // rotated row + the row as given (at most 120 KB)
    const void* fn = x_bf16 ? (const void*)k_orbit_rows<true> : (const void*)k_orbit_rows<false>;
    if (lds > 65536) {                                         // beyond the default dynamic LDS limit
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (x_bf16) k_orbit_rows<true><<<(unsigned)rows, 256, lds, st>>>(a);
    else k_orbit_rows<false><<<(unsigned)rows, 256, lds, st>>>(a);
    return hipGetLastError();
}

template <class T>
hipError_t zalloc(T** p, size_t count, size_t* total) {
    *p = nullptr;
    if (count == 0) return hipSuccess;
    hipError_t e = hipMalloc((void**)p, count * sizeof(T));
    if (e != hipSuccess) {
        *p = nullptr;
        return e;
    }
    *total += count * sizeof(T);
    return hipMemset(*p, 0, count * sizeof(T));
}

void free_orbit(dq_orbit* o) {
    if (!o) return;
    DeviceGuard dg(o->device);
    (void)hipFree(o->perm);
    (void)hipFree(o->wdec);
    (void)hipFree(o->wcodes);
    (void)hipFree(o->wscale);
    delete o;
}

void free_orbit_act(dq_orbit_act* a) {
    if (!a) return;
    DeviceGuard dg(a->device);
    (void)hipFree(a->xdec);
    (void)hipFree(a->xcodes);
    (void)hipFree(a->xscale);
    (void)hipFree(a->rows);
    (void)hipFree(a->sink);
    delete a;
}

}  // namespace
}  // namespace dq

using namespace dq;

extern "C" {

dq_status dq_orbit_prepare(const void* w_host, dq_dtype dt, int64_t Ci, int64_t Co, const int32_t* perm_host,
                           int32_t wbits, int32_t abits, int32_t device, dq_orbit** out) {
    set_error("");
    if (!out) return fail(DQ_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!w_host || !perm_host) return fail(DQ_ERR_INVALID_ARG, "w_host or perm_host is NULL");
    if (dt != DQ_F32 && dt != DQ_BF16) return fail(DQ_ERR_INVALID_ARG, "unknown dtype");
    if (Ci < OBLOCK || Ci % OBLOCK != 0 || Ci > MAX_CI) return fail(DQ_ERR_SHAPE, "Ci must be a multiple of 256, at most 15360");
    if (Co < 1 || Co > (1 << 24)) return fail(DQ_ERR_SHAPE, "Co must be in [1, 2^24]");
    if (wbits < 2 || wbits > 4 || abits < 2 || abits > 4) return fail(DQ_ERR_INVALID_ARG, "wbits and abits must be 2, 3 or 4");
    {   // a permutation of 0 .. Ci - 1 (the kernels index rows with it)
        std::vector<char> seen((size_t)Ci, 0);
        for (int64_t c = 0; c < Ci; ++c) {
            const int32_t v = perm_host[c];
            if (v < 0 || v >= Ci || seen[(size_t)v]) return fail(DQ_ERR_INVALID_ARG, "perm is not a permutation of 0 .. Ci - 1");
            seen[(size_t)v] = 1;
        }
    }
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return fail(DQ_ERR_DEVICE, "no HIP device available");
    if (device < 0 || device >= n) return fail(DQ_ERR_INVALID_ARG, "device index out of range");
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return fail(DQ_ERR_DEVICE, "hipGetDeviceProperties failed");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return fail(DQ_ERR_UNSUPPORTED, "gfx950 required");
    DeviceGuard dg(device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");
    auto* o = new (std::nothrow) dq_orbit();
    if (!o) return fail(DQ_ERR_OUT_OF_MEMORY, "host allocation failed");
    std::unique_ptr<dq_orbit, void (*)(dq_orbit*)> guard(o, free_orbit);
    o->device = device;
    o->Ci = Ci;
    o->Co = Co;
    o->Kp = round_up(Ci, KPAD);
    o->Cop = round_up(Co, NPAD);
    o->wbits = wbits;
    o->abits = abits;
    codebook(wbits, o->wlev);
    codebook(abits, o->alev);
    const size_t esz = dt == DQ_BF16 ? 2 : 4;
    void* wd = nullptr;
    hipError_t e;
    if ((e = zalloc(&o->perm, (size_t)Ci, &o->bytes)) != hipSuccess ||
        (e = zalloc(&o->wdec, (size_t)(o->Cop * o->Kp), &o->bytes)) != hipSuccess ||
        (e = zalloc(&o->wcodes, (size_t)(o->Cop * o->Kp / 2), &o->bytes)) != hipSuccess ||
        (e = zalloc(&o->wscale, (size_t)o->Cop, &o->bytes)) != hipSuccess)
        return hip_fail(e, "hipMalloc weight");
    if ((e = hipMemcpy(o->perm, perm_host, (size_t)Ci * 4, hipMemcpyHostToDevice)) != hipSuccess) return hip_fail(e, "copy perm");
    if ((e = hipMalloc(&wd, (size_t)(Ci * Co) * esz)) != hipSuccess) return hip_fail(e, "hipMalloc W");
    if ((e = hipMemcpy(wd, w_host, (size_t)(Ci * Co) * esz, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = launch_rows(wd, dt == DQ_BF16, Co, (int)Ci, (int)o->Kp, o->perm, o->wlev, 1 << wbits, o->wcodes, o->wscale,
                         o->wdec, nullptr)) != hipSuccess ||
        (e = hipDeviceSynchronize()) != hipSuccess) {
        (void)hipFree(wd);
        return hip_fail(e, "weight rotation");
    }
    (void)hipFree(wd);
    *out = guard.release();
    return DQ_OK;
}

void dq_orbit_destroy(dq_orbit* o) { free_orbit(o); }

dq_status dq_orbit_export(const dq_orbit* o, uint16_t* wlev_host, uint16_t* alev_host, uint8_t* wcodes_host,
                          float* wscale_host) {
    set_error("");
    if (!o) return fail(DQ_ERR_INVALID_ARG, "weight handle is NULL");
    if (wlev_host) std::memcpy(wlev_host, o->wlev, (size_t)(2 << o->wbits));
    if (alev_host) std::memcpy(alev_host, o->alev, (size_t)(2 << o->abits));
    DeviceGuard dg(o->device);
    hipError_t e;
    if (wcodes_host) {
        std::vector<uint8_t> buf((size_t)(o->Cop * o->Kp / 2));
        if ((e = hipMemcpy(buf.data(), o->wcodes, buf.size(), hipMemcpyDeviceToHost)) != hipSuccess) return hip_fail(e, "copy codes");
        for (int64_t j = 0; j < o->Co; ++j) std::memcpy(wcodes_host + j * (o->Ci / 2), &buf[(size_t)(j * (o->Kp / 2))], (size_t)(o->Ci / 2));
    }
    if (wscale_host && (e = hipMemcpy(wscale_host, o->wscale, (size_t)o->Co * 4, hipMemcpyDeviceToHost)) != hipSuccess)
        return hip_fail(e, "copy scales");
    return DQ_OK;
}

dq_status dq_orbit_act_create(const dq_orbit* o, int64_t N, dq_orbit_act** out) {
    set_error("");
    if (!out) return fail(DQ_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!o) return fail(DQ_ERR_INVALID_ARG, "weight handle is NULL");
    if (N < 1 || N > (int64_t(1) << 31) - MPAD) return fail(DQ_ERR_SHAPE, "N must be in [1, 2^31 - 256]");
    if (N * o->Co >= (int64_t(1) << 40)) return fail(DQ_ERR_SHAPE, "workspace too large");
    DeviceGuard dg(o->device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");
    auto* a = new (std::nothrow) dq_orbit_act();
    if (!a) return fail(DQ_ERR_OUT_OF_MEMORY, "host allocation failed");
    std::unique_ptr<dq_orbit_act, void (*)(dq_orbit_act*)> guard(a, free_orbit_act);
    a->device = o->device;
    a->N = N;
    a->N_pad = round_up(N, MPAD);
    a->Ci = o->Ci;
    a->Kp = o->Kp;
    hipError_t e;
    if ((e = zalloc(&a->xdec, (size_t)(a->N_pad * a->Kp), &a->bytes)) != hipSuccess ||
        (e = zalloc(&a->xcodes, (size_t)(a->N_pad * a->Kp / 2), &a->bytes)) != hipSuccess ||
        (e = zalloc(&a->xscale, (size_t)a->N_pad, &a->bytes)) != hipSuccess ||
        (e = zalloc(&a->rows, (size_t)a->N_pad, &a->bytes)) != hipSuccess ||
        (e = zalloc(&a->sink, (size_t)512, &a->bytes)) != hipSuccess)
        return hip_fail(e, "hipMalloc workspace");
    const Geom g{1, 1, (int)N, 1, 1, 1, 1, 1, (int)N, 1, (long long)N, (long long)N, (long long)N};
    if ((e = launch_slot_tokens(g, 0, a->rows, a->N_pad, nullptr)) != hipSuccess) return hip_fail(e, "row table");
    if ((e = hipDeviceSynchronize()) != hipSuccess) return hip_fail(e, "workspace init");
    *out = guard.release();
    return DQ_OK;
}

void dq_orbit_act_destroy(dq_orbit_act* a) { free_orbit_act(a); }

static dq_status orbit_pair(const dq_orbit* o, const dq_orbit_act* a) {
    if (!o) return fail(DQ_ERR_INVALID_ARG, "weight handle is NULL");
    if (!a) return fail(DQ_ERR_INVALID_ARG, "workspace handle is NULL");
    if (a->Ci != o->Ci || a->device != o->device) return fail(DQ_ERR_INVALID_ARG, "workspace was created for a different weight");
    return DQ_OK;
}

dq_status dq_orbit_quantize_act(const dq_orbit* o, const void* x_dev, dq_dtype dt, dq_orbit_act* a, void* stream) {
    set_error("");
    dq_status st = orbit_pair(o, a);
    if (st != DQ_OK) return st;
    if (!x_dev) return fail(DQ_ERR_INVALID_ARG, "x_dev is NULL");
    if (((uintptr_t)x_dev) % 16 != 0) return fail(DQ_ERR_INVALID_ARG, "x_dev must be 16-byte aligned");
    if (dt != DQ_F32 && dt != DQ_BF16) return fail(DQ_ERR_INVALID_ARG, "unknown dtype");
    DeviceGuard dg(a->device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");
    hipError_t e = launch_rows(x_dev, dt == DQ_BF16, a->N, (int)a->Ci, (int)a->Kp, o->perm, o->alev, 1 << o->abits,
                               a->xcodes, a->xscale, a->xdec, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "rotation launch");
    return DQ_OK;
}

dq_status dq_orbit_forward(const dq_orbit* o, dq_orbit_act* a, float* y_dev, void* stream) {
    set_error("");
    dq_status st = orbit_pair(o, a);
    if (st != DQ_OK) return st;
    if (!y_dev) return fail(DQ_ERR_INVALID_ARG, "y_dev is NULL");
    if (((uintptr_t)y_dev) % 4 != 0) return fail(DQ_ERR_INVALID_ARG, "y_dev must be 4-byte aligned");
    DeviceGuard dg(a->device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");
    hipError_t e = launch_orbit_gemm(o->wdec, a->xdec, o->Kp, o->Cop, a->N_pad, o->Co, a->rows, a->xscale, o->wscale, y_dev,
                                     a->sink, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "GEMM launch");
    return DQ_OK;
}

dq_status dq_orbit_linear(const dq_orbit* o, const void* x_dev, dq_dtype dt, dq_orbit_act* a, float* y_dev, void* stream) {
    dq_status st = dq_orbit_quantize_act(o, x_dev, dt, a, stream);
    if (st != DQ_OK) return st;
    return dq_orbit_forward(o, a, y_dev, stream);
}

dq_status dq_orbit_act_export(const dq_orbit_act* a, uint8_t* codes_host, float* scale_host, void* stream) {
    set_error("");
    if (!a) return fail(DQ_ERR_INVALID_ARG, "workspace handle is NULL");
    DeviceGuard dg(a->device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "stream synchronize");
    try {
        if (codes_host) {
            std::vector<uint8_t> buf((size_t)(a->N_pad * a->Kp / 2));
            if ((e = hipMemcpy(buf.data(), a->xcodes, buf.size(), hipMemcpyDeviceToHost)) != hipSuccess) return hip_fail(e, "copy codes");
            for (int64_t n = 0; n < a->N; ++n) std::memcpy(codes_host + n * (a->Ci / 2), &buf[(size_t)(n * (a->Kp / 2))], (size_t)(a->Ci / 2));
        }
        if (scale_host && (e = hipMemcpy(scale_host, a->xscale, (size_t)a->N * 4, hipMemcpyDeviceToHost)) != hipSuccess)
            return hip_fail(e, "copy scales");
    } catch (const std::bad_alloc&) {
        return fail(DQ_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    return DQ_OK;
}

}  // extern "C"
