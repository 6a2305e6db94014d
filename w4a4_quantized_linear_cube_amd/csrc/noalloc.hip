// dq_linear_noalloc: the whole layer (activation pass, core term, delta
// term) with the activation workspace carved from a fixed device array
// instead of memory allocated by dq_qact_create, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The kernels are those of dq_linear.
//
// The array `scratch` is a file-scope device variable: each GPU the library
// runs on holds its own copy (NOALLOC_SCRATCH_BYTES) until the process ends.
// In host code its name is only a host-side stand-in, so every host use goes
// through the device address that hipGetSymbolAddress returns for the current
// device, taken once per device at the first call there and kept in g_scratch.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "dq.h"
#include "dq_internal.h"

static __device__ __align__(256) uint8_t scratch[dq::NOALLOC_SCRATCH_BYTES];

namespace dq {
namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
uint8_t* g_scratch[MAX_DEVICES];      // device address of `scratch` on each device, null until set up

// p[0 .. n16) = 0 (16-byte units): clears with a kernel rather than a memset
// node, which graph capture handles reliably.
__global__ __launch_bounds__(256) void k_zero16(uint4* p, long long n16) {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n16; i += (long long)gridDim.x * 256)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t zero_bytes(void* p, size_t bytes, hipStream_t st) {
    const long long n16 = (long long)(bytes / 16);
    if (n16 == 0) return hipSuccess;
    const unsigned blocks = (unsigned)std::min<long long>((n16 + 255) / 256, 4096);
    k_zero16<<<blocks, 256, 0, st>>>((uint4*)p, n16);
    return hipGetLastError();
}

// The current device's copy of `scratch` (set up on first use: its address,
// and its zero page cleared on `st`).
dq_status scratch_of(int dev, hipStream_t st, uint8_t** out) {
    if (dev < 0 || dev >= MAX_DEVICES) return fail(DQ_ERR_UNSUPPORTED, "device index beyond the scratch table");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if ((e = zero_bytes(p, 512, st)) != hipSuccess) return hip_fail(e, "scratch zero page");
        g_scratch[dev] = (uint8_t*)p;
    }
    *out = g_scratch[dev];
    return DQ_OK;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace
}  // namespace dq

using namespace dq;

extern "C" dq_status dq_linear_noalloc(const dq_weights* w, const void* x_dev, dq_dtype dt, dq_geom geom,
                                       float* y_dev, void* stream) {
    set_error("");
    if (!w) return fail(DQ_ERR_INVALID_ARG, "weights handle is NULL");
    if (!x_dev || !y_dev) return fail(DQ_ERR_INVALID_ARG, "x_dev or y_dev is NULL");
    if (((uintptr_t)x_dev) % 16 != 0) return fail(DQ_ERR_INVALID_ARG, "x_dev must be 16-byte aligned");
    if (((uintptr_t)y_dev) % 4 != 0) return fail(DQ_ERR_INVALID_ARG, "y_dev must be 4-byte aligned");
    if (dt != DQ_F32 && dt != DQ_BF16) return fail(DQ_ERR_INVALID_ARG, "unknown dtype");
    // the workspace lives on the host stack; its buffers in the scratch array
    dq_qact q{};
    int64_t max_partials = 0;
    dq_status st = plan_qact(w, geom, 32, 8, &q, &max_partials);
    if (st != DQ_OK) return st;
    // layout: zero page, sink, codes and scales (cleared below when Ci is
    // not a multiple of 128), U, per-cube term, slot table, fp32 cores and
    // block partials (cubes of more than 64 tokens), the core GEMM's K-chunk
    // partials and the activation pass's U partials (the same splits as
    // dq_qact_create's, so the same results)
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    const size_t o_zero = take(512), o_sink = take(2048);
    const size_t o_dq = take((size_t)(q.Nslot_pad * q.Kp / 2)), o_ds = take((size_t)(q.Nslot_pad * q.Kp / 32));
    const size_t o_cq = take((size_t)(q.K_pad * q.Kp)), o_cs = take((size_t)(q.K_pad * q.Kp / 32));
    const size_t codes_end = off;
    const size_t o_u = take((size_t)(q.Nslot_pad * q.rp * 2));
    const size_t o_bias = take((size_t)(q.K_pad * q.Cop * 4));
    const size_t o_stok = take((size_t)(q.Nslot_pad * 4));
    const size_t o_coref = max_partials ? take((size_t)(q.K_pad * q.Kp * 4)) : 0;
    const size_t o_part = max_partials ? take((size_t)(max_partials * q.Kp * 4)) : 0;
    const size_t o_kpart = q.ks.rm ? take(q.ks.part_bytes()) : 0;
    const bool upart = q.upart_rows > 0 && q.rp > 0;
    const size_t o_upart = upart ? take((size_t)(QMAXPARTS * q.upart_rows * q.rp * 4)) : 0;
    if (off > NOALLOC_SCRATCH_BYTES)
        return fail(DQ_ERR_SHAPE, "this layer needs " + std::to_string(off) + " bytes of scratch; the static scratch of "
                                  "dq_linear_noalloc holds " + std::to_string(NOALLOC_SCRATCH_BYTES));
    DeviceGuard dg(w->device);
    if (!dg.ok) return fail(DQ_ERR_DEVICE, "hipSetDevice failed");
    hipStream_t s = (hipStream_t)stream;
    uint8_t* base = nullptr;
    if ((st = scratch_of(w->device, s, &base)) != DQ_OK) return st;
    q.zero = base + o_zero;
    q.sink = (float*)(base + o_sink);
    q.dq = base + o_dq;
    q.ds = base + o_ds;
    q.cq = base + o_cq;
    q.cs = base + o_cs;
    q.u = (uint16_t*)(base + o_u);
    q.bias = (float*)(base + o_bias);
    q.stok = (int*)(base + o_stok);
    q.coref = max_partials ? (float*)(base + o_coref) : nullptr;
    q.part = max_partials ? (float*)(base + o_part) : nullptr;
    q.kpart = q.ks.rm ? (float*)(base + o_kpart) : nullptr;
    q.upart = upart ? (float*)(base + o_upart) : nullptr;
    hipError_t e;
    // The activation pass writes every code and scale of channels below Ci;
    // the padding channels up to Kp must hold zero codes and scale codes
    // (the array keeps the last call's bytes, which could decode as NaN).
    if (q.Kp != q.Ci && (e = zero_bytes(base + o_dq, codes_end - o_dq, s)) != hipSuccess)
        return hip_fail(e, "clearing the code buffers");
    for (int i = 0; i < q.nseg; ++i) {
        const dq_segment& sg = q.seg[i];
        const int64_t rows = (i + 1 < q.nseg ? q.seg[i + 1].row0 : q.Nslot_pad) - sg.row0;
        if ((e = launch_slot_tokens(sg.g, sg.tok0, q.stok + sg.row0, rows, s)) != hipSuccess)
            return hip_fail(e, "slot table");
    }
    if ((e = launch_quantize(w, x_dev, dt == DQ_BF16, &q, s)) != hipSuccess) return hip_fail(e, "activation pass launch");
    if ((e = launch_forward(w, &q, y_dev, FWD_CORE | FWD_DELTA, s)) != hipSuccess) return hip_fail(e, "forward launch");
    return DQ_OK;
}
