// Internal declarations of the delta-W4A4 library: handle layouts, kernel
// argument blocks and the host-side launchers implemented in the .hip files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "dq.h"

namespace dq {

// Padding of the internal buffers.  Channel dimensions of code/scale rows are
// padded to KPAD so the GEMM's 128-wide K steps never leave a row, and row
// counts to MPAD / NPAD so its 256 x 256 tiles never leave a buffer; padding
// holds zero codes with zero scale codes, which contribute exactly 0.
constexpr int KPAD = 128;
constexpr int MPAD = 256;
constexpr int NPAD = 256;
constexpr int RPAD = 32;      // low-rank width padded for 32x32 bf16 MFMA tiles
constexpr int CORE_BLOCK = 64;  // tokens per fp32 partial sum of a cube's core
// Size of the per-device array that dq_linear_noalloc carves its activation
// workspace from (128 MiB: the Wan 1.3B projection, 32 760 tokens of
// 1536 channels in 4-token cubes, needs about 92 MB).
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(128) << 20;

inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Operand layout of the GEMMs.  A code (or scale) matrix of rows x Kp
// channels, rows a multiple of 256 and Kp of 128, is stored step-major:
// [row / 256][Kp / 128][row % 256][bytes of one row's 128-channel step], so
// one GEMM tile's K step (256 rows x 128 channels) is a single contiguous
// block that the GEMM copies into LDS unchanged.  Inside a row's step the
// 16-byte chunks are XOR-swizzled by the row, which makes the GEMM's
// fragment reads from LDS free of bank conflicts:
//   FP4 codes:  64 bytes per row step, chunk c (channels 32c .. 32c + 31,
//               element 2i in the low nibble of byte i) at (c ^ swz4(row));
//   FP8 codes: 128 bytes per row step, chunk c (channels 16c .. 16c + 15)
//               at (c ^ swz8(row));
//   E8M0 scale codes: one byte per row and 32-channel group, 1 KB per
//               tile step, in the order given at off_scale.
__host__ __device__ inline int swz4(int r) { return ((r >> 1) ^ ((r >> 3) & 1)) & 3; }
__host__ __device__ inline int swz8(int r) { return (r ^ ((r >> 3) & 1)) & 7; }
// Offsets inside one tile step-block sequence: row r < 256 of its tile,
// 32-bit (a tile of the largest operands spans well under 4 GB).
// byte offset of FP4 group G (32 channels, 16 bytes) of tile row r
__host__ __device__ inline uint32_t toff_fp4(int r, int G) {
    return ((uint32_t)(G >> 2) * 256 + (uint32_t)r) * 64 + (uint32_t)(((G & 3) ^ swz4(r)) << 4);
}
// byte offset of 16-byte chunk c (channels 16c .. 16c + 15 of K step ks) of FP8 tile row r
__host__ __device__ inline uint32_t toff_fp8(int r, int ks, int c) {
    return ((uint32_t)ks * 256 + (uint32_t)r) * 128 + (uint32_t)((c ^ swz8(r)) << 4);
}
// byte offset of the scale code of group G of tile row r.  A step's scale
// block (256 rows x 4 groups, 1 KB) is ordered [row / 128][G % 2][row % 32]
// [(row % 128) / 32][(G % 4) / 2], so the 8 codes one GEMM lane needs in a K
// step (its four 32-row blocks x its two groups) are 8 consecutive bytes.
__host__ __device__ inline uint32_t toff_scale(int r, int G) {
    return (uint32_t)(G >> 2) * 1024 + (uint32_t)((((r >> 7) * 2 + (G & 1)) * 32 + (r & 31)) * 8 + ((r >> 5) & 3) * 2 + ((G & 3) >> 1));
}
// FP6 codes (the 6-bit layers): 96 bytes per row step, four 32-channel
// groups of 24 bytes (channel i of a group at bits [6 i, 6 i + 6),
// little-endian), i.e. twelve 8-byte words, group G holding words
// 3 (G % 4) .. 3 (G % 4) + 2.  The words are rotated by the row's octet:
// word w sits at position (w + rot6(r)) % 12, so the 32 lanes of a GEMM
// fragment read (rows r0 .. r0 + 31, one word each) hit 64 distinct banks.
__host__ __device__ inline int rot6(int r) { return (r >> 3) & 3; }
// byte offset of word i (0 .. 2) of group G of tile row r
__host__ __device__ inline uint32_t toff_fp6(int r, int G, int i) {
    return ((uint32_t)(G >> 2) * 256 + (uint32_t)r) * 96 + (uint32_t)(((3 * (G & 3) + i + rot6(r)) % 12) * 8);
}
// the same for any row of a matrix of nks K steps
__host__ __device__ inline size_t off_fp6(long long row, long long G, int i, long long nks) {
    return (size_t)(row >> 8) * (size_t)nks * 24576 + toff_fp6((int)(row & 255), (int)G, i);
}
// the same for any row of a matrix of nks K steps
__host__ __device__ inline size_t off_fp4(long long row, long long G, long long nks) {
    return (size_t)(row >> 8) * (size_t)nks * 16384 + toff_fp4((int)(row & 255), (int)G);
}
__host__ __device__ inline size_t off_fp8(long long row, long long ks, int c, long long nks) {
    return (size_t)(row >> 8) * (size_t)nks * 32768 + toff_fp8((int)(row & 255), (int)ks, c);
}
__host__ __device__ inline size_t off_scale(long long row, long long G, long long nks) {
    return (size_t)(row >> 8) * (size_t)nks * 1024 + toff_scale((int)(row & 255), (int)G);
}

// bf16 operands of the bf16 GEMM (the 16-bit cores and Q4(R) decoded to
// bf16): 32 channels (64 bytes) per row step, laid out like the FP4 codes
// (16-byte chunk c, channels 8 c .. 8 c + 7 of the step, at chunk c ^ swz4(r)),
// so a 32x32x16 bf16 MFMA fragment is one chunk, read like an FP4 one.
// Byte offset of channel ch of row `row` in a matrix of nks32 = Kp / 32 steps.
__host__ __device__ inline size_t off_bf16(long long row, long long ch, long long nks32) {
    const int r = (int)(row & 255);
    const int c = (int)((ch >> 3) & 3);
    return (size_t)(row >> 8) * (size_t)nks32 * 16384 + ((size_t)(ch >> 5) * 256 + (size_t)r) * 64 +
           (size_t)((c ^ swz4(r)) << 4) + (size_t)(ch & 7) * 2;
}

// Token grid and cube shape, with derived counts, as kernels see them.
struct Geom {
    int T, H, W, t, h, w;
    int Tc, Hc, Wc, S;
    long long N, K, Nslot;
};

// K split of a plain-store GEMM's last, partly filled round.  The persistent
// GEMM runs its tiles in rounds of one tile per workgroup; when the tile
// count is not a multiple of the grid, the last round leaves most CUs idle
// for a whole tile.  Instead, one launch runs the full rounds (walk tiles
// 0 .. main_tiles - 1), a second runs the rm remaining tiles (walk tiles
// main_tiles ..) as rm x p units, unit u taking K chunk u / rm of tile
// u % rm into its own 256 x 256 fp32 partial, and a third sums each tile's
// p partials in chunk order into the output.  rm == 0: one launch.
struct KSplit {
    int main_tiles = 0, rm = 0, p = 1;
    size_t part_bytes() const { return (size_t)rm * (size_t)p * 65536 * 4; }
};
// Channel split of an activation-pass segment with few blocks (a frame
// segment of a clipped last frame group: a few dozen blocks of up to 108
// chunks each would keep most CUs idle): the largest part count up to
// QMAXPARTS that divides its nchunks chunks, leaves at least 4 chunks per
// part and keeps nblocks x parts within the CUs; 1 (no split) when the
// blocks fill more than half of the CUs.
constexpr int QMAXPARTS = 8;
inline int quant_kparts(long long nblocks, int nchunks, int cus) {
    if (nblocks * 2 > cus) return 1;
    int best = 1;
    for (int p = 2; p <= QMAXPARTS; ++p)
        if (nchunks % p == 0 && nchunks / p >= 4 && nblocks * p <= cus) best = p;
    return best;
}

// The split of an mt x nt tile GEMM with nks K steps of about step_us each
// (per tile, with every CU busy) on `cus` CUs, ring depth ns: the chunk count
// that saves the most time (each chunk at least ns steps), or none.
KSplit plan_ksplit(int mt, int nt, int nks, int ns, int cus, double step_us);

}  // namespace dq

struct dq_weights {
    int device = 0;
    int64_t Ci = 0, Co = 0, Kp = 0, Cop = 0;
    int rank = 0, rp = 0;
    int wfmt = 4;              // R's codes: MX-FP4 (4), or MX-FP6 E2M3 (2) / E3M2 (3) for the 6-bit layers
    uint8_t* rq = nullptr;     // Cop x Kp/2    Q4(R) codes (Cop x 3 Kp/4 for Q6(R)), step-major (device)
    uint8_t* rs = nullptr;     // Cop x Kp/32   Q4(R) scale codes, step-major (device)
    float* r = nullptr;        // [Co][Ci]      fp32 residual R^T (device, for export)
    uint16_t* l1t = nullptr;   // [rp][Kp]      L1^T bf16 (device)
    uint16_t* l2t = nullptr;   // [Cop][rp]     L2^T bf16 (device)
    std::vector<uint16_t> l1, l2;   // host copies [Ci][rank], [rank][Co]
    size_t bytes = 0;
};

// Frame segments.  Frames are the slowest token axis, so when t does not
// divide T the clipped cubes of the last frame group form a regular grid of
// their own: frames [0, T - T % t) with t x h x w cubes and the last T % t
// frames with (T % t) x h x w cubes.  The two segments hold the same cubes,
// tokens and slot order within each cube as the full grid, but the second
// needs no pad slots for the missing frames.  Segment i's slot rows start at
// row0, its cube rows (core codes, per-cube term) at krow0, both multiples of
// 256 (GEMM tiles); its tokens are tok0 + its own token numbers, its cubes
// k0 + its own cube numbers.
struct dq_segment {
    dq::Geom g{};
    int64_t tok0 = 0, k0 = 0, row0 = 0, krow0 = 0;
    int core_mode = 0;         // 0: cores inside the activation pass (S <= 64); 1: separate passes
    int64_t nblk = 0;          // 64-token blocks per cube (core_mode 1)
};

struct dq_qact {
    int device = 0;
    int64_t Ci = 0, Co = 0, Kp = 0, Cop = 0;
    int rp = 0, rank = 0;
    dq::Geom g{};              // the full token grid and cube shape
    int core_group = 32;       // channels per exponent of the cores (32 or 64)
    int core_bits = 8;         // cores as MX-FP8 (8), MX-FP4 (4, the FP4 layout in cq) or bf16 (16, in cbf)
    uint16_t* cbf = nullptr;   // K_pad x Kp         bf16 cores, step-major (off_bf16) (core_bits 16)
    uint16_t* rbf = nullptr;   // Cop x Kp           Q4(R) decoded to bf16, step-major (off_bf16) (core_bits 16)
    int nseg = 1;
    dq_segment seg[2]{};
    int64_t Nslot_pad = 0, K_pad = 0;
    uint8_t* dq = nullptr;     // Nslot_pad x Kp/2   delta codes, slot order, step-major
    uint8_t* ds = nullptr;     // Nslot_pad x Kp/32  delta scale codes, step-major
    uint8_t* cq = nullptr;     // K_pad x Kp         core FP8 codes, step-major
    uint8_t* cs = nullptr;     // K_pad x Kp/32      core scale codes, step-major
    uint16_t* u = nullptr;     // [Nslot_pad][rp]    U = bf16(bf16(X) L1), slot order
    float* bias = nullptr;     // [K_pad][Cop]       per-cube core term Q8(core) Q4(R)
    int* stok = nullptr;       // [Nslot_pad]        token of each slot, -1 for pad slots
    uint8_t* zero = nullptr;   // [512]              zero bytes (copy source of absent rows)
    float* sink = nullptr;     // [512]              target of the GEMM's discarded 16-byte stores
    float* coref = nullptr;    // [K_pad][Kp]        fp32 cores (segments of core_mode 1), cube rows
    float* part = nullptr;     // [K*nblk][Kp]       fp32 block partials (core_mode 1; the segments take turns)
    int64_t upart_rows = 0;    // largest slot count of a segment the activation pass may split by channels
    float* upart = nullptr;    // [QMAXPARTS][upart_rows][rp] fp32 U partials of such a segment (upart_rows > 0, rp > 0)
    dq::KSplit ks{};           // K split of the core GEMM's last round (set by plan_qact)
    int cus = 256;             // compute units of the device (set by plan_qact)
    float* kpart = nullptr;    // [ks.rm * ks.p][256][256] fp32 K-chunk partials of that round (ks.rm > 0)
    size_t bytes = 0;
};

// Workspace of a 6-bit layer: N text tokens (no cubes).
struct dq_act6 {
    int device = 0;
    int64_t N = 0, N_pad = 0, Ci = 0, Co = 0, Kp = 0, Cop = 0;
    int rp = 0, rank = 0, wfmt = 2;
    uint8_t* xq = nullptr;     // N_pad x 3 Kp/4   Q6(X) codes, step-major
    uint8_t* xs = nullptr;     // N_pad x Kp/32    scale codes, step-major
    uint16_t* u = nullptr;     // [N_pad][rp]      U = bf16(bf16(X) L1)
    float* upart = nullptr;    // [splits][N_pad][rp] partial sums of U
    int* stok = nullptr;       // [N_pad]          row -> token (identity, -1 past N)
    float* sink = nullptr;     // [512]            target of the GEMM's discarded stores
    size_t bytes = 0;
};

namespace dq {

void set_error(const std::string& msg);
// Record `msg` as the thread's last error and return `s`; the HIP flavour
// maps hipErrorOutOfMemory to DQ_ERR_OUT_OF_MEMORY, the rest to DQ_ERR_DEVICE.
dq_status fail(dq_status s, const std::string& msg);
dq_status hip_fail(hipError_t e, const char* what);
// Checks a geometry and the core options against a weight and fills the
// workspace's sizes, frame segments and the core GEMM's K split (no
// allocation, no device work);
// *max_partials is the row count of the block-partial buffer (0 if no
// segment has cubes of more than 64 tokens).
dq_status plan_qact(const dq_weights* w, const dq_geom& geom, int core_group, int core_bits, dq_qact* q,
                    int64_t* max_partials);

// Makes a handle's device current for the scope and restores the caller's.
struct DeviceGuard {
    int prev = -1;
    bool ok = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

// ---- launchers (quant.hip) ----
hipError_t launch_residual(const void* w_dev, int w_bf16, const uint16_t* l1_dev, const uint16_t* l2_dev,
                           int64_t Ci, int64_t Co, int rank, float* r_dev, hipStream_t st);
hipError_t launch_encode_fp4_rows(const float* src, int64_t rows, int64_t cols, int64_t ld_src, int64_t Kp,
                                  uint8_t* codes, uint8_t* scales, hipStream_t st);
hipError_t launch_quantize(const dq_weights* w, const void* x, int x_bf16, dq_qact* q, hipStream_t st);
hipError_t launch_slot_tokens(const Geom& g, int64_t tok0, int* stok, int64_t n, hipStream_t st);
hipError_t launch_decode_fp4_bf16(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t Kp, uint16_t* out,
                                  hipStream_t st);

// 6-bit layers: MX-FP6 encode of rows (src fp32, or bf16 when src_bf16) into
// the step-major FP6 layout; U of text tokens (part: text_lowrank_splits(Ci)
// x Npad x rp fp32).
hipError_t launch_encode_fp6(const void* src, int src_bf16, int64_t rows, int64_t cols, int64_t ld_src, int64_t Kp,
                             uint8_t* codes, uint8_t* scales, int e3m2, hipStream_t st);
hipError_t launch_text_lowrank(const void* x, int x_bf16, int64_t N, int64_t Npad, int Ci, int Kp, const uint16_t* l1t,
                               int rp, float* part, uint16_t* u, hipStream_t st);
int text_lowrank_splits(int Ci);

// ---- launchers (gemm.hip) ----
constexpr int FWD_CORE = 1, FWD_DELTA = 2;   // parts of the forward pass
hipError_t launch_forward(const dq_weights* w, dq_qact* q, float* y, int parts, hipStream_t st);
// The one-kernel forward (core and delta partial sums in one K loop) and the
// shapes it takes (4-slot cubes, FP8 cores, one frame segment, rank 32,
// Co % 256 == 0, Ci of 512 or more, y 16-byte aligned).
bool fused_applies(const dq_weights* w, const dq_qact* q, const float* y);
// ... and whether the whole forward takes it (small layers: at most 16 rounds of tiles)
bool fused_preferred(const dq_weights* w, const dq_qact* q, const float* y);
hipError_t launch_forward_fused(const dq_weights* w, dq_qact* q, float* y, hipStream_t st);
// y = U L2 + Q6(X) Q6(R) for a 6-bit layer
hipError_t launch_forward6(const dq_weights* w, dq_act6* a, float* y, hipStream_t st);
// y[n][j] = (sum_c wdec[j][c] xdec[n][c]) s_x[n] s_w[j] over bf16 operands in the off_bf16 layout
hipError_t launch_orbit_gemm(const uint16_t* wdec, const uint16_t* xdec, int64_t Kp, int64_t Cop, int64_t Npad, int64_t Co,
                             const int* rows, const float* xscale, const float* wscale, float* y, float* sink,
                             hipStream_t st);

}  // namespace dq
