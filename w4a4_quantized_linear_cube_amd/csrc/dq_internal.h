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

// Token grid and cube shape, with derived counts, as kernels see them.
struct Geom {
    int T, H, W, t, h, w;
    int Tc, Hc, Wc, S;
    long long N, K, Nslot;
};

}  // namespace dq

struct dq_weights {
    int device = 0;
    int64_t Ci = 0, Co = 0, Kp = 0, Cop = 0;
    int rank = 0, rp = 0;
    uint8_t* rq = nullptr;     // Cop x Kp/2    Q4(R) codes, step-major (device)
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
    uint16_t* cbf = nullptr;   // [K_pad][Kp]        bf16 cores (core_bits 16)
    uint16_t* rbf = nullptr;   // [Cop][Kp]          Q4(R) decoded to bf16 (core_bits 16)
    void* blas = nullptr;      // rocBLAS handle of the bf16 core GEMM (core_bits 16)
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
    size_t bytes = 0;
};

namespace dq {

void set_error(const std::string& msg);

// ---- launchers (quant.hip) ----
hipError_t launch_residual(const void* w_dev, int w_bf16, const uint16_t* l1_dev, const uint16_t* l2_dev,
                           int64_t Ci, int64_t Co, int rank, float* r_dev, hipStream_t st);
hipError_t launch_encode_fp4_rows(const float* src, int64_t rows, int64_t cols, int64_t ld_src, int64_t Kp,
                                  uint8_t* codes, uint8_t* scales, hipStream_t st);
hipError_t launch_quantize(const dq_weights* w, const void* x, int x_bf16, dq_qact* q, hipStream_t st);
hipError_t launch_slot_tokens(const Geom& g, int64_t tok0, int* stok, int64_t n, hipStream_t st);
hipError_t launch_decode_fp4_bf16(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t Kp, uint16_t* out,
                                  hipStream_t st);

// ---- launchers (gemm.hip) ----
constexpr int FWD_CORE = 1, FWD_DELTA = 2;   // parts of the forward pass
hipError_t launch_forward(const dq_weights* w, dq_qact* q, float* y, int parts, hipStream_t st);

}  // namespace dq
