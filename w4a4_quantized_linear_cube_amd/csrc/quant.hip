// Activation pass and weight preparation kernels (gfx950).
//
// Activation pass (DeltaQuant notes, 关键设计 2-4 and the implementation
// paragraph of 损失函数/训练策略, which fuses core generation into the
// activation quantizer):
//   core_k  = fl32( fp32 sum of cube k's tokens, lexicographic order / count )
//   delta_n = fl32( x_n - core_k(n) )
//   Q8(core), Q4(delta): MX, one E8M0 scale per 32 channels
//   U_n     = bf16( bf16(x_n) L1 )   (fp32 MFMA accumulation)
//
// The pass works on blocks of 64 slot rows (whole cubes when a cube has at
// most 64 tokens) and walks each block's channels in chunks: the chunk of X
// is staged in LDS once (channel-contiguous, coalesced row segments) and then
// used three times -- for the cube sums, for the deltas, and as the bf16 MFMA
// operand of U -- so X is read from HBM exactly once.  Cubes of more than 64
// tokens take two extra small passes (64-token partial sums, then their
// ordered combine) and X is read twice.
#include <algorithm>
#include <type_traits>

#include "dq_device.h"

namespace dq {

constexpr int QROWS = 64;                  // slot rows per block
constexpr int QROWB = 256;                 // bytes of one row's channel chunk in LDS
constexpr int QCHUNK = QROWS * QROWB;      // 16 KB
constexpr int QDMA = QCHUNK / 2 / 1024;    // 1 KB X copies per copy wave per chunk
constexpr int QKEEP = 4;                   // rows of a cube the quantizer keeps in registers

template <typename XT> struct XTraits;
template <> struct XTraits<float> {
    static constexpr int CC = QROWB / 4;   // 64 channels per chunk
    __device__ static float f(float v) { return v; }
};
template <> struct XTraits<uint16_t> {
    static constexpr int CC = QROWB / 2;   // 128 channels per chunk
    __device__ static float f(uint16_t v) { return bf16_to_f32(v); }
};

struct QuantArgs {
    const void* x;            // [N][Ci]
    Geom g;
    int Ci, Kp, rp;
    int core_mode;            // 0: cores computed here (S <= 64); 1: read from coref
    long long nblocks;        // 64-slot blocks
    uint8_t* dq;              // Nslot_pad x Kp/2, step-major
    uint8_t* ds;              // Nslot_pad x Kp/32, step-major
    uint8_t* cq;              // K_pad x Kp, step-major
    uint8_t* cs;              // K_pad x Kp/32, step-major
    uint16_t* u;              // [Nslot_pad][rp]
    const uint16_t* l1t;      // [rp][Kp], zero beyond Ci
    const float* coref;       // [K][Kp] (core_mode 1)
    const uint8_t* zero;      // 256 zero bytes (source of absent rows and channels)
    const int* stok;          // [Nslot_pad] token of each slot, -1 for pad slots
    int core_g64;             // cores: one exponent per 64 channels (the maximum of two 32-channel groups)
    int core_fp4;             // cores as MX-FP4 (the FP4 layout in cq) instead of MX-FP8
    uint16_t* cbf;            // bf16 cores, step-major (off_bf16) (16-bit cores), else null
    // Channel split of a segment with few blocks: block b's chunks are taken
    // by kparts workgroup blocks (nblocks counts those), part j taking the
    // j-th run of chunks; each part's U sum goes to upart[j][slot][rank]
    // (fp32, urows rows per part) for a later sum in part order.  kparts 1:
    // one part, U stored here as bf16.
    int kparts;
    long long urows;
    float* upart;
};

// bf16 bits of n consecutive core values (n = 2, 4, 8), packed for one store
__device__ __forceinline__ uint32_t bf16x2(float a, float b) { return (uint32_t)bf16_rne(a) | ((uint32_t)bf16_rne(b) << 16); }
// address of channel ch of cube row k of the bf16 cores (1, 2, 4 or 8
// channels aligned to their count are contiguous)
__device__ __forceinline__ uint16_t* cbf_at(uint16_t* cbf, long long k, long long ch, int Kp) {
    return (uint16_t*)((uint8_t*)cbf + off_bf16(k, ch, Kp / 32));
}

// LDS chunk layout: 16-byte piece c of row r at r QROWB + ((c ^ (r & 15)) << 4);
// the XOR makes the quantizer's row reads and the MFMA's column reads free of
// bank conflicts.
__device__ __forceinline__ int qoff(int r, int c) { return r * QROWB + ((c ^ (r & 15)) << 4); }

// Block b: its first slot, first cube, rows and cubes.  Cubes of at most 64
// tokens: whole cubes (64 / S of them); larger cubes: 64 slots.  With a
// channel split, workgroup block v is part v % kparts of block v / kparts.
struct QBlock {
    long long slot0, k_first;
    int nrows, ncores;
    int part;
};
__device__ __forceinline__ QBlock qblock(const QuantArgs& a, long long v) {
    QBlock q;
    const long long b = v / a.kparts;
    q.part = (int)(v - b * a.kparts);
    if (a.core_mode == 0) {
        const int cpb = QROWS / a.g.S;
        q.k_first = b * cpb;
        q.ncores = (int)min((long long)cpb, a.g.K - q.k_first);
        q.slot0 = q.k_first * a.g.S;
        q.nrows = q.ncores * a.g.S;
    } else {
        q.slot0 = b * QROWS;
        q.nrows = (int)min((long long)QROWS, a.g.Nslot - q.slot0);
        q.k_first = q.slot0 / a.g.S;
        q.ncores = (int)((q.slot0 + q.nrows - 1) / a.g.S - q.k_first + 1);
    }
    return q;
}

// 8 channels (a quarter of a group) of row r from a chunk buffer, as fp32,
// OR-ed with sgn: a pad row (zero bytes in the buffer) read with
// sgn = 0x80000000 gives -0.0, which is an exact identity of IEEE addition
// (x + -0 = x for every x, zeros included), so pad rows drop out of the
// cube's sum in slot order without a branch.
template <typename XT>
struct QRaw {
    uint4 w[sizeof(XT) == 2 ? 1 : 2];
};
template <typename XT>
__device__ __forceinline__ QRaw<XT> qraw8(const uint8_t* buf, int r, int gc, int qq) {
    QRaw<XT> q;
    if constexpr (sizeof(XT) == 2) {
        q.w[0] = *(const uint4*)(buf + qoff(r, 4 * gc + qq));
    } else {
        q.w[0] = *(const uint4*)(buf + qoff(r, 8 * gc + 2 * qq));
        q.w[1] = *(const uint4*)(buf + qoff(r, 8 * gc + 2 * qq + 1));
    }
    return q;
}
template <typename XT>
__device__ __forceinline__ void qconv8(const QRaw<XT>& q, uint32_t sgn, float* v) {
    if constexpr (sizeof(XT) == 2) {
        const uint32_t d[4] = {q.w[0].x, q.w[0].y, q.w[0].z, q.w[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float((d[i] << 16) | sgn);
            v[2 * i + 1] = __uint_as_float((d[i] & 0xffff0000u) | sgn);
        }
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v[4 * h] = __uint_as_float(q.w[h].x | sgn);
            v[4 * h + 1] = __uint_as_float(q.w[h].y | sgn);
            v[4 * h + 2] = __uint_as_float(q.w[h].z | sgn);
            v[4 * h + 3] = __uint_as_float(q.w[h].w | sgn);
        }
    }
}
template <typename XT>
__device__ __forceinline__ void qload8(const uint8_t* buf, int r, int gc, int qq, uint32_t sgn, float* v) {
    if constexpr (sizeof(XT) == 2) {
        const uint4 w = *(const uint4*)(buf + qoff(r, 4 * gc + qq));
        const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float((d[i] << 16) | sgn);
            v[2 * i + 1] = __uint_as_float((d[i] & 0xffff0000u) | sgn);
        }
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint4 w = *(const uint4*)(buf + qoff(r, 8 * gc + 2 * qq + h));
            v[4 * h] = __uint_as_float(w.x | sgn);
            v[4 * h + 1] = __uint_as_float(w.y | sgn);
            v[4 * h + 2] = __uint_as_float(w.z | sgn);
            v[4 * h + 3] = __uint_as_float(w.w | sgn);
        }
    }
}

// channels 4 e .. 4 e + 3 (e < 8) of group gc of row r: raw bits (bf16: an
// 8-byte half of a piece; fp32: a whole piece), and as fp32 OR-ed with sgn
template <typename XT>
__device__ __forceinline__ uint4 qraw4(const uint8_t* buf, int r, int gc, int e) {
    if constexpr (sizeof(XT) == 2) {
        const uint2 w = *(const uint2*)(buf + qoff(r, 4 * gc + (e >> 1)) + 8 * (e & 1));
        return make_uint4(w.x, w.y, 0u, 0u);
    } else {
        return *(const uint4*)(buf + qoff(r, 8 * gc + e));
    }
}
template <typename XT>
__device__ __forceinline__ void qconv4(uint4 q, uint32_t sgn, float* v) {
    if constexpr (sizeof(XT) == 2) {
        v[0] = __uint_as_float((q.x << 16) | sgn);
        v[1] = __uint_as_float((q.x & 0xffff0000u) | sgn);
        v[2] = __uint_as_float((q.y << 16) | sgn);
        v[3] = __uint_as_float((q.y & 0xffff0000u) | sgn);
    } else {
        v[0] = __uint_as_float(q.x | sgn);
        v[1] = __uint_as_float(q.y | sgn);
        v[2] = __uint_as_float(q.z | sgn);
        v[3] = __uint_as_float(q.w | sgn);
    }
}

// Ring depth for sp chunks per barrier: at most (depth - sp) chunks of
// copies outstanding (63, the vmcnt range), at most 150 KB of LDS, at most 8.
constexpr int qnbuf(int stage, int dmaw, int sp) {
    const int a = sp + 63 / dmaw, b = 150 * 1024 / stage;
    return a < b ? (a < 8 ? a : 8) : (b < 8 ? b : 8);
}

// Geometry of the activation pass for input type XT and NCT 32-wide rank
// tiles: channels per chunk, LDS stage (X chunk + L1 slice), copies per copy
// wave per chunk, chunks per barrier, ring depth, waves (wave 0: U; waves
// 1-2: copies; then one quantizer group of four waves per chunk of a period).
template <typename XT, int NCT>
struct QCfg {
    static constexpr int CC = XTraits<XT>::CC;
    static constexpr int LROWB = 2 * CC;
    static constexpr int LRPC = 1024 / LROWB;
    static constexpr int LDMA = NCT * 32 / LRPC / 2;
    static constexpr int QDMAW = QDMA + LDMA;
    static constexpr int STAGE = QCHUNK + NCT * 32 * LROWB;
    static constexpr int SP = qnbuf(STAGE, QDMAW, 2) >= 5 ? 2 : 1;
    static constexpr int NB = qnbuf(STAGE, QDMAW, SP);
    static constexpr int THREADS = (3 + 4 * SP) * 64;
};

// Cross-lane maxima of group maxima.  These are maxima of absolute values
// (non-negative floats; no NaN arises), ordered like their bit patterns as
// unsigned integers, so the exchanges take integer maxima: no NaN
// canonicalisation, and the DPP moves fold into the max instructions.
template <int CTRL>
__device__ __forceinline__ uint32_t umax_dpp(uint32_t b) {
    // (every lane reads a lane of its own row: bound_ctrl never applies, and
    // setting it lets the move fold into the max)
    return max(b, (uint32_t)__builtin_amdgcn_mov_dpp((int)b, CTRL, 0xF, 0xF, true));
}

// maximum over the four lanes of a quad (DPP quad_perm exchanges)
__device__ __forceinline__ float quad_max(float v) {
    uint32_t b = __float_as_uint(v);
    b = umax_dpp<0xB1>(b);
    b = umax_dpp<0x4E>(b);
    return __uint_as_float(b);
}

// maximum over a row of 16 lanes (quad exchanges, then the half-row and row
// mirrors: lane i meets lane 7 - i, then lane 15 - i)
__device__ __forceinline__ float row16_max(float v) {
    uint32_t b = __float_as_uint(quad_max(v));
    b = umax_dpp<0x141>(b);
    b = umax_dpp<0x140>(b);
    return __uint_as_float(b);
}

// maximum over an aligned group of 8 lanes (quad exchanges, then the
// half-row mirror: lane i meets lane 7 - i)
__device__ __forceinline__ float oct_max(float v) {
    return __uint_as_float(umax_dpp<0x141>(__float_as_uint(quad_max(v))));
}

// The maximum of a 64-channel core group from those of its two 32-channel
// halves, when their lanes are `d` apart in aligned blocks of 2 d lanes: the
// half-row mirror (d = 4), the row mirror (d = 8), a swizzle (d = 16) or a
// permute (d = 32).  Unchanged for 32-channel groups.
template <int D>
__device__ __forceinline__ float core_pair_max(float m, int g64) {
    if (!g64) return m;
    const uint32_t b = __float_as_uint(m);
    uint32_t o;
    if constexpr (D == 4) o = (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0x141, 0xF, 0xF, true);
    else if constexpr (D == 8) o = (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0x140, 0xF, 0xF, true);
    else if constexpr (D == 16) o = (uint32_t)__builtin_amdgcn_ds_swizzle((int)b, 0x401F);
    else o = (uint32_t)__builtin_amdgcn_ds_bpermute((int)((__lane_id() ^ 32) << 2), (int)b);
    return __uint_as_float(max(b, o));
}

// channels ch, ch + 1 (ch even, chunk-relative) of row r as raw bits, and
// as fp32 OR-ed with sgn (see qconv8: pad rows read as -0.0)
template <typename XT>
__device__ __forceinline__ uint2 qraw2(const uint8_t* buf, int r, int ch) {
    constexpr int EPC = 16 / (int)sizeof(XT);
    const uint8_t* pc = buf + qoff(r, ch / EPC) + (ch % EPC) * (int)sizeof(XT);
    if constexpr (sizeof(XT) == 2) return make_uint2(*(const uint32_t*)pc, 0u);
    else return *(const uint2*)pc;
}
template <typename XT>
__device__ __forceinline__ float2 qconv2(uint2 d, uint32_t sgn) {
    if constexpr (sizeof(XT) == 2)
        return make_float2(__uint_as_float((d.x << 16) | sgn), __uint_as_float((d.x & 0xffff0000u) | sgn));
    else
        return make_float2(__uint_as_float(d.x | sgn), __uint_as_float(d.y | sgn));
}

// Persistent activation pass.  Workgroup w takes the 64-slot blocks w, w + G,
// w + 2G, ... and walks each block's channels in chunks of 256 bytes per row
// (with a channel split, those are parts of blocks, each a run of the
// block's chunks); the chunks of all its blocks form one stream.  Waves 1-2 copy chunks
// straight into an LDS ring (global_load_lds, one 16-byte piece per lane,
// absent rows and channels from a zero page) up to seven chunks ahead, across
// block boundaries, together with the chunk's slice of L1; they issue nothing
// else, so their copy counters track the ring exactly.  Wave 0 accumulates
// U = bf16(X) L1 with 32x32x16 bf16 MFMAs from the stage and stores it after
// a block's last chunk (a part's fp32 sum, with a channel split).  Waves 3-6 quantize: one
// (cube, 32-channel group, quarter) per thread, the quad of a group's four
// quarters sharing its maxima by DPP: the cube's core (fp32 sum in slot
// order, then the division), its FP8 codes, each row's delta FP4 codes.
// X is read from HBM exactly once.
//
// CM selects how a chunk's quantizer work is split:
//   0: one pass; each (cube, group, quarter) thread also codes the cube's
//      rows (blocks of 7 or more cubes);
//   2: two phases for blocks of at most 3 cubes (cubes of 17 to 64 tokens):
//      the (cube, group, quarter) threads write the fp32 core to LDS, a
//      second barrier per period follows, and then every thread of the
//      group codes (row, group, quarter) deltas;
//   1: cubes of more than 64 tokens: their cores come from a pass before
//      this one, and every thread of the group codes (row, group, quarter)
//      deltas reading them (one barrier per period);
//   3: one pass with one wave per cube, for blocks of 4 to 6 cubes (cubes
//      of 10 to 16 tokens): the core by channel pairs, then the cube's
//      (row, group, quarter) deltas, both on the same wave;
//   4: one pass for cubes of exactly 8 tokens: one (cube, group, eighth)
//      per thread (4 channels, 8 lanes per group), all 8 rows kept in
//      registers, so the block's 8 cubes fill the group's 256 threads.
template <typename XT, int NCT, int CM>
__global__ __launch_bounds__((QCfg<XT, NCT>::THREADS), 1) void k_quantize(QuantArgs a) {
    constexpr int CC = XTraits<XT>::CC;
    constexpr int NGC = CC / 32;                     // groups per chunk
    constexpr int EPC = 16 / (int)sizeof(XT);        // elements per 16-byte piece
    // L1 chunk (rank tile ct, row = rank, 2 CC bytes per row, pieces swizzled
    // like X) follows the X chunk in each ring stage
    constexpr int LROWB = 2 * CC;
    constexpr int LNP = LROWB / 16;                  // 16-byte pieces per L1 row
    constexpr int LRPC = 1024 / LROWB;               // L1 rows per 1 KB copy
    constexpr int LDMA = NCT * 32 / LRPC / 2;        // L1 copies per copy wave per chunk
    constexpr int QDMAW = QDMA + LDMA;               // copies per copy wave per chunk
    constexpr int STAGE = QCHUNK + NCT * 32 * LROWB;
    // chunks per barrier: two when the ring is deep enough (each quantizer
    // group then has two chunk periods for its chunk), else one
    constexpr int SP = QCfg<XT, NCT>::SP;
    constexpr int QNBUF = QCfg<XT, NCT>::NB;         // ring stages
    static_assert(QNBUF >= 2 * SP, "ring too shallow");
    __shared__ __attribute__((aligned(1024))) uint8_t xbuf[QNBUF * STAGE];
    __shared__ int tok_s[2][2][QROWS];              // [group][buffer]
    __shared__ int4 meta_s[2][2][QROWS];            // per cube: first row, end row, present rows (bit j: row first + j), tokens
    constexpr bool TWO = CM == 1 || CM == 2;         // (row, group, quarter) delta tasks over the whole group
    constexpr bool BAR2 = CM == 2;                   // phase 1 in the quantizers: two barriers per period
    constexpr int TCUBES = 8;                        // cubes per block in the two-phase forms
    constexpr bool CORES = CM == 2 || CM == 3;       // fp32 cores of the group's chunk in LDS
    __shared__ float core_s[CORES ? SP : 1][CORES ? TCUBES : 1][CC];
    __shared__ uint64_t pres_s[2][2];               // [group][buffer]: bit r = row r holds a token

    const Geom& g = a.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int nchunks = (a.Ci + CC - 1) / CC / a.kparts;   // chunks per (part of a) block
    const long long nmine = a.nblocks > (long long)blockIdx.x ? (a.nblocks - 1 - blockIdx.x) / gridDim.x + 1 : 0;
    if (nmine == 0) return;
    const long long total = nmine * nchunks;
    const uint32_t lds0 = (uint32_t)(uintptr_t)xbuf;
    const XT* __restrict__ x = (const XT*)a.x;
    const int qgrp = (wave - 3) >> 2;                // quantizer group (waves 3-6, 7-10)
    const int qtid = tid - 192 - 256 * qgrp;         // thread within the group

    // block metadata of a quantizer group, double-buffered: token of each
    // row; per cube its row range, which of its first 32 rows hold tokens,
    // and its token count
    auto fill_meta = [&](int mb, long long i) {
        const QBlock B = qblock(a, blockIdx.x + i * gridDim.x);
        int* const tok_s_ = tok_s[qgrp][mb];
        int4* const meta_s_ = meta_s[qgrp][mb];
        if (qtid < QROWS) {
            // (the group's first wave: one row per lane; the ballot gives
            // every row's presence, so no cube walks its rows in memory)
            const int tk = qtid < B.nrows ? a.stok[B.slot0 + qtid] : -1;
            tok_s_[qtid] = tk;
            const uint64_t pres = __ballot(tk >= 0);
            if (qtid == 0) pres_s[qgrp][mb] = pres;
            const int rb = qtid < B.ncores ? (int)max(0LL, (B.k_first + qtid) * g.S - B.slot0) : 0;
            const int re = qtid < B.ncores ? (int)min((long long)B.nrows, (B.k_first + qtid + 1) * g.S - B.slot0) : 0;
            const int n = re - rb;                             // rows of the cube in this block
            const int pm = n <= 0 ? 0 : (int)(uint32_t)((pres >> rb) & (n >= 32 ? 0xffffffffull : ((1ull << n) - 1)));
            int ct, ch, cw;
            const int cnt = qtid < B.ncores ? cube_count(g, B.k_first + qtid, &ct, &ch, &cw) : 0;
            meta_s_[qtid] = make_int4(rb, re, pm, cnt);
        }
    };

    // ---- copy waves: wave 1 rows 0-31, wave 2 rows 32-63 of each chunk; copy
    // j covers rows 4 j .. 4 j + 3 of the wave's half (lane: row + lane / 16,
    // piece lane % 16).  The cursor (block i_f, chunk c_f) runs past the end on
    // zero-page copies into buffers no one reads, so every chunk step issues
    // the same number of copies.
    const int cw = __builtin_amdgcn_readfirstlane(wave - 1);
    long long i_f = 0, s_f = 0;
    int c_f = 0, clo_f = 0;          // chunk within the part; the part's first chunk
    int tokr[QDMA];
    // tokens of a block's rows: scalar loads (they count on lgkmcnt, so the
    // copy counter keeps tracking the copies alone), then each lane picks its row
    typedef const __attribute__((address_space(4))) int cint;
    cint* stok_c = (cint*)(uintptr_t)a.stok;
    auto load_toks = [&](long long i) {
        int t[QDMA][4];
        const QBlock Bn = qblock(a, blockIdx.x + min(i, nmine - 1) * gridDim.x);
        clo_f = Bn.part * nchunks;
#pragma unroll
        for (int j = 0; j < QDMA; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = 32 * cw + 4 * j + q;
                t[j][q] = (i < nmine && r < Bn.nrows) ? stok_c[Bn.slot0 + r] : -1;
            }
        const int sel = lane >> 4;
#pragma unroll
        for (int j = 0; j < QDMA; ++j) tokr[j] = sel == 0 ? t[j][0] : sel == 1 ? t[j][1] : sel == 2 ? t[j][2] : t[j][3];
    };
    auto issue = [&]() {
        const uint32_t stage = lds0 + (uint32_t)(s_f % QNBUF) * STAGE;
        const uint32_t base = stage + cw * (QCHUNK / 2);
        const int c0 = (clo_f + c_f) * CC;
#pragma unroll
        for (int j = 0; j < QDMA; ++j) {
            const int r = 32 * cw + 4 * j + (lane >> 4);
            const int ch = c0 + ((lane & 15) ^ (r & 15)) * EPC;   // first channel of the logical piece at this position
            const void* src = (tokr[j] >= 0 && ch < a.Ci) ? (const void*)(x + (long long)tokr[j] * a.Ci + ch)
                                                          : (const void*)(a.zero + 16 * (lane & 15));
            // (nontemporal: each byte of X is read once; the L1 rows below are
            // read by every block and keep the default policy)
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(__builtin_amdgcn_readfirstlane(base + j * 1024)), "v"(src)
                         : "memory", "m0");
        }
        // L1 rows of the chunk (in bounds: l1t rows are Kp wide, zero past Ci)
#pragma unroll
        for (int j = 0; j < LDMA; ++j) {
            const int lr = (cw * LDMA + j) * LRPC + lane / LNP;            // L1 row (rank) of this lane
            const int pc = (lane % LNP) ^ (lr % LNP);                      // logical piece at this position
            const uint16_t* src = a.l1t + (long long)lr * a.Kp + c0 + 8 * pc;
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(__builtin_amdgcn_readfirstlane(stage + QCHUNK + (cw * LDMA + j) * 1024)),
                         "v"(src) : "memory", "m0");
        }
        ++s_f;
        if (++c_f == nchunks) {
            c_f = 0;
            load_toks(++i_f);
        }
    };
    auto barrier = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // ---- U accumulators (wave 0): two 32-row tiles x NCT 32-wide rank tiles
    v16f uacc[2][NCT > 0 ? NCT : 1];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < (NCT > 0 ? NCT : 1); ++j) uacc[i][j] = (v16f){};

    // The three roles run their own loops over the chunk stream, one barrier
    // per period of SP chunks: chunks SP u .. SP u + SP - 1 have landed and
    // are visible at barrier u, and every wave is done with the previous
    // period's chunks, whose stages take the copies of chunks
    // SP u + QNBUF - SP .. SP u + QNBUF - 1.  Quantizer group q takes chunk
    // SP u + q.
    const long long nsteps = (total + SP - 1) / SP;   // barrier periods
    if (wave == 1 || wave == 2) {
        load_toks(0);
        for (int k = 0; k < QNBUF - SP; ++k) issue();
        for (long long u = 0; u < nsteps; ++u) {
            // chunks SP u .. SP u + SP - 1 landed: later copies in flight
            constexpr int LATER = (QNBUF - 2 * SP) * QDMAW;
            __builtin_amdgcn_s_waitcnt((LATER & 15) | ((LATER >> 4) << 14) | 0x0F70);
            barrier();
#pragma unroll
            for (int k = 0; k < SP; ++k) issue();
            if constexpr (BAR2) barrier();
        }
        // the surplus copies land before the wave ends (no copy may write
        // LDS after the workgroup has released it)
        __builtin_amdgcn_s_waitcnt(0x0F70);
        return;
    }
    long long i = 0;      // block ordinal of chunk step s
    int c = 0;            // chunk of step s within its block
    QBlock B = qblock(a, blockIdx.x);
    auto next_chunk = [&]() {
        if (++c == nchunks) {
            c = 0;
            ++i;
            if (i < nmine) B = qblock(a, blockIdx.x + i * gridDim.x);
        }
    };
    if (wave == 0) {
        for (long long s = 0; s < total; ++s, next_chunk()) {
            if (s % SP == 0) {
                barrier();
                if constexpr (BAR2) barrier();
            }
            if constexpr (NCT == 0) continue;
            const uint8_t* buf = xbuf + (int)(s % QNBUF) * STAGE;
            // ---- U += bf16(X chunk) L1 chunk, both operands from the stage
            auto a_frag = [&](int rt, int kk) {
                const int r = rt * 32 + (lane & 31);
                if constexpr (sizeof(XT) == 2) {
                    return __builtin_bit_cast(v8bf, *(const uint4*)(buf + qoff(r, kk / 8 + (lane >> 5))));
                } else {
                    const int cq = (kk + 8 * (lane >> 5)) / 4;
                    const float4 p0 = *(const float4*)(buf + qoff(r, cq));
                    const float4 p1 = *(const float4*)(buf + qoff(r, cq + 1));
                    const float f8[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
                    v8bf v;
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(__bf16, bf16_rne(f8[e]));
                    return v;
                }
            };
            auto b_frag = [&](int ct, int kk) {
                const int lr = ct * 32 + (lane & 31);
                const int pc = kk / 8 + (lane >> 5);
                return __builtin_bit_cast(v8bf, *(const uint4*)(buf + QCHUNK + lr * LROWB + ((pc ^ (lr % LNP)) << 4)));
            };
            // (Kp is a multiple of 128, so a chunk never passes it)
#pragma unroll
            for (int q = 0; q < CC / 16; ++q) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const v8bf bv = b_frag(ct, 16 * q);
                    uacc[0][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_frag(0, 16 * q), bv, uacc[0][ct], 0, 0, 0);
                    uacc[1][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_frag(1, 16 * q), bv, uacc[1][ct], 0, 0, 0);
                }
            }
            if (c + 1 == nchunks) {
                // ---- U -> bf16, slot order (rows of absent tokens were zero)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int row = rt * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                            if (row >= B.nrows) continue;
                            if (a.kparts == 1)
                                a.u[(B.slot0 + row) * a.rp + ct * 32 + (lane & 31)] = bf16_rne(uacc[rt][ct][e]);
                            else
                                a.upart[((long long)B.part * a.urows + B.slot0 + row) * a.rp + ct * 32 + (lane & 31)] = uacc[rt][ct][e];
                        }
                        uacc[rt][ct] = (v16f){};
                    }
            }
        }
        // barriers of the periods after the last chunk's (none: total chunks
        // fill nsteps periods, the last one possibly partly)
        return;
    }
    // quantizer groups: group q takes chunks q, q + SP, q + 2 SP, ...
    // Their waves issue ahead of the U and copy waves sharing their SIMDs
    // (those have slack: they wait at the barriers), so a period ends when
    // the quantizers' work does (2-5 % faster on the 720p FFN layers).
    __builtin_amdgcn_s_setprio(1);
    for (int k = 0; k < qgrp; ++k) next_chunk();
    int mb = 0;                                      // the group's metadata buffer of its current block
    if (qgrp < total) fill_meta(0, i);
    if constexpr (TWO) {
        const long long nks = a.Kp / 128;
        constexpr int NT2 = QROWS * NGC * 4 / 256;   // (row, group, quarter) delta tasks per thread
        // CM 1: the cores of the group's next chunk, loaded from the earlier
        // pass's rows one period ahead (they land during the barrier wait
        // instead of stalling the chunk); rows past the last slot clamp to a
        // valid cube and columns stay below Kp
        float4 kn[CM == 1 ? NT2 : 1][2];
        auto load_cores = [&]() {
            if constexpr (CM == 1) {
#pragma unroll
                for (int n = 0; n < NT2; ++n) {
                    const int t = qtid + 256 * n;
                    const int qq = t & 3, pr = t >> 2;
                    const int r = pr / NGC, gc = pr - r * NGC;
                    const long long k = min((B.slot0 + r) / g.S, g.K - 1);
                    const float4* cp = (const float4*)(a.coref + k * (long long)a.Kp + ((B.part * nchunks + c) * CC + gc * 32) + 8 * qq);
                    kn[n][0] = cp[0];
                    kn[n][1] = cp[1];
                }
            }
        };
        if (qgrp < total) load_cores();
        for (long long u = 0; u < nsteps; ++u) {
            barrier();
            const long long s = SP * u + qgrp;
            const bool have = s < total;
            const int c0 = (B.part * nchunks + c) * CC;
            const uint8_t* buf = xbuf + (int)(s % QNBUF) * STAGE;
            float(*const cs_)[CC] = core_s[qgrp];
            // ---- phase 1 (CM 2): the cores, one (cube, channel pair) per
            // thread, 16 lanes per 32-channel group.  (CM 1 reads the cores
            // from the earlier pass in phase 2 and has no phase 1.)
            if constexpr (CM == 2) {
                const uint64_t pres = pres_s[qgrp][mb];
                // the second group's tasks start at its third wave, so the two
                // groups' first tasks (all of them when a block has one cube)
                // run on different SIMDs (waves go round-robin over the four)
                const int tq = (qtid + 128 * qgrp) & 255;
                // blocks of one cube: one (cube, channel) per thread, 32 lanes
                // per group (the sums are chains in slot order, so a channel
                // is the finest split; pairs would keep one wave per group
                // busy).  With more cubes, pairs (fewer instructions per
                // channel) already spread over the SIMDs.
                const int nsingle = have && B.ncores * CC <= 128 ? B.ncores * CC : 0;
                for (int t = tq; t < nsingle; t += 256) {
                    const int cr = t / CC, ch = t - cr * CC;
                    if (c0 + ch >= a.Ci) continue;             // the same for the group's 32 lanes
                    const long long k = B.k_first + cr;
                    const int rb = cr * g.S, re = rb + g.S, cnt = meta_s[qgrp][mb][cr].w;
                    // fp32 sum of the present rows in slot order (pad rows read as
                    // -0.0 and drop out exactly); sixteen rows' loads in flight
                    const uint8_t* const pc = buf + (ch % EPC) * (int)sizeof(XT);
                    const int pch = ch / EPC;
                    // the raw bits of row r's element (the bf16 widening
                    // happens after the reads: a widening inside the read
                    // would be a use, and the compiler would wait for each
                    // read before issuing the next)
                    auto raw1 = [&](int r) -> uint32_t {
                        if constexpr (sizeof(XT) == 2) return (uint32_t)*(const uint16_t*)(pc + qoff(r, pch));
                        else return *(const uint32_t*)(pc + qoff(r, pch));
                    };
                    auto val1 = [&](uint32_t v, uint32_t sgn) -> float {
                        if constexpr (sizeof(XT) == 2) return __uint_as_float((v << 16) | sgn);
                        else return __uint_as_float(v | sgn);
                    };
                    float s0 = -0.0f;
                    int r = rb;
                    // (a cube with all its tokens needs no pad-row masks)
                    const uint32_t full = cnt == g.S ? 0xffffffffu : 0u;
                    // Batches of sixteen rows: the batch's values are widened
                    // (and masked) first, then the next batch's reads go out,
                    // then the sixteen adds of the chain issue back to back
                    // while those reads are in flight.
                    uint32_t raw[16];
                    if (r + 16 <= re) {
#pragma unroll
                        for (int j = 0; j < 16; ++j) raw[j] = raw1(r + j);
                    }
                    for (; r + 16 <= re; r += 16) {
                        float v[16];
                        if (full) {
#pragma unroll
                            for (int j = 0; j < 16; ++j) v[j] = val1(raw[j], 0u);
                        } else {
                            const uint32_t absent = ~(uint32_t)(pres >> r);   // bit j: row r + j has no token
#pragma unroll
                            for (int j = 0; j < 16; ++j) v[j] = val1(raw[j], (absent << (31 - j)) & 0x80000000u);
                        }
                        if (r + 32 <= re) {
#pragma unroll
                            for (int j = 0; j < 16; ++j) raw[j] = raw1(r + 16 + j);
                        }
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int j = 0; j < 16; ++j) s0 += v[j];
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    for (; r < re; ++r) s0 += val1(raw1(r), ((pres >> r) & 1) ? 0u : 0x80000000u);
                    if ((cnt & (cnt - 1)) == 0) s0 *= inv_pow2(cnt);   // exact power-of-two scaling
                    else s0 = __fdiv_rn(s0, (float)cnt);
                    float amax = row16_max(fabsf(s0));
                    amax = fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, amax), 0x401F)));   // lane ^ 16
                    const float cmax = core_pair_max<32>(amax, a.core_g64);
                    const int ex = a.core_fp4 ? mx_exp_fp4(cmax) : mx_exp_fp8(cmax);
                    const int gch = c0 + ch;                       // channel within the row
                    if (a.cbf) *cbf_at(a.cbf, k, gch, a.Kp) = bf16_rne(s0);
                    if (a.core_fp4) {
                        // a channel pair's two nibbles meet in its even lane
                        const float s1 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s0), 0xB1, 0xF, 0xF, false));
                        const uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, s0, s1, pow2f(ex), 0);
                        if ((ch & 1) == 0) *(uint8_t*)(a.cq + off_fp4(k, gch >> 5, nks) + ((gch & 31) >> 1)) = (uint8_t)w;
                    } else {
                        v2s z = {0, 0};
                        const v2s cd = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, s0, 0.0f, pow2f(ex), false);
                        *(uint8_t*)(a.cq + off_fp8(k, gch >> 7, (gch & 127) >> 4, nks) + (gch & 15)) =
                            (uint8_t)__builtin_bit_cast(uint32_t, cd);
                    }
                    if ((ch & 31) == 0) a.cs[off_scale(k, gch >> 5, nks)] = (uint8_t)(ex + 127);
                    cs_[cr][ch] = s0;
                }
                const int ntask = have && !nsingle ? B.ncores * (CC / 2) : 0;   // a multiple of 16: groups stay whole
                for (int t = tq; t < ntask; t += 256) {
                    const int cr = t / (CC / 2), ch = 2 * (t - cr * (CC / 2));
                    if (c0 + ch >= a.Ci) continue;             // the same for the group's 16 lanes
                    const long long k = B.k_first + cr;
                    const int rb = cr * g.S, re = rb + g.S, cnt = meta_s[qgrp][mb][cr].w;
                    // fp32 sum of the present rows in slot order (pad rows read as
                    // -0.0 and drop out exactly); sixteen rows' loads in flight
                    float s0 = -0.0f, s1 = -0.0f;
                    int r = rb;
                    const uint32_t full = cnt == g.S ? 0xffffffffu : 0u;   // all tokens: no pad-row masks
                    for (; r + 16 <= re; r += 16) {
                        uint2 raw[16];
#pragma unroll
                        for (int j = 0; j < 16; ++j) raw[j] = qraw2<XT>(buf, r + j, ch);
                        __builtin_amdgcn_sched_barrier(0);     // all sixteen reads issued before the first use
                        if (full) {
#pragma unroll
                            for (int j = 0; j < 16; ++j) {
                                const float2 v = qconv2<XT>(raw[j], 0u);
                                s0 += v.x;
                                s1 += v.y;
                            }
                        } else {
                            const uint32_t absent = ~(uint32_t)(pres >> r);   // bit j: row r + j has no token
#pragma unroll
                            for (int j = 0; j < 16; ++j) {
                                const float2 v = qconv2<XT>(raw[j], (absent << (31 - j)) & 0x80000000u);
                                s0 += v.x;
                                s1 += v.y;
                            }
                        }
                    }
                    if (r + 8 <= re) {                     // cubes of 8 to 15 rows (or the rest of one)
                        uint2 raw[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) raw[j] = qraw2<XT>(buf, r + j, ch);
                        __builtin_amdgcn_sched_barrier(0);
                        const uint32_t absent = ~(uint32_t)(pres >> r);
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const float2 v = qconv2<XT>(raw[j], (absent << (31 - j)) & 0x80000000u);
                            s0 += v.x;
                            s1 += v.y;
                        }
                        r += 8;
                    }
                    for (; r < re; ++r) {
                        const float2 v = qconv2<XT>(qraw2<XT>(buf, r, ch), ((pres >> r) & 1) ? 0u : 0x80000000u);
                        s0 += v.x;
                        s1 += v.y;
                    }
                    if ((cnt & (cnt - 1)) == 0) {                  // exact power-of-two scaling
                        const float rc = inv_pow2(cnt);
                        s0 *= rc;
                        s1 *= rc;
                    } else {
                        s0 = __fdiv_rn(s0, (float)cnt);
                        s1 = __fdiv_rn(s1, (float)cnt);
                    }
                    const float amax = row16_max(fmaxf(fabsf(s0), fabsf(s1)));
                    const float cmax = core_pair_max<16>(amax, a.core_g64);
                    const int ex = a.core_fp4 ? mx_exp_fp4(cmax) : mx_exp_fp8(cmax);
                    const int gch = c0 + ch;                       // channel within the row
                    if (a.cbf) *(uint32_t*)cbf_at(a.cbf, k, gch, a.Kp) = bf16x2(s0, s1);
                    if (a.core_fp4) {
                        *(uint8_t*)(a.cq + off_fp4(k, gch >> 5, nks) + ((gch & 31) >> 1)) =
                            (uint8_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, s0, s1, pow2f(ex), 0);
                    } else {
                        v2s z = {0, 0};
                        const v2s cd = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, s0, s1, pow2f(ex), false);
                        *(uint16_t*)(a.cq + off_fp8(k, gch >> 7, (gch & 127) >> 4, nks) + (gch & 15)) =
                            (uint16_t)__builtin_bit_cast(uint32_t, cd);
                    }
                    if ((ch & 31) == 0) a.cs[off_scale(k, gch >> 5, nks)] = (uint8_t)(ex + 127);
                    *(float2*)&cs_[cr][ch] = make_float2(s0, s1);
                }
                barrier();                                     // the group's cores are in LDS
            }
            // ---- phase 2: the deltas, one (row, group, quarter) per thread
            if (have) {
                const uint64_t pres = pres_s[qgrp][mb];
                // every task computed first in straight-line code (absent rows
                // and channels read zeros from the stage and index a written or
                // stale core row in bounds), then the stores, predicated, so the
                // tasks' LDS reads and DPP maxima interleave and quads stay whole
                uint32_t code[NT2];
                int exq[NT2];
                bool live[NT2];
#pragma unroll
                for (int n = 0; n < NT2; ++n) {
                    const int t = qtid + 256 * n;
                    const int qq = t & 3, pr = t >> 2;
                    const int r = pr / NGC, gc = pr - r * NGC;
                    const long long G = (c0 >> 5) + gc;
                    live[n] = G * 32 < a.Ci && ((pres >> r) & 1);   // (pres has no bit for rows past the block)
                    float v[8];
                    qload8<XT>(buf, r, gc, qq, 0u, v);
                    float4 k0, k1;
                    if constexpr (CM == 1) {
                        k0 = kn[n][0];                         // loaded one period ahead
                        k1 = kn[n][1];
                    } else {
                        const int cr = r / g.S;
                        k0 = *(const float4*)&cs_[cr][gc * 32 + qq * 8];
                        k1 = *(const float4*)&cs_[cr][gc * 32 + qq * 8 + 4];
                    }
                    const float core[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
                    float dv[8];
                    float amax = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        dv[e] = v[e] - core[e];
                        amax = fmaxf(amax, fabsf(dv[e]));
                    }
                    amax = quad_max(amax);
                    exq[n] = mx_exp_fp4(amax);
                    const float sc = pow2f(exq[n]);
                    uint32_t w = 0u;
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, dv[0], dv[1], sc, 0);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, dv[2], dv[3], sc, 1);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, dv[4], dv[5], sc, 2);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, dv[6], dv[7], sc, 3);
                    code[n] = w;
                }
                // blocks of exactly 64 slots start at multiples of 64: their
                // rows lie in one 256-row tile (32-bit offsets)
                const bool tile64 = B.nrows == 64 && (B.slot0 & 63) == 0;
                uint8_t* const dq_t = a.dq + (size_t)(B.slot0 >> 8) * (size_t)nks * 16384;
                uint8_t* const ds_t = a.ds + (size_t)(B.slot0 >> 8) * (size_t)nks * 1024;
                if constexpr (NT2 == 4) {
                    // four groups per chunk: a thread's tasks are rows r0, r0 + 16,
                    // r0 + 32, r0 + 48 (r0 = thread / 16) of its (group, quarter),
                    // and a quad holds the four quarters of those rows; a 4 x 4
                    // transpose inside the quad (exchanges at distance 1, then 2)
                    // gives lane qq row r0 + 16 qq's whole 16-byte group code, one
                    // store per lane, and that row's scale code
                    const int qq_l = qtid & 3, gc_l = (qtid >> 2) & 3;
                    auto xchg = [&](uint32_t* v, auto dd, auto cc) {
                        constexpr int d = decltype(dd)::value, ctrl = decltype(cc)::value;
                        const bool hi = (qq_l & d) != 0;
#pragma unroll
                        for (int n = 0; n < 4; ++n) {
                            if (n & d) continue;                       // slot pair (n, n + d)
                            const uint32_t send = hi ? v[n] : v[n + d];
                            const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, ctrl, 0xF, 0xF, true);
                            v[n] = hi ? recv : v[n];
                            v[n + d] = hi ? v[n + d] : recv;
                        }
                    };
                    xchg(code, std::integral_constant<int, 1>{}, std::integral_constant<int, 0xB1>{});   // quad_perm [1, 0, 3, 2]
                    xchg(code, std::integral_constant<int, 2>{}, std::integral_constant<int, 0x4E>{});   // quad_perm [2, 3, 0, 1]
                    // liveness and scale of a row are the same in the four lanes of its quad
                    const bool lv = qq_l == 0 ? live[0] : qq_l == 1 ? live[1] : qq_l == 2 ? live[2] : live[3];
                    const int ex = qq_l == 0 ? exq[0] : qq_l == 1 ? exq[1] : qq_l == 2 ? exq[2] : exq[3];
                    const int r = (qtid >> 4) + 16 * qq_l;
                    // (delta codes: nontemporal stores, read once by the delta GEMM)
                    if (lv) {
                        if (tile64) {
                            const int G = (c0 >> 5) + gc_l, rt = (int)(B.slot0 & 255) + r;
                            __builtin_nontemporal_store(v4i{(int)code[0], (int)code[1], (int)code[2], (int)code[3]}, (v4i*)(dq_t + toff_fp4(rt, G)));
                            ds_t[toff_scale(rt, G)] = (uint8_t)(ex + 127);
                        } else {
                            const long long G = (c0 >> 5) + gc_l, sl = B.slot0 + r;
                            __builtin_nontemporal_store(v4i{(int)code[0], (int)code[1], (int)code[2], (int)code[3]}, (v4i*)(a.dq + off_fp4(sl, G, nks)));
                            a.ds[off_scale(sl, G, nks)] = (uint8_t)(ex + 127);
                        }
                    }
                } else {
#pragma unroll
                for (int n = 0; n < NT2; ++n) {
                    if (!live[n]) continue;
                    const int t = qtid + 256 * n;
                    const int qq = t & 3, pr = t >> 2;
                    const int r = pr / NGC, gc = pr - r * NGC;
                    if (tile64) {
                        const int G = (c0 >> 5) + gc, rt = (int)(B.slot0 & 255) + r;
                        __builtin_nontemporal_store(code[n], (uint32_t*)(dq_t + toff_fp4(rt, G) + 4 * qq));
                        if (qq == 0) ds_t[toff_scale(rt, G)] = (uint8_t)(exq[n] + 127);
                    } else {
                        const long long G = (c0 >> 5) + gc, sl = B.slot0 + r;
                        __builtin_nontemporal_store(code[n], (uint32_t*)(a.dq + off_fp4(sl, G, nks) + 4 * qq));
                        if (qq == 0) a.ds[off_scale(sl, G, nks)] = (uint8_t)(exq[n] + 127);
                    }
                }
                }
                const long long i_prev = i;
#pragma unroll
                for (int k = 0; k < SP; ++k) next_chunk();
                if (i != i_prev && i < nmine) {
                    mb ^= 1;
                    fill_meta(mb, i);
                }
                load_cores();
            }
        }
    } else {
    // The common one-pass case (see fast4 below): per-thread task constants.
    const bool fast4 = CM == 0 && sizeof(XT) == 2 && g.S == 4 && !a.core_fp4 && !a.cbf;
    const int f4_qq = qtid & 3, f4_gc = (qtid >> 2) & 3, f4_cr = qtid >> 4;
    uint32_t f4_lds[QKEEP];
#pragma unroll
    for (int j = 0; j < QKEEP; ++j) f4_lds[j] = (uint32_t)qoff(4 * f4_cr + j, 4 * f4_gc + f4_qq);
    long long f4_block = -1;
    uint32_t f4_drow = 0, f4_ds = 0, f4_cq = 0, f4_cs = 0;
    // One (cube, group, quarter) task of a 4-slot cube: the same arithmetic
    // as the general task below in its FULL form (fp32 sum of the rows in
    // slot order, pad rows as -0.0; the core divided, FP8-coded; the deltas
    // FP4-coded), with the offsets above.  K step kc of the outputs.
    auto task4 = [&](const uint8_t* buf, int kc, uint8_t* dq_t, uint8_t* ds_t, uint8_t* cq_t, uint8_t* cs_t) {
      if constexpr (sizeof(XT) == 2) {
        const int4 md = meta_s[qgrp][mb][f4_cr];
        const int pm = md.z, cnt = md.w;
        float core[8], xr[QKEEP][8];
        uint4 raw[QKEEP];
#pragma unroll
        for (int j = 0; j < QKEEP; ++j) raw[j] = *(const uint4*)(buf + f4_lds[j]);
#pragma unroll
        for (int j = 0; j < QKEEP; ++j) {
            QRaw<XT> q;
            q.w[0] = raw[j];
            qconv8<XT>(q, ((pm >> j) & 1) ? 0u : 0x80000000u, xr[j]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) core[e] = ((xr[0][e] + xr[1][e]) + xr[2][e]) + xr[3][e];
        if ((cnt & (cnt - 1)) == 0) {                      // exact power-of-two scaling
            const float rc = inv_pow2(cnt);
#pragma unroll
            for (int e = 0; e < 8; ++e) core[e] *= rc;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) core[e] = __fdiv_rn(core[e], (float)cnt);
        }
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(core[e]));
        amax = core_pair_max<4>(quad_max(amax), a.core_g64);
        const int cex = mx_exp_fp8(amax);
        const float csc = pow2f(cex);
        uint32_t d[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v2s z = {0, 0};
            v2s lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, core[4 * h], core[4 * h + 1], csc, false);
            v2s hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, core[4 * h + 2], core[4 * h + 3], csc, true);
            d[h] = __builtin_bit_cast(uint32_t, hi);
        }
        *(uint2*)(cq_t + (size_t)kc * 32768 + f4_cq) = make_uint2(d[0], d[1]);
        if (f4_qq == 0) cs_t[(size_t)kc * 1024 + f4_cs] = (uint8_t)(cex + 127);
        float am[QKEEP];
        uint32_t code[QKEEP];
        int ex[QKEEP];
#pragma unroll
        for (int j = 0; j < QKEEP; ++j) {
            am[j] = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                xr[j][e] = xr[j][e] - core[e];
                am[j] = fmaxf(am[j], fabsf(xr[j][e]));
            }
        }
#pragma unroll
        for (int j = 0; j < QKEEP; ++j) am[j] = quad_max(am[j]);
#pragma unroll
        for (int j = 0; j < QKEEP; ++j) {
            ex[j] = mx_exp_fp4(am[j]);
            const float sc = pow2f(ex[j]);
            uint32_t w = 0u;
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xr[j][0], xr[j][1], sc, 0);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xr[j][2], xr[j][3], sc, 1);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xr[j][4], xr[j][5], sc, 2);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xr[j][6], xr[j][7], sc, 3);
            code[j] = w;
        }
        // Lane qq holds 4 bytes (its 8 channels) of each row's 16-byte group
        // code; a 4 x 4 transpose inside the quad (lane exchanges at distance
        // 1, then 2) gives lane qq row qq's whole code, stored with one
        // 16-byte store (the quads of a row's four groups then write its
        // 64 bytes in full).  Exchange at distance d: a lane keeps slot j when
        // bit d of j equals its own and takes the partner's slot j ^ d
        // otherwise.
        auto xchg = [&](uint32_t* v, auto dd, auto cc) {
            constexpr int d = decltype(dd)::value, ctrl = decltype(cc)::value;
            const bool hi = (f4_qq & d) != 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j & d) continue;                           // slot pair (j, j + d)
                const uint32_t send = hi ? v[j] : v[j + d];
                const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, ctrl, 0xF, 0xF, true);
                v[j] = hi ? recv : v[j];
                v[j + d] = hi ? v[j + d] : recv;
            }
        };
        xchg(code, std::integral_constant<int, 1>{}, std::integral_constant<int, 0xB1>{});   // quad_perm [1, 0, 3, 2]
        xchg(code, std::integral_constant<int, 2>{}, std::integral_constant<int, 0x4E>{});   // quad_perm [2, 3, 0, 1]
        // (nontemporal: the delta codes stream out and are read once, by the
        // delta GEMM; the core codes keep the default policy, which measures
        // faster for them)
        {
            const v4i cv = {(int)code[0], (int)code[1], (int)code[2], (int)code[3]};
            __builtin_nontemporal_store(cv, (v4i*)(dq_t + (size_t)kc * 16384 + f4_drow));
        }
        const int exq = f4_qq == 0 ? ex[0] : f4_qq == 1 ? ex[1] : f4_qq == 2 ? ex[2] : ex[3];
        ds_t[(size_t)kc * 1024 + f4_ds] = (uint8_t)(exq + 127);
      }
    };
    for (long long u = 0; u < nsteps; ++u) {
        barrier();
        const long long s = SP * u + qgrp;
        if (s >= total) continue;
        const int c0 = (B.part * nchunks + c) * CC;
        const uint8_t* buf = xbuf + (int)(s % QNBUF) * STAGE;
        // ---- quantizer: one (cube, group, quarter) per thread
        const long long nks = a.Kp / 128;
        const int ntask = B.ncores * NGC * 4;
        // FULL: whole cubes of at least QKEEP rows with 64 % S == 0, so a
        // block's rows (and its cubes) lie in one 256-row tile of the outputs
        const bool full = CM == 0 && g.S >= QKEEP && 64 % g.S == 0;
        uint8_t* const dq_t = a.dq + (size_t)(B.slot0 >> 8) * (size_t)nks * 16384;
        uint8_t* const ds_t = a.ds + (size_t)(B.slot0 >> 8) * (size_t)nks * 1024;
        // blocks of exactly 64 slots start at multiples of 64: their rows lie in one 256-row tile
        const bool tile64 = B.ncores * g.S == 64 && (B.slot0 & 63) == 0;
        uint8_t* const cq_t = a.cq + (size_t)(B.k_first >> 8) * (size_t)nks * 32768;
        uint8_t* const cs_t = a.cs + (size_t)(B.k_first >> 8) * (size_t)nks * 1024;
        // one task (FULL: the case above, so the kept rows need no bound checks)
        auto task = [&](int t, auto full) {
            constexpr bool FULL = decltype(full)::value;
            const int qq = t & 3, pr = t >> 2;
            const int cr = pr / NGC, gc = pr - cr * NGC;
            const long long G = (c0 >> 5) + gc;
            if (G * 32 >= a.Ci) return;                        // the same for the quad
            const int4 md = meta_s[qgrp][mb][cr];
            const int rb = CM != 1 ? cr * g.S : md.x, re = CM != 1 ? rb + g.S : md.y, pm = md.z;   // whole cubes unless CM 1
            const int nr = CM != 1 ? g.S : re - rb;            // rows of the cube in this block
            const long long k = B.k_first + cr;
            float core[8], xr[QKEEP][8];                       // rows rb .. rb + QKEEP - 1 kept for the deltas
            QRaw<XT> raw[QKEEP];                               // all kept rows' LDS reads in flight together
#pragma unroll
            for (int j = 0; j < QKEEP; ++j)
                if (FULL || j < nr) raw[j] = qraw8<XT>(buf, rb + j, gc, qq);
#pragma unroll
            for (int j = 0; j < QKEEP; ++j)
                if (FULL || j < nr) qconv8<XT>(raw[j], ((pm >> j) & 1) ? 0u : 0x80000000u, xr[j]);
            if constexpr (CM == 0) {
                // fp32 sum of the present rows in slot order (pad rows read as
                // -0.0 and drop out exactly), then the division
#pragma unroll
                for (int e = 0; e < 8; ++e) core[e] = -0.0f;
#pragma unroll
                for (int j = 0; j < QKEEP; ++j)
                    if (FULL || j < nr)
#pragma unroll
                        for (int e = 0; e < 8; ++e) core[e] += xr[j][e];
                for (int r = rb + QKEEP; r < re; ++r) {
                    float v[8];
                    qload8<XT>(buf, r, gc, qq, tok_s[qgrp][mb][r] >= 0 ? 0u : 0x80000000u, v);
#pragma unroll
                    for (int e = 0; e < 8; ++e) core[e] += v[e];
                }
                const int cnt = md.w;
                if ((cnt & (cnt - 1)) == 0) {                  // exact power-of-two scaling
                    const float rc = inv_pow2(cnt);
#pragma unroll
                    for (int e = 0; e < 8; ++e) core[e] *= rc;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) core[e] = __fdiv_rn(core[e], (float)cnt);
                }
                float amax = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(core[e]));
                amax = core_pair_max<4>(quad_max(amax), a.core_g64);
                const int ex = a.core_fp4 ? mx_exp_fp4(amax) : mx_exp_fp8(amax);
                const float sc = pow2f(ex);
                if (a.cbf)
                    *(uint4*)cbf_at(a.cbf, k, G * 32 + 8 * qq, a.Kp) = make_uint4(bf16x2(core[0], core[1]), bf16x2(core[2], core[3]),
                                                                            bf16x2(core[4], core[5]), bf16x2(core[6], core[7]));
                if (a.core_fp4) {
                    uint32_t w = 0u;
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, core[0], core[1], sc, 0);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, core[2], core[3], sc, 1);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, core[4], core[5], sc, 2);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, core[6], core[7], sc, 3);
                    *(uint32_t*)(a.cq + off_fp4(k, G, nks) + 4 * qq) = w;
                    if (qq == 0) a.cs[off_scale(k, G, nks)] = (uint8_t)(ex + 127);
                } else {
                uint32_t d[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    v2s z = {0, 0};
                    v2s p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, core[4 * h], core[4 * h + 1], sc, false);
                    v2s q = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, core[4 * h + 2], core[4 * h + 3], sc, true);
                    d[h] = __builtin_bit_cast(uint32_t, q);
                }
                if constexpr (FULL) {
                    const int kt = (int)(B.k_first & 255) + cr;    // the block's cubes share one 256-cube tile
                    *(uint2*)(cq_t + toff_fp8(kt, (int)(G >> 2), 2 * (int)(G & 3) + (qq >> 1)) + 8 * (qq & 1)) = make_uint2(d[0], d[1]);
                    if (qq == 0) cs_t[toff_scale(kt, (int)G)] = (uint8_t)(ex + 127);
                } else {
                    *(uint2*)(a.cq + off_fp8(k, G >> 2, 2 * (int)(G & 3) + (qq >> 1), nks) + 8 * (qq & 1)) = make_uint2(d[0], d[1]);
                    if (qq == 0) a.cs[off_scale(k, G, nks)] = (uint8_t)(ex + 127);
                }
                }
            } else {
                const float4* cp = (const float4*)(a.coref + k * (long long)a.Kp + G * 32 + 8 * qq);
                const float4 w0 = cp[0], w1 = cp[1];
                core[0] = w0.x; core[1] = w0.y; core[2] = w0.z; core[3] = w0.w;
                core[4] = w1.x; core[5] = w1.y; core[6] = w1.z; core[7] = w1.w;
            }
            // Deltas of every row, pad rows included: their codes are never
            // read back as a token's (the forward pass discards pad rows' outputs).
            auto delta = [&](int r, const float* v) {
                float dv[8];
                float amax = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    dv[e] = v[e] - core[e];
                    amax = fmaxf(amax, fabsf(dv[e]));
                }
                amax = quad_max(amax);
                const int ex = mx_exp_fp4(amax);
                const float sc = pow2f(ex);
                uint32_t code = 0u;
                code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(code, dv[0], dv[1], sc, 0);
                code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(code, dv[2], dv[3], sc, 1);
                code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(code, dv[4], dv[5], sc, 2);
                code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(code, dv[6], dv[7], sc, 3);
                const long long sl = B.slot0 + r;
                *(uint32_t*)(a.dq + off_fp4(sl, G, nks) + 4 * qq) = code;
                if (qq == 0) a.ds[off_scale(sl, G, nks)] = (uint8_t)(ex + 127);
            };
            if constexpr (FULL) {
                // the kept rows together: their maxima, exponents and codes
                // interleave; lane qq writes row qq's scale code
                const int rt0 = (int)(B.slot0 & 255) + rb;          // the block's rows share one 256-row tile
                float am[QKEEP];
                uint32_t code[QKEEP];
                int ex[QKEEP];
#pragma unroll
                for (int j = 0; j < QKEEP; ++j) {
                    am[j] = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        xr[j][e] = xr[j][e] - core[e];
                        am[j] = fmaxf(am[j], fabsf(xr[j][e]));
                    }
                }
#pragma unroll
                for (int j = 0; j < QKEEP; ++j) am[j] = quad_max(am[j]);
#pragma unroll
                for (int j = 0; j < QKEEP; ++j) {
                    ex[j] = mx_exp_fp4(am[j]);
                    const float sc = pow2f(ex[j]);
                    uint32_t w = 0u;
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xr[j][0], xr[j][1], sc, 0);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xr[j][2], xr[j][3], sc, 1);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xr[j][4], xr[j][5], sc, 2);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xr[j][6], xr[j][7], sc, 3);
                    code[j] = w;
                }
                // rt0 is a multiple of 4 (cubes of 4, 8, .. 64 slots from a
                // tile row that is a multiple of S), so rows rt0 + j take
                // toff_fp4's swizzle of rt0 with j / 2 flipped into it: rows
                // j and j + 1 (j even) sit 64 bytes apart from one address
                static_assert(QKEEP == 4, "two row pairs");
                uint8_t* const d01 = dq_t + toff_fp4(rt0, (int)G) + 4 * qq;
                uint8_t* const d23 = dq_t + toff_fp4(rt0 + 2, (int)G) + 4 * qq;
                *(uint32_t*)d01 = code[0];
                *(uint32_t*)(d01 + 64) = code[1];
                *(uint32_t*)d23 = code[2];
                *(uint32_t*)(d23 + 64) = code[3];
                const int exq = qq == 0 ? ex[0] : qq == 1 ? ex[1] : qq == 2 ? ex[2] : ex[3];
                ds_t[toff_scale(rt0 + qq, (int)G)] = (uint8_t)(exq + 127);
            } else if (g.S > 1) {                           // one-token cubes: every delta is 0, not stored
#pragma unroll
                for (int j = 0; j < QKEEP; ++j)
                    if (j < nr) delta(rb + j, xr[j]);
            }
            for (int r = rb + QKEEP; r < re; ++r) {
                if (tok_s[qgrp][mb][r] < 0) continue;
                float v[8];
                qload8<XT>(buf, r, gc, qq, 0u, v);
                delta(r, v);
            }
        };
        if constexpr (CM == 3) {
            // one wave per cube (4 to 8 cubes per block, 1 or 2 per wave):
            // the wave's lanes take channel pairs for the cube's core, write
            // it to LDS, and then take (row, group, quarter) delta tasks of
            // the same cube; the core passes between lanes of one wave only
            // (LDS operations of a wave complete in order), so no barrier
            const int wq = qtid >> 6;                      // wave within the group
            const uint64_t pres = pres_s[qgrp][mb];
            float(*const cs_)[CC] = core_s[qgrp];
            for (int cr = wq; cr < B.ncores; cr += 4) {    // wave-uniform
                const long long k = B.k_first + cr;
                const int rb = cr * g.S, S = g.S;
                // core: channels ch, ch + 1 of the chunk, rows in slot order
                // (pad rows add -0.0: exact), every row's read in flight
                const int ch = 2 * lane;
                float s0 = -0.0f, s1 = -0.0f;
                int r = 0;
                const int cnt = meta_s[qgrp][mb][cr].w;
                const uint32_t full = cnt == S ? 0xffffffffu : 0u;   // all tokens: no pad-row masks
                for (; r + 8 <= S; r += 8) {
                    uint2 raw[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) raw[j] = qraw2<XT>(buf, rb + r + j, ch);
                    __builtin_amdgcn_sched_barrier(0);
                    if (full) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const float2 v = qconv2<XT>(raw[j], 0u);
                            s0 += v.x;
                            s1 += v.y;
                        }
                    } else {
                        const uint32_t absent = ~(uint32_t)(pres >> (rb + r));
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const float2 v = qconv2<XT>(raw[j], (absent << (31 - j)) & 0x80000000u);
                            s0 += v.x;
                            s1 += v.y;
                        }
                    }
                }
                for (; r < S; ++r) {
                    const float2 v = qconv2<XT>(qraw2<XT>(buf, rb + r, ch), ((pres >> (rb + r)) & 1) ? 0u : 0x80000000u);
                    s0 += v.x;
                    s1 += v.y;
                }
                if ((cnt & (cnt - 1)) == 0) {              // exact power-of-two scaling
                    const float rc = inv_pow2(cnt);
                    s0 *= rc;
                    s1 *= rc;
                } else {
                    s0 = __fdiv_rn(s0, (float)cnt);
                    s1 = __fdiv_rn(s1, (float)cnt);
                }
                {
                    const float amax = row16_max(fmaxf(fabsf(s0), fabsf(s1)));   // 16 lanes: one 32-channel group
                    const float cmax = core_pair_max<16>(amax, a.core_g64);
                    const int ex = a.core_fp4 ? mx_exp_fp4(cmax) : mx_exp_fp8(cmax);
                    v2s z = {0, 0};
                    const uint16_t cd = a.core_fp4
                        ? (uint16_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, s0, s1, pow2f(ex), 0)
                        : (uint16_t)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, s0, s1, pow2f(ex), false));
                    // (fp32 chunks have CC = 64 channels: lanes 32-63 store
                    // nothing; the conditions hold for whole 16-lane groups)
                    const int gch = c0 + ch;               // channel within the row
                    if (ch < CC) {
                        if (gch < a.Ci) {
                            if (a.cbf) *(uint32_t*)cbf_at(a.cbf, k, gch, a.Kp) = bf16x2(s0, s1);
                            if (a.core_fp4) *(uint8_t*)(a.cq + off_fp4(k, gch >> 5, nks) + ((gch & 31) >> 1)) = (uint8_t)cd;
                            else *(uint16_t*)(a.cq + off_fp8(k, gch >> 7, (gch & 127) >> 4, nks) + (gch & 15)) = cd;
                            if ((ch & 31) == 0) a.cs[off_scale(k, gch >> 5, nks)] = (uint8_t)(ex + 127);
                        }
                        *(float2*)&cs_[cr][ch] = make_float2(s0, s1);
                    }
                }
                // deltas: (row, group, quarter) tasks of this cube, computed
                // side by side, stores predicated (absent rows and channels
                // read zeros and in-bounds rows; quads stay whole)
                constexpr int NTW = (16 * NGC * 4 + 63) / 64;   // tasks per lane for cubes of up to 16 rows
                uint32_t code[NTW];
                int exq[NTW];
                bool live[NTW];
                // a lane's tasks share their (group, quarter), so their core slice is read once
                const int qq_l = lane & 3, gc_l = (lane >> 2) % NGC;
                const float4 k0 = *(const float4*)&cs_[cr][gc_l * 32 + qq_l * 8];
                const float4 k1 = *(const float4*)&cs_[cr][gc_l * 32 + qq_l * 8 + 4];
                const float core[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
                for (int n = 0; n < NTW; ++n) {
                    const int t = lane + 64 * n;
                    const int qq = t & 3, pr = t >> 2;
                    const int j = pr / NGC, gc = pr - j * NGC;
                    const int rr = min(rb + j, QROWS - 1);
                    const long long G = (c0 >> 5) + gc;
                    live[n] = j < S && G * 32 < a.Ci && ((pres >> rr) & 1);
                    float v[8];
                    qload8<XT>(buf, rr, gc, qq, 0u, v);
                    float dv[8];
                    float amax = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        dv[e] = v[e] - core[e];
                        amax = fmaxf(amax, fabsf(dv[e]));
                    }
                    amax = quad_max(amax);
                    exq[n] = mx_exp_fp4(amax);
                    const float sc = pow2f(exq[n]);
                    uint32_t w = 0u;
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, dv[0], dv[1], sc, 0);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, dv[2], dv[3], sc, 1);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, dv[4], dv[5], sc, 2);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, dv[6], dv[7], sc, 3);
                    code[n] = w;
                }
                if constexpr (NTW == 4) {
                    // four groups per chunk: a lane's tasks are rows j0, j0 + 4,
                    // j0 + 8, j0 + 12 (j0 = lane / 16) of its (group, quarter),
                    // and a quad holds the four quarters of those rows.  A 4 x 4
                    // transpose inside the quad (lane exchanges at distance 1,
                    // then 2; a lane keeps slot n when bit d of n equals its own
                    // and takes the partner's slot n ^ d otherwise) gives lane qq
                    // row j0 + 4 qq's whole 16-byte group code: one store per
                    // lane, and the row's scale code from the same lane.
                    auto xchg = [&](uint32_t* v, auto dd, auto cc) {
                        constexpr int d = decltype(dd)::value, ctrl = decltype(cc)::value;
                        const bool hi = (qq_l & d) != 0;
#pragma unroll
                        for (int n = 0; n < 4; ++n) {
                            if (n & d) continue;                       // slot pair (n, n + d)
                            const uint32_t send = hi ? v[n] : v[n + d];
                            const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, ctrl, 0xF, 0xF, true);
                            v[n] = hi ? recv : v[n];
                            v[n + d] = hi ? v[n + d] : recv;
                        }
                    };
                    xchg(code, std::integral_constant<int, 1>{}, std::integral_constant<int, 0xB1>{});   // quad_perm [1, 0, 3, 2]
                    xchg(code, std::integral_constant<int, 2>{}, std::integral_constant<int, 0x4E>{});   // quad_perm [2, 3, 0, 1]
                    // liveness and scale of a row are the same in the four lanes of its quad
                    const bool lv = qq_l == 0 ? live[0] : qq_l == 1 ? live[1] : qq_l == 2 ? live[2] : live[3];
                    const int ex = qq_l == 0 ? exq[0] : qq_l == 1 ? exq[1] : qq_l == 2 ? exq[2] : exq[3];
                    const int j = (lane >> 4) + 4 * qq_l;
                    if (lv) {
                        if (tile64) {                              // 32-bit offsets in the block's tile
                            const int G = (c0 >> 5) + gc_l, rt = (int)(B.slot0 & 255) + rb + j;
                            *(uint4*)(dq_t + toff_fp4(rt, G)) = make_uint4(code[0], code[1], code[2], code[3]);
                            ds_t[toff_scale(rt, G)] = (uint8_t)(ex + 127);
                        } else {
                            const long long G = (c0 >> 5) + gc_l, sl = B.slot0 + rb + j;
                            *(uint4*)(a.dq + off_fp4(sl, G, nks)) = make_uint4(code[0], code[1], code[2], code[3]);
                            a.ds[off_scale(sl, G, nks)] = (uint8_t)(ex + 127);
                        }
                    }
                } else {
#pragma unroll
                for (int n = 0; n < NTW; ++n) {
                    if (!live[n]) continue;
                    const int t = lane + 64 * n;
                    const int qq = t & 3, pr = t >> 2;
                    const int j = pr / NGC, gc = pr - j * NGC;
                    if (tile64) {                              // 32-bit offsets in the block's tile
                        const int G = (c0 >> 5) + gc, rt = (int)(B.slot0 & 255) + rb + j;
                        *(uint32_t*)(dq_t + toff_fp4(rt, G) + 4 * qq) = code[n];
                        if (qq == 0) ds_t[toff_scale(rt, G)] = (uint8_t)(exq[n] + 127);
                    } else {
                        const long long G = (c0 >> 5) + gc, sl = B.slot0 + rb + j;
                        *(uint32_t*)(a.dq + off_fp4(sl, G, nks) + 4 * qq) = code[n];
                        if (qq == 0) a.ds[off_scale(sl, G, nks)] = (uint8_t)(exq[n] + 127);
                    }
                }
                }
            }
        } else if constexpr (CM == 4) {
            // cubes of 8 rows, whole in the block (64 of its slots, one
            // 256-row tile of the outputs): one (cube, group, eighth) per thread
            for (int t = qtid; t < B.ncores * NGC * 8; t += 256) {
                const int e = t & 7, pr = t >> 3;
                const int cr = pr / NGC, gc = pr - cr * NGC;
                const long long G = (c0 >> 5) + gc;
                if (G * 32 >= a.Ci) continue;                  // the same for the 8 lanes
                const int rb = cr * 8, pm = meta_s[qgrp][mb][cr].z;
                uint4 raw[8];
                float xr[8][4], core[4];
#pragma unroll
                for (int j = 0; j < 8; ++j) raw[j] = qraw4<XT>(buf, rb + j, gc, e);
#pragma unroll
                for (int j = 0; j < 8; ++j) qconv4<XT>(raw[j], ((pm >> j) & 1) ? 0u : 0x80000000u, xr[j]);
                // fp32 sum of the present rows in slot order (pad rows read as
                // -0.0 and drop out exactly), then the division
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    core[q] = -0.0f;
#pragma unroll
                    for (int j = 0; j < 8; ++j) core[q] += xr[j][q];
                }
                const int cnt = meta_s[qgrp][mb][cr].w;
                if ((cnt & (cnt - 1)) == 0) {                  // exact power-of-two scaling
                    const float rc = inv_pow2(cnt);
#pragma unroll
                    for (int q = 0; q < 4; ++q) core[q] *= rc;
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) core[q] = __fdiv_rn(core[q], (float)cnt);
                }
                const int kt = (int)(B.k_first & 255) + cr;    // the block's cubes share one 256-cube tile
                {
                    float amax = 0.0f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) amax = fmaxf(amax, fabsf(core[q]));
                    const float cmax = core_pair_max<8>(oct_max(amax), a.core_g64);
                    const int ex = a.core_fp4 ? mx_exp_fp4(cmax) : mx_exp_fp8(cmax);
                    const float sc = pow2f(ex);
                    if (a.cbf)
                        *(uint2*)cbf_at(a.cbf, B.k_first + cr, G * 32 + 4 * e, a.Kp) = make_uint2(bf16x2(core[0], core[1]), bf16x2(core[2], core[3]));
                    if (a.core_fp4) {
                        uint32_t w = 0u;
                        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, core[0], core[1], sc, 0);
                        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, core[2], core[3], sc, 1);
                        *(uint16_t*)(a.cq + off_fp4(B.k_first + cr, G, nks) + 2 * e) = (uint16_t)w;
                    } else {
                        v2s z = {0, 0};
                        const v2s lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, core[0], core[1], sc, false);
                        const v2s cd = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, core[2], core[3], sc, true);
                        *(uint32_t*)(cq_t + toff_fp8(kt, (int)(G >> 2), 2 * (int)(G & 3) + (e >> 2)) + 4 * (e & 3)) =
                            __builtin_bit_cast(uint32_t, cd);
                    }
                    if (e == 0) cs_t[toff_scale(kt, (int)G)] = (uint8_t)(ex + 127);
                }
                // deltas of the 8 rows (pad rows too: never read back as a
                // token's); lane e writes row e's scale code
                const int rt0 = (int)(B.slot0 & 255) + rb;     // the block's rows share one 256-row tile
                float am[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    am[j] = 0.0f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        xr[j][q] = xr[j][q] - core[q];
                        am[j] = fmaxf(am[j], fabsf(xr[j][q]));
                    }
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) am[j] = oct_max(am[j]);
                int exs = 0;
                uint32_t cd[8];                                // row j's codes of this eighth (2 bytes)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int ex = mx_exp_fp4(am[j]);
                    const float sc = pow2f(ex);
                    uint32_t w = 0u;
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xr[j][0], xr[j][1], sc, 0);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xr[j][2], xr[j][3], sc, 1);
                    cd[j] = w & 0xffffu;
                    exs = e == j ? ex : exs;
                }
                // Two exchanges inside the quad of eighths (e, e ^ 1, e ^ 2,
                // e ^ 3): at distance 1 a lane keeps the rows of its parity and
                // packs its eighth with the partner's (4 bytes), at distance 2
                // the rows whose bit 1 is its own and packs the two pairs (8
                // bytes).  Lane e then holds bytes 8 (e / 4) .. + 7 of rows
                // e % 4 and e % 4 + 4: two 8-byte stores instead of eight
                // 2-byte ones.
                const bool o1 = (e & 1) != 0, o2 = (e & 2) != 0;
                uint32_t d1[4];                                // row 2 m + e % 2, eighths 2 (e / 2), + 1
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const uint32_t send = o1 ? cd[2 * m] : cd[2 * m + 1];
                    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, true);   // lane ^ 1
                    const uint32_t own = o1 ? cd[2 * m + 1] : cd[2 * m];
                    d1[m] = o1 ? (recv | (own << 16)) : (own | (recv << 16));
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {                  // row 4 h + e % 4, eighths 4 (e / 4) .. + 3
                    const uint32_t send = o2 ? d1[2 * h] : d1[2 * h + 1];
                    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x4E, 0xF, 0xF, true);  // lane ^ 2
                    const uint32_t own = o2 ? d1[2 * h + 1] : d1[2 * h];
                    *(uint2*)(dq_t + toff_fp4(rt0 + 4 * h + (e & 3), (int)G) + 8 * (e >> 2)) =
                        o2 ? make_uint2(recv, own) : make_uint2(own, recv);
                }
                ds_t[toff_scale(rt0 + e, (int)G)] = (uint8_t)(exs + 127);
            }
        } else if (CM == 0 && g.S == 1) {
            // one-token cubes: the core is the token itself (x / 1, exact) and
            // every delta is 0 (not stored); one (row, group, quarter) per
            // thread codes the row, stores through the block's 256-row tile
            // (its 64 cubes start at a multiple of 64)
            for (int t = qtid; t < ntask; t += 256) {
                const int qq = t & 3, pr = t >> 2;
                const int cr = pr / NGC, gc = pr - cr * NGC;
                const int G = (c0 >> 5) + gc;
                if (G * 32 >= a.Ci) continue;                  // the same for the quad
                float v[8];
                qload8<XT>(buf, cr, gc, qq, 0u, v);
                float amax = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
                amax = core_pair_max<4>(quad_max(amax), a.core_g64);
                const int kt = (int)(B.k_first & 255) + cr;
                if (a.cbf)
                    *(uint4*)cbf_at(a.cbf, B.k_first + cr, G * 32 + 8 * qq, a.Kp) = make_uint4(bf16x2(v[0], v[1]), bf16x2(v[2], v[3]),
                                                                                         bf16x2(v[4], v[5]), bf16x2(v[6], v[7]));
                if (a.core_fp4) {
                    const int ex = mx_exp_fp4(amax);
                    const float sc = pow2f(ex);
                    uint32_t w = 0u;
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], sc, 0);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], sc, 1);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], sc, 2);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], sc, 3);
                    *(uint32_t*)(a.cq + off_fp4(B.k_first + cr, G, nks) + 4 * qq) = w;
                    if (qq == 0) cs_t[toff_scale(kt, G)] = (uint8_t)(ex + 127);
                } else {
                    const int ex = mx_exp_fp8(amax);
                    const float sc = pow2f(ex);
                    uint32_t d[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        v2s z = {0, 0};
                        v2s lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, v[4 * h], v[4 * h + 1], sc, false);
                        v2s hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, v[4 * h + 2], v[4 * h + 3], sc, true);
                        d[h] = __builtin_bit_cast(uint32_t, hi);
                    }
                    *(uint2*)(cq_t + toff_fp8(kt, G >> 2, 2 * (G & 3) + (qq >> 1)) + 8 * (qq & 1)) = make_uint2(d[0], d[1]);
                    if (qq == 0) cs_t[toff_scale(kt, G)] = (uint8_t)(ex + 127);
                }
            }
        } else {
            if (fast4) {
                // cubes of 4 slots, bf16 rows, FP8 cores without a bf16 copy:
                // thread t's (cube, group, quarter) is the same in every chunk
                // of every block, so its LDS and output offsets are fixed, up
                // to per-block parts (taken when the block changes) and the
                // chunk's K step (uniform)
                if (i != f4_block) {
                    f4_block = i;
                    const int rt0 = (int)(B.slot0 & 255) + 4 * f4_cr, kt = (int)(B.k_first & 255) + f4_cr;
                    f4_drow = toff_fp4(rt0 + f4_qq, f4_gc);
                    f4_ds = toff_scale(rt0 + f4_qq, f4_gc);
                    f4_cq = toff_fp8(kt, 0, 2 * f4_gc + (f4_qq >> 1)) + 8 * (f4_qq & 1);
                    f4_cs = toff_scale(kt, f4_gc);
                }
                if (qtid < ntask && c0 + 32 * f4_gc < a.Ci) task4(buf, B.part * nchunks + c, dq_t, ds_t, cq_t, cs_t);
            } else {
            for (int t = qtid; t < ntask; t += 256) {
                if (full) task(t, std::true_type{});
                else task(t, std::false_type{});
            }
            }
        }
        // the group's next chunk; a new block's metadata goes to the other
        // buffer now and is read after the next barrier
        const long long i_prev = i;
#pragma unroll
        for (int k = 0; k < SP; ++k) next_chunk();
        if (i != i_prev && i < nmine) {
            mb ^= 1;
            fill_meta(mb, i);
        }
    }
    }
}

// ---- cubes of more than 64 tokens: fp32 partial sums of 64-token blocks
struct PartialArgs {
    const void* x;
    Geom g;
    int Ci, Kp;
    long long nblk;
    float* part;   // [K*nblk][Kp]
};

// One workgroup per (cube, 64-token block) and 256 x EPT channels; each
// thread sums EPT channels (one 16-byte load per token) over the block's
// tokens in order, eight tokens' loads in flight.
template <typename XT>
__global__ __launch_bounds__(256) void k_core_partial(PartialArgs a) {
    constexpr int EPT = 16 / (int)sizeof(XT);      // channels per thread
    const Geom& g = a.g;
    long long kb = blockIdx.x;
    long long k = kb / a.nblk;
    long long b = kb - k * a.nblk;
    const int c = (blockIdx.y * 256 + threadIdx.x) * EPT;
    if (c >= a.Ci) return;                         // Ci is a multiple of 32: all EPT channels or none
    int ct, ch, cw;
    int cnt = cube_count(g, k, &ct, &ch, &cw);
    long long j0 = b * CORE_BLOCK;
    if (j0 >= cnt) return;
    int j1 = (int)min((long long)cnt, j0 + CORE_BLOCK);
    long long kw = k % g.Wc, kh = (k / g.Wc) % g.Hc, kt = k / ((long long)g.Wc * g.Hc);
    const XT* x = (const XT*)a.x;
    // tokens j0 .. j1 - 1 of the cube (lexicographic in the clipped cube),
    // summed in order per channel (the first one starts the sum)
    int dw = (int)(j0 % cw), dh = (int)((j0 / cw) % ch), dt = (int)(j0 / (cw * ch));
    const long long n0 = ((kt * g.t) * g.H + kh * g.h) * g.W + kw * g.w;   // token (0, 0, 0) of the cube
    float s[EPT];
    for (int j = (int)j0; j < j1; j += 8) {
        uint4 raw[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (j + q < j1) {
                const long long n = n0 + ((long long)dt * g.H + dh) * g.W + dw;
                raw[q] = *(const uint4*)(x + n * a.Ci + c);
                if (++dw == cw) {
                    dw = 0;
                    if (++dh == ch) {
                        dh = 0;
                        ++dt;
                    }
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (j + q >= j1) continue;
            float v[EPT];
            if constexpr (sizeof(XT) == 2) {
                const uint32_t d[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[2 * e] = __uint_as_float(d[e] << 16);
                    v[2 * e + 1] = __uint_as_float(d[e] & 0xffff0000u);
                }
            } else {
                v[0] = __uint_as_float(raw[q].x);
                v[1] = __uint_as_float(raw[q].y);
                v[2] = __uint_as_float(raw[q].z);
                v[3] = __uint_as_float(raw[q].w);
            }
#pragma unroll
            for (int e = 0; e < EPT; ++e) s[e] = (j + q == j0) ? v[e] : s[e] + v[e];
        }
    }
    float* out = a.part + kb * a.Kp + c;
#pragma unroll
    for (int e = 0; e < EPT; e += 4) *(float4*)(out + e) = make_float4(s[e], s[e + 1], s[e + 2], s[e + 3]);
}

struct CombineArgs {
    Geom g;
    int Ci, Kp;
    long long nblk;
    const float* part;
    float* coref;    // [K][Kp]
    uint8_t* cq;     // K_pad x Kp, step-major
    uint8_t* cs;     // K_pad x Kp/32, step-major
    int core_g64;    // one exponent per 64 channels
    int core_fp4;    // MX-FP4 cores (FP4 layout in cq)
    uint16_t* cbf;   // bf16 cores, step-major (off_bf16) (16-bit cores), else null
};

// core = fl32(sum of the block partials in block order / count), then FP8 codes.
__global__ __launch_bounds__(256) void k_core_combine(CombineArgs a) {
    __shared__ float tile[256];
    const Geom& g = a.g;
    long long k = blockIdx.x;
    int c = blockIdx.y * 256 + threadIdx.x;
    int ct, ch, cw;
    int cnt = cube_count(g, k, &ct, &ch, &cw);
    int nb = (cnt + CORE_BLOCK - 1) / CORE_BLOCK;
    float core = 0.0f;
    if (c < a.Ci) {
        const float* p = a.part + k * a.nblk * a.Kp + c;
        float s = p[0];
        int b = 1;
        for (; b + 64 <= nb; b += 64) {                   // in block order, 64 loads in flight (large cubes)
            float v[64];
#pragma unroll
            for (int q = 0; q < 64; ++q) v[q] = p[(long long)(b + q) * a.Kp];
#pragma unroll
            for (int q = 0; q < 64; ++q) s = s + v[q];
        }
        for (; b < nb; b += 16) {                         // the rest, sixteen loads in flight
            float v[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) v[q] = b + q < nb ? p[(long long)(b + q) * a.Kp] : 0.0f;
#pragma unroll
            for (int q = 0; q < 16; ++q)
                if (b + q < nb) s = s + v[q];
        }
        core = mean_div(s, cnt);
        a.coref[k * a.Kp + c] = core;
    }
    tile[threadIdx.x] = core;
    __syncthreads();
    int j = threadIdx.x;
    int cg = blockIdx.y * 256 + 32 * j;
    if (j < 8 && cg < a.Ci) {
        float v[32];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            v[i] = tile[32 * j + i];
            amax = fmaxf(amax, fabsf(v[i]));
        }
        if (a.core_g64)                                 // the other half of the 64-channel group
#pragma unroll
            for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(tile[32 * (j ^ 1) + i]));
        const long long G = cg >> 5, nks = a.Kp / 128;
        if (a.cbf)
#pragma unroll
            for (int i = 0; i < 32; i += 8)
                *(uint4*)cbf_at(a.cbf, k, cg + i, a.Kp) = make_uint4(bf16x2(v[i], v[i + 1]), bf16x2(v[i + 2], v[i + 3]),
                                                                  bf16x2(v[i + 4], v[i + 5]), bf16x2(v[i + 6], v[i + 7]));
        int e;
        if (a.core_fp4) {
            e = mx_exp_fp4(amax);
            *(uint4*)(a.cq + off_fp4(k, G, nks)) = encode_fp4x32(v, pow2f(e));
        } else {
            e = mx_exp_fp8(amax);
            uint4 lo, hi;
            encode_fp8x32(v, pow2f(e), lo, hi);
            *(uint4*)(a.cq + off_fp8(k, G >> 2, 2 * (int)(G & 3), nks)) = lo;
            *(uint4*)(a.cq + off_fp8(k, G >> 2, 2 * (int)(G & 3) + 1, nks)) = hi;
        }
        a.cs[off_scale(k, G, nks)] = (uint8_t)(e + 127);
    }
}

// ---- weight preparation: R^T = fl32(W^T - (L1 L2)^T), fp64 sum in rank order
template <typename WT>
__global__ __launch_bounds__(256) void k_residual(const WT* w, const uint16_t* l1, const uint16_t* l2,
                                                 long long Ci, long long Co, int rank, float* r) {
    long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= Ci * Co) return;
    long long j = idx / Ci, c = idx - j * Ci;
    double p = 0.0;
    for (int q = 0; q < rank; ++q)
        p += (double)bf16_to_f32(l1[c * rank + q]) * (double)bf16_to_f32(l2[(long long)q * Co + j]);
    double wv = (double)XTraits<WT>::f(w[idx]);
    r[idx] = (float)(wv - p);
}

// MX-FP4 encode of rows into the GEMM's step-major layout: one (row, 32-group) per thread.
__global__ __launch_bounds__(256) void k_encode_fp4_rows(const float* src, long long rows, long long cols,
                                                        long long ld_src, long long Kp, uint8_t* codes,
                                                        uint8_t* scales) {
    long long ng = cols / 32;
    long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * ng) return;
    long long rrow = idx / ng, grp = idx - rrow * ng;
    const float* p = src + rrow * ld_src + grp * 32;
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        v[i] = p[i];
        amax = fmaxf(amax, fabsf(v[i]));
    }
    int e = mx_exp_fp4(amax);
    *(uint4*)(codes + off_fp4(rrow, grp, Kp / 128)) = encode_fp4x32(v, pow2f(e));
    scales[off_scale(rrow, grp, Kp / 128)] = (uint8_t)(e + 127);
}

// ---- the 6-bit layers (text tokens: no cubes) ----
// MX-FP6 encode of rows (Q6(R) at weight preparation, Q6(X) per call) into
// the GEMM's step-major FP6 layout: one (row, 32-group) per thread; rows of
// `src` are `ld_src` elements apart.
template <typename ST>
__global__ __launch_bounds__(256) void k_encode_fp6(const ST* src, long long rows, long long cols, long long ld_src,
                                                   long long Kp, uint8_t* codes, uint8_t* scales, int e3m2) {
    const long long ng = cols / 32;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * ng) return;
    const long long rrow = idx / ng, grp = idx - rrow * ng;
    const ST* p = src + rrow * ld_src + grp * 32;
    float v[32];
    if constexpr (std::is_same<ST, float>::value) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 f = ((const float4*)p)[i];
            v[4 * i] = f.x;
            v[4 * i + 1] = f.y;
            v[4 * i + 2] = f.z;
            v[4 * i + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 b = ((const uint4*)p)[i];
            const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
                v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
            }
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const int e = mx_exp_fp6(amax, e3m2 != 0);
    uint32_t d[6];
    encode_fp6x32(v, pow2f(e), e3m2 != 0, d);
    const long long nks = Kp / 128;
#pragma unroll
    for (int i = 0; i < 3; ++i) *(uint2*)(codes + off_fp6(rrow, grp, i, nks)) = make_uint2(d[2 * i], d[2 * i + 1]);
    scales[off_scale(rrow, grp, nks)] = (uint8_t)(e + 127);
}

// U = bf16(bf16(X) L1) for text tokens, in two passes: partial sums over
// channel splits of USPLIT channels (one wave per (32 tokens, split):
// 32x32x16 bf16 MFMAs, D[rank][token], fp32 accumulation), then their sum in
// split order and the bf16 rounding.
constexpr int USPLIT = 256;
template <typename XT>
__global__ __launch_bounds__(64) void k_u_partial(const XT* x, long long N, int Ci, int Kp, const uint16_t* l1t,
                                                  int rp, float* part, long long Npad) {
    const int lane = threadIdx.x, l32 = lane & 31, g = lane >> 5;
    const long long n = (long long)blockIdx.x * 32 + l32;
    const bool live = n < N;
    const int c0 = blockIdx.y * USPLIT, c1 = min(Ci, c0 + USPLIT);
    const int nct = rp / 32;
    v16f acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = (v16f){};
    for (int c = c0; c < c1; c += 16) {
        uint4 xr = make_uint4(0u, 0u, 0u, 0u);           // bf16 of channels c + 8 g .. c + 8 g + 7 of token n
        if (live) {
            if constexpr (std::is_same<XT, float>::value) {
                const float4 f0 = *(const float4*)(x + n * Ci + c + 8 * g), f1 = *(const float4*)(x + n * Ci + c + 8 * g + 4);
                xr = make_uint4(bf16x2(f0.x, f0.y), bf16x2(f0.z, f0.w), bf16x2(f1.x, f1.y), bf16x2(f1.z, f1.w));
            } else {
                xr = *(const uint4*)(x + n * Ci + c + 8 * g);
            }
        }
        const v8bf xb = __builtin_bit_cast(v8bf, xr);
#pragma unroll
        for (int t = 0; t < 4; ++t)
            if (t < nct) {
                const v8bf a = __builtin_bit_cast(v8bf, *(const uint4*)(l1t + (long long)(t * 32 + l32) * Kp + c + 8 * g));
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xb, acc[t], 0, 0, 0);
            }
    }
    if (!live) return;
    float* dst = part + ((long long)blockIdx.y * Npad + n) * rp;
#pragma unroll
    for (int t = 0; t < 4; ++t)
        if (t < nct)
#pragma unroll
            for (int i = 0; i < 4; ++i)   // ranks t 32 + 8 i + 4 g .. + 3
                *(float4*)(dst + t * 32 + 8 * i + 4 * g) =
                    make_float4(acc[t][4 * i], acc[t][4 * i + 1], acc[t][4 * i + 2], acc[t][4 * i + 3]);
}

__global__ __launch_bounds__(256) void k_u_combine(const float* part, int nsplit, long long N, long long Npad, int rp,
                                                   uint16_t* u) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= N * rp) return;
    float s = part[idx];
    for (int k = 1; k < nsplit; ++k) s = s + part[(long long)k * Npad * rp + idx];
    u[idx] = bf16_rne(s);
}

hipError_t launch_encode_fp6(const void* src, int src_bf16, int64_t rows, int64_t cols, int64_t ld_src, int64_t Kp,
                             uint8_t* codes, uint8_t* scales, int e3m2, hipStream_t st) {
    const long long n = rows * (cols / 32);
    if (n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (src_bf16)
        k_encode_fp6<uint16_t><<<blocks, 256, 0, st>>>((const uint16_t*)src, rows, cols, ld_src, Kp, codes, scales, e3m2);
    else
        k_encode_fp6<float><<<blocks, 256, 0, st>>>((const float*)src, rows, cols, ld_src, Kp, codes, scales, e3m2);
    return hipGetLastError();
}

hipError_t launch_text_lowrank(const void* x, int x_bf16, int64_t N, int64_t Npad, int Ci, int Kp, const uint16_t* l1t,
                               int rp, float* part, uint16_t* u, hipStream_t st) {
    if (rp == 0 || N == 0) return hipSuccess;
    const int nsplit = (Ci + USPLIT - 1) / USPLIT;
    dim3 grid((unsigned)((N + 31) / 32), (unsigned)nsplit);
    if (x_bf16) k_u_partial<uint16_t><<<grid, 64, 0, st>>>((const uint16_t*)x, N, Ci, Kp, l1t, rp, part, Npad);
    else k_u_partial<float><<<grid, 64, 0, st>>>((const float*)x, N, Ci, Kp, l1t, rp, part, Npad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_u_combine<<<(unsigned)((N * rp + 255) / 256), 256, 0, st>>>(part, nsplit, N, Npad, rp, u);
    return hipGetLastError();
}

int text_lowrank_splits(int Ci) { return (Ci + USPLIT - 1) / USPLIT; }

// Q4(R) decoded to bf16 (exact: an FP4 value times a power of two), in the
// bf16 GEMM's step-major layout (off_bf16), for the bf16-core ablation.  One
// (row, 32-group) per thread.
__global__ __launch_bounds__(256) void k_decode_fp4_bf16(const uint8_t* codes, const uint8_t* scales, long long rows,
                                                        long long Kp, uint16_t* out) {
    const long long ng = Kp / 32, idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * ng) return;
    const long long r = idx / ng, G = idx - r * ng, nks = Kp / 128;
    const uint4 w = *(const uint4*)(codes + off_fp4(r, G, nks));
    const float sc = ldexpf(1.0f, (int)scales[off_scale(r, G, nks)] - 127);
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
    constexpr float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    uint32_t o[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t byte = (d[i >> 2] >> (8 * (i & 3))) & 255u;
        const float lo = ((byte & 8u) ? -1.0f : 1.0f) * mag[byte & 7u] * sc;
        const float hi = ((byte & 128u) ? -1.0f : 1.0f) * mag[(byte >> 4) & 7u] * sc;
        o[i] = bf16x2(lo, hi);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *(uint4*)((uint8_t*)out + off_bf16(r, G * 32 + 8 * i, Kp / 32)) = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
}

hipError_t launch_decode_fp4_bf16(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t Kp, uint16_t* out,
                                  hipStream_t st) {
    const long long n = rows * (Kp / 32);
    k_decode_fp4_bf16<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(codes, scales, rows, Kp, out);
    return hipGetLastError();
}

// Slot -> token table of the GEMM epilogue (-1 for pad slots).
__global__ __launch_bounds__(256) void k_slot_tokens(Geom g, long long tok0, int* stok, long long n) {
    long long s = (long long)blockIdx.x * 256 + threadIdx.x;
    if (s < n) {
        const long long t = s < g.Nslot ? slot_token(g, s) : -1;
        stok[s] = t >= 0 ? (int)(tok0 + t) : -1;
    }
}

// ------------------------------------------------------------ launchers ----
hipError_t launch_residual(const void* w_dev, int w_bf16, const uint16_t* l1_dev, const uint16_t* l2_dev,
                           int64_t Ci, int64_t Co, int rank, float* r_dev, hipStream_t st) {
    long long n = Ci * Co;
    unsigned blocks = (unsigned)((n + 255) / 256);
    if (w_bf16)
        k_residual<uint16_t><<<blocks, 256, 0, st>>>((const uint16_t*)w_dev, l1_dev, l2_dev, Ci, Co, rank, r_dev);
    else
        k_residual<float><<<blocks, 256, 0, st>>>((const float*)w_dev, l1_dev, l2_dev, Ci, Co, rank, r_dev);
    return hipGetLastError();
}

hipError_t launch_encode_fp4_rows(const float* src, int64_t rows, int64_t cols, int64_t ld_src, int64_t Kp,
                                  uint8_t* codes, uint8_t* scales, hipStream_t st) {
    long long n = rows * (cols / 32);
    unsigned blocks = (unsigned)((n + 255) / 256);
    k_encode_fp4_rows<<<blocks, 256, 0, st>>>(src, rows, cols, ld_src, Kp, codes, scales);
    return hipGetLastError();
}

// One frame segment: its geometry, and the buffers advanced to its first slot
// row and first cube row (whole 256-row tiles of the step-major layouts).
static hipError_t launch_quantize_segment(const dq_weights* w, const void* x, int x_bf16, dq_qact* q,
                                          const dq_segment& sg, hipStream_t st) {
    const Geom& g = sg.g;
    const size_t nks = (size_t)(q->Kp / 128);
    uint8_t* const cq = q->cq + (size_t)(sg.krow0 / 256) * nks * 32768;
    uint8_t* const cq4 = q->cq + (size_t)(sg.krow0 / 256) * nks * 16384;   // FP4 cores: 16 KB per tile step
    uint8_t* const cs = q->cs + (size_t)(sg.krow0 / 256) * nks * 1024;
    float* const coref = q->coref ? q->coref + sg.krow0 * q->Kp : nullptr;
    if (sg.core_mode == 1) {
        // (the partial-sum pass finds tokens from the segment's own grid)
        const void* xs = (const char*)x + (size_t)sg.tok0 * (size_t)q->Ci * (x_bf16 ? 2 : 4);
        PartialArgs pa{xs, g, (int)q->Ci, (int)q->Kp, sg.nblk, q->part};
        const int ept = x_bf16 ? 8 : 4;                // channels per thread (16-byte loads)
        dim3 grid((unsigned)(g.K * sg.nblk), (unsigned)((q->Ci + 256 * ept - 1) / (256 * ept)));
        if (x_bf16) k_core_partial<uint16_t><<<grid, 256, 0, st>>>(pa);
        else k_core_partial<float><<<grid, 256, 0, st>>>(pa);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        CombineArgs ca{g, (int)q->Ci, (int)q->Kp, sg.nblk, q->part, coref, q->core_bits == 4 ? cq4 : cq, cs,
                       q->core_group == 64, q->core_bits == 4, q->cbf ? q->cbf + sg.krow0 * q->Kp : nullptr};
        dim3 grid2((unsigned)g.K, (unsigned)((q->Ci + 255) / 256));
        k_core_combine<<<grid2, 256, 0, st>>>(ca);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    QuantArgs a{};
    a.x = x;                                           // rows by token number, through the slot table
    a.g = g;
    a.Ci = (int)q->Ci;
    a.Kp = (int)q->Kp;
    a.rp = q->rp;
    a.core_mode = sg.core_mode;
    a.dq = q->dq + (size_t)(sg.row0 / 256) * nks * 16384;
    a.ds = q->ds + (size_t)(sg.row0 / 256) * nks * 1024;
    a.cq = cq;
    a.cs = cs;
    a.u = q->u + sg.row0 * q->rp;
    a.l1t = w->l1t;
    a.coref = coref;
    a.zero = q->zero;
    a.stok = q->stok + sg.row0;
    a.core_g64 = q->core_group == 64;
    a.core_fp4 = q->core_bits == 4;
    a.cbf = q->cbf ? q->cbf + sg.krow0 * q->Kp : nullptr;
    if (a.core_fp4) a.cq = cq4;
    const long long cpb = QROWS / g.S;
    const long long nblocks = sg.core_mode == 0 ? (g.K + cpb - 1) / cpb : (g.Nslot + QROWS - 1) / QROWS;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    // few blocks: split their channel chunks over several workgroups (the U
    // partials then summed in part order below)
    const int cc = x_bf16 ? 128 : 64;                  // channels per chunk
    int kparts = quant_kparts(nblocks, (int)((q->Ci + cc - 1) / cc), cus);
    if (q->rp > 0 && !(q->upart && g.Nslot <= q->upart_rows)) kparts = 1;
    a.kparts = kparts;
    a.urows = g.Nslot;
    a.upart = q->upart;
    a.nblocks = nblocks * kparts;
    const unsigned blocks = (unsigned)std::min<long long>(a.nblocks, cus);   // persistent: one workgroup per CU
    const int nct = q->rp / 32;
    // one-pass quantizer for blocks of 7 or more cubes (a thread per (cube,
    // group, quarter)), with eighths instead of quarters for 8-token cubes;
    // a wave per cube for blocks of 4 to 6; two phases for blocks of at most
    // 3 and for cubes of more than 64 tokens (measured on the 720p FFN
    // layers: 8 cubes per block one-pass 0.43-0.48 ms, eighths 0.35,
    // two-phase 0.45, wave per cube 0.48; 4 cubes per block 0.79, 0.46, 0.41)
    const int cm = a.core_mode == 1 ? 1 : (g.S == 8 ? 4 : (cpb <= 3 ? 2 : (cpb <= 6 ? 3 : 0)));
    auto go = [&](auto XT_, auto NCT_) {
        using XT = decltype(XT_);
        constexpr int THREADS = QCfg<XT, decltype(NCT_)::value>::THREADS;
        if (cm == 0) k_quantize<XT, decltype(NCT_)::value, 0><<<blocks, THREADS, 0, st>>>(a);
        else if (cm == 1) k_quantize<XT, decltype(NCT_)::value, 1><<<blocks, THREADS, 0, st>>>(a);
        else if (cm == 2) k_quantize<XT, decltype(NCT_)::value, 2><<<blocks, THREADS, 0, st>>>(a);
        else if (cm == 3) k_quantize<XT, decltype(NCT_)::value, 3><<<blocks, THREADS, 0, st>>>(a);
        else k_quantize<XT, decltype(NCT_)::value, 4><<<blocks, THREADS, 0, st>>>(a);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    auto by_rank = [&](auto XT_) {
        switch (nct) {
            case 0: go(XT_, I0{}); break;
            case 1: go(XT_, I1{}); break;
            case 2: go(XT_, I2{}); break;
            case 3: go(XT_, I3{}); break;
            default: go(XT_, I4{}); break;
        }
    };
    if (x_bf16) by_rank(uint16_t{});
    else by_rank(float{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || kparts == 1 || q->rp == 0) return e;
    // U = bf16 of the parts' fp32 sums, added in part order
    k_u_combine<<<(unsigned)((g.Nslot * q->rp + 255) / 256), 256, 0, st>>>(q->upart, kparts, g.Nslot, g.Nslot, q->rp, a.u);
    return hipGetLastError();
}

hipError_t launch_quantize(const dq_weights* w, const void* x, int x_bf16, dq_qact* q, hipStream_t st) {
    for (int i = 0; i < q->nseg; ++i) {
        hipError_t e = launch_quantize_segment(w, x, x_bf16, q, q->seg[i], st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_slot_tokens(const Geom& g, int64_t tok0, int* stok, int64_t n, hipStream_t st) {
    k_slot_tokens<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(g, tok0, stok, n);
    return hipGetLastError();
}

}  // namespace dq
