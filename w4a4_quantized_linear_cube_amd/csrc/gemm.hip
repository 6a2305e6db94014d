// Scaled-MFMA GEMMs of the delta-W4A4 layer (gfx950).
//
// DeltaQuant notes, 关键设计 4 (the three-term equation):
//   y_n = U_n L2 + Q8(core_k(n)) Q4(R) + Q4(delta_n) Q4(R)
// The core term is one row per cube (the "dynamic token bias", broadcast to
// the cube's tokens); the delta term is one row per token.  Two launches of
// one kernel template: the core GEMM (FP8 E4M3 cores, one row per cube)
// writes the per-cube term; the delta GEMM (FP4 E2M1 deltas, one row per
// slot) adds U L2, adds its cube's core term in the epilogue and scatters rows
// to token order.  Both are V_MFMA_SCALE_F32_32X32X64_F8F6F4 contractions
// over Ci with the E8M0 block scales applied inside the instruction, fp32
// accumulation.
//
// Operand roles: the MFMA's A operand is Q4(R) (its rows are output
// channels) and its B operand is the activation (rows are slots or cubes), so
// the accumulator tile is the transposed output: each lane holds, for one
// token, runs of four consecutive output channels, which the epilogue writes
// as 16-byte stores straight into the token's output row.
//
// Work decomposition: a 256-thread workgroup computes a 256-channel x
// 256-slot tile; its four waves each own 128 x 128 (4 x 4 MFMA tiles of
// 32 x 32, 256 accumulator registers).
//
// Data movement: all operands are stored step-major (one tile's 256 rows x
// 128-channel K step is one contiguous block, 16-byte chunks pre-swizzled
// for conflict-free LDS reads), so a K step lands in LDS by plain 1 KB
// global_load_lds copies (no staging registers).  A ring of NS stages runs
// NS - 2 steps ahead of the MFMAs.  Each K step is two 64-channel halves; the
// fragments of one half are read from LDS while the MFMAs of the other half
// run, so MFMAs never wait for LDS, and one barrier per step hands a landed
// stage to all waves and frees the oldest one for the next copy.
//
// Tile order: workgroups are dispatched round-robin over the 8 XCDs; tile
// indices are remapped so the workgroups resident on one XCD at a time cover
// a compact block of 4 channel tiles x 8 slot tiles and share their operand
// steps in that XCD's L2.
#include <type_traits>

#include "dq_device.h"

namespace dq {

struct GemmArgs {
    const uint8_t* a;   // A = Q4(R) codes, step-major, rows = output channels
    const uint8_t* as;  // A scale codes, step-major
    const uint8_t* b;   // B = activation codes (FP4 deltas / FP8 cores), step-major
    const uint8_t* bs;  // B scale codes, step-major
    int nks;            // K steps (Kp / 128)
    int mtiles, ntiles; // 256-row tiles of A and of B
    float* c;           // plain store epilogue: c[b row][a row], leading dimension ldc
    long long ldc;
    float* y;           // token epilogue: y[token][channel], Co channels per row
    int Co;
    int vec4;           // y rows are 16-byte aligned (Co % 4 == 0, y 16-byte aligned)
    const int* stok;    // slot -> token (-1 for pad slots), Nslot_pad entries
    int S;              // slots per cube (rows below split)
    int split;          // first slot row of the second frame segment (its cube rows from ksplit,
    int S2, ksplit;     //   S2 slots per cube); past the last row if there is one segment
    int kmax;           // last cube row
    const float* bias;  // per-cube core term [K_pad][ldbias]
    long long ldbias;
    const uint16_t* u;     // [Nslot_pad][rp]
    const uint16_t* l2t;   // [Cop][rp]
    int rp;
    float* sink;        // 2 KB the token epilogue stores lanes without an output to (never read)
};

constexpr int EPI_STORE = 0;      // plain fp32 stores c[b row][a row]
constexpr int EPI_TOKENS = 1;     // low-rank branch + core term, rows scattered to token order
constexpr int EPI_TOKENS_Q = 2;   // the same for cubes of a multiple of 4 slots, rank 32, Co a multiple of 256

// Direct global -> LDS copies (global_load_lds, saddr form): lane i copies
// 16 (or 4) bytes from base + voff_i to LDS address m0 + 16 i (or 4 i), with
// m0 and base uniform over the wave.  Issued as inline assembly: the copies
// have no destination registers, and keeping them out of the compiler's
// wait-count bookkeeping is what lets the MFMAs run on one LDS stage while
// later stages land (the compiler would otherwise wait for every copy in
// flight before any LDS read).  Completion is awaited explicitly with
// wait_vm<> and a barrier before any wave reads a stage; the "memory" clobber
// keeps LDS accesses in program order around the copies.
// `base` and `lds` are wave-uniform by construction; readfirstlane states it.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    uint64_t v = (uint64_t)(uintptr_t)p;
    uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// `base` must come from uniform_ptr.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff),
                 "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff),
                 "s"(base) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// load at a 32-bit byte offset from a base pointer
template <class T>
__device__ __forceinline__ T ld_off(const void* base, uint32_t off) {
    return *(const T*)((const char*)base + off);
}

// value of lane J of each group of four lanes (DPP quad_perm broadcast).
// quad_perm never reads outside the quad, so the fill value (0, with
// bound_ctrl) is never used; being the identity of an add, it lets the
// compiler fold the broadcast into the add that consumes it (v_add_f32_dpp).
template <int J>
__device__ __forceinline__ float4 quad_bcast(float4 v) {
    auto b = [](float f) {   // quad_perm [J, J, J, J]
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, f), 0x55 * J, 0xF, 0xF, true));
    };
    return make_float4(b(v.x), b(v.y), b(v.z), b(v.w));
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in
// bits 15:14; expcnt 7 and lgkmcnt 15 mean no wait on those counters)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Persistent schedule.  Workgroup b runs on XCD b & 7 (dispatch is
// round-robin over the 8 XCDs) and takes the tiles of its XCD's share: XCD x
// owns tile indices [x per, (x + 1) per), and its workgroups walk them with
// stride G / 8, so the workgroups resident on one XCD at one time hold
// consecutive indices.  Index v -> (channel tile, slot tile) in groups of gm
// channel tiles x all slot tiles, column-major inside a group, so those
// resident workgroups cover a compact block of 4 channel tiles x 8 slot
// tiles and share their operand steps in the XCD's L2.  Long K loops (64 or
// more steps) take groups of 8 (a 8 x 4 block: fewer re-reads of the slot
// panels, whose steps are then the larger share of each tile's bytes; 2 %
// faster on a 108-step layer, 0.6-1.5 % slower on 40-step ones).
struct TileWalk {
    int x, y0, ystride, ylim, per, mt, nt, gm;
    __device__ int count() const { return y0 < ylim ? (ylim - y0 + ystride - 1) / ystride : 0; }
    __device__ void coords(int it, int* tm, int* tn) const {
        const int v = x * per + y0 + it * ystride;
        const int grp = v / (gm * nt);
        const int first = grp * gm;
        const int g = min(gm, mt - first);
        const int within = v - grp * gm * nt;
        *tm = first + within % g;
        *tn = within / g;
    }
};
__device__ __forceinline__ TileWalk tile_walk(int b, int G, int mt, int nt, int nks) {
    TileWalk w;
    w.gm = nks >= 64 ? 8 : 4;
    const int total = mt * nt;
    w.per = (total + 7) / 8;
    w.x = b & 7;
    w.y0 = b >> 3;
    w.ystride = G >> 3;
    w.ylim = min(w.per, total - w.x * w.per);
    w.mt = mt;
    w.nt = nt;
    return w;
}

// SMALLK: a K loop shorter than NS steps (the copy cursor may then run
// ahead of the MFMAs' tile from a tile's first step on, or several tiles
// ahead); that form recomputes the copy sources every step, the other one
// only once per tile.
template <int BFMT, int EPI, bool SMALLK>
__global__ __launch_bounds__(256, 1) void k_gemm(GemmArgs p) {
    constexpr int BROW = BFMT == FMT_FP4 ? 64 : 128;         // B bytes per row per K step
    constexpr int A_STEP = 256 * 64;                          // A bytes per tile step
    constexpr int B_STEP = 256 * BROW;
    constexpr int B_OFF = A_STEP;
    constexpr int SA_OFF = B_OFF + B_STEP;
    constexpr int SB_OFF = SA_OFF + 1024;
    constexpr int STAGE = SB_OFF + 1024;
    constexpr int NS = BFMT == FMT_FP4 ? 4 : 3;               // LDS stages in the ring
    constexpr int APC = A_STEP / 1024 / 4;                    // 1 KB copies per wave: A
    constexpr int BPC = B_STEP / 1024 / 4;                    //                       B
    constexpr int DMAS = APC + BPC + 2;                       // copies per wave per stage
    static_assert((NS - 2) * DMAS < 63, "vmcnt range");
    // With four stages a stage's copies go out in two halves: H1 of them in
    // phase 2 of one step, the rest in phase 1 of the next, so the copy
    // stream (and the wait to issue it) is spread over the whole step.
    constexpr bool SPLIT = NS >= 4;
    constexpr int H1 = SPLIT ? DMAS / 2 : DMAS;
    // Split copies sit after every third MFMA of a phase (phase 1 from MFMA
    // 0, phase 2 from MFMA 2), which measured faster than issuing them after
    // consecutive MFMAs; unsplit, copy j follows MFMA j.
    static_assert(!SPLIT || (3 * (DMAS - H1 - 1) < 16 && 2 + 3 * (H1 - 1) < 16), "copy slots");
    auto p1_copy = [](int i) { return SPLIT && i % 3 == 0 && i / 3 < DMAS - H1 ? H1 + i / 3 : -1; };
    auto p2_copy = [](int i) { return SPLIT ? (i >= 2 && (i - 2) % 3 == 0 && (i - 2) / 3 < H1 ? (i - 2) / 3 : -1) : (i < H1 ? i : -1); };
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int g = lane >> 5, l32 = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const TileWalk walk = tile_walk(blockIdx.x, gridDim.x, p.mtiles, p.ntiles, p.nks);
    const int ntiles = walk.count();
    if (ntiles == 0) return;
    const int nk = p.nks;
    const int nsteps = ntiles * nk;

    // ---- copies.  Global step s (over all of this workgroup's tiles) is
    // K step s % nk of tile s / nk; the issue cursor walks them in order.
    // Per-lane offsets are 32-bit; tile bases are uniform (scalar registers).
    const uint32_t lds0 = lds_addr(smem);
    const uint32_t va = (uint32_t)lane * 16 + wv * APC * 1024, vb = (uint32_t)lane * 16 + wv * BPC * 1024;
    const uint32_t vs = (uint32_t)lane * 4 + wv * 256;
    // The copy cursor (tile tf, K step kf) runs NS - 1 steps ahead of the
    // MFMAs.  Past the last step it stays on it: those surplus copies land in
    // buffers no step reads and keep the number of copies per step uniform.
    // The step body must stay free of branches (the compiler would move the
    // MFMAs across them), so the cursor advances by selects.
    int tf = 0, kf = 0;
    struct Src {
        const uint8_t *a, *b, *as, *bs;
    };
    auto src_of = [&](int t, int k) {
        int tm, tn;
        walk.coords(t, &tm, &tn);
        Src r;
        r.a = (const uint8_t*)uniform_ptr(p.a + ((size_t)tm * p.nks + k) * A_STEP);
        r.b = (const uint8_t*)uniform_ptr(p.b + ((size_t)tn * p.nks + k) * B_STEP);
        r.as = (const uint8_t*)uniform_ptr(p.as + ((size_t)tm * p.nks + k) * 1024);
        r.bs = (const uint8_t*)uniform_ptr(p.bs + ((size_t)tn * p.nks + k) * 1024);
        return r;
    };
    // copy number j (0 .. DMAS - 1) of a step into LDS buffer buf
    auto dma = [&](const Src& src, int buf, int j) {
        const uint32_t st = lds0 + buf * STAGE;
        if (j < APC) {
            dma16(src.a, va + j * 1024, st + (wv * APC + j) * 1024);
        } else if (j < APC + BPC) {
            const int jb = j - APC;
            dma16(src.b, vb + jb * 1024, st + B_OFF + (wv * BPC + jb) * 1024);
        } else if (j == APC + BPC) {
            dma4(src.as, vs, st + SA_OFF + wv * 256);
        } else {
            dma4(src.bs, vs, st + SB_OFF + wv * 256);
        }
    };
    // Cursor advance.  General form: recompute from (tf, kf).  Otherwise
    // (nk >= NS) the cursor is in the MFMAs' tile it when that tile starts and
    // wraps into tile it + 1 at step nk - NS: pointer increments inside a
    // tile, and at the wrap the sources of the next tile's first step
    // (prepared at the start of tile it in `nsrc`; for the last tile, its own
    // last step with zero increments, `ninc` = 0).
    Src src = src_of(0, 0), nsrc{};
    int inc = 1, ninc = 1;
    auto advance = [&]() {
        const bool wrap = kf + 1 == nk;
        const bool stay = wrap && tf + 1 == ntiles;
        if constexpr (SMALLK) {
            kf = stay ? kf : (wrap ? 0 : kf + 1);
            tf = (wrap && !stay) ? tf + 1 : tf;
            src = src_of(tf, kf);
        } else {
            kf = wrap ? 0 : kf + 1;
            src.a = wrap ? nsrc.a : src.a + inc * A_STEP;
            src.b = wrap ? nsrc.b : src.b + inc * B_STEP;
            src.as = wrap ? nsrc.as : src.as + inc * 1024;
            src.bs = wrap ? nsrc.bs : src.bs + inc * 1024;
            inc = wrap ? ninc : inc;
        }
    };
    auto prepare_next = [&](int it) {                  // tile it + 1 (or the clamp), for the cursor's wrap
        if constexpr (!SMALLK) {
            if (it + 1 < ntiles) {
                nsrc = src_of(it + 1, 0);
                ninc = 1;
            } else {
                nsrc = src_of(ntiles - 1, nk - 1);
                ninc = 0;
            }
        }
    };

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (v16f){};

    // ---- fragments of one 64-channel half step, byte addresses within a stage
    const int arow0 = wr * 128 + l32;            // + 32 mi
    const int brow0 = wc * 128 + l32;            // + 32 ni
    const int asw = swz4(arow0);                 // the swizzles depend on row % 16 only
    const int bsw = BFMT == FMT_FP4 ? swz4(brow0) : swz8(brow0);
    // Scale codes: one 8-byte read per operand gives the lane's codes for the
    // whole step (four 32-row blocks x two halves); code (block r, half kk) is
    // byte 2 (r % 2) + kk of dword r / 2, selected by the MFMA's op_sel.
    const int sa_off = SA_OFF + ((wr * 2 + g) * 32 + l32) * 8;
    const int sb_off = SB_OFF + ((wc * 2 + g) * 32 + l32) * 8;
    struct Half {
        uint4 a[4];
        uint4 b[BFMT == FMT_FP4 ? 4 : 1];      // FP4 B fragments
        v8i b8[BFMT == FMT_FP4 ? 1 : 4];       // FP8 B fragments (two 16-byte chunks each)
        uint2 sa, sb;
    };
    // LDS read number i (0 .. 9) of half kk's fragments, in the order of
    // their first use by the MFMA sequence below: a0 b0 sa sb b1 b2 b3 a1 a2 a3.
    auto rd = [&](int buf, int kk, Half& F, int i) {
        const uint8_t* st = smem + buf * STAGE;
        auto rda = [&](int mi) { F.a[mi] = *(const uint4*)(st + (arow0 + 32 * mi) * 64 + (((2 * kk + g) ^ asw) << 4)); };
        auto rdb = [&](int ni) {
            const uint8_t* rowp = st + B_OFF + (brow0 + 32 * ni) * BROW;
            if constexpr (BFMT == FMT_FP4) {
                F.b[ni] = *(const uint4*)(rowp + (((2 * kk + g) ^ bsw) << 4));
            } else {
                const v4i lo = *(const v4i*)(rowp + (((4 * kk + g) ^ bsw) << 4));
                const v4i hi = *(const v4i*)(rowp + (((4 * kk + 2 + g) ^ bsw) << 4));
                F.b8[ni] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        };
        switch (i) {
            case 0: rda(0); break;
            case 1: rdb(0); break;
            case 2: F.sa = *(const uint2*)(st + sa_off); break;
            case 3: F.sb = *(const uint2*)(st + sb_off); break;
            case 4: rdb(1); break;
            case 5: rdb(2); break;
            case 6: rdb(3); break;
            case 7: rda(1); break;
            case 8: rda(2); break;
            default: rda(3); break;
        }
    };
    constexpr int NRD = 10;                      // LDS reads per half step
    // MFMA number i (0 .. 15) of half kk: row block mi = i / 4, column block ni = i % 4
    auto mma = [&](const Half& F, int kk, int i) {
        const int mi = i >> 2, ni = i & 3;
        const uint4 v = F.a[mi];
        const v8i af = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        v8i bf;
        if constexpr (BFMT == FMT_FP4) {
            const uint4 u = F.b[ni];
            bf = (v8i){(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
        } else {
            bf = F.b8[ni];
        }
        const int sa = (mi >> 1) ? (int)F.sa.y : (int)F.sa.x, sb = (ni >> 1) ? (int)F.sb.y : (int)F.sb.x;
        // op_sel operands must be constants: spell out the byte choices
#define DQ_MFMA(OA, OB) acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, acc[mi][ni], FMT_FP4, BFMT, OA, sa, OB, sb)
        const int oa = 2 * (mi & 1) + kk, ob = 2 * (ni & 1) + kk;
        switch (oa * 4 + ob) {
            case 0: DQ_MFMA(0, 0); break;   case 1: DQ_MFMA(0, 1); break;   case 2: DQ_MFMA(0, 2); break;   case 3: DQ_MFMA(0, 3); break;
            case 4: DQ_MFMA(1, 0); break;   case 5: DQ_MFMA(1, 1); break;   case 6: DQ_MFMA(1, 2); break;   case 7: DQ_MFMA(1, 3); break;
            case 8: DQ_MFMA(2, 0); break;   case 9: DQ_MFMA(2, 1); break;   case 10: DQ_MFMA(2, 2); break;  case 11: DQ_MFMA(2, 3); break;
            case 12: DQ_MFMA(3, 0); break;  case 13: DQ_MFMA(3, 1); break;  case 14: DQ_MFMA(3, 2); break;  default: DQ_MFMA(3, 3); break;
        }
#undef DQ_MFMA
    };

    // ---- output transposition.  An accumulator block holds, per lane, 16
    // channels of one B row in 16-byte pieces 8 channels apart, so direct
    // stores would write 32 rows x 32 bytes per instruction.  Each wave
    // passes its blocks through two 4 KB LDS buffers (32 rows x 128 bytes,
    // pieces XOR-swizzled by row: conflict-free both ways) and reads them
    // back as 8 rows x 128 contiguous bytes per instruction.  The buffers sit
    // in the stage of the tile's last K step, which no wave reads after the
    // epilogue's first barrier and no copy fills before the next tile's first
    // barrier.
    int tstage = 0;                                       // stage of the tile's last K step

    // ---- core-term rows of the token epilogue.  A cube spans a multiple of
    // 4 slots and tiles and frame segments start at multiples of 256 rows, so the four lanes of a quad
    // hold slots of one cube; lane u of the quad loads the quarter of the
    // cube's row that is piece (mi, u) of every lane's 16 pieces, and the
    // epilogue exchanges the quarters by DPP broadcasts.  They are loaded
    // CORE_AHEAD steps before the tile's K loop ends (at its start if K is
    // shorter): issued ahead of the last steps' copies, they have landed when
    // the epilogue starts instead of queueing behind those copies.
    // (32-bit byte offsets from the uniform base: one address register per
    // row, the rest in the instructions' offset fields; each element is read
    // once, so the loads allocate no cache lines.)
    constexpr int CORE_AHEAD = 6;
    // cube row of slot row sl (pad slots: some valid row, never stored)
    auto cube_row = [&](int sl) {
        const int k = sl < p.split ? sl / p.S : p.ksplit + (sl - p.split) / p.S2;
        return min(k, p.kmax);
    };
    float4 bq[4][4];
    auto load_core = [&](int tm, int tn) {
        const uint32_t chq0 = (uint32_t)(tm * 256 + wr * 128 + 4 * g + 8 * (l32 & 3));
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const int k = cube_row(tn * 256 + wc * 128 + 32 * ni + l32);
            const uint32_t bo = ((uint32_t)k * (uint32_t)p.ldbias + chq0) * 4;
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                bq[ni][mi] = __builtin_bit_cast(float4, __builtin_nontemporal_load((const v4f*)((const char*)p.bias + bo + 128 * mi)));
        }
    };
    auto tbuf = [&](int b) { return smem + tstage * STAGE + wv * 8192 + b * 4096; };
    auto tput = [&](int b, const float4* o) {           // piece j of this lane's row l32 is channels 8 j + 4 g ..
        uint8_t* t = tbuf(b) + l32 * 128;
#pragma unroll
        for (int j = 0; j < 4; ++j) *(float4*)(t + (((2 * j + g) ^ ((l32 >> 1) & 7)) << 4)) = o[j];
    };
    auto tget = [&](int b, int i) {                     // row 8 i + lane / 8, channels 4 (lane % 8) ..
        const int rr = 8 * i + (lane >> 3);
        return *(const float4*)(tbuf(b) + rr * 128 + (((lane & 7) ^ ((rr >> 1) & 7)) << 4));
    };

    // ---- tile epilogue: acc[mi][ni][4 j + q] is channel m0 + wr 128 + 32 mi
    // + 8 j + 4 g + q of B row n0 + wc 128 + 32 ni + l32.
    auto epilogue = [&](int tm, int tn) {
        const int m0 = tm * 256, n0 = tn * 256;
        const int ch0 = m0 + wr * 128 + 4 * g;             // + 32 mi + 8 j
        if constexpr (EPI == EPI_STORE) {
            __syncthreads();                                // every wave is done with the last step's stage
#pragma unroll
            for (int b = 0; b < 17; ++b) {
                if (b < 16) {                               // block b: mi = b % 4, ni = b / 4
                    const v16f& a = acc[b & 3][b >> 2];
                    float4 o[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) o[j] = make_float4(a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]);
                    tput(b & 1, o);
                }
                if (b > 0) {
                    const int pb = b - 1, mi = pb & 3, ni = pb >> 2;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = 8 * i + (lane >> 3);
                        const float4 v = tget(pb & 1, i);
                        __builtin_nontemporal_store(__builtin_bit_cast(v4f, v),   // read once, by the delta GEMM
                                                    (v4f*)(p.c + (long long)(n0 + wc * 128 + 32 * ni + rr) * p.ldc + m0 + wr * 128 + 32 * mi + 4 * (lane & 7)));
                    }
                }
            }
            return;
        }
        if constexpr (EPI == EPI_TOKENS_Q) {
            // Every global load is issued before the first wait, so their
            // latencies (and that of the copies still in flight) overlap: the
            // slot -> token map and the low-rank operands (the core-term rows,
            // bq, were loaded during the K loop).
            // (32-bit byte offsets from the uniform bases: one address register
            // per row, the rest in the instructions' offset fields)
            int tok[4];
            v8bf la[2][4], ub[2][4];
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) tok[ni] = ld_off<int>(p.stok, (uint32_t)(n0 + wc * 128 + 32 * ni + l32) * 4);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const uint32_t lo = ((uint32_t)(m0 + wr * 128 + l32 + 32 * mi) * 32 + 8 * g) * 2;
                la[0][mi] = __builtin_bit_cast(v8bf, ld_off<uint4>(p.l2t, lo));
                la[1][mi] = __builtin_bit_cast(v8bf, ld_off<uint4>(p.l2t, lo + 32));
            }
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const uint32_t uo = ((uint32_t)(n0 + wc * 128 + l32 + 32 * ni) * 32 + 8 * g) * 2;
                ub[0][ni] = __builtin_bit_cast(v8bf, ld_off<uint4>(p.u, uo));
                ub[1][ni] = __builtin_bit_cast(v8bf, ld_off<uint4>(p.u, uo + 32));
            }
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();                                // every wave is done with the last step's stage
            // the copies of the next tile's first stages land before the next
            // tile reads them (its first steps wait loosely)
            wait_vm<0>();
            // low-rank branch: acc += (U L2)^T, 32x32x16 bf16 MFMAs over the 32 ranks
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[h][mi], ub[h][ni], acc[mi][ni], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            // y[token] = acc + core term of the token's cube, through the
            // transposition buffers.  The broadcasts run in every lane (a pad
            // slot's lane still serves its quad); a row is stored if its slot
            // holds a token.  (Co is a multiple of 256 here: every channel of
            // the tile exists.)
            const int chq = m0 + wr * 128 + 4 * (lane & 7);   // this lane's channels after the transposition (+ 32 mi)
            float* rowp[4];
#pragma unroll
            for (int b = 0; b < 17; ++b) {
                if (b < 16) {                               // block b: mi = b % 4, ni = b / 4
                    const int mi = b & 3, ni = b >> 2;
                    const v16f& a = acc[mi][ni];
                    float4 bv[4], o[4];
                    bv[0] = quad_bcast<0>(bq[ni][mi]);     // piece (mi, j) comes from quad lane j
                    bv[1] = quad_bcast<1>(bq[ni][mi]);
                    bv[2] = quad_bcast<2>(bq[ni][mi]);
                    bv[3] = quad_bcast<3>(bq[ni][mi]);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        o[j] = make_float4(a[4 * j] + bv[j].x, a[4 * j + 1] + bv[j].y, a[4 * j + 2] + bv[j].z,
                                           a[4 * j + 3] + bv[j].w);
                    tput(b & 1, o);
                }
                if (b > 0) {
                    // rows 8 i + lane / 8 of block b - 1.  A row's destination
                    // (its token's y row, or the sink for a slot without a
                    // token) is the same for the four blocks of one ni: found
                    // once, at mi = 0, and offset by 32 mi channels (the
                    // stores' immediate offsets).  Every lane stores, so no
                    // branch splits the LDS reads and their waits.
                    const int pb = b - 1, mi = pb & 3, ni = pb >> 2;
                    if (mi == 0) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int t = __builtin_amdgcn_ds_bpermute((8 * i + (lane >> 3)) * 4, tok[ni]);   // token of row rr (lane rr)
                            float* yrow = p.y + (uint32_t)(t * p.Co + chq);
                            rowp[i] = t >= 0 ? yrow : p.sink + 4 * lane;
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float4 v = tget(pb & 1, i);
                        __builtin_nontemporal_store(__builtin_bit_cast(v4f, v), (v4f*)(rowp[i] + 32 * mi));   // y is not read back
                    }
                }
            }
            return;
        }
        // low-rank branch: acc += (U L2)^T with 32x32x16 bf16 MFMAs over the padded rank
        for (int kq = 0; kq < p.rp; kq += 16) {
            v8bf la[4], ub[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const long long ch = m0 + wr * 128 + l32 + 32 * mi;
                la[mi] = __builtin_bit_cast(v8bf, *(const uint4*)(p.l2t + ch * p.rp + kq + 8 * g));
            }
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const long long slot = n0 + wc * 128 + l32 + 32 * ni;
                ub[ni] = __builtin_bit_cast(v8bf, *(const uint4*)(p.u + slot * p.rp + kq + 8 * g));
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[mi], ub[ni], acc[mi][ni], 0, 0, 0);
        }
        // y[token] = acc + core term of the token's cube (16-byte loads of the
        // cube's row of the per-cube term, 16-byte stores into the token's row)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const int slot = n0 + wc * 128 + 32 * ni + l32;
            const int tok = p.stok[slot];
            const int k = cube_row(slot);
            float4 bv[4][4];
            if (p.bias) {
                const float* brow = p.bias + (long long)k * p.ldbias + ch0;
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int j = 0; j < 4; ++j) bv[mi][j] = *(const float4*)(brow + 32 * mi + 8 * j);
            } else {                                        // no per-cube term
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int j = 0; j < 4; ++j) bv[mi][j] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            if (tok < 0) continue;
            float* yrow = p.y + (long long)tok * p.Co;
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const v16f& a = acc[mi][ni];
                    const float4 o = make_float4(a[4 * j] + bv[mi][j].x, a[4 * j + 1] + bv[mi][j].y,
                                                 a[4 * j + 2] + bv[mi][j].z, a[4 * j + 3] + bv[mi][j].w);
                    const int ch = ch0 + 32 * mi + 8 * j;
                    if (p.vec4 && ch + 4 <= p.Co) {
                        __builtin_nontemporal_store(__builtin_bit_cast(v4f, o), (v4f*)(yrow + ch));
                    } else {
                        if (ch < p.Co) yrow[ch] = o.x;
                        if (ch + 1 < p.Co) yrow[ch + 1] = o.y;
                        if (ch + 2 < p.Co) yrow[ch + 2] = o.z;
                        if (ch + 3 < p.Co) yrow[ch + 3] = o.w;
                    }
                }
        }
    };

    // ---- K loop over all global steps.  Step gs has two phases of 16 MFMAs,
    // every MFMA followed by its companions (kept in place by scheduling
    // barriers):
    //   phase 1: MFMAs of half 0 of stage gs (fragments F0); companions read
    //            half 1 of stage gs into F1;
    //   then wait for this wave's copies of stage gs + 1 and barrier: all
    //            copies of gs + 1 have landed, and every wave is done with
    //            stage gs - 1, whose buffer takes the copies of gs + NS - 1;
    //   phase 2: MFMAs of half 1 (F1); companions issue the copies of stage
    //            gs + NS - 1 (possibly the next tile's) and read half 0 of
    //            stage gs + 1 into F0.
    // After the last step of a tile: wait for every copy in flight, then the
    // epilogue (whose stores drain while the next tile runs), clear acc and
    // read half 0 of the next tile's first stage.
    // Fragments are read one phase before their MFMAs, so LDS latency hides
    // behind 16 MFMAs.
    // Prologue: stages 0 .. NS - 2 (the last of them only its first half
    // when split; the cursor then stays on it).
    for (int s = 0; s < NS - 1; ++s) {
        const bool half = SPLIT && s == NS - 2;
#pragma unroll
        for (int j = 0; j < DMAS; ++j)
            if (!half || j < H1) dma(src, s, j);
        if (!half) advance();
    }
    wait_vm<(NS - 2) * DMAS - (DMAS - H1)>();                  // stage 0 landed
    __syncthreads();
    Half F0, F1;
#pragma unroll
    for (int i = 0; i < NRD; ++i) rd(0, 0, F0, i);
    // Stage gs + 1 must have landed before the barrier of step gs.  Copies go
    // out every step (past the end too), so normally NS - 3 later stages may
    // still be in flight (split: the copies issued after stage gs + 1's last
    // half are the two halves of stage gs + 2, the same count).  In a tile's
    // first NS - 2 steps (split: NS - 3) after the first tile, stage gs + 1
    // was issued in full before the previous tile's epilogue, whose full wait
    // already covered it; a loose count there lets the epilogue's stores stay
    // in flight.  Half 0 of stage gs + 1 is read in every step, at a tile's
    // last step too (it is the next tile's first stage).
    int gs = 0;
    for (int it = 0; it < ntiles; ++it) {
        prepare_next(it);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = (v16f){};
        auto kstep = [&](int ks) __attribute__((always_inline)) {
            const int cur = (unsigned)gs % NS, nxt = (unsigned)(gs + 1) % NS, fill = (unsigned)(gs + NS - 1) % NS;
            const int fillp = (unsigned)(gs + NS - 2) % NS;   // the cursor's stage in phase 1 (its second half)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                mma(F0, 0, i);
                if (i < NRD) rd(cur, 1, F1, i);
                if (p1_copy(i) >= 0) dma(src, fillp, p1_copy(i));
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (SPLIT) advance();
            // Wait and barrier in one asm block (no branch for the compiler to
            // move code across).  Every wave's reads of stage gs - 1 completed
            // before its MFMAs of step gs - 1, so a bare barrier suffices; the
            // memory clobber keeps the LDS reads below it.
            const int loose = __builtin_amdgcn_readfirstlane((it > 0 && ks < NS - 2 - (SPLIT ? 1 : 0)) ? 1 : 0);
            asm volatile(
                "s_cmp_eq_u32 %0, 0\n\t"
                "s_cbranch_scc1 1f\n\t"
                "s_waitcnt vmcnt(63)\n\t"
                "s_branch 2f\n"
                "1:\n\t"
                "s_waitcnt vmcnt(%1)\n"
                "2:\n\t"
                "s_barrier" ::"s"(loose), "n"((NS - 3) * DMAS) : "memory", "scc");
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                mma(F1, 1, i);
                if (p2_copy(i) >= 0) dma(src, fill, p2_copy(i));
                if (i < NRD) rd(nxt, 0, F0, i);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (!SPLIT) advance();
        };
        int ks = 0;
        if constexpr (EPI == EPI_TOKENS_Q) {
            for (; ks < nk - CORE_AHEAD; ++ks, ++gs) kstep(ks);
            if (p.bias) {
                int tm, tn;
                walk.coords(it, &tm, &tn);
                load_core(tm, tn);
            } else {                                       // no per-cube term: add zeros
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) bq[i][j] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        for (; ks < nk; ++ks, ++gs) kstep(ks);
        if (EPI != EPI_TOKENS_Q) wait_vm<0>();   // that epilogue waits after issuing its loads
        int tm, tn;
        walk.coords(it, &tm, &tn);
        tstage = (unsigned)(gs - 1) % NS;
        epilogue(tm, tn);
        // The last step already read half 0 of the next tile's first stage
        // (landed: its barrier covered it); reading it again here keeps those
        // registers free during the epilogue.
#pragma unroll
        for (int i = 0; i < NRD; ++i) rd((unsigned)gs % NS, 0, F0, i);
    }
}

// One persistent workgroup per CU (a multiple of 8, one share per XCD),
// never more than the tiles need.
static int persistent_grid(int total) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    int grid = max(8, cus / 8 * 8);
    return min(grid, (total + 7) / 8 * 8);
}

template <int BFMT, int EPI>
static hipError_t launch(const GemmArgs& a, hipStream_t st) {
    constexpr int NS = BFMT == FMT_FP4 ? 4 : 3;      // the kernel's LDS stages
    const int grid = persistent_grid(a.mtiles * a.ntiles);
    if (a.nks < NS) k_gemm<BFMT, EPI, true><<<grid, 256, 0, st>>>(a);
    else k_gemm<BFMT, EPI, false><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_forward(const dq_weights* w, dq_qact* q, float* y, int parts, hipStream_t st) {
    GemmArgs d{};
    d.a = w->rq;
    d.as = w->rs;
    d.nks = (int)(w->Kp / 128);
    d.mtiles = (int)(w->Cop / 256);
    d.b = q->dq;
    d.bs = q->ds;
    d.ntiles = (int)(q->Nslot_pad / 256);
    d.y = y;
    d.Co = (int)w->Co;
    d.vec4 = (w->Co % 4 == 0) && ((uintptr_t)y % 16 == 0);
    d.stok = q->stok;
    d.S = q->seg[0].g.S;
    d.split = q->nseg > 1 ? (int)q->seg[1].row0 : (int)q->Nslot_pad;
    d.S2 = q->seg[q->nseg - 1].g.S;
    d.ksplit = (int)q->seg[q->nseg - 1].krow0;
    d.kmax = (int)(q->K_pad - 1);
    d.u = q->u;
    d.l2t = w->l2t;
    d.rp = w->rp;
    d.sink = q->sink;
    // (32-bit element offsets into y and into the per-cube term)
    const bool off32 = q->g.N * w->Co < (1ll << 31) && q->K_pad * w->Cop * 4 < (1ll << 32);
    if (q->g.S == 1 && q->core_bits != 16) {
        // One-token cubes: every delta is x - x = 0 exactly, so y = Q8(x) Q4(R)
        // + U L2 (Q4(x) for 4-bit cores), one GEMM over the cubes (cube k is
        // slot k) with the token epilogue and no per-cube term.  It is the delta half's work; the
        // core half has nothing to do.
        if (!(parts & FWD_DELTA)) return hipSuccess;
        d.b = q->cq;
        d.bs = q->cs;
        d.ntiles = (int)(q->K_pad / 256);
        d.bias = nullptr;
        if (q->core_bits == 4) {
            if (d.rp == 32 && d.vec4 && off32 && d.Co % 256 == 0) return launch<FMT_FP4, EPI_TOKENS_Q>(d, st);
            return launch<FMT_FP4, EPI_TOKENS>(d, st);
        }
        if (d.rp == 32 && d.vec4 && off32 && d.Co % 256 == 0) return launch<FMT_FP8, EPI_TOKENS_Q>(d, st);
        return launch<FMT_FP8, EPI_TOKENS>(d, st);
    }
    if (parts & FWD_CORE) {
        // per-cube core term bias[k] = Q8(core_k) Q4(R) (Q4(core_k) for 4-bit cores)
        GemmArgs c = d;
        c.b = q->cq;
        c.bs = q->cs;
        c.ntiles = (int)(q->K_pad / 256);
        c.c = q->bias;
        c.ldc = w->Cop;
        hipError_t e = q->core_bits == 4 ? launch<FMT_FP4, EPI_STORE>(c, st) : launch<FMT_FP8, EPI_STORE>(c, st);
        if (e != hipSuccess) return e;
    }
    if (parts & FWD_DELTA) {
        // delta term + low-rank branch + the cube's core term -> y (token order)
        d.bias = q->bias;
        d.ldbias = w->Cop;
        if (d.S % 4 == 0 && d.S2 % 4 == 0 && d.rp == 32 && d.vec4 && off32 && d.Co % 256 == 0)
            return launch<FMT_FP4, EPI_TOKENS_Q>(d, st);
        return launch<FMT_FP4, EPI_TOKENS>(d, st);
    }
    return hipSuccess;
}

}  // namespace dq
