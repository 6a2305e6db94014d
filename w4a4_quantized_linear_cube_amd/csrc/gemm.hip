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
// accumulation.  The core GEMM's last, partly filled round may run split
// along K: K-chunk units write fp32 partials that k_ksum adds in order.
//
// Operand roles: the MFMA's A operand is Q4(R) (its rows are output
// channels) and its B operand is the activation (rows are slots or cubes), so
// the accumulator tile is the transposed output: each lane holds, for one
// token, runs of four consecutive output channels.  The epilogues pass them
// through LDS and store 128-byte row segments (the general token epilogue
// stores the 16-byte runs directly).
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
#include <algorithm>
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
    const float* xscale;   // general token epilogue: y = (acc x xscale[slot]) x wscale[channel] when set
    const float* wscale;   //   (the rotated-basis layers' per-row scales), [Nslot_pad] and [Cop]
    // K split of the plain-store GEMM's last round (KSplit).  ttotal > 0:
    // run only walk tiles 0 .. ttotal - 1.  su_rm > 0: workgroup u runs K
    // steps [c nks / su_p, (c + 1) nks / su_p), c = u / su_rm, of walk tile
    // su_v0 + u % su_rm and stores the 256 x 256 partial at c + u 65536.
    int ttotal;
    int su_v0, su_rm, su_p;
};

constexpr int EPI_STORE = 0;      // plain fp32 stores c[b row][a row]
constexpr int EPI_TOKENS = 1;     // low-rank branch + core term, rows scattered to token order
constexpr int EPI_TOKENS_Q = 2;   // the same for cubes of a multiple of 4 slots, rank 32, Co a multiple of 256
constexpr int EPI_ROWS_Q = 3;     // y[row] = (acc x xscale[row]) x wscale[channel]: rows in order, Co a multiple of 256

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
// The same with an immediate byte offset OFF (0 .. 4095) on the source:
// base + voff_i + OFF -> LDS lds + 16 i.  The instruction's offset field is
// added to the LDS address as well as to the global one, so m0 takes
// lds - OFF (lds >= OFF).
template <int OFF>
__device__ __forceinline__ void dma16o(const void* base, uint32_t voff, uint32_t lds) {
    static_assert(OFF >= 0 && OFF < 4096, "offset field");
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%3" ::"s"(__builtin_amdgcn_readfirstlane(lds - OFF)),
                 "v"(voff), "s"(base), "n"(OFF) : "memory", "m0");
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
// round-robin over the 8 XCDs).  The tiles, in the order below, are taken
// in windows of G (one per iteration of every workgroup): XCD x takes the
// x-th G / 8 tiles of each window, its workgroups one each.  Index v ->
// (channel tile, slot tile) in groups of gm channel tiles x all slot tiles,
// column-major inside a group, so an XCD's resident workgroups cover a
// compact block of 4 channel tiles x 8 slot tiles and share their operand
// steps in the XCD's L2, and the eight XCDs work on neighbouring slot tiles
// of the same channel tiles: the weight panels they share come from the
// Infinity Cache once one XCD has fetched them from HBM.  (Giving each XCD a
// contiguous eighth of the tiles instead measured 1.6-2.9 % slower on the
// 720p FFN layers' delta GEMMs.)
// Long K loops (64 or more steps) take groups of 8 (a 8 x 4 block: fewer
// re-reads of the slot panels, whose steps are then the larger share of each
// tile's bytes; 2 % faster on a 108-step layer, 0.6-1.5 % slower on 40-step
// ones).
struct TileWalk {
    int base, G, total, mt, nt, gm;
    __device__ int count() const { return base < total ? (total - base + G - 1) / G : 0; }
    __device__ void coords(int it, int* tm, int* tn) const {
        const int v = it * G + base;
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
    w.total = mt * nt;
    w.G = G;
    w.base = (b & 7) * (G >> 3) + (b >> 3);     // XCD b & 7, its (b >> 3)-th workgroup
    w.mt = mt;
    w.nt = nt;
    return w;
}

// SMALLK: a K loop shorter than NS steps (the copy cursor may then run
// ahead of the MFMAs' tile from a tile's first step on, or several tiles
// ahead); that form recomputes the copy sources every step, the other one
// only once per tile.
// AFMT: Q4(R) (FMT_FP4) or, for the 6-bit layers, Q6(R) (FMT_FP6 E2M3 or
// FMT_BF6 E3M2, with BFMT the same 6-bit format), or Q4(R) decoded to bf16
// with bf16 cores (FMT_BF16 for both: 32x32x16 bf16 MFMAs, no scales, K
// steps of 32 channels in the FP4 layout's 64-byte rows).
template <int AFMT, int BFMT, int EPI, bool SMALLK>
__global__ __launch_bounds__(256, 1) void k_gemm(GemmArgs p) {
    constexpr bool A6 = AFMT == FMT_FP6 || AFMT == FMT_BF6;
    constexpr bool B6 = BFMT == FMT_FP6 || BFMT == FMT_BF6;
    constexpr bool BF = AFMT == FMT_BF16;
    static_assert(A6 == B6, "6-bit operands come in pairs");
    static_assert(BF == (BFMT == FMT_BF16), "bf16 operands come in pairs");
    constexpr int AROW = A6 ? 96 : 64;                        // A bytes per row per K step
    constexpr int BROW = (BFMT == FMT_FP4 || BF) ? 64 : (B6 ? 96 : 128);   // B bytes per row per K step
    constexpr int A_STEP = 256 * AROW;                        // A bytes per tile step
    constexpr int B_STEP = 256 * BROW;
    constexpr int B_OFF = A_STEP;
    constexpr int SA_OFF = B_OFF + B_STEP;
    constexpr int SB_OFF = SA_OFF + 1024;
    constexpr int STAGE = SB_OFF + 1024;
    constexpr int NS = (BFMT == FMT_FP4 || BF) ? 4 : 3;       // LDS stages in the ring (50 KB stages: 3)
    constexpr int APC = A_STEP / 1024 / 4;                    // 1 KB copies per wave: A
    constexpr int BPC = B_STEP / 1024 / 4;                    //                       B
    constexpr int DMAS = APC + BPC + (BF ? 0 : 2);            // copies per wave per stage (+ scale codes)
    static_assert((NS - 2) * DMAS < 63, "vmcnt range");
    // With four stages a stage's copies go out in two halves: H1 of them in
    // phase 2 of one step, the rest in phase 1 of the next, so the copy
    // stream (and the wait to issue it) is spread over the whole step.
    constexpr bool SPLIT = NS >= 4;
    constexpr int H1 = SPLIT ? DMAS / 2 : DMAS;
    // DEFER (the token epilogue with a three-stage ring): the copies of a
    // tile's last steps do not run into the next tile.  The cursor holds on
    // the tile's last step (those copies repeat it, into stages nothing reads
    // before they are written again), and the epilogue issues the next tile's
    // first NS - 1 stages once its own loads are in: its full wait then covers
    // no slow copies, and its stores hide the new copies' latency.  The wait
    // counts are those of the uniform stream (every step still issues DMAS
    // copies).  (720p FFN down, one-token cubes, FP8 x FP4: 3.75 -> 3.71 ms;
    // with the four-stage FP4 ring, whose copies lead by three steps, the FFN
    // up delta GEMM measured 0.7 % slower, so it keeps the continuous stream.)
    constexpr bool DEFER = !SMALLK && EPI == EPI_TOKENS_Q && NS == 3;
    // after the deferred stage 0: the other deferred copies and the epilogue's 64 stores
    static_assert(!DEFER || (NS - 3) * DMAS + (SPLIT ? H1 : DMAS) + 64 >= 63, "stage 0 covered by vmcnt(63)");
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
    TileWalk walk = tile_walk(blockIdx.x, gridDim.x, p.mtiles, p.ntiles, p.nks);
    int k0 = 0, nk = p.nks;                      // the K steps this workgroup runs of each tile
    if constexpr (EPI == EPI_STORE) {
        if (p.ttotal > 0) walk.total = p.ttotal;
        if (p.su_rm > 0) {                       // one split-K unit
            const int u = blockIdx.x, c = u / p.su_rm;
            walk.base = p.su_v0 + u % p.su_rm;
            walk.total = walk.base + 1;
            k0 = c * p.nks / p.su_p;
            nk = (c + 1) * p.nks / p.su_p - k0;
        }
    }
    const int ntiles = walk.count();
    if (ntiles == 0) return;

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
        r.a = (const uint8_t*)uniform_ptr(p.a + ((size_t)tm * p.nks + k0 + k) * A_STEP);
        r.b = (const uint8_t*)uniform_ptr(p.b + ((size_t)tn * p.nks + k0 + k) * B_STEP);
        r.as = (const uint8_t*)uniform_ptr(p.as + ((size_t)tm * p.nks + k0 + k) * 1024);
        r.bs = (const uint8_t*)uniform_ptr(p.bs + ((size_t)tn * p.nks + k0 + k) * 1024);
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
        } else if constexpr (DEFER) {
            const int d = wrap ? 0 : inc;                  // hold on the tile's last step
            kf = wrap ? kf : kf + 1;
            src.a += d * A_STEP;
            src.b += d * B_STEP;
            src.as += d * 1024;
            src.bs += d * 1024;
        } else {
            kf = wrap ? 0 : kf + 1;
            src.a = wrap ? nsrc.a : src.a + inc * A_STEP;
            src.b = wrap ? nsrc.b : src.b + inc * B_STEP;
            src.as = wrap ? nsrc.as : src.as + inc * 1024;
            src.bs = wrap ? nsrc.bs : src.bs + inc * 1024;
            inc = wrap ? ninc : inc;
        }
    };
    // K order of the plain-store GEMM (nk >= NS): a workgroup's odd tiles
    // run their K steps backwards.  The workgroups of an XCD start a tile
    // together and keep their channel tiles from one tile to the next, so the
    // operand steps a tile starts with are those its predecessor ended with,
    // still in L2.  (The token-epilogue GEMM measured faster in one order.)
    constexpr bool SERP = !SMALLK && EPI == EPI_STORE;
    auto kdir = [&](int t) { return SERP ? 1 - 2 * (t & 1) : 1; };
    auto prepare_next = [&](int it) {                  // tile it + 1 (or the clamp), for the cursor's wrap
        if constexpr (!SMALLK) {
            if (it + 1 < ntiles) {
                ninc = kdir(it + 1);
                nsrc = src_of(it + 1, ninc > 0 ? 0 : nk - 1);
            } else {
                nsrc = src_of(ntiles - 1, kdir(ntiles - 1) > 0 ? nk - 1 : 0);
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
    const int bsw = (BFMT == FMT_FP4 || BF) ? swz4(brow0) : swz8(brow0);   // bf16 rows use the FP4 layout
    const int r6 = rot6(l32);                    // FP6 word rotation (rows arow0 + 32 mi, brow0 + 32 ni: rot6(l32))
    // Scale codes: one 8-byte read per operand gives the lane's codes for the
    // whole step (four 32-row blocks x two halves); code (block r, half kk) is
    // byte 2 (r % 2) + kk of dword r / 2, selected by the MFMA's op_sel.
    const int sa_off = SA_OFF + ((wr * 2 + g) * 32 + l32) * 8;
    const int sb_off = SB_OFF + ((wc * 2 + g) * 32 + l32) * 8;
    struct Half {
        uint4 a[A6 ? 1 : 4];                   // FP4 A fragments
        uint2 a6[A6 ? 4 : 1][3];               // FP6 A fragments (three 8-byte words each)
        uint4 b[(BFMT == FMT_FP4 || BF) ? 4 : 1];   // FP4 (or bf16) B fragments
        v8i b8[BFMT == FMT_FP8 ? 4 : 1];       // FP8 B fragments (two 16-byte chunks each)
        uint2 b6[B6 ? 4 : 1][3];               // FP6 B fragments
        uint2 sa, sb;
    };
    // the three words of FP6 group Gl (0 .. 3 within the step) of a row whose
    // step starts at rowp
    auto rd6 = [&](const uint8_t* rowp, int Gl, uint2* w) {
#pragma unroll
        for (int i = 0; i < 3; ++i) w[i] = *(const uint2*)(rowp + ((3 * Gl + i + r6) % 12) * 8);
    };
    // LDS read number i (0 .. 9) of half kk's fragments, in the order of
    // their first use by the MFMA sequence below: a0 b0 sa sb b1 b2 b3 a1 a2 a3.
    auto rd = [&](int buf, int kk, Half& F, int i) {
        const uint8_t* st = smem + buf * STAGE;
        auto rda = [&](int mi) {
            if constexpr (A6) rd6(st + (arow0 + 32 * mi) * AROW, 2 * kk + g, F.a6[mi]);
            else F.a[mi] = *(const uint4*)(st + (arow0 + 32 * mi) * 64 + (((2 * kk + g) ^ asw) << 4));
        };
        auto rdb = [&](int ni) {
            const uint8_t* rowp = st + B_OFF + (brow0 + 32 * ni) * BROW;
            if constexpr (B6) {
                rd6(rowp, 2 * kk + g, F.b6[ni]);
            } else if constexpr (BFMT == FMT_FP4 || BF) {
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
            case 2: if constexpr (!BF) F.sa = *(const uint2*)(st + sa_off); break;
            case 3: if constexpr (!BF) F.sb = *(const uint2*)(st + sb_off); break;
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
        if constexpr (BF) {
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, F.a[mi]),
                                                                  __builtin_bit_cast(v8bf, F.b[ni]), acc[mi][ni], 0, 0, 0);
            return;
        }
        v8i af, bf;
        if constexpr (A6) {
            const uint2* w = F.a6[mi];
            af = (v8i){(int)w[0].x, (int)w[0].y, (int)w[1].x, (int)w[1].y, (int)w[2].x, (int)w[2].y, 0, 0};
        } else {
            const uint4 v = F.a[mi];
            af = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        }
        if constexpr (B6) {
            const uint2* w = F.b6[ni];
            bf = (v8i){(int)w[0].x, (int)w[0].y, (int)w[1].x, (int)w[1].y, (int)w[2].x, (int)w[2].y, 0, 0};
        } else if constexpr (BFMT == FMT_FP4) {
            const uint4 u = F.b[ni];
            bf = (v8i){(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
        } else {
            bf = F.b8[ni];
        }
        const int sa = (mi >> 1) ? (int)F.sa.y : (int)F.sa.x, sb = (ni >> 1) ? (int)F.sb.y : (int)F.sb.x;
        // op_sel operands must be constants: spell out the byte choices
#define DQ_MFMA(OA, OB) acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, acc[mi][ni], AFMT, BFMT, OA, sa, OB, sb)
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
    // The next tile's first NS - 1 stages (DEFER), as in the prologue, into
    // the stages after the tile's last one (global steps gs ..); the last of
    // them only its first half when split, the cursor then staying on it.
    auto issue_next = [&]() {
        src = nsrc;
        inc = ninc;
        kf = 0;
        const int g0 = tstage + 1;
#pragma unroll
        for (int s = 0; s < NS - 1; ++s) {
            const bool half = SPLIT && s == NS - 2;
#pragma unroll
            for (int j = 0; j < DMAS; ++j)
                if (!half || j < H1) dma(src, (g0 + s) % NS, j);
            if (!half) advance();
        }
    };

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
            // the tile's rows of c, or the unit's own partial (split-K units)
            float* const cb = p.su_rm > 0 ? p.c + (size_t)blockIdx.x * 65536 : p.c + (long long)n0 * p.ldc + m0;
            const long long ldc = p.su_rm > 0 ? 256 : p.ldc;
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
                                                    (v4f*)(cb + (long long)(wc * 128 + 32 * ni + rr) * ldc + wr * 128 + 32 * mi + 4 * (lane & 7)));
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
            // token of each row the lane stores after the transposition (row
            // 8 i + lane / 8 of the blocks of ni: lane rr's slot), all 16
            // permutes in flight together
            int trow[4][4];
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int i = 0; i < 4; ++i) trow[ni][i] = __builtin_amdgcn_ds_bpermute((8 * i + (lane >> 3)) * 4, tok[ni]);
            // low-rank branch: acc += (U L2)^T, 32x32x16 bf16 MFMAs over the 32 ranks
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[h][mi], ub[h][ni], acc[mi][ni], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (DEFER) issue_next();
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
                            // bit select (no branch): the token's y row, or the sink
                            const int t = trow[ni][i];
                            const uint64_t yrow = (uint64_t)(p.y + (uint32_t)(t * p.Co + chq));
                            const uint64_t sink = (uint64_t)(p.sink + 4 * lane);
                            const uint64_t m = (uint64_t)(int64_t)(t >> 31);   // all ones for a slot without a token
                            rowp[i] = (float*)((yrow & ~m) | (sink & m));
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
        if constexpr (EPI == EPI_ROWS_Q) {
            // Rows scaled by their row scale, then by the channel scales, each
            // product rounded: the loads go out before the one full wait; the
            // output passes through the transposition buffers as in the token
            // epilogue, and is scaled after it (the lane then holds 4
            // consecutive channels of one row).
            int tok[4];
            float sx[4][4];
            float4 sw[4];
            const int chq = m0 + wr * 128 + 4 * (lane & 7);   // this lane's channels after the transposition (+ 32 mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                tok[ni] = ld_off<int>(p.stok, (uint32_t)(n0 + wc * 128 + 32 * ni + l32) * 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) sx[ni][i] = ld_off<float>(p.xscale, (uint32_t)(n0 + wc * 128 + 32 * ni + 8 * i + (lane >> 3)) * 4);
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) sw[mi] = ld_off<float4>(p.wscale, (uint32_t)(chq + 32 * mi) * 4);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();                                // every wave is done with the last step's stage
            wait_vm<0>();
            int trow[4][4];
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int i = 0; i < 4; ++i) trow[ni][i] = __builtin_amdgcn_ds_bpermute((8 * i + (lane >> 3)) * 4, tok[ni]);
            float* rowp[4];
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
                    if (mi == 0) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int t = trow[ni][i];
                            const uint64_t yrow = (uint64_t)(p.y + (uint32_t)(t * p.Co + chq));
                            const uint64_t sink = (uint64_t)(p.sink + 4 * lane);
                            const uint64_t m = (uint64_t)(int64_t)(t >> 31);   // all ones for a row past the end
                            rowp[i] = (float*)((yrow & ~m) | (sink & m));
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float4 v = tget(pb & 1, i);
                        const float r = sx[ni][i];
                        const float4 o = make_float4((v.x * r) * sw[mi].x, (v.y * r) * sw[mi].y, (v.z * r) * sw[mi].z,
                                                     (v.w * r) * sw[mi].w);
                        __builtin_nontemporal_store(__builtin_bit_cast(v4f, o), (v4f*)(rowp[i] + 32 * mi));
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
                    float4 o = make_float4(a[4 * j] + bv[mi][j].x, a[4 * j + 1] + bv[mi][j].y,
                                           a[4 * j + 2] + bv[mi][j].z, a[4 * j + 3] + bv[mi][j].w);
                    const int ch = ch0 + 32 * mi + 8 * j;
                    if (p.xscale) {                         // (acc s_x) s_w, each product rounded
                        const float sx = p.xscale[slot];
                        const float4 sw = *(const float4*)(p.wscale + ch);
                        o = make_float4((o.x * sx) * sw.x, (o.y * sx) * sw.y, (o.z * sx) * sw.z, (o.w * sx) * sw.w);
                    }
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
        if (EPI != EPI_TOKENS_Q && EPI != EPI_ROWS_Q) wait_vm<0>();   // those epilogues wait after issuing their loads
        int tm, tn;
        walk.coords(it, &tm, &tn);
        tstage = (unsigned)(gs - 1) % NS;
        epilogue(tm, tn);
        if constexpr (DEFER) {                             // the next tile's stage 0, every wave's copies
            wait_vm<63>();
            __syncthreads();
        }
        // The last step already read half 0 of the next tile's first stage
        // (landed: its barrier covered it); reading it again here keeps those
        // registers free during the epilogue.
#pragma unroll
        for (int i = 0; i < NRD; ++i) rd((unsigned)gs % NS, 0, F0, i);
    }
    if constexpr (DEFER) wait_vm<0>();                   // the last tile's surplus copies land before the LDS is released
}

// ---- The fused form: core term and delta term in one K loop --------------
// For cubes of 4 slots with FP8 cores, one kernel computes, per 256-channel x
// 256-slot tile, both the delta term over the tile's 256 slots and the core
// term Q8(core) Q4(R) over its 64 cubes, accumulating the core partial sums
// beside the delta ones as the pages' kernel does (DeltaQuant notes,
// 损失函数/训练策略), so the per-cube term never goes to memory.
//  - Both contractions share the Q4(R) fragments of every K step.  A wave's
//    core block is its 32 cubes x its 128 channels: 4 FP8 x FP4 MFMAs per half
//    step beside the 16 FP4 x FP4 ones, 64 fp32 accumulators in VGPRs.
//  - Slot rows are permuted on their way into LDS: accumulator row
//    32 ni + l (of a wave's 128-row half) holds slot 4 l + ni, so in every
//    block ni lane l holds a slot of cube l, the cube whose core term the
//    lane's own core accumulators hold, and the epilogue adds them with no
//    exchange between lanes.  The copies move each slot row's 64 bytes to its
//    new place and re-swizzle its chunks for that row; the delta scale codes
//    are copied unchanged and each lane reads its four rows' codes apart.
//  - LDS: 3 stages of 42.5 KB (A, B, their scales, the 64 cube rows' FP8 step
//    and their scales) and, apart from the ring, the epilogue's transposition
//    buffers (32 KB).  A stage is released at the barrier of its own step: the
//    wave waits for its reads of the step's second half before the barrier, so
//    the copy stream leads the MFMAs by as many steps as with four stages.
struct FusedArgs {
    const uint8_t *a, *as;   // Q4(R) codes and scales, step-major (256-channel tiles)
    const uint8_t *b, *bs;   // delta codes and scales, step-major (256-slot tiles, slot order)
    const uint8_t *c, *cs;   // core FP8 codes and scales, step-major (256-cube tiles)
    int nks, mtiles, ntiles;
    float* y;                // [N][Co] token order, Co a multiple of 256
    int Co;
    const int* stok;         // slot -> token (-1 for pad slots)
    const uint16_t* u;       // [Nslot_pad][32]
    const uint16_t* l2t;     // [Cop][32]
    float* sink;
};

// One FP4 x FP8 scaled MFMA (A = 32 FP4 codes, B = 32 FP8 codes per lane)
// into an accumulator held in architectural VGPRs.  Written as an asm
// statement because the compiler gives every MFMA of a kernel an AGPR
// accumulator: with the delta term's 256 already there, it would shuttle
// tuples between the two files on every step.  Byte SA of the A scale
// register and byte SB of the B one select the E8M0 codes (op_sel holds the
// low bit, op_sel_hi the high one).  The s_nop gives a VALU write of an
// operand (the B scale is shifted into place just before) the wait states
// an MFMA read needs after it; the accumulator is written only by this MFMA
// and read again only after the tile's K loop.
template <int SA, int SB>
__device__ __forceinline__ void core_mfma(v16f& acc, uint4 a4, v8i b, int sa, uint32_t sb) {
    const v4i a = __builtin_bit_cast(v4i, a4);
    asm volatile("s_nop 4\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[%5,%6,0] op_sel_hi:[%7,%8,0] cbsz:4 blgp:0"
                 : "+v"(acc)
                 : "v"(a), "v"(b), "v"(sa), "v"(sb), "n"(SA & 1), "n"(SB & 1), "n"(SA >> 1), "n"(SB >> 1));
}

__global__ __launch_bounds__(256, 1) void k_fused(FusedArgs p) {
    constexpr int A_STEP = 16384, B_STEP = 16384;
    constexpr int B_OFF = A_STEP, SA_OFF = B_OFF + B_STEP, SB_OFF = SA_OFF + 1024;
    constexpr int C_OFF = SB_OFF + 1024;       // 64 cube rows x 128 bytes
    constexpr int SC_OFF = C_OFF + 8192;       // 64 dwords of core scale codes (+ 192 bytes the copies overrun into)
    constexpr int STAGE = SC_OFF + 512;        // (stages start at multiples of 256 bytes: the swizzles' bank pattern)
    constexpr int NS = 3;
    constexpr int T_OFF = NS * STAGE;          // transposition buffers, 8 KB per wave
    constexpr int DMAS = 13;                   // copies per wave per stage: A 4, B 4, scales 2, cores 2, core scales 1
    constexpr int H1 = 6;                      // the first half (issued in phase 2), the rest in phase 1 of the next step
    static_assert(T_OFF + 32768 <= 163840, "LDS");
    static_assert(DMAS + H1 < 63, "vmcnt range");
    // copies sit after every third MFMA of a phase (phase 1 from MFMA 0, phase 2 from MFMA 2)
    auto p1_copy = [](int i) { return i % 3 == 0 && i / 3 < DMAS - H1 ? H1 + i / 3 : -1; };
    auto p2_copy = [](int i) { return i >= 2 && (i - 2) % 3 == 0 && (i - 2) / 3 < H1 ? (i - 2) / 3 : -1; };
    __shared__ __attribute__((aligned(1024))) uint8_t smem[T_OFF + 32768];

    const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const TileWalk walk = tile_walk(blockIdx.x, gridDim.x, p.mtiles, p.ntiles, p.nks);
    const int nk = p.nks;
    const int ntiles = walk.count();
    if (ntiles == 0) return;

    // ---- per-lane offsets of the copies and of the fragment reads, derived
    // from the thread index t.  The tile loop recomputes them at every tile's
    // start from a copy of the index the compiler cannot see through, so none
    // stays live across an epilogue, whose registers they would take.
    struct Lanes {
        uint32_t va, vb, vs, vc, vsc;   // copy offsets: A, B (permuted rows), scales, cores, core scales
        int aoff[2], boff[2];           // fragment offsets within a stage, half kk (+ 2048 per 32-row block)
        int sa_off, sb_off, sc_off;
        int coff[2][2];                 // core fragment, half kk: low and high 16 bytes
        uint32_t sb_sh, sc_sh;          // where a lane's two scale codes sit in the dwords read
    };
    auto lanes_of = [&](int t) {
        const int lane = t & 63, wave = t >> 6;
        const int wr = wave >> 1, wc = wave & 1;
        const int g = lane >> 5, l32 = lane & 31;
        Lanes L;
        L.va = (uint32_t)lane * 16 + wv * 4096;
        // delta rows: LDS row R = 64 wv + 16 jb + lane / 4 of copy jb takes
        // slot row s(R) = (R & 128) | (R % 32) 4 | (R / 32) % 4, its chunk pc
        // (of R) holding logical chunk pc ^ swz4(R), found at
        // (pc ^ swz4(R)) ^ swz4(s) in the slot row.  s = s0 + 64 (jb % 2) +
        // jb / 2, and neither swizzle depends on jb (they read row bits 1-3),
        // so copy jb reads at vb + 64 (jb / 2) from the step base + 4096 (jb % 2).
        {
            const int R = wv * 64 + (lane >> 2), pc = lane & 3;
            const int s = (R & 128) | ((R & 31) << 2) | ((R >> 5) & 3);
            L.vb = (uint32_t)s * 64 + (uint32_t)(((pc ^ swz4(R)) ^ swz4(s)) << 4);
        }
        L.vs = (uint32_t)lane * 4 + wv * 256;
        L.vc = (uint32_t)lane * 16 + wv * 2048;
        // core scale codes: dword d = 32 g + l (cube row l of the half g
        // reads) of the LDS block is the dword that holds cube l's codes in
        // the step's scale block; wave w writes dwords 16 w .. 16 w + 63 (the
        // last ones repeat dword 63 past the block's 64, into the overrun bytes)
        L.vsc = (uint32_t)min(16 * wv + lane, 63) * 8;
        const int arow0 = wr * 128 + l32, brow0 = wc * 128 + l32;
        const int asw = swz4(arow0), bsw = swz4(brow0), csw = swz8(l32);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            L.aoff[kk] = arow0 * 64 + (((2 * kk + g) ^ asw) << 4);
            L.boff[kk] = B_OFF + brow0 * 64 + (((2 * kk + g) ^ bsw) << 4);
            L.coff[kk][0] = C_OFF + (wc * 32 + l32) * 128 + (((4 * kk + g) ^ csw) << 4);
            L.coff[kk][1] = C_OFF + (wc * 32 + l32) * 128 + (((4 * kk + 2 + g) ^ csw) << 4);
        }
        L.sa_off = SA_OFF + ((wr * 2 + g) * 32 + l32) * 8;
        // delta scale codes of LDS row brow0 + 32 ni (slot wc 128 + 4 l32 +
        // ni): the 2 bytes (kk 0, 1) at entry (wc, g, (4 l32 + ni) % 32),
        // bytes 2 (l32 / 8) ..; read as the dword that holds them
        // ((4 l32 + ni) % 32 = 4 (l32 % 8) + ni: ni in the read's offset
        // field) and shifted into bytes 0, 1 where an MFMA uses them
        L.sb_off = SB_OFF + (wc * 2 + g) * 256 + ((l32 >> 4) & 1) * 4 + (l32 & 7) * 32;
        L.sb_sh = ((l32 >> 3) & 1) * 16;
        L.sc_off = SC_OFF + (g * 32 + l32) * 4;    // bytes 2 wc + kk of the lane's dword
        L.sc_sh = 16 * wc;
        return L;
    };
    auto opaque_tid = []() {
        int t = (int)threadIdx.x;
        asm volatile("" : "+v"(t));
        return t;
    };

    // ---- copies (tile step bases uniform)
    const uint32_t lds0 = lds_addr(smem);
    struct Src {
        const uint8_t *a, *b, *as, *bs, *c, *cs;
    };
    auto src_of = [&](int t, int k) {
        int tm, tn;
        walk.coords(t, &tm, &tn);
        const int kt = tn >> 2, q = tn & 3;      // the tile's 64 cubes: rows 64 q .. of core tile kt
        Src r;
        r.a = (const uint8_t*)uniform_ptr(p.a + ((size_t)tm * nk + k) * A_STEP);
        r.b = (const uint8_t*)uniform_ptr(p.b + ((size_t)tn * nk + k) * B_STEP);
        r.as = (const uint8_t*)uniform_ptr(p.as + ((size_t)tm * nk + k) * 1024);
        r.bs = (const uint8_t*)uniform_ptr(p.bs + ((size_t)tn * nk + k) * 1024);
        r.c = (const uint8_t*)uniform_ptr(p.c + ((size_t)kt * nk + k) * 32768 + q * 8192);
        // rows 64 q + 32 h + l sit in entry (q / 2, half g, l), dword q % 2
        // (bytes 2 h + kk) of the step's scale block
        r.cs = (const uint8_t*)uniform_ptr(p.cs + ((size_t)kt * nk + k) * 1024 + (q >> 1) * 512 + 4 * (q & 1));
        return r;
    };
    auto dma = [&](const Lanes& L, const Src& src, int buf, int j) {
        const uint32_t st = lds0 + buf * STAGE;
        if (j < 4) {
            switch (j) {
                case 0: dma16o<0>(src.a, L.va, st + (wv * 4) * 1024); break;
                case 1: dma16o<1024>(src.a, L.va, st + (wv * 4 + 1) * 1024); break;
                case 2: dma16o<2048>(src.a, L.va, st + (wv * 4 + 2) * 1024); break;
                default: dma16o<3072>(src.a, L.va, st + (wv * 4 + 3) * 1024); break;
            }
        } else if (j < 8) {
            // jb = 0 2 1 3: the copies that share cache lines one after the other
            switch (j) {
                case 4: dma16o<0>(src.b, L.vb, st + B_OFF + (wv * 4) * 1024); break;
                case 5: dma16o<64>(src.b, L.vb, st + B_OFF + (wv * 4 + 2) * 1024); break;
                case 6: dma16o<0>(uniform_ptr(src.b + 4096), L.vb, st + B_OFF + (wv * 4 + 1) * 1024); break;
                default: dma16o<64>(uniform_ptr(src.b + 4096), L.vb, st + B_OFF + (wv * 4 + 3) * 1024); break;
            }
        } else if (j == 8) {
            dma4(src.as, L.vs, st + SA_OFF + wv * 256);
        } else if (j == 9) {
            dma4(src.bs, L.vs, st + SB_OFF + wv * 256);
        } else if (j == 10) {
            dma16o<0>(src.c, L.vc, st + C_OFF + (wv * 2) * 1024);
        } else if (j == 11) {
            dma16o<1024>(src.c, L.vc, st + C_OFF + (wv * 2 + 1) * 1024);
        } else {
            dma4(src.cs, L.vsc, st + SC_OFF + wv * 64);
        }
    };
    // Cursor (tile tf, step kf): it runs three steps ahead of the MFMAs and
    // holds on the last tile's last step; inside a tile by pointer
    // increments, into the next tile at the wrap (sources prepared at the
    // tile's start in nsrc; ninc = 0 for the last tile).  Branch-free.
    int kf = 0;
    Src src = src_of(0, 0), nsrc{};
    int inc = 1, ninc = 1;
    auto advance = [&]() {
        const bool wrap = kf + 1 == nk;
        kf = wrap ? 0 : kf + 1;
        src.a = wrap ? nsrc.a : src.a + inc * A_STEP;
        src.b = wrap ? nsrc.b : src.b + inc * B_STEP;
        src.as = wrap ? nsrc.as : src.as + inc * 1024;
        src.bs = wrap ? nsrc.bs : src.bs + inc * 1024;
        src.c = wrap ? nsrc.c : src.c + inc * 32768;
        src.cs = wrap ? nsrc.cs : src.cs + inc * 1024;
        inc = wrap ? ninc : inc;
    };
    auto prepare_next = [&](int it) {
        if (it + 1 < ntiles) {
            ninc = 1;
            nsrc = src_of(it + 1, 0);
        } else {
            nsrc = src_of(ntiles - 1, nk - 1);
            ninc = 0;
        }
    };

    v16f acc[4][4];      // delta term (+ low-rank branch): channel block mi x slot block ni
    v16f cacc[4];        // core term: channel block mi x the wave's 32 cubes

    // ---- fragments of one 64-channel half step
    struct Half {
        uint4 a[4], b[4];
        uint2 sa;
        uint32_t sb[4];      // block ni's two codes (kk 0, 1) in bytes sb_sh / 8 ..
        v8i c;
        uint32_t sc;         // the cube's two codes in bytes sc_sh / 8 ..
    };
    // LDS read number i (0 .. NRD - 1) of half kk, in the order of first use
    auto rd = [&](const Lanes& L, int buf, int kk, Half& F, int i) {
        const uint8_t* st = smem + buf * STAGE;
        auto rda = [&](int mi) { F.a[mi] = *(const uint4*)(st + L.aoff[kk] + mi * 2048); };
        auto rdb = [&](int ni) { F.b[ni] = *(const uint4*)(st + L.boff[kk] + ni * 2048); };
        auto sbh = [&](int ni) { return *(const uint32_t*)(st + L.sb_off + ni * 8); };
        switch (i) {
            case 0: rda(0); break;
            case 1: rdb(0); break;
            case 2: F.sa = *(const uint2*)(st + L.sa_off); break;
            case 3:
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) F.sb[ni] = sbh(ni);
                break;
            case 4: rdb(1); break;
            case 5: rdb(2); break;
            case 6: rdb(3); break;
            case 7: rda(1); break;
            case 8: rda(2); break;
            case 9: rda(3); break;
            case 10: {
                const v4i lo = *(const v4i*)(st + L.coff[kk][0]);
                const v4i hi = *(const v4i*)(st + L.coff[kk][1]);
                F.c = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                break;
            }
            default: F.sc = *(const uint32_t*)(st + L.sc_off); break;
        }
    };
    constexpr int NRD = 12;
    // MFMA number i (0 .. 19) of half kk: 16 delta MFMAs (block mi = i / 4,
    // ni = i % 4), then the 4 core MFMAs (block mi = i - 16)
    auto mma = [&](const Lanes& L, const Half& F, int kk, int i) {
        const int mi = i < 16 ? i >> 2 : i - 16, ni = i & 3;
        const uint4 v = F.a[mi];
        const v8i af = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        const int sa = (mi >> 1) ? (int)F.sa.y : (int)F.sa.x;
        const int oa = 2 * (mi & 1) + kk;
        if (i >= 16) {
            switch (oa * 2 + kk) {
                case 0: core_mfma<0, 0>(cacc[mi], v, F.c, sa, F.sc >> L.sc_sh); break;
                case 1: core_mfma<0, 1>(cacc[mi], v, F.c, sa, F.sc >> L.sc_sh); break;
                case 2: core_mfma<1, 0>(cacc[mi], v, F.c, sa, F.sc >> L.sc_sh); break;
                case 3: core_mfma<1, 1>(cacc[mi], v, F.c, sa, F.sc >> L.sc_sh); break;
                case 4: core_mfma<2, 0>(cacc[mi], v, F.c, sa, F.sc >> L.sc_sh); break;
                case 5: core_mfma<2, 1>(cacc[mi], v, F.c, sa, F.sc >> L.sc_sh); break;
                case 6: core_mfma<3, 0>(cacc[mi], v, F.c, sa, F.sc >> L.sc_sh); break;
                default: core_mfma<3, 1>(cacc[mi], v, F.c, sa, F.sc >> L.sc_sh); break;
            }
            return;
        }
        const uint4 u = F.b[ni];
        const v8i bf = (v8i){(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
        const int sb = (int)(F.sb[ni] >> L.sb_sh);
#define DQ_MFMA(OA, OB) acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, acc[mi][ni], FMT_FP4, FMT_FP4, OA, sa, OB, sb)
        switch (oa * 2 + kk) {
            case 0: DQ_MFMA(0, 0); break;  case 1: DQ_MFMA(0, 1); break;
            case 2: DQ_MFMA(1, 0); break;  case 3: DQ_MFMA(1, 1); break;
            case 4: DQ_MFMA(2, 0); break;  case 5: DQ_MFMA(2, 1); break;
            case 6: DQ_MFMA(3, 0); break;  default: DQ_MFMA(3, 1); break;
        }
#undef DQ_MFMA
    };

    // ---- tile epilogue: acc[mi][ni][4 j + q] is channel m0 + wr 128 + 32 mi
    // + 8 j + 4 g + q of slot n0 + wc 128 + 4 l32 + ni (cube row l32 of the
    // wave's half), cacc[mi][4 j + q] the same channel of that cube.
    auto epilogue = [&](int tm, int tn) {
        // The epilogue's lane offsets are derived here, from a copy of the
        // thread index the compiler cannot see through, so they are not
        // hoisted out of the tile loop and kept live across the K loop
        // (where the registers are taken).
        int tid_e = (int)threadIdx.x;
        asm volatile("" : "+v"(tid_e));
        const int lane = tid_e & 63, wave = tid_e >> 6;
        const int wr = wave >> 1, wc = wave & 1;
        const int g = lane >> 5, l32 = lane & 31;
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        // transposition buffers (as in k_gemm's token epilogue), outside the ring
        auto tbuf = [&](int b) { return smem + T_OFF + wv * 8192 + b * 4096; };
        auto tput = [&](int b, const float4* o) {
            uint8_t* t = tbuf(b) + l32 * 128;
#pragma unroll
            for (int j = 0; j < 4; ++j) *(float4*)(t + (((2 * j + g) ^ ((l32 >> 1) & 7)) << 4)) = o[j];
        };
        auto tget = [&](int b, int i) {
            const int rr = 8 * i + (lane >> 3);
            return *(const float4*)(tbuf(b) + rr * 128 + (((lane & 7) ^ ((rr >> 1) & 7)) << 4));
        };
        const int m0 = tm * 256, n0 = tn * 256;
        const uint32_t slot0 = (uint32_t)(n0 + wc * 128 + 4 * l32);      // + ni
        int tok[4];
        v8bf la[2][4], ub[2][4];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) tok[ni] = ld_off<int>(p.stok, (slot0 + ni) * 4);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const uint32_t lo = ((uint32_t)(m0 + wr * 128 + l32 + 32 * mi) * 32 + 8 * g) * 2;
            la[0][mi] = __builtin_bit_cast(v8bf, ld_off<uint4>(p.l2t, lo));
            la[1][mi] = __builtin_bit_cast(v8bf, ld_off<uint4>(p.l2t, lo + 32));
        }
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const uint32_t uo = ((slot0 + ni) * 32 + 8 * g) * 2;
            ub[0][ni] = __builtin_bit_cast(v8bf, ld_off<uint4>(p.u, uo));
            ub[1][ni] = __builtin_bit_cast(v8bf, ld_off<uint4>(p.u, uo + 32));
        }
        __builtin_amdgcn_sched_barrier(0);
        // every copy in flight (the next tile's first stages) and the loads above
        wait_vm<0>();
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[h][mi], ub[h][ni], acc[mi][ni], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        const int chq = m0 + wr * 128 + 4 * (lane & 7);
        float* rowp[4];
#pragma unroll
        for (int b = 0; b < 17; ++b) {
            if (b < 16) {                               // block b: mi = b % 4, ni = b / 4
                const int mi = b & 3, ni = b >> 2;
                const v16f& a = acc[mi][ni];
                const v16f& c = cacc[mi];
                float4 o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    o[j] = make_float4(a[4 * j] + c[4 * j], a[4 * j + 1] + c[4 * j + 1], a[4 * j + 2] + c[4 * j + 2],
                                       a[4 * j + 3] + c[4 * j + 3]);
                tput(b & 1, o);
            }
            if (b > 0) {
                const int pb = b - 1, mi = pb & 3, ni = pb >> 2;
                if (mi == 0) {
                    // the tokens of the rows this lane stores (row 8 i + lane / 8
                    // of the slot block: lane 8 i + lane / 8's slot), fetched
                    // when the block's first rows go out
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = __builtin_amdgcn_ds_bpermute((8 * i + (lane >> 3)) * 4, tok[ni]);
                        const uint64_t yrow = (uint64_t)(p.y + (uint32_t)(t * p.Co + chq));
                        const uint64_t sink = (uint64_t)(p.sink + 4 * lane);
                        const uint64_t m = (uint64_t)(int64_t)(t >> 31);   // all ones for a slot without a token
                        rowp[i] = (float*)((yrow & ~m) | (sink & m));
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 v = tget(pb & 1, i);
                    __builtin_nontemporal_store(__builtin_bit_cast(v4f, v), (v4f*)(rowp[i] + 32 * mi));
                }
            }
        }
    };

    // ---- K loop.  Step gs: phase 1 runs the MFMAs of half 0 of stage gs
    // (F0) while reading half 1 into F1 and issuing the second half of stage
    // gs + 2's copies; then the wave waits for its F1 reads and for its copies
    // of stage gs + 1, and the barrier: stage gs + 1 has landed and no wave
    // reads stage gs any more; phase 2 runs half 1 (F1) while issuing the
    // first half of stage gs + 3's copies into stage gs's buffer and reading
    // half 0 of stage gs + 1 into F0.
    // Prologue: stages 0 and 1, and the first half of stage 2 (the cursor
    // then stays on step 2).
    {
        const Lanes L = lanes_of((int)threadIdx.x);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int j = 0; j < DMAS; ++j) dma(L, src, s, j);
            advance();
        }
#pragma unroll
        for (int j = 0; j < H1; ++j) dma(L, src, 2, j);
    }
    wait_vm<DMAS + H1>();                                  // stage 0 landed
    __syncthreads();
    Half F0, F1;
    // Stage gs + 1 must have landed at the barrier of step gs: the copies
    // issued after it are stage gs + 2's, DMAS of them.  In a tile's first
    // step after the first tile, stage gs + 1 was covered by the previous
    // epilogue's full wait, and a loose count lets that epilogue's stores
    // stay in flight.
    int gs = 0;
    for (int it = 0; it < ntiles; ++it) {
        const Lanes L = lanes_of(opaque_tid());
        // half 0 of the tile's first stage (landed: the previous step's
        // barrier, or the prologue's, covered it)
#pragma unroll
        for (int i = 0; i < NRD; ++i) rd(L, (unsigned)gs % NS, 0, F0, i);
        prepare_next(it);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            cacc[i] = (v16f){};
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = (v16f){};
        }
        __builtin_amdgcn_sched_barrier(0);
        for (int ks = 0; ks < nk; ++ks, ++gs) {
            const int cur = (unsigned)gs % NS, nxt = (unsigned)(gs + 1) % NS, fillp = (unsigned)(gs + 2) % NS;
#pragma unroll
            for (int i = 0; i < 20; ++i) {
                mma(L, F0, 0, i);
                if (i < NRD) rd(L, cur, 1, F1, i);
                if (p1_copy(i) >= 0) dma(L, src, fillp, p1_copy(i));
                __builtin_amdgcn_sched_barrier(0);
            }
            advance();
            const int loose = __builtin_amdgcn_readfirstlane((it > 0 && ks == 0) ? 1 : 0);
            asm volatile(
                "s_waitcnt lgkmcnt(0)\n\t"
                "s_cmp_eq_u32 %0, 0\n\t"
                "s_cbranch_scc1 1f\n\t"
                "s_waitcnt vmcnt(63)\n\t"
                "s_branch 2f\n"
                "1:\n\t"
                "s_waitcnt vmcnt(%1)\n"
                "2:\n\t"
                "s_barrier" ::"s"(loose), "n"(DMAS) : "memory", "scc");
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 20; ++i) {
                mma(L, F1, 1, i);
                if (p2_copy(i) >= 0) dma(L, src, cur, p2_copy(i));
                if (i < NRD) rd(L, nxt, 0, F0, i);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        int tm, tn;
        walk.coords(it, &tm, &tn);
        epilogue(tm, tn);
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

template <int BFMT, int EPI, int AFMT = FMT_FP4>
static hipError_t launch(const GemmArgs& a, hipStream_t st) {
    constexpr int NS = (BFMT == FMT_FP4 || BFMT == FMT_BF16) ? 4 : 3;      // the kernel's LDS stages
    const int grid = persistent_grid(a.ttotal > 0 ? a.ttotal : a.mtiles * a.ntiles);
    if (a.nks < NS) k_gemm<AFMT, BFMT, EPI, true><<<grid, 256, 0, st>>>(a);
    else k_gemm<AFMT, BFMT, EPI, false><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

// Sum of the split-K partials: c[tile rows][tile channels] = sum over chunks
// j = 0 .. p - 1, in that order, of partial j rm + r, for the rm tail tiles
// r (walk tiles v0 + r).  64 workgroups per tile, one float4 per thread.
__global__ __launch_bounds__(256) void k_ksum(const float* part, float* c, long long ldc, int mt, int nt, int nks,
                                              int v0, int rm, int p) {
    const int r = blockIdx.x >> 6;
    const int e = ((blockIdx.x & 63) << 8) + threadIdx.x;           // float4 of the tile: row e / 64, channels 4 (e % 64) ..
    const v4f* src = (const v4f*)part + (size_t)r * 16384 + e;
    v4f acc = __builtin_nontemporal_load(src);
    for (int j = 1; j < p; ++j) {
        const v4f v = __builtin_nontemporal_load(src + (size_t)j * rm * 16384);
        acc[0] += v[0];
        acc[1] += v[1];
        acc[2] += v[2];
        acc[3] += v[3];
    }
    TileWalk w = tile_walk(0, 8, mt, nt, nks);
    w.base = v0 + r;
    int tm, tn;
    w.coords(0, &tm, &tn);
    __builtin_nontemporal_store(acc, (v4f*)(c + (long long)(tn * 256 + (e >> 6)) * ldc + tm * 256 + 4 * (e & 63)));
}

// The plain-store GEMM, with the K split `ks` when it has one (partials in
// `part`, ks.part_bytes()).
template <int BFMT, int AFMT = FMT_FP4>
static hipError_t launch_store(const GemmArgs& a, const KSplit& ks, float* part, hipStream_t st) {
    constexpr int NS = (BFMT == FMT_FP4 || BFMT == FMT_BF16) ? 4 : 3;
    if (ks.rm == 0) return launch<BFMT, EPI_STORE, AFMT>(a, st);
    // the plan must fit this GEMM: whole chunks of at least NS steps, one unit per workgroup slot
    if (!part || ks.p < 2 || a.nks / ks.p < NS || ks.main_tiles + ks.rm != a.mtiles * a.ntiles ||
        (long long)ks.rm * ks.p > 65535)
        return hipErrorInvalidValue;
    if (ks.main_tiles > 0) {
        GemmArgs m = a;
        m.ttotal = ks.main_tiles;
        hipError_t e = launch<BFMT, EPI_STORE, AFMT>(m, st);
        if (e != hipSuccess) return e;
    }
    GemmArgs t = a;
    t.c = part;
    t.su_v0 = ks.main_tiles;
    t.su_rm = ks.rm;
    t.su_p = ks.p;
    k_gemm<AFMT, BFMT, EPI_STORE, false><<<ks.rm * ks.p, 256, 0, st>>>(t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_ksum<<<ks.rm * 64, 256, 0, st>>>(part, a.c, a.ldc, a.mtiles, a.ntiles, a.nks, ks.main_tiles, ks.rm, ks.p);
    return hipGetLastError();
}

// The fused form (fused_applies: cubes of exactly 4 slots with FP8 cores in
// one frame segment, so a 256-slot tile's cubes are the 64 rows 64 tn .. of
// the core codes) is the dq_linear_forward_fused entry point, and the whole
// forward of the layers fused_preferred picks (small ones: the two kernels
// measured faster on large layers, whose fused K loop carries the cores'
// operand steps too and is bound by operand delivery).
hipError_t launch_forward_fused(const dq_weights* w, dq_qact* q, float* y, hipStream_t st) {
    if (!fused_applies(w, q, y)) return hipErrorInvalidValue;
    FusedArgs f{};
    f.a = w->rq;
    f.as = w->rs;
    f.b = q->dq;
    f.bs = q->ds;
    f.c = q->cq;
    f.cs = q->cs;
    f.nks = (int)(w->Kp / 128);
    f.mtiles = (int)(w->Cop / 256);
    f.ntiles = (int)(q->Nslot_pad / 256);
    f.y = y;
    f.Co = (int)w->Co;
    f.stok = q->stok;
    f.u = q->u;
    f.l2t = w->l2t;
    f.sink = q->sink;
    k_fused<<<persistent_grid(f.mtiles * f.ntiles), 256, 0, st>>>(f);
    return hipGetLastError();
}

hipError_t launch_forward(const dq_weights* w, dq_qact* q, float* y, int parts, hipStream_t st) {
    if ((parts & FWD_CORE) && (parts & FWD_DELTA) && fused_preferred(w, q, y)) return launch_forward_fused(w, q, y, st);
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
    if ((parts & FWD_CORE) && q->core_bits == 16) {
        // bf16 cores: bias[k] = bf16(core_k) Q4(R), with Q4(R) decoded to bf16
        // (exact), 32x32x16 bf16 MFMAs with fp32 accumulation
        GemmArgs c = d;
        c.a = (const uint8_t*)q->rbf;
        c.as = nullptr;
        c.b = (const uint8_t*)q->cbf;
        c.bs = nullptr;
        c.nks = (int)(w->Kp / 32);
        c.ntiles = (int)(q->K_pad / 256);
        c.c = q->bias;
        c.ldc = w->Cop;
        hipError_t e = launch_store<FMT_BF16, FMT_BF16>(c, q->ks, q->kpart, st);
        if (e != hipSuccess) return e;
    } else if (parts & FWD_CORE) {
        // per-cube core term bias[k] = Q8(core_k) Q4(R) (Q4(core_k) for 4-bit cores)
        GemmArgs c = d;
        c.b = q->cq;
        c.bs = q->cs;
        c.ntiles = (int)(q->K_pad / 256);
        c.c = q->bias;
        c.ldc = w->Cop;
        hipError_t e = q->core_bits == 4 ? launch_store<FMT_FP4>(c, q->ks, q->kpart, st)
                                         : launch_store<FMT_FP8>(c, q->ks, q->kpart, st);
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

// The 6-bit layers: one FP6 x FP6 GEMM over the text tokens with the
// low-rank branch in the epilogue (no per-cube term).  Tokens are their own
// rows (the table is the identity), grouped in fours only for the quad layout
// of the fast epilogue.
hipError_t launch_forward6(const dq_weights* w, dq_act6* a, float* y, hipStream_t st) {
    GemmArgs d{};
    d.a = w->rq;
    d.as = w->rs;
    d.nks = (int)(w->Kp / 128);
    d.mtiles = (int)(w->Cop / 256);
    d.b = a->xq;
    d.bs = a->xs;
    d.ntiles = (int)(a->N_pad / 256);
    d.y = y;
    d.Co = (int)w->Co;
    d.vec4 = (w->Co % 4 == 0) && ((uintptr_t)y % 16 == 0);
    d.stok = a->stok;
    d.S = 4;
    d.S2 = 4;
    d.split = (int)a->N_pad;
    d.ksplit = 0;
    d.kmax = 0;
    d.bias = nullptr;
    d.u = a->u;
    d.l2t = w->l2t;
    d.rp = w->rp;
    d.sink = a->sink;
    const bool fast = d.rp == 32 && d.vec4 && a->N * w->Co < (1ll << 31) && d.Co % 256 == 0;
    if (w->wfmt == FMT_BF6)
        return fast ? launch<FMT_BF6, EPI_TOKENS_Q, FMT_BF6>(d, st) : launch<FMT_BF6, EPI_TOKENS, FMT_BF6>(d, st);
    return fast ? launch<FMT_FP6, EPI_TOKENS_Q, FMT_FP6>(d, st) : launch<FMT_FP6, EPI_TOKENS, FMT_FP6>(d, st);
}

// The rotated-basis (OrbitQuant-style) layers: the decoded Lloyd-Max levels
// as bf16 operands, y = (acc s_x[token]) s_w[channel] in the token epilogue.
hipError_t launch_orbit_gemm(const uint16_t* wdec, const uint16_t* xdec, int64_t Kp, int64_t Cop, int64_t Npad, int64_t Co,
                             const int* rows, const float* xscale, const float* wscale, float* y, float* sink,
                             hipStream_t st) {
    GemmArgs d{};
    d.a = (const uint8_t*)wdec;
    d.b = (const uint8_t*)xdec;
    d.nks = (int)(Kp / 32);
    d.mtiles = (int)(Cop / 256);
    d.ntiles = (int)(Npad / 256);
    d.y = y;
    d.Co = (int)Co;
    d.vec4 = (Co % 4 == 0) && ((uintptr_t)y % 16 == 0);
    d.stok = rows;
    d.S = 1;
    d.S2 = 1;
    d.split = (int)Npad;
    d.kmax = 0;
    d.rp = 0;
    d.sink = sink;
    d.xscale = xscale;
    d.wscale = wscale;
    if (d.vec4 && Co % 256 == 0 && Npad * Co < (1ll << 31)) return launch<FMT_BF16, EPI_ROWS_Q, FMT_BF16>(d, st);
    return launch<FMT_BF16, EPI_TOKENS, FMT_BF16>(d, st);
}

}  // namespace dq
