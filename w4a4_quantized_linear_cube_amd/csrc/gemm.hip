// Scaled-MFMA GEMMs of the delta-W4A4 layer (gfx950).
//
// DeltaQuant notes, 关键设计 4 (the three-term equation):
//   y_n = U_n L2 + Q8(core_k(n)) Q4(R) + Q4(delta_n) Q4(R)
// The core term is one row per cube (the "dynamic token bias", broadcast to
// the cube's tokens); the delta term is one row per token.  Two launches of
// one kernel template: the core GEMM (A = FP8 E4M3 cores, one row per cube)
// writes the per-cube term; the delta GEMM (A = FP4 E2M1 deltas, one row per
// slot) adds U L2, adds its cube's core term in the epilogue and scatters rows
// to token order.  Both are V_MFMA_SCALE_F32_32X32X64_F8F6F4 contractions
// over Ci with the E8M0 block scales applied inside the instruction, fp32
// accumulation.
//
// Work decomposition: a 256-thread workgroup computes a 256 x 256 output
// tile; its four waves each own 128 x 128 (4 x 4 MFMA tiles of 32 x 32,
// 256 accumulator registers).
//
// Data movement: three LDS stages of one K step (128 channels) each.  A
// codes, B codes and their E8M0 scale bytes go straight from global memory
// into the stage two steps ahead (global_load_lds, no staging registers)
// while the MFMAs run on the current stage; before the barrier that ends a
// step each wave waits only for its copies of the next stage.  LDS rows hold
// 16-byte chunks XOR-swizzled so every fragment read is free of bank
// conflicts.  Rows, columns and K of every operand are padded to the tile
// with zero codes and zero scales, so the main loop has no bounds checks.
//
// Tile order: workgroups are dispatched round-robin over the 8 XCDs; tile
// indices are remapped so the workgroups resident on one XCD at a time cover
// a compact block of 4 row tiles x 8 column tiles and share their A and B
// stages in that XCD's L2.
#include <type_traits>

#include "dq_device.h"

namespace dq {

struct GemmArgs {
    const uint8_t* a;   // A codes, rows of lda bytes
    const uint8_t* as;  // A scale codes, rows of ldas bytes
    long long lda, ldas;
    const uint8_t* b;   // B = Q4(R) codes [Cop][Kp/2]
    const uint8_t* bs;  // B scale codes [Cop][Kp/32]
    long long ldb, ldbs;
    int Kp;             // multiple of 128
    int mtiles, ntiles;
    float* c;           // plain store epilogue: c[row][col]
    long long ldc;
    float* y;           // token epilogue: y[token][col]
    int Co;
    Geom g;
    const float* bias;  // per-cube core term [K_pad][ldbias]
    long long ldbias;
    const uint16_t* u;     // [Nslot_pad][rp]
    const uint16_t* l2t;   // [Cop][rp]
    int rp;
};

constexpr int EPI_STORE = 0;
constexpr int EPI_TOKENS = 1;

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
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff),
                 "s"(uniform_ptr(base)) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff),
                 "s"(uniform_ptr(base)) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in
// bits 15:14; expcnt 7 and lgkmcnt 15 mean no wait on those counters)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// XOR swizzles of 16-byte chunks within an LDS row.
__device__ __forceinline__ int swz64(int row) { return (row >> 1) & 3; }   // 64-byte rows (4 chunks)
__device__ __forceinline__ int swz128(int row) { return row & 7; }         // 128-byte rows (8 chunks)

template <int AFMT, int OPSEL>
__device__ __forceinline__ v16f mfma32(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, AFMT, FMT_FP4, OPSEL, sa, OPSEL, sb);
}

// Tile of workgroup `bid` (see the file comment); returns false for the
// padding workgroups beyond the tile count.
__device__ __forceinline__ bool tile_of(int bid, int mt, int nt, int* tm, int* tn) {
    const int total = mt * nt;
    const int per = (total + 7) / 8;
    const int v = (bid & 7) * per + (bid >> 3);
    if (v >= total) return false;
    constexpr int GM = 4;
    const int grp = v / (GM * nt);
    const int first = grp * GM;
    const int gm = min(GM, mt - first);
    const int within = v - grp * GM * nt;
    *tm = first + within % gm;
    *tn = within / gm;
    return true;
}

template <int AFMT, int EPI>
__global__ __launch_bounds__(256, 1) void k_gemm(GemmArgs p) {
    constexpr int AROW = AFMT == FMT_FP4 ? 64 : 128;            // A bytes per row per 128-wide K step
    constexpr int A_BYTES = 256 * AROW;
    constexpr int B_BYTES = 256 * 64;
    constexpr int SA_OFF = A_BYTES + B_BYTES;
    constexpr int SB_OFF = SA_OFF + 1024;
    constexpr int STAGE = SB_OFF + 1024;
    constexpr int NS = AFMT == FMT_FP4 ? 4 : 3;                // LDS stages in the ring
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];
    __shared__ long long rtok[EPI == EPI_TOKENS ? 256 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int g = lane >> 5, l32 = lane & 31;
    int tm, tn;
    if (!tile_of(blockIdx.x, p.mtiles, p.ntiles, &tm, &tn)) return;
    const long long m0 = (long long)tm * 256, n0 = (long long)tn * 256;

    if (EPI == EPI_TOKENS) {
        long long slot = m0 + tid;
        rtok[tid] = slot < p.g.Nslot ? slot_token(p.g, slot) : -1;
    }

    // ---- this lane's copy sources: uniform tile bases + per-lane 32-bit offsets.
    // A: 256 rows x AROW bytes per stage = APC pieces of 1 KB per wave.
    constexpr int APC = A_BYTES / 1024 / 4;       // pieces per wave (4 or 8)
    constexpr int ACH = AROW / 16;                // 16-byte chunks per A row
    constexpr int DMAS = APC + 4 + 2;             // copies per wave per stage
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    uint32_t aoff[APC], boff[4];
#pragma unroll
    for (int j = 0; j < APC; ++j) {
        int lin = (wv * APC + j) * 64 + lane;     // 16-byte chunk index within the stage
        int row = lin / ACH, pc = lin % ACH;
        int ch = AFMT == FMT_FP4 ? (pc ^ swz64(row)) : (pc ^ swz128(row));
        aoff[j] = (uint32_t)(row * p.lda + ch * 16);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        int lin = (wv * 4 + j) * 64 + lane;
        int row = lin >> 2, pc = lin & 3;
        boff[j] = (uint32_t)(row * p.ldb + (pc ^ swz64(row)) * 16);
    }
    const uint32_t asoff = (uint32_t)((wv * 64 + lane) * p.ldas);
    const uint32_t bsoff = (uint32_t)((wv * 64 + lane) * p.ldbs);
    const uint8_t* abase = p.a + m0 * p.lda;
    const uint8_t* bbase = p.b + n0 * p.ldb;
    const uint8_t* asbase = p.as + m0 * p.ldas;
    const uint8_t* bsbase = p.bs + n0 * p.ldbs;
    const uint32_t lds0 = lds_addr(smem);

    auto issue = [&](int kt, int buf) {
        const uint32_t st = lds0 + buf * STAGE;
#pragma unroll
        for (int j = 0; j < APC; ++j) dma16(abase + (long long)kt * AROW, aoff[j], st + (wv * APC + j) * 1024);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(bbase + kt * 64, boff[j], st + A_BYTES + (wv * 4 + j) * 1024);
        dma4(asbase + kt * 4, asoff, st + SA_OFF + wv * 256);
        dma4(bsbase + kt * 4, bsoff, st + SB_OFF + wv * 256);
    };

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (v16f){};

    // ---- low-rank branch first (registers are free here): acc = U L2 with
    // 32x32x16 bf16 MFMAs over the padded rank; the K loop accumulates on top.
    if (EPI == EPI_TOKENS) {
        for (int kq = 0; kq < p.rp; kq += 16) {
            v8bf ua[4], lb[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                long long row = m0 + wr * 128 + l32 + 32 * mi;
                ua[mi] = __builtin_bit_cast(v8bf, *(const uint4*)(p.u + row * p.rp + kq + 8 * g));
            }
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                long long col = n0 + wc * 128 + l32 + 32 * ni;
                lb[ni] = __builtin_bit_cast(v8bf, *(const uint4*)(p.l2t + col * p.rp + kq + 8 * g));
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ua[mi], lb[ni], acc[mi][ni], 0, 0, 0);
        }
    }
    // LDS fragment addresses (bytes within a stage)
    const int arow0 = wr * 128 + l32;           // + 32 mi
    const int brow0 = wc * 128 + l32;           // + 32 ni
    const int sa_sw = AFMT == FMT_FP4 ? swz64(arow0) : swz128(arow0);
    const int sb_sw = swz64(brow0);

    // Fragments of one K step (both 64-wide halves), read from LDS one step
    // ahead of their MFMAs into a second register set.
    struct Frag {
        uint4 a[2][4], a2[AFMT == FMT_FP4 ? 1 : 2][4], b[2][4];
        uint32_t sa[4], sb[4];
    };
    auto load_frags = [&](int buf, Frag& F) {
        const uint8_t* st = smem + buf * STAGE;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) F.sa[mi] = *(const uint32_t*)(st + SA_OFF + (arow0 + 32 * mi) * 4) >> (8 * g);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) F.sb[ni] = *(const uint32_t*)(st + SB_OFF + (brow0 + 32 * ni) * 4) >> (8 * g);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const uint8_t* rowp = st + (arow0 + 32 * mi) * AROW;
                if constexpr (AFMT == FMT_FP4) {
                    F.a[kk][mi] = *(const uint4*)(rowp + (((2 * kk + g) ^ sa_sw) << 4));
                } else {
                    F.a[kk][mi] = *(const uint4*)(rowp + (((4 * kk + g) ^ sa_sw) << 4));
                    F.a2[kk][mi] = *(const uint4*)(rowp + (((4 * kk + 2 + g) ^ sa_sw) << 4));
                }
            }
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                F.b[kk][ni] = *(const uint4*)(st + A_BYTES + (brow0 + 32 * ni) * 64 + (((2 * kk + g) ^ sb_sw) << 4));
        }
    };
    auto mfma_step = [&](const Frag& F) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const uint4 v = F.a[kk][mi];
                v8i af;
                if constexpr (AFMT == FMT_FP4) {
                    af = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
                } else {
                    const uint4 w = F.a2[kk][mi];
                    af = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, (int)w.x, (int)w.y, (int)w.z, (int)w.w};
                }
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) {
                    const uint4 u = F.b[kk][ni];
                    const v8i bf = (v8i){(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
                    if (kk == 0)
                        acc[mi][ni] = mfma32<AFMT, 0>(af, bf, acc[mi][ni], (int)F.sa[mi], (int)F.sb[ni]);
                    else
                        acc[mi][ni] = mfma32<AFMT, 2>(af, bf, acc[mi][ni], (int)F.sa[mi], (int)F.sb[ni]);
                }
            }
    };

    const int nk = p.Kp / 128;
    if constexpr (AFMT == FMT_FP4) {
        // ---- K loop over a ring of NS stages.  Step kt: copies for stage
        // kt + NS - 1 go out (into the stage whose fragments were read at step
        // kt - 2, long since consumed); wait for this wave's copies of stage
        // kt + 1; barrier (now every wave's copies of kt + 1 have landed); read
        // the fragments of kt + 1; run the MFMAs of kt from the fragments read
        // one step earlier, so the MFMAs never wait for LDS.
        for (int st = 0; st < NS - 1; ++st)
            if (st < nk) issue(st, st);
        if (nk >= NS - 1) wait_vm<(NS - 2) * DMAS>();   // stage 0 landed
        else wait_vm<0>();
        __syncthreads();
        Frag F0, F1;
        load_frags(0, F0);
        auto step = [&](int kt, Frag& cur, Frag& nxt, auto STEADY) {
            if constexpr (decltype(STEADY)::value) {
                issue(kt + NS - 1, (kt + NS - 1) % NS);
                wait_vm<(NS - 2) * DMAS>();              // stage kt + 1 landed; later ones may be in flight
            } else {
                if (kt + NS - 1 < nk) issue(kt + NS - 1, (kt + NS - 1) % NS);
                wait_vm<0>();
            }
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 1 < nk) load_frags((kt + 1) % NS, nxt);
            mfma_step(cur);
        };
        int kt = 0;
        for (; kt + NS < nk; kt += 2) {                 // steps kt and kt + 1 both issue copies
            step(kt, F0, F1, std::true_type{});
            step(kt + 1, F1, F0, std::true_type{});
        }
        for (; kt < nk; kt += 2) {                      // kt stays even: F0 always serves even steps
            step(kt, F0, F1, std::false_type{});
            if (kt + 1 < nk) step(kt + 1, F1, F0, std::false_type{});
        }
    } else {
        // FP8 fragments are twice as wide, so a second register set does not
        // fit beside 256 accumulators: read each step's fragments in the step.
        // Step kt: copies for kt + NS - 1 out, fragments of kt read and MFMAs
        // run, then wait for stage kt + 1 and barrier.
        for (int st = 0; st < NS - 1; ++st)
            if (st < nk) issue(st, st);
        if (nk >= NS - 1) wait_vm<(NS - 2) * DMAS>();
        else wait_vm<0>();
        __syncthreads();
        // one 64-wide K half at a time keeps only half the fragments live
        auto compute = [&](int buf) {
            const uint8_t* st = smem + buf * STAGE;
            uint32_t sa[4], sb[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) sa[mi] = *(const uint32_t*)(st + SA_OFF + (arow0 + 32 * mi) * 4) >> (8 * g);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) sb[ni] = *(const uint32_t*)(st + SB_OFF + (brow0 + 32 * ni) * 4) >> (8 * g);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                v8i af[4], bf[4];
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    const uint8_t* rowp = st + (arow0 + 32 * mi) * AROW;
                    uint4 v0 = *(const uint4*)(rowp + (((4 * kk + g) ^ sa_sw) << 4));
                    uint4 v1 = *(const uint4*)(rowp + (((4 * kk + 2 + g) ^ sa_sw) << 4));
                    af[mi] = (v8i){(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
                }
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) {
                    uint4 v = *(const uint4*)(st + A_BYTES + (brow0 + 32 * ni) * 64 + (((2 * kk + g) ^ sb_sw) << 4));
                    bf[ni] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
                }
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        if (kk == 0) acc[mi][ni] = mfma32<AFMT, 0>(af[mi], bf[ni], acc[mi][ni], (int)sa[mi], (int)sb[ni]);
                        else acc[mi][ni] = mfma32<AFMT, 2>(af[mi], bf[ni], acc[mi][ni], (int)sa[mi], (int)sb[ni]);
                    }
            }
        };
        int kt = 0;
        for (; kt + NS - 1 < nk; ++kt) {
            issue(kt + NS - 1, (kt + NS - 1) % NS);
            compute(kt % NS);
            __builtin_amdgcn_sched_barrier(0);          // keep the MFMAs above the wait
            wait_vm<(NS - 2) * DMAS>();
            __syncthreads();
        }
        for (; kt < nk; ++kt) {
            compute(kt % NS);
            __builtin_amdgcn_sched_barrier(0);
            wait_vm<0>();
            __syncthreads();
        }
    }
    __syncthreads();

    if (EPI == EPI_STORE) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    long long row = m0 + wr * 128 + mi * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                    long long col = n0 + wc * 128 + ni * 32 + l32;
                    p.c[row * p.ldc + col] = acc[mi][ni][i];
                }
        return;
    }

    // ---- epilogue: y = acc + bias[cube], rows scattered to token order.
    // The cube's core-term rows are staged in LDS, 64 slots (one 32-row MFMA
    // block mi of each wave row) per phase, with the same register-free
    // direct copies: one 1 KB row per wave instruction.
    float* bl = (float*)smem;                              // [64 slots][256 columns]
    const int S = p.g.S;
    const long long kmax = p.g.K - 1;
    auto bias_rows = [&](int mi) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int q = wv * 16 + j;                     // LDS row: wave row q / 32, row q % 32 of block mi
            const long long slot = m0 + (q >> 5) * 128 + mi * 32 + (q & 31);
            const long long k = min(slot / S, kmax);       // pad slots: any valid row, never stored
            dma16(p.bias + k * p.ldbias + n0, (uint32_t)lane * 16, lds0 + q * 1024);
        }
    };
    bias_rows(0);

#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        wait_vm<0>();
        __syncthreads();                                   // phase mi's rows have landed
        long long yoff[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const long long t = rtok[wr * 128 + mi * 32 + 8 * (i >> 2) + 4 * g + (i & 3)];
            yoff[i] = t < 0 ? -1 : t * (long long)p.Co + n0;
        }
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const int col = wc * 128 + ni * 32 + l32;
            float bv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) bv[i] = bl[(wr * 32 + 8 * (i >> 2) + 4 * g + (i & 3)) * 256 + col];
            if (n0 + col < p.Co) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (yoff[i] >= 0) p.y[yoff[i] + col] = acc[mi][ni][i] + bv[i];
            }
        }
        __syncthreads();                                   // every wave is done with phase mi's rows
        if (mi < 3) bias_rows(mi + 1);
    }
}

template <int AFMT, int EPI>
static hipError_t launch(const GemmArgs& a, hipStream_t st) {
    int total = a.mtiles * a.ntiles;
    int grid = (total + 7) / 8 * 8;
    k_gemm<AFMT, EPI><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_forward(const dq_weights* w, dq_qact* q, float* y, hipStream_t st) {
    GemmArgs d{};
    d.b = w->rq;
    d.bs = w->rs;
    d.ldb = w->Kp / 2;
    d.ldbs = w->Kp / 32;
    d.Kp = (int)w->Kp;
    d.ntiles = (int)(w->Cop / 256);
    d.a = q->dq;
    d.as = q->ds;
    d.lda = q->Kp / 2;
    d.ldas = q->Kp / 32;
    d.mtiles = (int)(q->Nslot_pad / 256);
    d.y = y;
    d.Co = (int)w->Co;
    d.g = q->g;
    d.u = q->u;
    d.l2t = w->l2t;
    d.rp = w->rp;
    // 1) per-cube core term bias[k] = Q8(core_k) Q4(R)
    GemmArgs c = d;
    c.a = q->cq;
    c.as = q->cs;
    c.lda = q->Kp;
    c.ldas = q->Kp / 32;
    c.mtiles = (int)(q->K_pad / 256);
    c.c = q->bias;
    c.ldc = w->Cop;
    hipError_t e = launch<FMT_FP8, EPI_STORE>(c, st);
    if (e != hipSuccess) return e;
    // 2) delta term + low-rank branch + the cube's core term -> y (token order)
    d.bias = q->bias;
    d.ldbias = w->Cop;
    return launch<FMT_FP4, EPI_TOKENS>(d, st);
}

}  // namespace dq
