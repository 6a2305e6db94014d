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
// One workgroup owns up to 64 slot rows (whole cubes when a cube has at most
// 64 tokens) and walks the channels in chunks: the chunk of X is staged in
// LDS once (channel-contiguous, coalesced row segments) and then used three
// times -- for the cube sums, for the deltas, and as the bf16 MFMA operand of
// U -- so X is read from HBM exactly once.  Cubes of more than 64 tokens take
// two extra small passes (64-token partial sums, then their ordered combine)
// and X is read twice.
#include <type_traits>

#include "dq_device.h"

namespace dq {

constexpr int QROWS = 64;          // slot rows per workgroup
constexpr int QTHREADS = 256;      // wave 0: copies; wave 1: U; waves 2-3: quantizer
constexpr int QROWB = 512;         // bytes of one row's channel chunk in LDS
constexpr int QCHUNK = QROWS * QROWB;
constexpr int QNBUF = 2;           // chunk buffers (two workgroups fit one CU)

template <typename XT> struct XTraits;
template <> struct XTraits<float> {
    static constexpr int CC = QROWB / 4;   // 128 channels per chunk
    __device__ static float f(float v) { return v; }
};
template <> struct XTraits<uint16_t> {
    static constexpr int CC = QROWB / 2;   // 256 channels per chunk
    __device__ static float f(uint16_t v) { return bf16_to_f32(v); }
};

struct QuantArgs {
    const void* x;            // [N][Ci]
    Geom g;
    int Ci, Kp, rp;
    int core_mode;            // 0: cores computed here (S <= 64); 1: read from coref
    uint8_t* dq;              // Nslot_pad x Kp/2, step-major
    uint8_t* ds;              // Nslot_pad x Kp/32, step-major
    uint8_t* cq;              // K_pad x Kp, step-major
    uint8_t* cs;              // K_pad x Kp/32, step-major
    uint16_t* u;              // [Nslot_pad][rp]
    const uint16_t* l1t;      // [rp][Kp], zero beyond Ci
    const float* coref;       // [K][Kp] (core_mode 1)
    const uint8_t* zero;      // QROWB zero bytes (source of absent rows and channels)
};

// LDS chunk layout: 16-byte chunk c of row r at r QROWB + ((c ^ (r & 15)) << 4);
// the XOR makes both the quantizer's row reads and the MFMA's column reads
// free of bank conflicts.
__device__ __forceinline__ int qoff(int r, int c) { return r * QROWB + ((c ^ (r & 15)) << 4); }

// 32 channels (one group) of row r from a chunk buffer, as fp32
template <typename XT>
__device__ __forceinline__ void qload(const uint8_t* buf, int r, int gc, float* v) {
    if constexpr (sizeof(XT) == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 w = *(const uint4*)(buf + qoff(r, 4 * gc + q));
            const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[8 * q + 2 * i] = __uint_as_float(d[i] << 16);
                v[8 * q + 2 * i + 1] = __uint_as_float(d[i] & 0xffff0000u);
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float4 w = *(const float4*)(buf + qoff(r, 8 * gc + q));
            v[4 * q] = w.x;
            v[4 * q + 1] = w.y;
            v[4 * q + 2] = w.z;
            v[4 * q + 3] = w.w;
        }
    }
}

// One workgroup owns up to 64 slot rows (whole cubes when a cube has at most
// 64 tokens) and walks the channels in chunks of 512 bytes per row.  Wave 0
// copies each chunk of X straight into LDS (global_load_lds, one 16-byte
// piece per lane, absent rows and channels from a zero page) one chunk ahead;
// wave 1 accumulates U = bf16(X) L1 with 32x32x16 bf16 MFMAs; waves 2-3 run
// one (cube, 32-channel group) per thread: the cube's core from its rows
// (fp32 sum in slot order, then the division), the core's FP8 codes, and each
// row's delta FP4 codes.  X is read from HBM exactly once.
template <typename XT, int NCT>
__global__ __launch_bounds__(QTHREADS, 2) void k_quantize(QuantArgs a) {
    constexpr int CC = XTraits<XT>::CC;
    constexpr int NGC = CC / 32;                     // groups per chunk
    constexpr int EPC = 16 / (int)sizeof(XT);        // elements per 16-byte chunk
    __shared__ __attribute__((aligned(1024))) uint8_t xbuf[QNBUF * QCHUNK];
    __shared__ int tok_s[QROWS];
    __shared__ int rb_s[QROWS], re_s[QROWS], cnt_s[QROWS];

    const Geom& g = a.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    // ---- rows and cubes of this workgroup
    long long k_first, slot0;
    int nrows, ncores;
    if (a.core_mode == 0) {
        const int cpb = QROWS / g.S;
        k_first = (long long)blockIdx.x * cpb;
        ncores = (int)min((long long)cpb, g.K - k_first);
        slot0 = k_first * g.S;
        nrows = ncores * g.S;
    } else {
        slot0 = (long long)blockIdx.x * QROWS;
        nrows = (int)min((long long)QROWS, g.Nslot - slot0);
        k_first = slot0 / g.S;
        ncores = (int)((slot0 + nrows - 1) / g.S - k_first + 1);
    }
    if (tid < QROWS) {
        const long long s = slot0 + tid;
        tok_s[tid] = tid < nrows ? (int)slot_token(g, s) : -1;
    }
    if (tid < ncores) {
        const long long k = k_first + tid;
        rb_s[tid] = (int)max(0LL, k * g.S - slot0);
        re_s[tid] = (int)min((long long)nrows, (k + 1) * g.S - slot0);
        int ct, ch, cw;
        cnt_s[tid] = cube_count(g, k, &ct, &ch, &cw);
    }
    __syncthreads();

    const int nchunks = (a.Ci + CC - 1) / CC;
    const uint32_t lds0 = (uint32_t)(uintptr_t)xbuf;
    const XT* __restrict__ x = (const XT*)a.x;

    // wave 0: the 32 copies of chunk ci into buffer ci % QNBUF (two rows per
    // copy; a lane of an absent row or channel reads the zero page)
    auto issue = [&](int ci) {
        const int c0 = ci * CC;
        const uint32_t base = lds0 + (uint32_t)(ci % QNBUF) * QCHUNK;
        int t[QROWS / 2];
#pragma unroll
        for (int j = 0; j < QROWS / 2; ++j) t[j] = tok_s[2 * j + (lane >> 5)];
#pragma unroll
        for (int j = 0; j < QROWS / 2; ++j) {
            const int r = 2 * j + (lane >> 5);
            const int ch = c0 + ((lane & 31) ^ (r & 15)) * EPC;   // first channel of the logical chunk at this position
            const void* src = (t[j] >= 0 && ch < a.Ci) ? (const void*)(x + (long long)t[j] * a.Ci + ch)
                                                       : (const void*)(a.zero + 16 * (lane & 31));
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(base + j * 2 * QROWB), "v"(src)
                         : "memory", "m0");
        }
    };
    auto barrier = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // U accumulators (wave 1): two 32-row tiles x NCT 32-wide rank tiles
    v16f uacc[2][NCT > 0 ? NCT : 1];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < (NCT > 0 ? NCT : 1); ++j) uacc[i][j] = (v16f){};
    // L1 fragments of rank tile ct for the chunk at channel c0 (16 channels per fragment)
    constexpr int NL = NCT == 1 ? CC / 16 : 4;       // fragments per load batch
    uint4 lcur[NL], lnext[NCT == 1 ? NL : 1];
    auto load_l1 = [&](int c0, int ct, uint4* dst) {
#pragma unroll
        for (int q = 0; q < NL; ++q) {
            const int c = c0 + 16 * q + 8 * (lane >> 5);
            dst[q] = c < a.Kp ? *(const uint4*)(a.l1t + (long long)(ct * 32 + (lane & 31)) * a.Kp + c) : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    if (NCT == 1 && wave == 1) load_l1(0, 0, lnext);

    if (wave == 0) {
        issue(0);
        if (nchunks > 1) issue(1);
    }
    for (int ci = 0; ci < nchunks; ++ci) {
        const int c0 = ci * CC;
        const uint8_t* buf = xbuf + (ci % QNBUF) * QCHUNK;
        if (wave == 0) {
            if (ci + 1 < nchunks) __builtin_amdgcn_s_waitcnt((32 & 15) | ((32 >> 4) << 14) | 0x0F70);   // chunk ci landed
            else __builtin_amdgcn_s_waitcnt(0x0F70);
        }
        barrier();   // chunk ci visible to every wave

        if (NCT > 0 && wave == 1) {
            // ---- U += bf16(X chunk) L1 chunk.  L1 fragments come from global
            // memory (L2-resident); with one rank tile they are loaded a chunk
            // ahead, otherwise one tile's worth per batch.
            const int kend = min(CC, a.Kp - c0);
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
            if constexpr (NCT == 1) {
#pragma unroll
                for (int q = 0; q < CC / 16; ++q) lcur[q] = lnext[q];
                if (ci + 1 < nchunks) load_l1(c0 + CC, 0, lnext);
#pragma unroll
                for (int q = 0; q < CC / 16; ++q) {
                    if (16 * q < kend) {
                        const v8bf bv = __builtin_bit_cast(v8bf, lcur[q]);
                        uacc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_frag(0, 16 * q), bv, uacc[0][0], 0, 0, 0);
                        uacc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_frag(1, 16 * q), bv, uacc[1][0], 0, 0, 0);
                    }
                }
            } else {
                for (int kb = 0; kb < kend; kb += 16 * NL) {
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        load_l1(c0 + kb, ct, lcur);
#pragma unroll
                        for (int q = 0; q < NL; ++q) {
                            if (kb + 16 * q < kend) {
                                const v8bf bv = __builtin_bit_cast(v8bf, lcur[q]);
                                uacc[0][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_frag(0, kb + 16 * q), bv, uacc[0][ct], 0, 0, 0);
                                uacc[1][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_frag(1, kb + 16 * q), bv, uacc[1][ct], 0, 0, 0);
                            }
                        }
                    }
                }
            }
        } else if (wave >= 2) {
            // ---- quantizer: one (cube, group) per thread
            const long long nks = a.Kp / 128;
            for (int t = tid - 128; t < ncores * NGC; t += 128) {
                const int cr = t / NGC, gc = t - cr * NGC;
                const long long G = (c0 >> 5) + gc;
                if (G * 32 >= a.Ci) continue;
                const int rb = rb_s[cr], re = re_s[cr];
                const long long k = k_first + cr;
                float core[32];
                if (a.core_mode == 0) {
                    bool first = true;
                    for (int r = rb; r < re; ++r) {
                        if (tok_s[r] < 0) continue;
                        float v[32];
                        qload<XT>(buf, r, gc, v);
#pragma unroll
                        for (int i = 0; i < 32; ++i) core[i] = first ? v[i] : core[i] + v[i];
                        first = false;
                    }
                    const int cnt = cnt_s[cr];
                    float amax = 0.0f;
#pragma unroll
                    for (int i = 0; i < 32; ++i) {
                        core[i] = mean_div(core[i], cnt);
                        amax = fmaxf(amax, fabsf(core[i]));
                    }
                    const int e = mx_exp_fp8(amax);
                    uint4 lo, hi;
                    encode_fp8x32(core, pow2f(e), lo, hi);
                    *(uint4*)(a.cq + off_fp8(k, G >> 2, 2 * (int)(G & 3), nks)) = lo;
                    *(uint4*)(a.cq + off_fp8(k, G >> 2, 2 * (int)(G & 3) + 1, nks)) = hi;
                    a.cs[off_scale(k, G, nks)] = (uint8_t)(e + 127);
                } else {
                    const float4* cp = (const float4*)(a.coref + k * (long long)a.Kp + G * 32);
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const float4 w = cp[q];
                        core[4 * q] = w.x;
                        core[4 * q + 1] = w.y;
                        core[4 * q + 2] = w.z;
                        core[4 * q + 3] = w.w;
                    }
                }
                for (int r = rb; r < re; ++r) {
                    if (tok_s[r] < 0) continue;
                    float v[32];
                    qload<XT>(buf, r, gc, v);
                    float amax = 0.0f;
#pragma unroll
                    for (int i = 0; i < 32; ++i) {
                        v[i] = v[i] - core[i];
                        amax = fmaxf(amax, fabsf(v[i]));
                    }
                    const int e = mx_exp_fp4(amax);
                    const long long s = slot0 + r;
                    *(uint4*)(a.dq + off_fp4(s, G, nks)) = encode_fp4x32(v, pow2f(e));
                    a.ds[off_scale(s, G, nks)] = (uint8_t)(e + 127);
                }
            }
        }
        barrier();   // every wave is done with buffer ci % QNBUF
        if (wave == 0 && ci + QNBUF < nchunks) issue(ci + QNBUF);
    }

    // ---- U -> bf16, slot order (rows of absent tokens were zero)
    if (wave == 1) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = rt * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                    if (row < nrows) a.u[(slot0 + row) * a.rp + ct * 32 + (lane & 31)] = bf16_rne(uacc[rt][ct][i]);
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

template <typename XT>
__global__ __launch_bounds__(256) void k_core_partial(PartialArgs a) {
    const Geom& g = a.g;
    long long kb = blockIdx.x;
    long long k = kb / a.nblk;
    long long b = kb - k * a.nblk;
    int c = blockIdx.y * 256 + threadIdx.x;
    if (c >= a.Ci) return;
    int ct, ch, cw;
    int cnt = cube_count(g, k, &ct, &ch, &cw);
    long long j0 = b * CORE_BLOCK;
    if (j0 >= cnt) return;
    int j1 = (int)min((long long)cnt, j0 + CORE_BLOCK);
    long long kw = k % g.Wc, kh = (k / g.Wc) % g.Hc, kt = k / ((long long)g.Wc * g.Hc);
    const XT* x = (const XT*)a.x;
    float s = 0.0f;
    for (int j = (int)j0; j < j1; ++j) {   // j-th present token, lexicographic in the clipped cube
        int dw = j % cw, dh = (j / cw) % ch, dt = j / (cw * ch);
        long long n = ((kt * g.t + dt) * g.H + kh * g.h + dh) * g.W + kw * g.w + dw;
        float v = XTraits<XT>::f(x[n * a.Ci + c]);
        s = (j == j0) ? v : s + v;
    }
    a.part[kb * a.Kp + c] = s;
}

struct CombineArgs {
    Geom g;
    int Ci, Kp;
    long long nblk;
    const float* part;
    float* coref;    // [K][Kp]
    uint8_t* cq;     // K_pad x Kp, step-major
    uint8_t* cs;     // K_pad x Kp/32, step-major
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
        for (int b = 1; b < nb; ++b) s = s + p[(long long)b * a.Kp];
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
        int e = mx_exp_fp8(amax);
        uint4 lo, hi;
        encode_fp8x32(v, pow2f(e), lo, hi);
        const long long G = cg >> 5, nks = a.Kp / 128;
        *(uint4*)(a.cq + off_fp8(k, G >> 2, 2 * (int)(G & 3), nks)) = lo;
        *(uint4*)(a.cq + off_fp8(k, G >> 2, 2 * (int)(G & 3) + 1, nks)) = hi;
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

// Slot -> token table of the GEMM epilogue (-1 for pad slots).
__global__ __launch_bounds__(256) void k_slot_tokens(Geom g, int* stok, long long n) {
    long long s = (long long)blockIdx.x * 256 + threadIdx.x;
    if (s < n) stok[s] = s < g.Nslot ? (int)slot_token(g, s) : -1;
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

hipError_t launch_quantize(const dq_weights* w, const void* x, int x_bf16, dq_qact* q, hipStream_t st) {
    const Geom& g = q->g;
    if (q->core_mode == 1) {
        PartialArgs pa{x, g, (int)q->Ci, (int)q->Kp, q->nblk, q->part};
        dim3 grid((unsigned)(g.K * q->nblk), (unsigned)((q->Ci + 255) / 256));
        if (x_bf16) k_core_partial<uint16_t><<<grid, 256, 0, st>>>(pa);
        else k_core_partial<float><<<grid, 256, 0, st>>>(pa);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        CombineArgs ca{g, (int)q->Ci, (int)q->Kp, q->nblk, q->part, q->coref, q->cq, q->cs};
        dim3 grid2((unsigned)g.K, (unsigned)((q->Ci + 255) / 256));
        k_core_combine<<<grid2, 256, 0, st>>>(ca);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    QuantArgs a{};
    a.x = x;
    a.g = g;
    a.Ci = (int)q->Ci;
    a.Kp = (int)q->Kp;
    a.rp = q->rp;
    a.core_mode = q->core_mode;
    a.dq = q->dq;
    a.ds = q->ds;
    a.cq = q->cq;
    a.cs = q->cs;
    a.u = q->u;
    a.l1t = w->l1t;
    a.coref = q->coref;
    a.zero = q->zero;
    const long long cpb = QROWS / g.S;
    unsigned blocks = q->core_mode == 0 ? (unsigned)((g.K + cpb - 1) / cpb) : (unsigned)((g.Nslot + QROWS - 1) / QROWS);
    const int nct = q->rp / 32;
    auto go = [&](auto XT_, auto NCT_) {
        using XT = decltype(XT_);
        k_quantize<XT, decltype(NCT_)::value><<<blocks, QTHREADS, 0, st>>>(a);
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
    return hipGetLastError();
}

hipError_t launch_slot_tokens(const Geom& g, int* stok, int64_t n, hipStream_t st) {
    k_slot_tokens<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(g, stok, n);
    return hipGetLastError();
}

}  // namespace dq
