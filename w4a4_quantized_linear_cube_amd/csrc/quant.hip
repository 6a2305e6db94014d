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
#include "dq_device.h"

namespace dq {

constexpr int QROWS = 64;          // slot rows per workgroup
constexpr int QTHREADS = 256;
constexpr int XTILE_BYTES = 16384; // X chunk staged per step: 64 rows x 256 bytes

template <typename XT> struct XTraits;
template <> struct XTraits<float> {
    static constexpr int CC = XTILE_BYTES / QROWS / 4;   // 64 channels per chunk
    __device__ static float f(float v) { return v; }
    __device__ static uint16_t bf(float v) { return bf16_rne(v); }
};
template <> struct XTraits<uint16_t> {
    static constexpr int CC = XTILE_BYTES / QROWS / 2;   // 128 channels per chunk
    __device__ static float f(uint16_t v) { return bf16_to_f32(v); }
    __device__ static uint16_t bf(uint16_t v) { return v; }
};

struct QuantArgs {
    const void* x;            // [N][Ci]
    Geom g;
    int Ci, Kp, rp;
    int cubes_per_block;      // core_mode 0: whole cubes per workgroup
    int core_mode;            // 0: cores computed here; 1: read from coref
    uint8_t* dq;              // Nslot_pad x Kp/2, step-major
    uint8_t* ds;              // Nslot_pad x Kp/32, step-major
    uint8_t* cq;              // K_pad x Kp, step-major
    uint8_t* cs;              // K_pad x Kp/32, step-major
    uint16_t* u;              // [Nslot_pad][rp]
    const uint16_t* l1t;      // [rp][Kp]
    const float* coref;       // [K][Kp] (core_mode 1)
};

template <typename XT>
__global__ __launch_bounds__(QTHREADS) void k_quantize(QuantArgs a) {
    constexpr int CC = XTraits<XT>::CC;
    constexpr int XLD = CC + 16 / (int)sizeof(XT);   // padded LDS row (elements)
    constexpr int CLD = CC + 4;                      // padded core row (floats)
    constexpr int NG = CC / 32;                      // groups per chunk
    __shared__ __attribute__((aligned(16))) XT xs[QROWS * XLD];
    __shared__ __attribute__((aligned(16))) float cs_tile[QROWS * CLD];
    __shared__ long long tok[QROWS];
    __shared__ long long slot_of[QROWS];
    __shared__ int core_row[QROWS];
    __shared__ int cnt_of[QROWS];

    const Geom& g = a.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const XT* __restrict__ x = (const XT*)a.x;

    // ---- rows of this workgroup
    long long k_first, slot0;
    int nrows, ncores;
    if (a.core_mode == 0) {
        k_first = (long long)blockIdx.x * a.cubes_per_block;
        ncores = (int)min((long long)a.cubes_per_block, g.K - k_first);
        slot0 = k_first * g.S;
        nrows = ncores * g.S;
    } else {
        slot0 = (long long)blockIdx.x * QROWS;
        nrows = (int)min((long long)QROWS, g.Nslot - slot0);
        k_first = slot0 / g.S;
        ncores = (int)((slot0 + nrows - 1) / g.S - k_first + 1);
    }
    if (tid < QROWS) {
        long long s = slot0 + tid;
        bool in = tid < nrows;
        tok[tid] = in ? slot_token(g, s) : -1;
        slot_of[tid] = s;
        core_row[tid] = in ? (int)(s / g.S - k_first) : 0;
    }
    if (a.core_mode == 0 && tid < ncores) {
        int ct, ch, cw;
        cnt_of[tid] = cube_count(g, k_first + tid, &ct, &ch, &cw);
    }
    __syncthreads();

    // ---- U accumulators: waves 0 and 1 own row tiles 0 and 1; rp/32 column tiles
    const int nct = a.rp / 32;
    v16f uacc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) uacc[i] = (v16f){};

    // global -> register staging of one X chunk: 4 x 16 bytes per thread
    constexpr int PIECES = 16;                  // 16-byte pieces per row chunk
    constexpr int EPP = 16 / (int)sizeof(XT);   // elements per piece
    uint4 stage[4];
    auto load_chunk = [&](int c0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int row = (tid >> 4) + 16 * i;
            int piece = tid & 15;
            long long n = tok[row];
            int c = c0 + piece * EPP;
            if (n >= 0 && c < a.Ci)
                stage[i] = *(const uint4*)(x + n * (long long)a.Ci + c);
            else
                stage[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_chunk = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int row = (tid >> 4) + 16 * i;
            int piece = tid & 15;
            *(uint4*)(&xs[row * XLD + piece * EPP]) = stage[i];
        }
    };

    const int nchunks = (a.Ci + CC - 1) / CC;
    load_chunk(0);
    for (int ci = 0; ci < nchunks; ++ci) {
        const int c0 = ci * CC;
        const int cvalid = min(CC, a.Ci - c0);
        store_chunk();
        if (ci + 1 < nchunks) load_chunk(c0 + CC);
        __syncthreads();

        // ---- cores of this chunk -> cs_tile
        if (a.core_mode == 0) {
            const int S = g.S;
            for (int idx = tid; idx < ncores * CC; idx += QTHREADS) {
                int cr = idx / CC, c = idx - cr * CC;
                if (c >= cvalid) continue;
                int r0 = cr * S;
                float s = 0.0f;
                bool first = true;
                for (int j = 0; j < S; ++j) {
                    if (tok[r0 + j] < 0) continue;
                    float v = XTraits<XT>::f(xs[(r0 + j) * XLD + c]);
                    s = first ? v : s + v;
                    first = false;
                }
                cs_tile[cr * CLD + c] = mean_div(s, cnt_of[cr]);
            }
        } else {
            for (int idx = tid; idx < ncores * CC; idx += QTHREADS) {
                int cr = idx / CC, c = idx - cr * CC;
                if (c >= cvalid) continue;
                cs_tile[cr * CLD + c] = a.coref[(k_first + cr) * (long long)a.Kp + c0 + c];
            }
        }

        // ---- U += bf16(X chunk) L1^T chunk  (32x32x16 bf16 MFMA, waves 0 and 1)
        if (wave < 2) {
            const int row = wave * 32 + (lane & 31);
            const int kh = (lane >> 5) * 8;
            for (int kk = 0; kk < cvalid; kk += 16) {
                v8bf av;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    av[e] = __builtin_bit_cast(__bf16, XTraits<XT>::bf(xs[row * XLD + kk + kh + e]));
                for (int ct = 0; ct < nct; ++ct) {
                    const uint16_t* bp = a.l1t + (long long)(ct * 32 + (lane & 31)) * a.Kp + c0 + kk + kh;
                    uint4 braw = *(const uint4*)bp;
                    v8bf bv = __builtin_bit_cast(v8bf, braw);
                    switch (ct) {
                        case 0: uacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, uacc[0], 0, 0, 0); break;
                        case 1: uacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, uacc[1], 0, 0, 0); break;
                        case 2: uacc[2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, uacc[2], 0, 0, 0); break;
                        default: uacc[3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, uacc[3], 0, 0, 0); break;
                    }
                }
            }
        }
        __syncthreads();

        // ---- core codes (core_mode 0): one (cube, group) per thread
        if (a.core_mode == 0) {
            for (int idx = tid; idx < ncores * NG; idx += QTHREADS) {
                int cr = idx / NG, j = idx - cr * NG;
                if (32 * j >= cvalid) continue;
                float v[32];
                float amax = 0.0f;
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    v[i] = cs_tile[cr * CLD + 32 * j + i];
                    amax = fmaxf(amax, fabsf(v[i]));
                }
                int e = mx_exp_fp8(amax);
                uint4 lo, hi;
                encode_fp8x32(v, pow2f(e), lo, hi);
                const long long k = k_first + cr, G = (c0 >> 5) + j, nks = a.Kp / 128;
                *(uint4*)(a.cq + off_fp8(k, G >> 2, 2 * (int)(G & 3), nks)) = lo;
                *(uint4*)(a.cq + off_fp8(k, G >> 2, 2 * (int)(G & 3) + 1, nks)) = hi;
                a.cs[off_scale(k, G, nks)] = (uint8_t)(e + 127);
            }
        }

        // ---- delta codes: one (row, group) per thread
        for (int idx = tid; idx < QROWS * NG; idx += QTHREADS) {
            int r = idx / NG, j = idx - r * NG;
            if (32 * j >= cvalid || tok[r] < 0) continue;
            const int cr = core_row[r];
            float v[32];
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                v[i] = XTraits<XT>::f(xs[r * XLD + 32 * j + i]) - cs_tile[cr * CLD + 32 * j + i];
                amax = fmaxf(amax, fabsf(v[i]));
            }
            int e = mx_exp_fp4(amax);
            uint4 codes = encode_fp4x32(v, pow2f(e));
            const long long s = slot_of[r], G = (c0 >> 5) + j, nks = a.Kp / 128;
            *(uint4*)(a.dq + off_fp4(s, G, nks)) = codes;
            a.ds[off_scale(s, G, nks)] = (uint8_t)(e + 127);
        }
        __syncthreads();
    }

    // ---- U -> bf16, slot order (pad rows hold zeros: their X rows were zero)
    if (wave < 2) {
        for (int ct = 0; ct < nct; ++ct) {
            v16f acc = ct == 0 ? uacc[0] : ct == 1 ? uacc[1] : ct == 2 ? uacc[2] : uacc[3];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                int row = wave * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                if (row < nrows) {
                    long long s = slot_of[row];
                    a.u[s * a.rp + ct * 32 + (lane & 31)] = bf16_rne(acc[i]);
                }
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
    a.cubes_per_block = q->core_mode == 0 ? QROWS / g.S : 0;
    a.dq = q->dq;
    a.ds = q->ds;
    a.cq = q->cq;
    a.cs = q->cs;
    a.u = q->u;
    a.l1t = w->l1t;
    a.coref = q->coref;
    unsigned blocks = q->core_mode == 0 ? (unsigned)((g.K + a.cubes_per_block - 1) / a.cubes_per_block)
                                        : (unsigned)((g.Nslot + QROWS - 1) / QROWS);
    if (x_bf16) k_quantize<uint16_t><<<blocks, QTHREADS, 0, st>>>(a);
    else k_quantize<float><<<blocks, QTHREADS, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_slot_tokens(const Geom& g, int* stok, int64_t n, hipStream_t st) {
    k_slot_tokens<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(g, stok, n);
    return hipGetLastError();
}

}  // namespace dq
