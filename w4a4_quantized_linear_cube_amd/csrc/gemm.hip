// Scaled-MFMA GEMMs of the delta-W4A4 layer (gfx950).
//
// DeltaQuant notes, 关键设计 4 (the three-term equation):
//   y_n = U_n L2 + Q8(core_k(n)) Q4(R) + Q4(delta_n) Q4(R)
// The core term is one row per cube ("dynamic token bias", broadcast to the
// cube's tokens); the delta term is one row per token.  Both are
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 contractions over Ci with the E8M0 block
// scales applied inside the instruction (A = FP8 E4M3 for cores, FP4 E2M1 for
// deltas; B = Q4(R) FP4 E2M1), fp32 accumulation.
//
// Tiling: a 256-thread workgroup computes a 256 x 256 output tile; its four
// waves each own 128 x 128 (4 x 4 MFMA tiles of 32 x 32, 256 accumulator
// registers).  K advances 128 per step; A/B code tiles and their scale bytes
// are staged through double-buffered LDS (XOR-swizzled 16-byte chunks) with
// one barrier per step.  Rows and columns of every operand are padded to the
// tile size and K to 128, padding holding zero codes and zero scales, so the
// main loop has no bounds checks.
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
    // plain store epilogue: c[row][col]
    float* c;
    long long ldc;
    // token epilogue: y[token][col] = acc + U L2 + bias[cube]
    float* y;
    int Co;
    Geom g;
    const float* bias;
    long long ldbias;
    const uint16_t* u;     // [Nslot_pad][rp]
    const uint16_t* l2t;   // [Cop][rp]
    int rp;
};

constexpr int EPI_STORE = 0;
constexpr int EPI_TOKENS = 1;

template <int AFMT, int OPSEL>
__device__ __forceinline__ v16f mfma_mx(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, AFMT, FMT_FP4, OPSEL, sa, OPSEL, sb);
}

template <int AFMT, int EPI>
__global__ __launch_bounds__(256, 1) void k_mxgemm(GemmArgs p) {
    constexpr int ABYTES = AFMT == FMT_FP4 ? 64 : 128;   // A bytes per row per 128-wide K step
    constexpr int ACH = ABYTES / 16;
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][256 * ABYTES];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][256 * 64];
    __shared__ uint32_t lds_as[2][256];
    __shared__ uint32_t lds_bs[2][256];
    __shared__ long long rtok[EPI == EPI_TOKENS ? 256 : 1];
    __shared__ long long rcube[EPI == EPI_TOKENS ? 256 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int g = lane >> 5, l32 = lane & 31;
    const int bid = blockIdx.x;
    const int tm = bid / p.ntiles, tn = bid - tm * p.ntiles;
    const long long m0 = (long long)tm * 256, n0 = (long long)tn * 256;

    if (EPI == EPI_TOKENS) {
        long long slot = m0 + tid;
        rtok[tid] = slot < p.g.Nslot ? slot_token(p.g, slot) : -1;
        rcube[tid] = slot / p.g.S;
    }

    auto swz_a = [](int row, int ch) { return AFMT == FMT_FP4 ? (ch ^ ((row >> 1) & 3)) : (ch ^ (row & 7)); };
    auto swz_b = [](int row, int ch) { return ch ^ ((row >> 1) & 3); };

    uint4 ra[ACH], rb[4];
    uint32_t ras, rbs;
    auto gload = [&](int kt) {
        const long long ka = (long long)kt * ABYTES, kb = (long long)kt * 64;
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            int q = tid + 256 * i, row = q / ACH, ch = q - row * ACH;
            ra[i] = *(const uint4*)(p.a + (m0 + row) * p.lda + ka + ch * 16);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int q = tid + 256 * i, row = q >> 2, ch = q & 3;
            rb[i] = *(const uint4*)(p.b + (n0 + row) * p.ldb + kb + ch * 16);
        }
        ras = *(const uint32_t*)(p.as + (m0 + tid) * p.ldas + kt * 4);
        rbs = *(const uint32_t*)(p.bs + (n0 + tid) * p.ldbs + kt * 4);
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            int q = tid + 256 * i, row = q / ACH, ch = q - row * ACH;
            *(uint4*)(&lds_a[buf][row * ABYTES + swz_a(row, ch) * 16]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int q = tid + 256 * i, row = q >> 2, ch = q & 3;
            *(uint4*)(&lds_b[buf][row * 64 + swz_b(row, ch) * 16]) = rb[i];
        }
        lds_as[buf][tid] = ras;
        lds_bs[buf][tid] = rbs;
    };

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (v16f){};

    auto compute_half = [&](int buf, auto KK) {
        constexpr int kk = decltype(KK)::value;
        v8i af[4], bfr[4];
        int sa[4], sb[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            int row = wr * 128 + mi * 32 + l32;
            const uint8_t* base = &lds_a[buf][row * ABYTES];
            if (AFMT == FMT_FP4) {
                uint4 v = *(const uint4*)(base + swz_a(row, 2 * kk + g) * 16);
                af[mi] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            } else {
                uint4 v0 = *(const uint4*)(base + swz_a(row, 4 * kk + g) * 16);
                uint4 v1 = *(const uint4*)(base + swz_a(row, 4 * kk + 2 + g) * 16);
                af[mi] = (v8i){(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
            }
            sa[mi] = (int)(lds_as[buf][row] >> (8 * g));
        }
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            int row = wc * 128 + ni * 32 + l32;
            uint4 v = *(const uint4*)(&lds_b[buf][row * 64 + swz_b(row, 2 * kk + g) * 16]);
            bfr[ni] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            sb[ni] = (int)(lds_bs[buf][row] >> (8 * g));
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                acc[mi][ni] = mfma_mx<AFMT, 2 * kk>(af[mi], bfr[ni], acc[mi][ni], sa[mi], sb[ni]);
    };

    const int nk = p.Kp / 128;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        compute_half(buf, std::integral_constant<int, 0>{});
        compute_half(buf, std::integral_constant<int, 1>{});
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

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

    // ---- low-rank branch: acc += U L2 (32x32x16 bf16 MFMA over the padded rank)
    for (int kq = 0; kq < p.rp; kq += 16) {
        v8bf ua[4], lb[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            long long row = m0 + wr * 128 + mi * 32 + l32;
            ua[mi] = __builtin_bit_cast(v8bf, *(const uint4*)(p.u + row * p.rp + kq + 8 * g));
        }
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            long long col = n0 + wc * 128 + ni * 32 + l32;
            lb[ni] = __builtin_bit_cast(v8bf, *(const uint4*)(p.l2t + col * p.rp + kq + 8 * g));
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ua[mi], lb[ni], acc[mi][ni], 0, 0, 0);
    }

    // ---- + per-cube core term, scatter rows to token order
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            int r = wr * 128 + mi * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
            long long t = rtok[r];
            if (t < 0) continue;
            const float* brow = p.bias + rcube[r] * p.ldbias;
            float* yrow = p.y + t * (long long)p.Co;
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                long long col = n0 + wc * 128 + ni * 32 + l32;
                if (col < p.Co) yrow[col] = acc[mi][ni][i] + brow[col];
            }
        }
}

hipError_t launch_forward(const dq_weights* w, dq_qact* q, float* y, hipStream_t st) {
    // 1) per-cube core term: bias[k] = Q8(core_k) Q4(R)
    GemmArgs c{};
    c.a = q->cq;
    c.as = q->cs;
    c.lda = q->Kp;
    c.ldas = q->Kp / 32;
    c.b = w->rq;
    c.bs = w->rs;
    c.ldb = w->Kp / 2;
    c.ldbs = w->Kp / 32;
    c.Kp = (int)w->Kp;
    c.mtiles = (int)(q->K_pad / 256);
    c.ntiles = (int)(w->Cop / 256);
    c.c = q->bias;
    c.ldc = w->Cop;
    k_mxgemm<FMT_FP8, EPI_STORE><<<c.mtiles * c.ntiles, 256, 0, st>>>(c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    // 2) delta term + low-rank branch + broadcast core term -> y (token order)
    GemmArgs d = c;
    d.a = q->dq;
    d.as = q->ds;
    d.lda = q->Kp / 2;
    d.ldas = q->Kp / 32;
    d.mtiles = (int)(q->Nslot_pad / 256);
    d.c = nullptr;
    d.y = y;
    d.Co = (int)w->Co;
    d.g = q->g;
    d.bias = q->bias;
    d.ldbias = w->Cop;
    d.u = q->u;
    d.l2t = w->l2t;
    d.rp = w->rp;
    k_mxgemm<FMT_FP4, EPI_TOKENS><<<d.mtiles * d.ntiles, 256, 0, st>>>(d);
    return hipGetLastError();
}

}  // namespace dq
