// wkv7_bwd.hip -- chunked WKV7 backward on the matrix cores (gfx950).
//
// Reverse-mode of the per-token update (rwkv-mlx page, "Metal kernel
// architecture", backward block: chunks in reverse, from checkpoints).  With
// X_t = dL/dS_t (all later uses of S_t, including y_t) the gradient state
// obeys X_{t-1} = X_t (diag w_t + b_t a_t^T) + dy_{t-1} r_{t-1}^T, the same
// diagonal-plus-rank-1 recurrence as the forward but in reverse time.  It
// does not involve the forward state, so it is a pass of its own:
//
// Kernel 1 (state gradient, one workgroup per head row block, chunks in
// reverse).  With G = dL/dS at the chunk's end and the chunk matrices of
// wkv7_device.h, Bbar = Btil diag(gamma_last), Kbar = Ktil diag(gamma_last):
//     DSA     = (I - Lab)^-T (Bbar G^T + Mrb^T DY)        dsa_t = X_t b_t
//     dv      = Kbar G^T + Lak^T DSA + Mrk^T DY            dv_t  = X_t k_t
//     G_start = G diag(gamma_last) + DY^T Rhat + DSA^T Ahat
// G_start (the gradient w.r.t. the state entering the chunk) goes to the
// workspace; after chunk 0 it is dh0.  Rows of G are independent.
//
// Kernel 2 (one workgroup per (head, chunk), all chunks at once).  From the
// checkpoint S0 and the end gradient Ge it recomputes U (= sa_t) as in the
// forward -- never by dividing the state by w -- and DSA as in kernel 1, then
//     dr = Gamma     * (DY S0  + tril(DY U^T) Btil  + tril(DY V^T) Ktil)
//     da = Gamma_-1  * (DSA S0 + stril(DSA U^T) Btil + stril(DSA V^T) Ktil)
//     dk = Gamma^-1  * (V Ge gamma_last + striu(V DSA^T) Ahat + triu(V DY^T) Rhat)
//     db = Gamma^-1  * (U Ge gamma_last + striu(U DSA^T) Ahat + triu(U DY^T) Rhat)
// and dw from the identity (exact in real arithmetic, derived from the
// update rule): with phi_t = w_t * dw_t and Gs = dL/dS0,
//     phi_t = sum_i Gs[i][j] S0[i][j] - sum_{s<=t} a_s da_s
//             + sum_{s<t} (k_s dk_s + b_s db_s - r_s dr_s),
//     dw_t  = phi_t / w_t.
#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

// ------------------------------------------------------------- kernel 1
template <int RB>
struct StateLayout {
    static constexpr int W = 0;
    static constexpr int A = W + C * LDA;
    static constexpr int R = A + C * LDA;
    static constexpr int Bt = R + C * LDA;
    static constexpr int Kt = Bt + C * LDA;
    static constexpr int G = Kt + C * LDA;       // RB x LDA (i, j)
    static constexpr int DYT = G + RB * LDA;     // RB x LDC (i, t)
    static constexpr int Lab = DYT + RB * LDC;
    static constexpr int Lak = Lab + C * LDC;
    static constexpr int Mrb = Lak + C * LDC;
    static constexpr int Mrk = Mrb + C * LDC;
    static constexpr int Tinv = Mrk + C * LDC;
    static constexpr int RhsT = Tinv + C * LDC;  // RB x LDC (i, t)
    static constexpr int DsaT = RhsT + RB * LDC; // RB x LDC (i, t)
    static constexpr int glast = DsaT + RB * LDC;
    static constexpr int qp = glast + D;
    static constexpr int total = qp + 8 * D;
    static constexpr size_t bytes = total * sizeof(float);
};

template <typename InT, bool SPLIT, int RB, int NT>
__global__ __launch_bounds__(NT) void bwd_state_kernel(BwdArgs p, int xcd) {
    extern __shared__ float sm[];
    using L = StateLayout<RB>;
    constexpr int NW = NT / 64;
    constexpr int NRB = D / RB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    int head, rb;
    block_map(blockIdx.x, NRB, xcd != 0, head, rb);
    const int bb = head / p.H, hh = head % p.H;
    const int row0 = rb * RB;
    const int64_t tstride = (int64_t)p.H * D;
    const int64_t soff = (int64_t)head * D * D + (int64_t)row0 * D;

    float* W = sm + L::W;
    float* A = sm + L::A;
    float* R = sm + L::R;
    float* Bt = sm + L::Bt;
    float* Kt = sm + L::Kt;
    float* G = sm + L::G;
    float* DYT = sm + L::DYT;
    float* Lab = sm + L::Lab;
    float* Lak = sm + L::Lak;
    float* Mrb = sm + L::Mrb;
    float* Mrk = sm + L::Mrk;
    float* Tinv = sm + L::Tinv;
    float* RhsT = sm + L::RhsT;
    float* DsaT = sm + L::DsaT;
    float* glast = sm + L::glast;
    float* qp = sm + L::qp;

    load_state_rows<NT, RB>(p.dhT ? p.dhT + soff : nullptr, G, tid);

    for (int c = p.NC - 1; c >= 0; --c) {
        const int t0 = c * C;
        const int Cc = min(C, p.T - t0);
        const int64_t base = ((int64_t)bb * p.T + t0) * tstride + (int64_t)hh * D;
        __syncthreads();
        load_chunk<InT, NT>(static_cast<const InT*>(p.w), base, tstride, Cc, 1.f, W, tid);
        load_chunk<InT, NT>(static_cast<const InT*>(p.a), base, tstride, Cc, 0.f, A, tid);
        load_chunk<InT, NT>(static_cast<const InT*>(p.r), base, tstride, Cc, 0.f, R, tid);
        load_chunk<InT, NT>(static_cast<const InT*>(p.b), base, tstride, Cc, 0.f, Bt, tid);
        load_chunk<InT, NT>(static_cast<const InT*>(p.k), base, tstride, Cc, 0.f, Kt, tid);
        load_chunk_cols_T<float, NT, RB>(p.dy, base, tstride, Cc, row0, DYT, tid);
        __syncthreads();
        chunk_prep<NT>(W, A, R, Bt, Kt, glast, qp, tid);

        chunk_cc<SPLIT, NT>(A, R, Bt, Kt, Lab, Lak, Mrb, Mrk, tid);
        for (int e = tid; e < RB * D; e += NT) {
            const int i = e >> 6, j = e & 63;
            G[i * LDA + j] *= glast[j];  // G diag(gamma_last)
        }
        __syncthreads();

        constexpr int NTILE = 2 * (RB / 16);
        if (wave == NW - 1) tri_inverse(Lab, Tinv, lane);
        if (NW == 1 || wave < NW - 1) {
            const int nwk = NW == 1 ? 1 : NW - 1;
            for (int job = wave; job < NTILE; job += nwk) {
                const int ti = job & 1, tn = job >> 1;
                f32x4 acc = mma<SPLIT, D>(zero4(), rows(Bt, LDA), ti * 16, rows(G, LDA), tn * 16, lane);
                acc = mma<SPLIT, C>(acc, cols(Mrb, LDC), ti * 16, rows(DYT, LDC), tn * 16, lane);
                store_tile<LDC, true, MASK_NONE>(RhsT, acc, ti * 16, tn * 16, lane);
            }
        }
        __syncthreads();

        for (int job = wave; job < NTILE; job += NW) {
            const int ti = job & 1, tn = job >> 1;
            const f32x4 acc = mma<SPLIT, C>(zero4(), cols(Tinv, LDC), ti * 16, rows(RhsT, LDC), tn * 16, lane);
            store_tile<LDC, true, MASK_NONE>(DsaT, acc, ti * 16, tn * 16, lane);
        }
        __syncthreads();

        // dv = Kbar G^T + Lak^T DSA + Mrk^T DY
        for (int job = wave; job < NTILE; job += NW) {
            const int ti = job & 1, tn = job >> 1;
            f32x4 acc = mma<SPLIT, D>(zero4(), rows(Kt, LDA), ti * 16, rows(G, LDA), tn * 16, lane);
            acc = mma<SPLIT, C>(acc, cols(Lak, LDC), ti * 16, rows(DsaT, LDC), tn * 16, lane);
            acc = mma<SPLIT, C>(acc, cols(Mrk, LDC), ti * 16, rows(DYT, LDC), tn * 16, lane);
            const int r = lane & 15, g = lane >> 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = ti * 16 + 4 * g + q;
                if (t < Cc && p.dv) p.dv[base + t * tstride + row0 + tn * 16 + r] = acc[q];
            }
        }

        // G <- G diag(gamma_last) + DY^T Rhat + DSA^T Ahat (G already scaled)
        constexpr int NGTILE = (RB / 16) * 4;
        constexpr int NPER = (NGTILE + NW - 1) / NW;
        f32x4 gnew[NPER];
#pragma unroll
        for (int q2 = 0; q2 < NPER; ++q2) {
            const int job = wave + q2 * NW;
            if (job < NGTILE) {
                const int tm = job >> 2, tn = job & 3;
                const int r = lane & 15, g = lane >> 4;
                f32x4 acc;
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] = G[(tm * 16 + 4 * g + q) * LDA + tn * 16 + r];
                acc = mma<SPLIT, C>(acc, rows(DYT, LDC), tm * 16, cols(R, LDA), tn * 16, lane);
                acc = mma<SPLIT, C>(acc, rows(DsaT, LDC), tm * 16, cols(A, LDA), tn * 16, lane);
                gnew[q2] = acc;
            }
        }
        __syncthreads();
        float* gout = p.gbuf + ((int64_t)head * p.NC + c) * D * D + (int64_t)row0 * D;
        float* dh0 = (c == 0 && p.dh0) ? p.dh0 + soff : nullptr;
#pragma unroll
        for (int q2 = 0; q2 < NPER; ++q2) {
            const int job = wave + q2 * NW;
            if (job < NGTILE) {
                const int tm = job >> 2, tn = job & 3;
                store_tile<LDA, false, MASK_NONE>(G, gnew[q2], tm * 16, tn * 16, lane);
                const int r = lane & 15, g = lane >> 4;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t o = (int64_t)(tm * 16 + 4 * g + q) * D + tn * 16 + r;
                    gout[o] = gnew[q2][q];
                    if (dh0) dh0[o] = gnew[q2][q];
                }
            }
        }
    }
}

// ------------------------------------------------------------- kernel 2
struct ChunkLayout {
    static constexpr int W = 0;
    static constexpr int A = W + C * LDA;
    static constexpr int R = A + C * LDA;
    static constexpr int Bt = R + C * LDA;
    static constexpr int Kt = Bt + C * LDA;
    static constexpr int V = Kt + C * LDA;      // (t, i)
    static constexpr int DY = V + C * LDA;      // (t, i)
    static constexpr int U = DY + C * LDA;      // (t, i)
    static constexpr int DSA = U + C * LDA;     // (t, i)
    static constexpr int S0 = DSA + C * LDA;    // D x LDA (i, j)
    static constexpr int Ge = S0 + D * LDA;     // D x LDA (i, j)
    static constexpr int P1 = Ge + D * LDA;     // C x LDC: Lab, then tril(DY U^T)
    static constexpr int P2 = P1 + C * LDC;     //          Lak, then tril(DY V^T)
    static constexpr int P3 = P2 + C * LDC;     //          Mrb, then stril(DSA U^T)
    static constexpr int P4 = P3 + C * LDC;     //          Mrk, then stril(DSA V^T)
    static constexpr int Tinv = P4 + C * LDC;
    static constexpr int Hh = Tinv + C * LDC;   // C x LDA: k dk + b db - r dr - a da
    static constexpr int Fa = Hh + C * LDA;     // C x LDA: a da
    static constexpr int glast = Fa + C * LDA;
    static constexpr int qp = glast + D;
    static constexpr int red = qp + 8 * D;
    static constexpr int total = red + 8 * D;
    static constexpr size_t bytes = total * sizeof(float);
};
static_assert(ChunkLayout::bytes <= 160 * 1024, "chunk kernel LDS exceeds 160 KiB");

template <typename InT, bool SPLIT, int NT>
__global__ __launch_bounds__(NT) void bwd_chunk_kernel(BwdArgs p, int xcd) {
    extern __shared__ float sm[];
    using L = ChunkLayout;
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    int head, c;
    block_map(blockIdx.x, p.NC, xcd != 0, head, c);
    const int bb = head / p.H, hh = head % p.H;
    const int64_t tstride = (int64_t)p.H * D;
    const int t0 = c * C;
    const int Cc = min(C, p.T - t0);
    const int64_t base = ((int64_t)bb * p.T + t0) * tstride + (int64_t)hh * D;
    const int64_t hoff = (int64_t)head * D * D;

    float* W = sm + L::W;
    float* A = sm + L::A;
    float* R = sm + L::R;
    float* Bt = sm + L::Bt;
    float* Kt = sm + L::Kt;
    float* V = sm + L::V;
    float* DY = sm + L::DY;
    float* U = sm + L::U;
    float* DSA = sm + L::DSA;
    float* S0 = sm + L::S0;
    float* Ge = sm + L::Ge;
    float* P1 = sm + L::P1;
    float* P2 = sm + L::P2;
    float* P3 = sm + L::P3;
    float* P4 = sm + L::P4;
    float* Tinv = sm + L::Tinv;
    float* Hh = sm + L::Hh;
    float* Fa = sm + L::Fa;
    float* glast = sm + L::glast;
    float* qp = sm + L::qp;
    float* red = sm + L::red;

    load_chunk<InT, NT>(static_cast<const InT*>(p.w), base, tstride, Cc, 1.f, W, tid);
    load_chunk<InT, NT>(static_cast<const InT*>(p.a), base, tstride, Cc, 0.f, A, tid);
    load_chunk<InT, NT>(static_cast<const InT*>(p.r), base, tstride, Cc, 0.f, R, tid);
    load_chunk<InT, NT>(static_cast<const InT*>(p.b), base, tstride, Cc, 0.f, Bt, tid);
    load_chunk<InT, NT>(static_cast<const InT*>(p.k), base, tstride, Cc, 0.f, Kt, tid);
    load_chunk<InT, NT>(static_cast<const InT*>(p.v), base, tstride, Cc, 0.f, V, tid);
    load_chunk<float, NT>(p.dy, base, tstride, Cc, 0.f, DY, tid);
    load_state_rows<NT, D>(p.ckpt + ((int64_t)head * p.NC + c) * D * D, S0, tid);
    const float* ge_src = (c + 1 < p.NC) ? p.gbuf + ((int64_t)head * p.NC + c + 1) * D * D
                                         : (p.dhT ? p.dhT + hoff : nullptr);
    load_state_rows<NT, D>(ge_src, Ge, tid);
    __syncthreads();
    chunk_prep<NT>(W, A, R, Bt, Kt, glast, qp, tid);

    chunk_cc<SPLIT, NT>(A, R, Bt, Kt, P1, P2, P3, P4, tid);  // Lab, Lak, Mrb, Mrk
    for (int e = tid; e < D * D; e += NT) {
        const int i = e >> 6, j = e & 63;
        Ge[i * LDA + j] *= glast[j];
    }
    __syncthreads();

    // Right-hand sides: U buffer <- Ahat S0^T + Lak V, DSA buffer <- Bbar Ge^T + Mrb^T DY.
    if (wave == NW - 1) tri_inverse(P1, Tinv, lane);
    if (NW == 1 || wave < NW - 1) {
        const int nwk = NW == 1 ? 1 : NW - 1;
        for (int job = wave; job < 16; job += nwk) {
            const int which = job >> 3, ti = (job >> 2) & 1, tn = job & 3;
            f32x4 acc;
            if (which == 0) {
                acc = mma<SPLIT, D>(zero4(), rows(A, LDA), ti * 16, rows(S0, LDA), tn * 16, lane);
                acc = mma<SPLIT, C>(acc, rows(P2, LDC), ti * 16, cols(V, LDA), tn * 16, lane);
                store_tile<LDA, false, MASK_NONE>(U, acc, ti * 16, tn * 16, lane);
            } else {
                acc = mma<SPLIT, D>(zero4(), rows(Bt, LDA), ti * 16, rows(Ge, LDA), tn * 16, lane);
                acc = mma<SPLIT, C>(acc, cols(P3, LDC), ti * 16, cols(DY, LDA), tn * 16, lane);
                store_tile<LDA, false, MASK_NONE>(DSA, acc, ti * 16, tn * 16, lane);
            }
        }
    }
    __syncthreads();

    // U = (I - Lab)^-1 RHS_U, DSA = (I - Lab)^-T RHS_D (in place via registers).
    {
        constexpr int NPER = (16 + NW - 1) / NW;
        f32x4 res[NPER];
#pragma unroll
        for (int q2 = 0; q2 < NPER; ++q2) {
            const int job = wave + q2 * NW;
            if (job < 16) {
                const int which = job >> 3, ti = (job >> 2) & 1, tn = job & 3;
                if (which == 0)
                    res[q2] = mma<SPLIT, C>(zero4(), rows(Tinv, LDC), ti * 16, cols(U, LDA), tn * 16, lane);
                else
                    res[q2] = mma<SPLIT, C>(zero4(), cols(Tinv, LDC), ti * 16, cols(DSA, LDA), tn * 16, lane);
            }
        }
        __syncthreads();
#pragma unroll
        for (int q2 = 0; q2 < NPER; ++q2) {
            const int job = wave + q2 * NW;
            if (job < 16) {
                const int which = job >> 3, ti = (job >> 2) & 1, tn = job & 3;
                store_tile<LDA, false, MASK_NONE>(which == 0 ? U : DSA, res[q2], ti * 16, tn * 16, lane);
            }
        }
    }
    __syncthreads();

    // P1 = tril(DY U^T), P2 = tril(DY V^T), P3 = stril(DSA U^T), P4 = stril(DSA V^T)
    for (int job = wave; job < 12; job += NW) {
        const int mat = job / 3, tile = job % 3;
        const int ti = tile == 0 ? 0 : 1, tj = tile == 2 ? 1 : 0;
        const Op X = rows(mat < 2 ? DY : DSA, LDA);
        const Op Y = rows((mat & 1) ? V : U, LDA);
        const f32x4 acc = mma<SPLIT, D>(zero4(), X, ti * 16, Y, tj * 16, lane);
        float* M = mat == 0 ? P1 : mat == 1 ? P2 : mat == 2 ? P3 : P4;
        if (mat < 2) store_tile<LDC, false, MASK_LOWER>(M, acc, ti * 16, tj * 16, lane);
        else store_tile<LDC, false, MASK_STRICT>(M, acc, ti * 16, tj * 16, lane);
    }
    for (int e = tid; e < 4 * 256; e += NT) {
        const int m = e >> 8, t = (e & 255) >> 4, s = 16 + (e & 15);
        float* M = m == 0 ? P1 : m == 1 ? P2 : m == 2 ? P3 : P4;
        M[t * LDC + s] = 0.f;
    }
    // partial sums of diag(Gs^T S0) over row groups (Gs = gradient entering the chunk)
    {
        const float* gs = p.gbuf + ((int64_t)head * p.NC + c) * D * D;
        constexpr int NG = NT / 64, RPG = D / NG;
        const int j = tid & 63, grp = tid >> 6;
        float acc = 0.f;
        for (int i = grp * RPG; i < (grp + 1) * RPG; ++i) acc = fmaf(gs[i * D + j], S0[i * LDA + j], acc);
        red[grp * 64 + j] = acc;
    }
    __syncthreads();

    // Outputs dr, da, dk, db per 16x16 position, plus the dw ingredients.
    for (int pos = wave; pos < 8; pos += NW) {
        const int ti = pos >> 2, tj = pos & 3;
        f32x4 aR = mma<SPLIT, D>(zero4(), rows(DY, LDA), ti * 16, cols(S0, LDA), tj * 16, lane);
        aR = mma<SPLIT, C>(aR, rows(P1, LDC), ti * 16, cols(Bt, LDA), tj * 16, lane);
        aR = mma<SPLIT, C>(aR, rows(P2, LDC), ti * 16, cols(Kt, LDA), tj * 16, lane);
        f32x4 aA = mma<SPLIT, D>(zero4(), rows(DSA, LDA), ti * 16, cols(S0, LDA), tj * 16, lane);
        aA = mma<SPLIT, C>(aA, rows(P3, LDC), ti * 16, cols(Bt, LDA), tj * 16, lane);
        aA = mma<SPLIT, C>(aA, rows(P4, LDC), ti * 16, cols(Kt, LDA), tj * 16, lane);
        f32x4 aK = mma<SPLIT, D>(zero4(), rows(V, LDA), ti * 16, cols(Ge, LDA), tj * 16, lane);
        aK = mma<SPLIT, C>(aK, cols(P4, LDC), ti * 16, cols(A, LDA), tj * 16, lane);
        aK = mma<SPLIT, C>(aK, cols(P2, LDC), ti * 16, cols(R, LDA), tj * 16, lane);
        f32x4 aB = mma<SPLIT, D>(zero4(), rows(U, LDA), ti * 16, cols(Ge, LDA), tj * 16, lane);
        aB = mma<SPLIT, C>(aB, cols(P3, LDC), ti * 16, cols(A, LDA), tj * 16, lane);
        aB = mma<SPLIT, C>(aB, cols(P1, LDC), ti * 16, cols(R, LDA), tj * 16, lane);
        const int r = lane & 15, g = lane >> 4;
        const int j = tj * 16 + r;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t = ti * 16 + 4 * g + q;
            const float gt = W[t * LDA + j];
            const float gp = t > 0 ? W[(t - 1) * LDA + j] : 1.f;
            const float inv = 1.f / gt;
            const float f = A[t * LDA + j] * aA[q];                       // a da
            const float e = Kt[t * LDA + j] * aK[q] + Bt[t * LDA + j] * aB[q] - R[t * LDA + j] * aR[q];
            Hh[t * LDA + j] = e - f;
            Fa[t * LDA + j] = f;
            if (t < Cc) {
                const int64_t o = base + t * tstride + j;
                p.dr[o] = aR[q] * gt;
                p.da[o] = aA[q] * gp;
                p.dk[o] = aK[q] * inv;
                p.db[o] = aB[q] * inv;
            }
        }
    }
    __syncthreads();

    if (tid < 64) {
        const int j = tid;
        constexpr int NG = NT / 64;
        float acc = 0.f;
#pragma unroll
        for (int grp = 0; grp < NG; ++grp) acc += red[grp * 64 + j];
        const InT* gw = static_cast<const InT*>(p.w);
        for (int t = 0; t < Cc; ++t) {
            const int64_t o = base + t * tstride + j;
            float wv;
            if constexpr (sizeof(InT) == 2) wv = __uint_as_float((uint32_t)gw[o] << 16);
            else wv = gw[o];
            p.dw[o] = (acc - Fa[t * LDA + j]) / wv;
            acc += Hh[t * LDA + j];
        }
    }
}

template <typename F>
hipError_t set_smem(F kern, size_t bytes, bool& done) {
    if (done) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) done = true;
    return e;
}

template <typename InT, bool SPLIT, int RB>
hipError_t launch_state(const BwdArgs& a, hipStream_t s) {
    constexpr int NT = 256;
    using L = StateLayout<RB>;
    auto kern = bwd_state_kernel<InT, SPLIT, RB, NT>;
    static bool done = false;
    hipError_t e = set_smem(kern, L::bytes, done);
    if (e != hipSuccess) return e;
    const int heads = a.B * a.H;
    const int xcd = (heads % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3(heads * (D / RB)), dim3(NT), L::bytes, s, a, xcd);
    return hipGetLastError();
}

template <typename InT, bool SPLIT>
hipError_t launch_state_typed(const BwdArgs& a, hipStream_t s) {
    const int heads = a.B * a.H;
    if (heads >= 256) return launch_state<InT, SPLIT, 64>(a, s);
    if (heads >= 128) return launch_state<InT, SPLIT, 32>(a, s);
    return launch_state<InT, SPLIT, 16>(a, s);
}

template <typename InT, bool SPLIT>
hipError_t launch_inputs_typed(const BwdArgs& a, hipStream_t s) {
    constexpr int NT = 256;
    auto kern = bwd_chunk_kernel<InT, SPLIT, NT>;
    static bool done = false;
    hipError_t e = set_smem(kern, ChunkLayout::bytes, done);
    if (e != hipSuccess) return e;
    const int heads = a.B * a.H;
    const int xcd = (heads % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3(heads * a.NC), dim3(NT), ChunkLayout::bytes, s, a, xcd);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_state(const BwdArgs& a, bool bf16, hipStream_t s) {
    if (bf16) return launch_state_typed<uint16_t, true>(a, s);
    return launch_state_typed<float, false>(a, s);
}

hipError_t launch_bwd_inputs(const BwdArgs& a, bool bf16, hipStream_t s) {
    if (bf16) return launch_inputs_typed<uint16_t, true>(a, s);
    return launch_inputs_typed<float, false>(a, s);
}

}  // namespace wkv7
