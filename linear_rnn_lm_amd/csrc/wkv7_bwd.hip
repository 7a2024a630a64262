// wkv7_bwd.hip -- per-token input gradients of the WKV7 backward (gfx950).
//
// Reverse-mode of the per-token update (rwkv-mlx page, "Metal kernel
// architecture", backward block: chunks in reverse, from checkpoints).  With
// X_t = dL/dS_t (all later uses of S_t, including y_t) the gradient state
// obeys X_{t-1} = X_t (diag w_t + b_t a_t^T) + dy_{t-1} r_{t-1}^T.  The scan
// kernel (wkv7_scan.hip) walks that recurrence over the chunks and leaves the
// gradient w.r.t. the state entering every chunk in dh_ckpt.  This kernel
// takes it from there, one workgroup per (head, chunk), all chunks at once.
// With the chunk matrices of wkv7_device.h, G' = Ge diag(gamma_last) for the
// gradient Ge at the chunk's end and T = (I - Lab)^-1 (from the prepare
// kernel), it recomputes from the checkpoint S0 -- never by dividing the
// state by w --
//     U   = T (Ahat S0^T + Lak V)                       u_t   = S_{t-1} a_t
//     DSA = T^T (Btil G'^T + Mrb^T DY)                  dsa_t = X_t b_t
// and then
//     dr = Gamma    * (DY S0  + tril(DY U^T) Btil   + tril(DY V^T) Ktil)
//     da = Gamma_-1 * (DSA S0 + stril(DSA U^T) Btil + stril(DSA V^T) Ktil)
//     dk = Gamma^-1 * (V Ge'  + striu(V DSA^T) Ahat + triu(V DY^T) Rhat)
//     db = Gamma^-1 * (U Ge'  + striu(U DSA^T) Ahat + triu(U DY^T) Rhat)
// and dw from an identity that follows from the update rule: with
// phi_t = w_t * dw_t and Gs = dL/dS0,
//     phi_t = sum_i Gs[i][j] S0[i][j] - sum_{s<=t} a_s da_s
//             + sum_{s<t} (k_s dk_s + b_s db_s - r_s dr_s),
//     dw_t  = phi_t / w_t.
#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

// LDS plan (byte offsets).  Region X holds what phases 0-3 need; region Y
// (phases 3-5) reuses region X's space once its contents are dead; region P
// lives throughout.  See the phase comments in the kernel.
template <bool SPLIT>
struct ChunkSmem {
    using F = Fmt<SPLIT>;
    static constexpr int RM = F::bytes(C, D), TM = F::bytes(D, C), SM = F::bytes(D, D), CM = F::bytes(C, C);
    static constexpr int F32C = C * LDF * 4;
    // region X (phases 0-3)
    static constexpr int XA = 0;                   // Ahat rows
    static constexpr int XB = XA + RM;             // Btil rows
    static constexpr int XR = XB + RM;             // Rhat rows   (dead after phase 1)
    static constexpr int XK = XR + RM;             // Ktil rows   (dead after phase 1)
    static constexpr int XVT = XK + RM;            // v^T (i, t)
    static constexpr int XDYT = XVT + TM;          // dy^T (i, t)
    static constexpr int XS0 = XDYT + TM;          // S0 rows (i, j)
    static constexpr int XGe = XS0 + SM;           // Ge' rows (i, j)
    static constexpr int XLak = XGe + SM;          // Lak rows (t, s)
    static constexpr int XMrbT = XLak + CM;        // Mrb^T (t, s)
    static constexpr int XRhsUT = XMrbT + CM;      // (i, t)
    static constexpr int XRhsDT = XRhsUT + TM;     // (i, t)
    static constexpr int XEND = XRhsDT + TM;
    // (I - Lab)^-1, rows and transposed, written in phase 2 over Rhat/Ktil
    static constexpr int XTinv = XR;               // (t, s)
    static constexpr int XTinvT = XTinv + CM;      // (t, s) = Tinv[s][t]
    static_assert(XTinvT + CM <= XVT, "inverse overflows Rhat/Ktil");
    // region Y (phases 3-5)
    static constexpr int YU = 0;                   // U rows (t, i)       over XA
    static constexpr int YDSA = YU + RM;           // DSA rows (t, i)     over XB
    static constexpr int YP = YDSA + RM;           // P1..P4 rows, then P1T..P4T
    static constexpr int YS0T = YP + 8 * CM;       // half S0^T (j', i)
    static constexpr int YGeT = YS0T + F::bytes(32, D);
    static constexpr int YAT = YGeT + F::bytes(32, D);  // half Ahat^T (j', t)
    static constexpr int YRT = YAT + F::bytes(32, C);
    static constexpr int YBT = YRT + F::bytes(32, C);
    static constexpr int YKT = YBT + F::bytes(32, C);
    static constexpr int YHh = YKT + F::bytes(32, C);   // fp32 C x LDG
    static constexpr int YFa = YHh + C * LDG * 4;
    static constexpr int YEND = YFa + C * LDG * 4;
    static_assert(YP >= XA + 2 * RM, "U/DSA must not overlap live phase-3 data");
    // region P
    static constexpr int P0 = (XEND > YEND ? XEND : YEND);
    static constexpr int Gam = P0;                 // fp32 gamma [t][j]
    static constexpr int DYr = Gam + C * LDG * 4;  // dy rows (t, i)
    static constexpr int Vr = DYr + RM;            // v rows (t, i)
    static constexpr int glast = Vr + RM;
    static constexpr int qp = glast + D * 4;
    static constexpr int red = qp + 8 * D * 4;
    static constexpr int total = red + 4 * D * 4;
};

template <typename InT, bool SPLIT, int NT>
__global__ __launch_bounds__(NT) void bwd_chunk_kernel(BwdArgs p, int xcd) {
    static_assert(NT == 256, "one raw-chunk thread shape");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    using L = ChunkSmem<SPLIT>;
    using M = Mat<SPLIT>;
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;

    int head, c;
    block_map(blockIdx.x, p.NC, xcd != 0, head, c);
    const int bb = head / p.H, hh = head % p.H;
    const int64_t tstride = (int64_t)p.H * D;
    const int t0 = c * C;
    const int Cc = min(C, p.T - t0);
    const int64_t base = ((int64_t)bb * p.T + t0) * tstride + (int64_t)hh * D;
    const int64_t hoff = (int64_t)head * D * D;

    const InT* gw = static_cast<const InT*>(p.w);

    // ---- phase 0: loads and chunk preparation
    RawChunk<NT, InT> raw;
    raw.load(gw, static_cast<const InT*>(p.a), static_cast<const InT*>(p.r), static_cast<const InT*>(p.b),
             static_cast<const InT*>(p.k), base, tstride, Cc, tid);
    RawCols<NT, D, InT> rv;
    RawCols<NT, D, float> rdy;
    rv.load(static_cast<const InT*>(p.v), base, tstride, Cc, 0, tid);
    rdy.load(p.dy, base, tstride, Cc, 0, tid);
    // four entries of the chunk's (I - Lab)^-1: row tid/8, columns 4*(tid%8)..
    const f32x4 tv = *reinterpret_cast<const f32x4*>(p.inv + ((int64_t)head * p.NC + c) * C * C + tid * 4);
    // state-sized inputs: thread holds row si = tid/4, columns sj0 .. sj0+15
    const int si = tid >> 2, sj0 = (tid & 3) * 16;
    const float* s0g = p.ckpt + ((int64_t)head * p.NC + c) * D * D;
    const float* geg = (c + 1 < p.NC) ? p.gbuf + ((int64_t)head * p.NC + c + 1) * D * D
                                      : (p.dhT ? p.dhT + hoff : nullptr);
    f32x4 s0v[4], gev[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        s0v[q] = *reinterpret_cast<const f32x4*>(s0g + si * D + sj0 + 4 * q);
        gev[q] = geg ? *reinterpret_cast<const f32x4*>(geg + si * D + sj0 + 4 * q) : zero4();
    }
    // partial sums of diag(Gs^T S0): thread column rj, rows 16*rgrp .. +15
    {
        const float* gsg = p.gbuf + ((int64_t)head * p.NC + c) * D * D;
        const int rj = tid & 63, rgrp = tid >> 6;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = rgrp * 16 + i;
            acc = fmaf(gsg[row * D + rj], s0g[row * D + rj], acc);
        }
        reinterpret_cast<float*>(smem + L::red)[rgrp * 64 + rj] = acc;
    }

    const M XA = make_mat<SPLIT>(smem, L::XA, C, D), XB = make_mat<SPLIT>(smem, L::XB, C, D);
    const M XR = make_mat<SPLIT>(smem, L::XR, C, D), XK = make_mat<SPLIT>(smem, L::XK, C, D);
    const M XVT = make_mat<SPLIT>(smem, L::XVT, D, C), XDYT = make_mat<SPLIT>(smem, L::XDYT, D, C);
    const M XS0 = make_mat<SPLIT>(smem, L::XS0, D, D), XGe = make_mat<SPLIT>(smem, L::XGe, D, D);
    const M XLak = make_mat<SPLIT>(smem, L::XLak, C, C), XMrbT = make_mat<SPLIT>(smem, L::XMrbT, C, C);
    const M XRhsUT = make_mat<SPLIT>(smem, L::XRhsUT, D, C), XRhsDT = make_mat<SPLIT>(smem, L::XRhsDT, D, C);
    const M XTinv = make_mat<SPLIT>(smem, L::XTinv, C, C), XTinvT = make_mat<SPLIT>(smem, L::XTinvT, C, C);
    float* gam = reinterpret_cast<float*>(smem + L::Gam);
    const M DYr = make_mat<SPLIT>(smem, L::DYr, C, D), Vr = make_mat<SPLIT>(smem, L::Vr, C, D);
    float* glast = reinterpret_cast<float*>(smem + L::glast);
    float* qp = reinterpret_cast<float*>(smem + L::qp);
    float* red = reinterpret_cast<float*>(smem + L::red);

    const PrepOut<SPLIT> po{XA, XR, XB, XK, XA, XA, XA, XA, true, true, true, true, false, false, false, false,
                            gam, glast};
    chunk_prep<NT, SPLIT>(raw, po, qp, tid);
    rv.template store_T<SPLIT, true>(XVT, tid);
    rv.template store_rows<SPLIT, true>(Vr, tid);
    rdy.template store_T<SPLIT, false>(XDYT, tid);
    rdy.template store_rows<SPLIT, false>(DYr, tid);
#pragma unroll
    for (int q = 0; q < 4; ++q) put4(XS0, si, sj0 + 4 * q, s0v[q]);
    lds_barrier();

    // ---- phase 1: C x C matrices; Ge' = Ge diag(gamma_last)
    const CcOut<SPLIT, NT> co{nullptr, XLak, XLak, XMrbT, XMrbT, XMrbT, XMrbT, true, false, false, true, false, false};
    chunk_cc<SPLIT, NT>(XA, XR, XB, XK, co, tid);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) gev[q][e] *= glast[sj0 + 4 * q + e];
        put4(XGe, si, sj0 + 4 * q, gev[q]);
    }
    lds_barrier();

    // ---- phase 2: RHS_U = Ahat S0^T + Lak V, RHS_D = Btil Ge'^T + Mrb^T DY; (I - Lab)^-1 to LDS
    put4(XTinv, tid >> 3, (tid & 7) * 4, tv);
#pragma unroll
    for (int q = 0; q < 4; ++q) put(XTinvT, (tid & 7) * 4 + q, tid >> 3, tv[q]);
    {
        for (int job = wave; job < 16; job += NW) {
            const int which = job >> 3, ti = (job >> 2) & 1, tn = job & 3;
            f32x4 acc;
            if (which == 0) {
                acc = mma<SPLIT, D>(zero4(), XA, ti * 16, XS0, tn * 16, lane);
                acc = mma<SPLIT, C, false, true>(acc, XLak, ti * 16, XVT, tn * 16, lane);
                store_cols<MASK_NONE>(XRhsUT, acc, ti * 16, tn * 16, lane);
            } else {
                acc = mma<SPLIT, D>(zero4(), XB, ti * 16, XGe, tn * 16, lane);
                acc = mma<SPLIT, C>(acc, XMrbT, ti * 16, XDYT, tn * 16, lane);
                store_cols<MASK_NONE>(XRhsDT, acc, ti * 16, tn * 16, lane);
            }
        }
    }
    lds_barrier();

    // ---- phase 3: U^T = RHS_U^T Tinv^T and DSA^T = RHS_D^T Tinv, stored as U, DSA rows (t, i)
    const M YU = make_mat<SPLIT>(smem, L::YU, C, D), YDSA = make_mat<SPLIT>(smem, L::YDSA, C, D);
    for (int job = wave; job < 16; job += NW) {
        const int which = job >> 3, ti = job & 3, tt = (job >> 2) & 1;   // ti: i tile, tt: t tile
        if (which == 0) {
            const f32x4 acc = mma<SPLIT, C>(zero4(), XRhsUT, ti * 16, XTinv, tt * 16, lane);
            store_cols<MASK_NONE>(YU, acc, ti * 16, tt * 16, lane);
        } else {
            const f32x4 acc = mma<SPLIT, C>(zero4(), XRhsDT, ti * 16, XTinvT, tt * 16, lane);
            store_cols<MASK_NONE>(YDSA, acc, ti * 16, tt * 16, lane);
        }
    }
    lds_barrier();

    // ---- phase 4: P1 = tril(DY U^T), P2 = tril(DY V^T), P3 = stril(DSA U^T), P4 = stril(DSA V^T),
    //      rows and transposed; first half of the j-indexed transposed operands.
    // P1..P4 rows at YP + m*CM, transposed at YP + (4+m)*CM (m = 0..3)
    auto Pr = [&](int m) { return make_mat<SPLIT>(smem, L::YP + m * L::CM, C, C); };
    auto Pt = [&](int m) { return make_mat<SPLIT>(smem, L::YP + (4 + m) * L::CM, C, C); };
    for (int job = wave; job < 12; job += NW) {
        const int mat = job / 3, tile = job % 3;
        const int ti = tile == 0 ? 0 : 1, tj = tile == 2 ? 1 : 0;
        const M X = mat < 2 ? DYr : YDSA;
        f32x4 acc;
        if (mat & 1) acc = mma<SPLIT, D, false, true>(zero4(), X, ti * 16, Vr, tj * 16, lane);
        else acc = mma<SPLIT, D>(zero4(), X, ti * 16, YU, tj * 16, lane);
        if (mat < 2) {
            store_rows<MASK_LOWER>(Pr(mat), acc, ti * 16, tj * 16, lane);
            store_cols<MASK_LOWER>(Pt(mat), acc, ti * 16, tj * 16, lane);
        } else {
            store_rows<MASK_STRICT>(Pr(mat), acc, ti * 16, tj * 16, lane);
            store_cols<MASK_STRICT>(Pt(mat), acc, ti * 16, tj * 16, lane);
        }
    }
    if (wave == NW - 1) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            zero_block(Pr(m), 0, 16, lane);
            zero_block(Pt(m), 16, 0, lane);
        }
    }

    const M YS0T = make_mat<SPLIT>(smem, L::YS0T, 32, D), YGeT = make_mat<SPLIT>(smem, L::YGeT, 32, D);
    const M YAT = make_mat<SPLIT>(smem, L::YAT, 32, C), YRT = make_mat<SPLIT>(smem, L::YRT, 32, C);
    const M YBT = make_mat<SPLIT>(smem, L::YBT, 32, C), YKT = make_mat<SPLIT>(smem, L::YKT, 32, C);
    float* hh_ = reinterpret_cast<float*>(smem + L::YHh);
    float* fa_ = reinterpret_cast<float*>(smem + L::YFa);

    // Writes the transposed operands for columns j in [32*half, 32*half + 32).
    auto fill_half = [&](int half) {
        if ((sj0 >> 5) == half) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int jl = sj0 - 32 * half + 4 * q + e;
                    put(YS0T, jl, si, s0v[q][e]);
                    put(YGeT, jl, si, gev[q][e]);
                }
            }
        }
        constexpr int TPG = RawChunk<NT, InT>::TPG;
        const int jp = tid & 31, q = tid >> 5;
        if ((jp >> 4) == half) {
            const int t0q = q * TPG;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int j = 2 * jp + e, jl = j - 32 * half;
                f32x4 av, rv4, bv, kv;
#pragma unroll
                for (int tt = 0; tt < TPG; ++tt) {
                    const int t = t0q + tt;
                    const float g = gam[t * LDG + j];
                    const float gp = t > 0 ? gam[(t - 1) * LDG + j] : 1.f;
                    const float ig = rcp(g);
                    const float2 a2 = raw.get(raw.a[tt], tt, tid, 0.f), r2 = raw.get(raw.r[tt], tt, tid, 0.f);
                    const float2 b2 = raw.get(raw.b[tt], tt, tid, 0.f), k2 = raw.get(raw.k[tt], tt, tid, 0.f);
                    av[tt] = (e ? a2.y : a2.x) * gp;
                    rv4[tt] = (e ? r2.y : r2.x) * g;
                    bv[tt] = (e ? b2.y : b2.x) * ig;
                    kv[tt] = (e ? k2.y : k2.x) * ig;
                }
                put4(YAT, jl, t0q, av);
                put4(YRT, jl, t0q, rv4);
                put4(YBT, jl, t0q, bv);
                put4(YKT, jl, t0q, kv);
            }
        }
    };
    static_assert(RawChunk<NT, InT>::TPG == 4, "fill_half packs four tokens");
    fill_half(0);
    lds_barrier();

    // ---- phase 5: outputs, one j half at a time
    for (int half = 0; half < 2; ++half) {
        // four 16 x 16 positions (t tile, j tile) per half, one per wave
        for (int pos = wave; pos < 4; pos += NW) {
            const int ti = pos >> 1, tj = pos & 1;
            const int jl0 = tj * 16;
            f32x4 aR = mma<SPLIT, D>(zero4(), DYr, ti * 16, YS0T, jl0, lane);
            aR = mma<SPLIT, C>(aR, Pr(0), ti * 16, YBT, jl0, lane);
            aR = mma<SPLIT, C>(aR, Pr(1), ti * 16, YKT, jl0, lane);
            f32x4 aA = mma<SPLIT, D>(zero4(), YDSA, ti * 16, YS0T, jl0, lane);
            aA = mma<SPLIT, C>(aA, Pr(2), ti * 16, YBT, jl0, lane);
            aA = mma<SPLIT, C>(aA, Pr(3), ti * 16, YKT, jl0, lane);
            f32x4 aK = mma<SPLIT, D, true, false>(zero4(), Vr, ti * 16, YGeT, jl0, lane);
            aK = mma<SPLIT, C>(aK, Pt(3), ti * 16, YAT, jl0, lane);
            aK = mma<SPLIT, C>(aK, Pt(1), ti * 16, YRT, jl0, lane);
            f32x4 aB = mma<SPLIT, D>(zero4(), YU, ti * 16, YGeT, jl0, lane);
            aB = mma<SPLIT, C>(aB, Pt(2), ti * 16, YAT, jl0, lane);
            aB = mma<SPLIT, C>(aB, Pt(0), ti * 16, YRT, jl0, lane);
            const int jl = jl0 + r16, j = 32 * half + jl;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = ti * 16 + 4 * g4 + q;
                const float g = gam[t * LDG + j];
                const float gp = t > 0 ? gam[(t - 1) * LDG + j] : 1.f;
                const float ig = rcp(g);
                if (t < Cc) {
                    const int64_t o = base + t * tstride + j;
                    p.dr[o] = aR[q] * g;
                    p.da[o] = aA[q] * gp;
                    p.dk[o] = aK[q] * ig;
                    p.db[o] = aB[q] * ig;
                }
                // k dk = Ktil * aK, b db = Btil * aB, r dr = Rhat * aR, a da = Ahat * aA
                const float fa = get(YAT, jl, t) * aA[q];
                const float ev = get(YKT, jl, t) * aK[q] + get(YBT, jl, t) * aB[q] - get(YRT, jl, t) * aR[q];
                hh_[t * LDG + j] = ev - fa;
                fa_[t * LDG + j] = fa;
            }
        }
        lds_barrier();
        if (half == 0) {
            fill_half(1);
            lds_barrier();
        }
    }

    // ---- dw: phi_t = diag(Gs^T S0) - sum_{s<=t} a da + sum_{s<t} (k dk + b db - r dr),
    //      dw_t = phi_t / w_t.  Thread (jp, q) scans tokens 4q..4q+3 of columns 2jp, 2jp+1.
    {
        constexpr int TPG = RawChunk<NT, InT>::TPG;
        const int jp = tid & 31, q = tid >> 5, j0 = 2 * jp;
        float2 hx[TPG], fx[TPG];
        float2 tot = make_float2(0.f, 0.f);
#pragma unroll
        for (int tt = 0; tt < TPG; ++tt) {
            const int t = q * TPG + tt;
            hx[tt] = *reinterpret_cast<const float2*>(hh_ + t * LDG + j0);
            fx[tt] = *reinterpret_cast<const float2*>(fa_ + t * LDG + j0);
            tot.x += hx[tt].x;
            tot.y += hx[tt].y;
        }
        qp[q * 64 + j0] = tot.x;
        qp[q * 64 + j0 + 1] = tot.y;
        lds_barrier();
        float2 acc = make_float2(red[j0] + red[64 + j0] + red[128 + j0] + red[192 + j0],
                                 red[j0 + 1] + red[64 + j0 + 1] + red[128 + j0 + 1] + red[192 + j0 + 1]);
        for (int q2 = 0; q2 < q; ++q2) {
            acc.x += qp[q2 * 64 + j0];
            acc.y += qp[q2 * 64 + j0 + 1];
        }
#pragma unroll
        for (int tt = 0; tt < TPG; ++tt) {
            const int t = q * TPG + tt;
            if (t < Cc) {
                const float2 wv = Pair<InT>::f(raw.w[tt]);
                *reinterpret_cast<float2*>(p.dw + base + t * tstride + j0) =
                    make_float2((acc.x - fx[tt].x) * rcp(wv.x), (acc.y - fx[tt].y) * rcp(wv.y));
            }
            acc.x += hx[tt].x;
            acc.y += hx[tt].y;
        }
    }
}

template <typename F>
hipError_t set_smem(F kern, int bytes, bool& done) {
    if (done) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done = true;
    return e;
}

template <typename InT, bool SPLIT>
hipError_t launch_inputs_typed(const BwdArgs& a, hipStream_t s) {
    constexpr int NT = 256;
    using L = ChunkSmem<SPLIT>;
    static_assert(L::total <= 160 * 1024, "chunk kernel LDS exceeds 160 KiB");
    auto kern = bwd_chunk_kernel<InT, SPLIT, NT>;
    static bool done = false;
    hipError_t e = set_smem(kern, L::total, done);
    if (e != hipSuccess) return e;
    const int heads = a.B * a.H;
    const int xcd = (heads % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3(heads * a.NC), dim3(NT), L::total, s, a, xcd);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_inputs(const BwdArgs& a, bool bf16, hipStream_t s) {
    if (bf16) return launch_inputs_typed<uint16_t, true>(a, s);
    return launch_inputs_typed<float, false>(a, s);
}

}  // namespace wkv7
