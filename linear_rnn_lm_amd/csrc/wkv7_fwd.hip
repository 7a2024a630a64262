// wkv7_fwd.hip -- chunked WKV7 forward on the matrix cores (gfx950).
//
// One workgroup owns RB rows of one head's state (rows are independent in the
// forward: row i only needs its own sa[i], v[i] and the shared column
// vectors) and walks the chunks of the sequence in order.  Per chunk it
//   1. stores the state entering the chunk as checkpoint c (rwkv-mlx page,
//      "Metal kernel architecture": a checkpoint every 32 tokens; here the
//      state entering the chunk, so checkpoint 0 is h0),
//   2. turns the chunk's r, w, k, a, b (prefetched into registers during the
//      previous chunk) into gamma and the scaled operands, and forms the four
//      C x C matrices and (I - Lab)^-1 (see wkv7_device.h for the algebra),
//   3. U = (I - Lab)^-1 (Ahat S^T + Lak V)        -- sa_t for every token
//      Y = Rhat S^T + Mrb U + Mrk V               -- y_t for every token
//      S <- (S + U^T Btil + V^T Ktil) diag(gamma_last)
// The fp32 state lives in the registers of the wave that owns each 16 x 16
// tile; LDS holds only its operand copy.
#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

template <bool SPLIT, int RB>
struct FwdSmem {
    using F = Fmt<SPLIT>;
    static constexpr int A = 0;                          // Ahat rows (t, j)
    static constexpr int R = A + F::bytes(C, D);         // Rhat rows
    static constexpr int Bm = R + F::bytes(C, D);        // Btil rows
    static constexpr int Km = Bm + F::bytes(C, D);       // Ktil rows
    static constexpr int BT = Km + F::bytes(C, D);       // Btil^T (j, t)
    static constexpr int KT = BT + F::bytes(D, C);       // Ktil^T (j, t)
    static constexpr int S = KT + F::bytes(D, C);        // state rows (i, j)
    static constexpr int VT = S + F::bytes(RB, D);       // v^T (i, t)
    static constexpr int Lak = VT + F::bytes(RB, C);     // (t, s)
    static constexpr int Mrb = Lak + F::bytes(C, C);
    static constexpr int Mrk = Mrb + F::bytes(C, C);
    static constexpr int Tinv = Mrk + F::bytes(C, C);
    static constexpr int RhsT = Tinv + F::bytes(C, C);   // (i, t)
    static constexpr int UT = RhsT + F::bytes(RB, C);    // (i, t)
    static constexpr int glast = UT + F::bytes(RB, C);
    static constexpr int qp = glast + D * 4;             // fp32 8 x 64
    static constexpr int total = qp + 8 * D * 4;
};

template <typename InT, bool SPLIT, int RB, int NT>
__global__ __launch_bounds__(NT) void fwd_chunked_kernel(FwdArgs p, int xcd) {
    static_assert(NT == 256, "one raw-chunk thread shape");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    using L = FwdSmem<SPLIT, RB>;
    using M = Mat<SPLIT>;
    constexpr int NW = NT / 64;
    constexpr int NRB = D / RB;
    constexpr int NTILE = 2 * (RB / 16);      // (C x RB) outputs
    constexpr int NST = (RB / 16) * 4;        // (RB x D) state tiles
    constexpr int NPER = (NST + NW - 1) / NW;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;

    int head, rb;
    block_map(blockIdx.x, NRB, xcd != 0, head, rb);
    const int bb = head / p.H, hh = head % p.H;
    const int row0 = rb * RB;
    const int64_t tstride = (int64_t)p.H * D;
    const int64_t soff = (int64_t)head * D * D + (int64_t)row0 * D;

    const InT* gr = static_cast<const InT*>(p.r);
    const InT* gw = static_cast<const InT*>(p.w);
    const InT* gk = static_cast<const InT*>(p.k);
    const InT* gv = static_cast<const InT*>(p.v);
    const InT* ga = static_cast<const InT*>(p.a);
    const InT* gb = static_cast<const InT*>(p.b);

    const M A = make_mat<SPLIT>(smem, L::A, C, D), R = make_mat<SPLIT>(smem, L::R, C, D);
    const M Bm = make_mat<SPLIT>(smem, L::Bm, C, D), Km = make_mat<SPLIT>(smem, L::Km, C, D);
    const M BT = make_mat<SPLIT>(smem, L::BT, D, C), KT = make_mat<SPLIT>(smem, L::KT, D, C);
    const M S = make_mat<SPLIT>(smem, L::S, RB, D), VT = make_mat<SPLIT>(smem, L::VT, RB, C);
    const M Lak = make_mat<SPLIT>(smem, L::Lak, C, C), Mrb = make_mat<SPLIT>(smem, L::Mrb, C, C);
    const M Mrk = make_mat<SPLIT>(smem, L::Mrk, C, C), Tinv = make_mat<SPLIT>(smem, L::Tinv, C, C);
    const M RhsT = make_mat<SPLIT>(smem, L::RhsT, RB, C), UT = make_mat<SPLIT>(smem, L::UT, RB, C);
    float* glast = reinterpret_cast<float*>(smem + L::glast);
    float* qp = reinterpret_cast<float*>(smem + L::qp);

    const PrepOut<SPLIT> po{A, R, Bm, Km, A, A, BT, KT, true, true, true, true, false, false, true, true,
                            nullptr, glast};
    const CcOut<SPLIT, NT> co{nullptr, Lak, Lak, Mrb, Mrb, Mrk, Mrk, true, false, true, false, true, false};

    // wave-owned state tiles, from h0
    f32x4 st[NPER];
#pragma unroll
    for (int q2 = 0; q2 < NPER; ++q2) {
        const int job = wave + q2 * NW;
        if (job < NST) {
            const int tm = job >> 2, tn = job & 3;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                st[q2][q] = p.h0 ? p.h0[soff + (tm * 16 + 4 * g4 + q) * D + tn * 16 + r16] : 0.f;
            store_rows<MASK_NONE>(S, st[q2], tm * 16, tn * 16, lane);
        }
    }

    RawChunk<NT, InT> raw;
    RawCols<NT, RB, InT> rv;
    f32x4 tv;   // four entries of the chunk's (I - Lab)^-1: row tid/8, columns 4*(tid%8)..
    const float* ginv = p.inv + (int64_t)head * p.NC * C * C + tid * 4;
    {
        const int Cc0 = min(C, p.T);
        const int64_t base0 = (int64_t)bb * p.T * tstride + (int64_t)hh * D;
        raw.load(gw, ga, gr, gb, gk, base0, tstride, Cc0, tid);
        rv.load(gv, base0, tstride, Cc0, row0, tid);
        tv = *reinterpret_cast<const f32x4*>(ginv);
    }

    // y of the previous chunk, stored at the start of the next one (so that no
    // store is issued between a prefetch and the wait for it)
    constexpr int NYPER = (NTILE + NW - 1) / NW;
    f32x4 yv[NYPER];
    int64_t ybase = 0;
    int yCc = 0;

    for (int c = 0; c < p.NC; ++c) {
        const int t0 = c * C;
        const int Cc = min(C, p.T - t0);
        const int64_t base = ((int64_t)bb * p.T + t0) * tstride + (int64_t)hh * D;

        chunk_prep<NT, SPLIT>(raw, po, qp, tid);
        rv.template store_T<SPLIT, true>(VT, tid);
        put4(Tinv, tid >> 3, (tid & 7) * 4, tv);

        // global stores of the previous chunk's y and of checkpoint c
        if (p.y && c > 0) {
#pragma unroll
            for (int q2 = 0; q2 < NYPER; ++q2) {
                const int job = wave + q2 * NW;
                if (job < NTILE) {
                    const int ti = job & 1, tn = job >> 1;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int t = ti * 16 + 4 * g4 + q;
                        if (t < yCc) p.y[ybase + t * tstride + row0 + tn * 16 + r16] = yv[q2][q];
                    }
                }
            }
        }
        if (p.ckpt) {
            float* ck = p.ckpt + ((int64_t)head * p.NC + c) * D * D + (int64_t)row0 * D;
#pragma unroll
            for (int q2 = 0; q2 < NPER; ++q2) {
                const int job = wave + q2 * NW;
                if (job < NST) {
                    const int tm = job >> 2, tn = job & 3;
#pragma unroll
                    for (int q = 0; q < 4; ++q) ck[(tm * 16 + 4 * g4 + q) * D + tn * 16 + r16] = st[q2][q];
                }
            }
        }
        // prefetch the next chunk (the last chunk re-reads itself)
        {
            const int cn = min(c + 1, p.NC - 1);
            const int64_t nbase = ((int64_t)bb * p.T + cn * C) * tstride + (int64_t)hh * D;
            const int nCc = min(C, p.T - cn * C);
            raw.load(gw, ga, gr, gb, gk, nbase, tstride, nCc, tid);
            rv.load(gv, nbase, tstride, nCc, row0, tid);
            tv = *reinterpret_cast<const f32x4*>(ginv + (int64_t)cn * C * C);
        }
        lds_barrier();

        chunk_cc<SPLIT, NT>(A, R, Bm, Km, co, tid);
        lds_barrier();

        // RHS = Ahat S^T + Lak V
        for (int job = wave; job < NTILE; job += NW) {
            const int ti = job & 1, tn = job >> 1;
            f32x4 acc = mma<SPLIT, D>(zero4(), A, ti * 16, S, tn * 16, lane);
            acc = mma<SPLIT, C, false, true>(acc, Lak, ti * 16, VT, tn * 16, lane);
            store_cols<MASK_NONE>(RhsT, acc, ti * 16, tn * 16, lane);
        }
        lds_barrier();

        // U = (I - Lab)^-1 RHS, kept transposed (i, t).
        for (int job = wave; job < NTILE; job += NW) {
            const int ti = job & 1, tn = job >> 1;
            const f32x4 acc = mma<SPLIT, C>(zero4(), Tinv, ti * 16, RhsT, tn * 16, lane);
            store_cols<MASK_NONE>(UT, acc, ti * 16, tn * 16, lane);
        }
        lds_barrier();

        // y = Rhat S^T + Mrb U + Mrk V (kept in registers until the next chunk)
#pragma unroll
        for (int q2 = 0; q2 < NYPER; ++q2) {
            const int job = wave + q2 * NW;
            if (job < NTILE) {
                const int ti = job & 1, tn = job >> 1;
                f32x4 acc = mma<SPLIT, D>(zero4(), R, ti * 16, S, tn * 16, lane);
                acc = mma<SPLIT, C>(acc, Mrb, ti * 16, UT, tn * 16, lane);
                yv[q2] = mma<SPLIT, C, false, true>(acc, Mrk, ti * 16, VT, tn * 16, lane);
            }
        }
        ybase = base;
        yCc = Cc;

        // S <- (S + U^T Btil + V^T Ktil) diag(gamma_last)
#pragma unroll
        for (int q2 = 0; q2 < NPER; ++q2) {
            const int job = wave + q2 * NW;
            if (job < NST) {
                const int tm = job >> 2, tn = job & 3;
                f32x4 acc = mma<SPLIT, C>(st[q2], UT, tm * 16, BT, tn * 16, lane);
                acc = mma<SPLIT, C, true, false>(acc, VT, tm * 16, KT, tn * 16, lane);
                const float gl = glast[tn * 16 + r16];
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] *= gl;
                st[q2] = acc;
            }
        }
        lds_barrier();
#pragma unroll
        for (int q2 = 0; q2 < NPER; ++q2) {
            const int job = wave + q2 * NW;
            if (job < NST) store_rows<MASK_NONE>(S, st[q2], (job >> 2) * 16, (job & 3) * 16, lane);
        }
    }

    if (p.y) {
#pragma unroll
        for (int q2 = 0; q2 < NYPER; ++q2) {
            const int job = wave + q2 * NW;
            if (job < NTILE) {
                const int ti = job & 1, tn = job >> 1;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int t = ti * 16 + 4 * g4 + q;
                    if (t < yCc) p.y[ybase + t * tstride + row0 + tn * 16 + r16] = yv[q2][q];
                }
            }
        }
    }
    if (p.hT) {
#pragma unroll
        for (int q2 = 0; q2 < NPER; ++q2) {
            const int job = wave + q2 * NW;
            if (job < NST) {
                const int tm = job >> 2, tn = job & 3;
#pragma unroll
                for (int q = 0; q < 4; ++q) p.hT[soff + (tm * 16 + 4 * g4 + q) * D + tn * 16 + r16] = st[q2][q];
            }
        }
    }
}

template <typename InT, bool SPLIT, int RB>
hipError_t launch_rb(const FwdArgs& a, hipStream_t s) {
    constexpr int NT = 256;
    using L = FwdSmem<SPLIT, RB>;
    static_assert(L::total <= 160 * 1024, "forward kernel LDS exceeds 160 KiB");
    auto kern = fwd_chunked_kernel<InT, SPLIT, RB, NT>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, L::total);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int heads = a.B * a.H;
    const int nblk = heads * (D / RB);
    const int xcd = (heads % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3(nblk), dim3(NT), L::total, s, a, xcd);
    return hipGetLastError();
}

template <typename InT, bool SPLIT>
hipError_t launch_typed(const FwdArgs& a, hipStream_t s) {
    const int heads = a.B * a.H;
    // Row blocks per head: as many workgroups as fit one per CU (256 CUs).
    if (heads > 128) return launch_rb<InT, SPLIT, 64>(a, s);
    if (heads > 64) return launch_rb<InT, SPLIT, 32>(a, s);
    return launch_rb<InT, SPLIT, 16>(a, s);
}

}  // namespace

hipError_t launch_fwd_chunked(const FwdArgs& a, bool bf16, hipStream_t s) {
    if (bf16) return launch_typed<uint16_t, true>(a, s);
    return launch_typed<float, false>(a, s);
}

}  // namespace wkv7
