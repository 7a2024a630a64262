// wkv7_fwd.hip -- chunked WKV7 forward on the matrix cores (gfx950).
//
// One workgroup owns RB rows of one head's state (rows are independent in the
// forward: row i only needs its own sa[i], v[i] and the shared column
// vectors) and walks the chunks of the sequence in order.  Per chunk it
//   1. stores the state entering the chunk as checkpoint c (rwkv-mlx page,
//      "Metal kernel architecture": a checkpoint every 32 tokens; here the
//      state entering the chunk, so checkpoint 0 is h0),
//   2. loads the chunk's r, w, k, a, b (all 64 columns) and its v rows,
//   3. forms gamma and the scaled operands, the four C x C matrices and
//      (I - Lab)^-1 (see wkv7_device.h for the algebra),
//   4. U = (I - Lab)^-1 (Ahat S^T + Lak V)        -- sa_t for every token
//      Y = Rhat S^T + Mrb U + Mrk V               -- y_t for every token
//      S <- (S + U^T Btil + V^T Ktil) diag(gamma_last)
// The state never leaves LDS between chunks.
#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

template <int RB>
struct FwdLayout {
    static constexpr int W = 0;
    static constexpr int A = W + C * LDA;
    static constexpr int R = A + C * LDA;
    static constexpr int Bt = R + C * LDA;
    static constexpr int Kt = Bt + C * LDA;
    static constexpr int S = Kt + C * LDA;      // RB x LDA   state rows (i, j)
    static constexpr int VT = S + RB * LDA;     // RB x LDC   v transposed (i, t)
    static constexpr int Lab = VT + RB * LDC;   // C x LDC each
    static constexpr int Lak = Lab + C * LDC;
    static constexpr int Mrb = Lak + C * LDC;
    static constexpr int Mrk = Mrb + C * LDC;
    static constexpr int Tinv = Mrk + C * LDC;
    static constexpr int RhsT = Tinv + C * LDC;  // RB x LDC  (i, t)
    static constexpr int UT = RhsT + RB * LDC;   // RB x LDC  (i, t)
    static constexpr int glast = UT + RB * LDC;  // D
    static constexpr int qp = glast + D;         // 8 x D
    static constexpr int total = qp + 8 * D;
    static constexpr size_t bytes = total * sizeof(float);
};

template <typename InT, bool SPLIT, int RB, int NT>
__global__ __launch_bounds__(NT) void fwd_chunked_kernel(FwdArgs p, int xcd) {
    extern __shared__ float sm[];
    using L = FwdLayout<RB>;
    constexpr int NW = NT / 64;
    constexpr int NRB = D / RB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    int head, rb;
    block_map(blockIdx.x, NRB, xcd != 0, head, rb);
    const int bb = head / p.H, hh = head % p.H;
    const int row0 = rb * RB;
    const int64_t tstride = (int64_t)p.H * D;
    const int64_t soff = (int64_t)head * D * D + (int64_t)row0 * D;

    const InT* __restrict__ gr = static_cast<const InT*>(p.r);
    const InT* __restrict__ gw = static_cast<const InT*>(p.w);
    const InT* __restrict__ gk = static_cast<const InT*>(p.k);
    const InT* __restrict__ gv = static_cast<const InT*>(p.v);
    const InT* __restrict__ ga = static_cast<const InT*>(p.a);
    const InT* __restrict__ gb = static_cast<const InT*>(p.b);

    float* W = sm + L::W;
    float* A = sm + L::A;
    float* R = sm + L::R;
    float* Bt = sm + L::Bt;
    float* Kt = sm + L::Kt;
    float* S = sm + L::S;
    float* VT = sm + L::VT;
    float* Lab = sm + L::Lab;
    float* Lak = sm + L::Lak;
    float* Mrb = sm + L::Mrb;
    float* Mrk = sm + L::Mrk;
    float* Tinv = sm + L::Tinv;
    float* RhsT = sm + L::RhsT;
    float* UT = sm + L::UT;
    float* glast = sm + L::glast;
    float* qp = sm + L::qp;

    load_state_rows<NT, RB>(p.h0 ? p.h0 + soff : nullptr, S, tid);

    for (int c = 0; c < p.NC; ++c) {
        const int t0 = c * C;
        const int Cc = min(C, p.T - t0);
        const int64_t base = ((int64_t)bb * p.T + t0) * tstride + (int64_t)hh * D;
        __syncthreads();
        if (p.ckpt)
            store_state_rows<NT, RB>(S, p.ckpt + ((int64_t)head * p.NC + c) * D * D + (int64_t)row0 * D, tid);
        load_chunk<InT, NT>(gw, base, tstride, Cc, 1.f, W, tid);
        load_chunk<InT, NT>(ga, base, tstride, Cc, 0.f, A, tid);
        load_chunk<InT, NT>(gr, base, tstride, Cc, 0.f, R, tid);
        load_chunk<InT, NT>(gb, base, tstride, Cc, 0.f, Bt, tid);
        load_chunk<InT, NT>(gk, base, tstride, Cc, 0.f, Kt, tid);
        load_chunk_cols_T<InT, NT, RB>(gv, base, tstride, Cc, row0, VT, tid);
        __syncthreads();
        chunk_prep<NT>(W, A, R, Bt, Kt, glast, qp, tid);

        chunk_cc<SPLIT, NT>(A, R, Bt, Kt, Lab, Lak, Mrb, Mrk, tid);
        __syncthreads();

        // (I - Lab)^-1 on the last wave; RHS = Ahat S^T + Lak V on the others.
        constexpr int NTILE = 2 * (RB / 16);  // (C x RB) outputs
        if (wave == NW - 1) tri_inverse(Lab, Tinv, lane);
        if (NW == 1 || wave < NW - 1) {
            const int nwk = NW == 1 ? 1 : NW - 1;
            for (int job = wave; job < NTILE; job += nwk) {
                const int ti = job & 1, tn = job >> 1;
                f32x4 acc = mma<SPLIT, D>(zero4(), rows(A, LDA), ti * 16, rows(S, LDA), tn * 16, lane);
                acc = mma<SPLIT, C>(acc, rows(Lak, LDC), ti * 16, rows(VT, LDC), tn * 16, lane);
                store_tile<LDC, true, MASK_NONE>(RhsT, acc, ti * 16, tn * 16, lane);
            }
        }
        __syncthreads();

        // U = (I - Lab)^-1 RHS, kept transposed (i, t).
        for (int job = wave; job < NTILE; job += NW) {
            const int ti = job & 1, tn = job >> 1;
            const f32x4 acc = mma<SPLIT, C>(zero4(), rows(Tinv, LDC), ti * 16, rows(RhsT, LDC), tn * 16, lane);
            store_tile<LDC, true, MASK_NONE>(UT, acc, ti * 16, tn * 16, lane);
        }
        __syncthreads();

        // y = Rhat S^T + Mrb U + Mrk V, straight to global memory.
        if (p.y) {
            for (int job = wave; job < NTILE; job += NW) {
                const int ti = job & 1, tn = job >> 1;
                f32x4 acc = mma<SPLIT, D>(zero4(), rows(R, LDA), ti * 16, rows(S, LDA), tn * 16, lane);
                acc = mma<SPLIT, C>(acc, rows(Mrb, LDC), ti * 16, rows(UT, LDC), tn * 16, lane);
                acc = mma<SPLIT, C>(acc, rows(Mrk, LDC), ti * 16, rows(VT, LDC), tn * 16, lane);
                const int r = lane & 15, g = lane >> 4;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int t = ti * 16 + 4 * g + q;
                    if (t < Cc) p.y[base + t * tstride + row0 + tn * 16 + r] = acc[q];
                }
            }
        }

        // S <- (S + U^T Btil + V^T Ktil) diag(gamma_last), via registers.
        constexpr int NSTILE = (RB / 16) * 4;
        constexpr int NPER = (NSTILE + NW - 1) / NW;
        f32x4 snew[NPER];
#pragma unroll
        for (int q2 = 0; q2 < NPER; ++q2) {
            const int job = wave + q2 * NW;
            if (job < NSTILE) {
                const int tm = job >> 2, tn = job & 3;
                const int r = lane & 15, g = lane >> 4;
                f32x4 acc;
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] = S[(tm * 16 + 4 * g + q) * LDA + tn * 16 + r];
                acc = mma<SPLIT, C>(acc, rows(UT, LDC), tm * 16, cols(Bt, LDA), tn * 16, lane);
                acc = mma<SPLIT, C>(acc, rows(VT, LDC), tm * 16, cols(Kt, LDA), tn * 16, lane);
                const float gl = glast[tn * 16 + r];
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] *= gl;
                snew[q2] = acc;
            }
        }
        __syncthreads();
#pragma unroll
        for (int q2 = 0; q2 < NPER; ++q2) {
            const int job = wave + q2 * NW;
            if (job < NSTILE) store_tile<LDA, false, MASK_NONE>(S, snew[q2], (job >> 2) * 16, (job & 3) * 16, lane);
        }
    }
    __syncthreads();
    if (p.hT) store_state_rows<NT, RB>(S, p.hT + soff, tid);
}

template <typename InT, bool SPLIT, int RB>
hipError_t launch_rb(const FwdArgs& a, hipStream_t s) {
    constexpr int NT = 256;
    using L = FwdLayout<RB>;
    auto kern = fwd_chunked_kernel<InT, SPLIT, RB, NT>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int heads = a.B * a.H;
    const int nblk = heads * (D / RB);
    const int xcd = (heads % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3(nblk), dim3(NT), L::bytes, s, a, xcd);
    return hipGetLastError();
}

template <typename InT, bool SPLIT>
hipError_t launch_typed(const FwdArgs& a, hipStream_t s) {
    const int heads = a.B * a.H;
    // Row blocks per head: enough workgroups to cover the 256 CUs.
    if (heads >= 256) return launch_rb<InT, SPLIT, 64>(a, s);
    if (heads >= 128) return launch_rb<InT, SPLIT, 32>(a, s);
    return launch_rb<InT, SPLIT, 16>(a, s);
}

}  // namespace

hipError_t launch_fwd_chunked(const FwdArgs& a, bool bf16, hipStream_t s) {
    if (bf16) return launch_typed<uint16_t, true>(a, s);
    return launch_typed<float, false>(a, s);
}

}  // namespace wkv7
