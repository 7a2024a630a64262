// wkv7_inv.hip -- per-chunk inverse (I - Lab)^-1 of the WKV7 chunked form.
//
// For every (head, chunk): gamma = running product of w within the chunk,
// Ahat = a * gamma_{t-1}, Btil = b / gamma_t, Lab = strict_lower(Ahat Btil^T)
// (wkv7_device.h has the algebra) and T = (I - Lab)^-1, written as fp32
// (B, H, NC, 32, 32) row-major.  T only depends on w, a, b of its chunk, so
// all chunks are independent: one wave per (head, chunk), no barriers.  The
// sequential kernels then take T from memory instead of solving the 32-step
// triangular system on their critical path.
#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

template <bool SPLIT>
struct InvSmem {
    using F = Fmt<SPLIT>;
    static constexpr int A = 0;                    // Ahat rows (t, j)
    static constexpr int Bm = A + F::bytes(C, D);  // Btil rows
    static constexpr int LabF = Bm + F::bytes(C, D);
    static constexpr int total = LabF + C * LDF * 4;
    // after Lab is formed, T and the scratch reuse Ahat's space
    static constexpr int TinvF = 0;
    static constexpr int Scr = TinvF + C * LDF * 4;
    static_assert(Scr + 16 * 20 * 4 <= Bm, "inverse scratch overflows Ahat");
};

template <typename InT, bool SPLIT>
__global__ __launch_bounds__(64) void chunk_inv_kernel(InvArgs p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    using L = InvSmem<SPLIT>;
    const int lane = threadIdx.x;
    const int item = blockIdx.x;              // (head, chunk)
    const int head = item / p.NC, c = item % p.NC;
    const int bb = head / p.H, hh = head % p.H;
    const int64_t tstride = (int64_t)p.H * D;
    const int t0 = c * C;
    const int Cc = min(C, p.T - t0);
    const int64_t base = ((int64_t)bb * p.T + t0) * tstride + (int64_t)hh * D;
    const InT* gw = static_cast<const InT*>(p.w);
    const InT* ga = static_cast<const InT*>(p.a);
    const InT* gb = static_cast<const InT*>(p.b);

    // lane j owns column j for all tokens
    const int j = lane;
    float wv[C], av[C], bv[C];
#pragma unroll
    for (int t = 0; t < C; ++t) {
        const int64_t o = base + min(t, Cc - 1) * tstride + j;
        wv[t] = load1(gw + o);
        av[t] = load1(ga + o);
        bv[t] = load1(gb + o);
    }
    const Mat<SPLIT> A = make_mat<SPLIT>(smem, L::A, C, D), Bm = make_mat<SPLIT>(smem, L::Bm, C, D);
    float g = 1.f;
#pragma unroll
    for (int t = 0; t < C; ++t) {
        const bool in = t < Cc;
        const float gprev = g;
        g *= in ? wv[t] : 1.f;
        put(A, t, j, in ? av[t] * gprev : 0.f);
        put(Bm, t, j, in ? bv[t] * rcp(g) : 0.f);
    }
    wave_lds_sync();

    float* labf = reinterpret_cast<float*>(smem + L::LabF);
    f32x4 t00 = mma<SPLIT, D>(zero4(), A, 0, Bm, 0, lane);
    f32x4 t10 = mma<SPLIT, D>(zero4(), A, 16, Bm, 0, lane);
    f32x4 t11 = mma<SPLIT, D>(zero4(), A, 16, Bm, 16, lane);
    store_f32<MASK_STRICT>(labf, LDF, t00, 0, 0, lane);
    store_f32<MASK_STRICT>(labf, LDF, t10, 16, 0, lane);
    store_f32<MASK_STRICT>(labf, LDF, t11, 16, 16, lane);
    for (int e = lane; e < 256; e += 64) labf[(e >> 4) * LDF + 16 + (e & 15)] = 0.f;
    wave_lds_sync();

    float* tinvf = reinterpret_cast<float*>(smem + L::TinvF);
    float* scr = reinterpret_cast<float*>(smem + L::Scr);
    tri_inverse(labf, tinvf, scr, lane);

    float* out = p.inv + (int64_t)item * C * C;
    // lane -> row lane/2, 16 columns
    const int t = lane >> 1, s0 = (lane & 1) * 16;
#pragma unroll
    for (int s4 = 0; s4 < 16; s4 += 4)
        *reinterpret_cast<f32x4*>(out + t * C + s0 + s4) = *reinterpret_cast<const f32x4*>(tinvf + t * LDF + s0 + s4);
}

template <typename InT, bool SPLIT>
hipError_t launch_typed(const InvArgs& a, hipStream_t s) {
    using L = InvSmem<SPLIT>;
    const int items = a.B * a.H * a.NC;
    hipLaunchKernelGGL((chunk_inv_kernel<InT, SPLIT>), dim3(items), dim3(64), L::total, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_inv(const InvArgs& a, bool bf16, hipStream_t s) {
    if (bf16) return launch_typed<uint16_t, true>(a, s);
    return launch_typed<float, false>(a, s);
}

}  // namespace wkv7
