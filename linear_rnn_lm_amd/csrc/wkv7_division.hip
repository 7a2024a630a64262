// wkv7_division.hip -- diagnostic: the backward of the rwkv-mlx page's Metal
// design, which rebuilds every earlier state from the later one by undoing
// the update (dividing by w) instead of recomputing it from a checkpoint.
//
// rwkv-mlx page, "Metal kernel architecture", backward block: the walk over
// a chunk starts from the exact checkpoint and, token by token in reverse,
// takes the per-token VJP and reconstructs the previous state as
// (h_cur - v k - sa b) / w; the paragraph after it puts the error growth of
// that division at (1/w)^N.  The page does not say how sa is recovered
// before the previous state is known; here it is solved exactly: with
// z = S_t[i] - v[i] k, the previous row x satisfies x w + (x . a) b = z, so
// sa = (z . (a/w)) / (1 + b . (a/w)) and x = (z - sa b) / w.
//
// One workgroup of one wave per head; lane i keeps state row i and gradient
// row i in registers (like the page's one thread per row).  The per-token
// vectors pass through LDS; the column sums over rows (dr, dw, dk, da, db)
// go through an LDS transpose.  This is a slow, plain kernel: it exists to
// measure the division's error growth on the GPU, not for training.
#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

constexpr int DIV_LD = D + 4;   // LDS row stride of the partial sums (16-byte rows, conflict-free columns)

// Keeps the compiler from hoisting the LDS reads of later column blocks above
// this point (all of them at once would not fit the registers).
__device__ __forceinline__ void block_fence() { asm volatile("" ::: "memory"); }

template <typename InT>
__device__ __forceinline__ float ld1(const InT* p);
template <>
__device__ __forceinline__ float ld1<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld1<uint16_t>(const uint16_t* p) { return __uint_as_float((uint32_t)(*p) << 16); }

template <typename InT>
__global__ __launch_bounds__(64) void bwd_division_kernel(DivArgs p) {
    __shared__ float vec[6][D];                         // r, w, k, v, a, b of the token
    __shared__ __attribute__((aligned(16))) float part[5][D * DIV_LD];   // rows i: dr, dw, dk, db, da terms
    const int i = threadIdx.x;                          // state row; also the column this lane sums
    const int head = blockIdx.x;
    const int bb = head / p.H, hh = head - bb * p.H;
    const int64_t tstride = (int64_t)p.H * D;
    const int64_t srow = (int64_t)head * D * D + (int64_t)i * D;
    const InT* src[6] = {static_cast<const InT*>(p.r), static_cast<const InT*>(p.w), static_cast<const InT*>(p.k),
                         static_cast<const InT*>(p.v), static_cast<const InT*>(p.a), static_cast<const InT*>(p.b)};

    float S[D], g[D];
#pragma unroll
    for (int j = 0; j < D; ++j) g[j] = p.dhT ? p.dhT[srow + j] : 0.f;

    // the next token's inputs are loaded one token ahead, into registers
    float nv[6], ndy = 0.f;
    auto load_token = [&](int t) {
        const int64_t base = ((int64_t)bb * p.T + t) * tstride + (int64_t)hh * D;
#pragma unroll
        for (int q = 0; q < 6; ++q) nv[q] = ld1<InT>(src[q] + base + i);
        ndy = p.dy[base + i];
    };
    load_token(p.T - 1);
    for (int t = p.T - 1; t >= 0; --t) {
        const int64_t base = ((int64_t)bb * p.T + t) * tstride + (int64_t)hh * D;
        if (t == p.T - 1 || (p.restart && t % C == C - 1)) {
            // the exact state after token t: hT, or the checkpoint entering the next chunk
            const float* e = (t == p.T - 1) ? p.hT + srow : p.ckpt + ((int64_t)head * p.NC + t / C + 1) * D * D + i * D;
#pragma unroll
            for (int j = 0; j < D; ++j) S[j] = e[j];
        }
        {
#pragma unroll
            for (int q = 0; q < 6; ++q) vec[q][i] = nv[q];
            const float dyi = ndy;
            if (t > 0) load_token(t - 1);
            lds_barrier();
            const float vi = vec[3][i];
            // S holds S_t.  dr_t[j] = sum_i dy[i] S_t[i][j]; g += dy r^T
            float num = 0.f, den = 1.f;
#pragma unroll
            for (int j = 0; j < D; ++j) {
                if (j % 16 == 0) block_fence();
                part[0][i * DIV_LD + j] = dyi * S[j];
                g[j] += dyi * vec[0][j];
                const float z = S[j] - vi * vec[2][j];
                const float aw = vec[4][j] / vec[1][j];
                S[j] = z;
                num += z * aw;
                den += vec[5][j] * aw;
            }
            // the previous state by division
            const float sa = num / den;
            float dv = 0.f, dsa = 0.f;
#pragma unroll
            for (int j = 0; j < D; ++j) {
                if (j % 16 == 0) block_fence();
                S[j] = (S[j] - sa * vec[5][j]) / vec[1][j];      // S_{t-1}[i][j]
                part[1][i * DIV_LD + j] = g[j] * S[j];           // dw
                part[2][i * DIV_LD + j] = g[j] * vi;             // dk
                part[3][i * DIV_LD + j] = g[j] * sa;             // db
                dv += g[j] * vec[2][j];
                dsa += g[j] * vec[5][j];
            }
#pragma unroll
            for (int j = 0; j < D; ++j) {
                if (j % 16 == 0) block_fence();
                part[4][i * DIV_LD + j] = dsa * S[j];            // da
                g[j] = vec[1][j] * g[j] + dsa * vec[4][j];
            }
            p.dv[base + i] = dv;
            lds_barrier();
            // column sums: lane i adds column i over the 64 rows
            float sums[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
            for (int r = 0; r < D; ++r) {
#pragma unroll
                for (int m = 0; m < 5; ++m) sums[m] += part[m][r * DIV_LD + i];
            }
            p.dr[base + i] = sums[0];
            p.dw[base + i] = sums[1];
            p.dk[base + i] = sums[2];
            p.db[base + i] = sums[3];
            p.da[base + i] = sums[4];
            lds_barrier();   // the token's LDS reads before the next token's writes
        }
    }
    if (p.dh0) {
#pragma unroll
        for (int j = 0; j < D; ++j) p.dh0[srow + j] = g[j];
    }
}

}  // namespace

hipError_t launch_bwd_division(const DivArgs& a, bool bf16, hipStream_t s) {
    const int heads = a.B * a.H;
    if (bf16) hipLaunchKernelGGL(bwd_division_kernel<uint16_t>, dim3(heads), dim3(64), 0, s, a);
    else hipLaunchKernelGGL(bwd_division_kernel<float>, dim3(heads), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace wkv7
