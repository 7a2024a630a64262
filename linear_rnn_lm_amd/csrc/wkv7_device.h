// wkv7_device.h -- device-side building blocks of the WKV7 kernels (gfx950).
//
// Chunked form used by the kernels.  Within one chunk of up to 32 tokens
// (t = 0..C-1, state S0 entering the chunk) let gamma_t = w_0 * ... * w_t
// (elementwise over the column index j, gamma_{-1} = 1) and define the scaled
// operands
//     Ahat_t = a_t * gamma_{t-1},  Rhat_t = r_t * gamma_t,
//     Btil_t = b_t / gamma_t,      Ktil_t = k_t / gamma_t.
// Unrolling the per-token update (state S_t = S_{t-1} (diag w_t + a_t b_t^T)
// + v_t k_t^T; rwkv-mlx page, "Metal kernel architecture", forward block)
// over the chunk gives, with u_t = S_{t-1} a_t (the "sa" vector):
//     S_t = (S0 + sum_{s<=t} u_s Btil_s^T + v_s Ktil_s^T) diag(gamma_t)
// so the chunk's u, y and end state are dense products of (C x 64) and
// (C x C) matrices -- work for the matrix cores (MFMA):
//     U   = (I - Lab)^-1 (Ahat S0^T + Lak V)
//     Y   = Rhat S0^T + Mrb U + Mrk V
//     S_C = (S0 + U^T Btil + V^T Ktil) diag(gamma_{C-1})
// where Lab = strict_lower(Ahat Btil^T), Lak = strict_lower(Ahat Ktil^T),
// Mrb = lower(Rhat Btil^T), Mrk = lower(Rhat Ktil^T).  The backward kernels
// use the same matrices (see wkv7_bwd.hip).
//
// Matrix products read fp32 operands from LDS.  Two precisions:
//   SPLIT = false : v_mfma_f32_16x16x4_f32 (full fp32; used for fp32 inputs)
//   SPLIT = true  : every fp32 operand x is split into bf16 hi = rn(x) and
//                   lo = rn(x - hi); hi*hi + hi*lo + lo*hi on
//                   v_mfma_f32_16x16x32_bf16 (about 2^-17 relative per
//                   product; used for bf16 inputs).
// Both accumulate in fp32 and produce the same 16x16 output layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv7 {

constexpr int D = 64;    // head size (state is D x D)
constexpr int C = 32;    // chunk length (checkpoint interval)
constexpr int LDA = 68;  // LDS row stride (floats) for rows of 64 values
constexpr int LDC = 36;  // LDS row stride (floats) for rows of 32 values

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Block -> (outer, inner) mapping.  Blocks that share `outer` (one head) and
// differ in `inner` (row block or chunk) read the same inputs; with xcd = true
// they are placed on the same XCD (blocks are dealt to the 8 XCDs round
// robin), so those reads share one L2.  Requires n_outer % 8 == 0.
__device__ __forceinline__ void block_map(int blk, int inner_n, bool xcd, int& outer, int& inner) {
    if (xcd) {
        const int x = blk & 7, slot = blk >> 3;
        outer = (slot / inner_n) * 8 + x;
        inner = slot % inner_n;
    } else {
        outer = blk / inner_n;
        inner = blk % inner_n;
    }
}

// ---------------------------------------------------------------------------
// Global loads of 8 consecutive values, widened to fp32.
__device__ __forceinline__ void load8(const float* p, float* o) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, float* o) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        o[2 * q] = __uint_as_float(w[q] << 16);              // bf16 -> fp32 is exact
        o[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
}

// Load one chunk (C tokens x 64 values) of a (B,T,H,D) tensor into LDS rows
// dst[t*LDA + j].  Tokens t >= Cc get `fill`.
template <typename InT, int NT>
__device__ __forceinline__ void load_chunk(const InT* __restrict__ src, int64_t base, int64_t tstride,
                                           int Cc, float fill, float* dst, int tid) {
    for (int e = tid; e < C * 8; e += NT) {
        const int t = e >> 3, j0 = (e & 7) * 8;
        float v[8];
        if (t < Cc) {
            load8(src + base + t * tstride + j0, v);
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = fill;
        }
        float4* d = reinterpret_cast<float4*>(dst + t * LDA + j0);
        d[0] = make_float4(v[0], v[1], v[2], v[3]);
        d[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// Load columns [col0, col0+NCOL) of one chunk transposed: dst[i*LDC + t].
template <typename InT, int NT, int NCOL>
__device__ __forceinline__ void load_chunk_cols_T(const InT* __restrict__ src, int64_t base, int64_t tstride,
                                                  int Cc, int col0, float* dst, int tid) {
    constexpr int G = NCOL / 8;
    for (int e = tid; e < C * G; e += NT) {
        const int t = e / G, i0 = (e % G) * 8;
        float v[8];
        if (t < Cc) {
            load8(src + base + t * tstride + col0 + i0, v);
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = 0.f;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) dst[(i0 + q) * LDC + t] = v[q];
    }
}

// Copy NROW rows of a row-major 64-wide fp32 global matrix into LDS rows
// (stride LDA); src == nullptr gives zeros.
template <int NT, int NROW>
__device__ __forceinline__ void load_state_rows(const float* __restrict__ src, float* dst, int tid) {
    for (int e = tid; e < NROW * 16; e += NT) {
        const int i = e >> 4, j4 = (e & 15) * 4;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (src) v = *reinterpret_cast<const float4*>(src + i * D + j4);
        *reinterpret_cast<float4*>(dst + i * LDA + j4) = v;
    }
}

template <int NT, int NROW>
__device__ __forceinline__ void store_state_rows(const float* src, float* __restrict__ dst, int tid) {
    for (int e = tid; e < NROW * 16; e += NT) {
        const int i = e >> 4, j4 = (e & 15) * 4;
        *reinterpret_cast<float4*>(dst + i * D + j4) = *reinterpret_cast<const float4*>(src + i * LDA + j4);
    }
}

// ---------------------------------------------------------------------------
// LDS operand view: element (m, k) = p[m*sm + k*sk].
struct Op {
    const float* p;
    int sm, sk;
};
__device__ __forceinline__ Op rows(const float* p, int ld) { return Op{p, ld, 1}; }  // (m,k) = p[m][k]
__device__ __forceinline__ Op cols(const float* p, int ld) { return Op{p, 1, ld}; }  // (m,k) = p[k][m]

// acc += X[m0:m0+16, 0:K] * Y[n0:n0+16, 0:K]^T   (one wave, one 16x16 tile)
// Output layout: acc[q] holds element (m0 + 4*(lane/16) + q, n0 + lane%16).
template <bool SPLIT, int K>
__device__ __forceinline__ f32x4 mma(f32x4 acc, Op X, int m0, Op Y, int n0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    if constexpr (!SPLIT) {
        const float* xp = X.p + (m0 + r) * X.sm + g * X.sk;
        const float* yp = Y.p + (n0 + r) * Y.sm + g * Y.sk;
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += 4)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xp[k0 * X.sk], yp[k0 * Y.sk], acc, 0, 0, 0);
    } else {
        const float* xp = X.p + (m0 + r) * X.sm + 8 * g * X.sk;
        const float* yp = Y.p + (n0 + r) * Y.sm + 8 * g * Y.sk;
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += 32) {
            bf16x8 xh, xl, yh, yl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xv = xp[(k0 + e) * X.sk];
                const float yv = yp[(k0 + e) * Y.sk];
                const __bf16 xhe = (__bf16)xv;
                const __bf16 yhe = (__bf16)yv;
                xh[e] = xhe;
                yh[e] = yhe;
                xl[e] = (__bf16)(xv - (float)xhe);
                yl[e] = (__bf16)(yv - (float)yhe);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, yh, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, yl, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, yh, acc, 0, 0, 0);
        }
    }
    return acc;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Write a 16x16 tile to an LDS matrix, optionally transposed, optionally
// keeping only the lower triangle of the full matrix (strict: row > col).
enum Mask { MASK_NONE = 0, MASK_LOWER = 1, MASK_STRICT = 2 };
template <int LD, bool TRANS, int MASK>
__device__ __forceinline__ void store_tile(float* M, f32x4 acc, int m0, int n0, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int m = m0 + 4 * g + q, n = n0 + r;
        float v = acc[q];
        if (MASK == MASK_LOWER && m < n) v = 0.f;
        if (MASK == MASK_STRICT && m <= n) v = 0.f;
        if (TRANS) M[n * LD + m] = v;
        else M[m * LD + n] = v;
    }
}

// ---------------------------------------------------------------------------
// Chunk preparation.  On entry W, A, R, Bt, Kt (C x LDA) hold raw w, a, r, b,
// k of the chunk (padding tokens: w = 1, the rest 0).  On exit W holds
// gamma_t, A = a*gamma_{t-1}, R = r*gamma_t, Bt = b/gamma_t, Kt = k/gamma_t,
// and glast[j] = gamma_{C-1}[j].  qp is LDS scratch of (NT/64) x 64 floats.
// Ends with a barrier.
template <int NT>
__device__ __forceinline__ void chunk_prep(float* W, float* A, float* R, float* Bt, float* Kt,
                                           float* glast, float* qp, int tid) {
    constexpr int NG = NT / 64, TPG = C / NG;
    static_assert(NT % 64 == 0 && C % NG == 0, "chunk_prep thread shape");
    const int j = tid & 63, q = tid >> 6;
    float loc[TPG];
    float p = 1.f;
#pragma unroll
    for (int tt = 0; tt < TPG; ++tt) {
        p *= W[(q * TPG + tt) * LDA + j];
        loc[tt] = p;
    }
    qp[q * 64 + j] = p;
    __syncthreads();
    float pre = 1.f, tot = 1.f;
#pragma unroll
    for (int q2 = 0; q2 < NG; ++q2) {
        const float x = qp[q2 * 64 + j];
        if (q2 < q) pre *= x;
        tot *= x;
    }
    float gprev = pre;
#pragma unroll
    for (int tt = 0; tt < TPG; ++tt) {
        const int t = q * TPG + tt;
        const float g = (q == 0) ? loc[tt] : pre * loc[tt];
        const float inv = 1.f / g;
        A[t * LDA + j] *= gprev;
        R[t * LDA + j] *= g;
        Bt[t * LDA + j] *= inv;
        Kt[t * LDA + j] *= inv;
        W[t * LDA + j] = g;
        gprev = g;
    }
    if (q == 0) glast[j] = tot;
    __syncthreads();
}

// Tinv = (I - L)^-1 for a strictly lower triangular C x C matrix L (row
// stride LDC), by forward substitution; one wave, lane k < 32 owns column k.
__device__ __forceinline__ void tri_inverse(const float* L, float* Tinv, int lane) {
    if (lane < C) {
        const int k = lane;
        float x[C];
#pragma unroll
        for (int t = 0; t < C; ++t) {
            float acc0 = (t == k) ? 1.f : 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
#pragma unroll
            for (int s = 0; s < t; s += 4) {
                acc0 = fmaf(L[t * LDC + s], x[s], acc0);
                if (s + 1 < t) acc1 = fmaf(L[t * LDC + s + 1], x[s + 1], acc1);
                if (s + 2 < t) acc2 = fmaf(L[t * LDC + s + 2], x[s + 2], acc2);
                if (s + 3 < t) acc3 = fmaf(L[t * LDC + s + 3], x[s + 3], acc3);
            }
            x[t] = (acc0 + acc1) + (acc2 + acc3);
        }
#pragma unroll
        for (int t = 0; t < C; ++t) Tinv[t * LDC + k] = x[t];
    }
}

// The four C x C matrices of a chunk: Lab, Lak (strictly lower), Mrb, Mrk
// (lower incl. diagonal).  12 lower tiles spread over the waves, plus the
// zero upper-right tile of each.  No barrier at the end.
template <bool SPLIT, int NT>
__device__ __forceinline__ void chunk_cc(const float* A, const float* R, const float* Bt, const float* Kt,
                                         float* Lab, float* Lak, float* Mrb, float* Mrk, int tid) {
    constexpr int NW = NT / 64;
    const int lane = tid & 63, wave = tid >> 6;
    for (int job = wave; job < 12; job += NW) {
        const int mat = job / 3, tile = job % 3;
        const int ti = tile == 0 ? 0 : 1, tj = tile == 2 ? 1 : 0;
        const Op X = rows(mat < 2 ? A : R, LDA);
        const Op Y = rows((mat & 1) ? Kt : Bt, LDA);
        const f32x4 acc = mma<SPLIT, D>(zero4(), X, ti * 16, Y, tj * 16, lane);
        float* M = mat == 0 ? Lab : mat == 1 ? Lak : mat == 2 ? Mrb : Mrk;
        if (mat < 2) store_tile<LDC, false, MASK_STRICT>(M, acc, ti * 16, tj * 16, lane);
        else store_tile<LDC, false, MASK_LOWER>(M, acc, ti * 16, tj * 16, lane);
    }
    for (int e = tid; e < 4 * 256; e += NT) {
        const int m = e >> 8, t = (e & 255) >> 4, s = 16 + (e & 15);
        float* M = m == 0 ? Lab : m == 1 ? Lak : m == 2 ? Mrb : Mrk;
        M[t * LDC + s] = 0.f;
    }
}

}  // namespace wkv7
