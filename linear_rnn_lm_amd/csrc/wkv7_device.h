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
//     S_C = (S0 + U^T Btil + V^T Ktil) diag(gamma_last)
// where Lab = strict_lower(Ahat Btil^T), Lak = strict_lower(Ahat Ktil^T),
// Mrb = lower(Rhat Btil^T), Mrk = lower(Rhat Ktil^T).  The backward kernels
// use the same matrices (wkv7_grad.hip).
//
// Every product is C[m][n] = sum_k X[m][k] Y[n][k] with both operands held in
// LDS with k contiguous ("Mat").  Two storage formats:
//   SPLIT = true  (bf16 inputs): each fp32 value x is stored once as two bf16
//                 planes, hi = rn(x) and lo = rn(x - hi); a product is
//                 hi*hi + hi*lo + lo*hi on v_mfma_f32_16x16x32_bf16 (about
//                 2^-17 relative per product, fp32 accumulation).  Operands
//                 known to be exact in bf16 (the raw v) skip their lo term.
//   SPLIT = false (fp32 inputs): one fp32 plane, v_mfma_f32_16x16x4_f32.
// Rows are padded (by 8 bf16 / 4 fp32) so that the 16-byte operand reads of
// one MFMA hit distinct LDS banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace wkv7 {

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_seq(f, std::make_integer_sequence<int, N>{});
}

constexpr int D = 64;  // head size (state is D x D)
constexpr int C = 32;  // chunk length (checkpoint interval)
constexpr int LDF = 36;  // row stride (floats) of fp32 C x C scratch matrices

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Wait for this wave's outstanding LDS operations and keep the compiler from
// moving memory accesses across (intra-wave LDS hand-off).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier for LDS hand-offs.  Unlike __syncthreads() it does not
// wait for the wave's outstanding global loads and stores, so prefetches of
// the next chunk stay in flight across it.  (No kernel here reads global
// data that another wave of the same workgroup wrote.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Sum over the 16 lanes of a DPP row: inclusive scan by row_shr 1, 2, 4, 8
// (lanes shifted in from outside the row read 0); lane 15 of each row holds
// the total.  Fixed order, so the result does not vary from run to run.
__device__ __forceinline__ float row_sum16(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));
    return x;
}

// Sum over the lanes l, l ^ 8, l ^ 16, ..., l ^ 56 (the eight lanes with equal
// l % 8), returned in all of them; VALU only.  The rotation by 8 inside a row
// of 16 pairs lane l with l ^ 8.  permlane16_swap(x, x) returns rows
// (x0, x0, x2, x2) and (x1, x1, x3, x3), whose sum pairs each row with its
// neighbour; permlane32_swap does the same for the two halves of the wave.
__device__ __forceinline__ float sum_stride8(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
    const auto h = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
    const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(w[0]) + __uint_as_float(w[1]);
}

// 1/x with v_rcp_f32 (at most 1 ulp off).
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Sum over the 32 lanes of a half wave (lanes 0-31 or 32-63), returned in all
// of them; VALU only.  Rotations by 8, 4, 2, 1 inside each DPP row of 16 leave
// the row's sum in every lane of the row; permlane16_swap then adds each row
// to its neighbour (see sum_stride8).
__device__ __forceinline__ float half_sum32(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));
    const auto h = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}

// Time-mix prologue (w, a, b from the layer's raw projections w_raw, kappa,
// alpha): w = exp(-e^-1/2 sigmoid(w_raw)), a = -kappa / |kappa|,
// b = kappa / |kappa| * sigmoid(alpha), the norm over the head's D channels
// (a zero kappa gives a = b = 0).  e^x is v_exp_f32 (2^x, 1 ulp) of x log2(e).
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kDecayScale = 0.60653065971263342f;   // e^-1/2
__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float logistic_f(float x) { return rcp(1.f + exp_f(-x)); }
__device__ __forceinline__ float proj_decay(float x) { return exp_f(-kDecayScale * logistic_f(x)); }

// One MFMA step: 16x16 tile, accumulator c (fp32).
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS matrix formats and handles.
template <bool SPLIT>
struct Fmt {
    static constexpr int pad = SPLIT ? 8 : 4;
    static constexpr int esz = SPLIT ? 2 : 4;
    static constexpr int planes = SPLIT ? 2 : 1;
    // bytes of a rows x K matrix (multiple of 16)
    static constexpr int bytes(int rows, int K) { return rows * (K + pad) * esz * planes; }
    static constexpr int ld(int K) { return K + pad; }
};

template <bool SPLIT>
struct Mat {
    char* p;    // LDS base
    int ld;     // row stride in elements
    int plane;  // elements per plane (lo plane offset, SPLIT only)
};

template <bool SPLIT>
__device__ __forceinline__ Mat<SPLIT> make_mat(char* smem, int off, int rows, int K) {
    return Mat<SPLIT>{smem + off, Fmt<SPLIT>::ld(K), rows * Fmt<SPLIT>::ld(K)};
}

__device__ __forceinline__ void split1(float v, __bf16& hi, __bf16& lo) {
    hi = (__bf16)v;
    lo = (__bf16)(v - (float)hi);
}

// element (m, k) <- v
__device__ __forceinline__ void put(Mat<true> M, int m, int k, float v) {
    __bf16* h = reinterpret_cast<__bf16*>(M.p) + m * M.ld + k;
    __bf16 hi, lo;
    split1(v, hi, lo);
    h[0] = hi;
    h[M.plane] = lo;
}
__device__ __forceinline__ void put(Mat<false> M, int m, int k, float v) {
    reinterpret_cast<float*>(M.p)[m * M.ld + k] = v;
}
// element (m, k) <- v, v exact in bf16 (hi plane only; lo is never read)
__device__ __forceinline__ void put_exact(Mat<true> M, int m, int k, float v) {
    reinterpret_cast<__bf16*>(M.p)[m * M.ld + k] = (__bf16)v;
}
__device__ __forceinline__ void put_exact(Mat<false> M, int m, int k, float v) { put(M, m, k, v); }

// value of element (m, k) (hi + lo for the split format)
__device__ __forceinline__ float get(Mat<true> M, int m, int k) {
    const __bf16* h = reinterpret_cast<const __bf16*>(M.p) + m * M.ld + k;
    return (float)h[0] + (float)h[M.plane];
}
__device__ __forceinline__ float get(Mat<false> M, int m, int k) {
    return reinterpret_cast<const float*>(M.p)[m * M.ld + k];
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// split of two values with packed conversions: hi = rn(v), lo = rn(v - hi)
__device__ __forceinline__ void split2(f32x2 v, bf16x2& hi, bf16x2& lo) {
    hi = __builtin_convertvector(v, bf16x2);
    const f32x2 back = __builtin_convertvector(hi, f32x2);
    lo = __builtin_convertvector(v - back, bf16x2);
}

// elements (m, k..k+1) <- v0, v1   (k even)
__device__ __forceinline__ void put2(Mat<true> M, int m, int k, float v0, float v1) {
    __bf16* h = reinterpret_cast<__bf16*>(M.p) + m * M.ld + k;
    bf16x2 hi, lo;
    split2(f32x2{v0, v1}, hi, lo);
    *reinterpret_cast<bf16x2*>(h) = hi;
    *reinterpret_cast<bf16x2*>(h + M.plane) = lo;
}
__device__ __forceinline__ void put2(Mat<false> M, int m, int k, float v0, float v1) {
    *reinterpret_cast<float2*>(reinterpret_cast<float*>(M.p) + m * M.ld + k) = make_float2(v0, v1);
}
__device__ __forceinline__ void put2_exact(Mat<true> M, int m, int k, float v0, float v1) {
    bf16x2 hi;
    hi[0] = (__bf16)v0;
    hi[1] = (__bf16)v1;
    *reinterpret_cast<bf16x2*>(reinterpret_cast<__bf16*>(M.p) + m * M.ld + k) = hi;
}
__device__ __forceinline__ void put2_exact(Mat<false> M, int m, int k, float v0, float v1) { put2(M, m, k, v0, v1); }

// elements (m, k..k+3) <- v   (k % 4 == 0)
__device__ __forceinline__ void put4(Mat<true> M, int m, int k, f32x4 v) {
    __bf16* h = reinterpret_cast<__bf16*>(M.p) + m * M.ld + k;
    bf16x2 h0, l0, h1, l1;
    split2(f32x2{v[0], v[1]}, h0, l0);
    split2(f32x2{v[2], v[3]}, h1, l1);
    *reinterpret_cast<bf16x4*>(h) = bf16x4{h0[0], h0[1], h1[0], h1[1]};
    *reinterpret_cast<bf16x4*>(h + M.plane) = bf16x4{l0[0], l0[1], l1[0], l1[1]};
}
__device__ __forceinline__ void put4(Mat<false> M, int m, int k, f32x4 v) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(M.p) + m * M.ld + k) = v;
}
// An accumulator-tile row quad, v = X[m][k0 + 4g .. + 3] of lane (g, r), with
// k8 = k0 + 8 (g / 2).  Lanes g and g ^ 1 (16 lanes apart, same m) swap
// halves with v_permlane16_swap so that the even one stores the hi values and
// the odd one the lo values of the eight columns k8 .. k8 + 7: one 16-byte LDS
// store per lane instead of two 8-byte ones.  (The swap exchanges the odd
// 16-lane rows of its first operand with the even rows of its second.)  Every
// lane of the wave must take part.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void put4_pair(Mat<true> M, int m, int k8, f32x4 v, int g) {
    bf16x2 h0, l0, h1, l1;
    split2(f32x2{v[0], v[1]}, h0, l0);
    split2(f32x2{v[2], v[3]}, h1, l1);
    const auto s0 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, h0), __builtin_bit_cast(unsigned, l0),
                                                     false, false);
    const auto s1 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, h1), __builtin_bit_cast(unsigned, l1),
                                                     false, false);
    __bf16* h = reinterpret_cast<__bf16*>(M.p) + m * M.ld + k8 + ((g & 1) ? M.plane : 0);
    *reinterpret_cast<u32x4_t*>(h) = u32x4_t{s0[0], s1[0], s0[1], s1[1]};
}
__device__ __forceinline__ void put4_pair(Mat<false> M, int m, int k8, f32x4 v, int g) {
    put4(M, m, k8 + 4 * (g & 1), v);
}


// ---------------------------------------------------------------------------
// acc += X[m0:m0+16, 0:K] * Y[n0:n0+16, 0:K]^T   (one wave, one 16x16 tile).
// XEX / YEX: operand exact in bf16 (skip its lo term; SPLIT only).
// Output layout: acc[q] holds element (m0 + 4*(lane/16) + q, n0 + lane%16).
template <bool SPLIT, int K, bool XEX = false, bool YEX = false>
__device__ __forceinline__ f32x4 mma(f32x4 acc, Mat<SPLIT> X, int m0, Mat<SPLIT> Y, int n0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    if constexpr (SPLIT) {
        const __bf16* xp = reinterpret_cast<const __bf16*>(X.p) + (m0 + r) * X.ld + 8 * g;
        const __bf16* yp = reinterpret_cast<const __bf16*>(Y.p) + (n0 + r) * Y.ld + 8 * g;
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += 32) {
            const bf16x8 xh = *reinterpret_cast<const bf16x8*>(xp + k0);
            const bf16x8 yh = *reinterpret_cast<const bf16x8*>(yp + k0);
            acc = mfma_bf16(xh, yh, acc);
            if constexpr (!YEX) {
                const bf16x8 yl = *reinterpret_cast<const bf16x8*>(yp + Y.plane + k0);
                acc = mfma_bf16(xh, yl, acc);
            }
            if constexpr (!XEX) {
                const bf16x8 xl = *reinterpret_cast<const bf16x8*>(xp + X.plane + k0);
                acc = mfma_bf16(xl, yh, acc);
            }
        }
    } else {
        const float* xp = reinterpret_cast<const float*>(X.p) + (m0 + r) * X.ld + g;
        const float* yp = reinterpret_cast<const float*>(Y.p) + (n0 + r) * Y.ld + g;
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += 4)
            acc = mfma_f32(xp[k0], yp[k0], acc);
    }
    return acc;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

enum Mask { MASK_NONE = 0, MASK_LOWER = 1, MASK_STRICT = 2 };

template <int MASK>
__device__ __forceinline__ float masked(float v, int m, int n) {
    if (MASK == MASK_LOWER && m < n) return 0.f;
    if (MASK == MASK_STRICT && m <= n) return 0.f;
    return v;
}

// Tile (m0.., n0..) -> M[m][n]  (row m, k = n)
template <int MASK, bool SPLIT>
__device__ __forceinline__ void store_rows(Mat<SPLIT> M, f32x4 acc, int m0, int n0, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int m = m0 + 4 * g + q, n = n0 + r;
        put(M, m, n, masked<MASK>(acc[q], m, n));
    }
}

// Tile (m0.., n0..) -> M[n][m]  (row n, k = m; four consecutive k per lane)
template <int MASK, bool SPLIT>
__device__ __forceinline__ void store_cols(Mat<SPLIT> M, f32x4 acc, int m0, int n0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    f32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = masked<MASK>(acc[q], m0 + 4 * g + q, n0 + r);
    put4(M, n0 + r, m0 + 4 * g, v);
}

// fp32 tile store, transposed: M[n][m] = element (m, n) (stride ld floats)
template <int MASK>
__device__ __forceinline__ void store_f32_t(float* M, int ld, f32x4 acc, int m0, int n0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    f32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = masked<MASK>(acc[q], m0 + 4 * g + q, n0 + r);
    *reinterpret_cast<f32x4*>(M + (n0 + r) * ld + m0 + 4 * g) = v;
}

// Zero the 16x16 block (m0.., k0..) of a matrix.
template <bool SPLIT>
__device__ __forceinline__ void zero_block(Mat<SPLIT> M, int m0, int k0, int lane) {
    const int m = m0 + (lane >> 2), k = k0 + (lane & 3) * 4;
    put4(M, m, k, zero4());
}

// ---------------------------------------------------------------------------
// Global loads of two consecutive values widened to fp32.
__device__ __forceinline__ float2 load2(const float* p) { return *reinterpret_cast<const float2*>(p); }
__device__ __forceinline__ float2 load2(const uint16_t* p) {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
    return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));  // bf16 -> fp32 exact
}
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t* p) { return __uint_as_float((uint32_t)(*p) << 16); }

// Block -> (outer, inner).  Blocks sharing `outer` (one head) differ in
// `inner` (row block or chunk) and read the same inputs; with xcd = true they
// are placed on one XCD (blocks are dealt to the 8 XCDs round robin), so those
// reads share one L2.  Requires n_outer % 8 == 0.
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
// Two consecutive input values as loaded from global memory (bf16 pair packed
// in one 32-bit word, or an fp32 pair), widened to fp32 only when used, so
// that a prefetch does not wait for its data.
template <typename InT>
struct Pair;
template <>
struct Pair<uint16_t> {
    using T = uint32_t;
    static __device__ __forceinline__ T load(const uint16_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
    static __device__ __forceinline__ float2 f(T u) {
        return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));  // exact
    }
};
template <>
struct Pair<float> {
    using T = float2;
    static __device__ __forceinline__ T load(const float* p) { return *reinterpret_cast<const float2*>(p); }
    static __device__ __forceinline__ float2 f(T v) { return v; }
};

// Raw chunk inputs, prefetched into registers one chunk ahead.  Thread tid
// holds columns 2*jp, 2*jp+1 (jp = tid % 32) of tokens q*TPG .. q*TPG+TPG-1
// (q = tid / 32) for w, a, r, b, k.  Tokens at or beyond `cc` (the chunk's
// length) read the last valid token and are replaced at use: w = 1, the
// rest 0.  With PROJ the w, a, b slots hold the raw projections w_raw, kappa,
// alpha, and fw, fa, fb apply the prologue; finish() must run first (once the
// loads have landed) to form each token's 1 / |kappa| from the 32 lanes that
// share the token.
template <int NT, typename InT, bool PROJ = false>
struct RawChunk {
    static constexpr int NG = NT / 32;
    static constexpr int TPG = C / NG;
    static_assert(NT % 32 == 0 && C % NG == 0 && TPG >= 1, "raw chunk thread shape");
    using W = typename Pair<InT>::T;
    W w[TPG], a[TPG], r[TPG], b[TPG], k[TPG];
    float inv[PROJ ? TPG : 1];   // PROJ: 1 / |kappa| of each token (0 for kappa = 0)
    int cc;

    __device__ __forceinline__ void load(const InT* pw, const InT* pa, const InT* pr, const InT* pb,
                                         const InT* pk, int64_t base, int64_t tstride, int Cc, int tid) {
        const int jp = tid & 31, q = tid >> 5;
        cc = Cc;
#pragma unroll
        for (int tt = 0; tt < TPG; ++tt) {
            const int t = min(q * TPG + tt, Cc - 1);
            const int64_t o = base + t * tstride + 2 * jp;
            w[tt] = Pair<InT>::load(pw + o);
            a[tt] = Pair<InT>::load(pa + o);
            r[tt] = Pair<InT>::load(pr + o);
            b[tt] = Pair<InT>::load(pb + o);
            k[tt] = Pair<InT>::load(pk + o);
        }
    }
    __device__ __forceinline__ bool valid(int tt, int tid) const { return (tid >> 5) * TPG + tt < cc; }
    __device__ __forceinline__ float2 get(const W& x, int tt, int tid, float fill) const {
        return valid(tt, tid) ? Pair<InT>::f(x) : make_float2(fill, fill);
    }
    __device__ __forceinline__ void finish() {
        if constexpr (PROJ) {
#pragma unroll
            for (int tt = 0; tt < TPG; ++tt) {
                const float2 kv = Pair<InT>::f(a[tt]);
                const float ss = half_sum32(kv.x * kv.x + kv.y * kv.y);
                inv[tt] = ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f;
            }
        }
    }
    __device__ __forceinline__ float2 fw(int tt, int tid) const {
        if constexpr (PROJ) {
            const float2 x = Pair<InT>::f(w[tt]);
            return valid(tt, tid) ? make_float2(proj_decay(x.x), proj_decay(x.y)) : make_float2(1.f, 1.f);
        } else {
            return get(w[tt], tt, tid, 1.f);
        }
    }
    // kappa / |kappa| (PROJ only)
    __device__ __forceinline__ float2 kappa_hat(int tt) const {
        const float2 x = Pair<InT>::f(a[tt]);
        return make_float2(x.x * inv[tt], x.y * inv[tt]);
    }
    __device__ __forceinline__ float2 fa(int tt, int tid) const {
        if constexpr (PROJ) {
            const float2 kh = kappa_hat(tt);
            return valid(tt, tid) ? make_float2(-kh.x, -kh.y) : make_float2(0.f, 0.f);
        } else {
            return get(a[tt], tt, tid, 0.f);
        }
    }
    __device__ __forceinline__ float2 fb(int tt, int tid) const {
        if constexpr (PROJ) {
            const float2 kh = kappa_hat(tt), al = Pair<InT>::f(b[tt]);
            return valid(tt, tid) ? make_float2(kh.x * logistic_f(al.x), kh.y * logistic_f(al.y))
                                  : make_float2(0.f, 0.f);
        } else {
            return get(b[tt], tt, tid, 0.f);
        }
    }
    __device__ __forceinline__ float2 fr(int tt, int tid) const { return get(r[tt], tt, tid, 0.f); }
    __device__ __forceinline__ float2 fk(int tt, int tid) const { return get(k[tt], tt, tid, 0.f); }
};

// Where chunk_prep writes.  Null handles are skipped.
template <bool SPLIT>
struct PrepOut {
    Mat<SPLIT> A, R, B, K;        // rows (t, j)
    Mat<SPLIT> AT, RT, BT, KT;    // transposed (j, t)
    bool a, r, b, k, at, rt, bt, kt;
    float* gamma;                 // fp32 [t][j] (stride 68) or null
    float* glast;                 // fp32 [64]
};
constexpr int LDG = 68;           // row stride of the fp32 gamma array

// Chunk preparation from the registers of RawChunk: gamma (cumulative product
// of w within the chunk), the scaled operands, gamma_last.  `qp` is LDS
// scratch of NG x 64 floats.  Contains two barriers; the caller must barrier
// before the outputs are read.  With PROJ, raw.finish() must have run.
template <int NT, bool SPLIT, typename InT, bool PROJ>
__device__ __forceinline__ void chunk_prep(const RawChunk<NT, InT, PROJ>& raw, const PrepOut<SPLIT>& o, float* qp,
                                           int tid) {
    constexpr int NG = RawChunk<NT, InT, PROJ>::NG, TPG = RawChunk<NT, InT, PROJ>::TPG;
    const int jp = tid & 31, q = tid >> 5, j0 = 2 * jp;
    float2 loc[TPG];
    float2 p = make_float2(1.f, 1.f);
#pragma unroll
    for (int tt = 0; tt < TPG; ++tt) {
        const float2 wv = raw.fw(tt, tid);
        p.x *= wv.x;
        p.y *= wv.y;
        loc[tt] = p;
    }
    qp[q * 64 + j0] = p.x;
    qp[q * 64 + j0 + 1] = p.y;
    lds_barrier();
    // wave 0, lane = column: the products over earlier groups, in place (and gamma_last)
    if (tid < 64) {
        float qv[NG];   // all reads first, then the products, then the writes
#pragma unroll
        for (int q2 = 0; q2 < NG; ++q2) qv[q2] = qp[q2 * 64 + tid];
        float run = 1.f;
#pragma unroll
        for (int q2 = 0; q2 < NG; ++q2) {
            const float v = qv[q2];
            qv[q2] = run;
            run *= v;
        }
#pragma unroll
        for (int q2 = 0; q2 < NG; ++q2) qp[q2 * 64 + tid] = qv[q2];
        o.glast[tid] = run;
    }
    lds_barrier();
    const float2 pre = *reinterpret_cast<const float2*>(qp + q * 64 + j0);
    float2 gprev = pre;
    float gt[2][TPG], at[2][TPG], rt[2][TPG], bt[2][TPG], kt[2][TPG];
#pragma unroll
    for (int tt = 0; tt < TPG; ++tt) {
        const int t = q * TPG + tt;
        const float2 g = (q == 0) ? loc[tt] : make_float2(pre.x * loc[tt].x, pre.y * loc[tt].y);
        const float ix = rcp(g.x), iy = rcp(g.y);
        const float2 av = raw.fa(tt, tid), rv = raw.fr(tt, tid);
        const float2 bv = raw.fb(tt, tid), kv = raw.fk(tt, tid);
        const float ax = av.x * gprev.x, ay = av.y * gprev.y;
        const float rx = rv.x * g.x, ry = rv.y * g.y;
        const float bx = bv.x * ix, by = bv.y * iy;
        const float kx = kv.x * ix, ky = kv.y * iy;
        if (o.a) put2(o.A, t, j0, ax, ay);
        if (o.r) put2(o.R, t, j0, rx, ry);
        if (o.b) put2(o.B, t, j0, bx, by);
        if (o.k) put2(o.K, t, j0, kx, ky);
        if (o.gamma) *reinterpret_cast<float2*>(o.gamma + t * LDG + j0) = g;
        gt[0][tt] = g.x; gt[1][tt] = g.y;
        at[0][tt] = ax; at[1][tt] = ay;
        rt[0][tt] = rx; rt[1][tt] = ry;
        bt[0][tt] = bx; bt[1][tt] = by;
        kt[0][tt] = kx; kt[1][tt] = ky;
        gprev = g;
    }
    // transposed copies: TPG consecutive tokens of one column per thread
    const int t0 = q * TPG;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
#pragma unroll
        for (int tt = 0; tt < TPG; tt += (TPG >= 4 ? 4 : TPG)) {
            if constexpr (TPG >= 4) {
                if (o.at) put4(o.AT, j0 + e, t0 + tt, f32x4{at[e][tt], at[e][tt + 1], at[e][tt + 2], at[e][tt + 3]});
                if (o.rt) put4(o.RT, j0 + e, t0 + tt, f32x4{rt[e][tt], rt[e][tt + 1], rt[e][tt + 2], rt[e][tt + 3]});
                if (o.bt) put4(o.BT, j0 + e, t0 + tt, f32x4{bt[e][tt], bt[e][tt + 1], bt[e][tt + 2], bt[e][tt + 3]});
                if (o.kt) put4(o.KT, j0 + e, t0 + tt, f32x4{kt[e][tt], kt[e][tt + 1], kt[e][tt + 2], kt[e][tt + 3]});
            } else {
#pragma unroll
                for (int u = 0; u < TPG; ++u) {
                    if (o.at) put(o.AT, j0 + e, t0 + u, at[e][u]);
                    if (o.rt) put(o.RT, j0 + e, t0 + u, rt[e][u]);
                    if (o.bt) put(o.BT, j0 + e, t0 + u, bt[e][u]);
                    if (o.kt) put(o.KT, j0 + e, t0 + u, kt[e][u]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Column block [col0, col0+NCOL) of one chunk of a (B,T,H,D) tensor, held in
// registers: thread tid holds the pair of columns col0 + 2*(tid % (NCOL/2))
// (+0, +1) for tokens tid / (NCOL/2) + s*(NT / (NCOL/2)), s = 0..PER-1.
template <int NT, int NCOL, typename InT>
struct RawCols {
    static constexpr int PAIRS = NCOL / 2;
    static constexpr int TSTEP = NT / PAIRS;          // tokens covered per sweep
    static constexpr int PER = (C + TSTEP - 1) / TSTEP;
    static_assert(NT % PAIRS == 0, "raw column thread shape");
    using W = typename Pair<InT>::T;
    W v[PER];
    int cc;

    __device__ __forceinline__ void load(const InT* src, int64_t base, int64_t tstride, int Cc, int col0, int tid) {
        const int ip = tid % PAIRS, t1 = tid / PAIRS;
        cc = Cc;
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int t = min(t1 + s * TSTEP, Cc - 1);
            v[s] = Pair<InT>::load(src + base + t * tstride + col0 + 2 * ip);
        }
    }
    __device__ __forceinline__ float2 value(int s, int tid) const {
        const int t = tid / PAIRS + s * TSTEP;
        return t < cc ? Pair<InT>::f(v[s]) : make_float2(0.f, 0.f);
    }
    // M[i][t] = value (transposed: row = column index i, k = token)
    template <bool SPLIT, bool EXACT>
    __device__ __forceinline__ void store_T(Mat<SPLIT> M, int tid) const {
        const int ip = tid % PAIRS, t1 = tid / PAIRS;
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int t = t1 + s * TSTEP;
            if (t < C) {
                const float2 x = value(s, tid);
                if (EXACT) {
                    put_exact(M, 2 * ip, t, x.x);
                    put_exact(M, 2 * ip + 1, t, x.y);
                } else {
                    put(M, 2 * ip, t, x.x);
                    put(M, 2 * ip + 1, t, x.y);
                }
            }
        }
    }
    // M[t][i] = value (rows: row = token, k = column index)
    template <bool SPLIT, bool EXACT>
    __device__ __forceinline__ void store_rows(Mat<SPLIT> M, int tid) const {
        const int ip = tid % PAIRS, t1 = tid / PAIRS;
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int t = t1 + s * TSTEP;
            if (t < C) {
                const float2 x = value(s, tid);
                if (EXACT) put2_exact(M, t, 2 * ip, x.x, x.y);
                else put2(M, t, 2 * ip, x.x, x.y);
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Store the three lower tiles of a C x C matrix as rows and/or transposed,
// zeroing the upper-right tile.
template <int MASK, bool SPLIT>
__device__ __forceinline__ void cc_store(Mat<SPLIT> Mr, bool rows_, Mat<SPLIT> Mt, bool trans, f32x4 t00,
                                         f32x4 t10, f32x4 t11, int lane) {
    if (rows_) {
        store_rows<MASK>(Mr, t00, 0, 0, lane);
        store_rows<MASK>(Mr, t10, 16, 0, lane);
        store_rows<MASK>(Mr, t11, 16, 16, lane);
        zero_block(Mr, 0, 16, lane);
    }
    if (trans) {
        store_cols<MASK>(Mt, t00, 0, 0, lane);
        store_cols<MASK>(Mt, t10, 16, 0, lane);
        store_cols<MASK>(Mt, t11, 16, 16, lane);
        zero_block(Mt, 16, 0, lane);
    }
}

// ---------------------------------------------------------------------------
// T = (I - L)^-1 for the strictly lower C x C matrix L, given transposed
// (LT[s][t] = L[t][s], fp32, stride LDF), by 16 x 16 blocks: T11 = (I - L11)^-1
// and T22 = (I - L22)^-1 by forward substitution (lanes 0..15 and 16..31, one
// column each), then T21 = T22 (L21 T11) with two fp32 MFMA products.  One
// wave.  `tf` (fp32, stride LDF) receives T except its zero block (rows 0-15,
// columns 16-31), which the caller writes; `scr` is 16 x 20 floats of scratch.
__device__ __forceinline__ void tri_inverse(const float* LT, float* tf, float* scr, int lane) {
    if (lane < 32) {
        const int k = lane & 15, base = lane & 16;
        // right-looking: once x[s] is final, every later row t takes L[t][s] x[s]; column s of
        // L is row s of LT, read in 16-byte pieces (the updates of one step are independent)
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) x[t] = (t == k) ? 1.f : 0.f;
        // The pieces do not depend on x: each third of the steps has all of its reads issued
        // before its first product (the scheduling barriers keep them there), so the reads'
        // latency is paid three times instead of once per step.
        auto part = [&](auto s_lo, auto s_hi) {
            constexpr int S0 = decltype(s_lo)::value, S1 = decltype(s_hi)::value;
            constexpr int NP = [] {
                int n = 0;
                for (int s = S0; s < S1; ++s) n += 4 - ((s + 1) >> 2);
                return n;
            }();
            f32x4 piece[NP];
            int n = 0;
#pragma unroll
            for (int s = S0; s < S1; ++s) {
#pragma unroll
                for (int q0 = ((s + 1) >> 2) << 2; q0 < 16; q0 += 4)
                    piece[n++] = *reinterpret_cast<const f32x4*>(LT + (base + s) * LDF + base + q0);
            }
            __builtin_amdgcn_sched_barrier(0);
            n = 0;
#pragma unroll
            for (int s = S0; s < S1; ++s) {
#pragma unroll
                for (int q0 = ((s + 1) >> 2) << 2; q0 < 16; q0 += 4) {
                    const f32x4 l = piece[n++];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (q0 + e > s) x[q0 + e] = fmaf(l[e], x[s], x[q0 + e]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        part(std::integral_constant<int, 0>{}, std::integral_constant<int, 5>{});
        part(std::integral_constant<int, 5>{}, std::integral_constant<int, 10>{});
        part(std::integral_constant<int, 10>{}, std::integral_constant<int, 15>{});
#pragma unroll
        for (int t = 0; t < 16; ++t) tf[(base + t) * LDF + base + k] = x[t];
    }
    wave_lds_sync();
    // P = L21 T11  (row t-16, column n); L21[r][c] = LT[c][16 + r]
    const int r = lane & 15, g = lane >> 4;
    f32x4 acc = zero4();
#pragma unroll
    for (int k0 = 0; k0 < 16; k0 += 4)
        acc = mfma_f32(LT[(k0 + g) * LDF + 16 + r], tf[(k0 + g) * LDF + r], acc);
#pragma unroll
    for (int q = 0; q < 4; ++q) scr[(4 * g + q) * 20 + r] = acc[q];
    wave_lds_sync();
    // T21 = T22 P
    acc = zero4();
#pragma unroll
    for (int k0 = 0; k0 < 16; k0 += 4)
        acc = mfma_f32(tf[(16 + r) * LDF + 16 + k0 + g], scr[(k0 + g) * 20 + r], acc);
#pragma unroll
    for (int q = 0; q < 4; ++q) tf[(16 + 4 * g + q) * LDF + r] = acc[q];
    wave_lds_sync();
}


// ---------------------------------------------------------------------------
// Buffer resources: a base address and a size in bytes.  Loads at or past the
// size return 0 and stores there are dropped by the hardware, so a ragged
// tail needs no branch (and a wave's counts of outstanding memory operations
// stay exact).  A size of 0 turns every access off.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
//
// The whole byte offset goes into the per-lane offset and the scalar offset
// stays the constant 0: the range check covers the per-lane offset, and a
// 128-bit store with a constant scalar offset is the form for which the
// compiler keeps the store's data registers untouched for the wait state the
// hardware needs before they are overwritten.  (Stores with a register
// scalar offset lost the last dword of the data to the next instruction's
// write of that register.)
//
// CP selects the cache policy: kCached for data the next kernel reads back
// (checkpoints, state gradients), kStream (non-temporal) for outputs that
// leave the library, kStreamDev (non-temporal, device scope) for outputs
// whose stores cover a cache line in pieces from several instructions: the
// gradient kernel's tiles write 64-byte row pieces, which with kStream alone
// cost 1.28x their bytes in HBM writes and with kStreamDev exactly their bytes.
constexpr int kCached = 0, kStream = 2, kStreamDev = 18;
template <int CP = kCached>
__device__ __forceinline__ void bstore(float v, Rsrc r, int voff, int soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff + soff, 0, CP);
}
template <int CP = kCached>
__device__ __forceinline__ void bstore2(float2 v, Rsrc r, int voff, int soff) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, voff + soff, 0, CP);
}
template <int CP = kCached>
__device__ __forceinline__ void bstore4(f32x4 v, Rsrc r, int voff, int soff) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff + soff, 0, CP);
}

// ---------------------------------------------------------------------------
// Fragments with a permuted k order (used by the chunk-operand kernels).
//
// A 32-wide block of the contraction index, [c0, c0 + 32), is dealt to the
// lanes of a 16 x 16 MFMA tile so that lane (g = lane / 16, r = lane % 16)
// holds the eight k values  c0 + 16h + 4g + q  (h = 0, 1; q = 0..3).  Both
// operands of a product use the same order, so the sum over k is unchanged.
// The point of this order: the accumulator of a 16 x 16 tile holds
// acc[q] = X[m0 + 4g + q][n0 + r], which is exactly such a fragment of the
// row n0 + r of X^T for k = m0 + 4g + q -- a result can be fed back as an
// operand without leaving the registers.
//   SPLIT = true : element e = 4h + q of bf16x8 hi / lo (value = hi + lo)
//   SPLIT = false: v[h][q] (fp32), consumed by four 16x16x4 steps per h
template <bool SPLIT>
struct Frag;
template <>
struct Frag<true> {
    bf16x8 hi, lo;
};
template <>
struct Frag<false> {
    f32x4 v[2];
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ bf16x4 as_bf16x4(i16x4 v) { return __builtin_bit_cast(bf16x4, v); }

// Fragment of two accumulator tiles: h = 0 from a0, h = 1 from a1.
template <bool SPLIT>
__device__ __forceinline__ Frag<SPLIT> frag_acc(f32x4 a0, f32x4 a1) {
    Frag<SPLIT> f;
    if constexpr (SPLIT) {
        bf16x2 h0, l0, h1, l1, h2, l2, h3, l3;
        split2(f32x2{a0[0], a0[1]}, h0, l0);
        split2(f32x2{a0[2], a0[3]}, h1, l1);
        split2(f32x2{a1[0], a1[1]}, h2, l2);
        split2(f32x2{a1[2], a1[3]}, h3, l3);
        f.hi = bf16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
        f.lo = bf16x8{l0[0], l0[1], l1[0], l1[1], l2[0], l2[1], l3[0], l3[1]};
    } else {
        f.v[0] = a0;
        f.v[1] = a1;
    }
    return f;
}

// Rows of an fp32 LDS matrix (row stride ld floats) as an operand fragment,
// split in registers for the bf16 format: lane (g, r) gets
// X[row0 + r][c0 + 16h + 4g + q] (the order of frag_n).
template <bool SPLIT>
__device__ __forceinline__ Frag<SPLIT> frag_n_f32(const float* X, int ld, int row0, int c0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const float* p = X + (row0 + r) * ld + c0 + 4 * g;
    return frag_acc<SPLIT>(*reinterpret_cast<const f32x4*>(p), *reinterpret_cast<const f32x4*>(p + 16));
}

// Fragment of values exact in bf16 (SPLIT: the lo part is never read).
template <bool SPLIT>
__device__ __forceinline__ Frag<SPLIT> frag_exact(f32x4 a0, f32x4 a1) {
    if constexpr (SPLIT) {
        Frag<SPLIT> f;
        const bf16x4 x0 = __builtin_convertvector(a0, bf16x4), x1 = __builtin_convertvector(a1, bf16x4);
        f.hi = cat8(x0, x1);
        f.lo = f.hi;
        return f;
    } else {
        return frag_acc<false>(a0, a1);
    }
}

// Rows: lane (g, r) gets X[row0 + r][c0 + 16h + 4g + q].
__device__ __forceinline__ Frag<true> frag_n(Mat<true> X, int row0, int c0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const __bf16* p = reinterpret_cast<const __bf16*>(X.p) + (row0 + r) * X.ld + c0 + 4 * g;
    Frag<true> f;
    f.hi = cat8(*reinterpret_cast<const bf16x4*>(p), *reinterpret_cast<const bf16x4*>(p + 16));
    f.lo = cat8(*reinterpret_cast<const bf16x4*>(p + X.plane), *reinterpret_cast<const bf16x4*>(p + X.plane + 16));
    return f;
}
__device__ __forceinline__ Frag<false> frag_n(Mat<false> X, int row0, int c0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const float* p = reinterpret_cast<const float*>(X.p) + (row0 + r) * X.ld + c0 + 4 * g;
    Frag<false> f;
    f.v[0] = *reinterpret_cast<const f32x4*>(p);
    f.v[1] = *reinterpret_cast<const f32x4*>(p + 16);
    return f;
}

// Columns: lane (g, r) gets X[c0 + 16h + 4g + q][col0 + r].  For the split
// format this is the LDS transpose read (ds_read_b64_tr_b16): within each
// group of 16 lanes, lane 4i + e receives element e of the 8-byte reads of
// lanes i, i + 4, i + 8, i + 12; so lane s reads X[c0 + 4g + (s%16)/4]
// [col0 + 4(s%4) .. +3].
__device__ __forceinline__ Frag<true> frag_t(Mat<true> X, int col0, int c0, int lane) {
    const int g = lane >> 4, l16 = lane & 15;
    const __bf16* p = reinterpret_cast<const __bf16*>(X.p) + (c0 + 4 * g + (l16 >> 2)) * X.ld + col0 + 4 * (l16 & 3);
    const __bf16* p1 = p + 16 * X.ld;
    Frag<true> f;
    f.hi = cat8(as_bf16x4(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p))),
                as_bf16x4(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1))));
    f.lo = cat8(as_bf16x4(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + X.plane))),
                as_bf16x4(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1 + X.plane))));
    return f;
}
__device__ __forceinline__ Frag<false> frag_t(Mat<false> X, int col0, int c0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const float* p = reinterpret_cast<const float*>(X.p) + (c0 + 4 * g) * X.ld + col0 + r;
    Frag<false> f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q) f.v[h][q] = p[(16 * h + q) * X.ld];
    return f;
}

// LDS transpose read of exact bf16 values (hi plane only), see frag_t.
__device__ __forceinline__ Frag<true> frag_t_exact(Mat<true> X, int col0, int c0, int lane) {
    const int g = lane >> 4, l16 = lane & 15;
    const __bf16* p = reinterpret_cast<const __bf16*>(X.p) + (c0 + 4 * g + (l16 >> 2)) * X.ld + col0 + 4 * (l16 & 3);
    Frag<true> f;
    f.hi = cat8(as_bf16x4(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p))),
                as_bf16x4(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 16 * X.ld))));
    f.lo = f.hi;
    return f;
}
__device__ __forceinline__ Frag<false> frag_t_exact(Mat<false> X, int col0, int c0, int lane) {
    return frag_t(X, col0, c0, lane);
}

// acc += X Y^T over one 32-wide k block.  XEX / YEX: operand exact in bf16.
template <bool XEX = false, bool YEX = false>
__device__ __forceinline__ f32x4 fmma(f32x4 acc, const Frag<true>& x, const Frag<true>& y) {
    acc = mfma_bf16(x.hi, y.hi, acc);
    if constexpr (!YEX) acc = mfma_bf16(x.hi, y.lo, acc);
    if constexpr (!XEX) acc = mfma_bf16(x.lo, y.hi, acc);
    return acc;
}
template <bool XEX = false, bool YEX = false>
__device__ __forceinline__ f32x4 fmma(f32x4 acc, const Frag<false>& x, const Frag<false>& y) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = mfma_f32(x.v[h][q], y.v[h][q], acc);
    return acc;
}

// Elements (m, k..k+3) of an LDS operand as fp32 (hi + lo for the split format).
__device__ __forceinline__ f32x4 get4(Mat<true> M, int m, int k) {
    const __bf16* h = reinterpret_cast<const __bf16*>(M.p) + m * M.ld + k;
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(h), lo = *reinterpret_cast<const bf16x4*>(h + M.plane);
    return __builtin_convertvector(hi, f32x4) + __builtin_convertvector(lo, f32x4);
}
__device__ __forceinline__ f32x4 get4(Mat<false> M, int m, int k) {
    return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(M.p) + m * M.ld + k);
}

// Four consecutive values into a global operand block: the split format keeps
// a hi plane and, `plane` elements further, a lo plane.
__device__ __forceinline__ void gput4(__bf16* X, int64_t plane, int64_t idx, f32x4 v) {
    bf16x2 h0, l0, h1, l1;
    split2(f32x2{v[0], v[1]}, h0, l0);
    split2(f32x2{v[2], v[3]}, h1, l1);
    *reinterpret_cast<bf16x4*>(X + idx) = bf16x4{h0[0], h0[1], h1[0], h1[1]};
    *reinterpret_cast<bf16x4*>(X + plane + idx) = bf16x4{l0[0], l0[1], l1[0], l1[1]};
}
__device__ __forceinline__ void gput4(float* X, int64_t, int64_t idx, f32x4 v) {
    *reinterpret_cast<f32x4*>(X + idx) = v;
}

// Accumulator tile (lane (g, r) holds row r, columns 4g .. 4g + 3) stored as
// tile `tile` of a plane-major sequence of row-major 16 x 16 tiles: the wave's
// stores fill one contiguous 512-byte (bf16) or 1 KiB (fp32) block per plane.
template <typename X>
__device__ __forceinline__ void tput4(X* base, int64_t plane, int tile, int lane, f32x4 v) {
    gput4(base, plane, (int64_t)tile * 256 + (lane & 15) * 16 + 4 * (lane >> 4), v);
}

}  // namespace wkv7
