// wkv7_seq.hip -- token-by-token WKV7 forward on the vector units (gfx950).
//
// The per-token update exactly as the rwkv-mlx page states it ("Metal kernel
// architecture", forward block): sa = S a, S = S diag(w) + v k^T + sa b^T,
// y = S r.  One workgroup per head; thread (i = tid/4, part = tid%4) keeps
// the 16 state values S[i][16*part .. 16*part+15] in registers, so the row
// dot products need a 4-lane reduction only.  This is the streaming path
// for very short sequences -- above all the one-token recurrent step, where
// the state is read from and written back to HBM once (in place if
// hT == h0) and the kernel is bound by HBM bandwidth.
#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

constexpr int SEQ_NT = 256;

template <typename InT>
__device__ __forceinline__ float load1(const InT* p);
template <>
__device__ __forceinline__ float load1<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t* p) {
    return __uint_as_float((uint32_t)(*p) << 16);
}

template <typename InT>
__global__ __launch_bounds__(SEQ_NT) void fwd_sequential_kernel(FwdArgs p) {
    __shared__ float vec[6][D];  // w, k, a, b, r, v of the current token
    const int tid = threadIdx.x;
    const int i = tid >> 2, part = tid & 3, j0 = part * 16;
    const int head = blockIdx.x;
    const int bb = head / p.H, hh = head % p.H;
    const int64_t tstride = (int64_t)p.H * D;
    const int64_t soff = (int64_t)head * D * D + (int64_t)i * D + j0;

    float s[16];
    if (p.h0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = *reinterpret_cast<const float4*>(p.h0 + soff + 4 * q);
            s[4 * q] = v.x; s[4 * q + 1] = v.y; s[4 * q + 2] = v.z; s[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) s[q] = 0.f;
    }

    const InT* srcs[6] = {static_cast<const InT*>(p.w), static_cast<const InT*>(p.k),
                          static_cast<const InT*>(p.a), static_cast<const InT*>(p.b),
                          static_cast<const InT*>(p.r), static_cast<const InT*>(p.v)};

    for (int t = 0; t < p.T; ++t) {
        const int64_t base = ((int64_t)bb * p.T + t) * tstride + (int64_t)hh * D;
        if (p.ckpt && (t % C) == 0) {
            float* dst = p.ckpt + ((int64_t)head * p.NC + t / C) * D * D + (int64_t)i * D + j0;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<float4*>(dst + 4 * q) = make_float4(s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]);
        }
        __syncthreads();  // previous token's reads of vec are done
        for (int e = tid; e < 6 * D; e += SEQ_NT) vec[e / D][e % D] = load1<InT>(srcs[e / D] + base + (e % D));
        __syncthreads();

        float sa = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) sa = fmaf(s[q], vec[2][j0 + q], sa);
        sa += __shfl_xor(sa, 1);
        sa += __shfl_xor(sa, 2);
        const float vi = vec[5][i];
        float y = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int j = j0 + q;
            s[q] = fmaf(vec[0][j], s[q], fmaf(vi, vec[1][j], sa * vec[3][j]));
            y = fmaf(s[q], vec[4][j], y);
        }
        y += __shfl_xor(y, 1);
        y += __shfl_xor(y, 2);
        if (p.y && part == 0) p.y[base + i] = y;
    }
    if (p.hT) {
        float* dst = p.hT + soff;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(dst + 4 * q) = make_float4(s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]);
    }
}

// Sum over the 16 lanes of a DPP row, the same value in every lane: a butterfly
// of lane pairs l ^ 1, l ^ 2 (quad permutes), l ^ 7 (half-row mirror) and
// l ^ 15 (row mirror); each step adds a pair in both lanes, so the lanes agree.
__device__ __forceinline__ float row16_allsum(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false));   // quad_perm 2,3,0,1
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false));  // row_half_mirror
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xf, 0xf, false));  // row_mirror
    return x;
}

template <typename InT>
__device__ __forceinline__ f32x4 load4(const InT* p);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
template <>
__device__ __forceinline__ f32x4 load4<uint16_t>(const uint16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                 __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
}

// One token (T = 1), the recurrent step: the same update as above, with the
// state accessed as one contiguous 16 KiB block per head.  Thread tid holds
// rows 4 (tid / 16) + q, q = 0..3, columns 4 (tid % 16) .. + 3: each access of
// a wave covers four whole 256-byte rows, and a thread's four rows are
// consecutive, so their v values arrive in one load and their y values leave
// in one store.  The 16 threads of a row are one DPP row, so the row dot
// products need no LDS.
// PROJ: the w, a, b pointers hold the raw projections w_raw, kappa, alpha and
// the time-mix prologue runs on the loaded values (the 16 lanes of a DPP row
// hold one token's 64 channels, so |kappa| is a row sum).
template <typename InT, bool PROJ>
__global__ __launch_bounds__(SEQ_NT) void step_kernel(FwdArgs p) {
    const int tid = threadIdx.x;
    const int head = blockIdx.x;
    const int bb = head / p.H, hh = head % p.H;
    const int64_t base = ((int64_t)bb * p.H + hh) * D;      // this head's token row (T = 1)
    const int c0 = 4 * (tid & 15), r0 = 4 * (tid >> 4);
    const int64_t hoff = (int64_t)head * D * D + r0 * D + c0;
    f32x4 st[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)   // streamed once: non-temporal
        st[q] = p.h0 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p.h0 + hoff + D * q)) : zero4();
    if (p.ckpt) {   // checkpoint 0: the state entering the (only) chunk
#pragma unroll
        for (int q = 0; q < 4; ++q) *reinterpret_cast<f32x4*>(p.ckpt + hoff + D * q) = st[q];
    }
    f32x4 w = load4(static_cast<const InT*>(p.w) + base + c0);
    const f32x4 k = load4(static_cast<const InT*>(p.k) + base + c0);
    f32x4 a = load4(static_cast<const InT*>(p.a) + base + c0), b = load4(static_cast<const InT*>(p.b) + base + c0);
    if constexpr (PROJ) {
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) ss = fmaf(a[c], a[c], ss);
        ss = row16_allsum(ss);
        const float inv = ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float kh = a[c] * inv;
            w[c] = proj_decay(w[c]);
            a[c] = -kh;
            b[c] = kh * logistic_f(b[c]);
        }
    }
    const f32x4 r = load4(static_cast<const InT*>(p.r) + base + c0);
    const f32x4 vr = load4(static_cast<const InT*>(p.v) + base + r0);   // v of rows r0 .. r0 + 3
    f32x4 yr;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float vi = vr[q];
        float sa = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) sa = fmaf(st[q][c], a[c], sa);
        sa = row16_allsum(sa);
        float y = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            st[q][c] = fmaf(w[c], st[q][c], fmaf(vi, k[c], sa * b[c]));
            y = fmaf(st[q][c], r[c], y);
        }
        yr[q] = row16_allsum(y);
    }
    if (p.y && (tid & 15) == 0) *reinterpret_cast<f32x4*>(p.y + base + r0) = yr;
    if (p.hT) {
#pragma unroll
        for (int q = 0; q < 4; ++q) __builtin_nontemporal_store(st[q], reinterpret_cast<f32x4*>(p.hT + hoff + D * q));
    }
}

}  // namespace

hipError_t launch_fwd_sequential(const FwdArgs& a, bool bf16, bool proj, hipStream_t s) {
    const int heads = a.B * a.H;
    if (a.T == 1) {   // the recurrent step: coalesced state access
        if (proj) {
            if (bf16) hipLaunchKernelGGL((step_kernel<uint16_t, true>), dim3(heads), dim3(SEQ_NT), 0, s, a);
            else hipLaunchKernelGGL((step_kernel<float, true>), dim3(heads), dim3(SEQ_NT), 0, s, a);
        } else {
            if (bf16) hipLaunchKernelGGL((step_kernel<uint16_t, false>), dim3(heads), dim3(SEQ_NT), 0, s, a);
            else hipLaunchKernelGGL((step_kernel<float, false>), dim3(heads), dim3(SEQ_NT), 0, s, a);
        }
        return hipGetLastError();
    }
    if (proj) return hipErrorInvalidValue;   // the prologue runs in the step and the chunked kernels only
    if (bf16) hipLaunchKernelGGL(fwd_sequential_kernel<uint16_t>, dim3(heads), dim3(SEQ_NT), 0, s, a);
    else hipLaunchKernelGGL(fwd_sequential_kernel<float>, dim3(heads), dim3(SEQ_NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace wkv7
