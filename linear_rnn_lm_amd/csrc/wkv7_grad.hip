// wkv7_grad.hip -- per-token input gradients of the WKV7 backward (gfx950).
//
// Reverse-mode of the per-token update (rwkv-mlx page, "Metal kernel
// architecture", backward block: chunks in reverse, from checkpoints).  With
// X_t = dL/dS_t (all later uses of S_t, including y_t) the gradient state
// obeys X_{t-1} = X_t (diag w_t + b_t a_t^T) + dy_{t-1} r_{t-1}^T.  The scan
// kernel (wkv7_scan.hip) walks that recurrence over the chunks and leaves the
// gradient w.r.t. the state entering every chunk in dh_ckpt.  This kernel
// takes it from there, one workgroup per (head, chunk), all chunks at once.
// With the chunk matrices of wkv7_device.h, Ge' = Ge diag(gamma_last) for the
// gradient Ge at the chunk's end and T = (I - Lab)^-1 (from the prepare
// kernel), it recomputes from the checkpoint S0 -- never by dividing the
// state by w --
//     U   = T (Ahat S0^T + Lak V)                       u_t   = S_{t-1} a_t
//     DSA = T^T (Btil Ge'^T + Mrb^T DY)                 dsa_t = X_t b_t
// and then, with P1 = tril(DY U^T), P2 = tril(DY V^T), P3 = stril(DSA U^T),
// P4 = stril(DSA V^T),
//     dr = Gamma    * (DY S0  + P1 Btil   + P2 Ktil)
//     da = Gamma_-1 * (DSA S0 + P3 Btil   + P4 Ktil)
//     dk = Gamma^-1 * (V Ge'  + P4^T Ahat + P2^T Rhat)
//     db = Gamma^-1 * (U Ge'  + P3^T Ahat + P1^T Rhat)
// and dw from an identity that follows from the update rule: with
// phi_t = w_t * dw_t and Gs = dL/dS0,
//     phi_t = sum_i Gs[i][j] S0[i][j] - sum_{s<=t} a_s da_s
//             + sum_{s<t} (k_s dk_s + b_s db_s - r_s dr_s),
//     dw_t  = phi_t / w_t.
// Every operand is staged once, in rows; products that need the other
// orientation read it with the LDS transpose (frag_t).  The outputs are
// computed transposed, (j, t), so that each lane stores four consecutive j.
#include <type_traits>

#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

constexpr int GNT = 512;  // threads per workgroup (8 waves)
constexpr int GNW = GNT / 64;

// LDS plan (byte offsets).  Region Q holds T, Lak, Mrb until U and DSA exist,
// then P1..P4 and the dw ingredients.
template <bool SPLIT>
struct GradSmem {
    using F = Fmt<SPLIT>;
    static constexpr int RM = F::bytes(C, D), SM = F::bytes(D, D), CM = F::bytes(C, C);
    static constexpr int A = 0;                      // Ahat rows (t, j)
    static constexpr int R = A + RM;                 // Rhat rows
    static constexpr int Bm = R + RM;                // Btil rows
    static constexpr int Km = Bm + RM;               // Ktil rows
    static constexpr int V = Km + RM;                // v rows (t, i), exact: one plane
    static constexpr int DY = V + C * F::ld(D) * (SPLIT ? 2 : 4);  // dy rows (t, i)
    static constexpr int S0 = DY + RM;               // S0 rows (i, j)
    static constexpr int Ge = S0 + SM;               // Ge' rows (i, j)
    static constexpr int Gam = Ge + SM;              // fp32 gamma [t][j], stride LDG
    static constexpr int glast = Gam + C * LDG * 4;
    static constexpr int qp = glast + D * 4;         // fp32 16 x 64
    static constexpr int red = qp + 16 * D * 4;      // fp32 10 x 64: parts of diag(Gs^T S0)
    static constexpr int Q = red + 10 * D * 4;
    // region Q, phases 0-3
    static constexpr int Tm = Q;                     // T rows (t, s)
    static constexpr int Lak = Tm + CM;              // Lak rows (t, s)
    static constexpr int Mrb = Lak + CM;             // Mrb rows (t, s)
    static constexpr int QEND1 = Mrb + CM;
    // region Q, phases 4-6
    static constexpr int P1 = Q;                     // P1..P4 rows (t, s)
    static constexpr int HH = P1 + 4 * CM;           // fp32 [t][j]: k dk + b db - r dr - a da
    static constexpr int FA = HH + C * LDG * 4;      // fp32 [t][j]: a da
    static constexpr int QEND2 = FA + C * LDG * 4;
    static constexpr int U = QEND1 > QEND2 ? QEND1 : QEND2;   // U rows (t, i)
    static constexpr int DSA = U + RM;               // DSA rows (t, i)
    static constexpr int total = DSA + RM;
    static_assert(total <= 160 * 1024, "gradient kernel LDS exceeds 160 KiB");
    // with the time-mix prologue, da and db (fp32 [t][j], stride LDG) pass from phase 5 to
    // phase 6 in the U and DSA rows
    static_assert(C * LDG * 4 <= RM, "da / db do not fit the U / DSA rows");
};

template <bool SPLIT>
__device__ __forceinline__ Mat<SPLIT> exact_mat(char* smem, int off, int K) {
    return Mat<SPLIT>{smem + off, Fmt<SPLIT>::ld(K), 0};   // one plane: lo reads see hi
}

// Position of work item idx (the block_map order: with xcd, consecutive items
// of one head stay on one XCD): head = bb * H + hh, chunk c.  The divisions
// use the launch's multipliers.
struct ChunkPos {
    int head, c, bb, hh;
    __device__ __forceinline__ ChunkPos(const BwdArgs& p, int idx, bool xcd) {
        const uint32_t slot = xcd ? (uint32_t)idx >> 3 : (uint32_t)idx;
        const uint32_t q = fdiv(slot, p.fd_nc);
        c = (int)(slot - q * (uint32_t)p.NC);
        head = xcd ? (int)(q * 8 + (idx & 7)) : (int)q;
        bb = (int)fdiv((uint32_t)head, p.fd_h);
        hh = head - bb * p.H;
    }
};

// Byte offset of element e of a token tensor (below 4 GiB, so unsigned 32 bit).
__device__ __forceinline__ int tok_bytes(int e, int es) { return (int)((uint32_t)e * (uint32_t)es); }

// Where one chunk's inputs live.  `on == false` (no next chunk) gives every
// buffer resource size 0, so the loads return zeros without touching memory.
// Token tensors (B, T, H, D) are addressed whole, with 32-bit byte offsets
// (the entry points keep them below 4 GiB): one scalar per chunk, tokc, and a
// per-lane part that does not change from chunk to chunk.
struct ChunkSrc {
    int tokc;       // element offset of the chunk's first token (head bb, hh)
    int64_t cs;     // element offset of the chunk's D x D state blocks
    int64_t ci;     // element offset of the chunk's C x C inverse
    int t0, cc;     // first token, tokens in the chunk
    bool on, has_ge;
    const float* ge;   // gradient at the chunk's end: next checkpoint's, dhT, or none

    __device__ __forceinline__ ChunkSrc(const BwdArgs& p, const ChunkPos& w, bool on_) {
        const int HD = p.H * D;
        tokc = (w.bb * p.T + w.c * C) * HD + w.hh * D;
        cs = ((int64_t)w.head * p.NC + w.c) * D * D;
        ci = ((int64_t)w.head * p.NC + w.c) * C * C;
        t0 = w.c * C;
        cc = min(C, p.T - t0);
        on = on_;
        has_ge = w.c + 1 < p.NC || p.dhT != nullptr;
        ge = (w.c + 1 < p.NC) ? p.gbuf + cs + D * D : (p.dhT ? p.dhT + (int64_t)w.head * D * D : p.gbuf);
    }
};

// Everything one chunk reads from global memory, held in registers so that
// the next chunk's loads are in flight while the current chunk computes.  The
// loads are issued in five parts spread over the compute phases, so that no wave
// stalls on a full memory queue; buffer loads without branches keep the
// wave's count of outstanding loads exact.
template <typename InT, bool PROJ>
struct GradIn {
    using W = typename Pair<InT>::T;
    static constexpr int ES = sizeof(InT);
    RawChunk<GNT, InT, PROJ> raw;    // w, a, r, b, k (PROJ: w_raw, kappa, r, alpha, k)
    RawCols<GNT, D, InT> rv;         // v
    RawCols<GNT, D, float> rdy;      // dy
    f32x4 s0v[2], gev[2];            // S0, Ge (gradient at the chunk's end): row si, 8 columns
    float2 tv;                       // two entries of T = (I - Lab)^-1

    template <typename X>
    static __device__ __forceinline__ X ld(Rsrc r, int off) {
        if constexpr (sizeof(X) == 4) {
            return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
        } else {
            return __builtin_bit_cast(X, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
        }
    }
    static __device__ __forceinline__ f32x4 ld4(Rsrc r, int off) {
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
    // A whole token tensor.  Tokens past the head's end in a ragged last chunk
    // read the next head's rows (or 0 past the tensor); the consumers mask them.
    static __device__ __forceinline__ Rsrc tok(const void* base, const BwdArgs& p, const ChunkSrc& s, int es) {
        return make_rsrc(base, s.on ? (uint32_t)p.B * (uint32_t)(p.T * p.H * D * es) : 0u);
    }
    // w, a, r, b, k: columns 2 jp, 2 jp + 1 of tokens q TPG + tt
    __device__ __forceinline__ void raw_part(W* dst, const void* src, const BwdArgs& p, const ChunkSrc& s, int tid) {
        constexpr int TPG = RawChunk<GNT, InT, PROJ>::TPG;
        const Rsrc r = tok(src, p, s, ES);
        const int jp = tid & 31, q = tid >> 5, HD = p.H * D;
#pragma unroll
        for (int tt = 0; tt < TPG; ++tt) dst[tt] = ld<W>(r, tok_bytes(s.tokc + (q * TPG + tt) * HD + 2 * jp, ES));
    }
    template <int PART>
    __device__ __forceinline__ void issue(const BwdArgs& p, const ChunkSrc& s, int tid) {
        using RC = RawCols<GNT, D, InT>;
        const int si = tid >> 3, sj0 = (tid & 7) * 8, soff = (si * D + sj0) * 4;
        const uint32_t sbytes = s.on ? D * D * 4 : 0u;
        if constexpr (PART == 0) {
            raw.cc = rv.cc = rdy.cc = s.cc;
            raw_part(raw.w, p.w, p, s, tid);
            raw_part(raw.a, p.a, p, s, tid);
            raw_part(raw.r, p.r, p, s, tid);
        } else if constexpr (PART == 1) {
            raw_part(raw.b, p.b, p, s, tid);
            raw_part(raw.k, p.k, p, s, tid);
            const Rsrc r = tok(p.v, p, s, ES);
            const int ip = tid % RC::PAIRS, t1 = tid / RC::PAIRS, HD = p.H * D;
#pragma unroll
            for (int u = 0; u < RC::PER; ++u) rv.v[u] = ld<W>(r, tok_bytes(s.tokc + (t1 + u * RC::TSTEP) * HD + 2 * ip, ES));
        } else if constexpr (PART == 2) {
            const Rsrc r = tok(p.dy, p, s, 4);
            const int ip = tid % RC::PAIRS, t1 = tid / RC::PAIRS, HD = p.H * D;
#pragma unroll
            for (int u = 0; u < RC::PER; ++u) rdy.v[u] = ld<float2>(r, tok_bytes(s.tokc + (t1 + u * RC::TSTEP) * HD + 2 * ip, 4));
            tv = ld<float2>(make_rsrc(p.inv + s.ci, s.on ? C * C * 4 : 0u), tid * 8);
        } else if constexpr (PART == 3) {
            const Rsrc r = make_rsrc(p.ckpt + s.cs, sbytes);
            s0v[0] = ld4(r, soff);
            s0v[1] = ld4(r, soff + 16);
        } else {
            const Rsrc r = make_rsrc(s.ge, s.has_ge ? sbytes : 0u);
            gev[0] = ld4(r, soff);
            gev[1] = ld4(r, soff + 16);
        }
    }
    __device__ __forceinline__ void issue_all(const BwdArgs& p, const ChunkSrc& s, int tid) {
        issue<0>(p, s, tid);
        issue<1>(p, s, tid);
        issue<2>(p, s, tid);
        issue<3>(p, s, tid);
        issue<4>(p, s, tid);
    }
};

// Persistent: each workgroup takes chunks blockIdx.x, + gridDim.x, ... of the
// total; while it works on one chunk the next chunk's inputs are loading.
template <typename InT, bool SPLIT, bool PROJ>
__global__ __launch_bounds__(GNT) void grad_kernel(BwdArgs p, int xcd, int total) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    using L = GradSmem<SPLIT>;
    using M = Mat<SPLIT>;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    const int r16 = lane & 15, g4 = lane >> 4;
    const int HD = p.H * D;
    // state-sized inputs: thread holds row si = tid / 8, columns sj0 .. sj0 + 7
    const int si = tid >> 3, sj0 = (tid & 7) * 8;

    int idx = blockIdx.x;
    GradIn<InT, PROJ> cur, nxt;
    cur.issue_all(p, ChunkSrc(p, ChunkPos(p, idx, xcd != 0), true), tid);
    // The first chunk needs these at once.  Waiting here also leaves nothing
    // pending on entry to the loop, so the compiler sizes the loop's waits for
    // the steady state (where the previous chunk's stores are still in flight)
    // instead of for this entry.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

  for (;;) {
    const ChunkPos cw(p, idx, xcd != 0);
    const int c = cw.c, bb = cw.bb, hh = cw.hh;
    const int nidx = idx + (int)gridDim.x;
    const bool more = nidx < total;
    const ChunkSrc nsrc(p, ChunkPos(p, more ? nidx : idx, xcd != 0), more);
    nxt.template issue<0>(p, nsrc, tid);
    const int t0 = c * C, cc = min(C, p.T - t0);
    // fp32 outputs: whole tensors; a token past the sequence's end gets an
    // offset beyond every tensor, so the hardware drops its store
    const int tokc = (bb * p.T + t0) * HD + hh * D;
    const uint32_t out_bytes = (uint32_t)p.B * (uint32_t)(p.T * HD * 4);
    auto out_off = [&](int t, int j) { return t < cc ? tok_bytes(tokc + t * HD + j, 4) : (int)kDropOffset; };

    // ---- phase 0: gamma and the scaled rows
    const M A = make_mat<SPLIT>(smem, L::A, C, D), R = make_mat<SPLIT>(smem, L::R, C, D);
    const M Bm = make_mat<SPLIT>(smem, L::Bm, C, D), Km = make_mat<SPLIT>(smem, L::Km, C, D);
    const M Vm = exact_mat<SPLIT>(smem, L::V, D), DYm = make_mat<SPLIT>(smem, L::DY, C, D);
    const M S0m = make_mat<SPLIT>(smem, L::S0, D, D), Gem = make_mat<SPLIT>(smem, L::Ge, D, D);
    const M Tm = make_mat<SPLIT>(smem, L::Tm, C, C), Lak = make_mat<SPLIT>(smem, L::Lak, C, C);
    const M Mrb = make_mat<SPLIT>(smem, L::Mrb, C, C);
    const M Um = make_mat<SPLIT>(smem, L::U, C, D), DSAm = make_mat<SPLIT>(smem, L::DSA, C, D);
    auto Pm = [&](int m) { return make_mat<SPLIT>(smem, L::P1 + m * L::CM, C, C); };
    float* gam = reinterpret_cast<float*>(smem + L::Gam);
    float* glast = reinterpret_cast<float*>(smem + L::glast);
    float* qp = reinterpret_cast<float*>(smem + L::qp);
    float* red = reinterpret_cast<float*>(smem + L::red);
    float* hh_ = reinterpret_cast<float*>(smem + L::HH);
    float* fa_ = reinterpret_cast<float*>(smem + L::FA);

    const PrepOut<SPLIT> po{A, R, Bm, Km, A, A, A, A, true, true, true, true, false, false, false, false,
                            gam, glast};
    cur.raw.finish();
    chunk_prep<GNT, SPLIT>(cur.raw, po, qp, tid);
    cur.rv.template store_rows<SPLIT, true>(Vm, tid);
    cur.rdy.template store_rows<SPLIT, false>(DYm, tid);
#pragma unroll
    for (int q = 0; q < 2; ++q) put4(S0m, si, sj0 + 4 * q, cur.s0v[q]);
    put2(Tm, tid >> 4, 2 * (tid & 15), cur.tv.x, cur.tv.y);
    lds_barrier();

    nxt.template issue<1>(p, nsrc, tid);
    // ---- phase 1: Lak = stril(Ahat Ktil^T), Mrb = tril(Rhat Btil^T) (rows); Ge' = Ge diag(gamma_last)
    if (wave < 6) {
        const int mat = wave / 3, tile = wave % 3;
        const int ti = tile == 0 ? 0 : 1, tj = tile == 2 ? 1 : 0;
        // accumulator element (s, t): lane (g, r) holds row t = 16 ti + r, columns s = 16 tj + 4g ..
        const int t = 16 * ti + r16, s0_ = 16 * tj + 4 * g4;
        if (mat == 0) {
            f32x4 acc = mma<SPLIT, D>(zero4(), Km, tj * 16, A, ti * 16, lane);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] = s0_ + q < t ? acc[q] : 0.f;
            put4_pair(Lak, t, 16 * tj + 8 * (g4 >> 1), acc, g4);
        } else {
            f32x4 acc = mma<SPLIT, D>(zero4(), Bm, tj * 16, R, ti * 16, lane);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] = s0_ + q <= t ? acc[q] : 0.f;
            put4_pair(Mrb, t, 16 * tj + 8 * (g4 >> 1), acc, g4);
        }
    } else {
        zero_block(wave == 6 ? Lak : Mrb, 0, 16, lane);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) cur.gev[q][e] *= glast[sj0 + 4 * q + e];
        put4(Gem, si, sj0 + 4 * q, cur.gev[q]);
    }
    {   // sum_i G'[i][j] S0[i][j] over this wave's 8 rows (lanes with equal tid % 8 share columns)
        f32x4 d0 = cur.gev[0] * cur.s0v[0], d1 = cur.gev[1] * cur.s0v[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            d0[e] = sum_stride8(d0[e]);
            d1[e] = sum_stride8(d1[e]);
        }
        if (lane < 8) {
            *reinterpret_cast<f32x4*>(red + wave * 64 + sj0) = d0;
            *reinterpret_cast<f32x4*>(red + wave * 64 + sj0 + 4) = d1;
        }
    }
    lds_barrier();

    nxt.template issue<2>(p, nsrc, tid);
    // ---- phases 2 and 3 (no barrier between them):
    // phase 2: RHS_U[s][i] = sum_j S0[i][j] Ahat[s][j] + sum_u V[u][i] Lak[s][u]
    //          RHS_D[s][i] = sum_j Ge'[i][j] Btil[s][j] + sum_u DY[u][i] Mrb[u][s]
    // phase 3: U[t][i] = sum_s T[t][s] RHS_U[s][i], DSA[t][i] = sum_s T[s][t] RHS_D[s][i].
    // Waves 0-3: RHS_U and U, waves 4-7: RHS_D and DSA; wave: column block ib, both blocks of s
    // (the i-side fragments are read once for both) and then both blocks of t.  The RHS tiles are
    // formed as accumulator elements (s, i), which in the fragment order are the operand rows i
    // over k = s of the U / DSA products: they never leave the registers.
    {
        using Fr = Frag<SPLIT>;
        const int ib = wave & 3;
        f32x4 a0, a1;
        if (wave < 4) {
            const Fr x0 = frag_n(S0m, 16 * ib, 0, lane), x1 = frag_n(S0m, 16 * ib, 32, lane);
            a0 = fmma(zero4(), frag_n(A, 0, 0, lane), x0);
            a1 = fmma(zero4(), frag_n(A, 16, 0, lane), x0);
            a0 = fmma(a0, frag_n(A, 0, 32, lane), x1);
            a1 = fmma(a1, frag_n(A, 16, 32, lane), x1);
            const Fr xv = frag_t_exact(Vm, 16 * ib, 0, lane);
            a0 = fmma<false, true>(a0, frag_n(Lak, 0, 0, lane), xv);
            a1 = fmma<false, true>(a1, frag_n(Lak, 16, 0, lane), xv);
        } else {
            const Fr x0 = frag_n(Gem, 16 * ib, 0, lane), x1 = frag_n(Gem, 16 * ib, 32, lane);
            a0 = fmma(zero4(), frag_n(Bm, 0, 0, lane), x0);
            a1 = fmma(zero4(), frag_n(Bm, 16, 0, lane), x0);
            a0 = fmma(a0, frag_n(Bm, 0, 32, lane), x1);
            a1 = fmma(a1, frag_n(Bm, 16, 32, lane), x1);
            const Fr xd = frag_t(DYm, 16 * ib, 0, lane);
            a0 = fmma(a0, frag_t(Mrb, 0, 0, lane), xd);
            a1 = fmma(a1, frag_t(Mrb, 16, 0, lane), xd);
        }
        nxt.template issue<3>(p, nsrc, tid);
        const Fr rhs = frag_acc<SPLIT>(a0, a1);   // rows i = 16 ib + r, k = s
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            // accumulator element (i, t)
            if (wave < 4) {
                const f32x4 au = fmma(zero4(), rhs, frag_n(Tm, 16 * tb, 0, lane));
                put4_pair(Um, 16 * tb + r16, 16 * ib + 8 * (g4 >> 1), au, g4);
            } else {
                const f32x4 ad = fmma(zero4(), rhs, frag_t(Tm, 16 * tb, 0, lane));
                put4_pair(DSAm, 16 * tb + r16, 16 * ib + 8 * (g4 >> 1), ad, g4);
            }
        }
    }
    lds_barrier();

    nxt.template issue<4>(p, nsrc, tid);
    // ---- phase 4: P1 = tril(DY U^T), P2 = tril(DY V^T), P3 = stril(DSA U^T), P4 = stril(DSA V^T),
    // rows (t, s); accumulator element (s, t)
    {   // wave: tile (wave % 4) of P(wave / 4) and P(wave / 4 + 2); tile 3 (s >= 16 > t) is zero
        const int tile = wave & 3, m0 = wave >> 2;
        if (tile == 3) {
            put4_pair(Pm(m0), r16, 16 + 8 * (g4 >> 1), zero4(), g4);
            put4_pair(Pm(m0 + 2), r16, 16 + 8 * (g4 >> 1), zero4(), g4);
        } else {
            const int sb = tile == 2 ? 1 : 0, tb = tile == 0 ? 0 : 1;
            // m0 = 0: P1 (DY U^T), P3 (DSA U^T); m0 = 1: P2 (DY V^T), P4 (DSA V^T)
            f32x4 a0, a1;
            if (m0 == 0) {
                a0 = fmma(zero4(), frag_n(Um, 16 * sb, 0, lane), frag_n(DYm, 16 * tb, 0, lane));
                a1 = fmma(zero4(), frag_n(Um, 16 * sb, 0, lane), frag_n(DSAm, 16 * tb, 0, lane));
                a0 = fmma(a0, frag_n(Um, 16 * sb, 32, lane), frag_n(DYm, 16 * tb, 32, lane));
                a1 = fmma(a1, frag_n(Um, 16 * sb, 32, lane), frag_n(DSAm, 16 * tb, 32, lane));
            } else {
                a0 = fmma<true, false>(zero4(), frag_n(Vm, 16 * sb, 0, lane), frag_n(DYm, 16 * tb, 0, lane));
                a1 = fmma<true, false>(zero4(), frag_n(Vm, 16 * sb, 0, lane), frag_n(DSAm, 16 * tb, 0, lane));
                a0 = fmma<true, false>(a0, frag_n(Vm, 16 * sb, 32, lane), frag_n(DYm, 16 * tb, 32, lane));
                a1 = fmma<true, false>(a1, frag_n(Vm, 16 * sb, 32, lane), frag_n(DSAm, 16 * tb, 32, lane));
            }
            const int t = 16 * tb + r16, s0_ = 16 * sb + 4 * g4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int s = s0_ + q;
                if (s > t) a0[q] = 0.f;    // P1, P2: s <= t
                if (s >= t) a1[q] = 0.f;   // P3, P4: s < t
            }
            put4_pair(Pm(m0), t, 16 * sb + 8 * (g4 >> 1), a0, g4);
            put4_pair(Pm(m0 + 2), t, 16 * sb + 8 * (g4 >> 1), a1, g4);
        }
    }
    lds_barrier();

    // ---- phase 5: outputs, accumulator element (j, t).  Waves 0-3 form dr and da, waves 4-7 dk and
    // db; each wave one t block and two j blocks, so the t-side operands are read once for both.
    // The dw ingredients: waves 4-7 store k dk + b db to hh_, waves 0-3 store a da to fa_ and, after
    // the next barrier, add -r dr - a da to hh_.  Waves 0-3 also complete diag(Gs^T S0): with
    // Gs = G' + DY^T Rhat + DSA^T Ahat it is sum_i G' S0 (phase 1) plus the column sums over t of
    // Rhat * (DY S0) and Ahat * (DSA S0), the first terms of the dr and da accumulators.
    {
        using Fr = Frag<SPLIT>;
        const int pr = wave >> 2, tb = (wave >> 1) & 1, jb0 = (wave & 1) * 2;
        const int t = 16 * tb + r16;
        f32x4 ac[2][2];   // [first / second output][j block]
        f32x4 xs[2][2];   // waves 0-3: DY S0 and DSA S0 tiles
        // k-step-major: each step reads two j-side and two t-side fragments and advances four
        // independent accumulators (two outputs x two j blocks).  fp32 fragments take twice the
        // registers; a compiler barrier between steps keeps only one step's fragments live.
        auto kstep = [&](f32x4 (&a)[2][2], const Fr& x0, const Fr& x1, const Fr& y0, const Fr& y1, auto ex) {
            constexpr bool YEX = decltype(ex)::value;
            a[0][0] = fmma<false, YEX>(a[0][0], x0, y0);
            a[0][1] = fmma<false, YEX>(a[0][1], x1, y0);
            a[1][0] = fmma(a[1][0], x0, y1);
            a[1][1] = fmma(a[1][1], x1, y1);
            if constexpr (!SPLIT) asm volatile("" ::: "memory");
        };
        using exact_t = std::integral_constant<bool, true>;
        using split_t = std::integral_constant<bool, false>;
#pragma unroll
        for (int o = 0; o < 2; ++o)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) ac[o][jj] = zero4();
        // The four k-steps' fragments.  Split format: each step's reads are issued before the
        // previous step's products (sched_barrier), so the LDS latency overlaps the MFMA work;
        // fp32 fragments are twice as large and are read right before their step.
        struct Step {
            Fr x0, x1, y0, y1;
        };
        auto run4 = [&](auto ld, auto ex01, auto on_step) {
            using I0 = std::integral_constant<int, 0>;
            using I1 = std::integral_constant<int, 1>;
            using I2 = std::integral_constant<int, 2>;
            using I3 = std::integral_constant<int, 3>;
            auto go = [&](const Step& st, int k) {
                if (k < 2) kstep(ac, st.x0, st.x1, st.y0, st.y1, ex01);
                else kstep(ac, st.x0, st.x1, st.y0, st.y1, split_t{});
                on_step(k);
            };
            if constexpr (SPLIT) {
                Step s0 = ld(I0{});
                Step s1 = ld(I1{});
                __builtin_amdgcn_sched_barrier(0);
                go(s0, 0);
                Step s2 = ld(I2{});
                __builtin_amdgcn_sched_barrier(0);
                go(s1, 1);
                Step s3 = ld(I3{});
                __builtin_amdgcn_sched_barrier(0);
                go(s2, 2);
                go(s3, 3);
            } else {
                go(ld(I0{}), 0);
                go(ld(I1{}), 1);
                go(ld(I2{}), 2);
                go(ld(I3{}), 3);
            }
        };
        auto no_op = [](int) {};
        if (pr == 0) {
            // aR = S0 DY + Btil P1 + Ktil P2, aA = S0 DSA + Btil P3 + Ktil P4 (j side first)
            auto ld = [&](auto kc) {
                constexpr int K = decltype(kc)::value;
                if constexpr (K < 2)
                    return Step{frag_t(S0m, 16 * jb0, 32 * K, lane), frag_t(S0m, 16 * jb0 + 16, 32 * K, lane),
                                frag_n(DYm, 16 * tb, 32 * K, lane), frag_n(DSAm, 16 * tb, 32 * K, lane)};
                else if constexpr (K == 2)
                    return Step{frag_t(Bm, 16 * jb0, 0, lane), frag_t(Bm, 16 * jb0 + 16, 0, lane),
                                frag_n(Pm(0), 16 * tb, 0, lane), frag_n(Pm(2), 16 * tb, 0, lane)};
                else
                    return Step{frag_t(Km, 16 * jb0, 0, lane), frag_t(Km, 16 * jb0 + 16, 0, lane),
                                frag_n(Pm(1), 16 * tb, 0, lane), frag_n(Pm(3), 16 * tb, 0, lane)};
            };
            run4(ld, split_t{}, [&](int k) {
                if (k == 1) {
#pragma unroll
                    for (int o = 0; o < 2; ++o)
#pragma unroll
                        for (int jj = 0; jj < 2; ++jj) xs[o][jj] = ac[o][jj];
                }
            });
        } else {
            // aK = Ge' V + Ahat P4^T + Rhat P2^T, aB = Ge' U + Ahat P3^T + Rhat P1^T
            auto ld = [&](auto kc) {
                constexpr int K = decltype(kc)::value;
                if constexpr (K < 2)
                    return Step{frag_t(Gem, 16 * jb0, 32 * K, lane), frag_t(Gem, 16 * jb0 + 16, 32 * K, lane),
                                frag_n(Vm, 16 * tb, 32 * K, lane), frag_n(Um, 16 * tb, 32 * K, lane)};
                else if constexpr (K == 2)
                    return Step{frag_t(A, 16 * jb0, 0, lane), frag_t(A, 16 * jb0 + 16, 0, lane),
                                frag_t(Pm(3), 16 * tb, 0, lane), frag_t(Pm(2), 16 * tb, 0, lane)};
                else
                    return Step{frag_t(R, 16 * jb0, 0, lane), frag_t(R, 16 * jb0 + 16, 0, lane),
                                frag_t(Pm(1), 16 * tb, 0, lane), frag_t(Pm(0), 16 * tb, 0, lane)};
            };
            run4(ld, exact_t{}, no_op);
        }
        const Rsrc r0 = make_rsrc(pr == 0 ? p.dr : p.dk, out_bytes);
        const Rsrc r1 = make_rsrc(pr == 0 ? p.da : p.db, out_bytes);
        const int tp = t > 0 ? t - 1 : 0;
        f32x4 evr[2];   // waves 0-3: -r dr - a da, added to hh_ after the barrier
        f32x4 o1[2];    // PROJ: da (waves 0-3) or db (waves 4-7), to LDS after the barrier
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int j0 = 16 * (jb0 + jj) + 4 * g4;
            const int voff = out_off(t, j0);
            const f32x4 g = *reinterpret_cast<const f32x4*>(gam + t * LDG + j0);
            f32x4 sc0, sc1;   // output scales
            if (pr == 0) {
                // dr = gamma_t aR, da = gamma_{t-1} aA; r dr = Rhat aR, a da = Ahat aA
                const f32x4 gpl = *reinterpret_cast<const f32x4*>(gam + tp * LDG + j0);
                sc0 = g;
                sc1 = t > 0 ? gpl : f32x4{1.f, 1.f, 1.f, 1.f};
                const f32x4 ah = get4(A, t, j0), rh = get4(R, t, j0);
                const f32x4 fa = ah * ac[1][jj];
                evr[jj] = -(rh * ac[0][jj]) - fa;
                *reinterpret_cast<f32x4*>(fa_ + t * LDG + j0) = fa;
                // this wave's 16 tokens of sum_t Rhat (DY S0) + Ahat (DSA S0); lane r16 = 15 holds the sum
                f32x4 dg = rh * xs[0][jj] + ah * xs[1][jj];
#pragma unroll
                for (int q = 0; q < 4; ++q) dg[q] = row_sum16(dg[q]);
                if (r16 == 15) *reinterpret_cast<f32x4*>(red + (8 + tb) * 64 + j0) = dg;
            } else {
                // dk = aK / gamma_t, db = aB / gamma_t; k dk = Ktil aK, b db = Btil aB
#pragma unroll
                for (int q = 0; q < 4; ++q) sc0[q] = rcp(g[q]);
                sc1 = sc0;
                *reinterpret_cast<f32x4*>(hh_ + t * LDG + j0) =
                    get4(Km, t, j0) * ac[0][jj] + get4(Bm, t, j0) * ac[1][jj];
            }
            // outside the branch: every wave issues the same stores, so the
            // compiler counts this chunk's outstanding stores exactly
            bstore4<kStreamDev>(ac[0][jj] * sc0, r0, voff, 0);
            if constexpr (PROJ) o1[jj] = ac[1][jj] * sc1;
            else bstore4<kStreamDev>(ac[1][jj] * sc1, r1, voff, 0);
        }
        lds_barrier();
        if (pr == 0) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                f32x4* h = reinterpret_cast<f32x4*>(hh_ + t * LDG + 16 * (jb0 + jj) + 4 * g4);
                *h = *h + evr[jj];
            }
        }
        if constexpr (PROJ) {
            // the prologue's backward (phase 6) needs da and db at one (t, j): they meet in the
            // U and DSA rows, which no wave reads after the products above
            float* dst = reinterpret_cast<float*>(smem + (pr == 0 ? L::U : L::DSA));
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
                *reinterpret_cast<f32x4*>(dst + t * LDG + 16 * (jb0 + jj) + 4 * g4) = o1[jj];
        }
    }
    lds_barrier();

    // ---- phase 6: dw: phi_t = diag(Gs^T S0) - sum_{s<=t} a da + sum_{s<t} (k dk + b db - r dr),
    //      dw_t = phi_t / w_t.  Thread (jp, q) scans tokens TPG q .. of columns 2jp, 2jp+1.
    {
        constexpr int TPG = RawChunk<GNT, InT, PROJ>::TPG, NG = RawChunk<GNT, InT, PROJ>::NG;
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
        // wave 0, lane = column: diag(Gs^T S0) (the 8 waves' G' S0 rows and the 2 token-block rows)
        // plus the sums over earlier token groups, in place
        if (wave == 0) {
            float rv[GNW + 2], qv[NG];   // all reads first, then the sums, then the writes
#pragma unroll
            for (int g = 0; g < GNW + 2; ++g) rv[g] = red[g * 64 + lane];
#pragma unroll
            for (int q2 = 0; q2 < NG; ++q2) qv[q2] = qp[q2 * 64 + lane];
            float run = 0.f;
#pragma unroll
            for (int g = 0; g < GNW + 2; ++g) run += rv[g];
#pragma unroll
            for (int q2 = 0; q2 < NG; ++q2) {
                const float v = qv[q2];
                qv[q2] = run;
                run += v;
            }
#pragma unroll
            for (int q2 = 0; q2 < NG; ++q2) qp[q2 * 64 + lane] = qv[q2];
        }
        lds_barrier();
        float2 acc = *reinterpret_cast<const float2*>(qp + q * 64 + j0);
        const Rsrc rdw = make_rsrc(p.dw, out_bytes);
#pragma unroll
        for (int tt = 0; tt < TPG; ++tt) {
            const int t = q * TPG + tt;
            const float2 phi = make_float2(acc.x - fx[tt].x, acc.y - fx[tt].y);   // dw_t w_t
            const float2 x = Pair<InT>::f(cur.raw.w[tt]);
            if constexpr (PROJ) {
                // dw_raw = dw w (-e^-1/2) s (1 - s), s = sigmoid(w_raw)
                const float sx = logistic_f(x.x), sy = logistic_f(x.y);
                bstore2<kStreamDev>(make_float2(-kDecayScale * phi.x * sx * (1.f - sx),
                                                -kDecayScale * phi.y * sy * (1.f - sy)), rdw, out_off(t, j0), 0);
            } else {
                bstore2<kStreamDev>(make_float2(phi.x * rcp(x.x), phi.y * rcp(x.y)), rdw, out_off(t, j0), 0);
            }
            acc.x += hx[tt].x;
            acc.y += hx[tt].y;
        }
        if constexpr (PROJ) {
            // the prologue's backward for a = -kh and b = kh sigmoid(alpha), kh = kappa / |kappa|:
            // g = -da + sigmoid(alpha) db (the gradient w.r.t. kh), dkappa = (g - kh (kh . g)) / |kappa|
            // with the dot product over the token's 64 columns (the 32 lanes of this half wave),
            // dalpha = db kh s (1 - s), s = sigmoid(alpha)
            const float* lda = reinterpret_cast<const float*>(smem + L::U);
            const float* ldb = reinterpret_cast<const float*>(smem + L::DSA);
            const Rsrc rka = make_rsrc(p.da, out_bytes), ral = make_rsrc(p.db, out_bytes);
#pragma unroll
            for (int tt = 0; tt < TPG; ++tt) {
                const int t = q * TPG + tt;
                const float2 dav = *reinterpret_cast<const float2*>(lda + t * LDG + j0);
                const float2 dbv = *reinterpret_cast<const float2*>(ldb + t * LDG + j0);
                const float2 kh = cur.raw.kappa_hat(tt), al = Pair<InT>::f(cur.raw.b[tt]);
                const float sx = logistic_f(al.x), sy = logistic_f(al.y);
                const float gx = dbv.x * sx - dav.x, gy = dbv.y * sy - dav.y;
                const float dot = half_sum32(kh.x * gx + kh.y * gy);
                const float iv = cur.raw.inv[tt];
                bstore2<kStreamDev>(make_float2((gx - kh.x * dot) * iv, (gy - kh.y * dot) * iv), rka,
                                    out_off(t, j0), 0);
                bstore2<kStreamDev>(make_float2(dbv.x * kh.x * sx * (1.f - sx), dbv.y * kh.y * sy * (1.f - sy)), ral,
                                    out_off(t, j0), 0);
            }
        }
    }
    // The next chunk's loads (issued in phases 0-4) are all back by now; wait
    // for them here, leaving only this chunk's output stores in flight (six;
    // eight with the prologue).  Otherwise the compiler's count for their first
    // uses (merged over the loop's back edge) would also wait for those stores
    // to complete.
    __builtin_amdgcn_s_waitcnt(PROJ ? 0x0F78 : 0x0F76);   // vmcnt(8) / vmcnt(6)
    if (!more) break;
    cur = nxt;
    idx = nidx;
    lds_barrier();   // this chunk's last LDS reads before the next chunk's writes
  }
}

template <typename InT, bool SPLIT, bool PROJ>
hipError_t launch_typed(BwdArgs a, hipStream_t s) {
    using L = GradSmem<SPLIT>;
    auto kern = grad_kernel<InT, SPLIT, PROJ>;
    static PerDeviceOnce once;
    hipError_t e = set_smem_once(once, kern, L::total);
    if (e != hipSuccess) return e;
    // one workgroup per CU (the LDS plan takes most of a CU's 160 KiB)
    int n_cu = 0;
    e = device_cus(&n_cu);
    if (e != hipSuccess) return e;
    const int heads = a.B * a.H;
    const int total = heads * a.NC;
    const int xcd = (heads % 8 == 0) ? 1 : 0;
    int grid = total < n_cu ? total : n_cu;
    if (xcd && grid > 8) grid -= grid % 8;   // a workgroup's chunks stay on one XCD
    a.fd_nc = make_fastdiv((uint32_t)a.NC);
    a.fd_h = make_fastdiv((uint32_t)a.H);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(GNT), L::total, s, a, xcd, total);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_inputs(const BwdArgs& a, bool bf16, bool proj, hipStream_t s) {
    if (proj) {
        if (bf16) return launch_typed<uint16_t, true, true>(a, s);
        return launch_typed<float, false, true>(a, s);
    }
    if (bf16) return launch_typed<uint16_t, true, false>(a, s);
    return launch_typed<float, false, false>(a, s);
}

}  // namespace wkv7
