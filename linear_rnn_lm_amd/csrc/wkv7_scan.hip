// wkv7_scan.hip -- the WKV7 chunk recurrence as a scan over per-chunk
// transition operands (gfx950).
//
// Unrolling the per-token update over one chunk (rwkv-mlx page, "Metal kernel
// architecture", forward block; wkv7_device.h has the chunk matrices Ahat,
// Rhat, Btil, Ktil, Lab, Lak, Mrb, Mrk) and eliminating U with
// T = (I - Lab)^-1, W1 = T Ahat and Z = T Lak gives, for the state S0
// entering the chunk and the chunk's v rows V,
//     S_end = S0 P + V^T M,        Y = E S0^T + F V
// with four operands that depend on the chunk's r, w, k, a, b only:
//     P = (I + W1^T Btil) diag(gamma_last)        (D x D, rows j, columns j')
//     M = (Z^T Btil + Ktil) diag(gamma_last)      (C x D)
//     E = Rhat + Mrb W1                           (C x D)
//     F = Mrb Z + Mrk                             (C x C, lower triangular)
// The backward (same page, backward block) runs the transposed map: with G
// the gradient at the chunk's end and DY the chunk's dy rows,
//     G_start = G P^T + DY^T E,     dv = M G^T + F^T DY.
//
// Kernel "prepare": one workgroup per (head, chunk), all chunks at once: the
// chunk matrices, T, and P, M, E, F, written to memory (T as fp32 for the
// input-gradient kernel, P, M, E, F in the operand format: two bf16 planes
// hi/lo for bf16 inputs, fp32 otherwise).
// Kernel "scan": 16 state rows per wave, chunks in order (forward) or in
// reverse (backward).  The state stays in the MFMA accumulators across
// chunks: with the permuted k order of Frag (wkv7_device.h) a 16 x 16 result
// tile is already an operand fragment of the next chunk's product, so the
// only serial work per chunk is one D x D product per wave.  The operands of
// the next chunk are fetched into registers one chunk ahead and staged in a
// double-buffered LDS copy shared by the workgroup's waves.
#include <type_traits>

#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

// Element offsets of P, M, E, F inside one chunk's operand block, in storage
// elements (bf16 for the split format, which keeps the hi plane of a matrix
// followed by its lo plane; fp32 otherwise).  Each plane is a sequence of
// 16 x 16 tiles, row-major over the tiles and row-major inside a tile (256
// elements), so that one wave stores a whole tile as one contiguous block.
template <bool SPLIT>
struct OpsLayout {
    using E = typename std::conditional<SPLIT, __bf16, float>::type;
    static constexpr int planes = SPLIT ? 2 : 1;
    static constexpr int P = 0;                        // (j, j')  64 x 64
    static constexpr int M = P + planes * D * D;       // (t, j)   32 x 64
    static constexpr int E_ = M + planes * C * D;      // (t, j)   32 x 64
    static constexpr int F = E_ + planes * C * D;      // (t, u)   32 x 32
    static constexpr int total = F + planes * C * C;
    static_assert(total * (int)sizeof(E) == kOpsBytes, "operand block size");
};

// ------------------------------------------------------------------ prepare
template <bool SPLIT>
struct PrepSmem {
    using F = Fmt<SPLIT>;
    static constexpr int A = 0;                        // Ahat rows (t, j)
    static constexpr int R = A + F::bytes(C, D);       // Rhat rows
    static constexpr int Bm = R + F::bytes(C, D);      // Btil rows
    static constexpr int Km = Bm + F::bytes(C, D);     // Ktil rows
    static constexpr int Lak = Km + F::bytes(C, D);    // Lak rows (t, s)
    static constexpr int Mrb = Lak + F::bytes(C, C);   // Mrb rows (t, s)
    static constexpr int W1 = Mrb + F::bytes(C, C);    // W1 rows (t, j)
    static constexpr int Zm = W1 + F::bytes(C, D);     // Z rows (t, u)
    static constexpr int LabF = Zm + F::bytes(C, C);   // fp32 Lab^T, stride LDF
    static constexpr int TF = LabF + C * LDF * 4;      // fp32 T, stride LDF
    static constexpr int Scr = TF + C * LDF * 4;       // 16 x 20 fp32
    static constexpr int glast = Scr + 16 * 20 * 4;    // fp32 [64]
    static constexpr int qp = glast + D * 4;           // fp32 8 x 64
    static constexpr int total = qp + 8 * D * 4;
    static_assert(total <= 80 * 1024, "two workgroups per CU");
};

// Persistent: workgroup b takes items (head, chunk) b, b + gridDim.x, ...; the
// next item's inputs load while the current one is processed.  PROJ: the w, a,
// b inputs are the raw projections w_raw, kappa, alpha (see RawChunk).
template <typename InT, bool SPLIT, bool PROJ>
__global__ __launch_bounds__(256, 2) void chunk_prepare_kernel(PrepArgs p, int items) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    using L = PrepSmem<SPLIT>;
    using M = Mat<SPLIT>;
    using O = OpsLayout<SPLIT>;
    using E = typename O::E;
    constexpr int NT = 256;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g4 = lane >> 4;
    const int64_t tstride = (int64_t)p.H * D;

    RawChunk<NT, InT, PROJ> raw;
    // raw <- the inputs of item `it` (tokens of a ragged last chunk: see RawChunk)
    auto load_item = [&](int it) {
        const int head = it / p.NC, c = it - head * p.NC;
        const int bb = head / p.H, hh = head - bb * p.H;
        const int t0 = c * C;
        const int64_t base = ((int64_t)bb * p.T + t0) * tstride + (int64_t)hh * D;
        raw.load(static_cast<const InT*>(p.w), static_cast<const InT*>(p.a), static_cast<const InT*>(p.r),
                 static_cast<const InT*>(p.b), static_cast<const InT*>(p.k), base, tstride, min(C, p.T - t0), tid);
    };
    int item = blockIdx.x;
    load_item(item);
  for (;;) {
    const int nitem = item + (int)gridDim.x;
    const bool more = nitem < items;

    const M A = make_mat<SPLIT>(smem, L::A, C, D), R = make_mat<SPLIT>(smem, L::R, C, D);
    const M Bm = make_mat<SPLIT>(smem, L::Bm, C, D), Km = make_mat<SPLIT>(smem, L::Km, C, D);
    const M Lak = make_mat<SPLIT>(smem, L::Lak, C, C);
    const M Mrb = make_mat<SPLIT>(smem, L::Mrb, C, C), W1 = make_mat<SPLIT>(smem, L::W1, C, D);
    const M Zm = make_mat<SPLIT>(smem, L::Zm, C, C);
    float* glast = reinterpret_cast<float*>(smem + L::glast);
    float* qp = reinterpret_cast<float*>(smem + L::qp);
    float* labf = reinterpret_cast<float*>(smem + L::LabF);
    float* tf = reinterpret_cast<float*>(smem + L::TF);
    float* scr = reinterpret_cast<float*>(smem + L::Scr);

    // ---- gamma, gamma_last and the scaled operand rows
    const PrepOut<SPLIT> po{A, R, Bm, Km, A, A, A, A, true, true, true, true, false, false, false, false,
                            nullptr, glast};
    raw.finish();
    chunk_prep<NT, SPLIT>(raw, po, qp, tid);
    load_item(more ? nitem : item);   // the last item loads itself again: no branch around the loads
    lds_barrier();

    // ---- Lab^T (fp32, for the inverse): one lower tile per wave 0-2, wave 3 the zero tile
    if (wave < 3) {
        const int ti = wave == 0 ? 0 : 1, tj = wave == 2 ? 1 : 0;
        const f32x4 t = mma<SPLIT, D>(zero4(), A, 16 * ti, Bm, 16 * tj, lane);
        store_f32_t<MASK_STRICT>(labf, LDF, t, 16 * ti, 16 * tj, lane);
    } else {
        // the zero blocks: Lab^T rows 16-31, columns 0-15 and T's rows 0-15, columns 16-31
        for (int e = lane; e < 256; e += 64) {
            labf[(16 + (e >> 4)) * LDF + (e & 15)] = 0.f;
            tf[(e >> 4) * LDF + 16 + (e & 15)] = 0.f;
        }
    }
    lds_barrier();

    // ---- T = (I - Lab)^-1 (wave 3) while waves 0-2 form Lak, Mrb and Mrk
    f32x4 mk0 = zero4(), mk1 = zero4(), mk2 = zero4();
    if (wave == 3) {
        tri_inverse(labf, tf, scr, lane);
    } else if (wave == 0) {
        const f32x4 t00 = mma<SPLIT, D>(zero4(), A, 0, Km, 0, lane);
        const f32x4 t10 = mma<SPLIT, D>(zero4(), A, 16, Km, 0, lane);
        const f32x4 t11 = mma<SPLIT, D>(zero4(), A, 16, Km, 16, lane);
        cc_store<MASK_STRICT>(Lak, true, Lak, false, t00, t10, t11, lane);
    } else if (wave == 1) {
        const f32x4 t00 = mma<SPLIT, D>(zero4(), R, 0, Bm, 0, lane);
        const f32x4 t10 = mma<SPLIT, D>(zero4(), R, 16, Bm, 0, lane);
        const f32x4 t11 = mma<SPLIT, D>(zero4(), R, 16, Bm, 16, lane);
        cc_store<MASK_LOWER>(Mrb, true, Mrb, false, t00, t10, t11, lane);
    } else {
        // Mrk as the start of F: element (u, t) = sum_j Ktil[u][j] Rhat[t][j], kept for u <= t.
        // Tiles (u block, t block) = (0, 0), (0, 1), (1, 1); (1, 0) is zero.
        mk0 = mma<SPLIT, D>(zero4(), Km, 0, R, 0, lane);
        mk1 = mma<SPLIT, D>(zero4(), Km, 0, R, 16, lane);
        mk2 = mma<SPLIT, D>(zero4(), Km, 16, R, 16, lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (4 * g4 + q > r16) {
                mk0[q] = 0.f;
                mk2[q] = 0.f;
            }
        }
    }
    lds_barrier();

    // ---- T to memory: wave w rows 8w .. 8w + 7, four columns per lane
    {
        const int t = 8 * wave + (lane >> 3), s4 = 4 * (lane & 7);
        const f32x4 v = *reinterpret_cast<const f32x4*>(tf + t * LDF + s4);
        *reinterpret_cast<f32x4*>(p.inv + (int64_t)item * C * C + t * C + s4) = v;
    }

    // ---- W1 = T Ahat (rows t, columns j) and Z = T Lak (rows t, columns u).  Wave w: W1 tiles
    // (t blocks 0, 1; j block w) and Z tile w of (u block, t block) = (0, 0), (0, 1), (1, 1); wave 3
    // the zero Z tile (t < 16 <= u).  T's rows come from its fp32 copy, split in registers.
    {
        const Frag<SPLIT> aw = frag_t(A, 16 * wave, 0, lane);
        const Frag<SPLIT> t0f = frag_n_f32<SPLIT>(tf, LDF, 0, 0, lane), t1f = frag_n_f32<SPLIT>(tf, LDF, 16, 0, lane);
        // element (j, t) = sum_s Ahat[s][j] T[t][s]
        const f32x4 w0 = fmma(zero4(), aw, t0f);
        const f32x4 w1 = fmma(zero4(), aw, t1f);
        if (wave < 3) {
            const int ub = wave == 2 ? 1 : 0, tb = wave == 0 ? 0 : 1;
            // element (u, t) = sum_s Lak[s][u] T[t][s]
            const f32x4 z = fmma(zero4(), frag_t(Lak, 16 * ub, 0, lane), tb == 0 ? t0f : t1f);
            put4(Zm, 16 * tb + r16, 16 * ub + 4 * g4, z);
        } else {
            put4(Zm, r16, 16 + 4 * g4, zero4());
        }
        put4(W1, r16, 16 * wave + 4 * g4, w0);
        put4(W1, 16 + r16, 16 * wave + 4 * g4, w1);
    }
    lds_barrier();

    // ---- P, M, E, F to the chunk's operand block; every lane writes four
    // consecutive columns of one row per tile
    E* ob = reinterpret_cast<E*>(static_cast<char*>(p.ops) + (int64_t)item * kOpsBytes);
    // Wave w: P tiles (row block w, column blocks 0..3), M and E tiles (column block w, row
    // blocks 0, 1); wave 2 also F, so wave 3 takes its P tile (2, 3); wave 3 F's zero tile.
    // The W1 and Btil fragments of column block w serve several tiles; all tiles of a wave are
    // independent chains.
    {
        using Fr = Frag<SPLIT>;
        const Fr w1w = frag_t(W1, 16 * wave, 0, lane);   // W1 columns 16w ..
        const Fr bw = frag_t(Bm, 16 * wave, 0, lane);    // Btil columns 16w ..
        f32x4 pa[4], ma[2], ea[2], px = zero4();
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
            if (wave != 2 || pb != 3) pa[pb] = fmma(zero4(), pb == wave ? bw : frag_t(Bm, 16 * pb, 0, lane), w1w);
        if (wave == 3) px = fmma(zero4(), frag_t(Bm, 48, 0, lane), frag_t(W1, 32, 0, lane));   // tile (2, 3)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            ma[tb] = fmma(zero4(), bw, frag_t(Zm, 16 * tb, 0, lane));
            ea[tb] = fmma(zero4(), w1w, frag_n(Mrb, 16 * tb, 0, lane));
        }
        // P[j][j'] = (delta + sum_t W1[t][j] Btil[t][j']) gamma_last[j']; element (j', j), j = 16 rb + r
        auto pstore = [&](f32x4 v, int rb, int pb) {
            const int j = 16 * rb + r16, jp0 = 16 * pb + 4 * g4;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = (v[q] + (jp0 + q == j ? 1.f : 0.f)) * glast[jp0 + q];
            tput4(ob + O::P, D * D, rb * 4 + pb, lane, v);
        };
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
            if (wave != 2 || pb != 3) pstore(pa[pb], wave, pb);
        if (wave == 3) pstore(px, 2, 3);
        // M[t][j] = (sum_s Z[s][t] Btil[s][j] + Ktil[t][j]) gamma_last[j]; element (j, t), j = 16w + 4g + q
        // E[t][j] = Rhat[t][j] + sum_s Mrb[t][s] W1[s][j]; element (j, t)
        const int j0 = 16 * wave + 4 * g4;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int t = 16 * tb + r16;
            const f32x4 kt = get4(Km, t, j0);
#pragma unroll
            for (int q = 0; q < 4; ++q) ma[tb][q] = (ma[tb][q] + kt[q]) * glast[j0 + q];
            tput4(ob + O::M, C * D, tb * 4 + wave, lane, ma[tb]);
            tput4(ob + O::E_, C * D, tb * 4 + wave, lane, ea[tb] + get4(R, t, j0));
        }
        if (wave == 2) {
            // F[t][u] = Mrk[t][u] + sum_s Mrb[t][s] Z[s][u]; accumulator element (u, t)
            const f32x4 f00 = fmma(mk0, frag_t(Zm, 0, 0, lane), frag_n(Mrb, 0, 0, lane));
            const f32x4 f01 = fmma(mk1, frag_t(Zm, 0, 0, lane), frag_n(Mrb, 16, 0, lane));
            const f32x4 f11 = fmma(mk2, frag_t(Zm, 16, 0, lane), frag_n(Mrb, 16, 0, lane));
            // F tiles (row block, column block): (0, 0), (1, 0), (1, 1)
            tput4(ob + O::F, C * C, 0, lane, f00);
            tput4(ob + O::F, C * C, 2, lane, f01);
            tput4(ob + O::F, C * C, 3, lane, f11);
        } else if (wave == 3) {
            tput4(ob + O::F, C * C, 1, lane, zero4());   // (0, 1): u >= 16 > t
        }
    }
    if (!more) break;
    item = nitem;
    lds_barrier();   // this item's last LDS reads before the next item's writes
  }
}

// --------------------------------------------------------------------- scan
// LDS image of one chunk's operands (operand rows in the Mat format of
// wkv7_device.h: padded rows, hi then lo plane for the split format).
template <bool SPLIT>
struct OpsImage {
    using F = Fmt<SPLIT>;
    static constexpr int P = 0;                        // (j, j')
    static constexpr int M = P + F::bytes(D, D);       // (t, j)
    static constexpr int E = M + F::bytes(C, D);       // (t, j)
    static constexpr int Fm = E + F::bytes(C, D);      // (t, u)
    static constexpr int bytes = Fm + F::bytes(C, C);
};

// One chunk's operand block, global (unpadded) -> registers -> LDS image.
// Thread tid of NT moves the 16-byte units tid + NT * u.  F's tile of
// columns 16-31 in rows 0-15 is zero (F is lower triangular): its units are
// loaded at an offset past the block, so the buffer load returns 0 without
// reading memory and the LDS image gets the zeros.  OpsMap holds the
// thread's (constant) offsets, OpsCopy one chunk's data in registers.
template <bool SPLIT, int NT>
struct OpsMap {
    static constexpr int N16 = kOpsBytes / 16;
    static constexpr int PER = N16 / NT;
    static_assert(N16 % NT == 0, "operand block split");
    int off[PER];  // LDS byte offsets inside a buffer
    int src[PER];  // byte offsets inside the operand block (past it for the zero tile)

    __device__ __forceinline__ void init(int tid) {
        using O = OpsLayout<SPLIT>;
        using I = OpsImage<SPLIT>;
        constexpr int EPU = SPLIT ? 8 : 4;  // storage elements per 16 bytes
        constexpr int ESZ = SPLIT ? 2 : 4;
        constexpr int PAD = Fmt<SPLIT>::pad;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = (tid + NT * u) * EPU;
            int first, lbase, cols, rows;
            if (e < O::M) { first = O::P; lbase = I::P; cols = D; rows = D; }
            else if (e < O::E_) { first = O::M; lbase = I::M; cols = D; rows = C; }
            else if (e < O::F) { first = O::E_; lbase = I::E; cols = D; rows = C; }
            else { first = O::F; lbase = I::Fm; cols = C; rows = C; }
            // local -> (plane, tile, row and column inside the tile) -> image row, column
            const int local = e - first;
            const int plane = local / (rows * cols), rem = local % (rows * cols);
            const int tile = rem >> 8, in = rem & 255;
            const int tr = tile / (cols / 16), tc = tile % (cols / 16);
            const int row = 16 * tr + (in >> 4), col = 16 * tc + (in & 15);
            off[u] = lbase + ((plane * rows + row) * (cols + PAD) + col) * ESZ;
            const bool zero_tile = first == O::F && tile == 1;
            src[u] = zero_tile ? (int)kDropOffset : (tid + NT * u) * 16;
        }
    }
};

// The units u of a thread with (u & 1) == PAR (PAR = -1: every unit; -2:
// none).  Registers of the other units are never touched.  (A split of each
// operand block between the two workgroups of a head, one parity fetched
// early and the partner's parity late as L2 hits, measured no faster.)
template <bool SPLIT, int NT, int PAR>
struct OpsCopy {
    using Map = OpsMap<SPLIT, NT>;
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    static constexpr bool has(int u) { return PAR == -1 || (PAR >= 0 && (u & 1) == PAR); }
    u32x4 v[Map::PER];

    // on == false (a chunk past the last): a size-0 resource, the loads
    // return 0 and touch no memory
    __device__ __forceinline__ void load(const char* base, bool on, const Map& m) {
        const Rsrc r = make_rsrc(base, on ? kOpsBytes : 0u);
#pragma unroll
        for (int u = 0; u < Map::PER; ++u)
            if (has(u)) v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, m.src[u], 0, 0));
    }
    __device__ __forceinline__ void store(char* buf, const Map& m) const {
#pragma unroll
        for (int u = 0; u < Map::PER; ++u)
            if (has(u)) *reinterpret_cast<u32x4*>(buf + m.off[u]) = v[u];
    }
};

// Chunks of operands and token rows in flight per memory thread (register
// sets).  Two cover the load latency: four measured the same (a CU streams
// cold operand blocks at about 12 B/cycle either way) with twice the registers.
constexpr int SCAN_DEPTH = 2;

// Token tensors (v or dy) of up to this many bytes are read into the caches
// in one pass at the start of the scan (see the memory waves).
constexpr uint64_t kTouchBytes = 32ull << 20;

// LDS plan of the scan: double buffers of one chunk's operands, of its
// token rows (v exact, or dy split) and of its output rows (y or dv, fp32).
template <bool SPLIT, int NWV, int NCW>
struct ScanLds {
    using F = Fmt<SPLIT>;
    static constexpr int NI = 16 * NWV;                 // state rows of the workgroup
    static constexpr int OPS = OpsImage<SPLIT>::bytes;
    static constexpr int XB = F::bytes(C, NI);          // rows (t, i)
    static constexpr int LDO = NI + 4;                  // fp32 output row stride
    static constexpr int OB = C * LDO * 4;
    // state halves passed between the two waves of a row block (two column
    // tiles, 16 bytes per lane each), double-buffered by chunk parity
    static constexpr int XW = NCW > NWV ? 2 * 64 * 16 : 0;
    static constexpr int X0 = 2 * OPS, O0 = X0 + 2 * XB, W0 = O0 + 2 * OB;
    static constexpr int total = W0 + 2 * NCW * XW;
    static_assert(total <= 160 * 1024, "scan LDS");
};

// The token rows of one chunk for a workgroup's NI columns, memory ->
// registers -> LDS.  Memory thread ct of NT moves the 16-byte pieces
// (ct + NT * u) mod NPC: piece -> (token t, NPR pieces per token row).  With
// fewer pieces than threads, two threads move the same piece to the same
// place.  Tokens past the end of the sequence read as 0 (buffer resource
// ending at the head's last token).
template <typename XT, bool SPLIT, int NWV, int NT>
struct XCopy {
    static constexpr int NI = 16 * NWV;
    static constexpr int EPP = 16 / (int)sizeof(XT);            // elements per piece
    static constexpr int NPR = NI / EPP;                        // pieces per token row
    static constexpr int NPC = C * NPR;                         // pieces per chunk
    static constexpr int PER = NPC >= NT ? NPC / NT : 1;
    static_assert(NPC % NT == 0 || NT % NPC == 0, "token row split");
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    u32x4 v[PER];

    static __device__ __forceinline__ int piece(int ct, int u) { return (ct + NT * u) % NPC; }
    __device__ __forceinline__ void load(Rsrc r, int c, int HD, int ct) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int pc = piece(ct, u), t = pc / NPR, e0 = (pc % NPR) * EPP;
            // byte offset inside the head's tokens: below 4 GiB, unsigned arithmetic
            const uint32_t off = ((uint32_t)t * HD + e0 + (uint32_t)c * C * HD) * (uint32_t)sizeof(XT);
            v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
        }
    }
    // rows (t, i) of an operand matrix: exact bf16 (v) or split (dy)
    __device__ __forceinline__ void store(Mat<SPLIT> X, int ct) const {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int pc = piece(ct, u), t = pc / NPR, e0 = (pc % NPR) * EPP;
            if constexpr (sizeof(XT) == 2) {
                *reinterpret_cast<u32x4*>(reinterpret_cast<__bf16*>(X.p) + t * X.ld + e0) = v[u];
            } else {
                // The split of the fp32 values is register arithmetic: pin it here, after the
                // preceding barrier, or it is hoisted to where the load was just issued and the
                // wave waits for it there.
                u32x4 w = v[u];
                asm volatile("" : "+v"(w));
                put4(X, t, e0, __builtin_bit_cast(f32x4, w));
            }
        }
    }
};

// Memory waves store one chunk's output rows (fp32, rows t, NI columns)
// from LDS: 16 bytes per piece, NT threads.
template <int NWV, int NT>
__device__ __forceinline__ void store_out(const float* ob, Rsrc r, int c, int HD, int ct) {
    constexpr int NI = 16 * NWV, NPR = NI / 4, PER = C * NPR / NT, LDO = NI + 4;
    static_assert(C * NPR % NT == 0 && PER >= 1, "output row split");
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int pc = ct + NT * u, t = pc / NPR, e0 = (pc % NPR) * 4;
        const uint32_t off = ((uint32_t)t * HD + e0 + (uint32_t)c * C * HD) * 4u;   // below 4 GiB
        bstore4<kStream>(*reinterpret_cast<const f32x4*>(ob + t * LDO + e0), r, (int)off, 0);
    }
}

// BWD = false: forward over v (InT), S from h0 -> y, checkpoints, hT.
// BWD = true : backward over dy (fp32), G from dhT -> dv, dh_ckpt, dh0.
//
// A workgroup has NCW compute waves and NMW memory waves.  Its NWV row
// blocks of 16 state rows go to one compute wave each (NCW = NWV) or to two
// (NCW = 2 NWV): then wave h of a block forms the new state's column tiles
// 2h, 2h + 1 and the output rows of token block h, and the two waves swap
// their new tiles through LDS at the chunk's end.  The products of a chunk
// read the whole previous state, so each wave keeps all four tiles.  The memory waves do all the streaming: the operand block and the
// token rows of chunk it + 1 into LDS while chunk it is computed (loaded two
// chunks ahead into two register sets), and the output rows of chunk it - 1
// from LDS to memory.  The compute waves read LDS, run the products and
// store only the state checkpoints.  Token tensors are addressed through
// per-head buffer resources that end after the head's last token: tokens
// past the end of a ragged last chunk read as 0 and their stores are
// dropped by the hardware, so no branch surrounds a memory access inside the
// chunk loop.
template <typename InT, bool SPLIT, int NWV, int NCW, int NMW, bool BWD>
__global__ __launch_bounds__(64 * (NCW + NMW)) void scan_kernel(ScanArgs p, int xcd) {
    constexpr int NSUB = 4 / NWV, NTC = 64 * NCW, NTM = 64 * NMW;
    constexpr bool HALF = NCW > NWV;   // two waves per row block
    static_assert(NCW == NWV || NCW == 2 * NWV, "compute waves");
    using XT = typename std::conditional<BWD, float, InT>::type;
    using I = OpsImage<SPLIT>;
    using L = ScanLds<SPLIT, NWV, NCW>;
    using M = Mat<SPLIT>;
    using Fr = Frag<SPLIT>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g4 = lane >> 4;
    int head, sub;
    block_map(blockIdx.x, NSUB, xcd != 0, head, sub);
    const int NC = p.NC;
    const int bb = head / p.H, hh = head % p.H;
    const int HD = p.H * D;                                            // token stride (elements)
    const int i0 = 16 * sub * NWV;                                     // the workgroup's first state row
    const int64_t tok0 = (int64_t)bb * p.T * HD + (int64_t)hh * D;     // token 0 of this head
    const uint32_t head_span = (uint32_t)((int64_t)(p.T - 1) * HD + D);  // elements up to its last token
    auto chunk_of = [&](int it) { return BWD ? NC - 1 - it : it; };
    auto xmat = [&](int it) { return make_mat<SPLIT>(smem, L::X0 + (it & 1) * L::XB, C, L::NI); };
    auto obuf = [&](int it) { return reinterpret_cast<float*>(smem + L::O0 + (it & 1) * L::OB); };

    if (wave >= NCW) {
        // ---- memory waves
        const int ct = tid - NTC;
        const char* ops = static_cast<const char*>(p.ops) + (int64_t)head * NC * kOpsBytes;
        auto ops_of = [&](int it) { return ops + (int64_t)chunk_of(min(it, NC - 1)) * kOpsBytes; };
        const Rsrc rx = make_rsrc(static_cast<const XT*>(p.x) + tok0 + i0, head_span * sizeof(XT));
        const Rsrc ro = make_rsrc(p.out ? p.out + tok0 + i0 : nullptr, p.out ? head_span * 4 : 0);
        const Rsrc rnull = make_rsrc(nullptr, 0);
        using Map = OpsMap<SPLIT, NTM>;
        using XC = XCopy<XT, SPLIT, NWV, NTM>;
        Map map;
        map.init(ct);
        // outputs of iteration it - 1 (nothing before the first or past the last)
        auto out = [&](int it) {
            const bool on = it > 0 && it <= NC;
            store_out<NWV, NTM>(obuf(it - 1), on ? ro : rnull, chunk_of(min(max(it - 1, 0), NC - 1)), HD, ct);
        };
        // SCAN_DEPTH register sets: chunk j travels in set j % SCAN_DEPTH
        OpsCopy<SPLIT, NTM, -1> o[SCAN_DEPTH];
        XC x[SCAN_DEPTH];
        auto fetch = [&](auto set_c, int it) {
            constexpr int S = decltype(set_c)::value;
            const bool on = it < NC;
            o[S].load(ops_of(it), on, map);
            x[S].load(on ? rx : rnull, chunk_of(min(it, NC - 1)), HD, ct);
        };
        auto put = [&](auto set_c, int it) {
            constexpr int S = decltype(set_c)::value;
            o[S].store(smem + (it & 1) * L::OPS, map);
            x[S].store(xmat(it), ct);
        };
        using S0 = std::integral_constant<int, 0>;
        fetch(S0{}, 0);
        // A token tensor that the previous kernel did not touch comes from
        // HBM, and each chunk's rows (32 lines at a stride of H D elements)
        // then miss while the operand blocks stream: those misses hold up the
        // operand loads of the whole CU behind them (11 us of the forward and
        // 9 us of the backward scan at B12 T1024 H6 after a cache flush).  A
        // tensor of up to kTouchBytes is therefore read once here, one word
        // per line of this workgroup's columns of every token, by the last
        // memory wave, so that its rows come from the caches; a larger one
        // would not stay cached while the operands stream.  The words go
        // straight to LDS (no registers), all into one 256-byte slot of the
        // second output-row buffer: they complete before this wave's chunk-1
        // rows (a wave's loads complete in order), so before the second
        // barrier, after which the compute waves first write that buffer.
        if (wave == NCW + NMW - 1 && (uint64_t)p.B * (uint64_t)p.T * (uint64_t)p.H * D * sizeof(XT) <= kTouchBytes) {
            constexpr int LPR = (16 * NWV * (int)sizeof(XT) + 127) / 128;   // lines per token row here
            __attribute__((address_space(3))) void* sink =
                (__attribute__((address_space(3))) void*)reinterpret_cast<char*>(obuf(1));
            for (int t0_ = 0; t0_ < p.T; t0_ += 64 * 8) {
#pragma unroll
                for (int u = 0; u < 8; ++u)
#pragma unroll
                    for (int l = 0; l < LPR; ++l)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rx, sink, 4, (int)((uint32_t)(t0_ + 64 * u + lane) * (uint32_t)HD * sizeof(XT) + 128u * l),
                            0, 0, 0);
            }
        }
        put(S0{}, 0);
        // Chunks 1 .. SCAN_DEPTH go out in order, so that the count of
        // outstanding loads at each put is exact (loads complete in order).
        static_for<SCAN_DEPTH>([&](auto s_c) {
            constexpr int S = decltype(s_c)::value;
            fetch(std::integral_constant<int, (S + 1) % SCAN_DEPTH>{}, S + 1);
        });
        lds_barrier();
        // SCAN_DEPTH iterations per trip, straight-line code (every wait
        // counted exactly).  In iteration it: chunk it + 1 goes into the
        // buffers the compute waves finished reading in iteration it - 1, its
        // register set is refilled with chunk it + 1 + SCAN_DEPTH, and the
        // outputs of chunk it - 1 go to memory.  The trip count is rounded up
        // to a multiple of SCAN_DEPTH; the compute waves match the extra
        // barriers.  Chunks past the last load nothing (size-0 resources).
        auto iter = [&](auto u_c, int it) {
            using S = std::integral_constant<int, (decltype(u_c)::value + 1) % SCAN_DEPTH>;
            put(S{}, it + 1);
            fetch(S{}, it + 1 + SCAN_DEPTH);
            out(it);
            lds_barrier();
        };
        const int trips = (NC + SCAN_DEPTH - 1) / SCAN_DEPTH;
        for (int tr = 0; tr < trips; ++tr)
            static_for<SCAN_DEPTH>([&](auto u_c) { iter(u_c, tr * SCAN_DEPTH + decltype(u_c)::value); });
        if (trips * SCAN_DEPTH == NC) out(NC);
        return;
    }

    // ---- compute waves
    const int rb = HALF ? wave % NWV : wave;    // row block: state rows n0 .. n0 + 15
    const int n0 = i0 + 16 * rb;
    const int roff = (n0 + r16) * D + 4 * g4;                          // this lane's part of a D x D state
    const int64_t soff = (int64_t)head * D * D + roff;
    // Checkpoints (or state gradients) of this head: one buffer resource per
    // chunk, based at that chunk's D x D block with a 64-bit address, so the
    // per-lane offset stays below 16 KiB for any number of chunks.
    float* const cbase = p.ckpt ? p.ckpt + (int64_t)head * NC * D * D : nullptr;
    auto ckpt_rsrc = [&](int c) {
        return make_rsrc(cbase ? cbase + (int64_t)c * D * D : nullptr, cbase ? D * D * 4 : 0);
    };

    // The loop for half HF (0 when the row block has one wave): straight-line
    // code, so the products' independent chains interleave.
    auto run = [&](auto hf_c) {
        constexpr int HF = decltype(hf_c)::value;
        constexpr bool YA = !HALF || HF == 0, YB = !HALF || HF == 1;   // token blocks 0-15, 16-31
        auto mine = [](int m) { return !HALF || (m >> 1) == HF; };      // column tiles formed here
        auto xbuf = [&](int it, int w) {
            return reinterpret_cast<f32x4*>(smem + L::W0 + ((it & 1) * NCW + w) * L::XW);
        };
        // state rows n0 + r: st[m][q] = X[n0 + r][16m + 4g + q]
        f32x4 st[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
            st[m] = p.s0 ? *reinterpret_cast<const f32x4*>(p.s0 + soff + 16 * m) : zero4();
        lds_barrier();

        for (int it = 0; it < NC; ++it) {
            const int c = chunk_of(it);
            const Rsrc rc = ckpt_rsrc(c);
            if constexpr (!BWD) {   // checkpoint c: the state entering the chunk
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (mine(m)) bstore4(st[m], rc, (roff + 16 * m) * 4, 0);
            }
            char* lb = smem + (it & 1) * L::OPS;
            const M Pm = make_mat<SPLIT>(lb, I::P, D, D), Mm = make_mat<SPLIT>(lb, I::M, C, D);
            const M Em = make_mat<SPLIT>(lb, I::E, C, D), Fm = make_mat<SPLIT>(lb, I::Fm, C, C);
            const M Xm = xmat(it);
            float* ob = obuf(it);
            const Fr s0f = frag_acc<SPLIT>(st[0], st[1]), s1f = frag_acc<SPLIT>(st[2], st[3]);
            f32x4 ya = zero4(), yb = zero4();
            if constexpr (!BWD) {
                const Fr vf = frag_t_exact(Xm, 16 * rb, 0, lane);
                // S_end^T[j'][i] = sum_j P[j][j'] S[i][j] + sum_t M[t][j'] V[t][i]
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    if (!mine(m)) continue;
                    f32x4 a = fmma(zero4(), frag_t(Pm, 16 * m, 0, lane), s0f);
                    a = fmma(a, frag_t(Pm, 16 * m, 32, lane), s1f);
                    st[m] = fmma<false, true>(a, frag_t(Mm, 16 * m, 0, lane), vf);
                }
                // Y[t][i] = sum_j E[t][j] S[i][j] + sum_s F[t][s] V[s][i]
                if constexpr (YA) {
                    ya = fmma(zero4(), frag_n(Em, 0, 0, lane), s0f);
                    ya = fmma(ya, frag_n(Em, 0, 32, lane), s1f);
                    ya = fmma<false, true>(ya, frag_n(Fm, 0, 0, lane), vf);
                }
                if constexpr (YB) {
                    yb = fmma(zero4(), frag_n(Em, 16, 0, lane), s0f);
                    yb = fmma(yb, frag_n(Em, 16, 32, lane), s1f);
                    yb = fmma<false, true>(yb, frag_n(Fm, 16, 0, lane), vf);
                }
            } else {
                const Fr df = frag_t(Xm, 16 * rb, 0, lane);
                // dv[t][i] = sum_j M[t][j] G[i][j] + sum_u F[u][t] DY[u][i]
                if constexpr (YA) {
                    ya = fmma(zero4(), frag_n(Mm, 0, 0, lane), s0f);
                    ya = fmma(ya, frag_n(Mm, 0, 32, lane), s1f);
                    ya = fmma(ya, frag_t(Fm, 0, 0, lane), df);
                }
                if constexpr (YB) {
                    yb = fmma(zero4(), frag_n(Mm, 16, 0, lane), s0f);
                    yb = fmma(yb, frag_n(Mm, 16, 32, lane), s1f);
                    yb = fmma(yb, frag_t(Fm, 16, 0, lane), df);
                }
                // G_start^T[j'][i] = sum_j P[j'][j] G[i][j] + sum_t E[t][j'] DY[t][i]
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    if (!mine(m)) continue;
                    f32x4 a = fmma(zero4(), frag_n(Pm, 16 * m, 0, lane), s0f);
                    a = fmma(a, frag_n(Pm, 16 * m, 32, lane), s1f);
                    st[m] = fmma(a, frag_t(Em, 16 * m, 0, lane), df);
                }
                // gradient w.r.t. the state entering chunk c
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (mine(m)) bstore4(st[m], rc, (roff + 16 * m) * 4, 0);
            }
            // output rows (t, i) of this chunk for the memory waves
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (YA) ob[(4 * g4 + q) * L::LDO + 16 * rb + r16] = ya[q];
                if constexpr (YB) ob[(16 + 4 * g4 + q) * L::LDO + 16 * rb + r16] = yb[q];
            }
            if constexpr (HALF) {   // this wave's new tiles for the other wave of the row block
                f32x4* x = xbuf(it, wave);
                x[lane] = st[2 * HF];
                x[64 + lane] = st[2 * HF + 1];
            }
            lds_barrier();
            if constexpr (HALF) {
                const f32x4* x = xbuf(it, rb + NWV * (1 - HF));
                st[2 * (1 - HF)] = x[lane];
                st[2 * (1 - HF) + 1] = x[64 + lane];
            }
        }
        for (int e = NC; e < (NC + SCAN_DEPTH - 1) / SCAN_DEPTH * SCAN_DEPTH; ++e)
            lds_barrier();   // the memory waves' last trip
        if (p.sT) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
                if (mine(m)) *reinterpret_cast<f32x4*>(p.sT + soff + 16 * m) = st[m];
        }
    };
    if (!HALF || wave < NWV) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
}

template <typename InT, bool SPLIT, bool PROJ>
hipError_t launch_prepare_typed(const PrepArgs& a, hipStream_t s) {
    using L = PrepSmem<SPLIT>;
    auto kern = chunk_prepare_kernel<InT, SPLIT, PROJ>;
    static PerDeviceOnce once;
    hipError_t e = set_smem_once(once, kern, L::total);
    if (e != hipSuccess) return e;
    int n_cu = 0;
    e = device_cus(&n_cu);
    if (e != hipSuccess) return e;
    const int items = a.B * a.H * a.NC;
    const int grid = items < 2 * n_cu ? items : 2 * n_cu;   // two workgroups per CU
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), L::total, s, a, items);
    return hipGetLastError();
}

template <typename InT, bool SPLIT, int NWV, int NCW, int NMW, bool BWD>
hipError_t launch_scan_typed(const ScanArgs& a, hipStream_t s) {
    constexpr int smem_bytes = ScanLds<SPLIT, NWV, NCW>::total;
    auto kern = scan_kernel<InT, SPLIT, NWV, NCW, NMW, BWD>;
    static PerDeviceOnce once;
    const hipError_t e = set_smem_once(once, kern, smem_bytes);
    if (e != hipSuccess) return e;
    const int heads = a.B * a.H;
    const bool xcd = heads % 8 == 0;
    hipLaunchKernelGGL(kern, dim3(heads * (4 / NWV)), dim3(64 * (NCW + NMW)), smem_bytes, s, a, xcd ? 1 : 0);
    return hipGetLastError();
}

template <typename InT, bool SPLIT, bool BWD>
hipError_t launch_scan_nwv(const ScanArgs& a, hipStream_t s) {
    // A head's 64 state rows go to as many workgroups as the CUs allow, one
    // workgroup per CU: four of 16 rows (two compute, two memory waves),
    // two of 32 rows (four and four) or one of 64.  Every workgroup streams
    // the head's whole operand block, but a CU with fewer compute waves
    // reads less of it from LDS per chunk (B4 T512 H12, 48 heads: four
    // workgroups 21.0 / 21.9 us against two 22.1 / 24.1 us, forward /
    // backward); two workgroups on one CU stream twice (B12 T1024 H6, 72
    // heads on 288 workgroups: 59 against 37 us).
    int n_cu = 0;
    const hipError_t e = device_cus(&n_cu);
    if (e != hipSuccess) return e;
    const int heads = a.B * a.H;
    if (4 * heads <= n_cu) return launch_scan_typed<InT, SPLIT, 1, 2, 2, BWD>(a, s);
    if (2 * heads <= n_cu) return launch_scan_typed<InT, SPLIT, 2, 4, 4, BWD>(a, s);
    return launch_scan_typed<InT, SPLIT, 4, 4, 4, BWD>(a, s);
}

}  // namespace

hipError_t launch_chunk_prepare(const PrepArgs& a, bool bf16, bool proj, hipStream_t s) {
    if (proj) {
        if (bf16) return launch_prepare_typed<uint16_t, true, true>(a, s);
        return launch_prepare_typed<float, false, true>(a, s);
    }
    if (bf16) return launch_prepare_typed<uint16_t, true, false>(a, s);
    return launch_prepare_typed<float, false, false>(a, s);
}

hipError_t launch_scan(const ScanArgs& a, bool bf16, bool bwd, hipStream_t s) {
    if (bf16) return bwd ? launch_scan_nwv<uint16_t, true, true>(a, s) : launch_scan_nwv<uint16_t, true, false>(a, s);
    return bwd ? launch_scan_nwv<float, false, true>(a, s) : launch_scan_nwv<float, false, false>(a, s);
}

}  // namespace wkv7
