// wkv7_api.hip -- the C ABI of libwkv7 (declared in include/wkv7.h):
// argument checks on the host, then kernel launches on the caller's stream.
#include <stdint.h>

#include "wkv7.h"
#include "wkv7_internal.h"

namespace {

// Scratch of wkv7_fwd_noalloc: the chunk operands of one forward call live in
// this file-scope device array instead of a caller-supplied workspace.  Every
// GPU the library runs on holds its own copy until the process ends.  Host
// code never uses the array's name as an address: the device address of each
// GPU's copy comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = size_t(128) << 20;
__device__ __align__(256) char scratch[kScratchBytes];

struct ScratchAddr {
    wkv7::PerDeviceOnce once;
    void* ptr[wkv7::kMaxDevices] = {};
};

// The current device's copy of `scratch` (nullptr and an error on failure).
hipError_t scratch_address(void** out) {
    static ScratchAddr sa;
    hipError_t e = sa.once.run([&](int d) {   // with device d current
        void* p = nullptr;
        const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (r == hipSuccess) sa.ptr[d] = p;   // published by run() before it reports success
        return r;
    });
    int dev = 0;
    if (e == hipSuccess) e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    *out = sa.ptr[dev];
    return *out ? hipSuccess : hipErrorInvalidSymbol;
}

constexpr int kVersion = 100;  // 0.1.0
constexpr int kD = 64;
constexpr int kChunk = 32;
// wkv7_fwd evaluates sequences of at most this many tokens token by token.
constexpr int kSequentialMaxT = 1;

struct Span {
    uintptr_t lo, hi;  // [lo, hi); empty if lo == hi
};

Span span(const void* p, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{lo, p ? lo + static_cast<uintptr_t>(bytes) : lo};
}

bool overlaps(Span a, Span b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Sizes {
    int64_t heads, nc, tok_elems, state_elems, ckpt_elems;
};

wkv7_status check_shape(int B, int T, int H, int D, Sizes* sz) {
    if (D != kD || B < 1 || T < 1 || H < 1) return WKV7_ERR_SHAPE;
    const int64_t heads = (int64_t)B * H;
    const int64_t nc = ((int64_t)T + kChunk - 1) / kChunk;
    // Grid sizes (heads * NC workgroups at most) must fit a 32-bit launch.
    if (heads * nc * 4 > INT32_MAX || heads * 4 > INT32_MAX) return WKV7_ERR_SHAPE;
    const int64_t tok = heads * (int64_t)T * kD;
    if (tok / T != heads * kD) return WKV7_ERR_SHAPE;
    if (tok > (INT64_MAX / 8)) return WKV7_ERR_SHAPE;
    // every token tensor, taken as fp32, is addressed with 32-bit byte offsets
    if (tok * 4 > (int64_t)wkv7::kMaxTensorBytes) return WKV7_ERR_SHAPE;
    sz->heads = heads;
    sz->nc = nc;
    sz->tok_elems = tok;
    sz->state_elems = heads * kD * kD;
    sz->ckpt_elems = heads * nc * kD * kD;
    if (sz->ckpt_elems > (INT64_MAX / 8)) return WKV7_ERR_SHAPE;
    return WKV7_OK;
}

int elem_size(wkv7_dtype dt) { return dt == WKV7_BF16 ? 2 : 4; }

wkv7_status check_dtype(int dt) { return (dt == WKV7_F32 || dt == WKV7_BF16) ? WKV7_OK : WKV7_ERR_DTYPE; }

// One buffer argument of an entry point.
struct Buf {
    const void* p;
    int64_t bytes;
    bool required;
    bool output;
};

// NULL and alignment checks over all buffers of a call.
wkv7_status check_bufs(const Buf* bufs, int n) {
    for (int i = 0; i < n; ++i)
        if (bufs[i].required && !bufs[i].p) return WKV7_ERR_ARG;
    for (int i = 0; i < n; ++i)
        if (bufs[i].p && !aligned16(bufs[i].p)) return WKV7_ERR_ALIGN;
    return WKV7_OK;
}

// Outputs may not overlap any other buffer; the one exception is
// `same_ok_a` == `same_ok_b` (the in-place state update): those two buffers
// may be the very same pointer.
wkv7_status check_alias(const Buf* bufs, int n, const void* same_ok_a = nullptr,
                        const void* same_ok_b = nullptr) {
    for (int i = 0; i < n; ++i) {
        if (!bufs[i].output || !bufs[i].p) continue;
        const Span si = span(bufs[i].p, bufs[i].bytes);
        for (int j = 0; j < n; ++j) {
            if (j == i || !bufs[j].p) continue;
            if (bufs[j].output && j < i) continue;  // pair already checked
            const bool exempt = same_ok_a && same_ok_a == same_ok_b &&
                                ((bufs[i].p == same_ok_a && bufs[j].p == same_ok_b) ||
                                 (bufs[j].p == same_ok_a && bufs[i].p == same_ok_b));
            if (exempt) continue;
            if (overlaps(si, span(bufs[j].p, bufs[j].bytes))) return WKV7_ERR_ALIAS;
        }
    }
    return WKV7_OK;
}

// Shared checks of the forward entry points.
wkv7_status check_fwd(int B, int T, int H, int D, wkv7_dtype dt, const void* r, const void* w,
                      const void* k, const void* v, const void* a, const void* b, const float* h0,
                      const float* y, const float* ckpt, const float* hT, Sizes* sz) {
    wkv7_status st = check_dtype(dt);
    if (st != WKV7_OK) return st;
    st = check_shape(B, T, H, D, sz);
    if (st != WKV7_OK) return st;
    const int64_t tin = sz->tok_elems * elem_size(dt), t32 = sz->tok_elems * 4, s32 = sz->state_elems * 4;
    const Buf bufs[10] = {{r, tin, true, false},  {w, tin, true, false},  {k, tin, true, false},
                          {v, tin, true, false},  {a, tin, true, false},  {b, tin, true, false},
                          {h0, s32, false, false}, {y, t32, false, true}, {ckpt, sz->ckpt_elems * 4, false, true},
                          {hT, s32, false, true}};
    st = check_bufs(bufs, 10);
    if (st != WKV7_OK) return st;
    if (!y && !ckpt && !hT) return WKV7_ERR_ARG;
    return check_alias(bufs, 10, h0, hT);
}

wkv7::FwdArgs fwd_args(int B, int T, int H, const Sizes& sz, const void* r, const void* w,
                       const void* k, const void* v, const void* a, const void* b, const float* inv,
                       const float* h0, float* y, float* ckpt, float* hT) {
    wkv7::FwdArgs fa;
    fa.r = r; fa.w = w; fa.k = k; fa.v = v; fa.a = a; fa.b = b;
    fa.inv = inv; fa.h0 = h0; fa.y = y; fa.ckpt = ckpt; fa.hT = hT;
    fa.B = B; fa.T = T; fa.H = H; fa.NC = (int)sz.nc;
    return fa;
}

wkv7::BwdArgs bwd_args(int B, int T, int H, const Sizes& sz, const float* dy, const float* dhT,
                       const void* r, const void* w, const void* k, const void* v, const void* a,
                       const void* b, const float* inv, const float* h_ckpt, float* dh_ckpt) {
    wkv7::BwdArgs ba = {};
    ba.r = r; ba.w = w; ba.k = k; ba.v = v; ba.a = a; ba.b = b; ba.inv = inv;
    ba.dy = dy; ba.dhT = dhT; ba.ckpt = h_ckpt; ba.gbuf = dh_ckpt;
    ba.B = B; ba.T = T; ba.H = H; ba.NC = (int)sz.nc;
    return ba;
}

wkv7_status status_of(hipError_t e) { return e == hipSuccess ? WKV7_OK : WKV7_ERR_HIP; }

// chunk_ops: the (I - Lab)^-1 of every chunk (fp32 32 x 32), then the
// transition operands of every chunk (kOpsBytes each).
int64_t inv_bytes(const Sizes& sz) { return sz.heads * sz.nc * kChunk * kChunk * 4; }
int64_t ops_bytes(const Sizes& sz) { return inv_bytes(sz) + sz.heads * sz.nc * wkv7::kOpsBytes; }

wkv7_status launch_prepare(int B, int T, int H, const Sizes& sz, bool bf16, bool proj, const void* r,
                           const void* w, const void* k, const void* a, const void* b, void* chunk_ops,
                           hipStream_t s) {
    wkv7::PrepArgs pa;
    pa.r = r; pa.w = w; pa.k = k; pa.a = a; pa.b = b;
    pa.inv = static_cast<float*>(chunk_ops);
    pa.ops = static_cast<char*>(chunk_ops) + inv_bytes(sz);
    pa.B = B; pa.T = T; pa.H = H; pa.NC = (int)sz.nc;
    return status_of(wkv7::launch_chunk_prepare(pa, bf16, proj, s));
}

wkv7_status launch_scan(int B, int T, int H, const Sizes& sz, bool bf16, bool bwd, const void* x,
                        const void* chunk_ops, const float* s0, float* out, float* ckpt, float* sT,
                        hipStream_t s) {
    wkv7::ScanArgs sa;
    sa.x = x;
    sa.ops = static_cast<const char*>(chunk_ops) + inv_bytes(sz);
    sa.s0 = s0; sa.out = out; sa.ckpt = ckpt; sa.sT = sT;
    sa.B = B; sa.T = T; sa.H = H; sa.NC = (int)sz.nc;
    return status_of(wkv7::launch_scan(sa, bf16, bwd, s));
}

}  // namespace

extern "C" {

int wkv7_version(void) { return kVersion; }

int wkv7_chunk_len(void) { return kChunk; }

int64_t wkv7_num_chunks(int64_t T) { return T < 1 ? 0 : (T + kChunk - 1) / kChunk; }

const char* wkv7_status_str(int status) {
    switch (status) {
        case WKV7_OK: return "WKV7_OK";
        case WKV7_ERR_ARG: return "WKV7_ERR_ARG: a required pointer is NULL or an argument is invalid";
        case WKV7_ERR_SHAPE: return "WKV7_ERR_SHAPE: D must be 64 and B, T, H at least 1 (and sizes must fit)";
        case WKV7_ERR_DTYPE: return "WKV7_ERR_DTYPE: in_dtype must be WKV7_F32 or WKV7_BF16";
        case WKV7_ERR_ALIGN: return "WKV7_ERR_ALIGN: every pointer must be 16-byte aligned";
        case WKV7_ERR_ALIAS: return "WKV7_ERR_ALIAS: an output overlaps an input or another output";
        case WKV7_ERR_HIP: return "WKV7_ERR_HIP: kernel launch failed";
        case WKV7_ERR_WORKSPACE: return "WKV7_ERR_WORKSPACE: workspace missing or too small";
        default: return "WKV7: unknown status";
    }
}

size_t wkv7_chunk_ops_bytes(int B, int T, int H, int D) {
    Sizes sz;
    if (check_shape(B, T, H, D, &sz) != WKV7_OK) return 0;
    return (size_t)ops_bytes(sz);
}

size_t wkv7_fwd_workspace_bytes(int B, int T, int H, int D) {
    Sizes sz;
    if (check_shape(B, T, H, D, &sz) != WKV7_OK) return 0;
    return T <= kSequentialMaxT ? 0 : (size_t)ops_bytes(sz);
}

size_t wkv7_bwd_workspace_bytes(int B, int T, int H, int D) {
    Sizes sz;
    if (check_shape(B, T, H, D, &sz) != WKV7_OK) return 0;
    return (size_t)(sz.ckpt_elems * 4 + ops_bytes(sz));
}

wkv7_status wkv7_chunk_prepare(int B, int T, int H, int D, wkv7_dtype in_dtype, const void* r, const void* w,
                               const void* k, const void* a, const void* b, void* chunk_ops, void* stream) {
    wkv7_status st = check_dtype(in_dtype);
    if (st != WKV7_OK) return st;
    Sizes sz;
    st = check_shape(B, T, H, D, &sz);
    if (st != WKV7_OK) return st;
    const int64_t tin = sz.tok_elems * elem_size(in_dtype);
    const Buf bufs[6] = {{r, tin, true, false}, {w, tin, true, false}, {k, tin, true, false},
                         {a, tin, true, false}, {b, tin, true, false}, {chunk_ops, ops_bytes(sz), true, true}};
    st = check_bufs(bufs, 6);
    if (st != WKV7_OK) return st;
    st = check_alias(bufs, 6);
    if (st != WKV7_OK) return st;
    return launch_prepare(B, T, H, sz, in_dtype == WKV7_BF16, false, r, w, k, a, b, chunk_ops,
                          static_cast<hipStream_t>(stream));
}

wkv7_status wkv7_fwd_scan(int B, int T, int H, int D, wkv7_dtype in_dtype, const void* v, const void* chunk_ops,
                          const float* h0, float* y, float* h_ckpt, float* hT, void* stream) {
    wkv7_status st = check_dtype(in_dtype);
    if (st != WKV7_OK) return st;
    Sizes sz;
    st = check_shape(B, T, H, D, &sz);
    if (st != WKV7_OK) return st;
    const int64_t tin = sz.tok_elems * elem_size(in_dtype), s32 = sz.state_elems * 4;
    const Buf bufs[6] = {{v, tin, true, false},  {chunk_ops, ops_bytes(sz), true, false},
                         {h0, s32, false, false}, {y, sz.tok_elems * 4, false, true},
                         {h_ckpt, sz.ckpt_elems * 4, false, true}, {hT, s32, false, true}};
    st = check_bufs(bufs, 6);
    if (st != WKV7_OK) return st;
    if (!y && !h_ckpt && !hT) return WKV7_ERR_ARG;
    st = check_alias(bufs, 6, h0, hT);
    if (st != WKV7_OK) return st;
    return launch_scan(B, T, H, sz, in_dtype == WKV7_BF16, false, v, chunk_ops, h0, y, h_ckpt, hT,
                       static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// wkv7_fwd and wkv7_fwd_proj (proj: w, a, b hold w_raw, kappa, alpha)
wkv7_status fwd_impl(int B, int T, int H, int D, wkv7_dtype in_dtype, bool proj, const void* r, const void* w,
                     const void* k, const void* v, const void* a, const void* b, const float* h0,
                     float* y, float* h_ckpt, float* hT, void* workspace, size_t workspace_bytes,
                     void* stream) {
    Sizes sz;
    wkv7_status st = check_fwd(B, T, H, D, in_dtype, r, w, k, v, a, b, h0, y, h_ckpt, hT, &sz);
    if (st != WKV7_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf16 = in_dtype == WKV7_BF16;
    if (T <= kSequentialMaxT) {
        const wkv7::FwdArgs fa = fwd_args(B, T, H, sz, r, w, k, v, a, b, nullptr, h0, y, h_ckpt, hT);
        return status_of(wkv7::launch_fwd_sequential(fa, bf16, proj, s));
    }
    if (workspace && !aligned16(workspace)) return WKV7_ERR_ALIGN;
    if (!workspace || workspace_bytes < (size_t)ops_bytes(sz)) return WKV7_ERR_WORKSPACE;
    const int64_t tin = sz.tok_elems * elem_size(in_dtype);
    const Buf bufs[11] = {{r, tin, true, false},   {w, tin, true, false},  {k, tin, true, false},
                          {v, tin, true, false},   {a, tin, true, false},  {b, tin, true, false},
                          {h0, sz.state_elems * 4, false, false},
                          {y, sz.tok_elems * 4, false, true}, {h_ckpt, sz.ckpt_elems * 4, false, true},
                          {hT, sz.state_elems * 4, false, true}, {workspace, ops_bytes(sz), true, true}};
    st = check_alias(bufs, 11, h0, hT);
    if (st != WKV7_OK) return st;
    st = launch_prepare(B, T, H, sz, bf16, proj, r, w, k, a, b, workspace, s);
    if (st != WKV7_OK) return st;
    return launch_scan(B, T, H, sz, bf16, false, v, workspace, h0, y, h_ckpt, hT, s);
}

// wkv7_bwd and wkv7_bwd_proj (proj: w, a, b hold w_raw, kappa, alpha, and dw, da, db
// receive dw_raw, dkappa, dalpha)
wkv7_status bwd_impl(int B, int T, int H, int D, wkv7_dtype in_dtype, bool proj, const float* dy,
                     const float* dhT, const void* r, const void* w, const void* k, const void* v, const void* a,
                     const void* b, const float* h_ckpt, float* dr, float* dw, float* dk, float* dv,
                     float* da, float* db, float* dh0, void* workspace, size_t workspace_bytes,
                     void* stream) {
    wkv7_status st = check_dtype(in_dtype);
    if (st != WKV7_OK) return st;
    Sizes sz;
    st = check_shape(B, T, H, D, &sz);
    if (st != WKV7_OK) return st;
    const int64_t tin = sz.tok_elems * elem_size(in_dtype), t32 = sz.tok_elems * 4, s32 = sz.state_elems * 4;
    const int64_t c32 = sz.ckpt_elems * 4;
    const int64_t need = c32 + ops_bytes(sz);
    const Buf bufs[17] = {{dy, t32, true, false}, {dhT, s32, false, false}, {r, tin, true, false},
                          {w, tin, true, false},  {k, tin, true, false},    {v, tin, true, false},
                          {a, tin, true, false},  {b, tin, true, false},    {h_ckpt, c32, true, false},
                          {dr, t32, true, true},  {dw, t32, true, true},    {dk, t32, true, true},
                          {dv, t32, true, true},  {da, t32, true, true},    {db, t32, true, true},
                          {dh0, s32, false, true}, {workspace, need, false, true}};
    st = check_bufs(bufs, 17);
    if (st != WKV7_OK) return st;
    if (!workspace || workspace_bytes < (size_t)need) return WKV7_ERR_WORKSPACE;
    st = check_alias(bufs, 17);
    if (st != WKV7_OK) return st;
    float* gbuf = static_cast<float*>(workspace);
    void* ops = gbuf + sz.ckpt_elems;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf16 = in_dtype == WKV7_BF16;
    st = launch_prepare(B, T, H, sz, bf16, proj, r, w, k, a, b, ops, s);
    if (st != WKV7_OK) return st;
    st = launch_scan(B, T, H, sz, bf16, true, dy, ops, dhT, dv, gbuf, dh0, s);
    if (st != WKV7_OK) return st;
    wkv7::BwdArgs ba = bwd_args(B, T, H, sz, dy, dhT, r, w, k, v, a, b, static_cast<const float*>(ops), h_ckpt,
                                gbuf);
    ba.dr = dr; ba.dw = dw; ba.dk = dk; ba.da = da; ba.db = db;
    return status_of(wkv7::launch_bwd_inputs(ba, bf16, proj, s));
}

}  // namespace

extern "C" {

wkv7_status wkv7_fwd(int B, int T, int H, int D, wkv7_dtype in_dtype, const void* r, const void* w,
                     const void* k, const void* v, const void* a, const void* b, const float* h0,
                     float* y, float* h_ckpt, float* hT, void* workspace, size_t workspace_bytes,
                     void* stream) {
    return fwd_impl(B, T, H, D, in_dtype, false, r, w, k, v, a, b, h0, y, h_ckpt, hT, workspace, workspace_bytes,
                    stream);
}

wkv7_status wkv7_fwd_proj(int B, int T, int H, int D, wkv7_dtype in_dtype, const void* r, const void* w_raw,
                          const void* k, const void* v, const void* kappa, const void* alpha, const float* h0,
                          float* y, float* h_ckpt, float* hT, void* workspace, size_t workspace_bytes,
                          void* stream) {
    return fwd_impl(B, T, H, D, in_dtype, true, r, w_raw, k, v, kappa, alpha, h0, y, h_ckpt, hT, workspace,
                    workspace_bytes, stream);
}

size_t wkv7_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

wkv7_status wkv7_fwd_noalloc(int B, int T, int H, int D, wkv7_dtype in_dtype, const void* r, const void* w,
                             const void* k, const void* v, const void* a, const void* b, const float* h0,
                             float* y, float* h_ckpt, float* hT, void* stream) {
    Sizes sz;
    wkv7_status st = check_fwd(B, T, H, D, in_dtype, r, w, k, v, a, b, h0, y, h_ckpt, hT, &sz);
    if (st != WKV7_OK) return st;
    if (T <= kSequentialMaxT)   // the one-token path uses no scratch
        return fwd_impl(B, T, H, D, in_dtype, false, r, w, k, v, a, b, h0, y, h_ckpt, hT, nullptr, 0, stream);
    if ((size_t)ops_bytes(sz) > kScratchBytes) return WKV7_ERR_WORKSPACE;
    void* ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return WKV7_ERR_HIP;
    // every byte of the chunk operands is written by the prepare kernel before
    // the scan reads it, so the scratch needs no clearing
    return fwd_impl(B, T, H, D, in_dtype, false, r, w, k, v, a, b, h0, y, h_ckpt, hT, ws, kScratchBytes, stream);
}

wkv7_status wkv7_fwd_sequential(int B, int T, int H, int D, wkv7_dtype in_dtype, const void* r,
                                const void* w, const void* k, const void* v, const void* a,
                                const void* b, const float* h0, float* y, float* h_ckpt, float* hT,
                                void* stream) {
    Sizes sz;
    wkv7_status st = check_fwd(B, T, H, D, in_dtype, r, w, k, v, a, b, h0, y, h_ckpt, hT, &sz);
    if (st != WKV7_OK) return st;
    const wkv7::FwdArgs fa = fwd_args(B, T, H, sz, r, w, k, v, a, b, nullptr, h0, y, h_ckpt, hT);
    return status_of(wkv7::launch_fwd_sequential(fa, in_dtype == WKV7_BF16, false, static_cast<hipStream_t>(stream)));
}

wkv7_status wkv7_bwd_scan(int B, int T, int H, int D, wkv7_dtype in_dtype, const float* dy, const float* dhT,
                          const void* chunk_ops, float* dh_ckpt, float* dv, float* dh0, void* stream) {
    wkv7_status st = check_dtype(in_dtype);
    if (st != WKV7_OK) return st;
    Sizes sz;
    st = check_shape(B, T, H, D, &sz);
    if (st != WKV7_OK) return st;
    const int64_t t32 = sz.tok_elems * 4, s32 = sz.state_elems * 4;
    const Buf bufs[6] = {{dy, t32, true, false},  {dhT, s32, false, false}, {chunk_ops, ops_bytes(sz), true, false},
                         {dh_ckpt, sz.ckpt_elems * 4, true, true}, {dv, t32, false, true}, {dh0, s32, false, true}};
    st = check_bufs(bufs, 6);
    if (st != WKV7_OK) return st;
    st = check_alias(bufs, 6);
    if (st != WKV7_OK) return st;
    return launch_scan(B, T, H, sz, in_dtype == WKV7_BF16, true, dy, chunk_ops, dhT, dv, dh_ckpt, dh0,
                       static_cast<hipStream_t>(stream));
}

wkv7_status wkv7_bwd_inputs(int B, int T, int H, int D, wkv7_dtype in_dtype, const float* dy,
                            const float* dhT, const void* r, const void* w, const void* k, const void* v,
                            const void* a, const void* b, const void* chunk_ops, const float* h_ckpt,
                            const float* dh_ckpt, float* dr, float* dw, float* dk, float* da, float* db,
                            void* stream) {
    wkv7_status st = check_dtype(in_dtype);
    if (st != WKV7_OK) return st;
    Sizes sz;
    st = check_shape(B, T, H, D, &sz);
    if (st != WKV7_OK) return st;
    const int64_t tin = sz.tok_elems * elem_size(in_dtype), t32 = sz.tok_elems * 4, s32 = sz.state_elems * 4;
    const int64_t c32 = sz.ckpt_elems * 4;
    const Buf bufs[16] = {{dy, t32, true, false},  {dhT, s32, false, false}, {r, tin, true, false},
                          {w, tin, true, false},   {k, tin, true, false},    {v, tin, true, false},
                          {a, tin, true, false},   {b, tin, true, false},    {chunk_ops, ops_bytes(sz), true, false},
                          {h_ckpt, c32, true, false}, {dh_ckpt, c32, true, false}, {dr, t32, true, true},
                          {dw, t32, true, true},   {dk, t32, true, true},    {da, t32, true, true},
                          {db, t32, true, true}};
    st = check_bufs(bufs, 16);
    if (st != WKV7_OK) return st;
    st = check_alias(bufs, 16);
    if (st != WKV7_OK) return st;
    wkv7::BwdArgs ba = bwd_args(B, T, H, sz, dy, dhT, r, w, k, v, a, b, static_cast<const float*>(chunk_ops),
                                h_ckpt, const_cast<float*>(dh_ckpt));
    ba.dr = dr; ba.dw = dw; ba.dk = dk; ba.da = da; ba.db = db;
    return status_of(wkv7::launch_bwd_inputs(ba, in_dtype == WKV7_BF16, false, static_cast<hipStream_t>(stream)));
}

wkv7_status wkv7_bwd(int B, int T, int H, int D, wkv7_dtype in_dtype, const float* dy, const float* dhT,
                     const void* r, const void* w, const void* k, const void* v, const void* a,
                     const void* b, const float* h_ckpt, float* dr, float* dw, float* dk, float* dv,
                     float* da, float* db, float* dh0, void* workspace, size_t workspace_bytes,
                     void* stream) {
    return bwd_impl(B, T, H, D, in_dtype, false, dy, dhT, r, w, k, v, a, b, h_ckpt, dr, dw, dk, dv, da, db, dh0,
                    workspace, workspace_bytes, stream);
}

wkv7_status wkv7_bwd_division(int B, int T, int H, int D, wkv7_dtype in_dtype, const float* dy, const float* dhT,
                              const void* r, const void* w, const void* k, const void* v, const void* a,
                              const void* b, const float* h_ckpt, const float* hT, int restart, float* dr,
                              float* dw, float* dk, float* dv, float* da, float* db, float* dh0, void* stream) {
    wkv7_status st = check_dtype(in_dtype);
    if (st != WKV7_OK) return st;
    Sizes sz;
    st = check_shape(B, T, H, D, &sz);
    if (st != WKV7_OK) return st;
    if (restart != 0 && restart != 1) return WKV7_ERR_ARG;
    if (restart && !h_ckpt) return WKV7_ERR_ARG;
    const int64_t tin = sz.tok_elems * elem_size(in_dtype), t32 = sz.tok_elems * 4, s32 = sz.state_elems * 4;
    const Buf bufs[17] = {{dy, t32, true, false}, {dhT, s32, false, false}, {r, tin, true, false},
                          {w, tin, true, false},  {k, tin, true, false},    {v, tin, true, false},
                          {a, tin, true, false},  {b, tin, true, false},    {h_ckpt, sz.ckpt_elems * 4, false, false},
                          {hT, s32, true, false}, {dr, t32, true, true},    {dw, t32, true, true},
                          {dk, t32, true, true},  {dv, t32, true, true},    {da, t32, true, true},
                          {db, t32, true, true},  {dh0, s32, false, true}};
    st = check_bufs(bufs, 17);
    if (st != WKV7_OK) return st;
    st = check_alias(bufs, 17);
    if (st != WKV7_OK) return st;
    wkv7::DivArgs da_ = {};
    da_.r = r; da_.w = w; da_.k = k; da_.v = v; da_.a = a; da_.b = b;
    da_.dy = dy; da_.dhT = dhT; da_.ckpt = h_ckpt; da_.hT = hT;
    da_.dr = dr; da_.dw = dw; da_.dk = dk; da_.dv = dv; da_.da = da; da_.db = db; da_.dh0 = dh0;
    da_.B = B; da_.T = T; da_.H = H; da_.NC = (int)sz.nc; da_.restart = restart;
    return status_of(wkv7::launch_bwd_division(da_, in_dtype == WKV7_BF16, static_cast<hipStream_t>(stream)));
}

wkv7_status wkv7_bwd_proj(int B, int T, int H, int D, wkv7_dtype in_dtype, const float* dy, const float* dhT,
                          const void* r, const void* w_raw, const void* k, const void* v, const void* kappa,
                          const void* alpha, const float* h_ckpt, float* dr, float* dw_raw, float* dk, float* dv,
                          float* dkappa, float* dalpha, float* dh0, void* workspace, size_t workspace_bytes,
                          void* stream) {
    return bwd_impl(B, T, H, D, in_dtype, true, dy, dhT, r, w_raw, k, v, kappa, alpha, h_ckpt, dr, dw_raw, dk, dv,
                    dkappa, dalpha, dh0, workspace, workspace_bytes, stream);
}

}  // extern "C"
