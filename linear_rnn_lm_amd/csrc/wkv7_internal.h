// wkv7_internal.h -- host-side launchers shared between the library's
// translation units.  Not part of the public ABI (include/wkv7.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv7 {

struct FwdArgs {
    const void *r, *w, *k, *v, *a, *b;
    const float* inv;  // (B,H,NC,32,32): (I - Lab)^-1 of every chunk
    const float* h0;
    float* y;
    float* ckpt;
    float* hT;
    int B, T, H, NC;
};

struct BwdArgs {
    const void *r, *w, *k, *v, *a, *b;
    const float* inv;  // (B,H,NC,32,32): (I - Lab)^-1 of every chunk
    const float* dy;
    const float* dhT;
    const float* ckpt;
    float *dr, *dw, *dk, *dv, *da, *db;
    float* dh0;
    float* gbuf;  // (B,H,NC,D,D): gradient w.r.t. the state entering each chunk
    int B, T, H, NC;
};

// Token tensors (B, T, H, D) are addressed with 32-bit byte offsets: the entry
// points reject shapes whose fp32 token tensors exceed kMaxTensorBytes, and a
// store at kDropOffset lies past every tensor, so the buffer range check drops
// it (with room for a 16-byte access before the offset would wrap).
constexpr uint32_t kMaxTensorBytes = 0xFFFFFF00u;
constexpr uint32_t kDropOffset = 0xFFFFFF00u;

// Bytes of one chunk's transition operands P, M, E, F (the same for both
// storage formats: two bf16 planes or one fp32 plane).
constexpr int kOpsBytes = 36864;

struct PrepArgs {
    const void *r, *w, *k, *a, *b;
    float* inv;  // output (B,H,NC,32,32): (I - Lab)^-1 of every chunk
    void* ops;   // output (B,H,NC) blocks of kOpsBytes
    int B, T, H, NC;
};

struct ScanArgs {
    const void* x;    // forward: v (input dtype); backward: dy (fp32)
    const void* ops;  // (B,H,NC) blocks of kOpsBytes
    const float* s0;  // forward: h0; backward: dhT (NULL = zero)
    float* out;       // forward: y; backward: dv (NULL = skip)
    float* ckpt;      // forward: state entering each chunk; backward: its gradient (NULL = skip)
    float* sT;        // forward: hT; backward: dh0 (NULL = skip)
    int B, T, H, NC;
};

// Each returns hipSuccess or the launch error.
hipError_t launch_chunk_prepare(const PrepArgs& a, bool bf16, hipStream_t s);
hipError_t launch_scan(const ScanArgs& a, bool bf16, bool bwd, hipStream_t s);
hipError_t launch_fwd_sequential(const FwdArgs& a, bool bf16, hipStream_t s);
hipError_t launch_bwd_inputs(const BwdArgs& a, bool bf16, hipStream_t s);

}  // namespace wkv7
