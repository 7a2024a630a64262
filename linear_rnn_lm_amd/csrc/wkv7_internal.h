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

struct InvArgs {
    const void *w, *a, *b;
    float* inv;  // output (B,H,NC,32,32)
    int B, T, H, NC;
};

// Each returns hipSuccess or the launch error.
hipError_t launch_chunk_inv(const InvArgs& a, bool bf16, hipStream_t s);
hipError_t launch_fwd_chunked(const FwdArgs& a, bool bf16, hipStream_t s);
hipError_t launch_fwd_sequential(const FwdArgs& a, bool bf16, hipStream_t s);
hipError_t launch_bwd_state(const BwdArgs& a, bool bf16, hipStream_t s);   // kernel 1
hipError_t launch_bwd_inputs(const BwdArgs& a, bool bf16, hipStream_t s);  // kernel 2

}  // namespace wkv7
