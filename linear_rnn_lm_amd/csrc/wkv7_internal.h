// wkv7_internal.h -- host-side launchers shared between the library's
// translation units.  Not part of the public ABI (include/wkv7.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

namespace wkv7 {

// One-time setup per device (a kernel's dynamic LDS limit), safe to reach
// from several host threads at once: the first caller on a device runs the
// setup under a lock; a failed setup is not recorded, so the next call tries
// again.  Nothing else in the library is mutable.
constexpr int kMaxDevices = 64;
struct PerDeviceOnce {
    std::atomic<bool> done[kMaxDevices] = {};
    std::mutex lock;
    template <typename F>
    hipError_t run(F&& setup) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
        if (done[dev].load(std::memory_order_acquire)) return hipSuccess;
        std::lock_guard<std::mutex> g(lock);
        if (done[dev].load(std::memory_order_relaxed)) return hipSuccess;
        e = setup(dev);
        if (e == hipSuccess) done[dev].store(true, std::memory_order_release);
        return e;
    }
};

// Raise a kernel's dynamic LDS limit to `bytes`, once per device.
template <typename K>
hipError_t set_smem_once(PerDeviceOnce& once, K kern, int bytes) {
    return once.run([&](int) {
        return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                   bytes);
    });
}

// Compute units of the current device (queried on every call: it is a
// cached attribute in the runtime, so nothing is kept here).
inline hipError_t device_cus(int* n_cu) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    return e;
}

struct FwdArgs {
    const void *r, *w, *k, *v, *a, *b;
    const float* inv;  // (B,H,NC,32,32): (I - Lab)^-1 of every chunk
    const float* h0;
    float* y;
    float* ckpt;
    float* hT;
    int B, T, H, NC;
};

// Division by a divisor that is fixed for a launch, without a divide
// instruction: for 0 <= n < 2^31, n / d = (umulhi(n, m) + n) >> s with
// s = ceil(log2 d) and the round-up multiplier m = floor(2^32 (2^s - d) / d) + 1
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994).
struct FastDiv {
    uint32_t d, m, s;
};
constexpr FastDiv make_fastdiv(uint32_t d) {
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    return FastDiv{d, (uint32_t)((((1ull << s) - d) << 32) / d + 1), s};
}
__host__ __device__ constexpr uint32_t fdiv(uint32_t n, FastDiv f) {
    return (uint32_t)(((((uint64_t)n * f.m) >> 32) + n) >> f.s);
}
static_assert(fdiv(0, make_fastdiv(1)) == 0 && fdiv(12345, make_fastdiv(1)) == 12345, "fastdiv");
static_assert(fdiv(31, make_fastdiv(32)) == 0 && fdiv(32, make_fastdiv(32)) == 1 && fdiv(2303, make_fastdiv(32)) == 71,
              "fastdiv");
static_assert(fdiv(71, make_fastdiv(6)) == 11 && fdiv(72, make_fastdiv(6)) == 12 && fdiv(0x7fffffff, make_fastdiv(6)) ==
              0x7fffffff / 6, "fastdiv");
static_assert(fdiv(0x7fffffff, make_fastdiv(7)) == 0x7fffffff / 7 && fdiv(0x7ffffffe, make_fastdiv(0x7fffffff)) == 0 &&
              fdiv(0x7fffffff, make_fastdiv(0x7fffffff)) == 1, "fastdiv");
static_assert(fdiv(999999, make_fastdiv(1000)) == 999 && fdiv(1000000, make_fastdiv(1000)) == 1000, "fastdiv");

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
    FastDiv fd_nc, fd_h;   // set by the launcher
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

// The division-walk backward (a diagnostic; wkv7_division.hip).
struct DivArgs {
    const void *r, *w, *k, *v, *a, *b;
    const float* dy;
    const float* dhT;   // NULL = zero
    const float* ckpt;  // (B,H,NC,D,D) states entering each chunk (read when restart != 0)
    const float* hT;    // (B,H,D,D) state after the last token
    float *dr, *dw, *dk, *dv, *da, *db;
    float* dh0;         // NULL = not wanted
    int B, T, H, NC;
    int restart;        // 1: each chunk's walk starts from the exact state at its end; 0: only the last
};

// Each returns hipSuccess or the launch error.  proj: the w, a, b pointers
// hold the raw projections w_raw, kappa, alpha, and the time-mix prologue runs
// inside the kernels' loads (backward: dw, da, db receive dw_raw, dkappa,
// dalpha).
hipError_t launch_chunk_prepare(const PrepArgs& a, bool bf16, bool proj, hipStream_t s);
hipError_t launch_scan(const ScanArgs& a, bool bf16, bool bwd, hipStream_t s);
hipError_t launch_fwd_sequential(const FwdArgs& a, bool bf16, bool proj, hipStream_t s);
hipError_t launch_bwd_inputs(const BwdArgs& a, bool bf16, bool proj, hipStream_t s);
hipError_t launch_bwd_division(const DivArgs& a, bool bf16, hipStream_t s);

}  // namespace wkv7
