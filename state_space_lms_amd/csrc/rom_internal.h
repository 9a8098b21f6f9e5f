// rom_internal.h -- host-side launcher interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "rom.h"

namespace rom {

// ---- per-device caches (the library's only state). Each entry is filled once per device, thread-safely.
constexpr int kMaxDevices = 64;

// A kernel's dynamic-LDS limit, raised once per device on first use (the attribute belongs to the kernel
// as loaded on the current device). One instance per kernel instantiation (a function-local static).
struct LdsAttrOnce {
    std::once_flag flag[kMaxDevices];
    hipError_t err[kMaxDevices] = {};
};
inline hipError_t set_lds_limit_once(LdsAttrOnce &o, const void *fn, size_t bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(o.flag[dev], [&] {
        o.err[dev] = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    });
    return o.err[dev];
}

// Compute units of the current device (cached per device; 256 if the query fails).
inline int device_cus() {
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Fewest tokens per workgroup of the router-logits kernel (8; 32 when T is large), tokens per
// workgroup of the scatter kernel.
constexpr int kRouteMinTokensPerWG = 8;
constexpr int kScatterTokensPerWG = 256;
// Up to this many tokens the whole routing runs in one workgroup, in one launch.
constexpr int kRouteSmallT = 8;

// Up to this many tokens the bf16 projections take the weight-streaming (decode) kernels.
constexpr int kDecodeMaxT = 64;

// Upper bound of router-logits workgroups for T tokens (sizes the per-workgroup histogram workspace).
inline int route_workgroups(int T) { return (T + kRouteMinTokensPerWG - 1) / kRouteMinTokensPerWG; }
inline int scatter_workgroups(int T) { return (T + kScatterTokensPerWG - 1) / kScatterTokensPerWG; }

// Router workspace (int32 words): the partial histograms [K][E][logits workgroups] (sized for the smallest
// tokens-per-workgroup), then the scatter bases [K][E][scatter workgroups] and the totals [K][E] that the
// prefix-scan kernel writes when the scatter would otherwise re-read too many partial histograms.
inline size_t route_workspace_words(int T, int E) {
    return (size_t)ROM_MAX_TOP_K * E * ((size_t)route_workgroups(T) + scatter_workgroups(T) + 1);
}
inline size_t route_bases_offset(int T, int E) { return (size_t)ROM_MAX_TOP_K * E * route_workgroups(T); }

// With more than this many (scatter workgroup, logits workgroup, expert) triples, a prefix-scan kernel turns
// the partial histograms into per-scatter-workgroup bases once, instead of every scatter workgroup summing all
// partial histograms before its own (whose cost grows with T squared).
constexpr long kScatterPrescanMin = 1L << 22;

// Each returns hipSuccess or the launch error. Arguments are already validated.
hipError_t launch_route(const void *X, rom_dtype dt, int T, int dm, const float *Wr, const float *bias, int E,
                        const rom_routing &r, void *X_perm, int32_t *wg_counts, hipStream_t s);

hipError_t launch_in_proj(const void *X, const rom_routing &r, rom_dtype dt, int T, int dm, int di,
                          const void *Wc, const void *Wg, void *x_out, void *z_out, hipStream_t s);

hipError_t launch_out_proj(const void *z, const void *h, const rom_routing &r, rom_dtype dt, int T, int dm, int di,
                           const void *Wo, void *out, void *workspace, hipStream_t s);

hipError_t launch_in_proj_weighted(const void *X, const rom_routing &r, rom_dtype dt, int T, int dm, int dout,
                                   const void *W, void *y, hipStream_t s);

hipError_t launch_conv1d(const void *x, rom_dtype dt, int nseq, int L, int C, const void *w, const void *bias,
                         int width, int act, void *y, hipStream_t s);

hipError_t launch_out_proj_backward(const void *g, const void *z, const void *h, const rom_routing &r, int T, int dm,
                                    int di, const void *Wo, void *dz, void *dh, float *dWo, void *ws, hipStream_t s);

hipError_t launch_in_proj_backward(const void *X, const void *dx, const void *dzg, const rom_routing &r, int T, int dm,
                                   int di, const void *Wc, const void *Wg, void *dX, float *dWc, float *dWg, void *ws,
                                   hipStream_t s);

// Workspace bytes either backward call needs for T tokens, E experts and top_k choices (bf16 data).
size_t backward_workspace_bytes(int T, int dm, int di, int E, int top_k);

// Workspace bytes the out-projection needs (the gated rows a, T * d_inner bf16 values; 0 for fp32 data).
size_t out_proj_workspace_bytes(int T, int di, rom_dtype dt);

}  // namespace rom
