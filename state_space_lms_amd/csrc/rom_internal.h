// rom_internal.h -- host-side launcher interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rom.h"

namespace rom {

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
