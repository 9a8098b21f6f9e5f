// rom_internal.h -- host-side launcher interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rom.h"

namespace rom {

// Tokens handled by one router workgroup on the multi-workgroup path.
constexpr int kRouteTokensPerWG = 256;
// Up to this many tokens the whole routing runs in one workgroup, in one launch.
constexpr int kRouteSmallT = 256;

inline int route_workgroups(int T) { return (T + kRouteTokensPerWG - 1) / kRouteTokensPerWG; }

// Each returns hipSuccess or the launch error. Arguments are already validated.
hipError_t launch_route(const void *X, rom_dtype dt, int T, int dm, const float *Wr, const float *bias, int E,
                        const rom_routing &r, void *X_perm, int32_t *wg_counts, hipStream_t s);

hipError_t launch_in_proj(const void *X, const rom_routing &r, rom_dtype dt, int T, int dm, int di,
                          const void *Wc, const void *Wg, void *x_out, void *z_out, hipStream_t s);

hipError_t launch_out_proj(const void *z, const void *h, const rom_routing &r, rom_dtype dt, int T, int dm, int di,
                           const void *Wo, void *out, hipStream_t s);

}  // namespace rom
