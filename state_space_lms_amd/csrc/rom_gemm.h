// rom_gemm.h -- arguments of the ragged grouped GEMM kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rom {

struct GemmArgs {
    const void *A0;       // in-proj: X [T][K];  out-proj: z [T][K]
    const void *A1;       // out-proj: h [T][K] (fp32 kernel only; NULL: A rows are used as they are)
    const void *B0;       // in-proj: W_conv [E][N0][K];  out-proj: W_out [E][N0][K]
    const void *B1;       // in-proj: W_gate [E][N0][K]
    void *C0;             // in-proj: x_out [T][N0];  out-proj: out [T][N0]
    void *C1;             // in-proj: z_out [T][N0]
    const int32_t *offsets;
    const int32_t *perm;
    const float *prob;
    int T, K, N0, E;
    int n_tiles;          // N-tiles over the concatenated columns (nB * N0 / BN)
    int n_tiles_per_b;    // N0 / BN
    int m_tiles;          // M-tiles launched (upper bound of the real ones)
    int group_m;          // XCD-aware order: M-tiles per group (0: plain row-major order)
    int per_xcd;          // XCD-aware order: tiles per chunk (the compute units of one XCD)
    int accumulate;       // 1: add to the values already in C (the second choice of a top-2 routing)
    int a_by_token;       // out-projection: A rows are in token order (gathered through perm), not slot order
    const void *A_hi;     // bf16 kernel, k_split > 0: columns [k_split, K) of the A rows come from A_hi
    int k_split;          // 0: A0 holds whole rows of K; else A0 rows hold k_split values, A_hi rows K - k_split
};

// The bf16 MFMA grouped GEMM over nB weight stacks (B0, B1), tile shape chosen by problem size.
// out = false: A rows gathered through perm, no scale; out = true: scaled by p, A rows in slot order
// unless a_by_token. Every field the kernels read must be set (zero-initialise the struct).
hipError_t launch_grouped_bf16(const GemmArgs &a, bool out, int nB, hipStream_t s);

// Decode-size kernels (rom_gemv.hip): every workgroup streams 16 (or 32) weight rows of one active expert and
// applies them to all of that expert's tokens. out: probability-scaled results (rows gathered in token order).
hipError_t launch_gemv_bf16(const GemmArgs &a, bool out, int nB, hipStream_t s);
// The same with the expert's token rows staged in LDS once per workgroup (gemv_lds_fits); gated (with out):
// the staged rows are bf16(SiLU(A0) * A1), the out-projection's gate computed on the fly.
constexpr size_t kGemvLdsBytes = 64 * 1024;
inline bool gemv_lds_fits(int T, int K) { return T <= 16 && (size_t)T * (K + 8) * 2 <= kGemvLdsBytes; }
hipError_t launch_gemv_lds_bf16(const GemmArgs &a, bool out, bool gated, int nB, hipStream_t s);
// Wide decode kernel: 16 waves over 64 to 256 weight rows, token rows (gathered through perm) staged through
// LDS in K chunks. gemv_wide_fits: the shape suits it (enough rows for a workgroup per compute unit).
bool gemv_wide_fits(int T, int E, int N0, int K, int nB);
hipError_t launch_gemv_wide_bf16(const GemmArgs &a, bool out, int nB, hipStream_t s);

}  // namespace rom
