// rom_conv.hip -- the shared short causal convolution that follows the in-projection.
//
// Routing Mamba landing page (chapterpal.com), Knowl 1: a short convolution is applied to H_t (the
// Conv projection's output, in token order) before the selective SSM; Knowl 9: that 1D convolution is
// shared by all experts. The page fixes no width, bias or activation; this library takes a depthwise
// causal convolution of width w per sequence, zeros before a sequence's first token, an optional bias
// and an optional SiLU:
//   u[b][t][c] = bias[c] + sum_{j<w} W[c][j] * x[b][t - (w-1) + j][c],   y = act ? SiLU(u) : u.
//
// Memory-bound (one read and one write of 2 bytes per bf16 element, plus a halo of w-1 rows per run of
// tokens). A thread owns 8 consecutive channels (one 16-byte chunk of a bf16 row) of a run of R
// consecutive tokens of one sequence, holds the run's inputs and the w-1 rows before it in registers,
// and reads each input once apart from the halo. The 64 lanes of a wave take 64 consecutive
// chunks of the same rows, so every row access is a contiguous 1 KiB (bf16) per wave, and consecutive
// waves take the next 64 chunks of the same run, so a workgroup reads whole row segments of 4 KiB.
// Results are written with non-temporal stores (the next reader is another kernel).
#include "rom_device.h"
#include "rom_internal.h"

namespace rom {

namespace {

constexpr int kConvRun = 16;  // tokens per thread

// One row chunk (8 channels) as loaded: 16 bytes of bf16, or 32 bytes of fp32.
template <typename T> struct Chunk;
template <> struct Chunk<uint16_t> {
    uint4 v;
    __device__ __forceinline__ void load(const uint16_t *p) { v = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ float get(int i) const {  // i is a compile-time constant after unrolling
        const uint32_t w = i < 2 ? v.x : i < 4 ? v.y : i < 6 ? v.z : v.w;
        return (i & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
    }
};
template <> struct Chunk<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = reinterpret_cast<const float4 *>(p)[0];
        b = reinterpret_cast<const float4 *>(p)[1];
    }
    __device__ __forceinline__ void zero() { a = b = make_float4(0, 0, 0, 0); }
    __device__ __forceinline__ float get(int i) const {
        const float4 &q = i < 4 ? a : b;
        const int j = i & 3;
        return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
    }
};

__device__ __forceinline__ void store8(uint16_t *p, const float f[8]) {
    const u32x4 v = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                     pack_bf16x2(f[6], f[7])};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ void store8(float *p, const float f[8]) {
    __builtin_nontemporal_store((f32x4){f[0], f[1], f[2], f[3]}, reinterpret_cast<f32x4 *>(p));
    __builtin_nontemporal_store((f32x4){f[4], f[5], f[6], f[7]}, reinterpret_cast<f32x4 *>(p) + 1);
}

// The run's outputs from its rows. Every output is computed unconditionally (the clamped loads make the
// tail rows valid), so the whole run is one basic block and each input is widened once; only the stores
// of a ragged run are guarded.
template <typename T, int W, bool RAGGED>
__device__ __forceinline__ void conv_outputs(const Chunk<T> (&rows)[W - 1 + kConvRun], const float (&wt)[W][8],
                                             const float (&bs)[8], int act, int n, T *ys, int C) {
#pragma unroll
    for (int r = 0; r < kConvRun; ++r) {
        float u[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float acc = bs[i];
#pragma unroll
            for (int j = 0; j < W; ++j) acc = fmaf(wt[j][i], rows[r + j].get(i), acc);
            u[i] = act ? silu_fast(acc) : acc;
        }
        if (!RAGGED || r < n) store8(ys + (size_t)r * C, u);
    }
}

// Every load of the run (the W-1 halo rows and the kConvRun own rows) is issued before the first output
// is computed; the output loop is fully unrolled, so the sliding window is plain register indexing.
// SiLU uses the hardware exp2 and reciprocal (v_exp_f32, v_rcp_f32; about 1 ulp each).
template <typename T, int W>
__global__ __launch_bounds__(256) void k_causal_conv1d(const T *__restrict__ x, const T *__restrict__ weight,
                                                       const T *__restrict__ bias, int L, int C, int runs_per_seq,
                                                       int total_runs, int act, T *__restrict__ y) {
    const int cpr = C >> 3;
    const int wpr = (cpr + 63) >> 6;                             // waves per run (64 chunks each)
    const int wu = blockIdx.x * 4 + (threadIdx.x >> 6);          // wave unit: consecutive units cover a run's
    const int run = wu / wpr;                                    // row segments left to right
    const int chunk = (wu - run * wpr) * 64 + (threadIdx.x & 63);
    if (chunk >= cpr || run >= total_runs) return;
    const int seq = run / runs_per_seq;
    const int t0 = (run - seq * runs_per_seq) * kConvRun;
    const int c0 = chunk * 8;
    const T *xs = x + (size_t)seq * L * C + c0;
    T *ys = y + (size_t)seq * L * C + c0;
    const int n = min(kConvRun, L - t0);  // tokens of this run (uniform over the wave)

    // rows[k] holds the input at time t0 - (W-1) + k
    Chunk<T> rows[W - 1 + kConvRun];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) {
        const int s = t0 - (W - 1) + k;
        if (s >= 0) rows[k].load(xs + (size_t)s * C);
        else rows[k].zero();
    }
#pragma unroll
    for (int r = 0; r < kConvRun; ++r) rows[W - 1 + r].load(xs + (size_t)(t0 + min(r, n - 1)) * C);  // clamped

    // taps: wt[j][i] multiplies channel c0 + i at time t - (W-1) + j
    float wt[W][8], bs[8];
    {
        float raw[8 * W];
#pragma unroll
        for (int q = 0; q < W; ++q) load8_f32(weight + (size_t)c0 * W + 8 * q, raw + 8 * q);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < W; ++j) wt[j][i] = raw[i * W + j];
    }
    if (bias != nullptr) {
        load8_f32(bias + c0, bs);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) bs[i] = 0.0f;
    }

    if (n == kConvRun) conv_outputs<T, W, false>(rows, wt, bs, act, n, ys + (size_t)t0 * C, C);
    else conv_outputs<T, W, true>(rows, wt, bs, act, n, ys + (size_t)t0 * C, C);
}

template <typename T>
hipError_t launch_conv_typed(const void *x, int nseq, int L, int C, const void *w, const void *bias, int width,
                             int act, void *y, hipStream_t s) {
    const int runs_per_seq = (L + kConvRun - 1) / kConvRun;
    const int total_runs = nseq * runs_per_seq;
    const long wave_units = (long)total_runs * ((C / 8 + 63) / 64);
    const dim3 grid((unsigned)((wave_units + 3) / 4));
    const T *xp = static_cast<const T *>(x), *wp = static_cast<const T *>(w), *bp = static_cast<const T *>(bias);
    T *yp = static_cast<T *>(y);
#define ROM_CONV_CASE(WW)                                                                                     \
    case WW:                                                                                                  \
        hipLaunchKernelGGL((k_causal_conv1d<T, WW>), grid, dim3(256), 0, s, xp, wp, bp, L, C, runs_per_seq, \
                           total_runs, act, yp);                                                              \
        break;
    switch (width) {
        ROM_CONV_CASE(1)
        ROM_CONV_CASE(2)
        ROM_CONV_CASE(3)
        ROM_CONV_CASE(4)
        ROM_CONV_CASE(5)
        ROM_CONV_CASE(6)
        ROM_CONV_CASE(7)
        ROM_CONV_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef ROM_CONV_CASE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv1d(const void *x, rom_dtype dt, int nseq, int L, int C, const void *w, const void *bias,
                         int width, int act, void *y, hipStream_t s) {
    if (dt == ROM_DTYPE_BF16) return launch_conv_typed<uint16_t>(x, nseq, L, C, w, bias, width, act, y, s);
    return launch_conv_typed<float>(x, nseq, L, C, w, bias, width, act, y, s);
}

}  // namespace rom
