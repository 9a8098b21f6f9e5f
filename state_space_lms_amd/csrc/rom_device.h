// rom_device.h -- device helpers shared by the gfx950 kernels of librom (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rom {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 <-> fp32. Widening is exact (the bf16 bits are the high half of the fp32 word).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest even (gfx950 converts natively).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

// Two fp32 -> packed bf16 pair (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return uint32_t(f32_to_bf16(a)) | (uint32_t(f32_to_bf16(b)) << 16);
}

// Eight consecutive elements widened to fp32 (p is 16-byte aligned for bf16, 32-byte for fp32).
__device__ __forceinline__ void load8_f32(const uint16_t *p, float f[8]) {
    uint4 v = *reinterpret_cast<const uint4 *>(p);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void load8_f32(const float *p, float f[8]) {
    float4 a = reinterpret_cast<const float4 *>(p)[0];
    float4 b = reinterpret_cast<const float4 *>(p)[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane i of the wave writes
// LDS bytes [lds + 16*i, lds + 16*i + 16). lds must be the same for every lane of the wave.
__device__ __forceinline__ void dma16_to_lds(const void *src, void *lds) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// SiLU(v) = v / (1 + exp(-v)), the sigmoid-weighted linear unit. silu_precise divides and uses the
// library expf; silu_fast uses the hardware exp2 (v_exp_f32, on v * log2(e)) and reciprocal (v_rcp_f32),
// about 1 ulp each, for results that are rounded to bf16 afterwards or feed an fp32 sum.
__device__ __forceinline__ float silu_precise(float v) { return v / (1.0f + expf(-v)); }
__device__ __forceinline__ float silu_fast(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

// ---- MFMA operand staging (shared by the forward and backward GEMMs)
// gfx950 LDS serves a 16-byte-per-lane read 16 lanes at a time across 256 bytes of banks: 16 slots of
// 16 bytes. An MFMA operand read has 16 consecutive lanes on 16 consecutive rows at one logical chunk,
// so the swizzle must send those 16 rows to 16 different slots. With 128-byte rows (BK = 64) a row's
// parity picks the half of the 256-byte window and (row >> 1) & 7 permutes the chunk within it; with
// 64-byte rows (BK = 32) row & 3 picks the quarter and (row >> 2) & 3 permutes within it.
template <int KCH>
__device__ __forceinline__ int lds_swz(int row) {
    return KCH == 8 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= n and lgkmcnt == 0, expcnt untouched.
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4); }

// Wait until at most `ahead` K steps of copies (PER_STEP instructions each) are still in flight.
template <int PER_STEP, int MAXAHEAD>
__device__ __forceinline__ void wait_copies(int ahead) {
    static_assert(PER_STEP * MAXAHEAD < 64, "vmcnt range");
    if (MAXAHEAD >= 3 && ahead >= 3) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(3 * PER_STEP));
    else if (MAXAHEAD >= 2 && ahead == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * PER_STEP));
    else if (MAXAHEAD >= 1 && ahead == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(PER_STEP));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
}

}  // namespace rom
