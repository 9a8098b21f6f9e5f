// rom_bwd.hip -- backward of the routed projections on gfx950 (bf16 data, fp32 accumulation).
//
// Routing Mamba landing page (chapterpal.com), Knowl 1, differentiated with the router probabilities
// held fixed. For a token t, its choices s with expert e_s and probability p_s, and a = SiLU(z) * h:
//   out-projection  da[t]   = sum_s p_s W_out[e_s]^T g[t]                  (g = dL/dout)
//                   dz[t]   = da[t] * h[t] * SiLU'(z[t]),  dh[t] = da[t] * SiLU(z[t])
//                   dW_out[e] = sum over the (t, s) routed to e of p_s g[t] a[t]^T
//   in-projection   dX[t]   = sum_s (W_conv[e_s]^T dx[t] + W_gate[e_s]^T dz[t])
//                   dW_conv[e] = sum over the (t, s) routed to e of dx[t] X[t]^T  (dW_gate with dz)
//
// Data gradients ("dgrad") are the forward's grouped GEMMs with transposed weight stacks: the weights
// are first transposed into the workspace (k_transpose_weights), so the MFMA operands stay K-contiguous.
// The in-projection's dgrad contracts over the concatenation [dx | dz] against [W_conv^T | W_gate^T] in
// one GEMM (the A rows switch source at k = d_inner).
//
// Weight gradients ("wgrad") contract over tokens, which are the rows of the token-major activations.
// The activations of each (expert, choice) group are therefore first laid out token-contiguous:
// k_rows_to_cols writes column j of a [features][columns] buffer from the j-th token of the group (in
// slot order), with every group's columns padded with zeros to a multiple of 64, expert-major and
// choice-minor, so an expert's columns form one range. k_wgrad_gemm_bf16 then computes, per expert,
// C_e = P[:, range_e] Q[:, range_e]^T with both operands K-contiguous, and writes fp32.
#include "rom_device.h"
#include "rom_gemm.h"
#include "rom_internal.h"

namespace rom {

namespace {

constexpr int kColTile = 64;  // wgrad column (token) granularity

// ---------------------------------------------------------------------------------------------
// out[e][c][col0 + r] = in[e][r][c] for in [E][R][C] (bf16), out rows of length ldo. 64 x 64 tiles
// through LDS: rows are read and written as 16-byte chunks.
__global__ __launch_bounds__(256) void k_transpose_weights(const uint16_t *__restrict__ in, int R, int C,
                                                           uint16_t *__restrict__ out, int ldo, int col0) {
    __shared__ uint16_t tile[64][64 + 8];
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64, e = blockIdx.z;
    const uint16_t *src = in + ((size_t)e * R + r0) * C + c0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = threadIdx.x + q * 256, r = idx >> 3, ch = idx & 7;
        // chunk ch of row r sits at chunk ch ^ ((r / 8) % 8): the transposed 2-byte reads below then spread
        // over 32 banks instead of 8
        *reinterpret_cast<uint4 *>(&tile[r][(ch ^ ((r >> 3) & 7)) * 8]) =
            *reinterpret_cast<const uint4 *>(src + (size_t)r * C + ch * 8);
    }
    __syncthreads();
    uint16_t *dst = out + ((size_t)e * C + c0) * ldo + col0 + r0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = threadIdx.x + q * 256, c = idx >> 3, ch = idx & 7;
        uint16_t v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = tile[ch * 8 + i][(((c >> 3) ^ ch) << 3) + (c & 7)];
        uint4 pk;
        pk.x = v[0] | (uint32_t(v[1]) << 16);
        pk.y = v[2] | (uint32_t(v[3]) << 16);
        pk.z = v[4] | (uint32_t(v[5]) << 16);
        pk.w = v[6] | (uint32_t(v[7]) << 16);
        *reinterpret_cast<uint4 *>(dst + (size_t)c * ldo + ch * 8) = pk;
    }
}

hipError_t transpose_weights(const void *in, int E, int R, int C, void *out, int ldo, int col0, hipStream_t s) {
    hipLaunchKernelGGL(k_transpose_weights, dim3((unsigned)(C / 64), (unsigned)(R / 64), (unsigned)E), dim3(256), 0, s,
                       static_cast<const uint16_t *>(in), R, C, static_cast<uint16_t *>(out), ldo, col0);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Gate backward, elementwise over 16-byte chunks: dz = da * h * SiLU'(z), dh = da * SiLU(z), with
// SiLU'(v) = s (1 + v (1 - s)), s = 1 / (1 + exp(-v)) (hardware exp2 and reciprocal). Memory-bound: every
// thread issues the loads of kGateBwdChunks chunks (indices clamped into range) before computing any, and
// workgroups stride over the chunk range.
constexpr int kGateBwdChunks = 4;
__global__ __launch_bounds__(256) void k_gate_backward(const uint16_t *__restrict__ da, const uint16_t *__restrict__ z,
                                                       const uint16_t *__restrict__ h, size_t nchunks,
                                                       uint16_t *__restrict__ dz, uint16_t *__restrict__ dh) {
    constexpr int U = kGateBwdChunks;
    const size_t stride = (size_t)gridDim.x * 256 * U;
    for (size_t u0 = (size_t)blockIdx.x * 256 * U + threadIdx.x; u0 < nchunks; u0 += stride) {
        u32x4 va[U], vzz[U], vhh[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const size_t u = u0 + (size_t)j * 256 < nchunks ? u0 + (size_t)j * 256 : nchunks - 1;
            va[j] = reinterpret_cast<const u32x4 *>(da)[u];
            vzz[j] = reinterpret_cast<const u32x4 *>(z)[u];
            vhh[j] = reinterpret_cast<const u32x4 *>(h)[u];
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const size_t u = u0 + (size_t)j * 256;
            if (u < nchunks) {
                uint32_t oz[4], oh[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float r[2][2];
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        const float a = b ? __uint_as_float(va[j][q] & 0xFFFF0000u) : __uint_as_float(va[j][q] << 16);
                        const float zv = b ? __uint_as_float(vzz[j][q] & 0xFFFF0000u) : __uint_as_float(vzz[j][q] << 16);
                        const float hv = b ? __uint_as_float(vhh[j][q] & 0xFFFF0000u) : __uint_as_float(vhh[j][q] << 16);
                        const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-zv));
                        r[0][b] = a * hv * (sg * fmaf(zv, 1.0f - sg, 1.0f));
                        r[1][b] = a * (zv * sg);
                    }
                    oz[q] = pack_bf16x2(r[0][0], r[0][1]);
                    oh[q] = pack_bf16x2(r[1][0], r[1][1]);
                }
                const u32x4 vz = {oz[0], oz[1], oz[2], oz[3]}, vh = {oh[0], oh[1], oh[2], oh[3]};
                __builtin_nontemporal_store(vz, reinterpret_cast<u32x4 *>(dz) + u);
                __builtin_nontemporal_store(vh, reinterpret_cast<u32x4 *>(dh) + u);
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Column layout of the wgrad operands. seg[e * K + k] = first column of the (expert e, choice k) group,
// seg[E * K] = total columns; a group has counts[k][e] columns rounded up to a multiple of 64.
__global__ void k_wgrad_segments(const int32_t *__restrict__ offsets, int E, int K, int32_t *__restrict__ seg) {
    if (threadIdx.x != 0) return;
    int acc = 0;
    for (int e = 0; e < E; ++e)
        for (int k = 0; k < K; ++k) {
            seg[e * K + k] = acc;
            const int c = offsets[k * (E + 1) + e + 1] - offsets[k * (E + 1) + e];
            acc += (c + kColTile - 1) / kColTile * kColTile;
        }
    seg[E * K] = acc;
}

enum ColMode { kColPlain = 0, kColScaled = 1, kColGated = 2 };

// out[f_off + f][j] for the 64 columns j of one group tile and 64 features f: the j-th token t of the
// group contributes src0[t][f] (plain), p * src0[t][f] (scaled by its probability for that choice) or
// bf16(SiLU(src0[t][f]) * src1[t][f]) (gated); padding columns are zero.
// Grid: x = column tiles of the largest possible layout (exits past seg[E*K]), y = feature tiles.
__global__ __launch_bounds__(256) void k_rows_to_cols(const uint16_t *__restrict__ src0, const uint16_t *__restrict__ src1,
                                                      int F, int mode, const int32_t *__restrict__ perm,
                                                      const int32_t *__restrict__ offsets,
                                                      const float *__restrict__ prob, int T, int E, int K,
                                                      const int32_t *__restrict__ seg, uint16_t *__restrict__ out,
                                                      size_t ldo, int f_off) {
    __shared__ uint16_t tile[64][64 + 8];  // [feature][column]
    __shared__ int s_tok[64];
    __shared__ float s_scale[64];
    __shared__ int s_grp;
    const int j0 = blockIdx.x * kColTile, f0 = blockIdx.y * 64;
    const int tid = threadIdx.x;
    if (j0 >= seg[E * K]) return;  // uniform
    if (tid < 64) {
        // the group holding column tile j0: the last g with seg[g] <= j0 (groups of zero width repeat starts)
        for (int g = tid; g < E * K; g += 64)
            if (seg[g] <= j0 && j0 < seg[g + 1]) s_grp = g;
    }
    __syncthreads();
    const int g = s_grp, e = g / K, k = g - e * K;
    if (tid < 64) {
        const int o0 = offsets[k * (E + 1) + e], o1 = offsets[k * (E + 1) + e + 1];
        const int slot = o0 + (j0 - seg[g]) + tid;
        const int t = slot < o1 ? perm[(size_t)k * T + slot] : -1;
        s_tok[tid] = t;
        s_scale[tid] = (t >= 0 && mode == kColScaled) ? prob[(size_t)k * T + t] : 1.0f;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = tid + q * 256, j = idx >> 3, ch = idx & 7;
        const int t = s_tok[j];
        uint16_t v[8];
        if (t < 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0;
        } else if (mode == kColPlain) {
            const uint4 w = *reinterpret_cast<const uint4 *>(src0 + (size_t)t * F + f0 + ch * 8);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) { v[2 * i] = ww[i] & 0xFFFF; v[2 * i + 1] = ww[i] >> 16; }
        } else {
            float a[8];
            load8_f32(src0 + (size_t)t * F + f0 + ch * 8, a);
            if (mode == kColGated) {
                float b[8];
                load8_f32(src1 + (size_t)t * F + f0 + ch * 8, b);
#pragma unroll
                for (int i = 0; i < 8; ++i) a[i] = silu_fast(a[i]) * b[i];
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) a[i] *= s_scale[j];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = f32_to_bf16(a[i]);
        }
        // 8-column group of (feature f, column j) in LDS: (j / 8) ^ ((f / 8) % 8), so that the 2-byte transposed
        // writes of a wave (8 features apart, 8 columns) spread over 32 banks instead of 8
        const int cgs = (((j >> 3) ^ ch) << 3) + (j & 7);
#pragma unroll
        for (int i = 0; i < 8; ++i) tile[ch * 8 + i][cgs] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = tid + q * 256, f = idx >> 3, ch = idx & 7;
        const uint4 w = *reinterpret_cast<const uint4 *>(&tile[f][(ch ^ ((f >> 3) & 7)) * 8]);
        *reinterpret_cast<uint4 *>(out + (size_t)(f_off + f0 + f) * ldo + j0 + ch * 8) = w;
    }
}

// ---------------------------------------------------------------------------------------------
// Per-expert weight-gradient GEMM: C_e[m][n] = sum over the columns j of expert e's range of
// P[m][j] * Q[n][j]; fp32 result rows m < M0 go to out0[e][m][n], the rest to out1[e][m - M0][n].
// Tiles BM x BN over (M, N) for every expert (grid: E x M/BM x N/BN), K steps of 64 columns through a
// 2-stage LDS ring filled by direct global -> LDS copies, v_mfma_f32_32x32x16_bf16 (the same staging
// and XOR swizzle as the forward grouped GEMM). An expert with no tokens gets zeros.
struct WgradArgs {
    const uint16_t *P, *Q;  // [M][ldk], [N][ldk]
    size_t ldk;
    const int32_t *seg;     // column ranges, see k_wgrad_segments
    int E, K, M, N, M0;
    float *out0, *out1;
};

template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void k_wgrad_gemm_bf16(WgradArgs p) {
    constexpr int BK = 64;  // two LDS stages (stage ^ 1 below)
    constexpr int NW = WGM * WGN, KCH = BK / 8, RG = 64 / KCH;
    constexpr int A_DMA = BM / RG / NW, B_DMA = BN / RG / NW, PER_STEP = A_DMA + B_DMA;
    constexpr int STAGE = (BM + BN) * BK;
    constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
    static_assert(A_DMA >= 1 && B_DMA >= 1 && FM >= 1 && FN >= 1, "shape");
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS addresses in SGPRs
    const int nmt = p.M / BM, nnt = p.N / BN;
    // Workgroups go round-robin to the 8 XCDs (b on XCD b % 8). Expert-major, N-tile-minor order puts N-tiles nt = x
    // (mod 8) on XCD x when nnt is a multiple of 8: each Q tile is fetched by one XCD and every P tile by all of them.
    // When P is the larger operand (M >= N) XCD x takes the M-tiles mt = x (mod 8) instead, expert by expert, so each
    // P tile is fetched once and shared through that XCD's L2 (T = 65536, E = 8, d_inner 4096, loads 60% to 2%: the
    // in-projection backward 5.2 -> 4.8 ms, its 1.07 GB of [dx | dz] columns no longer read by every XCD).
    int e, mt, nt;
    if (p.M >= p.N && nmt % 8 == 0) {
        // per: the tiles of one expert on one XCD
        const int x = blockIdx.x & 7, j = blockIdx.x >> 3, per = (nmt >> 3) * nnt;
        e = j / per;
        const int r = j - e * per;
        mt = (r / nnt) * 8 + x;
        nt = r % nnt;
    } else {
        e = blockIdx.x / (nmt * nnt);
        const int rem = blockIdx.x - e * nmt * nnt;
        mt = rem / nnt;
        nt = rem % nnt;
    }
    const int m0 = mt * BM, n0 = nt * BN;
    const int kb = p.seg[e * p.K], ke = p.seg[(e + 1) * p.K];
    const int nk = (ke - kb) / BK;

    const int dr = lane / KCH, dpc = lane % KCH;
    const uint16_t *a_dma[A_DMA];
    const uint16_t *b_dma[B_DMA];
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) {
        const int row = (wave * A_DMA + j) * RG + dr;
        a_dma[j] = p.P + (size_t)(m0 + row) * p.ldk + kb + (dpc ^ lds_swz<KCH>(row)) * 8;
    }
#pragma unroll
    for (int j = 0; j < B_DMA; ++j) {
        const int row = (wave * B_DMA + j) * RG + dr;
        b_dma[j] = p.Q + (size_t)(n0 + row) * p.ldk + kb + (dpc ^ lds_swz<KCH>(row)) * 8;
    }
    auto issue_copies = [&](int kt, int stage) {
        uint16_t *as = smem + stage * STAGE;
        uint16_t *bs = as + BM * BK;
        const int k0 = kt * BK;
#pragma unroll
        for (int j = 0; j < A_DMA; ++j) dma16_to_lds(a_dma[j] + k0, as + (wave * A_DMA + j) * RG * BK);
#pragma unroll
        for (int j = 0; j < B_DMA; ++j) dma16_to_lds(b_dma[j] + k0, bs + (wave * B_DMA + j) * RG * BK);
    };
    // as the forward GEMM: the next step's copy addresses before the barrier, only the copies after it (skewed block
    // forward + backward 11.03 -> 10.87-10.89 ms; rom1p3b 0.5-0.9% slower, samba421m within noise)
    const uint16_t *ca[A_DMA], *cb[B_DMA];
    auto prep_copies = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int j = 0; j < A_DMA; ++j) ca[j] = a_dma[j] + k0;
#pragma unroll
        for (int j = 0; j < B_DMA; ++j) cb[j] = b_dma[j] + k0;
    };
    auto fire_copies = [&](int stage) {
        uint16_t *as = smem + stage * STAGE;
        uint16_t *bs = as + BM * BK;
#pragma unroll
        for (int j = 0; j < A_DMA; ++j) dma16_to_lds(ca[j], as + (wave * A_DMA + j) * RG * BK);
#pragma unroll
        for (int j = 0; j < B_DMA; ++j) dma16_to_lds(cb[j], bs + (wave * B_DMA + j) * RG * BK);
    };

    const int wm = wave / WGN, wn = wave % WGN;
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    int a_frag[FM], b_frag[FN];
    const int half = lane >> 5;
#pragma unroll
    for (int i = 0; i < FM; ++i) a_frag[i] = (wm * WM + i * 32 + (lane & 31)) * BK;
#pragma unroll
    for (int j = 0; j < FN; ++j) b_frag[j] = BM * BK + (wn * WN + j * 32 + (lane & 31)) * BK;
    const int swz = lds_swz<KCH>(lane & 31);

    // The K loop over the expert's column range (nk steps; none for an expert without tokens, which stores zeros).
    // Tiles with more MFMA blocks per wave than fragment reads per sub-step take the forward grouped GEMM's
    // early-barrier schedule: a wave joins each step's barrier once its fragment reads and the step's copies are
    // done, then issues the next step's copies into the stage just read and the first fragment reads of the next
    // step, and only then the step's last MFMAs, which cover those reads; within a step, the next sub-step's
    // fragment reads are slotted between the MFMAs. Copies run one step ahead, and the last step copies its own
    // data again into the free stage (never read), so every barrier sees the same count of copies in flight
    // (T = 65536, E = 8, d_inner 4096, loads 60% to 2%: in-projection backward 4.85 -> 4.75 ms). The 64 x 64 tile
    // keeps the plain loop: wait, barrier, issue the next copies, then the step's reads and MFMAs.
    constexpr int NR = FM + FN, NM = FM * FN, NG = (NR + 1) / 2;  // reads, MFMAs, MFMAs with reads after them
    constexpr int NKK = BK / 16;                                   // MFMA sub-steps per K step
    auto barrier = [&]() {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    if constexpr (NM > NG) {
        bf16x8 af[2][FM], bfr[2][FN];
        auto load_frags = [&](int stg, int kk, int set) {
            const uint16_t *st = smem + stg * STAGE;
            const int co = ((kk * 2 + half) ^ swz) * 8;
#pragma unroll
            for (int i = 0; i < FM; ++i) af[set][i] = *reinterpret_cast<const bf16x8 *>(st + a_frag[i] + co);
#pragma unroll
            for (int j = 0; j < FN; ++j) bfr[set][j] = *reinterpret_cast<const bf16x8 *>(st + b_frag[j] + co);
        };
        auto mfmas = [&](int set) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[set][j], af[set][i], acc[i][j], 0, 0, 0);
        };
        // issue order of one sub-step: an MFMA, two fragment reads of the next sub-step, ..., the remaining MFMAs
        auto slot_reads = [&]() {
#pragma unroll
            for (int q = 0; q < NR / 2; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            if constexpr (NR % 2 == 1) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NM - NG, 0);
        };
        // sub-steps 0 .. NKK-2 of the step in stage stg, each with the next sub-step's reads
        auto body = [&](int stg) {
#pragma unroll
            for (int kk = 1; kk < NKK; ++kk) {
                load_frags(stg, kk, kk & 1);
                mfmas((kk - 1) & 1);
            }
#pragma unroll
            for (int kk = 1; kk < NKK; ++kk) slot_reads();
        };
        if (nk > 0) {  // uniform
            issue_copies(0, 0);
            wait_copies<PER_STEP, 0>(0);
            barrier();
            issue_copies(min(1, nk - 1), 1);
            load_frags(0, 0, 0);
            int stage = 0;
            for (int kt = 0; kt + 1 < nk; ++kt) {
                body(stage);
                prep_copies(min(kt + 2, nk - 1));
                __builtin_amdgcn_sched_barrier(0);  // the step's MFMAs stay ahead of the wait
                wait_copies<PER_STEP, 0>(0);
                barrier();
                fire_copies(stage);
                const int next = stage ^ 1;
                load_frags(next, 0, 0);
                mfmas((NKK - 1) & 1);
                __builtin_amdgcn_sched_group_barrier(0x020, PER_STEP, 0);
                slot_reads();
                stage = next;
            }
            body(stage);
            mfmas((NKK - 1) & 1);
            wait_copies<PER_STEP, 0>(0);  // the spare copies
        }
    } else {
        if (nk > 0) issue_copies(0, 0);
        for (int kt = 0; kt < nk; ++kt) {
            const int stage = kt & 1;
            wait_copies<PER_STEP, 0>(0);
            barrier();
            if (kt + 1 < nk) issue_copies(kt + 1, stage ^ 1);
            const uint16_t *st = smem + stage * STAGE;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const int co = ((kk * 2 + half) ^ swz) * 8;
                bf16x8 af[FM], bfr[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8 *>(st + a_frag[i] + co);
#pragma unroll
                for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const bf16x8 *>(st + b_frag[j] + co);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
            }
        }
    }
    // C^T layout: register r of block (i, j) holds column 8*(r/4) + 4*half + r%4 of row lane%32
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WM + i * 32 + (lane & 31);
        float *row = m < p.M0 ? p.out0 + ((size_t)e * p.M0 + m) * p.N
                              : p.out1 + ((size_t)e * (p.M - p.M0) + (m - p.M0)) * p.N;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WN + j * 32 + 8 * g + 4 * half;
                const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(row + n));
            }
    }
}

template <int BM, int BN, int WGM, int WGN>
hipError_t launch_wgrad_t(const WgradArgs &a, hipStream_t s) {
    const size_t smem = (size_t)2 * (BM + BN) * 64 * 2;
    static LdsAttrOnce attr;
    hipError_t err =
        set_lds_limit_once(attr, reinterpret_cast<const void *>(&k_wgrad_gemm_bf16<BM, BN, WGM, WGN>), smem);
    if (err != hipSuccess) return err;
    const unsigned grid = (unsigned)(a.E * (a.M / BM) * (a.N / BN));
    hipLaunchKernelGGL((k_wgrad_gemm_bf16<BM, BN, WGM, WGN>), dim3(grid), dim3(64 * WGM * WGN), smem, s, a);
    return hipGetLastError();
}

hipError_t launch_wgrad(const WgradArgs &a, hipStream_t s) {
    if (a.M % 256 == 0 && a.N % 256 == 0) return launch_wgrad_t<256, 256, 2, 4>(a, s);
    if (a.M % 128 == 0 && a.N % 128 == 0) return launch_wgrad_t<128, 128, 2, 2>(a, s);
    return launch_wgrad_t<64, 64, 2, 2>(a, s);
}

// ---------------------------------------------------------------------------------------------
// Workspace layout (all offsets 256-byte aligned):
//   seg      int32 [E*K + 1]
//   weights  bf16  the transposed weight stack(s)
//   cols     bf16  [F][ldk] wgrad operands, ldk = the largest column count, K * T + K * E * 63 rounded to 64
//   (out-projection) da  bf16 [T][d_inner]
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t col_capacity(int T, int E, int K) {
    const size_t c = (size_t)K * T + (size_t)K * E * (kColTile - 1);
    return (c + kColTile - 1) / kColTile * kColTile;
}

struct BwdLayout {
    size_t seg, weights, cols, da, total, ldk;
};

BwdLayout layout(int T, int dm, int di, int E, int K, bool out) {
    BwdLayout L{};
    L.ldk = col_capacity(T, E, K);
    L.seg = 0;
    L.weights = align256(sizeof(int32_t) * (size_t)(E * K + 1));
    const size_t wbytes = out ? (size_t)E * di * dm * 2 : (size_t)E * dm * 2 * di * 2;
    L.cols = L.weights + align256(wbytes);
    const size_t feats = out ? (size_t)dm + di : (size_t)dm + 2 * di;
    L.da = L.cols + align256(feats * L.ldk * 2);
    L.total = L.da + (out ? align256((size_t)T * di * 2) : 0);
    return L;
}

GemmArgs choice_args(GemmArgs a, const rom_routing &r, int T, int k) {
    a.offsets = r.offsets + k * (r.E + 1);
    a.perm = r.perm + (size_t)k * T;
    a.prob = r.prob + (size_t)k * T;
    a.accumulate = k > 0;
    return a;
}

hipError_t rows_to_cols(const void *src0, const void *src1, int F, int mode, const rom_routing &r, int T,
                        const int32_t *seg, uint16_t *cols, size_t ldk, int f_off, hipStream_t s) {
    const dim3 grid((unsigned)(ldk / kColTile), (unsigned)(F / 64));
    hipLaunchKernelGGL(k_rows_to_cols, grid, dim3(256), 0, s, static_cast<const uint16_t *>(src0),
                       static_cast<const uint16_t *>(src1), F, mode, r.perm, r.offsets, r.prob, T, r.E, r.top_k,
                       seg, cols, ldk, f_off);
    return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(int T, int dm, int di, int E, int K) {
    const size_t a = layout(T, dm, di, E, K, true).total, b = layout(T, dm, di, E, K, false).total;
    return a > b ? a : b;
}

#define ROM_TRY(x)                              \
    do {                                        \
        hipError_t err_ = (x);                  \
        if (err_ != hipSuccess) return err_;    \
    } while (0)

hipError_t launch_out_proj_backward(const void *g, const void *z, const void *h, const rom_routing &r, int T, int dm,
                                    int di, const void *Wo, void *dz, void *dh, float *dWo, void *ws,
                                    hipStream_t s) {
    const int E = r.E, K = r.top_k;
    const BwdLayout L = layout(T, dm, di, E, K, true);
    char *base = static_cast<char *>(ws);
    int32_t *seg = reinterpret_cast<int32_t *>(base + L.seg);
    uint16_t *WoT = reinterpret_cast<uint16_t *>(base + L.weights);  // [E][di][dm]
    uint16_t *cols = reinterpret_cast<uint16_t *>(base + L.cols);    // rows [0, dm): p*g; [dm, dm+di): a
    uint16_t *da = reinterpret_cast<uint16_t *>(base + L.da);        // [T][di]

    // da = sum_s p_s W_out[e_s]^T g: the probability-scaled grouped GEMM on the transposed stack,
    // A rows (g) gathered by token, results un-permuted to token order, choices added in order
    ROM_TRY(transpose_weights(Wo, E, dm, di, WoT, dm, 0, s));
    GemmArgs a{};
    a.A0 = g;
    a.B0 = WoT;
    a.C0 = da;
    a.T = T;
    a.K = dm;
    a.N0 = di;
    a.E = E;
    a.a_by_token = 1;
    for (int k = 0; k < K; ++k) ROM_TRY(launch_grouped_bf16(choice_args(a, r, T, k), true, 1, s));
    const size_t nchunks = (size_t)T * di / 8, per_wg = 256 * kGateBwdChunks;
    const unsigned gblocks = (unsigned)((nchunks + per_wg - 1) / per_wg < 4096 ? (nchunks + per_wg - 1) / per_wg : 4096);
    hipLaunchKernelGGL(k_gate_backward, dim3(gblocks), dim3(256), 0, s, da, static_cast<const uint16_t *>(z),
                       static_cast<const uint16_t *>(h), nchunks, static_cast<uint16_t *>(dz),
                       static_cast<uint16_t *>(dh));
    ROM_TRY(hipGetLastError());

    // dW_out[e] = (p g)_e^T a_e over the expert's tokens of both choices
    hipLaunchKernelGGL(k_wgrad_segments, dim3(1), dim3(64), 0, s, r.offsets, E, K, seg);
    ROM_TRY(hipGetLastError());
    ROM_TRY(rows_to_cols(g, nullptr, dm, kColScaled, r, T, seg, cols, L.ldk, 0, s));
    ROM_TRY(rows_to_cols(z, h, di, kColGated, r, T, seg, cols, L.ldk, dm, s));
    WgradArgs w{};
    w.P = cols;
    w.Q = cols + (size_t)dm * L.ldk;
    w.ldk = L.ldk;
    w.seg = seg;
    w.E = E;
    w.K = K;
    w.M = dm;
    w.N = di;
    w.M0 = dm;
    w.out0 = dWo;
    w.out1 = dWo;
    return launch_wgrad(w, s);
}

hipError_t launch_in_proj_backward(const void *X, const void *dx, const void *dzg, const rom_routing &r, int T, int dm,
                                   int di, const void *Wc, const void *Wg, void *dX, float *dWc, float *dWg, void *ws,
                                   hipStream_t s) {
    const int E = r.E, K = r.top_k;
    const BwdLayout L = layout(T, dm, di, E, K, false);
    char *base = static_cast<char *>(ws);
    int32_t *seg = reinterpret_cast<int32_t *>(base + L.seg);
    uint16_t *WT = reinterpret_cast<uint16_t *>(base + L.weights);  // [E][dm][2 di] = [W_conv^T | W_gate^T]
    uint16_t *cols = reinterpret_cast<uint16_t *>(base + L.cols);   // rows [0, 2di): dx, dz; [2di, 2di+dm): X

    // dX = sum_s [W_conv | W_gate][e_s]^T [dx | dz]: one grouped GEMM per choice over K = 2 d_inner
    ROM_TRY(transpose_weights(Wc, E, di, dm, WT, 2 * di, 0, s));
    ROM_TRY(transpose_weights(Wg, E, di, dm, WT, 2 * di, di, s));
    GemmArgs a{};
    a.A0 = dx;
    a.A_hi = dzg;
    a.k_split = di;
    a.B0 = WT;
    a.C0 = dX;
    a.T = T;
    a.K = 2 * di;
    a.N0 = dm;
    a.E = E;
    for (int k = 0; k < K; ++k) ROM_TRY(launch_grouped_bf16(choice_args(a, r, T, k), false, 1, s));

    // dW_conv[e] = dx_e^T X_e and dW_gate[e] = dz_e^T X_e in one wgrad GEMM over M = 2 d_inner rows
    hipLaunchKernelGGL(k_wgrad_segments, dim3(1), dim3(64), 0, s, r.offsets, E, K, seg);
    ROM_TRY(hipGetLastError());
    ROM_TRY(rows_to_cols(dx, nullptr, di, kColPlain, r, T, seg, cols, L.ldk, 0, s));
    ROM_TRY(rows_to_cols(dzg, nullptr, di, kColPlain, r, T, seg, cols, L.ldk, di, s));
    ROM_TRY(rows_to_cols(X, nullptr, dm, kColPlain, r, T, seg, cols, L.ldk, 2 * di, s));
    WgradArgs w{};
    w.P = cols;
    w.Q = cols + (size_t)2 * di * L.ldk;
    w.ldk = L.ldk;
    w.seg = seg;
    w.E = E;
    w.K = K;
    w.M = 2 * di;
    w.N = dm;
    w.M0 = di;
    w.out0 = dWc;
    w.out1 = dWg;
    return launch_wgrad(w, s);
}

}  // namespace rom
