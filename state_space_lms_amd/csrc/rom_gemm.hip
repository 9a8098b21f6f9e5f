// rom_gemm.hip -- ragged grouped GEMMs of the Routing Mamba projection experts on gfx950.
//
// Method: Routing Mamba landing page (chapterpal.com), Knowl 1. For a token t routed to expert e:
//   in-projection   x[t] = W_conv[e] X[t],  z[t] = W_gate[e] X[t]         (indicator only, no scale)
//   out-projection  out[t] = p_t * W_out[e] (SiLU(z[t]) * h[t])          (h stands in for Y_t)
// with weights stored [out][in]. Tokens are grouped by expert (slot order from the router's stable
// counting sort); every expert group is a dense GEMM C_e[n_e x N] = A_e[n_e x K] * W_e[N x K]^T.
//
// Work decomposition: one workgroup per (M-tile, N-tile). M-tiles are numbered expert by expert,
// ceil(n_e / BM) tiles for expert e; the grid is launched for the upper bound
// floor((T + E*(BM-1)) / BM) M-tiles so the host never reads the counts, and workgroups past the
// last real tile exit at once. A rows are gathered through perm (token order -> slot order) while
// they are staged into LDS; the epilogue scatters rows back to token order (the un-permute).
//
// bf16 path (T > 64): workgroups of WGM x WGN waves (8 for the default 256 x 256 tile, and for the 320 x 256
// tile chosen when it needs fewer rounds over the compute units), each wave owning a (BM/WGM) x (BN/WGN)
// block of 32x32 MFMA tiles (v_mfma_f32_32x32x16_bf16, fp32 accumulators). Operand rows are copied
// global -> LDS directly (no register round trip), NSTAGE - 1 K steps ahead of the MFMAs; in the default
// two-stage schedule each step's barrier sits ahead of its last MFMAs, which then cover the first operand
// reads of the next step. LDS rows are XOR-swizzled so that MFMA operand reads are free of bank conflicts. The tile is written back through LDS
// as whole 16-byte row chunks. Details at k_grouped_gemm_bf16. The backward's data gradients run the same
// kernels on transposed weight stacks (KSPLIT: the A rows switch source at k_split).
//
// Decode path (T <= 64): weight-streaming kernels in rom_gemv.hip. fp32 data: k_grouped_gemm_f32.
#include <stdlib.h>

#include "rom_device.h"
#include "rom_gemm.h"
#include "rom_internal.h"

namespace rom {


// Tile (mt, nt) of workgroup blockIdx.x; false if the workgroup has no tile.
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on XCD b % 8), each with its
// own L2. With group_m > 0 the tiles follow a grouped order in which group_m consecutive M-tiles share
// every N-tile, cut into chunks of per_xcd tiles (the compute units of one XCD), and XCD x takes chunks
// x, x + 8, x + 16, ...: the workgroups resident on one XCD at a time then need group_m A tiles and
// per_xcd / group_m B tiles, so more operand reads hit that XCD's L2, and as the real tiles are a
// prefix of the grouped order every XCD gets nearly the same number of them.
__device__ __forceinline__ bool tile_of_block(const GemmArgs &p, int &mt, int &nt) {
    int L = blockIdx.x;
    if (p.group_m > 0) {
        const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
        L = ((j / p.per_xcd) * 8 + x) * p.per_xcd + j % p.per_xcd;
        const int span = p.group_m * p.n_tiles;
        const int g = L / span, in = L - g * span;
        mt = g * p.group_m + in % p.group_m;
        nt = in / p.group_m;
    } else {
        mt = L / p.n_tiles;
        nt = L % p.n_tiles;
    }
    return mt < p.m_tiles;
}

// Expert and row range of M-tile mt: returns false if mt lies past the last real tile.
template <int BM>
__device__ __forceinline__ bool locate_mtile(const int32_t *__restrict__ offsets, int E, int mt, int &e,
                                             int &slot0, int &rows) {
    int acc = 0;
    for (int i = 0; i < E; ++i) {
        const int o0 = offsets[i], o1 = offsets[i + 1];
        const int c = o1 - o0;
        const int nt = (c + BM - 1) / BM;
        if (mt < acc + nt) {
            const int m0 = (mt - acc) * BM;
            e = i;
            slot0 = o0 + m0;
            rows = min(BM, c - m0);
            return true;
        }
        acc += nt;
    }
    return false;
}

// ---------------------------------------------------------------------------------------------
// bf16 MFMA grouped GEMM. OUT = false: in-projection, A rows are the tokens' X rows (gathered
// through perm). OUT = true: out-projection, A rows are the gated rows a = bf16(SiLU(z) * h) that
// k_gate_permute has already laid out in slot order, and results are scaled by p_t.
//
// Block tile BM x BN, K step BK (64 or 32), NSTAGE LDS stages, WGM x WGN waves, each wave owning a
// (BM/WGM) x (BN/WGN) block of 32x32 MFMA tiles (v_mfma_f32_32x32x16_bf16, fp32 accumulators).
//
// Staging: A and B rows are copied global -> LDS directly (global_load_lds_dwordx4: lane i of a
// wave writes 16 bytes at LDS base + 16*i), NSTAGE-1 K steps ahead of the MFMAs, with no register
// round trip; before each step a wave waits only until its copies for that step have landed
// (vmcnt counts the later steps' copies still in flight), then the workgroup meets at a barrier
// (in the default schedule, ahead of the step's last MFMAs: see the main loop).
// LDS rows hold BK bf16 values as BK/8 16-byte chunks; chunk c of row r sits at c ^ swz(r) so the
// MFMA operand reads (16 lanes = 16 consecutive rows, one chunk each) spread over all banks.
//
// The MFMA computes the transposed tile C^T = W A^T (W operand first): a lane's 16 accumulators of
// a 32x32 block belong to ONE token row (lane % 32) and hold 4 runs of 4 consecutive output columns,
// which the epilogue scales by that token's probability and sends to the token's output row (the
// un-permute).
// ---- staged epilogue. Scattering the C^T-layout accumulators straight to the token rows costs one
// store instruction per 8 bytes and touches 32 rows (cache lines) per instruction. Instead each wave
// writes its block, converted to bf16 and scaled per row, into an LDS tile of BM x BN, and the
// workgroup then writes whole 16-byte chunks, consecutive lanes along a row, so one instruction covers
// 2 (BN = 256) to 8 (BN = 64) full rows. The 16-byte chunk c of LDS row r sits at c ^ (r & (CPR - 1))
// (CPR = chunks per row, at most 32): the 8-byte writes of 32 consecutive rows at one column and the
// row-wise 16-byte reads both spread over the banks. The output is not read again by this kernel, so
// the stores are non-temporal.
template <int BN>
__device__ __forceinline__ int ctile_swz(int row) {
    constexpr int CPR = BN / 8;
    return row & ((CPR < 32 ? CPR : 32) - 1);
}

// One wave's FM x FN blocks of 32 x 32 (C^T layout: register r of block (i, j) holds column
// 8*(r/4) + 4*(lane/32) + r%4 of row lane%32) into LDS rows [row0 + 32 i ..], columns [col0 + 32 j ..],
// scaled by sc[i].
template <int FM, int FN, int BN>
__device__ __forceinline__ void acc_to_ctile(const f32x16 (&acc)[FM][FN], uint16_t *ct, int row0, int col0,
                                             int lane, const float (&sc)[FM]) {
    const int half = lane >> 5;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int row = row0 + i * 32 + (lane & 31);
        uint16_t *crow = ct + row * BN;
        const int swz = ctile_swz<BN>(row);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = col0 + j * 32 + 8 * g + 4 * half;
                uint2 pk;
                pk.x = pack_bf16x2(acc[i][j][4 * g] * sc[i], acc[i][j][4 * g + 1] * sc[i]);
                pk.y = pack_bf16x2(acc[i][j][4 * g + 2] * sc[i], acc[i][j][4 * g + 3] * sc[i]);
                *reinterpret_cast<uint2 *>(crow + (((col >> 3) ^ swz) << 3) + (col & 7)) = pk;
            }
    }
}

// LDS rows [0, nrows) of the tile to their token rows of C (row r goes to row tok[r]), columns
// [n0, n0 + BN); rows at or past `valid` are not stored.
template <int BN, int NT>
__device__ __forceinline__ void ctile_to_global(const uint16_t *ct, int nrows, int valid, const int *tok, uint16_t *C,
                                                int N0, int n0, int tid) {
    constexpr int CPR = BN / 8;
#pragma unroll 4
    for (int idx = tid; idx < nrows * CPR; idx += NT) {
        const int r = idx / CPR, c = idx % CPR;
        if (r < valid) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(ct + r * BN + ((c ^ ctile_swz<BN>(r)) << 3));
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(C + (size_t)tok[r] * N0 + n0 + c * 8));
        }
    }
}

// LDS of a bf16 tile configuration: the pipeline stages, or the C tile of the epilogue if larger.
// The C tile goes through LDS in one pass when BM x BN bf16 fits in 144 KiB, otherwise in WGM passes of
// BM / WGM rows (one row band of waves at a time). The accumulate epilogue (second choice of a top-2
// routing) reuses the same bytes for its fp32 passes.
constexpr int ctile_passes(int BM, int BN, int WGM) { return BM * BN * 2 <= 144 * 1024 ? 1 : WGM; }
constexpr size_t gemm_lds_bytes(int BM, int BN, int BK, int NSTAGE, int WGM) {
    const int crows = BM / ctile_passes(BM, BN, WGM);
    return (size_t)(NSTAGE * (BM + BN) * BK > crows * BN ? NSTAGE * (BM + BN) * BK : crows * BN) * 2;
}

// Epilogue of the bf16 grouped GEMMs: the accumulators of wave (wm, wn) (FM x FN blocks of 32 x 32 in the
// C^T layout) go back to their tokens' rows of C, columns [n0, n0 + BN), scaled by p_t for the out-projection;
// with p.accumulate they are added to the values already stored (one rounding of the sum). The LDS bytes of
// the pipeline stages are reused; the caller has no copies in flight.
template <int BM, int BN, int BK, int NSTAGE, int WGM, int WGN, bool OUT>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs &p, f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32], int wm,
                                              int wn, int rows, int n0, uint16_t *C, const int *s_tok,
                                              const float *s_prob, uint16_t *smem) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int FM = WM / 32, FN = WN / 32;
    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
    // epilogue; rows go back to their tokens, scaled by p_t for the out-projection
    if (p.accumulate) {
        // C += result (one rounding of the sum), through LDS in fp32: pass q takes block rows
        // [q*IPP, q*IPP + IPP) of every wave, i.e. rows wm*WM + i*32 + (0..31) of the tile. Register r of block
        // (i, j) holds column 8*(r/4) + 4*half + r%4 of row lane%32; it is written as 4-float chunks
        // (16-byte chunk index XOR-swizzled by the pass row), then every thread adds 8 consecutive columns to
        // the stored bf16 values of a token row with 16-byte loads and stores.
        constexpr int CPR4 = BN / 4;                                  // 16-byte fp32 chunks per row
        constexpr int PROWS = WGM * 32;                               // pass rows per block row
        constexpr int IPP = (int)(gemm_lds_bytes(BM, BN, BK, NSTAGE, WGM) / ((size_t)PROWS * BN * 4));
        static_assert(IPP >= 1, "fp32 accumulate pass");
        constexpr int NPASS = (FM + IPP - 1) / IPP;
        constexpr int SWM = (CPR4 < 32 ? CPR4 : 32) - 1;             // chunk swizzle mask (stays in the row)
        float *ct = reinterpret_cast<float *>(smem);
        auto prow_of = [&](int wmr, int ii, int r) { return (ii * WGM + wmr) * 32 + r; };  // LDS row
        constexpr int CPR = BN / 8;  // 8-column units per row
        constexpr int UNITS = IPP * PROWS * CPR;
        constexpr int UPT = UNITS % NT == 0 ? UNITS / NT : 0;  // units per thread, when they divide evenly
#pragma unroll
        for (int q = 0; q < NPASS; ++q) {
            // the pass's stored values are loaded first, all at once, so that their latency overlaps the LDS
            // pass below instead of one round trip per unit (rows clamped into the tile: every load is in
            // bounds, and only the stored rows are used)
            uint4 old[UPT > 0 ? UPT : 1];
            if constexpr (UPT > 0) {
#pragma unroll
                for (int k = 0; k < UPT; ++k) {
                    const int u = tid + k * NT;
                    const int lr = u / CPR, c = u % CPR;
                    const int ii = lr / PROWS, wmr = (lr / 32) % WGM, i = q * IPP + ii;
                    const int row = min(wmr * WM + i * 32 + (lr & 31), BM - 1);
                    old[k] = *reinterpret_cast<const uint4 *>(C + (size_t)s_tok[row] * p.N0 + n0 + c * 8);
                }
            }
            __syncthreads();
#pragma unroll
            for (int ii = 0; ii < IPP; ++ii) {
                const int i = q * IPP + ii;
                if (i < FM) {
                    const int lr = prow_of(wm, ii, lane & 31);
                    const float sc = OUT ? s_prob[wm * WM + i * 32 + (lane & 31)] : 1.0f;
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int ch = (wn * WN + j * 32 + 8 * g + 4 * half) >> 2;
                            float4 v;
                            v.x = acc[i][j][4 * g] * sc;
                            v.y = acc[i][j][4 * g + 1] * sc;
                            v.z = acc[i][j][4 * g + 2] * sc;
                            v.w = acc[i][j][4 * g + 3] * sc;
                            *reinterpret_cast<float4 *>(ct + lr * BN + ((ch ^ (lr & SWM)) << 2)) = v;
                        }
                }
            }
            __syncthreads();
            // unit u: LDS row lr = u / CPR (tile row wmr * WM + i * 32 + lr % 32), 8 columns from 8 (u % CPR)
            auto add_store = [&](int u, const uint4 &ov) {
                const int lr = u / CPR, c = u % CPR;
                const int ii = lr / PROWS, wmr = (lr / 32) % WGM, i = q * IPP + ii;
                const int row = wmr * WM + i * 32 + (lr & 31);  // tile row
                if (i < FM && row < rows) {
                    uint4 *dst = reinterpret_cast<uint4 *>(C + (size_t)s_tok[row] * p.N0 + n0 + c * 8);
                    const float4 a = *reinterpret_cast<const float4 *>(ct + lr * BN + (((2 * c) ^ (lr & SWM)) << 2));
                    const float4 b = *reinterpret_cast<const float4 *>(ct + lr * BN + (((2 * c + 1) ^ (lr & SWM)) << 2));
                    uint4 pk;
                    pk.x = pack_bf16x2(__uint_as_float(ov.x << 16) + a.x, __uint_as_float(ov.x & 0xFFFF0000u) + a.y);
                    pk.y = pack_bf16x2(__uint_as_float(ov.y << 16) + a.z, __uint_as_float(ov.y & 0xFFFF0000u) + a.w);
                    pk.z = pack_bf16x2(__uint_as_float(ov.z << 16) + b.x, __uint_as_float(ov.z & 0xFFFF0000u) + b.y);
                    pk.w = pack_bf16x2(__uint_as_float(ov.w << 16) + b.z, __uint_as_float(ov.w & 0xFFFF0000u) + b.w);
                    *dst = pk;
                }
            };
            if constexpr (UPT > 0) {
#pragma unroll
                for (int k = 0; k < UPT; ++k) add_store(tid + k * NT, old[k]);
            } else {
                for (int u = tid; u < UNITS; u += NT) {
                    const int lr = u / CPR, c = u % CPR;
                    const int ii = lr / PROWS, wmr = (lr / 32) % WGM, i = q * IPP + ii;
                    const int row = min(wmr * WM + i * 32 + (lr & 31), BM - 1);
                    add_store(u, *reinterpret_cast<const uint4 *>(C + (size_t)s_tok[row] * p.N0 + n0 + c * 8));
                }
            }
        }
        return;
    }
    // through LDS (no copies are in flight after the last step), in one pass or one band of waves at a time
    float sc[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) sc[i] = OUT ? s_prob[wm * WM + i * 32 + (lane & 31)] : 1.0f;
    constexpr int PASSES = ctile_passes(BM, BN, WGM);
    if constexpr (PASSES == 1) {
        __syncthreads();
        acc_to_ctile<FM, FN, BN>(acc, smem, wm * WM, wn * WN, lane, sc);
        __syncthreads();
        ctile_to_global<BN, NT>(smem, BM, rows, s_tok, C, p.N0, n0, tid);
    } else {
#pragma unroll
        for (int q = 0; q < PASSES; ++q) {
            __syncthreads();
            if (wm == q) acc_to_ctile<FM, FN, BN>(acc, smem, 0, wn * WN, lane, sc);
            __syncthreads();
            ctile_to_global<BN, NT>(smem, WM, rows - q * WM, s_tok + q * WM, C, p.N0, n0, tid);
        }
    }
}

template <int BM, int BN, int BK, int NSTAGE, int WGM, int WGN, bool OUT, int SCHED, bool KSPLIT>
__global__ __launch_bounds__(64 * WGM * WGN) void k_grouped_gemm_bf16(GemmArgs p) {
    constexpr int NW = WGM * WGN;
    constexpr int NT = 64 * NW;
    constexpr int KCH = BK / 8;                     // 16-byte chunks per LDS row
    constexpr int RG = 64 / KCH;                    // rows covered by one wave-wide 1 KiB copy
    constexpr int A_DMA = BM / RG / NW;             // copy instructions per wave per K step
    constexpr int B_DMA = BN / RG / NW;
    constexpr int PER_STEP = A_DMA + B_DMA;
    constexpr int STAGE = (BM + BN) * BK;           // bf16 elements per stage
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int FM = WM / 32, FN = WN / 32;
    static_assert(BK == 64 || BK == 32, "BK");
    static_assert((BM / RG) % NW == 0 && A_DMA >= 1 && (BN / RG) % NW == 0 && B_DMA >= 1, "copy split");
    static_assert(NSTAGE >= 2 && NSTAGE <= 5 && FM >= 1 && FN >= 1, "shape");

    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    __shared__ int s_tok[BM];
    __shared__ int s_arow[BM];
    __shared__ float s_prob[OUT ? BM : 1];

    // the wave index read as a uniform value: the copies' LDS destinations are then computed on the scalar unit and
    // moved to M0 directly, with no v_readfirstlane per copy after each step's barrier (skewed block in-projection
    // 1907-1946 -> 1868-1870 us, two interleaved runs)
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int mt, nt, e, slot0, rows;
    if (!tile_of_block(p, mt, nt)) return;
    if (!locate_mtile<BM>(p.offsets, p.E, mt, e, slot0, rows)) return;
    const int which = nt / p.n_tiles_per_b;
    const int n0 = (nt % p.n_tiles_per_b) * BN;
    const int K = p.K;
    const uint16_t *Bsrc = static_cast<const uint16_t *>(which ? p.B1 : p.B0) + ((size_t)e * p.N0 + n0) * K;
    uint16_t *C = static_cast<uint16_t *>(which ? p.C1 : p.C0);

    // rows past the group's end repeat its last row (in-bounds, finite data); they are never stored
    for (int i = tid; i < BM; i += NT) {
        const int slot = slot0 + min(i, rows - 1);
        const int tok = p.perm[slot];
        s_tok[i] = tok;
        s_arow[i] = (OUT && !p.a_by_token) ? slot : tok;
        if (OUT) s_prob[i] = p.prob[tok];
    }
    __syncthreads();

    // ---- per-lane copy sources. Copy group g covers rows [g*RG, g*RG+RG); lane i fills row
    // g*RG + i/KCH, physical chunk i%KCH, i.e. logical chunk (i%KCH) ^ swz(row).
    const int dr = lane / KCH, dpc = lane % KCH;
    const uint16_t *a_dma[A_DMA];
    const uint16_t *b_dma[B_DMA];
    const int k_lo = KSPLIT ? p.k_split : K;  // row length of A0
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) {
        const int row = (wave * A_DMA + j) * RG + dr;
        const int c = dpc ^ lds_swz<KCH>(row);
        a_dma[j] = static_cast<const uint16_t *>(p.A0) + (size_t)s_arow[row] * k_lo + c * 8;
    }
#pragma unroll
    for (int j = 0; j < B_DMA; ++j) {
        const int row = (wave * B_DMA + j) * RG + dr;
        const int c = dpc ^ lds_swz<KCH>(row);
        b_dma[j] = Bsrc + (size_t)row * K + c * 8;
    }
    // KSPLIT: copies are issued in increasing k, so the A sources switch to A_hi once, at the first step at
    // or past k_split (rows re-read from LDS; a second pointer set would cost registers all along)
    bool a_in_hi = false;
    auto issue_copies = [&](int kt, int stage) {
        uint16_t *as = smem + stage * STAGE;
        uint16_t *bs = as + BM * BK;
        const int k0 = kt * BK;
        if (KSPLIT && !a_in_hi && k0 >= k_lo) {  // uniform
#pragma unroll
            for (int j = 0; j < A_DMA; ++j) {
                const int row = (wave * A_DMA + j) * RG + dr;
                const int c = dpc ^ lds_swz<KCH>(row);
                a_dma[j] = static_cast<const uint16_t *>(p.A_hi) + (size_t)s_arow[row] * (K - k_lo) + c * 8;
            }
            a_in_hi = true;
        }
        const int ka = KSPLIT && a_in_hi ? k0 - k_lo : k0;
#pragma unroll
        for (int j = 0; j < A_DMA; ++j) dma16_to_lds(a_dma[j] + ka, as + (wave * A_DMA + j) * RG * BK);
#pragma unroll
        for (int j = 0; j < B_DMA; ++j) dma16_to_lds(b_dma[j] + k0, bs + (wave * B_DMA + j) * RG * BK);
    };
    // the same in two halves: the source addresses of step kt (prep_copies, before the barrier, under the step's
    // last MFMAs) and the copies into `stage` (fire_copies, after it), so that little but the copies themselves
    // lies between the barrier and the next MFMAs (skewed block in-projection 1884-1887 -> 1851-1859 us)
    const uint16_t *ca[A_DMA], *cb[B_DMA];
    auto prep_copies = [&](int kt) {
        const int k0 = kt * BK;
        if (KSPLIT && !a_in_hi && k0 >= k_lo) {  // uniform
#pragma unroll
            for (int j = 0; j < A_DMA; ++j) {
                const int row = (wave * A_DMA + j) * RG + dr;
                const int c = dpc ^ lds_swz<KCH>(row);
                a_dma[j] = static_cast<const uint16_t *>(p.A_hi) + (size_t)s_arow[row] * (K - k_lo) + c * 8;
            }
            a_in_hi = true;
        }
        const int ka = KSPLIT && a_in_hi ? k0 - k_lo : k0;
#pragma unroll
        for (int j = 0; j < A_DMA; ++j) ca[j] = a_dma[j] + ka;
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

    // fragment addresses (element offsets within a stage); rows of a fragment differ by multiples
    // of 32, so they share one swizzle
    int a_frag[FM], b_frag[FN];
    const int half = lane >> 5;
#pragma unroll
    for (int i = 0; i < FM; ++i) a_frag[i] = (wm * WM + i * 32 + (lane & 31)) * BK;
#pragma unroll
    for (int j = 0; j < FN; ++j) b_frag[j] = BM * BK + (wn * WN + j * 32 + (lane & 31)) * BK;
    const int swz = lds_swz<KCH>(lane & 31);

    auto compute = [&](int stage) {
        const uint16_t *st = smem + stage * STAGE;
        bf16x8 af[2][FM], bfr[2][FN];
        auto load_frags = [&](int kk, int set) {
            const int co = ((kk * 2 + half) ^ swz) * 8;
#pragma unroll
            for (int i = 0; i < FM; ++i) af[set][i] = *reinterpret_cast<const bf16x8 *>(st + a_frag[i] + co);
#pragma unroll
            for (int j = 0; j < FN; ++j) bfr[set][j] = *reinterpret_cast<const bf16x8 *>(st + b_frag[j] + co);
        };
        load_frags(0, 0);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            if (kk + 1 < BK / 16) load_frags(kk + 1, (kk + 1) & 1);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[kk & 1][j], af[kk & 1][i], acc[i][j], 0, 0, 0);
        }
        if (SCHED == 1) {
            // issue order: the first sub-step's fragment reads, then for every sub-step but the last its
            // MFMAs with the next sub-step's fragment reads slotted between them, then the last MFMAs
            constexpr int NR = FM + FN, NM = FM * FN;
            __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
            for (int kk = 0; kk + 1 < BK / 16; ++kk) {
#pragma unroll
                for (int q = 0; q < NR; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                if (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
        }
    };

    const int nk = K / BK;
    if constexpr (SCHED == 2) {
        // Early-barrier schedule: once a wave's fragment reads of stage kt and its copies of step kt+1
        // are complete it joins the barrier, then issues the copies of step kt+NSTAGE into the stage just
        // read and the first fragment reads of step kt+1, and only then the last MFMAs of step kt, which
        // cover the latency of those reads. Copies are in flight for NSTAGE-1 steps. The loop body is one
        // block split only by the barrier: steps past the last copy the last step's data again into a
        // stage that no later step reads (in bounds, never read), so the number of copies in flight is
        // the same at every barrier and the fragment reads can be slotted between the MFMAs.
        constexpr int NKK = BK / 16;  // MFMA sub-steps per K step
        static_assert(NKK == 2 || NKK == 4, "early-barrier schedule");
        constexpr int NR = FM + FN, NM = FM * FN;
        constexpr int NG = (NR + 1) / 2;  // MFMAs that get fragment reads slotted after them
        static_assert(NM > NG, "read slots");
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
        // issue order of one sub-step: an MFMA, two fragment reads of the next sub-step, ..., then the
        // remaining MFMAs
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
        auto barrier = [&]() {
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
        };
        // sub-steps 0 .. NKK-2 of the step in `stage`, each with the next sub-step's reads
        auto body = [&](int stg) {
#pragma unroll
            for (int kk = 1; kk < NKK; ++kk) {
                load_frags(stg, kk, kk & 1);
                mfmas((kk - 1) & 1);
            }
#pragma unroll
            for (int kk = 1; kk < NKK; ++kk) slot_reads();
        };
#pragma unroll
        for (int s = 0; s + 1 < NSTAGE; ++s) issue_copies(min(s, nk - 1), s);
        wait_copies<PER_STEP, NSTAGE - 2>(NSTAGE - 2);
        barrier();
        issue_copies(min(NSTAGE - 1, nk - 1), NSTAGE - 1);
        load_frags(0, 0, 0);
        int stage = 0;
        for (int kt = 0; kt + 1 < nk; ++kt) {
            body(stage);
            prep_copies(min(kt + NSTAGE, nk - 1));
            __builtin_amdgcn_sched_barrier(0);  // the step's MFMAs stay ahead of the wait (they cover the reads)
            wait_copies<PER_STEP, NSTAGE - 2>(NSTAGE - 2);
            barrier();
            fire_copies(stage);
            const int next = stage + 1 == NSTAGE ? 0 : stage + 1;
            load_frags(next, 0, 0);
            mfmas((NKK - 1) & 1);
            __builtin_amdgcn_sched_group_barrier(0x020, PER_STEP, 0);
            slot_reads();
            stage = next;
        }
        body(stage);
        mfmas((NKK - 1) & 1);
        wait_copies<PER_STEP, 0>(0);  // the spare copies
    } else {
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s)
        if (s < nk) issue_copies(s, s);
    int stage = 0;
    for (int kt = 0; kt < nk; ++kt) {
        // step kt's copies have landed once at most the later steps' copies are in flight; this
        // wave's LDS reads of the previous step are done at lgkmcnt(0). Then a plain s_barrier: a
        // full __syncthreads() fence would also wait for the copies of later steps.
        wait_copies<PER_STEP, NSTAGE - 2>(min(NSTAGE - 2, nk - 1 - kt));
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (kt + NSTAGE - 1 < nk) issue_copies(kt + NSTAGE - 1, (stage + NSTAGE - 1) % NSTAGE);
        compute(stage);
        stage = (stage + 1) % NSTAGE;
    }
    }

    gemm_epilogue<BM, BN, BK, NSTAGE, WGM, WGN, OUT>(p, acc, wm, wn, rows, n0, C, s_tok, s_prob, smem);
}

// ---------------------------------------------------------------------------------------------
// Gate and permute for the out-projection (bf16): a[pos][n] = bf16(SiLU(z[t][n]) * h[t][n]) with
// t = perm[pos], fp32 arithmetic, rows written in slot order so the GEMM reads each expert's rows
// contiguously; with perm == NULL, t = pos (token order, shared by the two choices of a top-2 routing
// and by the decode kernels). Memory-bound: a workgroup owns gate_rows_per_wg(d_inner) consecutive
// output rows (about 1024 16-byte chunks) and its 256 threads stride over their chunks, 4 chunks of z
// and h in flight per thread, so even a single row is spread over the whole workgroup. The row of
// chunk unit u is u / cpr, computed as umulhi(u, cpr_magic) with cpr_magic = floor(2^32 / cpr) + 1,
// exact for every u below rows_per_wg * cpr and cpr < 2^16 (an integer division would cost more than
// the memory traffic).
inline int gate_rows_per_wg(int di) { return di / 8 >= 1024 ? 1 : 1024 / (di / 8); }
inline uint32_t gate_cpr_magic(int di) { return (uint32_t)((1ull << 32) / (uint64_t)(di / 8) + 1); }

__global__ __launch_bounds__(256) void k_gate_permute(const uint16_t *__restrict__ z, const uint16_t *__restrict__ h,
                                                      const int32_t *__restrict__ perm, int T, int di, int rows_per_wg,
                                                      uint32_t cpr_magic, uint16_t *__restrict__ a) {
    const int cpr = di >> 3;  // 16-byte chunks per row
    const int r0 = blockIdx.x * rows_per_wg;
    const int n = min(rows_per_wg, T - r0) * cpr;  // chunk units of this workgroup
    for (int ub = threadIdx.x; ub < n; ub += 4 * 256) {
        uint4 zv[4], hv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int u = min(ub + j * 256, n - 1);  // clamped: every load is in bounds
            const int rr = (int)__umulhi((uint32_t)u, cpr_magic), c = u - rr * cpr;
            const int pos = r0 + rr;
            const int tok = perm != nullptr ? perm[pos] : pos;
            zv[j] = reinterpret_cast<const uint4 *>(z + (size_t)tok * di)[c];
            hv[j] = reinterpret_cast<const uint4 *>(h + (size_t)tok * di)[c];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t zw[4] = {zv[j].x, zv[j].y, zv[j].z, zv[j].w};
            const uint32_t hw[4] = {hv[j].x, hv[j].y, hv[j].z, hv[j].w};
            uint32_t o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float z0 = __uint_as_float(zw[q] << 16), z1 = __uint_as_float(zw[q] & 0xFFFF0000u);
                const float h0 = __uint_as_float(hw[q] << 16), h1 = __uint_as_float(hw[q] & 0xFFFF0000u);
                o[q] = pack_bf16x2(silu_fast(z0) * h0, silu_fast(z1) * h1);
            }
            if (ub + j * 256 < n) {
                const int u = ub + j * 256;
                const int rr = (int)__umulhi((uint32_t)u, cpr_magic), c = u - rr * cpr;
                reinterpret_cast<uint4 *>(a + (size_t)(r0 + rr) * di)[c] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// fp32 grouped GEMM (fp32 storage; plain FMA, fp32 accumulation). 64x64 tiles, BK = 16, 256
// threads, 4x4 outputs per thread. Used for fp32 data, where exact fp32 products are wanted.
template <bool OUT>
__global__ __launch_bounds__(256) void k_grouped_gemm_f32(GemmArgs p) {
    constexpr int BM = 64, BN = 64, BK = 16;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[BK][BN + 4];
    __shared__ int s_tok[BM];
    __shared__ float s_prob[BM];
    const int tid = threadIdx.x;
    const int mt = blockIdx.x / p.n_tiles, nt = blockIdx.x % p.n_tiles;
    int e, slot0, rows;
    if (!locate_mtile<BM>(p.offsets, p.E, mt, e, slot0, rows)) return;
    const int which = nt / p.n_tiles_per_b;
    const int n0 = (nt % p.n_tiles_per_b) * BN;
    const int K = p.K;
    const float *Bsrc = static_cast<const float *>(which ? p.B1 : p.B0) + ((size_t)e * p.N0 + n0) * K;
    float *C = static_cast<float *>(which ? p.C1 : p.C0);
    if (tid < BM) {
        const int tok = tid < rows ? p.perm[slot0 + tid] : -1;
        s_tok[tid] = tok;
        s_prob[tid] = (OUT && tok >= 0) ? p.prob[tok] : 0.0f;
    }
    __syncthreads();
    const int lr = tid >> 2, lk = (tid & 3) * 4;  // row 0..63, k offset 0,4,8,12
    const int tok = s_tok[lr];
    const float *a_src = tok >= 0 ? static_cast<const float *>(p.A0) + (size_t)tok * K + lk : nullptr;
    const float *h_src =
        (OUT && p.A1 != nullptr && tok >= 0) ? static_cast<const float *>(p.A1) + (size_t)tok * K + lk : nullptr;
    const float *b_src = Bsrc + (size_t)lr * K + lk;
    const int ty = tid >> 4, tx = tid & 15;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += BK) {
        float4 a = a_src ? *reinterpret_cast<const float4 *>(a_src + k0) : make_float4(0, 0, 0, 0);
        if (OUT && h_src) {
            const float4 h = *reinterpret_cast<const float4 *>(h_src + k0);
            a.x = silu_precise(a.x) * h.x;
            a.y = silu_precise(a.y) * h.y;
            a.z = silu_precise(a.z) * h.z;
            a.w = silu_precise(a.w) * h.w;
        }
        const float4 b = *reinterpret_cast<const float4 *>(b_src + k0);
        As[lk + 0][lr] = a.x; As[lk + 1][lr] = a.y; As[lk + 2][lr] = a.z; As[lk + 3][lr] = a.w;
        Bs[lk + 0][lr] = b.x; Bs[lk + 1][lr] = b.y; Bs[lk + 2][lr] = b.z; Bs[lk + 3][lr] = b.w;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            float av[4], bv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) { av[q] = As[k][ty * 4 + q]; bv[q] = Bs[k][tx * 4 + q]; }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = ty * 4 + i;
        if (row < rows) {
            const int t = s_tok[row];
            const float sc = OUT ? s_prob[row] : 1.0f;
            float4 v = make_float4(acc[i][0] * sc, acc[i][1] * sc, acc[i][2] * sc, acc[i][3] * sc);
            float4 *dst = reinterpret_cast<float4 *>(C + (size_t)t * p.N0 + n0 + tx * 4);
            if (p.accumulate) {
                const float4 o = *dst;
                v = make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w);
            }
            *dst = v;
        }
    }
}

// ---------------------------------------------------------------------------------------------


// XCD-aware grouping of M-tiles (0 = off); ROM_GROUP_M overrides it for tuning sweeps.
static int env_int(const char *name, int dflt, int lo, int hi) {
    const char *v = getenv(name);
    const int c = v ? atoi(v) : dflt;
    return (c < lo || c > hi) ? dflt : c;
}
// read once per process (thread-safe static initialisation)
static int group_m_choice() {
    static const int v = env_int("ROM_GROUP_M", 0, 0, 64);
    return v;
}

template <int BM, int BN, int BK, int NSTAGE, int WGM, int WGN, bool OUT, int SCHED, bool KSPLIT>
static hipError_t launch_bf16(const GemmArgs &a0, int nB, hipStream_t s) {
    GemmArgs a = a0;
    a.n_tiles_per_b = a.N0 / BN;
    a.n_tiles = nB * a.n_tiles_per_b;
    a.m_tiles = (a.T + a.E * (BM - 1)) / BM;
    a.group_m = group_m_choice();
    unsigned grid;
    if (a.group_m > 0) {
        const int groups = (a.m_tiles + a.group_m - 1) / a.group_m;
        const long total = (long)groups * a.group_m * a.n_tiles;
        a.per_xcd = max(1, device_cus() / 8);
        const long round = 8L * a.per_xcd;
        grid = (unsigned)((total + round - 1) / round * round);
    } else {
        grid = (unsigned)a.m_tiles * a.n_tiles;
    }
    const size_t smem = gemm_lds_bytes(BM, BN, BK, NSTAGE, WGM);
    static LdsAttrOnce attr;
    hipError_t err = set_lds_limit_once(
        attr, reinterpret_cast<const void *>(&k_grouped_gemm_bf16<BM, BN, BK, NSTAGE, WGM, WGN, OUT, SCHED, KSPLIT>),
        smem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((k_grouped_gemm_bf16<BM, BN, BK, NSTAGE, WGM, WGN, OUT, SCHED, KSPLIT>), dim3(grid), dim3(64 * WGM * WGN),
                       smem, s, a);
    return hipGetLastError();
}

// Tile shapes available to the bf16 path.
struct TileCfg { int bm, bn, bk, nstage, wgm, wgn, sched; };
constexpr TileCfg kTiles[] = {
    {256, 256, 64, 2, 2, 4, 0},  // 0: 8 waves (128x64 each), BK 64, 2 stages (128 KiB LDS)
    {256, 256, 32, 4, 2, 4, 0},  // 1: 8 waves, BK 32, 4 stages (128 KiB)
    {256, 256, 64, 2, 2, 4, 1},  // 2: as 0, fragment reads interleaved with the MFMAs
    {256, 128, 64, 3, 2, 2, 0},  // 3: 4 waves (128x64 each), BK 64, 3 stages (144 KiB)
    {128, 128, 64, 4, 2, 2, 0},  // 4: 4 waves (64x64 each), BK 64, 4 stages (128 KiB)
    {128, 64, 64, 4, 2, 2, 0},   // 5: 4 waves (64x32 each), BK 64, 4 stages (96 KiB)
    {256, 256, 32, 4, 2, 4, 1},  // 6: as 1, interleaved
    {320, 256, 64, 2, 2, 4, 1},  // 7: 8 waves (160x64 each), BK 64, 2 stages (144 KiB), C tile in 2 passes
    {256, 256, 64, 2, 2, 4, 2},  // 8: as 0, barrier ahead of each step's last MFMAs
    {320, 256, 64, 2, 2, 4, 2},  // 9: as 7, barrier ahead of each step's last MFMAs
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

// Optional override of the tile choice (tuning sweeps): ROM_TILE_IN / ROM_TILE_OUT = index above.
static int tile_override(bool out) {
    static const int in_v = env_int("ROM_TILE_IN", -1, 0, kNumTiles - 1);
    static const int out_v = env_int("ROM_TILE_OUT", -1, 0, kNumTiles - 1);
    return out ? out_v : in_v;
}


// Default tile shape by problem: with enough rows and columns, 8-wave blocks of 320 x 256 or 256 x 256 with
// the early-barrier schedule (measured best on MI355X at T = 16384 and 65536). 320-row blocks move 10% fewer
// operand bytes per flop (operand copies, not MFMAs, limit these kernels), so they are taken unless their extra
// padding is large: the launch's upper bound on padded rows, T + E*(BM-1), must grow by at most 5% over
// 256-row blocks, or the 320-row blocks must need fewer rounds of workgroups over the compute units for the
// same rows (rounds x rows per tile smaller; the host never reads the expert counts). Smaller blocks for small T
// or narrow N.
static int default_tile(const GemmArgs &a, int nB) {
    if (a.T >= 4096 && a.N0 % 256 == 0) {
        const long cus = device_cus(), nt = (long)nB * (a.N0 / 256);
        const long rows256 = a.T + (long)a.E * 255, rows320 = a.T + (long)a.E * 319;
        const long t256 = rows256 / 256 * nt, t320 = rows320 / 320 * nt;
        const long r256 = (t256 + cus - 1) / cus, r320 = (t320 + cus - 1) / cus;
        if (rows320 * 20 <= rows256 * 21 || r320 * 320 < r256 * 256) return 9;
        return 8;
    }
    if (a.N0 % 128 == 0) return 4;
    return 5;
}

template <bool OUT, bool KSPLIT = false>
static hipError_t launch_bf16_auto(const GemmArgs &a, int nB, hipStream_t s) {
    int t = tile_override(OUT);
    if (t < 0 || a.N0 % kTiles[t].bn != 0) t = default_tile(a, nB);
    switch (t) {
        case 0: return launch_bf16<256, 256, 64, 2, 2, 4, OUT, 0, KSPLIT>(a, nB, s);
        case 1: return launch_bf16<256, 256, 32, 4, 2, 4, OUT, 0, KSPLIT>(a, nB, s);
        case 2: return launch_bf16<256, 256, 64, 2, 2, 4, OUT, 1, KSPLIT>(a, nB, s);
        case 3: return launch_bf16<256, 128, 64, 3, 2, 2, OUT, 0, KSPLIT>(a, nB, s);
        case 4: return launch_bf16<128, 128, 64, 4, 2, 2, OUT, 0, KSPLIT>(a, nB, s);
        case 6: return launch_bf16<256, 256, 32, 4, 2, 4, OUT, 1, KSPLIT>(a, nB, s);
        case 7: return launch_bf16<320, 256, 64, 2, 2, 4, OUT, 1, KSPLIT>(a, nB, s);
        case 8: return launch_bf16<256, 256, 64, 2, 2, 4, OUT, 2, KSPLIT>(a, nB, s);
        case 9: return launch_bf16<320, 256, 64, 2, 2, 4, OUT, 2, KSPLIT>(a, nB, s);
        default: return launch_bf16<128, 64, 64, 4, 2, 2, OUT, 0, KSPLIT>(a, nB, s);
    }
}

template <bool OUT>
static hipError_t launch_f32(const GemmArgs &a0, int nB, hipStream_t s) {
    GemmArgs a = a0;
    a.n_tiles_per_b = a.N0 / 64;
    a.n_tiles = nB * a.n_tiles_per_b;
    const int max_mtiles = (a.T + a.E * 63) / 64;
    hipLaunchKernelGGL((k_grouped_gemm_f32<OUT>), dim3((unsigned)max_mtiles * a.n_tiles), dim3(256), 0, s, a);
    return hipGetLastError();
}

// Choice k of a stacked top-K routing as the arguments of one top-1 grouped product: the second choice
// adds to what the first wrote.
static void set_choice(GemmArgs &a, const rom_routing &r, int T, int k) {
    a.offsets = r.offsets + k * (r.E + 1);
    a.perm = r.perm + (size_t)k * T;
    a.prob = r.prob + (size_t)k * T;
    a.accumulate = k > 0;
}

hipError_t launch_in_proj(const void *X, const rom_routing &r, rom_dtype dt, int T, int dm, int di, const void *Wc,
                          const void *Wg, void *x_out, void *z_out, hipStream_t s) {
    GemmArgs a{};
    a.A0 = X;
    a.B0 = Wc;
    a.B1 = Wg;
    a.C0 = x_out;
    a.C1 = z_out;
    a.T = T;
    a.K = dm;
    a.N0 = di;
    a.E = r.E;
    for (int k = 0; k < r.top_k; ++k) {
        set_choice(a, r, T, k);
        hipError_t err;
        if (dt == ROM_DTYPE_F32) err = launch_f32<false>(a, 2, s);
        else if (gemv_lds_fits(T, dm)) err = launch_gemv_lds_bf16(a, false, false, 2, s);
        else if (gemv_wide_fits(T, r.E, di, dm, 2)) err = launch_gemv_wide_bf16(a, false, 2, s);
        else if (T <= kDecodeMaxT) err = launch_gemv_bf16(a, false, 2, s);
        else err = launch_bf16_auto<false>(a, 2, s);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

hipError_t launch_out_proj(const void *z, const void *h, const rom_routing &r, rom_dtype dt, int T, int dm, int di,
                           const void *Wo, void *out, void *workspace, hipStream_t s) {
    GemmArgs a{};
    a.A0 = z;
    a.A1 = h;
    a.B0 = Wo;
    a.C0 = out;
    a.T = T;
    a.K = di;
    a.N0 = dm;
    a.E = r.E;
    if (dt == ROM_DTYPE_BF16 && gemv_lds_fits(T, di)) {
        // the smallest T: the decode kernel gates the token rows itself while staging them in LDS
        for (int k = 0; k < r.top_k; ++k) {
            set_choice(a, r, T, k);
            hipError_t err = launch_gemv_lds_bf16(a, true, true, 1, s);
            if (err != hipSuccess) return err;
        }
        return hipSuccess;
    }
    if (dt == ROM_DTYPE_BF16) {
        // gated rows a = bf16(SiLU(z) * h) into the workspace, once per token: in slot order for top-1 at
        // T > 64 (the GEMM then reads each expert's rows contiguously), otherwise in token order (both
        // choices of a top-2 routing, and the decode kernels, gather rows from it)
        const bool slot_order = r.top_k == 1 && T > kDecodeMaxT;
        const int rpw = gate_rows_per_wg(di);
        hipLaunchKernelGGL(k_gate_permute, dim3((unsigned)((T + rpw - 1) / rpw)), dim3(256), 0, s,
                           static_cast<const uint16_t *>(z), static_cast<const uint16_t *>(h),
                           slot_order ? r.perm : nullptr, T, di, rpw, gate_cpr_magic(di),
                           static_cast<uint16_t *>(workspace));
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        a.A0 = workspace;
        a.A1 = nullptr;
        a.a_by_token = !slot_order;
    }
    for (int k = 0; k < r.top_k; ++k) {
        set_choice(a, r, T, k);
        hipError_t err;
        if (dt == ROM_DTYPE_F32) err = launch_f32<true>(a, 1, s);
        else if (gemv_wide_fits(T, r.E, dm, di, 1)) err = launch_gemv_wide_bf16(a, true, 1, s);
        else if (T <= kDecodeMaxT) err = launch_gemv_bf16(a, true, 1, s);
        else err = launch_bf16_auto<true>(a, 1, s);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

// Routing-weighted in-projection (Swimba): y[t] = sum over the token's choices of p_t,e * W[e] X[t]. It is
// the out-projection's grouped product (probability-scaled epilogue, rows gathered in token order through
// perm) applied to X itself, with no gate.
hipError_t launch_in_proj_weighted(const void *X, const rom_routing &r, rom_dtype dt, int T, int dm, int dout,
                                   const void *W, void *y, hipStream_t s) {
    GemmArgs a{};
    a.A0 = X;
    a.A1 = nullptr;
    a.B0 = W;
    a.C0 = y;
    a.T = T;
    a.K = dm;
    a.N0 = dout;
    a.E = r.E;
    a.a_by_token = 1;
    for (int k = 0; k < r.top_k; ++k) {
        set_choice(a, r, T, k);
        hipError_t err;
        if (dt == ROM_DTYPE_F32) err = launch_f32<true>(a, 1, s);
        else if (gemv_lds_fits(T, dm)) err = launch_gemv_lds_bf16(a, true, false, 1, s);
        else if (gemv_wide_fits(T, r.E, dout, dm, 1)) err = launch_gemv_wide_bf16(a, true, 1, s);
        else if (T <= kDecodeMaxT) err = launch_gemv_bf16(a, true, 1, s);
        else err = launch_bf16_auto<true>(a, 1, s);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

hipError_t launch_grouped_bf16(const GemmArgs &a, bool out, int nB, hipStream_t s) {
    if (a.k_split > 0) return out ? hipErrorInvalidValue : launch_bf16_auto<false, true>(a, nB, s);
    return out ? launch_bf16_auto<true>(a, nB, s) : launch_bf16_auto<false>(a, nB, s);
}

size_t out_proj_workspace_bytes(int T, int di, rom_dtype dt) {
    if (dt != ROM_DTYPE_BF16) return 0;
    return (size_t)T * di * sizeof(uint16_t);
}

}  // namespace rom
