// rom_gemv.hip -- decode-size (T <= 64) grouped projections of the Routing Mamba experts on gfx950.
//
// Method: Routing Mamba landing page (chapterpal.com), Knowl 1: the same expert products as rom_gemm.hip
// (x = W_conv[e] X, z = W_gate[e] X; out = p W_out[e] (SiLU(z) * h); Swimba's y = p W_in[e] X). With a few
// tokens per expert the cost is streaming each active expert's weights from HBM once: these kernels give every
// workgroup 16 to 256 weight rows of one active expert and all of that expert's tokens, and use 16x16x32
// MFMAs only to apply each weight fragment to up to 16 tokens at once. Three kernels: k_grouped_gemv_bf16
// (both operands' fragments from memory into registers), k_grouped_gemv_lds (the smallest T: the token rows
// staged in LDS once, the out-projection's gate computed there), k_grouped_gemv_wide (17..64 tokens: 16 waves
// over up to 256 rows, the token rows staged through LDS in K chunks).
#include "rom_device.h"
#include "rom_gemm.h"
#include "rom_internal.h"

namespace rom {

// ---------------------------------------------------------------------------------------------
// Decode path (T <= 64): the cost is streaming each active expert's weights from HBM once; the MFMA
// work is tiny. A workgroup owns RB blocks of 16 weight rows of one expert and every token routed to it
// (at most 64, i.e. NB blocks of 16), and its NW waves split K. The weight fragment of a 16x16x32 MFMA
// comes straight from global memory (lane l: row l%16, 8 elements at k + 8*(l/16)), the token fragments
// likewise through perm (for the out-projection, from the gated rows k_gate_permute wrote in token
// order: the gate is evaluated once per token, not once per workgroup and padding column); each wave
// keeps U K-steps of loads in flight. Every workgroup reads all of its expert's token rows, so with more
// tokens (RB = 2 from 32 tokens on) a workgroup takes 32 weight rows and the token rows are read half as
// often. Partial sums of the waves are added in wave order through LDS (deterministic), then scaled
// (out-projection) and stored.
// Grid: (weight rows / (16 RB)) x min(E, T): the second index is the rank among experts that received
// tokens; each workgroup runs the variant sized for its expert's token-block count.
template <int NW, int RB, int NB, int U, bool OUT>
__device__ __forceinline__ void gemv_block(const GemmArgs &p, int e, int o0, int ne, int rb,
                                           float (*s_red)[RB * 4][16][16]) {
    constexpr int NT = 64 * NW;
    __shared__ int s_tok[64];
    __shared__ float s_prob[64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nglob = rb * 16 * RB;  // N0 is a multiple of 64, so the RB blocks lie in one output
    const int which = nglob / p.N0, n0 = nglob % p.N0;
    const int K = p.K;
    const uint16_t *W = static_cast<const uint16_t *>(which ? p.B1 : p.B0) + ((size_t)e * p.N0 + n0) * K;
    uint16_t *C = static_cast<uint16_t *>(which ? p.C1 : p.C0);
    const int tok_first = p.perm[o0];
    for (int i = tid; i < 64; i += NT) {
        const int tok = i < ne ? p.perm[o0 + i] : tok_first;
        s_tok[i] = tok;
        s_prob[i] = OUT ? p.prob[tok] : 1.0f;
    }
    __syncthreads();

    const int r = lane & 15, g = lane >> 4;
    const uint16_t *wp[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) wp[j] = W + (size_t)(j * 16 + r) * K + g * 8;
    const uint16_t *xp[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) xp[b] = static_cast<const uint16_t *>(p.A0) + (size_t)s_tok[b * 16 + r] * K + g * 8;
    f32x4 acc[RB][NB];
#pragma unroll
    for (int j = 0; j < RB; ++j)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[j][b] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // U K-steps of loads in flight per wave (indices clamped, so every load is in bounds), then their MFMAs.
    // With 8 waves each wave streams a contiguous K range (U consecutive steps: 32 U contiguous elements of
    // each row per batch); with 16 waves the steps are interleaved (the 16 waves' loads of one batch cover
    // 16 consecutive steps), which measured faster for the one-workgroup-per-CU launch.
    constexpr bool CONTIG = NW == 8;
    const int nsteps = K / 32;
    const int spw = CONTIG ? (nsteps + NW - 1) / NW : 0;
    const int sbeg = CONTIG ? wave * spw : wave, send = CONTIG ? min(nsteps, sbeg + spw) : nsteps;
    constexpr int SU = CONTIG ? 1 : NW;  // step stride within a batch
    for (int s0 = sbeg; s0 < send; s0 += SU * U) {
        bf16x8 wf[U][RB], xf[U][NB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k0 = min(s0 + u * SU, send - 1) * 32;
#pragma unroll
            for (int j = 0; j < RB; ++j) wf[u][j] = *reinterpret_cast<const bf16x8 *>(wp[j] + k0);
#pragma unroll
            for (int b = 0; b < NB; ++b) xf[u][b] = *reinterpret_cast<const bf16x8 *>(xp[b] + k0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (s0 + u * SU < send) {  // uniform
#pragma unroll
                for (int j = 0; j < RB; ++j)
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        acc[j][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u][j], xf[u][b], acc[j][b], 0, 0, 0);
            }
        }
    }
    // accumulator register i of lane l: weight row 4*(l/16) + i (of block j), token column l%16
#pragma unroll
    for (int j = 0; j < RB; ++j)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_red[wave][j * NB + b][4 * g + i][r] = acc[j][b][i];
    __syncthreads();
    for (int idx = tid; idx < RB * NB * 256; idx += NT) {
        const int jb = idx >> 8, n = (idx >> 4) & 15, m = idx & 15;
        const int j = jb / NB, b = jb - j * NB;
        const int col = b * 16 + m;
        if (col < ne) {
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) v += s_red[w][jb][n][m];
            uint16_t *dst = C + (size_t)s_tok[col] * p.N0 + n0 + j * 16 + n;
            *dst = f32_to_bf16(p.accumulate ? fmaf(v, s_prob[col], bf16_to_f32(*dst)) : v * s_prob[col]);
        }
    }
}

// NBMAX: the most token blocks any expert can hold (T <= 16 NBMAX), so that small T instantiates only the
// small variants and keeps fewer registers.
template <int NW, int RB, int NBMAX, bool OUT>
__global__ __launch_bounds__(64 * NW) void k_grouped_gemv_bf16(GemmArgs p) {
    __shared__ float s_red[NW][RB * 4][16][16];
    const int rb = blockIdx.x % p.n_tiles, rank = blockIdx.x / p.n_tiles;
    int e = -1, o0 = 0, ne = 0;
    for (int i = 0, j = 0; i < p.E; ++i) {
        const int c = p.offsets[i + 1] - p.offsets[i];
        if (c > 0) {
            if (j == rank) { e = i; o0 = p.offsets[i]; ne = c; break; }
            ++j;
        }
    }
    if (e < 0) return;
    const int nb = (ne + 15) >> 4;  // token blocks of this expert (1..NBMAX), uniform per workgroup
    if (NBMAX == 1 || nb == 1) gemv_block<NW, RB, 1, 8, OUT>(p, e, o0, ne, rb, s_red);
    else if (NBMAX == 2 || nb == 2) gemv_block<NW, RB, 2, 4, OUT>(p, e, o0, ne, rb, s_red);
    else if (nb == 3) gemv_block<NW, RB, 3, 4, OUT>(p, e, o0, ne, rb, s_red);
    else gemv_block<NW, RB, 4, 4, OUT>(p, e, o0, ne, rb, s_red);
}

// Wide decode GEMV: 16 waves, each owning 16 weight rows of one active expert and a 1/KQ share of K (KQ = 1, 2
// or 4 waves per row block), so a workgroup covers 256 / KQ rows and reads its expert's token rows once per
// 256 / KQ rows instead of once per 16 or 32. The token rows (only the nb blocks of 16 in use) are staged
// through LDS in chunks of 512 to 2048 values of K (the fewer blocks in use, the longer), double-buffered:
// chunk c + 1 is loaded while chunk c's MFMAs run, and one barrier per chunk hands the buffers over. Each wave
// streams its weight rows in batches of U K-steps with the next batch's loads in flight (two register
// buffers), also across the chunk barriers, which wait only for LDS. With KQ > 1 the row block's KQ partial
// sums are added through LDS in wave order (deterministic), then scaled and stored. For the out-projection
// the rows are the gated rows the gate pass wrote in token order (gating them here instead, once per
// workgroup, measured slower: every row block would repeat the SiLU of all of its expert's tokens).
constexpr int kWideKC = 512;
constexpr int kWideWaves = 16;
constexpr int wide_rows(int kq) { return 16 * kWideWaves / kq; }
constexpr size_t wide_lds_bytes(int nbmax) { return (size_t)2 * nbmax * 16 * (kWideKC + 8) * 2; }

// Workgroup barrier that waits for this wave's LDS operations only: loads to registers stay in flight.
__device__ __forceinline__ void barrier_lds_only() {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int NBMAX, int KQ, bool OUT>
__global__ __launch_bounds__(64 * kWideWaves) void k_grouped_gemv_wide(GemmArgs p) {
    constexpr int NT = 64 * kWideWaves, NTOK = NBMAX * 16, BUF = NTOK * (kWideKC + 8);
    constexpr int SPW0 = kWideKC / 32 / KQ;                     // K-steps per wave in the smallest chunk
    // weight loads per batch (two batches in flight): 2 for the in-projection (decode_T64, two stacks of 8192 rows:
    // 94.8 us against 98.1 with 4), else 4 or 8 (Swimba's one stack and the out-projection: no gain from fewer)
    constexpr int UMAX = !OUT ? 2 : NBMAX > 2 ? 4 : 8, U = SPW0 < UMAX ? SPW0 : UMAX;
    constexpr int UQ = NTOK * (kWideKC / 8) / NT;               // staging loads per thread and chunk (bound)
    static_assert(SPW0 % U == 0 && UQ >= 1, "batches per chunk");
    extern __shared__ __attribute__((aligned(16))) uint16_t s_x[];  // [2][BUF]; partial sums at the end
    __shared__ int s_tok[NTOK];
    __shared__ float s_prob[NTOK];
    const int rb = blockIdx.x % p.n_tiles, rank = blockIdx.x / p.n_tiles;
    int e = -1, o0 = 0, ne = 0;
    for (int i = 0, j = 0; i < p.E; ++i) {
        const int c = p.offsets[i + 1] - p.offsets[i];
        if (c > 0) {
            if (j == rank) { e = i; o0 = p.offsets[i]; ne = c; break; }
            ++j;
        }
    }
    if (e < 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave / KQ, kq = wave % KQ;  // row block of 16, share of K
    const int nglob = rb * wide_rows(KQ);      // N0 is a multiple of the rows per workgroup: one output
    const int which = nglob / p.N0, n0 = nglob % p.N0;
    const int K = p.K;
    const uint16_t *W = static_cast<const uint16_t *>(which ? p.B1 : p.B0) + ((size_t)e * p.N0 + n0) * K;
    uint16_t *C = static_cast<uint16_t *>(which ? p.C1 : p.C0);
    const uint16_t *A = static_cast<const uint16_t *>(p.A0);
    if (tid < NTOK) {
        const int tok = p.perm[o0 + min(tid, ne - 1)];  // rows past ne repeat the last token (discarded)
        s_tok[tid] = tok;
        s_prob[tid] = OUT ? p.prob[tok] : 1.0f;
    }
    __syncthreads();
    const int nb = (ne + 15) >> 4;        // token blocks in use, uniform
    // chunk length: the LDS sized for NBMAX blocks of 512 values holds longer chunks of fewer blocks
    // (fewer barriers per weight byte); the rows of a chunk are padded by 8 values (16 bytes), which puts
    // the 16 rows of an MFMA operand read in 16 different bank slots
    int mult = NBMAX / (nb <= 1 ? 1 : nb <= 2 ? 2 : 4);
    while (mult > 1 && K % (kWideKC * mult) != 0) mult >>= 1;
    const int KC = kWideKC * mult, TP = KC + 8, cpr_sh = __builtin_ctz(KC / 8);
    const int SPW = KC / 32 / KQ, BPC = SPW / U;  // K-steps per wave and chunk; batches per chunk
    const int units = nb * 16 * (KC / 8);         // staged 16-byte pieces per chunk (at most NTOK * 64)

    u32x4 st[UQ];
    auto stage_load = [&](int c) {
#pragma unroll
        for (int q = 0; q < UQ; ++q) {
            const int u = min(tid + q * NT, units - 1), row = u >> cpr_sh, cc = u & ((1 << cpr_sh) - 1);
            const size_t off = (size_t)s_tok[row] * K + c * KC + cc * 8;  // u clamped: in bounds
            st[q] = *reinterpret_cast<const u32x4 *>(A + off);
        }
    };
    auto stage_store = [&](int b) {
#pragma unroll
        for (int q = 0; q < UQ; ++q) {
            const int u = tid + q * NT, row = u >> cpr_sh, cc = u & ((1 << cpr_sh) - 1);
            if (u < units)
                *reinterpret_cast<u32x4 *>(s_x + (size_t)b * BUF + row * TP + cc * 8) = st[q];
        }
    };
    const int r = lane & 15, g = lane >> 4;
    const uint16_t *wp = W + (size_t)(wr * 16 + r) * K + g * 8 + kq * SPW * 32;
    f32x4 acc[NBMAX];
#pragma unroll
    for (int bb = 0; bb < NBMAX; ++bb) acc[bb] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Staggered K order (KQ = 1). All 16 waves of every workgroup would read their rows at the same K offset
    // at the same time, and rows and workgroups lie power-of-two distances apart, so the concurrent requests
    // would share their low address bits and crowd a few memory channels (Swimba decode_T64's in-projection:
    // 127 us; staggered: 102 us). So each workgroup takes its chunks starting at chunk (blockIdx mod nchunks),
    // and inside a chunk each wave takes its batches starting at batch (wave mod BPC); a row's sum still runs
    // in a fixed order (deterministic). With KQ > 1 the waves' K shares already spread the requests (staggering
    // them as well measured slower, decode_T64's out-projection 60 -> 67 us).
    const int nchunks = K / KC, nbatch = nchunks * BPC;
    const int crot = KQ == 1 ? (int)(blockIdx.x % (unsigned)nchunks) : 0, brot = KQ == 1 ? wave % BPC : 0;
    auto chunk_at = [&](int c) { return c + crot < nchunks ? c + crot : c + crot - nchunks; };
    auto batch_at = [&](int j) { return j + brot < BPC ? j + brot : j + brot - BPC; };
    bf16x8 wa[U], wb[U];
    auto wload = [&](bf16x8 (&w)[U], int bi) {
        const int c = bi / BPC, j0 = batch_at(bi - c * BPC) * U;
        const uint16_t *q = wp + chunk_at(c) * KC + j0 * 32;
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = *reinterpret_cast<const bf16x8 *>(q + u * 32);
    };
    auto compute = [&](const bf16x8 (&w)[U], int bi) {
        const int c = bi / BPC, j0 = batch_at(bi - c * BPC) * U;
        const uint16_t *xs = s_x + (size_t)(c & 1) * BUF + g * 8 + (kq * SPW + j0) * 32;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int bb = 0; bb < NBMAX; ++bb) {
                if (bb < nb) {  // uniform
                    const bf16x8 xf = *reinterpret_cast<const bf16x8 *>(xs + (size_t)(bb * 16 + r) * TP + u * 32);
                    acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[u], xf, acc[bb], 0, 0, 0);
                }
            }
    };
    // chunk c + 1's token rows are loaded when chunk c begins and stored to the other buffer when it ends
    auto chunk_begin = [&](int bi) {
        if (bi % BPC == 0 && bi / BPC + 1 < nchunks) stage_load(chunk_at(bi / BPC + 1));
    };
    auto chunk_end = [&](int bi) {
        if ((bi + 1) % BPC == 0 && bi / BPC + 1 < nchunks) {  // uniform
            stage_store((bi / BPC + 1) & 1);  // that buffer was last read in the previous chunk
            barrier_lds_only();
        }
    };

    stage_load(chunk_at(0));
    wload(wa, 0);
    stage_store(0);
    barrier_lds_only();
    for (int bi = 0; bi < nbatch; bi += 2) {
        chunk_begin(bi);
        if (bi + 1 < nbatch) wload(wb, bi + 1);
        compute(wa, bi);
        chunk_end(bi);
        if (bi + 1 < nbatch) {
            chunk_begin(bi + 1);
            if (bi + 2 < nbatch) wload(wa, bi + 2);
            compute(wb, bi + 1);
            chunk_end(bi + 1);
        }
    }
    // accumulator register i of lane l: weight row 4*(l/16) + i of the row block, token column l%16 of block bb
    if (KQ > 1) {
        float *s_part = reinterpret_cast<float *>(s_x);  // [wave][bb][i][lane]; the staged rows are no longer read
        __syncthreads();
        if (kq > 0) {
#pragma unroll
            for (int bb = 0; bb < NBMAX; ++bb)
#pragma unroll
                for (int i = 0; i < 4; ++i) s_part[((wave * NBMAX + bb) * 4 + i) * 64 + lane] = acc[bb][i];
        }
        __syncthreads();
        if (kq == 0) {
#pragma unroll
            for (int q = 1; q < KQ; ++q)
#pragma unroll
                for (int bb = 0; bb < NBMAX; ++bb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[bb][i] += s_part[(((wave + q) * NBMAX + bb) * 4 + i) * 64 + lane];
        }
    }
    if (kq == 0) {
#pragma unroll
        for (int bb = 0; bb < NBMAX; ++bb) {
            const int col = bb * 16 + r;
            if (bb < nb && col < ne) {
                const int tok = s_tok[col];
                const float sc = s_prob[col];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint16_t *dst = C + (size_t)tok * p.N0 + n0 + wr * 16 + 4 * g + i;
                    *dst = f32_to_bf16(p.accumulate ? fmaf(acc[bb][i], sc, bf16_to_f32(*dst)) : acc[bb][i] * sc);
                }
            }
        }
    }
}

template <int NBMAX, int KQ, bool OUT>
static hipError_t launch_wide_n(const GemmArgs &a, long nwg, hipStream_t s) {
    static LdsAttrOnce attr;
    const size_t smem = wide_lds_bytes(NBMAX);
    const void *fn = reinterpret_cast<const void *>(&k_grouped_gemv_wide<NBMAX, KQ, OUT>);
    hipError_t err = set_lds_limit_once(attr, fn, smem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((k_grouped_gemv_wide<NBMAX, KQ, OUT>), dim3((unsigned)nwg), dim3(64 * kWideWaves), smem, s, a);
    return hipGetLastError();
}

template <int KQ, bool OUT>
static hipError_t launch_wide_kq(const GemmArgs &a, long nwg, hipStream_t s) {
    if (a.T <= 16) return launch_wide_n<1, KQ, OUT>(a, nwg, s);
    if (a.T <= 32) return launch_wide_n<2, KQ, OUT>(a, nwg, s);
    return launch_wide_n<4, KQ, OUT>(a, nwg, s);
}

// Waves per row block of the wide kernel: the fewest (1, 2 or 4) that give every compute unit a workgroup,
// or 0 when the shape does not suit it (too few output rows, K not a multiple of the chunk, T outside
// [wide_min_t, 64]).
static int wide_min_t() {
    static const int v = [] {
        const char *s = getenv("ROM_WIDE_MIN_T");
        const int x = s ? atoi(s) : 17;
        return x < 1 ? 1 : x;
    }();
    return v;
}
static int wide_kq(int T, int E, int N0, int K, int nB) {
    if (T < wide_min_t() || T > kDecodeMaxT || K % kWideKC != 0) return 0;
    const long active = T < E ? T : E;
    for (int kq = 1; kq <= 4; kq *= 2)
        if (N0 % wide_rows(kq) == 0 && (long)nB * N0 / wide_rows(kq) * active >= device_cus()) return kq;
    return 0;
}

bool gemv_wide_fits(int T, int E, int N0, int K, int nB) { return wide_kq(T, E, N0, K, nB) > 0; }

template <bool OUT>
static hipError_t launch_wide_t(const GemmArgs &a0, int nB, hipStream_t s) {
    GemmArgs a = a0;
    const int kq = wide_kq(a.T, a.E, a.N0, a.K, nB);
    if (kq == 0) return hipErrorInvalidValue;
    const int active = a.T < a.E ? a.T : a.E;
    a.n_tiles = nB * a.N0 / wide_rows(kq);
    a.n_tiles_per_b = a.N0 / wide_rows(kq);
    const long nwg = (long)a.n_tiles * active;
    if (kq == 1) return launch_wide_kq<1, OUT>(a, nwg, s);
    if (kq == 2) return launch_wide_kq<2, OUT>(a, nwg, s);
    return launch_wide_kq<4, OUT>(a, nwg, s);
}

hipError_t launch_gemv_wide_bf16(const GemmArgs &a, bool out, int nB, hipStream_t s) {
    return out ? launch_wide_t<true>(a, nB, s) : launch_wide_t<false>(a, nB, s);
}

template <bool OUT>
static hipError_t launch_gemv_t(const GemmArgs &a0, int nB, hipStream_t s) {
    GemmArgs a = a0;
    const int active = a.T < a.E ? a.T : a.E;
    // From 32 tokens on, 32 weight rows per workgroup (every workgroup reads all of its expert's token rows)
    const int rbk = a.T >= 32 ? 2 : 1;
    a.n_tiles = nB * a.N0 / (16 * rbk);
    a.n_tiles_per_b = a.N0 / (16 * rbk);
    const long nwg = (long)a.n_tiles * active;
    // At most one workgroup per compute unit (the out-projection of a single token): 16 waves, so that each
    // wave streams half as many K-steps and a compute unit keeps twice the loads in flight.
    const dim3 grid((unsigned)nwg);
    if (rbk == 2) {
        if (a.T <= 32) hipLaunchKernelGGL((k_grouped_gemv_bf16<8, 2, 2, OUT>), grid, dim3(512), 0, s, a);
        else hipLaunchKernelGGL((k_grouped_gemv_bf16<8, 2, 4, OUT>), grid, dim3(512), 0, s, a);
    } else if (nwg <= device_cus()) {
        if (a.T <= 16) hipLaunchKernelGGL((k_grouped_gemv_bf16<16, 1, 1, OUT>), grid, dim3(1024), 0, s, a);
        else hipLaunchKernelGGL((k_grouped_gemv_bf16<16, 1, 2, OUT>), grid, dim3(1024), 0, s, a);
    } else {
        if (a.T <= 16) hipLaunchKernelGGL((k_grouped_gemv_bf16<8, 1, 1, OUT>), grid, dim3(512), 0, s, a);
        else hipLaunchKernelGGL((k_grouped_gemv_bf16<8, 1, 2, OUT>), grid, dim3(512), 0, s, a);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Decode GEMV with the token rows staged in LDS, for the smallest T (every expert holds at most 16 tokens and
// the T rows of K values fit kGemvLdsBytes). A workgroup owns 16 weight rows of one active expert, as in
// k_grouped_gemv_bf16, but first copies its expert's ne token rows into LDS once (rows padded by 16 bytes, so
// the 16 rows an MFMA operand read touches fall in 16 different bank slots); the K loop then streams only the
// weight rows from HBM and reads the token fragments from LDS. This keeps fewer registers than holding both
// operands' fragments in flight, so more workgroups stay resident (one round over the CUs for the T = 1
// in-projection). GATED (out-projection): the staged rows are the gated rows bf16(SiLU(z) * h), computed here
// with the gate pass's arithmetic, so that pass and its launch are skipped. The first batch of weight loads is
// issued before the token rows arrive: ungated, even before the perm loads, since the weight rows depend only
// on the expert (T = 1 in-projection, 16384 rows of 4096: 26.4 -> 26.1 us); gated, right after the token-row
// loads, which the gate needs first. Each wave then keeps U weight loads in flight as a ring (U from
// gemv_lds_ring), and takes its steps in a rotated order (decode at T = 1, d_model 4096, d_inner 8192, E = 4, cold:
// out-projection 18.3 -> 17.5 us, step 50.2 -> 49.0 us with 8 loads, against batches of 8 issued only after the
// previous batch's MFMAs; then 15.9 us with a ring of 2).

// The K loop, wave reduction and store of the LDS-staged decode GEMV. The wave owns K-steps [sbeg, send) of the
// workgroup's 16 weight rows, taken in the order sbeg + (j + rot) mod (send - sbeg), whose first U are already in
// wf, and each slot is refilled with the step U ahead once its MFMA has been issued (U loads stay in flight);
// xrow is this lane's staged token row (token column lane % 16). The waves' partial sums are added in wave order
// through s_red (deterministic), scaled by s_prob[m] and written to row s_tok[m], columns n0 .. n0 + 15 of C, for
// the token columns m < ne.
template <int NW, int U>
__device__ __forceinline__ void gemv_lds_tail(const GemmArgs &p, const uint16_t *wp, int sbeg, int send,
                                              bf16x8 (&wf)[U], const uint16_t *xrow, int ne, const int *s_tok,
                                              const float *s_prob, float (*s_red)[16][16], uint16_t *C, int n0,
                                              int rot) {
    constexpr int NT = 64 * NW;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r = lane & 15, g = lane >> 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // ring of U weight loads: slot u is refilled with the step U ahead as soon as its MFMA has been issued, so
    // U loads stay in flight until the wave's last steps
    const int nw = send - sbeg;
    auto phys = [&](int j) { int q = j + rot; q -= q >= nw ? nw : 0; return sbeg + q; };
    for (int j0 = 0; j0 < nw; j0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (j0 + u < nw) {  // uniform
                const int st = phys(j0 + u);
                const bf16x8 xf = *reinterpret_cast<const bf16x8 *>(xrow + st * 32);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u], xf, acc, 0, 0, 0);
                if (j0 + U + u < nw) wf[u] = *reinterpret_cast<const bf16x8 *>(wp + phys(j0 + U + u) * 32);
            }
        }
    }
    // accumulator register i of lane l: weight row 4*(l/16) + i, token column l%16; waves added in order
#pragma unroll
    for (int i = 0; i < 4; ++i) s_red[wave][4 * g + i][r] = acc[i];
    __syncthreads();
    for (int idx = tid; idx < 256; idx += NT) {
        const int n = idx >> 4, m = idx & 15;
        if (m < ne) {
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) v += s_red[w][n][m];
            uint16_t *dst = C + (size_t)s_tok[m] * p.N0 + n0 + n;
            *dst = f32_to_bf16(p.accumulate ? fmaf(v, s_prob[m], bf16_to_f32(*dst)) : v * s_prob[m]);
        }
    }
}

// Weight loads each wave keeps in flight (the ring's length). More is not better: the decode_T1 shape (d_model 4096,
// d_inner 8192, cold) measured the gated out-projection (256 workgroups of 16 waves) at 15.9 / 16.2 / 17.3 /
// 20.7 us with 2 / 4 / 8 / 16 loads, Swimba's weighted in-projection (1024 workgroups of 8 waves, one stack of
// 16384 rows) at 24.9 us with 4 against 25.2 with 8, and the in-projection (the same grid over two stacks) at
// 25.6 / 26.0 / 26.4 us with 8 / 4 / 2.
constexpr int gemv_lds_ring(bool out, bool gated) { return gated ? 2 : out ? 4 : 8; }

// UL: staging loads per thread (at least T K / 8 / (64 NW), chosen at launch).
template <int NW, int UL, bool OUT, bool GATED>
__global__ __launch_bounds__(64 * NW) void k_grouped_gemv_lds(GemmArgs p) {
    constexpr int NT = 64 * NW, U = gemv_lds_ring(OUT, GATED);
    extern __shared__ __attribute__((aligned(16))) uint16_t s_x[];  // [ne][K + 8] bf16
    __shared__ float s_red[NW][16][16];
    __shared__ int s_tok[16];
    __shared__ float s_prob[16];
    const int rb = blockIdx.x % p.n_tiles, rank = blockIdx.x / p.n_tiles;
    int e = -1, o0 = 0, ne = 0;
    for (int i = 0, j = 0; i < p.E; ++i) {
        const int c = p.offsets[i + 1] - p.offsets[i];
        if (c > 0) {
            if (j == rank) { e = i; o0 = p.offsets[i]; ne = c; break; }
            ++j;
        }
    }
    if (e < 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nglob = rb * 16;  // N0 is a multiple of 64, so the 16 rows lie in one output
    const int which = nglob / p.N0, n0 = nglob % p.N0;
    const int K = p.K, pitch = K + 8;
    const uint16_t *W = static_cast<const uint16_t *>(which ? p.B1 : p.B0) + ((size_t)e * p.N0 + n0) * K;
    uint16_t *C = static_cast<uint16_t *>(which ? p.C1 : p.C0);

    // the first batch of weight loads goes out first: K split over the waves in contiguous ranges
    const int r = lane & 15, g = lane >> 4;
    const uint16_t *wp = W + (size_t)r * K + g * 8;
    const int nsteps = K / 32, spw = (nsteps + NW - 1) / NW;
    const int sbeg = wave * spw, send = min(nsteps, sbeg + spw);
    bf16x8 wf[U];
    // the wave's steps are taken in a rotated order, starting at batch (wave + workgroup) mod batches, so that
    // the concurrent loads of the waves and workgroups (rows a power of two apart) spread over the memory channels
    const int nwk = send - sbeg;
    const int rot = nwk > U ? (((wave + (int)blockIdx.x) % ((nwk + U - 1) / U)) * U) % nwk : 0;
    auto first_batch = [&]() {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int q = min(u, nwk - 1) + rot;
            q -= q >= nwk ? nwk : 0;
            wf[u] = *reinterpret_cast<const bf16x8 *>(wp + (sbeg + q) * 32);
        }
    };
    // ungated: the weight rows do not depend on perm, so their first batch goes out before the perm loads
    if (!GATED && sbeg < send) first_batch();
    // token rows: unit q of this thread is chunk (tid + q NT) of the ne x K/8 chunks, tokens read through perm
    const int cpr = K / 8, units = ne * cpr;
    u32x4 va[UL], vb[UL];
    int tk[UL];
#pragma unroll
    for (int q = 0; q < UL; ++q) {
        const int u = min(tid + q * NT, units - 1);  // clamped: in bounds
        tk[q] = p.perm[o0 + u / cpr];
    }
#pragma unroll
    for (int q = 0; q < UL; ++q) {
        const int u = min(tid + q * NT, units - 1);
        const int row = u / cpr, c = u - row * cpr;
        va[q] = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p.A0) + (size_t)tk[q] * K)[c];
        if (GATED) vb[q] = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p.A1) + (size_t)tk[q] * K)[c];
    }
    if (GATED && sbeg < send) first_batch();
    if (tid < 16) {
        const int tok = p.perm[o0 + (tid < ne ? tid : 0)];
        s_tok[tid] = tok;
        s_prob[tid] = OUT ? p.prob[tok] : 1.0f;
    }
    // gated: the token rows have landed once at most the U weight loads (issued after them) are in flight;
    // ungated: the weight batch went out first, so every load is waited for
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(GATED ? U : 0));
#pragma unroll
    for (int q = 0; q < UL; ++q) {
        const int u = tid + q * NT;
        if (u < units) {
            const int row = u / cpr, c = u - row * cpr;
            u32x4 v = va[q];
            if (GATED) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float z0 = __uint_as_float(va[q][i] << 16), z1 = __uint_as_float(va[q][i] & 0xFFFF0000u);
                    const float h0 = __uint_as_float(vb[q][i] << 16), h1 = __uint_as_float(vb[q][i] & 0xFFFF0000u);
                    v[i] = pack_bf16x2(silu_fast(z0) * h0, silu_fast(z1) * h1);
                }
            }
            *reinterpret_cast<u32x4 *>(s_x + (size_t)row * pitch + c * 8) = v;
        }
    }
    // LDS writes visible to the workgroup; the weight loads stay in flight (their results go to registers)
    barrier_lds_only();

    // token column r of the MFMA reads staged row r (rows past ne repeat row 0; their results are discarded)
    const uint16_t *xrow = s_x + (size_t)(r < ne ? r : 0) * pitch + g * 8;
    gemv_lds_tail<NW, U>(p, wp, sbeg, send, wf, xrow, ne, s_tok, s_prob, s_red, C, n0, rot);
}

template <int NW, int UL, bool OUT, bool GATED>
static hipError_t launch_gemv_lds_n(const GemmArgs &a, long nwg, size_t smem, hipStream_t s) {
    static LdsAttrOnce attr;
    hipError_t err = set_lds_limit_once(
        attr, reinterpret_cast<const void *>(&k_grouped_gemv_lds<NW, UL, OUT, GATED>), kGemvLdsBytes);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((k_grouped_gemv_lds<NW, UL, OUT, GATED>), dim3((unsigned)nwg), dim3(64 * NW), smem, s, a);
    return hipGetLastError();
}

template <int NW, bool OUT, bool GATED>
static hipError_t launch_gemv_lds_w(const GemmArgs &a, long nwg, size_t smem, hipStream_t s) {
    // staging loads per thread: the chunks of the largest expert group (at most T rows of K / 8) over the threads
    const long per = ((long)a.T * (a.K / 8) + 64 * NW - 1) / (64 * NW);
    if (per <= 1) return launch_gemv_lds_n<NW, 1, OUT, GATED>(a, nwg, smem, s);
    if (per <= 2) return launch_gemv_lds_n<NW, 2, OUT, GATED>(a, nwg, smem, s);
    if (per <= 4) return launch_gemv_lds_n<NW, 4, OUT, GATED>(a, nwg, smem, s);
    if (per <= 8) return launch_gemv_lds_n<NW, 8, OUT, GATED>(a, nwg, smem, s);
    return hipErrorInvalidValue;  // excluded by gemv_lds_fits
}

template <bool OUT, bool GATED>
static hipError_t launch_gemv_lds_t(const GemmArgs &a0, int nB, hipStream_t s) {
    GemmArgs a = a0;
    const int active = a.T < a.E ? a.T : a.E;
    a.n_tiles = nB * a.N0 / 16;
    a.n_tiles_per_b = a.N0 / 16;
    const long nwg = (long)a.n_tiles * active;
    const size_t smem = (size_t)a.T * (a.K + 8) * 2;
    // at most one workgroup per compute unit: 16 waves (each streams half as many K steps), as for the
    // register-staged kernels
    if (nwg <= device_cus()) return launch_gemv_lds_w<16, OUT, GATED>(a, nwg, smem, s);
    return launch_gemv_lds_w<8, OUT, GATED>(a, nwg, smem, s);
}



hipError_t launch_gemv_bf16(const GemmArgs &a, bool out, int nB, hipStream_t s) {
    return out ? launch_gemv_t<true>(a, nB, s) : launch_gemv_t<false>(a, nB, s);
}

hipError_t launch_gemv_lds_bf16(const GemmArgs &a, bool out, bool gated, int nB, hipStream_t s) {
    if (gated) return out ? launch_gemv_lds_t<true, true>(a, nB, s) : hipErrorInvalidValue;
    return out ? launch_gemv_lds_t<true, false>(a, nB, s) : launch_gemv_lds_t<false, false>(a, nB, s);
}

}  // namespace rom
