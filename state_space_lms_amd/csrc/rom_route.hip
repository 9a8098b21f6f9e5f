// rom_route.hip -- the shared router of a Routing Mamba block on gfx950, and the grouping of tokens
// by expert (histogram, scan, stable counting-sort scatter, optional permute).
//
// Method: Routing Mamba landing page (chapterpal.com), Knowl 1: p_t = Softmax(x_t W_r) over the
// experts, S_t = the K largest (K = 1 or 2; the page's 8top1, 16top1 and 8top2 settings), r_t,i =
// p_t,i (not renormalised). The grouping is not on the page; a dropless grouped GEMM (Knowl 12: no
// capacity factor, no token dropping) needs it. With K = 2 the routing is kept as two stacked top-1
// routings (choice k of every token, grouped on its own), which the projections run one after the other.
//
// Router arithmetic is fp32: logit_t,j = sum_k X[t][k] * W_r[k][j] (+ bias[j]); argmax keeps the
// lowest index on ties (strict > in ascending j); prob = 1 / sum_j exp(logit_j - logit_max).
// The router reads X once (HBM-bound: E flops per element). A wave computes the logits of 8 tokens at
// a time with all 64 lanes splitting d_model, so each W_r value a lane loads serves 8 tokens; W_r is
// staged once per workgroup in LDS (when it fits) in a layout where the 64 lanes of a wave read 64
// consecutive 16-byte words. Each lane keeps two chunks of its 8 rows in flight, and the first two are
// requested before W_r is staged.
//
// Launches: T <= 8: one workgroup does everything. Otherwise (1) logits + top-1 + per-workgroup
// histogram, 32 tokens per workgroup when that gives >= 512 workgroups (one wave per 8 tokens), else
// 8 tokens per workgroup (the four waves split d_model); on that wide path bf16 rows with 8 experts and
// d_model in {512, 1024, 1536, 2048} go to the matrix cores instead (k_route_logits_mfma, 64 tokens per
// workgroup); (2) per-expert totals and bases, stable scatter (ballot ranks inside each 256-token
// workgroup), optional permute.
#include <type_traits>

#include "rom_device.h"
#include "rom_internal.h"
#include "rom_router_dev.h"

namespace rom {

// Largest W_r staged in LDS (bytes).
constexpr int kRouteLdsW = 64 * 1024;

// W_r [d_model][E] -> LDS as float4 words: word (kk, x4, c) holds W_r[8c+kk][4*x4 .. 4*x4+4), stored at
// d = ((kk * E/4 + x4) * nchunk + c), so lanes reading consecutive chunks c read consecutive words.
// Requires E % 4 == 0. The words are copied global -> LDS directly (global_load_lds_dwordx4, no register
// stage): copy m of the workgroup fills words [64 m, 64 m + 64), lane i reading the source word of
// destination word 64 m + i, and wave w issues copies w, w + 4, ... (dm * E/4 is a multiple of 64, as
// d_model is). Completion is tracked by vmcnt like any load, in issue order: call it before the X rows
// are issued, and before the barrier that precedes the reads wait until at most the loads issued after
// it are in flight. Requires E/4 to be a power of two and dm * E/4 <= 4096 words (64 KiB): d / nchunk is
// then umulhi(d, floor((2^32 - 1) / nchunk) + 1), exact for d * nchunk < 2^32, and the rest are shifts.
__device__ __forceinline__ void stage_router_weight(const float *__restrict__ Wr, int dm, int E, float4 *wl) {
    const unsigned e4 = (unsigned)E >> 2, nchunk = (unsigned)dm >> 3, n4 = (unsigned)dm * e4;
    const unsigned lg_e4 = __builtin_ctz(e4), magic = 0xFFFFFFFFu / nchunk + 1u;
    const unsigned lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float4 *src = reinterpret_cast<const float4 *>(Wr);
    for (unsigned m = wave; m * 64 < n4; m += 4) {
        const unsigned d = m * 64 + lane;
        const unsigned q = __umulhi(d, magic), c = d - q * nchunk;  // q = kk * e4 + x4
        const unsigned kk = q >> lg_e4, x4 = q & (e4 - 1);
        dma16_to_lds(src + (8 * c + kk) * e4 + x4, wl + m * 64);
    }
}

// Stable ranks of one token per thread within the workgroup (256 threads, 4 waves):
// returns #{threads tid' < tid with the same expert}. e < 0 marks an absent token.
// s_wcnt is [4][ROM_MAX_EXPERTS] in LDS. Contains a __syncthreads.
__device__ __forceinline__ int wg_stable_rank(int e, int E, int (*s_wcnt)[ROM_MAX_EXPERTS]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int rank = 0;
    for (int x = 0; x < E; ++x) {
        const uint64_t m = __ballot(e == x);
        if (e == x) rank = __popcll(m & lanemask_lt());
        if (lane == 0) s_wcnt[wave][x] = __popcll(m);
    }
    __syncthreads();
    if (e >= 0)
        for (int w = 0; w < wave; ++w) rank += s_wcnt[w][e];
    return rank;
}

// Copy the rows of this workgroup's tokens to their slots (the materialised permute).
template <typename TX>
__device__ __forceinline__ void permute_rows(const TX *X, TX *Xp, int dm, int tok_base, int n_rows, const int *s_pos) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int chunks = dm * (int)sizeof(TX) / 16;
    for (int r = wave; r < n_rows; r += 4) {
        const int p = s_pos[r];
        const uint4 *src = reinterpret_cast<const uint4 *>(X + (size_t)(tok_base + r) * dm);
        uint4 *dst = reinterpret_cast<uint4 *>(Xp + (size_t)p * dm);
        for (int c = lane; c < chunks; c += 64) dst[c] = src[c];
    }
}

// ---------------------------------------------------------------------------------------------
// Multi-workgroup path, kernel 1: logits, top-1, probability, and this workgroup's histogram.
// WPG = 1: 32 tokens per workgroup (8 per wave); WPG = 4: 8 tokens per workgroup.
template <typename TX, int EG, int EMAX, int WPG>
__global__ __launch_bounds__(256) void k_route_logits(const TX *__restrict__ X, int T, int dm,
                                                      const float *__restrict__ Wr, const float *__restrict__ bias,
                                                      int E, int K, int use_lds, int32_t *__restrict__ ids,
                                                      float *__restrict__ prob, int32_t *__restrict__ wg_counts,
                                                      int nwg) {
    constexpr int TPW = 32 / WPG;  // tokens per workgroup
    extern __shared__ float4 wl_dyn[];
    __shared__ int hist[ROM_MAX_TOP_K * ROM_MAX_EXPERTS];
    __shared__ float s_red[WPG == 4 ? 4 : 1][8][EMAX];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < K * E; i += 256) hist[i] = 0;
    if (use_lds) stage_router_weight(Wr, dm, E, wl_dyn);
    __builtin_amdgcn_sched_barrier(0);  // the W_r copies stay ahead of the X loads (vmcnt counts in issue order)
    XRows<TX> xr;
    {
        int g0, jl;
        wg_token_group<WPG>(blockIdx.x * TPW, g0, jl);
        xrows_issue<TX, WPG * 64>(xr, X, T, dm, g0, jl);
    }
    // This wave's W_r copies have landed once at most the first chunk set of its 8 rows (8 loads per
    // set, 16 for fp32) is in flight, and its LDS stores at lgkmcnt(0). Then a plain barrier: the fence of
    // __syncthreads() would also wait for every X load, while kept in flight they let the FMAs of the
    // first chunks start as those arrive instead of after the last row's.
    if (use_lds) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kXrowsSetLoads<TX>));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
    barrier_no_fence();
    float lg[EMAX];
    const int tok0 = wg_logits<TX, EG, EMAX, WPG>(xr, X, T, dm, Wr, use_lds ? wl_dyn : nullptr, E, blockIdx.x * TPW,
                                                  lg, s_red);
    const int t = tok0 + lane;
    if (lane < 8 && (WPG == 1 || wave == 0) && t < T) {
        int best[2];
        float p[2];
        select_topk<EMAX>(lg, bias, E, K, best, p);
#pragma unroll
        for (int k = 0; k < ROM_MAX_TOP_K; ++k) {
            if (k < K) {
                ids[(size_t)k * T + t] = best[k];
                prob[(size_t)k * T + t] = p[k];
                atomicAdd(&hist[k * E + best[k]], 1);
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < K * E; i += 256) wg_counts[(size_t)i * nwg + blockIdx.x] = hist[i];
}

// Multi-workgroup path, kernel 1 on the matrix cores (bf16 X, E = 8, d_model = 32 NKS with NKS a
// multiple of 16 up to 64): logits, top-K, probability and this workgroup's histogram for 64 tokens (16
// per wave), with the same outputs as k_route_logits.
//
// fp32 W_r is split exactly into three bf16 parts, w = hi + mid + lo: hi = bf16(w), mid = bf16(w - hi),
// lo = w - hi - mid (both differences are exact in fp32, and lo has at most 8 significant bits, so bf16
// holds it). A bf16 x times a bf16 part is exact in fp32 and the MFMA adds in fp32, so every logit is an
// fp32 sum of the exact products x_k * w_k, in another order than the VALU kernel's.
//
// v_mfma_f32_16x16x32_bf16 with the parts as the first operand (16 rows) and 16 tokens as the second:
// lane l supplies row (or token) l % 16 and features 8 (l / 16) .. + 8 of a 32-feature step, and
// receives rows 4 (l / 16) + i, i = 0..3, of token l % 16. One MFMA per step on the main table (rows
// 0..7 hi of experts 0..7, rows 8..15 mid) and one on the low table (rows 0..7 lo, rows 8..15 zero).
// Lanes 0..15 then hold hi + lo of experts 0..3, lanes 16..31 of experts 4..7, lanes 32..63 the mids:
// two shuffles give lanes 0..15 all 8 logits of their token.
//
// LDS tables, in 16-byte words, for feature octet o = 4 s + g (features 8 o .. 8 o + 7):
//   main[o * 16 + r]: r < 8 hi of expert r, r >= 8 mid of expert r - 8;  low[o * 8 + r]: lo of expert r.
// At step s lane l reads main word 64 s + l (one contiguous KiB per wave) and low word 32 s + 8 g + (l & 7).
//
// Each lane streams its token row through a ring of kRouteMfmaRing 16-byte loads, refilled as the MFMAs
// consume them; everything is unrolled at compile time, so each MFMA waits only for its own load. The
// W_r values for the tables are loaded before the X rows and split while those are in flight.
constexpr int kRouteMfmaTokensPerWG = 64;
constexpr int kRouteMfmaRing = 16;
constexpr size_t route_mfma_lds_bytes(int dm) { return (size_t)dm / 8 * 24 * 16; }

template <int NKS>
__global__ __launch_bounds__(256) void k_route_logits_mfma(const uint16_t *__restrict__ X, int T,
                                                           const float *__restrict__ Wr,
                                                           const float *__restrict__ bias, int K,
                                                           int32_t *__restrict__ ids, float *__restrict__ prob,
                                                           int32_t *__restrict__ wg_counts, int nwg) {
    constexpr int DM = NKS * 32, NOCT = DM / 8, NIT = NOCT * 8 / 256, R = kRouteMfmaRing;
    static_assert(NKS % 16 == 0 && NKS >= R && NIT >= 1, "shape");
    extern __shared__ uint4 rt_dyn[];
    __shared__ int hist[ROM_MAX_TOP_K * 8];
    uint4 *tmain = rt_dyn, *tlow = rt_dyn + NOCT * 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < K * 8) hist[tid] = 0;

    // table items q = tid + 256 it: expert e = q & 7 of octet o = q >> 3 (8 consecutive lanes read one
    // 32-byte W_r row)
    float wv[NIT][8];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int q = tid + 256 * it, e = q & 7, o = q >> 3;
#pragma unroll
        for (int j = 0; j < 8; ++j) wv[it][j] = Wr[(size_t)(8 * o + j) * 8 + e];
    }
    __builtin_amdgcn_sched_barrier(0);  // the W_r loads go out ahead of the X rows

    const int r16 = lane & 15, g = lane >> 4;
    const int tok0 = blockIdx.x * kRouteMfmaTokensPerWG + wave * 16;
    const uint16_t *xp = X + (size_t)min(tok0 + r16, T - 1) * DM + 8 * g;  // + 32 s for step s
    uint4 ring[R];
#pragma unroll
    for (int u = 0; u < R; ++u) ring[u] = *reinterpret_cast<const uint4 *>(xp + 32 * u);
    __builtin_amdgcn_sched_barrier(0);  // the X rows are in flight before the first wait for W_r

#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int q = tid + 256 * it, e = q & 7, o = q >> 3;
        uint32_t hi[4], mid[4], lo[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            float rm[2], rl[2];
            uint16_t bh[2], bm[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const float w = wv[it][2 * h + b];
                bh[b] = f32_to_bf16(w);
                rm[b] = w - bf16_to_f32(bh[b]);
                bm[b] = f32_to_bf16(rm[b]);
                rl[b] = rm[b] - bf16_to_f32(bm[b]);
            }
            hi[h] = uint32_t(bh[0]) | (uint32_t(bh[1]) << 16);
            mid[h] = uint32_t(bm[0]) | (uint32_t(bm[1]) << 16);
            lo[h] = pack_bf16x2(rl[0], rl[1]);
        }
        tmain[o * 16 + e] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        tmain[o * 16 + 8 + e] = make_uint4(mid[0], mid[1], mid[2], mid[3]);
        tlow[o * 8 + e] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    // the tables and the histogram's zeros are in LDS at lgkmcnt(0); the X rows stay in flight
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
    barrier_no_fence();

    f32x4 am = {0.0f, 0.0f, 0.0f, 0.0f}, al = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        const uint4 xw = ring[s % R];
        const uint4 wm = tmain[s * 64 + lane];
        uint4 wl = tlow[s * 32 + g * 8 + (r16 & 7)];
        if (r16 >= 8) wl = make_uint4(0u, 0u, 0u, 0u);
        am = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wm), __builtin_bit_cast(bf16x8, xw),
                                                     am, 0, 0, 0);
        al = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wl), __builtin_bit_cast(bf16x8, xw),
                                                     al, 0, 0, 0);
        if (s + R < NKS) ring[s % R] = *reinterpret_cast<const uint4 *>(xp + 32 * (s + R));
    }

    // lanes 0..31: hi + lo (the low table's rows 8..15 are zero, so lanes 32..63 keep the mids exactly)
    float v[4], lg[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = am[i] + al[i];
        v[i] += __shfl_xor(v[i], 32);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float other = __shfl_xor(v[i], 16);
        lg[i] = (g & 1) ? other : v[i];
        lg[4 + i] = (g & 1) ? v[i] : other;
    }
    const int t = tok0 + lane;
    if (lane < 16 && t < T) {
        int best[2];
        float p[2];
        select_topk<8>(lg, bias, 8, K, best, p);
#pragma unroll
        for (int k = 0; k < ROM_MAX_TOP_K; ++k) {
            if (k < K) {
                ids[(size_t)k * T + t] = best[k];
                prob[(size_t)k * T + t] = p[k];
                atomicAdd(&hist[k * 8 + best[k]], 1);
            }
        }
    }
    __syncthreads();
    if (tid < K * 8) wg_counts[(size_t)tid * nwg + blockIdx.x] = hist[tid];
}

// Multi-workgroup path, kernel 2: per-expert totals and bases, then the stable scatter of 256 tokens
// per workgroup (= sub logits workgroups).
// With `bases` (written by k_route_scan), each workgroup reads its own per-expert bases and the totals instead.
__global__ __launch_bounds__(256) void k_route_scatter(const int32_t *__restrict__ ids, int T, int E,
                                                       const int32_t *__restrict__ wg_counts, int nwg, int sub,
                                                       const int32_t *__restrict__ bases, int nsc,
                                                       int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                       int32_t *__restrict__ perm, int32_t *__restrict__ inv_perm) {
    __shared__ int s_before[ROM_MAX_EXPERTS], s_total[ROM_MAX_EXPERTS], s_base[ROM_MAX_EXPERTS];
    __shared__ int s_wcnt[4][ROM_MAX_EXPERTS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wg = blockIdx.x;
    // choice k = blockIdx.y: the k-th stacked top-1 routing
    ids += (size_t)blockIdx.y * T;
    wg_counts += (size_t)blockIdx.y * E * nwg;
    counts += blockIdx.y * E;
    offsets += blockIdx.y * (E + 1);
    perm += (size_t)blockIdx.y * T;
    inv_perm += (size_t)blockIdx.y * T;
    const int first = wg * sub;  // logits workgroups before this one contribute to the base
    const int t = wg * kScatterTokensPerWG + tid;
    const int te = t < T ? ids[t] : -1;  // this thread's token's expert, in flight with the partial histograms
    if (bases != nullptr) {
        // [K][E][nsc] bases before this workgroup, then the [K][E] totals
        const int32_t *bk = bases + (size_t)blockIdx.y * E * nsc;
        const int32_t *tk = bases + (size_t)gridDim.y * E * nsc + (size_t)blockIdx.y * E;
        if (tid < E) {
            s_before[tid] = bk[(size_t)tid * nsc + wg];
            s_total[tid] = tk[tid];
        }
    }
    // wave w sums the partial histograms of experts w, w + 4, ..., two experts at a time with all of their
    // loads (4 per 256 logits workgroups each) in flight before the first add
    for (int e0 = bases != nullptr ? E : wave; e0 < E; e0 += 8) {
        const int e1 = e0 + 4;
        int b0 = 0, t0 = 0, b1 = 0, t1 = 0;
        auto chunk = [&](int w0) {
            // unconditional loads from clamped (in-bounds) indices, the surplus zeroed afterwards: straight-line
            // code, so no branch join makes the compiler wait between them
            int c0[4], c1[4];
            const size_t r0 = (size_t)e0 * nwg, r1 = (size_t)min(e1, E - 1) * nwg;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int w = min(w0 + 64 * u + lane, nwg - 1);
                c0[u] = wg_counts[r0 + w];
                c1[u] = wg_counts[r1 + w];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int w = w0 + 64 * u + lane;
                const int v0 = w < nwg ? c0[u] : 0, v1 = (w < nwg && e1 < E) ? c1[u] : 0;
                t0 += v0;
                t1 += v1;
                b0 += w < first ? v0 : 0;
                b1 += w < first ? v1 : 0;
            }
        };
        chunk(0);  // outside the loop, so that no loop-head wait holds these loads back
        for (int w0 = 256; w0 < nwg; w0 += 256) chunk(w0);
        for (int m = 32; m >= 1; m >>= 1) {
            b0 += __shfl_xor(b0, m);
            t0 += __shfl_xor(t0, m);
            b1 += __shfl_xor(b1, m);
            t1 += __shfl_xor(t1, m);
        }
        if (lane == 0) {
            s_before[e0] = b0;
            s_total[e0] = t0;
            if (e1 < E) { s_before[e1] = b1; s_total[e1] = t1; }
        }
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int e = 0; e < E; ++e) {
            s_base[e] = run + s_before[e];
            if (wg == 0) { counts[e] = s_total[e]; offsets[e] = run; }
            run += s_total[e];
        }
        if (wg == 0) offsets[E] = run;
    }
    __syncthreads();
    const int rank = wg_stable_rank(te, E, s_wcnt);
    if (te >= 0) {
        const int pos = s_base[te] + rank;
        perm[pos] = t;
        inv_perm[t] = pos;
    }
}

// The materialised permute (top-1): X_perm[inv_perm[t]] = X[t], a streaming copy over the whole chip. A
// workgroup owns perm_rows_per_wg(cpr) consecutive source rows (about 2048 16-byte chunks; cpr chunks per row)
// and its threads stride over their chunks with kPermChunks loads in flight each, issued before the stores:
// source rows are read in token order, destination rows are written whole. The row of chunk unit u is
// umulhi(u, magic) with magic = floor(2^32 / cpr) + 1, exact for u < max(2048, cpr) and cpr < 2^16.
constexpr int kPermChunks = 8;
inline int perm_rows_per_wg(int cpr) { return cpr >= 2048 ? 1 : 2048 / cpr; }
template <typename TX>
__global__ __launch_bounds__(256) void k_permute_rows(const TX *__restrict__ X, const int32_t *__restrict__ inv_perm,
                                                      int T, int cpr, int rows_per_wg, uint32_t magic,
                                                      TX *__restrict__ Xp) {
    const int r0 = blockIdx.x * rows_per_wg;
    const int n = min(rows_per_wg, T - r0) * cpr;  // chunk units of this workgroup
    const u32x4 *src = reinterpret_cast<const u32x4 *>(X) + (size_t)r0 * cpr;
    for (int ub = threadIdx.x; ub < n; ub += kPermChunks * 256) {
        u32x4 v[kPermChunks];
#pragma unroll
        for (int j = 0; j < kPermChunks; ++j) v[j] = src[min(ub + j * 256, n - 1)];  // clamped: in bounds
#pragma unroll
        for (int j = 0; j < kPermChunks; ++j) {
            const int u = ub + j * 256;
            if (u < n) {
                const int rr = (int)__umulhi((uint32_t)u, magic), c = u - rr * cpr;
                __builtin_nontemporal_store(v[j], reinterpret_cast<u32x4 *>(Xp) + (size_t)inv_perm[r0 + rr] * cpr + c);
            }
        }
    }
}

// Prefix scan of the partial histograms (large T): workgroup (e, k) reads the nwg partial counts of expert e
// in choice k once and writes, for every scatter workgroup s (= logits workgroups [s * sub, s * sub + sub)),
// the tokens of expert e in the logits workgroups before s, and the expert's total. Groups of 256 scatter
// workgroups are scanned in turn (a wave-level inclusive scan, then the four waves' sums through LDS), with
// a running carry.
__global__ __launch_bounds__(256) void k_route_scan(const int32_t *__restrict__ wg_counts, int nwg, int sub,
                                                    int nsc, int32_t *__restrict__ bases) {
    __shared__ int s_wsum[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = gridDim.x, e = blockIdx.x, k = blockIdx.y;
    const int32_t *v = wg_counts + ((size_t)k * E + e) * nwg;
    int32_t *out = bases + ((size_t)k * E + e) * nsc;
    int carry = 0;
    for (int c0 = 0; c0 < nsc; c0 += 256) {
        const int s = c0 + tid;
        int g = 0;
        if (s < nsc) {
            const int w1 = min(nwg, (s + 1) * sub);
            for (int w = s * sub; w < w1; ++w) g += v[w];
        }
        int incl = g;  // inclusive scan within the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int up = __shfl_up(incl, d);
            if (lane >= d) incl += up;
        }
        if (lane == 63) s_wsum[wave] = incl;
        __syncthreads();
        int before = carry;
        for (int w = 0; w < wave; ++w) before += s_wsum[w];
        if (s < nsc) out[s] = before + incl - g;
        carry += s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
        __syncthreads();
    }
    if (tid == 0) bases[(size_t)gridDim.y * E * nsc + (size_t)k * E + e] = carry;
}

// ---------------------------------------------------------------------------------------------
// Small-T path (T <= 8): the whole routing in one workgroup and one launch. Its WPG waves split d_model
// (64 WPG lanes, each with at most one or two 8-element chunks), so that every X and W_r load goes out at
// once, in one round trip; W_r is read from L2/HBM directly (each of its values serves at most 8 tokens).
// The grouping of at most 8 tokens is counted directly: slot = (tokens of lower experts) + (earlier tokens
// of the same expert).
template <typename TX, int EG, int EMAX, int WPG>
__global__ __launch_bounds__(64 * WPG) void k_route_small(const TX *__restrict__ X, int T, int dm,
                                                          const float *__restrict__ Wr, const float *__restrict__ bias,
                                                          int E, int K, int32_t *__restrict__ ids,
                                                          float *__restrict__ prob, int32_t *__restrict__ counts,
                                                          int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
                                                          int32_t *__restrict__ inv_perm, TX *__restrict__ Xp) {
    __shared__ int s_ids[ROM_MAX_TOP_K * kRouteSmallT];
    __shared__ int s_pos[kRouteSmallT];
    __shared__ float s_red[WPG][8][EMAX];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    XRows<TX> xr;
    WrChunk<EG> wpre;
    constexpr bool kPre = EMAX == EG;  // one expert group: no second copy of the logits code
    {
        int g0, jl;
        wg_token_group<WPG>(0, g0, jl);
        // the W_r rows of this lane's first chunk go out with its X rows: one round trip for both
        if (kPre && jl < (dm >> 3)) wr_chunk_load<EG>(wpre, Wr, E, 0, jl);
        xrows_issue<TX, 64 * WPG>(xr, X, T, dm, g0, jl);
    }
    float lg[EMAX];
    wg_logits<TX, EG, EMAX, WPG, kPre>(xr, X, T, dm, Wr, nullptr, E, 0, lg, s_red, &wpre);
    if (wave == 0 && lane < T) {
        int best[2];
        float p[2];
        select_topk<EMAX>(lg, bias, E, K, best, p);
#pragma unroll
        for (int k = 0; k < ROM_MAX_TOP_K; ++k) {
            if (k < K) {
                ids[k * T + lane] = best[k];
                prob[k * T + lane] = p[k];
                s_ids[k * kRouteSmallT + lane] = best[k];
            }
        }
    }
    __syncthreads();
    for (int k = 0; k < K; ++k) {  // the K stacked top-1 routings
        const int *sid = s_ids + k * kRouteSmallT;
        if (tid < T) {
            const int e = sid[tid];
            int pos = 0;
            for (int t = 0; t < T; ++t) pos += (sid[t] < e) || (sid[t] == e && t < tid);
            perm[k * T + pos] = tid;
            inv_perm[k * T + tid] = pos;
            s_pos[tid] = pos;
        }
        if (tid < E) {
            int c = 0, below = 0;
            for (int t = 0; t < T; ++t) {
                c += sid[t] == tid;
                below += sid[t] < tid;
            }
            counts[k * E + tid] = c;
            offsets[k * (E + 1) + tid] = below;
            if (tid == E - 1) offsets[k * (E + 1) + E] = T;
        }
        if (Xp && k == 0) {  // top-1 only
            __syncthreads();
            if (wave < 4) permute_rows<TX>(X, Xp, dm, 0, T, s_pos);
        }
    }
}

// Smallest-T path (T <= kRouteTinyT) for bf16 rows and at most 8 experts: route_tiny in one workgroup of 512
// threads, then the optional permute (top-1).
template <int TMAX, int EMAX>
__global__ __launch_bounds__(512) void k_route_tiny(const uint16_t *__restrict__ X, int T, int dm,
                                                    const float *__restrict__ Wr, const float *__restrict__ bias,
                                                    int E, int K, int32_t *__restrict__ ids, float *__restrict__ prob,
                                                    int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                    int32_t *__restrict__ perm, int32_t *__restrict__ inv_perm,
                                                    uint16_t *__restrict__ Xp) {
    __shared__ RouteTinyLds<TMAX, EMAX> sm;
    route_tiny<TMAX, EMAX>(X, T, dm, Wr, bias, E, K, ids, prob, counts, offsets, perm, inv_perm, sm);
    if (Xp && (threadIdx.x >> 6) < 4) permute_rows<uint16_t>(X, Xp, dm, 0, T, sm.pos);
}

template <int EMAX>
static hipError_t launch_route_tiny(const uint16_t *X, int T, int dm, const float *Wr, const float *bias, int E,
                                    const rom_routing &r, uint16_t *Xp, hipStream_t s) {
#define ROM_TINY(TM)                                                                                               \
    hipLaunchKernelGGL((k_route_tiny<TM, EMAX>), dim3(1), dim3(512), 0, s, X, T, dm, Wr, bias, E, r.top_k,          \
                       r.expert_id, r.prob, r.counts, r.offsets, r.perm, r.inv_perm, Xp)
    if (T <= 1) ROM_TINY(1);
    else ROM_TINY(2);
#undef ROM_TINY
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------

template <int NKS>
static hipError_t launch_route_mfma_n(const uint16_t *X, int T, const float *Wr, const float *bias,
                                      const rom_routing &r, int32_t *wg_counts, int nwg, hipStream_t s) {
    const size_t smem = route_mfma_lds_bytes(NKS * 32);
    static LdsAttrOnce attr;
    hipError_t err = set_lds_limit_once(attr, reinterpret_cast<const void *>(&k_route_logits_mfma<NKS>), smem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((k_route_logits_mfma<NKS>), dim3(nwg), dim3(256), smem, s, X, T, Wr, bias, r.top_k,
                       r.expert_id, r.prob, wg_counts, nwg);
    return hipGetLastError();
}

// d_model values with a matrix-core router kernel (bf16 X, E = 8, wide path)
inline bool route_mfma_dm(int dm) { return dm == 512 || dm == 1024 || dm == 1536 || dm == 2048; }

static hipError_t launch_route_mfma(const uint16_t *X, int T, int dm, const float *Wr, const float *bias,
                                    const rom_routing &r, int32_t *wg_counts, int nwg, hipStream_t s) {
    switch (dm) {
        case 512: return launch_route_mfma_n<16>(X, T, Wr, bias, r, wg_counts, nwg, s);
        case 1024: return launch_route_mfma_n<32>(X, T, Wr, bias, r, wg_counts, nwg, s);
        case 1536: return launch_route_mfma_n<48>(X, T, Wr, bias, r, wg_counts, nwg, s);
        case 2048: return launch_route_mfma_n<64>(X, T, Wr, bias, r, wg_counts, nwg, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename TX, int EG, int EMAX>
static hipError_t launch_route_t(const TX *X, int T, int dm, const float *Wr, const float *bias, int E,
                                 const rom_routing &r, TX *Xp, int32_t *wg_counts, hipStream_t s) {
    const size_t wbytes = (size_t)dm * E * sizeof(float);
    // enough 32-token workgroups to fill the chip: one wave per 8 tokens; otherwise 8 tokens per
    // workgroup with the waves splitting d_model. W_r is staged in LDS only on the wide path: with 8
    // tokens per workgroup each W_r value serves too few tokens to repay the staging round trip, and for
    // T <= 8 one compute unit copying all of W_r was slower (decode_T1 7.7 -> 8.0 us) than reading it.
    const bool wide = (T + 31) / 32 >= 512;
    const int use_lds = wide && (E % 4 == 0) && (((E >> 2) & ((E >> 2) - 1)) == 0) && wbytes <= (size_t)kRouteLdsW;
    const size_t smem = use_lds ? wbytes : 0;
    if constexpr (std::is_same<TX, uint16_t>::value && EMAX <= 8) {
        // one or two bf16 rows: route_tiny's one round trip per thread beats k_route_small (decode_T1's router,
        // cold: 9.8 -> 7.5 us); from three rows on its per-token butterflies cost more than they save
        if (T <= kRouteTinyT) return launch_route_tiny<EMAX>(X, T, dm, Wr, bias, E, r, Xp, s);
    }
    if (T <= kRouteSmallT) {
        // 8 waves (one chunk per lane at d_model 4096) when the chunks and logits (bf16 rows, up to 8 experts)
        // fit the registers of 2 waves per SIMD, else 4
        constexpr int WPG = (EMAX <= 8 && sizeof(TX) == 2) ? 8 : 4;
        hipLaunchKernelGGL((k_route_small<TX, EG, EMAX, WPG>), dim3(1), dim3(64 * WPG), 0, s, X, T, dm, Wr, bias, E,
                           r.top_k, r.expert_id, r.prob, r.counts, r.offsets, r.perm, r.inv_perm, Xp);
        return hipGetLastError();
    }
    static LdsAttrOnce attr[2];
    const void *fns[2] = {reinterpret_cast<const void *>(&k_route_logits<TX, EG, EMAX, 1>),
                          reinterpret_cast<const void *>(&k_route_logits<TX, EG, EMAX, 4>)};
    for (int f = 0; f < 2; ++f) {
        hipError_t err = set_lds_limit_once(attr[f], fns[f], kRouteLdsW);
        if (err != hipSuccess) return err;
    }
    // bf16 rows, 8 experts and a d_model with a matrix-core kernel: 64 tokens per workgroup
    const bool mfma = std::is_same<TX, uint16_t>::value && wide && E == 8 && route_mfma_dm(dm);
    const int tpw = mfma ? kRouteMfmaTokensPerWG : wide ? 32 : 8;
    const int nwg = (T + tpw - 1) / tpw;
    hipError_t err = hipSuccess;
    if constexpr (std::is_same<TX, uint16_t>::value) {
        if (mfma) err = launch_route_mfma(X, T, dm, Wr, bias, r, wg_counts, nwg, s);
    }
    if (!mfma) {
        if (wide)
            hipLaunchKernelGGL((k_route_logits<TX, EG, EMAX, 1>), dim3(nwg), dim3(256), smem, s, X, T, dm, Wr, bias,
                               E, r.top_k, use_lds, r.expert_id, r.prob, wg_counts, nwg);
        else
            hipLaunchKernelGGL((k_route_logits<TX, EG, EMAX, 4>), dim3(nwg), dim3(256), smem, s, X, T, dm, Wr, bias,
                               E, r.top_k, use_lds, r.expert_id, r.prob, wg_counts, nwg);
        err = hipGetLastError();
    }
    if (err != hipSuccess) return err;
    const int nsc = scatter_workgroups(T), sub = kScatterTokensPerWG / tpw;
    int32_t *bases = nullptr;
    if ((long)nsc * nwg * E > kScatterPrescanMin) {
        bases = wg_counts + route_bases_offset(T, E);
        hipLaunchKernelGGL(k_route_scan, dim3(E, r.top_k), dim3(256), 0, s, wg_counts, nwg, sub, nsc, bases);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(k_route_scatter, dim3(nsc, r.top_k), dim3(256), 0, s, r.expert_id, T, E, wg_counts, nwg,
                       sub, bases, nsc, r.counts, r.offsets, r.perm, r.inv_perm);
    err = hipGetLastError();
    if (err != hipSuccess || Xp == nullptr) return err;
    const int cpr = dm * (int)sizeof(TX) / 16, rpw = perm_rows_per_wg(cpr);
    const uint32_t magic = (uint32_t)((1ull << 32) / (uint64_t)cpr + 1);
    hipLaunchKernelGGL((k_permute_rows<TX>), dim3((unsigned)((T + rpw - 1) / rpw)), dim3(256), 0, s, X, r.inv_perm, T,
                       cpr, rpw, magic, Xp);
    return hipGetLastError();
}

template <typename TX>
static hipError_t launch_route_e(const TX *X, int T, int dm, const float *Wr, const float *bias, int E,
                                 const rom_routing &r, TX *Xp, int32_t *wg_counts, hipStream_t s) {
    if (E <= 4) return launch_route_t<TX, 4, 4>(X, T, dm, Wr, bias, E, r, Xp, wg_counts, s);
    if (E <= 8) return launch_route_t<TX, 8, 8>(X, T, dm, Wr, bias, E, r, Xp, wg_counts, s);
    if (E <= 16) return launch_route_t<TX, 8, 16>(X, T, dm, Wr, bias, E, r, Xp, wg_counts, s);
    if (E <= 32) return launch_route_t<TX, 8, 32>(X, T, dm, Wr, bias, E, r, Xp, wg_counts, s);
    return launch_route_t<TX, 8, 64>(X, T, dm, Wr, bias, E, r, Xp, wg_counts, s);
}

hipError_t launch_route(const void *X, rom_dtype dt, int T, int dm, const float *Wr, const float *bias, int E,
                        const rom_routing &r, void *X_perm, int32_t *wg_counts, hipStream_t s) {
    if (dt == ROM_DTYPE_BF16)
        return launch_route_e<uint16_t>(static_cast<const uint16_t *>(X), T, dm, Wr, bias, E, r,
                                        static_cast<uint16_t *>(X_perm), wg_counts, s);
    return launch_route_e<float>(static_cast<const float *>(X), T, dm, Wr, bias, E, r, static_cast<float *>(X_perm),
                                 wg_counts, s);
}

}  // namespace rom
