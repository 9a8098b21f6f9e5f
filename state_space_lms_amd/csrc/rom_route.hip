// rom_route.hip -- the shared router of a Routing Mamba block on gfx950, and the grouping of tokens
// by expert (histogram, scan, stable counting-sort scatter, optional permute).
//
// Method: Routing Mamba landing page (chapterpal.com), Knowl 1: p_t = Softmax(x_t W_r) over the
// experts, S_t = the top-1 expert, r_t = p_t,e* (not renormalised). The grouping is not on the page;
// a dropless grouped GEMM (Knowl 12: no capacity factor, no token dropping) needs it.
//
// Router arithmetic is fp32: logit_t,j = sum_k X[t][k] * W_r[k][j] (+ bias[j]); argmax keeps the
// lowest index on ties (strict > in ascending j); prob = 1 / sum_j exp(logit_j - logit_max).
// The router reads X once (HBM-bound: E flops per element); W_r (d_model * E * 4 bytes) stays in
// L1/L2 and each lane reuses the W_r values it loads across 8 tokens.
#include "rom_device.h"
#include "rom_internal.h"

namespace rom {

// ---------------------------------------------------------------------------------------------
// Logits of a group of 8 tokens [tok0, tok0+8) for the experts [e0, e0+EG), computed by LPT lanes
// (LPT = 8 or 64, consecutive lanes). Lane jl (0..LPT-1) sums the 8-element chunks c = jl, jl+LPT,
// ... of d_model. Partial sums are then reduce-scattered over lane bits 0..2 (each lane keeps one
// token) and, for LPT = 64, all-reduced over bits 3..5. On return lane jl holds the logits of token
// tok0 + (jl & 7) in out[0..EG). Must be called by every lane of the wave (it shuffles).
template <typename TX, int LPT, int EG>
__device__ __forceinline__ void logits_group8(const TX *__restrict__ X, int T, int dm, const float *__restrict__ Wr,
                                              int E, int e0, int tok0, int jl, float out[EG]) {
    float acc[8][EG];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int x = 0; x < EG; ++x) acc[q][x] = 0.0f;

    const int nchunk = dm >> 3;
    const bool vecw = (E % 4 == 0) && (EG % 4 == 0) && (e0 + EG <= E);
    for (int c = jl; c < nchunk; c += LPT) {
        float w[8][EG];
        const float *wrow = Wr + (size_t)(c * 8) * E + e0;
        if (vecw) {
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                for (int x = 0; x < EG; x += 4) {
                    float4 v = *reinterpret_cast<const float4 *>(wrow + (size_t)kk * E + x);
                    w[kk][x] = v.x; w[kk][x + 1] = v.y; w[kk][x + 2] = v.z; w[kk][x + 3] = v.w;
                }
        } else {
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                for (int x = 0; x < EG; ++x) w[kk][x] = (e0 + x < E) ? wrow[(size_t)kk * E + x] : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int t = tok0 + q;
            if (t < T) {
                float xf[8];
                load8_f32(X + (size_t)t * dm + c * 8, xf);
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                    for (int x = 0; x < EG; ++x) acc[q][x] = fmaf(xf[kk], w[kk][x], acc[q][x]);
            }
        }
    }
    // reduce-scatter over lane bits 2, 1, 0: after the three steps lane j keeps token (j & 7)
    const int j = jl & 7;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int x = 0; x < EG; ++x) {
            const float keep = (j & 4) ? acc[q + 4][x] : acc[q][x];
            const float send = (j & 4) ? acc[q][x] : acc[q + 4][x];
            acc[q][x] = keep + __shfl_xor(send, 4);
        }
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int x = 0; x < EG; ++x) {
            const float keep = (j & 2) ? acc[q + 2][x] : acc[q][x];
            const float send = (j & 2) ? acc[q][x] : acc[q + 2][x];
            acc[q][x] = keep + __shfl_xor(send, 2);
        }
#pragma unroll
    for (int x = 0; x < EG; ++x) {
        const float keep = (j & 1) ? acc[1][x] : acc[0][x];
        const float send = (j & 1) ? acc[0][x] : acc[1][x];
        out[x] = keep + __shfl_xor(send, 1);
    }
    if (LPT > 8) {
#pragma unroll
        for (int m = 8; m < LPT; m <<= 1)
#pragma unroll
            for (int x = 0; x < EG; ++x) out[x] += __shfl_xor(out[x], m);
    }
}

// All E logits of token (tok0 + (jl & 7)) into lg[0..EMAX) (entries >= E are -inf).
template <typename TX, int LPT, int EG, int EMAX>
__device__ __forceinline__ void logits_token(const TX *X, int T, int dm, const float *Wr, int E, int tok0, int jl,
                                             float lg[EMAX]) {
#pragma unroll
    for (int g = 0; g < EMAX / EG; ++g) {
        if (g * EG < E) {  // uniform
            float o[EG];
            logits_group8<TX, LPT, EG>(X, T, dm, Wr, E, g * EG, tok0, jl, o);
#pragma unroll
            for (int x = 0; x < EG; ++x) lg[g * EG + x] = (g * EG + x < E) ? o[x] : -INFINITY;
        } else {
#pragma unroll
            for (int x = 0; x < EG; ++x) lg[g * EG + x] = -INFINITY;
        }
    }
}

// Bias, argmax (lowest index on ties), and the top-1 softmax probability.
template <int EMAX>
__device__ __forceinline__ void select_top1(float lg[EMAX], const float *bias, int E, int &best, float &p) {
    if (bias) {
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
            if (e < E) lg[e] = lg[e] + bias[e];
    }
    best = 0;
    float lmax = lg[0];
#pragma unroll
    for (int e = 1; e < EMAX; ++e)
        if (e < E && lg[e] > lmax) { lmax = lg[e]; best = e; }
    float denom = 0.0f;
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
        if (e < E) denom += expf(lg[e] - lmax);
    p = 1.0f / denom;
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
// 256 tokens per workgroup; lane groups of 8 lanes each own 8 tokens.
template <typename TX, int EG, int EMAX>
__global__ __launch_bounds__(256) void k_route_logits(const TX *__restrict__ X, int T, int dm,
                                                      const float *__restrict__ Wr, const float *__restrict__ bias,
                                                      int E, int32_t *__restrict__ ids, float *__restrict__ prob,
                                                      int32_t *__restrict__ wg_counts, int nwg) {
    __shared__ int hist[ROM_MAX_EXPERTS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < E; i += 256) hist[i] = 0;
    __syncthreads();
    const int jl = lane & 7;
    const int tok0 = blockIdx.x * kRouteTokensPerWG + wave * 64 + (lane >> 3) * 8;
    float lg[EMAX];
    logits_token<TX, 8, EG, EMAX>(X, T, dm, Wr, E, tok0, jl, lg);
    const int t = tok0 + jl;
    if (t < T) {
        int best;
        float p;
        select_top1<EMAX>(lg, bias, E, best, p);
        ids[t] = best;
        prob[t] = p;
        atomicAdd(&hist[best], 1);
    }
    __syncthreads();
    for (int i = tid; i < E; i += 256) wg_counts[(size_t)i * nwg + blockIdx.x] = hist[i];
}

// Multi-workgroup path, kernel 2: per-expert totals and bases, then the stable scatter.
template <typename TX>
__global__ __launch_bounds__(256) void k_route_scatter(const int32_t *__restrict__ ids, int T, int E,
                                                       const int32_t *__restrict__ wg_counts, int nwg,
                                                       int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                       int32_t *__restrict__ perm, int32_t *__restrict__ inv_perm,
                                                       const TX *__restrict__ X, TX *__restrict__ Xp, int dm) {
    __shared__ int s_before[ROM_MAX_EXPERTS], s_total[ROM_MAX_EXPERTS], s_base[ROM_MAX_EXPERTS];
    __shared__ int s_wcnt[4][ROM_MAX_EXPERTS];
    __shared__ int s_pos[kRouteTokensPerWG];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wg = blockIdx.x;
    for (int e = wave; e < E; e += 4) {
        int before = 0, total = 0;
        for (int w = lane; w < nwg; w += 64) {
            const int c = wg_counts[(size_t)e * nwg + w];
            total += c;
            before += (w < wg) ? c : 0;
        }
        for (int m = 32; m >= 1; m >>= 1) {
            before += __shfl_xor(before, m);
            total += __shfl_xor(total, m);
        }
        if (lane == 0) { s_before[e] = before; s_total[e] = total; }
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
    const int t = wg * kRouteTokensPerWG + tid;
    const int e = t < T ? ids[t] : -1;
    const int rank = wg_stable_rank(e, E, s_wcnt);
    int pos = -1;
    if (e >= 0) {
        pos = s_base[e] + rank;
        perm[pos] = t;
        inv_perm[t] = pos;
    }
    if (Xp) {
        s_pos[tid] = pos;
        __syncthreads();
        permute_rows<TX>(X, Xp, dm, wg * kRouteTokensPerWG, min(kRouteTokensPerWG, T - wg * kRouteTokensPerWG), s_pos);
    }
}

// ---------------------------------------------------------------------------------------------
// Small-T path (T <= 256): the whole routing in one workgroup and one launch. Each wave takes
// groups of 8 tokens and splits d_model over all 64 lanes.
template <typename TX, int EG, int EMAX>
__global__ __launch_bounds__(256) void k_route_small(const TX *__restrict__ X, int T, int dm,
                                                     const float *__restrict__ Wr, const float *__restrict__ bias,
                                                     int E, int32_t *__restrict__ ids, float *__restrict__ prob,
                                                     int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                     int32_t *__restrict__ perm, int32_t *__restrict__ inv_perm,
                                                     TX *__restrict__ Xp) {
    __shared__ int s_ids[kRouteSmallT];
    __shared__ int s_base[ROM_MAX_EXPERTS];
    __shared__ int s_wcnt[4][ROM_MAX_EXPERTS];
    __shared__ int s_pos[kRouteSmallT];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ngroups = (T + 7) >> 3;
    for (int g = wave; g < ngroups; g += 4) {
        float lg[EMAX];
        logits_token<TX, 64, EG, EMAX>(X, T, dm, Wr, E, g * 8, lane, lg);
        const int t = g * 8 + lane;
        if (lane < 8 && t < T) {
            int best;
            float p;
            select_top1<EMAX>(lg, bias, E, best, p);
            ids[t] = best;
            prob[t] = p;
            s_ids[t] = best;
        }
    }
    __syncthreads();
    if (tid < E) {
        int c = 0;
        for (int t = 0; t < T; ++t) c += (s_ids[t] == tid);
        s_wcnt[0][tid] = c;  // borrowed as the histogram until the scan below
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int e = 0; e < E; ++e) {
            const int c = s_wcnt[0][e];
            s_base[e] = run;
            counts[e] = c;
            offsets[e] = run;
            run += c;
        }
        offsets[E] = run;
    }
    __syncthreads();
    const int e = tid < T ? s_ids[tid] : -1;
    const int rank = wg_stable_rank(e, E, s_wcnt);
    int pos = -1;
    if (e >= 0) {
        pos = s_base[e] + rank;
        perm[pos] = tid;
        inv_perm[tid] = pos;
    }
    if (Xp) {
        s_pos[tid] = pos;
        __syncthreads();
        permute_rows<TX>(X, Xp, dm, 0, T, s_pos);
    }
}

// ---------------------------------------------------------------------------------------------

template <typename TX, int EG, int EMAX>
static hipError_t launch_route_t(const TX *X, int T, int dm, const float *Wr, const float *bias, int E,
                                 const rom_routing &r, TX *Xp, int32_t *wg_counts, hipStream_t s) {
    if (T <= kRouteSmallT) {
        hipLaunchKernelGGL((k_route_small<TX, EG, EMAX>), dim3(1), dim3(256), 0, s, X, T, dm, Wr, bias, E,
                           r.expert_id, r.prob, r.counts, r.offsets, r.perm, r.inv_perm, Xp);
        return hipGetLastError();
    }
    const int nwg = route_workgroups(T);
    hipLaunchKernelGGL((k_route_logits<TX, EG, EMAX>), dim3(nwg), dim3(256), 0, s, X, T, dm, Wr, bias, E,
                       r.expert_id, r.prob, wg_counts, nwg);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((k_route_scatter<TX>), dim3(nwg), dim3(256), 0, s, r.expert_id, T, E, wg_counts, nwg,
                       r.counts, r.offsets, r.perm, r.inv_perm, X, Xp, dm);
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
