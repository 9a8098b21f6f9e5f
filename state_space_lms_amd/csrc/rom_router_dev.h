// rom_router_dev.h -- device code of the router's logits, softmax, top-k selection and small-T grouping
// (internal header of rom_route.hip).
//
// Method: Routing Mamba landing page (chapterpal.com), Knowl 1: logit_t,j = sum_k X[t][k] * W_r[k][j] in fp32,
// p_t = Softmax(logits), S_t = the K largest.
#pragma once

#include "rom_device.h"
#include "rom_internal.h"

namespace rom {

// Raw 8-element chunk of an X row (kept packed until used, to hold two chunk sets in registers).
template <typename TX> struct Chunk8;
template <> struct Chunk8<uint16_t> {
    uint4 v;
    __device__ __forceinline__ void load(const uint16_t *p) { v = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ void unpack(float f[8]) const {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
};
template <> struct Chunk8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = reinterpret_cast<const float4 *>(p)[0];
        b = reinterpret_cast<const float4 *>(p)[1];
    }
    __device__ __forceinline__ void unpack(float f[8]) const {
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
};

// The 8 token rows of a group [tok0, tok0+8) and two 8-row chunk buffers: lane jl (of LPT lanes) reads
// the 8-element chunks c = jl, jl+LPT, ... of d_model, chunk jl into `a` and jl+LPT into `b`, so two
// chunks per row are in flight at a time. Tokens past T read row T-1 and are discarded; chunks past the
// row end are not loaded.
template <typename TX> struct XRows {
    const TX *row[8];
    Chunk8<TX> a[8], b[8];
};

// s_barrier without the memory fence of __syncthreads(): the caller has waited for what the other
// waves read after it.
__device__ __forceinline__ void barrier_no_fence() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Vector loads per chunk set of XRows (one set = one 8-element chunk of each of the 8 rows).
template <typename TX> constexpr int kXrowsSetLoads = 8 * (int)sizeof(TX) / 2;

// Issues the loads of chunks jl and jl+LPT. Called before the router weight is staged, so that the first
// X fetches overlap the staging.
template <typename TX, int LPT>
__device__ __forceinline__ void xrows_issue(XRows<TX> &xr, const TX *__restrict__ X, int T, int dm, int tok0, int jl) {
    const int nchunk = dm >> 3;
#pragma unroll
    for (int q = 0; q < 8; ++q) xr.row[q] = X + (size_t)min(tok0 + q, T - 1) * dm;
    const int c0 = min(jl, nchunk - 1);
#pragma unroll
    for (int q = 0; q < 8; ++q) xr.a[q].load(xr.row[q] + c0 * 8);
    if (jl + LPT < nchunk) {
#pragma unroll
        for (int q = 0; q < 8; ++q) xr.b[q].load(xr.row[q] + (jl + LPT) * 8);
    }
}

// W_r rows [8c, 8c+8) of one chunk c for the experts [e0, e0+EG) (zeros past E), held in registers.
template <int EG> struct WrChunk {
    float w[8][EG];
};
template <int EG>
__device__ __forceinline__ void wr_chunk_load(WrChunk<EG> &wc, const float *__restrict__ Wr, int E, int e0, int c) {
    const bool vecw = (E % 4 == 0) && (EG % 4 == 0) && (e0 + EG <= E);
    const float *wrow = Wr + (size_t)(c * 8) * E + e0;
    if (vecw) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
            for (int x = 0; x < EG; x += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(wrow + (size_t)kk * E + x);
                wc.w[kk][x] = v.x; wc.w[kk][x + 1] = v.y; wc.w[kk][x + 2] = v.z; wc.w[kk][x + 3] = v.w;
            }
    } else {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
            for (int x = 0; x < EG; ++x) wc.w[kk][x] = (e0 + x < E) ? wrow[(size_t)kk * E + x] : 0.0f;
    }
}

// Logits of the 8 tokens of xr (whose first two chunks are in flight) for the experts [e0, e0+EG),
// computed by LPT lanes (LPT = 64 * waves; lane jl = 0..LPT-1). Each lane's partial sums over its chunks
// are then reduce-scattered over lane bits 0..2 (each lane keeps one token) and all-reduced over lane
// bits 3..5. On return every lane of the wave with (lane & 7) == j holds this wave's partial logits of
// token tok0 + j in out[0..EG); with LPT > 64 the caller still sums the waves. Must be called by every
// lane of the wave (it shuffles). wl != nullptr: W_r is read from the LDS copy made by
// stage_router_weight. Rows q >= nrows (tokens past T) get no FMAs; their zero sums are discarded.
// PRE: the W_r rows of the lane's first chunk (jl) are already in `pre` (loaded with the X rows, so that both
// come back in one round trip; when the loop below loads them, the compiler makes those loads wait for the X rows,
// whose registers later iterations refill).
template <typename TX, int LPT, int EG, bool PRE = false>
__device__ __forceinline__ void logits_group8(XRows<TX> &xr, int dm, const float *__restrict__ Wr, const float4 *wl,
                                              int E, int e0, int jl, int nrows, float out[EG],
                                              const WrChunk<EG> *pre = nullptr) {
    float acc[8][EG];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int x = 0; x < EG; ++x) acc[q][x] = 0.0f;

    const int nchunk = dm >> 3;
    const bool vecw = (E % 4 == 0) && (EG % 4 == 0) && (e0 + EG <= E);
    const int e4 = E >> 2;
    // acc += the 8 rows' chunk c (held in buf) times the W_r rows w
    auto fma8 = [&](const Chunk8<TX>(&buf)[8], const float (&w)[8][EG]) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (q < nrows) {  // uniform; rows past T repeat row T - 1 and are discarded
                float xf[8];
                buf[q].unpack(xf);
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                    for (int x = 0; x < EG; ++x) acc[q][x] = fmaf(xf[kk], w[kk][x], acc[q][x]);
            }
        }
    };
    // acc += the 8 rows' chunk c (held in buf) times W_r rows [8c, 8c+8)
    auto mac = [&](const Chunk8<TX>(&buf)[8], int c) {
        float w[8][EG];
        if (wl != nullptr && vecw) {
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                for (int x = 0; x < EG; x += 4) {
                    const float4 v = wl[(kk * e4 + ((e0 + x) >> 2)) * nchunk + c];
                    w[kk][x] = v.x; w[kk][x + 1] = v.y; w[kk][x + 2] = v.z; w[kk][x + 3] = v.w;
                }
        } else if (vecw) {
            const float *wrow = Wr + (size_t)(c * 8) * E + e0;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                for (int x = 0; x < EG; x += 4) {
                    const float4 v = *reinterpret_cast<const float4 *>(wrow + (size_t)kk * E + x);
                    w[kk][x] = v.x; w[kk][x + 1] = v.y; w[kk][x + 2] = v.z; w[kk][x + 3] = v.w;
                }
        } else {
            const float *wrow = Wr + (size_t)(c * 8) * E + e0;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                for (int x = 0; x < EG; ++x) w[kk][x] = (e0 + x < E) ? wrow[(size_t)kk * E + x] : 0.0f;
        }
        fma8(buf, w);
    };
    int cstart = jl;
    if constexpr (PRE) {
        // the first chunk pair with the pre-loaded W_r rows of chunk jl
        if (jl < nchunk) {
            fma8(xr.a, pre->w);
            if (jl + 2 * LPT < nchunk) {
#pragma unroll
                for (int q = 0; q < 8; ++q) xr.a[q].load(xr.row[q] + (jl + 2 * LPT) * 8);
            }
            if (jl + LPT < nchunk) {
                mac(xr.b, jl + LPT);
                if (jl + 3 * LPT < nchunk) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) xr.b[q].load(xr.row[q] + (jl + 3 * LPT) * 8);
                }
            }
        }
        cstart = jl + 2 * LPT;
    }
    // chunks c (in a) and c + LPT (in b); each buffer is refilled two strides ahead as soon as it is used
    for (int c = cstart; c < nchunk; c += 2 * LPT) {
        mac(xr.a, c);
        if (c + 2 * LPT < nchunk) {
#pragma unroll
            for (int q = 0; q < 8; ++q) xr.a[q].load(xr.row[q] + (c + 2 * LPT) * 8);
        }
        if (c + LPT < nchunk) {
            mac(xr.b, c + LPT);
            if (c + 3 * LPT < nchunk) {
#pragma unroll
                for (int q = 0; q < 8; ++q) xr.b[q].load(xr.row[q] + (c + 3 * LPT) * 8);
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
#pragma unroll
    for (int m = 8; m < 64; m <<= 1)
#pragma unroll
        for (int x = 0; x < EG; ++x) out[x] += __shfl_xor(out[x], m);
}

// All E logits (this wave's share when LPT > 64) of token (tok0 + (jl & 7)) into lg[0..EMAX)
// (entries >= E are -inf). xr holds the issued first chunks; later expert groups re-read X.
template <typename TX, int LPT, int EG, int EMAX, bool PRE = false>
__device__ __forceinline__ void logits_token(XRows<TX> &xr, const TX *X, int T, int dm, const float *Wr,
                                             const float4 *wl, int E, int tok0, int jl, float lg[EMAX],
                                             const WrChunk<EG> *pre = nullptr) {
#pragma unroll
    for (int g = 0; g < EMAX / EG; ++g) {
        if (g * EG < E) {  // uniform
            if (g > 0) xrows_issue<TX, LPT>(xr, X, T, dm, tok0, jl);
            float o[EG];
            if (PRE && g == 0)
                logits_group8<TX, LPT, EG, true>(xr, dm, Wr, wl, E, 0, jl, min(8, T - tok0), o, pre);
            else
                logits_group8<TX, LPT, EG>(xr, dm, Wr, wl, E, g * EG, jl, min(8, T - tok0), o);
#pragma unroll
            for (int x = 0; x < EG; ++x) lg[g * EG + x] = (g * EG + x < E) ? o[x] : -INFINITY;
        } else {
#pragma unroll
            for (int x = 0; x < EG; ++x) lg[g * EG + x] = -INFINITY;
        }
    }
}

// The token group and lane index of this thread in wg_logits: WPG = 1: wave w owns the 8 tokens
// [tok_base + 8w, +8) with lanes 0..63; WPG = 4: the four waves split d_model (lanes 0..255) for the 8
// tokens [tok_base, +8).
template <int WPG>
__device__ __forceinline__ void wg_token_group(int tok_base, int &tok0, int &jl) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    tok0 = WPG == 1 ? tok_base + wave * 8 : tok_base;
    jl = WPG == 1 ? lane : wave * 64 + lane;
}

// Logits of the workgroup's tokens (xr issued by xrows_issue for the group of wg_token_group). With
// WPG = 4 the waves' partial sums are added in wave order through LDS (s_red). On return, lanes 0..7
// of every wave (WPG = 1) or of wave 0 (WPG = 4) hold the full logits of token tok0 + lane, where tok0
// is returned.
template <typename TX, int EG, int EMAX, int WPG, bool PRE = false>
__device__ __forceinline__ int wg_logits(XRows<TX> &xr, const TX *X, int T, int dm, const float *Wr, const float4 *wl,
                                         int E, int tok_base, float lg[EMAX], float (*s_red)[8][EMAX],
                                         const WrChunk<EG> *pre = nullptr) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int tok0, jl;
    wg_token_group<WPG>(tok_base, tok0, jl);
    if (WPG == 1) {
        logits_token<TX, 64, EG, EMAX, PRE>(xr, X, T, dm, Wr, wl, E, tok0, jl, lg, pre);
        return tok0;
    }
    logits_token<TX, 64 * WPG, EG, EMAX, PRE>(xr, X, T, dm, Wr, wl, E, tok0, jl, lg, pre);
    if (lane < 8) {
#pragma unroll
        for (int e = 0; e < EMAX; ++e) s_red[wave][lane][e] = lg[e];
    }
    __syncthreads();
    if (lane < 8) {  // the waves' partial sums, added in wave order
#pragma unroll
        for (int e = 0; e < EMAX; ++e) {
            float v = s_red[0][lane][e];
#pragma unroll
            for (int w = 1; w < WPG; ++w) v += s_red[w][lane][e];
            lg[e] = v;
        }
    }
    return tok_base;
}

// Bias, the K (1 or 2) largest logits (each choice keeps the lowest index on ties), and their softmax
// probabilities over all E experts (not renormalised over the choice).
template <int EMAX>
__device__ __forceinline__ void select_topk(float lg[EMAX], const float *bias, int E, int K, int (&best)[2],
                                            float (&p)[2]) {
    if (bias) {
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
            if (e < E) lg[e] = lg[e] + bias[e];
    }
    int b0 = 0;
    float l0 = lg[0];
#pragma unroll
    for (int e = 1; e < EMAX; ++e)
        if (e < E && lg[e] > l0) { l0 = lg[e]; b0 = e; }
    int b1 = -1;
    float l1 = -INFINITY;
    if (K > 1) {
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
            if (e < E && e != b0 && (b1 < 0 || lg[e] > l1)) { l1 = lg[e]; b1 = e; }
    }
    float denom = 0.0f;
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
        if (e < E) denom += expf(lg[e] - l0);
    best[0] = b0;
    best[1] = b1;
    p[0] = 1.0f / denom;
    p[1] = K > 1 ? expf(l1 - l0) / denom : 0.0f;
}


// ---------------------------------------------------------------------------------------------
// The whole routing of a few tokens (T <= TMAX <= 8) by one workgroup of 512 threads, for bf16 rows and at most
// 8 experts. Thread i owns the 8-element chunks c = i, i + 512, ... of d_model: it loads the T tokens' chunk c
// (16 bytes each) and W_r rows 8c .. 8c + 7 (E fp32 each) at once, and accumulates x[t][8c + kk] * W_r[8c + kk][e]
// in fp32, kk ascending; each wave then sums its lanes with an xor butterfly (offsets 32, 16, .., 1) and the 8
// waves' sums are added in wave order. With one token that is E accumulators and one round trip to memory per
// thread. Then, for each choice k < K, the bias, top-k and probability of select_topk, and the grouping counted
// directly: slot = (tokens of lower experts) + (earlier tokens of the same expert). s_pos receives the slot of
// each token of choice 0 (for the permute).
// Tokens up to which the router takes route_tiny (bf16 rows, at most 8 experts).
constexpr int kRouteTinyT = 2;
static_assert(kRouteTinyT <= 8, "route_tiny keeps at most 8 tokens");

template <int TMAX, int EMAX>
struct RouteTinyLds {
    float part[8][TMAX][EMAX];          // the waves' partial logits
    int ids[ROM_MAX_TOP_K][8];          // choice k of token t
    int pos[8];                         // token -> slot, choice 0
};

template <int TMAX, int EMAX>
__device__ __forceinline__ void route_tiny(const uint16_t *__restrict__ X, int T, int dm, const float *__restrict__ Wr,
                                           const float *__restrict__ bias, int E, int K, int32_t *ids, float *prob,
                                           int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_perm,
                                           RouteTinyLds<TMAX, EMAX> &sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float acc[TMAX][EMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
#pragma unroll
        for (int e = 0; e < EMAX; ++e) acc[t][e] = 0.0f;
    const int nchunk = dm >> 3;
    const bool vecw = (E & 3) == 0;
    for (int c = tid; c < nchunk; c += 512) {
        uint4 xv[TMAX];
#pragma unroll
        for (int t = 0; t < TMAX; ++t) xv[t] = *reinterpret_cast<const uint4 *>(X + (size_t)min(t, T - 1) * dm + c * 8);
        float w[8][EMAX];
        const float *wrow = Wr + (size_t)(c * 8) * E;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            if (vecw) {
#pragma unroll
                for (int e = 0; e < EMAX; e += 4) {
                    const float4 v = e < E ? *reinterpret_cast<const float4 *>(wrow + kk * E + e)
                                           : make_float4(0.f, 0.f, 0.f, 0.f);
                    w[kk][e] = v.x; w[kk][e + 1] = v.y; w[kk][e + 2] = v.z; w[kk][e + 3] = v.w;
                }
            } else {
#pragma unroll
                for (int e = 0; e < EMAX; ++e) w[kk][e] = e < E ? wrow[kk * E + e] : 0.0f;
            }
        }
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t < T) {  // uniform
                const uint32_t xw[4] = {xv[t].x, xv[t].y, xv[t].z, xv[t].w};
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const float xf = (kk & 1) ? __uint_as_float(xw[kk >> 1] & 0xFFFF0000u)
                                              : __uint_as_float(xw[kk >> 1] << 16);
#pragma unroll
                    for (int e = 0; e < EMAX; ++e) acc[t][e] = fmaf(xf, w[kk][e], acc[t][e]);
                }
            }
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
#pragma unroll
        for (int t = 0; t < TMAX; ++t)
#pragma unroll
            for (int e = 0; e < EMAX; ++e) acc[t][e] += __shfl_xor(acc[t][e], m);
    if (lane == 0) {
#pragma unroll
        for (int t = 0; t < TMAX; ++t)
#pragma unroll
            for (int e = 0; e < EMAX; ++e) sm.part[wave][t][e] = acc[t][e];
    }
    __syncthreads();
    if (tid < T) {  // token tid: the waves' sums in wave order, then the choices
        float lg[EMAX];
#pragma unroll
        for (int e = 0; e < EMAX; ++e) {
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < 8; ++w) v += sm.part[w][tid][e];  // tid < T <= TMAX
            lg[e] = e < E ? v : -INFINITY;
        }
        int best[2];
        float p[2];
        select_topk<EMAX>(lg, bias, E, K, best, p);
#pragma unroll
        for (int k = 0; k < ROM_MAX_TOP_K; ++k) {
            if (k < K) {
                sm.ids[k][tid] = best[k];
                ids[k * T + tid] = best[k];
                prob[k * T + tid] = p[k];
            }
        }
    }
    __syncthreads();
    for (int k = 0; k < K; ++k) {  // the K stacked top-1 groupings
        const int *sid = sm.ids[k];
        if (tid < T) {
            const int e = sid[tid];
            int pos = 0;
            for (int t = 0; t < T; ++t) pos += (sid[t] < e) || (sid[t] == e && t < tid);
            perm[k * T + pos] = tid;
            inv_perm[k * T + tid] = pos;
            if (k == 0) sm.pos[tid] = pos;
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
    }
    __syncthreads();
}

}  // namespace rom
