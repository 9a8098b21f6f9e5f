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
// bf16 path: 256 threads = 2 x 2 waves; each wave owns a (BM/2) x (BN/2) block of 32x32 MFMA tiles
// (v_mfma_f32_32x32x16_bf16, fp32 accumulators). K advances in BK = 64 steps through two LDS
// buffers: the next A/B tiles are fetched into registers while the current ones feed the MFMAs.
// LDS rows are 128 bytes of 8 16-byte chunks, chunk c of row r stored at position c ^ (r & 7), so
// the 16-byte MFMA operand reads of 8 consecutive rows hit 8 different bank groups.
#include "rom_device.h"
#include "rom_internal.h"

namespace rom {

struct GemmArgs {
    const void *A0;       // in-proj: X [T][K];  out-proj: z [T][K]
    const void *A1;       // out-proj: h [T][K]
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
};

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
// bf16 MFMA grouped GEMM. OUT = false: in-projection; OUT = true: out-projection.
template <int BM, int BN, bool OUT>
__global__ __launch_bounds__(256) void k_grouped_gemm_bf16(GemmArgs p) {
    constexpr int BK = 64;
    constexpr int KCH = BK / 8;              // 16-byte chunks per LDS row
    constexpr int RPP = 256 / KCH;           // rows one 16-byte load per thread covers
    constexpr int A_LD = BM / RPP, B_LD = BN / RPP;
    constexpr int WM = BM / 2, WN = BN / 2;  // wave block
    constexpr int FM = WM / 32, FN = WN / 32;
    static_assert(BM % RPP == 0 && BN % RPP == 0 && FM >= 1 && FN >= 1, "tile shape");

    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    uint16_t *As = smem;                     // [2][BM*BK]
    uint16_t *Bs = smem + 2 * BM * BK;       // [2][BN*BK]
    __shared__ int s_tok[BM];
    __shared__ float s_prob[OUT ? BM : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int mt = blockIdx.x / p.n_tiles, nt = blockIdx.x % p.n_tiles;
    int e, slot0, rows;
    if (!locate_mtile<BM>(p.offsets, p.E, mt, e, slot0, rows)) return;
    const int which = nt / p.n_tiles_per_b;
    const int n0 = (nt % p.n_tiles_per_b) * BN;
    const int K = p.K;
    const uint16_t *Bsrc = static_cast<const uint16_t *>(which ? p.B1 : p.B0) + ((size_t)e * p.N0 + n0) * K;
    uint16_t *C = static_cast<uint16_t *>(which ? p.C1 : p.C0);

    for (int i = tid; i < BM; i += 256) {
        const int tok = i < rows ? p.perm[slot0 + i] : -1;
        s_tok[i] = tok;
        if (OUT) s_prob[i] = tok >= 0 ? p.prob[tok] : 0.0f;
    }
    __syncthreads();

    // global -> register slots: thread loads 16 bytes of row (lr + i*RPP), chunk lc
    const int lr = tid / KCH, lc = tid % KCH;
    const uint16_t *a_src[A_LD];
    const uint16_t *h_src[OUT ? A_LD : 1];
    int a_dst[A_LD], b_dst[B_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int r = lr + i * RPP;
        const int tok = s_tok[r];
        a_src[i] = tok >= 0 ? static_cast<const uint16_t *>(p.A0) + (size_t)tok * K + lc * 8 : nullptr;
        if (OUT) h_src[i] = tok >= 0 ? static_cast<const uint16_t *>(p.A1) + (size_t)tok * K + lc * 8 : nullptr;
        a_dst[i] = (r * KCH + (lc ^ (r & 7))) * 8;
    }
    const uint16_t *b_src[B_LD];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int r = lr + i * RPP;
        b_src[i] = Bsrc + (size_t)r * K + lc * 8;
        b_dst[i] = (r * KCH + (lc ^ (r & 7))) * 8;
    }

    uint4 ra[A_LD], rh[OUT ? A_LD : 1], rb[B_LD];
    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            ra[i] = a_src[i] ? *reinterpret_cast<const uint4 *>(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
            if (OUT) rh[i] = h_src[i] ? *reinterpret_cast<const uint4 *>(h_src[i] + k0) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) rb[i] = *reinterpret_cast<const uint4 *>(b_src[i] + k0);
    };
    auto store_tiles = [&](int buf) {
        uint16_t *as = As + buf * BM * BK;
        uint16_t *bs = Bs + buf * BN * BK;
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            uint4 v = ra[i];
            if (OUT) {
                // a = bf16(SiLU(z) * h), fp32 arithmetic
                const uint32_t zw[4] = {v.x, v.y, v.z, v.w};
                const uint32_t hw[4] = {rh[i].x, rh[i].y, rh[i].z, rh[i].w};
                uint32_t o[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float z0 = __uint_as_float(zw[q] << 16), z1 = __uint_as_float(zw[q] & 0xFFFF0000u);
                    const float h0 = __uint_as_float(hw[q] << 16), h1 = __uint_as_float(hw[q] & 0xFFFF0000u);
                    o[q] = pack_bf16x2(silu_fast(z0) * h0, silu_fast(z1) * h1);
                }
                v = make_uint4(o[0], o[1], o[2], o[3]);
            }
            *reinterpret_cast<uint4 *>(as + a_dst[i]) = v;
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) *reinterpret_cast<uint4 *>(bs + b_dst[i]) = rb[i];
    };

    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = K / BK;
    load_tiles(0);
    store_tiles(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_tiles((kt + 1) * BK);
        const uint16_t *as = As + buf * BM * BK;
        const uint16_t *bs = Bs + buf * BN * BK;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int chunk = kk * 2 + (lane >> 5);
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = wm * WM + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const bf16x8 *>(as + (r * KCH + (chunk ^ (r & 7))) * 8);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int r = wn * WN + j * 32 + (lane & 31);
                bfr[j] = *reinterpret_cast<const bf16x8 *>(bs + (r * KCH + (chunk ^ (r & 7))) * 8);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store_tiles(buf ^ 1);
        __syncthreads();
    }

    // epilogue: accumulator register r of a 32x32 block holds row 8*(r/4) + 4*(lane/32) + (r%4),
    // column lane%32; rows go back to their tokens (un-permute), scaled by p_t for the out-projection
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int col = wn * WN + j * 32 + (lane & 31);
                if (row < rows) {
                    const int tok = s_tok[row];
                    float v = acc[i][j][r];
                    if (OUT) v *= s_prob[row];
                    C[(size_t)tok * p.N0 + n0 + col] = f32_to_bf16(v);
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
    const float *h_src = (OUT && tok >= 0) ? static_cast<const float *>(p.A1) + (size_t)tok * K + lk : nullptr;
    const float *b_src = Bsrc + (size_t)lr * K + lk;
    const int ty = tid >> 4, tx = tid & 15;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += BK) {
        float4 a = a_src ? *reinterpret_cast<const float4 *>(a_src + k0) : make_float4(0, 0, 0, 0);
        if (OUT && a_src) {
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
            *reinterpret_cast<float4 *>(C + (size_t)t * p.N0 + n0 + tx * 4) = v;
        }
    }
}

// ---------------------------------------------------------------------------------------------

template <int BM, int BN, bool OUT>
static hipError_t launch_bf16(const GemmArgs &a0, int nB, hipStream_t s) {
    GemmArgs a = a0;
    a.n_tiles_per_b = a.N0 / BN;
    a.n_tiles = nB * a.n_tiles_per_b;
    const int max_mtiles = (a.T + a.E * (BM - 1)) / BM;
    const size_t smem = (size_t)2 * (BM + BN) * 64 * sizeof(uint16_t);
    static bool attr_set = false;  // per process; the attribute is per function
    if (!attr_set) {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_grouped_gemm_bf16<BM, BN, OUT>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    hipLaunchKernelGGL((k_grouped_gemm_bf16<BM, BN, OUT>), dim3((unsigned)max_mtiles * a.n_tiles), dim3(256), smem, s,
                       a);
    return hipGetLastError();
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

hipError_t launch_in_proj(const void *X, const rom_routing &r, rom_dtype dt, int T, int dm, int di, const void *Wc,
                          const void *Wg, void *x_out, void *z_out, hipStream_t s) {
    GemmArgs a{};
    a.A0 = X;
    a.B0 = Wc;
    a.B1 = Wg;
    a.C0 = x_out;
    a.C1 = z_out;
    a.offsets = r.offsets;
    a.perm = r.perm;
    a.prob = r.prob;
    a.T = T;
    a.K = dm;
    a.N0 = di;
    a.E = r.E;
    if (dt == ROM_DTYPE_F32) return launch_f32<false>(a, 2, s);
    if (di % 128 == 0) return launch_bf16<128, 128, false>(a, 2, s);
    return launch_bf16<128, 64, false>(a, 2, s);
}

hipError_t launch_out_proj(const void *z, const void *h, const rom_routing &r, rom_dtype dt, int T, int dm, int di,
                           const void *Wo, void *out, hipStream_t s) {
    GemmArgs a{};
    a.A0 = z;
    a.A1 = h;
    a.B0 = Wo;
    a.C0 = out;
    a.offsets = r.offsets;
    a.perm = r.perm;
    a.prob = r.prob;
    a.T = T;
    a.K = di;
    a.N0 = dm;
    a.E = r.E;
    if (dt == ROM_DTYPE_F32) return launch_f32<true>(a, 1, s);
    if (dm % 128 == 0) return launch_bf16<128, 128, true>(a, 1, s);
    return launch_bf16<128, 64, true>(a, 1, s);
}

}  // namespace rom
