/*
 * rom.h -- C ABI of the MI355X (gfx950) Routing Mamba routed-projection library (librom.so).
 *
 * The operations follow "Routing Mamba: Scaling State Space Models with Mixture-of-Experts
 * Projection" as summarised on its chapterpal.com landing page, Knowl 1 ("RoM uses one sparse
 * routing decision for Mamba projection experts"):
 *   p_t = Softmax(x_t W_r) over N experts, S_t = the K largest, r_t,i = p_t,i 1[i in S_t];
 *   H_t = sum_i 1[i in S_t] x_t W_in,i         G_t = SiLU(sum_i 1[i in S_t] x_t W_g,i);
 *   O_t = sum_i r_t,i (Y_t (.) G_t) W_out,i.
 * One router per block, shared by the Conv (input), Gate and Out projections (Knowl 1, and the
 * authors' rebuttal on the paperhub.cn page, reply to reviewer VBDT), one (top-1) or two (top-2)
 * of the experts per token, dropless: no capacity factor and no token dropping (Knowl 12). The page's
 * scaling notes (Knowl 1) measure the 8top1, 16top1 and 8top2 settings.
 *
 * Conventions for every entry point
 *  - Pointers named in a signature are DEVICE pointers unless marked "host". The caller owns every
 *    buffer; the library allocates nothing and keeps no state apart from per-device caches (device
 *    properties, kernel attributes, the scratch address of rom_route_noalloc), each filled once per device,
 *    thread-safely. Tensors are dense, row-major, and 16-byte aligned.
 *  - Calls enqueue kernels on `stream` (a hipStream_t; NULL is the null stream) and return without
 *    synchronising. The projections read what rom_route wrote: run them on the same stream, or
 *    order them after it. No count is ever read back to the host.
 *  - Arguments are validated before anything is enqueued; on a non-OK return nothing was enqueued,
 *    except for ROM_ERR_HIP, which reports a failed launch. rom_last_error() gives details.
 *  - T == 0 is a valid no-op (ROM_OK, nothing enqueued, no buffer touched).
 *  - Supported range: 1 <= E <= ROM_MAX_EXPERTS, 1 <= top_k <= min(E, ROM_MAX_TOP_K), d_model and
 *    d_inner multiples of 64 and at most ROM_MAX_DIM, T <= ROM_MAX_TOKENS. dtype is the storage type of X, the expert stacks, z, h and all outputs;
 *    the router weight and bias are always fp32. bf16 data is accumulated in fp32 on MFMA; fp32
 *    data is computed in fp32 throughout.
 *  - Expert matrices are stored transposed relative to the page's x_t W notation, as [out][in]
 *    (K-contiguous, the nn.Linear layout): W_conv[e] is the page's W_in,e transposed.
 *  - Results are deterministic: no floating-point atomics; the grouping is a stable counting sort.
 */
#ifndef ROM_H
#define ROM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ROM_ABI_VERSION 8
#ifndef ROM_API
#define ROM_API __attribute__((visibility("default")))
#endif
#define ROM_MAX_EXPERTS 64
#define ROM_MAX_TOP_K 2
#define ROM_MAX_TOKENS (1 << 24)
#define ROM_MAX_DIM 65536     /* largest d_model, d_inner, d_out or channel count */
#define ROM_MAX_CONV_WIDTH 8
#define ROM_NOALLOC_SCRATCH_BYTES (4u << 20)  /* static router scratch of rom_route_noalloc, per device */

typedef enum {
    ROM_OK = 0,
    ROM_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative or inconsistent size, misalignment */
    ROM_ERR_UNSUPPORTED = 2,        /* valid but outside the supported range (top_k > 2, E > 64, ...) */
    ROM_ERR_WORKSPACE_TOO_SMALL = 3,
    ROM_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} rom_status;

typedef enum { ROM_DTYPE_F32 = 0, ROM_DTYPE_BF16 = 1 } rom_dtype;

typedef enum { ROM_ACT_NONE = 0, ROM_ACT_SILU = 1 } rom_activation;

/*
 * The routing decision of one block for T tokens (Knowl 1: S_t and r_t,i), plus the grouping that the
 * grouped projections use. A host struct of caller-owned DEVICE buffers: rom_route fills the buffers
 * and stamps T, E and top_k; rom_in_proj and rom_out_proj read them.
 *
 * With top_k = K the buffers hold K stacked top-1 routings, choice k = 0 .. K-1 (k = 0 the largest
 * logit, k = 1 the second largest): each array below is K times the size shown, slice k at offset
 * k * (size shown). Slice k groups the tokens by their k-th choice on its own.
 */
typedef struct rom_routing {
    int32_t T, E, top_k;     /* stamped by rom_route; checked by the projections */
    int32_t reserved;        /* zero */
    int32_t *expert_id;      /* [K][T]   choice k of token t; ties keep the lowest index */
    float *prob;             /* [K][T]   p_t,e of that expert: the full softmax over E experts, not renormalised */
    int32_t *counts;         /* [K][E]   tokens whose choice k is each expert (sum over e = T) */
    int32_t *offsets;        /* [K][E+1] exclusive prefix sum of counts; offsets[k][E] = T */
    int32_t *perm;           /* [K][T]   slot -> token: expert-major, ascending token id within an expert */
    int32_t *inv_perm;       /* [K][T]   token -> slot (perm[k][inv_perm[k][t]] == t) */
} rom_routing;

/* ROM_ABI_VERSION of the loaded library. */
ROM_API int rom_abi_version(void);

/* Bytes of device workspace rom_route needs for T tokens and E experts, for any top_k (0 when T == 0). */
ROM_API size_t rom_route_workspace_bytes(int32_t T, int32_t E);

/*
 * Router, histogram, stable counting sort and (optionally) permute.
 * Knowl 1's router: logit_t,j = sum_k X[t][k] * W_router[k][j] (+ bias[j]) in fp32 (bf16 X is
 * widened exactly); choice 0 = argmax_j logit_t,j with the lowest index on ties, choice 1 (top_k = 2)
 * = the argmax over the other experts, again lowest index on ties; the probability of expert e is
 * exp(logit_t,e - logit_t,max) / sum_j exp(logit_t,j - logit_t,max). The grouping of each choice k
 * (not on the page; a dropless grouped computation needs it, Knowl 12): counts, offsets, and slot
 * pos(t) = offsets[e_t] + #{t' < t : e_t' = e_t}, written as perm[pos(t)] = t, inv_perm[t] = pos(t).
 *
 *   X         [T][d_model], x_dtype
 *   W_router  [d_model][E] fp32;  bias [E] fp32 or NULL (a workload device; the page has none)
 *   top_k     1 or 2 (at most E)
 *   routing   host pointer to a struct whose six device buffers are sized as documented above
 *   X_perm    NULL, or [T][d_model] x_dtype: receives X_perm[pos] = X[perm[pos]] (the permute;
 *             top_k = 1 only)
 *   workspace device scratch of at least rom_route_workspace_bytes(T, E) bytes; its contents on
 *             entry do not matter and are clobbered
 */
ROM_API rom_status rom_route(const void *X, rom_dtype x_dtype, int32_t T, int32_t d_model,
                     const float *W_router, const float *bias, int32_t E, int32_t top_k,
                     rom_routing *routing, void *X_perm, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * rom_route for callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same arguments, kernels and results (bit for bit) as rom_route,
 * without the workspace: the router's partial histograms live in a static device array of
 * ROM_NOALLOC_SCRATCH_BYTES that the library owns (each GPU the library runs on holds its own copy until the
 * process ends). The call allocates nothing. It returns ROM_ERR_UNSUPPORTED when
 * rom_route_workspace_bytes(T, E) exceeds ROM_NOALLOC_SCRATCH_BYTES (e.g. E = 8 beyond about 500K tokens).
 * Every call on one GPU shares that GPU's array and nothing in it needs to start at zero: calls that overlap
 * in time on one GPU (on different streams, or from host threads without ordering between them) race on it
 * and give undefined results, so order them (one stream, or events).
 */
ROM_API rom_status rom_route_noalloc(const void *X, rom_dtype x_dtype, int32_t T, int32_t d_model,
                             const float *W_router, const float *bias, int32_t E, int32_t top_k,
                             rom_routing *routing, void *X_perm, void *stream);

/*
 * In-projection experts (Knowl 1, H_t and the argument of SiLU in G_t): for every token t,
 *   x_out[t][n] = sum_{e in S_t} sum_k X[t][k] * W_conv[e][n][k]   (z_out likewise with W_gate)
 * with no probability scale (the indicator only). Computed as one ragged grouped GEMM per choice k
 * over the expert groups of slice k of `routing`; the choices are added in the order k = 0, 1, the
 * first rounded to dtype before the second is added. Outputs are in token order. z_out is the
 * pre-activation gate: SiLU is applied by rom_out_proj.
 *   X [T][d_model]; W_conv, W_gate [E][d_inner][d_model]; x_out, z_out [T][d_inner]; all dtype.
 *   X may not alias an output; x_out and z_out may not overlap.
 */
ROM_API rom_status rom_in_proj(const void *X, const rom_routing *routing, rom_dtype dtype, int32_t T,
                       int32_t d_model, int32_t d_inner, const void *W_conv, const void *W_gate,
                       void *x_out, void *z_out, void *stream);

/*
 * Routing-weighted in-projection of Switch Mamba (Swimba project page, extended abstract): expert
 * in-projections behind a token-level softmax router, whose output streams are each weighted by the
 * routing weight and summed into the single input of the (unchanged) SSM kernel. The routing weight is
 * the router probability p_t,e of a selected expert, as in r_t,i above (not renormalised):
 *   y_out[t][n] = sum_{e in S_t} p_t,e * sum_k X[t][k] * W_in[e][n][k]
 * The same grouped products as rom_out_proj, applied to X with no gate; accumulation is fp32 (MFMA for
 * bf16 data), each choice's contribution is rounded once, and the choices are added in the order
 * k = 0, 1 as for rom_in_proj. Output in token order. Swimba routes 4 experts, top-1 per token.
 *   X [T][d_model]; W_in [E][d_out][d_model]; y_out [T][d_out]; all dtype; d_out a multiple of 64.
 *   X may not alias y_out.
 */
ROM_API rom_status rom_in_proj_weighted(const void *X, const rom_routing *routing, rom_dtype dtype, int32_t T,
                                int32_t d_model, int32_t d_out, const void *W_in, void *y_out, void *stream);

/*
 * The shared short causal convolution between the in-projection and the selective SSM (Knowl 1: the
 * short convolution applied to H_t; Knowl 9: shared across experts, not expertized). The page fixes no
 * width, bias or activation; this call takes a depthwise causal convolution of each sequence:
 *   u[b][t][c] = bias[c] + sum_{j<width} weight[c][j] * x[b][t - (width-1) + j][c]
 *   y[b][t][c] = activation == ROM_ACT_SILU ? SiLU(u) : u
 * with x at times before a sequence's first token taken as zero (sequences never mix), so
 * weight[c][width-1] multiplies the current token. Accumulation is fp32 in the order bias, oldest tap
 * first; y is rounded once to dtype.
 *   x, y      [n_seq][seq_len][channels] dtype, token order (x is rom_in_proj's x_out when
 *             n_seq * seq_len = T); y may not overlap x
 *   weight    [channels][width] dtype;  bias [channels] dtype or NULL (16-byte aligned)
 *   width     1 .. ROM_MAX_CONV_WIDTH;  channels a multiple of 64;  activation ROM_ACT_NONE or ROM_ACT_SILU
 * n_seq * seq_len == 0 is a no-op.
 */
ROM_API rom_status rom_conv1d(const void *x, rom_dtype dtype, int32_t n_seq, int32_t seq_len, int32_t channels,
                      const void *weight, const void *bias, int32_t width, int32_t activation, void *y,
                      void *stream);

/*
 * Backward of the routed projections: the exact derivatives of Knowl 1's H_t, G_t and O_t (the
 * forward entry points above) with the router probabilities held fixed, for bf16 data (fp32
 * accumulation). The gradient that reaches the router through p_t,e or through the selection S_t is
 * not computed (the page's training recipe handles the router separately). Weight gradients are
 * written (not accumulated) in fp32, in the weights' [E][out][in] layout; an expert that received no
 * token gets zeros. Both calls need a caller-provided device workspace of at least
 * rom_backward_workspace_bytes(T, d_model, d_inner, E, top_k) bytes, 256-byte aligned, whose contents
 * on entry do not matter (the transposed weight stacks and token-contiguous copies of the operands
 * are built there). Outputs may not overlap the inputs, the workspace or each other.
 */
ROM_API size_t rom_backward_workspace_bytes(int32_t T, int32_t d_model, int32_t d_inner, int32_t E, int32_t top_k);

/*
 * Out-projection backward. With g = d_out (dL/dout [T][d_model]) and a = SiLU(z) * h:
 *   da[t]     = sum_{e in S_t} p_t,e * W_out[e]^T g[t]            (accumulated in fp32, rounded to bf16)
 *   dz[t][n]  = da[t][n] * h[t][n] * SiLU'(z[t][n]),  SiLU'(v) = s (1 + v (1 - s)), s = sigmoid(v)
 *   dh[t][n]  = da[t][n] * SiLU(z[t][n])
 *   dW_out[e] = sum over the tokens t with e in S_t of p_t,e * g[t] a[t]^T   (a rounded to bf16, as in
 *               the forward)
 *   d_out [T][d_model], z, h, dz, dh [T][d_inner], W_out [E][d_model][d_inner] bf16; dW_out
 *   [E][d_model][d_inner] fp32.
 */
ROM_API rom_status rom_out_proj_backward(const void *d_out, const void *z, const void *h, const rom_routing *routing,
                                 rom_dtype dtype, int32_t T, int32_t d_model, int32_t d_inner, const void *W_out,
                                 void *dz, void *dh, float *dW_out, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * In-projection backward. With dx = dL/dx_out and dz = dL/dz_out (the pre-activation gate, as
 * rom_out_proj_backward returns it):
 *   dX[t]      = sum_{e in S_t} (W_conv[e]^T dx[t] + W_gate[e]^T dz[t])   (one fp32 sum per choice; the
 *                choices are added in the order k = 0, 1 as in the forward)
 *   dW_conv[e] = sum over the tokens t with e in S_t of dx[t] X[t]^T;  dW_gate[e] likewise with dz
 *   X, dX [T][d_model], dx, dz [T][d_inner], W_conv, W_gate [E][d_inner][d_model] bf16; dW_conv,
 *   dW_gate [E][d_inner][d_model] fp32.
 */
ROM_API rom_status rom_in_proj_backward(const void *X, const void *dx, const void *dz, const rom_routing *routing,
                                rom_dtype dtype, int32_t T, int32_t d_model, int32_t d_inner, const void *W_conv,
                                const void *W_gate, void *dX, float *dW_conv, float *dW_gate, void *workspace,
                                size_t workspace_bytes, void *stream);

/* Bytes of device workspace rom_out_proj needs (T * d_inner bf16 values for bf16 data; 0 for fp32 data). */
ROM_API size_t rom_out_proj_workspace_bytes(int32_t T, int32_t d_inner, rom_dtype dtype);

/*
 * Out-projection experts (Knowl 1, O_t), with h standing in for the SSM-core output Y_t:
 *   a[t][n]   = SiLU(z[t][n]) * h[t][n],  SiLU(v) = v / (1 + exp(-v)), in fp32
 *   out[t][m] = sum_{e in S_t} p_t,e * sum_n a[t][n] * W_out[e][m][n]
 * The probability scale is r_t,e of Knowl 1 (stated only in that secondary summary: the authors'
 * own text does not write the formula). For bf16 data, a is rounded to bf16 once before the
 * MFMA product; accumulation is fp32; each choice's contribution is rounded once, added in the order
 * k = 0, 1 as for the in-projection. For bf16 data the gated rows a are first written to the workspace
 * (in slot order for top_k = 1 and T > 64, otherwise in token order), which the grouped products read.
 *   z, h [T][d_inner]; W_out [E][d_model][d_inner]; out [T][d_model]; all dtype. out may not alias z or h.
 *   workspace  device scratch of at least rom_out_proj_workspace_bytes(T, d_inner, dtype) bytes
 *              (may be NULL when that is 0); contents on entry do not matter and are clobbered.
 */
ROM_API rom_status rom_out_proj(const void *z, const void *h, const rom_routing *routing, rom_dtype dtype,
                        int32_t T, int32_t d_model, int32_t d_inner, const void *W_out, void *out,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Static description of a status code. */
ROM_API const char *rom_status_string(rom_status s);

/* Detail of the last non-OK return on the calling thread ("" if none). */
ROM_API const char *rom_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ROM_H */
