// rom_api.hip -- the C ABI of librom (declared in include/rom.h): argument validation, status codes,
// and dispatch to the gfx950 kernels. Every check runs before the first HIP call, so invalid
// arguments enqueue nothing and need no GPU.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "rom.h"
#include "rom_internal.h"

namespace {

thread_local char g_last_error[512] = "";

rom_status fail(rom_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

rom_status hip_fail(hipError_t err, const char *what) {
    return fail(ROM_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(err), (int)err);
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_size(rom_dtype dt) { return dt == ROM_DTYPE_BF16 ? 2 : 4; }

bool overlap(const void *a, size_t an, const void *b, size_t bn) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bn && y < x + an;
}

#define ROM_CHECK_PTR(p, align)                                                                      \
    do {                                                                                             \
        if ((p) == nullptr) return fail(ROM_ERR_INVALID_ARGUMENT, "%s is NULL", #p);                 \
        if (!aligned((p), (align)))                                                                  \
            return fail(ROM_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", #p, (int)(align));    \
    } while (0)

rom_status check_dims(int32_t T, int32_t d, const char *dname) {
    if (T < 0) return fail(ROM_ERR_INVALID_ARGUMENT, "T = %d is negative", T);
    if (T > ROM_MAX_TOKENS) return fail(ROM_ERR_UNSUPPORTED, "T = %d exceeds ROM_MAX_TOKENS", T);
    if (d <= 0) return fail(ROM_ERR_INVALID_ARGUMENT, "%s = %d must be positive", dname, d);
    if (d % 64 != 0) return fail(ROM_ERR_UNSUPPORTED, "%s = %d is not a multiple of 64", dname, d);
    if (d > ROM_MAX_DIM) return fail(ROM_ERR_UNSUPPORTED, "%s = %d exceeds ROM_MAX_DIM (%d)", dname, d, ROM_MAX_DIM);
    return ROM_OK;
}

rom_status check_dtype(int dt) {
    if (dt != ROM_DTYPE_F32 && dt != ROM_DTYPE_BF16) return fail(ROM_ERR_INVALID_ARGUMENT, "unknown dtype %d", dt);
    return ROM_OK;
}

rom_status check_experts(int32_t E, int32_t top_k) {
    if (E < 1) return fail(ROM_ERR_INVALID_ARGUMENT, "E = %d must be at least 1", E);
    if (E > ROM_MAX_EXPERTS) return fail(ROM_ERR_UNSUPPORTED, "E = %d exceeds ROM_MAX_EXPERTS (%d)", E, ROM_MAX_EXPERTS);
    if (top_k < 1 || top_k > E) return fail(ROM_ERR_INVALID_ARGUMENT, "top_k = %d outside [1, E]", top_k);
    if (top_k > ROM_MAX_TOP_K)
        return fail(ROM_ERR_UNSUPPORTED, "top_k = %d exceeds ROM_MAX_TOP_K (%d)", top_k, ROM_MAX_TOP_K);
    return ROM_OK;
}

// The projections' view of a routing struct filled by rom_route.
rom_status check_routing_for_proj(const rom_routing *r, int32_t T) {
    if (r == nullptr) return fail(ROM_ERR_INVALID_ARGUMENT, "routing is NULL");
    if (r->T != T) return fail(ROM_ERR_INVALID_ARGUMENT, "routing->T = %d but T = %d", r->T, T);
    rom_status s = check_experts(r->E, r->top_k);
    if (s != ROM_OK) return s;
    if (T > 0) {
        ROM_CHECK_PTR(r->offsets, 4);
        ROM_CHECK_PTR(r->perm, 4);
        ROM_CHECK_PTR(r->prob, 4);
    }
    return ROM_OK;
}

rom_status check_bwd_common(rom_dtype dtype, const rom_routing *routing, int32_t T, int32_t d_model, int32_t d_inner,
                            void *workspace, size_t workspace_bytes) {
    rom_status s;
    if ((s = check_dtype(dtype)) != ROM_OK) return s;
    if (dtype != ROM_DTYPE_BF16) return fail(ROM_ERR_UNSUPPORTED, "the backward supports bf16 data only");
    if ((s = check_dims(T, d_model, "d_model")) != ROM_OK) return s;
    if ((s = check_dims(T, d_inner, "d_inner")) != ROM_OK) return s;
    if ((s = check_routing_for_proj(routing, T)) != ROM_OK) return s;
    if (T == 0) return ROM_OK;
    const size_t need = rom::backward_workspace_bytes(T, d_model, d_inner, routing->E, routing->top_k);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(ROM_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed",
                    workspace == nullptr ? (size_t)0 : workspace_bytes, need);
    if (!aligned(workspace, 256)) return fail(ROM_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    return ROM_OK;
}

}  // namespace

extern "C" {

int rom_abi_version(void) { return ROM_ABI_VERSION; }

size_t rom_route_workspace_bytes(int32_t T, int32_t E) {
    if (T <= 0 || E <= 0) return 0;
    const size_t b = rom::route_workspace_words(T, E) * sizeof(int32_t);
    return (b + 255) & ~(size_t)255;
}

}  // extern "C"

namespace {

// Validation shared by rom_route and rom_route_noalloc (workspace checks excluded).
rom_status check_route_args(const void *X, rom_dtype x_dtype, int32_t T, int32_t d_model, const float *W_router,
                            const float *bias, int32_t E, int32_t top_k, rom_routing *routing, void *X_perm) {
    rom_status s;
    if ((s = check_dtype(x_dtype)) != ROM_OK) return s;
    if ((s = check_dims(T, d_model, "d_model")) != ROM_OK) return s;
    if ((s = check_experts(E, top_k)) != ROM_OK) return s;
    if (routing == nullptr) return fail(ROM_ERR_INVALID_ARGUMENT, "routing is NULL");
    if (T == 0) return ROM_OK;
    ROM_CHECK_PTR(X, 16);
    ROM_CHECK_PTR(W_router, 16);
    if (bias != nullptr && !aligned(bias, 4)) return fail(ROM_ERR_INVALID_ARGUMENT, "bias is not 4-byte aligned");
    ROM_CHECK_PTR(routing->expert_id, 4);
    ROM_CHECK_PTR(routing->prob, 4);
    ROM_CHECK_PTR(routing->counts, 4);
    ROM_CHECK_PTR(routing->offsets, 4);
    ROM_CHECK_PTR(routing->perm, 4);
    ROM_CHECK_PTR(routing->inv_perm, 4);
    if (X_perm != nullptr) {
        if (top_k != 1) return fail(ROM_ERR_UNSUPPORTED, "X_perm (the materialised permute) needs top_k == 1");
        if (!aligned(X_perm, 16)) return fail(ROM_ERR_INVALID_ARGUMENT, "X_perm is not 16-byte aligned");
        const size_t xb = (size_t)T * d_model * elem_size(x_dtype);
        if (overlap(X, xb, X_perm, xb)) return fail(ROM_ERR_INVALID_ARGUMENT, "X_perm overlaps X");
    }
    return ROM_OK;
}

rom_status route_enqueue(const void *X, rom_dtype x_dtype, int32_t T, int32_t d_model, const float *W_router,
                         const float *bias, int32_t E, int32_t top_k, rom_routing *routing, void *X_perm,
                         int32_t *workspace, void *stream, const char *what) {
    routing->T = T;
    routing->E = E;
    routing->top_k = top_k;
    routing->reserved = 0;
    hipError_t err = rom::launch_route(X, x_dtype, T, d_model, W_router, bias, E, *routing, X_perm, workspace,
                                       static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, what);
    return ROM_OK;
}

}  // namespace

// ---- the scratch of rom_route_noalloc: a library-owned static device array (each device that loads the
// library holds its own copy until the process ends). Host code never uses the array's name as an address:
// its device address is taken once per device with hipGetSymbolAddress, with that device current.
static __device__ __align__(256) int32_t scratch[ROM_NOALLOC_SCRATCH_BYTES / sizeof(int32_t)];

namespace {

std::once_flag g_scratch_once[rom::kMaxDevices];
int32_t *g_scratch_ptr[rom::kMaxDevices];
hipError_t g_scratch_err[rom::kMaxDevices];

// Device address of the current device's scratch array.
hipError_t scratch_address(int32_t **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= rom::kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [&] {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = static_cast<int32_t *>(p);
    });
    if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
    if (g_scratch_ptr[dev] == nullptr) return hipErrorInvalidSymbol;
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

rom_status rom_route_noalloc(const void *X, rom_dtype x_dtype, int32_t T, int32_t d_model, const float *W_router,
                             const float *bias, int32_t E, int32_t top_k, rom_routing *routing, void *X_perm,
                             void *stream) {
    g_last_error[0] = '\0';
    rom_status s = check_route_args(X, x_dtype, T, d_model, W_router, bias, E, top_k, routing, X_perm);
    if (s != ROM_OK) return s;
    if (T == 0) {
        routing->T = 0;
        routing->E = E;
        routing->top_k = top_k;
        return ROM_OK;
    }
    const size_t need = rom_route_workspace_bytes(T, E);
    if (need > ROM_NOALLOC_SCRATCH_BYTES)
        return fail(ROM_ERR_UNSUPPORTED, "T = %d, E = %d need %zu bytes of router scratch; the static scratch of "
                    "rom_route_noalloc holds %zu (use rom_route with a workspace)", T, E, need,
                    (size_t)ROM_NOALLOC_SCRATCH_BYTES);
    int32_t *ws = nullptr;
    hipError_t err = scratch_address(&ws);
    if (err != hipSuccess) return hip_fail(err, "rom_route_noalloc scratch address");
    return route_enqueue(X, x_dtype, T, d_model, W_router, bias, E, top_k, routing, X_perm, ws, stream,
                         "rom_route_noalloc launch");
}

rom_status rom_route(const void *X, rom_dtype x_dtype, int32_t T, int32_t d_model, const float *W_router,
                     const float *bias, int32_t E, int32_t top_k, rom_routing *routing, void *X_perm,
                     void *workspace, size_t workspace_bytes, void *stream) {
    g_last_error[0] = '\0';
    rom_status s = check_route_args(X, x_dtype, T, d_model, W_router, bias, E, top_k, routing, X_perm);
    if (s != ROM_OK) return s;
    if (T == 0) {
        routing->T = 0;
        routing->E = E;
        routing->top_k = top_k;
        return ROM_OK;
    }
    const size_t need = rom_route_workspace_bytes(T, E);
    if (T > rom::kRouteSmallT) {
        if (workspace == nullptr) return fail(ROM_ERR_WORKSPACE_TOO_SMALL, "workspace is NULL (%zu bytes needed)", need);
        if (!aligned(workspace, 4)) return fail(ROM_ERR_INVALID_ARGUMENT, "workspace is not 4-byte aligned");
    }
    if (workspace_bytes < need && T > rom::kRouteSmallT)
        return fail(ROM_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    return route_enqueue(X, x_dtype, T, d_model, W_router, bias, E, top_k, routing, X_perm,
                         static_cast<int32_t *>(workspace), stream, "rom_route launch");
}

rom_status rom_in_proj(const void *X, const rom_routing *routing, rom_dtype dtype, int32_t T, int32_t d_model,
                       int32_t d_inner, const void *W_conv, const void *W_gate, void *x_out, void *z_out,
                       void *stream) {
    g_last_error[0] = '\0';
    rom_status s;
    if ((s = check_dtype(dtype)) != ROM_OK) return s;
    if ((s = check_dims(T, d_model, "d_model")) != ROM_OK) return s;
    if ((s = check_dims(T, d_inner, "d_inner")) != ROM_OK) return s;
    if ((s = check_routing_for_proj(routing, T)) != ROM_OK) return s;
    if (T == 0) return ROM_OK;
    ROM_CHECK_PTR(X, 16);
    ROM_CHECK_PTR(W_conv, 16);
    ROM_CHECK_PTR(W_gate, 16);
    ROM_CHECK_PTR(x_out, 16);
    ROM_CHECK_PTR(z_out, 16);
    const size_t es = elem_size(dtype);
    const size_t xb = (size_t)T * d_model * es, ob = (size_t)T * d_inner * es;
    if (overlap(x_out, ob, z_out, ob)) return fail(ROM_ERR_INVALID_ARGUMENT, "x_out and z_out overlap");
    if (overlap(X, xb, x_out, ob) || overlap(X, xb, z_out, ob))
        return fail(ROM_ERR_INVALID_ARGUMENT, "X overlaps an output");
    hipError_t err = rom::launch_in_proj(X, *routing, dtype, T, d_model, d_inner, W_conv, W_gate, x_out, z_out,
                                         static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, "rom_in_proj launch");
    return ROM_OK;
}

rom_status rom_in_proj_weighted(const void *X, const rom_routing *routing, rom_dtype dtype, int32_t T,
                                int32_t d_model, int32_t d_out, const void *W_in, void *y_out, void *stream) {
    g_last_error[0] = '\0';
    rom_status s;
    if ((s = check_dtype(dtype)) != ROM_OK) return s;
    if ((s = check_dims(T, d_model, "d_model")) != ROM_OK) return s;
    if ((s = check_dims(T, d_out, "d_out")) != ROM_OK) return s;
    if ((s = check_routing_for_proj(routing, T)) != ROM_OK) return s;
    if (T == 0) return ROM_OK;
    ROM_CHECK_PTR(X, 16);
    ROM_CHECK_PTR(W_in, 16);
    ROM_CHECK_PTR(y_out, 16);
    const size_t es = elem_size(dtype);
    if (overlap(X, (size_t)T * d_model * es, y_out, (size_t)T * d_out * es))
        return fail(ROM_ERR_INVALID_ARGUMENT, "X overlaps y_out");
    hipError_t err = rom::launch_in_proj_weighted(X, *routing, dtype, T, d_model, d_out, W_in, y_out,
                                                  static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, "rom_in_proj_weighted launch");
    return ROM_OK;
}

rom_status rom_conv1d(const void *x, rom_dtype dtype, int32_t n_seq, int32_t seq_len, int32_t channels,
                      const void *weight, const void *bias, int32_t width, int32_t activation, void *y,
                      void *stream) {
    g_last_error[0] = '\0';
    rom_status s;
    if ((s = check_dtype(dtype)) != ROM_OK) return s;
    if (n_seq < 0 || seq_len < 0) return fail(ROM_ERR_INVALID_ARGUMENT, "n_seq = %d, seq_len = %d", n_seq, seq_len);
    if ((int64_t)n_seq * seq_len > ROM_MAX_TOKENS)
        return fail(ROM_ERR_UNSUPPORTED, "n_seq * seq_len exceeds ROM_MAX_TOKENS");
    if ((s = check_dims(0, channels, "channels")) != ROM_OK) return s;
    if (width < 1 || width > ROM_MAX_CONV_WIDTH)
        return fail(width < 1 ? ROM_ERR_INVALID_ARGUMENT : ROM_ERR_UNSUPPORTED, "width = %d outside [1, %d]", width,
                    ROM_MAX_CONV_WIDTH);
    if (activation != ROM_ACT_NONE && activation != ROM_ACT_SILU)
        return fail(ROM_ERR_INVALID_ARGUMENT, "unknown activation %d", activation);
    if ((int64_t)n_seq * seq_len == 0) return ROM_OK;
    ROM_CHECK_PTR(x, 16);
    ROM_CHECK_PTR(weight, 16);
    ROM_CHECK_PTR(y, 16);
    if (bias != nullptr && !aligned(bias, 16)) return fail(ROM_ERR_INVALID_ARGUMENT, "bias is not 16-byte aligned");
    const size_t xb = (size_t)n_seq * seq_len * channels * elem_size(dtype);
    if (overlap(x, xb, y, xb)) return fail(ROM_ERR_INVALID_ARGUMENT, "y overlaps x");
    hipError_t err = rom::launch_conv1d(x, dtype, n_seq, seq_len, channels, weight, bias, width, activation, y,
                                        static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, "rom_conv1d launch");
    return ROM_OK;
}

size_t rom_backward_workspace_bytes(int32_t T, int32_t d_model, int32_t d_inner, int32_t E, int32_t top_k) {
    if (T <= 0 || d_model <= 0 || d_inner <= 0 || E < 1 || E > ROM_MAX_EXPERTS || top_k < 1 || top_k > ROM_MAX_TOP_K)
        return 0;
    return rom::backward_workspace_bytes(T, d_model, d_inner, E, top_k);
}


rom_status rom_out_proj_backward(const void *d_out, const void *z, const void *h, const rom_routing *routing,
                                 rom_dtype dtype, int32_t T, int32_t d_model, int32_t d_inner, const void *W_out,
                                 void *dz, void *dh, float *dW_out, void *workspace, size_t workspace_bytes,
                                 void *stream) {
    g_last_error[0] = '\0';
    rom_status s = check_bwd_common(dtype, routing, T, d_model, d_inner, workspace, workspace_bytes);
    if (s != ROM_OK || T == 0) return s;
    ROM_CHECK_PTR(d_out, 16);
    ROM_CHECK_PTR(z, 16);
    ROM_CHECK_PTR(h, 16);
    ROM_CHECK_PTR(W_out, 16);
    ROM_CHECK_PTR(dz, 16);
    ROM_CHECK_PTR(dh, 16);
    ROM_CHECK_PTR(dW_out, 16);
    const size_t ib = (size_t)T * d_inner * 2, gb = (size_t)T * d_model * 2;
    const size_t wb = (size_t)routing->E * d_model * d_inner * 4;
    const size_t need = rom::backward_workspace_bytes(T, d_model, d_inner, routing->E, routing->top_k);
    const void *ins[4] = {d_out, z, h, workspace};
    const size_t insb[4] = {gb, ib, ib, need};
    void *outs[3] = {dz, dh, dW_out};
    const size_t outsb[3] = {ib, ib, wb};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 4; ++i)
            if (overlap(outs[o], outsb[o], ins[i], insb[i]))
                return fail(ROM_ERR_INVALID_ARGUMENT, "an output overlaps an input or the workspace");
        for (int q = o + 1; q < 3; ++q)
            if (overlap(outs[o], outsb[o], outs[q], outsb[q])) return fail(ROM_ERR_INVALID_ARGUMENT, "outputs overlap");
    }
    hipError_t err = rom::launch_out_proj_backward(d_out, z, h, *routing, T, d_model, d_inner, W_out, dz, dh, dW_out,
                                                   workspace, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, "rom_out_proj_backward launch");
    return ROM_OK;
}

rom_status rom_in_proj_backward(const void *X, const void *dx, const void *dz, const rom_routing *routing,
                                rom_dtype dtype, int32_t T, int32_t d_model, int32_t d_inner, const void *W_conv,
                                const void *W_gate, void *dX, float *dW_conv, float *dW_gate, void *workspace,
                                size_t workspace_bytes, void *stream) {
    g_last_error[0] = '\0';
    rom_status s = check_bwd_common(dtype, routing, T, d_model, d_inner, workspace, workspace_bytes);
    if (s != ROM_OK || T == 0) return s;
    ROM_CHECK_PTR(X, 16);
    ROM_CHECK_PTR(dx, 16);
    ROM_CHECK_PTR(dz, 16);
    ROM_CHECK_PTR(W_conv, 16);
    ROM_CHECK_PTR(W_gate, 16);
    ROM_CHECK_PTR(dX, 16);
    ROM_CHECK_PTR(dW_conv, 16);
    ROM_CHECK_PTR(dW_gate, 16);
    const size_t xb = (size_t)T * d_model * 2, ib = (size_t)T * d_inner * 2;
    const size_t wb = (size_t)routing->E * d_model * d_inner * 4;
    const size_t need = rom::backward_workspace_bytes(T, d_model, d_inner, routing->E, routing->top_k);
    const void *ins[4] = {X, dx, dz, workspace};
    const size_t insb[4] = {xb, ib, ib, need};
    void *outs[3] = {dX, dW_conv, dW_gate};
    const size_t outsb[3] = {xb, wb, wb};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 4; ++i)
            if (overlap(outs[o], outsb[o], ins[i], insb[i]))
                return fail(ROM_ERR_INVALID_ARGUMENT, "an output overlaps an input or the workspace");
        for (int q = o + 1; q < 3; ++q)
            if (overlap(outs[o], outsb[o], outs[q], outsb[q])) return fail(ROM_ERR_INVALID_ARGUMENT, "outputs overlap");
    }
    hipError_t err = rom::launch_in_proj_backward(X, dx, dz, *routing, T, d_model, d_inner, W_conv, W_gate, dX,
                                                  dW_conv, dW_gate, workspace, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, "rom_in_proj_backward launch");
    return ROM_OK;
}

size_t rom_out_proj_workspace_bytes(int32_t T, int32_t d_inner, rom_dtype dtype) {
    if (T <= 0 || d_inner <= 0 || (dtype != ROM_DTYPE_F32 && dtype != ROM_DTYPE_BF16)) return 0;
    return rom::out_proj_workspace_bytes(T, d_inner, dtype);
}

rom_status rom_out_proj(const void *z, const void *h, const rom_routing *routing, rom_dtype dtype, int32_t T,
                        int32_t d_model, int32_t d_inner, const void *W_out, void *out, void *workspace,
                        size_t workspace_bytes, void *stream) {
    g_last_error[0] = '\0';
    rom_status s;
    if ((s = check_dtype(dtype)) != ROM_OK) return s;
    if ((s = check_dims(T, d_model, "d_model")) != ROM_OK) return s;
    if ((s = check_dims(T, d_inner, "d_inner")) != ROM_OK) return s;
    if ((s = check_routing_for_proj(routing, T)) != ROM_OK) return s;
    if (T == 0) return ROM_OK;
    ROM_CHECK_PTR(z, 16);
    ROM_CHECK_PTR(h, 16);
    ROM_CHECK_PTR(W_out, 16);
    ROM_CHECK_PTR(out, 16);
    const size_t es = elem_size(dtype);
    const size_t ib = (size_t)T * d_inner * es, ob = (size_t)T * d_model * es;
    if (overlap(out, ob, z, ib) || overlap(out, ob, h, ib))
        return fail(ROM_ERR_INVALID_ARGUMENT, "out overlaps z or h");
    const size_t need = rom::out_proj_workspace_bytes(T, d_inner, dtype);
    if (need > 0) {
        if (workspace == nullptr || workspace_bytes < need)
            return fail(ROM_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed",
                        workspace == nullptr ? (size_t)0 : workspace_bytes, need);
        if (!aligned(workspace, 16)) return fail(ROM_ERR_INVALID_ARGUMENT, "workspace is not 16-byte aligned");
        if (overlap(workspace, need, z, ib) || overlap(workspace, need, h, ib) || overlap(workspace, need, out, ob))
            return fail(ROM_ERR_INVALID_ARGUMENT, "workspace overlaps z, h or out");
    }
    hipError_t err = rom::launch_out_proj(z, h, *routing, dtype, T, d_model, d_inner, W_out, out, workspace,
                                          static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, "rom_out_proj launch");
    return ROM_OK;
}

const char *rom_status_string(rom_status s) {
    switch (s) {
        case ROM_OK: return "ROM_OK";
        case ROM_ERR_INVALID_ARGUMENT: return "ROM_ERR_INVALID_ARGUMENT";
        case ROM_ERR_UNSUPPORTED: return "ROM_ERR_UNSUPPORTED";
        case ROM_ERR_WORKSPACE_TOO_SMALL: return "ROM_ERR_WORKSPACE_TOO_SMALL";
        case ROM_ERR_HIP: return "ROM_ERR_HIP";
    }
    return "unknown rom_status";
}

const char *rom_last_error(void) { return g_last_error; }

}  // extern "C"
