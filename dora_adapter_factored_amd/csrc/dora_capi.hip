// C ABI of the DoRA hot path: host-side validation, workspace queries and
// dispatch to the kernel launchers.  Nothing is enqueued unless every argument
// checks out; errors carry a thread-local detail string.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "../../include/dora.h"
#include "dora_launch.h"

namespace {

thread_local char g_detail[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_detail[0] = '\0';
    return DORA_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(DORA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

constexpr int64_t kMaxDim = (int64_t)1 << 31;

bool dim_ok(int64_t v, int64_t lo) { return v >= lo && v < kMaxDim; }
bool dtype_ok(int dt) { return dt == DORA_F32 || dt == DORA_BF16 || dt == DORA_F16; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255) == 0; }

// the transpose of A runs one grid row per 64 values of r
constexpr int64_t kMaxMergeRank = (int64_t)65535 * 64 - 64;

int check_norm_args(const void* W0, const void* A, const void* B, const float* m, int64_t d_out, int64_t d_in,
                    int64_t r, int dtype, float s, float eps, const float* wnorm, const float* g) {
    if (!W0 || !A || !B) return fail(DORA_ERR_INVALID_ARG, "W0, A and B must be non-NULL");
    if (!wnorm) return fail(DORA_ERR_INVALID_ARG, "wnorm must be non-NULL");
    if (m && !g) return fail(DORA_ERR_INVALID_ARG, "g must be non-NULL when m is given");
    if (!dim_ok(d_out, 1) || !dim_ok(d_in, 1) || !dim_ok(r, 1))
        return fail(DORA_ERR_INVALID_ARG, "sizes must satisfy 1 <= d_out, d_in, r < 2^31 (got %lld, %lld, %lld)",
                    (long long)d_out, (long long)d_in, (long long)r);
    if (!dtype_ok(dtype)) return fail(DORA_ERR_INVALID_ARG, "unknown dtype code %d", dtype);
    if (dtype == DORA_F16) return fail(DORA_ERR_UNSUPPORTED, "factored norm supports bf16 and fp32 inputs");
    if (!std::isfinite(s)) return fail(DORA_ERR_INVALID_ARG, "s must be finite");
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(DORA_ERR_INVALID_ARG, "eps must be finite and >= 0");
    return DORA_OK;
}

// Scratch of the allocation-free norm entry point: one array per GPU, held
// by the loaded code object until the process ends.  In host code `scratch`
// names a host-side shadow, not device memory, so its device address is taken
// once per device with hipGetSymbolAddress (with that device current) and
// only that address is handed to kernels.
constexpr size_t kScratchBytes = DORA_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

int scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(DORA_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (!p || !aligned256(p)) return fail(DORA_ERR_HIP, "scratch address %p is not 256-byte aligned", p);
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return DORA_OK;
}

}  // namespace

extern "C" {

const char* dora_status_string(int status) {
    switch (status) {
        case DORA_OK: return "ok";
        case DORA_ERR_INVALID_ARG: return "invalid argument";
        case DORA_ERR_UNSUPPORTED: return "unsupported";
        case DORA_ERR_WORKSPACE: return "workspace missing or too small";
        case DORA_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char* dora_last_error_detail(void) { return g_detail; }

int dora_version(void) { return 200; }

int dora_factored_norm_workspace_size(int64_t d_out, int64_t d_in, int64_t r, int dtype, size_t* bytes) {
    if (!bytes) return fail(DORA_ERR_INVALID_ARG, "bytes is NULL");
    if (!dim_ok(d_out, 1) || !dim_ok(d_in, 1) || !dim_ok(r, 1))
        return fail(DORA_ERR_INVALID_ARG, "sizes must satisfy 1 <= d_out, d_in, r < 2^31 (got %lld, %lld, %lld)",
                    (long long)d_out, (long long)d_in, (long long)r);
    if (!dtype_ok(dtype)) return fail(DORA_ERR_INVALID_ARG, "unknown dtype code %d", dtype);
    if (dtype == DORA_F16) return fail(DORA_ERR_UNSUPPORTED, "factored norm supports bf16 and fp32 inputs");
    // The s == 0 path needs less; the query reports the general size.
    *bytes = dora::plan_norm(d_out, d_in, r, dtype, false).bytes_needed;
    return ok();
}

int dora_factored_norm(const void* W0, const void* A, const void* B, const float* m, int64_t d_out, int64_t d_in,
                       int64_t r, int dtype, float s, float eps, float* wnorm, float* g, void* workspace,
                       size_t workspace_bytes, void* stream) {
    const int st = check_norm_args(W0, A, B, m, d_out, d_in, r, dtype, s, eps, wnorm, g);
    if (st != DORA_OK) return st;
    const dora::NormPlan plan = dora::plan_norm(d_out, d_in, r, dtype, s == 0.0f);
    if (plan.bytes_needed > 0) {
        if (!workspace) return fail(DORA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", plan.bytes_needed);
        if (workspace_bytes < plan.bytes_needed)
            return fail(DORA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes,
                        plan.bytes_needed);
        if (!aligned256(workspace)) return fail(DORA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    }
    hipError_t e = dora::launch_norm(plan, W0, A, B, m, s, eps, wnorm, g, workspace,
                                     static_cast<hipStream_t>(stream));
    return hip_status(e, "dora_factored_norm launch");
}

int dora_factored_norm_noalloc(const void* W0, const void* A, const void* B, const float* m, int64_t d_out,
                               int64_t d_in, int64_t r, int dtype, float s, float eps, float* wnorm, float* g,
                               void* stream) {
    const int st = check_norm_args(W0, A, B, m, d_out, d_in, r, dtype, s, eps, wnorm, g);
    if (st != DORA_OK) return st;
    const dora::NormPlan plan = dora::plan_norm(d_out, d_in, r, dtype, s == 0.0f);
    if (plan.bytes_needed > kScratchBytes)
        return fail(DORA_ERR_WORKSPACE, "these sizes need %zu bytes of scratch; the static scratch holds %zu",
                    plan.bytes_needed, kScratchBytes);
    void* ws = nullptr;
    const int sst = scratch_of_current_device(&ws);
    if (sst != DORA_OK) return sst;
    hipError_t e = dora::launch_norm(plan, W0, A, B, m, s, eps, wnorm, g, ws, static_cast<hipStream_t>(stream));
    return hip_status(e, "dora_factored_norm_noalloc launch");
}

static_assert(DORA_MAX_NORM_GROUP == dora::kMaxNormGroup, "group size limit");

int dora_factored_norm_group_workspace_size(int n, const int64_t* d_out, const int64_t* d_in, int64_t r, int dtype,
                                            size_t* bytes) {
    if (!bytes || !d_out || !d_in) return fail(DORA_ERR_INVALID_ARG, "bytes, d_out and d_in must be non-NULL");
    if (n < 1 || n > DORA_MAX_NORM_GROUP) return fail(DORA_ERR_INVALID_ARG, "n must be in 1..%d", DORA_MAX_NORM_GROUP);
    if (!dim_ok(r, 1)) return fail(DORA_ERR_INVALID_ARG, "r must satisfy 1 <= r < 2^31");
    if (!dtype_ok(dtype)) return fail(DORA_ERR_INVALID_ARG, "unknown dtype code %d", dtype);
    if (dtype == DORA_F16) return fail(DORA_ERR_UNSUPPORTED, "factored norm supports bf16 and fp32 inputs");
    for (int j = 0; j < n; ++j)
        if (!dim_ok(d_out[j], 1) || !dim_ok(d_in[j], 1))
            return fail(DORA_ERR_INVALID_ARG, "member %d: d_out or d_in out of range", j);
    *bytes = dora::norm_group_workspace_bytes(n, d_out, d_in, r, dtype);
    return ok();
}

int dora_factored_norm_group(int n, const DoraNormMember* members, int64_t r, int dtype, float eps,
                             void* workspace, size_t workspace_bytes, void* stream) {
    if (!members) return fail(DORA_ERR_INVALID_ARG, "members must be non-NULL");
    if (n < 1 || n > DORA_MAX_NORM_GROUP) return fail(DORA_ERR_INVALID_ARG, "n must be in 1..%d", DORA_MAX_NORM_GROUP);
    if (!dim_ok(r, 1)) return fail(DORA_ERR_INVALID_ARG, "r must satisfy 1 <= r < 2^31 (got %lld)", (long long)r);
    if (!dtype_ok(dtype)) return fail(DORA_ERR_INVALID_ARG, "unknown dtype code %d", dtype);
    if (dtype == DORA_F16) return fail(DORA_ERR_UNSUPPORTED, "factored norm supports bf16 and fp32 inputs");
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(DORA_ERR_INVALID_ARG, "eps must be finite and >= 0");
    int64_t d_outs[DORA_MAX_NORM_GROUP], d_ins[DORA_MAX_NORM_GROUP];
    dora::NormMember mem[DORA_MAX_NORM_GROUP];
    for (int j = 0; j < n; ++j) {
        const DoraNormMember& M = members[j];
        if (!M.W0 || !M.A || !M.B) return fail(DORA_ERR_INVALID_ARG, "member %d: W0, A and B must be non-NULL", j);
        if (!M.wnorm) return fail(DORA_ERR_INVALID_ARG, "member %d: wnorm must be non-NULL", j);
        if (M.m && !M.g) return fail(DORA_ERR_INVALID_ARG, "member %d: g must be non-NULL when m is given", j);
        if (!dim_ok(M.d_out, 1)) return fail(DORA_ERR_INVALID_ARG, "member %d: d_out out of range", j);
        if (!dim_ok(M.d_in, 1)) return fail(DORA_ERR_INVALID_ARG, "member %d: d_in out of range", j);
        if (!std::isfinite(M.s)) return fail(DORA_ERR_INVALID_ARG, "member %d: s must be finite", j);
        d_outs[j] = M.d_out;
        d_ins[j] = M.d_in;
        mem[j] = dora::NormMember{M.W0, M.A, M.B, M.m, M.wnorm, M.m ? M.g : nullptr, M.d_out, M.d_in, M.s};
    }
    const size_t need = dora::norm_group_workspace_bytes(n, d_outs, d_ins, r, dtype);
    if (!workspace) return fail(DORA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need) return fail(DORA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if (!aligned256(workspace)) return fail(DORA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    hipError_t e = dora::launch_norm_group(n, mem, r, dtype, eps, workspace, static_cast<hipStream_t>(stream));
    return hip_status(e, "dora_factored_norm_group launch");
}

int dora_compose(const void* base_out, const void* lora_out, const float* g, float s, int64_t T, int64_t d_out,
                 int dtype, int delta_only, void* y, void* stream) {
    if (!g) return fail(DORA_ERR_INVALID_ARG, "g must be non-NULL");
    if (T != 0 && (!base_out || !lora_out || !y))
        return fail(DORA_ERR_INVALID_ARG, "base_out, lora_out and y must be non-NULL when T > 0");
    if (!dim_ok(d_out, 1) || T < 0 || T >= ((int64_t)1 << 40))
        return fail(DORA_ERR_INVALID_ARG, "sizes must satisfy 1 <= d_out < 2^31, 0 <= T < 2^40 (got T=%lld, d_out=%lld)",
                    (long long)T, (long long)d_out);
    if (!dtype_ok(dtype)) return fail(DORA_ERR_INVALID_ARG, "unknown dtype code %d", dtype);
    if (delta_only != 0 && delta_only != 1) return fail(DORA_ERR_INVALID_ARG, "delta_only must be 0 or 1");
    if (!std::isfinite(s)) return fail(DORA_ERR_INVALID_ARG, "s must be finite");
    if (T != 0 && y == lora_out) return fail(DORA_ERR_INVALID_ARG, "y may alias base_out only");
    hipError_t e = dora::launch_compose_fwd(base_out, lora_out, g, s, T, d_out, dtype, delta_only != 0, y, nullptr,
                                            static_cast<hipStream_t>(stream));
    return hip_status(e, "dora_compose launch");
}

int dora_compose_dual(const void* base_out, const void* lora_out, const float* g, float s, int64_t T,
                      int64_t d_out, int dtype, int delta_only, void* y, void* inner, void* stream) {
    if (!g) return fail(DORA_ERR_INVALID_ARG, "g must be non-NULL");
    if (T != 0 && (!base_out || !lora_out || !y || !inner))
        return fail(DORA_ERR_INVALID_ARG, "base_out, lora_out, y and inner must be non-NULL when T > 0");
    if (!dim_ok(d_out, 1) || T < 0 || T >= ((int64_t)1 << 40))
        return fail(DORA_ERR_INVALID_ARG, "sizes must satisfy 1 <= d_out < 2^31, 0 <= T < 2^40 (got T=%lld, d_out=%lld)",
                    (long long)T, (long long)d_out);
    if (!dtype_ok(dtype)) return fail(DORA_ERR_INVALID_ARG, "unknown dtype code %d", dtype);
    if (delta_only != 0 && delta_only != 1) return fail(DORA_ERR_INVALID_ARG, "delta_only must be 0 or 1");
    if (!std::isfinite(s)) return fail(DORA_ERR_INVALID_ARG, "s must be finite");
    if (T != 0 && (y == lora_out || inner == base_out || y == inner))
        return fail(DORA_ERR_INVALID_ARG, "y may alias base_out only and inner lora_out only");
    hipError_t e = dora::launch_compose_fwd(base_out, lora_out, g, s, T, d_out, dtype, delta_only != 0, y, inner,
                                            static_cast<hipStream_t>(stream));
    return hip_status(e, "dora_compose_dual launch");
}

int dora_compose_backward_workspace_size(int64_t T, int64_t d_out, size_t* bytes) {
    if (!bytes) return fail(DORA_ERR_INVALID_ARG, "bytes is NULL");
    if (!dim_ok(d_out, 1) || T < 0 || T >= ((int64_t)1 << 40))
        return fail(DORA_ERR_INVALID_ARG, "sizes must satisfy 1 <= d_out < 2^31, 0 <= T < 2^40");
    *bytes = dora::compose_bwd_workspace_bytes(T, d_out);
    return ok();
}

int dora_compose_backward(const void* dy, const void* base_out, const void* lora_out, const float* g,
                          const float* wnorm, float s, float eps, int64_t T, int64_t d_out, int dtype,
                          int delta_only, void* d_base, void* d_lora, float* d_m, void* workspace,
                          size_t workspace_bytes, void* stream) {
    if (!g) return fail(DORA_ERR_INVALID_ARG, "g must be non-NULL");
    if (T != 0 && !dy) return fail(DORA_ERR_INVALID_ARG, "dy must be non-NULL when T > 0");
    if (d_m && !wnorm) return fail(DORA_ERR_INVALID_ARG, "wnorm must be non-NULL when d_m is requested");
    if (d_m && T != 0 && (!base_out || !lora_out))
        return fail(DORA_ERR_INVALID_ARG, "base_out and lora_out must be non-NULL when d_m is requested and T > 0");
    if (!dim_ok(d_out, 1) || T < 0 || T >= ((int64_t)1 << 40))
        return fail(DORA_ERR_INVALID_ARG, "sizes must satisfy 1 <= d_out < 2^31, 0 <= T < 2^40 (got T=%lld, d_out=%lld)",
                    (long long)T, (long long)d_out);
    if (!dtype_ok(dtype)) return fail(DORA_ERR_INVALID_ARG, "unknown dtype code %d", dtype);
    if (delta_only != 0 && delta_only != 1) return fail(DORA_ERR_INVALID_ARG, "delta_only must be 0 or 1");
    if (!std::isfinite(s)) return fail(DORA_ERR_INVALID_ARG, "s must be finite");
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(DORA_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (T != 0 && d_base && d_lora && d_base == d_lora)
        return fail(DORA_ERR_INVALID_ARG, "d_base and d_lora must differ");
    if (d_m) {
        const size_t need = dora::compose_bwd_workspace_bytes(T, d_out);
        if (need > 0) {
            if (!workspace) return fail(DORA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
            if (workspace_bytes < need)
                return fail(DORA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
            if (!aligned256(workspace)) return fail(DORA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        }
    }
    hipError_t e = dora::launch_compose_bwd(dy, base_out, lora_out, g, wnorm, s, eps, T, d_out, dtype,
                                            delta_only != 0, false, d_base, d_lora, d_m, workspace,
                                            static_cast<hipStream_t>(stream));
    return hip_status(e, "dora_compose_backward launch");
}

int dora_compose_backward_inner(const void* dy, const void* inner, const float* g, const float* wnorm, float s,
                                float eps, int64_t T, int64_t d_out, int dtype, int delta_only, void* d_base,
                                void* d_lora, float* d_m, void* workspace, size_t workspace_bytes, void* stream) {
    if (!g) return fail(DORA_ERR_INVALID_ARG, "g must be non-NULL");
    if (T != 0 && !dy) return fail(DORA_ERR_INVALID_ARG, "dy must be non-NULL when T > 0");
    if (d_m && !wnorm) return fail(DORA_ERR_INVALID_ARG, "wnorm must be non-NULL when d_m is requested");
    if (d_m && T != 0 && !inner)
        return fail(DORA_ERR_INVALID_ARG, "inner must be non-NULL when d_m is requested and T > 0");
    if (!dim_ok(d_out, 1) || T < 0 || T >= ((int64_t)1 << 40))
        return fail(DORA_ERR_INVALID_ARG, "sizes must satisfy 1 <= d_out < 2^31, 0 <= T < 2^40 (got T=%lld, d_out=%lld)",
                    (long long)T, (long long)d_out);
    if (!dtype_ok(dtype)) return fail(DORA_ERR_INVALID_ARG, "unknown dtype code %d", dtype);
    if (delta_only != 0 && delta_only != 1) return fail(DORA_ERR_INVALID_ARG, "delta_only must be 0 or 1");
    if (!std::isfinite(s)) return fail(DORA_ERR_INVALID_ARG, "s must be finite");
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(DORA_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (T != 0 && d_base && d_lora && d_base == d_lora)
        return fail(DORA_ERR_INVALID_ARG, "d_base and d_lora must differ");
    if (T != 0 && d_m && (d_base == inner || d_lora == inner))
        return fail(DORA_ERR_INVALID_ARG, "d_base and d_lora must not alias inner");
    if (d_m) {
        const size_t need = dora::compose_bwd_workspace_bytes(T, d_out);
        if (need > 0) {
            if (!workspace) return fail(DORA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
            if (workspace_bytes < need)
                return fail(DORA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
            if (!aligned256(workspace)) return fail(DORA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        }
    }
    hipError_t e = dora::launch_compose_bwd(dy, inner, nullptr, g, wnorm, s, eps, T, d_out, dtype, delta_only != 0,
                                            true, d_base, d_lora, d_m, workspace, static_cast<hipStream_t>(stream));
    return hip_status(e, "dora_compose_backward_inner launch");
}

int dora_merge_workspace_size(int64_t d_in, int64_t r, int dtype, size_t* bytes) {
    if (!bytes) return fail(DORA_ERR_INVALID_ARG, "bytes is NULL");
    if (!dim_ok(d_in, 1) || !dim_ok(r, 1) || r > kMaxMergeRank)
        return fail(DORA_ERR_INVALID_ARG, "sizes must satisfy 1 <= d_in < 2^31, 1 <= r <= %lld",
                    (long long)kMaxMergeRank);
    if (!dtype_ok(dtype)) return fail(DORA_ERR_INVALID_ARG, "unknown dtype code %d", dtype);
    if (dtype == DORA_F16) return fail(DORA_ERR_UNSUPPORTED, "merge supports bf16 and fp32 weights");
    *bytes = dora::merge_workspace_bytes(d_in, r, dtype);
    return ok();
}

int dora_merge(const void* W0, const void* A, const void* B, const float* g, float s, int64_t d_out, int64_t d_in,
               int64_t r, int dtype, void* W, void* workspace, size_t workspace_bytes, void* stream) {
    if (!W0 || !A || !B || !g || !W) return fail(DORA_ERR_INVALID_ARG, "W0, A, B, g and W must be non-NULL");
    if (!dim_ok(d_out, 1) || !dim_ok(d_in, 1) || !dim_ok(r, 1) || r > kMaxMergeRank)
        return fail(DORA_ERR_INVALID_ARG, "sizes must satisfy 1 <= d_out, d_in < 2^31, 1 <= r <= %lld (got %lld, %lld, %lld)",
                    (long long)kMaxMergeRank, (long long)d_out, (long long)d_in, (long long)r);
    if (((d_out + 127) / 128) * ((d_in + 127) / 128) >= ((int64_t)1 << 30))
        return fail(DORA_ERR_INVALID_ARG, "d_out x d_in too large (%lld x %lld)", (long long)d_out, (long long)d_in);
    if (!dtype_ok(dtype)) return fail(DORA_ERR_INVALID_ARG, "unknown dtype code %d", dtype);
    if (dtype == DORA_F16) return fail(DORA_ERR_UNSUPPORTED, "merge supports bf16 and fp32 weights");
    if (!std::isfinite(s)) return fail(DORA_ERR_INVALID_ARG, "s must be finite");
    if (W == A || W == B || W == static_cast<const void*>(g) || W == workspace)
        return fail(DORA_ERR_INVALID_ARG, "W may alias W0 only");
    const size_t need = dora::merge_workspace_bytes(d_in, r, dtype);
    if (!workspace) return fail(DORA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need) return fail(DORA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if (!aligned256(workspace)) return fail(DORA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    hipError_t e = dora::launch_merge(W0, A, B, g, s, d_out, d_in, r, dtype, W, workspace,
                                      static_cast<hipStream_t>(stream));
    return hip_status(e, "dora_merge launch");
}

}  // extern "C"
