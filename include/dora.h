/*
 * dora.h -- C ABI of the MI355X (gfx950) DoRA hot path: factored row norm and
 * fused compose, forward and backward.
 *
 * Sources, cited by short title and section:
 *   [ScalingDoRA]  "Scaling DoRA: High-Rank Adaptation via Factored Norms and
 *                  Fused Kernels" (arXiv:2603.22276, paperlayer.ai summary).
 *   [DoRA-wiki]    "DoRA" (aiwiki entry), DoRALinear.
 *   [LoRA&DoRA]    "LoRA & DoRA: The Math, Memory, and Trade-offs".
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers to dense, row-major, contiguous
 *     arrays (no strides).  W0, A, B and the activations share one element
 *     type `dtype`; m, g, wnorm and d_m are always fp32.
 *   - Layouts: W0 [d_out, d_in] (nn.Linear layout), A [r, d_in],
 *     B [d_out, r]; activations [T, d_out] with the per-feature vectors
 *     (g, wnorm, m, d_m) broadcast along the last axis.
 *   - Ownership: the caller owns every buffer, workspace included.  The
 *     library allocates nothing and keeps no mutable global state beyond the
 *     static scratch of dora_factored_norm_noalloc (and its per-device
 *     address), so calls are re-entrant; calls that share a workspace must
 *     not overlap.
 *   - Execution: work is enqueued on `stream` (a hipStream_t; NULL is the
 *     null stream) and the call returns without synchronising.  Arguments are
 *     validated on the host before anything is enqueued; on any error nothing
 *     is launched and no output is written.
 *   - Errors: every entry point returns a dora_status_t.  DORA_ERR_HIP means a
 *     HIP runtime call or a launch failed (dora_last_error_detail() names it);
 *     faults inside kernels surface at the caller's next synchronisation.
 *   - Sizes: any d_out, d_in, r >= 1 and T >= 0 are accepted (no multiple-of
 *     tile requirement); each dimension must be below 2^31.
 */
#ifndef DORA_H_
#define DORA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DORA_F32 = 0,   /* IEEE binary32 */
    DORA_BF16 = 1,  /* bfloat16 */
    DORA_F16 = 2    /* IEEE binary16 (compose only) */
} dora_dtype_t;

typedef enum {
    DORA_OK = 0,
    DORA_ERR_INVALID_ARG = 1,  /* NULL pointer, bad size, bad dtype code, bad flag */
    DORA_ERR_UNSUPPORTED = 2,  /* valid request this library does not implement */
    DORA_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than the size query */
    DORA_ERR_HIP = 4           /* HIP runtime or launch failure */
} dora_status_t;

/* Static string naming a status code (unknown codes give "unknown status"). */
const char* dora_status_string(int status);

/* Text of the last error raised on the calling thread ("" if none). */
const char* dora_last_error_detail(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int dora_version(void);

/*
 * Workspace bytes needed by dora_factored_norm for these sizes (host call,
 * launches nothing).  *bytes receives the size; 0 is possible.
 */
int dora_factored_norm_workspace_size(int64_t d_out, int64_t d_in, int64_t r, int dtype,
                                      size_t* bytes);

/*
 * Factored row norm and magnitude scale, never forming B @ A.
 *
 * [ScalingDoRA] §2 (squared row norm = base + cross + Gram terms through
 * O(d_out r + r^2) intermediates), App. B (assembly max(base + 2s cross +
 * s^2 ba, 0), square root) and §4 (g = m / max(wnorm, eps)):
 *   wnorm_i = sqrt(max(||W0_i||^2 + 2s B_i.(W0 A^T)_i + s^2 B_i (A A^T) B_i^T, 0))
 *   g_i     = m_i / max(wnorm_i, eps)
 * which equals ||W0_i + s (BA)_i|| ([DoRA-wiki] forward).  Accumulation is
 * fp32 whatever the input dtype ([ScalingDoRA] §2, Data Availability).
 *
 *   W0, A, B  device, dtype DORA_BF16 or DORA_F32 (DORA_F16 returns
 *             DORA_ERR_UNSUPPORTED), layouts above.
 *   m         device fp32 [d_out], or NULL to compute wnorm only.
 *   s         LoRA scale (alpha / r); s == 0 takes a base-norm-only path.
 *   eps       clamp of the magnitude division, >= 0.
 *   wnorm     device fp32 [d_out], output.
 *   g         device fp32 [d_out], output; required when m != NULL, ignored
 *             (may be NULL) when m == NULL.
 *   workspace device scratch of at least dora_factored_norm_workspace_size()
 *             bytes, 256-byte aligned; contents need no initialisation.
 */
int dora_factored_norm(const void* W0, const void* A, const void* B, const float* m,
                       int64_t d_out, int64_t d_in, int64_t r, int dtype, float s, float eps,
                       float* wnorm, float* g, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Bytes of the static per-GPU scratch behind dora_factored_norm_noalloc. */
#define DORA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * dora_factored_norm without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, outputs, kernels and results
 * are those of dora_factored_norm (bitwise the same); the workspace is a
 * static array of DORA_NOALLOC_SCRATCH_BYTES in the library's code object,
 * one per GPU, held until the process ends.  Its device address is looked up
 * once per device on the first call made with that device current; the call
 * itself allocates nothing.
 *
 *   The call runs on the current device; `stream` must belong to it.
 *   Sizes whose dora_factored_norm_workspace_size() exceeds
 *   DORA_NOALLOC_SCRATCH_BYTES return DORA_ERR_WORKSPACE before anything is
 *   launched; r <= 512 with d_out, d_in <= 32768 fits in bf16 and fp32.
 *   Every call on one GPU shares that GPU's scratch and leaves its contents
 *   behind; the kernels initialise what they read.  Calls that overlap in
 *   time on one GPU (different streams, or threads without ordering) race on
 *   the scratch and give undefined results: order them on one stream.
 */
int dora_factored_norm_noalloc(const void* W0, const void* A, const void* B, const float* m,
                               int64_t d_out, int64_t d_in, int64_t r, int dtype, float s, float eps,
                               float* wnorm, float* g, void* stream);

/*
 * One member of a grouped norm call: the operands and outputs of one
 * dora_factored_norm call (same meanings and layouts).  W0 is [d_out, d_in],
 * A [r, d_in], B [d_out, r]; m may be NULL (then g is not written).
 */
typedef struct DoraNormMember {
    const void* W0;
    const void* A;
    const void* B;
    const float* m;
    float* wnorm;
    float* g;
    int64_t d_out;
    int64_t d_in;
    float s;
} DoraNormMember;

/* Maximum members of one grouped norm call. */
#define DORA_MAX_NORM_GROUP 8

/*
 * Workspace bytes needed by dora_factored_norm_group for members of these
 * sizes (host call, launches nothing): d_out and d_in are host arrays of n
 * entries, member j being [d_out[j], d_in[j]].
 */
int dora_factored_norm_group_workspace_size(int n, const int64_t* d_out, const int64_t* d_in, int64_t r, int dtype,
                                            size_t* bytes);

/*
 * Factored row norms of up to DORA_MAX_NORM_GROUP adapted projections that
 * share r and the dtype (for example every projection of one layer, whose
 * norms depend on its weights alone), in one call.  Each member computes
 * exactly what dora_factored_norm computes for it, with bitwise the same
 * result; when every member is bf16 with 16-byte aligned operands and
 * r > 128, each stage of the method ([ScalingDoRA] §2: Gram, the W0 pass with
 * its row epilogue, assembly) runs as one launch for the whole group, so
 * small projections (k/v rows) share the chip instead of paying launch and
 * tail costs one by one, and long ones fill each other's last round.
 *
 *   n         1 .. DORA_MAX_NORM_GROUP.
 *   members   host array of n members, each with its own d_out and d_in;
 *             every member's pointers are device pointers, validated as in
 *             dora_factored_norm.  Outputs of different members must not
 *             overlap.
 *   r, dtype, eps   shared by all members.
 *   workspace device scratch of at least
 *             dora_factored_norm_group_workspace_size() bytes, 256-byte
 *             aligned.
 */
int dora_factored_norm_group(int n, const DoraNormMember* members, int64_t r, int dtype, float eps,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused compose forward, one pass: 2 reads + 1 write per element.
 *
 * [ScalingDoRA] §3 (compose kernel, numerically stable form with fp32
 * intermediates and an explicit (g - 1) correction), Data Availability
 * (module contract dY = g*(s lora) + (g - 1)*base) and App. B (g broadcast
 * along the last axis; activations stay in their dtype):
 *   delta_only == 0:  y = base + ((g - 1)*base + (g*s)*lora)
 *   delta_only == 1:  y =         (g - 1)*base + (g*s)*lora
 * evaluated in fp32 and rounded once (round-to-nearest-even) to dtype.
 *
 *   base_out, lora_out  device [T, d_out], dtype; lora_out excludes s.
 *   g                   device fp32 [d_out].
 *   y                   device [T, d_out], dtype, output; may alias base_out
 *                       exactly (in-place), must not partially overlap.
 * T == 0 is a no-op; the activation pointers may then be NULL.
 */
int dora_compose(const void* base_out, const void* lora_out, const float* g, float s,
                 int64_t T, int64_t d_out, int dtype, int delta_only, void* y, void* stream);

/*
 * Dual-output compose forward of the training tier, one pass: 2 reads + 2
 * writes per element.
 *
 * [ScalingDoRA] §4 (Tier 1: the layer output and the inner term come from one
 * kernel, so the backward needs no second forward pass):
 *   y      exactly as dora_compose (delta_only selects y or the delta)
 *   inner  = base + s*lora, in fp32, rounded once (round-to-nearest-even)
 * inner is the only activation dora_compose_backward_inner needs besides dy.
 *
 *   base_out, lora_out  device [T, d_out], dtype; lora_out excludes s.
 *   g                   device fp32 [d_out].
 *   y, inner            device [T, d_out], dtype, outputs; y may alias base_out
 *                       and inner may alias lora_out exactly (in-place); y and
 *                       inner must differ; no partial overlaps.
 * T == 0 is a no-op; the activation pointers may then be NULL.
 */
int dora_compose_dual(const void* base_out, const void* lora_out, const float* g, float s,
                      int64_t T, int64_t d_out, int dtype, int delta_only, void* y, void* inner,
                      void* stream);

/* Workspace bytes needed by dora_compose_backward and
 * dora_compose_backward_inner when d_m != NULL. */
int dora_compose_backward_workspace_size(int64_t T, int64_t d_out, size_t* bytes);

/*
 * Fused compose backward with the norm detached.
 *
 * [ScalingDoRA] §3 (backward kernel: d_lora and d_base in one pass; the
 * magnitude gradient as a separate deterministic reduction, no atomics),
 * Data Availability (norm detached); [DoRA-wiki] .detach() note:
 *   d_base = g*dy          (delta_only: (g - 1)*dy)
 *   d_lora = (g*s)*dy
 *   d_m_j  = sum_t dy_tj*(base_tj + s*lora_tj) / max(wnorm_j, eps)
 * d_m is summed in a fixed order, so results are bitwise reproducible.
 *
 *   dy                  device [T, d_out], dtype.
 *   base_out, lora_out  device [T, d_out], dtype; read only when d_m != NULL
 *                       (may be NULL otherwise).
 *   g                   device fp32 [d_out]; wnorm device fp32 [d_out] (read
 *                       only when d_m != NULL).
 *   d_base, d_lora      device [T, d_out], dtype, outputs, each may be NULL
 *                       to skip it; either may alias dy exactly.
 *   d_m                 device fp32 [d_out], output (overwritten, not
 *                       accumulated), or NULL when the magnitude is frozen.
 *   workspace           needed only when d_m != NULL: at least
 *                       dora_compose_backward_workspace_size() bytes,
 *                       256-byte aligned, no initialisation needed.
 * T == 0 writes zeros to d_m and nothing else; the activation pointers may
 * then be NULL.
 */
int dora_compose_backward(const void* dy, const void* base_out, const void* lora_out,
                          const float* g, const float* wnorm, float s, float eps, int64_t T,
                          int64_t d_out, int dtype, int delta_only, void* d_base, void* d_lora,
                          float* d_m, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Compose backward of the training tier from (dy, inner): 2 reads + 2 writes
 * per element instead of 3 + 2.
 *
 * [ScalingDoRA] §4 (Tier 1) and §3 (backward kernel; magnitude gradient as a
 * separate deterministic reduction), norm detached:
 *   d_base = g*dy          (delta_only: (g - 1)*dy)
 *   d_lora = (g*s)*dy
 *   d_m_j  = sum_t dy_tj*inner_tj / max(wnorm_j, eps)
 * with inner = base + s*lora as written by dora_compose_dual.  d_m is summed
 * in a fixed order, so results are bitwise reproducible.
 *
 *   dy                  device [T, d_out], dtype.
 *   inner               device [T, d_out], dtype; read only when d_m != NULL
 *                       (may be NULL otherwise).
 *   g, wnorm            as dora_compose_backward.
 *   d_base, d_lora      device [T, d_out], dtype, outputs, each may be NULL;
 *                       either may alias dy exactly, neither may alias inner.
 *   d_m                 device fp32 [d_out], output (overwritten), or NULL
 *                       when the magnitude is frozen.
 *   workspace           needed only when d_m != NULL: at least
 *                       dora_compose_backward_workspace_size() bytes,
 *                       256-byte aligned, no initialisation needed.
 * T == 0 writes zeros to d_m and nothing else.
 */
int dora_compose_backward_inner(const void* dy, const void* inner, const float* g,
                                const float* wnorm, float s, float eps, int64_t T, int64_t d_out,
                                int dtype, int delta_only, void* d_base, void* d_lora, float* d_m,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes needed by dora_merge (host call, launches nothing): A
 * transposed, with d_in rounded up to whole 256-row tiles and r to whole
 * 64-byte k-tiles.
 */
int dora_merge_workspace_size(int64_t d_in, int64_t r, int dtype, size_t* bytes);

/*
 * DoRA merge for serving: one weight with the adapter folded in.
 *
 * [LoRA&DoRA] §6 (merged DoRA weight m (W0 + sBA) / ||W0 + sBA||_row, an
 * ordinary matrix at inference) with the scale g = m / max(wnorm, eps) that
 * dora_factored_norm returns ([ScalingDoRA] §4):
 *   W_ij = g_i * (W0_ij + s * sum_k B_ik A_kj)
 * The product B A is accumulated in fp32 (MFMA), W0 + s*(BA) is one fused
 * multiply-add in fp32, the product with g is fp32, and the result is
 * rounded once (round-to-nearest-even) to dtype.
 *
 *   W0, A, B  device, dtype DORA_BF16 or DORA_F32 (DORA_F16 returns
 *             DORA_ERR_UNSUPPORTED), layouts above.
 *   g         device fp32 [d_out] (the g output of dora_factored_norm).
 *   s         LoRA scale (alpha / r).
 *   r         at most 4,194,176.
 *   W         device [d_out, d_in], dtype, output; may alias W0 exactly (an
 *             in-place merge), must not overlap A, B, g or the workspace.
 *   workspace device scratch of at least dora_merge_workspace_size() bytes,
 *             256-byte aligned; it receives A transposed (bf16: as 8 KB
 *             blocks of 128 rows by one k-tile, the layout the tile kernel's
 *             LDS stages take), no initialisation needed.
 */
int dora_merge(const void* W0, const void* A, const void* B, const float* g, float s, int64_t d_out,
               int64_t d_in, int64_t r, int dtype, void* W, void* workspace, size_t workspace_bytes,
               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DORA_H_ */
