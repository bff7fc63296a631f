// Host-side launchers behind the C ABI.  Arguments reaching these functions
// have already been validated by dora_capi.hip; launchers only pick a kernel
// variant and grid, enqueue on the stream, and report hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dora {

enum Dtype { kF32 = 0, kBF16 = 1, kF16 = 2 };

inline size_t dtype_size(int dt) { return dt == kF32 ? 4 : 2; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ------------------------------------------------------------ factored norm

// Tiling decisions are pure functions of the sizes, so that the workspace
// query and the launch agree.
struct NormPlan {
    int dtype;
    int64_t d_out, d_in, r;
    // W0 pass
    int cfg;            // tile configuration index (see norm.hip)
    bool big;           // 256 x 384 tiles (bf16, 16-byte aligned operands)
    int bm, bn, bk;     // rows of W0 per workgroup, columns of r per workgroup, K per tile
    int n_mtiles, n_ntiles;
    int nkt_w0, nkt_g;  // K tiles over d_in, then over the Gram block (r)
    int ksplit;
    // balanced K split of the large-tile pass (bal_nwg > 0): workgroup w of
    // bal_nwg owns an equal range of the m-tile-major (m-tile, k-tile) pairs,
    // bal_units of them, bal_nkt k-tiles per m-tile; ksplit is then the most
    // partial slots any m-tile has
    int bal_nwg, bal_nkt;
    int64_t bal_units;
    // Gram
    int gram_tiles;     // tiles per side (64 wide)
    int gram_split;
    bool gram_xcd;      // bf16 split-per-XCD Gram kernel (aligned operands)
    int64_t ldg;        // leading dimension of the scaled Gram operand
    // workspace layout (byte offsets)
    size_t off_gs, off_gpart, off_pbase, off_pcross, bytes;
    size_t bytes_needed;   // workspace to request: covers this plan and its unaligned fallback
    bool base_only;     // s == 0: only the base term is needed
};

NormPlan plan_norm(int64_t d_out, int64_t d_in, int64_t r, int dtype, bool base_only);

// Members of one grouped norm call (sizes validated by the caller).
constexpr int kMaxNormGroup = 8;
struct NormMember {
    const void* W0;
    const void* A;
    const void* B;
    const float* m;
    float* wnorm;
    float* g;
    int64_t d_out;
    int64_t d_in;
    float s;
};

// Workspace of a group: each member's own region, 256-byte aligned, in order.
size_t norm_group_workspace_bytes(int n, const int64_t* d_out, const int64_t* d_in, int64_t r, int dtype);

hipError_t launch_norm_group(int n, const NormMember* mem, int64_t r, int dtype, float eps, void* workspace,
                             hipStream_t stream);

hipError_t launch_norm(const NormPlan& p, const void* W0, const void* A, const void* B,
                       const float* m, float s, float eps, float* wnorm, float* g,
                       void* workspace, hipStream_t stream);

// ------------------------------------------------------------------ compose

size_t compose_bwd_workspace_bytes(int64_t T, int64_t d_out);

// inner may be nullptr; when set, inner = base + s * lora is written too.
hipError_t launch_compose_fwd(const void* base, const void* lora, const float* g, float s,
                              int64_t T, int64_t d_out, int dtype, bool delta_only, void* y,
                              void* inner, hipStream_t stream);

// inner_mode: `base` holds inner = base + s * lora and `lora` is unused.
hipError_t launch_compose_bwd(const void* dy, const void* base, const void* lora,
                              const float* g, const float* wnorm, float s, float eps,
                              int64_t T, int64_t d_out, int dtype, bool delta_only, bool inner_mode,
                              void* d_base, void* d_lora, float* d_m, void* workspace,
                              hipStream_t stream);

// -------------------------------------------------------------------- merge

size_t merge_workspace_bytes(int64_t d_in, int64_t r, int dtype);

// W = diag(g) (W0 + s B A); W may alias W0.
hipError_t launch_merge(const void* W0, const void* A, const void* B, const float* g, float s,
                        int64_t d_out, int64_t d_in, int64_t r, int dtype, void* W, void* workspace,
                        hipStream_t stream);

}  // namespace dora
