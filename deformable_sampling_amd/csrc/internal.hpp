// Host-side launch interface between the C ABI (api.cpp) and the kernel files.
// Arguments reaching a launcher have already been validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "dcn.h"

namespace dcn {

struct CoreLaunch {
    const void *x;
    const void *offset;  // elements of om_dtype
    const void *mask;    // may be NULL
    void *out;
    int N, H, W, G, C, kh, kw, sh, sw, ph, pw, dh, dw, Ho, Wo;
    float offset_scale;
    int softmax;
    dcn_dtype dtype;
    // Offsets and masks: pair (output pixel p = (n*Ho + ho)*Wo + wo, group g) reads its
    // K (dx, dy) pairs at offset + p*off_pix + g*off_grp and its K masks at
    // mask + p*mask_pix + g*mask_grp (elements of om_dtype). om_plain: fp32 with
    // off_grp = 2K, off_pix = G*2K, mask_grp = K, mask_pix = G*K (separate tensors).
    dcn_dtype om_dtype;
    int off_pix, off_grp, mask_pix, mask_grp;
    bool om_plain;
};
hipError_t launch_dcn_core(const CoreLaunch &a, hipStream_t stream);

// Core backward (dcn_core_bwd.hip). grad_x / grad_offset / grad_mask may be NULL.
struct CoreBwdLaunch {
    const void *x;
    const float *offset;
    const float *mask;  // may be NULL
    const void *grad_out;
    void *grad_x;
    float *grad_offset;
    float *grad_mask;
    void *workspace;
    int N, H, W, G, C, kh, kw, sh, sw, ph, pw, dh, dw, Ho, Wo;
    float offset_scale;
    int softmax;
    dcn_dtype dtype;
    unsigned path;  // DCN_BWD_* flags (0: the default kernels)
};
// Workspace plan of the backward. Binned (the default): bin counts, fill cursors,
// bin starts and one 16-byte record per sample. Fallback (sizes beyond the record
// packing, or force_fallback): an fp32 grad_x accumulator for fp16/bf16.
struct CoreBwdPlan {
    bool binned;
    int TY, TX, TYr, TXr;  // bin grid (floor(H/16)+1 x floor(W/16)+1), real tiles (ceil)
    long long nbins, nsamples;
    size_t off_counts, off_fill, off_starts, off_rec, off_acc, total;
};
void plan_core_bwd(int N, int H, int W, int G, int C, int Ho, int Wo, int K, dcn_dtype dtype,
                   bool force_fallback, CoreBwdPlan &plan);
hipError_t launch_dcn_core_bwd(const CoreBwdLaunch &a, const CoreBwdPlan &plan, hipStream_t stream);

// LDS halo-tile variant of the core (dcn_core_tile.hip).
struct CoreTilePlan {
    int N, H, W, G, C, kh, kw, sh, sw, ph, pw, dh, dw, Ho, Wo;
    float offset_scale;
    int softmax, has_mask;
    int off_pix, off_grp, mask_pix, mask_grp;  // as CoreLaunch (packed layouts)
    int GB, S, NC;           // groups per block, lanes per pair, 16-B chunks per lane
    int cpp, cpp_log2, lpp;  // 16-B chunks per region pixel (2^cpp_log2), lanes per pixel
    int TH, TW, halo, RH, RW;
    int tiles_x, tiles_y, gblocks, nblocks, threads;  // nblocks = number of tiles
    size_t lds_bytes;
};
bool plan_core_tile(const CoreLaunch &a, CoreTilePlan &plan);
hipError_t launch_dcn_core_tile(const CoreLaunch &a, const CoreTilePlan &plan, hipStream_t stream);
// grad_x records of the core backward (see dcn_core_bwd.hip): the record array, the
// bin starts from the scan, the fill cursors, and the bin grid (tiles per column/row).
struct CoreRecArgs {
    uint4 *rec;
    const unsigned *starts;
    unsigned *fill;
    int TY, TX;
};
// grad_offset / grad_mask of the core backward on a forward tile plan with S == 1 and
// plain fp32 offsets (a.out = grad_out); hipErrorInvalidValue for other plans. With
// ra != NULL the kernel also files the grad_x records when its variant can (then
// *rec_done = true; otherwise the caller files them).
hipError_t launch_dcn_core_bwd_tile(const CoreLaunch &a, const CoreTilePlan &plan, float *goff,
                                    float *gmask, const CoreRecArgs *ra, bool *rec_done,
                                    hipStream_t stream);

// Workspace plan of the DCNv2 path (all offsets 256-byte aligned).
struct V2Plan {
    int Ho, Wo, K;
    long long P;      // N*Ho*Wo output pixels
    int Cin_pad;      // Cin rounded up to the channel vector (8 elements)
    int R;            // K*Cin_pad: columns per pixel (tap-major, channel-minor)
    int Rp;           // R rounded up to the GEMM K tile
    long long Pp;     // P rounded up to the GEMM N tile
    int Mp;           // Cout rounded up to the GEMM M tile
    size_t off_xt, off_wp, off_col, total;
    bool fused;       // deform-im2col fused into the GEMM (the column region unused)
};
bool plan_dcn_v2(int N, int Cin, int H, int W, int Cout, int kh, int kw, int sh, int sw, int ph,
                 int pw, int dh, int dw, dcn_dtype dtype, V2Plan &plan);
// Whether a forward call on this plan forms its columns on chip inside the GEMM (then
// only the workspace bytes [0, off_col) are touched).
bool v2_fused_applies(const V2Plan &plan, int dg, bool has_weight);

struct V2Launch {
    const void *x;
    const float *offset;
    const float *mask;  // may be NULL
    const void *weight;
    const void *packed_weight;  // non-NULL: the weight already in the fused kernel's order
    void *out;
    void *workspace;
    int N, Cin, H, W, Cout, kh, kw, sh, sw, ph, pw, dh, dw, dg, softmax;
    dcn_dtype dtype;
    V2Plan plan;
};
hipError_t launch_dcn_v2(const V2Launch &a, hipStream_t stream);
// The weight [Cout, Cin, kh, kw] permuted into the fused kernel's order (plan: Mp, Rp,
// Cin_pad, K from plan_dcn_v2) at `packed`.
hipError_t launch_dcn_v2_pack_weight(const void *weight, void *packed, int Cout, int Cin, const V2Plan &plan,
                                     hipStream_t stream);

// DCNv2 backward (dcn_v2_bwd.hip). Workspace regions (byte offsets, 256-aligned):
// xt [N,H,W,Cin_pad], wT [Rr][CoK], gcl [Pp][CoK], goT [CoM][Pp], colT [Rr][Pp] (dtype);
// gcol [P][R], weight partials [splits][Cout][R] (fp32); bucket counts + fill cursors
// [2][D], starts [D] (int32, D = N*H*W*dg); entries [P*dg*K*4] (8 bytes).
struct V2BwdPlan {
    int Ho, Wo, K, Cin_pad, R, Rr, CoK, CoM, splits;
    long long P, Pp, D, entries;
    size_t off_xt, off_wt, off_gcl, off_got, off_colt, off_gcol, off_wpart, off_cnt, off_starts,
        off_entries, total;
};
bool plan_dcn_v2_bwd(int N, int Cin, int H, int W, int Cout, int kh, int kw, int sh, int sw, int ph,
                     int pw, int dh, int dw, int dg, dcn_dtype dtype, V2BwdPlan &plan);
struct V2BwdLaunch {
    const void *x;
    const float *offset;
    const float *mask;  // may be NULL
    const void *weight;
    const void *grad_out;
    void *grad_x;         // may be NULL
    float *grad_offset;   // may be NULL
    float *grad_mask;     // may be NULL
    float *grad_weight;   // may be NULL
    void *workspace;
    int N, Cin, H, W, Cout, kh, kw, sh, sw, ph, pw, dh, dw, dg, softmax;
    dcn_dtype dtype;
    V2BwdPlan plan;
};
hipError_t launch_dcn_v2_bwd(const V2BwdLaunch &a, hipStream_t stream);

constexpr int kAggMaxMaps = 64;
struct AggMaps {
    int H[kAggMaxMaps];
    int W[kAggMaxMaps];
    int start[kAggMaxMaps];
};
struct AggLaunch {
    const void *feat;
    const float *loc;
    const float *weights;
    void *out;
    int B, P_total, A, pts, cams, scales, G, Cg, softmax;
    dcn_dtype dtype;
    AggMaps maps;
};
hipError_t launch_deform_agg(const AggLaunch &a, hipStream_t stream);

// Aggregation backward (deform_agg_bwd.hip). grad_feat / grad_loc / grad_weights
// may be NULL. Workspace: per-group grad_loc partials, then either the feature
// buckets (normalised weights [B*A*T*G] fp32, counts + fill cursors [2][B*P_total],
// starts [B*P_total] and scan block sums uint32, entries [B*A*T*4] of 8 bytes) or, past the bucket
// limits, an fp32 grad_feat accumulator (fp16/bf16 only).
struct AggBwdLaunch {
    const void *feat;
    const float *loc;
    const float *weights;
    const void *grad_out;
    void *grad_feat;
    float *grad_loc;
    float *grad_weights;
    void *workspace;
    int B, P_total, A, pts, cams, scales, G, Cg, softmax;
    dcn_dtype dtype;
    AggMaps maps;
    unsigned path;  // DCN_BWD_* flags (0: the default kernels)
};
struct AggBwdPlan {
    bool binned;
    long long D, nent;
    size_t off_loc, off_acc, off_wn, off_cnt, off_starts, off_bsum, off_ent, off_gt, off_us, total;
};
void plan_agg_bwd(int B, int P_total, int A, int pts, int cams, int scales, int G, int Cg,
                  dcn_dtype dtype, bool force_atomic, AggBwdPlan &plan);
hipError_t launch_deform_agg_bwd(const AggBwdLaunch &a, const AggBwdPlan &plan, hipStream_t stream);

// Deformable RoI pooling (deform_roi_pool.hip).
struct RoiLaunch {
    const void *x;
    const float *rois;
    const float *offset;  // may be NULL
    void *out;
    int N, H, W, C, R, k, S;
    float spatial_scale, gamma;
    dcn_dtype dtype;
};
hipError_t launch_deform_roi_pool(const RoiLaunch &a, hipStream_t stream);

// MFMA rate probe (probe.hip): blocks of 256 threads, iters rounds of four
// 32x32x16 bf16 MFMAs per wave; sink gets blocks*256 floats.
hipError_t launch_mfma_probe(float *sink, int blocks, int iters, hipStream_t stream);

}  // namespace dcn
