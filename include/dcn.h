/*
 * dcn.h — C ABI of the MI355X (gfx950) deformable-sampling library, libdcn.so.
 *
 * Forward operations and two backward passes, each enqueued on a caller-supplied HIP stream:
 *
 *   dcn_core_forward    DCNv3/v4 core (also DCNv1 when mask == NULL), channels-last.
 *   dcn_core_forward_packed  the same with DCNv4's packed offset+mask tensor, fp32/fp16/bf16.
 *   dcn_core_backward   gradients of the core w.r.t. x, offsets and modulation.
 *   dcn_v2_forward      DCNv2 modulated deformable convolution, NCHW: deform-im2col
 *                       and an MFMA GEMM (fused, or in two stages through the workspace).
 *   dcn_v2_im2col       the deform-im2col stage alone: columns into the workspace.
 *   dcn_v2_forward_noalloc  dcn_v2_forward with a static in-library workspace.
 *   dcn_v2_pack_weight, dcn_v2_forward_prepacked  the weight permuted once into the
 *                       fused kernel's order, and the forward that reads it.
 *   dcn_v2_backward     gradients of DCNv2 w.r.t. x, offsets, masks and the weight.
 *   deform_agg_forward  Sparse4D-style multi-camera, multi-scale aggregation.
 *   deform_agg_backward gradients of the aggregation w.r.t. features, locations, weights.
 *   deform_roi_pool_forward  deformable RoI pooling, channels-last.
 *   dcn_core_backward_path, deform_agg_backward_path  the two backward passes with an
 *                       explicit choice among their alternative kernel paths.
 *
 * What is computed (page title, section):
 *  - Deformable sum y(p0) = sum_n w(p_n) x(p0 + p_n + dp_n), fractional positions
 *    read through the bilinear kernel G(q,p) = g(qx,px) g(qy,py),
 *    g(a,b) = max(0, 1 - |a-b|): "Hands-on DCNv1 in PyTorch" (agent.csdn.net),
 *    sections 1 and 2.
 *  - Modulation scalars multiplying each sample: "DCNv2 in YOLOv5" (cyqw.cn),
 *    section 1.
 *  - Channel groups with their own offsets and modulation; DCNv3 normalises the
 *    modulation with a softmax over the K points of a group, DCNv4 does not;
 *    channels-last tensors and offset_scale: "DCNv4 in YOLOv11" (lpnh.cn),
 *    sections 1.1 and 3.2.
 *  - Aggregation inputs (features flattened to [B, N*H*W, C], spatial shapes, scale
 *    start index, sampling locations, weights) and softmax-normalised weights:
 *    "Sparse4D deformable_aggregation" (mlqm.cn), sections 2.1, 2.2 and 7.
 *
 * Conventions shared by all entry points
 *  - Every tensor argument is dense, contiguous device memory in the stated
 *    order, owned by the caller. The library allocates nothing, copies nothing
 *    between host and device and never synchronises: it validates the arguments
 *    on the host, enqueues its kernels on `stream` and returns. Buffers must stay
 *    alive until that stream work has completed. `out` is fully overwritten and
 *    must not overlap any input.
 *  - Sampling: zero outside the image, per bilinear corner. A corner outside the
 *    image contributes exactly 0; every memory read stays inside the image (such
 *    corners read a clamped in-image pixel or on-chip zeros), so inputs must be
 *    finite. Kernel point k = i*kw + j (i along H). The grid base of
 *    output (ho, wo) and point (i, j) is (ho*stride_h - pad_h + i*dil_h,
 *    wo*stride_w - pad_w + j*dil_w); offsets are (dx, dy) pairs, x first.
 *  - Ho = (H + 2*pad_h - dil_h*(kh-1) - 1)/stride_h + 1, likewise Wo.
 *  - Arithmetic is fp32 with fp32 accumulation; fp16/bf16 outputs are rounded
 *    once (round-to-nearest-even).
 *  - Errors: an integer status, never an abort. All argument checks run on the
 *    host before any HIP call, so a rejected call has no effect. DCN_ERR_HIP means
 *    a launch failed; dcn_last_hip_error() then returns the hipError_t (per thread).
 *    Zero-sized work (N, H, W or A equal to 0) returns DCN_OK and launches nothing.
 *  - Thread-safe and re-entrant; the only state is the per-thread last HIP error (and
 *    the static workspace of dcn_v2_forward_noalloc, whose overlapping calls race).
 */
#ifndef DCN_H_
#define DCN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DCN_F32 = 0, DCN_F16 = 1, DCN_BF16 = 2 } dcn_dtype;

typedef enum {
    DCN_OK = 0,
    DCN_ERR_NULL = 1,      /* a required pointer is NULL                           */
    DCN_ERR_SHAPE = 2,     /* a size is negative, Ho/Wo <= 0, or a size limit hit   */
    DCN_ERR_PARAM = 3,     /* stride/dilation <= 0, pad < 0, bad group split, ...   */
    DCN_ERR_DTYPE = 4,     /* dtype not supported by this entry point               */
    DCN_ERR_ALIGN = 5,     /* a pointer is not aligned to its element size          */
    DCN_ERR_WORKSPACE = 6, /* workspace NULL, misaligned (256 B) or too small       */
    DCN_ERR_HIP = 7,       /* a HIP launch failed; see dcn_last_hip_error()         */
    DCN_ERR_SCRATCH = 8    /* dcn_v2_forward_noalloc: the call needs more than the
                              library's static scratch (DCN_V2_NOALLOC_SCRATCH_BYTES) */
} dcn_status;

/*
 * DCNv3/v4 core forward (DCNv1-style when mask == NULL), channels-last.
 *
 *   x       [N, H, W, G*C]        dtype
 *   offset  [N, Ho, Wo, G, K, 2]  fp32, (dx, dy) in pixels, K = kh*kw
 *   mask    [N, Ho, Wo, G, K]     fp32 modulation (logits when softmax != 0), or NULL
 *   out     [N, Ho, Wo, G*C]      dtype
 *
 * out[n,ho,wo,g*C+c] = sum_k m_k * bilinear(x[n,:,:,g*C+c], y_k, x_k), where
 * y_k = base_y + fl32(offset_scale*dy_k) and x_k = base_x + fl32(offset_scale*dx_k),
 * and m_k = mask (1 when NULL) or, with softmax != 0, the softmax over the K points
 * of (n, ho, wo, g) (DCNv3). Limits: K <= 64; each image H*W*G*C < 2^31 elements.
 * Pointers must be aligned to their element size; 16-byte alignment of x/out with
 * C*sizeof(dtype) a multiple of 16 selects the widest vector path.
 */
dcn_status dcn_core_forward(const void *x, const float *offset, const float *mask, void *out,
                            int N, int H, int W, int G, int C, int kh, int kw,
                            int stride_h, int stride_w, int pad_h, int pad_w,
                            int dil_h, int dil_w, float offset_scale, int softmax,
                            dcn_dtype dtype, hipStream_t stream);

/*
 * dcn_core_forward with DCNv4's packed offset+mask tensor ("DCNv4 in YOLOv11",
 * section 3.2: one offset-generating projection per group yields both the offsets
 * and the modulation) in fp32, fp16 or bf16:
 *
 *   offset_mask  [N, Ho, Wo, om_pixel_stride]  om_dtype; for group g the row at
 *                element g*3K holds the K (dx, dy) pairs (x first) and then the K
 *                masks (logits when softmax != 0); om_pixel_stride >= G*3K (pixel
 *                rows may be padded, e.g. to a multiple of 8 elements)
 *
 * Offsets and masks are widened exactly to fp32; everything else, results included,
 * is as dcn_core_forward (the scaled offset fl32(offset_scale * dx) is the same fp32
 * quantity). Halving the offset/mask bytes is what the fp16/bf16 forms are for.
 * offset_mask must be aligned to its element size. DCN_ERR_PARAM if
 * om_pixel_stride < G*3K.
 */
dcn_status dcn_core_forward_packed(const void *x, const void *offset_mask, void *out, int N, int H,
                                   int W, int G, int C, int kh, int kw, int stride_h, int stride_w,
                                   int pad_h, int pad_w, int dil_h, int dil_w, float offset_scale,
                                   int softmax, int om_pixel_stride, dcn_dtype om_dtype,
                                   dcn_dtype dtype, hipStream_t stream);

/*
 * Workspace bytes dcn_core_backward needs when grad_x is requested (0 if the sizes
 * are invalid). grad_x is formed without atomics: the samples are sorted by
 * destination tile through the workspace, which holds per-bin counters and start
 * offsets (4 * N*G*(H/16+1)*(W/16+1) bins of 4 bytes, three arrays) and one
 * 16-byte record per sample (N*Ho*Wo*G*K records), each region 256-byte aligned.
 * Beyond N*Ho*Wo*G*K >= 2^31 or Ho*Wo >= 2^24 the backward instead accumulates
 * grad_x with fp32 atomic adds, and the workspace is an fp32 copy of x's shape for
 * fp16/bf16 (0 for fp32).
 */
size_t dcn_core_backward_workspace_bytes(int N, int H, int W, int G, int C, int kh, int kw,
                                         int stride_h, int stride_w, int pad_h, int pad_w,
                                         int dil_h, int dil_w, dcn_dtype dtype);

/*
 * DCNv3/v4 core backward: the gradients of dcn_core_forward's output (same
 * arguments) w.r.t. x, the offsets and the mask. The pages define only the forward
 * sum; these are its derivatives:
 *
 *   grad_out     [N, Ho, Wo, G*C]        dtype, the gradient of the loss w.r.t. out
 *   grad_x       [N, H, W, G*C]          dtype, overwritten, or NULL (not computed)
 *   grad_offset  [N, Ho, Wo, G, K, 2]    fp32, overwritten, or NULL
 *   grad_mask    [N, Ho, Wo, G, K]       fp32, overwritten, or NULL; w.r.t. the mask
 *                                        argument (the logits when softmax != 0), or,
 *                                        when mask == NULL, w.r.t. the implied unit
 *                                        modulation (zero logits with softmax)
 *
 * With w_ab the bilinear weights of tap k's corners and B_k, dB_k/dy, dB_k/dx the
 * sample and its derivatives in the position (taken from the right at integer
 * positions):
 *   grad_x[corner]   += m_k * w_ab * grad_out          (corners inside the image)
 *   grad_m_k          = sum_c grad_out[c] * B_k[c]
 *   grad_offset[k]    = offset_scale * m_k * sum_c grad_out[c] * (dB_k/dx, dB_k/dy)[c]
 *   softmax != 0:     grad_logit_k = m_k * (grad_m_k - sum_j m_j grad_m_j)
 * grad_x sums in fp32 and is rounded once to dtype; the order of its sums varies
 * from run to run (within fp32 accumulation error); grad_offset and grad_mask are
 * deterministic. workspace: dcn_core_backward_workspace_bytes bytes, 256-byte
 * aligned, used only when grad_x != NULL (may be NULL otherwise, or when that size
 * is 0); its contents on entry are ignored. Limits and alignment as
 * dcn_core_forward; the outputs must not overlap each other or any input.
 */
dcn_status dcn_core_backward(const void *x, const float *offset, const float *mask,
                             const void *grad_out, void *grad_x, float *grad_offset,
                             float *grad_mask, void *workspace, size_t workspace_bytes,
                             int N, int H, int W, int G, int C, int kh, int kw,
                             int stride_h, int stride_w, int pad_h, int pad_w,
                             int dil_h, int dil_w, float offset_scale, int softmax,
                             dcn_dtype dtype, hipStream_t stream);

/*
 * Workspace bytes dcn_v2_forward and dcn_v2_im2col need for these sizes (0 if they
 * are invalid). Layout (256-byte aligned regions, in this order): x transposed to
 * channels-last [N][H][W][Cin_pad], the weight permuted to [Cout_pad][Rp] (entry
 * k*Cin_pad + ci, tap-major; in the packed order of dcn_v2_pack_weight when the columns
 * are formed on chip) and the deform-im2col columns [P_pad][Rp], one row per output
 * pixel p = (n*Ho + ho)*Wo + wo with column k*Cin_pad + ci. Cin_pad = Cin rounded up
 * to 8, Rp = K*Cin_pad rounded up to 64, Cout_pad = Cout rounded up to 128, P_pad =
 * N*Ho*Wo rounded up to 128; padding entries are zero.
 */
size_t dcn_v2_workspace_bytes(int N, int Cin, int H, int W, int Cout, int kh, int kw,
                              int stride_h, int stride_w, int pad_h, int pad_w,
                              int dil_h, int dil_w, dcn_dtype dtype);

/*
 * DCNv2 modulated deformable convolution (DCNv1 when mask == NULL), NCHW.
 *
 *   x        [N, Cin, H, W]                 dtype (DCN_F16 or DCN_BF16)
 *   offset   [N, dg*K*2, Ho, Wo]            fp32; channel (g*K + k)*2 is dx, +1 is dy
 *   mask     [N, dg*K, Ho, Wo]              fp32 (post-sigmoid modulation) or NULL;
 *                                           logits when softmax != 0 (softmax over K
 *                                           per deformable group)
 *   weight   [Cout, Cin, kh, kw]            dtype
 *   out      [N, Cout, Ho, Wo]              dtype, fp32 accumulation, no bias
 *   workspace, workspace_bytes              >= dcn_v2_workspace_bytes(...), 256-B aligned
 *
 * out[n,co,ho,wo] = sum_{ci,k} weight[co,ci,k] * m_k * bilinear(x[n,ci], pos_k), channel ci
 * using deformable group ci / (Cin/dg). The sampled columns are rounded to dtype before
 * the MFMA contraction. Limits: K <= 64, dg divides Cin (and Cin/dg is a multiple of 8
 * when dg > 1). When Cin is a multiple of 64 the columns are formed on chip inside the
 * GEMM and never written (the workspace's column region is then left untouched);
 * otherwise they pass through the workspace.
 */
dcn_status dcn_v2_forward(const void *x, const float *offset, const float *mask,
                          const void *weight, void *out, void *workspace, size_t workspace_bytes,
                          int N, int Cin, int H, int W, int Cout, int kh, int kw,
                          int stride_h, int stride_w, int pad_h, int pad_w,
                          int dil_h, int dil_w, int deform_groups, int softmax,
                          dcn_dtype dtype, hipStream_t stream);

/*
 * The deform-im2col stage of dcn_v2_forward on its own (same arguments without weight
 * and out; Cout only fixes the workspace layout): writes x channels-last and the
 * columns col[p][k*Cin_pad + ci] = m_k(p) * bilinear(x[n,ci], pos_k(p)), rounded to
 * dtype, into their workspace regions. Same validation and errors as dcn_v2_forward.
 */
dcn_status dcn_v2_im2col(const void *x, const float *offset, const float *mask, void *workspace,
                         size_t workspace_bytes, int N, int Cin, int H, int W, int Cout, int kh,
                         int kw, int stride_h, int stride_w, int pad_h, int pad_w, int dil_h,
                         int dil_w, int deform_groups, int softmax, dcn_dtype dtype,
                         hipStream_t stream);

/*
 * dcn_v2_forward for callers that cannot allocate device memory or pass a workspace:
 * code being captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments and results as dcn_v2_forward, without workspace and
 * workspace_bytes; it allocates nothing (no hipMalloc, hipFree or allocating library
 * call). Its workspace is a static device array of DCN_V2_NOALLOC_SCRATCH_BYTES
 * (64 MiB) inside the library, one per GPU, which that GPU holds from the library's
 * first use there until the process ends. A call needing more than that
 * (dcn_v2_noalloc_bytes) returns DCN_ERR_SCRATCH before any HIP call; the shapes that
 * form their columns on chip need only the channels-last x and the permuted weight
 * (7.7 MB for 8x256x40x40 with Cout 256). Every call on one GPU uses the same array:
 * calls that may overlap on one GPU (several host threads, or several streams without
 * ordering between them) race and must be serialised by the caller. The first call on
 * a device looks up the array's address there (hipGetDevice, hipGetSymbolAddress);
 * later calls only launch.
 */
#define DCN_V2_NOALLOC_SCRATCH_BYTES (64u << 20)
size_t dcn_v2_noalloc_bytes(int N, int Cin, int H, int W, int Cout, int kh, int kw,
                            int stride_h, int stride_w, int pad_h, int pad_w,
                            int dil_h, int dil_w, int deform_groups, dcn_dtype dtype);
dcn_status dcn_v2_forward_noalloc(const void *x, const float *offset, const float *mask,
                                  const void *weight, void *out, int N, int Cin, int H, int W,
                                  int Cout, int kh, int kw, int stride_h, int stride_w,
                                  int pad_h, int pad_w, int dil_h, int dil_w, int deform_groups,
                                  int softmax, dcn_dtype dtype, hipStream_t stream);

/*
 * The weight of dcn_v2_forward permuted once, for layers whose weight does not change
 * between calls (inference): dcn_v2_forward_prepacked then skips that step of every
 * call. Only for layers that form their columns on chip (Cin a multiple of 64; see
 * dcn_v2_forward).
 *
 *   dcn_v2_packed_weight_bytes(Cout, Cin, kh, kw)  bytes of the packed weight
 *       (Cout_pad * Rp * 2, as in dcn_v2_workspace_bytes), 0 if the sizes are invalid.
 *   dcn_v2_pack_weight: weight [Cout, Cin, kh, kw] (dtype DCN_F16 or DCN_BF16) ->
 *       packed, a caller-owned device buffer of packed_bytes >= that size, 16-byte
 *       aligned (DCN_ERR_WORKSPACE if smaller, DCN_ERR_ALIGN if not aligned). Layout:
 *       the value weight[co, ci, k] has K index r = k*Cin_pad + ci; the eight values of
 *       (co, r0..r0+7), r0 = 16 q + 8 h, sit at 16-byte slot
 *       ((co/32 * Rp/16 + q) * 2 + h) * 32 + co%32, so the operand of one 32x32x16 MFMA
 *       (32 output channels x 16 K values) is 1 KB of consecutive memory. Padding
 *       entries are zero.
 *   dcn_v2_forward_prepacked: dcn_v2_forward with packed_weight/packed_bytes (made by
 *       dcn_v2_pack_weight for the same Cout, Cin, kh, kw and dtype) in place of
 *       weight; same other arguments, validation and errors, plus DCN_ERR_PARAM when
 *       the layer does not form its columns on chip and DCN_ERR_WORKSPACE when
 *       packed_bytes is too small. Results are bit-identical to dcn_v2_forward. The
 *       workspace's weight region is not used.
 */
size_t dcn_v2_packed_weight_bytes(int Cout, int Cin, int kh, int kw);
dcn_status dcn_v2_pack_weight(const void *weight, void *packed, size_t packed_bytes, int Cout, int Cin,
                              int kh, int kw, dcn_dtype dtype, hipStream_t stream);
dcn_status dcn_v2_forward_prepacked(const void *x, const float *offset, const float *mask,
                                    const void *packed_weight, size_t packed_bytes, void *out,
                                    void *workspace, size_t workspace_bytes, int N, int Cin, int H,
                                    int W, int Cout, int kh, int kw, int stride_h, int stride_w,
                                    int pad_h, int pad_w, int dil_h, int dil_w, int deform_groups,
                                    int softmax, dcn_dtype dtype, hipStream_t stream);

/*
 * Workspace bytes dcn_v2_backward needs (0 if the sizes are invalid). Regions, each
 * 256-byte aligned: x channels-last, the weight transposed, grad_out channels-last
 * and pixel-major, the forward's columns transposed (dtype); the column gradient
 * [N*Ho*Wo][K*Cin_pad] and split partial sums of the weight gradient (fp32); bucket
 * counters and entries of the grad_x gather.
 */
size_t dcn_v2_backward_workspace_bytes(int N, int Cin, int H, int W, int Cout, int kh, int kw,
                                       int stride_h, int stride_w, int pad_h, int pad_w,
                                       int dil_h, int dil_w, int deform_groups, dcn_dtype dtype);

/*
 * Gradients of dcn_v2_forward (the derivative of the modulated deformable
 * convolution of "DCNv2 in YOLOv5" (cyqw.cn), section 1, with the bilinear kernel of
 * "Hands-on DCNv1 in PyTorch", section 2; the pages print no backward pass).
 * Inputs as dcn_v2_forward, plus
 *   grad_out     [N, Cout, Ho, Wo]        dtype
 * Outputs (any may be NULL to skip it; each is fully overwritten):
 *   grad_x       [N, Cin, H, W]           dtype (fp32 accumulation, one rounding)
 *   grad_offset  [N, dg*K*2, Ho, Wo]      fp32
 *   grad_mask    [N, dg*K, Ho, Wo]        fp32, w.r.t. the mask argument (the logits
 *                                         with softmax); with mask == NULL w.r.t. the
 *                                         implied modulation (ones; zero logits)
 *   grad_weight  [Cout, Cin, kh, kw]      fp32
 * grad_weight contracts grad_out with the columns as the forward forms them (rounded
 * to dtype); the column gradient sum_co weight * grad_out is kept in fp32 for the
 * sampling derivative. At an integer position the derivative w.r.t. the offset is
 * taken from the cell floor() selects. grad_x sums its contributions in an order set
 * by atomic bucket filling, so its last bits may differ between runs. Limits as
 * dcn_v2_forward, and N*Ho*Wo*dg*K*4 < 2^31.
 */
dcn_status dcn_v2_backward(const void *x, const float *offset, const float *mask,
                           const void *weight, const void *grad_out, void *grad_x,
                           float *grad_offset, float *grad_mask, float *grad_weight,
                           void *workspace, size_t workspace_bytes, int N, int Cin, int H, int W,
                           int Cout, int kh, int kw, int stride_h, int stride_w, int pad_h,
                           int pad_w, int dil_h, int dil_w, int deform_groups, int softmax,
                           dcn_dtype dtype, hipStream_t stream);

/*
 * Multi-camera, multi-scale deformable aggregation (Sparse4D).
 *
 *   feat           [B, P_total, G*Cg]          dtype, all maps flattened (rows = pixels)
 *   spatial_shape  HOST int32 [cams, scales, 2] (H_s, W_s) of map (cam, s)
 *   scale_start    HOST int32 [cams, scales]    first row of map (cam, s) in feat
 *   loc            [B, A, pts, cams, 2]         fp32 (u, v) normalised to the camera image
 *   weights        [B, A, pts, cams, scales, G] fp32 (logits when softmax != 0)
 *   out            [B, A, G*Cg]                 dtype
 *
 * out[b,a,g*Cg+c] = sum over (p, cam, s) of w[b,a,p,cam,s,g] *
 *   bilinear(map_{cam,s}[:, :, g*Cg+c], y, x) with x = fl32(u*W_s) - 0.5 and
 *   y = fl32(v*H_s) - 0.5 (pixel centres at (i + 1/2)/W_s). With softmax != 0 the
 *   weights of (b, a, g) are softmax-normalised over all pts*cams*scales taps.
 * The two small host arrays are copied by value into the launch; they need not
 * outlive the call. Limits: cams*scales <= 64; every map must satisfy
 * scale_start + H_s*W_s <= P_total; B*P_total*G*Cg < 2^31 elements.
 */
dcn_status deform_agg_forward(const void *feat, const int32_t *spatial_shape,
                              const int32_t *scale_start, const float *loc,
                              const float *weights, void *out,
                              int B, int P_total, int A, int pts, int cams, int scales,
                              int G, int Cg, int softmax, dcn_dtype dtype, hipStream_t stream);

/* Human-readable name of a status code (static string). */
const char *dcn_status_string(dcn_status s);

/*
 * Workspace bytes deform_agg_backward needs (0 if the sizes are invalid), each region
 * 256-byte aligned: per-group partial sums of grad_loc (G*B*A*pts*cams*2 floats); the
 * per-sample sums g_t of grad_weights (B*A*T*G floats, T = pts*cams*scales) and three
 * floats per (anchor, group) (3*G*B*A: softmax maximum, 1/sum, sum of wt g_t); then
 * the feature-gradient buckets: the normalised weights (B*A*T*G floats), per-feature-row
 * counts and fill cursors (2*B*P_total uint32), their
 * starts (B*P_total uint32), the scan's block sums (one uint32 per 4096 rows) and one
 * 8-byte entry per sample corner (B*A*T*4). Where
 * the entries would reach 2^31 the buckets are replaced by fp32 atomic adds, and
 * fp16/bf16 then need an fp32 grad_feat accumulator (B*P_total*G*Cg floats) instead.
 */
size_t deform_agg_backward_workspace_bytes(int B, int P_total, int A, int pts, int cams,
                                           int scales, int G, int Cg, dcn_dtype dtype);

/*
 * Backward of deform_agg_forward (same arguments): the gradients of its output
 * w.r.t. the features, the sampling locations and the weights ("Sparse4D
 * deformable_aggregation", section 2.1, names these three; the spatial shapes and
 * scale starts have none). The pages give no formulas; these are the derivatives:
 *
 *   grad_out      [B, A, G*Cg]                 dtype
 *   grad_feat     [B, P_total, G*Cg]           dtype, overwritten (rows outside every
 *                                              map get 0), or NULL
 *   grad_loc      [B, A, pts, cams, 2]         fp32, overwritten, or NULL
 *   grad_weights  [B, A, pts, cams, scales, G] fp32 w.r.t. the weights argument (the
 *                                              logits when softmax != 0), or NULL
 *
 * With wt the (normalised) weight of sample t at x = fl32(u*W_s) - 0.5,
 * y = fl32(v*H_s) - 0.5, w_ab its bilinear weights and B_t, dB_t/dx, dB_t/dy the
 * sample and its derivatives in the pixel position (from the right at integer
 * positions): grad_feat[corner] += wt * w_ab * grad_out; grad_w_t = sum_c
 * grad_out[c] B_t[c] (softmax: wt (grad_w_t - sum_j wj grad_w_j)); grad_u =
 * sum over scales and groups of wt * W_s * sum_c grad_out[c] dB_t/dx[c], grad_v
 * likewise with H_s and dB_t/dy. grad_feat is gathered per feature row from
 * buckets of sample corners and summed in fp32 (the order within a bucket follows
 * an atomic fill, so its rounding varies run to run within fp32 accumulation
 * error), then rounded once to dtype; grad_loc and grad_weights are deterministic.
 * workspace: deform_agg_backward_workspace_bytes bytes, 256-byte aligned, needed
 * when grad_loc != NULL or grad_feat != NULL (with the atomic fallback: grad_feat
 * in fp16/bf16), else may be NULL (grad_weights alone then takes a slower kernel,
 * whose results may differ in the last bits from a call with a workspace);
 * contents on entry are ignored. Limits as the forward, and Cg <= 512. With A == 0
 * and grad_feat != NULL the call writes zeros to grad_feat (the one exception to
 * "zero-sized work launches nothing").
 */
dcn_status deform_agg_backward(const void *feat, const int32_t *spatial_shape,
                               const int32_t *scale_start, const float *loc, const float *weights,
                               const void *grad_out, void *grad_feat, float *grad_loc,
                               float *grad_weights, void *workspace, size_t workspace_bytes, int B,
                               int P_total, int A, int pts, int cams, int scales, int G, int Cg,
                               int softmax, dcn_dtype dtype, hipStream_t stream);

/*
 * Deformable RoI pooling ("Hands-on DCNv1 in PyTorch", section 3: per-bin offsets
 * normalised by the RoI size, dp_ij = gamma * dp^_ij o (w, h); bilinear sampling;
 * pooling), channels-last:
 *
 *   x       [N, H, W, C]   dtype
 *   rois    [R, 5]         fp32 (batch index, x1, y1, x2, y2) in input coordinates
 *   offset  [R, k, k, 2]   fp32 normalised (dx, dy) per bin, x first, or NULL (none)
 *   out     [R, k, k, C]   dtype
 *
 * With x1s = x1*spatial_scale, w = (x2 - x1)*spatial_scale (y likewise), bin (i, j)
 * is the mean of S x S bilinear samples (S = sampling_ratio) at
 *   y = y1s + (i + (sy + 1/2)/S) * h/k + gamma*dy_ij*h,
 *   x = x1s + (j + (sx + 1/2)/S) * w/k + gamma*dx_ij*w,
 * pixel q at integer coordinate q, zero outside the image per corner (the page names
 * no sampling grid, coordinate convention or border rule; these are the readings).
 * Positions are this fixed sequence of fp32 operations, each rounded once to nearest
 * even and none fused with another: x1s = fl(x1*s), w = fl(fl(x2 - x1)*s),
 * bw = fl(w/k), dx = fl(fl(gamma*dx^)*w), tx = fl((2(j*S + sx) + 1) / (2S)),
 * x = fl(fl(x1s + fl(tx*bw)) + dx), y likewise. A RoI whose batch index is not in
 * [0, N) pools to zeros. Limits: 1 <= sampling_ratio <= 64; (H+1)*(W+1)*C < 2^31; R*k*k*C < 2^31.
 * offset must be 8-byte aligned; x and out aligned to their element size.
 */
dcn_status deform_roi_pool_forward(const void *x, const float *rois, const float *offset, void *out,
                                   int N, int H, int W, int C, int R, int k, int sampling_ratio,
                                   float spatial_scale, float gamma, dcn_dtype dtype,
                                   hipStream_t stream);

/*
 * Alternative kernel paths of the two backward passes. dcn_core_backward and
 * deform_agg_backward pick their kernels from the sizes alone; the *_path entry
 * points below take that choice as an argument, so that every path can be run and
 * checked at any size (each computes the same gradients, within fp32 accumulation
 * error). Flags may be combined; a flag that does not apply to an entry point is
 * ignored by it. Nothing else selects these paths: the library reads no environment
 * variable and keeps no setting between calls.
 *   DCN_BWD_ATOMIC            grad_x (core) / grad_feat (aggregation) by fp32 atomic
 *                             adds, the path taken past the sorting limits; the
 *                             workspace size changes with it (use the matching
 *                             *_workspace_bytes_path call)
 *   DCN_BWD_PAIR_PASS         core: grad_offset / grad_mask from the per-pair pass with
 *                             direct corner loads instead of the LDS halo tiles
 *   DCN_BWD_PAIR_PASS_RECORDS core: the grad_x records filed by the per-pair pass even
 *                             where the tiled gradient kernel could file them
 *   DCN_BWD_UNSTAGED_GATHER   core: the grad_x gather reads each record's grad_out
 *                             slice from memory instead of through LDS
 *   DCN_BWD_GENERAL_MAIN      aggregation: the general per-sample kernel instead of
 *                             the pipelined one
 * An unknown flag bit gives DCN_ERR_PARAM (the workspace-size calls return 0).
 */
typedef enum {
    DCN_BWD_DEFAULT = 0,
    DCN_BWD_ATOMIC = 1,
    DCN_BWD_PAIR_PASS = 2,
    DCN_BWD_PAIR_PASS_RECORDS = 4,
    DCN_BWD_UNSTAGED_GATHER = 8,
    DCN_BWD_GENERAL_MAIN = 16
} dcn_bwd_path;

size_t dcn_core_backward_workspace_bytes_path(int N, int H, int W, int G, int C, int kh, int kw,
                                              int stride_h, int stride_w, int pad_h, int pad_w,
                                              int dil_h, int dil_w, dcn_dtype dtype,
                                              unsigned path);
dcn_status dcn_core_backward_path(const void *x, const float *offset, const float *mask,
                                  const void *grad_out, void *grad_x, float *grad_offset,
                                  float *grad_mask, void *workspace, size_t workspace_bytes,
                                  int N, int H, int W, int G, int C, int kh, int kw,
                                  int stride_h, int stride_w, int pad_h, int pad_w,
                                  int dil_h, int dil_w, float offset_scale, int softmax,
                                  dcn_dtype dtype, unsigned path, hipStream_t stream);
size_t deform_agg_backward_workspace_bytes_path(int B, int P_total, int A, int pts, int cams,
                                                int scales, int G, int Cg, dcn_dtype dtype,
                                                unsigned path);
dcn_status deform_agg_backward_path(const void *feat, const int32_t *spatial_shape,
                                    const int32_t *scale_start, const float *loc,
                                    const float *weights, const void *grad_out, void *grad_feat,
                                    float *grad_loc, float *grad_weights, void *workspace,
                                    size_t workspace_bytes, int B, int P_total, int A, int pts,
                                    int cams, int scales, int G, int Cg, int softmax,
                                    dcn_dtype dtype, unsigned path, hipStream_t stream);

/*
 * Measurement probe, not part of any operation: `blocks` blocks of 256 threads each run
 * `iters` rounds of four dense bf16 MFMAs (v_mfma_f32_32x32x16_bf16, 32768 flops each)
 * per wavefront on register operands, with no memory traffic, and write one float per
 * thread to sink [blocks*256] (device, fp32). Timed by the caller, it gives the
 * sustained MFMA rate the DCNv2 contraction is compared with beside the published peak:
 * flops = blocks * 4 waves * iters * 4 * 32768.
 */
dcn_status dcn_mfma_probe(float *sink, int blocks, int iters, hipStream_t stream);

/* hipError_t of this thread's last DCN_ERR_HIP (0 if none). */
int dcn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DCN_H_ */
