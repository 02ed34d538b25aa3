/*
 * ipa.h -- C ABI of the fused invariant point attention (IPA) forward pass
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (one call = one forward over a batch) follows
 *   - "Flash Invariant Point Attention" (arXiv 2505.11580), TL;DR and
 *     abstract: IPA over scalar, point and pair channels with a factorised
 *     pair representation z_ij = sum_r z1_ir * z2_jr, lifted into one
 *     softmax attention so that no L x L tensor is stored (linear memory);
 *   - MEET ("Scalable peptide design with memory-efficient equivariant
 *     transformers"), section 2.2, eq. 6-8: a squared point distance in the
 *     logit is carried by augmented query and key columns;
 *   - "Geometric direction-and-distance attention" (BioTorch), Required
 *     behavior: frame convention (rotation maps local column vectors to the
 *     global frame, translation is the origin), an edge is allowed when both
 *     frames are valid, all-masked rows return exact zeros, and inputs are
 *     never modified.
 *
 * Per head h, residues i (query) and j (key), with global points
 * x_g = R x + t:
 *   S_ijh  = w_L * ( q_ih.k_jh / sqrt(C) + sum_c Z_ijc W_b[c,h]
 *                    - gamma_h * w_C / 2 * sum_p |T_i q_ihp - T_j k_jhp|^2 )
 *   a_ijh  = softmax over allowed j
 *   out_s[b,i,h,:]        = sum_j a v_jh
 *   out_pts[b,i,h,p,:]    = R_i^T ( sum_j a (R_j v_jhp + t_j) - t_i )
 *   out_pts_norm[b,i,h,p] = |out_pts[b,i,h,p,:]|        (no epsilon)
 *   out_pair[b,i,h,:]     = sum_j a Z_ij,  Z_ij = sum_r z1_ir * z2_jr
 * Rows whose own mask entry is 0 get +0.0 in every output.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers, row-major and contiguous in
 *     the shapes given below. They are owned by the caller; the library keeps
 *     no reference after the call returns and never writes its inputs.
 *   - Returns IPA_OK (0) or a negative status; see ipa_status_string().
 *     Every argument is validated before anything is launched: on a negative
 *     status nothing was written.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream). The library allocates no device memory: scratch space
 *     is the caller's `workspace`, sized by ipa_workspace_bytes(), except
 *     for ipa_forward_noalloc, whose workspace is a fixed static array.
 *   - Reentrant; no global mutable state apart from ipa_forward_noalloc's
 *     static workspace. Calls that share a workspace must be ordered on one
 *     stream.
 */
#ifndef IPA_MI355_H
#define IPA_MI355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Problem dimensions.
 *   B   batch size                    L   (padded) residues per batch element
 *   H   heads                         C   scalar channels per head
 *   Pqk query/key points per head     Pv  value points per head
 *   R   rank of the factorised pair   Cz  pair channels
 * Supported envelope: every dim >= 1, C <= 16, Pqk <= 5, Pv <= 8,
 * Cz % 8 == 0, Cz <= 128, R * Cz <= 256 (bf16) or <= 128 (fp32),
 * L <= 65536, B * H * L < 2^31. Other shapes return IPA_ERR_UNSUPPORTED. */
typedef struct {
  int32_t B, L, H, C, Pqk, Pv, R, Cz;
} ipa_dims;

/* Storage type of q, k, v, q_pts, k_pts, v_pts, z1, z2.
 * IPA_F32: float32 storage, float32 arithmetic throughout.
 * IPA_BF16: bfloat16 storage, matrix-core products with float32
 * accumulation:
 *   - scalar and point columns of Q.K^T and all of P.V: bf16 products
 *     (point coordinates centred per 64-residue block and carried as bf16
 *     hi/lo pairs; their norms and block offsets stay float32);
 *   - pair columns of Q.K^T: fp16 products of z2 and of the per-head query
 *     operand w_L log2(e) W_b[c,h] z1[c] (rounded to nearest). Range: both
 *     must lie within +-65504 (fp16's finite range) or they saturate there
 *     and the logits are no longer those of the definition; magnitudes
 *     below 2^-14 are fp16 subnormals and keep an absolute precision of
 *     2^-24. Ordinary normalised pair factors sit far inside it.
 * Frames, w_b, gamma and every output are float32 for both. */
typedef enum { IPA_F32 = 0, IPA_BF16 = 1 } ipa_dtype;

enum {
  IPA_OK = 0,
  IPA_ERR_NULL = -1,        /* a required pointer is NULL                   */
  IPA_ERR_DIMS = -2,        /* a dimension is < 1 or too large              */
  IPA_ERR_DTYPE = -3,       /* dtype is not an ipa_dtype value              */
  IPA_ERR_WORKSPACE = -4,   /* workspace_bytes < ipa_workspace_bytes(...)   */
  IPA_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned             */
  IPA_ERR_UNSUPPORTED = -6, /* dims outside the supported envelope          */
  IPA_ERR_HIP = -7,         /* a HIP launch failed                          */
  IPA_ERR_ARG = -8,         /* a scalar argument is not finite / negative   */
  IPA_ERR_LIMIT = -9        /* ipa_forward_noalloc: the dims need more than
                               IPA_NOALLOC_WORKSPACE_BYTES of workspace      */
};

/* Bytes of device workspace that ipa_forward needs for these dims and dtype.
 * Linear in B*L (no L x L term). Returns 0 if the dims are invalid or
 * unsupported. */
size_t ipa_workspace_bytes(const ipa_dims* dims, int32_t dtype);

/* Fused IPA forward.
 *   q, k, v   [B,L,H,C]        dtype storage
 *   q_pts     [B,L,H,Pqk,3]    local query points, dtype storage
 *   k_pts     [B,L,H,Pqk,3]    local key points, dtype storage
 *   v_pts     [B,L,H,Pv,3]     local value points, dtype storage
 *   rot       [B,L,3,3] float32, rot[b,l] maps local column vectors to global
 *   trans     [B,L,3]   float32, global origin of each frame
 *   z1, z2    [B,L,R,Cz]       pair factors, dtype storage
 *   w_b       [Cz,H]    float32, pair-bias projection
 *   gamma     [H]       float32, point weight per head (already positive)
 *   mask      [B,L]     uint8, 1 = valid residue; NULL = all valid. An edge
 *                       (i,j) is used when both mask entries are 1.
 *   w_L, w_C  logit weights (finite, >= 0); the usual values are sqrt(1/3)
 *             and sqrt(2 / (9 Pqk)).
 *   out_s        [B,L,H,C]      float32
 *   out_pts      [B,L,H,Pv,3]   float32
 *   out_pts_norm [B,L,H,Pv]     float32
 *   out_pair     [B,L,H,Cz]     float32
 *   workspace    device scratch of at least ipa_workspace_bytes(dims, dtype)
 *                bytes, 256-byte aligned; its contents on entry are ignored.
 *   stream       hipStream_t to enqueue on.
 * Every output element is overwritten. Padded rows may hold any finite
 * values in every input; they never influence valid rows. */
int32_t ipa_forward(const ipa_dims* dims, int32_t dtype,
                    const void* q, const void* k, const void* v,
                    const void* q_pts, const void* k_pts, const void* v_pts,
                    const float* rot, const float* trans,
                    const void* z1, const void* z2,
                    const float* w_b, const float* gamma,
                    const uint8_t* mask,
                    float w_L, float w_C,
                    float* out_s, float* out_pts, float* out_pts_norm,
                    float* out_pair,
                    void* workspace, size_t workspace_bytes,
                    void* stream);

/* The two stages of ipa_forward, for callers that time or schedule them
 * separately. ipa_lift applies the frames and writes the lifted query/key/
 * value operands into `workspace`; ipa_attend runs the fused attention and
 * the output epilogue from that workspace. ipa_attend must follow an
 * ipa_lift with identical arguments on the same stream (or after it has
 * completed); ipa_lift + ipa_attend is exactly ipa_forward. Arguments,
 * validation and status codes are those of ipa_forward. */
int32_t ipa_lift(const ipa_dims* dims, int32_t dtype,
                 const void* q, const void* k, const void* v,
                 const void* q_pts, const void* k_pts, const void* v_pts,
                 const float* rot, const float* trans,
                 const void* z1, const void* z2,
                 const float* w_b, const float* gamma,
                 const uint8_t* mask,
                 float w_L, float w_C,
                 float* out_s, float* out_pts, float* out_pts_norm,
                 float* out_pair,
                 void* workspace, size_t workspace_bytes,
                 void* stream);
int32_t ipa_attend(const ipa_dims* dims, int32_t dtype,
                   const void* q, const void* k, const void* v,
                   const void* q_pts, const void* k_pts, const void* v_pts,
                   const float* rot, const float* trans,
                   const void* z1, const void* z2,
                   const float* w_b, const float* gamma,
                   const uint8_t* mask,
                   float w_L, float w_C,
                   float* out_s, float* out_pts, float* out_pts_norm,
                   float* out_pair,
                   void* workspace, size_t workspace_bytes,
                   void* stream);

/* Size of the static device workspace of ipa_forward_noalloc: 64 MiB, one
 * copy on each GPU the library runs on, held until the process ends. It
 * covers ipa_workspace_bytes() up to, for example, B*L = 8192 residues with
 * H = 12, C = 16, Pqk = 4, Pv = 8, R = 2, Cz = 128 in bf16 (48.5 MiB). */
#define IPA_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)

/* ipa_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. It allocates nothing (no
 * hipMalloc, no hipFree, no allocating library routine); its workspace is a
 * file-scope device array of IPA_NOALLOC_WORKSPACE_BYTES bytes in the
 * library, whose address is looked up once per GPU, on the first call made
 * with that GPU current.
 * Arguments, layouts, results and status codes are ipa_forward's (the same
 * kernels run), plus IPA_ERR_LIMIT, returned before anything is enqueued
 * when ipa_workspace_bytes(dims, dtype) exceeds IPA_NOALLOC_WORKSPACE_BYTES,
 * and IPA_ERR_HIP if the array's address cannot be obtained. `stream` must
 * belong to the calling thread's current device.
 * Every call on one GPU shares that GPU's array, and the array keeps the
 * last call's contents (nothing in it needs clearing: all that the
 * attention reads is written by the same call's lift). Calls ordered on
 * one stream are safe; calls that overlap on one GPU (different streams, or
 * threads without ordering between them) race on the array and their
 * results are undefined. */
int32_t ipa_forward_noalloc(const ipa_dims* dims, int32_t dtype,
                            const void* q, const void* k, const void* v,
                            const void* q_pts, const void* k_pts, const void* v_pts,
                            const float* rot, const float* trans,
                            const void* z1, const void* z2,
                            const float* w_b, const float* gamma,
                            const uint8_t* mask,
                            float w_L, float w_C,
                            float* out_s, float* out_pts, float* out_pts_norm,
                            float* out_pair,
                            void* stream);

/* Residue frames from backbone atoms.
 * "Flash Invariant Point Attention", Figure 1: the C-alpha atom is the
 * centre of a residue's frame, the vectors from C-alpha to N and to C span
 * it, and Gram-Schmidt completes it. Here
 *   e1 = (C - CA) / |C - CA|
 *   e2 = unit component of (N - CA) orthogonal to e1
 *   e3 = e1 x e2                      (right-handed)
 *   rot_out = [e1 e2 e3] (the axes as columns: local -> global), trans_out = CA,
 * the `rot` / `trans` convention of ipa_forward.
 *   n, ca, c    [B,L,3]   float32 atom positions
 *   rot_out     [B,L,3,3] float32
 *   trans_out   [B,L,3]   float32
 * Pointers must be non-NULL and 4-byte aligned; B, L >= 1 and B*L < 2^31.
 * Residues whose C coincides with C-alpha, or whose N lies on the
 * C-alpha -> C line, have no frame: their outputs are not finite. */
int32_t ipa_frames_from_atoms(int32_t B, int32_t L, const float* n, const float* ca,
                              const float* c, float* rot_out, float* trans_out,
                              void* stream);

/* Distance-penalised attention over one point per residue.
 * MEET ("Scalable peptide design with memory-efficient equivariant
 * transformers"), section 2.2, eq. 6-8: per head h,
 *   S_ijh = rho_h * ( q_ih . k_jh - s_h^2 * |x_i - x_j|^2 )
 *   a_ijh = softmax over allowed j,   out[b,i,h,:] = sum_j a v_jh.
 * It runs on the IPA kernels as a configuration of ipa_forward's logit:
 * identity frames at the points x, one zero local point per head, no pair
 * term, scalar weight rho_h in place of w_L / sqrt(C) and point weight
 * rho_h * s_h^2 in place of w_L * gamma_h * w_C / 2. Masks, padding and
 * status codes behave as in ipa_forward.
 *   dims      B, L, H, C (every dim >= 1, C <= 16, L <= 65536)
 *   q, k, v   [B,L,H,C] dtype storage
 *   x         [B,L,3]   float32 points in one global frame
 *   rho, s    [H]       float32 per-head weights (finite)
 *   mask      [B,L]     uint8, 1 = valid residue; NULL = all valid
 *   out       [B,L,H,C] float32, every element overwritten
 *   workspace ipa_meet_workspace_bytes(dims, dtype) bytes, 256-byte aligned.
 * Tensor pointers must be 16-byte aligned. */
typedef struct {
  int32_t B, L, H, C;
} ipa_meet_dims;
size_t ipa_meet_workspace_bytes(const ipa_meet_dims* dims, int32_t dtype);
int32_t ipa_meet_forward(const ipa_meet_dims* dims, int32_t dtype,
                         const void* q, const void* k, const void* v,
                         const float* x, const float* rho, const float* s,
                         const uint8_t* mask, float* out,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/* The full IPA layer around ipa_forward.
 * Reading taken (the pages fix the attention, not its wrap; "Flash
 * Invariant Point Attention", TL;DR and abstract: per-residue scalar,
 * point and factorised pair features feed it): one affine map of the
 * single representation s gives every input feature,
 *   x = s W_in + b_in = [q | k | v | q_pts | k_pts | v_pts | z1 | z2]
 * (blocks flattened head-major: q [H,C], q_pts [H,Pqk,3], z1 [R,Cz], ...),
 * the features are stored in `dtype` (bf16: round to nearest even), the
 * attention runs as ipa_forward, and its outputs are read out as
 *   out = [o_s | o_pts | o_norm | o_pair] W_out + b_out
 * flattened head-major with xyz last; rows whose mask entry is 0 give +0.0.
 *   dims, dtype   as ipa_forward;  c_s >= 1 the width of s and out
 *   s      [B,L,c_s] float32      rot, trans, mask, w_b, gamma, w_L, w_C as ipa_forward
 *   w_in   [c_s, 3HC + 6HPqk + 3HPv + 2RCz] float32, b_in [..] or NULL
 *   w_out  [H(C + 3Pv + Pv + Cz), c_s] float32, b_out [c_s] or NULL
 *   out    [B,L,c_s] float32, every element overwritten
 *   workspace ipa_layer_workspace_bytes(dims, c_s, dtype) bytes, 256-byte aligned
 * Pointers 16-byte aligned. The projections and the readout run on the
 * matrix cores: fp32 products for IPA_F32; for IPA_BF16 (features rounded
 * to bf16 anyway) each fp32 operand split into bf16 hi + lo, three bf16
 * products, about 2^-17 relative per term. The attention's envelope and
 * statuses are those of ipa_forward. */
size_t ipa_layer_workspace_bytes(const ipa_dims* dims, int32_t c_s, int32_t dtype);
int32_t ipa_layer_forward(const ipa_dims* dims, int32_t c_s, int32_t dtype,
                          const float* s, const float* rot, const float* trans,
                          const uint8_t* mask,
                          const float* w_in, const float* b_in,
                          const float* w_b, const float* gamma, float w_L, float w_C,
                          const float* w_out, const float* b_out,
                          float* out,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/* Gradient of ipa_forward (float32 path).
 * Training goes through this attention ("Flash Invariant Point Attention",
 * abstract: training at previously unattainable lengths). For output
 * cotangents g_s, g_pts, g_pts_norm, g_pair this returns the gradient of
 *   sum <g_s, out_s> + <g_pts, out_pts> + <g_pts_norm, out_pts_norm> + <g_pair, out_pair>
 * with respect to every input of ipa_forward, computed on the lifted rows
 * one chunk of query rows at a time (the chunk's scores, at most 2^26
 * floats per buffer, are the only quadratic-size data):
 *   inputs        as ipa_forward (IPA_F32 storage only), mask may be NULL
 *   out_s, out_pts, out_pair   the forward's outputs for these inputs
 *   g_*           cotangents, shaped like the outputs
 *   dq, dk, dv [B,L,H,C]; dq_pts, dk_pts [B,L,H,Pqk,3]; dv_pts [B,L,H,Pv,3];
 *   drot [B,L,3,3]; dtrans [B,L,3]; dz1, dz2 [B,L,R,Cz]; dw_b [Cz,H];
 *   dgamma [H]: every element overwritten (float32).
 * The derivative of |out_pts| at 0 is taken as 0. Rows whose mask entry is
 * 0 pass no gradient and receive none. Supported envelope: C <= 16,
 * Pqk <= 5, Pv <= 8, R*Cz <= 256, B*H <= 65535. Pointers 4-byte aligned,
 * workspace ipa_backward_workspace_bytes(dims) bytes, 256-byte aligned.
 * Products: the scores QA KA^T (lifted dot only), the two value-side
 * products (A z2 and A^T GA) and the scalar and pair columns of the query-
 * and key-side products split each fp32 operand into bf16 hi + lo and take
 * three bf16 products (about 2^-17 relative per term); dP = GA VA^T is
 * fp32-accurate (hi + mid + lo, six bf16 products, or fp32 products where
 * the operands' alignment does not allow the copies the split kernel
 * uses); the point columns of the query- and key-side products, which
 * cancel, use fp32 products. Deterministic: repeated calls give identical
 * bits. */
size_t ipa_backward_workspace_bytes(const ipa_dims* dims);
int32_t ipa_backward(const ipa_dims* dims,
                     const float* q, const float* k, const float* v,
                     const float* q_pts, const float* k_pts, const float* v_pts,
                     const float* rot, const float* trans,
                     const float* z1, const float* z2,
                     const float* w_b, const float* gamma,
                     const uint8_t* mask, float w_L, float w_C,
                     const float* out_s, const float* out_pts, const float* out_pair,
                     const float* g_s, const float* g_pts, const float* g_pts_norm,
                     const float* g_pair,
                     float* dq, float* dk, float* dv,
                     float* dq_pts, float* dk_pts, float* dv_pts,
                     float* drot, float* dtrans, float* dz1, float* dz2,
                     float* dw_b, float* dgamma,
                     void* workspace, size_t workspace_bytes,
                     void* stream);

/* Gradient of ipa_forward in flash form: the same result as ipa_backward,
 * with scores, probabilities and their derivative formed tile by tile and
 * never stored, so the workspace is linear in L ("Flash Invariant Point
 * Attention", abstract: training at lengths that quadratic memory rules out;
 * TL;DR: linear memory).
 *   dtype         storage of q, k, v, q_pts, k_pts, v_pts, z1, z2: IPA_F32
 *                 (4-byte aligned) or IPA_BF16 (2-byte aligned); rot, trans,
 *                 w_b, gamma, the outputs, the cotangents and every gradient
 *                 are float32 (4-byte aligned)
 *   other arguments as ipa_backward; workspace
 *   ipa_backward_flash_workspace_bytes(dims) bytes (linear in B L H),
 *   256-byte aligned.
 * Two passes over bf16 lifted rows: a query pass (online softmax; dq side,
 * the row statistics) and a key pass (dk, dv side). Products: the lifted
 * dot, the scalar and pair parts of dP and the accumulating products take
 * one bf16 product per term (probabilities and dS rounded to bf16), fp32
 * accumulation; the point part of dP takes bf16 hi + lo splits (three
 * products, about 2^-17 relative); the distance term and every sum against
 * the points run in float32 from explicit differences. Accuracy is that of
 * the bf16 forward, not of ipa_backward. Same envelope and statuses as
 * ipa_backward, plus IPA_ERR_DTYPE. Deterministic. */
size_t ipa_backward_flash_workspace_bytes(const ipa_dims* dims);
int32_t ipa_backward_flash(const ipa_dims* dims, int32_t dtype,
                           const void* q, const void* k, const void* v,
                           const void* q_pts, const void* k_pts, const void* v_pts,
                           const float* rot, const float* trans,
                           const void* z1, const void* z2,
                           const float* w_b, const float* gamma,
                           const uint8_t* mask, float w_L, float w_C,
                           const float* out_s, const float* out_pts, const float* out_pair,
                           const float* g_s, const float* g_pts, const float* g_pts_norm,
                           const float* g_pair,
                           float* dq, float* dk, float* dv,
                           float* dq_pts, float* dk_pts, float* dv_pts,
                           float* drot, float* dtrans, float* dz1, float* dz2,
                           float* dw_b, float* dgamma,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/* Geometric direction-and-distance attention (ESM3-style).
 * "Geometric direction-and-distance attention" (BioTorch), Required
 * behavior. Per batch b, head h, query i and key j, with frames (R, t) that
 * map local column vectors to the global frame:
 *   qd_i = R_i q_direction_i,          kd_j = R_j k_direction_j
 *   qp_i = R_i q_point_i + t_i,        kp_j = R_j k_point_j + t_j
 *   a_ijh = ( softplus(direction_scale_h) (qd_i . kd_j)
 *             - softplus(distance_scale_h) |qp_i - kp_j| ) / sqrt(3)
 *   (the distance itself, not squared, no epsilon; softplus stable)
 *   allowed_ijh = frame_mask_i and frame_mask_j and pair_mask[b,h,i,j]
 *   A_ijh = softmax over allowed j; a query with no allowed key gets 0
 *   vectors[b,i,h,m,:] = R_i^T sum_j A_ijh R_j values[b,j,h,m,:]  (no translation)
 *   output[b,i,:] = flatten_{h,m,xyz}(vectors[b,i]) @ output_weight + output_bias,
 *                   +0.0 when no head of query i has an allowed key.
 * Arithmetic is float32 throughout; memory is linear in N unless the
 * attention matrix is requested.
 *   dims            B, N, H, M, Cout (every dim >= 1, M <= 8, N <= 2^24, Cout <= 65536,
 *                   B*H <= 65535, B*N*H*3*M < 2^31, B*N*Cout < 2^31,
 *                   3*H*M*Cout < 2^29)
 *   rot             [B,N,3,3] float32 (proper rotations on valid frames)
 *   trans           [B,N,3]   float32
 *   q_direction, k_direction, q_point, k_point  [B,N,H,3] float32
 *   values          [B,N,H,M,3] float32
 *   direction_scale, distance_scale  [H] float32 raw (pre-softplus) logits
 *   output_weight   [3*H*M, Cout] float32; output_bias [Cout] or NULL
 *   frame_mask      [B,N] uint8, 1 = valid frame (required)
 *   pair_mask       uint8 or NULL (every edge allowed); element (b,h,i,j) is
 *                   pair_mask[b*s0 + h*s1 + i*s2 + j*s3] with
 *                   pair_mask_strides = {s0,s1,s2,s3} (>= 0; 0 broadcasts)
 *   vectors         [B,N,H,M,3] float32, every element overwritten
 *   output          [B,N,Cout]  float32, every element overwritten
 *   attention       [B,H,N,N]   float32 or NULL (not computed); O(N^2) bytes
 *   workspace       ipa_dirdist_workspace_bytes(dims) bytes, 256-byte aligned
 * Float pointers must be 4-byte aligned. Invalid frames may hold any finite
 * values; they are never read past the mask. Returns IPA_ERR_UNSUPPORTED
 * for dims outside the envelope (ipa_dirdist_workspace_bytes then returns
 * 0) and IPA_ERR_ARG for a negative stride. */
typedef struct {
  int32_t B, N, H, M, Cout;
} ipa_dirdist_dims;
size_t ipa_dirdist_workspace_bytes(const ipa_dirdist_dims* dims);
int32_t ipa_dirdist_forward(const ipa_dirdist_dims* dims,
                            const float* rot, const float* trans,
                            const float* q_direction, const float* k_direction,
                            const float* q_point, const float* k_point,
                            const float* values,
                            const float* direction_scale, const float* distance_scale,
                            const float* output_weight, const float* output_bias,
                            const uint8_t* frame_mask,
                            const uint8_t* pair_mask, const int64_t* pair_mask_strides,
                            float* vectors, float* output, float* attention,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/* Static, NUL-terminated description of a status code. */
const char* ipa_status_string(int32_t status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t ipa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* IPA_MI355_H */
