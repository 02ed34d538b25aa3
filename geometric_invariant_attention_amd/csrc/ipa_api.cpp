// Host side of the C ABI declared in include/ipa.h: argument validation,
// workspace layout and the two launches (lift, fused attention) on the
// caller's stream. Nothing is launched unless every check passes.

#include "../../include/ipa.h"
#include "ipa_internal.h"

#include <cmath>
#include <cstdint>

namespace ipa {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool make_layout(const int32_t d[8], int esize, Layout* o) {
  const int64_t B = d[0], L = d[1], H = d[2], C = d[3], Pqk = d[4], Pv = d[5], R = d[6], Cz = d[7];
  if (B < 1 || L < 1 || H < 1 || C < 1 || Pqk < 1 || Pv < 1 || R < 1 || Cz < 1) return false;
  if (C > kCSlot || Pv > kPvSlot || kCSlot + 9 * Pqk > kHeadW) return false;
  if (Cz % 8 != 0 || Cz > 128 || R * Cz > kMaxD - kHeadW) return false;
  const int64_t Lp = (L + kTileM - 1) / kTileM * kTileM;
  if (Lp / kTileN > kMaxTiles) return false;
  if (B * H * Lp >= (int64_t(1) << 31) || B * L * R * Cz >= (int64_t(1) << 31)) return false;
  const int64_t PW = (R * Cz + 63) / 64 * 64;
  Layout& ly = *o;
  ly.B = (int)B; ly.L = (int)L; ly.H = (int)H; ly.C = (int)C; ly.Pqk = (int)Pqk;
  ly.Pv = (int)Pv; ly.R = (int)R; ly.Cz = (int)Cz;
  ly.Lp = (int)Lp; ly.nJ = (int)(Lp / kTileN); ly.PW = (int)PW; ly.D = (int)(kHeadW + PW);
  ly.esize = esize;
  if (esize == 4 && ly.D > kMaxDF32) return false;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = align256(off + bytes); return at; };
  const size_t es = (size_t)esize;
  ly.off_qh = take((size_t)B * H * Lp * kHeadW * es);
  ly.off_kh = take((size_t)B * H * Lp * kHeadW * es);
  ly.off_kz = take((size_t)B * ly.nJ * PW * kTileN * es);
  ly.off_vth = take((size_t)B * H * ly.nJ * kHeadW * kTileN * es);
  ly.off_vtz = take((size_t)B * ly.nJ * PW * kTileN * es);
  ly.off_kcol = take((size_t)B * H * Lp * 16);
  ly.off_qrow = take((size_t)B * H * Lp * 16);
  ly.off_cen = take((size_t)B * ly.nJ * 16);
  ly.off_pdiag = take((size_t)B * H * Lp * 16);
  ly.total = off;
  return true;
}

}  // namespace ipa

namespace {

bool valid_dims_struct(const ipa_dims* d, int32_t out[8]) {
  if (!d) return false;
  out[0] = d->B; out[1] = d->L; out[2] = d->H; out[3] = d->C;
  out[4] = d->Pqk; out[5] = d->Pv; out[6] = d->R; out[7] = d->Cz;
  return true;
}

bool basic_dims_ok(const int32_t v[8]) {
  for (int e = 0; e < 8; ++e)
    if (v[e] < 1) return false;
  return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

namespace {

enum Stage { kLift = 1, kAttend = 2, kBoth = 3 };

int32_t run(int stages, const ipa_dims* dims, int32_t dtype,
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
            void* stream, const long long* out_pitch = nullptr) {
  int32_t dv[8];
  if (!valid_dims_struct(dims, dv)) return IPA_ERR_NULL;
  if (!basic_dims_ok(dv)) return IPA_ERR_DIMS;
  if (dtype != IPA_F32 && dtype != IPA_BF16) return IPA_ERR_DTYPE;
  const void* req[] = {q, k, v, q_pts, k_pts, v_pts, rot, trans, z1, z2, w_b, gamma,
                       out_s, out_pts, out_pts_norm, out_pair, workspace};
  for (const void* p : req)
    if (!p) return IPA_ERR_NULL;
  for (const void* p : req)
    if (!aligned16(p)) return IPA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return IPA_ERR_ALIGN;
  if (!std::isfinite(w_L) || !std::isfinite(w_C) || w_L < 0.f || w_C < 0.f) return IPA_ERR_ARG;

  ipa::FwdArgs a;
  const bool bf16 = dtype == IPA_BF16;
  if (!ipa::make_layout(dv, bf16 ? 2 : 4, &a.lay)) return IPA_ERR_UNSUPPORTED;
  if (workspace_bytes < a.lay.total) return IPA_ERR_WORKSPACE;

  a.q = q; a.k = k; a.v = v; a.q_pts = q_pts; a.k_pts = k_pts; a.v_pts = v_pts;
  a.rot = rot; a.trans = trans; a.z1 = z1; a.z2 = z2; a.w_b = w_b; a.gamma = gamma;
  a.mask = mask; a.w_L = w_L; a.w_C = w_C;
  a.out_s = out_s; a.out_pts = out_pts; a.out_pts_norm = out_pts_norm; a.out_pair = out_pair;
  const long long H = dims->H;
  const long long packed[4] = {H * dims->C, 3 * H * dims->Pv, H * dims->Pv, H * dims->Cz};
  for (int e = 0; e < 4; ++e) a.out_pitch[e] = out_pitch ? out_pitch[e] : packed[e];
  a.ws = static_cast<unsigned char*>(workspace);
  a.meet_rho = nullptr; a.meet_s = nullptr;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((stages & kLift) && ipa::launch_lift(a, bf16, s) != hipSuccess) return IPA_ERR_HIP;
  if ((stages & kAttend) && ipa::launch_attn(a, bf16, s) != hipSuccess) return IPA_ERR_HIP;
  return IPA_OK;
}

}  // namespace

extern "C" {

size_t ipa_workspace_bytes(const ipa_dims* dims, int32_t dtype) {
  int32_t v[8];
  if (!valid_dims_struct(dims, v) || !basic_dims_ok(v)) return 0;
  if (dtype != IPA_F32 && dtype != IPA_BF16) return 0;
  ipa::Layout ly;
  if (!ipa::make_layout(v, dtype == IPA_BF16 ? 2 : 4, &ly)) return 0;
  return ly.total;
}

#define IPA_ARGS_DECL                                                               \
  const ipa_dims *dims, int32_t dtype, const void *q, const void *k, const void *v, \
      const void *q_pts, const void *k_pts, const void *v_pts, const float *rot,     \
      const float *trans, const void *z1, const void *z2, const float *w_b,          \
      const float *gamma, const uint8_t *mask, float w_L, float w_C, float *out_s,   \
      float *out_pts, float *out_pts_norm, float *out_pair, void *workspace,         \
      size_t workspace_bytes, void *stream
#define IPA_ARGS_PASS                                                                \
  dims, dtype, q, k, v, q_pts, k_pts, v_pts, rot, trans, z1, z2, w_b, gamma, mask,   \
      w_L, w_C, out_s, out_pts, out_pts_norm, out_pair, workspace, workspace_bytes, stream

int32_t ipa_forward(IPA_ARGS_DECL) { return run(kBoth, IPA_ARGS_PASS); }
int32_t ipa_lift(IPA_ARGS_DECL) { return run(kLift, IPA_ARGS_PASS); }
int32_t ipa_attend(IPA_ARGS_DECL) { return run(kAttend, IPA_ARGS_PASS); }

int32_t ipa_frames_from_atoms(int32_t B, int32_t L, const float* n, const float* ca, const float* c,
                              float* rot_out, float* trans_out, void* stream) {
  if (B < 1 || L < 1 || (int64_t)B * L >= (int64_t(1) << 31)) return IPA_ERR_DIMS;
  const void* req[] = {n, ca, c, rot_out, trans_out};
  for (const void* p : req)
    if (!p) return IPA_ERR_NULL;
  for (const void* p : req)
    if ((reinterpret_cast<uintptr_t>(p) & 3u) != 0) return IPA_ERR_ALIGN;
  if (ipa::launch_frames(B * L, n, ca, c, rot_out, trans_out, static_cast<hipStream_t>(stream)) != hipSuccess)
    return IPA_ERR_HIP;
  return IPA_OK;
}

// The distance attention runs on the IPA kernels with one (zero) local
// point per head for queries, keys and values and one all-zero pair panel.
static bool meet_ipa_dims(const ipa_meet_dims* d, int32_t out[8]) {
  if (!d) return false;
  out[0] = d->B; out[1] = d->L; out[2] = d->H; out[3] = d->C;
  out[4] = 1; out[5] = 1; out[6] = 1; out[7] = 32;
  return true;
}

size_t ipa_meet_workspace_bytes(const ipa_meet_dims* dims, int32_t dtype) {
  int32_t v[8];
  if (!meet_ipa_dims(dims, v) || !basic_dims_ok(v)) return 0;
  if (dtype != IPA_F32 && dtype != IPA_BF16) return 0;
  ipa::Layout ly;
  if (!ipa::make_layout(v, dtype == IPA_BF16 ? 2 : 4, &ly)) return 0;
  return ly.total;
}

int32_t ipa_meet_forward(const ipa_meet_dims* dims, int32_t dtype, const void* q, const void* k,
                         const void* v, const float* x, const float* rho, const float* s,
                         const uint8_t* mask, float* out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  int32_t dv[8];
  if (!meet_ipa_dims(dims, dv)) return IPA_ERR_NULL;
  if (!basic_dims_ok(dv)) return IPA_ERR_DIMS;
  if (dtype != IPA_F32 && dtype != IPA_BF16) return IPA_ERR_DTYPE;
  const void* req[] = {q, k, v, x, rho, s, out, workspace};
  for (const void* p : req)
    if (!p) return IPA_ERR_NULL;
  for (const void* p : req)
    if (!aligned16(p)) return IPA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return IPA_ERR_ALIGN;

  ipa::FwdArgs a;
  const bool bf16 = dtype == IPA_BF16;
  if (!ipa::make_layout(dv, bf16 ? 2 : 4, &a.lay)) return IPA_ERR_UNSUPPORTED;
  if (workspace_bytes < a.lay.total) return IPA_ERR_WORKSPACE;
  a.q = q; a.k = k; a.v = v;
  a.q_pts = nullptr; a.k_pts = nullptr; a.v_pts = nullptr;
  a.rot = nullptr; a.trans = x; a.z1 = nullptr; a.z2 = nullptr; a.w_b = nullptr; a.gamma = nullptr;
  a.mask = mask; a.w_L = 0.f; a.w_C = 0.f;
  a.out_s = out; a.out_pts = nullptr; a.out_pts_norm = nullptr; a.out_pair = nullptr;
  a.out_pitch[0] = (long long)dims->H * dims->C;
  a.out_pitch[1] = a.out_pitch[2] = a.out_pitch[3] = 0;
  a.ws = static_cast<unsigned char*>(workspace);
  a.meet_rho = rho; a.meet_s = s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (ipa::launch_lift(a, bf16, st) != hipSuccess) return IPA_ERR_HIP;
  if (ipa::launch_attn(a, bf16, st) != hipSuccess) return IPA_ERR_HIP;
  return IPA_OK;
}

}  // extern "C"

namespace {

struct DDLayout {
  size_t off_q, off_klog, off_kval, off_part, off_stats, total;
  int Np, PW, splits;
};

bool dd_layout(const ipa_dirdist_dims* d, DDLayout* o) {
  if (!d) return false;
  const int64_t B = d->B, N = d->N, H = d->H, M = d->M, Cout = d->Cout;
  if (B < 1 || N < 1 || H < 1 || M < 1 || Cout < 1) return false;
  if (M > ipa::kDDMaxM || N > (1 << 24) || H > 65535 || Cout > 65536) return false;
  if (B * N * H >= (int64_t(1) << 31) || B * N * Cout >= (int64_t(1) << 31) ||
      B * N * 3 * H * M >= (int64_t(1) << 31) || B * H > 65535 ||
      3 * H * M * Cout >= (int64_t(1) << 29))
    return false;
  o->Np = ipa::dd_padded_keys((int)N);
  o->PW = ipa::dd_part_width((int)M);
  o->splits = ipa::dd_splits((int)B, (int)N, (int)H);
  if (B * o->splits > 65535) return false;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = ipa::align256(off + bytes); return at; };
  o->off_q = take((size_t)B * H * o->Np * 8 * 4);
  o->off_klog = take((size_t)B * H * o->Np * ipa::kKeyLog * 4);
  o->off_kval = take((size_t)B * H * o->Np * ipa::kValW * 4);
  o->off_part = take((size_t)o->splits * B * N * H * o->PW * 4);
  o->off_stats = take((size_t)B * H * N * 8);
  o->total = off;
  return true;
}

}  // namespace

extern "C" {

size_t ipa_dirdist_workspace_bytes(const ipa_dirdist_dims* dims) {
  DDLayout ly;
  return dd_layout(dims, &ly) ? ly.total : 0;
}

int32_t ipa_dirdist_forward(const ipa_dirdist_dims* dims, const float* rot, const float* trans,
                            const float* q_direction, const float* k_direction,
                            const float* q_point, const float* k_point, const float* values,
                            const float* direction_scale, const float* distance_scale,
                            const float* output_weight, const float* output_bias,
                            const uint8_t* frame_mask, const uint8_t* pair_mask,
                            const int64_t* pair_mask_strides, float* vectors, float* output,
                            float* attention, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!dims) return IPA_ERR_NULL;
  if (dims->B < 1 || dims->N < 1 || dims->H < 1 || dims->M < 1 || dims->Cout < 1) return IPA_ERR_DIMS;
  const float* fin[] = {rot, trans, q_direction, k_direction, q_point, k_point, values,
                        direction_scale, distance_scale, output_weight};
  for (const float* p : fin)
    if (!p) return IPA_ERR_NULL;
  if (!frame_mask || !vectors || !output || !workspace) return IPA_ERR_NULL;
  if (pair_mask && !pair_mask_strides) return IPA_ERR_NULL;
  const void* al[] = {rot, trans, q_direction, k_direction, q_point, k_point, values,
                      direction_scale, distance_scale, output_weight, output_bias, vectors,
                      output, attention};
  for (const void* p : al)
    if ((reinterpret_cast<uintptr_t>(p) & 3u) != 0) return IPA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return IPA_ERR_ALIGN;
  DDLayout ly;
  if (!dd_layout(dims, &ly)) return IPA_ERR_UNSUPPORTED;
  if (workspace_bytes < ly.total) return IPA_ERR_WORKSPACE;
  ipa::DDArgs a{};
  if (pair_mask) {
    for (int e = 0; e < 4; ++e)
      if (pair_mask_strides[e] < 0) return IPA_ERR_ARG;
    a.pm_sb = pair_mask_strides[0]; a.pm_sh = pair_mask_strides[1];
    a.pm_si = pair_mask_strides[2]; a.pm_sj = pair_mask_strides[3];
  }
  a.B = dims->B; a.N = dims->N; a.H = dims->H; a.M = dims->M; a.Cout = dims->Cout;
  a.Np = ly.Np; a.PW = ly.PW; a.splits = ly.splits;
  a.rot = rot; a.trans = trans; a.q_direction = q_direction; a.k_direction = k_direction;
  a.q_point = q_point; a.k_point = k_point; a.values = values;
  a.direction_scale = direction_scale; a.distance_scale = distance_scale;
  a.w_out = output_weight; a.b_out = output_bias;
  a.frame_mask = frame_mask; a.pair_mask = pair_mask;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  a.qbuf = reinterpret_cast<float*>(ws + ly.off_q);
  a.klog = reinterpret_cast<float*>(ws + ly.off_klog);
  a.kval = reinterpret_cast<float*>(ws + ly.off_kval);
  a.part = reinterpret_cast<float*>(ws + ly.off_part);
  a.stats = reinterpret_cast<float*>(ws + ly.off_stats);
  a.vectors = vectors; a.output = output; a.attention = attention;
  if (ipa::launch_dirdist(a, static_cast<hipStream_t>(stream)) != hipSuccess) return IPA_ERR_HIP;
  return IPA_OK;
}

}  // extern "C"

namespace {

struct BwdLayout {
  size_t off[18];
  size_t total;
  int QC;
};

// query rows per chunk: the two score buffers hold at most 2^26 floats each
int bwd_chunk(int64_t BH, int64_t L) {
  int64_t qc = (int64_t(1) << 26) / (BH * L);
  if (qc >= L) return (int)L;
  qc = qc / 64 * 64;
  return (int)(qc < 64 ? 64 : qc);
}

bool bwd_layout(const ipa_dims* d, BwdLayout* o) {
  if (!d) return false;
  const int64_t B = d->B, L = d->L, H = d->H, C = d->C, P = d->Pqk, Pv = d->Pv, R = d->R, Cz = d->Cz;
  if (B < 1 || L < 1 || H < 1 || C < 1 || P < 1 || Pv < 1 || R < 1 || Cz < 1) return false;
  if (C > 16 || P > 5 || Pv > 8 || R * Cz > 256) return false;
  if (B * H > 65535 || B * L * H * 296 >= (int64_t(1) << 31) || B * L * (Cz * H + H) >= (int64_t(1) << 31))
    return false;
  const int QC = bwd_chunk(B * H, L);
  if (B * H * (int64_t)QC * L >= (int64_t(1) << 31)) return false;
  o->QC = QC;
  const size_t rows = (size_t)(B * H * L), DA = (size_t)(C + R * Cz), DV = (size_t)(C + 3 * Pv + R * Cz);
  // lifted rows padded to a multiple of 4 floats (16-byte aligned rows)
  const size_t P3 = (size_t)(3 * P), DAQ = (DA + P3 + 4) & ~(size_t)3, DAK = (DA + P3 + 3) & ~(size_t)3,
               xs = (size_t)(B * H) * QC * L;
  const size_t sizes[18] = {rows * DAQ, rows * DAK, rows * DV, rows * DV, rows * P3, rows * P3, rows,
                            rows * DAK, rows * R * Cz, rows, rows,
                            rows * DAQ, rows * DV,
                            (size_t)(B * L * H) * 12, (size_t)(B * L) * (size_t)(Cz * H + H), xs, xs,
                            (size_t)((B * L + 127) / 128) * (size_t)(Cz * H + H)};
  size_t off = 0;
  for (int e = 0; e < 18; ++e) {
    o->off[e] = off;
    off = ipa::align256(off + sizes[e] * 4);
  }
  o->total = off;
  return true;
}

struct BwdfLayout {
  size_t off[17];
  size_t total;
  int WQ, WG;
};

// flash form: every buffer is linear in B L H (no score rows)
bool bwdf_layout(const ipa_dims* d, BwdfLayout* o) {
  if (!d) return false;
  const int64_t B = d->B, L = d->L, H = d->H, C = d->C, P = d->Pqk, Pv = d->Pv, R = d->R, Cz = d->Cz;
  if (B < 1 || L < 1 || H < 1 || C < 1 || P < 1 || Pv < 1 || R < 1 || Cz < 1) return false;
  if (C > 16 || P > 5 || Pv > 8 || R * Cz > 256) return false;
  const int64_t WQ = (C + ((R * Cz + 31) & ~int64_t(31)) + 31) & ~int64_t(31);
  const int64_t WG = (C + 9 * Pv + R * Cz + 31) & ~int64_t(31);
  if (B * H > 65535 || B * L * H * WG >= (int64_t(1) << 31) || B * L * (Cz * H + H) >= (int64_t(1) << 31))
    return false;
  o->WQ = (int)WQ;
  o->WG = (int)WG;
  const size_t rows = (size_t)(B * H * L), DA = (size_t)(C + R * Cz), DV = (size_t)(C + 3 * Pv + R * Cz);
  const size_t P3 = (size_t)(3 * P), DAQ = (DA + P3 + 4) & ~(size_t)3, DAK = (DA + P3 + 3) & ~(size_t)3;
  // bytes of: QX, KX, GX, VX (bf16), QP, KP, Dv, ST, dQA, U, gam, rsum, dKA, dVA, fpart, share, red1
  const size_t sizes[17] = {rows * WQ * 2, rows * WQ * 2, rows * WG * 2, rows * WG * 2,
                            rows * P3 * 4, rows * P3 * 4, rows * 4, rows * 8,
                            rows * DAK * 4, rows * R * Cz * 4, rows * 4, rows * 4,
                            rows * DAQ * 4, rows * DV * 4,
                            (size_t)(B * L * H) * 12 * 4, (size_t)(B * L) * (size_t)(Cz * H + H) * 4,
                            (size_t)((B * L + 127) / 128) * (size_t)(Cz * H + H) * 4};
  size_t off = 0;
  for (int e = 0; e < 17; ++e) {
    o->off[e] = off;
    off = ipa::align256(off + sizes[e]);
  }
  o->total = off;
  return true;
}

}  // namespace

extern "C" {

size_t ipa_backward_flash_workspace_bytes(const ipa_dims* dims) {
  BwdfLayout ly;
  return bwdf_layout(dims, &ly) ? ly.total : 0;
}

int32_t ipa_backward_flash(const ipa_dims* dims, int32_t dtype, const void* q, const void* k, const void* v,
                           const void* q_pts, const void* k_pts, const void* v_pts,
                           const float* rot, const float* trans, const void* z1, const void* z2,
                           const float* w_b, const float* gamma, const uint8_t* mask, float w_L, float w_C,
                           const float* out_s, const float* out_pts, const float* out_pair,
                           const float* g_s, const float* g_pts, const float* g_pts_norm, const float* g_pair,
                           float* dq, float* dk, float* dv, float* dq_pts, float* dk_pts, float* dv_pts,
                           float* drot, float* dtrans, float* dz1, float* dz2, float* dw_b, float* dgamma,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!dims) return IPA_ERR_NULL;
  if (dims->B < 1 || dims->L < 1 || dims->H < 1 || dims->C < 1 || dims->Pqk < 1 || dims->Pv < 1 ||
      dims->R < 1 || dims->Cz < 1)
    return IPA_ERR_DIMS;
  if (dtype != IPA_F32 && dtype != IPA_BF16) return IPA_ERR_DTYPE;
  const uintptr_t in_align = dtype == IPA_BF16 ? 1u : 3u;
  const void* ins[] = {q, k, v, q_pts, k_pts, v_pts, z1, z2};
  for (const void* p : ins) {
    if (!p) return IPA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(p) & in_align) != 0) return IPA_ERR_ALIGN;
  }
  const void* ptrs[] = {rot, trans, w_b, gamma, out_s, out_pts, out_pair, g_s, g_pts, g_pts_norm, g_pair,
                        dq, dk, dv, dq_pts, dk_pts, dv_pts, drot, dtrans, dz1, dz2, dw_b, dgamma, workspace};
  for (const void* p : ptrs) {
    if (!p) return IPA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(p) & 3u) != 0) return IPA_ERR_ALIGN;
  }
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return IPA_ERR_ALIGN;
  if (!std::isfinite(w_L) || !std::isfinite(w_C) || w_L < 0.f || w_C < 0.f) return IPA_ERR_ARG;
  BwdfLayout ly;
  if (!bwdf_layout(dims, &ly)) return IPA_ERR_UNSUPPORTED;
  if (workspace_bytes < ly.total) return IPA_ERR_WORKSPACE;
  ipa::BwdArgs a{};
  a.B = dims->B; a.L = dims->L; a.H = dims->H; a.C = dims->C; a.Pqk = dims->Pqk; a.Pv = dims->Pv;
  a.R = dims->R; a.Cz = dims->Cz;
  a.DA = a.C + a.R * a.Cz; a.DV = a.C + 3 * a.Pv + a.R * a.Cz; a.P3 = 3 * a.Pqk;
  a.DAQ = (a.DA + a.P3 + 4) & ~3; a.DAK = (a.DA + a.P3 + 3) & ~3; a.QC = a.L;
  a.WQ = ly.WQ; a.WG = ly.WG;
  a.w_L = w_L; a.w_C = w_C;
  a.in_bf16 = dtype == IPA_BF16;
  a.q = q; a.k = k; a.v = v; a.q_pts = q_pts; a.k_pts = k_pts; a.v_pts = v_pts;
  a.rot = rot; a.trans = trans; a.z1 = z1; a.z2 = z2; a.w_b = w_b; a.gamma = gamma; a.mask = mask;
  a.o_s = out_s; a.o_pts = out_pts; a.o_pair = out_pair;
  a.g_s = g_s; a.g_pts = g_pts; a.g_norm = g_pts_norm; a.g_pair = g_pair;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dq_pts = dq_pts; a.dk_pts = dk_pts; a.dv_pts = dv_pts;
  a.drot = drot; a.dtrans = dtrans; a.dz1 = dz1; a.dz2 = dz2; a.dw_b = dw_b; a.dgamma = dgamma;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  uint16_t** h16[4] = {&a.QX, &a.KX, &a.GX, &a.VX};
  for (int e = 0; e < 4; ++e) *h16[e] = reinterpret_cast<uint16_t*>(ws + ly.off[e]);
  float** f32s[13] = {&a.QP, &a.KP, &a.Dv, &a.ST, &a.dQA, &a.U, &a.gam, &a.rsum, &a.dKA, &a.dVA,
                      &a.fpart, &a.share, &a.red1};
  for (int e = 0; e < 13; ++e) *f32s[e] = reinterpret_cast<float*>(ws + ly.off[4 + e]);
  if (ipa::launch_backward_flash(a, static_cast<hipStream_t>(stream)) != hipSuccess) return IPA_ERR_HIP;
  return IPA_OK;
}

size_t ipa_backward_workspace_bytes(const ipa_dims* dims) {
  BwdLayout ly;
  return bwd_layout(dims, &ly) ? ly.total : 0;
}

int32_t ipa_backward(const ipa_dims* dims, const float* q, const float* k, const float* v,
                     const float* q_pts, const float* k_pts, const float* v_pts,
                     const float* rot, const float* trans, const float* z1, const float* z2,
                     const float* w_b, const float* gamma, const uint8_t* mask, float w_L, float w_C,
                     const float* out_s, const float* out_pts, const float* out_pair,
                     const float* g_s, const float* g_pts, const float* g_pts_norm, const float* g_pair,
                     float* dq, float* dk, float* dv, float* dq_pts, float* dk_pts, float* dv_pts,
                     float* drot, float* dtrans, float* dz1, float* dz2, float* dw_b, float* dgamma,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!dims) return IPA_ERR_NULL;
  if (dims->B < 1 || dims->L < 1 || dims->H < 1 || dims->C < 1 || dims->Pqk < 1 || dims->Pv < 1 ||
      dims->R < 1 || dims->Cz < 1)
    return IPA_ERR_DIMS;
  const void* ptrs[] = {q, k, v, q_pts, k_pts, v_pts, rot, trans, z1, z2, w_b, gamma,
                        out_s, out_pts, out_pair, g_s, g_pts, g_pts_norm, g_pair,
                        dq, dk, dv, dq_pts, dk_pts, dv_pts, drot, dtrans, dz1, dz2, dw_b, dgamma, workspace};
  for (const void* p : ptrs) {
    if (!p) return IPA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(p) & 3u) != 0) return IPA_ERR_ALIGN;
  }
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return IPA_ERR_ALIGN;
  if (!std::isfinite(w_L) || !std::isfinite(w_C) || w_L < 0.f || w_C < 0.f) return IPA_ERR_ARG;
  BwdLayout ly;
  if (!bwd_layout(dims, &ly)) return IPA_ERR_UNSUPPORTED;
  if (workspace_bytes < ly.total) return IPA_ERR_WORKSPACE;
  ipa::BwdArgs a{};
  a.B = dims->B; a.L = dims->L; a.H = dims->H; a.C = dims->C; a.Pqk = dims->Pqk; a.Pv = dims->Pv;
  a.R = dims->R; a.Cz = dims->Cz;
  a.DA = a.C + a.R * a.Cz; a.DV = a.C + 3 * a.Pv + a.R * a.Cz; a.P3 = 3 * a.Pqk;
  a.DAQ = (a.DA + a.P3 + 4) & ~3; a.DAK = (a.DA + a.P3 + 3) & ~3; a.QC = ly.QC;
  a.w_L = w_L; a.w_C = w_C;
  a.q = q; a.k = k; a.v = v; a.q_pts = q_pts; a.k_pts = k_pts; a.v_pts = v_pts;
  a.rot = rot; a.trans = trans; a.z1 = z1; a.z2 = z2; a.w_b = w_b; a.gamma = gamma; a.mask = mask;
  a.o_s = out_s; a.o_pts = out_pts; a.o_pair = out_pair;
  a.g_s = g_s; a.g_pts = g_pts; a.g_norm = g_pts_norm; a.g_pair = g_pair;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dq_pts = dq_pts; a.dk_pts = dk_pts; a.dv_pts = dv_pts;
  a.drot = drot; a.dtrans = dtrans; a.dz1 = dz1; a.dz2 = dz2; a.dw_b = dw_b; a.dgamma = dgamma;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float** slots[18] = {&a.QA, &a.KA, &a.VA, &a.GA, &a.QP, &a.KP, &a.Dv, &a.dQA, &a.U, &a.gam,
                       &a.rsum, &a.dKA, &a.dVA, &a.fpart, &a.share, &a.X, &a.Y, &a.red1};
  for (int e = 0; e < 18; ++e) *slots[e] = reinterpret_cast<float*>(ws + ly.off[e]);
  if (ipa::launch_backward(a, static_cast<hipStream_t>(stream)) != hipSuccess) return IPA_ERR_HIP;
  return IPA_OK;
}

}  // extern "C"

namespace {

// The full layer is three launches around the attention: x = s W_in + b_in
// as one GEMM whose epilogue writes each column block straight into the
// attention's input array in its storage type; the attention, which writes
// its four outputs as the column blocks of one row-major matrix (or, when a
// block would not start on a 16-byte boundary, into packed arrays followed
// by a gather); and
// y = [o_s | o_pts | o_norm | o_pair] W_out + b_out as one GEMM with the
// reduction split across the grid, the partials added in order with the
// bias by a second kernel that also zeroes masked rows.
struct LayerLayout {
  size_t off_feat[8], off_ipa, off_out[4], off_cat, off_part, total, ipa_bytes;
  int n_in, n_out, widths[8], splits;
};

bool layer_layout(const ipa_dims* d, int32_t c_s, int32_t dtype, LayerLayout* o) {
  if (!d || c_s < 1 || c_s > 65536) return false;
  if (dtype != IPA_F32 && dtype != IPA_BF16) return false;
  const size_t ipa_bytes = ipa_workspace_bytes(d, dtype);
  if (ipa_bytes == 0) return false;
  const int64_t B = d->B, L = d->L, H = d->H, C = d->C, P = d->Pqk, Pv = d->Pv, R = d->R, Cz = d->Cz;
  const int w[8] = {(int)(H * C), (int)(H * C), (int)(H * C), (int)(H * P * 3), (int)(H * P * 3),
                    (int)(H * Pv * 3), (int)(R * Cz), (int)(R * Cz)};
  int n_in = 0;
  for (int e = 0; e < 8; ++e) { o->widths[e] = w[e]; n_in += w[e]; }
  o->n_in = n_in;
  o->n_out = (int)(H * (C + 3 * Pv + Pv + Cz));
  const int64_t rows = B * L;
  if (rows * (int64_t)n_in >= (int64_t(1) << 31) || rows * (int64_t)c_s >= (int64_t(1) << 31) ||
      rows * (int64_t)o->n_out >= (int64_t(1) << 31))
    return false;
  // readout reduction slices: enough workgroups to fill the chip, >= 64 steps each
  const int64_t tiles = ((rows + 63) / 64) * ((c_s + 63) / 64);
  int sp = (int)((1024 + tiles - 1) / tiles);
  const int cap = (o->n_out + 63) / 64;
  o->splits = sp < 1 ? 1 : (sp > cap ? cap : sp);
  if (o->splits * rows * (int64_t)c_s >= (int64_t(1) << 31)) return false;
  const size_t es = dtype == IPA_BF16 ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = ipa::align256(off + bytes); return at; };
  for (int e = 0; e < 8; ++e) o->off_feat[e] = take((size_t)rows * w[e] * es);
  o->off_ipa = take(ipa_bytes);
  o->ipa_bytes = ipa_bytes;
  const size_t outw[4] = {(size_t)(H * C), (size_t)(H * Pv * 3), (size_t)(H * Pv), (size_t)(H * Cz)};
  for (int e = 0; e < 4; ++e) o->off_out[e] = take((size_t)rows * outw[e] * 4);
  o->off_cat = take((size_t)rows * o->n_out * 4);
  o->off_part = take((size_t)o->splits * rows * c_s * 4);
  o->total = off;
  return true;
}

}  // namespace

extern "C" {

size_t ipa_layer_workspace_bytes(const ipa_dims* dims, int32_t c_s, int32_t dtype) {
  LayerLayout ly;
  return layer_layout(dims, c_s, dtype, &ly) ? ly.total : 0;
}

int32_t ipa_layer_forward(const ipa_dims* dims, int32_t c_s, int32_t dtype, const float* s,
                          const float* rot, const float* trans, const uint8_t* mask,
                          const float* w_in, const float* b_in, const float* w_b, const float* gamma,
                          float w_L, float w_C, const float* w_out, const float* b_out, float* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!dims) return IPA_ERR_NULL;
  if (dims->B < 1 || dims->L < 1 || dims->H < 1 || dims->C < 1 || dims->Pqk < 1 || dims->Pv < 1 ||
      dims->R < 1 || dims->Cz < 1 || c_s < 1)
    return IPA_ERR_DIMS;
  if (dtype != IPA_F32 && dtype != IPA_BF16) return IPA_ERR_DTYPE;
  const void* req[] = {s, rot, trans, w_in, w_b, gamma, w_out, out, workspace};
  for (const void* p : req)
    if (!p) return IPA_ERR_NULL;
  const void* al[] = {s, rot, trans, w_in, b_in, w_b, gamma, w_out, b_out, out};
  for (const void* p : al)
    if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return IPA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return IPA_ERR_ALIGN;
  if (!std::isfinite(w_L) || !std::isfinite(w_C) || w_L < 0.f || w_C < 0.f) return IPA_ERR_ARG;
  LayerLayout ly;
  if (!layer_layout(dims, c_s, dtype, &ly)) return IPA_ERR_UNSUPPORTED;
  if (workspace_bytes < ly.total) return IPA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const long long rows = (long long)dims->B * dims->L;
  // x = s W_in + b_in, each column block written straight into the
  // attention's input array in its storage type
  void* feat[8];
  for (int e = 0; e < 8; ++e) feat[e] = ws + ly.off_feat[e];
  ipa::Gemm g{};
  g.M = (int)rows; g.N = ly.n_in; g.K = c_s;
  g.A = s; g.am = c_s; g.ak = 1;
  g.B = w_in; g.bk = ly.n_in; g.bn = 1;
  g.bias = b_in;
  g.nseg = 8; g.seg_bf16 = dtype == IPA_BF16;
  // with bf16 storage the features are rounded to 2^-9 anyway: the split
  // path (about 2^-17 per term) is ample; fp32 storage keeps fp32 products
  g.x3 = dtype == IPA_BF16;
  int c0 = 0;
  for (int e = 0; e < 8; ++e) {
    g.seg_start[e] = c0;
    c0 += ly.widths[e];
    g.seg_out[e] = feat[e];
  }
  g.seg_start[8] = c0;
  if (ipa::gemm(g, 1, st) != hipSuccess) return IPA_ERR_HIP;
  // the attention: its four outputs go straight into the columns of the
  // readout's left operand [rows][n_out] when every block starts on a
  // 16-byte boundary, else into packed arrays that a gather concatenates
  const int H = dims->H, C = dims->C, Pv = dims->Pv, Cz = dims->Cz;
  const int wo[4] = {H * C, H * Pv * 3, H * Pv, H * Cz};
  int start[5];
  start[0] = 0;
  for (int e = 0; e < 4; ++e) start[e + 1] = start[e] + wo[e];
  float* const cat = reinterpret_cast<float*>(ws + ly.off_cat);
  const bool direct = ly.n_out % 4 == 0 && start[1] % 4 == 0 && start[2] % 4 == 0 && start[3] % 4 == 0;
  if (direct) {
    const long long pitch[4] = {ly.n_out, ly.n_out, ly.n_out, ly.n_out};
    const int32_t rc = run(kBoth, dims, dtype, feat[0], feat[1], feat[2], feat[3], feat[4], feat[5], rot, trans,
                           feat[6], feat[7], w_b, gamma, mask, w_L, w_C, cat + start[0], cat + start[1],
                           cat + start[2], cat + start[3], ws + ly.off_ipa, ly.ipa_bytes, stream, pitch);
    if (rc != IPA_OK) return rc;
  } else {
    float* o[4];
    for (int e = 0; e < 4; ++e) o[e] = reinterpret_cast<float*>(ws + ly.off_out[e]);
    const int32_t rc = ipa_forward(dims, dtype, feat[0], feat[1], feat[2], feat[3], feat[4], feat[5], rot, trans,
                                   feat[6], feat[7], w_b, gamma, mask, w_L, w_C, o[0], o[1], o[2], o[3],
                                   ws + ly.off_ipa, ly.ipa_bytes, stream);
    if (rc != IPA_OK) return rc;
    ipa::LayerGather ga{};
    for (int e = 0; e < 4; ++e) {
      ga.src[e] = o[e];
      ga.start[e] = start[e];
    }
    ga.start[4] = start[4];
    ga.rows = rows; ga.n_out = ly.n_out;
    ga.cat = cat;
    if (ipa::launch_layer_gather(ga, st) != hipSuccess) return IPA_ERR_HIP;
  }
  // y = [o_s | o_pts | o_norm | o_pair] W_out + b_out, masked rows 0
  ipa::Gemm q{};
  q.M = (int)rows; q.N = c_s; q.K = ly.n_out;
  q.A = cat; q.am = ly.n_out; q.ak = 1;
  q.B = w_out; q.bk = c_s; q.bn = 1;
  q.C = out; q.cm = c_s; q.bias = b_out; q.rowmask = mask;
  q.x3 = dtype == IPA_BF16;
  if (ipa::gemm_splitk(q, ly.splits, reinterpret_cast<float*>(ws + ly.off_part), st) != hipSuccess) return IPA_ERR_HIP;
  return IPA_OK;
}

const char* ipa_status_string(int32_t status) {
  switch (status) {
    case IPA_OK: return "ok";
    case IPA_ERR_NULL: return "a required pointer is NULL";
    case IPA_ERR_DIMS: return "a dimension is < 1 or too large";
    case IPA_ERR_DTYPE: return "dtype must be IPA_F32 or IPA_BF16";
    case IPA_ERR_WORKSPACE: return "workspace is smaller than ipa_workspace_bytes()";
    case IPA_ERR_ALIGN: return "a pointer is not 16-byte aligned (workspace: 256-byte)";
    case IPA_ERR_UNSUPPORTED: return "dims outside the supported envelope";
    case IPA_ERR_HIP: return "a HIP kernel launch failed";
    case IPA_ERR_ARG: return "a scalar argument is out of range (w_L, w_C finite and >= 0; strides >= 0)";
    case IPA_ERR_LIMIT:
      return "the dims need more workspace than ipa_forward_noalloc's static array (IPA_NOALLOC_WORKSPACE_BYTES)";
    default: return "unknown status";
  }
}

int32_t ipa_version(void) { return 100; }

}  // extern "C"
