// Internal declarations shared by the host entry points and the HIP kernels
// of the fused IPA forward. Not part of the public ABI (include/ipa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ipa {

// Key tile of the attention kernel and the residue block whose mean
// translation centres the global points (the same 64 residues).
constexpr int kTileN = 64;
// Largest number of key tiles (L <= kMaxTiles * kTileN).
constexpr int kMaxTiles = 1024;
// Query rows per attention workgroup (4 waves x 32 rows).
constexpr int kTileM = 128;
// Width of the per-head part of a lifted row (scalar + point columns).
constexpr int kHeadW = 64;
// Largest supported lifted row width (head part + pair part).
constexpr int kMaxD = 320;
// Largest lifted row width of the float32 path.
constexpr int kMaxDF32 = 192;
// Scalar channels and value points are laid out in slots of these sizes.
constexpr int kCSlot = 16;
constexpr int kPvSlot = 8;
// fp32 path: first column of the unscaled centred query points in a query
// head row (key points start at kCSlot).
constexpr int kFpQPts = 32;
constexpr float kLog2e = 1.4426950408889634f;

// Byte layout of the caller-supplied workspace. Everything the attention
// kernel reads is produced here by the lift kernel; sizes are linear in
// B * L.
struct Layout {
  int B, L, H, C, Pqk, Pv, R, Cz;
  int Lp;     // L rounded up to kTileM
  int nJ;     // Lp / kTileN key tiles (= centring blocks)
  int D;      // lifted row width: kHeadW + PW
  int PW;     // pair part width: R * Cz rounded up to 64
  int esize;  // bytes per lifted element (2 bf16, 4 fp32)
  size_t off_qh;    // [B][H][Lp][kHeadW]        query head part
  size_t off_kh;    // [B][H][Lp][kHeadW]        key head part
  size_t off_kz;    // [B][nJ][PW/64][64][64]    key pair part (z2) in 64x64 panels, shared by heads
  size_t off_vth;   // [B][H][nJ][kHeadW][64]    value head part, feature-major
  size_t off_vtz;   // [B][nJ][PW][64]           value pair part (z2), feature-major
  size_t off_kcol;  // [B][H][Lp] float4         per-key column terms
  size_t off_qrow;  // [B][H][Lp] float4         per-query row terms (w: own-key head logit)
  size_t off_cen;   // [B][nJ] float4            block centre xyz, valid count
  size_t off_pdiag; // [B][H][Lp] float4        per-panel pair bias of the query's own key (seed)
  size_t total;
};

// Returns false if the dims are outside the supported envelope.
bool make_layout(const int32_t d[8], int esize, Layout* out);

struct FwdArgs {
  Layout lay;
  const void* q; const void* k; const void* v;
  const void* q_pts; const void* k_pts; const void* v_pts;
  const float* rot; const float* trans;
  const void* z1; const void* z2;
  const float* w_b; const float* gamma;
  const uint8_t* mask;
  float w_L, w_C;
  float* out_s; float* out_pts; float* out_pts_norm; float* out_pair;
  // floats between the outputs of consecutive residues (b, i) for o_s,
  // o_pts, o_norm, o_pair: H C, 3 H Pv, H Pv, H Cz when packed, wider when
  // the four are columns of one matrix (multiples of 4 there)
  long long out_pitch[4];
  unsigned char* ws;
  // Distance-attention configuration (both NULL for the IPA forward): per
  // head, scalar weight rho_h replaces w_L / sqrt(C) and point weight
  // rho_h s_h^2 replaces w_L gamma_h w_C / 2. In that configuration the
  // points, rotations, pair factors, W_b and all outputs but out_s may be
  // NULL: missing inputs read as zeros, missing outputs are not written.
  const float* meet_rho; const float* meet_s;
};

// Kernel launchers (return the hipError_t of the launch).
hipError_t launch_lift(const FwdArgs& a, bool bf16, hipStream_t s);
hipError_t launch_attn(const FwdArgs& a, bool bf16, hipStream_t s);
hipError_t launch_frames(int n, const float* atom_n, const float* atom_ca, const float* atom_c,
                         float* rot, float* trans, hipStream_t s);

// ---------------------------------------------------------------------------
// Direction-and-distance attention (ipa_dirdist.hip)
// ---------------------------------------------------------------------------
constexpr int kDDMaxM = 8;        // value vectors per head
constexpr int kMaxSplits = 16;    // key splits across workgroups
// floats per key: logit part (global direction, validity bias, global point,
// pad) and rotated-value part (3M values, zero padded to one 32-column block)
constexpr int kKeyLog = 8;
constexpr int kValW = 32;
// floats per partial row: running max, sum, 3M accumulators
constexpr int dd_part_width(int M) { return (2 + 3 * M + 3) / 4 * 4; }

struct DDArgs {
  int B, N, H, M, Cout;
  int Np;       // N rounded up to the key chunk
  int PW;       // dd_part_width(M)
  int splits;   // key splits across workgroups (1..kMaxSplits)
  const float* rot; const float* trans;
  const float* q_direction; const float* k_direction;
  const float* q_point; const float* k_point;
  const float* values;
  const float* direction_scale; const float* distance_scale;
  const float* w_out; const float* b_out;
  const uint8_t* frame_mask;
  const uint8_t* pair_mask;                  // NULL: every edge allowed
  long long pm_sb, pm_sh, pm_si, pm_sj;      // element strides (0 = broadcast)
  float* qbuf;    // [B][H][Np][8]        scaled global direction, global point
  float* klog;    // [B][H][Np][kKeyLog]  global direction, bias, global point
  float* kval;    // [B][H][Np][kValW]    rotated values
  float* part;    // [splits][B][N][H][PW]
  float* stats;   // [B][H][N] float2 (running max, sum)
  float* vectors; float* output; float* attention;
};

// ---------------------------------------------------------------------------
// Batched fp32 GEMM (ipa_gemm.hip): C[z](m, n) = sum_k A[z](m, k) B[z](k, n)
// (+ C[z](m, n) when acc, + bias[n], rows with rowmask[m] == 0 set to 0)
// ---------------------------------------------------------------------------
struct Gemm {
  int M, N, K;
  const float* A; long long sAb, am, ak;
  const float* B; long long sBb, bk, bn;
  float* C; long long sCb, cm;
  int acc;
  const float* bias;        // [N] or NULL
  const uint8_t* rowmask;   // [M] or NULL
  int kpart;                // set by gemm_splitk: reduction slice per grid z
  int nseg;                 // > 0: segmented output (C unused)
  int seg_start[9];         // first column of each block, then N
  void* seg_out[8];         // block b stored [M][width_b]
  int seg_bf16;             // blocks stored as bf16 (nearest even)
  int x3;                   // each operand split into bf16 hi + lo, three
                            // bf16 products (about 2^-17 relative per term)
  int x6;                   // fp32-accurate products: where the operands
                            // suit the copies to LDS, each split into bf16
                            // hi + mid + lo and six bf16 products (terms
                            // below 2^-24 relative dropped), else fp32
                            // products; x3 must be 0
};
hipError_t gemm(const Gemm& g, int batch, hipStream_t s);
// the reduction split into `splits` slices along the grid; partials in
// `part` ([splits][M][N] floats), then reduced in order into g.C (row
// stride N) with g.bias and g.rowmask; g.acc must be 0
hipError_t gemm_splitk(const Gemm& g, int splits, float* part, hipStream_t s);

// ---------------------------------------------------------------------------
// Full layer (ipa_layer.hip): the attention's four outputs gathered into one
// row-major matrix [rows][n_out] for the readout
// ---------------------------------------------------------------------------
struct LayerGather {
  const float* src[4];   // o_s, o_pts, o_norm, o_pair, each [rows][width]
  int start[5];          // first column of each block, then n_out
  long long rows;
  int n_out;
  float* cat;
};
hipError_t launch_layer_gather(const LayerGather& g, hipStream_t s);

// ---------------------------------------------------------------------------
// Gradient of the IPA forward (ipa_bwd.hip), float32
// ---------------------------------------------------------------------------
struct BwdArgs {
  int B, L, H, C, Pqk, Pv, R, Cz;
  int DA, DV, P3;   // C + R Cz, C + 3 Pv + R Cz, 3 Pqk
  int DAQ, DAK;     // DA + P3 + 1 (QA' = [QA | Qg | 1]), DA + P3 (KA' = [KA | Kg]),
                    // each rounded up to a multiple of 4 (zero columns)
  int QC;           // query rows per chunk of the score buffers
  float w_L, w_C;
  // q, k, v, the points, z1 and z2: float32, or bf16 when in_bf16 (read by ldin)
  int in_bf16;
  const void* q; const void* k; const void* v;
  const void* q_pts; const void* k_pts; const void* v_pts;
  const float* rot; const float* trans;
  const void* z1; const void* z2; const float* w_b; const float* gamma;
  const uint8_t* mask;
  const float* o_s; const float* o_pts; const float* o_pair;   // forward outputs
  const float* g_s; const float* g_pts; const float* g_norm; const float* g_pair;
  float* dq; float* dk; float* dv; float* dq_pts; float* dk_pts; float* dv_pts;
  float* drot; float* dtrans; float* dz1; float* dz2; float* dw_b; float* dgamma;
  // workspace, rows [B][H][L][...]
  float* QA; float* KA; float* VA; float* GA; float* QP; float* KP; float* Dv;
  float* dQA; float* U; float* gam; float* rsum;
  float* dKA; float* dVA;
  float* X; float* Y;   // [B H][QC][L] score buffers: S then A, dP then dS
  float* fpart;   // [B][L][H][12]  per-head frame gradient shares
  float* share;   // [B][L][H Cz + H] per-residue shares of dW_b ([h][c]) and dgamma
  float* red1;    // [ceil(B L / 128)][Cz H + H] partial column sums of the shares
  // flash form (ipa_backward_flash): bf16 lifted rows, widths multiples of 32
  int WQ, WG;     // pad32(C + pad32(R Cz)), pad32(C + 9 Pv + R Cz)
  uint16_t* QX; uint16_t* KX;   // [B H][L][WQ]  [w_L/sqrt(C) q | w_L W_b z1 | 0], [k | z2 | 0]
  uint16_t* GX; uint16_t* VX;   // [B H][L][WG]  [g_s | Rg hi | Rg hi | Rg lo | z1 g_pair | 0],
                                //               [v | Vg hi | Vg lo | Vg hi | z2 | 0]
  float* ST;      // [B H][L] float2: row max (base 2) and 1 / row sum of the softmax
};
hipError_t launch_backward(const BwdArgs& a, hipStream_t s);
hipError_t launch_backward_flash(const BwdArgs& a, hipStream_t s);
// per-residue chain rule shared by both gradient forms (post, z, frames, reductions)
hipError_t launch_backward_tail(const BwdArgs& a, hipStream_t s);

// an input element stored as float32 or (bf) as bf16
__device__ __forceinline__ float ldin(const void* p, size_t i, int bf) {
  return bf ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16) : static_cast<const float*>(p)[i];
}

int dd_splits(int B, int N, int H);
int dd_padded_keys(int N);
hipError_t launch_dirdist(const DDArgs& a, hipStream_t s);

}  // namespace ipa
