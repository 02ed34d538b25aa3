// ipa_bwd: gradient of the fused IPA forward (float32).
//
// The forward ("Flash Invariant Point Attention", TL;DR and abstract; MEET
// section 2.2 eq. 6 for the distance term) is one softmax attention over
// lifted rows. Per batch b and head h, with global points Qg = R q_pts + t,
// Kg = R k_pts + t, Vg = R v_pts + t and kappa = w_L gamma_h w_C / 2:
//   S_ij  = QA_i . KA_j - kappa sum_p |Qg_ip - Kg_jp|^2
//           QA_i = [ w_L/sqrt(C) q_i | w_L W_b[:,h] * z1_ir (r = 1..R) ]
//           KA_j = [ k_j | z2_jr ]
//   A_ij  = softmax_j(S_ij) over allowed keys
//   O_i   = sum_j A_ij VA_j,   VA_j = [ v_j | Vg_jp | z2_jr ]
// and the four outputs are o_s = O_s, o_pts = R_i^T (O_pts - t_i),
// |o_pts|, o_pair = sum_r z1_ir * O_pair_r. The backward is that of a
// softmax attention (FlashAttention-2 style, nothing O(L^2) is stored):
//   GA_i  = [ g_s | R_i g_tot_ip | z1_ir * g_pair ]     (dO of the lifted rows,
//           g_tot = g_pts + g_norm o_pts / |o_pts|, 0 at o_pts = 0)
//   D_i   = GA_i . O_i  = g_s.o_s + sum_p (R g_tot).(R o_pts + t) + g_pair.o_pair
//   dS_ij = A_ij (GA_i . VA_j - D_i)
//   dQA_i = sum_j dS_ij KA_j,  dKA_j = sum_i dS_ij QA_i,  dVA_j = sum_i A_ij GA_i
//   point terms from explicit differences: sum_j dS_ij (Qg_ip - Kg_jp) and
//   sum_i dS_ij (Qg_ip - Kg_jp), and sum_j dS_ij |Qg_i - Kg_j|^2 for gamma
//   U_i   = sum_j A_ij z2_jr   (the pair output before z1, for dz1)
// then the chain rule through the lifting and the frames, per residue.
//
// Stages (one stream; workspace linear in B * L):
//   bwd_prep    per (b, i, h): QA, KA, VA, GA, Qg, Kg rows and D_i.
//   bwd_dq      per (b, h, 16 queries): over key tiles, S and dP for a
//               16 x 16 tile (one pair per thread), the running maximum and
//               sum of the softmax (online, as in the forward), and the
//               accumulations dQA, U, the query point term and the gamma
//               term, rescaled with the running maximum; writes them and
//               the row log-sum-exp.
//   bwd_dkv     per (b, h, 16 keys): over query tiles, A from the saved
//               log-sum-exp, dS, and the accumulations dKA, dVA and the key
//               point term.
//   bwd_post    per (b, i, h): dq, dk, dv, the point gradients through R,
//               and this head's share of the frame gradient.
//   bwd_z       per (b, i, c): dz1, dz2 (summed over heads) and the
//               residue's share of dW_b and dgamma.
//   bwd_frames  per (b, i): drot, dtrans (summed over heads).
//   bwd_reduce  column sums of the shares: dW_b, dgamma (fixed order).
// Float32 vector arithmetic throughout; the tiles live in LDS.

#include "ipa_internal.h"

namespace ipa {
namespace {

constexpr int kT = 16;     // queries x keys per tile
constexpr int kMaxDA = 272, kMaxDV = 296, kMaxP3 = 15;

__device__ __forceinline__ void rot3(const float* R, const float* x, float* o) {
  o[0] = R[0] * x[0] + R[1] * x[1] + R[2] * x[2];
  o[1] = R[3] * x[0] + R[4] * x[1] + R[5] * x[2];
  o[2] = R[6] * x[0] + R[7] * x[1] + R[8] * x[2];
}
__device__ __forceinline__ void rot3t(const float* R, const float* x, float* o) {
  o[0] = R[0] * x[0] + R[3] * x[1] + R[6] * x[2];
  o[1] = R[1] * x[0] + R[4] * x[1] + R[7] * x[2];
  o[2] = R[2] * x[0] + R[5] * x[1] + R[8] * x[2];
}

__device__ __forceinline__ bool row_valid(const BwdArgs& a, int b, int i) {
  return a.mask == nullptr || a.mask[(size_t)b * a.L + i] != 0;
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void bwd_prep_kernel(BwdArgs a) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int H = a.H, L = a.L, C = a.C, P = a.Pqk, Pv = a.Pv, RCz = a.R * a.Cz, Cz = a.Cz;
  if (t >= (long long)a.B * L * H) return;
  const int h = (int)(t % H);
  const int i = (int)((t / H) % L);
  const int b = (int)(t / ((long long)H * L));
  const size_t bi = (size_t)b * L + i, bih = bi * H + h;
  const size_t row = ((size_t)b * H + h) * L + i;
  const bool valid = row_valid(a, b, i);
  float R[9], T[3];
  for (int c = 0; c < 9; ++c) R[c] = a.rot[bi * 9 + c];
  for (int c = 0; c < 3; ++c) T[c] = a.trans[bi * 3 + c];
  const float alpha = a.w_L / sqrtf((float)C);
  float* qa = a.QA + row * a.DA;
  float* ka = a.KA + row * a.DA;
  float* va = a.VA + row * a.DV;
  float* ga = a.GA + row * a.DV;
  float* qp = a.QP + row * a.P3;
  float* kp = a.KP + row * a.P3;
  for (int c = 0; c < C; ++c) {
    qa[c] = alpha * a.q[bih * C + c];
    ka[c] = a.k[bih * C + c];
    va[c] = a.v[bih * C + c];
  }
  for (int rc = 0; rc < RCz; ++rc) {
    const float w = a.w_L * a.w_b[(size_t)(rc % Cz) * H + h];
    qa[C + rc] = w * a.z1[bi * RCz + rc];
    ka[C + rc] = a.z2[bi * RCz + rc];
    va[C + 3 * Pv + rc] = a.z2[bi * RCz + rc];
  }
  for (int p = 0; p < P; ++p) {
    float o[3];
    rot3(R, a.q_pts + (bih * P + p) * 3, o);
    for (int x = 0; x < 3; ++x) qp[3 * p + x] = o[x] + T[x];
    rot3(R, a.k_pts + (bih * P + p) * 3, o);
    for (int x = 0; x < 3; ++x) kp[3 * p + x] = o[x] + T[x];
  }
  for (int p = 0; p < Pv; ++p) {
    float o[3];
    rot3(R, a.v_pts + (bih * Pv + p) * 3, o);
    for (int x = 0; x < 3; ++x) va[C + 3 * p + x] = o[x] + T[x];
  }
  // lifted output cotangent and D_i; rows whose outputs are forced to zero
  // pass no gradient
  float D = 0.f;
  if (valid) {
    for (int c = 0; c < C; ++c) {
      const float g = a.g_s[bih * C + c];
      ga[c] = g;
      D = fmaf(g, a.o_s[bih * C + c], D);
    }
    for (int p = 0; p < Pv; ++p) {
      const float* op = a.o_pts + (bih * Pv + p) * 3;
      const float* gp = a.g_pts + (bih * Pv + p) * 3;
      const float n2 = op[0] * op[0] + op[1] * op[1] + op[2] * op[2];
      const float gn = a.g_norm[bih * Pv + p];
      const float s = n2 > 0.f ? gn / sqrtf(n2) : 0.f;
      const float gt[3] = {gp[0] + s * op[0], gp[1] + s * op[1], gp[2] + s * op[2]};
      float dog[3], og[3];
      rot3(R, gt, dog);
      rot3(R, op, og);
      for (int x = 0; x < 3; ++x) {
        ga[C + 3 * p + x] = dog[x];
        D = fmaf(dog[x], og[x] + T[x], D);
      }
    }
    for (int rc = 0; rc < RCz; ++rc) {
      const float gp = a.g_pair[bih * Cz + rc % Cz];
      ga[C + 3 * Pv + rc] = a.z1[bi * RCz + rc] * gp;
    }
    for (int c = 0; c < Cz; ++c) D = fmaf(a.g_pair[bih * Cz + c], a.o_pair[bih * Cz + c], D);
  } else {
    for (int c = 0; c < a.DV; ++c) ga[c] = 0.f;
  }
  a.Dv[row] = D;
}

// ---------------------------------------------------------------------------
// Shared tile evaluation: thread (r, c) of a 16 x 16 tile computes, for its
// query row qi and key row kj, the logit S, the distance sum d and dP.
struct PairOut { float s, d, dp; };

__device__ __forceinline__ PairOut pair_eval(const float* qa, const float* ka, const float* qp,
                                             const float* kp, const float* ga, const float* va,
                                             int DA, int DV, int P3, float kappa) {
  float s = 0.f, d = 0.f, dp = 0.f;
  for (int c = 0; c < DA; ++c) s = fmaf(qa[c], ka[c], s);
  for (int c = 0; c < P3; ++c) {
    const float e = qp[c] - kp[c];
    d = fmaf(e, e, d);
  }
  for (int c = 0; c < DV; ++c) dp = fmaf(ga[c], va[c], dp);
  return {fmaf(-kappa, d, s), d, dp};
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a) {
  const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
  const int H = a.H, L = a.L, DA = a.DA, DV = a.DV, P3 = a.P3, C = a.C, RCz = a.R * a.Cz;
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
  const int i0 = blockIdx.x * kT;
  const float kappa = a.w_L * a.gamma[h] * a.w_C * 0.5f;
  __shared__ float qa[kT][kMaxDA + 1], ga[kT][kMaxDV + 1], qp[kT][kMaxP3 + 1];
  __shared__ float ka[kT][kMaxDA + 1], va[kT][kMaxDV + 1], kp[kT][kMaxP3 + 1];
  __shared__ float st[kT][kT + 1], dpt[kT][kT + 1], dd[kT][kT + 1], ps[kT][kT + 1], dsd[kT][kT + 1];
  __shared__ float frow[kT], Dq[kT];
  __shared__ int qv[kT], kv[kT];
  const size_t base = (size_t)bh * L;
  for (int e = tid; e < kT * DA; e += 256) {
    const int r = e / DA, c = e - r * DA, i = i0 + r;
    qa[r][c] = i < L ? a.QA[(base + i) * DA + c] : 0.f;
  }
  for (int e = tid; e < kT * DV; e += 256) {
    const int r = e / DV, c = e - r * DV, i = i0 + r;
    ga[r][c] = i < L ? a.GA[(base + i) * DV + c] : 0.f;
  }
  for (int e = tid; e < kT * P3; e += 256) {
    const int r = e / P3, c = e - r * P3, i = i0 + r;
    qp[r][c] = i < L ? a.QP[(base + i) * P3 + c] : 0.f;
  }
  if (tid < kT) {
    const int i = i0 + tid;
    qv[tid] = i < L && row_valid(a, b, i);
    Dq[tid] = i < L ? a.Dv[base + i] : 0.f;
  }
  // accumulators of row tr: dQA channels tc + 16 k, U channels tc + 16 k,
  // point channel tc (tc < P3), gamma term (tc == 15)
  float accA[(kMaxDA + 15) / 16], accU[256 / 16], accP = 0.f, accG = 0.f;
  for (int k = 0; k < (kMaxDA + 15) / 16; ++k) accA[k] = 0.f;
  for (int k = 0; k < 16; ++k) accU[k] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;   // used by threads tid < 16 (row tid)
  for (int j0 = 0; j0 < L; j0 += kT) {
    __syncthreads();
    for (int e = tid; e < kT * DA; e += 256) {
      const int r = e / DA, c = e - r * DA, j = j0 + r;
      ka[r][c] = j < L ? a.KA[(base + j) * DA + c] : 0.f;
    }
    for (int e = tid; e < kT * DV; e += 256) {
      const int r = e / DV, c = e - r * DV, j = j0 + r;
      va[r][c] = j < L ? a.VA[(base + j) * DV + c] : 0.f;
    }
    for (int e = tid; e < kT * P3; e += 256) {
      const int r = e / P3, c = e - r * P3, j = j0 + r;
      kp[r][c] = j < L ? a.KP[(base + j) * P3 + c] : 0.f;
    }
    if (tid < kT) {
      const int j = j0 + tid;
      kv[tid] = j < L && row_valid(a, b, j);
    }
    __syncthreads();
    {
      const PairOut po = pair_eval(qa[tr], ka[tc], qp[tr], kp[tc], ga[tr], va[tc], DA, DV, P3, kappa);
      st[tr][tc] = (qv[tr] && kv[tc]) ? po.s : -INFINITY;
      dd[tr][tc] = po.d;
      dpt[tr][tc] = po.dp;
    }
    __syncthreads();
    if (tid < kT) {
      float cm = -INFINITY;
      for (int j = 0; j < kT; ++j) cm = fmaxf(cm, st[tid][j]);
      const float mn = fmaxf(m_run, cm);
      const float f = m_run == -INFINITY ? 0.f : expf(m_run - mn);
      float ls = 0.f;
      for (int j = 0; j < kT; ++j) {
        const float p = st[tid][j] == -INFINITY ? 0.f : expf(st[tid][j] - mn);
        ps[tid][j] = p;
        dsd[tid][j] = p * (dpt[tid][j] - Dq[tid]);
        ls += p;
      }
      l_run = fmaf(l_run, f, ls);
      m_run = mn;
      frow[tid] = f;
    }
    __syncthreads();
    const float f = frow[tr];
    for (int k = 0; k < (kMaxDA + 15) / 16; ++k) {
      const int c = tc + 16 * k;
      if (c < DA) {
        float v = accA[k] * f;
        for (int j = 0; j < kT; ++j) v = fmaf(dsd[tr][j], ka[j][c], v);
        accA[k] = v;
      }
    }
    for (int k = 0; k < 16; ++k) {
      const int c = tc + 16 * k;
      if (c < RCz) {
        float v = accU[k] * f;
        for (int j = 0; j < kT; ++j) v = fmaf(ps[tr][j], ka[j][C + c], v);
        accU[k] = v;
      }
    }
    if (tc < P3) {
      float v = accP * f;
      for (int j = 0; j < kT; ++j) v = fmaf(dsd[tr][j], qp[tr][tc] - kp[j][tc], v);
      accP = v;
    }
    if (tc == 15) {
      float v = accG * f;
      for (int j = 0; j < kT; ++j) v = fmaf(dsd[tr][j], dd[tr][j], v);
      accG = v;
    }
  }
  __syncthreads();
  if (tid < kT) {
    frow[tid] = l_run > 0.f ? 1.f / l_run : 0.f;
    const int i = i0 + tid;
    if (i < L) a.LSE[base + i] = l_run > 0.f ? m_run + logf(l_run) : INFINITY;
  }
  __syncthreads();
  const int i = i0 + tr;
  if (i >= L) return;
  const float inv = frow[tr];
  const size_t row = base + i;
  for (int k = 0; k < (kMaxDA + 15) / 16; ++k) {
    const int c = tc + 16 * k;
    if (c < DA) a.dQA[row * DA + c] = accA[k] * inv;
  }
  for (int k = 0; k < 16; ++k) {
    const int c = tc + 16 * k;
    if (c < RCz) a.U[row * RCz + c] = accU[k] * inv;
  }
  if (tc < P3) a.dQP[row * P3 + tc] = accP * inv;
  if (tc == 15) a.gam[row] = accG * inv;
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_dkv_kernel(BwdArgs a) {
  const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
  const int H = a.H, L = a.L, DA = a.DA, DV = a.DV, P3 = a.P3;
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
  const int j0 = blockIdx.x * kT;
  const float kappa = a.w_L * a.gamma[h] * a.w_C * 0.5f;
  __shared__ float qa[kT][kMaxDA + 1], ga[kT][kMaxDV + 1], qp[kT][kMaxP3 + 1];
  __shared__ float ka[kT][kMaxDA + 1], va[kT][kMaxDV + 1], kp[kT][kMaxP3 + 1];
  __shared__ float pt[kT][kT + 1], dst[kT][kT + 1];
  __shared__ float lse[kT], Dq[kT];
  __shared__ int qv[kT], kv[kT];
  const size_t base = (size_t)bh * L;
  for (int e = tid; e < kT * DA; e += 256) {
    const int r = e / DA, c = e - r * DA, j = j0 + r;
    ka[r][c] = j < L ? a.KA[(base + j) * DA + c] : 0.f;
  }
  for (int e = tid; e < kT * DV; e += 256) {
    const int r = e / DV, c = e - r * DV, j = j0 + r;
    va[r][c] = j < L ? a.VA[(base + j) * DV + c] : 0.f;
  }
  for (int e = tid; e < kT * P3; e += 256) {
    const int r = e / P3, c = e - r * P3, j = j0 + r;
    kp[r][c] = j < L ? a.KP[(base + j) * P3 + c] : 0.f;
  }
  if (tid < kT) {
    const int j = j0 + tid;
    kv[tid] = j < L && row_valid(a, b, j);
  }
  // accumulators of key row tr: dKA channels tc + 16 k, dVA channels tc + 16 k,
  // point channel tc (tc < P3)
  float accK[(kMaxDA + 15) / 16], accV[(kMaxDV + 15) / 16], accP = 0.f;
  for (int k = 0; k < (kMaxDA + 15) / 16; ++k) accK[k] = 0.f;
  for (int k = 0; k < (kMaxDV + 15) / 16; ++k) accV[k] = 0.f;
  for (int i0 = 0; i0 < L; i0 += kT) {
    __syncthreads();
    for (int e = tid; e < kT * DA; e += 256) {
      const int r = e / DA, c = e - r * DA, i = i0 + r;
      qa[r][c] = i < L ? a.QA[(base + i) * DA + c] : 0.f;
    }
    for (int e = tid; e < kT * DV; e += 256) {
      const int r = e / DV, c = e - r * DV, i = i0 + r;
      ga[r][c] = i < L ? a.GA[(base + i) * DV + c] : 0.f;
    }
    for (int e = tid; e < kT * P3; e += 256) {
      const int r = e / P3, c = e - r * P3, i = i0 + r;
      qp[r][c] = i < L ? a.QP[(base + i) * P3 + c] : 0.f;
    }
    if (tid < kT) {
      const int i = i0 + tid;
      qv[tid] = i < L && row_valid(a, b, i);
      lse[tid] = i < L ? a.LSE[base + i] : INFINITY;
      Dq[tid] = i < L ? a.Dv[base + i] : 0.f;
    }
    __syncthreads();
    {
      // thread (tr, tc): key row tr, query row tc
      const PairOut po = pair_eval(qa[tc], ka[tr], qp[tc], kp[tr], ga[tc], va[tr], DA, DV, P3, kappa);
      const float p = (qv[tc] && kv[tr]) ? expf(po.s - lse[tc]) : 0.f;
      pt[tr][tc] = p;
      dst[tr][tc] = p * (po.dp - Dq[tc]);
    }
    __syncthreads();
    for (int k = 0; k < (kMaxDA + 15) / 16; ++k) {
      const int c = tc + 16 * k;
      if (c < DA) {
        float v = accK[k];
        for (int i = 0; i < kT; ++i) v = fmaf(dst[tr][i], qa[i][c], v);
        accK[k] = v;
      }
    }
    for (int k = 0; k < (kMaxDV + 15) / 16; ++k) {
      const int c = tc + 16 * k;
      if (c < DV) {
        float v = accV[k];
        for (int i = 0; i < kT; ++i) v = fmaf(pt[tr][i], ga[i][c], v);
        accV[k] = v;
      }
    }
    if (tc < P3) {
      float v = accP;
      for (int i = 0; i < kT; ++i) v = fmaf(dst[tr][i], qp[i][tc] - kp[tr][tc], v);
      accP = v;
    }
  }
  const int j = j0 + tr;
  if (j >= L) return;
  const size_t row = base + j;
  for (int k = 0; k < (kMaxDA + 15) / 16; ++k) {
    const int c = tc + 16 * k;
    if (c < DA) a.dKA[row * DA + c] = accK[k];
  }
  for (int k = 0; k < (kMaxDV + 15) / 16; ++k) {
    const int c = tc + 16 * k;
    if (c < DV) a.dVA[row * DV + c] = accV[k];
  }
  if (tc < P3) a.dKP[row * P3 + tc] = accP;
}

// ---------------------------------------------------------------------------
// per (b, i, h): dq, dk, dv, point gradients, this head's frame share
__global__ __launch_bounds__(64) void bwd_post_kernel(BwdArgs a) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int H = a.H, L = a.L, C = a.C, P = a.Pqk, Pv = a.Pv;
  if (t >= (long long)a.B * L * H) return;
  const int h = (int)(t % H);
  const int i = (int)((t / H) % L);
  const int b = (int)(t / ((long long)H * L));
  const size_t bi = (size_t)b * L + i, bih = bi * H + h;
  const size_t row = ((size_t)b * H + h) * L + i;
  float* fp = a.fpart + bih * 12;
  if (!row_valid(a, b, i)) {
    for (int c = 0; c < C; ++c) { a.dq[bih * C + c] = 0.f; a.dk[bih * C + c] = 0.f; a.dv[bih * C + c] = 0.f; }
    for (int c = 0; c < 3 * P; ++c) { a.dq_pts[bih * 3 * P + c] = 0.f; a.dk_pts[bih * 3 * P + c] = 0.f; }
    for (int c = 0; c < 3 * Pv; ++c) a.dv_pts[bih * 3 * Pv + c] = 0.f;
    for (int c = 0; c < 12; ++c) fp[c] = 0.f;
    return;
  }
  float R[9];
  for (int c = 0; c < 9; ++c) R[c] = a.rot[bi * 9 + c];
  const float alpha = a.w_L / sqrtf((float)C);
  const float kappa = a.w_L * a.gamma[h] * a.w_C * 0.5f;
  for (int c = 0; c < C; ++c) {
    a.dq[bih * C + c] = alpha * a.dQA[row * a.DA + c];
    a.dk[bih * C + c] = a.dKA[row * a.DA + c];
    a.dv[bih * C + c] = a.dVA[row * a.DV + c];
  }
  float dR[9] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, dT[3] = {0.f, 0.f, 0.f};
  // global-frame point gradient u of local point x: d(local) = R^T u,
  // dR += u x^T, dt += u
  auto through_frame = [&](const float* u, const float* x, float* dloc) {
    rot3t(R, u, dloc);
    for (int r = 0; r < 3; ++r) {
      dT[r] += u[r];
      for (int c = 0; c < 3; ++c) dR[3 * r + c] = fmaf(u[r], x[c], dR[3 * r + c]);
    }
  };
  for (int p = 0; p < P; ++p) {
    float u[3], dl[3];
    for (int x = 0; x < 3; ++x) u[x] = -2.f * kappa * a.dQP[row * a.P3 + 3 * p + x];
    through_frame(u, a.q_pts + (bih * P + p) * 3, dl);
    for (int x = 0; x < 3; ++x) a.dq_pts[(bih * P + p) * 3 + x] = dl[x];
    for (int x = 0; x < 3; ++x) u[x] = 2.f * kappa * a.dKP[row * a.P3 + 3 * p + x];
    through_frame(u, a.k_pts + (bih * P + p) * 3, dl);
    for (int x = 0; x < 3; ++x) a.dk_pts[(bih * P + p) * 3 + x] = dl[x];
  }
  for (int p = 0; p < Pv; ++p) {
    float u[3], dl[3];
    for (int x = 0; x < 3; ++x) u[x] = a.dVA[row * a.DV + C + 3 * p + x];
    through_frame(u, a.v_pts + (bih * Pv + p) * 3, dl);
    for (int x = 0; x < 3; ++x) a.dv_pts[(bih * Pv + p) * 3 + x] = dl[x];
    // the output o_pts = R^T (og - t): with g_tot its cotangent,
    // dR += (og - t) g_tot^T = (R o_pts) g_tot^T and dt -= R g_tot
    const float* op = a.o_pts + (bih * Pv + p) * 3;
    const float* gp = a.g_pts + (bih * Pv + p) * 3;
    const float n2 = op[0] * op[0] + op[1] * op[1] + op[2] * op[2];
    const float s = n2 > 0.f ? a.g_norm[bih * Pv + p] / sqrtf(n2) : 0.f;
    const float gt[3] = {gp[0] + s * op[0], gp[1] + s * op[1], gp[2] + s * op[2]};
    float y[3], dog[3];
    rot3(R, op, y);
    rot3(R, gt, dog);
    for (int r = 0; r < 3; ++r) {
      dT[r] -= dog[r];
      for (int c = 0; c < 3; ++c) dR[3 * r + c] = fmaf(y[r], gt[c], dR[3 * r + c]);
    }
  }
  for (int c = 0; c < 9; ++c) fp[c] = dR[c];
  for (int c = 0; c < 3; ++c) fp[9 + c] = dT[c];
}

// per (b, i, c): dz1, dz2 and the residue's share of dW_b and dgamma
__global__ __launch_bounds__(64) void bwd_z_kernel(BwdArgs a) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int H = a.H, L = a.L, C = a.C, R = a.R, Cz = a.Cz, Pv = a.Pv, RCz = R * Cz;
  if (t >= (long long)a.B * L * Cz) return;
  const int c = (int)(t % Cz);
  const long long bi = t / Cz;
  const int i = (int)(bi % L), b = (int)(bi / L);
  float* share = a.share + (size_t)bi * (Cz * H + H);
  if (!row_valid(a, b, i)) {
    for (int r = 0; r < R; ++r) { a.dz1[bi * RCz + r * Cz + c] = 0.f; a.dz2[bi * RCz + r * Cz + c] = 0.f; }
    for (int h = 0; h < H; ++h) share[c * H + h] = 0.f;
    if (c == 0) for (int h = 0; h < H; ++h) share[Cz * H + h] = 0.f;
    return;
  }
  for (int r = 0; r < R; ++r) {
    const int rc = r * Cz + c;
    const float z1 = a.z1[bi * RCz + rc];
    float d1 = 0.f, d2 = 0.f;
    for (int h = 0; h < H; ++h) {
      const size_t row = ((size_t)b * H + h) * L + i;
      const float e = a.dQA[row * a.DA + C + rc];   // sum_j dS_ij z2_j
      const float wb = a.w_b[(size_t)c * H + h];
      d1 = fmaf(a.w_L * wb, e, d1);
      d1 = fmaf(a.g_pair[((size_t)bi * H + h) * Cz + c], a.U[row * RCz + rc], d1);
      d2 += a.dKA[row * a.DA + C + rc] + a.dVA[row * a.DV + C + 3 * Pv + rc];
      // dW_b[c, h] share: w_L z1_irc e_ihrc, summed over r
      if (r == 0) share[c * H + h] = 0.f;
      share[c * H + h] = fmaf(a.w_L * z1, e, share[c * H + h]);
    }
    a.dz1[bi * RCz + rc] = d1;
    a.dz2[bi * RCz + rc] = d2;
  }
  if (c == 0) {
    for (int h = 0; h < H; ++h) {
      const size_t row = ((size_t)b * H + h) * L + i;
      share[Cz * H + h] = -0.5f * a.w_L * a.w_C * a.gam[row];
    }
  }
}

// per (b, i): drot, dtrans
__global__ __launch_bounds__(64) void bwd_frames_kernel(BwdArgs a) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (long long)a.B * a.L) return;
  float acc[12] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int h = 0; h < a.H; ++h)
    for (int c = 0; c < 12; ++c) acc[c] += a.fpart[((size_t)t * a.H + h) * 12 + c];
  for (int c = 0; c < 9; ++c) a.drot[(size_t)t * 9 + c] = acc[c];
  for (int c = 0; c < 3; ++c) a.dtrans[(size_t)t * 3 + c] = acc[9 + c];
}

// column sums of the per-residue shares, in a fixed order: 4 row groups per
// column, then the groups added in order
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a) {
  const int ncol = a.Cz * a.H + a.H;
  const int col = blockIdx.x * 64 + (threadIdx.x & 63), g = threadIdx.x >> 6;
  const long long rows = (long long)a.B * a.L;
  __shared__ float part[4][64];
  float s = 0.f;
  if (col < ncol)
    for (long long r = g; r < rows; r += 4) s += a.share[(size_t)r * ncol + col];
  part[g][threadIdx.x & 63] = s;
  __syncthreads();
  if (g != 0 || col >= ncol) return;
  const float v = ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) + part[3][threadIdx.x];
  if (col < a.Cz * a.H) a.dw_b[col] = v;
  else a.dgamma[col - a.Cz * a.H] = v;
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t s) {
  const long long bih = (long long)a.B * a.L * a.H;
  const unsigned g64 = (unsigned)((bih + 63) / 64);
  hipLaunchKernelGGL(bwd_prep_kernel, dim3(g64), dim3(64), 0, s, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const dim3 gt((a.L + kT - 1) / kT, a.B * a.H);
  hipLaunchKernelGGL(bwd_dq_kernel, gt, dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(bwd_dkv_kernel, gt, dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(bwd_post_kernel, dim3(g64), dim3(64), 0, s, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const long long biz = (long long)a.B * a.L * a.Cz;
  hipLaunchKernelGGL(bwd_z_kernel, dim3((unsigned)((biz + 63) / 64)), dim3(64), 0, s, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const long long bi = (long long)a.B * a.L;
  hipLaunchKernelGGL(bwd_frames_kernel, dim3((unsigned)((bi + 63) / 64)), dim3(64), 0, s, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const int ncol = a.Cz * a.H + a.H;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((ncol + 63) / 64), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  return hipSuccess;
}

}  // namespace ipa
