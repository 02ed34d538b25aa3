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
// softmax attention, taken query chunk by query chunk:
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
// Stages (one stream):
//   bwd_prep    per (b, i, h): the lifted rows QA' = [QA | Qg | 1],
//               KA' = [KA | Kg], VA, GA, the points and D_i.
//   per chunk of QC query rows (QC bounds the two score buffers to
//   2 x 2^26 floats, so memory stays linear in L):
//     gemm      S = QA KA^T (split path) and dP = GA VA^T (fp32-accurate)
//     bwd_rows  per query row: the point term -kappa |Qg_i - Kg_j|^2 from
//               explicit differences, the masked softmax A, dS, and the
//               row sums of dS and of dS |Qg_i - Kg_j|^2
//     gemm      dQA' = dS KA' (with sum_j dS Kg_j), U = A z2,
//               dKA' += dS^T QA' (with sum_i dS Qg_i and the column sum),
//               dVA += A^T GA
//   bwd_post    per (b, i, h): dq, dk, dv, the point gradients through R,
//               and this head's share of the frame gradient.
//   bwd_z       per (b, i, c): dz1, dz2 (summed over heads) and the
//               residue's share of dW_b and dgamma.
//   bwd_frames  per (b, i): drot, dtrans (summed over heads).
//   bwd_reduce1/2  column sums of the shares: dW_b, dgamma (fixed order).
// The last four stages (launch_backward_tail) also finish the flash form
// (ipa_bwd_flash.hip), which fills the same per-row arrays without score rows.
// The point sums of dS against Qg, Kg come from the GEMMs and the
// corrections Qg_i sum_j dS_ij, Kg_j sum_i dS_ij; the coordinates are a
// few hundred A at most and the dS sums vanish up to rounding, so the
// products lose no significant digits at float32.

#include "ipa_internal.h"

namespace ipa {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
constexpr int kMaxP3 = 15;   // 3 Pqk

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
// bwd_prep: one wave per (b, i, h); lanes over the columns of the lifted
// rows, so every row is written with coalesced stores.
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int H = a.H, L = a.L, C = a.C, P = a.Pqk, Pv = a.Pv, RCz = a.R * a.Cz, Cz = a.Cz;
  if (t >= (long long)a.B * L * H) return;
  const int h = (int)(t % H);
  const int i = (int)((t / H) % L);
  const int b = (int)(t / ((long long)H * L));
  const size_t bi = (size_t)b * L + i, bih = bi * H + h;
  const size_t row = ((size_t)b * H + h) * L + i;
  const bool valid = row_valid(a, b, i);
  const float* R = a.rot + bi * 9;
  const float* T = a.trans + bi * 3;
  const float alpha = a.w_L / sqrtf((float)C);
  float* qa = a.QA + row * a.DAQ;
  float* ka = a.KA + row * a.DAK;
  float* va = a.VA + row * a.DV;
  float* ga = a.GA + row * a.DV;
  // global point coordinate x of local point pt: R[x] . pt + t[x]
  auto gpt = [&](const void* base, size_t e, int x) {
    const float p0 = ldin(base, e, a.in_bf16), p1 = ldin(base, e + 1, a.in_bf16), p2 = ldin(base, e + 2, a.in_bf16);
    return R[3 * x] * p0 + R[3 * x + 1] * p1 + R[3 * x + 2] * p2 + T[x];
  };
  for (int c = lane; c < a.DAQ; c += 64) {
    float vq, vk = 0.f;
    if (c < C) {
      vq = alpha * ldin(a.q, bih * C + c, a.in_bf16);
      vk = ldin(a.k, bih * C + c, a.in_bf16);
    } else if (c < a.DA) {
      const int rc = c - C;
      vq = a.w_L * a.w_b[(size_t)(rc % Cz) * H + h] * ldin(a.z1, bi * RCz + rc, a.in_bf16);
      vk = ldin(a.z2, bi * RCz + rc, a.in_bf16);
    } else if (c < a.DA + a.P3) {
      const int e = c - a.DA, p = e / 3, x = e - 3 * p;
      vq = gpt(a.q_pts, (bih * P + p) * 3, x);
      vk = gpt(a.k_pts, (bih * P + p) * 3, x);
      a.QP[row * a.P3 + e] = vq;
      a.KP[row * a.P3 + e] = vk;
    } else {
      // dS^T times this column: the column sums of dS; then zero padding
      vq = c == a.DA + a.P3 ? 1.f : 0.f;
    }
    qa[c] = vq;
    if (c < a.DAK) ka[c] = vk;
  }
  // VA and the lifted output cotangent GA; rows whose outputs are forced to
  // zero pass no gradient. D_i = GA_i . O_i, O_i from the outputs.
  float D = 0.f;
  for (int c = lane; c < a.DV; c += 64) {
    float vv, gv = 0.f;
    if (c < C) {
      vv = ldin(a.v, bih * C + c, a.in_bf16);
      if (valid) {
        gv = a.g_s[bih * C + c];
        D = fmaf(gv, a.o_s[bih * C + c], D);
      }
    } else if (c < C + 3 * Pv) {
      const int e = c - C, p = e / 3, x = e - 3 * p;
      vv = gpt(a.v_pts, (bih * Pv + p) * 3, x);
      if (valid) {
        const float* op = a.o_pts + (bih * Pv + p) * 3;
        const float* gp = a.g_pts + (bih * Pv + p) * 3;
        const float n2 = op[0] * op[0] + op[1] * op[1] + op[2] * op[2];
        const float s = n2 > 0.f ? a.g_norm[bih * Pv + p] / sqrtf(n2) : 0.f;
        const float gt[3] = {gp[0] + s * op[0], gp[1] + s * op[1], gp[2] + s * op[2]};
        gv = R[3 * x] * gt[0] + R[3 * x + 1] * gt[1] + R[3 * x + 2] * gt[2];   // R g_tot
        D = fmaf(gv, R[3 * x] * op[0] + R[3 * x + 1] * op[1] + R[3 * x + 2] * op[2] + T[x], D);                                      // . (R o_pts + t)
      }
    } else {
      const int rc = c - C - 3 * Pv;
      vv = ldin(a.z2, bi * RCz + rc, a.in_bf16);
      if (valid) gv = ldin(a.z1, bi * RCz + rc, a.in_bf16) * a.g_pair[bih * Cz + rc % Cz];
    }
    va[c] = vv;
    ga[c] = gv;
  }
  if (valid)
    for (int c = lane; c < Cz; c += 64) D = fmaf(a.g_pair[bih * Cz + c], a.o_pair[bih * Cz + c], D);
  for (int o = 32; o > 0; o >>= 1) D += __shfl_xor(D, o);
  if (lane == 0) a.Dv[row] = D;
}

// ---------------------------------------------------------------------------
// bwd_rows: a workgroup takes kRowsPerWG query rows of one (b, h), a wave
// one row at a time. X holds S (without the point term) and becomes A; Y
// holds dP and becomes dS. The head's key points are staged in LDS,
// coordinate-major, kKeyBlock keys at a time (lane j reads key j: no bank
// conflicts), together with a per-key bias (0, or -inf for a masked key),
// so each row reads them from LDS instead of L2. Pass 1 takes the row max
// and sum kUnroll keys per lane at a time (one rescale per group, no
// divergent branches); pass 2 writes A and dS. In both passes a wave
// handles its two rows side by side so that their loads overlap.
// ---------------------------------------------------------------------------
constexpr int kRowsPerWG = 8, kKeyBlock = 512, kUnroll = 8;

// e^x for x <= 0 through the hardware base-2 exponential (about 1 ulp)
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

template <int KPL>
__global__ __launch_bounds__(256) void bwd_rows_kernel(BwdArgs a, int q0, int qc) {
  // KPL consecutive keys per lane and group (4: 16-byte loads and stores,
  // rows of L a multiple of 4), U groups per lane per pass over a key block
  constexpr int U = kUnroll / KPL;
  static_assert(KPL * U == kUnroll && 64 * kUnroll == kKeyBlock, "one group sweep per key block");
  typedef float fvec __attribute__((ext_vector_type(KPL)));
  __shared__ __attribute__((aligned(16))) float kps[kMaxP3 + 1][kKeyBlock];   // rows 0 .. P3 - 1: points; row kMaxP3: key bias
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int bh = blockIdx.y, H = a.H, L = a.L, P3 = a.P3;
  const int b = bh / H, h = bh - b * H;
  const float kappa = a.w_L * a.gamma[h] * a.w_C * 0.5f;
  const float* KP = a.KP + (size_t)bh * L * P3;
  const int r0 = blockIdx.x * kRowsPerWG;
  // per row of this wave: running max and sum (pass 1), then A, dS (pass 2)
  float m[kRowsPerWG / 4], l[kRowsPerWG / 4], qp[kRowsPerWG / 4][kMaxP3];
  bool qv[kRowsPerWG / 4];
#pragma unroll
  for (int u = 0; u < kRowsPerWG / 4; ++u) {
    const int r = r0 + w + 4 * u, i = q0 + r;
    qv[u] = r < qc && row_valid(a, b, i);
    m[u] = -INFINITY;
    l[u] = 0.f;
#pragma unroll
    for (int c = 0; c < kMaxP3; ++c) qp[u][c] = (r < qc && c < P3) ? a.QP[((size_t)bh * L + i) * P3 + c] : 0.f;
  }
  auto stage = [&](int k0, int nk) {
    __syncthreads();
    // thread j copies key j's coordinates (no division by P3)
    for (int j = threadIdx.x; j < kKeyBlock; j += 256) {
      const float* src = KP + (size_t)(k0 + j) * P3;
#pragma unroll
      for (int c = 0; c < kMaxP3; ++c)
        if (c < P3 && j < nk) kps[c][j] = src[c];
      kps[kMaxP3][j] = (j < nk && row_valid(a, b, k0 + j)) ? 0.f : -INFINITY;
    }
    __syncthreads();
  };
  // first key (within the block) of group t of this lane
  auto key0 = [&](int t) { return (64 * t + lane) * KPL; };
  // squared distances of row point set q to the KPL keys of group t, and their biases
  auto dist = [&](const float (&q)[kMaxP3], int j0, fvec& d, fvec& bias) {
    d = fvec{};
#pragma unroll
    for (int c = 0; c < kMaxP3; ++c) {
      if (c < P3) {
        const fvec kv = *reinterpret_cast<const fvec*>(&kps[c][j0]);
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
          const float df = q[c] - kv[e];
          d[e] = fmaf(df, df, d[e]);
        }
      }
    }
    bias = *reinterpret_cast<const fvec*>(&kps[kMaxP3][j0]);
  };
  // pass 1: the wave's rows side by side, so that all their loads of a
  // group are in flight together
  constexpr int NR = kRowsPerWG / 4;
  for (int k0 = 0; k0 < L; k0 += kKeyBlock) {
    const int nk = L - k0 < kKeyBlock ? L - k0 : kKeyBlock;
    stage(k0, nk);
    fvec sv[NR][U];
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const float* X = a.X + ((size_t)bh * a.QC + r0 + w + 4 * u) * L + k0;
#pragma unroll
      for (int t = 0; t < U; ++t) {
        const int jj = key0(t);
        sv[u][t] = (qv[u] && jj < nk) ? *reinterpret_cast<const fvec*>(X + jj) : fvec{};
      }
    }
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      float mt = m[u];
#pragma unroll
      for (int t = 0; t < U; ++t) {
        const int jj = key0(t);
        fvec d, bias;
        dist(qp[u], jj, d, bias);
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
          sv[u][t][e] = (qv[u] && jj + e < nk) ? fmaf(-kappa, d[e], sv[u][t][e]) + bias[e] : -INFINITY;
          mt = fmaxf(mt, sv[u][t][e]);
        }
      }
      // every key so far masked: nothing to add yet
      const float sc = mt == -INFINITY ? 0.f : mt;
      float acc = l[u] * fexp(m[u] - sc);
#pragma unroll
      for (int t = 0; t < U; ++t)
#pragma unroll
        for (int e = 0; e < KPL; ++e) acc += fexp(sv[u][t][e] - sc);
      l[u] = acc;
      m[u] = mt;
    }
  }
  float inv[kRowsPerWG / 4];
#pragma unroll
  for (int u = 0; u < kRowsPerWG / 4; ++u) {
    float mw = m[u];
    for (int o = 32; o > 0; o >>= 1) mw = fmaxf(mw, __shfl_xor(mw, o));
    float lw = m[u] == -INFINITY ? 0.f : l[u] * fexp(m[u] - mw);
    for (int o = 32; o > 0; o >>= 1) lw += __shfl_xor(lw, o);
    m[u] = mw;
    inv[u] = lw > 0.f ? 1.f / lw : 0.f;
  }
  // pass 2
  float rs[kRowsPerWG / 4], gs[kRowsPerWG / 4];
#pragma unroll
  for (int u = 0; u < kRowsPerWG / 4; ++u) rs[u] = gs[u] = 0.f;
  float Dr[NR], mu[NR];
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const int r = r0 + w + 4 * u;
    Dr[u] = r < qc ? a.Dv[(size_t)bh * L + q0 + r] : 0.f;
    // a row with no valid key (or a masked row) writes zeros
    mu[u] = m[u] == -INFINITY ? 0.f : m[u];
  }
  for (int k0 = 0; k0 < L; k0 += kKeyBlock) {
    const int nk = L - k0 < kKeyBlock ? L - k0 : kKeyBlock;
    if (k0 > 0 || L > kKeyBlock) stage(k0, nk);
    fvec xv[NR][U], yv[NR][U];
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const size_t row = (size_t)bh * a.QC + r0 + w + 4 * u;
      const bool rin = r0 + w + 4 * u < qc;
#pragma unroll
      for (int t = 0; t < U; ++t) {
        const int jj = key0(t);
        xv[u][t] = (rin && jj < nk) ? *reinterpret_cast<const fvec*>(a.X + row * L + k0 + jj) : fvec{};
        yv[u][t] = (rin && jj < nk) ? *reinterpret_cast<const fvec*>(a.Y + row * L + k0 + jj) : fvec{};
      }
    }
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int r = r0 + w + 4 * u;
      if (r >= qc) continue;
      float* X = a.X + ((size_t)bh * a.QC + r) * L + k0;
      float* Y = a.Y + ((size_t)bh * a.QC + r) * L + k0;
#pragma unroll
      for (int t = 0; t < U; ++t) {
        const int jj = key0(t);
        if (jj >= nk) continue;   // (nk is a multiple of KPL)
        fvec p = fvec{}, ds = fvec{};
        if (qv[u]) {
          fvec d, bias;
          dist(qp[u], jj, d, bias);
#pragma unroll
          for (int e = 0; e < KPL; ++e) {
            p[e] = fexp(fmaf(-kappa, d[e], xv[u][t][e]) + bias[e] - mu[u]) * inv[u];
            ds[e] = p[e] * (yv[u][t][e] - Dr[u]);
            rs[u] += ds[e];
            gs[u] = fmaf(ds[e], d[e], gs[u]);
          }
        }
        *reinterpret_cast<fvec*>(X + jj) = p;
        *reinterpret_cast<fvec*>(Y + jj) = ds;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kRowsPerWG / 4; ++u) {
    float r1 = rs[u], g1 = gs[u];
    for (int o = 32; o > 0; o >>= 1) {
      r1 += __shfl_xor(r1, o);
      g1 += __shfl_xor(g1, o);
    }
    const int r = r0 + w + 4 * u;
    if (lane == 0 && r < qc) {
      a.rsum[(size_t)bh * L + q0 + r] = r1;
      a.gam[(size_t)bh * L + q0 + r] = g1;
    }
  }
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
    a.dq[bih * C + c] = alpha * a.dQA[row * a.DAK + c];
    a.dk[bih * C + c] = a.dKA[row * a.DAQ + c];
    a.dv[bih * C + c] = a.dVA[row * a.DV + c];
  }
  // sum_j dS_ij (Qg_i - Kg_j) and sum_i dS_ij (Qg_i - Kg_j) per coordinate
  const float rsum = a.rsum[row], csum = a.dKA[row * a.DAQ + a.DA + a.P3];
  float dR[9] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, dT[3] = {0.f, 0.f, 0.f};
  // global-frame point gradient u of local point x: d(local) = R^T u,
  // dR += u x^T, dt += u
  auto through_frame = [&](const float* u, const void* base, size_t e, float* dloc) {
    const float x[3] = {ldin(base, e, a.in_bf16), ldin(base, e + 1, a.in_bf16), ldin(base, e + 2, a.in_bf16)};
    rot3t(R, u, dloc);
    for (int r = 0; r < 3; ++r) {
      dT[r] += u[r];
      for (int c = 0; c < 3; ++c) dR[3 * r + c] = fmaf(u[r], x[c], dR[3 * r + c]);
    }
  };
  for (int p = 0; p < P; ++p) {
    float u[3], dl[3];
    for (int x = 0; x < 3; ++x) {
      const int c = 3 * p + x;
      u[x] = -2.f * kappa * (a.QP[row * a.P3 + c] * rsum - a.dQA[row * a.DAK + a.DA + c]);
    }
    through_frame(u, a.q_pts, (bih * P + p) * 3, dl);
    for (int x = 0; x < 3; ++x) a.dq_pts[(bih * P + p) * 3 + x] = dl[x];
    for (int x = 0; x < 3; ++x) {
      const int c = 3 * p + x;
      u[x] = 2.f * kappa * (a.dKA[row * a.DAQ + a.DA + c] - a.KP[row * a.P3 + c] * csum);
    }
    through_frame(u, a.k_pts, (bih * P + p) * 3, dl);
    for (int x = 0; x < 3; ++x) a.dk_pts[(bih * P + p) * 3 + x] = dl[x];
  }
  for (int p = 0; p < Pv; ++p) {
    float u[3], dl[3];
    for (int x = 0; x < 3; ++x) u[x] = a.dVA[row * a.DV + C + 3 * p + x];
    through_frame(u, a.v_pts, (bih * Pv + p) * 3, dl);
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
    for (int h = 0; h < H; ++h) share[h * Cz + c] = 0.f;
    if (c == 0) for (int h = 0; h < H; ++h) share[Cz * H + h] = 0.f;
    return;
  }
  for (int r = 0; r < R; ++r) {
    const int rc = r * Cz + c;
    const float z1 = ldin(a.z1, bi * RCz + rc, a.in_bf16);
    float d1 = 0.f, d2 = 0.f;
    for (int h = 0; h < H; ++h) {
      const size_t row = ((size_t)b * H + h) * L + i;
      const float e = a.dQA[row * a.DAK + C + rc];   // sum_j dS_ij z2_j
      const float wb = a.w_b[(size_t)c * H + h];
      d1 = fmaf(a.w_L * wb, e, d1);
      d1 = fmaf(a.g_pair[((size_t)bi * H + h) * Cz + c], a.U[row * RCz + rc], d1);
      d2 += a.dKA[row * a.DAQ + C + rc] + a.dVA[row * a.DV + C + 3 * Pv + rc];
      // dW_b[c, h] share: w_L z1_irc e_ihrc, summed over r
      // (stored [h][c]: consecutive lanes write consecutive floats)
      share[h * Cz + c] = r == 0 ? a.w_L * z1 * e : fmaf(a.w_L * z1, e, share[h * Cz + c]);
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

// column sums of the per-residue shares, in a fixed order: stage 1 sums
// blocks of kRedRows rows (4 row groups per column, added in order) into
// partial rows, stage 2 adds the partial rows in order
constexpr int kRedRows = 128;

__global__ __launch_bounds__(256) void bwd_reduce1_kernel(BwdArgs a) {
  const int ncol = a.Cz * a.H + a.H;
  const int col = blockIdx.x * 64 + (threadIdx.x & 63), g = threadIdx.x >> 6;
  const long long rows = (long long)a.B * a.L, r0 = (long long)blockIdx.y * kRedRows;
  __shared__ float part[4][64];
  float s = 0.f;
  if (col < ncol)
    for (long long r = r0 + g; r < r0 + kRedRows && r < rows; r += 4) s += a.share[(size_t)r * ncol + col];
  part[g][threadIdx.x & 63] = s;
  __syncthreads();
  if (g != 0 || col >= ncol) return;
  a.red1[(size_t)blockIdx.y * ncol + col] =
      ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) + part[3][threadIdx.x];
}

__global__ __launch_bounds__(256) void bwd_reduce2_kernel(BwdArgs a, int nblk) {
  const int ncol = a.Cz * a.H + a.H;
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= ncol) return;
  float v = 0.f;
  for (int k = 0; k < nblk; ++k) v += a.red1[(size_t)k * ncol + col];
  if (col < a.Cz * a.H) a.dw_b[(size_t)(col % a.Cz) * a.H + col / a.Cz] = v;   // share column h Cz + c
  else a.dgamma[col - a.Cz * a.H] = v;
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t s) {
  const long long bih = (long long)a.B * a.L * a.H;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((bih + 3) / 4)), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const int BH = a.B * a.H, L = a.L, RCz = a.R * a.Cz;
  const long long rowsQ = (long long)L * a.DAQ, rowsK = (long long)L * a.DAK, rowsV = (long long)L * a.DV;
  const long long xs = (long long)a.QC * L;
  for (int q0 = 0; q0 < L; q0 += a.QC) {
    const int qc = L - q0 < a.QC ? L - q0 : a.QC;
    // S = QA KA^T (the first DA columns of both)
    Gemm g{};
    g.M = qc; g.N = L; g.K = a.DA;
    g.A = a.QA + (size_t)q0 * a.DAQ; g.sAb = rowsQ; g.am = a.DAQ; g.ak = 1;
    g.B = a.KA; g.sBb = rowsK; g.bk = 1; g.bn = a.DAK;
    g.C = a.X; g.sCb = xs; g.cm = L; g.acc = 0;
    g.x3 = 1;
    if (gemm(g, BH, s) != hipSuccess) return hipErrorLaunchFailure;
    // dP = GA VA^T, fp32-accurate (three-way split where it applies)
    g.x3 = 0;
    g.x6 = 1;
    g.K = a.DV;
    g.A = a.GA + (size_t)q0 * a.DV; g.sAb = rowsV; g.am = a.DV;
    g.B = a.VA; g.sBb = rowsV; g.bk = 1; g.bn = a.DV;
    g.C = a.Y;
    if (gemm(g, BH, s) != hipSuccess) return hipErrorLaunchFailure;
    g.x6 = 0;
    // four keys per lane when the score rows are 16-byte aligned
    if (L % 4 == 0)
      hipLaunchKernelGGL(bwd_rows_kernel<4>, dim3((qc + kRowsPerWG - 1) / kRowsPerWG, BH), dim3(256), 0, s, a, q0, qc);
    else
      hipLaunchKernelGGL(bwd_rows_kernel<1>, dim3((qc + kRowsPerWG - 1) / kRowsPerWG, BH), dim3(256), 0, s, a, q0, qc);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    // Precision of the products: S, U = A z2, dVA = A^T GA and the scalar and
    // pair columns of dQA' and dKA' run on the split path (each fp32 operand
    // as bf16 hi + lo, three bf16 products, about 2^-17 relative per term).
    // S holds the lifted dot only (its point term is added from explicit
    // differences in the row kernel), scalar and pair products of random
    // sign with no large common part: its error, about 2^-17 of the sum of
    // the terms' magnitudes, moved every gradient by about 1e-5 relative at
    // L = 2048 and 4096, a twentieth of the 2e-4 bar. dP enters the
    // difference dP - D (the two-way split there moved the gamma gradient by
    // 2.8e-4 relative): it takes fp32-accurate products, the three-way split
    // (hi + mid + lo, six bf16 products) where the operands suit it. The
    // point columns of dQA' and dKA' (sum_j dS_ij Kg_j against
    // Qg_i sum_j dS_ij, coordinates of a hundred angstroms or more) cancel by
    // an order of magnitude and stay on fp32 products (narrow tiles).
    // dQA' = dS KA' (rows q0 .. q0 + qc): the scalar and pair columns on
    // the split path, the point columns (which cancel, see above) on fp32
    // products
    g.x3 = 1;
    g.M = qc; g.N = a.DA; g.K = L;
    g.A = a.Y; g.sAb = xs; g.am = L; g.ak = 1;
    g.B = a.KA; g.sBb = rowsK; g.bk = a.DAK; g.bn = 1;
    g.C = a.dQA + (size_t)q0 * a.DAK; g.sCb = rowsK; g.cm = a.DAK; g.acc = 0;
    if (gemm(g, BH, s) != hipSuccess) return hipErrorLaunchFailure;
    g.x3 = 0;
    g.N = a.DAK - a.DA;
    g.B = a.KA + a.DA;
    g.C = a.dQA + (size_t)q0 * a.DAK + a.DA;
    if (gemm(g, BH, s) != hipSuccess) return hipErrorLaunchFailure;
    // U = A z2
    g.x3 = 1;
    g.N = RCz;
    g.A = a.X;
    g.B = a.KA + a.C;
    g.C = a.U + (size_t)q0 * RCz; g.sCb = (long long)L * RCz; g.cm = RCz;
    if (gemm(g, BH, s) != hipSuccess) return hipErrorLaunchFailure;
    // dKA' += dS^T QA' (all keys): the scalar and pair columns on the split
    // path, the point columns on fp32 products, as for dQA'
    g.x3 = 1;
    g.M = L; g.N = a.DA; g.K = qc;
    g.A = a.Y; g.sAb = xs; g.am = 1; g.ak = L;
    g.B = a.QA + (size_t)q0 * a.DAQ; g.sBb = rowsQ; g.bk = a.DAQ; g.bn = 1;
    g.C = a.dKA; g.sCb = rowsQ; g.cm = a.DAQ; g.acc = q0 > 0;
    if (gemm(g, BH, s) != hipSuccess) return hipErrorLaunchFailure;
    g.x3 = 0;
    g.N = a.DAQ - a.DA;
    g.B = a.QA + (size_t)q0 * a.DAQ + a.DA;
    g.C = a.dKA + a.DA;
    if (gemm(g, BH, s) != hipSuccess) return hipErrorLaunchFailure;
    // dVA += A^T GA
    g.x3 = 1;
    g.N = a.DV;
    g.A = a.X;
    g.B = a.GA + (size_t)q0 * a.DV; g.sBb = rowsV; g.bk = a.DV; g.bn = 1;
    g.C = a.dVA; g.sCb = rowsV; g.cm = a.DV;
    if (gemm(g, BH, s) != hipSuccess) return hipErrorLaunchFailure;
  }
  return launch_backward_tail(a, s);
}

hipError_t launch_backward_tail(const BwdArgs& a, hipStream_t s) {
  const long long bih = (long long)a.B * a.L * a.H;
  const unsigned g64 = (unsigned)((bih + 63) / 64);
  hipLaunchKernelGGL(bwd_post_kernel, dim3(g64), dim3(64), 0, s, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const long long biz = (long long)a.B * a.L * a.Cz;
  hipLaunchKernelGGL(bwd_z_kernel, dim3((unsigned)((biz + 63) / 64)), dim3(64), 0, s, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const long long bi = (long long)a.B * a.L;
  hipLaunchKernelGGL(bwd_frames_kernel, dim3((unsigned)((bi + 63) / 64)), dim3(64), 0, s, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const int ncol = a.Cz * a.H + a.H;
  const int nblk = (int)((bi + kRedRows - 1) / kRedRows);
  hipLaunchKernelGGL(bwd_reduce1_kernel, dim3((ncol + 63) / 64, nblk), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(bwd_reduce2_kernel, dim3((ncol + 255) / 256), dim3(256), 0, s, a, nblk);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  return hipSuccess;
}

}  // namespace ipa
