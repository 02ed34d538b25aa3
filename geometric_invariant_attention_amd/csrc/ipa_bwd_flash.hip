// ipa_bwd_flash: the gradient of the fused IPA forward in flash form.
//
// The forward ("Flash Invariant Point Attention", TL;DR and abstract; MEET
// section 2.2 eq. 6 for the distance term) is one softmax attention over
// lifted rows; its gradient (written out in ipa_bwd.hip) needs, per batch b
// and head h, the scores S, the probabilities A and dS = A (dP - D) of every
// (query, key) pair. Here none of them is stored: they are formed tile by
// tile in registers and LDS and used at once, so the workspace is linear in
// L (the abstract's point: training at lengths that quadratic memory rules
// out). Three passes over the same lifted rows:
//
//   statistics  one workgroup per 32 query rows of one (b, h), keys streamed
//               in tiles of 64: scores and dP on the matrix cores, the point
//               term from explicit differences, an online softmax (running
//               max, rescaled sums). Stores the row max, 1 / row sum and
//               D_i = sum_j A_ij dP_ij. D is taken from the products the
//               other passes form rather than from the forward outputs
//               (GA . O): dP rounds GA to bf16 once per row, and only the
//               matching D keeps sum_j dS_ij = 0 (with a single key, dS = 0).
//   query pass  the same blocks: A and dS = A (dP - D) from the statistics;
//               dQA = sum_j dS_ij KA_j, U = sum_j A_ij z2_j, the row sums of
//               dS, dS Kg and dS d (gamma).
//   key pass    one workgroup per 32 keys, queries streamed in tiles of 64:
//               dKA = sum_i dS_ij QA_i, dVA = sum_i A_ij GA_i, the column sums
//               of dS and dS Qg.
//
// All passes run the same loop with the roles of the two sides swapped:
//   phase 1  T1 = A1 B1^T (lifted dot, K = WQ) and T2 = A2 B2^T (dP, K = WG),
//            32 x 64 each; the four waves take one 32 x 32 block each
//            (v_mfma_f32_32x32x16_bf16, both operands from LDS: the
//            stationary rows are staged once per workgroup);
//   phase V  per element on the vector units: the squared point distance,
//            the logit, A (exp2), dS, the row or column sums; A and dS
//            rounded to bf16 into LDS;
//   phase 2  the accumulating products over the tile's 64 streamed rows,
//            output blocks of 32 x 32 dealt round-robin to the waves (not in
//            the statistics pass).
// The next tile's rows are loaded into registers while the current one is
// computed.
//
// Operands (bf16, round to nearest even; widths padded with zeros to
// multiples of 32): QX = [w_L/sqrt(C) q | w_L W_b[:,h] z1], KX = [k | z2];
// dP = GA . VA is taken as GX . VX with GX = [g_s | Rg hi | Rg hi | Rg lo |
// z1 g_pair], VX = [v | Vg hi | Vg lo | Vg hi | z2], so the point part
// (global coordinates of a hundred angstrom or more, which cancel in
// dP - D) carries hi*hi + hi*lo + lo*hi, about 2^-17 relative, while the
// scalar and pair parts take one bf16 product. dVA's point columns are the
// sum of the hi and lo columns of P^T GX. The distance term and every sum
// against the points stay in fp32 on the vector units.
//
// The per-residue chain rule (dq ... dgamma) is the one of the chunked form,
// launch_backward_tail in ipa_bwd.hip.

#include "ipa_internal.h"

namespace ipa {
namespace {

typedef __bf16 fbf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t fu16x8 __attribute__((ext_vector_type(8)));
typedef float ff32x16 __attribute__((ext_vector_type(16)));
typedef float ff32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int uint32x4_t __attribute__((ext_vector_type(4)));

constexpr int kFR = 32;                 // stationary rows per workgroup
constexpr int kFT = 64;                 // streamed rows per tile
constexpr int kMaxWQ = 288, kMaxWG = 352;
constexpr int kMaxPQ = 296, kMaxPG = 360;   // LDS row pitches (elements)
constexpr int kFMaxP3 = 15;
constexpr int kMaxBlk = (kMaxWQ + kMaxWG) / 32 / 4;          // output blocks per wave
constexpr int kU1 = (kFT * kMaxWQ / 8 + 255) / 256;   // 16-byte loads per thread per tile of B1
constexpr int kU2 = (kFT * kMaxWG / 8 + 255) / 256;   // and of B2
static_assert(kFR * ((kMaxWQ + kMaxWG) + 4) * 4 <= kFT * (kMaxPQ + kMaxPG) * 2, "epilogue staging fits the tile buffer");

// LDS pitch of a row of W bf16 (W a multiple of 32): 16-byte aligned rows,
// 8 consecutive rows on disjoint banks for 16-byte reads, and rows 8 apart
// on disjoint bank halves for the 2-byte reads of the accumulating products.
__host__ __device__ constexpr int fpitch(int W) { return W + ((W & 63) ? 8 : 40); }

__device__ __forceinline__ uint16_t to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float from_bf16(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

__device__ __forceinline__ bool fvalid(const BwdArgs& a, int b, int i) {
  return a.mask == nullptr || a.mask[(size_t)b * a.L + i] != 0;
}

__device__ __forceinline__ ff32x16 fmma(fbf16x8 x, fbf16x8 y, ff32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// bwdf_prep: one wave per (b, i, h); lanes over the columns of the lifted rows.
__global__ __launch_bounds__(256) void bwdf_prep_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int H = a.H, L = a.L, C = a.C, P = a.Pqk, Pv = a.Pv, RCz = a.R * a.Cz, Cz = a.Cz, bf = a.in_bf16;
  if (t >= (long long)a.B * L * H) return;
  const int h = (int)(t % H);
  const int i = (int)((t / H) % L);
  const int b = (int)(t / ((long long)H * L));
  const size_t bi = (size_t)b * L + i, bih = bi * H + h;
  const size_t row = ((size_t)b * H + h) * L + i;
  const bool valid = fvalid(a, b, i);
  const float* R = a.rot + bi * 9;
  const float* T = a.trans + bi * 3;
  const float alpha = a.w_L / sqrtf((float)C);
  auto gpt = [&](const void* base, size_t e, int x) {
    return R[3 * x] * ldin(base, e, bf) + R[3 * x + 1] * ldin(base, e + 1, bf) + R[3 * x + 2] * ldin(base, e + 2, bf) + T[x];
  };
  for (int c = lane; c < a.WQ; c += 64) {
    float vq = 0.f, vk = 0.f;
    if (c < C) {
      vq = alpha * ldin(a.q, bih * C + c, bf);
      vk = ldin(a.k, bih * C + c, bf);
    } else if (c < C + RCz) {
      const int rc = c - C;
      vq = a.w_L * a.w_b[(size_t)(rc % Cz) * H + h] * ldin(a.z1, bi * RCz + rc, bf);
      vk = ldin(a.z2, bi * RCz + rc, bf);
    }
    a.QX[row * a.WQ + c] = to_bf16(vq);
    a.KX[row * a.WQ + c] = to_bf16(vk);
  }
  for (int e = lane; e < a.P3; e += 64) {
    const int p = e / 3, x = e - 3 * p;
    a.QP[row * a.P3 + e] = gpt(a.q_pts, (bih * P + p) * 3, x);
    a.KP[row * a.P3 + e] = gpt(a.k_pts, (bih * P + p) * 3, x);
  }
  // GX, VX (D_i comes from the statistics pass)
  const int P3v = 3 * Pv;
  for (int c = lane; c < a.WG; c += 64) {
    uint16_t gx = 0, vx = 0;
    if (c < C) {
      vx = to_bf16(ldin(a.v, bih * C + c, bf));
      if (valid) gx = to_bf16(a.g_s[bih * C + c]);
    } else if (c < C + 3 * P3v) {
      const int e = c - C, seg = e / P3v, e3 = e - seg * P3v, p = e3 / 3, x = e3 - 3 * p;
      const float vg = gpt(a.v_pts, (bih * Pv + p) * 3, x);
      const uint16_t vh = to_bf16(vg), vl = to_bf16(vg - from_bf16(vh));
      float rg = 0.f;
      if (valid) {
        const float* op = a.o_pts + (bih * Pv + p) * 3;
        const float* gp = a.g_pts + (bih * Pv + p) * 3;
        const float n2 = op[0] * op[0] + op[1] * op[1] + op[2] * op[2];
        const float s = n2 > 0.f ? a.g_norm[bih * Pv + p] / sqrtf(n2) : 0.f;
        rg = R[3 * x] * (gp[0] + s * op[0]) + R[3 * x + 1] * (gp[1] + s * op[1]) + R[3 * x + 2] * (gp[2] + s * op[2]);
      }
      const uint16_t gh = to_bf16(rg), gl = to_bf16(rg - from_bf16(gh));
      gx = seg == 2 ? gl : gh;
      vx = seg == 1 ? vl : vh;
    } else if (c < C + 3 * P3v + RCz) {
      const int rc = c - C - 3 * P3v;
      vx = to_bf16(ldin(a.z2, bi * RCz + rc, bf));
      if (valid) gx = to_bf16(ldin(a.z1, bi * RCz + rc, bf) * a.g_pair[bih * Cz + rc % Cz]);
    }
    a.GX[row * a.WG + c] = gx;
    a.VX[row * a.WG + c] = vx;
  }
}

// ---------------------------------------------------------------------------
// bwdf_pass: MODE 0 the statistics pass, 1 the query pass, 2 the key pass
// (see the top).
template <int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwdf_pass_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sB[kFT * (kMaxPQ + kMaxPG)];   // B1 tile, then B2 tile
  __shared__ __attribute__((aligned(16))) uint16_t sA[kFR * (kMaxPQ + kMaxPG)];   // A1 rows, then A2 rows
  __shared__ __attribute__((aligned(16))) float sT[2][kFR][kFT + 4];             // T1, T2
  __shared__ __attribute__((aligned(16))) uint16_t sX[2][kFR][kFT + 8];          // A, dS (bf16)
  __shared__ __attribute__((aligned(16))) float sPt[kFMaxP3][kFT];               // streamed points
  __shared__ __attribute__((aligned(16))) ff32x4 sSt[kFT];                       // streamed row terms

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  constexpr bool KEYS = MODE == 2, STATS = MODE == 0;
  const int bh = blockIdx.y, H = a.H, L = a.L, P3 = a.P3;
  const int b = bh / H, h = bh - b * H;
  const int r0 = blockIdx.x * kFR;
  const int WQ = a.WQ, WG = a.WG, pQ = fpitch(WQ), pG = fpitch(WG);
  const float kappa = a.w_L * a.gamma[h] * a.w_C * 0.5f;
  const size_t rowbase = (size_t)bh * L;
  const uint16_t* A1 = KEYS ? a.KX : a.QX;
  const uint16_t* A2 = KEYS ? a.VX : a.GX;
  const uint16_t* B1 = KEYS ? a.QX : a.KX;
  const uint16_t* B2 = KEYS ? a.GX : a.VX;
  const float* SP = KEYS ? a.KP : a.QP;
  const float* TP = KEYS ? a.QP : a.KP;
  const int n1 = WQ / 32, n2 = KEYS ? WG / 32 : (a.R * a.Cz + 31) / 32, nblk = n1 + n2;
  const int nmine = (!STATS && nblk > w) ? (nblk - w + 3) / 4 : 0;

  // stationary rows of both products in LDS (read by phase 1 of every tile)
  const int sel = w >> 1, nb = w & 1;
  const int nk1 = (sel ? WG : WQ) / 16;
  {
    const int nQ8 = WQ / 8, nG8 = WG / 8, nA = kFR * (nQ8 + nG8);
    for (int e = tid; e < nA; e += 256) {
      const bool one = e < kFR * nQ8;
      const int ee = one ? e : e - kFR * nQ8, n8 = one ? nQ8 : nG8, q = ee / n8, ch = ee - q * n8, r = r0 + q;
      uint4 v = {0u, 0u, 0u, 0u};
      if (r < L) v = *reinterpret_cast<const uint4*>((one ? A1 : A2) + (rowbase + r) * (size_t)(8 * n8) + 8 * ch);
      *reinterpret_cast<uint4*>(one ? sA + q * pQ + 8 * ch : sA + kFR * pQ + q * pG + 8 * ch) = v;
    }
  }
  // this thread's row and columns in phase V
  const int rr = tid >> 3, c0 = 8 * (tid & 7), myrow = r0 + rr;
  float sp[kFMaxP3];
#pragma unroll
  for (int c = 0; c < kFMaxP3; ++c) sp[c] = (c < P3 && myrow < L) ? SP[(rowbase + myrow) * P3 + c] : 0.f;
  const bool rvalid = myrow < L && fvalid(a, b, myrow);
  // the query pass's own row: max (base 2), 1 / sum and D from the statistics pass
  const float mr = (MODE == 1 && myrow < L) ? a.ST[2 * (rowbase + myrow)] : 0.f;
  const float invr = (MODE == 1 && myrow < L) ? a.ST[2 * (rowbase + myrow) + 1] : 0.f;
  const float Dr = (MODE == 1 && myrow < L) ? a.Dv[rowbase + myrow] : 0.f;

  // streamed tile copies through buffer loads: 16-byte unit u of this thread
  // is row q, chunk ch of B1 (units of key1) or B2 (key2); a key packs the
  // byte offset within the tile (low 16 bits) and the LDS element offset
  // (high 16 bits). Rows past L lie beyond the resource and load zeros.
  const int nQ8 = WQ / 8, nG8 = WG / 8;
  uint32_t key1[kU1], key2[kU2];
#pragma unroll
  for (int u = 0; u < kU1; ++u) {
    const int e = tid + 256 * u, q = e / nQ8, ch = e - q * nQ8;
    key1[u] = e < kFT * nQ8 ? (uint32_t)(q * WQ * 2 + 16 * ch) | (uint32_t)(q * pQ + 8 * ch) << 16 : 0xffffffffu;
  }
#pragma unroll
  for (int u = 0; u < kU2; ++u) {
    const int e = tid + 256 * u, q = e / nG8, ch = e - q * nG8;
    key2[u] = e < kFT * nG8 ? (uint32_t)(q * WG * 2 + 16 * ch) | (uint32_t)(q * pG + 8 * ch) << 16 : 0xffffffffu;
  }
  uint4 pf1[kU1], pf2[kU2];
  float pp[4];
  ff32x4 pst = {0.f, 0.f, 0.f, 0.f};
  auto prefetch = [&](int s0) {
    const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(B1 + (rowbase + s0) * (size_t)WQ), (short)0, (int)((L - s0) * WQ * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t r2 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(B2 + (rowbase + s0) * (size_t)WG), (short)0, (int)((L - s0) * WG * 2), 0x00020000);
#pragma unroll
    for (int u = 0; u < kU1; ++u) {
      const uint32x4_t v = key1[u] != 0xffffffffu ? __builtin_amdgcn_raw_buffer_load_b128(r1, key1[u] & 0xffffu, 0, 0)
                                                 : uint32x4_t{0u, 0u, 0u, 0u};
      pf1[u] = uint4{v[0], v[1], v[2], v[3]};
    }
#pragma unroll
    for (int u = 0; u < kU2; ++u) {
      const uint32x4_t v = key2[u] != 0xffffffffu ? __builtin_amdgcn_raw_buffer_load_b128(r2, key2[u] & 0xffffu, 0, 0)
                                                 : uint32x4_t{0u, 0u, 0u, 0u};
      pf2[u] = uint4{v[0], v[1], v[2], v[3]};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u;
      float v = 0.f;
      if (e < kFT * P3) {
        const int q = e / P3, s = s0 + q;
        if (s < L) v = TP[(rowbase + s) * P3 + (e - q * P3)];
      }
      pp[u] = v;
    }
    if (tid < kFT) {
      const int s = s0 + tid;
      if (KEYS) {
        pst = s < L ? ff32x4{a.ST[2 * (rowbase + s)], a.ST[2 * (rowbase + s) + 1], a.Dv[rowbase + s], 0.f}
                    : ff32x4{0.f, 0.f, 0.f, 0.f};
      } else {
        pst = ff32x4{(s < L && fvalid(a, b, s)) ? 0.f : -INFINITY, 0.f, 0.f, 0.f};
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < kU1; ++u)
      if (key1[u] != 0xffffffffu) *reinterpret_cast<uint4*>(sB + (key1[u] >> 16)) = pf1[u];
#pragma unroll
    for (int u = 0; u < kU2; ++u)
      if (key2[u] != 0xffffffffu) *reinterpret_cast<uint4*>(sB + kFT * pQ + (key2[u] >> 16)) = pf2[u];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u;
      if (e < kFT * P3) {
        const int q = e / P3;
        sPt[e - q * P3][q] = pp[u];
      }
    }
    if (tid < kFT) sSt[tid] = pst;
  };

  ff32x16 acc[kMaxBlk];
#pragma unroll
  for (int j = 0; j < kMaxBlk; ++j) acc[j] = ff32x16{};
  // phase V state: running max (query pass), partial sums of this thread
  float m = -INFINITY, lp = 0.f, rs = 0.f, gm = 0.f, pq[kFMaxP3];
#pragma unroll
  for (int c = 0; c < kFMaxP3; ++c) pq[c] = 0.f;

  const int ntile = (L + kFT - 1) / kFT;
  prefetch(0);
  for (int t = 0; t < ntile; ++t) {
    stage();
    __syncthreads();
    if (t + 1 < ntile) prefetch((t + 1) * kFT);

    // phase 1: one 32 x 32 block of T1 (waves 0, 1) or T2 (waves 2, 3)
    {
      const int pitch = sel ? pG : pQ;
      const uint16_t* bt = sB + (sel ? kFT * pQ : 0) + (32 * nb + l32) * pitch + 8 * half;
      const uint16_t* at = sA + (sel ? kFR * pQ : 0) + l32 * pitch + 8 * half;
      ff32x16 c = ff32x16{};
#pragma unroll 2
      for (int k = 0; k < nk1; ++k)
          c = fmma(__builtin_bit_cast(fbf16x8, *reinterpret_cast<const uint4*>(at + 16 * k)),
                   __builtin_bit_cast(fbf16x8, *reinterpret_cast<const uint4*>(bt + 16 * k)), c);
#pragma unroll
      for (int i = 0; i < 16; ++i) sT[sel][8 * (i >> 2) + 4 * half + (i & 3)][32 * nb + l32] = c[i];
    }
    __syncthreads();

    // phase V
    {
      const ff32x4* t1v = reinterpret_cast<const ff32x4*>(&sT[0][rr][c0]);
      const ff32x4* t2v = reinterpret_cast<const ff32x4*>(&sT[1][rr][c0]);
      const ff32x4 t1a = t1v[0], t1b = t1v[1], t2a = t2v[0], t2b = t2v[1];
      float t1[8] = {t1a[0], t1a[1], t1a[2], t1a[3], t1b[0], t1b[1], t1b[2], t1b[3]};
      float t2[8] = {t2a[0], t2a[1], t2a[2], t2a[3], t2b[0], t2b[1], t2b[2], t2b[3]};
      float d[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) d[e] = 0.f;
#pragma unroll
      for (int c = 0; c < kFMaxP3; ++c) {
        if (c < P3) {
          const ff32x4 va = *reinterpret_cast<const ff32x4*>(&sPt[c][c0]);
          const ff32x4 vb = *reinterpret_cast<const ff32x4*>(&sPt[c][c0 + 4]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float df = sp[c] - (e < 4 ? va[e] : vb[e - 4]);
            d[e] = fmaf(df, df, d[e]);
          }
        }
      }
      float p[8], ds[8];
      if (STATS) {
        // online max and sum; D_i = sum_j A_ij dP_ij from the same dP the
        // other passes form, so that sum_j dS_ij vanishes up to rounding
        float x[8], tm = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[e] = rvalid ? fmaf(-kappa, d[e], t1[e]) * kLog2e + sSt[c0 + e][0] : -INFINITY;
          tm = fmaxf(tm, x[e]);
        }
        tm = fmaxf(tm, __shfl_xor(tm, 1));
        tm = fmaxf(tm, __shfl_xor(tm, 2));
        tm = fmaxf(tm, __shfl_xor(tm, 4));
        const float mn = fmaxf(m, tm);
        const float al = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mn);
        const float ms = mn == -INFINITY ? 0.f : mn;
        lp *= al;
        rs *= al;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = __builtin_amdgcn_exp2f(x[e] - ms);
          lp += pe;
          rs = fmaf(pe, t2[e], rs);
          p[e] = ds[e] = 0.f;
        }
        m = mn;
      } else if (MODE == 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = rvalid ? fmaf(-kappa, d[e], t1[e]) * kLog2e + sSt[c0 + e][0] : -INFINITY;
          p[e] = __builtin_amdgcn_exp2f(x - mr) * invr;
          ds[e] = p[e] * (t2[e] - Dr);
          rs += ds[e];
          gm = fmaf(ds[e], d[e], gm);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const ff32x4 st = sSt[c0 + e];
          const float x = fmaf(-kappa, d[e], t1[e]) * kLog2e;
          p[e] = st[1] > 0.f ? __builtin_amdgcn_exp2f(x - st[0]) * st[1] : 0.f;
          ds[e] = p[e] * (t2[e] - st[2]);
          rs += ds[e];
        }
      }
      // sums of dS against the streamed points (Kg on the query pass, Qg on the key pass)
#pragma unroll
      for (int c = 0; c < kFMaxP3; ++c) {
        if (!STATS && c < P3) {
          const ff32x4 va = *reinterpret_cast<const ff32x4*>(&sPt[c][c0]);
          const ff32x4 vb = *reinterpret_cast<const ff32x4*>(&sPt[c][c0 + 4]);
          float s = pq[c];
#pragma unroll
          for (int e = 0; e < 8; ++e) s = fmaf(ds[e], e < 4 ? va[e] : vb[e - 4], s);
          pq[c] = s;
        }
      }
      fu16x8 pb, sb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[e] = to_bf16(p[e]);
        sb[e] = to_bf16(ds[e]);
      }
      if (!STATS) {
        *reinterpret_cast<fu16x8*>(&sX[0][rr][c0]) = pb;
        *reinterpret_cast<fu16x8*>(&sX[1][rr][c0]) = sb;
      }
    }
    if (STATS) {
      __syncthreads();
      continue;
    }
    __syncthreads();

    // phase 2: accumulate dS B1 (blocks < n1) and A B1[:, C ..] (query
    // pass) or A B2 (key pass) over the tile's 64 streamed rows
    {
      fbf16x8 aP[4], aS[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        aP[kk] = __builtin_bit_cast(fbf16x8, *reinterpret_cast<const uint4*>(&sX[0][l32][16 * kk + 8 * half]));
        aS[kk] = __builtin_bit_cast(fbf16x8, *reinterpret_cast<const uint4*>(&sX[1][l32][16 * kk + 8 * half]));
      }
#pragma unroll
      for (int j = 0; j < kMaxBlk; ++j) {
        if (j < nmine) {
          const int blk = w + 4 * j;
          const bool first = blk < n1;
          const uint16_t* bt;
          int pitch;
          if (first) {
            bt = sB + 32 * blk + l32;
            pitch = pQ;
          } else if (!KEYS) {
            bt = sB + a.C + 32 * (blk - n1) + l32;
            pitch = pQ;
          } else {
            bt = sB + kFT * pQ + 32 * (blk - n1) + l32;
            pitch = pG;
          }
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const uint16_t* col = bt + (16 * kk + 8 * half) * pitch;
            fu16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = col[e * pitch];
            acc[j] = fmma(first ? aS[kk] : aP[kk], __builtin_bit_cast(fbf16x8, v), acc[j]);
          }
        }
      }
    }
    __syncthreads();
  }

  // row (query pass) or column (key pass) sums over the eight lanes of a row
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    lp += __shfl_xor(lp, o);
    rs += __shfl_xor(rs, o);
    gm += __shfl_xor(gm, o);
#pragma unroll
    for (int c = 0; c < kFMaxP3; ++c) pq[c] += __shfl_xor(pq[c], o);
  }
  if ((tid & 7) == 0 && myrow < L) {
    const size_t g = rowbase + myrow;
    if (STATS) {
      const float inv = lp > 0.f ? 1.f / lp : 0.f;
      a.ST[2 * g] = m == -INFINITY ? 0.f : m;
      a.ST[2 * g + 1] = inv;
      a.Dv[g] = rs * inv;
    } else if (MODE == 1) {
      a.rsum[g] = rs;
      a.gam[g] = gm;
      for (int c = 0; c < P3; ++c) a.dQA[g * a.DAK + a.DA + c] = pq[c];
    } else {
      for (int c = 0; c < P3; ++c) a.dKA[g * a.DAQ + a.DA + c] = pq[c];
      a.dKA[g * a.DAQ + a.DA + P3] = rs;
    }
  }
  if (STATS) return;
  // accumulators through LDS (the tile buffer, free after the loop's last
  // barrier) so that every output row is written by consecutive lanes
  float* stg = reinterpret_cast<float*>(sB);
  const int NS = 32 * nblk + 4;
#pragma unroll
  for (int j = 0; j < kMaxBlk; ++j)
    if (j < nmine)
#pragma unroll
      for (int i = 0; i < 16; ++i) stg[(8 * (i >> 2) + 4 * half + (i & 3)) * NS + 32 * (w + 4 * j) + l32] = acc[j][i];
  __syncthreads();
  const int C = a.C, RCz = a.R * a.Cz, DA = a.DA, Pv3 = 3 * a.Pv;
  for (int r = w; r < kFR; r += 4) {
    const int row = r0 + r;
    if (row >= L) break;
    const float* sr = stg + r * NS;
    const size_t g = rowbase + row;
    if (!KEYS) {
      for (int c = lane; c < DA; c += 64) a.dQA[g * a.DAK + c] = sr[c];
      for (int c = lane; c < RCz; c += 64) a.U[g * RCz + c] = sr[32 * n1 + c];
    } else {
      for (int c = lane; c < DA; c += 64) a.dKA[g * a.DAQ + c] = sr[c];
      const float* sv = sr + 32 * n1;
      for (int c = lane; c < a.DV; c += 64) {
        float v;
        if (c < C) v = sv[c];
        else if (c < C + Pv3) v = sv[c] + sv[c + 2 * Pv3];
        else v = sv[c + 2 * Pv3];
        a.dVA[g * a.DV + c] = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_backward_flash(const BwdArgs& a, hipStream_t s) {
  if (a.WQ > kMaxWQ || a.WG > kMaxWG || a.P3 > kFMaxP3 || (a.WQ & 31) || (a.WG & 31)) return hipErrorInvalidValue;
  const long long bih = (long long)a.B * a.L * a.H;
  hipLaunchKernelGGL(bwdf_prep_kernel, dim3((unsigned)((bih + 3) / 4)), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const dim3 grid((unsigned)((a.L + kFR - 1) / kFR), (unsigned)(a.B * a.H));
  hipLaunchKernelGGL(bwdf_pass_kernel<0>, grid, dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(bwdf_pass_kernel<1>, grid, dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(bwdf_pass_kernel<2>, grid, dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  return launch_backward_tail(a, s);
}

}  // namespace ipa
