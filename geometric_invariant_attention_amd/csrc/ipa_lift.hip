// ipa_lift: frames -> centred global points -> lifted query/key/value rows.
//
// For every residue block J of 64 residues and every head h this kernel
// writes the operands that the fused attention kernel consumes, so that the
// logit of "Flash Invariant Point Attention" (TL;DR: lift every IPA term
// into one regular attention) is a plain dot product plus cheap per-row /
// per-column terms:
//
//   query head row  [ a q | 2 k A'hi | 2 k A'hi | 2 k A'lo | 0 ]   (64 wide)
//   key head row    [   k |    B'hi  |    B'lo  |    B'hi  | 0 ]   (64 wide)
//   key pair row    [ z2_j1 | ... | z2_jR | 0 ]        (shared by all heads,
//                                                      stored in 64x64 panels)
//   value head row  [ v | G'hi x,y,z (8 each) | G'lo x,y,z | ]     (64 wide)
//   value pair row  [ z2_j1 | ... | z2_jR | 0 ]        (shared by all heads)
//
// with a = w_L log2(e) / sqrt(C), k = w_L gamma_h w_C / 2 log2(e), and
// A', B', G' the global query/key/value points R x + t minus the centre of
// their residue block. The squared distance of MEET's eq. 6 is expanded as
// in its eq. 7-8 (a distance becomes an inner product of augmented rows),
// here in the compact form |A|^2 + |B|^2 - 2 A.B; the norms and the
// block-centre offsets stay in float32 (kcol / qrow below), and the cross
// term A'.B' is carried by three bf16 products (hi.hi + hi.lo + lo.hi) so
// that bf16 rounding of coordinates does not reach the logits. The query
// pair part (w_L log2(e) W_b[:,h] * z1) is formed by the attention kernel
// itself from z1 and W_b.
//
// The pair parts of the query and key rows are fp16 on the bf16 path: the
// query side w_L W_b[:,h] * z1 is a rounded product, and fp16's 11-bit
// significand keeps the pair bias 8x closer to exact than bf16 would (z2
// itself converts exactly); all other lifted columns are bf16.
//
// (float32 storage has no hi/lo split: there the key head row carries B' at
// column 16 and the query head row carries the unscaled A' at column 32, and
// the attention kernel forms the point term from explicit differences.)
//
// Value rows are stored feature-major per 64-key block with the key order
// permuted to match the register layout of the attention probabilities, so
// the attention kernel reads them as matrix-core A operands directly.
//
// Residues with mask 0 and rows past L get all-zero rows and a key column
// term of -inf, so padding garbage never reaches a valid output.
//
// Grid: (block J, head h or pair panel, batch b). Head workgroups stage the
// block's frames and points in LDS and write the head rows with 16-byte
// stores; pair workgroups each write one 64-wide panel of z2 in both
// layouts.

#include "ipa_internal.h"

namespace ipa {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even (the hardware conversion; inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Loads from the inputs go through global-address-space pointers: generic
// loads could alias the LDS stores between them and would then each wait for
// the previous one; these issue back to back.
template <typename X>
__device__ __forceinline__ X ldg(const void* p, size_t i) {
  return static_cast<const __attribute__((address_space(1))) X*>(
      (const __attribute__((address_space(1))) void*)p)[i];
}

template <typename T> struct Elt;
template <> struct Elt<float> {
  static __device__ __forceinline__ float load(const void* p, size_t i) { return ldg<float>(p, i); }
  // hi/lo split of a value: fp32 storage keeps the value whole.
  static __device__ __forceinline__ void split(float x, float& hi, float& lo) {
    hi = x; lo = 0.f;
  }
  using S = float;
  static __device__ __forceinline__ S pack(float x) { return x; }
  static __device__ __forceinline__ S pack_pair(float x) { return x; }
};
template <> struct Elt<uint16_t> {
  static __device__ __forceinline__ float load(const void* p, size_t i) { return bf16_to_f32(ldg<uint16_t>(p, i)); }
  static __device__ __forceinline__ void split(float x, float& hi, float& lo) {
    hi = bf16_to_f32(f32_to_bf16(x));
    lo = bf16_to_f32(f32_to_bf16(x - hi));
  }
  using S = uint16_t;
  static __device__ __forceinline__ S pack(float x) { return f32_to_bf16(x); }
  // key pair columns (z2) are stored as fp16: exact for bf16 inputs in the
  // fp16 normal range, saturated beyond it
  static __device__ __forceinline__ S pack_pair(float x) {
    x = fminf(fmaxf(x, -65504.f), 65504.f);
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
};

// Key stored at position `pos` of a 64-key value block. The order matches
// the probability registers of the attention kernel's 32x32 products: for
// bf16 (K = 16 per product) each group of 16 keys is stored as 0-3, 8-11,
// 4-7, 12-15; for fp32 (K = 2 per product) each group of 32 keys is stored
// as pairs (8k+e, 8k+4+e).
template <typename T> __device__ __forceinline__ int key_of_pos(int pos);
template <> __device__ __forceinline__ int key_of_pos<uint16_t>(int pos) {
  int base = pos & ~15, p = pos & 15;
  int g = p >> 3, s = p & 7;
  return base + 8 * (s >> 2) + 4 * g + (s & 3);
}
template <> __device__ __forceinline__ int key_of_pos<float>(int pos) {
  int base = pos & ~31, p = pos & 31;
  int g = p & 1, st = p >> 1;
  return base + 8 * (st >> 2) + 4 * g + (st & 3);
}

// Store one 16-byte chunk of packed elements.
template <typename S, int N>
__device__ __forceinline__ void store16(S* dst, const S (&v)[N]) {
  static_assert(N * sizeof(S) == 16, "16-byte chunk");
  uint32_t w[4];
  __builtin_memcpy(w, v, 16);
  *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
}

template <typename T>
__global__ __launch_bounds__(256) void ipa_lift_kernel(FwdArgs a) {
  using S = typename Elt<T>::S;
  constexpr int EPC = 16 / sizeof(S);        // elements per 16-byte chunk
  const Layout& ly = a.lay;
  const int J = blockIdx.x, y = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int L = ly.L, H = ly.H, C = ly.C, Pqk = ly.Pqk, Pv = ly.Pv, RCz = ly.R * ly.Cz;
  const int Lp = ly.Lp, PW = ly.PW;

  __shared__ float sCen[4];
  __shared__ int sValid[kTileN];

  // --- block centre: mean translation of the valid residues (wave 0) ---
  if (tid < 64) {
    // loads are unconditional (rows past L read row L - 1) and their values
    // dropped afterwards, so that they issue together
    const int i = J * kTileN + tid, ic = i < L ? i : L - 1;
    const bool valid = (i < L) && (a.mask == nullptr || ldg<uint8_t>(a.mask, (size_t)b * L + ic) != 0);
    const size_t tb = ((size_t)b * L + ic) * 3;
    float tx = ldg<float>(a.trans, tb), ty = ldg<float>(a.trans, tb + 1), tz = ldg<float>(a.trans, tb + 2);
    if (!valid) { tx = 0.f; ty = 0.f; tz = 0.f; }
    float sx = tx, sy = ty, sz = tz, sn = valid ? 1.f : 0.f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      sx += __shfl_xor(sx, o, 64);
      sy += __shfl_xor(sy, o, 64);
      sz += __shfl_xor(sz, o, 64);
      sn += __shfl_xor(sn, o, 64);
    }
    const float inv = sn > 0.f ? 1.f / sn : 0.f;
    if (tid == 0) {
      sCen[0] = sx * inv; sCen[1] = sy * inv; sCen[2] = sz * inv; sCen[3] = sn;
      if (y == 0)
        reinterpret_cast<float4*>(a.ws + ly.off_cen)[(size_t)b * ly.nJ + J] =
            make_float4(sx * inv, sy * inv, sz * inv, sn);
    }
    sValid[tid] = valid ? 1 : 0;
  }
  __syncthreads();

  if (y < H) {
    // ================= head workgroup =================
    const int h = y;
    __shared__ float sS[3][kTileN][kCSlot + 1];     // q, k, v scalars (zero past C)
    __shared__ float sA[kTileN][16];                // centred query points (unscaled)
    __shared__ float sB[kTileN][16];                // centred key points
    __shared__ float sG[kTileN][3 * kPvSlot + 1];   // centred value points, [x|y|z] x 8
    const float log2e = kLog2e;
    const float alpha = a.w_L * rsqrtf((float)C) * log2e;
    const float kap = a.w_L * ldg<float>(a.gamma, h) * a.w_C * 0.5f * log2e;

    // ---- stage this head's inputs for the block in LDS ----
    // All threads copy, consecutive lanes on consecutive elements of the
    // residues' rows: frames, this head's query/key/value points and its
    // q/k/v scalars. Trip counts are fixed and every load is unconditional
    // (rows past L read row L - 1, columns past the row read column 0), so
    // the loads issue together; values outside the data are zeroed when the
    // rows are used.
    __shared__ float sFr[kTileN][12];                  // rotation (9), translation (3)
    __shared__ float sPt[kTileN][2 * 15 + 3 * kPvSlot];  // q points, k points, v points
    {
      const int nq = 3 * Pqk, nv = 3 * Pv;
      const float rq = 1.f / (float)nq, rv = 1.f / (float)nv;
      const size_t row0 = (size_t)b * L;
      auto res = [&](int j) -> size_t { const int i = J * kTileN + j; return row0 + (i < L ? i : L - 1); };
      constexpr int NR = (kTileN * 9 + 255) / 256, NT = (kTileN * 3 + 255) / 256;
      constexpr int NQ = (kTileN * 15 + 255) / 256, NV = (kTileN * 3 * kPvSlot + 255) / 256;
      constexpr int NS = 3 * kTileN * kCSlot / 256;
      float vr[NR], vt[NT], vq[NQ], vk[NQ], vv[NV], vs[NS];
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        const int e = tid + 256 * k, ec = e < kTileN * 9 ? e : 0;
        vr[k] = ldg<float>(a.rot, res(ec / 9) * 9 + ec % 9);
      }
#pragma unroll
      for (int k = 0; k < NT; ++k) {
        const int e = tid + 256 * k, ec = e < kTileN * 3 ? e : 0;
        vt[k] = ldg<float>(a.trans, res(ec / 3) * 3 + ec % 3);
      }
      // element e of the block's point rows: residue e / n, component e % n
      // (quotients from a float reciprocal: e < 1536 and n <= 24 keep
      // (e + 0.5) / n well clear of an integer)
#pragma unroll
      for (int k = 0; k < NQ; ++k) {
        const int e = tid + 256 * k, ec = e < kTileN * nq ? e : 0;
        const int j = (int)(((float)ec + 0.5f) * rq), c = ec - j * nq;
        const size_t o = (res(j) * H + h) * nq + c;
        vq[k] = Elt<T>::load(a.q_pts, o);
        vk[k] = Elt<T>::load(a.k_pts, o);
      }
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int e = tid + 256 * k, ec = e < kTileN * nv ? e : 0;
        const int j = (int)(((float)ec + 0.5f) * rv), c = ec - j * nv;
        vv[k] = Elt<T>::load(a.v_pts, (res(j) * H + h) * nv + c);
      }
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const int e = tid + 256 * k;
        const int which = e / (kTileN * kCSlot), j = (e / kCSlot) % kTileN, c = e % kCSlot;
        const void* src = which == 0 ? a.q : which == 1 ? a.k : a.v;
        vs[k] = Elt<T>::load(src, (res(j) * H + h) * C + (c < C ? c : 0));
      }
      // into LDS
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        const int e = tid + 256 * k;
        if (e < kTileN * 9) sFr[e / 9][e % 9] = vr[k];
      }
#pragma unroll
      for (int k = 0; k < NT; ++k) {
        const int e = tid + 256 * k;
        if (e < kTileN * 3) sFr[e / 3][9 + e % 3] = vt[k];
      }
#pragma unroll
      for (int k = 0; k < NQ; ++k) {
        const int e = tid + 256 * k;
        if (e < kTileN * nq) {
          const int j = (int)(((float)e + 0.5f) * rq), c = e - j * nq;
          sPt[j][c] = vq[k];
          sPt[j][15 + c] = vk[k];
        }
      }
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int e = tid + 256 * k;
        if (e < kTileN * nv) {
          const int j = (int)(((float)e + 0.5f) * rv), c = e - j * nv;
          sPt[j][30 + c] = vv[k];
        }
      }
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const int e = tid + 256 * k;
        const int which = e / (kTileN * kCSlot), j = (e / kCSlot) % kTileN, c = e % kCSlot;
        sS[which][j][c] = (sValid[j] && c < C) ? vs[k] : 0.f;
      }
    }
    __syncthreads();

    // wave 0: frames and points of one residue per lane, from LDS
    if (tid < 64) {
      const int j = tid, i = J * kTileN + j;
      const bool v = sValid[j];
      float R[9], tc[3];
#pragma unroll
      for (int e = 0; e < 9; ++e) R[e] = sFr[j][e];
#pragma unroll
      for (int x = 0; x < 3; ++x) tc[x] = sFr[j][9 + x] - sCen[x];
      float ax = 0.f, ay = 0.f, az = 0.f, bx = 0.f, by = 0.f, bz = 0.f, bn = 0.f;
#pragma unroll
      for (int p = 0; p < 5; ++p) {
        float A[3] = {0.f, 0.f, 0.f}, Bk[3] = {0.f, 0.f, 0.f};
        if (v && p < Pqk) {
          const float q0 = sPt[j][3 * p], q1 = sPt[j][3 * p + 1], q2 = sPt[j][3 * p + 2];
          const float k0 = sPt[j][15 + 3 * p], k1 = sPt[j][15 + 3 * p + 1], k2 = sPt[j][15 + 3 * p + 2];
#pragma unroll
          for (int x = 0; x < 3; ++x) {
            A[x] = R[3 * x] * q0 + R[3 * x + 1] * q1 + R[3 * x + 2] * q2 + tc[x];
            Bk[x] = R[3 * x] * k0 + R[3 * x + 1] * k1 + R[3 * x + 2] * k2 + tc[x];
          }
        }
#pragma unroll
        for (int x = 0; x < 3; ++x) { sA[j][3 * p + x] = A[x]; sB[j][3 * p + x] = Bk[x]; }
        ax += A[0]; ay += A[1]; az += A[2];
        bx += Bk[0]; by += Bk[1]; bz += Bk[2];
        bn += Bk[0] * Bk[0] + Bk[1] * Bk[1] + Bk[2] * Bk[2];
      }
      sA[j][15] = 0.f; sB[j][15] = 0.f;
#pragma unroll
      for (int p = 0; p < kPvSlot; ++p) {
        float G[3] = {0.f, 0.f, 0.f};
        if (v && p < Pv) {
          const float v0 = sPt[j][30 + 3 * p], v1 = sPt[j][30 + 3 * p + 1], v2 = sPt[j][30 + 3 * p + 2];
#pragma unroll
          for (int x = 0; x < 3; ++x) G[x] = R[3 * x] * v0 + R[3 * x + 1] * v1 + R[3 * x + 2] * v2 + tc[x];
        }
#pragma unroll
        for (int x = 0; x < 3; ++x) sG[j][kPvSlot * x + p] = G[x];
      }
      const size_t o = ((size_t)b * H + h) * Lp + i;
      // fp32 takes the whole point term from explicit differences
      reinterpret_cast<float4*>(a.ws + ly.off_kcol)[o] =
          !v ? make_float4(0.f, 0.f, 0.f, -INFINITY)
             : (sizeof(T) == 2 ? make_float4(bx, by, bz, -kap * bn) : make_float4(0.f, 0.f, 0.f, 0.f));
      reinterpret_cast<float4*>(a.ws + ly.off_qrow)[o] = make_float4(ax, ay, az, 0.f);
    }
    __syncthreads();

    // --- query / key head rows: 64 rows x 64 features ---
    S* qh = reinterpret_cast<S*>(a.ws + ly.off_qh) + (((size_t)b * H + h) * Lp + (size_t)J * kTileN) * kHeadW;
    S* kh = reinterpret_cast<S*>(a.ws + ly.off_kh) + (((size_t)b * H + h) * Lp + (size_t)J * kTileN) * kHeadW;
    const int G3 = 3 * Pqk;
    // u / G3 for u < 48: (u + 0.5) / G3 stays well clear of an integer, so
    // the float reciprocal gives the exact quotient without an integer divide
    const float rG3 = 1.f / (float)G3;
    for (int ch = tid; ch < kTileN * (kHeadW / EPC); ch += 256) {
      const int j = ch / (kHeadW / EPC), f0 = (ch % (kHeadW / EPC)) * EPC;
      S qv[EPC], kv[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const int f = f0 + e;
        float qo = 0.f, ko = 0.f;
        if (f < kCSlot) {
          qo = alpha * sS[0][j][f];
          ko = sS[1][j][f];
        } else if constexpr (sizeof(T) == 2) {
          const int u = f - kCSlot, grp = (int)(((float)u + 0.5f) * rG3), w = u - grp * G3;
          if (grp < 3) {
            float hi, lo;
            Elt<T>::split(2.f * kap * sA[j][w], hi, lo);
            qo = (grp == 2) ? lo : hi;
            Elt<T>::split(sB[j][w], hi, lo);
            ko = (grp == 1) ? lo : hi;
          }
        } else {
          // fp32: centred key points at 16.., centred query points (unscaled)
          // at 32..; the attention kernel takes the squared distance from
          // their explicit differences, so they must not meet in the product
          const int u = f - kCSlot;
          if (u < G3) ko = sB[j][u];
          if (f >= kFpQPts && f - kFpQPts < G3) qo = sA[j][f - kFpQPts];
        }
        qv[e] = Elt<T>::pack(qo);
        kv[e] = Elt<T>::pack(ko);
      }
      store16(qh + (size_t)j * kHeadW + f0, qv);
      store16(kh + (size_t)j * kHeadW + f0, kv);
    }

    // --- value head block, feature-major [64 features][64 key positions] ---
    S* vth = reinterpret_cast<S*>(a.ws + ly.off_vth) + (((size_t)b * H + h) * ly.nJ + J) * (kHeadW * kTileN);
    for (int ch = tid; ch < kHeadW * (kTileN / EPC); ch += 256) {
      const int f = ch / (kTileN / EPC), p0 = (ch % (kTileN / EPC)) * EPC;
      S vv[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const int j = key_of_pos<T>(p0 + e);
        float o = 0.f;
        if (f < kCSlot) {
          o = sS[2][j][f];
        } else {
          const int u = f - kCSlot;             // 0..47
          const int half = u / (3 * kPvSlot);   // 0 = hi, 1 = lo
          const int w = u - half * 3 * kPvSlot;
          float hi, lo;
          Elt<T>::split(sG[j][w], hi, lo);
          o = half ? lo : hi;
        }
        vv[e] = Elt<T>::pack(o);
      }
      store16(vth + (size_t)f * kTileN + p0, vv);
    }
  } else {
    // ================= pair workgroup: one 64-wide panel of z2 =================
    const int P = y - H;
    __shared__ float sZ[kTileN][64 + 1];
    {
      constexpr int NE = kTileN * 64 / 256;
      float val[NE];
#pragma unroll
      for (int k = 0; k < NE; ++k) {
        const int e = tid + 256 * k;
        const int j = e / 64, u = P * 64 + e % 64;
        const int i = J * kTileN + j, ic = i < L ? i : L - 1;
        val[k] = Elt<T>::load(a.z2, ((size_t)b * L + ic) * RCz + (u < RCz ? u : 0));
      }
#pragma unroll
      for (int k = 0; k < NE; ++k) {
        const int e = tid + 256 * k;
        const int j = e / 64, uu = e % 64;
        sZ[j][uu] = (sValid[j] && P * 64 + uu < RCz) ? val[k] : 0.f;
      }
    }
    __syncthreads();
    S* kz = reinterpret_cast<S*>(a.ws + ly.off_kz) + (((size_t)b * ly.nJ + J) * (PW / 64) + P) * (64 * kTileN);
    for (int ch = tid; ch < kTileN * (64 / EPC); ch += 256) {
      const int j = ch / (64 / EPC), u0 = (ch % (64 / EPC)) * EPC;
      S zv[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) zv[e] = Elt<T>::pack_pair(sZ[j][u0 + e]);
      store16(kz + (size_t)j * 64 + u0, zv);
    }
    S* vtz = reinterpret_cast<S*>(a.ws + ly.off_vtz) + (((size_t)b * ly.nJ + J) * PW + P * 64) * kTileN;
    for (int ch = tid; ch < 64 * (kTileN / EPC); ch += 256) {
      const int uu = ch / (kTileN / EPC), p0 = (ch % (kTileN / EPC)) * EPC;
      S zv[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) zv[e] = Elt<T>::pack(sZ[key_of_pos<T>(p0 + e)][uu]);
      store16(vtz + (size_t)uu * kTileN + p0, zv);
    }
  }
}

}  // namespace

hipError_t launch_lift(const FwdArgs& a, bool bf16, hipStream_t s) {
  dim3 grid(a.lay.nJ, a.lay.H + a.lay.PW / 64, a.lay.B);
  if (bf16)
    hipLaunchKernelGGL(ipa_lift_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(ipa_lift_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ipa
