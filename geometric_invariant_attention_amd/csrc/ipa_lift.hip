// ipa_lift: frames -> centred global points -> lifted query/key/value rows.
//
// For every residue block J of 64 residues (the key tile of the attention
// kernel) and every head h this kernel writes the operands that the fused
// attention kernel consumes, so that the logit of "Flash Invariant Point
// Attention" (TL;DR: lift every IPA term into one regular attention) is a
// plain dot product plus cheap per-row / per-column terms:
//
//   query head row  [ a q | 2 k A'hi | 2 k A'hi | 2 k A'lo | 0 ]   (64 wide)
//   key head row    [   k |    B'hi  |    B'lo  |    B'hi  | 0 ]   (64 wide)
//   key pair row    [ z2_j1 | ... | z2_jR | 0 ]        (shared by all heads,
//                                                      stored in 64x64 panels)
//
// The pair parts of the query and key rows are fp16 on the bf16 path: the
// query side w_L W_b[:,h] * z1 is a rounded product, and fp16's 11-bit
// significand keeps the pair bias 8x closer to exact than bf16 would (z2
// itself converts exactly); all other lifted columns are bf16.
//   value head row  [ v | G'hi x,y,z (8 each) | G'lo x,y,z | ]     (64 wide)
//
// (float32 storage has no hi/lo split: there the key head row carries B' at
// column 16 and the query head row carries the unscaled A' at column 32, and
// the attention kernel forms the point term from explicit differences.)
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
// itself from z1 and the transposed weights written here.
//
// Value rows are stored feature-major per 64-key tile with the key order
// permuted to match the register layout of the attention probabilities, so
// the attention kernel reads them as matrix-core A operands directly.
//
// Residues with mask 0 and rows past L get all-zero rows and a key column
// term of -inf, so padding garbage never reaches a valid output.

#include "ipa_internal.h"

namespace ipa {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even; inputs are finite by construction.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct Elt;
template <> struct Elt<float> {
  static __device__ __forceinline__ float load(const void* p, size_t i) {
    return static_cast<const float*>(p)[i];
  }
  // hi/lo split of a value: fp32 storage keeps the value whole.
  static __device__ __forceinline__ void split(float x, float& hi, float& lo) {
    hi = x; lo = 0.f;
  }
  static __device__ __forceinline__ float store_val(float x) { return x; }
  using S = float;
  static __device__ __forceinline__ S pack(float x) { return x; }
  static __device__ __forceinline__ S pack_pair(float x) { return x; }
};
template <> struct Elt<uint16_t> {
  static __device__ __forceinline__ float load(const void* p, size_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
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

// Key stored at position `pos` of a 64-key value tile. The order matches the
// probability registers of the attention kernel's 32x32 products: for bf16
// (K = 16 per product) each group of 16 keys is stored as
// 0-3, 8-11, 4-7, 12-15; for fp32 (K = 2 per product) each group of 32 keys
// is stored as pairs (8k+e, 8k+4+e).
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

struct alignas(16) Vec16 { uint32_t w[4]; };

template <typename T>
__global__ __launch_bounds__(256) void ipa_lift_kernel(FwdArgs a) {
  using S = typename Elt<T>::S;
  const Layout& ly = a.lay;
  const int J = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int L = ly.L, H = ly.H, C = ly.C, Pqk = ly.Pqk, Pv = ly.Pv, RCz = ly.R * ly.Cz;
  const int Lp = ly.Lp, PW = ly.PW;

  __shared__ float sR[kTileN][9];
  __shared__ float sT[kTileN][3];   // t - c (translation relative to the block centre)
  __shared__ int sValid[kTileN];
  __shared__ float sCen[4];

  // --- block centre: mean translation of the valid residues (wave 0) ---
  if (tid < 64) {
    const int i = J * kTileN + tid;
    const bool valid = (i < L) && (a.mask == nullptr || a.mask[(size_t)b * L + i] != 0);
    float tx = 0.f, ty = 0.f, tz = 0.f, n = valid ? 1.f : 0.f;
    if (valid) {
      const float* t = a.trans + ((size_t)b * L + i) * 3;
      tx = t[0]; ty = t[1]; tz = t[2];
    }
    float sx = tx, sy = ty, sz = tz, sn = n;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      sx += __shfl_xor(sx, o, 64);
      sy += __shfl_xor(sy, o, 64);
      sz += __shfl_xor(sz, o, 64);
      sn += __shfl_xor(sn, o, 64);
    }
    const float inv = sn > 0.f ? 1.f / sn : 0.f;
    const float cx = sx * inv, cy = sy * inv, cz = sz * inv;
    if (tid == 0) {
      sCen[0] = cx; sCen[1] = cy; sCen[2] = cz; sCen[3] = sn;
      float4* cen = reinterpret_cast<float4*>(a.ws + ly.off_cen);
      cen[(size_t)b * ly.nJ + J] = make_float4(cx, cy, cz, sn);
    }
    sValid[tid] = valid ? 1 : 0;
    if (valid) {
      const float* r = a.rot + ((size_t)b * L + i) * 9;
#pragma unroll
      for (int e = 0; e < 9; ++e) sR[tid][e] = r[e];
      sT[tid][0] = tx - cx; sT[tid][1] = ty - cy; sT[tid][2] = tz - cz;
    } else {
#pragma unroll
      for (int e = 0; e < 9; ++e) sR[tid][e] = 0.f;
      sT[tid][0] = sT[tid][1] = sT[tid][2] = 0.f;
    }
  }
  __syncthreads();

  const float log2e = kLog2e;
  const float alpha = a.w_L * rsqrtf((float)C) * log2e;

  // centred global point x of residue slot j: R_j p + (t_j - c)
  auto gpt = [&](int j, const void* pts, size_t base, int x) -> float {
    const float p0 = Elt<T>::load(pts, base + 0);
    const float p1 = Elt<T>::load(pts, base + 1);
    const float p2 = Elt<T>::load(pts, base + 2);
    return sR[j][3 * x + 0] * p0 + sR[j][3 * x + 1] * p1 + sR[j][3 * x + 2] * p2 + sT[j][x];
  };

  // --- query / key head rows: H x 64 rows x 8 chunks of 8 features ---
  {
    S* qh = reinterpret_cast<S*>(a.ws + ly.off_qh);
    S* kh = reinterpret_cast<S*>(a.ws + ly.off_kh);
    const int G3 = 3 * Pqk;
    for (int ch = tid; ch < H * kTileN * 8; ch += 256) {
      const int h = ch / (kTileN * 8), j = (ch >> 3) & 63, f0 = (ch & 7) * 8;
      const int i = J * kTileN + j;
      const float kap2 = 2.f * a.w_L * a.gamma[h] * a.w_C * 0.5f * log2e;
      S qv[8], kv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int f = f0 + e;
        float qo = 0.f, ko = 0.f;
        if (sValid[j]) {
          const size_t rowhc = (((size_t)b * L + i) * H + h);
          if (f < kCSlot) {
            if (f < C) {
              qo = alpha * Elt<T>::load(a.q, rowhc * C + f);
              ko = Elt<T>::load(a.k, rowhc * C + f);
            }
          } else {
            const int u = f - kCSlot, grp = u / G3, w = u - grp * G3;
            if constexpr (sizeof(T) == 2) {
              if (grp < 3) {
                const int p = w / 3, x = w - 3 * p;
                const size_t pb = (rowhc * Pqk + p) * 3;
                float hi, lo;
                Elt<T>::split(kap2 * gpt(j, a.q_pts, pb, x), hi, lo);
                qo = (grp == 2) ? lo : hi;
                Elt<T>::split(gpt(j, a.k_pts, pb, x), hi, lo);
                ko = (grp == 1) ? lo : hi;
              }
            } else {
              // fp32: centred key points at 16.., centred query points
              // (unscaled) at 32..; the attention kernel takes the squared
              // distance from their explicit differences, so they must not
              // meet in the product (each side is zero where the other is set)
              if (u < G3) {
                ko = gpt(j, a.k_pts, (rowhc * Pqk + u / 3) * 3, u % 3);
              } else if (f >= kFpQPts && f - kFpQPts < G3) {
                const int v = f - kFpQPts;
                qo = gpt(j, a.q_pts, (rowhc * Pqk + v / 3) * 3, v % 3);
              }
            }
          }
        }
        qv[e] = Elt<T>::pack(qo);
        kv[e] = Elt<T>::pack(ko);
      }
      const size_t row = (((size_t)b * H + h) * Lp + i) * kHeadW + f0;
#pragma unroll
      for (int e = 0; e < 8; ++e) { qh[row + e] = qv[e]; kh[row + e] = kv[e]; }
    }
  }

  // --- value head tile, feature-major: H x 64 features x 8 chunks of 8 keys ---
  {
    S* vth = reinterpret_cast<S*>(a.ws + ly.off_vth);
    for (int ch = tid; ch < H * kHeadW * 8; ch += 256) {
      const int h = ch / (kHeadW * 8), f = (ch >> 3) & 63, p0 = (ch & 7) * 8;
      S vv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = key_of_pos<T>(p0 + e);
        const int i = J * kTileN + j;
        float o = 0.f;
        if (sValid[j]) {
          const size_t rowhc = (((size_t)b * L + i) * H + h);
          if (f < kCSlot) {
            if (f < C) o = Elt<T>::load(a.v, rowhc * C + f);
          } else {
            const int u = f - kCSlot;           // 0..47
            const int half = u / (3 * kPvSlot);  // 0 = hi, 1 = lo
            const int w = u - half * 3 * kPvSlot;
            const int x = w / kPvSlot, p = w - x * kPvSlot;
            if (p < Pv) {
              float hi, lo;
              Elt<T>::split(gpt(j, a.v_pts, (rowhc * Pv + p) * 3, x), hi, lo);
              o = half ? lo : hi;
            }
          }
        }
        vv[e] = Elt<T>::pack(o);
      }
      const size_t base = ((((size_t)b * H + h) * ly.nJ + J) * kHeadW + f) * kTileN + p0;
#pragma unroll
      for (int e = 0; e < 8; ++e) vth[base + e] = vv[e];
    }
  }

  // --- key pair panels [PW/64][64 keys][64] and value pair tile [PW][64 keys]
  //     (head-independent) ---
  {
    S* kz = reinterpret_cast<S*>(a.ws + ly.off_kz);
    S* vtz = reinterpret_cast<S*>(a.ws + ly.off_vtz);
    const int nch = kTileN * (PW / 8);
    for (int ch = tid; ch < nch; ch += 256) {
      const int P = ch / (kTileN * 8), j = (ch >> 3) & 63, u0 = P * 64 + (ch & 7) * 8;
      const int i = J * kTileN + j;
      S zv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int u = u0 + e;
        float o = 0.f;
        if (sValid[j] && u < RCz) o = Elt<T>::load(a.z2, ((size_t)b * L + i) * RCz + u);
        zv[e] = Elt<T>::pack_pair(o);
      }
      const size_t base = ((((size_t)b * ly.nJ + J) * (PW / 64) + P) * kTileN + j) * 64 + (ch & 7) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) kz[base + e] = zv[e];
    }
    for (int ch = tid; ch < PW * 8; ch += 256) {
      const int u = ch >> 3, p0 = (ch & 7) * 8;
      S zv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = key_of_pos<T>(p0 + e);
        const int i = J * kTileN + j;
        float o = 0.f;
        if (sValid[j] && u < RCz) o = Elt<T>::load(a.z2, ((size_t)b * L + i) * RCz + u);
        zv[e] = Elt<T>::pack(o);
      }
      const size_t base = (((size_t)b * ly.nJ + J) * PW + u) * kTileN + p0;
#pragma unroll
      for (int e = 0; e < 8; ++e) vtz[base + e] = zv[e];
    }
  }

  // --- per-(residue, head) float32 terms ---
  {
    float4* kcol = reinterpret_cast<float4*>(a.ws + ly.off_kcol);
    float4* qrow = reinterpret_cast<float4*>(a.ws + ly.off_qrow);
    for (int it = tid; it < H * kTileN; it += 256) {
      const int h = it / kTileN, j = it % kTileN;
      const int i = J * kTileN + j;
      const size_t o = ((size_t)b * H + h) * Lp + i;
      if (!sValid[j]) {
        kcol[o] = make_float4(0.f, 0.f, 0.f, -INFINITY);
        qrow[o] = make_float4(0.f, 0.f, 0.f, 0.f);
        continue;
      }
      const float kap = a.w_L * a.gamma[h] * a.w_C * 0.5f * log2e;
      const size_t rowhc = (((size_t)b * L + i) * H + h);
      float ax = 0.f, ay = 0.f, az = 0.f, bx = 0.f, by = 0.f, bz = 0.f, bn = 0.f;
      for (int p = 0; p < Pqk; ++p) {
        const size_t pb = (rowhc * Pqk + p) * 3;
        const float A0 = gpt(j, a.q_pts, pb, 0), A1 = gpt(j, a.q_pts, pb, 1), A2 = gpt(j, a.q_pts, pb, 2);
        const float B0 = gpt(j, a.k_pts, pb, 0), B1 = gpt(j, a.k_pts, pb, 1), B2 = gpt(j, a.k_pts, pb, 2);
        ax += A0; ay += A1; az += A2;
        bx += B0; by += B1; bz += B2;
        bn += B0 * B0 + B1 * B1 + B2 * B2;
      }
      // fp32 takes the whole point term from explicit differences
      kcol[o] = sizeof(T) == 2 ? make_float4(bx, by, bz, -kap * bn) : make_float4(0.f, 0.f, 0.f, 0.f);
      qrow[o] = make_float4(ax, ay, az, 0.f);
    }
  }

  // --- transposed, pre-scaled pair-bias weights (one block writes them) ---
  if (J == 0 && b == 0) {
    float* wbt = reinterpret_cast<float*>(a.ws + ly.off_wbt);
    const float s = a.w_L * log2e;
    for (int e = tid; e < H * ly.Cz; e += 256) {
      const int h = e / ly.Cz, c = e % ly.Cz;
      wbt[e] = s * a.w_b[(size_t)c * H + h];
    }
  }
}

}  // namespace

hipError_t launch_lift(const FwdArgs& a, bool bf16, hipStream_t s) {
  dim3 grid(a.lay.nJ, a.lay.B);
  if (bf16)
    hipLaunchKernelGGL(ipa_lift_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(ipa_lift_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ipa
