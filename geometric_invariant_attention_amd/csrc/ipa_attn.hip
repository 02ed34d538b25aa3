// ipa_attn: one fused online-softmax attention over the lifted IPA rows,
// with the output epilogue (T_i^-1, point norms, pair re-expansion) fused
// into its tail. No L x L tensor ever leaves the registers ("Flash Invariant
// Point Attention", abstract: linear memory through a flash-style kernel).
//
// Work split. One workgroup = 4 waves = 128 query rows of one (batch, head);
// each wave owns 32 query rows for the whole key loop (one wave per SIMD,
// all 512 registers per lane available). Keys are visited in tiles of 32:
// the key tile row-major [key][feature] and the value tile feature-major
// [feature][key] are double-buffered in LDS, staged through registers (the
// next tile's global loads are in flight while the current tile computes),
// with one workgroup barrier per tile.
//
// Products are taken transposed, S^T = K Q^T and O^T = V^T P^T, on 32x32
// matrix-core tiles: lane l then holds query l % 32 for both products, the
// probabilities of the first product feed the second straight from
// registers (the value tile is stored in the matching key order), and a
// query's row max / row sum needs only the partner lane l ^ 32.
//
// Logit of query i, key j (base-2 units, see ipa_lift):
//   s_ij = Q_i . K_j + col_j + row_i(J)    (+ a per-row constant that cancels)
//   col_j = -k |B'_j|^2 + 2 k delta . sum B'_j       (float32, per key)
//   row_i = -k (2 delta . sum A'_i + Pqk |delta|^2)  (float32, per query)
//   delta = c_I - c_J (query and key block centres).
// The running max is only moved when a tile's max exceeds it by more than
// kLazy (base-2) units; probabilities can then reach 2^kLazy, which bf16 and
// float32 hold exactly, and the final division by the row sum is unchanged.
// Probabilities are rounded to bf16 once and the same rounded values feed
// the value product, the row sum and the block-centre correction, so the
// output is a convex combination of the value rows.

#include "ipa_internal.h"

#include <type_traits>

namespace ipa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLazy = 8.0f;
// Keys per tile of the key loop (the centring blocks stay 64 residues).
constexpr int kKT = 32;
// Operand fragments read ahead of the matrix-core products that use them.
constexpr int kLook = 4;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Round to nearest even fp16, saturating at the largest finite value.
__device__ __forceinline__ uint16_t f32_to_f16_sat(float f) {
  f = fminf(fmaxf(f, -65504.f), 65504.f);
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Element-type policy: bf16 storage with 32x32x16 bf16 products, or fp32
// storage with 32x32x2 fp32 products.
template <typename T> struct Mma;
template <> struct Mma<uint16_t> {
  static constexpr int kStep = 16;   // reduction length of one product
  static constexpr int kPad = 8;     // LDS row padding (elements)
  static constexpr int kEpc = 8;     // elements per 16-byte chunk
  using Frag = bf16x8;               // per-lane operand of one product
};
template <> struct Mma<float> {
  static constexpr int kStep = 2;
  static constexpr int kPad = 4;
  static constexpr int kEpc = 4;
  using Frag = float;
};

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
// pair part of S^T on the bf16 path: fp16 operands (bits carried in bf16x8)
__device__ __forceinline__ f32x16 mma_pair(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                               __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma_pair(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// N registers of 16 bytes addressed by compile-time index only (no array, so
// they always stay in registers).
template <int N> struct Regs : Regs<N - 1> { u32x4 v; };
template <> struct Regs<0> {};
template <int M, int N>
__device__ __forceinline__ u32x4& reg(Regs<N>& r) { return static_cast<Regs<M + 1>&>(r).v; }

template <typename T> __device__ __forceinline__ float ld_in(const void* p, size_t i);
template <> __device__ __forceinline__ float ld_in<uint16_t>(const void* p, size_t i) {
  return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <> __device__ __forceinline__ float ld_in<float>(const void* p, size_t i) {
  return static_cast<const float*>(p)[i];
}

// LDS layout. The key tile is kNP panels of [32 keys][64 features], the
// value tile [D features][32 keys]; every row is padded by one 16-byte chunk,
// which spreads the 32 rows that one matrix-core operand read touches over
// distinct LDS banks. Two buffers of each.
template <typename T, int D>
struct Smem {
  static constexpr int kPW = D - kHeadW;
  static constexpr int kEpc = Mma<T>::kEpc;
  static constexpr int kNP = D / 64;                               // 64-feature panels
  static constexpr int kKRow = 64 + Mma<T>::kPad;                  // elements per key-panel row
  static constexpr int kKPanel = kKT * kKRow;                      // elements per key panel
  static constexpr int kKBuf = kNP * kKPanel;                      // elements per key buffer
  static constexpr int kVRow = kKT + Mma<T>::kPad;                 // elements per value row
  static constexpr int kVBuf = D * kVRow;                          // elements per value buffer
  static constexpr int kCzMax = kPW < 128 ? kPW : 128;
  static constexpr int kPairBytes = 4 * 32 * (kCzMax > 0 ? kCzMax : 1) * 4;
  // the key buffers also hold the pair-output buffer of the epilogue
  static constexpr int kKBytes = 2 * kKBuf * (int)sizeof(T) > kPairBytes
                                     ? 2 * kKBuf * (int)sizeof(T) : kPairBytes;
  static constexpr int kVBytes = 2 * kVBuf * (int)sizeof(T);
  // 16-byte chunks each thread stages per tile (key part or value part)
  static constexpr int kCPT = kNP * (64 / kEpc) * kKT / 256;
};

template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ipa_attn_kernel(FwdArgs a) {
  using M = Mma<T>;
  using Frag = typename M::Frag;
  using SM = Smem<T, D>;
  constexpr int NKS = D / M::kStep;        // products per S^T tile
  constexpr int NKH = kHeadW / M::kStep;   // of which cover the head part
  constexpr int NFB = D / 32;              // 32-feature blocks of O^T
  constexpr int NP = SM::kNP;
  constexpr int EPC = M::kEpc;
  constexpr int NST = kKT / M::kStep;      // products per O^T block per tile
  constexpr int CPT = SM::kCPT;
  static_assert(CPT * 256 == NP * (64 / EPC) * kKT, "tile chunks must split over 256 threads");

  __shared__ __attribute__((aligned(16))) unsigned char smemK[SM::kKBytes];
  __shared__ __attribute__((aligned(16))) unsigned char smemV[SM::kVBytes];
  __shared__ float4 kcS[2][kKT];
  __shared__ float colbuf[4][kKT];
  // per 64-key block: centre xyz and valid-key count, staged once so the key
  // loop issues no vector-memory reads besides its tile loads
  __shared__ float4 cenS[kMaxTiles];

  T* const Kb = reinterpret_cast<T*>(smemK);
  T* const Vb = reinterpret_cast<T*>(smemV);

  const Layout& ly = a.lay;
  const int L = ly.L, H = ly.H, Lp = ly.Lp, nJ = ly.nJ;
  const int C = ly.C, Pqk = ly.Pqk, Pv = ly.Pv, Cz = ly.Cz, RCz = ly.R * ly.Cz;
  const int nQB = Lp / kTileM;
  const int nT = Lp / kKT;

  // XCD-aware order: consecutive workgroup ids are dealt to the 8 XCDs in
  // turn, so remap them so that the query blocks of one (batch, head), which
  // read the same key/value tiles, run on the same XCD and share its L2.
  const int nwg = gridDim.x, id = blockIdx.x;
  const int xcd = id & 7, loc = id >> 3, per = nwg >> 3, rem = nwg & 7;
  const int nid = (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
  const int qb = nid % nQB, h = (nid / nQB) % H, b = nid / (nQB * H);

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int n = lane & 31, g = lane >> 5;
  const int qw = qb * kTileM + 32 * w;  // first query row of this wave
  const int i = qw + n;                 // this lane's query row

  const size_t bh = (size_t)b * H + h;
  const T* Kh = reinterpret_cast<const T*>(a.ws + ly.off_kh) + bh * Lp * kHeadW;
  const T* Kz = reinterpret_cast<const T*>(a.ws + ly.off_kz) + (size_t)b * nJ * (NP - 1) * 4096;
  const T* Vth = reinterpret_cast<const T*>(a.ws + ly.off_vth) + bh * nJ * 4096;
  const T* Vtz = reinterpret_cast<const T*>(a.ws + ly.off_vtz) + (size_t)b * nJ * (NP - 1) * 4096;
  const float4* kcol = reinterpret_cast<const float4*>(a.ws + ly.off_kcol) + bh * Lp;
  {
    const float4* cen = reinterpret_cast<const float4*>(a.ws + ly.off_cen) + (size_t)b * nJ;
    for (int e = tid; e < nJ; e += 256) cenS[e] = cen[e];
  }

  const float kap = a.w_L * a.gamma[h] * a.w_C * 0.5f * kLog2e;
  const bool row_valid = (i < L) && (a.mask == nullptr || a.mask[(size_t)b * L + i] != 0);

  // ---- query operand (B operand of S^T = K Q^T), held for the whole loop ----
  Frag qf[NKS];
  {
    const T* Qh = reinterpret_cast<const T*>(a.ws + ly.off_qh) + (bh * Lp + i) * kHeadW;
    const float* wbt = reinterpret_cast<const float*>(a.ws + ly.off_wbt) + (size_t)h * Cz;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const int f0 = 16 * s + 8 * g;
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (f0 < kHeadW) {
          raw = *reinterpret_cast<const uint4*>(Qh + f0);
        } else {
          const int u0 = f0 - kHeadW;
          if (u0 < RCz && i < L) {
            const int c0 = u0 % Cz;
            const uint16_t* zp = static_cast<const uint16_t*>(a.z1) + ((size_t)b * L + i) * RCz + u0;
            const uint4 zr = *reinterpret_cast<const uint4*>(zp);
            const uint32_t zw[4] = {zr.x, zr.y, zr.z, zr.w};
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float lo = __uint_as_float(zw[e] << 16) * wbt[c0 + 2 * e];
              const float hi = __uint_as_float(zw[e] & 0xFFFF0000u) * wbt[c0 + 2 * e + 1];
              o[e] = (uint32_t)f32_to_f16_sat(lo) | ((uint32_t)f32_to_f16_sat(hi) << 16);
            }
            raw = make_uint4(o[0], o[1], o[2], o[3]);
          }
        }
        qf[s] = __builtin_bit_cast(bf16x8, raw);
      }
    } else {
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const int f = 2 * s + g;
        float v = 0.f;
        if (f < kHeadW) {
          v = reinterpret_cast<const float*>(Qh)[f];
        } else {
          const int uu = f - kHeadW;
          if (uu < RCz && i < L)
            v = static_cast<const float*>(a.z1)[((size_t)b * L + i) * RCz + uu] * wbt[uu % Cz];
        }
        qf[s] = v;
      }
    }
  }
  const float4 qr = reinterpret_cast<const float4*>(a.ws + ly.off_qrow)[bh * Lp + i];
  // fp32 path: the centred query points themselves (the point term is taken
  // from explicit differences, see below)
  float apt[sizeof(T) == 4 ? 15 : 1];
  if constexpr (sizeof(T) == 4) {
    const float* Qh = reinterpret_cast<const float*>(a.ws + ly.off_qh) + (bh * Lp + i) * kHeadW;
#pragma unroll
    for (int e = 0; e < 15; ++e) apt[e] = e < 3 * Pqk ? Qh[kFpQPts + e] : 0.f;
  }
  __syncthreads();  // cenS
  const float4 cI = cenS[qw / kTileN];

  // ---- tile staging: global -> registers -> LDS ----
  // Key tile t (keys 32t .. 32t+31): chunk m of this thread lies in panel
  // ch / (32 * KCPR), key (ch / KCPR) % 32, column chunk ch % KCPR, with
  // ch = tid + 256 m. Value tile: chunk m is feature ch / VCPR, key chunk
  // ch % VCPR of the tile's half of its 64-key value block.
  constexpr int KCPR = 64 / EPC;               // chunks per key-panel row
  constexpr int VCPR = kKT / EPC;              // chunks per value row
  Regs<CPT> st;
  float4 kcst = make_float4(0.f, 0.f, 0.f, 0.f);
  auto load_k = [&](int t) {
    const int J = t >> 1, half = t & 1;
    static_for<0, CPT>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      const int ch = tid + 256 * m;
      const int P = ch / (kKT * KCPR), r = (ch / KCPR) % kKT, c = ch % KCPR;
      const int key = 32 * half + r;                      // key within the 64-block
      const T* src = P == 0 ? Kh + ((size_t)J * 64 + key) * kHeadW + c * EPC
                            : Kz + (((size_t)J * (NP - 1) + P - 1) * 64 + key) * 64 + c * EPC;
      reg<m>(st) = *reinterpret_cast<const u32x4*>(src);
    });
    if (tid < kKT) kcst = kcol[(size_t)t * kKT + tid];
  };
  auto store_k = [&](int bf) {
    static_for<0, CPT>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      const int ch = tid + 256 * m;
      const int P = ch / (kKT * KCPR), r = (ch / KCPR) % kKT, c = ch % KCPR;
      *reinterpret_cast<u32x4*>(Kb + bf * SM::kKBuf + P * SM::kKPanel + r * SM::kKRow + c * EPC) = reg<m>(st);
    });
    if (tid < kKT) kcS[bf][tid] = kcst;
  };
  auto load_v = [&](int t) {
    const int J = t >> 1, half = t & 1;
    static_for<0, CPT>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      const int ch = tid + 256 * m;
      const int f = ch / VCPR, c = ch % VCPR;
      const T* src = f < kHeadW ? Vth + ((size_t)J * 64 + f) * 64 + 32 * half + c * EPC
                                : Vtz + ((size_t)J * (NP - 1) * 64 + (f - kHeadW)) * 64 + 32 * half + c * EPC;
      reg<m>(st) = *reinterpret_cast<const u32x4*>(src);
    });
  };
  auto store_v = [&](int bf) {
    static_for<0, CPT>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      const int ch = tid + 256 * m;
      const int f = ch / VCPR, c = ch % VCPR;
      *reinterpret_cast<u32x4*>(Vb + bf * SM::kVBuf + f * SM::kVRow + c * EPC) = reg<m>(st);
    });
  };

  // key tiles are visited starting at this block's own diagonal tile; tiles
  // whose 64-key block has no valid key are skipped (they could only add zeros)
  const int T0 = (qb * kTileM / kKT) % nT;
  auto tile_of = [&](int uu) { int t = T0 + uu; return t >= nT ? t - nT : t; };
  auto next_nonempty = [&](int uu) {
    while (uu < nT && cenS[tile_of(uu) >> 1].w == 0.f) ++uu;
    return uu;
  };

  f32x16 oacc[NFB];
#pragma unroll
  for (int fb = 0; fb < NFB; ++fb) oacc[fb] = f32x16{};
  float m_run = -INFINITY, l_own = 0.f;
  float ocx = 0.f, ocy = 0.f, ocz = 0.f;

  int u = next_nonempty(0);
  int buf = 0;
  if (u < nT) {
    load_k(tile_of(u));
    store_k(0);
    load_v(tile_of(u));
    store_v(0);
  }
  __syncthreads();

  while (u < nT) {
    const int t = tile_of(u);
    const int un = next_nonempty(u + 1);
    const bool more = un < nT;
    const int tn = more ? tile_of(un) : 0;
    if (more) load_k(tn);

    // ---------------- phase A: scores and probabilities ----------------
    const float4 cJ = cenS[t >> 1];
    const float dx = cI.x - cJ.x, dy = cI.y - cJ.y, dz = cI.z - cJ.z;
    if (lane < kKT) {
      const float4 kc = kcS[buf][lane];
      colbuf[w][lane] = kc.w + 2.f * kap * (dx * kc.x + dy * kc.y + dz * kc.z);
    }
    const float rterm = sizeof(T) == 4 ? 0.f
                        : -kap * (2.f * (dx * qr.x + dy * qr.y + dz * qr.z) +
                                  (float)Pqk * (dx * dx + dy * dy + dz * dz));
    f32x16 sacc = f32x16{};
    {
      // operand reads run kLook products ahead of the matrix core
      const T* krow = Kb + buf * SM::kKBuf + n * SM::kKRow;
      auto kfrag = [&](int s) -> Frag {
        const int f = M::kStep * s;
        const T* r = krow + (f / 64) * SM::kKPanel + (f % 64);
        if constexpr (sizeof(T) == 2)
          return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(r + 8 * g));
        else
          return r[g];
      };
      Frag look[kLook];
#pragma unroll
      for (int x = 0; x < kLook; ++x) look[x] = kfrag(x);
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const Frag cur = look[s % kLook];
        if (s + kLook < NKS) look[s % kLook] = kfrag(s + kLook);
        if (s < NKH)
          sacc = mma(cur, qf[s], sacc);
        else
          sacc = mma_pair(cur, qf[s], sacc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (sizeof(T) == 4) {
      // fp32: -k * sum_p |A'_ip + delta - B'_jp|^2 from explicit differences;
      // the expanded form would lose ~1e-5 logits to float32 cancellation
      float ad[15];
#pragma unroll
      for (int e = 0; e < 15; ++e) ad[e] = apt[e] + (e % 3 == 0 ? dx : e % 3 == 1 ? dy : dz);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = 8 * (v >> 2) + 4 * g + (v & 3);
        const float* bp = reinterpret_cast<const float*>(Kb) + buf * SM::kKBuf + j * SM::kKRow + kCSlot;
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 15; ++e) {
          if (e < 3 * Pqk) {
            const float tt = ad[e] - bp[e];
            d = fmaf(tt, tt, d);
          }
        }
        sacc[v] = fmaf(-kap, d, sacc[v]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 cv = *reinterpret_cast<const float4*>(&colbuf[w][8 * k + 4 * g]);
      sacc[4 * k + 0] += cv.x;
      sacc[4 * k + 1] += cv.y;
      sacc[4 * k + 2] += cv.z;
      sacc[4 * k + 3] += cv.w;
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sacc[4 * k + e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float Mt = mx + rterm;
    const bool need = Mt > m_run + kLazy;
    if (__any(need)) {
      const float mn = need ? Mt : m_run;
      const float al = (mn == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - mn);
      m_run = mn;
      l_own *= al; ocx *= al; ocy *= al; ocz *= al;
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
        for (int v = 0; v < 16; v += 4) {
          // a few registers at a time keeps the accumulator copies short-lived
          oacc[fb][v] *= al; oacc[fb][v + 1] *= al; oacc[fb][v + 2] *= al; oacc[fb][v + 3] *= al;
          __builtin_amdgcn_sched_barrier(0);
        }
    }
    const float shift = (m_run == -INFINITY) ? 0.f : m_run - rterm;

    // probabilities -> B operand of O^T = V^T P^T
    Frag pf[NST];
    float lt = 0.f;
    if constexpr (sizeof(T) == 2) {
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int s2 = 0; s2 < NST; ++s2) {
        bf16x2 pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f32x2 pv = {__builtin_amdgcn_exp2f(sacc[8 * s2 + 2 * e] - shift),
                      __builtin_amdgcn_exp2f(sacc[8 * s2 + 2 * e + 1] - shift)};
          pk[e] = __builtin_convertvector(pv, bf16x2);
          lt = __builtin_amdgcn_fdot2_f32_bf16(pk[e], ones, lt, false);
        }
        pf[s2] = bf16x8{pk[0][0], pk[0][1], pk[1][0], pk[1][1],
                        pk[2][0], pk[2][1], pk[3][0], pk[3][1]};
      }
    } else {
#pragma unroll
      for (int s2 = 0; s2 < NST; ++s2) {
        const float p = __builtin_amdgcn_exp2f(sacc[s2] - shift);
        pf[s2] = p;
        lt += p;
      }
    }
    l_own += lt;
    ocx += lt * cJ.x; ocy += lt * cJ.y; ocz += lt * cJ.z;

    if (more) {
      store_k(buf ^ 1);
      load_v(tn);
    }

    // ---------------- phase B: O^T += V^T P^T ----------------
    {
      const T* vrow = Vb + buf * SM::kVBuf + n * SM::kVRow;
      auto vfrag = [&](int idx) -> Frag {
        const int fb = idx / NST, s2 = idx % NST;
        const T* r = vrow + 32 * fb * SM::kVRow;
        if constexpr (sizeof(T) == 2)
          return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(r + 16 * s2 + 8 * g));
        else
          return r[2 * s2 + g];
      };
      constexpr int NB = NFB * NST;
      Frag look[kLook];
#pragma unroll
      for (int x = 0; x < kLook; ++x) look[x] = vfrag(x);
#pragma unroll
      for (int idx = 0; idx < NB; ++idx) {
        const Frag cur = look[idx % kLook];
        if (idx + kLook < NB) look[idx % kLook] = vfrag(idx + kLook);
        oacc[idx / NST] = mma(cur, pf[idx % NST], oacc[idx / NST]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (more) store_v(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    u = un;
  }

  // ---------------- epilogue ----------------
  const float l_tot = l_own + __shfl_xor(l_own, 32, 64);
  const float gx_c = ocx + __shfl_xor(ocx, 32, 64);
  const float gy_c = ocy + __shfl_xor(ocy, 32, 64);
  const float gz_c = ocz + __shfl_xor(ocz, 32, 64);
  const bool ok = row_valid && l_tot > 0.f;
  const float inv = ok ? 1.f / l_tot : 0.f;
  const bool in_range = i < L;
  const size_t rowh = ((size_t)b * L + i) * H + h;

  if (in_range) {
    // scalar channels: features 8k + 4g + e (k = 0, 1) of the first block
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = 8 * k + 4 * g + e;
        if (f < C) a.out_s[rowh * C + f] = ok ? oacc[0][4 * k + e] * inv : 0.f;
      }
    // value points 4g + e: hi x/y/z in registers (0,8+e) (0,12+e) (1,e),
    // lo x/y/z in (1,4+e) (1,8+e) (1,12+e)
    float R[9], tr[3];
#pragma unroll
    for (int e = 0; e < 9; ++e) R[e] = ok ? a.rot[((size_t)b * L + i) * 9 + e] : 0.f;
#pragma unroll
    for (int e = 0; e < 3; ++e) tr[e] = ok ? a.trans[((size_t)b * L + i) * 3 + e] : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = 4 * g + e;
      if (p < Pv) {
        float lx = 0.f, lyv = 0.f, lz = 0.f, nr = 0.f;
        if (ok) {
          const float gx = (oacc[0][8 + e] + oacc[1][4 + e] + gx_c) * inv - tr[0];
          const float gy = (oacc[0][12 + e] + oacc[1][8 + e] + gy_c) * inv - tr[1];
          const float gz = (oacc[1][e] + oacc[1][12 + e] + gz_c) * inv - tr[2];
          lx = R[0] * gx + R[3] * gy + R[6] * gz;
          lyv = R[1] * gx + R[4] * gy + R[7] * gz;
          lz = R[2] * gx + R[5] * gy + R[8] * gz;
          nr = sqrtf(lx * lx + lyv * lyv + lz * lz);
        }
        float* op = a.out_pts + (rowh * Pv + p) * 3;
        op[0] = lx; op[1] = lyv; op[2] = lz;
        a.out_pts_norm[rowh * Pv + p] = nr;
      }
    }
  }

  // pair channels: accumulate sum_r z1_ir * O_pair,r in LDS, then write rows
  __syncthreads();  // every wave is done with the key/value tiles
  float* pbuf = reinterpret_cast<float*>(smemK) + (size_t)w * 32 * Cz;
  for (int e = lane; e < 32 * Cz; e += 64) pbuf[e] = 0.f;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (ok) {
#pragma unroll
    for (int fb = 2; fb < NFB; ++fb)
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int uu = 32 * (fb - 2) + 8 * k + 4 * g + e;
          if (uu < RCz) {
            const int c = uu % Cz;
            const float z = ld_in<T>(a.z1, ((size_t)b * L + i) * RCz + uu);
            pbuf[n * Cz + c] += z * oacc[fb][4 * k + e] * inv;
          }
        }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  for (int e = lane; e < 32 * Cz; e += 64) {
    const int nn = e / Cz, c = e - nn * Cz;
    const int ii = qw + nn;
    if (ii < L) a.out_pair[(((size_t)b * L + ii) * H + h) * Cz + c] = pbuf[e];
  }
}

template <typename T, int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  const int nwg = (a.lay.Lp / kTileM) * a.lay.H * a.lay.B;
  hipLaunchKernelGGL((ipa_attn_kernel<T, D>), dim3(nwg), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bf16(const FwdArgs& a, hipStream_t s) {
  switch (a.lay.D) {
    case 64: return launch_d<uint16_t, 64>(a, s);
    case 128: return launch_d<uint16_t, 128>(a, s);
    case 192: return launch_d<uint16_t, 192>(a, s);
    case 256: return launch_d<uint16_t, 256>(a, s);
    case 320: return launch_d<uint16_t, 320>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// The fp32 path keeps its whole query row in registers as 32-bit values;
// rows wider than kMaxDF32 are rejected by the host checks.
hipError_t launch_f32(const FwdArgs& a, hipStream_t s) {
  switch (a.lay.D) {
    case 64: return launch_d<float, 64>(a, s);
    case 128: return launch_d<float, 128>(a, s);
    case 192: return launch_d<float, 192>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn(const FwdArgs& a, bool bf16, hipStream_t s) {
  return bf16 ? launch_bf16(a, s) : launch_f32(a, s);
}

}  // namespace ipa
