// ipa_attn: one fused online-softmax attention over the lifted IPA rows,
// with the output epilogue (T_i^-1, point norms, pair re-expansion) fused
// into its tail. No L x L tensor ever leaves the registers ("Flash Invariant
// Point Attention", abstract: linear memory through a flash-style kernel).
//
// Work split. One workgroup = 4 waves = 128 query rows of one (batch, head);
// each wave owns 32 query rows for the whole key loop (one wave per SIMD,
// all 512 registers per lane available). Keys are visited in tiles of 32.
// The key tile (row-major [key][feature]) and the value tile (feature-major
// [feature][key]) of the next tile are copied global -> LDS by direct-to-LDS
// buffer loads while the current tile computes; the two buffers of each are
// separate LDS arrays and the loop is unrolled by two, so the compiler can
// see that reads of the current buffers never wait for loads into the next
// ones. One workgroup barrier per tile.
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

namespace ipa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

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

template <typename T> __device__ __forceinline__ float ld_in(const void* p, size_t i);
template <> __device__ __forceinline__ float ld_in<uint16_t>(const void* p, size_t i) {
  return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <> __device__ __forceinline__ float ld_in<float>(const void* p, size_t i) {
  return static_cast<const float*>(p)[i];
}

// Buffer resource over `bytes` bytes at `base` (raw buffer, 32-bit data
// format); loads outside the range return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Wait until every vector-memory load of this wave (the direct-to-LDS tile
// loads) has completed; a builtin, so the compiler's own bookkeeping knows.
__device__ __forceinline__ void wait_vmem() {
  // vmcnt(0), expcnt and lgkmcnt unconstrained (gfx9 encoding)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// LDS layout. The key tile is kNP panels of [32 keys][64 features], the
// value tile [D features][32 keys]; rows are unpadded runs of 16-byte chunks
// and chunk c of row r sits in slot c ^ sw(r) (Swz below). Without padding
// one wave-wide direct-to-LDS load fills whole rows, and the swizzle spreads
// the 16 rows that 16 consecutive lanes read in one LDS cycle over distinct
// banks.
template <typename T, int D>
struct Smem {
  static constexpr int kPW = D - kHeadW;
  static constexpr int kNP = D / 64;                               // 64-feature panels
  static constexpr int kKPanel = kKT * 64 * (int)sizeof(T);         // bytes per key panel
  static constexpr int kKBuf = kNP * kKPanel;                       // bytes per key buffer
  static constexpr int kVPanel = 64 * kKT * (int)sizeof(T);         // bytes per 64 value rows
  static constexpr int kVBuf = kNP * kVPanel;                       // bytes per value buffer
  static constexpr int kCzMax = kPW < 128 ? kPW : 128;
  static constexpr int kPRow = kCzMax + 1;                          // floats per pair-buffer row
};

// XOR swizzle of rows made of RCH 16-byte chunks (RCH a power of two, <= 16).
// The LDS bank pattern repeats every 256 bytes, i.e. every kRPB = 16 / RCH
// rows; sw(r) = (r / kRPB) % RCH gives the rows that share bank positions
// distinct slots.
template <int RCH>
struct Swz {
  static_assert(RCH >= 1 && RCH <= 16 && (RCH & (RCH - 1)) == 0, "chunks per row");
  static constexpr int kRPB = 16 / RCH;   // rows per 256-byte bank period
  static constexpr int kRPL = 64 / RCH;   // rows per wave-wide 16-byte-per-lane load
  __device__ static __forceinline__ int sw(int r) { return (r / kRPB) % RCH; }
  // byte offset of element e (of `es` bytes) of row r
  __device__ static __forceinline__ int at(int r, int e, int es) {
    const int epc = 16 / es;
    return r * RCH * 16 + (((e / epc) ^ sw(r)) * 16) + (e % epc) * es;
  }
  // Per-lane source byte offset for the wave-wide load number k of a block
  // of rows (source rows srcRow bytes apart). Load k covers rows
  // k kRPL .. k kRPL + kRPL - 1 and lane l lands in LDS slot l % RCH of row
  // l / RCH, so it fetches source chunk (l % RCH) ^ sw(row). Since
  // kRPL = 4 kRPB and RCH <= 16, sw(row) depends on k only through k % 4:
  // a wave that issues loads k = w, w + 4, ... keeps one offset for all.
  __device__ static __forceinline__ uint32_t voff(int lane, int k, int srcRow) {
    const int r = k * kRPL + lane / RCH;
    return (uint32_t)((lane / RCH) * srcRow + (((lane % RCH) ^ sw(r)) * 16));
  }
};

// One wave-wide direct-to-LDS load: 16 bytes per lane from
// rsrc + soff + voff into LDS bytes lds + 16 lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff,
                                      unsigned char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, soff, 0, 0);
}

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
  constexpr int ES = (int)sizeof(T);

  // key rows: 64 elements of one panel; value rows: 32 keys
  using KS = Swz<64 * ES / 16>;
  using VS = Swz<kKT * ES / 16>;
  constexpr int KJ = kKT / KS::kRPL / 4;   // key loads per panel per wave
  constexpr int VJ = 64 / VS::kRPL / 4;    // value loads per 64 rows per wave
  static_assert(KJ >= 1 && KJ * 4 * KS::kRPL == kKT, "key tile rows per load");
  static_assert(VJ >= 1 && VJ * 4 * VS::kRPL == 64, "value tile rows per load");

  __shared__ __attribute__((aligned(16))) unsigned char K0[SM::kKBuf];
  __shared__ __attribute__((aligned(16))) unsigned char K1[SM::kKBuf];
  __shared__ __attribute__((aligned(16))) unsigned char V0[SM::kVBuf];
  __shared__ __attribute__((aligned(16))) unsigned char V1[SM::kVBuf];
  __shared__ __attribute__((aligned(16))) float4 kc0[kKT];
  __shared__ __attribute__((aligned(16))) float4 kc1[kKT];
  __shared__ float colbuf[4][kKT];
  // per 64-key block: centre xyz and valid-key count, staged once so the key
  // loop reads nothing else from global memory
  __shared__ float4 cenS[kMaxTiles];
  // pair-output accumulation of the epilogue (two waves at a time)
  __shared__ float pbuf[2][32][SM::kPRow];

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

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int n = lane & 31, g = lane >> 5;
  const int qw = qb * kTileM + 32 * w;  // first query row of this wave
  const int i = qw + n;                 // this lane's query row

  const size_t bh = (size_t)b * H + h;
  const unsigned char* Kh = a.ws + ly.off_kh + bh * Lp * kHeadW * ES;
  const unsigned char* Kz = a.ws + ly.off_kz + (size_t)b * nJ * (NP - 1) * 4096 * ES;
  const unsigned char* Vth = a.ws + ly.off_vth + bh * nJ * 4096 * ES;
  const unsigned char* Vtz = a.ws + ly.off_vtz + (size_t)b * nJ * (NP - 1) * 4096 * ES;
  const unsigned char* kcol = a.ws + ly.off_kcol + bh * Lp * 16;
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

  // ---- direct-to-LDS copy of one tile (keys 32 t .. 32 t + 31) ----
  // Wave w issues loads w, w + 4, ... of every panel, so its per-lane source
  // offsets are fixed; all tile-dependent parts are wave-uniform (scalar).
  const __amdgpu_buffer_rsrc_t rKh = make_rsrc(Kh, (uint32_t)Lp * 64 * ES);
  const __amdgpu_buffer_rsrc_t rKz = make_rsrc(Kz, (uint32_t)nJ * (NP - 1) * 4096 * ES);
  const __amdgpu_buffer_rsrc_t rVh = make_rsrc(Vth, (uint32_t)nJ * 4096 * ES);
  const __amdgpu_buffer_rsrc_t rVz = make_rsrc(Vtz, (uint32_t)nJ * (NP - 1) * 4096 * ES);
  const __amdgpu_buffer_rsrc_t rKc = make_rsrc(kcol, (uint32_t)Lp * 16);
  const uint32_t voK = KS::voff(lane, w, 64 * ES);
  const uint32_t voV = VS::voff(lane, w, 64 * ES);
  auto copy_tile = [&](int t, unsigned char* Kd, unsigned char* Vd, float4* kcd) {
    const int J = t >> 1, half = t & 1;
#pragma unroll
    for (int P = 0; P < NP; ++P) {
      // key rows 32 half .. of 64-key block J, panel P (source rows of 64 elements)
      const uint32_t kbase = P == 0 ? (uint32_t)(J * 64 + 32 * half) * 64 * ES
                                    : (uint32_t)((J * (NP - 1) + P - 1) * 64 + 32 * half) * 64 * ES;
#pragma unroll
      for (int j = 0; j < KJ; ++j) {
        const int k = w + 4 * j;
        dma16(P == 0 ? rKh : rKz, voK, kbase + (uint32_t)(k * KS::kRPL * 64 * ES),
              Kd + P * SM::kKPanel + k * 1024);
      }
      // value rows 64 P .. 64 P + 63 (features), keys 32 half .. of block J
      const uint32_t vbase = (P == 0 ? (uint32_t)J * 4096 * ES : (uint32_t)(J * (NP - 1) + P - 1) * 4096 * ES) +
                             (uint32_t)(32 * half * ES);
#pragma unroll
      for (int j = 0; j < VJ; ++j) {
        const int k = w + 4 * j;
        dma16(P == 0 ? rVh : rVz, voV, vbase + (uint32_t)(k * VS::kRPL * 64 * ES),
              Vd + P * SM::kVPanel + k * 1024);
      }
    }
    if (w == 0 && lane < kKT)
      dma16(rKc, (uint32_t)lane * 16, (uint32_t)t * kKT * 16, reinterpret_cast<unsigned char*>(kcd));
  };

  // key tiles are visited starting at this block's own diagonal tile; tiles
  // whose 64-key block has no valid key are skipped (they could only add zeros)
  const int T0 = (qb * kTileM / kKT) % nT;
  auto tile_of = [&](int uu) { int t = T0 + uu; return t >= nT ? t - nT : t; };
  // (the valid-key count is read from LDS; readfirstlane tells the compiler
  // that it, and hence every tile index and copy address, is wave-uniform)
  auto next_nonempty = [&](int uu) {
    while (uu < nT && __builtin_amdgcn_readfirstlane(__float_as_int(cenS[tile_of(uu) >> 1].w)) == 0) ++uu;
    return uu;
  };

  f32x16 oacc[NFB];
#pragma unroll
  for (int fb = 0; fb < NFB; ++fb) oacc[fb] = f32x16{};
  float m_run = -INFINITY, l_own = 0.f;
  float ocx = 0.f, ocy = 0.f, ocz = 0.f;

  // ---- one tile of the key loop on the buffers Kc / Vc / kcc ----
  auto compute_tile = [&](int t, const unsigned char* Kc, const unsigned char* Vc, const float4* kcc) {
    // ---------------- phase A: scores and probabilities ----------------
    const float4 cJ = cenS[t >> 1];
    const float dx = cI.x - cJ.x, dy = cI.y - cJ.y, dz = cI.z - cJ.z;
    if (lane < kKT) {
      const float4 kc = kcc[lane];
      colbuf[w][lane] = kc.w + 2.f * kap * (dx * kc.x + dy * kc.y + dz * kc.z);
    }
    const float rterm = sizeof(T) == 4 ? 0.f
                        : -kap * (2.f * (dx * qr.x + dy * qr.y + dz * qr.z) +
                                  (float)Pqk * (dx * dx + dy * dy + dz * dz));
    f32x16 sacc = f32x16{};
    {
      // operand reads run kLook products ahead of the matrix core
      auto kfrag = [&](int s) -> Frag {
        const int f = M::kStep * s;
        const unsigned char* r = Kc + (f / 64) * SM::kKPanel;
        if constexpr (sizeof(T) == 2)
          return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(r + KS::at(n, f % 64 + 8 * g, 2)));
        else
          return *reinterpret_cast<const float*>(r + KS::at(n, f % 64 + g, 4));
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
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 15; ++e) {
          if (e < 3 * Pqk) {
            const float tt = ad[e] - *reinterpret_cast<const float*>(Kc + KS::at(j, kCSlot + e, 4));
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
          // a few registers at a time keeps the temporaries short-lived
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

    // ---------------- phase B: O^T += V^T P^T ----------------
    {
      auto vfrag = [&](int idx) -> Frag {
        const int fb = idx / NST, s2 = idx % NST;
        const unsigned char* r = Vc + 32 * fb * kKT * ES;
        if constexpr (sizeof(T) == 2)
          return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(r + VS::at(n, 16 * s2 + 8 * g, 2)));
        else
          return *reinterpret_cast<const float*>(r + VS::at(n, 2 * s2 + g, 4));
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
  };

  // ---- key loop, unrolled by two over the buffer pairs (0 -> 1 -> 0 ...);
  //      the second half is a branch of the body, not a second loop exit, so
  //      the accumulators keep their registers across iterations ----
  int u = next_nonempty(0);
  if (u < nT) copy_tile(tile_of(u), K0, V0, kc0);
  wait_vmem();
  __syncthreads();
  while (u < nT) {
    int un = next_nonempty(u + 1);
    if (un < nT) copy_tile(tile_of(un), K1, V1, kc1);
    compute_tile(tile_of(u), K0, V0, kc0);
    wait_vmem();
    __syncthreads();
    u = un;
    if (u < nT) {
      un = next_nonempty(u + 1);
      if (un < nT) copy_tile(tile_of(un), K0, V0, kc0);
      compute_tile(tile_of(u), K1, V1, kc1);
      wait_vmem();
      __syncthreads();
      u = un;
    }
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

  // pair channels: sum_r z1_ir * O_pair,r accumulated in LDS (rows padded by
  // one float, so the 32 rows of a wave fall in distinct banks), two waves
  // at a time, then written out row by row
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if ((w >> 1) == pass) {
      float* pb = &pbuf[w & 1][0][0];
      for (int e = lane; e < 32 * SM::kPRow; e += 64) pb[e] = 0.f;
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
                pb[n * SM::kPRow + c] += z * oacc[fb][4 * k + e] * inv;
              }
            }
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      for (int e = lane; e < 32 * Cz; e += 64) {
        const int nn = e / Cz, c = e - nn * Cz;
        const int ii = qw + nn;
        if (ii < L) a.out_pair[(((size_t)b * L + ii) * H + h) * Cz + c] = pb[nn * SM::kPRow + c];
      }
    }
    __syncthreads();
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
