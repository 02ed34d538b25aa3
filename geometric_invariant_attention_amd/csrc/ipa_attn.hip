// ipa_attn: one fused online-softmax attention over the lifted IPA rows,
// with the output epilogue (T_i^-1, point norms, pair re-expansion) fused
// into its tail. No L x L tensor ever leaves the registers ("Flash Invariant
// Point Attention", abstract: linear memory through a flash-style kernel).
//
// Work split. One workgroup = 4 waves = 128 query rows of one (batch, head);
// each wave owns 32 query rows for the whole key loop. Key tiles of 64 keys
// are staged in LDS: the key tile row-major [key][feature] and the value tile
// feature-major [feature][key].
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
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLazy = 8.0f;
// Operand fragments read ahead of the matrix-core products that use them.
constexpr int kLook = 4;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
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
// pair part of S^T on the bf16 path: fp16 operands (bits carried in bf16x8)
__device__ __forceinline__ f32x16 mma_pair(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                               __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma_pair(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ float ld_in(const void* p, size_t i);
template <> __device__ __forceinline__ float ld_in<uint16_t>(const void* p, size_t i) {
  return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <> __device__ __forceinline__ float ld_in<float>(const void* p, size_t i) {
  return static_cast<const float*>(p)[i];
}

// LDS tiles are made of panels: 64 rows x 64 features (key tile, row =
// key) or 64 rows x 64 keys (value tile, row = feature). Each panel row is
// padded by one 16-byte chunk, which spreads the 32 rows that one
// matrix-core operand read touches over distinct LDS banks.
template <typename T, int D>
struct Smem {
  static constexpr int kPW = D - kHeadW;
  static constexpr int kEpc = Mma<T>::kEpc;
  static constexpr int kRow = 64 + Mma<T>::kPad;                 // elements per padded panel row
  static constexpr int kPanel = 64 * kRow * (int)sizeof(T);       // bytes per panel
  static constexpr int kNP = D / 64;                              // panels per tile
  static constexpr int kK = 0;                                    // key tile panels
  static constexpr int kV = kK + kNP * kPanel;                    // value tile panels
  static constexpr int kMain = kV + kNP * kPanel;
  static constexpr int kCzMax = kPW < 128 ? kPW : 128;
  static constexpr int kPairBytes = 4 * 32 * (kCzMax > 0 ? kCzMax : 1) * 4;
  static constexpr int kBytes = kMain > kPairBytes ? kMain : kPairBytes;
};

// Buffer resource over `bytes` bytes at `base` (raw buffer, 32-bit data
// format); loads outside the range return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct-to-LDS panel loads. A panel's source is 64 contiguous rows of 64
// elements; in LDS each row takes kRC = 64/EPC + 1 chunks. One wave-wide
// load writes 64 consecutive LDS chunks (lane l -> chunk l), so a load that
// covers kRPL whole padded rows has the same per-lane source offset for
// every load: lane l copies chunk l % kRC (the padding chunk copies any
// chunk of its row) of row l / kRC, and lanes past kRPL rows stay idle.
template <typename T>
struct PanelLoad {
  static constexpr int kEpc = Mma<T>::kEpc;
  static constexpr int kDC = 64 / kEpc;                 // data chunks per row
  static constexpr int kRC = kDC + 1;                   // LDS chunks per row
  static constexpr int kRPL = 64 / kRC;                 // rows per load
  static constexpr int kLoads = (64 + kRPL - 1) / kRPL; // loads per panel
  static constexpr uint32_t kSrcBytes = 64u * kDC * 16u;
  int lane_off;   // source byte offset of this lane within its rows, -1 = idle lane
  int lane_row;   // row of this lane within a load
  __device__ void init(int lane) {
    lane_row = lane / kRC;
    const int c = lane - lane_row * kRC;
    const int cc = c < kDC ? c : kDC - 1;
    lane_off = lane_row < kRPL ? (lane_row * kDC + cc) * 16 : -1;
  }
  // Enqueue loads k = k0, k0 + kStride, ... of one panel.
  __device__ void load(const unsigned char* src, unsigned char* lds, int k0, int kStride) const {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src, kSrcBytes);
    for (int k = k0; k < kLoads; k += kStride) {
      if (lane_off >= 0 && k * kRPL + lane_row < 64)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(lds + k * kRPL * kRC * 16), 16,
            lane_off, k * kRPL * kDC * 16, 0, 0);
    }
  }
};

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ipa_attn_kernel(FwdArgs a) {
  using M = Mma<T>;
  using Frag = typename M::Frag;
  using SM = Smem<T, D>;
  constexpr int NKS = D / M::kStep;     // products per 32-key block of S^T
  constexpr int NFB = D / 32;           // 32-feature blocks of O^T
  constexpr int NKH = kHeadW / M::kStep; // products over the head part of a row
  constexpr int EPC = M::kEpc;
  constexpr int NP = SM::kNP;
  constexpr int NST = kTileN / M::kStep;  // products per 32-feature block of O^T

  __shared__ __attribute__((aligned(1024))) unsigned char smem[SM::kBytes];
  __shared__ __attribute__((aligned(1024))) float4 kcS[kTileN];
  __shared__ float colbuf[4][kTileN];

  const T* Ks = reinterpret_cast<const T*>(smem + SM::kK);
  const T* Vs = reinterpret_cast<const T*>(smem + SM::kV);

  const Layout& ly = a.lay;
  const int L = ly.L, H = ly.H, Lp = ly.Lp, nJ = ly.nJ, PW = ly.PW;
  const int C = ly.C, Pqk = ly.Pqk, Pv = ly.Pv, Cz = ly.Cz, RCz = ly.R * ly.Cz;
  const int nQB = Lp / kTileM;

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
  constexpr size_t kPanelSrc = 64 * 64 * sizeof(T);   // bytes of one source panel
  const unsigned char* Kh = a.ws + ly.off_kh + bh * Lp * kHeadW * sizeof(T);
  const unsigned char* Kz = a.ws + ly.off_kz + (size_t)b * nJ * (NP - 1) * kPanelSrc;
  const unsigned char* Vth = a.ws + ly.off_vth + bh * nJ * kPanelSrc;
  const unsigned char* Vtz = a.ws + ly.off_vtz + (size_t)b * nJ * (NP - 1) * kPanelSrc;
  const unsigned char* kcol = a.ws + ly.off_kcol + bh * Lp * 16;
  const float4* cen = reinterpret_cast<const float4*>(a.ws + ly.off_cen) + (size_t)b * nJ;

  PanelLoad<T> pl;
  pl.init(lane);

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
          const int u = f - kHeadW;
          if (u < RCz && i < L)
            v = static_cast<const float*>(a.z1)[((size_t)b * L + i) * RCz + u] * wbt[u % Cz];
        }
        qf[s] = v;
      }
    }
  }
  const float4 qr = reinterpret_cast<const float4*>(a.ws + ly.off_qrow)[bh * Lp + (i < Lp ? i : 0)];
  // fp32 path: the centred query points themselves (the point term is taken
  // from explicit differences, see below)
  float apt[sizeof(T) == 4 ? 15 : 1];
  if constexpr (sizeof(T) == 4) {
    const float* Qh = reinterpret_cast<const float*>(a.ws + ly.off_qh) + (bh * Lp + i) * kHeadW;
#pragma unroll
    for (int e = 0; e < 15; ++e) apt[e] = e < 3 * Pqk ? Qh[kFpQPts + e] : 0.f;
  }
  const float4 cI = cen[qw / kTileN];

  // ---- tile loaders: global -> LDS directly, no registers involved ----
  auto load_k = [&](int J) {
    pl.load(Kh + (size_t)J * kPanelSrc, smem + SM::kK, w, 4);
#pragma unroll
    for (int P = 1; P < NP; ++P)
      pl.load(Kz + ((size_t)J * (NP - 1) + P - 1) * kPanelSrc, smem + SM::kK + P * SM::kPanel, w, 4);
    if (w == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          make_rsrc(kcol + (size_t)J * kTileN * 16, kTileN * 16),
          (__attribute__((address_space(3))) void*)kcS, 16, lane * 16, 0, 0, 0);
  };
  auto load_v = [&](int J) {
    pl.load(Vth + (size_t)J * kPanelSrc, smem + SM::kV, w, 4);
#pragma unroll
    for (int P = 1; P < NP; ++P)
      pl.load(Vtz + ((size_t)J * (NP - 1) + P - 1) * kPanelSrc, smem + SM::kV + P * SM::kPanel, w, 4);
  };

  // key tiles are visited starting at this block's own diagonal tile; tiles
  // with no valid key are skipped (their keys could only add zeros)
  const int J0 = (qb * kTileM / kTileN) % nJ;
  auto tile_of = [&](int t) {
    int J = J0 + t;
    return __builtin_amdgcn_readfirstlane(J >= nJ ? J - nJ : J);
  };
  auto next_nonempty = [&](int t) {
    while (t < nJ && cen[tile_of(t)].w == 0.f) ++t;
    return t;
  };

  f32x16 oacc[NFB];
#pragma unroll
  for (int fb = 0; fb < NFB; ++fb) oacc[fb] = f32x16{};
  float m_run = -INFINITY, l_own = 0.f;
  float ocx = 0.f, ocy = 0.f, ocz = 0.f;

  int t = next_nonempty(0);
  if (t < nJ) load_k(tile_of(t));
  wait_vm();
  __syncthreads();

  while (t < nJ) {
    const int J = tile_of(t);
    const int tn = next_nonempty(t + 1);
    load_v(J);

    // ---------------- phase A: scores and probabilities ----------------
    const float4 cJ = cen[J];
    const float dx = cI.x - cJ.x, dy = cI.y - cJ.y, dz = cI.z - cJ.z;
    {
      const float4 kc = kcS[lane];
      colbuf[w][lane] = kc.w + 2.f * kap * (dx * kc.x + dy * kc.y + dz * kc.z);
    }
    const float rterm = sizeof(T) == 4 ? 0.f
                        : -kap * (2.f * (dx * qr.x + dy * qr.y + dz * qr.z) +
                                  (float)Pqk * (dx * dx + dy * dy + dz * dz));
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    {
      // operand reads run kLook products ahead of the matrix core
      const T* krow = Ks + n * SM::kRow;
      auto kfrag = [&](int idx) -> Frag {
        const int s = idx >> 1, kb = idx & 1;
        const int f = M::kStep * s;
        const T* r = krow + (f / 64) * (SM::kPanel / (int)sizeof(T)) + 32 * kb * SM::kRow + (f % 64);
        if constexpr (sizeof(T) == 2)
          return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(r + 8 * g));
        else
          return r[g];
      };
      constexpr int NA = 2 * NKS;
      Frag buf[kLook];
#pragma unroll
      for (int x = 0; x < kLook; ++x) buf[x] = kfrag(x);
#pragma unroll
      for (int idx = 0; idx < NA; ++idx) {
        const Frag cur = buf[idx % kLook];
        if (idx + kLook < NA) buf[idx % kLook] = kfrag(idx + kLook);
        if ((idx >> 1) < NKH)
          sacc[idx & 1] = mma(cur, qf[idx >> 1], sacc[idx & 1]);
        else
          sacc[idx & 1] = mma_pair(cur, qf[idx >> 1], sacc[idx & 1]);
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
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = 32 * kb + 8 * (v >> 2) + 4 * g + (v & 3);
          const float* bp = reinterpret_cast<const float*>(Ks) + j * SM::kRow + kCSlot;
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < 15; ++e) {
            if (e < 3 * Pqk) {
              const float t = ad[e] - bp[e];
              d = fmaf(t, t, d);
            }
          }
          sacc[kb][v] = fmaf(-kap, d, sacc[kb][v]);
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 cv = *reinterpret_cast<const float4*>(&colbuf[w][32 * kb + 8 * k + 4 * g]);
        sacc[kb][4 * k + 0] += cv.x;
        sacc[kb][4 * k + 1] += cv.y;
        sacc[kb][4 * k + 2] += cv.z;
        sacc[kb][4 * k + 3] += cv.w;
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sacc[kb][4 * k + e]);
      }
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
      for (int fb = 0; fb < NFB; ++fb) oacc[fb] *= al;
    }
    const float shift = (m_run == -INFINITY) ? 0.f : m_run - rterm;

    // probabilities -> B operand of O^T = V^T P^T
    Frag pf[sizeof(T) == 2 ? 4 : 32];
    float lt = 0.f;
    if constexpr (sizeof(T) == 2) {
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int kb = st >> 1, v0 = 8 * (st & 1);
        bf16x2 pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f32x2 pv = {__builtin_amdgcn_exp2f(sacc[kb][v0 + 2 * e] - shift),
                      __builtin_amdgcn_exp2f(sacc[kb][v0 + 2 * e + 1] - shift)};
          pk[e] = __builtin_convertvector(pv, bf16x2);
          lt = __builtin_amdgcn_fdot2_f32_bf16(pk[e], ones, lt, false);
        }
        pf[st] = bf16x8{pk[0][0], pk[0][1], pk[1][0], pk[1][1],
                        pk[2][0], pk[2][1], pk[3][0], pk[3][1]};
      }
    } else {
#pragma unroll
      for (int st = 0; st < 32; ++st) {
        const float p = __builtin_amdgcn_exp2f(sacc[st >> 4][st & 15] - shift);
        pf[st] = p;
        lt += p;
      }
    }
    l_own += lt;
    ocx += lt * cJ.x; ocy += lt * cJ.y; ocz += lt * cJ.z;

    wait_vm();        // this wave's part of the value tile has landed
    __syncthreads();  // ... and everyone's; all waves are done with the key tile
    if (tn < nJ) load_k(tile_of(tn));

    // ---------------- phase B: O^T += V^T P^T ----------------
    {
      auto vfrag = [&](int idx) -> Frag {
        const int fb = idx / NST, st = idx % NST;
        const T* vrow = Vs + (fb / 2) * (SM::kPanel / (int)sizeof(T)) + (32 * (fb % 2) + n) * SM::kRow;
        if constexpr (sizeof(T) == 2)
          return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(vrow + 16 * st + 8 * g));
        else
          return vrow[2 * st + g];
      };
      constexpr int NB = NFB * NST;
      Frag buf[kLook];
#pragma unroll
      for (int x = 0; x < kLook; ++x) buf[x] = vfrag(x);
#pragma unroll
      for (int idx = 0; idx < NB; ++idx) {
        const Frag cur = buf[idx % kLook];
        if (idx + kLook < NB) buf[idx % kLook] = vfrag(idx + kLook);
        oacc[idx / NST] = mma(cur, pf[idx % NST], oacc[idx / NST]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_vm();        // next key tile has landed
    __syncthreads();  // all waves are done with the value tile
    t = tn;
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

  // scalar channels: features 8k + 4g + e (k = 0, 1) of the first block
  if (in_range) {
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
  float* pbuf = reinterpret_cast<float*>(smem) + (size_t)w * 32 * Cz;
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
          const int u = 32 * (fb - 2) + 8 * k + 4 * g + e;
          if (u < RCz) {
            const int c = u % Cz;
            const float z = ld_in<T>(a.z1, ((size_t)b * L + i) * RCz + u);
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
