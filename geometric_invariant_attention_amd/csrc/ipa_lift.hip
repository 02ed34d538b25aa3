// ipa_lift: frames -> centred global points -> lifted query/key/value rows.
//
// For every residue block J of 64 residues and every head h this kernel
// writes the operands that the fused attention kernel consumes, so that the
// logit of "Flash Invariant Point Attention" (TL;DR: lift every IPA term
// into one regular attention) is a plain dot product plus cheap per-row /
// per-column terms. On the bf16 path (point groups of 15 slots; unused
// slots, 3 Pqk .. 14, are zero):
//
//   query head row  [ a q (16) | 2k A'hi (15) | 2k A'hi (15) | 2k A'lo (15) | 0 (3) ]
//   key head row    [   k (16) |    B'hi (15) |    B'lo (15) |    B'hi (15) | 0 (3) ]
//   key pair row    [ z2_j1 | ... | z2_jR | 0 ]   (shared by all heads, 64x64 panels)
//   value head row  [ v (16) | G'hi x, y, z (8 each) | G'lo x, y, z (8 each) ]
//   value pair row  [ z2_j1 | ... | z2_jR | 0 ]   (shared by all heads)
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
// Work split. Grid (block J, head h or pair panel, batch b), 4 waves, one
// residue per lane: in a head workgroup wave 0 writes the query rows, wave 1
// the key rows and the key column terms, waves 2 and 3 the two halves of the
// value block (lane = key position); every wave forms the block centre
// itself with cross-lane sums. In a pair workgroup wave 0 writes the key
// pair panel and waves 1 and 2 the two halves of the value pair panel. Rows
// are assembled in registers and written through per-wave LDS staging with
// 16-byte stores (value blocks: one coalesced row of 64 positions per
// store); all loads are unconditional buffer loads (rows past L read row
// L - 1) whose values invalid residues drop, each lane reading its input
// rows with 16-byte loads where their length and alignment allow.
//
// On the bf16 path the kernel also assembles, for every query and head, the
// logit of the query with its own key, which the attention kernel takes as
// the start of its running max: the head part (the key wave hands its rows
// to the query wave through LDS) plus the key's column term in the w of the
// query row term, and the pair part per 64-wide panel from the pair
// workgroups (all four waves, heads split between them).

#include "ipa_internal.h"

namespace ipa {
namespace {

constexpr int kPtSlot = 15;   // query/key point coordinates per group (3 Pqk <= 15)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// round to nearest even (hardware conversion; inputs are finite)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// fp16, round to nearest even, saturated to the finite range
__device__ __forceinline__ uint16_t f32_to_f16_sat(float x) {
  x = fminf(fmaxf(x, -65504.f), 65504.f);
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Resource over `bytes` bytes `off` bytes into `p`, or an empty resource
// (every load reads zero, every store is dropped) when `p` is NULL; no
// offset is ever applied to a NULL pointer.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_or_empty(const void* p, size_t off, uint32_t bytes) {
  return p ? make_rsrc(static_cast<const unsigned char*>(p) + off, bytes) : make_rsrc(nullptr, 0u);
}

// Element-type policy of the lifted rows.
template <typename T> struct Elt;
template <> struct Elt<uint16_t> {
  using S = uint16_t;
  static constexpr int kES = 2;
  static __device__ __forceinline__ S pack(float x) { return f32_to_bf16(x); }
  // hi/lo split: hi = bf16(x), lo = bf16(x - hi)
  static __device__ __forceinline__ void split(float x, S& hi, S& lo) {
    hi = f32_to_bf16(x);
    lo = f32_to_bf16(x - bf16_to_f32(hi));
  }
  static __device__ __forceinline__ S pack_pair(float x) { return f32_to_f16_sat(x); }
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, int byte_off, S v) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, byte_off, 0, 0);
  }
};
template <> struct Elt<float> {
  using S = float;
  static constexpr int kES = 4;
  static __device__ __forceinline__ S pack(float x) { return x; }
  static __device__ __forceinline__ void split(float x, S& hi, S& lo) { hi = x; lo = 0.f; }
  static __device__ __forceinline__ S pack_pair(float x) { return x; }
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, int byte_off, S v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_off, 0, 0);
  }
};

// Elements 0 .. NS-1 of the input row that starts `off` bytes into a buffer
// resource, `wide` bytes per load: 16 when the row length and the base keep
// 16-byte alignment, else 4, else one element. A lane reads its whole row
// with a few wide loads instead of one load per element (each load touches
// one cache line per lane, so the count of loads sets the cost). Elements
// past the row's end come from whatever follows it, or are zero past the
// end of the buffer; callers drop them.
template <typename T, int NS>
__device__ __forceinline__ void load_row(__amdgpu_buffer_rsrc_t r, int off, int wide, float (&out)[NS]) {
  if constexpr (sizeof(T) == 2) {
    if (wide == 16) {
#pragma unroll
      for (int k = 0; k < (NS + 7) / 8; ++k) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * k, 0, 0);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (8 * k + e < NS) out[8 * k + e] = __uint_as_float(e & 1 ? v[e / 2] & 0xFFFF0000u : v[e / 2] << 16);
      }
    } else if (wide == 4) {
#pragma unroll
      for (int k = 0; k < (NS + 1) / 2; ++k) {
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * k, 0, 0);
        out[2 * k] = __uint_as_float(v << 16);
        if (2 * k + 1 < NS) out[2 * k + 1] = __uint_as_float(v & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int k = 0; k < NS; ++k) out[k] = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, off + 2 * k, 0, 0));
    }
  } else {
    if (wide == 16) {
#pragma unroll
      for (int k = 0; k < (NS + 3) / 4; ++k) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * k, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * k + e < NS) out[4 * k + e] = __uint_as_float(v[e]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < NS; ++k) out[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * k, 0, 0));
    }
  }
}

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

// Pack N elements into 32-bit words.
template <int N>
__device__ __forceinline__ void pack_words(const uint16_t (&v)[N], uint32_t (&wv)[N / 2]) {
#pragma unroll
  for (int e = 0; e < N / 2; ++e) wv[e] = (uint32_t)v[2 * e] | ((uint32_t)v[2 * e + 1] << 16);
}
template <int N>
__device__ __forceinline__ void pack_words(const float (&v)[N], uint32_t (&wv)[N]) {
#pragma unroll
  for (int e = 0; e < N; ++e) wv[e] = __float_as_uint(v[e]);
}

// Per-wave LDS staging of a 64-row output block, so that global stores go
// out as whole contiguous 1 KB pieces instead of one row (or one 2-byte
// column element) per lane. Rows are padded by 16 bytes (conflict-free
// 16-byte accesses).
template <int ES>
struct Stage {
  static constexpr int kRowB = 64 * ES;        // bytes per row of 64 elements
  static constexpr int kPitch = kRowB + 16;    // padded LDS row
  static constexpr int kNC = kRowB / 16;       // 16-byte chunks per row
  static constexpr int kBytes = 64 * kPitch;
  // lane `lane` holds row `lane` (64 elements, words packed in w[]) and the
  // block [64 rows][64 elements] is written contiguously at dst
  static __device__ __forceinline__ void rows(unsigned char* xb, int lane, const uint32_t (&wv)[kRowB / 4],
                                              unsigned char* dst) {
#pragma unroll
    for (int c = 0; c < kNC; ++c)
      *reinterpret_cast<uint4*>(xb + lane * kPitch + 16 * c) =
          make_uint4(wv[4 * c], wv[4 * c + 1], wv[4 * c + 2], wv[4 * c + 3]);
    __builtin_amdgcn_wave_barrier();
    const int c = lane % kNC, r0 = lane / kNC;
#pragma unroll
    for (int k = 0; k < kNC; ++k) {
      const int r = r0 + k * (64 / kNC);
      *reinterpret_cast<uint4*>(dst + r * kRowB + 16 * c) = *reinterpret_cast<const uint4*>(xb + r * kPitch + 16 * c);
    }
  }
};

// 32 feature rows of a feature-major value block: lane p holds element p of
// each row; the rows (64 elements each) are written contiguously at dst.
template <typename S>
__device__ __forceinline__ void store_cols(unsigned char* xb, int lane, const S (&v)[32], unsigned char* dst) {
  constexpr int ES = (int)sizeof(S);
  using ST = Stage<ES>;
#pragma unroll
  for (int f = 0; f < 32; ++f) *reinterpret_cast<S*>(xb + f * ST::kPitch + lane * ES) = v[f];
  __builtin_amdgcn_wave_barrier();
  const int c = lane % ST::kNC, r0 = lane / ST::kNC;
#pragma unroll
  for (int k = 0; k < 32 / (64 / ST::kNC); ++k) {
    const int r = r0 + k * (64 / ST::kNC);
    *reinterpret_cast<uint4*>(dst + r * ST::kRowB + 16 * c) = *reinterpret_cast<const uint4*>(xb + r * ST::kPitch + 16 * c);
  }
}

// Sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <typename T>
__global__ __launch_bounds__(256) void ipa_lift_kernel(FwdArgs a) {
  using E = Elt<T>;
  using S = typename E::S;
  constexpr int ES = E::kES;
  const Layout& ly = a.lay;
  const int J = blockIdx.x, y = blockIdx.y, b = blockIdx.z;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int L = ly.L, H = ly.H, C = ly.C, Pqk = ly.Pqk, Pv = ly.Pv, RCz = ly.R * ly.Cz;
  const int Lp = ly.Lp, PW = ly.PW, nJ = ly.nJ;
  const size_t rb = (size_t)b * L;  // first residue row of batch b
  using ST = Stage<ES>;
  __shared__ __attribute__((aligned(16))) unsigned char xbuf[4][ST::kBytes];
  unsigned char* xb = xbuf[w];
  // bf16 path: the key wave's lifted head rows and column terms, handed to
  // the query wave for the logit of each query with its own key
  constexpr int XR = sizeof(T) == 2 ? kTileN : 1;
  __shared__ uint32_t kxr[XR][kHeadW / 2 + 1];
  __shared__ float kxc[XR];
  // bf16 path, pair workgroups: per wave, W_b weights of four heads over the
  // 64 columns of the panel
  __shared__ __attribute__((aligned(16))) float wtab[4][sizeof(T) == 2 ? 4 * 64 : 4];

  if (y < H) {
    // ================= head workgroup =================
    const int h = y;
    // residue of this lane; value waves take the key of their position
    const int j = w >= 2 ? key_of_pos<T>(lane) : lane;
    const int i = J * kTileN + j, ic = i < L ? i : L - 1;
    const bool valid = i < L && (a.mask == nullptr || a.mask[rb + ic] != 0);

    // frame of the residue and the block centre (mean translation of the
    // block's valid residues; every wave forms it for itself)
    float R[9], t[3];
    {
      const __attribute__((address_space(1))) float* tp =
          (const __attribute__((address_space(1))) float*)(a.trans + (rb + ic) * 3);
      // no rotations (distance attention): every local point is zero, so
      // the rotation never matters
      if (a.rot) {
        const __attribute__((address_space(1))) float* rp =
            (const __attribute__((address_space(1))) float*)(a.rot + (rb + ic) * 9);
#pragma unroll
        for (int e = 0; e < 9; ++e) R[e] = rp[e];
      } else {
#pragma unroll
        for (int e = 0; e < 9; ++e) R[e] = 0.f;
      }
#pragma unroll
      for (int x = 0; x < 3; ++x) t[x] = tp[x];
    }
    const float vf = valid ? 1.f : 0.f;
    const float cn = wave_sum(vf);
    const float cinv = cn > 0.f ? 1.f / cn : 0.f;
    const float cx = wave_sum(t[0] * vf) * cinv, cy = wave_sum(t[1] * vf) * cinv, cz = wave_sum(t[2] * vf) * cinv;
    if (h == 0 && w == 0 && lane == 0)
      reinterpret_cast<float4*>(a.ws + ly.off_cen)[(size_t)b * nJ + J] = make_float4(cx, cy, cz, cn);
    const float tc[3] = {t[0] - cx, t[1] - cy, t[2] - cz};

    // this head's input rows of the residue, through buffer resources over
    // batch b (32-bit offsets; the range check never faults)
    // (an absent input gets an empty range: its loads read zeros)
    auto in_rsrc = [&](const void* p, int per_row) {
      return rsrc_or_empty(p, rb * H * per_row * ES, (uint32_t)((size_t)L * H * per_row * ES));
    };
    // widest load that every row of this input keeps aligned
    auto width_of = [&](const void* p, int per_row) -> int {
      const uintptr_t base = reinterpret_cast<uintptr_t>(p) + rb * H * per_row * ES;
      const int rowb = per_row * ES;
      if (rowb % 16 == 0 && base % 16 == 0) return 16;
      if (rowb % 4 == 0 && base % 4 == 0) return 4;
      return ES;
    };
    const int row = ic * H + h;   // (residue, head) row within the batch

    const size_t o = ((size_t)b * H + h) * Lp + i;  // row of the per-(b, h) arrays
    // scalar and point weights (base 2): w_L / sqrt(C) and w_L gamma_h w_C / 2,
    // or rho_h and rho_h s_h^2 for the distance attention
    const float alpha = (a.meet_rho ? a.meet_rho[h] : a.w_L * rsqrtf((float)C)) * kLog2e;
    const float kap = (a.meet_rho ? a.meet_rho[h] * a.meet_s[h] * a.meet_s[h] : a.w_L * a.gamma[h] * a.w_C * 0.5f) * kLog2e;

    uint32_t own[kHeadW * ES / 4];   // query wave: its packed head row
    float4 qrow_v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (w <= 1) {
      // ---- query (wave 0) or key (wave 1) head row ----
      const __amdgpu_buffer_rsrc_t rs = in_rsrc(w == 0 ? a.q : a.k, C);
      const __amdgpu_buffer_rsrc_t rp = in_rsrc(w == 0 ? a.q_pts : a.k_pts, 3 * Pqk);
      float sc[kCSlot], pt[kPtSlot];
      load_row<T>(rs, row * C * ES, width_of(w == 0 ? a.q : a.k, C), sc);
      load_row<T>(rp, row * 3 * Pqk * ES, width_of(w == 0 ? a.q_pts : a.k_pts, 3 * Pqk), pt);
      // global, centred points
      float P[kPtSlot];
#pragma unroll
      for (int p = 0; p < 5; ++p)
#pragma unroll
        for (int x = 0; x < 3; ++x) {
          const float g = R[3 * x] * pt[3 * p] + R[3 * x + 1] * pt[3 * p + 1] + R[3 * x + 2] * pt[3 * p + 2] + tc[x];
          P[3 * p + x] = (valid && p < Pqk) ? g : 0.f;
        }
      S rowv[kHeadW];
#pragma unroll
      for (int c = 0; c < kCSlot; ++c) {
        const float s = (valid && c < C) ? sc[c] : 0.f;
        rowv[c] = E::pack(w == 0 ? alpha * s : s);
      }
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int u = 0; u < kPtSlot; ++u) {
          S hi, lo;
          E::split(w == 0 ? 2.f * kap * P[u] : P[u], hi, lo);
          // query [hi | hi | lo], key [hi | lo | hi]
          rowv[kCSlot + u] = hi;
          rowv[kCSlot + kPtSlot + u] = w == 0 ? hi : lo;
          rowv[kCSlot + 2 * kPtSlot + u] = w == 0 ? lo : hi;
        }
#pragma unroll
        for (int f = kCSlot + 3 * kPtSlot; f < kHeadW; ++f) rowv[f] = 0;
      } else {
        // fp32: key points at kCSlot.., unscaled query points at kFpQPts..;
        // the attention kernel forms the point term from explicit
        // differences, so they must not meet in the product
#pragma unroll
        for (int f = kCSlot; f < kHeadW; ++f) rowv[f] = 0.f;
        if (w == 0) {
#pragma unroll
          for (int u = 0; u < kPtSlot; ++u) rowv[kFpQPts + u] = P[u];
        } else {
#pragma unroll
          for (int u = 0; u < kPtSlot; ++u) rowv[kCSlot + u] = P[u];
        }
      }
      uint32_t wv[kHeadW * ES / 4];
      pack_words(rowv, wv);
      // rows J*64 .. J*64 + 63 of (b, h) are contiguous; lane j holds row j
      unsigned char* dst = a.ws + (w == 0 ? ly.off_qh : ly.off_kh) +
                           (((size_t)b * H + h) * Lp + (size_t)J * kTileN) * kHeadW * ES;
      ST::rows(xb, lane, wv, dst);
      float sx = 0.f, sy = 0.f, sz = 0.f, sn = 0.f;
#pragma unroll
      for (int p = 0; p < 5; ++p) {
        sx += P[3 * p]; sy += P[3 * p + 1]; sz += P[3 * p + 2];
        sn += P[3 * p] * P[3 * p] + P[3 * p + 1] * P[3 * p + 1] + P[3 * p + 2] * P[3 * p + 2];
      }
      if (w == 0) {
        qrow_v = make_float4(sx, sy, sz, 0.f);
#pragma unroll
        for (int e = 0; e < kHeadW * ES / 4; ++e) own[e] = wv[e];
      } else {
        // fp32 takes the whole point term from explicit differences
        const float4 kc = !valid ? make_float4(0.f, 0.f, 0.f, -INFINITY)
                                 : (sizeof(T) == 2 ? make_float4(sx, sy, sz, -kap * sn) : make_float4(0.f, 0.f, 0.f, 0.f));
        reinterpret_cast<float4*>(a.ws + ly.off_kcol)[o] = kc;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < kHeadW / 2; ++e) kxr[lane][e] = wv[e];
          kxc[lane] = kc.w;
        }
      }
    } else {
      // ---- value head block, feature-major [64 features][64 positions];
      //      wave 2 writes features 0..31, wave 3 features 32..63 ----
      const __amdgpu_buffer_rsrc_t rs = in_rsrc(a.v, C);
      const __amdgpu_buffer_rsrc_t rp = in_rsrc(a.v_pts, 3 * Pv);
      float G[3][kPvSlot];
      float vs[kCSlot];
      if (w == 2) load_row<T>(rs, row * C * ES, width_of(a.v, C), vs);
      {
        float pv[3 * kPvSlot];
        load_row<T>(rp, row * 3 * Pv * ES, width_of(a.v_pts, 3 * Pv), pv);
#pragma unroll
        for (int p = 0; p < kPvSlot; ++p)
#pragma unroll
          for (int x = 0; x < 3; ++x) {
            const float g = R[3 * x] * pv[3 * p] + R[3 * x + 1] * pv[3 * p + 1] + R[3 * x + 2] * pv[3 * p + 2] + tc[x];
            G[x][p] = (valid && p < Pv) ? g : 0.f;
          }
      }
      S out[32];
      if (w == 2) {
        // v (16), G'hi x (8), G'hi y (8)
#pragma unroll
        for (int c = 0; c < kCSlot; ++c) out[c] = E::pack((valid && c < C) ? vs[c] : 0.f);
#pragma unroll
        for (int p = 0; p < kPvSlot; ++p) {
          S hi, lo;
          E::split(G[0][p], hi, lo); out[16 + p] = hi;
          E::split(G[1][p], hi, lo); out[24 + p] = hi;
        }
      } else {
        // G'hi z (8), G'lo x, y, z (8 each)
#pragma unroll
        for (int p = 0; p < kPvSlot; ++p) {
          S hx, lx, hy, ly2, hz, lz;
          E::split(G[0][p], hx, lx);
          E::split(G[1][p], hy, ly2);
          E::split(G[2][p], hz, lz);
          out[p] = hz;
          out[8 + p] = lx;
          out[16 + p] = ly2;
          out[24 + p] = lz;
        }
      }
      const size_t blk = ((size_t)b * H + h) * nJ + J;   // value block of (b, h, J)
      store_cols(xb, lane, out, a.ws + ly.off_vth + (blk * kHeadW + (w - 2) * 32) * kTileN * ES);
    }
    // query row term; on the bf16 path its w holds the head part of the
    // logit of the query with its own key (lifted rows as the attention
    // products see them, plus the key's column term: the block offset is
    // zero), the running-max seed of the attention kernel
    if constexpr (sizeof(T) == 2) {
      __syncthreads();   // kxr, kxc
      if (w == 0) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < kHeadW / 2; ++e) {
          const uint32_t qe = own[e], ke = kxr[lane][e];
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qe), __builtin_bit_cast(bf16x2, ke), d, false);
        }
        qrow_v.w = d + kxc[lane];
      }
    }
    if (w == 0) reinterpret_cast<float4*>(a.ws + ly.off_qrow)[o] = qrow_v;
  } else {
    // ================= pair workgroup: one 64-wide panel of z2 =================
    // waves 0-2 write the panel; on the bf16 path wave 3 joins the pair
    // bias work below
    if (sizeof(T) == 4 && w == 3) return;
    const int P = y - H;
    const int j = (w == 0 || w == 3) ? lane : key_of_pos<T>(lane);
    const int i = J * kTileN + j, ic = i < L ? i : L - 1;
    const bool valid = i < L && (a.mask == nullptr || a.mask[rb + ic] != 0);
    // z2 row segment u = 64 P .. 64 P + 63 of the residue (16-byte loads:
    // R Cz is a multiple of 8, so rows and panels are 16-byte aligned; a
    // segment past the end of the batch reads zeros)
    const __amdgpu_buffer_rsrc_t rz = rsrc_or_empty(a.z2, rb * RCz * ES, (uint32_t)((size_t)L * RCz * ES));
    // bf16 path: the z1 segment and the first head group's W_b weights for
    // the pair bias below, issued together with the z2 loads
    constexpr int NZ1 = sizeof(T) == 2 ? 8 : 1;
    u32x4 z1r[NZ1];
    float wl0[4];
    const int uu = 64 * P + lane, cu = uu % ly.Cz;
    const float wsc = a.w_L * kLog2e;
    auto weights = [&](int h0, float (&wl)[4]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int hc = h0 + 4 * c < H ? h0 + 4 * c : H - 1;
        wl[c] = a.w_b ? wsc * a.w_b[(size_t)cu * H + hc] : 0.f;
      }
    };
    if constexpr (sizeof(T) == 2) {
      const __amdgpu_buffer_rsrc_t r1 = rsrc_or_empty(a.z1, rb * RCz * ES, (uint32_t)((size_t)L * RCz * ES));
#pragma unroll
      for (int c = 0; c < 8; ++c) z1r[c] = __builtin_amdgcn_raw_buffer_load_b128(r1, (ic * RCz + 64 * P) * ES + 16 * c, 0, 0);
      weights(w, wl0);
    }
    float z[64];
    u32x4 z2r[64 * ES / 16];
#pragma unroll
    for (int c = 0; c < 64 * ES / 16; ++c) z2r[c] = __builtin_amdgcn_raw_buffer_load_b128(rz, (ic * RCz + 64 * P) * ES + 16 * c, 0, 0);
    // keeps every load above in flight together (the compiler would
    // otherwise issue the z1 and weight loads only after the z2 work)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int c = 0; c < 64 * ES / 16; ++c) {
      const u32x4 r = z2r[c];
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          z[8 * c + 2 * e] = __uint_as_float(r[e] << 16);
          z[8 * c + 2 * e + 1] = __uint_as_float(r[e] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) z[4 * c + e] = __uint_as_float(r[e]);
      }
    }
#pragma unroll
    for (int u = 0; u < 64; ++u) z[u] = (valid && 64 * P + u < RCz) ? z[u] : 0.f;
    // bf16 path: this panel's share of each residue's pair bias with itself,
    // sum_u w_L log2(e) W_b[u mod Cz, h] z1[u] z2[u], for every head: the
    // pair part of the attention kernel's running-max seed. Wave w takes
    // heads w, w + 4, ... in groups of four: lane u loads the weights of
    // panel column u for the whole group at once, and they are broadcast
    // through this wave's LDS block.
    if constexpr (sizeof(T) == 2) {
      float zz[64];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const u32x4 r = z1r[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          zz[8 * c + 2 * e] = __uint_as_float(r[e] << 16) * z[8 * c + 2 * e];
          zz[8 * c + 2 * e + 1] = __uint_as_float(r[e] & 0xFFFF0000u) * z[8 * c + 2 * e + 1];
        }
      }
      float* const wt = wtab[w];
      float4* const pd = reinterpret_cast<float4*>(a.ws + ly.off_pdiag);
      for (int h0 = w; h0 < H; h0 += 16) {
        float wl[4];
        if (h0 == w) {
#pragma unroll
          for (int c = 0; c < 4; ++c) wl[c] = wl0[c];
        } else {
          weights(h0, wl);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) wt[64 * c + lane] = uu < RCz ? wl[c] : 0.f;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float acc = 0.f;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const float4 v = *reinterpret_cast<const float4*>(wt + 64 * c + 4 * q);
            acc = fmaf(v.x, zz[4 * q], acc);
            acc = fmaf(v.y, zz[4 * q + 1], acc);
            acc = fmaf(v.z, zz[4 * q + 2], acc);
            acc = fmaf(v.w, zz[4 * q + 3], acc);
          }
          const int h = h0 + 4 * c;
          if (h < H) reinterpret_cast<float*>(pd + ((size_t)b * H + h) * Lp + i)[P] = acc;
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      }
      if (w == 3) return;
    }
    if (w == 0) {
      // key pair row of residue j: [64 features] in panel P
      S rowv[64];
#pragma unroll
      for (int u = 0; u < 64; ++u) rowv[u] = E::pack_pair(z[u]);
      uint32_t wv[64 * ES / 4];
      pack_words(rowv, wv);
      ST::rows(xb, lane, wv, a.ws + ly.off_kz + ((((size_t)b * nJ + J) * (PW / 64) + P) * (64 * kTileN)) * ES);
    } else {
      // value pair block, feature-major: wave 1 features 0..31, wave 2 32..63
      const size_t blk = ((size_t)b * nJ + J) * PW + 64 * P;   // first feature row
      S out[32];
      if (w == 1) {
#pragma unroll
        for (int f = 0; f < 32; ++f) out[f] = E::pack(z[f]);
      } else {
#pragma unroll
        for (int f = 0; f < 32; ++f) out[f] = E::pack(z[32 + f]);
      }
      store_cols(xb, lane, out, a.ws + ly.off_vtz + (blk + (w - 1) * 32) * kTileN * ES);
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
