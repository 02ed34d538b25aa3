// ipa_lift: frames -> centred global points -> lifted query/key/value rows.
//
// For every residue block J of 64 residues and every head h this kernel
// writes the operands that the fused attention kernel consumes, so that the
// logit of "Flash Invariant Point Attention" (TL;DR: lift every IPA term
// into one regular attention) is a plain dot product plus cheap per-row /
// per-column terms. On the bf16 path (point groups of 16 slots, 15 for the
// coordinates and one zero; unused slots, 3 Pqk .. 14, are zero too):
//
//   query head row  [ a q (16) | 2k A'hi (15) 0 | 2k A'hi (15) 0 | 2k A'lo (15) 0 ]
//   key head row    [   k (16) |    B'hi (15) 0 |    B'lo (15) 0 |    B'hi (15) 0 ]
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
// Work split. Grid (block J, head h or pair panel, batch b), 4 waves. In a
// head workgroup (one residue per lane) wave 0 writes the query rows, wave
// 1 the key rows and the key column terms, waves 2 and 3 the two halves of
// the value block (lane = key position); every wave forms the block centre
// itself with cross-lane sums. Rows are assembled in registers and written
// through per-wave LDS staging with 16-byte stores (value blocks: one
// coalesced row of 64 positions per store). In a pair workgroup each
// residue's 64-wide panel segment is split over four lanes (16 features
// each, wave w taking residues 16 w .. 16 w + 15): key pair rows leave
// straight from registers, the value pair block goes through one LDS
// transpose. All loads are unconditional buffer loads (rows past L read row
// L - 1) whose values invalid residues drop, issued before the first of
// them is used, each lane reading its input rows with 16-byte loads where
// their length and alignment allow.
//
// On the bf16 path the kernel also assembles, for every query and head, the
// logit of the query with its own key, which the attention kernel takes as
// the start of its running max: the head part (the key wave hands its rows
// to the query wave through LDS) plus the key's column term in the w of the
// query row term, and the pair part per 64-wide panel from the pair
// workgroups (matrix-core products when no operand nears fp16's limit).

#include "ipa_internal.h"

namespace ipa {
namespace {

constexpr int kPtSlot = 15;   // query/key point coordinates per group (3 Pqk <= 15)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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

// 32-bit words that hold NS row elements of type T as issue_row loads them.
template <typename T> constexpr int raw_words(int NS) { return sizeof(T) == 2 ? 4 * ((NS + 7) / 8) : NS; }

// Issues the loads of elements 0 .. NS-1 of the input row that starts `off`
// bytes into a buffer resource, `wide` bytes per load: 16 when the row
// length and the base keep 16-byte alignment, else 4, else one element. A
// lane reads its whole row with a few wide loads instead of one load per
// element (each load touches one cache line per lane, so the count of loads
// sets the cost). The raw words land in `raw` (bf16 rows: element k in half
// k % 2 of word k / 2) and, for the wide loads, nothing here reads them, so
// the loads stay in flight until unpack_row; element-wise bf16 loads (rows
// that keep no 4-byte alignment) are packed here and wait. Elements past
// the row's end come from whatever follows it, or are zero past the end of
// the buffer; callers drop them.
template <typename T, int NS>
__device__ __forceinline__ void issue_row(__amdgpu_buffer_rsrc_t r, int off, int wide,
                                          uint32_t (&raw)[raw_words<T>(NS)]) {
  constexpr int EPL = 16 / sizeof(T);   // elements per 16-byte load
#pragma unroll
  for (int k = 0; k < raw_words<T>(NS); ++k) raw[k] = 0;
  if (wide == 16) {
#pragma unroll
    for (int k = 0; k < (NS + EPL - 1) / EPL; ++k) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * k, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * k + e < raw_words<T>(NS)) raw[4 * k + e] = v[e];
    }
  } else if (sizeof(T) == 4 || wide == 4) {
#pragma unroll
    for (int k = 0; k < (NS * (int)sizeof(T) + 3) / 4; ++k) raw[k] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * k, 0, 0);
  } else {
#pragma unroll
    for (int k = 0; k < (NS + 1) / 2; ++k) {
      const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, off + 4 * k, 0, 0);
      const uint32_t hi = 2 * k + 1 < NS ? __builtin_amdgcn_raw_buffer_load_b16(r, off + 4 * k + 2, 0, 0) : 0u;
      raw[k] = lo | hi << 16;
    }
  }
}

// The row elements of issue_row's raw words, as float32.
template <typename T, int NS, int NR>
__device__ __forceinline__ void unpack_row(const uint32_t (&raw)[NR], float (&out)[NS]) {
  static_assert(NR >= raw_words<T>(NS), "raw words too few for the row");
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    if constexpr (sizeof(T) == 2)
      out[k] = __uint_as_float(k & 1 ? raw[k / 2] & 0xFFFF0000u : raw[k / 2] << 16);
    else
      out[k] = __uint_as_float(raw[k]);
  }
}

// Key stored at position `pos` of a 64-key value block. The order matches
// the probability registers of the attention kernel's 32x32 products: for
// bf16 (K = 16 per product) each group of 16 keys is stored as 0-3, 8-11,
// 4-7, 12-15; for fp32 (K = 2 per product) each group of 32 keys is stored
// as pairs (8k+e, 8k+4+e).
template <typename T> __host__ __device__ constexpr int key_of_pos(int pos) {
  if (sizeof(T) == 2) {
    const int base = pos & ~15, p = pos & 15;
    const int g = p >> 3, s = p & 7;
    return base + 8 * (s >> 2) + 4 * g + (s & 3);
  }
  const int base = pos & ~31, p = pos & 31;
  const int g = p & 1, st = p >> 1;
  return base + 8 * (st >> 2) + 4 * g + (st & 3);
}

// Position of key k in its 64-key value block (the inverse of key_of_pos).
template <typename T> __host__ __device__ constexpr int pos_of_key(int k) {
  return sizeof(T) == 2 ? (k & ~15) + 8 * ((k >> 2) & 1) + 4 * ((k >> 3) & 1) + (k & 3)
                        : (k & ~31) + 8 * ((k & 31) >> 3) + 2 * (k & 3) + ((k >> 2) & 1);
}
template <typename T> constexpr bool positions_invert() {
  for (int p = 0; p < 64; ++p)
    if (pos_of_key<T>(key_of_pos<T>(p)) != p) return false;
  return true;
}
static_assert(positions_invert<uint16_t>() && positions_invert<float>(), "pos_of_key inverts key_of_pos");

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

// x of another lane of the same 16-lane row, by a DPP lane pattern (CTRL:
// 0x00-0xFF quad permutation, 0x140 row mirror, 0x141 half-row mirror).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 4 lanes of a quad (lanes 4k .. 4k + 3), in every one of them.
__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<0xB1>(x);   // lanes 1, 0, 3, 2 of the quad
  return x + dpp<0x4E>(x);   // lanes 2, 3, 0, 1
}

// Sum over the 64 lanes of a wave: quads, half rows and rows by DPP, then
// across rows. Every step adds two values that its partner lane adds in the
// other order, so all lanes end with the same value.
__device__ __forceinline__ float wave_sum(float x) {
  x = quad_sum(x);
  x += dpp<0x141>(x);   // the other quad of the half row
  x += dpp<0x140>(x);   // the other half of the row
  x += __shfl_xor(x, 16, 64);
  return x + __shfl_xor(x, 32, 64);
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
  // bf16 path, pair workgroups: W_b weights of 16 heads over the 64 columns
  // of the panel, and the largest |weight| each wave staged
  __shared__ __attribute__((aligned(16))) float wtab[sizeof(T) == 2 ? 16 : 1][64];
  __shared__ float wmax[4];

  if (y < H) {
    // ================= head workgroup =================
    const int h = y;
    // residue of this lane; value waves take the key of their position
    const int j = w >= 2 ? key_of_pos<T>(lane) : lane;
    const int i = J * kTileN + j, ic = i < L ? i : L - 1;
    const int row = ic * H + h;   // (residue, head) row within the batch

    // Every global load of the wave is issued here, before the first use of
    // any of them, so that the wave waits out one memory latency rather than
    // a chain of them. Absent inputs read through empty resources (zeros):
    // no rotations (distance attention) make every local point zero, so the
    // rotation never matters there.
    const uint32_t mbyte = __builtin_amdgcn_raw_buffer_load_b8(rsrc_or_empty(a.mask, rb, (uint32_t)L), ic, 0, 0);
    float R[9], t[3];
    {
      const __amdgpu_buffer_rsrc_t rr = rsrc_or_empty(a.rot, rb * 36, (uint32_t)((size_t)L * 36));
      const __amdgpu_buffer_rsrc_t rt = make_rsrc(a.trans + rb * 3, (uint32_t)((size_t)L * 12));
#pragma unroll
      for (int e = 0; e < 9; ++e) R[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rr, ic * 36 + 4 * e, 0, 0));
#pragma unroll
      for (int x = 0; x < 3; ++x) t[x] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rt, ic * 12 + 4 * x, 0, 0));
    }
    // per-head weights: gamma_h, or rho_h and s_h for the distance attention
    const float g_h = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc_or_empty(a.gamma, 0, 4u * H), 4 * h, 0, 0));
    const float rho_h = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc_or_empty(a.meet_rho, 0, 4u * H), 4 * h, 0, 0));
    const float s_h = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc_or_empty(a.meet_s, 0, 4u * H), 4 * h, 0, 0));

    // this head's input rows of the residue, through buffer resources over
    // batch b (32-bit offsets; the range check never faults)
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
    // scalar and point rows: the query (wave 0) or key (wave 1) rows, or the
    // value rows (waves 2, 3; only wave 2 writes the scalar part). One load
    // sequence for every wave: point rows are read 3 kPvSlot elements long
    // (the query and key waves drop the tail).
    const void* sp = w == 0 ? a.q : w == 1 ? a.k : a.v;
    const void* pp = w == 0 ? a.q_pts : w == 1 ? a.k_pts : a.v_pts;
    const int np = w <= 1 ? 3 * Pqk : 3 * Pv;
    uint32_t rsc[raw_words<T>(kCSlot)], rpt[raw_words<T>(3 * kPvSlot)];
    issue_row<T, kCSlot>(in_rsrc(sp, C), row * C * ES, width_of(sp, C), rsc);
    issue_row<T, 3 * kPvSlot>(in_rsrc(pp, np), row * np * ES, width_of(pp, np), rpt);

    // the block centre: mean translation of the block's valid residues
    // (every wave forms it for itself)
    const bool valid = i < L && (a.mask == nullptr || mbyte != 0);
    const float vf = valid ? 1.f : 0.f;
    const float cn = wave_sum(vf);
    const float cinv = cn > 0.f ? 1.f / cn : 0.f;
    const float cx = wave_sum(t[0] * vf) * cinv, cy = wave_sum(t[1] * vf) * cinv, cz = wave_sum(t[2] * vf) * cinv;
    if (h == 0 && w == 0 && lane == 0)
      reinterpret_cast<float4*>(a.ws + ly.off_cen)[(size_t)b * nJ + J] = make_float4(cx, cy, cz, cn);
    const float tc[3] = {t[0] - cx, t[1] - cy, t[2] - cz};

    const size_t o = ((size_t)b * H + h) * Lp + i;  // row of the per-(b, h) arrays
    // scalar and point weights (base 2): w_L / sqrt(C) and w_L gamma_h w_C / 2,
    // or rho_h and rho_h s_h^2 for the distance attention
    const float alpha = (a.meet_rho ? rho_h : a.w_L * rsqrtf((float)C)) * kLog2e;
    const float kap = (a.meet_rho ? rho_h * s_h * s_h : a.w_L * g_h * a.w_C * 0.5f) * kLog2e;

    // Lifted head row of a query (isq) or key from its input rows, packed
    // into words, and the sums of its centred global points (x, y, z, and
    // the squared norm in w).
    auto head_row = [&](bool isq, const float (&s_in)[kCSlot], const float (&p_in)[kPtSlot],
                        uint32_t (&wv)[kHeadW * ES / 4]) -> float4 {
      // global, centred points
      float P[kPtSlot];
#pragma unroll
      for (int p = 0; p < 5; ++p)
#pragma unroll
        for (int x = 0; x < 3; ++x) {
          const float g = R[3 * x] * p_in[3 * p] + R[3 * x + 1] * p_in[3 * p + 1] + R[3 * x + 2] * p_in[3 * p + 2] + tc[x];
          P[3 * p + x] = (valid && p < Pqk) ? g : 0.f;
        }
      if constexpr (sizeof(T) == 2) {
        // two elements per word, converted in pairs (round to nearest even):
        // the scalar part, then three 16-slot point groups, each 15
        // coordinates and a zero, query [hi | hi | lo], key [hi | lo | hi]
#pragma unroll
        for (int k = 0; k < kCSlot / 2; ++k) {
          f32x2 x;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float v = (valid && 2 * k + e < C) ? s_in[2 * k + e] : 0.f;
            x[e] = isq ? alpha * v : v;
          }
          wv[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
        }
        const float ps = isq ? 2.f * kap : 1.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const f32x2 x = {ps * P[2 * k], 2 * k + 1 < kPtSlot ? ps * P[2 * k + 1] : 0.f};
          const uint32_t hw = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
          const f32x2 r = {x[0] - __uint_as_float(hw << 16), x[1] - __uint_as_float(hw & 0xFFFF0000u)};
          const uint32_t lw = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
          wv[kCSlot / 2 + k] = hw;
          wv[kCSlot / 2 + 8 + k] = isq ? hw : lw;
          wv[kCSlot / 2 + 16 + k] = isq ? lw : hw;
        }
      } else {
        S rowv[kHeadW];
#pragma unroll
        for (int c = 0; c < kCSlot; ++c) {
          const float v = (valid && c < C) ? s_in[c] : 0.f;
          rowv[c] = E::pack(isq ? alpha * v : v);
        }
        // fp32: key points at kCSlot.., unscaled query points at kFpQPts..;
        // the attention kernel forms the point term from explicit
        // differences, so they must not meet in the product
#pragma unroll
        for (int f = kCSlot; f < kHeadW; ++f) rowv[f] = 0.f;
        if (isq) {
#pragma unroll
          for (int u = 0; u < kPtSlot; ++u) rowv[kFpQPts + u] = P[u];
        } else {
#pragma unroll
          for (int u = 0; u < kPtSlot; ++u) rowv[kCSlot + u] = P[u];
        }
        pack_words(rowv, wv);
      }
      float sx = 0.f, sy = 0.f, sz = 0.f, sn = 0.f;
#pragma unroll
      for (int p = 0; p < 5; ++p) {
        sx += P[3 * p]; sy += P[3 * p + 1]; sz += P[3 * p + 2];
        sn += P[3 * p] * P[3 * p] + P[3 * p + 1] * P[3 * p + 1] + P[3 * p + 2] * P[3 * p + 2];
      }
      return make_float4(sx, sy, sz, sn);
    };
    // column term of a key (fp32 takes the whole point term from explicit
    // differences)
    auto key_col = [&](float4 ps) {
      return !valid ? make_float4(0.f, 0.f, 0.f, -INFINITY)
                    : (sizeof(T) == 2 ? make_float4(ps.x, ps.y, ps.z, -kap * ps.w) : make_float4(0.f, 0.f, 0.f, 0.f));
    };

    // Every wave forms its rows first; on the bf16 path the key wave hands
    // its rows and column terms to the query wave through LDS, and after one
    // barrier every wave writes its rows out while the query wave takes the
    // logit of each query with its own key.
    uint32_t wv[kHeadW * ES / 4];   // query or key wave: its packed head row
    float4 ps = make_float4(0.f, 0.f, 0.f, 0.f);
    S out[32];                      // value waves: their 32 feature rows
    if (w <= 1) {
      // ---- query (wave 0) or key (wave 1) head row ----
      float sc[kCSlot], pt[kPtSlot];
      unpack_row<T>(rsc, sc);
      unpack_row<T>(rpt, pt);
      ps = head_row(w == 0, sc, pt, wv);
      if (sizeof(T) == 2 && w == 1) {
#pragma unroll
        for (int e = 0; e < kHeadW / 2; ++e) kxr[lane][e] = wv[e];
        kxc[lane] = key_col(ps).w;
      }
    } else {
      // ---- value head block, feature-major [64 features][64 positions];
      //      wave 2 writes features 0..31, wave 3 features 32..63 ----
      float sc[kCSlot], pv[3 * kPvSlot];
      if (w == 2) unpack_row<T>(rsc, sc);
      unpack_row<T>(rpt, pv);
      float G[3][kPvSlot];
#pragma unroll
      for (int p = 0; p < kPvSlot; ++p)
#pragma unroll
        for (int x = 0; x < 3; ++x) {
          const float g = R[3 * x] * pv[3 * p] + R[3 * x + 1] * pv[3 * p + 1] + R[3 * x + 2] * pv[3 * p + 2] + tc[x];
          G[x][p] = (valid && p < Pv) ? g : 0.f;
        }
      if (w == 2) {
        // v (16), G'hi x (8), G'hi y (8)
#pragma unroll
        for (int c = 0; c < kCSlot; ++c) out[c] = E::pack((valid && c < C) ? sc[c] : 0.f);
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
    }
    if constexpr (sizeof(T) == 2) __syncthreads();   // kxr, kxc
    if (w <= 1) {
      // rows J*64 .. J*64 + 63 of (b, h) are contiguous; lane j holds row j
      unsigned char* dst = a.ws + (w == 0 ? ly.off_qh : ly.off_kh) +
                           (((size_t)b * H + h) * Lp + (size_t)J * kTileN) * kHeadW * ES;
      ST::rows(xb, lane, wv, dst);
      if (w == 0) {
        // query row term; on the bf16 path its w holds the head part of the
        // logit of the query with its own key (lifted rows as the attention
        // products see them, plus the key's column term: the block offset
        // is zero), the running-max seed of the attention kernel
        float4 qrow_v = make_float4(ps.x, ps.y, ps.z, 0.f);
        if constexpr (sizeof(T) == 2) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < kHeadW / 2; ++e)
            d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv[e]), __builtin_bit_cast(bf16x2, kxr[lane][e]), d, false);
          qrow_v.w = d + kxc[lane];
        }
        reinterpret_cast<float4*>(a.ws + ly.off_qrow)[o] = qrow_v;
      } else {
        reinterpret_cast<float4*>(a.ws + ly.off_kcol)[o] = key_col(ps);
      }
    } else {
      const size_t blk = ((size_t)b * H + h) * nJ + J;   // value block of (b, h, J)
      store_cols(xb, lane, out, a.ws + ly.off_vth + (blk * kHeadW + (w - 2) * 32) * kTileN * ES);
    }
  } else {
    // ================= pair workgroup: one 64-wide panel of z2 =================
    // 64 residues x 64 features of the panel: wave w takes residues
    // 16 w .. 16 w + 15 with four lanes per residue, lane 16 q + r' holding
    // features 16 q .. 16 q + 15 of residue 16 w + r'. Every input is read
    // once per workgroup, each lane does a quarter of a residue's work, and
    // the key pair rows leave straight from registers (each lane's 16
    // features are contiguous in the panel row).
    const int P = y - H;
    const int r = 16 * w + (lane & 15), q = lane >> 4;
    const int i = J * kTileN + r, ic = i < L ? i : L - 1;
    constexpr int EQ = ES;   // 16-byte pieces of a lane's 16 features
    // every load is unconditional (absent inputs read zeros), so that all of
    // them are in flight together; R Cz is a multiple of 8, so every piece
    // is 16-byte aligned, and a piece past the end of the batch reads zeros
    const uint32_t mbyte = __builtin_amdgcn_raw_buffer_load_b8(rsrc_or_empty(a.mask, rb, (uint32_t)L), ic, 0, 0);
    const __amdgpu_buffer_rsrc_t rz = rsrc_or_empty(a.z2, rb * RCz * ES, (uint32_t)((size_t)L * RCz * ES));
    const int zoff = (ic * RCz + 64 * P + 16 * q) * ES;
    u32x4 z2r[EQ];
#pragma unroll
    for (int c = 0; c < EQ; ++c) z2r[c] = __builtin_amdgcn_raw_buffer_load_b128(rz, zoff + 16 * c, 0, 0);
    // bf16 path: the lane's z1 features and the first chunk of W_b weights
    // (entries tid, tid + 256, ... of a [16 heads][64 columns] block: column
    // t = tid % 64 of the panel, heads tid / 64 + 4 k of the chunk)
    u32x4 z1r[sizeof(T) == 2 ? EQ : 1];
    const int tcol = threadIdx.x & 63, uu = 64 * P + tcol;
    const int cu = uu % ly.Cz;
    const float wsc = a.w_L * kLog2e;
    const __amdgpu_buffer_rsrc_t rw = rsrc_or_empty(a.w_b, 0, (uint32_t)((size_t)ly.Cz * H * 4));
    auto weight = [&](int h) {
      const float x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rw, (cu * H + (h < H ? h : H - 1)) * 4, 0, 0));
      return (h < H && uu < RCz) ? wsc * x : 0.f;
    };
    float wl[4];
    if constexpr (sizeof(T) == 2) {
      const __amdgpu_buffer_rsrc_t r1 = rsrc_or_empty(a.z1, rb * RCz * ES, (uint32_t)((size_t)L * RCz * ES));
#pragma unroll
      for (int c = 0; c < EQ; ++c) z1r[c] = __builtin_amdgcn_raw_buffer_load_b128(r1, zoff + 16 * c, 0, 0);
#pragma unroll
      for (int k = 0; k < 4; ++k) wl[k] = weight((threadIdx.x >> 6) + 4 * k);
    }
    const bool valid = i < L && (a.mask == nullptr || mbyte != 0);

    // z2 of the lane's features as float, zero for invalid residues and for
    // features past R Cz
    float z2f[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float x;
      if constexpr (sizeof(T) == 2) {
        const uint32_t wd = z2r[e / 8][(e % 8) / 2];
        x = __uint_as_float(e & 1 ? wd & 0xFFFF0000u : wd << 16);
      } else {
        x = __uint_as_float(z2r[e / 4][e % 4]);
      }
      z2f[e] = (valid && 64 * P + 16 * q + e < RCz) ? x : 0.f;
    }

    // key pair row piece: features 16 q .. 16 q + 15 of residue r
    {
      S kv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) kv[e] = E::pack_pair(z2f[e]);
      uint32_t kw[16 * ES / 4];
      pack_words(kv, kw);
      unsigned char* dst = a.ws + ly.off_kz +
                           ((((size_t)b * nJ + J) * (PW / 64) + P) * (64 * kTileN) + (size_t)r * 64 + 16 * q) * ES;
#pragma unroll
      for (int c = 0; c < EQ; ++c)
        *reinterpret_cast<uint4*>(dst + 16 * c) = make_uint4(kw[4 * c], kw[4 * c + 1], kw[4 * c + 2], kw[4 * c + 3]);
    }
    // value pair block, feature-major [64 features][64 positions] (position
    // of key r: pos_of_key), transposed through LDS
    unsigned char* const vs = &xbuf[0][0];
    {
      const int pos = pos_of_key<T>(r);
#pragma unroll
      for (int e = 0; e < 16; ++e) *reinterpret_cast<S*>(vs + (16 * q + e) * ST::kPitch + pos * ES) = E::pack(z2f[e]);
    }

    // bf16 path: this panel's share of each residue's pair bias with itself,
    // sum_u q[u] k[u] with the pair operands as the attention kernel's
    // products take them: q[u] = w_L log2(e) W_b[u mod Cz, h] z1[u] and
    // k[u] = z2[u], each saturated to fp16's finite range (+-65504), for
    // every head: the pair part of the attention kernel's running-max seed,
    // so that the seed is a logit of those products (it then never exceeds
    // the row's largest logit by more than their rounding, whatever the
    // inputs). Heads go in chunks of 16, whose weights over the panel's 64
    // columns are staged in LDS. When no operand can reach the limit (the
    // largest |z1| of the lane times the largest staged |weight|, and |z2|,
    // within range) saturation is the identity, and the sums of a wave's 16
    // residues for 16 heads are one matrix product, [16 residues x 64
    // features] (z1 z2, fp16) times [64 features x 16 heads] (W_b, fp16),
    // four 16x16x16 products with float32 accumulation (feature 16 q + 4 s
    // + j of lane 16 q + r' is the reduction index 4 q + j of step s, on
    // both operands). Otherwise each lane sums its 16 saturated products and
    // the four lanes of a residue combine their sums.
    if constexpr (sizeof(T) == 2) {
      float z1f[16], zz[16];
      float m1 = 0.f, m2 = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t wd = z1r[e / 8][(e % 8) / 2];
        z1f[e] = __uint_as_float(e & 1 ? wd & 0xFFFF0000u : wd << 16);
        m1 = fmaxf(m1, fabsf(z1f[e]));
        m2 = fmaxf(m2, fabsf(z2f[e]));
        zz[e] = z1f[e] * z2f[e];
      }
      float4* const pd = reinterpret_cast<float4*>(a.ws + ly.off_pdiag);
      for (int h0 = 0; h0 < H; h0 += 16) {
        if (h0 > 0) {
#pragma unroll
          for (int k = 0; k < 4; ++k) wl[k] = weight(h0 + (threadIdx.x >> 6) + 4 * k);
        }
        float mx = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          wtab[(threadIdx.x >> 6) + 4 * k][tcol] = wl[k];
          mx = fmaxf(mx, fabsf(wl[k]));
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        if (lane == 0) wmax[w] = mx;
        __syncthreads();   // wtab, wmax (and, in the first chunk, the value block)
        const float mw = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        const bool plain = __all(m2 <= 65504.f && m1 * mw <= 65504.f);
        auto sat = [](float x) { return fminf(fmaxf(x, -65504.f), 65504.f); };
        const int nh = H - h0 < 16 ? H - h0 : 16;
        // (the products z1 z2 must be within fp16 range too; wave-uniform, as
        // the matrix-core products run on the whole wave)
        if (__all(plain && m1 * m2 <= 65504.f)) {
          f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const float4 wv = *reinterpret_cast<const float4*>(&wtab[lane & 15][16 * q + 4 * st]);
            const f16x4 bo = {(_Float16)wv.x, (_Float16)wv.y, (_Float16)wv.z, (_Float16)wv.w};
            const f16x4 ao = {(_Float16)zz[4 * st], (_Float16)zz[4 * st + 1], (_Float16)zz[4 * st + 2],
                              (_Float16)zz[4 * st + 3]};
            d = __builtin_amdgcn_mfma_f32_16x16x16f16(ao, bo, d, 0, 0, 0);
          }
          // lane l: residues 16 w + 4 (l / 16) + v, head h0 + l % 16
          const int hd = h0 + (lane & 15);
          if (hd < H) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              reinterpret_cast<float*>(pd + ((size_t)b * H + hd) * Lp + J * kTileN + 16 * w + 4 * q + v)[P] = d[v];
          }
          if (h0 + 16 < H) __syncthreads();   // wtab is refilled
          continue;
        }
        float acc[16];
#pragma unroll
        for (int hh = 0; hh < 16; ++hh) {
          const float* wr = &wtab[hh][16 * q];
          float x = 0.f;
          if (hh < nh) {
#pragma unroll
            for (int e = 0; e < 16; ++e) x = fmaf(plain ? wr[e] * z1f[e] : sat(wr[e] * z1f[e]), plain ? z2f[e] : sat(z2f[e]), x);
          }
          acc[hh] = x;
        }
        // the four lanes of the residue (lanes r', r' + 16, r' + 32, r' + 48)
        // combine their sums; lane 16 q + r' stores heads q, q + 4, ...
#pragma unroll
        for (int hh = 0; hh < 16; ++hh) {
          float x = acc[hh] + __shfl_xor(acc[hh], 16, 64);
          x += __shfl_xor(x, 32, 64);
          if (hh < nh && q == (hh & 3)) reinterpret_cast<float*>(pd + ((size_t)b * H + h0 + hh) * Lp + i)[P] = x;
        }
        if (h0 + 16 < H) __syncthreads();   // wtab is refilled
      }
    } else {
      __syncthreads();   // the value block
    }
    // rows 16 w .. 16 w + 15 of the value block, 16 bytes per lane per store
    {
      unsigned char* dst = a.ws + ly.off_vtz + (((size_t)b * nJ + J) * PW + 64 * P) * kTileN * ES;
#pragma unroll
      for (int k = 0; k < 16 * ST::kNC / 64; ++k) {
        const int c = lane + 64 * k, f = 16 * w + c / ST::kNC, ch = c % ST::kNC;
        *reinterpret_cast<uint4*>(dst + (size_t)f * ST::kRowB + 16 * ch) =
            *reinterpret_cast<const uint4*>(vs + f * ST::kPitch + 16 * ch);
      }
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
