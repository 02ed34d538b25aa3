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
// kLazy (base-2) units. Probabilities can then reach 2^kLazy; floating point
// is scale-free, so only overflow bounds kLazy: with 2^64, up to 2^16 keys
// and value entries below 2^16 in magnitude the accumulators stay under
// 2^96, far inside bf16/float32 range, and the final division by the row
// sum is unchanged. In practice the max then moves once, on the first tile
// with a valid key, and the output accumulators are never rescaled.
// Probabilities are rounded to bf16 once and the same rounded values feed
// the value product, the row sum and the block-centre correction, so the
// output is a convex combination of the value rows.

#include <type_traits>

#include "ipa_internal.h"

namespace ipa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLazy = 64.0f;
// Keys per tile of the key loop (the centring blocks stay 64 residues).
constexpr int kKT = 32;
// Bytes of one head's key and value rows above which the query blocks of a
// head start their key loop together (about three quarters of the 4 MB L2
// of one XCD, on which the blocks of a head run).
constexpr size_t kL2Share = (size_t)3 << 20;
// Operand fragments read ahead of the matrix-core products that use them.
constexpr int kLook = 6;

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
  using Frag = bf16x8;               // per-lane operand of one product
};
template <> struct Mma<float> {
  static constexpr int kStep = 2;
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


// Step boundary of a hand-scheduled product loop: memory operations (operand
// reads, tile copies) stay in their step; the instruction scheduler may still
// interleave the arithmetic across steps.
__device__ __forceinline__ void step_fence() { asm volatile("" ::: "memory"); }

// An empty, ordered statement that takes an accumulator tile in place: a
// product whose result passes through it stays in its step. No instruction
// is emitted and no register is read.
__device__ __forceinline__ void pin_step(f32x16& acc) { asm volatile("" : "+a"(acc)); }

// o *= al for one 32x32 accumulator tile, in place in the accumulation
// registers, so that the output accumulators never leave them (plain vector
// code on them would move the whole tile to architectural registers and
// back on every iteration). The caller first waits out the matrix-core write
// latency (acc_settle) and, after the last tile, lets the writes settle
// before the next product reads them.
__device__ __forceinline__ void scale_acc(f32x16& o, float al) {
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float t;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "v_mul_f32 %1, %1, %2\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(o[v]), "=&v"(t)
        : "v"(al));
  }
}
// 32 wait states: more than any matrix-core result or accumulation-register
// write needs before the next access to the same registers.
__device__ __forceinline__ void acc_settle() { asm volatile("s_nop 15\n\ts_nop 15"); }

// Buffer resource over `bytes` bytes at `base` (raw buffer, 32-bit data
// format); loads outside the range return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Resource over `bytes` bytes `off` bytes into `p`, or an empty resource
// (every load reads zero, every store is dropped) when `p` is NULL; no
// offset is ever applied to a NULL pointer.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_or_empty(const void* p, size_t off, uint32_t bytes) {
  return p ? make_rsrc(static_cast<const unsigned char*>(p) + off, bytes) : make_rsrc(nullptr, 0u);
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

// ZP: the pair panels are known to be zero (the distance attention, which
// has no pair representation, runs on 128-wide rows whose pair panel the lift
// leaves at zero): their copies, products and outputs are skipped, and so
// is every read of z1.
template <typename T, int D, bool ZP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ipa_attn_kernel(FwdArgs a) {
  using M = Mma<T>;
  using Frag = typename M::Frag;
  using SM = Smem<T, D>;
  constexpr int NKS = D / M::kStep;        // products per S^T tile
  constexpr int NKH = kHeadW / M::kStep;   // of which cover the head part
  constexpr int NFB = D / 32;              // 32-feature blocks of O^T
  constexpr int NP = SM::kNP;
  constexpr int NPC = ZP ? 1 : NP;         // panels copied per tile
  constexpr int NST = kKT / M::kStep;      // products per O^T block per tile
  // the probabilities of a tile are formed two per score step (bf16)
  static_assert(sizeof(T) == 4 || NKS >= 8, "at least 8 score steps per tile");
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
  __shared__ float colbuf[4][kKT];
  // per 64-key block: centre xyz and valid-key count, staged once so the key
  // loop reads nothing else from global memory
  __shared__ float4 cenS[kMaxTiles];
  // visiting order of the non-empty 32-key tiles (tile indices)
  __shared__ uint16_t seqS[2 * kMaxTiles];
  // w_L log2(e) W_b[:, h], the per-channel scale of the query pair columns
  __shared__ __attribute__((aligned(16))) float wbS[128];
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
    const float ws = a.w_L * kLog2e;
    for (int e = tid; e < Cz; e += 256) wbS[e] = a.w_b ? ws * a.w_b[(size_t)e * H + h] : 0.f;
  }
  __syncthreads();  // cenS, wbS

  // point weight (base 2): w_L gamma_h w_C / 2, or rho_h s_h^2 for the
  // distance attention
  const float kap = (a.meet_rho ? a.meet_rho[h] * a.meet_s[h] * a.meet_s[h] : a.w_L * a.gamma[h] * a.w_C * 0.5f) * kLog2e;
  const bool row_valid = (i < L) && (a.mask == nullptr || a.mask[(size_t)b * L + i] != 0);

  // ---- query operand (B operand of S^T = K Q^T), held for the whole loop ----
  // Loads are unconditional buffer loads (rows past L clamp to row 0, and
  // are zeroed afterwards) so that they all issue back to back.
  Frag qf[NKS];
  const int ic = i < L ? i : 0;
  if constexpr (sizeof(T) == 2) {
    const __amdgpu_buffer_rsrc_t rQ = make_rsrc(a.ws + ly.off_qh + bh * Lp * kHeadW * ES, (uint32_t)Lp * kHeadW * ES);
    const __amdgpu_buffer_rsrc_t rZ = rsrc_or_empty(a.z1, (size_t)b * L * RCz * ES, (uint32_t)L * RCz * ES);
    const int vq = (i * kHeadW + 8 * g) * ES;
    const int vz = (ic * RCz + 8 * g) * ES;
#pragma unroll
    for (int s = 0; s < NKH; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rQ, vq + 32 * s, 0, 0));
    u32x4 zr[NKS - NKH];
#pragma unroll
    for (int s = NKH; s < NKS; ++s)
      zr[s - NKH] = ZP ? u32x4{0u, 0u, 0u, 0u} : __builtin_amdgcn_raw_buffer_load_b128(rZ, vz + 32 * (s - NKH), 0, 0);
    // pair column u0 = 16 (s - NKH) + 8 g scales channel u0 mod Cz (stepped
    // without division; Cz >= 8)
    int c0 = 8 * g;
    if (c0 >= Cz) c0 -= Cz;
#pragma unroll
    for (int s = NKH; s < NKS; ++s) {
      const int u0 = 16 * (s - NKH) + 8 * g;
      const float4 w0 = *reinterpret_cast<const float4*>(&wbS[c0]);
      const float4 w1 = *reinterpret_cast<const float4*>(&wbS[c0 + 4]);
      const float ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t zw = zr[s - NKH][e];
        const float lo = __uint_as_float(zw << 16) * ws[2 * e];
        const float hi = __uint_as_float(zw & 0xFFFF0000u) * ws[2 * e + 1];
        o[e] = (uint32_t)f32_to_f16_sat(lo) | ((uint32_t)f32_to_f16_sat(hi) << 16);
      }
      const bool use = u0 < RCz && i < L;
      qf[s] = __builtin_bit_cast(bf16x8, use ? u32x4{o[0], o[1], o[2], o[3]} : u32x4{0u, 0u, 0u, 0u});
      c0 += 16;
      if (c0 >= Cz) c0 -= Cz;
      if (c0 >= Cz) c0 -= Cz;
    }
  } else {
    const float* Qh = reinterpret_cast<const float*>(a.ws + ly.off_qh) + (bh * Lp + i) * kHeadW;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int f = 2 * s + g;
      float v = 0.f;
      if (f < kHeadW) {
        v = Qh[f];
      } else {
        const int uu = f - kHeadW;
        if (a.z1 && uu < RCz && i < L) v = static_cast<const float*>(a.z1)[((size_t)b * L + i) * RCz + uu] * wbS[uu % Cz];
      }
      qf[s] = v;
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
  const float4 cI = cenS[qw / kTileN];

  // ---- direct-to-LDS copy of one tile (keys 32 t .. 32 t + 31) ----
  // Wave w issues loads w, w + 4, ... of every panel, so its per-lane source
  // offsets are fixed; all tile-dependent parts are wave-uniform (scalar).
  const __amdgpu_buffer_rsrc_t rKh = make_rsrc(Kh, (uint32_t)Lp * 64 * ES);
  const __amdgpu_buffer_rsrc_t rKz = make_rsrc(Kz, (uint32_t)nJ * (NP - 1) * 4096 * ES);
  const __amdgpu_buffer_rsrc_t rVh = make_rsrc(Vth, (uint32_t)nJ * 4096 * ES);
  const __amdgpu_buffer_rsrc_t rVz = make_rsrc(Vtz, (uint32_t)nJ * (NP - 1) * 4096 * ES);
  const __amdgpu_buffer_rsrc_t rKc = make_rsrc(kcol, (uint32_t)Lp * 16);

  // Running-max seed (bf16 path): the row's own logit s_ii, assembled by
  // the lift kernel (head part plus the key's column term in the row term's
  // w, the pair part per 64-wide panel; the block offset is zero). A real
  // logit, so a lower bound of the row max, and close to it: the query's own
  // residue is the key nearest in space. With the lazy threshold the first
  // key tiles then leave the max where it is instead of each nearer tile
  // moving it and rescaling the output.
  float m_seed = -INFINITY;
  if constexpr (sizeof(T) == 2) {
    const float4 pd = reinterpret_cast<const float4*>(a.ws + ly.off_pdiag)[bh * Lp + i];
    float sd = qr.w + pd.x;
    if constexpr (NP - 1 > 1) sd += pd.y;
    if constexpr (NP - 1 > 2) sd += pd.z;
    if constexpr (NP - 1 > 3) sd += pd.w;
    m_seed = sd;
  }
  const uint32_t voK = KS::voff(lane, w, 64 * ES);
  const uint32_t voV = VS::voff(lane, w, 64 * ES);
  // Key tiles are visited starting at this block's own diagonal tile, or,
  // on the bf16 path when a head's key and value rows exceed kL2Share
  // bytes, at tile 0: the query blocks of a head then stream the same tiles
  // at about the same time and share them in their XCD's L2 instead of each
  // pulling a different part of a working set that no longer fits there
  // (the running-max seed makes the first tile's position irrelevant to the
  // softmax; the fp32 path has no seed and keeps the diagonal start). Tiles
  // whose 64-key block has no valid key are skipped (they could only add
  // zeros). seqS[0 .. nseq) lists the visited tiles in order: built once,
  // 64 candidates per ballot, so that the key loop does no searching.
  const bool common_start = sizeof(T) == 2 && (size_t)Lp * (2 * kHeadW + 2 * (D - kHeadW)) * ES > kL2Share;
  const int T0 = common_start ? 0 : (qb * kTileM / kKT) % nT;
  int nseq = 0;
  for (int c = 0; c < nT; c += 64) {
    const int uu = c + lane;
    int t = T0 + uu;
    if (t >= nT) t -= nT;
    const bool f = uu < nT && cenS[(uu < nT ? t : 0) >> 1].w != 0.f;
    const uint64_t m = __ballot(f);
    if (f && w == 0) seqS[nseq + __popcll(m & ((1ull << lane) - 1ull))] = (uint16_t)t;
    nseq += __popcll(m);
  }
  __syncthreads();  // seqS
  // tile at sequence position s (past the end: the last one, a valid tile
  // whose copies are never read); readfirstlane marks it wave-uniform, and
  // with it every copy address
  auto tile_at = [&](int sq) -> int {
    return __builtin_amdgcn_readfirstlane((int)seqS[sq < nseq ? sq : nseq - 1]);
  };

  f32x16 oacc[NFB];
#pragma unroll
  for (int fb = 0; fb < NFB; ++fb) oacc[fb] = f32x16{};
  float m_run = m_seed, l_own = 0.f;
  float ocx = 0.f, ocy = 0.f, ocz = 0.f;

  // Column data of tile t (key lane & 31), read straight into registers one
  // iteration before use; lanes 32..63 duplicate lanes 0..31.
  auto load_kc = [&](int t) -> float4 {
    const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(rKc, (lane & 31) * 16, t * kKT * 16, 0);
    return make_float4(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[2]), __uint_as_float(r[3]));
  };
  // Column term of tile t (key lane & 31; both halves of the wave write the
  // same value) into colbuf[w]; returns the row term of this lane's query
  // against tile t.
  auto col_prep = [&](const float4 kc, const float4 cJ) -> float {
    const float dx = cI.x - cJ.x, dy = cI.y - cJ.y, dz = cI.z - cJ.z;
    colbuf[w][lane & 31] = kc.w + 2.f * kap * (dx * kc.x + dy * kc.y + dz * kc.z);
    return sizeof(T) == 4 ? 0.f
                          : -kap * (2.f * (dx * qr.x + dy * qr.y + dz * qr.z) +
                                    (float)Pqk * (dx * dx + dy * dy + dz * dz));
  };

  // Scores of tile t: S^T = K Q^T on the key buffer Kc, accumulated onto
  // sacc (lane (n, g) register v holds key 8 (v / 4) + 4 g + v % 4 of
  // query n). Each step issues the operand read kLook products ahead, one
  // product and side(step), a slice of independent vector work that runs in
  // the product's shadow; scheduling fences keep exactly this order.
  auto phase_a = [&](const float4 cJ, const unsigned char* Kc, f32x16 sacc, auto&& side) -> f32x16 {
    auto kfrag = [&](int s) -> Frag {
      if (ZP && s >= NKH) return Frag{};   // never used
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
    step_fence();
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const Frag cur = look[s % kLook];
      if (s + kLook < NKS) look[s % kLook] = kfrag(s + kLook);
      if (s < NKH)
        sacc = mma(cur, qf[s], sacc);
      else if constexpr (!ZP)
        sacc = mma_pair(cur, qf[s], sacc);
      // ties the product to this step (an ordered, empty statement that the
      // next product depends on); without it the products, which have no
      // side effects, may all be placed after the last step
      pin_step(sacc);
      side(s);
      step_fence();
    }
    if constexpr (sizeof(T) == 4) {
      // fp32: -k * sum_p |A'_ip + delta - B'_jp|^2 from explicit differences;
      // the expanded form would lose ~1e-5 logits to float32 cancellation
      const float dx = cI.x - cJ.x, dy = cI.y - cJ.y, dz = cI.z - cJ.z;
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
    return sacc;
  };

  // Column term of the keys this lane holds (colbuf[w] in the score layout).
  auto col_vals = [&]() -> f32x16 {
    f32x16 cv;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 c4 = *reinterpret_cast<const float4*>(&colbuf[w][8 * k + 4 * g]);
      cv[4 * k + 0] = c4.x; cv[4 * k + 1] = c4.y; cv[4 * k + 2] = c4.z; cv[4 * k + 3] = c4.w;
    }
    return cv;
  };

  // Row max of a score tile (this lane's 16 keys, then the partner lane's).
  auto row_max = [&](const f32x16& sc) -> float {
    float mx = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
#pragma unroll
    for (int v = 3; v < 16; ++v) mx = fmaxf(mx, sc[v]);
    return fmaxf(mx, __shfl_xor(mx, 32, 64));
  };

  // O^T += V^T P^T on the value buffer Vc, with side work as in phase_a.
  auto phase_b = [&](const unsigned char* Vc, const Frag* pf, auto&& side) {
    auto vfrag = [&](int idx) -> Frag {
      const int fb = idx / NST, s2 = idx % NST;
      if (ZP && fb >= kHeadW / 32) return Frag{};   // never used
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
    step_fence();
#pragma unroll
    for (int idx = 0; idx < NB; ++idx) {
      const Frag cur = look[idx % kLook];
      if (idx + kLook < NB) look[idx % kLook] = vfrag(idx + kLook);
      if (!ZP || idx / NST < kHeadW / 32) oacc[idx / NST] = mma(cur, pf[idx % NST], oacc[idx / NST]);
      side(idx);
      step_fence();
    }
  };

  // ---- software-pipelined key loop ----
  // Sequence index s visits the non-empty tiles u_0, u_1, ... Iteration s
  // holds the scores of u_s (sacc, with their row max) and
  //   1. starts the copies V(u_{s+1}) -> Vbuf[1-p], K(u_{s+2}) -> Kbuf[p]
  //      (p = s & 1; both buffers were last read in iteration s - 1),
  //   2. moves the running max if the scores of u_s call for it,
  //   3. turns the scores of u_s into probabilities while the matrix core
  //      computes the scores of u_{s+1} from Kbuf[1-p],
  //   4. accumulates V(u_s)^T P^T from Vbuf[p] while the row max of the new
  //      scores is taken,
  //   5. waits for its copies and meets the other waves at a barrier.
  // The exponentials and the max thus run in the shadow of the products.
  // Past the last tile the scores of a stale buffer are computed and
  // dropped (their values are finite or -inf).
  auto copy_k = [&](int t, unsigned char* Kd) {
    const int J = t >> 1, half = t & 1;
#pragma unroll
    for (int P = 0; P < NPC; ++P) {
      const uint32_t kbase = P == 0 ? (uint32_t)(J * 64 + 32 * half) * 64 * ES
                                    : (uint32_t)((J * (NP - 1) + P - 1) * 64 + 32 * half) * 64 * ES;
#pragma unroll
      for (int j = 0; j < KJ; ++j) {
        const int k = w + 4 * j;
        dma16(P == 0 ? rKh : rKz, voK, kbase + (uint32_t)(k * KS::kRPL * 64 * ES),
              Kd + P * SM::kKPanel + k * 1024);
      }
    }
  };
  // Source offsets of tile t: the head part (h) and the first pair panel
  // (z) of its key rows or value block; every copy op adds a constant of its
  // own (panel and wave), which the compiler keeps out of the loop.
  struct TileOff { uint32_t h, z; };
  auto key_off = [&](int t) -> TileOff {
    return {(uint32_t)t * (kKT * 64 * ES), (uint32_t)((t >> 1) * (NP - 1) * 64 + 32 * (t & 1)) * 64 * ES};
  };
  auto val_off = [&](int t) -> TileOff {
    return {(uint32_t)(t >> 1) * 4096 * ES + (uint32_t)(32 * (t & 1) * ES),
            (uint32_t)(t >> 1) * (NP - 1) * 4096 * ES + (uint32_t)(32 * (t & 1) * ES)};
  };
  // Direct-to-LDS copy op k of a tile pair: ops 0 .. NP VJ - 1 copy the
  // value tile at vo into Vd, the next NP KJ ops the key tile at ko into Kd.
  constexpr int NDMA = NPC * (VJ + KJ);
  auto dma_op = [&](int k, TileOff vo, unsigned char* Vd, TileOff ko, unsigned char* Kd) {
    if (k < NPC * VJ) {
      const int P = k / VJ, j = k % VJ;
      const int kk = w + 4 * j;
      const uint32_t c = (P == 0 ? 0u : (uint32_t)(P - 1) * 4096 * ES) + (uint32_t)(kk * VS::kRPL * 64 * ES);
      dma16(P == 0 ? rVh : rVz, voV, (P == 0 ? vo.h : vo.z) + c, Vd + P * SM::kVPanel + kk * 1024);
    } else {
      const int q = k - NPC * VJ;
      const int P = q / KJ, j = q % KJ;
      const int kk = w + 4 * j;
      const uint32_t c = (P == 0 ? 0u : (uint32_t)(P - 1) * 64 * 64 * ES) + (uint32_t)(kk * KS::kRPL * 64 * ES);
      dma16(P == 0 ? rKh : rKz, voK, (P == 0 ? ko.h : ko.z) + c, Kd + P * SM::kKPanel + kk * 1024);
    }
  };
  // The copy ops of one iteration, spread evenly over its first NKS +
  // 0.7 NB product steps (op k at step k NSPAN / NDMA): the address unit
  // drains them alongside the products instead of holding the wave up in a
  // burst, and the last one still has about a third of the value phase to
  // land before the iteration's wait. (Measured at L = 2048: spreading over
  // the whole iteration left ~200 cycles of that wait per tile, and packing
  // them into the score phase cost as much in issue slots.)
  constexpr int NSPAN = NKS + 7 * NFB * NST / 10;
  auto dma_at = [&](int step, TileOff tv, unsigned char* Vd, TileOff tk, unsigned char* Kd) {
#pragma unroll
    for (int k = 0; k < NDMA; ++k)
      if (k * NSPAN / NDMA == step) dma_op(k, tv, Vd, tk, Kd);
  };
  auto copy_v = [&](int t, unsigned char* Vd) {
    const int J = t >> 1, half = t & 1;
#pragma unroll
    for (int P = 0; P < NPC; ++P) {
      const uint32_t vbase = (P == 0 ? (uint32_t)J * 4096 * ES : (uint32_t)(J * (NP - 1) + P - 1) * 4096 * ES) +
                             (uint32_t)(32 * half * ES);
#pragma unroll
      for (int j = 0; j < VJ; ++j) {
        const int k = w + 4 * j;
        dma16(P == 0 ? rVh : rVz, voV, vbase + (uint32_t)(k * VS::kRPL * 64 * ES),
              Vd + P * SM::kVPanel + k * 1024);
      }
    }
  };

  if (nseq > 0) {
    int sq = 0;                                   // sequence position of this iteration
    int t0 = tile_at(0), t1 = tile_at(1), t2 = tile_at(2);
    copy_k(t0, K0);
    copy_v(t0, V0);
    copy_k(t1, K1);
    const float4 kc0 = load_kc(t0);
    float4 kc_n = load_kc(t1);                    // column data of t1
    float4 cJ0 = cenS[t0 >> 1], cJ1 = cenS[t1 >> 1];
    wait_vmem();
    __syncthreads();
    float rterm = col_prep(kc0, cJ0);
    // the column term is added by vector code, as in the loop, so that the
    // score tile enters the loop in the registers the loop carries it in
    f32x16 sacc = phase_a(cJ0, K0, f32x16{}, [](int) {});
    {
      const f32x16 cv = col_vals();
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[v] += cv[v];
    }
    float mx = row_max(sacc);
    __syncthreads();   // K0 is refilled from iteration 0 on

    // Iteration sq holds the scores of t0 = seq[sq] (sacc, row max mx) and
    //   1. moves the running max if those scores call for it,
    //   2. computes the scores of t1 = seq[sq + 1] from Kcur while, in the
    //      products' shadow, it turns the scores of t0 into probabilities,
    //      issues the copies V(t1) -> Vfill and K(t2) -> Kfill one per
    //      step, fetches the column data of t2 and writes the column term
    //      of t1,
    //   3. accumulates V(t0)^T P^T from Vcur while it adds the column term
    //      to the new scores, takes their row max and fetches seq[sq + 3]
    //      and the centre of t2 for the next iterations,
    //   4. waits for its copies and meets the other waves at a barrier.
    // The buffers alternate (p = sq & 1): Kcur holds K(t1), Vcur V(t0);
    // Kfill and Vfill were last read in iteration sq - 1. Past the end of the
    // sequence, t1 and t2 repeat its last tile: their scores and copies are
    // computed and never used.
    auto iteration = [&](auto pc) {
      constexpr int p = decltype(pc)::value;
      unsigned char* Kcur = p ? K0 : K1;
      unsigned char* Kfill = p ? K1 : K0;
      unsigned char* Vcur = p ? V1 : V0;
      unsigned char* Vfill = p ? V0 : V1;

      const float Mt = mx + rterm;
      const bool need = Mt > m_run + kLazy;
      if (__any(need)) {
        const float mn = need ? Mt : m_run;
        const float al = (mn == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - mn);
        // while every lane's running max is still -inf nothing has been
        // accumulated (all probabilities so far were zero): O needs no scaling
        const bool any_acc = __any(m_run != -INFINITY);
        m_run = mn;
        l_own *= al; ocx *= al; ocy *= al; ocz *= al;
        if (any_acc) {
          acc_settle();
#pragma unroll
          for (int fb = 0; fb < NFB; ++fb) scale_acc(oacc[fb], al);
          acc_settle();
        }
      }
      const float shift = (m_run == -INFINITY) ? 0.f : m_run - rterm;

      // scores of t1; the probabilities of t0 (bf16, rounded once: the same
      // values feed V^T P^T and the row sum) are formed two per product step
      Frag pf[NST];
      float lt = 0.f;
      bf16x2 pk[8];
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      float4 kc_nn;
      float rterm_n;
      const TileOff vo1 = val_off(t1), ko2 = key_off(t2);
      f32x16 sacc_n = phase_a(cJ1, Kcur, f32x16{}, [&](int st) {
        if constexpr (sizeof(T) == 2) {
          if (st < 8) {
            const f32x2 pv = {__builtin_amdgcn_exp2f(sacc[2 * st] - shift),
                              __builtin_amdgcn_exp2f(sacc[2 * st + 1] - shift)};
            pk[st] = __builtin_convertvector(pv, bf16x2);
            lt = __builtin_amdgcn_fdot2_f32_bf16(pk[st], ones, lt, false);
          }
        }
        dma_at(st, vo1, Vfill, ko2, Kfill);
        if (st == NKS - 3) kc_nn = load_kc(t2);
        if (st == NKS - 2) rterm_n = col_prep(kc_n, cJ1);
      });
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int s2 = 0; s2 < NST; ++s2)
          pf[s2] = bf16x8{pk[4 * s2][0], pk[4 * s2][1], pk[4 * s2 + 1][0], pk[4 * s2 + 1][1],
                          pk[4 * s2 + 2][0], pk[4 * s2 + 2][1], pk[4 * s2 + 3][0], pk[4 * s2 + 3][1]};
      } else {
#pragma unroll
        for (int s2 = 0; s2 < NST; ++s2) {
          const float pp = __builtin_amdgcn_exp2f(sacc[s2] - shift);
          pf[s2] = pp;
          lt += pp;
        }
      }
      l_own += lt;
      ocx += lt * cJ0.x; ocy += lt * cJ0.y; ocz += lt * cJ0.z;

      // values of t0; the column term is added to the new scores and their
      // row max taken in the shadow of the products (from step 2 on, when the
      // last score product has completed)
      const f32x16 cv = col_vals();
      float mxn = -INFINITY;
      int t3raw = 0;
      float4 cJ2;
      // (the side work is placed by step number, clamped to the phase: the
      // value phase has NB = 2 NFB products, 8 for the narrowest rows)
      constexpr int NB = NFB * NST;
      constexpr int kColEnd = NB < 10 ? NB : 10;         // column adds in steps 2 .. kColEnd - 1
      constexpr int kStCen = NB - 2 < 10 ? NB - 2 : 10;  // centre of t2
      constexpr int kStSeq = NB - 1 < 11 ? NB - 1 : 11;  // visiting order, seq[sq + 3]
      phase_b(Vcur, pf, [&](int st) {
        if constexpr (sizeof(T) == 2) {
          if (st >= 2 && st < kColEnd) {
            const int v = 2 * (st - 2);
            sacc_n[v] += cv[v];
            sacc_n[v + 1] += cv[v + 1];
            mxn = fmaxf(fmaxf(mxn, sacc_n[v]), sacc_n[v + 1]);
          }
        }
        dma_at(NKS + st, vo1, Vfill, ko2, Kfill);
        if (st == kStCen) cJ2 = cenS[t2 >> 1];
        // a plain LDS read here; it is made wave-uniform after the loop, so
        // that waiting for it does not stall the operand reads
        if (st == kStSeq) t3raw = seqS[sq + 3 < nseq ? sq + 3 : nseq - 1];
      });
      const int t3 = __builtin_amdgcn_readfirstlane(t3raw);
      if constexpr (sizeof(T) == 2) {
        // column adds the phase had no steps left for
#pragma unroll
        for (int v = 2 * (kColEnd - 2); v < 16; ++v) {
          sacc_n[v] += cv[v];
          mxn = fmaxf(mxn, sacc_n[v]);
        }
      }
      if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          sacc_n[v] += cv[v];
          mxn = fmaxf(mxn, sacc_n[v]);
        }
      }
      mx = fmaxf(mxn, __shfl_xor(mxn, 32, 64));
      sacc = sacc_n;
      rterm = rterm_n;
      kc_n = kc_nn;
      wait_vmem();
      __syncthreads();
      ++sq;
      t0 = t1; t1 = t2; t2 = t3;
      cJ0 = cJ1; cJ1 = cJ2;
    };
    // unrolled by two (static buffer parity); the second half is a branch of
    // the body rather than a second loop exit, so the accumulators keep
    // their registers across iterations
    while (sq < nseq) {
      iteration(std::integral_constant<int, 0>{});
      if (sq < nseq) iteration(std::integral_constant<int, 1>{});
    }
  }

  // ---------------- epilogue ----------------
  const float l_tot = l_own + __shfl_xor(l_own, 32, 64);
  const float gx_c = ocx + __shfl_xor(ocx, 32, 64);
  const float gy_c = ocy + __shfl_xor(ocy, 32, 64);
  const float gz_c = ocz + __shfl_xor(ocz, 32, 64);
  const bool ok = row_valid && l_tot > 0.f;
  const float inv = ok ? 1.f / l_tot : 0.f;

  // Every global access of the epilogue moves whole rows through this
  // wave's own staging block, one of the tile buffers (the loop's last
  // barrier follows every wave's last read of them and every copy into
  // them): row-major inputs are fetched with consecutive lanes on
  // consecutive pieces of consecutive rows, and outputs leave the same way,
  // rather than one cache line per lane per access in the register layout.
  // A wave's LDS operations execute in order, so the block is reused without
  // barriers; wave_sync only keeps the compiler from reordering them.
  unsigned char* const xs = w == 0 ? K0 : w == 1 ? K1 : w == 2 ? V0 : V1;
  static_assert(SM::kVBuf == SM::kKBuf && SM::kKBuf == 32 * D * ES, "staging block size");
  const int nrow = L - qw < 32 ? L - qw : 32;   // rows of this wave inside L (none if <= 0)
  auto wave_sync = [] {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  };

  // (1) the frames of rows qw .. qw + 31, then their z1 rows, are loaded;
  //     the frames go to LDS as [32][9] rotations and [32][3] translations
  //     at the end of the staging block, while the z1 loads stay in flight
  //     through the scalar and point outputs below. Rows past L read zeros.
  const int RB = RCz * ES;                      // bytes per z1 row, a multiple of 16
  const int CPR = RB / 16;                      // 16-byte chunks per row
  const int zm = (CPR & 7) == 0 ? 7 : (CPR & 3) == 0 ? 3 : (CPR & 1) == 0 ? 1 : 0;
  constexpr int kFrBytes = 32 * 12 * 4;
  static_assert(32 * (kCSlot + 3 * kPvSlot + kPvSlot + 3) * 4 + kFrBytes <= SM::kKBuf &&
                32 * SM::kPW * ES + kFrBytes <= SM::kKBuf, "staged outputs or z1 rows reach the frames");
  float* const fr = reinterpret_cast<float*>(xs + SM::kKBuf - kFrBytes);
  constexpr int NZL = (SM::kPW * ES / 16 + 1) / 2;   // loads for the widest z1 row
  u32x4 zv[NZL];
  int zo[NZL];
  {
    const __amdgpu_buffer_rsrc_t rZ = rsrc_or_empty(a.z1, (size_t)b * L * RB, (uint32_t)L * RB);
    const __amdgpu_buffer_rsrc_t rR = rsrc_or_empty(a.rot, (size_t)b * L * 36, (uint32_t)L * 36);
    const __amdgpu_buffer_rsrc_t rT = rsrc_or_empty(a.trans, (size_t)b * L * 12, (uint32_t)L * 12);
    float rv[5], tv[2];
#pragma unroll
    for (int s = 0; s < 5; ++s) rv[s] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rR, (qw * 9 + 64 * s + lane) * 4, 0, 0));
#pragma unroll
    for (int s = 0; s < 2; ++s) tv[s] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rT, (qw * 3 + 64 * s + lane) * 4, 0, 0));
    // chunk 64 s + lane of the block: row zr, chunk zc (stepped, no division
    // in the loop); chunk c of row r goes to slot c ^ (r & zm), so that the
    // 8 rows that 8 lanes read at once fall on distinct banks
    int zr = lane / CPR, zc = lane - zr * CPR;
    const int dr = 64 / CPR, dc = 64 - dr * CPR;
#pragma unroll
    for (int s = 0; s < NZL; ++s) {
      if (!ZP && 64 * s < 32 * CPR) zv[s] = __builtin_amdgcn_raw_buffer_load_b128(rZ, (qw + zr) * RB + 16 * zc, 0, 0);
      zo[s] = zr * RB + 16 * (zc ^ (zr & zm));
      zr += dr;
      zc += dc;
      if (zc >= CPR) { zc -= CPR; ++zr; }
    }
#pragma unroll
    for (int s = 0; s < 5; ++s)
      if (64 * s + lane < 32 * 9) fr[64 * s + lane] = rv[s];
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (64 * s + lane < 32 * 3) fr[32 * 9 + 64 * s + lane] = tv[s];
  }
  wave_sync();
  // (2) this lane's frame
  float R[9], tr[3];
#pragma unroll
  for (int e = 0; e < 9; ++e) R[e] = fr[9 * n + e];
#pragma unroll
  for (int e = 0; e < 3; ++e) tr[e] = fr[32 * 9 + 3 * n + e];

  // (3) scalar channels, points (T_i^-1 of the averaged global points) and
  //     their norms of row n, staged as [32][kCSlot + 1], [32][3 kPvSlot + 1]
  //     and [32][kPvSlot + 1] floats (columns past C, 3 Pv, Pv are never
  //     stored) and written out row-contiguously
  constexpr int PS = kCSlot + 1, PP = 3 * kPvSlot + 1, PN = kPvSlot + 1;
  float* const so = reinterpret_cast<float*>(xs);
  float* const sp = so + 32 * PS;
  float* const sn = sp + 32 * PP;
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) so[n * PS + 8 * k + 4 * g + e] = ok ? oacc[0][4 * k + e] * inv : 0.f;
  // value points 4g + e: hi x/y/z in registers (0,8+e) (0,12+e) (1,e),
  // lo x/y/z in (1,4+e) (1,8+e) (1,12+e)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int p = 4 * g + e;
    const float gx = (oacc[0][8 + e] + oacc[1][4 + e] + gx_c) * inv - tr[0];
    const float gy = (oacc[0][12 + e] + oacc[1][8 + e] + gy_c) * inv - tr[1];
    const float gz = (oacc[1][e] + oacc[1][12 + e] + gz_c) * inv - tr[2];
    const float lx = R[0] * gx + R[3] * gy + R[6] * gz;
    const float lyv = R[1] * gx + R[4] * gy + R[7] * gz;
    const float lz = R[2] * gx + R[5] * gy + R[8] * gz;
    const float nr = sqrtf(lx * lx + lyv * lyv + lz * lz);
    float* const pp = sp + n * PP + 3 * p;
    pp[0] = ok ? lx : 0.f;
    pp[1] = ok ? lyv : 0.f;
    pp[2] = ok ? lz : 0.f;
    sn[n * PN + p] = ok ? nr : 0.f;
  }
  wave_sync();
  // [32][cols] block staged at src (row pitch SP > cols) -> rows `pitch`
  // floats apart from dst; consecutive lanes take consecutive floats. Every
  // staged value is read first (rows clamped into the block), then the
  // stores go out back to back; the store resource ends after row nrow - 1,
  // so rows past L are dropped by its range check.
  // (an absent output gets an empty resource: nothing is written)
  auto store_rows = [&](auto sp_c, const float* src, int cols, float* out, size_t first, int pitch) {
    constexpr int SP = decltype(sp_c)::value;
    constexpr int NIT = 32 * (SP - 1) / 64;
    const __amdgpu_buffer_rsrc_t rs =
        rsrc_or_empty(out, first * 4, nrow > 0 ? (uint32_t)(((nrow - 1) * pitch + cols) * 4) : 0u);
    float v[NIT];
    int off[NIT];
    int r = lane / cols, c = lane - r * cols;
    const int dr = 64 / cols, dc = 64 - dr * cols;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      v[it] = src[(r < 32 ? r : 31) * SP + c];
      off[it] = (r * pitch + c) * 4;
      r += dr;
      c += dc;
      if (c >= cols) { c -= cols; ++r; }
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[it]), rs, off[it], 0, 0);
  };
  const size_t bi0 = (size_t)b * L + qw;   // residue (b, qw): first output row of this wave
  const int pS = (int)a.out_pitch[0], pP = (int)a.out_pitch[1], pN = (int)a.out_pitch[2], pZ = (int)a.out_pitch[3];
  store_rows(std::integral_constant<int, PS>{}, so, C, a.out_s, bi0 * pS + (size_t)h * C, pS);
  store_rows(std::integral_constant<int, PP>{}, sp, 3 * Pv, a.out_pts, bi0 * pP + (size_t)h * 3 * Pv, pP);
  store_rows(std::integral_constant<int, PN>{}, sn, Pv, a.out_pts_norm, bi0 * pN + (size_t)h * Pv, pN);
  if constexpr (ZP) return;   // no pair channels

  // (4) the z1 rows into the staging block (over the staged outputs above,
  //     whose reads precede these writes in this wave's LDS order), then
  //     this lane's z1 groups 8 q + 4 g .. + 3 of row n, kept packed until
  //     used
  wave_sync();
#pragma unroll
  for (int s = 0; s < NZL; ++s)
    if (!ZP && 64 * s + lane < 32 * CPR) *reinterpret_cast<u32x4*>(xs + zo[s]) = zv[s];
  wave_sync();
  constexpr int NG = (NFB - 2) * 4;              // pair feature groups per lane
  constexpr int ZW = sizeof(T) == 2 ? 2 : 4;     // 32-bit words per group
  uint32_t zp[NG][ZW];
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    if constexpr (sizeof(T) == 2) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(xs + n * RB + 16 * (q ^ (n & zm)) + 8 * g);
      zp[q][0] = v[0]; zp[q][1] = v[1];
    } else {
      const u32x4 v = *reinterpret_cast<const u32x4*>(xs + n * RB + 16 * ((2 * q + g) ^ (n & zm)));
#pragma unroll
      for (int e = 0; e < 4; ++e) zp[q][e] = v[e];
    }
  }
  auto zval = [&](int q, int e) -> float {
    if constexpr (sizeof(T) == 2)
      return __uint_as_float(e & 1 ? zp[q][e >> 1] & 0xFFFF0000u : zp[q][e >> 1] << 16);
    else
      return __uint_as_float(zp[q][e]);
  };

  // ---- pair channels: o_pair[c] = sum_r z1[r Cz + c] O[r Cz + c] / l ----
  // Lane (n, g) holds O at features 32 fb + 8 k + 4 g + e of query n: 4-wide
  // groups at feature 8 q + 4 g (q = 4 (fb - 2) + k). Cz is a multiple of 8,
  // so every rank component of a channel lands in the same lane.
  //
  // Cz a multiple of 32: rank component r of channel c = 32 m + 8 k + 4 g + e
  // is register 4 k + e of tile 2 + m + r Cz / 32, so the sum over r is
  // formed in registers (one specialisation per Cz / 32). Each 32-channel
  // group of the 32 rows is staged as [32][32] floats (chunk c of row r in
  // slot c ^ (r & 7)), two groups alternating, and stored as 128-byte row
  // pieces. Other Cz go through LDS below.
  bool pair_done = false;
  auto pair_regs = [&](auto sc) {
    constexpr int S = decltype(sc)::value;
    if constexpr (S * 32 <= SM::kCzMax) {
      constexpr int RMAX = (NFB - 2) / S;
      const __amdgpu_buffer_rsrc_t rs =
          rsrc_or_empty(a.out_pair, (bi0 * pZ + (size_t)h * Cz) * 4, nrow > 0 ? (uint32_t)(((nrow - 1) * pZ + Cz) * 4) : 0u);
#pragma unroll
      for (int m = 0; m < S; ++m) {
        unsigned char* const pb = xs + (m & 1) * 4096;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // only groups of rank components r < R (features < R Cz) are read
          float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int r = 0; r < RMAX; ++r) {
            if (r < ly.R) {
              const int fb = 2 + m + r * S, q = 4 * (m + r * S) + k;
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[e] = fmaf(zval(q, e), oacc[fb][4 * k + e], acc[e]);
            }
          }
          // rows that output zeros write +0.0
          *reinterpret_cast<float4*>(pb + n * 128 + 16 * ((2 * k + g) ^ (n & 7))) =
              ok ? make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        wave_sync();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = (lane >> 3) + 8 * j, c = lane & 7;
          const u32x4 v = *reinterpret_cast<const u32x4*>(pb + r * 128 + 16 * (c ^ (r & 7)));
          __builtin_amdgcn_raw_buffer_store_b128(v, rs, (r * pZ + 32 * m + 4 * c) * 4, 0, 0);
        }
      }
      pair_done = true;
    }
  };
  if ((Cz & 31) == 0) {
    switch (Cz >> 5) {
      case 1: pair_regs(std::integral_constant<int, 1>{}); break;
      case 2: pair_regs(std::integral_constant<int, 2>{}); break;
      case 3: pair_regs(std::integral_constant<int, 3>{}); break;
      case 4: pair_regs(std::integral_constant<int, 4>{}); break;
      default: break;
    }
  }
  if (pair_done) return;

  // general Cz: products into registers (groups past R Cz and rows that
  // output zeros take z = 0), then summed over r in a padded per-wave LDS
  // block, two waves at a time, and written out row by row
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    const int fb = 2 + q / 4, k = q % 4;
    const bool use = ok && 8 * q + 4 * g < RCz;
#pragma unroll
    for (int e = 0; e < 4; ++e) oacc[fb][4 * k + e] *= (use ? zval(q, e) : 0.f) * inv;
  }
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if ((w >> 1) == pass) {
      float* pb = &pbuf[w & 1][0][0];
      for (int e = lane; e < 32 * SM::kPRow; e += 64) pb[e] = 0.f;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      // channel of group q: (8 q + 4 g) mod Cz, stepped without division
      int c0 = 4 * g;
#pragma unroll
      for (int q = 0; q < NG; ++q) {
        const int fb = 2 + q / 4, k = q % 4;
        if (8 * q + 4 * g < RCz) {
          float* row = pb + n * SM::kPRow + c0;
#pragma unroll
          for (int e = 0; e < 4; ++e) row[e] += oacc[fb][4 * k + e];
        }
        c0 += 8;
        if (c0 >= Cz) c0 -= Cz;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      // 32 rows of Cz floats; lane walks entries lane, lane + 64, ...
      const int dq = 64 / Cz, dr = 64 - dq * Cz;
      int nn = lane / Cz, c = lane - nn * Cz;
      for (int e = lane; e < 32 * Cz; e += 64) {
        const int ii = qw + nn;
        if (a.out_pair && ii < L) a.out_pair[((size_t)b * L + ii) * pZ + (size_t)h * Cz + c] = pb[nn * SM::kPRow + c];
        nn += dq;
        c += dr;
        if (c >= Cz) { c -= Cz; ++nn; }
      }
    }
    __syncthreads();
  }
}

template <typename T, int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  const int nwg = (a.lay.Lp / kTileM) * a.lay.H * a.lay.B;
  // the distance attention: no pair factors, no pair output, one zero panel
  if constexpr (D == 128) {
    if (a.z1 == nullptr && a.z2 == nullptr && a.out_pair == nullptr) {
      hipLaunchKernelGGL((ipa_attn_kernel<T, D, true>), dim3(nwg), dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
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
