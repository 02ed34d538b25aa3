// ipa_gemm: batched fp32 GEMM on the fp32 matrix cores, for the plain
// dense products around the attention (the gradient's score tiles, the
// layer's projections and output Linear).

#include "ipa_internal.h"

#include <type_traits>

namespace ipa {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Two values x as bf16 hi + lo halves (nearest even, the hardware's packed
// conversion), x = hi + lo + O(2^-18 x); hi and lo packed two per word.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){x0, x1}, bf16x2));
  const floatx2 r = {x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xFFFF0000u)};
  hi = h;
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
}

// Two values x as bf16 hi + mid + lo (each nearest even from the residue
// of the one before), x = hi + mid + lo + O(2^-26 x); packed two per word.
__device__ __forceinline__ void split3(float x0, float x1, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  uint32_t h, r;
  split2(x0, x1, h, r);   // r: bf16 of the residue x - hi, itself rounded
  const floatx2 r1 = {x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xFFFF0000u)};
  const floatx2 r2 = {r1[0] - __uint_as_float(r << 16), r1[1] - __uint_as_float(r & 0xFFFF0000u)};
  hi = h;
  mid = r;
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r2, bf16x2));
}

// Compiler fence: memory operations stay on their side of it.
__device__ __forceinline__ void fence() { asm volatile("" ::: "memory"); }
// An empty, ordered statement that takes an accumulator tile in place: a
// product whose result passes through it stays between its fences.
__device__ __forceinline__ void pin(floatx16& acc) { asm volatile("" : "+a"(acc)); }

// Epilogue shared by the GEMM kernels: wave (wm, wn) writes its TM x TN
// blocks of 32 x 32 (lane (l32, half) holds column l32 and rows
// 8 (e / 4) + 4 half + e % 4 of each block), with the accumulate, bias,
// row-mask and segmented-output options.
template <int TM, int TN>
__device__ __forceinline__ void store_tile(const Gemm& g, floatx16 (&c)[TM][TN], int m0, int n0, int wm, int wn,
                                           int half, int l32, int z) {
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + 32 * (wn * TN + j) + l32;
    if (n >= g.N) continue;
    if (g.nseg > 0) {
      // segmented output: column n belongs to block blk of width wd, stored
      // [m][wd] in fp32 or bf16 (nearest even)
      int blk = 0;
      while (blk + 1 < g.nseg && n >= g.seg_start[blk + 1]) ++blk;
      const int wd = g.seg_start[blk + 1] - g.seg_start[blk], nc = n - g.seg_start[blk];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + 32 * (wm * TM + i) + 8 * (e >> 2) + 4 * half + (e & 3);
          if (m >= g.M) continue;
          float v = c[i][j][e];
          if (g.bias) v += g.bias[n];
          const size_t at = (size_t)m * wd + nc;
          if (g.seg_bf16) {
            const uint32_t u = __float_as_uint(v);
            reinterpret_cast<uint16_t*>(g.seg_out[blk])[at] = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
          } else {
            reinterpret_cast<float*>(g.seg_out[blk])[at] = v;
          }
        }
      continue;
    }
    float* C = g.C + (size_t)z * g.sCb;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 32 * (wm * TM + i) + 8 * (e >> 2) + 4 * half + (e & 3);
        if (m < g.M) {
          float* dst = C + (size_t)m * g.cm + n;
          float v = g.acc ? *dst + c[i][j][e] : c[i][j][e];
          if (g.bias) v += g.bias[n];
          if (g.rowmask && !g.rowmask[m]) v = 0.f;
          *dst = v;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Batched fp32 GEMM on v_mfma_f32_32x32x2f32:
//   C[z](m, n) = sum_k A[z](m, k) B[z](k, n)  (+ C[z](m, n) when acc)
// with A(m, k) at A + z sAb + m am + k ak, B(k, n) at B + z sBb + k bk + n bn,
// C(m, n) at C + z sCb + m cm + n, then + bias[n] and rows m with
// rowmask[m] == 0 set to 0 when those are given.
//
// A workgroup of four waves (2 x 2) owns a (64 TM) x (64 TN) tile, each wave
// TM x TN blocks of 32 x 32. The reduction runs in steps of 32: the step's
// A and B slices are staged in LDS k-contiguous ([m][k] and [n][k], rows
// padded to 36 floats, two buffers), loaded from global memory along
// whichever of their two strides is 1; the next step's loads and LDS writes
// are spread over this step's products. Within a step, product s (0..15) takes reduction
// indices s (lanes 0-31) and 16 + s (lanes 32-63), so that every lane reads
// its operands for the whole step as four 16-byte LDS reads per block.
// Options: the reduction split over the grid's z (partials reduced in order
// by a second kernel), and a segmented epilogue that writes column blocks to
// separate arrays (fp32 or bf16).
// ---------------------------------------------------------------------------
template <int TM, int TN, bool AK1, bool BK1, bool X3, int WGM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gemm_kernel(Gemm g) {
  constexpr int KS = 32;              // reduction step
  constexpr int PK = KS + 4;          // LDS row pitch (floats)
  // split path: an LDS row holds the step's 32 bf16 halves (64 bytes, no
  // padding) as four 16-byte chunks, chunk c of row r in slot c ^ ((r / 4) % 4);
  // 16 consecutive rows at one chunk then cover all 64 banks, for the
  // operand reads and for the staging writes alike
  constexpr int PKB = KS;
  // the four waves as WGM x (4 / WGM): 2 x 2, or 4 x 1 for narrow products
  constexpr int BM = 32 * WGM * TM, BN = 32 * (4 / WGM) * TN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w % WGM, wn = w / WGM, half = lane >> 5, l32 = lane & 31;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN, z = blockIdx.z;
  // z indexes the batch, or the slice of the reduction when it is split
  const int kbeg = g.kpart ? z * g.kpart : 0;
  const int kend = g.kpart ? (g.K < kbeg + g.kpart ? g.K : kbeg + g.kpart) : g.K;
  const float* A = g.A + (g.kpart ? 0 : (size_t)z * g.sAb);
  const float* B = g.B + (g.kpart ? 0 : (size_t)z * g.sBb);
  // two buffers per operand: step s reads buffer s & 1 while the next
  // step's slices are written into the other. fp32 path: [buf][row][k]
  // floats; split path (X3): [buf][hi / lo][row][k] bf16.
  // (the arrays of the path not taken shrink to one row)
  __shared__ __attribute__((aligned(16))) float As[2][X3 ? 1 : BM][PK];
  __shared__ __attribute__((aligned(16))) float Bs[2][X3 ? 1 : BN][PK];
  __shared__ __attribute__((aligned(16))) uint16_t Ah[2][2][X3 ? BM : 1][PKB];
  __shared__ __attribute__((aligned(16))) uint16_t Bh[2][2][X3 ? BN : 1][PKB];
  // Element u of this thread's share of the A slice (BM m x KS k) and of
  // the B slice (KS k x BN n), chosen so that consecutive threads read
  // consecutive addresses: along k when that stride is 1 (AK1 / BK1),
  // along m / n otherwise (then that stride is 1).
  constexpr int NA = BM * KS / 256, NB = BN * KS / 256;
  // Split path, operand with m (n) as the stride-1 dimension (BM, BN of 64
  // or 128): consecutive threads take consecutive rows and each thread
  // stages whole units of eight consecutive reduction indices of its row
  // (element u is index u % 8 of unit u / 8), written as one 16-byte chunk
  // per half once its last element is loaded; single 2-byte writes down a
  // column of rows would hit each bank several times. With k as the
  // stride-1 dimension a thread stages pairs of consecutive reduction
  // indices (element u is index u % 2 of pair u / 2; sixteen threads cover
  // a row), each pair converted together and written as one 4-byte word
  // per half; the fp32 path stages single elements along a row.
  auto a_mk = [&](int u, int& m, int& k) {
    if (AK1 && X3) { k = 2 * (tid & 15) + (u & 1); m = (tid >> 4) + 16 * (u >> 1); }
    else if (AK1) { k = tid & (KS - 1); m = (tid >> 5) + 8 * u; }
    else if (X3) { m = tid % BM; k = 8 * (tid / BM + (256 / BM) * (u >> 3)) + (u & 7); }
    else { m = tid % BM; k = tid / BM + (256 / BM) * u; }
  };
  auto b_kn = [&](int u, int& k, int& n) {
    if (BK1 && X3) { k = 2 * (tid & 15) + (u & 1); n = (tid >> 4) + 16 * (u >> 1); }
    else if (BK1) { k = tid & (KS - 1); n = (tid >> 5) + 8 * u; }
    else if (X3) { n = tid % BN; k = 8 * (tid / BN + (256 / BN) * (u >> 3)) + (u & 7); }
    else { n = tid % BN; k = tid / BN + (256 / BN) * u; }
  };
  static_assert(!X3 || ((BM == 64 || BM == 128) && (BN == 64 || BN == 128)), "split path tiles");
  // LDS element offset of reduction index k in row r of a split-path slice
  auto xsw = [](int r, int k) { return r * PKB + ((((k >> 3) ^ (r >> 2)) & 3) << 3) + (k & 7); };
  // Operands are read through buffer resources over their slices (below
  // 2^29 elements, checked at launch). The per-lane byte offset is that of
  // the first element of a group of elements on one row (one element on
  // the fp32 path; a pair or a unit of eight reduction indices on the split
  // path); the element's place in its group and the step's reduction index
  // go into the scalar offset, which the buffer's range check leaves out.
  // Groups outside the product (rows past M, columns past N) and, in the
  // last step, elements past kend take the per-lane offset kOut, beyond
  // every slice, and load 0.
  constexpr uint32_t kOut = 0x80000000u;
  constexpr int GA = X3 ? (AK1 ? 2 : 8) : 1, GB = X3 ? (BK1 ? 2 : 8) : 1;
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(A), (short)0, (int)(((long long)(g.M - 1) * g.am + (long long)(g.K - 1) * g.ak + 1) * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(B), (short)0, (int)(((long long)(g.K - 1) * g.bk + (long long)(g.N - 1) * g.bn + 1) * 4), 0x00020000);
  uint32_t oa[NA / GA], ob[NB / GB];
#pragma unroll
  for (int v = 0; v < NA / GA; ++v) {
    int m, k;
    a_mk(v * GA, m, k);
    const int mm = m0 + m;
    oa[v] = mm < g.M ? (uint32_t)(AK1 ? mm * (int)g.am + k : mm + k * (int)g.ak) * 4u : kOut;
  }
#pragma unroll
  for (int v = 0; v < NB / GB; ++v) {
    int k, n;
    b_kn(v * GB, k, n);
    const int nn = n0 + n;
    ob[v] = nn < g.N ? (uint32_t)(BK1 ? nn * (int)g.bn + k : nn + k * (int)g.bk) * 4u : kOut;
  }
  const int ak = AK1 ? 1 : (int)g.ak, bk = BK1 ? 1 : (int)g.bk;
  // scalar byte offset of element u (of A, of B) in a step at k0: the
  // group members are consecutive reduction indices
  auto sa = [&](int k0, int u) { return (uint32_t)(k0 + u % GA) * (uint32_t)ak * 4u; };
  auto sb = [&](int k0, int u) { return (uint32_t)(k0 + u % GB) * (uint32_t)bk * 4u; };
  float ra[NA], rb[NB];
  // element u of a full step: A for u < NA, then B
  auto load_one = [&](int k0, int u) {
    if (u < NA) ra[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rA, oa[u / GA], sa(k0, u), 0));
    else rb[u - NA] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rB, ob[(u - NA) / GB], sb(k0, u - NA), 0));
  };
  // eight values as 16 bytes of bf16 hi halves and 16 bytes of lo halves
  auto split8 = [&](const float* x, uint4& hi, uint4& lo) {
    split2(x[0], x[1], hi.x, lo.x);
    split2(x[2], x[3], hi.y, lo.y);
    split2(x[4], x[5], hi.z, lo.z);
    split2(x[6], x[7], hi.w, lo.w);
  };
  auto stage_one = [&](int p, int u) {
    if constexpr (X3) {
      float x[8];
      uint4 hi, lo;
      if (u < NA) {
        int m, k;
        a_mk(u, m, k);
        if (AK1) {
          if (u & 1) {   // the pair is written with its second element
            const int at = xsw(m, k - 1);
            split2(ra[u - 1], ra[u], *reinterpret_cast<uint32_t*>(&Ah[p][0][0][at]),
                   *reinterpret_cast<uint32_t*>(&Ah[p][1][0][at]));
          }
        } else if ((u & 7) == 7) {   // the unit is written with its last element
          const int u0 = u - 7;
          a_mk(u0, m, k);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = ra[u0 + e];
          split8(x, hi, lo);
          *reinterpret_cast<uint4*>(&Ah[p][0][0][xsw(m, k)]) = hi;
          *reinterpret_cast<uint4*>(&Ah[p][1][0][xsw(m, k)]) = lo;
        }
      } else {
        const int ub = u - NA;
        int k, n;
        b_kn(ub, k, n);
        if (BK1) {
          if (ub & 1) {
            const int at = xsw(n, k - 1);
            split2(rb[ub - 1], rb[ub], *reinterpret_cast<uint32_t*>(&Bh[p][0][0][at]),
                   *reinterpret_cast<uint32_t*>(&Bh[p][1][0][at]));
          }
        } else if ((ub & 7) == 7) {
          const int u0 = ub - 7;
          b_kn(u0, k, n);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = rb[u0 + e];
          split8(x, hi, lo);
          *reinterpret_cast<uint4*>(&Bh[p][0][0][xsw(n, k)]) = hi;
          *reinterpret_cast<uint4*>(&Bh[p][1][0][xsw(n, k)]) = lo;
        }
      }
      return;
    }
    if (u < NA) {
      int m, k;
      a_mk(u, m, k);
      As[p][m][k] = ra[u];
    } else {
      int k, n;
      b_kn(u - NA, k, n);
      Bs[p][n][k] = rb[u - NA];
    }
  };
  auto gload = [&](int k0) {
    if (k0 + KS <= kend) {
#pragma unroll
      for (int u = 0; u < NA + NB; ++u) load_one(k0, u);
    } else {
      // last, partial step: indices past kend load 0
#pragma unroll
      for (int u = 0; u < NA; ++u) {
        int m, k;
        a_mk(u, m, k);
        ra[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                              rA, k0 + k < kend ? oa[u / GA] : kOut, sa(k0, u), 0));
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        int k, n;
        b_kn(u, k, n);
        rb[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                              rB, k0 + k < kend ? ob[u / GB] : kOut, sb(k0, u), 0));
      }
    }
  };
  floatx16 c[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) c[i][j] = floatx16{};
  if (kbeg < kend) {
    gload(kbeg);
#pragma unroll
    for (int u = 0; u < NA + NB; ++u) stage_one(0, u);
  }
  __syncthreads();
  // Each step is a fixed sequence of NM products. The operands of quarter
  // q + 1 of the step (four products per block pair) are read from LDS
  // while quarter q runs; the next step's global loads go out one or two per
  // product over the first half and their LDS writes over the second half,
  // so both run in the products' shadow. Memory operations are held in
  // their product step by compiler fences.
  constexpr int NM = 16 * TM * TN, NU = NA + NB, HALF = NM / 2;
  auto read_q = [&](int p, int q, float4 (&av)[TM], float4 (&bv)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      av[i] = *reinterpret_cast<const float4*>(&As[p][32 * (wm * TM + i) + l32][16 * half + 4 * q]);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bv[j] = *reinterpret_cast<const float4*>(&Bs[p][32 * (wn * TN + j) + l32][16 * half + 4 * q]);
  };
  // MODE 0: the next step is a full one (its loads spread over the
  // products); 1: the next step is the partial last one (its loads up
  // front); 2: no next step.
  // split path: per step two reduction substeps of 16, each three bf16
  // products per block pair (hi hi, hi lo, lo hi; the lo lo term is below
  // the split's own error), the products of one kind taken over all block
  // pairs before the next so consecutive products use different
  // accumulators; the operands of substep 1 are read while substep 0 runs
  constexpr int NMX = 2 * 3 * TM * TN, HALFX = NMX / 2;
  auto read_x = [&](int p, int s2, bf16x8 (&ah)[TM], bf16x8 (&al)[TM], bf16x8 (&bh)[TN], bf16x8 (&bl)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = 32 * (wm * TM + i) + l32, at = xsw(r, 16 * s2 + 8 * half);
      ah[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&Ah[p][0][0][at]));
      al[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&Ah[p][1][0][at]));
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = 32 * (wn * TN + j) + l32, at = xsw(r, 16 * s2 + 8 * half);
      bh[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&Bh[p][0][0][at]));
      bl[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&Bh[p][1][0][at]));
    }
  };
  auto iter_x = [&](int k0, int p, auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    if (MODE == 1) gload(k0 + KS);
    bf16x8 ah[2][TM], al[2][TM], bh[2][TN], bl[2][TN];
    read_x(p, 0, ah[0], al[0], bh[0], bl[0]);
    fence();
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      if (s2 == 0) read_x(p, 1, ah[1], al[1], bh[1], bl[1]);
#pragma unroll
      for (int kind = 0; kind < 3; ++kind)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int st = 3 * TM * TN * s2 + TM * TN * kind + TN * i + j;
            const bf16x8 a = kind == 2 ? al[s2][i] : ah[s2][i];
            const bf16x8 b = kind == 1 ? bl[s2][j] : bh[s2][j];
            c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[i][j], 0, 0, 0);
            pin(c[i][j]);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
              if (MODE == 0 && u * HALFX / NU == st) load_one(k0 + KS, u);
              if (MODE != 2 && HALFX + u * HALFX / NU == st) stage_one(p ^ 1, u);
            }
            fence();
          }
    }
    __syncthreads();
  };
  auto iter = [&](int k0, int p, auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    if constexpr (X3) {
      iter_x(k0, p, mode_c);
      return;
    }
    if (MODE == 1) gload(k0 + KS);
    float4 av[2][TM], bv[2][TN];
    read_q(p, 0, av[0], bv[0]);
    fence();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q < 3) read_q(p, q + 1, av[(q + 1) & 1], bv[(q + 1) & 1]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int st = 16 * TM * TN / 4 * q + TM * TN * e + TN * i + j;
            c[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[q & 1][i][e], bv[q & 1][j][e], c[i][j], 0, 0, 0);
            pin(c[i][j]);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
              if (MODE == 0 && u * HALF / NU == st) load_one(k0 + KS, u);
              if (MODE != 2 && HALF + u * HALF / NU == st) stage_one(p ^ 1, u);
            }
            fence();
          }
    }
    __syncthreads();
  };
  int k0 = kbeg, p = 0;
  for (; k0 + 2 * KS <= kend; k0 += KS, p ^= 1) iter(k0, p, std::integral_constant<int, 0>{});
  if (k0 + KS < kend) {
    iter(k0, p, std::integral_constant<int, 1>{});
    k0 += KS;
    p ^= 1;
  }
  if (k0 < kend) iter(k0, p, std::integral_constant<int, 2>{});
  store_tile<TM, TN>(g, c, m0, n0, wm, wn, half, l32, z);
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector
// memory operations of the wave are outstanding, the other counters free
constexpr int vm_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Workgroup barrier for LDS traffic only: the wave's LDS operations
// complete, then s_barrier; the memory clobber keeps the compiler from
// moving memory operations across it. Unlike __syncthreads() it adds no
// wait for outstanding global loads.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// Split-path GEMM with the reduction steps copied global -> LDS ahead of
// their use, for operands whose rows along the stride-1 dimension are
// 16-byte aligned, K a multiple of 4, no split reduction. The split path's
// steps are short (twelve bf16 products per wave per 32 reduction indices),
// too short to hide a global load issued one step ahead; here each step's
// raw fp32 slices are copied by direct-to-LDS buffer loads NS - 1 steps
// ahead, into NS stage arrays (separate LDS arrays, so that the compiler
// can see that a read of one stage never waits for copies into another),
// and the bf16 hi / lo halves are formed when a wave reads its operands.
//
// A stage holds the step's A slice, then its B slice. An operand with k as
// its stride-1 dimension (AK1 / BK1) is held as rows of 32 k (8 chunks of
// 16 bytes), chunk c of row r in slot c ^ (r % 8); one wave-wide copy fills
// 8 rows (lane l: row l / 8, slot l % 8) and a fragment (8 consecutive k of
// one row) is two 16-byte reads. An operand with m (n) as its stride-1
// dimension is held as 32 rows of k, each the tile's R = BM (BN) values,
// element x of row k at x ^ (32 ((k / 8) % 2)) (chunk-granular, so that
// the two lane halves of a fragment read, k and k + 8 apart, fall on
// different banks); one copy fills 256 / R rows (lane l: row l / (R / 4),
// slot l % (R / 4)) and a fragment is eight 4-byte reads. Rows past M or N
// (chunks past M or N: those extents are then multiples of 4) and, in the
// last step, chunks or rows past K take an offset beyond the resource's
// range and read 0; past-K values are never read otherwise (K is a
// multiple of 4).
// The steps end in a plain barrier after each wave's counted wait for its
// own copies of the next step: __syncthreads() would add a fence that
// waits for every outstanding copy, the ones issued ahead included.
// ---------------------------------------------------------------------------
template <int TM, int TN, int NS, bool AK1, bool BK1, bool X6>
__global__ __launch_bounds__(256) void gemm_x3k_kernel(Gemm g) {
  constexpr int KS = 32;
  constexpr int BM = 64 * TM, BN = 64 * TN;
  // 1 KB copies per stage and wave: OPA of A, OPB of B
  constexpr int OPA = BM / 32, OPB = BN / 32, OPW = OPA + OPB;
  constexpr uint32_t kOut = 0x80000000u;
  constexpr int SA = BM * KS, SF = (BM + BN) * KS;    // floats: A part, whole stage
  constexpr int kWaitAhead = vm_wait(OPW * (NS - 2));
  __shared__ __attribute__((aligned(16))) float S0[SF];
  __shared__ __attribute__((aligned(16))) float S1[SF];
  __shared__ __attribute__((aligned(16))) float S2[NS > 2 ? SF : 4];
  __shared__ __attribute__((aligned(16))) float S3[NS > 3 ? SF : 4];
  __shared__ __attribute__((aligned(16))) float S4[NS > 4 ? SF : 4];
  static_assert(NS >= 2 && NS <= 5, "stages");
  // (the wave index made visibly uniform: the copies' LDS addresses are)
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w & 1, wn = w >> 1, half = lane >> 5, l32 = lane & 31;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN, z = blockIdx.z;
  const float* A = g.A + (size_t)z * g.sAb;
  const float* B = g.B + (size_t)z * g.sBb;
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(A), (short)0, (int)(((long long)(g.M - 1) * g.am + (long long)(g.K - 1) * g.ak + 1) * 4),
      0x00020000);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(B), (short)0, (int)(((long long)(g.N - 1) * g.bn + (long long)(g.K - 1) * g.bk + 1) * 4),
      0x00020000);
  // Per copy q of this wave: the per-lane byte offset at reduction index 0
  // (kOut outside the product), the k of the lane's row (rows of k only,
  // else -1: then the chunk's k decides) and the LDS row of the copy.
  // x0, X: the tile's first m (n) and the extent; rs: stride of the row
  // dimension (k-contiguous), ks: stride of k (mn-contiguous).
  struct Copy { uint32_t vo; int krow, kchunk; };
  auto geom = [&](bool k1, int R, int q, int x0, int X, int rs, int ks) -> Copy {
    Copy c;
    if (k1) {
      const int r = 8 * (w + 4 * q) + (lane >> 3), ch = (lane & 7) ^ (lane >> 3);
      c.vo = x0 + r < X ? (uint32_t)((x0 + r) * rs + 4 * ch) * 4u : kOut;
      c.krow = -1;
      c.kchunk = 4 * ch;
    } else {
      const int cpr = R / 4, kr = (256 / R) * (w + 4 * q) + lane / cpr;
      const int ch = (lane % cpr) ^ (8 * ((kr >> 3) & 1));
      c.vo = x0 + 4 * ch < X ? (uint32_t)(kr * ks + x0 + 4 * ch) * 4u : kOut;
      c.krow = kr;
      c.kchunk = 0;
    }
    return c;
  };
  uint32_t vo[OPW];
  int kq[OPW];   // reduction index (within a step) below which the lane's chunk or row lies
#pragma unroll
  for (int q = 0; q < OPA; ++q) {
    const Copy c = geom(AK1, BM, q, m0, g.M, (int)g.am, (int)g.ak);
    vo[q] = c.vo;
    kq[q] = AK1 ? c.kchunk : c.krow;
  }
#pragma unroll
  for (int q = 0; q < OPB; ++q) {
    const Copy c = geom(BK1, BN, q, n0, g.N, (int)g.bn, (int)g.bk);
    vo[OPA + q] = c.vo;
    kq[OPA + q] = BK1 ? c.kchunk : c.krow;
  }
  const uint32_t aks = AK1 ? 4u : (uint32_t)g.ak * 4u, bks = BK1 ? 4u : (uint32_t)g.bk * 4u;
  auto stage_ptr = [&](auto sc) -> float* {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return S0;
    else if constexpr (S == 1) return S1;
    else if constexpr (S == 2) return S2;
    else if constexpr (S == 3) return S3;
    else return S4;
  };
  // copies of the step at k0 into stage S. In the last, partial step
  // (TAIL) the step's offset moves into the per-lane offset, so that the
  // range check sees it, and chunks or rows past K take kOut (selects, no
  // branches: the compiler's wait tracking then keeps the stages apart).
  auto issue_t = [&](int k0, auto sc, auto tc) {
    constexpr bool tail = decltype(tc)::value;
    float* st = stage_ptr(sc);
#pragma unroll
    for (int q = 0; q < OPW; ++q) {
      const bool isA = q < OPA;
      const uint32_t step = (uint32_t)k0 * (isA ? aks : bks);
      // (kOut + step keeps bit 31 set: still beyond every range)
      const uint32_t past = (tail && k0 + kq[q] >= g.K) ? kOut : 0u;
      const uint32_t v = tail ? ((vo[q] + step) | past) : vo[q];
      const int qq = isA ? q : q - OPA;
      const int at = isA ? (AK1 ? 8 * (w + 4 * qq) * KS : (256 / BM) * (w + 4 * qq) * BM)
                         : SA + (BK1 ? 8 * (w + 4 * qq) * KS : (256 / BN) * (w + 4 * qq) * BN);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isA ? rA : rB, (__attribute__((address_space(3))) void*)(st + at), 16,
                                               v, tail ? 0u : step, 0, 0);
    }
  };
  auto issue = [&](int k0, auto sc) {
    if (k0 + KS > g.K) issue_t(k0, sc, std::true_type{});
    else issue_t(k0, sc, std::false_type{});
  };
  floatx16 c[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) c[i][j] = floatx16{};
  // fragment of tile row (column) r of an operand part p: reduction indices
  // 16 s2 + 8 half + 0..7 of the step, split into bf16 hi and lo (X6: hi,
  // mid and lo, the residue after hi split again)
  auto frag = [&](const float* p, bool k1, int R, int r, int s2, bf16x8& hi, bf16x8& mid, bf16x8& lo) {
    float x[8];
    if (k1) {
      const int c0 = 4 * s2 + 2 * half, sw = r & 7;
      // whole 16-byte reads (an empty asm takes each as one value): a read
      // split into single floats and merged again later loses the alias
      // scope that keeps it from waiting for the copies into other stages
      u32x4 u0 = *reinterpret_cast<const u32x4*>(p + r * KS + 4 * (c0 ^ sw));
      u32x4 u1 = *reinterpret_cast<const u32x4*>(p + r * KS + 4 * ((c0 + 1) ^ sw));
      asm("" : "+v"(u0));
      asm("" : "+v"(u1));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = __uint_as_float(u0[e]);
        x[4 + e] = __uint_as_float(u1[e]);
      }
    } else {
      const float* col = p + (16 * s2 + 8 * half) * R + (r ^ (32 * half));
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = col[e * R];
    }
    uint4 h, l;
    if constexpr (X6) {
      uint4 m;
      split3(x[0], x[1], h.x, m.x, l.x);
      split3(x[2], x[3], h.y, m.y, l.y);
      split3(x[4], x[5], h.z, m.z, l.z);
      split3(x[6], x[7], h.w, m.w, l.w);
      mid = __builtin_bit_cast(bf16x8, m);
    } else {
      split2(x[0], x[1], h.x, l.x);
      split2(x[2], x[3], h.y, l.y);
      split2(x[4], x[5], h.z, l.z);
      split2(x[6], x[7], h.w, l.w);
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
  };
  // step at k0 on stage S; the copies of step k0 + (NS - 1) KS go into the
  // stage that step k0 - KS read (every wave has passed the barrier after
  // it). STEADY: that step exists and is a full one (no tail code, so that
  // nothing merges in front of the stage reads).
  auto step = [&](int k0, auto sc, auto steady_c) {
    constexpr int S = decltype(sc)::value;
    constexpr bool steady = decltype(steady_c)::value;
    using Ahead = std::integral_constant<int, (S + NS - 1) % NS>;
    const bool more = steady || k0 + (NS - 1) * KS < g.K;
    if constexpr (steady) issue_t(k0 + (NS - 1) * KS, Ahead{}, std::false_type{});
    else if (more) issue(k0 + (NS - 1) * KS, Ahead{});
    const float* st = stage_ptr(sc);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 ah[TM], am[TM], al[TM], bh[TN], bm[TN], bl[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) frag(st, AK1, BM, 32 * (wm * TM + i) + l32, s2, ah[i], am[i], al[i]);
#pragma unroll
      for (int j = 0; j < TN; ++j) frag(st + SA, BK1, BN, 32 * (wn * TN + j) + l32, s2, bh[j], bm[j], bl[j]);
      // the products as (part of A, part of B): split path hi hi, hi lo,
      // lo hi (0 hi, 1 lo); X6 hi hi, hi mid, mid hi, hi lo, lo hi, mid mid
      // (0 hi, 1 mid, 2 lo), the terms left out below 2^-24 relative
      constexpr int NK = X6 ? 6 : 3;
      constexpr int ka3[3] = {0, 0, 1}, kb3[3] = {0, 1, 0};
      constexpr int ka6[6] = {0, 0, 1, 0, 2, 1}, kb6[6] = {0, 1, 0, 2, 0, 1};
#pragma unroll
      for (int kind = 0; kind < NK; ++kind)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int pa = X6 ? ka6[kind] : ka3[kind], pb = X6 ? kb6[kind] : kb3[kind];
            const bf16x8 a = X6 ? (pa == 2 ? al[i] : pa == 1 ? am[i] : ah[i]) : (pa == 1 ? al[i] : ah[i]);
            const bf16x8 b = X6 ? (pb == 2 ? bl[j] : pb == 1 ? bm[j] : bh[j]) : (pb == 1 ? bl[j] : bh[j]);
            c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[i][j], 0, 0, 0);
          }
    }
    // this wave's copies of the next step have landed once no more than
    // the copies issued after them (NS - 2 steps' worth, when all exist)
    // are outstanding; the barrier then makes every wave's copies visible
    // and closes the reads of stage S
    if (more) __builtin_amdgcn_s_waitcnt(kWaitAhead);
    else __builtin_amdgcn_s_waitcnt(vm_wait(0));
    lds_barrier();
  };
  // prologue: steps 0 .. NS - 2 into stages 0 .. NS - 2
  issue(0, std::integral_constant<int, 0>{});
  if constexpr (NS > 2)
    if (KS < g.K) issue(KS, std::integral_constant<int, 1>{});
  if constexpr (NS > 3)
    if (2 * KS < g.K) issue(2 * KS, std::integral_constant<int, 2>{});
  if constexpr (NS > 4)
    if (3 * KS < g.K) issue(3 * KS, std::integral_constant<int, 3>{});
  if ((NS - 2) * KS < g.K) __builtin_amdgcn_s_waitcnt(kWaitAhead);
  else __builtin_amdgcn_s_waitcnt(vm_wait(0));
  lds_barrier();
  using Steady = std::true_type;
  using Any = std::false_type;
  int k0 = 0;
  // steady state: the step issued ahead is a full one
  for (;;) {
    if (k0 + NS * KS > g.K) break;
    step(k0, std::integral_constant<int, 0>{}, Steady{});
    k0 += KS;
    if (k0 + NS * KS > g.K) break;
    step(k0, std::integral_constant<int, 1>{}, Steady{});
    k0 += KS;
    if constexpr (NS > 2) {
      if (k0 + NS * KS > g.K) break;
      step(k0, std::integral_constant<int, 2>{}, Steady{});
      k0 += KS;
    }
    if constexpr (NS > 3) {
      if (k0 + NS * KS > g.K) break;
      step(k0, std::integral_constant<int, 3>{}, Steady{});
      k0 += KS;
    }
    if constexpr (NS > 4) {
      if (k0 + NS * KS > g.K) break;
      step(k0, std::integral_constant<int, 4>{}, Steady{});
      k0 += KS;
    }
  }
  // the last steps (at most NS), the stages continuing the rotation
  for (; k0 < g.K; k0 += KS) {
    const int st = (k0 / KS) % NS;
    if (st == 0) step(k0, std::integral_constant<int, 0>{}, Any{});
    else if (st == 1) step(k0, std::integral_constant<int, 1>{}, Any{});
    else if (NS > 2 && st == 2) step(k0, std::integral_constant<int, (NS > 2 ? 2 : 0)>{}, Any{});
    else if (NS > 3 && st == 3) step(k0, std::integral_constant<int, (NS > 3 ? 3 : 0)>{}, Any{});
    else if (NS > 4) step(k0, std::integral_constant<int, (NS > 4 ? 4 : 0)>{}, Any{});
  }
  store_tile<TM, TN>(g, c, m0, n0, wm, wn, half, l32, z);
}

// out(m, n) = sum_z part[z](m, n) (+ bias[n]), rows with rowmask[m] == 0
// set to 0; the slices are added in order
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* part, int splits, int M, int N,
                                                            const float* bias, const uint8_t* rowmask,
                                                            float* out) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (long long)M * N) return;
  const int n = (int)(t % N), m = (int)(t / N);
  float v = 0.f;
  for (int z = 0; z < splits; ++z) v += part[(size_t)z * M * N + t];
  if (bias) v += bias[n];
  if (rowmask && !rowmask[m]) v = 0.f;
  out[t] = v;
}

// Tile shape for an M x N product over `z` grid slices: the shape with the
// least work on the busiest compute unit, taking workgroups as dealt out
// evenly (ceil(workgroups / 256) per unit), each costing its padded tile
// area over the shape's relative speed (larger tiles reuse each staged
// operand more often; speeds and the single-workgroup penalty measured on
// the gradient's and the layer's products).
struct TileShape { int tm, tn; };
TileShape pick_tile(int M, int N, int z, bool x3) {
  const TileShape cand[4] = {{2, 2}, {2, 1}, {1, 2}, {1, 1}};
  const double speed[4] = {1.0, 0.85, 0.85, 0.65};
  int best = 3;
  double best_cost = 0.0;
  // (the split path's LDS holds two bf16 halves per element: 128 x 64 at most)
  for (int c = x3 ? 1 : 0; c < 4; ++c) {
    const long long gm = (M + 64 * cand[c].tm - 1) / (64 * cand[c].tm), gn = (N + 64 * cand[c].tn - 1) / (64 * cand[c].tn);
    const long long per_cu = (gm * gn * z + 255) / 256;
    // a unit left with one workgroup runs one wave per SIMD, which hides
    // less of the load and LDS latency
    const double cost = (double)per_cu * (64.0 * cand[c].tm) * (64.0 * cand[c].tn) / speed[c] * (per_cu == 1 ? 1.4 : 1.0);
    if (c == (x3 ? 1 : 0) || cost < best_cost) { best = c; best_cost = cost; }
  }
  return cand[best];
}

template <int TM, int TN, bool X3, int WGM = 2>
void launch_layout(const Gemm& g, dim3 grid, hipStream_t s) {
  const bool ak1 = g.ak == 1, bk1 = g.bk == 1;
  if (ak1 && bk1) hipLaunchKernelGGL((gemm_kernel<TM, TN, true, true, X3, WGM>), grid, dim3(256), 0, s, g);
  else if (ak1) hipLaunchKernelGGL((gemm_kernel<TM, TN, true, false, X3, WGM>), grid, dim3(256), 0, s, g);
  else if (bk1) hipLaunchKernelGGL((gemm_kernel<TM, TN, false, true, X3, WGM>), grid, dim3(256), 0, s, g);
  else hipLaunchKernelGGL((gemm_kernel<TM, TN, false, false, X3, WGM>), grid, dim3(256), 0, s, g);
}
template <int TM, int TN>
void launch_shape(const Gemm& g, dim3 grid, hipStream_t s) {
  if constexpr (TM == 2 && TN == 2) launch_layout<2, 2, false>(g, grid, s);   // split path: 128 x 64 at most
  else if (g.x3) launch_layout<TM, TN, true>(g, grid, s);
  else launch_layout<TM, TN, false>(g, grid, s);
}

// Stages of the direct-to-LDS split-path kernel (copies run NS - 1 steps
// ahead; 3 x 24 KB of LDS, two workgroups per compute unit).
constexpr int kX3Stages = 3;

// Tile of the direct-to-LDS kernel for an M x N product over z slices:
// 128 x 64, 64 x 128 or 64 x 64, the one that finishes first when
// workgroups run in rounds of c per compute unit (c = 2 for the two larger
// tiles, 3 for the smallest, by LDS), each round costing c tile areas over
// the shape's speed (the 64 x 64 tile splits a third more operand values
// per product).
TileShape pick_tile_x3k(int M, int N, int z) {
  const TileShape cand[3] = {{2, 1}, {1, 2}, {1, 1}};
  const int conc[3] = {2, 2, 3};
  const double speed[3] = {1.0, 1.0, 0.75};
  int best = 0;
  double best_cost = 0.0;
  for (int c = 0; c < 3; ++c) {
    const long long gm = (M + 64 * cand[c].tm - 1) / (64 * cand[c].tm), gn = (N + 64 * cand[c].tn - 1) / (64 * cand[c].tn);
    const long long rounds = (gm * gn * z + 256LL * conc[c] - 1) / (256LL * conc[c]);
    const double cost = (double)rounds * conc[c] * (64.0 * cand[c].tm) * (64.0 * cand[c].tn) / speed[c];
    if (c == 0 || cost < best_cost) { best = c; best_cost = cost; }
  }
  return cand[best];
}

template <int TM, int TN, bool AK1, bool BK1, bool X6>
void launch_x3k_shape(const Gemm& g, int z, hipStream_t s) {
  hipLaunchKernelGGL((gemm_x3k_kernel<TM, TN, kX3Stages, AK1, BK1, X6>),
                     dim3((g.M + 64 * TM - 1) / (64 * TM), (g.N + 64 * TN - 1) / (64 * TN), z), dim3(256), 0, s, g);
}

template <bool AK1, bool BK1, bool X6>
void launch_x3k(const Gemm& g, int z, hipStream_t s) {
  const TileShape t = pick_tile_x3k(g.M, g.N, z);
  if (t.tm == 2) launch_x3k_shape<2, 1, AK1, BK1, X6>(g, z, s);
  else if (t.tn == 2) launch_x3k_shape<1, 2, AK1, BK1, X6>(g, z, s);
  else launch_x3k_shape<1, 1, AK1, BK1, X6>(g, z, s);
}

template <bool X6>
void launch_x3k_layout(const Gemm& g, int z, hipStream_t s) {
  const bool ak1 = g.ak == 1, bk1 = g.bk == 1;
  if (ak1 && bk1) launch_x3k<true, true, X6>(g, z, s);
  else if (ak1) launch_x3k<true, false, X6>(g, z, s);
  else if (bk1) launch_x3k<false, true, X6>(g, z, s);
  else launch_x3k<false, false, X6>(g, z, s);
}

// One launch; every operand slice spans fewer than 2^29 elements.
hipError_t launch_one(const Gemm& g, int z, hipStream_t s) {
  // split path whose operands suit the copies to LDS: rows along the
  // stride-1 dimension 16-byte aligned, the extents along it (K for a
  // k-contiguous operand, M or N otherwise) multiples of 4
  // (x6: the three-way split there, for N wider than the narrow tiles;
  // otherwise fp32 products below)
  const bool ak1 = g.ak == 1, bk1 = g.bk == 1;
  const bool fits = g.kpart == 0 && g.K % 4 == 0 && (ak1 ? g.am % 4 == 0 : (g.ak % 4 == 0 && g.M % 4 == 0)) &&
                    (bk1 ? g.bn % 4 == 0 : (g.bk % 4 == 0 && g.N % 4 == 0)) && g.sAb % 4 == 0 && g.sBb % 4 == 0 &&
                    ((uintptr_t)g.A & 15) == 0 && ((uintptr_t)g.B & 15) == 0;
  if (fits && g.x3) {
    launch_x3k_layout<false>(g, z, s);
    return hipGetLastError();
  }
  if (fits && g.x6 && g.N > 32) {
    launch_x3k_layout<true>(g, z, s);
    return hipGetLastError();
  }
  if (g.N <= 32 && !g.x3) {
    // narrow product: 128 x 32 tiles (the four waves stacked along M), a
    // quarter of the padding of a 64-wide tile
    launch_layout<1, 1, false, 4>(g, dim3((g.M + 127) / 128, (g.N + 31) / 32, z), s);
    return hipGetLastError();
  }
  const TileShape t = pick_tile(g.M, g.N, z, g.x3 != 0);
  const dim3 grid((g.M + 64 * t.tm - 1) / (64 * t.tm), (g.N + 64 * t.tn - 1) / (64 * t.tn), z);
  if (t.tm == 2 && t.tn == 2) launch_shape<2, 2>(g, grid, s);
  else if (t.tm == 2) launch_shape<2, 1>(g, grid, s);
  else if (t.tn == 2) launch_shape<1, 2>(g, grid, s);
  else launch_shape<1, 1>(g, grid, s);
  return hipGetLastError();
}

// The kernel addresses each operand slice through a buffer resource with
// 32-bit byte offsets, so a launch's slices must span fewer than 2^29
// elements. B must on its own; A is split along M into launches that do
// (the rows of one launch are a contiguous run of A, C, the row mask and
// the segmented outputs).
hipError_t launch_gemm(const Gemm& g, int z, hipStream_t s) {
  if (!(g.ak == 1 || g.am == 1) || !(g.bk == 1 || g.bn == 1)) return hipErrorInvalidValue;
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  constexpr double kMaxExt = 536870912.0;   // 2^29
  if ((double)(g.K - 1) * g.bk + (double)(g.N - 1) * g.bn + 1.0 >= kMaxExt) return hipErrorInvalidValue;
  const double krun = (double)(g.K - 1) * g.ak + 1.0;
  if ((double)(g.M - 1) * g.am + krun < kMaxExt) return launch_one(g, z, s);
  // rows per launch: a multiple of 128 (whole tiles of every shape)
  const long long rows = (long long)((kMaxExt - 1.0 - krun) / (double)g.am) / 128 * 128;
  if (rows < 128) return hipErrorInvalidValue;
  for (long long m0 = 0; m0 < g.M; m0 += rows) {
    Gemm c = g;
    c.M = (int)(g.M - m0 < rows ? g.M - m0 : rows);
    c.A = g.A + m0 * g.am;
    if (g.C) c.C = g.C + m0 * g.cm;
    if (g.rowmask) c.rowmask = g.rowmask + m0;
    for (int b = 0; b < g.nseg; ++b) {
      const long long wd = g.seg_start[b + 1] - g.seg_start[b];
      c.seg_out[b] = static_cast<unsigned char*>(g.seg_out[b]) + m0 * wd * (g.seg_bf16 ? 2 : 4);
    }
    const hipError_t e = launch_one(c, z, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t gemm(const Gemm& g, int batch, hipStream_t s) { return launch_gemm(g, batch, s); }

hipError_t gemm_splitk(const Gemm& g0, int splits, float* part, hipStream_t s) {
  Gemm g = g0;
  g.kpart = ((g.K + splits - 1) / splits + 31) / 32 * 32;
  const int used = (g.K + g.kpart - 1) / g.kpart;
  g.C = part; g.cm = g.N; g.sCb = (long long)g.M * g.N; g.acc = 0;
  g.bias = nullptr; g.rowmask = nullptr; g.nseg = 0;
  if (launch_gemm(g, used, s) != hipSuccess) return hipErrorLaunchFailure;
  const long long total = (long long)g.M * g.N;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     part, used, g.M, g.N, g0.bias, g0.rowmask, g0.C);
  return hipGetLastError();
}

}  // namespace ipa

