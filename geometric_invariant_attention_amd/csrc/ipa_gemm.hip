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

// Two values x as bf16 hi + lo halves (nearest even, the hardware's packed
// conversion), x = hi + lo + O(2^-18 x); hi and lo packed two per word.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){x0, x1}, bf16x2));
  const floatx2 r = {x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xFFFF0000u)};
  hi = h;
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
}

// Compiler fence: memory operations stay on their side of it.
__device__ __forceinline__ void fence() { asm volatile("" ::: "memory"); }
// An empty, ordered statement that takes an accumulator tile in place: a
// product whose result passes through it stays between its fences.
__device__ __forceinline__ void pin(floatx16& acc) { asm volatile("" : "+a"(acc)); }

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

// One launch; every operand slice spans fewer than 2^29 elements.
hipError_t launch_one(const Gemm& g, int z, hipStream_t s) {
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

