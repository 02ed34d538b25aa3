// ipa_gemm: batched fp32 GEMM on the fp32 matrix cores, for the plain
// dense products around the attention (the gradient's score tiles, the
// layer's projections and output Linear).

#include "ipa_internal.h"

namespace ipa {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Batched fp32 GEMM on v_mfma_f32_32x32x2f32:
//   C[z](m, n) = sum_k A[z](m, k) B[z](k, n)  (+ C[z](m, n) when acc)
// with A(m, k) at A + z sAb + m am + k ak, B(k, n) at B + z sBb + k bk + n bn,
// C(m, n) at C + z sCb + m cm + n, then + bias[n] and rows m with
// rowmask[m] == 0 set to 0 when those are given. A workgroup of four waves owns a 64 x 64
// tile (a 32 x 32 quadrant per wave); the reduction runs in steps of 32,
// each step's A and B slices staged in LDS with loads along whichever of
// their two strides is 1, the next step's loads in flight in registers
// while this step's 16 products per wave run. Options: the reduction split
// over the grid's z (partials reduced in order by a second kernel), and a
// segmented epilogue that writes column blocks to separate arrays (fp32 or
// bf16).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemm_kernel(Gemm g) {
  constexpr int KS = 32;   // reduction step
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wn = w >> 1, half = lane >> 5, l32 = lane & 31;
  const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 64, z = blockIdx.z;
  // z indexes the batch, or the slice of the reduction when it is split
  const int kbeg = g.kpart ? z * g.kpart : 0;
  const int kend = g.kpart ? (g.K < kbeg + g.kpart ? g.K : kbeg + g.kpart) : g.K;
  const float* A = g.A + (g.kpart ? 0 : (size_t)z * g.sAb);
  const float* B = g.B + (g.kpart ? 0 : (size_t)z * g.sBb);
  __shared__ float As[KS][64 + 4], Bs[KS][64 + 4];
  // element u of this thread's share of the A slice (64 m x KS k) and of
  // the B slice (KS k x 64 n), chosen so that consecutive threads read
  // consecutive addresses
  const bool a_k1 = g.ak == 1, b_n1 = g.bn == 1;
  auto a_mk = [&](int u, int& m, int& k) {
    const int e = tid + 256 * u;
    if (a_k1) { k = e & (KS - 1); m = e / KS; } else { m = e & 63; k = e >> 6; }
  };
  auto b_kn = [&](int u, int& k, int& n) {
    const int e = tid + 256 * u;
    if (b_n1) { n = e & 63; k = e >> 6; } else { k = e & (KS - 1); n = e / KS; }
  };
  constexpr int NU = 64 * KS / 256;
  float ra[NU], rb[NU];
  auto gload = [&](int k0) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      int m, k;
      a_mk(u, m, k);
      const int gm = m0 + m, gk = k0 + k;
      ra[u] = (gm < g.M && gk < kend) ? A[(size_t)gm * g.am + (size_t)gk * g.ak] : 0.f;
      int kb, n;
      b_kn(u, kb, n);
      const int gkb = k0 + kb, gn = n0 + n;
      rb[u] = (gkb < kend && gn < g.N) ? B[(size_t)gkb * g.bk + (size_t)gn * g.bn] : 0.f;
    }
  };
  gload(kbeg);
  floatx16 c = {};
  for (int k0 = kbeg; k0 < kend; k0 += KS) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      int m, k, kb, n;
      a_mk(u, m, k);
      b_kn(u, kb, n);
      As[k][m] = ra[u];
      Bs[kb][n] = rb[u];
    }
    __syncthreads();
    if (k0 + KS < kend) gload(k0 + KS);
    __builtin_amdgcn_sched_barrier(0);   // the next step's loads go out before the products
    float av[KS / 2], bv[KS / 2];
#pragma unroll
    for (int s2 = 0; s2 < KS / 2; ++s2) {
      av[s2] = As[2 * s2 + half][32 * wm + l32];
      bv[s2] = Bs[2 * s2 + half][32 * wn + l32];
    }
#pragma unroll
    for (int s2 = 0; s2 < KS / 2; ++s2) c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s2], bv[s2], c, 0, 0, 0);
    __syncthreads();
  }
  const int n = n0 + 32 * wn + l32;
  if (n >= g.N) return;
  if (g.nseg > 0) {
    // segmented output: column n belongs to block blk of width w, stored
    // [m][w] in fp32 or bf16 (nearest even)
    int blk = 0;
    while (blk + 1 < g.nseg && n >= g.seg_start[blk + 1]) ++blk;
    const int wd = g.seg_start[blk + 1] - g.seg_start[blk], nc = n - g.seg_start[blk];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + 32 * wm + 8 * (e >> 2) + 4 * half + (e & 3);
      if (m >= g.M) continue;
      float v = c[e];
      if (g.bias) v += g.bias[n];
      const size_t at = (size_t)m * wd + nc;
      if (g.seg_bf16) {
        const uint32_t u = __float_as_uint(v);
        reinterpret_cast<uint16_t*>(g.seg_out[blk])[at] = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
      } else {
        reinterpret_cast<float*>(g.seg_out[blk])[at] = v;
      }
    }
    return;
  }
  float* C = g.C + (size_t)z * g.sCb;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int m = m0 + 32 * wm + 8 * (e >> 2) + 4 * half + (e & 3);
    if (m < g.M) {
      float* dst = C + (size_t)m * g.cm + n;
      float v = g.acc ? *dst + c[e] : c[e];
      if (g.bias) v += g.bias[n];
      if (g.rowmask && !g.rowmask[m]) v = 0.f;
      *dst = v;
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

}  // namespace

hipError_t gemm(const Gemm& g, int batch, hipStream_t s) {
  const dim3 grid((g.M + 63) / 64, (g.N + 63) / 64, batch);
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t gemm_splitk(const Gemm& g0, int splits, float* part, hipStream_t s) {
  Gemm g = g0;
  g.kpart = ((g.K + splits - 1) / splits + 31) / 32 * 32;
  const int used = (g.K + g.kpart - 1) / g.kpart;
  g.C = part; g.cm = g.N; g.sCb = (long long)g.M * g.N; g.acc = 0;
  g.bias = nullptr; g.rowmask = nullptr; g.nseg = 0;
  const dim3 grid((g.M + 63) / 64, (g.N + 63) / 64, used);
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, s, g);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const long long total = (long long)g.M * g.N;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     part, used, g.M, g.N, g0.bias, g0.rowmask, g0.C);
  return hipGetLastError();
}

}  // namespace ipa

