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
// tile (a 32 x 32 quadrant per wave); the reduction runs in steps of 16,
// each step's A and B slices staged in LDS with loads along whichever of
// their two strides is 1, the next step's loads in flight in registers
// while this step's 8 products per wave run.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemm_kernel(Gemm g) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wn = w >> 1, half = lane >> 5, l32 = lane & 31;
  const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 64, z = blockIdx.z;
  const float* A = g.A + (size_t)z * g.sAb;
  const float* B = g.B + (size_t)z * g.sBb;
  __shared__ float As[16][64 + 4], Bs[16][64 + 4];
  // element u of this thread's share of the A slice (64 m x 16 k) and of
  // the B slice (16 k x 64 n), chosen so that consecutive threads read
  // consecutive addresses
  const bool a_k1 = g.ak == 1, b_n1 = g.bn == 1;
  auto a_mk = [&](int u, int& m, int& k) {
    const int e = tid + 256 * u;
    if (a_k1) { k = e & 15; m = e >> 4; } else { m = e & 63; k = e >> 6; }
  };
  auto b_kn = [&](int u, int& k, int& n) {
    const int e = tid + 256 * u;
    if (b_n1) { n = e & 63; k = e >> 6; } else { k = e & 15; n = e >> 4; }
  };
  float ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int m, k;
      a_mk(u, m, k);
      const int gm = m0 + m, gk = k0 + k;
      ra[u] = (gm < g.M && gk < g.K) ? A[(size_t)gm * g.am + (size_t)gk * g.ak] : 0.f;
      int kb, n;
      b_kn(u, kb, n);
      const int gkb = k0 + kb, gn = n0 + n;
      rb[u] = (gkb < g.K && gn < g.N) ? B[(size_t)gkb * g.bk + (size_t)gn * g.bn] : 0.f;
    }
  };
  gload(0);
  floatx16 c = {};
  for (int k0 = 0; k0 < g.K; k0 += 16) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int m, k, kb, n;
      a_mk(u, m, k);
      b_kn(u, kb, n);
      As[k][m] = ra[u];
      Bs[kb][n] = rb[u];
    }
    __syncthreads();
    if (k0 + 16 < g.K) gload(k0 + 16);
    __builtin_amdgcn_sched_barrier(0);   // the next step's loads go out before the products
    float av[8], bv[8];
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) {
      av[s2] = As[2 * s2 + half][32 * wm + l32];
      bv[s2] = Bs[2 * s2 + half][32 * wn + l32];
    }
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s2], bv[s2], c, 0, 0, 0);
    __syncthreads();
  }
  float* C = g.C + (size_t)z * g.sCb;
  const int n = n0 + 32 * wn + l32;
  if (n >= g.N) return;
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

}  // namespace

hipError_t gemm(const Gemm& g, int batch, hipStream_t s) {
  const dim3 grid((g.M + 63) / 64, (g.N + 63) / 64, batch);
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace ipa

