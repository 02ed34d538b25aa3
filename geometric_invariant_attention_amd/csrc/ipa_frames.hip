// ipa_frames: residue frames from backbone atoms.
//
// "Flash Invariant Point Attention", Figure 1: the C-alpha atom is the centre
// of the residue frame; the vectors from C-alpha to N and to C span it and
// Gram-Schmidt completes it. Per residue (float32):
//   e1 = (C - CA) / |C - CA|
//   e2 = (u / |u|),  u = (N - CA) - (e1 . (N - CA)) e1
//   e3 = e1 x e2
//   rot = [e1 e2 e3] (axes as columns, local -> global), trans = CA.
//
// One residue per thread; the work is a few dozen flops per 48 bytes moved,
// so the kernel is bound by memory traffic, and its loads and stores are
// laid out for it: a workgroup of 256 residues reads its 3 x 256 x 12
// bytes of atoms and writes its 256 x 48 bytes of frames as contiguous
// blocks, staged through LDS, instead of one 12- or 36-byte piece per lane.

#include "ipa_internal.h"

namespace ipa {
namespace {

constexpr int kRes = 256;   // residues per workgroup (one per thread)

__global__ __launch_bounds__(kRes) void frames_kernel(int n, const float* __restrict__ atom_n,
                                                      const float* __restrict__ atom_ca,
                                                      const float* __restrict__ atom_c,
                                                      float* __restrict__ rot, float* __restrict__ trans) {
  __shared__ float in_s[3][kRes * 3];
  __shared__ float rot_s[kRes * 9];
  const int tid = threadIdx.x;
  const long long r0 = (long long)blockIdx.x * kRes;
  const int nr = n - r0 < kRes ? (int)(n - r0) : kRes;   // residues of this block

  // contiguous loads of the block's atoms
  const float* src[3] = {atom_n + r0 * 3, atom_ca + r0 * 3, atom_c + r0 * 3};
#pragma unroll
  for (int a = 0; a < 3; ++a)
    for (int e = tid; e < nr * 3; e += kRes) in_s[a][e] = src[a][e];
  __syncthreads();

  if (tid < nr) {
    float N[3], A[3], Cc[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      N[x] = in_s[0][3 * tid + x];
      A[x] = in_s[1][3 * tid + x];
      Cc[x] = in_s[2][3 * tid + x];
    }
    float e1[3], v2[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      e1[x] = Cc[x] - A[x];
      v2[x] = N[x] - A[x];
    }
    const float inv1 = 1.f / sqrtf(e1[0] * e1[0] + e1[1] * e1[1] + e1[2] * e1[2]);
#pragma unroll
    for (int x = 0; x < 3; ++x) e1[x] *= inv1;
    const float d = e1[0] * v2[0] + e1[1] * v2[1] + e1[2] * v2[2];
    float e2[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) e2[x] = v2[x] - d * e1[x];
    const float inv2 = 1.f / sqrtf(e2[0] * e2[0] + e2[1] * e2[1] + e2[2] * e2[2]);
#pragma unroll
    for (int x = 0; x < 3; ++x) e2[x] *= inv2;
    const float e3[3] = {e1[1] * e2[2] - e1[2] * e2[1], e1[2] * e2[0] - e1[0] * e2[2],
                         e1[0] * e2[1] - e1[1] * e2[0]};
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      rot_s[9 * tid + 3 * x + 0] = e1[x];
      rot_s[9 * tid + 3 * x + 1] = e2[x];
      rot_s[9 * tid + 3 * x + 2] = e3[x];
    }
  }
  __syncthreads();

  // contiguous stores: rotations, then the translations (the C-alpha atoms)
  float* rdst = rot + r0 * 9;
  for (int e = tid; e < nr * 9; e += kRes) rdst[e] = rot_s[e];
  float* tdst = trans + r0 * 3;
  for (int e = tid; e < nr * 3; e += kRes) tdst[e] = in_s[1][e];
}

}  // namespace

hipError_t launch_frames(int n, const float* atom_n, const float* atom_ca, const float* atom_c,
                         float* rot, float* trans, hipStream_t s) {
  const int blocks = (n + kRes - 1) / kRes;
  hipLaunchKernelGGL(frames_kernel, dim3(blocks), dim3(kRes), 0, s, n, atom_n, atom_ca, atom_c, rot, trans);
  return hipGetLastError();
}

}  // namespace ipa
