// ipa_layer: the pieces of the full IPA layer that are not GEMMs.
//
// The layer (read from "Flash Invariant Point Attention", TL;DR and
// abstract: per-residue scalar, point and factorised pair features feed
// the attention) maps the single representation s to
//   x = s W_in + b_in = [q | k | v | q_pts | k_pts | v_pts | z1 | z2]
// (one GEMM), splits x into the attention's input arrays in its storage
// type (this file), runs the attention, and reads its outputs out with
//   y = [o_s | o_pts | o_norm | o_pair] W_out + b_out
// (four accumulating GEMMs, the last adding the bias and zeroing masked
// rows).

#include "ipa_internal.h"

namespace ipa {
namespace {

__device__ __forceinline__ uint16_t to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// one thread per element of x: its column picks the block, the block's
// array gets the element at the same row
__global__ __launch_bounds__(256) void layer_split_kernel(LayerSplit a) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (long long)a.rows * a.n_in) return;
  const int col = (int)(t % a.n_in);
  const long long row = t / a.n_in;
  int blk = 0;
  while (blk + 1 < kLayerBlocks && col >= a.start[blk + 1]) ++blk;
  const int w = a.start[blk + 1] - a.start[blk];
  const size_t at = (size_t)row * w + (col - a.start[blk]);
  const float v = a.x[t];
  if (a.bf16)
    reinterpret_cast<uint16_t*>(a.out[blk])[at] = to_bf16_rne(v);
  else
    reinterpret_cast<float*>(a.out[blk])[at] = v;
}

}  // namespace

hipError_t launch_layer_split(const LayerSplit& a, hipStream_t s) {
  const long long total = (long long)a.rows * a.n_in;
  hipLaunchKernelGGL(layer_split_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ipa
