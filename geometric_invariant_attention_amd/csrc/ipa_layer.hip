// ipa_layer: the one piece of the full IPA layer that is not a GEMM or the
// attention.
//
// The layer (read from "Flash Invariant Point Attention", TL;DR and
// abstract: per-residue scalar, point and factorised pair features feed
// the attention) maps the single representation s to
//   x = s W_in + b_in = [q | k | v | q_pts | k_pts | v_pts | z1 | z2]
// (one GEMM whose epilogue writes each column block straight into the
// attention's input array in its storage type), runs the attention, gathers
// its four outputs into one row-major matrix (this file) and reads it out
// with
//   y = [o_s | o_pts | o_norm | o_pair] W_out + b_out
// (one GEMM with the reduction split across the grid, the partials added in
// order with the bias, masked rows set to zero).

#include "ipa_internal.h"

namespace ipa {
namespace {

// one thread per element of the concatenated outputs [rows][n_out]
__global__ __launch_bounds__(256) void layer_gather_kernel(LayerGather g) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= g.rows * g.n_out) return;
  const int col = (int)(t % g.n_out);
  const long long row = t / g.n_out;
  int blk = 0;
  while (blk + 1 < 4 && col >= g.start[blk + 1]) ++blk;
  const int w = g.start[blk + 1] - g.start[blk];
  g.cat[t] = g.src[blk][(size_t)row * w + (col - g.start[blk])];
}

}  // namespace

hipError_t launch_layer_gather(const LayerGather& g, hipStream_t s) {
  const long long total = g.rows * g.n_out;
  hipLaunchKernelGGL(layer_gather_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace ipa
