// ipa_dirdist: geometric direction-and-distance attention (ESM3-style).
//
// "Geometric direction-and-distance attention" (BioTorch exercise), section
// "Required behavior". Per batch b, head h, query i, key j, with frames
// (R, t) that map local column vectors to the global frame:
//   a_ijh = ( softplus(ds_h) (R_i qdir_i . R_j kdir_j)
//             - softplus(dd_h) |R_i qpt_i + t_i - R_j kpt_j - t_j| ) / sqrt(3)
//   softmax over allowed keys (both frames valid and the pair mask set),
//   vectors_ihm = R_i^T sum_j A_ijh R_j values_jhm   (rotation only),
//   output_i    = flatten_{h,m,xyz}(vectors_i) W + bias, zero when no head of
//                 query i has an allowed key.
//
// The distance is not squared, so unlike the squared-distance logits of IPA
// and MEET it cannot be folded into a dot product of lifted rows: every
// (i, j, h) needs its own square root. The loop is plain fp32 vector
// arithmetic, bound by the VALU issue rate, and laid out for it:
//   * one query row per lane, 64 rows per wave, all of a wave's key data
//     wave-uniform, so it is read with scalar loads into SGPRs and used as
//     the scalar operand of each vector instruction (no LDS traffic, no
//     VGPRs for keys);
//   * per key and row: 3 FMA for the direction dot, 6 for the squared
//     distance, one square root, one FMA to combine, the online-softmax
//     exponential and 3M FMA for the rotated values;
//   * exponentials in base 2 (log2 e folded into the scales), the running
//     maximum raised lazily (only when a chunk's maximum exceeds it by more
//     than 2^8), so most chunks skip the rescale.
// Stages (one stream, all sizes linear in B * N):
//   dd_lift    per (b, n, h): global directions (the query one pre-scaled),
//              global points, rotated values, key validity -> qbuf, kbuf.
//   dd_attn    per (b, h, 64 queries, key split): 4 waves take 4 key ranges,
//              merge their (m, l, acc) through LDS, write one partial.
//   dd_finish  per (b, i, h): merge the partials, divide, rotate back by
//              R_i^T, write vectors and the row statistics (m, l).
//   dd_readout output = vectors W + bias on fp32 matrix cores (32x32 tiles),
//              zeroed for queries with no allowed key in any head.
//   dd_probs   (only when the attention matrix is requested, O(N^2) bytes)
//              recomputes each logit and writes exp2(s - m) / l.

#include "ipa_internal.h"

namespace ipa {
namespace {

constexpr float kSqrt3Inv = 0.57735026918962576f;
constexpr float kLazy = 8.f;   // a chunk maximum this far above the running one forces a rescale
constexpr int kChunk = 8;      // keys per online-softmax chunk (the key axis is padded to it)

__device__ __forceinline__ float softplus_dev(float x) {
  return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
}

// Per-head factor of the distance, in base-2 logit units.
__device__ __forceinline__ float dist_coef(const float* distance_scale, int h) {
  return softplus_dev(distance_scale[h]) * kSqrt3Inv * kLog2e;
}

__device__ __forceinline__ void rotate(const float* R, float x, float y, float z, float* o) {
  o[0] = R[0] * x + R[1] * y + R[2] * z;
  o[1] = R[3] * x + R[4] * y + R[5] * z;
  o[2] = R[6] * x + R[7] * y + R[8] * z;
}

// ---------------------------------------------------------------------------
// dd_lift
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dd_lift_kernel(DDArgs a) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int H = a.H, M = a.M, Np = a.Np, N = a.N, KW = a.KW;
  const long long total = (long long)a.B * Np * H;
  if (t >= total) return;
  const int h = (int)(t % H);
  const int n = (int)((t / H) % Np);
  const int b = (int)(t / ((long long)H * Np));
  float* qo = a.qbuf + (((size_t)b * H + h) * Np + n) * 8;
  float* ko = a.kbuf + (((size_t)b * H + h) * Np + n) * KW;
  const bool valid = n < N && a.frame_mask[(size_t)b * N + n] != 0;
  if (!valid) {
    // padded keys and invalid frames: no contribution (bias -inf), zero data
    for (int c = 0; c < 8; ++c) qo[c] = 0.f;
    for (int c = 0; c < KW; ++c) ko[c] = 0.f;
    ko[3] = -INFINITY;
    return;
  }
  const size_t bn = (size_t)b * N + n;
  float R[9];
  for (int c = 0; c < 9; ++c) R[c] = a.rot[bn * 9 + c];
  const float* T = a.trans + bn * 3;
  const size_t v3 = (bn * H + h) * 3;
  const float cd = softplus_dev(a.direction_scale[h]) * kSqrt3Inv * kLog2e;
  float o[3];
  rotate(R, a.q_direction[v3], a.q_direction[v3 + 1], a.q_direction[v3 + 2], o);
  qo[0] = cd * o[0]; qo[1] = cd * o[1]; qo[2] = cd * o[2]; qo[3] = 0.f;
  rotate(R, a.q_point[v3], a.q_point[v3 + 1], a.q_point[v3 + 2], o);
  qo[4] = o[0] + T[0]; qo[5] = o[1] + T[1]; qo[6] = o[2] + T[2]; qo[7] = 0.f;
  rotate(R, a.k_direction[v3], a.k_direction[v3 + 1], a.k_direction[v3 + 2], o);
  ko[0] = o[0]; ko[1] = o[1]; ko[2] = o[2]; ko[3] = 0.f;
  rotate(R, a.k_point[v3], a.k_point[v3 + 1], a.k_point[v3 + 2], o);
  ko[4] = o[0] + T[0]; ko[5] = o[1] + T[1]; ko[6] = o[2] + T[2]; ko[7] = 0.f;
  const float* vv = a.values + (bn * H + h) * (size_t)M * 3;
  for (int m = 0; m < M; ++m) {
    rotate(R, vv[3 * m], vv[3 * m + 1], vv[3 * m + 2], o);
    ko[8 + 3 * m] = o[0]; ko[9 + 3 * m] = o[1]; ko[10 + 3 * m] = o[2];
  }
  for (int c = 8 + 3 * M; c < KW; ++c) ko[c] = 0.f;
}

// ---------------------------------------------------------------------------
// dd_attn
// ---------------------------------------------------------------------------
template <int M, bool PM>
__global__ __launch_bounds__(256) void dd_attn_kernel(DDArgs a) {
  constexpr int V = 3 * M;
  constexpr int KW = dd_key_width(M);
  constexpr int PW = dd_part_width(M);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.H, N = a.N, Np = a.Np, S = a.splits;
  const int h = blockIdx.y;
  const int b = blockIdx.z / S, s = blockIdx.z - b * S;
  const int i = blockIdx.x * 64 + lane;
  const int ic = i < N ? i : N - 1;

  // this wave's key range, in chunks
  const int nchunk = Np / kChunk, parts = 4 * S, part = s * 4 + w;
  const int c0 = (int)((long long)nchunk * part / parts);
  const int c1 = (int)((long long)nchunk * (part + 1) / parts);

  const float4* qrow = reinterpret_cast<const float4*>(a.qbuf + (((size_t)b * H + h) * Np + ic) * 8);
  const float4 qd = qrow[0], qp = qrow[1];
  const float cs = dist_coef(a.distance_scale, h);
  const float* __restrict__ kb = a.kbuf + ((size_t)b * H + h) * Np * KW;
  const uint8_t* pmrow = nullptr;
  if constexpr (PM)
    pmrow = a.pair_mask + (size_t)b * a.pm_sb + (size_t)h * a.pm_sh + (size_t)ic * a.pm_si;

  float m_run = -INFINITY, l = 0.f;
  float acc[V];
#pragma unroll
  for (int c = 0; c < V; ++c) acc[c] = 0.f;

  for (int ch = c0; ch < c1; ++ch) {
    const float* __restrict__ kc = kb + (size_t)ch * kChunk * KW;
    float sv[kChunk];
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const float* kk = kc + k * KW;
      const float dot = qd.x * kk[0] + qd.y * kk[1] + qd.z * kk[2];
      const float dx = qp.x - kk[4], dy = qp.y - kk[5], dz = qp.z - kk[6];
      const float d = __builtin_amdgcn_sqrtf(dx * dx + dy * dy + dz * dz);
      float lg = fmaf(-cs, d, dot) + kk[3];
      if constexpr (PM) {
        // padded keys (j >= N) already carry a -inf bias and have no mask entry
        const int j = ch * kChunk + k;
        if (j < N && !pmrow[(size_t)j * a.pm_sj]) lg = -INFINITY;
      }
      sv[k] = lg;
    }
    float cm = sv[0];
#pragma unroll
    for (int k = 1; k < kChunk; ++k) cm = fmaxf(cm, sv[k]);
    if (__builtin_amdgcn_ballot_w64(cm > m_run + kLazy)) {
      const float mn = fmaxf(m_run, cm);
      const float f = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
      l *= f;
#pragma unroll
      for (int c = 0; c < V; ++c) acc[c] *= f;
      m_run = mn;
    }
    const float ms = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const float* kk = kc + k * KW;
      const float p = __builtin_amdgcn_exp2f(sv[k] - ms);
      l += p;
#pragma unroll
      for (int c = 0; c < V; ++c) acc[c] = fmaf(p, kk[8 + c], acc[c]);
    }
  }

  // merge the four waves' key ranges through LDS
  constexpr int LS = V + 3;   // odd row pitch: conflict-free per-lane rows
  __shared__ float red[4][64][LS];
  red[w][lane][0] = m_run;
  red[w][lane][1] = l;
#pragma unroll
  for (int c = 0; c < V; ++c) red[w][lane][2 + c] = acc[c];
  __syncthreads();
  if (w != 0 || i >= N) return;
  float mm = red[0][lane][0];
  for (int u = 1; u < 4; ++u) mm = fmaxf(mm, red[u][lane][0]);
  float fu[4];
  float lt = 0.f;
  for (int u = 0; u < 4; ++u) {
    const float mu = red[u][lane][0];
    fu[u] = mu == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mu - mm);
    lt = fmaf(red[u][lane][1], fu[u], lt);
  }
  float* po = a.part + ((((size_t)s * a.B + b) * N + i) * H + h) * PW;
  po[0] = mm;
  po[1] = lt;
#pragma unroll
  for (int c = 0; c < V; ++c) {
    float v = 0.f;
    for (int u = 0; u < 4; ++u) v = fmaf(red[u][lane][2 + c], fu[u], v);
    po[2 + c] = v;
  }
}

// ---------------------------------------------------------------------------
// dd_finish
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dd_finish_kernel(DDArgs a) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int H = a.H, M = a.M, N = a.N, S = a.splits, PW = a.PW;
  if (t >= (long long)a.B * N * H) return;
  const int h = (int)(t % H);
  const int i = (int)((t / H) % N);
  const int b = (int)(t / ((long long)H * N));
  const size_t bi = (size_t)b * N + i;
  float* vo = a.vectors + (bi * H + h) * (size_t)M * 3;
  float2* st = reinterpret_cast<float2*>(a.stats) + ((size_t)b * H + h) * N + i;
  if (!a.frame_mask[bi]) {
    for (int c = 0; c < 3 * M; ++c) vo[c] = 0.f;
    *st = make_float2(0.f, 0.f);
    return;
  }
  const size_t pstride = (size_t)a.B * N * H * PW;
  const float* p0 = a.part + (bi * H + h) * PW;
  float mm = -INFINITY;
  for (int s = 0; s < S; ++s) mm = fmaxf(mm, p0[s * pstride]);
  float l = 0.f;
  float fs[kMaxSplits];
  for (int s = 0; s < S; ++s) {
    const float ms = p0[s * pstride];
    fs[s] = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - mm);
    l = fmaf(p0[s * pstride + 1], fs[s], l);
  }
  *st = make_float2(mm == -INFINITY ? 0.f : mm, l);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float R[9];
  for (int c = 0; c < 9; ++c) R[c] = a.rot[bi * 9 + c];
  for (int m = 0; m < M; ++m) {
    float g[3];
    for (int x = 0; x < 3; ++x) {
      float v = 0.f;
      for (int s = 0; s < S; ++s) v = fmaf(p0[s * pstride + 2 + 3 * m + x], fs[s], v);
      g[x] = v * inv;
    }
    // R_i^T g: column x of R dotted with g
    for (int x = 0; x < 3; ++x) vo[3 * m + x] = (R[x] * g[0] + R[3 + x] * g[1] + R[6 + x] * g[2]) + 0.f;
  }
}

// ---------------------------------------------------------------------------
// dd_readout: out[r][c] = sum_k vec[r][k] W[k][c] + bias[c] on
// v_mfma_f32_32x32x2f32, one wave per 32 x 32 output tile. Lanes 0-31 feed
// reduction slot 0 and lanes 32-63 slot 1 of each product; the reduction
// index is permuted (slot 0 takes k = 8t..8t+3, slot 1 k = 8t+4..8t+7 over
// four products) so each lane reads its A row as one float4 per four steps.
// ---------------------------------------------------------------------------
typedef float floatx16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(64) void dd_readout_kernel(DDArgs a) {
  const int lane = threadIdx.x;
  const int rows = a.B * a.N, K = 3 * a.H * a.M, Cout = a.Cout;
  const int r0 = blockIdx.x * 32, c0 = blockIdx.y * 32;
  const int half = lane >> 5, li = lane & 31;
  const int ar = r0 + li < rows ? r0 + li : rows - 1;   // A row of this lane
  const int bc = c0 + li;                               // B column of this lane
  const bool bcol = bc < Cout;
  const float* arow = a.vectors + (size_t)ar * K;
  floatx16 c = {};
  for (int k8 = 0; k8 < K; k8 += 8) {
    const int kb = k8 + 4 * half;
    float av[4], bv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = kb + u;
      av[u] = k < K ? arow[k] : 0.f;
      bv[u] = (k < K && bcol) ? a.w_out[(size_t)k * Cout + bc] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[u], bv[u], c, 0, 0, 0);
  }
  // which of this tile's rows have an allowed key in some head
  __shared__ int row_any[32];
  if (lane < 32) {
    int any = 0;
    const int r = r0 + lane;
    if (r < rows) {
      const int b = r / a.N, i = r - b * a.N;
      const float2* st = reinterpret_cast<const float2*>(a.stats);
      for (int h = 0; h < a.H && !any; ++h) any = st[((size_t)b * a.H + h) * a.N + i].y > 0.f;
    }
    row_any[lane] = any;
  }
  __syncthreads();
  if (!bcol) return;
  const float bias = a.b_out ? a.b_out[bc] : 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int rr = 8 * (e >> 2) + 4 * half + (e & 3);
    const int r = r0 + rr;
    if (r < rows) a.output[(size_t)r * Cout + bc] = row_any[rr] ? c[e] + bias : 0.f;
  }
}

// ---------------------------------------------------------------------------
// dd_probs: attention[b][h][i][j] = exp2(s_ij - m_i) / l_i on allowed edges.
// One row i per wave iteration, keys across lanes (coalesced writes).
// ---------------------------------------------------------------------------
constexpr int kProbRows = 4;

__global__ __launch_bounds__(256) void dd_probs_kernel(DDArgs a) {
  const int H = a.H, N = a.N, Np = a.Np, KW = a.KW;
  const int bh = blockIdx.z, b = bh / H, h = bh - b * H;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= N) return;
  const float cs = dist_coef(a.distance_scale, h);
  const float4* kr = reinterpret_cast<const float4*>(a.kbuf + (((size_t)b * H + h) * Np + j) * KW);
  const float4 kd = kr[0], kp = kr[1];
  const float2* st = reinterpret_cast<const float2*>(a.stats) + (size_t)bh * N;
  for (int i0 = blockIdx.y * kProbRows; i0 < N; i0 += gridDim.y * kProbRows)
  for (int r = 0; r < kProbRows; ++r) {
    const int i = i0 + r;
    if (i >= N) break;
    const float4* qr = reinterpret_cast<const float4*>(a.qbuf + (((size_t)bh) * Np + i) * 8);
    const float4 qd = qr[0], qp = qr[1];
    const float2 ml = st[i];
    float p = 0.f;
    if (ml.y > 0.f) {
      const float dot = qd.x * kd.x + qd.y * kd.y + qd.z * kd.z;
      const float dx = qp.x - kp.x, dy = qp.y - kp.y, dz = qp.z - kp.z;
      const float d = __builtin_amdgcn_sqrtf(dx * dx + dy * dy + dz * dz);
      float lg = fmaf(-cs, d, dot) + kd.w;
      if (a.pair_mask &&
          !a.pair_mask[(size_t)b * a.pm_sb + (size_t)h * a.pm_sh + (size_t)i * a.pm_si + (size_t)j * a.pm_sj])
        lg = -INFINITY;
      p = __builtin_amdgcn_exp2f(lg - ml.x) / ml.y;
    }
    a.attention[((size_t)bh * N + i) * N + j] = p + 0.f;
  }
}

template <int M>
hipError_t launch_attn_m(const DDArgs& a, hipStream_t s) {
  const dim3 grid((a.N + 63) / 64, a.H, a.B * a.splits);
  if (a.pair_mask)
    hipLaunchKernelGGL((dd_attn_kernel<M, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((dd_attn_kernel<M, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int dd_splits(int B, int N, int H) {
  // aim for about 3072 waves (3 per SIMD) while keeping >= 64 keys per wave
  const long long base = (long long)((N + 63) / 64) * H * B * 4;
  const int Np = (N + kChunk - 1) / kChunk * kChunk;
  int s = (int)((3072 + base - 1) / base);
  const int cap = Np / (4 * 64);
  if (s > cap) s = cap;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : s;
}

int dd_padded_keys(int N) { return (N + kChunk - 1) / kChunk * kChunk; }

hipError_t launch_dirdist(const DDArgs& a, hipStream_t s) {
  {
    const long long total = (long long)a.B * a.Np * a.H;
    hipLaunchKernelGGL(dd_lift_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  hipError_t e;
  switch (a.M) {
    case 1: e = launch_attn_m<1>(a, s); break;
    case 2: e = launch_attn_m<2>(a, s); break;
    case 3: e = launch_attn_m<3>(a, s); break;
    case 4: e = launch_attn_m<4>(a, s); break;
    case 5: e = launch_attn_m<5>(a, s); break;
    case 6: e = launch_attn_m<6>(a, s); break;
    case 7: e = launch_attn_m<7>(a, s); break;
    case 8: e = launch_attn_m<8>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  {
    const long long total = (long long)a.B * a.N * a.H;
    hipLaunchKernelGGL(dd_finish_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  {
    const dim3 grid((a.B * a.N + 31) / 32, (a.Cout + 31) / 32);
    hipLaunchKernelGGL(dd_readout_kernel, grid, dim3(64), 0, s, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  if (a.attention) {
    const int gy = (a.N + kProbRows - 1) / kProbRows;
    const dim3 grid((a.N + 255) / 256, gy < 65535 ? gy : 65535, a.B * a.H);
    hipLaunchKernelGGL(dd_probs_kernel, grid, dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  return hipSuccess;
}

}  // namespace ipa
