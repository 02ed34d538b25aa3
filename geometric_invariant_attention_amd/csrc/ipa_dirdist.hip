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
// (i, j, h) needs its own square root. The logits are fp32 vector work, the
// weighted sum of the values a small dense product:
//   * logits: one query row per lane, 64 rows per wave; the 8 floats of a
//     key's logit data (global direction, validity bias, global point) are
//     wave-uniform, read with scalar loads a chunk of 8 keys at a time and
//     used as the scalar operand of each vector instruction; per key and
//     row: 3 FMA for the direction dot, 6 for the squared distance, one
//     square root, one FMA to combine, the online-softmax exponential;
//   * P.V on bf16 matrix cores (v_mfma_f32_32x32x16_bf16) in three
//     products per 16-key chunk and 32-row block, Ph Vh + Ph Vl + Pl Vh,
//     with P and V split into bf16 hi + lo pairs (the dropped lo * lo term
//     is below 2^-18 relative, so the product keeps near-fp32 accuracy at a
//     fifth of the matrix-core time of fp32 products). 32 value columns: 3M values and a column of
//     ones that accumulates the softmax sum. A lane-half swap
//     (v_permlane32_swap) turns the row-per-lane P into the A operands of
//     both 32-row blocks; the B operand is the rotated values of 8 keys in
//     one column per lane, loaded with plain vector loads a chunk ahead;
//   * exponentials in base 2 (log2 e folded into the scales), the running
//     maximum raised lazily (only when a chunk's maximum exceeds it by more
//     than 2^8), so most chunks skip the rescale.
// Stages (one stream, all sizes linear in B * N):
//   dd_lift    per (b, n, h): global directions (the query one pre-scaled),
//              global points, rotated values, key validity -> qbuf, klog, kval.
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
constexpr int kChunk = 16;     // keys per online-softmax chunk (the key axis is padded to it)

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 values as bf16 pairs hi + lo: hi is each value rounded to bf16
// (nearest even), lo the exact fp32 remainder rounded to bf16, so
// |x - hi - lo| <= 2^-18 |x| and |lo| <= 2^-9 |x|: in a product of two
// split operands the dropped lo * lo term is below 2^-18 relative. The
// first value goes to the low half of each register.
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const f32x2 x = {x0, x1};
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
  const f32x2 r = {x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xffff0000u)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
}

// Value column whose entry is 1 for every valid key: the product P V then
// carries the softmax sum of each row in that column (3M <= 24 < 31).
constexpr int kSumCol = kValW - 1;

// acc[e] *= f[e] in place in the accumulation registers: plain vector code
// on the tile would move it to architectural registers and back on every
// iteration of the loop. The caller lets the matrix-core writes settle
// before (acc_settle) and after.
__device__ __forceinline__ void scale_acc(floatx16& acc, const float (&f)[16]) {
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float t;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "v_mul_f32 %1, %1, %2\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(acc[e]), "=&v"(t)
        : "v"(f[e]));
  }
}
// 32 wait states: more than any matrix-core result or accumulation-register
// write needs before the next access to the same registers.
__device__ __forceinline__ void acc_settle() { asm volatile("s_nop 15\n\ts_nop 15"); }

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
__global__ __launch_bounds__(64) void dd_lift_kernel(DDArgs a) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int H = a.H, M = a.M, Np = a.Np, N = a.N;
  const long long total = (long long)a.B * Np * H;
  if (t >= total) return;
  const int h = (int)(t % H);
  const int n = (int)((t / H) % Np);
  const int b = (int)(t / ((long long)H * Np));
  const size_t row = ((size_t)b * H + h) * Np + n;
  float4* qo = reinterpret_cast<float4*>(a.qbuf + row * 8);
  float4* ko = reinterpret_cast<float4*>(a.klog + row * kKeyLog);
  float4* vo = reinterpret_cast<float4*>(a.kval + row * kValW);
  const bool valid = n < N && a.frame_mask[(size_t)b * N + n] != 0;
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  if (!valid) {
    // padded keys and invalid frames: no contribution (bias -inf), zero data
    qo[0] = z4; qo[1] = z4;
    ko[0] = make_float4(0.f, 0.f, 0.f, -INFINITY); ko[1] = z4;
    for (int c = 0; c < kValW / 4; ++c) vo[c] = z4;
    return;
  }
  const size_t bn = (size_t)b * N + n;
  float R[9];
  for (int c = 0; c < 9; ++c) R[c] = a.rot[bn * 9 + c];
  const float* T = a.trans + bn * 3;
  const size_t v3 = (bn * H + h) * 3;
  const float cd = softplus_dev(a.direction_scale[h]) * kSqrt3Inv * kLog2e;
  float o[3], p[3];
  rotate(R, a.q_direction[v3], a.q_direction[v3 + 1], a.q_direction[v3 + 2], o);
  rotate(R, a.q_point[v3], a.q_point[v3 + 1], a.q_point[v3 + 2], p);
  qo[0] = make_float4(cd * o[0], cd * o[1], cd * o[2], 0.f);
  qo[1] = make_float4(p[0] + T[0], p[1] + T[1], p[2] + T[2], 0.f);
  rotate(R, a.k_direction[v3], a.k_direction[v3 + 1], a.k_direction[v3 + 2], o);
  rotate(R, a.k_point[v3], a.k_point[v3 + 1], a.k_point[v3 + 2], p);
  ko[0] = make_float4(o[0], o[1], o[2], 0.f);
  ko[1] = make_float4(p[0] + T[0], p[1] + T[1], p[2] + T[2], 0.f);
  const float* vv = a.values + (bn * H + h) * (size_t)M * 3;
  float g[kValW];
#pragma unroll
  for (int c = 0; c < kValW; ++c) g[c] = 0.f;
#pragma unroll
  for (int m = 0; m < kDDMaxM; ++m)
    if (m < M) rotate(R, vv[3 * m], vv[3 * m + 1], vv[3 * m + 2], g + 3 * m);
  g[kSumCol] = 1.f;   // P times this column is the softmax sum
#pragma unroll
  for (int c = 0; c < kValW / 4; ++c) vo[c] = make_float4(g[4 * c], g[4 * c + 1], g[4 * c + 2], g[4 * c + 3]);
}

// ---------------------------------------------------------------------------
// dd_attn
// ---------------------------------------------------------------------------
template <int M, bool PM>
__global__ __launch_bounds__(256) void dd_attn_kernel(DDArgs a) {
  constexpr int V = 3 * M;
  constexpr int PW = dd_part_width(M);
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
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

  const size_t bh = (size_t)b * H + h;
  const float4* qrow = reinterpret_cast<const float4*>(a.qbuf + (bh * Np + ic) * 8);
  const float4 qd = qrow[0], qp = qrow[1];
  const float cs = dist_coef(a.distance_scale, h);
  const float* __restrict__ klog = a.klog + bh * Np * kKeyLog;
  // this lane's B elements: value column l32 of keys 8 half .. 8 half + 7 of a chunk
  const float* __restrict__ kval = a.kval + bh * Np * kValW + half * 8 * kValW + l32;
  const uint8_t* pmrow = nullptr;
  if constexpr (PM) pmrow = a.pair_mask + (size_t)b * a.pm_sb + (size_t)h * a.pm_sh + (size_t)ic * a.pm_si;

  static_assert(kChunk == 16, "one 32x32x16 product per chunk and operand split");
  float bnext[8];
  auto load_b = [&](int ch) {
#pragma unroll
    for (int j = 0; j < 8; ++j) bnext[j] = kval[(size_t)(ch * kChunk + j) * kValW];
  };
  if (c0 < c1) load_b(c0);

  // Logit data of a chunk (8 keys x 8 floats) is staged through a per-wave
  // double buffer in LDS: lane l fetches float l of the chunk (one coalesced
  // 256-byte load), the wave writes it, and every lane then reads each key
  // as two broadcast float4. The global load runs two chunks ahead, the LDS
  // reads return in order, so neither waits for a full memory round trip.
  __shared__ float kls[4][2][kChunk * kKeyLog];
  float* kls_w = &kls[w][0][0];
  constexpr int NG = kChunk * kKeyLog / 64;   // floats per lane per chunk
  const float* __restrict__ klog_lane = klog + lane;
  float gnext[NG];
  if (c0 < c1) {
#pragma unroll
    for (int g = 0; g < NG; ++g) kls_w[64 * g + lane] = klog_lane[(size_t)c0 * kChunk * kKeyLog + 64 * g];
  }
  if (c0 + 1 < c1) {
#pragma unroll
    for (int g = 0; g < NG; ++g) gnext[g] = klog_lane[(size_t)(c0 + 1) * kChunk * kKeyLog + 64 * g];
  }
  asm volatile("" ::: "memory");

  // rows 0-31 and 32-63 of the wave, 32 value columns (the last one the
  // softmax sum)
  floatx16 acc0 = {}, acc1 = {};
  float m_run = -INFINITY;

  for (int ch = c0; ch < c1; ++ch) {
    const int buf = (ch - c0) & 1;
    // B = the chunk's values as bf16 hi + lo pairs
    uint32_t bh4[4], bl4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) split_pair(bnext[2 * j], bnext[2 * j + 1], bh4[j], bl4[j]);
    const u32x4 bhi = {bh4[0], bh4[1], bh4[2], bh4[3]}, blo = {bl4[0], bl4[1], bl4[2], bl4[3]};
    if (ch + 1 < c1) {
      load_b(ch + 1);
#pragma unroll
      for (int g = 0; g < NG; ++g) kls_w[(buf ^ 1) * kChunk * kKeyLog + 64 * g + lane] = gnext[g];
    }
    if (ch + 2 < c1) {
#pragma unroll
      for (int g = 0; g < NG; ++g) gnext[g] = klog_lane[(size_t)(ch + 2) * kChunk * kKeyLog + 64 * g];
    }
    const float4* kc = reinterpret_cast<const float4*>(kls_w + buf * kChunk * kKeyLog);
    float sv[kChunk];
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const float4 ka = kc[2 * k], kb = kc[2 * k + 1];
      const float dot = qd.x * ka.x + qd.y * ka.y + qd.z * ka.z;
      const float dx = qp.x - kb.x, dy = qp.y - kb.y, dz = qp.z - kb.z;
      const float d = __builtin_amdgcn_sqrtf(dx * dx + dy * dy + dz * dz);
      float lg = fmaf(-cs, d, dot) + ka.w;
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
      m_run = mn;
      // the factor of each accumulator row, fetched from the lane that owns
      // the row: register e of a 32-row block holds row 8 (e/4) + 4 half + e%4
      const int fi = __float_as_int(f);
      float f0[16], f1[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int src = 8 * (e >> 2) + 4 * half + (e & 3);
        f0[e] = __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, fi));
        f1[e] = __int_as_float(__builtin_amdgcn_ds_bpermute((32 + src) << 2, fi));
      }
      acc_settle();
      scale_acc(acc0, f0);
      scale_acc(acc1, f1);
      acc_settle();
    }
    const float ms = m_run == -INFINITY ? 0.f : m_run;
    float p[kChunk];
#pragma unroll
    for (int k = 0; k < kChunk; ++k) p[k] = __builtin_amdgcn_exp2f(sv[k] - ms);
    // P split the same way, two keys per register; one lane-half swap per
    // register pair gives the A operands of both 32-row blocks: block 0
    // takes keys 0-7 of rows 0-31 in lanes 0-31 and keys 8-15 of the same
    // rows in lanes 32-63, block 1 likewise for rows 32-63
    uint32_t phi[8], plo[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) split_pair(p[2 * j], p[2 * j + 1], phi[j], plo[j]);
    uint32_t a0h4[4], a1h4[4], a0l4[4], a1l4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto sh = __builtin_amdgcn_permlane32_swap(phi[j], phi[4 + j], false, false);
      const auto sl = __builtin_amdgcn_permlane32_swap(plo[j], plo[4 + j], false, false);
      a0h4[j] = sh[0]; a1h4[j] = sh[1];
      a0l4[j] = sl[0]; a1l4[j] = sl[1];
    }
    const u32x4 a0h = {a0h4[0], a0h4[1], a0h4[2], a0h4[3]}, a1h = {a1h4[0], a1h4[1], a1h4[2], a1h4[3]};
    const u32x4 a0l = {a0l4[0], a0l4[1], a0l4[2], a0l4[3]}, a1l = {a1l4[0], a1l4[1], a1l4[2], a1l4[3]};
    const bf16x8 Bh = __builtin_bit_cast(bf16x8, bhi), Bl = __builtin_bit_cast(bf16x8, blo);
    const bf16x8 A0h = __builtin_bit_cast(bf16x8, a0h), A0l = __builtin_bit_cast(bf16x8, a0l);
    const bf16x8 A1h = __builtin_bit_cast(bf16x8, a1h), A1l = __builtin_bit_cast(bf16x8, a1l);
    // P V ~ Ph Vh + Ph Vl + Pl Vh (the dropped Pl Vl is below 2^-18 relative)
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0h, Bh, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1h, Bh, acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0h, Bl, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1h, Bl, acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0l, Bh, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1l, Bh, acc1, 0, 0, 0);
    // the next iteration reads the buffer written above and rewrites this
    // one: LDS operations of a wave complete in order, only the compiler
    // must keep them in program order
    asm volatile("" ::: "memory");
  }

  // merge the four waves' key ranges through LDS
  constexpr int LS = V + 1;   // odd row pitch: conflict-free per-lane rows
  __shared__ float red_ml[4][64][2];
  __shared__ float red_acc[4][64][LS];
  red_ml[w][lane][0] = m_run;
  if (l32 < V) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = 8 * (e >> 2) + 4 * half + (e & 3);
      red_acc[w][r][l32] = acc0[e];
      red_acc[w][32 + r][l32] = acc1[e];
    }
  } else if (l32 == kSumCol) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = 8 * (e >> 2) + 4 * half + (e & 3);
      red_ml[w][r][1] = acc0[e];
      red_ml[w][32 + r][1] = acc1[e];
    }
  }
  __syncthreads();
  if (w != 0 || i >= N) return;
  float mm = red_ml[0][lane][0];
  for (int u = 1; u < 4; ++u) mm = fmaxf(mm, red_ml[u][lane][0]);
  float fu[4];
  float lt = 0.f;
  for (int u = 0; u < 4; ++u) {
    const float mu = red_ml[u][lane][0];
    fu[u] = mu == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mu - mm);
    lt = fmaf(red_ml[u][lane][1], fu[u], lt);
  }
  float* po = a.part + ((((size_t)s * a.B + b) * N + i) * H + h) * PW;
  po[0] = mm;
  po[1] = lt;
#pragma unroll
  for (int c = 0; c < V; ++c) {
    float v = 0.f;
    for (int u = 0; u < 4; ++u) v = fmaf(red_acc[u][lane][c], fu[u], v);
    po[2 + c] = v;
  }
}

// ---------------------------------------------------------------------------
// dd_finish: one thread per (b, i, h, m): merge the key splits' partials,
// divide by the softmax sum, rotate back by R_i^T. The m = 0 thread of each
// (b, i, h) also writes the row statistics.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dd_finish_kernel(DDArgs a) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int H = a.H, M = a.M, N = a.N, S = a.splits, PW = a.PW;
  if (t >= (long long)a.B * N * H * M) return;
  const int m = (int)(t % M);
  const long long bih = t / M;             // (b * N + i) * H + h
  const int h = (int)(bih % H);
  const long long bi = bih / H;
  const int i = (int)(bi % N), b = (int)(bi / N);
  float* vo = a.vectors + (size_t)t * 3;
  float2* st = reinterpret_cast<float2*>(a.stats) + ((size_t)b * H + h) * N + i;
  if (!a.frame_mask[bi]) {
    vo[0] = 0.f; vo[1] = 0.f; vo[2] = 0.f;
    if (m == 0) *st = make_float2(0.f, 0.f);
    return;
  }
  const size_t pstride = (size_t)a.B * N * H * PW;
  const float* p0 = a.part + (size_t)bih * PW;
  // running merge over the splits: (mm, l, g) rescaled whenever a split
  // brings a larger maximum
  float mm = -INFINITY, l = 0.f, gx = 0.f, gy = 0.f, gz = 0.f;
  for (int s = 0; s < S; ++s) {
    const float* ps = p0 + s * pstride;
    const float msp = ps[0];
    if (msp == -INFINITY) continue;   // an empty split adds nothing
    const float mn = fmaxf(mm, msp);
    const float fo = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mm - mn);
    const float fn = __builtin_amdgcn_exp2f(msp - mn);
    l = fmaf(ps[1], fn, l * fo);
    gx = fmaf(ps[2 + 3 * m], fn, gx * fo);
    gy = fmaf(ps[3 + 3 * m], fn, gy * fo);
    gz = fmaf(ps[4 + 3 * m], fn, gz * fo);
    mm = mn;
  }
  if (m == 0) *st = make_float2(mm == -INFINITY ? 0.f : mm, l);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  gx *= inv; gy *= inv; gz *= inv;
  const float* R = a.rot + bi * 9;
  // R_i^T g: column x of R dotted with g
  vo[0] = (R[0] * gx + R[3] * gy + R[6] * gz) + 0.f;
  vo[1] = (R[1] * gx + R[4] * gy + R[7] * gz) + 0.f;
  vo[2] = (R[2] * gx + R[5] * gy + R[8] * gz) + 0.f;
}

// ---------------------------------------------------------------------------
// dd_readout: out[r][c] = sum_k vec[r][k] W[k][c] + bias[c] on
// v_mfma_f32_32x32x2f32. A workgroup of four waves owns a 32 x 32 output
// tile and splits the reduction in four; each wave issues all of its
// operand loads at once (buffer loads straight into registers), runs its
// products, and the four partial tiles are summed through LDS. Lane l feeds
// row / column l % 32 and reduction slot l / 32 of each product; the
// reduction index is permuted (slot 0 takes k = 8t..8t+3, slot 1
// k = 8t+4..8t+7 over four products) so a lane reads its vector row as one
// float4 per four products.
// ---------------------------------------------------------------------------
constexpr int kRoTile = 32, kRoWaves = 4, kRoMaxK8 = 12;   // up to 96 reduction steps per wave

template <bool V4>   // K % 4 == 0: each lane reads its 4 vector elements as one 16-byte load
__global__ __launch_bounds__(64 * kRoWaves) void dd_readout_kernel(DDArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int half = lane >> 5, li = lane & 31;
  const int rows = a.B * a.N, K = 3 * a.H * a.M, Cout = a.Cout;
  const int r0 = blockIdx.x * kRoTile, c0 = blockIdx.y * kRoTile;
  const int nk8 = (K + 7) / 8;                       // groups of 8 reduction steps
  // buffer loads: an offset past the end of the resource reads 0, so the
  // ragged edges (rows past B*N, k past K, columns past Cout) need no branch
  constexpr uint32_t kOut = 0x80000000u;
  const int nr = rows - r0 < kRoTile ? rows - r0 : kRoTile;
  const __amdgpu_buffer_rsrc_t ra_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.vectors) + (size_t)r0 * K, (short)0, (int)((size_t)nr * K * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.w_out) + c0, (short)0, (int)(((size_t)K * Cout - c0) * 4), 0x00020000);
  const bool row_ok = li < nr, col_ok = c0 + li < Cout;
  floatx16 c = {};
  // this wave's share of the k8 groups, processed kRoMaxK8 at a time
  const int g0 = nk8 * wv / kRoWaves, g1 = nk8 * (wv + 1) / kRoWaves;
  for (int gb = g0; gb < g1; gb += kRoMaxK8) {
    float av[kRoMaxK8][4], bv[kRoMaxK8][4];
#pragma unroll
    for (int t = 0; t < kRoMaxK8; ++t) {
      const int kb = 8 * (gb + t) + 4 * half;          // first k of this lane's float4
      const bool in = gb + t < g1;
      if constexpr (V4) {
        // kb % 4 == 0 and K % 4 == 0: the four elements are in range together
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
            ra_rs, (in && kb < K && row_ok) ? (uint32_t)(li * K + kb) * 4u : kOut, 0, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) av[t][u] = __uint_as_float(v[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = kb + u;
        const bool ok = in && k < K;
        if constexpr (!V4)
          av[t][u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              ra_rs, (ok && row_ok) ? (uint32_t)(li * K + k) * 4u : kOut, 0, 0));
        bv[t][u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rw_rs, (ok && col_ok) ? (uint32_t)(k * Cout + li) * 4u : kOut, 0, 0));
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // every load in flight before the first product
#pragma unroll
    for (int t = 0; t < kRoMaxK8; ++t)
#pragma unroll
      for (int u = 0; u < 4; ++u) c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[t][u], bv[t][u], c, 0, 0, 0);
  }
  // sum the four waves' partial tiles
  __shared__ float red[kRoWaves - 1][16][64];
  __shared__ int row_any[kRoTile];
  if (wv > 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) red[wv - 1][e][lane] = c[e];
  }
  if (tid < kRoTile) {
    int any = 0;
    const int r = r0 + tid;
    if (r < rows) {
      const int b = r / a.N, i = r - b * a.N;
      const float2* st = reinterpret_cast<const float2*>(a.stats);
      for (int h = 0; h < a.H && !any; ++h) any = st[((size_t)b * a.H + h) * a.N + i].y > 0.f;
    }
    row_any[tid] = any;
  }
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int e = 0; e < 16; ++e)
    for (int u = 0; u < kRoWaves - 1; ++u) c[e] += red[u][e][lane];
  const int col = c0 + li;
  if (col >= Cout) return;
  const float bias = a.b_out ? a.b_out[col] : 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int rr = 8 * (e >> 2) + 4 * half + (e & 3);
    const int r = r0 + rr;
    if (r < rows) a.output[(size_t)r * Cout + col] = row_any[rr] ? c[e] + bias : 0.f;
  }
}

// ---------------------------------------------------------------------------
// dd_probs: attention[b][h][i][j] = exp2(s_ij - m_i) / l_i on allowed edges.
// One row i per wave iteration, keys across lanes (coalesced writes).
// ---------------------------------------------------------------------------
constexpr int kProbRows = 4;

__global__ __launch_bounds__(256) void dd_probs_kernel(DDArgs a) {
  const int H = a.H, N = a.N, Np = a.Np;
  const int bh = blockIdx.z, b = bh / H, h = bh - b * H;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= N) return;
  const float cs = dist_coef(a.distance_scale, h);
  const float4* kr = reinterpret_cast<const float4*>(a.klog + ((size_t)bh * Np + j) * kKeyLog);
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
    hipLaunchKernelGGL(dd_lift_kernel, dim3((unsigned)((total + 63) / 64)), dim3(64), 0, s, a);
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
    const long long total = (long long)a.B * a.N * a.H * a.M;
    hipLaunchKernelGGL(dd_finish_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  {
    const dim3 grid((a.B * a.N + kRoTile - 1) / kRoTile, (a.Cout + kRoTile - 1) / kRoTile);
    if ((3 * a.H * a.M) % 4 == 0)
      hipLaunchKernelGGL(dd_readout_kernel<true>, grid, dim3(64 * kRoWaves), 0, s, a);
    else
      hipLaunchKernelGGL(dd_readout_kernel<false>, grid, dim3(64 * kRoWaves), 0, s, a);
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
