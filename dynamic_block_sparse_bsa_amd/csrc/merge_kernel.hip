// Split-K merge for gfx950 (Tessera paper, section 4.3 "Split-K"): the
// partial states (m, l, O) that several workgroups wrote for one query tile
// are rescaled to their common maximum, summed and normalized.  Running
// maxima are in log2 units (scores times log2(e)/sqrt(d)), so the weights are
// exp2(m_p - m*).  A row whose partitions are all empty (l = 0) outputs zeros.
//
// One workgroup per (split query tile, 16 output columns), so even a few
// split tiles spread over many CUs.  The per-row weights w_p l_p / sum_q w_q l_q
// are computed once per workgroup (one thread per row) into LDS; the threads
// then stream the partial outputs, four output columns per thread item,
// reading [slot][d/2][T_Q] rows of bf16 pairs contiguously.  Each partial is
// its partition's output normalized by its own exponential sum, so the
// weights carry l_p.  HBM-bound: each partial element is
// read once and each output element written once.
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kMaxParts = 32;   // partitions whose weights are held in LDS
constexpr int kMaxTq = 256;
constexpr int kCols = 16;       // output columns per workgroup

__global__ __launch_bounds__(256) void k_merge(const MergeArgs a) {
  __shared__ float wgt[kMaxParts][kMaxTq];
  if (a.guard && *a.guard == 0ull) return;
  const int g = blockIdx.x;
  const int parts = a.parts[g];
  if (parts <= 1) return;
  const int h = g / a.n_qtiles_head;
  const int qt = g - h * a.n_qtiles_head;
  const int bat = h / a.heads;
  const size_t head_off = (size_t)bat * a.batch_stride + (size_t)(h - bat * a.heads) * a.head_stride;
  const int sb = a.slot_base[g];
  const int TQ = a.tq;
  const int D = a.d;
  const int t = threadIdx.x;
  // (1) per-row common maximum and normalizer; weights of the first kMaxParts
  // partitions go to LDS, further ones are recomputed while streaming
  float mstar = -INFINITY, inv = 0.0f;
  if (t < TQ) {
#pragma unroll 4
    for (int p = 0; p < parts; ++p) {
      const size_t s = (size_t)(sb + p) * TQ + t;
      if (a.ws_l[s] > 0.0f) mstar = fmaxf(mstar, a.ws_m[s]);
    }
    float den = 0.0f;
#pragma unroll 4
    for (int p = 0; p < parts; ++p) {
      const size_t s = (size_t)(sb + p) * TQ + t;
      const float l = a.ws_l[s];
      const float w = l > 0.0f ? __builtin_amdgcn_exp2f(a.ws_m[s] - mstar) : 0.0f;
      den += w * l;
      if (p < kMaxParts) wgt[p][t] = w * l;  // the partials are normalized by their own l
    }
    inv = den > 0.0f ? 1.0f / den : 0.0f;
    for (int p = 0; p < min(parts, kMaxParts); ++p) wgt[p][t] *= inv;
  }
  __syncthreads();
  // (2) out[r][c..c+3] = sum_p wgt[p][r] * O_p[c..c+3][r] (O_p normalized,
  // stored as bf16 pairs), c in this workgroup's kCols columns; the
  // partition loop is unrolled so several partitions' loads are in flight
  // together
  const int nitems = TQ * (kCols / 4);
  for (int item = t; item < nitems; item += 256) {
    const int r = item % TQ;
    const int c = blockIdx.y * kCols + (item / TQ) * 4;
    const int row = qt * TQ + r;
    if (row >= a.N) continue;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
    for (int p = 0; p < parts; ++p) {
      float w;
      if (p < kMaxParts) {
        w = wgt[p][r];
      } else {  // recompute (rare: more than kMaxParts partitions)
        float ms = -INFINITY, den = 0.0f;
        for (int q = 0; q < parts; ++q) {
          const size_t s = (size_t)(sb + q) * TQ + r;
          if (a.ws_l[s] > 0.0f) ms = fmaxf(ms, a.ws_m[s]);
        }
        for (int q = 0; q < parts; ++q) {
          const size_t s = (size_t)(sb + q) * TQ + r;
          if (a.ws_l[s] > 0.0f) den += __builtin_amdgcn_exp2f(a.ws_m[s] - ms) * a.ws_l[s];
        }
        const size_t s = (size_t)(sb + p) * TQ + r;
        const float l = a.ws_l[s];
        w = (l > 0.0f && den > 0.0f) ? __builtin_amdgcn_exp2f(a.ws_m[s] - ms) * l / den : 0.0f;
      }
      const uint32_t* o = a.ws_o + (size_t)(sb + p) * (D / 2) * TQ + (size_t)(c >> 1) * TQ + r;
      const uint32_t x0 = o[0], x1 = o[TQ];  // columns (c, c+1) and (c+2, c+3)
      acc[0] += w * __uint_as_float(x0 << 16);
      acc[1] += w * __uint_as_float(x0 & 0xffff0000u);
      acc[2] += w * __uint_as_float(x1 << 16);
      acc[3] += w * __uint_as_float(x1 & 0xffff0000u);
    }
    __bf16 ov[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ov[i] = (__bf16)acc[i];
    *reinterpret_cast<uint2*>(a.o + head_off + (size_t)row * a.row_stride + c) =
        *reinterpret_cast<const uint2*>(ov);
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int32_t n_qtiles, hipStream_t s) {
  if (a.tq > kMaxTq) return hipErrorInvalidValue;
  if (a.d % kCols) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_merge, dim3(n_qtiles, a.d / kCols), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bsa
