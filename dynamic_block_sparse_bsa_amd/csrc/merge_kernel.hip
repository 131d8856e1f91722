// Split-K merge for gfx950 (Tessera paper, section 4.3 "Split-K"): the
// partial states (m, l, O) that several workgroups wrote for one query tile
// are rescaled to their common maximum, summed and normalized.  Running
// maxima are in log2 units (scores times log2(e)/sqrt(d)), so the weights are
// exp2(m_p - m*).  A row whose partitions are all empty (l = 0) outputs zeros.
// HBM-bound: each partial element is read once, each output written once.
#include "bsa_internal.h"

namespace bsa {
namespace {

__global__ __launch_bounds__(256) void k_merge(const MergeArgs a) {
  const int g = blockIdx.x;
  const int parts = a.parts[g];
  if (parts <= 1) return;
  const int h = g / a.n_qtiles_head;
  const int qt = g - h * a.n_qtiles_head;
  const int sb = a.slot_base[g];
  const int TQ = a.tq;
  const int D = a.d;
  const int nch = D / 8;  // 8 output values per thread item
  for (int item = threadIdx.x; item < TQ * nch; item += 256) {
    const int r = item % TQ;
    const int dc = item / TQ;
    const int row = qt * TQ + r;
    if (row >= a.N) continue;
    float mstar = -INFINITY;
    for (int p = 0; p < parts; ++p) {
      const size_t s = (size_t)(sb + p);
      if (a.ws_l[s * TQ + r] > 0.0f) mstar = fmaxf(mstar, a.ws_m[s * TQ + r]);
    }
    float num[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float den = 0.0f;
    for (int p = 0; p < parts; ++p) {
      const size_t s = (size_t)(sb + p);
      const float l = a.ws_l[s * TQ + r];
      if (!(l > 0.0f)) continue;
      const float wgt = __builtin_amdgcn_exp2f(a.ws_m[s * TQ + r] - mstar);
      den += wgt * l;
      const float* o = a.ws_o + s * (size_t)D * TQ + (size_t)(dc * 8) * TQ + r;
#pragma unroll
      for (int i = 0; i < 8; ++i) num[i] += wgt * o[(size_t)i * TQ];
    }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    __bf16 outv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) outv[i] = (__bf16)(num[i] * inv);
    __bf16* op = a.o + ((size_t)h * a.N + row) * D + dc * 8;
    *reinterpret_cast<uint4*>(op) = *reinterpret_cast<const uint4*>(outv);
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int32_t n_qtiles, hipStream_t s) {
  hipLaunchKernelGGL(k_merge, dim3(n_qtiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bsa
