// Split-K merge for gfx950 (Tessera paper, section 4.3 "Split-K"): the
// partial states (m, l, O) that several workgroups wrote for one query tile
// are rescaled to their common maximum, summed and normalized.  Running
// maxima are in log2 units (scores times log2(e)/sqrt(d)), so the weights are
// exp2(m_p - m*).  A row whose partitions are all empty (l = 0) outputs zeros.
//
// One workgroup per (split query tile, 16 output columns), so even a few
// split tiles spread over many CUs.  256 is a multiple of T_Q, so every thread
// owns one row (t mod T_Q) and 4-column quads of it; it computes its row's
// weights w_p l_p / sum_q w_q l_q in registers (each partial is its
// partition's output normalized by its own exponential sum, so the weights
// carry l_p) and streams the partial outputs, stored as [slot][d][T_Q] fp32
// (so a split row is rounded to bf16 once, at the output, like an unsplit
// one), with the loads of all partitions in flight together (addresses past
// the last partition are clamped to it and weighted 0).  No LDS and no
// barrier.  HBM-bound: each partial element is read once and each output
// element written once.
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kMaxTq = 256;
constexpr int kCols = kMergeCols;  // output columns per item

struct MergeRow {
  const MergeArgs* a;
  int sb, parts, TQ, r;
  int c0;        // first output column of the item's column group
  size_t o_row;  // output element offset of the row
};

// Weights of row r for partitions [0, P) (P >= parts; entries past parts are 0).
template <int P>
__device__ __forceinline__ void row_weights(const MergeRow& m, float (&w)[P]) {
  const MergeArgs& a = *m.a;
  float mp[P], lp[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const size_t s = (size_t)(m.sb + min(p, m.parts - 1)) * m.TQ + m.r;
    mp[p] = a.ws_m[s];
    lp[p] = p < m.parts ? a.ws_l[s] : 0.0f;
  }
  float mstar = -INFINITY;
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (lp[p] > 0.0f) mstar = fmaxf(mstar, mp[p]);
  float den = 0.0f;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    w[p] = lp[p] > 0.0f ? __builtin_amdgcn_exp2f(mp[p] - mstar) * lp[p] : 0.0f;
    den += w[p];
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
  for (int p = 0; p < P; ++p) w[p] *= inv;
}

__device__ __forceinline__ void store_quad(const MergeRow& m, int c, const float (&acc)[4]) {
  __bf16 ov[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) ov[i] = (__bf16)acc[i];
  *reinterpret_cast<uint2*>(m.a->o + m.o_row + c) = *reinterpret_cast<const uint2*>(ov);
}

// Up to P partitions: weights and every partial load of a quad in registers.
template <int P>
__device__ __forceinline__ void merge_row(const MergeRow& m, int q0, int qstep) {
  const MergeArgs& a = *m.a;
  float w[P];
  row_weights<P>(m, w);
  for (int qi = q0; qi < kCols / 4; qi += qstep) {
    const int c = m.c0 + qi * 4;
    float x[P][4];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const float* o = a.ws_o + (size_t)(m.sb + min(p, m.parts - 1)) * a.d * m.TQ + (size_t)c * m.TQ + m.r;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[p][i] = o[(size_t)i * m.TQ];  // column c + i
    }
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += w[p] * x[p][i];
    store_quad(m, c, acc);
  }
}

// Any number of partitions: the weights are recomputed per partition from
// two passes over (m, l) (rare: more than 16 partitions).
__device__ void merge_row_any(const MergeRow& m, int q0, int qstep) {
  const MergeArgs& a = *m.a;
  float mstar = -INFINITY, den = 0.0f;
  for (int p = 0; p < m.parts; ++p) {
    const size_t s = (size_t)(m.sb + p) * m.TQ + m.r;
    if (a.ws_l[s] > 0.0f) mstar = fmaxf(mstar, a.ws_m[s]);
  }
  for (int p = 0; p < m.parts; ++p) {
    const size_t s = (size_t)(m.sb + p) * m.TQ + m.r;
    const float l = a.ws_l[s];
    if (l > 0.0f) den += __builtin_amdgcn_exp2f(a.ws_m[s] - mstar) * l;
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  for (int qi = q0; qi < kCols / 4; qi += qstep) {
    const int c = m.c0 + qi * 4;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
    for (int p = 0; p < m.parts; ++p) {
      const size_t s = (size_t)(m.sb + p) * m.TQ + m.r;
      const float l = a.ws_l[s];
      const float w = l > 0.0f ? __builtin_amdgcn_exp2f(a.ws_m[s] - mstar) * l * inv : 0.0f;
      const float* o = a.ws_o + (size_t)(m.sb + p) * a.d * m.TQ + (size_t)c * m.TQ + m.r;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += w * o[(size_t)i * m.TQ];
    }
    store_quad(m, c, acc);
  }
}

// One (query tile g, column group cg) item: this thread's row of the tile.
__device__ __forceinline__ void merge_item(const MergeArgs& a, int g, int cg) {
  const int parts = a.parts[g];
  if (parts <= 1) return;
  const int h = g / a.n_qtiles_head;
  const int qt = g - h * a.n_qtiles_head;
  const int t = threadIdx.x;
  MergeRow m;
  m.a = &a;
  m.sb = a.slot_base[g];
  m.parts = parts;
  m.TQ = a.tq;
  m.r = t % m.TQ;
  m.c0 = cg * kCols;
  const int row = qt * m.TQ + m.r;
  if (row >= a.N) return;
  const int bat = h / a.heads;
  m.o_row = (size_t)bat * a.batch_stride + (size_t)(h - bat * a.heads) * a.head_stride + (size_t)row * a.row_stride;
  const int q0 = t / m.TQ, qstep = 256 / m.TQ;  // this thread's 4-column quads of the group
  if (parts <= 2) merge_row<2>(m, q0, qstep);
  else if (parts <= 4) merge_row<4>(m, q0, qstep);
  else if (parts <= 8) merge_row<8>(m, q0, qstep);
  else if (parts <= 16) merge_row<16>(m, q0, qstep);
  else merge_row_any(m, q0, qstep);
}

// Grid (query tiles, column groups), or with the compact list of split tiles
// a fixed number of workgroups looping over (listed tile, column group)
// items (no barrier, so a workgroup's threads need not stay in step).
__global__ __launch_bounds__(256) void k_merge(const MergeArgs a) {
  if (a.guard && *a.guard == 0ull) return;
  if (a.split_tiles) {
    const int ng = a.d / kCols;
    const long long items = (long long)(*a.n_split) * ng;
    for (long long it = blockIdx.x; it < items; it += gridDim.x)
      merge_item(a, a.split_tiles[it / ng], (int)(it % ng));
  } else {
    merge_item(a, blockIdx.x, blockIdx.y);
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int32_t n_qtiles, hipStream_t s, int32_t grid_items) {
  if (a.tq > kMaxTq || 256 % a.tq != 0) return hipErrorInvalidValue;
  if (a.d % kCols) return hipErrorInvalidValue;
  if (a.split_tiles) {
    if (grid_items <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_merge, dim3(grid_items), dim3(256), 0, s, a);
  } else
    hipLaunchKernelGGL(k_merge, dim3(n_qtiles, a.d / kCols), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bsa
