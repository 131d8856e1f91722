// Block-sparse attention mainloop for gfx950 (CDNA4), bf16 MFMA with fp32
// accumulation.
//
// Tessera paper, section 2.3: a FlashAttention-style traversal keeps one query
// tile, its online-softmax state (running max m, scaled exponential sum l,
// output accumulator O) and the output on chip while K/V tiles stream through
// the mainloop; section 4.2 defines the physical tile T = (T_Q, T_KV) that a
// plan maps logical blocks to (Direct, Coarsened with membership masking
// before the softmax update, Refined); section 4.3 defines split-K partial
// states that a later kernel merges.
//
// Design on gfx950 (one workgroup = T_Q/32 waves, each wave owns 32 queries):
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane then holds 16 keys of ONE query
//    column, so the softmax max and sum are lane-local except for a single
//    exchange with lane^32.  The output is accumulated transposed too,
//    O^T += V^T P^T, and the probabilities P^T are consumed straight from the
//    score accumulators (no cross-lane shuffle) because the K rows are fed to
//    the QK^T MFMA in a bit-permuted order that makes the result layout equal
//    the B-operand layout of the PV MFMA.
//  * Q stays in VGPRs (B operand) for the whole task.  K is staged in LDS
//    row-major, V transposed (keys contiguous), both with XOR swizzles on 16-
//    byte chunks so the MFMA operand reads are bank-conflict free.  The next
//    K/V tile is fetched into registers while the current one is computed.
//  * Softmax runs in the exp2 domain with the 1/sqrt(d) scale folded into one
//    FMA per score; a fully masked row never produces NaN (running max -inf is
//    treated as 0 for the exponent offset) and ends with O = 0.
#pragma once

#include "bsa_internal.h"

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Row order of K fed to the QK^T MFMA: swaps bits 2 and 3 of the row index
// within each group of 16 (an involution).
__device__ __forceinline__ int kperm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <int TQ, int TKV, int D>
struct AttnShape {
  static constexpr int WAVES = TQ / 32;
  static constexpr int NT = WAVES * 64;
  static constexpr int KCH = D / 8;                    // 16-byte chunks per K row
  static constexpr int CPT = TKV * D / 8 / NT;         // chunks per thread per tile
  static constexpr int NST = TKV / 32;                 // 32-key sub-tiles
  static constexpr int DB = D / 32;                    // 32-wide blocks of d
  static constexpr int DK = D / 16;                    // k-steps of the QK^T MFMA
  static constexpr int VCH = TKV / 8;                  // 16-byte chunks per V^T row
  static constexpr int VRPB = (TKV * 2 >= 128) ? 1 : 128 / (TKV * 2);  // V^T rows per 128 B
  static constexpr int KBYTES = TKV * D * 2;
  static constexpr int VBYTES = TKV * D * 2;
  static_assert(CPT >= 1, "tile too small for the workgroup");
  static_assert(TQ % 32 == 0 && TKV % 32 == 0 && D % 32 == 0, "shape");
};

// byte offset of (row, 16B chunk) in the K tile
template <int TQ, int TKV, int D>
__device__ __forceinline__ int k_off(int row, int ch) {
  using S = AttnShape<TQ, TKV, D>;
  const int sw = kperm(row & 15) & (S::KCH - 1);
  return row * (D * 2) + ((ch ^ sw) << 4);
}

// byte offset of (d row, 16B key chunk) in the V^T tile
template <int TQ, int TKV, int D>
__device__ __forceinline__ int v_off(int drow, int kc) {
  using S = AttnShape<TQ, TKV, D>;
  const int sw = (drow / S::VRPB) & (S::VCH - 1);
  return drow * (TKV * 2) + ((kc ^ sw) << 4);
}

template <int TQ, int TKV, int D>
__global__ __launch_bounds__(TQ * 2) void attn_fwd_kernel(const AttnArgs a) {
  using S = AttnShape<TQ, TKV, D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::KBYTES + S::VBYTES];
  unsigned char* const kl = smem;
  unsigned char* const vl = smem + S::KBYTES;

  // ---- task -------------------------------------------------------------
  int bid = blockIdx.x;
  if (a.xcd_remap) {
    const int per = a.grid >> 3;
    bid = (bid & 7) * per + (bid >> 3);
  }
  if ((unsigned long long)bid >= *a.n_tasks) return;
  const Task task = a.tasks[bid];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;   // query column within the wave (B operand / C column)
  const int hh = lane >> 5;  // lane half
  const int N = a.N;
  const size_t head_off = (size_t)task.head * N * D;
  const int qrow = task.qtile * TQ + w * 32 + n;

  // ---- Q fragment: B operand of S^T = K Q^T, resident for the task -------
  bf16x8 qf[S::DK];
  {
    const bool ok = qrow < N;
    const __bf16* qp = a.q + head_off + (size_t)qrow * D + 8 * hh;
#pragma unroll
    for (int c = 0; c < S::DK; ++c) {
      if (ok) {
        qf[c] = *reinterpret_cast<const bf16x8*>(qp + 16 * c);
      } else {
        for (int i = 0; i < 8; ++i) qf[c][i] = (__bf16)0.0f;
      }
    }
  }

  // membership: which logical sub-row of a coarsened tile this wave covers
  const int sub_row = (a.coarsen_q > 1) ? (w * 32) / a.bq : 0;
  const uint32_t full_kv = (a.coarsen_kv >= 32) ? 0xffffffffu : ((1u << a.coarsen_kv) - 1u);

  // ---- online-softmax state (lane-local; l is a half-sum over this lane's keys)
  float m_run = -INFINITY;
  float l_run = 0.0f;
  f32x16 acc[S::DB];
#pragma unroll
  for (int b = 0; b < S::DB; ++b)
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.0f;

  const int nsub = 1 << a.sub_log2;
  const int total = (task.end - task.begin) << a.sub_log2;

  // register staging of the next tile
  u32x4 kreg[S::CPT];
  u32x4 vreg[S::CPT];
  const int vdc = tid % S::KCH;      // V loader: 16B column chunk (8 d values)
  const int vrg = tid / S::KCH;      // V loader: group of CPT consecutive key rows

  auto tile_kv0 = [&](int j) -> int {
    const int it = task.begin + (j >> a.sub_log2);
    const int sub = j & (nsub - 1);
    return ((a.tcol[it] << a.sub_log2) + sub) * TKV;
  };
  auto load_tile = [&](int kv0) {
    const __bf16* kp = a.k + head_off;
    const __bf16* vp = a.v + head_off;
#pragma unroll
    for (int i = 0; i < S::CPT; ++i) {
      const int g = tid + i * S::NT;
      const int row = g / S::KCH;
      const int ch = g % S::KCH;
      const int key = kv0 + row;
      if (key < N)
        kreg[i] = *reinterpret_cast<const u32x4*>(kp + (size_t)key * D + ch * 8);
      else
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < S::CPT; ++i) {
      const int key = kv0 + vrg * S::CPT + i;
      if (key < N)
        vreg[i] = *reinterpret_cast<const u32x4*>(vp + (size_t)key * D + vdc * 8);
      else
        vreg[i] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < S::CPT; ++i) {
      const int g = tid + i * S::NT;
      const int row = g / S::KCH;
      const int ch = g % S::KCH;
      *reinterpret_cast<u32x4*>(kl + k_off<TQ, TKV, D>(row, ch)) = kreg[i];
    }
    // transpose CPT key rows x 8 d values into 8 d rows x CPT keys
    const int k0 = vrg * S::CPT;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int drow = vdc * 8 + c;
      uint32_t packed[(S::CPT + 1) / 2];
#pragma unroll
      for (int p = 0; p < (S::CPT + 1) / 2; ++p) {
        const uint32_t lo = vreg[2 * p][c >> 1];
        const uint32_t hi = (2 * p + 1 < S::CPT) ? vreg[2 * p + 1][c >> 1] : 0u;
        packed[p] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      if constexpr (S::CPT >= 8) {
#pragma unroll
        for (int q8 = 0; q8 < S::CPT / 8; ++q8) {
          const int kc = (k0 >> 3) + q8;
          *reinterpret_cast<u32x4*>(vl + v_off<TQ, TKV, D>(drow, kc)) =
              u32x4{packed[4 * q8], packed[4 * q8 + 1], packed[4 * q8 + 2], packed[4 * q8 + 3]};
        }
      } else if constexpr (S::CPT == 4) {
        const int kc = k0 >> 3;
        *reinterpret_cast<u32x2*>(vl + v_off<TQ, TKV, D>(drow, kc) + (k0 & 7) * 2) =
            u32x2{packed[0], packed[1]};
      } else if constexpr (S::CPT == 2) {
        const int kc = k0 >> 3;
        *reinterpret_cast<uint32_t*>(vl + v_off<TQ, TKV, D>(drow, kc) + (k0 & 7) * 2) = packed[0];
      } else {
        static_assert(S::CPT == 1 || S::CPT == 2 || S::CPT == 4 || S::CPT % 8 == 0, "CPT");
        const int kc = k0 >> 3;
        *reinterpret_cast<unsigned short*>(vl + v_off<TQ, TKV, D>(drow, kc) + (k0 & 7) * 2) =
            (unsigned short)(packed[0] & 0xffffu);
      }
    }
  };

  // skip trailing refined sub-tiles that start at or beyond N
  int j = 0;
  int kv0 = 0;
  auto next_valid = [&](int from, int& kvs) -> int {
    int jj = from;
    while (jj < total) {
      kvs = tile_kv0(jj);
      if (kvs < N) break;
      ++jj;
    }
    return jj;
  };
  j = next_valid(0, kv0);
  if (j < total) load_tile(kv0);

  while (j < total) {
    const int it = task.begin + (j >> a.sub_log2);
    uint32_t wbits = full_kv;
    if (a.tbits) wbits = (a.tbits[it] >> (sub_row * a.coarsen_kv)) & full_kv;
    const int cur_kv0 = kv0;

    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();  // tile visible

    int kvn = 0;
    const int jn = next_valid(j + 1, kvn);
    if (jn < total) load_tile(kvn);

    if (wbits != 0u) {
      // ---- S^T = K Q^T ---------------------------------------------------
      f32x16 s[S::NST];
#pragma unroll
      for (int st = 0; st < S::NST; ++st) {
        for (int i = 0; i < 16; ++i) s[st][i] = 0.0f;
        const int krow = st * 32 + kperm(n);
#pragma unroll
        for (int c = 0; c < S::DK; ++c) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + k_off<TQ, TKV, D>(krow, 2 * c + hh));
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[st], 0, 0, 0);
        }
      }
      // ---- masking: keys >= N and inactive logical blocks of the tile ----
      const bool ragged = cur_kv0 + TKV > N;
      if (ragged || wbits != full_kv) {
#pragma unroll
        for (int st = 0; st < S::NST; ++st)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kk = st * 32 + 16 * (v >> 3) + 8 * hh + (v & 7);
            const bool ok = (cur_kv0 + kk < N) && ((wbits >> (kk >> a.bkv_log2)) & 1u);
            if (!ok) s[st][v] = -INFINITY;
          }
      }
      // ---- online softmax (exp2 domain) ----------------------------------
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < S::NST; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[st][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * a.scale_log2);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < S::DB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[b][i] *= alpha;

      bf16x8 pf[S::NST][2];
#pragma unroll
      for (int st = 0; st < S::NST; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[st][v], a.scale_log2, -m_use));
          l_run += p;
          pf[st][v >> 3][v & 7] = (__bf16)p;
        }
      // ---- O^T += V^T P^T --------------------------------------------------
#pragma unroll
      for (int b = 0; b < S::DB; ++b)
#pragma unroll
        for (int st = 0; st < S::NST; ++st)
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
                vl + v_off<TQ, TKV, D>(b * 32 + n, st * 4 + c2 * 2 + hh));
            acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[st][c2], acc[b], 0, 0, 0);
          }
    }
    j = jn;
    kv0 = kvn;
  }

  // ---- epilogue ------------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const int r = w * 32 + n;  // row within the query tile
  if (task.slot < 0) {
    if (qrow < N) {
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      __bf16* op = a.o + head_off + (size_t)qrow * D;
#pragma unroll
      for (int b = 0; b < S::DB; ++b)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          bf16x4 ov;
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(acc[b][4 * jj + i] * inv);
          *reinterpret_cast<bf16x4*>(op + b * 32 + 8 * jj + 4 * hh) = ov;
        }
    }
  } else {
    const size_t sl = (size_t)task.slot;
    if (hh == 0) {
      a.ws_m[sl * TQ + r] = m_run;
      a.ws_l[sl * TQ + r] = l_tot;
    }
    float* wo = a.ws_o + sl * (size_t)D * TQ;
#pragma unroll
    for (int b = 0; b < S::DB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int dd = b * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
        wo[(size_t)dd * TQ + r] = acc[b][v];
      }
  }
}

template <int TQ, int TKV, int D>
hipError_t launch_attn(const AttnArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_fwd_kernel<TQ, TKV, D>), dim3(grid), dim3(TQ * 2), 0, s, a);
  return hipGetLastError();
}

}  // namespace bsa
