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
//  * Q stays in VGPRs (B operand) for the whole task.  K and V are staged in
//    LDS row-major with XOR swizzles on 16-byte chunks; K is read with
//    ds_read_b128 and V with the gfx950 transposing read ds_read_b64_tr_b16,
//    both bank-conflict free.  Tiles are fetched straight into LDS
//    (global_load_lds) one stage ahead of the tile being computed.
//  * Softmax runs in the exp2 domain: the exponent of a raw fp32 score s is
//    fma(s, log2(e)/sqrt(d), -m), one FMA per score, so Q and K enter the
//    MFMA unmodified; a fully masked row never produces NaN (running max -inf
//    is treated as 0 for the exponent offset) and ends with O = 0.
#pragma once

#include <type_traits>

#include "bsa_internal.h"

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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
  // LDS stages of the K/V pipeline: three (two tiles in flight while one is
  // computed) when three stages of a workgroup fit 48 KB, else two.
  static constexpr int NSTAGE = (3 * (KBYTES + VBYTES) <= 48 * 1024) ? 3 : 2;
  static_assert(CPT >= 1, "tile too small for the workgroup");
  static_assert(TQ % 32 == 0 && TKV % 32 == 0 && D % 32 == 0, "shape");
};

// 16-byte chunk swizzle of a row-major [rows][D] bf16 tile in LDS.  A 16-byte
// chunk's bank group is its byte address / 16 mod 16.  For D >= 128 (rows of
// 256 or 512 B, so the group is the chunk index mod 16) the two 2-bit fields
// of row%16 are swapped into the chunk index; for D=64 (two rows per 256 B)
// row/2 is XORed in; for D=32 (four rows per 256 B) (row/4)%4.  Both the
// QK^T A-operand reads (ds_read_b128, 16 consecutive permuted rows per lane
// group) and the PV transposed reads (ds_read_b64_tr_b16, 8 rows x 4 chunks
// per instruction half) then hit every 16-byte bank group at most the
// minimum number of times.
template <int D>
__device__ __forceinline__ int chunk_swz(int row) {
  if constexpr (D >= 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else if constexpr (D == 64) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}

template <int D>
__device__ __forceinline__ int tile_off(int row, int ch) {
  return row * (D * 2) + ((ch ^ chunk_swz<D>(row)) << 4);
}

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Value of lane (l ^ 32): v_permlane32_swap exchanges the upper half of one
// operand with the lower half of the other; swapping x with itself yields
// {x[l % 32]} in one result and {x[32 + l % 32]} in the other.
__device__ __forceinline__ float other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// s_waitcnt vmcnt(CNT) with the other counters left at their maximum (gfx9
// encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <class F, int... Is>
__device__ __forceinline__ void sfor_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void sfor(F&& f) {
  sfor_impl(f, std::make_integer_sequence<int, N>{});
}

// ds_read_b64_tr_b16 issued from inline assembly.  The compiler's own form of
// this read is treated as aliasing every in-flight global->LDS transfer and
// gets an s_waitcnt vmcnt(0) in front of it, which would serialize the K/V
// prefetch with the PV product.  The K/V stage being read was completed
// (counted vmcnt wait + workgroup barrier) before any read of it, so the
// prefetch into another stage cannot alias it.  Results must be fenced with
// lgkm_wait before use: the compiler does not know they are still in flight.
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16(uint32_t addr) {
  u32x2 r;
  if constexpr (OFF < 65536) {
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  } else {
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr + (uint32_t)OFF));
  }
  return r;
}

// ds_read_b128 from inline assembly, for the same reason: the K fragment
// reads then run several MFMAs ahead of their use with counted waits.
template <int OFF>
__device__ __forceinline__ u32x4 ds_read_b128(uint32_t addr) {
  u32x4 r;
  if constexpr (OFF < 65536) {
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  } else {
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr + (uint32_t)OFF));
  }
  return r;
}

// s_waitcnt lgkmcnt(CNT) that also ties the given registers, so no use of
// them can be scheduled above the wait.  LDS operations complete in issue
// order, so CNT = number of LDS reads issued after the ones being waited for.
template <int CNT, class Arr>
__device__ __forceinline__ void lgkm_wait(Arr& regs) {
  static_assert(CNT >= 0 && CNT < 16, "lgkmcnt field is 4 bits");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(CNT));
  constexpr int n = sizeof(Arr) / sizeof(u32x2);
  u32x2* r = reinterpret_cast<u32x2*>(&regs);
#pragma unroll
  for (int i = 0; i < n; ++i) asm volatile("" : "+v"(r[i]));
}

template <int CNT>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(CNT >= 0 && CNT < 64, "vmcnt field is 6 bits");
  __builtin_amdgcn_s_waitcnt((CNT & 15) | ((CNT >> 4) << 14) | 0x0F70);
}

// Entry-point choice (see the entry points below): 32-key tiles at d = 128
// with at most 128 queries run three waves per SIMD.
template <int TQ, int TKV, int D>
constexpr bool use_w3() { return TKV == 32 && D == 128 && TQ == 128; }
// 128x64 tiles at d = 128: registers capped at 256 so two workgroups (two
// waves per SIMD) fit a CU; uncapped the compiler takes 300 and one fits.
template <int TQ, int TKV, int D>
constexpr bool use_w2() { return TKV == 64 && D == 128 && TQ == 128; }
// K fragments read ahead of their MFMA.  Four fit every variant, the
// 168-register three-waves-per-SIMD one included; six spill there.
template <int TQ, int TKV, int D>
constexpr int kpf_depth() { return 4; }

template <int TQ, int TKV, int D>
__device__ __forceinline__ void attn_task(const AttnArgs& a, const Task task) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using S = AttnShape<TQ, TKV, D>;
  constexpr int STAGE = S::KBYTES + S::VBYTES;
  constexpr int LPW = S::KBYTES / 1024 / S::WAVES;  // 1 KB wave-loads per wave per operand
  static_assert(LPW >= 1 && LPW * 1024 * S::WAVES == S::KBYTES, "tile/wave split");
  constexpr int NSTAGE = S::NSTAGE;
  __shared__ __attribute__((aligned(1024))) unsigned char smem_arr[NSTAGE * STAGE];
  unsigned char* const smem = smem_arr;  // lambdas capture this pointer, not the array

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int n = lane & 31;   // query column within the wave (B operand / C column)
  const int hh = lane >> 5;  // lane half
  const int N = a.N;
  const int bat = task.head / a.heads;
  const size_t head_off = (size_t)bat * a.batch_stride + (size_t)(task.head - bat * a.heads) * a.head_stride;
  const int RS = a.row_stride;  // elements between consecutive rows
  const int qrow = task.qtile * TQ + w * 32 + n;

  // ---- Q fragment: B operand of S^T = K Q^T, resident for the task -------
  // Q enters the MFMA exactly as given (bf16): the scale log2(e)/sqrt(d) is
  // applied to the fp32 scores, so it adds no rounding of its own.  Rows past
  // N read row 0 (finite values, never written back).
  bf16x8 qf[S::DK];
  {
    const __bf16* qp = a.q + head_off + (size_t)(qrow < N ? qrow : 0) * RS + 8 * hh;
#pragma unroll
    for (int c = 0; c < S::DK; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qp + 16 * c);
  }
  const float scale = a.scale_log2;

  // membership: which logical sub-row of a coarsened tile this wave covers
  // Membership of a coarsened tile: bit a*coarsen_kv + b marks logical block
  // (a, b) of the tile active.  With B_Q >= 32 all 32 rows of a wave lie in
  // one logical row, sub_row; with B_Q = 16 they span rows 2w and 2w + 1
  // (lane n's row is 2w + n/16), so the skip test uses both rows' bits and
  // the masking is per lane.
  const bool lane_rows = a.bq < 32;
  const int sub_row = (a.coarsen_q > 1) ? (lane_rows ? 2 * w : (w * 32) / a.bq) : 0;
  const uint32_t full_kv = (a.coarsen_kv >= 32) ? 0xffffffffu : ((1u << a.coarsen_kv) - 1u);
  const uint32_t wave_kv = lane_rows ? (full_kv | (full_kv << a.coarsen_kv)) : full_kv;
  const int lane_shift = lane_rows ? (n >> 4) * a.coarsen_kv : 0;
  const uint32_t full_kv_all = 0xffffffffu;  // uncoarsened tiles: every block active

  // ---- online-softmax state (lane-local; l is a half-sum over this lane's keys)
  // m_run is the row's reference in log2 units: the maximum of the tile that
  // last moved it (see the softmax step).  The exponent of a raw score s is
  // fma(s, scale, negm) with negm = -m_run (0 while m_run = -inf, so a
  // masked score stays -inf).
  float m_run = -INFINITY;
  float negm = 0.0f;
  float l_run = 0.0f;
  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};
  const f32x16 zero16 = {};
  f32x16 acc[S::DB];
#pragma unroll
  for (int b = 0; b < S::DB; ++b) acc[b] = f32x16{};

  const int sub_log2 = a.sub_log2;
  const int total = (task.end - task.begin) << sub_log2;

  // Tile-list window: lane l holds entry wbase + l of the task's column list
  // (and its membership word), the next window is loaded one window ahead, so
  // looking an entry up is a v_readlane and never waits on memory inside the
  // loop.  Indices past the task's last entry are clamped (never used).
  const bool has_bits = a.tbits != nullptr;
  const int last_e = task.end - 1;
  int wbase = task.begin;
  auto load_win = [&](int base, int& col, uint32_t& bits) {
    const int e = min(base + lane, last_e);
    col = a.tcol[e];
    bits = has_bits ? a.tbits[e] : 0u;
  };
  int col_w = 0, col_x = 0;
  uint32_t bits_w = 0u, bits_x = 0u;
  if (total > 0) {
    load_win(wbase, col_w, bits_w);
    load_win(wbase + 64, col_x, bits_x);
  }
  // column and membership of entry e (e never decreases between calls)
  auto entry = [&](int e, int& col, uint32_t& bits) {
    if (e - wbase >= 64) {
      wbase += 64;
      col_w = col_x;
      bits_w = bits_x;
      load_win(wbase + 64, col_x, bits_x);
    }
    const int i = e - wbase;
    col = __builtin_amdgcn_readlane(col_w, i);
    bits = has_bits ? (uint32_t)__builtin_amdgcn_readlane((int)bits_w, i) : full_kv_all;
  };
  // Direct-to-LDS fetch of one K and one V tile into stage `buf`: wave-load i
  // of wave w fills 1 KB of the stage; lane l's 16 bytes land at byte 16*l of
  // it, so each lane fetches the (row, chunk) that the swizzle places there.
  // The per-lane byte offsets within a tile are fixed for the whole task.
  // Rows past N (only in the last tile of a row) are clamped to N-1: finite
  // data whose scores are masked to -inf.
  int goff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int slot = (i * S::WAVES + w) * 64 + lane;
    const int row = slot / S::KCH;
    goff[i] = row * (RS * 2) + (((slot % S::KCH) ^ chunk_swz<D>(row)) << 4);
  }
  const char* const kh = reinterpret_cast<const char*>(a.k + head_off);
  const char* const vh = reinterpret_cast<const char*>(a.v + head_off);
  // raw buffer descriptors over this head's K and V rows (bytes
  // [0, (N-1)*RS*2 + D*2); the host keeps N*RS*2 below 2^31)
  constexpr int kRsrcWord3 = 0x00020000;
  const int range = (N - 1) * (RS * 2) + D * 2;
  const __amdgpu_buffer_rsrc_t krsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kh), (short)0, range, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vh), (short)0, range, kRsrcWord3);
  auto issue = [&](int kv0, int buf) {
    unsigned char* kb = smem + buf * STAGE + w * 1024;
    unsigned char* vb = kb + S::KBYTES;
    const char* kt = kh + (size_t)kv0 * (RS * 2);
    const char* vt = vh + (size_t)kv0 * (RS * 2);
    if (kv0 + TKV <= N) {
      // buffer loads: head base in the descriptor, tile offset in an SGPR,
      // per-lane offset in a VGPR fixed for the task -- no address VALU work
      const int soff = kv0 * (RS * 2);
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (lds_void*)(kb + i * S::WAVES * 1024), 16, goff[i],
                                                 soff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, (lds_void*)(vb + i * S::WAVES * 1024), 16, goff[i],
                                                 soff, 0, 0);
      }
    } else {
      const int last = N - 1 - kv0;  // row N-1 within the tile
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int row = ((i * S::WAVES + w) * 64 + lane) / S::KCH;
        const int off = min(row, last) * (RS * 2) + (goff[i] - row * (RS * 2));
        __builtin_amdgcn_global_load_lds(kt + off, (lds_void*)(kb + i * S::WAVES * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vt + off, (lds_void*)(vb + i * S::WAVES * 1024), 16, 0, 0);
      }
    }
  };

  // K/V tile start of sub-tile j (entry begin + (j >> sub_log2)); refined
  // sub-tiles of the last logical column may start at or past N: they are
  // neither fetched nor computed.
  auto lookup = [&](int jj, int& kvs, uint32_t& bits) {
    int col;
    entry(task.begin + (jj >> sub_log2), col, bits);
    kvs = ((col << sub_log2) + (jj & ((1 << sub_log2) - 1))) * TKV;
  };
  // Tiles j .. j+NSTAGE-2 are in flight: kvq[i] / bitsq[i] describe tile
  // j+i (kvq = N: no such tile).
  int kvq[NSTAGE - 1];
  uint32_t bitsq[NSTAGE - 1];
  int j = 0;
#pragma unroll
  for (int i = 0; i < NSTAGE - 1; ++i) {
    kvq[i] = N;
    bitsq[i] = 0u;
    if (i < total) {
      lookup(i, kvq[i], bitsq[i]);
      if (kvq[i] < N) issue(kvq[i], i);
    }
  }

  // Per-lane LDS read bases.  Because the swizzle only XORs the chunk index,
  // each operand read is lane_base ^ (step << 5 or << 6) plus an immediate row
  // offset, so the loop needs three base registers and one XOR per step.
  //   K (A operand of S^T): row st*32 + kperm(n), chunk 2c + hh
  //   V (A operand of O^T, transposed read): row st*32 + c2*16 + 8*(g>>1) + 4r
  //     + ((lane&15)>>2), chunk 4b + 2*(g&1) + ((lane&3)>>1), half (lane&1),
  //     with g = lane/16 and r = 0/1 for key slots 0-3 / 4-7.
  const int krow0 = kperm(n);
  const int kbase = krow0 * (D * 2) + 16 * (hh ^ chunk_swz<D>(krow0));
  const int vgrp = lane >> 4;
  const int vch0 = 2 * (vgrp & 1) + ((lane & 3) >> 1);
  const int vrow0 = 8 * (vgrp >> 1) + ((lane & 15) >> 2);
  const int vbase0 = vrow0 * (D * 2) + 16 * (vch0 ^ chunk_swz<D>(vrow0)) + 8 * (lane & 1);
  const int vbase1 = (vrow0 + 4) * (D * 2) + 16 * (vch0 ^ chunk_swz<D>(vrow0 + 4)) + 8 * (lane & 1);
  // LDS byte addresses of the transposed V reads per d-block (the stage and
  // row offsets are added as instruction immediates)
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const lds_u8*)smem_arr;
  uint32_t kaddr[S::DK];
#pragma unroll
  for (int c = 0; c < S::DK; ++c) kaddr[c] = lds0 + (uint32_t)(kbase ^ (c << 5));
  uint32_t vaddr0[S::DB], vaddr1[S::DB];
#pragma unroll
  for (int b = 0; b < S::DB; ++b) {
    vaddr0[b] = lds0 + (uint32_t)(vbase0 ^ (b << 6));
    vaddr1[b] = lds0 + (uint32_t)(vbase1 ^ (b << 6));
  }

  // One K/V tile per step; the LDS stage index is a compile-time constant so
  // every LDS operand read uses an immediate offset (the loop is unrolled by
  // the two stages).
  auto step = [&](auto stage_c) {
    constexpr int buf = decltype(stage_c)::value;
    const int cur_kv0 = kvq[0];
    const uint32_t wbits = (bitsq[0] >> (sub_row * a.coarsen_kv)) & wave_kv;
    const int jn = j + NSTAGE - 1;
    int kvn = N;
    uint32_t bitsn = 0u;
    if (jn < total) lookup(jn, kvn, bitsn);

    // Wait for this wave's loads of tile j.  Vector-memory loads complete in
    // issue order, so it is enough that no more than the loads issued after
    // tile j's (tile j+1's, when three stages are in use) are outstanding.
    if constexpr (NSTAGE == 3) {
      if (kvq[1] < N) wait_vmcnt<2 * LPW>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();  // every wave's tile j landed; tile j-1 fully consumed
    if (kvn < N) issue(kvn, (buf + NSTAGE - 1) % NSTAGE);

    const lds_u8* kl = (const lds_u8*)(smem + buf * STAGE);
    const lds_u8* vl = kl + S::KBYTES;

    if (wbits != 0u && cur_kv0 < N) {
      // ---- S^T = K Q^T ---------------------------------------------------
      // K fragment i = (st, c) is read KPF fragments ahead of its MFMA.
      f32x16 s[S::NST];
      {
        constexpr int NK = S::NST * S::DK;
        constexpr int KPF = NK < kpf_depth<TQ, TKV, D>() ? NK : kpf_depth<TQ, TKV, D>();
        u32x4 kr[KPF];
        auto kread = [&](auto ic) {
          constexpr int i = decltype(ic)::value;
          kr[i % KPF] = ds_read_b128<buf * STAGE + (i / S::DK) * 32 * (D * 2)>(kaddr[i % S::DK]);
        };
        sfor<KPF>(kread);
        sfor<NK>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          constexpr int st = i / S::DK, c = i % S::DK;
          constexpr int later = (NK - 1 - i) < (KPF - 1) ? (NK - 1 - i) : (KPF - 1);
          lgkm_wait<later>(kr[i % KPF]);
          const bf16x8 kf = __builtin_bit_cast(bf16x8, kr[i % KPF]);
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], c == 0 ? zero16 : s[st], 0, 0, 0);
          if constexpr (i + KPF < NK) kread(std::integral_constant<int, i + KPF>{});
        });
      }
      // ---- masking: inactive logical blocks of the tile, keys >= N ---------
      // A 16-key group (st, v/8) never straddles a logical K/V block (B_KV >=
      // 16), so membership is one bit test per group: wave-uniform, or per
      // lane when the wave's rows span two logical rows.
      if (wbits != wave_kv) {
        if (!lane_rows) {
#pragma unroll
          for (int g = 0; g < 2 * S::NST; ++g) {
            if (!((wbits >> ((16 * g) >> a.bkv_log2)) & 1u)) {
#pragma unroll
              for (int v = 0; v < 8; ++v) s[g >> 1][8 * (g & 1) + v] = -INFINITY;
            }
          }
        } else {
          const uint32_t lbits = (wbits >> lane_shift) & full_kv;
#pragma unroll
          for (int g = 0; g < 2 * S::NST; ++g) {
            const bool off = !((lbits >> ((16 * g) >> a.bkv_log2)) & 1u);
#pragma unroll
            for (int v = 0; v < 8; ++v)
              s[g >> 1][8 * (g & 1) + v] = off ? -INFINITY : s[g >> 1][8 * (g & 1) + v];
          }
        }
      }
      if (cur_kv0 + TKV > N) {
        const int lim = N - cur_kv0 - 8 * hh;  // keys at or past N are masked
#pragma unroll
        for (int st = 0; st < S::NST; ++st)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (st * 32 + 16 * (v >> 3) + (v & 7) >= lim) s[st][v] = -INFINITY;
      }
      // ---- online softmax (exp2 domain, optimistic reference) -------------
      // Each score's exponent is fma(s, scale, -m_run) against the row's
      // reference m_run (log2 units).  The reference moves only when it must:
      // at the row's first active tile (no reference yet), or when this
      // tile's weights sum to more than 2^64 (a score about 59 or more above
      // the reference, or an exp overflow to infinity).  Then the tile's row
      // maximum becomes the reference, O and l are rescaled and the tile's
      // weights are recomputed.  Weights up to 2^64 lose nothing in bf16 P or
      // the fp32 sums, so the row maximum -- eight dependent v_max3, a lane
      // exchange and the compares -- is skipped on almost every tile.  l sums
      // the bf16-rounded weights that enter the PV product, two per v_dot2
      // against (1, 1), in two independent chains.
      bf16x8 pf[S::NST][2];
      float lt0 = 0.0f, lt1 = 0.0f;
      auto weights = [&]() {
#pragma unroll
        for (int st = 0; st < S::NST; ++st)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            pf[st][v >> 3][v & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[st][v], scale, negm));
        lt0 = 0.0f;
        lt1 = 0.0f;
#pragma unroll
        for (int st = 0; st < S::NST; ++st)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2 p0 = {pf[st][0][2 * e], pf[st][0][2 * e + 1]};
            const bf16x2 p1 = {pf[st][1][2 * e], pf[st][1][2 * e + 1]};
            lt0 = __builtin_amdgcn_fdot2_f32_bf16(p0, ones2, lt0, false);
            lt1 = __builtin_amdgcn_fdot2_f32_bf16(p1, ones2, lt1, false);
          }
      };
      bool redo = __builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0ull;
      if (!redo) {
        weights();
        redo = __builtin_amdgcn_ballot_w64(!(lt0 + lt1 <= 0x1p64f)) != 0ull;
      }
      if (redo) {
        // the row maximum is taken on the raw scores (the scale is positive)
        float mx = -INFINITY;
#pragma unroll
        for (int st = 0; st < S::NST; ++st)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[st][v]);
        mx = fmaxf(mx, other_half(mx)) * scale;
        const bool grow = mx > m_run;  // also at the first tile (m_run = -inf)
        const float alpha = (grow && m_run != -INFINITY) ? __builtin_amdgcn_exp2f(m_run - mx) : 1.0f;
        if (grow) m_run = mx;
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < S::DB; ++b) acc[b] *= alpha;
        negm = (m_run == -INFINITY) ? 0.0f : -m_run;
        weights();
      }
      l_run += lt0 + lt1;
      // ---- O^T += V^T P^T; V^T fragments via LDS transpose reads ----------
      // The product runs in chunks of (one 32-wide d-block) x (up to two
      // 32-key sub-tiles); the reads of chunk q+1 are in flight while the
      // MFMAs of chunk q run (two chunk buffers of at most 16 registers).
      constexpr int VOFF = buf * STAGE + S::KBYTES;  // V tile of this stage
      constexpr int NSTG = S::NST < 2 ? S::NST : 2;  // sub-tiles per chunk
      constexpr int NG = S::NST / NSTG;              // chunks per d-block
      constexpr int NQ = S::DB * NG;
      constexpr int NVR = NSTG * 2 * 2;              // transposed reads per chunk
      u32x2 vr[2][NSTG][2][2];
      auto vread = [&](auto qc, auto slot) {
        constexpr int q = decltype(qc)::value;
        constexpr int b = q / NG, g = q % NG;
        sfor<NSTG>([&](auto stc) {
          constexpr int sl = decltype(stc)::value;
          sfor<2>([&](auto c2c) {
            constexpr int c2 = decltype(c2c)::value;
            constexpr int off = VOFF + ((g * NSTG + sl) * 32 + c2 * 16) * (D * 2);
            vr[decltype(slot)::value][sl][c2][0] = ds_read_tr16<off>(vaddr0[b]);
            vr[decltype(slot)::value][sl][c2][1] = ds_read_tr16<off>(vaddr1[b]);
          });
        });
      };
      vread(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
      sfor<NQ>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        constexpr int b = q / NG, g = q % NG;
        constexpr int cur = q & 1;
        if constexpr (q + 1 < NQ) {
          vread(std::integral_constant<int, q + 1>{}, std::integral_constant<int, cur ^ 1>{});
          lgkm_wait<(NVR < 16 ? NVR : 15)>(vr[cur]);  // 15: also waits for one of q+1
        } else {
          lgkm_wait<0>(vr[cur]);
        }
        sfor<NSTG>([&](auto stc) {
          constexpr int sl = decltype(stc)::value;
          sfor<2>([&](auto c2c) {
            constexpr int c2 = decltype(c2c)::value;
            const u32x4 raw = {vr[cur][sl][c2][0][0], vr[cur][sl][c2][0][1], vr[cur][sl][c2][1][0],
                               vr[cur][sl][c2][1][1]};
            const bf16x8 vf = __builtin_bit_cast(bf16x8, raw);
            acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[g * NSTG + sl][c2], acc[b], 0, 0, 0);
          });
        });
      });
    }
#pragma unroll
    for (int i = 0; i + 1 < NSTAGE - 1; ++i) {
      kvq[i] = kvq[i + 1];
      bitsq[i] = bitsq[i + 1];
    }
    kvq[NSTAGE - 2] = kvn;
    bitsq[NSTAGE - 2] = bitsn;
    ++j;
  };
  for (int round = 0; round < total; round += NSTAGE) {
    step(std::integral_constant<int, 0>{});
    if (round + 1 < total) step(std::integral_constant<int, 1>{});
    if constexpr (NSTAGE == 3) {
      if (round + 2 < total) step(std::integral_constant<int, 2>{});
    }
  }

  // ---- epilogue ------------------------------------------------------------
  const float l_tot = l_run + other_half(l_run);
  const int r = w * 32 + n;  // row within the query tile
  if (task.slot < 0) {
    if (qrow < N) {
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      __bf16* op = a.o + head_off + (size_t)qrow * RS;
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
    // the partial output normalized by its own l, fp32, [d][T_Q] per slot:
    // each lane stores 4 bytes and a wave's 32 rows fill 128 contiguous bytes
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    float* wo = a.ws_o + sl * (size_t)D * TQ;
#pragma unroll
    for (int b = 0; b < S::DB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int dd = b * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
        wo[(size_t)dd * TQ + r] = acc[b][v] * inv;
      }
  }
#endif
}

// Tasks of queue y (the runs y, y + 8, ... of the XCD organization) with n
// tasks in all; position p of the queue is task ((p / C) * 8 + y) * C + p % C.
__device__ __forceinline__ int queue_len(long long n, int C, int y) {
  const long long rounds = n / (8LL * C), rem = n - rounds * 8LL * C;
  return (int)(rounds * C + min(max(rem - (long long)y * C, 0LL), (long long)C));
}
// The task of this workgroup (see launch_xq_init): in the static prefix of
// its queue (y = id mod 8, position id / 8) that position; past it, a claim
// on the front of its own queue's dynamic suffix, else on the back of the
// other queues' suffixes in turn; -1 when they are all empty.
__device__ __forceinline__ int claim_task(const AttnArgs& a) {
  const int C = a.xcd_remap;
  const long long n = (long long)*a.n_tasks;
  const int y0 = (int)(blockIdx.x & 7u), k = (int)(blockIdx.x >> 3);
  const int n0 = queue_len(n, C, y0);
  if (k < n0 - (n0 >> 3)) return ((k / C) * 8 + y0) * C + k % C;
#pragma unroll 1
  for (int j = 0; j < 8; ++j) {
    const int y = (y0 + j) & 7;
    const int ny = queue_len(n, C, y);
    const unsigned long long old = atomicAdd(&a.xq[y], j == 0 ? 1ull : 0xffffffff00000000ull);
    const int head = (int)(uint32_t)old, tail = (int)(uint32_t)(old >> 32);
    if (head < tail) {
      const int p = ny - (ny >> 3) + (j == 0 ? head : tail - 1);
      return ((p / C) * 8 + y) * C + p % C;
    }
  }
  return -1;
}

// Task dispatch: one task per workgroup -- in the task list's order, or for
// the XCD organizations through the per-XCD queues (a static prefix by
// workgroup id and a claimed tail; claim_task) -- or, with the stream
// organization (a separate instantiation, so the one-task kernels keep their
// register allocation), the workgroup's own run of tasks [seg_ptr[k],
// seg_ptr[k+1]), one after another.
template <int TQ, int TKV, int D, bool STREAM>
__device__ __forceinline__ void attn_fwd_body(const AttnArgs& a) {
  if constexpr (STREAM) {
    if (*a.n_tasks == 0ull) return;  // a guarded run that must do nothing
    const int t0 = a.seg_ptr[blockIdx.x], t1 = a.seg_ptr[blockIdx.x + 1];
    for (int t = t0; t < t1; ++t) {
      if (t > t0) __syncthreads();  // every wave is done with the previous task's LDS
      attn_task<TQ, TKV, D>(a, a.tasks[t]);
    }
  } else {
    // one task per workgroup: through the XCD queues, or by id (the static
    // remap over the XCDs when an XCD organization runs without queues)
    __shared__ int s_task;
    int t;
    if (a.xq) {
      if (threadIdx.x == 0) s_task = claim_task(a);
      __syncthreads();
      t = s_task;
      if (t < 0) return;
    } else {
      int bid = blockIdx.x;
      if (a.xcd_remap > 0) {
        // Workgroups are dealt to the 8 XCDs round-robin by id.  Remap so that
        // each XCD receives runs of xcd_remap consecutive tasks (neighbouring
        // query tiles of a head, which share K/V tiles in that XCD's L2), while
        // all XCDs still advance through the task list together.
        const int C = a.xcd_remap;
        const int s = bid >> 3;
        bid = (s / C) * (8 * C) + (bid & 7) * C + (s % C);
      }
      if ((unsigned long long)bid >= *a.n_tasks) return;
      t = bid;
    }
    attn_task<TQ, TKV, D>(a, a.tasks[t]);
  }
}

// Entry points: the generic kernel, the one for 32-key tiles at d = 128 with
// at most 128 queries, whose registers are capped at 168 so three waves fit a
// SIMD (the lower-occupancy schedule measured slower), and the one for 128x64
// tiles at d = 128, capped at 256 for two waves per SIMD (no spills).
template <int TQ, int TKV, int D, bool STREAM>
__global__ __launch_bounds__(TQ * 2) void attn_fwd_kernel(const AttnArgs a) {
  attn_fwd_body<TQ, TKV, D, STREAM>(a);
}
template <int TQ, int TKV, int D, bool STREAM>
__global__ __launch_bounds__(TQ * 2) __attribute__((amdgpu_waves_per_eu(3)))
__attribute__((amdgpu_num_vgpr(168))) void attn_fwd_kernel_w3(const AttnArgs a) {
  attn_fwd_body<TQ, TKV, D, STREAM>(a);
}
template <int TQ, int TKV, int D, bool STREAM>
__global__ __launch_bounds__(TQ * 2) __attribute__((amdgpu_waves_per_eu(2)))
__attribute__((amdgpu_num_vgpr(256))) void attn_fwd_kernel_w2(const AttnArgs a) {
  attn_fwd_body<TQ, TKV, D, STREAM>(a);
}
template <int TQ, int TKV, int D, bool STREAM>
void launch_attn_as(const AttnArgs& a, int grid, hipStream_t s) {
  if constexpr (use_w3<TQ, TKV, D>())
    hipLaunchKernelGGL((attn_fwd_kernel_w3<TQ, TKV, D, STREAM>), dim3(grid), dim3(TQ * 2), 0, s, a);
  else if constexpr (use_w2<TQ, TKV, D>())
    hipLaunchKernelGGL((attn_fwd_kernel_w2<TQ, TKV, D, STREAM>), dim3(grid), dim3(TQ * 2), 0, s, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<TQ, TKV, D, STREAM>), dim3(grid), dim3(TQ * 2), 0, s, a);
}
template <int TQ, int TKV, int D>
hipError_t launch_attn(const AttnArgs& a, int grid, hipStream_t s) {
  if (a.seg_ptr)
    launch_attn_as<TQ, TKV, D, true>(a, grid, s);
  else
    launch_attn_as<TQ, TKV, D, false>(a, grid, s);
  return hipGetLastError();
}

}  // namespace bsa
