// Planning kernels for gfx950: the shared mask state (block-CSR and scalar
// statistics) and the launch preparation of the selected plan.
//
// Tessera paper, section 5.2 "Regime lookup": the runtime builds the shared
// mask state mu(M) on the GPU -- block-CSR offsets, active K/V column indices
// and scalar statistics -- and transfers only the statistics to the host.
// Section 5.2 "Launch preparation": only the selected plan's metadata is
// derived from the shared block-CSR (tile membership for Coarsened plans,
// split-K partition information, traversal descriptors).
//
// All kernels are wave64; integer reductions use ballot/popcount and integer
// atomics only, so every result is deterministic.
#include "bsa_internal.h"

namespace bsa {
namespace {

__device__ inline unsigned lane_id() { return __lane_id(); }

__device__ inline unsigned prefix_count(unsigned long long ballot) {
  // number of set bits of `ballot` below this lane
  return __builtin_amdgcn_mbcnt_hi((unsigned)(ballot >> 32),
                                   __builtin_amdgcn_mbcnt_lo((unsigned)ballot, 0u));
}

__global__ void k_zero_stats(MaskStats* st) {
  if (threadIdx.x == 0) {
    st->nnz = 0;
    st->long_run = 0;
    st->max_row_nnz = 0;
    st->empty_rows = 0;
    st->n_tasks = 0;
  }
}

// One wave per query-block row: active count, and the number of active blocks
// whose left or right neighbour in the row is active (exactly the blocks that
// lie in runs of length >= 2, paper section 5.1).
__global__ __launch_bounds__(256) void k_row_count(const uint8_t* __restrict__ mask, int32_t nrows,
                                                   int32_t nkb, int32_t* __restrict__ row_cnt,
                                                   MaskStats* st) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= nrows) return;
  const unsigned l = lane_id();
  const uint8_t* row = mask + (size_t)wave * nkb;
  unsigned cnt = 0, lng = 0;
  for (int base = 0; base < nkb; base += 64) {
    const int p = base + (int)l;
    bool a = false, left = false, right = false;
    if (p < nkb) {
      a = row[p] != 0;
      left = p > 0 && row[p - 1] != 0;
      right = p + 1 < nkb && row[p + 1] != 0;
    }
    const unsigned long long ba = __ballot(a);
    const unsigned long long bl = __ballot(a && (left || right));
    cnt += __popcll(ba);
    lng += __popcll(bl);
  }
  if (l == 0) {
    row_cnt[wave] = (int32_t)cnt;
    if (lng) atomicAdd(&st->long_run, (unsigned long long)lng);
    atomicMax(&st->max_row_nnz, cnt);
    if (cnt == 0) atomicAdd(&st->empty_rows, 1u);
  }
}

// Exclusive scan of n int32 values by one workgroup of 1024 threads; out has
// n + 1 entries (out[n] = total); *total (if non-null) receives the total.
__global__ __launch_bounds__(1024) void k_scan(const int32_t* __restrict__ in,
                                               int32_t* __restrict__ out, int32_t n,
                                               unsigned long long* total) {
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int b = t * per;
  const int e = min(n, b + per);
  int32_t s = 0;
  for (int i = b; i < e; ++i) s += in[i];
  part[t] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 partial sums
  for (int off = 1; off < 1024; off <<= 1) {
    int32_t v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int32_t run = t > 0 ? part[t - 1] : 0;
  for (int i = b; i < e; ++i) {
    out[i] = run;
    run += in[i];
  }
  if (t == 1023) {
    out[n] = part[1023];
    if (total) *total = (unsigned long long)part[1023];
  }
}

// One wave per query-block row: write the active column indices, ascending.
__global__ __launch_bounds__(256) void k_compact(const uint8_t* __restrict__ mask, int32_t nrows,
                                                 int32_t nkb, const int32_t* __restrict__ row_ptr,
                                                 int32_t* __restrict__ cols) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= nrows) return;
  const unsigned l = lane_id();
  const uint8_t* row = mask + (size_t)wave * nkb;
  int32_t out = row_ptr[wave];
  for (int base = 0; base < nkb; base += 64) {
    const int p = base + (int)l;
    const bool a = p < nkb && row[p] != 0;
    const unsigned long long ba = __ballot(a);
    if (a) cols[out + (int)prefix_count(ba)] = p;
    out += __popcll(ba);
  }
}

// Coarsened tile list: tile row tr of head h covers logical rows
// [tr*cq, tr*cq + cq) and tile column tc covers logical columns
// [tc*ckv, tc*ckv + ckv).  A tile exists iff one of its blocks is active;
// its membership bit a*ckv + b is set iff logical block
// (tr*cq + a, tc*ckv + b) is active (paper section 4.2, "Coarsened").
// One workgroup per tile row; the row's union is built in an LDS bitmap.
// With trow_ptr == nullptr the kernel writes counts, else the tile entries.
__global__ __launch_bounds__(256) void k_coarsen(const int32_t* __restrict__ row_ptr,
                                                 const int32_t* __restrict__ cols, int32_t nqb,
                                                 int32_t cq, int32_t ckv, int32_t ntr,
                                                 int32_t ntc, int32_t* __restrict__ trow_cnt,
                                                 const int32_t* __restrict__ trow_ptr,
                                                 int32_t* __restrict__ tcol,
                                                 uint32_t* __restrict__ tbits) {
  extern __shared__ uint32_t bitmap[];
  __shared__ int32_t wave_tot[4];
  const int g = blockIdx.x;  // h * ntr + tr
  const int h = g / ntr;
  const int tr = g - h * ntr;
  for (int i = threadIdx.x; i < ntc; i += 256) bitmap[i] = 0u;
  __syncthreads();
  for (int a = 0; a < cq; ++a) {
    const int r = tr * cq + a;
    if (r >= nqb) break;
    const int rr = h * nqb + r;
    const int b = row_ptr[rr], e = row_ptr[rr + 1];
    for (int i = b + threadIdx.x; i < e; i += 256) {
      const int c = cols[i];
      const int tc = c / ckv;
      atomicOr(&bitmap[tc], 1u << (a * ckv + (c - tc * ckv)));
    }
  }
  __syncthreads();
  const unsigned l = lane_id();
  const int w = threadIdx.x >> 6;
  if (!trow_ptr) {
    int cnt = 0;
    for (int i = threadIdx.x; i < ntc; i += 256) cnt += bitmap[i] != 0u;
    // wave reduction then workgroup reduction
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    if (l == 0) wave_tot[w] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) trow_cnt[g] = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    return;
  }
  // ordered compaction: process the bitmap in chunks of 256 entries
  int32_t out = trow_ptr[g];
  for (int base = 0; base < ntc; base += 256) {
    const int i = base + threadIdx.x;
    const uint32_t bits = i < ntc ? bitmap[i] : 0u;
    const unsigned long long bal = __ballot(bits != 0u);
    if (l == 0) wave_tot[w] = __popcll(bal);
    __syncthreads();
    int before = 0;
    for (int k = 0; k < w; ++k) before += wave_tot[k];
    const int total = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    if (bits) {
      const int pos = out + before + (int)prefix_count(bal);
      tcol[pos] = i;
      tbits[pos] = bits;
    }
    out += total;
    __syncthreads();
  }
}

// Split-K partition count per query tile (paper section 4.3, "Split-K"):
// a query tile whose tile-list row holds more than `split` entries is cut into
// ceil(n / split) partitions of near-equal size; split == 0 never splits.
// parts[q] = partitions (>= 1; a tile with no entries still gets one task that
// writes zeros), slots[q] = workspace slots (parts if split, else 0).
__global__ __launch_bounds__(256) void k_task_count(const int32_t* __restrict__ trow_ptr,
                                                    int32_t H, int32_t nqt_head, int32_t ntr,
                                                    int32_t refine_q, int32_t split,
                                                    int32_t* __restrict__ parts,
                                                    int32_t* __restrict__ slots) {
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g >= H * nqt_head) return;
  const int h = g / nqt_head;
  const int qt = g - h * nqt_head;
  const int tr = qt / refine_q;
  const int n = trow_ptr[h * ntr + tr + 1] - trow_ptr[h * ntr + tr];
  const int p = (split > 0 && n > split) ? (n + split - 1) / split : 1;
  parts[g] = p;
  slots[g] = p > 1 ? p : 0;
}

__global__ __launch_bounds__(256) void k_task_write(const int32_t* __restrict__ trow_ptr,
                                                    int32_t H, int32_t nqt_head, int32_t ntr,
                                                    int32_t refine_q,
                                                    const int32_t* __restrict__ parts,
                                                    const int32_t* __restrict__ task_off,
                                                    const int32_t* __restrict__ slot_off,
                                                    Task* __restrict__ tasks) {
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g >= H * nqt_head) return;
  const int h = g / nqt_head;
  const int qt = g - h * nqt_head;
  const int tr = qt / refine_q;
  const int b = trow_ptr[h * ntr + tr];
  const int e = trow_ptr[h * ntr + tr + 1];
  const int p = parts[g];
  const int n = e - b;
  const int chunk = (n + p - 1) / p;
  const int t0 = task_off[g];
  for (int i = 0; i < p; ++i) {
    Task t;
    t.head = h;
    t.qtile = qt;
    t.begin = min(e, b + i * chunk);
    t.end = min(e, b + (i + 1) * chunk);
    t.slot = p > 1 ? slot_off[g] + i : -1;
    t.pad0 = t.pad1 = t.pad2 = 0;
    tasks[t0 + i] = t;
  }
}

}  // namespace

hipError_t launch_zero_stats(MaskStats* st, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_stats, dim3(1), dim3(64), 0, s, st);
  return hipGetLastError();
}

hipError_t launch_row_count(const uint8_t* mask, int32_t nrows, int32_t nkb, int32_t* row_cnt,
                            MaskStats* st, hipStream_t s) {
  hipLaunchKernelGGL(k_row_count, dim3((nrows + 3) / 4), dim3(256), 0, s, mask, nrows, nkb,
                     row_cnt, st);
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* in, int32_t* out, int32_t n, unsigned long long* total,
                       hipStream_t s) {
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, in, out, n, total);
  return hipGetLastError();
}

hipError_t launch_compact(const uint8_t* mask, int32_t nrows, int32_t nkb, const int32_t* row_ptr,
                          int32_t* cols, hipStream_t s) {
  hipLaunchKernelGGL(k_compact, dim3((nrows + 3) / 4), dim3(256), 0, s, mask, nrows, nkb, row_ptr,
                     cols);
  return hipGetLastError();
}

hipError_t launch_coarsen(const int32_t* row_ptr, const int32_t* cols, int32_t H, int32_t nqb,
                          int32_t nkb, int32_t cq, int32_t ckv, int32_t ntr, int32_t ntc,
                          int32_t* trow_cnt, const int32_t* trow_ptr, int32_t* tcol,
                          uint32_t* tbits, hipStream_t s) {
  (void)nkb;
  const size_t lds = (size_t)ntc * sizeof(uint32_t);
  hipLaunchKernelGGL(k_coarsen, dim3(H * ntr), dim3(256), lds, s, row_ptr, cols, nqb, cq, ckv, ntr,
                     ntc, trow_cnt, trow_ptr, tcol, tbits);
  return hipGetLastError();
}

hipError_t launch_task_count(const int32_t* trow_ptr, int32_t H, int32_t nqt_head, int32_t ntr,
                             int32_t refine_q, int32_t split, int32_t* parts, int32_t* slots,
                             hipStream_t s) {
  const int n = H * nqt_head;
  hipLaunchKernelGGL(k_task_count, dim3((n + 255) / 256), dim3(256), 0, s, trow_ptr, H, nqt_head,
                     ntr, refine_q, split, parts, slots);
  return hipGetLastError();
}

hipError_t launch_task_write(const int32_t* trow_ptr, int32_t H, int32_t nqt_head, int32_t ntr,
                             int32_t refine_q, const int32_t* parts, const int32_t* task_off,
                             const int32_t* slot_off, Task* tasks, hipStream_t s) {
  const int n = H * nqt_head;
  hipLaunchKernelGGL(k_task_write, dim3((n + 255) / 256), dim3(256), 0, s, trow_ptr, H, nqt_head,
                     ntr, refine_q, parts, task_off, slot_off, tasks);
  return hipGetLastError();
}

}  // namespace bsa
