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
// All kernels are wave64; reductions use ballot/popcount, LDS and integer
// atomics only, so every result is deterministic.
#include <algorithm>

#include "bsa_internal.h"

namespace bsa {
namespace {

__device__ inline unsigned lane_id() { return __lane_id(); }

__device__ inline unsigned prefix_count(unsigned long long ballot) {
  // number of set bits of `ballot` below this lane
  return __builtin_amdgcn_mbcnt_hi((unsigned)(ballot >> 32),
                                   __builtin_amdgcn_mbcnt_lo((unsigned)ballot, 0u));
}

// Hand-over of a record to the host through fine-grained host memory: the
// fields are written with system-scope (write-through) stores, the wave waits
// until they have completed (s_waitcnt vmcnt(0)), and only then stores the
// sequence number that the host spins on.  A system-scope release would in
// addition write back every dirty line of the XCD's L2 (buffer_wbl2), which
// costs microseconds after a kernel that wrote megabytes and which the host,
// reading only this record, does not need.
template <class T>
__device__ inline void sys_store(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ inline void sys_publish_seq(unsigned long long* p, unsigned long long seq) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the field stores have completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  sys_store(p, seq);
}
__device__ inline void publish_stats(MaskStats* h, const MaskStats& r) {
  sys_store(&h->nnz, r.nnz);
  sys_store(&h->long_run, r.long_run);
  sys_store(&h->max_row_nnz, r.max_row_nnz);
  sys_store(&h->empty_rows, r.empty_rows);
  sys_store(&h->n_tasks, 0ull);
  sys_store(&h->n_split, 0ull);
  sys_publish_seq(&h->seq, r.seq);
}

// Active count per query-block row, and per-workgroup partial statistics:
// active blocks lying in runs of length >= 2 (an active block whose left or
// right neighbour in the row is active; paper section 5.1), the largest row
// count and the number of empty rows.  Each wave walks whole rows
// (grid-stride), one byte per lane per 64-column chunk; the neighbour tests
// are shifts of the chunk's ballot, carried across chunk boundaries.
__global__ __launch_bounds__(256) void k_row_count(const uint8_t* __restrict__ mask, int32_t nrows,
                                                   int32_t nkb, int32_t* __restrict__ row_cnt,
                                                   RowPartial* __restrict__ part) {
  __shared__ unsigned long long s_long[4];
  __shared__ unsigned s_max[4], s_empty[4];
  const unsigned l = lane_id();
  const int wv = threadIdx.x >> 6;
  unsigned long long lng_w = 0;
  unsigned max_w = 0, empty_w = 0;
  const int nwaves = gridDim.x * 4;
  for (int row = blockIdx.x * 4 + wv; row < nrows; row += nwaves) {
    const uint8_t* r = mask + (size_t)row * nkb;
    unsigned cnt = 0, lng = 0;
    unsigned long long prev = 0;  // ballot of the previous chunk (bit 63 = its last column)
    unsigned long long cur = __ballot((int)l < nkb && r[l] != 0);
    for (int base = 0; base < nkb; base += 64) {
      const int p = base + 64 + (int)l;
      const unsigned long long next = (base + 64 < nkb) ? __ballot(p < nkb && r[p] != 0) : 0ull;
      const unsigned long long left = (cur << 1) | (prev >> 63);
      const unsigned long long right = (cur >> 1) | (next << 63);
      cnt += __popcll(cur);
      lng += __popcll(cur & (left | right));
      prev = cur;
      cur = next;
    }
    if (l == 0) row_cnt[row] = (int32_t)cnt;
    lng_w += lng;
    max_w = max(max_w, cnt);
    empty_w += (cnt == 0);
  }
  if (l == 0) {
    s_long[wv] = lng_w;
    s_max[wv] = max_w;
    s_empty[wv] = empty_w;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    RowPartial rp;
    rp.long_run = s_long[0] + s_long[1] + s_long[2] + s_long[3];
    rp.max_row = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
    rp.empty = s_empty[0] + s_empty[1] + s_empty[2] + s_empty[3];
    part[blockIdx.x] = rp;
  }
}

// Inclusive scan of one int32 per lane across the wave (64 lanes).
__device__ inline int32_t wave_scan(int32_t x) {
  const int l = (int)lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off, 64);
    if (l >= off) x += y;
  }
  return x;
}

// Block-wide exclusive scan of one int32 per thread (1024 threads = 16
// waves); returns the exclusive prefix and sets *tot to the block total.
// Uses lds[0..31]; consecutive calls need no barrier in between.
__device__ int32_t block_scan(int32_t v, int32_t* lds, int32_t* tot) {
  const int t = threadIdx.x;
  const int l = t & 63, w = t >> 6;
  const int32_t x = wave_scan(v);
  if (l == 63) lds[w] = x;
  __syncthreads();
  if (w == 0) {
    const int32_t s = wave_scan(l < 16 ? lds[l] : 0);
    if (l < 16) lds[16 + l] = s;
  }
  __syncthreads();
  *tot = lds[31];
  return (w > 0 ? lds[15 + w] : 0) + x - v;
}

// Exclusive scan of n int32 values by one workgroup of 1024 threads; out has
// n + 1 entries (out[n] = total).  The input is walked in coalesced tiles of
// 4096 values (four consecutive values per thread).  With `st` non-null the
// kernel also completes the mask statistics: nnz = total, the reduction of
// the row-count kernel's `npart` partials, and n_tasks = 0.
__global__ __launch_bounds__(1024) void k_scan(const int32_t* __restrict__ in,
                                               int32_t* __restrict__ out, int32_t n,
                                               const RowPartial* __restrict__ part, int32_t npart,
                                               MaskStats* st, MaskStats* host_st,
                                               unsigned long long seq) {
  __shared__ int32_t lds[32];
  const int t = threadIdx.x;
  int32_t carry = 0;
  for (int base = 0; base < n; base += 4096) {
    const int i0 = base + 4 * t;
    int32_t v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = (i0 + k < n) ? in[i0 + k] : 0;
    int32_t tot;
    int32_t run = carry + block_scan(v[0] + v[1] + v[2] + v[3], lds, &tot);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (i0 + k < n) out[i0 + k] = run;
      run += v[k];
    }
    carry += tot;
  }
  if (t == 0) out[n] = carry;
  if (st) {
    // reduce the partial statistics: thread t folds partials t, t+1024, ...,
    // then a butterfly per wave and one thread over the 16 wave results
    __shared__ unsigned long long s_long[16];
    __shared__ unsigned s_max[16], s_empty[16];
    unsigned long long lg = 0;
    unsigned mx = 0, em = 0;
    for (int i = t; i < npart; i += 1024) {
      lg += part[i].long_run;
      mx = max(mx, part[i].max_row);
      em += part[i].empty;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      lg += __shfl_xor(lg, off, 64);
      mx = max(mx, (unsigned)__shfl_xor((int)mx, off, 64));
      em += (unsigned)__shfl_xor((int)em, off, 64);
    }
    if ((t & 63) == 0) {
      s_long[t >> 6] = lg;
      s_max[t >> 6] = mx;
      s_empty[t >> 6] = em;
    }
    __syncthreads();
    if (t == 0) {
      for (int w = 1; w < 16; ++w) {
        s_long[0] += s_long[w];
        s_max[0] = max(s_max[0], s_max[w]);
        s_empty[0] += s_empty[w];
      }
    }
    if (t == 0) {
      MaskStats r;
      r.nnz = (unsigned long long)carry;
      r.long_run = s_long[0];
      r.max_row_nnz = s_max[0];
      r.empty_rows = s_empty[0];
      r.n_tasks = 0;
      r.n_split = 0;
      r.seq = seq;
      *st = r;
      // fine-grained host memory, read by the host while this stream runs on
      if (host_st) publish_stats(host_st, r);
    }
  }
}

// One wave per query-block row: write the active column indices, ascending.
__global__ __launch_bounds__(256) void k_compact(const uint8_t* __restrict__ mask, int32_t nrows,
                                                 int32_t nkb, const int32_t* __restrict__ row_ptr,
                                                 int32_t* __restrict__ cols, int32_t* __restrict__ rsig) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= nrows) return;
  const unsigned l = lane_id();
  const uint8_t* row = mask + (size_t)wave * nkb;
  int32_t out = row_ptr[wave];
  const int32_t mid = (out + row_ptr[wave + 1] - 1) >> 1;  // the row's median entry
  for (int base = 0; base < nkb; base += 64) {
    const int p = base + (int)l;
    const bool a = p < nkb && row[p] != 0;
    const unsigned long long ba = __ballot(a);
    if (a) {
      const int32_t o = out + (int)prefix_count(ba);
      cols[o] = p;
      if (o == mid) rsig[wave] = p;
    }
    out += __popcll(ba);
  }
}

// Row bits of a 16-byte aligned mask, 16 columns per lane: the row's bytes
// [start, start + nkb) are covered by the aligned 16-byte chunks from a0 =
// start & ~15; window w holds chunks a0 + 1024 w + 16 l (lane l).  Bit i of a
// lane's value is byte (chunk + i) != 0, with bytes outside the row cleared.
// A chunk that would cross the end of the mask buffer is read bytewise.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

__device__ inline uint32_t nz_bits16(const u32x4v x);

__device__ inline uint32_t row_chunk_bits(const uint8_t* __restrict__ mask, size_t total, size_t start,
                                          int nkb, size_t a0, int w, int lane) {
  const size_t c = a0 + (size_t)w * 1024 + 16 * (size_t)lane;
  const size_t end = start + (size_t)nkb;
  if (c >= end) return 0u;
  uint32_t m;
  if (c + 16 <= total) {
    m = nz_bits16(*reinterpret_cast<const u32x4v*>(mask + c));
  } else {
    m = 0u;
    for (int i = 0; c + i < total; ++i) m |= (uint32_t)(mask[c + i] != 0) << i;
  }
  if (c < start) m &= 0xffffu << (unsigned)(start - c);
  if (c + 16 > end) m &= (1u << (unsigned)(end - c)) - 1u;
  return m & 0xffffu;
}

// k_row_count for a 16-byte aligned mask (same outputs): a wave per row reads
// the row 1 KB per load; run neighbours cross lanes by shuffles and windows
// by carrying the previous window's last bit and peeking the next window's
// first.
__global__ __launch_bounds__(256) void k_row_count16(const uint8_t* __restrict__ mask, int32_t nrows,
                                                     int32_t nkb, int32_t* __restrict__ row_cnt,
                                                     RowPartial* __restrict__ part) {
  __shared__ unsigned long long s_long[4];
  __shared__ unsigned s_max[4], s_empty[4];
  const int l = (int)lane_id();
  const int wv = threadIdx.x >> 6;
  const size_t total = (size_t)nrows * (size_t)nkb;
  unsigned long long lng_w = 0;
  unsigned max_w = 0, empty_w = 0;
  const int nwaves = gridDim.x * 4;
  for (int row = blockIdx.x * 4 + wv; row < nrows; row += nwaves) {
    const size_t start = (size_t)row * (size_t)nkb;
    const size_t a0 = start & ~(size_t)15;
    const int nwin = (int)((start + nkb - a0 + 1023) / 1024);
    unsigned cnt = 0, lng = 0, prevtop = 0u;
    uint32_t cur = row_chunk_bits(mask, total, start, nkb, a0, 0, l);
    for (int w = 0; w < nwin; ++w) {
      const uint32_t nxt = (w + 1 < nwin) ? row_chunk_bits(mask, total, start, nkb, a0, w + 1, l) : 0u;
      const uint32_t up = (uint32_t)__shfl_up((int)cur, 1, 64);
      const uint32_t dn = (uint32_t)__shfl_down((int)cur, 1, 64);
      const uint32_t nxt0 = (uint32_t)__shfl((int)nxt, 0, 64);
      const uint32_t top = (uint32_t)__shfl((int)cur, 63, 64);
      const uint32_t lbit = l == 0 ? prevtop : ((up >> 15) & 1u);
      const uint32_t rbit = l == 63 ? (nxt0 & 1u) : (dn & 1u);
      const uint32_t left = ((cur << 1) | lbit) & 0xffffu;
      const uint32_t right = (cur >> 1) | (rbit << 15);
      cnt += __popc(cur);
      lng += __popc(cur & (left | right));
      prevtop = (top >> 15) & 1u;
      cur = nxt;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      cnt += (unsigned)__shfl_xor((int)cnt, o, 64);
      lng += (unsigned)__shfl_xor((int)lng, o, 64);
    }
    if (l == 0) row_cnt[row] = (int32_t)cnt;
    lng_w += lng;
    max_w = max(max_w, cnt);
    empty_w += (cnt == 0);
  }
  if (l == 0) {
    s_long[wv] = lng_w;
    s_max[wv] = max_w;
    s_empty[wv] = empty_w;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    RowPartial rp;
    rp.long_run = s_long[0] + s_long[1] + s_long[2] + s_long[3];
    rp.max_row = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
    rp.empty = s_empty[0] + s_empty[1] + s_empty[2] + s_empty[3];
    part[blockIdx.x] = rp;
  }
}

// k_compact for a 16-byte aligned mask (same outputs): a wave per row, 16
// columns per lane per window, lane offsets by a wave scan of the lanes' bit
// counts.
__global__ __launch_bounds__(256) void k_compact16(const uint8_t* __restrict__ mask, int32_t nrows,
                                                   int32_t nkb, const int32_t* __restrict__ row_ptr,
                                                   int32_t* __restrict__ cols, int32_t* __restrict__ rsig) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= nrows) return;
  const int l = (int)lane_id();
  const size_t total = (size_t)nrows * (size_t)nkb;
  const size_t start = (size_t)row * (size_t)nkb;
  const size_t a0 = start & ~(size_t)15;
  const int nwin = (int)((start + nkb - a0 + 1023) / 1024);
  int32_t out = row_ptr[row];
  const int32_t mid = (out + row_ptr[row + 1] - 1) >> 1;  // the row's median entry
  for (int w = 0; w < nwin; ++w) {
    uint32_t m = row_chunk_bits(mask, total, start, nkb, a0, w, l);
    const int32_t c = (int32_t)__popc(m);
    const int32_t incl = wave_scan(c);
    int32_t o = out + incl - c;
    const int32_t base = (int32_t)(a0 + (size_t)w * 1024 + 16 * (size_t)l - start);  // column of bit 0
    while (m) {
      const int32_t col = base + __ffs(m) - 1;
      if (o == mid) rsig[row] = col;
      cols[o++] = col;
      m &= m - 1u;
    }
    out += __shfl(incl, 63, 64);
  }
}

// Bit i (i < 4) set iff byte i of x is nonzero: per byte, adding 0x7f to
// its low seven bits sets bit 7 iff they are nonzero (no carry leaves the
// byte), OR-ing x adds its own bit 7; the four byte flags are then gathered.
__device__ inline uint32_t nz_bits4(uint32_t x) {
  const uint32_t y = (((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x) & 0x80808080u;
  return ((y >> 7) | (y >> 14) | (y >> 21) | (y >> 28)) & 0xfu;
}

__device__ inline uint32_t nz_bits16(const u32x4v x) {
  return nz_bits4(x[0]) | (nz_bits4(x[1]) << 4) | (nz_bits4(x[2]) << 8) | (nz_bits4(x[3]) << 12);
}

// The whole mask state of a small mask in one launch (one workgroup of 1024):
// the mask is packed into a bitmap in LDS (one 32-bit word of 32 consecutive
// mask bytes per thread, from two 16-byte loads), then one thread per
// query-block row counts its active blocks and those with an active left or
// right neighbour, the counts are scanned into row_ptr, the statistics are
// stored (and published to the host, sequence number last), and only then
// are the columns compacted from the bitmap, so the host's plan selection
// overlaps the compaction.  Same outputs as k_row_count + k_scan + k_compact.
template <int TPT>
__device__ __forceinline__ void build_tasks(const int32_t* trow_ptr, int32_t H, int32_t nqt_head, int32_t ntr, int32_t refine_q,
                            int32_t split, int32_t split_min, int32_t order, int32_t max_len, int32_t* __restrict__ parts,
                            int32_t* __restrict__ slot_base, Task* __restrict__ tasks, MaskStats* st,
                            int32_t dev_split, int32_t slots, int32_t* __restrict__ split_tiles,
                            unsigned long long stat_nnz, unsigned stat_max_row,
                            const int32_t* __restrict__ tsig = nullptr, int32_t ncol = 0);

__global__ __launch_bounds__(1024) void k_mask_small(const uint8_t* __restrict__ mask, int32_t nrows,
                                                     int32_t nkb, int32_t* __restrict__ row_ptr,
                                                     int32_t* __restrict__ cols, int32_t* __restrict__ rsig,
                                                     MaskStats* st, MaskStats* host_st, unsigned long long seq,
                                                     const TaskSpec spec) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __shared__ uint32_t bits[kSmallMaskBytes / 32 + 1];  // + a zero word read past the last row
  __shared__ int32_t off[kSmallMaskRows + 1];
  __shared__ unsigned long long s_nnz;
  __shared__ unsigned s_maxrow;
  __shared__ int32_t lds[32];
  __shared__ unsigned long long s_long[16];
  __shared__ unsigned s_max[16], s_empty[16];
  const int t = threadIdx.x;
  const int bytes = nrows * nkb;
  const int nwords = (bytes + 31) >> 5;
  // pack (the host only picks this kernel for a 16-byte aligned mask)
  for (int i = t; i < nwords; i += 1024) {
    const int b0 = i << 5;
    uint32_t w = 0;
    if (b0 + 32 <= bytes) {
      const u32x4 x = reinterpret_cast<const u32x4*>(mask + b0)[0];
      const u32x4 y = reinterpret_cast<const u32x4*>(mask + b0)[1];
      w = nz_bits4(x[0]) | (nz_bits4(x[1]) << 4) | (nz_bits4(x[2]) << 8) | (nz_bits4(x[3]) << 12) |
          (nz_bits4(y[0]) << 16) | (nz_bits4(y[1]) << 20) | (nz_bits4(y[2]) << 24) | (nz_bits4(y[3]) << 28);
    } else {
      for (int j = 0; b0 + j < bytes; ++j) w |= (uint32_t)(mask[b0 + j] != 0) << j;
    }
    bits[i] = w;
  }
  if (t == 0) bits[nwords] = 0u;
  __syncthreads();
  // columns [32k, 32k + 32) of row r, zero past nkb
  auto row_word = [&](int r, int k) -> uint32_t {
    const int c0 = k << 5;
    const int b = r * nkb + c0;
    const int wi = b >> 5, sh = b & 31;
    uint32_t v = bits[wi] >> sh;
    if (sh) v |= bits[wi + 1] << (32 - sh);
    const int rem = nkb - c0;
    if (rem < 32) v &= (1u << rem) - 1u;
    return v;
  };
  const int nw = (nkb + 31) >> 5;
  // per-row counts and run statistics, one thread per row
  unsigned long long lng_t = 0;
  unsigned max_t = 0, empty_t = 0;
  for (int r = t; r < nrows; r += 1024) {
    unsigned cnt = 0, lng = 0;
    uint32_t prev = 0u, cur = row_word(r, 0);
    for (int k = 0; k < nw; ++k) {
      const uint32_t next = k + 1 < nw ? row_word(r, k + 1) : 0u;
      const uint32_t left = (cur << 1) | (prev >> 31);
      const uint32_t right = (cur >> 1) | (next << 31);
      cnt += __popc(cur);
      lng += __popc(cur & (left | right));
      prev = cur;
      cur = next;
    }
    off[r] = (int32_t)cnt;
    lng_t += lng;
    max_t = max(max_t, cnt);
    empty_t += (cnt == 0);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lng_t += __shfl_xor(lng_t, o, 64);
    max_t = max(max_t, (unsigned)__shfl_xor((int)max_t, o, 64));
    empty_t += (unsigned)__shfl_xor((int)empty_t, o, 64);
  }
  if ((t & 63) == 0) {
    s_long[t >> 6] = lng_t;
    s_max[t >> 6] = max_t;
    s_empty[t >> 6] = empty_t;
  }
  __syncthreads();
  // exclusive scan of the counts (in place in LDS, and to row_ptr)
  int32_t carry = 0;
  for (int base = 0; base < nrows; base += 1024) {
    const int i = base + t;
    const int32_t v = i < nrows ? off[i] : 0;
    int32_t tot;
    const int32_t ex = carry + block_scan(v, lds, &tot);
    if (i < nrows) {
      off[i] = ex;
      row_ptr[i] = ex;
    }
    carry += tot;
  }
  if (t == 0) {
    row_ptr[nrows] = carry;
    MaskStats r;
    r.nnz = (unsigned long long)carry;
    r.long_run = 0;
    r.max_row_nnz = 0;
    r.empty_rows = 0;
    for (int w = 0; w < 16; ++w) {
      r.long_run += s_long[w];
      r.max_row_nnz = max(r.max_row_nnz, s_max[w]);
      r.empty_rows += s_empty[w];
    }
    r.n_tasks = 0;
    r.n_split = 0;
    r.seq = seq;
    *st = r;
    if (host_st) publish_stats(host_st, r);
    off[nrows] = carry;
    s_nnz = r.nnz;
    s_maxrow = r.max_row_nnz;
  }
  if (spec.enabled) {
    // the speculative task list, from the row offsets in LDS
    __syncthreads();
    build_tasks<4>(off, spec.H, spec.nqt_head, spec.ntr, spec.refine_q, 0, 0, spec.order, 0, spec.parts,
                spec.slot_base, spec.tasks, st, spec.dev_split, spec.slots, spec.split_tiles, s_nnz, s_maxrow);
  }
  // column compaction, one thread per (row, 32-column word): the word's
  // first output slot is the row offset plus the row's earlier words' bits
  __syncthreads();
  for (int it = t; it < nrows * nw; it += 1024) {
    const int r = it / nw, k = it - r * nw;
    const int32_t mid = (off[r] + off[r + 1] - 1) >> 1;  // the row's median entry
    int32_t o = off[r];
    for (int kk = 0; kk < k; ++kk) o += (int32_t)__popc(row_word(r, kk));
    uint32_t v = row_word(r, k);
    while (v) {
      const int32_t c = (k << 5) + __ffs(v) - 1;
      if (o == mid) rsig[r] = c;
      cols[o++] = c;
      v &= v - 1u;
    }
  }
}

// Coarsened tile list: tile row tr of head h covers logical rows
// [tr*cq, tr*cq + cq) and tile column tc covers logical columns
// [tc*ckv, tc*ckv + ckv).  A tile exists iff one of its blocks is active;
// its membership bit a*ckv + b is set iff logical block
// (tr*cq + a, tc*ckv + b) is active (paper section 4.2, "Coarsened").
// One workgroup per tile row; the row's union is built in an LDS bitmap of
// kCoarsenWin tile columns, one window of columns after another (a single
// window unless the row has more than kCoarsenWin tile columns).  With
// trow_ptr == nullptr the kernel writes counts, else the tile entries.
constexpr int kCoarsenWin = 8192;
__global__ __launch_bounds__(256) void k_coarsen(const int32_t* __restrict__ row_ptr,
                                                 const int32_t* __restrict__ cols, int32_t nqb,
                                                 int32_t cq, int32_t ckv, int32_t ntr,
                                                 int32_t ntc, int32_t* __restrict__ trow_cnt,
                                                 const int32_t* __restrict__ trow_ptr,
                                                 int32_t* __restrict__ tcol,
                                                 uint32_t* __restrict__ tbits,
                                                 int32_t* __restrict__ tsig) {
  __shared__ uint32_t bitmap[kCoarsenWin];
  __shared__ int32_t wave_tot[4];
  const int g = blockIdx.x;  // h * ntr + tr
  const int h = g / ntr;
  const int tr = g - h * ntr;
  const unsigned l = lane_id();
  const int w = threadIdx.x >> 6;
  int cnt = 0;                                   // count pass: this thread's share
  int32_t out = trow_ptr ? trow_ptr[g] : 0;      // write pass: next entry
  const int32_t mid = trow_ptr ? (out + trow_ptr[g + 1] - 1) >> 1 : -1;  // the row's median entry
  for (int w0 = 0; w0 < ntc; w0 += kCoarsenWin) {
    const int wn = min(kCoarsenWin, ntc - w0);
    for (int i = threadIdx.x; i < wn; i += 256) bitmap[i] = 0u;
    __syncthreads();
    for (int a = 0; a < cq; ++a) {
      const int r = tr * cq + a;
      if (r >= nqb) break;
      const int rr = h * nqb + r;
      const int b = row_ptr[rr], e = row_ptr[rr + 1];
      for (int i = b + threadIdx.x; i < e; i += 256) {
        const int c = cols[i];
        const int tc = c / ckv - w0;
        if (tc >= 0 && tc < wn) atomicOr(&bitmap[tc], 1u << (a * ckv + (c - (tc + w0) * ckv)));
      }
    }
    __syncthreads();
    if (!trow_ptr) {
      for (int i = threadIdx.x; i < wn; i += 256) cnt += bitmap[i] != 0u;
    } else {
      // ordered compaction: process the window in chunks of 256 entries
      for (int base = 0; base < wn; base += 256) {
        const int i = base + threadIdx.x;
        const uint32_t bits = i < wn ? bitmap[i] : 0u;
        const unsigned long long bal = __ballot(bits != 0u);
        if (l == 0) wave_tot[w] = __popcll(bal);
        __syncthreads();
        int before = 0;
        for (int k = 0; k < w; ++k) before += wave_tot[k];
        const int total = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
        if (bits) {
          const int pos = out + before + (int)prefix_count(bal);
          tcol[pos] = w0 + i;
          tbits[pos] = bits;
          if (pos == mid) tsig[g] = w0 + i;
        }
        out += total;
        __syncthreads();
      }
    }
    __syncthreads();  // the window is read out before the next one is cleared
  }
  if (!trow_ptr) {
    // wave reduction then workgroup reduction
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    if (l == 0) wave_tot[w] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) trow_cnt[g] = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
  }
}


// Task list (paper section 4.3, "Grouping and traversal" and "Split-K"), one
// workgroup: query tile g = h * nqt_head + qt traverses tile-list row
// h * ntr + qt / refine_q.  A row with more than `split` entries is cut into
// ceil(n / split) contiguous partitions of near-equal size (split == 0 never
// splits); every query tile gets at least one task, so rows without entries
// still write zeros.  Writes, per query tile, its partition count and first
// workspace slot (for the merge kernel), the tasks, and the task count into
// st->n_tasks.
//
// Traversal order (paper section 3, task organization): order == 0 lists the
// tasks in query-tile order; order == 1 lists them longest first, so that the
// in-order dispatch of workgroups approximates a longest-processing-time
// schedule and the short tasks fill the tail; order == 2 lists them by head
// and, within a head, by a signature of the query tile's K/V columns (the
// median entry of its tile-list row), so that query tiles that traverse
// mostly the same K/V tiles -- the rows of one cluster of a clustered mask --
// are dispatched together (and, with XCD runs, onto one XCD, whose L2 they
// then share).  Lengths (entries) are counted into kLenBuckets buckets --
// exact lengths while max_len < kLenBuckets, else proportional buckets of
// max_len -- or (head, signature) into kSigBuckets buckets (kSigBuckets / H
// signature bands per head, fine enough that a band holds a handful of
// neighbouring query tiles of a smoothly varying mask), and placed by a
// counting sort.  Within a bucket, tasks of an earlier chunk of the walk
// (1024 threads x TPT consecutive tiles) come first; inside a chunk their
// order follows the LDS atomics (the partitions of one tile that share a
// bucket stay together).  Every task writes a fixed part of the output (split
// partials a fixed workspace slot), so the order changes timing, not results.
constexpr int kLenBuckets = 1024;
constexpr int kSigBuckets = 8192;

struct RowTasks {
  int h, qt, b, e, p, chunk;
};

__device__ inline RowTasks row_tasks(const int32_t* __restrict__ trow_ptr, int g, int nqt_head,
                                     int ntr, int refine_q, int split, int split_min) {
  RowTasks r;
  r.h = g / nqt_head;
  r.qt = g - r.h * nqt_head;
  const int tr = r.qt / refine_q;
  r.b = trow_ptr[r.h * ntr + tr];
  r.e = trow_ptr[r.h * ntr + tr + 1];
  const int n = r.e - r.b;
  r.p = (split > 0 && n > split_min) ? (n + split - 1) / split : 1;
  r.chunk = (n + r.p - 1) / r.p;
  return r;
}

__device__ inline int len_bucket(int len, int max_len) {
  // descending length -> ascending bucket index
  len = min(len, max_len);
  const int k = max_len < kLenBuckets ? len : (int)(((long long)len * (kLenBuckets - 1)) / max_len);
  return kLenBuckets - 1 - k;
}

// Signature bucket of a query tile's row (order == 2): head-major, then the
// row's median column sig (its entry (b + e - 1) / 2, which the compaction or
// the coarsening stored per row) in bph equal bands of the ncol tile-list
// columns.
__device__ inline int sig_bucket(const RowTasks& r, int sig, int ncol, int H) {
  const int bph = max(1, kSigBuckets / max(H, 1));
  const int band = min(bph - 1, (int)(((long long)sig * bph) / max(ncol, 1)));
  return min(kSigBuckets - 1, r.h * bph + band);
}

__device__ inline Task make_task(const RowTasks& r, int i, int slot0) {
  Task tk;
  tk.head = r.h;
  tk.qtile = r.qt;
  tk.begin = min(r.e, r.b + i * r.chunk);
  tk.end = min(r.e, r.b + (i + 1) * r.chunk);
  tk.slot = r.p > 1 ? slot0 + i : -1;
  tk.pad0 = tk.pad1 = tk.pad2 = 0;
  return tk;
}

//
// A row of n > split_min entries is cut into ceil(n / split) partitions.
// dev_split >= 0: split, split_min and max_len are not given but derived here
// from the statistics in *st with the host's balance rule for a plan of
// split share dev_split (in halves; 0 = never split) over `slots` resident
// workgroups and an uncoarsened tile list, so the builder can be queued
// before the host has read the statistics.
// The builder runs in one workgroup of 1024 threads: as its own kernel
// (k_tasks) or inside k_mask_small.  stat_nnz / stat_max_row are the
// statistics the device split rule reads (dev_split >= 0).  TPT: query tiles
// per thread and chunk of the walk (more tiles in flight, more registers).
template <int TPT>
__device__ __forceinline__ void build_tasks(const int32_t* trow_ptr, int32_t H, int32_t nqt_head, int32_t ntr, int32_t refine_q,
                            int32_t split, int32_t split_min, int32_t order, int32_t max_len, int32_t* __restrict__ parts,
                            int32_t* __restrict__ slot_base, Task* __restrict__ tasks, MaskStats* st,
                            int32_t dev_split, int32_t slots, int32_t* __restrict__ split_tiles,
                            unsigned long long stat_nnz, unsigned stat_max_row,
                            const int32_t* __restrict__ tsig, int32_t ncol) {
  __shared__ int32_t lds[32];
  __shared__ int32_t cursor[kSigBuckets];
  constexpr int kChunk = 1024 * TPT;  // query tiles per chunk; a thread's TPT loads are issued together
  const int t = threadIdx.x;
  const int nbk = order == 2 ? kSigBuckets : kLenBuckets;  // buckets in use
  constexpr int kPer = kSigBuckets / 1024;                 // buckets per thread at most
  const int nqt = H * nqt_head;
  if (dev_split >= 0) {
    const long long W = (long long)refine_q * (long long)stat_nnz;
    const long long row_max = (long long)stat_max_row;
    long long sp = 0, smin = 0;
    if (dev_split > 0) {
      const long long den = (long long)slots * dev_split;
      sp = max(4LL, (2 * max(W, 1LL) + den - 1) / den);
      const long long mean = (max(W, 1LL) + nqt - 1) / nqt;
      smin = max(sp, kSplitRowFactor * mean);
      if (row_max <= smin) sp = 0;
    }
    split = (int32_t)sp;
    split_min = (int32_t)min(smin, (long long)(1 << 30));
    max_len = sp > 0 ? (int32_t)sp : (int32_t)min(row_max, (long long)(1 << 30));
  }
  max_len = max(max_len, 1);
  if (order)
    for (int i = t; i < nbk; i += 1024) cursor[i] = 0;
  __syncthreads();
  // Buckets of a tile's partitions: order 2 puts all of them in the row's
  // signature bucket; order 1 puts the full-length ones (all but the last) in
  // their length's bucket and the last, which may be shorter, in its own.
  // Bucket a takes partitions [0, na), bucket b partition p - 1 when nb = 1.
  struct Place {
    int a, na, b, nb;
  };
  auto place = [&](const RowTasks& r, int sig) {
    Place q;
    if (order == 2) {
      q.a = sig;
      q.na = r.p;
      q.b = 0;
      q.nb = 0;
    } else {
      q.a = len_bucket(r.chunk, max_len);
      q.na = r.p - 1;
      q.b = len_bucket((r.e - r.b) - (r.p - 1) * r.chunk, max_len);
      q.nb = 1;
    }
    return q;
  };
  // the chunk's rows and, for order 2, their signature buckets
  auto load_rows = [&](int g0, RowTasks (&r)[TPT], int32_t (&sig)[TPT]) {
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      r[k].p = 0;
      if (g0 + k < nqt) r[k] = row_tasks(trow_ptr, g0 + k, nqt_head, ntr, refine_q, split, split_min);
    }
#pragma unroll
    for (int k = 0; k < TPT; ++k)
      sig[k] = (order == 2 && g0 + k < nqt)
                   ? sig_bucket(r[k], r[k].e > r[k].b ? tsig[r[k].h * ntr + r[k].qt / refine_q] : 0, ncol, H)
                   : 0;
  };
  // pass 1: partition counts and workspace slots in query-tile order; the
  // tasks themselves (query-tile order) or their bucket histogram
  int32_t carry_t = 0, carry_s = 0, carry_x = 0;
  for (int base = 0; base < nqt; base += kChunk) {
    const int g0 = base + TPT * t;
    RowTasks r[TPT];
    int32_t sig[TPT];
    load_rows(g0, r, sig);
    int32_t sum_t = 0, sum_s = 0;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      sum_t += r[k].p;
      sum_s += r[k].p > 1 ? r[k].p : 0;
    }
    int32_t tot_t, tot_s;
    int32_t off_t = carry_t + block_scan(sum_t, lds, &tot_t);
    int32_t off_s = carry_s + block_scan(sum_s, lds, &tot_s);
    if (split_tiles) {
      int32_t nsp = 0, tot_x;
#pragma unroll
      for (int k = 0; k < TPT; ++k) nsp += r[k].p > 1;
      int32_t off_x = carry_x + block_scan(nsp, lds, &tot_x);
#pragma unroll
      for (int k = 0; k < TPT; ++k)
        if (r[k].p > 1) split_tiles[off_x++] = g0 + k;
      carry_x += tot_x;
    }
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int g = g0 + k;
      if (g >= nqt) break;
      parts[g] = r[k].p;
      slot_base[g] = off_s;
      if (order) {
        const Place q = place(r[k], sig[k]);
        if (q.na) atomicAdd(&cursor[q.a], q.na);
        if (q.nb) atomicAdd(&cursor[q.b], q.nb);
      } else {
        for (int i = 0; i < r[k].p; ++i) tasks[off_t + i] = make_task(r[k], i, off_s);
      }
      off_t += r[k].p;
      off_s += r[k].p > 1 ? r[k].p : 0;
    }
    carry_t += tot_t;
    carry_s += tot_s;
  }
  if (t == 0) {
    st->n_tasks = (unsigned long long)carry_t;
    st->n_split = (unsigned long long)carry_x;
  }
  if (!order) return;
  // bucket starts, then pass 2 places every task at its bucket's cursor
  __syncthreads();
  {
    // exclusive scan of the bucket counts: thread t owns buckets
    // [t * per, (t + 1) * per)
    const int per = nbk / 1024;
    int32_t c[kPer];
    int32_t sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      c[i] = i < per ? cursor[t * per + i] : 0;
      sum += c[i];
    }
    int32_t tot;
    int32_t run = block_scan(sum, lds, &tot);
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (i < per) {
        cursor[t * per + i] = run;
        run += c[i];
      }
  }
  __syncthreads();
  carry_s = 0;
  for (int base = 0; base < nqt; base += kChunk) {
    const int g0 = base + TPT * t;
    RowTasks r[TPT];
    int32_t sig[TPT];
    int32_t tot_s;
    load_rows(g0, r, sig);  // again: holding every chunk's rows would spill
    int32_t sum_s = 0;
#pragma unroll
    for (int k = 0; k < TPT; ++k) sum_s += r[k].p > 1 ? r[k].p : 0;
    int32_t off_s = carry_s + block_scan(sum_s, lds, &tot_s);
    // claim every tile's places first (independent atomics), then write
    int32_t pa[TPT], pb[TPT];
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      pa[k] = pb[k] = 0;
      if (g0 + k < nqt) {
        const Place q = place(r[k], sig[k]);
        if (q.na) pa[k] = atomicAdd(&cursor[q.a], q.na);
        if (q.nb) pb[k] = atomicAdd(&cursor[q.b], q.nb);
      }
    }
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      if (g0 + k >= nqt) break;
      const Place q = place(r[k], sig[k]);
      for (int i = 0; i < q.na; ++i) tasks[pa[k] + i] = make_task(r[k], i, off_s);
      if (q.nb) tasks[pb[k]] = make_task(r[k], r[k].p - 1, off_s);
      off_s += r[k].p > 1 ? r[k].p : 0;
    }
    carry_s += tot_s;
    __syncthreads();  // this chunk's tasks precede the next chunk's in each bucket
  }
}

__global__ __launch_bounds__(1024) void k_tasks(const int32_t* __restrict__ trow_ptr, int32_t H,
                                                int32_t nqt_head, int32_t ntr, int32_t refine_q,
                                                int32_t split, int32_t split_min, int32_t order,
                                                int32_t max_len, int32_t* __restrict__ parts,
                                                int32_t* __restrict__ slot_base,
                                                Task* __restrict__ tasks, MaskStats* st,
                                                int32_t dev_split, int32_t slots,
                                                int32_t* __restrict__ split_tiles,
                                                const int32_t* __restrict__ tsig, int32_t ncol) {
  const unsigned long long nnz = dev_split >= 0 ? st->nnz : 0ull;
  const unsigned max_row = dev_split >= 0 ? st->max_row_nnz : 0u;
  build_tasks<8>(trow_ptr, H, nqt_head, ntr, refine_q, split, split_min, order, max_len, parts, slot_base, tasks,
              st, dev_split, slots, split_tiles, nnz, max_row, tsig, ncol);
}

// Stream organization: the concatenated entries of all query tiles (head,
// query tile, entry order; W in total) are cut into G equal ranges, one per
// resident workgroup: workgroup k owns positions [ceil(kW/G), ceil((k+1)W/G)).
// A query tile whose entries span several ranges becomes one task per range
// (a partition with its own workspace slot); a tile without entries is one
// empty task of the range its position falls in.  Tasks are written in
// (tile, range) order, which is also range order, and seg_ptr[k] is the first
// task of workgroup k (seg_ptr[G] = number of tasks).  G shrinks to W when W
// < G, so every range owns at least one position.  One workgroup of 1024.
__device__ inline int stream_group(long long x, long long W, int G) {
  // the range that position x falls in (W > 0), clamped for trailing empty tiles
  return (int)min((long long)G - 1, (x * G) / W);
}

__global__ __launch_bounds__(1024) void k_tasks_stream(const int32_t* __restrict__ trow_ptr, int32_t H,
                                                       int32_t nqt_head, int32_t ntr, int32_t refine_q,
                                                       int32_t G, int32_t* __restrict__ parts,
                                                       int32_t* __restrict__ slot_base,
                                                       Task* __restrict__ tasks,
                                                       int32_t* __restrict__ seg_ptr, MaskStats* st) {
  __shared__ int32_t lds[32];
  __shared__ int32_t hist[kMaxStreamGroups];
  const int t = threadIdx.x;
  const int nqt = H * nqt_head;
  // pass A: W = all entries
  long long W = 0;
  for (int base = 0; base < nqt; base += 4096) {
    int32_t sum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int g = base + 4 * t + k;
      if (g < nqt) {
        const RowTasks r = row_tasks(trow_ptr, g, nqt_head, ntr, refine_q, 0, 0);
        sum += r.e - r.b;
      }
    }
    int32_t tot;
    (void)block_scan(sum, lds, &tot);
    W += tot;
  }
  const int Ge = W > 0 ? (int)min((long long)G, W) : 1;
  for (int k = t; k < G; k += 1024) hist[k] = 0;
  __syncthreads();
  // pass B: tasks in (tile, range) order, partition counts and slots
  long long carry_p = 0;
  int32_t carry_t = 0, carry_s = 0;
  for (int base = 0; base < nqt; base += 4096) {
    const int g0 = base + 4 * t;
    RowTasks r[4];
    int wfirst[4];
    int32_t sum_n = 0, sum_t = 0, sum_s = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      r[k].p = 0;
      r[k].b = r[k].e = 0;
      if (g0 + k < nqt) {
        r[k] = row_tasks(trow_ptr, g0 + k, nqt_head, ntr, refine_q, 0, 0);
        sum_n += r[k].e - r[k].b;
      }
    }
    int32_t tot_n, tot_t, tot_s;
    long long pos = carry_p + block_scan(sum_n, lds, &tot_n);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (g0 + k >= nqt) break;
      const int n = r[k].e - r[k].b;
      wfirst[k] = W > 0 ? stream_group(pos, W, Ge) : 0;
      const int wlast = n > 0 ? stream_group(pos + n - 1, W, Ge) : wfirst[k];
      r[k].p = wlast - wfirst[k] + 1;
      r[k].chunk = (int)(pos - carry_p);  // position within the chunk (restored below)
      pos += n;
      sum_t += r[k].p;
      sum_s += r[k].p > 1 ? r[k].p : 0;
    }
    int32_t off_t = carry_t + block_scan(sum_t, lds, &tot_t);
    int32_t off_s = carry_s + block_scan(sum_s, lds, &tot_s);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int g = g0 + k;
      if (g >= nqt) break;
      const long long P = carry_p + r[k].chunk;
      const int n = r[k].e - r[k].b;
      parts[g] = r[k].p;
      slot_base[g] = off_s;
      for (int j = 0; j < r[k].p; ++j) {
        const int w = wfirst[k] + j;
        Task tk;
        tk.head = r[k].h;
        tk.qtile = r[k].qt;
        if (n > 0) {
          const long long cb = (w * W + Ge - 1) / Ge, ce = ((w + 1) * W + Ge - 1) / Ge;
          tk.begin = r[k].b + (int)(max(P, cb) - P);
          tk.end = r[k].b + (int)(min(P + n, ce) - P);
        } else {
          tk.begin = tk.end = r[k].b;
        }
        tk.slot = r[k].p > 1 ? off_s + j : -1;
        tk.pad0 = w;
        tk.pad1 = tk.pad2 = 0;
        tasks[off_t + j] = tk;
        atomicAdd(&hist[w], 1);
      }
      off_t += r[k].p;
      off_s += r[k].p > 1 ? r[k].p : 0;
    }
    carry_p += tot_n;
    carry_t += tot_t;
    carry_s += tot_s;
  }
  if (t == 0) st->n_tasks = (unsigned long long)carry_t;
  __syncthreads();
  // seg_ptr = exclusive scan of the per-range task counts
  int32_t carry = 0;
  for (int base = 0; base < G; base += 1024) {
    const int k = base + t;
    const int32_t c = k < G ? hist[k] : 0;
    int32_t tot;
    const int32_t off = carry + block_scan(c, lds, &tot);
    if (k < G) seg_ptr[k] = off;
    carry += tot;
  }
  if (t == 0) seg_ptr[G] = carry;
}

// Plan cache, exact-repeat check: flags[c] = 1 when the request mask differs
// from cached copy c anywhere (grid-stride over 16-byte words when both
// pointers allow, else bytes; blockIdx.y = candidate).  Every writer stores
// the same value, so the race between writers is benign.
__global__ __launch_bounds__(256) void k_mask_compare(const CompareArgs a) {
  const int c = blockIdx.y;
  const uint8_t* m = a.mask;
  const uint8_t* o = a.cand[c];
  const int64_t stride = (int64_t)gridDim.x * 256;
  bool diff = false;
  if (((reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(o)) & 15) == 0) {
    const int64_t words = a.bytes / 16;
    const uint4* mw = reinterpret_cast<const uint4*>(m);
    const uint4* ow = reinterpret_cast<const uint4*>(o);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += stride) {
      const uint4 x = mw[i], y = ow[i];
      diff |= (x.x != y.x) | (x.y != y.y) | (x.z != y.z) | (x.w != y.w);
    }
    for (int64_t i = words * 16 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < a.bytes; i += stride)
      diff |= m[i] != o[i];
  } else {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < a.bytes; i += stride) diff |= m[i] != o[i];
  }
  if (diff) a.flags[c] = 1;
}

// Copies the flags to the host record (then the sequence number, system-scope
// release), sets the speculative-run guard, and clears the flags for the next
// check.
__global__ __launch_bounds__(64) void k_compare_publish(int32_t* flags, int32_t ncand, CompareResult* host,
                                                        unsigned long long seq,
                                                        const unsigned long long* spec_ntasks,
                                                        unsigned long long* guard) {
  const int t = threadIdx.x;
  if (t < kMaxCompare) {
    const int32_t f = t < ncand ? flags[t] : 1;
    sys_store(&host->differs[t], f);
    if (t == 0 && guard) *guard = f == 0 ? *spec_ntasks : 0ull;
    flags[t] = 0;
  }
  // one wave: its own field stores are the ones the wait covers
  if (t == 0) sys_publish_seq(&host->seq, seq);
}

}  // namespace

hipError_t launch_mask_compare(const CompareArgs& a, CompareResult* host, unsigned long long seq,
                               hipStream_t s) {
  if (a.ncand < 1 || a.ncand > kMaxCompare) return hipErrorInvalidValue;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((a.bytes + 4095) / 4096, 512));
  hipLaunchKernelGGL(k_mask_compare, dim3((unsigned)blocks, (unsigned)a.ncand), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_compare_publish, dim3(1), dim3(64), 0, s, a.flags, a.ncand, host, seq, a.spec_ntasks,
                     a.guard);
  return hipGetLastError();
}

int row_count_blocks(int32_t nrows) { return std::max(1, std::min((nrows + 3) / 4, 2048)); }

hipError_t launch_row_count(const uint8_t* mask, int32_t nrows, int32_t nkb, int32_t* row_cnt,
                            RowPartial* part, hipStream_t s) {
  if (((uintptr_t)mask & 15) == 0)
    hipLaunchKernelGGL(k_row_count16, dim3(row_count_blocks(nrows)), dim3(256), 0, s, mask, nrows, nkb,
                       row_cnt, part);
  else
    hipLaunchKernelGGL(k_row_count, dim3(row_count_blocks(nrows)), dim3(256), 0, s, mask, nrows, nkb,
                       row_cnt, part);
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* in, int32_t* out, int32_t n, const RowPartial* part,
                       int32_t npart, MaskStats* st, MaskStats* host_st, unsigned long long seq,
                       hipStream_t s) {
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, in, out, n, part, npart, st, host_st, seq);
  return hipGetLastError();
}

bool mask_small_ok(const uint8_t* mask, int32_t nrows, int32_t nkb) {
  return ((uintptr_t)mask & 15) == 0 && nrows <= kSmallMaskRows && nkb <= kSmallMaskCols &&
         (int64_t)nrows * nkb <= kSmallMaskBytes;
}

hipError_t launch_mask_small(const uint8_t* mask, int32_t nrows, int32_t nkb, int32_t* row_ptr, int32_t* cols,
                             int32_t* rsig, MaskStats* st, MaskStats* host_st, unsigned long long seq, hipStream_t s,
                             const TaskSpec& spec) {
  if (!mask_small_ok(mask, nrows, nkb) || !rsig) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mask_small, dim3(1), dim3(1024), 0, s, mask, nrows, nkb, row_ptr, cols, rsig, st, host_st,
                     seq, spec);
  return hipGetLastError();
}

hipError_t launch_compact(const uint8_t* mask, int32_t nrows, int32_t nkb, const int32_t* row_ptr,
                          int32_t* cols, int32_t* rsig, hipStream_t s) {
  if (!rsig) return hipErrorInvalidValue;
  if (((uintptr_t)mask & 15) == 0)
    hipLaunchKernelGGL(k_compact16, dim3((nrows + 3) / 4), dim3(256), 0, s, mask, nrows, nkb, row_ptr, cols,
                       rsig);
  else
    hipLaunchKernelGGL(k_compact, dim3((nrows + 3) / 4), dim3(256), 0, s, mask, nrows, nkb, row_ptr,
                       cols, rsig);
  return hipGetLastError();
}

hipError_t launch_coarsen(const int32_t* row_ptr, const int32_t* cols, int32_t H, int32_t nqb,
                          int32_t nkb, int32_t cq, int32_t ckv, int32_t ntr, int32_t ntc,
                          int32_t* trow_cnt, const int32_t* trow_ptr, int32_t* tcol,
                          uint32_t* tbits, int32_t* tsig, hipStream_t s) {
  (void)nkb;
  if (trow_ptr && !tsig) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_coarsen, dim3(H * ntr), dim3(256), 0, s, row_ptr, cols, nqb, cq, ckv, ntr, ntc, trow_cnt,
                     trow_ptr, tcol, tbits, tsig);
  return hipGetLastError();
}

hipError_t launch_tasks_stream(const int32_t* trow_ptr, int32_t H, int32_t nqt_head, int32_t ntr,
                               int32_t refine_q, int32_t groups, int32_t* parts, int32_t* slot_base, Task* tasks,
                               int32_t* seg_ptr, MaskStats* st, hipStream_t s) {
  if (groups < 1 || groups > kMaxStreamGroups) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_tasks_stream, dim3(1), dim3(1024), 0, s, trow_ptr, H, nqt_head, ntr, refine_q, groups,
                     parts, slot_base, tasks, seg_ptr, st);
  return hipGetLastError();
}

// Queue y of the per-XCD task queues holds the positions of the tasks t <
// n_tasks with (t / run) % 8 == y: whole rounds of 8 runs give each queue
// `run` of them, the last partial round what falls in its run.  Its word
// covers the dynamic suffix, the last len / 8 positions.
__global__ void k_xq_init(unsigned long long* __restrict__ xq, const unsigned long long* __restrict__ n_tasks,
                          int32_t run) {
  const int y = threadIdx.x;
  if (y >= 8) return;
  const long long n = (long long)*n_tasks;
  const long long per_round = 8LL * run;
  const long long rounds = n / per_round, rem = n - rounds * per_round;
  const long long len = rounds * run + min(max(rem - (long long)y * run, 0LL), (long long)run);
  // head 0, tail len / 8 (stored by an atomic, where the claims' atomics act)
  atomicExch(&xq[y], (unsigned long long)(len >> 3) << 32);
}

hipError_t launch_xq_init(unsigned long long* xq, const unsigned long long* n_tasks, int32_t run, hipStream_t s) {
  if (!xq || !n_tasks || run < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_xq_init, dim3(1), dim3(64), 0, s, xq, n_tasks, run);
  return hipGetLastError();
}

hipError_t launch_tasks(const int32_t* trow_ptr, int32_t H, int32_t nqt_head, int32_t ntr,
                        int32_t refine_q, int32_t split, int32_t split_min, int32_t order, int32_t max_len,
                        int32_t* parts, int32_t* slot_base, Task* tasks, MaskStats* st,
                        hipStream_t s, int32_t dev_split, int32_t slots, int32_t* split_tiles,
                        const int32_t* tsig, int32_t ncol) {
  if (order == 2 && !tsig) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_tasks, dim3(1), dim3(1024), 0, s, trow_ptr, H, nqt_head, ntr, refine_q, split,
                     split_min, order, max_len, parts, slot_base, tasks, st, dev_split, slots, split_tiles,
                     tsig, ncol);
  return hipGetLastError();
}

}  // namespace bsa
