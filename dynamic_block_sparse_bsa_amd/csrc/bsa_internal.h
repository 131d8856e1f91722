// Internal declarations shared by the host code and the gfx950 kernels of the
// block-sparse attention library.  Nothing here is part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

// One workgroup task of the attention launch: a query tile of one head and a
// contiguous range [begin, end) of entries of the tile list (the block-CSR for
// Direct and Refined mappings, the coarsened tile list otherwise).  slot >= 0
// marks a split-K partition whose partial state goes to workspace slot `slot`.
struct Task {
  int32_t head;
  int32_t qtile;
  int32_t begin;
  int32_t end;
  int32_t slot;
  int32_t pad0, pad1, pad2;
};
static_assert(sizeof(Task) == 32, "Task is 32 bytes");

// Statistics of the shared mask state, filled on the GPU and copied to the
// host in one transfer.
struct MaskStats {
  unsigned long long nnz;            // active logical blocks
  unsigned long long long_run;       // active blocks inside runs of length >= 2
  unsigned int max_row_nnz;          // largest active count of a query-block row
  unsigned int empty_rows;           // query-block rows with no active block
  unsigned long long n_tasks;        // tasks written by the task builder
  unsigned long long n_split;        // query tiles with more than one partition
  unsigned long long seq;            // host copy: request sequence number, written last
};

// Exact-repeat check of the plan cache: which of up to kMaxCompare cached
// masks differ from the request's mask.
constexpr int kMaxCompare = 8;
struct CompareArgs {
  const uint8_t* mask;                  // request mask (device)
  const uint8_t* cand[kMaxCompare];     // cached mask copies (device)
  int32_t ncand;
  int64_t bytes;
  int32_t* flags;                       // device [kMaxCompare], zero on entry and on exit
  // Optional guard of a speculative run of candidate 0's plan: set to that
  // plan's task count when candidate 0 matches, else to 0 (the guarded
  // kernels then exit at once).
  const unsigned long long* spec_ntasks;
  unsigned long long* guard;
};
// Host record of the check, written by the GPU into coherent host memory.
struct CompareResult {
  int32_t differs[kMaxCompare];
  unsigned long long seq;               // written last
};

// Per-workgroup partial statistics of the row-count kernel.
struct RowPartial {
  unsigned long long long_run;
  unsigned int max_row;
  unsigned int empty;
};

// Arguments of the attention mainloop kernels.
struct AttnArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  const Task* tasks;
  const unsigned long long* n_tasks;  // device count written by the task builder
  const int32_t* tcol;    // tile-list column (in units of the list's column width)
  const uint32_t* tbits;  // membership bits per tile-list entry, or nullptr
  float* ws_m;            // [slot][T_Q]           running max (log2 units)
  float* ws_l;            // [slot][T_Q]           exponential sum
  float* ws_o;            // [slot][d][T_Q] fp32: the partial output
                          // normalized by its own l (0 when l = 0)
  // Tensor layout (elements; d is contiguous): head g of the task list is
  // head g % heads of batch entry g / heads, at g/heads * batch_stride +
  // g%heads * head_stride, and consecutive rows are row_stride apart.
  int64_t batch_stride;
  int64_t head_stride;
  int32_t heads;
  int32_t row_stride;
  int32_t N;
  int32_t sub_log2;       // log2(refine_kv): K/V tiles per tile-list entry
  int32_t bkv_log2;       // log2(B_KV)
  int32_t coarsen_kv;     // logical K/V blocks per tile (membership decode)
  int32_t bq;             // B_Q (membership decode when coarsen_q > 1)
  int32_t coarsen_q;
  int32_t xcd_remap;      // > 0: runs of this many consecutive tasks per XCD
  unsigned long long* xq; // nullable (with xcd_remap): the 8 per-XCD task queues
                          // (k_xq_init sets them before each launch)
  const int32_t* seg_ptr; // stream organization: workgroup k runs tasks
                          // [seg_ptr[k], seg_ptr[k+1]); nullptr: one task each
  int32_t grid;           // workgroups launched (multiple of 8 * xcd_remap when remapped)
  float scale_log2;       // log2(e) / sqrt(d)
};

struct MergeArgs {
  __bf16* o;
  const unsigned long long* guard;  // nullptr, or a word that is 0 when the run must do nothing
  int64_t batch_stride;     // layout of O, as in AttnArgs
  int64_t head_stride;
  int32_t heads;
  int32_t row_stride;
  const int32_t* parts;     // [n_qtiles] partitions per query tile
  const int32_t* slot_base; // [n_qtiles] first workspace slot of the query tile
  const float* ws_m;
  const float* ws_l;
  const float* ws_o;        // [slot][d][T_Q] fp32, normalized partials
  // Optional compact list of the split query tiles (ascending) and its
  // device count; the launch then loops over (listed tile, column group)
  // items instead of one workgroup per (tile, column group).
  const int32_t* split_tiles;
  const unsigned long long* n_split;
  int32_t N;
  int32_t n_qtiles_head;    // query tiles per head
  int32_t tq;
  int32_t d;
};

// Kernel launchers (defined in the .hip translation units).
using AttnLauncher = hipError_t (*)(const AttnArgs&, int grid, hipStream_t);

int row_count_blocks(int32_t nrows);  // workgroups (= partials) of the row-count kernel
hipError_t launch_row_count(const uint8_t* mask, int32_t nrows, int32_t nkb, int32_t* row_cnt,
                            RowPartial* part, hipStream_t s);
// Exclusive scan; with st non-null also completes the mask statistics (and
// copies them to host_st, fine-grained host memory, when non-null).
hipError_t launch_scan(const int32_t* in, int32_t* out, int32_t n, const RowPartial* part,
                       int32_t npart, MaskStats* st, MaskStats* host_st, unsigned long long seq,
                       hipStream_t s);
constexpr int kMaxStreamGroups = 4096;  // workgroups of the stream organization
hipError_t launch_tasks_stream(const int32_t* trow_ptr, int32_t H, int32_t nqt_head, int32_t ntr,
                               int32_t refine_q, int32_t groups, int32_t* parts, int32_t* slot_base, Task* tasks,
                               int32_t* seg_ptr, MaskStats* st, hipStream_t s);
hipError_t launch_mask_compare(const CompareArgs& a, CompareResult* host, unsigned long long seq,
                               hipStream_t s);
// A task list to build on the device with the split derived from the
// statistics (k_tasks' device split mode) for an uncoarsened entry: the
// speculative list of a repeated request key.  enabled = 0: none.
struct TaskSpec {
  int32_t enabled;
  int32_t H, nqt_head, ntr, refine_q, order, dev_split, slots;
  int32_t* parts;
  int32_t* slot_base;
  Task* tasks;
  int32_t* split_tiles;  // nullable
};

// Single-launch mask state (counts, statistics, scan, compaction) for masks
// of at most kSmallMaskBytes bytes, kSmallMaskRows rows and kSmallMaskCols
// columns at a 16-byte aligned address; outputs as launch_row_count +
// launch_scan + launch_compact.
constexpr int kSmallMaskBytes = 32768;
constexpr int kSmallMaskRows = 2048;
constexpr int kSmallMaskCols = 256;
bool mask_small_ok(const uint8_t* mask, int32_t nrows, int32_t nkb);
// spec.enabled: the kernel also builds that task list, right after the
// statistics are published and before the compaction.
// The compaction (k_mask_small, k_compact*) also stores, per block-CSR row,
// the column of its median entry (row_ptr[r] + row_ptr[r + 1] - 1) / 2 into
// rsig[r] (rows without entries are left unwritten), and the coarsening's
// write pass does the same per tile row into tsig: the traversal signature
// of the signature order.
hipError_t launch_mask_small(const uint8_t* mask, int32_t nrows, int32_t nkb, int32_t* row_ptr, int32_t* cols,
                             int32_t* rsig, MaskStats* st, MaskStats* host_st, unsigned long long seq, hipStream_t s,
                             const TaskSpec& spec);
hipError_t launch_compact(const uint8_t* mask, int32_t nrows, int32_t nkb, const int32_t* row_ptr,
                          int32_t* cols, int32_t* rsig, hipStream_t s);
hipError_t launch_coarsen(const int32_t* row_ptr, const int32_t* cols, int32_t H, int32_t nqb,
                          int32_t nkb, int32_t cq, int32_t ckv, int32_t ntr, int32_t ntc,
                          int32_t* trow_cnt, const int32_t* trow_ptr, int32_t* tcol,
                          uint32_t* tbits, int32_t* tsig, hipStream_t s);
// A query tile's row of n > split_min entries is cut into ceil(n / split)
// partitions.  dev_split >= 0: split, split_min and max_len are derived on
// the device from *st (the balance rule with split share dev_split in halves
// over `slots` workgroups, uncoarsened tile list); -1: the given values are
// used.  split_tiles (nullable): receives the query tiles with more than one
// partition, ascending; their count goes to st->n_split.
// The balance rule leaves rows of up to kSplitRowFactor times the mean row
// length whole: cutting rows of an even mask only adds partials to merge.
// order: 0 query-tile order, 1 longest first, 2 by head and column signature
// (needs each tile row's median column tsig and the tile-list column count
// ncol).
constexpr int kSplitRowFactor = 2;
// Per-XCD task queues of the XCD organizations.  Queue x holds the tasks of
// runs x, x + 8, x + 16, ... (runs of `run` consecutive tasks), in order.
// Workgroup i (on XCD i mod 8) runs position i / 8 of queue i mod 8 while
// that lies in the queue's first 7/8 (the static order, which keeps the
// L2-sharing runs together best).  The last 1/8 of each queue is claimed:
// its word is (tail << 32) | head over the suffix, positions [head, tail)
// unclaimed; a workgroup past the prefix takes the front of its own queue's
// suffix (atomic add of 1) or, once that is empty, the back of another
// queue's suffix (atomic add of -1 << 32); a claim is valid iff the returned
// head < tail, so every task runs exactly once and nothing waits.  The XCDs
// run at different speeds (a few percent apart, the same XCDs from launch to
// launch), and the fast ones take the slow ones' last tasks.  The grid adds
// one spare workgroup per kXcdSpareDiv tasks (so a fast XCD has workgroups
// left to steal with; spares that find every queue empty exit) and is
// rounded up to whole rounds of 8 runs: a queue holds at most grid / 8
// tasks, so every position of its static prefix has its workgroup.
constexpr int kXcdSpareDiv = 8;  // spare workgroups: one per kXcdSpareDiv tasks
hipError_t launch_xq_init(unsigned long long* xq, const unsigned long long* n_tasks, int32_t run, hipStream_t s);
hipError_t launch_tasks(const int32_t* trow_ptr, int32_t H, int32_t nqt_head, int32_t ntr,
                        int32_t refine_q, int32_t split, int32_t split_min, int32_t order, int32_t max_len,
                        int32_t* parts, int32_t* slot_base, Task* tasks, MaskStats* st,
                        hipStream_t s, int32_t dev_split = -1, int32_t slots = 0,
                        int32_t* split_tiles = nullptr, const int32_t* tsig = nullptr, int32_t ncol = 0);
// With a.split_tiles, grid_items (> 0) workgroups loop over the listed
// (tile, column group) items; otherwise one workgroup per (query tile,
// column group).  A column group is kMergeCols output columns.
constexpr int kMergeCols = 16;
hipError_t launch_merge(const MergeArgs& a, int32_t n_qtiles, hipStream_t s, int32_t grid_items = 0);

// Fixed per-device scratch array of the entry point that allocates nothing
// (static_scratch.hip): its device address on the current device (looked up
// once per device) and its size in bytes.
constexpr size_t kStaticScratchBytes = size_t(128) << 20;
hipError_t static_scratch(void** ptr, size_t* bytes);

// Attention kernel table: returns nullptr when (tq, tkv, d) has no kernel.
AttnLauncher attn_launcher(int tq, int tkv, int d);
// Resident workgroups per CU of that kernel (0 if it has none).
int attn_wg_per_cu(int tq, int tkv, int d, bool stream);  // resident workgroups per CU

}  // namespace bsa
