// Native kernel catalog and plan selection (host side).
//
// Tessera paper, section 4.1: a physical plan P = <g_Q, g_KV, sigma, e> binds
// the mapping of the logical block geometry B to a physical tile T on each
// dimension, a task organization sigma (grouping, traversal, K/V reduction
// partitions, pipeline depth) and the native kernel(s) e.  Section 4.4: the
// catalog keeps plans with an implementation for the architecture;
// Eligible(P, R) holds when the plan supports the request's logical geometry,
// tensor properties, metadata format and available workspace while
// preserving E(M).  Section 5: the plan table maps performance regimes to
// rankings; the runtime scans a regime's ranking for the first eligible plan
// and uses the key's base plan on a lookup miss.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/bsa.h"

namespace bsa {

struct CatalogEntry {
  int id;
  int tq, tkv, d;
  int split;      // 0: one task per query tile; s >= 1: balance rule with
                  // partitions of at most 2/s of the even share per slot
  int xcd_remap;  // > 0: runs of this many consecutive tasks per XCD
  int order;      // 0: tasks in query-tile order; 1: longest first; 2: by head
                  // and K/V-column signature
  std::string name;
};

// Mapping of a logical dimension of size b onto a tile dimension of size t.
struct DimMap {
  bool ok = false;
  int coarsen = 1;  // logical blocks per tile
  int refine = 1;   // tiles per logical block
};

// Smallest logical query block a coarsened query tile may hold: a wave owns
// 32 query rows, which then span at most two logical rows.
constexpr int kMinCoarsenBlockQ = 16;
DimMap map_dim(int block, int tile, int min_coarsen_block);

const std::vector<CatalogEntry>& catalog();
uint64_t catalog_hash_value();

// Geometry / tensor eligibility; the workspace part is checked by the caller
// once the split rule is known (ws_bytes < 0 skips it).
bool eligible(const CatalogEntry& e, const bsa_request& r, int64_t ws_bytes, std::string* why);

// Base plan of the request key: Direct (T = B) when the catalog has it with
// the default organization, else the eligible entry with the smallest tile.
int base_plan(const bsa_request& r);

struct Selection {
  int regime = -1;
  std::vector<int> candidates;  // ranked; base plan last
};

// Regime lookup (stage 1: key = (arch, B, dtype, d, layout); stage 2: feature
// buckets of H, N, density, run coverage and row skew).
Selection lookup(const bsa_request& r, double density, double run_coverage, double row_skew);

bsa_status table_load_file(const char* path, std::string* err);
bsa_status table_load_text(const std::string& text, std::string* err);
const std::string& table_version();

}  // namespace bsa
