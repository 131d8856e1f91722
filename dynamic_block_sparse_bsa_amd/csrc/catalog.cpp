// Catalog, eligibility, and the versioned plan table (host only; no GPU calls).
#include "catalog.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <fstream>
#include <mutex>
#include <sstream>

namespace bsa {

namespace {

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

constexpr int kXcdRun = 16;      // tasks per XCD run of the "_xcd" organization
constexpr int kXcdRunLong = 128; // ... and of "_xcd128" (wan720p-like masks: −2.6%;
                                 // clustered hunyuan-like masks: +3.5%)

// Task organizations {split, XCD runs, order} (split in halves: partitions
// of at most 2/split of the even share of entries per resident workgroup
// slot; order 1 = longest task first).
struct Org {
  const char* name;
  int split, xcd, order;
};
constexpr Org kSplitK = {"splitk", 2, 0, 0};  // the default (base) organization
constexpr Org kSplitKLpt = {"splitk_lpt", 2, 0, 1};
constexpr Org kNoSplitLpt = {"nosplit_lpt", 0, 0, 1};
constexpr Org kSplitKXcd = {"splitk_xcd", 2, kXcdRun, 0};
constexpr Org kSplitK15Lpt = {"splitk15_lpt", 3, 0, 1};
constexpr Org kSplitK2Lpt = {"splitk2_lpt", 4, 0, 1};
constexpr Org kSplitKXcd128 = {"splitk_xcd128", 2, kXcdRunLong, 0};
// query tiles ordered by head and K/V-column signature, then XCD runs
constexpr Org kSplitKSimXcd = {"splitk_sim_xcd", 2, kXcdRun, 2};

std::vector<CatalogEntry> build_catalog() {
  // Kernel tile shapes instantiated for gfx950 (attn_kernels.hip) and the
  // organizations offered with each.  Every shape has the default
  // organization (a key's base plan uses it); at d = 64 and 128 the others
  // were kept where they were the fastest plan on some profiling cases: of
  // 104 shape x organization entries, dropping all but these 31 raised the
  // corpus's best-achievable geometric-mean latency by under 0.1%.
  struct Shape {
    int tq, tkv, d;
    std::vector<Org> orgs;
  };
  const std::vector<Shape> shapes = {
      {128, 32, 128, {kSplitK, kSplitKLpt, kNoSplitLpt, kSplitKXcd, kSplitK15Lpt, kSplitK2Lpt, kSplitKXcd128}},
      {128, 64, 128, {kSplitK, kSplitKLpt, kNoSplitLpt, kSplitKXcd, kSplitK15Lpt, kSplitK2Lpt, kSplitKXcd128}},
      {64, 64, 128, {kSplitK, kSplitKXcd}},
      {256, 64, 128, {kSplitK, kSplitKXcd, kSplitK15Lpt}},
      {128, 128, 128, {kSplitK}},
      {64, 64, 64, {kSplitK}},
      {64, 32, 64, {kSplitK, kNoSplitLpt, kSplitKXcd128}},
      {128, 32, 64, {kSplitK, kNoSplitLpt}},
      {128, 64, 64, {kSplitK, kNoSplitLpt, kSplitKLpt, kSplitK2Lpt, kSplitKXcd}},
      // further head dimensions (request property x, section 4.4), default
      // organization only (no profiled regimes: their requests use the base plan)
      {64, 32, 32, {kSplitK}},
      {64, 64, 32, {kSplitK}},
      {128, 64, 32, {kSplitK}},
      {128, 128, 32, {kSplitK}},
      {64, 32, 256, {kSplitK}},
      {128, 32, 256, {kSplitK}},
      // signature order (kept last so the ids of the entries above are stable)
      {128, 32, 128, {kSplitKSimXcd}},
      {128, 64, 128, {kSplitKSimXcd}},
  };
  std::vector<CatalogEntry> c;
  for (const Shape& sh : shapes) {
    for (const Org& o : sh.orgs) {
      CatalogEntry e;
      e.id = (int)c.size();
      e.tq = sh.tq;
      e.tkv = sh.tkv;
      e.d = sh.d;
      e.split = o.split;
      e.xcd_remap = o.xcd;
      e.order = o.order;
      char buf[48];
      std::snprintf(buf, sizeof buf, "T%dx%d_d%d_%s", e.tq, e.tkv, e.d, o.name);
      e.name = buf;
      c.push_back(e);
    }
  }
  return c;
}

struct Bounds {
  std::vector<double> H, N, density, runcov, skew;
};

// A threshold test on one regime feature (a decision-tree leaf is the
// conjunction of the tests on its path).
struct Cond {
  int feature;  // 0 H, 1 N, 2 density, 3 run coverage, 4 row skew
  bool less;    // true: x < v; false: x >= v
  double v;
};

struct Regime {
  int bq, bkv, d;
  int hb, nb, db, rb, sb;  // bucket index per feature, -1 = any
  std::vector<Cond> conds;  // rule regimes: every test must hold
  std::vector<int> ranking;
};

struct Table {
  std::string version = "builtin-empty";
  Bounds bounds;
  std::vector<Regime> regimes;
};

std::mutex g_table_mu;
Table g_table;
bool g_table_init = false;

int bucket(const std::vector<double>& b, double x) {
  int k = 0;
  while (k < (int)b.size() && x >= b[k]) ++k;
  return k;
}

const char* builtin_table_text();
bsa_status parse_table(const std::string& text, Table* out, std::string* err);

// Called with g_table_mu held: install the built-in artifact on first use.
void ensure_table() {
  if (g_table_init) return;
  g_table_init = true;
  Table t;
  std::string err;
  if (parse_table(builtin_table_text(), &t, &err) == BSA_OK) g_table = t;
}

}  // namespace

DimMap map_dim(int block, int tile, int min_coarsen_block) {
  DimMap m;
  if (block <= 0 || tile <= 0 || !pow2(block) || !pow2(tile)) return m;
  if (tile == block) {
    m.ok = true;
  } else if (tile > block) {
    if (block < min_coarsen_block) return m;
    m.ok = true;
    m.coarsen = tile / block;
  } else {
    m.ok = true;
    m.refine = block / tile;
  }
  return m;
}

const std::vector<CatalogEntry>& catalog() {
  static const std::vector<CatalogEntry> c = build_catalog();
  return c;
}

uint64_t catalog_hash_value() {
  // FNV-1a over every entry's name and parameters, so a table compiled for
  // another catalog (including one that only changed a parameter) is refused
  uint64_t h = 1469598103934665603ull;
  auto mix = [&](unsigned char ch) {
    h ^= ch;
    h *= 1099511628211ull;
  };
  for (auto& e : catalog()) {
    for (char ch : e.name) mix((unsigned char)ch);
    mix(0xff);
    for (int v : {e.tq, e.tkv, e.d, e.split, e.xcd_remap, e.order})
      for (int b = 0; b < 4; ++b) mix((unsigned char)(v >> (8 * b)));
  }
  return h;
}

bool eligible(const CatalogEntry& e, const bsa_request& r, int64_t ws_bytes, std::string* why) {
  auto no = [&](const char* s) {
    if (why) *why = s;
    return false;
  };
  if (r.dtype != BSA_DTYPE_BF16) return no("dtype");
  if (r.layout != BSA_LAYOUT_HND && r.layout != BSA_LAYOUT_NHD) return no("layout");
  if (r.d != e.d) return no("head dim");
  // a wave owns 32 query rows: a coarsened query tile needs B_Q >= 16 (with
  // B_Q = 16 the kernel resolves a wave's two logical rows per lane)
  DimMap mq = map_dim(r.block_q, e.tq, kMinCoarsenBlockQ);
  DimMap mk = map_dim(r.block_kv, e.tkv, 1);
  if (!mq.ok) return no("query geometry");
  if (!mk.ok) return no("key/value geometry");
  if (mq.coarsen * mk.coarsen > 32) return no("membership bits");
  if (ws_bytes >= 0 && r.workspace_limit > 0 && ws_bytes > r.workspace_limit) return no("workspace");
  return true;
}

int base_plan(const bsa_request& r) {
  const auto& c = catalog();
  for (auto& e : c)
    if (e.tq == r.block_q && e.tkv == r.block_kv && e.d == r.d && e.split == 2 && e.xcd_remap == 0 &&
        e.order == 0 && eligible(e, r, -1, nullptr))
      return e.id;
  int best = -1;
  for (auto& e : c) {
    if (e.split != 2 || e.xcd_remap != 0 || e.order != 0 || !eligible(e, r, -1, nullptr)) continue;
    if (best < 0 || e.tq * e.tkv < c[best].tq * c[best].tkv) best = e.id;
  }
  return best;
}

Selection lookup(const bsa_request& r, double density, double run_coverage, double row_skew) {
  std::lock_guard<std::mutex> lk(g_table_mu);
  ensure_table();
  Selection s;
  const Table& t = g_table;
  const int hb = bucket(t.bounds.H, r.H), nb = bucket(t.bounds.N, r.N);
  const int db = bucket(t.bounds.density, density), rb = bucket(t.bounds.runcov, run_coverage);
  const int sb = bucket(t.bounds.skew, row_skew);
  const double x[5] = {(double)r.H, (double)r.N, density, run_coverage, row_skew};
  for (size_t i = 0; i < t.regimes.size(); ++i) {
    const Regime& g = t.regimes[i];
    if (g.bq != r.block_q || g.bkv != r.block_kv || g.d != r.d) continue;
    if ((g.hb >= 0 && g.hb != hb) || (g.nb >= 0 && g.nb != nb) || (g.db >= 0 && g.db != db) ||
        (g.rb >= 0 && g.rb != rb) || (g.sb >= 0 && g.sb != sb))
      continue;
    bool ok = true;
    for (const Cond& c : g.conds) ok = ok && (c.less ? x[c.feature] < c.v : x[c.feature] >= c.v);
    if (!ok) continue;
    s.regime = (int)i;
    s.candidates = g.ranking;
    break;
  }
  const int base = base_plan(r);
  if (base >= 0 && std::find(s.candidates.begin(), s.candidates.end(), base) == s.candidates.end())
    s.candidates.push_back(base);
  return s;
}

// ---- table text format ------------------------------------------------------
//   bsa-plan-table <version>
//   arch gfx950
//   catalog <hex hash of the catalog>
//   bounds <H|N|density|run_coverage> v1 v2 ...     (bucket k: b[k-1] <= x < b[k])
//   bounds row_skew v1 ...   (row skew = max row count * rows / active blocks)
//   regime <B_Q> <B_KV> <d> <hb> <nb> <db> <rb> <sb> : <plan name> <plan name> ...
//   rule <B_Q> <B_KV> <d> [<feature><op><value> ...] : <plan name> ...
//       (a decision-tree leaf: feature in H N density run_coverage row_skew,
//        op '<' or '>=', every test must hold; no tests = the whole key)
// Lines starting with '#' are comments; '*' matches any bucket.  Regimes of
// both kinds are tried in file order and the first match is taken.
namespace {
bsa_status parse_table(const std::string& text, Table* out, std::string* err) {
  Table t;
  std::istringstream is(text);
  std::string line;
  bool have_header = false, have_arch = false, have_cat = false;
  int lineno = 0;
  auto fail = [&](const std::string& m) {
    if (err) *err = "plan table line " + std::to_string(lineno) + ": " + m;
    return BSA_ERR_TABLE;
  };
  std::vector<std::string> names;
  for (auto& e : catalog()) names.push_back(e.name);
  while (std::getline(is, line)) {
    ++lineno;
    if (line.empty() || line[0] == '#') continue;
    std::istringstream ls(line);
    std::string kw;
    ls >> kw;
    if (kw.empty()) continue;
    if (kw == "bsa-plan-table") {
      ls >> t.version;
      if (t.version.empty()) return fail("missing version");
      have_header = true;
    } else if (kw == "arch") {
      std::string a;
      ls >> a;
      if (a != "gfx950") return fail("table built for architecture " + a);
      have_arch = true;
    } else if (kw == "catalog") {
      std::string h;
      ls >> h;
      char buf[32];
      std::snprintf(buf, sizeof buf, "%016llx", (unsigned long long)catalog_hash_value());
      if (h != buf) return fail("catalog hash " + h + " does not match " + buf);
      have_cat = true;
    } else if (kw == "bounds") {
      std::string f;
      ls >> f;
      std::vector<double> v;
      double x;
      while (ls >> x) v.push_back(x);
      if (!std::is_sorted(v.begin(), v.end())) return fail("bounds not sorted");
      if (f == "H") t.bounds.H = v;
      else if (f == "N") t.bounds.N = v;
      else if (f == "density") t.bounds.density = v;
      else if (f == "run_coverage") t.bounds.runcov = v;
      else if (f == "row_skew") t.bounds.skew = v;
      else return fail("unknown feature " + f);
    } else if (kw == "regime" || kw == "rule") {
      Regime g;
      const int nfield = kw == "regime" ? 8 : 3;
      std::string tok[8];
      for (int i = 0; i < nfield; ++i) ls >> tok[i];
      for (int i = nfield; i < 8; ++i) tok[i] = "*";
      auto num = [&](const std::string& s, int* out) {
        if (s == "*") {
          *out = -1;
          return true;
        }
        char* end = nullptr;
        long v = std::strtol(s.c_str(), &end, 10);
        if (s.empty() || *end) return false;
        *out = (int)v;
        return true;
      };
      int* outs[8] = {&g.bq, &g.bkv, &g.d, &g.hb, &g.nb, &g.db, &g.rb, &g.sb};
      for (int i = 0; i < 8; ++i)
        if (!num(tok[i], outs[i])) return fail("bad regime field '" + tok[i] + "'");
      if (g.bq < 0 || g.bkv < 0 || g.d < 0) return fail("regime key must be explicit");
      if (kw == "rule") {
        static const char* feats[5] = {"H", "N", "density", "run_coverage", "row_skew"};
        std::string c;
        while (ls >> c && c != ":") {
          const size_t lt = c.find('<'), ge = c.find(">=");
          const bool less = lt != std::string::npos;
          const size_t at = less ? lt : ge;
          if (at == std::string::npos || at == 0) return fail("bad rule test '" + c + "'");
          const std::string f = c.substr(0, at), v = c.substr(at + (less ? 1 : 2));
          int fi = -1;
          for (int k = 0; k < 5; ++k)
            if (f == feats[k]) fi = k;
          if (fi < 0) return fail("unknown feature " + f);
          char* end = nullptr;
          const double x = std::strtod(v.c_str(), &end);
          if (v.empty() || *end) return fail("bad threshold '" + v + "'");
          g.conds.push_back({fi, less, x});
        }
        if (c != ":") return fail("expected ':'");
      } else {
        std::string colon;
        ls >> colon;
        if (colon != ":") return fail("expected ':'");
      }
      std::string nm;
      while (ls >> nm) {
        auto it = std::find(names.begin(), names.end(), nm);
        if (it == names.end()) return fail("unknown plan " + nm);
        g.ranking.push_back((int)(it - names.begin()));
      }
      if (g.ranking.empty()) return fail("empty ranking");
      t.regimes.push_back(g);
    } else {
      return fail("unknown keyword " + kw);
    }
  }
  if (!have_header || !have_arch || !have_cat) {
    lineno = 0;
    return fail("missing header, arch or catalog line");
  }
  *out = t;
  return BSA_OK;
}
}  // namespace

bsa_status table_load_text(const std::string& text, std::string* err) {
  Table t;
  bsa_status st = parse_table(text, &t, err);
  if (st != BSA_OK) return st;
  std::lock_guard<std::mutex> lk(g_table_mu);
  g_table = t;
  g_table_init = true;
  return BSA_OK;
}

bsa_status table_load_file(const char* path, std::string* err) {
  if (!path) {
    std::lock_guard<std::mutex> lk(g_table_mu);
    g_table_init = false;
    g_table = Table();
    ensure_table();
    return BSA_OK;
  }
  std::ifstream f(path);
  if (!f) {
    if (err) *err = std::string("cannot open plan table ") + path;
    return BSA_ERR_TABLE;
  }
  std::stringstream ss;
  ss << f.rdbuf();
  return table_load_text(ss.str(), err);
}

const std::string& table_version() {
  std::lock_guard<std::mutex> lk(g_table_mu);
  ensure_table();
  return g_table.version;
}

namespace {
const char* builtin_table_text() {
  return
#include "table_builtin.inc"
      ;
}
}  // namespace

}  // namespace bsa
