// qlin_table.cpp -- the offline per-shape selection table and the built-in
// default rule.
//
// "Building a High-Performance and Portable vLLM Linear Backend with Helion",
// section "Per-shape Config Tuning": every (GEMM shape, num_tokens) in the
// tuned range gets its own configuration, num_tokens in {1,2,4,8,16,24,32};
// section "Kernel Implementation": the schedule (split_k, swap_ab) is part of
// that configuration.  Here the configurations are measured offline on the
// GPU and stored as a text table; a runtime token count rounds up to the next
// tuned bucket.
//
// Table format (text, '#' starts a comment):
//   qlin-table <abi version> <gfx arch>
//   <format> <N> <K> <M bucket> <swap_ab> <split_k> <tile_m> <tile_n> <waves> <k_waves>
//            <reduce> <act_path>
// with <format> one of fp8_dynamic, w8a8_int8, block_fp8.
#include <dlfcn.h>

#include <cstdio>
#include <cstdlib>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "qlin_internal.h"

namespace qlin {
namespace {

typedef std::tuple<int, int, int, int> Key;  // fmt, N, K, M bucket

struct TableState {
    std::mutex mu;
    std::map<Key, qlin_config> entries;
    bool loaded = false;   // a load was attempted (explicitly or lazily)
    int strict = -1;       // -1: not decided yet (read QLIN_STRICT)
};

TableState &state() {
    static TableState s;
    return s;
}

const int kBuckets[] = {1, 2, 4, 8, 16, 24, 32, 64, 128, 256, 512};

int parse_format(const char *s) {
    if (!strcmp(s, "fp8_dynamic")) return QLIN_FP8_DYNAMIC;
    if (!strcmp(s, "w8a8_int8")) return QLIN_W8A8_INT8;
    if (!strcmp(s, "block_fp8")) return QLIN_BLOCK_FP8;
    return -1;
}

std::string default_table_path() {
    const char *env = getenv("QLIN_TABLE");
    if (env && *env) return env;
    Dl_info info;
    if (dladdr(reinterpret_cast<void *>(&default_table_path), &info) && info.dli_fname) {
        std::string p(info.dli_fname);
        const size_t slash = p.rfind('/');
        const std::string dir = slash == std::string::npos ? "." : p.substr(0, slash);
        return dir + "/tables/gfx950.tbl";
    }
    return "tables/gfx950.tbl";
}

// Parses a table file into `out`; QLIN_ERR_TABLE on any malformed line.
qlin_status parse_file(const std::string &path, std::map<Key, qlin_config> *out) {
    FILE *f = fopen(path.c_str(), "r");
    if (!f) return QLIN_ERR_TABLE;
    char line[512];
    bool header = false;
    qlin_status st = QLIN_OK;
    while (fgets(line, sizeof line, f)) {
        char *hash = strchr(line, '#');
        if (hash) *hash = 0;
        char a[64];
        if (sscanf(line, "%63s", a) != 1) continue;  // blank
        if (!header) {
            int ver = 0;
            char arch[64];
            if (sscanf(line, "qlin-table %d %63s", &ver, arch) != 2 || ver != QLIN_ABI_VERSION ||
                strcmp(arch, "gfx950") != 0) {
                st = QLIN_ERR_TABLE;
                break;
            }
            header = true;
            continue;
        }
        char fmt_s[64];
        int N, K, M, swap, split, tm, tn, waves, kwv, red, fuse;
        char extra[8];
        const int n = sscanf(line, "%63s %d %d %d %d %d %d %d %d %d %d %d %7s", fmt_s, &N, &K, &M,
                             &swap, &split, &tm, &tn, &waves, &kwv, &red, &fuse, extra);
        const int fmt = parse_format(fmt_s);
        if (n != 12 || fmt < 0) {
            st = QLIN_ERR_TABLE;
            break;
        }
        qlin_config c{swap, split, tm, tn, waves, kwv, red, fuse};
        Plan p;
        if (token_bucket(M) != M || make_plan((qlin_format)fmt, M, N, K, c, true, &p) != QLIN_OK) {
            st = QLIN_ERR_TABLE;
            break;
        }
        (*out)[Key(fmt, N, K, M)] = c;
    }
    fclose(f);
    if (st == QLIN_OK && !header) st = QLIN_ERR_TABLE;
    return st;
}

void ensure_loaded(TableState &s) {
    if (s.strict < 0) {
        const char *env = getenv("QLIN_STRICT");
        s.strict = (env && atoi(env) != 0) ? 1 : 0;
    }
    if (s.loaded) return;
    s.loaded = true;
    std::map<Key, qlin_config> m;
    if (parse_file(default_table_path(), &m) == QLIN_OK) s.entries.swap(m);
}

}  // namespace

int token_bucket(int M) {
    for (int b : kBuckets)
        if (M <= b) return b;
    return -1;  // beyond the largest bucket
}

bool strict_mode() {
    TableState &s = state();
    std::lock_guard<std::mutex> lk(s.mu);
    ensure_loaded(s);
    return s.strict == 1;
}

qlin_status table_lookup(qlin_format fmt, int M, int N, int K, qlin_config *out, bool *found) {
    TableState &s = state();
    std::lock_guard<std::mutex> lk(s.mu);
    ensure_loaded(s);
    *found = false;
    const int b = token_bucket(M);
    if (b < 0) return QLIN_OK;
    auto it = s.entries.find(Key((int)fmt, N, K, b));
    if (it != s.entries.end()) {
        *out = it->second;
        *found = true;
    }
    return QLIN_OK;
}

// Configuration of the tuned shape nearest to (N, K) in the same token
// bucket, for shapes the table does not list (permissive mode).  Distance is
// |log2 N/N'| + |log2 K/K'|, plus 1/2 for an entry of another per-token
// format (the fp8 and int8 schedules stream the same bytes) and 1 between
// the per-token and the block-scaled formats.  An entry whose configuration
// does not fit the shape is passed over (one with fused or direct
// activations first falls back to staged ones).
qlin_status table_nearest(qlin_format fmt, int M, int N, int K, qlin_config *out, bool *found) {
    TableState &s = state();
    std::lock_guard<std::mutex> lk(s.mu);
    ensure_loaded(s);
    *found = false;
    const int b = token_bucket(M);
    if (b < 0) return QLIN_OK;
    double best = 1e30;
    for (const auto &e : s.entries) {
        const int efmt = std::get<0>(e.first), eN = std::get<1>(e.first), eK = std::get<2>(e.first);
        if (std::get<3>(e.first) != b) continue;
        double d = fabs(log2((double)N / eN)) + fabs(log2((double)K / eK));
        if (efmt != (int)fmt) d += (efmt == QLIN_BLOCK_FP8) != (fmt == QLIN_BLOCK_FP8) ? 1.0 : 0.5;
        if (d >= best) continue;
        qlin_config c = e.second;
        Plan p;
        if (make_plan(fmt, M, N, K, c, true, &p) != QLIN_OK) {
            if (c.act_path == QLIN_ACT_STAGED) continue;
            c.act_path = QLIN_ACT_STAGED;
            if (make_plan(fmt, M, N, K, c, true, &p) != QLIN_OK) continue;
        }
        best = d;
        *out = c;
        *found = true;
    }
    return QLIN_OK;
}

// Built-in rule for shapes with no usable table entry (permissive mode, an
// empty table or more than 512 tokens).  Up to 64 tokens: 64-column tiles of
// four waves, each K block range shared by two waves, and the smallest
// power-of-two split that gives at least 192 workgroups (about three
// quarters of a workgroup per compute unit) while each wave keeps at least
// one K block; splits of four and more go through Swap-AB.  This is the
// pick that measured closest to the best forced schedule over the 8B-class
// shapes of all three formats.  Up to four tokens quantize inside the GEMM
// where the rows fit.  From 128 tokens on it takes the large-M kernel
// (64-token tiles).
void default_config(qlin_format fmt, int M, int N, int K, qlin_config *out) {
    qlin_config c;
    if (M >= 128) {
        // the large-M kernel, 64-token tiles, no split
        c = qlin_config{0, 1, 64, 128, 4, 1, 0, 0};
        *out = c;
        return;
    }
    c.tile_m = M <= 16 ? 16 : 32;
    c.waves = 4;
    c.k_waves = 2;
    c.tile_n = 64;
    const int n_tiles = (N + c.tile_n - 1) / c.tile_n;
    const int m_tiles = (M + c.tile_m - 1) / c.tile_m;
    const int nkb = (K + kGroup - 1) / kGroup;
    int split = 1;
    while (split < kMaxSplit && (int64_t)n_tiles * m_tiles * split < 192 &&
           nkb / (split * 2) >= c.k_waves)
        split *= 2;
    c.split_k = split;
    c.swap_ab = split >= 4 ? 1 : 0;
    c.reduce = 0;
    c.act_path = M <= 4 && c.tile_m == 16 ? QLIN_ACT_FUSED : QLIN_ACT_STAGED;
    Plan p;
    if (c.act_path == QLIN_ACT_FUSED && make_plan(fmt, M, N, K, c, true, &p) != QLIN_OK) c.act_path = QLIN_ACT_STAGED;
    *out = c;
}

}  // namespace qlin

using namespace qlin;

extern "C" qlin_status qlin_load_table(const char *path) {
    std::map<Key, qlin_config> m;
    const std::string p = path ? std::string(path) : default_table_path();
    const qlin_status st = parse_file(p, &m);
    if (st != QLIN_OK) return st;
    TableState &s = state();
    std::lock_guard<std::mutex> lk(s.mu);
    if (s.strict < 0) {
        const char *env = getenv("QLIN_STRICT");
        s.strict = (env && atoi(env) != 0) ? 1 : 0;
    }
    s.entries.swap(m);
    s.loaded = true;
    return QLIN_OK;
}

extern "C" qlin_status qlin_set_strict(int strict) {
    TableState &s = state();
    std::lock_guard<std::mutex> lk(s.mu);
    ensure_loaded(s);
    s.strict = strict ? 1 : 0;
    return QLIN_OK;
}

extern "C" int qlin_table_entries(void) {
    TableState &s = state();
    std::lock_guard<std::mutex> lk(s.mu);
    ensure_loaded(s);
    return (int)s.entries.size();
}
