// tune.cpp -- the table of measured tile picks (LyCORIS "Backend Selection"
// page, "Tile selection": a shortlist from an analytic model is timed once,
// best of three, and the winner cached in memory and in a JSON file, keyed by
// device, op, bucketed shape and dtype).  The timing itself runs in api.cpp
// (lyc_lora_linear_tune); this file keeps the table and its file format.
#include "tune.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>

#include "kernels.h"

namespace lyc {

namespace {
std::mutex g_mu;
std::map<std::string, TuneChoice> g_table;

// "gfx950-256cu" per device id, looked up once
std::string device_tag() {
    static std::mutex mu;
    static std::map<int, std::string> tags;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return std::string();
    std::lock_guard<std::mutex> lk(mu);
    auto it = tags.find(dev);
    if (it != tags.end()) return it->second;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return std::string();
    std::string arch(prop.gcnArchName);
    const size_t colon = arch.find(':');
    if (colon != std::string::npos) arch.resize(colon);
    const std::string tag = arch + "-" + std::to_string(prop.multiProcessorCount) + "cu";
    tags[dev] = tag;
    return tag;
}

int64_t bucket(int64_t m) {
    int64_t b = 16;
    while (b < m) b <<= 1;
    return b;
}

// the value after "name": on a line, as a string or a number
bool field(const char* line, const char* name, char* out, size_t n) {
    char pat[64];
    std::snprintf(pat, sizeof pat, "\"%s\":", name);
    const char* p = std::strstr(line, pat);
    if (!p) return false;
    p += std::strlen(pat);
    while (*p == ' ') ++p;
    size_t i = 0;
    if (*p == '"') {
        ++p;
        while (*p && *p != '"' && i + 1 < n) out[i++] = *p++;
        if (*p != '"') return false;
    } else {
        while (*p && *p != ',' && *p != '}' && *p != ' ' && i + 1 < n) out[i++] = *p++;
    }
    out[i] = 0;
    return i > 0;
}
}  // namespace

std::string tune_key(const char* op, int64_t M, int64_t N, int64_t K, int r_pad, int c_dt, int o_dt) {
    const std::string dev = device_tag();
    if (dev.empty()) return dev;
    char buf[256];
    std::snprintf(buf, sizeof buf, "%s|%s|M%lld|N%lld|K%lld|r%d|c%d|o%d", dev.c_str(), op, (long long)bucket(M),
                  (long long)N, (long long)K, r_pad, c_dt, o_dt);
    return buf;
}

bool tune_lookup(const std::string& key, TuneChoice* out) {
    if (key.empty()) return false;
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_table.find(key);
    if (it == g_table.end()) return false;
    if (out) *out = it->second;
    return true;
}

void tune_store(const std::string& key, const TuneChoice& c) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_table[key] = c;
}

int tune_count() {
    std::lock_guard<std::mutex> lk(g_mu);
    return (int)g_table.size();
}

void tune_clear() {
    std::lock_guard<std::mutex> lk(g_mu);
    g_table.clear();
}

// {"version": 1, "entries": [ one entry per line ]}
int tune_save(const char* path) {
    std::lock_guard<std::mutex> lk(g_mu);
    FILE* f = std::fopen(path, "w");
    if (!f) return -1;
    std::fprintf(f, "{\"version\": 1, \"entries\": [\n");
    size_t i = 0;
    for (const auto& kv : g_table) {
        int tn, tm;
        gemm_tile_dims(kv.second.tile, &tn, &tm);
        std::fprintf(f, "{\"key\": \"%s\", \"tile_n\": %d, \"tile_m\": %d, \"ksplit\": %d, \"ms\": %.6f}%s\n",
                     kv.first.c_str(), tn, tm, kv.second.ksplit, kv.second.ms, ++i < g_table.size() ? "," : "");
    }
    std::fprintf(f, "]}\n");
    return std::fclose(f) == 0 ? 0 : -1;
}

int tune_load(const char* path, int* loaded) {
    FILE* f = std::fopen(path, "r");
    if (!f) return -1;
    char line[1024], key[512], v[64];
    int n = 0, bad = 0;
    std::map<std::string, TuneChoice> got;
    while (std::fgets(line, sizeof line, f)) {
        if (!std::strstr(line, "\"key\":")) continue;
        TuneChoice c{-1, 1, 0.0};
        int tn = 0, tm = 0;
        if (!field(line, "key", key, sizeof key) || !field(line, "tile_n", v, sizeof v)) { ++bad; continue; }
        tn = std::atoi(v);
        if (!field(line, "tile_m", v, sizeof v)) { ++bad; continue; }
        tm = std::atoi(v);
        if (!field(line, "ksplit", v, sizeof v)) { ++bad; continue; }
        c.ksplit = std::atoi(v);
        if (field(line, "ms", v, sizeof v)) c.ms = std::atof(v);
        for (int t = 0; t < 4; ++t) {
            int a, b;
            gemm_tile_dims(t, &a, &b);
            if (a == tn && b == tm) c.tile = t;
        }
        if (c.tile < 0 || c.ksplit < 1 || c.ksplit > 8) { ++bad; continue; }
        got[key] = c;
        ++n;
    }
    std::fclose(f);
    if (bad) return -2;   // nothing is taken from a file with a malformed entry
    std::lock_guard<std::mutex> lk(g_mu);
    for (const auto& kv : got) g_table[kv.first] = kv.second;
    if (loaded) *loaded = n;
    return 0;
}

}  // namespace lyc
