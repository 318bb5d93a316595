// C ABI of the fused GEMM + bias + activation library (declared in gba.h):
// argument checks, device check, schedule choice (forced, on-disk cache, or
// heuristic), kernel launch, the autotuner and its schedule cache.
#include <errno.h>
#include <fcntl.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <sys/file.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "gba.h"
#include "gba_kernels.hpp"
#include "gba_registry.hpp"

#define GBA_VERSION_STRING "0.3.0"

namespace gba {
extern const ScheduleEntry s_128x128x32_w2x2;
extern const ScheduleEntry i_256x128x64_w2x2_s3_l4_p1_m16;
extern const ScheduleEntry i_128x256x64_w2x2_s3_l4_p1_m16;
extern const ScheduleEntry i_128x128x64_w2x2_s3_l4_p1_m16;
extern const ScheduleEntry i_128x128x64_w2x2_s4_l4_p1_m16;
extern const ScheduleEntry i_64x64x64_w4x1_s4_l4_p1_m16;
extern const ScheduleEntry p_256x256x64_w2x2;
extern const F8LaunchFn f8_e4m3[2][kNumActs];
extern const F8LaunchFn f8_e5m2[2][kNumActs];
extern const F8PartialLaunchFn f8_e4m3_part;
extern const F8PartialLaunchFn f8_e5m2_part;
}  // namespace gba

namespace {

using gba::ScheduleEntry;

const ScheduleEntry *const kTable[] = {
    // persistent kernel: one workgroup per CU walks its 256x256 tiles as one
    // stream of K slices (the built-in choice when the tiles fill the CUs)
    &gba::p_256x256x64_w2x2,
    // interleaved direct-to-LDS kernels with 16x16x32 MFMAs, one tile per workgroup
    &gba::i_256x128x64_w2x2_s3_l4_p1_m16, &gba::i_128x256x64_w2x2_s3_l4_p1_m16,
    &gba::i_128x128x64_w2x2_s3_l4_p1_m16, &gba::i_128x128x64_w2x2_s4_l4_p1_m16,
    &gba::i_64x64x64_w4x1_s4_l4_p1_m16,
    // register-staged kernel at the pages' 128x128x32 starting tile
    &gba::s_128x128x32_w2x2,
};
constexpr int kNumTable = sizeof(kTable) / sizeof(kTable[0]);
constexpr long long kLdsBytes = 160 * 1024;

thread_local hipStream_t t_stream = nullptr;
thread_local bool t_forced = false;
thread_local gba_schedule t_forced_sched;
thread_local int t_last_hip = 0;

// Per-candidate results of this thread's last gba_autotune call.
struct Trial {
    gba_schedule s;
    double ms;
    int resumed;   // 1: taken from the tuning journal, not timed by that call
};
thread_local std::vector<Trial> t_trials;

bool log_enabled() {
    static int v = -1;
    if (v < 0) {
        const char *e = getenv("GBA_LOG");
        v = (e && *e && strcmp(e, "0") != 0) ? 1 : 0;
    }
    return v == 1;
}

int hip_fail(hipError_t e) {
    t_last_hip = (int)e;
    return GBA_ERR_HIP;
}

// ------------------------------------------------------------- device ----

struct DeviceInfo {
    bool checked = false;
    bool ok = false;
    int cus = 0;
    std::string arch;
};

std::mutex g_dev_mu;
DeviceInfo g_dev[64];

// GBA_OK when the current device is a gfx950; fills *info.
int current_device(const DeviceInfo **info) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        t_last_hip = (int)e;
        return GBA_ERR_DEVICE;
    }
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DeviceInfo &d = g_dev[dev];
    if (!d.checked) {
        hipDeviceProp_t p;
        e = hipGetDeviceProperties(&p, dev);
        d.checked = true;
        if (e == hipSuccess) {
            d.arch = p.gcnArchName;
            d.cus = p.multiProcessorCount;
            d.ok = d.arch.compare(0, 6, "gfx950") == 0;
        } else {
            (void)hipGetLastError();
            t_last_hip = (int)e;
        }
        if (log_enabled())
            fprintf(stderr, "[gba] device %d arch=%s cus=%d supported=%d\n", dev, d.arch.c_str(),
                    d.cus, (int)d.ok);
    }
    *info = &d;
    return d.ok ? GBA_OK : GBA_ERR_DEVICE;
}

// ------------------------------------------------------------ argument checks --

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void *a, size_t an, const void *b, size_t bn) {
    if (!a || !b || an == 0 || bn == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

int check_enums(int act, int dtype) {
    if (dtype != GBA_DTYPE_F16 && dtype != GBA_DTYPE_BF16) return GBA_ERR_DTYPE;
    if (act < GBA_ACT_NONE || act > GBA_ACT_GELU_TANH) return GBA_ERR_ACT;
    return GBA_OK;
}

// Shared checks of the GEMM entry points. *nothing is set when there is no work.
// lay: operand layouts, LAY_TB (B stored (N,K)) | LAY_TA (A stored (K,M)): the
// bits of the public GBA_TRANSPOSE_B / GBA_TRANSPOSE_A flags.
constexpr int LAY_TB = GBA_TRANSPOSE_B, LAY_TA = GBA_TRANSPOSE_A;

int check_gemm_args(const void *A, const void *B, const void *bias, const void *C, int64_t M,
                    int64_t N, int64_t K, int act, int dtype, bool *nothing, int lay = 0) {
    int s = check_enums(act, dtype);
    if (s) return s;
    if (M < 0 || N < 0 || K < 0) return GBA_ERR_SHAPE;
    // 32-bit buffer offsets inside the kernels: a tile's byte offsets (256 rows of
    // A, 64 rows of B) stay below 2^31. With A stored (K,M), M is a row pitch
    // like N (64 rows of At per slice).
    if (M > ((lay & LAY_TA) ? (1LL << 23) : 0x7fffffffLL) || N > (1LL << 23) || K > (1LL << 21))
        return GBA_ERR_SHAPE;
    *nothing = (M == 0 || N == 0);
    if (*nothing) return GBA_OK;
    if (!C) return GBA_ERR_NULL;
    if (K > 0 && (!A || !B)) return GBA_ERR_NULL;
    if ((K % 8) || (N % 8) || ((lay & LAY_TA) && (M % 8))) return GBA_ERR_ALIGN;
    if (!aligned16(C) || (A && !aligned16(A)) || (B && !aligned16(B)) ||
        (bias && !aligned16(bias)))
        return GBA_ERR_ALIGN;
    const size_t cb = (size_t)M * N * 2;
    if (overlaps(C, cb, A, (size_t)M * K * 2) || overlaps(C, cb, B, (size_t)K * N * 2) ||
        overlaps(C, cb, bias, (size_t)N * 2))
        return GBA_ERR_ALIAS;
    return GBA_OK;
}

// ------------------------------------------------------------ schedules ----

int find_entry(const gba_schedule &s) {
    for (int i = 0; i < kNumTable; ++i) {
        const gba_schedule &t = kTable[i]->sched;
        if (t.bm == s.bm && t.bn == s.bn && t.bk == s.bk && t.wm == s.wm && t.wn == s.wn &&
            t.stages == s.stages && t.kernel == s.kernel && t.loaders == s.loaders &&
            t.spread == s.spread)
            return i;
    }
    return -1;
}

bool sched_valid(const gba_schedule &s) {
    if (find_entry(s) < 0) return false;
    if (s.raster != 0 && s.raster != 1) return false;
    if (s.group_m < 1 || s.group_m > 64) return false;
    return true;
}

long long lds_bytes(const gba_schedule &s) {
    return (long long)(s.bm * s.bk + s.bk * s.bn) * 2 * s.stages;
}

// Built-in choice when neither a forced schedule nor a cached one applies:
// for shapes that fill the CUs, 256x256 tiles on the persistent kernel (same
// tile and loop as kernel 3, measured 1-2% faster with one tile per CU and
// 4-6% faster with several) or 256x128 / 128x256 tiles, by rounds of tiles;
// below that the largest tile that still gives every CU about one tile.
gba_schedule heuristic(int64_t M, int64_t N, int cus, int lay) {
    auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    auto rounds = [&](int64_t t) { return (double)((t + cus - 1) / cus); };
    const int64_t want = (int64_t)cus * 9 / 10;
    const ScheduleEntry *half =
        M >= N ? &gba::i_256x128x64_w2x2_s3_l4_p1_m16 : &gba::i_128x256x64_w2x2_s3_l4_p1_m16;
    const int64_t t_full = tiles(256, 256), t_half = tiles(half->sched.bm, half->sched.bn);
    const ScheduleEntry *e;
    if (t_full >= want || t_half >= want) {
        // Whichever finishes in less time by rounds of one tile per CU: a
        // 256x256 round costs 1 (0.95 from the second round on, where the
        // persistent kernel overlaps each epilogue with the next tile), a
        // 256x128 round 0.58 (measured 0.53-0.62 of a 256x256 round). So 1.25
        // or 1.5 rounds of 256x256 tiles (4096x5120, 6144x4096: 2 rounds) lose
        // to 3 rounds of half tiles (8-18 % faster measured), 1.56 rounds
        // (5120x5120) do not, nor does 0.75 of a round (3072x4096: 256x256
        // 25 % faster than 2 rounds of half tiles).
        const double r_full = rounds(t_full) * (rounds(t_full) >= 2 ? 0.95 : 1.0);
        const double r_half = rounds(t_half) * 0.58;
        e = r_full <= r_half ? &gba::p_256x256x64_w2x2 : half;
    } else if (2 * tiles(128, 128) > cus || (lay & LAY_TA))   // 64x64 has no (K,M) A path
        e = &gba::i_128x128x64_w2x2_s4_l4_p1_m16;   // 4 stages: 10-20 % faster than 3 here
    else
        // 128x128 tiles would leave half the CUs or more idle: 4x the tiles
        // (1024^3 5-21 % faster, 1024x2048x1024 10 %, K = 4096..8192 40-50 %;
        // at 144 and 256 tiles of 128x128 the larger tile is 24-26 % faster)
        e = &gba::i_64x64x64_w4x1_s4_l4_p1_m16;
    return e->sched;
}

// ------------------------------------------------------------ disk cache ----
//
// The schedule cache of the autotuner ("TileLang: Write, Autotune, and Ship
// Fused Tensor-Core Kernels from Python", Autotuning: how it works and how much
// it costs: re-runs hit an on-disk cache, which can be kept across CI runs and
// switched off by an environment variable). One JSON object per line in
// $GBA_CACHE_DIR/schedules.json, keyed by (arch, CU count, build id, dtype,
// act, operand layouts, M, N, K). The build id is a hash of the library's
// sources, so a schedule timed on other kernels is never used (its entry stays
// in the file for the build that wrote it). Every write re-reads the file under
// an exclusive flock on schedules.json.lock and merges into it, so concurrent
// writers lose nothing; the merged file replaces the old one by rename, so a
// reader never sees half of it. The in-memory copy is tied to the file's path:
// a changed GBA_CACHE_DIR is re-read. Tuning progress (each timed candidate)
// goes to tuning.json in the same directory with the same rules, so that an
// interrupted or budget-limited tuning run resumes where it stopped.

#ifndef GBA_BUILD_ID
#define GBA_BUILD_ID "unhashed"
#endif

const char *kDtName[2] = {"f16", "bf16"};
const char *kActName[gba::kNumActs] = {"none", "relu", "sigmoid", "gelu", "softplus", "gelu_tanh"};

struct CacheRec {
    gba_schedule s;
    double ms;
};
using CacheMap = std::unordered_map<std::string, CacheRec>;

std::mutex g_cache_mu;          // guards the three below
bool g_cache_loaded = false;
std::string g_cache_path;       // file the in-memory copy was read from
CacheMap g_cache;

bool cache_disabled() {
    const char *e = getenv("GBA_DISABLE_CACHE");
    return e && *e && strcmp(e, "0") != 0;
}

std::string cache_dir() {
    const char *d = getenv("GBA_CACHE_DIR");
    if (d && *d) return d;
    const char *h = getenv("HOME");
    return std::string(h && *h ? h : "/tmp") + "/.cache/gba";
}

std::string cache_file() { return cache_dir() + "/schedules.json"; }
std::string journal_file() { return cache_dir() + "/tuning.json"; }

// Layout in the key: "nn", "nt" (B stored (N,K)), "tn" (A stored (K,M)), "tt".
const char *kLayName[4] = {"nn", "nt", "tn", "tt"};
std::string cache_key(const char *arch, int cus, int dtype, int act, int lay, int64_t M, int64_t N,
                      int64_t K) {
    char buf[320];
    snprintf(buf, sizeof buf, "%s|%d|%s|%s|%s|%s|%lld|%lld|%lld", arch, cus, GBA_BUILD_ID,
             kDtName[dtype], kActName[act],
             kLayName[((lay & LAY_TA) ? 2 : 0) | ((lay & LAY_TB) ? 1 : 0)], (long long)M,
             (long long)N, (long long)K);
    return buf;
}
std::string cache_key(const DeviceInfo &d, int dtype, int act, int lay, int64_t M, int64_t N,
                      int64_t K) {
    return cache_key(d.arch.c_str(), d.cus, dtype, act, lay, M, N, K);
}

bool json_int(const char *line, const char *name, int *out) {
    char pat[64];
    snprintf(pat, sizeof pat, "\"%s\":", name);
    const char *p = strstr(line, pat);
    if (!p) return false;
    p += strlen(pat);
    char *end;
    long v = strtol(p, &end, 10);
    if (end == p) return false;
    *out = (int)v;
    return true;
}

// One record per line: {"key": "...", "bm": 256, ..., "ms": 0.08}. A file
// without the format header, and lines that do not parse or name no
// compiled-in schedule, are skipped. Several records may share a key (the
// tuning journal); `add` sees each in file order.
template <class F>
void read_records(const std::string &path, F add) {
    FILE *f = fopen(path.c_str(), "r");
    if (!f) return;
    char line[1024];
    bool header_ok = false;
    while (fgets(line, sizeof line, f)) {
        if (strstr(line, "\"format\": \"gba-schedule-cache\"") && strstr(line, "\"version\": 1"))
            header_ok = true;
        if (!header_ok) continue;
        const char *k = strstr(line, "\"key\": \"");
        if (!k) continue;
        k += 8;
        const char *ke = strchr(k, '"');
        if (!ke) continue;
        CacheRec r;
        if (!json_int(line, "bm", &r.s.bm) || !json_int(line, "bn", &r.s.bn) ||
            !json_int(line, "bk", &r.s.bk) || !json_int(line, "wm", &r.s.wm) ||
            !json_int(line, "wn", &r.s.wn) || !json_int(line, "stages", &r.s.stages) ||
            !json_int(line, "raster", &r.s.raster) || !json_int(line, "group_m", &r.s.group_m) ||
            !json_int(line, "kernel", &r.s.kernel) || !json_int(line, "loaders", &r.s.loaders) ||
            !json_int(line, "spread", &r.s.spread))
            continue;
        const char *m = strstr(line, "\"ms\":");
        r.ms = m ? atof(m + 5) : 0.0;
        if (!sched_valid(r.s)) continue;
        add(std::string(k, ke), r);
    }
    fclose(f);
}

int mkdir_p(const std::string &path) {
    std::string cur;
    for (size_t i = 0; i < path.size(); ++i) {
        cur += path[i];
        if ((path[i] == '/' && i > 0) || i + 1 == path.size()) {
            if (mkdir(cur.c_str(), 0755) != 0 && errno != EEXIST) return -1;
        }
    }
    struct stat st;
    return stat(path.c_str(), &st) == 0 && S_ISDIR(st.st_mode) ? 0 : -1;
}

// Writes records (key, rec) to `path` through a temporary file and a rename.
int write_records(const std::string &path, const std::vector<std::pair<std::string, CacheRec>> &recs) {
    static std::atomic<unsigned> serial{0};
    char tmpn[96];
    snprintf(tmpn, sizeof tmpn, ".tmp.%d.%u", (int)getpid(), serial.fetch_add(1));
    const std::string tmp = path + tmpn;
    FILE *f = fopen(tmp.c_str(), "w");
    if (!f) return GBA_ERR_CACHE;
    fprintf(f, "{\"format\": \"gba-schedule-cache\", \"version\": 1, \"entries\": [\n");
    for (size_t i = 0; i < recs.size(); ++i) {
        const gba_schedule &s = recs[i].second.s;
        fprintf(f,
                "{\"key\": \"%s\", \"bm\": %d, \"bn\": %d, \"bk\": %d, \"wm\": %d, \"wn\": %d, "
                "\"stages\": %d, \"raster\": %d, \"group_m\": %d, \"kernel\": %d, "
                "\"loaders\": %d, \"spread\": %d, \"ms\": %.6f}%s\n",
                recs[i].first.c_str(), s.bm, s.bn, s.bk, s.wm, s.wn, s.stages, s.raster, s.group_m,
                s.kernel, s.loaders, s.spread, recs[i].second.ms, i + 1 < recs.size() ? "," : "");
    }
    fprintf(f, "]}\n");
    bool ok = fflush(f) == 0;
    ok = fsync(fileno(f)) == 0 && ok;
    ok = fclose(f) == 0 && ok;
    if (!ok || rename(tmp.c_str(), path.c_str()) != 0) {
        unlink(tmp.c_str());
        return GBA_ERR_CACHE;
    }
    return GBA_OK;
}

// Exclusive advisory lock on <dir>/schedules.json.lock for a read-merge-write
// of the cache or the journal; -1 if the directory cannot be made or locked.
int lock_cache_dir() {
    const std::string dir = cache_dir();
    if (mkdir_p(dir) != 0) return -1;
    const int fd = open((dir + "/schedules.json.lock").c_str(), O_RDWR | O_CREAT | O_CLOEXEC, 0644);
    if (fd < 0) return -1;
    while (flock(fd, LOCK_EX) != 0) {
        if (errno != EINTR) {
            close(fd);
            return -1;
        }
    }
    return fd;
}
void unlock_cache_dir(int fd) {
    flock(fd, LOCK_UN);
    close(fd);
}

// Brings the in-memory copy up to date with the current cache file (read once
// per path). Caller holds g_cache_mu.
void cache_sync_locked() {
    const std::string path = cache_file();
    if (g_cache_loaded && path == g_cache_path) return;
    g_cache.clear();
    g_cache_path = path;
    g_cache_loaded = true;
    read_records(path, [](const std::string &k, const CacheRec &r) { g_cache[k] = r; });
}

// The cached schedule for `key`, if the cache is on and holds one.
bool cache_get(const std::string &key, CacheRec *out) {
    if (cache_disabled()) return false;
    std::lock_guard<std::mutex> lk(g_cache_mu);
    cache_sync_locked();
    auto it = g_cache.find(key);
    if (it == g_cache.end()) return false;
    *out = it->second;
    return true;
}

// Merges (key, rec) into the cache file and the in-memory copy. GBA_OK when
// the cache is disabled (nothing written), GBA_ERR_CACHE if it cannot be
// written.
int cache_put(const std::string &key, const CacheRec &rec) {
    if (cache_disabled()) return GBA_OK;
    std::lock_guard<std::mutex> lk(g_cache_mu);
    const int fd = lock_cache_dir();
    if (fd < 0) return GBA_ERR_CACHE;
    const std::string path = cache_file();
    CacheMap merged;
    read_records(path, [&](const std::string &k, const CacheRec &r) { merged[k] = r; });
    merged[key] = rec;
    std::vector<std::pair<std::string, CacheRec>> recs(merged.begin(), merged.end());
    std::sort(recs.begin(), recs.end(),
              [](const std::pair<std::string, CacheRec> &a, const std::pair<std::string, CacheRec> &b) {
                  return a.first < b.first;
              });
    const int st = write_records(path, recs);
    unlock_cache_dir(fd);
    g_cache = std::move(merged);
    g_cache_path = path;
    g_cache_loaded = true;
    return st;
}

bool same_sched(const gba_schedule &a, const gba_schedule &b) {
    return a.bm == b.bm && a.bn == b.bn && a.bk == b.bk && a.wm == b.wm && a.wn == b.wn &&
           a.stages == b.stages && a.raster == b.raster && a.group_m == b.group_m &&
           a.kernel == b.kernel && a.loaders == b.loaders && a.spread == b.spread;
}

// Tuning journal: the candidates already timed for `key`.
std::vector<CacheRec> journal_get(const std::string &key) {
    std::vector<CacheRec> out;
    if (cache_disabled()) return out;
    std::lock_guard<std::mutex> lk(g_cache_mu);
    const int fd = lock_cache_dir();
    if (fd < 0) return out;
    read_records(journal_file(), [&](const std::string &k, const CacheRec &r) {
        if (k == key) out.push_back(r);
    });
    unlock_cache_dir(fd);
    return out;
}

// Replaces the journal's records for `key` by `recs` (none: the key's tuning is
// finished), keeping every other key's.
int journal_set(const std::string &key, const std::vector<CacheRec> &recs) {
    if (cache_disabled()) return GBA_OK;
    std::lock_guard<std::mutex> lk(g_cache_mu);
    const int fd = lock_cache_dir();
    if (fd < 0) return GBA_ERR_CACHE;
    const std::string path = journal_file();
    std::vector<std::pair<std::string, CacheRec>> all;
    read_records(path, [&](const std::string &k, const CacheRec &r) {
        if (k != key) all.emplace_back(k, r);
    });
    for (const CacheRec &r : recs) all.emplace_back(key, r);
    int st = GBA_OK;
    if (all.empty()) {
        if (unlink(path.c_str()) != 0 && errno != ENOENT) st = GBA_ERR_CACHE;
    } else {
        st = write_records(path, all);
    }
    unlock_cache_dir(fd);
    return st;
}

gba_schedule choose(const DeviceInfo &d, int64_t M, int64_t N, int64_t K, int act, int dtype,
                    int lay, const char **why) {
    if (t_forced) {
        *why = "forced";
        return t_forced_sched;
    }
    CacheRec rec;
    if (cache_get(cache_key(d, dtype, act, lay, M, N, K), &rec)) {
        *why = "cache";
        return rec.s;
    }
    *why = "heuristic";
    return heuristic(M, N, d.cus, lay);
}

// The instance of schedule s for (dtype, act, operand layouts), or null.
gba::GemmLaunchFn launcher(const gba_schedule &s, int dtype, int act, int lay) {
    const int i = find_entry(s);
    if (i < 0) return nullptr;
    const bool tb = (lay & LAY_TB) != 0;
    if (lay & LAY_TA) return kTable[i]->ta[tb ? 1 : 0][dtype][act];
    return tb ? kTable[i]->tb[dtype][act] : kTable[i]->fn[dtype][act];
}

// Split-K first pass of schedule entry i for (dtype, operand layouts), or null.
gba::PartialLaunchFn partial_launcher(int i, int dtype, int lay) {
    const int tb = (lay & LAY_TB) ? 1 : 0;
    return (lay & LAY_TA) ? kTable[i]->part_ta[dtype][tb] : kTable[i]->part[dtype][tb];
}

// The persistent kernel streams at least two K slices per tile. With one (K <=
// 64) it hands the call to the 128x128 four-stage kernel 3: per output element
// the same MFMAs in the same order (two 32-deep steps), so the same bits.
gba_schedule effective(const gba_schedule &s0, int64_t K) {
    if (s0.kernel == 4 && K <= s0.bk) {
        gba_schedule s = gba::i_128x128x64_w2x2_s4_l4_p1_m16.sched;
        s.raster = s0.raster;
        s.group_m = s0.group_m;
        return s;
    }
    return s0;
}

int launch(const gba_schedule &s0, const void *A, const void *B, const void *bias, void *C,
           int64_t M, int64_t N, int64_t K, int act, int dtype, int lay) {
    const gba_schedule s = effective(s0, K);
    const gba::GemmLaunchFn f = launcher(s, dtype, act, lay);
    if (!f) return GBA_ERR_SCHEDULE;   // unknown, or no path for these layouts in this kernel
    hipError_t e = f(A, B, bias, C, (int)M, (int)N, (int)K, s.raster, s.group_m, t_stream);
    return e == hipSuccess ? GBA_OK : hip_fail(e);
}

// Split-K factor for schedule s: > 1 only for schedules with a split-K first
// pass, when their tiles leave CUs idle and the split pays for itself. Units
// (tiles x splits) stay within the CU count, each split keeps at least two K
// slices, at most 16 splits. Cost model (measured on MI355X): a K slice takes
// ~0.37 us per 128x128 tile and ~0.22 us per 64x64 tile (latency-bound); the
// split adds the fp32 partials' round trip, 2 S M N 4 bytes at ~4 TB/s, and
// ~6 us for the second kernel, its launch and the first pass's short units.
// Split only if that saves at least 15 %. (At 1024^3 it does not; at
// 256x256x4096 it does: 11.3 us split against 14.7 us whole; at 129x136x2056
// it does not: 10.1 us split against 9.6 us whole.) *t_pred: the model's time
// for the returned factor.
int split_count(const gba_schedule &s0, int64_t M, int64_t N, int64_t K, int cus, int dtype,
                int lay, double *t_pred = nullptr) {
    const gba_schedule s = effective(s0, K);
    const int i = find_entry(s);
    const int64_t nk = K > 0 ? (K + s.bk - 1) / s.bk : 0;
    const double t_slice = (int64_t)s.bm * s.bn <= 64 * 64 ? 0.22e-6 : 0.37e-6;
    const double bw = 4.0e12, t_fixed = 6.0e-6;
    const double whole = nk * t_slice;
    if (t_pred) *t_pred = whole;
    if (i < 0 || !partial_launcher(i, dtype, lay) || K <= 0) return 1;
    const int64_t tiles = ((M + s.bm - 1) / s.bm) * ((N + s.bn - 1) / s.bn);
    int64_t smax = tiles > 0 ? cus / tiles : 1;
    smax = std::min<int64_t>(smax, nk / 2);
    smax = std::min<int64_t>(smax, 16);
    int best = 1;
    double best_t = whole;
    for (int64_t S = 2; S <= smax; ++S) {
        const double t = ((nk + S - 1) / S) * t_slice + 2.0 * S * (double)M * N * 4.0 / bw + t_fixed;
        if (t < best_t) {
            best_t = t;
            best = (int)S;
        }
    }
    if (best_t < 0.85 * whole) {
        if (t_pred) *t_pred = best_t;
        return best;
    }
    return 1;
}

// Schedule and split factor of a call that may split K. The chosen schedule
// with split_count's factor; but when the built-in choice is the 64x64 tile
// (few tiles), the 128x128 tile split instead if the model predicts that
// faster: its fewer tiles leave room for more splits (128x4096x14336: 64x64
// whole 50 us, 64x64 in 2 splits 33 us, 128x128 in 8 splits 28 us).
int split_plan(const DeviceInfo &d, int64_t M, int64_t N, int64_t K, int act, int dtype, int lay,
               gba_schedule *sch, const char **why) {
    *sch = choose(d, M, N, K, act, dtype, lay, why);
    double t = 0.0;
    int S = split_count(*sch, M, N, K, d.cus, dtype, lay, &t);
    const gba_schedule &small = gba::i_64x64x64_w4x1_s4_l4_p1_m16.sched;
    if (strcmp(*why, "heuristic") == 0 && sch->bm == small.bm && sch->bn == small.bn) {
        const gba_schedule alt = gba::i_128x128x64_w2x2_s4_l4_p1_m16.sched;
        double t2 = 0.0;
        const int S2 = split_count(alt, M, N, K, d.cus, dtype, lay, &t2);
        if (S2 > 1 && t2 < t) {
            *sch = alt;
            S = S2;
        }
    }
    return S;
}

template <int DT, int ACT>
hipError_t launch_splitk_reduce_t(const float *P, int S, const void *bias, void *C, int M, int N,
                                  hipStream_t st) {
    const int cpr = N / 8;
    const int gx = (cpr + 255) / 256;
    int gy = M;
    const int max_y = std::max(1, 8192 / gx);
    if (gy > max_y) gy = max_y;
    hipLaunchKernelGGL((gba::splitk_reduce_kernel<DT, ACT>), dim3(gx, gy), dim3(256), 0, st, P, S,
                       (const uint16_t *)bias, (uint16_t *)C, M, N);
    return hipGetLastError();
}

using ReduceFn = hipError_t (*)(const float *, int, const void *, void *, int, int, hipStream_t);
const ReduceFn kReduce[2][gba::kNumActs] = {
    {launch_splitk_reduce_t<0, 0>, launch_splitk_reduce_t<0, 1>, launch_splitk_reduce_t<0, 2>,
     launch_splitk_reduce_t<0, 3>, launch_splitk_reduce_t<0, 4>, launch_splitk_reduce_t<0, 5>},
    {launch_splitk_reduce_t<1, 0>, launch_splitk_reduce_t<1, 1>, launch_splitk_reduce_t<1, 2>,
     launch_splitk_reduce_t<1, 3>, launch_splitk_reduce_t<1, 4>, launch_splitk_reduce_t<1, 5>},
};

int gemm_common(const void *A, const void *B, const void *bias, void *C, int64_t M, int64_t N,
                int64_t K, int act, int dtype, int lay, void *ws = nullptr, size_t ws_bytes = 0) {
    bool nothing = false;
    int s = check_gemm_args(A, B, bias, C, M, N, K, act, dtype, &nothing, lay);
    if (s || nothing) return s;
    if (ws) {
        if (!aligned16(ws)) return GBA_ERR_ALIGN;
        if (overlaps(ws, ws_bytes, A, (size_t)M * K * 2) || overlaps(ws, ws_bytes, B, (size_t)K * N * 2) ||
            overlaps(ws, ws_bytes, bias, (size_t)N * 2) || overlaps(ws, ws_bytes, C, (size_t)M * N * 2))
            return GBA_ERR_ALIAS;
    }
    const DeviceInfo *d;
    s = current_device(&d);
    if (s) return s;
    const char *why = "";
    if (ws) {
        gba_schedule ss;
        const int S = split_plan(*d, M, N, K, act, dtype, lay, &ss, &why);
        if (S > 1 && ws_bytes >= (size_t)S * (size_t)M * (size_t)N * 4u) {
            if (log_enabled())
                fprintf(stderr, "[gba] M=%lld N=%lld K=%lld act=%s dtype=%s -> split-K %d x k%d %dx%dx%d (%s)\n",
                        (long long)M, (long long)N, (long long)K, kActName[act], kDtName[dtype], S,
                        ss.kernel, ss.bm, ss.bn, ss.bk, why);
            const gba_schedule s3 = effective(ss, K);
            const gba::PartialLaunchFn pf = partial_launcher(find_entry(s3), dtype, lay);
            hipError_t e = pf(A, B, (float *)ws, (int)M, (int)N, (int)K, S, s3.raster, s3.group_m,
                              t_stream);
            if (e != hipSuccess) return hip_fail(e);
            e = kReduce[dtype][act]((const float *)ws, S, bias, C, (int)M, (int)N, t_stream);
            return e == hipSuccess ? GBA_OK : hip_fail(e);
        }
    }
    const gba_schedule sch = choose(*d, M, N, K, act, dtype, lay, &why);
    if (log_enabled())
        fprintf(stderr,
                "[gba] M=%lld N=%lld K=%lld act=%s dtype=%s A=%s B=%s -> k%d %dx%dx%d w%dx%d s%d r%d "
                "g%d (%s)\n",
                (long long)M, (long long)N, (long long)K, kActName[act], kDtName[dtype],
                (lay & LAY_TA) ? "KM" : "MK", (lay & LAY_TB) ? "NK" : "KN", sch.kernel, sch.bm, sch.bn, sch.bk, sch.wm, sch.wn, sch.stages,
                sch.raster, sch.group_m, why);
    return launch(sch, A, B, bias, C, M, N, K, act, dtype, lay);
}

template <int DT, int ACT>
hipError_t launch_bias_act_t(const void *X, const void *bias, void *Y, int M, int N,
                             hipStream_t st) {
    const int cpr = N / 8;
    const int gx = (cpr + 255) / 256;
    // Enough workgroups to keep every CU busy several times over; each thread
    // then walks rows with a 4-row unroll.
    int gy = gba::ceil_div(M, 4);
    const int max_y = std::max(1, 4096 / gx);
    if (gy > max_y) gy = max_y;
    hipLaunchKernelGGL((gba::bias_act_kernel<DT, ACT>), dim3(gx, gy), dim3(256), 0, st,
                       (const uint16_t *)X, (const uint16_t *)bias, (uint16_t *)Y, M, N);
    return hipGetLastError();
}

using BiasActFn = hipError_t (*)(const void *, const void *, void *, int, int, hipStream_t);
const BiasActFn kBiasAct[2][gba::kNumActs] = {
    {launch_bias_act_t<0, 0>, launch_bias_act_t<0, 1>, launch_bias_act_t<0, 2>, launch_bias_act_t<0, 3>,
     launch_bias_act_t<0, 4>, launch_bias_act_t<0, 5>},
    {launch_bias_act_t<1, 0>, launch_bias_act_t<1, 1>, launch_bias_act_t<1, 2>, launch_bias_act_t<1, 3>,
     launch_bias_act_t<1, 4>, launch_bias_act_t<1, 5>},
};

// Split factor of the 8-bit kernel (256x256 tiles, 128-deep slices): as
// split_count, with the 8-bit slice time (~1.8 us per 256x256x128 slice).
int split_count_fp8(int64_t M, int64_t N, int64_t K, int cus) {
    if (K <= 0) return 1;
    const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t nk = (K + 127) / 128;
    int64_t smax = tiles > 0 ? cus / tiles : 1;
    smax = std::min<int64_t>(smax, nk / 2);
    smax = std::min<int64_t>(smax, 16);
    const double t_slice = 1.8e-6, bw = 4.0e12, t_fixed = 5.0e-6;
    const double whole = std::max<int64_t>(nk, 2) * t_slice;
    int best = 1;
    double best_t = whole;
    for (int64_t S = 2; S <= smax; ++S) {
        const double t = ((nk + S - 1) / S) * t_slice + 2.0 * S * (double)M * N * 4.0 / bw + t_fixed;
        if (t < best_t) {
            best_t = t;
            best = (int)S;
        }
    }
    return best_t < 0.85 * whole ? best : 1;
}

int fp8_common(const void *A, const void *W, const void *bias, void *C, int64_t M, int64_t N,
               int64_t K, float scale, int act, int fmt, int dtype, void *ws, size_t ws_bytes) {
    int s = check_enums(act, dtype);
    if (s) return s;
    if (fmt != GBA_FP8_E4M3 && fmt != GBA_FP8_E5M2) return GBA_ERR_DTYPE;
    if (M < 0 || N < 0 || K < 0) return GBA_ERR_SHAPE;
    if (M > 0x7fffffffLL || N > (1LL << 23) || K > (1LL << 21)) return GBA_ERR_SHAPE;
    if (!(scale == scale) || scale - scale != 0.0f) return GBA_ERR_SHAPE;   // NaN or inf
    if (M == 0 || N == 0) return GBA_OK;
    if (!C) return GBA_ERR_NULL;
    if (K > 0 && (!A || !W)) return GBA_ERR_NULL;
    if ((K % 16) || (N % 8)) return GBA_ERR_ALIGN;
    if (!aligned16(C) || (A && !aligned16(A)) || (W && !aligned16(W)) || (bias && !aligned16(bias)))
        return GBA_ERR_ALIGN;
    const size_t cb = (size_t)M * N * 2;
    if (overlaps(C, cb, A, (size_t)M * K) || overlaps(C, cb, W, (size_t)N * K) ||
        overlaps(C, cb, bias, (size_t)N * 2))
        return GBA_ERR_ALIAS;
    if (ws) {
        if (!aligned16(ws)) return GBA_ERR_ALIGN;
        if (overlaps(ws, ws_bytes, A, (size_t)M * K) || overlaps(ws, ws_bytes, W, (size_t)N * K) ||
            overlaps(ws, ws_bytes, bias, (size_t)N * 2) || overlaps(ws, ws_bytes, C, cb))
            return GBA_ERR_ALIAS;
    }
    const DeviceInfo *d;
    s = current_device(&d);
    if (s) return s;
    if (ws) {
        const int S = split_count_fp8(M, N, K, d->cus);
        if (S > 1 && ws_bytes >= (size_t)S * (size_t)M * (size_t)N * 4u) {
            if (log_enabled())
                fprintf(stderr, "[gba] fp8 M=%lld N=%lld K=%lld -> split-K %d\n", (long long)M,
                        (long long)N, (long long)K, S);
            const gba::F8PartialLaunchFn pf =
                fmt == GBA_FP8_E4M3 ? gba::f8_e4m3_part : gba::f8_e5m2_part;
            hipError_t e = pf(A, W, (float *)ws, (int)M, (int)N, (int)K, scale, S, 1, 4, t_stream);
            if (e != hipSuccess) return hip_fail(e);
            e = kReduce[dtype][act]((const float *)ws, S, bias, C, (int)M, (int)N, t_stream);
            return e == hipSuccess ? GBA_OK : hip_fail(e);
        }
    }
    const gba::F8LaunchFn f = (fmt == GBA_FP8_E4M3 ? gba::f8_e4m3 : gba::f8_e5m2)[dtype][act];
    if (log_enabled())
        fprintf(stderr, "[gba] fp8 M=%lld N=%lld K=%lld act=%s fmt=%s out=%s scale=%g\n",
                (long long)M, (long long)N, (long long)K, kActName[act],
                fmt == GBA_FP8_E4M3 ? "e4m3" : "e5m2", kDtName[dtype], (double)scale);
    hipError_t e = f(A, W, bias, C, (int)M, (int)N, (int)K, scale, 1, 4, t_stream);
    return e == hipSuccess ? GBA_OK : hip_fail(e);
}

// ------------------------------------------------- static scratch ----
//
// Device memory for callers that cannot allocate (gemm_bias_act_noalloc): the
// split-K partial sums live in this file-scope array instead of a caller's
// workspace. Every GPU the library runs on holds its own copy until the process
// ends. Host code never uses the array's name as an address: the device address
// is taken once per device with hipGetSymbolAddress (with that device current)
// and kept in g_scratch[].
//
// Size: the split needs S * M * N * 4 bytes with S <= CUs / tiles of 128 x 128,
// so at most CUs * 128 * 128 * 4 bytes = 16 MiB on a 256-CU MI355X.
constexpr size_t kScratchBytes = (size_t)16 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch[64];   // device address of `scratch` per device (null: not taken yet)

int scratch_of_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        t_last_hip = (int)e;
        return GBA_ERR_DEVICE;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return GBA_OK;
}

}  // namespace

// =================================================================== C ABI ===

extern "C" {

const char *gba_version(void) { return GBA_VERSION_STRING; }

const char *gba_status_string(int s) {
    switch (s) {
    case GBA_OK: return "ok";
    case GBA_ERR_NULL: return "null pointer";
    case GBA_ERR_SHAPE: return "bad shape";
    case GBA_ERR_DTYPE: return "bad dtype";
    case GBA_ERR_ACT: return "bad activation";
    case GBA_ERR_ALIGN: return "misaligned pointer, or K or N not a multiple of 8 (K of 16 for 8-bit inputs)";
    case GBA_ERR_ALIAS: return "output overlaps an input";
    case GBA_ERR_DEVICE: return "no gfx950 device";
    case GBA_ERR_HIP: return "HIP runtime error";
    case GBA_ERR_SCHEDULE: return "unknown schedule";
    case GBA_ERR_CACHE: return "schedule cache not writable";
    case GBA_TUNE_INCOMPLETE: return "tuning stopped at its candidate budget; call again to resume";
    case GBA_ERR_SCRATCH: return "split-K partials larger than the static scratch of gemm_bias_act_noalloc";
    default: return "unknown status";
    }
}

int gba_last_hip_error(void) { return t_last_hip; }

int gba_set_stream(void *s) {
    t_stream = (hipStream_t)s;
    return GBA_OK;
}

int gba_set_schedule(const gba_schedule *s) {
    if (!s) {
        t_forced = false;
        return GBA_OK;
    }
    if (!sched_valid(*s)) return GBA_ERR_SCHEDULE;
    t_forced_sched = *s;
    t_forced = true;
    return GBA_OK;
}

int gba_num_schedules(void) { return kNumTable; }

int gba_list_schedule(int i, gba_schedule *out) {
    if (i < 0 || i >= kNumTable) return GBA_ERR_SCHEDULE;
    if (!out) return GBA_ERR_NULL;
    *out = kTable[i]->sched;
    return GBA_OK;
}

static int get_schedule(int64_t M, int64_t N, int64_t K, int act, int dtype, int lay,
                        gba_schedule *out) {
    if (!out) return GBA_ERR_NULL;
    int s = check_enums(act, dtype);
    if (s) return s;
    if (M < 0 || N < 0 || K < 0) return GBA_ERR_SHAPE;
    const DeviceInfo *d;
    s = current_device(&d);
    if (s) return s;
    const char *why;
    *out = choose(*d, M, N, K, act, dtype, lay, &why);
    return GBA_OK;
}

int gba_get_schedule(int64_t M, int64_t N, int64_t K, int act, int dtype, gba_schedule *out) {
    return get_schedule(M, N, K, act, dtype, 0, out);
}

int gba_get_schedule_nt(int64_t M, int64_t N, int64_t K, int act, int dtype, gba_schedule *out) {
    return get_schedule(M, N, K, act, dtype, LAY_TB, out);
}

int gba_get_schedule_ex(int64_t M, int64_t N, int64_t K, int act, int dtype, int flags,
                        gba_schedule *out) {
    if (flags & ~(GBA_TRANSPOSE_B | GBA_TRANSPOSE_A)) return GBA_ERR_SHAPE;
    return get_schedule(M, N, K, act, dtype, flags & (GBA_TRANSPOSE_B | GBA_TRANSPOSE_A), out);
}

int gba_split_plan(int64_t M, int64_t N, int64_t K, int act, int dtype, int flags,
                   gba_schedule *sched, int *splits) {
    if (!sched || !splits) return GBA_ERR_NULL;
    if (flags & ~(GBA_TRANSPOSE_B | GBA_TRANSPOSE_A)) return GBA_ERR_SHAPE;
    int s = check_enums(act, dtype);
    if (s) return s;
    if (M < 0 || N < 0 || K < 0) return GBA_ERR_SHAPE;
    const DeviceInfo *d;
    s = current_device(&d);
    if (s) return s;
    const char *why;
    int S = 1;
    gba_schedule sch;
    if (M > 0 && N > 0) S = split_plan(*d, M, N, K, act, dtype, flags, &sch, &why);
    if (S <= 1) {
        S = 1;
        sch = choose(*d, M, N, K, act, dtype, flags, &why);
    }
    *sched = sch;
    *splits = S;
    return GBA_OK;
}

int gemm_bias_act(const void *A, const void *B, const void *bias, void *C, int64_t M, int64_t N,
                  int64_t K, int act, int dtype) {
    return gemm_common(A, B, bias, C, M, N, K, act, dtype, 0);
}

int gemm(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int dtype) {
    return gemm_common(A, B, nullptr, C, M, N, K, GBA_ACT_NONE, dtype, 0);
}

int gemm_bias_act_nt(const void *A, const void *W, const void *bias, void *C, int64_t M,
                     int64_t N, int64_t K, int act, int dtype) {
    return gemm_common(A, W, bias, C, M, N, K, act, dtype, LAY_TB);
}

int gemm_nt(const void *A, const void *W, void *C, int64_t M, int64_t N, int64_t K, int dtype) {
    return gemm_common(A, W, nullptr, C, M, N, K, GBA_ACT_NONE, dtype, LAY_TB);
}

int gemm_bias_act_ex(const void *A, const void *B, const void *bias, void *C, int64_t M,
                     int64_t N, int64_t K, int act, int dtype, int flags, void *workspace,
                     size_t workspace_bytes) {
    if (flags & ~(GBA_TRANSPOSE_B | GBA_TRANSPOSE_A)) return GBA_ERR_SHAPE;
    return gemm_common(A, B, bias, C, M, N, K, act, dtype,
                       flags & (GBA_TRANSPOSE_B | GBA_TRANSPOSE_A), workspace,
                       workspace ? workspace_bytes : 0);
}

int gemm_bias_act_noalloc(const void *A, const void *B, const void *bias, void *C, int64_t M,
                          int64_t N, int64_t K, int act, int dtype, int flags) {
    if (flags & ~(GBA_TRANSPOSE_B | GBA_TRANSPOSE_A)) return GBA_ERR_SHAPE;
    const int lay = flags & (GBA_TRANSPOSE_B | GBA_TRANSPOSE_A);
    bool nothing = false;
    int s = check_gemm_args(A, B, bias, C, M, N, K, act, dtype, &nothing, lay);
    if (s || nothing) return s;
    const DeviceInfo *d;
    s = current_device(&d);
    if (s) return s;
    void *ws = nullptr;
    s = scratch_of_current_device(&ws);
    if (s) return s;
    // The split this call would make, and whether its partials fit the scratch.
    const char *why;
    gba_schedule sch;
    const int S = split_plan(*d, M, N, K, act, dtype, lay, &sch, &why);
    if (S > 1 && (size_t)S * (size_t)M * (size_t)N * 4u > kScratchBytes) return GBA_ERR_SCRATCH;
    return gemm_common(A, B, bias, C, M, N, K, act, dtype, lay, ws, kScratchBytes);
}

size_t gba_noalloc_scratch_bytes(void) { return kScratchBytes; }

int gba_workspace_size(int64_t M, int64_t N, int64_t K, int act, int dtype, int flags,
                       size_t *bytes) {
    if (!bytes) return GBA_ERR_NULL;
    *bytes = 0;
    if (flags & ~(GBA_TRANSPOSE_B | GBA_INPUT_FP8 | GBA_TRANSPOSE_A)) return GBA_ERR_SHAPE;
    int s = check_enums(act, dtype);
    if (s) return s;
    if (M < 0 || N < 0 || K < 0) return GBA_ERR_SHAPE;
    if (M == 0 || N == 0) return GBA_OK;
    const DeviceInfo *d;
    s = current_device(&d);
    if (s) return s;
    if (flags & GBA_INPUT_FP8) {
        const int S8 = split_count_fp8(M, N, K, d->cus);
        if (S8 > 1) *bytes = (size_t)S8 * (size_t)M * (size_t)N * 4u;
        return GBA_OK;
    }
    const int lay = flags & (GBA_TRANSPOSE_B | GBA_TRANSPOSE_A);
    const char *why;
    gba_schedule sch;
    const int S = split_plan(*d, M, N, K, act, dtype, lay, &sch, &why);
    if (S > 1) *bytes = (size_t)S * (size_t)M * (size_t)N * 4u;
    return GBA_OK;
}

int bias_act(const void *X, const void *bias, void *Y, int64_t M, int64_t N, int act,
             int dtype) {
    int s = check_enums(act, dtype);
    if (s) return s;
    if (M < 0 || N < 0 || M > 0x7fffffffLL || N > (1LL << 30)) return GBA_ERR_SHAPE;
    if (M == 0 || N == 0) return GBA_OK;
    if (!X || !Y) return GBA_ERR_NULL;
    if (N % 8) return GBA_ERR_ALIGN;
    if (!aligned16(X) || !aligned16(Y) || (bias && !aligned16(bias))) return GBA_ERR_ALIGN;
    const size_t nb = (size_t)M * N * 2;
    if (X != Y && overlaps(X, nb, Y, nb)) return GBA_ERR_ALIAS;
    if (overlaps(Y, nb, bias, (size_t)N * 2)) return GBA_ERR_ALIAS;
    const DeviceInfo *d;
    s = current_device(&d);
    if (s) return s;
    hipError_t e = kBiasAct[dtype][act](X, bias, Y, (int)M, (int)N, t_stream);
    return e == hipSuccess ? GBA_OK : hip_fail(e);
}


int gemm_bias_act_fp8_nt(const void *A, const void *W, const void *bias, void *C, int64_t M,
                         int64_t N, int64_t K, float scale, int act, int fmt, int dtype) {
    return fp8_common(A, W, bias, C, M, N, K, scale, act, fmt, dtype, nullptr, 0);
}

int gemm_bias_act_fp8_ex(const void *A, const void *W, const void *bias, void *C, int64_t M,
                         int64_t N, int64_t K, float scale, int act, int fmt, int dtype,
                         void *workspace, size_t workspace_bytes) {
    return fp8_common(A, W, bias, C, M, N, K, scale, act, fmt, dtype, workspace,
                      workspace ? workspace_bytes : 0);
}

int gba_epilogue_probe(const float *z, float *y, int64_t n, int act) {
    if (act < GBA_ACT_NONE || act > GBA_ACT_GELU_TANH) return GBA_ERR_ACT;
    if (n < 0) return GBA_ERR_SHAPE;
    if (n == 0) return GBA_OK;
    if (!z || !y) return GBA_ERR_NULL;
    const DeviceInfo *d;
    int s = current_device(&d);
    if (s) return s;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    switch (act) {
    case 0: hipLaunchKernelGGL(gba::epilogue_probe_kernel<0>, dim3(blocks), dim3(256), 0, t_stream, z, y, (long long)n); break;
    case 1: hipLaunchKernelGGL(gba::epilogue_probe_kernel<1>, dim3(blocks), dim3(256), 0, t_stream, z, y, (long long)n); break;
    case 2: hipLaunchKernelGGL(gba::epilogue_probe_kernel<2>, dim3(blocks), dim3(256), 0, t_stream, z, y, (long long)n); break;
    case 3: hipLaunchKernelGGL(gba::epilogue_probe_kernel<3>, dim3(blocks), dim3(256), 0, t_stream, z, y, (long long)n); break;
    case 4: hipLaunchKernelGGL(gba::epilogue_probe_kernel<4>, dim3(blocks), dim3(256), 0, t_stream, z, y, (long long)n); break;
    default: hipLaunchKernelGGL(gba::epilogue_probe_kernel<5>, dim3(blocks), dim3(256), 0, t_stream, z, y, (long long)n); break;
    }
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? GBA_OK : hip_fail(e);
}

namespace {
// Shader clock of the CU a workgroup runs on: s_memtime counts core clock
// cycles, s_memrealtime a constant-rate wall clock. One wave spins until
// `ticks` wall-clock ticks have passed (or a fixed iteration cap, so every wave
// ends) and writes both elapsed counts for the host to divide.
__global__ void __launch_bounds__(64) clock_probe_kernel(unsigned long long *out, unsigned long long ticks) {
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    unsigned long long r1 = r0;
    for (int it = 0; it < (1 << 20) && r1 - r0 < ticks; ++it) r1 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = c1 - c0;
        out[2 * blockIdx.x + 1] = r1 - r0;
    }
}
}  // namespace

int gba_clock_probe(uint64_t *out, int n_wg, int spin_us, int *wall_khz) {
    if (!out || !wall_khz) return GBA_ERR_NULL;
    if (n_wg < 1 || n_wg > 65536 || spin_us < 1 || spin_us > 100000) return GBA_ERR_SHAPE;
    const DeviceInfo *d;
    int s = current_device(&d);
    if (s) return s;
    int dev = 0, khz = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (e != hipSuccess) return hip_fail(e);
    if (khz <= 0) return GBA_ERR_DEVICE;
    *wall_khz = khz;
    const unsigned long long ticks = (unsigned long long)khz * (unsigned long long)spin_us / 1000ull;
    hipLaunchKernelGGL(clock_probe_kernel, dim3((unsigned)n_wg), dim3(64), 0, t_stream,
                       reinterpret_cast<unsigned long long *>(out), ticks);
    e = hipGetLastError();
    return e == hipSuccess ? GBA_OK : hip_fail(e);
}

int gba_autotune(const void *A, const void *B, const void *bias, void *C, int64_t M, int64_t N,
                 int64_t K, int act, int dtype, int flags, gba_schedule *best_out,
                 double *best_ms_out) {
    t_trials.clear();
    const int lay = ((flags & GBA_TUNE_TRANSPOSE_B) ? LAY_TB : 0) |
                    ((flags & GBA_TUNE_TRANSPOSE_A) ? LAY_TA : 0);
    bool nothing = false;
    int s = check_gemm_args(A, B, bias, C, M, N, K, act, dtype, &nothing, lay);
    if (s) return s;
    const DeviceInfo *d;
    s = current_device(&d);
    if (s) return s;
    if (nothing) {
        gba_schedule h = heuristic(M, N, d->cus, lay);
        if (best_out) *best_out = h;
        if (best_ms_out) *best_ms_out = 0.0;
        return GBA_OK;
    }
    std::vector<gba_schedule> cands;
    const int groups_all[] = {1, 2, 4, 8, 16};
    for (int i = 0; i < kNumTable; ++i) {
        gba_schedule c = kTable[i]->sched;
        if (lds_bytes(c) > kLdsBytes) continue;   // the pages' shared-memory filter
        if (!launcher(c, 0, 0, lay)) continue;   // no path for these layouts
        gba_schedule r0 = c;
        r0.raster = 0;
        cands.push_back(r0);
        if (flags & GBA_TUNE_ALL_GROUPS) {
            for (int g : groups_all) {
                gba_schedule r1 = c;
                r1.raster = 1;
                r1.group_m = g;
                cands.push_back(r1);
            }
        } else {
            cands.push_back(c);
        }
    }
    // Candidates timed by an earlier, interrupted or budget-limited run with the
    // same key are taken from the journal, not timed again.
    const std::string key = cache_key(*d, dtype, act, lay, M, N, K);
    std::vector<CacheRec> done = journal_get(key);
    long budget = -1;   // GBA_TUNE_BUDGET: at most this many candidates timed by this call
    if (const char *e = getenv("GBA_TUNE_BUDGET")) {
        if (*e) budget = strtol(e, nullptr, 10);
    }
    hipEvent_t ev[51];
    for (auto &e : ev) {
        hipError_t he = hipEventCreate(&e);
        if (he != hipSuccess) return hip_fail(he);
    }
    int status = GBA_OK, journal_status = GBA_OK;
    bool incomplete = false;
    long timed = 0;
    for (const gba_schedule &c : cands) {
        const CacheRec *prev = nullptr;
        for (const CacheRec &r : done)
            if (same_sched(r.s, c)) prev = &r;
        if (prev) {
            t_trials.push_back(Trial{c, prev->ms, 1});
            continue;
        }
        if (budget >= 0 && timed >= budget) {
            incomplete = true;
            continue;
        }
        for (int w = 0; w < 10 && status == GBA_OK; ++w)
            status = launch(c, A, B, bias, C, M, N, K, act, dtype, lay);
        for (int r = 0; r < 50 && status == GBA_OK; ++r) {
            hipEventRecord(ev[r], t_stream);
            status = launch(c, A, B, bias, C, M, N, K, act, dtype, lay);
        }
        if (status) break;
        hipEventRecord(ev[50], t_stream);
        hipError_t he = hipEventSynchronize(ev[50]);
        if (he != hipSuccess) {
            status = hip_fail(he);
            break;
        }
        std::vector<float> t(50);
        for (int r = 0; r < 50; ++r) hipEventElapsedTime(&t[r], ev[r], ev[r + 1]);
        std::nth_element(t.begin(), t.begin() + 25, t.end());
        const double med = t[25];
        if (log_enabled())
            fprintf(stderr, "[gba] tune k%d %dx%dx%d w%dx%d s%d r%d g%d: %.4f ms\n", c.kernel,
                    c.bm, c.bn, c.bk, c.wm, c.wn, c.stages, c.raster, c.group_m, med);
        t_trials.push_back(Trial{c, med, 0});
        done.push_back(CacheRec{c, med});
        ++timed;
        const int js = journal_set(key, done);   // progress survives an interruption
        if (js) journal_status = js;
    }
    for (auto &e : ev) hipEventDestroy(e);
    if (status) return status;
    if (t_trials.empty()) return GBA_TUNE_INCOMPLETE;   // a budget of 0 with nothing journaled
    const Trial *best = &t_trials[0];
    for (const Trial &t : t_trials)
        if (t.ms < best->ms) best = &t;
    // Leave the best result so far in C.
    status = launch(best->s, A, B, bias, C, M, N, K, act, dtype, lay);
    if (status) return status;
    hipError_t he = hipStreamSynchronize(t_stream);
    if (he != hipSuccess) return hip_fail(he);
    if (best_out) *best_out = best->s;
    if (best_ms_out) *best_ms_out = best->ms;
    if (incomplete) return journal_status ? journal_status : GBA_TUNE_INCOMPLETE;
    status = cache_put(key, CacheRec{best->s, best->ms});
    const int js = journal_set(key, {});
    if (status) return status;
    return js ? js : journal_status;
}

int gba_autotune_num_trials(void) { return (int)t_trials.size(); }

int gba_autotune_trial(int i, gba_schedule *sched, double *ms, int *resumed) {
    if (i < 0 || i >= (int)t_trials.size()) return GBA_ERR_SHAPE;
    if (sched) *sched = t_trials[i].s;
    if (ms) *ms = t_trials[i].ms;
    if (resumed) *resumed = t_trials[i].resumed;
    return GBA_OK;
}

const char *gba_build_id(void) { return GBA_BUILD_ID; }

static int cache_args(const char *arch, int cus, int64_t M, int64_t N, int64_t K, int act,
                      int dtype, int flags) {
    if (!arch) return GBA_ERR_NULL;
    if (strlen(arch) > 64 || strchr(arch, '"') || strchr(arch, '|') || strchr(arch, '\n'))
        return GBA_ERR_DEVICE;
    if (cus <= 0 || M < 0 || N < 0 || K < 0) return GBA_ERR_SHAPE;
    if (flags & ~(GBA_TRANSPOSE_B | GBA_TRANSPOSE_A)) return GBA_ERR_SHAPE;
    return check_enums(act, dtype);
}

int gba_cache_lookup(const char *arch, int cus, int64_t M, int64_t N, int64_t K, int act,
                     int dtype, int flags, gba_schedule *out, double *ms) {
    int s = cache_args(arch, cus, M, N, K, act, dtype, flags);
    if (s) return s;
    CacheRec r;
    if (!cache_get(cache_key(arch, cus, dtype, act, flags, M, N, K), &r)) return GBA_ERR_SCHEDULE;
    if (out) *out = r.s;
    if (ms) *ms = r.ms;
    return GBA_OK;
}

int gba_cache_store(const char *arch, int cus, int64_t M, int64_t N, int64_t K, int act,
                    int dtype, int flags, const gba_schedule *sched, double ms) {
    int s = cache_args(arch, cus, M, N, K, act, dtype, flags);
    if (s) return s;
    if (!sched) return GBA_ERR_NULL;
    if (!sched_valid(*sched)) return GBA_ERR_SCHEDULE;
    if (!(ms >= 0.0) || ms > 1e12) return GBA_ERR_SHAPE;
    return cache_put(cache_key(arch, cus, dtype, act, flags, M, N, K), CacheRec{*sched, ms});
}

}  // extern "C"
