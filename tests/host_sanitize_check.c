/* Host-side check program for the AddressSanitizer / UndefinedBehaviorSanitizer build
 * of the library's host code (tests/test_host_sanitizers_cpu.py builds and runs
 * it). It exercises every path that needs no GPU:
 *   - version, build id and status strings;
 *   - the compiled-in schedule table and gba_set_schedule's validation;
 *   - argument errors of every compute entry point, each returned before any
 *     device work (NULL pointers, bad enums, bad shapes, misaligned or
 *     overlapping pointers, unknown flags; M == 0 is "nothing to do");
 *   - the on-disk schedule cache: round trips, bad arguments, missing,
 *     corrupt, truncated and oversized files, an unwritable directory,
 *     GBA_DISABLE_CACHE, and writers in several threads.
 * No call here should reach a launch: pointers are NULL or fail a host-side
 * check. As a second guard the program runs only where no GPU is visible (exit
 * 77 otherwise), since a check that wrongly passed would launch on dummy
 * pointers. Prints "host sanitize check ok" and exits 0 when every check holds. */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <sys/stat.h>

#include "gba.h"

/* HIP runtime (C linkage; 0 is hipSuccess). */
extern int hipGetDeviceCount(int *count);

static int g_fail = 0;
#define CHECK(cond)                                                             \
    do {                                                                        \
        if (!(cond)) {                                                          \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            g_fail = 1;                                                         \
        }                                                                       \
    } while (0)

static const char *ARCH = "gfx950:sramecc+:xnack-";
static char g_base[4096];

/* Points GBA_CACHE_DIR at a fresh directory under the base (the library re-reads
 * the cache whenever the variable changes). */
static void use_dir(const char *name, char *out, size_t n) {
    snprintf(out, n, "%s/%s", g_base, name);
    mkdir(out, 0700);
    setenv("GBA_CACHE_DIR", out, 1);
}

static void write_file(const char *dir, const char *name, const char *data, size_t len) {
    char p[4200];
    snprintf(p, sizeof p, "%s/%s", dir, name);
    FILE *f = fopen(p, "wb");
    if (!f) {
        fprintf(stderr, "cannot write %s\n", p);
        g_fail = 1;
        return;
    }
    fwrite(data, 1, len, f);
    fclose(f);
}

static int same_sched(const gba_schedule *a, const gba_schedule *b) {
    return a->bm == b->bm && a->bn == b->bn && a->bk == b->bk && a->wm == b->wm && a->wn == b->wn &&
           a->stages == b->stages && a->kernel == b->kernel && a->loaders == b->loaders &&
           a->spread == b->spread && a->raster == b->raster && a->group_m == b->group_m;
}

static void strings_and_table(void) {
    CHECK(gba_version() && strlen(gba_version()) > 0);
    CHECK(gba_build_id() && strlen(gba_build_id()) > 0);
    for (int s = -5; s < 40; ++s) CHECK(gba_status_string(s) != NULL);
    const int n = gba_num_schedules();
    CHECK(n >= 2);
    gba_schedule s;
    CHECK(gba_list_schedule(-1, &s) != GBA_OK);
    CHECK(gba_list_schedule(n, &s) != GBA_OK);
    CHECK(gba_list_schedule(0, NULL) == GBA_ERR_NULL);
    for (int i = 0; i < n; ++i) {
        CHECK(gba_list_schedule(i, &s) == GBA_OK);
        CHECK(gba_set_schedule(&s) == GBA_OK);
        gba_schedule bad = s;
        bad.bm = 7;
        CHECK(gba_set_schedule(&bad) == GBA_ERR_SCHEDULE);
        bad = s;
        bad.raster = 9;
        CHECK(gba_set_schedule(&bad) == GBA_ERR_SCHEDULE);
        bad = s;
        bad.group_m = -3;
        CHECK(gba_set_schedule(&bad) == GBA_ERR_SCHEDULE);
    }
    CHECK(gba_set_schedule(NULL) == GBA_OK);
    CHECK(gba_set_stream(NULL) == GBA_OK);
    CHECK(gba_autotune_num_trials() == 0);
    CHECK(gba_autotune_trial(0, NULL, NULL, NULL) == GBA_ERR_SHAPE);
    CHECK(gba_autotune_trial(-1, NULL, NULL, NULL) == GBA_ERR_SHAPE);
    CHECK(gba_noalloc_scratch_bytes() > 0);
}

static void argument_errors(void) {
    /* Pointers that only serve host-side checks: never dereferenced, and every
     * call below fails (or has nothing to do) before any device work. */
    char *const p = (char *)(uintptr_t)0x100000;   /* 16-byte aligned */
    char *const odd = p + 2;                        /* misaligned */
    const int64_t M = 64, N = 64, K = 64;
    CHECK(gemm_bias_act(NULL, p, NULL, p + 65536, M, N, K, GBA_ACT_GELU, GBA_DTYPE_F16) == GBA_ERR_NULL);
    CHECK(gemm_bias_act(p, NULL, NULL, p + 65536, M, N, K, GBA_ACT_GELU, GBA_DTYPE_F16) == GBA_ERR_NULL);
    CHECK(gemm_bias_act(p, p + 16384, NULL, NULL, M, N, K, GBA_ACT_GELU, GBA_DTYPE_F16) == GBA_ERR_NULL);
    CHECK(gemm_bias_act(p, p + 16384, NULL, p + 65536, M, N, K, 99, GBA_DTYPE_F16) == GBA_ERR_ACT);
    CHECK(gemm_bias_act(p, p + 16384, NULL, p + 65536, M, N, K, -1, GBA_DTYPE_F16) == GBA_ERR_ACT);
    CHECK(gemm_bias_act(p, p + 16384, NULL, p + 65536, M, N, K, GBA_ACT_GELU, 7) == GBA_ERR_DTYPE);
    CHECK(gemm_bias_act(p, p + 16384, NULL, p + 65536, -1, N, K, GBA_ACT_GELU, GBA_DTYPE_F16) == GBA_ERR_SHAPE);
    CHECK(gemm_bias_act(p, p + 16384, NULL, p + 65536, M, -8, K, GBA_ACT_GELU, GBA_DTYPE_F16) == GBA_ERR_SHAPE);
    CHECK(gemm_bias_act(p, p + 16384, NULL, p + 65536, M, N, (int64_t)1 << 40, GBA_ACT_GELU, GBA_DTYPE_F16) ==
          GBA_ERR_SHAPE);
    CHECK(gemm_bias_act(odd, p + 16384, NULL, p + 65536, M, N, K, GBA_ACT_GELU, GBA_DTYPE_F16) == GBA_ERR_ALIGN);
    CHECK(gemm_bias_act(p, p + 16384, NULL, p + 65536, M, N, 60, GBA_ACT_GELU, GBA_DTYPE_F16) == GBA_ERR_ALIGN);
    CHECK(gemm_bias_act(p, p + 16384, NULL, p + 65536, M, 60, K, GBA_ACT_GELU, GBA_DTYPE_F16) == GBA_ERR_ALIGN);
    /* C overlapping A */
    CHECK(gemm_bias_act(p, p + 65536, NULL, p + 16, M, N, K, GBA_ACT_GELU, GBA_DTYPE_F16) == GBA_ERR_ALIAS);
    /* nothing to do */
    CHECK(gemm_bias_act(p, p + 16384, NULL, p + 65536, 0, N, K, GBA_ACT_GELU, GBA_DTYPE_F16) == GBA_OK);
    CHECK(gemm_bias_act(p, p + 16384, NULL, p + 65536, M, 0, K, GBA_ACT_GELU, GBA_DTYPE_F16) == GBA_OK);
    CHECK(gemm(NULL, p, p + 65536, M, N, K, GBA_DTYPE_BF16) == GBA_ERR_NULL);
    CHECK(gemm_nt(p, NULL, p + 65536, M, N, K, GBA_DTYPE_BF16) == GBA_ERR_NULL);
    CHECK(gemm_bias_act_nt(p, p + 16384, NULL, p + 65536, M, N, K, 42, GBA_DTYPE_F16) == GBA_ERR_ACT);
    CHECK(bias_act(NULL, NULL, p, M, N, GBA_ACT_RELU, GBA_DTYPE_F16) == GBA_ERR_NULL);
    CHECK(bias_act(p, NULL, p + 65536, M, 12, GBA_ACT_RELU, GBA_DTYPE_F16) == GBA_ERR_ALIGN);
    CHECK(bias_act(p, NULL, p, 0, N, GBA_ACT_RELU, GBA_DTYPE_F16) == GBA_OK);
    CHECK(gemm_bias_act_ex(p, p + 16384, NULL, p + 65536, M, N, K, GBA_ACT_NONE, GBA_DTYPE_F16, 1 << 20, NULL,
                           0) == GBA_ERR_SHAPE);
    CHECK(gemm_bias_act_ex(NULL, p + 16384, NULL, p + 65536, M, N, K, GBA_ACT_NONE, GBA_DTYPE_F16, 0, NULL, 0) ==
          GBA_ERR_NULL);
    CHECK(gemm_bias_act_noalloc(NULL, p, NULL, p + 65536, M, N, K, GBA_ACT_NONE, GBA_DTYPE_F16, 0) ==
          GBA_ERR_NULL);
    CHECK(gemm_bias_act_noalloc(p, p + 16384, NULL, p + 65536, M, N, K, GBA_ACT_NONE, GBA_DTYPE_F16, 64) ==
          GBA_ERR_SHAPE);
    CHECK(gemm_bias_act_fp8_nt(NULL, p, NULL, p + 65536, M, N, K, 1.0f, GBA_ACT_NONE, 0, GBA_DTYPE_F16) ==
          GBA_ERR_NULL);
    CHECK(gemm_bias_act_fp8_ex(p, p + 16384, NULL, p + 65536, M, N, K, 1.0f, GBA_ACT_NONE, 9, GBA_DTYPE_F16,
                               NULL, 0) != GBA_OK);
    CHECK(gemm_bias_act_fp8_ex(p, p + 16384, NULL, p + 65536, M, N, K, NAN, GBA_ACT_NONE, 0, GBA_DTYPE_F16,
                               NULL, 0) != GBA_OK);
    size_t nb = 1;
    CHECK(gba_workspace_size(M, N, K, GBA_ACT_NONE, GBA_DTYPE_F16, 0, NULL) == GBA_ERR_NULL);
    CHECK(gba_workspace_size(-1, N, K, GBA_ACT_NONE, GBA_DTYPE_F16, 0, &nb) == GBA_ERR_SHAPE && nb == 0);
    CHECK(gba_workspace_size(M, N, K, GBA_ACT_NONE, GBA_DTYPE_F16, 1 << 20, &nb) == GBA_ERR_SHAPE);
    CHECK(gba_workspace_size(0, N, K, GBA_ACT_NONE, GBA_DTYPE_F16, 0, &nb) == GBA_OK && nb == 0);
    gba_schedule s;
    int splits = 0;
    CHECK(gba_split_plan(M, N, K, GBA_ACT_NONE, GBA_DTYPE_F16, 0, NULL, &splits) == GBA_ERR_NULL);
    CHECK(gba_split_plan(M, N, K, GBA_ACT_NONE, GBA_DTYPE_F16, 1 << 20, &s, &splits) == GBA_ERR_SHAPE);
    CHECK(gba_get_schedule(M, N, K, 77, GBA_DTYPE_F16, &s) == GBA_ERR_ACT);
    CHECK(gba_get_schedule_ex(M, N, K, GBA_ACT_NONE, GBA_DTYPE_F16, 1 << 20, &s) == GBA_ERR_SHAPE);
    CHECK(gba_epilogue_probe(NULL, NULL, 16, GBA_ACT_GELU) == GBA_ERR_NULL);
    int khz = 0;
    CHECK(gba_clock_probe(NULL, 1, 10, &khz) == GBA_ERR_NULL);
    CHECK(gba_autotune(NULL, p, NULL, p + 65536, M, N, K, GBA_ACT_NONE, GBA_DTYPE_F16, 0, NULL, NULL) ==
          GBA_ERR_NULL);
}

static void cache_round_trips(void) {
    char dir[4200];
    use_dir("c1", dir, sizeof dir);
    unsetenv("GBA_DISABLE_CACHE");
    const int n = gba_num_schedules();
    gba_schedule s, got;
    double ms = -1;
    CHECK(gba_cache_lookup(ARCH, 256, 4096, 4096, 4096, GBA_ACT_GELU, GBA_DTYPE_F16, 0, &got, &ms) ==
          GBA_ERR_SCHEDULE);
    for (int i = 0; i < n; ++i) {
        CHECK(gba_list_schedule(i, &s) == GBA_OK);
        const int64_t M = 64 * (i + 1), N = 128, K = 256 * (i + 2);
        const int act = i % 6, dt = i % 2, fl = (i % 3 == 1) ? 1 : 0;
        CHECK(gba_cache_store(ARCH, 256, M, N, K, act, dt, fl, &s, 0.001 * (i + 1)) == GBA_OK);
    }
    for (int i = 0; i < n; ++i) {
        CHECK(gba_list_schedule(i, &s) == GBA_OK);
        const int64_t M = 64 * (i + 1), N = 128, K = 256 * (i + 2);
        const int act = i % 6, dt = i % 2, fl = (i % 3 == 1) ? 1 : 0;
        CHECK(gba_cache_lookup(ARCH, 256, M, N, K, act, dt, fl, &got, &ms) == GBA_OK);
        CHECK(same_sched(&s, &got) && fabs(ms - 0.001 * (i + 1)) < 1e-12);
        /* another CU count, arch or layout is another key */
        CHECK(gba_cache_lookup(ARCH, 255, M, N, K, act, dt, fl, &got, NULL) == GBA_ERR_SCHEDULE);
        CHECK(gba_cache_lookup("gfx950:other", 256, M, N, K, act, dt, fl, NULL, NULL) == GBA_ERR_SCHEDULE);
        CHECK(gba_cache_lookup(ARCH, 256, M, N, K, act, dt, fl ^ 4, NULL, NULL) == GBA_ERR_SCHEDULE);
    }
    /* bad arguments */
    CHECK(gba_list_schedule(0, &s) == GBA_OK);
    CHECK(gba_cache_store(NULL, 256, 1, 8, 8, 0, 0, 0, &s, 1.0) == GBA_ERR_NULL);
    CHECK(gba_cache_store(ARCH, 256, 1, 8, 8, 0, 0, 0, NULL, 1.0) == GBA_ERR_NULL);
    CHECK(gba_cache_lookup(NULL, 256, 1, 8, 8, 0, 0, 0, NULL, NULL) == GBA_ERR_NULL);
    CHECK(gba_cache_store("gfx950\"x", 256, 1, 8, 8, 0, 0, 0, &s, 1.0) == GBA_ERR_DEVICE);
    CHECK(gba_cache_store("gfx950|x", 256, 1, 8, 8, 0, 0, 0, &s, 1.0) == GBA_ERR_DEVICE);
    CHECK(gba_cache_lookup("gfx950\nx", 256, 1, 8, 8, 0, 0, 0, NULL, NULL) == GBA_ERR_DEVICE);
    char longarch[200];
    memset(longarch, 'g', sizeof longarch - 1);
    longarch[sizeof longarch - 1] = 0;
    CHECK(gba_cache_store(longarch, 256, 1, 8, 8, 0, 0, 0, &s, 1.0) == GBA_ERR_DEVICE);
    CHECK(gba_cache_lookup(longarch, 256, 1, 8, 8, 0, 0, 0, NULL, NULL) == GBA_ERR_DEVICE);
    CHECK(gba_cache_store(ARCH, 0, 1, 8, 8, 0, 0, 0, &s, 1.0) == GBA_ERR_SHAPE);
    CHECK(gba_cache_store(ARCH, 256, -1, 8, 8, 0, 0, 0, &s, 1.0) == GBA_ERR_SHAPE);
    CHECK(gba_cache_store(ARCH, 256, 1, 8, 8, 0, 0, 1 << 12, &s, 1.0) == GBA_ERR_SHAPE);
    CHECK(gba_cache_store(ARCH, 256, 1, 8, 8, 0, 0, 0, &s, -1.0) == GBA_ERR_SHAPE);
    CHECK(gba_cache_store(ARCH, 256, 1, 8, 8, 0, 0, 0, &s, NAN) == GBA_ERR_SHAPE);
    CHECK(gba_cache_store(ARCH, 256, 1, 8, 8, 0, 0, 0, &s, INFINITY) == GBA_ERR_SHAPE);
    CHECK(gba_cache_store(ARCH, 256, 1, 8, 8, 9, 0, 0, &s, 1.0) == GBA_ERR_ACT);
    CHECK(gba_cache_store(ARCH, 256, 1, 8, 8, 0, 5, 0, &s, 1.0) == GBA_ERR_DTYPE);
    gba_schedule bad = s;
    bad.bk = 3;
    CHECK(gba_cache_store(ARCH, 256, 1, 8, 8, 0, 0, 0, &bad, 1.0) == GBA_ERR_SCHEDULE);
}

static void corrupt_caches(void) {
    static const char *bodies[] = {
        "",
        "not json at all\n",
        "{\"format\": \"gba-schedule-cache\", \"version\": 1, \"entries\": [\n{\"key\": \"",
        "{\"format\": \"gba-schedule-cache\", \"version\": 1, \"entries\": [\n"
        "{\"key\": \"x\", \"bm\": \"oops\"},\n{\"key\": 5},\n]}\n",
        "{\"format\": \"gba-schedule-cache\", \"version\": 99, \"entries\": []}\n",
        "\x01\x02\x03\xff\xfe\x00\x00\x7f binary",
    };
    gba_schedule s, got;
    CHECK(gba_list_schedule(0, &s) == GBA_OK);
    char dir[4200];
    for (size_t b = 0; b < sizeof bodies / sizeof bodies[0] + 1; ++b) {
        char name[32];
        snprintf(name, sizeof name, "bad%zu", b);
        use_dir(name, dir, sizeof dir);
        if (b < sizeof bodies / sizeof bodies[0]) {
            write_file(dir, "schedules.json", bodies[b], b == 5 ? 16 : strlen(bodies[b]));
            write_file(dir, "tuning.json", bodies[b], b == 5 ? 16 : strlen(bodies[b]));
        } else {
            /* one 4 MiB line with no newline */
            size_t len = 4u << 20;
            char *big = malloc(len);
            memset(big, '{', len);
            write_file(dir, "schedules.json", big, len);
            free(big);
        }
        CHECK(gba_cache_lookup(ARCH, 256, 128, 128, 128, 0, 0, 0, &got, NULL) == GBA_ERR_SCHEDULE);
        /* a store replaces what it cannot read, and is read back */
        CHECK(gba_cache_store(ARCH, 256, 128, 128, 128, 0, 0, 0, &s, 0.5) == GBA_OK);
        CHECK(gba_cache_lookup(ARCH, 256, 128, 128, 128, 0, 0, 0, &got, NULL) == GBA_OK && same_sched(&s, &got));
    }
    /* unwritable: the cache directory's parent is a regular file */
    use_dir("plainfile", dir, sizeof dir);
    write_file(dir, "f", "x", 1);
    char sub[4300];
    snprintf(sub, sizeof sub, "%s/f/cache", dir);
    setenv("GBA_CACHE_DIR", sub, 1);
    CHECK(gba_cache_store(ARCH, 256, 128, 128, 128, 0, 0, 0, &s, 0.5) == GBA_ERR_CACHE);
    CHECK(gba_cache_lookup(ARCH, 256, 128, 128, 128, 0, 0, 0, &got, NULL) == GBA_ERR_SCHEDULE);
    /* disabled */
    use_dir("disabled", dir, sizeof dir);
    setenv("GBA_DISABLE_CACHE", "1", 1);
    CHECK(gba_cache_store(ARCH, 256, 128, 128, 128, 0, 0, 0, &s, 0.5) == GBA_OK);
    CHECK(gba_cache_lookup(ARCH, 256, 128, 128, 128, 0, 0, 0, &got, NULL) == GBA_ERR_SCHEDULE);
    unsetenv("GBA_DISABLE_CACHE");
}

/* Writers in several threads into one cache. */
enum { NTHREADS = 8, PER_THREAD = 24 };
static void *writer(void *arg) {
    const int t = (int)(intptr_t)arg;
    gba_schedule s;
    const int n = gba_num_schedules();
    for (int i = 0; i < PER_THREAD; ++i) {
        if (gba_list_schedule((t + i) % n, &s) != GBA_OK ||
            gba_cache_store(ARCH, 256, 8 * (t * PER_THREAD + i + 1), 64, 64, 0, 0, 0, &s, 1.0 + i) != GBA_OK)
            g_fail = 1;
        gba_schedule got;
        if (gba_cache_lookup(ARCH, 256, 8 * (t * PER_THREAD + i + 1), 64, 64, 0, 0, 0, &got, NULL) != GBA_OK)
            g_fail = 1;
    }
    return NULL;
}

static void threaded_writers(void) {
    char dir[4200];
    use_dir("threads", dir, sizeof dir);
    pthread_t th[NTHREADS];
    for (int t = 0; t < NTHREADS; ++t) pthread_create(&th[t], NULL, writer, (void *)(intptr_t)t);
    for (int t = 0; t < NTHREADS; ++t) pthread_join(th[t], NULL);
    gba_schedule got;
    for (int t = 0; t < NTHREADS; ++t)
        for (int i = 0; i < PER_THREAD; ++i)
            CHECK(gba_cache_lookup(ARCH, 256, 8 * (t * PER_THREAD + i + 1), 64, 64, 0, 0, 0, &got, NULL) ==
                  GBA_OK);
}

int main(int argc, char **argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s <scratch directory>\n", argv[0]);
        return 2;
    }
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) == 0 && ndev > 0) {
        printf("a GPU is visible: this check runs only without one\n");
        return 77;
    }
    snprintf(g_base, sizeof g_base, "%s", argv[1]);
    strings_and_table();
    argument_errors();
    cache_round_trips();
    corrupt_caches();
    threaded_writers();
    if (g_fail) {
        fprintf(stderr, "host sanitize check: FAILED\n");
        return 1;
    }
    printf("host sanitize check ok\n");
    return 0;
}
