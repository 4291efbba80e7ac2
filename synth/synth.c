/*
 * synth.c -- seeded synthetic inputs: R-MAT and web-like edge lists, and the
 * dense vectors of the benchmark workloads.
 *
 * Input generation only: nothing here builds a tree or computes a product.
 * Both the library's tests/benchmark and the oracle's tests feed on these
 * arrays.  Every random number is counter-based (the splitmix64 output
 * function applied to seed-derived counters), so results do not depend on
 * the thread count.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#include <omp.h>

static inline uint64_t mix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
/* counter-based stream: draw k of stream s under a seed */
static inline uint64_t draw(uint64_t seed, uint64_t s, uint64_t k) {
    return mix64(mix64(seed ^ (s * 0xD1B54A32D192ED03ull)) + k * 0x9E3779B97F4A7C15ull);
}
static inline double unit(uint64_t v) { return (double)(v >> 11) * (1.0 / 9007199254740992.0); }

/* ------------------------------------------------------------------ R-MAT */

static void rmat_edge(uint64_t seed, uint64_t k, int scale, double a, double ab, double abc,
                      uint32_t *r, uint32_t *c) {
    uint32_t rr = 0, cc = 0;
    for (int lv = 0; lv < scale; lv++) {
        double u = unit(draw(seed, 1, k * (uint64_t)scale + (uint64_t)lv));
        uint32_t b1, b0;
        if (u < a) { b1 = 0; b0 = 0; }
        else if (u < ab) { b1 = 0; b0 = 1; }
        else if (u < abc) { b1 = 1; b0 = 0; }
        else { b1 = 1; b0 = 1; }
        rr = (rr << 1) | b1;
        cc = (cc << 1) | b0;
    }
    *r = rr; *c = cc;
}

/* Open-addressing set of 64-bit keys (key+1 stored, 0 = empty). */
typedef struct { uint64_t *slot; uint64_t mask; uint64_t used; } kset;

static int kset_init(kset *s, uint64_t want) {
    uint64_t cap = 1024;
    while (cap < 2 * want + 16) cap <<= 1;
    s->slot = (uint64_t *)calloc(cap, sizeof(uint64_t));
    s->mask = cap - 1; s->used = 0;
    return s->slot ? 0 : -1;
}
static int kset_grow(kset *s) {
    uint64_t cap = (s->mask + 1) * 2;
    uint64_t *ns = (uint64_t *)calloc(cap, sizeof(uint64_t));
    if (!ns) return -1;
    for (uint64_t i = 0; i <= s->mask; i++) {
        uint64_t v = s->slot[i];
        if (!v) continue;
        uint64_t h = mix64(v) & (cap - 1);
        while (ns[h]) h = (h + 1) & (cap - 1);
        ns[h] = v;
    }
    free(s->slot); s->slot = ns; s->mask = cap - 1;
    return 0;
}
/* returns 1 if inserted (new), 0 if present */
static int kset_insert(kset *s, uint64_t key) {
    if (2 * (s->used + 1) > s->mask + 1) kset_grow(s);
    uint64_t v = key + 1, h = mix64(v) & s->mask;
    while (s->slot[h]) {
        if (s->slot[h] == v) return 0;
        h = (h + 1) & s->mask;
    }
    s->slot[h] = v; s->used++;
    return 1;
}

/*
 * R-MAT edges on 2^scale vertices, exactly n_edges distinct directed edges,
 * kept in generation order (first occurrence).  symmetric != 0: each drawn
 * pair (u, v), u != v, stands for the undirected edge and yields (u,v) and
 * (v,u); self-loops are skipped; n_edges must then be even.
 * Returns 0, or -1 on bad arguments / out of memory.
 */
int synth_rmat(int scale, uint64_t n_edges, double a, double b, double c, uint64_t seed,
               int symmetric, uint32_t *rows, uint32_t *cols, int threads) {
    if (scale < 1 || scale > 31) return -1;
    if (symmetric && (n_edges & 1)) return -1;
    uint64_t target = symmetric ? n_edges / 2 : n_edges;      /* distinct keys wanted */
    double maxpairs = symmetric ? ldexp(1.0, scale) * (ldexp(1.0, scale) - 1) / 2
                                : ldexp(1.0, 2 * scale);
    if ((double)target > 0.5 * maxpairs) return -1;
    if (threads < 1) threads = 1;
    if (threads > 255) threads = 255;
    int P = threads;
    kset *sets = (kset *)calloc((size_t)P, sizeof(kset));
    for (int p = 0; p < P; p++)
        if (kset_init(&sets[p], target / (uint64_t)P + 1)) return -1;

    uint64_t found = 0, next_k = 0;
    uint64_t block = target + target / 4 + 1024;
    uint64_t *cand = NULL;
    uint8_t *fresh = NULL, *owner = NULL;
    while (found < target) {
        uint64_t nb = block;
        cand = (uint64_t *)realloc(cand, nb * sizeof(uint64_t));
        fresh = (uint8_t *)realloc(fresh, nb);
        owner = (uint8_t *)realloc(owner, nb);
        if (!cand || !fresh || !owner) return -1;
        #pragma omp parallel for num_threads(threads) schedule(static)
        for (int64_t i = 0; i < (int64_t)nb; i++) {
            uint32_t r, cc;
            rmat_edge(seed, next_k + (uint64_t)i, scale, a, a + b, a + b + c, &r, &cc);
            if (symmetric) {
                if (r == cc) { cand[i] = UINT64_MAX; continue; }
                uint32_t lo = r < cc ? r : cc, hi = r < cc ? cc : r;
                /* keep the drawn orientation in the low bit of a wider key */
                cand[i] = ((uint64_t)lo << 32 | hi) ;
                fresh[i] = (uint8_t)(r < cc);      /* 1: drawn as (lo,hi) */
            } else {
                cand[i] = (uint64_t)r << 32 | cc;
            }
            owner[i] = (uint8_t)(mix64(cand[i] ^ 0x5bd1e995ull) % (uint64_t)P);
        }
        /* each thread owns the keys that hash to it; marks first sightings */
        #pragma omp parallel num_threads(P)
        {
            int p = omp_get_thread_num();
            for (uint64_t i = 0; i < nb; i++) {
                uint64_t key = cand[i];
                if (key == UINT64_MAX || owner[i] != p) continue;
                int isnew = kset_insert(&sets[p], key);
                if (symmetric) fresh[i] = (uint8_t)(isnew ? (2 | fresh[i]) : 0);
                else fresh[i] = (uint8_t)isnew;
            }
        }
        for (uint64_t i = 0; i < nb && found < target; i++) {
            uint64_t key = cand[i];
            if (key == UINT64_MAX || !fresh[i]) continue;
            uint32_t hi32 = (uint32_t)(key >> 32), lo32 = (uint32_t)key;
            if (symmetric) {
                uint32_t u = (fresh[i] & 1) ? hi32 : lo32, v = (fresh[i] & 1) ? lo32 : hi32;
                rows[2 * found] = u; cols[2 * found] = v;
                rows[2 * found + 1] = v; cols[2 * found + 1] = u;
            } else {
                rows[found] = hi32; cols[found] = lo32;
            }
            found++;
        }
        next_k += nb;
        block = (target - found) * 2 + 1024;
    }
    for (int p = 0; p < P; p++) free(sets[p].slot);
    free(sets); free(cand); free(fresh); free(owner);
    return 0;
}

/* --------------------------------------------------------------- web-like */

/* E[min(cap, floor(X))] for X Pareto with scale xm and tail index alpha. */
static double capped_floor_mean(double xm, double alpha, uint32_t cap) {
    double s = 0;
    for (uint32_t k = 1; k <= cap; k++) {
        double p = (k <= xm) ? 1.0 : pow(xm / (double)k, alpha);
        s += p;
    }
    return s;
}

double synth_pareto_scale(double mean, double alpha, uint32_t cap) {
    double lo = 1e-9, hi = (double)cap;
    for (int it = 0; it < 200; it++) {
        double mid = 0.5 * (lo + hi);
        if (capped_floor_mean(mid, alpha, cap) < mean) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
}

static uint32_t web_degree(uint64_t seed, uint64_t i, double xm, double alpha, uint32_t cap) {
    double u = 1.0 - unit(draw(seed, 2, i));            /* (0, 1] */
    double x = xm * pow(u, -1.0 / alpha);
    if (x >= (double)cap) return cap;
    return (uint32_t)floor(x);
}

/* Out-degrees of all n sources; returns their sum. */
uint64_t synth_web_degrees(uint64_t n, double mean, double alpha, uint32_t cap, uint64_t seed,
                           uint32_t *deg, int threads) {
    double xm = synth_pareto_scale(mean, alpha, cap);
    uint64_t total = 0;
    #pragma omp parallel for num_threads(threads) reduction(+:total) schedule(static)
    for (int64_t i = 0; i < (int64_t)n; i++) {
        deg[i] = web_degree(seed, (uint64_t)i, xm, alpha, cap);
        total += deg[i];
    }
    return total;
}

/*
 * Web-like edges: source i has deg[i] edges (from synth_web_degrees); each
 * target is, with probability p_local, i + U{-window..window} (mod n), else
 * uniform on [0, n).  rows/cols hold sum(deg) entries, sources ascending.
 * Duplicates are left in (a Boolean matrix drops them on construction).
 */
int synth_web_edges(uint64_t n, const uint32_t *deg, double p_local, uint32_t window,
                    uint64_t seed, uint32_t *rows, uint32_t *cols, int threads) {
    uint64_t *start = (uint64_t *)malloc((size_t)(n + 1) * sizeof(uint64_t));
    if (!start) return -1;
    start[0] = 0;
    for (uint64_t i = 0; i < n; i++) start[i + 1] = start[i] + deg[i];
    uint64_t span = 2ull * window + 1;
    #pragma omp parallel for num_threads(threads) schedule(dynamic, 4096)
    for (int64_t ii = 0; ii < (int64_t)n; ii++) {
        uint64_t i = (uint64_t)ii;
        for (uint64_t e = start[i]; e < start[i + 1]; e++) {
            uint64_t v1 = draw(seed, 3, e), v2 = draw(seed, 4, e);
            uint64_t t;
            if (unit(v1) < p_local) {
                int64_t delta = (int64_t)(v2 % span) - (int64_t)window;
                int64_t tt = ((int64_t)i + delta) % (int64_t)n;
                if (tt < 0) tt += (int64_t)n;
                t = (uint64_t)tt;
            } else {
                t = v2 % n;
            }
            rows[e] = (uint32_t)i;
            cols[e] = (uint32_t)t;
        }
    }
    free(start);
    return 0;
}

/* ---------------------------------------------------------------- vectors */

/* fp32 k * 2^-24, k uniform on [0, 2^24): uniform on [0, 1), exact in fp32 */
void synth_uniform01(uint64_t count, uint64_t seed, float *out, int threads) {
    #pragma omp parallel for num_threads(threads) schedule(static)
    for (int64_t i = 0; i < (int64_t)count; i++)
        out[i] = (float)(draw(seed, 5, (uint64_t)i) >> 40) * (1.0f / 16777216.0f);
}

/* with probability p_finite uniform on [0, hi), else +inf */
void synth_tropical(uint64_t count, double p_finite, double hi, uint64_t seed, float *out,
                    int threads) {
    #pragma omp parallel for num_threads(threads) schedule(static)
    for (int64_t i = 0; i < (int64_t)count; i++) {
        if (unit(draw(seed, 6, (uint64_t)i)) < p_finite)
            out[i] = (float)(unit(draw(seed, 7, (uint64_t)i)) * hi);
        else
            out[i] = INFINITY;
    }
}

/* 32 independent bits per word, each set with probability p */
void synth_bitmask(uint64_t count, double p, uint64_t seed, uint32_t *out, int threads) {
    #pragma omp parallel for num_threads(threads) schedule(static)
    for (int64_t i = 0; i < (int64_t)count; i++) {
        uint32_t w = 0;
        for (int b = 0; b < 32; b++)
            if (unit(draw(seed, 8, (uint64_t)i * 32 + (uint64_t)b)) < p) w |= 1u << b;
        out[i] = w;
    }
}
