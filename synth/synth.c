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

static inline uint64_t stream_key(uint64_t seed, uint64_t s) {
    return mix64(seed ^ (s * 0xD1B54A32D192ED03ull));
}
/* draw k of a stream whose key is sk (same values as draw(seed, s, k)) */
static inline uint64_t draw_k(uint64_t sk, uint64_t k) { return mix64(sk + k * 0x9E3779B97F4A7C15ull); }

static void rmat_edge(uint64_t sk, uint64_t k, int scale, double a, double ab, double abc,
                      uint32_t *r, uint32_t *c) {
    uint32_t rr = 0, cc = 0;
    for (int lv = 0; lv < scale; lv++) {
        double u = unit(draw_k(sk, k * (uint64_t)scale + (uint64_t)lv));
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

/* Stable LSD radix sort of (key, idx) pairs on the low 'bits' bits of key. */
static int sort_pairs(uint64_t *key, uint32_t *idx, uint64_t n, int bits, int threads) {
    uint64_t *k2 = (uint64_t *)malloc((n ? n : 1) * sizeof(uint64_t));
    uint32_t *i2 = (uint32_t *)malloc((n ? n : 1) * sizeof(uint32_t));
    uint64_t *hist = (uint64_t *)calloc((size_t)threads * 256, sizeof(uint64_t));
    if (!k2 || !i2 || !hist) { free(k2); free(i2); free(hist); return -1; }
    uint64_t *ka = key, *kb = k2;
    uint32_t *ia = idx, *ib = i2;
    for (int sh = 0; sh < bits; sh += 8) {
        memset(hist, 0, (size_t)threads * 256 * sizeof(uint64_t));
        #pragma omp parallel num_threads(threads)
        {
            int t = omp_get_thread_num();
            uint64_t lo = n * (uint64_t)t / (uint64_t)threads, hi = n * (uint64_t)(t + 1) / (uint64_t)threads;
            uint64_t *h = hist + (size_t)t * 256;
            for (uint64_t i = lo; i < hi; i++) h[(ka[i] >> sh) & 255]++;
            #pragma omp barrier
            #pragma omp single
            {
                uint64_t run = 0;
                for (int d = 0; d < 256; d++)
                    for (int q = 0; q < threads; q++) {
                        uint64_t c = hist[(size_t)q * 256 + d];
                        hist[(size_t)q * 256 + d] = run;
                        run += c;
                    }
            }
            for (uint64_t i = lo; i < hi; i++) {
                uint64_t o = h[(ka[i] >> sh) & 255]++;
                kb[o] = ka[i];
                ib[o] = ia[i];
            }
        }
        uint64_t *tk = ka; ka = kb; kb = tk;
        uint32_t *ti = ia; ia = ib; ib = ti;
    }
    if (ka != key) {
        memcpy(key, ka, n * sizeof(uint64_t));
        memcpy(idx, ia, n * sizeof(uint32_t));
    }
    free(hist);
    free(k2);
    free(i2);
    return 0;
}

/*
 * R-MAT edges on 2^scale vertices, exactly n_edges distinct directed edges,
 * kept in generation order (first occurrence).  symmetric != 0: each drawn
 * pair (u, v), u != v, stands for the undirected edge and yields (u,v) and
 * (v,u); self-loops are skipped; n_edges must then be even.
 * Candidates are drawn in one batch (25% spare); duplicates are found by a
 * stable sort of the candidates' keys, which keeps each key's first draw; a
 * batch that falls short is redrawn twice as long (same prefix of draws).
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
    const uint64_t sk = stream_key(seed, 1);
    const uint64_t invalid = 1ull << (2 * scale);
    uint64_t nb = target + target / 4 + 1024;
    for (;;) {
        if (nb >= (1ull << 32)) return -1;
        uint64_t *key = (uint64_t *)malloc(nb * sizeof(uint64_t));
        uint32_t *idx = (uint32_t *)malloc(nb * sizeof(uint32_t));
        uint8_t *fresh = (uint8_t *)calloc(nb, 1);
        uint8_t *orient = (uint8_t *)malloc(nb);
        if (!key || !idx || !fresh || !orient) { free(key); free(idx); free(fresh); free(orient); return -1; }
        #pragma omp parallel for num_threads(threads) schedule(static)
        for (int64_t i = 0; i < (int64_t)nb; i++) {
            uint32_t r, cc;
            rmat_edge(sk, (uint64_t)i, scale, a, a + b, a + b + c, &r, &cc);
            idx[i] = (uint32_t)i;
            if (symmetric) {
                uint32_t lo = r < cc ? r : cc, hi = r < cc ? cc : r;
                key[i] = (r == cc) ? invalid : (((uint64_t)lo << scale) | hi);
                orient[i] = (uint8_t)(r < cc);     /* 1: drawn as (lo, hi) */
            } else {
                key[i] = ((uint64_t)r << scale) | cc;
            }
        }
        uint64_t *keys_by_idx = (uint64_t *)malloc(nb * sizeof(uint64_t));
        if (!keys_by_idx) { free(key); free(idx); free(fresh); free(orient); return -1; }
        memcpy(keys_by_idx, key, nb * sizeof(uint64_t));
        if (sort_pairs(key, idx, nb, 2 * scale + 1, threads)) {
            free(key); free(idx); free(fresh); free(orient); free(keys_by_idx); return -1;
        }
        /* the first of each run of equal keys is the earliest draw */
        #pragma omp parallel for num_threads(threads) schedule(static)
        for (int64_t i = 0; i < (int64_t)nb; i++)
            if (key[i] != invalid && (i == 0 || key[i] != key[i - 1])) fresh[idx[i]] = 1;
        free(key); free(idx);
        /* keep the first 'target' fresh draws, in draw order */
        uint64_t *cnt = (uint64_t *)calloc((size_t)threads + 1, sizeof(uint64_t));
        #pragma omp parallel num_threads(threads)
        {
            int t = omp_get_thread_num();
            uint64_t lo = nb * (uint64_t)t / (uint64_t)threads, hi = nb * (uint64_t)(t + 1) / (uint64_t)threads;
            uint64_t k = 0;
            for (uint64_t i = lo; i < hi; i++) k += fresh[i];
            cnt[t + 1] = k;
        }
        for (int t = 0; t < threads; t++) cnt[t + 1] += cnt[t];
        if (cnt[threads] < target) {
            free(cnt); free(fresh); free(orient); free(keys_by_idx);
            nb *= 2;
            continue;
        }
        #pragma omp parallel num_threads(threads)
        {
            int t = omp_get_thread_num();
            uint64_t lo = nb * (uint64_t)t / (uint64_t)threads, hi = nb * (uint64_t)(t + 1) / (uint64_t)threads;
            uint64_t o = cnt[t];
            for (uint64_t i = lo; i < hi && o < target; i++) {
                if (!fresh[i]) continue;
                uint64_t kk = keys_by_idx[i];
                uint32_t k_hi = (uint32_t)(kk >> scale), k_lo = (uint32_t)(kk & ((1ull << scale) - 1));
                if (symmetric) {
                    uint32_t u = orient[i] ? k_hi : k_lo, v = orient[i] ? k_lo : k_hi;
                    rows[2 * o] = u; cols[2 * o] = v;
                    rows[2 * o + 1] = v; cols[2 * o + 1] = u;
                } else {
                    rows[o] = k_hi; cols[o] = k_lo;
                }
                o++;
            }
        }
        free(cnt); free(fresh); free(orient); free(keys_by_idx);
        return 0;
    }
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
