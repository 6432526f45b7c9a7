/*
 * Sanitizer driver for the oracle's C recurrence (oracle/recurrence.c),
 * built by tests/test_sanitizers_cpu.py with AddressSanitizer +
 * UndefinedBehaviorSanitizer, and again with ThreadSanitizer, and run on the
 * CPU.  Every array is allocated at exactly the size the documented layout
 * needs, so a read or write past any of them is reported.  Cases: every
 * kind, sizes from 1 up, T = 0, with and without h0, one and several
 * threads, and the argument checks.  Exit status 0 when every call returned
 * what it should and every output is finite.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_forward(int kind, const double* q, const double* k, const double* v, const double* g,
                   const double* beta, const double* h0, double* o, double* hT, int B, int T, int H, int Dk,
                   int Dv, int nthreads);

static unsigned seed = 12345u;
static double uni(void)   /* uniform in [0, 1) */
{
    seed = seed * 1664525u + 1013904223u;
    return (double)(seed >> 8) / 16777216.0;
}

static double* alloc_fill(size_t n, double lo, double hi)
{
    double* p = (double*)malloc(n ? n * sizeof(double) : 1);
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * uni();
    return p;
}

static int finite_all(const double* p, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

int main(void)
{
    static const int sizes[][5] = {{1, 1, 1, 1, 1}, {2, 37, 3, 8, 5}, {1, 0, 2, 4, 4}, {3, 65, 2, 16, 16},
                                   {1, 130, 1, 3, 7}};
    int bad = 0;
    for (int kind = 0; kind < 3; ++kind)
        for (size_t s = 0; s < sizeof(sizes) / sizeof(sizes[0]); ++s)
            for (int with_h0 = 0; with_h0 < 2; ++with_h0)
                for (int threads = 1; threads <= 3; threads += 2) {
                    const int B = sizes[s][0], T = sizes[s][1], H = sizes[s][2], Dk = sizes[s][3], Dv = sizes[s][4];
                    const size_t nk = (size_t)B * T * H * Dk, nv = (size_t)B * T * H * Dv, nr = (size_t)B * T * H;
                    const size_t ns = (size_t)B * H * Dv * Dk;
                    double* q = alloc_fill(nk, -1, 1);
                    double* k = alloc_fill(nk, -1, 1);
                    double* v = alloc_fill(nv, -1, 1);
                    double* g = alloc_fill(kind == 0 ? nk : nr, -0.1, 0.0);
                    double* beta = alloc_fill(nr, 0.0, 1.0);
                    double* h0 = with_h0 ? alloc_fill(ns, -0.2, 0.2) : NULL;
                    double* o = alloc_fill(nv, 0, 0);
                    double* hT = alloc_fill(ns, 0, 0);
                    const int rc = oracle_forward(kind, q, k, v, g, kind == 2 ? NULL : beta, h0, o, hT, B, T, H, Dk,
                                                  Dv, threads);
                    if (rc != 0 || !finite_all(o, nv) || !finite_all(hT, ns)) {
                        fprintf(stderr, "case kind=%d B=%d T=%d H=%d Dk=%d Dv=%d h0=%d threads=%d: rc %d\n", kind,
                                B, T, H, Dk, Dv, with_h0, threads, rc);
                        ++bad;
                    }
                    free(q); free(k); free(v); free(g); free(beta); free(h0); free(o); free(hT);
                }
    /* argument checks: no array is touched */
    double x = 0.0;
    if (oracle_forward(3, &x, &x, &x, &x, &x, NULL, &x, &x, 1, 1, 1, 1, 1, 1) != -1) ++bad;
    if (oracle_forward(0, &x, &x, &x, &x, &x, NULL, &x, &x, 1, 1, 1, 0, 1, 1) != -1) ++bad;
    if (oracle_forward(0, NULL, &x, &x, &x, &x, NULL, &x, &x, 1, 1, 1, 1, 1, 1) != -1) ++bad;
    if (oracle_forward(1, &x, &x, &x, &x, NULL, NULL, &x, &x, 1, 1, 1, 1, 1, 1) != -1) ++bad;
    if (oracle_forward(0, &x, &x, &x, &x, &x, NULL, NULL, &x, 1, 1, 1, 1, 1, 1) != -1) ++bad;
    printf("oracle driver: %d failure(s)\n", bad);
    return bad ? 1 : 0;
}
