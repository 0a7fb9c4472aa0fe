/*
 * Exhaustive check of the oracle's binary32 -> OCP E4M3 and binary32 -> bf16
 * encoders over all 2^32 inputs, against a brute-force nearest-code search.
 *
 * The brute force shares nothing with the oracle's encoders: it decodes every
 * non-negative finite code of each format into its exact value (from the
 * format's definition: E4M3 with bias 7, 3 fraction bits, subnormal spacing
 * 2^-9, largest finite 448; bf16 = upper half of a binary32), then picks the
 * code nearest to |v| by binary search, breaking exact ties toward the code
 * with an even last bit.  Rules that are readings rather than arithmetic are
 * applied as stated: E4M3 saturates every |v| >= 448 (infinities included) to
 * 448 and maps NaN to S.1111.111; bf16 overflows to infinity past the largest
 * finite value by the same nearest rule (as if the exponent range continued)
 * and maps NaN to the quiet NaN with the same sign and upper payload.
 *
 * Usage: encoder_sweep <path to libmsa_oracle.so>; exit status 0 iff no mismatch.
 */
#include <dlfcn.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

typedef uint8_t (*e4m3_fn)(float);
typedef uint16_t (*bf16_fn)(float);

static double e4m3_val[127];   /* codes 0x00..0x7E */
static double bf16_val[0x7F81]; /* codes 0x0000..0x7F7F, plus 0x7F80 standing for 2^128 */

static void build_tables(void)
{
    for (int c = 0; c <= 0x7E; ++c) {
        int E = (c >> 3) & 15, M = c & 7;
        e4m3_val[c] = E == 0 ? ldexp((double)M, -9) : ldexp((double)(8 + M), E - 7 - 3);
    }
    for (int c = 0; c <= 0x7F7F; ++c) {
        uint32_t u = (uint32_t)c << 16;
        float f;
        memcpy(&f, &u, 4);
        bf16_val[c] = (double)f;
    }
    bf16_val[0x7F80] = ldexp(1.0, 128);
}

/* nearest code in table[0..last] to a (0 <= a < table[last]), ties to even code */
static int nearest(const double* table, int last, double a)
{
    int lo = 0, hi = last;
    while (hi - lo > 1) {              /* invariant: table[lo] <= a < table[hi] */
        int mid = (lo + hi) / 2;
        if (table[mid] <= a) lo = mid; else hi = mid;
    }
    if (table[lo] == a) return lo;
    double m = 0.5 * (table[lo] + table[hi]);  /* exact: both have few significant bits */
    if (a < m) return lo;
    if (a > m) return hi;
    return (lo & 1) ? hi : lo;
}

static uint8_t brute_e4m3(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    uint8_t sign = (u >> 31) ? 0x80 : 0;
    if (isnan(f)) return sign | 0x7F;
    double a = fabs((double)f);
    if (a >= 448.0) return sign | 0x7E;
    return sign | (uint8_t)nearest(e4m3_val, 0x7E, a);
}

static uint16_t brute_bf16(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    uint16_t sign = (u >> 31) ? 0x8000 : 0;
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040);
    if (isinf(f)) return sign | 0x7F80;
    double a = fabs((double)f);
    return sign | (uint16_t)nearest(bf16_val, 0x7F80, a);
}

int main(int argc, char** argv)
{
    if (argc < 2) { fprintf(stderr, "usage: %s liboracle.so\n", argv[0]); return 2; }
    void* h = dlopen(argv[1], RTLD_NOW);
    if (!h) { fprintf(stderr, "dlopen: %s\n", dlerror()); return 2; }
    e4m3_fn enc8 = (e4m3_fn)dlsym(h, "msa_oracle_e4m3");
    bf16_fn enc16 = (bf16_fn)dlsym(h, "msa_oracle_bf16");
    if (!enc8 || !enc16) { fprintf(stderr, "missing symbols\n"); return 2; }
    build_tables();
    long long bad8 = 0, bad16 = 0;
    #pragma omp parallel for reduction(+:bad8, bad16) schedule(static)
    for (long long i = 0; i < (1LL << 32); ++i) {
        uint32_t u = (uint32_t)i;
        float f;
        memcpy(&f, &u, 4);
        uint8_t e = brute_e4m3(u), g = enc8(f);
        if (e != g) {
            if (bad8 < 4) printf("e4m3 mismatch 0x%08x: oracle 0x%02x brute 0x%02x\n", u, g, e);
            ++bad8;
        }
        uint16_t b = brute_bf16(u), c = enc16(f);
        if (b != c) {
            if (bad16 < 4) printf("bf16 mismatch 0x%08x: oracle 0x%04x brute 0x%04x\n", u, c, b);
            ++bad16;
        }
    }
    printf("e4m3 mismatches: %lld\nbf16 mismatches: %lld\n", bad8, bad16);
    return (bad8 || bad16) ? 1 : 0;
}
