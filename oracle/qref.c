/*
 * CPU oracle, quantised-weight part.  TEST INFRASTRUCTURE ONLY: the library
 * never links or calls this file; only the tests, the smoke check and the CPU
 * baseline leg of the benchmark do.
 *
 * What it computes (plain definitions, fp64):
 *   - decode of GGUF Q4_0 / Q8_0 blocks (Q4_0 weights: SwarmLLM README, model
 *     table and architecture paragraph; 8-bit weights: ChatTorrent README,
 *     "What it can run"):
 *       Q4_0: 18 bytes = fp16 d, 16 code bytes; byte j holds weight j in the
 *             low nibble and weight j+16 in the high nibble; w = (q - 8) * d
 *       Q8_0: 34 bytes = fp16 d, 32 signed code bytes; w = q * d
 *   - y = W x for one or several right-hand sides, every product and sum in
 *     fp64, rows in order, blocks in order, elements in order.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math).
 * OpenMP only splits the independent output rows between threads; each row's
 * sum is the same sequential loop on every thread count.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

#define ORC_Q4_0 2
#define ORC_Q8_0 8

/* IEEE 754 binary16 -> double, written out from the format definition. */
double orc_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)mant, -24);              /* subnormal: mant * 2^-14 * 2^-10 */
    } else if (expo == 31) {
        v = mant ? NAN : INFINITY;
    } else {
        v = ldexp((double)(mant + 1024), expo - 25); /* (1 + mant/1024) * 2^(expo-15) */
    }
    return sign ? -v : v;
}

int orc_block_bytes(int qtype) {
    if (qtype == ORC_Q4_0) return 18;
    if (qtype == ORC_Q8_0) return 34;
    return -1;
}

/* Decode one block into 32 doubles. */
static void decode_block(int qtype, const uint8_t *blk, double *out) {
    uint16_t dbits = (uint16_t)(blk[0] | (blk[1] << 8));
    double d = orc_half_to_double(dbits);
    if (qtype == ORC_Q4_0) {
        const uint8_t *qs = blk + 2;
        for (int j = 0; j < 16; ++j) {
            int lo = qs[j] & 0x0f;
            int hi = qs[j] >> 4;
            out[j] = (double)(lo - 8) * d;
            out[j + 16] = (double)(hi - 8) * d;
        }
    } else {
        const int8_t *qs = (const int8_t *)(blk + 2);
        for (int j = 0; j < 32; ++j) out[j] = (double)qs[j] * d;
    }
}

/* W: rows x (cols/32) blocks, row-major.  out: rows x cols doubles. */
int orc_dequant(int qtype, const uint8_t *w, int64_t rows, int64_t cols, double *out) {
    int bb = orc_block_bytes(qtype);
    if (bb < 0 || cols % 32) return -1;
    int64_t nb = cols / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b)
            decode_block(qtype, w + (r * nb + b) * bb, out + r * cols + b * 32);
    return 0;
}

/*
 * Y[t][r] = sum_c W[r][c] * X[t][c] for t < nrhs.  X: nrhs x cols, Y: nrhs x rows.
 * Each row is decoded once per call and used for every right-hand side.
 */
int orc_gemv(int qtype, const uint8_t *w, int64_t rows, int64_t cols,
             int nrhs, const double *x, double *y) {
    int bb = orc_block_bytes(qtype);
    if (bb < 0 || cols % 32 || nrhs < 1 || nrhs > 64) return -1;
    int64_t nb = cols / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double acc[64];
        double wv[32];
        int nt = nrhs;
        for (int t = 0; t < nt; ++t) acc[t] = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            decode_block(qtype, w + (r * nb + b) * bb, wv);
            for (int t = 0; t < nt; ++t) {
                const double *xb = x + (int64_t)t * cols + b * 32;
                double s = acc[t];
                for (int j = 0; j < 32; ++j) s += wv[j] * xb[j];
                acc[t] = s;
            }
        }
        for (int t = 0; t < nt; ++t) y[(int64_t)t * rows + r] = acc[t];
    }
    return 0;
}
