/*
 * Exhaustive check of the oracle's integer contraction on 4 x 4 ternary
 * weight matrices: all 3^16 = 43,046,721 of them, each against six
 * fixed int8 activation rows (including the extremes +-127 and 0).
 *
 * The expected value is built without a multiplication: each weight matrix
 * is enumerated as a base-3 number, split into a mask of +1 positions and a
 * mask of -1 positions, and the output is the sum of the activations under
 * the first mask minus the sum under the second (the pages: with ternary
 * weights the product reduces to integer additions -- anthology note-168 on
 * arXiv 2402.17764, "The part that is a bet rather than a measurement").
 *
 * Prints "ok <count>" and exits 0, or prints the first mismatch and exits 1.
 */
#include <stdint.h>
#include <stdio.h>

#include "../../oracle/oracle.h"

static const int8_t Q[6][4] = {
    {127, -127, 0, 1}, {100, -50, 25, -12}, {0, 0, 0, 0},
    {127, 127, 127, 127}, {-127, -127, -127, -127}, {-77, 33, 91, -2},
};

int main(void)
{
    int8_t T[16];
    int32_t acc[6 * 4];
    long count = 0;
    for (long code = 0; code < 43046721L; ++code) {
        long c = code;
        unsigned plus = 0, minus = 0;
        for (int i = 0; i < 16; ++i) {
            int d = (int)(c % 3);
            c /= 3;
            T[i] = (int8_t)(d - 1);
            if (d == 2) plus |= 1u << i;
            if (d == 0) minus |= 1u << i;
        }
        oracle_matmul(&Q[0][0], T, 6, 4, 4, acc);
        for (int m = 0; m < 6; ++m) {
            for (int n = 0; n < 4; ++n) {
                int32_t e = 0;
                for (int k = 0; k < 4; ++k) {
                    int bit = 4 * n + k;
                    if (plus >> bit & 1u) e += Q[m][k];
                    if (minus >> bit & 1u) e -= Q[m][k];
                }
                if (e != acc[m * 4 + n]) {
                    printf("mismatch code=%ld m=%d n=%d got=%d want=%d\n", code, m, n,
                           acc[m * 4 + n], e);
                    return 1;
                }
            }
        }
        ++count;
    }
    printf("ok %ld\n", count);
    return 0;
}
