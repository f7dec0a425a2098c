/* Exhaustive check of the oracle's exp over every binary32 d in [-80, 0]:
 * error in units in the last place against libm's double exp rounded to
 * float, and how far it ever steps up as d decreases.  Test code: compiled
 * and loaded by tests/test_oracle_pins.py; it calls the oracle through a
 * function pointer. */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef float (*expf_fn)(float);

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static int32_t to_bits(float f) { int32_t u; memcpy(&u, &f, 4); return u; }

/* result[0] = max |ulp error| against (float)exp((double)d)
 * result[1] = largest upward step, in ulp, between d and the next float below
 * result[2] = number of upward steps
 * result[3] = number of values checked
 * result[4] = bits of f(0) */
void sweep(expf_fn f, int64_t *result)
{
    int64_t max_ulp = 0, max_up = 0, n_up = 0, count = 0;
    const uint32_t lo = 0x80000000u;      /* -0.0 */
    const uint32_t hi = 0xC2A00000u;      /* -80.0 */
    const int64_t n = (int64_t)(hi - lo) + 1;
#pragma omp parallel for reduction(max:max_ulp,max_up) reduction(+:n_up,count) schedule(static)
    for (int64_t k = 0; k < n; ++k) {
        float d = from_bits(lo + (uint32_t)k);
        float got = f(d);
        float want = (float)exp((double)d);
        int64_t du = (int64_t)to_bits(got) - (int64_t)to_bits(want);
        if (du < 0) du = -du;
        if (du > max_ulp) max_ulp = du;
        if (k + 1 < n) {
            float below = f(from_bits(lo + (uint32_t)k + 1));  /* next smaller d */
            int64_t step = (int64_t)to_bits(below) - (int64_t)to_bits(got);
            if (step > 0) {
                n_up += 1;
                if (step > max_up) max_up = step;
            }
        }
        count += 1;
    }
    result[0] = max_ulp;
    result[1] = max_up;
    result[2] = n_up;
    result[3] = count;
    result[4] = to_bits(f(0.0f));
}
