/* Exhaustive host check of the division-free group scale used by the activation quantizer:
 * for every non-negative finite float a (subnormals and zero included),
 *     q1 = RN(a * RN(1/7));  q = RN(fma(RN(fma(-7, q1, a)), RN(1/7), q1))
 * equals the IEEE quotient RN(a / 7). Exit status 0 when every value matches.
 * Optional argument: a stride (1 = every value; larger strides sample). */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bits_to_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t float_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(int argc, char** argv) {
  const uint32_t stride = argc > 1 ? (uint32_t)strtoul(argv[1], NULL, 10) : 1u;
  fesetround(FE_TONEAREST);
  volatile float seven = 7.0f;
  const float rcp7 = 1.0f / seven;
  if (float_to_bits(rcp7) != 0x3E124925u) { printf("unexpected RN(1/7) %08x\n", float_to_bits(rcp7)); return 2; }
  uint64_t checked = 0, bad = 0;
  for (uint64_t u = 0; u < 0x7F800000u; u += stride) {
    const float a = bits_to_float((uint32_t)u);
    const float ieee = a / seven;
    const float q1 = a * rcp7;
    const float q = fmaf(fmaf(-7.0f, q1, a), rcp7, q1);
    if (float_to_bits(q) != float_to_bits(ieee)) {
      if (bad < 5) printf("mismatch at %08x: %08x vs %08x\n", (uint32_t)u, float_to_bits(q), float_to_bits(ieee));
      ++bad;
    }
    ++checked;
  }
  printf("checked %llu values, %llu mismatches\n", (unsigned long long)checked, (unsigned long long)bad);
  return bad != 0;
}
