/* Exhaustive check of the activation quantizers' quotient (CPU only).
 *
 * The quantizers divide each bf16 value a of a row by the row's scale
 * s = absmax / FMAX (reading: IEEE fp32 division). The GPU kernels compute
 * the quotient as a reciprocal with one fused multiply-add correction
 * (Markstein's correction of a reciprocal quotient):
 *     y = RN(1 / s),  q0 = RN(a * y),  r = fma(-q0, s, a),  q = fma(r, y, q0),
 * then copy a's sign onto q, and only when s >= 2^-100 and y is finite
 * (other rows divide). This program enumerates every positive finite bf16
 * absmax, FMAX in {448, 240, 127} (OCP E4M3, E4M3FNUZ, int8) and every bf16
 * a with |a| <= absmax, both signs, and counts the pairs where the two
 * quotients can give different codes: the bits differ and either quotient
 * is at least 2^-12 in magnitude (below 2^-12 every format's code is a zero,
 * signed like the quotient, and the sign copy keeps the signs equal).
 * Output: "checked <pairs> same_bits <pairs> bad <pairs> divided_rows <n>".
 * Built with -ffp-contract=off so that only fmaf fuses.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16_value(uint32_t b) {
  const uint32_t u = b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint32_t bits_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

int main(void) {
  static const float kFmax[3] = {448.0f, 240.0f, 127.0f};
  const float tiny = 0x1p-12f;
  long long checked = 0, same = 0, bad = 0, divided = 0;
  for (int f = 0; f < 3; ++f) {
#pragma omp parallel for reduction(+ : checked, same, bad, divided) schedule(dynamic, 16)
    for (int ab = 1; ab < 0x7F80; ++ab) { /* positive finite bf16 absmax */
      const float s = bf16_value((uint32_t)ab) / kFmax[f];
      const float y = 1.0f / s;
      if (!(s >= 0x1p-100f) || !isfinite(y)) {
        divided++;
        continue;
      }
      for (int xb = 0; xb <= ab; ++xb) {
        for (int sg = 0; sg < 2; ++sg) {
          const float a = bf16_value((uint32_t)xb | ((uint32_t)sg << 15));
          const float qi = a / s;
          const float q0 = a * y;
          const float q = copysignf(fmaf(fmaf(-q0, s, a), y, q0), a);
          checked++;
          if (bits_of(qi) == bits_of(q)) {
            same++;
          } else if (fabsf(qi) >= tiny || fabsf(q) >= tiny) {
            bad++;
          }
        }
      }
    }
  }
  printf("checked %lld same_bits %lld bad %lld divided_rows %lld\n", checked, same, bad, divided);
  return bad != 0;
}
