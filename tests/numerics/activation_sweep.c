/* Accuracy of the device activations' evaluation method, on the CPU.
 *
 * Mirrors gelu_f32 and silu_f32 of segmented_dual_scale_amd/csrc/act_kernels.hip
 * operation by operation in fp32 (fmaf where the device uses FMA), with the
 * hardware reciprocal, exp2 and the library expf each off by -1, 0 or +1 ulp
 * in every combination.  Every finite bf16 input is checked against the fp64
 * definitions, GELU z/2 erfc(-z/sqrt 2) and SiLU z/(1+e^-z):
 *   |f32 result - fp64 value| <= 2^-19 |fp64 value| + 2^-140,
 * the bound the GPU tests apply to the device results.  Exit status 0 when
 * every input is within the bound and finite; prints the largest relative
 * error.  Build: cc -O2 -ffp-contract=off activation_sweep.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float ulps(float x, int d) { /* x moved by d ulps (finite nonzero x) */
  uint32_t u;
  memcpy(&u, &x, 4);
  if (x != 0.0f && isfinite(x)) u += (uint32_t)d;
  memcpy(&x, &u, 4);
  return x;
}

static int d_rcp, d_e1, d_e2, d_exp;

/* erfc in the Numerical Recipes form (Press et al., Numerical Recipes in C,
 * 2nd ed., section 6.2), -x^2 carried exactly, as on the device */
static float gelu32(float z) {
  const float kLog2e = 1.44269504f, kLog2eLo = 1.92596303e-08f;
  const float a = fminf(fabsf(z), 20.0f);
  const float x = a * 0.70710678f;
  const float t = ulps(1.0f / fmaf(0.5f, x, 1.0f), d_rcp);
  float P = fmaf(t, 0.17087277f, -0.82215223f);
  P = fmaf(t, P, 1.48851587f);
  P = fmaf(t, P, -1.13520398f);
  P = fmaf(t, P, 0.27886807f);
  P = fmaf(t, P, -0.18628806f);
  P = fmaf(t, P, 0.09678418f);
  P = fmaf(t, P, 0.37409196f);
  P = fmaf(t, P, 1.00002368f);
  P = fmaf(t, P, -1.26551223f);
  const float p = a * a, e = fmaf(a, a, -p);
  const float q = -0.5f * p, qe = -0.5f * e;
  const float hi = q * kLog2e;
  float lo = fmaf(q, kLog2e, -hi);
  lo = fmaf(q, kLog2eLo, lo);
  lo = fmaf(qe + P, kLog2e, lo);
  const int deep = hi < -120.0f;
  const float eh = ulps(exp2f(deep ? hi + 64.0f : hi), d_e1) * (deep ? 0x1p-64f : 1.0f);
  const float E = t * eh * ulps(exp2f(lo), d_e2);
  return 0.5f * z * (z < 0.0f ? E : 2.0f - E);
}

static float silu32(float z) {
  const float ez = ulps(expf(-fabsf(z)), d_exp);
  const float r = 1.0f / (1.0f + ez);
  return z * (z >= 0.0f ? r : ez * r);
}

static int sweep(const char *name, float (*f)(float), double (*ref)(double)) {
  double worst = 0.0, worst_z = 0.0;
  for (uint32_t bits = 0; bits < 65536u; ++bits) {
    float z;
    const uint32_t b = bits << 16;
    memcpy(&z, &b, 4);
    if (!isfinite(z)) continue;
    const float g = f(z);
    const double v = ref((double)z);
    if (!isfinite(g)) {
      printf("%s: non-finite result at z=%.9g\n", name, z);
      return 1;
    }
    const double err = fabs((double)g - v), bound = ldexp(fabs(v), -19) + ldexp(1.0, -140);
    if (!(err <= bound)) {
      printf("%s: z=%.9g value %.9g, fp64 %.9g, outside the bound\n", name, z, g, v);
      return 1;
    }
    if (fabs(v) > 1e-30 && err / fabs(v) > worst) {
      worst = err / fabs(v);
      worst_z = z;
    }
  }
  printf("%s (rcp %+d, exp2 %+d %+d, expf %+d): max relative error 2^%.2f at z=%g\n", name, d_rcp,
         d_e1, d_e2, d_exp, worst > 0 ? log2(worst) : -INFINITY, worst_z);
  return 0;
}

static double gelu64(double z) { return 0.5 * z * erfc(-z / sqrt(2.0)); }
static double silu64(double z) { return z / (1.0 + exp(-z)); }

int main(void) {
  for (d_rcp = -1; d_rcp <= 1; ++d_rcp)
    for (d_e1 = -1; d_e1 <= 1; ++d_e1)
      for (d_e2 = -1; d_e2 <= 1; ++d_e2)
        if (sweep("gelu", gelu32, gelu64)) return 1;
  d_rcp = d_e1 = d_e2 = 0;
  for (d_exp = -1; d_exp <= 1; ++d_exp)
    if (sweep("silu", silu32, silu64)) return 1;
  return 0;
}
