/* Running sums of a sequence of float32 increments, three ways:
 *   - as the decode kernel updates a slot's score each step: plain float32
 *     adds (s += w, c stays 0) for the first `plain` increments, then
 *     compensated ones: y = w - c; t = s + y; c = (t - s) - y; s = t;
 *   - plain float32 (s += w);
 *   - float64 (the reference).
 * Build without contraction or fast math, so every float operation is one
 * IEEE binary32 add or subtract rounded to nearest even, as on the GPU. */
#include <stdint.h>

void kahan_drift(const float* w, int64_t n, int64_t plain_n, int64_t every, float* s_out, float* c_out,
                 float* plain_out, double* exact_out) {
  float s = 0.f, c = 0.f, plain = 0.f;
  double exact = 0.0;
  int64_t k = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (i < plain_n) {
      s = s + w[i];
    } else {
      const float y = w[i] - c;
      const float t = s + y;
      c = (t - s) - y;
      s = t;
    }
    plain += w[i];
    exact += (double)w[i];
    if ((i + 1) % every == 0) {
      s_out[k] = s;
      c_out[k] = c;
      plain_out[k] = plain;
      exact_out[k] = exact;
      ++k;
    }
  }
}
