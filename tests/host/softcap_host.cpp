// Host build of the softcap helpers of device_common.hpp, for
// tests/test_softcap_host.py: reads (m, T) and raw accumulator values a
// (float32, binary) from stdin, writes the capped logits z (float32, binary)
// to stdout, computed with CapSeries / softcap_value exactly as the kernels
// apply them (the device replaces the division by a hardware reciprocal and
// exp2 by the hardware exp2).
#include <cstdio>
#include <cstdint>
#include <vector>

#include "device_common.hpp"

int main() {
  float mt[2];
  int64_t n = 0;
  if (fread(mt, sizeof(float), 2, stdin) != 2 || fread(&n, sizeof(n), 1, stdin) != 1 || n < 0) return 2;
  std::vector<float> a(static_cast<size_t>(n)), z(static_cast<size_t>(n));
  if (fread(a.data(), sizeof(float), a.size(), stdin) != a.size()) return 3;
  const float m = mt[0], T = mt[1];
  const flce::CapSeries c(m, T > 0.0f ? 1.0f / T : 0.0f, T > 0.0f ? T : 0.0f);
  for (size_t i = 0; i < a.size(); ++i) z[i] = T > 0.0f ? flce::softcap_value(a[i], c) : a[i] * m;
  if (fwrite(z.data(), sizeof(float), z.size(), stdout) != z.size()) return 4;
  return 0;
}
