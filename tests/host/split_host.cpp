// Host build of the chunk planner's grad_h split rule (grad_h_split in
// flce_internal.hpp).  For tests/test_split_rule_host.py: reads lines
// "tiles ksteps s_max" from stdin and writes "splits per" for each.
#include <cstdio>

#include "flce_internal.hpp"

int main() {
  long long tiles = 0, ksteps = 0, s_max = 0;
  while (std::scanf("%lld %lld %lld", &tiles, &ksteps, &s_max) == 3) {
    const flce::SplitChoice c = flce::grad_h_split(tiles, ksteps, s_max);
    std::printf("%d %d\n", c.splits, c.per);
  }
  return 0;
}
