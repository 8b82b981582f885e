// Host-side checks of index arithmetic in cpr_io.hpp: the scan's chunk-state index on
// adversarial cu_seqlens (overlapping full-length ranges, negative and out-of-range offsets,
// decreasing entries), printed as "case <name> first=<i> last=<i> max=<i> total=<t>"; and
// the workgroup -> (pair, row block) map, printed as "case <name> bijective=<0|1>
// together=<0|1>" (together: the row blocks and heads of one sequence and q/k head share
// one XCD, workgroup id mod 8, whenever their group of 8 units is whole).
#include <cstdio>
#include <vector>

#include "cpr_io.hpp"

using gdn::io::block_work;
using gdn::io::clamp_chunk_index;
using gdn::io::full_chunks;

static void run_map(int pairs, int rblocks, int G) {
  const int n = pairs * rblocks;
  std::vector<int> seen(n, 0), xcd(pairs / G, -1);
  bool together = true;
  const int whole_units = (pairs / G) / 8 * 8;
  for (int b = 0; b < n; ++b) {
    int pair, rb;
    block_work(b, pairs, rblocks, G, pair, rb);
    if (pair < 0 || pair >= pairs || rb < 0 || rb >= rblocks) {
      std::printf("case map_P%d_R%d_G%d bijective=0 together=0\n", pairs, rblocks, G);
      return;
    }
    seen[pair * rblocks + rb] += 1;
    const int unit = pair / G;
    if (unit < whole_units) {
      if (xcd[unit] < 0) xcd[unit] = b % 8;
      together = together && xcd[unit] == b % 8;
    }
  }
  bool bij = true;
  for (int c : seen) bij = bij && c == 1;
  std::printf("case map_P%d_R%d_G%d bijective=%d together=%d\n", pairs, rblocks, G, (int)bij,
              (int)together);
}

static void run(const char *name, const std::vector<int32_t> &cu, int64_t T, int C,
                int64_t total) {
  const int N = (int)cu.size() - 1;
  unsigned long long sum = 0;
  int64_t first = -1, last = -1, mx = -1;
  for (int n = 0; n < N; ++n) {
    const int64_t idx = clamp_chunk_index(sum, total);
    if (n == 0) first = idx;
    last = idx;
    if (idx > mx) mx = idx;
    sum += full_chunks(cu.data(), n, T, C);
  }
  std::printf("case %s first=%lld last=%lld max=%lld total=%lld\n", name, (long long)first,
              (long long)last, (long long)mx, (long long)total);
}

int main() {
  const int64_t T = 2147483647;  // the largest admitted total_tokens
  std::vector<int32_t> overlap;  // every other sequence covers [0, T): 2^15 full ranges
  for (int n = 0; n < 65536; ++n) overlap.push_back(n % 2 ? (int32_t)T : 0);
  overlap.push_back((int32_t)T);
  run("overlapping_full_ranges", overlap, T, 16, T / 16);
  std::vector<int32_t> wild = {-5, 2147483647, -2147483647 - 1, 100, 50, 2147483647, 7};
  run("negative_and_decreasing", wild, T, 16, T / 16);
  std::vector<int32_t> plain = {0, 64, 64, 200, 1000};
  run("plain", plain, 1000, 64, 1 + 2 + 12);
  const int maps[][3] = {{64, 8, 1}, {32, 8, 2}, {2048, 2, 2}, {8192, 8, 2}, {96, 3, 4},
                         {40, 1, 4}, {7, 5, 1}, {6, 4, 2}, {1, 1, 1}, {1100 * 16, 1, 1}};
  for (const auto &m : maps) run_map(m[0], m[1], m[2]);
  return 0;
}
