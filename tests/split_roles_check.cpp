// Host-only check of the split kernels' role layout (split_roles.hpp): over
// many host and HBM work-group counts and XCD counts, every host work-group
// number and every HBM work number is taken by exactly one work-group of the
// grid split_grid sizes; with the host XCD, host work-groups run only on
// XCD 0 (work-group b on XCD b mod n_xcd) and XCD 0 takes no HBM work; the
// grid has no round that is idle on every XCD; and the host-XCD rule follows
// its byte-ratio bound.
#include <cstdio>
#include <vector>

#include "split_roles.hpp"

using namespace dak;

static int fails = 0;
#define CHECK(c, ...)                    \
  do {                                   \
    if (!(c)) {                          \
      if (fails++ < 20) {                \
        std::printf("FAIL %s: ", #c);    \
        std::printf(__VA_ARGS__);        \
        std::printf("\n");               \
      }                                  \
    }                                    \
  } while (0)

static void check(int64_t host_wgs, int64_t hbm_wgs, int n_xcd) {
  const int64_t grid = split_grid(host_wgs, hbm_wgs, n_xcd);
  std::vector<int> host_seen(host_wgs, 0), hbm_seen(hbm_wgs, 0);
  for (int64_t b = 0; b < grid; ++b) {
    const SplitRole r = split_role(b, host_wgs, n_xcd);
    if (r.idle) {
      CHECK(n_xcd > 0 && b % n_xcd == 0, "b=%lld idle off the host XCD", (long long)b);
      continue;
    }
    if (r.host) {
      CHECK(r.index >= 0 && r.index < host_wgs, "host index %lld of %lld", (long long)r.index, (long long)host_wgs);
      if (r.index >= 0 && r.index < host_wgs) host_seen[r.index]++;
      if (n_xcd > 0) CHECK(b % n_xcd == 0, "host work-group b=%lld on XCD %lld", (long long)b, (long long)(b % n_xcd));
    } else {
      if (n_xcd > 0) CHECK(b % n_xcd != 0, "HBM work on the host XCD, b=%lld", (long long)b);
      if (r.index < hbm_wgs) {
        CHECK(r.index >= 0, "negative HBM index");
        if (r.index >= 0) hbm_seen[r.index]++;
      }
    }
  }
  for (int64_t i = 0; i < host_wgs; ++i)
    CHECK(host_seen[i] == 1, "host %lld seen %d times (host %lld hbm %lld xcd %d)", (long long)i, host_seen[i],
          (long long)host_wgs, (long long)hbm_wgs, n_xcd);
  for (int64_t i = 0; i < hbm_wgs; ++i)
    CHECK(hbm_seen[i] == 1, "hbm %lld seen %d times (host %lld hbm %lld xcd %d)", (long long)i, hbm_seen[i],
          (long long)host_wgs, (long long)hbm_wgs, n_xcd);
  if (n_xcd > 0 && grid > 0) {
    // the last round still holds a host work-group or HBM work
    const int64_t j = grid / n_xcd - 1;
    CHECK(j < host_wgs || j * (n_xcd - 1) < hbm_wgs, "an idle last round (host %lld hbm %lld xcd %d)",
          (long long)host_wgs, (long long)hbm_wgs, n_xcd);
  }
}

int main() {
  int cases = 0;
  for (int n_xcd : {0, 2, 3, 4, 8})
    for (int64_t host : {0, 1, 2, 3, 4, 7, 8, 16, 31, 32, 33, 100})
      for (int64_t hbm : {0, 1, 5, 6, 7, 8, 63, 64, 127, 384, 448, 1000, 1792}) {
        if (n_xcd > 0 && host == 0) continue;   // the host XCD needs a host role
        check(host, hbm, n_xcd);
        ++cases;
      }
  // The rule: a host share within three times the HBM time at a 110x rate
  // ratio; never without host work-groups, HBM rows or a second XCD.
  const int64_t hbm = 470LL << 20;
  CHECK(use_host_xcd(hbm / 110 * 3, hbm, 4, 8), "at the bound");
  CHECK(!use_host_xcd(hbm / 110 * 3 + 1, hbm, 4, 8), "past the bound");
  CHECK(use_host_xcd(3670016, 469762048, 4, 8), "70B down, one host tile-row");
  CHECK(!use_host_xcd(2621440, 47710208, 16, 8), "Llama-8B qkv at x = 0.05");
  CHECK(!use_host_xcd(1, hbm, 0, 8), "no host work-groups");
  CHECK(!use_host_xcd(1, hbm, 4, 1), "one XCD");
  CHECK(!use_host_xcd(1, 0, 4, 8), "no HBM rows");
  std::printf("%d layouts checked, %d failures\n", cases, fails);
  return fails ? 1 : 0;
}
