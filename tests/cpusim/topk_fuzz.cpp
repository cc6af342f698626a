// Fuzz of the workgroup top-(k-1) (wg_topk, recsa_device.hpp) built for the
// host: every GPU lane is a host thread (tests/cpusim/shim), so the kernel's
// own code -- LDS histograms, radix passes, small-bin ranking, compaction,
// and its barrier placement -- runs under AddressSanitizer, UBSan or
// ThreadSanitizer.  Each case checks the kept set against the exact top-(k-1)
// of the importances the kernel itself wrote (value descending, then lower
// position), the count, the current node last, and the kept-position bitmap.
#include <algorithm>
#include <cstdio>
#include <random>
#include <thread>

#include "recsa_device.hpp"

using namespace recsa;

template <int G, int NT, int CKM>
static bool run_case(std::mt19937& rng, int n, int k, int mode, int CK) {
  std::vector<float> lg(static_cast<size_t>(G) * CK, 0.f);
  std::normal_distribution<float> nd(0.f, 2.f);
  for (int g = 0; g < G; ++g)
    for (int p = 0; p < n; ++p) {
      float v = nd(rng);
      if (mode == 1) v = std::round(v * 2.f) / 2.f;        // many exact ties
      if (mode == 2) v = 0.5f;                              // all equal
      if (mode == 3) v = (p % 7 == 0) ? 3.f : -1.f;         // two levels
      if (mode == 4) v = 1.f + 1e-6f * static_cast<float>(p % 5);   // near-equal
      lg[static_cast<size_t>(g) * CK + p] = v;
    }
  std::vector<int32_t> sel(static_cast<size_t>(k), -7);
  int32_t cnt = -7;
  std::vector<uint32_t> bm(static_cast<size_t>((CK + 31) / 32), 0xDEADBEEFu);
  std::vector<float> imp(static_cast<size_t>(CK), -1.f);
  auto sm = std::make_unique<TopkSmem>();
  std::memset(sm.get(), 0xCD, sizeof(TopkSmem));       // stale LDS contents
  ListView lv;
  lv.len = n + 1;
  lv.cur = n;
  lv.up = nullptr;                                     // prefix list: node p at position p
  cpusim::Block block(NT);
  std::vector<std::thread> th;
  for (int t = 0; t < NT; ++t)
    th.emplace_back([&, t] {
      cpusim::blk = &block;
      threadIdx.x = static_cast<unsigned>(t);
      wg_topk<G, NT, CKM>(lg.data(), n, k, CK, lv, sel.data(), &cnt, bm.data(), imp.data(), *sm);
    });
  for (auto& x : th) x.join();
  // reference: exact top-(k-1) of the kernel's own importances
  std::vector<int> order(static_cast<size_t>(n));
  for (int p = 0; p < n; ++p) order[p] = p;
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return imp[a] > imp[b] || (imp[a] == imp[b] && a < b); });
  std::vector<int> want(order.begin(), order.begin() + (k - 1));
  std::sort(want.begin(), want.end());
  std::vector<int> got(sel.begin(), sel.begin() + (k - 1));
  std::sort(got.begin(), got.end());
  bool ok = cnt == k && sel[k - 1] == n && got == want;
  for (int p = n; p < CK; ++p) ok = ok && imp[p] == 0.f;
  for (int p = 0; p < CK; ++p) {
    const bool kept = std::binary_search(want.begin(), want.end(), p);
    ok = ok && (((bm[p / 32] >> (p % 32)) & 1u) != 0) == kept;
  }
  if (!ok) std::fprintf(stderr, "FAIL G=%d NT=%d n=%d k=%d mode=%d cnt=%d\n", G, NT, n, k, mode, cnt);
  return ok;
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 20;
  std::mt19937 rng(12345);
  int fails = 0, cases = 0;
  const int ks[] = {4, 16, 64, 256};
  for (int it = 0; it < iters; ++it) {
    const int k = ks[it % 4];
    const int CK = 16 * k;
    const int mode = (it / 4) % 5;
    std::uniform_int_distribution<int> nd(k, CK - 1);
    const int n = (it % 3 == 0) ? CK - 1 : nd(rng);
    const bool wide = it % 2;
    if (it % 3 == 2)
      fails += !run_case<1, 256, 4096>(rng, n, k, mode, CK);
    else if (wide)
      fails += !run_case<4, 512, 4096>(rng, n, k, mode, CK);
    else
      fails += !run_case<4, 256, 4096>(rng, n, k, mode, CK);
    ++cases;
  }
  // the k = 512 class (lists of up to 8191 candidates)
  for (int it = 0; it < iters / 5 + 1; ++it) {
    std::uniform_int_distribution<int> nd(512, 8191);
    fails += !run_case<2, 512, 8192>(rng, it == 0 ? 8191 : nd(rng), 512, it % 5, 8192);
    ++cases;
  }
  std::printf("%d cases, %d failed\n", cases, fails);
  return fails != 0;
}
