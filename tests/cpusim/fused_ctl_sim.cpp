// CPU emulation of the fused decode's control protocol (recsa_fused_ctl.hpp,
// built for the host: each emulated workgroup is 64 host threads, its
// thread 0 runs the protocol's atomics as the kernel's thread 0 does).
// Every member runs the kernel's control skeleton -- placement mark, one
// barrier per scored level, its partial, then the final arrival and the
// merge (XCD-local form) or the final flags and member 0's merge
// (device-wide form) -- and the checks are the contract of recsa_decode:
//   a normal call: output = the merged partials, error word 0, every control
//     word left zero (so the next call can start);
//   members on two XCDs: NaN output, error bit 1 (sharing one L2) or bit 0
//     (two L2s: every wait times out, no member merges);
//   a straggler that arrives after the others' waits ran out: NaN output and
//     a nonzero error word, whatever it does afterwards; once the caller
//     zeroes the control block (as the header requires), calls work again.
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <memory>
#include <thread>
#include <vector>

#include "recsa_fused_ctl.hpp"

using namespace recsa;

namespace {

constexpr int kNT = 64;                 // threads per emulated workgroup
constexpr int kWords = 16 + 16 * kFusedMaxW;

struct Device {
  uint32_t ctl[kWords];                 // the group's control block
  uint32_t l2b[kWords];                 // a second XCD's L2 copy of the XCD-local words
  float part[kFusedMaxW];
  std::atomic<float> out;               // several timed-out members may poison it at once
  std::atomic<int> finished{0};         // members whose run has ended
};

struct Member {                         // one workgroup
  int w;
  int xcd;
  bool other_l2;                        // its XCD-local words live in l2b
  bool straggler;                       // starts only after every other member finished
  std::unique_ptr<cpusim::Block> blk;
  uint32_t s_fail = 0, s_last = 0, s_bad = 0;
};

void run_member(Device& dev, Member& mb, bool xl, int W, int n_rounds, uint32_t spin, int t) {
  cpusim::blk = mb.blk.get();
  threadIdx.x = static_cast<unsigned>(t);
  sim_xcc = mb.xcd;
  if (mb.straggler) {
    while (dev.finished.load() < W - 1) std::this_thread::yield();
  }
  FusedCtl c = fused_ctl(dev.ctl);
  if (mb.other_l2) c.counter = dev.l2b + 2;            // its L2's copy of the arrival words
  if (t == 0) {
    mb.s_fail = 0u;
    if (xl) ctl_mark_xcd(c, &mb.s_fail);
  }
  uint32_t gen = 0;
  for (int l = 0; l < n_rounds; ++l) {
    ++gen;
    if (xl)
      group_barrier_xcd(c.counter, gen * static_cast<uint32_t>(W), c.err, &mb.s_fail, spin);
    else
      group_barrier(c.flags, mb.w, W, gen, c.err, &mb.s_fail, spin);
  }
  if (t == 0) dev.part[mb.w] = static_cast<float>(mb.w + 1);
  __syncthreads();
  if (mb.s_fail && t == 0) dev.out.store(std::nanf(""));   // a timed-out wait poisons the output
  auto merged = [&] {
    float s = 0.f;
    for (int i = 0; i < W; ++i) s += dev.part[i];
    return s;
  };
  if (xl) {
    __syncthreads();
    FusedStatus st;
    if (t == 0) mb.s_last = xl_final_arrival(c, gen, W, st) ? 1u : 0u;
    __syncthreads();
    if (mb.s_last) {
      const float m = merged();
      if (t == 0) mb.s_bad = xl_result_bad(c, st, mb.s_fail) ? 1u : 0u;
      __syncthreads();
      if (t == 0) {
        dev.out.store(mb.s_bad ? std::nanf("") : m);
        xl_reset(c);
      }
    }
  } else if (mb.w != 0) {
    __syncthreads();
    if (t == 0) dw_final_flag(c, mb.w, gen);
  } else {
    group_barrier(c.flags, 0, W, gen + 1, c.err, &mb.s_fail, spin);
    const float m = merged();
    __syncthreads();
    if (t == 0) dev.out.store(dw_result_bad(c, mb.s_fail) ? std::nanf("") : m);
    dw_reset(c, t, W);
  }
  __syncthreads();
  if (t == 0) dev.finished.fetch_add(1);
}

struct Scenario {
  const char* name;
  bool xl;
  int W, n_rounds;
  uint32_t spin;
  int split;            // 0: one XCD; 1: members w >= W/2 on XCD 1, same L2; 2: on XCD 1 with its own L2
  int straggler;        // member index, or -1
};

// Runs one call; returns the output and leaves the device state.
float call(Device& dev, const Scenario& sc) {
  dev.out.store(-1.f);
  dev.finished = 0;
  for (int i = 0; i < kFusedMaxW; ++i) dev.part[i] = 0.f;
  std::vector<Member> mbs(static_cast<size_t>(sc.W));
  std::vector<std::thread> th;
  for (int w = 0; w < sc.W; ++w) {
    Member& mb = mbs[static_cast<size_t>(w)];
    mb.w = w;
    const bool hi = sc.split > 0 && w >= sc.W / 2;
    mb.xcd = hi ? 1 : 0;
    mb.other_l2 = hi && sc.split == 2;
    mb.straggler = w == sc.straggler;
    mb.blk = std::make_unique<cpusim::Block>(kNT);
  }
  for (int w = 0; w < sc.W; ++w)
    for (int t = 0; t < kNT; ++t)
      th.emplace_back(run_member, std::ref(dev), std::ref(mbs[static_cast<size_t>(w)]), sc.xl, sc.W,
                      sc.n_rounds, sc.spin, t);
  for (auto& x : th) x.join();
  return dev.out.load();
}

bool ctl_zero(const Device& dev) {
  for (int i = 0; i < kWords; ++i)
    if (dev.ctl[i] != 0u || dev.l2b[i] != 0u) return false;
  return true;
}

int fails = 0;
void check(bool ok, const char* what, const Scenario& sc) {
  std::printf("%-4s %-44s %s\n", ok ? "ok" : "FAIL", sc.name, what);
  if (!ok) ++fails;
}

}  // namespace

int main() {
  auto dev = std::make_unique<Device>();
  std::memset(dev->ctl, 0, sizeof(dev->ctl));
  std::memset(dev->l2b, 0, sizeof(dev->l2b));
  const uint32_t kLong = 1u << 22;      // never runs out in a normal call
  const uint32_t kShort = 2000;         // runs out while a member is missing
  for (bool xl : {true, false}) {
    for (int W : {4, 28}) {
      Scenario sc{xl ? "XCD-local, normal" : "device-wide, normal", xl, W, 2, kLong, 0, -1};
      for (int rep = 0; rep < 2; ++rep) {          // two calls in a row on the same words
        const float o = call(*dev, sc);
        check(o == W * (W + 1) / 2.f, "merged output", sc);
        check(dev->ctl[1] == 0u, "error word 0", sc);
        check(ctl_zero(*dev), "control words left zero", sc);
      }
    }
  }
  {
    Scenario sc{"XCD-local, members on two XCDs, one L2", true, 8, 2, kLong, 1, -1};
    const float o = call(*dev, sc);
    check(std::isnan(o), "NaN output", sc);
    check((dev->ctl[1] & 2u) != 0u, "error bit 1 (split placement)", sc);
    check(dev->ctl[2] == 0u && dev->ctl[16] == 0u, "arrival and mask words reset", sc);
    dev->ctl[1] = 0u;                               // the caller clears the error word
  }
  {
    Scenario sc{"XCD-local, members on two XCDs, two L2s", true, 8, 2, kShort, 2, -1};
    const float o = call(*dev, sc);
    check(std::isnan(o), "NaN output (every wait runs out)", sc);
    check((dev->ctl[1] & 1u) != 0u, "error bit 0 (timed out)", sc);
    std::memset(dev->ctl, 0, sizeof(dev->ctl));     // the caller re-zeroes the block
    std::memset(dev->l2b, 0, sizeof(dev->l2b));
  }
  for (bool xl : {true, false}) {
    Scenario sc{xl ? "XCD-local, straggler after the others ran out"
                   : "device-wide, straggler after the others ran out",
                xl, 8, 2, kShort, 0, 5};
    const float o = call(*dev, sc);
    check(std::isnan(o), "NaN output", sc);
    check((dev->ctl[1] & 1u) != 0u, "error bit 0 (timed out)", sc);
    std::memset(dev->ctl, 0, sizeof(dev->ctl));     // the caller re-zeroes the block
    std::memset(dev->l2b, 0, sizeof(dev->l2b));
    Scenario ok{xl ? "XCD-local, normal after re-zeroing" : "device-wide, normal after re-zeroing",
                xl, 8, 2, kLong, 0, -1};
    const float o2 = call(*dev, ok);
    check(o2 == 36.f && dev->ctl[1] == 0u && ctl_zero(*dev), "merged output, words zero", ok);
  }
  std::printf("%d failed\n", fails);
  return fails != 0;
}
