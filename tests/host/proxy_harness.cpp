// Host-only harness for arx::Proxy (no GPU, no HIP): a fake device thread
// plays the GPU side of the protocol against ordinary memory. Each scenario
// prints "ok <name>" or "FAIL <name>: why" and the process exits non-zero on
// any failure. Built with g++ by tests/test_proxy_host.py, also under
// ThreadSanitizer.
#include <atomic>
#include <chrono>
#include <cstdio>
#include <string>
#include <thread>
#include <vector>

#include "arx_proxy.h"

using namespace std::chrono_literals;

static int failures = 0;
#define CHECK(cond, name, ...)                         \
  do {                                                 \
    if (!(cond)) {                                     \
      printf("FAIL %s: ", name);                       \
      printf(__VA_ARGS__);                             \
      printf("\n");                                    \
      ++failures;                                      \
      return;                                          \
    }                                                  \
  } while (0)

struct Words {
  alignas(64) uint64_t pub = 0;
  alignas(64) uint64_t done = 0;
  alignas(64) uint64_t flags[8] = {};
};

static uint64_t ld(const uint64_t* p) { return __atomic_load_n(p, __ATOMIC_ACQUIRE); }
static void st(uint64_t* p, uint64_t v) { __atomic_store_n(p, v, __ATOMIC_RELEASE); }

// The device side of K calls: publish s, wait for every peer flag to reach
// s, check the flags never ran more than the mode allows ahead, finish s.
static bool fake_gpu(Words& w, int world, int rank, uint64_t K, uint64_t lead, std::string& why) {
  for (uint64_t s = 1; s <= K; ++s) {
    st(&w.pub, s);
    const auto t0 = std::chrono::steady_clock::now();
    for (int j = 0; j < world; ++j) {
      if (j == rank) continue;
      while (ld(&w.flags[j]) < s) {
        if (std::chrono::steady_clock::now() - t0 > 5s) { why = "flag never came for seq " + std::to_string(s); return false; }
      }
      if (ld(&w.flags[j]) > s + lead) { why = "flag ran ahead at seq " + std::to_string(s); return false; }
    }
    st(&w.done, s);
  }
  return true;
}

static void scenario_mode(const char* name, int mode, uint64_t lead) {
  for (int world : {2, 3, 8}) {
    const int rank = world - 1;
    Words w;
    arx::Proxy p(&w.pub, &w.done, w.flags, world, rank);
    p.mode = mode;
    std::vector<uint64_t> seen;
    std::atomic<bool> stop{false};
    std::thread t([&] { p.run(stop); });
    std::string why;
    const uint64_t K = 20000;
    const bool ok = fake_gpu(w, world, rank, K, lead, why);
    // run-ahead posts K + 1 after seeing K published: let it finish first
    const auto t0 = std::chrono::steady_clock::now();
    while (p.posted() < K + lead && std::chrono::steady_clock::now() - t0 < 5s) {}
    stop = true;
    t.join();
    CHECK(ok, name, "world %d: %s", world, why.c_str());
    CHECK(p.posted() == K + lead, name, "posted %llu, want %llu", (unsigned long long)p.posted(),
          (unsigned long long)(K + lead));
    for (int j = 0; j < world; ++j) {
      const uint64_t want = j == rank ? 0 : K + lead;
      CHECK(w.flags[j] == want, name, "flag %d = %llu, want %llu", j, (unsigned long long)w.flags[j],
            (unsigned long long)want);
    }
  }
  printf("ok %s\n", name);
}

static void scenario_manual() {
  const char* name = "manual";
  Words w;
  arx::Proxy p(&w.pub, &w.done, w.flags, 4, 0);
  p.mode = arx::PROXY_MANUAL;
  std::atomic<bool> stop{false};
  std::thread t([&] { p.run(stop); });
  st(&w.pub, 3);
  std::this_thread::sleep_for(20ms);
  CHECK(p.posted() == 0 && ld(&w.flags[1]) == 0, name, "manual mode posted on its own");
  CHECK(!p.publish(2), name, "publish(2) before 1 accepted");
  CHECK(ld(&w.flags[1]) == 0, name, "refused publish wrote a flag");
  CHECK(p.publish(1) && p.publish(2), name, "in-order publish refused");
  CHECK(!p.publish(2), name, "repeated publish accepted");
  CHECK(ld(&w.flags[0]) == 0 && ld(&w.flags[3]) == 2, name, "flags %llu %llu", (unsigned long long)w.flags[0],
        (unsigned long long)w.flags[3]);
  stop = true;
  t.join();
  printf("ok %s\n", name);
}

// Lockstep never posts a seq before it is published; a switch to run-ahead
// posts exactly one more.
static void scenario_no_skip_no_lead() {
  const char* name = "no_skip_no_lead";
  Words w;
  arx::Proxy p(&w.pub, &w.done, w.flags, 2, 0);
  for (uint64_t s = 1; s <= 50; ++s) {
    p.step();
    CHECK(p.posted() == s - 1, name, "posted %llu before seq %llu was published", (unsigned long long)p.posted(),
          (unsigned long long)s);
    st(&w.pub, s);
    p.step();
    CHECK(p.posted() == s, name, "seq %llu not posted", (unsigned long long)s);
  }
  p.mode = arx::PROXY_RUNAHEAD;
  p.step();
  p.step();
  CHECK(p.posted() == 51, name, "run-ahead posted %llu", (unsigned long long)p.posted());
  printf("ok %s\n", name);
}

// The watchdog, on a fake clock: one report per stall, re-armed by progress.
static void scenario_watchdog() {
  const char* name = "watchdog";
  Words w;
  arx::Proxy p(&w.pub, &w.done, w.flags, 3, 0);
  p.mode = arx::PROXY_MANUAL;
  auto t = arx::Proxy::Clock::time_point{};
  p.now = [&] { return t; };
  std::vector<std::string> reports;
  p.report = [&](const std::string& s) { reports.push_back(s); };
  st(&w.pub, 5);
  st(&w.done, 3);
  p.publish(1);
  p.step();                          // arms
  t += std::chrono::milliseconds(1500);
  p.step();
  CHECK(reports.empty(), name, "reported before 2 s");
  t += std::chrono::milliseconds(600);
  p.step();
  CHECK(reports.size() == 1, name, "%zu reports after 2.1 s", reports.size());
  CHECK(reports[0].find("STALL: published 5 posted 1 done 3") != std::string::npos, name, "%s", reports[0].c_str());
  CHECK(reports[0].find("r1=1 r2=1") != std::string::npos, name, "%s", reports[0].c_str());
  t += std::chrono::seconds(10);
  p.step();
  CHECK(reports.size() == 1, name, "reported twice for one stall");
  st(&w.done, 4);                    // progress re-arms
  p.step();
  t += std::chrono::seconds(3);
  p.step();
  CHECK(reports.size() == 2 && p.stalls == 2, name, "%zu reports after a second stall", reports.size());
  st(&w.done, 5);                    // caught up: no stall however long
  p.step();
  t += std::chrono::seconds(100);
  p.step();
  CHECK(reports.size() == 2, name, "reported while idle and caught up");
  printf("ok %s\n", name);
}

// A publish racing the proxy thread in a posting mode is either the next
// seq (accepted) or refused; flags never go backwards or skip.
static void scenario_concurrent_publish() {
  const char* name = "concurrent_publish";
  Words w;
  arx::Proxy p(&w.pub, &w.done, w.flags, 2, 1);
  std::atomic<bool> stop{false};
  std::thread t([&] { p.run(stop); });
  uint64_t last = 0;
  for (uint64_t s = 1; s <= 5000; ++s) {
    st(&w.pub, s);
    p.publish(p.posted() + 1);       // may lose the race; either way stays in order
    const uint64_t f = ld(&w.flags[0]);
    CHECK(f >= last, name, "flag went backwards");
    last = f;
  }
  stop = true;
  t.join();
  CHECK(p.posted() >= 5000 && p.posted() <= 5001, name, "posted %llu", (unsigned long long)p.posted());
  printf("ok %s\n", name);
}

// Stress mode: the data for seq s is written before s is posted, so a
// device that sees flag s always finds data s.
static void scenario_stress() {
  const char* name = "stress";
  Words w;
  uint64_t data = 0;
  arx::Proxy p(&w.pub, &w.done, w.flags, 4, 0);
  p.before_post = [&](uint64_t s) { __atomic_store_n(&data, s, __ATOMIC_RELEASE); return true; };
  p.mode = arx::PROXY_STRESS;
  std::atomic<bool> stop{false};
  std::thread t([&] { p.run(stop); });
  bool ok = true;
  for (uint64_t s = 1; s <= 20000 && ok; ++s) {
    st(&w.pub, s);
    while (ld(&w.flags[2]) < s) {}
    ok = ld(&data) >= s;
    st(&w.done, s);
  }
  stop = true;
  t.join();
  CHECK(ok, name, "a flag was seen before its data");
  arx::Proxy q(&w.pub, &w.done, w.flags, 4, 0);
  q.before_post = [](uint64_t) { return false; };
  q.mode = arx::PROXY_STRESS;
  CHECK(!q.step(), name, "a failed data copy did not fail the post");
  printf("ok %s\n", name);
}

// Leaving stress mode, then swapping the data source under locked(): once
// locked() has returned, no data copy may run on the old source, nor start
// at all, since the mode has left stress mode. Each round publishes new
// seqs while holding the proxy's lock and waits, so the proxy has read the
// new target (and the mode, still stress) and blocks on the lock; the mode
// then leaves stress mode and the source is retired before the lock is
// released. A proxy that copied data on the mode it read before taking the
// lock would run the copy on the retired source.
static void scenario_stress_switch() {
  const char* name = "stress_switch";
  struct Source {
    bool valid;
  };
  Source good{true}, retired{false};
  const Source* source = &good;  // read by before_post, replaced under locked()
  int bad = 0;                   // written by before_post, under the lock
  Words w;
  arx::Proxy p(&w.pub, &w.done, w.flags, 4, 0);
  p.before_post = [&](uint64_t) {
    if (!source->valid) ++bad;
    return true;
  };
  std::atomic<bool> stop{false};
  std::thread t([&] { p.run(stop); });
  uint64_t s = 0;
  bool ok = true;
  auto wait_flags = [&](uint64_t target) {
    const auto t0 = std::chrono::steady_clock::now();
    while (ld(&w.flags[1]) < target)
      if (std::chrono::steady_clock::now() - t0 > 5s) return false;
    return true;
  };
  for (int round = 0; round < 100 && ok; ++round) {
    p.locked([&] { good.valid = true; source = &good; });
    p.mode = arx::PROXY_STRESS;
    s += 2;
    st(&w.pub, s);  // two posts in stress mode, with their copies
    ok = wait_flags(s);
    p.locked([&] {
      s += 2;
      st(&w.pub, s);
      std::this_thread::sleep_for(std::chrono::microseconds(300));
      p.mode = arx::PROXY_LOCKSTEP;
      good.valid = false;
      source = &retired;
    });
    ok = ok && wait_flags(s);
    st(&w.done, s);
  }
  stop = true;
  t.join();
  CHECK(ok, name, "the proxy stopped posting");
  int nbad = 0;
  p.locked([&] { nbad = bad; });
  CHECK(nbad == 0, name, "%d data copies ran on a retired source", nbad);
  printf("ok %s\n", name);
}

int main() {
  scenario_mode("lockstep", arx::PROXY_LOCKSTEP, 0);
  scenario_mode("runahead", arx::PROXY_RUNAHEAD, 1);
  scenario_manual();
  scenario_no_skip_no_lead();
  scenario_watchdog();
  scenario_concurrent_publish();
  scenario_stress();
  scenario_stress_switch();
  return failures ? 1 : 0;
}
