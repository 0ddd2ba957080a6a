// arx_proxy.h — the host proxy that posts the virtual peers' flags, and its
// stall watchdog. Plain C++ (no HIP): it only reads and writes host-visible
// words, so the same code runs against the pinned control block in libarx
// and against ordinary memory in host-only tests.
//
// Page "arx.cu", proxy_loop: the proxy watches the seq this rank published
// and posts the seqs one after another, never skipping one (a skipped seq would let
// a peer accept a later flag over stale data); between posts it is the
// watchdog, which reports once when published work has not finished for
// 2 s, with what this rank posted and each peer's flag.
#pragma once

#include <atomic>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <functional>
#include <mutex>
#include <string>

namespace arx {

enum : int { PROXY_LOCKSTEP = 0, PROXY_RUNAHEAD = 1, PROXY_MANUAL = 2, PROXY_STRESS = 3 };

class Proxy {
 public:
  using Clock = std::chrono::steady_clock;

  // pub: the seq this rank published (written by the device); done: the
  // last seq whose reduction finished; flags: one u64 per rank, the virtual
  // peers' flags this proxy posts (the entry at `rank` is never written).
  Proxy(const uint64_t* pub, const uint64_t* done, uint64_t* flags, int world, int rank)
      : pub_(pub), done_(done), flags_(flags), world_(world), rank_(rank) {}

  std::atomic<int> mode{PROXY_LOCKSTEP};
  std::atomic<uint64_t> stalls{0};
  std::function<Clock::time_point()> now = [] { return Clock::now(); };
  std::function<void(const std::string&)> report = [](const std::string& s) { fprintf(stderr, "%s\n", s.c_str()); };
  std::chrono::milliseconds stall_after{2000};
  // Called before seq s is posted in PROXY_STRESS mode, to put the peers'
  // data for s in place (the data then precedes its flag); false fails the
  // post.
  std::function<bool(uint64_t)> before_post;

  uint64_t posted() const { return posted_.load(std::memory_order_acquire); }

  // The peers publish seq s: flags[src] = s (store-release) for every
  // src != rank. s must be posted() + 1; returns false (and writes
  // nothing) otherwise.
  bool publish(uint64_t s) {
    std::lock_guard<std::mutex> g(mu_);
    return publish_locked(s);
  }

  // Runs f while no post is in progress (posts hold the same lock), e.g. to
  // replace what before_post reads.
  template <typename F>
  void locked(F&& f) {
    std::lock_guard<std::mutex> g(mu_);
    f();
  }

  // Sets the posted seq and every peer flag to s, as if seqs 1..s had been
  // posted (state set-up for tests; no call may be in flight).
  void reset(uint64_t s) {
    std::lock_guard<std::mutex> g(mu_);
    for (int src = 0; src < world_; ++src)
      if (src != rank_) __atomic_store_n(&flags_[src], s, __ATOMIC_RELEASE);
    posted_.store(s, std::memory_order_release);
  }

  // One pass of the loop: post up to the seq the mode allows (in stress
  // mode each post is preceded by before_post; the mode is read again under
  // the lock for each post, so once the mode has left stress mode and a
  // locked() call has returned, before_post is not running and is not
  // called again), or else run the watchdog check. Returns false if posting failed: before_post failed, or an order
  // error, which cannot happen unless publish() was also called
  // concurrently in a posting mode.
  bool step() {
    const uint64_t pub = __atomic_load_n(pub_, __ATOMIC_ACQUIRE);
    const int m = mode.load(std::memory_order_acquire);
    const uint64_t have = posted();
    uint64_t target = have;
    if (m == PROXY_LOCKSTEP || m == PROXY_STRESS) target = pub;
    else if (m == PROXY_RUNAHEAD) target = pub + 1;
    if (target > have) {
      std::lock_guard<std::mutex> g(mu_);
      for (uint64_t s = posted() + 1; s <= target; ++s) {
        if (mode.load(std::memory_order_acquire) == PROXY_STRESS && before_post && !before_post(s)) return false;
        if (!publish_locked(s)) return false;
      }
      return true;
    }
    watchdog(pub, have);
    return true;
  }

  // Runs step() until `stop` becomes true; returns false on a posting error.
  bool run(const std::atomic<bool>& stop) {
    unsigned spin = 0;
    while (!stop.load(std::memory_order_acquire)) {
      if (!step()) return false;
      if ((++spin & 63u) == 0) cpu_relax();
    }
    return true;
  }

 private:
  static void cpu_relax() {
#if defined(__x86_64__)
    __builtin_ia32_pause();
#endif
  }

  bool publish_locked(uint64_t s) {
    if (s != posted() + 1) return false;
    for (int src = 0; src < world_; ++src)
      if (src != rank_) __atomic_store_n(&flags_[src], s, __ATOMIC_RELEASE);
    posted_.store(s, std::memory_order_release);
    return true;
  }

  // Work published but not finished, with no progress for stall_after, is
  // reported once; progress (done moving) or catching up re-arms it.
  void watchdog(uint64_t pub, uint64_t have) {
    const uint64_t done = __atomic_load_n(done_, __ATOMIC_ACQUIRE);
    const auto t = now();
    if (!armed_ || done != last_done_ || done >= pub) {
      armed_ = true;
      last_done_ = done;
      last_move_ = t;
      reported_ = false;
      return;
    }
    if (!reported_ && t - last_move_ > stall_after) {
      reported_ = true;
      stalls.fetch_add(1);
      std::string s = "arx rank " + std::to_string(rank_) + " STALL: published " + std::to_string(pub) + " posted " +
                      std::to_string(have) + " done " + std::to_string(done) + "; flags:";
      for (int j = 0; j < world_; ++j)
        if (j != rank_)
          s += " r" + std::to_string(j) + "=" + std::to_string(__atomic_load_n(&flags_[j], __ATOMIC_ACQUIRE));
      report(s);
    }
  }

  const uint64_t* pub_;
  const uint64_t* done_;
  uint64_t* flags_;
  int world_, rank_;
  std::atomic<uint64_t> posted_{0};
  std::mutex mu_;
  bool armed_ = false, reported_ = false;
  uint64_t last_done_ = 0;
  Clock::time_point last_move_{};
};

}  // namespace arx
