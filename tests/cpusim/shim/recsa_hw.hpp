// Host versions of the three hardware operations of recsa_hw.hpp (this
// directory precedes the library's sources on the include path): the L1
// invalidation is a full fence, the XCD id is the emulated workgroup's
// (set by the harness), and a pause yields the host thread.
#pragma once

#include <atomic>
#include <thread>

namespace recsa {

inline thread_local int sim_xcc = 0;

inline void l1_invalidate() { std::atomic_thread_fence(std::memory_order_seq_cst); }
inline int xcc_id() { return sim_xcc; }
inline void spin_pause() { std::this_thread::yield(); }

}  // namespace recsa
