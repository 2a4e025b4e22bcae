// Hand-out order of the work-queue cursor slots of a plan.  Pure host logic
// (no HIP calls), so it is testable on its own.
//
// A persistent attention launch needs a zeroed cursor slot for the time it
// runs; the last of its workgroups clears the slot again.  Launches take the
// plan's slots round-robin.  A slot handed out before belongs to a launch
// that may still be running (on another stream), so the launcher makes the
// new launch wait for the event recorded after that launch: take() reports
// whether that is needed.  Callers serialise take() and the event record
// that follows it (the plan's launch mutex), so a reused slot's event is
// always the one of its previous user.
#pragma once

#include <cstdint>

namespace ug {

template <int kSlots>
class SlotRing {
 public:
  struct Ticket {
    int slot;     // cursor slot index, 0 .. kSlots-1
    bool reused;  // an earlier launch used this slot: wait for its event first
  };
  Ticket take() {
    const int s = int(next_ % uint64_t(kSlots));
    const bool r = next_ >= uint64_t(kSlots);
    ++next_;
    return {s, r};
  }
  uint64_t handed_out() const { return next_; }

 private:
  uint64_t next_ = 0;
};

}  // namespace ug
