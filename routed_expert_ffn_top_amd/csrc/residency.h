// Residency table of the slot arena (EStream, section 3.3, "Bounded
// Parameter Arena and Safe Slot Reuse"), independent of the GPU runtime.
//
// A slot is Available, Filling (reserved for an expert whose slices are being
// written; in no placement map), Ready (published) or In-use (named by a
// submitted invocation). The pages' two guarantees -- no expert executes
// before its parameters are ready, and no slot is overwritten while a queued
// invocation still references it -- are carried by stream-ordered events
// instead of host waits:
//   ready[s]   recorded on the loading stream after slot s's slices are
//              written; every invocation that reads s makes its stream wait
//              for it first (acquire);
//   release    each invocation records one event of a ring on its stream
//              after its work (release_after), and remembers it per slot; a
//              later load into the slot makes the loading stream wait for it
//              (load).
// The ring has kRing entries; before an entry is recorded again the host
// waits for its previous record (then kRing invocations old) and forgets
// the slots that pointed at it.
//
// The backend supplies streams, events and their operations:
//   typename Bk::Stream, typename Bk::Event
//   int create(Event *), void destroy(Event), int record(Event, Stream),
//   int wait(Stream, Event), int sync(Event)       (0 = success)
// The library instantiates it with HIP streams and events; a host-only test
// instantiates it with worker threads that play the streams.
#pragma once

#include <stdint.h>
#include <stdio.h>

#include <vector>

#include "moe.h"

namespace moe {

template <class Bk>
class ResidencyTable {
public:
    using Stream = typename Bk::Stream;
    using Event = typename Bk::Event;
    static constexpr int kRing = 32;

    ResidencyTable(Bk &bk, int P, int n_exp)
        : bk_(bk), P_(P), ne_(n_exp), state_(P, MOE_SLOT_AVAILABLE), owner_(P, -1), ready_(P, Event()),
          ready_gen_(P, 0), waited_stream_(P, Stream()), waited_gen_(P, 0), ring_(kRing, Event()),
          ring_set_(kRing, 0), last_use_(P, -1), has_ready_(P, 0)
    {
    }
    ~ResidencyTable()
    {
        for (int s = 0; s < P_; ++s)
            if (has_ready_[s]) bk_.destroy(ready_[s]);
        for (int i = 0; i < kRing; ++i)
            if (ring_set_[i]) bk_.destroy(ring_[i]);
    }
    ResidencyTable(const ResidencyTable &) = delete;
    ResidencyTable &operator=(const ResidencyTable &) = delete;

    int P() const { return P_; }
    int n_exp() const { return ne_; }
    int state(int s) const { return state_[s]; }
    int owner(int s) const { return owner_[s]; }
    const char *msg() const { return msg_; }
    void clear_msg() { msg_[0] = 0; }

    // Available/Ready/In-use -> Filling for (slot, expert): the slot's old
    // mapping is withdrawn. Refused for a Filling slot or an expert that holds
    // or fills another slot.
    moe_status reserve(int slot, int expert)
    {
        if (slot < 0 || slot >= P_) return err(MOE_ERR_INVALID_ARG, "slot %d outside [0, P)", slot);
        if (expert < 0 || expert >= ne_) return err(MOE_ERR_INVALID_ARG, "expert %d outside [0, %d)", expert, ne_);
        if (state_[slot] == MOE_SLOT_FILLING) return err(MOE_ERR_SLOT_STATE, "slot %d is Filling", slot);
        for (int s2 = 0; s2 < P_; ++s2)
            if (s2 != slot && owner_[s2] == expert)
                return err(MOE_ERR_SLOT_STATE, "expert %d already occupies slot %d", expert, s2);
        owner_[slot] = expert;
        state_[slot] = MOE_SLOT_FILLING;
        return MOE_OK;
    }

    // A Filling slot whose load did not happen: back to Available.
    void abort_fill(int slot)
    {
        owner_[slot] = -1;
        state_[slot] = MOE_SLOT_AVAILABLE;
    }

    // Loads experts ex[i] into slots sl[i], i < n, on stream st: every slot is
    // reserved (Filling), st waits for each slot's last release, write(st)
    // enqueues the slices' writes, each slot's ready event is recorded on st
    // and the slot is published (Ready). On failure the slots reserved here
    // return to Available and nothing is published.
    template <class Write>
    moe_status load(const int *sl, const int *ex, int n, Stream st, Write write)
    {
        int reserved = 0;
        moe_status rc = MOE_OK;
        while (reserved < n && rc == MOE_OK) {
            rc = reserve(sl[reserved], ex[reserved]);
            if (rc == MOE_OK) ++reserved;
        }
        if (rc == MOE_OK) rc = ensure_ring();
        for (int i = 0; i < n && rc == MOE_OK; ++i) rc = ensure_ready_event(sl[i]);
        for (int i = 0; i < n && rc == MOE_OK; ++i)
            if (last_use_[sl[i]] >= 0 && bk_.wait(st, ring_[last_use_[sl[i]]]))
                rc = err(MOE_ERR_HIP, "wait for slot %d's release", sl[i]);
        if (rc == MOE_OK) rc = write(st);
        for (int i = 0; i < n && rc == MOE_OK; ++i)
            if (bk_.record(ready_[sl[i]], st)) rc = err(MOE_ERR_HIP, "record slot %d's ready event", sl[i]);
        if (rc != MOE_OK) {
            for (int i = 0; i < reserved; ++i)
                if (state_[sl[i]] == MOE_SLOT_FILLING) abort_fill(sl[i]);
            return rc;
        }
        for (int i = 0; i < n; ++i) publish_recorded(sl[i]);
        return MOE_OK;
    }

    // Publishes a slot whose slices the caller wrote on `st`: a slot Filling
    // for `expert` is published as it stands, any other slot is reserved
    // first. The ready event is recorded on st.
    moe_status publish(int slot, int expert, Stream st)
    {
        if (slot < 0 || slot >= P_) return err(MOE_ERR_INVALID_ARG, "slot %d outside [0, P)", slot);
        if (!(state_[slot] == MOE_SLOT_FILLING && owner_[slot] == expert)) {
            const moe_status rc = reserve(slot, expert);
            if (rc != MOE_OK) return rc;
        }
        moe_status rc = ensure_ring();
        if (rc == MOE_OK) rc = ensure_ready_event(slot);
        if (rc == MOE_OK && bk_.record(ready_[slot], st)) rc = err(MOE_ERR_HIP, "record slot %d's ready event", slot);
        if (rc != MOE_OK) {
            abort_fill(slot);
            return rc;
        }
        publish_recorded(slot);
        return MOE_OK;
    }

    // Every slot phi names must be Ready or In-use with that expert; st then
    // waits for each such slot's ready event (once per stream and load).
    moe_status acquire(const int32_t *phi, Stream st)
    {
        for (int e = 0; e < ne_; ++e) {
            const int s = phi[e];
            if (s < 0) continue;
            if (s >= P_ || (state_[s] != MOE_SLOT_READY && state_[s] != MOE_SLOT_IN_USE) || owner_[s] != e)
                return err(MOE_ERR_SLOT_STATE, "phi maps expert %d to slot %d, which is not Ready with it", e, s);
        }
        for (int e = 0; e < ne_; ++e) {
            const int s = phi[e];
            if (s < 0 || (waited_stream_[s] == st && waited_gen_[s] == ready_gen_[s])) continue;
            if (bk_.wait(st, ready_[s])) return err(MOE_ERR_HIP, "wait for slot %d's ready event", s);
            waited_stream_[s] = st;
            waited_gen_[s] = ready_gen_[s];
        }
        return MOE_OK;
    }

    // After an invocation's work on st: record a release event and mark the
    // slots phi names In-use with it as their last use. The ring's events are
    // created by the first load or publication, so an invocation (whose slots
    // must have been loaded) creates none.
    moe_status release_after(const int32_t *phi, Stream st)
    {
        const int pos = ring_pos_;
        if (!ring_set_[pos]) {
            if (bk_.create(&ring_[pos])) return err(MOE_ERR_HIP, "create a release event");
            ring_set_[pos] = 1;
        } else {
            if (bk_.sync(ring_[pos])) return err(MOE_ERR_HIP, "wait for an old release event");
            for (int s = 0; s < P_; ++s)
                if (last_use_[s] == pos) last_use_[s] = -1;
        }
        if (bk_.record(ring_[pos], st)) return err(MOE_ERR_HIP, "record a release event");
        ring_pos_ = (pos + 1) % kRing;
        for (int e = 0; e < ne_; ++e) {
            const int s = phi[e];
            if (s < 0) continue;
            last_use_[s] = pos;
            state_[s] = MOE_SLOT_IN_USE;
        }
        return MOE_OK;
    }

    // Withdraws a slot's mapping (Ready or In-use -> Available). A later load
    // into it still waits for its last release.
    moe_status release(int slot)
    {
        if (slot < 0 || slot >= P_) return err(MOE_ERR_INVALID_ARG, "slot %d outside [0, P)", slot);
        if (state_[slot] == MOE_SLOT_FILLING) return err(MOE_ERR_SLOT_STATE, "slot %d is Filling", slot);
        owner_[slot] = -1;
        state_[slot] = MOE_SLOT_AVAILABLE;
        return MOE_OK;
    }

    // Every slot Available (a new layer's mapping starts empty); loads into
    // them still wait for their last releases.
    void forget_mapping()
    {
        for (int s = 0; s < P_; ++s) {
            owner_[s] = -1;
            state_[s] = MOE_SLOT_AVAILABLE;
        }
    }

    // phi[e] = slot of expert e over Ready and In-use slots, else -1 (e < n).
    void placement(int32_t *phi, int n) const
    {
        for (int e = 0; e < n; ++e) phi[e] = -1;
        for (int s = 0; s < P_; ++s)
            if (state_[s] == MOE_SLOT_READY || state_[s] == MOE_SLOT_IN_USE) phi[owner_[s]] = s;
    }

private:
    moe_status ensure_ring()
    {
        for (int i = 0; i < kRing; ++i) {
            if (ring_set_[i]) continue;
            if (bk_.create(&ring_[i])) return err(MOE_ERR_HIP, "create a release event");
            ring_set_[i] = 1;
        }
        return MOE_OK;
    }
    moe_status ensure_ready_event(int slot)
    {
        if (has_ready_[slot]) return MOE_OK;
        if (bk_.create(&ready_[slot])) return err(MOE_ERR_HIP, "create slot %d's ready event", slot);
        has_ready_[slot] = 1;
        return MOE_OK;
    }
    void publish_recorded(int slot)
    {
        ready_gen_[slot] += 1;
        state_[slot] = MOE_SLOT_READY;
    }
    moe_status err(moe_status st, const char *m)
    {
        snprintf(msg_, sizeof msg_, "%s", m);
        return st;
    }
    template <class A0, class... A>
    moe_status err(moe_status st, const char *fmt, A0 a0, A... args)
    {
        snprintf(msg_, sizeof msg_, fmt, a0, args...);
        return st;
    }

    Bk &bk_;
    int P_, ne_;
    std::vector<int> state_, owner_;
    std::vector<Event> ready_;
    std::vector<uint64_t> ready_gen_;
    std::vector<Stream> waited_stream_;
    std::vector<uint64_t> waited_gen_;
    std::vector<Event> ring_;
    std::vector<char> ring_set_;
    int ring_pos_ = 0;
    std::vector<int> last_use_;   // per slot: ring entry of its last use, or -1
    std::vector<char> has_ready_;
    char msg_[256] = {0};
};

}  // namespace moe
