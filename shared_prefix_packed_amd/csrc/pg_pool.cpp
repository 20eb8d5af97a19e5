// Reusable upload buffers for layouts: each slot pairs a pinned host staging
// area with a device buffer of the same capacity. A layout takes a slot at
// upload and gives it back at destroy; the slot becomes reusable once the
// work enqueued on every stream that used the layout has completed (one
// event per stream, polled with hipEventQuery). Neither step waits for the
// device, so a caller that builds a new layout per batch overlaps the host
// build of batch i+1 with the kernels of batch i.
//
// Slots are kept for the life of the process (they are small: the per-token
// descriptors and the work list of one batch).
//
// Graph capture: an event recorded on a capturing stream becomes a node of
// the graph and says nothing about when the graph's replays read the slot, and
// a captured upload copy re-reads the pinned staging area on every replay. A
// slot touched while a stream is capturing is therefore marked captured and
// is never handed out again, so a graph stays valid after the layout it was
// captured with is destroyed (the slot's memory is held until the process
// ends).
#include <mutex>
#include <vector>

#include "pg_internal.h"

namespace {

struct Cache {
  std::mutex mu;
  std::vector<pg_slot*> slots;   // every slot ever made, in or out of use
};

Cache& cache() {
  static Cache* c = new Cache();   // never destroyed: the HIP runtime may be gone at exit
  return *c;
}

size_t round_capacity(size_t bytes) {
  size_t cap = size_t(64) << 10;
  while (cap < bytes) cap += cap / 2;
  return (cap + 255) / 256 * 256;
}

// True when the last work enqueued with the slot on each stream has completed.
bool slot_idle(pg_slot* s) {
  for (int i = 0; i < s->nev; ++i) {
    hipError_t e = hipEventQuery(s->ev[i]);
    if (e == hipErrorNotReady) return false;
    if (e != hipSuccess) {
      (void)hipGetLastError();
      (void)hipEventSynchronize(s->ev[i]);
    }
  }
  s->nev = 0;
  return true;
}

void free_slot_memory(pg_slot* s) {
  if (s->dev) (void)hipFree(s->dev);
  if (s->host) (void)hipHostFree(s->host);
  s->dev = nullptr;
  s->host = nullptr;
  s->cap = 0;
}

}  // namespace

pg_status pg_slot_acquire(int device, size_t bytes, pg_slot** out) {
  *out = nullptr;
  Cache& c = cache();
  std::lock_guard<std::mutex> lock(c.mu);
  pg_slot* best = nullptr;
  pg_slot* spare = nullptr;   // an idle slot that is too small
  for (pg_slot* s : c.slots) {
    if (s->in_use || s->device != device || !slot_idle(s)) continue;
    if (s->cap >= bytes) {
      if (!best || s->cap < best->cap) best = s;
    } else if (!spare) {
      spare = s;
    }
  }
  if (!best) {
    best = spare;
    if (!best) {
      best = new (std::nothrow) pg_slot();
      if (!best) return pg_fail(PG_ERR_OOM, "host allocation failed");
      best->device = device;
      c.slots.push_back(best);
    }
    free_slot_memory(best);
    const size_t cap = round_capacity(bytes);
    hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&best->host), cap, hipHostMallocDefault);
    if (e == hipSuccess) e = hipMalloc(&best->dev, cap);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      free_slot_memory(best);
      return e == hipErrorOutOfMemory
                 ? pg_fail(PG_ERR_OOM, "upload buffer of %zu bytes: out of memory", cap)
                 : pg_fail(PG_ERR_HIP, "upload buffer allocation: %s", hipGetErrorString(e));
    }
    best->cap = cap;
  }
  best->in_use = true;
  *out = best;
  return PG_OK;
}

// True unless `stream` is known not to be capturing (an error counts as
// capturing: the slot is then kept, which is always safe).
bool stream_capturing(hipStream_t stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &st) != hipSuccess) {
    (void)hipGetLastError();
    return true;
  }
  return st != hipStreamCaptureStatusNone;
}

void pg_slot_note_use(pg_slot* s, hipStream_t stream) {
  if (!s) return;
  std::lock_guard<std::mutex> lock(s->mu);
  if (stream_capturing(stream)) {
    s->captured = true;
    return;
  }
  int i = 0;
  while (i < s->nev && s->stream[i] != stream) ++i;
  if (i == kSlotEvents) {
    s->overflow = true;   // too many streams: release waits for the device
    return;
  }
  if (!s->ev[i] && hipEventCreateWithFlags(&s->ev[i], hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    s->ev[i] = nullptr;
    s->overflow = true;
    return;
  }
  if (hipEventRecord(s->ev[i], stream) != hipSuccess) {
    (void)hipGetLastError();
    s->overflow = true;
    return;
  }
  s->stream[i] = stream;
  if (i == s->nev) s->nev = i + 1;
}

void pg_slot_release(pg_slot* s) {
  if (!s) return;
  {
    std::lock_guard<std::mutex> lock(s->mu);
    if (s->captured) return;   // a captured graph may still read it: never reused
  }
  if (s->overflow) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != s->device) (void)hipSetDevice(s->device);
    (void)hipDeviceSynchronize();
    if (cur != s->device && cur >= 0) (void)hipSetDevice(cur);
    s->nev = 0;
    s->overflow = false;
  }
  Cache& c = cache();
  std::lock_guard<std::mutex> lock(c.mu);
  s->in_use = false;
}
