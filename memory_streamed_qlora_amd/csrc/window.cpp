// Host-to-device block-prefetch window (event-ordered slots of fixed layer positions).
//
// The pages' forward streams frozen blocks through a small GPU window with
// asynchronous prefetch on side streams; the backward walks the blocks in reverse and
// reloads each one; eviction is a pointer release because the base is read-only, so
// nothing is ever copied back ("Poros" research post, training-step paragraph;
// "Limitations", "Pretraining is out of scope").  Their block-size sweep (peak memory
// at block sizes 1..16, "Poros" research post, memory paragraph) grows by two
// blocks' worth per doubling, consistent with one window computing while the next
// one loads: at least two slots.  More slots let the copies run further ahead.
//
// Layout.  A slot holds one window of window_blocks layers.  Position q of every slot
// (the q-th layer of whichever window the slot holds) has one fixed byte range, as large
// as the largest layer any window puts at position q; so the ranges of different
// positions never overlap, whatever the layer sizes.
//
// Ordering is kept per (slot, position): the copy into a position waits on the
// position's "freed" event (recorded on the compute stream when the layer that held it
// was released) and on its previous "ready" event (the last copy into it, in case that
// copy ran on another copy stream), then records "ready" again after its copy; acquire
// makes the compute stream wait on the layer's own "ready".  Since a position's byte range
// belongs to it alone, these two waits are all a copy needs.  A window is still claimed
// and copied as one unit, but its layers are copied in the order the slot's previous
// layers were released (ascending after a forward, descending after a backward), so the
// first layer of the next window lands as soon as the first layer of the last one is
// done.  Layer l is copied on copy stream l % n_copy_streams: with two streams, one
// layer's copy can run while the next one waits for its position to be released.
//
// The host never blocks on the hot path: copy durations are read from their events only
// once the events have completed (polled without waiting), or when the statistics are
// asked for.  A prefetch of a window that a free slot still holds issues no copy (the
// windows in the slots at the end of the forward are the first the backward needs).
#include <string.h>

#include <algorithm>
#include <deque>
#include <vector>

#include "../../include/msq.h"
#include "internal.hpp"

using namespace msq;

namespace {
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

enum SlotState { SLOT_FREE = 0, SLOT_HELD = 1 };

struct TimingPair {
  hipEvent_t start = nullptr, end = nullptr;
};
}  // namespace

struct msq_window {
  int n_layers = 0, window_blocks = 0, n_windows = 0, n_slots = 0;
  std::vector<const void*> host;
  std::vector<size_t> bytes;
  std::vector<size_t> pos_off;  // byte offset of each position inside a slot
  size_t slot_bytes = 0;
  std::vector<char*> slot_base;
  std::vector<hipStream_t> copies;  // layer l is copied on copies[l % copies.size()]
  // per (slot, position) events, index slot * window_blocks + position
  std::vector<hipEvent_t> ready, freed;
  std::vector<char> ready_recorded, freed_recorded;
  std::vector<std::vector<int>> release_order;  // positions in the order they were released
  std::vector<std::vector<char>> released;      // per slot and position: released since claimed
  std::vector<int> slot_window;  // window whose bytes the slot holds (or will hold)
  std::vector<int> state;
  std::vector<uint64_t> release_tick;
  uint64_t tick = 0;
  msq_window_stats stats = {0, 0, 0, 0.0, 0, 0.0};
  // copy timing: a (start, end) event pair around each layer copy.  Pairs whose end has
  // completed are read without waiting (hipEventQuery) and recycled; a copy takes a recycled
  // pair or a new one.  Spans are measured from t_ref (recorded on copy stream 0 at creation
  // and again after each statistics call, which has waited for every copy) so that the busy
  // time can be the union of the spans of all copy streams.
  std::deque<TimingPair> pending;
  std::vector<TimingPair> spare;
  std::vector<hipEvent_t> all_timing_events;
  hipEvent_t t_ref = nullptr;
  std::vector<std::pair<double, double>> spans;
};

namespace {

// Per-position range sizes: position q is as large as the largest layer at position q of
// any window.
std::vector<size_t> position_sizes(const size_t* blob_bytes, int n_layers, int wb) {
  std::vector<size_t> s(wb, 0);
  for (int l = 0; l < n_layers; ++l) s[l % wb] = std::max(s[l % wb], align256(blob_bytes[l]));
  return s;
}

size_t slot_size(const size_t* blob_bytes, int n_layers, int wb) {
  size_t t = 0;
  for (size_t v : position_sizes(blob_bytes, n_layers, wb)) t += v;
  return t;
}

// Length of the union of the kept spans, which are then dropped; with `keep` > 0 the last
// `keep` merged spans stay (later copies may still overlap them).
double merge_spans(msq_window* w, size_t keep) {
  std::vector<std::pair<double, double>>& v = w->spans;
  std::sort(v.begin(), v.end());
  std::vector<std::pair<double, double>> m;
  for (const auto& s : v) {
    if (!m.empty() && s.first <= m.back().second)
      m.back().second = std::max(m.back().second, s.second);
    else
      m.push_back(s);
  }
  const size_t done = m.size() > keep ? m.size() - keep : 0;
  double total = 0.0;
  for (size_t i = 0; i < done; ++i) total += m[i].second - m[i].first;
  v.assign(m.begin() + done, m.end());
  return total;
}

// Adds a completed pair's duration and span to the statistics and recycles it.
hipError_t account(msq_window* w, const TimingPair& p) {
  float ms = 0.0f, t0 = 0.0f, t1 = 0.0f;
  hipError_t e = hipEventElapsedTime(&ms, p.start, p.end);
  if (e == hipSuccess) e = hipEventElapsedTime(&t0, w->t_ref, p.start);
  if (e == hipSuccess) e = hipEventElapsedTime(&t1, w->t_ref, p.end);
  if (e != hipSuccess) return e;
  w->stats.copy_ms += ms;
  w->stats.copies_timed++;
  w->spans.emplace_back(t0, t1);
  if (w->spans.size() > 4096) w->stats.busy_ms += merge_spans(w, 64);
  w->spare.push_back(p);
  return hipSuccess;
}

// Reads the pairs whose copies have completed, oldest first, without waiting; with `wait`,
// waits for all of them.
hipError_t harvest(msq_window* w, bool wait) {
  while (!w->pending.empty()) {
    const TimingPair p = w->pending.front();
    hipError_t e = wait ? hipEventSynchronize(p.end) : hipEventQuery(p.end);
    if (e == hipErrorNotReady) {
      (void)hipGetLastError();  // not an error: the copy is still running
      return hipSuccess;
    }
    if (e != hipSuccess) return e;
    w->pending.pop_front();
    e = account(w, p);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t take_pair(msq_window* w, TimingPair* out) {
  if (!w->spare.empty()) {
    *out = w->spare.back();
    w->spare.pop_back();
    return hipSuccess;
  }
  TimingPair p;
  hipError_t e = hipEventCreate(&p.start);
  if (e != hipSuccess) return e;
  w->all_timing_events.push_back(p.start);
  e = hipEventCreate(&p.end);
  if (e != hipSuccess) return e;
  w->all_timing_events.push_back(p.end);
  *out = p;
  return hipSuccess;
}

int find_slot(const msq_window* w, int win, int state) {
  for (int i = 0; i < w->n_slots; ++i)
    if (w->slot_window[i] == win && w->state[i] == state) return i;
  return -1;
}

void destroy_events(msq_window* w) {
  for (hipEvent_t e : w->ready)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : w->freed)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : w->all_timing_events)
    if (e) (void)hipEventDestroy(e);
  if (w->t_ref) (void)hipEventDestroy(w->t_ref);
}

// The blob must be pinned host memory over its whole range: the copies are asynchronous
// DMA reads of it.
int check_pinned(int l, const void* p, size_t n) {
  const char* ends[2] = {(const char*)p, (const char*)p + n - 1};
  for (const char* q : ends) {
    hipPointerAttribute_t a;
    memset(&a, 0, sizeof(a));
    const hipError_t e = hipPointerGetAttributes(&a, q);
    if (e == hipErrorInvalidValue || (e == hipSuccess && a.type != hipMemoryTypeHost)) {
      (void)hipGetLastError();
      return set_error(MSQ_E_INVAL,
                       "block_stream_create: layer %d's blob (%p, %zu bytes) is not pinned host memory "
                       "(hipHostMalloc or registered) over its whole range",
                       l, p, n);
    }
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return set_error(MSQ_E_HIP, "block_stream_create: cannot check that layer %d's blob is pinned host memory: %s (%d)",
                       l, hipGetErrorString(e), (int)e);
    }
  }
  return MSQ_OK;
}

}  // namespace

extern "C" {

size_t block_stream_arena_bytes(const size_t* blob_bytes, int n_layers, int window_blocks,
                                int n_slots) {
  if (!blob_bytes || n_layers <= 0 || window_blocks <= 0 || window_blocks > n_layers || n_slots < 2 ||
      n_slots > 1024)
    return 0;
  return (size_t)n_slots * slot_size(blob_bytes, n_layers, window_blocks);
}

int block_stream_create(msq_window** out, const void* const* host_blobs, const size_t* blob_bytes,
                        int n_layers, int window_blocks, int n_slots, void* dev_arena,
                        size_t arena_bytes, const msq_stream_t* copy_streams, int n_copy_streams) {
  if (!out || !host_blobs || !blob_bytes || !dev_arena || !copy_streams)
    return set_error(MSQ_E_INVAL, "block_stream_create: null pointer");
  *out = nullptr;
  if (n_copy_streams < 1 || n_copy_streams > MSQ_MAX_COPY_STREAMS)
    return set_error(MSQ_E_INVAL, "block_stream_create: n_copy_streams=%d outside [1, %d]", n_copy_streams,
                     MSQ_MAX_COPY_STREAMS);
  if (n_layers <= 0 || window_blocks <= 0 || window_blocks > n_layers || n_slots < 2 || n_slots > 1024)
    return set_error(MSQ_E_INVAL, "block_stream_create: n_layers=%d window_blocks=%d n_slots=%d", n_layers,
                     window_blocks, n_slots);
  if ((uintptr_t)dev_arena % 256)
    return set_error(MSQ_E_INVAL, "block_stream_create: arena must be 256-byte aligned");
  for (int l = 0; l < n_layers; ++l)
    if (!host_blobs[l] || blob_bytes[l] == 0)
      return set_error(MSQ_E_INVAL, "block_stream_create: layer %d has no host blob", l);
  const size_t need = (size_t)n_slots * slot_size(blob_bytes, n_layers, window_blocks);
  if (arena_bytes < need) {
    int fit = 0;
    for (int wb = window_blocks - 1; wb >= 1; --wb)
      if ((size_t)n_slots * slot_size(blob_bytes, n_layers, wb) <= arena_bytes) {
        fit = wb;
        break;
      }
    if (fit > 0)
      return set_error(MSQ_E_WINDOW, "block_stream_create: arena %zu bytes < %zu needed for window_blocks=%d; largest window that fits: window_blocks=%d",
                       arena_bytes, need, window_blocks, fit);
    return set_error(MSQ_E_WINDOW, "block_stream_create: arena %zu bytes < %zu needed for window_blocks=%d; not even one layer per window fits",
                     arena_bytes, need, window_blocks);
  }
  // host-side validation is complete; the pinned check is the first HIP call
  for (int l = 0; l < n_layers; ++l) {
    const int rc = check_pinned(l, host_blobs[l], blob_bytes[l]);
    if (rc) return rc;
  }
  msq_window* w = new msq_window();
  w->n_layers = n_layers;
  w->window_blocks = window_blocks;
  w->n_windows = (n_layers + window_blocks - 1) / window_blocks;
  w->host.assign(host_blobs, host_blobs + n_layers);
  w->bytes.assign(blob_bytes, blob_bytes + n_layers);
  const std::vector<size_t> psz = position_sizes(blob_bytes, n_layers, window_blocks);
  w->pos_off.assign(window_blocks, 0);
  for (int q = 1; q < window_blocks; ++q) w->pos_off[q] = w->pos_off[q - 1] + psz[q - 1];
  w->n_slots = n_slots;
  w->slot_bytes = need / n_slots;
  w->slot_base.resize(n_slots);
  for (int i = 0; i < n_slots; ++i) w->slot_base[i] = (char*)dev_arena + (size_t)i * w->slot_bytes;
  const int ne = n_slots * window_blocks;
  w->ready.assign(ne, nullptr);
  w->freed.assign(ne, nullptr);
  w->ready_recorded.assign(ne, 0);
  w->freed_recorded.assign(ne, 0);
  w->release_order.assign(n_slots, std::vector<int>());
  w->released.assign(n_slots, std::vector<char>(window_blocks, 0));
  w->slot_window.assign(n_slots, -1);
  w->state.assign(n_slots, SLOT_FREE);
  w->release_tick.assign(n_slots, 0);
  for (int i = 0; i < n_copy_streams; ++i) w->copies.push_back((hipStream_t)copy_streams[i]);
  hipError_t e = hipSuccess;
  for (int i = 0; i < ne && e == hipSuccess; ++i) {
    e = hipEventCreateWithFlags(&w->ready[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&w->freed[i], hipEventDisableTiming);
  }
  if (e == hipSuccess) e = hipEventCreate(&w->t_ref);
  if (e == hipSuccess) e = hipEventRecord(w->t_ref, w->copies[0]);
  if (e != hipSuccess) {
    destroy_events(w);
    delete w;
    return hip_error(e, "block_stream_create: events");
  }
  *out = w;
  return MSQ_OK;
}

int block_stream_prefetch(msq_window* w, int first_layer) {
  if (!w) return set_error(MSQ_E_INVAL, "block_stream_prefetch: null window");
  if (first_layer < 0 || first_layer >= w->n_layers || first_layer % w->window_blocks)
    return set_error(MSQ_E_INVAL, "block_stream_prefetch: first_layer=%d is not a window start", first_layer);
  const int win = first_layer / w->window_blocks;
  if (find_slot(w, win, SLOT_HELD) >= 0) return MSQ_OK;  // already prefetched and not released
  int slot = find_slot(w, win, SLOT_FREE);
  if (slot >= 0) {  // the free slot still holds this window's bytes
    w->state[slot] = SLOT_HELD;
    w->release_order[slot].clear();
    std::fill(w->released[slot].begin(), w->released[slot].end(), 0);
    w->stats.windows_reused++;
    return MSQ_OK;
  }
  // least recently released free slot
  slot = -1;
  for (int i = 0; i < w->n_slots; ++i)
    if (w->state[i] == SLOT_FREE && (slot < 0 || w->release_tick[i] < w->release_tick[slot])) slot = i;
  if (slot < 0)
    return set_error(MSQ_E_ORDER, "block_stream_prefetch: no free slot for window %d (release a window first)", win);
  hipError_t e = harvest(w, false);  // completed copies' timings, without waiting
  // the slot's old contents are about to be overwritten
  w->slot_window[slot] = -1;
  const int wb = w->window_blocks;
  const int count = std::min(wb, w->n_layers - first_layer);
  // copy order: the positions in the order the slot's last layers were released, then
  // any position not released before (a fresh slot, or a shorter last window)
  std::vector<int> order = w->release_order[slot];
  for (int q = 0; q < wb; ++q)
    if (std::find(order.begin(), order.end(), q) == order.end()) order.push_back(q);
  size_t total = 0;
  for (int q : order) {
    if (q >= count || e != hipSuccess) continue;
    const int l = first_layer + q;
    const int ev = slot * wb + q;
    hipStream_t cs = w->copies[l % w->copies.size()];
    // the position's range is free once the compute stream released its last layer and
    // the previous copy into it (possibly on another copy stream) is done
    if (w->freed_recorded[ev]) e = hipStreamWaitEvent(cs, w->freed[ev], 0);
    if (e == hipSuccess && w->ready_recorded[ev]) e = hipStreamWaitEvent(cs, w->ready[ev], 0);
    TimingPair tp;
    if (e == hipSuccess) e = take_pair(w, &tp);
    if (e == hipSuccess) e = hipEventRecord(tp.start, cs);
    if (e == hipSuccess)
      e = hipMemcpyAsync(w->slot_base[slot] + w->pos_off[q], w->host[l], w->bytes[l], hipMemcpyHostToDevice, cs);
    if (e == hipSuccess) e = hipEventRecord(tp.end, cs);
    if (e == hipSuccess) w->pending.push_back(tp);
    if (e == hipSuccess) e = hipEventRecord(w->ready[ev], cs);
    if (e == hipSuccess) w->ready_recorded[ev] = 1;
    total += w->bytes[l];
  }
  if (e != hipSuccess) return hip_error(e, "block_stream_prefetch: copy");
  w->slot_window[slot] = win;
  w->state[slot] = SLOT_HELD;
  w->release_order[slot].clear();
  std::fill(w->released[slot].begin(), w->released[slot].end(), 0);
  w->stats.bytes_copied += total;
  w->stats.windows_copied++;
  return MSQ_OK;
}

int block_stream_acquire(msq_window* w, int layer, msq_stream_t compute, const void** dev_blob) {
  if (!w || !dev_blob) return set_error(MSQ_E_INVAL, "block_stream_acquire: null pointer");
  if (layer < 0 || layer >= w->n_layers) return set_error(MSQ_E_INVAL, "block_stream_acquire: layer %d out of range", layer);
  const int win = layer / w->window_blocks;
  const int slot = find_slot(w, win, SLOT_HELD);
  if (slot < 0) return set_error(MSQ_E_ORDER, "block_stream_acquire: window %d (layer %d) was not prefetched", win, layer);
  const int q = layer % w->window_blocks;
  const hipError_t e = hipStreamWaitEvent((hipStream_t)compute, w->ready[slot * w->window_blocks + q], 0);
  if (e != hipSuccess) return hip_error(e, "block_stream_acquire: hipStreamWaitEvent");
  *dev_blob = w->slot_base[slot] + w->pos_off[q];
  return MSQ_OK;
}

}  // extern "C"

namespace {

// Records that position q of `slot` is no longer read by work queued on `compute`; the slot
// becomes free once every position of its window is released.
int release_position(msq_window* w, int slot, int q, hipStream_t compute, const char* fn) {
  const int wb = w->window_blocks;
  const int count = std::min(wb, w->n_layers - w->slot_window[slot] * wb);
  if (w->released[slot][q]) return set_error(MSQ_E_ORDER, "%s: layer %d was already released", fn, w->slot_window[slot] * wb + q);
  const hipError_t e = hipEventRecord(w->freed[slot * wb + q], compute);
  if (e != hipSuccess) return hip_error(e, fn);
  w->freed_recorded[slot * wb + q] = 1;
  w->released[slot][q] = 1;
  w->release_order[slot].push_back(q);
  if ((int)w->release_order[slot].size() == count) {
    w->state[slot] = SLOT_FREE;
    w->release_tick[slot] = ++w->tick;
  }
  return MSQ_OK;
}

}  // namespace

extern "C" {

int block_stream_release(msq_window* w, int first_layer, msq_stream_t compute) {
  if (!w) return set_error(MSQ_E_INVAL, "block_stream_release: null window");
  if (first_layer < 0 || first_layer >= w->n_layers || first_layer % w->window_blocks)
    return set_error(MSQ_E_INVAL, "block_stream_release: first_layer=%d is not a window start", first_layer);
  const int win = first_layer / w->window_blocks;
  const int slot = find_slot(w, win, SLOT_HELD);
  if (slot < 0) return set_error(MSQ_E_ORDER, "block_stream_release: window %d is not held", win);
  const int count = std::min(w->window_blocks, w->n_layers - first_layer);
  for (int q = 0; q < count; ++q) {
    if (w->released[slot][q]) continue;
    const int rc = release_position(w, slot, q, (hipStream_t)compute, "block_stream_release");
    if (rc) return rc;
  }
  return MSQ_OK;
}

int block_stream_release_layer(msq_window* w, int layer, msq_stream_t compute) {
  if (!w) return set_error(MSQ_E_INVAL, "block_stream_release_layer: null window");
  if (layer < 0 || layer >= w->n_layers) return set_error(MSQ_E_INVAL, "block_stream_release_layer: layer %d out of range", layer);
  const int win = layer / w->window_blocks;
  const int slot = find_slot(w, win, SLOT_HELD);
  if (slot < 0) return set_error(MSQ_E_ORDER, "block_stream_release_layer: window %d (layer %d) is not held", win, layer);
  return release_position(w, slot, layer % w->window_blocks, (hipStream_t)compute, "block_stream_release_layer");
}

int block_stream_stats(msq_window* w, msq_window_stats* out) {
  if (!w || !out) return set_error(MSQ_E_INVAL, "block_stream_stats: null pointer");
  hipError_t e = harvest(w, true);
  if (e != hipSuccess) return hip_error(e, "block_stream_stats: copy timing");
  w->stats.busy_ms += merge_spans(w, 0);
  // every copy issued so far is done: later spans are measured from a fresh reference
  e = hipEventRecord(w->t_ref, w->copies[0]);
  if (e != hipSuccess) return hip_error(e, "block_stream_stats: hipEventRecord");
  *out = w->stats;
  return MSQ_OK;
}

int block_stream_destroy(msq_window* w) {
  if (!w) return MSQ_OK;
  hipError_t e = hipSuccess;
  for (size_t i = 0; i < w->ready.size(); ++i)
    if (w->ready[i] && w->ready_recorded[i]) {
      const hipError_t e1 = hipEventSynchronize(w->ready[i]);
      if (e == hipSuccess) e = e1;
    }
  destroy_events(w);
  delete w;
  return e == hipSuccess ? MSQ_OK : hip_error(e, "block_stream_destroy");
}

}  // extern "C"

extern "C" {

int msq_host_alloc(size_t bytes, void** out) {
  if (!out) return set_error(MSQ_E_INVAL, "msq_host_alloc: out is NULL");
  *out = nullptr;
  if (bytes == 0 || bytes > ((size_t)1 << 46))
    return set_error(MSQ_E_INVAL, "msq_host_alloc: bytes=%zu outside [1, 2^46]", bytes);
  void* p = nullptr;
  const hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocDefault);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return set_error(MSQ_E_HIP, "msq_host_alloc: hipHostMalloc of %zu bytes: %s (%d)", bytes, hipGetErrorString(e),
                     (int)e);
  }
  if ((uintptr_t)p % 256) {
    (void)hipHostFree(p);
    return set_error(MSQ_E_HIP, "msq_host_alloc: hipHostMalloc returned %p, not 256-byte aligned", p);
  }
  *out = p;
  return MSQ_OK;
}

int msq_host_free(void* p) {
  if (!p) return MSQ_OK;
  const hipError_t e = hipHostFree(p);
  return e == hipSuccess ? MSQ_OK : hip_error(e, "msq_host_free");
}

}  // extern "C"
