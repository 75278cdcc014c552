// Host-to-device block-prefetch window (double-buffered, event-ordered).
//
// The pages' forward streams frozen blocks through a small GPU window with
// asynchronous prefetch on side streams; the backward walks the blocks in reverse and
// reloads each one; eviction is a pointer release because the base is read-only, so
// nothing is ever copied back ("Poros" research post, training-step paragraph;
// "Limitations", "Pretraining is out of scope").  Their block-size sweep (peak memory
// at block sizes 1..16, "Poros" research post, memory paragraph) grows by two
// blocks' worth per doubling, consistent with one window computing while the next
// one loads: the default is two slots.  More slots let the copies run further ahead,
// and single-layer slots let a slot be refilled as soon as its one layer is done.
//
// Ordering is kept per layer position inside a slot: the copy stream waits on the
// position's "freed" event (recorded on the compute stream when the layer that held it
// was released) before overwriting it, and records the position's "ready" event after
// its copy; acquire makes the compute stream wait on the layer's own "ready".  A window
// is still claimed and copied as one unit, but its layers are copied in the order the
// slot's previous layers were released (ascending after a forward, descending after a
// backward), so the first layer of the next window lands as soon as the first layer of
// the last one is done, and compute on a layer starts as soon as that layer has landed.
// The host never blocks.  A prefetch of a window that a free slot still holds issues no
// copy (the windows in the slots at the end of the forward are the first the backward
// needs).
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/msq.h"
#include "internal.hpp"

using namespace msq;

namespace {
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

enum SlotState { SLOT_FREE = 0, SLOT_HELD = 1 };
}  // namespace

struct msq_window {
  int n_layers = 0, window_blocks = 0, n_windows = 0, n_slots = 0;
  std::vector<const void*> host;
  std::vector<size_t> bytes;
  std::vector<size_t> offset;  // offset of each layer inside its window's slot
  size_t slot_bytes = 0;
  std::vector<char*> slot_base;
  hipStream_t copy = nullptr;
  // per (slot, position) events, index slot * window_blocks + position
  std::vector<hipEvent_t> ready, freed;
  std::vector<char> freed_recorded;
  std::vector<std::vector<int>> release_order;  // positions in the order they were released
  std::vector<std::vector<char>> released;      // per slot and position: released since claimed
  std::vector<int> slot_window;  // window whose bytes the slot holds (or will hold)
  std::vector<int> state;
  std::vector<uint64_t> release_tick;
  uint64_t tick = 0;
  msq_window_stats stats = {0, 0, 0, 0.0, 0};
  // copy timing: one (start, end) event pair per issued layer copy, from a ring; a pair is
  // read (and its duration added to stats.copy_ms) when the ring comes round to it or when
  // the statistics are asked for
  static constexpr int TIMING_RING = 64;
  hipEvent_t t_start[TIMING_RING] = {}, t_end[TIMING_RING] = {};
  bool t_pending[TIMING_RING] = {};
  int t_next = 0;
};

namespace {

size_t window_bytes(const size_t* blob_bytes, int n_layers, int first, int wb) {
  size_t s = 0;
  for (int l = first; l < first + wb && l < n_layers; ++l) s += align256(blob_bytes[l]);
  return s;
}

size_t max_window_bytes(const size_t* blob_bytes, int n_layers, int wb) {
  size_t m = 0;
  for (int f = 0; f < n_layers; f += wb) m = std::max(m, window_bytes(blob_bytes, n_layers, f, wb));
  return m;
}

// Adds the duration of timing pair i to the statistics once its copies are done.
hipError_t collect_timing(msq_window* w, int i) {
  if (!w->t_pending[i]) return hipSuccess;
  hipError_t e = hipEventSynchronize(w->t_end[i]);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, w->t_start[i], w->t_end[i]);
  if (e != hipSuccess) return e;
  w->stats.copy_ms += ms;
  w->stats.copies_timed++;
  w->t_pending[i] = false;
  return hipSuccess;
}

int find_slot(const msq_window* w, int win, int state) {
  for (int i = 0; i < w->n_slots; ++i)
    if (w->slot_window[i] == win && w->state[i] == state) return i;
  return -1;
}

}  // namespace

extern "C" {

size_t block_stream_arena_bytes(const size_t* blob_bytes, int n_layers, int window_blocks,
                                int n_slots) {
  if (!blob_bytes || n_layers <= 0 || window_blocks <= 0 || n_slots < 2) return 0;
  return (size_t)n_slots * max_window_bytes(blob_bytes, n_layers, window_blocks);
}

int block_stream_create(msq_window** out, const void* const* host_blobs, const size_t* blob_bytes,
                        int n_layers, int window_blocks, int n_slots, void* dev_arena,
                        size_t arena_bytes, msq_stream_t copy_stream) {
  if (!out || !host_blobs || !blob_bytes || !dev_arena)
    return set_error(MSQ_E_INVAL, "block_stream_create: null pointer");
  *out = nullptr;
  if (n_layers <= 0 || window_blocks <= 0 || window_blocks > n_layers || n_slots < 2 || n_slots > 1024)
    return set_error(MSQ_E_INVAL, "block_stream_create: n_layers=%d window_blocks=%d n_slots=%d", n_layers,
                     window_blocks, n_slots);
  if ((uintptr_t)dev_arena % 256)
    return set_error(MSQ_E_INVAL, "block_stream_create: arena must be 256-byte aligned");
  for (int l = 0; l < n_layers; ++l)
    if (!host_blobs[l] || blob_bytes[l] == 0)
      return set_error(MSQ_E_INVAL, "block_stream_create: layer %d has no host blob", l);
  const size_t need = (size_t)n_slots * max_window_bytes(blob_bytes, n_layers, window_blocks);
  if (arena_bytes < need) {
    int fit = 0;
    for (int wb = window_blocks - 1; wb >= 1; --wb)
      if ((size_t)n_slots * max_window_bytes(blob_bytes, n_layers, wb) <= arena_bytes) {
        fit = wb;
        break;
      }
    if (fit > 0)
      return set_error(MSQ_E_WINDOW, "block_stream_create: arena %zu bytes < %zu needed for window_blocks=%d; largest window that fits: window_blocks=%d",
                       arena_bytes, need, window_blocks, fit);
    return set_error(MSQ_E_WINDOW, "block_stream_create: arena %zu bytes < %zu needed for window_blocks=%d; not even one layer per window fits",
                     arena_bytes, need, window_blocks);
  }
  msq_window* w = new msq_window();
  w->n_layers = n_layers;
  w->window_blocks = window_blocks;
  w->n_windows = (n_layers + window_blocks - 1) / window_blocks;
  w->host.assign(host_blobs, host_blobs + n_layers);
  w->bytes.assign(blob_bytes, blob_bytes + n_layers);
  w->offset.resize(n_layers);
  for (int f = 0; f < n_layers; f += window_blocks) {
    size_t o = 0;
    for (int l = f; l < f + window_blocks && l < n_layers; ++l) {
      w->offset[l] = o;
      o += align256(blob_bytes[l]);
    }
  }
  w->n_slots = n_slots;
  w->slot_bytes = need / n_slots;
  w->slot_base.resize(n_slots);
  for (int i = 0; i < n_slots; ++i) w->slot_base[i] = (char*)dev_arena + (size_t)i * w->slot_bytes;
  const int ne = n_slots * window_blocks;
  w->ready.assign(ne, nullptr);
  w->freed.assign(ne, nullptr);
  w->freed_recorded.assign(ne, 0);
  w->release_order.assign(n_slots, std::vector<int>());
  w->released.assign(n_slots, std::vector<char>(window_blocks, 0));
  w->slot_window.assign(n_slots, -1);
  w->state.assign(n_slots, SLOT_FREE);
  w->release_tick.assign(n_slots, 0);
  w->copy = (hipStream_t)copy_stream;
  hipError_t e = hipSuccess;
  for (int i = 0; i < ne && e == hipSuccess; ++i) {
    e = hipEventCreateWithFlags(&w->ready[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&w->freed[i], hipEventDisableTiming);
  }
  for (int i = 0; i < msq_window::TIMING_RING && e == hipSuccess; ++i) {
    e = hipEventCreate(&w->t_start[i]);
    if (e == hipSuccess) e = hipEventCreate(&w->t_end[i]);
  }
  if (e != hipSuccess) {
    for (int j = 0; j < ne; ++j) {
      if (w->ready[j]) (void)hipEventDestroy(w->ready[j]);
      if (w->freed[j]) (void)hipEventDestroy(w->freed[j]);
    }
    for (int j = 0; j < msq_window::TIMING_RING; ++j) {
      if (w->t_start[j]) (void)hipEventDestroy(w->t_start[j]);
      if (w->t_end[j]) (void)hipEventDestroy(w->t_end[j]);
    }
    delete w;
    return hip_error(e, "block_stream_create: hipEventCreate");
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
  hipError_t e = hipSuccess;
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
    if (w->freed_recorded[ev]) e = hipStreamWaitEvent(w->copy, w->freed[ev], 0);
    const int ti = w->t_next;
    w->t_next = (w->t_next + 1) % msq_window::TIMING_RING;
    if (e == hipSuccess) e = collect_timing(w, ti);  // the ring's oldest pair, long complete
    if (e == hipSuccess) e = hipEventRecord(w->t_start[ti], w->copy);
    if (e == hipSuccess)
      e = hipMemcpyAsync(w->slot_base[slot] + w->offset[l], w->host[l], w->bytes[l], hipMemcpyHostToDevice, w->copy);
    if (e == hipSuccess) e = hipEventRecord(w->t_end[ti], w->copy);
    if (e == hipSuccess) w->t_pending[ti] = true;
    if (e == hipSuccess) e = hipEventRecord(w->ready[ev], w->copy);
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
  const hipError_t e =
      hipStreamWaitEvent((hipStream_t)compute, w->ready[slot * w->window_blocks + layer % w->window_blocks], 0);
  if (e != hipSuccess) return hip_error(e, "block_stream_acquire: hipStreamWaitEvent");
  *dev_blob = w->slot_base[slot] + w->offset[layer];
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
  for (int i = 0; i < msq_window::TIMING_RING; ++i) {
    const hipError_t e = collect_timing(w, i);
    if (e != hipSuccess) return hip_error(e, "block_stream_stats: copy timing");
  }
  *out = w->stats;
  return MSQ_OK;
}

int block_stream_destroy(msq_window* w) {
  if (!w) return MSQ_OK;
  hipError_t e = hipSuccess;
  for (size_t i = 0; i < w->ready.size(); ++i) {
    if (w->ready[i]) {
      const hipError_t e1 = hipEventSynchronize(w->ready[i]);
      if (e == hipSuccess) e = e1;
      (void)hipEventDestroy(w->ready[i]);
    }
    if (w->freed[i]) (void)hipEventDestroy(w->freed[i]);
  }
  for (int i = 0; i < msq_window::TIMING_RING; ++i) {
    if (w->t_start[i]) (void)hipEventDestroy(w->t_start[i]);
    if (w->t_end[i]) (void)hipEventDestroy(w->t_end[i]);
  }
  delete w;
  return e == hipSuccess ? MSQ_OK : hip_error(e, "block_stream_destroy");
}

}  // extern "C"
