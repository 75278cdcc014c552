// Streamed quantizing load: a bf16 host source (for instance a memory-mapped
// checkpoint) becomes NF4 codes + absmax in host memory without the base ever being
// whole on the device.
//
// The pages' loader stages one tensor at a time, quantizes it and evicts it before the
// next, so its device peak stays far below a standard load that materialises the base,
// and its output is byte-identical to the standard load's ("Poros" research post, the
// streamed-loader paragraph).  Here every tensor is cut into row chunks (NF4 blocks
// never cross a row, so a chunk quantizes exactly as it would inside the whole
// tensor) that rotate through two staging slots:
//
//   host: copy chunk c of the source into pinned bounce buffer c % 2 (several threads)
//   stream: H2D bounce -> device slot c % 2, nf4_quantize, D2H codes and absmax into
//           the destination
//
// so the host copy of chunk c+1 overlaps the device work on chunk c.  The host waits
// only for the H2D that last read a bounce buffer before refilling it; device slots are
// reused in stream order.  Device memory: two slots of chunk_rows x max_cols, whatever
// the model size.
#include <string.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "../../include/msq.h"
#include "internal.hpp"

using namespace msq;

namespace {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct SlotLayout {
  size_t w, codes, absmax, slot;  // offsets inside a slot and the slot's size
};

SlotLayout slot_layout(int64_t elems) {
  SlotLayout L;
  L.w = 0;
  L.codes = align256((size_t)elems * 2);
  L.absmax = L.codes + align256((size_t)elems / 2);
  L.slot = L.absmax + align256((size_t)elems / 16);
  return L;
}

void parallel_copy(void* dst, const void* src, size_t bytes, int threads) {
  const size_t min_piece = (size_t)4 << 20;
  const int t = (int)std::min<size_t>((size_t)threads, std::max<size_t>(1, bytes / min_piece));
  if (t <= 1) {
    memcpy(dst, src, bytes);
    return;
  }
  std::vector<std::thread> pool;
  const size_t piece = (bytes + t - 1) / t;
  for (int i = 0; i < t; ++i) {
    const size_t o = (size_t)i * piece;
    if (o >= bytes) break;
    const size_t n = std::min(piece, bytes - o);
    pool.emplace_back([=] { memcpy((char*)dst + o, (const char*)src + o, n); });
  }
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

size_t nf4_stream_load_device_bytes(int64_t max_cols, int64_t chunk_rows) {
  if (max_cols <= 0 || max_cols % 64 || chunk_rows <= 0) return 0;
  return 2 * slot_layout(chunk_rows * max_cols).slot;
}

size_t nf4_stream_load_host_bytes(int64_t max_cols, int64_t chunk_rows) {
  if (max_cols <= 0 || max_cols % 64 || chunk_rows <= 0) return 0;
  return 2 * align256((size_t)(chunk_rows * max_cols) * 2);
}

int nf4_stream_load(const msq_quant_job* jobs, int n_jobs, int64_t chunk_rows, void* dev_staging,
                    size_t dev_bytes, void* host_bounce, size_t host_bytes, int host_threads,
                    msq_stream_t stream) {
  if (n_jobs < 0 || (n_jobs > 0 && !jobs)) return set_error(MSQ_E_INVAL, "nf4_stream_load: bad job list");
  if (chunk_rows <= 0) return set_error(MSQ_E_INVAL, "nf4_stream_load: chunk_rows=%lld", (long long)chunk_rows);
  if (host_threads < 1 || host_threads > 64)
    return set_error(MSQ_E_INVAL, "nf4_stream_load: host_threads=%d outside [1, 64]", host_threads);
  int64_t max_cols = 0;
  for (int i = 0; i < n_jobs; ++i) {
    const msq_quant_job& j = jobs[i];
    if (j.rows < 0 || j.cols <= 0) return set_error(MSQ_E_INVAL, "nf4_stream_load: job %d rows=%lld cols=%lld", i, (long long)j.rows, (long long)j.cols);
    if (j.cols % 64) return set_error(MSQ_E_SHAPE, "nf4_stream_load: job %d cols=%lld is not a multiple of 64", i, (long long)j.cols);
    if (j.rows > 0 && (!j.src || !j.codes || !j.absmax)) return set_error(MSQ_E_INVAL, "nf4_stream_load: job %d null pointer", i);
    max_cols = std::max(max_cols, j.cols);
  }
  if (max_cols == 0) return MSQ_OK;
  const size_t need_dev = nf4_stream_load_device_bytes(max_cols, chunk_rows);
  const size_t need_host = nf4_stream_load_host_bytes(max_cols, chunk_rows);
  if (!dev_staging || !host_bounce) return set_error(MSQ_E_INVAL, "nf4_stream_load: null staging buffer");
  if (((uintptr_t)dev_staging % 256) || ((uintptr_t)host_bounce % 256))
    return set_error(MSQ_E_INVAL, "nf4_stream_load: staging buffers must be 256-byte aligned");
  if (dev_bytes < need_dev || host_bytes < need_host)
    return set_error(MSQ_E_WORKSPACE, "nf4_stream_load: staging %zu (device) / %zu (host) bytes < %zu / %zu", dev_bytes,
                     host_bytes, need_dev, need_host);

  hipStream_t s = (hipStream_t)stream;
  const int64_t chunk_elems = chunk_rows * max_cols;
  const SlotLayout L = slot_layout(chunk_elems);
  char* dev[2] = {(char*)dev_staging, (char*)dev_staging + L.slot};
  char* bounce[2] = {(char*)host_bounce, (char*)host_bounce + need_host / 2};
  hipEvent_t h2d_done[2] = {nullptr, nullptr};
  bool pending[2] = {false, false};
  hipError_t e = hipSuccess;
  for (int i = 0; i < 2 && e == hipSuccess; ++i) e = hipEventCreateWithFlags(&h2d_done[i], hipEventDisableTiming);
  int64_t c = 0;  // chunk counter: slot c % 2
  for (int i = 0; i < n_jobs && e == hipSuccess; ++i) {
    const msq_quant_job& j = jobs[i];
    const int64_t rows_per = std::max<int64_t>(1, chunk_elems / j.cols);
    for (int64_t r0 = 0; r0 < j.rows && e == hipSuccess; r0 += rows_per, ++c) {
      const int slot = (int)(c & 1);
      const int64_t rows = std::min(rows_per, j.rows - r0);
      const size_t elems = (size_t)(rows * j.cols);
      if (pending[slot]) {
        e = hipEventSynchronize(h2d_done[slot]);  // the bounce buffer's last H2D has read it
        if (e != hipSuccess) break;
      }
      parallel_copy(bounce[slot], (const char*)j.src + (size_t)r0 * j.cols * 2, elems * 2, host_threads);
      e = hipMemcpyAsync(dev[slot] + L.w, bounce[slot], elems * 2, hipMemcpyHostToDevice, s);
      if (e == hipSuccess) e = hipEventRecord(h2d_done[slot], s);
      pending[slot] = true;
      if (e == hipSuccess)
        e = launch_quantize((const uint16_t*)(dev[slot] + L.w), (int64_t)(elems / 64), (uint8_t*)(dev[slot] + L.codes),
                            (float*)(dev[slot] + L.absmax), s);
      if (e == hipSuccess)
        e = hipMemcpyAsync(j.codes + (size_t)r0 * (j.cols / 2), dev[slot] + L.codes, elems / 2, hipMemcpyDeviceToHost, s);
      if (e == hipSuccess)
        e = hipMemcpyAsync(j.absmax + (size_t)r0 * (j.cols / 64), dev[slot] + L.absmax, elems / 16,
                           hipMemcpyDeviceToHost, s);
    }
  }
  const hipError_t es = hipStreamSynchronize(s);
  if (e == hipSuccess) e = es;
  for (int i = 0; i < 2; ++i)
    if (h2d_done[i]) (void)hipEventDestroy(h2d_done[i]);
  return e == hipSuccess ? MSQ_OK : hip_error(e, "nf4_stream_load");
}

}  // extern "C"
