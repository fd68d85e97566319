// Save and restore of one sequence's decode state: the window ring, the compressor
// tail rings and the pages of its compressed caches, packed into one flat buffer
// (dsv4 book Ch.5 "Decode-time cache state"; infra transcript: the KV cache split
// into a classical cache of compressed entries and a state cache of the recent window
// and the compressors' unfinished blocks).  A pure copy: the restored sequence
// continues bit for bit as the saved one would have.
#include "common.h"
#include "kernels.h"

namespace ca {

// The flat buffer: [window rows W * dim * esz][tail job 0][tail job 1][pages of cache
// job 0][pages of cache job 1], each part starting at a multiple of 256 bytes.
// Workgroups copy 4 KB chunks: the chunks of the window, of each tail, then of each
// page in page-table order (pages missing on the side read from, or written to, are
// skipped).
__global__ void __launch_bounds__(256) state_copy_kernel(StatePlan p, int to_buffer) {
  int64_t c = blockIdx.x;
  const uint8_t* src = nullptr;
  uint8_t* dst = nullptr;
  int64_t n = 0;
  for (int part = 0; part < p.n_parts; ++part) {
    const StatePart& q = p.part[part];
    const int64_t chunks = q.n_items * q.chunks_per_item;
    if (c >= chunks) {
      c -= chunks;
      continue;
    }
    const int64_t item = c / q.chunks_per_item, ck = c % q.chunks_per_item;
    int64_t off_live = item * q.item_bytes;              // the item in its live storage
    if (q.page_table != nullptr) {                       // an item is one page of a cache
      const int32_t pg = q.page_table[item];
      if (pg < 0 || pg >= q.n_pages) return;
      off_live = (int64_t)pg * q.item_bytes;
    }
    uint8_t* live = q.live + off_live + ck * 4096;
    uint8_t* flat = p.buffer + q.flat_offset + item * q.item_bytes + ck * 4096;
    n = q.item_bytes - ck * 4096 < 4096 ? q.item_bytes - ck * 4096 : 4096;
    src = to_buffer ? live : flat;
    dst = to_buffer ? flat : live;
    break;
  }
  if (src == nullptr) return;
  // 16-byte vectors where both sides allow it (every part is 16-byte aligned in both)
  for (int64_t i = 16 * threadIdx.x; i < n; i += 16 * blockDim.x) *(u32x4*)(dst + i) = *(const u32x4*)(src + i);
}

hipError_t launch_state_copy(const StatePlan& p, int to_buffer, hipStream_t st) {
  int64_t chunks = 0;
  for (int i = 0; i < p.n_parts; ++i) chunks += p.part[i].n_items * p.part[i].chunks_per_item;
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)chunks), dim3(256), 0, st, p, to_buffer);
  return hipGetLastError();
}

}  // namespace ca
