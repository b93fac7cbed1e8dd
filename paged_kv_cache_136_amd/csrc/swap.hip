// Preemption copies between the paged KV cache and pinned host memory.
//
// "qaqbuyan.com article 130", continuous-batching scheduler,
// _preempt_request: when blocks run out, the victim's KV blocks are copied
// to CPU memory and freed; the sequence comes back later into fresh blocks.
//
// A block of one layer is block_bytes contiguous bytes in K and as many in
// V, and the victim's blocks are scattered through the pool, so a
// per-piece DMA copy would take 2 * layers * blocks API calls.  Instead one
// kernel moves every (block, layer, K|V) piece: the GPU reads or writes the
// pinned host buffer directly over the host link, 16 bytes per lane, with
// consecutive lanes on consecutive chunks so each wave moves 1 KiB runs.
// Host-side reads have microsecond latency, so every lane keeps several
// 16-byte loads in flight before storing.
//
// Host record layout: a record is one block of every layer, R = num_layers
// * 2 * block_bytes bytes; within it, layer l, c = 0 (K) / 1 (V) sits at
// byte (l * 2 + c) * block_bytes.  Entry i of the block list uses record
// host_slots[i] (a slot of a host swap pool), or record i when no slot
// list is given.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>

#include "pagedkv.h"
#include "status.hpp"

namespace pkv {
namespace {

constexpr int kMaxLayersPerLaunch = 32;
constexpr int kSwapThreads = 256;
constexpr int kSwapUnroll = 4;   // 16-byte loads in flight per lane

struct SwapArgs {
  uint4* k[kMaxLayersPerLaunch];
  uint4* v[kMaxLayersPerLaunch];
  uint4* host;              // device-visible address of the host records
  const int32_t* blocks;
  const int32_t* host_slots;  // record of each entry; nullptr = entry index
  int64_t num_records;        // records the host buffer holds
  int64_t chunks_per_block;
  int32_t num_blocks;
  int32_t layer0;           // first layer of this launch
  int32_t num_layers;       // layers in the whole record (all launches)
};

// grid: x = chunk groups of one piece, y = list entry, z = 2 * layer + c.
template <bool TO_HOST>
__global__ __launch_bounds__(kSwapThreads) void swap_kernel(SwapArgs a) {
  const int i = blockIdx.y;
  const int layer = blockIdx.z >> 1, c = blockIdx.z & 1;
  const int32_t b = a.blocks[i];
  const int64_t r = a.host_slots ? a.host_slots[i] : i;
  if (b < 0 || b >= a.num_blocks || r < 0 || r >= a.num_records) return;
  uint4* cache = (c ? a.v[layer] : a.k[layer]) + static_cast<int64_t>(b) * a.chunks_per_block;
  uint4* rec = a.host + ((r * a.num_layers + a.layer0 + layer) * 2 + c) * a.chunks_per_block;
  const uint4* src = TO_HOST ? cache : rec;
  uint4* dst = TO_HOST ? rec : cache;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kSwapThreads;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kSwapThreads + threadIdx.x;
       base < a.chunks_per_block; base += kSwapUnroll * stride) {
    uint4 r[kSwapUnroll];
#pragma unroll
    for (int u = 0; u < kSwapUnroll; ++u) {
      const int64_t j = base + u * stride;
      if (j < a.chunks_per_block) r[u] = src[j];
    }
#pragma unroll
    for (int u = 0; u < kSwapUnroll; ++u) {
      const int64_t j = base + u * stride;
      if (j < a.chunks_per_block) dst[j] = r[u];
    }
  }
}

// The device-visible address of [p, p + bytes), or nullptr unless the whole
// range is host memory that HIP has pinned and mapped for the device
// (pageable memory would fault the GPU).  Three independent checks: both
// ends report host memory, both ends map to device addresses exactly
// bytes - 1 apart (one mapping covers the range), and HIP hands out a
// device pointer for the start.  A failed query's error is cleared so it
// cannot surface from a later, unrelated call.
void* mapped_host_range(const void* p, int64_t bytes) {
  hipPointerAttribute_t at{}, end{};
  const char* last = static_cast<const char*>(p) + (bytes - 1);
  void* dev = nullptr;
  if (hipPointerGetAttributes(&at, p) != hipSuccess ||
      hipPointerGetAttributes(&end, last) != hipSuccess ||
      hipHostGetDevicePointer(&dev, const_cast<void*>(p), 0) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (at.type != hipMemoryTypeHost || end.type != hipMemoryTypeHost || !at.devicePointer ||
      !end.devicePointer || dev != at.devicePointer ||
      static_cast<char*>(end.devicePointer) - static_cast<char*>(at.devicePointer) != bytes - 1)
    return nullptr;
  return dev;
}

template <bool TO_HOST>
int swap_impl(const char* name, void* const* k_caches, void* const* v_caches, int32_t num_layers,
              int64_t block_bytes, int32_t num_blocks, const int32_t* blocks,
              const int32_t* host_slots, int32_t n, const void* host, int64_t host_bytes,
              void* stream) {
  const std::string who(name);
  if (num_layers < 0 || n < 0 || num_blocks <= 0 || block_bytes <= 0 || block_bytes % 16)
    return fail(PA_ERR_INVALID, who + ": bad sizes (block_bytes must be a positive multiple of 16)");
  if (num_layers == 0 || n == 0) { clear_error(); return PA_OK; }
  if (!k_caches || !v_caches || !blocks || !host) return fail(PA_ERR_INVALID, who + ": null pointer");
  if (n > 65535) return fail(PA_ERR_UNSUPPORTED, who + ": more than 65535 blocks per call");
  const int64_t record = static_cast<int64_t>(num_layers) * 2 * block_bytes;
  const int64_t num_records = host_bytes / record;
  if (!host_slots && num_records < n)
    return fail(PA_ERR_INVALID, who + ": host buffer holds " + std::to_string(host_bytes) +
                                    " bytes, " + std::to_string(n * record) + " needed");
  if (num_records < 1)
    return fail(PA_ERR_INVALID, who + ": host buffer holds " + std::to_string(host_bytes) +
                                    " bytes, at least one record (" + std::to_string(record) +
                                    ") needed");
  const int64_t need = num_records * record;
  if (reinterpret_cast<uintptr_t>(host) & 15)
    return fail(PA_ERR_INVALID, who + ": host buffer must be 16-byte aligned");
  for (int32_t l = 0; l < num_layers; ++l) {
    if (!k_caches[l] || !v_caches[l]) return fail(PA_ERR_INVALID, who + ": null cache pointer");
    if ((reinterpret_cast<uintptr_t>(k_caches[l]) | reinterpret_cast<uintptr_t>(v_caches[l])) & 15)
      return fail(PA_ERR_INVALID, who + ": caches must be 16-byte aligned");
  }
  void* dev_host = mapped_host_range(host, need);
  if (!dev_host)
    return fail(PA_ERR_INVALID, who + ": host buffer is not pinned host memory mapped for the GPU "
                                      "(allocate it with hipHostMalloc / torch pin_memory)");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t cpb = block_bytes / 16;
  int64_t gx = (cpb + kSwapThreads * kSwapUnroll - 1) / (kSwapThreads * kSwapUnroll);
  gx = std::max<int64_t>(1, std::min<int64_t>(gx, 1024));
  for (int32_t l0 = 0; l0 < num_layers; l0 += kMaxLayersPerLaunch) {
    const int32_t nl = std::min(kMaxLayersPerLaunch, num_layers - l0);
    SwapArgs a{};
    for (int32_t i = 0; i < nl; ++i) {
      a.k[i] = static_cast<uint4*>(k_caches[l0 + i]);
      a.v[i] = static_cast<uint4*>(v_caches[l0 + i]);
    }
    a.host = static_cast<uint4*>(dev_host);
    a.blocks = blocks;
    a.host_slots = host_slots;
    a.num_records = num_records;
    a.chunks_per_block = cpb;
    a.num_blocks = num_blocks;
    a.layer0 = l0;
    a.num_layers = num_layers;
    swap_kernel<TO_HOST><<<dim3(static_cast<unsigned>(gx), n, 2 * nl), kSwapThreads, 0, st>>>(a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
      return fail(PA_ERR_DEVICE, who + ": launch failed: " + hipGetErrorString(err));
  }
  clear_error();
  return PA_OK;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int pa_swap_out(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                           int64_t block_bytes, int32_t num_blocks, const int32_t* blocks,
                           const int32_t* host_slots, int32_t n, void* host_dst,
                           int64_t host_bytes, void* stream) {
  return swap_impl<true>("pa_swap_out", k_caches, v_caches, num_layers, block_bytes, num_blocks,
                         blocks, host_slots, n, host_dst, host_bytes, stream);
}

extern "C" int pa_swap_in(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                          int64_t block_bytes, int32_t num_blocks, const int32_t* blocks,
                          const int32_t* host_slots, int32_t n, const void* host_src,
                          int64_t host_bytes, void* stream) {
  return swap_impl<false>("pa_swap_in", k_caches, v_caches, num_layers, block_bytes, num_blocks,
                          blocks, host_slots, n, host_src, host_bytes, stream);
}
