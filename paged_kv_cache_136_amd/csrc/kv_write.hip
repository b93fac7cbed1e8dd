// Paged KV write and copy-on-write block copy for gfx950.
//
// pa_write_kv: each new token's K and V rows are stored at the token's flat
// slot ("qaqbuyan.com article 130", KV-cache section: a decode step computes
// the new token's K/V and appends them to the cache; "day31": the token goes
// into the last, partly filled block, or a fresh one).
// pa_copy_blocks: "day31", toy COW append -- the new private block receives
// the old block's KV bytes; here the whole block, every layer, K and V.
//
// Both are pure byte moves.  One K/V row of a token (Hkv*D*elem bytes) is
// contiguous in the source and in the destination slot, so each lane moves
// one 16-byte chunk with a dwordx4 load/store; consecutive lanes touch
// consecutive chunks.  They are HBM-bound at 2 bytes moved per byte copied.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>

#include "pagedkv.h"
#include "status.hpp"

namespace pkv {
namespace {

// grid-stride over T * chunks_per_row 16-byte chunks.
__global__ __launch_bounds__(256) void write_kv_kernel(uint4* __restrict__ k, uint4* __restrict__ v,
                                                       const uint4* __restrict__ kn,
                                                       const uint4* __restrict__ vn,
                                                       const int64_t* __restrict__ slots, int64_t total,
                                                       int32_t chunks_per_row, int64_t num_slots) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t t = i / chunks_per_row;
    const int32_t c = static_cast<int32_t>(i - t * chunks_per_row);
    const int64_t s = slots[t];
    if (s < 0 || s >= num_slots) continue;
    const int64_t dst = s * chunks_per_row + c;
    k[dst] = kn[i];
    v[dst] = vn[i];
  }
}

constexpr int kMaxLayersPerLaunch = 32;

struct CopyArgs {
  uint4* k[kMaxLayersPerLaunch];
  uint4* v[kMaxLayersPerLaunch];
  const int32_t* pairs;
  int64_t chunks_per_block;
  int32_t num_pairs;
  int32_t num_blocks;
};

// grid: x = groups of kCopyGroup chunks of a block, y = pair,
// z = 2 * layer + {0: K, 1: V}.  A thread moves kCopyPerThread chunks per
// group, all loads issued before the stores, so they are in flight
// together.  Plain (cached) loads and stores: the decode that follows a
// copy-on-write reads both blocks again.
constexpr int kCopyPerThread = 4;
constexpr int kCopyGroup = 256 * kCopyPerThread;   // chunks per workgroup pass

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a) {
  const int pair = blockIdx.y;
  const int layer = blockIdx.z >> 1;
  const int32_t src = a.pairs[2 * pair], dst = a.pairs[2 * pair + 1];
  if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks) return;
  uint4* base = (blockIdx.z & 1) ? a.v[layer] : a.k[layer];
  const uint4* s = base + static_cast<int64_t>(src) * a.chunks_per_block;
  uint4* d = base + static_cast<int64_t>(dst) * a.chunks_per_block;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* sv = reinterpret_cast<const u32x4*>(s);
  u32x4* dv = reinterpret_cast<u32x4*>(d);
  for (int64_t g = blockIdx.x * static_cast<int64_t>(kCopyGroup); g < a.chunks_per_block;
       g += static_cast<int64_t>(gridDim.x) * kCopyGroup) {
    u32x4 r[kCopyPerThread];
    if (g + kCopyGroup <= a.chunks_per_block) {
      // A whole group: no per-chunk test, so the loads issue back to back.
#pragma unroll
      for (int u = 0; u < kCopyPerThread; ++u) r[u] = sv[g + u * 256 + threadIdx.x];
#pragma unroll
      for (int u = 0; u < kCopyPerThread; ++u) dv[g + u * 256 + threadIdx.x] = r[u];
    } else {
#pragma unroll
      for (int u = 0; u < kCopyPerThread; ++u) {
        const int64_t i = g + u * 256 + threadIdx.x;
        if (i < a.chunks_per_block) r[u] = sv[i];
      }
#pragma unroll
      for (int u = 0; u < kCopyPerThread; ++u) {
        const int64_t i = g + u * 256 + threadIdx.x;
        if (i < a.chunks_per_block) dv[i] = r[u];
      }
    }
  }
}

int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PA_DTYPE_F32: return 4;
    case PA_DTYPE_F16: return 2;
    case PA_DTYPE_BF16: return 2;
    default: return 0;
  }
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int pa_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, int32_t T, int32_t num_blocks,
                           int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                           int32_t dtype, void* stream) {
  if (T < 0 || num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PA_ERR_INVALID, "pa_write_kv: bad sizes");
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(PA_ERR_UNSUPPORTED, "pa_write_kv: unknown dtype");
  if (T == 0) { clear_error(); return PA_OK; }
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping)
    return fail(PA_ERR_INVALID, "pa_write_kv: null pointer");
  const int64_t row_bytes = static_cast<int64_t>(num_kv_heads) * head_dim * eb;
  if (row_bytes % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "pa_write_kv: num_kv_heads*head_dim*elem must be a multiple of 16 bytes");
  if ((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache) |
       reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return fail(PA_ERR_INVALID, "pa_write_kv: buffers must be 16-byte aligned");
  const int32_t cpr = static_cast<int32_t>(row_bytes / 16);
  const int64_t total = static_cast<int64_t>(T) * cpr;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipStream_t st = static_cast<hipStream_t>(stream);
  write_kv_kernel<<<static_cast<unsigned>(blocks), 256, 0, st>>>(
      static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), static_cast<const uint4*>(k_new),
      static_cast<const uint4*>(v_new), slot_mapping, total, cpr,
      static_cast<int64_t>(num_blocks) * block_size);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return fail(PA_ERR_DEVICE, std::string("pa_write_kv: launch failed: ") + hipGetErrorString(err));
  clear_error();
  return PA_OK;
}

extern "C" int pa_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                              int64_t block_bytes, int32_t num_blocks, const int32_t* pairs,
                              int32_t num_pairs, void* stream) {
  if (num_layers < 0 || num_pairs < 0 || num_blocks <= 0 || block_bytes <= 0 || block_bytes % 16)
    return fail(PA_ERR_INVALID, "pa_copy_blocks: bad sizes (block_bytes must be a positive multiple of 16)");
  if (num_layers == 0 || num_pairs == 0) { clear_error(); return PA_OK; }
  if (!k_caches || !v_caches || !pairs) return fail(PA_ERR_INVALID, "pa_copy_blocks: null pointer");
  if (num_pairs > 65535) return fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: more than 65535 pairs");
  for (int32_t l = 0; l < num_layers; ++l) {
    if (!k_caches[l] || !v_caches[l]) return fail(PA_ERR_INVALID, "pa_copy_blocks: null cache pointer");
    if ((reinterpret_cast<uintptr_t>(k_caches[l]) | reinterpret_cast<uintptr_t>(v_caches[l])) & 15)
      return fail(PA_ERR_INVALID, "pa_copy_blocks: caches must be 16-byte aligned");
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t cpb = block_bytes / 16;
  int64_t gx = (cpb + kCopyGroup - 1) / kCopyGroup;   // kCopyPerThread chunks per thread
  if (gx < 1) gx = 1;
  if (gx > 1024) gx = 1024;
  for (int32_t l0 = 0; l0 < num_layers; l0 += kMaxLayersPerLaunch) {
    const int32_t nl = std::min(kMaxLayersPerLaunch, num_layers - l0);
    CopyArgs a{};
    for (int32_t i = 0; i < nl; ++i) {
      a.k[i] = static_cast<uint4*>(k_caches[l0 + i]);
      a.v[i] = static_cast<uint4*>(v_caches[l0 + i]);
    }
    a.pairs = pairs;
    a.chunks_per_block = cpb;
    a.num_pairs = num_pairs;
    a.num_blocks = num_blocks;
    copy_blocks_kernel<<<dim3(static_cast<unsigned>(gx), num_pairs, 2 * nl), 256, 0, st>>>(a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
      return fail(PA_ERR_DEVICE, std::string("pa_copy_blocks: launch failed: ") + hipGetErrorString(err));
  }
  clear_error();
  return PA_OK;
}
