// Prefill attention of an uncached suffix over the paged KV cache (gfx950).
//
// What is computed: "P06 · BlockManager" spec overview and key-question
// answers -- after the first num_cached_tokens tokens of a prompt were
// prefix hits, only the rest needs a forward pass (at least the last token,
// whose output yields the next token); "qaqbuyan.com article 130",
// system-prompt section -- a request reuses the shared prompt's blocks and
// computes what follows.  Suffix token i of a sequence of total length n
// and suffix length q sits at position n - q + i and attends, causally, to
// every token 0 .. n - q + i through the block table (slot = table[pos/bs]
// * bs + pos % bs), its own K/V already written.  Scale 1/sqrt(head_dim)
// and float output as in the article's kernel listing.
//
// Design.  One workgroup of 4 waves per (query heads, query tile,
// sequence): hg = 4, 2 or 1 query heads of one KV group (the largest that
// divides the group) over 128 / hg rows, wave w serving head w % hg and
// rows 32 (w / hg) .. +31 as two 16-row query tiles.  The tile's K/V blocks are
// streamed through LDS once for all four waves, two blocks (32 keys) per
// stage (double-buffered, one barrier per stage; the next stage's loads are
// in flight while the current one is used), with block ids read by scalar
// loads and range-checked.  Per stage and wave, on the matrix cores (every
// K and V^T operand read from LDS feeds both query tiles):
//   S^T = K Q^T  v_mfma_f32_16x16x32, A = 16 keys from LDS, B = Q^T of the
//                wave's 16 query rows (registers); lane (qa, t) gets the
//                scores of keys 4qa .. 4qa+3 for query row t;
//   causal mask  key position <= query position, element by element;
//   softmax      online, exp2 domain, one update per stage; the running max
//                moves only when a stage max exceeds it by more than 2^8
//                (one wave-uniform test); per query row the stage max is a
//                2-step butterfly over the four qa lanes;
//   O^T += V^T P^T  v_mfma_f32_16x16x32 over the stage's two blocks, A = V^T
//                via transposed LDS reads, B = the lane's own p values; for
//                bfloat16 p is split into a high and a low part (two MFMAs)
//                so its 8-bit rounding does not reach the output.
// A wave skips stages past its last query row but keeps loading and
// synchronizing with the others.
#include <hip/hip_runtime.h>

#include <cmath>
#include <string>

#include "device_common.hpp"
#include "mfma_ops.hpp"
#include "pagedkv.h"
#include "status.hpp"

namespace pkv {
namespace {

constexpr int kPWaves = 4;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kPBlock = 16;                 // tokens per KV block
constexpr float kPMinusBig = -1e30f;
constexpr float kPRescaleLog2 = 8.f;
constexpr int kPRsrcWord3 = 0x00020000;     // buffer descriptor word 3: 32-bit raw access
constexpr int kQW = 2;                      // 16-row query tiles per wave
constexpr int kKB = 2;                      // KV blocks per LDS stage (one barrier each)
constexpr int kWavesPerEu = 3;              // waves per SIMD the register budget is fitted to
constexpr int kQTile = 16 * kQW * kPWaves;  // query rows per workgroup of one head

struct PrefillArgs {
  float* out;
  const char* q;
  const char* k;
  const char* v;
  const int32_t* tables;
  const int32_t* qstart;       // [B + 1]
  const int32_t* lens;         // [B]
  int32_t num_tokens;          // rows of q and out
  int32_t max_blocks, max_query_len, hq, hkv, num_blocks;
  int32_t hg;                  // query heads per workgroup (1, 2 or 4; divides hq / hkv)
  float scale_log2;
};

// Max over the lanes t, t + 16, t + 32 and t + 48 of a wave (every lane gets
// it), with the gfx950 lane-swap instructions: swapping a value with itself
// across rows of 16 (then halves of 32) puts each lane's partner beside it,
// an exact xor-16 then xor-32 butterfly without a round trip through LDS.
__device__ __forceinline__ float max_across_rows(float x) {
  const int xi = __float_as_int(x);
  const auto a = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  const float y = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
  const int yi = __float_as_int(y);
  const auto b = __builtin_amdgcn_permlane32_swap(yi, yi, false, false);
  return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}

template <int DT, int D>
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEu, kWavesPerEu))) void prefill_mfma(PrefillArgs a) {
  using M = MfmaOps<DT>;
  constexpr int ELEM = 2;
  constexpr int KSTEPS = D / 32;
  constexpr int NT = D / 16;
  constexpr int VROW = D * ELEM + 32;              // padded LDS row (bytes)
  constexpr int SROWS = kKB * kPBlock;             // key rows per stage
  constexpr int CPR = D * ELEM / 16;               // 16-byte chunks per row
  constexpr int CHUNKS = SROWS * CPR;              // chunks per stage (K or V)
  constexpr int LPT = (CHUNKS + kPThreads - 1) / kPThreads;   // chunks per thread
  // bfloat16 keeps 8 bits of p: p goes through the MFMA as a high and a
  // low part.  float16 keeps 11, enough on its own.
  constexpr bool SPLIT = DT == PA_DTYPE_BF16;

  __shared__ __attribute__((aligned(16))) char s_k[2][SROWS * VROW];
  __shared__ __attribute__((aligned(16))) char s_v[2][SROWS * VROW];

  // Heaviest tiles first: a tile's keys grow with its index (causal), so
  // the grid dispatches the last tiles first and the cheap ones fill in.
  const int tile = gridDim.y - 1 - blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar
  const int t = lane & 15, qa = lane >> 4;
  // The workgroup takes hg query heads of one KV group over rows_wg rows:
  // wave w serves head h0 + w % hg and the 32-row block w / hg, so every
  // K/V stage staged in LDS is read for hg heads.
  const int hg = a.hg, rows_wg = kQTile / hg;
  const int h0 = blockIdx.x * hg, h = h0 + w % hg;
  const int g = h0 / (a.hq / a.hkv);
  const int q0 = a.qstart[b], q1 = a.qstart[b + 1], total = a.num_tokens;
  const int ql = q1 - q0, n = a.lens[b];
  const bool valid = ql >= 0 && ql <= a.max_query_len && ql <= n &&
                     n <= a.max_blocks * kPBlock && q0 >= 0 && q1 <= total;
  if (!valid) {
    // Invalid lengths: NaN rows for this sequence's queries (when the row
    // range itself is sane), written once by tile 0.
    if (tile == 0 && q0 >= 0 && q1 <= total && q0 <= q1)
      for (int i = tid; i < (q1 - q0) * D * hg; i += kPThreads) {
        const int r = i / (D * hg), hh = (i / D) % hg;
        a.out[(static_cast<size_t>(q0 + r) * a.hq + h0 + hh) * D + i % D] = __builtin_nanf("");
      }
    return;
  }
  const int row0 = tile * rows_wg;
  if (row0 >= ql) return;
  const int cached = n - ql;
  const int rows_here = min(rows_wg, ql - row0);
  const int last_pos_wg = cached + row0 + rows_here - 1;   // last query position of the tile
  const int nblk = last_pos_wg / kPBlock + 1;
  const int nstage = (nblk + kKB - 1) / kKB;
  // This wave's rows: kQW tiles of 16; lane t is row t of each tile.
  const int wrow0 = row0 + 16 * kQW * (w / hg);
  const int wrows = max(0, min(16 * kQW, ql - wrow0));
  const int wave_last_pos = wrows > 0 ? cached + wrow0 + wrows - 1 : -1;
  int my_pos[kQW];
  uint4 qb[kQW][KSTEPS];
#pragma unroll
  for (int u = 0; u < kQW; ++u) {
    const int row = wrow0 + 16 * u + t;
    const bool ok = 16 * u + t < wrows;
    my_pos[u] = ok ? cached + row : -1;
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j)
      qb[u][j] = ok ? *reinterpret_cast<const uint4*>(
                          a.q + ((static_cast<size_t>(q0 + row) * a.hq + h) * D + 32 * j + 8 * qa) * ELEM)
                    : make_uint4(0u, 0u, 0u, 0u);
  }

  f32x4_t acc[kQW][NT];
#pragma unroll
  for (int u = 0; u < kQW; ++u)
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[u][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Row sums of p accumulate on the matrix cores (A = ones): the sum lands
  // in every register of the query row's lanes, already reduced over keys,
  // and it uses the same rounded p as the P V product.
  float m[kQW];
  f32x4_t lsum[kQW];
#pragma unroll
  for (int u = 0; u < kQW; ++u) { m[u] = kPMinusBig; lsum[u] = f32x4_t{0.f, 0.f, 0.f, 0.f}; }

  const uint32_t row_bytes = static_cast<uint32_t>(a.hkv) * D * ELEM;
  const uint32_t block_bytes = row_bytes * kPBlock;
  const int32_t* trow = a.tables + static_cast<size_t>(b) * a.max_blocks;
  bool bad = false;
  // Stage s holds blocks kKB*s .. +kKB-1; thread tid moves chunks tid,
  // tid + 256, ... (row = chunk / CPR within the stage).  K/V are read with
  // buffer loads: a scalar descriptor per block (base = block start, range
  // = one block) and a lane offset that does not change from stage to
  // stage.  A key past the tile's last query position gets the offset just
  // past the block, which the hardware's range check turns into zeros, so
  // neither NaN poison nor a block outside the tile's range reaches the
  // MFMAs and nothing waits on the loads before the stage's compute.  The
  // chunks of one load index all lie in one block (a row of chunks spans
  // 2*D bytes of 16-byte chunks), so the block is wave-uniform.
  static_assert(CHUNKS % kPThreads == 0, "whole chunks per thread");
  uint32_t coff[LPT];
  int crow[LPT], cblk[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int c = tid + i * kPThreads;
    crow[i] = c / CPR;
    cblk[i] = __builtin_amdgcn_readfirstlane(crow[i] / kPBlock);
    coff[i] = (crow[i] % kPBlock) * row_bytes + static_cast<uint32_t>(g * D * ELEM) + (c % CPR) * 16;
  }
  uint4 kr[LPT], vr[LPT];
  auto load = [&](int stage) {
    int32_t ids[kKB];
#pragma unroll
    for (int bb = 0; bb < kKB; ++bb) {
      const int j = stage * kKB + bb;
      const int32_t e = j < nblk ? trow[j] : 0;
      const bool ok = e >= 0 && e < a.num_blocks;
      bad |= !ok;
      ids[bb] = ok ? e : 0;
    }
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      int32_t id = ids[0];          // select, not an indexed (scratch) array
#pragma unroll
      for (int q = 1; q < kKB; ++q) id = cblk[i] == q ? ids[q] : id;
      const size_t boff = static_cast<size_t>(id) * block_bytes;
      const auto kd = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a.k + boff), 0,
                                                        static_cast<int>(block_bytes), kPRsrcWord3);
      const auto vd = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a.v + boff), 0,
                                                        static_cast<int>(block_bytes), kPRsrcWord3);
      const uint32_t off = stage * SROWS + crow[i] <= last_pos_wg ? coff[i] : block_bytes;
      kr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kd, off, 0, 0));
      vr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vd, off, 0, 0));
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = tid + i * kPThreads;
      const int off = (c / CPR) * VROW + (c % CPR) * 16;
      *reinterpret_cast<uint4*>(s_k[buf] + off) = kr[i];
      *reinterpret_cast<uint4*>(s_v[buf] + off) = vr[i];
    }
  };
  typedef typename M::lds_x4 lds_x4;
  constexpr uint32_t kOne2 = DT == PA_DTYPE_F16 ? 0x3C003C00u : 0x3F803F80u;   // two 1.0s
  const uint4 kOnes = make_uint4(kOne2, kOne2, kOne2, kOne2);

  load(0);
  stash(0);
  __syncthreads();
  for (int st = 0; st < nstage; ++st) {
    const int buf = st & 1;
    if (st + 1 < nstage) load(st + 1);
    const int key_base = st * SROWS;
    if (key_base <= wave_last_pos) {
      // Scores of every (block, query tile) of the stage first.
      f32x4_t sacc[kKB][kQW];
#pragma unroll
      for (int bb = 0; bb < kKB; ++bb) {
#pragma unroll
        for (int u = 0; u < kQW; ++u) sacc[bb][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const uint4 kk = *reinterpret_cast<const uint4*>(
              s_k[buf] + (bb * kPBlock + t) * VROW + (32 * s + 8 * qa) * ELEM);
#pragma unroll
          for (int u = 0; u < kQW; ++u) sacc[bb][u] = M::qk(kk, qb[u][s], sacc[bb][u]);
        }
      }
      // One softmax update over the stage's keys, per query tile.  Scores
      // stay unscaled (scale > 0, so the max commutes with it) and the
      // causal mask is only applied where the stage reaches past a row's
      // position: a full wave whose first row is at or after the stage's
      // last key needs none.
      const bool no_mask = wrows == 16 * kQW && cached + wrow0 >= key_base + SROWS - 1;
      float sc[kKB][kQW][4];
#pragma unroll
      for (int bb = 0; bb < kKB; ++bb)
#pragma unroll
        for (int u = 0; u < kQW; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[bb][u][r] = sacc[bb][u][r];
      if (!no_mask) {
#pragma unroll
        for (int bb = 0; bb < kKB; ++bb)
#pragma unroll
          for (int u = 0; u < kQW; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = key_base + bb * kPBlock + 4 * qa + r;
              sc[bb][u][r] = key <= my_pos[u] ? sc[bb][u][r] : -INFINITY;
            }
      }
      float bm[kQW];
      bool grow = false;
#pragma unroll
      for (int u = 0; u < kQW; ++u) {
        float mx = -INFINITY;
#pragma unroll
        for (int bb = 0; bb < kKB; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[bb][u][r]);
        bm[u] = max_across_rows(mx) * a.scale_log2;
        grow |= bm[u] > m[u] + kPRescaleLog2;
      }
      if (__any(grow)) {
#pragma unroll
        for (int u = 0; u < kQW; ++u) {
          const float mn = fmaxf(m[u], bm[u]);
          const float alpha = fast_exp2(m[u] - mn);
          m[u] = mn;
          lsum[u] *= alpha;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[u][nt] *= alpha;
        }
      }
      uint2 ph[kKB][kQW], pl[kKB][kQW];
#pragma unroll
      for (int bb = 0; bb < kKB; ++bb)
#pragma unroll
        for (int u = 0; u < kQW; ++u) {
          float p[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) p[r] = fast_exp2(fmaf(sc[bb][u][r], a.scale_log2, -m[u]));
          M::split(p, ph[bb][u], pl[bb][u]);
        }
      // O^T += V^T P^T with the K=32 MFMA over two blocks at once (the
      // K=16 form runs at half the rate on gfx950): the reduction index k =
      // 8qa + e stands for key 4qa + e of the pair's first block (e < 4) and
      // of its second block (e >= 4), in both operands -- two transposed V
      // reads side by side as A, the lane's p values of both blocks as B.
      // Each V read feeds every query tile.
      static_assert(kKB % 2 == 0, "blocks are taken in pairs");
#pragma unroll
      for (int bp = 0; bp < kKB; bp += 2) {
        lds_x4* tr0 = (lds_x4*)((__attribute__((address_space(3))) char*)(s_v[buf]) +
                                (bp * kPBlock + 4 * qa + (t >> 2)) * VROW + 8 * (t & 3));
        lds_x4* tr1 = (lds_x4*)((__attribute__((address_space(3))) char*)tr0 + kPBlock * VROW);
        uint4 pb[kQW], pbl[kQW];
#pragma unroll
        for (int u = 0; u < kQW; ++u) {
          pb[u] = make_uint4(ph[bp][u].x, ph[bp][u].y, ph[bp + 1][u].x, ph[bp + 1][u].y);
          pbl[u] = make_uint4(pl[bp][u].x, pl[bp][u].y, pl[bp + 1][u].x, pl[bp + 1][u].y);
          lsum[u] = M::qk(kOnes, pb[u], lsum[u]);
          if constexpr (SPLIT) lsum[u] = M::qk(kOnes, pbl[u], lsum[u]);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint2 v0 = M::read_tr(tr0 + 4 * nt), v1 = M::read_tr(tr1 + 4 * nt);
          const uint4 vt = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
          for (int u = 0; u < kQW; ++u) {
            acc[u][nt] = M::qk(vt, pb[u], acc[u][nt]);
            if constexpr (SPLIT) acc[u][nt] = M::qk(vt, pbl[u], acc[u][nt]);
          }
        }
      }
    }
    if (st + 1 < nstage) stash(buf ^ 1);
    __syncthreads();
  }
  // The rest of the sequence's table too, so a bad entry anywhere in it
  // gives NaN rows for the whole sequence, whichever tile reaches it.
  // Every thread reads the same entries, so `bad` is uniform.
  for (int j = nblk; j < (n + kPBlock - 1) / kPBlock; ++j) {
    const int32_t e = trow[j];
    bad |= !(e >= 0 && e < a.num_blocks);
  }

#pragma unroll
  for (int u = 0; u < kQW; ++u) {
    const float l = lsum[u][0];
    if (16 * u + t < wrows) {
      const float inv = 1.f / l;
      float* orow = a.out + (static_cast<size_t>(q0 + wrow0 + 16 * u + t) * a.hq + h) * D;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float4 o;
        o.x = bad ? __builtin_nanf("") : acc[u][nt][0] * inv;
        o.y = bad ? __builtin_nanf("") : acc[u][nt][1] * inv;
        o.z = bad ? __builtin_nanf("") : acc[u][nt][2] * inv;
        o.w = bad ? __builtin_nanf("") : acc[u][nt][3] * inv;
        *reinterpret_cast<float4*>(orow + 16 * nt + 4 * qa) = o;
      }
    }
  }
}

template <int DT>
hipError_t launch_prefill(const PrefillArgs& a, int B, int D, hipStream_t st) {
  const int rows_wg = kQTile / a.hg;
  const int tiles = (a.max_query_len + rows_wg - 1) / rows_wg;
  dim3 grid(a.hq / a.hg, tiles, B);
  if (D == 64)
    prefill_mfma<DT, 64><<<grid, kPThreads, 0, st>>>(a);
  else
    prefill_mfma<DT, 128><<<grid, kPThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int pa_prefill(float* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* query_start, const int32_t* context_lens, int32_t B,
                          int32_t num_tokens, int32_t max_query_len, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                          int32_t dtype, void* stream) {
  if (B < 0 || num_tokens < 0 || max_query_len < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq < 0)
    return fail(PA_ERR_INVALID, "pa_prefill: bad sizes");
  if (num_q_heads % num_kv_heads) return fail(PA_ERR_INVALID, "pa_prefill: Hq % Hkv != 0");
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "pa_prefill: head_dim must be 64 or 128");
  if (block_size != kPBlock) return fail(PA_ERR_UNSUPPORTED, "pa_prefill: block_size must be 16");
  if (dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: float16 or bfloat16 only (matrix-core path)");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(PA_ERR_INVALID, "pa_prefill: bad scale");
  if (B == 0 || num_tokens == 0 || max_query_len == 0) { clear_error(); return PA_OK; }
  // A table of width 0 has no entries and may be NULL.
  if (!out || !q || !k_cache || !v_cache || (!block_tables && max_blocks_per_seq > 0) || !query_start ||
      !context_lens)
    return fail(PA_ERR_INVALID, "pa_prefill: null pointer");
  const int32_t group = num_q_heads / num_kv_heads;
  const int32_t hg = group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
  if (B > 65535 || (max_query_len + kQTile / hg - 1) / (kQTile / hg) > 65535)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: grid too large");
  if (static_cast<size_t>(num_kv_heads) * head_dim * 2 * kPBlock * static_cast<size_t>(num_blocks) >
      (static_cast<size_t>(1) << 47))
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: cache too large");
  if (static_cast<size_t>(num_kv_heads) * head_dim * 2 * kPBlock >= (static_cast<size_t>(1) << 31))
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: KV block larger than 2 GiB");
  if ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(q) |
       reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) & 15)
    return fail(PA_ERR_INVALID, "pa_prefill: buffers must be 16-byte aligned");
  PrefillArgs a{};
  a.out = out;
  a.q = static_cast<const char*>(q);
  a.k = static_cast<const char*>(k_cache);
  a.v = static_cast<const char*>(v_cache);
  a.tables = block_tables;
  a.qstart = query_start;
  a.lens = context_lens;
  a.num_tokens = num_tokens;
  a.max_blocks = max_blocks_per_seq;
  a.max_query_len = max_query_len;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.num_blocks = num_blocks;
  a.hg = hg;
  a.scale_log2 = scale * 1.4426950408889634f;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err = dtype == PA_DTYPE_F16 ? launch_prefill<PA_DTYPE_F16>(a, B, head_dim, st)
                                         : launch_prefill<PA_DTYPE_BF16>(a, B, head_dim, st);
  if (err != hipSuccess)
    return fail(PA_ERR_DEVICE, std::string("pa_prefill: launch failed: ") + hipGetErrorString(err));
  clear_error();
  return PA_OK;
}
