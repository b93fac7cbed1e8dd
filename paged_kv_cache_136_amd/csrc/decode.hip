// Paged decode attention for gfx950.
//
// What is computed: "qaqbuyan.com article 130", paged_attention pseudocode
// (gather a sequence's K/V through its block table, then scaled dot-product
// attention of the one query token) and kernel listing (cache layout
// [num_blocks][block_size][heads][head_dim], float output, scale
// 1/sqrt(head_dim)); slot of token pos = table[pos/bs]*bs + pos%bs ("P06 ·
// BlockManager" spec overview).  Unlike that listing, only context_len
// tokens are attended (the last block may be partly filled), the softmax is
// an online (running max / running sum) softmax so scores never need to be
// stored, and long sequences are split into partitions whose partial
// results a second kernel combines.
//
// Phase 1, vector ALU (query groups of 1 and 2, and fp32 K/V) -- one
// workgroup of 4 waves per (KV head, sequence, partition):
//   * wave w takes the partition's blocks w, w+4, w+8, ..., reading their ids
//     from the block table with scalar loads (range-checked);
//   * a token row of one KV head (head_dim elements) is read by
//     LPR = head_dim*elem/16 lanes with one 16-byte load each, so one load
//     instruction covers 64/LPR rows and a 16-token block takes 16*LPR/64
//     loads for K and as many for V; the next blocks' loads are issued
//     before the current block is consumed;
//   * QK partial dots are summed over the LPR lanes of a row with DPP;
//     every query head of the GQA group reuses the same K/V registers;
//   * running max m, sum l and output o are kept per query head in float32,
//     in the exp2 domain (q.k is scaled by scale*log2(e));
//   * the four waves' (m, l, o) are merged through LDS; a sequence with one
//     partition writes out[] directly, otherwise (m, l, o/l) go to the
//     workspace.
// Phase 1, matrix cores (query groups of 4 and 8, 16-bit K/V): QK^T and PV
//   as MFMAs; a workgroup takes four consecutive partitions of one (KV
//   head, sequence), its waves take their blocks in turn, two in flight
//   each, and the four waves' results are merged before one partial row is
//   written (decode_phase1_mfma).
// Shared-prefix plans add a matrix-core pass over each group's shared
//   partitions, read once for all members, before the private pass.
// pa_write_decode and pa_write_decode_shared (APPEND): the phase-1 wave
//   that reads a sequence's last block also writes the new token's K/V row
//   there, and uses it in place of what it loaded.
// Phase 2 merges the partitions: one workgroup of 4 waves per (query head,
//   sequence), or, with at most 16 partitions and at least 1024 such pairs,
//   one wave per pair and four pairs per workgroup (decode_reduce_wave).
//   It is skipped when one workgroup of the private grid holds every
//   private partition of a sequence (one partition on the vector path, four
//   on the matrix cores): phase 1 then merges the shared slots, if any, and
//   writes out[] itself.
//
// Memory traffic is dominated by K and V: 2*len*Hkv*head_dim*elem bytes per
// sequence and layer; every byte is read once.  Q, tables and partials are
// under 1% of that at the supported shapes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>

#include "device_common.hpp"
#include "mfma_ops.hpp"
#include "pagedkv.h"
#include "status.hpp"

namespace pkv {
namespace {

constexpr int kWaves = 4;          // waves per phase-1 workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kBlock = 16;         // tokens per KV block
constexpr float kLog2e = 1.4426950408889634f;
// Buffer-descriptor word 3 for raw (untyped) dword access on CDNA:
// DATA_FORMAT = 32-bit, everything else 0.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kLoadAux = 2;        // cache policy of K/V loads: nontemporal (read once)
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left at their
// maxima (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8): wait for every vector memory operation of the wave, stores included.
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kNbuf = 3;           // K/V blocks in flight per wave, vector path (groups of 1, 2)
constexpr int kNbufG4 = 1;         // same, fp32 query group of 4 (VGPR-limited)
constexpr int kNbufMfma = 2;       // same, matrix-core path (groups of 4 and 8)
constexpr int kNbufShared = 2;     // same, shared-prefix pass (a few long streams per group)
constexpr int kNbufHeads = 1;      // same, four-heads private pass (runs of at most 8 blocks):
                                   // 88 VGPRs, so five waves per SIMD hide its round trips

struct DecodeArgs {
  float* out;            // [B][Hq][D]
  float* ws_o;           // [B][Hkv][P][G][D]  partition output, normalized
  float* ws_m;           // [B][Hkv][P][G]     partition max (exp2 domain)
  float* ws_l;           // [B][Hkv][P][G]     partition sum
  const char* q;         // [B][Hq][D]
  const char* k;         // [num_blocks][16][Hkv][D]
  const char* v;
  char* k_w;             // the same caches, written by pa_write_decode only
  char* v_w;
  const int32_t* tables; // [B][max_blocks]
  const int32_t* lens;   // [B]
  int32_t max_blocks;
  int32_t max_len;
  int32_t hq, hkv;
  int32_t num_blocks;
  int32_t part_blocks;   // blocks per partition
  int32_t num_parts;     // workspace slots per (sequence, head): the split of max_len, +1 with a plan
  float scale_log2;      // scale * log2(e)
  // Shared-prefix plan (seq_group == nullptr: none).
  const int32_t* seq_group;  // [B]
  const int32_t* groups;     // [n_groups][PA_SHARED_ROW]
  int32_t n_groups;
  int32_t max_shared_parts;
  int32_t batch;             // B
  int32_t qgroup;            // query heads per KV head
  int32_t grid_parts;        // z extent of the private grid (<= the split of max_len)
  int32_t private_blocks;    // host hint: most blocks a sequence reads outside the shared
                             // pass (0: unknown); picks the private pass's wave mapping
  int32_t finish;            // 1: one workgroup of the private grid holds all of a
                             // sequence's private partitions, so phase 1 merges them with
                             // the shared slots and writes out[]; no reduce runs
  // pa_write_decode: each valid, non-empty sequence's new token (position
  // len - 1) has its K/V row here instead of in the cache; phase 1 writes
  // it to its slot and uses it (null otherwise).
  const char* k_new;         // [B][Hkv][D]
  const char* v_new;
};

__device__ __forceinline__ bool len_valid(int n, const DecodeArgs& a) {
  return n >= 0 && n <= a.max_len && (n + kBlock - 1) / kBlock <= a.max_blocks;
}

// Workgroup -> (KV head, y, z).  The hardware deals workgroups to the 8
// XCDs round-robin by linear id, and x (the head) is the fastest index, so
// with head = x every XCD would read the same head columns of every block
// (with 32 heads, XCD k gets heads k, k+8, ...: fixed 256-byte columns of
// each 8 KB row).  The head is therefore rotated by rot: every XCD still
// gets a share of every (y, z) tile, which keeps the XCDs balanced when
// tiles differ in cost (mixed lengths), while its reads spread over all
// head columns; measured 3-5% more bandwidth than head = x.  The caller
// picks rot so that sequences sharing blocks (forks, beams: same first
// block) keep one head -> XCD assignment and meet their shared blocks in
// that XCD's L2.
struct WgCoord {
  int g, y, z;
};
__device__ __forceinline__ WgCoord wg_coord(int) {
  return {static_cast<int>(blockIdx.x), static_cast<int>(blockIdx.y), static_cast<int>(blockIdx.z)};
}

__device__ __forceinline__ int rotate_head(int g, int hkv, uint32_t rot) {
  return static_cast<int>((g + rot) % hkv);
}

// The scalar reads a private-grid workgroup starts with, issued together
// so the first K/V loads wait for one round trip: the sequence's length,
// its shared-prefix group (with a plan), its first table entry (for the
// head rotation) and the table entries of
// the wave's first NBUF blocks of partition z (used when there is no
// shared-prefix plan, whose partitions start elsewhere).  Every index is
// clamped into the row and no read sits behind a branch; a table of width
// 0 is replaced by the length array (B >= 1 entries), whose values then
// serve only as a rotation, since such a table has no block to read.
template <int NBUF>
struct Prologue {
  const int32_t* trow;
  int32_t n;
  int32_t spec[NBUF];
  uint32_t rot;
  int32_t gi;            // the sequence's plan group (-1 without a plan)
};

// z: the partition the ids are read for; rot_z: the one the rotation adds
// (the workgroup's, so every wave of a workgroup takes the same head).
template <int NBUF, int WAVES = kWaves>
__device__ __forceinline__ Prologue<NBUF> prologue(const DecodeArgs& a, int b, int z, int wv,
                                                   int rot_z) {
  Prologue<NBUF> p;
  p.trow = a.max_blocks > 0 ? a.tables + static_cast<size_t>(b) * a.max_blocks : a.lens;
  const int last_idx = max(a.max_blocks, 1) - 1;
  const uint32_t e0 = static_cast<uint32_t>(p.trow[0]);
  p.n = a.lens[b];
  p.gi = a.seq_group != nullptr ? a.seq_group[b] : -1;
#pragma unroll
  for (int sl = 0; sl < NBUF; ++sl)
    p.spec[sl] = p.trow[min(z * a.part_blocks + wv + sl * WAVES, last_idx)];
  // Rotation: a hash of the first block id (sequences sharing a prefix
  // share it; unrelated ones get spread-out values, also when a free list
  // hands out blocks in order) plus the partition.
  p.rot = ((e0 * 2654435761u) >> 16) + static_cast<uint32_t>(rot_z);
  return p;
}

// Workspace row of the partial result of (sequence b, query head h,
// partition part): rows are [B][Hkv][P][G], so the G query heads of one KV
// head and partition are adjacent and a workgroup writes its partial (G
// rows of D floats, and G values of m and l) as one contiguous piece.
__device__ __forceinline__ size_t ws_row(const DecodeArgs& a, int b, int h, int part) {
  const int g = h / a.qgroup, c = h - g * a.qgroup;
  return ((static_cast<size_t>(b) * a.hkv + g) * a.num_parts + part) * a.qgroup + c;
}

// Partitions of S shared blocks: the shared kernel cuts them at the
// partition size from block 0, the last one possibly short.
__device__ __forceinline__ int shared_parts_of(int S, int part_blocks) {
  return (S + part_blocks - 1) / part_blocks;
}

// Shared leading blocks S of a group row when S is in range and leaves at
// least one private block to a sequence of nblk blocks, else 0.  Both the
// shared and the private kernels decide membership through this one rule,
// so every block of every sequence is read by exactly one of them.
__device__ __forceinline__ int shared_blocks_for(const DecodeArgs& a, const int32_t* row, int nblk) {
  const int S = row[0];
  const bool ok = S >= 1 && S < nblk && shared_parts_of(S, a.part_blocks) <= a.max_shared_parts;
  return ok ? S : 0;
}

// Blocks of sequence b read by the shared kernel (0: not a member).  gi is
// seq_group[b] (read by the caller, so it can travel with its other first
// reads); nblk is b's block count, 0 for an invalid length.
__device__ __forceinline__ int shared_start(const DecodeArgs& a, int b, int gi, int nblk) {
  if (a.seq_group == nullptr || gi < 0 || gi >= a.n_groups) return 0;
  const int32_t* row = a.groups + static_cast<size_t>(gi) * PA_SHARED_ROW;
  const int slots = PA_SHARED_MAX_MEMBERS / a.qgroup;
  bool listed = false;
  for (int sl = 0; sl < slots; ++sl) listed |= row[1 + sl] == b;
  return listed ? shared_blocks_for(a, row, nblk) : 0;
}

// Partition geometry of sequence b (nblk blocks, 0 for an invalid length).
// A member's S shared blocks fill workspace slots 0 .. Ps-1 (shared
// kernel); its private partitions start at block S, private partition i
// covering blocks S + i*pb .. and filling slot Ps + i.  A sequence in no
// group has S = Ps = 0: partition i covers blocks i*pb .. (slot i).
// `total` counts every slot (1 for an empty or invalid sequence, which
// phase 1 answers directly); with S not a multiple of pb it can exceed
// the partitions of the plain split by one.
struct SeqParts {
  int S, Ps, total;
};
__device__ __forceinline__ SeqParts seq_parts(const DecodeArgs& a, int b, int gi, int nblk) {
  const int S = shared_start(a, b, gi, nblk);
  const int Ps = shared_parts_of(S, a.part_blocks);
  const int Pp = nblk == 0 ? 1 : (nblk - S + a.part_blocks - 1) / a.part_blocks;
  return {S, Ps, Ps + Pp};
}

// Final output of a sequence from phase 1 (DecodeArgs::finish): its Ps
// shared partitions sit complete in workspace slots 0 .. Ps-1 (the shared
// kernel ran earlier on the stream) and this workgroup holds the merge of
// all its private blocks, with max M, sum L and unnormalized output O.
// The merge is the reduce's, done in place: out = (O 2^(M - Mx) +
// sum_s l_s o_s 2^(m_s - Mx)) / (L 2^(M - Mx) + sum_s l_s 2^(m_s - Mx)).
// A shared slot of weight exactly 0 (an empty marker) adds nothing, even
// where its row holds NaN; a NaN weight (a bad shared slot) keeps its NaN.
// With Ps = 0 this is O / L.
//
// Wave-cooperative: all 64 lanes call shared_tail with the same sequence,
// head, M and L.  Lane s reads slot s's (m, l), so the first 64 slots cost
// one round trip, and the rows are then read four at a time.
struct SharedTail {
  size_t row0;           // workspace row of slot 0
  int Ps;
  float Mx, f, inv;      // overall max, private factor 2^(M - Mx), 1 / total sum
  float wl;              // weight of slot `lane` (lane < Ps), unnormalized
};
// The (m, l) of the first 64 shared slots, slot `lane` in each lane: the
// finish's only reads that do not depend on the private result, so a caller
// can issue them early and let them travel with its K/V loads.
struct SlotPair {
  size_t row0;
  int Ps;
  float m0, l0;
};
__device__ __forceinline__ SlotPair shared_slots(const DecodeArgs& a, int b, int h, int Ps,
                                                 int lane) {
  SlotPair p;
  p.row0 = Ps > 0 ? ws_row(a, b, h, 0) : 0;
  p.Ps = Ps;
  const bool in0 = lane < Ps;
  const size_t G = static_cast<size_t>(a.qgroup);
  p.m0 = in0 ? a.ws_m[p.row0 + lane * G] : -INFINITY;
  p.l0 = in0 ? a.ws_l[p.row0 + lane * G] : 0.f;
  return p;
}
__device__ __forceinline__ SharedTail shared_tail(const DecodeArgs& a, const SlotPair& p, float M,
                                                  float L, int lane) {
  SharedTail t;
  t.row0 = p.row0;
  t.Ps = p.Ps;
  const size_t G = static_cast<size_t>(a.qgroup);
  float Mx = fmaxf(M, p.m0);
  for (int s = lane + 64; s < p.Ps; s += 64) Mx = fmaxf(Mx, a.ws_m[t.row0 + s * G]);
  Mx = group_max<1, 64>(Mx);
  t.wl = lane < p.Ps ? p.l0 * fast_exp2(p.m0 - Mx) : 0.f;
  float Ls = t.wl;
  for (int s = lane + 64; s < p.Ps; s += 64)
    Ls = fmaf(a.ws_l[t.row0 + s * G], fast_exp2(a.ws_m[t.row0 + s * G] - Mx), Ls);
  Ls = group_sum<1, 64>(Ls);
  t.Mx = Mx;
  t.f = fast_exp2(M - Mx);
  t.inv = 1.f / fmaf(L, t.f, Ls);
  return t;
}
__device__ __forceinline__ SharedTail shared_tail(const DecodeArgs& a, int b, int h, int Ps,
                                                  float M, float L, int lane) {
  return shared_tail(a, shared_slots(a, b, h, Ps, lane), M, L, lane);
}
// o[e], the unnormalized private output at dim d0 + e, becomes the output.
template <int D, int N>
__device__ __forceinline__ void shared_tail_apply(const DecodeArgs& a, const SharedTail& t, int d0,
                                                  float (&o)[N]) {
  const size_t G = static_cast<size_t>(a.qgroup);
#pragma unroll
  for (int e = 0; e < N; ++e) o[e] *= t.f;
  for (int s0 = 0; s0 < t.Ps; s0 += 4) {
    float w[4], v[4][N];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = s0 + u;
      // rows past Ps are not read: their loads repeat the last valid row
      const float* src = a.ws_o + (t.row0 + min(s, t.Ps - 1) * G) * D + d0;
#pragma unroll
      for (int e = 0; e < N; ++e) v[u][e] = src[e];
      float ws = s < 64 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t.wl), min(s, 63)))
                        : a.ws_l[t.row0 + s * G] * fast_exp2(a.ws_m[t.row0 + s * G] - t.Mx);
      w[u] = s < t.Ps ? ws : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < N; ++e) o[e] = fmaf(w[u], w[u] != 0.f ? v[u][e] : 0.f, o[e]);
  }
#pragma unroll
  for (int e = 0; e < N; ++e) o[e] *= t.inv;
}

// Running softmax state of one lane: every lane of a row group (the LPR
// lanes that share token rows) holds the same m and l and its own chunk of o.
// Row groups are independent until the end of the wave's work, so no lane
// exchange happens per block.  m starts at a large finite negative value so
// that a row group that has seen only masked rows stays NaN-free
// (alpha = 2^0 = 1, p = 2^-inf = 0).
constexpr float kMinusBig = -1.0e30f;
constexpr float kRescaleLog2 = 8.0f;   // lazy-rescale threshold, log2 domain

template <int DT, int D, int G>
struct RowState {
  static constexpr int EPL = 16 / ElemTraits<DT>::bytes;
  float m[G], l[G], o[G][EPL];
};

// One block: scores for the lane's LPB rows, online-softmax update, PV.
// MASKED: rows at or past valid_rows get score -inf and a zero V chunk
// (a select, so poisoned slots never reach the arithmetic).
template <int DT, int D, int G, int LPB, int RPI, bool MASKED>
__device__ __forceinline__ void consume_block(RowState<DT, D, G>& st, const uint4 (&q)[G],
                                              const uint4 (&kw)[LPB], const uint4 (&vw)[LPB],
                                              float scale_log2, int r, int valid_rows) {
  constexpr int LPR = 64 / RPI;
  float s[G][LPB];
#pragma unroll
  for (int i = 0; i < LPB; ++i) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float acc = group_sum<1, LPR>(chunk_dot<DT>(q[hh], kw[i])) * scale_log2;
      if constexpr (MASKED) acc = (i * RPI + r < valid_rows) ? acc : -INFINITY;
      s[hh][i] = acc;
    }
  }
  uint4 v[LPB];
#pragma unroll
  for (int i = 0; i < LPB; ++i) {
    v[i] = vw[i];
    if constexpr (MASKED) {
      if (i * RPI + r >= valid_rows) v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float bm = s[hh][0];
#pragma unroll
    for (int i = 1; i < LPB; ++i) bm = fmaxf(bm, s[hh][i]);
    const float mn = fmaxf(st.m[hh], bm);
    const float alpha = fast_exp2(st.m[hh] - mn);
    st.m[hh] = mn;
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < RowState<DT, D, G>::EPL; ++e) st.o[hh][e] *= alpha;
#pragma unroll
    for (int i = 0; i < LPB; ++i) {
      const float p = fast_exp2(s[hh][i] - mn);
      ps += p;
      chunk_axpy<DT>(st.o[hh], p, v[i]);
    }
    st.l[hh] = fmaf(st.l[hh], alpha, ps);
  }
}

// HEADS: the waves of a workgroup take four adjacent KV heads of one
// (sequence, partition) instead of splitting one head's blocks, and each
// writes its own result (no merge through LDS).  Used for the private pass
// of a shared-prefix plan, whose partitions are often a block or two long:
// one head per workgroup would leave three of its four waves idle there.
// APPEND (pa_write_decode, pa_write_decode_shared): the wave that reads a
// sequence's last block takes the new token's row from k_new / v_new
// instead of the cache and stores it there, once per (sequence, KV head).
// With a plan the last block is always private (never in a shared pass),
// so the private pass is the one that reads it.
template <int DT, int D, int G, int NBUF, bool HEADS = false, bool APPEND = false>
__global__ __launch_bounds__(kThreads) void decode_phase1(DecodeArgs a) {
  constexpr int ELEM = ElemTraits<DT>::bytes;
  constexpr int EPL = 16 / ELEM;          // elements per lane per load
  constexpr int LPR = D * ELEM / 16;      // lanes per token row
  constexpr int RPI = 64 / LPR;           // rows per load instruction
  constexpr int LPB = kBlock / RPI;       // loads per block (K or V)
  static_assert(LPR >= 1 && LPR <= 64 && RPI * LPR == 64 && LPB * RPI == kBlock, "shape");

  __shared__ int32_t s_bad[kWaves];
  __shared__ float s_m[kWaves][G], s_l[kWaves][G];
  __shared__ float s_o[kWaves][G][D];

  // Grid: x = KV head (rotated by wg_coord), y = sequence, z = partition.
  // Workgroups are dealt to the 8 XCDs round-robin by linear id, so the
  // fastest index must not correlate with work size: heads of one
  // (sequence, partition) cost the same, and partitions that a sequence
  // does not have (the cheap exits) collect at the end of the grid.
  // With a shared-prefix plan, a member's first partitions belong to the
  // shared kernel and z counts from the first private one.
  const WgCoord wc = wg_coord(a.hkv);
  const int b = wc.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane / LPR, c = lane % LPR;
  const int wv = __builtin_amdgcn_readfirstlane(w);
  // The wave's first block and block stride within the partition.
  constexpr int kStep = HEADS ? 1 : kWaves;
  const int w0 = HEADS ? 0 : wv;
  const Prologue<NBUF> pro = HEADS ? prologue<NBUF, 1>(a, b, wc.z, 0, wc.z)
                                   : prologue<NBUF>(a, b, wc.z, wv, wc.z);
  const int g = HEADS ? wc.g * kWaves + wv : rotate_head(wc.g, a.hkv, pro.rot);
  const int32_t* trow = pro.trow;
  const int n = pro.n;
  const bool valid = len_valid(n, a);
  const int nblk = valid ? (n + kBlock - 1) / kBlock : 0;
  const SeqParts sp = seq_parts(a, b, pro.gi, nblk);
  const int nparts = sp.total;
  const int slot = sp.Ps + wc.z;           // this private partition's workspace slot
  if (slot >= nparts) return;
  const int h0 = g * G;

  // Degenerate rows: empty sequence -> 0, invalid length -> NaN.
  if (!valid || n == 0) {
    const float fill = valid ? 0.f : __builtin_nanf("");
    for (int i = HEADS ? lane : tid; i < G * D; i += HEADS ? 64 : kThreads)
      a.out[(static_cast<size_t>(b) * a.hq + h0 + i / D) * D + i % D] = fill;
    return;
  }

  // Query chunk of every head of the group, raw (same element type as K).
  uint4 q[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
    q[hh] = *reinterpret_cast<const uint4*>(
        a.q + ((static_cast<size_t>(b) * a.hq + h0 + hh) * D + c * EPL) * ELEM);

  RowState<DT, D, G> st;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    st.m[hh] = kMinusBig;
    st.l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) st.o[hh][e] = 0.f;
  }

  // K/V rows are read with buffer loads: a scalar descriptor per block
  // (base = block start, range = one block, so the hardware bounds-checks
  // every access), one VGPR lane offset, and the row stride of load i in the
  // scalar offset.
  const uint32_t row_bytes = static_cast<uint32_t>(a.hkv) * D * ELEM;
  const uint32_t block_bytes = row_bytes * kBlock;
  const uint32_t lane_off = r * row_bytes + static_cast<uint32_t>(g * D + c * EPL) * ELEM;

  const int first = sp.S + wc.z * a.part_blocks;
  const int last = min(nblk, first + a.part_blocks);   // exclusive
  // Block ids come straight from the table with scalar loads (uniform
  // addresses, served by the scalar cache; tables are tiny and stay in L2),
  // so a wave starts streaming without any LDS staging or barrier.  An id
  // outside the pool is replaced by block 0 (never read out of range) and
  // flags the sequence; its output becomes NaN after the merge.
  // A grid sized below this sequence's private partitions (a host bound
  // that was too small) leaves some uncomputed: flag it like a bad id.
  bool bad_ids = nparts - sp.Ps > static_cast<int>(gridDim.z);
  auto check_id = [&](int32_t e) -> int {
    const bool ok = e >= 0 && e < a.num_blocks;
    bad_ids |= !ok;
    return ok ? e : 0;
  };
  auto block_id = [&](int j) -> int { return check_id(trow[j]); };

  auto load_block = [&](int blk, uint4 (&kw)[LPB], uint4 (&vw)[LPB]) {
    const size_t boff = static_cast<size_t>(blk) * block_bytes;
    const auto kd = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a.k + boff), 0,
                                                      static_cast<int>(block_bytes), kRsrcWord3);
    const auto vd = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a.v + boff), 0,
                                                      static_cast<int>(block_bytes), kRsrcWord3);
#pragma unroll
    for (int i = 0; i < LPB; ++i)
      kw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            kd, lane_off, i * RPI * row_bytes, kLoadAux));
#pragma unroll
    for (int i = 0; i < LPB; ++i)
      vw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            vd, lane_off, i * RPI * row_bytes, kLoadAux));
  };
  // APPEND: the wave that reads the sequence's last block (lb) loads the new
  // token's row (len - 1) of head g from k_new / v_new before its first
  // K/V loads, stores it to the cache right after issuing them (when the
  // block id is valid: an invalid one flags the sequence and writes
  // nothing), and takes it into the loaded registers in place of whatever
  // its own load of that block returns.  Nothing else reads that row in
  // this launch.  Storing early keeps the store's completion off the wave's
  // critical path (the merge barrier waits for outstanding stores).
  // HEADS keeps the row in LDS rather than in registers through the ring,
  // which holds it to five waves per SIMD.
  const int lb = nblk - 1;
  const bool has_last = APPEND && lb >= first + w0 && lb < last && (lb - first - w0) % kStep == 0;
  const int nr = n - 1 - lb * kBlock;      // the new row within block lb
  __shared__ uint4 s_new[APPEND && HEADS ? kWaves : 1][2][64];
  uint4 knew{}, vnew{};
  if (has_last) {
    const size_t src = ((static_cast<size_t>(b) * a.hkv + g) * D + c * EPL) * ELEM;
    knew = *reinterpret_cast<const uint4*>(a.k_new + src);
    vnew = *reinterpret_cast<const uint4*>(a.v_new + src);
  }
  auto consume = [&](const uint4 (&kw)[LPB], const uint4 (&vw)[LPB], int gblk) {
    const int vr = n - gblk * kBlock;
    if (vr >= kBlock)
      consume_block<DT, D, G, LPB, RPI, false>(st, q, kw, vw, a.scale_log2, r, kBlock);
    else
      consume_block<DT, D, G, LPB, RPI, true>(st, q, kw, vw, a.scale_log2, r, vr);
  };

  // HEADS with the finish: the shared slots' (m, l) go out with the first
  // K/V loads (the finish would otherwise start with that round trip).
  SlotPair pre[HEADS ? G : 1];
  if constexpr (HEADS) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) pre[hh] = shared_slots(a, b, h0 + hh, a.finish ? sp.Ps : 0, lane);
  }

  // This wave's blocks are first+wv, first+wv+4, ... (HEADS: every block
  // of the partition); NBUF of them are in flight in a register ring (the
  // loop is unrolled by NBUF so each ring slot is a fixed set of registers).
  uint4 kr[NBUF][LPB], vr[NBUF][LPB];
#pragma unroll
  for (int sl = 0; sl < NBUF; ++sl) {
    const int jj = first + w0 + sl * kStep;
    if (jj < last) load_block(check_id(a.seq_group == nullptr ? pro.spec[sl] : trow[jj]), kr[sl], vr[sl]);
  }
  if (has_last) {
    const int32_t id = trow[lb];
    if (r == nr % RPI && id >= 0 && id < a.num_blocks) {
      const size_t off = static_cast<size_t>(id) * block_bytes + static_cast<size_t>(nr) * row_bytes +
                         static_cast<size_t>(g * D + c * EPL) * ELEM;
      *reinterpret_cast<uint4*>(a.k_w + off) = knew;
      *reinterpret_cast<uint4*>(a.v_w + off) = vnew;
    }
    if constexpr (HEADS) {
      s_new[wv][0][lane] = knew;
      s_new[wv][1][lane] = vnew;
    }
  }
  for (int j = first + w0; j < last; j += NBUF * kStep) {
#pragma unroll
    for (int sl = 0; sl < NBUF; ++sl) {
      const int jj = j + sl * kStep;
      if (jj < last) {
        if constexpr (APPEND) {
          if (jj == lb) {
            // (HEADS: K, then V, back from LDS, one at a time)
            const uint4 kn = HEADS ? s_new[wv][0][lane] : knew;
#pragma unroll
            for (int i = 0; i < LPB; ++i) kr[sl][i] = select4(i * RPI + r == nr, kn, kr[sl][i]);
            const uint4 vn = HEADS ? s_new[wv][1][lane] : vnew;
#pragma unroll
            for (int i = 0; i < LPB; ++i) vr[sl][i] = select4(i * RPI + r == nr, vn, vr[sl][i]);
          }
        }
        consume(kr[sl], vr[sl], jj);
        const int jn = jj + NBUF * kStep;
        if (jn < last) load_block(block_id(jn), kr[sl], vr[sl]);
      }
    }
  }

  // Wave result: merge the RPI row groups (each with its own running max).
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float M = group_max<LPR, 64>(st.m[hh]);
    const float f = fast_exp2(st.m[hh] - M);
    st.l[hh] = group_sum<LPR, 64>(st.l[hh] * f);
#pragma unroll
    for (int e = 0; e < EPL; ++e) st.o[hh][e] = group_sum<LPR, 64>(st.o[hh][e] * f);
    st.m[hh] = M;
  }
  if constexpr (HEADS) {
    // The wave's result is final: row group 0 writes it (m and l are the
    // same in every lane after the merge above).
    if (a.finish) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const SharedTail tl = shared_tail(a, pre[hh], st.m[hh], st.l[hh], lane);
        if (r == 0) {
          const size_t bh = static_cast<size_t>(b) * a.hq + h0 + hh;
          float o[EPL];
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[e] = st.o[hh][e];
          shared_tail_apply<D>(a, tl, c * EPL, o);
#pragma unroll
          for (int e = 0; e < EPL; ++e) a.out[bh * D + c * EPL + e] = bad_ids ? __builtin_nanf("") : o[e];
        }
      }
      return;
    }
    if (r == 0) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const size_t bh = static_cast<size_t>(b) * a.hq + h0 + hh;
        const float inv = 1.f / st.l[hh];
        const size_t bhp = nparts == 1 ? 0 : ws_row(a, b, h0 + hh, slot);
        float* dst = nparts == 1 ? a.out + bh * D : a.ws_o + bhp * D;
#pragma unroll
        for (int e = 0; e < EPL; ++e)
          dst[c * EPL + e] = bad_ids ? __builtin_nanf("") : st.o[hh][e] * inv;
        if (nparts > 1 && c == 0) {
          a.ws_m[bhp] = bad_ids ? 0.f : st.m[hh];
          a.ws_l[bhp] = bad_ids ? __builtin_nanf("") : st.l[hh];
        }
      }
    }
    return;
  }
  if (r == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[w][hh][c * EPL + e] = st.o[hh][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      s_m[w][hh] = st.m[hh];
      s_l[w][hh] = st.l[hh];
    }
    s_bad[w] = bad_ids;
  }
  __syncthreads();

  const bool bad = (s_bad[0] | s_bad[1] | s_bad[2] | s_bad[3]) != 0;
  for (int i = tid; i < G * D; i += kThreads) {
    const int hh = i / D, d = i % D;
    float M = s_m[0][hh];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww][hh]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = fast_exp2(s_m[ww][hh] - M);   // 0 for a wave with no block
      L = fmaf(s_l[ww][hh], f, L);
      O = fmaf(s_o[ww][hh][d], f, O);
    }
    const size_t bh = static_cast<size_t>(b) * a.hq + h0 + hh;
    if (a.finish) {
      // every lane of the wave is here (G * D is a multiple of 64), with
      // the same head
      float o[1] = {O};
      shared_tail_apply<D>(a, shared_tail(a, b, h0 + hh, sp.Ps, M, L, lane), d, o);
      a.out[bh * D + d] = bad ? __builtin_nanf("") : o[0];
      continue;
    }
    const float res = bad ? __builtin_nanf("") : O / L;
    if (nparts == 1) {
      a.out[bh * D + d] = res;
    } else {
      const size_t bhp = ws_row(a, b, h0 + hh, slot);
      a.ws_o[bhp * D + d] = res;
      if (d == 0) {
        a.ws_m[bhp] = bad ? 0.f : M;
        a.ws_l[bhp] = bad ? __builtin_nanf("") : L;
      }
    }
  }
}

// ---- Phase 1 on the matrix cores: query groups of 4 or 8, 16-bit K/V ------
// With G query heads per KV head the block's QK^T and PV are small
// contractions (16 tokens x D x G), so they run as MFMAs and the vector ALU
// keeps only the softmax.  Lane coordinates: t = lane % 16, qa = lane / 16.
//  QK   S = K Q^T with v_mfma_f32_16x16x32: A = K (token t, dims 32j+8qa..),
//       B = Q^T (head t, same dims; zero for t >= G).  C: lane (qa, t),
//       reg r holds S[token 4qa+r][head t].
//  softmax  per lane = per head t; the block max is reduced over the four
//       qa lanes of a head (2 lane exchanges per block for all heads).
//  PV   O^T = V^T P^T with v_mfma_f32_16x16x16: A = V^T for 16 dims (read
//       from a wave-private LDS copy of the block with ds_read_tr16_b64),
//       B = P^T, which is exactly the lane's four p values.  P is split into
//       high and low 16-bit parts (two MFMAs) so the 16-bit rounding of P
//       (2^-9 for bf16) does not reach the output (2^-18 after the split).
//       C: lane (qa, t), reg r holds O[head t][dim 16n + 4qa + r], so the
//       rescale by alpha is lane-local.
// Work split: four partitions per workgroup, merged once.  A workgroup of
//       4 waves takes 4 consecutive partitions (grid z = partitions / 4),
//       and wave w streams blocks w, w+4, w+8, ... of their range, with no
//       barrier until its blocks are done.  The four results are then merged
//       through LDS (each wave's staging space is free by then) and written
//       once, at the group's first partition; the other three partitions
//       get only m = -big, l = 0, which the reduce skips.  Writing every
//       partition's G output rows instead cost the long GQA batch ~12% of
//       its read bandwidth for 0.8% more bytes; with four waves splitting
//       each partition the cost is per workgroup as well, and this form has
//       a quarter as many.  (Giving each wave one whole partition instead
//       of every fourth block measured ~1% slower.)
// SHARED: the workgroups run over (KV head, plan group, shared partitions).
//       The 16 query columns are (member slot t / qgroup, query head
//       t % qgroup) of the group's members, the blocks come from the table
//       row of the group's first slot, and each column's (m, l, o) goes to
//       its member's workspace row.  Every member checks that its own table
//       holds the same ids over the partition (NaN output otherwise).
template <int DT, int D, int G, int NBUF, bool SHARED, bool APPEND = false>
__global__ __launch_bounds__(kThreads) void decode_phase1_mfma(DecodeArgs a) {
  static_assert(!(SHARED && APPEND), "the shared pass never reads a last block");
  static_assert(DT != PA_DTYPE_F32 && (D == 64 || D == 128), "shape");
  static_assert(SHARED ? G == 16 : (G == 4 || G == 8), "query columns");
  using M = MfmaOps<DT>;
  constexpr int ELEM = 2;
  constexpr int KSTEPS = D / 32;          // QK MFMAs per block
  constexpr int NT = D / 16;              // PV dim tiles per block
  constexpr int LPR = D * ELEM / 16;      // lanes per row in the V row loads
  constexpr int RPI = 64 / LPR;           // rows per V load instruction
  constexpr int VLOADS = kBlock / RPI;    // V loads per block
  constexpr int VROW = D * ELEM + 32;     // padded LDS row (bytes)

  // Per wave: V rows, then K rows, while streaming; the wave's unnormalized
  // result (16 columns x D, padded rows) plus m, l and a bad flag per
  // column once its partition is done.
  constexpr int WBYTES = 2 * kBlock * VROW;
  constexpr int OROW = D + 4;             // floats per staged output row (bank stagger)
  static_assert(16 * OROW * 4 + 3 * 16 * 4 <= WBYTES, "merge staging fits the K/V staging");
  __shared__ __attribute__((aligned(16))) char s_wave[kWaves][WBYTES];
  __shared__ int32_t s_colseq[16];

  const WgCoord wc = wg_coord(a.hkv);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int t = lane & 15, qa = lane >> 4;
  const int zp = wc.z * kWaves + w;       // this wave's partition, counted in the grid
  // Private grid: the prologue's reads (length, rotation, first ids).  The
  // shared grid reads each block once, so it rotates by (group, z).  The
  // rotation is the workgroup's: its four waves take the same head, which
  // the merge below relies on.
  Prologue<NBUF> pro{};
  if constexpr (!SHARED) pro = prologue<NBUF, kWaves>(a, wc.y, wc.z * kWaves, w, wc.z);
  const int g = rotate_head(wc.g, a.hkv, SHARED ? wc.y + wc.z : pro.rot);
  const int h0 = g * (SHARED ? a.qgroup : G);
  // b: sequence (private) or plan group (shared).  n: tokens the blocks
  // [first, last) are cut from; trow: the table row they are read from.
  int b = wc.y, part, n, nblk, nparts, first, last;
  int ps = 0;                             // private: the sequence's shared slots
  bool short_grid = false;
  const int32_t* trow;
  // SHARED: column t's member (-1 if none); the member slot this lane
  // checks (slot t); whether the group's source row is usable.
  int col_seq = -1, chk_seq = -1;
  bool src_ok = true;
  // Waves whose partition does not exist stream nothing but still take
  // part in the merge (the barrier needs every wave).
  bool active;
  int p0, pend;                           // the group's partitions: [p0, pend)
  if constexpr (SHARED) {
    const int32_t* row = a.groups + static_cast<size_t>(b) * PA_SHARED_ROW;
    const int S = row[0];                 // shared blocks
    part = zp;
    p0 = wc.z * kWaves;
    // uniform over the workgroup (S is checked before its partitions are
    // counted, so a wild value cannot overflow them)
    if (S < 1 || S > static_cast<int64_t>(a.max_shared_parts) * a.part_blocks) return;
    const int P = shared_parts_of(S, a.part_blocks);
    if (p0 >= P) return;
    pend = min(P, p0 + kWaves);
    active = true;
    const int slots = PA_SHARED_MAX_MEMBERS / a.qgroup;
    // Membership as the private kernels decide it.
    auto member = [&](int sl) -> int {
      if (sl >= slots) return -1;
      const int m = row[1 + sl];
      if (m < 0 || m >= a.batch || a.seq_group[m] != b) return -1;
      const int nm = a.lens[m];
      if (!len_valid(nm, a)) return -1;
      return shared_blocks_for(a, row, (nm + kBlock - 1) / kBlock) > 0 ? m : -1;
    };
    col_seq = member(t / a.qgroup);
    chk_seq = member(t);
    if (!__any(col_seq >= 0)) return;     // no column has a member (uniform)
    const int lead = row[1];
    src_ok = lead >= 0 && lead < a.batch;
    trow = a.tables + static_cast<size_t>(src_ok ? lead : 0) * a.max_blocks;
    // The workgroup's partitions [p0, pend), their blocks dealt to the
    // waves in turn, so a group with fewer than four partitions still
    // keeps every wave streaming (within max_blocks: a member exists).
    first = p0 * a.part_blocks;
    last = src_ok ? min(pend * a.part_blocks, S) : first;
    n = last * kBlock;                               // shared blocks are full
    nblk = last;
    nparts = 0;
  } else {
    const int nn = pro.n;
    const bool valid = len_valid(nn, a);
    n = nn;
    nblk = valid ? (n + kBlock - 1) / kBlock : 0;
    const SeqParts sp = seq_parts(a, b, pro.gi, nblk);
    nparts = sp.total;
    ps = sp.Ps;
    // the workgroup streams private partitions p0 .. pend-1 (slots Ps +
    // ...); its merged result goes to its first slot p0
    part = sp.Ps + zp;
    p0 = sp.Ps + wc.z * kWaves;
    if (p0 >= nparts) return;             // uniform over the workgroup
    pend = min(nparts, p0 + kWaves);
    active = true;
    short_grid = nparts - sp.Ps > static_cast<int>(gridDim.z) * kWaves;
    if (!valid || n == 0) {               // uniform: nparts == 1, p0 == 0
      const float fill = valid ? 0.f : __builtin_nanf("");
      for (int i = threadIdx.x; i < G * D; i += kThreads)
        a.out[(static_cast<size_t>(b) * a.hq + h0 + i / D) * D + i % D] = fill;
      return;
    }
    trow = pro.trow;
    // the workgroup's partitions [p0, pend), their blocks dealt to the
    // waves in turn
    first = sp.S + (p0 - sp.Ps) * a.part_blocks;
    last = min(nblk, sp.S + (pend - sp.Ps) * a.part_blocks);
  }

  // Q^T as the QK B operand: column t, dims 32j + 8qa .. +8 (zero for a
  // column without a query head).
  const int qhead = SHARED ? h0 + t % a.qgroup : h0 + t;
  const int qseq = SHARED ? col_seq : (t < G ? b : -1);
  uint4 qb[KSTEPS];
#pragma unroll
  for (int j = 0; j < KSTEPS; ++j)
    qb[j] = qseq >= 0 ? *reinterpret_cast<const uint4*>(
                            a.q + ((static_cast<size_t>(qseq) * a.hq + qhead) * D + 32 * j + 8 * qa) * ELEM)
                      : make_uint4(0u, 0u, 0u, 0u);

  f32x4_t acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kMinusBig, lsum = 0.f;

  const uint32_t row_bytes = static_cast<uint32_t>(a.hkv) * D * ELEM;
  const uint32_t block_bytes = row_bytes * kBlock;
  // K and V are loaded in row layout (token i*RPI + vr, dims 8vc .. +8)
  // and K is re-read from LDS in the MFMA A layout.
  const int vr = lane / LPR, vc = lane % LPR;
  const uint32_t v_off = vr * row_bytes + static_cast<uint32_t>(g * D + 8 * vc) * ELEM;
  char* lds_v = s_wave[w];
  char* lds_k = s_wave[w] + kBlock * VROW;
  typedef typename M::lds_x4 lds_x4;
  // Transpose-read address: lane 16qa + 4e + q points at the 4 dims
  // 16n + 4q .. +3 of token 4qa + e; the instruction then hands lane
  // 16qa + j the four tokens 4qa .. 4qa+3 of dim 16n + j.
  lds_x4* tr_base = (lds_x4*)((__attribute__((address_space(3))) char*)(s_wave[w]) +
                              (4 * qa + (t >> 2)) * VROW + 8 * (t & 3));

  // Block ids come straight from the table with scalar loads (uniform
  // addresses, served by the scalar cache; tables are tiny and stay in L2).
  // An id outside the pool is replaced by block 0 (never read out of range)
  // and flags the partition; its output becomes NaN.
  bool bad_ids = short_grid;
  auto check_id = [&](int32_t e) -> int {
    const bool ok = e >= 0 && e < a.num_blocks;
    bad_ids |= !ok;
    return ok ? e : 0;
  };
  auto block_id = [&](int j) -> int { return check_id(trow[j]); };

  auto load_block = [&](int blk, uint4 (&kw)[KSTEPS], uint4 (&vw)[VLOADS]) {
    const size_t boff = static_cast<size_t>(blk) * block_bytes;
    const auto kd = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a.k + boff), 0,
                                                      static_cast<int>(block_bytes), kRsrcWord3);
    const auto vd = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a.v + boff), 0,
                                                      static_cast<int>(block_bytes), kRsrcWord3);
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j)
      kw[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            kd, v_off, j * RPI * row_bytes, kLoadAux));
#pragma unroll
    for (int i = 0; i < VLOADS; ++i)
      vw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            vd, v_off, i * RPI * row_bytes, kLoadAux));
  };

  auto consume = [&](const uint4 (&kw)[KSTEPS], const uint4 (&vw)[VLOADS], int gblk) {
    const int valid_rows = min(kBlock, n - gblk * kBlock);
    // V block -> wave-private LDS rows (rows past the length as zeros, so
    // poisoned slots never meet a zero weight inside the MFMA).
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int row = i * RPI + vr;
      const uint4 val = row < valid_rows ? vw[i] : make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(lds_v + row * VROW + 16 * vc) = val;
    }
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
    // K rows through LDS too: row-layout loads, MFMA-layout reads.
    static_assert(KSTEPS == VLOADS, "K row loads reuse the V row mapping");
#pragma unroll
    for (int i = 0; i < VLOADS; ++i)
      *reinterpret_cast<uint4*>(lds_k + (i * RPI + vr) * VROW + 16 * vc) = kw[i];
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      const uint4 kk = *reinterpret_cast<const uint4*>(lds_k + t * VROW + (32 * j + 8 * qa) * ELEM);
      sacc = M::qk(kk, qb[j], sacc);
    }
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (4 * qa + r < valid_rows) ? sacc[r] * a.scale_log2 : -INFINITY;
    float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    bm = group_max<16, 64>(bm);
    // Lazy rescaling: the running max moves only when some head's block max
    // exceeds it by more than 2^kRescaleLog2 (p then stays <= 2^8).  One
    // wave-uniform test covers every head, and the common path leaves the
    // accumulators to the MFMAs alone.
    if (__any(bm > m + kRescaleLog2)) {
      const float mn = fmaxf(m, bm);
      const float alpha = fast_exp2(m - mn);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(sc[r] - m);
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    uint2 ph, pl;
    M::split(p, ph, pl);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint2 vt = M::read_tr(tr_base + 4 * nt);   // 16 dims = 32 bytes = 4 x 8 B
      acc[nt] = M::pv(vt, ph, acc[nt]);
      acc[nt] = M::pv(vt, pl, acc[nt]);
    }
  };

  // The wave's blocks in order, NBUF of them in flight: blocks w, w+4, ...
  // of the workgroup's range (its four partitions, or fewer).
  constexpr int kStep = kWaves;
  const int w0 = w;
  // APPEND: the wave that reads the sequence's last block first stores the
  // new token's row of head g there (the lanes of row len - 1, each its
  // 16-byte chunk, dims 8vc .. +8, when the block id is valid: an invalid
  // one flags the sequence and writes nothing), waits for the stores, and
  // then reads the row back with its other loads; no other wave reads that
  // row in this launch.  (Taking the row into the loaded registers instead,
  // as the vector kernel does, costs this kernel a wave per SIMD.)
  if constexpr (APPEND) {
    const int lb = nblk - 1;
    if (lb >= first + w0 && lb < last && (lb - first - w0) % kStep == 0) {
      const int nr = n - 1 - lb * kBlock;
      const int32_t id = trow[lb];
      if (vr == nr % RPI && id >= 0 && id < a.num_blocks) {
        const size_t src = ((static_cast<size_t>(b) * a.hkv + g) * D + 8 * vc) * ELEM;
        const size_t off = static_cast<size_t>(id) * block_bytes + static_cast<size_t>(nr) * row_bytes +
                           static_cast<size_t>(g * D + 8 * vc) * ELEM;
        *reinterpret_cast<uint4*>(a.k_w + off) = *reinterpret_cast<const uint4*>(a.k_new + src);
        *reinterpret_cast<uint4*>(a.v_w + off) = *reinterpret_cast<const uint4*>(a.v_new + src);
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
  }
  uint4 kr[NBUF][KSTEPS], vrg[NBUF][VLOADS];
#pragma unroll
  for (int sl = 0; sl < NBUF; ++sl) {
    const int jj = first + w0 + sl * kStep;
    if (jj < last)
      load_block(check_id(!SHARED && a.seq_group == nullptr ? pro.spec[sl] : trow[jj]), kr[sl],
                 vrg[sl]);
  }
  for (int j = first + w0; j < last; j += NBUF * kStep) {
#pragma unroll
    for (int sl = 0; sl < NBUF; ++sl) {
      const int jj = j + sl * kStep;
      if (jj < last) {
        consume(kr[sl], vrg[sl], jj);
        const int jn = jj + NBUF * kStep;
        if (jn < last) load_block(block_id(jn), kr[sl], vrg[sl]);
      }
    }
  }

  // Result of column t: m is uniform over the four qa lanes, and their
  // partial sums add up.
  lsum = group_sum<16, 64>(lsum);
  bool bad = bad_ids || !src_ok;
  if constexpr (SHARED) {
    // Member slot t's own table must hold the source row's ids over the
    // wave's blocks: lane qa of slot t compares blocks w + 4qa, +16, ...
    // (the four waves together cover [first, last)).
    bool mismatch = false;
    if (chk_seq >= 0 && src_ok) {
      const int32_t* mrow = a.tables + static_cast<size_t>(chk_seq) * a.max_blocks;
      for (int j = first + w0 + kStep * qa; j < last; j += 4 * kStep) mismatch |= mrow[j] != trow[j];
    }
    const float mis = group_max<16, 64>(mismatch ? 1.f : 0.f);   // slot t's flag, every qa lane
    bad |= __shfl(mis, t / a.qgroup) != 0.f;                      // the flag of column t's slot
  }
  // Stage this wave's result in its own staging space (its streaming is
  // over; the other waves use only theirs), then merge the four.
  float* st = reinterpret_cast<float*>(s_wave[w]);
  float* st_m = st + 16 * OROW;
  float* st_l = st_m + 16;
  int32_t* st_bad = reinterpret_cast<int32_t*>(st_l + 16);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    *reinterpret_cast<float4*>(st + t * OROW + 16 * nt + 4 * qa) =
        make_float4(acc[nt][0], acc[nt][1], acc[nt][2], acc[nt][3]);
  if (qa == 0) {
    st_m[t] = active ? m : kMinusBig;
    st_l[t] = active ? lsum : 0.f;
    st_bad[t] = active && bad;
    if (w == 0) s_colseq[t] = SHARED ? col_seq : (t < G ? b : -1);
  }
  __syncthreads();

  // Merged result of column c: M = max m_w, L = sum l_w 2^(m_w - M),
  // O = sum o_w 2^(m_w - M) (o_w unnormalized), written as O / L at the
  // group's first partition p0.
  constexpr int C = SHARED ? 16 : G;     // columns that can carry a row
  for (int i = threadIdx.x; i < C * D; i += kThreads) {
    const int c = i / D, d = i % D;
    const int oseq = s_colseq[c];
    if (oseq < 0) continue;
    const int oh = SHARED ? h0 + c % a.qgroup : h0 + c;
    float Mx = kMinusBig;
    bool badc = false;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float* sw = reinterpret_cast<const float*>(s_wave[ww]);
      Mx = fmaxf(Mx, sw[16 * OROW + c]);
      badc |= reinterpret_cast<const int32_t*>(sw + 16 * OROW + 32)[c] != 0;
    }
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float* sw = reinterpret_cast<const float*>(s_wave[ww]);
      const float f = fast_exp2(sw[16 * OROW + c] - Mx);   // 0 for a wave without a partition
      L = fmaf(sw[16 * OROW + 16 + c], f, L);
      O = fmaf(sw[c * OROW + d], f, O);
    }
    if (!SHARED && a.finish) {
      // the wave covers 64 dims of one column here, whole
      float o[1] = {O};
      shared_tail_apply<D>(a, shared_tail(a, oseq, oh, ps, Mx, L, lane), d, o);
      a.out[(static_cast<size_t>(oseq) * a.hq + oh) * D + d] = badc ? __builtin_nanf("") : o[0];
      continue;
    }
    const float res = badc ? __builtin_nanf("") : O / L;
    if (!SHARED && nparts == 1) {
      a.out[(static_cast<size_t>(oseq) * a.hq + oh) * D + d] = res;
      continue;
    }
    const size_t row = ws_row(a, oseq, oh, p0);
    a.ws_o[row * D + d] = res;
    if (d == 0) {
      a.ws_m[row] = badc ? 0.f : Mx;
      a.ws_l[row] = badc ? __builtin_nanf("") : L;
    } else if (d < pend - p0) {
      // the group's other partitions: empty (the reduce reads no row there)
      const size_t er = ws_row(a, oseq, oh, p0 + d);
      a.ws_m[er] = kMinusBig;
      a.ws_l[er] = 0.f;
    }
  }
}

// Phase 2: out = sum_p w_p * o_p with w_p = l_p 2^(m_p - M) / sum_q l_q 2^(m_q - M).
//
// Every memory access of a pair is issued so that few round trips are
// serial: the (m, l) of the first 64 partitions are read once, one lane
// each; a 64-partition window's weights are computed lane-parallel and each
// is broadcast from its lane; and the partial rows are read four at a time
// with buffer loads issued together.  A partition of weight exactly 0 (an
// empty marker left by the matrix-core kernel's per-workgroup merge) adds
// nothing, and its load gets an out-of-range offset, which the hardware
// answers with zeros and no memory access; a NaN weight is read, so a bad
// id keeps its NaN.

// M = max_p m_p and the inverse of L = sum_p l_p 2^(m_p - M), the same in
// every lane; l0 and m0 are this lane's partition of the first window.
struct PairScale {
  float M, inv, m0, l0;
};
__device__ __forceinline__ PairScale pair_scale(const DecodeArgs& a, size_t row0, int nparts, int lane) {
  const int G = a.qgroup;
  const float* pm = a.ws_m + row0;
  const float* pl = a.ws_l + row0;
  const bool in0 = lane < nparts;
  PairScale ps;
  ps.m0 = in0 ? pm[static_cast<size_t>(lane) * G] : -INFINITY;
  ps.l0 = in0 ? pl[static_cast<size_t>(lane) * G] : 0.f;
  float M = fmaxf(-INFINITY, ps.m0);
  for (int p = lane + 64; p < nparts; p += 64) M = fmaxf(M, pm[static_cast<size_t>(p) * G]);
  M = group_max<1, 64>(M);
  float L = in0 ? ps.l0 * fast_exp2(ps.m0 - M) : 0.f;
  for (int p = lane + 64; p < nparts; p += 64)
    L += pl[static_cast<size_t>(p) * G] * fast_exp2(pm[static_cast<size_t>(p) * G] - M);
  L = group_sum<1, 64>(L);
  ps.M = M;
  ps.inv = 1.f / L;
  return ps;
}

// Weight of partition q0 + lane (0 past the last partition).
__device__ __forceinline__ float window_weight(const DecodeArgs& a, size_t row0, int nparts, int q0,
                                               const PairScale& ps, int lane) {
  const int p = q0 + lane;
  if (p >= nparts) return 0.f;
  if (q0 == 0) return ps.l0 * fast_exp2(ps.m0 - ps.M) * ps.inv;
  const size_t pr = static_cast<size_t>(p) * a.qgroup;
  return a.ws_l[row0 + pr] * fast_exp2(a.ws_m[row0 + pr] - ps.M) * ps.inv;
}

// acc += w_p * o_p for p = q0 + lo .. q0 + hi - 1 in increasing order
// (hi <= 64 and q0 + hi <= nparts; lo, hi wave-uniform), wl holding the
// weight of partition q0 + lane.  Each lane owns D/64 adjacent dims.
template <int D>
__device__ __forceinline__ void accumulate_window(const DecodeArgs& a, size_t row0, int nparts, int q0,
                                                  int lo, int hi, float wl, int lane,
                                                  float (&acc)[D / 64]) {
  constexpr int PER = D / 64;
  const uint32_t row_stride = static_cast<uint32_t>(a.qgroup) * D * sizeof(float);
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(a.ws_o + row0 * D, 0,
                                                    static_cast<int>(nparts * row_stride), kRsrcWord3);
  const uint32_t lane_off = static_cast<uint32_t>(PER * lane) * sizeof(float);
  for (int u0 = lo; u0 < hi; u0 += 4) {
    float wt[4], v[4][PER];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int uu = u0 + u;
      wt[u] = uu < hi ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), min(uu, 63))) : 0.f;
      const uint32_t off =
          wt[u] != 0.f ? static_cast<uint32_t>(q0 + uu) * row_stride + lane_off : 0x80000000u;
      if constexpr (PER == 2) {
        const auto t = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
        v[u][0] = __uint_as_float(t[0]);
        v[u][1] = __uint_as_float(t[1]);
      } else {
        v[u][0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (wt[u] != 0.f) {
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(wt[u], v[u][e], acc[e]);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_reduce(DecodeArgs a) {
  // One workgroup per (query head, sequence).  Each 64-partition window is
  // split into four contiguous runs, one per wave, and the four partial
  // sums meet in LDS.
  constexpr int PER = D / 64;
  static_assert(PER == 1 || PER == 2, "head_dim 64 or 128");
  __shared__ float s_acc[kWaves][D];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = a.lens[b];
  if (!len_valid(n, a)) return;
  const int gi = a.seq_group != nullptr ? a.seq_group[b] : -1;
  const int nparts = seq_parts(a, b, gi, (n + kBlock - 1) / kBlock).total;
  if (nparts <= 1) return;                 // phase 1 wrote the output
  const size_t bh = static_cast<size_t>(b) * a.hq + h;
  // Partition p's row is row0 + p * G (rows are [B][Hkv][P][G]).
  const size_t row0 = ws_row(a, b, h, 0);
  const PairScale ps = pair_scale(a, row0, nparts, lane);
  float acc[PER] = {};
  for (int q0 = 0; q0 < nparts; q0 += 64) {
    const int cnt = min(64, nparts - q0);
    const int per = (cnt + kWaves - 1) / kWaves;
    const float wl = window_weight(a, row0, nparts, q0, ps, lane);
    accumulate_window<D>(a, row0, nparts, q0, min(w * per, cnt), min((w + 1) * per, cnt), wl, lane, acc);
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) s_acc[w][PER * lane + e] = acc[e];
  __syncthreads();
  if (tid < D)
    a.out[bh * D + tid] = (s_acc[0][tid] + s_acc[1][tid]) + (s_acc[2][tid] + s_acc[3][tid]);
}

// The same reduce with one wave per (query head, sequence) and four heads
// per workgroup, for batches of at most kReduceWaveParts partitions and
// enough pairs to give every CU a workgroup: there a pair's few partial rows
// leave four waves mostly waiting, and the LDS merge and barrier are pure
// latency.
constexpr int kReduceWaveParts = 16;
constexpr int kReduceWaveMinPairs = kWaves * 256;   // one workgroup per CU

template <int D>
__global__ __launch_bounds__(kThreads) void decode_reduce_wave(DecodeArgs a) {
  constexpr int PER = D / 64;
  static_assert(PER == 1 || PER == 2, "head_dim 64 or 128");
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int b = blockIdx.y;
  if (h >= a.hq) return;
  const int n = a.lens[b];
  if (!len_valid(n, a)) return;
  const int gi = a.seq_group != nullptr ? a.seq_group[b] : -1;
  const int nparts = seq_parts(a, b, gi, (n + kBlock - 1) / kBlock).total;
  if (nparts <= 1) return;                 // phase 1 wrote the output
  const size_t row0 = ws_row(a, b, h, 0);
  const PairScale ps = pair_scale(a, row0, nparts, lane);
  float acc[PER] = {};
  for (int q0 = 0; q0 < nparts; q0 += 64) {
    const float wl = window_weight(a, row0, nparts, q0, ps, lane);
    accumulate_window<D>(a, row0, nparts, q0, 0, min(64, nparts - q0), wl, lane, acc);
  }
  float* orow = a.out + (static_cast<size_t>(b) * a.hq + h) * D + PER * lane;
  if constexpr (PER == 2)
    *reinterpret_cast<float2*>(orow) = make_float2(acc[0], acc[1]);
  else
    orow[0] = acc[0];
}

template <int DT, int D>
hipError_t launch_dt_d(const DecodeArgs& args, int B, int group, hipStream_t st) {
  // Shared partitions first (they fill workspace rows the private pass
  // skips), then every sequence's private partitions, then the reduce.
  // When one workgroup of the private grid holds every private partition
  // of a sequence (grid z extent 1), phase 1 finishes the sequence itself:
  // it merges the shared slots, which are complete by then, and writes
  // out[]; the reduce, its launch and the private partials' workspace round
  // trip go away.
  constexpr bool kMfmaOk = DT != PA_DTYPE_F32;
  const bool mfma = kMfmaOk && (group == 4 || group == 8);
  const int zext = mfma ? (args.grid_parts + kWaves - 1) / kWaves : args.grid_parts;
  DecodeArgs a = args;
  a.finish = zext == 1;
  if constexpr (DT != PA_DTYPE_F32) {
    if (a.n_groups > 0)
      decode_phase1_mfma<DT, D, 16, kNbufShared, true>
          <<<dim3(a.hkv, a.n_groups, (a.max_shared_parts + kWaves - 1) / kWaves), kThreads, 0, st>>>(a);
  }
  dim3 grid(a.hkv, B, a.grid_parts);
  // The matrix-core kernel gives each wave a whole partition.
  dim3 grid_w(a.hkv, B, (a.grid_parts + kWaves - 1) / kWaves);
  // The private pass of a shared-prefix plan whose sequences read at most
  // kHeadsMaxBlocks blocks outside the shared pass (16-bit K/V only): four
  // KV heads per workgroup.  Longer private runs keep the head-per-workgroup
  // mapping, whose shorter workgroups leave a shorter tail (the fork
  // batch's 17-block runs measured 2-4% slower the other way).
  constexpr bool kHeadsOk = DT != PA_DTYPE_F32;
  constexpr int kHeadsMaxBlocks = 8;
  const bool heads = kHeadsOk && a.n_groups > 0 && a.hkv % kWaves == 0 &&
                     a.private_blocks > 0 && a.private_blocks <= kHeadsMaxBlocks;
  dim3 grid_h(a.hkv / kWaves, B, a.grid_parts);
  const bool append = a.k_new != nullptr;
  switch (group) {
    case 1:
      if (heads && append) decode_phase1<DT, D, 1, kNbufHeads, kHeadsOk, true><<<grid_h, kThreads, 0, st>>>(a);
      else if (heads) decode_phase1<DT, D, 1, kNbufHeads, kHeadsOk><<<grid_h, kThreads, 0, st>>>(a);
      else if (append) decode_phase1<DT, D, 1, kNbuf, false, true><<<grid, kThreads, 0, st>>>(a);
      else decode_phase1<DT, D, 1, kNbuf><<<grid, kThreads, 0, st>>>(a);
      break;
    case 2:
      if (heads && append) decode_phase1<DT, D, 2, kNbufHeads, kHeadsOk, true><<<grid_h, kThreads, 0, st>>>(a);
      else if (heads) decode_phase1<DT, D, 2, kNbufHeads, kHeadsOk><<<grid_h, kThreads, 0, st>>>(a);
      else if (append) decode_phase1<DT, D, 2, kNbuf, false, true><<<grid, kThreads, 0, st>>>(a);
      else decode_phase1<DT, D, 2, kNbuf><<<grid, kThreads, 0, st>>>(a);
      break;
    case 4:
      if constexpr (DT != PA_DTYPE_F32) {
        if (append) decode_phase1_mfma<DT, D, 4, kNbufMfma, false, true><<<grid_w, kThreads, 0, st>>>(a);
        else decode_phase1_mfma<DT, D, 4, kNbufMfma, false><<<grid_w, kThreads, 0, st>>>(a);
      } else {
        if (append) decode_phase1<DT, D, 4, kNbufG4, false, true><<<grid, kThreads, 0, st>>>(a);
        else decode_phase1<DT, D, 4, kNbufG4><<<grid, kThreads, 0, st>>>(a);
      }
      break;
    case 8:
      if constexpr (DT != PA_DTYPE_F32) {
        if (append) decode_phase1_mfma<DT, D, 8, kNbufMfma, false, true><<<grid_w, kThreads, 0, st>>>(a);
        else decode_phase1_mfma<DT, D, 8, kNbufMfma, false><<<grid_w, kThreads, 0, st>>>(a);
      } else {
        if (append) decode_phase1<DT, D, 8, 2, false, true><<<grid, kThreads, 0, st>>>(a);
        else decode_phase1<DT, D, 8, 2><<<grid, kThreads, 0, st>>>(a);
      }
      break;
    default: return hipErrorInvalidValue;
  }
  // One wave per pair where that still gives every CU a workgroup (the
  // 13B layer's 400 pairs do not: there four waves per pair win).
  const bool wave_reduce = a.num_parts <= kReduceWaveParts &&
                           static_cast<int64_t>(B) * a.hq >= kReduceWaveMinPairs;
  if (a.finish || a.num_parts <= 1) return hipGetLastError();
  if (!wave_reduce)
    decode_reduce<D><<<dim3(a.hq, B), kThreads, 0, st>>>(a);
  else
    decode_reduce_wave<D><<<dim3((a.hq + kWaves - 1) / kWaves, B), kThreads, 0, st>>>(a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const DecodeArgs& a, int B, int D, int group, hipStream_t st) {
  if (D == 64) return launch_dt_d<DT, 64>(a, B, group, st);
  return launch_dt_d<DT, 128>(a, B, group, st);
}

int32_t part_blocks_for(int32_t max_len, int32_t partition_tokens) {
  if (partition_tokens > 0) return partition_tokens / kBlock;
  const int32_t nb = (max_len + kBlock - 1) / kBlock;
  return nb > 0 ? nb : 1;
}

struct WsLayout {
  size_t o_off, m_off, l_off, total;
};

WsLayout ws_layout(int32_t B, int32_t hq, int32_t D, int32_t P) {
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  WsLayout w{};
  if (P <= 1) return w;
  const size_t bhp = static_cast<size_t>(B) * hq * P;
  w.o_off = 0;
  w.m_off = al(bhp * D * sizeof(float));
  w.l_off = w.m_off + al(bhp * sizeof(float));
  w.total = w.l_off + al(bhp * sizeof(float));
  return w;
}

// Partitions of the plain split of max_context_len.
int32_t plain_parts(int32_t max_context_len, int32_t part_blocks) {
  const int32_t nb = (max_context_len + kBlock - 1) / kBlock;
  return nb == 0 ? 1 : (nb + part_blocks - 1) / part_blocks;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" size_t pa_decode_workspace_bytes(int32_t B, int32_t num_q_heads, int32_t head_dim,
                                            int32_t max_context_len, int32_t partition_tokens) {
  if (B <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0 || partition_tokens < 0)
    return 0;
  const int32_t pb = part_blocks_for(max_context_len, partition_tokens);
  if (pb <= 0) return 0;
  return ws_layout(B, num_q_heads, head_dim, plain_parts(max_context_len, pb)).total;
}

// With a shared-prefix plan a member's shared blocks need not end on a
// partition boundary: its slots can number one more than the plain split.
extern "C" size_t pa_decode_shared_workspace_bytes(int32_t B, int32_t num_q_heads, int32_t head_dim,
                                                   int32_t max_context_len, int32_t partition_tokens) {
  if (B <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0 || partition_tokens <= 0)
    return 0;
  const int32_t pb = part_blocks_for(max_context_len, partition_tokens);
  return ws_layout(B, num_q_heads, head_dim, plain_parts(max_context_len, pb) + 1).total;
}

// Split-KV scratch of pa_decode_noalloc: the partition results live in this
// file-scope device array instead of a caller's workspace.  Each GPU the
// library runs on holds its own copy for the life of the process.  Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in): the device address comes from hipGetSymbolAddress, taken once
// per device with that device current and kept per device.
constexpr size_t kScratchBytes = static_cast<size_t>(64) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_ptr(const std::string& name, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(PA_ERR_DEVICE, name + ": hipGetDevice failed: " + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_ERR_UNSUPPORTED, name + ": device index beyond " + std::to_string(kMaxDevices));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(PA_ERR_DEVICE, name + ": hipGetSymbolAddress(scratch) failed: " +
                                     hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

int decode_impl(const char* fn, float* out, const void* q, const void* k_cache,
                const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                const int32_t* context_lens, int32_t max_context_len, int32_t B,
                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                int32_t num_blocks, float scale, int32_t partition_tokens, int32_t dtype,
                const int32_t* seq_group, const int32_t* groups, int32_t n_groups,
                int32_t max_shared_parts, int32_t max_private_parts, int32_t max_private_blocks,
                void* workspace, size_t workspace_bytes, void* stream, bool use_scratch = false,
                const void* k_new = nullptr, const void* v_new = nullptr) {
  const std::string name(fn);
  auto err_ = [&](int code, const std::string& msg) { return fail(code, name + ": " + msg); };
  if (B < 0 || max_context_len < 0 || max_blocks_per_seq < 0 || num_blocks <= 0)
    return err_(PA_ERR_INVALID, "negative size or empty pool");
  if (n_groups < 0 || max_shared_parts < 0 || max_private_parts < 0 || max_private_blocks < 0)
    return err_(PA_ERR_INVALID,
                "negative n_groups, max_shared_parts, max_private_parts or max_private_blocks");
  if (B == 0) { clear_error(); return PA_OK; }
  // A table of width 0 has no entries and may be NULL.
  if (!out || !q || !k_cache || !v_cache || (!block_tables && max_blocks_per_seq > 0) || !context_lens)
    return err_(PA_ERR_INVALID, "null pointer");
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return err_(PA_ERR_INVALID, "num_q_heads must be a positive multiple of num_kv_heads");
  const int group = num_q_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return err_(PA_ERR_UNSUPPORTED, "query group size must be 1, 2, 4 or 8");
  if (block_size != kBlock) return err_(PA_ERR_UNSUPPORTED, "block_size must be 16");
  if (head_dim != 64 && head_dim != 128)
    return err_(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16)
    return err_(PA_ERR_UNSUPPORTED, "unknown dtype");
  if (partition_tokens < 0 || partition_tokens % kBlock != 0)
    return err_(PA_ERR_INVALID, "partition_tokens must be 0 or a multiple of 16");
  if (!std::isfinite(scale)) return err_(PA_ERR_INVALID, "scale must be finite");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache)) & 15)
    return err_(PA_ERR_INVALID, "q and caches must be 16-byte aligned");
  if ((k_new == nullptr) != (v_new == nullptr))
    return err_(PA_ERR_INVALID, "k_new and v_new must both be given");
  if (k_new && ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15))
    return err_(PA_ERR_INVALID, "k_new and v_new must be 16-byte aligned");
  const size_t block_bytes = static_cast<size_t>(num_kv_heads) * head_dim * kBlock *
                             (dtype == PA_DTYPE_F32 ? 4 : 2);
  if (block_bytes >= (static_cast<size_t>(1) << 31))
    return err_(PA_ERR_UNSUPPORTED, "one block of one layer must be under 2 GiB");
  // Grid limits: KV heads on x, sequences on y (<= 65535), partitions on z.
  if (B > 65535) return err_(PA_ERR_UNSUPPORTED, "more than 65535 sequences");

  if (n_groups > 0) {
    if (!seq_group || !groups) return err_(PA_ERR_INVALID, "null plan pointer");
    if (dtype == PA_DTYPE_F32)
      return err_(PA_ERR_UNSUPPORTED, "a shared-prefix plan needs F16 or BF16 K/V");
    if (partition_tokens == 0)
      return err_(PA_ERR_INVALID, "a shared-prefix plan needs partition_tokens > 0");
    if (n_groups > 65535 || max_shared_parts > 65535)
      return err_(PA_ERR_UNSUPPORTED, "more than 65535 plan groups or shared partitions");
  }
  // With a plan in force a member's slots can exceed the plain split by
  // one (its shared blocks need not end on a partition boundary).
  const bool plan = n_groups > 0 && max_shared_parts > 0;

  DecodeArgs a{};
  a.part_blocks = part_blocks_for(max_context_len, partition_tokens);
  const int32_t P = plain_parts(max_context_len, a.part_blocks);
  if (P > 65535)
    return err_(PA_ERR_UNSUPPORTED, "more than 65535 partitions; use larger partitions");
  a.num_parts = P + (plan ? 1 : 0);        // workspace slots per (sequence, head)
  const WsLayout wl = ws_layout(B, num_q_heads, head_dim, a.num_parts);
  if (use_scratch && wl.total > 0) {
    if (wl.total > kScratchBytes)
      return err_(PA_ERR_INVALID, "needs " + std::to_string(wl.total) +
                                      " bytes of split-KV scratch; the library's scratch holds " +
                                      std::to_string(kScratchBytes) +
                                      " (use larger partitions, fewer sequences, or pa_decode)");
    const int st = scratch_ptr(name, &workspace);
    if (st != PA_OK) return st;
    workspace_bytes = kScratchBytes;
  }
  if (wl.total > 0) {
    if (!workspace || workspace_bytes < wl.total)
      return err_(PA_ERR_INVALID, "workspace too small (need " +
                                      std::to_string(wl.total) + " bytes)");
    if (reinterpret_cast<uintptr_t>(workspace) & 15)
      return err_(PA_ERR_INVALID, "workspace must be 16-byte aligned");
    char* ws = static_cast<char*>(workspace);
    a.ws_o = reinterpret_cast<float*>(ws + wl.o_off);
    a.ws_m = reinterpret_cast<float*>(ws + wl.m_off);
    a.ws_l = reinterpret_cast<float*>(ws + wl.l_off);
  }
  a.out = out;
  a.q = static_cast<const char*>(q);
  a.k = static_cast<const char*>(k_cache);
  a.v = static_cast<const char*>(v_cache);
  if (k_new) {
    // the caches are the caller's writable device memory (pa_write_decode
    // takes them as non-const pointers)
    a.k_w = static_cast<char*>(const_cast<void*>(k_cache));
    a.v_w = static_cast<char*>(const_cast<void*>(v_cache));
    a.k_new = static_cast<const char*>(k_new);
    a.v_new = static_cast<const char*>(v_new);
  }
  a.tables = block_tables;
  a.lens = context_lens;
  a.max_blocks = max_blocks_per_seq;
  a.max_len = max_context_len;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.num_blocks = num_blocks;
  a.scale_log2 = scale * kLog2e;
  a.batch = B;
  a.qgroup = group;
  a.grid_parts = P;                        // private partitions of any sequence <= P
  if (plan) {
    a.seq_group = seq_group;
    a.groups = groups;
    a.n_groups = n_groups;
    a.max_shared_parts = max_shared_parts;
    if (max_private_parts > 0) a.grid_parts = std::min(P, max_private_parts);
    a.private_blocks = max_private_blocks;
  }

  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  switch (dtype) {
    case PA_DTYPE_F32: err = launch_dt<PA_DTYPE_F32>(a, B, head_dim, group, st); break;
    case PA_DTYPE_F16: err = launch_dt<PA_DTYPE_F16>(a, B, head_dim, group, st); break;
    default: err = launch_dt<PA_DTYPE_BF16>(a, B, head_dim, group, st); break;
  }
  if (err != hipSuccess)
    return err_(PA_ERR_DEVICE, std::string("launch failed: ") + hipGetErrorString(err));
  clear_error();
  return PA_OK;
}

}  // namespace

extern "C" int pa_decode(float* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t max_context_len, int32_t B,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, float scale,
                         int32_t partition_tokens, int32_t dtype, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return decode_impl("pa_decode", out, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                     context_lens, max_context_len, B, num_q_heads, num_kv_heads, head_dim,
                     block_size, num_blocks, scale, partition_tokens, dtype, nullptr, nullptr, 0,
                     0, 0, 0, workspace, workspace_bytes, stream);
}

extern "C" int pa_decode_shared(float* out, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t max_context_len, int32_t B, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t num_blocks, float scale, int32_t partition_tokens,
                                int32_t dtype, const int32_t* seq_group, const int32_t* groups,
                                int32_t n_groups, int32_t max_shared_parts,
                                int32_t max_private_parts, int32_t max_private_blocks,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl("pa_decode_shared", out, q, k_cache, v_cache, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, B, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, scale, partition_tokens,
                     dtype, seq_group, groups, n_groups, max_shared_parts, max_private_parts,
                     max_private_blocks, workspace, workspace_bytes, stream);
}

extern "C" int pa_write_decode(float* out, const void* q, void* k_cache, void* v_cache,
                               const void* k_new, const void* v_new,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t max_context_len, int32_t B,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks, float scale,
                               int32_t partition_tokens, int32_t dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (B > 0 && (!k_new || !v_new)) return fail(PA_ERR_INVALID, "pa_write_decode: null pointer");
  return decode_impl("pa_write_decode", out, q, k_cache, v_cache, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, B, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, scale, partition_tokens,
                     dtype, nullptr, nullptr, 0, 0, 0, 0, workspace, workspace_bytes, stream, false,
                     k_new, v_new);
}

extern "C" int pa_write_decode_shared(float* out, const void* q, void* k_cache, void* v_cache,
                                      const void* k_new, const void* v_new,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t max_context_len,
                                      int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      float scale, int32_t partition_tokens, int32_t dtype,
                                      const int32_t* seq_group, const int32_t* groups,
                                      int32_t n_groups, int32_t max_shared_parts,
                                      int32_t max_private_parts, int32_t max_private_blocks,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (B > 0 && (!k_new || !v_new))
    return fail(PA_ERR_INVALID, "pa_write_decode_shared: null pointer");
  return decode_impl("pa_write_decode_shared", out, q, k_cache, v_cache, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, B, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, scale, partition_tokens,
                     dtype, seq_group, groups, n_groups, max_shared_parts, max_private_parts,
                     max_private_blocks, workspace, workspace_bytes, stream, false, k_new, v_new);
}

extern "C" size_t pa_decode_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" int pa_decode_noalloc(float* out, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t max_context_len, int32_t B, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, float scale, int32_t partition_tokens,
                                 int32_t dtype, void* stream) {
  return decode_impl("pa_decode_noalloc", out, q, k_cache, v_cache, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, B, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, scale, partition_tokens,
                     dtype, nullptr, nullptr, 0, 0, 0, 0, nullptr, 0, stream, true);
}
