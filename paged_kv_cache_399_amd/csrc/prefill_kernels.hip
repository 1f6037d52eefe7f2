// Paged prefill attention for gfx950 (MI355X): causal attention of a chunk of
// newly appended tokens over everything the sequence holds.
//
// The chunk's blocks are handed out as the tokens arrive ("PagedAttention
// Internals", "Fixed-Size KV Blocks"; "pagedattention" topic page, third
// paragraph) and cache_append has stored them; then for sequence b with L
// tokens of which the last n are new, query i (position L - n + i) and query
// head h (KV head g = h / G) computes
//     out[i,h] = sum_{t <= L-n+i} softmax_t(scale * q[i,h] . K[t,g]) V[t,g]
// with K / V reached through the block table as in decode.
//
// Unlike decode this is a dense contraction: every key/value chunk serves a
// whole tile of queries, so it is staged once in LDS per workgroup and all
// waves run both products on matrix cores from there.
//
// Work decomposition: one workgroup per (query tile, sequence, KV head, head
// half), on a one-dimensional XCD-aware grid (see prefill_mfma_kernel); a
// workgroup of four waves takes 128 query rows: BT = 128 / GW query tokens
// of GW query heads of one KV head (GW the largest of 8, 4, 2, 1 dividing G;
// the G / GW parts of a head group take workgroups of their own).
// Wave w takes two 16-row tiles, k = 2w and 2w + 1, tile k being tokens
// 16 (k / GW) .. + 15 of head k % GW, so every key / value fragment a wave
// reads from LDS feeds two matrix-core products.  Tiles are launched
// last-first: later tiles see more keys, so the dispatcher starts the longest
// work first.
//
// Lane layout (as in the decode matrix-core kernel, with query tokens in the
// 16-wide N dimension): lane l has n = l % 16 (its query column) and
// r = l / 16.  For a 32-key chunk, two 16x16x32 MFMA chains per tile produce
// the scores of keys 8r .. 8r + 7 for query n; those eight probabilities are
// the B operand of the value MFMA, whose A operand is the 16-byte run of the
// token-minor value tile (dims 16 j + n, keys 8r .. 8r + 7).  The maximum over
// a query's 32 keys crosses the four row groups with two lane swaps (32
// apart, then 16 apart) on the vector ALU; the sum comes from one more
// product with an all-ones A operand.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "device_common.hpp"
#include "internal.hpp"
#include "tile_common.hpp"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct PrefillArgs {
  void* out;
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* table;
  const int32_t* ctx;
  const int32_t* qstart;
  int32_t n_seqs, hq, hkv, p, lp, num_blocks, max_blocks;  // p = 1 << lp
  int32_t n_tiles;   // query tiles per sequence (ceil(max_query_len / tokens per workgroup))
  KStrides ks;       // key cache: elements between KV heads, between tokens
  float scale_log2;  // scale * log2(e): scores are kept in log2 units
  int32_t* err;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// How far (log2 units) a chunk's maximum score may exceed the running
// reference before the reference moves and the accumulators are rescaled.
constexpr float kRefSlack = 8.f;

constexpr int kXcds = 8;  // accelerator complex dies (separate L2 caches) on MI355X

// pair_max32 / pair_max16 (row-group maxima) and kswz (the key-row LDS
// swizzle) are in tile_common.hpp.

// Wave w stages the keys [c0 + 16 w, c0 + 16 w + 16) of each 64-key chunk,
// which lie in one block (two with blocks of 8), so the blocks' addresses are
// uniform over the wave (scalar registers) and every lane's offsets inside
// them are fixed for the whole loop.  The keys and values go straight from
// HBM into LDS (global_load_lds_dwordx4: no staging registers, no vector-ALU
// address arithmetic), keys two chunks ahead and values one, and the loop is
// software-pipelined: the score products of chunk i + 1 are issued between
// the softmax instructions of chunk i.
template <int D, int GW>
__global__ __launch_bounds__(256, 2) void prefill_mfma_kernel(PrefillArgs a) {
  constexpr int NT = 256;             // threads: four waves
  constexpr int BT = 16 * (8 / GW);   // query tokens per workgroup
  constexpr int NH = 2;               // 32-key halves per chunk
  constexpr int CH = 32 * NH;         // keys per chunk
  constexpr int KI = D / 32;          // score MFMA steps over head_dim
  constexpr int NJ = D / 16;          // value MFMA output tiles over head_dim
  constexpr int KS = D;               // LDS key row (elements); 16-byte pieces swizzled, see kswz
  constexpr int KU = CH * D / 8 / NT; // 16-byte key pieces per thread per chunk
  constexpr int VU = D * CH / 8 / NT; // 16-byte value pieces per thread per chunk
  constexpr int TW = 1024;            // block-table window (entries)
  static_assert(KU >= 1 && VU >= 1, "chunk pieces");
  __shared__ __align__(16) uint16_t k_lds[2][CH * KS];
  __shared__ __align__(16) uint16_t v_lds[2][D * CH];
  __shared__ int32_t tab[TW];

  const int32_t G = a.hq / a.hkv;
  const int32_t halves = G / GW;
  // XCD-aware order: workgroup L runs on XCD L % 8.  Group (sequence, KV
  // head, head half) j is pinned to XCD j % 8, so all query tiles that read
  // its keys and values share one L2; an XCD runs its groups one after the
  // other, each group's tiles last first (longest work first), so the
  // workgroups resident on an XCD read a few groups' keys and values at once.
  const int32_t n_groups = a.n_seqs * a.hkv * halves;
  const int32_t xcd = (int32_t)blockIdx.x % kXcds, slot = (int32_t)blockIdx.x / kXcds;
  const int32_t group = (slot / a.n_tiles) * kXcds + xcd;
  if (group >= n_groups) return;  // padding of the last XCD row (uniform)
  const int32_t tile = a.n_tiles - 1 - slot % a.n_tiles;
  const int32_t b = group / (a.hkv * halves), gz = group - b * (a.hkv * halves);
  const int32_t g = gz / halves, hpart = gz - g * halves;
  const int32_t q0 = a.qstart[b];
  const int32_t n = a.qstart[b + 1] - q0;
  if (n <= 0 || tile * BT >= n) return;  // uniform over the workgroup
  // more new tokens than the grid's tiles cover (max_query_len too small):
  // the rows past the last tile stay unwritten, so flag it
  if (tile == a.n_tiles - 1 && hpart == 0 && threadIdx.x == 0 && (int64_t)a.n_tiles * BT < n)
    atomicOr(a.err, PKV_DEVERR_CONTEXT_LEN);
  const int32_t P = a.p, lp = a.lp;  // block size, a power of two
  const int32_t L = a.ctx[b];
  if (L < n || (int64_t)L > (int64_t)a.max_blocks * P) {
    if (threadIdx.x == 0 && tile == 0 && hpart == 0) atomicOr(a.err, PKV_DEVERR_CONTEXT_LEN);
    return;  // the sequence's rows are left unwritten
  }
  const int32_t base = L - n;  // position of query 0
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nq = lane & 15, r = lane >> 4;
  const float c = a.scale_log2;

  // this wave's two tiles
  int32_t head[2], tok0[2], qi[2], qpos[2];
  bool on[2];
  int32_t wave_last = -1;  // last query (within the chunk of new tokens) of the wave
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int k = 2 * w + t;
    head[t] = g * G + hpart * GW + k % GW;
    tok0[t] = tile * BT + 16 * (k / GW);
    on[t] = tok0[t] < n;  // uniform
    qi[t] = min(tok0[t] + nq, n - 1);  // columns past the end repeat the last query
    qpos[t] = base + qi[t];
    if (on[t]) wave_last = max(wave_last, min(tok0[t] + 15, n - 1));
  }
  const int32_t wave_kend = wave_last >= 0 ? base + wave_last + 1 : 0;         // keys [0, wave_kend)
  const int32_t kend = base + min(tile * BT + BT - 1, n - 1) + 1;             // the workgroup's keys
  const int32_t nchunks = (kend + CH - 1) / CH;

  // query fragments (B operand of the score MFMA): dims 32 i + 8 r of query qi
  bf16x8 qf[2][KI];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)(q0 + qi[t]) * a.hq + head[t]) * D + 8 * r;
#pragma unroll
    for (int i = 0; i < KI; ++i)
      qf[t][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + 32 * i));
  }

  const uint16_t* kc = (const uint16_t*)a.kc;
  const uint16_t* vc = (const uint16_t*)a.vc;
  const int32_t* trow = a.table + (int64_t)b * a.max_blocks;
  const int64_t blk_stride = (int64_t)a.hkv * P * D;
  const int64_t khead = (int64_t)g * a.ks.head, vhead = (int64_t)g * P * D;
  const int32_t last_blk = (kend - 1) >> lp;

  // block-table window: tab[i] = physical block of logical block wb + i
  int32_t wb = 0;
  auto load_tab = [&](int32_t first) {
    for (int i = tid; i < TW; i += NT) {
      const int32_t lb = first + i;
      int32_t e = 0;
      if (lb <= last_blk) {
        e = trow[lb];
        if ((uint32_t)e >= (uint32_t)a.num_blocks) {
          atomicOr(a.err, PKV_DEVERR_TABLE_ENTRY);
          e = 0;
        }
      }
      tab[i] = e;
    }
  };

  // Wave-group staging: wave w stages the 16 keys [c0 + 16 w, + 16) of
  // each chunk, KU = D / 32 loads of 64 lanes x 16 bytes for the keys and as
  // many for the values.  A key load covers KR = 512 / D rows: lane row wkr,
  // 16-byte column wdc.
  static_assert(KU == D / 32 && VU == D / 32, "one 16-key group per wave");
  constexpr int KR = 512 / D;
  const int wkr = lane / (D / 8), wdc = lane % (D / 8);
  // one wave's 16-key group of a chunk: keys [kb, kb + 16), or for a group
  // past the context end the last group that holds keys (in bounds; zeroed
  // with the boundary mask).  With blocks of 16 or more the group lies in one
  // block (offA; offB the same); with blocks of 8 its keys 8..15 lie in a
  // second block (offB), the tile's last block where the group ends early.
  // (direct: the entries read from the table row itself, for the first
  // chunks, staged before the table window is in LDS)
  const bool p8 = P < 16;  // uniform
  auto group_base = [&](int32_t c0, int64_t& offA, int64_t& offB, bool direct = false) -> int32_t {
    const int32_t kb = c0 + 16 * w;  // uniform
    const int32_t kl = min(kb, kend - 1) & ~15;
    const int32_t la = kl >> lp, lb2 = p8 ? min(la + 1, last_blk) : la;
    int32_t ba, bb;
    if (direct) {
      ba = __builtin_amdgcn_readfirstlane(trow[la]);
      bb = p8 ? __builtin_amdgcn_readfirstlane(trow[lb2]) : ba;
      if ((uint32_t)ba >= (uint32_t)a.num_blocks) ba = 0;  // flagged by the window load
      if ((uint32_t)bb >= (uint32_t)a.num_blocks) bb = 0;
    } else {
      ba = __builtin_amdgcn_readfirstlane(tab[la - wb]);
      bb = p8 ? __builtin_amdgcn_readfirstlane(tab[lb2 - wb]) : ba;
    }
    offA = (int64_t)ba * blk_stride;
    offB = (int64_t)bb * blk_stride;
    return kl & (P - 1);  // offset of the group inside its (first) block
  };
  // Direct global-to-LDS staging: each global_load_lds_dwordx4 puts
  // lane i's 16 bytes at the wave-uniform LDS address + 16 i, so a lane loads
  // whichever global piece belongs at its slot.  Keys: the swizzled rows
  // above, instruction u covering rows 16 w + u KR .. + KR - 1 (lane: row
  // + wkr, slot wdc, so the piece wdc ^ kswz(row)).  Values: group-major,
  // [8-key group][head_dim][8 keys]; wave w fills groups 2 w and 2 w + 1,
  // instruction u covering head_dim rows 64 (u % VPG) .. + 63 of group
  // 2 w + u / VPG.  The value-fragment reads of 16 consecutive rows of one
  // group are then 256 contiguous bytes.
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  typedef __attribute__((address_space(1))) void* gptr_t;
  constexpr int VPG = D / 64;  // value instructions per 8-key group
  uint32_t kdoff[KU];          // bytes from the first key row of the instruction's block
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int row = u * KR + wkr;
    const int grow = p8 && u * KR >= 8 ? row - 8 : row;  // (rows 8..15 of blocks of 8: second block)
    kdoff[u] = (uint32_t)(grow * a.ks.tok * 2 + (wdc ^ kswz<D>(16 * w + row)) * 16);
  }
  const uint32_t vdoff = (uint32_t)(lane * P * 2);  // bytes: this lane's head_dim row
  auto vslot = [&](int vbuf, int u) -> uint16_t* {   // instruction u's LDS run
    return &v_lds[vbuf][((2 * w + u / VPG) * D + (u % VPG) * 64) * 8];
  };
  // (instruction u covers key rows u KR .. u KR + KR - 1 of the group, all
  // in one block also with blocks of 8, since KR divides 8; value
  // instruction u covers the 8-key group u / VPG, one block of 8)
  auto kload_direct = [&](int32_t c0, int kbuf, bool direct = false) {
    int64_t oa, ob;
    const int32_t o = group_base(c0, oa, ob, direct);
    const char* ka = (const char*)(kc + oa + khead + (int64_t)o * a.ks.tok);
    const char* kb2 = (const char*)(kc + ob + khead);
#pragma unroll
    for (int u = 0; u < KU; ++u)
      __builtin_amdgcn_global_load_lds((gptr_t)((p8 && u * KR >= 8 ? kb2 : ka) + kdoff[u]),
                                       (lds_ptr_t)&k_lds[kbuf][(16 * w + u * KR) * KS], 16, 0, 0);
  };
  auto vload_direct = [&](int32_t c0, int vbuf, bool direct = false) {
    int64_t oa, ob;
    const int32_t o = group_base(c0, oa, ob, direct);
    const char* va = (const char*)(vc + oa + vhead + o);
    const char* vb2 = (const char*)(vc + ob + vhead);
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const char* vb = p8 ? (u / VPG ? vb2 : va) : va + (u / VPG) * 16;
      __builtin_amdgcn_global_load_lds((gptr_t)(vb + (u % VPG) * 64 * P * 2 + vdoff),
                                       (lds_ptr_t)vslot(vbuf, u), 16, 0, 0);
    }
  };
  // After this wave's loads of a group that reaches past the context end
  // have landed (vmcnt 0): zero the values of keys >= kend in its own slots
  // (those slots of the last block hold no token yet; a group wholly past
  // the end was loaded from the last group that holds keys).
  auto vfix = [&](int32_t c0, int vbuf) {
    const int32_t kb = c0 + 16 * w;
    if (kb + 16 <= kend) return;  // uniform
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int32_t t0 = kb + 8 * (u / VPG);
      const int32_t nv = t0 >= kend ? 0 : min(kend - t0, 8);
      const uint32_t m0 = nv >= 2 ? 0xffffffffu : (nv == 1 ? 0x0000ffffu : 0u);
      const uint32_t m1 = nv >= 4 ? 0xffffffffu : (nv == 3 ? 0x0000ffffu : 0u);
      const uint32_t m2 = nv >= 6 ? 0xffffffffu : (nv == 5 ? 0x0000ffffu : 0u);
      const uint32_t m3 = nv >= 8 ? 0xffffffffu : (nv == 7 ? 0x0000ffffu : 0u);
      uint4* sl = reinterpret_cast<uint4*>(vslot(vbuf, u) + lane * 8);
      uint4 x = *sl;
      x.x &= m0;
      x.y &= m1;
      x.z &= m2;
      x.w &= m3;
      *sl = x;
    }
  };

  f32x4 acc[2][NJ];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};
  // Row sums on the matrix cores: an all-ones A operand turns the value
  // product into sum_k p_k, in every row of the tile (the bf16-rounded
  // probabilities that the numerator uses, summed in fp32).
  f32x4 lsum[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  const int krow_x = 8 * (nq >> 2) + (nq & 3);  // key of chain-X row nq within the chunk
  // the swizzle of every key row this lane reads (chains X and Y, both halves)
  const int kx = kswz<D>(krow_x);
  // the first chunks' blocks straight from the table row, so their loads are
  // in flight while the table window is brought into LDS
  kload_direct(0, 0, true);
  vload_direct(0, 0, true);
  if (nchunks > 1) kload_direct(CH, 1, true);
  load_tab(0);
  __syncthreads();
  // Software-pipelined loop.  Iteration ci runs the softmax of chunk ci in
  // the same basic block as the score products of chunk ci + 1 (they are
  // independent, so the in-order issue alternates vector-ALU and
  // matrix-core instructions), then the value products of chunk ci.  Keys
  // are staged two chunks ahead, values one: the key buffer of chunk ci is
  // free once its scores are taken (in iteration ci - 1), the value buffer
  // of chunk ci - 1 once its products are taken.
  struct Sc {
    f32x4 x[2][NH], y[2][NH];
  };
  auto scores = [&](int kbuf) -> Sc {
    const uint16_t* kl = k_lds[kbuf];
    Sc sc;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int h = 0; h < NH; ++h) sc.x[t][h] = sc.y[t][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const int cb = ((4 * i + r) ^ kx) * 8;
        const bf16x8 ax = *reinterpret_cast<const bf16x8*>(&kl[(32 * h + krow_x) * KS + cb]);
        const bf16x8 ay = *reinterpret_cast<const bf16x8*>(&kl[(32 * h + krow_x + 4) * KS + cb]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          sc.x[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax, qf[t][i], sc.x[t][h], 0, 0, 0);
          sc.y[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ay, qf[t][i], sc.y[t][h], 0, 0, 0);
        }
      }
    }
    return sc;
  };
  // causal mask of chunk c0's scores (rare: only chunks that reach past
  // some query's position)
  auto mask = [&](Sc& sc, int32_t c0) {
    if (c0 + CH - 1 > base + min(tok0[0], tok0[1])) {  // uniform
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int32_t kx0 = c0 + 32 * h + 8 * r + e;
            sc.x[t][h][e] = kx0 <= qpos[t] ? sc.x[t][h][e] : -INFINITY;
            sc.y[t][h][e] = kx0 + 4 <= qpos[t] ? sc.y[t][h][e] : -INFINITY;
          }
    }
  };
  // Softmax of one chunk: probabilities (bf16) against the running
  // reference, which moves (branch-free, per column) only when the chunk's
  // maximum exceeds it by more than 2^8; the accumulators are rescaled
  // afterwards, in a rare branch, by 2^((m_old - m_new) c).
  float m_old[2];
  auto softmax = [&](const Sc& sc, bf16x8 (&pb)[2][NH]) -> bool {
    bool moved = false;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float x = sc.x[t][0][0];
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) x = fmaxf(x, fmaxf(sc.x[t][h][e], sc.y[t][h][e]));
      const float cm = pair_max16(pair_max32(x));
      const bool up = (cm - m_run[t]) * c > kRefSlack;
      m_old[t] = m_run[t];
      m_run[t] = up ? fmaxf(m_run[t], cm) : m_run[t];
      moved |= up;
      const float mc = m_run[t] * c;
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pb[t][h][e] = (__bf16)fast_exp2(fmaf(sc.x[t][h][e], c, -mc));
          pb[t][h][e + 4] = (__bf16)fast_exp2(fmaf(sc.y[t][h][e], c, -mc));
        }
    }
    return moved;
  };
  // Scores of the next chunk fused with the softmax of the current one, in
  // a fixed issue order: segment k reads two key fragments ahead and issues
  // the four products of step k (both tiles, chains X and Y); its vector
  // work is the two row-maximum reductions (segments 0, 1), then an equal
  // share of the exponentials.  A scheduling fence after every segment
  // keeps the order, so the matrix core works on the next chunk while the
  // vector ALU works on this one.
  // key fragments of one chunk for the fused step: segment k's pair
  constexpr int NSEG = NH * KI;
  struct Kf {
    bf16x8 x[NSEG], y[NSEG];
  };
  auto kread = [&](int kbuf, Kf& f, int k) {
    const uint16_t* kl = k_lds[kbuf];
    const int h = k / KI, i = k % KI;
    const int cb = ((4 * i + r) ^ kx) * 8;
    f.x[k] = *reinterpret_cast<const bf16x8*>(&kl[(32 * h + krow_x) * KS + cb]);
    f.y[k] = *reinterpret_cast<const bf16x8*>(&kl[(32 * h + krow_x + 4) * KS + cb]);
  };
  // (the caller has read segment 0 into kf)
  auto fused = [&](int kbuf, Kf& kf, Sc& nx, const Sc& cu, bf16x8 (&pb)[2][NH]) -> bool {
    constexpr int NE = 2 * NH * 8;  // probabilities per lane per chunk
    bf16x8 (&ax)[NSEG] = kf.x;
    bf16x8 (&ay)[NSEG] = kf.y;
    auto kmfma = [&](int k) {
      const int h = k / KI, i = k % KI;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        nx.x[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax[k], qf[t][i], i ? nx.x[t][h] : f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        nx.y[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ay[k], qf[t][i], i ? nx.y[t][h] : f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      }
    };
    bool moved = false;
    float mc[2];
    auto rowmax = [&](int t) {
      float x = cu.x[t][0][0];
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) x = fmaxf(x, fmaxf(cu.x[t][h][e], cu.y[t][h][e]));
      // the column's maximum over its four lanes is needed only where the
      // reference moves: tested on each lane's own maximum first (a rare,
      // uniform branch)
      m_old[t] = m_run[t];
      if (__builtin_amdgcn_ballot_w64((x - m_run[t]) * c > kRefSlack) != 0) {
        const float cm = pair_max16(pair_max32(x));
        const bool up = (cm - m_run[t]) * c > kRefSlack;
        m_run[t] = up ? fmaxf(m_run[t], cm) : m_run[t];
        moved |= up;
      }
      mc[t] = m_run[t] * c;
    };
    // probability q (q = ((t * NH + h) * 2 + xy) * 4 + e) of this lane
    auto prob = [&](int q) {
      const int e = q & 3, xy = (q >> 2) & 1, h = (q >> 3) % NH, t = (q >> 3) / NH;
      const float sv = xy ? cu.y[t][h][e] : cu.x[t][h][e];
      pb[t][h][e + 4 * xy] = (__bf16)fast_exp2(fmaf(sv, c, -mc[t]));
    };
    if (NSEG > 1) kread(kbuf, kf, 1);
#pragma unroll
    for (int k = 0; k < NSEG; ++k) {
      if (k + 2 < NSEG) kread(kbuf, kf, k + 2);
      kmfma(k);
      if (k < 2) {
        rowmax(k);
      } else {
        constexpr int per = (NE + NSEG - 3) / (NSEG - 2);
#pragma unroll
        for (int q = (k - 2) * per; q < (k - 1) * per && q < NE; ++q) prob(q);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return moved;
  };
  // Value products of one chunk.  The value fragments are read VA head_dim
  // tiles ahead of their products, in a fixed order (a scheduling fence
  // after every tile), so each LDS read has the products of the tiles
  // before it to hide behind; left to itself the compiler reuses one
  // register quad and waits for every read.  The row sums need no fragment
  // and cover the first reads.
  auto values = [&](int vbuf, const bf16x8 (&pb)[2][NH]) {
    constexpr int VA = 3;
    const uint16_t* vl = v_lds[vbuf];
    bf16x8 av[NJ][NH];
    auto vread = [&](int j) {
#pragma unroll
      for (int h = 0; h < NH; ++h)
        av[j][h] = *reinterpret_cast<const bf16x8*>(&vl[((4 * h + r) * D + 16 * j + nq) * 8]);
    };
#pragma unroll
    for (int j = 0; j < VA && j < NJ; ++j) vread(j);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int h = 0; h < NH; ++h)
        lsum[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[t][h], lsum[t], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j + VA < NJ) vread(j + VA);
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[j][h], pb[t][h], acc[t][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
  vfix(0, 0);
  __syncthreads();
  // one iteration: chunk ci's softmax and value products, chunk ci + 1's
  // scores into `nxt`; unrolled by two below so that the two score sets
  // trade roles without register copies
  auto step = [&](int32_t ci, Sc& cur, Sc& nxt) {
    const int32_t c0 = ci * CH;
    const bool more = ci + 1 < nchunks, more2 = ci + 2 < nchunks;  // uniform
    if (more && min(c0 + 3 * CH, kend) - 1 >= (wb + TW) * P) {
      // the staged chunks leave the table window; every read of it is
      // behind the last barrier
      wb = (c0 + CH) >> lp;
      load_tab(wb);
      __syncthreads();
    }
    // the next chunk's first key fragments are read before this step's
    // loads are issued, so their LDS latency passes while those wait to issue
    const bool fuse = c0 < wave_kend && more && c0 + CH < wave_kend;  // uniform
    Kf kf;
    if (fuse) kread((ci + 1) & 1, kf, 0);
    if (more2) kload_direct(c0 + 2 * CH, ci & 1);
    if (more) vload_direct(c0 + CH, (ci + 1) & 1);
    if (c0 < wave_kend) {  // uniform over the wave
      mask(cur, c0);
      bf16x8 pb[2][NH];
      bool moved;
      if (fuse) {
        moved = fused((ci + 1) & 1, kf, nxt, cur, pb);
      } else {
        moved = softmax(cur, pb);
      }
      // keep the probabilities computed here, beside the score products,
      // rather than sunk past the rare rescale branch below
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int h = 0; h < NH; ++h) asm volatile("" : "+v"(pb[t][h]));
      if (__builtin_amdgcn_ballot_w64(moved) != 0) {  // rare
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float alpha = fast_exp2((m_old[t] - m_run[t]) * c);
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[t][j] *= alpha;
          lsum[t] *= alpha;
        }
      }
      __builtin_amdgcn_s_setprio(1);  // value products issue first on this SIMD
      values(ci & 1, pb);
      __builtin_amdgcn_s_setprio(0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
    if (more) vfix(c0 + CH, (ci + 1) & 1);
    __syncthreads();
  };
  Sc sa, sb;
  if (0 < wave_kend) sa = scores(0);  // uniform
  // every wave has read chunk 0's keys before step 0 loads chunk 2 over them
  __syncthreads();
  for (int32_t ci = 0; ci < nchunks; ci += 2) {
    step(ci, sa, sb);
    if (ci + 1 < nchunks) step(ci + 1, sb, sa);
  }

  // totals over the four row groups, then the output rows of each tile
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (!on[t]) continue;  // uniform
    const float l_tot = lsum[t][0];  // every row of the ones product holds the column's sum
    if (tok0[t] + nq >= n) continue;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = (uint16_t*)a.out + ((int64_t)(q0 + qi[t]) * a.hq + head[t]) * D + 4 * r;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const __bf16 o0 = (__bf16)(acc[t][j][0] * inv), o1 = (__bf16)(acc[t][j][1] * inv);
      const __bf16 o2 = (__bf16)(acc[t][j][2] * inv), o3 = (__bf16)(acc[t][j][3] * inv);
      uint2 wv;
      wv.x = (uint32_t)__builtin_bit_cast(uint16_t, o0) | ((uint32_t)__builtin_bit_cast(uint16_t, o1) << 16);
      wv.y = (uint32_t)__builtin_bit_cast(uint16_t, o2) | ((uint32_t)__builtin_bit_cast(uint16_t, o3) << 16);
      *reinterpret_cast<uint2*>(orow + 16 * j) = wv;
    }
  }
}

template <int D, int GW>
void launch_prefill_g(PrefillArgs a, int32_t max_q, hipStream_t st) {
  constexpr int BT = 16 * (8 / GW);
  const int64_t halves = (a.hq / a.hkv) / GW;
  a.n_tiles = (max_q + BT - 1) / BT;
  const int64_t n_groups = (int64_t)a.n_seqs * a.hkv * halves;
  const int64_t wgs = (n_groups + kXcds - 1) / kXcds * kXcds * a.n_tiles;
  hipLaunchKernelGGL((prefill_mfma_kernel<D, GW>), dim3((unsigned)wgs), dim3(256), 0, st, a);
}

// Query heads per workgroup for G query heads per KV head: the largest of 8,
// 4, 2, 1 that divides G (a workgroup's 128 rows are 128 / GW tokens of GW
// heads; the G / GW parts of a head group take workgroups of their own).
int32_t prefill_gw(int32_t G) { return G % 8 == 0 ? 8 : G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1; }

template <int D>
void launch_prefill(const PrefillArgs& a, int32_t max_q, hipStream_t st) {
  switch (prefill_gw(a.hq / a.hkv)) {
    case 1: launch_prefill_g<D, 1>(a, max_q, st); break;
    case 2: launch_prefill_g<D, 2>(a, max_q, st); break;
    case 4: launch_prefill_g<D, 4>(a, max_q, st); break;
    default: launch_prefill_g<D, 8>(a, max_q, st); break;
  }
}

}  // namespace
}  // namespace pkv

using pkv::fail;

extern "C" int pkv_paged_attention_prefill(void* out, const void* q, const void* k_cache,
                                           const void* v_cache, const int32_t* d_block_table,
                                           const int32_t* d_context_lens,
                                           const int32_t* d_query_start, int32_t n_seqs,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t num_blocks, int32_t max_blocks_per_seq,
                                           int32_t max_query_len, float scale, pkv_dtype dtype,
                                           pkv_layout k_layout, void* stream) {
  PKV_TRY_BEGIN
  if (n_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq < 0 || max_query_len < 0)
    return fail(PKV_ERR_INVALID_ARG, "bad sizes");
  if (num_q_heads % num_kv_heads) return fail(PKV_ERR_INVALID_ARG, "num_q_heads is not a multiple of num_kv_heads");
  if (!pkv::dtype_valid(dtype)) return fail(PKV_ERR_INVALID_ARG, "bad dtype");
  if (!pkv::layout_valid(k_layout)) return fail(PKV_ERR_INVALID_ARG, "bad key layout");
  if (!pkv::resolve_scale(&scale, head_dim))
    return fail(PKV_ERR_INVALID_ARG, "scale must be 0 (1/sqrt(head_dim)) or finite and positive");
  const int32_t G = num_q_heads / num_kv_heads;
  const bool pow2 = block_size >= 8 && block_size <= 256 && (block_size & (block_size - 1)) == 0;
  if (dtype != PKV_BF16 || (head_dim != 64 && head_dim != 128) || !pow2)
    return fail(PKV_ERR_UNSUPPORTED,
                "prefill needs bf16, head_dim 64/128, block_size a power of two in [8, 256]");
  {
    const int32_t GW = pkv::prefill_gw(G);
    const int64_t bt = 16 * 8 / GW;
    const int64_t groups = (int64_t)n_seqs * num_kv_heads * (G / GW);
    // one-dimensional grid: workgroups x 256 threads must stay below 2^32
    if (((groups + 7) / 8 * 8) * ((max_query_len + bt - 1) / bt) >= (int64_t)1 << 24)
      return fail(PKV_ERR_UNSUPPORTED, "grid too large (2^24 workgroups)");
  }
  if (n_seqs == 0 || max_query_len == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !d_context_lens || !d_query_start || !d_block_table)
    return fail(PKV_ERR_INVALID_ARG, "NULL pointer");
  const uintptr_t mis = (uintptr_t)out | (uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache;
  if (mis % 16) return fail(PKV_ERR_UNSUPPORTED, "prefill needs 16-byte aligned buffers");
  int32_t* err = nullptr;
  int rc = pkv::device_error_word(&err);
  if (rc) return rc;
  pkv::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.table = d_block_table;
  a.ctx = d_context_lens;
  a.qstart = d_query_start;
  a.n_seqs = n_seqs;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.p = block_size;
  a.lp = __builtin_ctz((unsigned)block_size);
  a.ks = pkv::k_strides(k_layout, num_kv_heads, block_size, head_dim);
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.err = err;
  hipStream_t st = (hipStream_t)stream;
  if (head_dim == 128) pkv::launch_prefill<128>(a, max_query_len, st);
  else pkv::launch_prefill<64>(a, max_query_len, st);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return PKV_OK;
  PKV_TRY_END
}
