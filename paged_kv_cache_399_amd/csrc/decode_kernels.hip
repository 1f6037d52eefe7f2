// Paged decode attention for gfx950 (MI355X).
//
// What is computed ("PagedAttention Internals", "The Block Table Map";
// "pagedattention" topic page, third paragraph: attention follows each
// sequence's block table to its keys and values): for sequence b, query head
// h, KV head g = h / G, context length L,
//     out[b,h] = sum_{t<L} softmax_t(scale * q[b,h] . K[t,g]) V[t,g]
// with K[t,g] = k_cache[table[b][t/P], g, t%P, :] and
//      V[t,g] = v_cache[table[b][t/P], g, :, t%P].
//
// Work decomposition.  A sequence's tokens are cut into partitions of T
// tokens (T a power of two, chosen on the host from the batch's size).  A
// workgroup of W waves handles one (partition, KV head) unit and all G query
// heads that share that KV head, so each key/value byte is read from HBM
// once per unit.  A small plan kernel lays the units out: full partitions
// first, the shorter last partitions of every sequence at the end of the
// grid, longest first.  A sequence with one partition writes its output
// directly; otherwise each partition writes (max, sum, normalised output) in
// fp32 to the sequence's partition slot and the merge kernel combines them.
// Summation order depends only on logical token positions, T and W, never on
// where the blocks sit.
//
// Shared blocks ("pagedattention" topic page, fourth paragraph; "PagedAttention
// Internals", "Sharing And Dynamic Growth": forked sequences point at the same
// physical blocks).  When the caller says how many leading tokens each
// sequence holds in the same blocks as the one before it, the plan packs up
// to 16 / G consecutive sharing sequences into one unit for each whole
// partition they share: the matrix-core kernel then gives each packed
// sequence's query heads their own MFMA columns and reads the shared keys and
// values once for the pack.  Each column's arithmetic is what its own unit
// would do, so results are bit-identical with or without packing.  Longer runs
// form wide packs of up to 128 / G sequences, whose shared tokens are read once
// for all their query rows as a dense product (wide_pack_unit; another
// summation order, within the same tolerance).
//
// Partition kernels:
//  * decode_mfma_kernel (bf16, head_dim 64/128, block size 1..64, any G):
//    scores and the value product run on v_mfma_f32_16x16x32_bf16 with the
//    head group (or a pack's head groups) as the 16-wide N dimension, padded
//    with zero queries; a group of more than 16 heads runs as several column
//    sets, one workgroup each.  Each lane loads exactly the 16-byte operand fragments
//    it feeds to the matrix core straight from HBM (keys token-major, values
//    token-minor), with the next 32-token chunk's loads in flight while the
//    current one is computed.  The score fragment a lane receives is already
//    the probability fragment it must feed to the value product, so no data
//    moves between lanes except for the max / sum reductions across the four
//    16-lane rows.
//  * decode_dpp_kernel (G <= 4, bf16 or fp32, head_dim 64/128): vector ALU,
//    DPP row reductions; multi-head attention and fp32 data.
//  * decode_valu_kernel (any other shape within limits): one token per lane
//    for scores, one head_dim element per lane for the value product.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "device_common.hpp"
#include "internal.hpp"
#include "tile_common.hpp"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

struct Plan {
  int32_t* counts;     // [0] units to run (0 if the plan overflowed), [1] full-length units,
                       // [2], [3] the sizing stamp of the call that planned
  int4* seq_info;      // [n_seqs]: (first slot, partials, partitions, leading piece slots);
                       // slots are contiguous
  int2* seq_pack;      // [n_seqs]: (tokens its pack shares or 0, pack size if it leads a pack
                       // else 0), kept between plan passes when one pass does not cover the batch
  int4* work;          // [max_units]: (sequence, first token, end token, sequences in the pack
                       // | (piece + 1) << 16 for a piece of a wide pack's shared partition)
  int2* work_out;      // [max_units]: (partial slot, partials) of the unit's first sequence
  float* part_ml;      // [max_units * Hq * 2] per slot: running max (log2 units), sum
  float* part_o;       // [max_units * Hq * D] per slot: normalised partial output
};

struct DecodeArgs {
  void* out;
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* table;
  const int32_t* ctx;
  const int32_t* shared;  // tokens each sequence holds in its predecessor's blocks, or null
  int32_t n_seqs, hq, hkv, d, p, num_blocks, max_blocks, part_tokens, max_units;
  int32_t pack_max;  // sequences one unit may take (1: no packing)
  int32_t wide_split;  // pieces each whole shared partition of a wide pack is cut into (1: none)
  // The G query heads of a KV head run in gparts column sets of at most gcols
  // heads (one set of G unless G > 16, the matrix-core kernel's columns);
  // each set is a workgroup of its own, in the partition and merge kernels.
  int32_t gparts, gcols;
  KStrides ks;       // key cache: elements between KV heads, between tokens
  int64_t len_cap;   // min(max_blocks * p, max_context_len): longer contexts are clamped
  float scale_log2;  // scale * log2(e): scores are kept in log2 units
  int2 stamp;        // the plan's sizing (partition length, units, packs), hashed on the host
  Plan plan;
  int32_t* err;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float((uint32_t)x << 16);
}

template <typename T>
__device__ __forceinline__ float load_f32(const T* p);
template <>
__device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_f32<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void store_f32(T* p, float v);
template <>
__device__ __forceinline__ void store_f32<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_f32<uint16_t>(uint16_t* p, float v) {
  const __bf16 b = (__bf16)v;  // round to nearest even
  *p = __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Keys and values are read once per decode step: streaming (nontemporal)
// loads keep them from displacing reusable lines and raise read bandwidth.
__device__ __forceinline__ uint4 load_stream16(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ uint2 load_stream8(const uint16_t* p) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return uint2{v.x, v.y};
}

__device__ __forceinline__ uint32_t load_stream4(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

__device__ __forceinline__ uint16_t load_stream2(const uint16_t* p) { return __builtin_nontemporal_load(p); }

// Key/value loads: nontemporal (streaming) for data read once.  Blocks that
// several sequences share are read once per pack of sharers, and every pack
// over the same blocks runs on the same XCD (same KV head); for those, cached
// loads (KEEP) let the next pack find them in that XCD's L2.
template <bool KEEP>
__device__ __forceinline__ uint4 load_kv16(const uint16_t* p) {
  if constexpr (KEEP) return *reinterpret_cast<const uint4*>(p);
  else return load_stream16(p);
}
template <bool KEEP>
__device__ __forceinline__ uint2 load_kv8(const uint16_t* p) {
  if constexpr (KEEP) return *reinterpret_cast<const uint2*>(p);
  else return load_stream8(p);
}
template <bool KEEP>
__device__ __forceinline__ uint32_t load_kv4(const uint16_t* p) {
  if constexpr (KEEP) return *reinterpret_cast<const uint32_t*>(p);
  else return load_stream4(p);
}
template <bool KEEP>
__device__ __forceinline__ uint16_t load_kv2(const uint16_t* p) {
  if constexpr (KEEP) return *p;
  else return load_stream2(p);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ int32_t uniform(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Unit bookkeeping common to the partition kernels.  A unit covers tokens
// [t0, t1) of sequences b .. b + pack - 1 (pack > 1 only for whole shared
// partitions); slot and nparts belong to sequence b.
struct Unit {
  int32_t b, t0, t1, pack, piece, slot, nparts, valid;
};

// A plan made for other sizing (a planned decode whose workspace holds
// another call's plan) runs nothing and is flagged.
__device__ __forceinline__ bool plan_matches(const DecodeArgs& a) {
  return a.plan.counts[2] == a.stamp.x && a.plan.counts[3] == a.stamp.y;
}

__device__ __forceinline__ Unit decode_unit(const DecodeArgs& a, int32_t unit) {
  Unit u;
  if (!plan_matches(a)) {
    if (unit == 0 && threadIdx.x == 0) atomicOr(a.err, PKV_DEVERR_PLAN);
    u.valid = false;
    return u;
  }
  u.valid = unit < a.plan.counts[0];
  if (!u.valid) return u;
  const int4 w = a.plan.work[unit];
  const int2 o = a.plan.work_out[unit];
  u.b = w.x;
  u.t0 = w.y;
  u.t1 = w.z;
  u.pack = w.w & 0xffff;
  u.piece = w.w >> 16;  // 0, or 1 + the piece of a wide pack's split shared partition
  u.slot = o.x;
  u.nparts = o.y;
  return u;
}

// ---------------------------------------------------------------------------
// Plan.  Sequence b of length L has partitions j = 0 .. np - 1 of T tokens
// (np = floor(L/T), plus one ragged partition if L % T != 0 or L == 0).  Its
// partial results occupy slots [first_b, first_b + count_b), contiguous and
// in sequence order: slot first_b + j for partition j, and one extra slot
// when a shared partition is split (below).  Work rows: the full-length
// units first in sequence order, then the shorter units longest first
// (bucketed by length), so the hardware dispatcher, which starts workgroups
// in grid order as slots free up, runs a longest-processing-time-first
// schedule and the launch ends on short units.  Row placement never changes
// results: partials are merged by slot, in partition order.
//
// Packs (pack_max > 1 and a shared-token array given).  Sequence m "joins"
// its predecessor with j_m = floor(min(shared[m], L_m, L_{m-1}) / 32) shared
// 32-token chunks; a run is a maximal stretch of consecutive sequences that
// each join the one before.  A run is cut into packs of pack_max sequences
// from its start; a pack of k >= 2 sequences shares Ls = 32 min j_m over its
// members after the first (equal block ids are transitive, so every member
// holds tokens [0, Ls) in the same blocks as the first).  The first sequence
// runs one pack unit per whole partition below Ls and, if Ls % T != 0, one
// "tail" pack unit over [floor(Ls/T) T, Ls).  A member's split partition
// j0 = floor(Ls/T) then has two pieces: the tail (its extra slot) and its own
// remainder [Ls, min((j0+1) T, L)) (slot first + j0); a member with no
// remainder takes the tail in slot first + j0.  Everything from partition
// j0 + 1 on (from j0 if Ls % T == 0) is the member's own.
// A wide pack (k G > 16 query rows, read as one dense product) costs far more
// per token than a streaming unit, so each of its whole shared partitions is
// cut into wide_split pieces of T / wide_split tokens (one unit each); every
// member keeps nsub = floor(Ls/T) (wide_split - 1) more slots for pieces 1 ..,
// placed before its partition slots (seq_info.w = nsub, partition j at slot
// first + nsub + j).
// One workgroup of NT threads (the smallest of 64, 128, 256 that covers the
// batch, else 1024), one length bucket per thread.
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;  // the plan workgroup for batches of more than 256 sequences
constexpr int kPackMax = 32;        // most sequences in one pack (wide packs)
constexpr int kShareChunk = 32;     // granularity of a pack's shared tokens (the decode chunk)

// Exclusive scans of two non-negative counts at once (packed in 64 bits; each
// total stays below 2^31).
__device__ int2 block_exclusive_scan2(int32_t v0, int32_t v1, int32_t* smem64, int2* total) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nw = blockDim.x >> 6;
  const int64_t v = ((int64_t)v0 << 32) | (uint32_t)v1;
  int64_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  int64_t* sm = reinterpret_cast<int64_t*>(smem64);
  if (lane == 63) sm[wid] = x;
  __syncthreads();
  int64_t before = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int64_t t = sm[w];
    before += w < wid ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = make_int2((int32_t)(tot >> 32), (int32_t)(tot & 0xffffffff));
  const int64_t ex = before + x - v;
  return make_int2((int32_t)(ex >> 32), (int32_t)(ex & 0xffffffff));
}

__device__ int32_t block_exclusive_scan(int32_t v, int32_t* smem, int32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nw = blockDim.x >> 6;
  int32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) smem[wid] = x;
  __syncthreads();
  int32_t before = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int32_t t = smem[w];
    before += w < wid ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

__device__ int32_t block_inclusive_max(int32_t v, int32_t* smem, int32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nw = blockDim.x >> 6;
  int32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x = max(x, y);
  }
  if (lane == 63) smem[wid] = x;
  __syncthreads();
  int32_t before = INT32_MIN, tot = INT32_MIN;
  for (int w = 0; w < nw; ++w) {
    const int32_t t = smem[w];
    if (w < wid) before = max(before, t);
    tot = max(tot, t);
  }
  __syncthreads();
  *total = tot;
  return max(before, x);
}

// The shorter units of sequence b (at most three): a pack's tail (its first
// sequence only), the remainder of a split partition, the ragged partition.
// f(t0, t1, pack, slot) is called for each.
template <typename F>
__device__ __forceinline__ void short_units(int32_t T, int64_t L, int32_t Ls, int32_t k_lead, int32_t first,
                                            F&& f) {
  const int32_t nfull = (int32_t)(L / T);
  const int32_t nshf = Ls / T, tail = Ls - nshf * T;
  if (Ls > 0 && tail > 0) {
    if (k_lead > 0) f(nshf * T, Ls, k_lead, first + nshf);
    const int32_t end = (int32_t)min((int64_t)(nshf + 1) * T, L);
    if (end > Ls) f(Ls, end, 1, first + nshf);
    if (nfull > nshf && L % T != 0) f(nfull * T, (int32_t)L, 1, first + nfull);
  } else if (L % T != 0 || L == 0) {
    f(nfull * T, (int32_t)L, 1, first + nfull);
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void plan_kernel(DecodeArgs a) {
  __shared__ int32_t smem[16];
  __shared__ __align__(8) int32_t smem64[32];
  __shared__ int32_t bucket[NT];  // counts, then the next free offset of each bucket
  // j_m for m in [base - kPackMax, base + NT + kPackMax)
  __shared__ int32_t jt[kPackMax + NT + kPackMax];
  const int32_t T = a.part_tokens;
  const int64_t cap = a.len_cap;
  const int32_t S = a.pack_max;
  const int32_t G = a.hq / a.hkv;
  const int tid = threadIdx.x;
  bucket[tid] = 0;
  if (tid < kPackMax) jt[tid] = 0;  // no sequence before the first
  __syncthreads();
  auto length_of = [&](int32_t b, bool flag) -> int64_t {
    int64_t L = a.ctx[b];
    if (L < 0 || L > cap) {
      if (flag) atomicOr(a.err, PKV_DEVERR_CONTEXT_LEN);
      L = L < 0 ? 0 : cap;
    }
    return L;
  };
  // shared 32-token chunks of sequence m with sequence m - 1 (0: none, or no packing)
  auto joins = [&](int32_t m) -> int32_t {
    if (S < 2 || m <= 0 || m >= a.n_seqs) return 0;
    const int64_t lim = min(length_of(m, false), length_of(m - 1, false));
    int64_t sh = a.shared[m];
    sh = sh < 0 ? 0 : (sh > lim ? lim : sh);
    return (int32_t)(sh / kShareChunk);
  };
  // a unit of c < T tokens: bucket 0 holds the longest (T - 1 tokens)
  const int lg_t = 31 - __builtin_clz((uint32_t)T);  // T is a power of two
  auto bucket_of = [&](int32_t c) -> int32_t {
    return (int32_t)(((int64_t)(T - 1 - c) * NT) >> lg_t);
  };

  // pass 1: slots and full-length rows in sequence order; shorter units counted per bucket
  int32_t row_base = 0, slot_base = 0, run_carry = 0;
  // this thread's last sequence, kept for pass 2 when one pass covers the batch
  int64_t keep_L = 0;
  int32_t keep_first = 0, keep_count = 0, keep_Ls = 0, keep_k = 0;
  for (int32_t base = 0; base < a.n_seqs; base += NT) {
    const int32_t b = base + tid;
    const bool in = b < a.n_seqs;
    int64_t L = 0;
    int32_t nfull = 0, np = 0;
    if (in) {
      L = length_of(b, true);
      nfull = (int32_t)(L / T);
      np = nfull + ((L % T != 0 || L == 0) ? 1 : 0);
    }
    int32_t k = 1, Ls = 0, lead = b;
    if (S >= 2) {  // uniform
      const int32_t jb = in ? joins(b) : 0;
      jt[kPackMax + tid] = jb;
      if (tid < kPackMax) jt[kPackMax + NT + tid] = joins(base + NT + tid);
      // start of the run holding b: the last sequence at or before b that joins nothing
      int32_t cmax;
      const int32_t st = max(run_carry, block_inclusive_max(in && jb == 0 ? b : -1, smem, &cmax));
      run_carry = max(run_carry, cmax);
      // jt is complete: block_inclusive_max synchronised after the writes above
      lead = st + (b - st) / S * S;  // first sequence of b's pack
      if (in) {
        int32_t mn = INT32_MAX;
        for (int32_t i = 1; i < S; ++i) {
          const int32_t jm = jt[kPackMax + lead + i - base];  // lead + i - base in [-31, NT + 31)
          if (jm == 0) break;
          mn = min(mn, jm);
          ++k;
        }
        if (k >= 2) Ls = mn * kShareChunk;
      }
    }
    const int32_t nshf = Ls / T, tail = Ls - nshf * T;
    const int32_t extra = (tail > 0 && L > Ls) ? 1 : 0;
    const bool leader = in && b == lead && k >= 2;
    const int32_t own_start = nshf + (tail > 0 ? 1 : 0);
    // a wide pack cuts each whole shared partition into SW pieces; pieces
    // 1 .. SW - 1 of partition j take the member's slots first + j (SW - 1)
    // + piece - 1, ahead of its partition slots (so nsub = nshf (SW - 1))
    const int32_t SW = (k >= 2 && k * G > 16) ? a.wide_split : 1;
    const int32_t nsub = nshf * (SW - 1), Tw = T / SW;
    const int32_t nrows = in ? (leader ? nshf * SW : 0) + max(nfull - own_start, 0) : 0;
    const int32_t count = in ? np + extra + nsub : 0;
    int2 tot;
    const int2 ex = block_exclusive_scan2(nrows, count, smem64, &tot);
    const int32_t r0 = row_base + ex.x, f0 = slot_base + ex.y;
    if (in) {
      a.plan.seq_info[b] = make_int4(f0, count, np, nsub);
      if (a.n_seqs > NT) a.plan.seq_pack[b] = make_int2(Ls, leader ? k : 0);  // for pass 2
      const int32_t fp = f0 + nsub;  // slot of partition 0
      int32_t row = r0;
      if (leader)
        for (int32_t j = 0; j < nshf; ++j)
          for (int32_t q = 0; q < SW; ++q, ++row)
            if (row < a.max_units) {
              const int32_t code = SW > 1 ? (q + 1) << 16 : 0;
              a.plan.work[row] = make_int4(b, j * T + q * Tw, j * T + (q + 1) * Tw, k | code);
              a.plan.work_out[row] = make_int2(q == 0 ? fp + j : f0 + j * (SW - 1) + q - 1, count);
            }
      for (int32_t j = own_start; j < nfull; ++j, ++row)
        if (row < a.max_units) {
          a.plan.work[row] = make_int4(b, j * T, (j + 1) * T, 1);
          a.plan.work_out[row] = make_int2(fp + j, count);
        }
      short_units(T, L, Ls, leader ? k : 0, fp, [&](int32_t t0, int32_t t1, int32_t, int32_t) {
        atomicAdd(&bucket[bucket_of(t1 - t0)], 1);
      });
      keep_L = L;
      keep_first = fp;
      keep_count = count;
      keep_Ls = Ls;
      keep_k = leader ? k : 0;
    }
    row_base += tot.x;
    slot_base += tot.y;
    if (S >= 2) {
      // carry the last kPackMax entries over as the next chunk's look-behind
      __syncthreads();
      if (tid < kPackMax) jt[tid] = jt[NT + tid];
      __syncthreads();
    }
  }
  __syncthreads();  // every short-unit count is in before the bucket totals are read
  const int32_t F = row_base, FS = slot_base;
  int32_t R;
  const int32_t cnt = bucket[tid];
  const int32_t off = block_exclusive_scan(cnt, smem, &R);
  bucket[tid] = off;
  __syncthreads();
  const bool overflow = (int64_t)F + R > a.max_units || FS > a.max_units;

  // pass 2: shorter units, longest bucket first (order inside a bucket is free)
  for (int32_t base = 0; base < a.n_seqs; base += NT) {
    const int32_t b = base + tid;
    if (b < a.n_seqs) {
      int64_t L = keep_L;
      int32_t first = keep_first, count = keep_count, Ls = keep_Ls, kl = keep_k;
      if (a.n_seqs > NT) {  // uniform: read back what this thread wrote in pass 1
        L = length_of(b, false);
        const int4 si = a.plan.seq_info[b];
        const int2 sp = a.plan.seq_pack[b];
        first = si.x + si.w;
        count = si.y;
        Ls = sp.x;
        kl = sp.y;
      }
      short_units(T, L, Ls, kl, first, [&](int32_t t0, int32_t t1, int32_t k, int32_t slot) {
        const int32_t row = F + atomicAdd(&bucket[bucket_of(t1 - t0)], 1);
        if (!overflow) {
          a.plan.work[row] = make_int4(b, t0, t1, k);
          a.plan.work_out[row] = make_int2(slot, count);
        }
      });
    }
  }
  if (tid == 0) {
    if (overflow) atomicOr(a.err, PKV_DEVERR_WORK_OVERFLOW);
    a.plan.counts[0] = overflow ? 0 : F + R;  // run nothing rather than overlapping rows
    a.plan.counts[1] = F;
    a.plan.counts[2] = a.stamp.x;
    a.plan.counts[3] = a.stamp.y;
  }
}

// ---------------------------------------------------------------------------
// Matrix-core partition kernel.
//
// Lane l of a wave: n = l % 16 (query head within the group, the MFMA N
// index) and r = l / 16 (row group).  A 32-token chunk starting at c0:
//   scores  S^T[tok, n] = K[tok, :] . Q[n, :] as two 16x16x32 MFMA chains
//           over head_dim: chain X holds tokens c0 + 8r' + i (i < 4) in
//           output row 4r' + i, chain Y holds c0 + 8r' + 4 + i.  So lane l
//           receives the scores of head n for tokens c0 + 8r + s, s = 0..7.
//   values  O^T[dim, n] += V^T[dim, tok] P^T[tok, n] with the MFMA reduction
//           index k = 8r + s mapped to token c0 + 8r + s: the B operand of
//           lane l is exactly its own eight probabilities, and its A operand
//           is the 16-byte run v_cache[blk, g, dim, off .. off+7].
// Key fragments: lane l reads 16 bytes of token row (chain X/Y row l % 16) at
// head_dim offset 32 i + 8 r for MFMA step i.
// ---------------------------------------------------------------------------
template <int D, int P>
struct MfmaChunk {
  static constexpr int KI = D / 32;  // MFMA steps over head_dim (scores)
  static constexpr int NJ = D / 16;  // 16-row output tiles over head_dim (values)
  uint4 kx[KI], ky[KI], v[NJ];
};

// ---------------------------------------------------------------------------
// Wide packs.  When sequences that share blocks form packs of more than 16
// MFMA columns (up to 128 / G sequences, pack * G query rows), a pack unit
// reads the shared tokens [t0, t1) of its first sequence once for all its
// rows: a dense product, as in paged prefill.  Four waves take two 16-row
// tiles each (row 16 k + n of tile k is query head (row % G) of pack member
// row / G); 64-key chunks go straight from HBM into LDS (each wave loads one
// 16-key group, which lies in one block, or in two with blocks of 8), keys
// two chunks ahead and values one, and the score products of chunk i + 1 are
// issued between the softmax instructions of chunk i.  Each row's (max, sum,
// normalised output) goes to its member's partial slot, exactly where the
// narrow pack path puts that column's partial.
// ---------------------------------------------------------------------------
constexpr int kWideRows = 128;     // query rows of a wide pack unit (eight 16-row tiles)
constexpr int kWideMaxPack = 32;   // sequences a wide pack may hold
constexpr int kWideTab = 1024;     // block-table entries of one unit (T / P <= 1024)
constexpr float kWideSlack = 8.f;  // log2 headroom before the running reference moves

template <int D>
struct WideLds {
  uint16_t k[2][64 * D];  // key rows, 16-byte pieces swizzled (kswz)
  uint16_t v[2][64 * D];  // [8-key group][head_dim][8 keys]
  int32_t tab[kWideTab];
  int32_t row_slot[kWideRows], row_np[kWideRows];
};

template <int D, int P>
__device__ __forceinline__ void wide_pack_unit(const DecodeArgs& a, const Unit& u, int32_t g,
                                               WideLds<D>& L) {
  static_assert(P % 8 == 0, "a 16-key group must lie in one block, or in two of 8");
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  typedef __attribute__((address_space(1))) void* gptr_t;
  constexpr int CH = 64, NH = 2, KI = D / 32, NJ = D / 16;
  constexpr int KU = D / 32, KR = 512 / D, VPG = D / 64;  // staging loads per wave, rows per key load
  constexpr int NSEG = NH * KI;                            // fused score / softmax segments
  constexpr int NE = 2 * NH * 8;                           // probabilities per lane per chunk
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int nq = lane & 15, r = lane >> 4;
  const int32_t G = a.hq / a.hkv;
  const int32_t rows = u.pack * G;
  const int32_t T = a.part_tokens;
  const int32_t t0 = u.t0, t1 = u.t1;
  const float c = a.scale_log2;

  // per row: the partial slot and partial count of its member.  Piece q >= 1
  // of shared partition j: slot first + j (SW - 1) + q - 1; otherwise the
  // narrow pack path's column rule, after the member's nsub piece slots
  if (tid < rows) {
    const int4 si = a.plan.seq_info[u.b + tid / G];
    const int32_t j = t0 / T;
    if (u.piece >= 2) {
      L.row_slot[tid] = si.x + j * (a.wide_split - 1) + u.piece - 2;
    } else {
      const bool tail = u.piece == 0 && (t1 & (T - 1)) != 0;
      L.row_slot[tid] = si.x + si.w + (tail && si.y > si.w + si.z ? si.z : j);
    }
    L.row_np[tid] = si.y;
  }
  // the first sequence's block ids of keys [t0, t1)
  const int32_t* trow = a.table + (int64_t)u.b * a.max_blocks;
  const int32_t blk0 = t0 / P;
  const int32_t nblk = min((t1 - 1) / P - blk0 + 1, kWideTab);
  for (int i = tid; i < nblk; i += 256) {
    int32_t e = trow[blk0 + i];
    if ((uint32_t)e >= (uint32_t)a.num_blocks) {
      atomicOr(a.err, PKV_DEVERR_TABLE_ENTRY);
      e = 0;
    }
    L.tab[i] = e;
  }
  // query fragments: column nq of tile k (= 2 w + t) is row 16 k + nq;
  // padding rows repeat the last row and are not written
  bf16x8 qf[2][KI];
  int32_t row_of[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int32_t row = 16 * (2 * w + t) + nq;
    row_of[t] = row;
    const int32_t rc = min(row, rows - 1);
    const int32_t mem = rc / G, hh = rc - mem * G;
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)(u.b + mem) * a.hq + g * G + hh) * D + 8 * r;
#pragma unroll
    for (int i = 0; i < KI; ++i) qf[t][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + 32 * i));
  }

  const uint16_t* kc = (const uint16_t*)a.kc;
  const uint16_t* vc = (const uint16_t*)a.vc;
  const int64_t blk_stride = (int64_t)a.hkv * P * D;
  const int64_t khead = (int64_t)g * a.ks.head, vhead = (int64_t)g * P * D;
  const int32_t nchunks = (t1 - t0 + CH - 1) / CH;

  // staging: wave w loads keys [c0 + 16 w, + 16); a group past t1 reads the
  // last group that holds keys (in bounds) and its values are zeroed.  With
  // blocks of 8 the group's keys 8..15 come from a second block (the unit's
  // last block where the group ends early); each load covers KR = 4 or 8 key
  // rows and each value load one 8-key group, so every load stays inside one
  // block.
  const int wkr = lane / (D / 8), wdc = lane % (D / 8);
  uint32_t kdoff[KU];  // bytes from the first key row of the load's block
#pragma unroll
  for (int uu = 0; uu < KU; ++uu) {
    const int row = uu * KR + wkr;
    const int grow = P == 8 && uu * KR >= 8 ? row - 8 : row;
    kdoff[uu] = (uint32_t)(grow * a.ks.tok * 2 + (wdc ^ kswz<D>(16 * w + row)) * 16);
  }
  const uint32_t vdoff = (uint32_t)(lane * P * 2);
  const int32_t blk_last = (t1 - 1) / P;
  auto group_base = [&](int32_t c0, int64_t& offA, int64_t& offB) -> int32_t {
    const int32_t kb = c0 + 16 * w;
    const int32_t kl = min(kb, t1 - 1) & ~15;
    const int32_t ba = __builtin_amdgcn_readfirstlane(L.tab[kl / P - blk0]);
    int32_t bb = ba;
    if constexpr (P == 8) bb = __builtin_amdgcn_readfirstlane(L.tab[min(kl / P + 1, blk_last) - blk0]);
    offA = (int64_t)ba * blk_stride;
    offB = (int64_t)bb * blk_stride;
    return kl & (P - 1);
  };
  auto kload = [&](int32_t c0, int buf) {
    int64_t oa, ob;
    const int32_t o = group_base(c0, oa, ob);
    const char* ka = (const char*)(kc + oa + khead + (int64_t)o * a.ks.tok);
    const char* kb2 = (const char*)(kc + ob + khead);
#pragma unroll
    for (int uu = 0; uu < KU; ++uu)
      __builtin_amdgcn_global_load_lds((gptr_t)((P == 8 && uu * KR >= 8 ? kb2 : ka) + kdoff[uu]),
                                       (lds_ptr_t)&L.k[buf][(16 * w + uu * KR) * D], 16, 0, 0);
  };
  auto vslot = [&](int buf, int uu) -> uint16_t* {
    return &L.v[buf][((2 * w + uu / VPG) * D + (uu % VPG) * 64) * 8];
  };
  auto vload = [&](int32_t c0, int buf) {
    int64_t oa, ob;
    const int32_t o = group_base(c0, oa, ob);
    const char* va = (const char*)(vc + oa + vhead + o);
    const char* vb2 = (const char*)(vc + ob + vhead);
#pragma unroll
    for (int uu = 0; uu < KU; ++uu) {
      const char* vb = P == 8 ? (uu / VPG ? vb2 : va) : va + (uu / VPG) * 16;
      __builtin_amdgcn_global_load_lds((gptr_t)(vb + (uu % VPG) * 64 * P * 2 + vdoff),
                                       (lds_ptr_t)vslot(buf, uu), 16, 0, 0);
    }
  };
  auto vfix = [&](int32_t c0, int buf) {
    const int32_t kb = c0 + 16 * w;
    if (kb + 16 <= t1) return;  // uniform
#pragma unroll
    for (int uu = 0; uu < KU; ++uu) {
      const int32_t tg = kb + 8 * (uu / VPG);
      const int32_t nv = tg >= t1 ? 0 : min(t1 - tg, 8);
      const uint32_t m0 = nv >= 2 ? 0xffffffffu : (nv == 1 ? 0x0000ffffu : 0u);
      const uint32_t m1 = nv >= 4 ? 0xffffffffu : (nv == 3 ? 0x0000ffffu : 0u);
      const uint32_t m2 = nv >= 6 ? 0xffffffffu : (nv == 5 ? 0x0000ffffu : 0u);
      const uint32_t m3 = nv >= 8 ? 0xffffffffu : (nv == 7 ? 0x0000ffffu : 0u);
      uint4* sl = reinterpret_cast<uint4*>(vslot(buf, uu) + lane * 8);
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
  f32x4 lsum[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  float m_run[2] = {-INFINITY, -INFINITY}, m_old[2];
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  const int krow_x = 8 * (nq >> 2) + (nq & 3);
  const int kx = kswz<D>(krow_x);

  struct Sc {
    f32x4 x[2][NH], y[2][NH];
  };
  auto scores = [&](int buf) -> Sc {
    const uint16_t* kl = L.k[buf];
    Sc sc;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int h = 0; h < NH; ++h) sc.x[t][h] = sc.y[t][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const int cb = ((4 * i + r) ^ kx) * 8;
        const bf16x8 ax = *reinterpret_cast<const bf16x8*>(&kl[(32 * h + krow_x) * D + cb]);
        const bf16x8 ay = *reinterpret_cast<const bf16x8*>(&kl[(32 * h + krow_x + 4) * D + cb]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          sc.x[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax, qf[t][i], sc.x[t][h], 0, 0, 0);
          sc.y[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ay, qf[t][i], sc.y[t][h], 0, 0, 0);
        }
      }
    return sc;
  };
  // keys at or past t1 in the last chunk (uniform test)
  auto mask = [&](Sc& sc, int32_t c0) {
    if (c0 + CH > t1) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int32_t kx0 = c0 + 32 * h + 8 * r + e;
            sc.x[t][h][e] = kx0 < t1 ? sc.x[t][h][e] : -INFINITY;
            sc.y[t][h][e] = kx0 + 4 < t1 ? sc.y[t][h][e] : -INFINITY;
          }
    }
  };
  float mc[2];
  bool moved;
  auto rowmax = [&](const Sc& cu, int t) {
    float x = cu.x[t][0][0];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) x = fmaxf(x, fmaxf(cu.x[t][h][e], cu.y[t][h][e]));
    const float cm = pair_max16(pair_max32(x));
    const bool up = (cm - m_run[t]) * c > kWideSlack;
    m_old[t] = m_run[t];
    m_run[t] = up ? fmaxf(m_run[t], cm) : m_run[t];
    moved |= up;
    mc[t] = m_run[t] * c;
  };
  auto prob = [&](const Sc& cu, bf16x8 (&pb)[2][NH], int q) {
    const int e = q & 3, xy = (q >> 2) & 1, h = (q >> 3) % NH, t = (q >> 3) / NH;
    const float sv = xy ? cu.y[t][h][e] : cu.x[t][h][e];
    pb[t][h][e + 4 * xy] = (__bf16)fast_exp2(fmaf(sv, c, -mc[t]));
  };
  // softmax of `cu` fused with the score products of the next chunk into `nx`
  auto fused = [&](int kbuf, Sc& nx, const Sc& cu, bf16x8 (&pb)[2][NH]) {
    const uint16_t* kl = L.k[kbuf];
    bf16x8 ax[NSEG], ay[NSEG];
    auto kread = [&](int k) {
      const int h = k / KI, i = k % KI;
      const int cb = ((4 * i + r) ^ kx) * 8;
      ax[k] = *reinterpret_cast<const bf16x8*>(&kl[(32 * h + krow_x) * D + cb]);
      ay[k] = *reinterpret_cast<const bf16x8*>(&kl[(32 * h + krow_x + 4) * D + cb]);
    };
    auto kmfma = [&](int k) {
      const int h = k / KI, i = k % KI;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        nx.x[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax[k], qf[t][i], i ? nx.x[t][h] : f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        nx.y[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ay[k], qf[t][i], i ? nx.y[t][h] : f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      }
    };
    kread(0);
    if (NSEG > 1) kread(1);
#pragma unroll
    for (int k = 0; k < NSEG; ++k) {
      if (k + 2 < NSEG) kread(k + 2);
      kmfma(k);
      if (k < 2) {
        rowmax(cu, k);
      } else {
        constexpr int per = (NE + NSEG - 3) / (NSEG - 2);
#pragma unroll
        for (int q = (k - 2) * per; q < (k - 1) * per && q < NE; ++q) prob(cu, pb, q);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto softmax = [&](const Sc& cu, bf16x8 (&pb)[2][NH]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) rowmax(cu, t);
#pragma unroll
    for (int q = 0; q < NE; ++q) prob(cu, pb, q);
  };
  auto values = [&](int buf, const bf16x8 (&pb)[2][NH]) {
    const uint16_t* vl = L.v[buf];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int h = 0; h < NH; ++h) lsum[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[t][h], lsum[t], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&vl[((4 * h + r) * D + 16 * j + nq) * 8]);
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[t][h], acc[t][j], 0, 0, 0);
      }
  };

  // prologue: keys of chunks 0 and 1, values of chunk 0
  __syncthreads();  // table window and row slots
  kload(t0, 0);
  vload(t0, 0);
  if (nchunks > 1) kload(t0 + CH, 1);
  __builtin_amdgcn_s_waitcnt(0);
  vfix(t0, 0);
  __syncthreads();
  auto step = [&](int32_t ci, Sc& cur, Sc& nxt) {
    const int32_t c0 = t0 + ci * CH;
    const bool more = ci + 1 < nchunks, more2 = ci + 2 < nchunks;  // uniform
    if (more2) kload(c0 + 2 * CH, ci & 1);
    if (more) vload(c0 + CH, (ci + 1) & 1);
    mask(cur, c0);
    bf16x8 pb[2][NH];
    moved = false;
    if (more) {
      fused((ci + 1) & 1, nxt, cur, pb);
    } else {
      softmax(cur, pb);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int h = 0; h < NH; ++h) asm volatile("" : "+v"(pb[t][h]));
    if (__builtin_amdgcn_ballot_w64(moved) != 0) {  // rare: a reference moved
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float alpha = fast_exp2((m_old[t] - m_run[t]) * c);
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[t][j] *= alpha;
        lsum[t] *= alpha;
      }
    }
    values(ci & 1, pb);
    __builtin_amdgcn_s_waitcnt(0);
    if (more) vfix(c0 + CH, (ci + 1) & 1);
    __syncthreads();
  };
  Sc sa = scores(0), sb;
  // every wave has read chunk 0's keys before step 0 loads chunk 2 over them
  __syncthreads();
  for (int32_t ci = 0; ci < nchunks; ci += 2) {
    step(ci, sa, sb);
    if (ci + 1 < nchunks) step(ci + 1, sb, sa);
  }

  // per row: (reference max in log2 units, sum, normalised output) to the
  // member's slot, or the output itself for a member with one partial
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int32_t row = row_of[t];
    if (row >= rows) continue;
    const int32_t mem = row / G, hh = row - mem * G;
    const int32_t qh = g * G + hh, seq = u.b + mem;
    const float l = lsum[t][0];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int32_t slot = L.row_slot[row], np = L.row_np[row];
    if (np == 1) {
      uint16_t* orow = (uint16_t*)a.out + ((int64_t)seq * a.hq + qh) * D + 4 * r;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) store_f32(orow + 16 * j + e, acc[t][j][e] * inv);
    } else {
      float* po = a.plan.part_o + ((int64_t)slot * a.hq + qh) * D + 4 * r;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const f32x4 x = acc[t][j] * inv;
        __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(po + 16 * j));
      }
      if (r == 0) {
        float* ml = a.plan.part_ml + ((int64_t)slot * a.hq + qh) * 2;
        ml[0] = m_run[t] * c;
        ml[1] = l;
      }
    }
  }
}

// Workgroup of W waves per (partition, KV head) unit.  Wave w streams the
// tokens [t0 + w TW, t0 + (w + 1) TW) of the partition (TW = T / W) with its
// own running max, sum and accumulator; the W states are combined through
// LDS at the end.  So a partial result goes to HBM once per workgroup, not
// once per wave: partial-result writes interleaved with the key/value read
// stream cost far more than their byte count.
template <int D, int P, int W, bool MIXED>
__global__ __launch_bounds__(64 * W, W == 4 ? 2 : 1) void decode_mfma_kernel(DecodeArgs a) {
  using Chunk = MfmaChunk<D, P>;
  constexpr int KI = Chunk::KI, NJ = Chunk::NJ;
  constexpr int CH = 32;     // tokens per chunk
  constexpr int DP = D + 4;  // padded LDS row of one head's accumulator
  static_assert((P < 8 || P % 8 == 0) && (P <= CH ? CH % P == 0 : P % CH == 0), "block size");
  // LDS: the combine buffers of this path, or (wide pack units, compiled into
  // the kernel that batches with packs launch) the wide path's staging, in
  // one allocation
  struct NarrowLds {
    float red_o[W][16][DP];
    float red_m[W][16], red_l[W][16];
    int32_t tab_lds[W][P < 8 ? 512 : 1];
    int32_t col_slot[16], col_np[16];  // per column of a pack: partial slot, partitions
  };
  constexpr bool kWide = MIXED && W == 4 && P % 8 == 0;
  constexpr size_t kLdsBytes =
      kWide && sizeof(WideLds<D>) > sizeof(NarrowLds) ? sizeof(WideLds<D>) : sizeof(NarrowLds);
  __shared__ __align__(16) unsigned char lds_raw[kLdsBytes];
  NarrowLds& nl = *reinterpret_cast<NarrowLds*>(lds_raw);
  auto& red_o = nl.red_o;
  auto& red_m = nl.red_m;
  auto& red_l = nl.red_l;
  auto& tab_lds = nl.tab_lds;
  auto& col_slot = nl.col_slot;
  auto& col_np = nl.col_np;

  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  // workgroup: (unit, KV head g, column set `part` of g's query heads)
  // (column sets run only in the cached-load variant, MIXED: the other one
  // compiles for one set)
  const int32_t gparts = MIXED ? a.gparts : 1;
  const int32_t hkv_v = a.hkv * gparts;
  const int32_t unit = blockIdx.x / hkv_v;
  const int32_t gv = blockIdx.x - unit * hkv_v;
  const int32_t g = gparts == 1 ? gv : gv / gparts, part = gv - g * gparts;
  if (unit >= a.max_units) return;  // uniform over the workgroup
  const Unit u = decode_unit(a, unit);
  if (!u.valid) return;             // uniform over the workgroup
  const int32_t G = a.hq / a.hkv;
  if constexpr (kWide) {
    if (u.pack > 1 && u.pack * G > 16) {  // uniform: a pack wider than the MFMA columns
      wide_pack_unit<D, P>(a, u, g, *reinterpret_cast<WideLds<D>*>(lds_raw));
      return;
    }
  }
  const int n = lane & 15, r = lane >> 4;
  // MFMA column n: query head h0 + n % GC of pack member n / GC (the unit's
  // own sequence when the pack is one sequence; packs have one column set,
  // GC = G); columns >= NC are padding
  const int32_t GC = MIXED ? a.gcols : G;
  const int32_t h0 = g * G + part * GC;
  int32_t NC, mem, head;
  if (gparts == 1) {  // uniform: one column set (pack members, G heads each)
    NC = u.pack * G;
    mem = n / G;
    head = h0 + (n - mem * G);
  } else {  // a column set of one sequence: heads h0 .. h0 + NC - 1
    NC = min(GC, G - part * GC);
    mem = 0;
    head = h0 + n;
  }
  const bool head_ok = n < NC;
  if (u.pack > 1 && threadIdx.x < NC) {
    // a shared piece of partition j = t0 / T of every member: slot first + j,
    // except a tail (t1 % T != 0) of a member that continues past it, which
    // goes to its extra slot first + partitions (narrow packs hold no split
    // pieces: si.w = 0)
    const int4 si = a.plan.seq_info[u.b + (int32_t)threadIdx.x / G];
    const bool tail = (u.t1 & (a.part_tokens - 1)) != 0;
    col_slot[threadIdx.x] = si.x + si.w + (tail && si.y > si.w + si.z ? si.z : u.t0 / a.part_tokens);
    col_np[threadIdx.x] = si.y;
  }

  const uint16_t* kc = (const uint16_t*)a.kc;
  const uint16_t* vc = (const uint16_t*)a.vc;
  const int64_t blk_stride = (int64_t)a.hkv * P * D;  // elements per physical block
  const int64_t head_off = (int64_t)g * P * D;        // value tile of head g
  const int64_t khead_off = (int64_t)g * a.ks.head;   // first key row of head g
  const int32_t ktok = a.ks.tok;                      // elements between key rows

  f32x4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale_log2;

  const int32_t TW = a.part_tokens / W;  // a multiple of the chunk length
  const int32_t s0 = u.t0 + w * TW;
  const int32_t s1 = min(u.t1, s0 + TW);
  if (s1 > s0) {
    // query fragments (B operand of the score MFMA): head n, dims 32 i + 8 r
    bf16x8 qf[KI];
    {
      const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)(u.b + mem) * a.hq + head) * D + 8 * r;
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        uint4 x = head_ok ? *reinterpret_cast<const uint4*>(qrow + 32 * i) : uint4{0, 0, 0, 0};
        qf[i] = __builtin_bit_cast(bf16x8, x);
      }
    }
    const int32_t* trow = a.table + (int64_t)u.b * a.max_blocks;
    // Block-table window of 64 KW blocks, entry wb + 64 k + i read by lane i.
    // Blocks of 8 tokens or more: one register (KW = 1), picked with uniform
    // lane reads.  Shorter blocks: KW = 8 / P entries per lane, so a window
    // still covers 512 tokens, kept in this wave's own LDS rows (written and
    // read by this wave only; its LDS operations complete in order).
    constexpr int KW = P < 8 ? 8 / P : 1;
    const int32_t last_blk = (s1 - 1) / P;
    int32_t* tab_row = tab_lds[w];
    int32_t tabv = 0;
    auto load_window = [&](int32_t base) {
#pragma unroll
      for (int k = 0; k < KW; ++k) {
        int32_t e = 0;
        if (base + 64 * k + lane <= last_blk) {
          e = trow[base + 64 * k + lane];
          if ((uint32_t)e >= (uint32_t)a.num_blocks) {
            atomicOr(a.err, PKV_DEVERR_TABLE_ENTRY);
            e = 0;
          }
        }
        if constexpr (P >= 8) tabv = e;
        else tab_row[64 * k + lane] = e;
      }
    };
    int32_t wb = 0, wlast = 0;
    const int32_t krow_x = 8 * (n >> 2) + (n & 3);  // token of chain-X row n within the chunk

    // Loads of one chunk; addresses are clamped to the window's last token.
    // A chunk spans at most NBC blocks; their ids are read from the window
    // with uniform lane reads and each lane picks its own.
    constexpr int NBC = CH / P > 1 ? CH / P : 1;
    auto issue = [&](Chunk& f, int32_t c0, auto keep_tag) {
      constexpr bool KEEP = decltype(keep_tag)::value;
      const int32_t tx = min(c0 + krow_x, wlast);
      const int32_t ty = min(c0 + krow_x + 4, wlast);
      if constexpr (P >= 8) {
        const int32_t cb = min(c0, wlast) / P;  // uniform: the chunk's first block
        int32_t bid[NBC];
        if constexpr (NBC <= 2) {
#pragma unroll
          for (int k = 0; k < NBC; ++k) bid[k] = __builtin_amdgcn_readlane(tabv, min(cb + k - wb, 63));
        }
        auto pick = [&](int32_t t) -> int32_t {
          if constexpr (NBC > 2) {
            // more than two blocks per chunk: a lane permute of the window
            return __builtin_amdgcn_ds_bpermute((t / P - wb) << 2, tabv);
          } else {
            const int32_t idx = t / P - cb;
            int32_t v = bid[0];
#pragma unroll
            for (int k = 1; k < NBC; ++k) v = idx == k ? bid[k] : v;
            return v;
          }
        };
        // rows tx and ty (tx + 4 unless clamped) lie in one block: P >= 8
        const int32_t pk = pick(tx);
        const uint16_t* kb = kc + (int64_t)pk * blk_stride + khead_off + 8 * r;
        const uint16_t* kxp = kb + (tx % P) * ktok;
        const uint16_t* kyp = kb + (ty % P) * ktok;
#pragma unroll
        for (int i = 0; i < KI; ++i) {
          f.kx[i] = load_kv16<KEEP>(kxp + 32 * i);
          f.ky[i] = load_kv16<KEEP>(kyp + 32 * i);
        }
        // values: tokens c0 + 8 r .. +7 of head_dim rows 16 j + n
        const int32_t tv = min(c0 + 8 * r, wlast);
        const int32_t pv = pick(tv);
        const uint16_t* vb = vc + (int64_t)pv * blk_stride + head_off + (int64_t)n * P + ((tv % P) & ~7);
        if constexpr (P > CH) {
          // A value row of one dim spans several chunks: the chunks before
          // the row's last use cached loads, so the next one finds the rest
          // of the line in L2; the last reader streams (uniform branch).
          if ((min(c0, wlast) % P) < P - CH) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) f.v[j] = *reinterpret_cast<const uint4*>(vb + 16 * j * P);
          } else {
#pragma unroll
            for (int j = 0; j < NJ; ++j) f.v[j] = load_kv16<KEEP>(vb + 16 * j * P);
          }
        } else {
#pragma unroll
          for (int j = 0; j < NJ; ++j) f.v[j] = load_kv16<KEEP>(vb + 16 * j * P);
        }
      } else {
        // Blocks of fewer than 8 tokens: each lane reads its entries from the
        // wave's LDS window
        auto pick = [&](int32_t t) -> int32_t { return tab_row[t / P - wb]; };
        const uint16_t* kxp = kc + (int64_t)pick(tx) * blk_stride + khead_off + 8 * r + (tx % P) * ktok;
        const uint16_t* kyp = kc + (int64_t)pick(ty) * blk_stride + khead_off + 8 * r + (ty % P) * ktok;
#pragma unroll
        for (int i = 0; i < KI; ++i) {
          f.kx[i] = load_kv16<KEEP>(kxp + 32 * i);
          f.ky[i] = load_kv16<KEEP>(kyp + 32 * i);
        }
        // values: tokens c0 + 8 r .. +7 of head_dim rows 16 j + n, as 8 / P
        // runs of P tokens (2 P bytes) from as many blocks; each run starts a
        // block, clamped to the block of the window's last token
        constexpr int NPC = 8 / P;
        const int32_t vlast_blk = wlast - wlast % P;
        const uint16_t* vp[NPC];
#pragma unroll
        for (int pi = 0; pi < NPC; ++pi) {
          const int32_t t = min(c0 + 8 * r + pi * P, vlast_blk);
          vp[pi] = vc + (int64_t)pick(t) * blk_stride + head_off + (int64_t)n * P;
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          uint32_t wv[4];
          if constexpr (P == 4) {
#pragma unroll
            for (int pi = 0; pi < 2; ++pi) {
              const uint2 x = load_kv8<KEEP>(vp[pi] + 16 * j * P);
              wv[2 * pi] = x.x;
              wv[2 * pi + 1] = x.y;
            }
          } else if constexpr (P == 2) {
#pragma unroll
            for (int pi = 0; pi < 4; ++pi) wv[pi] = load_kv4<KEEP>(vp[pi] + 16 * j * P);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              wv[e] = (uint32_t)load_kv2<KEEP>(vp[2 * e] + 16 * j) |
                      ((uint32_t)load_kv2<KEEP>(vp[2 * e + 1] + 16 * j) << 16);
          }
          f.v[j] = uint4{wv[0], wv[1], wv[2], wv[3]};
        }
      }
    };

    auto compute = [&](Chunk& f, int32_t c0) {
      f32x4 sx = {0.f, 0.f, 0.f, 0.f}, sy = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        sx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f.kx[i]), qf[i], sx, 0, 0, 0);
        sy = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f.ky[i]), qf[i], sy, 0, 0, 0);
      }
      float s[8] = {sx[0], sx[1], sx[2], sx[3], sy[0], sy[1], sy[2], sy[3]};
      if (c0 + CH > s1) {  // ragged chunk (uniform): mask tokens >= s1
        const int32_t nv = min(max(s1 - (c0 + 8 * r), 0), 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = e < nv ? s[e] : -INFINITY;
        // zero the value columns of masked tokens so stale data cannot leak
        const uint32_t m0 = nv >= 2 ? 0xffffffffu : (nv == 1 ? 0x0000ffffu : 0u);
        const uint32_t m1 = nv >= 4 ? 0xffffffffu : (nv == 3 ? 0x0000ffffu : 0u);
        const uint32_t m2 = nv >= 6 ? 0xffffffffu : (nv == 5 ? 0x0000ffffu : 0u);
        const uint32_t m3 = nv >= 8 ? 0xffffffffu : (nv == 7 ? 0x0000ffffu : 0u);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          f.v[j].x &= m0;
          f.v[j].y &= m1;
          f.v[j].z &= m2;
          f.v[j].w &= m3;
        }
      }
      float cm = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                       fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
      cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
      cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
      const float m_new = fmaxf(m_run, cm);
      const float alpha = fast_exp2((m_run - m_new) * c);
      const float mc = m_new * c;
      bf16x8 pb;
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 x = (__bf16)fast_exp2(fmaf(s[e], c, -mc));
        pb[e] = x;
        psum += (float)x;
      }
      l_run = fmaf(l_run, alpha, psum);
      m_run = m_new;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        acc[j] *= alpha;
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f.v[j]), pb, acc[j], 0, 0, 0);
      }
    };

    // Windows of 64 blocks (one table entry per lane).  Window starts are
    // multiples of 64 P tokens past s0 (itself a multiple of the chunk
    // length), so chunks never straddle two windows.  Within a window the
    // next chunk's loads are in flight while the current one is computed;
    // the prefetch past the window end reads clamped, in-bounds addresses.
    auto stream = [&](auto keep_tag) {
      for (int32_t ws = s0; ws < s1;) {
        wb = uniform(ws / P);
        const int32_t we = min(s1, (wb + 64 * KW) * P);
        wlast = we - 1;
        load_window(wb);
        Chunk f0, f1;
        int32_t c0 = ws;
        issue(f0, c0, keep_tag);
        while (true) {
          issue(f1, c0 + CH, keep_tag);
          compute(f0, c0);
          c0 += CH;
          if (c0 >= we) break;
          issue(f0, c0 + CH, keep_tag);
          compute(f1, c0);
          c0 += CH;
          if (c0 >= we) break;
        }
        ws = we;
      }
    };
    // a pack's tokens are shared by all its members and by the packs after
    // it: cached loads; everything else streams.  Only batches with packs
    // get the second copy of the loop (MIXED).
    if constexpr (MIXED) {
      if (u.pack > 1) stream(std::true_type{});  // uniform
      else stream(std::false_type{});
    } else {
      stream(std::false_type{});
    }
  }

  // this wave's state -> LDS; the four row groups hold disjoint token subsets
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (r == 0) {
    red_m[w][n] = m_run;
    red_l[w][n] = l_tot;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    *reinterpret_cast<f32x4*>(&red_o[w][n][16 * j + 4 * r]) = acc[j];
  __syncthreads();

  // combine the W waves: out = sum_v 2^((m_v - M) c) o_v / sum_v 2^((m_v - M) c) l_v
  for (int32_t e = threadIdx.x; e < NC * D; e += 64 * W) {
    const int32_t h = e / D, dd = e - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < W; ++v)
      if (red_l[v][h] > 0.f) M = fmaxf(M, red_m[v][h]);
    float sum = 0.f, o = 0.f;
#pragma unroll
    for (int v = 0; v < W; ++v) {
      const float lv = red_l[v][h];
      if (lv > 0.f) {
        const float wt = fast_exp2((red_m[v][h] - M) * c);
        sum = fmaf(lv, wt, sum);
        o = fmaf(wt, red_o[v][h][dd], o);
      }
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    const int32_t hm = gparts == 1 ? h / G : 0;
    const int32_t qh = h0 + (h - hm * G);
    const int32_t seq = u.b + hm;
    const int32_t slot = u.pack > 1 ? col_slot[h] : u.slot;
    const int32_t np = u.pack > 1 ? col_np[h] : u.nparts;
    if (np == 1) {
      store_f32((uint16_t*)a.out + ((int64_t)seq * a.hq + qh) * D + dd, o * inv);
    } else {
      __builtin_nontemporal_store(o * inv, a.plan.part_o + ((int64_t)slot * a.hq + qh) * D + dd);
      if (dd == 0) {
        float* ml = a.plan.part_ml + ((int64_t)slot * a.hq + qh) * 2;
        ml[0] = M * c;
        ml[1] = sum;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Vector-ALU partition kernel for small head groups (G <= 4: multi-head
// attention, or fp32 data), where the score and value products are too thin
// for matrix cores.  Same unit / workgroup / LDS-combine structure as the
// matrix-core kernel (W waves per (partition, KV head) unit).
//
// Scores: a key row of D elements is LPR = D / EPC lanes wide (EPC elements
// per 16-byte piece), so one load instruction covers TPI = 64 / LPR tokens;
// lane l holds piece l % LPR of token l / LPR.  Each lane forms partial dot
// products with its piece of every query head, and the LPR lanes of a row are
// summed with DPP row permutations (quad swaps, half-row and row mirrors).
// The chunk maximum crosses rows with two or three shuffles.  The row's first
// lane puts the probabilities in LDS; for the value product lane l owns head
// dims l, l + 64, ... and reads every probability of the chunk back from LDS,
// while its value loads are 16-byte runs of the token-minor value tile.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false);
  return v + __builtin_bit_cast(float, moved);
}

// sum over aligned groups of N lanes (N = 2, 4, 8, 16, 32), result in every lane
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if (N >= 2) v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  if (N >= 4) v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  if (N >= 8) v = dpp_add<0x141>(v);  // row_half_mirror: the other quad of the half-row
  if (N >= 16) v = dpp_add<0x140>(v); // row_mirror: the other half of the row
  if (N >= 32) v += __shfl_xor(v, 16, 64);
  return v;
}

template <typename T>
__device__ __forceinline__ void unpack16(const uint4& x, float* f);
template <>
__device__ __forceinline__ void unpack16<uint16_t>(const uint4& x, float* f) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void unpack16<float>(const uint4& x, float* f) {
  f[0] = __uint_as_float(x.x);
  f[1] = __uint_as_float(x.y);
  f[2] = __uint_as_float(x.z);
  f[3] = __uint_as_float(x.w);
}

template <typename T, int D, int GMAX>
__global__ __launch_bounds__(256) void decode_dpp_kernel(DecodeArgs a) {
  constexpr int W = 4;                       // waves per workgroup
  constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte piece
  constexpr int LPR = D / EPC;               // lanes per key row
  constexpr int TPI = 64 / LPR;              // tokens per load instruction
  constexpr int CH = sizeof(T) == 2 ? 32 : 16;  // tokens per chunk
  constexpr int KL = CH / TPI;               // key loads per lane per chunk
  constexpr int DPL = D / 64;                // head dims per lane in the value product
  constexpr int VP = CH / EPC;               // 16-byte value pieces per dim per chunk
  constexpr int DP = D + 4;
  static_assert(D % 64 == 0 && LPR >= 2 && LPR <= 32 && 64 % LPR == 0, "shape");
  __shared__ float red_o[W][GMAX][DP];
  __shared__ float red_m[W][GMAX], red_l[W][GMAX];
  __shared__ float p_lds[W][GMAX][CH];

  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int32_t unit = blockIdx.x / a.hkv;
  const int32_t g = blockIdx.x - unit * a.hkv;
  if (unit >= a.max_units) return;  // uniform over the workgroup
  const Unit u = decode_unit(a, unit);
  if (!u.valid) return;             // uniform over the workgroup
  const int32_t G = a.hq / a.hkv;
  const int32_t P = a.p;
  const int rr = lane / LPR, cc = lane % LPR;  // token within an instruction, piece within the row

  const T* kc = (const T*)a.kc;
  const T* vc = (const T*)a.vc;
  const int64_t blk_stride = (int64_t)a.hkv * P * D;
  const int64_t head_off = (int64_t)g * P * D;       // value tile of head g
  const int64_t khead_off = (int64_t)g * a.ks.head;  // first key row of head g
  const float c = a.scale_log2;

  float acc[GMAX][DPL];
  float m_run = -INFINITY;
  float l_run[GMAX];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    l_run[h] = 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[h][j] = 0.f;
  }
  float mh[GMAX];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) mh[h] = -INFINITY;

  const int32_t TW = a.part_tokens / W;  // a multiple of CH
  const int32_t s0 = u.t0 + w * TW;
  const int32_t s1 = min(u.t1, s0 + TW);
  if (s1 > s0) {
    // this lane's piece of every query head, as fp32
    float qf[GMAX][EPC];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      uint4 x = uint4{0, 0, 0, 0};
      if (h < G) x = *reinterpret_cast<const uint4*>((const T*)a.q + ((int64_t)u.b * a.hq + g * G + h) * D + cc * EPC);
      unpack16<T>(x, qf[h]);
    }
    const int32_t* trow = a.table + (int64_t)u.b * a.max_blocks;
    const int32_t last_blk = (s1 - 1) / P;
    int32_t wb = 0, tabv = 0, wlast = 0;
    auto load_window = [&](int32_t base) -> int32_t {
      int32_t e = 0;
      if (base + lane <= last_blk) {
        e = trow[base + lane];
        if ((uint32_t)e >= (uint32_t)a.num_blocks) {
          atomicOr(a.err, PKV_DEVERR_TABLE_ENTRY);
          e = 0;
        }
      }
      return e;
    };
    int32_t vlast = 0, klast = 0;
    struct Chunk {
      uint4 kx[KL], vx[DPL][VP];
    };
    // loads of one chunk: key pieces, then value pieces, addresses clamped to
    // the window (so the prefetch past its end stays in bounds)
    // The TPI rows of one key load and the EPC tokens of one value piece lie
    // in one block (TPI and EPC divide P), so each load's block id is
    // wave-uniform and comes from a lane read, not a cross-lane shuffle.
    auto issue = [&](Chunk& f, int32_t c0) {
#pragma unroll
      for (int i = 0; i < KL; ++i) {
        const int32_t tb = min(c0 + TPI * i, klast);  // uniform, first row of the load
        const int32_t pb = __builtin_amdgcn_readlane(tabv, tb / P - wb);
        f.kx[i] = load_stream16((const uint16_t*)(kc + (int64_t)pb * blk_stride + khead_off +
                                                  (int64_t)(tb % P + rr) * a.ks.tok + cc * EPC));
      }
#pragma unroll
      for (int k = 0; k < VP; ++k) {
        const int32_t t = min(c0 + EPC * k, vlast);   // uniform
        const int32_t pb = __builtin_amdgcn_readlane(tabv, t / P - wb);
        const T* vrow = vc + (int64_t)pb * blk_stride + head_off + (t % P);
#pragma unroll
        for (int j = 0; j < DPL; ++j)
          f.vx[j][k] = load_stream16((const uint16_t*)(vrow + (int64_t)(lane + 64 * j) * P));
      }
    };
    auto compute = [&](Chunk& f, int32_t c0) {
      // scores: partial dots, row sums
      float sc[GMAX][KL];
#pragma unroll
      for (int i = 0; i < KL; ++i) {
        float kf[EPC];
        unpack16<T>(f.kx[i], kf);
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
          float d0 = 0.f;
#pragma unroll
          for (int e = 0; e < EPC; ++e) d0 = fmaf(qf[h][e], kf[e], d0);
          sc[h][i] = group_sum<LPR>(d0);
        }
      }
      const bool ragged = c0 + CH > s1;  // uniform
#pragma unroll
      for (int i = 0; i < KL; ++i) {
        const bool ok = !ragged || c0 + TPI * i + rr < s1;
#pragma unroll
        for (int h = 0; h < GMAX; ++h) sc[h][i] = ok ? sc[h][i] : -INFINITY;
      }
      // chunk maximum per head: within the lane, then across the TPI rows
      float alpha[GMAX];
#pragma unroll
      for (int h = 0; h < GMAX; ++h) {
        float x = -INFINITY;
#pragma unroll
        for (int i = 0; i < KL; ++i) x = fmaxf(x, sc[h][i]);
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
        const float mn = fmaxf(mh[h], x);
        alpha[h] = fast_exp2((mh[h] - mn) * c);
        mh[h] = mn;
      }
      // probabilities -> LDS (first lane of each row), row partial sums
#pragma unroll
      for (int h = 0; h < GMAX; ++h) {
        const float mc = mh[h] * c;
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < KL; ++i) {
          const float pr = fast_exp2(fmaf(sc[h][i], c, -mc));
          ps += pr;
          if (cc == 0) p_lds[w][h][TPI * i + rr] = pr;
        }
        l_run[h] = fmaf(l_run[h], alpha[h], ps);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // value product: lane owns dims lane + 64 j
#pragma unroll
      for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[h][j] *= alpha[h];
#pragma unroll
      for (int k = 0; k < VP; ++k) {
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          float vf[EPC];
          unpack16<T>(f.vx[j][k], vf);
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            // masked tokens: probability 0 and value 0, so stale data cannot leak
            const float vv = (!ragged || c0 + EPC * k + e < s1) ? vf[e] : 0.f;
#pragma unroll
            for (int h = 0; h < GMAX; ++h) acc[h][j] = fmaf(p_lds[w][h][EPC * k + e], vv, acc[h][j]);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    // windows of 64 blocks; the next chunk's loads are in flight while the
    // current one is computed
    Chunk f0, f1;
    for (int32_t ws = s0; ws < s1;) {
      wb = uniform(ws / P);
      const int32_t we = min(s1, (wb + 64) * P);
      wlast = we - 1;
      // value pieces start at multiples of EPC inside a block; the window's
      // last piece starts here
      vlast = wlast - wlast % EPC;
      // last key load of the window starts here (its rows stay in wlast's block)
      klast = wlast - wlast % TPI;
      tabv = load_window(wb);
      int32_t c0 = ws;
      issue(f0, c0);
      while (true) {
        issue(f1, c0 + CH);
        compute(f0, c0);
        c0 += CH;
        if (c0 >= we) break;
        issue(f0, c0 + CH);
        compute(f1, c0);
        c0 += CH;
        if (c0 >= we) break;
      }
      ws = we;
    }
  }
  // this wave's state -> LDS; lanes of one row hold the same token sums
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    float lt = l_run[h];
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) lt += __shfl_xor(lt, o, 64);
    if (lane == 0) {
      red_m[w][h] = mh[h];
      red_l[w][h] = lt;
    }
#pragma unroll
    for (int j = 0; j < DPL; ++j) red_o[w][h][lane + 64 * j] = acc[h][j];
  }
  __syncthreads();
  for (int32_t e = threadIdx.x; e < G * D; e += 64 * W) {
    const int32_t h = e / D, dd = e - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < W; ++v)
      if (red_l[v][h] > 0.f) M = fmaxf(M, red_m[v][h]);
    float sum = 0.f, o = 0.f;
#pragma unroll
    for (int v = 0; v < W; ++v) {
      const float lv = red_l[v][h];
      if (lv > 0.f) {
        const float wt = fast_exp2((red_m[v][h] - M) * c);
        sum = fmaf(lv, wt, sum);
        o = fmaf(wt, red_o[v][h][dd], o);
      }
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    const int32_t qh = g * G + h;
    if (u.nparts == 1) {
      store_f32((T*)a.out + ((int64_t)u.b * a.hq + qh) * D + dd, o * inv);
    } else {
      __builtin_nontemporal_store(o * inv, a.plan.part_o + ((int64_t)u.slot * a.hq + qh) * D + dd);
      if (dd == 0) {
        float* ml = a.plan.part_ml + ((int64_t)u.slot * a.hq + qh) * 2;
        ml[0] = M * c;
        ml[1] = sum;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// VALU partition kernel: one wave per unit, any block size, head_dim <= 256.
// ---------------------------------------------------------------------------
template <typename T, int GMAX, int DK>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodeArgs a) {
  __shared__ float qs[GMAX][DK * 64];
  __shared__ float ps[GMAX][64];
  const int lane = threadIdx.x;
  const int32_t unit = blockIdx.x / a.hkv;
  const int32_t g = blockIdx.x - unit * a.hkv;
  if (unit >= a.max_units) return;
  const Unit u = decode_unit(a, unit);
  if (!u.valid) return;
  const int32_t G = a.hq / a.hkv, D = a.d, P = a.p;
  const T* q = (const T*)a.q;
  const T* kc = (const T*)a.kc;
  const T* vc = (const T*)a.vc;
  const int32_t* trow = a.table + (int64_t)u.b * a.max_blocks;

  for (int32_t i = lane; i < G * D; i += 64)
    qs[i / D][i % D] = load_f32(q + ((int64_t)u.b * a.hq + (int64_t)g * G) * D + i);
  __syncthreads();

  float m[GMAX], l[GMAX], acc[GMAX][DK];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int k = 0; k < DK; ++k) acc[h][k] = 0.f;
  }
  const float c = a.scale_log2;
  auto phys_of = [&](int32_t t) -> int64_t {
    int32_t e = trow[t / P];
    if ((uint32_t)e >= (uint32_t)a.num_blocks) {
      atomicOr(a.err, PKV_DEVERR_TABLE_ENTRY);
      e = 0;
    }
    return e;
  };

  for (int32_t c0 = u.t0; c0 < u.t1; c0 += 64) {
    const int32_t t = c0 + lane;
    const bool valid = t < u.t1;
    float s[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) s[h] = 0.f;
    if (valid) {
      const T* kr = kc + phys_of(t) * a.hkv * P * D + (int64_t)g * a.ks.head + (int64_t)(t % P) * a.ks.tok;
      for (int32_t dd = 0; dd < D; ++dd) {
        const float kv = load_f32(kr + dd);
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
          if (h < G) s[h] = fmaf(qs[h][dd], kv, s[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h >= G) continue;
      const float sh = valid ? s[h] * c : -INFINITY;
      const float mn = fmaxf(m[h], wave_max(sh));
      const float al = fast_exp2(m[h] - mn);
      const float pv = fast_exp2(sh - mn);
      l[h] = fmaf(l[h], al, wave_sum(pv));
      ps[h][lane] = pv;
#pragma unroll
      for (int k = 0; k < DK; ++k) acc[h][k] *= al;
      m[h] = mn;
    }
    __syncthreads();
    const int32_t nt = min(64, u.t1 - c0);
    for (int32_t i = 0; i < nt; ++i) {
      const int32_t tt = c0 + i;
      const T* vcol = vc + (phys_of(tt) * a.hkv + g) * D * P + tt % P;
#pragma unroll
      for (int k = 0; k < DK; ++k) {
        const int32_t dd = lane + 64 * k;
        if (dd < D) {
          const float vv = load_f32(vcol + (int64_t)dd * P);
#pragma unroll
          for (int h = 0; h < GMAX; ++h)
            if (h < G) acc[h][k] = fmaf(ps[h][i], vv, acc[h][k]);
        }
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h >= G) continue;
    const int32_t head = g * G + h;
    const float inv = l[h] > 0.f ? 1.f / l[h] : 0.f;
    if (u.nparts == 1) {
      T* orow = (T*)a.out + ((int64_t)u.b * a.hq + head) * D;
#pragma unroll
      for (int k = 0; k < DK; ++k) {
        const int32_t dd = lane + 64 * k;
        if (dd < D) store_f32(orow + dd, acc[h][k] * inv);
      }
    } else {
      float* prow = a.plan.part_o + ((int64_t)u.slot * a.hq + head) * D;
#pragma unroll
      for (int k = 0; k < DK; ++k) {
        const int32_t dd = lane + 64 * k;
        if (dd < D) prow[dd] = acc[h][k] * inv;
      }
      if (lane == 0) {
        float* ml = a.plan.part_ml + ((int64_t)u.slot * a.hq + head) * 2;
        ml[0] = m[h];
        ml[1] = l[h];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Merge.  For query head h of a sequence with n > 1 partial results in slots
// f0 .. f0 + n - 1 (partition order), over the slots with l_i > 0:
//   M = max_i m_i,  w_i = l_i 2^(m_i - M),  out = sum_i w_i o_i / sum_i w_i.
// One workgroup per (sequence, KV head, column set) takes the query heads of
// that set (G of them; G / gparts with more than 16), EPT output elements per
// thread (G D / EPT threads, rounded up to whole waves), so the grid is
// n_seqs * Hkv * gparts workgroups; those
// of a sequence with one partition return at once (it wrote its output
// directly).  Wave w finds M, the weights (to LDS, the first kMergeSlots
// slots) and their total for heads w, w + W, ...; before any of that waits,
// every thread has issued the loads of its elements' first kMergePre partial
// outputs and of the first 64 slots' (m, l) of its wave's first kMergeHeads
// heads, so a merge of up to kMergePre partitions costs one round trip to
// memory (later slots: one more per kMergePre).  Each output element sums its
// slots in order, so the result does not depend on the launch.
// ---------------------------------------------------------------------------
constexpr int kMergeSlots = 128;  // weights kept in LDS per head; later ones are recomputed
constexpr int kMergePre = 4;      // partial outputs loaded before the weights are known
constexpr int kMergeElems = 4;    // most output elements per thread (G D up to 4096)
constexpr int kMergeHeads = 4;    // heads per wave whose first slots' (m, l) are loaded up front

// threads of a merge workgroup for `ept` elements per thread (per = G * D <= 4096)
inline int merge_threads(int32_t per, int ept) {
  const int32_t t = (per + ept - 1) / ept;
  return std::min(1024, std::max(64, (t + 63) / 64 * 64));
}

template <typename T, int EPT>
__global__ __launch_bounds__(1024) void merge_kernel(DecodeArgs a) {
  __shared__ float wts[16][kMergeSlots];
  __shared__ float m_head[16], tot_head[16];
  // workgroup: (sequence b, KV head g, column set `part` of g's query heads)
  const int32_t hkv_v = a.hkv * a.gparts;
  const int32_t b = blockIdx.x / hkv_v;
  const int32_t gv = blockIdx.x - b * hkv_v;
  const int32_t g = a.gparts == 1 ? gv : gv / a.gparts, part = gv - g * a.gparts;
  const int4 si = a.plan.seq_info[b];
  const int32_t f0 = si.x, n = si.y;
  if (!plan_matches(a)) return;       // another call's plan (flagged by the partition kernel)
  if (n <= 1) return;                 // uniform
  if (a.plan.counts[0] == 0) return;  // plan overflowed
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  // this workgroup's G query heads, from head h0 (at most 16)
  const int32_t GA = a.hq / a.hkv;
  const int32_t G = a.gparts > 1 ? min(a.gcols, GA - part * a.gcols) : GA;
  const int32_t h0 = g * GA + part * a.gcols;
  const int32_t D = a.d, GD = G * D;
  const int64_t slot_stride = (int64_t)a.hq;  // (slot, head) rows per slot
  const int64_t row0 = (int64_t)f0 * slot_stride + h0;  // (slot f0, head h0)

  // this thread's output elements: head hk[k], element dk[k] (ok[k]: in range)
  int32_t hk[EPT], dk[EPT];
  bool ok[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int32_t e = threadIdx.x + k * blockDim.x;
    ok[k] = e < GD;
    hk[k] = ok[k] ? e / D : 0;
    dk[k] = ok[k] ? e - hk[k] * D : 0;
  }
  auto o_ptr = [&](int32_t j, int k) -> const float* {
    return a.plan.part_o + (row0 + j * slot_stride + hk[k]) * D + dk[k];
  };
  auto ml_ptr = [&](int32_t i, int32_t hh) -> const float* {
    return a.plan.part_ml + (row0 + i * slot_stride + hh) * 2;
  };

  // Loads issued before anything waits: the first kMergePre partial outputs
  // of this thread's elements, and (m, l) of slot `lane` for the wave's first
  // kMergeHeads heads.
  float pre[EPT][kMergePre];
#pragma unroll
  for (int k = 0; k < EPT; ++k)
#pragma unroll
    for (int j = 0; j < kMergePre; ++j) pre[k][j] = (ok[k] && j < n) ? *o_ptr(j, k) : 0.f;
  float m0[kMergeHeads], l0[kMergeHeads];
#pragma unroll
  for (int r = 0; r < kMergeHeads; ++r) {
    const int32_t hh = w + r * W;
    m0[r] = 0.f;
    l0[r] = 0.f;
    if (hh < G && lane < n) {
      m0[r] = ml_ptr(lane, hh)[0];
      l0[r] = ml_ptr(lane, hh)[1];
    }
  }

  // maximum, weights and total of head hh (uniform per wave); mf, lf: slot `lane`
  auto head_stats = [&](int32_t hh, float mf, float lf) {
    float mx = lf > 0.f ? mf : -INFINITY;
    for (int32_t i = lane + 64; i < n; i += 64) {
      const float mi = ml_ptr(i, hh)[0], li = ml_ptr(i, hh)[1];
      if (li > 0.f) mx = fmaxf(mx, mi);
    }
    mx = wave_max(mx);
    float tot = 0.f;
    for (int32_t i = lane; i < n; i += 64) {
      float mi = mf, li = lf;
      if (i >= 64) {
        mi = ml_ptr(i, hh)[0];
        li = ml_ptr(i, hh)[1];
      }
      const float wi = li > 0.f ? li * fast_exp2(mi - mx) : 0.f;
      if (i < kMergeSlots) wts[hh][i] = wi;
      tot += wi;
    }
    tot = wave_sum(tot);
    if (lane == 0) {
      m_head[hh] = mx;
      tot_head[hh] = tot;
    }
  };
#pragma unroll
  for (int r = 0; r < kMergeHeads; ++r)
    if (w + r * W < G) head_stats(w + r * W, m0[r], l0[r]);
  for (int32_t hh = w + kMergeHeads * W; hh < G; hh += W) {
    float mf = 0.f, lf = 0.f;
    if (lane < n) {
      mf = ml_ptr(lane, hh)[0];
      lf = ml_ptr(lane, hh)[1];
    }
    head_stats(hh, mf, lf);
  }
  __syncthreads();

  float acc[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    acc[k] = 0.f;
#pragma unroll
    for (int j = 0; j < kMergePre; ++j)
      if (ok[k] && j < n) acc[k] = fmaf(wts[hk[k]][j], pre[k][j], acc[k]);
  }
  // later slots, kMergePre at a time with all their loads issued together
  for (int32_t j0 = kMergePre; j0 < n; j0 += kMergePre) {
    float ov[EPT][kMergePre];
#pragma unroll
    for (int k = 0; k < EPT; ++k)
#pragma unroll
      for (int u = 0; u < kMergePre; ++u) ov[k][u] = (ok[k] && j0 + u < n) ? *o_ptr(j0 + u, k) : 0.f;
#pragma unroll
    for (int k = 0; k < EPT; ++k)
#pragma unroll
      for (int u = 0; u < kMergePre; ++u) {
        const int32_t j = j0 + u;
        if (!ok[k] || j >= n) continue;
        float wj;
        if (j < kMergeSlots) {
          wj = wts[hk[k]][j];
        } else {
          const float* ml = ml_ptr(j, hk[k]);
          wj = ml[1] > 0.f ? ml[1] * fast_exp2(ml[0] - m_head[hk[k]]) : 0.f;
        }
        acc[k] = fmaf(wj, ov[k][u], acc[k]);
      }
  }
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    if (!ok[k]) continue;
    const float tot = tot_head[hk[k]];
    store_f32((T*)a.out + ((int64_t)b * a.hq + h0 + hk[k]) * D + dk[k], tot > 0.f ? acc[k] / tot : 0.f);
  }
}

// ---------------------------------------------------------------------------
// Host side: partition size, workspace layout, dispatch.
// ---------------------------------------------------------------------------
int device_cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

constexpr int32_t kWholeLen = 1024;  // contexts this short are not split

int32_t env_int(const char* name, int32_t dflt) {
  const char* s = std::getenv(name);
  if (!s || !*s) return dflt;
  return (int32_t)std::strtol(s, nullptr, 10);
}

bool env_is(const char* name, const char* val) {
  const char* s = std::getenv(name);
  return s && std::strcmp(s, val) == 0;
}

int32_t pow2_floor(int64_t x) {
  int32_t p = 1;
  while ((int64_t)p * 2 <= x && p < (1 << 30)) p *= 2;
  return p;
}

enum Kind { kKindMfma, kKindDpp, kKindGeneric };

struct Choice {
  int kind;
  int32_t waves_per_group;  // waves sharing one unit (matrix-core and DPP kernels)
  int32_t part_tokens;
  int64_t max_units;
  bool need_partials;
  bool may_pack;  // sized for packs of sharing sequences (one extra slot per sequence)
  bool wide;          // packs may be wide (dense product over up to kWideRows query rows)
  int32_t wide_split; // pieces per whole shared partition of a wide pack
  int32_t gparts, gcols;  // column sets of a KV head's query heads, heads per set
};

enum { kMathAuto, kMathValu, kMathMfma, kMathDpp, kMathGeneric };

int math_mode() {
  if (env_is("PKV_DECODE_MATH", "valu")) return kMathValu;      // any vector-ALU kernel
  if (env_is("PKV_DECODE_MATH", "mfma")) return kMathMfma;
  if (env_is("PKV_DECODE_MATH", "dpp")) return kMathDpp;
  if (env_is("PKV_DECODE_MATH", "generic")) return kMathGeneric;
  return kMathAuto;
}

bool mfma_shape_ok(int32_t hq, int32_t hkv, int32_t d, int32_t p, pkv_dtype dt) {
  const int32_t G = hq / hkv;
  // (any G: beyond 16 the query heads run in several column sets)
  return dt == PKV_BF16 && (d == 64 || d == 128) && (p == 1 || p == 2 || p == 4 || p == 8 || p == 16 || p == 32 || p == 64) &&
         G >= 1;
}

// DPP kernel: head_dim 64 / 128, head groups up to 4, block rows of whole
// 16-byte pieces (block_size a multiple of 8 for bf16, of 4 for fp32)
bool dpp_shape_ok(int32_t hq, int32_t hkv, int32_t d, int32_t p, pkv_dtype dt) {
  const int32_t G = hq / hkv;
  const int32_t epc = dt == PKV_BF16 ? 8 : 4;
  return (d == 64 || d == 128) && G >= 1 && G <= 4 && p % epc == 0;
}

bool generic_shape_ok(int32_t hq, int32_t hkv, int32_t d) { return d <= 256 && hq / hkv <= 16; }

int choose(int32_t n_seqs, int32_t hq, int32_t hkv, int32_t d, int32_t p, int32_t max_len,
           int64_t total, int64_t unshared, pkv_dtype dt, Choice* out) {
  const int mode = math_mode();
  const bool mshape = mfma_shape_ok(hq, hkv, d, p, dt);
  const bool dshape = dpp_shape_ok(hq, hkv, d, p, dt);
  int kind;
  if (mode == kMathMfma) {
    if (!mshape) return fail(PKV_ERR_UNSUPPORTED, "matrix-core decode needs bf16, head_dim 64/128, block size a power of two up to 64");
    kind = kKindMfma;
  } else if (mode == kMathDpp) {
    if (!dshape) return fail(PKV_ERR_UNSUPPORTED, "DPP decode needs head_dim 64/128, G <= 4, 16-byte block rows");
    kind = kKindDpp;
  } else if (mode == kMathGeneric) {
    kind = kKindGeneric;
  } else if (mode == kMathValu) {
    kind = dshape ? kKindDpp : kKindGeneric;
  } else if (mshape) {
    // matrix cores for every bf16 head group, multi-head (G = 1) included:
    // with 15 of 16 columns padding the products cost nothing next to the
    // loads, and its 16-byte fragment loads stream faster than the DPP
    // kernel's (32 x 32/32 heads, D = 128, L in [1024, 4096]: 6.27 TB/s
    // against 5.53; 64 x 32/32, L in [128, 4096]: 6.34 against 4.28)
    kind = kKindMfma;
  } else {
    kind = dshape ? kKindDpp : kKindGeneric;
  }
  if (kind == kKindGeneric && !generic_shape_ok(hq, hkv, d))
    return fail(PKV_ERR_UNSUPPORTED, "decode supports head_dim <= 256 and Hq/Hkv <= 16");
  const int64_t L = std::max<int32_t>(max_len, 1);
  // more than 16 query heads per KV head (matrix-core kernel only): column
  // sets of at most 16, each reading the KV head's keys and values
  const int32_t G = hq / hkv;
  out->gparts = kind == kKindMfma && G > 16 ? (G + 15) / 16 : 1;
  out->gcols = (G + out->gparts - 1) / out->gparts;
  // packs need the matrix-core kernel, one column set and a batch not known
  // to share nothing
  const bool may_pack = kind == kKindMfma && out->gparts == 1 &&
                        !(unshared >= 0 && total >= 0 && unshared >= total);
  if (total < 0) total = (int64_t)n_seqs * L;
  // W waves share a partition of T tokens; each wave's share is whole chunks
  int32_t W = 1, tmin = 64, tmax = 512;
  if (kind == kKindMfma) {
    W = env_int("PKV_DECODE_WAVES", 4) == 8 ? 8 : 4;
    tmin = 32 * W;
    tmax = 16384;
  } else if (kind == kKindDpp) {
    W = 4;
    tmin = W * (dt == PKV_BF16 ? 32 : 16);
    tmax = 16384;
  }
  int32_t T;
  const int32_t forced = env_int("PKV_PARTITION_TOKENS", 0);
  if (env_is("PKV_DECODE_SPLIT", "off")) {
    T = tmin;
    while (T < L) T *= 2;
  } else if (forced > 0) {
    T = std::max(tmin, pow2_floor(forced));
  } else {
    // The largest partition whose single unit still takes a small share of
    // the whole launch (about half of it with two resident workgroups per
    // compute unit): longer partitions mean fewer partial results written to
    // HBM, shorter ones a shorter tail.  A batch with at least eight
    // (sequence, KV head) pairs per compute unit balances with half as many
    // splits (measured: fan-out -2.7%, long and shared prefix unchanged; a
    // batch of 64 sequences with 8 KV heads is 1.4% slower that way).
    const int cus = device_cu_count();
    const int32_t div_default = (int64_t)n_seqs * hkv >= 8LL * cus ? 2 : 4;
    const int64_t div = std::max(1, env_int("PKV_SPLIT_DIV", div_default));
    // (units are partitions x KV heads x column sets.)  Matrix-core units
    // shorter than 256 tokens cost more in per-unit overhead than they gain in
    // spread.  Measured (planned decode, head_dim 128, lengths up to 4096):
    // 64 sequences on one KV head 48.4 us at 128 against 36.1 at 256; 16 on
    // one 27.1 against 23.0; 4 on eight 20.1 against 17.6; 8 on two 17.2
    // against 16.8; with 64 query heads on one KV head, counting the four
    // column sets, 124.5 against 72.2.
    const int64_t want = total * hkv * out->gparts / ((int64_t)cus * div);
    const int32_t tfloor = kind == kKindMfma ? 256 : tmin;
    T = (int32_t)std::min<int64_t>(tmax, std::max<int64_t>(tfloor, pow2_floor(std::max<int64_t>(want, 1))));
    // Contexts of at most kWholeLen tokens: one partition per sequence and
    // no merge launch.  Measured (plan + partition + merge, 16-token blocks):
    // longest context 512, batches of 8 and 64: 16.4-16.9 us against
    // 19.4-21.2 split; longest 1024: batch 16 22.9 against 22.4, batch 32
    // 24.5 against 31.0; longest 2048 and 4096 split far better (19.8
    // against 29.3, 26.2 against 51.7).
    if (L <= kWholeLen) {
      int32_t t = tmin;
      while (t < L) t *= 2;
      T = std::min(tmax, std::max(T, t));
    }
  }
  const int64_t by_len = (int64_t)n_seqs * ((L + T - 1) / T);
  const int64_t by_total = total / T + n_seqs;
  out->kind = kind;
  out->waves_per_group = W;
  out->part_tokens = T;
  // wide packs: four waves, blocks of 8 to 64 tokens (a 16-key group in one
  // block, or two of 8), units of at most kWideTab blocks
  out->wide = may_pack && W == 4 && p % 8 == 0 && T / p <= kWideTab && !env_is("PKV_DECODE_WIDE", "off");
  out->wide_split = 1;
  if (out->wide) {
    // pieces of at least one 64-key chunk.  Measured on 128 sequences sharing
    // a 2048-token prefix (T = 2048, packs of 32): whole partitions 0.0756 ms,
    // halves 0.0693, quarters 0.0729, eighths 0.0791 (more pieces, more
    // partials to write and merge)
    const int32_t want_split = std::max(1, env_int("PKV_WIDE_SPLIT", 2));
    while (out->wide_split * 2 <= want_split && T / (out->wide_split * 2) >= 64) out->wide_split *= 2;
  }
  // a split shared partition adds one slot (and one unit) per sequence; the
  // pieces of wide packs add wide_split - 1 per whole shared partition
  const int64_t whole = std::min<int64_t>((int64_t)n_seqs * (L / T), total / T);
  out->max_units = std::max<int64_t>(1, std::min(by_len, by_total)) + (may_pack ? n_seqs : 0) +
                   (int64_t)(out->wide_split - 1) * whole;
  out->need_partials = T < L || may_pack;
  out->may_pack = may_pack;
  return PKV_OK;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  size_t counts, seq_info, seq_pack, work, work_out, part_ml, part_o, total;
};

Layout layout_of(int32_t n_seqs, int32_t hq, int32_t d, const Choice& c) {
  Layout l;
  size_t off = 0;
  l.counts = off;
  off = align256(off + 4 * sizeof(int32_t));
  l.seq_info = off;
  off = align256(off + (size_t)n_seqs * sizeof(int4));
  l.seq_pack = off;
  off = align256(off + (size_t)n_seqs * sizeof(int2));
  l.work = off;
  off = align256(off + (size_t)c.max_units * sizeof(int4));
  l.work_out = off;
  off = align256(off + (size_t)c.max_units * sizeof(int2));
  l.part_ml = off;
  if (c.need_partials) off = align256(off + (size_t)c.max_units * hq * 2 * sizeof(float));
  l.part_o = off;
  if (c.need_partials) off = align256(off + (size_t)c.max_units * hq * d * sizeof(float));
  l.total = off;
  return l;
}

template <int D, int P>
void launch_mfma(const DecodeArgs& a, int32_t waves_per_group, int64_t groups, hipStream_t st) {
  // a batch that packs sequences sharing blocks reads the packs' tokens with
  // cached loads, and so do the column sets of one KV head (adjacent
  // workgroups over the same keys and values)
  const bool keep = a.pack_max > 1 || a.gparts > 1;
  if (waves_per_group == 8) {
    if (keep) hipLaunchKernelGGL((decode_mfma_kernel<D, P, 8, true>), dim3((unsigned)groups), dim3(512), 0, st, a);
    else hipLaunchKernelGGL((decode_mfma_kernel<D, P, 8, false>), dim3((unsigned)groups), dim3(512), 0, st, a);
  } else {
    if (keep) hipLaunchKernelGGL((decode_mfma_kernel<D, P, 4, true>), dim3((unsigned)groups), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((decode_mfma_kernel<D, P, 4, false>), dim3((unsigned)groups), dim3(256), 0, st, a);
  }
}

template <int D>
void launch_mfma_p(const DecodeArgs& a, int32_t p, int32_t waves_per_group, int64_t groups, hipStream_t st) {
  switch (p) {
    case 1: launch_mfma<D, 1>(a, waves_per_group, groups, st); break;
    case 2: launch_mfma<D, 2>(a, waves_per_group, groups, st); break;
    case 4: launch_mfma<D, 4>(a, waves_per_group, groups, st); break;
    case 8: launch_mfma<D, 8>(a, waves_per_group, groups, st); break;
    case 16: launch_mfma<D, 16>(a, waves_per_group, groups, st); break;
    case 32: launch_mfma<D, 32>(a, waves_per_group, groups, st); break;
    default: launch_mfma<D, 64>(a, waves_per_group, groups, st); break;
  }
}

template <typename T, int D>
void launch_dpp_d(const DecodeArgs& a, int64_t groups, hipStream_t st) {
  const int32_t G = a.hq / a.hkv;
  if (G <= 1) hipLaunchKernelGGL((decode_dpp_kernel<T, D, 1>), dim3((unsigned)groups), dim3(256), 0, st, a);
  else if (G <= 2) hipLaunchKernelGGL((decode_dpp_kernel<T, D, 2>), dim3((unsigned)groups), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((decode_dpp_kernel<T, D, 4>), dim3((unsigned)groups), dim3(256), 0, st, a);
}

template <typename T>
void launch_dpp(const DecodeArgs& a, int64_t groups, hipStream_t st) {
  if (a.d == 128) launch_dpp_d<T, 128>(a, groups, st);
  else launch_dpp_d<T, 64>(a, groups, st);
}

template <typename T, int GMAX>
void launch_valu_g(const DecodeArgs& a, int64_t waves, hipStream_t st) {
  const int dk = (a.d + 63) / 64;
  switch (dk) {
    case 1: hipLaunchKernelGGL((decode_valu_kernel<T, GMAX, 1>), dim3((unsigned)waves), dim3(64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((decode_valu_kernel<T, GMAX, 2>), dim3((unsigned)waves), dim3(64), 0, st, a); break;
    case 3: hipLaunchKernelGGL((decode_valu_kernel<T, GMAX, 3>), dim3((unsigned)waves), dim3(64), 0, st, a); break;
    default: hipLaunchKernelGGL((decode_valu_kernel<T, GMAX, 4>), dim3((unsigned)waves), dim3(64), 0, st, a); break;
  }
}

template <typename T>
void launch_valu(const DecodeArgs& a, int64_t waves, hipStream_t st) {
  const int32_t G = a.hq / a.hkv;
  if (G <= 1) launch_valu_g<T, 1>(a, waves, st);
  else if (G <= 2) launch_valu_g<T, 2>(a, waves, st);
  else if (G <= 4) launch_valu_g<T, 4>(a, waves, st);
  else if (G <= 8) launch_valu_g<T, 8>(a, waves, st);
  else launch_valu_g<T, 16>(a, waves, st);
}

template <typename T>
void launch_merge(const DecodeArgs& a, unsigned grid, hipStream_t st) {
  // Elements per thread: measured best is one for small batches (more waves
  // hide the latency of a short launch) and two for large ones (fewer waves
  // to dispatch); raised until G * D fits 1024 threads.
  const int32_t gd = a.gcols * a.d;  // a column set's output elements
  const int64_t elems = (int64_t)a.n_seqs * a.hkv * a.gparts * gd;
  const int dflt = elems <= (int64_t)1 << 19 ? 1 : 2;
  const int want = env_int("PKV_MERGE_ELEMS", dflt);
  int ept = want >= 4 ? 4 : (want >= 2 ? 2 : 1);  // an instantiated width
  while (ept < kMergeElems && gd > 1024 * ept) ept *= 2;  // G D <= 4096 = 1024 * kMergeElems
  const dim3 block(merge_threads(gd, ept));
  if (ept == 1) hipLaunchKernelGGL((merge_kernel<T, 1>), grid, block, 0, st, a);
  else if (ept == 2) hipLaunchKernelGGL((merge_kernel<T, 2>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((merge_kernel<T, 4>), grid, block, 0, st, a);
}

}  // namespace
}  // namespace pkv

using pkv::fail;

extern "C" int pkv_decode_workspace_bytes(int32_t n_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size,
                                          int32_t max_context_len, int64_t total_context_tokens,
                                          int64_t unshared_context_tokens, pkv_dtype dtype,
                                          size_t* bytes_out) {
  PKV_TRY_BEGIN
  if (!bytes_out) return fail(PKV_ERR_INVALID_ARG, "bytes_out is NULL");
  if (n_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_context_len < 0 || num_q_heads % num_kv_heads)
    return fail(PKV_ERR_INVALID_ARG, "bad sizes");
  if (!pkv::dtype_valid(dtype)) return fail(PKV_ERR_INVALID_ARG, "bad dtype");
  pkv::Choice c;
  int rc = pkv::choose(n_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
                       total_context_tokens, unshared_context_tokens, dtype, &c);
  if (rc) return rc;
  *bytes_out = pkv::layout_of(n_seqs, num_q_heads, head_dim, c).total;
  return PKV_OK;
  PKV_TRY_END
}

// ---------------------------------------------------------------------------
// Library-owned scratch for pkv_paged_attention_decode_noalloc, for callers
// that cannot allocate device memory.  One copy per device (each device's
// code object holds its own), held until the process ends.  Host code never
// uses the array's name as an address: the device address is looked up once
// per device with hipGetSymbolAddress and kept in scratch_ptr.
// ---------------------------------------------------------------------------
namespace pkv {
namespace {
constexpr size_t kScratchBytes = PKV_DECODE_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
void* scratch_ptr[kMaxScratchDevices] = {};
std::mutex scratch_mu;

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices) return fail(PKV_ERR_UNSUPPORTED, "device id %d", dev);
  std::lock_guard<std::mutex> lk(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(PKV_ERR_HIP, "hipGetSymbolAddress(decode scratch): %s", hipGetErrorString(e));
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return PKV_OK;
}

// The plan's sizing stamp: every input of the plan kernel except the device
// lengths and shared counts (FNV-1a over them; never zero in both words).
int2 plan_stamp(const Choice& c, const DecodeArgs& a) {
  const int64_t v[] = {a.n_seqs, a.hq, a.hkv, a.part_tokens, a.max_units, a.pack_max,
                       a.wide_split, c.kind, a.len_cap, a.shared ? 1 : 0};
  uint64_t h = 1469598103934665603ull;
  for (int64_t x : v)
    for (int i = 0; i < 8; ++i) {
      h ^= (uint64_t)(x >> (8 * i)) & 0xff;
      h *= 1099511628211ull;
    }
  return make_int2((int32_t)(uint32_t)(h >> 32), (int32_t)((uint32_t)h | 1u));
}

enum DecodeMode {
  kPlanAndRun,  // plan, partition, merge (pkv_paged_attention_decode)
  kPlanOnly,    // plan into the workspace (pkv_decode_plan)
  kRunPlanned,  // partition and merge on the workspace's plan (pkv_paged_attention_decode_planned)
};

// The decode call proper.  With use_scratch the workspace arguments are
// ignored and the current device's library scratch is used instead.
int decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* d_block_table, const int32_t* d_context_lens,
                const int32_t* d_shared_prev, int32_t n_seqs, int32_t num_q_heads,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                int32_t max_blocks_per_seq, int32_t max_context_len, int64_t total_context_tokens,
                int64_t unshared_context_tokens, float scale, pkv_dtype dtype, pkv_layout k_layout,
                void* workspace, size_t workspace_bytes, bool use_scratch, DecodeMode mode,
                void* stream) {
  const bool plan_only = mode == kPlanOnly;
  if (n_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      (!plan_only && num_blocks <= 0) || max_blocks_per_seq < 0 || max_context_len < 0)
    return fail(PKV_ERR_INVALID_ARG, "bad sizes");
  if (num_q_heads % num_kv_heads) return fail(PKV_ERR_INVALID_ARG, "num_q_heads is not a multiple of num_kv_heads");
  if (num_q_heads > 65535) return fail(PKV_ERR_UNSUPPORTED, "more than 65535 query heads");
  if (!pkv::dtype_valid(dtype)) return fail(PKV_ERR_INVALID_ARG, "bad dtype");
  if (!pkv::layout_valid(k_layout)) return fail(PKV_ERR_INVALID_ARG, "bad key layout");
  if (!pkv::resolve_scale(&scale, head_dim))
    return fail(PKV_ERR_INVALID_ARG, "scale must be 0 (1/sqrt(head_dim)) or finite and positive");
  if (n_seqs == 0) return PKV_OK;
  if (!d_context_lens ||
      (!plan_only && (!out || !q || !k_cache || !v_cache || (max_blocks_per_seq > 0 && !d_block_table))))
    return fail(PKV_ERR_INVALID_ARG, "NULL pointer");
  if ((int64_t)max_blocks_per_seq * block_size < max_context_len)
    return fail(PKV_ERR_INVALID_ARG, "max_context_len exceeds the block-table capacity");
  pkv::Choice c;
  int rc = pkv::choose(n_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
                       total_context_tokens, unshared_context_tokens, dtype, &c);
  if (rc) return rc;
  if (c.kind != pkv::kKindGeneric && !plan_only) {
    const uintptr_t mis = (uintptr_t)out | (uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache;
    if (mis % 16) {
      const int math = pkv::math_mode();
      // (the generic kernel takes at most 16 query heads per KV head)
      if (math == pkv::kMathMfma || math == pkv::kMathDpp || mode == kRunPlanned || c.gparts > 1)
        return fail(PKV_ERR_UNSUPPORTED, "this decode kernel needs 16-byte aligned buffers");
      // same partition length and workspace; the generic kernel takes any
      c.kind = pkv::kKindGeneric;
    }
  }
  // one-dimensional grid: workgroups (units x KV heads x column sets) of up
  // to 512 threads must stay below 2^32 threads
  if ((int64_t)c.max_units * num_kv_heads * c.gparts * 512 >= (int64_t)1 << 32)
    return fail(PKV_ERR_UNSUPPORTED, "too many partitions");
  const pkv::Layout lay = pkv::layout_of(n_seqs, num_q_heads, head_dim, c);
  if (use_scratch) {
    if (lay.total > kScratchBytes)
      return fail(PKV_ERR_WORKSPACE,
                  "this batch needs %zu bytes of decode workspace; the library scratch holds %zu "
                  "(pass a workspace to pkv_paged_attention_decode instead)", lay.total, kScratchBytes);
    int src = scratch_address(&workspace);
    if (src) return src;
    workspace_bytes = kScratchBytes;
  } else if (!workspace || workspace_bytes < lay.total) {
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, lay.total);
  }
  int32_t* err = nullptr;
  rc = pkv::device_error_word(&err);
  if (rc) return rc;

  char* ws = (char*)workspace;
  pkv::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.table = d_block_table;
  a.ctx = d_context_lens;
  a.shared = d_shared_prev;
  a.n_seqs = n_seqs;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.d = head_dim;
  a.p = block_size;
  a.ks = pkv::k_strides(k_layout, num_kv_heads, block_size, head_dim);
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.part_tokens = c.part_tokens;
  a.max_units = (int32_t)c.max_units;
  // packs of sequences that share blocks: matrix-core kernel only (its 16
  // columns take 16 / G sequences' head groups).  A hint that nothing is
  // shared (unshared == total) skips the array and the plan's pack pass.
  a.pack_max = 1;
  if (d_shared_prev && c.may_pack && c.kind == pkv::kKindMfma && !pkv::env_is("PKV_DECODE_SHARE", "off")) {
    // narrow packs fill the 16 MFMA columns (16 / G sequences); wide packs
    // (four waves, blocks of 8 to 64 tokens, units of at most
    // kWideTab blocks) take up to 128 / G sequences, read with a dense product
    const int32_t G = num_q_heads / num_kv_heads;
    a.pack_max = c.wide ? std::min(pkv::kWideMaxPack, pkv::kWideRows / G) : std::max(1, 16 / G);
  }
  a.wide_split = a.pack_max > 1 && c.wide ? c.wide_split : 1;
  a.gparts = c.gparts;
  a.gcols = c.gcols;
  a.len_cap = std::min<int64_t>((int64_t)max_blocks_per_seq * block_size, max_context_len);
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.plan.counts = (int32_t*)(ws + lay.counts);
  a.plan.seq_info = (int4*)(ws + lay.seq_info);
  a.plan.seq_pack = (int2*)(ws + lay.seq_pack);
  a.plan.work = (int4*)(ws + lay.work);
  a.plan.work_out = (int2*)(ws + lay.work_out);
  a.plan.part_ml = c.need_partials ? (float*)(ws + lay.part_ml) : nullptr;
  a.plan.part_o = c.need_partials ? (float*)(ws + lay.part_o) : nullptr;
  a.err = err;
  a.stamp = plan_stamp(c, a);

  hipStream_t st = (hipStream_t)stream;
  if (mode != kRunPlanned) {
    // fewer plan threads finish sooner (fewer waves per SIMD on one compute unit)
    if (n_seqs <= 64) hipLaunchKernelGGL(pkv::plan_kernel<64>, dim3(1), dim3(64), 0, st, a);
    else if (n_seqs <= 128) hipLaunchKernelGGL(pkv::plan_kernel<128>, dim3(1), dim3(128), 0, st, a);
    else if (n_seqs <= 256) hipLaunchKernelGGL(pkv::plan_kernel<256>, dim3(1), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(pkv::plan_kernel<pkv::kPlanThreads>, dim3(1), dim3(pkv::kPlanThreads), 0, st, a);
  }
  if (plan_only) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "decode plan launch: %s", hipGetErrorString(e));
    return PKV_OK;
  }
  const int64_t waves = c.max_units * num_kv_heads * c.gparts;
  if (c.kind == pkv::kKindMfma) {
    const int32_t W = c.waves_per_group;
    if (head_dim == 128) pkv::launch_mfma_p<128>(a, block_size, W, waves, st);
    else pkv::launch_mfma_p<64>(a, block_size, W, waves, st);
  } else if (c.kind == pkv::kKindDpp) {
    if (dtype == PKV_BF16) pkv::launch_dpp<uint16_t>(a, waves, st);
    else pkv::launch_dpp<float>(a, waves, st);
  } else if (dtype == PKV_BF16) {
    pkv::launch_valu<uint16_t>(a, waves, st);
  } else {
    pkv::launch_valu<float>(a, waves, st);
  }
  // some sequence has several partials: a partition split, or a split shared partition
  if (c.need_partials && (c.part_tokens < std::max<int32_t>(max_context_len, 1) || a.pack_max > 1)) {
    const unsigned grid = (unsigned)((int64_t)n_seqs * num_kv_heads * c.gparts);
    if (dtype == PKV_BF16) pkv::launch_merge<uint16_t>(a, grid, st);
    else pkv::launch_merge<float>(a, grid, st);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                                          const void* v_cache, const int32_t* d_block_table,
                                          const int32_t* d_context_lens,
                                          const int32_t* d_shared_prev, int32_t n_seqs,
                                          int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                          int32_t max_blocks_per_seq, int32_t max_context_len,
                                          int64_t total_context_tokens,
                                          int64_t unshared_context_tokens, float scale,
                                          pkv_dtype dtype, pkv_layout k_layout, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  PKV_TRY_BEGIN
  return pkv::decode_impl(out, q, k_cache, v_cache, d_block_table, d_context_lens, d_shared_prev,
                          n_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                          max_blocks_per_seq, max_context_len, total_context_tokens,
                          unshared_context_tokens, scale, dtype, k_layout, workspace,
                          workspace_bytes, false, pkv::kPlanAndRun, stream);
  PKV_TRY_END
}

extern "C" int pkv_decode_plan(const int32_t* d_context_lens, const int32_t* d_shared_prev,
                               int32_t n_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                               int32_t max_context_len, int64_t total_context_tokens,
                               int64_t unshared_context_tokens, pkv_dtype dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  PKV_TRY_BEGIN
  return pkv::decode_impl(nullptr, nullptr, nullptr, nullptr, nullptr, d_context_lens, d_shared_prev,
                          n_seqs, num_q_heads, num_kv_heads, head_dim, block_size, 0,
                          max_blocks_per_seq, max_context_len, total_context_tokens,
                          unshared_context_tokens, 0.f, dtype, PKV_LAYOUT_HEAD_MAJOR, workspace,
                          workspace_bytes, false, pkv::kPlanOnly, stream);
  PKV_TRY_END
}

extern "C" int pkv_paged_attention_decode_planned(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* d_block_table, const int32_t* d_context_lens, const int32_t* d_shared_prev,
    int32_t n_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
    int64_t total_context_tokens, int64_t unshared_context_tokens, float scale, pkv_dtype dtype,
    pkv_layout k_layout, void* workspace, size_t workspace_bytes, void* stream) {
  PKV_TRY_BEGIN
  return pkv::decode_impl(out, q, k_cache, v_cache, d_block_table, d_context_lens, d_shared_prev,
                          n_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                          max_blocks_per_seq, max_context_len, total_context_tokens,
                          unshared_context_tokens, scale, dtype, k_layout, workspace,
                          workspace_bytes, false, pkv::kRunPlanned, stream);
  PKV_TRY_END
}

extern "C" int pkv_paged_attention_decode_noalloc(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* d_block_table, const int32_t* d_context_lens, const int32_t* d_shared_prev,
    int32_t n_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
    int64_t total_context_tokens, int64_t unshared_context_tokens, float scale, pkv_dtype dtype,
    pkv_layout k_layout, void* stream) {
  PKV_TRY_BEGIN
  return pkv::decode_impl(out, q, k_cache, v_cache, d_block_table, d_context_lens, d_shared_prev,
                          n_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                          max_blocks_per_seq, max_context_len, total_context_tokens,
                          unshared_context_tokens, scale, dtype, k_layout, nullptr, 0, true,
                          pkv::kPlanAndRun, stream);
  PKV_TRY_END
}
