// cache_append and copy_blocks: bit copies into the paged K/V caches.
//
// "PagedAttention Internals", section "Fixed-Size KV Blocks": each generated
// token is stored in its sequence's current block; the slot comes from the
// host pool.  "pagedattention" topic page, fourth paragraph: shared blocks are
// copied only when a sharer diverges (copy_blocks performs that copy).
//
// Layout: k_cache [NB, Hkv, P, D] (token rows), v_cache [NB, Hkv, D, P]
// (value columns per token).  Elements are moved as raw 16- or 32-bit words.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "device_common.hpp"
#include "internal.hpp"

namespace pkv {
namespace {

// One workgroup per token (grid-stride).  Keys: each token row of every head
// is contiguous in the cache, so threads move 16-byte pieces (vec_ok) or
// single elements.  Values: the token's column is strided by P elements, so
// threads move single elements, consecutive threads taking consecutive head_dim
// rows (a store instruction covers one compact run of the value tiles),
// kAppendBatch elements per thread per batch with the batch's loads issued
// before its stores.  The first key piece and the first value batch do not
// depend on the slot and are loaded before it is tested.
constexpr int kAppendBatch = 4;

template <typename E>
__global__ __launch_bounds__(256) void cache_append_kernel(
    E* __restrict__ kc, E* __restrict__ vc, const E* __restrict__ kn, const E* __restrict__ vn,
    const int32_t* __restrict__ slots, int32_t n_tokens, int64_t num_slots, int32_t hkv,
    int32_t d, int32_t p, KStrides ks, int32_t vec_ok, int32_t* __restrict__ err) {
  constexpr int V = 16 / sizeof(E);  // elements per 16-byte piece
  const int32_t hd = hkv * d;
  const int32_t nvec = vec_ok ? hd / V : 0;  // key pieces per row
  const int32_t tid = threadIdx.x, nt = blockDim.x;
  for (int32_t tok = blockIdx.x; tok < n_tokens; tok += gridDim.x) {
    const E* ksrc = kn + (int64_t)tok * hd;
    const E* vsrc = vn + (int64_t)tok * hd;
    // loads that do not depend on the slot
    uint4 kx = uint4{0, 0, 0, 0};
    if (tid < nvec) kx = *reinterpret_cast<const uint4*>(ksrc + tid * V);
    uint32_t vb[kAppendBatch];
#pragma unroll
    for (int u = 0; u < kAppendBatch; ++u) {
      const int32_t e = tid + u * nt;
      vb[u] = e < hd ? (uint32_t)vsrc[e] : 0u;
    }
    const int32_t s = slots[tok];
    if (s < 0) continue;
    if ((int64_t)s >= num_slots) {
      if (tid == 0) atomicOr(err, PKV_DEVERR_SLOT);
      continue;
    }
    const int64_t blk = s / p, off = s % p;
    E* krow = kc + blk * hd * p + off * ks.tok;  // + h * ks.head + dd
    if (vec_ok) {
      for (int32_t i = tid; i < nvec; i += nt) {
        const uint4 x = i == tid ? kx : *reinterpret_cast<const uint4*>(ksrc + i * V);
        const int32_t e = i * V, h = e / d, dd = e % d;
        *reinterpret_cast<uint4*>(krow + h * ks.head + dd) = x;
      }
    } else {
      for (int32_t e = tid; e < hd; e += nt) krow[(e / d) * ks.head + e % d] = ksrc[e];
    }
    E* vtile = vc + blk * hkv * d * p + off;  // + ((h d) + dd) p = e p
    for (int32_t e0 = tid; e0 < hd; e0 += kAppendBatch * nt) {
      uint32_t w[kAppendBatch];
#pragma unroll
      for (int u = 0; u < kAppendBatch; ++u) {
        const int32_t e = e0 + u * nt;
        w[u] = e0 == tid ? vb[u] : (e < hd ? (uint32_t)vsrc[e] : 0u);
      }
#pragma unroll
      for (int u = 0; u < kAppendBatch; ++u) {
        const int32_t e = e0 + u * nt;
        if (e < hd) vtile[(int64_t)e * p] = (E)w[u];
      }
    }
  }
}

// Bulk appends (a prefill writes whole blocks).  Workgroup w takes the token
// rows [w kWin, w kWin + kWin) and finds the runs of P rows whose slots fill
// one whole block in order (a run starts at a row whose slot is a multiple of
// P).  A window owns every run that starts inside it, also one that reaches
// up to P - 1 rows past its end, so window edges cut no run; rows covered by
// a run the previous window owns are left to that window.  A run's key tile
// is a straight copy and its value tile is transposed through LDS and written
// as full rows of P tokens, so HBM sees whole-sector writes instead of one 2-
// or 4-byte write per value element.  Rows outside runs (partial blocks,
// skipped or bad slots) are copied element by element.  Runs write disjoint
// blocks, so the order in which a workgroup takes them does not matter.
constexpr int kTileLdsBytes = 32768;
constexpr int kWin = 256;
constexpr int kTileMaxBlock = 256;            // longest block the tile path takes
constexpr int kHalo = kTileMaxBlock - 1;      // rows a window looks past either edge

template <typename E>
__global__ __launch_bounds__(256) void cache_append_tiles_kernel(
    E* __restrict__ kc, E* __restrict__ vc, const E* __restrict__ kn, const E* __restrict__ vn,
    const int32_t* __restrict__ slots, int32_t n_tokens, int64_t num_slots, int32_t hkv,
    int32_t d, int32_t p, KStrides ks, int32_t* __restrict__ err) {
  __shared__ uint4 lds_raw[kTileLdsBytes / 16];
  __shared__ int32_t ws[kWin + 2 * kHalo];        // slots of rows [lo, hi)
  __shared__ uint8_t covered[kWin + 2 * kHalo];
  __shared__ int32_t run_start[kWin], loose[kWin];  // rows relative to the window start
  __shared__ int32_t n_runs, n_loose;
  constexpr int V = 16 / sizeof(E);  // elements per 16-byte chunk
  const int32_t hd = hkv * d;
  const int32_t tid = threadIdx.x, nth = blockDim.x;
  const int32_t n_win = (n_tokens + kWin - 1) / kWin;
  for (int32_t wdx = blockIdx.x; wdx < n_win; wdx += gridDim.x) {
    const int32_t i0 = wdx * kWin, cnt = min(kWin, n_tokens - i0);
    const int32_t lo = max(0, i0 - (p - 1)), hi = min(n_tokens, i0 + cnt + (p - 1));
    const int32_t ext = hi - lo, base = i0 - lo;  // window row t is ws[base + t]
    for (int32_t x = tid; x < ext; x += nth) {
      ws[x] = slots[lo + x];
      covered[x] = 0;
    }
    if (tid == 0) {
      n_runs = 0;
      n_loose = 0;
    }
    __syncthreads();
    // runs starting in [lo, i0 + cnt): all mark their rows, the ones starting
    // at or after i0 are this window's
    for (int32_t x = tid; x < base + cnt; x += nth) {
      const int32_t s0 = ws[x];
      bool ok = s0 >= 0 && s0 % p == 0 && x + p <= ext && (int64_t)s0 + p <= num_slots;
      for (int32_t j = 1; ok && j < p; ++j) ok = ws[x + j] == s0 + j;
      if (ok) {
        for (int32_t j = 0; j < p; ++j) covered[x + j] = 1;
        if (x >= base) run_start[atomicAdd(&n_runs, 1)] = x - base;
      }
    }
    __syncthreads();
    for (int32_t t = tid; t < cnt; t += nth)
      if (!covered[base + t] && ws[base + t] >= 0) loose[atomicAdd(&n_loose, 1)] = t;
    __syncthreads();
    // rows outside runs, element by element
    for (int32_t e = tid; e < n_loose * hd; e += nth) {
      const int32_t q = e / hd, r = e - q * hd;
      const int32_t row = loose[q], sl = ws[base + row];
      if (sl < 0) continue;
      if ((int64_t)sl >= num_slots) {
        if (r == 0) atomicOr(err, PKV_DEVERR_SLOT);
        continue;
      }
      const int64_t blk = sl / p, off = sl % p;
      const int32_t h = r / d, dd = r - h * d;
      kc[blk * hd * p + h * ks.head + off * ks.tok + dd] = kn[(int64_t)(i0 + row) * hd + r];
      vc[((blk * hkv + h) * d + dd) * p + off] = vn[(int64_t)(i0 + row) * hd + r];
    }
    // whole-block runs.  The value tile sits in LDS with token rows of
    // d elements plus one 4-byte word: the transposed reads walk a column,
    // and without the pad the lanes of one column (rows 256 bytes apart for
    // head_dim 128 in bf16) would all hit one bank.
    const int32_t dv = d / V, pv = p / V;
    const int32_t per = p * dv;                             // 16-byte chunks per head tile
    const int32_t rw = d * (int32_t)sizeof(E) / 4 + 1;      // LDS words per token row
    const int32_t hb = max(1, (kTileLdsBytes / 4) / (p * rw));  // heads per LDS pass
    uint32_t* tile_w = reinterpret_cast<uint32_t*>(lds_raw);
    const int32_t nr = n_runs;
    for (int32_t ri = 0; ri < nr; ++ri) {
      const int32_t t0 = run_start[ri];
      const int64_t blk = ws[base + t0] / p;
      const int64_t row0 = i0 + t0;
      for (int32_t h0 = 0; h0 < hkv; h0 += hb) {
        const int32_t nh = min(hb, hkv - h0);
        for (int32_t c = tid; c < nh * per; c += nth) {
          const int32_t hh = c / per, r = c - hh * per, j = r / dv, x = r - j * dv;
          const int64_t src = (row0 + j) * hd + (h0 + hh) * d;
          *reinterpret_cast<uint4*>(kc + blk * hd * p + (h0 + hh) * ks.head + j * ks.tok + x * V) =
              reinterpret_cast<const uint4*>(kn + src)[x];
          const uint4 vv = reinterpret_cast<const uint4*>(vn + src)[x];
          uint32_t* dst = tile_w + (hh * p + j) * rw + 4 * x;
          dst[0] = vv.x;
          dst[1] = vv.y;
          dst[2] = vv.z;
          dst[3] = vv.w;
        }
        __syncthreads();
        const int32_t outc = d * pv;                        // 16-byte chunks per transposed tile
        for (int32_t c = tid; c < nh * outc; c += nth) {
          const int32_t hh = c / outc, r = c - hh * outc, dd = r / pv, j0 = (r - dd * pv) * V;
          const E* srct = reinterpret_cast<const E*>(tile_w + hh * p * rw);
          const int32_t es = rw * 4 / (int32_t)sizeof(E);   // elements per padded row (bf16: 2 rw)
          E chunk[V];
#pragma unroll
          for (int k = 0; k < V; ++k) chunk[k] = srct[(j0 + k) * es + dd];
          reinterpret_cast<uint4*>(vc + (blk * hkv + h0 + hh) * d * p)[r] =
              *reinterpret_cast<const uint4*>(chunk);
        }
        __syncthreads();
      }
    }
    __syncthreads();  // the next window reuses the shared lists
  }
}

constexpr int kMaxPairsPerLaunch = 128;

struct CopyPairs {
  int32_t src[kMaxPairsPerLaunch];
  int32_t dst[kMaxPairsPerLaunch];
};

// grid (chunks, pairs): every block is one contiguous run of `words` words in
// each cache, whatever the layout inside it.  Each thread moves kCopyUnroll
// words of each cache, all loads issued before the stores.  One word per
// thread measured best: copy-on-write batches are small (a decode step copies
// at most one block per sequence), so spreading them over more workgroups
// beats deeper per-thread pipelines.
constexpr int kCopyUnroll = 1;

template <typename W>
__global__ __launch_bounds__(256) void copy_blocks_kernel(W* __restrict__ kc, W* __restrict__ vc,
                                                          CopyPairs pairs, int64_t words,
                                                          int32_t num_blocks,
                                                          int32_t* __restrict__ err) {
  const int32_t src = pairs.src[blockIdx.y], dst = pairs.dst[blockIdx.y];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(err, PKV_DEVERR_COPY_PAIR);
    return;
  }
  const W* ks = kc + (int64_t)src * words;
  const W* vs = vc + (int64_t)src * words;
  W* kd = kc + (int64_t)dst * words;
  W* vd = vc + (int64_t)dst * words;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i0 < words;
       i0 += stride * kCopyUnroll) {
    W k[kCopyUnroll], v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < words) {
        k[u] = ks[i];
        v[u] = vs[i];
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < words) {
        kd[i] = k[u];
        vd[i] = v[u];
      }
    }
  }
}

// Apply one block-table patch (incremental table upload).  The host has
// checked every row, column and count against the table's shape.
__global__ __launch_bounds__(256) void table_patch_kernel(TablePatchArgs p) {
  const int32_t tid = threadIdx.x, nth = blockDim.x;
  const int32_t* w = p.w;
  for (int32_t i = tid; i < p.n_len; i += nth) p.lens[p.len0 + i] = w[i];
  for (int32_t i = tid; i < p.n_sh; i += nth) p.shared[p.sh0 + i] = w[p.n_len + i];
  for (int32_t i = tid; i < p.n_slot; i += nth) p.slots[p.slot0 + i] = w[p.n_len + p.n_sh + i];
  const int32_t* e = w + p.n_len + p.n_sh + p.n_slot;
  for (int32_t i = tid; i < p.n_ent; i += nth)
    p.table[(int64_t)e[3 * i] * p.max_blocks + e[3 * i + 1]] = e[3 * i + 2];
  const int32_t* r = e + 3 * p.n_ent;
  for (int32_t k = 0; k < p.n_reset; ++k) {
    int32_t* row = p.table + (int64_t)r[2 * k] * p.max_blocks;
    for (int32_t c = r[2 * k + 1] + tid; c < p.max_blocks; c += nth) row[c] = -1;
  }
}

}  // namespace

int launch_table_patch(const TablePatchArgs& args, void* stream) {
  hipLaunchKernelGGL(table_patch_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, args);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "table patch launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // namespace pkv

using pkv::fail;

extern "C" int pkv_cache_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                                const int32_t* d_slot_mapping, int32_t n_tokens, int32_t num_blocks,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                pkv_dtype dtype, pkv_layout k_layout, void* stream) {
  PKV_TRY_BEGIN
  if (n_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID_ARG, "bad sizes");
  if (!pkv::dtype_valid(dtype)) return fail(PKV_ERR_INVALID_ARG, "bad dtype");
  if (!pkv::layout_valid(k_layout)) return fail(PKV_ERR_INVALID_ARG, "bad key layout");
  const pkv::KStrides ks = pkv::k_strides(k_layout, num_kv_heads, block_size, head_dim);
  if (n_tokens == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !d_slot_mapping)
    return fail(PKV_ERR_INVALID_ARG, "NULL pointer");
  int32_t* err = nullptr;
  int rc = pkv::device_error_word(&err);
  if (rc) return rc;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  const size_t es = pkv::dtype_size(dtype);
  const int32_t vec_ok = ((size_t)head_dim * es % 16 == 0) &&
                         ((uintptr_t)k_cache % 16 == 0) && ((uintptr_t)k_new % 16 == 0);
  hipStream_t st = (hipStream_t)stream;
  // whole-block tile path for bulk appends (every row and tile 16-byte aligned)
  const size_t tile_bytes = (size_t)block_size * (head_dim * es + 4);  // padded LDS rows
  const bool tiles_fit = vec_ok && ((size_t)block_size * es) % 16 == 0 &&
                         block_size <= pkv::kTileMaxBlock &&
                         tile_bytes <= (size_t)pkv::kTileLdsBytes && (uintptr_t)v_cache % 16 == 0 &&
                         (uintptr_t)v_new % 16 == 0;
  const char* mode = std::getenv("PKV_APPEND_TILES");
  bool tiles = tiles_fit && n_tokens >= 4096;
  if (mode && std::strcmp(mode, "on") == 0) tiles = tiles_fit;
  if (mode && std::strcmp(mode, "off") == 0) tiles = false;
  if (tiles) {
    const int groups = (int)std::min<int64_t>((n_tokens + pkv::kWin - 1) / pkv::kWin, 1 << 16);
    if (dtype == PKV_BF16)
      hipLaunchKernelGGL(pkv::cache_append_tiles_kernel<uint16_t>, dim3(groups), dim3(256), 0, st,
                         (uint16_t*)k_cache, (uint16_t*)v_cache, (const uint16_t*)k_new,
                         (const uint16_t*)v_new, d_slot_mapping, n_tokens, num_slots, num_kv_heads,
                         head_dim, block_size, ks, err);
    else
      hipLaunchKernelGGL(pkv::cache_append_tiles_kernel<uint32_t>, dim3(groups), dim3(256), 0, st,
                         (uint32_t*)k_cache, (uint32_t*)v_cache, (const uint32_t*)k_new,
                         (const uint32_t*)v_new, d_slot_mapping, n_tokens, num_slots, num_kv_heads,
                         head_dim, block_size, ks, err);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "cache_append launch: %s", hipGetErrorString(e));
    return PKV_OK;
  }
  const int grid = (int)std::min<int32_t>(n_tokens, 1 << 16);
  if (dtype == PKV_BF16)
    hipLaunchKernelGGL(pkv::cache_append_kernel<uint16_t>, dim3(grid), dim3(256), 0, st,
                       (uint16_t*)k_cache, (uint16_t*)v_cache, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, d_slot_mapping, n_tokens, num_slots, num_kv_heads,
                       head_dim, block_size, ks, vec_ok, err);
  else
    hipLaunchKernelGGL(pkv::cache_append_kernel<uint32_t>, dim3(grid), dim3(256), 0, st,
                       (uint32_t*)k_cache, (uint32_t*)v_cache, (const uint32_t*)k_new,
                       (const uint32_t*)v_new, d_slot_mapping, n_tokens, num_slots, num_kv_heads,
                       head_dim, block_size, ks, vec_ok, err);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "cache_append launch: %s", hipGetErrorString(e));
  return PKV_OK;
  PKV_TRY_END
}

extern "C" int pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t n_pairs,
                               int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, pkv_dtype dtype, void* stream) {
  PKV_TRY_BEGIN
  if (n_pairs < 0 || num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID_ARG, "bad sizes");
  if (!pkv::dtype_valid(dtype)) return fail(PKV_ERR_INVALID_ARG, "bad dtype");
  if (n_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !pairs) return fail(PKV_ERR_INVALID_ARG, "NULL pointer");
  int32_t* err = nullptr;
  int rc = pkv::device_error_word(&err);
  if (rc) return rc;
  const int64_t bytes = (int64_t)num_kv_heads * block_size * head_dim * pkv::dtype_size(dtype);
  const bool vec = bytes % 16 == 0 && (uintptr_t)k_cache % 16 == 0 && (uintptr_t)v_cache % 16 == 0;
  const int64_t words = vec ? bytes / 16 : bytes / 2;
  const int chunks = (int)std::max<int64_t>(
      1, std::min<int64_t>(64, (words + 256 * pkv::kCopyUnroll - 1) / (256 * pkv::kCopyUnroll)));
  hipStream_t st = (hipStream_t)stream;
  for (int32_t base = 0; base < n_pairs; base += pkv::kMaxPairsPerLaunch) {
    const int32_t n = std::min(pkv::kMaxPairsPerLaunch, n_pairs - base);
    pkv::CopyPairs cp;
    for (int32_t i = 0; i < n; ++i) {
      cp.src[i] = pairs[2 * (base + i)];
      cp.dst[i] = pairs[2 * (base + i) + 1];
    }
    if (vec)
      hipLaunchKernelGGL(pkv::copy_blocks_kernel<uint4>, dim3(chunks, n), dim3(256), 0, st,
                         (uint4*)k_cache, (uint4*)v_cache, cp, words, num_blocks, err);
    else
      hipLaunchKernelGGL(pkv::copy_blocks_kernel<uint16_t>, dim3(chunks, n), dim3(256), 0, st,
                         (uint16_t*)k_cache, (uint16_t*)v_cache, cp, words, num_blocks, err);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "copy_blocks launch: %s", hipGetErrorString(e));
  }
  return PKV_OK;
  PKV_TRY_END
}
