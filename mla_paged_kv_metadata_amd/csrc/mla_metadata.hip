// Split-KV schedule (tile_scheduler_metadata and num_splits).
//
// topnet.top "Was ist FlashMLA?", "MLA-Metadaten abrufen": the decode needs
// metadata computed from cache_seqlens and the number of query rows per KV
// head, once per decode step, then reused by every layer.  The pages do not
// say what it holds; this library defines it as follows.
//
// A unit is one sequence (dense) or one (sequence, query token) pair
// (sparse: each query token has its own index list).  Unit u spans n_u >= 1
// blocks of 64 keys.  Units are laid end to end on a line of cost positions,
// each preceded by c0 positions of overhead (queries in, result out); block j
// of unit u sits at C_u + c0 + j with C_u = sum_{v<u} (n_v + c0).  With P
// parts and T = ceil(total / P), a block belongs to part floor(pos / T).
// Every part thus receives at most T positions of work, and a unit is split
// over the parts its blocks fall into.
//
// One 1024-thread workgroup does it all in a single launch (one wave for
// up to 64 dense units): block counts
// (for sparse units, up to one past the last index entry that lies inside
// the sequence, so trailing masked entries cost nothing; one wave per unit),
// the total cost, then the units in chunks of 1024 with two workgroup scans
// each.  The part rows are assembled in LDS and written out at the end.
// Besides its range, a part row carries the length and block count of its
// first unit, so that the decode can start that unit without reading them.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kMdThreads = 1024;
constexpr int kMdWaves = kMdThreads / 64;
constexpr int kUnitCache = 4096;                 // units whose count and length stay in LDS
constexpr int kSmallSparse = 4 * kMdWaves;       // sparse units read in a single pass

template <typename V>
__device__ __forceinline__ V wave_inclusive_scan(V x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const V y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// Exclusive prefix of v over the workgroup, and the workgroup total.  One
// barrier; callers alternate between two `sh` buffers so that a buffer is
// rewritten only after every wave has passed the next call's barrier.
template <typename V>
__device__ __forceinline__ V wg_exclusive_scan(V v, V* sh, V* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const V incl = wave_inclusive_scan(v, lane);
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  const V wt = wave_inclusive_scan(lane < kMdWaves ? sh[lane] : V(0), lane);
  *total = __shfl(wt, kMdWaves - 1);
  const V before = wave > 0 ? __shfl(wt, wave - 1) : V(0);
  return before + incl - v;
}

// Largest entry position in [lo, hi) of index row idx whose value lies in
// [0, L), or -1 (wave-wide; lo, hi multiples of 4 when vec4).  The row is
// read in batches of eight loads per lane, all issued before any is used.
__device__ __forceinline__ int last_valid_in(const int32_t* __restrict__ idx, int lo, int hi, int L, bool vec4,
                                             int lane) {
  constexpr int kBatch = 8;
  int last = -1;
  if (vec4) {
    const int4* idx4 = (const int4*)idx;
    for (int base = lo / 4; base < hi / 4; base += 64 * kBatch) {
      int4 t[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int e4 = base + lane + 64 * k;
        t[k] = e4 < hi / 4 ? idx4[e4] : make_int4(-1, -1, -1, -1);
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int e = 4 * (base + lane + 64 * k);
        if (t[k].x >= 0 && t[k].x < L) last = max(last, e);
        if (t[k].y >= 0 && t[k].y < L) last = max(last, e + 1);
        if (t[k].z >= 0 && t[k].z < L) last = max(last, e + 2);
        if (t[k].w >= 0 && t[k].w < L) last = max(last, e + 3);
      }
    }
  } else {
    for (int base = lo; base < hi; base += 64 * kBatch) {
      int t[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int e = base + lane + 64 * k;
        t[k] = e < hi ? idx[e] : -1;
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        if (t[k] >= 0 && t[k] < L) last = max(last, base + lane + 64 * k);
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) last = max(last, __shfl_xor(last, m));
  return last;
}

// The last kTail entries of an index row, one 16-byte load per lane (vec4)
// or four 4-byte loads per lane, issued without waiting for them.
constexpr int kTail = 256;
struct Tail {
  int4 t;
};
__device__ __forceinline__ Tail load_tail(const int32_t* __restrict__ idx, int topk, bool vec4, int lane) {
  Tail r;
  const int lo = topk > kTail ? topk - kTail : 0;
  if (vec4) {
    const int e4 = lo / 4 + lane;
    r.t = e4 < topk / 4 ? ((const int4*)idx)[e4] : make_int4(-1, -1, -1, -1);
  } else {
    const int e = lo + 4 * lane;
    r.t.x = e < topk ? idx[e] : -1;
    r.t.y = e + 1 < topk ? idx[e + 1] : -1;
    r.t.z = e + 2 < topk ? idx[e + 2] : -1;
    r.t.w = e + 3 < topk ? idx[e + 3] : -1;
  }
  return r;
}
// Largest valid entry position in the tail (wave-wide), or -1.
__device__ __forceinline__ int tail_last(const Tail& r, int topk, int L, int lane) {
  const int e = (topk > kTail ? topk - kTail : 0) + 4 * lane;
  int last = -1;
  if (r.t.x >= 0 && r.t.x < L) last = e;
  if (r.t.y >= 0 && r.t.y < L) last = e + 1;
  if (r.t.z >= 0 && r.t.z < L) last = e + 2;
  if (r.t.w >= 0 && r.t.w < L) last = e + 3;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) last = max(last, __shfl_xor(last, m));
  return last;
}

// Blocks of 64 keys that sparse units ua and ub (ub < 0: none) span, up to
// each one's last entry pointing into its sequence.  One wave; the rows are
// read from the end: the last 256 entries of both rows first, the rest of a
// row only when none of those is valid.
__device__ __forceinline__ void sparse_unit_blocks(const int32_t* __restrict__ indices,
                                                   const int32_t* __restrict__ seqlens, int s_q, int topk,
                                                   int ua, int ub, bool vec4, int lane, int* na, int* nb) {
  const int32_t* ia = indices + (size_t)ua * topk;
  const int32_t* ib = indices + (size_t)(ub >= 0 ? ub : ua) * topk;
  const int La = seqlens[ua / s_q];
  const int Lb = ub >= 0 ? seqlens[ub / s_q] : 0;
  const Tail ta = load_tail(ia, topk, vec4, lane);
  const Tail tb = load_tail(ib, topk, vec4, lane);
  int la = tail_last(ta, topk, La, lane);
  int lb = ub >= 0 ? tail_last(tb, topk, Lb, lane) : -1;
  const int rest = topk > kTail ? topk - kTail : 0;
  if (la < 0 && rest > 0) la = last_valid_in(ia, 0, rest, La, vec4, lane);
  if (ub >= 0 && lb < 0 && rest > 0) lb = last_valid_in(ib, 0, rest, Lb, vec4, lane);
  *na = max(1, (la + 1 + kPage - 1) / kPage);
  *nb = max(1, (lb + 1 + kPage - 1) / kPage);
}

__device__ __forceinline__ int dense_unit_blocks(int L) {
  const int n = (L + kPage - 1) / kPage;
  return n < 1 ? 1 : n;
}

}  // namespace

// Unit positions on the cost line, split counts and the part rows, 1024
// units at a time (Pos: the integer type of cost positions).  Part indices
// stay below kMaxParts and fit an int.
template <bool SPARSE, typename Pos>
__device__ __forceinline__ void place_units(const int32_t* __restrict__ seqlens, const int32_t* unit_blocks,
                                            const int32_t* ucnt, const int32_t* ulen, int s_q, int units, Pos T,
                                            int32_t* rows, int32_t* __restrict__ num_splits, Pos (*sh)[kMdWaves]) {
  const int tid = threadIdx.x;
  const Pos c0 = kUnitOverhead;
  Pos carry_c = 0, carry_k = 0;
  for (int base = 0; base < units; base += kMdThreads) {
    const int u = base + tid;
    const bool live = u < units;
    Pos nb = 0;
    int Lu = 0;
    if (live) {
      if (u < kUnitCache) {
        Lu = ulen[u];
        nb = SPARSE ? ucnt[u] : dense_unit_blocks(Lu);
      } else {
        Lu = seqlens[SPARSE ? u / s_q : u];
        nb = SPARSE ? unit_blocks[u] : dense_unit_blocks(Lu);
      }
    }
    const Pos c = live ? nb + c0 : 0;
    Pos chunk_c, chunk_k;
    const Pos Cu = carry_c + wg_exclusive_scan(c, sh[1], &chunk_c);
    int f = 0, l = -1;
    if (live) {
      f = (int)((Cu + c0) / T);
      l = (int)((Cu + c0 + nb - 1) / T);
    }
    const Pos k = live ? (Pos)(l - f + 1) : 0;
    const Pos Ku = carry_k + wg_exclusive_scan(k, sh[0], &chunk_k);
    if (live) {
      num_splits[u + 1] = (int32_t)(Ku + k);
      // Parts whose first unit is u: those of u's parts that the previous
      // unit (whose last block sits at position Cu - 1) does not reach.
      const int lo = u > 0 ? max(f, (int)((Cu - 1) / T) + 1) : f;
      for (int pp = lo; pp <= l; ++pp) {
        int32_t* row = rows + kPartRow * pp;
        row[0] = u;
        row[1] = (int32_t)(pp == f ? 0 : (Pos)pp * T - Cu - c0);
        row[4] = pp - f;
        row[5] = Lu;
        row[6] = (int32_t)nb;
      }
      // Parts whose last unit is u: those the next unit does not start in.
      const int hi = (u + 1 < units) ? min(l, (int)((Cu + c + c0) / T) - 1) : l;
      for (int pp = f; pp <= hi; ++pp) {
        int32_t* row = rows + kPartRow * pp;
        row[2] = u;
        row[3] = (int32_t)(pp == l ? nb : (Pos)(pp + 1) * T - Cu - c0);
      }
    }
    carry_c += chunk_c;
    carry_k += chunk_k;
  }
}

template <bool SPARSE>
__global__ __launch_bounds__(kMdThreads) void metadata_kernel(const int32_t* __restrict__ seqlens,
                                                              const int32_t* __restrict__ indices,
                                                              int s_q, int topk, int vec4, int units,
                                                              int num_parts, int32_t* __restrict__ md,
                                                              int32_t* __restrict__ num_splits) {
  __shared__ long long sh[2][kMdWaves];
  __shared__ uint32_t sh32[2][kMdWaves];
  __shared__ int32_t rows[kMaxParts * kPartRow];
  // Sparse: bit u set when unit u's block count is known from its last
  // index entry alone (units below kDoneBits).
  constexpr int kDoneBits = SPARSE ? 65536 : 32;
  __shared__ uint32_t done[kDoneBits / 32];
  // Block counts and sequence lengths of units below kUnitCache, kept here
  // so that the positions pass below reads no global memory for them.
  __shared__ int32_t ucnt[kUnitCache];
  __shared__ int32_t ulen[kUnitCache];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = num_parts;
  const long long c0 = kUnitOverhead;
  int32_t* unit_blocks = md + kHeader + kPartRow * P;

  // Every part starts empty.
  for (int i = tid; i < P * kPartRow; i += kMdThreads) {
    const int f = i & (kPartRow - 1);
    rows[i] = (f == 0 || f == 2) ? -1 : 0;
  }

  // Block counts and the total cost.
  long long cost = 0;
  if (SPARSE && units <= kSmallSparse) {
    // Few units: wave w takes units w, w + 16, w + 32 and w + 48 and loads
    // the last 256 entries of all of them at once; a row is scanned further
    // only when none of those entries points into its sequence.
    Tail t[kSmallSparse / kMdWaves];
    int L[kSmallSparse / kMdWaves];
#pragma unroll
    for (int k = 0; k < kSmallSparse / kMdWaves; ++k) {
      const int u = wave + kMdWaves * k;
      if (u < units) {
        L[k] = seqlens[u / s_q];
        t[k] = load_tail(indices + (size_t)u * topk, topk, vec4 != 0, lane);
      }
    }
    const int rest = topk > kTail ? topk - kTail : 0;
#pragma unroll
    for (int k = 0; k < kSmallSparse / kMdWaves; ++k) {
      const int u = wave + kMdWaves * k;
      if (u < units) {
        int last = tail_last(t[k], topk, L[k], lane);
        if (last < 0 && rest > 0) last = last_valid_in(indices + (size_t)u * topk, 0, rest, L[k], vec4 != 0, lane);
        const int n = max(1, (last + 1 + kPage - 1) / kPage);
        if (lane == 0) {
          unit_blocks[u] = n;
          ucnt[u] = n;
          ulen[u] = L[k];
          cost += n + c0;
        }
      }
    }
  } else if (SPARSE) {
    for (int i = tid; i < kDoneBits / 32; i += kMdThreads) done[i] = 0u;
    __syncthreads();
    // A row whose last entry points into the sequence spans all its blocks
    // (the usual case): one thread per unit reads just that entry.  Only
    // units that have a done bit are settled here; the scan below counts
    // every other unit (units from kDoneBits on are always scanned).
    const int n_all = (topk + kPage - 1) / kPage;
    for (int u = tid; u < units; u += kMdThreads) {
      const int Lu = seqlens[u / s_q];
      if (u < kUnitCache) ulen[u] = Lu;
      if (u >= kDoneBits) continue;
      const int last = indices[(size_t)u * topk + topk - 1];
      if (last >= 0 && last < Lu) {
        unit_blocks[u] = n_all;
        if (u < kUnitCache) ucnt[u] = n_all;
        cost += n_all + c0;
        atomicOr(&done[u >> 5], 1u << (u & 31));
      }
    }
    __syncthreads();
    // The other rows: wave w looks at units w, w + 16, w + 32, ... (lane l
    // of a chunk of 1024 units at unit 16 l + w, so that neighbouring open
    // rows go to different waves) and scans the open rows two at a time
    // from the end.
    for (int base = 0; base < units; base += 64 * kMdWaves) {
      const int u = base + kMdWaves * lane + wave;
      const bool open = u < units && (u >= kDoneBits || ((done[u >> 5] >> (u & 31)) & 1u) == 0u);
      uint64_t todo = __ballot(open);
      while (todo != 0ull) {
        const int ua = base + kMdWaves * __builtin_ctzll(todo) + wave;
        todo &= todo - 1;
        int ub = -1;
        if (todo != 0ull) {
          ub = base + kMdWaves * __builtin_ctzll(todo) + wave;
          todo &= todo - 1;
        }
        int n, n2;
        sparse_unit_blocks(indices, seqlens, s_q, topk, ua, ub, vec4 != 0, lane, &n, &n2);
        if (lane == 0) {
          unit_blocks[ua] = n;
          if (ua < kUnitCache) ucnt[ua] = n;
          cost += n + c0;
          if (ub >= 0) {
            unit_blocks[ub] = n2;
            if (ub < kUnitCache) ucnt[ub] = n2;
            cost += n2 + c0;
          }
        }
      }
    }
  } else {
    for (int u = tid; u < units; u += kMdThreads) {
      const int Lu = seqlens[u];
      const int n = dense_unit_blocks(Lu);
      if (u < kUnitCache) ulen[u] = Lu;
      unit_blocks[u] = n;
      cost += n + c0;
    }
  }
  // Counts and lengths of units at or above kUnitCache are read back from
  // global memory below; the barrier in the scan orders them (and the LDS
  // entries) after these stores.
  long long tot_cost;
  wg_exclusive_scan(cost, sh[0], &tot_cost);
  const long long T = tot_cost > 0 ? (tot_cost + P - 1) / P : 1;
  const long long tot_blocks = tot_cost - c0 * units;
  // Positions in 32 bits whenever the whole cost line allows it (then
  // P * T < 2^31 + P as well): the divisions by T are then short.
  if (tot_cost < (1LL << 31))
    place_units<SPARSE, uint32_t>(seqlens, unit_blocks, ucnt, ulen, s_q, units, (uint32_t)T, rows, num_splits, sh32);
  else
    place_units<SPARSE, long long>(seqlens, unit_blocks, ucnt, ulen, s_q, units, T, rows, num_splits, sh);
  __syncthreads();

  if (tid == 0) {
    num_splits[0] = 0;
  }
  if (tid < kHeader) {
    const int32_t v = tid == 0 ? P
                      : tid == 1 ? (int32_t)T
                      : tid == 2 ? (int32_t)c0
                      : tid == 3 ? units
                      : tid == 4 ? (int32_t)tot_blocks
                      : tid == 5 ? kMagic : 0;
    md[tid] = v;
  }
  for (int i = tid; i < P * kPartRow; i += kMdThreads) md[kHeader + i] = rows[i];
}

// Dense schedules of at most 64 units: one wave, one lane per unit, the
// same arithmetic as metadata_kernel without its workgroup scans.  With
// n_u <= 2^25 (L_b < 2^31) and at most 64 units every cost position is
// below 2^32, so the cost line is kept in 32-bit unsigned arithmetic.
__global__ __launch_bounds__(64) void metadata_wave_kernel(const int32_t* __restrict__ seqlens, int units,
                                                          int num_parts, int32_t* __restrict__ md,
                                                          int32_t* __restrict__ num_splits) {
  // num_parts rows of LDS (dynamic: small enough to share a CU with a
  // decode workgroup when schedules are built alongside a decode).
  extern __shared__ int32_t rows[];
  const int lane = threadIdx.x;
  const int P = num_parts;
  const uint32_t c0 = kUnitOverhead;
  int32_t* unit_blocks = md + kHeader + kPartRow * P;
  const bool live = lane < units;
  const int Lu = live ? seqlens[lane] : 0;
  for (int i = lane; i < P * kPartRow; i += 64) {
    const int f = i & (kPartRow - 1);
    rows[i] = (f == 0 || f == 2) ? -1 : 0;
  }
  const uint32_t nb = live ? (uint32_t)dense_unit_blocks(Lu) : 0u;
  if (live) unit_blocks[lane] = (int32_t)nb;
  const uint32_t c = live ? nb + c0 : 0u;
  const uint32_t incl = wave_inclusive_scan<uint32_t>(c, lane);
  const uint32_t tot_cost = __shfl(incl, 63);
  const uint32_t T = tot_cost > 0 ? (tot_cost - 1) / (uint32_t)P + 1 : 1u;
  const uint32_t Cu = incl - c;
  // Part indices (below 2048) in signed arithmetic, positions unsigned.
  int f = 0, l = -1;
  if (live) {
    f = (int)((Cu + c0) / T);
    l = (int)((Cu + c0 + nb - 1) / T);
  }
  const uint32_t k = live ? (uint32_t)(l - f + 1) : 0u;
  const uint32_t kincl = wave_inclusive_scan<uint32_t>(k, lane);
  __syncthreads();   // row defaults before the rows below
  if (live) {
    num_splits[lane + 1] = (int32_t)kincl;
    // Parts whose first unit is this one: those the previous unit (whose
    // last block sits at position Cu - 1) does not reach.
    const int lo = lane > 0 ? max(f, (int)((Cu - 1) / T) + 1) : f;
    for (int pp = lo; pp <= l; ++pp) {
      int32_t* row = rows + kPartRow * pp;
      row[0] = lane;
      row[1] = pp == f ? 0 : (int32_t)((uint32_t)pp * T - Cu - c0);
      row[4] = pp - f;
      row[5] = Lu;
      row[6] = (int32_t)nb;
    }
    // Parts whose last unit is this one: those the next unit does not
    // start in.
    const int hi = (lane + 1 < units) ? min(l, (int)((Cu + c + c0) / T) - 1) : l;
    for (int pp = f; pp <= hi; ++pp) {
      int32_t* row = rows + kPartRow * pp;
      row[2] = lane;
      row[3] = pp == l ? (int32_t)nb : (int32_t)((uint32_t)(pp + 1) * T - Cu - c0);
    }
  }
  __syncthreads();
  if (lane == 0) num_splits[0] = 0;
  if (lane < kHeader) {
    const int32_t v = lane == 0 ? P
                      : lane == 1 ? (int32_t)T
                      : lane == 2 ? (int32_t)c0
                      : lane == 3 ? units
                      : lane == 4 ? (int32_t)(tot_cost - c0 * (uint32_t)units)
                      : lane == 5 ? kMagic : 0;
    md[lane] = v;
  }
  // The rows, 16 bytes per lane and store when the buffer allows it.
  int32_t* dst = md + kHeader;
  if (((uintptr_t)dst & 15) == 0) {
    const int4* src4 = (const int4*)rows;
    int4* dst4 = (int4*)dst;
    for (int i = lane; i < P * kPartRow / 4; i += 64) dst4[i] = src4[i];
  } else {
    for (int i = lane; i < P * kPartRow; i += 64) dst[i] = rows[i];
  }
}

hipError_t launch_metadata(const int32_t* seqlens, const int32_t* indices, int s_q, int topk,
                           int units, int num_parts, int32_t* md, int32_t* num_splits,
                           hipStream_t stream) {
  if (num_parts < 1 || num_parts > kMaxParts) return hipErrorInvalidValue;
  if (indices == nullptr && units <= 64) {
    hipLaunchKernelGGL(metadata_wave_kernel, dim3(1), dim3(64), (size_t)num_parts * kPartRow * sizeof(int32_t),
                       stream, seqlens, units, num_parts, md, num_splits);
  } else if (indices == nullptr) {
    hipLaunchKernelGGL(metadata_kernel<false>, dim3(1), dim3(kMdThreads), 0, stream, seqlens, indices,
                       s_q, topk, 0, units, num_parts, md, num_splits);
  } else {
    const int vec4 = (topk % 4 == 0) && ((uintptr_t)indices % 16 == 0);
    hipLaunchKernelGGL(metadata_kernel<true>, dim3(1), dim3(kMdThreads), 0, stream, seqlens, indices,
                       s_q, topk, vec4, units, num_parts, md, num_splits);
  }
  return hipGetLastError();
}

}  // namespace mla
