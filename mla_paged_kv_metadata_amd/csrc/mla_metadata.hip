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
// Two kernels: one wave per unit counts its blocks (for sparse units, up to
// one past the last index entry that lies inside the sequence, so trailing
// masked entries cost nothing); then a single 1024-thread workgroup scans the
// units in chunks and writes every part's row in closed form.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

__global__ __launch_bounds__(256) void unit_blocks_kernel(const int32_t* __restrict__ seqlens,
                                                          const int32_t* __restrict__ indices,
                                                          int s_q, int topk, int units,
                                                          int32_t* __restrict__ unit_blocks) {
  const int lane = threadIdx.x & 63;
  const int u = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (u >= units) return;
  int n;
  if (indices == nullptr) {
    const int L = seqlens[u];
    n = (L + kPage - 1) / kPage;
  } else {
    const int L = seqlens[u / s_q];
    const int32_t* idx = indices + (size_t)u * topk;
    int last = -1;
    for (int e = lane; e < topk; e += 64) {
      const int t = idx[e];
      if (t >= 0 && t < L) last = e;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) last = max(last, __shfl_xor(last, m));
    n = (last + 1 + kPage - 1) / kPage;
  }
  if (lane == 0) unit_blocks[u] = n < 1 ? 1 : n;
}

// Exclusive scan of one int64 value per thread over a 1024-thread block.
// Returns the exclusive prefix; *total receives the block sum.
__device__ long long block_exclusive_scan(long long v, long long* total, long long* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  long long x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long long y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    long long acc = 0;
    for (int w = 0; w < 16; ++w) {
      const long long t = sh[w];
      sh[w] = acc;
      acc += t;
    }
    sh[16] = acc;
  }
  __syncthreads();
  const long long excl = sh[wave] + x - v;
  *total = sh[16];
  __syncthreads();
  return excl;
}

__global__ __launch_bounds__(1024) void schedule_kernel(int units, int num_parts,
                                                        int32_t* __restrict__ md,
                                                        int32_t* __restrict__ num_splits) {
  __shared__ long long sh[17];
  const int tid = threadIdx.x;
  const int P = num_parts;
  const long long c0 = kUnitOverhead;
  const int32_t* unit_blocks = md + kHeader + kPartRow * P;

  // Pass 1: total cost and total blocks.
  long long cost = 0, blocks = 0;
  for (int u = tid; u < units; u += 1024) {
    const int nb = unit_blocks[u];
    blocks += nb;
    cost += nb + c0;
  }
  long long tot_cost, tot_blocks;
  block_exclusive_scan(cost, &tot_cost, sh);
  block_exclusive_scan(blocks, &tot_blocks, sh);
  const long long T = tot_cost > 0 ? (tot_cost + P - 1) / P : 1;

  if (tid == 0) {
    md[0] = P;
    md[1] = (int32_t)T;
    md[2] = (int32_t)c0;
    md[3] = units;
    md[4] = (int32_t)tot_blocks;
    md[5] = kMagic;
    md[6] = 0;
    md[7] = 0;
    num_splits[0] = 0;
  }
  for (int p = tid; p < P; p += 1024) {
    int32_t* row = md + kHeader + kPartRow * p;
    row[0] = -1;
    row[1] = 0;
    row[2] = -1;
    row[3] = 0;
    row[4] = 0;
    row[5] = 0;
    row[6] = 0;
    row[7] = 0;
  }
  __threadfence_block();
  __syncthreads();

  // Pass 2: unit positions, split counts and the part rows.
  long long carry_c = 0, carry_k = 0;
  for (int base = 0; base < units; base += 1024) {
    const int u = base + tid;
    const bool live = u < units;
    const long long nb = live ? unit_blocks[u] : 0;
    const long long c = live ? nb + c0 : 0;
    long long chunk_c;
    const long long Cu = carry_c + block_exclusive_scan(c, &chunk_c, sh);
    long long f = 0, l = -1;
    if (live) {
      f = (Cu + c0) / T;
      l = (Cu + c0 + nb - 1) / T;
    }
    const long long k = live ? l - f + 1 : 0;
    long long chunk_k;
    const long long Ku = carry_k + block_exclusive_scan(k, &chunk_k, sh);
    if (live) {
      num_splits[u + 1] = (int32_t)(Ku + k);
      // Parts whose first unit is u: those of u's parts that the previous
      // unit (whose last block sits at position Cu - 1) does not reach.
      const long long lo = u > 0 ? max(f, (Cu - 1) / T + 1) : f;
      for (long long p = lo; p <= l; ++p) {
        int32_t* row = md + kHeader + kPartRow * p;
        row[0] = u;
        row[1] = (int32_t)(p == f ? 0 : p * T - Cu - c0);
        row[4] = (int32_t)(p - f);
      }
      // Parts whose last unit is u: those the next unit does not start in.
      const long long hi = (u + 1 < units) ? min(l, (Cu + c + c0) / T - 1) : l;
      for (long long p = f; p <= hi; ++p) {
        int32_t* row = md + kHeader + kPartRow * p;
        row[2] = u;
        row[3] = (int32_t)(p == l ? nb : (p + 1) * T - Cu - c0);
      }
    }
    carry_c += chunk_c;
    carry_k += chunk_k;
  }
}

hipError_t launch_unit_blocks(const int32_t* seqlens, const int32_t* indices, int batch, int s_q,
                              int topk, int units, int32_t* unit_blocks, hipStream_t stream) {
  (void)batch;
  if (units <= 0) return hipSuccess;
  const int grid = (units + 3) / 4;
  hipLaunchKernelGGL(unit_blocks_kernel, dim3(grid), dim3(256), 0, stream, seqlens, indices, s_q,
                     topk, units, unit_blocks);
  return hipGetLastError();
}

hipError_t launch_schedule(int units, int num_parts, int32_t* md, int32_t* num_splits,
                           hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, stream, units, num_parts, md,
                     num_splits);
  return hipGetLastError();
}

}  // namespace mla
