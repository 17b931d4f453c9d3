// Token permutation: expert histogram, capacity + prefix sums, stable
// scatter (the sort of assignments by expert id), gather of token rows.
//
// Method (MegaBlocks chapter "01 · MoE 为什么难算：变长专家输入", sections 4.1,
// 4.2, 4.5, 4.6): the flattened expert ids (T*k of them) are sorted by expert
// id, counted per expert (tokens_per_expert) and turned into per-expert end
// positions by a running sum; with a capacity C an expert keeps its first C
// assignments and later ones are dropped (they add nothing to the output).
// C = floor(cf * T*k / E); a computed C of zero means "never drop".
//
// gfx950 design: no radix sort.  E <= 256 means one 8-bit digit, so a single
// *stable counting scatter* does the sort:
//   hist    : each block of 64 tokens (64*k consecutive assignments) counts its
//             experts in LDS (order-free atomics) -> blk_counts[b][e]; inside the
//             layer the router's selection kernel does this on the same blocks;
//   scan    : one workgroup of 1024 turns the counts into pre-drop ranks per block
//             (blk_base), kept counts, exclusive offsets, the GEMM m-tile
//             schedule and the aux loss (fixed summation order);
//   scatter : each block ranks its assignments in order with wave ballots
//             (a multisplit on the expert-id bits: lanes with the same expert
//             in lower lanes are counted by popcount), then across its 4 waves
//             and its rounds of 256 through LDS.  Rank = blk_base + in-block rank, so
//             the result equals a stable sort for any number of blocks.
// With a single block of tokens the layer's selection kernel runs the scan and the
// scatter itself (single_block_permute in permute_dev.h).
#include <limits.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "permute_dev.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void hist_kernel(const int* __restrict__ topk_idx, int T, int k, int E,
                                                   int* __restrict__ blk_counts) {
  __shared__ int cnt[256];
  const int tid = threadIdx.x;
  cnt[tid] = 0;
  __syncthreads();
  const int64_t n = (int64_t)T * k;
  const int pb = kSelTokens * k;
  const int64_t base = (int64_t)blockIdx.x * pb;
  for (int r = tid; r < pb; r += 256) {
    const int64_t s = base + r;
    if (s < n) {
      const int e = topk_idx[s];
      if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  if (tid < E) blk_counts[(size_t)blockIdx.x * E + tid] = cnt[tid];
}

// Inclusive Hillis-Steele scan of one value per thread over the first 256 threads of the
// workgroup (all threads of the workgroup must call it).
__device__ int block_inclusive_scan256(int v, int* sh) {
  const int tid = threadIdx.x;
  if (tid < 256) sh[tid] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    int add = 0;
    if (tid < 256 && tid >= o) add = sh[tid - o];
    __syncthreads();
    if (tid < 256) sh[tid] += add;
    __syncthreads();
  }
  int r = tid < 256 ? sh[tid] : 0;
  __syncthreads();
  return r;
}

constexpr int kScanThreads = 1024;

// One workgroup: per-(block, expert) rank origins, pre-drop counts, capacity-clamped
// offsets, the m-tile list and the aux loss.  Every sum has a fixed order (wave shuffles
// and LDS in index order), so the results do not vary from run to run.
__global__ __launch_bounds__(kScanThreads) void scan_kernel(ScanArgs a) {
  __shared__ int cnt_sh[256];
  __shared__ int wsum[2][4];
  __shared__ double dterm[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E;
  int ep = 1;
  while (ep < E) ep <<= 1;
  // Per-expert running ranks over the blocks: P consecutive lanes of one wave per expert;
  // each owns a contiguous range of blocks, sums it (independent loads, kept in registers
  // when the range is short), the lanes scan their sums, then each writes its range's
  // exclusive ranks.
  {
    constexpr int kCache = 16;
    const int P = min(64, kScanThreads / ep);
    const int e = tid / P, part = tid % P;
    const bool act = e < E;
    const int per = (a.nhb + P - 1) / P;
    const int b0 = min(part * per, a.nhb), b1 = min(b0 + per, a.nhb);
    int c[kCache];
    int sum = 0;
    if (act) {
      if (per <= kCache) {
#pragma unroll
        for (int i = 0; i < kCache; ++i) c[i] = b0 + i < b1 ? a.blk_counts[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
        for (int i = 0; i < kCache; ++i) sum += c[i];
      } else {
        for (int b = b0; b < b1; ++b) sum += a.blk_counts[(size_t)b * E + e];
      }
    }
    const int incl = wave_incl_scan(sum, lane, P);
    int pre = incl - sum;
    if (act) {
      if (part == P - 1) cnt_sh[e] = incl;
      if (per <= kCache) {
#pragma unroll
        for (int i = 0; i < kCache; ++i)
          if (b0 + i < b1) {
            a.blk_base[(size_t)(b0 + i) * E + e] = pre;
            pre += c[i];
          }
      } else {
        for (int b = b0; b < b1; ++b) {
          const int v = a.blk_counts[(size_t)b * E + e];
          a.blk_base[(size_t)b * E + e] = pre;
          pre += v;
        }
      }
    }
  }
  __syncthreads();
  // kept counts -> offsets, m-tiles -> tile list: exclusive scans over the experts (4 waves)
  const int cnt = tid < E ? cnt_sh[tid] : 0;
  int kept = tid < E ? min(cnt, a.C) : 0;
  if (a.binned) {
    // fixed buckets: C rows each (the largest count when no capacity is given)
    __shared__ int cmax_sh;
    if (tid == 0) cmax_sh = 0;
    __syncthreads();
    if (tid < E) atomicMax(&cmax_sh, cnt);
    __syncthreads();
    const int cb = a.C == INT_MAX ? cmax_sh : a.C;
    kept = tid < E ? cb : 0;
    if (tid == 0 && a.cap_out != nullptr) *a.cap_out = cb;
  }
  const int mt = (tid < E && a.BM > 0) ? m_tile_count(kept, a.BM, a.big) : 0;
  int ik = wave_incl_scan(kept, lane, 64), im = wave_incl_scan(mt, lane, 64);
  if (wave < 4 && lane == 63) {
    wsum[0][wave] = ik;
    wsum[1][wave] = im;
  }
  __syncthreads();
  if (tid < 256) {
    for (int w = 0; w < wave; ++w) {
      ik += wsum[0][w];
      im += wsum[1][w];
    }
  }
  if (tid < E) {
    a.counts[tid] = cnt;
    a.offsets[tid] = ik - kept;
    if (tid == E - 1) a.offsets[E] = ik;
    if (a.BM > 0 && a.tile_off != nullptr) {
      a.tile_off[tid] = im - mt;
      if (tid == E - 1) a.tile_off[E] = im;
    }
  }
  if (a.aux != nullptr && (a.prob_part != nullptr || a.prob_sum != nullptr)) {
    // sum_t p[t,e]: few experts -- a wave per expert, lanes stride the blocks; many experts --
    // P = 1024/ep threads per expert stride the blocks, then a fixed tree over the P sums
    const double n = (double)a.T * (double)a.k;
    if (E <= 16) {
      for (int e = wave; e < E; e += kScanThreads / 64) {
        double ps = 0.0;
        if (a.prob_part != nullptr) {
          for (int b = lane; b < a.nrb; b += 64) ps += (double)a.prob_part[(size_t)b * E + e];
        } else if (lane == 0) {
          ps = (double)a.prob_sum[e];
        }
        ps = wave_sum_f64(ps);
        if (lane == 0) dterm[e] = ((double)cnt_sh[e] / n) * (ps / (double)a.T);
      }
    } else {
      __shared__ double dsh[kScanThreads];
      const int P = kScanThreads / ep;
      const int e = tid % ep, part = tid / ep;
      double ps = 0.0;
      if (e < E) {
        if (a.prob_part != nullptr) {
          for (int b = part; b < a.nrb; b += P) ps += (double)a.prob_part[(size_t)b * E + e];
        } else if (part == 0) {
          ps = (double)a.prob_sum[e];
        }
      }
      dsh[tid] = ps;
      __syncthreads();
      for (int o = P / 2; o >= 1; o >>= 1) {
        if (part < o) dsh[tid] += dsh[tid + o * ep];
        __syncthreads();
      }
      if (tid < E) dterm[tid] = ((double)cnt_sh[tid] / n) * (dsh[tid] / (double)a.T);
    }
    __syncthreads();
    if (wave == 0) {
      double t = 0.0;
      for (int e = lane; e < E; e += 64) t += dterm[e];
      t = wave_sum_f64(t);
      if (lane == 0) *a.aux = (float)((double)E * t);
    }
  }
}

// The scan and the scatter in one launch (one workgroup of 256 per kSelTokens-token block),
// for when every block can afford to read all the block histograms: block b sums each
// expert's column of blk_counts over all histogram blocks (the counts) and over those of
// the tokens before its own (its rank origins; hpb histogram blocks per token block when
// the histogram was counted per fewer tokens), P threads per expert, each over a contiguous range of at most PER blocks with
// all its loads in flight at once.  Every block then has the same counts, so the same
// offsets; block 0 also writes counts, offsets, the m-tile list and the aux loss.  Integer
// sums are exact, and the aux loss is summed in a fixed order, so the results are those of
// the separate scan and scatter kernels (the aux loss up to the order of its fp64 sum).
template <int PER>
__global__ __launch_bounds__(256) void scan_scatter_kernel(ScanArgs a, const int* __restrict__ topk_idx, int nbits,
                                                           int* __restrict__ slot_pos, int* __restrict__ sorted_slot,
                                                           int* __restrict__ perm_token) {
  __shared__ int cnt_sh[256], base_sh[256], off_sh[256];
  __shared__ int wsum[2][4];
  __shared__ double dterm[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, blk = blockIdx.x;
  int ep = 1;
  while (ep < E) ep <<= 1;
  const int P = min(64, 256 / ep);  // threads per expert (a power of two dividing 64)
  const int e = tid / P, part = tid % P;
  const bool act = e < E;
  const int ec = min(e, E - 1);
  const int per = (a.nhb + P - 1) / P;  // <= PER (checked by the launcher)
  const int b0 = part * per;
  int tot = 0, pre = 0;
  {
    int c[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) c[i] = a.blk_counts[(size_t)min(b0 + i, a.nhb - 1) * E + ec];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int bi = b0 + i;
      const int v = (act && i < per && bi < a.nhb) ? c[i] : 0;
      tot += v;
      pre += bi < blk * a.hpb ? v : 0;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    if (o < P) {
      tot += __shfl_xor(tot, o, kWave);
      pre += __shfl_xor(pre, o, kWave);
    }
  }
  if (act && part == 0) {
    cnt_sh[e] = tot;
    base_sh[e] = pre;
  }
  __syncthreads();
  // kept counts -> offsets, m-tiles -> tile list: exclusive scans over the experts (4 waves)
  const int cnt = tid < E ? cnt_sh[tid] : 0;
  const int kept = tid < E ? min(cnt, a.C) : 0;
  const int mt = (tid < E && a.BM > 0) ? m_tile_count(kept, a.BM, a.big) : 0;
  int ik = wave_incl_scan(kept, lane, 64), im = wave_incl_scan(mt, lane, 64);
  if (lane == 63) {
    wsum[0][wave] = ik;
    wsum[1][wave] = im;
  }
  __syncthreads();
  for (int w = 0; w < wave; ++w) {
    ik += wsum[0][w];
    im += wsum[1][w];
  }
  if (tid < E) off_sh[tid] = ik - kept;
  if (blk == 0 && tid < E) {
    a.counts[tid] = cnt;
    a.offsets[tid] = ik - kept;
    if (tid == E - 1) a.offsets[E] = ik;
    if (a.BM > 0 && a.tile_off != nullptr) {
      a.tile_off[tid] = im - mt;
      if (tid == E - 1) a.tile_off[E] = im;
    }
  }
  if (blk == 0 && a.aux != nullptr && (a.prob_part != nullptr || a.prob_sum != nullptr)) {
    // sum_t p[t,e] in fp64: the same P-thread ranges over the blocks' softmax sums, then a
    // butterfly over the parts (each step adds the same two values on both lanes, so every
    // lane of a group holds the same sum)
    double ps = 0.0;
    if (a.prob_part != nullptr) {
      float q[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) q[i] = a.prob_part[(size_t)min(b0 + i, a.nrb - 1) * E + ec];
#pragma unroll
      for (int i = 0; i < PER; ++i) ps += (act && i < per && b0 + i < a.nrb) ? (double)q[i] : 0.0;
    } else if (act && part == 0) {
      ps = (double)a.prob_sum[e];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
      if (o < P) ps += __shfl_xor(ps, o, kWave);
    const double n = (double)a.T * (double)a.k;
    if (act && part == 0) dterm[e] = ((double)cnt_sh[e] / n) * (ps / (double)a.T);
    __syncthreads();
    if (wave == 0) {
      double t = 0.0;
      for (int x = lane; x < E; x += 64) t += dterm[x];
      t = wave_sum_f64(t);
      if (lane == 0) *a.aux = (float)((double)E * t);
    }
  }
  __syncthreads();
  scatter_block(blk, topk_idx, a.T, E, a.k, nbits, a.C, off_sh, base_sh, slot_pos, sorted_slot, perm_token);
}

__global__ __launch_bounds__(256) void tiles_kernel(const int* __restrict__ offsets, int E, int BM, int big,
                                                    int* __restrict__ tile_off) {
  __shared__ int sh[256];
  const int tid = threadIdx.x;
  const int rows = tid < E ? offsets[tid + 1] - offsets[tid] : 0;
  const int mt = tid < E ? m_tile_count(rows, BM, big) : 0;
  const int incl = block_inclusive_scan256(mt, sh);
  if (tid < E) {
    tile_off[tid] = incl - mt;
    if (tid == E - 1) tile_off[E] = incl;
  }
}

__global__ __launch_bounds__(256) void scatter_kernel(const int* __restrict__ topk_idx, int T, int E,
                                                      int k, int nbits, int C,
                                                      const int* __restrict__ offsets,
                                                      const int* __restrict__ blk_base,
                                                      int* __restrict__ slot_pos,
                                                      int* __restrict__ sorted_slot,
                                                      int* __restrict__ perm_token) {
  scatter_block(blockIdx.x, topk_idx, T, E, k, nbits, C, offsets, blk_base + (size_t)blockIdx.x * E, slot_pos,
                sorted_slot, perm_token);
}

// x_perm[r] = x[perm_token[r]] for r < offsets[E]; one workgroup per row.
__global__ __launch_bounds__(256) void gather_kernel(const u32x4* __restrict__ x,
                                                     const int* __restrict__ perm_token,
                                                     const int* __restrict__ offsets, int E,
                                                     int vec_per_row, u32x4* __restrict__ x_perm) {
  const int r = blockIdx.x;
  if (r >= offsets[E]) return;
  const size_t src = (size_t)perm_token[r] * vec_per_row;
  const size_t dst = (size_t)r * vec_per_row;
  for (int i = threadIdx.x; i < vec_per_row; i += 256) x_perm[dst + i] = x[src + i];
}

// Fixed-capacity buckets: one workgroup per bucket row; filled rows copy their token's
// row of x, the others are zero ([MB] section 4.5: slots past an expert's count stay zero).
__global__ __launch_bounds__(256) void binned_gather_kernel(const u32x4* __restrict__ x,
                                                            const int* __restrict__ perm_token,
                                                            const int* __restrict__ offsets,
                                                            const int* __restrict__ counts, int E,
                                                            int vec_per_row, u32x4* __restrict__ x_bins) {
  const int r = blockIdx.x;
  if (r >= offsets[E]) return;
  const int C = offsets[1] - offsets[0];
  const int e = r / C, i = r - e * C;
  const size_t dst = (size_t)r * vec_per_row;
  if (i < min(counts[e], C)) {
    const size_t src = (size_t)perm_token[r] * vec_per_row;
    for (int v = threadIdx.x; v < vec_per_row; v += 256) x_bins[dst + v] = x[src + v];
  } else {
    for (int v = threadIdx.x; v < vec_per_row; v += 256) x_bins[dst + v] = u32x4{0u, 0u, 0u, 0u};
  }
}

}  // namespace

hipError_t launch_binned_gather(const void* x, const int* perm_token, const int* offsets, const int* counts, int E,
                                int R_max, int h, int elem_bytes, void* x_bins, hipStream_t st) {
  if (R_max <= 0) return hipSuccess;
  const int vec = h * elem_bytes / 16;
  hipLaunchKernelGGL(binned_gather_kernel, dim3(R_max), dim3(256), 0, st, (const u32x4*)x, perm_token, offsets,
                     counts, E, vec, (u32x4*)x_bins);
  return hipGetLastError();
}

hipError_t launch_hist(const int* topk_idx, int T, int k, int E, int* blk_counts, hipStream_t st) {
  hipLaunchKernelGGL(hist_kernel, dim3(route_blocks(T)), dim3(256), 0, st, topk_idx, T, k, E, blk_counts);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, st, a);
  return hipGetLastError();
}

namespace {
// blocks each thread of the fused scan + scatter sums (P threads per expert), 0 = not fusable
int scan_scatter_per(int nhb, int nrb, int E) {
  if (E <= 0 || E > 256 || nrb > nhb) return 0;
  int ep = 1;
  while (ep < E) ep <<= 1;
  const int P = std::min(64, 256 / ep);
  const int per = (nhb + P - 1) / P;
  return per <= 64 ? per : 0;
}
}  // namespace

bool scan_scatter_fusable(int nhb, int nrb, int E) { return scan_scatter_per(nhb, nrb, E) > 0; }

hipError_t launch_scan_scatter(const ScanArgs& a, const int* topk_idx, int* slot_pos, int* sorted_slot,
                               int* perm_token, hipStream_t st) {
  const int per = scan_scatter_per(a.nhb, a.prob_part != nullptr ? a.nrb : 0, a.E);
  if (per == 0 || a.binned) return hipErrorInvalidValue;
  const int nbits = expert_bits(a.E);
  if (a.hpb < 1 || (size_t)route_blocks(a.T) * a.hpb < (size_t)a.nhb) return hipErrorInvalidValue;
  const dim3 grid(route_blocks(a.T)), block(256);  // one workgroup per scatter block
#define MOE_SCAN_SCATTER(PER_)                                                                                    \
  hipLaunchKernelGGL(scan_scatter_kernel<PER_>, grid, block, 0, st, a, topk_idx, nbits, slot_pos, sorted_slot, \
                     perm_token)
  if (per <= 1) MOE_SCAN_SCATTER(1);
  else if (per <= 2) MOE_SCAN_SCATTER(2);
  else if (per <= 4) MOE_SCAN_SCATTER(4);
  else if (per <= 8) MOE_SCAN_SCATTER(8);
  else if (per <= 16) MOE_SCAN_SCATTER(16);
  else if (per <= 32) MOE_SCAN_SCATTER(32);
  else MOE_SCAN_SCATTER(64);
#undef MOE_SCAN_SCATTER
  return hipGetLastError();
}

hipError_t launch_tiles(const int* offsets, int E, int BM, int big, int* tile_off, hipStream_t st) {
  hipLaunchKernelGGL(tiles_kernel, dim3(1), dim3(256), 0, st, offsets, E, BM, big, tile_off);
  return hipGetLastError();
}

hipError_t launch_scatter(const int* topk_idx, int T, int E, int k, int C, const int* offsets,
                          const int* blk_base, int* slot_pos, int* sorted_slot, int* perm_token,
                          hipStream_t st) {
  const int nbits = expert_bits(E);
  hipLaunchKernelGGL(scatter_kernel, dim3(route_blocks(T)), dim3(256), 0, st, topk_idx, T, E, k, nbits, C,
                     offsets, blk_base, slot_pos, sorted_slot, perm_token);
  return hipGetLastError();
}

hipError_t launch_gather(const void* x, const int* perm_token, const int* offsets, int E, int R_max,
                         int h, int elem_bytes, void* x_perm, hipStream_t st) {
  if (R_max <= 0) return hipSuccess;
  const int vec = h * elem_bytes / 16;
  hipLaunchKernelGGL(gather_kernel, dim3(R_max), dim3(256), 0, st, (const u32x4*)x, perm_token, offsets,
                     E, vec, (u32x4*)x_perm);
  return hipGetLastError();
}

}  // namespace moe
