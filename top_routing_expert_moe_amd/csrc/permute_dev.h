// Device code shared by the permutation kernels and the router's selection kernel: wave
// scans and sums in a fixed order, the stable scatter of one token block, and the scan +
// scatter of a layer whose tokens fit one block (the selection kernel runs them itself).
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

__device__ __forceinline__ int wave_incl_scan(int v, int lane, int width) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, kWave);
    if (o < width && (lane % width) >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// The stable scatter of token block `blk` (assignments blk * pb .. blk * pb + pb - 1, pb =
// kSelTokens * k), by the first 256 threads of the workgroup; every thread of the workgroup
// reaches the barriers.  bb[e]: the rank origin of expert e's assignments in this block
// (null: zero, the first block); offsets may point to LDS.
__device__ __forceinline__ void scatter_block(int blk, const int* __restrict__ topk_idx, int T, int E, int k,
                                              int nbits, int C, const int* offsets, const int* __restrict__ bb,
                                              int* __restrict__ slot_pos, int* __restrict__ sorted_slot,
                                              int* __restrict__ perm_token) {
  __shared__ int run[256];
  __shared__ int wcnt[4][256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool act = tid < 256;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  if (act) run[tid] = 0;
  const int64_t n = (int64_t)T * k;
  const int pb = kSelTokens * k;
  const int64_t base = (int64_t)blk * pb;
  for (int r0 = 0; r0 < pb; r0 += 256) {
    if (act) {
      wcnt[0][tid] = 0;
      wcnt[1][tid] = 0;
      wcnt[2][tid] = 0;
      wcnt[3][tid] = 0;
    }
    __syncthreads();
    const int64_t s = base + r0 + tid;
    const bool in = act && (r0 + tid < pb) && s < n;
    int e = -1;
    if (in) e = topk_idx[s];
    const bool valid = (unsigned)e < (unsigned)E;
    int rank_w = 0;
    if (act) {  // whole waves: the ballots see only this block's lanes
      uint64_t match = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool on = valid && ((e >> bit) & 1);
        const uint64_t b = __ballot(on);
        match &= on ? b : ~b;
      }
      rank_w = __popcll(match & lt_mask);
      if (valid && rank_w == 0) wcnt[w][e] = __popcll(match);
    }
    __syncthreads();
    if (valid) {
      int pre = run[e];
      for (int q = 0; q < w; ++q) pre += wcnt[q][e];
      const int g = (bb != nullptr ? bb[e] : 0) + pre + rank_w;  // rank among all earlier assignments to e
      if (g < C) {
        const int row = offsets[e] + g;
        slot_pos[s] = row;
        sorted_slot[row] = (int)s;
        perm_token[row] = (int)(s / k);
      } else {
        slot_pos[s] = -1;
      }
    } else if (in) {
      slot_pos[s] = -1;
    }
    __syncthreads();
    if (act) run[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
    __syncthreads();
  }
}

// Counts, kept counts, offsets, the m-tile list, the aux loss and the stable scatter for a
// layer whose T <= kSelTokens tokens are one block, by the whole workgroup (at least 256
// threads; every thread calls this).  cnt: the block's pre-drop histogram, psum: its
// per-expert softmax sums (both in LDS, complete).  The same arithmetic as the scan and
// scatter kernels on one block, so the results are those of the separate kernels.
__device__ __forceinline__ void single_block_permute(const int* cnt, const float* psum, int T, int E, int k,
                                                     const int* __restrict__ topk_idx, const SmallPermute& sp) {
  __shared__ int wsum[2][4];
  __shared__ int off_sh[256];
  __shared__ double dterm[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid < E ? cnt[tid] : 0;
  const int kept = tid < E ? min(c, sp.C) : 0;
  const int mt = (tid < E && sp.BM > 0) ? m_tile_count(kept, sp.BM, sp.big) : 0;
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
  const double n = (double)T * (double)k;
  if (tid < E) {
    sp.counts[tid] = c;
    sp.offsets[tid] = ik - kept;
    off_sh[tid] = ik - kept;
    if (tid == E - 1) sp.offsets[E] = ik;
    if (sp.BM > 0 && sp.tile_off != nullptr) {
      sp.tile_off[tid] = im - mt;
      if (tid == E - 1) sp.tile_off[E] = im;
    }
    dterm[tid] = ((double)c / n) * ((double)psum[tid] / (double)T);
  }
  __syncthreads();
  if (sp.aux != nullptr && wave == 0) {
    double t = 0.0;
    for (int e = lane; e < E; e += 64) t += dterm[e];
    t = wave_sum_f64(t);
    if (lane == 0) *sp.aux = (float)((double)E * t);
  }
  scatter_block(0, topk_idx, T, E, k, sp.nbits, sp.C, off_sh, nullptr, sp.slot_pos, sp.sorted_slot, sp.perm_token);
}

}  // namespace moe
