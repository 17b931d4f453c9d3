// Router: logits = x . W_gate (+ bias) in fp32, then softmax statistics,
// top-k selection and renormalised gate weights.
//
// Method: the router is one bias-free linear map followed by softmax and a
// top-k *selection*; the chosen k weights are rescaled to sum to one
// (ops-transformer MoE article, "原理" Steps 1-2 and the MoEGatingForward
// sketch; "MoE Router：谁来决定 Token 去哪个 Expert", MoERouter snippet).  The
// logits stay in fp32 (Colossal-AI MoE tutorial, SparseMLP data flow step 2).
//
// gfx950 design, two kernels:
//  * logits.  For bf16 activations the contraction runs on the matrix cores
//    at fp32 accuracy: W_gate (fp32) is split exactly into three bf16 planes
//    hi + mid + lo (each the bf16 rounding of what the previous ones left, 24
//    significant bits in total), a bf16 x times a bf16 plane is exact in fp32,
//    and v_mfma_f32_16x16x32_bf16 accumulates the three products in fp32.  Each
//    wave streams 16 token rows straight from HBM into MFMA operands (no LDS).
//    Up to 16 experts each wave splits the fp32 weights it loads in registers;
//    from 32 experts up (where that split would cost as much as the MFMAs) a
//    first kernel writes the planes ([3][E16][h], k-contiguous; small, they stay
//    in L2).  For fp32 activations a plain fp32 FMA kernel is used instead.
//  * select.  A group of lanes per token (a whole wave from 64 experts up): lane
//    e holds the logits of experts e, e+64, ...; softmax sums and k rounds of a
//    64-bit group arg-max pick the experts.
//    The key orders by logit (IEEE order, -0 == +0) then by the lower expert
//    index, so ties are deterministic.  The same kernel counts its block's
//    assignments per expert (the histogram) and sums the softmax per expert.
//    Inside the layer, when all tokens are one block (decode), it then also
//    does the permutation's scan and stable scatter (permute_dev.h), which saves
//    two launches.
#include "common.h"
#include "kernels.h"
#include "permute_dev.h"

namespace moe {

namespace {

__device__ __forceinline__ uint32_t ordered_bits(float l) {
  l = l + 0.0f;  // -0.0 -> +0.0
  uint32_t u = __float_as_uint(l);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o ^ 0x80000000u) : ~o;
  return __uint_as_float(u);
}

__device__ __forceinline__ float bf16_round(float v) { return __uint_as_float(f32_to_bf16_bits(v) << 16); }

// w == hi + mid + lo exactly (fp32 w: 24 significant bits, 8 per bf16 part), each part
// the bf16 rounding of what the previous parts leave
__device__ __forceinline__ void split3(float w, float& hi, float& mid, float& lo) {
  hi = bf16_round(w);
  const float r1 = w - hi;  // exact
  mid = bf16_round(r1);
  lo = bf16_round(r1 - mid);
}

// ---------------------------------------------------------------------------
// W_gate [h,E] fp32 -> planes [3][E16][h] bf16 with hi + mid + lo == W (to fp32 precision)
__global__ __launch_bounds__(256) void wsplit_kernel(const float* __restrict__ W_gate, int h, int E, int E16,
                                                     bf16_t* __restrict__ planes) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)E16 * h) return;
  const int e = (int)(idx / h), i = (int)(idx % h);
  const float w = e < E ? W_gate[(size_t)i * E + e] : 0.f;
  float hi, mid, lo;
  split3(w, hi, mid, lo);
  const size_t plane = (size_t)E16 * h;
  planes[idx] = (bf16_t)(__float_as_uint(hi) >> 16);
  planes[plane + idx] = (bf16_t)(__float_as_uint(mid) >> 16);
  planes[2 * plane + idx] = (bf16_t)(__float_as_uint(lo) >> 16);
}

// ---------------------------------------------------------------------------
// logits for bf16 x on MFMA.  Workgroup = NW waves = TW token-waves x KS k-splits;
// each wave: TG groups of 16 tokens x NB*16 experts over h/KS (the weight fragments
// loaded for one k-step serve all TG token groups).  Few experts: 16 waves split h 16
// ways, so each wave has a single batch of loads in flight and the kernel costs about
// one memory round trip.  Many experts: each wave takes 64 tokens, so the router
// weights are read once per 64 tokens instead of once per 16.
// With gridDim.z = SH > 1 (few tokens), workgroup z covers h / SH of the contraction and
// writes partial sums to logits + z * T * E (the selection kernel adds them).
// WF32: the weights come as W_gate itself ([h][E] fp32) and each lane splits the eight
// k-values of its expert column that it loads (exactly what the split kernel writes);
// otherwise they come as the bf16 planes.
template <int NB, int TW, int NW, int TG = 1, bool WF32 = false>
__global__ __launch_bounds__(NW * 64) void logits_mfma_kernel(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ planes,
                                                          const float* __restrict__ W_gate,
                                                          const float* __restrict__ bias, int T, int h, int E,
                                                          int E16, float* __restrict__ logits) {
  constexpr int KS = NW / TW;
  // k-steps of 32 per batch of loads (bounded by registers: 128 per lane at 16 waves)
  constexpr int U = NB >= 4 ? 2 : (NB == 2 ? 4 : (NW > 4 ? 4 : 8));
  __shared__ floatx4 red[KS > 1 ? KS - 1 : 1][TW][TG][NB][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tw = wave % TW, ks = wave / TW;
  const int t0 = blockIdx.x * (16 * TW * TG) + tw * 16 * TG;
  const int e0 = blockIdx.y * (16 * NB);
  const int kspan = h / (KS * gridDim.z);
  const int kb = (blockIdx.z * KS + ks) * kspan, ke = kb + kspan;
  if (gridDim.z > 1) {
    logits += (size_t)blockIdx.z * T * E;
    if (blockIdx.z > 0) bias = nullptr;
  }

  bool tvalid[TG];
  const bf16_t* xrow[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int tok = t0 + 16 * tg + (lane & 15);
    tvalid[tg] = tok < T;
    xrow[tg] = x + (size_t)(tvalid[tg] ? tok : 0) * h + 8 * (lane >> 4);
  }
  const size_t plane = (size_t)E16 * h;
  const bf16_t* wrow[NB];
  const float* wcol[NB];  // WF32: W_gate[8 * (lane >> 4)][e], clamped to expert E-1 past E (masked by wok)
  bool wok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int e = e0 + nb * 16 + (lane & 15);
    wok[nb] = e < E;
    if (WF32) wcol[nb] = W_gate + (size_t)(8 * (lane >> 4)) * E + min(e, E - 1);
    else wrow[nb] = planes + (size_t)e * h + 8 * (lane >> 4);
  }

  floatx4 acc[TG][NB];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[tg][nb] = floatx4{0.f, 0.f, 0.f, 0.f};

  constexpr int UU = TG > 1 ? 1 : U;
  for (int k0 = kb; k0 < ke; k0 += 32 * UU) {
    const int steps = min(UU, (ke - k0) / 32);
    bf16x8 xb[UU][TG], wa[UU][NB][3];
#pragma unroll
    for (int u = 0; u < UU; ++u) {
      if (u < steps) {
        const int kk = k0 + 32 * u;
        // (xrow points at a valid row for every lane; the invalid tokens' results are not stored)
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) xb[u][tg] = *(const bf16x8*)(xrow[tg] + kk);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          if (WF32) {
            float wv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) wv[j] = wcol[nb][(size_t)(kk + j) * E];
#pragma unroll
            for (int j = 0; j < 8; ++j) wv[j] = wok[nb] ? wv[j] : 0.f;
            uint32_t pk[3][4];
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
              float p0[3], p1[3];
              split3(wv[j], p0[0], p0[1], p0[2]);
              split3(wv[j + 1], p1[0], p1[1], p1[2]);
#pragma unroll
              for (int p = 0; p < 3; ++p)
                pk[p][j / 2] = (__float_as_uint(p0[p]) >> 16) | (__float_as_uint(p1[p]) & 0xFFFF0000u);
            }
#pragma unroll
            for (int p = 0; p < 3; ++p)
              wa[u][nb][p] = __builtin_bit_cast(bf16x8, u32x4{pk[p][0], pk[p][1], pk[p][2], pk[p][3]});
          } else {
#pragma unroll
            for (int p = 0; p < 3; ++p) wa[u][nb][p] = *(const bf16x8*)(wrow[nb] + p * plane + kk);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UU; ++u) {
      if (u < steps) {
#pragma unroll
        for (int tg = 0; tg < TG; ++tg)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int p = 0; p < 3; ++p)
              acc[tg][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[u][nb][p], xb[u][tg], acc[tg][nb], 0, 0, 0);
      }
    }
  }
  // lane holds token (lane & 15) of each group, experts 4*(lane>>4) + 0..3 of each 16-block
  if (KS > 1) {
    if (ks > 0) {
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) red[ks - 1][tw][tg][nb][lane] = acc[tg][nb];
    }
    __syncthreads();
    if (ks > 0) return;
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int s = 0; s < KS - 1; ++s) acc[tg][nb] += red[s][tw][tg][nb][lane];
  }
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    if (!tvalid[tg]) continue;
    const int tok = t0 + 16 * tg + (lane & 15);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = e0 + nb * 16 + 4 * (lane >> 4) + r;
        if (e < E) logits[(size_t)tok * E + e] = acc[tg][nb][r] + (bias ? bias[e] : 0.f);
      }
  }
}

// ---------------------------------------------------------------------------
// logits for fp32 x on the vector ALUs: 32 tokens x all experts per workgroup.
template <int EP>
__global__ __launch_bounds__(256) void logits_f32_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ W_gate,
                                                         const float* __restrict__ bias, int T, int h, int E,
                                                         float* __restrict__ logits) {
  constexpr int TT = 32, KC = 32;
  constexpr int TE = EP > 64 ? EP / 64 : 1;
  constexpr int NEG = EP / TE;
  constexpr int TM = TT * NEG / 256;
  __shared__ float xs[KC][TT];
  __shared__ float ws[KC][EP];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * TT;
  const int eg = tid % NEG, tg = tid / NEG;
  float acc[TM][TE];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TE; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < h; k0 += KC) {
    {
      const int tt = tid >> 3, kk = (tid & 7) * 4;
      const int t = t0 + tt;
      floatx4 v = floatx4{0.f, 0.f, 0.f, 0.f};
      if (t < T) v = *(const floatx4*)(x + (size_t)t * h + k0 + kk);
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[kk + i][tt] = v[i];
    }
    for (int idx = tid; idx < KC * EP; idx += 256) {
      const int kk = idx / EP, e = idx % EP;
      ws[kk][e] = e < E ? W_gate[(size_t)(k0 + kk) * E + e] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < KC; ++kk) {
      float xv[TM], wv[TE];
#pragma unroll
      for (int i = 0; i < TM; ++i) xv[i] = xs[kk][tg * TM + i];
#pragma unroll
      for (int j = 0; j < TE; ++j) wv[j] = ws[kk][eg * TE + j];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TE; ++j) acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int t = t0 + tg * TM + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < TE; ++j) {
      const int e = eg * TE + j;
      if (e < E) logits[(size_t)t * E + e] = acc[i][j] + (bias ? bias[e] : 0.f);
    }
  }
}

// ---------------------------------------------------------------------------
// selection: 64 tokens per workgroup, 16 per wave.  A token is handled by a group of G
// lanes (G = E rounded up to a power of two, at most 64; lane gl of the group holds
// experts gl, gl + 64, ...), so a wave works on 64/G tokens at once.  All of a wave's
// logits are loaded before any is used: the kernel costs one memory round trip.
// With SH > 1 the logits arrive as SH partial sums (lpart[z][t][e]); they are added in
// ascending z and the sums written to `logits`.
// Router variants: `noise` [T,E] (or null) is added to the logits before anything else
// uses them (the stored logits stay the router's own); the softmax and the weights use
// logits * inv_temp (selection ranks the logits themselves, the same order for any
// positive temperature); `vflags` bit 0 (uniform assignment): the ids written (and
// counted) are (t*k + j) % E while the weights stay those of the real top-k; bit 1
// (soft top-K): the weights are the full softmax at the selected experts, not
// renormalised over them.
// FUSE (T <= kSelTokens, one workgroup): the workgroup then also does the scan and the
// scatter (single_block_permute) into the outputs named by sp.
template <int NV, int G, bool HSPLIT, int NWS = 4, bool FUSE = false>
__global__ __launch_bounds__(NWS * 64) void select_kernel(float* __restrict__ logits, const float* __restrict__ lpart,
                                                     int SH, int T, int E, int k,
                                                     int* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                     float* __restrict__ prob_part, int* __restrict__ blk_counts,
                                                     const float* __restrict__ noise, float inv_temp, int vflags,
                                                     SmallPermute sp) {
  static_assert(G == 64 || NV == 1, "several values per lane only with whole-wave groups");
  constexpr int TPW = 64 / G;                  // tokens per wave and pass
  constexpr int NQ = kSelTokens / NWS / TPW;   // passes per wave
  static_assert(NQ >= 1, "tokens per wave");
  __shared__ float pp[NWS][64 * NV];
  __shared__ int cnt[256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sub = lane / G, gl = lane % G;
  const int t0 = blockIdx.x * kSelTokens + w * (kSelTokens / NWS);
  if (tid < 256) cnt[tid] = 0;
  __syncthreads();

  // Every load is unconditional, at an index clamped into the arrays (token T-1, expert
  // E-1, part SH-1), so all of a wave's loads are in flight together; the values of
  // tokens, experts and parts past the ends are masked afterwards.
  float v[NQ][NV];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int t = t0 + q * TPW + sub;
    const size_t tc = (size_t)min(t, T - 1);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = gl + 64 * i;
      const size_t at = tc * E + min(e, E - 1);
      float l = 0.f;
      if (HSPLIT) {
        // SH <= 8 parts, added in ascending z
        float pz[8];
#pragma unroll
        for (int z = 0; z < 8; ++z) pz[z] = lpart[(size_t)min(z, SH - 1) * T * E + at];
#pragma unroll
        for (int z = 0; z < 8; ++z) l += z < SH ? pz[z] : 0.f;
      } else {
        l = logits[at];
      }
      const float nz = noise != nullptr ? noise[at] : 0.f;
      if (HSPLIT && e < E && t < T) logits[at] = l;
      v[q][i] = (e < E && t < T) ? (noise != nullptr ? l + nz : l) : (e < E ? 0.f : -INFINITY);
    }
  }
  float psum[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) psum[i] = 0.f;

#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int t = t0 + q * TPW + sub;
    const bool tv = t < T;
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i) m = fmaxf(m, v[q][i]);
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    float ex[NV], s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      ex[i] = gl + 64 * i < E ? expf((v[q][i] - m) * inv_temp) : 0.f;
      s += ex[i];
    }
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
    const float inv = 1.0f / s;
    if (tv) {
#pragma unroll
      for (int i = 0; i < NV; ++i) psum[i] += ex[i] * inv;
    }

    bool taken[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) taken[i] = false;
    float lmax = 0.f, wsum = 0.f, my_l = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = gl + 64 * i;
        if (e < E && !taken[i]) {
          const uint64_t key = ((uint64_t)ordered_bits(v[q][i]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
          best = key > best ? key : best;
        }
      }
#pragma unroll
      for (int o = G / 2; o >= 1; o >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)best, o, kWave);
        const uint32_t hi = __shfl_xor((uint32_t)(best >> 32), o, kWave);
        const uint64_t b2 = ((uint64_t)hi << 32) | lo;
        best = b2 > best ? b2 : best;
      }
      const int e_sel = (int)(0xFFFFFFFFu - (uint32_t)best);
      const float l_sel = from_ordered((uint32_t)(best >> 32));
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (gl + 64 * i == e_sel) taken[i] = true;
      if (j == 0) lmax = l_sel;
      wsum += expf((l_sel - lmax) * inv_temp);
      if (gl == j) { my_l = l_sel; my_e = e_sel; }
    }
    if (tv && gl < k) {
      const int e_out = (vflags & 1) ? (int)(((int64_t)t * k + gl) % E) : my_e;
      topk_idx[(size_t)t * k + gl] = e_out;
      // lmax is the token's largest logit, m: the same value
      const float ew = expf((my_l - lmax) * inv_temp);
      topk_w[(size_t)t * k + gl] = (vflags & 2) ? ew * inv : ew / wsum;
      if (blk_counts != nullptr) atomicAdd(&cnt[e_out], 1);
    }
  }
  // the token groups of a wave hold partial sums of the same experts: add them (fixed tree)
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int o = G; o < 64; o <<= 1) psum[i] += __shfl_xor(psum[i], o, kWave);
  if (prob_part != nullptr && sub == 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) pp[w][gl + 64 * i] = psum[i];
  }
  __syncthreads();
  if (prob_part != nullptr)
    for (int e = tid; e < E; e += NWS * 64) {
      float sum = pp[0][e];
#pragma unroll
      for (int q = 1; q < NWS; ++q) sum += pp[q][e];
      prob_part[(size_t)blockIdx.x * E + e] = sum;
    }
  if (blk_counts != nullptr && tid < E) blk_counts[(size_t)blockIdx.x * E + tid] = cnt[tid];
  if (FUSE) {
    __shared__ float psum_sh[256];  // this block's softmax sums, as prob_part holds them
    for (int e = tid; e < E; e += NWS * 64) {
      float sum = pp[0][e];
#pragma unroll
      for (int q = 1; q < NWS; ++q) sum += pp[q][e];
      psum_sh[e] = sum;
    }
    __syncthreads();  // also makes this block's topk_idx visible to the whole workgroup
    single_block_permute(cnt, psum_sh, T, E, k, topk_idx, sp);
  }
}

// prob_sum[e] = sum over blocks of prob_part[b][e], in block order
__global__ void reduce_prob_kernel(const float* __restrict__ prob_part, int nblk, int E,
                                   float* __restrict__ prob_sum) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  float s = 0.f;
  for (int b = 0; b < nblk; ++b) s += prob_part[(size_t)b * E + e];
  prob_sum[e] = s;
}

template <int NB, int TW, int NW = 4, int TG = 1>
void launch_logits_mfma(const RouteArgs& a, int E16, hipStream_t st, int SH = 1, float* out = nullptr) {
  const dim3 grid((a.T + 16 * TW * TG - 1) / (16 * TW * TG), E16 / (16 * NB), SH);
  if constexpr (NB == 1) {
    if (E16 <= 16) {  // weights split in registers
      hipLaunchKernelGGL((logits_mfma_kernel<NB, TW, NW, TG, true>), grid, dim3(NW * 64), 0, st,
                         (const bf16_t*)a.x, nullptr, a.W_gate, a.bias, a.T, a.h, a.E, E16, out ? out : a.logits);
      return;
    }
  }
  hipLaunchKernelGGL((logits_mfma_kernel<NB, TW, NW, TG, false>), grid, dim3(NW * 64), 0, st, (const bf16_t*)a.x,
                     (const bf16_t*)a.planes, nullptr, a.bias, a.T, a.h, a.E, E16, out ? out : a.logits);
}

}  // namespace

// the bf16 planes of the router weights (from 32 experts up; fewer are split in registers)
int route_planes_elems(int h, int E) {
  const int E16 = (E + 15) / 16 * 16;
  return E16 > 16 ? 3 * E16 * h : 0;
}

int route_hsplit(int T, int h, int E, bool bf16) {
  // few tokens: too few workgroups to stream the router weights and x at full rate, so the
  // contraction over h is split across workgroups (partial logits added in the selection)
  const int E16 = (E + 15) / 16 * 16;
  if (!bf16 || E16 > 16 || T > 1024) return 1;
  const int nwg = (T + 15) / 16;
  int SH = 1;
  // (8-way at most: the selection adds the parts; measured best at T = 64, h = 4096)
  while (SH < 8 && nwg * SH * 2 <= 512 && h % (SH * 2 * 4 * 32) == 0) SH *= 2;
  return SH;
}

size_t route_scratch_bytes(int T, int h, int E, bool bf16) {
  if (!bf16) return 0;
  const size_t planes = ((size_t)route_planes_elems(h, E) * 2 + 255) / 256 * 256;
  const int SH = route_hsplit(T, h, E, bf16);
  return planes + (SH > 1 ? (size_t)SH * T * E * 4 : 0);
}

float* route_lpart(const RouteArgs& a) {
  const size_t planes = ((size_t)route_planes_elems(a.h, a.E) * 2 + 255) / 256 * 256;
  return (float*)((char*)a.planes + planes);
}

int route_blocks(int T) { return (T + kSelTokens - 1) / kSelTokens; }

hipError_t launch_logits(const RouteArgs& a, hipStream_t st) {
  {
    if (a.bf16) {
      const int E16 = (a.E + 15) / 16 * 16;
      const int64_t n = (int64_t)E16 * a.h;
      if (E16 > 16)
        hipLaunchKernelGGL(wsplit_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.W_gate, a.h, a.E,
                           E16, (bf16_t*)a.planes);
      // k split across waves needs h/KS to be a multiple of 32
      const int SH = route_hsplit(a.T, a.h, a.E, true);
      if (SH > 1) {
        launch_logits_mfma<1, 1>(a, E16, st, SH, route_lpart(a));
      } else if (E16 <= 16) {
        if (a.h % 512 == 0) launch_logits_mfma<1, 1, 16>(a, E16, st);
        else if (a.h % 128 == 0) launch_logits_mfma<1, 1>(a, E16, st);
        else launch_logits_mfma<1, 2>(a, E16, st);
      } else if (E16 == 32) {
        if (a.h % 128 == 0) launch_logits_mfma<2, 1>(a, E16, st);
        else launch_logits_mfma<2, 2>(a, E16, st);
      } else if (E16 % 64 == 0) {
        // Many tokens: each wave takes several 16-token groups, so the router weights are
        // read once per group of groups.  64 experts: 32 tokens per wave and an 8-way k
        // split, eight waves (more loads in flight; measured 36 -> 28 us at T = 8192,
        // h = 1024).  More experts: 64 tokens per wave and a 4-way k split (the weight
        // planes, 4x larger, are then read half as often; 8 waves of 32 tokens measured
        // 94 -> 139 us at T = 4096, h = 4096, E = 256).  h / KS must be a multiple of 32.
        if (E16 == 64 && a.h % 256 == 0 && a.T >= 1024) launch_logits_mfma<4, 1, 8, 2>(a, E16, st);
        else if (a.h % 128 == 0 && a.T >= 1024) launch_logits_mfma<4, 1, 4, 4>(a, E16, st);
        else launch_logits_mfma<4, 4>(a, E16, st);
      } else if (E16 % 32 == 0) {
        launch_logits_mfma<2, 4>(a, E16, st);
      } else {
        launch_logits_mfma<1, 4>(a, E16, st);
      }
    } else {
      const dim3 grid((a.T + 31) / 32);
      int p = 8;
      while (p < a.E) p <<= 1;
#define MOE_LOGITS_F32(EPV)                                                                                   \
  case EPV:                                                                                                   \
    hipLaunchKernelGGL(logits_f32_kernel<EPV>, grid, dim3(256), 0, st, (const float*)a.x, a.W_gate, a.bias, a.T, \
                       a.h, a.E, a.logits);                                                                   \
    break;
      switch (p) {
        MOE_LOGITS_F32(8)
        MOE_LOGITS_F32(16)
        MOE_LOGITS_F32(32)
        MOE_LOGITS_F32(64)
        MOE_LOGITS_F32(128)
        MOE_LOGITS_F32(256)
        default: return hipErrorInvalidValue;
      }
#undef MOE_LOGITS_F32
    }
  }
  return hipGetLastError();
}

hipError_t launch_select(const RouteArgs& a, hipStream_t st) {
  const dim3 grid(route_blocks(a.T));
  // partial logits from a split contraction (never with logits given as input)
  const int SH = a.logits_in ? 1 : route_hsplit(a.T, a.h, a.E, a.bf16);
  const float* lpart = SH > 1 ? route_lpart(a) : nullptr;
  const bool fuse = a.permute != nullptr;
  if (fuse && (route_blocks(a.T) != 1 || a.blk_counts == nullptr)) return hipErrorInvalidValue;
  const SmallPermute sp = fuse ? *a.permute : SmallPermute{};
#define MOE_SELECT_F(NV, G, HS, NWS, F)                                                                          \
  hipLaunchKernelGGL((select_kernel<NV, G, HS, NWS, F>), grid, dim3(NWS * 64), 0, st, a.logits, lpart, SH, a.T, \
                     a.E, a.k, a.topk_idx, a.topk_w, a.prob_part, a.blk_counts, a.noise, a.inv_temp,       \
                     (a.uniform ? 1 : 0) | (a.soft ? 2 : 0), sp)
#define MOE_SELECT_W(NV, G, HS, NWS)              \
  do {                                            \
    if (fuse) MOE_SELECT_F(NV, G, HS, NWS, true); \
    else MOE_SELECT_F(NV, G, HS, NWS, false);     \
  } while (0)
#define MOE_SELECT(NV, G, HS) MOE_SELECT_W(NV, G, HS, 4)
  if (SH > 1 && a.E > 16) return hipErrorInvalidValue;  // the h split is for few experts only
  if (a.E <= 4) { if (SH > 1) MOE_SELECT(1, 4, true); else MOE_SELECT(1, 4, false); }
  else if (a.E <= 8) { if (SH > 1) MOE_SELECT(1, 8, true); else MOE_SELECT(1, 8, false); }
  else if (a.E <= 16) { if (SH > 1) MOE_SELECT(1, 16, true); else MOE_SELECT(1, 16, false); }
  else if (a.E <= 32) MOE_SELECT(1, 32, false);
  // a whole wave per token: 16 waves, 4 tokens each, to keep enough selections in flight
  else if (a.E <= 64) MOE_SELECT_W(1, 64, false, 16);
  else if (a.E <= 128) MOE_SELECT_W(2, 64, false, 16);
  else MOE_SELECT_W(4, 64, false, 16);
#undef MOE_SELECT
#undef MOE_SELECT_W
#undef MOE_SELECT_F
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  if (!a.logits_in) {
    const hipError_t e = launch_logits(a, st);
    if (e != hipSuccess) return e;
  }
  return launch_select(a, st);
}

// Jitter of the router input: out = x * u elementwise, rounded to the storage dtype
// (bf16: the exact fp32 product rounded to nearest even).  8 elements per thread.
__global__ __launch_bounds__(256) void jitter_kernel(const u32x4* __restrict__ x, const u32x4* __restrict__ u,
                                                     int64_t n_vec, int bf16, u32x4* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_vec) return;
  const u32x4 a = x[i], b = u[i];
  u32x4 r;
  if (bf16) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float lo = __uint_as_float(a[c] << 16) * __uint_as_float(b[c] << 16);
      const float hi = __uint_as_float(a[c] & 0xFFFF0000u) * __uint_as_float(b[c] & 0xFFFF0000u);
      r[c] = pack_bf16x2(lo, hi);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) r[c] = __float_as_uint(__uint_as_float(a[c]) * __uint_as_float(b[c]));
  }
  out[i] = r;
}

hipError_t launch_jitter(const void* x, const void* u, int64_t n_elems, bool bf16, void* out, hipStream_t st) {
  const int64_t n_vec = n_elems * (bf16 ? 2 : 4) / 16;
  if (n_vec <= 0) return hipSuccess;
  hipLaunchKernelGGL(jitter_kernel, dim3((unsigned)((n_vec + 255) / 256)), dim3(256), 0, st, (const u32x4*)x,
                     (const u32x4*)u, n_vec, bf16 ? 1 : 0, (u32x4*)out);
  return hipGetLastError();
}

hipError_t launch_reduce_prob(const float* prob_part, int nblk, int E, float* prob_sum, hipStream_t st) {
  hipLaunchKernelGGL(reduce_prob_kernel, dim3((E + 255) / 256), dim3(256), 0, st, prob_part, nblk, E, prob_sum);
  return hipGetLastError();
}

}  // namespace moe
