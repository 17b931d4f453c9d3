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
//    hi + mid + lo (each the top 16 bits of what the previous ones left, 24
//    significant bits in total), a bf16 x times a bf16 plane is exact in fp32,
//    and v_mfma_f32_16x16x32_bf16 accumulates the three products in fp32.  Each
//    wave streams 16 token rows straight from HBM into MFMA operands (no LDS).
//    Up to 16 experts, and 64 experts or more over many tokens, each wave splits the
//    fp32 weights it loads in registers (a mask, a subtraction, a mask, a subtraction
//    and a byte permute per pair); otherwise a first kernel writes the planes
//    ([3][E16][h], k-contiguous; small, they stay in L2), and with several expert
//    groups the workgroups on one XCD share a group, so its planes stay in that
//    XCD's L2.  Each wave keeps the loads of its next k-steps in flight while it
//    multiplies the current ones.  For fp32 activations a plain fp32 FMA kernel is
//    used instead.
//  * select.  G lanes per token (4 up to 64 experts, 8, 16 beyond), each lane
//    holding a contiguous chunk of E/G experts: softmax sums and k rounds of a 64-bit
//    group arg-max, exchanged between the G lanes with DPP and swizzles, pick the experts.
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

// w == hi + mid + lo exactly, each part a bf16 value: hi is w with its low 16 bits cleared
// (same sign and exponent, so w - hi is exact and holds the 16 low significand bits), mid
// is that remainder with its low 16 bits cleared, and lo = remainder - mid, exact and of at
// most 8 significant bits, so a bf16 too.  Returned as fp32 bit patterns with zero low halves.
__device__ __forceinline__ void split3(float w, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = __float_as_uint(w) & 0xFFFF0000u;
  const float r1 = w - __uint_as_float(hi);  // exact
  mid = __float_as_uint(r1) & 0xFFFF0000u;
  lo = __float_as_uint(r1 - __uint_as_float(mid));  // exact; low 16 bits zero
}

// the bf16 pair (lo16 = upper half of a, hi16 = upper half of b) in one v_perm_b32
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Row stride of the weight planes (elements): h + 32, so that consecutive expert rows start
// 64 bytes apart modulo 128.  A wave's 16-row fragment loads then fall half in each 64-byte
// half of their 128-byte lines instead of all in one (measured at T = 4096, h = 4096,
// E = 256: the logits 79 -> 64 us; 16- or 128-byte shifts gave 70 and 79 us).
__host__ __device__ __forceinline__ int plane_ld(int h) { return h + 32; }

// ---------------------------------------------------------------------------
// W_gate [h,E] fp32 -> planes [3][E16][h] bf16 with hi + mid + lo == W (to fp32 precision)
__global__ __launch_bounds__(256) void wsplit_kernel(const float* __restrict__ W_gate, int h, int E, int E16,
                                                     bf16_t* __restrict__ planes) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)E16 * h) return;
  const int e = (int)(idx / h), i = (int)(idx % h);
  const int64_t at = (int64_t)e * plane_ld(h) + i;
  const float w = e < E ? W_gate[(size_t)i * E + e] : 0.f;
  uint32_t hi, mid, lo;
  split3(w, hi, mid, lo);
  const size_t plane = (size_t)E16 * plane_ld(h);
  planes[at] = (bf16_t)(hi >> 16);
  planes[plane + at] = (bf16_t)(mid >> 16);
  planes[2 * plane + at] = (bf16_t)(lo >> 16);
}

// ---------------------------------------------------------------------------
// Lane exchanges and the per-token selection.

// v from lane (lane ^ O): quad permutes for O = 1, 2; ds_swizzle (bit mode, xor mask O) up to
// 16; every lane of the wave takes part
template <int O>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  static_assert(O == 1 || O == 2 || O == 4 || O == 8 || O == 16 || O == 32, "xor distance");
  if constexpr (O == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  else if constexpr (O == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  else if constexpr (O < 32) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (O << 10) | 0x1F);
  else return (uint32_t)__shfl_xor((int)v, O, kWave);
}
template <int O>
__device__ __forceinline__ float lane_xor_f(float v) { return __uint_as_float(lane_xor<O>(__float_as_uint(v))); }

// reductions over the aligned groups of G lanes, exchanges at distance 1, 2, ..., G/2 (each
// step combines the same two values on both lanes, so every lane ends with the same result)
template <int G, int O = 1>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (O < G) return group_max<G, 2 * O>(fmaxf(v, lane_xor_f<O>(v)));
  else return v;
}
template <int G, int O = 1>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (O < G) return group_sum<G, 2 * O>(v + lane_xor_f<O>(v));
  else return v;
}
template <int G, int O = 1>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
  if constexpr (O < G) {
    const uint64_t o = ((uint64_t)lane_xor<O>((uint32_t)(v >> 32)) << 32) | lane_xor<O>((uint32_t)v);
    return group_max_u64<G, 2 * O>(o > v ? o : v);
  } else {
    return v;
  }
}
// sum over the lanes that share lane % G (the token groups of a wave), distances G .. 32
template <int G, int O = G>
__device__ __forceinline__ float across_groups_sum(float v) {
  if constexpr (O < 64) return across_groups_sum<G, 2 * O>(v + lane_xor_f<O>(v));
  else return v;
}

// The selection for one token t: the G lanes of the token (lane gl holding experts gl*NV ..
// gl*NV + NV - 1 in v, -INF past E) compute the softmax sums and k rounds of the group
// arg-max, and write the token's topk_idx and topk_w (t < T); cnt (LDS, or null) counts the
// ids written, and psum gains the token's softmax (t < T).
template <int NV, int G>
__device__ __forceinline__ void select_token(const float (&v)[NV], int t, int T, int E, int k, int gl,
                                             float inv_temp, int vflags, int* __restrict__ topk_idx,
                                             float* __restrict__ topk_w, int* cnt, float (&psum)[NV]) {
  constexpr int KR = (16 + G - 1) / G;  // selections a lane stores (k <= 16)
  static_assert((NV & (NV - 1)) == 0, "experts per lane: a power of two");
  const int eb = gl * NV;
  const bool tv = t < T;
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV; ++i) m = fmaxf(m, v[i]);
  m = group_max<G>(m);
  float ex[NV], s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    ex[i] = eb + i < E ? expf((v[i] - m) * inv_temp) : 0.f;
    s += ex[i];
  }
  s = group_sum<G>(s);
  const float inv = 1.0f / s;
  if (tv) {
#pragma unroll
    for (int i = 0; i < NV; ++i) psum[i] += ex[i] * inv;
  }

  // The 64-bit keys (ordered logit bits, then ~e): unique, and the larger is selected first.
  // 0 stands for an expert past E and, once it is selected, for that expert (every real
  // key is above 0).  Built once; each round takes the largest and clears it.
  uint64_t key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i)
    key[i] = eb + i < E ? ((uint64_t)ordered_bits(v[i]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)(eb + i)) : 0;
  float lmax = 0.f, wsum = 0.f;
  float my_l[KR];
  int my_e[KR];
#pragma unroll
  for (int r = 0; r < KR; ++r) {
    my_l[r] = 0.f;
    my_e[r] = 0;
  }
  for (int j = 0; j < k; ++j) {
    // the lane's largest key, as a tree (independent compares)
    uint64_t mx[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) mx[i] = key[i];
#pragma unroll
    for (int w = NV / 2; w >= 1; w /= 2)
#pragma unroll
      for (int i = 0; i < w; ++i) mx[i] = mx[i + w] > mx[i] ? mx[i + w] : mx[i];
    const uint64_t best = group_max_u64<G>(mx[0]);
    const int e_sel = (int)(0xFFFFFFFFu - (uint32_t)best);
    const float l_sel = from_ordered((uint32_t)(best >> 32));
#pragma unroll
    for (int i = 0; i < NV; ++i)  // the low words (~e) tell the experts apart
      if ((uint32_t)key[i] == (uint32_t)best) key[i] = 0;
    if (j == 0) lmax = l_sel;
    wsum += expf((l_sel - lmax) * inv_temp);
#pragma unroll
    for (int r = 0; r < KR; ++r)
      if (j == gl + G * r) {
        my_l[r] = l_sel;
        my_e[r] = e_sel;
      }
  }
  if (tv) {
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int j = gl + G * r;
      if (j < k) {
        const int e_out = (vflags & 1) ? (int)(((int64_t)t * k + j) % E) : my_e[r];
        topk_idx[(size_t)t * k + j] = e_out;
        // lmax is the token's largest logit, m: the same value
        const float ew = expf((my_l[r] - lmax) * inv_temp);
        topk_w[(size_t)t * k + j] = (vflags & 2) ? ew * inv : ew / wsum;
        if (cnt != nullptr) atomicAdd(&cnt[e_out], 1);
      }
    }
  }
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
// One batch of a wave's operands: UU k-steps of x (TG groups of 16 tokens) and of the
// router weights (NB groups of 16 experts), as loaded: the three bf16 planes, or (WF32)
// eight fp32 k-values of the lane's expert column.
template <int UU, int TG, int NB, bool WF32>
struct LogitBatch {
  bf16x8 x[UU][TG];
  bf16x8 p[WF32 ? 1 : UU][WF32 ? 1 : NB][3];
  float w[WF32 ? UU : 1][WF32 ? NB : 1][8];
};

// The selection's outputs and variant arguments, for a logits kernel that also selects.
struct SelOut {
  int* topk_idx;
  float* topk_w;
  float* prob_part;   // [T / 16][E] or null
  int* blk_counts;    // [T / 16][E] or null
  const float* noise;
  float inv_temp;
  int vflags, k;
};

// EC > 0: E is EC (the fp32 weights' row stride then folds into the loads' offsets).
// SEL (one group of 16 tokens per workgroup, at most 16 experts): the workgroup then also
// selects its tokens' experts, as select_kernel does for 64, and writes its 16-token
// block's histogram and softmax sums (row blockIdx.x of so.blk_counts / so.prob_part).
template <int NB, int TW, int NW, int TG = 1, bool WF32 = false, int EC = 0, bool SEL = false>
__global__ __launch_bounds__(NW * 64) void logits_mfma_kernel(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ planes,
                                                          const float* __restrict__ W_gate,
                                                          const float* __restrict__ bias, int T, int h, int E,
                                                          int E16, float* __restrict__ logits, int gx, int gy,
                                                          SelOut so) {
  constexpr int KS = NW / TW;
  static_assert(!SEL || (NB == 1 && TW == 1 && TG == 1 && KS > 1), "selection: one 16 x 16 fragment");
  // k-steps of 32 per batch of loads; two batches are live (the next one is in flight while
  // this one is multiplied), so the batch shrinks as the fragments per step grow
  constexpr int FR = NB * TG;
  constexpr int UU = FR >= 4 ? 1 : (FR >= 2 ? 2 : (NW > 4 ? 2 : 4));
  using Batch = LogitBatch<UU, TG, NB, WF32>;
  __shared__ floatx4 red[KS > 1 ? KS : 1][TW][TG][NB][64];
  if (EC > 0) E = EC;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tw = wave % TW, ks = wave / TW;
  int bx = blockIdx.x, by = 0;
  if (gy > 1) {
    // gx token tiles x gy expert groups on a 1-D grid (a multiple of 8): workgroups are
    // dispatched round-robin over the 8 XCDs, and the ones on one XCD take consecutive
    // tiles of one expert group, so that group's weight planes stay in that XCD's L2
    const int n = gx * gy, per = (n + 7) >> 3;
    const int L = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (L >= n) return;
    by = L / gx;
    bx = L - by * gx;
  }
  const int t0 = bx * (16 * TW * TG) + tw * 16 * TG;
  const int e0 = by * (16 * NB);
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
    xrow[tg] = x + (size_t)(tvalid[tg] ? tok : 0) * h;
  }
  // lane group g = lane >> 4 takes k 8g .. 8g + 7 of each step of 32
  const int goff = 8 * (lane >> 4);
  auto step_k = [&](int st) { return kb + st * 32 + goff; };
  const size_t plane = (size_t)E16 * plane_ld(h);
  const bf16_t* wrow[NB];
  const float* wcol[NB];  // WF32: W_gate[0][e], clamped to expert E-1 past E (masked by wok)
  bool wok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int e = e0 + nb * 16 + (lane & 15);
    wok[nb] = e < E;
    if (WF32) wcol[nb] = W_gate + min(e, E - 1);
    else wrow[nb] = planes + (size_t)e * plane_ld(h);
  }

  // few fragments per step: one accumulator per plane, so no MFMA waits on the one before
  constexpr int PA = NB * TG >= 4 ? 1 : 3;
  floatx4 acc[TG][NB], accp[PA][TG][NB];
#pragma unroll
  for (int q = 0; q < PA; ++q)
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) accp[q][tg][nb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Loads of the batch at k0; every step is clamped to the wave's last one so that all
  // loads are unconditional (steps past ke re-read the last one and are not multiplied).
  const int nsteps = kspan / 32;
  auto load = [&](int k0, Batch& b) {
#pragma unroll
    for (int u = 0; u < UU; ++u) {
      const int kk = step_k(min((k0 - kb) / 32 + u, nsteps - 1));  // this lane's first k
      // (xrow points at a valid row for every lane; the invalid tokens' results are not stored)
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) b.x[u][tg] = *(const bf16x8*)(xrow[tg] + kk);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (WF32) {
#pragma unroll
          for (int j = 0; j < 8; ++j) b.w[u][nb][j] = wcol[nb][(size_t)(kk + j) * E];
        } else {
#pragma unroll
          for (int p = 0; p < 3; ++p) b.p[u][nb][p] = *(const bf16x8*)(wrow[nb] + p * plane + kk);
        }
      }
    }
  };
  // Per k-step: the weight fragments of every expert group first, then the MFMAs with the
  // plane outermost, so consecutive MFMAs update different accumulators (NB*TG of them)
  // rather than one accumulator three times in a row.
  auto multiply = [&](int steps, const Batch& b) {
#pragma unroll
    for (int u = 0; u < UU; ++u) {
      if (u < steps) {
        bf16x8 wp[NB][3];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          if constexpr (WF32) {
            uint32_t pk[3][4];
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
              uint32_t p0[3], p1[3];
              split3(wok[nb] ? b.w[u][nb][j] : 0.f, p0[0], p0[1], p0[2]);
              split3(wok[nb] ? b.w[u][nb][j + 1] : 0.f, p1[0], p1[1], p1[2]);
#pragma unroll
              for (int p = 0; p < 3; ++p) pk[p][j / 2] = pack_hi16(p0[p], p1[p]);
            }
#pragma unroll
            for (int p = 0; p < 3; ++p)
              wp[nb][p] = __builtin_bit_cast(bf16x8, u32x4{pk[p][0], pk[p][1], pk[p][2], pk[p][3]});
          } else {
#pragma unroll
            for (int p = 0; p < 3; ++p) wp[nb][p] = b.p[u][nb][p];
          }
        }
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int tg = 0; tg < TG; ++tg)
              accp[p % PA][tg][nb] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(wp[nb][p], b.x[u][tg], accp[p % PA][tg][nb], 0, 0, 0);
      }
    }
  };
  {
    // two batches in ping-pong: the loads of one are in flight while the other is multiplied
    Batch b0, b1;
    int k0 = kb;
    load(k0, b0);
    while (true) {
      load(k0 + 32 * UU, b1);
      multiply(min(UU, (ke - k0) / 32), b0);
      k0 += 32 * UU;
      if (k0 >= ke) break;
      load(k0 + 32 * UU, b0);
      multiply(min(UU, (ke - k0) / 32), b1);
      k0 += 32 * UU;
      if (k0 >= ke) break;
    }
  }
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      acc[tg][nb] = accp[0][tg][nb];
#pragma unroll
      for (int q = 1; q < PA; ++q) acc[tg][nb] += accp[q][tg][nb];
    }
  // the workgroup's logits for the selection: [token][expert], 17 words per row
  __shared__ float lsel[SEL ? 16 : 1][17];
  __shared__ int cnt[16];
  if (SEL && threadIdx.x < 16) cnt[threadIdx.x] = 0;
  // lane holds token (lane & 15) of each group, experts 4*(lane>>4) + 0..3 of each 16-block
  auto store = [&](int tg, int nb, const floatx4& v) {
    const int tok = t0 + 16 * tg + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = e0 + nb * 16 + 4 * (lane >> 4) + r;
      const float l = v[r] + (bias && e < E ? bias[e] : 0.f);
      if (SEL) lsel[lane & 15][4 * (lane >> 4) + r] = l;
      if (e < E && tok < T) logits[(size_t)tok * E + e] = l;
    }
  };
  if constexpr (KS > 1) {
    // every wave parks its partial sums; the TG*NB fragments of a token-wave are then
    // shared out over its KS k-waves, each adding the KS parts of its own in k order
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) red[ks][tw][tg][nb][lane] = acc[tg][nb];
    __syncthreads();
    for (int q = ks; q < TG * NB; q += KS) {
      const int tg = q / NB, nb = q - (q / NB) * NB;
      floatx4 v = red[0][tw][tg][nb][lane];
#pragma unroll
      for (int z = 1; z < KS; ++z) v += red[z][tw][tg][nb][lane];
      store(tg, nb, v);
    }
    if constexpr (SEL) {
      // Wave 0 selects for the 16 tokens, G = 4 lanes per token (lane = 4 * token + gl,
      // lane gl holding experts gl * NV .. gl * NV + NV - 1), with the selection kernel's
      // per-token function; the block's histogram is counted in LDS.
      constexpr int NV = EC > 0 && EC <= 8 ? 2 : 4;
      __syncthreads();
      if (wave == 0) {
        const int sub = lane >> 2, gl = lane & 3, t = t0 + sub;
        float v[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const int e = gl * NV + i;
          const float nz = so.noise != nullptr ? so.noise[(size_t)min(t, T - 1) * E + min(e, E - 1)] : 0.f;
          v[i] = e < E ? (t < T ? lsel[sub][e] + nz : 0.f) : -INFINITY;
        }
        float psum[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) psum[i] = 0.f;
        select_token<NV, 4>(v, t, T, E, so.k, gl, so.inv_temp, so.vflags, so.topk_idx, so.topk_w,
                            so.blk_counts != nullptr ? cnt : nullptr, psum);
        // the 16 token groups' softmax sums, added by a fixed tree; lanes 0..3 then hold them
#pragma unroll
        for (int i = 0; i < NV; ++i) psum[i] = across_groups_sum<4>(psum[i]);
        if (so.prob_part != nullptr && sub == 0) {
#pragma unroll
          for (int i = 0; i < NV; ++i)
            if (gl * NV + i < E) so.prob_part[(size_t)blockIdx.x * E + gl * NV + i] = psum[i];
        }
      }
      __syncthreads();
      if (so.blk_counts != nullptr && threadIdx.x < E) so.blk_counts[(size_t)blockIdx.x * E + threadIdx.x] = cnt[threadIdx.x];
    }
  } else {
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) store(tg, nb, acc[tg][nb]);
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
// selection: 64 tokens per workgroup of NWS waves.  All of a wave's logits are loaded
// before any is used: the kernel costs one memory round trip.
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
// Layout: G lanes per token (a power of two, at most 16), lane gl of a token holding the
// NV experts gl*NV .. gl*NV + NV - 1 (E <= G*NV), so the reductions over a token (max,
// sum, arg-max) take log2(G) lane exchanges (DPP within quads, swizzles beyond).

template <int NV, int G, bool HSPLIT, int NWS = 4, bool FUSE = false>
__global__ __launch_bounds__(NWS * 64) void select_kernel(float* __restrict__ logits, const float* __restrict__ lpart,
                                                     int SH, int T, int E, int k,
                                                     int* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                     float* __restrict__ prob_part, int* __restrict__ blk_counts,
                                                     const float* __restrict__ noise, float inv_temp, int vflags,
                                                     SmallPermute sp) {
  static_assert(G >= 1 && G <= 16 && (G & (G - 1)) == 0 && G * NV <= 256, "lanes per token");
  constexpr int TPW = 64 / G;                  // tokens per wave and pass
  constexpr int NQ = kSelTokens / NWS / TPW;   // passes per wave
  static_assert(NQ >= 1 && NWS * 64 >= 256, "tokens per wave; 256 threads for the histogram");
  __shared__ float pp[NWS][256];
  __shared__ int cnt[256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sub = lane / G, gl = lane % G;
  const int eb = gl * NV;  // this lane's first expert
  const int t0 = blockIdx.x * kSelTokens + w * (kSelTokens / NWS);
  if (tid < 256) cnt[tid] = 0;
  __syncthreads();

  // Every load is unconditional, at an index clamped into the arrays (token T-1, expert
  // E-1, part SH-1), so all of a wave's loads are in flight together; the values of
  // tokens, experts and parts past the ends are masked afterwards.  Rows whose lanes'
  // chunks all lie inside (E == G*NV) on 16-byte aligned arrays take 16-byte loads.
  const bool vec4 = NV % 4 == 0 && E == G * NV && ((uintptr_t)logits & 15) == 0 &&
                    ((uintptr_t)noise & 15) == 0;
  float v[NQ][NV];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int t = t0 + q * TPW + sub;
    const size_t row = (size_t)min(t, T - 1) * E;
    float l[NV], nz[NV];
    if (HSPLIT) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const size_t at = row + min(eb + i, E - 1);
        // SH <= 8 parts, added in ascending z
        float pz[8];
#pragma unroll
        for (int z = 0; z < 8; ++z) pz[z] = lpart[(size_t)min(z, SH - 1) * T * E + at];
        l[i] = 0.f;
#pragma unroll
        for (int z = 0; z < 8; ++z) l[i] += z < SH ? pz[z] : 0.f;
        nz[i] = noise != nullptr ? noise[at] : 0.f;
        if (eb + i < E && t < T) logits[at] = l[i];
      }
    } else if (vec4) {
#pragma unroll
      for (int i = 0; i < NV; i += 4) {
        const floatx4 lv = *(const floatx4*)(logits + row + eb + i);
        const floatx4 nv = noise != nullptr ? *(const floatx4*)(noise + row + eb + i) : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          l[i + j] = lv[j];
          nz[i + j] = nv[j];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const size_t at = row + min(eb + i, E - 1);
        l[i] = logits[at];
        nz[i] = noise != nullptr ? noise[at] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const bool ev = eb + i < E;
      v[q][i] = (ev && t < T) ? (noise != nullptr ? l[i] + nz[i] : l[i]) : (ev ? 0.f : -INFINITY);
    }
  }
  float psum[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) psum[i] = 0.f;

#pragma unroll
  for (int q = 0; q < NQ; ++q)
    select_token<NV, G>(v[q], t0 + q * TPW + sub, T, E, k, gl, inv_temp, vflags, topk_idx, topk_w,
                        blk_counts != nullptr ? cnt : nullptr, psum);
  // the token groups of a wave hold partial sums of the same experts: add them (fixed tree)
#pragma unroll
  for (int i = 0; i < NV; ++i) psum[i] = across_groups_sum<G>(psum[i]);
  if (prob_part != nullptr && sub == 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (eb + i < 256) pp[w][eb + i] = psum[i];
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

template <int NB, int TW, int NW = 4, int TG = 1, int EC = 0>
hipError_t launch_logits_mfma(const RouteArgs& a, int E16, hipStream_t st, int SH = 1, float* out = nullptr,
                              bool wf32 = false) {
  // every wave's share of the contraction is whole steps of 32 (else a wave would read
  // before its range)
  if (a.h % (32 * (NW / TW) * SH) != 0) return hipErrorInvalidValue;
  const int gx = (a.T + 16 * TW * TG - 1) / (16 * TW * TG), gy = E16 / (16 * NB);
  // one expert group: gx x SH grid; several: a 1-D grid, XCD-aware (SH is then 1)
  const dim3 grid = gy > 1 ? dim3((unsigned)((gx * gy + 7) / 8 * 8)) : dim3(gx, 1, SH);
  if (a.hist_tokens == 16) {
    // the selection in the same kernel: one 16-token group per workgroup, no split of h
    if constexpr (NB == 1 && TW == 1 && TG == 1 && NW / TW > 1) {
      if (E16 != 16 || SH != 1 || out != nullptr || a.logits_in || a.permute != nullptr) return hipErrorInvalidValue;
      const SelOut so{a.topk_idx, a.topk_w, a.prob_part, a.blk_counts, a.noise, a.inv_temp,
                      (a.uniform ? 1 : 0) | (a.soft ? 2 : 0), a.k};
      hipLaunchKernelGGL((logits_mfma_kernel<NB, TW, NW, TG, true, EC, true>), grid, dim3(NW * 64), 0, st,
                         (const bf16_t*)a.x, nullptr, a.W_gate, a.bias, a.T, a.h, a.E, E16, a.logits, gx, gy, so);
      return hipSuccess;
    }
    return hipErrorInvalidValue;
  }
  if (wf32 || E16 <= 16)  // weights split in registers (planes at 16 experts measured 22.8 + 4.4 us
                          // against 13.6 at T = 4096, h = 4096)
    hipLaunchKernelGGL((logits_mfma_kernel<NB, TW, NW, TG, true, EC>), grid, dim3(NW * 64), 0, st,
                       (const bf16_t*)a.x, nullptr, a.W_gate, a.bias, a.T, a.h, a.E, E16, out ? out : a.logits, gx,
                       gy, SelOut{});
  else
    hipLaunchKernelGGL((logits_mfma_kernel<NB, TW, NW, TG, false, 0>), grid, dim3(NW * 64), 0, st,
                       (const bf16_t*)a.x, (const bf16_t*)a.planes, nullptr, a.bias, a.T, a.h, a.E, E16,
                       out ? out : a.logits, gx, gy, SelOut{});
  return hipSuccess;
}

// 64 experts or more, many tokens: the kernel splits the fp32 weights itself (no planes
// kernel, and 4 bytes per weight read instead of 6).  Measured at T = 8192, h = 1024, E = 64:
// the logits 22.3 -> 17.8 us and the 4.4 us planes kernel gone; at T = 4096, h = 4096,
// E = 256: 63.7 -> 59.5 us and the 8.9 us planes kernel gone.
bool logits_wf32(int T, int h, int E16) {
  if (E16 > 64 && E16 % 64 == 0 && h % 128 == 0 && T >= 1024) return true;
  return E16 == 64 && h % 256 == 0 && T >= 1024;
}
}  // namespace

// the bf16 planes of the router weights (from 32 experts up; fewer are split in registers)
int route_planes_elems(int h, int E) {
  const int E16 = (E + 15) / 16 * 16;
  return E16 > 16 ? 3 * E16 * plane_ld(h) : 0;
}

int route_hsplit(int T, int h, int E, bool bf16) {
  // few tokens: too few workgroups to stream the router weights and x at full rate, so the
  // contraction over h is split across workgroups (partial logits added in the selection)
  const int E16 = (E + 15) / 16 * 16;
  if (!bf16 || E16 > 16) return 1;
  // (many tokens: none; a 2- or 4-way split with 32 or 64 tokens per workgroup measured
  // slower at T = 4096, h = 4096, E = 8)
  if (T > 1024) return 1;
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

// (At T = 4096, h = 4096, E = 8 the selection kernel took 4.3-4.9 us after a 13.8 us logits
// kernel.)
int route_hist_tokens(int T, int h, int E, bool bf16) {
  const int E16 = (E + 15) / 16 * 16;
  if (!bf16 || E16 != 16 || h % 512 != 0 || route_blocks(T) <= 1 || route_hsplit(T, h, E, bf16) != 1)
    return kSelTokens;
  const int nhb = (T + 15) / 16;
  return scan_scatter_fusable(nhb, nhb, E) ? 16 : kSelTokens;
}

int route_hist_blocks(int T, int h, int E, bool bf16) {
  const int ht = route_hist_tokens(T, h, E, bf16);
  return (T + ht - 1) / ht;
}

hipError_t launch_logits(const RouteArgs& a, hipStream_t st) {
  hipError_t err = hipSuccess;
  {
    if (a.bf16) {
      const int E16 = (a.E + 15) / 16 * 16;
      const int64_t n = (int64_t)E16 * a.h;
      const bool wf32 = logits_wf32(a.T, a.h, E16);
      if (E16 > 16 && !wf32)
        hipLaunchKernelGGL(wsplit_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.W_gate, a.h, a.E,
                           E16, (bf16_t*)a.planes);
      // k split across waves needs h/KS to be a multiple of 32
      const int SH = route_hsplit(a.T, a.h, a.E, true);
      if (SH > 1 && E16 <= 16) {
        err = launch_logits_mfma<1, 1>(a, E16, st, SH, route_lpart(a));
      } else if (E16 <= 16) {
        if (a.h % 512 == 0) {
          if (a.E == 8) err = launch_logits_mfma<1, 1, 16, 1, 8>(a, E16, st);
          else err = launch_logits_mfma<1, 1, 16>(a, E16, st);
        } else if (a.h % 128 == 0) {
          err = launch_logits_mfma<1, 1>(a, E16, st);
        } else {
          err = launch_logits_mfma<1, 2>(a, E16, st);
        }
      } else if (E16 == 32) {
        if (a.h % 128 == 0) err = launch_logits_mfma<2, 1>(a, E16, st);
        else err = launch_logits_mfma<2, 2>(a, E16, st);
      } else if (E16 % 64 == 0) {
        // Many tokens: each wave takes several 16-token groups, so the router weights are
        // read once per group of groups.  64 experts: 32 tokens per wave and an 8-way k
        // split, eight waves (more loads in flight; measured 36 -> 28 us at T = 8192,
        // h = 1024).  More experts: 64 tokens per wave (the weights, 4x larger, are then
        // read half as often; 8 waves of 32 tokens measured 94 -> 139 us at T = 4096,
        // h = 4096, E = 256), eight waves with an 8-way k split where h allows it, else
        // four with a 4-way split.  h / KS must be a multiple of 32.
        // (At T = 8192, h = 1024, E = 64 the eight waves of 32 tokens took 14.5 us; 16 waves
        // of 16 tokens 29.8, 32 experts per workgroup 15.6, 64 tokens per workgroup 19.6,
        // 16 tokens per workgroup 20.7, four waves 15.1.)
        if (E16 == 64 && a.h % 256 == 0 && a.T >= 1024) {
          if (a.E == 64) err = launch_logits_mfma<4, 1, 8, 2, 64>(a, E16, st, 1, nullptr, wf32);
          else err = launch_logits_mfma<4, 1, 8, 2>(a, E16, st, 1, nullptr, wf32);
        } else if (a.h % 256 == 0 && a.T >= 1024) {
          // eight waves, an 8-way k split (at T = 4096, h = 4096, E = 256: 58.2 us with four
          // waves and a 4-way split, 51.3 so; 16-token pairs per wave 72.7, 32 experts per
          // workgroup 65.9)
          err = launch_logits_mfma<4, 1, 8, 4>(a, E16, st, 1, nullptr, wf32);
        } else if (a.h % 128 == 0 && a.T >= 1024) {
          err = launch_logits_mfma<4, 1, 4, 4>(a, E16, st, 1, nullptr, wf32);
        } else {
          err = launch_logits_mfma<4, 4>(a, E16, st);
        }
      } else if (E16 % 32 == 0) {
        err = launch_logits_mfma<2, 4>(a, E16, st);
      } else {
        err = launch_logits_mfma<1, 4>(a, E16, st);
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
  if (err != hipSuccess) return err;
  return hipGetLastError();
}

hipError_t launch_select(const RouteArgs& a, hipStream_t st) {
  if (a.hist_tokens == 16) return a.logits_in ? hipErrorInvalidValue : hipSuccess;  // done by the logits kernel
  if (a.hist_tokens != kSelTokens) return hipErrorInvalidValue;
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
  // four lanes per token (sixteen tokens per wave) up to 32 experts, then 16, 8 and 16
  // lanes, one pass per wave
  if (a.E <= 4) { if (SH > 1) MOE_SELECT(1, 4, true); else MOE_SELECT(1, 4, false); }
  else if (a.E <= 8) { if (SH > 1) MOE_SELECT(2, 4, true); else MOE_SELECT(2, 4, false); }
  else if (a.E <= 16) { if (SH > 1) MOE_SELECT(4, 4, true); else MOE_SELECT(4, 4, false); }
  else if (a.E <= 32) MOE_SELECT(8, 4, false);
  else if (a.E <= 64) {
    // 16 lanes per token, 16 waves of 4 tokens (measured at T = 8192: 6.8 us with 4 lanes
    // per token and 4 waves of 16 tokens, 4.7 us so)
    MOE_SELECT_W(4, 16, false, 16);
  }
  else if (a.E <= 128) MOE_SELECT_W(16, 8, false, 8);
  // (T = 4096, E = 256: 36 us with 4 waves of 4 passes, 18.6 us with 16 waves of one)
  else MOE_SELECT_W(16, 16, false, 16);
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
