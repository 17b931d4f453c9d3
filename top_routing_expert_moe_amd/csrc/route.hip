// Router: logits = x . W_gate (+ bias) in fp32, fused softmax statistics,
// top-k selection and renormalised gate weights.
//
// Method: the router is one bias-free linear map followed by softmax and a
// top-k *selection*; the chosen k weights are rescaled to sum to one
// (ops-transformer MoE article, "原理" Steps 1-2 and the MoEGatingForward
// sketch; "MoE Router：谁来决定 Token 去哪个 Expert", MoERouter snippet).  The
// logits stay in fp32 (Colossal-AI MoE tutorial, SparseMLP data flow step 2).
//
// Layout: one workgroup of 256 threads owns TT=32 tokens and all E experts.
// The h-loop stages a 32-wide slice of x (converted to fp32, stored k-major so
// that a thread's token values are one broadcast read) and of W_gate in LDS;
// each thread accumulates a TM x TE register tile.  Then each wave takes 8
// tokens: lane e holds the logits of experts e, e+64, ...; softmax sums and k
// rounds of a 64-bit wave arg-max select the experts.  The key orders by
// logit (IEEE order, -0 == +0) then by lower expert index, so ties are broken
// deterministically.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int TT = 32;   // tokens per workgroup
constexpr int KC = 32;   // h-chunk staged per iteration

__device__ __forceinline__ uint32_t ordered_bits(float l) {
  l = l + 0.0f;  // -0.0 -> +0.0
  uint32_t u = __float_as_uint(l);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o ^ 0x80000000u) : ~o;
  return __uint_as_float(u);
}

template <typename XT, int EP, bool LOGITS_IN>
__global__ __launch_bounds__(256) void route_kernel(
    const XT* __restrict__ x, const float* __restrict__ W_gate, const float* __restrict__ bias,
    int T, int h, int E, int k, float* __restrict__ logits, int* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ prob_part) {
  constexpr int TE = EP > 64 ? EP / 64 : 1;   // experts per thread
  constexpr int NEG = EP / TE;                // expert groups (<= 64)
  constexpr int TM = TT * NEG / 256;          // tokens per thread
  constexpr int NV = EP >= 64 ? EP / 64 : 1;  // logits per lane in the selection phase
  static_assert(TM >= 1 && TM * (256 / NEG) == TT, "tile");

  __shared__ float xs[KC][TT];
  __shared__ float ws[KC][EP];
  __shared__ float lg[TT][EP + 1];
  __shared__ float pp[4][EP];

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * TT;

  if (!LOGITS_IN) {
    const int eg = tid % NEG, tg = tid / NEG;
    float acc[TM][TE];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TE; ++j) acc[i][j] = 0.f;

    for (int k0 = 0; k0 < h; k0 += KC) {
      {  // x slice: 32 tokens x 32 h, 4 consecutive h per thread
        const int tt = tid >> 3, kk = (tid & 7) * 4;
        const int t = t0 + tt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = 0.f;
          if (t < T) v = Elem<XT>::load(x, (size_t)t * h + k0 + kk + i);
          xs[kk + i][tt] = v;
        }
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
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TE; ++j) {
        const int e = eg * TE + j;
        float v = acc[i][j];
        if (bias != nullptr && e < E) v += bias[e];
        lg[tg * TM + i][e] = v;
      }
    __syncthreads();
    for (int idx = tid; idx < TT * E; idx += 256) {
      const int tt = idx / E, e = idx % E;
      if (t0 + tt < T) logits[(size_t)(t0 + tt) * E + e] = lg[tt][e];
    }
  } else {
    for (int idx = tid; idx < TT * E; idx += 256) {
      const int tt = idx / E, e = idx % E;
      lg[tt][e] = (t0 + tt < T) ? logits[(size_t)(t0 + tt) * E + e] : 0.f;
    }
    __syncthreads();
  }

  // ---- selection: wave w handles tokens w*8 .. w*8+7
  const int lane = tid & 63, w = tid >> 6;
  float psum[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) psum[i] = 0.f;

  for (int q = 0; q < TT / 4; ++q) {
    const int tt = w * (TT / 4) + q;
    const int t = t0 + tt;
    if (t >= T) break;
    float v[NV];
    bool valid[NV];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i;
      valid[i] = e < E;
      v[i] = valid[i] ? lg[tt][e] : -INFINITY;
      m = fmaxf(m, v[i]);
    }
    m = wave_max(m);
    float ex[NV], s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      ex[i] = valid[i] ? expf(v[i] - m) : 0.f;
      s += ex[i];
    }
    s = wave_sum(s);
    const float inv = 1.0f / s;
#pragma unroll
    for (int i = 0; i < NV; ++i) psum[i] += ex[i] * inv;

    bool taken[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) taken[i] = false;
    float lmax = 0.f, wsum = 0.f;
    float my_l = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = lane + 64 * i;
        if (valid[i] && !taken[i]) {
          uint64_t key = ((uint64_t)ordered_bits(v[i]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
          best = key > best ? key : best;
        }
      }
      best = wave_max_u64(best);
      const int e_sel = (int)(0xFFFFFFFFu - (uint32_t)best);
      const float l_sel = from_ordered((uint32_t)(best >> 32));
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (lane + 64 * i == e_sel) taken[i] = true;
      if (j == 0) lmax = l_sel;
      wsum += expf(l_sel - lmax);
      if (lane == j) { my_l = l_sel; my_e = e_sel; }
    }
    if (lane < k) {
      topk_idx[(size_t)t * k + lane] = my_e;
      topk_w[(size_t)t * k + lane] = expf(my_l - lmax) / wsum;
    }
  }
  if (prob_part != nullptr) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i;
      if (e < EP) pp[w][e] = psum[i];
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256)
      prob_part[(size_t)blockIdx.x * E + e] = ((pp[0][e] + pp[1][e]) + pp[2][e]) + pp[3][e];
  }
}

__global__ void reduce_prob_kernel(const float* __restrict__ prob_part, int nblk, int E,
                                   float* __restrict__ prob_sum) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  float s = 0.f;
  for (int b = 0; b < nblk; ++b) s += prob_part[(size_t)b * E + e];
  prob_sum[e] = s;
}

template <typename XT, bool LIN>
hipError_t launch_route_t(const RouteArgs& a, hipStream_t st) {
  const int nblk = route_blocks(a.T);
  dim3 grid(nblk), block(256);
  const void* xp = a.x;
#define MOE_ROUTE_CASE(EPV)                                                                        \
  case EPV:                                                                                        \
    hipLaunchKernelGGL((route_kernel<XT, EPV, LIN>), grid, block, 0, st, (const XT*)xp, a.W_gate,  \
                       a.bias, a.T, a.h, a.E, a.k, a.logits, a.topk_idx, a.topk_w, a.prob_part);   \
    break;
  switch (expert_pad(a.E)) {
    MOE_ROUTE_CASE(8)
    MOE_ROUTE_CASE(16)
    MOE_ROUTE_CASE(32)
    MOE_ROUTE_CASE(64)
    MOE_ROUTE_CASE(128)
    MOE_ROUTE_CASE(256)
    default: return hipErrorInvalidValue;
  }
#undef MOE_ROUTE_CASE
  return hipGetLastError();
}

}  // namespace

int expert_pad(int E) {
  int p = 8;
  while (p < E) p <<= 1;
  return p;
}

int route_blocks(int T) { return (T + TT - 1) / TT; }

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  if (a.logits_in) {
    return a.bf16 ? launch_route_t<bf16_t, true>(a, st) : launch_route_t<float, true>(a, st);
  }
  return a.bf16 ? launch_route_t<bf16_t, false>(a, st) : launch_route_t<float, false>(a, st);
}

hipError_t launch_reduce_prob(const float* prob_part, int nblk, int E, float* prob_sum, hipStream_t st) {
  hipLaunchKernelGGL(reduce_prob_kernel, dim3((E + 255) / 256), dim3(256), 0, st, prob_part, nblk, E,
                     prob_sum);
  return hipGetLastError();
}

}  // namespace moe
