// Backward pass of the layer: the adjoint of each forward step, in reverse order.
//
// The pages name a backward pass for the gating operator (ops-transformer MoE article,
// operator list: moe_gating holds the router's forward and backward) and autograd
// wrappers around the permutation's gather and scatter (MegaBlocks chapter "01 · MoE
// 为什么难算", section 5 file map) without writing them out; what is computed here is
// the plain derivative of the forward:
//  * combine:   dw[t,j] = <dy[t], O[r]>,  dO[r] = w[t,j] dy[t]   (r = slot of (t, j));
//  * experts:   dHm = dO W2[e]^T; SwiGLU da = dHm g silu'(a), dg = dHm silu(a) (GELU:
//               da = dHm gelu'(a)); dX = da W1[e]^T (+ dg W3[e]^T);
//               dW2[e] = Hm^T dO, dW1[e] = X^T da, dW3[e] = X^T dg over the expert's rows;
//  * permutation adjoint: dx[t] += sum_j dX[slot of (t, j)];
//  * router:    softmax over the selected logits, dl[t,S_j] = w_j (dw_j - sum w dw); aux
//               loss d_aux (E/T) p_i (f_i - sum_e f_e p_e) with the full softmax p;
//               dW_gate = x^T dl, dx += dl W_gate^T.
//
// The GEMMs are grouped "NT" products C[r, n] = sum_k A[r, k] B_e[n, k] over the expert
// segments (the data gradients; B is the weight read along its contiguous dimension) and
// grouped "TN" products C_e[m, n] = sum_r A[row(r), m] B[r, n] over each expert's rows
// (the weight gradients).  bf16 operands run on the matrix cores: the large products on
// bwd_tile_kernel (the expert GEMM's direct-to-LDS pipeline), the others on
// gemm_bwd_mfma_kernel (register-staged); fp32 operands, and the router's small products,
// on the vector ALUs in fp32 (64 x 64 tiles, 4 x 4 per thread).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

template <typename T> __device__ __forceinline__ float ld(const T* p, size_t i);
template <> __device__ __forceinline__ float ld<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<bf16_t>(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
template <typename T> __device__ __forceinline__ void st(T* p, size_t i, float v);
template <> __device__ __forceinline__ void st<float>(float* p, size_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void st<bf16_t>(bf16_t* p, size_t i, float v) {
  p[i] = (bf16_t)f32_to_bf16_bits(v);
}

__device__ __forceinline__ float silu_grad(float z) {
  const float s = 1.0f / (1.0f + expf(-z));
  return s * (1.0f + z * (1.0f - s));
}
__device__ __forceinline__ float gelu_grad(float z) {
  return 0.5f * (1.0f + erff(z * 0.70710678118654752f)) + z * expf(-0.5f * z * z) * 0.39894228040143268f;
}

// counts[e] = sum over the 64-token blocks of the selection kernel's histogram
__global__ void counts_kernel(const int* __restrict__ blk_counts, int nblk, int E, int* __restrict__ counts) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  int s = 0;
  for (int b = 0; b < nblk; ++b) s += blk_counts[(size_t)b * E + e];
  counts[e] = s;
}

// tile_off[e] = exclusive scan of ceil(rows_e / BM) over the segments (one workgroup)
__global__ void tile_scan_kernel(const int* __restrict__ offsets, int E, int BM, int* __restrict__ tile_off) {
  if (threadIdx.x != 0) return;
  int acc = 0;
  for (int e = 0; e < E; ++e) {
    tile_off[e] = acc;
    acc += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
  }
  tile_off[E] = acc;
}

// Four consecutive elements at p + i (i a multiple of 4; rows of h, h a multiple of 64, keep
// them 16-byte aligned for fp32 and 8-byte aligned for bf16).
__device__ __forceinline__ floatx4 ld4(const float* p, size_t i) { return *(const floatx4*)(p + i); }
__device__ __forceinline__ floatx4 ld4(const bf16_t* p, size_t i) {
  const u32x2 v = *(const u32x2*)(p + i);
  return floatx4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u), __uint_as_float(v[1] << 16),
                 __uint_as_float(v[1] & 0xFFFF0000u)};
}
__device__ __forceinline__ void st4(float* p, size_t i, floatx4 v) { *(floatx4*)(p + i) = v; }
__device__ __forceinline__ void st4(bf16_t* p, size_t i, floatx4 v) {
  *(u32x2*)(p + i) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// One workgroup per token: dw[t,j] = <dy[t], O[r]> (O = sum of the down projection's
// K parts) and dO[r] = w[t,j] dy[t]; dropped slots get dw = 0 and write nothing.  Each
// thread takes four consecutive columns at a time.
template <typename TD>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const TD* __restrict__ dy, const float* __restrict__ O,
                                                          int n_parts, size_t part_stride,
                                                          const int* __restrict__ slot_pos,
                                                          const float* __restrict__ topk_w, int T, int h, int k,
                                                          float* __restrict__ dw, TD* __restrict__ dO) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int h4 = h >> 2;
  for (int j = 0; j < k; ++j) {
    const int r = slot_pos[(size_t)t * k + j];
    if (r < 0) {
      if (tid == 0) dw[(size_t)t * k + j] = 0.f;
      continue;
    }
    const float wj = topk_w[(size_t)t * k + j];
    float part = 0.f;
    for (int i4 = tid; i4 < h4; i4 += 256) {
      const floatx4 g = ld4(dy, (size_t)t * h + 4 * i4);
      floatx4 o = ld4(O, (size_t)r * h + 4 * i4);
      for (int p = 1; p < n_parts; ++p) o += ld4(O + p * part_stride, (size_t)r * h + 4 * i4);
      part += (g[0] * o[0] + g[1] * o[1]) + (g[2] * o[2] + g[3] * o[3]);
      st4(dO, (size_t)r * h + 4 * i4, floatx4{wj * g[0], wj * g[1], wj * g[2], wj * g[3]});
    }
    part = wave_sum(part);
    if ((tid & 63) == 0) red[tid >> 6] = part;
    __syncthreads();
    if (tid == 0) dw[(size_t)t * k + j] = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
  }
}

// One wave per token: the logit gradient of the renormalised selection and of the aux
// loss.  Lane l holds experts l, l + 64, ...
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ logits,
                                                         const float* __restrict__ noise,
                                                         const int* __restrict__ topk_idx,
                                                         const float* __restrict__ topk_w,
                                                         const float* __restrict__ dw,
                                                         const int* __restrict__ counts, int T, int E, int k,
                                                         float d_aux, float inv_temp, int soft,
                                                         float* __restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  constexpr int NQ = 4;  // E <= 256
  float l[NQ], p[NQ], fe[NQ];
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = lane + 64 * q;
    l[q] = e < E ? logits[(size_t)t * E + e] + (noise != nullptr ? noise[(size_t)t * E + e] : 0.f) : -INFINITY;
    m = fmaxf(m, l[q]);
  }
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = lane + 64 * q;
    p[q] = e < E ? expf((l[q] - m) * inv_temp) : 0.f;
    s += p[q];
  }
  s = wave_sum(s);
  const float inv = 1.0f / s;
  const float scale = 1.0f / (float)((int64_t)T * k);
  float fp = 0.f;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = lane + 64 * q;
    p[q] *= inv;
    fe[q] = e < E ? (float)counts[e] * scale : 0.f;
    fp += fe[q] * p[q];
  }
  fp = wave_sum(fp);
  // softmax(l / tau) has the Jacobian p_a (delta_ab - p_b) / tau
  const float ca = d_aux * (float)E / (float)T * inv_temp;
  float g[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) g[q] = ca * p[q] * (fe[q] - fp);
  float swd = 0.f;
  for (int j = 0; j < k; ++j) swd += topk_w[(size_t)t * k + j] * dw[(size_t)t * k + j];
  if (soft) {
    // weights p[S_j] (not renormalised): p_b (dw_b - sum_j w_j dw_j) / tau for every expert b
    float own[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) own[q] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[(size_t)t * k + j];
      const float d = dw[(size_t)t * k + j];
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if (lane + 64 * q == e) own[q] = d;
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) g[q] += p[q] * (own[q] - swd) * inv_temp;
  } else {
    // the renormalised softmax over the selection: w_j (dw_j - sum_j' w_j' dw_j') / tau
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[(size_t)t * k + j];
      const float v = topk_w[(size_t)t * k + j] * (dw[(size_t)t * k + j] - swd) * inv_temp;
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if (lane + 64 * q == e) g[q] += v;
    }
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = lane + 64 * q;
    if (e < E) dl[(size_t)t * E + e] = g[q];
  }
}

constexpr int VT = 64, VK = 16;  // VALU GEMM tile and k step

// C[r, n] = sum_k A[r, k] B(e, k, n) over the 64-row tiles of the segments, with
// B(e, k, n) = B1[e*sbe + n*ldb + k] for k < K1, else B2[e*sbe + n*ldb + k - K1].
// EPI = ACT_NONE: C fp32 [R, ldc].  EPI = ACT_SWIGLU / ACT_GELU: C is dHm; the epilogue
// forms the activation's input gradients from the pre-activations (a at pa[r*ld_ag + n],
// g at pg[r*ld_ag + n]) and writes da (and dg) to DAG [R, n_up*N] in TA.
template <typename TA, typename TB, int EPI>
__global__ __launch_bounds__(256) void gemm_nt_valu_kernel(const TA* __restrict__ A, int lda,
                                                           const TB* __restrict__ B1, const TB* __restrict__ B2,
                                                           int K1, long long sbe, int ldb, int K, int N,
                                                           const int* __restrict__ offsets,
                                                           const int* __restrict__ tile_off, int E,
                                                           float* __restrict__ C, int ldc,
                                                           const float* __restrict__ pa, const float* __restrict__ pg,
                                                           int ld_ag, TA* __restrict__ DAG) {
  __shared__ float As[VK][VT + 4];
  __shared__ float Bs[VK][VT + 4];
  const int tid = threadIdx.x;
  const int mt = blockIdx.y;
  if (mt >= tile_off[E]) return;
  const int e = find_expert(tile_off, E, mt);
  const int row0 = offsets[e] + (mt - tile_off[e]) * VT;
  const int row_end = offsets[e + 1];
  const int n0 = blockIdx.x * VT;
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  const int lr = tid / 4, lk = (tid % 4) * 4;  // loader: row / column lr, k lk .. lk+3
  for (int k0 = 0; k0 < K; k0 += VK) {
    {
      const int r = row0 + lr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = k0 + lk + q;
        As[lk + q][lr] = (r < row_end && kk < K) ? ld(A, (size_t)r * lda + kk) : 0.f;
      }
      const int n = n0 + lr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = k0 + lk + q;
        float v = 0.f;
        if (n < N && kk < K)
          v = kk < K1 ? ld(B1, (size_t)e * sbe + (size_t)n * ldb + kk)
                      : ld(B2, (size_t)e * sbe + (size_t)n * ldb + (kk - K1));
        Bs[lk + q][lr] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < VK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = row0 + ty * 4 + i;
    if (r >= row_end) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      const float v = acc[i][j];
      if (EPI == ACT_NONE) {
        C[(size_t)r * ldc + n] = v;
      } else if (EPI == ACT_SWIGLU) {
        const float a = pa[(size_t)r * ld_ag + n], g = pg[(size_t)r * ld_ag + n];
        const float sa = a / (1.0f + expf(-a));
        st(DAG, (size_t)r * 2 * N + n, v * g * silu_grad(a));
        st(DAG, (size_t)r * 2 * N + N + n, v * sa);
      } else {
        const float a = pa[(size_t)r * ld_ag + n];
        st(DAG, (size_t)r * N + n, v * gelu_grad(a));
      }
    }
  }
}

// C_e[m, n] = sum over the rows r of segment e of A[row(r), m] B[r, n]; written to
// C1[e*sce + m*ldc + n] for n < N1, else C2[e*sce + m*ldc + n - N1].  Rows past the
// segment read as zero; an empty segment writes zeros.
// With rows_per_split > 0 (one segment only): blockIdx.z takes rows_per_split rows of it
// and writes its partial sums to C1 + z * sce (added by reduce_parts_kernel).
template <typename TA, typename TB, bool GATHER>
__global__ __launch_bounds__(256) void gemm_tn_valu_kernel(const TA* __restrict__ A, int lda,
                                                           const int* __restrict__ a_rows,
                                                           const TB* __restrict__ B, int ldb, int M, int N,
                                                           const int* __restrict__ offsets,
                                                           float* __restrict__ C1, float* __restrict__ C2, int N1,
                                                           long long sce, int ldc, int rows_per_split) {
  __shared__ float As[VK][VT + 4];
  __shared__ float Bs[VK][VT + 4];
  const int tid = threadIdx.x;
  const int e = rows_per_split > 0 ? 0 : blockIdx.z;
  const int m0 = blockIdx.y * VT, n0 = blockIdx.x * VT;
  int rb = offsets[e], re = offsets[e + 1];
  if (rows_per_split > 0) {
    rb += blockIdx.z * rows_per_split;
    re = min(re, rb + rows_per_split);
    C1 += (size_t)blockIdx.z * sce;
    C2 = C1;
  }
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  const int lk = tid / 16, lc = (tid % 16) * 4;  // loader: k row lk, columns lc .. lc+3
  for (int r0 = rb; r0 < re; r0 += VK) {
    const int r = r0 + lk;
    const bool rv = r < re;
    const size_t arow = rv ? (size_t)(GATHER ? a_rows[r] : r) : 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = m0 + lc + q, n = n0 + lc + q;
      As[lk][lc + q] = (rv && m < M) ? ld(A, arow * lda + m) : 0.f;
      Bs[lk][lc + q] = (rv && n < N) ? ld(B, (size_t)r * ldb + n) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < VK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      if (rows_per_split > 0) C1[(size_t)m * ldc + n] = acc[i][j];
      else if (n < N1) C1[(size_t)e * sce + (size_t)m * ldc + n] = acc[i][j];
      else C2[(size_t)e * sce + (size_t)m * ldc + (n - N1)] = acc[i][j];
    }
  }
}

// out[i] = sum over s = 0 .. S-1 (ascending) of part[s * n + i]
__global__ __launch_bounds__(256) void reduce_parts_kernel(const float* __restrict__ part, int S, int64_t n,
                                                           float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = 0.f;
  for (int p = 0; p < S; ++p) v += part[(size_t)p * n + i];
  out[i] = v;
}

// ---------------------------------------------------------------------------
// The same grouped NT / TN products for bf16 operands on MFMA (v_mfma_f32_32x32x16_bf16,
// fp32 accumulation).  Workgroup tile 128 x 128, four waves of 64 x 64 (2 x 2 blocks of
// 32 x 32), k in stages of 64, two LDS buffers: the next stage's 16-byte global loads
// are in flight while the current stage's MFMAs run, then go to the other buffer.
// Operand layouts in LDS:
//  * K-contiguous (NT: both operands) -- [TS rows][64 k], rows padded to 72 elements
//    (144 B) so that the 16 rows of one 16-byte read phase hit distinct banks; the MFMA
//    fragment (8 consecutive k of one row) is one 16-byte read;
//  * M/N-contiguous (TN: both operands) -- [64 k][TS cols], rows padded by 16 elements
//    (rows 8 banks apart); the fragment (8 consecutive k of one column) is two transposing
//    8-byte reads (ds_read_b64_tr_b16: in a 16-lane group, lane j receives element j & 3
//    of the 8-byte block addressed by lane 4i + (j >> 2)).
// Tile sizes: TS = 128 (four waves of 64 x 64, two workgroups per CU) or TS = 256 (eight
// waves of 64 x 128, one workgroup per CU): the larger tile reads each operand half as
// often, which is what bounds these products when both operands stream from HBM.
constexpr int MKB = 64;
constexpr int LDK = MKB + 8;    // K-contiguous row stride (elements)
typedef short v4i16b __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16b v4i16_lds;

template <bool MC, int LDM>
__device__ __forceinline__ bf16x8 frag(const bf16_t* buf, int rc0, int kh, int lane) {
  if (!MC) {
    return *(const bf16x8*)&buf[(rc0 + (lane & 31)) * LDK + 16 * kh + 8 * (lane >> 5)];
  } else {
    const int g = lane >> 4, s = lane & 15;
    const int col = rc0 + 16 * (g & 1) + 4 * (s & 3);
    const int r = 16 * kh + 8 * (g >> 1) + (s >> 2);
    const v4i16b lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4i16_lds*)&buf[r * LDM + col]);
    const v4i16b hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4i16_lds*)&buf[(r + 4) * LDM + col]);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

template <int TS> struct BwdTile {
  static constexpr int NW = TS == 256 ? 8 : 4;           // waves
  static constexpr int WMW = TS == 256 ? 4 : 2, WNW = 2;  // waves along m / along n
  static constexpr int WTM = TS / WMW, WTN = TS / WNW;    // wave tile
  static constexpr int IB = WTM / 32, JB = WTN / 32;
  static constexpr int LDM = TS + 16;
  static constexpr int KC_ELEMS = TS * LDK, MC_ELEMS = MKB * LDM;
  static constexpr int NQ = TS * 8 / (NW * 64);           // 16-byte chunks per thread and operand
};

// MODE 0 = NT over the TS-row tiles of the segments, MODE 1 = TN over each segment's rows.
template <int MODE, int EPI, bool GATHER, int TS>
__global__ __launch_bounds__(BwdTile<TS>::NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void
gemm_bwd_mfma_kernel(const bf16_t* __restrict__ A, int lda, const int* __restrict__ a_rows,
                     const bf16_t* __restrict__ B1, const bf16_t* __restrict__ B2, int K1, long long sbe, int ldb,
                     int K, int M, int N, const int* __restrict__ offsets, const int* __restrict__ tile_off, int E,
                     float* __restrict__ C1, float* __restrict__ C2, int N1, long long sce, int ldc,
                     const float* __restrict__ pa, const float* __restrict__ pg, int ld_ag, bf16_t* __restrict__ DAG) {
  using TC = BwdTile<TS>;
  constexpr int NT_ = TC::NW * 64;
  constexpr bool MC = MODE == 1;
  constexpr int SZ = MC ? TC::MC_ELEMS : TC::KC_ELEMS;
  constexpr int IB = TC::IB, JB = TC::JB, NQ = TC::NQ, CPR = TS / 8;  // chunks per M/N-contiguous row
  __shared__ __attribute__((aligned(16))) bf16_t As[2][SZ];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][SZ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / TC::WNW, wn = wave % TC::WNW;
  int e, m0, row_end, kb, ke;
  const int n0 = blockIdx.x * TS;
  if (MODE == 0) {
    const int mt = blockIdx.y;
    if (mt >= tile_off[E]) return;
    e = find_expert(tile_off, E, mt);
    m0 = offsets[e] + (mt - tile_off[e]) * TS;  // segment rows
    row_end = offsets[e + 1];
    kb = 0;
    ke = K;
  } else {
    e = blockIdx.z;
    m0 = blockIdx.y * TS;                       // output rows (columns of A)
    row_end = M;
    kb = offsets[e];                            // k runs over the segment's rows
    ke = offsets[e + 1];
  }
  const bf16_t* Be1 = B1 + (size_t)e * sbe;
  const bf16_t* Be2 = B2 + (size_t)e * sbe;

  u32x4 ra[NQ], rb[NQ];
  // global -> registers for the stage starting at k0 (zero outside the operands)
  auto gload = [&](int k0) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int c = tid + NT_ * q;
      if (MODE == 0) {
        const int row = c >> 3, kc = (c & 7) * 8;   // TS rows x 8 chunks
        const int r = m0 + row;
        ra[q] = r < row_end ? *(const u32x4*)&A[(size_t)r * lda + k0 + kc] : u32x4{0u, 0u, 0u, 0u};
        const int n = n0 + row;
        const bf16_t* bp = k0 < K1 ? Be1 + (size_t)n * ldb + k0 + kc : Be2 + (size_t)n * ldb + (k0 - K1) + kc;
        rb[q] = n < N ? *(const u32x4*)bp : u32x4{0u, 0u, 0u, 0u};
      } else {
        const int kr = c / CPR, cc = (c % CPR) * 8;  // 64 k-rows x TS/8 chunks
        const int r = k0 + kr;
        const bool rv = r < ke;
        const int arow = rv ? (GATHER ? a_rows[r] : r) : 0;
        ra[q] = (rv && m0 + cc < M) ? *(const u32x4*)&A[(size_t)arow * lda + m0 + cc] : u32x4{0u, 0u, 0u, 0u};
        rb[q] = (rv && n0 + cc < N) ? *(const u32x4*)&B1[(size_t)r * ldb + n0 + cc] : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int c = tid + NT_ * q;
      int off;
      if (MODE == 0) off = (c >> 3) * LDK + (c & 7) * 8;
      else off = (c / CPR) * TC::LDM + (c % CPR) * 8;
      *(u32x4*)&As[buf][off] = ra[q];
      *(u32x4*)&Bs[buf][off] = rb[q];
    }
  };

  floatx16 acc[IB][JB];
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (ke - kb + MKB - 1) / MKB;
  if (nk > 0) {
    gload(kb);
    lstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kb + (kt + 1) * MKB);
#pragma unroll
    for (int kh = 0; kh < MKB / 16; ++kh) {
      bf16x8 fa[IB], fb[JB];
#pragma unroll
      for (int i = 0; i < IB; ++i) fa[i] = frag<MC, TC::LDM>(As[cur], wm * TC::WTM + 32 * i, kh, lane);
#pragma unroll
      for (int j = 0; j < JB; ++j) fb[j] = frag<MC, TC::LDM>(Bs[cur], wn * TC::WTN + 32 * j, kh, lane);
#pragma unroll
      for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }
  // lane holds, for acc element 4q + p of block (i, j): row wm*WTM + 32i + 8q + 4*(lane >> 5) + p,
  // column wn*WTN + 32j + (lane & 31)
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int m = m0 + wm * TC::WTM + 32 * i + 8 * q + 4 * (lane >> 5) + p;
          const int n = n0 + wn * TC::WTN + 32 * j + (lane & 31);
          if (m >= row_end || n >= N) continue;
          const float v = acc[i][j][4 * q + p];
          if (MODE == 1) {
            if (n < N1) C1[(size_t)e * sce + (size_t)m * ldc + n] = v;
            else C2[(size_t)e * sce + (size_t)m * ldc + (n - N1)] = v;
          } else if (EPI == ACT_NONE) {
            C1[(size_t)m * ldc + n] = v;
          } else if (EPI == ACT_SWIGLU) {
            const float a = pa[(size_t)m * ld_ag + n], g = pg[(size_t)m * ld_ag + n];
            const float sa = a / (1.0f + expf(-a));
            DAG[(size_t)m * 2 * N + n] = (bf16_t)f32_to_bf16_bits(v * g * silu_grad(a));
            DAG[(size_t)m * 2 * N + N + n] = (bf16_t)f32_to_bf16_bits(v * sa);
          } else {
            const float a = pa[(size_t)m * ld_ag + n];
            DAG[(size_t)m * N + n] = (bf16_t)f32_to_bf16_bits(v * gelu_grad(a));
          }
        }
}

// ---------------------------------------------------------------------------
// The large products (bf16 operands; tiles of 256 P x 256 or 128 Q) with the expert GEMM's
// pipeline: operands go from global memory straight into LDS (global_load_lds_dwordx4,
// no register staging), the P operand three stages ahead and the Q operand two, and
// each wave waits only for its own copies of the stage it is about to read.
// P is the MFMA row operand: a lane's accumulators hold four consecutive P indices
// (8q + 4(lane >> 5) + 0..3 of a 32-block), stored as one vector; Q is the column
// operand (index lane & 31).
//  * NT (data gradients): C[r, n] = sum_k A[r, k] B(e, n, k); P = n (rows of B), Q = r
//    (rows of A).  Both are staged [256 rows][64 k], k contiguous, 16-byte chunks XOR-ed
//    by kswz(row); a fragment (8 consecutive k of one row) is one 16-byte read.
//  * TN (weight gradients): C_e[m, n] = sum_{r in segment e} A[r, m] B[r, n]; P = n,
//    Q = m.  Both are staged [64 r][256 columns], chunks XOR-ed by cswz(r); a fragment is
//    two transposing 8-byte reads.  A segment's last stage is partial: the copies read a
//    valid row in place of the missing ones and the fragments' k-values past the segment
//    are set to zero before the MFMAs.
typedef __attribute__((address_space(3))) void lds_void_t;

namespace bt {
constexpr int TS = 256, KB = 64, WAVES = 8;  // P extent of a tile, k per stage, waves
constexpr int NSP = 3, NSQ = 2;              // LDS stages of P and Q
constexpr int STP = TS * KB;                 // elements per P stage
constexpr int NIP = STP / 512 / WAVES;       // 1 KiB copies per wave and P stage
constexpr int BLK = 512;                     // elements per 1 KiB copy
constexpr int GM = 4, GN = 8;                // tile groups, as in the forward GEMM
}  // namespace bt

__device__ __forceinline__ int kswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int cswz(int r) { return ((r & 3) << 1) ^ ((r & 3) << 2); }

// one 16-byte-per-lane copy from global memory into the wave's 1 KiB LDS block at the
// byte address in m0 (no destination registers: nothing stays in flight in a register)
__device__ __forceinline__ void bt_copy16(const void* gptr, uint32_t lds_block) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_block) : "memory", "m0");
}

// tile l of an expert's me x NT tiles, in groups of GM m-tiles x GN n-tiles (m fastest)
__device__ __forceinline__ void bt_group(int l, int me, int NT, int& mt, int& nt) {
  const int mg = l / (bt::GM * NT);
  const int gm = min(bt::GM, me - mg * bt::GM);
  const int r = l - mg * bt::GM * NT;
  const int ng = r / (gm * bt::GN);
  const int r2 = r - ng * gm * bt::GN;
  mt = mg * bt::GM + r2 % gm;
  nt = ng * bt::GN + r2 / gm;
}

// zero the k-values k0 + t (t = 0..7) of a fragment that lie at or past `valid`
__device__ __forceinline__ bf16x8 bt_mask(bf16x8 v, int k0, int valid) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 s = __builtin_bit_cast(s16x8, v);
#pragma unroll
  for (int t = 0; t < 8; ++t)
    if (k0 + t >= valid) s[t] = 0;
  return __builtin_bit_cast(bf16x8, s);
}

// MODE 0 = NT over the TQ-row tiles of the segments (tile_off: their list), in S K parts
// (part s of C at C1 + s * R_max * ldc); MODE 1 = TN over each segment's rows (TQ = 256).
// The Q extent TQ of a tile is 256 (4 x 2 waves of 64 x 128) or 128 (2 x 4 waves of 64 x 64).
template <int MODE, int EPI, bool SPLIT, int TQ = 256>
__global__ __launch_bounds__(bt::WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void
bwd_tile_kernel(const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ B1,
                const bf16_t* __restrict__ B2, int K1, long long sbe, int ldb, int K, int M, int N,
                const int* __restrict__ offsets, const int* __restrict__ tile_off, int E, int NT, int MT, int S,
                int R_max, float* __restrict__ C1, float* __restrict__ C2, int N1, long long sce, int ldc,
                const float* __restrict__ pa, const float* __restrict__ pg, int ld_ag, bf16_t* __restrict__ DAG) {
  using namespace bt;
  static_assert(TQ == 256 || (TQ == 128 && MODE == 0), "tile shapes");
  constexpr int WQ = TQ / 64, WP = WAVES / WQ;  // waves along Q / along P
  constexpr int WTQ = 64, WTP = TS / WP;         // wave tile
  constexpr int IB = WTP / 32, JB = WTQ / 32;    // 32 x 32 blocks per wave
  constexpr int STQ = TQ * KB;                   // elements per Q stage
  constexpr int NIQ = STQ / BLK / WAVES;         // 1 KiB copies per wave and Q stage
  __shared__ __attribute__((aligned(1024))) bf16_t smem[NSP * STP + NSQ * STQ];
  bf16_t(*Ps)[STP] = reinterpret_cast<bf16_t(*)[STP]>(smem);
  bf16_t(*Qs)[STQ] = reinterpret_cast<bf16_t(*)[STQ]>(smem + NSP * STP);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int uwave = __builtin_amdgcn_readfirstlane(wave);

  // ---- tile.  NT tiles all do the same work: each XCD takes a contiguous range of the
  // tile list, so tiles that share operands share its L2.  TN tiles do work in proportion
  // to their expert's rows, so they are dealt round-robin over the XCDs (launch order),
  // which spreads every expert over the whole chip.
  int e, p0, q0, kb, ke, row_end = 0, ks = 0;
  {
    const int n_tiles = MODE == 0 ? tile_off[E] * NT : E * MT * NT;
    const int n_real = n_tiles * (SPLIT ? S : 1);
    int L = blockIdx.x;
    if (MODE == 0) {
      const int per = (n_real + 7) >> 3;
      const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
      if (slot >= per) return;
      L = xcd * per + slot;
    }
    if (L >= n_real) return;
    if (SPLIT) {
      ks = L / n_tiles;
      L -= ks * n_tiles;
    }
    int mt, nt;
    if (MODE == 0) {
      int lo = 0, hi = E;  // expert: tile_off[e] * NT <= L < tile_off[e + 1] * NT
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tile_off[mid] * NT <= L) lo = mid; else hi = mid;
      }
      e = lo;
      bt_group(L - tile_off[e] * NT, tile_off[e + 1] - tile_off[e], NT, mt, nt);
      q0 = offsets[e] + mt * TQ;
      row_end = offsets[e + 1];
      const int Kc = SPLIT ? K / S : K;
      kb = ks * Kc;
      ke = kb + Kc;
    } else {
      e = L / (MT * NT);
      bt_group(L - e * MT * NT, MT, NT, mt, nt);
      q0 = mt * TQ;
      kb = offsets[e];
      ke = offsets[e + 1];
    }
    p0 = nt * TS;
  }
  const int nk = (ke - kb + KB - 1) / KB;

  // ---- copy plan: P copy i of wave w fills 1 KiB block NIP * w + i of a P stage, Q copy
  // i block NIQ * w + i of a Q stage
  const bf16_t* pb1[NIP];
  const bf16_t* pb2[NIP];
  const bf16_t* qa[NIQ];
  int rl[NIP];  // TN: the stage row (k) of each copy (the same for both operands)
#pragma unroll
  for (int i = 0; i < NIP; ++i) {
    if (MODE == 0) {
      const int r = 8 * (NIP * wave + i) + (lane >> 3);  // stage row (n)
      const int ch = ((lane & 7) ^ kswz(r)) << 3;
      const size_t n = (size_t)min(p0 + r, N - 1);
      pb1[i] = B1 + (size_t)e * sbe + n * ldb + ch;
      pb2[i] = B2 + (size_t)e * sbe + n * ldb + ch;
    } else {
      rl[i] = 2 * (NIP * wave + i) + (lane >> 5);
      const int ch = ((lane & 31) ^ cswz(rl[i])) << 3;
      pb1[i] = B1 + min(p0 + ch, N - 8);
    }
  }
#pragma unroll
  for (int i = 0; i < NIQ; ++i) {
    if (MODE == 0) {
      const int r = 8 * (NIQ * wave + i) + (lane >> 3);  // stage row (r)
      const int ch = ((lane & 7) ^ kswz(r)) << 3;
      qa[i] = A + (size_t)min(q0 + r, row_end - 1) * lda + ch;
    } else {
      const int ch = ((lane & 31) ^ cswz(rl[i])) << 3;  // TQ = 256: the same rows as P
      qa[i] = A + min(q0 + ch, M - 8);
    }
  }
  const uint32_t ps_lds = (uint32_t)(uintptr_t)(lds_void_t*)&Ps[0][0];
  const uint32_t qs_lds = (uint32_t)(uintptr_t)(lds_void_t*)&Qs[0][0];
  auto copy_q = [&](int i, int kt, int buf) {
    const bf16_t* src;
    if (MODE == 0) src = qa[i] + kb + kt * KB;
    else src = qa[i] + (size_t)min(kb + kt * KB + rl[i], ke - 1) * lda;
    bt_copy16(src, qs_lds + 2u * (uint32_t)(buf * STQ + BLK * (NIQ * uwave + i)));
  };
  auto copy_p = [&](int i, int kt, int buf) {
    const bf16_t* src;
    if (MODE == 0) {
      const int k0 = kb + kt * KB;
      src = k0 < K1 ? pb1[i] + k0 : pb2[i] + (k0 - K1);
    } else {
      src = pb1[i] + (size_t)min(kb + kt * KB + rl[i], ke - 1) * ldb;
    }
    bt_copy16(src, ps_lds + 2u * (uint32_t)(buf * STP + BLK * (NIP * uwave + i)));
  };
  // copies of MFMA group `part` of `parts`: the Q copies of stage qkt take the first
  // four groups, the P copies of stage pkt every other group after them when there are
  // 16 groups, the next four when there are 8 (parts == 1: all at once); ALL: both
  // stages are known to exist
  auto issue_part = [&](int qkt, int qnb, int pkt, int pnb, int part, int parts, bool all = false) {
    const int sp = parts < 8 ? parts : 8;
    const bool split = parts > 1;
#pragma unroll
    for (int i = 0; i < NIQ; ++i)
      if ((all || qkt >= 0) && (split ? i * (sp / 2) / NIQ : 0) == part) copy_q(i, qkt, qnb);
#pragma unroll
    for (int i = 0; i < NIP; ++i)
      if ((all || pkt >= 0) && (split ? sp / 2 + i * (parts >= 2 * sp ? sp : sp / 2) / NIP : 0) == part)
        copy_p(i, pkt, pnb);
  };

  // ---- fragment offsets (elements within a stage) for 16-k step kh and half h
  const int wn = wave % WP, wm = wave / WP;
  const int g = lane >> 4, s = lane & 15, l31 = lane & 31, hf = lane >> 5;
  int poff[KB / 16][2][IB], qoff[KB / 16][2][JB];
#pragma unroll
  for (int kh = 0; kh < KB / 16; ++kh)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (MODE == 0) {  // one 16-byte read (h = 0 only)
#pragma unroll
        for (int ib = 0; ib < IB; ++ib) {
          const int r = wn * WTP + 32 * ib + l31;
          poff[kh][h][ib] = r * KB + (((2 * kh + hf) ^ kswz(r)) << 3);
        }
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const int r = wm * WTQ + 32 * jb + l31;
          qoff[kh][h][jb] = r * KB + (((2 * kh + hf) ^ kswz(r)) << 3);
        }
      } else {  // transposing reads: lane s of group g reads row 16kh + 8(g>>1) + 4h + (s>>2)
        const int r = 16 * kh + 8 * (g >> 1) + 4 * h + (s >> 2);
#pragma unroll
        for (int ib = 0; ib < IB; ++ib) {
          const int col = wn * WTP + 32 * ib + 16 * (g & 1) + 4 * (s & 3);
          poff[kh][h][ib] = r * TS + (((col >> 3) ^ cswz(r)) << 3) + (col & 7);
        }
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const int col = wm * WTQ + 32 * jb + 16 * (g & 1) + 4 * (s & 3);
          qoff[kh][h][jb] = r * TS + (((col >> 3) ^ cswz(r)) << 3) + (col & 7);
        }
      }
    }
  auto frag = [&](const bf16_t* buf, int off0, int off1) -> bf16x8 {
    if (MODE == 0) return *(const bf16x8*)&buf[off0];
    const v4i16b lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4i16_lds*)&buf[off0]);
    const v4i16b hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4i16_lds*)&buf[off1]);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  floatx16 acc[IB][JB];
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // MFMAs of one stage (`valid` k-values of it are real), with the copies of later
  // stages issued between the MFMA groups
  auto compute = [&](int qbuf, int pbuf, int qkt, int qnb, int pkt, int pnb, bool all, int valid) {
    const bf16_t* Pb = Ps[pbuf];
    const bf16_t* Qb = Qs[qbuf];
    constexpr int PARTS = (KB / 16) * IB;
    // every copy must fall in one of the PARTS groups (issue_part's mapping)
    constexpr int SP = PARTS < 8 ? PARTS : 8;
    static_assert((NIQ - 1) * (SP / 2) / NIQ < SP / 2 &&
                      SP / 2 + (NIP - 1) * (PARTS >= 2 * SP ? SP : SP / 2) / NIP < PARTS,
                  "copy groups");
#pragma unroll
    for (int kh = 0; kh < KB / 16; ++kh) {
      bf16x8 a[IB], b[JB];
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) b[jb] = frag(Qb, qoff[kh][0][jb], qoff[kh][1][jb]);
#pragma unroll
      for (int ib = 0; ib < IB; ++ib) a[ib] = frag(Pb, poff[kh][0][ib], poff[kh][1][ib]);
      if (MODE == 1 && valid < KB) {
        const int k0 = 16 * kh + 8 * hf;
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) b[jb] = bt_mask(b[jb], k0, valid);
#pragma unroll
        for (int ib = 0; ib < IB; ++ib) a[ib] = bt_mask(a[ib], k0, valid);
      }
#pragma unroll
      for (int ib = 0; ib < IB; ++ib) {
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
          acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ib], b[jb], acc[ib][jb], 0, 0, 0);
        issue_part(qkt, qnb, pkt, pnb, kh * IB + ib, PARTS, all);
      }
    }
  };

  // ---- pipeline: stage kt in Q buffer kt % NSQ and P buffer kt % NSP.  During stage kt
  // the Q copies of stage kt + 1 and the P copies of stage kt + 2 are issued (in that
  // order), so at the top of stage kt + 1 only the newest NIP copies may still be in
  // flight; the barrier then makes every wave's copies visible and releases the buffers
  // the new copies go to.
#pragma unroll
  for (int p = 0; p < NSP - 1; ++p)
    if (p < nk) issue_part(p < NSQ - 1 ? p : -1, p, p, p, 0, 1);
  constexpr int U = NSP * NSQ;  // stages per unrolled step: every buffer index is a constant
  int kt = 0;
  for (; kt + U + NSP - 2 < nk; kt += U) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NIP) : "memory");
      __syncthreads();
      compute(j % NSQ, j % NSP, kt + j + NSQ - 1, (j + NSQ - 1) % NSQ, kt + j + NSP - 1, (j + NSP - 1) % NSP, true,
              KB);
    }
  }
  for (; kt < nk; ++kt) {
    if (kt + 1 < nk) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NIP) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int qkt = kt + NSQ - 1 < nk ? kt + NSQ - 1 : -1;
    const int pkt = kt + NSP - 1 < nk ? kt + NSP - 1 : -1;
    compute(kt % NSQ, kt % NSP, qkt, qkt % NSQ, pkt, pkt % NSP, false, min(KB, ke - kb - kt * KB));
  }

  // ---- epilogue: acc[ib][jb][4q + i] is P index wn*WTP + 32ib + 8q + 4hf + i and Q index
  // wm*WTQ + 32jb + l31.  The tile goes through LDS (fp32, half of its Q rows at a time) so
  // that each output row is written by one wave, 16 contiguous bytes per lane: written
  // straight from the accumulators, every store instruction would touch 32 rows.
  constexpr int LDR = TS + 4;  // staged row stride (floats)
  constexpr int HQ = TQ / 2;   // Q rows per half
  static_assert(HQ * LDR * 4 <= (NSP * STP + NSQ * STQ) * 2, "staging fits in LDS");
  float* stg = reinterpret_cast<float*>(smem);
  const int qend = MODE == 0 ? row_end : M;
  __syncthreads();  // every wave is done reading the last stage
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm / (WQ / 2) == half) {
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int ib = 0; ib < IB; ++ib)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = (wm % (WQ / 2)) * WTQ + 32 * jb + l31;
            const int col = wn * WTP + 32 * ib + 8 * q + 4 * hf;
            *(floatx4*)&stg[row * LDR + col] = floatx4{acc[ib][jb][4 * q], acc[ib][jb][4 * q + 1],
                                                       acc[ib][jb][4 * q + 2], acc[ib][jb][4 * q + 3]};
          }
    }
    __syncthreads();
    const int n = p0 + 4 * lane;
    for (int rr = 0; rr < HQ / WAVES; ++rr) {
      const int row = uwave * (HQ / WAVES) + rr;
      const int qi = q0 + half * HQ + row;
      if (qi >= qend || n >= N) continue;
      const floatx4 v = *(const floatx4*)&stg[row * LDR + 4 * lane];
      if (MODE == 1) {
        float* dst = n < N1 ? C1 + (size_t)e * sce + (size_t)qi * ldc + n
                            : C2 + (size_t)e * sce + (size_t)qi * ldc + (n - N1);
        *(floatx4*)dst = v;
      } else if (EPI == ACT_NONE) {
        *(floatx4*)&C1[((size_t)(SPLIT ? ks * R_max : 0) + qi) * ldc + n] = v;
      } else if (EPI == ACT_SWIGLU) {
        const floatx4 a4 = *(const floatx4*)&pa[(size_t)qi * ld_ag + n];
        const floatx4 g4 = *(const floatx4*)&pg[(size_t)qi * ld_ag + n];
        float da[4], dg[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = a4[i];
          da[i] = v[i] * g4[i] * silu_grad(a);
          dg[i] = v[i] * (a / (1.0f + expf(-a)));
        }
        bf16_t* orow = DAG + (size_t)qi * 2 * N;
        *(u32x2*)&orow[n] = u32x2{pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3])};
        *(u32x2*)&orow[N + n] = u32x2{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
      } else {
        const floatx4 a4 = *(const floatx4*)&pa[(size_t)qi * ld_ag + n];
        float da[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) da[i] = v[i] * gelu_grad(a4[i]);
        *(u32x2*)&DAG[(size_t)qi * N + n] = u32x2{pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3])};
      }
    }
    __syncthreads();
  }
}

// xp[r] = x[rows[r]] for the rows of the segments (r < offsets[E]), 16 bytes per lane
__global__ __launch_bounds__(256) void gather_rows_kernel(const u32x4* __restrict__ x, const int* __restrict__ rows,
                                                          const int* __restrict__ offsets, int E, int cpr,
                                                          u32x4* __restrict__ xp) {
  const int r = blockIdx.x;
  if (r >= offsets[E]) return;
  const u32x4* src = x + (size_t)rows[r] * cpr;
  for (int c = threadIdx.x; c < cpr; c += 256) xp[(size_t)r * cpr + c] = src[c];
}

// dx[t] = dx_router[t] + sum over kept slots j (ascending) of dX[slot of (t, j)], where
// dX is the sum of the `parts` K parts of dXp (part p at dXp + p * part_stride), in order;
// four consecutive columns per thread at a time
template <typename TD>
__global__ __launch_bounds__(256) void dx_final_kernel(const float* __restrict__ dx_router,
                                                       const TD* __restrict__ jitter,
                                                       const float* __restrict__ dXp, int parts, size_t part_stride,
                                                       const int* __restrict__ slot_pos, int T, int h, int k,
                                                       TD* __restrict__ dx) {
  const int t = blockIdx.x;
  const int h4 = h >> 2;
  for (int i4 = threadIdx.x; i4 < h4; i4 += 256) {
    const size_t at = (size_t)t * h + 4 * i4;
    // the router read x * u: its share of the gradient is multiplied by u
    floatx4 v = ld4(dx_router, at);
    if (jitter != nullptr) v *= ld4(jitter, at);
    for (int j = 0; j < k; ++j) {
      const int r = slot_pos[(size_t)t * k + j];
      if (r < 0) continue;
      floatx4 d = ld4(dXp, (size_t)r * h + 4 * i4);
      for (int p = 1; p < parts; ++p) d += ld4(dXp + p * part_stride, (size_t)r * h + 4 * i4);
      v += d;
    }
    st4(dx, at, v);
  }
}

}  // namespace

// one segment of T rows and its 64-row tile list: seg = {0, T}, seg + 2 = {0, ceil(T / 64)}
__global__ void seg_init_kernel(int* seg, int T) {
  if (threadIdx.x == 0) {
    seg[0] = 0;
    seg[1] = T;
    seg[2] = 0;
    seg[3] = (T + VT - 1) / VT;
  }
}

hipError_t launch_seg_init(int* seg, int T, hipStream_t st) {
  hipLaunchKernelGGL(seg_init_kernel, dim3(1), dim3(64), 0, st, seg, T);
  return hipGetLastError();
}

hipError_t launch_counts(const int* blk_counts, int nblk, int E, int* counts, hipStream_t st) {
  hipLaunchKernelGGL(counts_kernel, dim3((E + 255) / 256), dim3(256), 0, st, blk_counts, nblk, E, counts);
  return hipGetLastError();
}

hipError_t launch_tile_scan(const int* offsets, int E, int BM, int* tile_off, hipStream_t st) {
  hipLaunchKernelGGL(tile_scan_kernel, dim3(1), dim3(64), 0, st, offsets, E, BM, tile_off);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const void* dy, const float* O, int n_parts, size_t part_stride, const int* slot_pos,
                              const float* topk_w, int T, int h, int k, bool bf16, float* dw, void* dO,
                              hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(combine_bwd_kernel<bf16_t>, dim3(T), dim3(256), 0, st, (const bf16_t*)dy, O, n_parts,
                       part_stride, slot_pos, topk_w, T, h, k, dw, (bf16_t*)dO);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<float>, dim3(T), dim3(256), 0, st, (const float*)dy, O, n_parts,
                       part_stride, slot_pos, topk_w, T, h, k, dw, (float*)dO);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const float* logits, const float* noise, const int* topk_idx, const float* topk_w,
                             const float* dw, const int* counts, int T, int E, int k, float d_aux, float inv_temp,
                             bool soft, float* dl, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (E > 256) return hipErrorInvalidValue;
  hipLaunchKernelGGL(router_bwd_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, noise, topk_idx, topk_w, dw,
                     counts, T, E, k, d_aux, inv_temp, soft ? 1 : 0, dl);
  return hipGetLastError();
}

namespace {
bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// the pipelined 256 x 256 kernel for an NT product, when its layout allows it
bool bt_nt_ok(const BwdNT& a) {
  const int S = std::max(a.ksplit, 1);
  if (!(a.a_bf16 && a.b_bf16 && (a.ts == 256 || a.ts == 128) && a.tile_off_ts != nullptr)) return false;
  if (a.K % (S * bt::KB) != 0 || a.K1 % bt::KB != 0 || a.lda % 8 || a.ldb % 8 || a.N % 4 || a.sbe % 8) return false;
  if (!al16(a.A) || !al16(a.B1) || !al16(a.B2)) return false;
  if (a.epi == ACT_NONE) return a.ldc % 4 == 0 && al16(a.C);
  return S == 1 && a.ld_ag % 4 == 0 && al16(a.pa) && (a.pg == nullptr || al16(a.pg)) &&
         ((uintptr_t)a.DAG & 7) == 0;
}

template <int TQ>
hipError_t launch_bt_nt_t(const BwdNT& a, hipStream_t st) {
  const int NT = (a.N + bt::TS - 1) / bt::TS;
  const int S = std::max(a.ksplit, 1);
  const long long slots = ((long long)(a.R_max + TQ - 1) / TQ + a.E) * NT * S;
  const long long grid = (slots + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
#define MOE_BTN(EPI, SP)                                                                                         \
  hipLaunchKernelGGL((bwd_tile_kernel<0, EPI, SP, TQ>), dim3((unsigned)grid), dim3(bt::WAVES * 64), 0, st,      \
                     (const bf16_t*)a.A, a.lda, (const bf16_t*)a.B1, (const bf16_t*)a.B2, a.K1, a.sbe, a.ldb,    \
                     a.K, 0, a.N, a.offsets, a.tile_off_ts, a.E, NT, 0, S, a.R_max, a.C, a.C, a.N, 0LL, a.ldc, \
                     a.pa, a.pg, a.ld_ag, (bf16_t*)a.DAG)
  if (a.epi == ACT_SWIGLU) MOE_BTN(ACT_SWIGLU, false);
  else if (a.epi == ACT_GELU) MOE_BTN(ACT_GELU, false);
  else if (S > 1) MOE_BTN(ACT_NONE, true);
  else MOE_BTN(ACT_NONE, false);
#undef MOE_BTN
  return hipGetLastError();
}

hipError_t launch_bt_nt(const BwdNT& a, hipStream_t st) {
  return a.ts == 256 ? launch_bt_nt_t<256>(a, st) : launch_bt_nt_t<128>(a, st);
}

// ... for a TN product (rows not gathered, both weight dimensions at least one tile)
bool bt_tn_ok(const BwdTN& a) {
  return a.a_bf16 && a.b_bf16 && a.a_rows == nullptr && a.ksplit <= 1 && a.M >= bt::TS && a.N >= bt::TS &&
         a.M % 8 == 0 && a.N % 8 == 0 && a.lda % 8 == 0 && a.ldb % 8 == 0 && a.ldc % 4 == 0 && a.N1 % 4 == 0 &&
         a.sce % 4 == 0 && al16(a.A) && al16(a.B) && al16(a.C1) && al16(a.C2);
}

hipError_t launch_bt_tn(const BwdTN& a, hipStream_t st) {
  const int MT = (a.M + bt::TS - 1) / bt::TS, NT = (a.N + bt::TS - 1) / bt::TS;
  const long long grid = ((long long)a.E * MT * NT + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_tile_kernel<1, ACT_NONE, false>), dim3((unsigned)grid), dim3(bt::WAVES * 64), 0, st,
                     (const bf16_t*)a.A, a.lda, (const bf16_t*)a.B, (const bf16_t*)a.B, 0, 0LL, a.ldb, 0, a.M, a.N,
                     a.offsets, nullptr, a.E, NT, MT, 1, 0, a.C1, a.C2, a.N1, a.sce, a.ldc, nullptr, nullptr, 0,
                     nullptr);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_nt(const BwdNT& a, hipStream_t st) {
  if (bt_nt_ok(a)) return launch_bt_nt(a, st);
  if (a.ksplit > 1) return hipErrorInvalidValue;  // K parts only on the pipelined kernel
  if (a.a_bf16 && a.b_bf16 && a.tile_off_ts != nullptr && a.K % MKB == 0 && a.K1 % MKB == 0 && a.lda % 8 == 0 &&
      a.ldb % 8 == 0 && (a.ts == 128 || a.ts == 256)) {
#define MOE_NTM(EPI, TS)                                                                                           \
  hipLaunchKernelGGL((gemm_bwd_mfma_kernel<0, EPI, false, TS>),                                                    \
                     dim3((a.N + TS - 1) / TS, (a.R_max + TS - 1) / TS + a.E), dim3(BwdTile<TS>::NW * 64), 0, st,  \
                     (const bf16_t*)a.A, a.lda, nullptr, (const bf16_t*)a.B1, (const bf16_t*)a.B2, a.K1, a.sbe,     \
                     a.ldb, a.K, 0, a.N, a.offsets, a.tile_off_ts, a.E, a.C, a.C, a.N, 0LL, a.ldc, a.pa, a.pg,     \
                     a.ld_ag, (bf16_t*)a.DAG)
    if (a.ts == 256) {
      if (a.epi == ACT_SWIGLU) MOE_NTM(ACT_SWIGLU, 256);
      else if (a.epi == ACT_GELU) MOE_NTM(ACT_GELU, 256);
      else MOE_NTM(ACT_NONE, 256);
    } else {
      if (a.epi == ACT_SWIGLU) MOE_NTM(ACT_SWIGLU, 128);
      else if (a.epi == ACT_GELU) MOE_NTM(ACT_GELU, 128);
      else MOE_NTM(ACT_NONE, 128);
    }
#undef MOE_NTM
    return hipGetLastError();
  }
  const dim3 grid((a.N + VT - 1) / VT, (a.R_max + VT - 1) / VT + a.E);
#define MOE_NT(TA, TB, EPI)                                                                                    \
  hipLaunchKernelGGL((gemm_nt_valu_kernel<TA, TB, EPI>), grid, dim3(256), 0, st, (const TA*)a.A, a.lda,        \
                     (const TB*)a.B1, (const TB*)a.B2, a.K1, a.sbe, a.ldb, a.K, a.N, a.offsets, a.tile_off, a.E, \
                     a.C, a.ldc, a.pa, a.pg, a.ld_ag, (TA*)a.DAG)
  if (a.a_bf16 && a.b_bf16) {
    if (a.epi == ACT_SWIGLU) MOE_NT(bf16_t, bf16_t, ACT_SWIGLU);
    else if (a.epi == ACT_GELU) MOE_NT(bf16_t, bf16_t, ACT_GELU);
    else MOE_NT(bf16_t, bf16_t, ACT_NONE);
  } else if (!a.a_bf16 && !a.b_bf16) {
    if (a.epi == ACT_SWIGLU) MOE_NT(float, float, ACT_SWIGLU);
    else if (a.epi == ACT_GELU) MOE_NT(float, float, ACT_GELU);
    else MOE_NT(float, float, ACT_NONE);
  } else {
    return hipErrorInvalidValue;
  }
#undef MOE_NT
  return hipGetLastError();
}

hipError_t launch_gemm_tn(const BwdTN& a, hipStream_t st) {
  if (bt_tn_ok(a)) return launch_bt_tn(a, st);
  if (a.ksplit > 1) {
    // one segment of rows split in a.ksplit slices: partial sums in a.part, added in order
    if (a.E != 1 || a.part == nullptr || a.a_rows != nullptr) return hipErrorInvalidValue;
    const int per = (a.rows + a.ksplit - 1) / a.ksplit;
    const dim3 g((a.N + VT - 1) / VT, (a.M + VT - 1) / VT, a.ksplit);
    const long long sz = (long long)a.M * a.ldc;
#define MOE_TNS(TA, TB)                                                                                         \
  hipLaunchKernelGGL((gemm_tn_valu_kernel<TA, TB, false>), g, dim3(256), 0, st, (const TA*)a.A, a.lda, nullptr, \
                     (const TB*)a.B, a.ldb, a.M, a.N, a.offsets, a.part, a.part, a.N, sz, a.ldc, per)
    if (a.a_bf16 && !a.b_bf16) MOE_TNS(bf16_t, float);
    else if (!a.a_bf16 && !a.b_bf16) MOE_TNS(float, float);
    else return hipErrorInvalidValue;
#undef MOE_TNS
    hipLaunchKernelGGL(reduce_parts_kernel, dim3((unsigned)((sz + 255) / 256)), dim3(256), 0, st, a.part, a.ksplit,
                       (int64_t)sz, a.C1);
    return hipGetLastError();
  }
  if (a.a_bf16 && a.b_bf16 && a.M % 8 == 0 && a.N % 8 == 0 && a.lda % 8 == 0 && a.ldb % 8 == 0) {
    // weight gradients: M and N are weight dimensions (large), so the 256 tile when both fill it
    const bool big = a.M >= 256 && a.N >= 256;
#define MOE_TNM(G, TS)                                                                                             \
  hipLaunchKernelGGL((gemm_bwd_mfma_kernel<1, ACT_NONE, G, TS>), dim3((a.N + TS - 1) / TS, (a.M + TS - 1) / TS, a.E), \
                     dim3(BwdTile<TS>::NW * 64), 0, st, (const bf16_t*)a.A, a.lda, a.a_rows, (const bf16_t*)a.B,     \
                     (const bf16_t*)a.B, 0, 0LL, a.ldb, 0, a.M, a.N, a.offsets, nullptr, a.E, a.C1, a.C2, a.N1,     \
                     a.sce, a.ldc, nullptr, nullptr, 0, nullptr)
    if (big) {
      if (a.a_rows) MOE_TNM(true, 256); else MOE_TNM(false, 256);
    } else {
      if (a.a_rows) MOE_TNM(true, 128); else MOE_TNM(false, 128);
    }
#undef MOE_TNM
    return hipGetLastError();
  }
  const dim3 grid((a.N + VT - 1) / VT, (a.M + VT - 1) / VT, a.E);
#define MOE_TN(TA, TB, G)                                                                                      \
  hipLaunchKernelGGL((gemm_tn_valu_kernel<TA, TB, G>), grid, dim3(256), 0, st, (const TA*)a.A, a.lda, a.a_rows, \
                     (const TB*)a.B, a.ldb, a.M, a.N, a.offsets, a.C1, a.C2, a.N1, a.sce, a.ldc, 0)
  const bool g = a.a_rows != nullptr;
  if (a.a_bf16 && a.b_bf16) {
    if (g) MOE_TN(bf16_t, bf16_t, true); else MOE_TN(bf16_t, bf16_t, false);
  } else if (a.a_bf16 && !a.b_bf16) {
    if (g) MOE_TN(bf16_t, float, true); else MOE_TN(bf16_t, float, false);
  } else if (!a.a_bf16 && !a.b_bf16) {
    if (g) MOE_TN(float, float, true); else MOE_TN(float, float, false);
  } else {
    return hipErrorInvalidValue;
  }
#undef MOE_TN
  return hipGetLastError();
}

hipError_t launch_dx_final(const float* dx_router, const void* jitter, const float* dXp, int parts,
                           size_t part_stride, const int* slot_pos, int T, int h, int k, bool bf16, void* dx,
                           hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (parts < 1) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(dx_final_kernel<bf16_t>, dim3(T), dim3(256), 0, st, dx_router, (const bf16_t*)jitter, dXp,
                       parts, part_stride, slot_pos, T, h, k, (bf16_t*)dx);
  else
    hipLaunchKernelGGL(dx_final_kernel<float>, dim3(T), dim3(256), 0, st, dx_router, (const float*)jitter, dXp,
                       parts, part_stride, slot_pos, T, h, k, (float*)dx);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int* rows, const int* offsets, int E, int R_max, int row_bytes,
                              void* xp, hipStream_t st) {
  if (R_max <= 0) return hipSuccess;
  if (row_bytes % 16 != 0 || ((uintptr_t)x | (uintptr_t)xp) % 16 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)R_max), dim3(256), 0, st, (const u32x4*)x, rows, offsets, E,
                     row_bytes / 16, (u32x4*)xp);
  return hipGetLastError();
}

}  // namespace moe
