// Grouped expert GEMMs over the variable-length expert segments.
//
// Method (MegaBlocks chapter "01 · MoE 为什么难算：变长专家输入", sections 2 and
// 4.3): each expert e multiplies the rows routed to it by its own weights --
// matmul, activation, matmul -- and the segments have data-dependent,
// skewed lengths.  SwiGLU experts gate the up projection with a second one
// (ops-transformer operator list names SwiGLU, "MoE 路由算子到底在做什么" §7).
//
// gfx950 design (bf16):
//  * one launch covers all experts: the m-tile -> expert map comes from the
//    device-side tile_off[] (exclusive scan of ceil(rows_e / 256)), so there
//    is no host synchronisation and experts with no rows cost nothing;
//  * workgroup tile 256 rows x 256 weight columns x 64 k, 4 waves of 128x128,
//    v_mfma_f32_32x32x16_bf16, fp32 accumulators (256 per lane);
//  * the weights are stored [K, N] with N contiguous, while MFMA wants 8
//    consecutive k per lane: each thread loads an 8x8 block (8 rows x 16 B)
//    and transposes it in registers before one 16-byte LDS store per column;
//  * LDS rows are 128 B (64 bf16) with the 16-byte chunk index XOR-swizzled by
//    (row ^ row>>3) & 7, conflict-free for both the column stores and the
//    MFMA fragment reads; two stages (128 KiB) double-buffer the k-loop;
//  * SwiGLU: the 256 weight columns of a tile are 128 of W1 and the same 128
//    of W3, arranged so each wave holds W1 and W3 accumulators of the same
//    output column in the same lane; silu(a)*g is applied in registers;
//  * the up projection reads its left operand straight from x through the
//    row -> token map (the gather is fused into the A-load);
//  * XCD-aware order: hardware workgroup i runs on XCD i%8; each XCD takes a
//    contiguous range of the tile list, with m-tiles fastest, so the m-tiles of
//    one expert that share a weight tile run together in one L2.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;

__device__ __forceinline__ void store4(bf16_t* p, const float* v) {
  *(u32x2*)p = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ void store4(float* p, const float* v) { *(floatx4*)p = floatx4{v[0], v[1], v[2], v[3]}; }

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
// element offset of (row, 16-byte chunk) in a [256][64] bf16 LDS tile
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * BK + ((chunk ^ swz(row)) << 3); }

template <int ACT, bool GATHER, typename OT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const int* __restrict__ a_rows, const bf16_t* __restrict__ W,
    const bf16_t* __restrict__ W3, int K, int N, OT* __restrict__ out,
    const int* __restrict__ offsets, const int* __restrict__ tile_off, int E, int NT) {
  constexpr int NO = ACT == ACT_SWIGLU ? BN / 2 : BN;  // output columns per tile
  __shared__ __attribute__((aligned(16))) bf16_t Wl[2][BN * BK];
  __shared__ __attribute__((aligned(16))) bf16_t Xl[2][BM * BK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---- tile schedule (XCD-aware), exits for surplus workgroups
  const int MT = tile_off[E];
  const int n_real = MT * NT;
  const int per = (n_real + 7) >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  if (slot >= per) return;
  const int L = xcd * per + slot;
  if (L >= n_real) return;
  const int mt = L % MT, nt = L / MT;
  const int e = find_expert(tile_off, E, mt);
  const int row0 = offsets[e] + (mt - tile_off[e]) * BM;
  const int row_end = min(row0 + BM, offsets[e + 1]);
  const int n0 = nt * NO;

  // ---- weight-tile loader: thread -> (8 LDS rows of group g, 8 k rows of group kg)
  const int g = tid & 31, kg = tid >> 5;
  const bf16_t* wsrc;
  bool wvalid;
  {
    int col;
    const bf16_t* Wm;
    if (ACT == ACT_SWIGLU) {
      const int wn = g >> 4, gg = g & 15;
      col = n0 + wn * 64 + (gg & 7) * 8;
      Wm = gg < 8 ? W : W3;
    } else {
      col = n0 + g * 8;
      Wm = W;
    }
    wvalid = col < N;
    wsrc = Wm + (size_t)e * K * N + (size_t)(kg * 8) * N + (wvalid ? col : 0);
  }
  // ---- activation-tile loader: thread -> chunk ch of rows (tid>>3) + 32*i
  const int ch = tid & 7;
  const bf16_t* xsrc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = row0 + (tid >> 3) + 32 * i;
    if (r < row_end) {
      const int src_row = GATHER ? a_rows[r] : r;
      xsrc[i] = A + (size_t)src_row * K + ch * 8;
    } else {
      xsrc[i] = nullptr;
    }
  }

  u32x4 wreg[8], xreg[8];
  auto load_tile = [&](int kt) {
    const size_t koff = (size_t)kt * BK * N;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (wvalid) wreg[r] = *(const u32x4*)(wsrc + koff + (size_t)r * N);
      else wreg[r] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (xsrc[i] != nullptr) xreg[i] = *(const u32x4*)(xsrc[i] + kt * BK);
      else xreg[i] = u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
    // transpose the 8x8 weight block: column c gets k-pairs (2d, 2d+1), d = 0..3
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      u32x4 v;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t lo = wreg[2 * d][c >> 1], hi = wreg[2 * d + 1][c >> 1];
        v[d] = (c & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
      }
      const int row = g * 8 + c;
      *(u32x4*)&Wl[buf][lds_off(row, kg)] = v;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (tid >> 3) + 32 * i;
      *(u32x4*)&Xl[buf][lds_off(row, ch)] = xreg[i];
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int wn = wave & 1, wm = wave >> 1;
  const int nk = K / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tile(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int chunk = 2 * ks + (lane >> 5);
      bf16x8 a[4], b[4];
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const int row = wn * 128 + ib * 32 + (lane & 31);
        a[ib] = *(const bf16x8*)&Wl[cur][lds_off(row, chunk)];
      }
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const int row = wm * 128 + jb * 32 + (lane & 31);
        b[jb] = *(const bf16x8*)&Xl[cur][lds_off(row, chunk)];
      }
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
          acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ib], b[jb], acc[ib][jb], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds token row (lane&31) of block jb and, for acc
  // element 4q+p, weight column 8q + 4*(lane>>5) + p of block ib.
  const int half = lane >> 5;
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    const int r = row0 + wm * 128 + jb * 32 + (lane & 31);
    if (r >= row_end) continue;
    OT* orow = out + (size_t)r * N;
    if (ACT == ACT_SWIGLU) {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn * 64 + ib * 32 + 8 * q + 4 * half;
          if (col >= N) continue;
          float v[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) v[p] = silu(acc[ib][jb][4 * q + p]) * acc[ib + 2][jb][4 * q + p];
          store4(orow + col, v);
        }
    } else {
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn * 128 + ib * 32 + 8 * q + 4 * half;
          if (col >= N) continue;
          float v[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const float z = acc[ib][jb][4 * q + p];
            v[p] = ACT == ACT_GELU ? gelu_erf(z) : z;
          }
          store4(orow + col, v);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 grouped GEMM on the vector ALUs (fp32 workloads: exact fp32 products,
// fp32 accumulation).  Tile 64 rows x 64 columns x 16 k, 4x4 per thread.
constexpr int FBM = 64, FBN = 64, FBK = 16;

template <int ACT, bool GATHER>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, const int* __restrict__ a_rows, const float* __restrict__ W,
    const float* __restrict__ W3, int K, int N, float* __restrict__ out,
    const int* __restrict__ offsets, const int* __restrict__ tile_off, int E, int NT) {
  __shared__ float As[FBK][FBM];
  __shared__ float Ws[FBK][FBN];
  __shared__ float W3s[ACT == ACT_SWIGLU ? FBK : 1][FBN];
  const int tid = threadIdx.x;
  const int MT = tile_off[E];
  const int mt = blockIdx.x / NT, nt = blockIdx.x % NT;
  if (mt >= MT) return;
  const int e = find_expert(tile_off, E, mt);
  const int row0 = offsets[e] + (mt - tile_off[e]) * FBM;
  const int row_end = min(row0 + FBM, offsets[e + 1]);
  const int n0 = nt * FBN;
  const float* We = W + (size_t)e * K * N;
  const float* W3e = ACT == ACT_SWIGLU ? W3 + (size_t)e * K * N : nullptr;

  const int am = tid >> 2, ak = (tid & 3) * 4;
  const int ar = row0 + am;
  const float* arow = nullptr;
  if (ar < row_end) arow = A + (size_t)(GATHER ? a_rows[ar] : ar) * K;
  const int wk = tid >> 4, wn4 = (tid & 15) * 4;
  const int tx = tid & 15, ty = tid >> 4;

  float acc[4][4], acc3[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = acc3[i][j] = 0.f;

  for (int k0 = 0; k0 < K; k0 += FBK) {
    floatx4 av = floatx4{0.f, 0.f, 0.f, 0.f};
    if (arow) av = *(const floatx4*)(arow + k0 + ak);
#pragma unroll
    for (int i = 0; i < 4; ++i) As[ak + i][am] = av[i];
    const bool nv = n0 + wn4 < N;
    floatx4 wv = nv ? *(const floatx4*)(We + (size_t)(k0 + wk) * N + n0 + wn4) : floatx4{0.f, 0.f, 0.f, 0.f};
    *(floatx4*)&Ws[wk][wn4] = wv;
    if (ACT == ACT_SWIGLU) {
      floatx4 w3 = nv ? *(const floatx4*)(W3e + (size_t)(k0 + wk) * N + n0 + wn4) : floatx4{0.f, 0.f, 0.f, 0.f};
      *(floatx4*)&W3s[wk][wn4] = w3;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      float a[4], b[4], b3[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Ws[kk][tx * 4 + j];
      if (ACT == ACT_SWIGLU) {
#pragma unroll
        for (int j = 0; j < 4; ++j) b3[j] = W3s[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
          if (ACT == ACT_SWIGLU) acc3[i][j] = fmaf(a[i], b3[j], acc3[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = row0 + ty * 4 + i;
    const int col = n0 + tx * 4;
    if (r >= row_end || col >= N) continue;
    floatx4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float z = acc[i][j];
      v[j] = ACT == ACT_SWIGLU ? silu(z) * acc3[i][j] : (ACT == ACT_GELU ? gelu_erf(z) : z);
    }
    *(floatx4*)(out + (size_t)r * N + col) = v;
  }
}

template <int ACT, bool G, typename OT>
hipError_t launch_bf16_t(const GemmArgs& a, hipStream_t st) {
  constexpr int NO = ACT == ACT_SWIGLU ? BN / 2 : BN;
  const int NT = (a.N + NO - 1) / NO;
  const long long slots = ((long long)(a.R_max + BM - 1) / BM + a.E) * NT;
  const long long grid = (slots + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<ACT, G, OT>), dim3((unsigned)grid), dim3(256), 0, st,
                     (const bf16_t*)a.A, a.a_rows, (const bf16_t*)a.W, (const bf16_t*)a.W3, a.K, a.N,
                     (OT*)a.out, a.offsets, a.tile_off, a.E, NT);
  return hipGetLastError();
}

template <int ACT, bool G>
hipError_t launch_f32_t(const GemmArgs& a, hipStream_t st) {
  const int NT = (a.N + FBN - 1) / FBN;
  const long long grid = ((long long)(a.R_max + FBM - 1) / FBM + a.E) * NT;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_f32_kernel<ACT, G>), dim3((unsigned)grid), dim3(256), 0, st,
                     (const float*)a.A, a.a_rows, (const float*)a.W, (const float*)a.W3, a.K, a.N,
                     (float*)a.out, a.offsets, a.tile_off, a.E, NT);
  return hipGetLastError();
}

template <bool BF, bool G>
hipError_t dispatch_act(const GemmArgs& a, hipStream_t st) {
  if (BF && a.out_f32) {
    if (a.act != ACT_NONE) return hipErrorInvalidValue;
    return launch_bf16_t<ACT_NONE, G, float>(a, st);
  }
  switch (a.act) {
    case ACT_NONE: return BF ? launch_bf16_t<ACT_NONE, G, bf16_t>(a, st) : launch_f32_t<ACT_NONE, G>(a, st);
    case ACT_GELU: return BF ? launch_bf16_t<ACT_GELU, G, bf16_t>(a, st) : launch_f32_t<ACT_GELU, G>(a, st);
    case ACT_SWIGLU: return BF ? launch_bf16_t<ACT_SWIGLU, G, bf16_t>(a, st) : launch_f32_t<ACT_SWIGLU, G>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int gemm_bm(bool bf16) { return bf16 ? BM : FBM; }

hipError_t launch_gemm(const GemmArgs& a, bool bf16, hipStream_t st) {
  if (bf16) return a.a_rows ? dispatch_act<true, true>(a, st) : dispatch_act<true, false>(a, st);
  return a.a_rows ? dispatch_act<false, true>(a, st) : dispatch_act<false, false>(a, st);
}

}  // namespace moe
