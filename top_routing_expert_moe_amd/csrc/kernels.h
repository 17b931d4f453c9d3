// Internal launchers of the MoE kernels (host side).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---- router
struct RouteArgs {
  const void* x;          // [T,h] fp32 or bf16
  const float* W_gate;    // [h,E]
  const float* bias;      // [E] or null
  int T, h, E, k;
  bool bf16;
  bool logits_in;         // logits is an input; x/W_gate/bias unused
  float* logits;          // [T,E]
  int* topk_idx;          // [T,k]
  float* topk_w;          // [T,k]
  float* prob_part;       // [route_blocks(T), E] or null
};
int expert_pad(int E);
int route_blocks(int T);
hipError_t launch_route(const RouteArgs& a, hipStream_t st);
hipError_t launch_reduce_prob(const float* prob_part, int nblk, int E, float* prob_sum, hipStream_t st);

// ---- permutation
constexpr int kPermBlock = 2048;  // assignments per histogram / scatter block
inline int perm_blocks(int64_t n) { return (int)((n + kPermBlock - 1) / kPermBlock); }

hipError_t launch_hist(const int* topk_idx, int n, int E, int* blk_counts, hipStream_t st);

struct ScanArgs {
  const int* blk_counts;   // [nhb,E]
  int nhb, E, T, k;
  int C;                   // capacity, INT32_MAX = none
  int BM;                  // rows per GEMM tile for tile_off; 0 = no tile schedule
  const float* prob_part;  // [nrb,E] or null
  int nrb;
  const float* prob_sum;   // [E] or null (used when prob_part is null)
  int* counts;             // [E]
  int* offsets;            // [E+1]
  int* blk_base;           // [nhb,E]
  int* tile_off;           // [E+1] or null
  float* aux;              // scalar or null
};
hipError_t launch_scan(const ScanArgs& a, hipStream_t st);

hipError_t launch_scatter(const int* topk_idx, int n, int E, int k, int C, const int* offsets,
                          const int* blk_base, int* slot_pos, int* sorted_slot, int* perm_token,
                          hipStream_t st);
hipError_t launch_gather(const void* x, const int* perm_token, const int* offsets, int E, int R_max,
                         int h, int elem_bytes, void* x_perm, hipStream_t st);
hipError_t launch_tiles(const int* offsets, int E, int BM, int* tile_off, hipStream_t st);

// ---- expert GEMMs
enum Act { ACT_NONE = 0, ACT_GELU = 1, ACT_SWIGLU = 2 };

struct GemmArgs {
  const void* A;        // rows of the left operand ([*, K], row-major)
  const int* a_rows;    // row r of the tile space -> row of A; null = identity
  const void* W;        // [E, K, N] row-major
  const void* W3;       // [E, K, N] (SwiGLU gate partner) or null
  int K, N;             // N = columns of W = columns of out
  void* out;            // [R_max, N]
  const int* offsets;   // [E+1] rows per expert (device)
  const int* tile_off;  // [E+1] m-tiles per expert, exclusive scan (device)
  int E;
  int R_max;            // upper bound of rows
  int act;
};
int gemm_bm(bool bf16);  // rows per m-tile of the expert GEMMs
hipError_t launch_gemm(const GemmArgs& a, bool bf16, hipStream_t st);

// ---- combine
hipError_t launch_combine(const void* O, const int* slot_pos, const float* topk_w, int T, int h, int k,
                          bool bf16, void* y, hipStream_t st);

}  // namespace moe
