// Internal launchers of the MoE kernels (host side).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---- router
constexpr int kSelTokens = 64;  // tokens per selection / histogram / scatter block

// The outputs of the scan and the scatter, for a selection kernel that produces them itself
// when the tokens are one block (T <= kSelTokens): see launch_select.
struct SmallPermute {
  int C;                   // capacity, INT32_MAX = none
  int BM;                  // rows per GEMM tile for tile_off; 0 = no tile list
  int big;                 // m_tile_rows threshold of the tile list (FfnPlan::big)
  int nbits;               // bits of an expert id (expert_bits)
  int* counts;             // [E] pre-drop
  int* offsets;            // [E+1] over kept
  int* tile_off;           // [E+1] or null
  float* aux;              // scalar or null
  int* slot_pos;           // [T*k]
  int* sorted_slot;        // [T*k]
  int* perm_token;         // [T*k]
};

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
  int* blk_counts;        // [route_blocks(T), E] or null: per-block expert histogram
  uint16_t* planes;       // bf16 x: route_scratch_bytes of scratch -- from 32 experts up [3][E16][h]
                          // bf16 split router weights, then (few tokens) [SH][T][E] fp32 partial
                          // logits
  // router variants (selection kernel): gate noise [T,E] added to the logits, softmax of
  // logits * inv_temp, ids replaced by (t*k + j) % E, soft top-K weights (the full
  // softmax at the selection, not renormalised)
  const float* noise = nullptr;
  float inv_temp = 1.0f;
  bool uniform = false;
  bool soft = false;
  // not null and T <= kSelTokens: the selection kernel also does the scan and the scatter
  const SmallPermute* permute = nullptr;
  // tokens per histogram block (prob_part and blk_counts rows): kSelTokens, or 16 when the
  // logits kernel also selects (route_hist_tokens); launch_select then launches nothing
  int hist_tokens = kSelTokens;
};
// router-input jitter: out = x * u elementwise in the storage dtype (n_elems * elem size % 16 == 0)
hipError_t launch_jitter(const void* x, const void* u, int64_t n_elems, bool bf16, void* out, hipStream_t st);
int route_planes_elems(int h, int E);
int route_hsplit(int T, int h, int E, bool bf16);              // h-split of the logits (1 = none)
size_t route_scratch_bytes(int T, int h, int E, bool bf16);   // bytes behind RouteArgs::planes
int route_blocks(int T);
// Tokens per histogram block of a layer's routing: 16 when the logits kernel selects the
// experts itself (bf16, at most 16 experts, h a multiple of 512, more than one 64-token
// block, no split of h and a fusable scan + scatter over the 16-token blocks), else
// kSelTokens.  A function of the sizes only, so that the backward finds the forward's blocks.
int route_hist_tokens(int T, int h, int E, bool bf16);
int route_hist_blocks(int T, int h, int E, bool bf16);  // ceil(T / route_hist_tokens)
hipError_t launch_logits(const RouteArgs& a, hipStream_t st);  // logits only (ignores logits_in)
hipError_t launch_select(const RouteArgs& a, hipStream_t st);  // softmax, top-k, weights, histogram
hipError_t launch_route(const RouteArgs& a, hipStream_t st);   // both (logits skipped when logits_in)
hipError_t launch_reduce_prob(const float* prob_part, int nblk, int E, float* prob_sum, hipStream_t st);

// ---- permutation (blocks of kSelTokens tokens = kSelTokens*k assignments)
hipError_t launch_hist(const int* topk_idx, int T, int k, int E, int* blk_counts, hipStream_t st);

struct ScanArgs {
  const int* blk_counts;   // [nhb,E]
  int nhb, E, T, k;
  int hpb = 1;             // histogram blocks per kSelTokens-token scatter block (fused scan only)
  int C;                   // capacity, INT32_MAX = none
  int BM;                  // rows per GEMM tile for tile_off; 0 = no tile schedule
  int big;                 // m_tile_rows threshold of the tile list (FfnPlan::big)
  const float* prob_part;  // [nrb,E] or null
  int nrb;
  const float* prob_sum;   // [E] or null (used when prob_part is null)
  int* counts;             // [E]
  int* offsets;            // [E+1]
  int* blk_base;           // [nhb,E]
  int* tile_off;           // [E+1] or null
  float* aux;              // scalar or null
  // fixed-capacity buckets: every expert gets C rows (offsets[e] = e * C), C = the
  // capacity, or the largest count when C == INT32_MAX; the bucket size goes to *cap_out
  bool binned;
  int* cap_out;            // scalar or null
};
hipError_t launch_scan(const ScanArgs& a, hipStream_t st);
// the scan and the scatter in one launch (not for fixed-capacity buckets); fusable: whether
// every block can read all nhb histograms (and the nrb softmax partial sums, nrb <= nhb)
bool scan_scatter_fusable(int nhb, int nrb, int E);
hipError_t launch_scan_scatter(const ScanArgs& a, const int* topk_idx, int* slot_pos, int* sorted_slot,
                               int* perm_token, hipStream_t st);
// bits of an expert id (at least 1): the scatter's match by ballots
inline int expert_bits(int E) {
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  return nbits;
}
// x_bins[r] = x[perm_token[r]] for filled bucket rows, zero for the rest of the E buckets
// (bucket size offsets[1] - offsets[0], fill min(counts[e], size)); rows >= offsets[E] untouched
hipError_t launch_binned_gather(const void* x, const int* perm_token, const int* offsets, const int* counts, int E,
                                int R_max, int h, int elem_bytes, void* x_bins, hipStream_t st);

hipError_t launch_scatter(const int* topk_idx, int T, int E, int k, int C, const int* offsets,
                          const int* blk_base, int* slot_pos, int* sorted_slot, int* perm_token,
                          hipStream_t st);
hipError_t launch_gather(const void* x, const int* perm_token, const int* offsets, int E, int R_max,
                         int h, int elem_bytes, void* x_perm, hipStream_t st);
hipError_t launch_tiles(const int* offsets, int E, int BM, int big, int* tile_off, hipStream_t st);

// ---- expert GEMMs
// ACT_SWIGLU_SEP is a kernel mode, not an activation: the raw SwiGLU pre-activations
// [a | g] in tiles that each take their weight columns from W1 alone or W3 alone.
enum Act { ACT_NONE = 0, ACT_GELU = 1, ACT_SWIGLU = 2, ACT_SWIGLU_SEP = 3 };

struct GemmArgs {
  const void* A;        // rows of the left operand ([*, K], row-major)
  const int* a_rows;    // row r of the tile space -> row of A; null = identity
  const void* W;        // [E, K, N] row-major
  const void* W3;       // [E, K, N] (SwiGLU gate partner) or null
  int K, N;             // N = columns of W = columns of out
  void* out;            // [R_max, N]; with ksplit > 1 the fp32 partial sums (see below)
  const int* offsets;   // [E+1] rows per expert (device)
  const int* tile_off;  // [E+1] m-tiles per expert, exclusive scan (device)
  int E;
  int R_max;            // upper bound of rows
  int act;
  bool out_f32;         // bf16 GEMM writing fp32 output (down projection inside the layer)
  int bm;               // rows per m-tile (gemm_bm); tile_off must be built with it
  int big;              // m_tile_rows threshold the tile list was built with
  // K split into ksplit equal parts (K / ksplit a multiple of 64).  With ksplit > 1
  // the kernel writes raw fp32 partial products, part s at out + s * R_max * NW
  // (row stride NW = 2N for SwiGLU -- W1 columns then W3 columns -- else N), and
  // launch_ffn_finish / the combine add the parts in ascending s.
  int ksplit;
  // raw: write the raw fp32 accumulators in the K-part layout (one part when ksplit <= 1),
  // no activation: the pre-activations [a | g] for the backward pass
  bool raw;
  // with raw, SwiGLU and 32-row tiles (bm 32, no K parts): each 512-column tile takes its
  // columns from W1 alone or W3 alone, so every k row of a weight stage is one 1 KiB run
  // (the layout of the output is the same)
  bool sep;
  // bf16 up projection (act SwiGLU or GELU) without K parts: not null = also write the
  // fp32 pre-activations here, in the raw layout ([R_max][2N] a | g, or [R_max][N])
  float* save;
};

// Tile height and K splits of one expert FFN (both GEMMs), a pure function of the sizes.
struct FfnPlan {
  int bm;       // rows per m-tile
  int s_up;     // K splits of the up projection (1 = none)
  int s_down;   // K splits of the down projection
  int big;      // with bm = 128: experts with at least this many rows take 256-row tiles (m_tile_rows)
};
FfnPlan plan_ffn(bool bf16, double rows_per_expert, int E, int R_max, int h, int f);
// rows per m-tile of the expert GEMMs, from the expected rows per expert
int gemm_bm(bool bf16, double rows_per_expert);
hipError_t launch_gemm(const GemmArgs& a, bool bf16, hipStream_t st);
// out[r, :] = act(sum_s part[s][r][:N] (, sum_s part[s][r][N:2N])) for r < offsets[E];
// act: ACT_NONE, ACT_GELU or ACT_SWIGLU; out is bf16 when out_bf16 else fp32.
// (save, act SwiGLU or GELU: the summed pre-activations are also written there, in the
// raw layout)
hipError_t launch_ffn_finish(const float* part, int S, int R_max, int N, int act, const int* offsets, int E,
                             bool out_bf16, void* out, hipStream_t st, float* save = nullptr);

// ---- combine
// O is fp32 when o_f32, else the y dtype.  With o_parts > 1 (fp32 only), O holds o_parts
// partial sums of the expert outputs, part s at O + s * o_part_stride elements.
hipError_t launch_combine(const void* O, bool o_f32, int o_parts, size_t o_part_stride, const int* slot_pos,
                          const float* topk_w, int T, int h, int k, bool bf16, void* y, hipStream_t st);

// ---- backward pass (backward.hip)
// grouped NT product over the 64-row tiles of the segments (tile_off built with BM = 64):
// C[r, n] = sum_k A[r, k] B(e, k, n), B(e, k, n) = B1[e*sbe + n*ldb + k] (k < K1) or
// B2[e*sbe + n*ldb + k - K1]; epi = ACT_SWIGLU / ACT_GELU turns dHm into da (| dg) in DAG
struct BwdNT {
  const void* A; int lda; bool a_bf16;
  const void* B1; const void* B2; int K1; long long sbe; int ldb; bool b_bf16;
  int K, N;
  const int* offsets; const int* tile_off; int E; int R_max;
  // bf16 operands run on MFMA with ts x ts tiles (128 or 256) over tile_off_ts, the ts-row
  // tile list of the same segments
  int ts; const int* tile_off_ts;
  float* C; int ldc;
  int epi; const float* pa; const float* pg; int ld_ag; void* DAG;
  // K parts (epi == ACT_NONE, 256-row tiles only): part p of C at C + p * R_max * ldc
  int ksplit;
};
// grouped TN product over each segment's rows: C_e[m, n] = sum_r A[row(r), m] B[r, n]
struct BwdTN {
  const void* A; int lda; const int* a_rows; bool a_bf16;
  const void* B; int ldb; bool b_bf16;
  int M, N;
  const int* offsets; int E;
  float* C1; float* C2; int N1; long long sce; int ldc;
  // one segment (E == 1, no gather) of `rows` rows in ksplit slices: fp32 partial sums
  // [ksplit][M][ldc] in `part`, then added in slice order
  int ksplit; int rows; float* part;
};
hipError_t launch_seg_init(int* seg, int T, hipStream_t st);
hipError_t launch_counts(const int* blk_counts, int nblk, int E, int* counts, hipStream_t st);
hipError_t launch_tile_scan(const int* offsets, int E, int BM, int* tile_off, hipStream_t st);
hipError_t launch_combine_bwd(const void* dy, const float* O, int n_parts, size_t part_stride, const int* slot_pos,
                              const float* topk_w, int T, int h, int k, bool bf16, float* dw, void* dO,
                              hipStream_t st);
// logit gradient of the weights and the aux loss; noise (or null) as in the forward's selection,
// p = softmax((logits + noise) * inv_temp); soft: the weights are p at the selection (soft top-K)
hipError_t launch_router_bwd(const float* logits, const float* noise, const int* topk_idx, const float* topk_w,
                             const float* dw, const int* counts, int T, int E, int k, float d_aux, float inv_temp,
                             bool soft, float* dl, hipStream_t st);
hipError_t launch_gemm_nt(const BwdNT& a, hipStream_t st);
hipError_t launch_gemm_tn(const BwdTN& a, hipStream_t st);
// dx[t] = dx_router[t] (* jitter[t], x's dtype, when not null) + sum over kept slots of the dX parts
hipError_t launch_dx_final(const float* dx_router, const void* jitter, const float* dXp, int parts,
                           size_t part_stride, const int* slot_pos, int T, int h, int k, bool bf16, void* dx,
                           hipStream_t st);
// xp[r] = x[rows[r]] (row_bytes each) for r < offsets[E]
hipError_t launch_gather_rows(const void* x, const int* rows, const int* offsets, int E, int R_max, int row_bytes,
                              void* xp, hipStream_t st);

}  // namespace moe
