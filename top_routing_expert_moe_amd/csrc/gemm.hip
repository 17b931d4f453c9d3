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
//    device-side tile_off[] (exclusive scan of ceil(rows_e / BM)), so there is
//    no host synchronisation and experts with no rows cost nothing;
//  * workgroup tile BM rows x 256 weight columns x 64 k per LDS stage, 8 waves,
//    v_mfma_f32_32x32x16_bf16 with fp32 accumulators.  BM follows the expected
//    rows per expert: 256 (4 x 2 waves of 64 x 128, compute-bound prefill) or 128
//    (2 x 4 waves of 64 x 64); an expert's last m-tile runs the shape its rows
//    need.  When every m-tile has at most 32 rows (decode) the launch only
//    streams weights, and its tiles are 32 rows x 512 weight columns (1 x 8 waves
//    of 32 x 64), so that each k row of a weight stage is a longer contiguous run
//    (SwiGLU: 512 columns of W1 alone or W3 alone, written as raw a and g for a
//    second pass that applies the activation -- ACT_SWIGLU_SEP);
//  * both operands go from global memory straight into LDS (global_load_lds,
//    16 B per lane) with no register staging.  The weights stay [K, N] with N
//    contiguous in LDS and the MFMA operand (8 consecutive k of one column) is
//    read with ds_read_b64_tr_b16, the transposing LDS read;
//  * the 16-byte chunk index of each LDS row is XOR-swizzled with a function of
//    the row so that both the transposing reads and the activation reads are
//    free of bank conflicts; the copies of the next stage are issued in small
//    groups between the MFMAs of the current one;
//  * SwiGLU: each wave's weight columns are half W1 and the same columns of W3,
//    so silu(a) * g is applied in registers in the epilogue;
//  * the up projection reads its left operand straight from x through the
//    row -> token map (the gather is fused into the copy);
//  * XCD-aware order: hardware workgroup i runs on XCD i%8; each XCD takes a
//    contiguous range of the tile list, which is ordered in 4 x 8 groups of
//    (m-tile, n-tile) inside each expert, so the workgroups running together in
//    one XCD share activation and weight tiles in its L2.
#include <algorithm>
#include <climits>
#include <cstdlib>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BN = 256;  // weight columns staged per tile

__device__ __forceinline__ void store4(bf16_t* p, const float* v) {
  *(u32x2*)p = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ void store4(float* p, const float* v) { *(floatx4*)p = floatx4{v[0], v[1], v[2], v[3]}; }


// Tile order.  Tiles are listed expert by expert; inside an expert (me m-tiles x NT
// n-tiles) they come in groups of GM m-tiles x GN n-tiles, m fastest inside a group,
// then the next n-group, then the next m-group.  Consecutive tiles -- which run at the
// same time on one XCD -- therefore share both their activation rows (across the GN
// n-tiles) and their weight columns (across the GM m-tiles) in that XCD's L2.
#ifndef MOE_GM
#define MOE_GM 4
#endif
#ifndef MOE_GN
#define MOE_GN 8
#endif
constexpr int GM = MOE_GM, GN = MOE_GN;

// Which workgroup runs which tile.  The hardware hands workgroup i to XCD i % 8, in launch
// order: workgroup i waits until XCD i % 8 has a free CU, even while other XCDs idle.  So
// the eight XCDs move through their workgroups in step, and a schedule is fast when, at
// each step, the eight get tiles of the same cost.
//  * kOrderRanges: XCD x runs the x-th eighth of the list (its workgroups take every
//    nslot-th tile of it).  Equal counts, but not equal costs when tile heights differ:
//    at T = 4096, E = 8, k = 2 three XCDs get only full 256-row tiles.
//  * kOrderNRange: XCD x runs n-tiles x, x + 8, x + 16, ... of every m-tile, in the grouped
//    order of a launch of those n-tiles.  With NT a multiple of 8 every XCD then has the
//    same sequence of tile heights, and its weight columns stay in its own L2.  It reads
//    every activation row once per XCD.  (Contiguous n-ranges per XCD instead fetched 10 %
//    more bytes into L2 and were 0.5 % slower.)
//  * kOrderLaunch: tile i runs on workgroup i, one m-tile at a time (n fastest), so the
//    tiles the eight XCDs take together are of one m-tile.
// Measured (one MI355X, A/B in one session, n-ranges then contiguous per XCD): at
// T = 4096, h = 4096, f = 14336, E = 8, k = 2 the up projection takes 1.770 ms with
// ranges, 1.716 ms with n-ranges and 1.736 ms in launch order, and the down projection
// 0.942 / 0.934 / 0.947 ms; at
// T = 8192, h = 1024, f = 4096, E = 64, k = 2 (capacity 320) the down projection takes
// 0.125 ms with ranges, 0.118 ms in launch order and 0.156 ms with n-ranges (NT = 4: half
// the XCDs idle); at T = 4096, h = 4096, f = 2048, E = 256, k = 8 the up projection takes
// 1.733 / 1.737 / 1.751 ms and the down projection 0.985 / 0.999 / 0.972 ms.  Ranges
// balanced by tile cost instead of count (256-row tile 4, 128-row 2, 32-row 1) made the
// prefill-shaped up projection slower (1.80 -> 1.98 ms): their counts differ, so the XCDs
// fall out of step.
enum TileOrder { kOrderRanges = 0, kOrderLaunch = 1, kOrderNRange = 2 };

// Reads of the tile list and the expert offsets: uniform addresses, loaded through the
// constant address space so that they are scalar loads (the GEMM counts its vector-memory
// operations by hand, and a vector load here would make the compiler wait for them all).
__device__ __forceinline__ int ldc(const int* p, int i) {
  return ((const __attribute__((address_space(4))) int*)p)[i];
}

struct TileInfo {
  int e, ks, row0, rows, n0;
};

// The tile at position L of the launch's list: K part ks = L / n_tiles, then position Lt
// in the tile list.  Expert e: tile_off[e] * NT <= Lt < tile_off[e + 1] * NT, searched from
// e_from (an expert at or before it; 0 for none) -- a few steps forward, then bisection.
// fh, big: the tile heights (m_tile_rows); NO: output columns per n-tile.
__device__ __forceinline__ TileInfo tile_at(int L, const int* __restrict__ tile_off, const int* __restrict__ offsets,
                                            int E, int NT, int n_tiles, bool split, int fh, int big, int NO,
                                            int e_from, int gmx = GM) {
  TileInfo t;
  t.ks = split ? L / n_tiles : 0;
  const int Lt = L - t.ks * n_tiles;
  int lo = e_from, hi = E;  // tile_off[lo] * NT <= Lt < tile_off[hi] * NT
  for (int st = 0; st < 4 && hi - lo > 1; ++st) {
    if (ldc(tile_off, lo + 1) * NT <= Lt) ++lo;
    else hi = lo + 1;
  }
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ldc(tile_off, mid) * NT <= Lt) lo = mid; else hi = mid;
  }
  const int e = lo;
  t.e = e;
  const int t0 = ldc(tile_off, e);
  const int me = ldc(tile_off, e + 1) - t0;
  const int l = Lt - t0 * NT;
  const int mg = l / (gmx * NT);
  const int gm = min(gmx, me - mg * gmx);
  const int r = l - mg * gmx * NT;
  const int ng = r / (gm * GN);
  const int r2 = r - ng * gm * GN;
  const int mt_local = mg * gmx + r2 % gm;
  const int nt = ng * GN + r2 / gm;
  const int o0 = ldc(offsets, e), o1 = ldc(offsets, e + 1);
  const int fe = m_tile_rows(o1 - o0, fh, big);  // this expert's tile height
  t.row0 = o0 + mt_local * fe;
  t.rows = min(fe, o1 - t.row0);
  t.n0 = nt * NO;
  return t;
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glob_void_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int KB = 64;    // k per LDS stage (4 MFMA k-steps of 16)
constexpr int WST = KB * BN;  // weight stage, elements: [64 k][256 n], n contiguous
constexpr int XCH = KB / 8;   // 16-byte chunks per activation row
#ifndef MOE_WAVES
#define MOE_WAVES 8
#endif
constexpr int kWaves = MOE_WAVES;  // waves per workgroup: two per SIMD
constexpr int NIW = 32 / kWaves;   // weight copies (1 KiB each, 32 per stage) per wave and stage

// Tile shapes by token-tile height: the wave grid (waves along m x along n) and the
// number of LDS stages that fit.  Eight waves, two per SIMD: while one waits on a barrier,
// an LDS read or a copy, the other issues MFMAs.  256 rows: 4 x 2 waves of 64 x 128
// (prefill); 128 rows: 2 x 4 waves of 64 x 64; 32 rows (an expert's last m-tile in a
// launch of 128- or 256-row tiles): 1 x 4 waves of 32 x 64 compute, the other four only
// copy (such tiles stream weights, and the deeper pipeline keeps more bytes in flight).
// SPREAD: the next stage's copies are issued between the first SPREAD groups of MFMAs
// of the current stage (issuing them early leaves them the most time to land; spreading
// them keeps the MFMA issue from stalling behind a full memory queue).
template <int BMT> struct TileCfg;
// NSTAGE counts activation stages; NSW weight stages (NSW = NSTAGE, or NSTAGE + 1 when a
// third weight stage fits: the weights, streamed from HBM, then run two stages ahead).
#ifndef MOE_NSW256
#define MOE_NSW256 3
#endif
template <> struct TileCfg<256> {
  static constexpr int WMW = kWaves == 8 ? 4 : 2, WNW = 2, NSTAGE = 2, NSW = MOE_NSW256, SPREAD = 8;
};
template <> struct TileCfg<128> {
  static constexpr int WMW = kWaves == 8 ? 2 : 1, WNW = 4, NSTAGE = 3, NSW = 3, SPREAD = 8;
};
template <> struct TileCfg<32> { static constexpr int WMW = 1, WNW = 4, NSTAGE = 4, NSW = 4, SPREAD = 8; };
// Weight-streaming launches (every m-tile at most 32 rows) use wide tiles: 512 weight
// columns (SwiGLU: 256 of W1 and the same 256 of W3), so every k row of a weight stage is
// a 512-byte run of each matrix instead of 256 bytes (measured on this chip: the decode
// up projection's weights stream at 6.3 TB/s in 512-byte runs, 5.8 in 256-byte runs).
// All eight waves compute (32 x 64 each); two 64 KiB weight stages, one workgroup per CU.
// Without K parts (the up projection) the next stage's copies are all issued right after
// the barrier (SPREAD 0) and tiles go to workgroups in launch order; with K parts (the
// down projection) the copies are spread and the order is XCD-aware as above.  (Measured
// at 16 rows per expert, h = 4096, f = 14336, E = 8: each choice is 2-4 % faster on the
// GEMM it is used for than the other.)
constexpr int BNW = 512;
template <bool SPLIT> struct TileCfgWide32 {
  static constexpr int WMW = 1, WNW = 8, NSTAGE = 2, NSW = 2, SPREAD = SPLIT ? 8 : 0;
};

// Swizzles (16-byte chunk index XOR a function of the row).  The LDS serves 256 bytes
// (64 banks) per cycle, i.e. 32 lanes of an 8-byte read or 16 lanes of a 16-byte read:
//  * weight stage rows are 256 n = 32 chunks.  The 32 lanes of a transposing read
//    served together touch rows r0 .. r0+3 (r0 a multiple of 4) at chunks 4b .. 4b+3;
//    XOR-ing with 2*(r & 3) ^ 4*(r & 3) gives each row a distinct 64-byte bank group;
//  * activation stage rows are 64 k = 8 chunks (128 B).  The 16 lanes read together touch
//    16 consecutive rows at one chunk; rows of equal parity share banks, so the XOR value
//    (r & 7) ^ ((r >> 3) & 1) is distinct across the 8 rows of either parity.
// (Measured with rocprofv3: no LDS bank-conflict cycles in either GEMM.)
__device__ __forceinline__ int wswz(int r) { return ((r & 3) << 1) ^ ((r & 3) << 2); }
__device__ __forceinline__ int xswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// One 16-byte-per-lane copy from global memory straight into LDS (the wave's 1 KiB
// block starts at the LDS byte address in m0).  Issued as a plain instruction so that
// the compiler does not serialise later LDS reads behind it: the pipeline below waits
// for these copies itself (s_waitcnt vmcnt + barrier) before any wave reads the stage.
// It has no destination registers, so nothing is left in flight in a register, and
// no other code in these kernels uses m0.
__device__ __forceinline__ void copy_to_lds16(const void* gptr, uint32_t lds_block) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_block) : "memory", "m0");
}

// The same for one 4-byte word per lane (lane l writes LDS bytes [4l, 4l+4) of the block).
__device__ __forceinline__ void copy_to_lds4(const void* gptr, uint32_t lds_block) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gptr), "s"(lds_block) : "memory", "m0");
}

constexpr int kSmemBytes = 160 * 1024;  // LDS of the largest tile shape
constexpr int kRowsBytes = kWaves * 256;  // per wave, 64 row indices of the next tile (see gemm_tile)

// The tile a workgroup runs after this one, when it has the same shape: its first stages
// can then be copied during this tile's last ones (ok), into the buffers it will read them
// from.
struct NextTile {
  bool ok;
  int e, row0, row_end, n0, ks;
};
// The activation copy offsets of a tile whose first stages a previous tile issued (its
// gather indices were read then, so the tile itself issues no load it must wait for).
struct XCarry {
  uint32_t v[4];
};

// One tile of BMT rows (row0 .. row_end-1 of expert e) x BNT weight columns from n0, over
// k in [ks * Kc, ks * Kc + Kc).  SPLIT: the raw fp32 accumulators go to K part ks of
// `out` (row stride NW = 2N for SwiGLU, else N; parts R_max rows apart) and the
// activation is applied when the parts are added.
// pre: the copies of this tile's first NSW - 1 stages are already in flight (issued by the
// previous tile of the workgroup).  nx: the next tile; returns whether its first stages
// were issued here (then the next call gets pre = true).  That happens when the stage
// buffers are one cycle (NSW == NSTAGE) that this tile's stage count fills exactly, so
// the next tile's stage q lands in buffer q % NSW, where its own prologue would put it.
template <int BMT, int ACT, bool GATHER, typename OT, bool SPLIT, int BNT = BN, typename CFG = TileCfg<BMT>>
__device__ __forceinline__ bool gemm_tile(char* smem, const bf16_t* __restrict__ A, const int* __restrict__ a_rows,
                                          const bf16_t* __restrict__ W, const bf16_t* __restrict__ W3, int K,
                                          int N, OT* __restrict__ out, int R_max, int e, int row0, int row_end,
                                          int n0, int ks, int Kc, float* __restrict__ save, bool pre,
                                          const NextTile& nx, XCarry& carry) {
  static_assert(!SPLIT || std::is_same<OT, float>::value, "K-split parts are fp32");
  constexpr int NSTAGE = CFG::NSTAGE, NSW = CFG::NSW, SPREAD = CFG::SPREAD;
  static_assert(NSW == NSTAGE || (NSW == 3 && NSTAGE == 2), "stage counts");
  constexpr int WMW = CFG::WMW, WNW = CFG::WNW;  // waves along m / along n
  constexpr int NCW = WMW * WNW;                                   // waves with MFMA work
  static_assert(NCW <= kWaves, "wave grid");
  constexpr int WTM = BMT / WMW, WTN = BNT / WNW;  // wave tile
  constexpr int WSTT = KB * BNT;                   // weight stage elements: [64 k][BNT n]
  constexpr int CPR = BNT / 8;                     // 16-byte chunks per weight stage row
  constexpr int RPI = 64 / CPR;                    // weight rows per 1 KiB copy (2 or 1)
  constexpr int NIWT = KB / RPI / kWaves;          // weight copies per wave and stage
  constexpr int IB = WTN / 32, JB = WTM / 32;     // 32 x 32 MFMA blocks per wave
  constexpr int XST = BMT * KB;                   // activation stage elements
  constexpr int XI = BMT / 8;                     // activation copies (1 KiB each) per stage
  constexpr int NIX = (XI + kWaves - 1) / kWaves; // ... per wave (waves past XI / NIX have none)
  static_assert(XI % NIX == 0, "activation copies");
  constexpr int ROWS_OFF = (NSW * WSTT + NSTAGE * XST) * 2;  // LDS bytes: the next tile's row indices
  static_assert(ROWS_OFF <= kSmemBytes && (NSW != NSTAGE || ROWS_OFF + kRowsBytes <= kSmemBytes), "LDS");
  static_assert(NIX <= 4, "XCarry");
  bf16_t(*Ws)[WSTT] = reinterpret_cast<bf16_t(*)[WSTT]>(smem);
  bf16_t(*Xs)[XST] = reinterpret_cast<bf16_t(*)[XST]>(smem + NSW * WSTT * 2);

  // An opaque copy of the thread index: the lane-dependent offsets below are then computed
  // per tile instead of being hoisted out of a workgroup's tile loop, where the offsets of
  // every tile shape would hold registers at once.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6;
  const int uwave = __builtin_amdgcn_readfirstlane(wave);
  const bool has_x = XI % kWaves == 0 || NIX * uwave < XI;  // this wave copies activations

  // ---- copy plan.  One wave instruction moves 1 KiB: lane l writes LDS bytes
  // [16l, 16l+16) of the instruction's block, i.e. swizzle slot (l % CPR) of weight
  // row (l / CPR) or slot (l & 7) of activation row (l >> 3); it fetches the global
  // chunk that the swizzle puts there.  Columns past N / rows past the segment fetch
  // a valid neighbour instead (their results are never stored).
  // Weight columns: each wave's WTN LDS columns hold, for SwiGLU, WTN/2 columns of W1
  // followed by the same WTN/2 columns of W3.
  auto plan_w = [&](int e_, int n0_, int ks_, const bf16_t* (&wsrc_)[NIWT]) {
#pragma unroll
    for (int i = 0; i < NIWT; ++i) {
      const int r = RPI * (NIWT * wave + i) + lane / CPR;  // weight stage row (k)
      const int c = (lane % CPR) ^ wswz(r);                // 16-byte chunk of 8 columns
      int col;
      const bf16_t* Wm;
      if (ACT == ACT_SWIGLU) {
        constexpr int CPW = WTN / 8;  // chunks per wave's columns
        const int wg = c / CPW, cc = c % CPW;
        col = n0_ + wg * (WTN / 2) + (cc % (CPW / 2)) * 8;
        Wm = cc < CPW / 2 ? W : W3;
      } else if (ACT == ACT_SWIGLU_SEP) {
        // column n0 + 8c of [W1 | W3] (N a multiple of 8: no chunk straddles the two)
        const int gc = n0_ + c * 8;
        col = gc < N ? gc : gc - N;
        Wm = gc < N ? W : W3;
      } else {
        col = n0_ + c * 8;
        Wm = W;
      }
      wsrc_[i] = Wm + (size_t)e_ * K * N + (size_t)(ks_ * Kc + r) * N + min(col, N - 8);
    }
  };
  // activation row xr of the stage (m) comes from source row src_row
  auto x_off = [&](int i, int src_row, int ks_) -> uint32_t {
    const int xr = 8 * (NIX * wave + i) + lane / XCH;
    return (uint32_t)src_row * (uint32_t)K + (uint32_t)(ks_ * Kc) + (uint32_t)((((lane % XCH) ^ xswz(xr))) << 3);
  };
  const bf16_t* wsrc[NIWT];
  uint32_t xsrc[NIX];
  const bf16_t* wsrc_n[NIWT];  // the next tile's (see below)
  uint32_t xsrc_n[NIX];
  plan_w(e, n0, ks, wsrc);
#pragma unroll
  for (int i = 0; i < NIX; ++i) {
    if (pre) {
      xsrc[i] = carry.v[i];
    } else {
      const int rr = min(row0 + 8 * (NIX * wave + i) + lane / XCH, row_end - 1);
      xsrc[i] = x_off(i, GATHER ? a_rows[rr] : rr, ks);
    }
  }
  // The next tile's first NSW - 1 stages follow this tile's last ones in the same buffers
  // (one cycle of NSW buffers, a whole number of cycles per tile).  At least 2 NSW stages:
  // then the gather indices copied below have landed when the next tile's copies start.
  const int nk = Kc / KB;
  const bool cont = NSW == NSTAGE && nx.ok && nk % NSW == 0 && nk >= 2 * NSW;
  const uint32_t rows_lds = (uint32_t)(uintptr_t)(lds_void_t*)(smem + ROWS_OFF) + 256u * (uint32_t)uwave;
  const uint32_t ws_lds = (uint32_t)(uintptr_t)(lds_void_t*)&Ws[0][0];
  const uint32_t xs_lds = (uint32_t)(uintptr_t)(lds_void_t*)&Xs[0][0];
  // The copies that belong to MFMA group `part` of `parts` (parts == 1: all of them):
  // activation copies of stage xkt into buffer xst (if xkt >= 0), then weight copies of
  // stage wkt into buffer wst (if wkt >= 0).  With equal stage counts, weight copy i and
  // activation copy j go to groups i * sp / NIWT and j * sp / NIX, sp = min(SPREAD, parts);
  // with a deeper weight pipeline the activation copies (needed first) take the first
  // sp/2 groups and the weight copies the next sp.
  // (ALL: both stages are known to exist, no checks)
  // (nxp: the stages xkt / wkt are the next tile's)
  auto issue_part = [&](int xkt, int xst, int wkt, int wst, int part, int parts, bool all = false, bool nxp = false) {
    const int sp = parts < SPREAD ? parts : (SPREAD > 0 ? SPREAD : 1);
    const bool split = NSW != NSTAGE && parts > 1;
#pragma unroll
    for (int i = 0; i < NIX; ++i)
      if ((all || xkt >= 0) && has_x && (split ? i * (sp / 2) / NIX : i * sp / NIX) == part)
        copy_to_lds16(A + (nxp ? xsrc_n[i] : xsrc[i]) + xkt * KB,
                      xs_lds + 2u * (uint32_t)(xst * XST + 8 * (NIX * uwave + i) * KB));
#pragma unroll
    for (int i = 0; i < NIWT; ++i)
      if ((all || wkt >= 0) && (split ? sp / 2 + i * sp / NIWT : i * sp / NIWT) == part)
        copy_to_lds16((nxp ? wsrc_n[i] : wsrc[i]) + (size_t)wkt * KB * N,
                      ws_lds + 2u * (uint32_t)(wst * WSTT + RPI * (NIWT * uwave + i) * BNT));
  };

  // ---- fragment addressing (v_mfma_f32_32x32x16_bf16).  Wave (wn, wm) owns weight
  // columns wn*WTN + [0,WTN) and activation rows wm*WTM + [0,WTM): IB x JB blocks of
  // 32 x 32, four 16-k halves (kh) per stage.
  // Weights (MFMA rows): two transposing 8-byte reads per block and half; in lane group
  // g = lane >> 4, lane s = lane & 15 points at row 16*kh + 8*(g >> 1) + 4*h + (s >> 2),
  // columns 32*ib + 16*(g & 1) + 4*(s & 3) .. +3, and receives k = 16*kh + 8*(g >> 1) +
  // 4*h + 0..3 of column 32*ib + (lane & 31): the MFMA row layout.
  // Activations (MFMA columns): one 16-byte read, row 32*jb + (lane & 31), k-chunk
  // 2*kh + (lane >> 5).
  const int wn = wave % WNW, wm = wave / WNW;
  const int g = lane >> 4, s = lane & 15, l31 = lane & 31, hf = lane >> 5;
  int aoff[KB / 16][2][IB];
#pragma unroll
  for (int kh = 0; kh < KB / 16; ++kh)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 16 * kh + 8 * (g >> 1) + 4 * h + (s >> 2);
#pragma unroll
      for (int ib = 0; ib < IB; ++ib) {
        const int col = wn * WTN + ib * 32 + 16 * (g & 1) + 4 * (s & 3);
        aoff[kh][h][ib] = r * BNT + ((((col >> 3) ^ wswz(r))) << 3) + (col & 7);
      }
    }
  const int xrow = wm * WTM + l31;
  int boff[KB / 16];  // + jb * 32 * KB
#pragma unroll
  for (int kh = 0; kh < KB / 16; ++kh) boff[kh] = xrow * KB + (((2 * kh + hf) ^ xswz(xrow)) << 3);

  floatx16 acc[IB][JB];
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // MFMAs of stage kt; the copies of later stages (see issue_part) are issued in
  // between, one share after each group of JB MFMAs.
  // (xkt, xnb) / (wkt, wnb): the stage whose copies are issued, and its buffer
  auto compute = [&](int xbuf, int wbuf, int xkt, int xnb, int wkt, int wnb, bool all, bool nxp = false) {
    const bf16_t* Wb = Ws[wbuf];
    const bf16_t* Xb = Xs[xbuf];
    constexpr int PARTS = (KB / 16) * IB;
    // every copy must fall in one of the PARTS groups (issue_part's mapping)
    constexpr int SP = PARTS < SPREAD ? PARTS : (SPREAD > 0 ? SPREAD : 1);
    static_assert(SPREAD == 0 || (NSW != NSTAGE
                                      ? SP / 2 + (NIWT - 1) * SP / NIWT < PARTS && (NIX - 1) * (SP / 2) / NIX < SP / 2
                                      : (NIWT - 1) * SP / NIWT < PARTS && (NIX - 1) * SP / NIX < PARTS),
                  "copy groups");
    const bool mf = NCW == kWaves || uwave < NCW;  // waves past the grid only copy
    if (SPREAD == 0) issue_part(xkt, xnb, wkt, wnb, 0, 1, all, nxp);  // all copies before the first LDS read
#pragma unroll
    for (int kh = 0; kh < KB / 16; ++kh) {
      bf16x8 a[IB], b[JB];
      if (mf) {
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) b[jb] = *(const bf16x8*)&Xb[boff[kh] + jb * 32 * KB];
#pragma unroll
        for (int ib = 0; ib < IB; ++ib) {
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)&Wb[aoff[kh][0][ib]]);
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)&Wb[aoff[kh][1][ib]]);
          a[ib] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
#pragma unroll
      for (int ib = 0; ib < IB; ++ib) {
        if (mf) {
#pragma unroll
          for (int jb = 0; jb < JB; ++jb)
            acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ib], b[jb], acc[ib][jb], 0, 0, 0);
        }
        if (SPREAD > 0) issue_part(xkt, xnb, wkt, wnb, kh * IB + ib, PARTS, all, nxp);
      }
    }
  };

  // ---- pipeline: stage kt lives in activation buffer kt % NSTAGE and weight buffer
  // kt % NSW.  During stage kt the activations of stage kt + NSTAGE - 1 and the weights of
  // stage kt + NSW - 1 are copied, into the buffers that the barrier of step kt has
  // released.  Each thread waits for its own copies of stage kt -- newer copies, issued
  // after them, may stay in flight -- then the barrier makes every thread's copies visible.
  if (!pre) {
#pragma unroll
    for (int p = 0; p < NSW - 1; ++p)
      if (p < nk) issue_part(p < NSTAGE - 1 ? p : -1, p, p, p, 0, 1);
  }
  // the next tile's gather indices: lane l copies row index 8 NIX uwave + min(l, 8 NIX - 1)
  // of the next tile (clamped to its last row) into this wave's 256 LDS bytes
  if (GATHER && cont && has_x) {
    const int rr = min(nx.row0 + 8 * NIX * uwave + min(lane, 8 * NIX - 1), nx.row_end - 1);
    copy_to_lds4(a_rows + rr, rows_lds);
  }
  // Steady state: U = lcm(NSTAGE, NSW) stages per iteration, so every buffer index is a
  // constant, and every copy of these stages exists.
  constexpr int U = NSW == NSTAGE ? NSW : NSW * NSTAGE;
  // stage kt's copies have landed when at most the newer stages' copies are in flight
  auto wait_steady = [&]() {
    if (NSW == NSTAGE) {
      if (NSTAGE >= 4) {
        if (has_x) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (NIWT + NIX)) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NIWT) : "memory");
      } else if (NSTAGE == 3) {
        if (has_x) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NIWT + NIX) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NIWT) : "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
    } else {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NIWT) : "memory");
    }
  };
  int kt = 0;
  for (; kt + U + NSW - 2 < nk; kt += U) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      wait_steady();
      __syncthreads();
      compute(j % NSTAGE, j % NSW, kt + j + NSTAGE - 1, (j + NSTAGE - 1) % NSTAGE, kt + j + NSW - 1,
              (j + NSW - 1) % NSW, true);
    }
  }
  if (NSW == NSTAGE && cont) {
    // The last NSW stages (kt = nk - NSW + j, buffer j): the first issues this tile's last
    // stage, the others the next tile's stages 0 .. NSW - 2, into buffers 0 .. NSW - 2.
    // The wait stays the steady one: NSW - 2 stages, of either tile, stay in flight.
#pragma unroll
    for (int j = 0; j < NSW; ++j) {
      wait_steady();
      __syncthreads();
      if (j == 0) {
        compute(0, 0, nk - 1, NSW - 1, nk - 1, NSW - 1, true);
      } else {
        if (j == 1) {
          plan_w(nx.e, nx.n0, nx.ks, wsrc_n);
          const int* rw = reinterpret_cast<const int*>(smem + ROWS_OFF + 256 * uwave);
#pragma unroll
          for (int i = 0; i < NIX; ++i) {
            int src;
            if (GATHER) src = rw[8 * i + lane / XCH];
            else src = min(nx.row0 + 8 * (NIX * wave + i) + lane / XCH, nx.row_end - 1);
            xsrc_n[i] = x_off(i, src, nx.ks);
            carry.v[i] = xsrc_n[i];
          }
        }
        compute(j, j, j - 1, j - 1, j - 1, j - 1, true, true);
      }
    }
    kt = nk;
  }
  // the remaining stages (the pipeline drains)
  for (; kt < nk; ++kt) {
    if (NSW == NSTAGE) {
      // stages newer than kt already issued, NIWT (+ NIX) copies each
      const int ahead = min(nk - 1 - kt, NSTAGE - 2);
      if (has_x) {
        if (ahead >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (NIWT + NIX)) : "memory");
        else if (ahead == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NIWT + NIX) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else {
        if (ahead >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NIWT) : "memory");
        else if (ahead == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NIWT) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
    } else {
      // the newest copies are the weights of stage kt + 1 (issued after the activations
      // of stage kt during step kt - 1, or in the prologue)
      if (kt + 1 < nk) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NIWT) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    const int xkt = kt + NSTAGE - 1 < nk ? kt + NSTAGE - 1 : -1;
    const int wkt = kt + NSW - 1 < nk ? kt + NSW - 1 : -1;
    compute(kt % NSTAGE, kt % NSW, xkt, xkt % NSTAGE, wkt, wkt % NSW, false);
  }

  // ---- epilogue: lane holds token row 32*jb + (lane & 31) and, for acc element
  // 4q+p, weight column 32*ib + 8q + 4*(lane >> 5) + p of its wave's columns.
  if (NCW < kWaves && uwave >= NCW) return cont;
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) {
    const int r = row0 + wm * WTM + jb * 32 + l31;
    if (r >= row_end) continue;
    if (SPLIT) {
      constexpr int NWM = ACT == ACT_SWIGLU ? 2 : 1;               // W1 | W3 halves in a tile
      constexpr int RW = ACT == ACT_SWIGLU || ACT == ACT_SWIGLU_SEP ? 2 : 1;  // row width / N
      constexpr int NC = ACT == ACT_SWIGLU_SEP ? 2 : 1;            // column bound / N
      OT* prow = out + ((size_t)ks * R_max + r) * (size_t)(RW * N);
#pragma unroll
      for (int ib = 0; ib < IB / NWM; ++ib)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn * (WTN / NWM) + ib * 32 + 8 * q + 4 * hf;
          if (col >= NC * N) continue;
          float v[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) v[p] = acc[ib][jb][4 * q + p];
          store4(prow + col, v);
          if (NWM == 2) {
#pragma unroll
            for (int p = 0; p < 4; ++p) v[p] = acc[ib + IB / 2][jb][4 * q + p];
            store4(prow + N + col, v);
          }
        }
      continue;
    }
    OT* orow = out + (size_t)r * N;
    if (ACT == ACT_SWIGLU) {
#pragma unroll
      for (int ib = 0; ib < IB / 2; ++ib)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn * (WTN / 2) + ib * 32 + 8 * q + 4 * hf;
          if (col >= N) continue;
          float v[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) v[p] = silu_fast(acc[ib][jb][4 * q + p]) * acc[ib + IB / 2][jb][4 * q + p];
          store4(orow + col, v);
          if (save != nullptr) {  // the pre-activations a | g, as the raw layout holds them
            float* srow = save + (size_t)r * 2 * N;
            float a4[4], g4[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              a4[p] = acc[ib][jb][4 * q + p];
              g4[p] = acc[ib + IB / 2][jb][4 * q + p];
            }
            store4(srow + col, a4);
            store4(srow + N + col, g4);
          }
        }
    } else {
#pragma unroll
      for (int ib = 0; ib < IB; ++ib)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn * WTN + ib * 32 + 8 * q + 4 * hf;
          if (col >= N) continue;
          float v[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const float z = acc[ib][jb][4 * q + p];
            v[p] = ACT == ACT_GELU ? gelu_erf(z) : z;
          }
          store4(orow + col, v);
          if (ACT == ACT_GELU && save != nullptr) {
            float a4[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) a4[p] = acc[ib][jb][4 * q + p];
            store4(save + (size_t)r * N + col, a4);
          }
        }
    }
  }
  return cont;
}

// The grouped GEMM over all experts in one launch.  The tile list (device-side
// tile_off, built with fh rows per m-tile) and the XCD-aware order give each workgroup
// an (expert, m-tile, n-tile[, K part]); the tile's code path is chosen by the rows it
// really has: an expert's last m-tile with few rows runs the 128- or 32-row shape
// instead of computing on padding.
template <int ACT, bool GATHER, typename OT, bool SPLIT>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4))) void
gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const int* __restrict__ a_rows, const bf16_t* __restrict__ W,
    const bf16_t* __restrict__ W3, int K, int N, OT* __restrict__ out, const int* __restrict__ offsets,
    const int* __restrict__ tile_off, int E, int NT, int S, int R_max, int fh, int big, float* __restrict__ save,
    int order) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  constexpr int NO = ACT == ACT_SWIGLU ? BN / 2 : BN;  // output columns per tile
  // ---- tile schedule (see TileOrder)
  const int nslot = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  // kOrderNRange: XCD x's list is that of a launch of its NTl n-tiles x, x + 8, x + 16, ...
  const bool nr = order == kOrderNRange;
  const int NTl = nr ? (NT - xcd + 7) / 8 : NT;
  const int n_tiles = ldc(tile_off, E) * NTl;
  const int n_real = n_tiles * (SPLIT ? S : 1);
  int L, Lend, step, gmx = GM;
  if (order == kOrderLaunch) {
    L = blockIdx.x;
    Lend = n_real;
    step = gridDim.x;
    gmx = 1;
  } else if (nr) {
    L = slot;
    Lend = n_real;
    step = nslot;
  } else {
    const int per = (n_real + 7) >> 3;
    L = xcd * per + slot;
    Lend = min((xcd + 1) * per, n_real);
    step = nslot;
  }
  if (L >= Lend) return;
  const int Kc = SPLIT ? K / S : K;  // each tile's k range: [ks * Kc, ks * Kc + Kc)
  // the tile's code path is chosen by the rows it really has
  auto shape = [](int rows) { return rows > 128 ? 2 : (rows > 32 ? 1 : 0); };
  TileInfo cur = tile_at(L, tile_off, offsets, E, NTl, n_tiles, SPLIT, fh, big, NO, 0, gmx);
  if (nr) cur.n0 = cur.n0 * 8 + xcd * NO;
  bool pre = false, first = true;
  XCarry carry;
  for (;;) {
    const int Ln = L + step;
    const bool more = Ln < Lend;
    TileInfo nxt = cur;
    if (more) {
      const bool same_part = !SPLIT || Ln / n_tiles == cur.ks;  // list positions only grow inside a part
      nxt = tile_at(Ln, tile_off, offsets, E, NTl, n_tiles, SPLIT, fh, big, NO, same_part ? cur.e : 0, gmx);
      if (nr) nxt.n0 = nxt.n0 * 8 + xcd * NO;
    }
    const int sh = shape(cur.rows);
    const NextTile nx{more && shape(nxt.rows) == sh, nxt.e, nxt.row0, nxt.row0 + nxt.rows, nxt.n0, nxt.ks};
    // a tile that starts its own copies waits until every wave is done with the buffers
    if (!pre && !first) __syncthreads();
    if (sh == 2)
      pre = gemm_tile<256, ACT, GATHER, OT, SPLIT>(smem, A, a_rows, W, W3, K, N, out, R_max, cur.e, cur.row0,
                                                   cur.row0 + cur.rows, cur.n0, cur.ks, Kc, save, pre, nx, carry);
    else if (sh == 1)
      pre = gemm_tile<128, ACT, GATHER, OT, SPLIT>(smem, A, a_rows, W, W3, K, N, out, R_max, cur.e, cur.row0,
                                                   cur.row0 + cur.rows, cur.n0, cur.ks, Kc, save, pre, nx, carry);
    else
      pre = gemm_tile<32, ACT, GATHER, OT, SPLIT>(smem, A, a_rows, W, W3, K, N, out, R_max, cur.e, cur.row0,
                                                  cur.row0 + cur.rows, cur.n0, cur.ks, Kc, save, pre, nx, carry);
    if (!more) break;
    first = false;
    L = Ln;
    cur = nxt;
  }
}

// The same grouped GEMM when every m-tile has at most 32 rows (fh = 32): wide tiles.
template <int ACT, bool GATHER, typename OT, bool SPLIT>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4))) void
gemm_bf16_wide_kernel(
    const bf16_t* __restrict__ A, const int* __restrict__ a_rows, const bf16_t* __restrict__ W,
    const bf16_t* __restrict__ W3, int K, int N, OT* __restrict__ out, const int* __restrict__ offsets,
    const int* __restrict__ tile_off, int E, int NT, int S, int R_max, int fh, int big, float* __restrict__ save) {
  // K parts: spread copies and the XCD-aware order; one part (the up projection, also
  // its separated raw form): copies after the barrier and launch order
  constexpr bool KP = SPLIT && ACT != ACT_SWIGLU_SEP;
  using CFG = TileCfgWide32<KP>;
  constexpr int LDS = (CFG::NSW * KB * BNW + CFG::NSTAGE * 32 * KB) * 2 + kRowsBytes;
  __shared__ __attribute__((aligned(1024))) char smem[LDS];
  constexpr int NO = ACT == ACT_SWIGLU ? BNW / 2 : BNW;  // output columns per tile
  const int n_tiles = ldc(tile_off, E) * NT;
  const int n_real = n_tiles * (SPLIT ? S : 1);
  int L, Lend, step;
  if (KP) {
    const int per = (n_real + 7) >> 3;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    L = xcd * per + slot;
    Lend = min((xcd + 1) * per, n_real);
    step = gridDim.x >> 3;
  } else {
    L = blockIdx.x;
    Lend = n_real;
    step = gridDim.x;
  }
  if (L >= Lend) return;
  const int Kc = SPLIT ? K / S : K;
  // fh is 32 here: every tile is 32 rows
  TileInfo cur = tile_at(L, tile_off, offsets, E, NT, n_tiles, SPLIT, fh, big, NO, 0);
  bool pre = false, first = true;
  XCarry carry;
  for (;;) {
    const int Ln = L + step;
    const bool more = Ln < Lend;
    TileInfo nxt = cur;
    if (more) {
      const bool same_part = !SPLIT || Ln / n_tiles == cur.ks;
      nxt = tile_at(Ln, tile_off, offsets, E, NT, n_tiles, SPLIT, fh, big, NO, same_part ? cur.e : 0);
    }
    const NextTile nx{more, nxt.e, nxt.row0, nxt.row0 + nxt.rows, nxt.n0, nxt.ks};
    if (!pre && !first) __syncthreads();
    pre = gemm_tile<32, ACT, GATHER, OT, SPLIT, BNW, CFG>(smem, A, a_rows, W, W3, K, N, out, R_max, cur.e, cur.row0,
                                                          cur.row0 + cur.rows, cur.n0, cur.ks, Kc, save, pre, nx,
                                                          carry);
    if (!more) break;
    first = false;
    L = Ln;
    cur = nxt;
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

// Workgroups of a bf16 GEMM launch.  By default one per tile slot, and the hardware hands
// tiles to CUs as they free up.  Launches of short tiles (a contraction of at most
// kPersistStages LDS stages per tile) instead start only as many workgroups as run at once
// (one per CU: each takes most of its LDS), rounded up to a multiple of 8 for the XCD-aware
// order; each runs its share of the tile list in turn and copies a tile's first stages
// during the previous tile's last ones.  (Measured at T = 8192, h = 1024, f = 4096,
// E = 64, k = 2, capacity 320: the up projection, 16 stages per tile, 143.5 -> 137.9 us;
// with 64 stages per tile -- T = 4096, h = 4096, f = 2048, E = 256, k = 8 -- the fixed
// schedule was slower than the hardware's, 1816 -> 1926 us, and it gained nothing on
// 256-row tiles.)  MOE_GEMM_WORKGROUPS (environment) sets the count for every launch;
// the results do not depend on it.
constexpr int kPersistStages = 16;
long long gemm_workgroups(long long slots, int stages) {
  if (const char* v = getenv("MOE_GEMM_WORKGROUPS")) {
    const long n = strtol(v, nullptr, 10);
    if (n > 0 && n <= (1L << 20)) return std::min(slots, (long long)(n + 7) / 8 * 8);
  }
  if (stages > kPersistStages) return slots;
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      n = 256;
    return n > 0 ? n : 256;
  }();
  return std::min(slots, (long long)(cus + 7) / 8 * 8);
}

// The tile order of a launch of m-tiles bm rows high and NT n-tiles (down: the output is
// the raw product): n-ranges for 256-row tiles over a multiple of 8 n-tiles, launch order
// for the down projections of 128-row tiles, else ranges.  MOE_GEMM_ORDER (environment:
// 0, 1 or 2) sets it for every launch; the results do not depend on it.
int tile_order(int bm, int NT, bool down) {
  if (const char* v = getenv("MOE_GEMM_ORDER")) {
    const long m = strtol(v, nullptr, 10);
    if (m >= kOrderRanges && m <= kOrderNRange) return (int)m;
  }
  if (bm == 256 && NT % 8 == 0) return kOrderNRange;
  if (bm == 128 && down) return kOrderLaunch;
  return kOrderRanges;
}

template <int ACT, bool G, typename OT, bool SPLIT>
hipError_t launch_bf16_k(const GemmArgs& a, hipStream_t st) {
  const bool wide = a.bm == 32;
  const int NO = ACT == ACT_SWIGLU ? (wide ? BNW : BN) / 2 : (wide ? BNW : BN);
  const int NT = ((ACT == ACT_SWIGLU_SEP ? 2 * a.N : a.N) + NO - 1) / NO;
  const int S = SPLIT ? std::max(a.ksplit, 1) : 1;
  const int order = wide ? kOrderRanges : tile_order(a.bm, NT, ACT == ACT_NONE);
  // (kOrderNRange: every XCD has slots for its ceil(NT / 8) n-tiles of every m-tile)
  const long long slots =
      ((long long)(a.R_max + a.bm - 1) / a.bm + a.E) * (order == kOrderNRange ? (NT + 7) / 8 * 8 : NT) * S;
  const long long grid = gemm_workgroups((slots + 7) / 8 * 8, a.K / S / KB);
  if (grid <= 0) return hipSuccess;
  float* save = SPLIT ? nullptr : a.save;
  if (wide)
    hipLaunchKernelGGL((gemm_bf16_wide_kernel<ACT, G, OT, SPLIT>), dim3((unsigned)grid), dim3(kWaves * 64), 0, st,
                       (const bf16_t*)a.A, a.a_rows, (const bf16_t*)a.W, (const bf16_t*)a.W3, a.K, a.N,
                       (OT*)a.out, a.offsets, a.tile_off, a.E, NT, S, a.R_max, a.bm, a.big, save);
  else if constexpr (ACT == ACT_SWIGLU_SEP)
    return hipErrorInvalidValue;  // wide tiles only
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<ACT, G, OT, SPLIT>), dim3((unsigned)grid), dim3(kWaves * 64), 0, st,
                       (const bf16_t*)a.A, a.a_rows, (const bf16_t*)a.W, (const bf16_t*)a.W3, a.K, a.N,
                       (OT*)a.out, a.offsets, a.tile_off, a.E, NT, S, a.R_max, a.bm, a.big, save, order);
  return hipGetLastError();
}

template <int ACT, bool G, typename OT>
hipError_t launch_bf16_t(const GemmArgs& a, hipStream_t st) {
  if (a.bm != 256 && a.bm != 128 && a.bm != 32) return hipErrorInvalidValue;
  // pre-activations are saved by the epilogue of a one-part up projection only
  if (a.save != nullptr && (a.ksplit > 1 || a.raw || ACT == ACT_NONE)) return hipErrorInvalidValue;
  if (a.sep) {  // raw SwiGLU pre-activations in 512-column tiles of W1 or W3 alone
    if (ACT != ACT_SWIGLU || !a.raw || a.ksplit > 1 || a.bm != 32 || a.N % 8 != 0) return hipErrorInvalidValue;
    return launch_bf16_k<ACT_SWIGLU_SEP, G, float, true>(a, st);
  }
  if (a.ksplit > 1 || a.raw) {
    // K parts: for few rows per expert, where there are too few tiles to fill the chip
    // (or one part of raw accumulators)
    if (a.K % (std::max(a.ksplit, 1) * KB) != 0) return hipErrorInvalidValue;
    constexpr int PA = ACT == ACT_SWIGLU ? ACT_SWIGLU : ACT_NONE;  // part layout
    return launch_bf16_k<PA, G, float, true>(a, st);
  }
  return launch_bf16_k<ACT, G, OT, false>(a, st);
}

// Adds the K parts of a split GEMM in ascending order and applies the activation.
template <int ACT, typename OT>
__global__ __launch_bounds__(256) void ffn_finish_kernel(const float* __restrict__ part, int S, int R_max, int N,
                                                         const int* __restrict__ offsets, int E,
                                                         OT* __restrict__ out, float* __restrict__ save) {
  const int R = offsets[E];
  const int groups = N >> 2;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)R * groups) return;
  const int r = (int)(gid / groups);
  const int c = (int)(gid % groups) * 4;
  constexpr int NWM = ACT == ACT_SWIGLU ? 2 : 1;
  const size_t stride = (size_t)R_max * NWM * N;
  const float* p = part + (size_t)r * NWM * N + c;
  floatx4 a = *(const floatx4*)p, g = floatx4{0.f, 0.f, 0.f, 0.f};
  if (NWM == 2) g = *(const floatx4*)(p + N);
  for (int s = 1; s < S; ++s) {
    a += *(const floatx4*)(p + s * stride);
    if (NWM == 2) g += *(const floatx4*)(p + s * stride + N);
  }
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = ACT == ACT_SWIGLU ? silu_fast(a[i]) * g[i] : (ACT == ACT_GELU ? gelu_erf(a[i]) : a[i]);
  store4(out + (size_t)r * N + c, v);
  if (ACT != ACT_NONE && save != nullptr) {  // the summed pre-activations, in the raw layout
    *(floatx4*)(save + (size_t)r * NWM * N + c) = a;
    if (NWM == 2) *(floatx4*)(save + (size_t)r * NWM * N + N + c) = g;
  }
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

hipError_t launch_ffn_finish(const float* part, int S, int R_max, int N, int act, const int* offsets, int E,
                             bool out_bf16, void* out, hipStream_t st, float* save) {
  // grid over the row bound; rows past offsets[E] exit
  const int64_t n = (int64_t)R_max * (N / 4);
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (grid == 0) return hipSuccess;
#define MOE_FIN(A, OT)                                                                              \
  hipLaunchKernelGGL((ffn_finish_kernel<A, OT>), dim3(grid), dim3(256), 0, st, part, S, R_max, N, offsets, E, \
                     (OT*)out, save)
  switch (act) {
    case ACT_NONE: if (out_bf16) MOE_FIN(ACT_NONE, bf16_t); else MOE_FIN(ACT_NONE, float); break;
    case ACT_GELU: if (out_bf16) MOE_FIN(ACT_GELU, bf16_t); else MOE_FIN(ACT_GELU, float); break;
    case ACT_SWIGLU: if (out_bf16) MOE_FIN(ACT_SWIGLU, bf16_t); else MOE_FIN(ACT_SWIGLU, float); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_FIN
  return hipGetLastError();
}

FfnPlan plan_ffn(bool bf16, double rows_per_expert, int E, int R_max, int h, int f) {
  FfnPlan p{gemm_bm(bf16, rows_per_expert), 1, 1, INT_MAX};
  if (!bf16) return p;
  if (p.bm == 128) {
    // Experts with many rows take 256-row tiles.  Four 128-row m-tiles of an expert run
    // together on one XCD and share its weight panels in L2, so an expert with more rows
    // streams its weights from HBM once per group of four: from 512 rows, 256-row tiles halve
    // those re-reads.  With a long up-projection contraction (h >= 2048) every expert past
    // one 128-row tile is better off with 256-row tiles (fewer tiles, one weight stream per
    // expert; measured at T = 4096, h = 4096, f = 2048, E = 256, k = 8: the up projection
    // 1.86 -> 1.73 ms); with h = 1024 (T = 8192, f = 4096, E = 64, k = 2, capacity 320)
    // 256-row tiles for its 320-row experts made the up projection 0.148 -> 0.194 ms.
    p.big = h >= 2048 ? 129 : 512;
  }
  constexpr double kCUs = 256.0;
  const double mt_max = ceil((double)R_max / p.bm) + E;
  if (p.bm == 32) {
    // Few rows per expert: the GEMMs stream weights, in wide tiles with one workgroup per
    // CU.  When there are fewer tiles than CUs (one 512-column tile per expert and column
    // block: the down projection at decode shapes), split K until there is about one per
    // CU; the fp32 parts are added by the combine.
    const double mt = std::min((double)E * ceil(rows_per_expert / p.bm), mt_max);  // expected m-tiles
    auto split = [&](int K, int N, int no) {
      const double tiles = mt * ceil((double)N / no);
      int S = 1;
      if (tiles >= kCUs) return S;
      while (S < 16 && tiles * S < kCUs && K % (2 * S * KB) == 0 && K / (2 * S) >= 8 * KB) S *= 2;
      return S;
    };
    p.s_up = split(h, f, BNW / 2);
    p.s_down = split(f, h, BNW);
    return p;
  }
  // Larger tiles: the last round of tiles may leave many CUs idle (the down projection
  // has only h/256 column blocks per m-tile).  Expected m-tiles: half a tile of padding
  // per expert on top of the rows.  Split the down projection's K in two when that
  // fills the last round markedly better; its two fp32 parts are added by the combine.
  const double mt = std::min((double)E * (rows_per_expert / p.bm + 0.5), mt_max);
  auto fill = [&](double tiles) {
    const double r = tiles / kCUs;
    return r / ceil(r);
  };
  const double tiles_down = mt * ceil((double)h / BN);
  if (f % (2 * KB) == 0 && f / 2 >= 16 * KB && fill(2 * tiles_down) > fill(tiles_down) + 0.08) p.s_down = 2;
  return p;
}

int gemm_bm(bool bf16, double rows_per_expert) {
  if (!bf16) return FBM;
  // (wide 32-row tiles up to 320 rows per expert measured slower at T = 8192, h = 1024,
  // f = 4096, E = 64: up 147 -> 175-192 us, down 121 -> 208-212 us)
  if (rows_per_expert <= 48.0) return 32;
  if (rows_per_expert <= 320.0) return 128;
  return 256;
}

hipError_t launch_gemm(const GemmArgs& a, bool bf16, hipStream_t st) {
  if (bf16) return a.a_rows ? dispatch_act<true, true>(a, st) : dispatch_act<true, false>(a, st);
  return a.a_rows ? dispatch_act<false, true>(a, st) : dispatch_act<false, false>(a, st);
}

}  // namespace moe
