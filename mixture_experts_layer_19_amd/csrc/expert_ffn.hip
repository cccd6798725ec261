// Expert FFN over ragged per-expert slices as grouped GEMMs ("Mixture of Experts: routing,
// sorted dispatch, Switch aux loss, aux-free bias" (L7.8) §2.2: each expert runs once on its
// contiguous slice; "15. Mixture of Experts" (RustingBrain) "Dropless": ragged batches).
//
//   up:   h = gelu(x_s W1^T + b1)              (GELU MLP, optional bias)
//         h = silu(x_s W1^T) * (x_s W3^T)      (SwiGLU; gate and up computed by the same
//                                                workgroup for the same columns, fused)
//   down: y_s = (h W2^T + b2) * gate_sorted    (gate applied before the single rounding)
//
// The m-tiles of every expert are listed once per call by tile_table_kernel from offsets,
// so the GEMM grids are sized from the worst case on the host and idle experts cost
// nothing: they own no tile and their weights are never read.
#include <atomic>
#include <algorithm>
#include <type_traits>

#include "moe_internal.h"

namespace moe {

enum Epi {
  kEpiGelu = 0,
  kEpiSwiglu = 1,
  kEpiDown = 2,
  // backward recompute of the up projection: also keep the pre-activations (c2) and write
  // the gate-scaled hidden activations w_a h_a (c)
  kEpiSwigluSave = 3,
  kEpiGeluSave = 4,
};
template <int EPI> constexpr bool kSwi = EPI == kEpiSwiglu || EPI == kEpiSwigluSave;
template <int EPI> constexpr bool kSave = EPI == kEpiSwigluSave || EPI == kEpiGeluSave;

// Tile table (layout and clamping: build_tile_table) from offsets; a bad offsets array sets
// the error word to MOE_ERR_INVALID_ARG and is otherwise clamped, so no access leaves the
// buffers.
__global__ __launch_bounds__(1024) void tile_table_kernel(const int* __restrict__ offsets, int E, int rows,
                                                          int bm, int narrow, int max_tiles, int* __restrict__ tiles,
                                                          int* __restrict__ err) {
  __shared__ int s_scan[kMaxExperts];
  __shared__ int s_bad;
  const int e = threadIdx.x;
  if (e == 0) s_bad = 0;
  __syncthreads();
  const int lo = e < E ? offsets[e] : 0;
  const int hi = e < E ? offsets[e + 1] : 0;
  build_tile_table(lo, hi, E, rows, bm, narrow, max_tiles, tiles, s_scan, &s_bad);
  if (e == 0 && s_bad && err) err[0] = MOE_ERR_INVALID_ARG;
}

struct GemmArgs {
  const void* a;        // [rows][K] T: x_sorted (up) or h (down)
  const void* b0;       // [E][N_b][K] T: W1 (up) or W2 (down)
  const void* b1;       // [E][N_b][K] T: W3 (SwiGLU up) or null
  const void* bias;     // [E][N_out] T or null
  const float* gate;    // [rows] or null (down only)
  void* c;              // [rows][N_out] T: h (up) or y_sorted (down); save: w_a h_a
  void* c2;             // save only: SwiGLU [rows][2 N_out] (gate | up pre-activations),
                        // GELU [rows][N_out] (pre-activation with b1)
  const int* tiles;     // tile table
  float* partial;       // down projection's tail: [kMaxTailItems][256][256] float32 partials
  int K, n_out;         // reduction length; output columns (= rows of each B matrix)
  int n_tiles_n;        // output column tiles
  int grid;             // tail_reduce_kernel: the GEMM launches' grid
  int pre_gated;        // down: a = gate * h already, so y = a W2^T + gate * b2
  int b_kp, b_np;       // B tiled (MOE_WEIGHTS_TILED): padded K and rows per expert; 0: row-major
  int a_kp;             // A tiled like h below (its padded K); 0: row-major
  int c_kp;             // the up projection writes h tiled: 128-row blocks of 32-column slabs,
                        // row pitch c_kp (n_out rounded up to 32); 0: row-major
  int nar_ok;           // the launch's kernel runs narrow tiles where the table lists them
                        // (set by launch_bf16_gemm; read by tail_reduce_kernel, so that it
                        // numbers the tail items exactly as the GEMM launches did)
};

// ---------------------------------------------------------------------------------------
// bfloat16 grouped GEMM on MFMA (v_mfma_f32_32x32x16_bf16), float32 accumulation.
//
// Two tile shapes, both 8 waves = 2 per SIMD with 128 rows x 64 B-rows per wave (4 x 2
// blocks of 32 x 32, 128 accumulators per lane):
//   full:   256 rows x 256 B-rows (waves 2 x 4), for m-tiles of more than 128 rows;
//   narrow: 128 rows x 512 B-rows (waves 1 x 8), for an expert's last m-tile of at most 128
//           rows, which a full tile would compute with half or more of its rows empty.
// GELU / down: one output column per B-row. SwiGLU: each wave's 64 B-rows are 32 gate rows
// then the 32 up rows of the same columns, so the gate and up value of an output land in the
// same lane and the activation is applied in registers (half as many output columns).
//
// Operands stream through LDS stages of 32 reduction elements written by
// global_load_lds_dwordx4 (memory straight to LDS, no VGPR staging): five stages of
// A 16 KiB + B 16 KiB (full) or four of A 8 KiB + B 32 KiB (narrow), all 160 KiB of the CU's
// LDS. The four 16-byte chunks of a 64-byte LDS row are XOR-swizzled by (row >> 2) mod 4, so
// the 16 rows one 256-byte LDS cycle of a 16-byte operand read serves (rows r .. r+15 at one
// logical chunk) fall in 16 distinct bank slots.
//
// Ping-pong: the waves form two groups offset by half a step. In every phase one group's
// wave on a SIMD issues its 16 multiplies (with the LDS refill copies spread between them)
// while the other group's wave reads the next slab's operands from LDS, then a barrier swaps
// the roles; so the MFMA pipe is fed by one wave while the other's LDS latency is hidden, and
// the copies are issued from the wave whose MFMAs keep the pipe busy meanwhile. With S
// stages:
//   phase 2k:   group 0 multiplies slab k, refills slab k+S-1   group 1 reads slab k
//   phase 2k+1: group 0 reads slab k+1          group 1 multiplies slab k, refills slab k+S
// Each wave issues C copies per refill (full 2 + 2, narrow 1 + 4 of A + B) and keeps S - 2
// refills in flight, so at every phase boundary `vmcnt((S - 2) C)` guarantees that the next
// slab to be read has landed for every wave. Refills past the last slab copy the last slab
// again into a stage that is never read, which keeps that count exact.
//
// Scheduling: a persistent grid of one workgroup per CU. The work sequence is split into 8
// contiguous chunks, one per XCD (workgroup i runs on XCD i mod 8), so tiles that share
// operands share an L2. Within an expert, full tiles are ordered in supertiles of 8 m-tiles x
// 4 n-tiles (m fastest), so the ~32 tiles an XCD runs at once reuse 8 A and 4 B slices. A
// narrow tile reads its expert's whole B on its own, so the narrow items are spread evenly
// through the sequence (decode_tile): every XCD runs its share of them, interleaved in time
// with full tiles, and their weight reads overlap the full tiles' compute.
// Rows past an expert's slice and columns past N are clamped to a valid row (their results
// are never stored); reduction chunks past K are loaded from inside the row and zeroed in
// LDS once they have landed.
// ---------------------------------------------------------------------------------------
constexpr int kBM = 256, kBNB = 256, kBK = 32;
constexpr int kStageElems = kBM * kBK;  // bf16 elements of one 16 KiB LDS array
constexpr int kGemmThreads = 512;

// lds_dma16, wait_vm_lds and stage_barrier: moe_common.h

// The launch's work items and the operand addresses: gemm_sched.h.

// A wave's share of a tile's operand copies into the LDS stages (full or narrow shape):
// stage j holds A at sa(j) and B at sb(j); copy instruction i of the wave fills 16 rows of a
// stage, lane l writing row (l >> 2) of them at physical chunk l & 3, which holds the logical
// chunk (l & 3) ^ ((row >> 2) & 3) = (l & 3) ^ ((l >> 4) & 3).
template <int EPI, int NAR>
struct TileLoads {
  static constexpr int TBM = NAR ? 128 : 256;           // tile rows
  static constexpr int TBN = NAR ? 512 : 256;           // tile B-rows
  static constexpr int CA = TBM / 128, CB = TBN / 128;  // copies of A / B per wave and slab
  static constexpr int CPR = CA + CB;                   // copies per refill
  static_assert(CA <= 4 && CB <= 4, "a copy group holds at most four copies");
  static constexpr int kCols = kSwi<EPI> ? TBN / 2 : TBN;  // output columns per tile
  // uniform bases (bytes) and 32-bit per-lane offsets of the wave's A and B copies of a tile
  struct Src {
    const char* a;
    const char* b[CB];
    uint32_t ao[CA], bo[CB];
  };
  const GemmArgs& g;
  uint16_t* smem;
  int wave, lrow, lchunk;
  MOE_DEV TileLoads(const GemmArgs& g_, uint16_t* smem_, int wave_, int lane)
      : g(g_), smem(smem_), wave(wave_), lrow(lane >> 2), lchunk(((lane & 3) ^ ((lane >> 4) & 3)) * 8) {}
  MOE_DEV uint16_t* sa(int j) const {
    return NAR ? smem + 8 * kStageElems + j * (kStageElems / 2) : smem + 2 * j * kStageElems;
  }
  MOE_DEV uint16_t* sb(int j) const { return NAR ? smem + 2 * j * kStageElems : smem + (2 * j + 1) * kStageElems; }
  MOE_DEV Src src(int e, int row0, int rows, int nt) const {
    const int K = g.K, n_out = g.n_out, n0 = nt * kCols;
    // B row pitch (row-major: K; tiled: the padded K) and rows per expert; n0 is a multiple
    // of 128, so a tile's B rows start a tiled block
    const bool tiled = g.b_kp > 0;
    const int Kb = tiled ? g.b_kp : K;
    const size_t b_off = ((size_t)e * (tiled ? g.b_np : n_out) + n0) * Kb * 2;
    // tiled A: offsets from the 128-row block holding row0 (rows are those of the whole A)
    const bool a_tiled = a_is_tiled();
    const int rb = row0 & ~(kTiledRows - 1);
    Src r;
    r.a = static_cast<const char*>(g.a) + (a_tiled ? (size_t)rb * g.a_kp * 2 : (size_t)row0 * K * 2);
    const char* b0_base = static_cast<const char*>(g.b0) + b_off;
    const char* b1_base = kSwi<EPI> ? static_cast<const char*>(g.b1) + b_off : b0_base;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int rr = (wave * CA + i) * 16 + lrow;  // stage row 0 .. TBM-1
      const int rc = min(rr, rows - 1);
      const int rel = row0 - rb + rc;  // tiled: row within the blocks from rb
      r.ao[i] = (a_tiled ? tiled_row_off(rel, g.a_kp, lchunk) : rm_row_off(rc, K, lchunk)) + (uint32_t)(3 - i) * 1024u;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int rr = (wave * CB + i) * 16 + lrow;  // B-row 0 .. TBN-1
      int cl;  // B-row's output column relative to n0
      if (kSwi<EPI>) {
        // B-rows 64 c .. 64 c + 31: gate of columns 32 c ..; the next 32: up of the same
        cl = (rr >> 6) * 32 + (rr & 31);
        r.b[i] = ((((wave * CB + i) * 16) & 63) >= 32) ? b1_base : b0_base;  // uniform per copy
      } else {
        cl = rr;
        r.b[i] = b0_base;
      }
      cl = min(cl, n_out - 1 - n0);
      // tiled: block cl / 128, row cl % 128 of its 32-element slab rows (the slab offset
      // is added per copy)
      r.bo[i] = (tiled ? tiled_row_off(cl, Kb, lchunk) : rm_row_off(cl, K, lchunk)) + (uint32_t)(3 - i) * 1024u;
    }
    return r;
  }
  // byte offset of reduction index k0 (a multiple of 32) in a tiled operand: slab k0 / 32 of
  // a block (128 x 32 elements each); lanes past K read the padding (zeroed in LDS later)
  MOE_DEV uint32_t dma_kt(int k0) const { return tiled_k_off(k0); }
  // A may be tiled (h for the down projection, moe_forward's x_sorted for the up one); the
  // save epilogues of the training path keep it row-major
  MOE_DEV bool a_is_tiled() const { return !kSave<EPI> && g.a_kp > 0; }
  // byte offset of reduction index k0 for this lane in a row-major operand; lanes past K read
  // the row's last chunk (zeroed once it has landed); a modular offset, added in 32 bits
  MOE_DEV uint32_t dma_k(int k0) const { return rm_k_off(g.K, k0, lchunk); }
  // copy c of a refill (full: A0 A1 B0 B1; narrow: A0 B0 B1 B2 B3) into stage j, at byte offset
  // ka (row-major operands) or kt (tiled ones) along K. A wave's copies of one operand fill
  // consecutive 1 KiB blocks of the stage and form a group with one M0 write (lds_m0, at the
  // group's first copy; immediate offset 1024 i for copy i, the row offsets being stored
  // 1024 (3 - i) higher and the base taken 3072 bytes lower), so a refill's copies are issued
  // in order c = 0 .. CPR - 1.
  // SA: every copy's K part is uniform (tiled operands, or K a multiple of 32; ku = k0 * 2
  // for row-major ones), taken into the scalar base of the saddr form (no per-copy vector
  // address arithmetic)
  template <bool SA>
  MOE_DEV void copy(const Src& sr, int c, int j, uint32_t ka, uint32_t kt, uint32_t ku) const {
    const bool is_a = NAR ? c == 0 : c < CA;
    const int i = is_a ? c : c - CA;
    if (c == 0) lds_m0(sa(j) + wave * CA * 16 * kBK);
    if (c == CA) lds_m0(sb(j) + wave * CB * 16 * kBK);
    const char* base = is_a ? sr.a : sr.b[i];
    const uint32_t row = is_a ? sr.ao[i] : sr.bo[i];
    const bool tl = is_a ? a_is_tiled() : g.b_kp > 0;
    if constexpr (SA) {
      const char* sbase = reinterpret_cast<const char*>(reinterpret_cast<uintptr_t>(base) + (tl ? kt : ku) - 3072u);
      switch (i) {
        case 0: lds_dma16_sg<0>(sbase, row); break;
        case 1: lds_dma16_sg<1>(sbase, row); break;
        case 2: lds_dma16_sg<2>(sbase, row); break;
        default: lds_dma16_sg<3>(sbase, row); break;
      }
    } else {
      const char* src = reinterpret_cast<const char*>(reinterpret_cast<uintptr_t>(base) - 3072u) + src_off(row, tl ? kt : ka);
      switch (i) {
        case 0: lds_dma16_g<0>(src); break;
        case 1: lds_dma16_g<1>(src); break;
        case 2: lds_dma16_g<2>(src); break;
        default: lds_dma16_g<3>(src); break;
      }
    }
  }
  // every copy of slab k (from the start of K) into stage j
  template <bool SA>
  MOE_DEV void refill(const Src& sr, int j, int k) const {
    const uint32_t ka = dma_k(k * kBK), kt = dma_kt(k * kBK), ku = (uint32_t)k * kBK * 2u;
#pragma unroll
    for (int c = 0; c < CPR; ++c) copy<SA>(sr, c, j, ka, kt, ku);
  }
};

// Global store instructions each wave issues in the epilogue of a tile whose rows and columns
// are all in range: 4 row blocks x 2 halves x the flushes of a half (one per output array:
// SwiGLU saving keeps gate and up pre-activations and the result, GELU saving the
// pre-activation and the result) x 16-byte chunks per lane (a 64-column half: 2, 32: 1).
template <int EPI> constexpr int kStores =
    8 * (EPI == kEpiSwigluSave ? 3 : EPI == kEpiGeluSave ? 2 : 1) * (kSwi<EPI> ? 1 : 2);

// One work item: tile (e, row0, rows, nt) over slabs [kso, kso + nk) of nk_all; NAR picks the
// narrow shape. PART 2 with q > 1 writes this item's float32 partial tile (item w).
//
// DEFER (full shape, whole-K items): the next item of the workgroup, s_next (-1: none), is
// decoded once this item's slabs are done (returned in *ne, *nrow0, *nrows, *nnt). When this
// tile's rows and columns are all in range (and nk >= NST), the next item's first NST - 1
// stages are issued before this item's epilogue stores, so that those stores drain while
// the next item starts instead of before it; the next item then runs with RLX: its first
// stages were issued by the previous item, followed by exactly kStores<EPI> stores that may
// still be in flight. Without RLX an item issues its own first stages. Returns for the next
// item: 2 = RLX, 1 = not.
template <int EPI, int PART, int NAR, bool SA, bool DEFER = false, bool RLX = false>
MOE_DEV int gemm_tile(const GemmArgs& g, uint16_t* smem, int tid, int wave, int e, int row0, int rows, int nt,
                      int kso, int nk, int nk_all, long long w, int q, long long s_next = -1, int NT = 0,
                      int* ne = nullptr, int* nrow0 = nullptr, int* nrows = nullptr, int* nnt = nullptr) {
  using TL = TileLoads<EPI, NAR>;
  constexpr int TBM = TL::TBM, TBN = TL::TBN;
  constexpr int NST = NAR ? 4 : 5;                // LDS stages
  constexpr int CA = TL::CA, CB = TL::CB, CPR = TL::CPR;
  constexpr int kVm = (NST - 2) * CPR;            // copies a wave may leave in flight at a boundary
  constexpr int kCols = TL::kCols;                // output columns per tile
  const int K = g.K, n_out = g.n_out;
  const int grp = wave >> 2;                                        // ping-pong group
  const int wm = NAR ? 0 : (wave & 1);                              // 128-row block of the tile
  const int wc = NAR ? wave : grp * 2 + ((wave >> 1) & 1);          // 64-B-row block
  const bool k_tail = (K % kBK) != 0;
  static_assert(!DEFER || (!NAR && PART != 2), "deferred stores: full shape, whole-K items");
  static_assert(DEFER || !RLX, "relaxed waits follow deferred stores");
  // Epilogue LDS (arrays 8 and 9, the last full stage, not refilled before the next item's
  // first barrier): each wave's 16-row staging buffer, then this tile's per-row gates (down
  // projection) and per-column biases.
  constexpr int kStageBuf = 16 * 72;  // elements of a wave's staging buffer (16 padded rows)
  float* s_gate = reinterpret_cast<float*>(smem + 8 * kStageElems + 8 * kStageBuf);
  float* s_bias = s_gate + kBM;

  // The lane index is made opaque per tile: otherwise the compiler hoists every
  // lane-dependent address out of the tile loop and spills them across it.
  int lane = tid & 63;
  asm volatile("" : "+v"(lane));
  const TL L(g, smem, wave, lane);
  auto sa = [&](int j) { return L.sa(j); };
  auto sb = [&](int j) { return L.sb(j); };
  // MFMA operand reads: row (lane & 31) of a 32-row block, logical chunk 2 ks + (lane >> 5),
  // physical chunk = logical ^ ((row >> 2) & 3); element offsets for ks = 0, 1.
  int rdk[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) rdk[ks] = (lane & 31) * kBK + (((2 * ks + (lane >> 5)) ^ (((lane & 31) >> 2) & 3)) * 8);
  const int a_rd = wm * 128 * kBK;
  const int b_rd = wc * 64 * kBK;
  const int n0 = nt * kCols;

  // Refills issued since the previous item's epilogue stores, while fewer than 3 (RLX): a
  // boundary then leaves those stores in flight (kVm + kStores<EPI>). That wait still covers
  // what the plain kVm covers, every copy but the last three refills, as the stores were
  // issued after all but those refills; with 3 refills after them it needs them done. The
  // count is a compile-time constant at every boundary (the first NST slabs are peeled).
  int relax = RLX ? 3 : 0;
  const typename TL::Src cur = L.src(e, row0, rows, nt);
  auto copy = [&](int c, int j, uint32_t ka, uint32_t kb, uint32_t ku) { L.template copy<SA>(cur, c, j, ka, kb, ku); };
  auto dma_k = [&](int k0) { return L.dma_k(k0); };
  auto refill = [&](int j, int slab) {
    L.template refill<SA>(cur, j, kso + slab);
    relax -= relax > 0;
  };
  // zero this wave's copied chunks of the last slab that lie past K (after they landed)
  // (the uniform slab test first: a launch with K a multiple of 32 pays a scalar compare)
  auto zero_tail = [&](int j, int slab) {
    if (__builtin_expect(!k_tail || kso + slab != nk_all - 1, 1)) return;
    if ((kso + slab) * kBK + L.lchunk < K) return;
#pragma unroll
    for (int i = 0; i < CA; ++i)
      *reinterpret_cast<uint4*>(sa(j) + (wave * CA + i) * 16 * kBK + lane * 8) = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < CB; ++i)
      *reinterpret_cast<uint4*>(sb(j) + (wave * CB + i) * 16 * kBK + lane * 8) = make_uint4(0, 0, 0, 0);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  bf16x8 fa[2][4], fb[2][2];  // operands of one slab: [ks][block]
  auto read_slab = [&](int j) {
    const uint16_t* a_st = sa(j);
    const uint16_t* b_st = sb(j);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        fa[ks][t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(a_st + a_rd + t * 32 * kBK + rdk[ks]));
#pragma unroll
      for (int t = 0; t < 2; ++t)
        fb[ks][t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(b_st + b_rd + t * 32 * kBK + rdk[ks]));
    }
  };
  // phase boundary; `next` = the slab group 0 reads in the coming phase, in stage j (its K
  // tail is zeroed here, once every wave's copies of it have landed), or -1: none
  auto boundary = [&](int j, int next) {
    __builtin_amdgcn_sched_barrier(0);  // the phase's multiplies / reads stay in the phase
    if (relax > 0) wait_vm_lds<kVm + kStores<EPI>>();
    else wait_vm_lds<kVm>();
    if (next >= 0) zero_tail(j, next);
    wait_vm_lds<63>();
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // multiply the slab in registers while refilling stage j with `slab`: copy c after MFMA
  // number floor((c + 1) 16 / CPR) - 1, so the copies spread over the phase
  auto multiply_refill = [&](int j, int slab) {
    const uint32_t ka = dma_k((kso + slab) * kBK), kb = L.dma_kt((kso + slab) * kBK);
    const uint32_t ku = (uint32_t)(kso + slab) * kBK * 2u;
#pragma unroll
    for (int mm = 0; mm < 16; ++mm) {
      const int ks = mm >> 3, i = (mm >> 1) & 3, jj = mm & 1;
      acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks][i], fb[ks][jj], acc[i][jj], 0, 0, 0);
#pragma unroll
      for (int c = 0; c < CPR; ++c)
        if (mm == (c + 1) * 16 / CPR - 1) {
          copy(c, j, ka, kb, ku);
          __builtin_amdgcn_sched_barrier(0);
        }
    }
    relax -= relax > 0;
  };
  // Slab k lives in stage k mod NST. Each group runs its own straight-line loop; both pass
  // the same sequence of barriers (two per slab plus one before the first):
  //   group 0: [read 0] | mult 0 | read 1 | mult 1 | read 2 | ...      (reads in odd phases)
  //   group 1: [ idle ] | read 0 | mult 0 | read 1 | mult 1 | ...      (reads in even phases)
  // A stage is refilled only when both groups are done with its previous slab.
  // group 0, slab k in stage j: multiply k and refill slab k+NST-1; then read k+1 (which
  // exists unless `last` may be the final slab)
  auto g0_step = [&](int j, int k, bool last) {
    multiply_refill((j + NST - 1) % NST, min(k + NST - 1, nk - 1));
    boundary((j + 1) % NST, k + 1);
    if (!last || k + 1 < nk) read_slab((j + 1) % NST);
    boundary((j + 1) % NST, -1);
  };
  // group 1, slab k in stage j: read k; then multiply k and refill its stage with slab k+NST
  auto g1_step = [&](int j, int k) {
    read_slab(j);
    boundary((j + 1) % NST, k + 1);
    multiply_refill(j, min(k + NST, nk - 1));
    boundary((j + 1) % NST, -1);
  };
  if (!RLX) {
#pragma unroll
    for (int j = 0; j < NST - 1; ++j) refill(j, min(j, nk - 1));
  }
  boundary(0, 0);
  int kt = 0;
  if (grp == 0) {
    read_slab(0);
    boundary(0, -1);
    if (RLX) {
#pragma unroll
      for (int j = 0; j < NST; ++j) g0_step(j, j, j == NST - 1);
      kt = NST;
    }
    for (; kt + NST <= nk; kt += NST) {
#pragma unroll
      for (int j = 0; j < NST; ++j) g0_step(j, kt + j, j == NST - 1);
    }
#pragma unroll
    for (int j = 0; j < NST - 1; ++j)
      if (kt + j < nk) g0_step(j, kt + j, true);
  } else {
    refill(NST - 1, min(NST - 1, nk - 1));
    boundary(0, -1);
    if (RLX) {
#pragma unroll
      for (int j = 0; j < NST; ++j) g1_step(j, j);
      kt = NST;
    }
    for (; kt + NST <= nk; kt += NST) {
#pragma unroll
      for (int j = 0; j < NST; ++j) g1_step(j, kt + j);
    }
#pragma unroll
    for (int j = 0; j < NST - 1; ++j)
      if (kt + j < nk) g1_step(j, kt + j);
  }
  // every wave's copies (those past the end included) have landed and every wave is done
  // reading the stages: the LDS is free for the epilogue (or the next tile). The explicit
  // wait is needed: the barrier's fence does not wait for LDS-DMA copies in flight.
  wait_vm_lds<0>();
  __syncthreads();
  if (PART == 2 && q > 1) {
    // a K piece of a tail tile: raw float32 accumulators to this item's partial tile
    // [TBM rows][TBN columns] (the sum and the epilogue follow in tail_reduce_kernel)
    float* pt = g.partial + (size_t)w * (kBM * kBNB);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * 128 + i * 32 + (v >> 2) * 8 + 4 * (lane >> 5) + (v & 3);
          const int col = wc * 64 + j * 32 + (lane & 31);
          pt[row * TBN + col] = acc[i][j][v];
        }
    return 0;
  }
  // the next item (its tile table entry is read with nothing else in flight), and whether
  // its first stages go ahead of this tile's stores (every store then has live lanes, so
  // each wave issues exactly kStores<EPI> of them)
  const bool has_next = DEFER && s_next >= 0;
  if (has_next) decode_tile(g.tiles, s_next, NT, false, 0, ne, nrow0, nrows, nnt);
  const bool pre_issue = has_next && rows == TBM && n0 + kCols <= n_out && nk_all >= NST;

  // per-row gate and per-column bias of the tile, staged once in LDS for the epilogue
  // (1 and 0 when absent, so the epilogue has no branches)
  if (tid < TBM)
    s_gate[tid] = ((EPI == kEpiDown || kSave<EPI>) && g.gate && tid < rows) ? g.gate[row0 + tid] : 1.f;
  if (tid < kCols)
    s_bias[tid] = (!kSwi<EPI> && g.bias && n0 + tid < n_out)
                      ? bf16_to_f32(static_cast<const uint16_t*>(g.bias)[(size_t)e * n_out + n0 + tid]) : 0.f;
  // the next item's first stages (arrays 0..7), behind the loads above and ahead of the stores
  if (pre_issue) {
    const typename TL::Src nx = L.src(*ne, *nrow0, *nrows, *nnt);
#pragma unroll
    for (int j = 0; j < NST - 1; ++j) L.template refill<SA>(nx, j, min(j, nk_all - 1));
  }
  __syncthreads();

  // ---- epilogue: activation / bias / gate in registers, then per 16-row half of a 32-row
  // block the wave's bf16 rows are staged in its own LDS buffer (rows padded by 16 bytes: the
  // two half-waves, 4 rows apart, hit disjoint banks) and written with 16-byte row stores.
  uint16_t* C = static_cast<uint16_t*>(g.c);
  constexpr int kWCols = kSwi<EPI> ? 32 : 64;               // wave output columns
  constexpr int kStride = kWCols + 8;                       // staged row length (elements)
  constexpr int kWChunks = kWCols / 8;                      // 16-byte chunks per row
  static_assert(16 * kStride <= kStageBuf, "staging buffer");
  uint16_t* stage = smem + 8 * kStageElems + wave * kStageBuf;
  const int col_base = n0 + wc * kWCols;                    // first output column of the wave
  // lane's element v (8 h <= v < 8 h + 8) of a 32 x 32 block, in half h: column lane & 31,
  // staged row 8 ((v >> 2) & 1) + 4 (lane >> 5) + (v & 3)
  uint16_t* st_lane = stage + ((lane >> 5) * 4) * kStride + (lane & 31);
  auto srow = [](int v) { return ((v >> 2) & 1) * 8 + (v & 3); };
  // each lane stores whole 16-byte chunks of the half's 16 staged rows to dst (row pitch
  // `pitch` elements, first column col_base)
  // (ckp > 0: dst is tiled with row pitch ckp; a store instruction then writes 16 rows of one
  // 32-column slab, 1 KiB contiguous within a 128-row block)
  auto flush = [&](int i, int h, uint16_t* dst, size_t pitch, int ckp = 0) {
#pragma unroll
    for (int it = 0; it < 16 * kWChunks / 64; ++it) {
      const int idx = it * 64 + lane;
      const int prow = idx / kWChunks, ch = idx % kWChunks;
      const int trow = wm * 128 + i * 32 + h * 16 + prow;
      const int col = col_base + ch * 8;
      const uint4 val = *reinterpret_cast<const uint4*>(stage + prow * kStride + ch * 8);
      const int R = row0 + trow;
      const size_t at = ckp > 0 ? (size_t)(R & ~(kTiledRows - 1)) * ckp + (size_t)(col >> 5) * (kTiledRows * kTiledK) +
                                      (R & (kTiledRows - 1)) * kTiledK + (col & 31)
                                : (size_t)R * pitch + col;
      if (trow < rows && col < n_out) *reinterpret_cast<uint4*>(dst + at) = val;
    }
  };
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // the gate of the lane's row of element v
      auto gate_of = [&](int v) { return s_gate[wm * 128 + i * 32 + h * 16 + srow(v) + (lane >> 5) * 4]; };
      if (EPI == kEpiSwigluSave) {
        // gate pre-activation, up pre-activation, then w_a silu(g) u, one staging pass each
        uint16_t* C2 = static_cast<uint16_t*>(g.c2);
#pragma unroll
        for (int v = 8 * h; v < 8 * h + 8; ++v) st_lane[srow(v) * kStride] = f32_to_bf16(acc[i][0][v]);
        flush(i, h, C2, 2 * (size_t)n_out);
#pragma unroll
        for (int v = 8 * h; v < 8 * h + 8; ++v) st_lane[srow(v) * kStride] = f32_to_bf16(acc[i][1][v]);
        flush(i, h, C2 + n_out, 2 * (size_t)n_out);
#pragma unroll
        for (int v = 8 * h; v < 8 * h + 8; ++v)
          st_lane[srow(v) * kStride] = f32_to_bf16(gate_of(v) * (silu_f(acc[i][0][v]) * acc[i][1][v]));
        flush(i, h, C, n_out);
      } else if (EPI == kEpiGeluSave) {
        // pre-activation (with b1), then w_a gelu(.)
        uint16_t* C2 = static_cast<uint16_t*>(g.c2);
#pragma unroll
        for (int v = 8 * h; v < 8 * h + 8; ++v)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            st_lane[srow(v) * kStride + j * 32] =
                f32_to_bf16(acc[i][j][v] + s_bias[wc * kWCols + j * 32 + (lane & 31)]);
        flush(i, h, C2, n_out);
#pragma unroll
        for (int v = 8 * h; v < 8 * h + 8; ++v) {
          const float gs = gate_of(v);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            st_lane[srow(v) * kStride + j * 32] =
                f32_to_bf16(gs * gelu_erf(acc[i][j][v] + s_bias[wc * kWCols + j * 32 + (lane & 31)]));
        }
        flush(i, h, C, n_out);
      } else {
        // the half block's values first, as independent chains the scheduler can overlap
        // (the activations' exp, rcp and erf have latencies of their own), then their
        // staging writes
        constexpr int kJ = kSwi<EPI> ? 1 : 2;
        float val[8][kJ];
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const int vv = 8 * h + v;
          if (EPI == kEpiSwiglu) {
            val[v][0] = silu_f(acc[i][0][vv]) * acc[i][1][vv];
          } else {
            const float gs = gate_of(vv);
#pragma unroll
            for (int j = 0; j < kJ; ++j) {
              const float bj = s_bias[wc * kWCols + j * 32 + (lane & 31)];
              if (EPI == kEpiGelu) val[v][j] = gelu_erf(acc[i][j][vv] + bj);
              else val[v][j] = g.pre_gated ? acc[i][j][vv] + bj * gs : (acc[i][j][vv] + bj) * gs;
            }
          }
        }
#pragma unroll
        for (int v = 0; v < 8; ++v)
#pragma unroll
          for (int j = 0; j < kJ; ++j) st_lane[srow(8 * h + v) * kStride + j * 32] = f32_to_bf16(val[v][j]);
        flush(i, h, C, n_out, EPI == kEpiDown ? 0 : g.c_kp);  // only h is written tiled
      }
      __builtin_amdgcn_sched_barrier(0);  // keep each half block's registers short-lived
    }
  }
  if (!DEFER) {
    // the staging area and the gates may be a narrow tile's first stages
    __syncthreads();
    return 0;
  }
  // the next item's first barrier comes before anything refills arrays 8 and 9
  return pre_issue ? 2 : 1;
}

// PART: 0 = every work item; 1 = only the whole rounds (the first floor(S / G) * G items of
// S = gemm_items, G = gridDim.x); 2 = the remaining S mod G items, each cut along K into q
// pieces (q = tail_pieces), one piece per workgroup, writing float32 partials when q > 1
// (tail_reduce_kernel sums them and applies the epilogue).
// NAR: whether the launch may run narrow tiles; without them the narrow shape is not
// compiled in, and the kernel keeps the registers of the full shape alone.
template <int EPI, int PART, bool NAR, bool SA>
MOE_DEV void bf16_run(const GemmArgs& g, uint16_t* smem) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  const int NT = g.n_tiles_n;
  const int nk_all = (g.K + kBK - 1) / kBK;
  // this launch's items and this workgroup's run of them (gemm_sched.h)
  const GemmPlan P = gemm_plan(g.tiles, NT, NAR && g.nar_ok, PART, gridDim.x, nk_all);
  const GemmRange R = gemm_range(P, PART, blockIdx.x, gridDim.x);
  const long long w_begin = R.begin, w_end = R.end;
  const int w_step = R.step;

  if constexpr (!NAR && PART != 2) {
    // full-shape, whole-K items: each item issues the next one's first stages before its
    // epilogue stores (gemm_tile, DEFER)
    if (w_begin >= w_end) return;
    int e, row0, rows, nt;
    decode_tile(g.tiles, w_begin, NT, false, 0, &e, &row0, &rows, &nt);
    int pre = 1;
    for (long long w = w_begin;; w += w_step) {
      int wave_i = wave, NT_i = NT;
      asm volatile("" : "+s"(wave_i), "+s"(NT_i));
      const int tid_i = wave_i * 64 + (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      const long long w2 = w + w_step;
      const long long sn = w2 < w_end ? w2 : -1;
      int ne = 0, nrow0 = 0, nrows = 0, nnt = 0;
      if (pre == 2)
        pre = gemm_tile<EPI, PART, 0, SA, true, true>(g, smem, tid_i, wave_i, e, row0, rows, nt, 0, nk_all, nk_all, w, 1,
                                                  sn, NT_i, &ne, &nrow0, &nrows, &nnt);
      else
        pre = gemm_tile<EPI, PART, 0, SA, true, false>(g, smem, tid_i, wave_i, e, row0, rows, nt, 0, nk_all, nk_all, w,
                                                   1, sn, NT_i, &ne, &nrow0, &nrows, &nnt);
      if (w2 >= w_end) break;
      e = ne;
      row0 = nrow0;
      rows = nrows;
      nt = nnt;
    }
  } else {
  for (long long w = w_begin; w < w_end; w += w_step) {
    int kso, nk, piece;  // this item's slabs [kso, kso + nk)
    const long long s = plan_item(P, PART, w, nk_all, &kso, &nk, &piece);  // position in the sequence
    // Rebuilt / made opaque per item, so that what the two tile shapes derive from them is
    // computed per tile instead of being held (and spilled to memory) across the whole loop;
    // the thread index comes from the wave index and the lane's position in the wave.
    int wave_i = wave, NT_i = NT;
    asm volatile("" : "+s"(wave_i), "+s"(NT_i));
    const int tid_i = wave_i * 64 + (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    int e, row0, rows, nt;
    const bool is_nar = decode_tile(g.tiles, s, NT_i, P.nar, P.n_tail, &e, &row0, &rows, &nt);
    if constexpr (NAR) {
      if (is_nar) gemm_tile<EPI, PART, 1, SA>(g, smem, tid_i, wave_i, e, row0, rows, nt, kso, nk, nk_all, w, P.q);
      else gemm_tile<EPI, PART, 0, SA>(g, smem, tid_i, wave_i, e, row0, rows, nt, kso, nk, nk_all, w, P.q);
    } else {
      (void)is_nar;
      gemm_tile<EPI, PART, 0, SA>(g, smem, tid_i, wave_i, e, row0, rows, nt, kso, nk, nk_all, w, P.q);
    }
  }
  }
}

template <int EPI, int PART = 0, bool NAR = false>
__global__ __launch_bounds__(kGemmThreads, 1) void expert_gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[10 * kStageElems];
  // copies in saddr form where every copy's K part is uniform (as in the 4-wave kernel).
  // Same-box A/B, 2 rounds: GPT-2-small layer 0.307-0.308 -> 0.296-0.301 ms, fine-grained
  // 1.769 -> 1.716-1.720 ms; DeepSeek-V3 (weight-stream bound) unchanged.
  const bool k_whole = (g.K % kBK) == 0;
  const bool a_uniform = (!kSave<EPI> && g.a_kp > 0) || k_whole;
  const bool b_uniform = g.b_kp > 0 || k_whole;
  if (a_uniform && b_uniform) bf16_run<EPI, PART, NAR, true>(g, smem);
  else bf16_run<EPI, PART, NAR, false>(g, smem);
}

// ---------------------------------------------------------------------------------------
// bfloat16 grouped GEMM, 4-wave shape: the launches without narrow tiles.
//
// A 256 x 256 tile per workgroup of 4 waves (2 x 2), each wave 128 rows x 128 B-rows on
// v_mfma_f32_16x16x32_bf16: 8 x 8 blocks of 16 x 16, 256 float32 accumulators per lane.
// Operands stream through kW4Stages LDS stages of one 32-element K slab (A 16 KiB + B 16 KiB,
// written by global_load_lds_dwordx4 as in the 8-wave kernel, with a swizzle suited to the
// 16x16x32 reads), and a 32 KiB epilogue area follows them (160 KiB in all).
//
// Slab pipeline, per wave: while slab s multiplies (64 MFMAs), the wave reads slab s+1's
// operand fragments into its other register set (16 ds_read_b128, one after every other MFMA
// of the first half) and refills slab s's stage with slab s + kW4Stages (8 copies, after MFMAs
// of the second half). One barrier per slab, at its end, once slab s+2 has landed: it makes
// slab s+2 visible and frees slab s+1's stage (its fragments are in registers by then). A
// fragment is thus read a whole slab (1024 MFMA cycles) before it is used, and the MFMA pipe
// sees one barrier per 64 MFMAs.
//
// SwiGLU: the wave's 8 B-row blocks alternate 16 gate rows and the 16 up rows of the same
// output columns, so gate and up of an output land in the same lane (64 output columns per
// wave, 128 per tile). GELU / down: 128 output columns per wave.
//
// Row blocks: an expert's last m-tile of at most 128 rows is multiplied with only as many
// 16-row blocks per wave as its rows need (4, 2 or 1; the two wave rows split its rows
// evenly), with the same copies, waits and barriers. Mixtral shape, same-box A/B, 3 rounds:
// executed MFMA work of the up projection 4.03 -> 3.92 TFLOP, its time 3.30-3.32 -> 3.24-3.26
// ms, the layer 1.2-1.9 % faster.
// ---------------------------------------------------------------------------------------
constexpr int kW4Threads = 256;
constexpr int kW4Stages = 4;
constexpr int kW4StageElems = 2 * kStageElems;  // A [256][32] then B [256][32]
constexpr int kW4Pitch = 136;                   // staged row pitch (elements) for 128 columns
constexpr int kW4WaveStage = 16 * kW4Pitch;     // elements of a wave's 16-row staging buffer
template <int EPI> constexpr int kW4Cols = kSwi<EPI> ? 64 : 128;  // output columns per wave
// global store instructions per wave in the epilogue of a tile whose rows and columns are all
// in range: 8 blocks x the flushes of a block x (columns / 32)
template <int EPI> constexpr int kW4Stores =
    8 * (EPI == kEpiSwigluSave ? 3 : EPI == kEpiGeluSave ? 2 : 1) * (kW4Cols<EPI> / 32);
// the next item's first stages go ahead of the epilogue stores when the relaxed wait
// (2 slabs of copies + the stores) fits the counter
template <int EPI> constexpr bool kW4Defer = 8 * (kW4Stages - 2) + kW4Stores<EPI> <= 63;

template <int EPI>
struct W4Loads {
  static constexpr int kCols = kSwi<EPI> ? 128 : 256;  // output columns per tile
  struct Src {
    const char* a;
    const char* b[4];
    uint32_t ao[4], bo[4];
  };
  const GemmArgs& g;
  uint16_t* smem;
  int wave, lchunk, lrow;
  // lane l writes row l >> 2 of a copy's 16 rows at physical chunk l & 3, which holds logical
  // chunk (l & 3) ^ ((row >> 1) & 3): the swizzle under which the 16x16x32 operand reads (16
  // consecutive rows at one logical chunk per 16 lanes) hit no bank conflict (measured with a
  // read-pattern probe: (row >> 2) & 3, the 8-wave kernel's, costs 0.8 conflict cycles per
  // ds_read_b128 of this pattern)
  // the launch's last slab when it runs past K (its chunks past K are zeroed once landed), else -1
  int ktail;
  MOE_DEV W4Loads(const GemmArgs& g_, uint16_t* smem_, int wave_, int lane)
      : g(g_), smem(smem_), wave(wave_), lchunk(((lane & 3) ^ ((lane >> 3) & 3)) * 8), lrow(lane >> 2),
        ktail((g_.K % kBK) != 0 ? (g_.K + kBK - 1) / kBK - 1 : -1) {}
  MOE_DEV uint16_t* sa(int j) const { return smem + j * kW4StageElems; }
  MOE_DEV uint16_t* sb(int j) const { return smem + j * kW4StageElems + kBM * kBK; }
  MOE_DEV bool a_tiled() const { return !kSave<EPI> && g.a_kp > 0; }
  // copy i (0..3) of A / B covers stage rows (wave * 4 + i) * 16 .. + 15. The four copies of
  // an operand form one group (one M0 write, immediate offsets 1024 i; lds_dma16_sg): the row
  // offsets are stored 1024 (3 - i) higher and the group's base is taken 3072 bytes lower, so
  // copy i reads base + row offset exactly, with no offset below zero.
  MOE_DEV Src src(int e, int row0, int rows, int nt) const {
    const int K = g.K, n_out = g.n_out, n0 = nt * kCols;
    const bool tiled = g.b_kp > 0;
    const int Kb = tiled ? g.b_kp : K;
    const size_t b_off = ((size_t)e * (tiled ? g.b_np : n_out) + n0) * Kb * 2;
    const int rb = row0 & ~(kTiledRows - 1);
    Src r;
    r.a = static_cast<const char*>(g.a) + (a_tiled() ? (size_t)rb * g.a_kp * 2 : (size_t)row0 * K * 2);
    const char* b0_base = static_cast<const char*>(g.b0) + b_off;
    const char* b1_base = kSwi<EPI> ? static_cast<const char*>(g.b1) + b_off : b0_base;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = (wave * 4 + i) * 16 + lrow;
      const int rc = min(rr, rows - 1);
      r.ao[i] = a_tiled() ? tiled_row_off(row0 - rb + rc, g.a_kp, lchunk) : rm_row_off(rc, K, lchunk);
      int cl;
      if (kSwi<EPI>) {
        // B-rows 32 c .. 32 c + 15: gate of output columns 16 c ..; the next 16: up of the same
        cl = (rr >> 5) * 16 + (rr & 15);
        r.b[i] = (((wave * 4 + i) & 1) != 0) ? b1_base : b0_base;  // uniform per copy
      } else {
        cl = rr;
        r.b[i] = b0_base;
      }
      cl = min(cl, n_out - 1 - n0);
      r.bo[i] = tiled ? tiled_row_off(cl, Kb, lchunk) : rm_row_off(cl, K, lchunk);
      r.ao[i] += (uint32_t)(3 - i) * 1024u;
      r.bo[i] += (uint32_t)(3 - i) * 1024u;
    }
    return r;
  }
  // copy c of a refill (0..3: A, 4..7: B) of global slab k into stage j; copies 0 and 4 set
  // their group's M0, so a refill's copies are issued in order c = 0 .. 7 with no other M0
  // write between them.
  // SA: the K part of every copy of the launch is uniform (tiled operands, or K a multiple of
  // 32), so it goes into the scalar base of the saddr form and a copy needs no vector address
  // arithmetic; otherwise the 64-bit per-lane address of the K-tail rule (rm_k_off).
  template <bool SA>
  MOE_DEV void copy(const Src& sr, int c, int j, int k) const {
    if (c == 0) lds_m0(sa(j) + wave * 4 * 16 * kBK);
    if (c == 4) lds_m0(sb(j) + wave * 4 * 16 * kBK);
    const bool isa = c < 4;
    const uint32_t kt = tiled_k_off(k * kBK);
    const char* base = isa ? sr.a : sr.b[c - 4];
    const uint32_t row = isa ? sr.ao[c] : sr.bo[c - 4];
    const bool tl = isa ? a_tiled() : g.b_kp > 0;
    if constexpr (SA) {
      const uint32_t ku = (uint32_t)k * kBK * 2u;
      const char* sbase = reinterpret_cast<const char*>(reinterpret_cast<uintptr_t>(base) + (tl ? kt : ku) - 3072u);
      switch (c & 3) {
        case 0: lds_dma16_sg<0>(sbase, row); break;
        case 1: lds_dma16_sg<1>(sbase, row); break;
        case 2: lds_dma16_sg<2>(sbase, row); break;
        default: lds_dma16_sg<3>(sbase, row); break;
      }
    } else {
      const uint32_t ka = rm_k_off(g.K, k * kBK, lchunk);
      const char* src = reinterpret_cast<const char*>(reinterpret_cast<uintptr_t>(base) - 3072u) + src_off(row, tl ? kt : ka);
      switch (c & 3) {
        case 0: lds_dma16_g<0>(src); break;
        case 1: lds_dma16_g<1>(src); break;
        case 2: lds_dma16_g<2>(src); break;
        default: lds_dma16_g<3>(src); break;
      }
    }
  }
  template <bool SA>
  MOE_DEV void refill(const Src& sr, int j, int k) const {
#pragma unroll
    for (int c = 0; c < 8; ++c) copy<SA>(sr, c, j, k);
  }
  // zero this wave's landed chunks of stage j that lie past K (global slab k is the last one).
  // The slab test is uniform and comes first, so a launch with K a multiple of 32 pays one
  // scalar compare per slab (the combined per-lane test cost ~60 cycles a slab in a probe).
  MOE_DEV void zero_tail(int j, int k, int nk_all, int lane) const {
    if (__builtin_expect(k != ktail, 1)) return;
    if (k * kBK + lchunk < g.K) return;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      *reinterpret_cast<uint4*>(sa(j) + (wave * 4 + c) * 16 * kBK + lane * 8) = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(sb(j) + (wave * 4 + c) * 16 * kBK + lane * 8) = make_uint4(0, 0, 0, 0);
    }
  }
};

// One work item on the 4-wave shape: tile (e, row0, rows, nt) over slabs [kso, kso + nk) of
// nk_all. PART 2 with q > 1 writes the float32 partial tile of item w. DEFER / RLX and the
// returned value as for gemm_tile (the relaxed waits count kW4Stores<EPI> stores).
template <int EPI, int PART, bool SA, bool DEFER = false, bool RLX = false, int MB = 8>
MOE_DEV int gemm_tile_w4(const GemmArgs& g, uint16_t* smem, int tid, int wave, int e, int row0, int rows, int nt,
                         int kso, int nk, int nk_all, long long w, int q, long long s_next = -1, int NT = 0,
                         int* ne = nullptr, int* nrow0 = nullptr, int* nrows = nullptr, int* nnt = nullptr) {
  static_assert(MB == 8 || MB == 4 || MB == 2 || MB == 1, "16-row blocks per wave");
  using TL = W4Loads<EPI>;
  constexpr int NST = kW4Stages;
  constexpr int kCols = TL::kCols;
  constexpr int kWn = 8 * (NST - 2);                      // copies younger than slab s+2
  constexpr int kWr = kWn + (RLX ? kW4Stores<EPI> : 0);   // ... with the previous tile's stores
  static_assert(!DEFER || (PART != 2 && kW4Defer<EPI>), "deferred stores: whole-K items that fit the counter");
  static_assert(DEFER || !RLX, "relaxed waits follow deferred stores");
  const int n_out = g.n_out;
  const int wm = wave & 1, wn = wave >> 1;
  int lane = tid & 63;
  asm volatile("" : "+v"(lane));
  const TL L(g, smem, wave, lane);
  const typename TL::Src cur = L.src(e, row0, rows, nt);
  // 16x16x32 operand read: row lane & 15 of a 16-row block, logical chunk lane >> 4
  const int r16 = (lane & 15) * kBK + (((lane >> 4) ^ (((lane & 15) >> 1) & 3)) * 8);
  // wave wm multiplies tile rows [16 MB wm, 16 MB (wm + 1)): all 256 for MB = 8; a tile of at
  // most 32 MB rows (its expert's last) splits its rows evenly between the two wave rows
  constexpr int kMR = 16 * MB;  // rows per wave
  const int a_rd = wm * kMR * kBK + r16, b_rd = wn * 128 * kBK + r16;
  // the slab held by pipeline position t (copies past the item's end repeat its last slab)
  auto slab_at = [&](int t) { return kso + min(t, nk - 1); };

  f32x4 acc[MB][8];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 fa[2][MB], fb[2][8];

  if (!RLX) {
#pragma unroll
    for (int t = 0; t < NST - 1; ++t) L.template refill<SA>(cur, t, slab_at(t));
  }
  L.template refill<SA>(cur, NST - 1, slab_at(NST - 1));
  // slabs 0 and 1 landed (the younger copies: slabs 2 .. NST-1, and with RLX the previous
  // item's stores, issued after this item's first NST-1 slabs); K tails zeroed
  wait_vm_lds<kWr>();
  L.zero_tail(0, slab_at(0), nk_all, lane);
  L.zero_tail(1, slab_at(1), nk_all, lane);
  wait_vm_lds<63>();
  stage_barrier();
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (t < MB) fa[0][t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(L.sa(0) + a_rd + t * 16 * kBK));
    fb[0][t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(L.sb(0) + b_rd + t * 16 * kBK));
  }
  // every wave's reads of stage 0 are done before slab 0's body refills it
  wait_vm_lds<kWr>();
  stage_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // slab s (fragments in set P) multiplies; slab s+1 is read into set 1-P; stage s % NST is
  // refilled with pipeline position s + NST; at the end slab s+2 has landed and is visible
  auto body = [&](int s, auto P_, auto W_) {
    constexpr int P = decltype(P_)::value;
    constexpr int W = decltype(W_)::value;
    const int st = s % NST;
    const int nst = (s + 1) % NST;
    const uint16_t* ra = L.sa(nst) + a_rd;
    const uint16_t* rb = L.sb(nst) + b_rd;
    const int rslab = slab_at(s + NST);
    // the slab's 8 MB MFMAs; its MB + 8 fragment reads spread over the first half (A blocks
    // first) and its 8 copies over the second (for MB = 8: a read after every even MFMA of the
    // first half, a copy after MFMAs 33, 37, .., 61)
    constexpr int kM = 8 * MB, kR = MB + 8, kH = kM / 2;
#pragma unroll
    for (int mm = 0; mm < kM; ++mm) {
      const int i = mm >> 3, j = mm & 7;
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[P][i], fb[P][j], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < kR; ++t) {
        if ((t * kH) / kR != mm) continue;
        if (t < MB) fa[1 - P][t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ra + t * 16 * kBK));
        else fb[1 - P][t - MB] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rb + (t - MB) * 16 * kBK));
      }
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (kH + (c * kH) / 8 + (kM >= 32 ? 1 : 0) == mm) L.template copy<SA>(cur, c, st, rslab);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm_lds<W>();
    L.zero_tail((s + 2) % NST, slab_at(s + 2), nk_all, lane);
    wait_vm_lds<63>();
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  body(0, I0{}, std::integral_constant<int, kWr>{});
  for (int s = 1; s < nk; s += 2) {
    body(s, I1{}, std::integral_constant<int, kWn>{});
    if (s + 1 < nk) body(s + 1, I0{}, std::integral_constant<int, kWn>{});
  }
  // every copy landed (those past the end included) and every wave is done with the stages
  wait_vm_lds<0>();
  __syncthreads();

  if (PART == 2 && q > 1) {
    // a K piece of a tail tile: raw float32 accumulators to this item's partial tile
    // [256 rows][256 B-rows] (summed with the epilogue by tail_reduce_kernel)
    float* pt = g.partial + (size_t)w * (kBM * kBNB);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = wm * kMR + i * 16 + 4 * (lane >> 4) + v;
          const int col = wn * 128 + j * 16 + (lane & 15);
          pt[row * kBNB + col] = acc[i][j][v];
        }
    return 0;
  }
  const bool has_next = DEFER && s_next >= 0;
  if (has_next) decode_tile(g.tiles, s_next, NT, false, 0, ne, nrow0, nrows, nnt);
  const int n0 = nt * kCols;
  const bool pre_issue = MB == 8 && has_next && rows == kBM && n0 + kCols <= n_out && nk_all >= NST;

  // epilogue area: each wave's 16-row staging buffer, then the tile's row gates and column biases
  uint16_t* epi = smem + NST * kW4StageElems;
  float* s_gate = reinterpret_cast<float*>(epi + 4 * kW4WaveStage);
  float* s_bias = s_gate + kBM;
  s_gate[tid] = ((EPI == kEpiDown || kSave<EPI>) && g.gate && tid < rows) ? g.gate[row0 + tid] : 1.f;
  if (tid < kCols)
    s_bias[tid] = (!kSwi<EPI> && g.bias && n0 + tid < n_out)
                      ? bf16_to_f32(static_cast<const uint16_t*>(g.bias)[(size_t)e * n_out + n0 + tid]) : 0.f;
  if (pre_issue) {
    const typename TL::Src nx = L.src(*ne, *nrow0, *nrows, *nnt);
    const int nk_next = nk_all;  // whole-K items
#pragma unroll
    for (int t = 0; t < NST - 1; ++t) L.template refill<SA>(nx, t, min(t, nk_next - 1));
  }
  __syncthreads();

  // ---- epilogue: per 16-row block i, the wave's outputs are staged as bf16 in its own LDS
  // buffer and written with 16-byte row stores (tiled h: a store covers 16 rows of one slab)
  uint16_t* C = static_cast<uint16_t*>(g.c);
  constexpr int kWC = kW4Cols<EPI>;
  uint16_t* stg = epi + wave * kW4WaveStage;
  const int col_base = n0 + wn * kWC;
  auto put = [&](int v, int c, float x) {  // lane's value for staged row 4 (lane >> 4) + v, column c
    stg[(4 * (lane >> 4) + v) * kW4Pitch + c] = f32_to_bf16(x);
  };
  auto flush = [&](int i, uint16_t* dst, size_t pitch, int ckp = 0) {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's staging writes are done
#pragma unroll
    for (int it = 0; it < kWC / 32; ++it) {
      const int idx = it * 64 + lane;
      const int prow = idx / (kWC / 8), ch = idx % (kWC / 8);
      const int trow = wm * kMR + i * 16 + prow;
      const int col = col_base + ch * 8;
      const uint4 val = *reinterpret_cast<const uint4*>(stg + prow * kW4Pitch + ch * 8);
      const int R = row0 + trow;
      const size_t at = ckp > 0 ? (size_t)(R & ~(kTiledRows - 1)) * ckp + (size_t)(col >> 5) * (kTiledRows * kTiledK) +
                                      (R & (kTiledRows - 1)) * kTiledK + (col & 31)
                                : (size_t)R * pitch + col;
      if (trow < rows && col < n_out) *reinterpret_cast<uint4*>(dst + at) = val;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // the staging reads are done before the next writes
  };
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int rbase = wm * kMR + i * 16 + 4 * (lane >> 4);  // tile row of v = 0
    if (kSwi<EPI>) {
      if (EPI == kEpiSwigluSave) {
        uint16_t* C2 = static_cast<uint16_t*>(g.c2);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int v = 0; v < 4; ++v) put(v, c * 16 + (lane & 15), acc[i][2 * c][v]);
        flush(i, C2, 2 * (size_t)n_out);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int v = 0; v < 4; ++v) put(v, c * 16 + (lane & 15), acc[i][2 * c + 1][v]);
        flush(i, C2 + n_out, 2 * (size_t)n_out);
      }
      // the block's 16 activations first, as independent chains the scheduler can overlap
      // (exp and rcp have latencies of their own), then their staging writes
      float hv[4][4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int v = 0; v < 4; ++v) hv[c][v] = silu_f(acc[i][2 * c][v]) * acc[i][2 * c + 1][v];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          put(v, c * 16 + (lane & 15), EPI == kEpiSwigluSave ? s_gate[rbase + v] * hv[c][v] : hv[c][v]);
      flush(i, C, n_out, EPI == kEpiSwiglu ? g.c_kp : 0);
    } else {
      if (EPI == kEpiGeluSave) {
        uint16_t* C2 = static_cast<uint16_t*>(g.c2);
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            put(v, j * 16 + (lane & 15), acc[i][j][v] + s_bias[wn * 128 + j * 16 + (lane & 15)]);
        flush(i, C2, n_out);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float bj = s_bias[wn * 128 + j * 16 + (lane & 15)];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gs = s_gate[rbase + v];
          float val;
          if (EPI == kEpiGelu) val = gelu_erf(acc[i][j][v] + bj);
          else if (EPI == kEpiGeluSave) val = gs * gelu_erf(acc[i][j][v] + bj);
          else val = g.pre_gated ? acc[i][j][v] + bj * gs : (acc[i][j][v] + bj) * gs;
          put(v, j * 16 + (lane & 15), val);
        }
      }
      flush(i, C, n_out, EPI == kEpiGelu ? g.c_kp : 0);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep each block's registers short-lived
  }
  if (!DEFER) {
    __syncthreads();  // the epilogue area before the next item's gates and biases
    return 0;
  }
  return pre_issue ? 2 : 1;
}

// 16-row blocks per wave for a tile of `rows` rows: 8 for more than 128 rows; else the
// smallest of 4, 2, 1 that covers rows / 2 (each of the two wave rows takes half the rows).
MOE_DEV int w4_row_blocks(int rows) { return rows > 128 ? 8 : rows > 64 ? 4 : rows > 32 ? 2 : 1; }
template <int V> using IC = std::integral_constant<int, V>;

// A workgroup's run of the 4-wave grouped GEMM; SA as for W4Loads::copy.
template <int EPI, int PART, bool SA>
MOE_DEV void w4_run(const GemmArgs& g, uint16_t* smem) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..3
  const int NT = g.n_tiles_n;
  const int nk_all = (g.K + kBK - 1) / kBK;
  const GemmPlan P = gemm_plan(g.tiles, NT, false, PART, gridDim.x, nk_all);
  const GemmRange R = gemm_range(P, PART, blockIdx.x, gridDim.x);
  const long long w_begin = R.begin, w_end = R.end;
  const int w_step = R.step;
  if constexpr (PART != 2 && kW4Defer<EPI>) {
    if (w_begin >= w_end) return;
    int e, row0, rows, nt;
    decode_tile(g.tiles, w_begin, NT, false, 0, &e, &row0, &rows, &nt);
    int pre = 1;
    for (long long w = w_begin;; w += w_step) {
      int wave_i = wave, NT_i = NT;
      asm volatile("" : "+s"(wave_i), "+s"(NT_i));
      const int tid_i = wave_i * 64 + (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      const long long w2 = w + w_step;
      const long long sn = w2 < w_end ? w2 : -1;
      int ne = 0, nrow0 = 0, nrows = 0, nnt = 0;
      auto item = [&](auto RLX_, auto MB_) {
        return gemm_tile_w4<EPI, PART, SA, true, decltype(RLX_)::value, decltype(MB_)::value>(
            g, smem, tid_i, wave_i, e, row0, rows, nt, 0, nk_all, nk_all, w, 1, sn, NT_i, &ne, &nrow0, &nrows, &nnt);
      };
      const int mb = w4_row_blocks(rows);
      if (pre == 2) {
        if (mb == 8) pre = item(std::true_type{}, IC<8>{});
        else if (mb == 4) pre = item(std::true_type{}, IC<4>{});
        else if (mb == 2) pre = item(std::true_type{}, IC<2>{});
        else pre = item(std::true_type{}, IC<1>{});
      } else {
        if (mb == 8) pre = item(std::false_type{}, IC<8>{});
        else if (mb == 4) pre = item(std::false_type{}, IC<4>{});
        else if (mb == 2) pre = item(std::false_type{}, IC<2>{});
        else pre = item(std::false_type{}, IC<1>{});
      }
      if (w2 >= w_end) break;
      e = ne;
      row0 = nrow0;
      rows = nrows;
      nt = nnt;
    }
  } else {
    for (long long w = w_begin; w < w_end; w += w_step) {
      int kso, nk, piece;
      const long long s = plan_item(P, PART, w, nk_all, &kso, &nk, &piece);
      int wave_i = wave, NT_i = NT;
      asm volatile("" : "+s"(wave_i), "+s"(NT_i));
      const int tid_i = wave_i * 64 + (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      int e, row0, rows, nt;
      decode_tile(g.tiles, s, NT_i, false, 0, &e, &row0, &rows, &nt);
      const int mb = w4_row_blocks(rows);
      if (mb == 8) gemm_tile_w4<EPI, PART, SA, false, false, 8>(g, smem, tid_i, wave_i, e, row0, rows, nt, kso, nk, nk_all, w, P.q);
      else if (mb == 4) gemm_tile_w4<EPI, PART, SA, false, false, 4>(g, smem, tid_i, wave_i, e, row0, rows, nt, kso, nk, nk_all, w, P.q);
      else if (mb == 2) gemm_tile_w4<EPI, PART, SA, false, false, 2>(g, smem, tid_i, wave_i, e, row0, rows, nt, kso, nk, nk_all, w, P.q);
      else gemm_tile_w4<EPI, PART, SA, false, false, 1>(g, smem, tid_i, wave_i, e, row0, rows, nt, kso, nk, nk_all, w, P.q);
    }
  }
}

// The 4-wave grouped GEMM (launches without narrow tiles). PART as for
// expert_gemm_bf16_kernel. Copies take the saddr form when every copy's K part is uniform:
// both operands tiled, or K a multiple of 32. The per-copy 64-bit address arithmetic it
// removes sat between the MFMAs. Mixtral shape, same-box A/B, 3 rounds: layer 4.76-4.77 ->
// 4.56-4.58 ms, up projection 3.18-3.19 -> 3.04 ms, down 1.45 -> 1.39 ms.
template <int EPI, int PART = 0>
__global__ __launch_bounds__(kW4Threads, 1) void expert_gemm_w4_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[kW4Stages * kW4StageElems + 2 * kStageElems];
  const bool k_whole = (g.K % kBK) == 0;
  const bool a_uniform = (!kSave<EPI> && g.a_kp > 0) || k_whole;
  const bool b_uniform = g.b_kp > 0 || k_whole;
  if (a_uniform && b_uniform) w4_run<EPI, PART, true>(g, smem);
  else w4_run<EPI, PART, false>(g, smem);
}

// The down projection's tail items (PART 2 with q > 1): y_s = (sum of the q partials, in
// piece order, + b2) * gate, rounded once. Unit (t, rg) covers 1 / 64 of tail item t's rows
// (4 of a full tile's 256, 2 of a narrow tile's 128), a thread per 4 columns. The tail's size
// is known on the device only, so a fixed grid walks the units (a grid sized for the largest
// tail left most workgroups to decode the plan and exit: Mixtral shape 22.8 us).
constexpr int kTailReduceGrid = 2048;
MOE_DEV void tail_reduce_unit(const GemmArgs& g, const GemmPlan& P, int t, int rg) {
  const int NT = g.n_tiles_n, n_out = g.n_out;
  const int q = P.q;
  int e, row0, rows, nt;
  const bool nar = decode_tile(g.tiles, P.S_main + t, NT, P.nar, P.n_tail, &e, &row0, &rows, &nt);
  const int tbn = nar ? 512 : 256;  // the partial tile's columns
  const int r = nar ? rg * 2 + (threadIdx.x >> 7) : rg * 4 + (threadIdx.x >> 6);
  const int c4 = nar ? (threadIdx.x & 127) * 4 : (threadIdx.x & 63) * 4;
  const int col = nt * tbn + c4;
  if (r >= rows || col >= n_out) return;
  const float* pt = g.partial + (size_t)t * q * (kBM * kBNB) + r * tbn + c4;
  const float gs = g.gate ? g.gate[row0 + r] : 1.f;
  const uint16_t* bias = static_cast<const uint16_t*>(g.bias);
  float b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = bias ? bf16_to_f32(bias[(size_t)e * n_out + col + i]) : 0.f;
  // the pieces in order; up to kBatch of them requested before the first add
  constexpr int kBatch = 8;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < q; p0 += kBatch) {
    float4 x[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      x[j] = p0 + j < q ? *reinterpret_cast<const float4*>(pt + (size_t)(p0 + j) * (kBM * kBNB))
                        : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (p0 + j < q) {
        v[0] += x[j].x;
        v[1] += x[j].y;
        v[2] += x[j].z;
        v[3] += x[j].w;
      }
  }
  float o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = g.pre_gated ? v[i] + b[i] * gs : (v[i] + b[i]) * gs;
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.c) + (size_t)(row0 + r) * n_out + col) =
      make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
}
__global__ __launch_bounds__(256) void tail_reduce_kernel(GemmArgs g) {
  // the same plan as the PART 2 launch (same table, narrow decision and grid)
  const GemmPlan P = gemm_plan(g.tiles, g.n_tiles_n, g.nar_ok != 0, 2, g.grid, (g.K + kBK - 1) / kBK);
  if (P.q <= 1) return;
  constexpr int kGroups = kBM / 4;  // row groups of a tail item
  const long long units = (P.S_all - P.S_main) * kGroups;
  for (long long u = blockIdx.x; u < units; u += gridDim.x) tail_reduce_unit(g, P, (int)(u / kGroups), (int)(u % kGroups));
}

// ---------------------------------------------------------------------------------------
// float32 grouped GEMM with FMA: 64 rows x 64 output columns per workgroup, K staged 16 at
// a time in LDS (k-major, so each thread's 4 x 4 register block reads broadcast rows).
// SwiGLU keeps a gate and an up accumulator for the same columns.
// ---------------------------------------------------------------------------------------
constexpr int kFBM = 64, kFBN = 64, kFBK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void expert_gemm_f32_kernel(GemmArgs g) {
  __shared__ float sA[kFBK][kFBM + 4];
  __shared__ float sB[kFBK][kFBN + 4];
  __shared__ float sU[kFBK][kFBN + 4];
  const int n_tiles_m = g.tiles[0];
  const int mt = blockIdx.x;
  if (mt >= n_tiles_m) return;
  const int e = g.tiles[kTileHdr + kTileInts * mt];
  const int row0 = g.tiles[kTileHdr + kTileInts * mt + 1];
  const int rows_valid = g.tiles[kTileHdr + kTileInts * mt + 2];
  const int K = g.K, n_out = g.n_out;
  const int n0 = blockIdx.y * kFBN;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const float* A = static_cast<const float*>(g.a);
  const float* B0 = static_cast<const float*>(g.b0) + (size_t)e * n_out * K;
  const float* B1 = (EPI == kEpiSwiglu) ? static_cast<const float*>(g.b1) + (size_t)e * n_out * K : nullptr;

  float acc[4][4] = {}, accu[4][4] = {};
  const int lr = tid >> 2, lk = (tid & 3) * 4;  // loader: row lr, 4 floats at lk
  for (int k0 = 0; k0 < K; k0 += kFBK) {
    const bool kin = (k0 + lk) < K;
    float4 va = make_float4(0, 0, 0, 0), vb = va, vu = va;
    if (lr < rows_valid && kin) va = *reinterpret_cast<const float4*>(A + (size_t)(row0 + lr) * K + k0 + lk);
    if (n0 + lr < n_out && kin) {
      vb = *reinterpret_cast<const float4*>(B0 + (size_t)(n0 + lr) * K + k0 + lk);
      if (EPI == kEpiSwiglu) vu = *reinterpret_cast<const float4*>(B1 + (size_t)(n0 + lr) * K + k0 + lk);
    }
    __syncthreads();
    sA[lk + 0][lr] = va.x; sA[lk + 1][lr] = va.y; sA[lk + 2][lr] = va.z; sA[lk + 3][lr] = va.w;
    sB[lk + 0][lr] = vb.x; sB[lk + 1][lr] = vb.y; sB[lk + 2][lr] = vb.z; sB[lk + 3][lr] = vb.w;
    if (EPI == kEpiSwiglu) {
      sU[lk + 0][lr] = vu.x; sU[lk + 1][lr] = vu.y; sU[lk + 2][lr] = vu.z; sU[lk + 3][lr] = vu.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFBK; ++kk) {
      float av[4], bv[4], uv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bv[j] = sB[kk][tx * 4 + j];
        if (EPI == kEpiSwiglu) uv[j] = sU[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
          if (EPI == kEpiSwiglu) accu[i][j] = fmaf(av[i], uv[j], accu[i][j]);
        }
    }
  }
  float* C = static_cast<float*>(g.c);
  const float* bias = g.bias ? static_cast<const float*>(g.bias) + (size_t)e * n_out : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lrow = ty * 4 + i;
    if (lrow >= rows_valid) continue;
    const int row = row0 + lrow;
    const float gs = (EPI == kEpiDown && g.gate) ? g.gate[row] : 1.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= n_out) continue;
      float v = acc[i][j];
      if (EPI == kEpiSwiglu) v = silu_f(v) * accu[i][j];
      else {
        if (bias) v += bias[col];
        v = (EPI == kEpiGelu) ? gelu_erf(v) : v * gs;
      }
      C[(size_t)row * n_out + col] = v;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------
int ffn_tile_rows(const moe_config& c) { return c.dtype == MOE_BF16 ? kBM : kFBM; }
// Narrow tiles pay where an expert's last m-tile is a large share of its work. The tile table
// lists them, and the up projection runs them, for experts of at most four full m-tiles on
// average (A / E <= 1024 rows). With more rows per expert they save little, and the narrow
// shape's registers slow the full tiles of the same kernel.
int ffn_narrow_rows(const moe_config& c) {
  return narrow_rows_for(c.n_tokens * c.top_k, c.n_experts, c.dtype == MOE_BF16);
}
// The down projection's split launches take narrow tiles only when they are a quarter of the
// m-tiles (use_narrow), which between 512 and 1024 rows per expert they mostly are not: there
// the full-shape kernel (which ignores the table's narrow lists) runs its full tiles faster
// (fine-grained shape, same-box A/B: down 0.550 ms with the narrow-capable kernel, 0.542 ms
// without).
static bool down_narrow(const moe_config& c) {
  return down_narrow_for(c.n_tokens * c.top_k, c.n_experts, c.dtype == MOE_BF16);
}

// A bf16 grouped GEMM launch: the instantiation with narrow tiles when the table may hold them.
// Which kernel a launch runs. Launches that may run narrow tiles take the 8-wave kernel. The
// others take the 4-wave kernel when the reduction is long (K >= kW4MinK), where its fewer
// barriers per MFMA and its slab-ahead operand reads pay, and the 8-wave kernel otherwise, whose
// per-tile costs (pipeline fill, an epilogue spread over twice the waves) are lower.
// Same-box A/B at the Mixtral shape, 20 steps, 3 rounds (layer ms): both projections on the
// 4-wave kernel 4.96-4.99; only the down projection (K = 14336) 5.02-5.03; neither 5.03-5.07.
// The up projection alone (K = 4096) runs 1 % slower on the 4-wave kernel (3.33-3.36 against
// 3.30-3.31 ms), but the down projection that follows it then takes 1.48 instead of 1.56-1.58
// ms. At K = 768 (GPT-2-small up, fine-grained down) the 4-wave kernel was 31 % and 14 % slower.
constexpr int kW4MinK = 4096;
template <int EPI, int PART = 0>
void launch_bf16_gemm(bool narrow, int grid, GemmArgs g, hipStream_t stream) {
  g.nar_ok = narrow ? 1 : 0;
  if (narrow) expert_gemm_bf16_kernel<EPI, PART, true><<<grid, kGemmThreads, 0, stream>>>(g);
  else if (g.K >= kW4MinK) expert_gemm_w4_kernel<EPI, PART><<<grid, kW4Threads, 0, stream>>>(g);
  else expert_gemm_bf16_kernel<EPI, PART, false><<<grid, kGemmThreads, 0, stream>>>(g);
}

// One persistent workgroup per CU (a multiple of 8, so every XCD gets the same count). The
// count is read once per device and cached for the process; concurrent first calls on one
// device store the same value.
int persistent_grid() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int c = cus[dev].load(std::memory_order_relaxed);
  if (!c) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    c = (n + 7) / 8 * 8;
    cus[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

// Tile table of one dense "expert" covering rows [0, n) (the shared expert).
__global__ __launch_bounds__(256) void dense_tiles_kernel(int n, int bm, int* __restrict__ tiles) {
  const int nt = (n + bm - 1) / bm;
  if (threadIdx.x < 4) tiles[4 + threadIdx.x] = 0;
  // all full; fmap (the identity) right after the entries, no nmap
  const int fmap = kTileHdr + kTileInts * nt;
  if (threadIdx.x == 0) {
    tiles[0] = nt;
    tiles[1] = nt;
    tiles[2] = fmap;
    tiles[3] = fmap + nt;
  }
  for (int t = threadIdx.x; t < nt; t += blockDim.x) {
    int* q = tiles + kTileHdr + kTileInts * t;
    q[0] = 0;
    q[1] = t * bm;
    q[2] = min(bm, n - t * bm);
    q[3] = 0;
    q[4] = nt;
    q[5] = 0;
    q[6] = nt;
    tiles[fmap + t] = t;
  }
}

static int shared_m_tiles(const moe_config& c) {
  return c.d_ff_shared > 0 ? (int)((c.n_tokens + ffn_tile_rows(c) - 1) / ffn_tile_rows(c)) : 0;
}

int ffn_max_m_tiles(const moe_config& c) {
  const long long A = c.n_tokens * c.top_k;
  const int bm = ffn_tile_rows(c);
  return (int)((A + bm - 1) / bm) + c.n_experts;
}

void carve_ffn(const moe_config& c, WsCarver& w, WsLayout* L) {
  const size_t A = (size_t)(c.n_tokens * c.top_k);
  // the shared expert (run after the routed experts) reuses the tile table and h
  const size_t tiles_n = (size_t)std::max(ffn_max_m_tiles(c), shared_m_tiles(c));
  // h: row-major [A, d_ff], or tiled (bf16) over A rounded up to 128 rows and d_ff to 32
  const size_t h_routed = ffn_h_tiled(c) ? (A + kTiledRows - 1) / kTiledRows * kTiledRows * (size_t)tiled_k(c, 1)
                                         : A * (size_t)c.d_ff;
  const size_t h_elems = std::max(h_routed, (size_t)c.n_tokens * (size_t)std::max(c.d_ff_shared, 0));
  int* tiles = w.take_t<int>((size_t)tile_table_ints((long long)tiles_n));
  void* h = w.take(h_elems * elem_size(c));
  // the down projection's tail partials (bfloat16 path, when its K allows several pieces)
  size_t part = 0;
  const long long nk_down = (c.d_ff + kBK - 1) / kBK;
  if (c.dtype == MOE_BF16 && nk_down / 4 >= 2) {
    const long long s_max = (long long)ffn_max_m_tiles(c) * ((c.d_model + kBNB - 1) / kBNB);
    part = (size_t)std::min<long long>(kMaxTailItems, s_max * (nk_down / 4)) * kBM * kBNB;
  }
  float* tail = w.take_t<float>(part);
  if (L) {
    L->tiles = tiles;
    L->h = h;
    L->tail_part = part ? tail : nullptr;
  }
}

hipError_t launch_ffn_tiles(const moe_config& c, const WsLayout& L, const int32_t* offsets, hipStream_t stream) {
  const int A = (int)(c.n_tokens * c.top_k);
  if (A == 0) return hipGetLastError();
  tile_table_kernel<<<1, 1024, 0, stream>>>(offsets, c.n_experts, A, ffn_tile_rows(c), ffn_narrow_rows(c),
                                            ffn_max_m_tiles(c), L.tiles, L.err);
  return hipGetLastError();
}

hipError_t launch_ffn_up(const moe_config& c, const WsLayout& L, const void* x_sorted,
                         const int32_t* offsets, const void* w1, const void* w3, const void* b1,
                         hipStream_t stream, int xs_kp) {
  const int A = (int)(c.n_tokens * c.top_k);
  if (A == 0) return hipGetLastError();
  GemmArgs g{};
  g.a = x_sorted;
  g.b0 = w1;
  g.b1 = w3;
  g.bias = (c.act == MOE_ACT_GELU && c.has_bias) ? b1 : nullptr;
  g.c = L.h;
  g.tiles = L.tiles;
  g.K = c.d_model;
  g.n_out = c.d_ff;
  if (c.weight_layout == MOE_WEIGHTS_TILED) {
    g.b_kp = tiled_k(c, 0);
    g.b_np = tiled_n(c, 0);
  }
  if (ffn_h_tiled(c)) g.c_kp = tiled_k(c, 1);  // h in the tiled layout (K of the down projection)
  g.a_kp = xs_kp;                                // x_sorted tiled (moe_forward, dropless bf16) or not
  const int mt = ffn_max_m_tiles(c);
  if (c.dtype == MOE_BF16) {
    g.n_tiles_n = (c.d_ff + (c.act == MOE_ACT_SWIGLU ? 127 : 255)) / (c.act == MOE_ACT_SWIGLU ? 128 : 256);
    const int grid = persistent_grid();
    const bool nar = ffn_narrow_rows(c) > 0;
    if (c.act == MOE_ACT_SWIGLU) launch_bf16_gemm<kEpiSwiglu>(nar, grid, g, stream);
    else launch_bf16_gemm<kEpiGelu>(nar, grid, g, stream);
  } else {
    dim3 grid(mt, (c.d_ff + kFBN - 1) / kFBN);
    if (c.act == MOE_ACT_SWIGLU) expert_gemm_f32_kernel<kEpiSwiglu><<<grid, 256, 0, stream>>>(g);
    else expert_gemm_f32_kernel<kEpiGelu><<<grid, 256, 0, stream>>>(g);
  }
  return hipGetLastError();
}

hipError_t launch_down(const moe_config& c, const int* tiles, int max_m_tiles, const void* h, int K, const void* w2,
                       const void* b2, const float* gate, bool pre_gated, void* y, float* tail_part,
                       hipStream_t stream, bool w2_tiled, int h_kp) {
  GemmArgs g{};
  g.a = h;
  g.a_kp = h_kp;
  g.b0 = w2;
  if (w2_tiled) {
    g.b_kp = tiled_k(c, 1);
    g.b_np = tiled_n(c, 1);
  }
  g.bias = (c.act == MOE_ACT_GELU && c.has_bias) ? b2 : nullptr;
  g.gate = gate;
  g.pre_gated = pre_gated ? 1 : 0;
  g.c = y;
  g.tiles = tiles;
  g.K = K;
  g.n_out = c.d_model;
  if (c.dtype == MOE_BF16) {
    g.n_tiles_n = (c.d_model + 255) / 256;
    const int grid = persistent_grid();
    if (!tail_part) {
      launch_bf16_gemm<kEpiDown>(down_narrow(c), grid, g, stream);
    } else {
      // whole rounds of tiles, then the last partial round cut along K so that it fills the
      // chip, then the fixed-order sum of the pieces with the epilogue
      g.partial = tail_part;
      g.grid = grid;
      g.nar_ok = down_narrow(c) ? 1 : 0;  // what the two GEMM launches use
      launch_bf16_gemm<kEpiDown, 1>(down_narrow(c), grid, g, stream);
      launch_bf16_gemm<kEpiDown, 2>(down_narrow(c), grid, g, stream);
      tail_reduce_kernel<<<kTailReduceGrid, 256, 0, stream>>>(g);
    }
  } else {
    dim3 grid(max_m_tiles, (c.d_model + kFBN - 1) / kFBN);
    expert_gemm_f32_kernel<kEpiDown><<<grid, 256, 0, stream>>>(g);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_down(const moe_config& c, const WsLayout& L, const int32_t* offsets,
                           const void* w2, const void* b2, const float* gate_sorted,
                           void* y_sorted, hipStream_t stream) {
  if (c.n_tokens * c.top_k == 0) return hipGetLastError();
  return launch_down(c, L.tiles, ffn_max_m_tiles(c), L.h, c.d_ff, w2, b2, gate_sorted, false, y_sorted, L.tail_part,
                     stream, c.weight_layout == MOE_WEIGHTS_TILED, ffn_h_tiled(c) ? tiled_k(c, 1) : 0);
}

hipError_t launch_dense_tiles(int n, int bm, int* tiles, hipStream_t stream) {
  dense_tiles_kernel<<<1, 256, 0, stream>>>(n, bm, tiles);
  return hipGetLastError();
}

hipError_t launch_up_save(const moe_config& c, const int* tiles, const void* a, const void* w1, const void* w3,
                          const void* b1, const float* gate, int n_out, void* pre, void* hw, hipStream_t stream) {
  GemmArgs g{};
  g.a = a;
  g.b0 = w1;
  g.b1 = w3;
  g.bias = (c.act == MOE_ACT_GELU && c.has_bias) ? b1 : nullptr;
  g.gate = gate;
  g.c = hw;
  g.c2 = pre;
  g.tiles = tiles;
  g.K = c.d_model;
  g.n_out = n_out;
  if (c.act == MOE_ACT_SWIGLU) {
    g.n_tiles_n = (n_out + 127) / 128;
    launch_bf16_gemm<kEpiSwigluSave>(ffn_narrow_rows(c) > 0, persistent_grid(), g, stream);
  } else {
    g.n_tiles_n = (n_out + 255) / 256;
    launch_bf16_gemm<kEpiGeluSave>(ffn_narrow_rows(c) > 0, persistent_grid(), g, stream);
  }
  return hipGetLastError();
}

hipError_t launch_shared(const moe_config& c, const WsLayout& L, const void* x, const void* s_w1,
                         const void* s_w3, const void* s_b1, const void* s_w2, const void* s_b2,
                         void* y_shared, hipStream_t stream) {
  const int N = (int)c.n_tokens;
  if (N == 0 || c.d_ff_shared <= 0) return hipGetLastError();
  const int bm = ffn_tile_rows(c);
  dense_tiles_kernel<<<1, 256, 0, stream>>>(N, bm, L.tiles);
  const int mt = shared_m_tiles(c);
  const bool bias = c.act == MOE_ACT_GELU && c.has_bias;
  GemmArgs g{};
  g.a = x;
  g.b0 = s_w1;
  g.b1 = s_w3;
  g.bias = bias ? s_b1 : nullptr;
  g.c = L.h;
  g.tiles = L.tiles;
  g.K = c.d_model;
  g.n_out = c.d_ff_shared;
  if (c.dtype == MOE_BF16) {
    g.n_tiles_n = (c.d_ff_shared + (c.act == MOE_ACT_SWIGLU ? 127 : 255)) / (c.act == MOE_ACT_SWIGLU ? 128 : 256);
    if (c.act == MOE_ACT_SWIGLU) launch_bf16_gemm<kEpiSwiglu>(false, persistent_grid(), g, stream);
    else launch_bf16_gemm<kEpiGelu>(false, persistent_grid(), g, stream);
  } else {
    dim3 grid(mt, (c.d_ff_shared + kFBN - 1) / kFBN);
    if (c.act == MOE_ACT_SWIGLU) expert_gemm_f32_kernel<kEpiSwiglu><<<grid, 256, 0, stream>>>(g);
    else expert_gemm_f32_kernel<kEpiGelu><<<grid, 256, 0, stream>>>(g);
  }
  GemmArgs d{};
  d.a = L.h;
  d.b0 = s_w2;
  d.bias = bias ? s_b2 : nullptr;
  d.gate = nullptr;
  d.c = y_shared;
  d.tiles = L.tiles;
  d.K = c.d_ff_shared;
  d.n_out = c.d_model;
  if (c.dtype == MOE_BF16) {
    d.n_tiles_n = (c.d_model + 255) / 256;
    launch_bf16_gemm<kEpiDown>(false, persistent_grid(), d, stream);
  } else {
    dim3 grid(mt, (c.d_model + kFBN - 1) / kFBN);
    expert_gemm_f32_kernel<kEpiDown><<<grid, 256, 0, stream>>>(d);
  }
  return hipGetLastError();
}

// Tiled weights (MOE_WEIGHTS_TILED, layout in moe.h): one thread per 16-byte chunk of the
// tiled copy, which is written in order; each chunk is 8 consecutive reduction elements of
// one row, read from the row-major source or zero in the padding (K is a multiple of 8, so a
// chunk is wholly inside or outside the row).
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint4* __restrict__ w, uint4* __restrict__ out,
                                                           long long n_chunks, int N, int K, int Np, int Kp) {
  const long long per_expert = (long long)Np * Kp / 8;
  const int kc = K / 8;
  for (long long q = (long long)blockIdx.x * blockDim.x + threadIdx.x; q < n_chunks;
       q += (long long)gridDim.x * blockDim.x) {
    const long long e = q / per_expert;
    const long long r = q - e * per_expert;      // chunk within the expert
    const long long blk = r / (kTiledRows * Kp / 8);  // 128-row block
    const int rr = (int)(r - blk * (kTiledRows * Kp / 8));
    const int slab = rr / (kTiledRows * kTiledK / 8);
    const int within = rr - slab * (kTiledRows * kTiledK / 8);
    const int row = (int)blk * kTiledRows + within / (kTiledK / 8);
    const int k8 = slab * (kTiledK / 8) + within % (kTiledK / 8);  // chunk index along K
    out[q] = (row < N && k8 < kc) ? w[(e * N + row) * (long long)kc + k8] : make_uint4(0, 0, 0, 0);
  }
}

hipError_t launch_pack_weights(const moe_config& c, int which, const void* w, void* w_tiled, hipStream_t stream) {
  const int N = which ? c.d_model : c.d_ff, K = which ? c.d_ff : c.d_model;
  const long long n_chunks = (long long)packed_weight_elems(c, which) / 8;
  if (n_chunks == 0) return hipGetLastError();
  const int grid = (int)std::min<long long>((n_chunks + 255) / 256, 65536);
  pack_weights_kernel<<<grid, 256, 0, stream>>>(static_cast<const uint4*>(w), static_cast<uint4*>(w_tiled),
                                                n_chunks, N, K, tiled_n(c, which), tiled_k(c, which));
  return hipGetLastError();
}

}  // namespace moe
