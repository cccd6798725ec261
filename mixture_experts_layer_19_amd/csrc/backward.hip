// Backward of the layer (bfloat16, dropless): gradients of
//     J = <dy, y> + aux_coef L + z_coef z_loss
// with respect to x, the router and every expert weight, by the chain rule through the
// forward steps ("Mixture of Experts: routing, sorted dispatch, Switch aux loss, aux-free
// bias" (L7.8) §2.1 output equation and routers table, §2.3 load-balancing loss, §2.5: the
// selection bias never weighs; "15. Mixture of Experts" (RustingBrain) §15.3 z-loss).
//
// Nothing is kept from the forward: routing, dispatch and the up projection are recomputed
// (the up projection by the forward's GEMM with an epilogue that keeps the pre-activations).
// Per expert e with sorted rows a (gate w_a, token t(a)), SwiGLU:
//   dh'_a   = dy_t W2_e                       (unscaled: dgate_a = <dh'_a, h_a> = <dy_t, o_a>)
//   dh_a    = w_a dh'_a;  dg = dh u s (1 + g (1 - s)), du = dh g s   (s = sigmoid(g))
//   dx_s_a  = dg W1_e + du W3_e;   dW2_e = sum_a dy_t^T (w_a h_a);   dW1_e = sum_a dg^T x_t
// GELU: da = dh gelu'(a) with a = x W1^T + b1, plus db1 / db2 column sums and the b2 term of
// dgate. The router gradient dz follows from dgate through the routers table's weights, the
// Switch loss through P = mean softmax(z) (f is piecewise constant) and the z-loss; then
// dx += dz W_g and dW_g = dz^T x.
//
// The products run on one grouped bfloat16 MFMA kernel (bwd_gemm_kernel) whose B operand is
// always stored with its output axis contiguous (weights [K][N] or activations [rows][N]),
// and whose A operand is either the row operand (grouped mode: expert-sorted rows, K
// contiguous) or, for weight gradients, a second activation with M contiguous (ragged K =
// the expert's rows). Operands stream into LDS as stored (global_load_lds); those that are
// not K-contiguous are turned into MFMA fragments by gfx950's LDS transpose read.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBM = 256, kBN = 256, kBK = 32, kThreads = 512, kStages = 4;
constexpr int kStageStride = 72;         // epilogue staging row (floats, 64 columns + 8): the
                                         // two half-waves, 4 rows apart, hit disjoint banks

enum Mode { kGrouped = 0, kWgrad = 1 };
enum Epi { kStoreT = 0, kStoreF32 = 1, kSwigluBwd = 2, kGeluBwd = 3 };

struct BwdGemm {
  // Segment s of the reduction: grouped: k in [0, klen[s]) of a[s] (rows of lda elements, K
  // contiguous) and b[s] (k rows of ldb elements, N contiguous, + e * b_estride per
  // expert); the segments follow each other along K (each padded to a multiple of 8).
  // wgrad: both operands are [rows][lda | ldb] with M (resp. N) contiguous; expert e reduces
  // over its rows [offsets[e], offsets[e+1]) (offsets null: rows [0, klen[0])), and a
  // second segment, when a[1] is set, repeats the same rows with a[1] / b[1].
  const uint16_t* a[2];
  const uint16_t* b[2];
  long long lda, ldb, b_estride;
  int klen[2];
  int M, N;
  const int* tiles;
  const int* offsets;
  int n_experts;
  int n_tiles_n;
  // output: grouped rows row0 + r; wgrad rows m of expert e (m < m_split: c, else c_hi)
  void* c;
  void* c_hi;
  long long ldc, c_estride;
  int m_split;
  const float* c_in;    // kStoreF32: added before the store (may alias c)
  const uint16_t* zero; // 16 zero bytes (the source of masked copies)
  // wgrad with split K: the expert's rows are cut into ksplit runs; run sp writes float32
  // partials to kpart [ksplit][n_experts][M][N] (reduced by wgrad_reduce_kernel)
  int ksplit;
  float* kpart;
  // weight gradients, balanced schedule (or null): cost prefix [E+1], per-XCD counters [8]
  const long long* sched;
  int* sched_cnt;
  // grouped, split tail (or null): workgroups [0, grid_static) take the first
  // floor(S / cu_grid) * cu_grid tiles, the later ones the K pieces of the rest, writing float32
  // partials [kMaxTailItems][256][256] (summed by bwd_tail_reduce_kernel)
  float* tpart;
  int grid_static, cu_grid;
  // activation backward (grouped): pre-activations, gates, row partials of <dh', h>
  const uint16_t* pre;  // SwiGLU [rows][2 N] (gate | up), GELU [rows][N]
  const float* gate;    // [rows] or null (1)
  float* part;          // [rows][n_part] or null
  int n_part;
};

MOE_DEV float gelu_grad(float a) {
  return 0.5f * (1.0f + erff(a * 0.70710678118654752440f)) + a * 0.39894228040143267794f * expf(-0.5f * a * a);
}

MOE_DEV void unpack8(const uint4& v, float* o) {
  o[0] = __uint_as_float(v.x << 16);
  o[1] = __uint_as_float(v.x & 0xffff0000u);
  o[2] = __uint_as_float(v.y << 16);
  o[3] = __uint_as_float(v.y & 0xffff0000u);
  o[4] = __uint_as_float(v.z << 16);
  o[5] = __uint_as_float(v.z & 0xffff0000u);
  o[6] = __uint_as_float(v.w << 16);
  o[7] = __uint_as_float(v.w & 0xffff0000u);
}
MOE_DEV uint4 pack8(const float* f) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

// slabs of a grouped product's reduction (each segment padded to whole slabs)
MOE_DEV int grouped_slabs(const BwdGemm& g) {
  return (g.klen[0] + kBK - 1) / kBK + (g.klen[1] + kBK - 1) / kBK;
}

// ---------------------------------------------------------------------------------------
// Grouped bfloat16 GEMM on MFMA (v_mfma_f32_32x32x16_bf16, float32 accumulation).
// Workgroup tile 256 x 256, eight waves (two per SIMD) of 64 x 128 (2 x 4 blocks of
// 32 x 32), one workgroup per CU. K advances 32 at a time through four LDS stages (128 KiB),
// three slabs in flight while one is multiplied.
// Grid: 8 * ceil(S / 8) workgroups for S tiles; workgroup b runs on XCD b mod 8 and takes
// tile (b mod 8) * ceil(S / 8) + b / 8, so each XCD works through a contiguous run of the
// tile order (expert-major, supertiles of 8 m-tiles x 4 n-tiles) and shares its operands in
// its own L2.
// ---------------------------------------------------------------------------------------
template <int MODE, int EPI>
__global__ __launch_bounds__(kThreads, 2) void bwd_gemm_kernel(BwdGemm g) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[kStages][kBM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kStages][kBN * kBK];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;
  const int NT = g.n_tiles_n;

  // ---- tile
  long long S;
  int MTe = 0;
  if (MODE == kGrouped) {
    S = (long long)g.tiles[0] * NT;
  } else {
    MTe = (g.M + kBM - 1) / kBM;
    S = (long long)g.n_experts * MTe * NT * g.ksplit;
  }
  // Static mapping: one tile per workgroup. Weight gradients with a schedule (g.sched): the
  // tile order is cut into 8 runs of equal cost (a tile costs its expert's slabs plus a fixed
  // overhead), one per XCD, and the XCD's persistent workgroups take the run's tiles in order
  // from an atomic counter, so a large expert's long tiles spread over the whole run.
  const bool dyn = MODE == kWgrad && g.sched != nullptr;
  int tail_w = -1, tail_q = 1;  // split-tail item (grouped) and the tail's pieces per tile
  const int xcd = blockIdx.x & 7;
  long long run_lo = 0, run_hi = 0, s = 0;
  if (dyn) {
    const long long tpe = (long long)MTe * NT;
    auto run_start = [&](int x) -> long long {
      const long long total = g.sched[g.n_experts];
      const long long target = total / 8 * x + (total % 8) * x / 8;
      int lo = 0, hi = g.n_experts;  // the last expert whose prefix is <= target
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (g.sched[mid] <= target) lo = mid;
        else hi = mid - 1;
      }
      if (lo >= g.n_experts) return (long long)g.n_experts * tpe;
      const long long per_tile = (g.sched[lo + 1] - g.sched[lo]) / tpe;
      return (long long)lo * tpe + min(tpe, (target - g.sched[lo]) / max(per_tile, 1ll));
    };
    run_lo = run_start(xcd);
    run_hi = xcd == 7 ? (long long)g.n_experts * tpe : run_start(xcd + 1);
  } else if (MODE == kGrouped && g.tpart) {
    const long long S_main = S / g.cu_grid * g.cu_grid;
    if ((int)blockIdx.x >= g.grid_static) {
      const int q = tail_pieces(S - S_main, grouped_slabs(g), g.cu_grid);
      tail_w = (int)blockIdx.x - g.grid_static;
      if (tail_w >= (S - S_main) * q) return;
      s = S_main + tail_w / q;
      tail_q = q;
    } else {
      const long long per = (S_main + 7) / 8;
      const long long slot = blockIdx.x >> 3;
      s = (long long)xcd * per + slot;
      if (slot >= per || s >= S_main) return;
    }
  } else {
    const long long per = (S + 7) / 8;
    const long long slot = blockIdx.x >> 3;
    s = (long long)xcd * per + slot;
    if (slot >= per || s >= S) return;
  }
  __shared__ int s_fetch;

  for (int iter = 0;; ++iter) {
  if (dyn) {
    if (tid == 0) s_fetch = atomicAdd(g.sched_cnt + xcd, 1);
    __syncthreads();
    s = run_lo + s_fetch;
    __syncthreads();
    if (s >= run_hi) break;
  } else if (iter > 0) {
    break;
  }

  int e, mt, nt, row0 = 0, rows = 0, m0 = 0, r0 = 0, kr = 0, sp = 0;
  if (MODE == kGrouped) {
    const int* probe = g.tiles + kTileHdr + kTileInts * (int)(s / NT);
    e = probe[0];
    const int ts = probe[3], me = probe[4];
    supertile(s - (long long)ts * NT, me, NT, &mt, &nt);
    const int* tq = g.tiles + kTileHdr + kTileInts * (ts + mt);
    row0 = tq[1];
    rows = tq[2];
  } else {
    // split sp of ksplit (outermost) takes the sp-th of ksplit near-equal runs of the rows
    const long long per_split = (long long)g.n_experts * MTe * NT;
    sp = (int)(s / per_split);
    const long long se = s - sp * per_split;
    e = (int)(se / ((long long)MTe * NT));
    supertile(se - (long long)e * MTe * NT, MTe, NT, &mt, &nt);
    m0 = mt * kBM;
    r0 = g.offsets ? g.offsets[e] : 0;
    const int r1 = g.offsets ? g.offsets[e + 1] : g.klen[0];
    const int all = max(r1 - r0, 0);
    const int chunk = (all + g.ksplit - 1) / g.ksplit;
    r0 += min(sp * chunk, all);
    kr = max(min(chunk, all - sp * chunk), 0);
  }
  const int n0 = nt * kBN;
  const int M = g.M, N = g.N;

  // ---- reduction length: each segment padded to whole slabs, so a slab lies in one segment
  int kp0, ktot, klen0, klen1;
  if (MODE == kGrouped) {
    klen0 = g.klen[0];
    klen1 = g.klen[1];
    kp0 = (klen0 + kBK - 1) / kBK * kBK;
    ktot = kp0 + (klen1 + kBK - 1) / kBK * kBK;
  } else {
    klen0 = klen1 = kr;
    kp0 = (kr + kBK - 1) / kBK * kBK;
    ktot = g.a[1] ? 2 * kp0 : kp0;
  }
  int nk = ktot / kBK;
  int kso = 0;  // first slab (a split-tail piece covers slabs [kso, kso + nk))
  if (tail_w >= 0) {
    const int piece = tail_w % tail_q;
    kso = piece * nk / tail_q;
    nk = (piece + 1) * nk / tail_q - kso;
  }

  // ---- operand stages in LDS, written by global_load_lds_dwordx4 (16 bytes per lane,
  // 1 KiB per wave instruction); a lane whose 16 bytes lie outside the operand (rows past the
  // tile or the expert, columns past N, k past a segment) copies zeros from g.zero instead.
  //   A, K-contiguous (grouped): [256 rows][32 k], 64-byte rows; chunk c of row r at physical
  //     chunk c ^ ((r >> 2) & 3); MFMA fragments by ds_read_b128.
  //   A, M-contiguous (wgrad):   [32 k][256 m]; B: [32 k][256 n]; 512-byte rows.
  //     Chunk c (8 columns) of k-row r at physical chunk c ^ ((r & 3) << 2); fragments by two
  //     ds_read_b64_tr_b16 (in each 16-lane group, lane 4 q + p reads 4 columns at 4 p of
  //     k-row q and lane i receives column i at 4 consecutive k): the four k-rows a half-wave
  //     reads then sit in four different 64-byte bank windows.
  // Four stages: slab kt + 3 is copied while slab kt is multiplied (one barrier per slab).
  // Per lane and copy instruction (2 of A, 4 of B): the element address at slab-local k = 0
  // of segment 0 (q*), the lane's k within the slab (lk*) and whether its row / column
  // exists (ok*); per slab only a uniform offset is added. Segment 1 is segment 0's address
  // plus a uniform distance (same row or column, other matrix).
  const uint16_t* qa[2];
  const uint16_t* qb[2];
  int lka[2], lkb[2];
  bool oka[2], okb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int inst = 2 * wave + i;  // 16 copy instructions per operand and slab
    if (MODE == kGrouped) {
      const int r = inst * 16 + (lane >> 2);
      lka[i] = 8 * ((lane & 3) ^ ((r >> 2) & 3));
      oka[i] = r < rows;
      qa[i] = g.a[0] + (size_t)(row0 + min(r, max(rows - 1, 0))) * g.lda + lka[i];
    } else {
      lka[i] = inst * 2 + (lane >> 5);
      const int m = m0 + 8 * ((lane & 31) ^ ((lka[i] & 3) << 2));
      oka[i] = m < M;
      qa[i] = g.a[0] + (size_t)(r0 + lka[i]) * g.lda + min(m, M - 1);
    }
    lkb[i] = inst * 2 + (lane >> 5);
    const int n = n0 + 8 * ((lane & 31) ^ ((lkb[i] & 3) << 2));
    okb[i] = n < N;
    const size_t row = (MODE == kGrouped) ? (size_t)lkb[i] : (size_t)(r0 + lkb[i]);
    const uint16_t* b0 = g.b[0] + (MODE == kGrouped ? (size_t)e * g.b_estride : 0);
    qb[i] = b0 + row * g.ldb + min(n, N - 8);
  }
  // uniform distance from segment 0 to segment 1 (elements)
  const long long da1 = g.a[1] ? (long long)(g.a[1] - g.a[0]) : 0;
  const long long db1 = g.b[1] ? (long long)(g.b[1] - g.b[0]) : 0;
  auto issue = [&](int slab, int buf) {
    const int kbase = (kso + slab) * kBK;
    const int sg = kbase >= kp0 ? 1 : 0;     // uniform
    const int kl = kbase - sg * kp0;         // slab start within the segment
    const int klen = sg ? klen1 : klen0;
    const long long ua = (MODE == kGrouped) ? (long long)kl + (sg ? da1 : 0)
                                            : (long long)kl * g.lda + (sg ? da1 : 0);
    const long long ub = (long long)kl * g.ldb + (sg ? db1 : 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int inst = 2 * wave + i;
      const bool ok = oka[i] && kl + lka[i] < klen;
      lds_dma16(ok ? qa[i] + ua : g.zero, &sA[buf][inst * 512]);   // 1 KiB = 512 elements
      const bool okb_ = okb[i] && kl + lkb[i] < klen;
      lds_dma16(okb_ ? qb[i] + ub : g.zero, &sB[buf][inst * 512]);
    }
  };

  // fragment addresses (elements within a stage) of this lane
  const int tg = lane >> 4, tq = (lane & 15) >> 2, tp = lane & 3;  // transpose-read roles
  int offa[2][2][2], offb[2][4][2];  // [ks][block][read]; the K-contiguous A uses [ks][block][0]
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int k = 16 * ks + 8 * (tg >> 1) + 4 * rd + tq;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (MODE == kGrouped) {
          const int r = wm * 64 + 32 * i + (lane & 31);
          offa[ks][i][rd] = r * kBK + (((2 * ks + (lane >> 5)) ^ ((r >> 2) & 3)) * 8);
        } else {
          const int m = wm * 64 + 32 * i + 16 * (tg & 1) + 4 * tp;
          offa[ks][i][rd] = k * kBM + (((m >> 3) ^ (tq << 2)) * 8) + 4 * ((m >> 2) & 1);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = wn * 128 + 32 * j + 16 * (tg & 1) + 4 * tp;
        offb[ks][j][rd] = k * kBN + (((n >> 3) ^ (tq << 2)) * 8) + 4 * ((n >> 2) & 1);
      }
    }
  }
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  auto tr_read = [](const uint16_t* base, int off) -> v4i16 {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds_void*)(base + off));
  };
  auto frag8 = [](v4i16 lo, v4i16 hi) -> bf16x8 {
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  if (nk > 0) {
    issue(0, 0);
    issue(min(1, nk - 1), 1);
    issue(min(2, nk - 1), 2);
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt % kStages;
      wait_vm_lds<8>();  // this wave's 4 copies of slab kt have landed (kt + 1, kt + 2 may not)
      stage_barrier();   // every wave's have, and every wave is done with slab kt - 1
      // slab kt + 3 into the stage slab kt - 1 used (past the end: the last slab again, into
      // a stage that is never read, which keeps the count above exact)
      issue(min(kt + 3, nk - 1), (kt + 3) % kStages);
      const uint16_t* a_st = sA[buf];
      const uint16_t* b_st = sB[buf];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 fa[2], fb[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (MODE == kGrouped) fa[i] = *reinterpret_cast<const bf16x8*>(a_st + offa[ks][i][0]);
          else fa[i] = frag8(tr_read(a_st, offa[ks][i][0]), tr_read(a_st, offa[ks][i][1]));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = frag8(tr_read(b_st, offb[ks][j][0]), tr_read(b_st, offb[ks][j][1]));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
    }
    wait_vm_lds<0>();  // the copies past the end land before the stages are reused
  }
  __syncthreads();

  // ---- epilogue: per 32-row block i and column pair jp (64 columns), the wave stages its
  // float32 accumulators in its own LDS area (rows padded to kStageStride floats, so the
  // half-waves, 4 rows apart, hit disjoint banks); then lane l takes row 8 it + (l >> 3)
  // (it = 0..3), columns 8 (l & 7) .. + 7, so one store instruction covers 8 rows x 64
  // columns (128 contiguous bytes per row in bfloat16).
  float* st = reinterpret_cast<float*>(wave < 4 ? &sA[0][0] : &sB[0][0]) + (wave & 3) * 32 * kStageStride;
  const int lr = lane >> 3, lc = 8 * (lane & 7);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float psum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      // SwiGLU backward: this step's gate and up pre-activations and gates for the lane's 4
      // rows, all requested before the accumulators are staged, so one memory round trip
      // overlaps the staging (rows and columns clamped into the tile's valid range; extra
      // values unused). The GELU backward loads per row: hoisted, its loads measured slower.
      uint4 pre_a[4], pre_b[4];
      float gate_w[4];
      if constexpr (EPI == kSwigluBwd) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int rl = wm * 64 + 32 * i + 8 * it + lr;
          const size_t grow = (size_t)(row0 + min(rl, max(rows - 1, 0)));
          const int cc = min(n0 + wn * 128 + 64 * jp + lc, N - 8);
          pre_a[it] = *reinterpret_cast<const uint4*>(g.pre + grow * 2 * (size_t)N + cc);
          pre_b[it] = *reinterpret_cast<const uint4*>(g.pre + grow * 2 * (size_t)N + N + cc);
          gate_w[it] = g.gate ? g.gate[grow] : 1.f;
        }
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          st[((v >> 2) * 8 + 4 * (lane >> 5) + (v & 3)) * kStageStride + 32 * jj + (lane & 31)] = acc[i][2 * jp + jj][v];
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int er = 8 * it + lr;
        const int rl = wm * 64 + 32 * i + er;  // tile row of this lane's output row
        float v8[8];
        {
          const float4 f0 = *reinterpret_cast<const float4*>(st + er * kStageStride + lc);
          const float4 f1 = *reinterpret_cast<const float4*>(st + er * kStageStride + lc + 4);
          v8[0] = f0.x; v8[1] = f0.y; v8[2] = f0.z; v8[3] = f0.w;
          v8[4] = f1.x; v8[5] = f1.y; v8[6] = f1.z; v8[7] = f1.w;
        }
        const int cc = n0 + wn * 128 + 64 * jp + lc;
        bool row_ok;
        size_t grow = 0;                       // grouped: sorted row
        uint16_t* crow = nullptr;              // wgrad: output row
        float* prow = nullptr;                 // wgrad with split K: this split's float32 partial row
        if (MODE == kGrouped) {
          row_ok = rl < rows;
          grow = (size_t)(row0 + rl);
        } else {
          const int m = m0 + rl;
          row_ok = m < M;
          if (row_ok && g.kpart)
            prow = g.kpart + (((size_t)sp * g.n_experts + e) * M + m) * (size_t)N;
          else if (row_ok)
            crow = (m < g.m_split) ? static_cast<uint16_t*>(g.c) + (size_t)e * g.c_estride + (size_t)m * g.ldc
                                   : static_cast<uint16_t*>(g.c_hi) + (size_t)e * g.c_estride + (size_t)(m - g.m_split) * g.ldc;
        }
        if (!row_ok || cc >= N) continue;
        if (MODE == kGrouped && tail_q > 1) {
          // a K piece of a split-tail tile: float32 partial of the tile, [256 rows][256 cols]
          float* tp = g.tpart + (size_t)tail_w * (kBM * kBN) + (size_t)rl * kBN + (cc - n0);
          *reinterpret_cast<float4*>(tp) = make_float4(v8[0], v8[1], v8[2], v8[3]);
          *reinterpret_cast<float4*>(tp + 4) = make_float4(v8[4], v8[5], v8[6], v8[7]);
        } else if (EPI == kStoreT && MODE == kWgrad && prow) {
          *reinterpret_cast<float4*>(prow + cc) = make_float4(v8[0], v8[1], v8[2], v8[3]);
          *reinterpret_cast<float4*>(prow + cc + 4) = make_float4(v8[4], v8[5], v8[6], v8[7]);
        } else if (EPI == kStoreT) {
          uint16_t* dst = (MODE == kGrouped) ? static_cast<uint16_t*>(g.c) + grow * g.ldc + cc : crow + cc;
          *reinterpret_cast<uint4*>(dst) = pack8(v8);
        } else if (EPI == kStoreF32) {
          float* dst = static_cast<float*>(g.c) + grow * g.ldc + cc;
          if (g.c_in) {
            const float* src = g.c_in + grow * g.ldc + cc;
            const float4 p0 = *reinterpret_cast<const float4*>(src);
            const float4 p1 = *reinterpret_cast<const float4*>(src + 4);
            v8[0] += p0.x; v8[1] += p0.y; v8[2] += p0.z; v8[3] += p0.w;
            v8[4] += p1.x; v8[5] += p1.y; v8[6] += p1.z; v8[7] += p1.w;
          }
          *reinterpret_cast<float4*>(dst) = make_float4(v8[0], v8[1], v8[2], v8[3]);
          *reinterpret_cast<float4*>(dst + 4) = make_float4(v8[4], v8[5], v8[6], v8[7]);
        } else if (EPI == kSwigluBwd) {
          const float w = gate_w[it];
          float gg[8], uu[8], dg[8], du[8];
          unpack8(pre_a[it], gg);
          unpack8(pre_b[it], uu);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float sg = sigmoid_f(gg[q]);
            psum[it] += v8[q] * (gg[q] * sg * uu[q]);
            const float dh = w * v8[q];
            dg[q] = dh * uu[q] * sg * (1.f + gg[q] * (1.f - sg));
            du[q] = dh * gg[q] * sg;
          }
          uint16_t* dst = static_cast<uint16_t*>(g.c) + grow * g.ldc + cc;
          *reinterpret_cast<uint4*>(dst) = pack8(dg);
          *reinterpret_cast<uint4*>(dst + N) = pack8(du);
        } else {  // kGeluBwd
          const float w = g.gate ? g.gate[grow] : 1.f;
          float aa[8], da[8];
          unpack8(*reinterpret_cast<const uint4*>(g.pre + grow * (size_t)N + cc), aa);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            psum[it] += v8[q] * gelu_erf(aa[q]);
            da[q] = w * v8[q] * gelu_grad(aa[q]);
          }
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(g.c) + grow * g.ldc + cc) = pack8(da);
        }
      }
      __builtin_amdgcn_wave_barrier();  // the next pair overwrites the staging area
    }
    if ((EPI == kSwigluBwd || EPI == kGeluBwd) && g.part) {
      // a row's 8 lanes hold its partial over this wave's 128 columns: fixed butterfly
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        float p = psum[it];
        p += __shfl_xor(p, 1, kWave);
        p += __shfl_xor(p, 2, kWave);
        p += __shfl_xor(p, 4, kWave);
        const int rl = wm * 64 + 32 * i + 8 * it + lr;
        if ((lane & 7) == 0 && rl < rows) g.part[(size_t)(row0 + rl) * g.n_part + 2 * nt + wn] = p;
      }
    }
  }
  __syncthreads();  // the next tile's copies reuse the stages
  }
}

// The split tail of a grouped bf16 product: out = bf16(sum of the tail tile's pieces, in
// piece order). Unit (t, rg): rows 4 rg .. 4 rg + 3 of tail tile t, a thread per 4 columns;
// a fixed grid walks the units (the tail's size is known on the device only).
constexpr int kBwdTailReduceGrid = 2048;
MOE_DEV void bwd_tail_reduce_unit(const BwdGemm& g, long long S_main, int q, int t, int rg) {
  const int NT = g.n_tiles_n;
  const long long s = S_main + t;
  const int* probe = g.tiles + kTileHdr + kTileInts * (int)(s / NT);
  const int ts = probe[3], me = probe[4];
  int mt, nt;
  supertile(s - (long long)ts * NT, me, NT, &mt, &nt);
  const int* tq = g.tiles + kTileHdr + kTileInts * (ts + mt);
  const int row0 = tq[1], rows = tq[2];
  const int r = rg * 4 + (threadIdx.x >> 6);
  const int c4 = (threadIdx.x & 63) * 4;
  const int col = nt * kBN + c4;
  if (r >= rows || col >= g.N) return;
  const float* pt = g.tpart + (size_t)t * q * (kBM * kBN) + (size_t)r * kBN + c4;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < q; ++p) {
    const float4 x = *reinterpret_cast<const float4*>(pt + (size_t)p * (kBM * kBN));
    v[0] += x.x; v[1] += x.y; v[2] += x.z; v[3] += x.w;
  }
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.c) + (size_t)(row0 + r) * g.ldc + col) =
      make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
__global__ __launch_bounds__(256) void bwd_tail_reduce_kernel(BwdGemm g) {
  const long long S = (long long)g.tiles[0] * g.n_tiles_n;
  const long long S_main = S / g.cu_grid * g.cu_grid;
  const int q = tail_pieces(S - S_main, grouped_slabs(g), g.cu_grid);
  if (q <= 1) return;
  constexpr int kGroups = kBM / 4;  // row groups of a tail tile
  const long long units = (S - S_main) * kGroups;
  for (long long u = blockIdx.x; u < units; u += gridDim.x)
    bwd_tail_reduce_unit(g, S_main, q, (int)(u / kGroups), (int)(u % kGroups));
}

// Cost prefix of the weight-gradient schedule: sched[e] = sum over experts e' < e of
// tiles_per_expert * (slabs(rows of e') + kTileCost), and the 8 per-XCD counters cleared.
constexpr int kTileCost = 4;  // a tile's fixed cost (prologue, epilogue) in slabs
__global__ __launch_bounds__(1024) void wgrad_sched_kernel(const int* __restrict__ offsets, int E, long long tpe,
                                                           long long* __restrict__ sched, int* __restrict__ cnt) {
  __shared__ long long s_scan[kMaxExperts];
  const int e = threadIdx.x;
  long long c = 0;
  if (e < E) c = tpe * ((max(offsets[e + 1] - offsets[e], 0) + kBK - 1) / kBK + kTileCost);
  if (e < kMaxExperts) s_scan[e] = c;
  __syncthreads();
  for (int o = 1; o < E; o <<= 1) {
    long long v = 0;
    if (e < E && e >= o) v = s_scan[e - o];
    __syncthreads();
    if (e < E) s_scan[e] += v;
    __syncthreads();
  }
  if (e < E) sched[e + 1] = s_scan[e];
  if (e == 0) sched[0] = 0;
  if (e < 8) cnt[e] = 0;
}

// ---------------------------------------------------------------------------------------
// Router backward, one wave per token: dJ/dw_{t,j} = <dh'_a, h_a> summed over the down
// projection's column tiles (+ <dy_t, b2_e> with GELU biases), then dz_t through the
// routers table's weights, plus the Switch loss term aux_coef (E/N) p (f - <p, f>) and the
// z-loss term z_coef (2 lse / N) p. Writes dz (float32), its split dz = hi + lo into two
// bfloat16 halves [t][0, E8) and [t][E8, 2 E8) (zero-padded) for the MFMA products with
// the router weights and x, and dgate.
// ---------------------------------------------------------------------------------------
constexpr int kRQ = kMaxExperts / kWave;

struct RouterBwd {
  const float* z;
  const int32_t* ids;
  const int32_t* inv_perm;
  const float* part;
  int n_part;
  const int32_t* counts;
  const uint16_t* dy;
  const uint16_t* b2;
  int n_tokens, E, k, d, router, norm_topk, E8;
  float sc, aux_coef, z_coef;
  float* dz;
  float* dgate;
  uint16_t* dz_hl;
};

__global__ __launch_bounds__(256) void router_backward_kernel(RouterBwd a) {
  __shared__ float s_dz[4][kMaxExperts];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.n_tokens) return;  // whole waves; no workgroup barrier below
  float* sd = s_dz[wave];
  const int E = a.E, k = a.k;
  const float* zt = a.z + (size_t)t * E;

  float zv[kRQ], ex[kRQ];
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < kRQ; ++q) {
    const int e = lane + kWave * q;
    zv[q] = e < E ? zt[e] : -INFINITY;
    m = fmaxf(m, zv[q]);
  }
  m = wave_max(m);
  float ssum = 0.f;
#pragma unroll
  for (int q = 0; q < kRQ; ++q) {
    ex[q] = (lane + kWave * q < E) ? expf(zv[q] - m) : 0.f;
    ssum += ex[q];
  }
  ssum = wave_sum(ssum);
  const float inv = 1.f / ssum;
  const float lse = m + logf(ssum);
  const float invN = 1.f / (float)a.n_tokens;

  float spf = 0.f;
  if (a.aux_coef != 0.f) {
#pragma unroll
    for (int q = 0; q < kRQ; ++q) {
      const int e = lane + kWave * q;
      if (e < E) spf += ex[q] * inv * ((float)a.counts[e] * invN);
    }
    spf = wave_sum(spf);
  }

  // the chosen experts: lane j < k holds choice j
  int id = 0;
  float dw = 0.f, zj = -INFINITY;
  if (lane < k) {
    id = a.ids[(size_t)t * k + lane];
    const int pos = a.inv_perm[(size_t)t * k + lane];
    const float* pp = a.part + (size_t)pos * a.n_part;
    for (int p = 0; p < a.n_part; ++p) dw += pp[p];
    zj = zt[id];
  }
  if (a.b2) {
    const uint16_t* dyt = a.dy + (size_t)t * a.d;
    for (int j = 0; j < k; ++j) {
      const int idj = __shfl(id, j, kWave);
      const uint16_t* bj = a.b2 + (size_t)idj * a.d;
      float acc = 0.f;
      for (int c = lane; c < a.d; c += kWave) acc += bf16_to_f32(dyt[c]) * bf16_to_f32(bj[c]);
      acc = wave_sum(acc);
      if (lane == j) dw += acc;
    }
  }

  // gate term of the chosen experts (contrib, added at id) and of every expert (base)
  float contrib = 0.f, cfull = 0.f;
  const bool chosen = lane < k;
  if (a.router == MOE_ROUTER_TOPK_SOFTMAX || (a.router == MOE_ROUTER_SOFTMAX_TOPK && a.norm_topk)) {
    const float zm = wave_max(chosen ? zj : -INFINITY);
    const float ej = chosen ? expf(zj - zm) : 0.f;
    const float wt = ej / wave_sum(ej);
    const float c = wave_sum(wt * dw);
    contrib = a.sc * wt * (dw - c);
  } else if (a.router == MOE_ROUTER_SOFTMAX_TOPK) {
    const float pj = chosen ? expf(zj - m) * inv : 0.f;
    cfull = wave_sum(pj * a.sc * dw);  // dz_e = p_e (gp_e - <p, gp>), gp = sc dw on the chosen
    contrib = pj * a.sc * dw;
  } else {
    const float sg = chosen ? sigmoid_f(zj) : 0.f;
    float dsg;
    if (a.norm_topk) {
      const float S = wave_sum(sg);
      const float c = wave_sum((sg / S) * dw);
      dsg = a.sc / S * (dw - c);
    } else {
      dsg = a.sc * dw;
    }
    contrib = dsg * sg * (1.f - sg);
  }

#pragma unroll
  for (int q = 0; q < kRQ; ++q) {
    const int e = lane + kWave * q;
    if (e < E) {
      const float p = ex[q] * inv;
      float v = -p * cfull;
      if (a.aux_coef != 0.f) v += a.aux_coef * ((float)E * invN) * p * ((float)a.counts[e] * invN - spf);
      if (a.z_coef != 0.f) v += a.z_coef * (2.f * lse * invN) * p;
      sd[e] = v;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  if (chosen) sd[id] += contrib;  // the k ids of a token are distinct
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int q = 0; q < kRQ; ++q) {
    const int e = lane + kWave * q;
    if (e < a.E8) {
      const float v = e < E ? sd[e] : 0.f;
      if (e < E) a.dz[(size_t)t * E + e] = v;
      const uint16_t hi = f32_to_bf16(v);
      a.dz_hl[(size_t)t * 2 * a.E8 + e] = hi;
      a.dz_hl[(size_t)t * 2 * a.E8 + a.E8 + e] = f32_to_bf16(v - bf16_to_f32(hi));
    }
  }
  if (chosen && a.dgate) a.dgate[(size_t)t * k + lane] = dw;
}

// Clears n 16-byte words (grid-stride; used instead of a memset so the sequence can be captured).
__global__ __launch_bounds__(256) void zero_kernel(uint4* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = make_uint4(0, 0, 0, 0);
}

// out[e][c] = sum over rows r of expert e (offsets, or rows [0, n_rows)) of scale[r] * M[r][c]
// (scale null: 1), rounded to bfloat16 once. A workgroup owns 64 columns of one expert: its
// 32 row phases each sum every 32nd row (8 columns per thread, 16-byte loads), then the 32
// partials of a column are added in phase order.
__global__ __launch_bounds__(256) void colsum_kernel(const uint16_t* __restrict__ Mx, long long ld,
                                                     const float* __restrict__ scale, const int* __restrict__ offsets,
                                                     int n_rows, int C, uint16_t* __restrict__ out) {
  __shared__ float s_part[32][65];
  const int t = threadIdx.x, e = blockIdx.y;
  const int cg = t & 7, ph = t >> 3;
  const int c0 = blockIdx.x * 64 + 8 * cg;
  const int lo = offsets ? offsets[e] : 0, hi = offsets ? offsets[e + 1] : n_rows;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c0 < C) {
    for (int r = lo + ph; r < hi; r += 32) {
      float v[8];
      unpack8(*reinterpret_cast<const uint4*>(Mx + (size_t)r * ld + c0), v);
      const float sc = scale ? scale[r] : 1.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += sc * v[q];
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) s_part[ph][8 * cg + q] = acc[q];
  __syncthreads();
  if (t < 64 && blockIdx.x * 64 + t < C) {
    float sum = 0.f;
    for (int p = 0; p < 32; ++p) sum += s_part[p][t];
    out[(size_t)e * C + blockIdx.x * 64 + t] = f32_to_bf16(sum);
  }
}

// Split-K weight gradients: out = bfloat16(sum over the ksplit partials, in split order), rows
// m < m_split of expert e to c, the others to c_hi (as the wgrad epilogue stores them).
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const float* __restrict__ kpart, int ksplit, int n_experts,
                                                           int M, int N, uint16_t* c, uint16_t* c_hi, int m_split,
                                                           long long ldc, long long c_estride) {
  const long long per_e = (long long)M * (N / 8);
  const long long total = per_e * n_experts;
  const size_t plane = (size_t)n_experts * M * N;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const int e = (int)(i / per_e);
    const long long r = i - e * per_e;
    const int m = (int)(r / (N / 8)), n = (int)(r - (long long)m * (N / 8)) * 8;
    const float* src = kpart + ((size_t)e * M + m) * N + n;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < ksplit; ++sp) {
      const float4 p0 = *reinterpret_cast<const float4*>(src + sp * plane);
      const float4 p1 = *reinterpret_cast<const float4*>(src + sp * plane + 4);
      acc[0] += p0.x; acc[1] += p0.y; acc[2] += p0.z; acc[3] += p0.w;
      acc[4] += p1.x; acc[5] += p1.y; acc[6] += p1.z; acc[7] += p1.w;
    }
    uint16_t* dst = (m < m_split) ? c + (size_t)e * c_estride + (size_t)m * ldc + n
                                  : c_hi + (size_t)e * c_estride + (size_t)(m - m_split) * ldc + n;
    *reinterpret_cast<uint4*>(dst) = pack8(acc);
  }
}

// dx[t] = sum_j dx_sorted[inv_perm[t k + j]] (j ascending) + R[t] (float32), rounded once;
// one wave per token, 8 columns per lane and step.
__global__ __launch_bounds__(256) void bwd_combine_kernel(const uint16_t* __restrict__ dxs, const int32_t* __restrict__ inv_perm,
                                                          const float* __restrict__ R, long long n_tokens, int k, int d,
                                                          uint16_t* __restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n_tokens) return;
  for (int c = 8 * lane; c < d; c += 8 * kWave) {
    float acc[8], v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int row = inv_perm[t * k + j];
      unpack8(*reinterpret_cast<const uint4*>(dxs + (size_t)row * d + c), v);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += v[q];
    }
    const float* rr = R + (size_t)t * d + c;
    const float4 p0 = *reinterpret_cast<const float4*>(rr);
    const float4 p1 = *reinterpret_cast<const float4*>(rr + 4);
    acc[0] += p0.x; acc[1] += p0.y; acc[2] += p0.z; acc[3] += p0.w;
    acc[4] += p1.x; acc[5] += p1.y; acc[6] += p1.z; acc[7] += p1.w;
    *reinterpret_cast<uint4*>(dx + (size_t)t * d + c) = pack8(acc);
  }
}

// ---------------------------------------------------------------------------------------
// Workspace of the backward (after the forward's route / ffn / forward regions).
// ---------------------------------------------------------------------------------------
struct BwdBufs {
  uint16_t* zero;   // 256 zero bytes (cleared by every call)
  int* tiles_dense; // m-tile table of one dense "expert" over the N token rows (shared, router)
  float* z;         // [N][E] logits
  float* dz;        // [N][E] (used when the caller passes none)
  float* part;      // [A][n_part]
  uint16_t* dz_hl;  // [N][2 E8]
  uint16_t* pre;    // [A][2 F] or [A][F]
  uint16_t* dpre;
  uint16_t* dxs;    // [A][d]
  float* R;         // [N][d] dz W_g (+ shared dx)
  uint16_t* pre_s;  // shared expert: [N][2 Fs] or [N][Fs]
  uint16_t* dpre_s;
  uint16_t* h_s;    // [N][Fs]
  float* kpart;     // split-K partials of the weight gradients that split
  float* tpart;     // split tail of dx_sorted: [kMaxTailItems][256][256]
  long long* sched; // weight-gradient schedule: cost prefix [E+1]
  int* sched_cnt;   // and its 8 per-XCD counters
  size_t bytes;
};

int n_part_of(int F) { return 2 * ((F + kBN - 1) / kBN); }

// K splits of a weight gradient: enough workgroups for the chip (about 1024) when the
// output has few tiles, with at least about 512 rows per split, at most 16 splits.
int wgrad_split(int M, int N, int n_experts, long long rows_total) {
  const long long tiles = (long long)n_experts * ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  if (tiles <= 0 || tiles >= 1024) return 1;
  const long long want = (1024 + tiles - 1) / tiles;
  const long long by_rows = std::max<long long>(1, rows_total / std::max(n_experts, 1) / 512);
  return (int)std::min<long long>(std::min(want, by_rows), 16);
}
size_t wgrad_part_floats(int M, int N, int n_experts, long long rows_total) {
  const int k = wgrad_split(M, N, n_experts, rows_total);
  return k > 1 ? (size_t)k * n_experts * M * N : 0;
}
int e8_of(int E) { return (E + 7) & ~7; }

BwdBufs bwd_bufs(const moe_config& c, char* base) {
  WsCarver w(base);
  const size_t N = (size_t)c.n_tokens, A = N * (size_t)c.top_k, E = (size_t)c.n_experts;
  const size_t d = (size_t)c.d_model, F = (size_t)c.d_ff, Fs = (size_t)std::max(c.d_ff_shared, 0);
  const size_t pf = c.act == MOE_ACT_SWIGLU ? 2 : 1;
  BwdBufs b{};
  b.zero = w.take_t<uint16_t>(128);
  b.tiles_dense = w.take_t<int>((size_t)tile_table_ints((N + kBM - 1) / kBM));
  b.z = w.take_t<float>(N * E);
  b.dz = w.take_t<float>(N * E);
  b.part = w.take_t<float>(A * (size_t)n_part_of((int)F));
  b.dz_hl = w.take_t<uint16_t>(N * 2 * (size_t)e8_of((int)E));
  b.pre = w.take_t<uint16_t>(A * pf * F);
  b.dpre = w.take_t<uint16_t>(A * pf * F);
  b.dxs = w.take_t<uint16_t>(A * d);
  b.R = w.take_t<float>(N * d);
  b.pre_s = w.take_t<uint16_t>(N * pf * Fs);
  b.dpre_s = w.take_t<uint16_t>(N * pf * Fs);
  b.h_s = w.take_t<uint16_t>(N * Fs);
  const int m = c.act == MOE_ACT_SWIGLU ? 2 : 1;
  size_t kp = 0;
  kp = std::max(kp, wgrad_part_floats((int)d, (int)F, (int)E, (long long)A));
  kp = std::max(kp, wgrad_part_floats(m * (int)F, (int)d, (int)E, (long long)A));
  if (Fs) {
    kp = std::max(kp, wgrad_part_floats((int)d, (int)Fs, 1, (long long)N));
    kp = std::max(kp, wgrad_part_floats(m * (int)Fs, (int)d, 1, (long long)N));
  }
  kp = std::max(kp, wgrad_part_floats((int)E, (int)d, 1, (long long)N));
  b.kpart = w.take_t<float>(kp);
  b.tpart = w.take_t<float>((size_t)kMaxTailItems * kBM * kBN);
  b.sched = w.take_t<long long>(E + 1);
  b.sched_cnt = w.take_t<int>(8);
  b.bytes = w.used();
  return b;
}

template <int MODE, int EPI>
hipError_t run_gemm(const BwdGemm& g, long long max_tiles, hipStream_t stream) {
  if (max_tiles <= 0) return hipGetLastError();
  const long long grid = (max_tiles + 7) / 8 * 8;
  if (grid > (1ll << 31) - 1) return hipErrorInvalidValue;
  bwd_gemm_kernel<MODE, EPI><<<(unsigned)grid, kThreads, 0, stream>>>(g);
  return hipGetLastError();
}

BwdGemm gemm_args(const uint16_t* zero) {
  BwdGemm g{};
  g.zero = zero;
  g.ksplit = 1;
  g.ldc = 0;
  g.m_split = 1 << 30;
  return g;
}

// dh' = dy_rows W2 (rows of a tile table) with the activation-backward epilogue.
hipError_t act_backward(const moe_config& c, const uint16_t* zero, const int* tiles, long long max_m_tiles, const uint16_t* dy_rows,
                        const void* w2, long long w2_estride, int F, const uint16_t* pre, const float* gate,
                        float* part, uint16_t* dpre, hipStream_t stream) {
  BwdGemm g = gemm_args(zero);
  g.a[0] = dy_rows;
  g.lda = c.d_model;
  g.klen[0] = c.d_model;
  g.b[0] = static_cast<const uint16_t*>(w2);
  g.ldb = F;
  g.b_estride = w2_estride;
  g.N = F;
  g.tiles = tiles;
  g.n_tiles_n = (F + kBN - 1) / kBN;
  g.pre = pre;
  g.gate = gate;
  g.part = part;
  g.n_part = n_part_of(F);
  g.c = dpre;
  const bool swi = c.act == MOE_ACT_SWIGLU;
  g.ldc = swi ? 2 * (long long)F : F;
  const long long S = max_m_tiles * g.n_tiles_n;
  return swi ? run_gemm<kGrouped, kSwigluBwd>(g, S, stream) : run_gemm<kGrouped, kGeluBwd>(g, S, stream);
}

// rows of dpre times [W1; W3] (or W1) -> out (T, or float32 with optional add)
template <int EPI>
hipError_t dx_rows(const moe_config& c, const uint16_t* zero, const int* tiles, long long max_m_tiles, const uint16_t* dpre, int F,
                   const void* w1, const void* w3, long long w_estride, void* out, const float* c_in,
                   float* tpart, hipStream_t stream) {
  BwdGemm g = gemm_args(zero);
  const bool swi = c.act == MOE_ACT_SWIGLU;
  g.a[0] = dpre;
  g.a[1] = swi ? dpre + F : nullptr;
  g.lda = swi ? 2 * (long long)F : F;
  g.klen[0] = F;
  g.klen[1] = swi ? F : 0;
  g.b[0] = static_cast<const uint16_t*>(w1);
  g.b[1] = swi ? static_cast<const uint16_t*>(w3) : nullptr;
  g.ldb = c.d_model;
  g.b_estride = w_estride;
  g.N = c.d_model;
  g.tiles = tiles;
  g.n_tiles_n = (c.d_model + kBN - 1) / kBN;
  g.c = out;
  g.ldc = c.d_model;
  g.c_in = c_in;
  const long long S_max = max_m_tiles * g.n_tiles_n;
  if (EPI != kStoreT || !tpart) return run_gemm<kGrouped, EPI>(g, S_max, stream);
  // whole rounds, then the last round's tiles in K pieces, then their fixed-order sum
  g.tpart = tpart;
  g.cu_grid = persistent_grid();
  g.grid_static = (int)((S_max + 7) / 8 * 8);
  bwd_gemm_kernel<kGrouped, EPI><<<(unsigned)(g.grid_static + kMaxTailItems), kThreads, 0, stream>>>(g);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  bwd_tail_reduce_kernel<<<kBwdTailReduceGrid, 256, 0, stream>>>(g);
  return hipGetLastError();
}

// C_e[M][N] = sum over the expert's rows r of A[r][m] B[r][n] (+ a second segment)
hipError_t wgrad(const BwdBufs& B, long long rows_total, const uint16_t* a0, const uint16_t* a1,
                 long long lda, const uint16_t* b0, const uint16_t* b1, long long ldb, int M, int N, const int* offsets,
                 int n_experts, int n_rows, void* c, void* c_hi, int m_split, long long ldc, long long c_estride,
                 hipStream_t stream) {
  float* kpart = B.kpart;
  BwdGemm g = gemm_args(B.zero);
  g.ksplit = wgrad_split(M, N, n_experts, rows_total);
  g.kpart = g.ksplit > 1 ? kpart : nullptr;
  g.a[0] = a0;
  g.a[1] = a1;
  g.b[0] = b0;
  g.b[1] = b1;
  g.lda = lda;
  g.ldb = ldb;
  g.M = M;
  g.N = N;
  g.offsets = offsets;
  g.n_experts = n_experts;
  g.klen[0] = n_rows;
  g.n_tiles_n = (N + kBN - 1) / kBN;
  g.c = c;
  g.c_hi = c_hi;
  g.m_split = m_split;
  g.ldc = ldc;
  g.c_estride = c_estride;
  const long long tpe = (long long)((M + kBM - 1) / kBM) * g.n_tiles_n;
  const long long S = n_experts * tpe * g.ksplit;
  hipError_t err;
  if (offsets && n_experts > 1 && g.ksplit == 1) {
    // routed experts of uneven sizes: the balanced persistent schedule
    wgrad_sched_kernel<<<1, 1024, 0, stream>>>(offsets, n_experts, tpe, B.sched, B.sched_cnt);
    g.sched = B.sched;
    g.sched_cnt = B.sched_cnt;
    bwd_gemm_kernel<kWgrad, kStoreT><<<persistent_grid(), kThreads, 0, stream>>>(g);
    err = hipGetLastError();
  } else {
    err = run_gemm<kWgrad, kStoreT>(g, S, stream);
  }
  if (err != hipSuccess || g.ksplit == 1) return err;
  const long long total = (long long)n_experts * M * (N / 8);
  wgrad_reduce_kernel<<<(unsigned)std::min<long long>((total + 255) / 256, 8192), 256, 0, stream>>>(
      kpart, g.ksplit, n_experts, M, N, static_cast<uint16_t*>(c), static_cast<uint16_t*>(c_hi), m_split, ldc, c_estride);
  return hipGetLastError();
}

hipError_t colsum(const uint16_t* Mx, long long ld, const float* scale, const int* offsets, int n_groups, int n_rows,
                  int C, void* out, hipStream_t stream) {
  dim3 grid((C + 63) / 64, n_groups);
  colsum_kernel<<<grid, 256, 0, stream>>>(Mx, ld, scale, offsets, n_rows, C, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

#define BWD_TRY(expr)                   \
  do {                                  \
    const hipError_t e_ = (expr);       \
    if (e_ != hipSuccess) return e_;    \
  } while (0)

}  // namespace

void carve_backward(const moe_config& c, WsCarver& w, WsLayout* L) {
  const size_t bytes = bwd_bufs(c, nullptr).bytes;
  void* p = w.take(bytes);
  if (L) L->bwd = p;
}

hipError_t launch_backward(const moe_config& c, const WsLayout& L, const BwdIn& in, const moe_grads& gr,
                           const RouteOut& ro, bool saved, void* const* events, hipStream_t s) {
  const BwdBufs B = bwd_bufs(c, static_cast<char*>(L.bwd));
  int next_event = 0;
  auto mark = [&](int upto) -> hipError_t {  // record every event up to index `upto`
    for (; events && next_event <= upto; ++next_event) {
      const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[next_event]), s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  };
  BWD_TRY(mark(0));
  zero_kernel<<<1, 256, 0, s>>>(reinterpret_cast<uint4*>(B.zero), 16);
  BWD_TRY(hipGetLastError());
  const int N = (int)c.n_tokens, E = c.n_experts, k = c.top_k, d = c.d_model, F = c.d_ff;
  const int A = N * k, Fs = c.d_ff_shared, E8 = e8_of(E);
  const bool swi = c.act == MOE_ACT_SWIGLU, bias = c.has_bias != 0;
  auto T = [](const void* p) { return static_cast<const uint16_t*>(p); };
  int32_t* ids = ro.topk_ids;
  float* dz = gr.dz ? gr.dz : B.dz;

  // recompute (unless a moe_forward_train left them in the workspace): routing with its
  // logits, the dispatch of x, the up projection's pre-activations and gate-scaled h
  if (!saved)
    BWD_TRY(launch_route(c, L, in.x, in.w_router, in.logit_bias, in.sel_bias, ids, ro.topk_w, ro.counts, ro.stats,
                         B.z, nullptr, true, s));
  if (N == 0) {
    // no token: every gradient is zero
    auto zero = [&](void* p, size_t bytes) {
      if (!p) return hipSuccess;
      zero_kernel<<<(unsigned)std::min<size_t>((bytes / 16 + 255) / 256, 4096), 256, 0, s>>>(static_cast<uint4*>(p), bytes / 16);
      return hipGetLastError();
    };
    const size_t t2 = 2;
    BWD_TRY(zero(gr.dw_router, (size_t)E * d * t2));
    BWD_TRY(zero(gr.dw1, (size_t)E * F * d * t2));
    BWD_TRY(zero(gr.dw3, (size_t)E * F * d * t2));
    BWD_TRY(zero(gr.db1, (size_t)E * F * t2));
    BWD_TRY(zero(gr.dw2, (size_t)E * d * F * t2));
    BWD_TRY(zero(gr.db2, (size_t)E * d * t2));
    BWD_TRY(zero(gr.ds_w1, (size_t)Fs * d * t2));
    BWD_TRY(zero(gr.ds_w3, (size_t)Fs * d * t2));
    BWD_TRY(zero(gr.ds_b1, (size_t)Fs * t2));
    BWD_TRY(zero(gr.ds_w2, (size_t)d * Fs * t2));
    BWD_TRY(zero(gr.ds_b2, (size_t)d * t2));
    BWD_TRY(hipGetLastError());
    return mark(MOE_BWD_EVENTS - 1);
  }
  if (!saved)
    BWD_TRY(launch_dispatch_scanned(c, L, in.x, ids, ro.topk_w, L.x_sorted, L.perm, L.inv_perm, L.gate_sorted, s));
  uint16_t* xs = static_cast<uint16_t*>(L.x_sorted);
  uint16_t* dys = static_cast<uint16_t*>(L.y_sorted);
  uint16_t* hw = static_cast<uint16_t*>(L.h);
  launch_copy(c, in.dy, L.inv_perm, dys, s);
  // the routed m-tile table is the forward's (routing's final reduction wrote it)
  if (ffn_tile_rows(c) != kBM) return hipErrorInvalidValue;
  const long long mtA = ffn_max_m_tiles(c);
  BWD_TRY(mark(1));
  if (!saved) BWD_TRY(launch_up_save(c, L.tiles, xs, in.w1, in.w3, in.b1, L.gate_sorted, F, B.pre, hw, s));
  BWD_TRY(mark(2));

  // routed experts: dh' with the activation backward, then dx_sorted and the weight gradients
  BWD_TRY(act_backward(c, B.zero, L.tiles, mtA, dys, in.w2, (long long)d * F, F, B.pre, L.gate_sorted, B.part, B.dpre, s));
  BWD_TRY(mark(3));
  {
    RouterBwd r{};
    r.z = B.z;
    r.ids = ids;
    r.inv_perm = L.inv_perm;
    r.part = B.part;
    r.n_part = n_part_of(F);
    r.counts = ro.counts;
    r.dy = T(in.dy);
    r.b2 = bias ? T(in.b2) : nullptr;
    r.n_tokens = N;
    r.E = E;
    r.k = k;
    r.d = d;
    r.router = c.router;
    r.norm_topk = c.norm_topk;
    r.E8 = E8;
    r.sc = c.routed_scaling;
    r.aux_coef = in.aux_coef;
    r.z_coef = in.z_coef;
    r.dz = dz;
    r.dgate = gr.dgate;
    r.dz_hl = B.dz_hl;
    router_backward_kernel<<<(N + 3) / 4, 256, 0, s>>>(r);
    BWD_TRY(hipGetLastError());
  }
  BWD_TRY(mark(4));
  BWD_TRY(dx_rows<kStoreT>(c, B.zero, L.tiles, mtA, B.dpre, F, in.w1, in.w3, (long long)F * d, B.dxs, nullptr, B.tpart, s));
  BWD_TRY(mark(5));
  BWD_TRY(wgrad(B, A, dys, nullptr, d, hw, nullptr, F, d, F, L.offsets, E, 0, gr.dw2, nullptr, d, F,
                (long long)d * F, s));
  BWD_TRY(mark(6));
  BWD_TRY(wgrad(B, A, B.dpre, nullptr, swi ? 2 * (long long)F : F, xs, nullptr, d, swi ? 2 * F : F, d, L.offsets, E, 0,
                gr.dw1, gr.dw3, F, d, (long long)F * d, s));
  if (bias) {
    BWD_TRY(colsum(B.dpre, F, nullptr, L.offsets, E, 0, F, gr.db1, s));
    BWD_TRY(colsum(dys, d, L.gate_sorted, L.offsets, E, 0, d, gr.db2, s));
  }
  BWD_TRY(mark(7));

  // shared expert over all N rows (gate 1); its dx lands in R
  BWD_TRY(launch_dense_tiles(N, kBM, B.tiles_dense, s));
  const long long mtN = (N + kBM - 1) / kBM;
  if (Fs > 0) {
    if (!saved) BWD_TRY(launch_up_save(c, B.tiles_dense, in.x, in.s_w1, in.s_w3, in.s_b1, nullptr, Fs, B.pre_s, B.h_s, s));
    BWD_TRY(act_backward(c, B.zero, B.tiles_dense, mtN, T(in.dy), in.s_w2, 0, Fs, B.pre_s, nullptr, nullptr, B.dpre_s, s));
    BWD_TRY(dx_rows<kStoreF32>(c, B.zero, B.tiles_dense, mtN, B.dpre_s, Fs, in.s_w1, in.s_w3, 0, B.R, nullptr, nullptr, s));
    BWD_TRY(wgrad(B, N, T(in.dy), nullptr, d, B.h_s, nullptr, Fs, d, Fs, nullptr, 1, N, gr.ds_w2, nullptr,
                  d, Fs, 0, s));
    BWD_TRY(wgrad(B, N, B.dpre_s, nullptr, swi ? 2 * (long long)Fs : Fs, T(in.x), nullptr, d, swi ? 2 * Fs : Fs, d,
                  nullptr, 1, N, gr.ds_w1, gr.ds_w3, Fs, d, 0, s));
    if (bias) {
      BWD_TRY(colsum(B.dpre_s, Fs, nullptr, nullptr, 1, N, Fs, gr.ds_b1, s));
      BWD_TRY(colsum(T(in.dy), d, nullptr, nullptr, 1, N, d, gr.ds_b2, s));
    }
  }
  BWD_TRY(mark(8));

  // router: dW_g = dz^T x and R (+)= dz W_g, both with dz = hi + lo in bfloat16
  BWD_TRY(wgrad(B, N, B.dz_hl, B.dz_hl + E8, 2 * (long long)E8, T(in.x), T(in.x), d, E, d, nullptr, 1, N, gr.dw_router,
                nullptr, E, d, 0, s));
  {
    BwdGemm g = gemm_args(B.zero);
    g.a[0] = B.dz_hl;
    g.a[1] = B.dz_hl + E8;
    g.lda = 2 * (long long)E8;
    g.klen[0] = E;
    g.klen[1] = E;
    g.b[0] = T(in.w_router);
    g.b[1] = T(in.w_router);
    g.ldb = d;
    g.N = d;
    g.tiles = B.tiles_dense;
    g.n_tiles_n = (d + kBN - 1) / kBN;
    g.c = B.R;
    g.ldc = d;
    g.c_in = Fs > 0 ? B.R : nullptr;
    BWD_TRY((run_gemm<kGrouped, kStoreF32>(g, mtN * g.n_tiles_n, s)));
  }
  bwd_combine_kernel<<<(N + 3) / 4, 256, 0, s>>>(B.dxs, L.inv_perm, B.R, N, k, d, static_cast<uint16_t*>(gr.dx));
  BWD_TRY(hipGetLastError());
  return mark(MOE_BWD_EVENTS - 1);
}

hipError_t launch_forward_train(const moe_config& c, const WsLayout& L, const BwdIn& in, void* y, const RouteOut& ro,
                                hipStream_t s) {
  const BwdBufs B = bwd_bufs(c, static_cast<char*>(L.bwd));
  const int N = (int)c.n_tokens, A = N * c.top_k, F = c.d_ff, Fs = c.d_ff_shared;
  BWD_TRY(launch_route(c, L, in.x, in.w_router, in.logit_bias, in.sel_bias, ro.topk_ids, ro.topk_w, ro.counts, ro.stats,
                       B.z, nullptr, true, s));
  if (N == 0) return hipGetLastError();
  if (ffn_tile_rows(c) != kBM) return hipErrorInvalidValue;
  BWD_TRY(launch_dispatch_scanned(c, L, in.x, ro.topk_ids, ro.topk_w, L.x_sorted, L.perm, L.inv_perm, L.gate_sorted,
                                  s));
  // up projection keeping the pre-activations; the down projection then reads w_a h_a
  BWD_TRY(launch_up_save(c, L.tiles, L.x_sorted, in.w1, in.w3, in.b1, L.gate_sorted, F, B.pre, L.h, s));
  BWD_TRY(launch_down(c, L.tiles, ffn_max_m_tiles(c), L.h, F, in.w2, in.b2, L.gate_sorted, true, L.y_sorted,
                      L.tail_part, s));
  // the shared expert the same way, its output in dx_sorted's buffer (A >= N rows; free until
  // the backward)
  const bool shared = Fs > 0;
  if (shared) {
    BWD_TRY(launch_dense_tiles(N, kBM, B.tiles_dense, s));
    BWD_TRY(launch_up_save(c, B.tiles_dense, in.x, in.s_w1, in.s_w3, in.s_b1, nullptr, Fs, B.pre_s, B.h_s, s));
    BWD_TRY(launch_down(c, B.tiles_dense, (N + kBM - 1) / kBM, B.h_s, Fs, in.s_w2, in.s_b2, nullptr, false, B.dxs,
                        nullptr, s));
  }
  (void)A;
  return launch_combine(c, L.y_sorted, nullptr, L.inv_perm, shared ? B.dxs : nullptr, y, s);
}

}  // namespace moe
