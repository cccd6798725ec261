// Work schedule and operand addresses of the bf16 grouped GEMMs: which (m-tile, n-tile,
// K piece) items a launch runs, in what order, and where a lane's 16-byte LDS-DMA copy reads
// its operand. Pure integer functions, compiled for the device (the kernels) and for the host
// (tests/sched_check.cpp checks them exhaustively with g++, no GPU), so the two cannot
// drift apart.
//
// Ragged per-expert slices follow "Mixture of Experts: routing, sorted dispatch, Switch aux
// loss, aux-free bias" (L7.8) §2.2: every expert's rows form one contiguous slice of the
// sorted order, and each expert runs once over its own slice.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define MOE_HD __host__ __device__ __forceinline__
#else
#define MOE_HD inline
#endif

namespace moe {

template <typename U> MOE_HD U smin(U a, U b) { return a < b ? a : b; }
template <typename U> MOE_HD U smax(U a, U b) { return a > b ? a : b; }

// ---- the m-tile table

// Header: tiles[0] = m-tiles, tiles[1] = full m-tiles, tiles[2] / tiles[3] = offsets (in ints,
// from tiles) of fmap / nmap, tiles[4..7] = 16 zero bytes. m-tile t (experts in order, each
// expert's rows in order) is tiles[kTileHdr + kTileInts t ..] = (expert, first row, rows in the
// tile, the expert's first m-tile, the expert's m-tile count, the expert's first full m-tile in
// fmap, the expert's full m-tiles). An expert's last m-tile is narrow when it has at most
// `narrow` rows; fmap[i] is the table index of the i-th full m-tile and nmap[j] that of the
// j-th narrow one.
constexpr int kTileHdr = 8, kTileInts = 8;
// ints of a tile table for at most cap m-tiles
constexpr long long tile_table_ints(long long cap) { return kTileHdr + (kTileInts + 2) * cap; }

// Tile shapes: full 256 rows x 256 B-rows, narrow 128 x 512; reduction slabs of 32.
constexpr int kSchedBM = 256, kSchedBK = 32;

// Narrow tiles pay where an expert's last m-tile is a large share of its work. The tile table
// lists them, and the up projection runs them, for experts of at most four full m-tiles on
// average (A / E <= 1024 rows): the rows at or below which a last m-tile is narrow (0: none).
MOE_HD int narrow_rows_for(long long assignments, int n_experts, bool bf16) {
  return (bf16 && assignments <= 1024LL * n_experts) ? kSchedBM / 2 : 0;
}
// The down projection's launches (which split their tail) run the narrow-capable kernel only
// at A / E <= 512 rows. Between 512 and 1024 the table still lists narrow tiles, and the
// launches, the tail's reducer included, must then all treat every m-tile as full.
MOE_HD bool down_narrow_for(long long assignments, int n_experts, bool bf16) {
  return narrow_rows_for(assignments, n_experts, bf16) > 0 && assignments <= 512LL * n_experts;
}

// K pieces of each tail tile: enough (tile, piece) pairs to fill the grid, at least 4 slabs
// per piece, at most kMaxTailItems pairs (the partial buffer's size).
constexpr int kMaxTailItems = 256;
MOE_HD int tail_pieces(long long s_tail, int nk_all, int grid) {
  if (s_tail <= 0) return 1;
  const long long q = smin((long long)grid / s_tail, (long long)kMaxTailItems / s_tail);
  return (int)smax(1ll, smin(q, (long long)(nk_all / 4)));
}

// Supertile order of a group of `me` m-tiles with NT n-tiles each: bands of kGM m-tiles, each
// walked in groups of kGN n-tiles with the m-tile fastest, so the tiles that run at the same
// time share A and B panels in L2. Local item l -> (m-tile within the group, n-tile).
constexpr int kGM = 8, kGN = 4;
MOE_HD void supertile(long long l, int me, int NT, int* mt, int* nt) {
  const int band = (int)(l / ((long long)kGM * NT));
  const int lb = (int)(l - (long long)band * kGM * NT);
  const int bm = smin(kGM, me - kGM * band);
  const int grpn = lb / (kGN * bm);
  const int r = lb - grpn * kGN * bm;
  *mt = kGM * band + r % bm;
  *nt = grpn * kGN + r / bm;
}

// Whether a launch runs narrow tiles, given that its kernel may (nar_ok). A narrow tile reads
// twice the B rows per item of a full one, and its expert's B on its own; a launch that splits
// its tail (the down projection, PART 1 / 2) runs all of its tail at once, so it uses them
// only when they are at least a quarter of the m-tiles (then most tiles stream their weights
// anyway and the halved MFMA work wins). Otherwise every m-tile runs with the full shape, in
// table order.
MOE_HD bool use_narrow(const int* tiles, bool nar_ok, bool split) {
  const int n_nar = tiles[0] - tiles[1];
  return nar_ok && n_nar > 0 && (!split || 4 * n_nar >= tiles[0]);
}

// Work items of a grouped GEMM with NT n-tiles per full m-tile: NT per m-tile, or with narrow
// tiles NT per full m-tile and ceil(NT / 2) per narrow one.
MOE_HD long long gemm_items(const int* tiles, int NT, bool nar) {
  return nar ? (long long)tiles[1] * NT + (long long)(tiles[0] - tiles[1]) * ((NT + 1) >> 1)
             : (long long)tiles[0] * NT;
}

// Narrow items a launch of `grid` persistent workgroups that splits the tail (PART 1 / 2)
// places last: as many as the tail (the last S mod grid items) holds, so that the whole
// rounds are made of full items where possible (every workgroup then runs the same work) and
// the narrow items' K pieces are balanced like any tail item's.
MOE_HD long long narrow_tail(const int* tiles, int NT, bool nar, int grid) {
  if (!nar) return 0;
  const long long S = gemm_items(tiles, NT, true);
  const long long S_nar = (long long)(tiles[0] - tiles[1]) * ((NT + 1) >> 1);
  return smin(S_nar, S - S / grid * grid);
}

// Work item u (0 <= u < gemm_items): its m-tile (expert, first row, rows) and n-tile; returns
// whether it is narrow. Without narrow tiles the items are expert-major, then in supertiles
// of the expert's m-tiles. With them, the full m-tiles (fmap) are ordered that way; the last
// n_tail items are narrow ones, and the other narrow items are spread evenly through the rest
// (item u is the narrow item floor(u Sn / S) when that count steps at u), so that every XCD's
// run and every round holds its share of them.
MOE_HD bool decode_tile(const int* tiles, long long u, int NT, bool use_nar, long long n_tail, int* e, int* row0,
                        int* rows, int* nt) {
  const int* T = tiles + kTileHdr;
  int t, m;
  bool nar = false;
  if (!use_nar) {
    const int* probe = T + kTileInts * (int)(u / NT);
    const int ts = probe[3];
    supertile(u - (long long)ts * NT, probe[4], NT, &m, nt);
    t = ts + m;
  } else {
    const int NT2 = (NT + 1) >> 1;
    const long long s_full = (long long)tiles[1] * NT;
    const long long S_nar = (long long)(tiles[0] - tiles[1]) * NT2 - n_tail;  // interleaved ones
    const long long S = s_full + S_nar;
    long long nb;  // narrow items before u
    if (u >= S) {
      nb = S_nar + (u - S);
      nar = true;
    } else {
      nb = u * S_nar / S;
      nar = (u + 1) * S_nar / S > nb;
    }
    if (nar) {
      const long long j = nb / NT2;
      t = tiles[tiles[3] + (int)j];
      *nt = (int)(nb - j * NT2);
    } else {
      const int* fmap = tiles + tiles[2];
      const long long s = u - nb;  // full item
      const int* probe = T + kTileInts * fmap[(int)(s / NT)];
      const int fs = probe[5];
      supertile(s - (long long)fs * NT, probe[6], NT, &m, nt);
      t = fmap[fs + m];
    }
  }
  const int* q = T + kTileInts * t;
  *e = q[0];
  *row0 = q[1];
  *rows = q[2];
  return nar;
}

// ---- one launch's items

// PART: 0 = every work item; 1 = only the whole rounds (the first floor(S / G) * G items of
// S = gemm_items, G = the grid); 2 = the remaining S mod G items, each cut along K into q
// pieces, one piece per workgroup. The GEMM launches and the tail's reducer all derive their
// items from this one plan, so they number the tail identically.
struct GemmPlan {
  bool nar;          // narrow tiles in this launch
  long long S_all;   // items of the table
  long long S_main;  // items run whole (the whole rounds for PART 1 / 2)
  int q;             // K pieces per tail item (PART 2), else 1
  long long n_tail;  // narrow items placed last (PART 1 / 2)
};
MOE_HD GemmPlan gemm_plan(const int* tiles, int NT, bool nar_ok, int part, int grid, int nk_all) {
  GemmPlan p;
  p.nar = use_narrow(tiles, nar_ok, part != 0);
  p.S_all = gemm_items(tiles, NT, p.nar);
  p.S_main = part == 0 ? p.S_all : p.S_all / grid * grid;
  p.q = part == 2 ? tail_pieces(p.S_all - p.S_main, nk_all, grid) : 1;
  p.n_tail = part == 0 ? 0 : narrow_tail(tiles, NT, p.nar, grid);
  return p;
}
// Workgroup b's run of item indices w: [begin, end) by step. PART 0 / 1: the items [0, S_main)
// are cut into 8 contiguous chunks, one per XCD (workgroup b runs on XCD b mod 8, as the
// hardware deals workgroups round-robin), and each XCD's workgroups take its chunk in turn.
// PART 2: w indexes the tail's (item, piece) pairs, one per workgroup.
struct GemmRange {
  long long begin, end;
  int step;
};
MOE_HD GemmRange gemm_range(const GemmPlan& p, int part, int b, int grid) {
  GemmRange r;
  if (part == 2) {
    r.begin = b;
    r.end = (p.S_all - p.S_main) * p.q;
    r.step = grid;
  } else {
    const int xcd = b & 7, slot = b >> 3;
    const long long chunk = (p.S_main + 7) / 8;
    r.begin = (long long)xcd * chunk + slot;
    r.end = smin(p.S_main, (long long)xcd * chunk + chunk);
    r.step = grid >> 3;
  }
  return r;
}
// Item index w of a launch: its position s in the work sequence (for decode_tile) and its K
// range, slabs [*kso, *kso + *nk) of nk_all; *piece is its K piece (0 unless PART 2).
MOE_HD long long plan_item(const GemmPlan& p, int part, long long w, int nk_all, int* kso, int* nk, int* piece) {
  if (part != 2) {
    *kso = 0;
    *nk = nk_all;
    *piece = 0;
    return w;
  }
  const int pc = (int)(w % p.q);
  *piece = pc;
  *kso = (int)((long long)pc * nk_all / p.q);
  *nk = (int)((long long)(pc + 1) * nk_all / p.q) - *kso;
  return p.S_main + w / p.q;
}

// ---- where a lane's 16-byte copy reads its operand
//
// A copy instruction fills 16 rows x 32 reduction elements of an LDS stage: lane l reads row
// (l >> 2) of them at the 8-element chunk lchunk = 8 ((l & 3) ^ ((l >> 4) & 3)) (the LDS
// swizzle). The offsets are split into a per-tile row part and a per-slab K part; both are
// unsigned 32-bit and are summed in 32 bits (src_off) before the sum meets the 64-bit base.

// Row-major operand [rows][K]: row rc's chunk lchunk, in bytes from the operand's tile base.
MOE_HD uint32_t rm_row_off(int rc, int K, int lchunk) { return (uint32_t)(rc * K + lchunk) * 2u; }
// K part for slab k0 (a multiple of 32). Where K is not a multiple of 32 the last slab runs
// past the row: a lane whose chunk lies past K re-reads the row's last chunk (elements K - 8
// .. K - 1, zeroed in LDS once landed), i.e. the K part moves the lane from lchunk to K - 8.
// The move is negative when lchunk > K - 8, which happens only for K < 32; as an unsigned
// 32-bit value it then wraps, and the 32-bit sum in src_off lands exactly on K - 8 of the
// same row.
MOE_HD uint32_t rm_k_off(int K, int k0, int lchunk) {
  return ((K % kSchedBK) != 0 && k0 + lchunk >= K) ? (uint32_t)(K - 8 - lchunk) * 2u : (uint32_t)k0 * 2u;
}
// Tiled operand (128-row blocks, each stored one 32-element slab after another; row pitch
// kp = K padded to 32): row `rel` (counted from the tile's first block) at lchunk.
constexpr int kTiledRows = 128, kTiledK = 32;
MOE_HD uint32_t tiled_row_off(int rel, int kp, int lchunk) {
  return (uint32_t)((rel & ~(kTiledRows - 1)) * kp + (rel & (kTiledRows - 1)) * kTiledK + lchunk) * 2u;
}
// K part of a tiled operand: slab k0 / 32 of the block; lanes past K read the zero padding.
MOE_HD uint32_t tiled_k_off(int k0) { return (uint32_t)k0 * (kTiledRows * 2u); }
// The lane's source, in bytes from the tile base: row part + K part in 32 bits.
MOE_HD uint32_t src_off(uint32_t row_off, uint32_t k_off) { return row_off + k_off; }

}  // namespace moe
