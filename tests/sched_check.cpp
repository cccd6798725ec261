// Host check of the grouped GEMM's schedule and operand addresses (gemm_sched.h, the same
// functions the kernels run), compiled with g++ by tests/test_sched_cpu.py. No GPU.
//
//  addr   every 16-byte LDS-DMA source stays inside its operand row (row-major) or its
//         128-row block (tiled), for every K in [8, 65536] step 8, every lane, the first
//         and last slabs; lanes inside K read exactly their own elements.
//  sched  for ragged per-expert row counts, every (m-tile, n-tile) of the table is computed
//         exactly once by a single launch and by the split launches (whole rounds, then the
//         tail in K pieces), and the tail's reducer sums exactly the pieces the split launch
//         wrote, for the same tiles.
//
// Prints "ok <checks>" and exits 0, or prints the first failure and exits 1.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "gemm_sched.h"

using namespace moe;

static long long n_checks = 0;
#define CHECK(cond, ...)                  \
  do {                                    \
    ++n_checks;                           \
    if (!(cond)) {                        \
      std::printf("FAIL: " __VA_ARGS__);  \
      std::printf("\n");                  \
      std::exit(1);                       \
    }                                     \
  } while (0)

// the chunk a copy lane reads: the 8-wave kernel's swizzle (map 0) and the 4-wave kernel's (map 1)
static int lane_chunk(int lane, int map = 0) {
  return ((lane & 3) ^ (map ? ((lane >> 3) & 3) : ((lane >> 4) & 3))) * 8;
}

static void check_addresses() {
  for (int K = 8; K <= 65536; K += 8) {
    const int nk = (K + kSchedBK - 1) / kSchedBK;
    const int kp = (K + kTiledK - 1) / kTiledK * kTiledK;
    const int slabs[4] = {0, 1, nk - 2, nk - 1};
    for (int si = 0; si < 4; ++si) {
      const int k = slabs[si];
      if (k < 0 || k >= nk) continue;
      const int k0 = k * kSchedBK;
      for (int lm = 0; lm < 128; ++lm) {
        const int lane = lm & 63, lc = lane_chunk(lane, lm >> 6);
        const bool inside = k0 + lc < K;
        // row-major [rows][K], rows 0, 1 and 255 of a tile
        const int rcs[3] = {0, 1, 255};
        for (int rc : rcs) {
          const unsigned long long off = src_off(rm_row_off(rc, K, lc), rm_k_off(K, k0, lc));
          const unsigned long long row = (unsigned long long)rc * K * 2;
          CHECK(off % 16 == 0, "row-major K=%d lane=%d slab=%d: unaligned offset %llu", K, lane, k, off);
          CHECK(off >= row && off + 16 <= row + 2ull * K,
                "row-major K=%d lane=%d slab=%d row=%d: offset %llu outside the row [%llu, %llu)", K, lane, k, rc, off,
                row, row + 2ull * K);
          if (inside)
            CHECK(off == row + 2ull * (k0 + lc), "row-major K=%d lane=%d slab=%d: reads %llu, not its chunk", K, lane,
                  k, off);
        }
        // tiled: 128-row blocks of 32-element slabs, row pitch kp
        const int rels[5] = {0, 1, 127, 128, 383};
        for (int rel : rels) {
          const unsigned long long off = src_off(tiled_row_off(rel, kp, lc), tiled_k_off(k0));
          const unsigned long long blk = (unsigned long long)(rel / kTiledRows) * kTiledRows * kp * 2;
          const unsigned long long want =
              blk + 2ull * ((unsigned long long)(k0 / kTiledK) * kTiledRows * kTiledK + (rel % kTiledRows) * kTiledK + lc);
          CHECK(off == want, "tiled K=%d lane=%d slab=%d rel=%d: offset %llu, layout says %llu", K, lane, k, rel, off,
                want);
          CHECK(off + 16 <= blk + 2ull * kTiledRows * kp, "tiled K=%d lane=%d slab=%d: past the block", K, lane, k);
        }
      }
    }
  }
}

// The tile table for per-expert row counts, built from its definition (gemm_sched.h).
static std::vector<int> make_table(const std::vector<int>& counts, int bm, int narrow) {
  int total = 0;
  for (int c : counts) total += (c + bm - 1) / bm;
  const int cap = total > 0 ? total : 1;
  std::vector<int> t((size_t)tile_table_ints(cap), 0);
  int* fmap = t.data() + kTileHdr + kTileInts * cap;
  int* nmap = fmap + cap;
  int m = 0, f = 0, nn = 0, row = 0;
  for (size_t e = 0; e < counts.size(); ++e) {
    const int c = counts[e], n = (c + bm - 1) / bm;
    const bool nar = n > 0 && c - (n - 1) * bm <= narrow;
    const int n_full = n - (nar ? 1 : 0);
    for (int i = 0; i < n; ++i) {
      int* q = t.data() + kTileHdr + kTileInts * (m + i);
      q[0] = (int)e;
      q[1] = row + i * bm;
      q[2] = smin(bm, c - i * bm);
      q[3] = m;
      q[4] = n;
      q[5] = f;
      q[6] = n_full;
      if (i < n_full) fmap[f + i] = m + i;
    }
    if (nar) nmap[nn++] = m + n - 1;
    m += n;
    f += n_full;
    row += c;
  }
  t[0] = m;
  t[1] = f;
  t[2] = kTileHdr + kTileInts * cap;
  t[3] = kTileHdr + (kTileInts + 1) * cap;
  return t;
}

struct Item {
  int e, row0, rows, nt;
  bool nar;
  bool operator==(const Item& o) const {
    return e == o.e && row0 == o.row0 && rows == o.rows && nt == o.nt && nar == o.nar;
  }
};

// m-tile index of (expert, first row) in the table
static int mtile_of(const std::vector<int>& t, int e, int row0) {
  for (int i = 0; i < t[0]; ++i) {
    const int* q = t.data() + kTileHdr + kTileInts * i;
    if (q[0] == e && q[1] == row0) return i;
  }
  return -1;
}

// Marks the (m-tile, full n-tile) cells an item covers, with `mult` per cell.
static void cover(const std::vector<int>& t, const Item& it, int NT, std::vector<int>& cells, int mult) {
  const int m = mtile_of(t, it.e, it.row0);
  CHECK(m >= 0, "item (e=%d row0=%d) is no m-tile of the table", it.e, it.row0);
  const int* q = t.data() + kTileHdr + kTileInts * m;
  CHECK(q[2] == it.rows, "item rows %d, table %d", it.rows, q[2]);
  if (it.nar) {
    CHECK(it.rows <= kSchedBM / 2, "narrow item with %d rows", it.rows);
    CHECK(m == q[3] + q[4] - 1, "narrow item is not its expert's last m-tile");
    for (int d = 0; d < 2; ++d)
      if (2 * it.nt + d < NT) cells[(size_t)m * NT + 2 * it.nt + d] += mult;
  } else {
    CHECK(it.nt >= 0 && it.nt < NT, "n-tile %d of %d", it.nt, NT);
    cells[(size_t)m * NT + it.nt] += mult;
  }
}

static Item decode(const std::vector<int>& t, const GemmPlan& p, long long s, int NT) {
  Item it;
  it.nar = decode_tile(t.data(), s, NT, p.nar, p.n_tail, &it.e, &it.row0, &it.rows, &it.nt);
  return it;
}

// One launch of a grid of persistent workgroups (the kernel's loop): every workgroup's items.
// Returns (item index w, K piece, slabs) -> tile.
struct Run {
  long long w;
  int kso, nk, piece;
  Item it;
};
static std::vector<Run> launch(const std::vector<int>& t, int NT, bool nar_ok, int part, int grid, int nk_all,
                               GemmPlan* plan_out) {
  const GemmPlan p = gemm_plan(t.data(), NT, nar_ok, part, grid, nk_all);
  if (plan_out) *plan_out = p;
  std::vector<Run> out;
  for (int b = 0; b < grid; ++b) {
    const GemmRange r = gemm_range(p, part, b, grid);
    for (long long w = r.begin; w < r.end; w += r.step) {
      Run x;
      x.w = w;
      const long long s = plan_item(p, part, w, nk_all, &x.kso, &x.nk, &x.piece);
      CHECK(s >= 0 && s < p.S_all, "item %lld outside [0, %lld)", s, p.S_all);
      x.it = decode(t, p, s, NT);
      out.push_back(x);
    }
  }
  return out;
}

static void check_schedule(const std::vector<int>& counts, int NT, int grid, int nk_all, bool single_nar_ok,
                           bool split_nar_ok) {
  const long long A = [&] { long long a = 0; for (int c : counts) a += c; return a; }();
  const int narrow = narrow_rows_for(A, (int)counts.size(), true);
  const std::vector<int> t = make_table(counts, kSchedBM, narrow);
  const size_t ncell = (size_t)t[0] * NT;
  // a single launch (PART 0): the up projection, or the down one without a split tail
  {
    std::vector<int> cells(ncell, 0);
    for (const Run& x : launch(t, NT, single_nar_ok, 0, grid, nk_all, nullptr)) {
      CHECK(x.kso == 0 && x.nk == nk_all, "PART 0 item with a K piece");
      cover(t, x.it, NT, cells, 1);
    }
    for (size_t i = 0; i < ncell; ++i) CHECK(cells[i] == 1, "PART 0: cell %zu computed %d times", i, cells[i]);
  }
  // the split down projection: PART 1, PART 2 (its K pieces), then the reducer
  {
    GemmPlan p1, p2;
    std::vector<int> cells(ncell, 0);
    for (const Run& x : launch(t, NT, split_nar_ok, 1, grid, nk_all, &p1)) cover(t, x.it, NT, cells, 1);
    const std::vector<Run> tail = launch(t, NT, split_nar_ok, 2, grid, nk_all, &p2);
    CHECK(p1.S_all == p2.S_all && p1.S_main == p2.S_main && p1.nar == p2.nar && p1.n_tail == p2.n_tail,
          "PART 1 and PART 2 plans differ");
    // K coverage per tail item: pieces 0..q-1 tile [0, nk_all) in order
    std::map<long long, std::vector<Run>> by_item;
    for (const Run& x : tail) by_item[(x.w / p2.q)].push_back(x);
    for (auto& kv : by_item) {
      int next = 0;
      for (int pc = 0; pc < p2.q; ++pc) {
        const Run* found = nullptr;
        for (const Run& x : kv.second)
          if (x.piece == pc) found = &x;
        CHECK(found, "tail item %lld misses piece %d", kv.first, pc);
        CHECK(found->kso == next && found->nk >= 1, "tail item %lld piece %d covers slabs [%d, +%d), expected %d",
              kv.first, pc, found->kso, found->nk, next);
        CHECK(found->w == kv.first * p2.q + pc, "partial index %lld for item %lld piece %d", found->w, kv.first, pc);
        CHECK(found->it == kv.second[0].it, "pieces of one tail item decode to different tiles");
        next += found->nk;
      }
      CHECK(next == nk_all, "tail item %lld covers %d of %d slabs", kv.first, next, nk_all);
      cover(t, kv.second[0].it, NT, cells, 1);
    }
    for (size_t i = 0; i < ncell; ++i) CHECK(cells[i] == 1, "split: cell %zu computed %d times", i, cells[i]);
    if (p2.q > 1) {
      CHECK((p2.S_all - p2.S_main) * p2.q <= kMaxTailItems, "tail partials %lld exceed the buffer",
            (p2.S_all - p2.S_main) * p2.q);
      // the reducer: workgroup b sums partials b q .. b q + q - 1 of item S_main + b, with the
      // plan it derives from the same table, narrow flag and grid
      const GemmPlan pr = gemm_plan(t.data(), NT, split_nar_ok, 2, grid, nk_all);
      CHECK(pr.q == p2.q && pr.S_main == p2.S_main && pr.S_all == p2.S_all, "reducer plan differs from PART 2");
      for (long long b = 0; b < pr.S_all - pr.S_main; ++b) {
        const Item it = decode(t, pr, pr.S_main + b, NT);
        CHECK(by_item.count(b) && it == by_item[b][0].it, "reducer item %lld is not the tile PART 2 computed", b);
      }
    }
  }
}

// supertile is a bijection of a group's items onto its (m-tile, n-tile) cells
static void check_supertile() {
  for (int me = 1; me <= 40; ++me)
    for (int NT : {1, 2, 3, 4, 5, 7, 16, 28, 112}) {
      std::vector<int> seen((size_t)me * NT, 0);
      for (long long l = 0; l < (long long)me * NT; ++l) {
        int mt, nt;
        supertile(l, me, NT, &mt, &nt);
        CHECK(mt >= 0 && mt < me && nt >= 0 && nt < NT, "supertile(%lld, %d, %d) = (%d, %d)", l, me, NT, mt, nt);
        ++seen[(size_t)mt * NT + nt];
      }
      for (size_t i = 0; i < seen.size(); ++i) CHECK(seen[i] == 1, "supertile %d x %d: cell %zu taken %d times", me, NT, i, seen[i]);
    }
}

int main() {
  check_addresses();
  const long long after_addr = n_checks;
  check_supertile();

  // The launch decisions of the down projection (narrow-capable kernel iff down_narrow_for)
  // over shapes that cross A / E = 512 and 1024, and skewed ones.
  std::mt19937_64 rng(12345);
  const int grids[3] = {256, 64, 8};
  const int nts[6] = {1, 2, 3, 16, 28, 56};
  const int nks[5] = {1, 8, 29, 128, 448};
  int cases = 0;
  for (int E : {1, 2, 8, 16, 64, 128, 256}) {
    for (int mean : {1, 100, 128, 129, 300, 512, 513, 600, 1000, 1024, 1025, 2048}) {
      for (int skew = 0; skew < 2; ++skew) {
        std::vector<int> counts(E);
        for (int e = 0; e < E; ++e) {
          if (!skew) counts[e] = mean;
          else {
            // geometric-ish spread with empty experts, total about E * mean
            const double u = std::uniform_real_distribution<double>(0.0, 1.0)(rng);
            counts[e] = (u < 0.15) ? 0 : (int)(mean * 3.0 * u * u);
          }
        }
        long long A = 0;
        for (int c : counts) A += c;
        if (A == 0) continue;
        const bool up_nar = narrow_rows_for(A, E, true) > 0;
        const bool down_nar = down_narrow_for(A, E, true);
        const int NT = nts[(cases) % 6], grid = grids[(cases / 6) % 3], nk = nks[(cases / 18) % 5];
        check_schedule(counts, NT, grid, nk, up_nar, down_nar);
        ++cases;
      }
    }
  }
  // The shapes of the finding that motivated the shared plan: 8 experts of 600 rows (table
  // with narrow tiles, down projection without) at the down projection's tile counts of
  // d_model = 256 .. 4096, and a Mixtral-shaped N = 2400 layer (A = 4800, d_model = 4096,
  // d_ff = 14336).
  for (int NT : {1, 2, 4, 8, 16})
    for (int nk : {9, 29, 448}) {
      check_schedule(std::vector<int>(8, 600), NT, 256, nk, true, down_narrow_for(4800, 8, true));
      ++cases;
    }
  // What the reducer used to do (its own narrow decision, ignoring the launch's): for 8 x 600
  // rows at NT = 16, K = 14336 it numbers the tail differently from the GEMM launches.
  {
    const std::vector<int> t = make_table(std::vector<int>(8, 600), kSchedBM, narrow_rows_for(4800, 8, true));
    const GemmPlan gemm = gemm_plan(t.data(), 16, false, 2, 256, 448);
    const GemmPlan old_reducer = gemm_plan(t.data(), 16, true, 2, 256, 448);
    CHECK(gemm.q != old_reducer.q || gemm.S_all != old_reducer.S_all,
          "the old reducer rule agrees with the launch here; the case no longer exercises the finding");
  }
  // What the copies used to do: add the row part and the K part to the 64-bit base one after
  // the other, so a wrapped K part (K < 32) moved the source about 4 GiB past the row.
  {
    const int K = 8, lane = 2, lc = lane_chunk(lane);  // lchunk 16 > K - 8
    const unsigned long long old_off = (unsigned long long)rm_row_off(0, K, lc) + (unsigned long long)rm_k_off(K, 0, lc);
    CHECK(old_off >= (1ull << 32), "K = 8: the separate 64-bit sum stays in the row; the case no longer shows the bug");
    CHECK(src_off(rm_row_off(0, K, lc), rm_k_off(K, 0, lc)) == 0, "K = 8: the 32-bit sum is not the row's last chunk");
  }
  std::printf("ok %lld checks (%lld address, %d schedule cases)\n", n_checks, after_addr, cases);
  return 0;
}
