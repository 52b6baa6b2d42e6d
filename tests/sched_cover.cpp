// Host check of the attention kernels' work schedules (built host-only by
// tests/test_schedule_cover.py; needs no GPU).
//
// The decoder the kernels run (attend_work, with xcd_split, xcd_rounds and
// split_tile) is taken from the library's own header and called on the host
// for every workgroup of a launch.  Each workgroup's items are turned into
// key-tile ranges the way the attention kernels do, and the combine
// kernel's block-to-pair mapping is replayed.  For every shape it checks:
//   * every key tile of every (head, query tile) pair is computed exactly
//     once, by one whole-pair workgroup or by exactly two parts of a cut
//     pair (a head or a tail; rounds: the two halves);
//   * the parts of a cut pair write the slots the combine kernel reads for
//     that pair (split: 2p, 2p + 1; rounds: slot0, slot0 + 1), every slot
//     lies inside the partial-result buffer and no two pairs share one;
//   * the combine kernel merges exactly the cut pairs;
//   * padding workgroups (rounds) do nothing.
// The schedule choice of the launcher (split when a partial-result buffer
// is given and 2 * pairs <= 2 * CUs, rounds when pairs > 2 * CUs and some
// XCD has a remainder to halve, else one workgroup per pair) is restated in
// plan() below.
#include <hip/hip_runtime.h>

// Make the device-only decoder callable from this host program.
#undef __device__
#define __device__ __attribute__((host, device))
#include "fkv_device.h"

#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

struct Plan {
  int sched, n_wg, slots_x, cut_max, combine_blocks, part_slots;
  bool has_part;
};

// The launcher's choice (two workgroups resident per CU).
Plan plan(int pairs, int cus, bool give_part) {
  Plan p{0, pairs, 0, 0, 0, 0, false};
  const int nb = 2 * cus;
  const bool have = give_part && nb > 0 && nb % 8 == 0;
  p.part_slots = 2 * nb;
  if (have && 2 * pairs <= nb) {
    p = Plan{1, nb, 0, 0, pairs, 2 * nb, true};
    return p;
  }
  if (have && pairs > nb) {
    int cut_max = 0, per_x = 0;
    for (int x = 0; x < 8; ++x) {
      const fkv::XcdRounds xr = fkv::xcd_rounds(pairs, nb / 8, x);
      cut_max = xr.s > cut_max ? xr.s : cut_max;
      per_x = xr.w + 2 * xr.s > per_x ? xr.w + 2 * xr.s : per_x;
    }
    if (cut_max > 0) p = Plan{2, 8 * per_x, nb / 8, cut_max, 8 * cut_max, 2 * nb, true};
  }
  return p;
}

int g_fail = 0;
#define CHECK(cond, ...)                                                 \
  do {                                                                   \
    if (!(cond)) {                                                       \
      if (g_fail < 20) {                                                 \
        std::printf("FAIL %s:%d: ", __FILE__, __LINE__);                 \
        std::printf(__VA_ARGS__);                                        \
        std::printf("\n");                                               \
      }                                                                  \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

// One launch: ntq query tiles per head, nt_h[h] key tiles for head h.
void check_launch(int ntq, const std::vector<int> &nt_h, int cus, bool give_part) {
  const int H = (int)nt_h.size();
  const int pairs = ntq * H;
  const Plan pl = plan(pairs, cus, give_part);
  // cover[p][t]: times tile t of pair p was computed.
  std::vector<std::vector<int>> cover(pairs);
  std::vector<int> parts(pairs, 0), wholes(pairs, 0);
  std::vector<int> slot_of(pairs * 2, -1);  // [2p + tail] -> slot written
  for (int p = 0; p < pairs; ++p) cover[p].assign(nt_h[p / ntq], 0);

  for (int b = 0; b < pl.n_wg; ++b) {
    const fkv::AttendWork w =
        fkv::attend_work(pairs, pl.has_part, pl.sched, pl.slots_x, pl.cut_max, pl.n_wg, b);
    if (w.n_items < 0) continue;  // padding
    for (int item = 0; item < w.n_items; ++item) {
      const int p = w.p0 + item;
      CHECK(p >= 0 && p < pairs, "pair %d out of [0, %d) (wg %d)", p, pairs, b);
      if (p < 0 || p >= pairs) continue;
      const int nt = nt_h[p / ntq];
      const int ts = w.k < 0 ? nt / 2 : fkv::split_tile(nt, w.k);
      const int t0 = w.tail ? ts : 0, t1 = w.tail ? nt : ts;
      if (t0 >= t1) continue;  // empty part: the kernel skips it
      for (int t = t0; t < t1; ++t) cover[p][t]++;
      if (t0 == 0 && t1 == nt) {
        wholes[p]++;
      } else {
        parts[p]++;
        const int slot = w.slot0 >= 0 ? w.slot0 + w.tail : 2 * p + w.tail;
        CHECK(slot >= 0 && slot < pl.part_slots, "slot %d outside %d", slot, pl.part_slots);
        CHECK(slot_of[2 * p + w.tail] < 0, "pair %d part %d written twice", p, w.tail);
        slot_of[2 * p + w.tail] = slot;
      }
    }
  }
  for (int p = 0; p < pairs; ++p) {
    for (int t = 0; t < (int)cover[p].size(); ++t)
      CHECK(cover[p][t] == 1, "pair %d tile %d computed %d times (sched %d, pairs %d, cus %d)", p,
            t, cover[p][t], pl.sched, pairs, cus);
    CHECK((wholes[p] == 1 && parts[p] == 0) || (wholes[p] == 0 && parts[p] == 2) ||
              (cover[p].empty() && wholes[p] + parts[p] == 0),
          "pair %d: %d whole, %d parts (sched %d)", p, wholes[p], parts[p], pl.sched);
  }
  // Slots: distinct across pairs.
  std::vector<int> owner(pl.part_slots > 0 ? pl.part_slots : 1, -1);
  for (int p = 0; p < pairs; ++p)
    for (int s = 0; s < 2; ++s) {
      const int slot = slot_of[2 * p + s];
      if (slot < 0) continue;
      CHECK(owner[slot] < 0, "slot %d shared by pairs %d and %d", slot, owner[slot], p);
      owner[slot] = p;
    }
  // The combine kernel's blocks: which pair each merges, from which slots.
  std::vector<int> merged(pairs, 0);
  for (int blk = 0; blk < pl.combine_blocks; ++blk) {
    int p, nt, ts, slot;
    if (pl.sched == 2) {
      const int x = blk & 7, c = blk >> 3;
      const fkv::XcdRounds xr = fkv::xcd_rounds(pairs, pl.slots_x, x);
      if (c >= xr.s) continue;
      p = xr.p_lo + xr.w + c;
      nt = nt_h[p / ntq];
      ts = nt / 2;
      slot = 2 * (x * pl.cut_max + c);
    } else {
      p = blk;
      int x = 0;
      while (x < 7 && p >= pairs * (x + 1) / 8) ++x;
      const fkv::XcdSplit sp = fkv::xcd_split(pairs, pl.n_wg, x);
      nt = nt_h[p / ntq];
      ts = fkv::split_tile(nt, sp.k);
      slot = 2 * p;
    }
    if (ts == 0 || ts == nt) continue;
    merged[p]++;
    CHECK(slot_of[2 * p] == slot && slot_of[2 * p + 1] == slot + 1,
          "combine of pair %d reads slots %d, %d; parts wrote %d, %d", p, slot, slot + 1,
          slot_of[2 * p], slot_of[2 * p + 1]);
  }
  for (int p = 0; p < pairs; ++p)
    CHECK(merged[p] == (parts[p] == 2 ? 1 : 0), "pair %d merged %d times with %d parts", p,
          merged[p], parts[p]);
}

}  // namespace

int main() {
  long cases = 0;
  unsigned seed = 12345u;
  auto rnd = [&](int n) {
    seed = seed * 1103515245u + 12345u;
    return (int)((seed >> 8) % (unsigned)n);
  };
  const int cus_list[] = {8, 16, 80, 104, 256, 304};
  for (int cus : cus_list)
    for (int give = 0; give < 2; ++give) {
      // Every pair count up to a few rounds, uniform and ragged tile counts.
      const int max_pairs = 5 * 2 * cus + 17;
      for (int pairs = 1; pairs <= max_pairs; pairs += (pairs < 64 ? 1 : 1 + pairs / 64)) {
        for (int ntq = 1; ntq <= 3; ++ntq) {
          if (pairs % ntq) continue;
          const int H = pairs / ntq;
          std::vector<int> nt_h(H);
          for (int h = 0; h < H; ++h) nt_h[h] = 1 + (h * 7) % 5;  // 1 .. 5 tiles
          check_launch(ntq, nt_h, cus, give);
          for (int h = 0; h < H; ++h) nt_h[h] = 1 + rnd(400);
          check_launch(ntq, nt_h, cus, give);
          for (int h = 0; h < H; ++h) nt_h[h] = rnd(3);  // empty heads too
          check_launch(ntq, nt_h, cus, give);
          cases += 3;
        }
      }
    }
  // The bench workloads on 256 CUs: 480P (37 query tiles x 12 heads, about
  // 375 key tiles per head) and 1080P (192 x 12, about 1900).
  std::vector<int> h480(12, 375), h1080(12, 1904);
  check_launch(37, h480, 256, true);
  check_launch(192, h1080, 256, true);
  cases += 2;
  if (g_fail) {
    std::printf("%d failures in %ld launches\n", g_fail, cases);
    return 1;
  }
  std::printf("OK %ld launches\n", cases);
  return 0;
}
