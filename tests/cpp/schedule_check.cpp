// CPU check of the bins decode schedule (test infrastructure): replays every
// wave's descriptor walk the way the decode kernel does, and checks that every
// (kv head, sequence, tile) is covered exactly once, that each segment split
// between the waves of a bin has exactly one merging wave, and that the LDS
// pieces that wave reads are the ones the other waves left for that segment.
// Built from the host source with the GPU launch helpers stubbed out.
#include "pkv_host.cpp"
#include <random>
#include <map>
#include <set>
#include <cassert>

// stubs for the GPU launch helpers referenced by pkv_host.cpp
namespace pkv {
hipError_t launch_decode(int, int, int, bool, int, const DecodeParams&, hipStream_t) { return hipSuccess; }
hipError_t launch_reduce(int, int, const ReduceParams&, hipStream_t) { return hipSuccess; }
int decode_blocks_per_cu(int, int, int, bool, int) { return 1; }
hipError_t launch_append(const void*, const void*, const int64_t*, int, void*, void*, int, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_append_quant(int, const void*, const void*, const int64_t*, int, void*, void*, int, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_copy_blocks(const int32_t*, int, void*, void*, int, int64_t, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_upload(const void*, void*, size_t, hipStream_t) { return hipSuccess; }
}

static int check(std::vector<int> ctx, int H, int nbins, bool expect_bins, int bs = 16) {
  pkv_pool P;
  pkv_pool* p = &P;
  p->shape.kv_heads = H;
  p->shape.block_size = bs;
  const int B = ctx.size();
  p->up_batch = B;
  int maxb = 0;
  for (int L : ctx) maxb = std::max<int>(maxb, (L + bs - 1) / bs);  // table entries
  p->up_stride = maxb;
  p->h_ctx = ctx;
  p->h_bt.assign((size_t)B * maxb, -1);
  int id = 0;
  for (int s = 0; s < B; ++s)
    for (int j = 0; j < (ctx[s] + bs - 1) / bs; ++j) p->h_bt[(size_t)s * maxb + j] = 1000 + id++;
  bool ok = build_bins(p, nbins);
  if (ok != expect_bins && expect_bins) { printf("bins refused (expected)\n"); return 1; }
  if (!ok) return 0;
  const int W = p->sched_nwaves, nseg = B * H;
  const int32_t* desc = p->h_sched.data();
  const int32_t* list = desc + 8 * (size_t)W + 2 * (size_t)nseg;
  // coverage: (g, s, j) -> count
  std::map<std::tuple<int,int,int>, int> cov;
  int merges = 0, errors = 0;
  for (int b = 0; b < nbins; ++b) {
    // pieces[(wave, slot)] = (s, g)
    std::map<std::pair<int,int>, std::pair<int,int>> pieces;
    std::vector<std::pair<int,int>> first_seg_of(8, {-1,-1});
    for (int wl = 0; wl < 8; ++wl) {
      const int32_t* d = desc + 8 * (size_t)(b * 8 + wl);
      int li = d[0], count = d[1], s = d[2], g = d[3], j0 = d[4], L = d[5], blk = d[6];
      if (count == 0) continue;
      if (li < 0 || li >= nseg) { printf("bad li\n"); return 1; }
      const int32_t* e0 = list + 4 * li;
      if (e0[0] != s || e0[1] != g || e0[2] != L) { printf("desc/list mismatch\n"); return 1; }
      if (blk != p->h_bt[(size_t)s * maxb + j0 * 16 / bs]) { printf("bad first blk\n"); return 1; }
      int x = 0; bool first = true;
      first_seg_of[wl] = {s, g};
      while (x < count) {
        int nblk = (L + 15) / 16;
        int take = std::min(count - x, nblk - j0);
        if (take <= 0) { printf("empty take\n"); return 1; }
        for (int j = j0; j < j0 + take; ++j) cov[{g, s, j}]++;
        bool whole = j0 == 0 && j0 + take == nblk;
        if (!whole) pieces[{wl, first ? 0 : 1}] = {s, g};
        x += take;
        if (x >= count) break;
        ++li;
        if (li >= nseg) { printf("li overflow\n"); return 1; }
        const int32_t* e = list + 4 * li;
        s = e[0]; g = e[1]; L = e[2]; j0 = 0; first = false;
        if (e[3] != p->h_bt[(size_t)s * maxb]) { printf("bad list blk\n"); return 1; }
      }
    }
    // merges
    std::set<std::pair<int,int>> merged;
    for (int wl = 0; wl < 8; ++wl) {
      const int32_t* d = desc + 8 * (size_t)(b * 8 + wl);
      int mi = d[7];
      if (!(mi & (1 << 16))) continue;
      int wa = mi & 0xff, wa_slot = (mi >> 8) & 1;
      auto seg = first_seg_of[wl];
      for (int v = wa; v <= wl; ++v) {
        int sl = v == wa ? wa_slot : 0;
        auto it = pieces.find({v, sl});
        if (it == pieces.end() || it->second != seg) { printf("merge piece missing b%d w%d v%d\n", b, wl, v); errors++; }
      }
      merged.insert(seg);
      merges++;
    }
    // every split segment in this bin merged exactly once
    std::set<std::pair<int,int>> split;
    for (auto& kv : pieces) split.insert(kv.second);
    if (split != merged) { printf("split/merged mismatch in bin %d (%zu vs %zu)\n", b, split.size(), merged.size()); errors++; }
  }
  for (int g = 0; g < H; ++g)
    for (int s = 0; s < B; ++s)
      for (int j = 0; j < (ctx[s] + 15) / 16; ++j)
        if (cov[{g, s, j}] != 1) { printf("tile (%d,%d,%d) covered %d\n", g, s, j, cov[{g,s,j}]); return 1; }
  printf("ok: B=%d H=%d bs=%d bins=%d waves=%d merges=%d errors=%d\n", B, H, bs, nbins, W, merges, errors);
  return errors;
}

int main() {
  std::mt19937 rng(1);
  int rc = 0;
  { std::vector<int> c(64); std::uniform_int_distribution<int> u(128, 2048); for (auto& x : c) x = u(rng); rc |= check(c, 8, 256, true); }
  { std::vector<int> c(256); std::uniform_int_distribution<int> u(16, 2048); for (auto& x : c) x = u(rng); rc |= check(c, 40, 256, true); }
  { std::vector<int> c(128); std::uniform_int_distribution<int> u(1025, 1537); for (auto& x : c) x = u(rng); rc |= check(c, 8, 256, true); }
  { std::vector<int> c(6); std::uniform_int_distribution<int> u(1, 700); for (auto& x : c) x = u(rng); rc |= check(c, 8, 4, false); }
  for (int bs : {8, 32}) {
    std::vector<int> c(64); std::uniform_int_distribution<int> u(128, 2048); for (auto& x : c) x = u(rng);
    rc |= check(c, 8, 256, true, bs);
  }
  for (int t = 0; t < 300; ++t) {
    std::uniform_int_distribution<int> nb(1, 64), lb(1, 3000), hb(1, 8), bb(1, 64);
    std::vector<int> c(nb(rng)); for (auto& x : c) x = lb(rng);
    const int bs = t % 3 == 0 ? 8 : t % 3 == 1 ? 16 : 32;
    rc |= check(c, hb(rng), bb(rng), false, bs);
  }
  printf(rc ? "FAILED\n" : "ALL OK\n");
  return rc;
}
